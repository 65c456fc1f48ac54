"""Host checks of the seeded input generator (CPU only)."""
import numpy as np
import torch

import synthetic


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even to bfloat16 agrees with torch's CPU cast."""
    x = np.concatenate([
        synthetic.random_values(1, (10000,)) * 7,
        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-30, 0.0, -0.0], dtype=np.float32),
    ]).astype(np.float32)
    ours = synthetic.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synthetic.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_streams_are_per_head_and_reproducible():
    a = synthetic.head_values(2, "q", 0, 3, 64, 8, "bf16")
    b = synthetic.head_values(2, "q", 0, 3, 64, 8, "bf16")
    c = synthetic.head_values(2, "k", 0, 3, 64, 8, "bf16")
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    full = synthetic.full_storage(2, "q", 1, 4, 64, 8, "bf16", threads=2)
    assert np.array_equal(synthetic.bf16_bits_to_f32(full[0, 3]), a)


def test_normal_moments():
    x = synthetic.head_values(3, "v", 1, 2, 4096, 64, "f32")
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01


def test_row_and_head_samples():
    r = synthetic.sample_rows(3, 8192, 512)
    assert len(r) >= 512 and r.min() == 0 and r.max() == 8191 and np.all(np.diff(r) > 0)
    # edges of the 64-, 128- and 256-row query blocks, first and last blocks
    assert {1, 63, 64, 127, 128, 255, 256, 511, 512, 7935, 7936, 8063, 8064, 8190}.issubset(set(r.tolist()))
    assert np.array_equal(r, synthetic.sample_rows(3, 8192, 512))
    heads = synthetic.sample_heads(3, 8, 32, 4)
    assert len(set(heads)) == 4 and all(0 <= b < 8 and 0 <= h < 32 for b, h in heads)


def test_workload_table():
    w = synthetic.WORKLOADS[3]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal) == (8, 32, 8192, 128, "bf16", True)
    assert abs(w.scale - 128 ** -0.5) < 1e-15
