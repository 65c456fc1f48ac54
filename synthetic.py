"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it draws i.i.d. N(0, 1) values
from counter-addressed NumPy PCG64 streams and rounds them to bfloat16
(round to nearest, ties to even) when a config asks for bf16 inputs, or
encodes 32 times them as OCP FP8 E4M3 codes for the 8-bit forward.  Both
the fp64 oracle and the HIP path consume exactly the values produced here.

Streams: one per (config, tensor, batch index, head index), seeded with the
sequence [0xFA, config_id, tensor_id, b, h], so any single head can be
regenerated without materialising the others.  Row samples use
[0xFA, config_id, 99, salt].

The workloads (sizes, causal flag, dtype) are the five attention problems
the method is measured on:
  1: B=1, H=1,  N=256,   d=64,  fp32, non-causal
  2: B=1, H=16, N=2048,  d=64,  bf16, causal
  3: B=8, H=32, N=8192,  d=128, bf16, causal   (the throughput workload)
  4: B=1, H=16, N=32768, d=128, bf16, causal   (long context, batch 1)
  5: B=2, H=16, N=4096,  d=128, bf16, causal   (forward plus backward)
and the decode problems (one query row per sequence against a cache of N
keys; q [B][H][d] is drawn as N = 1 rows of the q stream, k and v as
[B][Hkv][N][d]):
  6: B=8, H=Hkv=32, N=32768, d=128, bf16   (decode, batch 8, 32 heads)
  7: B=1, H=Hkv=32, N=32768, d=128, bf16   (decode, batch 1)
  8: B=8, H=32, Hkv=8, N=32768, d=128, bf16 (decode, 4 query heads per
     key/value head)
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


@dataclass(frozen=True)
class Workload:
    config_id: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32", "bf16" or "f16"
    causal: bool

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    1: Workload(1, "single-head fp32 non-causal B1 H1 N256 d64", 1, 1, 256, 64, "f32", False),
    2: Workload(2, "causal bf16 B1 H16 N2048 d64", 1, 16, 2048, 64, "bf16", True),
    3: Workload(3, "causal bf16 B8 H32 N8192 d128", 8, 32, 8192, 128, "bf16", True),
    4: Workload(4, "long-context causal bf16 B1 H16 N32768 d128", 1, 16, 32768, 128, "bf16", True),
    5: Workload(5, "causal bf16 forward and backward B2 H16 N4096 d128", 2, 16, 4096, 128, "bf16", True),
}


@dataclass(frozen=True)
class DecodeWorkload:
    config_id: int
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


DECODE_WORKLOADS = {
    6: DecodeWorkload(6, "decode bf16 B8 H32 N32768 d128", 8, 32, 32, 32768, 128),
    7: DecodeWorkload(7, "decode bf16 B1 H32 N32768 d128", 1, 32, 32, 32768, 128),
    8: DecodeWorkload(8, "decode bf16 B8 H32 Hkv8 N32768 d128", 8, 32, 8, 32768, 128),
}


def decode_storage(config_id: int, B: int, H: int, Hkv: int, N: int, d: int, threads: int = 8,
                   dtype: str = "bf16") -> dict:
    """Storage form (bf16 bits or float16) of a decode problem: q [B][H][d],
    k and v [B][Hkv][N][d]."""
    return {
        "q": full_storage(config_id, "q", B, H, 1, d, dtype, threads).reshape(B, H, d),
        "k": full_storage(config_id, "k", B, Hkv, N, d, dtype, threads),
        "v": full_storage(config_id, "v", B, Hkv, N, d, dtype, threads),
    }


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs are finite normal draws; no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


# e4m3 inputs: the N(0, 1) draw times 32, rounded to OCP FP8 E4M3, so each
# e4m3 tensor's dequantisation factor is 1/32 (|x| up to 14 is representable,
# values near 1 keep 3 mantissa bits; N(0, 1) draws never saturate).
E4M3_GAIN = 32.0
E4M3_DESCALE = 1.0 / E4M3_GAIN


def e4m3_round_bits(x: np.ndarray) -> np.ndarray:
    """float -> OCP FP8 E4M3 codes (uint8): round to nearest, ties to even,
    saturating at +-448 (exponent bias 7, 3 mantissa bits, subnormals
    below 2^-6).  Inputs are finite."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    neg = np.signbit(np.asarray(x, dtype=np.float64))
    a = np.minimum(a, 448.0)
    # binade of a (subnormals share the quantum of the lowest binade, 2^-9)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    quantum = np.exp2(e - 3)
    v = np.rint(a / quantum) * quantum  # np.rint: ties to even
    v = np.minimum(v, 448.0)
    # encode the rounded value (which may have moved up one binade)
    ev = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    normal = v >= 2.0 ** -6
    exp_field = np.where(normal, ev + 7, 0)
    mant = np.where(normal, v / np.exp2(ev - 3) - 8, v / 2.0 ** -9)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(v == 0, 0, code)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exactly equal fp32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def head_stream(config_id: int, tensor: str, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([0xFA, config_id, TENSOR_IDS[tensor], b, h]))


def head_values(config_id: int, tensor: str, b: int, h: int, n: int, d: int, dtype: str) -> np.ndarray:
    """One head's (n, d) tensor as fp32 values (representable in the dtype)."""
    x = head_stream(config_id, tensor, b, h).standard_normal((n, d), dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(bf16_round_bits(x))
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)  # IEEE round to nearest even
    return x


def head_storage(config_id: int, tensor: str, b: int, h: int, n: int, d: int, dtype: str) -> np.ndarray:
    """One head's (n, d) tensor in storage form: uint16 bf16 bits, uint8
    e4m3 codes (of the draw times E4M3_GAIN), float16 or float32."""
    x = head_stream(config_id, tensor, b, h).standard_normal((n, d), dtype=np.float32)
    if dtype == "bf16":
        return bf16_round_bits(x)
    if dtype == "e4m3":
        return e4m3_round_bits(x * E4M3_GAIN)
    if dtype == "f16":
        return x.astype(np.float16)
    return x


def full_storage(config_id: int, tensor: str, B: int, H: int, N: int, d: int, dtype: str,
                 threads: int = 8) -> np.ndarray:
    """The whole [B][H][N][d] tensor in storage form (uint16 bf16 bits, uint8
    e4m3 codes, float16 or float32)."""
    out = np.empty((B, H, N, d), dtype={"bf16": np.uint16, "f16": np.float16, "e4m3": np.uint8}.get(dtype, np.float32))

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = head_storage(config_id, tensor, b, h, N, d, dtype)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def workload_storage(w: Workload, tensors=("q", "k", "v"), threads: int = 8) -> dict:
    return {t: full_storage(w.config_id, t, w.B, w.H, w.N, w.d, w.dtype, threads) for t in tensors}


def sample_rows(config_id: int, n: int, count: int, salt: int = 0) -> np.ndarray:
    """Sorted query-row sample: `count` seeded rows plus the edge rows of
    every query block size in use (64, 128 and 256 rows: the last row of the
    first and second blocks and the first of the next ones), the first two
    rows, and the rows around the start of the last 128- and 256-row blocks
    and at the end (those inside 0..n-1)."""
    rng = np.random.Generator(np.random.PCG64([0xFA, config_id, 99, salt]))
    count = min(count, n)
    picked = rng.choice(n, size=count, replace=False)
    edges = [0, 1, n - 2, n - 1]
    for b in (64, 128, 256):
        edges += [b - 1, b, 2 * b - 1, 2 * b]
        last = (n - 1) // b * b  # first row of the last b-row block
        edges += [last - 1, last]
    edges = [r for r in edges if 0 <= r < n]
    return np.unique(np.concatenate([picked, np.array(edges, dtype=np.int64)]))


def sample_heads(config_id: int, B: int, H: int, count: int) -> list:
    """`count` distinct seeded (b, h) pairs."""
    rng = np.random.Generator(np.random.PCG64([0xFA, config_id, 98]))
    flat = rng.choice(B * H, size=min(count, B * H), replace=False)
    return [divmod(int(x), H) for x in sorted(flat)]


def random_values(seed: int, shape, dtype: str = "f32") -> np.ndarray:
    """Free-form seeded N(0, 1) draws (fp32 values, bf16-rounded if asked)."""
    x = np.random.Generator(np.random.PCG64([0xFA, 7, seed])).standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(bf16_round_bits(x))
    return x
