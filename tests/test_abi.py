"""CPU checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments before touching the GPU.

No compute call is made here: every fa_fwd call below fails validation,
which runs before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


def declared_functions():
    names = set()
    for fn in os.listdir(HEADER_DIR):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def fa():
    import aware_softmax_amd

    return aware_softmax_amd


def test_header_declares_entry_points():
    names = declared_functions()
    for required in ("fa_fwd", "fa_status_string", "fa_fwd_tile", "fa_version"):
        assert required in names


def test_every_declared_symbol_is_exported(fa):
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_library_carries_gfx950_code_object(fa):
    """The library built here embeds a code object for the gfx950 target."""
    with open(fa.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_status_strings(fa):
    for code in range(9):
        s = fa.status_string(code)
        assert s.startswith("FA_")
    assert fa.status_string(99) == "unknown fa_status_t"
    assert "gfx950" in fa.version()


def test_tile_config(fa):
    bq, bk, w = fa.tile_config(128, fa.DTYPE_BF16)
    assert bk == 64 and bq == 32 * w and w in (4, 8)
    assert fa.tile_config(64, fa.DTYPE_BF16)[0] > 0
    assert fa.tile_config(64, fa.DTYPE_F32)[0] > 0
    with pytest.raises(fa.FaError) as e:
        fa.tile_config(96, fa.DTYPE_BF16)
    assert e.value.code == 4
    with pytest.raises(fa.FaError) as e:
        fa.tile_config(64, 7)
    assert e.value.code == 3


# Fake, never-dereferenced device addresses: validation rejects each call
# before any HIP call is made.
A = 0x10000000
GOOD = dict(q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000, lse=A + 0x4000000,
            B=1, H=2, N=64, d=64, causal=1, scale=0.125, dtype=1, stream=None)


def call(fa, **over):
    a = dict(GOOD)
    a.update(over)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                     a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1), (dict(lse=0), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(N=0), 2), (dict(d=0), 2),
    (dict(B=1 << 20, H=1 << 12, N=1 << 20), 2),
    (dict(dtype=2), 3), (dict(dtype=-1), 3),
    (dict(d=96), 4), (dict(d=256), 4), (dict(d=32), 4),
    (dict(q=A + 8), 5), (dict(o=A + 0x3000004), 5), (dict(lse=A + 0x4000002), 5),
    (dict(scale=float("nan")), 6), (dict(scale=float("inf")), 6),
    (dict(o=A), 8), (dict(lse=A + 0x3000100), 8), (dict(lse=A + 0x2000000), 8),
])
def test_validation_rejects_before_launch(fa, over, code):
    assert call(fa, **over) == code


def test_python_binding_rejects_host_tensors(fa):
    import torch

    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.fwd(q.half(), q.half(), q.half())


def test_schedule_is_a_bijection(tmp_path):
    """The workgroup -> (head, query block) remap covers every pair once."""
    src = tmp_path / "sched.cpp"
    src.write_text(r"""
#include <cstdio>
#include <vector>
#include "fa_schedule.h"
int main() {
  const int cases[][2] = {{1,1},{1,3},{7,1},{16,16},{256,64},{16,256},{3,5},{13,9},{32,128},{5,1}};
  for (auto& c : cases) {
    const int heads = c[0], nqb = c[1], total = heads * nqb;
    for (int hf = 0; hf < 2; ++hf) {
      std::vector<int> seen(total, 0);
      for (int id = 0; id < total; ++id) {
        int bh, qb; fa::map_block(id, total, nqb, hf != 0, &bh, &qb);
        if (bh < 0 || bh >= heads || qb < 0 || qb >= nqb) { printf("out of range\n"); return 1; }
        seen[bh * nqb + qb]++;
      }
      for (int x : seen) if (x != 1) { printf("not a bijection\n"); return 1; }
      // every XCD (id % 8) gets a contiguous run of (head, block) pairs
      if (hf) {
        int bh, qb; fa::map_block(0, total, nqb, true, &bh, &qb);
        if (bh != 0 || qb != nqb - 1) { printf("heavy block not first\n"); return 1; }
      }
    }
  }
  printf("ok\n");
  return 0;
}
""")
    exe = tmp_path / "sched"
    csrc = os.path.join(ROOT, "aware_softmax_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", csrc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
