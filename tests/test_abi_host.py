"""Host-side checks of the C ABI library (no GPU needed): it loads, exports
every entry point include/jagg.h declares, and its host-only geometry and
argument checking agree with the pages' definitions (via the oracle)."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jagg.h")

from oracle import oracle as O  # noqa: E402
from tensor_relational_einsum_amd import jagg  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(jagg_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = jagg.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"{n} declared in jagg.h but not exported"
    assert set(names) == set(jagg.EXPORTS)


def test_calibration_library_exports_every_declared_function():
    # libjagg_calib.so: the machine-peak probes the benchmark times
    from tensor_relational_einsum_amd import build as B
    text = open(os.path.join(ROOT, "include", "jagg_calib.h")).read()
    names = sorted(set(re.findall(r"\b(jagg_\w+)\s*\(", text)))
    assert names == ["jagg_calib_mfma_bf16", "jagg_calib_mfma_f32"]
    L = ctypes.CDLL(B.CALIB_LIB)
    for n in names:
        assert hasattr(L, n), f"{n} declared in jagg_calib.h but not exported"


@pytest.mark.parametrize("letters,ext,blk,dtype", [
    ("ij", (256, 256), (4, 4), "f32"),
    ("abcd", (96, 300, 64, 48), (5, 7, 4, 3), "f32"),
    ("cde", (64, 48, 1000), (4, 3, 6), "f32"),
    ("abcd", (32, 128, 64, 64), (4, 8, 1, 1), "bf16"),
    ("a", (10,), (4,), "bf16"),
])
def test_relation_bytes_matches_oracle_geometry(letters, ext, blk, dtype):
    got = jagg.relation_bytes(letters, ext, blk, dtype)
    want = O.relation_elems(letters, dict(zip(letters, ext)), dict(zip(letters, blk))) * jagg.ESZ[dtype]
    assert got == want


@pytest.mark.parametrize("letters,ext,blk,dtype", [
    ("sd", (4096, 128), ([0, 1024, 2560, 4096], 1), "bf16"),   # packed sequences (Example 3.10)
    ("ij", (11, 6), ([0, 3, 4, 11], [0, 1, 6]), "f32"),
    ("abc", (7, 5, 6), (2, [0, 2, 5], 3), "f32"),
    ("h", (32,), ([4 * m for m in range(9)],), "bf16"),
])
def test_interval_relation_bytes_match_oracle_geometry(letters, ext, blk, dtype):
    got = jagg.relation_bytes(letters, ext, blk, dtype)
    want = O.relation_elems(letters, dict(zip(letters, ext)), dict(zip(letters, blk))) * jagg.ESZ[dtype]
    assert got == want


def test_interval_relation_bytes_reject_bad_bounds():
    for bnd, status in (([1, 4, 8], -3), ([0, 4, 7], -3), ([0, 4, 4, 8], -3), ([0, 5, 3, 8], -3),
                        (list(range(33)) + [64], -4)):
        with pytest.raises(jagg.JaggError) as e:
            jagg.relation_bytes("a", (max(8, bnd[-1]) if status == -4 else 8,), (bnd,), "f32")
        assert e.value.status == status, bnd


def test_relation_bytes_rejects_bad_blockings():
    with pytest.raises(jagg.JaggError) as e:
        jagg.relation_bytes("a", (10,), (6,), "f32")  # last block empty
    assert e.value.status == -3
    with pytest.raises(jagg.JaggError) as e:
        jagg.relation_bytes("a", (10,), (11,), "f32")
    assert e.value.status == -3
    with pytest.raises(jagg.JaggError) as e:
        jagg.relation_bytes("a", (0,), (1,), "f32")
    assert e.value.status == -2


def test_join_shape_examples_and_3d_counts():
    # Example 3.8 / 3.9: one key of two tuples; two keys of two tuples each
    assert jagg.join_shape("ij,jk->ik", dict(i=256, j=512, k=256), dict(i=1, j=2, k=1)) == (1, 2)
    assert jagg.join_shape("ij,jk->ik", dict(i=256, j=512, k=256), dict(i=2, j=2, k=1)) == (2, 2)
    for a, b, c in [(4, 4, 4), (2, 3, 5), (8, 1, 1)]:
        assert jagg.join_shape("ij,jk->ik", dict(i=64, j=64, k=64), dict(i=a, j=b, k=c)) == (a * c, b)
    assert jagg.join_shape("abcd,cde->abe", dict(a=96, b=300, c=64, d=48, e=1000),
                           dict(a=5, b=7, c=4, d=3, e=6)) == (210, 12)


def test_join_shape_rejects_malformed_spec():
    L = jagg.lib()
    for bad in [b"ij,jk", b"iJ,jk->ik", b"ii,jk->ik", b"ij,jk->iz"]:
        s = jagg.jagg_spec()
        s.einsum = bad
        nk, pk = ctypes.c_int64(), ctypes.c_int64()
        rc = L.jagg_join_shape(ctypes.byref(s), jagg._i64([4, 4, 4]), jagg._i32([1, 1, 1]), ctypes.byref(nk),
                               ctypes.byref(pk))
        assert rc == -1, bad


def test_status_strings():
    L = jagg.lib()
    for code, text in jagg.STATUS.items():
        assert L.jagg_status_str(code).decode() == text


FASTDIV_PROG = r"""
#include <cstdio>
#include <random>
#include "jagg_internal.h"
using namespace jagg;
int main() {
  std::mt19937_64 rng(7);
  const uint32_t ds[] = {1u, 2u, 3u, 7u, 10u, 16u, 43u, 167u, 1000u, 1024u, 8192u, 65535u, 65536u,
                         2147483647u, 2147483648u, 4294967295u};
  long bad = 0;
  for (uint32_t d : ds) {
    FastDiv f = make_fastdiv(d);
    for (int i = 0; i < 200000; ++i) {
      uint32_t n = uint32_t(rng());
      if (i < 100) n = uint32_t(i);
      if (i >= 100 && i < 200) n = 4294967295u - uint32_t(i - 100);
      if (fd_div(n, f) != n / d) ++bad;
    }
  }
  for (int i = 0; i < 200000; ++i) {
    uint32_t d = uint32_t(rng()) | 1u, n = uint32_t(rng());
    if (fd_div(n, make_fastdiv(d)) != n / d) ++bad;
  }
  printf("%ld\n", bad);
  return bad != 0;
}
"""


def test_fastdiv_host_exact(tmp_path):
    """The multiply-high division used by the kernels, compiled for the host
    from the same header, against integer division."""
    src = tmp_path / "fd.cpp"
    src.write_text(FASTDIV_PROG)
    exe = tmp_path / "fd"
    inc = os.path.join(ROOT, "tensor_relational_einsum_amd", "csrc")
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", f"-I{inc}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "0", out.stdout


def test_product_and_oracle_do_not_import_each_other():
    pkg = os.path.join(ROOT, "tensor_relational_einsum_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "liboracle" not in text and "oracle.c" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "tensor_relational_einsum_amd" not in text and "jagg.h" not in text, f


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define JAGG_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m, "JAGG_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == jagg.NOALLOC_SCRATCH_BYTES
