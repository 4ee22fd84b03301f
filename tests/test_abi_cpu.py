"""The C-ABI library on the CPU: it loads, exports every entry point that
include/et.h declares, and rejects bad arguments before touching the GPU.

No test here launches a kernel: every call below fails host-side validation
(which runs before any HIP call) and passes only fake pointers that are never
dereferenced.  They are skipped where a GPU is visible, so that a validation
bug can never send a fake pointer to a real device; the GPU tests cover the
same paths with real tensors.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "et.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(et_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_ops():
    names = _declared()
    for op in ("rmsnorm", "add_rmsnorm", "rope", "rope_qk", "rmsnorm_rope_qk", "silu_mul", "add",
               "embedding", "argmax", "softmax", "layernorm", "geglu"):
        for sfx in ("f32", "bf16", "f16"):
            assert f"et_{op}_{sfx}" in names
    assert "et_argmax_workspace_bytes" in names and "et_status_string" in names
    assert "et_softmax_workspace_bytes" in names
    assert "et_rope_cache_f32" in names
    for sfx in ("f32", "bf16", "f16"):
        assert f"et_rope_qk_cached_{sfx}" in names
        assert f"et_rope_multi_{sfx}" in names


def test_library_exports_every_declared_symbol():
    import elementwise_transformer_amd as et
    out = subprocess.run(["nm", "-D", "--defined-only", et.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (et_[a-z0-9_]+)$", out, re.M))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        getattr(et.lib, n)          # resolvable through ctypes as well


def test_abi_version_and_status_strings():
    import elementwise_transformer_amd as et
    assert et.abi_version() == 1
    for code in range(7):
        assert et.lib.et_status_string(code).decode()
    assert et.lib.et_status_string(99).decode() == "unknown status"


gpu_visible = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0,
    reason="fake-pointer validation tests run only where no GPU is visible")

P = ctypes.c_void_p
G = 1 << 32          # fake buffers 4 GiB apart, 16-byte aligned, never dereferenced
A = P(1 * G)
B = P(2 * G)
C = P(3 * G)
D = P(4 * G)
E5 = P(5 * G)
NULL = None
S = P(0)             # default stream


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_rmsnorm_validation(sfx):
    import elementwise_transformer_amd as et
    f = getattr(et.lib, f"et_rmsnorm_{sfx}")
    assert f(A, B, C, -1, 8, 1e-5, S) == 2                   # negative rows
    assert f(A, B, C, 4, -8, 1e-5, S) == 2                   # negative d
    assert f(A, B, C, 4, 0, 1e-5, S) == 2                    # empty final axis
    assert f(A, B, C, 1 << 40, 1 << 40, 1e-5, S) == 2        # size product overflows
    assert f(A, B, C, 4, 8, -1.0, S) == 3                    # eps < 0
    assert f(A, B, C, 4, 8, float("nan"), S) == 3
    assert f(A, B, C, 4, 8, float("inf"), S) == 3
    assert f(NULL, B, C, 4, 8, 1e-5, S) == 1
    assert f(A, NULL, C, 4, 8, 1e-5, S) == 1
    assert f(A, B, NULL, 4, 8, 1e-5, S) == 1
    assert f(A, B, P(G + 16), 4, 8, 1e-5, S) == 4           # y overlaps x partially
    assert f(A, B, B, 4, 8, 1e-5, S) == 4                    # y over the gain
    assert f(NULL, NULL, NULL, 0, 8, 1e-5, S) == 0           # rows == 0: no-op


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_add_rmsnorm_validation(sfx):
    import elementwise_transformer_amd as et
    f = getattr(et.lib, f"et_add_rmsnorm_{sfx}")
    assert f(A, NULL, C, D, E5, 4, 8, 1e-5, S) == 1
    assert f(A, B, C, D, NULL, 4, 8, 1e-5, S) == 1
    assert f(A, B, C, D, D, 4, 8, 1e-5, S) == 4              # h == y
    assert f(A, B, C, B, E5, 4, 8, 1e-5, S) == 4    # y == residual
    assert f(A, B, C, A, A, 4, 8, 1e-5, S) == 4              # h == x while y == x
    assert f(A, B, C, D, E5, 4, 8, -2.0, S) == 3


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_rope_validation(sfx):
    import elementwise_transformer_amd as et
    f = getattr(et.lib, f"et_rope_{sfx}")
    assert f(A, B, 4, 2, 8, 3, C, 1.0, 0, S) == 3            # odd d_rot
    assert f(A, B, 4, 2, 8, 10, C, 1.0, 0, S) == 3           # d_rot > D
    assert f(A, B, 4, 2, 8, -2, C, 1.0, 0, S) == 3
    assert f(A, B, 4, 2, 8, 8, C, 1.0, 2, S) == 3            # bad layout
    assert f(A, B, 4, 2, 8, 8, C, float("inf"), 0, S) == 3   # attn_scaling
    assert f(A, B, -4, 2, 8, 8, C, 1.0, 0, S) == 2
    assert f(A, NULL, 4, 2, 8, 8, C, 1.0, 0, S) == 1         # pos
    assert f(A, B, 4, 2, 8, 8, NULL, 1.0, 0, S) == 1         # inv_freq
    assert f(NULL, B, 4, 2, 8, 8, C, 1.0, 0, S) == 1
    assert f(A, P(G + 8), 4, 2, 8, 8, C, 1.0, 0, S) == 4  # pos inside x
    assert f(NULL, NULL, 0, 2, 8, 8, NULL, 1.0, 0, S) == 0   # T == 0
    q = getattr(et.lib, f"et_rope_qk_{sfx}")
    assert q(A, 2, P(G + 16), 2, B, 4, 8, 8, C, 1.0, 0, S) == 4   # q and k overlap
    assert q(A, 2, NULL, 3, B, 4, 8, 8, C, 1.0, 0, S) == 1          # k NULL with Hk > 0


@gpu_visible
def test_rope_cache_validation():
    import elementwise_transformer_amd as et
    f = et.lib.et_rope_cache_f32
    assert f(A, 16, 7, B, C, S) == 3                         # odd d_rot
    assert f(A, -1, 8, B, C, S) == 2
    assert f(A, 16, -2, B, C, S) == 2
    assert f(A, 1 << 31, 8, B, C, S) == 2                    # positions are int32
    assert f(A, 1 << 30, 16, B, C, S) == 2                   # 2^33 entries
    assert f(NULL, 16, 8, B, C, S) == 1
    assert f(A, 16, 8, NULL, C, S) == 1
    assert f(A, 16, 8, B, B, S) == 4                         # cos == sin
    assert f(A, 16, 8, B, P(2 * G + 64), S) == 4             # sin inside cos
    assert f(P(2 * G + 16), 16, 8, B, C, S) == 4             # inv_freq inside cos
    assert f(NULL, 0, 8, NULL, NULL, S) == 0                 # empty cache: no-op


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_rope_cached_validation(sfx):
    import elementwise_transformer_amd as et
    f = getattr(et.lib, f"et_rope_qk_cached_{sfx}")
    # q, Hq, k, Hk, pos, T, D, d_rot, cos, sin, max_pos, mu, layout, stream
    assert f(A, 2, B, 2, C, 4, 8, 8, NULL, E5, 16, 1.0, 0, S) == 1   # cos NULL
    assert f(A, 2, B, 2, C, 4, 8, 8, D, NULL, 16, 1.0, 0, S) == 1    # sin NULL
    assert f(A, 2, B, 2, NULL, 4, 8, 8, D, E5, 16, 1.0, 0, S) == 1   # pos NULL
    assert f(A, 2, B, 2, C, 4, 8, 8, D, E5, -1, 1.0, 0, S) == 2
    assert f(A, 2, B, 2, C, 4, 8, 8, D, E5, 1 << 31, 1.0, 0, S) == 2
    assert f(A, 2, B, 2, C, 4, 8, 7, D, E5, 16, 1.0, 0, S) == 3      # odd d_rot
    assert f(A, 2, B, 2, C, 4, 8, 8, D, E5, 16, 1.0, 5, S) == 3      # bad layout
    assert f(A, 2, B, 2, C, 4, 8, 8, P(G + 64), E5, 16, 1.0, 0, S) == 4   # cos inside q
    assert f(A, 2, B, 2, C, 4, 8, 8, D, P(2 * G + 32), 16, 1.0, 0, S) == 4  # sin inside k
    assert f(NULL, 0, NULL, 0, NULL, 4, 8, 8, NULL, NULL, 0, 1.0, 0, S) == 0  # no heads


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_rope_multi_validation(sfx):
    import elementwise_transformer_amd as et
    f = getattr(et.lib, f"et_rope_multi_{sfx}")

    def dims(*d):
        return ctypes.cast((ctypes.c_int64 * len(d))(*d), P)

    # q, Hq, k, Hk, pos, T, D, n_axes, dims (host), inv_freq, mu, layout, stream
    assert f(A, 2, B, 2, C, 4, 16, 0, dims(4), D, 1.0, 0, S) == 3                 # no axes
    assert f(A, 2, B, 2, C, 4, 16, 9, dims(*[2] * 9), D, 1.0, 0, S) == 3          # more than 8
    assert f(A, 2, B, 2, C, 4, 16, 3, NULL, D, 1.0, 0, S) == 1                    # dims NULL
    assert f(A, 2, B, 2, C, 4, 16, 3, dims(4, 5, 4), D, 1.0, 0, S) == 3           # odd width
    assert f(A, 2, B, 2, C, 4, 16, 2, dims(4, -2), D, 1.0, 0, S) == 3             # negative width
    assert f(A, 2, B, 2, C, 4, 16, 3, dims(8, 6, 4), D, 1.0, 0, S) == 3           # span > D
    assert f(A, 2, B, 2, C, 4, 2048, 2, dims(1100, 900), D, 1.0, 0, S) == 2       # span > 1024
    assert f(A, 2, B, 2, NULL, 4, 16, 3, dims(4, 6, 4), D, 1.0, 0, S) == 1        # pos NULL
    assert f(A, 2, B, 2, C, 4, 16, 3, dims(4, 6, 4), NULL, 1.0, 0, S) == 1        # inv_freq NULL
    assert f(A, 2, B, 2, C, 4, 16, 3, dims(4, 6, 4), D, 1.0, 3, S) == 3           # bad layout
    assert f(A, 2, B, 2, C, 4, 16, 3, dims(4, 6, 4), D, float("nan"), 0, S) == 3  # attn_scaling
    assert f(A, 2, B, 2, P(G + 64), 4, 16, 3, dims(4, 6, 4), D, 1.0, 0, S) == 4   # pos inside q
    assert f(A, 2, P(G + 32), 2, C, 4, 16, 3, dims(4, 6, 4), D, 1.0, 0, S) == 4   # q and k overlap
    assert f(NULL, 0, NULL, 0, NULL, 4, 16, 3, dims(4, 6, 4), NULL, 1.0, 0, S) == 0  # no heads


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_rmsnorm_rope_validation(sfx):
    import elementwise_transformer_amd as et
    f = getattr(et.lib, f"et_rmsnorm_rope_qk_{sfx}")
    assert f(A, NULL, 2, B, C, 2, 1e-6, D, 4, 8, 8, E5, 1.0, 0, S) == 1  # gq
    assert f(A, C, 2, B, NULL, 2, 1e-6, D, 4, 8, 8, E5, 1.0, 0, S) == 1  # gk
    assert f(A, C, 2, B, C, 2, -1.0, D, 4, 8, 8, E5, 1.0, 0, S) == 3     # eps
    assert f(A, C, 2, B, C, 2, 1e-6, D, 4, 8, 7, E5, 1.0, 0, S) == 3     # odd d_rot
    assert f(A, A, 2, B, C, 2, 1e-6, D, 4, 8, 8, E5, 1.0, 0, S) == 4     # gq inside q


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_flat_validation(sfx):
    import elementwise_transformer_amd as et
    for op in ("add", "silu_mul"):
        f = getattr(et.lib, f"et_{op}_{sfx}")
        assert f(A, B, C, -1, S) == 2
        assert f(NULL, B, C, 4, S) == 1
        assert f(A, B, P(G + 4), 64, S) == 4              # y overlaps a partially
        assert f(NULL, NULL, NULL, 0, S) == 0
        assert f(A, B, C, 1 << 62, S) == 2


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_embedding_and_argmax_validation(sfx):
    import elementwise_transformer_amd as et
    e = getattr(et.lib, f"et_embedding_{sfx}")
    assert e(A, 10, B, C, -1, 8, S) == 2
    assert e(A, 10, NULL, C, 4, 8, S) == 1
    assert e(A, 10, B, A, 4, 8, S) == 4                      # out over the table
    assert e(A, 10, B, C, 0, 8, S) == 0
    a = getattr(et.lib, f"et_argmax_{sfx}")
    assert a(A, -1, 8, B, NULL, 0, S) == 2
    assert a(A, 4, 1 << 31, B, NULL, 0, S) == 2               # n > INT32_MAX
    assert a(A, 4, 8, NULL, NULL, 0, S) == 1
    assert a(A, 4, 8, B, NULL, 64, S) == 1                    # NULL workspace, nonzero size
    need = et.argmax_workspace_bytes(4, 128256)
    assert need > 0
    assert a(A, 4, 128256, B, C, need - 1, S) == 5            # workspace too small
    assert a(A, 4, 128256, B, P(3 * G + 8), need, S) == 5     # workspace not 16-byte aligned
    assert a(A, 4, 8, A, NULL, 0, S) == 4                     # out inside x
    assert a(NULL, 0, 8, NULL, NULL, 0, S) == 0


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_softmax_validation(sfx):
    import elementwise_transformer_amd as et
    f = getattr(et.lib, f"et_softmax_{sfx}")
    assert f(A, B, -1, 8, 1.0, NULL, 0, S) == 2
    assert f(A, B, 4, 1 << 31, 1.0, NULL, 0, S) == 2           # n > INT32_MAX
    assert f(A, B, 4, 8, 0.0, NULL, 0, S) == 3                  # temperature must be > 0
    assert f(A, B, 4, 8, -1.0, NULL, 0, S) == 3
    assert f(A, B, 4, 8, float("inf"), NULL, 0, S) == 3
    assert f(A, B, 4, 8, float("nan"), NULL, 0, S) == 3
    assert f(NULL, B, 4, 8, 1.0, NULL, 0, S) == 1
    assert f(A, NULL, 4, 8, 1.0, NULL, 0, S) == 1
    assert f(A, B, 4, 8, 1.0, NULL, 64, S) == 1                 # NULL workspace, nonzero size
    assert f(A, P(G + 4), 4, 8, 1.0, NULL, 0, S) == 4           # y overlaps x partially
    need = et.softmax_workspace_bytes(256, 128256)
    assert f(A, B, 256, 128256, 1.0, C, need - 1, S) == 5       # workspace too small
    assert f(A, B, 256, 128256, 1.0, P(3 * G + 8), need, S) == 5  # not 16-byte aligned
    assert f(A, B, 256, 128256, 1.0, P(G + 64), need, S) == 4   # workspace inside x
    assert f(NULL, NULL, 0, 8, 1.0, NULL, 0, S) == 0
    assert f(A, B, 4, 0, 1.0, NULL, 0, S) == 0


@gpu_visible
def test_softmax_wait_limit_validation():
    """The explicit-wait entry point: the storage code and the limit are
    checked first, then every check of the typed entry points."""
    import elementwise_transformer_amd as et
    f = et.lib.et_softmax_wait_limit
    for code in (0, 1, 2):
        assert f(code, A, B, 4, 8, 1.0, NULL, 0, -1, S) == 3        # limit below 0
        assert f(code, A, B, 4, 8, 1.0, NULL, 0, 65537, S) == 3     # limit above 65536
        assert f(code, A, B, 4, 8, 0.0, NULL, 0, 0, S) == 3         # temperature
        assert f(code, A, B, -1, 8, 1.0, NULL, 0, 0, S) == 2
        assert f(code, NULL, B, 4, 8, 1.0, NULL, 0, 0, S) == 1
        assert f(code, A, P(G + 4), 4, 8, 1.0, NULL, 0, 0, S) == 4
        assert f(code, A, B, 4, 0, 1.0, NULL, 0, 65536, S) == 0
    for code in (-1, 3, 7):
        assert f(code, A, B, 4, 8, 1.0, NULL, 0, 0, S) == 3         # unknown storage


@gpu_visible
@pytest.mark.parametrize("sfx", ["f32", "bf16", "f16"])
def test_layernorm_and_geglu_validation(sfx):
    import elementwise_transformer_amd as et
    f = getattr(et.lib, f"et_layernorm_{sfx}")
    assert f(A, B, C, D, -1, 8, 1e-5, S) == 2
    assert f(A, B, C, D, 4, 0, 1e-5, S) == 2                    # nonempty final axis
    assert f(A, B, C, D, 4, 8, -1.0, S) == 3                    # eps >= 0
    assert f(A, B, C, D, 4, 8, float("nan"), S) == 3
    assert f(NULL, B, C, D, 4, 8, 1e-5, S) == 1
    assert f(A, NULL, C, D, 4, 8, 1e-5, S) == 1
    assert f(A, B, C, P(G + 4), 4, 8, 1e-5, S) == 4             # y overlaps x partially
    assert f(A, B, C, B, 4, 8, 1e-5, S) == 4                    # y over the gain
    assert f(A, B, C, C, 4, 8, 1e-5, S) == 4                    # y over the bias
    assert f(NULL, NULL, NULL, NULL, 0, 8, 1e-5, S) == 0
    g = getattr(et.lib, f"et_geglu_{sfx}")
    assert g(A, B, C, -1, 0, S) == 2
    assert g(A, B, C, 8, 2, S) == 3                             # approximate must be 0 or 1
    assert g(A, B, C, 8, -1, S) == 3
    assert g(NULL, B, C, 8, 1, S) == 1
    assert g(A, B, P(G + 4), 64, 0, S) == 4
    assert g(NULL, NULL, NULL, 0, 1, S) == 0


def test_softmax_workspace_sizes():
    import elementwise_transformer_amd as et
    assert et.softmax_workspace_bytes(0, 100000) == 0
    assert et.softmax_workspace_bytes(256, 32768) == 0           # register path: none needed
    # two counters per row (rounded up to 16 bytes), then (m, s) per 8192-element chunk
    assert et.softmax_workspace_bytes(256, 32769) == 256 * 8 + 256 * 5 * 8
    assert et.softmax_workspace_bytes(256, 128256) == 256 * 8 + 256 * 16 * 8
    assert et.softmax_workspace_bytes(3, 40000) == 32 + 3 * 5 * 8


def test_argmax_workspace_sizes():
    import elementwise_transformer_amd as et
    assert et.argmax_workspace_bytes(0, 100) == 0
    assert et.argmax_workspace_bytes(4, 0) == 0
    assert et.argmax_workspace_bytes(100000, 1000) == 0       # one chunk per row: none needed
    assert et.argmax_workspace_bytes(1024, 128256) == 0       # 1024 rows: one workgroup each
    assert et.argmax_workspace_bytes(1023, 128256) == 1023 * 16  # per row: a 64-bit key and a counter
    assert et.argmax_workspace_bytes(256, 128256) == 256 * 16
    assert et.argmax_workspace_bytes(1, 128256) == 16
    assert et.argmax_workspace_bytes(6, 4096) == 0            # one granule per row: no split


def test_fastdiv_host_logic():
    """Exact division by run-time constants (host side of et_common.hpp),
    compiled as plain host C++ and checked against integer division."""
    src = r'''
#include "et_common.hpp"
#include <cstdio>
#include <cstdint>
int main() {
  const uint32_t divs[] = {1u, 2u, 3u, 5u, 6u, 7u, 8u, 40u, 64u, 72u, 320u, 576u, 1000u, 4096u,
                           65535u, 65536u, 65537u, 1000003u, 2147483647u, 2147483648u, 4294967295u};
  const uint32_t ns[] = {0u, 1u, 2u, 3u, 7u, 8u, 63u, 64u, 65u, 1000u, 65535u, 65536u,
                         2147483647u, 2147483648u, 4294967294u, 4294967295u};
  for (uint32_t d : divs) {
    et::FastDiv f = et::make_fastdiv(d);
    for (uint32_t n : ns) if (et::fdiv(n, f) != n / d) { std::printf("%u/%u\n", n, d); return 1; }
    uint64_t x = 12345;
    for (int k = 0; k < 200000; ++k) {
      x = x * 6364136223846793005ull + 1442695040888963407ull;
      const uint32_t n = static_cast<uint32_t>(x >> 32);
      if (et::fdiv(n, f) != n / d) { std::printf("%u/%u\n", n, d); return 1; }
    }
  }
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "fd.cpp")
        exe = os.path.join(tmp, "fd")
        with open(c, "w") as f:
            f.write(src)
        inc = [f"-I{os.path.join(ROOT, 'include')}",
               f"-I{os.path.join(ROOT, 'elementwise_transformer_amd', 'csrc')}"]
        r = subprocess.run(["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-O2", *inc,
                            c, "-o", exe], capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail(r.stderr[-3000:])
        assert subprocess.run([exe]).returncode == 0


@gpu_visible
def test_stream_probe_validation():
    """The plain-stream probe the benchmark measures against
    (probe/libet_probe.so) rejects bad sizes, stream shapes, vector counts,
    grid sizes, NULL and misaligned buffers before any HIP call."""
    lib = ctypes.CDLL(os.path.join(ROOT, "probe", "libet_probe.so"))
    f = lib.et_probe_stream
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, vp]
    f.restype = ctypes.c_int
    A, B, Y, H = 0x100000, 0x200000, 0x300000, 0x400000   # fake, never dereferenced
    bad = [
        (A, B, Y, H, 0, 1, 1, 4, 0, 0),          # empty
        (A, B, Y, H, 24, 1, 1, 4, 0, 0),         # not whole 16-byte words
        (A, B, Y, H, 1 << 31, 1, 1, 4, 0, 0),    # past 32-bit buffer offsets
        (A, B, Y, H, 64, 0, 0, 4, 0, 0),         # nothing streamed
        (A, B, Y, H, 64, 3, 1, 4, 0, 0),         # three reads
        (A, B, Y, H, 64, 0, 2, 4, 0, 0),         # a shape not offered
        (A, B, Y, H, 64, 2, 0, 4, 0, 0),
        (A, B, Y, H, 64, 1, 1, 5, 0, 0),         # vectors per lane
        (A, B, Y, H, 64, 1, 1, 4, 0, -1),        # persistent grid size
        (A, B, Y, H, 64, 1, 1, 4, 0, 65537),
        (None, B, Y, H, 64, 1, 1, 4, 0, 0),      # missing read buffer
        (A, None, Y, H, 64, 2, 1, 4, 0, 0),
        (A, B, None, H, 64, 1, 0, 4, 0, 0),      # y is needed even for a pure read
        (A, B, Y, None, 64, 2, 2, 4, 1, 0),
        (A + 4, B, Y, H, 64, 1, 1, 4, 0, 0),     # misaligned
        (A, B, Y + 8, H, 64, 1, 1, 8, 1, 2048),
    ]
    for args in bad:
        assert f(*args, None) == 1, args


@gpu_visible
def test_probe_hold_validation():
    """The benchmark's hold kernel (probe/libet_probe.so) rejects times
    outside 1 us .. 100 ms before touching the device."""
    lib = ctypes.CDLL(os.path.join(ROOT, "probe", "libet_probe.so"))
    f = lib.et_probe_hold
    f.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    f.restype = ctypes.c_int
    for bad in (0, -5, 100001, 1 << 40):
        assert f(bad, None) == 1
