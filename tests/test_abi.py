"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments before any device work (these
calls never reach a kernel, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

from tests._support import ensure_built, ROOT
from local_linear_attention_flashlla_amd import _lib

HEADER = os.path.join(ROOT, "include", "lla.h")


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(_lib.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_matches_header(lib):
    m = re.search(r"#define LLA_VERSION (\d+)", open(HEADER).read())
    assert lib.lla_version() == int(m.group(1))


def test_status_strings(lib):
    assert _lib.status_string(0) == "LLA_OK"
    assert _lib.status_string(-1) == "LLA_ERR_INVALID_ARG"
    assert _lib.status_string(-2) == "LLA_ERR_UNSUPPORTED"
    assert _lib.status_string(-3) == "LLA_ERR_HIP"
    assert _lib.status_string(-4) == "LLA_ERR_WORKSPACE"
    assert _lib.status_string(7) == "LLA_ERR_UNKNOWN"


def test_struct_layout_matches_header():
    # 4 ints/ptrs ... the struct must be what the C compiler lays out; check
    # offsets of a few fields that follow padding.
    A = _lib.LlaFwdArgs
    assert A.q.offset == 8 and A.out.offset == 32 and A.B.offset == 40
    assert A.omega.offset == 72 and A.workspace_bytes.offset == 120 and A.kernel.offset == 128
    assert A.ev_main_end.offset == 144 and A.rho_c.offset == 152 and ctypes.sizeof(A) == 160


# Fake, well-aligned device addresses: validation only does pointer arithmetic.
BASE = 0x7F0000000000
GAP = 1 << 32


def _args(**kw):
    a = _lib.LlaFwdArgs()
    a.dtype = kw.get("dtype", _lib.LLA_DTYPE_BF16)
    a.q, a.k, a.v, a.out = BASE, BASE + GAP, BASE + 2 * GAP, BASE + 3 * GAP
    a.B, a.H, a.n, a.d = 2, 3, 100, 64
    a.lambda_ = 1.0
    a.cg_max_iters = 8
    a.cg_rel_tol = 1e-4
    for key, val in kw.items():
        setattr(a, key, val)
    return a


def _call(lib, a):
    return lib.lla_forward_ex(ctypes.byref(a), None)


@pytest.mark.parametrize("field,value,status", [
    ("q", 0, -1), ("k", 0, -1), ("v", 0, -1), ("out", 0, -1),
    ("B", 0, -1), ("H", -1, -1), ("n", 0, -1),
    ("d", 48, -2), ("d", 256, -2), ("d", 0, -2),
    ("n", (1 << 23) + 1, -2),            # one head's key tiles would pass 2 GiB
    ("lambda_", 0.0, -1), ("lambda_", -1.0, -1), ("lambda_", float("nan"), -1),
    ("lambda_", float("inf"), -1),
    ("cg_max_iters", -1, -1), ("cg_max_iters", 100001, -1),
    ("cg_rel_tol", -1e-3, -1), ("cg_rel_tol", float("nan"), -1), ("cg_rel_tol", float("inf"), -1),
    ("dtype", 7, -1), ("kernel", 9, -1), ("flags", 8, -1),
    ("q", BASE + 8, -1),                 # misaligned
    ("out", BASE + GAP + 64, -1),        # overlaps k
    ("rho", BASE + 3 * GAP + 4096, -1),  # overlaps out
    ("rho_c", BASE + 3 * GAP + 4096, -1),  # overlaps out
    ("rho_c", BASE + 6 * GAP + 8, -1),     # misaligned
    ("omega", BASE + 4 * GAP + 4, -1),   # misaligned optional output
])
def test_invalid_arguments_are_rejected_on_the_host(lib, field, value, status):
    a = _args(**{field: value})
    assert _call(lib, a) == status
    assert _lib.last_error() != ""


@pytest.mark.parametrize("B,H,n", [(1 << 16, 1 << 15, 1),     # B*H = 2^31
                                   (1 << 15, 1 << 15, 1025)])  # B*H*n > 2^40
def test_too_many_heads_or_rows_are_unsupported(lib, B, H, n):
    assert _call(lib, _args(B=B, H=H, n=n)) == -2
    assert lib.lla_workspace_bytes(B, H, n, 64, _lib.LLA_DTYPE_BF16, _lib.LLA_KERNEL_MFMA) == 0


def test_workspace_query_respects_the_sequence_limits(lib):
    bf16, mfma, auto = _lib.LLA_DTYPE_BF16, _lib.LLA_KERNEL_MFMA, _lib.LLA_KERNEL_AUTO
    # the matrix-core path takes n <= 2^21; above it the size query reports
    # nothing, and AUTO resolves to the vector path, which needs no workspace
    assert lib.lla_workspace_bytes(1, 1, 1 << 21, 128, bf16, mfma) > 0
    assert lib.lla_workspace_bytes(1, 1, 1 << 21, 128, bf16, auto) > 0
    assert lib.lla_workspace_bytes(1, 1, (1 << 21) + 32, 128, bf16, mfma) == 0
    assert lib.lla_workspace_bytes(1, 1, (1 << 21) + 32, 128, bf16, auto) == 0
    assert lib.lla_workspace_bytes(1, 1, (1 << 23) + 1, 128, bf16, auto) == 0


@pytest.mark.parametrize("kernel", [_lib.LLA_KERNEL_MFMA])
def test_matrix_core_sequence_limit_is_rejected_before_any_device_work(lib, kernel):
    # fake device pointers: a call that got past validation would fault or fail
    # in HIP; this one must come back UNSUPPORTED from the host checks alone
    a = _args(n=(1 << 21) + 32, d=128, B=1, H=1, kernel=kernel)
    assert _call(lib, a) == _lib.LLA_ERR_UNSUPPORTED
    assert "2^21" in _lib.last_error()
    assert _call(lib, _args(n=(1 << 21) + 32, d=64, B=1, H=1, kernel=kernel)) == _lib.LLA_ERR_UNSUPPORTED
    rho_in = ctypes.c_void_p(BASE + 5 * GAP)
    assert lib.lla_output_given_rho(ctypes.byref(a), rho_in, None) == _lib.LLA_ERR_UNSUPPORTED


def test_library_reports_the_hash_of_this_trees_sources(lib):
    from local_linear_attention_flashlla_amd import build
    assert lib.lla_source_hash().decode() == build.source_hash()
    assert _lib.is_current(lib)


@pytest.mark.parametrize("rho_in,kw,status", [
    (0, {}, -1),                                  # NULL rho_in
    (BASE + 5 * GAP + 4, {}, -1),                 # misaligned rho_in
    (BASE + 3 * GAP + 64, {}, -1),                # rho_in overlaps out
    (BASE + 5 * GAP, {"omega": BASE + 5 * GAP + 1024}, -1),  # an output overlaps rho_in
    (BASE + 5 * GAP, {"rho_c": BASE + 6 * GAP}, -1),          # rho_c has no meaning here
    (BASE + 5 * GAP, {"B": 0}, -1),               # the forward's own checks run too
    (BASE + 5 * GAP, {"d": 48}, -2),
])
def test_output_given_rho_rejects_invalid_arguments(lib, rho_in, kw, status):
    a = _args(**kw)
    assert lib.lla_output_given_rho(ctypes.byref(a), ctypes.c_void_p(rho_in), None) == status
    assert _lib.last_error() != ""


def _dargs(**kw):
    a = _lib.LlaDecodeArgs()
    a.dtype = kw.get("dtype", _lib.LLA_DTYPE_BF16)
    a.q, a.k, a.v, a.out = BASE, BASE + GAP, BASE + 2 * GAP, BASE + 3 * GAP
    a.B, a.H, a.n, a.d = 2, 3, 100, 128
    a.lambda_ = 1.0
    a.cg_max_iters = 8
    a.cg_rel_tol = 0.0
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("q", 0, -1), ("k", 0, -1), ("v", 0, -1), ("out", 0, -1),
    ("B", 0, -1), ("n", 0, -1), ("d", 32, -2), ("d", 16, -2),
    ("lambda_", 0.0, -1), ("cg_max_iters", -1, -1), ("cg_rel_tol", float("nan"), -1),
    ("dtype", 5, -1), ("H", 70000, -2),
    ("k", BASE + GAP + 8, -1),            # misaligned
    ("out", BASE + GAP + 512, -1),        # overlaps k
    ("rho", BASE + 3 * GAP + 256, -1),    # overlaps out ([B][H][d] fp32 = 3 KiB)
])
def test_decode_invalid_arguments_are_rejected_on_the_host(lib, field, value, status):
    a = _dargs(**{field: value})
    assert lib.lla_decode_ex(ctypes.byref(a), None) == status
    assert _lib.last_error() != ""


def test_decode_workspace_is_linear_in_n(lib):
    assert lib.lla_decode_workspace_bytes(1, 1, 100, 32, _lib.LLA_DTYPE_BF16) == 0
    # fp32 caches: the score buffer grows with n; the Gram partials do not
    sizes = [lib.lla_decode_workspace_bytes(4, 8, n, 128, _lib.LLA_DTYPE_F32)
             for n in (4096, 8192, 16384)]
    assert all(s > 0 for s in sizes)
    assert sizes[1] - sizes[0] >= 4 * 8 * 4096 * 4 and sizes[2] - sizes[1] >= 4 * 8 * 8192 * 4
    # bf16 caches (one pass over the cache): chunk partials of 4 + 2d + 2d^2
    # floats, at most one chunk per 512 keys and about 256 chunks in all, and
    # with several chunks per head one combined partial per head
    psz = (4 + 2 * 128 + 2 * 128 * 128) * 4
    for bh, n in ((32, 1), (32, 100), (32, 4096), (32, 16384), (256, 4096), (1, 65536)):
        got = lib.lla_decode_workspace_bytes(bh, 1, n, 128, _lib.LLA_DTYPE_BF16)
        per_head = max(1, min(64, 256 // bh, n // 512))
        want = bh * per_head * psz + (bh * psz if per_head > 1 else 0)
        assert want <= got < want + 512, (bh, n, got, want)


def test_null_args_pointer(lib):
    assert lib.lla_forward_ex(None, None) == -1


def test_mfma_kernel_needs_bf16(lib):
    a = _args(dtype=_lib.LLA_DTYPE_F32, kernel=_lib.LLA_KERNEL_MFMA)
    assert _call(lib, a) == -2


def test_too_small_workspace_is_reported(lib):
    need = lib.lla_workspace_bytes(2, 3, 100, 64, _lib.LLA_DTYPE_BF16, _lib.LLA_KERNEL_MFMA)
    if need == 0:
        pytest.skip("MFMA kernel not available in this build")
    a = _args(kernel=_lib.LLA_KERNEL_MFMA, workspace=BASE + 5 * GAP, workspace_bytes=need - 16)
    assert _call(lib, a) == -4


def _nslots(n):
    """Preconditioners per head (include/lla.h): one per prefix length, the
    lengths 32 g' of groups g = 1 .. ceil(n / 32) - 1 (g' = g for g < 8, then
    four lengths per doubling of g)."""
    G = (n + 31) // 32
    if G < 2:
        return 0
    g = G - 1
    if g < 8:
        return g
    e = g.bit_length() - 1
    return 7 + 4 * (e - 3) + (g >> (e - 2)) - 4 + 1


def _pc_bytes(BH, n, d):
    """Workspace bytes of the preconditioners: a d x d matrix in two fp16 terms,
    a float scale and a d-float key sum each (256-byte aligned regions):
    O(d^2 log n) per head."""
    al = lambda x: (x + 255) // 256 * 256
    return al(BH * _nslots(n) * 2 * d * d * 2) + al(BH * _nslots(n) * 4) + al(BH * _nslots(n) * d * 4)


def test_workspace_sizes(lib):
    # the VALU kernel keeps its state on chip
    assert lib.lla_workspace_bytes(1, 1, 256, 16, _lib.LLA_DTYPE_F32, _lib.LLA_KERNEL_VALU) == 0
    assert lib.lla_workspace_bytes(0, 1, 256, 16, _lib.LLA_DTYPE_F32, 0) == 0
    assert lib.lla_workspace_bytes(1, 1, 256, 48, _lib.LLA_DTYPE_F32, 0) == 0
    # when the MFMA kernel is present its workspace grows linearly in n
    sizes = [lib.lla_workspace_bytes(1, 16, n, 128, _lib.LLA_DTYPE_BF16, _lib.LLA_KERNEL_MFMA)
             for n in (1024, 2048, 4096, 8192, 16384)]
    if sizes[0] == 0:
        pytest.skip("MFMA kernel not available in this build")
    pc = [_pc_bytes(16, n, 128) for n in (1024, 2048, 4096, 8192, 16384)]
    assert [_nslots(n) for n in (1024, 2048, 4096, 8192, 16384)] == [15, 19, 23, 27, 31]
    lin = [a - b for a, b in zip(sizes, pc)]
    diffs = [b - a for a, b in zip(lin, lin[1:])]
    # the rest is linear: doubling n adds twice the previous increment
    assert diffs[1] == 2 * diffs[0] and diffs[2] == 2 * diffs[1] and diffs[3] == 2 * diffs[2]


def test_rejected_call_leaves_no_stale_error_after_success_path(lib):
    a = _args(B=0)
    assert _call(lib, a) == -1
    assert "B, H, n" in _lib.last_error()


def _bargs(**kw):
    a = _lib.LlaBwdArgs()
    a.dtype = kw.get("dtype", _lib.LLA_DTYPE_BF16)
    a.q, a.k, a.v = BASE, BASE + GAP, BASE + 2 * GAP
    a.out, a.dout, a.rho_c = BASE + 3 * GAP, BASE + 4 * GAP, BASE + 5 * GAP
    a.dq, a.dk, a.dv = BASE + 6 * GAP, BASE + 7 * GAP, BASE + 8 * GAP
    a.B, a.H, a.n, a.d = 2, 3, 100, 128
    a.lambda_ = 1.0
    a.cg_max_iters = 8
    a.cg_rel_tol = 0.0
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("q", 0, -1), ("dout", 0, -1), ("rho_c", 0, -1), ("dq", 0, -1), ("dk", 0, -1), ("dv", 0, -1),
    ("B", 0, -1), ("n", 0, -1), ("d", 48, -2), ("dtype", 5, -1), ("kernel", 9, -1),
    ("lambda_", float("inf"), -1), ("cg_max_iters", -1, -1), ("cg_rel_tol", -1.0, -1),
    ("n", (1 << 21) + 1, -2),
    ("rho_c", BASE + 5 * GAP + 4, -1),    # misaligned
    ("dk", BASE + 6 * GAP + 1024, -1),    # overlaps dq
    ("dv", BASE + 2 * GAP + 256, -1),     # overlaps v
    ("adj_iters", BASE + 7 * GAP + 16, -1),  # overlaps dk
])
def test_backward_invalid_arguments_are_rejected_on_the_host(lib, field, value, status):
    a = _bargs(**{field: value})
    assert lib.lla_backward_ex(ctypes.byref(a), None) == status
    assert _lib.last_error() != ""
    assert lib.lla_backward_ex(None, None) == -1


@pytest.mark.parametrize("kw", [dict(dtype=_lib.LLA_DTYPE_F32, kernel=_lib.LLA_KERNEL_MFMA),
                                dict(d=32, kernel=_lib.LLA_KERNEL_MFMA)])
def test_backward_matrix_core_path_needs_bf16_and_d_64_or_128(lib, kw):
    a = _bargs(**kw)
    assert lib.lla_backward_ex(ctypes.byref(a), None) == -2


def test_backward_workspace_is_linear_in_n(lib):
    assert lib.lla_backward_workspace_bytes(1, 1, 100, 32, _lib.LLA_DTYPE_BF16) == 0
    assert lib.lla_backward_workspace_bytes(1, 1, 100, 64, _lib.LLA_DTYPE_F32) == 0
    sizes = [lib.lla_backward_workspace_bytes(1, 16, n, 128, _lib.LLA_DTYPE_BF16)
             for n in (1024, 2048, 4096, 8192)]
    assert all(s > 0 for s in sizes)
    lin = [a - _pc_bytes(16, n, 128) for a, n in zip(sizes, (1024, 2048, 4096, 8192))]
    diffs = [b - a for a, b in zip(lin, lin[1:])]
    assert diffs[1] == 2 * diffs[0] and diffs[2] == 2 * diffs[1]
    # and it holds the forward's workspace
    assert sizes[0] > lib.lla_workspace_bytes(1, 16, 1024, 128, _lib.LLA_DTYPE_BF16, _lib.LLA_KERNEL_MFMA)
    a = _bargs(workspace=BASE + 9 * GAP,
               workspace_bytes=lib.lla_backward_workspace_bytes(2, 3, 100, 128, _lib.LLA_DTYPE_BF16) - 16)
    assert lib.lla_backward_ex(ctypes.byref(a), None) == -4


@pytest.mark.parametrize("cname,mirror", [("lla_fwd_args", "LlaFwdArgs"),
                                           ("lla_decode_args", "LlaDecodeArgs"),
                                           ("lla_bwd_args", "LlaBwdArgs")])
def test_struct_layout_matches_c_compiler(tmp_path, cname, mirror):
    """Compile a tiny C program against include/lla.h with the host compiler
    and compare offsetof() of every field with the ctypes mirror."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    M = getattr(_lib, mirror)
    fields = [f[0] for f in M._fields_]
    cfields = ["lambda" if f == "lambda_" else f for f in fields]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("%zu\\n", offsetof({cname}, {f}));' for f in cfields)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "lla.h"\nint main(void){\n'
                   + body + f'\n  printf("%zu\\n", sizeof({cname}));\n  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run([cc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = [getattr(M, f).offset for f in fields] + [ctypes.sizeof(M)]
    assert got == want


def test_noalloc_decode_rejects_a_workspace_and_oversized_calls_on_the_host(lib):
    # fake device pointers: both calls must come back from the host checks
    a = _dargs(workspace=BASE + 7 * GAP, workspace_bytes=1 << 20)
    assert lib.lla_decode_noalloc(ctypes.byref(a), None) == _lib.LLA_ERR_INVALID_ARG
    big = 1 << 40   # room for 64 GiB caches between the fake pointers
    a = _dargs(B=64, H=64, n=65536, d=128, q=BASE, k=BASE + big, v=BASE + 2 * big, out=BASE + 3 * big)
    need = lib.lla_decode_workspace_bytes(64, 64, 65536, 128, _lib.LLA_DTYPE_BF16)
    assert need > _lib.LLA_DECODE_NOALLOC_SCRATCH_BYTES
    assert lib.lla_decode_noalloc(ctypes.byref(a), None) == _lib.LLA_ERR_WORKSPACE
    assert "static scratch" in _lib.last_error()
    assert lib.lla_decode_noalloc(ctypes.byref(_dargs(d=48)), None) == _lib.LLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(kernel=_lib.LLA_KERNEL_VALU), -1), (dict(kernel=_lib.LLA_KERNEL_MFMA), -1),
    (dict(flags=_lib.LLA_FLAG_SPLIT_U), -1),
    (dict(rho_c=BASE + 6 * GAP), -1),
    (dict(n=(1 << 16) + 1), -2),
    (dict(B=256, H=256), -2),               # B*H = 65536 heads: more than the grid holds
    (dict(d=48), -2), (dict(lambda_=0.0), -1), (dict(q=0), -1),
    (dict(out=BASE + GAP + 64), -1),        # overlaps k
])
def test_naive_forward_rejects_invalid_arguments_on_the_host(lib, kw, status):
    a = _args(**kw)
    assert lib.lla_forward_naive(ctypes.byref(a), None) == status
    assert _lib.last_error() != ""


def test_naive_workspace_holds_the_pairwise_differences_and_moment_matrices(lib):
    # z_ij (BH n^2 d), w_ij (BH n^2), Sigma_i (BH n d^2), mu_i and rho_i
    # (BH n d each), omega_i and the row max (BH n each), in fp32, each region
    # 256-byte aligned
    al = lambda x: (x + 255) // 256 * 256
    for B, H, n, d in [(1, 1, 1, 16), (2, 3, 100, 64), (1, 16, 1024, 128), (1, 1, 4096, 128)]:
        r = B * H * n
        want = (al(4 * r * n * d) + al(4 * r * n) + al(4 * r * d * d) + 2 * al(4 * r * d)
                + 2 * al(4 * r))
        assert lib.lla_naive_workspace_bytes(B, H, n, d, _lib.LLA_DTYPE_BF16) == want
    # quadratic in n, against the linear workspace of the blocked forward
    w1 = lib.lla_naive_workspace_bytes(1, 16, 2048, 128, _lib.LLA_DTYPE_BF16)
    w2 = lib.lla_naive_workspace_bytes(1, 16, 4096, 128, _lib.LLA_DTYPE_BF16)
    assert 3.8 < w2 / w1 < 4.0   # the n^2 d term dominates; Sigma_i grows as n d^2
    assert lib.lla_naive_workspace_bytes(1, 1, (1 << 16) + 1, 16, _lib.LLA_DTYPE_F32) == 0
    assert lib.lla_naive_workspace_bytes(256, 256, 16, 16, _lib.LLA_DTYPE_F32) == 0
    assert lib.lla_naive_workspace_bytes(1, 1, 16, 48, _lib.LLA_DTYPE_F32) == 0
