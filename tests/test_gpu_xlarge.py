"""Maximum sizes: tensors of more than 2^31 elements (B*H*n*d), so that the
per-head offsets and output rows past that boundary need 64-bit addressing
in every kernel of the path.

The inputs are a few seeded heads (the workloads' recipes) replicated along
the batch dimension on the device. Each head's result depends on that head's
inputs only and every kernel here is deterministic, so every copy of a head
must reproduce the first copy's result bit for bit; and the copies in the
last batch row, which starts at element 2^31 or later, are compared with the
float64 oracle on sampled rows. Each test needs tens of GB of device memory
(up to about 160 GB for the backward) and is skipped, saying so, where that
much is not free."""
import gc

import numpy as np
import pytest

from tests._support import check_parity, ensure_built, to_device
from tests.test_gpu_backward import check_grads
from tests.test_gpu_decode import check as check_decode, upload
from local_linear_attention_flashlla_amd.workloads import make_cotangent, make_random, make_workload
from oracle import lla_oracle as O
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-3
GiB = 1 << 30


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


@pytest.fixture(autouse=True)
def release(torch):
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def need_free(torch, nbytes):
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes * 1.05:
        pytest.skip(f"needs {nbytes / GiB:.0f} GiB of free device memory, {free / GiB:.0f} GiB free")


def replicate(torch, t, reps):
    """[1, H, n, d] -> [reps, H, n, d], contiguous on the device."""
    return t.expand(reps, *t.shape[1:]).contiguous()


def first_mismatch(torch, t):
    """First batch row of t [B, ...] that differs from row 0 in any bit, or None."""
    ref = t[0:1]
    for b0 in range(1, t.shape[0], 128):
        b1 = min(t.shape[0], b0 + 128)
        if not torch.equal(t[b0:b1], ref.expand(b1 - b0, *ref.shape[1:])):
            for b in range(b0, b1):
                if not torch.equal(t[b], t[0]):
                    return b
    return None


def elements(B, wl):
    return B * wl.H * wl.n * wl.d


def test_forward_matrix_cores_past_2_31_elements(torch):
    # standard recipe, 64 heads of n = 256, d = 128; batch row 1024 starts at
    # element 1024 * 64 * 256 * 128 = 2^31
    wl = make_workload("standard", B=1, H=64, n=256)
    B = 1025
    assert elements(B - 1, wl) == 1 << 31
    ws = lla.workspace_bytes(B, wl.H, wl.n, wl.d, "bf16", lla.LLA_KERNEL_MFMA)
    need_free(torch, elements(B, wl) * (3 * 2 + 4) + ws)
    print(f"\n[case] forward matrix cores B={B} H={wl.H} n={wl.n} d={wl.d} bf16: "
          f"{elements(B, wl) / 2**31:.4f} x 2^31 elements per tensor, workspace "
          f"{ws / GiB:.1f} GiB", flush=True)
    q1, k1, v1 = to_device(wl)
    q, k, v = (replicate(torch, t, B) for t in (q1, k1, v1))
    del q1, k1, v1
    out = lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, kernel=lla.LLA_KERNEL_MFMA)
    torch.cuda.synchronize()
    bad = first_mismatch(torch, out)
    assert bad is None, f"batch row {bad} differs from batch row 0 (same inputs)"
    last = out[B - 1:B].cpu().numpy().astype(np.float64)
    del q, k, v, out
    heads_rows = [((0, h), O.sample_rows(wl.n, seed=h)) for h in (0, 37, 63)]
    stats = check_parity(wl, last, heads_rows, BF16_TOL, label="past 2^31, matrix cores")
    assert stats["rows"] > 0


def test_forward_vector_path_past_2_31_elements(torch):
    # fp32, 64 heads of n = 256, d = 64; batch row 2048 starts at element 2^31
    wl = make_random(1, 64, 256, 64, "f32", seed=21)
    B = 2049
    assert elements(B - 1, wl) == 1 << 31
    need_free(torch, elements(B, wl) * (3 * 4 + 4))
    print(f"\n[case] forward vector path B={B} H={wl.H} n={wl.n} d={wl.d} fp32: "
          f"{elements(B, wl) / 2**31:.4f} x 2^31 elements per tensor", flush=True)
    q1, k1, v1 = to_device(wl)
    q, k, v = (replicate(torch, t, B) for t in (q1, k1, v1))
    del q1, k1, v1
    out = lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, kernel=lla.LLA_KERNEL_VALU)
    torch.cuda.synchronize()
    bad = first_mismatch(torch, out)
    assert bad is None, f"batch row {bad} differs from batch row 0 (same inputs)"
    last = out[B - 1:B].cpu().numpy().astype(np.float64)
    del q, k, v, out
    heads_rows = [((0, h), O.sample_rows(wl.n, seed=h)) for h in (0, 63)]
    stats = check_parity(wl, last, heads_rows, F32_TOL, label="past 2^31, vector path")
    assert stats["rows"] > 0


def test_backward_matrix_cores_past_2_31_elements(torch):
    # standard recipe, 64 heads of n = 256, d = 128, as the forward test above
    wl = make_workload("standard", B=1, H=64, n=256)
    B = 1025
    ne = elements(B, wl)
    ws_f = lla.workspace_bytes(B, wl.H, wl.n, wl.d, "bf16", lla.LLA_KERNEL_MFMA)
    ws_b = lla.backward_workspace_bytes(B, wl.H, wl.n, wl.d, "bf16")
    # q, k, v (bf16); out, rho_c, dout, dq, dk, dv (fp32); one workspace for
    # both calls (the backward's contains the forward's), passed in so that
    # no stream-ordered pool holds a freed forward workspace beside it
    need_free(torch, ne * (3 * 2 + 6 * 4) + max(ws_f, ws_b))
    print(f"\n[case] backward matrix cores B={B} H={wl.H} n={wl.n} d={wl.d} bf16: "
          f"{ne / 2**31:.4f} x 2^31 elements per tensor, workspaces {ws_f / GiB:.1f} + "
          f"{ws_b / GiB:.1f} GiB", flush=True)
    T, tol, lam = wl.cg_max_iters, wl.cg_rel_tol, wl.lam
    g = make_cotangent(1, wl.H, wl.n, wl.d, seed=4)
    q1, k1, v1 = to_device(wl)
    q, k, v = (replicate(torch, t, B) for t in (q1, k1, v1))
    dout = replicate(torch, torch.from_numpy(np.ascontiguousarray(g)).cuda(), B)
    del q1, k1, v1
    rho_c = torch.empty((B, wl.H, wl.n, wl.d), device="cuda")
    ws = torch.empty(max(ws_f, ws_b), dtype=torch.uint8, device="cuda")
    out = lla.forward(q, k, v, lam, T, tol, kernel=lla.LLA_KERNEL_MFMA, rho_c=rho_c, workspace=ws)
    dq, dk, dv = lla.backward(q, k, v, out, dout, rho_c, lam, T, tol, kernel=lla.LLA_KERNEL_MFMA,
                              workspace=ws)
    torch.cuda.synchronize()
    del q, k, v, out, dout, rho_c, ws
    res = {}
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        bad = first_mismatch(torch, t)
        assert bad is None, f"{name}: batch row {bad} differs from batch row 0 (same inputs)"
        res[name] = t[B - 1:B].cpu().numpy().astype(np.float64)
    del dq, dk, dv
    rows = list(O.sample_rows(wl.n, seed=5))
    check_grads(wl, g, res, [(0, 0), (0, 63)], rows, wl.n - 48, T, tol, lam,
                "past 2^31, backward")


def test_decode_past_2_31_cache_elements(torch):
    # standard recipe, 64 caches of n = 264 keys, d = 128; batch rows 993 and
    # later start past element 2^31 of the key and value caches
    wl = make_workload("standard", B=1, H=64, n=264)
    B = 1023
    ne = elements(B, wl)
    assert elements(B - 1, wl) > 1 << 31
    T, tol, lam = wl.cg_max_iters, wl.cg_rel_tol, wl.lam
    ws = lla.decode_workspace_bytes(B, wl.H, wl.n, wl.d, "bf16")
    need_free(torch, ne * 2 * 2 + ws)
    print(f"\n[case] decode B={B} H={wl.H} n={wl.n} d={wl.d} bf16: {ne / 2**31:.4f} x 2^31 "
          f"cache elements, workspace {ws / GiB:.1f} GiB", flush=True)
    q1 = upload(torch, wl.q_dev[:, :, wl.n - 1], "bf16")
    k1, v1 = upload(torch, wl.k_dev, "bf16"), upload(torch, wl.v_dev, "bf16")
    q = q1.expand(B, *q1.shape[1:]).contiguous()
    k, v = replicate(torch, k1, B), replicate(torch, v1, B)
    del q1, k1, v1
    shp = (B, wl.H)
    kw = dict(omega=torch.empty(shp, device="cuda"), rowmax=torch.empty(shp, device="cuda"),
              rho=torch.empty(shp + (wl.d,), device="cuda"),
              cg_iters=torch.empty(shp, dtype=torch.int32, device="cuda"),
              cg_resid=torch.empty(shp, device="cuda"))
    out = lla.decode(q, k, v, lam, T, tol, **kw)
    torch.cuda.synchronize()
    del q, k, v
    res = {}
    for name, t in [("out", out)] + list(kw.items()):
        bad = first_mismatch(torch, t)
        assert bad is None, f"{name}: batch row {bad} differs from batch row 0 (same inputs)"
        res[name] = t[B - 1:B].cpu().numpy()
    res["out"] = res["out"].astype(np.float64)
    check_decode(wl, res, T, tol, lam, "past 2^31")
