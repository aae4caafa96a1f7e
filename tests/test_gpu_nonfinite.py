"""Non-finite inputs are not checked; they propagate, within bounds. Every
head is computed from its own inputs only. Within a head, a NaN query row
reaches only its own output row; a NaN key or value at position j reaches the
rows from 32 floor(j / 32) on, because the diagonal tile is computed for a
whole 32-query group at once and a masked weight of 0 times a NaN operand is
NaN. These tests plant a NaN and check that everything outside those bounds
is unchanged, bit for bit where the kernels are deterministic (the vector
backward adds dk and dv with atomics: to rounding there). Every loop in the
kernels is bounded by a size or the CG cap, so a NaN ends iterations instead
of extending them."""
import numpy as np
import pytest

from tests._support import ensure_built
from local_linear_attention_flashlla_amd.workloads import make_cotangent, make_random
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

MFMA, VALU = lla.LLA_KERNEL_MFMA, lla.LLA_KERNEL_VALU


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def inputs(torch, dtype, d, seed=3):
    wl = make_random(1, 3, 100, d, dtype, seed=seed, qk_scale=4.0)
    if dtype == "f32":
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    else:
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return wl, [up(a) for a in (wl.q_dev, wl.k_dev, wl.v_dev)]


def same(torch, a, b):
    return torch.equal(a, b)


@pytest.mark.parametrize("kernel,dtype,d", [(MFMA, "bf16", 64), (VALU, "f32", 32)])
def test_forward_nan_stays_in_its_rows(torch, kernel, dtype, d):
    print(f"\n[case] forward NaN kernel={kernel} dtype={dtype} d={d}", flush=True)
    wl, (q, k, v) = inputs(torch, dtype, d)
    run = lambda q, k, v: lla.forward(q, k, v, 1.0, 16, 0.0, kernel=kernel)
    clean = run(q, k, v)
    # a NaN in query row 40 of head 1: only that output row may change
    qn = q.clone()
    qn[0, 1, 40, 5] = float("nan")
    out = run(qn, k, v)
    torch.cuda.synchronize()
    keep = torch.ones(wl.n, dtype=torch.bool, device="cuda")
    keep[40] = False
    assert same(torch, out[0, 0], clean[0, 0]) and same(torch, out[0, 2], clean[0, 2])
    assert same(torch, out[0, 1][keep], clean[0, 1][keep])
    # a NaN in key 70 of head 2: the rows before its 32-row group (0..63) and
    # the other heads unchanged
    kn = k.clone()
    kn[0, 2, 70, 3] = float("nan")
    out = run(q, kn, v)
    torch.cuda.synchronize()
    assert same(torch, out[0, :2], clean[0, :2])
    assert same(torch, out[0, 2, :64], clean[0, 2, :64])
    bad = int((~torch.isfinite(out[0, 2, 70:])).any(dim=-1).sum())
    print(f"[nonfinite] kernel={kernel}: rows 70.. of the head with the NaN key: {bad} of 30 not finite",
          flush=True)


def test_decode_nan_stays_in_its_head(torch):
    print("\n[case] decode NaN", flush=True)
    wl, (q, k, v) = inputs(torch, "bf16", 128)
    q1 = q[:, :, wl.n - 1].contiguous()
    clean = lla.decode(q1, k, v, 1.0, 16, 0.0)
    vn = v.clone()
    vn[0, 1, 10, 0] = float("nan")
    out = lla.decode(q1, k, vn, 1.0, 16, 0.0)
    torch.cuda.synchronize()
    assert same(torch, out[0, 0], clean[0, 0]) and same(torch, out[0, 2], clean[0, 2])


@pytest.mark.parametrize("kernel,dtype,d", [(MFMA, "bf16", 64), (VALU, "f32", 32)])
def test_backward_nan_stays_in_its_head(torch, kernel, dtype, d):
    print(f"\n[case] backward NaN kernel={kernel} dtype={dtype} d={d}", flush=True)
    wl, (q, k, v) = inputs(torch, dtype, d)
    shape = (1, 3, wl.n, d)
    rho_c = torch.empty(shape, device="cuda")
    out = lla.forward(q, k, v, 1.0, 16, 0.0, kernel=kernel, rho_c=rho_c)
    g = torch.from_numpy(make_cotangent(*shape, seed=5)).cuda()
    clean = lla.backward(q, k, v, out, g, rho_c, 1.0, 16, 0.0, kernel=kernel)
    gn = g.clone()
    gn[0, 1, 50, 2] = float("nan")
    grads = lla.backward(q, k, v, out, gn, rho_c, 1.0, 16, 0.0, kernel=kernel)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), grads, clean):
        for h in (0, 2):
            if kernel == MFMA:
                assert same(torch, a[0, h], b[0, h]), f"{name} of head {h} changed"
            else:
                err = ((a[0, h] - b[0, h]).abs().max() / b[0, h].abs().max()).item()
                assert err <= 1e-6, f"{name} of head {h} changed by {err:.2e}"
