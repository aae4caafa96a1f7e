"""lla_decode_noalloc, the decode entry point for callers that cannot
allocate: its output must equal lla_decode_ex's (same kernels, same scratch
layout, no atomics: bit for bit) on two calls in a row, the second smaller
than the first, so that the second reads a static scratch the first left
full. Also checked against the float64 oracle's last row on the small call."""
import numpy as np
import pytest

from tests._support import ensure_built, row_errors, oracle_rows
from local_linear_attention_flashlla_amd.workloads import make_workload, make_random
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def _caches(torch, wl, B=None):
    """q = the last query of each head, k/v = the whole caches."""
    def up(a):
        if wl.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    q = up(wl.q_dev[:, :, wl.n - 1])
    return q, up(wl.k_dev), up(wl.v_dev)


def _both(torch, wl):
    q, k, v = _caches(torch, wl)
    B, H = wl.B, wl.H
    need = lla.decode_workspace_bytes(B, H, wl.n, wl.d, wl.dtype)
    assert 0 < need <= lla._lib.LLA_DECODE_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref = lla.decode(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, workspace=ws)
    out = torch.full((B, H, wl.d), float("nan"), device="cuda")
    it = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
    it_ref = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
    lla.decode(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, cg_iters=it, noalloc=True)
    lla.decode(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, cg_iters=it_ref, workspace=ws)
    torch.cuda.synchronize()
    return out, ref, it, it_ref


def test_noalloc_decode_matches_decode_ex_on_two_calls(torch):
    # first call: the standard caches (B=4, H=8, n=4096, d=128, bf16)
    big = make_workload("standard")
    print(f"\n[case] noalloc decode, call 1: B={big.B} H={big.H} n={big.n} d={big.d} {big.dtype}", flush=True)
    out, ref, it, it_ref = _both(torch, big)
    assert torch.equal(out, ref) and torch.equal(it, it_ref)
    # second call, smaller and of another shape and dtype: B=1, H=3, n=700, d=64, fp32
    small = make_random(1, 3, 700, 64, "f32", seed=31, qk_scale=2.0)
    print(f"[case] noalloc decode, call 2: B=1 H=3 n=700 d=64 f32", flush=True)
    out, ref, it, it_ref = _both(torch, small)
    assert torch.equal(out, ref) and torch.equal(it, it_ref)
    ex = oracle_rows(small, [((0, h), [small.n - 1]) for h in range(small.H)])
    e = np.array([row_errors(out.cpu().numpy()[0, h][None].astype(np.float64), x["b"])[0]
                  for h, x in enumerate(ex)])
    print(f"[parity] noalloc decode small call vs exact oracle: max {e.max():.2e}", flush=True)
    assert e.max() <= 1e-3
