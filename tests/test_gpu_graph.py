"""Every entry point under HIP graph capture (torch.cuda.graph, which captures
the library's launches on torch's current stream): with a caller workspace
the library makes no allocation, memset or synchronisation, so the captured
launches are the whole call. Each graph is replayed several times with other
eager work and synchronisations in between, and every replay must give the
eager call's result: bit for bit where the kernels are deterministic, to
rounding where the vector backward adds dk and dv with atomics."""
import numpy as np
import pytest

from tests._support import ensure_built, to_device
from local_linear_attention_flashlla_amd.workloads import make_cotangent, make_random, make_workload
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def workspace(torch, nbytes):
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")


def replay_and_compare(torch, g, outputs, expected, label, exact=True):
    """Replay g REPLAYS times; after each, compare outputs with expected."""
    noise = torch.randn(1 << 20, device="cuda")
    for r in range(REPLAYS):
        for t in outputs:
            t.fill_(float("nan"))          # a replay must rewrite every element
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outputs, expected):
            if exact:
                assert torch.equal(t, e), f"{label}: replay {r} differs from the eager call"
            else:
                err = ((t - e).abs().max() / e.abs().max()).item()
                assert err <= 1e-6, f"{label}: replay {r} differs by {err:.2e}"
        noise.mul_(1.0001).add_(0.5)       # unrelated eager work between replays
        torch.cuda.synchronize()
    print(f"[graph] {label}: {REPLAYS} replays match the eager call", flush=True)


def capture(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # warm-up off the capture, as torch advises
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kernel", [lla.LLA_KERNEL_MFMA, lla.LLA_KERNEL_VALU])
def test_forward_under_graph_capture(torch, kernel):
    wl = make_workload("standard", B=1, H=4, n=600)
    print(f"\n[case] forward graph kernel={kernel} B={wl.B} H={wl.H} n={wl.n} d={wl.d}", flush=True)
    q, k, v = to_device(wl)
    shape = (wl.B, wl.H, wl.n, wl.d)
    ws = workspace(torch, lla.workspace_bytes(wl.B, wl.H, wl.n, wl.d, "bf16", kernel))
    out = torch.empty(shape, device="cuda")
    rho_c = torch.empty(shape, device="cuda")
    iters = torch.empty(shape[:3], dtype=torch.int32, device="cuda")

    def call():
        lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, rho_c=rho_c,
                    cg_iters=iters, workspace=ws, kernel=kernel)

    call()
    torch.cuda.synchronize()
    expected = [out.clone(), rho_c.clone(), iters.clone()]
    g = capture(torch, call)
    replay_and_compare(torch, g, [out, rho_c], expected[:2], f"forward kernel={kernel}")
    assert torch.equal(iters, expected[2])


@pytest.mark.parametrize("kernel", [lla.LLA_KERNEL_MFMA, lla.LLA_KERNEL_VALU])
def test_backward_under_graph_capture(torch, kernel):
    wl = make_workload("standard", B=1, H=2, n=300)
    print(f"\n[case] backward graph kernel={kernel} B={wl.B} H={wl.H} n={wl.n} d={wl.d}", flush=True)
    q, k, v = to_device(wl)
    shape = (wl.B, wl.H, wl.n, wl.d)
    T, tol, lam = wl.cg_max_iters, wl.cg_rel_tol, wl.lam
    rho_c = torch.empty(shape, device="cuda")
    out = lla.forward(q, k, v, lam, T, tol, kernel=kernel, rho_c=rho_c)
    dout = torch.from_numpy(np.ascontiguousarray(make_cotangent(*shape, seed=9))).cuda()
    ws = workspace(torch, lla.backward_workspace_bytes(*shape, "bf16") if kernel == lla.LLA_KERNEL_MFMA else 0)
    dq, dk, dv = (torch.empty(shape, device="cuda") for _ in range(3))

    def call():
        lla.backward(q, k, v, out, dout, rho_c, lam, T, tol, dq=dq, dk=dk, dv=dv, workspace=ws,
                     kernel=kernel)

    call()
    torch.cuda.synchronize()
    expected = [dq.clone(), dk.clone(), dv.clone()]
    g = capture(torch, call)
    replay_and_compare(torch, g, [dq, dk, dv], expected, f"backward kernel={kernel}",
                       exact=kernel == lla.LLA_KERNEL_MFMA)


def test_decode_under_graph_capture(torch):
    wl = make_random(2, 3, 700, 128, "bf16", seed=41, qk_scale=4.0)
    print(f"\n[case] decode graph B={wl.B} H={wl.H} n={wl.n} d={wl.d}", flush=True)
    n = wl.n
    cast = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    q, k, v = cast(wl.q_dev[:, :, n - 1]), cast(wl.k_dev), cast(wl.v_dev)
    ws = workspace(torch, lla.decode_workspace_bytes(wl.B, wl.H, n, wl.d, "bf16"))
    out = torch.empty((wl.B, wl.H, wl.d), device="cuda")

    def call():
        lla.decode(q, k, v, 1.0, 16, 0.0, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    expected = [out.clone()]
    g = capture(torch, call)
    replay_and_compare(torch, g, [out], expected, "decode")
