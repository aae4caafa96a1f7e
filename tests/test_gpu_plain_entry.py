"""The two plain entry points of the C ABI, called directly through ctypes
with the argument list of the requested signature
lla_forward(q, k, v, out, B, H, n, d, lambda, cg_max_iters, cg_rel_tol, stream):
lla_forward_f32 on the fp32 tiny workload (every row) and lla_forward_bf16 on
the standard workload's recipe, against the float64 oracle, and bit for bit
against lla_forward_ex with default arguments."""
import ctypes

import numpy as np
import pytest

from tests._support import check_parity, ensure_built, to_device
from local_linear_attention_flashlla_amd.workloads import make_workload
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


@pytest.mark.parametrize("name,n,tol", [("tiny", 256, 1e-3), ("standard", 300, 2e-2)])
def test_plain_entry_point(torch, name, n, tol):
    wl = make_workload(name, B=1, H=2, n=n)
    print(f"\n[case] plain entry {name} n={n} dtype={wl.dtype}", flush=True)
    lib = ensure_built()
    q, k, v = to_device(wl)
    out = torch.empty((wl.B, wl.H, wl.n, wl.d), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fn = lib.lla_forward_f32 if wl.dtype == "f32" else lib.lla_forward_bf16
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), wl.B, wl.H, wl.n, wl.d,
            ctypes.c_float(wl.lam), wl.cg_max_iters, ctypes.c_float(wl.cg_rel_tol), stream)
    assert st == 0, lla._lib.last_error()
    ref = lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    heads_rows = [((0, h), range(wl.n)) for h in range(wl.H)]
    check_parity(wl, out.cpu().numpy().astype(np.float64), heads_rows, tol,
                 label=f"plain entry {name}-{n}")
