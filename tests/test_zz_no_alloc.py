"""dcn4_backward_noalloc, the backward entry point that allocates nothing
(its gathered grad_x takes the library's static 64 MiB device workspace),
against dcn4_backward_ws with a caller-owned workspace, through the C ABI.

Two calls in a row on one GPU, the second on a smaller problem, so the second
runs on the workspace the first left behind.  Each call's grad_offset_mask
equals the _ws entry point's bit for bit (its sums have a fixed order), and
each grad_x lies within the fp32 summation bound of the oracle's (its sums
follow the order in which atomics were granted, as in the _ws entry point),
the bound of the backward tests: (n + 8) * 2^-24 * sum |terms|."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
from oracle import Shape  # noqa: E402
from test_gpu_backward import bwd_inputs, check_bound  # noqa: E402
from test_gpu_parity import desc_of, dev_f32, say, to_dev  # noqa: E402

import dynamic_sparse_vision_dcn4_amd as d4  # noqa: E402

pytestmark = pytest.mark.gpu
SCRATCH = 64 << 20


def ptr(t):
    return None if t is None else t.data_ptr()


def call(plan, s, inp, gy_raw, dt, noalloc):
    x, om, gy = to_dev(inp.x, dt), to_dev(inp.om, dt), to_dev(gy_raw, dt)
    sc = None if inp.scales is None else torch.from_numpy(inp.scales).cuda()
    ps = dev_f32(inp.pscales)
    gx = torch.full((s.N, s.H, s.W, s.C), float("nan"), dtype=torch.float32, device="cuda")
    gom = torch.full(plan.om_shape(), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = d4.dcn4_backward_noalloc(plan.handle, x.data_ptr(), om.data_ptr(), ptr(sc), ptr(ps),
                                      gy.data_ptr(), gx.data_ptr(), gom.data_ptr(), stream)
    else:
        need = plan.backward_workspace_bytes()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        st = d4.dcn4_backward_ws(plan.handle, x.data_ptr(), om.data_ptr(), ptr(sc), ptr(ps),
                                 gy.data_ptr(), gx.data_ptr(), gom.data_ptr(), ws.data_ptr(),
                                 need, stream)
    assert st == d4.DCN4_OK, d4.dcn4_last_error()
    torch.cuda.synchronize()
    return gx.cpu().numpy(), gom.cpu().numpy()


# the larger problem first, then a smaller one (bf16 standard geometry; then
# group scales with predicted scales, fp16)
CASES = [(Shape(2, 30, 28, 64, 4), "bf16"),
         (Shape(1, 13, 11, 48, 2, multiscale=True, pixel_scales=True, max_scale=2.5), "f16")]


def test_noalloc_matches_caller_workspace():
    o = oracle.get()
    for i, (s, dt) in enumerate(CASES):
        plan = d4.Plan(desc_of(s, dt))
        need = plan.backward_workspace_bytes()
        say(f"no-alloc call {i}: {s} {dt}, workspace {need} bytes")
        assert 0 < need <= SCRATCH
        inp, gy = bwd_inputs(s, dt, seed=900 + i)
        ref = o.backward(s, dt, inp.x, inp.om, gy, inp.scales, inp.pscales)
        gx_n, gom_n = call(plan, s, inp, gy, dt, noalloc=True)
        gx_w, gom_w = call(plan, s, inp, gy, dt, noalloc=False)
        check_bound(gx_n, ref["gx"], ref["gx_abs"], ref["max_terms"], f"no-alloc {i} grad_x")
        check_bound(gx_w, ref["gx"], ref["gx_abs"], ref["max_terms"], f"workspace {i} grad_x")
        assert np.array_equal(gom_n.view(np.uint32), gom_w.view(np.uint32)), \
            f"call {i}: grad_offset_mask differs between the entry points"
