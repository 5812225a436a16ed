"""The forward and the backward captured in a HIP graph (torch.cuda.CUDAGraph
around calls of the C ABI on the capturing stream) and replayed several
times, with eager work and synchronisations of the program between the
replays: every replay must reproduce the eager results (the forward and
grad_offset_mask bit for bit; grad_x, summed in no fixed order, within the
fp32 summation bound of the oracle).  The benchmark times its K steps this
way."""
import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle import Shape

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import dynamic_sparse_vision_dcn4_amd as d4  # noqa: E402
from test_gpu_parity import desc_of, fuzz_inputs, to_dev, to_raw_np  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [(Shape(2, 24, 20, 64, 4), "bf16"), (Shape(1, 17, 19, 72, 1, multiscale=True), "bf16"),
         (Shape(2, 12, 12, 32, 2, dh=2, dw=2, ph=2, pw=2), "f16"), (Shape(1, 9, 13, 16, 1), "f32")]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forward_graph_replays(case):
    s, dt = CASES[case]
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    plan = d4.Plan(desc_of(s, dt))
    sets = []
    for r in range(2):
        inp = fuzz_inputs(s, dt, Ho, Wo, seed=900 + 10 * case + r)
        sc = None if inp.scales is None else torch.from_numpy(inp.scales).cuda()
        sets.append((to_dev(inp.x, dt), to_dev(inp.om, dt), sc,
                     torch.empty(plan.out_shape(), dtype=to_dev(inp.x, dt).dtype, device="cuda"),
                     inp))
    eager = [plan.forward(x, om, sc) for x, om, sc, _, _ in sets]
    torch.cuda.synchronize()
    for (x, om, sc, y, inp), ye in zip(sets, eager):
        ref = o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=16)
        assert np.array_equal(to_raw_np(ye, dt), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream().cuda_stream
        for x, om, sc, y, _ in sets:
            plan.forward(x, om, sc, out=y, stream=st)
    say(f"graph case {case}: {s} {dt}")
    for rep in range(4):
        for _, _, _, y, _ in sets:
            y.zero_()                                      # eager work between replays
        other = plan.forward(sets[1][0], sets[0][1], sets[0][2])  # an eager launch too
        if rep % 2:
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, ((_, _, _, y, _), ye) in enumerate(zip(sets, eager)):
            same = torch.equal(y.view(torch.int16 if dt != "f32" else torch.int32),
                               ye.view(torch.int16 if dt != "f32" else torch.int32))
            assert same, f"replay {rep}, set {k}: differs from the eager result"
        del other


def test_backward_graph_replays():
    """dcn4_backward_ws (gathered grad_x, clearing by fill kernels) in a
    graph: grad_offset_mask bit for bit, grad_x within the bound."""
    s, dt = Shape(2, 20, 18, 64, 4), "bf16"
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    plan = d4.Plan(desc_of(s, dt))
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=77)
    rng = np.random.default_rng(78)
    gy_raw = workloads.to_raw(rng.standard_normal((s.N, Ho, Wo, s.C)).astype(np.float32), dt)
    x, om, gy = to_dev(inp.x, dt), to_dev(inp.om, dt), to_dev(gy_raw, dt)
    ws = torch.empty(plan.backward_workspace_bytes(), dtype=torch.uint8, device="cuda")
    gx_e, gom_e = plan.backward(x, om, gy, workspace=ws)
    torch.cuda.synchronize()
    ref = o.backward(s, dt, inp.x, inp.om, gy_raw)
    gx = torch.empty_like(gx_e)
    gom = torch.empty_like(gom_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.backward(x, om, gy, grad_x=gx, grad_om=gom, workspace=ws,
                      stream=torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        gx.fill_(float("nan"))
        gom.zero_()
        if rep == 1:
            plan.backward(x, om, gy, workspace=ws)  # eager use of the same workspace
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gom, gom_e), f"replay {rep}: grad_offset_mask differs"
        got = gx.cpu().numpy().astype(np.float64)
        bound = (ref["max_terms"] + 8) * 2.0 ** -24 * ref["gx_abs"] + 1e-37
        err = np.abs(got - ref["gx"])
        say(f"backward replay {rep}: grad_x largest error / bound "
            f"{float(np.max(err / bound)):.3g}")
        assert np.all(err <= bound), f"replay {rep}: grad_x beyond the bound"
