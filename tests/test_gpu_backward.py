"""Parity of the HIP backward pass (dcn4_backward_ws / dcn4_backward) with the
oracle's.

grad_x is summed in fp32 in no fixed order -- gathered from per-cell buckets
(the default, with a workspace) or scattered with fp32 atomics (no
workspace) -- and grad_offset_mask with fp32 sums in the kernel's order,
while the oracle sums in fp64 (with the same sampling decisions as the fp32
forward).  The tolerance is the fp32
summation bound: for an output with terms t_i (at most n of them per output),
|gpu - oracle| <= (n + 8) * 2^-24 * sum_i |t_i|, the sum of absolute terms
coming from the oracle (n + 8 covers the n additions and the few roundings
of each product).  The bound is checked on every element."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import workloads  # noqa: E402
from oracle import Shape  # noqa: E402
from test_gpu_parity import (NTHREADS, desc_of, dev_f32, say, shape_of,  # noqa: E402
                             to_dev)
from workloads import WORKLOADS, make_inputs, to_raw  # noqa: E402

import dynamic_sparse_vision_dcn4_amd as d4  # noqa: E402

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def check_bound(got, want, absum, n_terms, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    bound = (n_terms + 8) * U * absum + 1e-37
    ratio = float(np.max(err / bound)) if err.size else 0.0
    bad = ~(err <= bound)
    say(f"{what}: max |gpu - oracle| / bound = {ratio:.3g} over {err.size} elements")
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the fp32 bound; "
                           f"first at {np.argwhere(bad)[:3].tolist()}")


def run_backward(plan, inp, gy_raw, dt, want_x=True, want_om=True, scatter=False):
    x = to_dev(inp.x, dt)
    om = to_dev(inp.om, dt)
    gy = to_dev(gy_raw, dt)
    sc = None if inp.scales is None else torch.from_numpy(inp.scales).cuda()
    gx, gom = plan.backward(x, om, gy, sc, dev_f32(inp.pscales), want_x=want_x,
                            want_om=want_om, scatter=scatter)
    torch.cuda.synchronize()
    return (None if gx is None else gx.cpu().numpy(),
            None if gom is None else gom.cpu().numpy())


def compare(s, dt, inp, gy_raw, plan, what, paths=("gather",)):
    o = oracle.get()
    ref = o.backward(s, dt, inp.x, inp.om, gy_raw, inp.scales, inp.pscales)
    for path in paths:
        gx, gom = run_backward(plan, inp, gy_raw, dt, scatter=path == "scatter")
        check_bound(gx, ref["gx"], ref["gx_abs"], ref["max_terms"], f"{what} {path} grad_x")
        check_bound(gom, ref["gom"], ref["gom_abs"], ref["max_terms"], f"{what} {path} grad_om")
    return gx, gom


def bwd_cases():
    rng = np.random.default_rng(4321)
    cases = []
    kernels = [(3, 3), (3, 3), (1, 1), (5, 5), (3, 5), (2, 2)]
    for t in range(18):
        dt = ["bf16", "f32", "f16"][t % 3]
        mode = ["std", "std", "scaled", "ms", "ps"][t % 5]
        kh, kw = kernels[int(rng.integers(len(kernels)))]
        if mode in ("ms", "ps") and (kh % 2 == 0 or kw % 2 == 0):
            kh, kw = 3, 3
        D = int(rng.choice([16, 24, 10, 72, 4, 32, 8]))
        G = int(rng.integers(1, 4))
        ms = mode in ("ms", "ps")
        sh, sw = (1, 1) if ms else (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        dh, dw = (1, 1) if ms else (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        s = Shape(int(rng.integers(1, 3)), int(rng.integers(5, 24)), int(rng.integers(5, 24)),
                  G * D, G, kh, kw, sh, sw, int(rng.integers(0, 3)), int(rng.integers(0, 3)),
                  dh, dw, 0.5 if mode == "scaled" else 1.0, ms, mode == "ps",
                  2.5 if mode == "ps" else 0.0)
        try:
            oracle.get().out_size(s)
        except ValueError:
            continue
        cases.append((t, s, dt))
    return cases


def bwd_inputs(s, dt, seed, off_range=3.0):
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    rng = np.random.default_rng(seed)
    K = s.K
    x = rng.standard_normal((s.N, s.H, s.W, s.C)).astype(np.float32)
    off = rng.uniform(-off_range, off_range, (s.N, Ho, Wo, s.G, 2 * K)).astype(np.float32)
    m = (rng.standard_normal((s.N, Ho, Wo, s.G, K)) / 3).astype(np.float32)
    scales = rng.uniform(0.5, 3.0, s.G).astype(np.float32) if s.multiscale else None
    ps = rng.uniform(0.5, 1.5, (s.N, Ho, Wo, s.G)).astype(np.float32) if s.pixel_scales else None
    gy = rng.standard_normal((s.N, Ho, Wo, s.C)).astype(np.float32)
    inp = workloads.Inputs(to_raw(x, dt), to_raw(np.concatenate([off, m], -1), dt), scales, ps)
    return inp, to_raw(gy, dt)


@pytest.mark.parametrize("t, s, dt", bwd_cases(), ids=lambda v: str(v) if isinstance(v, int) else None)
def test_backward_parity(t, s, dt):
    """Both grad_x paths: gathered (workspace) and scattered (atomics)."""
    inp, gy = bwd_inputs(s, dt, seed=t)
    plan = d4.Plan(desc_of(s, dt))
    say(f"backward case {t}: {s} {dt}")
    compare(s, dt, inp, gy, plan, f"backward {t}", paths=("gather", "scatter"))


@pytest.mark.parametrize("name", ["ldm_unet_block_bf16", "flowdcn_pixelscale_bf16"])
def test_backward_full_size(name):
    """The headline block and FlowDCN's tokens with predicted scales, every
    output element against the fp64 oracle."""
    w = WORKLOADS[name]
    s = shape_of(w)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = make_inputs(w, Ho, Wo)
    rng = np.random.default_rng(11)
    gy = to_raw(rng.standard_normal((s.N, Ho, Wo, s.C), dtype=np.float32), w.dtype)
    say(f"backward full size: {w.describe()}")
    compare(s, w.dtype, inp, gy, d4.Plan(desc_of(s, w.dtype)), name,
            paths=("gather", "scatter"))


def test_backward_reproducible_and_partial():
    """grad_offset_mask is bit-reproducible (no atomics) on each path: the
    direct kernel (a call that scatters grad_x) and the tiled one (a call
    that gathers grad_x, or asks for no grad_x: the same kernel, so the same
    bits); each gradient can be asked for alone and stays within the bound."""
    s = Shape(2, 19, 23, 64, 4)
    dt = "bf16"
    inp, gy = bwd_inputs(s, dt, seed=99)
    plan = d4.Plan(desc_of(s, dt))
    assert plan.info()["backward_kernel"] == 2
    ref = oracle.get().backward(s, dt, inp.x, inp.om, gy)
    gx1, gom1 = run_backward(plan, inp, gy, dt, scatter=True)
    gx2, gom2 = run_backward(plan, inp, gy, dt, scatter=True)
    assert np.array_equal(gom1.view(np.uint32), gom2.view(np.uint32))
    gx3, gom3 = run_backward(plan, inp, gy, dt)
    _, gom4 = run_backward(plan, inp, gy, dt, want_x=False)
    assert np.array_equal(gom3.view(np.uint32), gom4.view(np.uint32))
    gx5, _ = run_backward(plan, inp, gy, dt, want_om=False)
    gx6, _ = run_backward(plan, inp, gy, dt, want_om=False, scatter=True)
    for g in (gom1, gom3):
        check_bound(g, ref["gom"], ref["gom_abs"], ref["max_terms"], "grad_om repeat")
    for g in (gx1, gx2, gx3, gx5, gx6):
        check_bound(g, ref["gx"], ref["gx_abs"], ref["max_terms"], "grad_x repeat")


def test_backward_empty_batch():
    p0 = d4.Plan(d4.Desc(0, 8, 8, 16, 1))
    assert d4.dcn4_backward(p0.handle, None, None, None, None, None, None, None, None) == d4.DCN4_OK


TILED_BWD = [
    # (shape, dtype, plan options, margins)
    (Shape(2, 21, 27, 32, 2), "bf16", {}, (0, 1, 4)),
    (Shape(1, 19, 33, 64, 2), "f16", {}, (0, 1, 4)),             # D=32: 2 lanes per group
    (Shape(2, 17, 22, 32, 2), "f32", {}, (0, 1, 4)),             # fp32: 8 channels per lane
    (Shape(1, 18, 20, 32, 2), "f32", {"channels_per_lane": 4}, (0, 1, 4)),  # 4 lanes per group
    (Shape(2, 23, 19, 32, 4), "bf16", {}, (0, 1, 4)),            # D=8: one vector per lane
    (Shape(1, 25, 31, 64, 4, dh=2, dw=2, ph=2, pw=2), "bf16", {}, (0, 1, 4)),  # dilation 2
    (Shape(1, 27, 23, 64, 4, sh=2, sw=2), "bf16", {}, (0, 1, 4)),  # stride 2
    (Shape(1, 20, 24, 64, 4, offset_scale=0.5), "f16", {}, (0, 1, 4)),
    (Shape(1, 22, 26, 128, 8), "bf16", {"tile_groups": 2}, (0, 1, 4)),
    (Shape(1, 18, 18, 32, 2, multiscale=True), "bf16", {}, (0, 1, 4)),  # group scales
    (Shape(1, 18, 20, 32, 2, multiscale=True, pixel_scales=True, max_scale=2.5), "f16", {},
     (0, 4)),                                                     # predicted scales, Smax
    (Shape(1, 13, 15, 144, 2, multiscale=True), "bf16", {}, (0, 1, 4)),  # D=72: 3 slices
    (Shape(2, 12, 14, 144, 2), "bf16", {}, (1, 4)),               # slices, standard geometry
    (Shape(1, 20, 24, 64, 4), "bf16", {}, (16,)),             # margin 16: 2 slices of 8
    # the whole-image window (samples off the image read window cell (0, 0)
    # and are zeroed)
    (Shape(2, 21, 27, 32, 2), "bf16", {"tile_window": 2}, (4,)),
    (Shape(2, 17, 22, 32, 2), "f32", {"tile_window": 2}, (4,)),
    (Shape(1, 18, 18, 32, 2, multiscale=True, pixel_scales=True, max_scale=2.5), "bf16",
     {"tile_window": 2}, (4,)),
    (Shape(1, 13, 15, 144, 2, multiscale=True), "bf16", {"tile_window": 2}, (4,)),
]
TILED_BWD_CASES = [(c, m) for c, (_, _, _, ms) in enumerate(TILED_BWD) for m in ms]


@pytest.mark.parametrize("case, margin", TILED_BWD_CASES)
def test_tiled_backward(case, margin):
    """The tiled backward (offset/weight gradients from the LDS window, for
    calls without grad_x or with a gathered one) against the oracle; margin 0
    sends every wave to the global path, 1 mixes the paths.  The same plan
    scattering grad_x runs the direct kernel for both gradients, which must
    agree within the bound too."""
    s, dt, opts, _ = TILED_BWD[case]
    inp, gy = bwd_inputs(s, dt, seed=500 + case)
    dp = opts.get("channels_per_lane", 0)
    rest = {k: v for k, v in opts.items() if k != "channels_per_lane"}
    rest.setdefault("tile_window", 1)  # the margin window unless the case asks otherwise
    plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp, tile_margin=margin, **rest)
    info = plan.info()
    say(f"tiled backward {case} margin {margin}: {s} {dt} {info}")
    assert info["backward_kernel"] == 2
    ref = oracle.get().backward(s, dt, inp.x, inp.om, gy, inp.scales, inp.pscales)
    _, gom = run_backward(plan, inp, gy, dt, want_x=False)
    check_bound(gom, ref["gom"], ref["gom_abs"], ref["max_terms"], f"tiled grad_om {case} m{margin}")
    if info["tile_om_unit"] == 1:
        # the rows read into registers (16-bit rows of one group) and staged
        # in LDS give the same bits
        staged = d4.Plan(desc_of(s, dt), channels_per_lane=dp, tile_margin=margin,
                         tile_om_unit=4, **rest)
        assert staged.info()["tile_om_unit"] == 4
        _, gom_s = run_backward(staged, inp, gy, dt, want_x=False)
        assert np.array_equal(gom.view(np.uint32), gom_s.view(np.uint32))
    gxg, gom_g = run_backward(plan, inp, gy, dt)
    assert np.array_equal(gom.view(np.uint32), gom_g.view(np.uint32))
    check_bound(gxg, ref["gx"], ref["gx_abs"], ref["max_terms"], f"gathered grad_x {case} m{margin}")
    gx, gom_d = run_backward(plan, inp, gy, dt, scatter=True)
    check_bound(gx, ref["gx"], ref["gx_abs"], ref["max_terms"], f"direct grad_x {case} m{margin}")
    check_bound(gom_d, ref["gom"], ref["gom_abs"], ref["max_terms"], f"direct grad_om {case} m{margin}")


OVERFLOW = [
    # (shape, dtype, bucket capacities): capacities far below the ~9 samples
    # of a cell send most samples through the overflow kernel's atomics
    (Shape(2, 19, 23, 64, 4), "bf16", (1, 2, 5)),
    (Shape(1, 21, 17, 48, 3, sh=2, sw=2, ph=1, pw=1), "f32", (1, 3)),
    (Shape(1, 16, 20, 40, 4, dh=2, dw=2, ph=2, pw=2), "f16", (1, 4)),  # D=10: element path
    (Shape(1, 18, 18, 32, 2, multiscale=True), "bf16", (1, 2)),
    (Shape(1, 18, 18, 32, 2, multiscale=True, pixel_scales=True, max_scale=2.5), "f16", (2,)),
    (Shape(1, 15, 17, 32, 2, offset_scale=0.5), "bf16", (1,)),
]
OVERFLOW_CASES = [(c, cap) for c, (_, _, caps) in enumerate(OVERFLOW) for cap in caps]


@pytest.mark.parametrize("case, cap", OVERFLOW_CASES)
def test_gather_overflow(case, cap):
    """Full buckets: the samples beyond a bucket's capacity are listed and
    added with atomics after the gather; the sum must stay within the bound."""
    s, dt, _ = OVERFLOW[case]
    inp, gy = bwd_inputs(s, dt, seed=700 + case)
    plan = d4.Plan(desc_of(s, dt), bucket_capacity=cap)
    assert plan.info()["bucket_capacity"] == cap
    say(f"gather overflow {case} cap {cap}: {s} {dt}")
    ref = oracle.get().backward(s, dt, inp.x, inp.om, gy, inp.scales, inp.pscales)
    gx, _ = run_backward(plan, inp, gy, dt, want_om=False)
    check_bound(gx, ref["gx"], ref["gx_abs"], ref["max_terms"], f"overflow {case} cap {cap}")


def test_gather_chunks():
    """The gathered grad_x runs in chunks of (image, group) pairs that reuse
    one workspace: with 1024 records per bucket one pair needs more than the
    operator's ideal bytes, so the default workspace holds one pair (32
    chunks); a caller's workspace of three and a half pairs runs the fewest
    chunks that fit it, three images of one group (the last chunk of each
    group holding two images)."""
    s = Shape(8, 64, 64, 64, 4)
    dt = "bf16"
    plan = d4.Plan(desc_of(s, dt), bucket_capacity=1024)
    one = d4.Plan(desc_of(Shape(1, 64, 64, 16, 1), dt), bucket_capacity=1024)
    ws = plan.backward_workspace_bytes()
    assert ws == one.backward_workspace_bytes() and ws > plan.ideal_bytes
    inp, gy = bwd_inputs(s, dt, seed=808)
    say(f"gather chunks: {s} {dt}, workspace {ws} bytes")
    ref = oracle.get().backward(s, dt, inp.x, inp.om, gy)
    gx, _ = run_backward(plan, inp, gy, dt, want_om=False)
    check_bound(gx, ref["gx"], ref["gx_abs"], ref["max_terms"], "gather chunks of one pair")
    big = torch.empty(ws * 7 // 2, dtype=torch.uint8, device="cuda")
    x, om, g = to_dev(inp.x, dt), to_dev(inp.om, dt), to_dev(gy, dt)
    gx2, _ = plan.backward(x, om, g, want_om=False, workspace=big)
    torch.cuda.synchronize()
    check_bound(gx2.cpu().numpy(), ref["gx"], ref["gx_abs"], ref["max_terms"],
                "gather chunks of three images")


def test_backward_allocating_entry():
    """dcn4_backward allocates its workspace stream-ordered and gathers."""
    s = Shape(2, 17, 19, 64, 4)
    dt = "bf16"
    inp, gy_raw = bwd_inputs(s, dt, seed=909)
    plan = d4.Plan(desc_of(s, dt))
    x, om, gy = to_dev(inp.x, dt), to_dev(inp.om, dt), to_dev(gy_raw, dt)
    gx = torch.full((s.N, s.H, s.W, s.C), float("nan"), dtype=torch.float32, device="cuda")
    gom = torch.empty(plan.om_shape(), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert d4.dcn4_backward(plan.handle, x.data_ptr(), om.data_ptr(), None, None,
                            gy.data_ptr(), gx.data_ptr(), gom.data_ptr(), st) == d4.DCN4_OK
    torch.cuda.synchronize()
    ref = oracle.get().backward(s, dt, inp.x, inp.om, gy_raw)
    check_bound(gx.cpu().numpy(), ref["gx"], ref["gx_abs"], ref["max_terms"], "allocating grad_x")
    check_bound(gom.cpu().numpy(), ref["gom"], ref["gom_abs"], ref["max_terms"], "allocating grad_om")


FAR = [
    # shapes whose gather stages grad_y in LDS (groups of 16, 32 or 48 bytes),
    # with displacements up to 12 pixels: many records come from output
    # pixels outside the staged window and read global memory
    (Shape(2, 37, 41, 64, 4), "bf16"),
    (Shape(1, 35, 70, 32, 4), "f16"),                               # D=8: 64 columns per strip
    (Shape(1, 33, 29, 72, 3), "bf16"),                              # D=24: 3 vectors per group
    (Shape(1, 40, 36, 64, 4, sh=2, sw=2, dh=2, dw=2, ph=2, pw=2), "bf16"),
    (Shape(1, 30, 34, 64, 4, multiscale=True), "f16"),
]


@pytest.mark.parametrize("case", range(len(FAR)))
def test_gather_far_samples(case):
    s, dt = FAR[case]
    inp, gy = bwd_inputs(s, dt, seed=900 + case, off_range=12.0)
    plan = d4.Plan(desc_of(s, dt))
    say(f"gather far samples {case}: {s} {dt}")
    ref = oracle.get().backward(s, dt, inp.x, inp.om, gy, inp.scales, inp.pscales)
    gx, _ = run_backward(plan, inp, gy, dt, want_om=False)
    check_bound(gx, ref["gx"], ref["gx_abs"], ref["max_terms"], f"far samples {case}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_backward_element_paths(dt):
    """Tensors that are only element-aligned -- x, the offset/weight tensor
    and grad_y one element into their buffers, grad_x one float into its --
    take the element-wise gather and the direct offset/weight-gradient
    kernel; both gradients within the bound, on both grad_x paths."""
    s = Shape(2, 19, 21, 32, 2)
    inp, gy_raw = bwd_inputs(s, dt, seed=77)
    plan = d4.Plan(desc_of(s, dt))
    x, om, gy = (to_dev(inp.x, dt, offset_elems=1), to_dev(inp.om, dt, offset_elems=1),
                 to_dev(gy_raw, dt, offset_elems=1))
    ref = oracle.get().backward(s, dt, inp.x, inp.om, gy_raw)
    say(f"backward element paths {s} {dt}")
    for scatter in (False, True):
        gxbuf = torch.empty(s.N * s.H * s.W * s.C + 1, dtype=torch.float32, device="cuda")
        gx = gxbuf[1:].view(s.N, s.H, s.W, s.C)
        gom = torch.empty(plan.om_shape(), dtype=torch.float32, device="cuda")
        plan.backward(x, om, gy, grad_x=gx, grad_om=gom, scatter=scatter)
        torch.cuda.synchronize()
        what = f"element paths {dt} {'scatter' if scatter else 'gather'}"
        check_bound(gx.cpu().numpy(), ref["gx"], ref["gx_abs"], ref["max_terms"], what + " grad_x")
        check_bound(gom.cpu().numpy(), ref["gom"], ref["gom_abs"], ref["max_terms"], what + " grad_om")


# ----------------------------------------------------- gradients of the scales
def scale_grad_cases():
    """group-scale plans: with and without predicted pixel scales and the
    Smax clamp, every dtype, 3x3 (compile-time kernel) and 5x5 / 1x1, group
    widths over 1 to 16 lanes"""
    rng = np.random.default_rng(8765)
    cases = []
    for t in range(12):
        dt = ["bf16", "f32", "f16"][t % 3]
        k = [3, 3, 5, 1][t % 4]
        ps = t % 2 == 1
        smax = [0.0, 2.0, 1.25][t % 3] if ps or t % 3 else 0.0
        D = int(rng.choice([8, 24, 72, 10, 16]))
        G = int(rng.integers(1, 5))
        s = Shape(int(rng.integers(1, 3)), int(rng.integers(5, 20)), int(rng.integers(5, 20)),
                  G * D, G, k, k, 1, 1, int(rng.integers(0, 3)), int(rng.integers(0, 3)),
                  multiscale=True, pixel_scales=ps, max_scale=smax)
        try:
            oracle.get().out_size(s)
        except ValueError:
            continue
        cases.append((t, s, dt))
    return cases


def run_scale_grads(plan, s, inp, gy_raw, dt):
    x, om, gy = to_dev(inp.x, dt), to_dev(inp.om, dt), to_dev(gy_raw, dt)
    sc = torch.from_numpy(inp.scales).cuda()
    gsg, gps = plan.backward_scales(x, om, gy, sc, dev_f32(inp.pscales))
    torch.cuda.synchronize()
    return gsg.cpu().numpy(), None if gps is None else gps.cpu().numpy()


def check_scale_grads(s, dt, inp, gy, plan, what):
    """dL/dsigma within the fp32 bound of its 4DK terms; dL/ds_g within the
    bound with the per-pixel partial sums added on top (atomics)"""
    o = oracle.get()
    ref = o.backward_scales(s, dt, inp.x, inp.om, gy, inp.scales, inp.pscales)
    gsg, gps = run_scale_grads(plan, s, inp, gy, dt)
    n_item = 4 * (s.C // s.G) * s.K + 16
    Ho, Wo = o.out_size(s)
    check_bound(gsg, ref["gs"], ref["gs_abs"], n_item + s.N * Ho * Wo, f"{what} dL/ds_g")
    if s.pixel_scales:
        check_bound(gps, ref["gp"], ref["gp_abs"], n_item, f"{what} dL/dsigma")
        if s.max_scale > 0:
            clamped = inp.scales[None, None, None, :] * inp.pscales > np.float32(s.max_scale)
            assert np.all(gps[clamped] == 0.0), f"{what}: nonzero gradient above the clamp"


@pytest.mark.parametrize("t, s, dt", scale_grad_cases(),
                         ids=lambda v: str(v) if isinstance(v, int) else None)
def test_scale_gradients(t, s, dt):
    inp, gy = bwd_inputs(s, dt, seed=700 + t)
    plan = d4.Plan(desc_of(s, dt))
    say(f"scale gradients case {t}: {s} {dt}")
    check_scale_grads(s, dt, inp, gy, plan, f"scale grads {t}")


def test_scale_gradients_full_size():
    """FlowDCN's tokens with predicted scales and Smax 4 at full size."""
    w = WORKLOADS["flowdcn_pixelscale_bf16"]
    s = shape_of(w)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = make_inputs(w, Ho, Wo)
    gy = to_raw(np.random.default_rng(11).standard_normal((s.N, Ho, Wo, s.C), dtype=np.float32),
                w.dtype)
    say(f"scale gradients, full size {w.describe()}")
    check_scale_grads(s, w.dtype, inp, gy, d4.Plan(desc_of(s, w.dtype)), "flowdcn full size")


def test_scale_gradients_requests():
    """Either output may be skipped; the group gradient of an empty batch is
    zero; a plan without group scales is refused."""
    s = Shape(2, 9, 8, 48, 2, multiscale=True, pixel_scales=True, max_scale=2.0)
    dt = "bf16"
    inp, gy = bwd_inputs(s, dt, seed=777)
    plan = d4.Plan(desc_of(s, dt))
    x, om, g = to_dev(inp.x, dt), to_dev(inp.om, dt), to_dev(gy, dt)
    sc, ps = torch.from_numpy(inp.scales).cuda(), dev_f32(inp.pscales)
    a, b = plan.backward_scales(x, om, g, sc, ps)
    a2, none = plan.backward_scales(x, om, g, sc, ps, want_pixel=False)
    none2, b2 = plan.backward_scales(x, om, g, sc, ps, want_group=False)
    torch.cuda.synchronize()
    assert none is None and none2 is None
    assert torch.equal(b.view(torch.int32), b2.view(torch.int32))
    ref = oracle.get().backward_scales(s, dt, inp.x, inp.om, gy, inp.scales, inp.pscales)
    n = 4 * 24 * 9 + 16 + s.N * 9 * 8
    check_bound(a2.cpu().numpy(), ref["gs"], ref["gs_abs"], n, "group gradient alone")
    empty = d4.Plan(desc_of(Shape(0, 9, 8, 48, 2, multiscale=True), dt))
    z = torch.full((2,), float("nan"), device="cuda")
    st = d4.dcn4_backward_scales(empty.handle, None, None, sc.data_ptr(), None, None,
                                 z.data_ptr(), None, None)
    torch.cuda.synchronize()
    assert st == d4.DCN4_OK and torch.equal(z.cpu(), torch.zeros(2))
    std = d4.Plan(desc_of(Shape(1, 9, 8, 48, 2), dt))
    assert d4.dcn4_backward_scales(std.handle, x.data_ptr(), om.data_ptr(), None, None,
                                   g.data_ptr(), z.data_ptr(), None, None) == d4.DCN4_ERR_INVALID_ARG
