"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Gates, written here:
  * every dtype: the output is compared element by element with the oracle's
    fp32 evaluation (same operation order, rounded the same way); the number
    of differing elements must be 0;
  * fp32 I/O: max_i |y_gpu - y_def| / (|y_def| + RMS(y_def)) <= 1e-5 against
    the fp64 definition (on sampled pixels at full size);
  * bf16/fp16 I/O: max_i |y_gpu - y_oracle| / RMS(y_oracle) <= 1e-2 with
    y_oracle the oracle's output rounded to the I/O dtype;
  * sample indices: the geometry probe equals the oracle's (y0, x0, lh, lw,
    inside) bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle import Shape
from workloads import WORKLOADS, from_raw, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import dynamic_sparse_vision_dcn4_amd as d4  # noqa: E402

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
NTHREADS = 16


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(raw, dt, offset_elems=0):
    """numpy raw -> CUDA tensor of the I/O dtype; offset_elems > 0 returns a
    view that starts that many elements into a larger buffer (misaligned)."""
    if dt == "f32":
        t = torch.from_numpy(np.ascontiguousarray(raw, np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(TORCH_DT[dt])
    if offset_elems:
        buf = torch.empty(t.numel() + offset_elems, dtype=t.dtype, device="cuda")
        v = buf[offset_elems:].view(t.shape)
        v.copy_(t.cuda())
        return v
    return t.cuda()


def to_raw_np(t, dt):
    t = t.detach().cpu().contiguous()
    if dt == "f32":
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def desc_of(s: Shape, dt: str) -> d4.Desc:
    return d4.Desc(s.N, s.H, s.W, s.C, s.G, s.kh, s.kw, s.sh, s.sw, s.ph, s.pw,
                   s.dh, s.dw, s.offset_scale, s.multiscale, dt, s.pixel_scales,
                   s.max_scale)


def shape_of(w) -> Shape:
    return Shape(w.N, w.H, w.W, w.C, w.G, w.kh, w.kw, w.sh, w.sw, w.ph, w.pw,
                 w.dh, w.dw, w.offset_scale, w.multiscale, w.pixel_scales,
                 w.max_scale)


def dev_f32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def gpu_forward(plan, inp, dt, offset_elems=0):
    x = to_dev(inp.x, dt, offset_elems)
    om = to_dev(inp.om, dt, offset_elems)
    sc = None if inp.scales is None else torch.from_numpy(inp.scales).cuda()
    out = None
    if offset_elems:
        buf = torch.empty(int(np.prod(plan.out_shape())) + offset_elems,
                          dtype=TORCH_DT[dt], device="cuda")
        out = buf[offset_elems:].view(plan.out_shape())
    y = plan.forward(x, om, sc, out=out, pixel_scales=dev_f32(inp.pscales))
    torch.cuda.synchronize()
    return to_raw_np(y, dt)


def bits_equal(a, b, dt):
    """element-wise equality of raw encodings, NaN == NaN (any payload)"""
    fa, fb = from_raw(a, dt), from_raw(b, dt)
    same = (np.asarray(a).view(np.uint16 if dt != "f32" else np.uint32) ==
            np.asarray(b).view(np.uint16 if dt != "f32" else np.uint32))
    return same | (np.isnan(fa) & np.isnan(fb))


def check_against_oracle(y_gpu, y_or, dt, what):
    eq = bits_equal(y_gpu, y_or, dt)
    ndiff = int((~eq).sum())
    fg = from_raw(y_gpu, dt).astype(np.float64)
    fo = from_raw(y_or, dt).astype(np.float64)
    fin = np.isfinite(fo)
    rms = np.sqrt(np.mean(fo[fin] ** 2)) if fin.any() else 1.0
    rms = rms if rms > 0 else 1.0
    err = np.abs(fg - fo)[fin].max(initial=0.0) / rms
    say(f"{what}: {ndiff} of {eq.size} elements differ; max|d|/RMS = {err:.3g}")
    if dt != "f32":
        assert err <= 1e-2, f"{what}: max|d|/RMS {err} > 1e-2"
    assert ndiff == 0, f"{what}: {ndiff} elements differ from the oracle"


def check_fp32_gate(y_gpu, y_def, what):
    g = from_raw(y_gpu, "f32").astype(np.float64)
    rms = np.sqrt(np.mean(y_def ** 2))
    rel = np.max(np.abs(g - y_def) / (np.abs(y_def) + rms))
    say(f"{what}: fp32 relative error vs fp64 definition {rel:.3g}")
    assert rel <= 1e-5


# ------------------------------------------------------------------ fuzz
def fuzz_cases(n=40, seed=1234):
    rng = np.random.default_rng(seed)
    cases = []
    kernels = [(3, 3), (1, 1), (5, 5), (3, 5), (2, 2), (3, 3), (3, 3)]
    for t in range(n):
        dt = ["f32", "bf16", "f16"][t % 3]
        ms = (t % 5 == 4)
        kh, kw = kernels[rng.integers(len(kernels))]
        if ms and (kh % 2 == 0 or kw % 2 == 0):
            kh, kw = 3, 3
        D = int(rng.choice([8, 16, 24, 32, 10, 72, 4]))
        G = int(rng.integers(1, 5))
        N = int(rng.integers(1, 4))
        H = int(rng.integers(5, 40))
        W = int(rng.integers(5, 40))
        sh, sw = (1, 1) if ms else (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        dh, dw = (1, 1) if ms else (int(rng.integers(1, 4)), int(rng.integers(1, 3)))
        ph, pw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        os_ = 1.0 if (ms or t % 4) else 0.5
        s = Shape(N, H, W, G * D, G, kh, kw, sh, sw, ph, pw, dh, dw, os_, ms)
        try:
            oracle.get().out_size(s)
        except ValueError:
            continue
        cases.append((t, s, dt))
    return cases


def fuzz_inputs(s, dt, Ho, Wo, seed):
    rng = np.random.default_rng(seed)
    K = s.K
    x = rng.standard_normal((s.N, s.H, s.W, s.C)).astype(np.float32)
    off = rng.uniform(-3, 3, (s.N, Ho, Wo, s.G, 2 * K)).astype(np.float32)
    m = (rng.standard_normal((s.N, Ho, Wo, s.G, K)) / 3).astype(np.float32)
    om = np.concatenate([off, m], -1)
    scales = (rng.uniform(0.5, 3.0, s.G).astype(np.float32) if s.multiscale else None)
    return workloads.Inputs(workloads.to_raw(x, dt), workloads.to_raw(om, dt), scales)


@pytest.mark.parametrize("kernel", [0, 1], ids=["auto", "direct"])
@pytest.mark.parametrize("t, s, dt", fuzz_cases(), ids=lambda v: str(v) if isinstance(v, int) else None)
def test_fuzz_parity(t, s, dt, kernel):
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=t)
    plan = d4.Plan(desc_of(s, dt), kernel=kernel)
    say(f"fuzz case {t}: {s} {dt} kernel {plan.info()['kernel']}")
    assert (plan.Ho, plan.Wo) == (Ho, Wo)
    y = gpu_forward(plan, inp, dt)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=NTHREADS)
    check_against_oracle(y, y_or, dt, f"fuzz {t}")
    if dt == "f32":
        check_fp32_gate(y, o.forward_f64(s, dt, inp.x, inp.om, inp.scales,
                                         nthreads=NTHREADS), f"fuzz {t}")
    # sample indices, bit for bit
    om_dev = to_dev(inp.om, dt)
    sc = None if inp.scales is None else torch.from_numpy(inp.scales).cuda()
    g = plan.probe_geometry(om_dev, sc)
    torch.cuda.synchronize()
    ref = o.geometry(s, dt, inp.om, inp.scales)
    for k in ("inside", "y0", "x0"):
        assert np.array_equal(g[k].cpu().numpy(), ref[k]), k
    for k in ("lh", "lw"):
        assert np.array_equal(g[k].cpu().numpy().view(np.uint32), ref[k].view(np.uint32)), k


# ------------------------------------------------------------ workloads
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(name):
    """Every pages' workload at its full size, in the launch configuration
    the benchmark times (default plan, 16-byte aligned tensors), and with the
    direct kernel forced."""
    w = WORKLOADS[name]
    o = oracle.get()
    s = shape_of(w)
    Ho, Wo = o.out_size(s)
    say(f"workload {w.describe()}")
    inp = make_inputs(w, Ho, Wo)
    plan = d4.Plan(desc_of(s, w.dtype))
    say(f"  plan {plan.info()}")
    y = gpu_forward(plan, inp, w.dtype)
    y_or = o.forward_f32(s, w.dtype, inp.x, inp.om, inp.scales, nthreads=NTHREADS,
                         pscales=inp.pscales)
    check_against_oracle(y, y_or, w.dtype, name)
    if plan.info()["kernel"] != 1:
        direct = d4.Plan(desc_of(s, w.dtype), kernel=1)
        check_against_oracle(gpu_forward(direct, inp, w.dtype), y_or, w.dtype,
                             name + " (direct kernel)")
    # the fp64 definition on sampled pixels
    rng = np.random.default_rng(7)
    npix = s.N * Ho * Wo
    pix = np.unique(np.concatenate([rng.integers(0, npix, 3000),
                                    [0, npix - 1, Wo - 1, npix - Wo]]))
    y64 = o.forward_f64(s, w.dtype, inp.x, inp.om, inp.scales, pix=pix,
                        nthreads=NTHREADS, pscales=inp.pscales)
    yg = y.reshape(npix, s.C)[pix]
    if w.dtype == "f32":
        check_fp32_gate(yg, y64, name)
    else:
        fg = from_raw(yg, w.dtype).astype(np.float64)
        err = np.max(np.abs(fg - y64)) / np.sqrt(np.mean(y64 ** 2))
        say(f"  {name}: max|y - fp64 definition|/RMS on {pix.size} pixels = {err:.3g} "
            "(includes the output rounding)")
    # geometry of the sampled pixels, bit for bit
    geo = plan.probe_geometry(to_dev(inp.om, w.dtype),
                              None if inp.scales is None else torch.from_numpy(inp.scales).cuda(),
                              pixel_scales=dev_f32(inp.pscales))
    torch.cuda.synchronize()
    ref = o.geometry(s, w.dtype, inp.om, inp.scales, pix=pix, pscales=inp.pscales)
    GK = s.G * s.K
    sel = (pix[:, None] * GK + np.arange(GK)[None, :]).reshape(-1)
    for k in ("inside", "y0", "x0"):
        assert np.array_equal(geo[k].cpu().numpy()[sel], ref[k]), k
    for k in ("lh", "lw"):
        assert np.array_equal(geo[k].cpu().numpy()[sel].view(np.uint32),
                              ref[k].view(np.uint32)), k


# ------------------------------------------------- FlowDCN predicted scale
def pixel_scale_cases():
    rng = np.random.default_rng(77)
    cases = []
    for t in range(12):
        dt = ["bf16", "f32", "f16"][t % 3]
        k = [3, 5, 1][t % 3]
        D = int(rng.choice([8, 16, 24, 72]))
        G = int(rng.integers(1, 5))
        smax = [0.0, 2.5, 0.75][t % 3 if t < 9 else 0]
        s = Shape(int(rng.integers(1, 3)), int(rng.integers(5, 30)), int(rng.integers(5, 30)),
                  G * D, G, k, k, 1, 1, int(rng.integers(0, 3)), int(rng.integers(0, 3)),
                  multiscale=True, pixel_scales=True, max_scale=smax)
        try:
            oracle.get().out_size(s)
        except ValueError:
            continue
        cases.append((t, s, dt))
    return cases


@pytest.mark.parametrize("t, s, dt", pixel_scale_cases(),
                         ids=lambda v: str(v) if isinstance(v, int) else None)
def test_pixel_scale_parity(t, s, dt):
    """FlowDCN's predicted per-pixel scale times the group prior, with and
    without the Smax clamp: output and sample geometry bit for bit, including
    a NaN and a zero predicted scale."""
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=100 + t)
    rng = np.random.default_rng(200 + t)
    ps = rng.uniform(0.25, 2.0, (s.N, Ho, Wo, s.G)).astype(np.float32)
    ps.reshape(-1)[0] = np.nan
    ps.reshape(-1)[-1] = 0.0
    inp = workloads.Inputs(inp.x, inp.om, inp.scales, ps)
    plan = d4.Plan(desc_of(s, dt))
    say(f"pixel scales case {t}: {s} {dt} {plan.info()}")
    y = gpu_forward(plan, inp, dt)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=NTHREADS, pscales=ps)
    check_against_oracle(y, y_or, dt, f"pixel scales {t}")
    if dt == "f32":
        check_fp32_gate(y, o.forward_f64(s, dt, inp.x, inp.om, inp.scales,
                                         nthreads=NTHREADS, pscales=ps), f"pixel scales {t}")
    g = plan.probe_geometry(to_dev(inp.om, dt), torch.from_numpy(inp.scales).cuda(),
                            pixel_scales=dev_f32(ps))
    torch.cuda.synchronize()
    ref = o.geometry(s, dt, inp.om, inp.scales, pscales=ps)
    for k in ("inside", "y0", "x0"):
        assert np.array_equal(g[k].cpu().numpy(), ref[k]), k
    for k in ("lh", "lw"):
        assert np.array_equal(g[k].cpu().numpy().view(np.uint32), ref[k].view(np.uint32)), k


# ------------------------------------------------------------ variants
@pytest.mark.parametrize("margin", [0, 1, 2, 3, 5])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_tiled_kernel_margins(dt, margin):
    """The tiled kernel gathers from LDS when a point's corners are in its
    window and falls back to global gathers for the wave otherwise; a small
    margin exercises the fallback on most points, a large one none.  Ragged
    tiles (H, W not multiples of the tile) and zero padding included."""
    w = WORKLOADS["ldm_unet_block_bf16"].with_(N=2, H=37, W=45, C=64, G=4, dtype=dt)
    s = shape_of(w)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = make_inputs(w, Ho, Wo)
    # fp32 lanes own 8 channels here so that the window fits in LDS
    plan = d4.Plan(desc_of(s, dt), channels_per_lane=8 if dt == "f32" else 0,
                   kernel=2, tile_margin=margin, tile_window=1)
    say(f"tiled margin {margin} {dt}: {plan.info()}")
    y = gpu_forward(plan, inp, dt)
    check_against_oracle(y, o.forward_f32(s, dt, inp.x, inp.om, None, nthreads=NTHREADS),
                         dt, f"tiled margin {margin}")


# (shape, dtype, channels per lane, extra options): margin windows shared by
# several tile rows -- 16-channel groups (square per-pass test), 3x3 and 5x5
# (generic point loop, whole-window test), stride 2, FlowDCN's geometry on
# 16-channel slices with predicted scales, two groups per workgroup; the heights leave
# the last workgroup's rows ragged or past the image
MARGIN_PASSES = [
    (Shape(2, 37, 45, 64, 4), "bf16", 0, {}),
    (Shape(2, 37, 45, 64, 4), "f16", 0, {}),
    (Shape(1, 50, 33, 64, 4), "f32", 8, {}),
    (Shape(1, 41, 35, 64, 8, 5, 5, 1, 1, 2, 2), "bf16", 0, {}),
    (Shape(2, 47, 30, 16, 2, 3, 3, 2, 2, 1, 1), "bf16", 0, {}),
    (Shape(1, 35, 29, 96, 2, multiscale=True, pixel_scales=True, max_scale=4.0),
     "bf16", 16, {}),
    (Shape(1, 40, 36, 64, 8), "bf16", 0, {"tile_groups": 2}),
]


@pytest.mark.parametrize("passes", [2, 3, 5])
@pytest.mark.parametrize("margin", [1, 4])
@pytest.mark.parametrize("case", range(len(MARGIN_PASSES)))
def test_tiled_margin_window_passes(case, margin, passes):
    """Several tile rows per workgroup under one staging of their joint
    margin window: each row tests its points against its own square (or the
    joint window) and takes the global path outside it; bit for bit with the
    oracle, and with the one-row plan."""
    s, dt, dp, extra = MARGIN_PASSES[case]
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=500 + 10 * case + margin)
    if s.pixel_scales:
        rng = np.random.default_rng(600 + case)
        ps = rng.uniform(0.25, 2.0, (s.N, Ho, Wo, s.G)).astype(np.float32)
        inp = workloads.Inputs(inp.x, inp.om, inp.scales, ps)
    one = d4.Plan(desc_of(s, dt), channels_per_lane=dp, kernel=2, tile_window=1,
                  tile_margin=margin, tile_passes=1, **extra)
    plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp, kernel=2, tile_window=1,
                   tile_margin=margin, tile_passes=passes, **extra)
    info = plan.info()
    say(f"margin passes {passes} case {case} {s} {dt} margin {margin}: {info}")
    assert info["kernel"] == 2 and info["tile_window"] == 1 and info["tile_passes"] > 1
    assert one.info()["tile_passes"] == 1
    y = gpu_forward(plan, inp, dt)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=NTHREADS,
                         pscales=inp.pscales)
    check_against_oracle(y, y_or, dt, f"margin passes {passes} case {case}")
    assert np.array_equal(bits_equal(gpu_forward(one, inp, dt), y, dt),
                          np.ones(y.shape, bool))


# (dtype, D, channels per lane, kernel size, stride, pixel scales, Smax):
# sliced windows (D 72 in 24-channel slices, D 48 in 16) and whole groups
# (D 16, 24), 3x3 and 5x5 (the generic point loop), stride 2, FlowDCN's
# predicted scales with and without the clamp
GS_TILED = [("bf16", 72, 24, 3, 1, False, 0.0), ("bf16", 72, 24, 3, 1, True, 4.0),
            ("f16", 48, 16, 3, 1, True, 0.0), ("f32", 16, 8, 3, 1, False, 0.0),
            ("bf16", 16, 16, 5, 1, True, 2.5), ("bf16", 24, 24, 3, 1, False, 0.0),
            ("bf16", 16, 16, 3, 2, False, 0.0), ("f16", 72, 24, 5, 1, False, 3.0)]


@pytest.mark.parametrize("margin", [0, 2, 6, 10])
@pytest.mark.parametrize("dt, D, dp, k, st, pix, smax", GS_TILED)
def test_tiled_group_scale(dt, D, dp, k, st, pix, smax, margin):
    """FlowDCN's multi-scale geometry on the tiled kernel (centre plus the
    group scale times grid point plus direction, the lane's scale from the
    prior, the predicted scale and Smax): bit for bit with the oracle, on
    the LDS path and the global fallback (margin 0 sends most waves there;
    the priors reach 4, so every margin leaves some points outside)."""
    G = 2  # 16-bit offset/weight rows of G*3K values must be 4-byte aligned to tile
    s = Shape(2, 21, 27, G * D, G, k, k, st, st, k // 2, k // 2,
              multiscale=True, pixel_scales=pix, max_scale=smax)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=D + k + margin)
    if pix:
        rng = np.random.default_rng(300 + D + margin)
        ps = rng.uniform(0.25, 2.0, (s.N, Ho, Wo, s.G)).astype(np.float32)
        ps.reshape(-1)[1] = np.nan
        ps.reshape(-1)[-2] = 0.0
        inp = workloads.Inputs(inp.x, inp.om, inp.scales, ps)
    try:
        plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp, kernel=2, tile_margin=margin,
                       tile_window=1)
    except d4.DCN4Error as e:
        # a wide margin's window can exceed LDS; margin 0 always fits here
        assert e.status == d4.DCN4_ERR_UNSUPPORTED and margin > 0
        return
    info = plan.info()
    say(f"tiled group scale {dt} D={D} dp={dp} k={k} s={st} pix={pix} smax={smax} "
        f"margin {margin}: {info}")
    assert info["kernel"] == 2
    y = gpu_forward(plan, inp, dt)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=NTHREADS,
                         pscales=inp.pscales)
    check_against_oracle(y, y_or, dt, f"tiled group scale D={D} margin {margin}")


@pytest.mark.parametrize("margin", [1, 4])
@pytest.mark.parametrize("dt, D, dp", [("bf16", 72, 24), ("f32", 24, 8)])
def test_tiled_channel_slices_standard_mode(dt, D, dp, margin):
    """Groups whose lanes do not divide the workgroup run one channel slice
    of a group per workgroup in the standard modes too (and offset_scale
    0.5): same bits as the oracle."""
    s = Shape(2, 23, 19, 2 * D, 2, offset_scale=0.5)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=7 + D + margin)
    plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp, kernel=2, tile_margin=margin,
                   tile_window=1)
    info = plan.info()
    say(f"sliced standard {dt} D={D} dp={dp} margin {margin}: {info}")
    assert info["kernel"] == 2 and info["tile_slices"] == D // dp
    check_against_oracle(gpu_forward(plan, inp, dt),
                         o.forward_f32(s, dt, inp.x, inp.om, None, nthreads=NTHREADS),
                         dt, f"sliced standard D={D} margin {margin}")


@pytest.mark.parametrize("swizzle", [0, 1, 3, 4, 6])
@pytest.mark.parametrize("dt, D, dp", [("bf16", 16, 16), ("f32", 16, 8), ("f16", 32, 16),
                                       ("bf16", 64, 32)])
def test_tiled_kernel_vector_order(dt, D, dp, swizzle):
    """Lanes that read their 16-byte vectors pairwise swapped (to spread LDS
    banks) must give the same bits, on the LDS path and on the global path
    (margin 1 sends most waves there)."""
    s = Shape(2, 27, 35, 2 * D, 2)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=swizzle + D)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, None, nthreads=NTHREADS)
    for margin in (1, 3):
        plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp, kernel=2, tile_margin=margin,
                       tile_swizzle=swizzle, tile_window=1)
        say(f"vector order: swizzle {swizzle} margin {margin} {dt} D={D}: {plan.info()}")
        check_against_oracle(gpu_forward(plan, inp, dt), y_or, dt,
                             f"swizzle {swizzle} margin {margin}")


# (shape, dtype, channels per lane): square images (the centred window test)
# and others, dilation, stride, 5x5 (the generic point loop), offset_scale,
# group scales with predicted scales and Smax, 72-channel groups in slices
WHOLE = [(Shape(2, 24, 24, 64, 2, dh=2, dw=2, ph=2, pw=2), "f16", 16),
         (Shape(2, 19, 27, 32, 2), "bf16", 0),
         (Shape(1, 21, 21, 32, 2), "f32", 8),
         (Shape(2, 20, 20, 32, 2, multiscale=True), "bf16", 0),
         (Shape(1, 17, 23, 32, 2, multiscale=True, pixel_scales=True, max_scale=2.5), "f16", 0),
         (Shape(1, 40, 16, 144, 2, multiscale=True), "bf16", 24),
         (Shape(2, 41, 18, 64, 4, sh=2, sw=2), "bf16", 0),
         (Shape(1, 22, 22, 32, 2, 5, 5, ph=2, pw=2), "bf16", 0),
         (Shape(1, 20, 20, 64, 2, offset_scale=0.5), "f16", 0)]


def wide_offset_inputs(s, dt, Ho, Wo, seed, reach=8.0):
    """x ~ N(0,1), offsets U[-reach, reach] (many samples leave the image),
    weights N(0, 1/9); group priors U[0.5, 3]; predicted scales U[0.25, 2]."""
    rng = np.random.default_rng(seed)
    K = s.K
    x = rng.standard_normal((s.N, s.H, s.W, s.C)).astype(np.float32)
    off = rng.uniform(-reach, reach, (s.N, Ho, Wo, s.G, 2 * K)).astype(np.float32)
    m = (rng.standard_normal((s.N, Ho, Wo, s.G, K)) / 3).astype(np.float32)
    om = np.concatenate([off, m], -1)
    scales = rng.uniform(0.5, 3.0, s.G).astype(np.float32) if s.multiscale else None
    ps = (rng.uniform(0.25, 2.0, (s.N, Ho, Wo, s.G)).astype(np.float32)
          if s.pixel_scales else None)
    return workloads.Inputs(workloads.to_raw(x, dt), workloads.to_raw(om, dt), scales, ps)


@pytest.mark.parametrize("case", range(len(WHOLE)))
def test_tiled_whole_image_window(case):
    """The whole-image window (the image plus a zero border in LDS): a
    sample whose cell leaves it is outside the image and adds nothing, so
    no wave takes the global path for it.  Offsets up to 8 pixels send many
    samples off the image; bit for bit with the oracle and with the margin
    window."""
    s, dt, dp = WHOLE[case]
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = wide_offset_inputs(s, dt, Ho, Wo, seed=40 + case)
    plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp, kernel=2, tile_window=2)
    info = plan.info()
    say(f"whole-image window {case}: {s} {dt} {info}")
    assert info["kernel"] == 2 and info["tile_window"] == 2
    y = gpu_forward(plan, inp, dt)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=NTHREADS,
                         pscales=inp.pscales)
    check_against_oracle(y, y_or, dt, f"whole-image window {case}")
    margin = d4.Plan(desc_of(s, dt), channels_per_lane=dp, kernel=2, tile_window=1,
                     tile_margin=2)
    assert margin.info()["tile_window"] == 1
    assert np.array_equal(bits_equal(gpu_forward(margin, inp, dt), y, dt),
                          np.ones(y.shape, bool))
    # a block of several tile rows and columns per workgroup under one
    # staging (the last ones ragged or past the image for some shapes): the
    # same bits
    for passes, passes_x in ((1, 1), (2, 1), (3, 1), (1, 2), (2, 2), (3, 3)):
        pp = d4.Plan(desc_of(s, dt), channels_per_lane=dp, kernel=2, tile_window=2,
                     tile_passes=passes, tile_passes_x=passes_x)
        say(f"  passes {passes} x {passes_x}: {pp.info()}")
        assert np.array_equal(bits_equal(gpu_forward(pp, inp, dt), y, dt),
                              np.ones(y.shape, bool))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_whole_image_window_nonfinite(dt):
    """Non-finite inputs under the whole-image window: an infinite or NaN
    weight still sends its wave to the global path (which weights corners
    outside the image by an exact zero), a NaN or infinite offset puts its
    sample outside the image, a NaN or infinite input value reaches the
    outputs that sample it."""
    s = Shape(1, 14, 14, 32, 2)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = wide_offset_inputs(s, "f32", Ho, Wo, seed=77, reach=4.0)
    x = from_raw(inp.x, "f32").copy()
    om = from_raw(inp.om, "f32").copy()
    x[0, 3, 4, :] = np.inf
    x[0, 7, 2, 5] = np.nan
    x[0, 0, 0, 7] = -np.inf
    om[0, 2, 2, 0, 4] = np.nan     # an offset
    om[0, 5, 6, 1, 20] = np.inf    # a weight
    om[0, 9, 9, 0, 19] = np.nan    # a weight
    om[0, 0, 0, 1, 0] = np.inf     # an offset pushing a sample outside
    inp = workloads.Inputs(workloads.to_raw(x, dt), workloads.to_raw(om, dt), None)
    plan = d4.Plan(desc_of(s, dt), kernel=2, tile_window=2)
    assert plan.info()["tile_window"] == 2
    say(f"whole-image window, non-finite values {dt}: {plan.info()}")
    check_against_oracle(gpu_forward(plan, inp, dt),
                         o.forward_f32(s, dt, inp.x, inp.om, None, nthreads=NTHREADS),
                         dt, "whole-image non-finite")


@pytest.mark.parametrize("groups, pad", [(1, 0), (2, 1), (4, 0), (4, 1)])
def test_tiled_kernel_group_chunks(groups, pad):
    w = WORKLOADS["ldm_unet_block_bf16"].with_(N=1, H=29, W=33, C=128, G=8)
    s = shape_of(w)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = make_inputs(w, Ho, Wo)
    plan = d4.Plan(desc_of(s, "bf16"), tile_margin=3, kernel=2, tile_groups=groups,
                   tile_pad=pad, tile_window=1)
    say(f"tiled groups {groups} pad {pad}: {plan.info()}")
    check_against_oracle(gpu_forward(plan, inp, "bf16"),
                         o.forward_f32(s, "bf16", inp.x, inp.om, None, nthreads=NTHREADS),
                         "bf16", f"tiled groups {groups}")



OM_UNIT_CASES = [("bf16", Shape(1, 29, 33, 128, 8), {"tile_groups": 1}),
                 ("bf16", Shape(1, 29, 33, 128, 8), {"tile_groups": 2, "tile_pad": 1}),
                 ("f32", Shape(2, 23, 21, 64, 4), {}),
                 ("f16", Shape(1, 20, 18, 128, 4, dh=2, dw=2, ph=2, pw=2), {}),
                 ("bf16", Shape(1, 19, 21, 144, 2, multiscale=True), {}),
                 ("bf16", Shape(1, 12, 12, 64, 4), {"tile_window": 2})]


@pytest.mark.parametrize("case", range(len(OM_UNIT_CASES)))
@pytest.mark.parametrize("unit", [1, 4, 16])
def test_tiled_om_copy_units(case, unit):
    """The tile's offset/weight values read by each lane from global memory
    into registers (1; one group per workgroup, else 4-byte units) or copied to LDS in 4- or 16-byte units (odd groups' 2-byte
    leads, group chunks, fp32 rows, whole-image windows whose later tile
    rows load their rows again, group-scale slices): the oracle bit for bit
    every way."""
    dt, s, opts = OM_UNIT_CASES[case]
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=700 + case)
    plan = d4.Plan(desc_of(s, dt), kernel=2, tile_om_unit=unit, **opts)
    direct_ok = opts.get("tile_groups", 1) == 1
    assert plan.info()["tile_om_unit"] == (4 if unit == 1 and not direct_ok else unit)
    say(f"om unit {unit} case {case}: {plan.info()}")
    check_against_oracle(gpu_forward(plan, inp, dt),
                         o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=NTHREADS),
                         dt, f"om unit {unit} case {case}")


@pytest.mark.parametrize("dt, D, dps", [("bf16", 16, (8, 16)), ("f32", 16, (4, 8, 12, 16)),
                                        ("f16", 32, (8, 16, 24, 32)),
                                        ("bf16", 72, (8, 24))])
def test_channels_per_lane_variants_identical(dt, D, dps):
    s = Shape(2, 23, 37, 2 * D, 2)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=D)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, None, nthreads=NTHREADS)
    for dp in dps:
        if D % dp:
            continue
        say(f"channels per lane {dp}: {s} {dt}")
        plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp)
        check_against_oracle(gpu_forward(plan, inp, dt), y_or, dt, f"D'={dp}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_element_path_for_misaligned_tensors(dt):
    """Tensors that are only element-aligned take the element-wise kernel."""
    s = Shape(2, 19, 21, 32, 2)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=5)
    say(f"element path {s} {dt}")
    plan = d4.Plan(desc_of(s, dt))
    y = gpu_forward(plan, inp, dt, offset_elems=1)
    check_against_oracle(y, o.forward_f32(s, dt, inp.x, inp.om, None,
                                          nthreads=NTHREADS), dt, "element path")


def test_nonfinite_values_propagate_like_the_oracle():
    s = Shape(1, 12, 13, 32, 2)
    dt = "f32"
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=9)
    inp.x[0, 3, 4, :] = np.inf
    inp.x[0, 7, 2, 5] = np.nan
    inp.x[0, 0, 0, 7] = -np.inf      # a border pixel
    inp.om[0, 2, 2, 0, 4] = np.nan   # an offset
    inp.om[0, 5, 6, 1, 20] = np.inf  # a weight
    inp.om[0, 0, 0, 1, 0] = np.inf   # an offset pushing a sample outside
    plan = d4.Plan(desc_of(s, dt))
    say("non-finite values")
    y = gpu_forward(plan, inp, dt)
    check_against_oracle(y, o.forward_f32(s, dt, inp.x, inp.om, None), dt, "non-finite")


# bf16 bit patterns at the edges of exact fp16 representability: a window
# holding only values of the first list is re-encoded as fp16, one holding any
# of the second stays bf16 (zero, magnitudes in [2^-17, 65280]; below 2^-17,
# above 65280, bf16 subnormals, inf, NaN)
F16_OK = [0x3700, 0xB700, 0x477F, 0xC77F, 0x8000, 0x0000, 0x3701, 0x387F, 0x3880]
F16_NOT = [0x36FF, 0xB6FF, 0x4780, 0xC780, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC0]
# (shape, plan options, method of option 1): the margin window with whole
# groups, the whole-image window, FlowDCN's 24-channel slices in group-scale
# mode at margin 4 (re-encoded through registers) and at its default margin
# of 5 (fifteen staging passes: bf16 unless re-encoded in LDS), and two tile
# rows per workgroup
F16_CASES = [(Shape(2, 40, 36, 64, 4), {"tile_window": 1}, 1),
             (Shape(2, 20, 22, 64, 4), {"tile_window": 2}, 1),
             (Shape(1, 33, 35, 144, 2, multiscale=True), {"tile_window": 1, "tile_margin": 4}, 1),
             (Shape(1, 33, 35, 144, 2, multiscale=True), {"tile_window": 1}, 0),
             (Shape(1, 70, 40, 64, 4), {"tile_window": 1, "tile_margin": 12, "tile_passes": 2}, 0)]


@pytest.mark.parametrize("case", range(len(F16_CASES)))
def test_f16_window_boundaries(case):
    """bf16 windows whose values all convert exactly are staged as fp16
    (re-encoded through registers or in LDS); any other window stays bf16.  Values at both sides of the boundaries
    (2^-17, 65280, subnormals, inf, NaN) are planted in some tiles' windows
    and not in others, so both encodings run in one launch; the output
    equals the oracle's and the plan without the re-encoding bit for bit."""
    s, opts, auto = F16_CASES[case]
    dt = "bf16"
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=300 + case)
    x = inp.x.view(np.uint16)
    rng = np.random.default_rng(400 + case)
    # the representable values anywhere; the others in the first image only,
    # in its top-left quarter, so that tiles of both kinds exist
    for v in F16_OK:
        n, yy, xx, c = (rng.integers(0, d) for d in x.shape)
        x[n, yy, xx, c] = v
    for v in F16_NOT:
        yy, xx = rng.integers(0, max(s.H // 4, 1)), rng.integers(0, max(s.W // 4, 1))
        x[0, yy, xx, rng.integers(0, s.C)] = v
    y_or = o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=NTHREADS)
    outs = []
    for f16w in (1, 2, 0):
        plan = d4.Plan(desc_of(s, dt), kernel=2, tile_f16_window=f16w, **opts)
        info = plan.info()
        say(f"f16 window case {case} ({f16w}): {s} {info}")
        assert info["tile_f16_window"] == (auto if f16w == 1 else f16w)
        y = gpu_forward(plan, inp, dt)
        check_against_oracle(y, y_or, dt, f"f16 window case {case} option {f16w}")
        outs.append(y)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_repeatable_and_stream_independent():
    w = WORKLOADS["dcn4_small_f32"].with_(N=4, H=33, W=29)
    s = shape_of(w)
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = make_inputs(w, Ho, Wo)
    plan = d4.Plan(desc_of(s, w.dtype))
    x, om = to_dev(inp.x, "f32"), to_dev(inp.om, "f32")
    y1 = plan.forward(x, om)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        y2 = plan.forward(x, om)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


# degenerate images: one row or column, a single pixel, images smaller than
# the kernel's footprint (every sample partly or wholly off the image)
TINY = [Shape(2, 1, 1, 32, 2), Shape(1, 1, 7, 32, 2), Shape(1, 5, 1, 16, 1),
        Shape(2, 2, 3, 64, 4), Shape(1, 3, 3, 32, 2, multiscale=True),
        Shape(1, 2, 2, 32, 2, 5, 5, ph=2, pw=2)]


@pytest.mark.parametrize("case", range(len(TINY)))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_degenerate_images(case, dt):
    """Tiny images on the automatic plan, the margin window, the whole-image
    window and the direct kernel: bit for bit with the oracle; and the
    backward within its bound."""
    s = TINY[case]
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = wide_offset_inputs(s, dt, Ho, Wo, seed=900 + case, reach=2.5)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, inp.scales, nthreads=NTHREADS)
    dp = 8 if dt == "f32" else 0
    variants = [dict(), dict(kernel=1), dict(kernel=2, tile_window=1),
                dict(kernel=2, tile_window=2)]
    for opts in variants:
        try:
            plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp, **opts)
        except d4.DCN4Error as e:
            # a forced tiled kernel may not fit some shapes' windows
            assert e.status == d4.DCN4_ERR_UNSUPPORTED and opts.get("kernel") == 2
            continue
        say(f"tiny {s} {dt} {opts}: {plan.info()}")
        check_against_oracle(gpu_forward(plan, inp, dt), y_or, dt, f"tiny {case} {opts}")
    plan = d4.Plan(desc_of(s, dt), channels_per_lane=dp)
    gy = workloads.to_raw(np.random.default_rng(5 + case).standard_normal(
        (s.N, Ho, Wo, s.C)).astype(np.float32), dt)
    ref = o.backward(s, dt, inp.x, inp.om, gy, inp.scales)
    x, om, g = to_dev(inp.x, dt), to_dev(inp.om, dt), to_dev(gy, dt)
    sc = None if inp.scales is None else torch.from_numpy(inp.scales).cuda()
    for scatter in (False, True):
        gx, gom = plan.backward(x, om, g, sc, None, scatter=scatter)
        torch.cuda.synchronize()
        for got, want, absum, what in ((gx, ref["gx"], ref["gx_abs"], "grad_x"),
                                       (gom, ref["gom"], ref["gom_abs"], "grad_om")):
            err = np.abs(got.cpu().numpy().astype(np.float64) - want)
            bound = (ref["max_terms"] + 8) * 2.0 ** -24 * absum + 1e-37
            assert (err <= bound).all(), f"tiny {case} {what} scatter={scatter}"


def test_empty_batch():
    plan = d4.Plan(d4.Desc(N=0, H=8, W=8, C=16, group=2, dtype="bf16"))
    x = torch.empty((0, 8, 8, 16), dtype=torch.bfloat16, device="cuda")
    om = torch.empty((0, 8, 8, 2, 27), dtype=torch.bfloat16, device="cuda")
    y = plan.forward(x, om)
    torch.cuda.synchronize()
    assert y.shape == (0, 8, 8, 16)
