"""The DCNv3-style comparison path through the C ABI against the oracle:
DCNv3's softmax over each (pixel, group) row's weights (dcn4_dcnv3_softmax)
and the aggregation with one thread per (output pixel, channel)
(dcn4_dcnv3_forward).

Gates, written here:
  * aggregation: the oracle's fp32 evaluation bit for bit (the kernel runs
    the same fp32 operations as dcn4_forward); zero differing elements;
  * softmax: the offsets copied bit for bit; every weight v within
    |v - w| <= u*(w + e) + e + t of the exact softmax w (the oracle, fp64),
    e = f*w with f = (2*spread + K + 12) * 2^-24 bounding the fp32 evaluation
    (the argument m_k - M rounded: |m_k - M| * 2^-24 relative after expf;
    expf itself a few ulp; a sum of K terms; one division), spread the row's
    largest minus smallest weight, u the I/O dtype's unit roundoff (0 for
    fp32, whose result is not rounded again) and t half its smallest
    subnormal step; NaN exactly where the oracle has NaN;
  * softmax then aggregation against the DCNv3 output in fp64 Y = sum_k
    w_k B_k with the sum of absolute terms A: |y - Y| <= u*(|Y| + E) + E + t,
    E = (u + 2f + (4K + 9) * 2^-24) * A + t_w * K * max|x| (the weights'
    rounding and fp32 error, the fp32 aggregation of R8, the fp32 weights of
    the reference, the weights' subnormal step t_w).
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
from test_gpu_parity import (bits_equal, desc_of, fuzz_cases, fuzz_inputs,  # noqa: E402
                             shape_of, to_dev, to_raw_np)

NTHREADS = 16
U = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
T = {"f32": 0.0, "bf16": 2.0 ** -134, "f16": 2.0 ** -25}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def row_spreads(om, dt, K):
    """largest minus smallest weight of each row (0 where not finite)"""
    m = from_raw(om, dt).astype(np.float64)[..., 2 * K:]
    with np.errstate(invalid="ignore"):
        sp = m.max(axis=-1) - m.min(axis=-1)
    return np.where(np.isfinite(sp), sp, 0.0)


def row_spread(om, dt, K):
    return float(row_spreads(om, dt, K).max(initial=0.0))


def check_softmax(got_raw, om_raw, s, dt, what):
    o = oracle.get()
    K = s.K
    want = o.softmax_weights(s, dt, om_raw)
    got = from_raw(got_raw, dt).astype(np.float64)
    # offsets: the same bits
    g_off = np.asarray(got_raw)[..., :2 * K]
    o_off = np.asarray(om_raw)[..., :2 * K]
    assert np.array_equal(g_off.view(np.uint16 if dt != "f32" else np.uint32),
                          o_off.view(np.uint16 if dt != "f32" else np.uint32)), \
        f"{what}: offsets changed"
    gw, ww = got[..., 2 * K:], want[..., 2 * K:]
    nan_w = np.isnan(ww)
    assert np.array_equal(np.isnan(gw), nan_w), f"{what}: NaN pattern differs"
    f = (2.0 * row_spreads(om_raw, dt, K)[..., None] + K + 12) * 2.0 ** -24
    e = np.broadcast_to(f, ww.shape)[~nan_w] * ww[~nan_w]
    bound = U[dt] * (ww[~nan_w] + e) + e + T[dt]
    err = np.abs(gw[~nan_w] - ww[~nan_w])
    ratio = float(np.max(err / bound, initial=0.0)) if err.size else 0.0
    exact = float(np.mean(err == 0.0)) if err.size else 1.0
    say(f"{what}: softmax weights {err.size}, largest error / bound {ratio:.3g}, "
        f"{100 * exact:.2f}% equal to the exact value's rounding")
    assert np.all(err <= bound), f"{what}: a weight beyond the bound ({ratio:.3g})"


def softmax_cases():
    return [(Shape(2, 9, 11, 16, 2), "f32"), (Shape(1, 17, 13, 24, 3), "bf16"),
            (Shape(3, 7, 5, 8, 1), "f16"),
            (Shape(1, 12, 10, 32, 4, kh=5, kw=5, ph=2, pw=2), "bf16"),
            (Shape(1, 9, 9, 8, 2, kh=3, kw=5, ph=1, pw=2), "f16"),
            (Shape(1, 8, 8, 16, 1, kh=1, kw=1, ph=0, pw=0), "f32"),
            (Shape(1, 20, 20, 16, 4, kh=7, kw=7, ph=3, pw=3), "f32"),   # 588-byte rows
            (Shape(2, 33, 31, 64, 4), "bf16")]                          # ragged workgroups


@pytest.mark.parametrize("case", range(len(softmax_cases())))
def test_softmax_parity(case):
    s, dt = softmax_cases()[case]
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    rng = np.random.default_rng(300 + case)
    K = s.K
    off = rng.uniform(-3, 3, (s.N, Ho, Wo, s.G, 2 * K)).astype(np.float32)
    m = (rng.standard_normal((s.N, Ho, Wo, s.G, K)) * [1 / 3, 1.0, 4.0][case % 3]).astype(np.float32)
    om = np.concatenate([off, m], -1)
    if dt == "f32":
        om[0, 0, 0, 0, 2 * K] = 1000.0                   # one weight takes its row
    om[0, 0, min(1, Wo - 1), 0, 2 * K + K // 2] = np.nan  # a NaN row
    om[0, min(1, Ho - 1), 0, 0, 2 * K:] = -np.inf        # a row of -inf
    if K > 1:
        om[0, min(1, Ho - 1), min(1, Wo - 1), 0, 2 * K] = -np.inf  # -inf next to finite
        om[-1, -1, -1, -1, 2 * K + 1] = np.inf           # a +inf row
    om_raw = workloads.to_raw(om, dt)
    plan = d4.Plan(desc_of(s, dt))
    say(f"softmax case {case}: {s} {dt}")
    out = plan.dcnv3_softmax(to_dev(om_raw, dt))
    torch.cuda.synchronize()
    check_softmax(to_raw_np(out, dt), om_raw, s, dt, f"softmax {case}")


@pytest.mark.parametrize("t, s, dt", [c for c in fuzz_cases(n=24, seed=4321) if not c[1].multiscale],
                         ids=lambda v: str(v) if isinstance(v, int) else None)
def test_aggregation_bit_exact(t, s, dt):
    """The one-thread-per-channel kernel equals the oracle's fp32 evaluation
    and dcn4_forward bit for bit."""
    o = oracle.get()
    Ho, Wo = o.out_size(s)
    inp = fuzz_inputs(s, dt, Ho, Wo, seed=500 + t)
    plan = d4.Plan(desc_of(s, dt))
    say(f"dcnv3 aggregation case {t}: {s} {dt}")
    x, om = to_dev(inp.x, dt), to_dev(inp.om, dt)
    y3 = plan.dcnv3_forward(x, om)
    y4 = plan.forward(x, om)
    torch.cuda.synchronize()
    y3r, y4r = to_raw_np(y3, dt), to_raw_np(y4, dt)
    y_or = o.forward_f32(s, dt, inp.x, inp.om, None, nthreads=NTHREADS)
    n_or = int((~bits_equal(y3r, y_or, dt)).sum())
    n_v4 = int((~bits_equal(y3r, y4r, dt)).sum())
    say(f"  {n_or} elements differ from the oracle, {n_v4} from dcn4_forward")
    assert n_or == 0 and n_v4 == 0


def test_aggregation_nonfinite_and_misaligned():
    """NaN/inf inputs, weights and offsets, and tensors that are only
    element-aligned: still the oracle bit for bit."""
    o = oracle.get()
    for dt in ("f32", "bf16", "f16"):
        s = Shape(2, 13, 11, 24, 3)
        Ho, Wo = o.out_size(s)
        rng = np.random.default_rng(17)
        x = rng.standard_normal((s.N, s.H, s.W, s.C)).astype(np.float32)
        x[0, 3, 4, 5] = np.nan
        x[1, 7, 2, 10] = np.inf
        off = rng.uniform(-2, 2, (s.N, Ho, Wo, s.G, 18)).astype(np.float32)
        off[0, 2, 2, 1, 4] = np.nan
        off[1, 5, 5, 0, 7] = -np.inf
        m = (rng.standard_normal((s.N, Ho, Wo, s.G, 9)) / 3).astype(np.float32)
        m[0, 6, 6, 2, 3] = np.inf
        m[1, 1, 8, 1, 0] = np.nan
        xr = workloads.to_raw(x, dt)
        omr = workloads.to_raw(np.concatenate([off, m], -1), dt)
        plan = d4.Plan(desc_of(s, dt))
        y = plan.dcnv3_forward(to_dev(xr, dt, 1), to_dev(omr, dt, 3))
        torch.cuda.synchronize()
        y_or = o.forward_f32(s, dt, xr, omr, None, nthreads=NTHREADS)
        nd = int((~bits_equal(to_raw_np(y, dt), y_or, dt)).sum())
        say(f"nonfinite/misaligned {dt}: {nd} differ")
        assert nd == 0


def test_headline_full_size():
    """The latent-diffusion U-Net block at full size: the aggregation equals
    dcn4_forward on every element and the oracle's fp32 evaluation on sampled
    pixels; softmax then aggregation against the fp64 DCNv3 output on the
    sampled pixels within the bound above; the softmax on every row."""
    w = WORKLOADS["ldm_unet_block_bf16"]
    o = oracle.get()
    s = shape_of(w)
    Ho, Wo = o.out_size(s)
    inp = make_inputs(w, Ho, Wo)
    plan = d4.Plan(desc_of(s, w.dtype))
    dt = w.dtype
    say(f"dcnv3 full size {w.describe()}")
    x, om = to_dev(inp.x, dt), to_dev(inp.om, dt)
    y3 = plan.dcnv3_forward(x, om)
    y4 = plan.forward(x, om)
    torch.cuda.synchronize()
    n_v4 = int((y3.view(torch.int16) != y4.view(torch.int16)).sum().item())
    say(f"  aggregation: {n_v4} elements differ from dcn4_forward")
    assert n_v4 == 0
    npix = s.N * Ho * Wo
    rng = np.random.default_rng(11)
    pix = np.unique(np.concatenate([rng.integers(0, npix, 1500), [0, npix - 1]]))
    y3r = to_raw_np(y3, dt).reshape(npix, s.C)[pix]
    y_or = o.forward_f32(s, dt, inp.x, inp.om, None, pix=pix, nthreads=NTHREADS)
    assert int((~bits_equal(y3r, y_or, dt)).sum()) == 0
    # softmax on every row, then DCNv3's output on the sampled pixels
    sm = plan.dcnv3_softmax(om)
    y = plan.dcnv3_forward(x, sm)
    torch.cuda.synchronize()
    check_softmax(to_raw_np(sm, dt), inp.om, s, dt, "full-size softmax")
    Y, A = o.dcnv3_forward_f64(s, dt, inp.x, inp.om, pix=pix, nthreads=NTHREADS)
    yg = from_raw(to_raw_np(y, dt).reshape(npix, s.C)[pix], dt).astype(np.float64)
    u = U[dt]
    f = (2.0 * row_spread(inp.om, dt, s.K) + s.K + 12) * 2.0 ** -24
    xmax = float(np.abs(from_raw(inp.x, dt)).max())
    E = (u + 2 * f + (4 * s.K + 9) * 2.0 ** -24) * A + T[dt] * s.K * xmax
    bound = u * (np.abs(Y) + E) + E + T[dt]
    err = np.abs(yg - Y)
    say(f"  DCNv3 output: largest error / bound {float(np.max(err / bound)):.3g}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_softmax_then_aggregation_small(dt):
    """The DCNv3 output on small seeded shapes, every pixel, within the bound."""
    o = oracle.get()
    for k, s in enumerate([Shape(2, 15, 14, 32, 4), Shape(1, 9, 12, 16, 2, kh=5, kw=5, ph=2, pw=2,
                                                           sh=2, dh=1)]):
        Ho, Wo = o.out_size(s)
        inp = fuzz_inputs(s, dt, Ho, Wo, seed=70 + k)
        plan = d4.Plan(desc_of(s, dt))
        x, om = to_dev(inp.x, dt), to_dev(inp.om, dt)
        y = plan.dcnv3_forward(x, plan.dcnv3_softmax(om))
        torch.cuda.synchronize()
        Y, A = o.dcnv3_forward_f64(s, dt, inp.x, inp.om, nthreads=NTHREADS)
        yg = from_raw(to_raw_np(y, dt), dt).astype(np.float64)
        u = U[dt]
        f = (2.0 * row_spread(inp.om, dt, s.K) + s.K + 12) * 2.0 ** -24
        xmax = float(np.abs(from_raw(inp.x, dt)).max())
        E = (u + 2 * f + (4 * s.K + 9) * 2.0 ** -24) * A + T[dt] * s.K * xmax
        bound = u * (np.abs(Y) + E) + E + T[dt]
        err = np.abs(yg - Y)
        say(f"dcnv3 {dt} case {k}: largest error / bound {float(np.max(err / bound)):.3g}")
        assert np.all(err <= bound)


def test_empty_batch():
    p0 = d4.Plan(d4.Desc(0, 8, 8, 16, 2, dtype="bf16"))
    x = torch.empty((0, 8, 8, 16), dtype=torch.bfloat16, device="cuda")
    om = torch.empty(p0.om_shape(), dtype=torch.bfloat16, device="cuda")
    assert p0.dcnv3_forward(x, om).shape[0] == 0
    assert p0.dcnv3_softmax(om).shape[0] == 0
