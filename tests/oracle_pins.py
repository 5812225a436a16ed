"""Pins of the CPU oracle: facts fixed by the pages or by mathematics that the
oracle must reproduce.  Each pin takes an ``oracle.Oracle`` and raises
AssertionError on a mismatch, so the same pins can be run against deliberately
broken oracle builds (test_oracle_mutants.py) to show that a plausible mistake
anywhere in the oracle fails at least one of them.

Pages cited (by title and section):
  [DCNv4 digest]  CSDN "（论文速读）DCNv4：高效可变形卷积算子"
  [FlowDCN]       kler.cn "NeurIPS'24 | FlowDCN：基于可变形卷积的任意分辨率图像生成模型"
  [CANN Conv2D]   intelliparadigm "CANN ops-nn 算子与 Stable Diffusion 的卷积实现"

Inputs are small and mostly dyadic (multiples of powers of two) so that the
expected values are exact in fp32 and fp64 and equality can be required.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from oracle import Shape
from workloads import from_raw, to_raw

DTYPES = ("f32", "bf16", "f16")


# ----------------------------------------------------------------- helpers
def pack_om(dx, dy, m):
    """[...,K] offsets x, offsets y, weights -> om [...,3K]: K interleaved
    (dx, dy) pairs then K weights (the boundary's layout)."""
    K = m.shape[-1]
    om = np.empty(m.shape[:-1] + (3 * K,), np.float32)
    om[..., 0:2 * K:2] = dx
    om[..., 1:2 * K:2] = dy
    om[..., 2 * K:] = m
    return om


def dyadic(rng, shape, lo, hi, denom):
    """uniform multiples of 1/denom in [lo, hi]"""
    a = rng.integers(int(round(lo * denom)), int(round(hi * denom)) + 1, size=shape)
    return (a / denom).astype(np.float32)


def run(o, s, dtype, x, om, scales=None, pscales=None, pix=None):
    """(fp64 definition, fp32 evaluation decoded to float64)"""
    xr, omr = to_raw(x, dtype), to_raw(om, dtype)
    y64 = o.forward_f64(s, dtype, xr, omr, scales, pix=pix, nthreads=2, pscales=pscales)
    y32 = from_raw(o.forward_f32(s, dtype, xr, omr, scales, pix=pix, nthreads=2,
                                 pscales=pscales), dtype).astype(np.float64)
    return y64, y32


def exact_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    if got.dtype.kind == "f" or want.dtype.kind == "f":
        got, want = got.astype(np.float64), want.astype(np.float64)
    bad = ~((got == want) | (np.isnan(got) & np.isnan(want)))
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} differ; "
                           f"first got {got[bad][:3]} want {want[bad][:3]}")


# Output size of the textbook convolution with padding and dilation
# ([CANN Conv2D] 2.1 extended), written out here independently of the oracle.
def conv_out(H, k, s, p, d):
    return (H + 2 * p - d * (k - 1) - 1) // s + 1


# ------------------------------------------------------------------- pins
def pin_output_size(o):
    """Output size equals the textbook convolution arithmetic."""
    cases = [Shape(1, 16, 16, 64, 4), Shape(2, 32, 32, 8, 2, dh=2, dw=2),
             Shape(1, 9, 7, 4, 1, kh=5, kw=3, sh=2, sw=2, ph=2, pw=0),
             Shape(1, 5, 5, 2, 2, kh=1, kw=1, ph=0, pw=0)]
    for s in cases:
        ho, wo = o.out_size(s)
        assert (ho, wo) == (conv_out(s.H, s.kh, s.sh, s.ph, s.dh),
                            conv_out(s.W, s.kw, s.sw, s.pw, s.dw)), s
    # the wide dilated block keeps padding 1 with dilation 2: 32 -> 30
    assert o.out_size(Shape(16, 32, 32, 1280, 40, dh=2, dw=2)) == (30, 30)


def pin_identity(o):
    """Zero offsets and a one-hot weight on the centre tap reproduce the input
    when the padding equals dilation*(k-1)/2 and the stride is 1."""
    rng = np.random.default_rng(1)
    for (kh, kw, dh, dw) in [(3, 3, 1, 1), (3, 3, 2, 2), (5, 5, 1, 1),
                             (3, 5, 1, 2), (1, 1, 1, 1)]:
        s = Shape(2, 7, 9, 8, 2, kh=kh, kw=kw, ph=dh * (kh - 1) // 2,
                  pw=dw * (kw - 1) // 2, dh=dh, dw=dw)
        K = kh * kw
        ho, wo = o.out_size(s)
        assert (ho, wo) == (s.H, s.W)
        x = dyadic(rng, (s.N, s.H, s.W, s.C), -4, 4, 8)
        z = np.zeros((s.N, ho, wo, s.G, K), np.float32)
        m = z.copy()
        m[..., (kh // 2) * kw + kw // 2] = 1.0
        om = pack_om(z, z, m)
        for dt in DTYPES:
            y64, y32 = run(o, s, dt, x, om)
            exact_equal(y64, x, f"identity f64 {dt} k{kh}x{kw} d{dh},{dw}")
            exact_equal(y32, x, f"identity f32 {dt} k{kh}x{kw} d{dh},{dw}")


def _gather_expected(s, x, dx, dy, m):
    """y = sum_k m_k * x[row_k, col_k] with integer rows/cols from the
    convolution index (y*s - p + i*d, [CANN Conv2D] 2.1) plus the offset;
    zero where the index leaves the image."""
    N, H, W, C = x.shape
    ho, wo = conv_out(H, s.kh, s.sh, s.ph, s.dh), conv_out(W, s.kw, s.sw, s.pw, s.dw)
    D = C // s.G
    y = np.zeros((N, ho, wo, C), np.float64)
    for n in range(N):
        for yo in range(ho):
            for xo in range(wo):
                for g in range(s.G):
                    for i in range(s.kh):
                        for j in range(s.kw):
                            k = i * s.kw + j
                            r = yo * s.sh - s.ph + i * s.dh + s.offset_scale * dy[n, yo, xo, g, k]
                            c = xo * s.sw - s.pw + j * s.dw + s.offset_scale * dx[n, yo, xo, g, k]
                            r, c = int(r), int(c)
                            if 0 <= r < H and 0 <= c < W:
                                y[n, yo, xo, g * D:(g + 1) * D] += (
                                    float(m[n, yo, xo, g, k]) *
                                    x[n, r, c, g * D:(g + 1) * D].astype(np.float64))
    return y


def pin_integer_gather(o):
    """Integer offsets make every sample land on a pixel: the output is an
    exact weighted gather of shifted input pixels (zero outside)."""
    rng = np.random.default_rng(2)
    shapes = [Shape(2, 6, 7, 6, 3),
              Shape(1, 9, 8, 4, 2, kh=3, kw=5, sh=2, sw=1, ph=0, pw=2, dh=2, dw=1),
              Shape(1, 8, 8, 4, 1, kh=2, kw=2, ph=0, pw=1),
              Shape(1, 7, 6, 4, 2, offset_scale=2.0)]
    for s in shapes:
        ho, wo = o.out_size(s)
        K = s.K
        dx = rng.integers(-3, 4, (s.N, ho, wo, s.G, K)).astype(np.float32)
        dy = rng.integers(-3, 4, (s.N, ho, wo, s.G, K)).astype(np.float32)
        # one-hot taps first, then all taps weighted
        onehot = np.zeros((s.N, ho, wo, s.G, K), np.float32)
        idx = rng.integers(0, K, (s.N, ho, wo, s.G))
        np.put_along_axis(onehot, idx[..., None], 0.5, axis=-1)
        multi = dyadic(rng, (s.N, ho, wo, s.G, K), -2, 2, 4)
        x = dyadic(rng, (s.N, s.H, s.W, s.C), -8, 8, 4)
        for m in (onehot, multi):
            want = _gather_expected(s, x, dx, dy, m)
            for dt in DTYPES:
                y64, y32 = run(o, s, dt, x, pack_om(dx, dy, m))
                exact_equal(y64, want, f"gather f64 {dt} {s}")
                exact_equal(y32, from_raw(to_raw(want, dt), dt), f"gather f32 {dt} {s}")


def pin_affine_reproduction(o):
    """Bilinear interpolation reproduces affine functions exactly: with
    x[.,r,c,ch] = a_ch*r + b_ch*c + e_ch and all four corners inside the
    image, each sample equals a*py + b*px + e at the sampled location.  This
    fixes which fraction weights rows and which columns, and the offset order
    (dx along W, dy along H)."""
    rng = np.random.default_rng(3)
    for s in [Shape(1, 12, 13, 4, 2, ph=0, pw=0),
              Shape(2, 14, 12, 6, 3, kh=3, kw=3, ph=0, pw=0, dh=2, dw=1)]:
        ho, wo = o.out_size(s)
        K = s.K
        rows = np.arange(s.H, dtype=np.float32)[:, None, None]
        cols = np.arange(s.W, dtype=np.float32)[None, :, None]
        a = rng.integers(-2, 3, s.C).astype(np.float32)
        b = rng.integers(-2, 3, s.C).astype(np.float32)
        a[0], b[0] = 1, 0  # a pure row ramp and
        a[1], b[1] = 0, 1  # a pure column ramp
        e = rng.integers(-4, 5, s.C).astype(np.float32)
        x = np.broadcast_to(a * rows + b * cols + e, (s.N, s.H, s.W, s.C)).copy()
        # multiples of 1/32 and 1/8 keep every fp32 partial sum exact
        dx = dyadic(rng, (s.N, ho, wo, s.G, K), -1.5, 1.5, 32)
        dy = dyadic(rng, (s.N, ho, wo, s.G, K), -1.5, 1.5, 32)
        m = dyadic(rng, (s.N, ho, wo, s.G, K), -1, 1, 8)
        D = s.C // s.G
        want = np.zeros((s.N, ho, wo, s.C), np.float64)
        for i in range(s.kh):
            for j in range(s.kw):
                k = i * s.kw + j
                py = (np.arange(ho)[None, :, None, None] * s.sh - s.ph + i * s.dh) + dy[..., k]
                px = (np.arange(wo)[None, None, :, None] * s.sw - s.pw + j * s.dw) + dx[..., k]
                val = (np.repeat(py, D, -1) * a + np.repeat(px, D, -1) * b + e)
                want += np.repeat(m[..., k], D, -1) * val
        # compare where every sample of the pixel is at least 1.5 px inside
        r0 = 2
        for dt in ("f32", "bf16"):
            y64, y32 = run(o, s, dt, x, pack_om(dx, dy, m))
            sl = (slice(None), slice(r0, ho - r0 - s.dh), slice(r0, wo - r0 - s.dw))
            exact_equal(y64[sl], want[sl], f"affine f64 {dt}")
            exact_equal(y32[sl], from_raw(to_raw(want[sl], dt), dt), f"affine f32 {dt}")


def _depthwise_bruteforce(x, wk, s):
    """[CANN Conv2D] 2.1's convolution, per channel (depthwise), with stride,
    zero padding and dilation; wk[c, i, j]."""
    N, H, W, C = x.shape
    ho, wo = conv_out(H, s.kh, s.sh, s.ph, s.dh), conv_out(W, s.kw, s.sw, s.pw, s.dw)
    y = np.zeros((N, ho, wo, C))
    for yo in range(ho):
        for xo in range(wo):
            for i in range(s.kh):
                for j in range(s.kw):
                    r = yo * s.sh - s.ph + i * s.dh
                    c = xo * s.sw - s.pw + j * s.dw
                    if 0 <= r < H and 0 <= c < W:
                        y[:, yo, xo, :] += x[:, r, c, :] * wk[:, i, j]
    return y


def pin_depthwise_conv(o):
    """Zero offsets and per-group weights that do not vary over pixels turn
    the operator into a depthwise convolution whose kernel is shared inside
    each group.  Checked against the textbook loop and torch's conv2d."""
    import torch
    rng = np.random.default_rng(4)
    for s in [Shape(2, 9, 8, 8, 2), Shape(1, 11, 10, 6, 3, kh=3, kw=5, sh=2, sw=1,
                                          ph=1, pw=2, dh=1, dw=2)]:
        ho, wo = o.out_size(s)
        K, D = s.K, s.C // s.G
        wg = rng.standard_normal((s.G, K)).astype(np.float32) / 3
        m = np.broadcast_to(wg, (s.N, ho, wo, s.G, K)).copy()
        z = np.zeros_like(m)
        x = rng.standard_normal((s.N, s.H, s.W, s.C)).astype(np.float32)
        wk = np.repeat(wg, D, axis=0).reshape(s.C, s.kh, s.kw).astype(np.float64)
        want = _depthwise_bruteforce(x.astype(np.float64), wk, s)
        ref = torch.nn.functional.conv2d(
            torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2),
            torch.from_numpy(wk)[:, None], stride=(s.sh, s.sw),
            padding=(s.ph, s.pw), dilation=(s.dh, s.dw), groups=s.C)
        ref = ref.permute(0, 2, 3, 1).numpy()
        np.testing.assert_allclose(want, ref, rtol=1e-12, atol=1e-12)
        y64, y32 = run(o, s, "f32", x, pack_om(z, z, m))
        scale = np.sqrt(np.mean(want ** 2))
        assert np.max(np.abs(y64 - want)) <= 1e-12 * scale, "depthwise f64"
        assert np.max(np.abs(y32 - want)) <= 1e-5 * scale, "depthwise f32"


def pin_zero_padding(o):
    """Samples far outside the image contribute exactly zero; a sample with a
    single corner inside contributes m * (corner weight) * value."""
    rng = np.random.default_rng(5)
    s = Shape(2, 6, 5, 4, 2)
    ho, wo = o.out_size(s)
    K = s.K
    sign = rng.choice([-1.0, 1.0], (s.N, ho, wo, s.G, K)).astype(np.float32)
    far = 1000.0 * sign
    m = rng.standard_normal((s.N, ho, wo, s.G, K)).astype(np.float32)
    x = rng.standard_normal((s.N, s.H, s.W, s.C)).astype(np.float32)
    for dt in DTYPES:
        y64, y32 = run(o, s, dt, x, pack_om(far, -far, m))
        exact_equal(y64, 0 * y64, f"far samples f64 {dt}")
        exact_equal(y32, 0 * y32, f"far samples f32 {dt}")
    # single-corner samples: output (0,0), tap (0,0) sits at (-1,-1)+(t,u):
    # only corner (0,0) is inside, weight t*u.  Output (Ho-1,Wo-1), tap (2,2)
    # sits at (H,W)+(t-1,u-1): only corner (H-1,W-1), weight (1-t)*(1-u).
    t, u = 0.375, 0.8125
    dx = np.zeros((s.N, ho, wo, s.G, K), np.float32)
    dy = np.zeros_like(dx)
    mm = np.zeros_like(dx)
    dy[:, 0, 0, :, 0], dx[:, 0, 0, :, 0], mm[:, 0, 0, :, 0] = t, u, 2.0
    dy[:, -1, -1, :, 8], dx[:, -1, -1, :, 8], mm[:, -1, -1, :, 8] = t - 1, u - 1, -0.5
    xd = dyadic(rng, (s.N, s.H, s.W, s.C), -4, 4, 8)
    for dt in ("f32", "bf16"):
        y64, y32 = run(o, s, dt, xd, pack_om(dx, dy, mm))
        w0 = 2.0 * t * u * xd[:, 0, 0, :]
        w1 = -0.5 * (1 - t) * (1 - u) * xd[:, -1, -1, :]
        exact_equal(y64[:, 0, 0, :], w0, f"corner (0,0) f64 {dt}")
        exact_equal(y64[:, -1, -1, :], w1, f"corner (H-1,W-1) f64 {dt}")
        exact_equal(y32[:, 0, 0, :], from_raw(to_raw(w0, dt), dt), f"corner (0,0) f32 {dt}")
        exact_equal(y32[:, -1, -1, :], from_raw(to_raw(w1, dt), dt), f"corner (H-1,W-1) f32 {dt}")
        assert not y64[:, 1:-1].any() and not y32[:, 1:-1].any()


def pin_partition_of_unity(o):
    """The four bilinear weights sum to one: a constant input c gives
    c * sum_k m_k wherever all corners are inside."""
    rng = np.random.default_rng(6)
    s = Shape(2, 12, 11, 6, 3, ph=0, pw=0)
    ho, wo = o.out_size(s)
    K = s.K
    cval = dyadic(rng, (s.C,), -3, 3, 4)
    x = np.broadcast_to(cval, (s.N, s.H, s.W, s.C)).copy()
    dx = dyadic(rng, (s.N, ho, wo, s.G, K), 0, 0.9375, 16)
    dy = dyadic(rng, (s.N, ho, wo, s.G, K), 0, 0.9375, 16)
    m = dyadic(rng, (s.N, ho, wo, s.G, K), -1, 1, 8)
    want = np.repeat(m.sum(-1), s.C // s.G, -1) * cval
    for dt in DTYPES:
        y64, y32 = run(o, s, dt, x, pack_om(dx, dy, m))
        sl = (slice(None), slice(0, ho - 1), slice(0, wo - 1))
        exact_equal(y64[sl], want[sl], f"unity f64 {dt}")
        exact_equal(y32[sl], from_raw(to_raw(want[sl], dt), dt), f"unity f32 {dt}")


def pin_linearity(o):
    """The output is linear in the weights m and in the input x (exact on
    dyadic data)."""
    rng = np.random.default_rng(7)
    s = Shape(1, 8, 9, 8, 2, sh=2, sw=1)
    ho, wo = o.out_size(s)
    K = s.K
    dx = dyadic(rng, (s.N, ho, wo, s.G, K), -2, 2, 16)
    dy = dyadic(rng, (s.N, ho, wo, s.G, K), -2, 2, 16)
    m1 = dyadic(rng, (s.N, ho, wo, s.G, K), -1, 1, 16)
    m2 = dyadic(rng, (s.N, ho, wo, s.G, K), -1, 1, 16)
    x1 = dyadic(rng, (s.N, s.H, s.W, s.C), -2, 2, 8)
    x2 = dyadic(rng, (s.N, s.H, s.W, s.C), -2, 2, 8)
    y = lambda x, m: run(o, s, "f32", x, pack_om(dx, dy, m))
    a1, b1 = y(x1, m1)
    a2, b2 = y(x1, m2)
    a3, b3 = y(x1, 2 * m1 - 0.5 * m2)
    exact_equal(a3, 2 * a1 - 0.5 * a2, "linear in m f64")
    exact_equal(b3, 2 * b1 - 0.5 * b2, "linear in m f32")
    c1, d1 = y(x2, m1)
    c3, d3 = y(x1 + x2, m1)
    exact_equal(c3, a1 + c1, "linear in x f64")
    exact_equal(d3, b1 + d1, "linear in x f32")
    assert np.abs(a1).max() > 0.5


def pin_multiscale(o):
    """FlowDCN groupwise multi-scale geometry ([FlowDCN] 3.1):
    (a) s_g = 1 with direction d equals standard mode with offset d;
    (b) integer s_g with zero direction equals standard mode with dilation s_g
        and padding p + s_g - 1 (3x3), i.e. the group samples a dilated grid;
    (c) fractional s_g on an affine input samples at centre + s_g*grid."""
    rng = np.random.default_rng(8)
    base = Shape(2, 10, 9, 8, 4, multiscale=True)
    ho, wo = o.out_size(base)
    K = base.K
    D = base.C // base.G
    x = dyadic(rng, (base.N, base.H, base.W, base.C), -4, 4, 8)
    dx = dyadic(rng, (base.N, ho, wo, base.G, K), -1, 1, 32)
    dy = dyadic(rng, (base.N, ho, wo, base.G, K), -1, 1, 32)
    m = dyadic(rng, (base.N, ho, wo, base.G, K), -1, 1, 8)
    ones = np.ones(base.G, np.float32)
    std = Shape(2, 10, 9, 8, 4)
    for dt in ("f32", "bf16"):
        a64, a32 = run(o, base, dt, x, pack_om(dx, dy, m), ones)
        b64, b32 = run(o, std, dt, x, pack_om(dx, dy, m))
        exact_equal(a64, b64, f"ms s=1 f64 {dt}")
        exact_equal(a32, b32, f"ms s=1 f32 {dt}")
    z = np.zeros_like(dx)
    sg = np.array([1, 2, 3, 2], np.float32)
    a64, a32 = run(o, base, "f32", x, pack_om(z, z, m), sg)
    for g in range(base.G):
        sgi = int(sg[g])
        st = Shape(2, 10, 9, 8, 4, ph=1 + sgi - 1, pw=1 + sgi - 1, dh=sgi, dw=sgi)
        b64, b32 = run(o, st, "f32", x, pack_om(z, z, m))
        sl = (Ellipsis, slice(g * D, (g + 1) * D))
        exact_equal(a64[sl], b64[sl], f"ms dilated group {g} f64")
        exact_equal(a32[sl], b32[sl], f"ms dilated group {g} f32")
    # (c) affine input, fractional scales, sample = centre + s*(grid + dir)
    s = Shape(1, 16, 16, 4, 2, multiscale=True)
    ho, wo = o.out_size(s)
    rows = np.arange(s.H, dtype=np.float32)[:, None, None]
    cols = np.arange(s.W, dtype=np.float32)[None, :, None]
    av = np.array([1, 0, 2, -1], np.float32)
    bv = np.array([0, 1, 1, 2], np.float32)
    xa = (av * rows + bv * cols)[None]
    sg = np.array([1.5, 2.25], np.float32)
    ddx = dyadic(rng, (1, ho, wo, s.G, K), -0.5, 0.5, 16)
    ddy = dyadic(rng, (1, ho, wo, s.G, K), -0.5, 0.5, 16)
    mm = dyadic(rng, (1, ho, wo, s.G, K), -1, 1, 4)
    want = np.zeros((1, ho, wo, s.C))
    for k in range(K):
        i, j = divmod(k, 3)
        py = np.arange(ho)[None, :, None, None] + np.repeat(sg, 2) * (i - 1 + np.repeat(ddy[..., k], 2, -1))
        px = np.arange(wo)[None, None, :, None] + np.repeat(sg, 2) * (j - 1 + np.repeat(ddx[..., k], 2, -1))
        want += np.repeat(mm[..., k], 2, -1) * (av * py + bv * px)
    y64, y32 = run(o, s, "f32", xa, pack_om(ddx, ddy, mm), sg)
    r = 5  # max reach 2.25*1.5 < 4 px: corners of rows/cols 5..10 are inside
    sl = (slice(None), slice(r, ho - r), slice(r, wo - r))
    exact_equal(y64[sl], want[sl], "ms affine f64")
    exact_equal(y32[sl], want[sl], "ms affine f32")


def pin_pixel_scales(o):
    """FlowDCN's predicted scale times the group prior, with the Smax clamp
    (reading R13 of [FlowDCN] 3.1 and 3.3), pinned to the group-scale mode
    (itself pinned above) and to closed forms:
    (a) sigma = 1 everywhere and no clamp equals the group-scale mode;
    (b) sigma = a power of two per (pixel, group) equals, pixel by pixel, the
        group-scale mode with scales s_g * sigma (the products are exact), so
        a transposed [N,Ho,Wo,G] index or a dropped factor fails;
    (c) a clamp Smax below every s_g * sigma equals the group-scale mode with
        every scale Smax; a clamp above them all changes nothing;
    (d) sigma = 0 puts all K samples on the centre pixel: y = (sum_k m_k) *
        x[centre] (zero when the centre is padding);
    (e) a NaN sigma puts that group's samples nowhere: zero output there, and
        the clamp does not turn the NaN into Smax."""
    rng = np.random.default_rng(21)
    base = Shape(2, 9, 10, 8, 4, multiscale=True)
    ps = Shape(2, 9, 10, 8, 4, multiscale=True, pixel_scales=True)
    ho, wo = o.out_size(base)
    K, G, D = base.K, base.G, base.C // base.G
    P = base.N * ho * wo
    x = dyadic(rng, (base.N, base.H, base.W, base.C), -4, 4, 8)
    dx = dyadic(rng, (base.N, ho, wo, G, K), -1, 1, 32)
    dy = dyadic(rng, (base.N, ho, wo, G, K), -1, 1, 32)
    m = dyadic(rng, (base.N, ho, wo, G, K), -1, 1, 8)
    om = pack_om(dx, dy, m)
    sg = np.array([1.0, 1.25, 2.0, 3.5], np.float32)
    # (a)
    ones = np.ones((base.N, ho, wo, G), np.float32)
    for dt in ("f32", "bf16"):
        a64, a32 = run(o, ps, dt, x, om, sg, pscales=ones)
        b64, b32 = run(o, base, dt, x, om, sg)
        exact_equal(a64, b64, f"pixel scales 1 f64 {dt}")
        exact_equal(a32, b32, f"pixel scales 1 f32 {dt}")
    # (b)
    e = (np.arange(P)[:, None] + 2 * np.arange(G)[None, :]) % 4 - 2
    sig = np.ldexp(np.ones((P, G), np.float32), e).astype(np.float32)
    a64, a32 = run(o, ps, "f32", x, om, sg, pscales=sig.reshape(base.N, ho, wo, G))
    a64 = a64.reshape(P, base.C)
    a32 = a32.reshape(P, base.C)
    for p in range(P):
        b64, b32 = run(o, base, "f32", x, om, sg * sig[p], pix=[p])
        exact_equal(a64[p], b64[0], f"pixel {p} scales f64")
        exact_equal(a32[p], b32[0], f"pixel {p} scales f32")
    # (c)
    sig = dyadic(rng, (base.N, ho, wo, G), 1, 2, 8)
    smax = 0.75
    lo = Shape(2, 9, 10, 8, 4, multiscale=True, pixel_scales=True, max_scale=smax)
    a64, a32 = run(o, lo, "f32", x, om, sg, pscales=sig)
    b64, b32 = run(o, base, "f32", x, om, np.full(G, smax, np.float32))
    exact_equal(a64, b64, "clamp below f64")
    exact_equal(a32, b32, "clamp below f32")
    hi = Shape(2, 9, 10, 8, 4, multiscale=True, pixel_scales=True, max_scale=8.0)
    a64, a32 = run(o, hi, "f32", x, om, sg, pscales=sig)
    b64, b32 = run(o, ps, "f32", x, om, sg, pscales=sig)
    exact_equal(a64, b64, "clamp above f64")
    exact_equal(a32, b32, "clamp above f32")
    # (d)
    zero = np.zeros((base.N, ho, wo, G), np.float32)
    a64, a32 = run(o, ps, "f32", x, om, sg, pscales=zero)
    want = np.zeros((base.N, ho, wo, base.C))
    msum = m.astype(np.float64).sum(-1)  # [N,ho,wo,G]
    for n in range(base.N):
        for yo in range(ho):
            for xo in range(wo):
                cy, cx = yo - base.ph + 1, xo - base.pw + 1
                if 0 <= cy < base.H and 0 <= cx < base.W:
                    want[n, yo, xo] = np.repeat(msum[n, yo, xo], D) * x[n, cy, cx]
    exact_equal(a64, want, "sigma 0 f64")
    assert np.allclose(a32, want, rtol=0, atol=1e-5), "sigma 0 f32"
    # (e)
    sig = np.ones((base.N, ho, wo, G), np.float32)
    sig[0, 3, 4, 2] = np.nan
    for shp in (ps, hi):
        a64, a32 = run(o, shp, "f32", x, om, sg, pscales=sig)
        b64, b32 = run(o, base, "f32", x, om, sg)
        sl = (0, 3, 4, slice(2 * D, 3 * D))
        exact_equal(a64[sl], np.zeros(D), "NaN sigma f64")
        exact_equal(a32[sl], np.zeros(D), "NaN sigma f32")
        b64[sl] = 0
        b32[sl] = 0
        exact_equal(a64, b64, "NaN sigma elsewhere f64")
        exact_equal(a32, b32, "NaN sigma elsewhere f32")


def _frac_offsets(rng, shape, lo, hi):
    """integer part in [lo, hi), fraction a multiple of 1/32 in [1/4, 3/4]"""
    ip = rng.integers(lo, hi, size=shape)
    fp = rng.integers(8, 25, size=shape) / 32.0
    return (ip + fp).astype(np.float32)


def _bwd_inputs(o, s, seed, scales=None):
    rng = np.random.default_rng(seed)
    ho, wo = o.out_size(s)
    K = s.K
    x = dyadic(rng, (s.N, s.H, s.W, s.C), -4, 4, 8)
    gy = dyadic(rng, (s.N, ho, wo, s.C), -2, 2, 8)
    m = dyadic(rng, (s.N, ho, wo, s.G, K), -1, 1, 8)
    if s.multiscale:
        # choose the scaled displacement t = S*(grid + d) with an in-cell
        # fraction, then d = t/S - grid (exact: S is a power of two)
        hy = (s.kh - 1) // 2
        grid_y = (np.arange(K) // s.kw - hy).astype(np.float32)
        grid_x = (np.arange(K) % s.kw - (s.kw - 1) // 2).astype(np.float32)
        S = np.asarray(scales, np.float32)[None, None, None, :, None]
        ty = _frac_offsets(rng, (s.N, ho, wo, s.G, K), -3, 3)
        tx = _frac_offsets(rng, (s.N, ho, wo, s.G, K), -3, 3)
        dy = (ty / S - grid_y).astype(np.float32)
        dx = (tx / S - grid_x).astype(np.float32)
    else:
        dy = (_frac_offsets(rng, (s.N, ho, wo, s.G, K), -2, 2) / s.offset_scale).astype(np.float32)
        dx = (_frac_offsets(rng, (s.N, ho, wo, s.G, K), -2, 2) / s.offset_scale).astype(np.float32)
    return x, dx, dy, m, gy


BWD_SHAPES = [(Shape(2, 7, 8, 8, 2), None),
              (Shape(1, 9, 6, 12, 3, sh=2, sw=1, ph=2, pw=0, dh=2, dw=1, offset_scale=0.5), None),
              (Shape(2, 8, 9, 8, 2, multiscale=True), [1.0, 2.0])]


def pin_backward_weights(o):
    """dL/dm: the forward is linear in m, so with one-hot weights on tap k it
    returns B_k, the bilinear samples of that tap; dL/dm_k = sum over the
    group's channels of gy * B_k (exact on dyadic inputs)."""
    for s, sc in BWD_SHAPES:
        x, dx, dy, m, gy = _bwd_inputs(o, s, 31, sc)
        scales = None if sc is None else np.asarray(sc, np.float32)
        for dt in ("f32", "bf16"):
            got = o.backward(s, dt, to_raw(x, dt), to_raw(pack_om(dx, dy, m), dt),
                             to_raw(gy, dt), scales, want_x=False)["gom"]
            D = s.C // s.G
            for k in range(s.K):
                onehot = np.zeros_like(m)
                onehot[..., k] = 1
                yk = o.forward_f64(s, dt, to_raw(x, dt), to_raw(pack_om(dx, dy, onehot), dt),
                                   scales, nthreads=2)
                prod = (gy.astype(np.float64) * yk).reshape(yk.shape[:-1] + (s.G, D))
                exact_equal(got[..., 2 * s.K + k], prod.sum(-1), f"dL/dm tap {k} {dt}")


def pin_backward_adjoint(o):
    """dL/dx: the forward is linear in x, so for any v,
    <gy, forward(v)> == <dL/dx, v> (exact on dyadic inputs)."""
    rng = np.random.default_rng(32)
    for s, sc in BWD_SHAPES:
        x, dx, dy, m, gy = _bwd_inputs(o, s, 33, sc)
        scales = None if sc is None else np.asarray(sc, np.float32)
        om = pack_om(dx, dy, m)
        for dt in ("f32", "f16"):
            gx = o.backward(s, dt, to_raw(x, dt), to_raw(om, dt), to_raw(gy, dt), scales,
                            want_om=False)["gx"]
            for _ in range(3):
                v = dyadic(rng, x.shape, -4, 4, 8)
                fv = o.forward_f64(s, dt, to_raw(v, dt), to_raw(om, dt), scales, nthreads=2)
                lhs = float(np.sum(gy.astype(np.float64) * fv))
                rhs = float(np.sum(gx * v.astype(np.float64)))
                assert lhs == rhs, f"adjoint {dt} {s}: {lhs} != {rhs}"


def pin_backward_offsets(o):
    """dL/d offsets: inside its cell the bilinear sample is linear in each
    coordinate, so shifting the offsets of tap k by h = 2^-10 (every sample
    stays in its cell) changes the loss <gy, y> by exactly h times the
    gradient, for each axis; this also fixes the factor offset_scale
    (standard) or the group scale (multi-scale)."""
    h = 2.0 ** -10
    for s, sc in BWD_SHAPES:
        x, dx, dy, m, gy = _bwd_inputs(o, s, 34, sc)
        scales = None if sc is None else np.asarray(sc, np.float32)
        dt = "f32"
        got = o.backward(s, dt, x, pack_om(dx, dy, m), gy, scales, want_x=False)["gom"]
        y0 = o.forward_f64(s, dt, x, pack_om(dx, dy, m), scales, nthreads=2)
        D = s.C // s.G
        for k in range(s.K):
            for axis, (ddx, ddy) in enumerate(((h, 0.0), (0.0, h))):
                dx2, dy2 = dx.copy(), dy.copy()
                dx2[..., k] += np.float32(ddx)
                dy2[..., k] += np.float32(ddy)
                y1 = o.forward_f64(s, dt, x, pack_om(dx2, dy2, m), scales, nthreads=2)
                want = ((gy.astype(np.float64) * (y1 - y0)).reshape(y0.shape[:-1] + (s.G, D))
                        .sum(-1) / h)
                exact_equal(got[..., 2 * k + axis], want, f"dL/d offset tap {k} axis {axis} {s}")


def _scale_grad_inputs(o, s, seed, S):
    """dyadic inputs whose samples sit at fractions 1/4, 1/2 or 3/4 of their
    cells for the effective scale S [N,Ho,Wo,G] (powers of two): the scaled
    displacement t = S*(grid + d) is chosen first, then d = t/S - grid."""
    rng = np.random.default_rng(seed)
    ho, wo = o.out_size(s)
    K = s.K
    x = dyadic(rng, (s.N, s.H, s.W, s.C), -2, 2, 8)
    gy = dyadic(rng, (s.N, ho, wo, s.C), -2, 2, 8)
    m = dyadic(rng, (s.N, ho, wo, s.G, K), -1, 1, 8)
    grid_y = (np.arange(K) // s.kw - (s.kh - 1) // 2).astype(np.float32)
    grid_x = (np.arange(K) % s.kw - (s.kw - 1) // 2).astype(np.float32)
    St = S[..., None]
    shape = (s.N, ho, wo, s.G, K)
    ty = rng.integers(-3, 3, size=shape) + rng.integers(1, 4, size=shape) / 4.0
    tx = rng.integers(-3, 3, size=shape) + rng.integers(1, 4, size=shape) / 4.0
    dy = (ty / St - grid_y).astype(np.float32)
    dx = (tx / St - grid_x).astype(np.float32)
    return x, pack_om(dx, dy, m), gy


def pin_backward_scales(o):
    """Gradients of FlowDCN's scales (reading R17): inside its cell the
    bilinear sample is a polynomial of degree 2 in a step h of the scale
    (both coordinates move by h*(grid + direction)), so the symmetric
    difference (L(s + h) - L(s - h)) / 2h of the loss L = <gy, y> is exactly
    its derivative on dyadic inputs with every sample kept in its cell:
    (a) per group prior s_g, with some groups above the clamp Smax (their
        effective scale is the constant Smax: derivative 0);
    (b) the predicted per-pixel scales along a random dyadic direction v:
        the difference equals sum dL/dsigma * v, pixels above the clamp
        included (zero there), and the prior's gradient sums sigma * dL/dS."""
    h = 2.0 ** -6
    loss = lambda s_, x, om, gy, sc, ps=None: float(np.sum(
        gy.astype(np.float64) * o.forward_f64(s_, "f32", x, om, sc, nthreads=2, pscales=ps)))
    # (a) group priors, groups 2 and 3 clamped (s_g = 4 > Smax = 2); no
    # prior at the clamp itself, where the derivative is one-sided
    s = Shape(2, 7, 8, 8, 4, multiscale=True, max_scale=2.0)
    ho, wo = o.out_size(s)
    sg = np.array([1.0, 0.5, 4.0, 4.0], np.float32)
    S = np.broadcast_to(np.minimum(sg, 2.0), (s.N, ho, wo, s.G)).astype(np.float32)
    x, om, gy = _scale_grad_inputs(o, s, 51, S)
    got = o.backward_scales(s, "f32", x, om, gy, sg)["gs"]
    for g in range(s.G):
        up, dn = sg.copy(), sg.copy()
        up[g] += np.float32(h)
        dn[g] -= np.float32(h)
        want = (loss(s, x, om, gy, up) - loss(s, x, om, gy, dn)) / (2 * h)
        assert got[g] == want, f"dL/ds_g group {g}: {got[g]} != {want}"
    assert got[2] == 0.0 and got[3] == 0.0
    # (b) pixel scales: sigma in {1/2, 1, 2}, priors 1/2 and 8, Smax 2: group
    # 0 below the clamp (S <= 1), group 1 above it (S = 2)
    s = Shape(2, 6, 7, 8, 2, multiscale=True, pixel_scales=True, max_scale=2.0)
    ho, wo = o.out_size(s)
    rng = np.random.default_rng(52)
    sg = np.array([0.5, 8.0], np.float32)
    sig = np.ldexp(np.ones((s.N, ho, wo, s.G), np.float32),
                   rng.integers(-1, 2, size=(s.N, ho, wo, s.G))).astype(np.float32)
    S = np.minimum(sg * sig, 2.0).astype(np.float32)
    x, om, gy = _scale_grad_inputs(o, s, 53, S)
    r = o.backward_scales(s, "f32", x, om, gy, sg, sig)
    v = rng.choice(np.array([-1.0, -0.5, 0.5, 1.0], np.float32), size=sig.shape)
    up = (sig + np.float32(h) * v).astype(np.float32)
    dn = (sig - np.float32(h) * v).astype(np.float32)
    want = (loss(s, x, om, gy, sg, up) - loss(s, x, om, gy, sg, dn)) / (2 * h)
    got = float(np.sum(r["gp"] * v.astype(np.float64)))
    assert got == want, f"dL/dsigma along v: {got} != {want}"
    clamped = sg * sig > 2.0
    assert clamped.any() and np.all(r["gp"][clamped] == 0.0)
    assert np.any(r["gp"][~clamped] != 0.0)
    for g in range(s.G):
        up, dn = sg.copy(), sg.copy()
        up[g] += np.float32(h)
        dn[g] -= np.float32(h)
        want = (loss(s, x, om, gy, up, sig) - loss(s, x, om, gy, dn, sig)) / (2 * h)
        assert r["gs"][g] == want, f"dL/ds_g with pixel scales, group {g}"


def pin_offset_linear(o):
    """The merged offset/weight layer ([DCNv4 digest] "方法3"):
    (a) an identity weight returns the features plus the bias;
    (b) one-hot features pick weight columns;
    (c) on dyadic inputs it equals numpy's matrix product exactly;
    (d) it is linear in the features."""
    rng = np.random.default_rng(41)
    M, Cin = 37, 32
    feat = dyadic(rng, (M, Cin), -4, 4, 8)
    bias = dyadic(rng, (Cin,), -2, 2, 4)
    for dt in ("f32", "bf16", "f16"):
        eye = np.eye(Cin, dtype=np.float32)
        out, _ = o.linear(dt, to_raw(feat, dt), to_raw(eye, dt), bias)
        exact_equal(out, feat.astype(np.float64) + bias, f"identity {dt}")
    W = dyadic(rng, (27, Cin), -1, 1, 16)
    onehot = np.zeros((Cin, Cin), np.float32)
    onehot[np.arange(Cin), np.arange(Cin)[::-1]] = 1
    out, _ = o.linear("f32", onehot, W, None)
    exact_equal(out, W.T[::-1].astype(np.float64), "one-hot rows")
    out, absum = o.linear("f32", feat, W, bias[:27])
    exact_equal(out, feat.astype(np.float64) @ W.T.astype(np.float64) + bias[:27], "matmul")
    assert np.all(absum >= np.abs(out) - 1e-12)
    f2 = dyadic(rng, (M, Cin), -4, 4, 8)
    o1, _ = o.linear("f32", feat, W, None)
    o2, _ = o.linear("f32", f2, W, None)
    o3, _ = o.linear("f32", feat + f2, W, None)
    exact_equal(o3, o1 + o2, "linearity")


def pin_nonfinite_offsets(o):
    """A NaN or infinite offset puts the sample nowhere in the image: the
    output equals the one where that point's weight is zero."""
    rng = np.random.default_rng(9)
    s = Shape(1, 6, 6, 4, 2)
    ho, wo = o.out_size(s)
    K = s.K
    dx = dyadic(rng, (1, ho, wo, s.G, K), -1, 1, 16)
    dy = dyadic(rng, (1, ho, wo, s.G, K), -1, 1, 16)
    m = dyadic(rng, (1, ho, wo, s.G, K), -1, 1, 8)
    x = dyadic(rng, (1, s.H, s.W, s.C), -2, 2, 8)
    dx2, dy2, m0 = dx.copy(), dy.copy(), m.copy()
    dx2[..., 4] = np.nan
    dy2[..., 2] = np.inf
    m0[..., 4] = 0
    m0[..., 2] = 0
    for dt in ("f32", "bf16", "f16"):
        a64, a32 = run(o, s, dt, x, pack_om(dx2, dy2, m))
        b64, b32 = run(o, s, dt, x, pack_om(dx, dy, m0))
        exact_equal(a64, b64, f"non-finite offsets f64 {dt}")
        exact_equal(a32, b32, f"non-finite offsets f32 {dt}")


def _cost_model():
    """The cost-model figures printed on the DCNv4 digest page (golden file)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "dcnv4_cost_model.json")) as f:
        return json.load(f)


def pin_term_count(o):
    """The definition has 4 bilinear corner terms per sample point and
    channel: 36*H*W*C per image for 3x3 with H and W kept ([DCNv4 digest],
    "GPU效率的理论分析")."""
    cm = _cost_model()
    f = cm["flops_per_HWC"]
    assert f == cm["flops_factors"]["spatial_points"] * cm["flops_factors"]["bilinear_corners"]
    rng = np.random.default_rng(10)
    for s, want in [(Shape(1, 16, 16, 64, 4), f * 16 * 16 * 64),
                    (Shape(3, 10, 12, 8, 2), 3 * f * 10 * 12 * 8),
                    (Shape(1, 9, 9, 4, 1, kh=5, kw=5, ph=2, pw=2), 4 * 25 * 81 * 4)]:
        ho, wo = o.out_size(s)
        om = rng.uniform(-3, 3, (s.N, ho, wo, s.G, 3 * s.K)).astype(np.float32)
        terms, inb = o.count_terms(s, "f32", om)
        assert terms == want, (terms, want)
        assert 0 < inb < terms


def pin_ideal_bytes(o):
    """Ideal traffic 2HWC + 27HWG elements for 3x3 ([DCNv4 digest],
    "GPU效率的理论分析"); about 3.7HWC when G = C/16; the no-cache worst case is
    36 + 27 + 1 = 64 accesses per output, about 17x the ideal; compute to
    memory ratios from about 0.6 to 9.7 (figures in the golden file)."""
    cm = _cost_model()
    a, b = cm["ideal_elements"]["HWC"], cm["ideal_elements"]["HWG"]
    s = Shape(1, 16, 16, 64, 4)
    assert o.ideal_bytes(s, "f32") == 4 * (a * 16 * 16 * 64 + b * 16 * 16 * 4)
    s = Shape(8, 128, 128, 320, 20)
    assert o.ideal_bytes(s, "bf16") == 2 * 8 * (a * 128 * 128 * 320 + b * 128 * 128 * 20)
    assert o.ideal_bytes(s, "bf16") == 309_329_920
    ratio = a + b / 16
    assert abs(ratio - cm["ideal_at_G_eq_C_over_16_HWC"]) < 0.02
    wc = cm["worst_case_accesses_per_output"]
    assert wc["interpolation_reads"] == cm["flops_per_HWC"]
    assert wc["offset_weight_reads"] == b
    assert wc["total"] == wc["interpolation_reads"] + wc["offset_weight_reads"] + wc["writes"]
    assert abs(wc["total"] / ratio - cm["worst_over_ideal"]) < 0.5
    lo, hi = cm["compute_to_memory_ratio_range"]
    assert abs(cm["flops_per_HWC"] / wc["total"] - lo) < 0.05
    assert abs(cm["flops_per_HWC"] / ratio - hi) < 0.1
    # Ho != H: input and output counted at their own sizes, fp32 scales added
    s = Shape(16, 32, 32, 1280, 40, dh=2, dw=2)
    assert o.ideal_bytes(s, "f16") == 2 * (16 * 32 * 32 * 1280 + 16 * 30 * 30 * 1280
                                           + 16 * 30 * 30 * 40 * 27)
    s = Shape(32, 32, 32, 1152, 16, multiscale=True)
    assert o.ideal_bytes(s, "bf16") == 2 * 32 * (2 * 32 * 32 * 1152 + 27 * 32 * 32 * 16) + 64


def _exact_definition(s, x, dx, dy, m, sg=None):
    """The definition in exact rational arithmetic (tiny shapes only)."""
    N, H, W, C = x.shape
    ho, wo = conv_out(H, s.kh, s.sh, s.ph, s.dh), conv_out(W, s.kw, s.sw, s.pw, s.dw)
    D = C // s.G
    y = np.empty((N, ho, wo, C), object)
    for n in range(N):
        for yo in range(ho):
            for xo in range(wo):
                for g in range(s.G):
                    for d in range(D):
                        c = g * D + d
                        acc = Fraction(0)
                        for i in range(s.kh):
                            for j in range(s.kw):
                                k = i * s.kw + j
                                ddy = Fraction(float(dy[n, yo, xo, g, k]))
                                ddx = Fraction(float(dx[n, yo, xo, g, k]))
                                if s.multiscale:
                                    hy, hx = (s.kh - 1) // 2, (s.kw - 1) // 2
                                    S = Fraction(float(sg[g]))
                                    py = yo * s.sh - s.ph + hy + S * (i - hy + ddy)
                                    px = xo * s.sw - s.pw + hx + S * (j - hx + ddx)
                                else:
                                    os_ = Fraction(s.offset_scale)
                                    py = yo * s.sh - s.ph + i * s.dh + os_ * ddy
                                    px = xo * s.sw - s.pw + j * s.dw + os_ * ddx
                                y0, x0 = math.floor(py), math.floor(px)
                                lh, lw = py - y0, px - x0
                                v = Fraction(0)
                                for a, wa in ((0, 1 - lh), (1, lh)):
                                    for b, wb in ((0, 1 - lw), (1, lw)):
                                        r, cc = y0 + a, x0 + b
                                        if 0 <= r < H and 0 <= cc < W:
                                            v += wa * wb * Fraction(float(x[n, r, cc, c]))
                                acc += Fraction(float(m[n, yo, xo, g, k])) * v
                        y[n, yo, xo, c] = acc
    return y


def pin_exact_rational(o):
    """On tiny random inputs the fp64 definition agrees with exact rational
    arithmetic to 1e-12, and the fp32 evaluation to the fp32 error bound
    (1e-5 of the output RMS, the fp32 tolerance)."""
    rng = np.random.default_rng(11)
    for s in [Shape(1, 5, 6, 4, 2), Shape(1, 6, 5, 4, 2, sh=2, sw=1, dh=2, dw=1, ph=2),
              Shape(1, 5, 5, 4, 2, offset_scale=0.75),
              Shape(1, 6, 6, 4, 2, multiscale=True)]:
        ho, wo = o.out_size(s)
        K = s.K
        x = rng.standard_normal((1, s.H, s.W, s.C)).astype(np.float32)
        dx = rng.uniform(-2, 2, (1, ho, wo, s.G, K)).astype(np.float32)
        dy = rng.uniform(-2, 2, (1, ho, wo, s.G, K)).astype(np.float32)
        m = (rng.standard_normal((1, ho, wo, s.G, K)) / 3).astype(np.float32)
        sg = np.array([1.0, 2.5], np.float32) if s.multiscale else None
        ex = _exact_definition(s, x, dx, dy, m, sg).astype(np.float64)
        y64, y32 = run(o, s, "f32", x, pack_om(dx, dy, m), sg)
        rms = np.sqrt(np.mean(ex ** 2))
        assert np.max(np.abs(y64 - ex)) <= 1e-12 * rms, f"exact f64 {s}"
        assert np.max(np.abs(y32 - ex)) <= 1e-5 * rms, f"exact f32 {s}"


def pin_geometry(o):
    """Sample locations next to integers and at the image border: integer
    part, fraction and the inside test (integer part in [-1,H-1]) are fixed.
    The fraction comes from the offset alone, so it stays exact even for a
    subnormal offset."""
    s = Shape(1, 16, 16, 4, 1, kh=1, kw=1, ph=0, pw=0)
    ho, wo = o.out_size(s)
    e = 2.0 ** -20
    # (output row, dy, expected inside, y0, lh); case number q sits at output
    # column q with dx = 0.25
    cases = [(5, -e, 1, 4, 1 - e), (5, e, 1, 5, e), (5, -0.0, 1, 5, 0.0),
             (0, -1.0, 1, -1, 0.0), (0, -1 + e, 1, -1, e), (0, -0.5, 1, -1, 0.5),
             (15, 1 - 2 * e, 1, 15, 1 - 2 * e), (15, 1.0, 0, 0, 0.0),
             (2, 2.0 ** -149, 1, 2, 2.0 ** -149), (0, 2.0 ** -149, 1, 0, 2.0 ** -149),
             (0, -1.0 - e, 0, 0, 0.0), (15, 0.5, 1, 15, 0.5)]
    om = np.zeros((1, ho, wo, 1, 3), np.float32)
    om[..., 2] = 1
    om[..., 0] = 0.25
    for q, (r, d, *_rest) in enumerate(cases):
        om[0, r, q, 0, 1] = d
    g = o.geometry(s, "f32", om)
    for q, (r, d, ins, y0, lh) in enumerate(cases):
        t = r * wo + q
        assert g["inside"][t] == ins, (r, d)
        if ins:
            assert g["y0"][t] == y0 and g["lh"][t] == np.float32(lh), (r, d, g["y0"][t], g["lh"][t])
            assert g["x0"][t] == q and g["lw"][t] == 0.25
    # column direction and the stride/dilation base on a 3x3 dilated, strided grid
    s = Shape(1, 20, 20, 4, 1, sh=2, sw=3, ph=1, pw=2, dh=2, dw=1)
    ho, wo = o.out_size(s)
    om = np.zeros((1, ho, wo, 1, 27), np.float32)
    om[..., 0:18:2] = 0.5     # dx
    om[..., 1:18:2] = -0.25   # dy
    g = o.geometry(s, "f32", om)
    for yo in range(ho):
        for xo in range(wo):
            for k in range(9):
                i, j = divmod(k, 3)
                t = (yo * wo + xo) * 9 + k
                py = yo * 2 - 1 + 2 * i - 0.25
                px = xo * 3 - 2 + j + 0.5
                inside = -1 <= math.floor(py) <= 19 and -1 <= math.floor(px) <= 19
                assert g["inside"][t] == inside
                if inside:
                    assert g["y0"][t] == math.floor(py) and g["lh"][t] == py - math.floor(py)
                    assert g["x0"][t] == math.floor(px) and g["lw"][t] == px - math.floor(px)


def pin_codecs(o):
    """bf16/fp16 decode is exact and encode rounds to nearest even: checked
    against torch's bf16 cast and numpy's float16 cast (library routines)."""
    import torch
    # every fp16 pattern decodes like numpy
    allh = np.arange(65536, dtype=np.uint16)
    ref = allh.view(np.float16).astype(np.float32)
    got = np.array([o.f16_to_f32(int(h)) for h in allh[::7]], np.float32)
    exact_equal(got, ref[::7], "f16 decode")
    # bf16 decode: a few known patterns
    for h, v in [(0x3F80, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -133), (0x7F80, np.inf)]:
        assert o.bf16_to_f32(h) == v
    rng = np.random.default_rng(12)
    f = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 4000),
        np.array([0.0, -0.0, 1.0, 65504, 65519.996, 65520, 1e-8, 6e-8, 2.0 ** -24,
                  2.0 ** -25, 2.0 ** -25 * 1.5, 2.0 ** -14, np.inf, -np.inf, 3.0e38], np.float32),
        # exact halfway cases for bf16 (ties to even both ways)
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80C000],
                 np.uint32).view(np.float32)])
    with np.errstate(over="ignore"):
        want16 = f.astype(np.float16).view(np.uint16)
    got16 = np.array([o.f32_to_f16(float(v)) for v in f], np.uint16)
    exact_equal(got16, want16, "f16 encode")
    wantb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gotb = np.array([o.f32_to_bf16(float(v)) for v in f], np.uint16)
    exact_equal(gotb, wantb, "bf16 encode")
    assert np.isnan(o.bf16_to_f32(o.f32_to_bf16(float("nan"))))
    assert np.isnan(o.f16_to_f32(o.f32_to_f16(float("nan"))))


def pin_dwconv3x3(o):
    """The depthwise 3x3 convolution in front of the offset/weight layer
    ([DCNv4 digest] "方法3"):
    (a) the identity kernel (centre tap 1) returns the input, all dtypes;
    (b) a single top-left tap moves the image one pixel down and right, with
        zeros shifted in (fixes the tap orientation and the zero padding);
    (c) a constant image c: interior outputs c * sum(w) + b, a corner pixel
        c * (the four taps that stay inside) + b;
    (d) equals torch's grouped conv2d (groups = C, padding 1; a library
        routine) in fp64 on dyadic inputs, and the fp32 evaluation equals it
        exactly there (every product and partial sum is exact);
    (e) linear in the input."""
    import torch
    rng = np.random.default_rng(53)
    N, H, W, C = 2, 7, 9, 5
    x = dyadic(rng, (N, H, W, C), -4, 4, 8)
    for dt in ("f32", "bf16", "f16"):
        w = np.zeros((3, 3, C), np.float32)
        w[1, 1, :] = 1.0
        a, r = o.dwconv3x3(dt, to_raw(x, dt), to_raw(w, dt))
        exact_equal(a, x.astype(np.float64), f"identity f64 {dt}")
        exact_equal(from_raw(r, dt), x, f"identity raw {dt}")
    w = np.zeros((3, 3, C), np.float32)
    w[0, 0, :] = 0.5
    a, _ = o.dwconv3x3("f32", x, w)
    want = np.zeros_like(x, dtype=np.float64)
    want[:, 1:, 1:, :] = 0.5 * x[:, :-1, :-1, :]
    exact_equal(a, want, "top-left tap")
    cst = np.full((1, 4, 6, C), 0.75, np.float32)
    w = dyadic(rng, (3, 3, C), -2, 2, 4)
    b = dyadic(rng, (C,), -1, 1, 4)
    a, _ = o.dwconv3x3("f32", cst, w, b)
    exact_equal(a[0, 1:3, 1:5, :], np.broadcast_to(0.75 * w.astype(np.float64).sum((0, 1)) + b,
                                                 (2, 4, C)), "constant interior")
    exact_equal(a[0, 0, 0, :], 0.75 * w[1:, 1:, :].astype(np.float64).sum((0, 1)) + b,
                "constant corner")
    w = dyadic(rng, (3, 3, C), -2, 2, 16)
    a, r = o.dwconv3x3("f32", x, w, b)
    ref = torch.nn.functional.conv2d(
        torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2),
        torch.from_numpy(w.astype(np.float64)).permute(2, 0, 1).unsqueeze(1),
        torch.from_numpy(b.astype(np.float64)), padding=1, groups=C).permute(0, 2, 3, 1).numpy()
    exact_equal(a, ref, "grouped conv2d")
    exact_equal(r, ref, "fp32 evaluation on exact data")
    x2 = dyadic(rng, (N, H, W, C), -4, 4, 8)
    a1, _ = o.dwconv3x3("f32", x, w)
    a2, _ = o.dwconv3x3("f32", x2, w)
    a3, _ = o.dwconv3x3("f32", x + x2, w)
    exact_equal(a3, a1 + a2, "linearity")


def pin_softmax_weights(o):
    """DCNv3's softmax over each (pixel, group) row's K weights (reading R18;
    [DCNv4 digest] section 1 names it as the step DCNv4 removes):
    (a) equal weights give the uniform 1/K; a 1x1 kernel gives exactly 1;
    (b) equals scipy's softmax (library routine) along the K weights of each
        (pixel, group), every dtype, with the offsets passed through unchanged;
    (c) adding a constant to a row's weights changes nothing;
    (d) a weight of 1000 (fp32) takes the whole row without overflow;
    (e) a NaN or +inf weight makes its row NaN and only its row; -inf
        weights get 0 next to finite ones;
    (f) with zero offsets and equal weights the DCNv3 output is the K-point
        box average: torch's depthwise conv2d with a 1/K kernel."""
    import scipy.special
    import torch
    rng = np.random.default_rng(61)
    # (a)
    s = Shape(1, 5, 6, 8, 2)
    ho, wo = o.out_size(s)
    z = np.zeros((s.N, ho, wo, s.G, s.K), np.float32)
    m = np.broadcast_to(dyadic(rng, (s.N, ho, wo, s.G, 1), -2, 2, 4), z.shape)
    w = o.softmax_weights(s, "f32", pack_om(z, z, m))[..., 2 * s.K:]
    assert np.all(w == 1.0 / s.K), "equal weights: uniform"
    s1 = Shape(1, 4, 5, 6, 3, kh=1, kw=1, ph=0, pw=0)
    ho1, wo1 = o.out_size(s1)
    om1 = rng.standard_normal((s1.N, ho1, wo1, s1.G, 3)).astype(np.float32) * 4
    assert np.all(o.softmax_weights(s1, "f32", om1)[..., 2] == 1.0), "1x1: weight 1"
    # (b)
    for dtype, s in [("f32", Shape(2, 6, 7, 12, 3)), ("bf16", Shape(1, 5, 5, 8, 4, kh=3, kw=5, pw=2)),
                     ("f16", Shape(1, 6, 4, 4, 1, sh=2))]:
        ho, wo = o.out_size(s)
        om = (rng.standard_normal((s.N, ho, wo, s.G, 3 * s.K)) * 2).astype(np.float32)
        raw = to_raw(om, dtype)
        dec = from_raw(raw, dtype).astype(np.float64)
        got = o.softmax_weights(s, dtype, raw)
        exact_equal(got[..., :2 * s.K], dec[..., :2 * s.K], f"offsets unchanged {dtype}")
        want = scipy.special.softmax(dec[..., 2 * s.K:], axis=-1)
        np.testing.assert_allclose(got[..., 2 * s.K:], want, rtol=1e-14, atol=0,
                                   err_msg=f"softmax {dtype}")
    # (c)
    s = Shape(1, 4, 4, 4, 2)
    ho, wo = o.out_size(s)
    om = dyadic(rng, (s.N, ho, wo, s.G, 3 * s.K), -3, 3, 16)
    om2 = om.copy()
    om2[..., 2 * s.K:] += 5.0
    np.testing.assert_allclose(o.softmax_weights(s, "f32", om2),
                               o.softmax_weights(s, "f32", om), rtol=1e-14, atol=0,
                               err_msg="shift invariance")
    # (d)
    om3 = om.copy()
    om3[..., 2 * s.K:] = 0.0
    om3[..., 2 * s.K + 4] = 1000.0
    w = o.softmax_weights(s, "f32", om3)[..., 2 * s.K:]
    assert np.all(w[..., 4] == 1.0) and np.all(np.delete(w, 4, axis=-1) == 0.0), "large weight"
    # (e)
    om4 = om.copy()
    om4[0, 1, 2, 0, 2 * s.K + 3] = np.nan
    om4[0, 2, 1, 1, 2 * s.K + 7] = np.inf
    om4[0, 3, 3, 0, 2 * s.K:2 * s.K + 4] = -np.inf
    w = o.softmax_weights(s, "f32", om4)[..., 2 * s.K:]
    ref = o.softmax_weights(s, "f32", om)[..., 2 * s.K:]
    assert np.all(np.isnan(w[0, 1, 2, 0])) and np.all(np.isnan(w[0, 2, 1, 1])), "NaN rows"
    assert np.all(w[0, 3, 3, 0, :4] == 0.0) and np.isclose(w[0, 3, 3, 0].sum(), 1.0, rtol=1e-15)
    keep = np.ones(w.shape[:-1], bool)
    keep[0, 1, 2, 0] = keep[0, 2, 1, 1] = keep[0, 3, 3, 0] = False
    exact_equal(w[keep], ref[keep], "other rows untouched")
    # (f)
    s = Shape(2, 7, 9, 6, 3)
    ho, wo = o.out_size(s)
    x = rng.standard_normal((s.N, s.H, s.W, s.C)).astype(np.float32)
    z = np.zeros((s.N, ho, wo, s.G, s.K), np.float32)
    mm = np.broadcast_to(rng.standard_normal((s.N, ho, wo, s.G, 1)).astype(np.float32), z.shape)
    y, a = o.dcnv3_forward_f64(s, "f32", x, pack_om(z, z, mm))
    ref = torch.nn.functional.conv2d(
        torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2),
        torch.full((s.C, 1, 3, 3), 1.0 / 9.0, dtype=torch.float64), padding=1, groups=s.C)
    ref = ref.permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-6 * np.abs(ref).max(),
                               err_msg="DCNv3 box average")
    assert np.all(a >= np.abs(y) - 1e-12), "absolute sum bounds the output"


ALL_PINS = [pin_output_size, pin_identity, pin_integer_gather,
            pin_affine_reproduction, pin_depthwise_conv, pin_zero_padding,
            pin_partition_of_unity, pin_linearity, pin_multiscale,
            pin_pixel_scales, pin_nonfinite_offsets, pin_term_count, pin_ideal_bytes,
            pin_exact_rational, pin_geometry, pin_codecs, pin_backward_weights,
            pin_backward_adjoint, pin_backward_offsets, pin_backward_scales,
            pin_offset_linear, pin_dwconv3x3, pin_softmax_weights]


if __name__ == "__main__":
    # Run every pin against the oracle library given on the command line and
    # report the first one that fails (used on mutant builds, in a child
    # process so that a crashing mutant cannot take the test runner down).
    import sys
    import oracle as _oracle
    lib = _oracle.Oracle(sys.argv[1])
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError as e:
            print(f"CAUGHT {pin.__name__}: {str(e)[:200]}")
            sys.exit(0)
        except ValueError as e:  # the mutant rejected a valid shape
            print(f"CAUGHT {pin.__name__} (rejected): {str(e)[:200]}")
            sys.exit(0)
    print("MISSED")
