"""Parity of the depthwise 3x3 convolution (dcn4_dwconv3x3) with the oracle.

The kernel and the oracle's fp32 evaluation perform the same operations in
the same order (an fma per tap in row-major order, taps outside the image
skipped, then the bias, one rounding to the I/O dtype), so every output must
be bit-identical; fp32 outputs are also checked against the fp64 definition
(relative error <= 1e-5 of |y| + RMS(y))."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
from test_gpu_parity import say  # noqa: E402
from workloads import from_raw, to_raw  # noqa: E402

import dynamic_sparse_vision_dcn4_amd as d4  # noqa: E402

pytestmark = pytest.mark.gpu
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def dev(raw, dt, offset_elems=0):
    if dt == "f32":
        t = torch.from_numpy(np.ascontiguousarray(raw))
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(TDT[dt])
    if offset_elems:
        # a view that starts offset_elems elements into a larger allocation
        big = torch.empty(t.numel() + offset_elems, dtype=t.dtype, device="cuda")
        return big[offset_elems:].view(t.shape).copy_(t.cuda())
    return t.cuda()


def host_raw(t, dt):
    t = t.cpu()
    return t.numpy() if dt == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def inputs(N, H, W, C, dt, seed, with_bias=True):
    rng = np.random.default_rng(seed)
    x = to_raw(rng.standard_normal((N, H, W, C), dtype=np.float32), dt)
    w = to_raw(rng.standard_normal((3, 3, C), dtype=np.float32) / np.float32(3.0), dt)
    b = rng.standard_normal(C, dtype=np.float32) * np.float32(0.5) if with_bias else None
    return x, w, b


def check(got_raw, x, w, b, dt, what):
    o = oracle.get()
    y64, want = o.dwconv3x3(dt, x, w, b)
    g = np.asarray(got_raw)
    bits = g.view(np.uint32) if dt == "f32" else g
    wbits = want.view(np.uint32) if dt == "f32" else want
    gv, wv = from_raw(g, dt), from_raw(want, dt)
    same = (bits == wbits) | (np.isnan(gv) & np.isnan(wv))
    say(f"{what}: {int((~same).sum())} of {same.size} differ from the oracle")
    assert same.all(), f"{what}: first differences at {np.argwhere(~same)[:3].tolist()}"
    if dt == "f32":
        fin = np.isfinite(y64)
        rms = np.sqrt(np.mean(y64[fin] ** 2)) if fin.any() else 1.0
        err = np.abs(gv.astype(np.float64) - y64)[fin] / (np.abs(y64[fin]) + rms)
        assert err.size == 0 or err.max() <= 1e-5, f"{what}: {err.max()}"


# (N, H, W, C): channels a multiple of the 16-byte vector and not (the
# element path), one-pixel and one-row images, the U-Net block's width
CASES = [(2, 7, 9, 16), (1, 1, 1, 8), (3, 1, 13, 24), (1, 11, 1, 40), (2, 5, 6, 13),
         (1, 17, 19, 320), (2, 3, 4, 1)]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N,H,W,C", CASES)
def test_dwconv_parity(N, H, W, C, dt):
    x, w, b = inputs(N, H, W, C, dt, seed=N * 1000 + H * 31 + W + C)
    y = d4.dwconv3x3(dev(x, dt), dev(w, dt), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    check(host_raw(y, dt), x, w, b, dt, f"dwconv {dt} {N}x{H}x{W}x{C}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_dwconv_element_path_and_no_bias(dt):
    """Tensors aligned only to their element size take the element path:
    same bits."""
    N, H, W, C = 2, 6, 7, 32
    x, w, _ = inputs(N, H, W, C, dt, seed=5, with_bias=False)
    es_off = 1
    xt = dev(x, dt, offset_elems=es_off)
    assert xt.data_ptr() % 16 != 0
    y = d4.dwconv3x3(xt, dev(w, dt))
    torch.cuda.synchronize()
    check(host_raw(y, dt), x, w, None, dt, f"dwconv element path {dt}")


def test_dwconv_nonfinite_weights_stay_out_of_the_padding():
    """A NaN weight on the top-left tap: the first row and column never use
    that tap, so they stay finite (the oracle skips taps outside the
    image)."""
    N, H, W, C, dt = 1, 5, 6, 16, "bf16"
    x, w, b = inputs(N, H, W, C, dt, seed=9)
    wv = from_raw(w, dt).copy()
    wv[0, 0, 3] = np.nan
    wv[2, 2, 5] = np.inf
    w = to_raw(wv, dt)
    y = d4.dwconv3x3(dev(x, dt), dev(w, dt), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    got = host_raw(y, dt)
    check(got, x, w, b, dt, "dwconv non-finite weights")
    assert np.isfinite(from_raw(got, dt)[0, 0, :, 3]).all()


def test_dwconv_full_size():
    """The U-Net block's features: 8 x 128 x 128 x 320, bf16, every element."""
    N, H, W, C, dt = 8, 128, 128, 320, "bf16"
    x, w, b = inputs(N, H, W, C, dt, seed=21)
    say("dwconv full size")
    y = d4.dwconv3x3(dev(x, dt), dev(w, dt), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    check(host_raw(y, dt), x, w, b, dt, "dwconv full size")


def test_dwconv_empty_batch():
    x = torch.empty((0, 4, 4, 16), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((3, 3, 16), dtype=torch.bfloat16, device="cuda")
    y = d4.dwconv3x3(x, w)
    torch.cuda.synchronize()
    assert y.shape == x.shape
