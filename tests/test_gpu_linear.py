"""Parity of the offset/weight linear layer (dcn4_offset_linear) with the
oracle's fp64 product.

The kernel forms exact products (a bf16 or fp16 product fits fp32), sums the
Cin of them plus the bias in fp32 in the matrix cores' order and rounds once
to the I/O dtype.  With s the exact sum, A the oracle's sum of absolute terms
and e = (Cin + 8) * 2^-24 * A the fp32 summation bound, the stored value v
obeys |v - s| <= u * (|s| + e) + e + t, with u the I/O dtype's unit roundoff
(2^-8 for bf16 with its 8 significant bits, 2^-11 for fp16 with 11) and t its half subnormal step.  The bound is
checked on every element; most outputs also match the correctly rounded
value bit for bit, which is reported."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
from test_gpu_parity import say  # noqa: E402
from workloads import from_raw, make_linear_inputs  # noqa: E402

import dynamic_sparse_vision_dcn4_amd as d4  # noqa: E402

pytestmark = pytest.mark.gpu
U = 2.0 ** -24
HALF_ULP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
HALF_SUB = {"bf16": 2.0 ** -134, "f16": 2.0 ** -25}
TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def dev16(raw, dt):
    return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(TDT[dt]).cuda()


def run_linear(feat, weight, bias, dt, out=None):
    f, w = dev16(feat, dt), dev16(weight, dt)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    y = d4.offset_linear(f, w, b, out=out)
    torch.cuda.synchronize()
    return y.cpu().view(torch.int16).numpy().view(np.uint16)


def check(got_raw, feat, weight, bias, dt, what, rows=None):
    o = oracle.get()
    if rows is not None:
        feat = feat[rows]
        got_raw = got_raw[rows]
    want, absum = o.linear(dt, feat, weight, bias)
    cin = feat.shape[1]
    got = from_raw(got_raw, dt).astype(np.float64)
    e = (cin + 8) * U * absum
    bound = HALF_ULP[dt] * (np.abs(want) + e) + e + HALF_SUB[dt]
    err = np.abs(got - want)
    bad = ~(err <= bound)
    # the correctly rounded value, for the bit-exact share
    exact = np.asarray(got_raw) == np.asarray(
        torch.from_numpy(want).to(TDT[dt]).view(torch.int16).numpy().view(np.uint16))
    say(f"{what}: max err/bound = {float(np.max(err / bound)):.3g}, "
        f"{exact.mean() * 100:.2f}% bit-exact over {err.size}")
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs beyond the bound; "
                           f"first at {np.argwhere(bad)[:3].tolist()}")


# (M, Cin, Nout, bias): one element; a ragged row block and an odd number of
# 16-wide steps; ragged column chunks (Nout > 288); several row blocks with
# the U-Net block's channel and output widths (G = 20 groups of 3 x 9) and
# with the FlowDCN token width (G = 16 of 27 over 1152 channels)
CASES = [(1, 16, 1, True), (200, 48, 54, True), (300, 64, 300, False),
         (129, 320, 540, True), (515, 320, 540, False), (260, 1152, 432, True),
         (77, 1280, 1080, True), (128, 16, 576, True),
         # every Cin that keeps the features in registers (64 .. 384 by 64),
         # with Nout % 4 != 0 (2-byte stores) and == 0 (8-byte stores)
         (300, 64, 54, True), (64, 128, 540, False), (33, 192, 81, True),
         (1000, 256, 216, True), (257, 384, 135, True), (130, 384, 32, False),
         (1, 320, 540, True),
         # the K-streamed GEMM's pipeline: two stages with a partial last
         # one, three stages, seven with a partial last one; ragged row
         # blocks of 256 and column chunks of 128
         (513, 80, 128, False), (600, 144, 100, True), (300, 400, 270, True)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("M,Cin,Nout,with_bias", CASES)
def test_linear_parity(M, Cin, Nout, with_bias, dt):
    say(f"linear {dt} M={M} Cin={Cin} Nout={Nout} bias={with_bias}")
    feat, weight, bias = make_linear_inputs(M, Cin, Nout, dt, seed=M + Cin + Nout,
                                            with_bias=with_bias)
    got = run_linear(feat, weight, bias, dt)
    check(got, feat, weight, bias, dt, f"{dt} {M}x{Cin}x{Nout}")


def test_linear_full_size_sampled():
    """The U-Net block's producer at full size: 8 x 128 x 128 pixels x 320
    channels -> 540 outputs (20 groups x 27), checked on 640 sampled rows
    that include the first and the last row block."""
    M, Cin, Nout, dt = 8 * 128 * 128, 320, 540, "bf16"
    say(f"linear full size {dt} M={M} Cin={Cin} Nout={Nout}")
    feat, weight, bias = make_linear_inputs(M, Cin, Nout, dt, seed=11)
    got = run_linear(feat, weight, bias, dt)
    rng = np.random.Generator(np.random.PCG64(5))
    rows = np.unique(np.concatenate([np.arange(128), np.arange(M - 128, M),
                                     rng.integers(0, M, 384)]))
    check(got, feat, weight, bias, dt, "full size (sampled rows)", rows=rows)


@pytest.mark.parametrize("Cin,Nout", [(32, 30), (64, 30), (320, 36)])
def test_linear_writes_only_its_output(Cin, Nout):
    """Rows past M and columns past Nout are never written: the output sits
    inside a larger buffer whose other bytes keep their sentinel."""
    M, dt = 130, "bf16"
    feat, weight, bias = make_linear_inputs(M, Cin, Nout, dt, seed=3)
    big = torch.full((M * Nout + 4096,), -7, dtype=torch.int16, device="cuda")
    out = big[:M * Nout].view(TDT[dt]).view(M, Nout)
    got = run_linear(feat, weight, bias, dt, out=out)
    check(got, feat, weight, bias, dt, "sentinel case")
    tail = big[M * Nout:].cpu().numpy()
    assert (tail == -7).all()


def test_linear_empty():
    f = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((54, 32), dtype=torch.bfloat16, device="cuda")
    y = d4.offset_linear(f, w)
    torch.cuda.synchronize()
    assert y.shape == (0, 54)
