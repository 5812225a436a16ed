"""C ABI of libdcn4.so on the CPU: exported symbols, planning, and every
error path (validation happens before any HIP call, so none of these touch a
GPU).  Output sizes and ideal bytes are checked against the oracle, which
computes them independently."""
import ctypes

import numpy as np
import os
import re
import subprocess

import pytest

import dynamic_sparse_vision_dcn4_amd as d4
import oracle
from oracle import Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcn4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dcn4_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dcn4_create", "dcn4_forward", "dcn4_destroy", "dcn4_query",
              "dcn4_status_string", "dcn4_probe_geometry", "dcn4_last_error",
              "dcn4_plan_info", "dcn4_plan_set_option", "dcn4_forward_scaled",
              "dcn4_backward", "dcn4_backward_ws", "dcn4_backward_workspace_size",
              "dcn4_offset_linear", "dcn4_dwconv3x3"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(d4.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and they are C symbols (no C++ mangling) in the dynamic symbol table
    out = subprocess.run(["nm", "-D", "--defined-only", d4.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    for n in declared_functions():
        assert re.search(rf"\sT\s{n}$", out, re.M), n


def mk(**kw):
    base = dict(N=2, H=16, W=16, C=64, group=4, dtype="bf16")
    base.update(kw)
    return d4.Desc(**base)


def create(desc):
    st, h = d4.dcn4_create(desc.c_struct())
    return st, h


@pytest.mark.parametrize("kw, want", [
    (dict(C=63), d4.DCN4_ERR_INVALID_ARG),                 # C % group != 0
    (dict(H=0), d4.DCN4_ERR_INVALID_ARG),
    (dict(N=-1), d4.DCN4_ERR_INVALID_ARG),
    (dict(group=0), d4.DCN4_ERR_INVALID_ARG),
    (dict(kernel_h=0), d4.DCN4_ERR_INVALID_ARG),
    (dict(stride_w=0), d4.DCN4_ERR_INVALID_ARG),
    (dict(pad_h=-1), d4.DCN4_ERR_INVALID_ARG),
    (dict(dilation_w=0), d4.DCN4_ERR_INVALID_ARG),
    (dict(H=2, pad_h=0), d4.DCN4_ERR_INVALID_ARG),          # empty output
    (dict(offset_scale=float("nan")), d4.DCN4_ERR_INVALID_ARG),
    (dict(use_group_scales=True, kernel_h=4), d4.DCN4_ERR_INVALID_ARG),
    (dict(use_group_scales=True, dilation_h=2), d4.DCN4_ERR_INVALID_ARG),
    (dict(use_group_scales=True, offset_scale=2.0), d4.DCN4_ERR_INVALID_ARG),
    (dict(H=1 << 21), d4.DCN4_ERR_INVALID_ARG),
    (dict(N=1, H=4096, W=4096, C=16, group=1), d4.DCN4_ERR_UNSUPPORTED),  # H*W >= 2^23
    (dict(N=1, H=1024, W=1024, C=2048, group=16), d4.DCN4_ERR_UNSUPPORTED),
])
def test_create_rejects(kw, want):
    st, h = create(mk(**kw))
    assert st == want, (st, d4.dcn4_last_error())
    assert h is None
    assert d4.dcn4_last_error() != ""


def test_create_null_arguments():
    h = ctypes.c_void_p()
    assert d4._lib.dcn4_create(None, ctypes.byref(h)) == d4.DCN4_ERR_NULL
    desc = mk().c_struct()
    assert d4._lib.dcn4_create(ctypes.byref(desc), None) == d4.DCN4_ERR_NULL
    assert d4.dcn4_query(None)[0] == d4.DCN4_ERR_NULL
    assert d4.dcn4_forward(None, 16, 16, None, 16, None) == d4.DCN4_ERR_NULL
    d4.dcn4_destroy(None)  # NULL-safe


def test_bad_dtype():
    desc = mk().c_struct()
    desc.dtype = 7
    h = ctypes.c_void_p()
    assert d4._lib.dcn4_create(ctypes.byref(desc), ctypes.byref(h)) == d4.DCN4_ERR_INVALID_ARG


WORKLOAD_SHAPES = [
    (Shape(1, 16, 16, 64, 4), "f32"),
    (Shape(64, 56, 56, 64, 4), "bf16"),
    (Shape(8, 128, 128, 320, 20), "bf16"),
    (Shape(16, 32, 32, 1280, 40, dh=2, dw=2), "f16"),
    (Shape(32, 32, 32, 1152, 16, multiscale=True), "bf16"),
    (Shape(32, 32, 32, 1152, 16, multiscale=True, pixel_scales=True, max_scale=4.0), "bf16"),
    (Shape(3, 9, 11, 24, 3, kh=5, kw=3, sh=2, sw=1, ph=2, pw=0, dh=1, dw=2,
           offset_scale=0.5), "f32"),
]


def desc_of(s: Shape, dt: str) -> d4.Desc:
    return d4.Desc(s.N, s.H, s.W, s.C, s.G, s.kh, s.kw, s.sh, s.sw, s.ph, s.pw,
                   s.dh, s.dw, s.offset_scale, s.multiscale, dt, s.pixel_scales,
                   s.max_scale)


@pytest.mark.parametrize("s, dt", WORKLOAD_SHAPES)
def test_query_matches_oracle(s, dt):
    o = oracle.get()
    p = d4.Plan(desc_of(s, dt))
    assert (p.Ho, p.Wo) == o.out_size(s)
    assert p.ideal_bytes == o.ideal_bytes(s, dt)
    info = p.info()
    D = s.C // s.G
    assert D % info["channels_per_lane"] == 0
    assert info["lanes_per_group"] * info["channels_per_lane"] == D
    assert info["launches"] >= 1 and info["blocks"] >= 1


def test_headline_plan_shape():
    p = d4.Plan(desc_of(Shape(8, 128, 128, 320, 20), "bf16"))
    info = p.info()
    # a lane owns a whole 16-channel group, two 128-bit loads per corner; the
    # tiled kernel runs 16x16 output tiles of one group with an LDS window
    # small enough for four workgroups per CU
    assert info["channels_per_lane"] == 16 and info["vector_bytes"] == 16
    assert info["kernel"] == 2
    assert (info["tile_h"], info["tile_w"], info["tile_groups"]) == (16, 16, 1)
    assert info["blocks"] == 8 * (128 // 16) * (128 // 16) * 20
    assert info["lds_bytes"] <= 160 * 1024 // 4
    p.set_option("kernel", 1)
    info = p.info()
    assert info["kernel"] == 1 and info["blocks"] == 8 * 128 * 128 * 20 // 256


def test_plan_options():
    # the margin window throughout (a 20x24 image's whole-image window would
    # otherwise win at the wider margins)
    p = d4.Plan(desc_of(Shape(2, 20, 24, 64, 4), "bf16"), tile_window=1)
    assert p.info()["kernel"] == 2 and p.info()["tile_window"] == 1
    for m in (0, 3, 5):
        p.set_option("tile_margin", m)
        assert p.info()["tile_margin"] == m
    for bad in (("tile_margin", -1), ("tile_margin", 17), ("tile_groups", 3),
                ("kernel", 3), ("tile_pad", 2), ("tile_swizzle", -1), ("tile_swizzle", 7),
                ("tile_window", 3), ("tile_window", -1)):
        with pytest.raises(d4.DCN4Error) as e:
            p.set_option(*bad)
        assert e.value.status == d4.DCN4_ERR_INVALID_ARG
    assert d4.dcn4_plan_set_option(p.handle, 99, 0) == d4.DCN4_ERR_INVALID_ARG
    # a rejected option leaves the plan as it was
    assert p.info()["tile_margin"] == 5
    p.set_option("tile_margin", 3)
    p.set_option("tile_groups", 4)
    assert p.info()["tile_groups"] == 4 and p.info()["tile_h"] * p.info()["tile_w"] == 64
    # a wide margin first halves the channels per lane (a smaller tile of
    # lanes); when no whole-group window fits, one channel slice of a group
    # per workgroup (one lane per pixel)
    p.set_option("tile_groups", 0)
    p.set_option("tile_margin", 12)
    assert p.info()["kernel"] == 2 and p.info()["channels_per_lane"] == 8
    assert p.info()["tile_slices"] == 1
    p.set_option("tile_margin", 16)
    i = p.info()
    assert i["kernel"] == 2 and i["channels_per_lane"] == 8 and i["tile_slices"] == 2
    assert (i["tile_h"], i["tile_w"]) == (16, 16)
    assert i["blocks"] == 2 * 2 * 2 * 4 * 2   # images x tiles (2 x 2) x groups x slices
    # group-scale plans tile too, with one pixel more of margin by default
    # (their points reach s_g times the grid)
    ms = d4.Plan(desc_of(Shape(2, 10, 10, 64, 4, multiscale=True), "bf16"))
    assert ms.info()["kernel"] == 2 and ms.info()["tile_margin"] == 5
    # FlowDCN's 72-channel groups: 24-channel slices
    fl = d4.Plan(desc_of(Shape(2, 32, 32, 1152, 16, multiscale=True), "bf16"))
    assert fl.info()["kernel"] == 2 and fl.info()["tile_slices"] == 3
    assert fl.info()["channels_per_lane"] == 24 and fl.info()["backward_kernel"] == 2
    # a window too large for LDS at every tile shape falls back to the direct
    # kernel, and a forced tiled kernel refuses it
    big = d4.Plan(desc_of(Shape(1, 64, 64, 64, 1), "f32"))
    big.set_option("tile_margin", 16)
    assert big.info()["kernel"] == 1
    big.set_option("tile_margin", 4)
    big.set_option("kernel", 2)
    with pytest.raises(d4.DCN4Error) as e:
        big.set_option("tile_margin", 16)
    assert e.value.status == d4.DCN4_ERR_UNSUPPORTED
    assert big.info()["tile_margin"] == 4


def test_tile_window_choice():
    """The whole-image window where it fits and stages at most 1.25x the
    margin window's bytes: the 32x32 wide block (two 16-channel slices of its
    32-channel groups, 16x16 tiles); the 128x128 U-Net block keeps the margin
    window, and forcing the whole image there leaves no tile."""
    wide = d4.Plan(desc_of(Shape(16, 32, 32, 1280, 40, dh=2, dw=2), "f16"))  # 30x30 output
    i = wide.info()
    assert i["kernel"] == 2 and i["tile_window"] == 2
    assert i["tile_slices"] == 2 and (i["tile_h"], i["tile_w"]) == (16, 16)
    # images x tile columns x groups x slices: a workgroup walks both tile
    # rows of its column under one staging (four workgroups per CU remain)
    assert i["tile_passes"] == 2 and i["tile_passes_x"] == 1
    assert i["blocks"] == 16 * 2 * 40 * 2
    wide.set_option("tile_passes", 1)
    assert wide.info()["tile_passes"] == 1 and wide.info()["blocks"] == 16 * 4 * 40 * 2
    wide.set_option("tile_passes", 9)   # at most the image's tile rows
    assert wide.info()["tile_passes"] == 2
    # both tile columns too: one workgroup per (image, group, slice)
    wide.set_option("tile_passes_x", 2)
    assert wide.info()["tile_passes_x"] == 2 and wide.info()["blocks"] == 16 * 40 * 2
    wide.set_option("tile_passes_x", 5)  # at most the image's tile columns
    assert wide.info()["tile_passes_x"] == 2
    with pytest.raises(d4.DCN4Error):
        wide.set_option("tile_passes_x", 65)
    wide.set_option("tile_passes_x", 0)
    assert wide.info()["tile_passes_x"] == 1
    with pytest.raises(d4.DCN4Error):
        wide.set_option("tile_passes", 65)
    wide.set_option("tile_window", 1)
    assert wide.info()["tile_window"] == 1 and wide.info()["tile_slices"] == 1
    unet = d4.Plan(desc_of(Shape(8, 128, 128, 320, 20), "bf16"))
    assert unet.info()["tile_window"] == 1
    unet.set_option("tile_window", 2)
    assert unet.info()["kernel"] == 1 and unet.info()["tile_window"] == 0
    with pytest.raises(d4.DCN4Error) as e:
        unet.set_option("kernel", 2)
    assert e.value.status == d4.DCN4_ERR_UNSUPPORTED


def test_f16_window_option():
    """bf16 tiled plans re-encode their windows as fp16 by default when the
    staging fits the kernel's register passes; other dtypes and the direct
    kernel never do; the option switches it off and back."""
    unet = d4.Plan(desc_of(Shape(8, 128, 128, 320, 20), "bf16"))
    assert unet.info()["tile_f16_window"] == 1
    unet.set_option("tile_f16_window", 0)
    assert unet.info()["tile_f16_window"] == 0
    unet.set_option("tile_f16_window", 1)
    assert unet.info()["tile_f16_window"] == 1
    unet.set_option("tile_f16_window", 2)   # re-encoded in LDS
    assert unet.info()["tile_f16_window"] == 2
    unet.set_option("tile_f16_window", 1)
    for bad in (-1, 3):
        with pytest.raises(d4.DCN4Error) as e:
            unet.set_option("tile_f16_window", bad)
        assert e.value.status == d4.DCN4_ERR_INVALID_ARG
    # FlowDCN's 24-channel slices: 48-byte window pixels; at margin 4 nine
    # staging passes (through registers), at the group-scale default margin
    # of 5 fifteen, more than the registers hold (bf16, or in LDS on request)
    fl = d4.Plan(desc_of(Shape(2, 32, 32, 1152, 16, multiscale=True), "bf16"), tile_margin=4)
    assert fl.info()["tile_f16_window"] == 1
    fl.set_option("tile_margin", 5)
    assert fl.info()["tile_f16_window"] == 0
    fl.set_option("tile_f16_window", 2)
    assert fl.info()["tile_f16_window"] == 2
    for dt in ("f16", "f32"):
        p = d4.Plan(desc_of(Shape(2, 40, 40, 64, 4), dt), channels_per_lane=8 if dt == "f32" else 0)
        assert p.info()["kernel"] == 2 and p.info()["tile_f16_window"] == 0
    direct = d4.Plan(desc_of(Shape(2, 40, 40, 64, 4), "bf16"), kernel=1)
    assert direct.info()["tile_f16_window"] == 0
    # a window of more staging passes than the registers hold stays bf16
    # (margin 14 and two tile rows per workgroup: 63 x 47 window pixels of 16
    # bytes, five rows per pass: 13 passes; one tile row: 47 rows, 10
    # passes, through registers)
    wide = d4.Plan(desc_of(Shape(1, 96, 96, 64, 4), "bf16"), tile_window=1, tile_margin=14,
                   tile_passes=2)
    i = wide.info()
    assert i["kernel"] == 2 and i["tile_passes"] == 2 and i["tile_f16_window"] == 0
    wide.set_option("tile_passes", 1)
    assert wide.info()["tile_f16_window"] == 1


def test_om_unit_option():
    """Offset/weight rows: read by the forward's lanes into registers (1)
    automatically for 3x3 kernels with one group per workgroup (the U-Net
    block, the InternImage stages); otherwise staged in 16-byte units when the
    per-pixel stride keeps the lanes' reads at most 4-way bank conflicted and
    the occupancy holds (fp32 InternImage stage), else 4-byte units; each can
    be forced (1 falls back to 4-byte units where rows cannot be read
    directly); other values are rejected.  Reading the rows directly leaves
    the window alone in the forward's LDS."""
    f32 = d4.Plan(d4.Desc(64, 56, 56, 64, 4, dtype="f32"))
    assert f32.info()["tile_om_unit"] == 1
    f32.set_option("tile_om_unit", 4)
    assert f32.info()["tile_om_unit"] == 4
    f32.set_option("tile_om_unit", 16)
    assert f32.info()["tile_om_unit"] == 16
    five = d4.Plan(d4.Desc(4, 20, 20, 64, 4, kernel_h=5, kernel_w=5, pad_h=2, pad_w=2,
                           dtype="bf16"), tile_om_unit=1)
    assert five.info()["tile_om_unit"] in (4, 16)   # 5x5: staged
    unet = d4.Plan(d4.Desc(8, 128, 128, 320, 20, dtype="bf16"))
    info = unet.info()
    assert info["tile_om_unit"] == 1
    window = info["tile_h"] + 2 + 2 * info["tile_margin"] + 1
    assert info["lds_bytes"] == window * window * 32 + 16   # window + encoding flags
    for unit in (4, 16):
        unet.set_option("tile_om_unit", unit)
        assert unet.info()["tile_om_unit"] == unit
        assert unet.info()["lds_bytes"] > info["lds_bytes"]
    assert d4.dcn4_plan_set_option(unet.handle, d4.DCN4_OPT_TILE_OM_UNIT, 12) == d4.DCN4_ERR_INVALID_ARG
    assert d4.dcn4_plan_set_option(unet.handle, d4.DCN4_OPT_TILE_OM_UNIT, 8) == d4.DCN4_ERR_INVALID_ARG
    assert d4.dcn4_plan_set_option(unet.handle, d4.DCN4_OPT_TILE_OM_UNIT, 2) == d4.DCN4_ERR_INVALID_ARG
    unet.set_option("tile_om_unit", 0)
    assert unet.info()["tile_om_unit"] == 1
    grouped = d4.Plan(d4.Desc(8, 128, 128, 320, 20, dtype="bf16"), tile_groups=2)
    assert grouped.info()["tile_om_unit"] in (4, 16)   # two groups per workgroup: staged


def test_channels_per_lane_override():
    p = d4.Plan(desc_of(Shape(2, 8, 8, 64, 2), "bf16"))   # D = 32
    for dp in (8, 16, 32):
        p.set_channels_per_lane(dp)
        assert p.info()["channels_per_lane"] == dp
    for bad in (4, 12, 24, 64):
        with pytest.raises(d4.DCN4Error):
            p.set_channels_per_lane(bad)
    p.set_channels_per_lane(0)
    assert p.info()["channels_per_lane"] == 16


def test_element_path_plan_when_group_is_not_vector_wide():
    p = d4.Plan(desc_of(Shape(1, 8, 8, 30, 3), "bf16"))   # D = 10: 20 bytes
    info = p.info()
    assert info["channels_per_lane"] == 1 and info["vector_bytes"] == 2


def test_many_images_split_into_launches():
    # direct kernel: lanes per launch stay below 2^31, 2^31 / (64*64*1024) =
    # 512 images per launch
    p = d4.Plan(d4.Desc(N=2000, H=64, W=64, C=1024, group=64, dtype="bf16"), kernel=1)
    assert p.info()["launches"] == 4
    # tiled kernel: workgroups per launch stay below 2^30
    p.set_option("kernel", 0)
    info = p.info()
    assert info["kernel"] == 2 and info["launches"] == 1


class TestForwardValidation:
    """dcn4_forward / dcn4_probe_geometry reject bad pointers before launching."""

    def setup_method(self):
        self.p = d4.Plan(mk())
        self.ms = d4.Plan(mk(use_group_scales=True))

    def fwd(self, p, x, om, sc, y):
        return d4.dcn4_forward(p.handle, x, om, sc, y, None)

    def test_null(self):
        assert self.fwd(self.p, None, 256, None, 512) == d4.DCN4_ERR_NULL
        assert self.fwd(self.p, 256, None, None, 512) == d4.DCN4_ERR_NULL
        assert self.fwd(self.p, 256, 256, None, None) == d4.DCN4_ERR_NULL

    def test_scales_against_mode(self):
        assert self.fwd(self.p, 256, 256, 1024, 512) == d4.DCN4_ERR_INVALID_ARG
        assert self.fwd(self.ms, 256, 256, None, 512) == d4.DCN4_ERR_NULL

    def test_misaligned(self):
        assert self.fwd(self.p, 257, 256, None, 512) == d4.DCN4_ERR_MISALIGNED
        assert self.fwd(self.p, 256, 255, None, 512) == d4.DCN4_ERR_MISALIGNED
        assert self.fwd(self.p, 256, 256, None, 513) == d4.DCN4_ERR_MISALIGNED
        assert self.fwd(self.ms, 256, 256, 1026, 512) == d4.DCN4_ERR_MISALIGNED
        f32 = d4.Plan(mk(dtype="f32"))
        assert self.fwd(f32, 258, 256, None, 512) == d4.DCN4_ERR_MISALIGNED

    def test_probe(self):
        h = self.p.handle
        assert d4.dcn4_probe_geometry(h, 256, None, None, None, 256, 256, 256, 256, None) == d4.DCN4_ERR_NULL
        assert d4.dcn4_probe_geometry(h, 256, None, None, 258, 256, 256, 256, 256, None) == d4.DCN4_ERR_MISALIGNED
        assert d4.dcn4_probe_geometry(h, None, None, None, 256, 256, 256, 256, 256, None) == d4.DCN4_ERR_NULL
        assert d4.dcn4_probe_geometry(h, 256, None, 1024, 256, 256, 256, 256, 256, None) == d4.DCN4_ERR_INVALID_ARG

    def test_pixel_scales(self):
        ps = d4.Plan(mk(use_group_scales=True, use_pixel_scales=True, max_scale=4.0))
        # the plain entry point refuses a plan that takes pixel scales
        assert d4.dcn4_forward(ps.handle, 256, 256, 1024, 512, None) == d4.DCN4_ERR_INVALID_ARG
        fs = lambda p, sc, pp: d4.dcn4_forward_scaled(p.handle, 256, 256, sc, pp, 512, None)
        assert fs(ps, 1024, None) == d4.DCN4_ERR_NULL
        assert fs(ps, 1024, 2050) == d4.DCN4_ERR_MISALIGNED
        assert fs(self.ms, 1024, 2048) == d4.DCN4_ERR_INVALID_ARG
        assert fs(self.p, None, 2048) == d4.DCN4_ERR_INVALID_ARG

    def test_backward(self):
        bw = lambda p, x, om, sc, gy, gx, gom: d4.dcn4_backward(p.handle, x, om, sc, None, gy,
                                                               gx, gom, None)
        assert bw(self.p, 256, 256, None, None, 512, 1024) == d4.DCN4_ERR_NULL
        assert bw(self.p, 256, 256, None, 257, 512, 1024) == d4.DCN4_ERR_MISALIGNED
        assert bw(self.p, 256, 256, None, 256, 514, 1024) == d4.DCN4_ERR_MISALIGNED
        assert bw(self.p, 256, 256, None, 256, 512, 1026) == d4.DCN4_ERR_MISALIGNED
        assert bw(self.p, 256, 256, 1024, 256, 512, 1024) == d4.DCN4_ERR_INVALID_ARG
        assert bw(self.ms, 256, 256, None, 256, 512, 1024) == d4.DCN4_ERR_NULL
        assert d4.dcn4_backward(None, 256, 256, None, None, 256, 512, 1024, None) == d4.DCN4_ERR_NULL

    def test_backward_workspace_checks(self):
        st, need = d4.dcn4_backward_workspace_size(self.p.handle)
        assert st == d4.DCN4_OK and need > 0
        assert d4.dcn4_backward_workspace_size(None)[0] == d4.DCN4_ERR_NULL
        # fake device addresses 16 MiB apart: no two ranges overlap
        M = 1 << 24
        bws = lambda ws, nb, gx=4 * M, x=M: d4.dcn4_backward_ws(
            self.p.handle, x, 2 * M, None, None, 3 * M, gx, 5 * M, ws, nb, None)
        assert bws(8 * M, need - 1) == d4.DCN4_ERR_INVALID_ARG
        assert bws(8 * M + 16, need) == d4.DCN4_ERR_MISALIGNED
        # the other arguments are checked first
        assert bws(8 * M, need - 1, gx=4 * M + 2) == d4.DCN4_ERR_MISALIGNED
        assert bws(8 * M, need - 1, x=None) == d4.DCN4_ERR_NULL
        assert d4.dcn4_backward_ws(None, M, 2 * M, None, None, 3 * M, 4 * M, 5 * M, 8 * M, need,
                                   None) == d4.DCN4_ERR_NULL
        # a workspace overlapping an input or an output
        assert bws(2 * M, need) == d4.DCN4_ERR_INVALID_ARG
        assert bws(4 * M + 256, need) == d4.DCN4_ERR_INVALID_ARG
        assert bws(5 * M - 256, need) == d4.DCN4_ERR_INVALID_ARG

    def test_noalloc_refuses_beyond_its_scratch(self):
        """dcn4_backward_noalloc gathers grad_x in the library's static 64 MiB
        workspace, in chunks of (image, group) pairs that fit it: a problem
        whose single pair needs more is refused before anything is enqueued,
        with a message naming the entry point to use instead."""
        G1 = 1 << 30   # fake device addresses 1 GiB apart: no overlap
        big = d4.Plan(desc_of(Shape(1, 1024, 1024, 16, 1), "bf16"))
        assert big.backward_workspace_bytes() > (64 << 20)
        st = d4.dcn4_backward_noalloc(big.handle, G1, 2 * G1, None, None, 3 * G1, 4 * G1,
                                      5 * G1, None)
        assert st == d4.DCN4_ERR_UNSUPPORTED
        assert "dcn4_backward_ws" in d4.dcn4_last_error()
        # argument errors come first, as in dcn4_backward
        assert d4.dcn4_backward_noalloc(big.handle, G1 + 1, 2 * G1, None, None, 3 * G1, 4 * G1,
                                        5 * G1, None) == d4.DCN4_ERR_MISALIGNED
        assert d4.dcn4_backward_noalloc(None, G1, 2 * G1, None, None, 3 * G1, 4 * G1, 5 * G1,
                                        None) == d4.DCN4_ERR_NULL
        assert d4.dcn4_backward_noalloc(big.handle, G1, 2 * G1, None, None, 3 * G1, G1 + 64,
                                        5 * G1, None) == d4.DCN4_ERR_INVALID_ARG

    def test_backward_scales_checks(self):
        """dcn4_backward_scales validates before launching: group-scale plans
        only, pixel-scale gradients only with pixel scales, aligned and
        non-overlapping outputs."""
        M = 1 << 24
        ms = d4.Plan(mk(use_group_scales=True))
        ps = d4.Plan(mk(use_group_scales=True, use_pixel_scales=True, max_scale=2.0))
        bs = lambda p, sc, pp, gs, gp: d4.dcn4_backward_scales(p.handle, M, 2 * M, sc, pp, 3 * M,
                                                               gs, gp, None)
        assert d4.dcn4_backward_scales(None, M, 2 * M, 4 * M, None, 3 * M, 5 * M, None,
                                       None) == d4.DCN4_ERR_NULL
        assert bs(self.p, None, None, 5 * M, None) == d4.DCN4_ERR_INVALID_ARG   # no group scales
        assert bs(ms, 4 * M, None, 5 * M, 6 * M) == d4.DCN4_ERR_INVALID_ARG     # no pixel scales
        assert bs(ms, None, None, 5 * M, None) == d4.DCN4_ERR_NULL              # scales missing
        assert bs(ms, 4 * M, None, 5 * M + 2, None) == d4.DCN4_ERR_MISALIGNED
        assert bs(ps, 4 * M, 7 * M, 5 * M, 6 * M + 2) == d4.DCN4_ERR_MISALIGNED
        assert bs(ms, 4 * M, None, M + 64, None) == d4.DCN4_ERR_INVALID_ARG     # over x
        assert bs(ps, 4 * M, 7 * M, 5 * M, 7 * M) == d4.DCN4_ERR_INVALID_ARG    # over sigma
        assert bs(ps, 4 * M, 7 * M, 6 * M + 8, 6 * M) == d4.DCN4_ERR_INVALID_ARG  # each other

    def test_overlapping_outputs_rejected(self):
        """No output may overlap an input or another output of the call (the
        byte ranges the plan implies); adjacent ranges are fine, so the
        rejection is the overlap itself."""
        M = 1 << 24
        p = self.p                                    # 2x16x16x64 bf16: 64 KiB tensors
        nx = 2 * 16 * 16 * 64 * 2
        fwd = lambda x, om, y: d4.dcn4_forward(p.handle, x, om, None, y, None)
        assert fwd(M, 2 * M, M + nx - 16) == d4.DCN4_ERR_INVALID_ARG      # y inside x
        assert fwd(M, 2 * M, M - nx + 16) == d4.DCN4_ERR_INVALID_ARG      # y's end inside x
        assert fwd(M, 2 * M, 2 * M + 4096) == d4.DCN4_ERR_INVALID_ARG     # y inside offset_mask
        ms = self.ms
        assert d4.dcn4_forward(ms.handle, M, 2 * M, 3 * M, 3 * M - 16, None) == \
            d4.DCN4_ERR_INVALID_ARG                                       # y over the scales
        bw = lambda x, om, gy, gx, gom: d4.dcn4_backward_ws(p.handle, x, om, None, None, gy,
                                                            gx, gom, None, 0, None)
        assert bw(M, 2 * M, 3 * M, M + 64, None) == d4.DCN4_ERR_INVALID_ARG   # grad_x over x
        assert bw(M, 2 * M, 3 * M, None, 3 * M) == d4.DCN4_ERR_INVALID_ARG    # grad_om over grad_y
        assert bw(M, 2 * M, 3 * M, 4 * M, 4 * M + 1024) == d4.DCN4_ERR_INVALID_ARG  # each other
        lin = lambda f, w, b, o: d4.dcn4_offset_linear(f, w, b, o, 1000, 64, 108,
                                                       d4.DCN4_BF16, None)
        assert lin(M, 2 * M, None, M + 1024) == d4.DCN4_ERR_INVALID_ARG      # over feat
        assert lin(M, 2 * M, None, 2 * M - 1000) == d4.DCN4_ERR_INVALID_ARG  # over weight
        assert lin(M, 2 * M, 3 * M, 3 * M - 64) == d4.DCN4_ERR_INVALID_ARG   # over bias
        dw = lambda x, w, b, o: d4.dcn4_dwconv3x3(x, w, b, o, 2, 16, 16, 64, d4.DCN4_BF16, None)
        assert dw(M, 2 * M, None, M + nx // 2) == d4.DCN4_ERR_INVALID_ARG    # over x
        assert dw(M, 2 * M, None, 2 * M - 64) == d4.DCN4_ERR_INVALID_ARG     # over the weight
        assert dw(M, 2 * M, 3 * M, 3 * M) == d4.DCN4_ERR_INVALID_ARG         # over the bias

    def test_dcnv3_checks(self):
        """dcn4_dcnv3_softmax and dcn4_dcnv3_forward validate before
        launching: standard-geometry plans only, non-NULL and aligned
        tensors, no overlap of an output with an input."""
        M = 1 << 24
        p, ms = self.p, self.ms
        sm = lambda pl, om, out: d4.dcn4_dcnv3_softmax(pl.handle if pl else None, om, out, None)
        fw = lambda pl, x, om, y: d4.dcn4_dcnv3_forward(pl.handle if pl else None, x, om, y, None)
        assert sm(None, M, 2 * M) == d4.DCN4_ERR_NULL
        assert sm(p, None, 2 * M) == d4.DCN4_ERR_NULL
        assert sm(p, M, None) == d4.DCN4_ERR_NULL
        assert sm(p, M + 1, 2 * M) == d4.DCN4_ERR_MISALIGNED
        assert sm(p, M, 2 * M + 1) == d4.DCN4_ERR_MISALIGNED
        assert sm(p, M, M + 4096) == d4.DCN4_ERR_INVALID_ARG            # out over offset_mask
        assert sm(ms, M, 2 * M) == d4.DCN4_ERR_UNSUPPORTED              # group scales
        assert fw(None, M, 2 * M, 3 * M) == d4.DCN4_ERR_NULL
        assert fw(p, None, 2 * M, 3 * M) == d4.DCN4_ERR_NULL
        assert fw(p, M, 2 * M, None) == d4.DCN4_ERR_NULL
        assert fw(p, M + 1, 2 * M, 3 * M) == d4.DCN4_ERR_MISALIGNED
        assert fw(p, M, 2 * M, M + 64) == d4.DCN4_ERR_INVALID_ARG       # y over x
        assert fw(p, M, 2 * M, 2 * M - 64) == d4.DCN4_ERR_INVALID_ARG   # y's end over offset_mask
        assert fw(ms, M, 2 * M, 3 * M) == d4.DCN4_ERR_UNSUPPORTED
        p0 = d4.Plan(mk(N=0))
        assert d4.dcn4_dcnv3_softmax(p0.handle, None, None, None) == d4.DCN4_OK
        assert d4.dcn4_dcnv3_forward(p0.handle, None, None, None, None) == d4.DCN4_OK

    def test_backward_workspace_size(self):
        """The documented layout: chunks of images x groups of at most as many
        (image, group) pairs as fit the operator's ideal traffic bytes (at
        least one pair, at most 2 GiB), as few chunks as possible and those
        evened out; a chunk's
        workspace is a 256-byte counter, 4 bytes per bucket, 4 bytes per
        sample (the first three regions rounded up to 256 bytes) and
        16 * capacity bytes per bucket."""
        r256 = lambda b: (b + 255) // 256 * 256

        def expected(plan, desc, cap):
            keys = (desc.H + 1) * (desc.W + 1)
            samples = plan.Ho * plan.Wo * desc.kernel_h * desc.kernel_w
            f = lambda n: 256 + r256(4 * n * keys) + r256(4 * n * samples) + 16 * n * keys * cap
            budget = max(min(plan.ideal_bytes, 2 << 30), f(1))
            pairs = max(n for n in range(1, desc.N * desc.group + 1) if f(n) <= budget) \
                if f(1) <= budget else 1
            # fewest chunks, then evened out: the smallest chunk for that count
            opts = []
            for gc in range(1, desc.group + 1):
                imgs = min(desc.N, pairs // gc)
                if imgs:
                    ci, cg = -(-desc.N // imgs), -(-desc.group // gc)
                    opts.append((ci * cg, -(-desc.N // ci) * -(-desc.group // cg)))
            return f(min(opts)[1])

        for desc, cap in ((mk(), 0), (mk(N=3, H=21, W=13, kernel_h=5, kernel_w=5, pad_h=2,
                                         pad_w=2), 7),
                          (mk(N=2, H=30, W=30, stride_h=2, stride_w=2), 0),
                          (mk(N=5, H=40, W=36, C=96, group=6), 4),
                          (mk(N=64, H=64, W=64, C=64, group=4), 1024)):
            plan = d4.Plan(desc, bucket_capacity=cap)
            c = plan.info()["bucket_capacity"]
            if cap:
                assert c == cap
            want = expected(plan, desc, c)
            assert plan.backward_workspace_bytes() == want, (desc, want)
            one = expected(plan, desc.__class__(**{**desc.__dict__, "N": 1, "group": 1,
                                                   "C": desc.C // desc.group}), c)
            assert want <= max(plan.ideal_bytes, one)
        # the latent-diffusion block's workspace stays within its ideal bytes
        unet = d4.Plan(desc_of(Shape(8, 128, 128, 320, 20), "bf16"))
        assert 0 < unet.backward_workspace_bytes() <= unet.ideal_bytes

    def test_bucket_capacity_option(self):
        p = d4.Plan(mk())
        # the automatic capacity: mean load + 3 Poisson deviations + 4, to a multiple of 4
        mu = 9 * 16 * 16 / (17 * 17)
        auto = int(np.ceil(mu + 3 * np.sqrt(mu) + 4))
        assert p.info()["bucket_capacity"] == (auto + 3) // 4 * 4
        for bad in (-1, 1025):
            assert d4.dcn4_plan_set_option(p.handle, d4.DCN4_OPT_BUCKET_CAPACITY, bad) == \
                d4.DCN4_ERR_INVALID_ARG
        assert d4.dcn4_plan_set_option(p.handle, d4.DCN4_OPT_BUCKET_CAPACITY, 3) == d4.DCN4_OK
        assert p.info()["bucket_capacity"] == 3

    def test_empty_batch_is_a_no_op(self):
        p0 = d4.Plan(mk(N=0))
        # nothing is enqueued, so no pointer is touched and no GPU is needed
        assert d4.dcn4_forward(p0.handle, None, None, None, None, None) == d4.DCN4_OK
        assert p0.ideal_bytes == 0


class TestOffsetLinearValidation:
    """dcn4_offset_linear rejects bad arguments before launching (fake device
    addresses: none of these calls reaches a launch)."""

    def lin(self, feat=256, weight=512, bias=None, om=1024, M=8, Cin=32, Nout=54,
            dtype=d4.DCN4_BF16):
        return d4.dcn4_offset_linear(feat, weight, bias, om, M, Cin, Nout, dtype, None)

    def test_dtype(self):
        assert self.lin(dtype=d4.DCN4_F32) == d4.DCN4_ERR_UNSUPPORTED
        assert self.lin(dtype=7) == d4.DCN4_ERR_INVALID_ARG

    def test_sizes(self):
        assert self.lin(M=-1) == d4.DCN4_ERR_INVALID_ARG
        assert self.lin(Cin=0) == d4.DCN4_ERR_INVALID_ARG
        assert self.lin(Nout=0) == d4.DCN4_ERR_INVALID_ARG
        assert self.lin(Cin=24) == d4.DCN4_ERR_UNSUPPORTED
        assert self.lin(Cin=1 << 22, Nout=300) == d4.DCN4_ERR_UNSUPPORTED

    def test_null_and_alignment(self):
        assert self.lin(feat=None) == d4.DCN4_ERR_NULL
        assert self.lin(weight=None) == d4.DCN4_ERR_NULL
        assert self.lin(om=None) == d4.DCN4_ERR_NULL
        assert self.lin(feat=264) == d4.DCN4_ERR_MISALIGNED
        assert self.lin(weight=520) == d4.DCN4_ERR_MISALIGNED
        assert self.lin(om=1025) == d4.DCN4_ERR_MISALIGNED
        assert self.lin(bias=2050) == d4.DCN4_ERR_MISALIGNED
        assert d4.DCN4Error  # the binding's exception type exists

    def test_empty_is_a_no_op(self):
        # nothing is enqueued, so no pointer is touched and no GPU is needed
        assert self.lin(feat=None, weight=None, om=None, M=0) == d4.DCN4_OK


class TestDwconvValidation:
    """dcn4_dwconv3x3 rejects bad arguments before launching (fake device
    addresses: none of these calls reaches a launch)."""

    def dw(self, x=256, w=512, bias=None, out=1024, N=1, H=4, W=5, C=16,
           dtype=d4.DCN4_BF16):
        return d4.dcn4_dwconv3x3(x, w, bias, out, N, H, W, C, dtype, None)

    def test_arguments(self):
        assert self.dw(dtype=5) == d4.DCN4_ERR_INVALID_ARG
        assert self.dw(N=-1) == d4.DCN4_ERR_INVALID_ARG
        assert self.dw(H=0) == d4.DCN4_ERR_INVALID_ARG
        assert self.dw(C=0) == d4.DCN4_ERR_INVALID_ARG
        assert self.dw(out=256) == d4.DCN4_ERR_INVALID_ARG   # out aliases x

    def test_null_and_alignment(self):
        assert self.dw(x=None) == d4.DCN4_ERR_NULL
        assert self.dw(w=None) == d4.DCN4_ERR_NULL
        assert self.dw(out=None) == d4.DCN4_ERR_NULL
        assert self.dw(x=257) == d4.DCN4_ERR_MISALIGNED
        assert self.dw(out=1025) == d4.DCN4_ERR_MISALIGNED
        assert self.dw(x=258, dtype=d4.DCN4_F32) == d4.DCN4_ERR_MISALIGNED
        assert self.dw(bias=2050) == d4.DCN4_ERR_MISALIGNED

    def test_empty_is_a_no_op(self):
        assert self.dw(x=None, w=None, out=None, N=0) == d4.DCN4_OK


@pytest.mark.parametrize("kw", [dict(use_pixel_scales=True),
                                dict(max_scale=2.0),
                                dict(use_group_scales=True, max_scale=-1.0),
                                dict(use_group_scales=True, max_scale=float("nan"))])
def test_create_rejects_bad_scale_settings(kw):
    st, h = d4.dcn4_create(mk(**kw).c_struct())
    assert st == d4.DCN4_ERR_INVALID_ARG and not h


def test_pixel_scale_plan_sizes_match_oracle():
    s = Shape(3, 11, 13, 64, 4, multiscale=True, pixel_scales=True, max_scale=3.0)
    p = d4.Plan(d4.Desc(s.N, s.H, s.W, s.C, s.G, use_group_scales=True, dtype="bf16",
                        use_pixel_scales=True, max_scale=3.0))
    o = oracle.get()
    assert (p.Ho, p.Wo) == o.out_size(s)
    assert p.ideal_bytes == o.ideal_bytes(s, "bf16")
    ho, wo = o.out_size(s)
    plain = d4.Plan(d4.Desc(s.N, s.H, s.W, s.C, s.G, use_group_scales=True, dtype="bf16"))
    assert p.ideal_bytes - plain.ideal_bytes == 4 * s.N * ho * wo * s.G


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert d4.dcn4_status_string(s).startswith("DCN4_")
    assert "unknown" in d4.dcn4_status_string(42)


def test_fast_division_exhaustive_ranges(tmp_path):
    """The kernels divide by run-time invariants with the multiply-high
    method; the host's constants must give exact quotients for n < 2^31."""
    src = tmp_path / "fd.cpp"
    src.write_text(r'''
#include <cstdio>
#include <cstdint>
#include "dcn4_internal.h"
int main() {
  uint64_t bad = 0, checked = 0;
  uint32_t ds[] = {1,2,3,4,5,7,9,20,27,40,48,64,144,900,1024,1080,3136,16384,
                   65535,65536,1000003,(1u<<30)+7,(1u<<31)-1};
  for (uint32_t d : ds) {
    dcn4::FastDiv f = dcn4::make_fastdiv(d);
    for (uint64_t n = 0; n < (1ull << 31); n += (n < 4000000 ? 1 : 999983)) {
      uint32_t q = (uint32_t)((((uint64_t)n * f.m) >> 32) + n) >> f.s;
      bad += (q != n / d); ++checked;
    }
    for (uint64_t k = 1; k * d < (1ull << 31) && k < 100000; k += 1 + k / 10) {
      for (int64_t r = -1; r <= 1; ++r) {
        uint64_t n = k * d + r;
        if (n >= (1ull << 31)) continue;
        uint32_t q = (uint32_t)((((uint64_t)n * f.m) >> 32) + n) >> f.s;
        bad += (q != n / d); ++checked;
      }
    }
  }
  printf("%llu %llu\n", (unsigned long long)bad, (unsigned long long)checked);
  return bad != 0;
}
''')
    exe = tmp_path / "fd"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "dynamic_sparse_vision_dcn4_amd", "csrc"),
                    str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout


class TestBindingChecks:
    """The Python binding checks every tensor before a pointer reaches the C
    ABI (which sees no sizes): dtype, exact shape, contiguity, then device.
    CPU tensors exercise every check up to the device one."""

    def setup_method(self):
        import torch
        self.torch = torch
        self.plan = d4.Plan(mk(N=2, H=8, W=6, C=32, group=2))   # x [2,8,6,32]

    def test_forward_tensor_checks(self):
        torch = self.torch
        x = torch.zeros((2, 8, 6, 32), dtype=torch.bfloat16)
        om = torch.zeros(self.plan.om_shape(), dtype=torch.bfloat16)
        with pytest.raises(TypeError, match="x must be torch.bfloat16"):
            self.plan.forward(x.float(), om)
        # same element count, transposed [N, W, H, C]: rejected by shape
        with pytest.raises(ValueError, match="x must have shape"):
            self.plan.forward(torch.zeros((2, 6, 8, 32), dtype=torch.bfloat16), om)
        with pytest.raises(ValueError, match="x must be contiguous"):
            self.plan.forward(x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3), om)
        with pytest.raises(ValueError, match="offset_mask must have shape"):
            self.plan._check(om.view(2, 8, 6, -1), self.plan.om_shape(), torch.bfloat16,
                             "offset_mask")
        with pytest.raises(TypeError, match="x must be a CUDA tensor"):
            self.plan.forward(x, om)
        with pytest.raises(TypeError, match="torch tensor"):
            self.plan.forward(x.float().numpy(), om)

    def test_backward_tensor_checks(self):
        torch = self.torch
        x = torch.zeros((2, 8, 6, 32), dtype=torch.bfloat16)
        om = torch.zeros(self.plan.om_shape(), dtype=torch.bfloat16)
        gy = torch.zeros(self.plan.out_shape(), dtype=torch.float16)
        with pytest.raises(TypeError, match="x must be a CUDA tensor"):
            self.plan.backward(x, om, gy.bfloat16())
        p16 = d4.Plan(mk(N=2, H=8, W=6, C=32, group=2, dtype="f16"))
        with pytest.raises(TypeError, match="grad_y must be torch.float16"):
            # reaches grad_y only after x and offset_mask pass their CPU-side checks
            p16._check(gy.bfloat16(), p16.out_shape(), torch.float16, "grad_y")

    def test_producer_tensor_checks(self):
        """offset_linear and dwconv3x3 check feat/x first (shape, dtype,
        device), then weight, bias and out against it with the same helper;
        on the CPU the first tensor stops at the device check, so the helper
        is exercised directly for the others."""
        torch = self.torch
        feat = torch.zeros((100, 64), dtype=torch.bfloat16)
        w = torch.zeros((108, 64), dtype=torch.bfloat16)
        with pytest.raises(TypeError, match="feat must be a CUDA tensor"):
            d4.offset_linear(feat, w)
        with pytest.raises(TypeError, match="feat must be bf16 or fp16"):
            d4.offset_linear(feat.float(), w)
        with pytest.raises(ValueError, match="feat must be a 2-d tensor"):
            d4.offset_linear(feat.view(10, 10, 64), w)
        with pytest.raises(ValueError, match="weight must have shape"):
            d4._require(torch.zeros((108, 32), dtype=torch.bfloat16), (108, 64),
                        torch.bfloat16, "weight")
        with pytest.raises(TypeError, match="bias must be torch.float32"):
            d4._require(torch.zeros(108, dtype=torch.bfloat16), (108,), torch.float32, "bias")
        with pytest.raises(ValueError, match="out must have shape"):
            d4._require(torch.zeros((100, 54), dtype=torch.bfloat16), (100, 108),
                        torch.bfloat16, "out")
        with pytest.raises(TypeError, match="out must be a CUDA tensor"):
            d4._require(torch.zeros((100, 108), dtype=torch.bfloat16), (100, 108),
                        torch.bfloat16, "out")
        x = torch.zeros((2, 8, 6, 32), dtype=torch.float16)
        with pytest.raises(TypeError, match="x must be a CUDA tensor"):
            d4.dwconv3x3(x, torch.zeros((3, 3, 32), dtype=torch.float16))
        with pytest.raises(ValueError, match="x must be a 4-d tensor"):
            d4.dwconv3x3(x[0], torch.zeros((3, 3, 32), dtype=torch.float16))
        with pytest.raises(TypeError, match="x must be fp32, bf16 or fp16"):
            d4.dwconv3x3(x.to(torch.int16), torch.zeros((3, 3, 32), dtype=torch.float16))
