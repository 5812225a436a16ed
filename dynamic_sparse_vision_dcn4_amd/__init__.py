"""Python binding of libdcn4.so, the MI355X (gfx950) DCNv4 forward library.

The functions below carry the C ABI's names (include/dcn4.h) and only
marshal arguments; every step of the operator runs in the HIP kernels of the
library.  PyTorch is used by ``Plan`` for device memory and the current
stream only.  There is no fallback: importing this package raises if the
built library is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdcn4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built: run `python dynamic_sparse_vision_dcn4_amd/build.py` "
        "(or __graft_entry__.build()) first")

# PyTorch ships its own HIP runtime under the same soname (libamdhip64.so.7)
# and loads it by absolute path.  Importing torch first makes libdcn4.so bind
# to that already-loaded runtime, so a process holds one HIP runtime; loading
# the library first would leave two runtimes side by side, and the second
# finds no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# dcn4_dtype
DCN4_F32, DCN4_BF16, DCN4_F16 = 0, 1, 2
DTYPE_CODES = {"f32": DCN4_F32, "bf16": DCN4_BF16, "f16": DCN4_F16}
# dcn4_status
DCN4_OK = 0
DCN4_ERR_INVALID_ARG = -1
DCN4_ERR_UNSUPPORTED = -2
DCN4_ERR_MISALIGNED = -3
DCN4_ERR_NULL = -4
DCN4_ERR_HIP = -5
DCN4_ERR_NOMEM = -6


class dcn4_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("N", "H", "W", "C", "group", "kernel_h", "kernel_w",
                 "stride_h", "stride_w", "pad_h", "pad_w", "dilation_h",
                 "dilation_w")] + [("offset_scale", ctypes.c_float),
                                   ("use_group_scales", ctypes.c_int32),
                                   ("dtype", ctypes.c_int32),
                                   ("use_pixel_scales", ctypes.c_int32),
                                   ("max_scale", ctypes.c_float)]


class dcn4_launch_info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32),
                ("channels_per_lane", ctypes.c_int32),
                ("vector_bytes", ctypes.c_int32),
                ("lanes_per_group", ctypes.c_int32),
                ("block_threads", ctypes.c_int32),
                ("blocks", ctypes.c_int64),
                ("launches", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32),
                ("tile_h", ctypes.c_int32),
                ("tile_w", ctypes.c_int32),
                ("tile_groups", ctypes.c_int32),
                ("tile_margin", ctypes.c_int32),
                ("backward_kernel", ctypes.c_int32),
                ("backward_lds_bytes", ctypes.c_int32),
                ("tile_slices", ctypes.c_int32),
                ("bucket_capacity", ctypes.c_int32),
                ("tile_window", ctypes.c_int32),
                ("tile_passes", ctypes.c_int32),
                ("tile_f16_window", ctypes.c_int32),
                ("tile_om_unit", ctypes.c_int32),
                ("tile_passes_x", ctypes.c_int32)]

# dcn4_option
DCN4_OPT_CHANNELS_PER_LANE = 0
DCN4_OPT_KERNEL = 1
DCN4_OPT_TILE_MARGIN = 2
DCN4_OPT_TILE_GROUPS = 3
DCN4_OPT_TILE_PAD = 4
DCN4_OPT_TILE_SWIZZLE = 5
DCN4_OPT_BUCKET_CAPACITY = 6
DCN4_OPT_TILE_WINDOW = 7
DCN4_OPT_TILE_PASSES = 8
DCN4_OPT_TILE_F16_WINDOW = 9
DCN4_OPT_TILE_OM_UNIT = 10
DCN4_OPT_TILE_PASSES_X = 11
OPTIONS = {"channels_per_lane": DCN4_OPT_CHANNELS_PER_LANE, "kernel": DCN4_OPT_KERNEL,
           "tile_margin": DCN4_OPT_TILE_MARGIN, "tile_groups": DCN4_OPT_TILE_GROUPS,
           "tile_pad": DCN4_OPT_TILE_PAD, "tile_swizzle": DCN4_OPT_TILE_SWIZZLE,
           "bucket_capacity": DCN4_OPT_BUCKET_CAPACITY, "tile_window": DCN4_OPT_TILE_WINDOW,
           "tile_passes": DCN4_OPT_TILE_PASSES, "tile_f16_window": DCN4_OPT_TILE_F16_WINDOW,
           "tile_om_unit": DCN4_OPT_TILE_OM_UNIT, "tile_passes_x": DCN4_OPT_TILE_PASSES_X}


_P = ctypes.c_void_p
_lib.dcn4_create.argtypes = [ctypes.POINTER(dcn4_desc), ctypes.POINTER(_P)]
_lib.dcn4_query.argtypes = [_P, ctypes.POINTER(ctypes.c_int32),
                            ctypes.POINTER(ctypes.c_int32),
                            ctypes.POINTER(ctypes.c_uint64)]
_lib.dcn4_plan_info.argtypes = [_P, ctypes.POINTER(dcn4_launch_info)]
_lib.dcn4_plan_set_option.argtypes = [_P, ctypes.c_int32, ctypes.c_int32]
_lib.dcn4_forward.argtypes = [_P, _P, _P, _P, _P, _P]
_lib.dcn4_forward_scaled.argtypes = [_P, _P, _P, _P, _P, _P, _P]
_lib.dcn4_dcnv3_softmax.argtypes = [_P, _P, _P, _P]
_lib.dcn4_dcnv3_forward.argtypes = [_P, _P, _P, _P, _P]
_lib.dcn4_probe_geometry.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.dcn4_backward.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.dcn4_backward_ws.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint64, _P]
_lib.dcn4_backward_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.dcn4_backward_scales.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.dcn4_backward_workspace_size.argtypes = [_P, ctypes.POINTER(ctypes.c_uint64)]
_lib.dcn4_offset_linear.argtypes = [_P, _P, _P, _P, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, _P]
_lib.dcn4_dwconv3x3.argtypes = [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
_lib.dcn4_destroy.argtypes = [_P]
_lib.dcn4_destroy.restype = None
_lib.dcn4_status_string.argtypes = [ctypes.c_int]
_lib.dcn4_status_string.restype = ctypes.c_char_p
_lib.dcn4_last_error.argtypes = []
_lib.dcn4_last_error.restype = ctypes.c_char_p
for _f in ("dcn4_create", "dcn4_query", "dcn4_plan_info",
           "dcn4_plan_set_option", "dcn4_forward", "dcn4_forward_scaled",
           "dcn4_probe_geometry", "dcn4_backward", "dcn4_backward_ws", "dcn4_backward_noalloc", "dcn4_backward_scales",
           "dcn4_backward_workspace_size", "dcn4_offset_linear",
           "dcn4_dwconv3x3", "dcn4_dcnv3_softmax", "dcn4_dcnv3_forward"):
    getattr(_lib, _f).restype = ctypes.c_int


# ---------------------------------------------------------------- C ABI
def dcn4_create(desc: dcn4_desc) -> Tuple[int, Optional[int]]:
    """-> (status, plan handle or None)"""
    h = _P()
    st = _lib.dcn4_create(ctypes.byref(desc) if desc is not None else None,
                          ctypes.byref(h))
    return st, h.value


def dcn4_query(plan) -> Tuple[int, int, int, int]:
    """-> (status, Ho, Wo, ideal_bytes)"""
    ho, wo, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_uint64()
    st = _lib.dcn4_query(plan, ctypes.byref(ho), ctypes.byref(wo), ctypes.byref(b))
    return st, ho.value, wo.value, b.value


def dcn4_plan_info(plan) -> Tuple[int, dict]:
    info = dcn4_launch_info()
    st = _lib.dcn4_plan_info(plan, ctypes.byref(info))
    return st, {f: getattr(info, f) for f, _ in dcn4_launch_info._fields_}


def dcn4_plan_set_option(plan, option: int, value: int) -> int:
    return _lib.dcn4_plan_set_option(plan, option, value)


def dcn4_forward(plan, x: int, offset_mask: int, group_scales: Optional[int],
                 y: int, stream: Optional[int]) -> int:
    """Raw device pointers (ints) and a hipStream_t handle (int or None)."""
    return _lib.dcn4_forward(plan, x, offset_mask, group_scales, y, stream)


def dcn4_forward_scaled(plan, x: int, offset_mask: int, group_scales: Optional[int],
                        pixel_scales: Optional[int], y: int,
                        stream: Optional[int]) -> int:
    return _lib.dcn4_forward_scaled(plan, x, offset_mask, group_scales,
                                    pixel_scales, y, stream)


def dcn4_dcnv3_softmax(plan, offset_mask: int, out: int, stream: Optional[int]) -> int:
    return _lib.dcn4_dcnv3_softmax(plan, offset_mask, out, stream)


def dcn4_dcnv3_forward(plan, x: int, offset_mask: int, y: int, stream: Optional[int]) -> int:
    return _lib.dcn4_dcnv3_forward(plan, x, offset_mask, y, stream)


def dcn4_backward(plan, x: int, offset_mask: int, group_scales: Optional[int],
                  pixel_scales: Optional[int], grad_y: int, grad_x: Optional[int],
                  grad_offset_mask: Optional[int], stream: Optional[int]) -> int:
    return _lib.dcn4_backward(plan, x, offset_mask, group_scales, pixel_scales, grad_y,
                              grad_x, grad_offset_mask, stream)


def dcn4_backward_ws(plan, x: int, offset_mask: int, group_scales: Optional[int],
                     pixel_scales: Optional[int], grad_y: int, grad_x: Optional[int],
                     grad_offset_mask: Optional[int], workspace: Optional[int],
                     workspace_bytes: int, stream: Optional[int]) -> int:
    return _lib.dcn4_backward_ws(plan, x, offset_mask, group_scales, pixel_scales, grad_y,
                                 grad_x, grad_offset_mask, workspace, workspace_bytes, stream)


def dcn4_backward_noalloc(plan, x: int, offset_mask: int, group_scales: Optional[int],
                          pixel_scales: Optional[int], grad_y: int, grad_x: Optional[int],
                          grad_offset_mask: Optional[int], stream: Optional[int]) -> int:
    return _lib.dcn4_backward_noalloc(plan, x, offset_mask, group_scales, pixel_scales,
                                      grad_y, grad_x, grad_offset_mask, stream)


def dcn4_backward_scales(plan, x: int, offset_mask: int, group_scales: Optional[int],
                         pixel_scales: Optional[int], grad_y: int,
                         grad_group_scales: Optional[int], grad_pixel_scales: Optional[int],
                         stream: Optional[int]) -> int:
    return _lib.dcn4_backward_scales(plan, x, offset_mask, group_scales, pixel_scales, grad_y,
                                     grad_group_scales, grad_pixel_scales, stream)


def dcn4_backward_workspace_size(plan):
    """(status, bytes)."""
    n = ctypes.c_uint64(0)
    st = _lib.dcn4_backward_workspace_size(plan, ctypes.byref(n) if plan is not None else None)
    return st, n.value


def _require(t, shape, dtype, name, device=None):
    """A CUDA tensor of exactly `shape` and `dtype`, contiguous, on `device`
    (when given): the C ABI sees only pointers, so sizes are checked here."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def dcn4_offset_linear(feat: int, weight: int, bias: Optional[int], offset_mask: int,
                       M: int, Cin: int, Nout: int, dtype: int, stream: Optional[int]) -> int:
    return _lib.dcn4_offset_linear(feat, weight, bias, offset_mask, M, Cin, Nout, dtype, stream)


def offset_linear(feat, weight, bias=None, out=None, stream=None):
    """offset_mask [M, Nout] = feat [M, Cin] @ weight[Nout, Cin]^T + bias
    (torch CUDA tensors, bf16 or fp16; bias fp32)."""
    if not isinstance(feat, torch.Tensor) or feat.dim() != 2:
        raise ValueError("feat must be a 2-d tensor [M, Cin]")
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be a 2-d tensor [Nout, Cin]")
    dt = {torch.bfloat16: DCN4_BF16, torch.float16: DCN4_F16}.get(feat.dtype)
    if dt is None:
        raise TypeError("feat must be bf16 or fp16")
    M, Cin = feat.shape
    Nout = weight.shape[0]
    _require(feat, (M, Cin), feat.dtype, "feat")
    dev = feat.device
    _require(weight, (Nout, Cin), feat.dtype, "weight", dev)
    if bias is not None:
        _require(bias, (Nout,), torch.float32, "bias", dev)
    if out is None:
        out = torch.empty((M, Nout), dtype=feat.dtype, device=dev)
    else:
        _require(out, (M, Nout), feat.dtype, "out", dev)
    if stream is None:
        stream = torch.cuda.current_stream(feat.device).cuda_stream
    st = dcn4_offset_linear(feat.data_ptr(), weight.data_ptr(),
                            None if bias is None else bias.data_ptr(), out.data_ptr(),
                            M, Cin, Nout, dt, stream)
    if st != DCN4_OK:
        raise DCN4Error(st, "dcn4_offset_linear")
    return out


def dcn4_dwconv3x3(x: int, weight: int, bias: Optional[int], out: int, N: int, H: int,
                   W: int, C: int, dtype: int, stream: Optional[int]) -> int:
    return _lib.dcn4_dwconv3x3(x, weight, bias, out, N, H, W, C, dtype, stream)


def dwconv3x3(x, weight, bias=None, out=None, stream=None):
    """out [N,H,W,C] = depthwise 3x3 convolution of x [N,H,W,C] with weight
    [3,3,C] (stride 1, zero padding 1) plus bias (fp32 [C] or None); torch
    CUDA tensors of one dtype."""
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("x must be a 4-d tensor [N, H, W, C]")
    dt = {torch.float32: DCN4_F32, torch.bfloat16: DCN4_BF16,
          torch.float16: DCN4_F16}.get(x.dtype)
    if dt is None:
        raise TypeError("x must be fp32, bf16 or fp16")
    N, H, W, C = x.shape
    _require(x, (N, H, W, C), x.dtype, "x")
    dev = x.device
    _require(weight, (3, 3, C), x.dtype, "weight", dev)
    if bias is not None:
        _require(bias, (C,), torch.float32, "bias", dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _require(out, (N, H, W, C), x.dtype, "out", dev)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = dcn4_dwconv3x3(x.data_ptr(), weight.data_ptr(),
                        None if bias is None else bias.data_ptr(), out.data_ptr(),
                        N, H, W, C, dt, stream)
    if st != DCN4_OK:
        raise DCN4Error(st, "dcn4_dwconv3x3")
    return out


def dcn4_probe_geometry(plan, offset_mask: int, group_scales: Optional[int],
                        pixel_scales: Optional[int], y0: int, x0: int, lh: int,
                        lw: int, inside: int, stream: Optional[int]) -> int:
    return _lib.dcn4_probe_geometry(plan, offset_mask, group_scales, pixel_scales,
                                    y0, x0, lh, lw, inside, stream)


def dcn4_destroy(plan) -> None:
    _lib.dcn4_destroy(plan)


def dcn4_status_string(status: int) -> str:
    return _lib.dcn4_status_string(status).decode()


def dcn4_last_error() -> str:
    return _lib.dcn4_last_error().decode()


class DCN4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dcn4_status_string(status)} -- {dcn4_last_error()}")


# ---------------------------------------------------------------- torch glue
@dataclass(frozen=True)
class Desc:
    """Operator descriptor (see dcn4_desc in include/dcn4.h)."""
    N: int
    H: int
    W: int
    C: int
    group: int
    kernel_h: int = 3
    kernel_w: int = 3
    stride_h: int = 1
    stride_w: int = 1
    pad_h: int = 1
    pad_w: int = 1
    dilation_h: int = 1
    dilation_w: int = 1
    offset_scale: float = 1.0
    use_group_scales: bool = False
    dtype: str = "bf16"
    use_pixel_scales: bool = False
    max_scale: float = 0.0

    def c_struct(self) -> dcn4_desc:
        return dcn4_desc(self.N, self.H, self.W, self.C, self.group,
                         self.kernel_h, self.kernel_w, self.stride_h,
                         self.stride_w, self.pad_h, self.pad_w,
                         self.dilation_h, self.dilation_w,
                         float(self.offset_scale), int(bool(self.use_group_scales)),
                         DTYPE_CODES[self.dtype], int(bool(self.use_pixel_scales)),
                         float(self.max_scale))


def _torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


class Plan:
    """Owns a dcn4_plan; forward() takes torch CUDA tensors."""

    def __init__(self, desc: Desc, channels_per_lane: int = 0, **options):
        """options: kernel, tile_margin, tile_groups, tile_pad, tile_swizzle,
        tile_window, tile_passes, tile_passes_x, tile_f16_window, bucket_capacity (dcn4_option).  The
        kernel choice is applied last, so a forced tiled
        kernel is checked against the tile options given with it."""
        self.desc = desc
        st, h = dcn4_create(desc.c_struct())
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_create")
        self._h = h
        if channels_per_lane:
            self.set_option("channels_per_lane", channels_per_lane)
        for k, v in sorted(options.items(), key=lambda kv: kv[0] == "kernel"):
            self.set_option(k, v)
        st, self.Ho, self.Wo, self.ideal_bytes = dcn4_query(h)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_query")

    @property
    def handle(self):
        return self._h

    def info(self) -> dict:
        st, info = dcn4_plan_info(self._h)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_plan_info")
        return info

    def set_option(self, name: str, value: int) -> None:
        st = dcn4_plan_set_option(self._h, OPTIONS[name], int(value))
        if st != DCN4_OK:
            raise DCN4Error(st, f"dcn4_plan_set_option({name})")

    def set_channels_per_lane(self, dp: int) -> None:
        self.set_option("channels_per_lane", dp)

    def out_shape(self):
        d = self.desc
        return (d.N, self.Ho, self.Wo, d.C)

    def om_shape(self):
        d = self.desc
        return (d.N, self.Ho, self.Wo, d.group, 3 * d.kernel_h * d.kernel_w)

    def _check(self, t, shape, dtype, name, device=None):
        _require(t, shape, dtype, name, device)

    def forward(self, x, om, scales=None, out=None, stream=None, pixel_scales=None):
        """y[N,Ho,Wo,C] = DCNv4(x[N,H,W,C], om[N,Ho,Wo,G,3K], scales[G],
        pixel_scales[N,Ho,Wo,G])."""
        import torch
        d = self.desc
        dt = _torch_dtype(d.dtype)
        self._check(x, (d.N, d.H, d.W, d.C), dt, "x")
        dev = x.device
        self._check(om, self.om_shape(), dt, "offset_mask", dev)
        if scales is not None:
            self._check(scales, (d.group,), torch.float32, "group_scales", dev)
        if pixel_scales is not None:
            self._check(pixel_scales, (d.N, self.Ho, self.Wo, d.group), torch.float32,
                        "pixel_scales", dev)
        if out is None:
            out = torch.empty(self.out_shape(), dtype=dt, device=dev)
        else:
            self._check(out, self.out_shape(), dt, "out", dev)
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        if d.use_pixel_scales or pixel_scales is not None:
            st = dcn4_forward_scaled(self._h, x.data_ptr(), om.data_ptr(),
                                     None if scales is None else scales.data_ptr(),
                                     None if pixel_scales is None else pixel_scales.data_ptr(),
                                     out.data_ptr(), stream)
            if st != DCN4_OK:
                raise DCN4Error(st, "dcn4_forward_scaled")
            return out
        st = dcn4_forward(self._h, x.data_ptr(), om.data_ptr(),
                          None if scales is None else scales.data_ptr(),
                          out.data_ptr(), stream)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_forward")
        return out

    def dcnv3_softmax(self, om, out=None, stream=None):
        """DCNv3's softmax over each (pixel, group) row's K weights of
        om[N,Ho,Wo,G,3K], offsets unchanged (dcn4_dcnv3_softmax)."""
        import torch
        dt = _torch_dtype(self.desc.dtype)
        self._check(om, self.om_shape(), dt, "offset_mask")
        if out is None:
            out = torch.empty(self.om_shape(), dtype=dt, device=om.device)
        else:
            self._check(out, self.om_shape(), dt, "out", om.device)
        if stream is None:
            stream = torch.cuda.current_stream(om.device).cuda_stream
        st = dcn4_dcnv3_softmax(self._h, om.data_ptr(), out.data_ptr(), stream)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_dcnv3_softmax")
        return out

    def dcnv3_forward(self, x, om, out=None, stream=None):
        """The aggregation with DCNv3's one-thread-per-channel layout
        (dcn4_dcnv3_forward); bit for bit dcn4_forward's result."""
        import torch
        d = self.desc
        dt = _torch_dtype(d.dtype)
        self._check(x, (d.N, d.H, d.W, d.C), dt, "x")
        dev = x.device
        self._check(om, self.om_shape(), dt, "offset_mask", dev)
        if out is None:
            out = torch.empty(self.out_shape(), dtype=dt, device=dev)
        else:
            self._check(out, self.out_shape(), dt, "out", dev)
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        st = dcn4_dcnv3_forward(self._h, x.data_ptr(), om.data_ptr(), out.data_ptr(), stream)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_dcnv3_forward")
        return out

    def backward_workspace_bytes(self) -> int:
        """Device workspace the gathered grad_x needs (dcn4_backward_workspace_size)."""
        st, n = dcn4_backward_workspace_size(self._h)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_backward_workspace_size")
        return n

    def backward(self, x, om, grad_y, scales=None, pixel_scales=None, want_x=True,
                 want_om=True, grad_x=None, grad_om=None, stream=None, workspace=None,
                 scatter=False):
        """(grad_x [N,H,W,C] fp32 or None, grad_om [N,Ho,Wo,G,3K] fp32 or
        None) for the upstream gradient grad_y [N,Ho,Wo,C].  grad_x is
        gathered through a workspace (a uint8 device tensor of at least
        backward_workspace_bytes(); allocated here when not given), or with
        scatter=True added with fp32 atomics and no workspace."""
        import torch
        d = self.desc
        dt = _torch_dtype(d.dtype)
        self._check(x, (d.N, d.H, d.W, d.C), dt, "x")
        dev = x.device
        self._check(om, self.om_shape(), dt, "offset_mask", dev)
        self._check(grad_y, self.out_shape(), dt, "grad_y", dev)
        if scales is not None:
            self._check(scales, (d.group,), torch.float32, "group_scales", dev)
        if pixel_scales is not None:
            self._check(pixel_scales, (d.N, self.Ho, self.Wo, d.group), torch.float32,
                        "pixel_scales", dev)
        if want_x and grad_x is None:
            grad_x = torch.empty((d.N, d.H, d.W, d.C), dtype=torch.float32, device=x.device)
        if want_om and grad_om is None:
            grad_om = torch.empty(self.om_shape(), dtype=torch.float32, device=x.device)
        if grad_x is not None:
            self._check(grad_x, (d.N, d.H, d.W, d.C), torch.float32, "grad_x", dev)
        if grad_om is not None:
            self._check(grad_om, self.om_shape(), torch.float32, "grad_offset_mask", dev)
        ws_ptr, ws_bytes = None, 0
        if grad_x is not None and not scatter:
            need = self.backward_workspace_bytes()
            if need and workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
            if need:
                if (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8
                        or workspace.device != x.device or not workspace.is_contiguous()):
                    raise ValueError("workspace must be a contiguous uint8 tensor on x's device")
                ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        st = dcn4_backward_ws(self._h, x.data_ptr(), om.data_ptr(),
                              None if scales is None else scales.data_ptr(),
                              None if pixel_scales is None else pixel_scales.data_ptr(),
                              grad_y.data_ptr(),
                              None if grad_x is None else grad_x.data_ptr(),
                              None if grad_om is None else grad_om.data_ptr(),
                              ws_ptr, ws_bytes, stream)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_backward_ws")
        return grad_x, grad_om

    def backward_scales(self, x, om, grad_y, scales, pixel_scales=None, want_group=True,
                        want_pixel=True, stream=None):
        """(grad_group_scales [G] fp32 or None, grad_pixel_scales [N,Ho,Wo,G]
        fp32 or None) for the upstream gradient grad_y (group-scale plans)."""
        import torch
        d = self.desc
        dt = _torch_dtype(d.dtype)
        self._check(x, (d.N, d.H, d.W, d.C), dt, "x")
        dev = x.device
        self._check(om, self.om_shape(), dt, "offset_mask", dev)
        self._check(grad_y, self.out_shape(), dt, "grad_y", dev)
        self._check(scales, (d.group,), torch.float32, "group_scales", dev)
        if pixel_scales is not None:
            self._check(pixel_scales, (d.N, self.Ho, self.Wo, d.group), torch.float32,
                        "pixel_scales", dev)
        gsg = torch.empty(d.group, dtype=torch.float32, device=dev) if want_group else None
        gps = (torch.empty((d.N, self.Ho, self.Wo, d.group), dtype=torch.float32, device=dev)
               if want_pixel and d.use_pixel_scales else None)
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        st = dcn4_backward_scales(self._h, x.data_ptr(), om.data_ptr(), scales.data_ptr(),
                                  None if pixel_scales is None else pixel_scales.data_ptr(),
                                  grad_y.data_ptr(), None if gsg is None else gsg.data_ptr(),
                                  None if gps is None else gps.data_ptr(), stream)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_backward_scales")
        return gsg, gps

    def probe_geometry(self, om, scales=None, stream=None, pixel_scales=None):
        """Device geometry of every (n, yo, xo, g, k): dict of tensors."""
        import torch
        d = self.desc
        self._check(om, self.om_shape(), _torch_dtype(d.dtype), "offset_mask")
        n = d.N * self.Ho * self.Wo * d.group * d.kernel_h * d.kernel_w
        dev = om.device
        out = dict(y0=torch.empty(n, dtype=torch.int32, device=dev),
                   x0=torch.empty(n, dtype=torch.int32, device=dev),
                   lh=torch.empty(n, dtype=torch.float32, device=dev),
                   lw=torch.empty(n, dtype=torch.float32, device=dev),
                   inside=torch.empty(n, dtype=torch.uint8, device=dev))
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        st = dcn4_probe_geometry(self._h, om.data_ptr(),
                                 None if scales is None else scales.data_ptr(),
                                 None if pixel_scales is None else pixel_scales.data_ptr(),
                                 *(out[k].data_ptr() for k in ("y0", "x0", "lh", "lw", "inside")),
                                 stream)
        if st != DCN4_OK:
            raise DCN4Error(st, "dcn4_probe_geometry")
        return out

    def __del__(self, _destroy=_lib.dcn4_destroy):
        h = getattr(self, "_h", None)
        if h:
            _destroy(h)
            self._h = None


def loaded_library_path() -> str:
    return LIB_PATH
