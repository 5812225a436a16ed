"""CPU oracle for the DCNv4 forward spatial aggregation -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It loads ``libdcn4_oracle.so``, built
from the plain C in ``dcn4_oracle.c`` (gcc, ``-O2 -ffp-contract=off``), and
shares no code with the HIP library in ``dynamic_sparse_vision_dcn4_amd``.

The arithmetic and the readings of the pages it follows are documented in
``dcn4_oracle.c``; this module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dcn4_oracle.c")
LIB_PATH = os.path.join(_HERE, "libdcn4_oracle.so")

F32, BF16, F16 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "bf16": BF16, "f16": F16}
RAW_NP = {F32: np.float32, BF16: np.uint16, F16: np.uint16}


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (plain IEEE arithmetic, no contraction)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-std=c11", "-Wall", "-shared", "-fPIC", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("N", "H", "W", "C", "G", "kh", "kw", "sh", "sw", "ph", "pw",
                 "dh", "dw")] + [("offset_scale", ctypes.c_float),
                                 ("multiscale", ctypes.c_int32),
                                 ("pixel_scales", ctypes.c_int32),
                                 ("max_scale", ctypes.c_float)]


@dataclass(frozen=True)
class Shape:
    """Operator geometry: input [N,H,W,C] channel-last, G groups."""
    N: int
    H: int
    W: int
    C: int
    G: int
    kh: int = 3
    kw: int = 3
    sh: int = 1
    sw: int = 1
    ph: int = 1
    pw: int = 1
    dh: int = 1
    dw: int = 1
    offset_scale: float = 1.0
    multiscale: bool = False
    pixel_scales: bool = False   # FlowDCN predicted scale per (pixel, group)
    max_scale: float = 0.0       # > 0: Smax clamp of the effective scale

    @property
    def K(self) -> int:
        return self.kh * self.kw

    def c_struct(self) -> _Shape:
        return _Shape(self.N, self.H, self.W, self.C, self.G, self.kh, self.kw,
                      self.sh, self.sw, self.ph, self.pw, self.dh, self.dw,
                      float(self.offset_scale), int(bool(self.multiscale)),
                      int(bool(self.pixel_scales)), float(self.max_scale))


class Oracle:
    """ctypes view of one built oracle library (a mutant build can be loaded
    from another path by the tests that check the pins catch mistakes)."""

    def __init__(self, path: str = LIB_PATH):
        if path == LIB_PATH and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        sp = ctypes.POINTER(_Shape)
        lib.dcn4o_check.argtypes = [sp, i32p, i32p]
        lib.dcn4o_forward_f64.argtypes = [sp, ctypes.c_int, P, P, P, P, P, P,
                                          ctypes.c_int64, ctypes.c_int]
        lib.dcn4o_forward_f32.argtypes = [sp, ctypes.c_int, P, P, P, P, P, P, P,
                                          ctypes.c_int64, ctypes.c_int]
        lib.dcn4o_geometry.argtypes = [sp, ctypes.c_int, P, P, P, P, P, P, P, P,
                                       P, ctypes.c_int64]
        lib.dcn4o_count_terms.argtypes = [sp, ctypes.c_int, P, P, P, i64p, i64p]
        lib.dcn4o_backward.argtypes = [sp, ctypes.c_int, P, P, P, P, P, P, P, P, P, i64p]
        lib.dcn4o_backward_scales.argtypes = [sp, ctypes.c_int, P, P, P, P, P, P, P, P, P]
        lib.dcn4o_softmax_weights.argtypes = [sp, ctypes.c_int, P, P]
        lib.dcn4o_linear_f64.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int, P, P, P, P, P]
        lib.dcn4o_dwconv3x3.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int, P, P, P, P, P]
        lib.dcn4o_ideal_bytes.argtypes = [sp, ctypes.c_int]
        lib.dcn4o_ideal_bytes.restype = ctypes.c_int64
        for f in ("dcn4o_bf16_to_f32", "dcn4o_f16_to_f32"):
            getattr(lib, f).argtypes = [ctypes.c_uint16]
            getattr(lib, f).restype = ctypes.c_float
        for f in ("dcn4o_f32_to_bf16", "dcn4o_f32_to_f16"):
            getattr(lib, f).argtypes = [ctypes.c_float]
            getattr(lib, f).restype = ctypes.c_uint16
        self.lib = lib

    # -- helpers ----------------------------------------------------------
    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    @staticmethod
    def _pix(pix):
        if pix is None:
            return None, 0
        pix = np.ascontiguousarray(pix, dtype=np.int64)
        return pix, pix.size

    def out_size(self, s: Shape):
        ho, wo = ctypes.c_int32(), ctypes.c_int32()
        r = self.lib.dcn4o_check(ctypes.byref(s.c_struct()), ctypes.byref(ho),
                                 ctypes.byref(wo))
        if r:
            raise ValueError(f"invalid shape {s}")
        return ho.value, wo.value

    def _prep(self, s, dtype, x, om, scales, pscales=None):
        dt = DTYPE_CODES[dtype]
        raw = RAW_NP[dt]
        x = None if x is None else np.ascontiguousarray(x, dtype=raw)
        om = np.ascontiguousarray(om, dtype=raw)
        if s.multiscale:
            scales = np.ascontiguousarray(scales, dtype=np.float32)
            assert scales.size == s.G
        else:
            scales = None
        if s.pixel_scales:
            ho, wo = self.out_size(s)
            pscales = np.ascontiguousarray(pscales, dtype=np.float32)
            assert pscales.size == s.N * ho * wo * s.G
        else:
            pscales = None
        return dt, x, om, scales, pscales

    # -- the oracle ---------------------------------------------------------
    def forward_f64(self, s: Shape, dtype: str, x, om, scales=None, pix=None,
                    nthreads: int = 8, pscales=None) -> np.ndarray:
        """The definition in fp64; returns [N,Ho,Wo,C] (or [npix,C]).
        pscales: [N,Ho,Wo,G] fp32 when s.pixel_scales."""
        dt, x, om, scales, pscales = self._prep(s, dtype, x, om, scales, pscales)
        ho, wo = self.out_size(s)
        pix, npix = self._pix(pix)
        shape = (s.N, ho, wo, s.C) if pix is None else (npix, s.C)
        y = np.empty(shape, np.float64)
        r = self.lib.dcn4o_forward_f64(ctypes.byref(s.c_struct()), dt,
                                       self._ptr(x), self._ptr(om),
                                       self._ptr(scales), self._ptr(pscales),
                                       self._ptr(y),
                                       self._ptr(pix), npix, nthreads)
        if r:
            raise ValueError("oracle rejected the call")
        return y

    def forward_f32(self, s: Shape, dtype: str, x, om, scales=None, pix=None,
                    nthreads: int = 8, want_acc: bool = False, pscales=None):
        """fp32 evaluation in the fixed order; returns the output in the I/O
        dtype's raw encoding (and the fp32 accumulators if asked)."""
        dt, x, om, scales, pscales = self._prep(s, dtype, x, om, scales, pscales)
        ho, wo = self.out_size(s)
        pix, npix = self._pix(pix)
        shape = (s.N, ho, wo, s.C) if pix is None else (npix, s.C)
        y = np.empty(shape, RAW_NP[dt])
        acc = np.empty(shape, np.float32) if want_acc else None
        r = self.lib.dcn4o_forward_f32(ctypes.byref(s.c_struct()), dt,
                                       self._ptr(x), self._ptr(om),
                                       self._ptr(scales), self._ptr(pscales),
                                       self._ptr(y),
                                       self._ptr(acc), self._ptr(pix), npix,
                                       nthreads)
        if r:
            raise ValueError("oracle rejected the call")
        return (y, acc) if want_acc else y

    def geometry(self, s: Shape, dtype: str, om, scales=None, pix=None, pscales=None):
        """Per (pixel, g, k): dict of inside, y0, x0, lh, lw arrays."""
        dt, _, om, scales, pscales = self._prep(s, dtype, None, om, scales, pscales)
        ho, wo = self.out_size(s)
        pix, npix = self._pix(pix)
        npx = s.N * ho * wo if pix is None else npix
        n = npx * s.G * s.K
        out = dict(y0=np.empty(n, np.int32), x0=np.empty(n, np.int32),
                   lh=np.empty(n, np.float32), lw=np.empty(n, np.float32),
                   inside=np.empty(n, np.uint8))
        r = self.lib.dcn4o_geometry(ctypes.byref(s.c_struct()), dt,
                                    self._ptr(om), self._ptr(scales),
                                    self._ptr(pscales),
                                    *(self._ptr(out[k]) for k in
                                      ("y0", "x0", "lh", "lw", "inside")),
                                    self._ptr(pix), npix)
        if r:
            raise ValueError("oracle rejected the call")
        return out

    def count_terms(self, s: Shape, dtype: str, om, scales=None, pscales=None):
        dt, _, om, scales, pscales = self._prep(s, dtype, None, om, scales, pscales)
        a, b = ctypes.c_int64(), ctypes.c_int64()
        r = self.lib.dcn4o_count_terms(ctypes.byref(s.c_struct()), dt,
                                       self._ptr(om), self._ptr(scales),
                                       self._ptr(pscales),
                                       ctypes.byref(a), ctypes.byref(b))
        if r:
            raise ValueError("oracle rejected the call")
        return a.value, b.value

    def backward(self, s: Shape, dtype: str, x, om, gy, scales=None, pscales=None,
                 want_x: bool = True, want_om: bool = True):
        """Gradients for upstream gy [N,Ho,Wo,C] (raw, I/O dtype): dict with
        gx [N,H,W,C] and gom [N,Ho,Wo,G,3K] (fp64), their absolute-term sums
        gx_abs, gom_abs, and max_terms."""
        dt, x, om, scales, pscales = self._prep(s, dtype, x, om, scales, pscales)
        gy = np.ascontiguousarray(gy, dtype=RAW_NP[dt])
        ho, wo = self.out_size(s)
        out = {}
        if want_x:
            out["gx"] = np.empty((s.N, s.H, s.W, s.C), np.float64)
            out["gx_abs"] = np.empty_like(out["gx"])
        if want_om:
            out["gom"] = np.empty((s.N, ho, wo, s.G, 3 * s.K), np.float64)
            out["gom_abs"] = np.empty_like(out["gom"])
        mt = ctypes.c_int64()
        r = self.lib.dcn4o_backward(ctypes.byref(s.c_struct()), dt, self._ptr(x),
                                    self._ptr(om), self._ptr(scales), self._ptr(pscales),
                                    self._ptr(gy), self._ptr(out.get("gx")),
                                    self._ptr(out.get("gom")), self._ptr(out.get("gx_abs")),
                                    self._ptr(out.get("gom_abs")), ctypes.byref(mt))
        if r:
            raise ValueError("oracle rejected the call")
        out["max_terms"] = mt.value
        return out

    def backward_scales(self, s: Shape, dtype: str, x, om, gy, scales, pscales=None):
        """Gradients of the group scales (group-scale mode) for upstream gy
        [N,Ho,Wo,C] (raw, I/O dtype): dict with gs [G] (dL/ds_g), gs_abs, and
        with pixel scales gp [N,Ho,Wo,G] (dL/dsigma), gp_abs; fp64."""
        dt, x, om, scales, pscales = self._prep(s, dtype, x, om, scales, pscales)
        gy = np.ascontiguousarray(gy, dtype=RAW_NP[dt])
        ho, wo = self.out_size(s)
        out = {"gs": np.empty(s.G, np.float64), "gs_abs": np.empty(s.G, np.float64)}
        if s.pixel_scales:
            out["gp"] = np.empty((s.N, ho, wo, s.G), np.float64)
            out["gp_abs"] = np.empty_like(out["gp"])
        r = self.lib.dcn4o_backward_scales(ctypes.byref(s.c_struct()), dt, self._ptr(x),
                                           self._ptr(om), self._ptr(scales), self._ptr(pscales),
                                           self._ptr(gy), self._ptr(out["gs"]),
                                           self._ptr(out["gs_abs"]), self._ptr(out.get("gp")),
                                           self._ptr(out.get("gp_abs")))
        if r:
            raise ValueError("oracle rejected the call")
        return out

    def softmax_weights(self, s: Shape, dtype: str, om) -> np.ndarray:
        """DCNv3's softmax over each (pixel, group) row's K weights (reading
        R18), offsets unchanged: fp64 [N,Ho,Wo,G,3K] from the raw om."""
        dt = DTYPE_CODES[dtype]
        om = np.ascontiguousarray(om, dtype=RAW_NP[dt])
        ho, wo = self.out_size(s)
        out = np.empty((s.N, ho, wo, s.G, 3 * s.K), np.float64)
        assert om.size == out.size
        r = self.lib.dcn4o_softmax_weights(ctypes.byref(s.c_struct()), dt,
                                           self._ptr(om), self._ptr(out))
        if r:
            raise ValueError("oracle rejected the call")
        return out

    def dcnv3_forward_f64(self, s: Shape, dtype: str, x, om, pix=None,
                          nthreads: int = 8):
        """The DCNv3-style output: the aggregation with softmax weights,
        sum_k w_k * bilinear(x, p_k), in fp64, and the sum of the absolute
        values of its terms (the aggregation of |x| with the same weights,
        which are positive). The weights enter the fp64 aggregation rounded to fp32 (a relative
        change of at most 2^-24 each); x is decoded exactly."""
        w = self.softmax_weights(s, dtype, om).astype(np.float32)
        dt = DTYPE_CODES[dtype]
        xr = np.ascontiguousarray(x, dtype=RAW_NP[dt])
        if dt == 0:
            xf = xr
        elif dt == 1:
            xf = (xr.astype(np.uint32) << 16).view(np.float32)
        else:
            xf = xr.view(np.float16).astype(np.float32)
        y = self.forward_f64(s, "f32", xf, w, pix=pix, nthreads=nthreads)
        a = self.forward_f64(s, "f32", np.abs(xf), w, pix=pix, nthreads=nthreads)
        return y, a

    def linear(self, dtype: str, feat, weight, bias=None):
        """The merged offset/weight layer in fp64: (out [M, Nout], absum).
        feat [M, Cin] and weight [Nout, Cin] raw in the I/O dtype."""
        dt = DTYPE_CODES[dtype]
        feat = np.ascontiguousarray(feat, dtype=RAW_NP[dt])
        weight = np.ascontiguousarray(weight, dtype=RAW_NP[dt])
        M, Cin = feat.shape
        Nout = weight.shape[0]
        assert weight.shape[1] == Cin
        bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        out = np.empty((M, Nout), np.float64)
        absum = np.empty((M, Nout), np.float64)
        r = self.lib.dcn4o_linear_f64(M, Cin, Nout, dt, self._ptr(feat), self._ptr(weight),
                                      self._ptr(bias), self._ptr(out), self._ptr(absum))
        if r:
            raise ValueError("oracle rejected the call")
        return out, absum

    def dwconv3x3(self, dtype: str, x, w, bias=None):
        """The depthwise 3x3 convolution (stride 1, zero padding 1) in front of
        the offset/weight layer: (out fp64 [N,H,W,C], out raw in the I/O dtype
        from the fp32 evaluation).  x [N,H,W,C] and w [3,3,C] raw in the I/O
        dtype, bias fp32 [C] or None."""
        dt = DTYPE_CODES[dtype]
        x = np.ascontiguousarray(x, dtype=RAW_NP[dt])
        w = np.ascontiguousarray(w, dtype=RAW_NP[dt])
        N, H, W, C = x.shape
        assert w.shape == (3, 3, C)
        bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        out64 = np.empty((N, H, W, C), np.float64)
        raw = np.empty((N, H, W, C), RAW_NP[dt])
        r = self.lib.dcn4o_dwconv3x3(N, H, W, C, dt, self._ptr(x), self._ptr(w),
                                     self._ptr(bias), self._ptr(out64), self._ptr(raw))
        if r:
            raise ValueError("oracle rejected the call")
        return out64, raw

    def ideal_bytes(self, s: Shape, dtype: str) -> int:
        return int(self.lib.dcn4o_ideal_bytes(ctypes.byref(s.c_struct()),
                                              DTYPE_CODES[dtype]))

    # -- codecs -------------------------------------------------------------
    def bf16_to_f32(self, h: int) -> float:
        return self.lib.dcn4o_bf16_to_f32(h)

    def f16_to_f32(self, h: int) -> float:
        return self.lib.dcn4o_f16_to_f32(h)

    def f32_to_bf16(self, f: float) -> int:
        return self.lib.dcn4o_f32_to_bf16(f)

    def f32_to_f16(self, f: float) -> int:
        return self.lib.dcn4o_f32_to_f16(f)


_default = None


def get() -> Oracle:
    """The oracle built from ``dcn4_oracle.c`` (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
