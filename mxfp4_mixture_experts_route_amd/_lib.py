"""ctypes binding of libmoe_mx4.so: the C ABI declared in include/moe_mx4.h, same names.

Argument marshalling only: each function checks tensor dtypes/devices, allocates missing
outputs with torch (device memory is PyTorch's job), and calls the C entry point on the current
HIP stream. Every step of the chain runs in the library's kernels; there is no fallback — if the
library is missing, loading fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MOE_MX4_LIB names another build of the same sources (e.g. a sanitized one)
LIB_PATH = os.environ.get("MOE_MX4_LIB") or os.path.join(PKG, "libmoe_mx4.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EALIGN, MOE_ELAUNCH = 0, 1, 2, 3, 4
MOE_ACT_NONE, MOE_ACT_SWIGLU_OAI, MOE_ACT_SWIGLU_OAI_MX8 = 0, 1, 2
MOE_MAX_K, MOE_MAX_E, MOE_MAX_TILE_M = 16, 1024, 256

EXPORTS = ("moe_strerror", "moe_mpad_max", "moe_route_topk", "moe_bucket", "mx4_pack_experts",
           "mx4_moe_gemv", "mx4_moe_gemm", "moe_combine", "mx4_moe_decode", "moe_timing_arm",
           "moe_timing_read", "mx8_quantize", "mx4_moe_gemm_mx8", "moe_router",
           "mx4_moe_decode_persistent", "mx4_moe_decode_persistent_static", "moe_probe_read",
           "moe_probe_mfma_bf16")
MOE_DECODE_WS_WORDS = 544
MOE_ROUTER_MAX_ROUTED = 16384
MOE_ROUTER_WS_WORDS = 67584
MOE_MX8_GEMM_MAX_K = 4096


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({strerror(status)})")


class Mx4ExpertsC(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("E", ctypes.c_int), ("N", ctypes.c_int), ("K", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library once; raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch first: the library and torch must share one HIP runtime. Both runtimes carry the
        # soname libamdhip64.so.7, and the process keeps whichever is loaded first; loaded
        # first, the library (RUNPATH: the system ROCm) would put torch on a runtime other than
        # the one it ships with, and launches then fail (launches rejected, then a crash in
        # torch's own copies)
        _torch()
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mxfp4_mixture_experts_route_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci, cf = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_strerror.argtypes = [ci]
        L.moe_mpad_max.restype = i64
        L.moe_mpad_max.argtypes = [i64, ci, ci, ci]
        L.moe_route_topk.restype = ci
        L.moe_route_topk.argtypes = [vp, i64, ci, ci, vp, vp, vp]
        L.moe_bucket.restype = ci
        L.moe_bucket.argtypes = [vp, i64, ci, ci, ci, i64, vp, vp, vp, vp, vp]
        L.mx4_pack_experts.restype = ci
        L.mx4_pack_experts.argtypes = [vp, vp, ci, ci, ci, vp, vp, vp]
        proj = [vp, vp, i64, ctypes.POINTER(Mx4ExpertsC), vp, vp, ci, i64, ci, cf, cf, vp, vp]
        for name in ("mx4_moe_gemv", "mx4_moe_gemm"):
            getattr(L, name).restype = ci
            getattr(L, name).argtypes = proj
        L.moe_combine.restype = ci
        L.moe_combine.argtypes = [vp, i64, vp, vp, i64, ci, ci, vp, vp]
        L.moe_timing_arm.restype = ci
        L.moe_timing_arm.argtypes = [ci]
        L.moe_timing_read.restype = ci
        L.moe_timing_read.argtypes = [ctypes.POINTER(ctypes.c_float), ci]
        pe = ctypes.POINTER(Mx4ExpertsC)
        L.mx4_moe_decode.restype = ci
        L.mx4_moe_decode.argtypes = [vp, vp, i64, ci, ci, pe, pe, cf, cf,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.mx4_moe_decode_persistent.restype = ci
        L.mx4_moe_decode_persistent.argtypes = [vp, vp, i64, ci, ci, pe, pe, cf, cf, vp, vp, vp,
                                                vp, vp, vp, vp, vp, vp, vp, ci, vp]
        L.mx4_moe_decode_persistent_static.restype = ci
        L.mx4_moe_decode_persistent_static.argtypes = [vp, vp, i64, ci, ci, pe, pe, cf, cf, vp,
                                                       vp, vp, vp, vp, vp, vp, vp, vp, ci, vp]
        L.moe_router.restype = ci
        L.moe_router.argtypes = [vp, vp, vp, i64, ci, ci, ci, ci, i64, vp, vp, vp, vp, vp, vp,
                                 vp, vp, vp]
        L.mx8_quantize.restype = ci
        L.mx8_quantize.argtypes = [vp, vp, i64, ci, vp, vp, vp]
        L.mx4_moe_gemm_mx8.restype = ci
        L.mx4_moe_gemm_mx8.argtypes = [vp, vp, vp, i64, ctypes.POINTER(Mx4ExpertsC), vp, vp, ci,
                                       i64, ci, cf, cf, vp, vp, vp]
        L.moe_probe_read.restype = ci
        L.moe_probe_read.argtypes = [vp, i64, vp, ci, vp]
        L.moe_probe_mfma_bf16.restype = ci
        L.moe_probe_mfma_bf16.argtypes = [ci, ci, vp, vp]
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def moe_mpad_max(T: int, k: int, E: int, tile_m: int) -> int:
    return int(lib().moe_mpad_max(int(T), int(k), int(E), int(tile_m)))


# ---------------------------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, dtype, name):
    torch = _torch()
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    del torch


def _call(fn: str, *args):
    st = getattr(lib(), fn)(*args)
    if st != MOE_OK:
        raise MoeError(fn, st)


class MX4Experts:
    """A device-resident MXFP4 expert stack in the chunked layout the projections read.

    Built from the checkpoint (row-major) layout — q u8 [E][N][K/2], s u8 [E][N][K/32] — with one
    mx4_pack_experts call on the current stream; bias f32 [E][N] or None. Holds the tensors alive
    and the C descriptor."""

    def __init__(self, q, s, bias=None, stream=None):
        torch = _torch()
        _check(q, torch.uint8, "q")
        _check(s, torch.uint8, "s")
        E, N, half_k = q.shape
        K = half_k * 2
        if tuple(s.shape) != (E, N, K // 32):
            raise ValueError(f"s: expected shape {(E, N, K // 32)}, got {tuple(s.shape)}")
        if bias is not None:
            _check(bias, torch.float32, "bias")
            if tuple(bias.shape) != (E, N):
                raise ValueError(f"bias: expected shape {(E, N)}")
        qp = torch.empty_like(q)
        sp = torch.empty((E, scale_row_bytes(K) // 16, N, 16), dtype=torch.uint8, device=q.device)
        _call("mx4_pack_experts", _ptr(q), _ptr(s), E, N, K, _ptr(qp), _ptr(sp), _stream(stream))
        self.q, self.s, self.bias = qp, sp, bias
        self.E, self.N, self.K = E, N, K
        self.c = Mx4ExpertsC(qp.data_ptr(), sp.data_ptr(),
                             None if bias is None else bias.data_ptr(), E, N, K)

    @classmethod
    def from_numpy(cls, d: dict, device="cuda"):
        torch = _torch()
        q = torch.from_numpy(np_contig(d["q"])).to(device)
        s = torch.from_numpy(np_contig(d["s"])).to(device)
        b = None if d.get("bias") is None else torch.from_numpy(np_contig(d["bias"])).to(device)
        return cls(q, s, b)

    @property
    def nbytes(self) -> int:
        return self.q.numel() + self.s.numel()


def np_contig(a):
    import numpy as np
    a = np.ascontiguousarray(a)
    return a if a.flags.writeable else a.copy()


def scale_row_bytes(K: int) -> int:
    """K/32 padded to a multiple of 16: the scale bytes per row of the chunked layout (in
    groups of 16) and the pitch of MXFP8 scale rows."""
    return (K // 32 + 15) // 16 * 16


def mx4_pack_experts(q, s, q_dst=None, s_dst=None, stream=None):
    """Checkpoint-layout MXFP4 stack -> chunked layout: q_dst like q, s_dst u8 [E][SP/16][N][16]
    (scale groups of 16 blocks, all rows of a group together)."""
    torch = _torch()
    _check(q, torch.uint8, "q")
    _check(s, torch.uint8, "s")
    E, N, half_k = q.shape
    q_dst = torch.empty_like(q) if q_dst is None else q_dst
    if s_dst is None:
        s_dst = torch.empty((E, scale_row_bytes(half_k * 2) // 16, N, 16), dtype=torch.uint8,
                            device=q.device)
    _call("mx4_pack_experts", _ptr(q), _ptr(s), E, N, half_k * 2, _ptr(q_dst), _ptr(s_dst),
          _stream(stream))
    return q_dst, s_dst


def moe_route_topk(logits, k: int, ids=None, w=None, stream=None):
    """ids i32 [T][k], w f32 [T][k] = top-k routing of f32 logits [T][E]."""
    torch = _torch()
    _check(logits, torch.float32, "logits")
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device) if w is None else w
    _call("moe_route_topk", _ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream))
    return ids, w


def moe_router(x, w_r, b_r, k: int, tile_m: int, ws, mpad_max: int | None = None,
               want_logits: bool = True, out=None, stream=None):
    """Router projection + top-k + bucket in one launch. x bf16 [T][D], w_r bf16 [E][D], b_r f32
    [E] or None, ws an int32/uint32 device tensor of MOE_ROUTER_WS_WORDS elements, zero before
    its first use and then left to the library (word 0 is left zero). Returns a dict: logits (if
    want_logits), ids, w, counts, basep, row_tok, pos, mpad."""
    torch = _torch()
    _check(x, torch.bfloat16, "x")
    _check(w_r, torch.bfloat16, "w_r")
    if b_r is not None:
        _check(b_r, torch.float32, "b_r")
    T, D = x.shape
    E = w_r.shape[0]
    if mpad_max is None:
        mpad_max = moe_mpad_max(T, k, E, tile_m)
    dev = x.device
    o = dict(out or {})
    shapes = {"ids": ((T, k), torch.int32), "w": ((T, k), torch.float32),
              "counts": ((E,), torch.int32), "basep": ((E + 1,), torch.int32),
              "row_tok": ((mpad_max,), torch.int32), "pos": ((T, k), torch.int32)}
    if want_logits:
        shapes["logits"] = ((T, E), torch.float32)
    for key, (shape, dt) in shapes.items():
        if key not in o:
            o[key] = torch.empty(shape, dtype=dt, device=dev)
    _call("moe_router", _ptr(x), _ptr(w_r), _ptr(b_r), T, D, E, k, tile_m, mpad_max,
          _ptr(o.get("logits")), _ptr(o["ids"]), _ptr(o["w"]), _ptr(o["counts"]), _ptr(o["basep"]),
          _ptr(o["row_tok"]), _ptr(o["pos"]), _ptr(ws), _stream(stream))
    o["mpad"] = mpad_max
    return o


def moe_bucket(ids, E: int, tile_m: int, mpad_max: int | None = None, out=None, stream=None):
    """(counts [E], basep [E+1], row_tok [mpad_max], pos [T][k]) of i32 ids [T][k]."""
    torch = _torch()
    _check(ids, torch.int32, "ids")
    T, k = ids.shape
    if mpad_max is None:
        mpad_max = moe_mpad_max(T, k, E, tile_m)
    if out is None:
        dev = ids.device
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(mpad_max, dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev))
    counts, basep, row_tok, pos = out
    _call("moe_bucket", _ptr(ids), T, k, E, tile_m, mpad_max, _ptr(counts), _ptr(basep),
          _ptr(row_tok), _ptr(pos), _stream(stream))
    return counts, basep, row_tok, pos


def _projection(fn, a, a_row, w: MX4Experts, counts, basep, tile_m, mpad_max, act, alpha, limit,
                out, stream):
    torch = _torch()
    _check(a, torch.int16 if a.dtype == torch.int16 else torch.bfloat16, "a")
    if a_row is not None:
        _check(a_row, torch.int32, "a_row")
    _check(counts, torch.int32, "counts")
    _check(basep, torch.int32, "basep")
    if out is None:
        if act == MOE_ACT_SWIGLU_OAI:
            out = torch.empty((mpad_max, w.N // 2), dtype=torch.bfloat16, device=a.device)
        else:
            out = torch.empty((mpad_max, w.N), dtype=torch.float32, device=a.device)
    _call(fn, _ptr(a), _ptr(a_row), a.shape[0], ctypes.byref(w.c), _ptr(counts), _ptr(basep),
          tile_m, mpad_max, act, float(alpha), float(limit), _ptr(out), _stream(stream))
    return out


def mx4_moe_gemv(a, a_row, w, counts, basep, tile_m, mpad_max, act=MOE_ACT_NONE, alpha=1.702,
                 limit=7.0, out=None, stream=None):
    return _projection("mx4_moe_gemv", a, a_row, w, counts, basep, tile_m, mpad_max, act, alpha,
                       limit, out, stream)


def mx4_moe_gemm(a, a_row, w, counts, basep, tile_m, mpad_max, act=MOE_ACT_NONE, alpha=1.702,
                 limit=7.0, out=None, stream=None):
    return _projection("mx4_moe_gemm", a, a_row, w, counts, basep, tile_m, mpad_max, act, alpha,
                       limit, out, stream)


def mx8_quantize(a, live=None, out=None, stream=None):
    """MXFP8 rows of bf16 rows a [rows][K]: (q u8 [rows][K] E4M3, s u8 [rows][SP] e8m0 with
    SP = roundup(K/32, 16), padding 0). Rows with live[r] < 0 are left unwritten."""
    torch = _torch()
    _check(a, torch.bfloat16, "a")
    if live is not None:
        _check(live, torch.int32, "live")
    rows, K = a.shape
    if out is None:
        out = (torch.empty((rows, K), dtype=torch.uint8, device=a.device),
               torch.empty((rows, scale_row_bytes(K)), dtype=torch.uint8, device=a.device))
    q, s = out
    _call("mx8_quantize", _ptr(a), _ptr(live), rows, K, _ptr(q), _ptr(s), _stream(stream))
    return q, s


def mx4_moe_gemm_mx8(aq, as_, a_row, w, counts, basep, tile_m, mpad_max, act=MOE_ACT_NONE,
                     alpha=1.702, limit=7.0, out=None, out_scale=None, stream=None):
    """mx4_moe_gemm over MXFP8 activation rows (aq, as_) from mx8_quantize. With
    MOE_ACT_SWIGLU_OAI_MX8 the SwiGLU rows come out as MXFP8 rows: returns (q, s)."""
    torch = _torch()
    _check(aq, torch.uint8, "aq")
    _check(as_, torch.uint8, "as")
    if a_row is not None:
        _check(a_row, torch.int32, "a_row")
    _check(counts, torch.int32, "counts")
    _check(basep, torch.int32, "basep")
    if act == MOE_ACT_SWIGLU_OAI_MX8:
        F = w.N // 2
        if out is None:
            out = torch.empty((mpad_max, F), dtype=torch.uint8, device=aq.device)
        if out_scale is None:
            out_scale = torch.empty((mpad_max, scale_row_bytes(F)), dtype=torch.uint8,
                                    device=aq.device)
    elif out is None:
        if act == MOE_ACT_SWIGLU_OAI:
            out = torch.empty((mpad_max, w.N // 2), dtype=torch.bfloat16, device=aq.device)
        else:
            out = torch.empty((mpad_max, w.N), dtype=torch.float32, device=aq.device)
    _call("mx4_moe_gemm_mx8", _ptr(aq), _ptr(as_), _ptr(a_row), aq.shape[0], ctypes.byref(w.c),
          _ptr(counts), _ptr(basep), tile_m, mpad_max, act, float(alpha), float(limit),
          _ptr(out), _ptr(out_scale), _stream(stream))
    return (out, out_scale) if act == MOE_ACT_SWIGLU_OAI_MX8 else out


def moe_combine(d, pos, w, out=None, stream=None):
    """y f32 [T][D] = slot-order routing-weighted sum of d rows."""
    torch = _torch()
    _check(d, torch.float32, "d")
    _check(pos, torch.int32, "pos")
    _check(w, torch.float32, "w")
    T, k = pos.shape
    D = d.shape[1]
    y = torch.empty((T, D), dtype=torch.float32, device=d.device) if out is None else out
    _call("moe_combine", _ptr(d), d.shape[0], _ptr(pos), _ptr(w), T, k, D, _ptr(y),
          _stream(stream))
    return y


def mx4_moe_decode(logits, x, gate_up: MX4Experts, down: MX4Experts, k: int,
                   alpha: float = 1.702, limit: float = 7.0, want_d: bool = False, out=None,
                   stream=None):
    """Fused decode chain of a few tokens (two launches). Returns a dict with ids, w, counts,
    basep, row_tok, pos (CSR with tile_m = 1), h [T*k][F] and d [T*k][D] in routed-row order
    (d only with want_d), and y [T][D]. `out` may hold preallocated tensors under those keys."""
    torch = _torch()
    _check(logits, torch.float32, "logits")
    _check(x, torch.bfloat16, "x")
    T, E = logits.shape
    D, F = gate_up.K, gate_up.N // 2
    dev = logits.device
    o = dict(out or {})
    shapes = {"ids": ((T, k), torch.int32), "w": ((T, k), torch.float32),
              "counts": ((E,), torch.int32), "basep": ((E + 1,), torch.int32),
              "row_tok": ((T * k,), torch.int32), "pos": ((T, k), torch.int32),
              "h": ((T * k, F), torch.bfloat16), "y": ((T, D), torch.float32)}
    if want_d:
        shapes["d"] = ((T * k, D), torch.float32)
    for key, (shape, dt) in shapes.items():
        if key not in o:
            o[key] = torch.empty(shape, dtype=dt, device=dev)
    _call("mx4_moe_decode", _ptr(logits), _ptr(x), T, E, k, ctypes.byref(gate_up.c),
          ctypes.byref(down.c), float(alpha), float(limit), _ptr(o["ids"]), _ptr(o["w"]),
          _ptr(o["counts"]), _ptr(o["basep"]), _ptr(o["row_tok"]), _ptr(o["pos"]), _ptr(o["h"]),
          _ptr(o.get("d")), _ptr(o["y"]), _stream(stream))
    return o


def mx4_moe_decode_persistent(logits, x, gate_up: MX4Experts, down: MX4Experts, k: int, ws,
                              alpha: float = 1.702, limit: float = 7.0, want_d: bool = False,
                              out=None, max_workgroups: int = 0, stream=None):
    """mx4_moe_decode in one launch. ws: an int32 device tensor of MOE_DECODE_WS_WORDS words,
    zero before its first use and then left to the library (word 3 is the error flag). Same
    outputs as mx4_moe_decode."""
    torch = _torch()
    _check(logits, torch.float32, "logits")
    _check(x, torch.bfloat16, "x")
    T, E = logits.shape
    D, F = gate_up.K, gate_up.N // 2
    dev = logits.device
    o = dict(out or {})
    shapes = {"ids": ((T, k), torch.int32), "w": ((T, k), torch.float32),
              "counts": ((E,), torch.int32), "basep": ((E + 1,), torch.int32),
              "row_tok": ((T * k,), torch.int32), "pos": ((T, k), torch.int32),
              "h": ((T * k, F), torch.bfloat16), "y": ((T, D), torch.float32)}
    if want_d:
        shapes["d"] = ((T * k, D), torch.float32)
    for key, (shape, dt) in shapes.items():
        if key not in o:
            o[key] = torch.empty(shape, dtype=dt, device=dev)
    _call("mx4_moe_decode_persistent", _ptr(logits), _ptr(x), T, E, k, ctypes.byref(gate_up.c),
          ctypes.byref(down.c), float(alpha), float(limit), _ptr(o["ids"]), _ptr(o["w"]),
          _ptr(o["counts"]), _ptr(o["basep"]), _ptr(o["row_tok"]), _ptr(o["pos"]), _ptr(o["h"]),
          _ptr(o.get("d")), _ptr(o["y"]), _ptr(ws), int(max_workgroups), _stream(stream))
    return o


def mx4_moe_decode_persistent_static(logits, x, gate_up: MX4Experts, down: MX4Experts, k: int,
                                     out: dict, alpha: float = 1.702, limit: float = 7.0,
                                     max_workgroups: int = 0, stream=None):
    """mx4_moe_decode_persistent with the library's own workspace (allocates nothing). out: the
    caller's output tensors, keys ids, w, counts, basep, row_tok, pos, h, y and optionally d."""
    torch = _torch()
    _check(logits, torch.float32, "logits")
    _check(x, torch.bfloat16, "x")
    T, E = logits.shape
    _call("mx4_moe_decode_persistent_static", _ptr(logits), _ptr(x), T, E, k,
          ctypes.byref(gate_up.c), ctypes.byref(down.c), float(alpha), float(limit),
          _ptr(out["ids"]), _ptr(out["w"]), _ptr(out["counts"]), _ptr(out["basep"]),
          _ptr(out["row_tok"]), _ptr(out["pos"]), _ptr(out["h"]), _ptr(out.get("d")),
          _ptr(out["y"]), int(max_workgroups), _stream(stream))
    return out


def moe_timing_arm(n: int) -> None:
    """Time the library's next n kernel launches (kernel execution only); 0 disarms."""
    _call("moe_timing_arm", int(n))


def moe_timing_read(n: int) -> list:
    """Durations in ms of the first n launches timed since moe_timing_arm (waits for them)."""
    buf = (ctypes.c_float * max(1, n))()
    _call("moe_timing_read", buf, int(n))
    return [float(buf[i]) for i in range(n)]


def moe_layer(x, logits, gate_up: MX4Experts, down: MX4Experts, k: int, tile_m: int,
              alpha: float = 1.702, limit: float = 7.0, projection: str = "gemm", stream=None):
    """One routed-expert MoE layer: route -> bucket -> gate_up+SwiGLU -> down -> combine.
    projection: "gemm" or "gemv" (bf16 activations), or "gemm_mx8" (MXFP8 activations on the
    MX-scaled MFMA: x quantized once, h written as MXFP8 rows by the gate_up epilogue; returns
    xq/xs/hq/hs and no bf16 h).
    Returns a dict of every intermediate (device tensors)."""
    if projection not in ("gemm", "gemv", "gemm_mx8"):
        raise ValueError(f"unknown projection {projection!r}")
    T, E = logits.shape
    ids, w = moe_route_topk(logits, k, stream=stream)
    mpad = moe_mpad_max(T, k, E, tile_m)
    counts, basep, row_tok, pos = moe_bucket(ids, E, tile_m, mpad, stream=stream)
    extra = {}
    if projection == "gemm_mx8":
        xq, xs = mx8_quantize(x, stream=stream)
        hq, hs = mx4_moe_gemm_mx8(xq, xs, row_tok, gate_up, counts, basep, tile_m, mpad,
                                  MOE_ACT_SWIGLU_OAI_MX8, alpha, limit, stream=stream)
        d = mx4_moe_gemm_mx8(hq, hs, None, down, counts, basep, tile_m, mpad, MOE_ACT_NONE,
                             alpha, limit, stream=stream)
        h = None
        extra = {"xq": xq, "xs": xs, "hq": hq, "hs": hs}
    else:
        fn = mx4_moe_gemm if projection == "gemm" else mx4_moe_gemv
        h = fn(x, row_tok, gate_up, counts, basep, tile_m, mpad, MOE_ACT_SWIGLU_OAI, alpha,
               limit, stream=stream)
        d = fn(h, None, down, counts, basep, tile_m, mpad, MOE_ACT_NONE, alpha, limit,
               stream=stream)
    y = moe_combine(d, pos, w, stream=stream)
    return {"ids": ids, "w": w, "mpad": mpad, "counts": counts, "basep": basep,
            "row_tok": row_tok, "pos": pos, "h": h, "d": d, "y": y, **extra}


# ---------------------------------------------------------------------------------------------
# attained-peak probes (measurement only)
# ---------------------------------------------------------------------------------------------

def moe_probe_read(buf, workgroups: int, sink=None, stream=None):
    """Read every byte of the device tensor `buf` once (moe_probe_read); returns the sink."""
    torch = _torch()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _call("moe_probe_read", _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
          int(workgroups), _stream(stream))
    return sink


def moe_probe_mfma_bf16(workgroups: int, iters: int, sink=None, stream=None):
    """workgroups * 4 * iters * 4 bf16 MFMAs of 32768 flops each (moe_probe_mfma_bf16)."""
    torch = _torch()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    _call("moe_probe_mfma_bf16", int(workgroups), int(iters), _ptr(sink), _stream(stream))
    return sink
