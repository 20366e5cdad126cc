"""qi4 oracle -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

A plain fp64 CPU implementation of the int4 (and 8-bit) group-quantized
linear layer and the routed MoE expert FFN (see ``qi4_oracle.c`` for the definitions and the
page passages they follow).  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import this package.  It shares no code
with the GPU library and never imports it.

This module is a thin ctypes shim: it widens activations to float64, checks
shapes and calls the C functions, which hold the method's arithmetic.  One step
is a library primitive instead: the router projection (``router_logits``) is a
numpy fp64 matrix product.
Every exported function is pinned by tests in ``tests/test_oracle_*.py``; a
function whose pin is missing would say "parity unpinned" here (none does).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
#: the compiled oracle; QI4O_LIB names another build of it (the sanitizer build,
#: or a deliberately broken copy that the pins must reject)
_LIB_PATH = os.environ.get("QI4O_LIB") or os.path.join(_HERE, "libqi4_oracle.so")
_lib = None

#: relative tolerance factor of one linear layer: |gpu - oracle| <= C_TOL * sum|w*x|
C_TOL = 2e-3
#: bound on the error of the fp32 combine weights relative to the fp64 ones
EPS_P = 1e-5

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i8p = ctypes.POINTER(ctypes.c_int8)
_i64 = ctypes.c_int64


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no FP contraction)."""
    from oracle.build import build_oracle
    return build_oracle(verbose=verbose)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.qi4o_abi_version.restype = ctypes.c_int
        L.qi4o_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.qi4o_f16_to_f64.restype = ctypes.c_double
        L.qi4o_f64_to_f16.argtypes = [ctypes.c_double]
        L.qi4o_f64_to_f16.restype = ctypes.c_uint16
        L.qi4o_silu.argtypes = [ctypes.c_double]
        L.qi4o_silu.restype = ctypes.c_double
        ci = ctypes.c_int
        L.qi4o_unpack.argtypes = [_u8p, _i64, _i64, ci, _u8p]
        L.qi4o_dequant.argtypes = [_u8p, _u16p, _u8p, _i64, _i64, _i64, ci, _dp]
        L.qi4o_linear.argtypes = [_dp, _i64, _i64, _u8p, _u16p, _u8p, _i64, _i64, ci,
                                  _dp, _dp, ci]
        L.qi4o_gate_up_silu.argtypes = [_dp, _i64, _i64, _u8p, _u16p, _u8p, _i64, _i64, ci,
                                        ctypes.c_double, _dp, _dp, ci]
        L.qi4o_topk_softmax.argtypes = [_fp, _i64, _i64, ctypes.c_int, _i32p, _dp]
        L.qi4o_sort.argtypes = [_i32p, _i64, ctypes.c_int, _i64, _i32p, _i32p, _i32p]
        L.qi4o_moe.argtypes = ([_dp, _i64, _i64, _i64, _i64, ctypes.c_int, _i32p, _dp]
                               + [_u8p, _u16p, _u8p] * 4
                               + [_i64, ci, ctypes.c_double, ctypes.c_double, _dp, _dp, ci])
        L.qi4o_quantize.argtypes = [_dp, _i64, _i64, _i64, ci, _u8p, _u16p, _u8p]
        L.qi4o_quantize_act.argtypes = [_fp, _i64, ctypes.c_float, _i8p]
        L.qi4o_moe_w4a8.argtypes = ([_fp, _i64, _i64, _i64, _i64, ctypes.c_int, _i32p, _dp]
                                    + [_u8p, _u16p, _u8p] * 4
                                    + [_i64, ctypes.c_float, ctypes.c_float, ctypes.c_double,
                                       ctypes.c_double, ctypes.c_double, _dp, _dp, ci])
        L.qi4o_dequant_act.argtypes = [_i8p, _i64, ctypes.c_float, _dp]
        for f in ("qi4o_unpack", "qi4o_dequant", "qi4o_linear", "qi4o_gate_up_silu",
                  "qi4o_topk_softmax", "qi4o_sort", "qi4o_moe", "qi4o_quantize",
                  "qi4o_quantize_act", "qi4o_dequant_act", "qi4o_moe_w4a8"):
            getattr(L, f).restype = ctypes.c_int
        if L.qi4o_abi_version() != 5:
            raise RuntimeError("stale oracle library: rebuild it (oracle.build())")
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None, t):
    if a is None:
        return ctypes.cast(None, t)
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(t)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---- activations --------------------------------------------------------

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Activations to float64.  ``dtype`` 'bf16' means x holds bf16 bit patterns
    (uint16): the value is those 16 bits followed by 16 zero bits read as an IEEE
    binary32 number, which widens exactly to binary64."""
    if dtype == "bf16":
        assert x.dtype == np.uint16
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.ascontiguousarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---- scalar helpers -----------------------------------------------------

def f16_to_f64(bits: int) -> float:
    return lib().qi4o_f16_to_f64(int(bits))


def f64_to_f16(v: float) -> int:
    return int(lib().qi4o_f64_to_f16(float(v)))


def silu(v: float) -> float:
    return lib().qi4o_silu(float(v))


# ---- the format ----------------------------------------------------------
# ``bits`` 4: two codes per byte (qweight [N][K/2]); 8: one code per byte
# (qweight [N][K]), zeros 0..255.

def code_bytes(N: int, K: int, bits: int = 4) -> int:
    return N * K if bits == 8 else N * (K // 2)


def unpack(qweight: np.ndarray, N: int, K: int, bits: int = 4) -> np.ndarray:
    qweight = np.ascontiguousarray(qweight, dtype=np.uint8)
    assert qweight.size == code_bytes(N, K, bits)
    q = np.empty((N, K), dtype=np.uint8)
    _check(lib().qi4o_unpack(_ptr(qweight, _u8p), N, K, bits, _ptr(q, _u8p)), "unpack")
    return q


def dequant(qweight, scales, zeros, N: int, K: int, group: int = 128, bits: int = 4) -> np.ndarray:
    qweight = np.ascontiguousarray(qweight, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    assert qweight.size == code_bytes(N, K, bits) and scales.size == N * (K // group) == zeros.size
    w = np.empty((N, K), dtype=np.float64)
    _check(lib().qi4o_dequant(_ptr(qweight, _u8p), _ptr(scales, _u16p), _ptr(zeros, _u8p),
                              N, K, group, bits, _ptr(w, _dp)), "dequant")
    return w


# ---- the linear layer ------------------------------------------------------

def linear(x64: np.ndarray, qweight, scales, zeros, N: int, K: int, group: int = 128,
           threads: int | None = None, bits: int = 4):
    """Return (y, S): y = x . dequant(W)^T and S = sum_k |x*w|, both [T][N] float64."""
    x64 = np.ascontiguousarray(x64, dtype=np.float64).reshape(-1, K)
    T = x64.shape[0]
    qweight = np.ascontiguousarray(qweight, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    assert qweight.size == code_bytes(N, K, bits) and scales.size == N * (K // group) == zeros.size
    y = np.empty((T, N), dtype=np.float64)
    S = np.empty((T, N), dtype=np.float64)
    _check(lib().qi4o_linear(_ptr(x64, _dp), T, K, _ptr(qweight, _u8p), _ptr(scales, _u16p),
                             _ptr(zeros, _u8p), N, group, bits, _ptr(y, _dp), _ptr(S, _dp),
                             threads or default_threads()), "linear")
    return y, S


# ---- W4A8: int8 activations with a static per-tensor scale (R30) -----------

def act_reciprocal(x_scale: float) -> np.float32:
    """r = float32(1 / s_x), the float32 quotient of the float32 scale."""
    return np.float32(1.0) / np.float32(x_scale)


def quantize_act(x32: np.ndarray, x_scale: float) -> np.ndarray:
    """int8 activations a = clamp(rint(float32(x * r)), -127, 127), same shape as x32
    (float32 values; bf16 inputs widen exactly)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    a = np.empty(x32.shape, dtype=np.int8)
    _check(lib().qi4o_quantize_act(_ptr(x32, _fp), x32.size, act_reciprocal(x_scale),
                                   _ptr(a, _i8p)), "quantize_act")
    return a


def dequant_act(a: np.ndarray, x_scale: float) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int8)
    xh = np.empty(a.shape, dtype=np.float64)
    _check(lib().qi4o_dequant_act(_ptr(a, _i8p), a.size, np.float32(x_scale), _ptr(xh, _dp)),
           "dequant_act")
    return xh


def linear_w4a8(x32: np.ndarray, x_scale: float, qweight, scales, zeros, N: int, K: int,
                group: int = 128, threads: int | None = None):
    """W4A8 linear: (y, S, a) with y = xhat . dequant(W)^T for xhat = a * s_x, the
    int8 activations a of quantize_act, and S = sum_k |xhat * w|."""
    a = quantize_act(x32, x_scale)
    y, S = linear(dequant_act(a, x_scale), qweight, scales, zeros, N, K, group, threads)
    return y, S, a


def gate_up_silu(x64: np.ndarray, qweight, scales, zeros, I: int, K: int, group: int = 128,
                 c: float = C_TOL, threads: int | None = None, bits: int = 4):
    """Return (h, tol_h) for the fused SiLU(gate)*up of a [gate; up] weight (2I x K)."""
    x64 = np.ascontiguousarray(x64, dtype=np.float64).reshape(-1, K)
    T = x64.shape[0]
    h = np.empty((T, I), dtype=np.float64)
    tol = np.empty((T, I), dtype=np.float64)
    _check(lib().qi4o_gate_up_silu(_ptr(x64, _dp), T, K,
                                   _ptr(np.ascontiguousarray(qweight, dtype=np.uint8), _u8p),
                                   _ptr(np.ascontiguousarray(scales, dtype=np.uint16), _u16p),
                                   _ptr(np.ascontiguousarray(zeros, dtype=np.uint8), _u8p),
                                   I, group, bits, c, _ptr(h, _dp), _ptr(tol, _dp),
                                   threads or default_threads()), "gate_up_silu")
    return h, tol


# ---- router and permutation ----------------------------------------------

def router_logits(x64: np.ndarray, w_bits: np.ndarray):
    """Router logits l[t][e] = sum_k x[t][k] * w[e][k] and the magnitude
    S[t][e] = sum_k |x[t][k] * w[e][k]|, in fp64, for bf16 router weights w [E][H]
    (bit patterns) and activations already widened to fp64.  The step before the
    top-k selection (reading R28: a plain bias-free projection of the hidden
    state onto the E experts); the library matmul is the step."""
    w64 = widen(np.ascontiguousarray(w_bits), "bf16")
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    return x64 @ w64.T, np.abs(x64) @ np.abs(w64).T


def topk_softmax(logits: np.ndarray, k: int):
    """Return (ids int32 [T][k], p float64 [T][k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    p = np.empty((T, k), dtype=np.float64)
    _check(lib().qi4o_topk_softmax(_ptr(logits, _fp), T, E, k, _ptr(ids, _i32p), _ptr(p, _dp)),
           "topk_softmax")
    return ids, p


def sort_tokens(ids: np.ndarray, E: int):
    """Return (sorted_pairs [T*k], offsets [E+1], pair_to_sorted [T*k]), all int32."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    sp = np.empty(T * k, dtype=np.int32)
    off = np.empty(E + 1, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    _check(lib().qi4o_sort(_ptr(ids, _i32p), T, k, E, _ptr(sp, _i32p), _ptr(off, _i32p),
                           _ptr(inv, _i32p)), "sort")
    return sp, off, inv


# ---- the MoE FFN -------------------------------------------------------------

def moe(x64: np.ndarray, ids: np.ndarray, p: np.ndarray, experts: dict, shared: dict | None,
        H: int, I: int, E: int, group: int = 128, c: float = C_TOL, eps_p: float = EPS_P,
        threads: int | None = None, bits: int = 4):
    """Return (out, tol), both [T][H] float64.

    ``experts`` holds canonical arrays for all E routed experts:
    gu_q [E][2I][H/2], gu_s/gu_z [E][2I][H/G], dn_q [E][H][I/2], dn_s/dn_z [E][H][I/G]
    (with ``bits`` 8 the code arrays are [E][2I][H] and [E][H][I]).
    ``shared`` holds the same keys for one expert (no leading E), or None.
    ``group`` 0 means one group per row of each matrix (H for gate/up, I for down).
    """
    x64 = np.ascontiguousarray(x64, dtype=np.float64).reshape(-1, H)
    T = x64.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    p = np.ascontiguousarray(p, dtype=np.float64)
    k = ids.shape[1]
    out = np.empty((T, H), dtype=np.float64)
    tol = np.empty((T, H), dtype=np.float64)

    def arrs(d):
        if d is None:
            return [None] * 6
        return [np.ascontiguousarray(d["gu_q"], dtype=np.uint8),
                np.ascontiguousarray(d["gu_s"], dtype=np.uint16),
                np.ascontiguousarray(d["gu_z"], dtype=np.uint8),
                np.ascontiguousarray(d["dn_q"], dtype=np.uint8),
                np.ascontiguousarray(d["dn_s"], dtype=np.uint16),
                np.ascontiguousarray(d["dn_z"], dtype=np.uint8)]

    ea, sa = arrs(experts), arrs(shared)
    types = [_u8p, _u16p, _u8p] * 2
    _check(lib().qi4o_moe(_ptr(x64, _dp), T, H, I, E, k, _ptr(ids, _i32p), _ptr(p, _dp),
                          *[_ptr(a, t) for a, t in zip(ea, types)],
                          *[_ptr(a, t) for a, t in zip(sa, types)],
                          group, bits, c, eps_p, _ptr(out, _dp), _ptr(tol, _dp),
                          threads or default_threads()), "moe")
    return out, tol


#: relative bound on the W4A8 GPU path's error in g and u (exact int32 sums; a few
#: float32 roundings), used only to find the int8 h decisions that may differ
C_AMB_W4A8 = 1e-4


def moe_w4a8(x32: np.ndarray, x_scale: float, h_scale: float, ids: np.ndarray, p: np.ndarray,
             experts: dict, shared: dict | None, H: int, I: int, E: int, group: int = 128,
             c: float = C_TOL, c_amb: float = C_AMB_W4A8, eps_p: float = EPS_P,
             threads: int | None = None):
    """W4A8 MoE layer: (out, tol), both [T][H] float64.  x32 float32 [T][H] (bf16
    inputs widen exactly); int8 activations with static scales x_scale (layer
    input) and h_scale (the down projection's input); 4-bit expert weights as in
    moe()."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32).reshape(-1, H)
    T = x32.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    p = np.ascontiguousarray(p, dtype=np.float64)
    k = ids.shape[1]
    out = np.empty((T, H), dtype=np.float64)
    tol = np.empty((T, H), dtype=np.float64)

    def arrs(d):
        if d is None:
            return [None] * 6
        return [np.ascontiguousarray(d["gu_q"], dtype=np.uint8),
                np.ascontiguousarray(d["gu_s"], dtype=np.uint16),
                np.ascontiguousarray(d["gu_z"], dtype=np.uint8),
                np.ascontiguousarray(d["dn_q"], dtype=np.uint8),
                np.ascontiguousarray(d["dn_s"], dtype=np.uint16),
                np.ascontiguousarray(d["dn_z"], dtype=np.uint8)]

    ea, sa = arrs(experts), arrs(shared)
    types = [_u8p, _u16p, _u8p] * 2
    _check(lib().qi4o_moe_w4a8(_ptr(x32, _fp), T, H, I, E, k, _ptr(ids, _i32p), _ptr(p, _dp),
                               *[_ptr(a, t) for a, t in zip(ea, types)],
                               *[_ptr(a, t) for a, t in zip(sa, types)],
                               group, np.float32(x_scale), np.float32(h_scale), c, c_amb, eps_p,
                               _ptr(out, _dp), _ptr(tol, _dp), threads or default_threads()),
           "moe_w4a8")
    return out, tol


# ---- reference quantizer -------------------------------------------------

def quantize(w: np.ndarray, group: int = 128, bits: int = 4):
    """Min/max asymmetric quantizer with 2^bits - 1 levels; returns canonical
    (qweight, scales, zeros)."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    N, K = w.shape
    qw = np.empty((N, K if bits == 8 else K // 2), dtype=np.uint8)
    s = np.empty((N, K // group), dtype=np.uint16)
    z = np.empty((N, K // group), dtype=np.uint8)
    _check(lib().qi4o_quantize(_ptr(w, _dp), N, K, group, bits, _ptr(qw, _u8p), _ptr(s, _u16p),
                               _ptr(z, _u8p)), "quantize")
    return qw, s, z
