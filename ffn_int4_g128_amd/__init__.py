"""Python binding of libqi4: int4 group-quantized linear layer (groups of 128 by
default; 64, multiples of 128, or one group per row; 8-bit codes with the flag
QI4_INT8) and routed MoE expert FFN for AMD MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libqi4.so`` (sources in ``csrc/``, C ABI in ``include/qi4.h``);
PyTorch supplies device memory and the current stream.  If the library is not
built this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqi4.so")

QI4_OK = 0
QI4_F32, QI4_BF16 = 0, 1
QI4_EPI_NONE, QI4_EPI_SILU_MUL = 0, 1
QI4_PACK_GATEUP = 1
QI4_INT8 = 2         # format flag: 8-bit codes (qweight [N][K], zeros 0..255)
GROUP = 128          # default group size; 0 means one group per row


def _code_shape(N: int, K: int, flags: int):
    return (N, K) if flags & QI4_INT8 else (N, K // 2)


def _ngroups(K: int, group: int) -> int:
    return 1 if group == 0 else K // group

_lib = None


class Qi4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().qi4_status_string(status).decode() if _lib is not None else "?"
        super().__init__(f"{what}: status {status} ({msg})")


class _MoeDesc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("inter", ctypes.c_int64), ("top_k", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("has_shared", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


def build(verbose: bool = False) -> str:
    from ffn_int4_g128_amd.build import build as _b
    return _b(verbose=verbose)


def lib():
    """Load libqi4.so (raises FileNotFoundError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        dp = ctypes.POINTER(_MoeDesc)
        sig = {
            "qi4_abi_version": (ci, []),
            "qi4_status_string": (ctypes.c_char_p, [ci]),
            "qi4_packed_bytes": (i64, [i64, i64, ci, ci]),
            "qi4_pack": (ci, [vp, vp, vp, i64, i64, ci, ci, vp, vp]),
            "qi4_unpack": (ci, [vp, i64, i64, ci, ci, vp, vp, vp, vp]),
            "qi4_dequant_f32": (ci, [vp, i64, i64, ci, ci, vp, vp]),
            "qi4_quantize": (ci, [vp, ci, i64, i64, ci, vp, vp, vp, vp]),
            "qi4_quantize_int8": (ci, [vp, ci, i64, i64, ci, vp, vp, vp, vp]),
            "qlinear_int4_g128": (ci, [vp, ci, i64, i64, vp, i64, ci, vp, ci, ci, vp]),
            "qlinear_int4": (ci, [vp, ci, i64, i64, vp, i64, ci, ci, vp, ci, ci, vp]),
            "qlinear_int8": (ci, [vp, ci, i64, i64, vp, i64, ci, ci, vp, ci, ci, vp]),
            "qlinear_w4a8_workspace_bytes": (i64, [i64, i64]),
            "qlinear_w4a8": (ci, [vp, ci, ctypes.c_float, i64, i64, vp, i64, ci, ci, vp, ci, ci,
                                  vp, i64, vp]),
            "moe_route_topk": (ci, [vp, i64, i64, i32, vp, vp, vp]),
            "moe_route_sort": (ci, [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp]),
            "moe_router_topk": (ci, [vp, i64, i64, vp, i64, i32, vp, vp, vp, vp]),
            "moe_sort_tokens": (ci, [vp, i64, i32, i64, vp, vp, vp, vp, vp]),
            "moe_ffn_int4_workspace_bytes": (i64, [dp, i64]),
            "moe_expert_gate_up": (ci, [dp, vp, i64, vp, vp, vp, vp, vp, vp, vp, i64, vp]),
            "moe_expert_down": (ci, [dp, vp, i64, vp, vp, vp, vp, vp, vp, i64, vp]),
            "moe_combine": (ci, [dp, vp, vp, vp, i64, vp, vp]),
            "moe_ffn_int4": (ci, [dp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]),
            "moe_ffn_w4a8_workspace_bytes": (i64, [dp, i64]),
            "moe_ffn_w4a8": (ci, [dp, vp, ctypes.c_float, ctypes.c_float, i64, vp, vp, vp, vp, vp,
                                  vp, vp, vp, vp, i64, vp]),
            "moe_ffn_int4_share": (ci, [dp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                        vp]),
            "moe_ffn_int4_noalloc": (ci, [dp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "qi4_probe_stream_read": (ci, [vp, i64, vp, vp]),
            "qi4_probe_mfma": (ci, [i64, i64, vp, vp]),
            "qi4_probe_mfma_flops": (i64, [i64, i64]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


# declared in include/qi4.h, in header order
EXPORTED = ["qi4_abi_version", "qi4_status_string", "qi4_packed_bytes", "qi4_pack", "qi4_unpack",
            "qi4_dequant_f32", "qi4_quantize", "qi4_quantize_int8", "qlinear_int4_g128",
            "qlinear_int4", "qlinear_int8", "qlinear_w4a8_workspace_bytes", "qlinear_w4a8",
            "moe_route_topk",
            "moe_route_sort", "moe_router_topk", "moe_sort_tokens",
            "moe_ffn_int4_workspace_bytes", "moe_expert_gate_up", "moe_expert_down",
            "moe_combine", "moe_ffn_int4", "moe_ffn_int4_share", "moe_ffn_w4a8_workspace_bytes",
            "moe_ffn_w4a8", "moe_ffn_int4_noalloc",
            # include/qi4_probe.h
            "qi4_probe_stream_read", "qi4_probe_mfma", "qi4_probe_mfma_flops"]

PROBE_READ_SINK_WORDS = 8192

#: bytes of the scratch array moe_ffn_int4_noalloc holds on each GPU
NOALLOC_SCRATCH_BYTES = 48 << 20


def _check(rc: int, what: str):
    if rc != QI4_OK:
        raise Qi4Error(rc, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, what):
    import torch
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    del torch


# ---- format -------------------------------------------------------------------

def packed_bytes(N: int, K: int, flags: int = 0, group: int = GROUP) -> int:
    n = lib().qi4_packed_bytes(N, K, group, flags)
    _check(int(n) if n < 0 else 0, "qi4_packed_bytes")
    return int(n)


def pack(qweight, scales, zeros, N: int, K: int, flags: int = 0, out=None, stream=None,
         group: int = GROUP):
    """Canonical (uint8 [N][K/2] -- [N][K] with QI4_INT8 --, int16/uint16 binary16
    bits [N][K/group], uint8 [N][K/group]) device tensors -> packed uint8 device
    tensor."""
    import torch
    _need(qweight, torch.uint8, "qweight")
    _need(zeros, torch.uint8, "zeros")
    if out is None:
        out = torch.empty(packed_bytes(N, K, flags, group), dtype=torch.uint8,
                          device=qweight.device)
    _check(lib().qi4_pack(_ptr(qweight), _ptr(scales), _ptr(zeros), N, K, group, flags,
                          _ptr(out), _stream(stream)), "qi4_pack")
    return out


def unpack(packed, N: int, K: int, flags: int = 0, stream=None, group: int = GROUP):
    import torch
    dev = packed.device
    ng = _ngroups(K, group)
    qw = torch.empty(_code_shape(N, K, flags), dtype=torch.uint8, device=dev)
    sc = torch.empty((N, ng), dtype=torch.int16, device=dev)
    zr = torch.empty((N, ng), dtype=torch.uint8, device=dev)
    _check(lib().qi4_unpack(_ptr(packed), N, K, group, flags, _ptr(qw), _ptr(sc), _ptr(zr),
                            _stream(stream)), "qi4_unpack")
    return qw, sc, zr


def dequant_f32(packed, N: int, K: int, flags: int = 0, stream=None, group: int = GROUP):
    import torch
    w = torch.empty((N, K), dtype=torch.float32, device=packed.device)
    _check(lib().qi4_dequant_f32(_ptr(packed), N, K, group, flags, _ptr(w), _stream(stream)),
           "qi4_dequant_f32")
    return w


def quantize(w, stream=None, group: int = GROUP, flags: int = 0):
    """float32 or bfloat16 device weights [N][K] -> canonical (qweight uint8 [N][K/2],
    scales int16 binary16 bits [N][K/group], zeros uint8 [N][K/group]) device tensors;
    8-bit codes (qweight [N][K]) with flags QI4_INT8."""
    import torch
    if w.dtype == torch.float32:
        wd = QI4_F32
    elif w.dtype == torch.bfloat16:
        wd = QI4_BF16
    else:
        raise ValueError(f"w must be float32 or bfloat16, got {w.dtype}")
    if not (w.is_cuda and w.is_contiguous() and w.dim() == 2):
        raise ValueError("w must be a contiguous 2-D device tensor")
    N, K = w.shape
    ng = _ngroups(K, group)
    qw = torch.empty(_code_shape(N, K, flags), dtype=torch.uint8, device=w.device)
    sc = torch.empty((N, ng), dtype=torch.int16, device=w.device)
    zr = torch.empty((N, ng), dtype=torch.uint8, device=w.device)
    fn = lib().qi4_quantize_int8 if flags & QI4_INT8 else lib().qi4_quantize
    _check(fn(_ptr(w), wd, N, K, group, _ptr(qw), _ptr(sc), _ptr(zr), _stream(stream)),
           "qi4_quantize")
    return qw, sc, zr


# ---- linear ----------------------------------------------------------------------

def qlinear(x, packed, N: int, flags: int = 0, out_dtype=None, epilogue: int = QI4_EPI_NONE,
            out=None, stream=None, group: int = GROUP):
    """y = epilogue(x . dequant(W)^T); x is bfloat16 or float32 [T][K]."""
    import torch
    if x.dtype == torch.bfloat16:
        xd = QI4_BF16
    elif x.dtype == torch.float32:
        xd = QI4_F32
    else:
        raise ValueError(f"x must be bfloat16 or float32, got {x.dtype}")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    T, K = x.shape
    out_dtype = out_dtype or x.dtype
    n_out = N // 2 if epilogue == QI4_EPI_SILU_MUL else N
    if out is None:
        out = torch.empty((T, n_out), dtype=out_dtype, device=x.device)
    yd = QI4_BF16 if out.dtype == torch.bfloat16 else QI4_F32
    if flags & QI4_INT8:
        _check(lib().qlinear_int8(_ptr(x), xd, T, K, _ptr(packed), N, group, flags, _ptr(out), yd,
                                  epilogue, _stream(stream)), "qlinear_int8")
    elif group == GROUP:
        _check(lib().qlinear_int4_g128(_ptr(x), xd, T, K, _ptr(packed), N, flags, _ptr(out), yd,
                                       epilogue, _stream(stream)), "qlinear_int4_g128")
    else:
        _check(lib().qlinear_int4(_ptr(x), xd, T, K, _ptr(packed), N, group, flags, _ptr(out), yd,
                                  epilogue, _stream(stream)), "qlinear_int4")
    return out


def qlinear_w4a8(x, x_scale: float, packed, N: int, flags: int = 0, out_dtype=None,
                 epilogue: int = QI4_EPI_NONE, out=None, workspace=None, stream=None,
                 group: int = GROUP):
    """W4A8: y = epilogue(x_scale * a . dequant(W)^T) with the int8 activations
    a = clamp(rint(x * float32(1 / x_scale)), -127, 127); x bfloat16 or float32 [T][K]."""
    import torch
    if x.dtype == torch.bfloat16:
        xd = QI4_BF16
    elif x.dtype == torch.float32:
        xd = QI4_F32
    else:
        raise ValueError(f"x must be bfloat16 or float32, got {x.dtype}")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    T, K = x.shape
    out_dtype = out_dtype or x.dtype
    n_out = N // 2 if epilogue == QI4_EPI_SILU_MUL else N
    if out is None:
        out = torch.empty((T, n_out), dtype=out_dtype, device=x.device)
    if workspace is None:
        nb = lib().qlinear_w4a8_workspace_bytes(T, K)
        _check(int(nb) if nb < 0 else 0, "qlinear_w4a8_workspace_bytes")
        workspace = torch.empty(max(int(nb), 1), dtype=torch.uint8, device=x.device)
    yd = QI4_BF16 if out.dtype == torch.bfloat16 else QI4_F32
    _check(lib().qlinear_w4a8(_ptr(x), xd, float(x_scale), T, K, _ptr(packed), N, group, flags,
                              _ptr(out), yd, epilogue, _ptr(workspace), workspace.numel(),
                              _stream(stream)), "qlinear_w4a8")
    return out


# ---- MoE -------------------------------------------------------------------------

@dataclass
class MoeWeights:
    """Packed weights of one MoE layer: routed experts stacked, plus an optional
    shared expert (all device tensors)."""
    E: int
    H: int
    I: int
    w_gate_up: object
    w_down: object
    shared_gate_up: object = None
    shared_down: object = None
    group: int = GROUP
    flags: int = 0       # QI4_INT8: 8-bit experts

    def desc(self, top_k: int) -> _MoeDesc:
        return _MoeDesc(self.E, self.H, self.I, top_k, self.group,
                        1 if self.shared_gate_up is not None else 0, self.flags)


def pack_moe(experts: dict, shared: dict | None, E: int, H: int, I: int, device="cuda",
             stream=None, group: int = GROUP, flags: int = 0) -> MoeWeights:
    """Pack canonical expert weights (numpy or torch; see workloads.moe_experts) expert by
    expert on the device."""
    import numpy as np
    import torch

    def dev(a, dt):
        if isinstance(a, np.ndarray):
            if dt == torch.int16:
                a = a.view(np.int16)
            a = torch.from_numpy(np.ascontiguousarray(a))
        return a.to(device)

    fg, fd = QI4_PACK_GATEUP | flags, flags
    gu_b, dn_b = packed_bytes(2 * I, H, fg, group), packed_bytes(H, I, fd, group)
    w_gu = torch.empty(E * gu_b, dtype=torch.uint8, device=device)
    w_dn = torch.empty(E * dn_b, dtype=torch.uint8, device=device)
    for e in range(E):
        pack(dev(experts["gu_q"][e], torch.uint8), dev(experts["gu_s"][e], torch.int16),
             dev(experts["gu_z"][e], torch.uint8), 2 * I, H, fg,
             out=w_gu[e * gu_b:(e + 1) * gu_b], stream=stream, group=group)
        pack(dev(experts["dn_q"][e], torch.uint8), dev(experts["dn_s"][e], torch.int16),
             dev(experts["dn_z"][e], torch.uint8), H, I, fd,
             out=w_dn[e * dn_b:(e + 1) * dn_b], stream=stream, group=group)
    sgu = sdn = None
    if shared is not None:
        sgu = pack(dev(shared["gu_q"], torch.uint8), dev(shared["gu_s"], torch.int16),
                   dev(shared["gu_z"], torch.uint8), 2 * I, H, fg, stream=stream,
                   group=group)
        sdn = pack(dev(shared["dn_q"], torch.uint8), dev(shared["dn_s"], torch.int16),
                   dev(shared["dn_z"], torch.uint8), H, I, fd, stream=stream, group=group)
    return MoeWeights(E, H, I, w_gu, w_dn, sgu, sdn, group, flags)


def moe_route_topk(logits, top_k: int, stream=None):
    import torch
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    wts = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(wts), _stream(stream)),
           "moe_route_topk")
    return ids, wts


def moe_route_sort(logits, top_k: int, stream=None):
    """Routing and permutation in one call: (ids, weights, sorted_pairs, offsets,
    pair_to_sorted, active)."""
    import torch
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    sp = torch.empty(T * top_k, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    inv = torch.empty(T * top_k, dtype=torch.int32, device=dev)
    act = torch.empty(E + 1, dtype=torch.int32, device=dev)
    _check(lib().moe_route_sort(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(wts), _ptr(sp), _ptr(off),
                                _ptr(inv), _ptr(act), _stream(stream)), "moe_route_sort")
    return ids, wts, sp, off, inv, act


def moe_router_topk(x, w_router, top_k: int, logits=None, stream=None):
    """x bf16 [T][H], w_router bf16 [E][H] -> (logits float32 [T][E], ids int32 [T][k],
    weights float32 [T][k])."""
    import torch
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
    wts = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    _check(lib().moe_router_topk(_ptr(x), T, H, _ptr(w_router), E, top_k, _ptr(logits), _ptr(ids),
                                 _ptr(wts), _stream(stream)), "moe_router_topk")
    return logits, ids, wts


def moe_sort_tokens(ids, E: int, stream=None):
    """Returns (sorted_pairs, expert_offsets, pair_to_sorted, active) int32 device tensors."""
    import torch
    _need(ids, torch.int32, "ids")
    T, k = ids.shape
    dev = ids.device
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    act = torch.empty(E + 1, dtype=torch.int32, device=dev)
    _check(lib().moe_sort_tokens(_ptr(ids), T, k, E, _ptr(sp), _ptr(off), _ptr(inv), _ptr(act),
                                 _stream(stream)), "moe_sort_tokens")
    return sp, off, inv, act


def moe_workspace_bytes(w: MoeWeights, top_k: int, T: int) -> int:
    d = w.desc(top_k)
    n = lib().moe_ffn_int4_workspace_bytes(ctypes.byref(d), T)
    _check(int(n) if n < 0 else 0, "moe_ffn_int4_workspace_bytes")
    return int(n)


def moe_workspace(w: MoeWeights, top_k: int, T: int, device="cuda"):
    import torch
    return torch.empty(moe_workspace_bytes(w, top_k, T), dtype=torch.uint8, device=device)


def moe_ffn(x, w: MoeWeights, top_k: int, logits=None, ids=None, weights=None, workspace=None,
            out=None, return_routing: bool = False, stream=None):
    """out[t] = sum_j p[t][j] * FFN_{ids[t][j]}(x_t) + FFN_shared(x_t); x bf16 [T][H]."""
    import torch
    _need(x, torch.bfloat16, "x")
    T = x.shape[0]
    d = w.desc(top_k)
    if workspace is None:
        workspace = moe_workspace(w, top_k, T, x.device)
    if out is None:
        out = torch.empty((T, w.H), dtype=torch.bfloat16, device=x.device)
    if logits is not None and return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
        weights = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    _check(lib().moe_ffn_int4(ctypes.byref(d), _ptr(x), T, _ptr(logits), _ptr(ids), _ptr(weights),
                              _ptr(w.w_gate_up), _ptr(w.w_down), _ptr(w.shared_gate_up),
                              _ptr(w.shared_down), _ptr(out), _ptr(workspace),
                              workspace.numel(), _stream(stream)), "moe_ffn_int4")
    if return_routing:
        return out, ids, weights
    return out


def moe_ffn_share(x, w: MoeWeights, top_k: int, gpu_experts, logits=None, ids=None,
                  weights=None, workspace=None, out=None, return_routing: bool = False,
                  stream=None):
    """This device's share of the layer: the routed experts with gpu_experts[e]
    nonzero (device uint8 [E]) plus the shared expert if w has one."""
    import torch
    _need(x, torch.bfloat16, "x")
    _need(gpu_experts, torch.uint8, "gpu_experts")
    T = x.shape[0]
    d = w.desc(top_k)
    if workspace is None:
        workspace = moe_workspace(w, top_k, T, x.device)
    if out is None:
        out = torch.empty((T, w.H), dtype=torch.bfloat16, device=x.device)
    if logits is not None and return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
        weights = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    _check(lib().moe_ffn_int4_share(ctypes.byref(d), _ptr(x), T, _ptr(logits), _ptr(ids),
                                    _ptr(weights), _ptr(w.w_gate_up), _ptr(w.w_down),
                                    _ptr(w.shared_gate_up), _ptr(w.shared_down), _ptr(gpu_experts),
                                    _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_ffn_int4_share")
    if return_routing:
        return out, ids, weights
    return out


def moe_ffn_noalloc(x, w: MoeWeights, top_k: int, logits=None, ids=None, weights=None,
                    out=None, return_routing: bool = False, stream=None):
    """moe_ffn through moe_ffn_int4_noalloc: no workspace argument; the library's
    per-GPU scratch array serves instead (calls overlapping on one GPU race)."""
    import torch
    _need(x, torch.bfloat16, "x")
    T = x.shape[0]
    d = w.desc(top_k)
    if out is None:
        out = torch.empty((T, w.H), dtype=torch.bfloat16, device=x.device)
    if logits is not None and return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
        weights = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    _check(lib().moe_ffn_int4_noalloc(ctypes.byref(d), _ptr(x), T, _ptr(logits), _ptr(ids),
                                      _ptr(weights), _ptr(w.w_gate_up), _ptr(w.w_down),
                                      _ptr(w.shared_gate_up), _ptr(w.shared_down), _ptr(out),
                                      _stream(stream)), "moe_ffn_int4_noalloc")
    if return_routing:
        return out, ids, weights
    return out


def moe_ffn_w4a8(x, w: MoeWeights, top_k: int, x_scale: float, h_scale: float, logits=None,
                 ids=None, weights=None, workspace=None, out=None, return_routing: bool = False,
                 stream=None):
    """W4A8 MoE layer: moe_ffn with int8 activations (static scales x_scale for x
    and h_scale for h = SiLU(g) * u); x bf16 [T][H]."""
    import torch
    _need(x, torch.bfloat16, "x")
    T = x.shape[0]
    d = w.desc(top_k)
    if workspace is None:
        nb = lib().moe_ffn_w4a8_workspace_bytes(ctypes.byref(d), T)
        _check(int(nb) if nb < 0 else 0, "moe_ffn_w4a8_workspace_bytes")
        workspace = torch.empty(max(int(nb), 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, w.H), dtype=torch.bfloat16, device=x.device)
    if logits is not None and return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
        weights = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    _check(lib().moe_ffn_w4a8(ctypes.byref(d), _ptr(x), float(x_scale), float(h_scale), T,
                              _ptr(logits), _ptr(ids), _ptr(weights), _ptr(w.w_gate_up),
                              _ptr(w.w_down), _ptr(w.shared_gate_up), _ptr(w.shared_down),
                              _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_ffn_w4a8")
    if return_routing:
        return out, ids, weights
    return out


def moe_gate_up(x, w: MoeWeights, top_k: int, sorted_pairs, offsets, active, h=None,
                workspace=None, stream=None):
    import torch
    T = x.shape[0]
    R = T * top_k + (T if w.shared_gate_up is not None else 0)
    if h is None:
        h = torch.empty((R, 2, w.I), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = moe_workspace(w, top_k, T, x.device)
    d = w.desc(top_k)
    _check(lib().moe_expert_gate_up(ctypes.byref(d), _ptr(x), T, _ptr(sorted_pairs), _ptr(offsets),
                                    _ptr(active), _ptr(w.w_gate_up), _ptr(w.shared_gate_up),
                                    _ptr(h), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_expert_gate_up")
    return h


def moe_down(h, T: int, w: MoeWeights, top_k: int, offsets, active, y=None, workspace=None,
             stream=None):
    import torch
    R = T * top_k + (T if w.shared_down is not None else 0)
    if y is None:
        y = torch.empty((R, w.H), dtype=torch.float32, device=h.device)
    if workspace is None:
        workspace = moe_workspace(w, top_k, T, h.device)
    d = w.desc(top_k)
    _check(lib().moe_expert_down(ctypes.byref(d), _ptr(h), T, _ptr(offsets), _ptr(active),
                                 _ptr(w.w_down), _ptr(w.shared_down), _ptr(y), _ptr(workspace),
                                 workspace.numel(), _stream(stream)), "moe_expert_down")
    return y


def moe_combine(y, weights, pair_to_sorted, T: int, w: MoeWeights, top_k: int, out=None,
                stream=None):
    import torch
    if out is None:
        out = torch.empty((T, w.H), dtype=torch.bfloat16, device=y.device)
    d = w.desc(top_k)
    _check(lib().moe_combine(ctypes.byref(d), _ptr(y), _ptr(weights), _ptr(pair_to_sorted), T,
                             _ptr(out), _stream(stream)), "moe_combine")
    return out


# ---- measurement probes (include/qi4_probe.h) -----------------------------------

def probe_stream_read(buf, sink=None, stream=None):
    """Read every byte of the device tensor `buf` once (qi4_probe_stream_read)."""
    import torch
    if sink is None:
        sink = torch.empty(PROBE_READ_SINK_WORDS, dtype=torch.int32, device=buf.device)
    _check(lib().qi4_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                       _stream(stream)), "qi4_probe_stream_read")
    return sink


def probe_mfma(iters: int, workgroups: int, sink=None, stream=None) -> int:
    """Run the matrix-core probe; returns the flops the launch performs."""
    import torch
    if sink is None:
        sink = torch.empty(1, dtype=torch.float32, device="cuda")
    _check(lib().qi4_probe_mfma(iters, workgroups, _ptr(sink), _stream(stream)), "qi4_probe_mfma")
    return int(lib().qi4_probe_mfma_flops(iters, workgroups))
