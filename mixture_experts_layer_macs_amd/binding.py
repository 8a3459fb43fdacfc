"""Python binding of the C ABI in include/moe_macs.h (ctypes).

Argument marshalling only: every function checks that its tensors live on
the GPU with the expected dtype and layout, passes raw device pointers and
the current HIP stream to the library, and raises on a nonzero status.  All
computation happens in the HIP kernels of libmoe_macs.so; there is no CPU
fallback, and importing this module fails when the library is not built.

torch is used for device memory and streams only.  It must be imported
before the library is loaded, so that the library binds to the same HIP
runtime (same soname) as torch.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_macs.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUP, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4
FFN_NOALLOC_MAX_BYTES = 32 << 20
MOE_F32, MOE_BF16, MOE_BF16_PANELS = 0, 1, 2
FLAG_SERE, FLAG_MACS, FLAG_DROP = 1, 2, 4
WEIGHT_ONE = 65536

_ERR = {MOE_EINVAL: "MOE_EINVAL (bad argument)",
        MOE_EUNSUP: "MOE_EUNSUP (unsupported type or shape)",
        MOE_EHIP: "MOE_EHIP (HIP launch error)",
        MOE_ESCRATCH: "MOE_ESCRATCH (larger than the fixed no-allocation buffer)"}

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_D = ctypes.c_double
_F = ctypes.c_float

_SIGS = {
    "moe_route": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_router_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "moe_similarity_workspace_size": (_SZ, [_I, ctypes.c_longlong, _I]),
    "moe_expert_similarity": (_I, [_P, _I, ctypes.c_longlong, _I, _P, _P, _SZ, _P]),
    "moe_router_topk": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                             _P, _SZ, _P]),
    "moe_sere_reroute": (_I, [_P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P]),
    "moe_capacity_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_capacity_assign": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                 _D, _D, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_dispatch_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_dispatch": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_routing_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "moe_entropy_workspace_size": (_SZ, [_I]),
    "moe_entropy_weights": (_I, [_P, _P, _I, _I, _I, _F, _F, _P, _P, _P, _SZ, _P]),
    "moe_routing_fused": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F,
                               _I, _D, _D, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_ffn_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_expert_ffn": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P,
                            _P, _SZ, _P]),
    "moe_ffn_combine_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_expert_ffn_combine": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I,
                                    _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "moe_ffn_down_combine": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                  _I, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                    _P, _P]),
    "moe_ffn_gate_up": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_ffn_down": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_pack_weights": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() "
            "(or python -m mixture_experts_layer_macs_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


# ------------------------------------------------------------------ helpers
def _check(rc: int, name: str):
    if rc != MOE_OK:
        raise RuntimeError(f"{name} failed: {_ERR.get(rc, rc)}")


def _dev(t: torch.Tensor, dtype, name: str, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype not in (
            dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    return t.data_ptr()


def _opt(t, dtype, name, shape=None):
    return None if t is None else _dev(t, dtype, name, shape)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _elem(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return MOE_BF16
    if dtype == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported element type {dtype}")


def _ffn_format(dtype: torch.dtype, panels: bool) -> int:
    """Format code of the expert FFN calls: panels selects the packed
    weights of moe_pack_weights (bf16 only)."""
    if not panels:
        return _elem(dtype)
    if dtype != torch.bfloat16:
        raise ValueError("packed (panel) weights are bf16 only")
    return MOE_BF16_PANELS


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ---------------------------------------------------------------- the ABI
def moe_route(logits, k, R, topk_ids=None, topk_gates=None, fallback_ids=None):
    T, N = logits.shape
    topk_ids = _empty((T, k), torch.int32, logits) if topk_ids is None else topk_ids
    topk_gates = _empty((T, k), torch.float32, logits) if topk_gates is None else topk_gates
    if fallback_ids is None:
        fallback_ids = _empty((T, R), torch.int32, logits)
    rc = _lib.moe_route(_dev(logits, torch.float32, "logits"), T, N, k, R,
                        _dev(topk_ids, torch.int32, "topk_ids", (T, k)),
                        _dev(topk_gates, torch.float32, "topk_gates", (T, k)),
                        _dev(fallback_ids, torch.int32, "fallback_ids", (T, R))
                        if R > 0 else None,
                        _stream())
    _check(rc, "moe_route")
    return topk_ids, topk_gates, fallback_ids


def moe_router_workspace_size(T, N, H, dtype) -> int:
    return int(_lib.moe_router_workspace_size(T, N, H, _elem(dtype)))


def moe_router_topk(x, w_gate, k, R, workspace, logits=None, topk_ids=None,
                    topk_gates=None, fallback_ids=None, want_logits=True):
    """Router scores x W_g^T and the route step over them, one launch.
    Returns (logits or None, topk_ids, topk_gates, fallback_ids)."""
    T, H = x.shape
    N = w_gate.shape[0]
    if logits is None and want_logits:
        logits = _empty((T, N), torch.float32, x)
    topk_ids = _empty((T, k), torch.int32, x) if topk_ids is None else topk_ids
    topk_gates = _empty((T, k), torch.float32, x) if topk_gates is None else topk_gates
    if fallback_ids is None:
        fallback_ids = _empty((T, R), torch.int32, x)
    rc = _lib.moe_router_topk(
        _dev(x, x.dtype, "x"), _dev(w_gate, x.dtype, "w_gate", (N, H)),
        T, N, H, k, R, _elem(x.dtype),
        _opt(logits, torch.float32, "logits", (T, N)),
        _dev(topk_ids, torch.int32, "topk_ids", (T, k)),
        _dev(topk_gates, torch.float32, "topk_gates", (T, k)),
        _dev(fallback_ids, torch.int32, "fallback_ids", (T, R)) if R > 0 else None,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_router_topk")
    return logits, topk_ids, topk_gates, fallback_ids


def moe_similarity_workspace_size(N, D, dtype) -> int:
    return int(_lib.moe_similarity_workspace_size(N, D, _elem(dtype)))


def moe_expert_similarity(acts, workspace, sim=None):
    """Frobenius similarity of the N rows of acts [N, ...] (each row one
    expert's flattened calibration activations); returns f32 [N, N]."""
    N = acts.shape[0]
    D = acts.numel() // N
    if not acts.is_contiguous():
        raise ValueError("acts must be contiguous")
    sim = _empty((N, N), torch.float32, acts) if sim is None else sim
    rc = _lib.moe_expert_similarity(
        _dev(acts, acts.dtype, "acts"), N, D, _elem(acts.dtype),
        _dev(sim, torch.float32, "sim", (N, N)),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_expert_similarity")
    return sim


def moe_sere_reroute(topk_ids, N, kprime, rho, sim, prot, slot_expert=None,
                     flags=None):
    T, k = topk_ids.shape
    slot_expert = _empty((T, k), torch.int32, topk_ids) if slot_expert is None else slot_expert
    flags = _empty((T, k), torch.uint8, topk_ids) if flags is None else flags
    rc = _lib.moe_sere_reroute(
        _dev(topk_ids, torch.int32, "topk_ids"), T, N, k, kprime, float(rho),
        _dev(sim, torch.float32, "sim", (N, N)),
        _dev(prot, torch.uint8, "prot", (N, N)),
        _dev(slot_expert, torch.int32, "slot_expert", (T, k)),
        _dev(flags, torch.uint8, "flags", (T, k)), _stream())
    _check(rc, "moe_sere_reroute")
    return slot_expert, flags


def moe_capacity_workspace_size(T, N, k) -> int:
    return int(_lib.moe_capacity_workspace_size(T, N, k))


def moe_dispatch_workspace_size(T, N, k) -> int:
    return int(_lib.moe_dispatch_workspace_size(T, N, k))


def moe_routing_workspace_size(T, N, k, R) -> int:
    """Workspace bytes of moe_routing_fused; 0 = shape not covered by the
    fused launch (use the separate calls)."""
    return int(_lib.moe_routing_workspace_size(T, N, k, R))


def moe_entropy_workspace_size(T) -> int:
    return int(_lib.moe_entropy_workspace_size(T))


def moe_entropy_weights(x, is_visual, delta, eps, workspace, entropy_w=None,
                        entropy=None):
    """Per-token semantic weights (and entropies) from the token features."""
    T, H = x.shape
    if entropy_w is None:
        entropy_w = _empty((T,), torch.float32, x)
    rc = _lib.moe_entropy_weights(
        _dev(x, x.dtype, "x"), _dev(is_visual, torch.uint8, "is_visual", (T,)),
        T, H, _elem(x.dtype), float(delta), float(eps),
        _dev(entropy_w, torch.float32, "entropy_w", (T,)),
        _opt(entropy, torch.float32, "entropy", (T,)),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_entropy_weights")
    return entropy_w


def moe_ffn_workspace_size(T, N, k, H, I, dtype) -> int:
    return int(_lib.moe_ffn_workspace_size(T, N, k, H, I, _elem(dtype)))


def moe_ffn_combine_workspace_size(T, N, k, H, I, dtype) -> int:
    return int(_lib.moe_ffn_combine_workspace_size(T, N, k, H, I, _elem(dtype)))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled workspace (the control words must start at zero)."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def moe_capacity_assign(topk_ids, slot_in, fallback_ids, is_visual, entropy_w,
                        modality, N, R, group, gamma, lam, workspace,
                        out=None):
    T, k = topk_ids.shape
    if out is None:
        dev = topk_ids
        out = dict(slot_out=_empty((T, k), torch.int32, dev),
                   flags=_empty((T, k), torch.uint8, dev),
                   load_q=_empty((N,), torch.int64, dev),
                   cap_q=_empty((N,), torch.int64, dev),
                   stats=_empty((4,), torch.int64, dev),
                   r_v=_empty((1,), torch.float64, dev))
    rc = _lib.moe_capacity_assign(
        _dev(topk_ids, torch.int32, "topk_ids"),
        _dev(slot_in, torch.int32, "slot_in", (T, k)),
        _dev(fallback_ids, torch.int32, "fallback_ids", (T, R)) if R > 0 else None,
        _dev(is_visual, torch.uint8, "is_visual", (T,)),
        _dev(entropy_w, torch.float32, "entropy_w", (T,)),
        _dev(modality, torch.int8, "modality", (N,)),
        T, N, k, R, group, float(gamma), float(lam),
        _dev(out["slot_out"], torch.int32, "slot_out", (T, k)),
        _dev(out["flags"], torch.uint8, "flags", (T, k)),
        _dev(out["load_q"], torch.int64, "load_q", (N,)),
        _dev(out["cap_q"], torch.int64, "cap_q", (N,)),
        _dev(out["stats"], torch.int64, "stats", (4,)),
        _dev(out["r_v"], torch.float64, "r_v", (1,)),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_capacity_assign")
    return out


def moe_dispatch(slot_expert, N, workspace, out=None):
    T, k = slot_expert.shape
    if out is None:
        dev = slot_expert
        out = dict(expert_offsets=_empty((N + 1,), torch.int32, dev),
                   row_token=_empty((T * k,), torch.int32, dev),
                   row_slot=_empty((T * k,), torch.int32, dev),
                   slot_row=_empty((T, k), torch.int32, dev))
    rc = _lib.moe_dispatch(
        _dev(slot_expert, torch.int32, "slot_expert"), T, N, k,
        _dev(out["expert_offsets"], torch.int32, "expert_offsets", (N + 1,)),
        _dev(out["row_token"], torch.int32, "row_token", (T * k,)),
        _dev(out["row_slot"], torch.int32, "row_slot", (T * k,)),
        _dev(out["slot_row"], torch.int32, "slot_row", (T, k)),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_dispatch")
    return out


def moe_routing_fused(logits, is_visual, entropy_w, modality, sim, prot, k, R,
                      kprime, rho, group, gamma, lam, workspace, topk_ids,
                      topk_gates, fallback_ids, slot_sere, cap, disp):
    """Route, SERE, capacity and dispatch in one launch; fills the given
    buffers exactly as the four separate calls would."""
    T, N = logits.shape
    rc = _lib.moe_routing_fused(
        _dev(logits, torch.float32, "logits"),
        _dev(is_visual, torch.uint8, "is_visual", (T,)),
        _dev(entropy_w, torch.float32, "entropy_w", (T,)),
        _dev(modality, torch.int8, "modality", (N,)),
        _opt(sim, torch.float32, "sim", (N, N)) if kprime else None,
        _opt(prot, torch.uint8, "prot", (N, N)) if kprime else None,
        T, N, k, R, kprime, float(rho), group, float(gamma), float(lam),
        _dev(topk_ids, torch.int32, "topk_ids", (T, k)),
        _dev(topk_gates, torch.float32, "topk_gates", (T, k)),
        _dev(fallback_ids, torch.int32, "fallback_ids", (T, R)) if R > 0 else None,
        _dev(slot_sere, torch.int32, "slot_sere", (T, k)) if kprime else None,
        _dev(cap["slot_out"], torch.int32, "slot_out", (T, k)),
        _dev(cap["flags"], torch.uint8, "flags", (T, k)),
        _dev(cap["load_q"], torch.int64, "load_q", (N,)),
        _dev(cap["cap_q"], torch.int64, "cap_q", (N,)),
        _dev(cap["stats"], torch.int64, "stats", (4,)),
        _dev(cap["r_v"], torch.float64, "r_v", (1,)),
        _dev(disp["expert_offsets"], torch.int32, "expert_offsets", (N + 1,)),
        _dev(disp["row_token"], torch.int32, "row_token", (T * k,)),
        _dev(disp["row_slot"], torch.int32, "row_slot", (T * k,)),
        _dev(disp["slot_row"], torch.int32, "slot_row", (T, k)),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_routing_fused")


def moe_pack_weights(w13=None, w2=None, w13_panels=None, w2_panels=None):
    """Copies of w13 [N,2I,H] and/or w2 [N,H,I] (bf16) in the panel layout
    that the expert FFN calls read with panels=True.  The packed tensors keep
    the shapes of the originals; only the order of their elements differs."""
    if w13 is None and w2 is None:
        raise ValueError("nothing to pack")
    if w13 is not None:
        N, I2, H = w13.shape
        I = I2 // 2
    else:
        N, H, I = w2.shape
    if w13 is not None and w2 is not None and tuple(w2.shape) != (N, H, I):
        raise ValueError("w13 and w2 shapes do not match")
    ref = w13 if w13 is not None else w2
    if w13 is not None and w13_panels is None:
        w13_panels = torch.empty_like(w13)
    if w2 is not None and w2_panels is None:
        w2_panels = torch.empty_like(w2)
    rc = _lib.moe_pack_weights(
        _opt(w13, torch.bfloat16, "w13", (N, 2 * I, H)),
        _opt(w2, torch.bfloat16, "w2", (N, H, I)), N, H, I, _elem(ref.dtype),
        _opt(w13_panels if w13 is not None else None, torch.bfloat16, "w13_panels",
             (N, 2 * I, H)),
        _opt(w2_panels if w2 is not None else None, torch.bfloat16, "w2_panels",
             (N, H, I)), _stream())
    _check(rc, "moe_pack_weights")
    return w13_panels, w2_panels


def moe_expert_ffn(x, row_token, expert_offsets, w13, w2, k, workspace,
                   out_rows=None, panels=False):
    T, H = x.shape
    N, I2, H2 = w13.shape
    I = I2 // 2
    if H2 != H or tuple(w2.shape) != (N, H, I):
        raise ValueError("expert weight shapes do not match x")
    dt = _ffn_format(x.dtype, panels)
    if out_rows is None:
        out_rows = _empty((T * k, H), x.dtype, x)
    rc = _lib.moe_expert_ffn(
        _dev(x, x.dtype, "x"), _dev(row_token, torch.int32, "row_token", (T * k,)),
        _dev(expert_offsets, torch.int32, "expert_offsets", (N + 1,)),
        _dev(w13, x.dtype, "w13"), _dev(w2, x.dtype, "w2"),
        T, N, k, H, I, dt, _dev(out_rows, x.dtype, "out_rows", (T * k, H)),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_expert_ffn")
    return out_rows


def moe_expert_ffn_combine(x, row_token, expert_offsets, w13, w2, slot_row,
                           topk_gates, k, workspace, out_rows=None, y=None,
                           panels=False):
    """moe_expert_ffn then moe_combine in one call (the combine folded into
    the down GEMV of decode batches on packed weights).  The workspace's
    ticket words start at zero (new_workspace allocates it zeroed)."""
    T, H = x.shape
    N, I2, H2 = w13.shape
    I = I2 // 2
    if H2 != H or tuple(w2.shape) != (N, H, I):
        raise ValueError("expert weight shapes do not match x")
    dt = _ffn_format(x.dtype, panels)
    if out_rows is None:
        out_rows = _empty((T * k, H), x.dtype, x)
    if y is None:
        y = _empty((T, H), x.dtype, x)
    rc = _lib.moe_expert_ffn_combine(
        _dev(x, x.dtype, "x"), _dev(row_token, torch.int32, "row_token", (T * k,)),
        _dev(expert_offsets, torch.int32, "expert_offsets", (N + 1,)),
        _dev(w13, x.dtype, "w13"), _dev(w2, x.dtype, "w2"),
        _dev(slot_row, torch.int32, "slot_row", (T, k)),
        _dev(topk_gates, torch.float32, "topk_gates", (T, k)),
        T, N, k, H, I, dt, _dev(out_rows, x.dtype, "out_rows", (T * k, H)),
        _dev(y, x.dtype, "y", (T, H)),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_expert_ffn_combine")
    return y


def moe_ffn_down_combine(h, row_token, expert_offsets, w2, slot_row, topk_gates,
                         T, k, workspace, out_rows, y, panels=False):
    """Second half of moe_expert_ffn_combine: the down GEMM and the combine
    (folded in where moe_expert_ffn_combine folds it), h given."""
    N, H, I = w2.shape
    dt = _ffn_format(h.dtype, panels)
    rc = _lib.moe_ffn_down_combine(
        _dev(h, h.dtype, "h", (T * k, I)),
        _dev(row_token, torch.int32, "row_token", (T * k,)),
        _dev(expert_offsets, torch.int32, "expert_offsets", (N + 1,)),
        _dev(w2, h.dtype, "w2"),
        _dev(slot_row, torch.int32, "slot_row", (T, k)),
        _dev(topk_gates, torch.float32, "topk_gates", (T, k)),
        T, N, k, H, I, dt, _dev(out_rows, h.dtype, "out_rows", (T * k, H)),
        _dev(y, h.dtype, "y", (T, H)),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _check(rc, "moe_ffn_down_combine")
    return y


def moe_expert_ffn_noalloc(x, row_token, expert_offsets, w13, w2, k,
                           out_rows=None, panels=False):
    """moe_expert_ffn with h in the library's fixed device buffer (no
    workspace; at most FFN_NOALLOC_MAX_BYTES of h)."""
    T, H = x.shape
    N, I2, H2 = w13.shape
    I = I2 // 2
    if H2 != H or tuple(w2.shape) != (N, H, I):
        raise ValueError("expert weight shapes do not match x")
    if out_rows is None:
        out_rows = _empty((T * k, H), x.dtype, x)
    rc = _lib.moe_expert_ffn_noalloc(
        _dev(x, x.dtype, "x"), _dev(row_token, torch.int32, "row_token", (T * k,)),
        _dev(expert_offsets, torch.int32, "expert_offsets", (N + 1,)),
        _dev(w13, x.dtype, "w13"), _dev(w2, x.dtype, "w2"),
        T, N, k, H, I, _ffn_format(x.dtype, panels),
        _dev(out_rows, x.dtype, "out_rows", (T * k, H)), _stream())
    _check(rc, "moe_expert_ffn_noalloc")
    return out_rows


def moe_ffn_gate_up(x, row_token, expert_offsets, w13, k, h, panels=False):
    T, H = x.shape
    N, I2, _ = w13.shape
    I = I2 // 2
    rc = _lib.moe_ffn_gate_up(
        _dev(x, x.dtype, "x"), _dev(row_token, torch.int32, "row_token", (T * k,)),
        _dev(expert_offsets, torch.int32, "expert_offsets", (N + 1,)),
        _dev(w13, x.dtype, "w13", (N, 2 * I, H)), T, N, k, H, I,
        _ffn_format(x.dtype, panels),
        _dev(h, x.dtype, "h", (T * k, I)), _stream())
    _check(rc, "moe_ffn_gate_up")
    return h


def moe_ffn_down(h, expert_offsets, w2, T, k, out_rows, panels=False):
    N, H, I = w2.shape
    rc = _lib.moe_ffn_down(
        _dev(h, h.dtype, "h", (T * k, I)),
        _dev(expert_offsets, torch.int32, "expert_offsets", (N + 1,)),
        _dev(w2, h.dtype, "w2"), T, N, k, H, I, _ffn_format(h.dtype, panels),
        _dev(out_rows, h.dtype, "out_rows", (T * k, H)), _stream())
    _check(rc, "moe_ffn_down")
    return out_rows


def moe_combine(out_rows, slot_row, topk_gates, y=None):
    T, k = slot_row.shape
    H = out_rows.shape[1]
    if y is None:
        y = _empty((T, H), out_rows.dtype, out_rows)
    rc = _lib.moe_combine(
        _dev(out_rows, out_rows.dtype, "out_rows"),
        _dev(slot_row, torch.int32, "slot_row", (T, k)),
        _dev(topk_gates, torch.float32, "topk_gates", (T, k)),
        T, k, H, _elem(out_rows.dtype),
        _dev(y, out_rows.dtype, "y", (T, H)), _stream())
    _check(rc, "moe_combine")
    return y


# ------------------------------------------------------------- one layer
class Layer:
    """Preallocated buffers for one layer shape; ``forward`` enqueues the
    calls on the current stream (route -> SERE -> capacity -> dispatch ->
    expert FFN and combine in one call) with no host synchronisation.  Decode-sized
    batches route with the single fused launch unless ``fused=False``."""

    def __init__(self, T, H, N, k, I, R, dtype, device="cuda"):
        self.T, self.H, self.N, self.k, self.I, self.R = T, H, N, k, I, R
        self.dtype = dtype
        dev = torch.device(device)
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.topk_ids = e((T, k), torch.int32)
        self.topk_gates = e((T, k), torch.float32)
        self.fallback_ids = e((T, R), torch.int32)
        self.slot_sere = e((T, k), torch.int32)
        self.flags_sere = e((T, k), torch.uint8)
        self.cap = dict(slot_out=e((T, k), torch.int32),
                        flags=e((T, k), torch.uint8),
                        load_q=e((N,), torch.int64), cap_q=e((N,), torch.int64),
                        stats=e((4,), torch.int64), r_v=e((1,), torch.float64))
        self.disp = dict(expert_offsets=e((N + 1,), torch.int32),
                         row_token=e((T * k,), torch.int32),
                         row_slot=e((T * k,), torch.int32),
                         slot_row=e((T, k), torch.int32))
        self.out_rows = e((T * k, H), dtype)
        self.y = e((T, H), dtype)
        self.ws_cap = new_workspace(moe_capacity_workspace_size(T, N, k), dev)
        self.ws_disp = new_workspace(moe_dispatch_workspace_size(T, N, k), dev)
        self.ws_ffn = new_workspace(moe_ffn_combine_workspace_size(T, N, k, H, I, dtype), dev)
        ws_route = moe_routing_workspace_size(T, N, k, R)
        self.can_fuse = ws_route > 0
        self.ws_route = new_workspace(ws_route, dev) if self.can_fuse else None

    def routing(self, logits, is_visual, entropy_w, modality, sim=None,
                prot=None, kprime=0, rho=0.5, gamma=math.inf, lam=1.0,
                group=None, fused=None):
        """Route, re-route, assign capacity and dispatch (fused launch or the
        four separate calls)."""
        N, k, R = self.N, self.k, self.R
        group = N if group is None else group
        if fused is None:
            fused = self.can_fuse
        if fused:
            moe_routing_fused(logits, is_visual, entropy_w, modality, sim, prot,
                              k, R, kprime, rho, group, gamma, lam,
                              self.ws_route, self.topk_ids, self.topk_gates,
                              self.fallback_ids, self.slot_sere, self.cap,
                              self.disp)
            return
        moe_route(logits, k, R, self.topk_ids, self.topk_gates, self.fallback_ids)
        slot_in = self.topk_ids
        if kprime:
            moe_sere_reroute(self.topk_ids, N, kprime, rho, sim, prot,
                             self.slot_sere, self.flags_sere)
            slot_in = self.slot_sere
        moe_capacity_assign(self.topk_ids, slot_in, self.fallback_ids,
                            is_visual, entropy_w, modality, N, R, group, gamma,
                            lam, self.ws_cap, self.cap)
        moe_dispatch(self.cap["slot_out"], N, self.ws_disp, self.disp)

    def forward(self, logits, x, w13, w2, is_visual, entropy_w, modality,
                sim=None, prot=None, kprime=0, rho=0.5, gamma=math.inf,
                lam=1.0, group=None, fused=None, panels=False):
        """panels: w13 and w2 are the packed copies of moe_pack_weights."""
        k = self.k
        self.routing(logits, is_visual, entropy_w, modality, sim, prot, kprime,
                     rho, gamma, lam, group, fused)
        moe_expert_ffn_combine(x, self.disp["row_token"], self.disp["expert_offsets"],
                               w13, w2, self.disp["slot_row"], self.topk_gates, k,
                               self.ws_ffn, self.out_rows, self.y, panels=panels)
        return self.y
