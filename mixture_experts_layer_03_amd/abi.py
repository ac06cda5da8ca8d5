"""Thin Python binding of libmoe's C ABI (include/moe.h).

Argument marshalling only: every function here takes torch tensors that
already live on the current HIP device, checks nothing beyond what ctypes
needs, passes raw pointers and sizes to the function of the same name in
libmoe.so, and raises MoeError on a non-zero status.  All arithmetic runs in
the library's kernels.  The library must have been built
(``python -m mixture_experts_layer_03_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

# the in-tree build; MOE_LIBRARY names another build of the same sources
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_F32 = 0
MOE_BF16 = 1

_c_void_p = ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t

# name -> (restype, argtypes)
_SIGS = {
    "moe_version": (_i32, []),
    "moe_strerror": (ctypes.c_char_p, [_i32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_router_logits": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32, _i32,
                                 _c_void_p, _c_void_p]),
    "moe_route": (_i32, [_c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "moe_permute_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_permute": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _i32,
                           _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _c_void_p, _sz, _c_void_p]),
    "moe_grouped_ffn_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32]),
    "moe_grouped_ffn_fwd": (_i32, [_c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _c_void_p,
                                   _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _sz, _c_void_p]),
    "moe_grouped_ffn_fwd_noalloc": (_i32, [_c_void_p, _c_void_p, _i32, _i64, _i32, _i32,
                                           _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p,
                                           _c_void_p, _c_void_p, _c_void_p]),
    "moe_grouped_ffn_bwd": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32,
                                   _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _sz, _c_void_p]),
    "moe_combine": (_i32, [_c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _c_void_p, _c_void_p]),
    "moe_combine_bwd": (_i32, [_c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _c_void_p, _c_void_p]),
    "moe_permute_bwd": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _c_void_p,
                               _c_void_p]),
    "moe_permute_bwd_router": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64,
                                      _i32, _i32, _i32, _c_void_p, _c_void_p]),
    "moe_route_bwd": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32,
                             _c_void_p, _c_void_p, _c_void_p]),
    "moe_router_logits_bwd_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_router_logits_bwd": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32, _i32,
                                     _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_route_biased": (_i32, [_c_void_p, _c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p,
                                _c_void_p]),
    "moe_expert_load_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_expert_load": (_i32, [_c_void_p, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p, _sz,
                               _c_void_p]),
    "moe_bias_update": (_i32, [_c_void_p, _i64, _i32, _i32, ctypes.c_float, _c_void_p,
                               _c_void_p]),
    "moe_aux_loss_workspace_size": (_sz, [_i64, _i32]),
    "moe_aux_loss": (_i32, [_c_void_p, _c_void_p, _i64, _i64, _i32, _i32, ctypes.c_float,
                            _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_grouped_ffn_lora_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32]),
    "moe_grouped_ffn_fwd_lora": (_i32, [_c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                        _c_void_p, _i32, ctypes.c_float, _i32, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                        _sz, _c_void_p]),
    "moe_grouped_ffn_bwd_lora": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64,
                                        _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                        ctypes.c_float, _c_void_p, _c_void_p, _i32, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                        _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_grouped_ffn_lora_bwd_saved": (_i32, [_c_void_p, _sz, _i64, _i32, _i32, _i32, _i32,
                                              ctypes.POINTER(_c_void_p), ctypes.POINTER(_c_void_p),
                                              ctypes.POINTER(_c_void_p)]),
    "moe_grouped_ffn_fwd_gather": (_i32, [_c_void_p, _i64, _c_void_p, _i32, _c_void_p, _i32,
                                          _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                          _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_grouped_ffn_bwd_gather": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                                          _c_void_p, _i32, _c_void_p,
                                          _c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p,
                                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                          _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_timing_enable": (_i32, [_i32]),
    "moe_timing_reset": (_i32, []),
    "moe_timing_query": (_i32, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_int64)]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed (status %d): %s" % (fn, status, msg))
        self.status = status


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built (%s); run "
                               "`python -m mixture_experts_layer_03_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc, (lib().moe_last_error() or b"").decode())


# ---------------------------------------------------------------- entry points

def moe_router_logits(x, w_r, bias, logit_add, logits, stream=None):
    T, d = x.shape
    E = w_r.shape[0]
    _check("moe_router_logits", lib().moe_router_logits(
        _p(x), _p(w_r), _p(bias), _p(logit_add), _dtype_code(x), T, d, E, _p(logits),
        _stream(stream)))


def moe_route(logits, k, topk_idx, topk_w, stream=None):
    T, E = logits.shape
    _check("moe_route", lib().moe_route(_p(logits), T, E, k, _p(topk_idx), _p(topk_w),
                                        _stream(stream)))


def moe_permute_workspace_size(T, E, k) -> int:
    return int(lib().moe_permute_workspace_size(T, E, k))


def moe_permute(x, topk_idx, topk_w, T, d, E, k, counts, offsets, slot_to_row, row_to_slot,
                x_perm, w_perm, ws, dtype=None, stream=None):
    dt = _dtype_code(x) if x is not None else (MOE_BF16 if dtype is None else dtype)
    _check("moe_permute", lib().moe_permute(
        _p(x), _p(topk_idx), _p(topk_w), dt, T, d, E, k, _p(counts), _p(offsets),
        _p(slot_to_row), _p(row_to_slot), _p(x_perm), _p(w_perm), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn_workspace_size(R, E, d, f, dtype) -> int:
    return int(lib().moe_grouped_ffn_workspace_size(R, E, d, f, dtype))


def moe_grouped_ffn_fwd(x_perm, offsets, E, w_gu, w_down, row_scale, gu, h, y_perm, ws,
                        stream=None):
    R, d = x_perm.shape
    f = w_down.shape[2]
    _check("moe_grouped_ffn_fwd", lib().moe_grouped_ffn_fwd(
        _p(x_perm), _p(offsets), E, R, d, f, _p(w_gu), _p(w_down), _p(row_scale),
        _dtype_code(x_perm), _p(gu), _p(h), _p(y_perm), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn_fwd_noalloc(x_perm, offsets, E, w_gu, w_down, row_scale, gu, h, y_perm,
                                stream=None):
    R, d = x_perm.shape
    f = w_down.shape[2]
    _check("moe_grouped_ffn_fwd_noalloc", lib().moe_grouped_ffn_fwd_noalloc(
        _p(x_perm), _p(offsets), E, R, d, f, _p(w_gu), _p(w_down), _p(row_scale),
        _dtype_code(x_perm), _p(gu), _p(h), _p(y_perm), _stream(stream)))


def moe_grouped_ffn_bwd(x_perm, gu, h, offsets, E, w_gu, w_down, row_scale, dy_perm, dgu,
                        dx_perm, dw_gu, dw_down, d_row_scale, ws, stream=None):
    R, d = x_perm.shape
    f = w_down.shape[2]
    _check("moe_grouped_ffn_bwd", lib().moe_grouped_ffn_bwd(
        _p(x_perm), _p(gu), _p(h), _p(offsets), E, R, d, f, _p(w_gu), _p(w_down),
        _p(row_scale), _p(dy_perm), _dtype_code(w_gu), _p(dgu), _p(dx_perm), _p(dw_gu),
        _p(dw_down), _p(d_row_scale), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn_fwd_gather(x, row_to_slot, k, offsets, E, w_gu, w_down, row_scale, gu, h,
                               y_perm, ws, stream=None):
    T, d = x.shape
    f = w_down.shape[2]
    _check("moe_grouped_ffn_fwd_gather", lib().moe_grouped_ffn_fwd_gather(
        _p(x), T, _p(row_to_slot), k, _p(offsets), E, d, f, _p(w_gu), _p(w_down), _p(row_scale),
        _p(gu), _p(h), _p(y_perm), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn_bwd_gather(x, dy, row_to_slot, slot_to_row, k, gu, h, offsets, E, w_gu,
                               w_down, row_scale, dgu, dx_perm, dw_gu, dw_down, d_row_scale, ws,
                               stream=None, x_perm=None):
    """x_perm given: the dW_gu GEMM reads it instead of gathering x."""
    T, d = dy.shape
    f = w_down.shape[2]
    _check("moe_grouped_ffn_bwd_gather", lib().moe_grouped_ffn_bwd_gather(
        _p(x), _p(x_perm), _p(dy), T, _p(row_to_slot), _p(slot_to_row), k, _p(gu), _p(h),
        _p(offsets), E, d, f,
        _p(w_gu), _p(w_down), _p(row_scale), _p(dgu), _p(dx_perm), _p(dw_gu), _p(dw_down),
        _p(d_row_scale), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_combine(y_perm, slot_to_row, T, k, y, stream=None):
    d = y_perm.shape[1]
    _check("moe_combine", lib().moe_combine(_p(y_perm), _p(slot_to_row), _dtype_code(y_perm),
                                            T, d, k, _p(y), _stream(stream)))


def moe_combine_bwd(dy, slot_to_row, k, dy_perm, stream=None):
    T, d = dy.shape
    _check("moe_combine_bwd", lib().moe_combine_bwd(_p(dy), _p(slot_to_row), _dtype_code(dy),
                                                    T, d, k, _p(dy_perm), _stream(stream)))


def moe_permute_bwd(dx_perm, slot_to_row, dx_add, T, k, dx, stream=None):
    d = dx_perm.shape[1]
    _check("moe_permute_bwd", lib().moe_permute_bwd(_p(dx_perm), _p(slot_to_row), _p(dx_add),
                                                    _dtype_code(dx_perm), T, d, k, _p(dx),
                                                    _stream(stream)))


def moe_permute_bwd_router(dx_perm, slot_to_row, d_logits, w_r, T, k, dx, stream=None):
    d = dx_perm.shape[1]
    E = w_r.shape[0]
    _check("moe_permute_bwd_router", lib().moe_permute_bwd_router(
        _p(dx_perm), _p(slot_to_row), _p(d_logits), _p(w_r), _dtype_code(dx_perm), T, d, E, k,
        _p(dx), _stream(stream)))


def moe_route_bwd(topk_idx, topk_w, d_row_scale, slot_to_row, E, d_topk_w, d_logits,
                  stream=None):
    T, k = topk_idx.shape
    _check("moe_route_bwd", lib().moe_route_bwd(_p(topk_idx), _p(topk_w), _p(d_row_scale),
                                                _p(slot_to_row), T, E, k, _p(d_topk_w),
                                                _p(d_logits), _stream(stream)))


def moe_router_logits_bwd_workspace_size(T, d, E) -> int:
    return int(lib().moe_router_logits_bwd_workspace_size(T, d, E))


def moe_router_logits_bwd(x, w_r, d_logits, dx_router, dw_r, ws, stream=None):
    T, d = x.shape
    E = w_r.shape[0]
    _check("moe_router_logits_bwd", lib().moe_router_logits_bwd(
        _p(x), _p(w_r), _p(d_logits), _dtype_code(x), T, d, E, _p(dx_router), _p(dw_r), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_route_biased(logits, sel_bias, k, topk_idx, topk_w, stream=None):
    T, E = logits.shape
    _check("moe_route_biased", lib().moe_route_biased(_p(logits), _p(sel_bias), T, E, k,
                                                      _p(topk_idx), _p(topk_w), _stream(stream)))


def moe_expert_load_workspace_size(T, E, k) -> int:
    return int(lib().moe_expert_load_workspace_size(T, E, k))


def moe_expert_load(topk_idx, n_valid, E, load, ws, stream=None):
    T, k = topk_idx.shape
    _check("moe_expert_load", lib().moe_expert_load(
        _p(topk_idx), T, n_valid, E, k, _p(load), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_bias_update(load, n_valid, k, rate, sel_bias, stream=None):
    E = load.shape[0]
    _check("moe_bias_update", lib().moe_bias_update(_p(load), n_valid, E, k, float(rate),
                                                    _p(sel_bias), _stream(stream)))


def moe_aux_loss_workspace_size(T, E) -> int:
    return int(lib().moe_aux_loss_workspace_size(T, E))


def moe_aux_loss(logits, load, n_valid, k, coeff, aux_out, d_logits, ws, stream=None):
    T, E = logits.shape
    _check("moe_aux_loss", lib().moe_aux_loss(
        _p(logits), _p(load), T, n_valid, E, k, float(coeff), _p(aux_out), _p(d_logits), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn_lora_workspace_size(R, E, d, f, r) -> int:
    return int(lib().moe_grouped_ffn_lora_workspace_size(R, E, d, f, r))


def moe_grouped_ffn_fwd_lora(x_perm, offsets, E, w_gu, w_down, row_scale, a_gu, b_gu, a_dn, b_dn,
                             scale, z_gu, z_dn, gu, h, y_perm, ws, stream=None):
    R, d = x_perm.shape
    f = w_down.shape[2]
    r = a_gu.shape[1]
    _check("moe_grouped_ffn_fwd_lora", lib().moe_grouped_ffn_fwd_lora(
        _p(x_perm), _p(offsets), E, R, d, f, _p(w_gu), _p(w_down), _p(row_scale), _p(a_gu),
        _p(b_gu), _p(a_dn), _p(b_dn), r, float(scale), _dtype_code(x_perm), _p(z_gu), _p(z_dn),
        _p(gu), _p(h), _p(y_perm), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn_bwd_lora(x_perm, gu, h, offsets, E, w_gu, w_down, row_scale, dy_perm, a_gu,
                             b_gu, a_dn, b_dn, scale, z_gu, z_dn, dgu, dx_perm, d_row_scale,
                             da_gu, db_gu, da_dn, db_dn, ws, stream=None):
    R, d = x_perm.shape
    f = w_down.shape[2]
    r = a_gu.shape[1]
    _check("moe_grouped_ffn_bwd_lora", lib().moe_grouped_ffn_bwd_lora(
        _p(x_perm), _p(gu), _p(h), _p(offsets), E, R, d, f, _p(w_gu), _p(w_down), _p(row_scale),
        _p(dy_perm), _p(a_gu), _p(b_gu), _p(a_dn), _p(b_dn), r, float(scale), _p(z_gu), _p(z_dn),
        _dtype_code(w_gu), _p(dgu), _p(dx_perm), _p(d_row_scale), _p(da_gu), _p(db_gu),
        _p(da_dn), _p(db_dn), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn_lora_bwd_saved(ws, R, E, d, f, r):
    """Views [R, r] (bf16) of u_dn, store(w u_dn) and u_gu inside the LoRA
    backward's workspace ws (a uint8 device tensor)."""
    import torch
    ptrs = [_c_void_p(), _c_void_p(), _c_void_p()]
    nbytes = ws.numel() * ws.element_size()
    _check("moe_grouped_ffn_lora_bwd_saved", lib().moe_grouped_ffn_lora_bwd_saved(
        _p(ws), nbytes, R, E, d, f, r, ctypes.byref(ptrs[0]), ctypes.byref(ptrs[1]),
        ctypes.byref(ptrs[2])))
    base = ws.data_ptr()
    out = []
    for p in ptrs:
        off = int(p.value) - base
        out.append(ws[off:off + 2 * R * r].view(torch.bfloat16).view(R, r))
    return tuple(out)


def moe_timing_enable(on: bool):
    _check("moe_timing_enable", lib().moe_timing_enable(1 if on else 0))


def moe_timing_reset():
    _check("moe_timing_reset", lib().moe_timing_reset())


def moe_timing_query(name: Optional[str]):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check("moe_timing_query", lib().moe_timing_query(None if name is None else name.encode(),
                                                      ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
