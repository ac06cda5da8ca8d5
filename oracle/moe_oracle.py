"""ORACLE for the MoE expert block -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports, links or calls anything under ``oracle/``,
and nothing here touches the HIP library.

What it computes is the plain definition of the block as the pages state the
problem, written as a loop over experts (the structure of the opt-in per-expert
loop that "Halo's 2.8x over TRL is not a kernel, and its own benchmark proves
it" compares against grouped GEMM in section "It is not the kernel, and Halo's
own numbers prove it"):

  forward  (section "Where the gap actually is", EP token-routing figure):
    fp32 router logits -> per-token top-k -> tokens sorted by expert ->
    per-expert gate/up GEMM with SwiGLU -> per-expert down GEMM, each output
    row weighted by its top-k probability -> rows returned to their token and
    summed.
  backward: the adjoint of each step, the routing adjoint written as a gather
    (no scatter-add; "Halo: Frontier-Lab Training for Everyone", section "Some
    of the hard problems along the way", on the atomic-free routing backward),
    plus the gradients of the expert weights and of the router.

Arithmetic: every GEMM is a library fp64 matmul (``numpy.matmul`` on float64);
every elementwise step runs in fp64.  Values are rounded only where the block
stores a tensor, to that tensor's storage type (bf16 for activations in the
bf16 workloads, fp32 otherwise).  The one exception is the router logits, for
which the pages fix fp32; their accumulation order is fixed in
``router_fma.c`` (a chain of fp32 fused multiply-adds over the hidden index).

Readings of points the pages leave open:
  * softmax over the k selected logits (equal to a full softmax renormalised
    over the selected experts);
  * top-k ordered by value, descending; equal values -> lower expert id first;
  * rows sorted by expert, and by slot index (token-major) within an expert;
  * dropless: every selected (token, expert) pair is computed;
  * W_gu[E, 2f, d] holds gate rows 0..f-1 then up rows f..2f-1; W_down[E, d, f];
    no expert biases; h = silu(g) * u with silu(x) = x / (1 + exp(-x));
  * the combine weight multiplies the down-projection output row;
  * weight and router gradients are fp32; activation gradients use the
    activation storage type.

Storage rounding points (bf16 workloads): X_perm (exact copy), GU, H (from the
stored g and u), Y_perm, Y, dY_perm (exact copy), S = w * dY_perm (the
row-scaled upstream gradient used by the down-projection weight gradient),
dGU, dX_perm, dX.  fp32 storage: logits, topk_w, w_perm, d_row_scale,
d_topk_w, d_logits, dX_router, dW_r, dW_gu, dW_down.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "router_fma.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liboracle_router.so")
_lib_handle = None


# ---------------------------------------------------------------------------
# build / load the C part (the fp32 fma-chain router logits)
# ---------------------------------------------------------------------------

def build(force: bool = False) -> str:
    """Compile router_fma.c with gcc into oracle/_build/ (host code only)."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _lib_handle
    if _lib_handle is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_router_logits.restype = ctypes.c_int
        lib.oracle_router_logits.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        _lib_handle = lib
    return _lib_handle


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# storage rounding (the oracle's own; shares nothing with the device code)
# ---------------------------------------------------------------------------

def to_bf16(a) -> np.ndarray:
    """Round to fp32, then to the nearest bf16 (ties to even); result as fp32."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1)))
         & np.uint64(0xFFFF0000)).astype(np.uint32)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = np.uint32(0x7FC00000)
    return r.view(np.float32).reshape(f.shape)


def store(a, bf16: bool) -> np.ndarray:
    """Value as stored by the block: fp32, or bf16 for bf16 activations."""
    return to_bf16(a) if bf16 else np.asarray(a, dtype=np.float32)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(x):
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


# ---------------------------------------------------------------------------
# forward steps
# ---------------------------------------------------------------------------

def router_logits(x, w_r, bias=None, noise=None) -> np.ndarray:
    """L[t,e] = fp32 fma chain of x[t,:]*w_r[e,:] in hidden order, + bias[e], + noise[t,e]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w_r = np.ascontiguousarray(w_r, dtype=np.float32)
    T, d = x.shape
    E = w_r.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    n = None if noise is None else np.ascontiguousarray(noise, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float32)
    rc = _lib().oracle_router_logits(_ptr(x), _ptr(w_r), _ptr(b), _ptr(n), T, d, E, _ptr(out))
    if rc != 0:
        raise MemoryError("oracle_router_logits failed")
    return out


def route(logits, k: int):
    """Per-token top-k (value descending, ties to the lower expert id) and the
    softmax over the k selected logits.  Returns (topk_idx int32 [T,k],
    topk_w fp32 [T,k]).  A NaN logit ranks below every number (NaNs among
    themselves by expert id); a selection holding a NaN, or whose largest
    logit is +inf, gets NaN weights."""
    L = np.asarray(logits, dtype=np.float32)
    # A stable sort of the negated values keeps equal values in expert order;
    # numpy sorts NaN after every number.
    idx = np.argsort(-L, axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = _f64(np.take_along_axis(L, idx, axis=1))
    with np.errstate(invalid="ignore"):
        ex = np.exp(sel - sel[:, :1])
        w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


def permute_maps(topk_idx, E: int):
    """Tokens sorted by expert.  Slot s = t*k + j.  Rows are ordered by expert,
    then by slot.  Returns counts[E], offsets[E+1], slot_to_row[R], row_to_slot[R]
    (all int32)."""
    flat = np.asarray(topk_idx, dtype=np.int64).ravel()
    row_to_slot = np.argsort(flat, kind="stable")
    slot_to_row = np.empty_like(row_to_slot)
    slot_to_row[row_to_slot] = np.arange(flat.size)
    counts = np.bincount(flat, minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    return (counts.astype(np.int32), offsets.astype(np.int32),
            slot_to_row.astype(np.int32), row_to_slot.astype(np.int32))


def permute_rows(x, topk_w, row_to_slot, k: int):
    """X_perm[r] = X[token of the slot at row r]; w_perm[r] = that slot's weight."""
    r2s = np.asarray(row_to_slot, dtype=np.int64)
    x_perm = np.asarray(x, dtype=np.float32)[r2s // k]
    w_perm = None if topk_w is None else np.asarray(topk_w, dtype=np.float32).ravel()[r2s]
    return x_perm, w_perm


def _ffn_rows(xr, w_gu_e, w_down_e, wr, bf16: bool):
    """One expert applied to the rows xr[M,d]; wr[M] is the row weight or None.
    Returns GU (stored), H (stored), Y (stored)."""
    f = w_gu_e.shape[0] // 2
    gu = store(_f64(xr) @ _f64(w_gu_e).T, bf16)
    h = store(silu(gu[:, :f]) * _f64(gu[:, f:]), bf16)
    y = _f64(h) @ _f64(w_down_e).T
    if wr is not None:
        y = _f64(wr)[:, None] * y
    return gu, h, store(y, bf16)


def expert_ffn_fwd(x_perm, offsets, w_gu, w_down, row_scale=None, bf16=True):
    """Loop over experts.  Returns GU[R,2f], H[R,f], Y_perm[R,d] (fp32 arrays
    holding the stored values)."""
    R, d = x_perm.shape
    E, f2, _ = w_gu.shape
    f = f2 // 2
    gu = np.zeros((R, 2 * f), np.float32)
    h = np.zeros((R, f), np.float32)
    y = np.zeros((R, d), np.float32)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        wr = None if row_scale is None else row_scale[a:b]
        gu[a:b], h[a:b], y[a:b] = _ffn_rows(x_perm[a:b], w_gu[e], w_down[e], wr, bf16)
    return gu, h, y


def combine(y_perm, slot_to_row, T: int, k: int, bf16=True):
    """Y[t] = sum over j of Y_perm[row of slot t*k+j] (fp64 sum, one rounding)."""
    s2r = np.asarray(slot_to_row, dtype=np.int64).reshape(T, k)
    acc = np.zeros((T, y_perm.shape[1]), np.float64)
    for j in range(k):
        acc += _f64(y_perm[s2r[:, j]])
    return store(acc, bf16)


# ---------------------------------------------------------------------------
# backward steps
# ---------------------------------------------------------------------------

def combine_bwd(dy, slot_to_row, k: int):
    """dY_perm[row of slot t*k+j] = dY[t] (the adjoint of the row sum is a copy)."""
    s2r = np.asarray(slot_to_row, dtype=np.int64)
    T, d = dy.shape
    out = np.empty((T * k, d), np.float32)
    out[s2r] = np.repeat(np.asarray(dy, np.float32), k, axis=0)
    return out


def _ffn_bwd_rows(xr, gur, dyr, wr, w_gu_e, w_down_e, bf16: bool):
    """Backward of one expert over rows.  Returns dGU (stored), dX (stored),
    d_row_scale (fp32), the fp64 pieces needed for the weight gradients."""
    f = w_gu_e.shape[0] // 2
    g = _f64(gur[:, :f])
    u = _f64(gur[:, f:])
    h = store(silu(g) * u, bf16)                     # recomputed exactly as forward
    gd = _f64(dyr) @ _f64(w_down_e)                    # dL/d(h) before the row weight
    d_row_scale = np.sum(_f64(h) * gd, axis=1)
    w = np.ones(len(xr)) if wr is None else _f64(wr)
    dh = w[:, None] * gd
    sg = sigmoid(g)
    dg = dh * u * sg * (1.0 + g * (1.0 - sg))
    du = dh * g * sg
    dgu = store(np.concatenate([dg, du], axis=1), bf16)
    dx = store(_f64(dgu) @ _f64(w_gu_e), bf16)
    s = store(w[:, None] * _f64(dyr), bf16)
    return dgu, dx, d_row_scale.astype(np.float32), h, s


def expert_ffn_bwd(x_perm, gu, offsets, w_gu, w_down, row_scale, dy_perm, bf16=True):
    """Loop over experts.  Returns dict with dGU[R,2f], dX_perm[R,d],
    d_row_scale[R], dW_gu[E,2f,d] (fp32), dW_down[E,d,f] (fp32)."""
    R, d = x_perm.shape
    E, f2, _ = w_gu.shape
    f = f2 // 2
    out = {
        "dgu": np.zeros((R, 2 * f), np.float32),
        "dx_perm": np.zeros((R, d), np.float32),
        "d_row_scale": np.zeros(R, np.float32),
        "dw_gu": np.zeros((E, 2 * f, d), np.float32),
        "dw_down": np.zeros((E, d, f), np.float32),
    }
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue            # an empty expert's weight gradients are zero
        wr = None if row_scale is None else row_scale[a:b]
        dgu, dx, drs, h, s = _ffn_bwd_rows(x_perm[a:b], gu[a:b], dy_perm[a:b], wr,
                                           w_gu[e], w_down[e], bf16)
        out["dgu"][a:b] = dgu
        out["dx_perm"][a:b] = dx
        out["d_row_scale"][a:b] = drs
        out["dw_down"][e] = (_f64(s).T @ _f64(h)).astype(np.float32)
        out["dw_gu"][e] = (_f64(dgu).T @ _f64(x_perm[a:b])).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# grouped LoRA on the fused expert weights (experts frozen)
# ---------------------------------------------------------------------------
#
# "Halo: Frontier-Lab Training for Everyone" (section "One trainer
# architecture, one parallelism stack") applies LoRA directly to the fused 3-D
# expert weights, with
# the experts frozen, so that they need no gradient or optimizer state.  The
# pages give no formulas; the plainest reading, used here, is standard LoRA on
# each expert matrix: W_gu[e] + s * B_gu[e] @ A_gu[e] and
# W_down[e] + s * B_dn[e] @ A_dn[e], with A_gu[E,r,d], B_gu[E,2f,r],
# A_dn[E,r,f], B_dn[E,d,r] (gate rows then up rows in B_gu, like W_gu) and
# a scale s.  The low-rank products are stored in bf16 like the other
# activations (storage points of this reading):
#   z_gu = store(s * X_perm A_gu^T)              [R, r]
#   GU   = store(X_perm W_gu^T + z_gu B_gu^T)      (one fp32 accumulation)
#   z_dn = store(s * H A_dn^T)                   [R, r]
#   Y    = store(w * (H W_down^T + z_dn B_dn^T))
# backward (no expert weight gradients):
#   u_dn = store(s * dY_perm B_dn)                [R, r]
#   Gd   = dY_perm W_down + u_dn A_dn  -> dSwiGLU and d_row_scale as before
#   u_gu = store(s * dGU B_gu)                    [R, r]
#   dX_perm = store(dGU W_gu + u_gu A_gu)
#   dB_gu = dGU^T z_gu, dA_gu = u_gu^T X_perm, dB_dn = S^T z_dn with
#   S = store(w * dY_perm), dA_dn = store(w * u_dn)^T H   (fp32 outputs;
#   the row-weighted u_dn is stored like S, the row-weighted dY)

def _ffn_rows_lora(xr, w_gu_e, w_down_e, wr, a_gu_e, b_gu_e, a_dn_e, b_dn_e, scale, bf16):
    f = w_gu_e.shape[0] // 2
    z_gu = store(scale * (_f64(xr) @ _f64(a_gu_e).T), bf16)
    gu = store(_f64(xr) @ _f64(w_gu_e).T + _f64(z_gu) @ _f64(b_gu_e).T, bf16)
    gate, up = _f64(gu[:, :f]), _f64(gu[:, f:])
    h = store(silu(gate) * up, bf16)
    z_dn = store(scale * (_f64(h) @ _f64(a_dn_e).T), bf16)
    y = _f64(h) @ _f64(w_down_e).T + _f64(z_dn) @ _f64(b_dn_e).T
    if wr is not None:
        y = _f64(wr)[:, None] * y
    return gu, h, store(y, bf16), z_gu, z_dn


def expert_ffn_fwd_lora(x_perm, offsets, w_gu, w_down, row_scale, a_gu, b_gu, a_dn, b_dn,
                        scale: float, bf16=True):
    """Loop over experts with LoRA on both expert matrices.  Returns GU, H,
    Y_perm, z_gu[R,r], z_dn[R,r] (stored values)."""
    R, d = x_perm.shape
    E, f2, _ = w_gu.shape
    f = f2 // 2
    r = a_gu.shape[1]
    gu = np.zeros((R, 2 * f), np.float32)
    h = np.zeros((R, f), np.float32)
    y = np.zeros((R, d), np.float32)
    z_gu = np.zeros((R, r), np.float32)
    z_dn = np.zeros((R, r), np.float32)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        wr = None if row_scale is None else row_scale[a:b]
        gu[a:b], h[a:b], y[a:b], z_gu[a:b], z_dn[a:b] = _ffn_rows_lora(
            x_perm[a:b], w_gu[e], w_down[e], wr, a_gu[e], b_gu[e], a_dn[e], b_dn[e], scale, bf16)
    return gu, h, y, z_gu, z_dn


def expert_ffn_bwd_lora(x_perm, gu, offsets, w_gu, w_down, row_scale, dy_perm, a_gu, b_gu,
                        a_dn, b_dn, scale: float, z_gu, z_dn, bf16=True):
    """Backward with frozen experts.  Returns dict with dGU, dX_perm,
    d_row_scale, u_gu, u_dn, uw_dn = store(w u_dn) (stored) and dA_gu[E,r,d],
    dB_gu[E,2f,r], dA_dn[E,r,f], dB_dn[E,d,r] (fp32)."""
    R, d = x_perm.shape
    E, f2, _ = w_gu.shape
    f = f2 // 2
    r = a_gu.shape[1]
    out = {
        "dgu": np.zeros((R, 2 * f), np.float32),
        "dx_perm": np.zeros((R, d), np.float32),
        "d_row_scale": np.zeros(R, np.float32),
        "u_gu": np.zeros((R, r), np.float32),
        "u_dn": np.zeros((R, r), np.float32),
        "uw_dn": np.zeros((R, r), np.float32),
        "da_gu": np.zeros((E, r, d), np.float32),
        "db_gu": np.zeros((E, 2 * f, r), np.float32),
        "da_dn": np.zeros((E, r, f), np.float32),
        "db_dn": np.zeros((E, d, r), np.float32),
    }
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue            # an empty expert's LoRA gradients are zero
        xr, dyr = x_perm[a:b], dy_perm[a:b]
        g = _f64(gu[a:b, :f])
        uu = _f64(gu[a:b, f:])
        h = store(silu(g) * uu, bf16)
        w = np.ones(b - a) if row_scale is None else _f64(row_scale[a:b])
        u_dn = store(scale * (_f64(dyr) @ _f64(b_dn[e])), bf16)
        gd = _f64(dyr) @ _f64(w_down[e]) + _f64(u_dn) @ _f64(a_dn[e])
        drs = np.sum(_f64(h) * gd, axis=1)
        dh = w[:, None] * gd
        sg = sigmoid(g)
        dg = dh * uu * sg * (1.0 + g * (1.0 - sg))
        du = dh * g * sg
        dgu = store(np.concatenate([dg, du], axis=1), bf16)
        u_gu = store(scale * (_f64(dgu) @ _f64(b_gu[e])), bf16)
        dx = store(_f64(dgu) @ _f64(w_gu[e]) + _f64(u_gu) @ _f64(a_gu[e]), bf16)
        s_ = store(w[:, None] * _f64(dyr), bf16)
        out["dgu"][a:b] = dgu
        out["dx_perm"][a:b] = dx
        out["d_row_scale"][a:b] = drs.astype(np.float32)
        out["u_gu"][a:b] = u_gu
        out["u_dn"][a:b] = u_dn
        out["db_gu"][e] = (_f64(dgu).T @ _f64(z_gu[a:b])).astype(np.float32)
        out["da_gu"][e] = (_f64(u_gu).T @ _f64(xr)).astype(np.float32)
        out["db_dn"][e] = (_f64(s_).T @ _f64(z_dn[a:b])).astype(np.float32)
        uw_dn = store(w[:, None] * _f64(u_dn), bf16)
        out["uw_dn"][a:b] = uw_dn
        out["da_dn"][e] = (_f64(uw_dn).T @ _f64(h)).astype(np.float32)
    return out


def permute_bwd(dx_perm, slot_to_row, T: int, k: int, dx_add=None, bf16=True):
    """dX[t] = sum over j of dX_perm[row of slot t*k+j] (+ dx_add[t]); fp64 sum."""
    s2r = np.asarray(slot_to_row, dtype=np.int64).reshape(T, k)
    acc = np.zeros((T, dx_perm.shape[1]), np.float64)
    for j in range(k):
        acc += _f64(dx_perm[s2r[:, j]])
    if dx_add is not None:
        acc += _f64(dx_add)
    return store(acc, bf16)


def route_bwd(topk_idx, topk_w, d_row_scale, slot_to_row, E: int):
    """Adjoint of the softmax over the selected logits.
    g_j = d_row_scale at slot (t,j);  dL/dl_{idx_j} = w_j (g_j - sum_i w_i g_i);
    unselected logits get 0.  Returns d_topk_w[T,k], d_logits[T,E] (fp32)."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    g = _f64(np.asarray(d_row_scale)[np.asarray(slot_to_row, np.int64)]).reshape(T, k)
    w = _f64(topk_w)
    s = np.sum(w * g, axis=1, keepdims=True)
    dl = np.zeros((T, E), np.float64)
    np.put_along_axis(dl, idx, w * (g - s), axis=1)
    return g.astype(np.float32), dl.astype(np.float32)


def router_logits_bwd(x, w_r, d_logits):
    """dX_router = d_logits @ W_r;  dW_r = d_logits^T @ X  (fp64, stored fp32)."""
    dl = _f64(d_logits)
    return (dl @ _f64(w_r)).astype(np.float32), (dl.T @ _f64(x)).astype(np.float32)


# ---------------------------------------------------------------------------
# router variants: selection-only bias, its balancing update, the
# load-balancing auxiliary loss, and statistics over a valid token prefix
# ---------------------------------------------------------------------------
#
# The pages name these features without formulas: LFM2's recipe sets
# ``moe_balancing: bias_update`` because that family has no router auxiliary
# loss, so balance is kept through a bias on expert *selection* ("Halo's 2.8x
# over TRL is not a kernel, and its own benchmark proves it", section "The
# small-hardware end", the LFM2 config and the paragraph after it); other
# models train with a router auxiliary loss whose coefficient is set per run,
# the routers applying its gradient and reporting the unscaled and scaled
# values (the TorchTurbo page, "inclusionAI open-sources TorchTurbo, a
# SuperNode-native post-training engine", section "Adapter", ms-swift DPO);
# and right-padded tails are excluded from MoE statistics, the valid prefix
# being described by the packed-sequence metadata (same TorchTurbo page,
# section "Model", sequence-parallel input contract).  The plainest readings,
# used here:
#   * selection score s[t,e] = fp32(L[t,e] + b_sel[e]) picks the k experts
#     (same order and tie rule as ``route``); the weights are the softmax of
#     the k selected *unbiased* logits, so the bias steers selection only;
#   * load_e = number of (t, j) with t < n_valid and topk_idx[t,j] = e;
#   * bias update: b_e += rate * sign(mean_load - load_e), mean_load =
#     n_valid * k / E (the sign decided exactly in integers);
#   * aux = E * sum_e f_e * P_e with f_e = load_e / (n_valid * k) and
#     P_e = mean over t < n_valid of softmax(L[t,:])_e (all E experts);
#     aux_scaled = coeff * aux; the gradient flows through P only (load is a
#     count), and padded tokens t >= n_valid get none.  Balanced routing with
#     uniform probabilities gives aux = 1.

def route_biased(logits, sel_bias, k: int):
    """Top-k by the fp32 selection score L + b_sel (value descending, ties to the
    lower expert id); weights = softmax over the k selected unbiased logits.
    Returns (topk_idx int32 [T,k], topk_w fp32 [T,k])."""
    L = np.asarray(logits, dtype=np.float32)
    if sel_bias is None:
        score = L
    else:
        score = L + np.asarray(sel_bias, dtype=np.float32)[None, :]   # one fp32 add
    idx = np.argsort(-score, axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = _f64(np.take_along_axis(L, idx, axis=1))
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


def expert_load(topk_idx, E: int, n_valid: Optional[int] = None) -> np.ndarray:
    """load[e] = selections of expert e by the tokens t < n_valid (int32 [E])."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    n = idx.shape[0] if n_valid is None else int(n_valid)
    return np.bincount(idx[:n].ravel(), minlength=E).astype(np.int32)


def bias_update(sel_bias, load, n_valid: int, k: int, rate: float) -> np.ndarray:
    """b_e + rate * sign(n_valid*k/E - load_e), in fp32 (one add per expert)."""
    b = np.asarray(sel_bias, dtype=np.float32)
    ld = np.asarray(load, dtype=np.int64)
    E = b.shape[0]
    sgn = np.sign(int(n_valid) * int(k) - E * ld)          # exact integer comparison
    step = np.where(sgn > 0, np.float32(rate), np.where(sgn < 0, np.float32(-rate),
                                                        np.float32(0.0))).astype(np.float32)
    return (b + step).astype(np.float32)


def aux_loss(logits, load, n_valid: int, k: int, coeff: float):
    """Load-balancing auxiliary loss and its gradient w.r.t. the logits.
    Returns (aux, aux_scaled, d_logits fp32 [T,E]); d_logits is zero on the
    padded tail and everywhere when n_valid = 0."""
    L = _f64(logits)
    T, E = L.shape
    n = int(n_valid)
    dl = np.zeros((T, E), np.float64)
    if n == 0:
        return 0.0, 0.0, dl.astype(np.float32)
    Lv = L[:n]
    p = np.exp(Lv - Lv.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)                 # softmax over all experts
    P = p.mean(axis=0)
    f = _f64(load) / (n * k)
    aux = E * float(np.sum(f * P))
    # d(coeff*aux)/dP_e = coeff*E*f_e;  dP_e/dp[t,e] = 1/n;  softmax Jacobian.
    g = coeff * E * f / n
    s = np.sum(p * g[None, :], axis=1, keepdims=True)
    dl[:n] = p * (g[None, :] - s)
    return aux, coeff * aux, dl.astype(np.float32)


# ---------------------------------------------------------------------------
# whole block
# ---------------------------------------------------------------------------

def layer_forward(x, w_r, w_gu, w_down, k: int, bias=None, noise=None, bf16=True,
                  sel_bias=None) -> Dict:
    T = x.shape[0]
    E = w_r.shape[0]
    o: Dict[str, np.ndarray] = {}
    o["logits"] = router_logits(x, w_r, bias, noise)
    if sel_bias is None:
        o["topk_idx"], o["topk_w"] = route(o["logits"], k)
    else:
        o["topk_idx"], o["topk_w"] = route_biased(o["logits"], sel_bias, k)
    o["counts"], o["offsets"], o["slot_to_row"], o["row_to_slot"] = permute_maps(o["topk_idx"], E)
    o["x_perm"], o["w_perm"] = permute_rows(x, o["topk_w"], o["row_to_slot"], k)
    o["gu"], o["h"], o["y_perm"] = expert_ffn_fwd(o["x_perm"], o["offsets"], w_gu, w_down,
                                                 o["w_perm"], bf16)
    o["y"] = combine(o["y_perm"], o["slot_to_row"], T, k, bf16)
    return o


def layer_backward(fwd: Dict, x, w_r, w_gu, w_down, dy, k: int, bf16=True,
                   aux_coeff: float = 0.0, n_valid: Optional[int] = None) -> Dict:
    """With aux_coeff != 0 the auxiliary-loss gradient (statistics over the
    first n_valid tokens, all tokens if None) is added to d_logits."""
    T = x.shape[0]
    E = w_r.shape[0]
    b: Dict[str, np.ndarray] = {}
    b["dy_perm"] = combine_bwd(dy, fwd["slot_to_row"], k)
    b.update(expert_ffn_bwd(fwd["x_perm"], fwd["gu"], fwd["offsets"], w_gu, w_down,
                            fwd["w_perm"], b["dy_perm"], bf16))
    b["d_topk_w"], b["d_logits"] = route_bwd(fwd["topk_idx"], fwd["topk_w"], b["d_row_scale"],
                                             fwd["slot_to_row"], E)
    if aux_coeff != 0.0:
        n = T if n_valid is None else int(n_valid)
        b["load"] = expert_load(fwd["topk_idx"], E, n)
        b["aux"], b["aux_scaled"], g = aux_loss(fwd["logits"], b["load"], n, k, aux_coeff)
        b["d_logits"] = (_f64(b["d_logits"]) + _f64(g)).astype(np.float32)
    b["dx_router"], b["dw_r"] = router_logits_bwd(x, w_r, b["d_logits"])
    b["dx"] = permute_bwd(b["dx_perm"], fwd["slot_to_row"], T, k, b["dx_router"], bf16)
    return b


# ---------------------------------------------------------------------------
# sampled variants for full-size checks (same arithmetic on subsets)
# ---------------------------------------------------------------------------

def expert_of_rows(offsets, rows) -> np.ndarray:
    off = np.asarray(offsets, dtype=np.int64)
    return np.searchsorted(off, np.asarray(rows, np.int64), side="right") - 1


def ffn_fwd_sampled_rows(x_perm, offsets, w_gu, w_down, row_scale, rows, bf16=True):
    """GU, H, Y_perm for the listed rows only."""
    rows = np.asarray(rows, np.int64)
    ex = expert_of_rows(offsets, rows)
    f = w_gu.shape[1] // 2
    gu = np.zeros((len(rows), 2 * f), np.float32)
    h = np.zeros((len(rows), f), np.float32)
    y = np.zeros((len(rows), w_down.shape[1]), np.float32)
    for e in np.unique(ex):
        m = ex == e
        wr = None if row_scale is None else np.asarray(row_scale)[rows[m]]
        gu[m], h[m], y[m] = _ffn_rows(np.asarray(x_perm)[rows[m]], w_gu[e], w_down[e], wr, bf16)
    return gu, h, y


def ffn_bwd_sampled_rows(x_perm, offsets, w_gu, w_down, row_scale, dy_perm, rows, bf16=True):
    """dGU, dX_perm, d_row_scale for the listed rows (GU recomputed by the oracle)."""
    rows = np.asarray(rows, np.int64)
    ex = expert_of_rows(offsets, rows)
    f = w_gu.shape[1] // 2
    d = w_gu.shape[2]
    dgu = np.zeros((len(rows), 2 * f), np.float32)
    dx = np.zeros((len(rows), d), np.float32)
    drs = np.zeros(len(rows), np.float32)
    for e in np.unique(ex):
        m = ex == e
        xr = np.asarray(x_perm)[rows[m]]
        wr = None if row_scale is None else np.asarray(row_scale)[rows[m]]
        gu, _, _ = _ffn_rows(xr, w_gu[e], w_down[e], wr, bf16)
        dgu[m], dx[m], drs[m], _, _ = _ffn_bwd_rows(xr, gu, np.asarray(dy_perm)[rows[m]], wr,
                                                    w_gu[e], w_down[e], bf16)
    return dgu, dx, drs


def weight_grads_sampled_cols(x_perm, offsets, w_gu, w_down, row_scale, dy_perm, e: int,
                              cols, bf16=True, operands=False):
    """For expert e and hidden-unit columns c in ``cols`` (0 <= c < f):
    dW_gu[e][c, :], dW_gu[e][f+c, :] and dW_down[e][:, c], from only the
    columns of GU, H and dGU that they need.  Returns (dw_gate[len,d],
    dw_up[len,d], dw_down_cols[d,len]), and with operands=True also a dict of
    the stored operands they are summed from (the expert's rows of the dGU
    gate and up columns, the H columns and S)."""
    cols = np.asarray(cols, np.int64)
    f = w_gu.shape[1] // 2
    a, b = int(offsets[e]), int(offsets[e + 1])
    d = w_gu.shape[2]
    if a == b:
        z = np.zeros((len(cols), d), np.float32)
        return z, z.copy(), np.zeros((d, len(cols)), np.float32)
    xr = _f64(np.asarray(x_perm)[a:b])
    dyr = _f64(np.asarray(dy_perm)[a:b])
    w = np.ones(b - a) if row_scale is None else _f64(np.asarray(row_scale)[a:b])
    g = _f64(store(xr @ _f64(w_gu[e][cols]).T, bf16))
    u = _f64(store(xr @ _f64(w_gu[e][f + cols]).T, bf16))
    h = _f64(store(silu(g) * u, bf16))
    gd = dyr @ _f64(w_down[e][:, cols])
    dh = w[:, None] * gd
    sg = sigmoid(g)
    dg = _f64(store(dh * u * sg * (1.0 + g * (1.0 - sg)), bf16))
    du = _f64(store(dh * g * sg, bf16))
    s = _f64(store(w[:, None] * dyr, bf16))
    out = ((dg.T @ xr).astype(np.float32), (du.T @ xr).astype(np.float32),
           (s.T @ h).astype(np.float32))
    if operands:
        return out + ({"dg": dg, "du": du, "h": h, "s": s},)
    return out
