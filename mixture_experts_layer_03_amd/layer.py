"""The MoE expert block as a sequence of C-ABI calls.

``MoEBlock`` owns the device buffers of one problem size (torch allocations)
and issues the library calls of the forward and backward passes in order, all
on one stream, with no host synchronisation in between:

  forward : moe_router_logits -> moe_route (moe_route_biased with a
            selection bias) -> moe_permute -> moe_grouped_ffn_fwd -> moe_combine
  backward: moe_combine_bwd -> moe_grouped_ffn_bwd -> moe_route_bwd ->
            [moe_expert_load -> moe_aux_loss, with an auxiliary-loss
            coefficient] -> moe_router_logits_bwd (dW_r) ->
            moe_permute_bwd_router (dX with the router term formed in the
            same pass; with fuse_router_dx=False, moe_router_logits_bwd also
            stores dx_router and moe_permute_bwd adds it)
  balance : moe_expert_load -> moe_bias_update (selection-bias step)

With ``gather`` the grouped GEMMs read the token rows of X and dY where they
load them (moe_grouped_ffn_fwd_gather / moe_grouped_ffn_bwd_gather; past
their size limits, gather_fits(), the block falls back to stored rows):
dY_perm is never stored and moe_combine_bwd drops out.  X_perm is still
written by moe_permute for the dW_gu GEMM (its stored rows are the faster
operand there) unless ``store_x_perm`` is False; then moe_permute writes only
the maps and w_perm and the dW_gu GEMM gathers X too.

With ``lora_rank`` set the experts are frozen and carry LoRA factors:
moe_grouped_ffn_fwd_lora / moe_grouped_ffn_bwd_lora replace the grouped-FFN
calls, and the backward forms the LoRA factor gradients instead of the expert
weight gradients.

This mirrors the EP forward path the pages describe (router logits in fp32,
per-token top-k, tokens sorted by expert, grouped matmul, rows returned and
weighted by the top-k probabilities: "Halo's 2.8x over TRL is not a kernel,
and its own benchmark proves it", section "Where the gap actually is"), with
the dispatch and combine all-to-alls reduced to on-GPU row permutations.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import abi


def gather_fits(T: int, d: int, k: int) -> bool:
    """Whether the gathered grouped-FFN calls take this size: their token-row
    offsets are 32-bit (T*d < 2^30) and the slot -> token division is exact
    while T*k*k < 2^32 (moe_grouped_ffn_fwd_gather's documented limits)."""
    return T * d < (1 << 30) and T * k * k < (1 << 32)


class MoEBlock:
    def __init__(self, T: int, d: int, E: int, k: int, f: int, dtype=torch.bfloat16,
                 device="cuda", backward: bool = True, fuse_router_dx: bool = True,
                 lora_rank: int = 0, lora_scale: float = 1.0, gather: bool = False,
                 store_x_perm: bool = True):
        if gather and (lora_rank or dtype != torch.bfloat16):
            raise ValueError("gather needs bf16 experts without LoRA")
        # beyond the gathered calls' limits the block runs on stored rows
        # (the same results bit for bit)
        self.gather_fallback = bool(gather and not gather_fits(T, d, k))
        if self.gather_fallback:
            gather = False
        self.gather = gather
        self.store_x_perm = store_x_perm or not gather
        self.T, self.d, self.E, self.k, self.f = T, d, E, k, f
        self.fuse_router_dx = fuse_router_dx
        self.lora_rank, self.lora_scale = lora_rank, lora_scale
        self.R = T * k
        self.dtype = dtype
        self.device = device
        dc = abi.MOE_BF16 if dtype == torch.bfloat16 else abi.MOE_F32
        self.dcode = dc
        R = self.R
        z = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=device)
        i32 = torch.int32
        f32 = torch.float32
        self.logits = z(T, E, dt=f32)
        self.topk_idx = z(T, k, dt=i32)
        self.topk_w = z(T, k, dt=f32)
        self.counts = z(E, dt=i32)
        self.offsets = z(E + 1, dt=i32)
        self.slot_to_row = z(R, dt=i32)
        self.row_to_slot = z(R, dt=i32)
        self.x_perm = z(R, d) if self.store_x_perm else None
        self.w_perm = z(R, dt=f32)
        self.gu = z(R, 2 * f)
        self.h = z(R, f)
        self.y_perm = z(R, d)
        self.y = z(T, d)
        ws_perm = abi.moe_permute_workspace_size(T, E, k)
        ws_ffn = abi.moe_grouped_ffn_workspace_size(R, E, d, f, dc)
        ws_rtr = abi.moe_router_logits_bwd_workspace_size(T, d, E) if backward else 0
        ws_stat = max(abi.moe_expert_load_workspace_size(T, E, k),
                      abi.moe_aux_loss_workspace_size(T, E))
        if lora_rank:
            ws_ffn = abi.moe_grouped_ffn_lora_workspace_size(R, E, d, f, lora_rank)
            self.z_gu = z(R, lora_rank)
            self.z_dn = z(R, lora_rank)
        # the grouped FFN's workspace is its own, so that what its backward
        # leaves there (e.g. the LoRA rank-r rows) survives the router calls
        self.ws = torch.empty(max(ws_perm, ws_rtr, ws_stat, 256), dtype=torch.uint8,
                              device=device)
        self.ws_ffn = torch.empty(max(ws_ffn, 256), dtype=torch.uint8, device=device)
        self.load = z(E, dt=i32)
        self.aux = z(2, dt=f32)
        self.has_bwd = backward
        if backward:
            self.dy_perm = None if gather else z(R, d)
            self.dgu = z(R, 2 * f)
            self.dx_perm = z(R, d)
            self.d_row_scale = z(R, dt=f32)
            self.d_topk_w = z(T, k, dt=f32)
            self.d_logits = z(T, E, dt=f32)
            # the router's fp32 dX is only stored when it is not fused into dX
            self.dx_router = None if fuse_router_dx else z(T, d, dt=f32)
            self.dw_r = z(E, d, dt=f32)
            if lora_rank:   # frozen experts: LoRA factor gradients only
                r = lora_rank
                self.da_gu, self.db_gu = z(E, r, d, dt=f32), z(E, 2 * f, r, dt=f32)
                self.da_dn, self.db_dn = z(E, r, f, dt=f32), z(E, d, r, dt=f32)
            else:
                self.dw_gu = z(E, 2 * f, d, dt=f32)
                self.dw_down = z(E, d, f, dt=f32)
            self.dx = z(T, d)

    # ------------------------------------------------------------ forward
    def forward(self, x, w_r, w_gu, w_down, bias=None, noise=None, stream=None, sel_bias=None,
                lora=None):
        """bias is added to the logits (it moves selection and weights);
        sel_bias only shifts the scores the top-k compares."""
        abi.moe_router_logits(x, w_r, bias, noise, self.logits, stream)
        if sel_bias is None:
            abi.moe_route(self.logits, self.k, self.topk_idx, self.topk_w, stream)
        else:
            abi.moe_route_biased(self.logits, sel_bias, self.k, self.topk_idx, self.topk_w, stream)
        self.permute(x, stream)
        self.experts_forward(w_gu, w_down, stream, lora, x=x)
        abi.moe_combine(self.y_perm, self.slot_to_row, self.T, self.k, self.y, stream)
        return self.y

    def permute(self, x, stream=None):
        if not self.store_x_perm:
            x = None   # maps and w_perm only
        abi.moe_permute(x, self.topk_idx, self.topk_w, self.T, self.d, self.E, self.k,
                        self.counts, self.offsets, self.slot_to_row, self.row_to_slot,
                        self.x_perm, self.w_perm, self.ws, dtype=self.dcode, stream=stream)

    def experts_forward(self, w_gu, w_down, stream=None, lora=None, x=None):
        """lora: (a_gu, b_gu, a_dn, b_dn) device tensors when lora_rank is set;
        x: the token rows, read by the gathered GEMM."""
        if self.gather:
            abi.moe_grouped_ffn_fwd_gather(x, self.row_to_slot, self.k, self.offsets, self.E,
                                           w_gu, w_down, self.w_perm, self.gu, self.h,
                                           self.y_perm, self.ws_ffn, stream)
            return
        if self.lora_rank:
            a_gu, b_gu, a_dn, b_dn = lora
            abi.moe_grouped_ffn_fwd_lora(self.x_perm, self.offsets, self.E, w_gu, w_down,
                                         self.w_perm, a_gu, b_gu, a_dn, b_dn, self.lora_scale,
                                         self.z_gu, self.z_dn, self.gu, self.h, self.y_perm,
                                         self.ws_ffn, stream)
            return
        abi.moe_grouped_ffn_fwd(self.x_perm, self.offsets, self.E, w_gu, w_down, self.w_perm,
                                self.gu, self.h, self.y_perm, self.ws_ffn, stream)

    # ------------------------------------------------------------ backward
    def backward(self, x, w_r, w_gu, w_down, dy, stream=None, aux_coeff: float = 0.0,
                 n_valid: Optional[int] = None, lora=None):
        """aux_coeff != 0 adds the load-balancing auxiliary loss's gradient to
        the router's; its statistics (and self.aux = [aux, aux_scaled]) cover
        the first n_valid tokens (all if None)."""
        assert self.has_bwd
        if not self.gather:
            abi.moe_combine_bwd(dy, self.slot_to_row, self.k, self.dy_perm, stream)
        self.experts_backward(w_gu, w_down, stream, lora, x=x, dy=dy)
        abi.moe_route_bwd(self.topk_idx, self.topk_w, self.d_row_scale, self.slot_to_row,
                          self.E, self.d_topk_w, self.d_logits, stream)
        if aux_coeff != 0.0:
            n = self.T if n_valid is None else n_valid
            abi.moe_expert_load(self.topk_idx, n, self.E, self.load, self.ws, stream)
            abi.moe_aux_loss(self.logits, self.load, n, self.k, aux_coeff, self.aux,
                             self.d_logits, self.ws, stream)
        if self.fuse_router_dx:
            abi.moe_router_logits_bwd(x, w_r, self.d_logits, None, self.dw_r, self.ws, stream)
            abi.moe_permute_bwd_router(self.dx_perm, self.slot_to_row, self.d_logits, w_r, self.T,
                                       self.k, self.dx, stream)
        else:
            abi.moe_router_logits_bwd(x, w_r, self.d_logits, self.dx_router, self.dw_r, self.ws,
                                      stream)
            abi.moe_permute_bwd(self.dx_perm, self.slot_to_row, self.dx_router, self.T, self.k,
                                self.dx, stream)
        return self.dx

    def balance_selection_bias(self, sel_bias, rate: float, n_valid: Optional[int] = None,
                               stream=None):
        """One selection-bias balancing step from the last forward's routing:
        self.load = per-expert load of the first n_valid tokens, then sel_bias
        moves by rate toward the mean load (in place)."""
        n = self.T if n_valid is None else n_valid
        abi.moe_expert_load(self.topk_idx, n, self.E, self.load, self.ws, stream)
        abi.moe_bias_update(self.load, n, self.k, rate, sel_bias, stream)

    def experts_backward(self, w_gu, w_down, stream=None, lora=None, x=None, dy=None):
        if self.gather:
            abi.moe_grouped_ffn_bwd_gather(x, dy, self.row_to_slot, self.slot_to_row, self.k,
                                           self.gu, self.h,
                                           self.offsets, self.E, w_gu, w_down, self.w_perm,
                                           self.dgu, self.dx_perm, self.dw_gu, self.dw_down,
                                           self.d_row_scale, self.ws_ffn, stream,
                                           x_perm=self.x_perm)
            return
        if self.lora_rank:
            a_gu, b_gu, a_dn, b_dn = lora
            abi.moe_grouped_ffn_bwd_lora(self.x_perm, self.gu, self.h, self.offsets, self.E, w_gu,
                                         w_down, self.w_perm, self.dy_perm, a_gu, b_gu, a_dn,
                                         b_dn, self.lora_scale, self.z_gu, self.z_dn, self.dgu,
                                         self.dx_perm, self.d_row_scale, self.da_gu, self.db_gu,
                                         self.da_dn, self.db_dn, self.ws_ffn, stream)
            return
        abi.moe_grouped_ffn_bwd(self.x_perm, self.gu, self.h, self.offsets, self.E, w_gu,
                                w_down, self.w_perm, self.dy_perm, self.dgu, self.dx_perm,
                                self.dw_gu, self.dw_down, self.d_row_scale, self.ws_ffn, stream)


class ExpertShare:
    """Grouped FFN alone over rows that arrive already sorted by expert (one
    expert-parallel rank's local share: its experts and the rows dispatched to
    it)."""

    def __init__(self, R: int, d: int, E: int, f: int, dtype=torch.bfloat16, device="cuda"):
        self.R, self.d, self.E, self.f = R, d, E, f
        z = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=device)
        f32 = torch.float32
        self.gu = z(R, 2 * f)
        self.h = z(R, f)
        self.y_perm = z(R, d)
        self.dgu = z(R, 2 * f)
        self.dx_perm = z(R, d)
        self.d_row_scale = z(R, dt=f32)
        self.dw_gu = z(E, 2 * f, d, dt=f32)
        self.dw_down = z(E, d, f, dt=f32)
        dc = abi.MOE_BF16 if dtype == torch.bfloat16 else abi.MOE_F32
        self.ws = torch.empty(max(256, abi.moe_grouped_ffn_workspace_size(R, E, d, f, dc)),
                              dtype=torch.uint8, device=device)

    def forward(self, x_perm, offsets, w_gu, w_down, w_perm, stream=None):
        abi.moe_grouped_ffn_fwd(x_perm, offsets, self.E, w_gu, w_down, w_perm, self.gu, self.h,
                                self.y_perm, self.ws, stream)
        return self.y_perm

    def backward(self, x_perm, offsets, w_gu, w_down, w_perm, dy_perm, stream=None):
        abi.moe_grouped_ffn_bwd(x_perm, self.gu, self.h, offsets, self.E, w_gu, w_down, w_perm,
                                dy_perm, self.dgu, self.dx_perm, self.dw_gu, self.dw_down,
                                self.d_row_scale, self.ws, stream)
        return self.dx_perm
