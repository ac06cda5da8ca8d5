"""The C-ABI library on the CPU (no GPU needed): it loads, exports every
function include/moe.h declares, and rejects invalid arguments on the host
before launching anything."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_03_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_hot_path():
    names = declared_functions()
    for n in ("moe_router_logits", "moe_route", "moe_permute", "moe_grouped_ffn_fwd",
              "moe_grouped_ffn_bwd", "moe_combine", "moe_combine_bwd", "moe_permute_bwd",
              "moe_route_bwd", "moe_router_logits_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = abi.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
        assert n in abi._SIGS, "binding lacks " + n


def test_status_strings():
    L = abi.lib()
    assert L.moe_strerror(0) == b"ok"
    assert L.moe_strerror(-3).startswith(b"workspace")
    assert L.moe_version() >= 100


P = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _rc_msg(rc):
    return rc, abi.lib().moe_last_error().decode()


def test_validation_rejects_before_launch():
    L = abi.lib()
    # k > E
    rc, msg = _rc_msg(L.moe_route(P, 10, 4, 5, P, P, None))
    assert rc == -2, msg
    # E out of range
    assert L.moe_route(P, 10, 2000, 2, P, P, None) == -2
    # d not a multiple of 8
    assert L.moe_router_logits(P, P, None, None, 1, 10, 12, 4, P, None) == -2
    # bad dtype
    assert L.moe_router_logits(P, P, None, None, 7, 10, 16, 4, P, None) == -2
    # null pointers with work to do
    assert L.moe_router_logits(None, P, None, None, 1, 10, 16, 4, P, None) == -1
    assert L.moe_combine(None, P, 1, 10, 16, 2, P, None) == -1
    # misaligned pointer
    assert L.moe_combine(ctypes.c_void_p(0x1002), P, 1, 10, 16, 2, P, None) == -1
    # R = T*k >= 2^31
    assert L.moe_combine(P, P, 1, 1 << 30, 16, 4, P, None) == -2
    # workspace too small
    need = L.moe_permute_workspace_size(100, 8, 2)
    assert need > 0
    assert L.moe_permute(P, P, None, 1, 100, 16, 8, 2, P, P, P, P, P, None, P, need - 1,
                         None) == -3
    need = L.moe_grouped_ffn_workspace_size(1000, 8, 64, 64, 1)
    assert L.moe_grouped_ffn_fwd(P, P, 8, 1000, 64, 64, P, P, None, 1, P, P, P, P, need - 1,
                                 None) == -3
    # backward needs bf16
    assert L.moe_grouped_ffn_bwd(P, P, P, P, 8, 1000, 64, 64, P, P, None, P, 0, P, P, P, P, None,
                                 P, need, None) == -2
    # negative sizes
    assert L.moe_permute_bwd(P, P, None, 1, -1, 16, 2, P, None) == -1
    assert "T < 0" in abi.lib().moe_last_error().decode()


def test_fused_router_dx_validation():
    L = abi.lib()
    assert L.moe_permute_bwd_router(P, P, P, P, 1, 10, 16, 2000, 2, P, None) == -2
    assert L.moe_permute_bwd_router(P, P, None, P, 1, 10, 16, 8, 2, P, None) == -1
    assert L.moe_permute_bwd_router(P, P, P, ctypes.c_void_p(0x1004), 1, 10, 16, 8, 2, P,
                                    None) == -1
    assert L.moe_permute_bwd_router(P, P, P, P, 1, 10, 12, 8, 2, P, None) == -2
    assert L.moe_permute_bwd_router(None, None, None, None, 1, 0, 16, 8, 2, None, None) == 0


def test_router_variant_validation_rejects_before_launch():
    L = abi.lib()
    F = ctypes.c_float
    # selection bias is required by the biased call
    assert L.moe_route_biased(P, None, 10, 4, 2, P, P, None) == -1
    assert L.moe_route_biased(P, P, 10, 4, 5, P, P, None) == -2
    assert L.moe_route_biased(None, None, 0, 4, 2, None, None, None) == 0
    # valid prefix outside [0, T]
    need = L.moe_expert_load_workspace_size(100, 8, 2)
    assert need >= 8 * 4
    rc, msg = _rc_msg(L.moe_expert_load(P, 100, 101, 8, 2, P, P, need, None))
    assert rc == -1 and "n_valid" in msg, msg
    assert L.moe_expert_load(P, 100, -1, 8, 2, P, P, need, None) == -1
    assert L.moe_expert_load(P, 100, 50, 8, 9, P, P, need, None) == -2
    assert L.moe_expert_load(P, 100, 100, 8, 2, None, P, need, None) == -1
    assert L.moe_expert_load(P, 100000, 100000, 8, 2, P, P, need, None) == -3
    # bias rate must be finite and non-negative
    assert L.moe_bias_update(P, 10, 8, 2, F(-0.5), P, None) == -1
    assert L.moe_bias_update(P, 10, 8, 2, F(float("nan")), P, None) == -1
    assert L.moe_bias_update(P, 10, 8, 2, F(float("inf")), P, None) == -1
    assert L.moe_bias_update(None, 10, 8, 2, F(0.1), P, None) == -1
    # aux loss
    wsz = L.moe_aux_loss_workspace_size(4096, 32)
    assert wsz >= 32 * 4
    assert L.moe_aux_loss(P, P, 100, 101, 8, 2, F(0.1), P, None, P, wsz, None) == -1
    assert L.moe_aux_loss(P, P, 100, 100, 8, 2, F(0.1), None, None, P, wsz, None) == -1
    assert L.moe_aux_loss(P, P, 100, 100, 8, 2, F(float("inf")), P, None, P, wsz, None) == -1
    assert L.moe_aux_loss(P, P, 1 << 20, 1 << 20, 8, 2, F(0.1), P, None, P, 256, None) == -3
    assert L.moe_aux_loss(P, P, 100, 100, 2000, 2, F(0.1), P, None, P, wsz, None) == -2


def test_gather_ffn_validation_rejects_before_launch():
    L = abi.lib()
    ws = L.moe_grouped_ffn_workspace_size(400, 8, 64, 64, 1)
    fwd = L.moe_grouped_ffn_fwd_gather
    # good shape, missing row_to_slot
    assert fwd(P, 100, None, 4, P, 8, 64, 64, P, P, None, P, P, P, P, ws, None) == -1
    # k out of range, d not a multiple of 8, E out of range
    assert fwd(P, 100, P, 33, P, 8, 64, 64, P, P, None, P, P, P, P, ws, None) == -2
    assert fwd(P, 100, P, 4, P, 8, 60, 64, P, P, None, P, P, P, P, ws, None) == -2
    assert fwd(P, 100, P, 4, P, 2000, 64, 64, P, P, None, P, P, P, P, ws, None) == -2
    # 32-bit offset limits: T*d and T*k*k
    rc, msg = _rc_msg(fwd(P, 1 << 25, P, 1, P, 8, 64, 64, P, P, None, P, P, P, P, ws, None))
    assert rc == -2 and "T*d" in msg, msg
    assert fwd(P, 1 << 24, P, 32, P, 8, 8, 64, P, P, None, P, P, P, P, ws, None) == -2
    # misaligned, small workspace, empty
    assert fwd(ctypes.c_void_p(0x1008), 100, P, 4, P, 8, 64, 64, P, P, None, P, P, P, P, ws,
               None) == -1
    assert fwd(P, 100, P, 4, P, 8, 64, 64, P, P, None, P, P, P, P, 16, None) == -3
    assert fwd(None, 0, None, 4, None, 8, 64, 64, None, None, None, None, None, None, None, 0,
               None) == 0
    bwd = L.moe_grouped_ffn_bwd_gather
    # x, x_perm, dy, T, row_to_slot, slot_to_row, k, gu, h, offsets, E, d, f, w_gu, w_down,
    # row_scale, dgu, dx_perm, dw_gu, dw_down, d_row_scale, ws, ws_bytes, stream
    args = [P, None, P, 100, P, P, 4, P, P, P, 8, 64, 64, P, P, None, P, P, P, P, None, P, ws,
            None]
    a = list(args); a[2] = None                      # dy
    assert bwd(*a) == -1
    a = list(args); a[0] = None                      # neither x nor x_perm
    assert bwd(*a) == -1
    a = list(args); a[4] = None                      # row_to_slot
    assert bwd(*a) == -1
    a = list(args); a[5] = None                      # slot_to_row
    assert bwd(*a) == -1
    a = list(args); a[6] = 0                         # k
    assert bwd(*a) == -2
    a = list(args); a[22] = 16                       # workspace
    assert bwd(*a) == -3
    a = list(args); a[18] = ctypes.c_void_p(0x1004)  # dw_gu alignment
    assert bwd(*a) == -1
    a = list(args); a[1] = ctypes.c_void_p(0x1008)   # x_perm alignment
    assert bwd(*a) == -1


def test_empty_inputs_are_ok_without_launch():
    L = abi.lib()
    assert L.moe_router_logits(None, None, None, None, 1, 0, 16, 4, None, None) == 0
    assert L.moe_route(None, 0, 4, 2, None, None, None) == 0
    assert L.moe_combine(None, None, 1, 0, 16, 2, None, None) == 0
    assert L.moe_combine_bwd(None, None, 1, 0, 16, 2, None, None) == 0
    assert L.moe_permute_bwd(None, None, None, 1, 0, 16, 2, None, None) == 0
    assert L.moe_route_bwd(None, None, None, None, 0, 4, 2, None, None, None) == 0
    assert L.moe_grouped_ffn_fwd(None, None, 4, 0, 16, 16, None, None, None, 1, None, None, None,
                                 None, 0, None) == 0


def test_workspace_sizes_scale_with_problem():
    L = abi.lib()
    a = L.moe_grouped_ffn_workspace_size(16384, 32, 2880, 2880, 1)
    b = L.moe_grouped_ffn_workspace_size(65536, 32, 2880, 2880, 1)
    assert 0 < a < b
    assert L.moe_router_logits_bwd_workspace_size(4096, 2880, 32) >= 32 * 4 * 2880 * 4


def test_gathered_block_falls_back_to_stored_rows_past_the_limits():
    from mixture_experts_layer_03_amd.layer import gather_fits
    assert gather_fits(4096, 2880, 4) and gather_fits(32768, 2048, 8)
    assert not gather_fits(400000, 2880, 4)          # T*d >= 2^30
    assert not gather_fits(1 << 20, 8, 64)            # T*k*k >= 2^32
    import torch
    from mixture_experts_layer_03_amd.layer import MoEBlock
    # the decision is taken before anything is allocated on a device
    blk = MoEBlock(2, 8, 2, 1, 8, device="cpu", gather=True)
    assert blk.gather and not blk.gather_fallback
