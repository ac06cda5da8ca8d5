"""GPU parity of the grouped LoRA path (frozen experts) against the oracle.

The grouped FFN with rank-r LoRA factors on both expert matrices, forward
and backward, through the C ABI, on rows sorted by expert (routing from the
oracle on the same inputs).  Bounds as for the grouped FFN: the stored
bf16 tensors that sum over accumulated intermediates (z, GU, H, Y_perm, dGU,
dX_perm, d_row_scale and the fp32 factor gradients) get rel-L2 5e-3 and
max-abs within max(2e-2, one bf16 ulp at the tensor's largest magnitude).
"""
import numpy as np
import pytest

from mixture_experts_layer_03_amd import inputs as I
from oracle import moe_oracle as O
from tests.gpu_util import close, down, need_gpu, up, up_i32

pytestmark = pytest.mark.gpu


def _case(T, d, E, k, f, routing, seed):
    return I.Workload("lora-T%d-d%d-E%d-k%d-f%d-%s" % (T, d, E, k, f, routing), T, d, E, k, f,
                      "bf16", True, routing, seed=seed)


CASES = [(_case(300, 328, 6, 2, 200, "uniform", 31), 16, 0.5),
         (_case(512, 256, 16, 4, 384, "zipf", 32), 32, 2.0),      # empty experts
         (_case(128, 64, 1, 1, 64, "uniform", 33), 64, 1.0),       # one expert
         (_case(400, 192, 8, 2, 136, "uniform", 34), 48, 0.25)]


def _routed(w):
    a = I.make_inputs(w)
    L = O.router_logits(a["x"], a["w_r"], a["bias"], a["noise"])
    idx, tw = O.route(L, w.k)
    counts, offsets, s2r, r2s = O.permute_maps(idx, w.E)
    x_perm, w_perm = O.permute_rows(a["x"], tw, r2s, w.k)
    dy_perm = O.combine_bwd(a["dy"], s2r, w.k)
    return a, offsets, x_perm, w_perm, dy_perm


@pytest.mark.parametrize("w,r,scale", CASES, ids=["%s-r%d" % (c[0].name, c[1]) for c in CASES])
def test_grouped_lora_matches_oracle(w, r, scale):
    import torch
    from mixture_experts_layer_03_amd import abi
    dev = need_gpu()
    print("GPU case", w.name, "rank", r, flush=True)
    a, offsets, x_perm, w_perm, dy_perm = _routed(w)
    lf = I.make_lora_factors(w, r)
    R, d, f, E = w.R, w.d, w.f, w.E
    bf = torch.bfloat16
    z = lambda *s, dt=bf: torch.empty(*s, dtype=dt, device=dev)
    gx, gwgu, gwd, gdy = (up(v, True, dev) for v in (x_perm, a["w_gu"], a["w_down"], dy_perm))
    gag, gbg, gad, gbd = (up(lf[n], True, dev) for n in ("a_gu", "b_gu", "a_dn", "b_dn"))
    goff = up_i32(offsets, dev)
    gwp = up(w_perm, False, dev)
    zg, zd, gu, h, yp = z(R, r), z(R, r), z(R, 2 * f), z(R, f), z(R, d)
    ws = torch.empty(abi.moe_grouped_ffn_lora_workspace_size(R, E, d, f, r), dtype=torch.uint8,
                     device=dev)
    abi.moe_grouped_ffn_fwd_lora(gx, goff, E, gwgu, gwd, gwp, gag, gbg, gad, gbd, scale, zg, zd,
                                 gu, h, yp, ws)
    dgu, dxp = z(R, 2 * f), z(R, d)
    drs = z(R, dt=torch.float32)
    dag, dbg = z(E, r, d, dt=torch.float32), z(E, 2 * f, r, dt=torch.float32)
    dad, dbd = z(E, r, f, dt=torch.float32), z(E, d, r, dt=torch.float32)
    for t in (dag, dbg, dad, dbd):
        t.fill_(7.0)                      # every element must be written
    abi.moe_grouped_ffn_bwd_lora(gx, gu, h, goff, E, gwgu, gwd, gwp, gdy, gag, gbg, gad, gbd,
                                 scale, zg, zd, dgu, dxp, drs, dag, dbg, dad, dbd, ws)
    torch.cuda.synchronize()
    o_gu, o_h, o_y, o_zg, o_zd = O.expert_ffn_fwd_lora(x_perm, offsets, a["w_gu"], a["w_down"],
                                                       w_perm, lf["a_gu"], lf["b_gu"], lf["a_dn"],
                                                       lf["b_dn"], scale, True)
    for n, g, o in (("z_gu", zg, o_zg), ("gu", gu, o_gu), ("h", h, o_h), ("z_dn", zd, o_zd),
                    ("y_perm", yp, o_y)):
        close(n, down(g), o, flip=True)
    # the backward on the device's own forward values (as the block runs it)
    b = O.expert_ffn_bwd_lora(x_perm, down(gu), offsets, a["w_gu"], a["w_down"], w_perm, dy_perm,
                              lf["a_gu"], lf["b_gu"], lf["a_dn"], lf["b_dn"], scale, down(zg),
                              down(zd), True)
    for n, g in (("dgu", dgu), ("dx_perm", dxp), ("d_row_scale", drs), ("da_gu", dag),
                 ("db_gu", dbg), ("da_dn", dad), ("db_dn", dbd)):
        close(n, down(g), b[n], flip=True)
    counts = np.diff(offsets)
    for e in np.where(counts == 0)[0]:
        for t in (dag, dbg, dad, dbd):
            assert float(t[e].abs().max()) == 0.0


BLOCK_CASES = [(_case(300, 328, 6, 2, 200, "uniform", 41), 16),
               (_case(512, 256, 16, 4, 384, "zipf", 42), 32)]


@pytest.mark.parametrize("w,r", BLOCK_CASES, ids=["%s-r%d" % (c[0].name, c[1]) for c in BLOCK_CASES])
def test_block_with_lora_matches_oracle(w, r):
    """The whole block in LoRA mode (router, routing, permutation, LoRA grouped
    FFN, combine and their backward) against the oracle's steps."""
    import torch
    from mixture_experts_layer_03_amd.layer import MoEBlock
    from tests.test_gpu_parity import check_forward
    dev = need_gpu()
    print("GPU case", w.name, "rank", r, flush=True)
    a = I.make_inputs(w)
    lf = I.make_lora_factors(w, r)
    scale = 0.75
    blk = MoEBlock(w.T, w.d, w.E, w.k, w.f, dtype=torch.bfloat16, device=dev, lora_rank=r,
                   lora_scale=scale)
    x, wr, wgu, wd = (up(a[n], True, dev) for n in ("x", "w_r", "w_gu", "w_down"))
    lora = tuple(up(lf[n], True, dev) for n in ("a_gu", "b_gu", "a_dn", "b_dn"))
    bias = None if a["bias"] is None else up(a["bias"], False, dev)
    blk.forward(x, wr, wgu, wd, bias, lora=lora)
    blk.backward(x, wr, wgu, wd, up(a["dy"], True, dev), lora=lora)
    torch.cuda.synchronize()
    g = {n: down(getattr(blk, n)) for n in (
        "logits", "topk_idx", "topk_w", "counts", "offsets", "slot_to_row", "row_to_slot",
        "x_perm", "w_perm", "gu", "h", "y_perm", "y", "z_gu", "z_dn", "dgu", "dx_perm",
        "d_row_scale", "d_logits", "dw_r", "dx", "da_gu", "db_gu", "da_dn", "db_dn")}
    # oracle: the same steps with the LoRA grouped FFN
    o = {}
    o["logits"] = O.router_logits(a["x"], a["w_r"], a["bias"], a["noise"])
    o["topk_idx"], o["topk_w"] = O.route(o["logits"], w.k)
    o["counts"], o["offsets"], o["slot_to_row"], o["row_to_slot"] = O.permute_maps(o["topk_idx"], w.E)
    o["x_perm"], o["w_perm"] = O.permute_rows(a["x"], o["topk_w"], o["row_to_slot"], w.k)
    o["gu"], o["h"], o["y_perm"], o["z_gu"], o["z_dn"] = O.expert_ffn_fwd_lora(
        o["x_perm"], o["offsets"], a["w_gu"], a["w_down"], o["w_perm"], lf["a_gu"], lf["b_gu"],
        lf["a_dn"], lf["b_dn"], scale, True)
    o["y"] = O.combine(o["y_perm"], o["slot_to_row"], w.T, w.k, True)
    check_forward(g, o)
    close("z_gu", g["z_gu"], o["z_gu"], flip=True)
    close("z_dn", g["z_dn"], o["z_dn"], flip=True)
    dyp = O.combine_bwd(a["dy"], o["slot_to_row"], w.k)
    b = O.expert_ffn_bwd_lora(o["x_perm"], o["gu"], o["offsets"], a["w_gu"], a["w_down"],
                              o["w_perm"], dyp, lf["a_gu"], lf["b_gu"], lf["a_dn"], lf["b_dn"],
                              scale, o["z_gu"], o["z_dn"], True)
    _, dl = O.route_bwd(o["topk_idx"], o["topk_w"], b["d_row_scale"], o["slot_to_row"], w.E)
    dxr, dwr = O.router_logits_bwd(a["x"], a["w_r"], dl)
    dx = O.permute_bwd(b["dx_perm"], o["slot_to_row"], w.T, w.k, dxr, True)
    for n, ref in (("dgu", b["dgu"]), ("dx_perm", b["dx_perm"]), ("d_row_scale", b["d_row_scale"]),
                   ("d_logits", dl), ("dw_r", dwr), ("da_gu", b["da_gu"]), ("db_gu", b["db_gu"]),
                   ("da_dn", b["da_dn"]), ("db_dn", b["db_dn"])):
        close(n, g[n], ref, flip=True)
    close("dx", g["dx"], dx)
