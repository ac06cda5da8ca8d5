"""GPU parity of the grouped LoRA path (frozen experts) against the oracle.

The grouped FFN with rank-r LoRA factors on both expert matrices, forward
and backward, through the C ABI, on rows sorted by expert (routing from the
oracle on the same inputs).  The oracle's backward runs on the oracle's own
forward values.  Bounds as for the grouped FFN (tests/parity.py): max-abs
2e-2 and rel-L2 5e-3, each element's max-abs widened only by its step's
derived bound; the rank-r rows the backward stores (u_dn, store(w u_dn),
u_gu) are read from its workspace and checked too.
"""
import numpy as np
import pytest

from mixture_experts_layer_03_amd import inputs as I
from oracle import moe_oracle as O
from tests import parity as PC
from tests.gpu_util import close, down, need_gpu, up, up_i32
from tests.test_gpu_parity import check_exact

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
    ud, uwd, ug = abi.moe_grouped_ffn_lora_bwd_saved(ws, R, E, d, f, r)
    got = dict(z_gu=zg, gu=gu, h=h, z_dn=zd, y_perm=yp, dgu=dgu, dx_perm=dxp, d_row_scale=drs,
               da_gu=dag, db_gu=dbg, da_dn=dad, db_dn=dbd, u_dn=ud, uw_dn=uwd, u_gu=ug)
    got = {n: down(v) for n, v in got.items()}
    check_lora_ffn(got, a, lf, scale, offsets, x_perm, w_perm, dy_perm)


def check_lora_ffn(got, a, lf, scale, offsets, x_perm, w_perm, dy_perm, wg=None):
    """The LoRA grouped FFN against the oracle, its backward on the oracle's
    own forward values."""
    o_gu, o_h, o_y, o_zg, o_zd = O.expert_ffn_fwd_lora(x_perm, offsets, a["w_gu"], a["w_down"],
                                                       w_perm, lf["a_gu"], lf["b_gu"], lf["a_dn"],
                                                       lf["b_dn"], scale, True)
    ref = dict(gu=o_gu, h=o_h, y_perm=o_y, z_gu=o_zg, z_dn=o_zd)
    ref.update(O.expert_ffn_bwd_lora(x_perm, o_gu, offsets, a["w_gu"], a["w_down"], w_perm,
                                     dy_perm, lf["a_gu"], lf["b_gu"], lf["a_dn"], lf["b_dn"],
                                     scale, o_zg, o_zd, True))
    # store(w u_dn) is one fp32 product rounded to bf16 on the device: bit for
    # bit the oracle's rounding of the device's own operands (pins the
    # device's round-to-nearest-even)
    wg_ = np.asarray(w_perm if wg is None else wg, np.float32)
    assert np.array_equal(got["uw_dn"], O.to_bf16(wg_[:, None] * got["u_dn"].astype(np.float32)))
    lora = (lf["a_gu"], lf["b_gu"], lf["a_dn"], lf["b_dn"], scale)
    return PC.check_ffn(got, ref, x_perm, offsets, a["w_gu"], a["w_down"],
                        w_perm if wg is None else wg, w_perm, dy_perm, lora=lora)


BLOCK_CASES = [(_case(300, 328, 6, 2, 200, "uniform", 41), 16),
               (_case(512, 256, 16, 4, 384, "zipf", 42), 32)]


@pytest.mark.parametrize("w,r", BLOCK_CASES, ids=["%s-r%d" % (c[0].name, c[1]) for c in BLOCK_CASES])
def test_block_with_lora_matches_oracle(w, r):
    """The whole block in LoRA mode (router, routing, permutation, LoRA grouped
    FFN, combine and their backward) against the oracle's steps."""
    import torch
    from mixture_experts_layer_03_amd import abi
    from mixture_experts_layer_03_amd.layer import MoEBlock
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
        "d_row_scale", "d_topk_w", "d_logits", "dw_r", "dx", "da_gu", "db_gu", "da_dn",
        "db_dn")}
    ud, uwd, ug = abi.moe_grouped_ffn_lora_bwd_saved(blk.ws_ffn, w.R, w.E, w.d, w.f, r)
    for n, v in (("u_dn", ud), ("uw_dn", uwd), ("u_gu", ug)):
        g[n] = down(v)
    # oracle: the same steps with the LoRA grouped FFN
    o = {}
    o["logits"] = O.router_logits(a["x"], a["w_r"], a["bias"], a["noise"])
    o["topk_idx"], o["topk_w"] = O.route(o["logits"], w.k)
    o["counts"], o["offsets"], o["slot_to_row"], o["row_to_slot"] = O.permute_maps(o["topk_idx"], w.E)
    o["x_perm"], o["w_perm"] = O.permute_rows(a["x"], o["topk_w"], o["row_to_slot"], w.k)
    check_exact(g, o)
    close("topk_w", g["topk_w"], o["topk_w"], max_abs=1e-6, rel_l2=1e-6)
    dyp = O.combine_bwd(a["dy"], o["slot_to_row"], w.k)
    dev = check_lora_ffn(g, a, lf, scale, o["offsets"], o["x_perm"], o["w_perm"], dyp,
                         wg=g["w_perm"])
    o_gu, _, o_y, o_zg, o_zd = O.expert_ffn_fwd_lora(
        o["x_perm"], o["offsets"], a["w_gu"], a["w_down"], o["w_perm"], lf["a_gu"], lf["b_gu"],
        lf["a_dn"], lf["b_dn"], scale, True)
    o["y_perm"] = o_y
    o["y"] = O.combine(o_y, o["slot_to_row"], w.T, w.k, True)
    b = O.expert_ffn_bwd_lora(o["x_perm"], o_gu, o["offsets"], a["w_gu"], a["w_down"],
                              o["w_perm"], dyp, lf["a_gu"], lf["b_gu"], lf["a_dn"], lf["b_dn"],
                              scale, o_zg, o_zd, True)
    b["d_topk_w"], b["d_logits"] = O.route_bwd(o["topk_idx"], o["topk_w"], b["d_row_scale"],
                                               o["slot_to_row"], w.E)
    b["dx_router"], b["dw_r"] = O.router_logits_bwd(a["x"], a["w_r"], b["d_logits"])
    b["dx"] = O.permute_bwd(b["dx_perm"], o["slot_to_row"], w.T, w.k, b["dx_router"], True)
    PC.check_tokens(g, o, b, a, w.k, dev)


@pytest.mark.slow
def test_lora_full_size():
    """The gpt-oss-20b-like layer (T=4096, d=f=2880, E=32, top-4) with frozen
    experts and rank-16 LoRA, as the benchmark times it, against the oracle:
    routing bit for bit, every row tensor and LoRA factor gradient in full."""
    import torch
    from mixture_experts_layer_03_amd import abi
    from mixture_experts_layer_03_amd.layer import MoEBlock
    dev_ = need_gpu()
    w, r, scale = I.GPTOSS, 16, 1.0
    print("GPU case", w.name, "LoRA rank", r, flush=True)
    a = I.make_inputs(w)
    lf = I.make_lora_factors(w, r)
    blk = MoEBlock(w.T, w.d, w.E, w.k, w.f, dtype=torch.bfloat16, device=dev_, lora_rank=r,
                   lora_scale=scale)
    x, wr, wgu, wd = (up(a[n], True, dev_) for n in ("x", "w_r", "w_gu", "w_down"))
    lora = tuple(up(lf[n], True, dev_) for n in ("a_gu", "b_gu", "a_dn", "b_dn"))
    blk.forward(x, wr, wgu, wd, lora=lora)
    blk.backward(x, wr, wgu, wd, up(a["dy"], True, dev_), lora=lora)
    torch.cuda.synchronize()
    names = ("logits", "topk_idx", "topk_w", "counts", "offsets", "slot_to_row", "row_to_slot",
             "x_perm", "w_perm", "gu", "h", "y_perm", "z_gu", "z_dn", "dgu", "dx_perm",
             "d_row_scale", "da_gu", "db_gu", "da_dn", "db_dn")
    g = {n: down(getattr(blk, n)) for n in names}
    ud, uwd, ug = abi.moe_grouped_ffn_lora_bwd_saved(blk.ws_ffn, w.R, w.E, w.d, w.f, r)
    for n, v in (("u_dn", ud), ("uw_dn", uwd), ("u_gu", ug)):
        g[n] = down(v)
    del blk
    o = {}
    o["logits"] = O.router_logits(a["x"], a["w_r"], a["bias"], a["noise"])
    o["topk_idx"], o["topk_w"] = O.route(o["logits"], w.k)
    o["counts"], o["offsets"], o["slot_to_row"], o["row_to_slot"] = O.permute_maps(o["topk_idx"], w.E)
    o["x_perm"], o["w_perm"] = O.permute_rows(a["x"], o["topk_w"], o["row_to_slot"], w.k)
    check_exact(g, o)
    close("topk_w", g["topk_w"], o["topk_w"], max_abs=1e-6, rel_l2=1e-6)
    dyp = O.combine_bwd(a["dy"], o["slot_to_row"], w.k)
    check_lora_ffn(g, a, lf, scale, o["offsets"], o["x_perm"], o["w_perm"], dyp, wg=g["w_perm"])
