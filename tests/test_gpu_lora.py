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
