"""GPU-vs-oracle comparison of the block with per-element bounds.

Exact: routing, maps and copies (checked by the callers).  Everything else:
max-abs 2e-2 and rel-L2 5e-3, each element's max-abs widened only by the
bound tests/tolerance.py derives from its own step (its rounding, the observed
deviation of its stored inputs, fp32 accumulation).

Row tensors (GU, H, Y_perm, dGU, dX_perm, d_row_scale and the LoRA rank-r
activations) are checked row by row, so the same code serves the full checks
and the sampled rows of the largest workloads; weight gradients are sums over
an expert's rows and are checked per expert (or per sampled column).
"""
import numpy as np

from oracle import moe_oracle as O
from tests import tolerance as TB
from tests.gpu_util import Tally, close

f64 = TB.f64
ROW_FWD = ("gu", "h", "y_perm")
ROW_BWD = ("dgu", "dx_perm", "d_row_scale")
LORA_FWD = ("z_gu", "z_dn")
LORA_BWD = ("u_dn", "uw_dn", "u_gu")
LORA_GRADS = ("db_gu", "da_gu", "db_dn", "da_dn")


def s_rows(w, dy):
    """S = store(w * dY) as the device forms it (fp32 product, bf16 store)."""
    return O.to_bf16(np.asarray(w, np.float32)[:, None] * np.asarray(dy, np.float32))


def s_rows_oracle(w, dy):
    return O.store(f64(w)[:, None] * f64(dy), True)


class Tallies(dict):
    def __missing__(self, name):
        v = self[name] = Tally(self.tag + name)
        return v

    def __init__(self, tag=""):
        super().__init__()
        self.tag = tag

    def finish(self):
        for v in self.values():
            v.finish()


def expert_rows(t, got, ref, X, dY, Wgu, Wd, wg, wr, lora=None, bwd=True, bf16=True):
    """Row checks for rows of one expert.  got / ref: dicts of row arrays (the
    same rows on both sides); X, dY: the rows' exact inputs; Wgu [2f,d],
    Wd [d,f]: the expert's weights; wg / wr: row weights of each side.
    lora: None or (a_gu, b_gu, a_dn, b_dn, scale) of the expert.
    Returns the observed deviations the later steps need."""
    d = X.shape[1]
    f = Wgu.shape[0] // 2
    X = f64(X)
    gu_g, gu_r = f64(got["gu"]), f64(ref["gu"])
    h_g, h_r = f64(got["h"]), f64(ref["h"])
    dv = {}
    extra_gu = None
    if lora is not None:
        Ag, Bg, Ad, Bd = (f64(v) for v in lora[:4])
        s = float(lora[4])
        zg_g, zg_r = f64(got["z_gu"]), f64(ref["z_gu"])
        t["z_gu"].add(zg_g, zg_r, TB.rounding(zg_g, zg_r) + s * TB.acc(d, TB.rownorm(X),
                                                                          TB.rownorm(Ag)))
        dv["z_gu"] = zg_g - zg_r
        extra_gu = TB.absdot(dv["z_gu"], Bg.T) + TB.acc(Ag.shape[0], TB.rownorm(zg_g),
                                                        TB.rownorm(Bg))
    t["gu"].add(gu_g, gu_r, TB.b_gemm_rows(gu_g, gu_r, X, f64(Wgu), d, extra_gu, bf16))
    t["h"].add(h_g, h_r, TB.b_h(h_g, h_r, gu_g, gu_r, f, bf16))
    dH = dv["h"] = h_g - h_r
    y_g, y_r = f64(got["y_perm"]), f64(ref["y_perm"])
    yb = TB.b_scaled_rows(y_g, y_r, wg, wr, dH, h_g, f64(Wd), f, bf16)
    if lora is not None:
        zd_g, zd_r = f64(got["z_dn"]), f64(ref["z_dn"])
        t["z_dn"].add(zd_g, zd_r, TB.rounding(zd_g, zd_r) + s * (
            TB.absdot(dH, Ad.T) + TB.acc(f, TB.rownorm(h_g), TB.rownorm(Ad))))
        dv["z_dn"] = zd_g - zd_r
        yb += f64(wg)[:, None] * (TB.absdot(dv["z_dn"], Bd.T)
                                  + TB.acc(Ad.shape[0], TB.rownorm(zd_g), TB.rownorm(Bd)))
    t["y_perm"].add(y_g, y_r, yb)
    dv["y_perm"] = y_g - y_r
    if not bwd:
        return dv
    dY = f64(dY)
    Wd = f64(Wd)
    gd = dY @ Wd                                        # exact Gd from the oracle's side
    dgd = TB.acc(d, TB.rownorm(dY), TB.colnorm(Wd))     # the device's Gd lies within this
    if lora is not None:
        ud_g, ud_r = f64(got["u_dn"]), f64(ref["u_dn"])
        t["u_dn"].add(ud_g, ud_r, TB.rounding(ud_g, ud_r) + s * TB.acc(d, TB.rownorm(dY),
                                                                          TB.colnorm(Bd)))
        uw_g, uw_r = f64(got["uw_dn"]), f64(ref["uw_dn"])
        t["uw_dn"].add(uw_g, uw_r, TB.rounding(uw_g, uw_r) + 2 * TB.U32 * np.abs(uw_r)
                       + np.abs(f64(wg)[:, None] * ud_g - f64(wr)[:, None] * ud_r))
        dv["u_dn"], dv["uw_dn"] = ud_g - ud_r, uw_g - uw_r
        gd = gd + ud_r @ Ad
        dgd = dgd + TB.absdot(dv["u_dn"], Ad) + TB.acc(Ad.shape[0], TB.rownorm(ud_g),
                                                       TB.colnorm(Ad))
    dgu_g, dgu_r = f64(got["dgu"]), f64(ref["dgu"])
    t["dgu"].add(dgu_g, dgu_r, TB.b_dgu(dgu_g, dgu_r, gu_g, gu_r, wg, wr, gd, dgd, f))
    ddgu = dv["dgu"] = dgu_g - dgu_r
    dx_g, dx_r = f64(got["dx_perm"]), f64(ref["dx_perm"])
    extra = TB.absdot(ddgu, f64(Wgu))
    if lora is not None:
        ug_g, ug_r = f64(got["u_gu"]), f64(ref["u_gu"])
        t["u_gu"].add(ug_g, ug_r, TB.rounding(ug_g, ug_r) + s * (
            TB.absdot(ddgu, Bg) + TB.acc(2 * f, TB.rownorm(dgu_g), TB.colnorm(Bg))))
        dv["u_gu"] = ug_g - ug_r
        extra = extra + TB.absdot(dv["u_gu"], Ag) + TB.acc(Ag.shape[0], TB.rownorm(ug_g),
                                                           TB.colnorm(Ag))
    t["dx_perm"].add(dx_g, dx_r, TB.b_gemm_rows(dx_g, dx_r, dgu_g, f64(Wgu).T, 2 * f, extra))
    dv["dx_perm"] = dx_g - dx_r
    drs_r = f64(ref["d_row_scale"])
    drs_b = TB.b_rowdot(dH, h_g, gd, dgd, f) + 2 * TB.U32 * np.abs(drs_r)
    t["d_row_scale"].add(got["d_row_scale"], drs_r, drs_b)
    dv["drs_bound"] = drs_b
    return dv


def expert_wgrads(t, e, got, ref, X, dY, wg, wr, dv, h_g, dgu_g, dgu_r, lora_rows=None):
    """Weight gradients of expert e from its rows (all of them)."""
    X, dY = f64(X), f64(dY)
    S_g, S_r = f64(s_rows(wg, dY)), f64(s_rows_oracle(wr, dY))
    if lora_rows is None:
        r = ref["dw_gu"][e]
        t["dw_gu"].add(got["dw_gu"][e], r, TB.b_wgrad(dv["dgu"], dgu_g, dgu_r, None, X, r))
        r = ref["dw_down"][e]
        t["dw_down"].add(got["dw_down"][e], r, TB.b_wgrad(S_g - S_r, S_g, S_r, dv["h"], h_g, r))
        return
    zg_g, zd_g, ug_g, ug_r, uw_g, uw_r = lora_rows
    r = ref["db_gu"][e]
    t["db_gu"].add(got["db_gu"][e], r, TB.b_wgrad(dv["dgu"], dgu_g, dgu_r, dv["z_gu"], zg_g, r))
    r = ref["da_gu"][e]
    t["da_gu"].add(got["da_gu"][e], r, TB.b_wgrad(dv["u_gu"], ug_g, ug_r, None, X, r))
    r = ref["db_dn"][e]
    t["db_dn"].add(got["db_dn"][e], r, TB.b_wgrad(S_g - S_r, S_g, S_r, dv["z_dn"], zd_g, r))
    r = ref["da_dn"][e]
    t["da_dn"].add(got["da_dn"][e], r, TB.b_wgrad(dv["uw_dn"], uw_g, uw_r, dv["h"], h_g, r))


def check_ffn(got, ref, xp, offsets, w_gu, w_down, wg, wr, dyp, lora=None, bwd=True, bf16=True,
              tag=""):
    """Grouped FFN forward (and backward) over rows sorted by expert.

    got / ref: dicts with the full row tensors (gu, h, y_perm, and dgu,
    dx_perm, d_row_scale, dw_gu, dw_down or the LoRA factor gradients);
    xp, dyp: the exact permuted rows; wg / wr: the row weights each side used
    (None: 1); lora: None or (a_gu, b_gu, a_dn, b_dn, scale).  Returns the
    observed deviations of Y_perm and dX_perm and the d_row_scale bound,
    row-indexed, for the routing checks."""
    E = w_gu.shape[0]
    R, d = xp.shape
    ones = np.ones(R, np.float32)
    wg = ones if wg is None else np.asarray(wg, np.float32)
    wr = ones if wr is None else np.asarray(wr, np.float32)
    t = Tallies(tag)
    names = (ROW_FWD + (LORA_FWD if lora else ())
             + ((ROW_BWD + (LORA_BWD if lora else ())) if bwd else ()))
    dev = {"y_perm": np.zeros((R, d), np.float32)}
    if bwd:
        dev["dx_perm"] = np.zeros((R, d), np.float32)
        dev["drs_bound"] = np.zeros(R, np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        sl = slice(a, b)
        gr = {n: got[n][sl] for n in names}
        rr = {n: ref[n][sl] for n in names}
        le = None if lora is None else tuple(v[e] for v in lora[:4]) + (lora[4],)
        dv = expert_rows(t, gr, rr, xp[sl], None if dyp is None else dyp[sl], w_gu[e], w_down[e],
                         wg[sl], wr[sl], le, bwd, bf16)
        dev["y_perm"][sl] = dv["y_perm"]
        if not bwd:
            continue
        dev["dx_perm"][sl] = dv["dx_perm"]
        dev["drs_bound"][sl] = dv["drs_bound"]
        lr = None
        if lora is not None:
            lr = (f64(gr["z_gu"]), f64(gr["z_dn"]), f64(gr["u_gu"]), f64(rr["u_gu"]),
                  f64(gr["uw_dn"]), f64(rr["uw_dn"]))
        expert_wgrads(t, e, got, ref, xp[sl], dyp[sl], wg[sl], wr[sl], dv, f64(gr["h"]),
                      f64(gr["dgu"]), f64(rr["dgu"]), lr)
    if bwd:
        counts = np.diff(np.asarray(offsets))
        grads = LORA_GRADS if lora is not None else ("dw_gu", "dw_down")
        for e in np.where(counts == 0)[0]:             # empty experts: exactly zero
            for n in grads:
                assert not np.any(got[n][e]), (n, e)
    t.finish()
    return dev


def check_tokens(g, o, b, a, k, dev, backward=True, bf16=True):
    """Token-level outputs: Y, and d_topk_w, d_logits, dW_r, dX."""
    T = a["x"].shape[0]
    s2r = np.asarray(o["slot_to_row"], np.int64).reshape(T, k)
    yp_g = f64(g["y_perm"])
    parts = [yp_g[s2r[:, j]] for j in range(k)]
    dparts = [dev["y_perm"][s2r[:, j]] for j in range(k)]
    close("y", g["y"], o["y"], bound=TB.b_sum_rows(g["y"], o["y"], parts, dparts, bf16=bf16))
    if not backward:
        return
    E = a["w_r"].shape[0]
    close("d_topk_w", g["d_topk_w"], b["d_topk_w"], bound=dev["drs_bound"][s2r])
    idx = np.asarray(o["topk_idx"], np.int64)
    bl = np.zeros((T, E))
    np.put_along_axis(bl, idx, TB.b_route_bwd(g["topk_w"], o["topk_w"], g["d_topk_w"],
                                              b["d_topk_w"]), axis=1)
    close("d_logits", g["d_logits"], b["d_logits"], bound=bl)
    ddl = f64(g["d_logits"]) - f64(b["d_logits"])
    X, Wr = f64(a["x"]), f64(a["w_r"])
    close("dw_r", g["dw_r"], b["dw_r"],
          bound=TB.b_wgrad(ddl, f64(g["d_logits"]), f64(b["d_logits"]), None, X, b["dw_r"]))
    dxp_g = f64(g["dx_perm"])
    parts = [dxp_g[s2r[:, j]] for j in range(k)]
    dparts = [dev["dx_perm"][s2r[:, j]] for j in range(k)]
    extra = TB.absdot(ddl, Wr) + (E + k) * TB.U32 * (np.abs(f64(g["d_logits"])) @ np.abs(Wr))
    close("dx", g["dx"], b["dx"], bound=TB.b_sum_rows(g["dx"], b["dx"], parts, dparts, extra))


def check_layer(g, o, b, a, k, backward=True, bf16=True, lora=None):
    """The whole block: g the device's tensors, o / b the oracle's forward and
    backward dicts (b None without backward), a the inputs."""
    close("topk_w", g["topk_w"], o["topk_w"], max_abs=1e-6, rel_l2=1e-6)
    ref = dict(o)
    if backward:
        ref.update(b)
    dev = check_ffn(g, ref, o["x_perm"], o["offsets"], a["w_gu"], a["w_down"], g["w_perm"],
                    o["w_perm"], b["dy_perm"] if backward else None, lora, backward, bf16)
    check_tokens(g, o, b, a, k, dev, backward, bf16)


def check_sampled_rows(g, rows, ref_rows, xp, dyp, offsets, w_gu, w_down, wg, wr, bwd=True):
    """Row checks on a sample of rows (any order, any experts): ref_rows holds
    the oracle's values for exactly those rows.  Returns row-indexed
    deviations (dicts keyed by the sampled row)."""
    rows = np.asarray(rows, np.int64)
    ex = O.expert_of_rows(offsets, rows)
    t = Tallies("")
    names = ROW_FWD + (ROW_BWD if bwd else ())
    out = {"y_perm": {}, "dx_perm": {}, "drs_bound": {}}
    for e in np.unique(ex):
        m = np.where(ex == e)[0]
        rr = rows[m]
        gr = {n: g[n][rr] for n in names}
        rf = {n: ref_rows[n][m] for n in names}
        dv = expert_rows(t, gr, rf, xp[rr], None if dyp is None else dyp[rr], w_gu[e],
                         w_down[e], np.asarray(wg)[rr], np.asarray(wr)[rr], None, bwd)
        for i, r_ in enumerate(rr):
            out["y_perm"][int(r_)] = dv["y_perm"][i]
            if bwd:
                out["dx_perm"][int(r_)] = dv["dx_perm"][i]
                out["drs_bound"][int(r_)] = dv["drs_bound"][i]
    t.finish()
    return out


def check_sampled_wgrad_cols(g_dw_gu_rows, g_dw_down_cols, e, cols, xp_e, dyp_e, w_gu, w_down,
                             wg_e, wr_e, dg_g, du_g, h_g, tag="", tallies=None):
    """Weight gradients of expert e at hidden units `cols`: the oracle forms
    them (and their operands) from only those columns; the bound carries the
    observed deviations of the device's stored dGU columns (dg_g gate, du_g
    up) and H columns (h_g), all over the expert's rows.  With `tallies`
    (a Tallies) the comparisons are added to its per-tensor tallies (one
    record over all the experts checked) instead of being finished here."""
    off = np.array([0, len(xp_e)])
    dg, du, dd, ops = O.weight_grads_sampled_cols(xp_e, off, w_gu[e:e + 1], w_down[e:e + 1],
                                                  wr_e, dyp_e, 0, cols, operands=True)
    X = f64(xp_e)
    dgg, dug, hg = f64(dg_g), f64(du_g), f64(h_g)
    S_g, S_r = f64(s_rows(wg_e, dyp_e)), ops["s"]
    checks = (("dw_gu[gate cols]", g_dw_gu_rows[0], dg,
               TB.b_wgrad(dgg - ops["dg"], dgg, ops["dg"], None, X, dg)),
              ("dw_gu[up cols]", g_dw_gu_rows[1], du,
               TB.b_wgrad(dug - ops["du"], dug, ops["du"], None, X, du)),
              ("dw_down[:, cols]", g_dw_down_cols, dd,
               TB.b_wgrad(S_g - S_r, S_g, S_r, hg - ops["h"], hg, dd)))
    for name, got, ref, bound in checks:
        if tallies is None:
            close(tag + name.replace("[", "[%d][" % e, 1), got, ref, bound=bound)
        else:
            tallies[name].add(got, ref, bound)
