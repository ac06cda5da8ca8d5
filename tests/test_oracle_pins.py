"""Pins of the oracle against things other than itself (CPU only).

Each test checks one part of ``oracle/moe_oracle.py`` against an independent
formulation (brute force, exact arithmetic, a library routine, torch autograd,
finite differences), a closed form, or an invariant the mathematics fixes.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute
from oracle import moe_oracle as O
from mixture_experts_layer_03_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _tiny(T=24, d=16, E=6, k=2, f=8, seed=0, bf16=False, bias=False, noise=False):
    w = I.Workload("t", T, d, E, k, f, "bf16" if bf16 else "fp32", True,
                   "zipf" if bias else ("noise" if noise else "uniform"), x_scale="unit", seed=seed)
    return w, I.make_inputs(w)


# ---------------------------------------------------------------- rounding

def test_bf16_rounding_matches_torch():
    import torch
    r = _rng(1)
    a = np.concatenate([
        r.standard_normal(20000).astype(np.float32) * 10.0,
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.0e38, 1e-40, -1e-41], np.float32),
        # exact ties: low 16 bits 0x8000 with even and odd kept lsb
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00008000], np.uint32).view(np.float32),
    ])
    ours = O.to_bf16(a)
    ref = torch.from_numpy(a.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(O.to_bf16(np.array([np.nan], np.float32)))[0]


def test_input_generator_is_seeded_and_bf16_exact():
    w, a = _tiny(bf16=True, seed=5)
    _, b = _tiny(bf16=True, seed=5)
    _, c = _tiny(bf16=True, seed=6)
    for key in ("x", "w_r", "w_gu", "w_down", "dy"):
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])
        assert np.array_equal(O.to_bf16(a[key]), a[key])


# ---------------------------------------------------------------- router logits

@pytest.mark.parametrize("bf16,bias,noise", [(False, False, False), (False, True, False),
                                              (True, False, True), (True, True, False)])
def test_router_logits_bit_exact_to_exact_arithmetic(bf16, bias, noise):
    w, a = _tiny(T=5, d=12, E=4, bf16=bf16, bias=bias, noise=noise, seed=11)
    got = O.router_logits(a["x"], a["w_r"], a["bias"], a["noise"])
    ref = brute.logits_exact(a["x"], a["w_r"], a["bias"], a["noise"])
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_router_logits_order_is_the_hidden_index_order():
    # bf16 inputs: every product is exact in fp32, so the chain equals a plain
    # fp32 multiply-then-add loop in hidden order; any other order differs
    # somewhere on this input.
    w, a = _tiny(T=64, d=256, E=8, bf16=True, seed=12)
    got = O.router_logits(a["x"], a["w_r"])
    acc = np.zeros((64, 8), np.float32)
    for c in range(256):
        acc = (acc + a["x"][:, c:c + 1] * a["w_r"][None, :, c]).astype(np.float32)
    assert np.array_equal(got, acc)
    rev = np.zeros((64, 8), np.float32)
    for c in reversed(range(256)):
        rev = (rev + a["x"][:, c:c + 1] * a["w_r"][None, :, c]).astype(np.float32)
    assert not np.array_equal(got, rev)
    ref = a["x"].astype(np.float64) @ a["w_r"].astype(np.float64).T
    assert np.max(np.abs(got - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref)))


# ---------------------------------------------------------------- top-k + softmax

def test_topk_matches_scan_and_softmax_sums_to_one():
    r = _rng(3)
    for E, k in [(8, 2), (32, 4), (128, 8), (5, 5), (1, 1), (16, 16)]:
        L = r.standard_normal((50, E)).astype(np.float32)
        L[::7] = np.round(L[::7])                      # many exact ties
        idx, w = O.route(L, k)
        for t in range(50):
            assert list(idx[t]) == brute.topk_by_scan(L[t], k)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
        assert np.all(np.diff(w, axis=1) <= 0)


def test_topk_ties_and_closed_forms():
    with open(os.path.join(GOLDEN, "routing_closed_forms.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        L = np.array(c["logits"], np.float32)
        if c.get("logits_expr") == "log3":
            L = np.array([[0.0, math.log(3.0), -5.0]], np.float32)
        idx, w = O.route(L, c["k"])
        assert idx.tolist() == c["topk_idx"], c["name"]
        np.testing.assert_allclose(w, np.array(c["topk_w"], np.float32), rtol=0, atol=c["atol"],
                                   err_msg=c["name"])


# ---------------------------------------------------------------- permutation

def _perm_by_loops(idx, E):
    flat = idx.ravel()
    s2r = np.full(flat.size, -1, np.int64)
    nxt = 0
    for e in range(E):
        for s in range(flat.size):
            if flat[s] == e:
                s2r[s] = nxt
                nxt += 1
    return s2r


def test_permutation_is_stable_sort_by_expert():
    r = _rng(4)
    for T, E, k in [(40, 8, 2), (33, 32, 4), (7, 3, 3), (0, 4, 2), (64, 1, 1)]:
        L = r.standard_normal((T, E)).astype(np.float32)
        idx, _ = O.route(L, k) if T else (np.zeros((0, k), np.int32), None)
        counts, offsets, s2r, r2s = O.permute_maps(idx, E)
        assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(s2r, _perm_by_loops(idx, E))
        assert np.array_equal(r2s[s2r], np.arange(T * k))       # bijection
        for e in range(E):
            rows = np.arange(offsets[e], offsets[e + 1])
            assert np.all(idx.ravel()[r2s[rows]] == e)
            assert np.all(np.diff(r2s[rows]) > 0)


def test_combine_of_permute_identities():
    r = _rng(5)
    T, d, E = 48, 24, 8
    x = O.to_bf16(r.standard_normal((T, d)).astype(np.float32))
    # (i) k = 1 with unit weights: exact identity
    idx, _ = O.route(r.standard_normal((T, E)).astype(np.float32), 1)
    _, _, s2r, r2s = O.permute_maps(idx, E)
    xp, _ = O.permute_rows(x, None, r2s, 1)
    assert np.array_equal(O.combine(xp, s2r, T, 1, True), x)
    # (ii) softmax weights (sum to one), rows scaled by their weight in bf16:
    #      the sum rounds back to x exactly
    for k in (2, 4, 8):
        idx, w = O.route(r.standard_normal((T, E)).astype(np.float32), k)
        _, _, s2r, r2s = O.permute_maps(idx, E)
        xp, wp = O.permute_rows(x, w, r2s, k)
        yp = O.to_bf16(wp[:, None].astype(np.float64) * xp)
        got = O.combine(yp, s2r, T, k, True)
        close = np.abs(got - x) <= 2.0 ** -7 * np.abs(x) + 1e-30
        assert close.all()
    # (iii) unweighted, k a power of two: exactly k * x
    for k in (2, 4):
        idx, _ = O.route(r.standard_normal((T, E)).astype(np.float32), k)
        _, _, s2r, r2s = O.permute_maps(idx, E)
        xp, _ = O.permute_rows(x, None, r2s, k)
        assert np.array_equal(O.combine(xp, s2r, T, k, True), (k * x).astype(np.float32))


# ---------------------------------------------------------------- forward

def test_forward_matches_dense_formulation_fp32():
    for seed, (T, d, E, k, f) in enumerate([(40, 16, 6, 2, 8), (31, 24, 8, 3, 16), (20, 8, 4, 4, 8)]):
        w, a = _tiny(T=T, d=d, E=E, k=k, f=f, seed=20 + seed, bias=(seed == 1))
        o = O.layer_forward(a["x"], a["w_r"], a["w_gu"], a["w_down"], k, a["bias"], a["noise"],
                            bf16=False)
        ref = brute.dense_forward(a["x"], a["w_r"], a["w_gu"], a["w_down"], k, a["bias"],
                                  a["noise"], logits=o["logits"])
        assert np.array_equal(o["topk_idx"], ref["sel"])
        scale = np.max(np.abs(ref["y"]))
        assert np.max(np.abs(o["y"] - ref["y"])) <= 1e-5 * scale
        # logits from fp64 dot agree closely with the fp32 chain
        ref2 = brute.dense_forward(a["x"], a["w_r"], a["w_gu"], a["w_down"], k, a["bias"], a["noise"])
        assert np.max(np.abs(ref2["logits"] - o["logits"])) < 1e-5


def test_forward_single_expert_is_dense_swiglu_with_bf16_storage():
    import torch
    r = _rng(6)
    T, d, f = 37, 32, 48
    x = O.to_bf16(r.standard_normal((T, d)).astype(np.float32))
    wgu = O.to_bf16((r.standard_normal((1, 2 * f, d)) / math.sqrt(d)).astype(np.float32))
    wd = O.to_bf16((r.standard_normal((1, d, f)) / math.sqrt(f)).astype(np.float32))
    wr = np.zeros((1, d), np.float32)
    o = O.layer_forward(x, wr, wgu, wd, 1, bf16=True)
    assert np.all(o["topk_w"] == 1.0)

    def bf(v):
        return torch.from_numpy(np.asarray(v, np.float64)).to(torch.float32).to(
            torch.bfloat16).to(torch.float64).numpy()

    X = x.astype(np.float64)
    g = bf(X @ wgu[0, :f].astype(np.float64).T)
    u = bf(X @ wgu[0, f:].astype(np.float64).T)
    h = bf(torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u)
    y = bf(h @ wd[0].astype(np.float64).T)
    assert np.array_equal(o["y"], y.astype(np.float32))
    assert np.array_equal(o["h"], h.astype(np.float32))


# ---------------------------------------------------------------- backward

def _fwd_bwd(a, k, bf16):
    o = O.layer_forward(a["x"], a["w_r"], a["w_gu"], a["w_down"], k, a["bias"], a["noise"], bf16=bf16)
    b = O.layer_backward(o, a["x"], a["w_r"], a["w_gu"], a["w_down"], a["dy"], k, bf16=bf16)
    return o, b


@pytest.mark.parametrize("shape", [(30, 16, 6, 2, 8), (25, 8, 4, 4, 12), (18, 12, 8, 1, 8)])
def test_backward_matches_torch_autograd_fp32(shape):
    T, d, E, k, f = shape
    w, a = _tiny(T=T, d=d, E=E, k=k, f=f, seed=40 + T, noise=True)
    o, b = _fwd_bwd(a, k, False)
    ref = brute.torch_dense_grads(a["x"], a["w_r"], a["w_gu"], a["w_down"], a["dy"], o["topk_idx"],
                                  a["bias"], a["noise"])
    for key, got in [("dx", b["dx"]), ("dw_r", b["dw_r"]), ("dw_gu", b["dw_gu"]),
                     ("dw_down", b["dw_down"]), ("d_logits", b["d_logits"])]:
        scale = max(1e-12, np.max(np.abs(ref[key])))
        err = np.max(np.abs(got - ref[key]))
        assert err <= 2e-5 * scale, (key, err, scale)


def test_backward_finite_differences_fp64_dense():
    # central differences of sum(Y*dY) on the fp64 dense formulation, for a few
    # entries of each weight, against the oracle's fp32-stored gradients
    T, d, E, k, f = 12, 8, 4, 2, 6
    w, a = _tiny(T=T, d=d, E=E, k=k, f=f, seed=77)
    o, b = _fwd_bwd(a, k, False)
    dy = a["dy"].astype(np.float64)

    def loss(**over):
        args = {n: a[n].astype(np.float64) for n in ("x", "w_r", "w_gu", "w_down")}
        args.update(over)
        ref = brute.dense_forward(args["x"], args["w_r"], args["w_gu"], args["w_down"], k,
                                  logits=None)
        assert np.array_equal(ref["sel"], o["topk_idx"])
        return np.sum(ref["y"] * dy)

    eps = 1e-6
    r = _rng(8)
    for name, grad in [("w_gu", b["dw_gu"]), ("w_down", b["dw_down"]), ("w_r", b["dw_r"]),
                       ("x", b["dx"])]:
        base = a[name].astype(np.float64)
        for _ in range(4):
            pos = tuple(int(r.integers(0, s)) for s in base.shape)
            p = base.copy(); p[pos] += eps
            m = base.copy(); m[pos] -= eps
            fd = (loss(**{name: p}) - loss(**{name: m})) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-4 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def test_backward_invariants():
    w, a = _tiny(T=64, d=16, E=8, k=2, f=8, seed=9, bias=True, bf16=True)
    o, b = _fwd_bwd(a, 2, True)
    # softmax Jacobian: each token's logit gradients sum to zero
    assert np.all(np.abs(b["d_logits"].astype(np.float64).sum(1))
                  <= 1e-6 * (1 + np.abs(b["d_logits"]).sum(1)))
    # unselected logits get exactly zero
    mask = np.ones_like(b["d_logits"], bool)
    np.put_along_axis(mask, o["topk_idx"].astype(np.int64), False, axis=1)
    assert np.all(b["d_logits"][mask] == 0)
    # empty experts have exactly zero weight gradients (the zipf bias leaves some)
    empty = np.where(o["counts"] == 0)[0]
    assert len(empty) > 0
    assert np.all(b["dw_gu"][empty] == 0) and np.all(b["dw_down"][empty] == 0)
    # d_row_scale is <dY_t, unscaled expert output row>
    e_of = O.expert_of_rows(o["offsets"], np.arange(len(o["w_perm"])))
    for r_ in range(0, len(e_of), 7):
        y_un = o["h"][r_].astype(np.float64) @ a["w_down"][e_of[r_]].astype(np.float64).T
        t = o["row_to_slot"][r_] // 2
        ref = np.dot(a["dy"][t].astype(np.float64), y_un)
        assert abs(ref - b["d_row_scale"][r_]) <= 1e-5 * (1 + abs(ref))
    # linearity in dY: doubling dY doubles every gradient exactly
    b2 = O.layer_backward(o, a["x"], a["w_r"], a["w_gu"], a["w_down"], 2 * a["dy"], 2, bf16=True)
    for key in ("dx", "dw_gu", "dw_down", "dw_r", "d_logits", "d_row_scale", "dx_perm", "dgu"):
        assert np.array_equal(b2[key], 2 * b[key]), key
    # stored activations are bf16 values; fp32 gradients are not all bf16 values
    for key in ("dx", "dgu", "dx_perm"):
        assert np.array_equal(O.to_bf16(b[key]), b[key])
    assert not np.array_equal(O.to_bf16(b["dw_gu"]), b["dw_gu"])


def test_bf16_rounding_points_stay_close_to_fp32_path():
    w, a = _tiny(T=48, d=32, E=4, k=2, f=32, seed=13, bf16=True)
    o1, b1 = _fwd_bwd(a, 2, True)
    o2, b2 = _fwd_bwd(a, 2, False)
    assert np.array_equal(o1["topk_idx"], o2["topk_idx"])
    for key, tol in [("y", 0.05), ("dx", 0.05), ("dw_gu", 0.05), ("dw_down", 0.05)]:
        src = o1 if key == "y" else b1
        ref = o2 if key == "y" else b2
        rel = np.linalg.norm(src[key] - ref[key]) / np.linalg.norm(ref[key])
        assert rel < tol, (key, rel)
        assert rel > 0


# ---------------------------------------------------------------- sampled variants

def test_sampled_variants_agree_with_full_oracle():
    w, a = _tiny(T=80, d=32, E=4, k=2, f=16, seed=14, bf16=True)
    o, b = _fwd_bwd(a, 2, True)
    rows = np.array([0, 3, 17, 50, 99, 159])
    gu, h, y = O.ffn_fwd_sampled_rows(o["x_perm"], o["offsets"], a["w_gu"], a["w_down"],
                                      o["w_perm"], rows)
    np.testing.assert_allclose(gu, o["gu"][rows], atol=1e-2)
    np.testing.assert_allclose(y, o["y_perm"][rows], atol=1e-2)
    dgu, dx, drs = O.ffn_bwd_sampled_rows(o["x_perm"], o["offsets"], a["w_gu"], a["w_down"],
                                          o["w_perm"], b["dy_perm"], rows)
    np.testing.assert_allclose(dgu, b["dgu"][rows], atol=1e-2)
    np.testing.assert_allclose(dx, b["dx_perm"][rows], atol=1e-2)
    np.testing.assert_allclose(drs, b["d_row_scale"][rows], rtol=1e-5, atol=1e-5)
    for e in range(4):
        cols = np.array([0, 5, 15])
        dg, du, dd = O.weight_grads_sampled_cols(o["x_perm"], o["offsets"], a["w_gu"], a["w_down"],
                                                 o["w_perm"], b["dy_perm"], e, cols)
        np.testing.assert_allclose(dg, b["dw_gu"][e][cols], rtol=1e-4, atol=1e-3)
        np.testing.assert_allclose(du, b["dw_gu"][e][16 + cols], rtol=1e-4, atol=1e-3)
        np.testing.assert_allclose(dd, b["dw_down"][e][:, cols], rtol=1e-4, atol=1e-3)


# ---------------------------------------------------------------- router variants

def _variants_golden():
    with open(os.path.join(GOLDEN, "router_variants_closed_forms.json")) as fh:
        return json.load(fh)


def test_route_biased_closed_forms():
    for c in _variants_golden()["route_biased"]:
        L = np.array(c["logits"], np.float32)
        idx, w = O.route_biased(L, np.array(c["sel_bias"], np.float32), c["k"])
        assert idx.tolist() == c["topk_idx"], c["name"]
        np.testing.assert_allclose(w, np.array(c["topk_w"], np.float32), rtol=0, atol=c["atol"],
                                   err_msg=c["name"])


def test_route_biased_matches_scan_on_exact_scores():
    r = _rng(11)
    for E, k in [(8, 2), (32, 4), (5, 5), (1, 1), (16, 3)]:
        L = r.standard_normal((40, E)).astype(np.float32)
        L[::5] = np.round(L[::5])                         # exact ties in the logits
        b = (r.standard_normal(E) * 0.7).astype(np.float32)
        b[::3] = np.round(b[::3])                         # and in the scores
        idx, w = O.route_biased(L, b, k)
        bidx, bw = brute.route_biased_by_scan(L, b, k)
        np.testing.assert_array_equal(idx, bidx)
        np.testing.assert_allclose(w, bw, rtol=0, atol=2e-7)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
        # the zero bias is plain top-k, bit for bit
        z_idx, z_w = O.route_biased(L, np.zeros(E, np.float32), k)
        p_idx, p_w = O.route(L, k)
        np.testing.assert_array_equal(z_idx, p_idx)
        np.testing.assert_array_equal(z_w, p_w)
    # a bias far above every logit gap forces its expert into every selection
    L = r.standard_normal((64, 8)).astype(np.float32)
    b = np.zeros(8, np.float32)
    b[5] = 100.0
    idx, _ = O.route_biased(L, b, 2)
    assert np.all(idx[:, 0] == 5)


def test_expert_load_by_loops_and_bias_update_closed_forms():
    for c in _variants_golden()["bias_update"]:
        idx = np.array(c["topk_idx"], np.int32)
        E = len(c["sel_bias"])
        load = O.expert_load(idx, E, c["n_valid"])
        assert load.tolist() == c["load"], c["name"]
        nb = O.bias_update(np.array(c["sel_bias"], np.float32), load, c["n_valid"], c["k"], c["rate"])
        assert nb.dtype == np.float32
        assert nb.tolist() == c["sel_bias_after"], c["name"]
    r = _rng(12)
    for E, k, T, n in [(8, 2, 50, 50), (32, 4, 64, 37), (6, 6, 9, 0), (128, 8, 40, 40)]:
        idx = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        load = O.expert_load(idx, E, n)
        by_loop = [0] * E
        for t in range(n):
            for j in range(k):
                by_loop[idx[t, j]] += 1
        assert load.tolist() == by_loop
        assert int(load.sum()) == n * k
        b = (r.standard_normal(E)).astype(np.float32)
        rate = 0.001
        nb = O.bias_update(b, load, n, k, rate)
        from fractions import Fraction
        mean = Fraction(n * k, E)
        for e in range(E):
            want = b[e] + (np.float32(rate) if load[e] < mean else
                           (-np.float32(rate) if load[e] > mean else np.float32(0.0)))
            assert nb[e] == np.float32(want)


def test_aux_loss_closed_forms():
    for c in _variants_golden()["aux_loss"]:
        L = np.array(c["logits"], np.float32)
        if c["name"].startswith("two experts"):
            L[0, 0] = np.float32(math.log(3.0))
        idx = np.array(c["topk_idx"], np.int32)
        E = L.shape[1]
        load = O.expert_load(idx, E, c["n_valid"])
        assert load.tolist() == c["load"], c["name"]
        aux, scaled, dl = O.aux_loss(L, load, c["n_valid"], c["k"], c["coeff"])
        tol = max(c["atol"], 1e-7)
        assert abs(aux - c["aux"]) <= tol, (c["name"], aux)
        assert abs(scaled - c["aux_scaled"]) <= tol, (c["name"], scaled)
        np.testing.assert_allclose(dl, np.array(c["d_logits"], np.float64), rtol=0, atol=tol,
                                   err_msg=c["name"])


def test_aux_loss_matches_loops_and_finite_differences():
    r = _rng(13)
    for E, k, T, n, coeff in [(8, 2, 30, 30, 0.01), (6, 3, 25, 17, 1.5), (32, 4, 40, 40, 0.1)]:
        L = (r.standard_normal((T, E)) * 1.5).astype(np.float32)
        idx, _ = O.route(L, k)
        load = O.expert_load(idx, E, n)
        aux, scaled, dl = O.aux_loss(L, load, n, k, coeff)
        baux, bscaled, bload = brute.aux_loss_by_loops(L, idx, n, k, coeff)
        assert load.tolist() == bload
        assert abs(aux - baux) <= 1e-12 * max(1.0, abs(baux))
        assert abs(scaled - bscaled) <= 1e-12 * max(1.0, abs(bscaled))
        # the gradient of coeff*aux w.r.t. the logits, with the load held fixed
        h = 1e-6
        Ld = L.astype(np.float64)
        for t in list(range(0, T, 3)):
            for e in range(E):
                Lp, Lm = Ld.copy(), Ld.copy()
                Lp[t, e] += h
                Lm[t, e] -= h
                fd = (O.aux_loss(Lp, load, n, k, coeff)[1] - O.aux_loss(Lm, load, n, k, coeff)[1]) / (2 * h)
                assert abs(fd - dl[t, e]) <= 1e-7 * max(1.0, coeff), (t, e, fd, dl[t, e])
        # softmax gradients sum to zero per token; the padded tail has none
        assert np.all(np.abs(dl.astype(np.float64).sum(1)) <= 1e-7)
        assert np.all(dl[n:] == 0)
        # statistics over the valid prefix do not see the tail
        aux2, _, dl2 = O.aux_loss(L[:n], load, n, k, coeff)
        assert aux2 == aux
        np.testing.assert_array_equal(dl2, dl[:n])


# ---------------------------------------------------------------- grouped LoRA

def _lora_case(T=40, d=24, E=5, k=2, f=16, r=8, seed=21, scale=0.5, zero_b=False):
    rng = _rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    w_r = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    w_gu = (rng.standard_normal((E, 2 * f, d)) / np.sqrt(d)).astype(np.float32)
    w_down = (rng.standard_normal((E, d, f)) / np.sqrt(f)).astype(np.float32)
    a_gu = (rng.standard_normal((E, r, d)) / np.sqrt(d)).astype(np.float32)
    b_gu = (rng.standard_normal((E, 2 * f, r)) * 0.3).astype(np.float32)
    a_dn = (rng.standard_normal((E, r, f)) / np.sqrt(f)).astype(np.float32)
    b_dn = (rng.standard_normal((E, d, r)) * 0.3).astype(np.float32)
    if zero_b:
        b_gu[:] = 0
        b_dn[:] = 0
    dy = rng.standard_normal((T, d)).astype(np.float32)
    L = O.router_logits(x, w_r)
    idx, tw = O.route(L, k)
    counts, offsets, s2r, r2s = O.permute_maps(idx, E)
    x_perm, w_perm = O.permute_rows(x, tw, r2s, k)
    return dict(x=x, w_gu=w_gu, w_down=w_down, a_gu=a_gu, b_gu=b_gu, a_dn=a_dn, b_dn=b_dn,
                dy=dy, idx=idx, tw=tw, offsets=offsets, s2r=s2r, r2s=r2s, x_perm=x_perm,
                w_perm=w_perm, scale=scale, T=T, k=k, E=E)


def _lora_run(c, bf16):
    gu, h, yp, zg, zd = O.expert_ffn_fwd_lora(c["x_perm"], c["offsets"], c["w_gu"], c["w_down"],
                                              c["w_perm"], c["a_gu"], c["b_gu"], c["a_dn"],
                                              c["b_dn"], c["scale"], bf16)
    y = O.combine(yp, c["s2r"], c["T"], c["k"], bf16)
    dyp = O.combine_bwd(c["dy"], c["s2r"], c["k"])
    b = O.expert_ffn_bwd_lora(c["x_perm"], gu, c["offsets"], c["w_gu"], c["w_down"], c["w_perm"],
                              dyp, c["a_gu"], c["b_gu"], c["a_dn"], c["b_dn"], c["scale"], zg, zd,
                              bf16)
    dx = O.permute_bwd(b["dx_perm"], c["s2r"], c["T"], c["k"], None, bf16)
    return dict(gu=gu, h=h, y_perm=yp, y=y, z_gu=zg, z_dn=zd, dx=dx, **b)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def test_lora_with_zero_b_is_the_plain_block():
    c = _lora_case(zero_b=True)
    for bf16 in (False, True):
        lo = _lora_run(c, bf16)
        gu, h, yp = O.expert_ffn_fwd(c["x_perm"], c["offsets"], c["w_gu"], c["w_down"],
                                     c["w_perm"], bf16)
        np.testing.assert_array_equal(lo["gu"], gu)
        np.testing.assert_array_equal(lo["y_perm"], yp)
        dyp = O.combine_bwd(c["dy"], c["s2r"], c["k"])
        pb = O.expert_ffn_bwd(c["x_perm"], gu, c["offsets"], c["w_gu"], c["w_down"], c["w_perm"],
                              dyp, bf16)
        for n in ("dgu", "dx_perm", "d_row_scale"):
            np.testing.assert_array_equal(lo[n], pb[n])
        assert not lo["da_gu"].any() and not lo["da_dn"].any()      # no path through B = 0
        assert lo["db_gu"].any() and lo["db_dn"].any()


def test_lora_forward_is_the_merged_weight_block():
    c = _lora_case()
    lo = _lora_run(c, False)
    s = c["scale"]
    wg = (c["w_gu"].astype(np.float64) + s * c["b_gu"].astype(np.float64) @ c["a_gu"].astype(np.float64))
    wd = (c["w_down"].astype(np.float64) + s * c["b_dn"].astype(np.float64) @ c["a_dn"].astype(np.float64))
    gu, h, yp = O.expert_ffn_fwd(c["x_perm"], c["offsets"], wg, wd, c["w_perm"], False)
    assert _rel(lo["gu"], gu) < 1e-6 and _rel(lo["y_perm"], yp) < 1e-6


def test_lora_gradients_match_torch_autograd():
    c = _lora_case()
    lo = _lora_run(c, False)
    T, E, k = c["T"], c["E"], c["k"]
    gate = np.zeros((T, E))
    np.put_along_axis(gate, c["idx"].astype(np.int64), c["tw"].astype(np.float64), axis=1)
    ref = brute.torch_dense_lora(c["x"], c["w_gu"], c["w_down"], c["a_gu"], c["b_gu"], c["a_dn"],
                                 c["b_dn"], c["scale"], gate, c["dy"])
    assert _rel(lo["y"], ref["y"]) < 1e-6
    for n in ("dx", "da_gu", "db_gu", "da_dn", "db_dn"):
        assert _rel(lo[n], ref[n]) < 1e-5, (n, _rel(lo[n], ref[n]))


# ---------------------------------------------------------------- storage points, rebuilt in torch
#
# One expert with row weights in (0, 1), rebuilt with torch: fp64 matmuls,
# torch's own fp32 -> bf16 conversion at exactly the block's storage points,
# and the SwiGLU adjoint from torch autograd.  Stored bf16 tensors must be
# equal; fp32 gradients within one fp32 ulp.  Dropping any one rounding moves
# a stored tensor by a bf16 ulp somewhere or a gradient by ~1e-3 relative.

def _t64(v):
    import torch
    return torch.from_numpy(np.asarray(v, np.float64).copy())


def _tbf(v):
    """torch's rounding to bf16 (through fp32), back in fp64."""
    import torch
    return v.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _swiglu_adjoint(g, u, dh):
    import torch
    g = g.clone().requires_grad_(True)
    u = u.clone().requires_grad_(True)
    h = torch.nn.functional.silu(g) * u
    dg, du = torch.autograd.grad(h, (g, u), dh)
    return dg.detach(), du.detach()


def _one_expert(seed, M=45, d=40, f=24, r=None):
    rng = _rng(seed)
    c = dict(
        x=O.to_bf16(rng.standard_normal((M, d)).astype(np.float32)),
        w_gu=O.to_bf16((rng.standard_normal((1, 2 * f, d)) / np.sqrt(d)).astype(np.float32)),
        w_down=O.to_bf16((rng.standard_normal((1, d, f)) / np.sqrt(f)).astype(np.float32)),
        dy=O.to_bf16(rng.standard_normal((M, d)).astype(np.float32)),
        w=(rng.random(M, dtype=np.float32) * 0.9 + 0.05).astype(np.float32),
        off=np.array([0, M], np.int32), f=f)
    if r is not None:
        c["a_gu"] = O.to_bf16((rng.standard_normal((1, r, d)) / np.sqrt(d)).astype(np.float32))
        c["b_gu"] = O.to_bf16((rng.standard_normal((1, 2 * f, r)) * 0.4).astype(np.float32))
        c["a_dn"] = O.to_bf16((rng.standard_normal((1, r, f)) / np.sqrt(f)).astype(np.float32))
        c["b_dn"] = O.to_bf16((rng.standard_normal((1, d, r)) * 0.4).astype(np.float32))
        c["scale"] = 0.75
    return c


def _same_stored(name, got, ref):
    ref = ref.numpy().astype(np.float32)
    assert np.array_equal(np.asarray(got, np.float32), ref), (
        name, int(np.count_nonzero(np.asarray(got, np.float32) != ref)))


def _same_fp32(name, got, ref):
    ref = ref.numpy()
    got = np.asarray(got, np.float64)
    tol = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= tol), (name, float(np.max(np.abs(got - ref))))


@pytest.mark.parametrize("seed", [61, 62])
def test_expert_backward_storage_points_by_torch(seed):
    import torch
    c = _one_expert(seed)
    f = c["f"]
    gu_o, h_o, y_o = O.expert_ffn_fwd(c["x"], c["off"], c["w_gu"], c["w_down"], c["w"], True)
    b = O.expert_ffn_bwd(c["x"], gu_o, c["off"], c["w_gu"], c["w_down"], c["w"], c["dy"], True)
    X, Wg, Wd, dY, w = (_t64(c[n]) for n in ("x", "w_gu", "w_down", "dy", "w"))
    Wg, Wd, w = Wg[0], Wd[0], w[:, None]
    gu = _tbf(X @ Wg.T)
    g, u = gu[:, :f], gu[:, f:]
    h = _tbf(torch.nn.functional.silu(g) * u)
    y = _tbf(w * (h @ Wd.T))
    _same_stored("gu", gu_o, gu)
    _same_stored("h", h_o, h)
    _same_stored("y_perm", y_o, y)
    gd = dY @ Wd                                   # d(loss)/d(w * h W_down^T) pulled to h
    drs = (h * gd).sum(1)
    dg, du = _swiglu_adjoint(g, u, w * gd)
    dgu = _tbf(torch.cat([dg, du], 1))
    dx = _tbf(dgu @ Wg)
    S = _tbf(w * dY)                               # the row-weighted upstream gradient, stored
    _same_stored("dgu", b["dgu"], dgu)
    _same_stored("dx_perm", b["dx_perm"], dx)
    _same_fp32("d_row_scale", b["d_row_scale"], drs)
    _same_fp32("dw_down", b["dw_down"][0], S.T @ h)
    _same_fp32("dw_gu", b["dw_gu"][0], dgu.T @ X)


@pytest.mark.parametrize("seed", [71, 72])
def test_lora_storage_points_by_torch(seed):
    import torch
    c = _one_expert(seed, r=8)
    f, s = c["f"], c["scale"]
    gu_o, h_o, y_o, zg_o, zd_o = O.expert_ffn_fwd_lora(
        c["x"], c["off"], c["w_gu"], c["w_down"], c["w"], c["a_gu"], c["b_gu"], c["a_dn"],
        c["b_dn"], s, True)
    b = O.expert_ffn_bwd_lora(c["x"], gu_o, c["off"], c["w_gu"], c["w_down"], c["w"], c["dy"],
                              c["a_gu"], c["b_gu"], c["a_dn"], c["b_dn"], s, zg_o, zd_o, True)
    X, Wg, Wd, dY, w = (_t64(c[n]) for n in ("x", "w_gu", "w_down", "dy", "w"))
    Ag, Bg, Ad, Bd = (_t64(c[n])[0] for n in ("a_gu", "b_gu", "a_dn", "b_dn"))
    Wg, Wd, w = Wg[0], Wd[0], w[:, None]
    # forward: the rank-r activations are stored, the products join the accumulation
    z_gu = _tbf(s * (X @ Ag.T))
    gu = _tbf(X @ Wg.T + z_gu @ Bg.T)
    g, u = gu[:, :f], gu[:, f:]
    h = _tbf(torch.nn.functional.silu(g) * u)
    z_dn = _tbf(s * (h @ Ad.T))
    y = _tbf(w * (h @ Wd.T + z_dn @ Bd.T))
    for n, got, ref in (("z_gu", zg_o, z_gu), ("gu", gu_o, gu), ("h", h_o, h),
                        ("z_dn", zd_o, z_dn), ("y_perm", y_o, y)):
        _same_stored(n, got, ref)
    # backward with frozen experts
    u_dn = _tbf(s * (dY @ Bd))
    gd = dY @ Wd + u_dn @ Ad
    dg, du = _swiglu_adjoint(g, u, w * gd)
    dgu = _tbf(torch.cat([dg, du], 1))
    u_gu = _tbf(s * (dgu @ Bg))
    dx = _tbf(dgu @ Wg + u_gu @ Ag)
    S = _tbf(w * dY)
    wu_dn = _tbf(w * u_dn)                         # the row-weighted u_dn, stored like S
    for n, got, ref in (("u_dn", b["u_dn"], u_dn), ("dgu", b["dgu"], dgu),
                        ("u_gu", b["u_gu"], u_gu), ("dx_perm", b["dx_perm"], dx)):
        _same_stored(n, got, ref)
    _same_fp32("d_row_scale", b["d_row_scale"], (h * gd).sum(1))
    _same_fp32("db_gu", b["db_gu"][0], dgu.T @ z_gu)
    _same_fp32("da_gu", b["da_gu"][0], u_gu.T @ X)
    _same_fp32("db_dn", b["db_dn"][0], S.T @ z_dn)
    _same_fp32("da_dn", b["da_dn"][0], wu_dn.T @ h)


def test_topk_order_with_nan_and_infinities():
    """NaN ranks below every number (NaNs by id); +-inf order as numbers;
    -0 ties +0.  Checked against a plain selection loop with that order."""
    inf, nan = np.inf, np.nan
    L = np.array([[1.0, nan, -inf, 2.0, nan, 0.5],
                  [nan, nan, nan, nan, 1.0, nan],
                  [-0.0, 0.0, -inf, -inf, nan, -1.0],
                  [inf, 3.0, nan, inf, -inf, 0.0]], np.float32)

    def key(v, e):                      # larger key = better
        return (0, 0.0, -e) if np.isnan(v) else (1, float(v), -e)

    for k in (1, 2, 3, 4, 6):
        idx, w = O.route(L, k)
        for t in range(L.shape[0]):
            order = sorted(range(L.shape[1]), key=lambda e: key(L[t, e], e), reverse=True)
            assert idx[t].tolist() == order[:k], (t, k)
            sel = L[t, order[:k]]
            if np.isnan(sel).any() or sel[0] == inf:
                assert np.isnan(w[t]).all()
            else:
                assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 1e-6
