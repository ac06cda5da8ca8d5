"""The pins must catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of ``oracle/moe_oracle.py`` (a dropped
term, a wrong sign, a wrong index map, a misplaced rounding), loads the copy as
a separate module, and runs the pin tests against it: at least one must fail.
"""
import importlib.util
import os
import sys

import pytest

import tests.test_oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "moe_oracle.py")

MUTATIONS = [
    ("dropped dSiLU term", "dg = dh * u * sg * (1.0 + g * (1.0 - sg))", "dg = dh * u * sg"),
    ("wrong sign in softmax adjoint", "w * (g - s), axis=1)", "w * (g + s), axis=1)"),
    ("up gradient uses sigmoid instead of silu", "\n    du = dh * g * sg\n", "\n    du = dh * sg\n"),
    ("row weight not applied to the expert output",
     "y = _f64(wr)[:, None] * y\n    return gu, h, store(y, bf16)\n",
     "y = y\n    return gu, h, store(y, bf16)\n"),
    ("row weight missing from the down-projection weight gradient",
     "s = store(w[:, None] * _f64(dyr), bf16)\n    return dgu", "s = store(_f64(dyr), bf16)\n    return dgu"),
    ("combine gathers with the wrong map", "s2r = np.asarray(slot_to_row, dtype=np.int64).reshape(T, k)\n    acc = np.zeros((T, y_perm",
     "s2r = np.argsort(np.asarray(slot_to_row)).reshape(T, k)\n    acc = np.zeros((T, y_perm"),
    ("slots of one expert in descending order", 'row_to_slot = np.argsort(flat, kind="stable")',
     'row_to_slot = np.lexsort((-np.arange(flat.size), flat))'),
    ("ties resolved to the higher id", 'idx = np.argsort(-L, axis=1, kind="stable")[:, :k]',
     'idx = (L.shape[1] - 1 - np.argsort(-L[:, ::-1], axis=1, kind="stable"))[:, :k]'),
    ("softmax over all experts, not renormalised",
     "sel[:, :1])\n        w = ex / ex.sum(axis=1, keepdims=True)",
     "sel[:, :1])\n        w = ex / np.exp(L.astype(np.float64) - sel[:, :1]).sum(axis=1, keepdims=True)"),
    ("H not rounded to bf16", "h = store(silu(gu[:, :f]) * _f64(gu[:, f:]), bf16)",
     "h = np.asarray(silu(gu[:, :f]) * _f64(gu[:, f:]), np.float32)"),
    ("gate and up halves swapped", "h = store(silu(gu[:, :f]) * _f64(gu[:, f:]), bf16)",
     "h = store(silu(gu[:, f:]) * _f64(gu[:, :f]), bf16)"),
    ("router weight gradient scaled", "return (dl @ _f64(w_r)).astype(np.float32), (dl.T @ _f64(x))",
     "return (dl @ _f64(w_r)).astype(np.float32), (dl.T @ _f64(x) * 0.5)"),
    ("router gradient not added to dX", "acc += _f64(dx_add)", "pass"),
    ("selection bias leaks into the weights", "sel = _f64(np.take_along_axis(L, idx, axis=1))\n    ex = np.exp(sel - sel.max(",
     "sel = _f64(np.take_along_axis(score, idx, axis=1))\n    ex = np.exp(sel - sel.max("),
    ("selection bias ignored", "score = L + np.asarray(sel_bias, dtype=np.float32)[None, :]", "score = L"),
    ("bias update with the sign flipped", "np.sign(int(n_valid) * int(k) - E * ld)",
     "np.sign(E * ld - int(n_valid) * int(k))"),
    ("padded tail counted in the load", "np.bincount(idx[:n].ravel(), minlength=E)",
     "np.bincount(idx.ravel(), minlength=E)"),
    ("aux load fraction over tokens, not slots", "f = _f64(load) / (n * k)", "f = _f64(load) / n"),
    ("aux gradient without the softmax centring", "dl[:n] = p * (g[None, :] - s)", "dl[:n] = p * g[None, :]"),
    ("aux gradient not scaled by the coefficient", "g = coeff * E * f / n", "g = E * f / n"),
    ("LoRA dH gradient without the scale", "u_dn = store(scale * (_f64(dyr) @ _f64(b_dn[e])), bf16)",
     "u_dn = store((_f64(dyr) @ _f64(b_dn[e])), bf16)"),
    ("LoRA term missing from dX", "dx = store(_f64(dgu) @ _f64(w_gu[e]) + _f64(u_gu) @ _f64(a_gu[e]), bf16)",
     "dx = store(_f64(dgu) @ _f64(w_gu[e]), bf16)"),
    ("LoRA dA_dn without the row weight", "uw_dn = store(w[:, None] * _f64(u_dn), bf16)",
     "uw_dn = store(_f64(u_dn), bf16)"),
    ("LoRA dB_dn from dY instead of S", "(_f64(s_).T @ _f64(z_dn[a:b]))", "(_f64(dyr).T @ _f64(z_dn[a:b]))"),
    ("LoRA down term added after the row weight",
     "    y = _f64(h) @ _f64(w_down_e).T + _f64(z_dn) @ _f64(b_dn_e).T\n    if wr is not None:\n        y = _f64(wr)[:, None] * y\n    return gu, h, store(y, bf16), z_gu, z_dn",
     "    y = _f64(h) @ _f64(w_down_e).T\n    if wr is not None:\n        y = _f64(wr)[:, None] * y\n    y = y + _f64(z_dn) @ _f64(b_dn_e).T\n    return gu, h, store(y, bf16), z_gu, z_dn"),
    ("S not rounded to bf16", "s = store(w[:, None] * _f64(dyr), bf16)\n    return dgu",
     "s = w[:, None] * _f64(dyr)\n    return dgu"),
    ("H recomputed in the backward without its rounding",
     "h = store(silu(g) * u, bf16)                     # recomputed",
     "h = silu(g) * u                                  # recomputed"),
    ("dGU not rounded before dX and dW_gu",
     "dgu = store(np.concatenate([dg, du], axis=1), bf16)\n    dx = store(_f64(dgu) @ _f64(w_gu_e), bf16)",
     "dgu = np.concatenate([dg, du], axis=1)\n    dx = store(_f64(dgu) @ _f64(w_gu_e), bf16)"),
    ("LoRA z_gu not rounded", "z_gu = store(scale * (_f64(xr) @ _f64(a_gu_e).T), bf16)",
     "z_gu = scale * (_f64(xr) @ _f64(a_gu_e).T)"),
    ("LoRA z_dn not rounded", "z_dn = store(scale * (_f64(h) @ _f64(a_dn_e).T), bf16)",
     "z_dn = scale * (_f64(h) @ _f64(a_dn_e).T)"),
    ("LoRA u_dn not rounded", "u_dn = store(scale * (_f64(dyr) @ _f64(b_dn[e])), bf16)",
     "u_dn = scale * (_f64(dyr) @ _f64(b_dn[e]))"),
    ("LoRA u_gu not rounded", "u_gu = store(scale * (_f64(dgu) @ _f64(b_gu[e])), bf16)",
     "u_gu = scale * (_f64(dgu) @ _f64(b_gu[e]))"),
    ("LoRA row-weighted u_dn not rounded", "uw_dn = store(w[:, None] * _f64(u_dn), bf16)",
     "uw_dn = w[:, None] * _f64(u_dn)"),
    ("LoRA S not rounded", "s_ = store(w[:, None] * _f64(dyr), bf16)", "s_ = w[:, None] * _f64(dyr)"),
    ("LoRA dGU not rounded",
     "dgu = store(np.concatenate([dg, du], axis=1), bf16)\n        u_gu",
     "dgu = np.concatenate([dg, du], axis=1)\n        u_gu"),
]

PIN_TESTS = [
    lambda: P.test_topk_ties_and_closed_forms(),
    lambda: P.test_topk_matches_scan_and_softmax_sums_to_one(),
    lambda: P.test_permutation_is_stable_sort_by_expert(),
    lambda: P.test_combine_of_permute_identities(),
    lambda: P.test_forward_matches_dense_formulation_fp32(),
    lambda: P.test_forward_single_expert_is_dense_swiglu_with_bf16_storage(),
    lambda: P.test_backward_matches_torch_autograd_fp32((25, 8, 4, 4, 12)),
    lambda: P.test_backward_matches_torch_autograd_fp32((30, 16, 6, 2, 8)),
    lambda: P.test_backward_invariants(),
    lambda: P.test_route_biased_closed_forms(),
    lambda: P.test_route_biased_matches_scan_on_exact_scores(),
    lambda: P.test_expert_load_by_loops_and_bias_update_closed_forms(),
    lambda: P.test_aux_loss_closed_forms(),
    lambda: P.test_aux_loss_matches_loops_and_finite_differences(),
    lambda: P.test_lora_with_zero_b_is_the_plain_block(),
    lambda: P.test_lora_forward_is_the_merged_weight_block(),
    lambda: P.test_lora_gradients_match_torch_autograd(),
    lambda: P.test_expert_backward_storage_points_by_torch(61),
    lambda: P.test_lora_storage_points_by_torch(71),
]


def _load_mutant(old, new, tag):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    src = src.replace(old, new)
    name = "oracle._mutant_%d" % abs(hash(tag))
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__file__ = SRC
    exec(compile(src, SRC, "exec"), mod.__dict__)
    sys.modules[name] = mod
    return mod


@pytest.mark.parametrize("tag,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tag, old, new, monkeypatch):
    mutant = _load_mutant(old, new, tag)
    monkeypatch.setattr(P, "O", mutant)
    caught = False
    for run in PIN_TESTS:
        try:
            run()
        except Exception:
            caught = True
            break
    assert caught, "no pin caught: " + tag
