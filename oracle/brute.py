"""ORACLE pins -- test infrastructure only (imported by tests/ alone).

Independent formulations used to pin ``moe_oracle`` on tiny inputs.  None of
them shares code with ``moe_oracle``:

  * ``dense_forward``: every token goes through every expert (no sorting, no
    permutation, no segments); the expert outputs are then mixed with a gate
    matrix built from a full softmax over all experts, masked to the top-k and
    renormalised.  This is the "dense" reading of the same layer: the MoE layer
    of the pages computes exactly this, only faster.
  * ``topk_by_scan``: top-k by repeated scans over a Python list.
  * ``torch_dense_grads``: the dense formulation in torch fp64 with autograd,
    for the backward pass.
  * ``logits_exact``: the router logit fma chain evaluated with exact rational
    arithmetic and one correct rounding to fp32 per step.
  * ``route_biased_by_scan``: selection on exactly rounded fp32 scores L + b,
    weights from the full softmax of the unbiased logits, masked to the
    selection and renormalised.
  * ``aux_loss_by_loops``: expert load and mean router probability counted
    token by token in Python, combined into the auxiliary loss.
"""
from __future__ import annotations

from fractions import Fraction
import math

import numpy as np


def topk_by_scan(row, k):
    """k indices of the largest values; equal values -> lower index first."""
    vals = [float(v) for v in row]
    taken = [False] * len(vals)
    out = []
    for _ in range(k):
        best = -1
        for i, v in enumerate(vals):
            if taken[i]:
                continue
            if best < 0 or v > vals[best]:
                best = i
        taken[best] = True
        out.append(best)
    return out


def _silu(x):
    return x / (1.0 + np.exp(-x))


def dense_forward(x, w_r, w_gu, w_down, k, bias=None, noise=None, logits=None):
    """fp64 dense formulation.  If ``logits`` is given it is used for the routing
    decision (so that a near-tie resolved in fp32 is resolved the same way);
    the gate values always come from the fp64 softmax of those logits."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    E = w_r.shape[0]
    f = w_gu.shape[1] // 2
    if logits is None:
        L = x @ np.asarray(w_r, np.float64).T
        if bias is not None:
            L = L + np.asarray(bias, np.float64)[None, :]
        if noise is not None:
            L = L + np.asarray(noise, np.float64)
    else:
        L = np.asarray(logits, np.float64)
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)          # full softmax over all experts
    gate = np.zeros((T, E))
    sel = np.zeros((T, k), np.int64)
    for t in range(T):
        s = topk_by_scan(L[t], k)
        sel[t] = s
        gate[t, s] = p[t, s] / p[t, s].sum()        # renormalised over the selected
    y = np.zeros((T, d))
    for e in range(E):                              # every token through every expert
        gu = x @ np.asarray(w_gu[e], np.float64).T
        h = _silu(gu[:, :f]) * gu[:, f:]
        y += gate[:, e:e + 1] * (h @ np.asarray(w_down[e], np.float64).T)
    return {"logits": L, "gate": gate, "sel": sel, "y": y}


def torch_dense_grads(x, w_r, w_gu, w_down, dy, sel, bias=None, noise=None):
    """Gradients of sum(Y * dY) for the dense formulation with the selection
    fixed to ``sel`` [T,k], via torch fp64 autograd on the CPU."""
    import torch
    dt = torch.float64
    X = torch.tensor(np.asarray(x), dtype=dt, requires_grad=True)
    Wr = torch.tensor(np.asarray(w_r), dtype=dt, requires_grad=True)
    Wgu = torch.tensor(np.asarray(w_gu), dtype=dt, requires_grad=True)
    Wd = torch.tensor(np.asarray(w_down), dtype=dt, requires_grad=True)
    f = Wgu.shape[1] // 2
    L = X @ Wr.T
    if bias is not None:
        L = L + torch.tensor(np.asarray(bias), dtype=dt)[None, :]
    if noise is not None:
        L = L + torch.tensor(np.asarray(noise), dtype=dt)
    L.retain_grad()
    S = torch.tensor(np.asarray(sel), dtype=torch.int64)
    w = torch.softmax(torch.gather(L, 1, S), dim=1)
    outs = []
    for e in range(Wgu.shape[0]):
        gu = X @ Wgu[e].T
        h = torch.nn.functional.silu(gu[:, :f]) * gu[:, f:]
        outs.append(h @ Wd[e].T)
    O = torch.stack(outs, dim=1)                      # [T, E, d]
    Osel = torch.gather(O, 1, S[:, :, None].expand(-1, -1, O.shape[2]))
    Y = (w[:, :, None] * Osel).sum(dim=1)
    loss = (Y * torch.tensor(np.asarray(dy), dtype=dt)).sum()
    loss.backward()
    return {"y": Y.detach().numpy(), "dx": X.grad.numpy(), "dw_r": Wr.grad.numpy(),
            "dw_gu": Wgu.grad.numpy(), "dw_down": Wd.grad.numpy(), "d_logits": L.grad.numpy()}


def _round_fraction_to_f32(q: Fraction) -> float:
    """Correct round-to-nearest-even of an exact rational to IEEE binary32."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix e so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                                  # subnormal spacing floor
    scale = Fraction(2) ** (23 - e)                   # 24 significant bits
    m = a * scale
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n) / scale)


def logits_exact(x, w_r, bias=None, noise=None):
    """Router logit chain with every fma evaluated exactly and rounded once."""
    x = np.asarray(x, np.float32)
    w_r = np.asarray(w_r, np.float32)
    T, d = x.shape
    E = w_r.shape[0]
    out = np.zeros((T, E), np.float32)
    for t in range(T):
        for e in range(E):
            acc = 0.0
            for c in range(d):
                acc = _round_fraction_to_f32(Fraction(float(x[t, c])) * Fraction(float(w_r[e, c]))
                                             + Fraction(acc))
            if bias is not None:
                acc = _round_fraction_to_f32(Fraction(acc) + Fraction(float(bias[e])))
            if noise is not None:
                acc = _round_fraction_to_f32(Fraction(acc) + Fraction(float(noise[t, e])))
            out[t, e] = acc
    return out


def route_biased_by_scan(L, b, k):
    """Selection by the scores fp32(L + b) (each add exact, then rounded once),
    weights from the fp64 full softmax of L renormalised over the selection."""
    L = np.asarray(L, np.float32)
    T, E = L.shape
    idx = np.zeros((T, k), np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        score = [_round_fraction_to_f32(Fraction(float(L[t, e])) + Fraction(float(b[e])))
                 for e in range(E)]
        sel = topk_by_scan(score, k)
        m = max(float(v) for v in L[t])
        p = [math.exp(float(v) - m) for v in L[t]]
        z = sum(p)
        p = [v / z for v in p]
        ps = sum(p[e] for e in sel)
        idx[t] = sel
        w[t] = [p[e] / ps for e in sel]
    return idx, w


def aux_loss_by_loops(L, topk_idx, n_valid, k, coeff):
    """aux = E * sum_e (load_e / (n k)) * (mean_t p[t,e]) over the first n_valid
    tokens, by explicit loops; returns (aux, coeff * aux, load)."""
    L = np.asarray(L, np.float64)
    T, E = L.shape
    load = [0] * E
    psum = [0.0] * E
    for t in range(int(n_valid)):
        for j in range(k):
            load[int(topk_idx[t][j])] += 1
        m = max(L[t])
        ex = [math.exp(L[t, e] - m) for e in range(E)]
        z = sum(ex)
        for e in range(E):
            psum[e] += ex[e] / z
    if n_valid == 0:
        return 0.0, 0.0, load
    aux = 0.0
    for e in range(E):
        aux += (load[e] / (n_valid * k)) * (psum[e] / n_valid)
    aux *= E
    return aux, coeff * aux, load


def torch_dense_lora(x, w_gu, w_down, a_gu, b_gu, a_dn, b_dn, scale, gate, dy):
    """Dense formulation with LoRA-merged expert weights W + s B A, every
    token through every expert, mixed by the fixed gate matrix [T,E]; torch
    fp64 autograd for the gradients of sum(Y * dY) with respect to x and the
    LoRA factors (expert weights frozen).  Returns y and the gradients."""
    import torch
    dt = torch.float64
    X = torch.tensor(np.asarray(x), dtype=dt, requires_grad=True)
    Ag = torch.tensor(np.asarray(a_gu), dtype=dt, requires_grad=True)
    Bg = torch.tensor(np.asarray(b_gu), dtype=dt, requires_grad=True)
    Ad = torch.tensor(np.asarray(a_dn), dtype=dt, requires_grad=True)
    Bd = torch.tensor(np.asarray(b_dn), dtype=dt, requires_grad=True)
    Wg = torch.tensor(np.asarray(w_gu), dtype=dt)
    Wd = torch.tensor(np.asarray(w_down), dtype=dt)
    G = torch.tensor(np.asarray(gate), dtype=dt)
    f = Wg.shape[1] // 2
    Y = 0
    for e in range(Wg.shape[0]):
        wg = Wg[e] + scale * Bg[e] @ Ag[e]
        wd = Wd[e] + scale * Bd[e] @ Ad[e]
        gu = X @ wg.T
        h = torch.nn.functional.silu(gu[:, :f]) * gu[:, f:]
        Y = Y + G[:, e:e + 1] * (h @ wd.T)
    (Y * torch.tensor(np.asarray(dy), dtype=dt)).sum().backward()
    return {"y": Y.detach().numpy(), "dx": X.grad.numpy(), "da_gu": Ag.grad.numpy(),
            "db_gu": Bg.grad.numpy(), "da_dn": Ad.grad.numpy(), "db_dn": Bd.grad.numpy()}
