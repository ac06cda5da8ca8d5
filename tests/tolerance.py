"""Per-element error bounds for the GPU-vs-oracle parity checks.

The bound of every checked element is the literal one (max-abs 2e-2), widened
only by what the arithmetic of that element's own step explains:

  * rounding: a tensor stored in bf16 is rounded once on each side, so the two
    stored values may lie half a bf16 ulp of each (rounded) value apart from
    their unrounded sources;
  * propagation: the step's stored inputs are themselves compared with the
    oracle, element by element; the deviation they actually show is carried
    through the step exactly (|A_g B_g - A_r B_r| <= |A_g - A_r||B_g| +
    |A_r||B_g - B_r| for the sums, the exact difference of the elementwise
    function for SwiGLU and its adjoint);
  * accumulation: a sum of K products accumulated in fp32 (any order) is
    within LAM * sqrt(K) * u * sum|a b| of the exact sum with probability at
    least 1 - 2 exp(-LAM^2 / 2) (Higham and Mary's probabilistic rounding-error
    bound, u = 2^-24), and sum|a b| <= ||a|| ||b|| (Cauchy-Schwarz).

Every tensor's bound therefore rests on checks of its inputs, so a mistake in
any step shows up in that step's own check.  tests/test_tolerance_model.py
pins these bounds on the CPU: a second implementation of the block that
accumulates in fp32 stays inside them, and planted mistakes do not.
"""
import numpy as np

U32 = 2.0 ** -24      # fp32 unit roundoff
LAM = 6.0             # 2 exp(-18) ~ 3e-8 per sum


def f64(a):
    return np.asarray(a, np.float64)


def ulp_bf16(v):
    """Spacing of bf16 values at magnitude |v|, elementwise (0 at 0)."""
    v = np.abs(f64(v))
    out = np.zeros_like(v)
    nz = v > 0
    out[nz] = np.exp2(np.floor(np.log2(v[nz])) - 7)
    return out


def ulp_f32(v):
    """Spacing of fp32 values at magnitude |v|, elementwise."""
    return f64(np.spacing(np.abs(np.asarray(v, np.float32))))


def rounding(got, ref, bf16=True):
    """Both sides round their value to the storage type once (the oracle from
    fp64 through fp32)."""
    if not bf16:
        return 0.5 * (ulp_f32(got) + ulp_f32(ref)) + U32 * np.abs(f64(ref))
    return 0.5 * (ulp_bf16(got) + ulp_bf16(ref)) + U32 * np.abs(f64(ref))


def acc(K, na, nb):
    """fp32 accumulation allowance of sums of K products, outer product of the
    operand norms (na over the rows of the result, nb over its columns)."""
    return LAM * np.sqrt(max(int(K), 1)) * U32 * np.multiply.outer(f64(na), f64(nb))


def absdot(dA, B):
    """|dA| @ |B| where dA is mostly zero (the observed deviation of a stored
    operand)."""
    from scipy import sparse
    dA = np.abs(f64(dA))
    if not dA.any():
        return np.zeros((dA.shape[0], B.shape[1]))
    return np.asarray(sparse.csr_matrix(dA) @ np.abs(f64(B)))


def rownorm(a):
    return np.sqrt(np.sum(f64(a) ** 2, axis=-1))


def colnorm(a):
    return np.sqrt(np.sum(f64(a) ** 2, axis=0))


# --------------------------------------------------------------- SwiGLU and its adjoint

def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def swiglu(g, u):
    g, u = f64(g), f64(u)
    return g * _sig(g) * u


def dswiglu(g, u, dh):
    """(d/dg, d/du) of silu(g) u times dh."""
    g, u, dh = f64(g), f64(u), f64(dh)
    s = _sig(g)
    return dh * u * s * (1.0 + g * (1.0 - s)), dh * g * s


def eval_slack(v, g):
    """Error of evaluating SwiGLU (or its adjoint) in fp32 on the device: a
    few fp32 roundings, amplified by at most (1 + |g|)^2 through exp."""
    return 64.0 * U32 * np.abs(f64(v)) * (1.0 + np.abs(f64(g))) ** 2


# --------------------------------------------------------------- bounds per step

def b_gemm_rows(got, ref, rows_a, w_b, K, extra=None, bf16=True):
    """Stored output of one fp32 accumulation over K of exact operands:
    rows_a [M,K] rows of the left operand, w_b [N,K] rows of the right one."""
    b = rounding(got, ref, bf16) + acc(K, rownorm(rows_a), rownorm(w_b))
    return b if extra is None else b + extra


def b_h(h_g, h_r, gu_g, gu_r, f, bf16=True):
    """H = store(silu(g) u) from the stored g, u of each side."""
    gg, ug, gr, ur = gu_g[:, :f], gu_g[:, f:], gu_r[:, :f], gu_r[:, f:]
    return (rounding(h_g, h_r, bf16) + np.abs(swiglu(gg, ug) - swiglu(gr, ur))
            + eval_slack(h_r, gr) + eval_slack(h_g, gg))


def b_scaled_rows(got, ref, w_g, w_r, dIn, In_g, W, K, bf16=True):
    """store(w * (In W^T)) with the row weight w and a stored input In whose
    observed deviation is dIn: |dw| |In_r W^T| + w_g (|dIn| |W|^T + acc)."""
    ulp = ulp_bf16(ref) if bf16 else ulp_f32(ref)
    un_r = (np.abs(f64(ref)) + ulp) / np.maximum(f64(w_r), 1e-30)[:, None]
    return (rounding(got, ref, bf16) + np.abs(f64(w_g) - f64(w_r))[:, None] * un_r
            + f64(w_g)[:, None] * (absdot(dIn, W.T) + acc(K, rownorm(In_g), rownorm(W)))
            + 2 * U32 * np.abs(f64(ref)))


def b_dgu(dgu_g, dgu_r, gu_g, gu_r, w_g, w_r, gd_r, dgd, f):
    """dGU = store(dSwiGLU(g, u; w Gd)) from each side's stored g, u and row
    weight; Gd (fp32, not stored) is within dgd of the exact gd_r."""
    gg, ug, gr, ur = gu_g[:, :f], gu_g[:, f:], gu_r[:, :f], gu_r[:, f:]
    dg_g, du_g = dswiglu(gg, ug, f64(w_g)[:, None] * gd_r)
    dg_r, du_r = dswiglu(gr, ur, f64(w_r)[:, None] * gd_r)
    pg, pu = dswiglu(gg, ug, f64(w_g)[:, None] * dgd)       # sensitivity to Gd
    prop = np.concatenate([np.abs(dg_g - dg_r) + np.abs(pg), np.abs(du_g - du_r) + np.abs(pu)], 1)
    ev = np.concatenate([eval_slack(dg_r, gr), eval_slack(du_r, gr)], 1)
    return rounding(dgu_g, dgu_r) + prop + 2 * ev


def b_rowdot(dA, A_g, B_r, dB, K):
    """fp32 row dot sum_c A[r,c] B[r,c] with A stored (observed deviation dA)
    and B internal (exact B_r, bound dB on the device's deviation)."""
    return (np.sum(np.abs(f64(dA)) * np.abs(f64(B_r)), 1) + np.sum(np.abs(f64(A_g)) * f64(dB), 1)
            + LAM * np.sqrt(K) * U32 * rownorm(A_g) * (rownorm(B_r) + rownorm(dB)))


def b_wgrad(dA, A_g, A_r, dB, B_g, ref):
    """fp32 D = A^T B summed over the rows (K = rows): |dA|^T |B_g| + |A_r|^T
    |dB| + accumulation.  dB None: B is exact on both sides."""
    K = A_g.shape[0]
    b = absdot(f64(dA).T, B_g)
    if dB is not None:
        b += absdot(f64(dB).T, A_r).T
    return b + acc(K, colnorm(A_g), colnorm(B_g)) + 2 * U32 * np.abs(f64(ref))


def b_sum_rows(got, ref, parts_g, dparts, extra=None, bf16=True):
    """store(sum over j of fp32 parts[j]) (+ extra): rounding + the parts'
    deviations + fp32 additions."""
    n = len(parts_g)
    b = rounding(got, ref, bf16) + sum(np.abs(f64(p)) for p in dparts)
    b += n * U32 * sum(np.abs(f64(p)) for p in parts_g)
    return b if extra is None else b + extra


def b_route_bwd(tw_g, tw_r, g_g, g_r):
    """d_logits at the selected experts: w_j (g_j - sum_i w_i g_i) from each
    side's fp32 weights and row-scale gradients."""
    tw_g, tw_r, g_g, g_r = f64(tw_g), f64(tw_r), f64(g_g), f64(g_r)
    dw, dg = np.abs(tw_g - tw_r), np.abs(g_g - g_r)
    s_r = np.sum(tw_r * g_r, 1, keepdims=True)
    ds = np.sum(dw * np.abs(g_r) + np.abs(tw_g) * dg, 1, keepdims=True)
    k = tw_r.shape[1]
    ev = 4 * k * U32 * np.abs(tw_g) * (np.abs(g_g) + np.sum(np.abs(tw_g * g_g), 1, keepdims=True))
    return dw * np.abs(g_r - s_r) + np.abs(tw_g) * (dg + ds) + ev
