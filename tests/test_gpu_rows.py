"""GPU: the row kernels -- forward permute rows, combine, combine backward and
permute backward -- against their definitions, bit for bit.

Copies are exact; the sums are fp32 additions in ascending j (a dropped slot
skipped) followed by one rounding to the stored dtype, recomputed here in
numpy.  The cases cover top-k 1..9 (k <= 8 with at most two rounds of
one-wave-per-piece units takes the persistent pipelined kernels; k = 9, the
permute backward's added term and larger inputs the one-wave-per-piece
ones), row widths that leave partial pieces and chunks, dropped slots
(expert id outside [0, E)), fp32 rows, and enough units that each wave of the
persistent grid walks several loop trips, ending on either half of one.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.gpu_util import down, need_gpu, up, up_i32

pytestmark = pytest.mark.gpu

CASES = [   # T, d, k, dtype, fraction of dropped slots
    (1, 8, 1, "bf16", 0.0),
    (37, 72, 3, "bf16", 0.1),
    (300, 328, 4, "bf16", 0.1),
    (257, 2880, 4, "bf16", 0.0),
    (129, 136, 5, "bf16", 0.1),
    (64, 2048, 8, "bf16", 0.1),
    (50, 64, 9, "bf16", 0.1),
    (97, 200, 4, "fp32", 0.1),
    (33, 48, 7, "fp32", 0.0),
    (2000, 24, 2, "bf16", 0.05),
    (16384, 256, 4, "bf16", 0.0),
    (5000, 520, 6, "bf16", 0.02),
    (9001, 1000, 6, "bf16", 0.02),
]


def _ids(c):
    return "T%d-d%d-k%d-%s-drop%g" % c


def _maps(idx, E):
    """Rows of the valid slots ordered by expert, then slot; a slot whose expert
    id is outside [0, E) gets no row (-1).  Without such slots these are the
    oracle's maps."""
    flat = idx.ravel().astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    order = np.argsort(np.where(valid, flat, E), kind="stable")
    n = int(valid.sum())
    s2r = np.full(flat.size, -1, np.int64)
    s2r[order[:n]] = np.arange(n)
    counts = np.bincount(flat[valid], minlength=E)[:E]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    if n == flat.size:
        oc, oo, os2r, _ = O.permute_maps(idx, E)
        assert np.array_equal(oc, counts) and np.array_equal(oo, offsets)
        assert np.array_equal(os2r, s2r)
    return counts, offsets, s2r, order[:n]


def _seq_sum(rows, s2r, T, k, add=None):
    """fp32 sum over j ascending of rows[s2r[t, j]] (s2r < 0 skipped), then add."""
    acc = np.zeros((T, rows.shape[1]), np.float32)
    s2r = s2r.reshape(T, k)
    for j in range(k):
        m = s2r[:, j] >= 0
        acc[m] = acc[m] + rows[s2r[m, j]]
    if add is not None:
        acc = acc + add
    return acc


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_row_kernels_match_their_definitions(case):
    import torch
    from mixture_experts_layer_03_amd import abi
    dev = need_gpu()
    T, d, k, dt, drop = case
    bf = dt == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32
    E = k + 3
    print("GPU rows case", _ids(case), flush=True)
    rng = np.random.default_rng(1000 + T + d + k)
    # distinct experts per token, some slots dropped
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    idx[rng.random((T, k)) < drop] = -1
    w = rng.random((T, k)).astype(np.float32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    if bf:
        x = O.to_bf16(x)
    R = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    s2r_t = torch.empty(R, dtype=torch.int32, device=dev)
    r2s_t = torch.empty(R, dtype=torch.int32, device=dev)
    x_perm = torch.zeros((R, d), dtype=tdt, device=dev)
    w_perm = torch.zeros(R, dtype=torch.float32, device=dev)
    ws = torch.empty(abi.moe_permute_workspace_size(T, E, k), dtype=torch.uint8, device=dev)
    abi.moe_permute(up(x, bf, dev), up_i32(idx, dev), up(w, False, dev), T, d, E, k, counts,
                    offsets, s2r_t, r2s_t, x_perm, w_perm, ws)
    torch.cuda.synchronize()
    c_ref, o_ref, s2r, r2s = _maps(idx, E)
    assert np.array_equal(down(counts), c_ref)
    assert np.array_equal(down(offsets), o_ref)
    assert np.array_equal(down(s2r_t), s2r)
    n = int(o_ref[-1])
    xp_ref, wp_ref = O.permute_rows(x, w, r2s, k)
    assert np.array_equal(down(x_perm)[:n], xp_ref)
    assert np.array_equal(down(w_perm)[:n], wp_ref)

    # combine bwd: a copy of dY[t] into each of the token's rows
    dy = rng.standard_normal((T, d)).astype(np.float32)
    if bf:
        dy = O.to_bf16(dy)
    dy_perm = torch.zeros((R, d), dtype=tdt, device=dev)
    abi.moe_combine_bwd(up(dy, bf, dev), s2r_t, k, dy_perm)
    # combine and permute bwd: sums over the token's rows
    y_perm = rng.standard_normal((R, d)).astype(np.float32)
    if bf:
        y_perm = O.to_bf16(y_perm)
    add = rng.standard_normal((T, d)).astype(np.float32)
    y = torch.empty((T, d), dtype=tdt, device=dev)
    dx = torch.empty((T, d), dtype=tdt, device=dev)
    dx_add = torch.empty((T, d), dtype=tdt, device=dev)
    yp = up(y_perm, bf, dev)
    abi.moe_combine(yp, s2r_t, T, k, y)
    abi.moe_permute_bwd(yp, s2r_t, None, T, k, dx)
    abi.moe_permute_bwd(yp, s2r_t, up(add, False, dev), T, k, dx_add)
    torch.cuda.synchronize()

    keep = s2r >= 0
    got = down(dy_perm)
    assert np.array_equal(got[s2r[keep]], np.repeat(dy, k, axis=0)[keep])
    ref = _seq_sum(y_perm, s2r, T, k)
    ref = O.to_bf16(ref) if bf else ref
    assert np.array_equal(down(y), ref)
    assert np.array_equal(down(dx), ref)
    ref_add = _seq_sum(y_perm, s2r, T, k, add)
    ref_add = O.to_bf16(ref_add) if bf else ref_add
    assert np.array_equal(down(dx_add), ref_add)
