"""Helpers for the GPU parity tests: upload/download and the tolerance check."""
import numpy as np
import pytest

from mixture_experts_layer_03_amd import inputs as I

MAX_ABS = 2e-2     # max-abs error bound on floating-point outputs
REL_L2 = 5e-3      # relative L2 error bound on floating-point outputs


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    return torch.device("cuda:0")


def up(a, bf16, dev):
    import torch
    if a is None:
        return None
    if bf16:
        return torch.from_numpy(I.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)


def up_i32(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)


def down(t):
    import torch
    if t.dtype == torch.bfloat16:
        return I.bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy()


def ulp_bf16(v: float) -> float:
    """Spacing of bf16 values at magnitude v (8 significant bits)."""
    if v <= 0:
        return 0.0
    return 2.0 ** (np.floor(np.log2(v)) - 7)


def close(name, got, ref, max_abs=MAX_ABS, rel_l2=REL_L2, flip=False):
    """rel-L2 <= rel_l2 and max-abs <= max_abs.

    flip=True: the tensor is, or sums over, a bf16-stored intermediate that was
    accumulated in fp32.  Two correct implementations that sum in different
    orders store such a value one bf16 ulp apart whenever the exact value lies
    within their accumulation error of a rounding midpoint, so the max-abs
    bound becomes max(max_abs, one bf16 ulp at the tensor's largest
    magnitude); rel-L2 keeps its bound.  The literal figures and the number of
    elements beyond max_abs are printed either way."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.all(np.isfinite(got)), name + ": non-finite values"
    diff = np.abs(got - ref)
    err = float(np.max(diff))
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got))
    mref = float(np.max(np.abs(ref)))
    bound = max(max_abs, ulp_bf16(mref)) if flip else max_abs
    over = int(np.count_nonzero(diff > max_abs))
    msg = "%s: max-abs %.3e (bound %.3e%s), rel-L2 %.3e (bound %.1e), max|ref| %.3e, " \
          "elements > %.0e: %d of %d" % (name, err, bound, ", flip-aware" if flip else "", rel,
                                         rel_l2, mref, max_abs, over, diff.size)
    print(msg)
    assert err <= bound and rel <= rel_l2, msg
