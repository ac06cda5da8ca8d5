"""The expert-parallel decomposition on one GPU.

Sharded by expert, each rank owns a contiguous range of experts, receives
the rows routed to them (its slice of the expert-sorted rows) and runs the
grouped FFN on its local segments; the combine then brings the rows back to
their tokens ("Halo's 2.8x over TRL is not a kernel, and its own benchmark
proves it", section "Where the gap actually is", EP token-routing figure).
Here the ranks' shares run one after another on the one GPU: every share's
outputs and weight gradients must equal, bit for bit, the corresponding
slice of the whole block's, and the combine of the shares' rows must equal
the block's Y.  Each output element is accumulated in a fixed order
independent of how many experts a launch holds, so nothing may differ.
"""
import numpy as np
import pytest

from mixture_experts_layer_03_amd import inputs as I
from tests.gpu_util import down, need_gpu, up
from tests.test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

ROWS = ("gu", "h", "y_perm", "dgu", "dx_perm", "d_row_scale")


def _bits(t):
    a = down(t)
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype == np.float32 else np.uint8)


@pytest.mark.parametrize("w,P", [(SMALL[5], 4), (SMALL[1], 4), (I.GPTOSS, 8)],
                         ids=["T1024-E8-P4", "T512-E16-zipf-P4", "gpt-oss-20b-like-P8"])
def test_expert_ranges_reproduce_the_block(w, P):
    import torch
    from mixture_experts_layer_03_amd import abi
    from mixture_experts_layer_03_amd.layer import ExpertShare, MoEBlock
    dev = need_gpu()
    print("GPU case EP decomposition", w.name, "ranks", P, flush=True)
    a = I.make_inputs(w)
    x, wr, wgu, wd, dy = (up(a[n], True, dev) for n in ("x", "w_r", "w_gu", "w_down", "dy"))
    bias = None if a["bias"] is None else up(a["bias"], False, dev)
    noise = None if a["noise"] is None else up(a["noise"], False, dev)
    blk = MoEBlock(w.T, w.d, w.E, w.k, w.f, device=dev)
    blk.forward(x, wr, wgu, wd, bias, noise)
    blk.backward(x, wr, wgu, wd, dy)
    torch.cuda.synchronize()
    off = down(blk.offsets).astype(np.int64)
    assert w.E % P == 0
    per = w.E // P
    y_perm_all = torch.empty_like(blk.y_perm)
    for p in range(P):
        e0, e1 = p * per, (p + 1) * per
        r0, r1 = int(off[e0]), int(off[e1])
        n = r1 - r0
        loc = torch.from_numpy((off[e0:e1 + 1] - r0).astype(np.int32)).to(dev)
        sh = ExpertShare(n, w.d, per, w.f, device=dev)
        sh.forward(blk.x_perm[r0:r1], loc, wgu[e0:e1], wd[e0:e1], blk.w_perm[r0:r1])
        sh.backward(blk.x_perm[r0:r1], loc, wgu[e0:e1], wd[e0:e1], blk.w_perm[r0:r1],
                    blk.dy_perm[r0:r1])
        torch.cuda.synchronize()
        for name in ROWS:
            assert np.array_equal(_bits(getattr(sh, name)), _bits(getattr(blk, name)[r0:r1])), \
                (p, name)
        assert np.array_equal(_bits(sh.dw_gu), _bits(blk.dw_gu[e0:e1])), (p, "dw_gu")
        assert np.array_equal(_bits(sh.dw_down), _bits(blk.dw_down[e0:e1])), (p, "dw_down")
        y_perm_all[r0:r1] = sh.y_perm
        del sh
    # the combine of the ranks' rows is the block's output
    y = torch.empty_like(blk.y)
    abi.moe_combine(y_perm_all, blk.slot_to_row, w.T, w.k, y)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(blk.y))
