"""Seeded synthetic inputs for the MoE expert block.

This module only draws random numbers and stores them; it holds none of the
block's arithmetic (no routing, no GEMM, no activation).  Both the oracle
(under ``oracle/``) and the HIP path are fed from the arrays it returns, so the
two sides never share anything else.

Workload shapes follow the pages:
  * gpt-oss-20b: 32 experts, top-4 (the EP token-routing figure in "Halo's 2.8x
    over TRL is not a kernel, and its own benchmark proves it", section
    "Where the gap actually is"); hidden size and expert width 2880.
  * Qwen3-30B-A3B: 128 experts (the Qwen3 row of "Halo: Frontier-Lab Training
    for Everyone", section "Halo vs. stock TRL"); top-8, hidden 2048, width 768.
The pages benchmark on a synthetic fixed-shape fixture rather than a dataset
("What stock TRL was configured as"); these generators play that role.

Draw order (fixed, so a seed names one input set):
  X, W_r, W_gu, W_down, dY, bias or noise, counts, w_perm.
Every tensor is drawn in fp32; for bf16 workloads it is then rounded to the
nearest bf16 (ties to even) so that the fp32 host copy is exactly the bf16
value the device sees.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (for the pre-routed EP-rank share: routed rows)
    d: int            # d_model
    E: int            # experts
    k: int            # top-k (1 for the pre-routed share)
    f: int            # d_ff (expert width)
    dtype: str        # "fp32" or "bf16"
    backward: bool    # whether the workload includes the backward pass
    routing: str      # "uniform", "zipf", "noise", "prerouted"
    x_scale: str = "unit"   # "unit": X ~ N(0,1); "fan_in": X ~ N(0,1)/sqrt(d)
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k if self.routing != "prerouted" else self.T


# The five workloads of the measurement plan.  Seeds are 1000 + number.
TINY = Workload("tiny-fp32-T256-d128-E8-k2-f256", 256, 128, 8, 2, 256, "fp32",
                False, "uniform", x_scale="fan_in", seed=1001)
GPTOSS = Workload("gpt-oss-20b-like-T4096-d2880-E32-k4-f2880", 4096, 2880, 32, 4, 2880,
                  "bf16", True, "uniform", seed=1002)
GPTOSS_SKEW = Workload("gpt-oss-20b-like-zipf-T16384-d2880-E32-k4-f2880", 16384, 2880, 32, 4,
                       2880, "bf16", True, "zipf", seed=1003)
EP8_SHARE = Workload("ep8-rank-share-rows8192-d2880-E4-f2880", 8192, 2880, 4, 1, 2880, "bf16",
                     True, "prerouted", seed=1004)
QWEN3 = Workload("qwen3-30b-a3b-like-T32768-d2048-E128-k8-f768", 32768, 2048, 128, 8, 768,
                 "bf16", True, "noise", seed=1005)

WORKLOADS = {w.name: w for w in (TINY, GPTOSS, GPTOSS_SKEW, EP8_SHARE, QWEN3)}
BY_KEY = {"c1": TINY, "c2": GPTOSS, "c3": GPTOSS_SKEW, "c4": EP8_SHARE, "c5": QWEN3}


def scaled(w: Workload, **changes) -> Workload:
    """Same recipe at other sizes (parity cases that the oracle finishes fast)."""
    return dataclasses.replace(w, name=w.name + "-scaled", **changes)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even), returned as fp32.  Input preparation only."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC00000
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-exact (device storage)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode bf16 storage (uint16) to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape, scale: float, bf16: bool) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return round_to_bf16(a) if bf16 else a


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one input set for workload ``w``.

    Returned keys (fp32 host arrays; bf16-exact for bf16 workloads):
      routed workloads: x[T,d], w_r[E,d], w_gu[E,2f,d] (gate rows then up rows),
        w_down[E,d,f], dy[T,d] (if backward), bias[E] or None, noise[T,E] or None
      pre-routed share: x_perm[R,d], w_gu, w_down, dy_perm[R,d], counts[E] int64,
        w_perm[R] fp32 in the open interval (0,1)
    """
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    bf16 = w.dtype == "bf16"
    T, d, E, f = w.T, w.d, w.E, w.f
    out: Dict[str, np.ndarray] = {}
    xs = 1.0 / math.sqrt(d) if w.x_scale == "fan_in" else 1.0
    if w.routing == "prerouted":
        out["x_perm"] = _normal(rng, (T, d), xs, bf16)
        out["w_gu"] = _normal(rng, (E, 2 * f, d), 1.0 / math.sqrt(d), bf16)
        out["w_down"] = _normal(rng, (E, d, f), 1.0 / math.sqrt(f), bf16)
        out["dy_perm"] = _normal(rng, (T, d), 1.0, bf16)
        p = rng.dirichlet(np.full(E, 2.0))
        out["counts"] = rng.multinomial(T, p).astype(np.int64)
        wp = rng.random(T, dtype=np.float32)
        while (wp == 0).any():
            z = wp == 0
            wp[z] = rng.random(int(z.sum()), dtype=np.float32)
        out["w_perm"] = wp
        return out
    out["x"] = _normal(rng, (T, d), xs, bf16)
    out["w_r"] = _normal(rng, (E, d), 1.0 / math.sqrt(d), bf16)
    out["w_gu"] = _normal(rng, (E, 2 * f, d), 1.0 / math.sqrt(d), bf16)
    out["w_down"] = _normal(rng, (E, d, f), 1.0 / math.sqrt(f), bf16)
    out["dy"] = _normal(rng, (T, d), 1.0, bf16) if w.backward else None
    out["bias"] = None
    out["noise"] = None
    if w.routing == "zipf":
        # per-expert bias 2*log(1/(e+1)^1.1), e zero-based, fp64 then fp32
        e = np.arange(E, dtype=np.float64)
        out["bias"] = (2.0 * np.log(1.0 / np.power(e + 1.0, 1.1))).astype(np.float32)
    elif w.routing == "noise":
        out["noise"] = rng.standard_normal(size=(T, E), dtype=np.float32) * np.float32(0.5)
    return out


def make_lora_factors(w: Workload, r: int, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """LoRA factors for the fused expert weights of workload ``w`` (rank r),
    drawn from their own stream (seed + 7919) in the order A_gu, B_gu, A_dn,
    B_dn: A ~ N(0,1)/sqrt(fan_in) (d for the gate/up factor, f for the down
    one), B ~ N(0,1)/(4 sqrt(r)): nonzero, so that every LoRA path carries
    signal (training would start B at zero), and a quarter of the base
    weights' scale, so that the adapted layer keeps the base layer's
    magnitudes, as a trained adapter does.  Shapes: a_gu[E,r,d],
    b_gu[E,2f,r], a_dn[E,r,f], b_dn[E,d,r]; bf16-exact for bf16 workloads."""
    seed = (w.seed if seed is None else seed) + 7919
    rng = np.random.Generator(np.random.PCG64(seed))
    bf16 = w.dtype == "bf16"
    E, d, f = w.E, w.d, w.f
    return {
        "a_gu": _normal(rng, (E, r, d), 1.0 / math.sqrt(d), bf16),
        "b_gu": _normal(rng, (E, 2 * f, r), 0.25 / math.sqrt(r), bf16),
        "a_dn": _normal(rng, (E, r, f), 1.0 / math.sqrt(f), bf16),
        "b_dn": _normal(rng, (E, d, r), 0.25 / math.sqrt(r), bf16),
    }
