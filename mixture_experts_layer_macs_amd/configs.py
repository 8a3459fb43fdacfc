"""Synthetic MoE-layer workloads: shapes and routing knobs.

Each workload fixes the shape of one mixture-of-experts layer (tokens T,
hidden H, experts N, top-k, expert intermediate I, element type) and the
routing settings the layer is run with:

* MACS capacity: capacity factor gamma (Eq. 3 of "MACS: Modality-Aware
  Capacity Scaling for Efficient Multimodal MoE Inference", §3.1), modality
  scaling strength lam (§3.3), fallback depth R and locality group g for the
  overflow re-route (§3.4 as announced in §1 and Fig. 1). gamma = inf turns
  capacity off.
* SERE re-routing (multi-image QA inference write-up, §4.1-§4.2): number of
  primary experts kprime (0 = off), similarity threshold rho, and the number
  of protected experts per layer (§5.3 protects 16).

The input recipe behind each workload (distributions, seeds, layouts) lives
in ``synth.py``.  Nothing here computes any part of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

INF = math.inf

# Scale of the Zipf(1.1) popularity bias added to router logits,
# b_j = -ZIPF_BETA * 1.1 * ln(rank_j).  Chosen once by bisection so that the
# mean top-8 batch union of a 128-token, 128-expert batch over seeds 0-9 is
# about 90 experts (the Qwen3-30B-A3B union at batch 128 reported in the
# multi-image QA write-up, §2.2).  tests/calibrate_zipf.py reproduces it.
ZIPF_BETA = 0.7735


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens in the batch
    H: int            # hidden size
    N: int            # experts
    k: int            # top-k
    I: int            # expert intermediate size (SwiGLU)
    dtype: str        # "f32" or "bf16": storage type of x, weights, h, y
    gamma: float      # capacity factor (inf = capacity off)
    lam: float        # modality scaling strength
    R: int            # fallback ranks tried for overflowed slots
    group: int        # locality group size g for fallback re-routes
    kprime: int       # SERE primaries per token (0 = SERE off)
    rho: float        # SERE similarity threshold
    n_protected: int  # SERE protected experts per layer
    logits: str       # "normal" | "zipf" | "straggler"
    visual: str       # "half" | "runs70" | "none" | "frac:<f>"
    vis_weight: str   # "uniform" (U(0.1,1)) | "beta25" (Beta(2,5)) | "one"
    modality: str     # "quarters" (N/4 +1, N/4 -1, N/2 0) | "zero"
    skew_expert0: float = 0.0   # extra logit on expert 0 (overflow variants)
    layers: int = 1

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Tiny fp32 layer that the oracle finishes in seconds.
TINY_F32 = Workload(
    name="tiny_f32", T=256, H=128, N=8, k=2, I=256, dtype="f32",
    gamma=1.25, lam=1.0, R=2, group=8, kprime=0, rho=0.5, n_protected=0,
    logits="normal", visual="half", vis_weight="uniform", modality="quarters")

# Qwen3-30B-A3B-shaped decode step at batch 128, SERE K'=2, rho=0.5.
QWEN3_DECODE = Workload(
    name="qwen3_decode_b128", T=128, H=2048, N=128, k=8, I=768, dtype="bf16",
    gamma=INF, lam=1.0, R=8, group=128, kprime=2, rho=0.5, n_protected=16,
    logits="zipf", visual="half", vis_weight="uniform", modality="quarters")

# Multimodal prefill with MACS: 70 % visual tokens in 1024-token image runs.
MM_PREFILL = Workload(
    name="mm_prefill_t8192", T=8192, H=2048, N=128, k=8, I=768, dtype="bf16",
    gamma=1.0, lam=1.0, R=8, group=128, kprime=0, rho=0.5, n_protected=0,
    logits="straggler", visual="runs70", vis_weight="beta25",
    modality="quarters")

# Mixtral-8x7B-shaped layer with the all-weights-1 (token count) load.
MIXTRAL_PREFILL = Workload(
    name="mixtral_prefill_t4096", T=4096, H=4096, N=8, k=2, I=14336,
    dtype="bf16", gamma=1.0, lam=1.0, R=2, group=8, kprime=0, rho=0.5,
    n_protected=0, logits="normal", visual="none", vis_weight="one",
    modality="zero")
MIXTRAL_DECODE = MIXTRAL_PREFILL.with_(name="mixtral_decode_t64", T=64)

# One layer of the 48-layer decode sweep (Qwen3-30B-A3B shape), MACS on.
SWEEP_LAYER = QWEN3_DECODE.with_(
    name="sweep_layer", gamma=1.25, R=8, visual="frac:0.5",
    vis_weight="uniform", layers=48)

WORKLOADS = {w.name: w for w in
             (TINY_F32, QWEN3_DECODE, MM_PREFILL, MIXTRAL_PREFILL,
              MIXTRAL_DECODE)}


def tiny_variants():
    """Tiny-layer variants that force the re-route and drop paths."""
    return {
        "tiny_f32": TINY_F32,
        "tiny_f32_skew": TINY_F32.with_(name="tiny_f32_skew", skew_expert0=2.0),
        "tiny_f32_tight": TINY_F32.with_(name="tiny_f32_tight", gamma=0.5),
        "tiny_f32_tight_r0": TINY_F32.with_(name="tiny_f32_tight_r0",
                                            gamma=0.5, R=0),
    }
