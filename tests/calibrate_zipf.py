"""Calibrate the Zipf popularity scale of the decode workload's router logits.

Finds beta such that the mean top-8 batch union over a 128-token,
128-expert batch, averaged over seeds 0-9, is 90 experts (the batch-128
union the multi-image QA write-up reports for Qwen3-30B-A3B in §2.2).
The union is computed with the oracle's router.  Run:
    python -m tests.calibrate_zipf
and copy the printed value into configs.ZIPF_BETA.
"""
import numpy as np

from mixture_experts_layer_macs_amd import synth
from mixture_experts_layer_macs_amd.configs import QWEN3_DECODE
from oracle.moe_oracle import route


def mean_union(beta: float, seeds=range(10)) -> float:
    u = []
    for sd in seeds:
        lg = synth.router_logits(QWEN3_DECODE, sd, zipf_beta=beta)
        topk, _, _ = route(lg, QWEN3_DECODE.k, 0)
        u.append(len(set(topk.ravel().tolist())))
    return float(np.mean(u))


def main(target: float = 90.0):
    lo, hi = 0.0, 3.0            # union falls as beta grows
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if mean_union(mid) > target:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 4)
    print(f"ZIPF_BETA = {beta}  mean union = {mean_union(beta):.2f}")


if __name__ == "__main__":
    main()
