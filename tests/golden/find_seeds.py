"""Select the seeded variants of the synthetic workloads with the CPU oracle.

Run:  python tests/golden/find_seeds.py   (writes tests/golden/seeds.json)

Calls only the oracle and the seeded input module.  For each workload it picks
the first router variant (and, for the batch-16 decode, x variant) such that

  * every token's gap between its k-th and (k+1)-th largest fp64 logit
    exceeds TAU = 1e-4, so a GPU whose fp32 logits stay within TAU/2 of the
    oracle's must select the same expert set;
  * decode16: the realised number of distinct experts is in [58, 62];
  * prefill: beta of the bias -1.1*beta*ln(rank) is bisected until the
    least-squares rank-frequency slope of the realised expert loads is
    -1.1 +- 0.05.
The values are copied into synthetic.CONFIGS; a CPU test checks they agree.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle as O  # noqa: E402
from bit_quantized_routed_router_amd import synthetic as S  # noqa: E402

TAU = 1e-4


def logits_for(cfg, router_variant, x_variant, bias):
    X = O.x_to_f64(S.gen_x(cfg, variant=x_variant), cfg.x_dtype)
    return O.router_logits(X, S.gen_router(cfg, variant=router_variant), bias)


def loads(logits, k, E):
    idx, _ = O.topk(logits, k)
    return np.bincount(idx.ravel(), minlength=E)


def find_decode1():
    cfg = S.CONFIGS["decode1"]
    for rv in range(100):
        L = logits_for(cfg, rv, 0, None)
        if O.topk_gap(L, cfg.k).min() > TAU:
            return dict(router_variant=rv, x_variant=0, min_gap=float(O.topk_gap(L, cfg.k).min()))
    raise RuntimeError("no decode1 variant")


def find_decode16():
    cfg = S.CONFIGS["decode16"]
    bias = S.gen_bias(cfg)
    for xv in range(1000):
        L = logits_for(cfg, 0, xv, bias)
        ld = loads(L, cfg.k, cfg.E)
        nd = int((ld > 0).sum())
        if 58 <= nd <= 62 and O.topk_gap(L, cfg.k).min() > TAU:
            return dict(router_variant=0, x_variant=xv, distinct=nd, min_gap=float(O.topk_gap(L, cfg.k).min()))
    raise RuntimeError("no decode16 variant")


def find_prefill():
    cfg = S.CONFIGS["prefill"]
    X = O.x_to_f64(S.gen_x(cfg), cfg.x_dtype)
    out = None
    for rv in range(200):
        base = O.router_logits(X, S.gen_router(cfg, variant=rv), None)
        lo, hi = 0.0, 4.0
        beta, slope = None, None
        for _ in range(30):
            mid = 0.5 * (lo + hi)
            b = S.gen_bias(cfg, beta=mid).astype(np.float64)
            slope = S.rank_frequency_slope(loads(base + b, cfg.k, cfg.E))
            beta = mid
            if abs(slope + 1.1) < 0.01:
                break
            if slope > -1.1:
                lo = mid  # too flat: more bias
            else:
                hi = mid
        beta = float(np.float32(beta))
        bias = S.gen_bias(cfg, beta=beta)
        L = base + bias.astype(np.float64)
        gap = O.topk_gap(L, cfg.k).min()
        ld = loads(L, cfg.k, cfg.E)
        slope = S.rank_frequency_slope(ld)
        if gap > TAU and abs(slope + 1.1) <= 0.05:
            out = dict(router_variant=rv, x_variant=0, zipf_beta=beta, slope=slope, min_gap=float(gap),
                       max_load=int(ld.max()), min_load=int(ld.min()), experts_hit=int((ld > 0).sum()),
                       share_below_ridge=float(ld[ld < 44].sum() / ld.sum()))
            return out
    raise RuntimeError("no prefill variant")


def main():
    res = dict(tau=TAU, decode1=find_decode1(), decode16=find_decode16(), prefill=find_prefill())
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "seeds.json")
    with open(path, "w") as fh:
        json.dump(res, fh, indent=2)
    print(json.dumps(res, indent=2))


if __name__ == "__main__":
    main()
