"""Fix the strength beta of the Zipf(1.1) router-logit bias and store it.

The skewed workloads add b_e = beta * ln p_e (p_e proportional to
(e+1)^-1.1) to the router logits.  The workload definition says only that
"8 hot experts take about 30% of assignments" for the 8192-token prefill; this
script picks beta by bisection so that the 8 most-assigned experts of that
workload take 0.300 of its T*k assignments, using only the oracle router.

Run:  python tests/golden/make_zipf_beta.py   (writes tests/golden/zipf_beta.json)
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import synthetic as S                      # noqa: E402
from oracle import moe_ref as R            # noqa: E402


def top8_share(l0, lp, beta, k):
    idx = R.topk(l0 + beta * lp[None, :], k)
    counts = np.bincount(idx.ravel(), minlength=lp.size)
    return np.sort(counts)[::-1][:8].sum() / idx.size


def main():
    cfg = S.config("prefill8192")
    x, kind = S.tokens(cfg)
    xf = S.bf16_to_f32(x) if kind == "bf16" else x
    l0 = R.router_logits(xf, S.router_weight(cfg))
    lp = S.zipf_log_p(cfg["n_experts"])
    lo, hi = 0.0, 4.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if top8_share(l0, lp, mid, cfg["top_k"]) < 0.300:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 6)
    share = top8_share(l0, lp, beta, cfg["top_k"])
    out = dict(beta=beta, top8_share_prefill8192=float(share),
               _source="tests/golden/make_zipf_beta.py (oracle router only); target: the 8 "
                       "most-assigned experts take 0.300 of the prefill8192 assignments")
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_beta.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
