"""Write tests/golden/kstart.json: the k_start that gives each target density.

Density of one sequence = sum_I kept(I) / sum_I (I + 1), i.e. the fraction of
causal (query block, key block) pairs that the schedule keeps, the diagonal
block included.  For each target the integer k_start whose density is
closest wins (ties to the smaller one).  Uses the oracle's budget rule only.

    python tests/golden/derive_kstart.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402


def density(nb, k_start, mu, alpha, n_init, n_window):
    kept = sum(O.kept_count(I, nb, k_start, mu, alpha, n_init, n_window) for I in range(nb))
    return kept / (nb * (nb + 1) / 2)


def best_kstart(nb, target, mu, alpha, n_init, n_window):
    # density is non-decreasing in k_start: bisect, then compare neighbours
    lo, hi = 0, 4 * nb
    while lo < hi:
        mid = (lo + hi) // 2
        if density(nb, mid, mu, alpha, n_init, n_window) < target:
            lo = mid + 1
        else:
            hi = mid
    best, bestd = None, None
    for k in (lo - 1, lo):
        if k < 0:
            continue
        dd = abs(density(nb, k, mu, alpha, n_init, n_window) - target)
        if bestd is None or dd < bestd - 1e-15:
            best, bestd = k, dd
    return best


def main():
    mu, n_init, n_window = 0.5, 1, 2
    out = {
        "n32k_32q8kv": [best_kstart(256, 0.25, mu, 0.7, n_init, n_window)],
        "n128k_32q8kv": [best_kstart(1024, 0.25, mu, 0.7, n_init, n_window)],
        "n64k_sweep": {str(t): best_kstart(512, t, mu, 0.7, n_init, n_window)
                      for t in (1.0, 0.5, 0.25, 0.2, 0.1)},
        "fp8_varlen_128k": [best_kstart(L // 128, 0.25, mu, 0.7, n_init, n_window)
                     for L in (8192, 16384, 32768, 73728)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kstart.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
