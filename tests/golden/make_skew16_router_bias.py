"""Write skew16_router_bias.txt: the router bias b_r [16] that makes the
16-expert layer's expert popularity follow Zipf(s = 1.2).

Only oracle/ (fp64 logits and top-2) and gen/ (the seeded inputs) are used.
Target share of expert e: p_e = (e + 1)^-s / sum_r r^-s.  Starting from b = 0,
each iteration routes all T = 8192 tokens with the oracle and moves
b_e <- b_e + 0.5 * ln(p_e / max(q_e, 0.5 / 2T)), where q_e is expert e's
observed share of the 2T assignments.  The fit stops after 100 iterations or
when every share is within 1% of its target; b is then rounded to fp32 and
stored as hex floats, with the achieved shares in the comments.

Run from the repository root:  python tests/golden/make_skew16_router_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import oracle  # noqa: E402


def main():
    cfg = gen.CONFIGS["skew16"]
    T = cfg.Ts[0]
    E = cfg.E
    x = gen.make_x(cfg, T)
    w_r = gen.make_router(cfg)
    lg = oracle.logits(x, w_r, None)
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-cfg.zipf_s)
    p /= p.sum()
    A = 2 * T

    def shares(b):
        idx = oracle.top2(lg + b[None, :])
        return np.bincount(idx.reshape(-1), minlength=E) / A

    b = np.zeros(E)
    it = 0
    for it in range(1, 101):
        q = shares(b)
        if np.all(np.abs(q - p) <= 0.01 * p):
            break
        b = b + 0.5 * np.log(p / np.maximum(q, 0.5 / A))
        b -= b.mean()
    b32 = b.astype(np.float32)
    # achieved shares with the stored fp32 bias, through the oracle's own bias path
    q = np.bincount(oracle.top2(oracle.logits(x, w_r, b32)).reshape(-1), minlength=E) / A
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew16_router_bias.txt")
    with open(out, "w") as f:
        f.write("# Router bias b_r [16] (fp32, hex) for the 16-expert Zipf(1.2)-skewed layer\n")
        f.write("# (E=16, d=3584, h=2560, T=8192, seed 0).  Written by make_skew16_router_bias.py\n")
        f.write(f"# from oracle logits; {it} fit iterations.\n")
        f.write("# columns: bias(hex)  bias(decimal)  target_share  achieved_share  assignments\n")
        for e in range(E):
            f.write(f"{float(b32[e]).hex()}  {b32[e]: .6f}  {p[e]:.5f}  {q[e]:.5f}  {int(round(q[e] * A))}\n")
        f.write(f"# max/mean expert load = {q.max() * E:.3f}\n")
    print(open(out).read())


if __name__ == "__main__":
    main()
