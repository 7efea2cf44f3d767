"""Calibrate the shared-mean strength c of the synthetic inputs (one-off script).

The pages report about 95% attention sparsity during training (MTraining review,
page 1, section 四; 93.7 +- 3.9% globally, section 五). Literal N(0,1) inputs
are nearly dense under a top-p budget, so the generator adds a shared mean
before the rotary embedding. This script bisects its strength c so that the
oracle's mean per-head sparsity at the 131072-token Qwen-shaped workload is
95%, and prints the per-head distribution. The result is frozen as
``synth.inputs.C_STAR``.

Usage: python -m oracle.calibrate [--config qwen128k] [--target 0.95]
"""
import argparse
import time

import numpy as np

from synth import config_by_name, generate
from oracle.index import build_index
from oracle.mask import sparsity


def sparsity_at(cfg):
    t = generate(cfg, tensors=("q", "k"), rows=slice(cfg.N - cfg.last_q, cfg.N))
    tk = generate(cfg, tensors=("k",))
    idx = build_index(t["q"], tk["k"], cfg.scale, cfg.N, cfg.top_p)
    return sparsity(cfg.N, idx["vert"], idx["slash"]), idx


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="qwen128k")
    ap.add_argument("--target", type=float, default=0.95)
    ap.add_argument("--lo", type=float, default=5.0)
    ap.add_argument("--hi", type=float, default=9.0)
    ap.add_argument("--iters", type=int, default=10)
    ap.add_argument("--eval", type=float, default=None, help="only report sparsity at this c")
    args = ap.parse_args()
    if args.eval is not None:
        cfg = config_by_name(args.config, c=args.eval)
        sp, idx = sparsity_at(cfg)
        print(f"c={args.eval:.4f} mean sparsity={sp.mean():.4f} per-head={np.round(sp, 4).tolist()}")
        print("verticals per head:", [len(x) for x in idx["vert"]])
        print("slashes per head:", [len(x) for x in idx["slash"]])
        return
    lo, hi = args.lo, args.hi
    for _ in range(args.iters):
        mid = 0.5 * (lo + hi)
        t0 = time.time()
        sp, _ = sparsity_at(config_by_name(args.config, c=mid))
        print(f"c={mid:.4f} mean sparsity={sp.mean():.4f} ({time.time() - t0:.1f}s)", flush=True)
        if sp.mean() < args.target:
            lo = mid
        else:
            hi = mid
    print(f"c* ~= {0.5 * (lo + hi):.4f}")


if __name__ == "__main__":
    main()
