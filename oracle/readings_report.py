"""How much the readings of the SSZ search's silent points matter -- a diagnostic
report, CPU only, test infrastructure like the rest of this directory.

The SSZ document ([SSZ] 收敛判断, 算法流程, 迭代优化阶段) leaves three choices open
that the oracle and the kernels fix one way: the two convergence tests combine
with OR, the "quantization error" is the channel's mean squared difference, and
each channel stops on its own.  This script runs the oracle's search under each
alternative on rows of the synthetic workloads and prints, per alternative, how
many rows end with a different scale or a different number of steps.

    python oracle/readings_report.py [--rows 512]

Inputs: the hidden-4096 prefill weights with the step's smoothing (alpha 0.5,
the 8 calibration batches of the same seeded activations) and one unsmoothed
QKV weight of the model-scale weight workload; the first `rows` rows of each.
"""
import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import synth  # noqa: E402

ALTERNATIVES = (("both tests required (AND)", dict(conv_and=True)),
                ("summed instead of mean error", dict(err_sum=True)),
                ("rows iterate until all converged", dict(global_loop=True)))


def samples(rows):
    for c in synth.cases("opt67b"):
        w = synth.widen(c.w())
        ax = None
        for b in range(c.calib_batches):
            ax = oracle.absmax_cols(synth.widen(c.x_batch(b)), ax)
        s = oracle.smooth_factors(ax, oracle.absmax_cols(w), 0.5)
        yield f"{c.name} (smoothed, alpha 0.5)", np.ascontiguousarray(w[:rows]), s, 8
    c = [c for c in synth.cases("ssz_scale") if c.name.endswith("qkv")][0]
    w = np.ascontiguousarray(synth.widen(c.w())[:rows])
    yield f"{c.name} (unsmoothed)", w, None, 8
    yield f"{c.name} (unsmoothed)", w, None, 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=512)
    a = ap.parse_args()
    print("| weight rows | bits | reading | mean steps | rows with another scale | rows with another step count | "
          "largest scale change | mean error change |")
    print("|---|---|---|---|---|---|---|---|")
    for name, w, s, bits in samples(a.rows):
        ref = oracle.ssz(w, s, bits)
        print(f"| {name} [{w.shape[0]} x {w.shape[1]}] | int{bits} | OR, mean, per row (used) | "
              f"{ref['iters'].mean():.2f} | - | - | - | - |", flush=True)
        for label, kw in ALTERNATIVES:
            v = oracle.ssz_variant(w, s, bits, **kw)
            rel = np.abs(v["S"].astype(np.float64) / ref["S"] - 1.0)
            err = v["mse"].sum() / ref["mse"].sum() - 1.0
            print(f"| | | {label} | {v['iters'].mean():.2f} | {int(np.sum(v['S'] != ref['S']))} | "
                  f"{int(np.sum(v['iters'] != ref['iters']))} | {rel.max():.2e} | {100 * err:+.4f}% |", flush=True)


if __name__ == "__main__":
    main()
