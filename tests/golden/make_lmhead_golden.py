"""Write the expected results of the lm_head verify workload.

Workload: M = 17 rows per step (16 drafts + 1), K = 5120, V = 248,320 and
its 65,536-row slice, 1000 seeded steps with fresh X per step and one
weight set per V; drafts equal the target argmax with probability 0.7.
Inputs come from verify_gemm_amd.synth (seeded), expected values ONLY from
the CPU oracle.  Output: tests/golden/lmhead_v{V}_s{steps}.npz holding the
drafts, the oracle argmax, decisiveness, accept lengths and the top-2 gap.

    python tests/golden/make_lmhead_golden.py [--steps 1000] [--vocab 248320 65536]
"""
import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from verify_gemm_amd import synth  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--vocab", type=int, nargs="+", default=[synth.VOCAB, synth.VOCAB_SLICE])
    args = ap.parse_args()
    T = synth.T_VERIFY
    for v in args.vocab:
        t0 = time.time()
        wq, ws, g = synth.lmhead_weights(v)
        x = synth.lmhead_steps_x(args.steps, v)
        r = oracle.lmhead_ref(x, wq, ws, g, T=T)          # argmax of every row, all steps
        am = r["argmax"].reshape(args.steps, T)
        drafts = synth.lmhead_steps_drafts(am, v)
        acc = np.array([oracle.accept_len_ref(drafts[s], am[s]) for s in range(args.steps)], np.int32)
        dec = r["decisive"].reshape(args.steps, T)
        step_dec = np.array([bool(dec[s, :min(int(acc[s]), T - 2) + 1].all()) for s in range(args.steps)])
        out = os.path.join(HERE, f"lmhead_v{v}_s{args.steps}.npz")
        np.savez_compressed(out, vocab=v, steps=args.steps, T=T, g=g, drafts=drafts, argmax=am,
                            decisive=dec, accept_len=acc, step_decisive=step_dec,
                            gap=(r["top1"] - r["top2"]).reshape(args.steps, T),
                            bound=np.maximum(r["b1"], r["b2"]).reshape(args.steps, T))
        print(f"V={v}: {time.time() - t0:.1f}s, decisive rows {dec.mean():.4f}, "
              f"decisive steps {step_dec.mean():.4f}, mean accept {acc.mean():.3f} -> {out}", flush=True)


if __name__ == "__main__":
    main()
