"""Host logic of the per-stage breakdown (verify_gemm_amd/stage_stamps.py):
stamps built so that every part has a known length."""
import numpy as np

from verify_gemm_amd import stage_stamps as ss


def test_stage_parts_recovers_known_parts():
    nstages, grid = 257, 4
    st = np.zeros((ss.KINDS, ss.STAGES, ss.WGS), dtype=np.uint64)
    t = 1000
    for s in range(nstages):
        k = s % 4
        compute = 500 + 100 * k            # 5, 6, 7, 8 us by stage kind
        det = t + 200                      # 2 us after the previous stage's last signal
        rdy = det + 100                    # 1 us copy
        done = rdy + compute
        sig = np.full(grid, done + 50)     # 0.5 us stores ...
        sig[s % grid] += 150               # ... and one straggler 1.5 us behind
        for w in range(grid):
            st[ss.DETECT, s, w], st[ss.READY, s, w], st[ss.DONE, s, w] = det, rdy, done
            st[ss.SIGNAL, s, w] = sig[w]
        t = int(sig.max())
    parts = ss.stage_parts(st, nstages, grid)
    for k in range(4):
        detect, ready, compute, stores, straggle, span = parts[k]
        assert np.isclose(detect, 2.0) and np.isclose(ready, 1.0) and np.isclose(stores, 0.5)
        assert np.isclose(compute, 5.0 + k) and np.isclose(straggle, 1.5)
        assert np.isclose(span, 2.0 + 1.0 + 5.0 + k + 0.5 + 1.5)
