"""The full weight pass of one decode / verify step, on one GPU.

A step of the ~27B hybrid streams every NVFP4 weight once: 64 layers of
{q, k, v, o: 5120x5120; gate, up: 17408x5120; down: 5120x17408} and the
lm_head (248,320 x 5120) with its fused argmax and greedy accept -- 449
matrices, 14,115,962,880 weight bytes.  The pages capture each decode step
as one graph so host launch cost disappears (ling-engine README, "Six
levers"; the veloGB10 docs list a switch to turn the decode graphs off);
on MI355X the whole step is ONE persistent launch of the native step
executor (vg_pass_run), which streams the 449 matrices in the per-layer
dependency order {q, k, v} -> o -> {gate, up} -> down with device-side stage
barriers.  The one-launch-per-matrix schedule is kept for comparison.

This module only holds device buffers and describes the jobs; all
sequencing and arithmetic happen in libvgemm.so.
"""
from __future__ import annotations

import torch

from . import binding, synth

HIDDEN, MLP, VOCAB = synth.HIDDEN, synth.MLP, synth.VOCAB


class PassWeights:
    """Device-resident weights of the synthetic pass, generated on the GPU
    from per-matrix seeds (codes uniform, scales 2**u, u in -4..2, g ~ U[0.5, 2])."""

    def __init__(self, device="cuda", layers: int = synth.LAYERS, vocab: int = VOCAB,
                 seed: int = synth.SEED_BASE + 4):
        self.device = torch.device(device)
        self.layers = layers
        self.vocab = vocab
        self.seed = seed
        self.mats = []
        for layer in range(layers):
            for j, (name, n, k) in enumerate(synth.LAYER_MATS):
                self.mats.append(self._make(name, layer, j, n, k))
        self.lmhead = self._make("lm_head", layers, 0, vocab, HIDDEN)

    def _make(self, name, layer, j, n, k):
        s = synth.pass_matrix_seed(layer, j, self.seed)
        wq, ws = synth.gen_weights_device(n, k, s, self.device)
        return {"name": name, "layer": layer, "j": j, "n": n, "k": k, "wq": wq, "ws": ws,
                "g": synth.pass_gscale(layer, j, self.seed)}

    @property
    def all_mats(self):
        return self.mats + [self.lmhead]

    def weight_bytes(self) -> int:
        return sum(m["wq"].numel() + m["ws"].numel() for m in self.all_mats)


class PassRun:
    """Activations, outputs and the lm_head buffers for one batch size M on
    top of shared PassWeights, and the step itself as a native vg_pass:
    ``run()`` is one persistent launch of the whole step, ``run_unfused()``
    the same work as one launch per matrix."""

    def __init__(self, weights: PassWeights, M: int, T: int | None = None, x_seed: int = 77):
        if T is None:
            T = synth.T_VERIFY if M % synth.T_VERIFY == 0 else 1
        self.w = weights
        self.M, self.T = M, T
        dev = weights.device
        self.x = {k: synth.gen_x_device(M, k, x_seed * 10 + k, dev) for k in (HIDDEN, MLP)}
        self.y = []
        gemms = []
        # stages: {q,k,v} -> o -> {gate,up} -> down per layer
        stage_of = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
        for m in weights.mats:
            y = torch.empty((M, m["n"]), dtype=torch.float32, device=dev)
            self.y.append(y)
            gemms.append((self.x[m["k"]], m["wq"], m["ws"], m["g"], y,
                          4 * m["layer"] + stage_of[m["name"]]))
        S = M // T
        gen = torch.Generator(device=dev)
        gen.manual_seed(x_seed)
        self.drafts = torch.randint(0, weights.vocab, (S, max(T - 1, 1)), dtype=torch.int32,
                                    device=dev, generator=gen)[:, :T - 1].contiguous()
        self.argmax = torch.empty(M, dtype=torch.int32, device=dev)
        self.accept_len = torch.empty(S, dtype=torch.int32, device=dev)
        lm = weights.lmhead
        self.step = binding.Pass(gemms, M, (self.x[HIDDEN], lm["wq"], lm["ws"], lm["g"], T,
                                            self.drafts, self.argmax, self.accept_len))
        self.graph = None

    def set_drafts(self, drafts: torch.Tensor):
        self.drafts.copy_(drafts)

    def run(self, stream=None):
        self.step.run(stream)

    def run_unfused(self, stream=None):
        self.step.run_unfused(stream)

    def capture_unfused(self) -> torch.cuda.CUDAGraph:
        """The one-launch-per-matrix schedule captured into a graph."""
        self.run_unfused()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self.run_unfused()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def check(self) -> int:
        return self.step.check()

    def close(self):
        self.step.close()
