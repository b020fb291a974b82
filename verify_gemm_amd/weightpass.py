"""The full weight pass of one decode / verify step, on one GPU.

A step of the ~27B hybrid streams every NVFP4 weight once: 64 layers of
{q, k, v, o: 5120x5120; gate, up: 17408x5120; down: 5120x17408} and the
lm_head (248,320 x 5120) with its fused argmax and greedy accept -- 449
matrices, 14,115,962,880 weight bytes.  The pages capture each decode step
as one graph so host launch cost disappears (ling-engine README, "Six
levers"; the veloGB10 docs list a switch to turn the decode graphs off);
on MI355X the native step executor (vg_pass_run) streams the matrices in
the per-layer dependency order {q, k, v} -> o -> {gate, up} -> down: at
M = 1 as ONE persistent launch with device-side stage barriers, at M >= 2
as one launch per dependency stage (the faster schedule there); the other
schedules are kept for comparison (run_persistent / run_staged /
run_unfused).

This module only holds device buffers and describes the jobs; all
sequencing and arithmetic happen in libvgemm.so.
"""
from __future__ import annotations

import torch

from . import binding, synth

HIDDEN, MLP, VOCAB = synth.HIDDEN, synth.MLP, synth.VOCAB


# Matrices stored back to back per layer, so that a fused job can read them
# as one matrix: {q, k, v} and {gate, up} (dgx-spark-qwen38 README, opening
# section; the fused projections cut the one-launch-per-matrix schedule
# from 449 to 257 launches).
FUSED_GROUPS = (("qkv", ("q", "k", "v")), ("gateup", ("gate", "up")))


class PassWeights:
    """Device-resident weights of the synthetic pass, generated on the GPU
    from per-matrix seeds (codes uniform, scales 2**u, u in -4..2, g ~ U[0.5, 2]).
    Each layer's q, k, v (and gate, up) are row slices of one contiguous
    matrix (``self.fused[layer][group]``), so both schedules share the bytes."""

    def __init__(self, device="cuda", layers: int = synth.LAYERS, vocab: int = VOCAB,
                 seed: int = synth.SEED_BASE + 4):
        self.device = torch.device(device)
        self.layers = layers
        self.vocab = vocab
        self.seed = seed
        self.mats = []
        self.fused = []
        shapes = {name: (n, k) for name, n, k in synth.LAYER_MATS}
        for layer in range(layers):
            groups = {}
            for gname, members in FUSED_GROUPS:
                k = shapes[members[0]][1]
                rows = sum(shapes[m][0] for m in members)
                groups[gname] = {"wq": torch.empty((rows, k // 2), dtype=torch.uint8, device=self.device),
                                 "ws": torch.empty((rows, k // 16), dtype=torch.uint8, device=self.device),
                                 "members": members, "n": rows, "k": k}
            self.fused.append(groups)
            for j, (name, n, k) in enumerate(synth.LAYER_MATS):
                self.mats.append(self._make(name, layer, j, n, k, groups))
        self.lmhead = self._make("lm_head", layers, 0, vocab, HIDDEN, {})

    def _make(self, name, layer, j, n, k, groups):
        s = synth.pass_matrix_seed(layer, j, self.seed)
        wq, ws = synth.gen_weights_device(n, k, s, self.device)
        for gname, grp in groups.items():
            if name in grp["members"]:
                r0 = sum(self.mats[-i - 1]["n"] for i in range(grp["members"].index(name)))
                grp["wq"][r0:r0 + n].copy_(wq)
                grp["ws"][r0:r0 + n].copy_(ws)
                wq, ws = grp["wq"][r0:r0 + n], grp["ws"][r0:r0 + n]
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
    ``run()`` is the step in vg_pass_run's schedule for this M,
    ``run_persistent()`` one persistent launch of the whole step,
    ``run_unfused()`` the same work as one launch per job,
    ``run_staged()`` one launch per dependency stage.

    ``fused``: {q, k, v} and {gate, up} run as one job each (4 jobs a layer,
    257 in all), reading the members' stacked rows as one matrix; each
    member keeps its own tensor scale through the job's per-row scales, so
    every output row has the same bits as with the separate jobs.  The fused
    jobs' outputs are [M][sum of the members' N]."""

    def __init__(self, weights: PassWeights, M: int, T: int | None = None, x_seed: int = 77,
                 fused: bool = False):
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
        group_of = {name: gname for gname, members in FUSED_GROUPS for name in members}
        by_name = {(m["layer"], m["name"]): m for m in weights.mats}
        for m in weights.mats:
            gname = group_of.get(m["name"])
            stage = 4 * m["layer"] + stage_of[m["name"]]
            if fused and gname is not None:
                f = weights.fused[m["layer"]][gname]
                if m["name"] != f["members"][0]:
                    continue
                rs = torch.cat([torch.full((by_name[(m["layer"], nm)]["n"],), by_name[(m["layer"], nm)]["g"],
                                           dtype=torch.float32, device=dev) for nm in f["members"]])
                y = torch.empty((M, f["n"]), dtype=torch.float32, device=dev)
                self.y.append(y)
                gemms.append((self.x[f["k"]], f["wq"], f["ws"], 1.0, y, stage, rs))
            else:
                y = torch.empty((M, m["n"]), dtype=torch.float32, device=dev)
                self.y.append(y)
                gemms.append((self.x[m["k"]], m["wq"], m["ws"], m["g"], y, stage))
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

    def run_persistent(self, stream=None):
        self.step.run_persistent(stream)

    def run_staged(self, stream=None):
        self.step.run_staged(stream)

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
