"""The full weight pass of one decode / verify step, on one GPU.

A step of the ~27B hybrid streams every NVFP4 weight once: 64 layers of
{q, k, v, o: 5120x5120; gate, up: 17408x5120; down: 5120x17408} and the
lm_head (248,320 x 5120) with its fused argmax and greedy accept -- 449
matrices, 14,115,962,880 weight bytes.  The pages capture each decode step
as one graph so host launch cost disappears (ling-engine README, "Six
levers"; the veloGB10 docs list a switch to turn the decode graphs off);
here the 449 launches go through the C ABI on one stream, in the per-layer
order {q, k, v} -> o -> {gate, up} -> down, and are captured once into a HIP
graph and replayed.

This module only sequences launches: it holds device buffers and precomputed
pointers and calls libvgemm.so.  All arithmetic is in the HIP kernels.
"""
from __future__ import annotations

import ctypes

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
    """Activations, outputs and workspaces for one batch size M on top of
    shared PassWeights; ``launch()`` enqueues the whole pass on the current
    stream, ``capture()`` records it into a graph."""

    def __init__(self, weights: PassWeights, M: int, T: int | None = None, x_seed: int = 77):
        if T is None:
            T = synth.T_VERIFY if M % synth.T_VERIFY == 0 else 1
        self.w = weights
        self.M, self.T = M, T
        dev = weights.device
        lib = binding.load()
        self.lib = lib
        self.x = {k: synth.gen_x_device(M, k, x_seed * 10 + k, dev) for k in (HIDDEN, MLP)}
        self.y = []
        self.calls = []
        self.workspaces = {}
        for m in weights.mats:
            n, k = m["n"], m["k"]
            y = torch.empty((M, n), dtype=torch.float32, device=dev)
            self.y.append(y)
            wsb = lib.vg_gemm_workspace_bytes(M, n, k)
            key = (n, k)
            if wsb and key not in self.workspaces:
                self.workspaces[key] = torch.zeros(wsb, dtype=torch.uint8, device=dev)
            wsp = self.workspaces.get(key)
            self.calls.append((self.x[k].data_ptr(), m["wq"].data_ptr(), m["ws"].data_ptr(),
                               ctypes.c_float(m["g"]), M, n, k, y.data_ptr(),
                               wsp.data_ptr() if wsp is not None else None,
                               wsp.numel() if wsp is not None else 0))
        S = M // T
        gen = torch.Generator(device=dev)
        gen.manual_seed(x_seed)
        self.drafts = torch.randint(0, weights.vocab, (S, max(T - 1, 1)), dtype=torch.int32,
                                    device=dev, generator=gen)[:, :T - 1].contiguous()
        self.argmax = torch.empty(M, dtype=torch.int32, device=dev)
        self.accept_len = torch.empty(S, dtype=torch.int32, device=dev)
        self.lm_ws = torch.zeros(lib.vg_lmhead_workspace_bytes(M), dtype=torch.uint8, device=dev)
        lm = weights.lmhead
        self.lm_call = (self.x[HIDDEN].data_ptr(), lm["wq"].data_ptr(), lm["ws"].data_ptr(),
                        ctypes.c_float(lm["g"]), self.drafts.data_ptr() if T > 1 else None,
                        M, HIDDEN, weights.vocab, T, self.argmax.data_ptr(),
                        self.accept_len.data_ptr(), self.lm_ws.data_ptr(), self.lm_ws.numel())
        self.graph = None

    def set_drafts(self, drafts: torch.Tensor):
        self.drafts.copy_(drafts)

    def launch(self, stream=None):
        s = int((stream or torch.cuda.current_stream()).cuda_stream)
        f = self.lib.nvfp4_gemm_ex
        for c in self.calls:
            st = f(*c, s)
            if st:
                raise binding.VgemmError(st, "nvfp4_gemm_ex")
        st = self.lib.lmhead_argmax_accept_ex(*self.lm_call, s)
        if st:
            raise binding.VgemmError(st, "lmhead_argmax_accept_ex")

    def capture(self) -> torch.cuda.CUDAGraph:
        # one eager pass first so every lazily initialised resource exists
        self.launch()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self.launch()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()
