"""The linear layers of one decode step, launched as one HIP graph.

A Qwen-7B-class decoder token runs 28 layers of seven W4A8 linears (q, k, v, o, gate,
up, down) and the lm_head: 197 GEMVs over 7,070,285,824 packed weights.  This module
replays exactly that sequence of ``gemv_w4a8`` calls from a captured graph, so the
launch gaps between kernels are the GPU's own and not Python's.  The Jetson Orin INT4
write-up ("Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s") lists CUDA
Graph capture of the decode step among its next steps (section 后续优化方向), next to
removing the repeated activation quantization of the q/k/v and gate/up projections.

The second item is the ``fused`` chain: q|k|v become one 3584 -> 4608 linear and
gate|up one 3584 -> 37888 linear, each quantizing its activation once.  With the tile
layout the packed weights of a concatenation along N are the concatenation of the
packed parts (row groups of 4 rows are stored one after another), so fusing needs
no repacking; each projection's output is a contiguous slice of the fused output.

Only the linear layers are chained: attention, norms and the residual stream are not
part of this library, so every linear reads a fixed activation of its input width and
the chain is a timing and launch-structure harness.  Each layer gets its own copy of
the packed weights, so every launch streams from HBM as in a real model.
"""
from __future__ import annotations

from . import gemv_w4a8

LAYERS = 28
HIDDEN, INTERMEDIATE, VOCAB, KV = 3584, 18944, 152064, 512
# (name, K, N) of one layer; the fused chain merges q|k|v and gate|up
LAYER_LINEARS = (("q_proj", HIDDEN, HIDDEN), ("k_proj", HIDDEN, KV), ("v_proj", HIDDEN, KV),
                 ("o_proj", HIDDEN, HIDDEN), ("gate_proj", HIDDEN, INTERMEDIATE),
                 ("up_proj", HIDDEN, INTERMEDIATE), ("down_proj", INTERMEDIATE, HIDDEN))
FUSED_GROUPS = (("qkv_proj", ("q_proj", "k_proj", "v_proj")), ("o_proj", ("o_proj",)),
                ("gate_up_proj", ("gate_proj", "up_proj")), ("down_proj", ("down_proj",)))


def w4a8_bytes(M: int, N: int, K: int) -> int:
    """Algorithmic bytes of one W4A8 linear: 0.5 B per weight, 4 B per scale, X and Y element."""
    return N * K // 2 + 4 * N + 4 * M * K + 4 * M * N


def fuse_along_n(parts):
    """Packed (Wq, w_scale) pairs of linears with the same K -> the packed pair of their
    concatenation along N.  Every part's N must be a multiple of 4 (whole row groups)."""
    import torch

    for wq, s in parts:
        if s.shape[0] % 4:
            raise ValueError("fusing along N needs N % 4 == 0, got %d" % s.shape[0])
    return (torch.cat([wq for wq, _ in parts]), torch.cat([s for _, s in parts]))


class DecodeChain:
    """The W4A8 linears of ``layers`` decoder layers plus the lm_head, one token (M = 1).

    ``layer`` maps each name of LAYER_LINEARS to its packed (Wq, w_scale) (from
    ``quantize_pack_w4``); every layer gets its own device copy.  ``lm_head`` is the
    packed (Wq, w_scale) of the lm_head, or None.  ``x_hidden`` [1][K_hidden] and
    ``x_inter`` [1][K_inter] (fp32) are the fixed inputs of the linears by input width.
    """

    def __init__(self, layer, lm_head, x_hidden, x_inter, layers: int = LAYERS,
                 fused: bool = False):
        import torch

        self.fused = fused
        self.x = {x_hidden.shape[1]: x_hidden, x_inter.shape[1]: x_inter}
        if fused:
            one = [(g, fuse_along_n([layer[p] for p in parts])) for g, parts in FUSED_GROUPS]
        else:
            one = [(name, layer[name]) for name, _, _ in LAYER_LINEARS]
        # (name, K, N, Wq, s) per launch, in decode order; layer 0 uses the given buffers
        self.launches = []
        for li in range(layers):
            for name, (wq, s) in one:
                if li > 0:
                    wq, s = wq.clone(), s.clone()
                self.launches.append((name, self._k_of(name), s.shape[0], wq, s))
        if lm_head is not None:
            self.launches.append(("lm_head", HIDDEN, lm_head[1].shape[0], lm_head[0], lm_head[1]))
        dev = x_hidden.device
        self.out = {}
        for name, K, N, _, _ in self.launches:
            if name not in self.out:
                self.out[name] = torch.empty((1, N), dtype=torch.float32, device=dev)
        for name, K, N, wq, s in self.launches:
            if K not in self.x:
                raise ValueError("no input of width %d for %s" % (K, name))

    @staticmethod
    def _k_of(name: str) -> int:
        return INTERMEDIATE if name == "down_proj" else HIDDEN

    @property
    def launches_per_token(self) -> int:
        return len(self.launches)

    @property
    def bytes_per_token(self) -> int:
        return sum(w4a8_bytes(1, N, K) for _, K, N, _, _ in self.launches)

    def run(self, stream=None) -> None:
        """One token's linears, launched eagerly on the current (or given) stream."""
        for name, K, N, wq, s in self.launches:
            gemv_w4a8(self.x[K], wq, s, out=self.out[name], stream=stream)

    def capture(self):
        """A torch.cuda.CUDAGraph (a HIP graph) of one token's linears."""
        import torch

        # warm-up on a side stream, as graph capture requires
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        return g
