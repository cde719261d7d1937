"""A whole decode step over all layers: one metadata build shared by every
layer, each layer's fused rotary write + split-K decode, captured once into a
HIP graph and replayed.

AstrAI docs/developer/internals.md, "Cache Architecture": the step's cache
metadata is computed once and shared across layers; docs/guides/inference.md,
"Attention Backend": the decode op writes the new token's k/v and attends.
The layers' own projections are outside this path: per-layer q, k_new, v_new
are inputs here and per-layer outputs are returned.  Capture records only
this library's kernel launches on torch's current stream; every buffer is
allocated before capture (nothing allocates, frees or clears memory inside the
graph), so a replay reruns exactly the eager launches.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import api


class DecodeStep:
    """n_layers x (astr_decode_attn_write) over one KVCache record.

    q: [n_layers, B, H, D] unrotated; k_new, v_new: [n_layers, B, Hkv, D]
    unrotated; out: [n_layers, B, H, D].  The split workspace is shared by
    the layers (they run in order on one stream).
    """

    def __init__(self, cache: api.KVCache, freqs_cis: torch.Tensor, q: torch.Tensor,
                 k_new: torch.Tensor, v_new: torch.Tensor, split_chunk: int,
                 layers: Optional[list] = None, sm_scale: float = 0.0):
        n_layers = int(cache.k_buffer.shape[0])
        self.layers = list(range(n_layers)) if layers is None else [int(x) for x in layers]
        api._need(q.dim() == 4 and q.shape[0] == len(self.layers), "q must be [layers, batch, heads, head_dim]")
        api._need(k_new.shape[0] == len(self.layers) and v_new.shape[0] == len(self.layers),
                  "k_new / v_new must have one slice per layer")
        self.cache, self.freqs, self.q, self.k_new, self.v_new = cache, freqs_cis, q, k_new, v_new
        self.split_chunk, self.sm_scale = int(split_chunk), float(sm_scale)
        self.out = torch.empty_like(q)
        h = int(q.shape[2])
        self.o_part, self.lse_part = api.decode_workspace(cache, h, split_chunk)   # (None, None): one split
        self.graph: Optional[torch.cuda.CUDAGraph] = None

    def run(self) -> torch.Tensor:
        """Launch every layer eagerly on the current stream."""
        for i, layer in enumerate(self.layers):
            api.decode_attn_write(self.q[i], self.k_new[i], self.v_new[i], self.cache, layer, self.freqs,
                                  self.split_chunk, self.sm_scale, out=self.out[i], o_part=self.o_part,
                                  lse_part=self.lse_part)
        return self.out

    def capture(self) -> torch.cuda.CUDAGraph:
        """Record one step into a graph (after one eager run, so that lazy
        library loading and any first-call work happen outside capture)."""
        self.run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self) -> torch.Tensor:
        if self.graph is None:
            raise RuntimeError("capture() first")
        self.graph.replay()
        return self.out
