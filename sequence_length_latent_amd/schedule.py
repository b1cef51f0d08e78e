"""Layer schedules of Stream-Factorized Attention and a multi-layer paged decode.

"Hidden Decoding at Scale" review, section Method: the majority of layers keep
each stream to itself, and the rest let streams see each other with the base
model's sliding-window or full pattern; the 80B model has 6 full + 23 sliding-window
+ 20 within-stream layers out of 49, the 617B model 25 full + 69
within-stream out of 94.  The pages give the counts, not the order: here the
layers of each kind are spread evenly over the depth (the order changes
neither any layer's result nor the work of a decode step).

``PagedDecodeStack`` holds one paged K/V pool per layer (all layers share the
page table, as a serving engine shares one block table across layers) and
runs one decode step of every layer through ``decode_step_paged``.  Every
attention computation runs in the library's kernels; this module only
allocates the pools and issues the calls.
"""
from __future__ import annotations

import torch

from . import MIX, WITHIN, decode_step_paged, decode_workspace_size

FULL, SLIDING, WITHIN_STREAM = "full", "sliding", "within"

SCHEDULES = {
    "80B": {FULL: 6, SLIDING: 23, WITHIN_STREAM: 20},
    "617B": {FULL: 25, WITHIN_STREAM: 69},
}


def layer_kinds(name: str) -> list:
    """The kinds of the model's layers in depth order, each kind spread evenly:
    layer i takes the kind whose running share is furthest behind its target."""
    counts = SCHEDULES[name]
    total = sum(counts.values())
    placed = {k: 0 for k in counts}
    kinds = []
    for i in range(total):
        # deficit of each kind after i+1 layers; ties go to the order in SCHEDULES
        best = max(counts, key=lambda k: (counts[k] * (i + 1) / total - placed[k]))
        placed[best] += 1
        kinds.append(best)
    return kinds


class PagedDecodeStack:
    """Per-layer paged caches and one decode step over all layers.

    kinds          layer kinds (FULL, SLIDING, WITHIN_STREAM)
    S, n, Hq, Hkv, D, page_size, pages_per_seq: cache geometry; sequence q
                   owns pages q*pages_per_seq .. (q+1)*pages_per_seq - 1 of
                   every layer's pool unless a page table is given
    window         sliding window (interleaved positions) of the SLIDING layers
    """

    def __init__(self, kinds, S, n, Hq, Hkv, D, page_size, pages_per_seq, window, device="cuda",
                 page_table=None, num_pages=None):
        self.kinds = list(kinds)
        self.S, self.n, self.Hq, self.Hkv, self.D = S, n, Hq, Hkv, D
        self.page_size, self.window = page_size, window
        num_pages = S * pages_per_seq if num_pages is None else num_pages
        if page_table is None:
            page_table = torch.arange(S * pages_per_seq, dtype=torch.int32,
                                      device=device).reshape(S, pages_per_seq)
        self.page_table = page_table
        shape = (num_pages, page_size, Hkv, D)
        self.k_pools = [torch.empty(shape, dtype=torch.bfloat16, device=device) for _ in self.kinds]
        self.v_pools = [torch.empty(shape, dtype=torch.bfloat16, device=device) for _ in self.kinds]
        self.capacity = pages_per_seq * page_size            # entries per sequence

    def workspace(self, max_tokens):
        need = decode_workspace_size(self.S, self.n, self.Hq, self.Hkv, self.D, max_tokens)
        return torch.empty(max(need, 16), dtype=torch.uint8, device=self.page_table.device)

    def layer_call(self, i):
        """(mode, window) of layer i."""
        kind = self.kinds[i]
        if kind == WITHIN_STREAM:
            return WITHIN, None
        return MIX, (self.window if kind == SLIDING else None)

    def step(self, q_new, k_new, v_new, tokens_before, max_tokens, scale, outs, workspace):
        """One decode step of every layer: layer i appends k_new[i] / v_new[i]
        and attends from q_new[i] into outs[i] (lists of per-layer tensors)."""
        for i in range(len(self.kinds)):
            mode, window = self.layer_call(i)
            decode_step_paged(q_new[i], k_new[i], v_new[i], self.k_pools[i], self.v_pools[i],
                              self.page_table, tokens_before, self.n, max_tokens, mode, scale,
                              window=window, workspace=workspace, out=outs[i])
        return outs

    def capture(self, q_new, k_new, v_new, tokens_before, max_tokens, scale, outs, workspace):
        """Record one decode step of every layer (append, attention and, where a
        view has several splits, combine: up to 3 kernels per layer) as a HIP
        graph over these buffers.  ``graph.replay()`` then runs the whole step
        with one host call on whatever the buffers hold at that time (the next
        token's rows in q_new / k_new / v_new, the next tokens_before, a changed
        page table).  The step launches kernels only (no memory fills), and
        allocates nothing given ``outs`` and ``workspace``."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step(q_new, k_new, v_new, tokens_before, max_tokens, scale, outs, workspace)
        return graph
