"""Decode-step HIP graphs per batch-size bucket.

A serving loop runs one decode step per iteration with a batch whose size
changes as requests join and finish.  Capturing the step once and replaying it
removes the per-step launch cost ("nano-vLLM offline" course, THE IMPORTANT
DETAILS item 03: the decode path runs under a captured graph, and a replay
reads new inputs and computes new results).  A captured graph fixes its
shapes and buffer addresses ("Visual atlas" ch.26: replay uses preallocated
buffers; values and valid lengths may change, the shape/address contract must
hold), so one graph is captured per bucket of batch sizes over static
buffers sized for the largest bucket.

A step with S sequences uses the smallest bucket B >= S: the inputs are copied
into the first S rows of the static buffers, rows S..B-1 are padding (context
length 0 and slot -1: the fused kernel writes a zero row for them, stores
nothing and reads nothing), and the bucket's graph is replayed.  The graph
holds one library call, ``pa_decode_store`` (store of the new K/V rows and
paged attention, plus the reduce pass when contexts are split), so every
kernel in it comes from libpa; the capture, instantiation and replay are the
library's own (pa_graph_*, plain HIP graph calls); the copies and padding fills
run outside the graph on the same stream.
"""
from __future__ import annotations

import bisect

import torch

from . import binding

DEFAULT_BUCKETS = (1, 2, 4, 8, 16, 32, 64, 128, 256)


def bucket_for(num_seqs: int, buckets) -> int:
    """Smallest bucket that holds num_seqs sequences (ValueError if none)."""
    bs = sorted(buckets)
    i = bisect.bisect_left(bs, num_seqs)
    if num_seqs < 1 or i == len(bs):
        raise ValueError(f"batch of {num_seqs} does not fit the buckets {bs}")
    return bs[i]


class DecodeGraphs:
    """Captured decode steps over a fixed pool.

    k_cache, v_cache: the pools [NB, block_size, Hkv, d] bf16 (caller-owned).
    max_blocks_per_seq / max_context_len: the largest table row and context a
    step may use; they size the static buffers and the captured grids.
    """

    def __init__(self, k_cache, v_cache, num_q_heads, max_blocks_per_seq, max_context_len,
                 scale, buckets=DEFAULT_BUCKETS, partition_size=0, stream=None):
        binding.load()
        self.k_cache, self.v_cache = k_cache, v_cache
        NB, bs, Hkv, d = k_cache.shape
        self.Hq, self.Hkv, self.d = num_q_heads, Hkv, d
        self.max_blocks, self.max_ctx = max_blocks_per_seq, max_context_len
        self.scale, self.part = scale, partition_size
        self.buckets = tuple(sorted(set(int(b) for b in buckets)))
        B = self.buckets[-1]
        dev = k_cache.device
        self.q = torch.zeros((B, num_q_heads, d), dtype=torch.bfloat16, device=dev)
        self.k_new = torch.zeros((B, Hkv, d), dtype=torch.bfloat16, device=dev)
        self.v_new = torch.zeros((B, Hkv, d), dtype=torch.bfloat16, device=dev)
        self.slots = torch.full((B,), -1, dtype=torch.int32, device=dev)
        self.ctx = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.tables = torch.zeros((B, max_blocks_per_seq), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, num_q_heads, d), dtype=torch.bfloat16, device=dev)
        need = max(binding.pa_decode_workspace_size(b, num_q_heads, Hkv, d, max_context_len,
                                                    partition_size) for b in self.buckets)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        self.stream = stream if stream is not None else torch.cuda.Stream()
        self.graphs = {}
        torch.cuda.synchronize()
        for b in self.buckets:
            self._launch(b)                      # warm the launch path outside capture
        torch.cuda.synchronize()
        for b in self.buckets:
            with binding.HipGraph.capture(self.stream) as g:
                self._launch(b)
            self.graphs[b] = g
        torch.cuda.synchronize()

    def _launch(self, b):
        binding.pa_decode_store(self.q[:b], self.k_new[:b], self.v_new[:b], self.slots[:b],
                                self.k_cache, self.v_cache, self.tables[:b], self.ctx[:b],
                                self.max_ctx, self.scale, workspace=self.ws, out=self.out[:b],
                                partition_size=self.part, stream=self.stream)

    def step(self, q, k_new, v_new, slot_mapping, context_lens, block_tables):
        """One decode step for S sequences (device tensors); returns out[:S] (a view
        of the static output buffer, valid until the next step)."""
        S = q.shape[0]
        b = bucket_for(S, self.buckets)
        if block_tables.shape[1] > self.max_blocks:
            raise ValueError("block table wider than the captured maximum")
        # context_lens must stay <= max_context_len (device data: the caller's contract)
        self.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            self.q[:S].copy_(q)
            self.k_new[:S].copy_(k_new)
            self.v_new[:S].copy_(v_new)
            self.slots[:S].copy_(slot_mapping)
            self.ctx[:S].copy_(context_lens)
            self.tables[:S, :block_tables.shape[1]].copy_(block_tables)
            if S < b:                            # padding rows: empty context, no store
                self.slots[S:b].fill_(-1)
                self.ctx[S:b].fill_(0)
            self.graphs[b].replay(self.stream)
        torch.cuda.current_stream().wait_stream(self.stream)
        return self.out[:S]
