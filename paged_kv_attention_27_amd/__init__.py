"""Paged KV attention for AMD MI355X (gfx950): KV-cache store, varlen causal
prefill and split-K paged decode, as hand-written HIP kernels behind the C-ABI
library ``libpa.so`` (declared in ``include/pa.h``).

The Python names mirror the C entry points; they only marshal arguments
(torch device tensors -> pointers, the current HIP stream) and raise when the
library is missing or returns an error.  See ``binding.py``.
"""
from .binding import (PaError, library_path, load, pa_decode, pa_decode_workspace_size,  # noqa: F401
                      pa_prefill_varlen, pa_prefill_workspace_size, pa_prefill_workspace,
                      pa_slot_mapping, pa_status_string, pa_store_kv,
                      pa_decode_num_partitions, pa_decode_split, pa_decode_reduce,
                      pa_decode_store, BlockManager, pa_bm_create, pa_bm_destroy,
                      pa_bm_num_free, pa_bm_ref_count, pa_bm_blocks_needed, pa_bm_allocate,
                      pa_bm_append, pa_bm_free, pa_kv_pool_layout, alloc_kv_pools,
                      pa_decode_noalloc, NOALLOC_SCRATCH_BYTES, HipGraph, pa_graph_begin,
                      pa_graph_end, pa_graph_launch, pa_graph_node_counts, pa_graph_destroy)

__all__ = ["PaError", "library_path", "load", "pa_store_kv", "pa_prefill_varlen",
           "pa_prefill_workspace_size", "pa_prefill_workspace", "pa_decode",
           "pa_decode_workspace_size", "pa_decode_num_partitions", "pa_decode_split",
           "pa_decode_reduce", "pa_decode_store", "pa_slot_mapping",
           "pa_status_string", "BlockManager", "pa_bm_create", "pa_bm_destroy",
           "pa_bm_num_free", "pa_bm_ref_count", "pa_bm_blocks_needed", "pa_bm_allocate",
           "pa_bm_append", "pa_bm_free", "pa_kv_pool_layout", "alloc_kv_pools",
           "pa_decode_noalloc", "NOALLOC_SCRATCH_BYTES", "HipGraph", "pa_graph_begin",
           "pa_graph_end", "pa_graph_launch", "pa_graph_node_counts", "pa_graph_destroy"]
