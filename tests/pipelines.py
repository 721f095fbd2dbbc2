"""Run one workload through the HIP library and through the CPU oracle.

Both sides start from the same arrays drawn by ``workloads``; each computes its
own slot mapping (the library's host routine on one side, the oracle's on the
other) and applies the phases in the same order: cached prefix store, prefill
store + attention, decode store + attention.  Nothing computed by one side is
fed to the other.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

PARITY_MAX = 2e-2    # max |gpu - oracle| on bf16 outputs (spec tolerance)
PARITY_MEAN = 2e-3   # mean |gpu - oracle|
# bytes of one half's partial in the prefill key-split workspace (include/pa.h): fp32 O / l
# [4 waves][64][64 lanes], then fp32 max and sum [4 waves][2][64 lanes]
PREFILL_PART_BYTES = (4 * 64 * 64 + 4 * 2 * 64) * 4


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_pools(pa, wl):
    """The workload's initial pools on the GPU in one allocation, placed as
    pa_kv_pool_layout recommends (the layout the benchmark times)."""
    nb, bs, hkv, d = wl.k_cache.shape
    kc, vc = pa.alloc_kv_pools(nb, bs, hkv, d)
    kc.copy_(dev_bf16(wl.k_cache))
    vc.copy_(dev_bf16(wl.v_cache))
    return kc, vc


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def cu_of(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def prefix_tables(wl):
    if "prefix_seq" in wl.extra:
        s = wl.extra["prefix_seq"]
        return np.ascontiguousarray(wl.block_tables[s:s + 1])
    return wl.block_tables


def check_close(gpu, ref, label, max_tol=PARITY_MAX, mean_tol=PARITY_MEAN):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if gpu.size == 0:   # e.g. a prefill whose every chunk is empty
        log(f"  {label}: empty output, shapes agree")
        return 0.0, 0.0
    assert np.isfinite(gpu).all(), f"{label}: non-finite GPU output"
    err = np.abs(gpu - ref)
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {label}: max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert mx <= max_tol and mean <= mean_tol, f"{label}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def gpu_pipeline(pa, wl, partition_size=0, keep_pools=True, one_allocation=True):
    """Run every phase of ``wl`` through libpa, with both pools in one allocation
    (pa_kv_pool_layout) or in two.  Returns host results."""
    if one_allocation:
        kc, vc = dev_pools(pa, wl)
    else:
        kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    bt = dev_i32(wl.block_tables)
    res = {}

    def store(phase, tables):
        slots = pa.pa_slot_mapping(phase.cu_seqlens_q, phase.seqlens_k, tables, wl.block_size)
        pa.pa_store_kv(dev_bf16(phase.k), dev_bf16(phase.v), kc, vc, slots.cuda())

    if wl.prefix is not None:
        store(wl.prefix, prefix_tables(wl))
    if wl.prefill is not None:
        ph = wl.prefill
        store(ph, wl.block_tables)
        q = dev_bf16(ph.q)
        cu_q = dev_i32(ph.cu_seqlens_q)
        if ph.paged:
            out = pa.pa_prefill_varlen(q, None, None, kc, vc, bt, cu_q, dev_i32(cu_of(ph.seqlens_k)),
                                       ph.max_seqlen_q, ph.max_seqlen_k, wl.num_kv_heads, wl.scale)
        else:
            out = pa.pa_prefill_varlen(q, dev_bf16(ph.k), dev_bf16(ph.v), None, None, None, cu_q,
                                       dev_i32(ph.cu_seqlens_k), ph.max_seqlen_q, ph.max_seqlen_k,
                                       wl.num_kv_heads, wl.scale)
        res["prefill"] = host_f64(out)
        res["prefill_bits"] = host_u16(out)
    if wl.decode is not None:
        ph = wl.decode
        store(ph, wl.block_tables)
        out = pa.pa_decode(dev_bf16(ph.q), kc, vc, bt, dev_i32(ph.seqlens_k), ph.max_seqlen_k,
                           wl.scale, partition_size=partition_size)
        res["decode"] = host_f64(out)
        res["decode_bits"] = host_u16(out)
    torch.cuda.synchronize()
    if keep_pools:
        res["k_cache"] = host_u16(kc)
        res["v_cache"] = host_u16(vc)
    del kc, vc
    return res


def oracle_pipeline(orc, wl, keep_pools=True, attention=True):
    kc = wl.k_cache.copy()
    vc = wl.v_cache.copy()
    res = {}

    def store(phase, tables):
        slots = orc.slot_mapping(phase.cu_seqlens_q, phase.seqlens_k, tables, wl.block_size)
        orc.store(phase.k, phase.v, slots, kc, vc)

    if wl.prefix is not None:
        store(wl.prefix, prefix_tables(wl))
    if wl.prefill is not None:
        ph = wl.prefill
        store(ph, wl.block_tables)
        if attention:
            if ph.paged:
                res["prefill"] = orc.attention(ph.q, ph.cu_seqlens_q, k_cache=kc, v_cache=vc,
                                               block_tables=wl.block_tables,
                                               seqlens_k=ph.seqlens_k, scale=wl.scale)
            else:
                res["prefill"] = orc.attention(ph.q, ph.cu_seqlens_q, k=ph.k, v=ph.v,
                                               cu_seqlens_k=ph.cu_seqlens_k, scale=wl.scale)
    if wl.decode is not None:
        ph = wl.decode
        store(ph, wl.block_tables)
        if attention:
            res["decode"] = orc.decode(ph.q, kc, vc, wl.block_tables, ph.seqlens_k, wl.scale)
    if keep_pools:
        res["k_cache"] = kc
        res["v_cache"] = vc
    return res
