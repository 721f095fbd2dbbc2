"""GPU decode parity on very long contexts, through the C-ABI.

A context of 2^19 keys at Hq 8 / Hkv 1 (the MFMA decode kernel) and of
131072 keys at Hq 16 / Hkv 8 (the dot-product kernel) is split into
thousands of partitions when the caller asks for short ones: the reduce then
walks the partials in several passes of its LDS stage, which the shorter
parity cases never reach.  The fused step on the library's own plan covers
the same contexts with its shrinking partitions.  Every variant is checked
against the fp64 oracle's store-then-decode ("Visual atlas" ch.21: one new
query attends every cached key of its sequence; ch.22: partials merged by
the log-sum-exp rule).
"""
import numpy as np
import pytest
import torch

from pipelines import check_close, dev_bf16, dev_i32, host_f64, host_u16, log

pytestmark = pytest.mark.gpu

LONG_CASES = {
    # (Hq, Hkv, block size, contexts, explicit partition sizes)
    "g8-512k": (8, 1, 256, [1 << 19], [256]),
    "g8-262k-p32": (8, 1, 256, [262144, 70001, 1], [32]),
    "g2-131k-bs16-p96": (16, 8, 16, [131072, 5], [96]),
}


@pytest.fixture(scope="module")
def pa():
    import paged_kv_attention_27_amd as pa
    pa.load()
    return pa


@pytest.mark.parametrize("case", list(LONG_CASES))
def test_decode_long_context(pa, orc, case):
    from paged_kv_attention_27_amd import workloads
    hq, hkv, bs, ctx, parts = LONG_CASES[case]
    wl = workloads.synthetic(q_lens=[1] * len(ctx), k_lens=ctx, num_q_heads=hq, num_kv_heads=hkv,
                             block_size=bs, seed=81, q_scale=4.0, v_position=True)
    fx, ph = wl.prefix, wl.prefill
    log(f"[long-context decode {case}: contexts {ctx}]")
    kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    slots = pa.pa_slot_mapping(fx.cu_seqlens_q, fx.seqlens_k, wl.block_tables, bs)
    pa.pa_store_kv(dev_bf16(fx.k), dev_bf16(fx.v), kc, vc, slots.cuda())
    q, bt, cl = dev_bf16(ph.q), dev_i32(wl.block_tables), dev_i32(ph.seqlens_k)
    new_slots = pa.pa_slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, wl.block_tables, bs)
    outs = {"fused, library plan": pa.pa_decode_store(q, dev_bf16(ph.k), dev_bf16(ph.v),
                                                      new_slots.cuda(), kc, vc, bt, cl,
                                                      max(ctx), wl.scale)}
    counts = {"library plan": pa.pa_decode_num_partitions(len(ctx), hq, hkv, max(ctx))}
    for part in parts:
        outs[f"split + reduce, {part}-key partitions"] = pa.pa_decode(
            q, kc, vc, bt, cl, max(ctx), wl.scale, partition_size=part)
        counts[part] = pa.pa_decode_num_partitions(len(ctx), hq, hkv, max(ctx), part)
    torch.cuda.synchronize()
    log(f"  partitions of the longest context: {counts}")
    assert max(counts[p] for p in parts) > 512, "the reduce never runs a second pass"

    okc, ovc = wl.k_cache.copy(), wl.v_cache.copy()
    for phase in (fx, ph):
        orc.store(phase.k, phase.v, orc.slot_mapping(phase.cu_seqlens_q, phase.seqlens_k,
                                                     wl.block_tables, bs), okc, ovc)
    ref = orc.decode(ph.q, okc, ovc, wl.block_tables, ph.seqlens_k, wl.scale)
    assert np.array_equal(host_u16(kc), okc) and np.array_equal(host_u16(vc), ovc), "pools differ"
    for label, out in outs.items():
        check_close(host_f64(out), ref, f"{case} {label}")
