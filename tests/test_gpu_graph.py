"""Decode step (store new K/V -> split-K -> reduce) captured once in a HIP graph
and replayed with new values and new context lengths inside the captured
maxima ("nano-vLLM offline" course, item 03: replay reads new inputs and
computes new results; "Visual atlas" ch.26: preallocated buffers, values and
valid lengths may change, the shape/address contract must hold).

The graphs are the library's own (pa_graph_begin / pa_graph_end /
pa_graph_launch through the C-ABI); each captured graph is checked to hold
kernel nodes only.  Every replay is checked against a fresh oracle run on the
same inputs, with eager library calls and synchronisations between replays.
"""
import numpy as np
import pytest
import torch

from pipelines import (PREFILL_PART_BYTES, check_close, dev_bf16, dev_i32, host_f64, host_u16, log,
                       prefix_tables)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["store+decode", "fused"])
def test_decode_graph_replays(orc, fused):
    import paged_kv_attention_27_amd as pa
    from paged_kv_attention_27_amd import workloads
    S, Hq, Hkv, d, bs = 6, 16, 8, 128, 256
    cap = [300, 1024, 2048, 700, 4096, 512]          # tokens each sequence may reach
    wl = workloads.synthetic(q_lens=[1] * S, k_lens=cap, block_size=bs, seed=31)
    # history: every position below cap-1 is stored once up front
    kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    ok, ov = wl.k_cache.copy(), wl.v_cache.copy()
    ph = wl.prefix
    pa.pa_store_kv(dev_bf16(ph.k), dev_bf16(ph.v), kc, vc,
                   pa.pa_slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, prefix_tables(wl), bs).cuda())
    orc.store(ph.k, ph.v, orc.slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, prefix_tables(wl), bs),
              ok, ov)

    max_ctx = max(cap)
    bt = dev_i32(wl.block_tables)
    q_s = torch.empty((S, Hq, d), dtype=torch.bfloat16, device="cuda")
    k_s = torch.empty((S, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v_s = torch.empty((S, Hkv, d), dtype=torch.bfloat16, device="cuda")
    slots_s = torch.empty(S, dtype=torch.int32, device="cuda")
    ctx_s = torch.ones(S, dtype=torch.int32, device="cuda")
    out_s = torch.empty((S, Hq, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(pa.pa_decode_workspace_size(S, Hq, Hkv, d, max_ctx), dtype=torch.uint8,
                     device="cuda")
    slots_s.fill_(-1)   # capture-time run stores nothing
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    with pa.HipGraph.capture(stream) as graph:
        if fused:
            pa.pa_decode_store(q_s, k_s, v_s, slots_s, kc, vc, bt, ctx_s, max_ctx, wl.scale,
                               workspace=ws, out=out_s, stream=stream)
        else:
            pa.pa_store_kv(k_s, v_s, kc, vc, slots_s, stream=stream)
            pa.pa_decode(q_s, kc, vc, bt, ctx_s, max_ctx, wl.scale, workspace=ws, out=out_s,
                         stream=stream)
    torch.cuda.synchronize()
    kernels, others = graph.node_counts()
    n_part = pa.pa_decode_num_partitions(S, Hq, Hkv, max_ctx)
    assert others == 0, "the captured step holds a node that is not a kernel"
    assert kernels == (0 if fused else 1) + 1 + (n_part > 1), (kernels, n_part)

    rng = np.random.default_rng(77)
    for r in range(4):
        ctx = np.array([rng.integers(1, c + 1) for c in cap], np.int32)
        if r == 3:
            ctx = np.array(cap, np.int32)
        q = workloads.normal_bf16(rng, (S, Hq, d), 2.0)
        k = workloads.normal_bf16(rng, (S, Hkv, d))
        v = workloads.normal_bf16(rng, (S, Hkv, d))
        cu1 = np.arange(S + 1, dtype=np.int32)
        slots = pa.pa_slot_mapping(cu1, ctx, wl.block_tables, bs)
        q_s.copy_(dev_bf16(q))
        k_s.copy_(dev_bf16(k))
        v_s.copy_(dev_bf16(v))
        slots_s.copy_(slots.cuda())
        ctx_s.copy_(dev_i32(ctx))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host_f64(out_s)
        # eager work between replays: a plain call on the default stream
        eager = pa.pa_decode(dev_bf16(q), kc, vc, bt, dev_i32(ctx), max_ctx, wl.scale)
        torch.cuda.synchronize()

        orc.store(k, v, orc.slot_mapping(cu1, ctx, wl.block_tables, bs), ok, ov)
        ref = orc.decode(q, ok, ov, wl.block_tables, ctx, wl.scale)
        log(f"replay {r}: ctx={ctx.tolist()}")
        check_close(got, ref, f"graph replay {r}")
        if not fused:   # the fused path sums the new token last: same result up to rounding
            assert np.array_equal(host_u16(out_s), host_u16(eager)), "replay differs from eager call"
        else:
            check_close(got, host_f64(eager), f"graph replay {r} vs eager")
    assert np.array_equal(host_u16(kc), ok) and np.array_equal(host_u16(vc), ov)


def test_decode_graph_buckets(orc):
    """One captured graph per batch-size bucket; steps of 1..40 sequences pick the
    smallest bucket, pad it with empty contexts, and match the oracle."""
    import paged_kv_attention_27_amd as pa
    from paged_kv_attention_27_amd import workloads
    from paged_kv_attention_27_amd.decode_graphs import DecodeGraphs
    S_all, Hq, Hkv, d, bs = 40, 16, 8, 128, 256
    rng = np.random.default_rng(91)
    cap = rng.integers(2, 2049, size=S_all)
    wl = workloads.synthetic(q_lens=[1] * S_all, k_lens=cap, block_size=bs, seed=92)
    kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    ok, ov = wl.k_cache.copy(), wl.v_cache.copy()
    ph = wl.prefix
    pa.pa_store_kv(dev_bf16(ph.k), dev_bf16(ph.v), kc, vc,
                   pa.pa_slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, prefix_tables(wl), bs).cuda())
    orc.store(ph.k, ph.v, orc.slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, prefix_tables(wl), bs),
              ok, ov)
    graphs = DecodeGraphs(kc, vc, Hq, wl.block_tables.shape[1], 2048, wl.scale,
                          buckets=(1, 4, 16, 64))
    for step, S in enumerate((1, 3, 16, 17, 40, 4)):
        pick = np.sort(rng.choice(S_all, size=S, replace=False))
        ctx = np.array([rng.integers(1, cap[i] + 1) for i in pick], np.int32)
        tables = np.ascontiguousarray(wl.block_tables[pick])
        q = workloads.normal_bf16(rng, (S, Hq, d), 2.0)
        k = workloads.normal_bf16(rng, (S, Hkv, d))
        v = workloads.normal_bf16(rng, (S, Hkv, d))
        cu1 = np.arange(S + 1, dtype=np.int32)
        slots = pa.pa_slot_mapping(cu1, ctx, tables, bs)
        out = graphs.step(dev_bf16(q), dev_bf16(k), dev_bf16(v), slots.cuda(), dev_i32(ctx),
                          dev_i32(tables))
        got = host_f64(out)
        torch.cuda.synchronize()
        orc.store(k, v, orc.slot_mapping(cu1, ctx, tables, bs), ok, ov)
        ref = orc.decode(q, ok, ov, tables, ctx, wl.scale)
        log(f"bucket step {step}: S={S}")
        check_close(got, ref, f"bucket step {step} (S={S})")
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(kc), ok) and np.array_equal(host_u16(vc), ov)


@pytest.mark.parametrize("split", [False, True], ids=["persistent", "key-split"])
def test_prefill_graph_replays(orc, split):
    """The chunked prefill (store of the new tokens, then attention over the pools)
    captured once and replayed with new values: batches with more query blocks
    than two per CU take the persistent schedule, which must keep no state
    between launches; with a workspace, a batch with few blocks per CU splits
    long blocks' key ranges, and the workspace's arrival counters must come back
    to zero after every replay."""
    import paged_kv_attention_27_amd as pa
    from paged_kv_attention_27_amd import workloads
    q_lens = [700, 64, 1, 300, 129, 512, 33, 1000, 90, 257, 640, 5]
    pres = [0, 512, 40, 100, 0, 256, 7, 24, 300, 0, 64, 500]
    if split:   # few, long blocks
        q_lens, pres = [64, 300], [4000, 2000]
    k_lens = [q + p for q, p in zip(q_lens, pres)]
    wl = workloads.synthetic(q_lens=q_lens, k_lens=k_lens, block_size=256, seed=41)
    items = -(-max(q_lens) // 64) * len(q_lens) * wl.num_kv_heads
    ws = None
    if split:
        ws = pa.pa_prefill_workspace(len(q_lens), max(q_lens), max(k_lens), wl.num_q_heads,
                                     wl.num_kv_heads)
        assert pa.pa_prefill_workspace_size(len(q_lens), max(q_lens), max(k_lens), wl.num_q_heads,
                                            wl.num_kv_heads) > 0, "the batch must be split"
    else:
        assert items > 512, "the batch must take the persistent schedule"
    kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    ok, ov = wl.k_cache.copy(), wl.v_cache.copy()
    ph, fx = wl.prefill, wl.prefix
    pa.pa_store_kv(dev_bf16(fx.k), dev_bf16(fx.v), kc, vc,
                   pa.pa_slot_mapping(fx.cu_seqlens_q, fx.seqlens_k, prefix_tables(wl), 256).cuda())
    orc.store(fx.k, fx.v, orc.slot_mapping(fx.cu_seqlens_q, fx.seqlens_k, prefix_tables(wl), 256),
              ok, ov)
    slots = pa.pa_slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, wl.block_tables, 256).cuda()
    cu_q = dev_i32(ph.cu_seqlens_q)
    cu_k = dev_i32(np.concatenate([[0], np.cumsum(ph.seqlens_k)]).astype(np.int32))
    bt = dev_i32(wl.block_tables)
    q_s = torch.empty((int(ph.cu_seqlens_q[-1]), wl.num_q_heads, 128), dtype=torch.bfloat16,
                      device="cuda")
    k_s = torch.empty((int(ph.cu_seqlens_q[-1]), wl.num_kv_heads, 128), dtype=torch.bfloat16,
                      device="cuda")
    v_s = torch.empty_like(k_s)
    out_s = torch.empty_like(q_s)
    k_s.zero_(), v_s.zero_(), q_s.zero_()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with pa.HipGraph.capture(stream) as graph:
        pa.pa_store_kv(k_s, v_s, kc, vc, slots, stream=stream)
        pa.pa_prefill_varlen(q_s, None, None, kc, vc, bt, cu_q, cu_k, ph.max_seqlen_q,
                             ph.max_seqlen_k, wl.num_kv_heads, wl.scale, out=out_s,
                             stream=stream, workspace=ws)
    torch.cuda.synchronize()
    assert graph.node_counts() == (2, 0), graph.node_counts()   # store + attention kernels
    rng = np.random.default_rng(42)
    for r in range(3):
        q = workloads.normal_bf16(rng, tuple(q_s.shape), 2.0 if r == 1 else 1.0)
        k = workloads.normal_bf16(rng, tuple(k_s.shape))
        v = workloads.normal_bf16(rng, tuple(v_s.shape))
        q_s.copy_(dev_bf16(q)), k_s.copy_(dev_bf16(k)), v_s.copy_(dev_bf16(v))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host_f64(out_s)
        if split:
            assert int(ws.count_nonzero()) > 0                    # the partials are there ...
            n_items = ws.numel() // (2 * PREFILL_PART_BYTES + 4)
            tail = ws[ws.numel() - 4 * n_items:]
            assert int(tail.count_nonzero()) == 0, "arrival counters not reset"   # ... not the counts
        eager = pa.pa_prefill_varlen(dev_bf16(q), None, None, kc, vc, bt, cu_q, cu_k,
                                     ph.max_seqlen_q, ph.max_seqlen_k, wl.num_kv_heads, wl.scale,
                                     workspace=ws)
        torch.cuda.synchronize()
        orc.store(k, v, orc.slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, wl.block_tables, 256),
                  ok, ov)
        ref = orc.attention(q, ph.cu_seqlens_q, k_cache=ok, v_cache=ov,
                            block_tables=wl.block_tables, seqlens_k=ph.seqlens_k, scale=wl.scale)
        log(f"prefill replay {r}")
        check_close(got, ref, f"prefill graph replay {r}")
        if split:   # which half merges is a race, so only the tolerance binds
            check_close(host_f64(eager), ref, f"prefill eager call {r}")
        else:
            assert np.array_equal(host_u16(out_s), host_u16(eager)), "replay differs from eager call"
    assert np.array_equal(host_u16(kc), ok) and np.array_equal(host_u16(vc), ov)


def test_graph_api_errors():
    """The capture calls' error paths on a real stream: ending a capture that never
    began, a failure inside a capture (the capture still ends and the stream works
    afterwards), and NULL arguments."""
    import ctypes
    import paged_kv_attention_27_amd as pa
    lib = pa.load()
    stream = torch.cuda.Stream()
    h = ctypes.c_void_p(123)
    assert lib.pa_graph_end(ctypes.c_void_p(stream.cuda_stream), ctypes.byref(h)) == 7   # GRAPH
    assert h.value is None
    x = torch.zeros(4, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        with pa.HipGraph.capture(stream):
            raise ValueError("inside the capture")
    assert lib.pa_graph_launch(None, ctypes.c_void_p(stream.cuda_stream)) == 1          # NULL
    with torch.cuda.stream(stream):
        x.add_(1)                           # the stream is out of capture again
    torch.cuda.synchronize()
    assert float(x[0]) == 1.0
    with pa.HipGraph.capture(stream) as g:   # an empty capture instantiates
        pass
    assert g.node_counts() == (0, 0)
    g.replay()
    torch.cuda.synchronize()
    g.close()
