"""GPU parity on seeded random problem shapes, through the C-ABI.

The other parity tests pick their shapes by hand; this sweep draws them:
every combination of KV heads (1, 2, 4, 8) and group size (1, 2, 4, 8), block
sizes from 1 to 768 including odd and non-power-of-two ones, 1 to 9
sequences whose lengths mix a few keys, tile-edge lengths and several
thousand keys, cached prefixes or flat prompts, empty chunks, peaky or
position-coded inputs, the prefill with or without a key-split workspace,
and the decode step (fused store, then split + reduce) on the library plan or
on a drawn partition size.  Every case is checked against the fp64 oracle:
pools bit for bit, outputs within the parity tolerance.  The draw of case i
depends only on i, so a failure names a case that can be rerun alone.
"""
import numpy as np
import pytest
import torch

from pipelines import (check_close, cu_of, dev_bf16, dev_i32, host_f64, host_u16, log,
                       oracle_pipeline, prefix_tables)

pytestmark = pytest.mark.gpu

N_CASES = 64
MAC_BUDGET = 1.2e9     # oracle multiply-adds per case (keeps the sweep to seconds)
BLOCK_SIZES = [1, 2, 3, 8, 16, 32, 48, 64, 96, 128, 256, 512, 768]
PARTITIONS = [0, 0, 32, 64, 96, 160, 512, 1024, 4096]


@pytest.fixture(scope="module")
def pa():
    import paged_kv_attention_27_amd as pa
    pa.load()
    return pa


def draw(i):
    """The problem of case i (host integers and flags only)."""
    rng = np.random.default_rng(5000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.integers(1, 10))
    kinds = rng.random(S)
    k_lens = np.where(kinds < 0.3, rng.integers(1, 130, S),
                      np.where(kinds < 0.8, rng.integers(130, 1600, S), rng.integers(1600, 6000, S)))
    paged = bool(rng.random() < 0.75)
    if paged:
        q_lens = np.minimum(k_lens, rng.integers(0, 700, S))
        q_lens[rng.random(S) < 0.15] = 0
    else:
        q_lens = k_lens.copy()
    macs = lambda: float((q_lens * k_lens).sum()) * g * hkv * 256
    while macs() > MAC_BUDGET:   # shrink the longest chunk until the oracle stays fast
        s = int(np.argmax(q_lens * k_lens))
        if paged:
            q_lens[s] //= 2
        else:
            k_lens[s] = q_lens[s] = max(1, k_lens[s] // 2)
    return dict(hq=g * hkv, hkv=hkv, bs=int(rng.choice(BLOCK_SIZES)), paged=paged,
                q_lens=[int(x) for x in q_lens], k_lens=[int(x) for x in k_lens],
                q_scale=float(rng.choice([1.0, 4.0])), v_position=bool(rng.random() < 0.5),
                split_ws=bool(rng.random() < 0.5), part=int(rng.choice(PARTITIONS)))


def _prefill(pa, orc, c, i):
    from paged_kv_attention_27_amd import workloads
    wl = workloads.synthetic(q_lens=c["q_lens"], k_lens=c["k_lens"], num_q_heads=c["hq"],
                             num_kv_heads=c["hkv"], block_size=c["bs"], paged=c["paged"],
                             seed=6000 + i, q_scale=c["q_scale"], v_position=c["v_position"])
    kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    bs = wl.block_size
    for ph, tables in ((wl.prefix, prefix_tables(wl)), (wl.prefill, wl.block_tables)):
        if ph is not None:
            slots = pa.pa_slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, tables, bs)
            pa.pa_store_kv(dev_bf16(ph.k), dev_bf16(ph.v), kc, vc, slots.cuda())
    ph = wl.prefill
    ws = None
    if c["split_ws"]:
        ws = pa.pa_prefill_workspace(len(c["q_lens"]), ph.max_seqlen_q, ph.max_seqlen_k, c["hq"],
                                     c["hkv"])
    if ph.paged:
        out = pa.pa_prefill_varlen(dev_bf16(ph.q), None, None, kc, vc, dev_i32(wl.block_tables),
                                   dev_i32(ph.cu_seqlens_q), dev_i32(cu_of(ph.seqlens_k)),
                                   ph.max_seqlen_q, ph.max_seqlen_k, c["hkv"], wl.scale,
                                   workspace=ws)
    else:
        out = pa.pa_prefill_varlen(dev_bf16(ph.q), dev_bf16(ph.k), dev_bf16(ph.v), None, None,
                                   None, dev_i32(ph.cu_seqlens_q), dev_i32(ph.cu_seqlens_k),
                                   ph.max_seqlen_q, ph.max_seqlen_k, c["hkv"], wl.scale,
                                   workspace=ws)
    torch.cuda.synchronize()
    o = oracle_pipeline(orc, wl)
    assert np.array_equal(host_u16(kc), o["k_cache"]) and np.array_equal(host_u16(vc), o["v_cache"])
    check_close(host_f64(out), o["prefill"], f"case {i} prefill")


def _decode(pa, orc, c, i):
    from paged_kv_attention_27_amd import workloads
    ctx = c["k_lens"]
    wl = workloads.synthetic(q_lens=[1] * len(ctx), k_lens=ctx, num_q_heads=c["hq"],
                             num_kv_heads=c["hkv"], block_size=c["bs"], seed=7000 + i,
                             q_scale=c["q_scale"], v_position=c["v_position"])
    bs = wl.block_size
    fx, ph = wl.prefix, wl.prefill
    kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    okc, ovc = wl.k_cache.copy(), wl.v_cache.copy()
    if fx is not None:
        slots = pa.pa_slot_mapping(fx.cu_seqlens_q, fx.seqlens_k, wl.block_tables, bs)
        pa.pa_store_kv(dev_bf16(fx.k), dev_bf16(fx.v), kc, vc, slots.cuda())
        orc.store(fx.k, fx.v, orc.slot_mapping(fx.cu_seqlens_q, fx.seqlens_k, wl.block_tables, bs),
                  okc, ovc)
    q, bt, cl = dev_bf16(ph.q), dev_i32(wl.block_tables), dev_i32(ph.seqlens_k)
    new_slots = pa.pa_slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, wl.block_tables, bs)
    part = c["part"]
    fused = pa.pa_decode_store(q, dev_bf16(ph.k), dev_bf16(ph.v), new_slots.cuda(), kc, vc, bt, cl,
                               max(ctx), wl.scale, partition_size=part)
    split = pa.pa_decode(q, kc, vc, bt, cl, max(ctx), wl.scale, partition_size=part)
    torch.cuda.synchronize()
    orc.store(ph.k, ph.v, orc.slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, wl.block_tables, bs),
              okc, ovc)
    ref = orc.decode(ph.q, okc, ovc, wl.block_tables, ph.seqlens_k, wl.scale)
    assert np.array_equal(host_u16(kc), okc) and np.array_equal(host_u16(vc), ovc)
    check_close(host_f64(fused), ref, f"case {i} fused decode")
    check_close(host_f64(split), ref, f"case {i} decode")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(pa, orc, i):
    c = draw(i)
    log(f"[random case {i}: {c}]")
    _prefill(pa, orc, c, i)
    _decode(pa, orc, c, i)
