"""GPU parity with pools larger than 4 GiB, through the C-ABI.

A device holds pools of hundreds of GB, so block ids whose byte offsets need
more than 32 bits are the normal case in service.  Every pool access (the
store, the paged prefill in its tile, per-row and key-split forms, both decode
kernels and the fused step) must form its addresses in 64 bits.  Here the
blocks a workload uses sit at id 0, at the block ending on the 2 GiB boundary
and above 4 GiB, with both pools in the one allocation the library recommends
(so every V address lies past 4 GiB too).  The rest of each pool is NaN, so a
read of any other block poisons the output, and a write outside the used
blocks shows up in a count of the pools' non-NaN elements.

The oracle runs on the workload's compact pools with the original tables:
attention does not depend on where a block is placed ("Visual atlas" ch.25:
the block table maps logical to physical blocks), which the oracle's
placement-invariance pin fixes.
"""
import numpy as np
import pytest
import torch

from pipelines import (PREFILL_PART_BYTES, check_close, cu_of, dev_bf16, dev_i32, host_f64,
                       host_u16, log, oracle_pipeline)

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0    # the pools' fill: a bf16 NaN


@pytest.fixture(scope="module")
def pa():
    import paged_kv_attention_27_amd as pa
    pa.load()
    return pa


@pytest.fixture(autouse=True)
def _release_pools():
    """Hand the 8 GiB of pools back to the device after each case."""
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _wl(**kw):
    from paged_kv_attention_27_amd import workloads
    return workloads.synthetic(**kw)


def _big_pools(pa, wl, seed):
    """NaN-filled pools of more than 4 GiB each (one allocation, the library's
    placement) and the workload's tables mapped onto them: one used block at
    id 0, one ending on the 2 GiB byte boundary, the rest past 4 GiB, in a
    seeded order.  Returns (k_cache, v_cache, tables, remap)."""
    nb, bs, hkv, d = wl.k_cache.shape
    blk = bs * hkv * d * 2
    lo = -(-(1 << 32) // blk)      # first block whose bytes start at or past 4 GiB
    mid = (1 << 31) // blk - 1     # the block that ends on the 2 GiB boundary
    rng = np.random.default_rng(seed)
    order = rng.permutation(nb)
    remap = np.empty(nb, np.int64)
    remap[order[0]] = 0
    remap[order[1]] = mid
    remap[order[2:]] = lo + rng.permutation(nb - 2)
    kc, vc = pa.alloc_kv_pools(lo + nb - 2, bs, hkv, d)
    kc.view(torch.int16).fill_(NAN_BITS)
    vc.view(torch.int16).fill_(NAN_BITS)
    bt = wl.block_tables
    tables = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    log(f"  pools: {kc.numel() * 2 / 2**30:.2f} GiB each, used block ids 0, {mid}, "
        f"{lo}..{lo + nb - 3}")
    return kc, vc, tables, remap


def _check_pools(kc, vc, remap, okc, ovc):
    """The used blocks equal the oracle's pools bit for bit and nothing else
    was written."""
    idx = torch.from_numpy(remap).cuda()
    for big, ref, name in ((kc, okc, "k_cache"), (vc, ovc, "v_cache")):
        used = big[idx]
        assert np.array_equal(host_u16(used), ref), f"{name}: used blocks differ"
        written = int((big.view(torch.int16) != NAN_BITS).sum())
        assert written == int((used.view(torch.int16) != NAN_BITS).sum()), \
            f"{name}: elements written outside the used blocks"


def _store(pa, kc, vc, phase, tables, bs):
    slots = pa.pa_slot_mapping(phase.cu_seqlens_q, phase.seqlens_k, tables, bs)
    pa.pa_store_kv(dev_bf16(phase.k), dev_bf16(phase.v), kc, vc, slots.cuda())


PREFILL_CASES = {
    # (Hq, Hkv, block size, q_lens, k_lens, key split)
    "g2-tile": (16, 8, 256, [64, 300, 1, 700], [600, 1500, 2000, 700], False),
    "g4-tile64": (32, 8, 64, [129, 5, 450], [1000, 5, 1200], False),
    "g8-row": (8, 1, 16, [64, 300, 1, 700], [600, 1500, 2000, 700], False),
    "g2-split": (16, 8, 256, [64], [4096], True),
}


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_large_pool_prefill(pa, orc, case):
    """Cached-prefix store and paged prefill over pools past 4 GiB: per-tile
    paging (block sizes 256 and 64), per-row paging (block size 16) and the
    key split of a long chunk (the eight-wave form), against the oracle on
    compact pools."""
    hq, hkv, bs, q_lens, k_lens, split = PREFILL_CASES[case]
    wl = _wl(q_lens=q_lens, k_lens=k_lens, num_q_heads=hq, num_kv_heads=hkv, block_size=bs,
             seed=71, q_scale=4.0, v_position=True)
    log(f"[large pool prefill {case}]")
    kc, vc, tables, remap = _big_pools(pa, wl, 71)
    if wl.prefix is not None:
        _store(pa, kc, vc, wl.prefix, tables, bs)
    ph = wl.prefill
    _store(pa, kc, vc, ph, tables, bs)
    ws = None
    if split:
        ws = pa.pa_prefill_workspace(len(q_lens), ph.max_seqlen_q, ph.max_seqlen_k, hq, hkv)
        assert ws.numel() >= 2 * PREFILL_PART_BYTES, "the key split was not planned"
    out = pa.pa_prefill_varlen(dev_bf16(ph.q), None, None, kc, vc, dev_i32(tables),
                               dev_i32(ph.cu_seqlens_q), dev_i32(cu_of(ph.seqlens_k)),
                               ph.max_seqlen_q, ph.max_seqlen_k, hkv, wl.scale, workspace=ws)
    torch.cuda.synchronize()
    o = oracle_pipeline(orc, wl)
    _check_pools(kc, vc, remap, o["k_cache"], o["v_cache"])
    check_close(host_f64(out), o["prefill"], f"large pool prefill {case}")


@pytest.mark.parametrize("hq,hkv,bs", [(16, 8, 256), (8, 2, 256), (8, 1, 256), (8, 1, 16)],
                         ids=["g2", "g4", "g8", "g8-bs16"])
def test_large_pool_decode(pa, orc, hq, hkv, bs):
    """The fused decode step (new token stored past 4 GiB, library partition
    plan) and the split + reduce passes with 512-key partitions over pools
    past 4 GiB, for both decode kernels (dot product for g <= 4, MFMA for
    g = 8) and for the block-in-partition and per-row table paths."""
    ctx = [1, 700, 5000, 9000]
    wl = _wl(q_lens=[1] * len(ctx), k_lens=ctx, num_q_heads=hq, num_kv_heads=hkv, block_size=bs,
             seed=72, q_scale=2.0, v_position=True)
    label = f"large pool decode Hq={hq} Hkv={hkv} bs={bs}"
    log(f"[{label}]")
    kc, vc, tables, remap = _big_pools(pa, wl, 72)
    okc, ovc = wl.k_cache.copy(), wl.v_cache.copy()
    fx, ph = wl.prefix, wl.prefill
    _store(pa, kc, vc, fx, tables, bs)
    orc.store(fx.k, fx.v, orc.slot_mapping(fx.cu_seqlens_q, fx.seqlens_k, wl.block_tables, bs),
              okc, ovc)
    slots = pa.pa_slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, tables, bs)
    assert int(slots.max()) * hkv * 128 * 2 >= 1 << 32, "new tokens not stored past 4 GiB"
    q, bt, cl = dev_bf16(ph.q), dev_i32(tables), dev_i32(ph.seqlens_k)
    fused = pa.pa_decode_store(q, dev_bf16(ph.k), dev_bf16(ph.v), slots.cuda(), kc, vc, bt, cl,
                               max(ctx), wl.scale)
    split = pa.pa_decode(q, kc, vc, bt, cl, max(ctx), wl.scale, partition_size=512)
    torch.cuda.synchronize()
    orc.store(ph.k, ph.v, orc.slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, wl.block_tables, bs),
              okc, ovc)
    ref = orc.decode(ph.q, okc, ovc, wl.block_tables, ph.seqlens_k, wl.scale)
    _check_pools(kc, vc, remap, okc, ovc)
    check_close(host_f64(fused), ref, label + " fused")
    check_close(host_f64(split), ref, label + " split + reduce")
