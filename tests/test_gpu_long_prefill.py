"""GPU prefill parity on long prompts, checked on sampled rows, through the C-ABI.

A 16384-token causal prompt (2048 work items of the persistent schedule) and
a 1024-token chunk over a 31744-token cached prefix (the key split of the
eight-wave form, 512 key tiles per item) are too large for the fp64 oracle
to recompute whole in seconds.  Row i of a causal prefill is the attention of
query i over keys 0 .. i alone ("Visual atlas" ch.17 and ch.21: the causal
mask leaves a query its own and earlier keys; decoding a token is the last
row of a prefill), so the oracle computes sampled rows one by one as
single-query problems over the same keys, stored into compact pools by the
oracle's own store.  The rows sampled are the first and last, both sides of
every tile and block edge near the start, the middle and the end, and
seeded random rows; each is compared over every head.
"""
import numpy as np
import pytest
import torch

from pipelines import check_close, cu_of, dev_bf16, dev_i32, host_f64, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import paged_kv_attention_27_amd as pa
    pa.load()
    return pa


def _rows(n, seed, count=24):
    """Rows 0 .. n-1 to check: edges of 64-key tiles and 256-key blocks at the
    start, the middle and the end, plus seeded random rows."""
    edges = {0, 1, 2, 63, 64, 65, 127, 128, 255, 256, 257}
    for c in (n // 2, n - 256, n - 64):
        edges |= {c - 1, c, c + 1}
    edges |= {n - 2, n - 1}
    rng = np.random.default_rng(seed)
    rand = set(rng.integers(0, n, size=count).tolist())
    return np.array(sorted(r for r in edges | rand if 0 <= r < n), dtype=np.int64)


def _oracle_rows(orc, q_rows, k_all, v_all, kcounts, bs, scale):
    """Each sampled query over its first kcounts[r] keys of k_all / v_all
    ([T, Hkv, d] bf16 bits), as a batch of one-query problems on one pool."""
    T, hkv, d = k_all.shape
    nb = -(-T // bs)
    kc = np.zeros((nb, bs, hkv, d), np.uint16)
    vc = np.zeros_like(kc)
    table = np.arange(nb, dtype=np.int32)[None, :]
    slots = orc.slot_mapping(np.array([0, T], np.int32), np.array([T], np.int32), table, bs)
    orc.store(k_all, v_all, slots, kc, vc)
    R = len(kcounts)
    bt = np.ascontiguousarray(np.repeat(table, R, axis=0))
    return orc.decode(np.ascontiguousarray(q_rows), kc, vc, bt,
                      np.asarray(kcounts, dtype=np.int32), scale)


@pytest.mark.parametrize("hq,hkv", [(16, 8), (8, 1)], ids=["g2", "g8"])
def test_prefill_long_prompt_sampled(pa, orc, hq, hkv):
    """One 16384-token causal prompt from flat K/V (persistent four-wave form)."""
    from paged_kv_attention_27_amd import workloads
    n = 16384
    wl = workloads.synthetic(q_lens=[n], k_lens=[n], num_q_heads=hq, num_kv_heads=hkv,
                             paged=False, seed=91, q_scale=4.0, v_position=True)
    ph = wl.prefill
    log(f"[long prompt {n} tokens, Hq={hq} Hkv={hkv}]")
    out = pa.pa_prefill_varlen(dev_bf16(ph.q), dev_bf16(ph.k), dev_bf16(ph.v), None, None, None,
                               dev_i32(ph.cu_seqlens_q), dev_i32(ph.cu_seqlens_k), n, n, hkv,
                               wl.scale)
    torch.cuda.synchronize()
    rows = _rows(n, 91)
    ref = _oracle_rows(orc, ph.q[rows], ph.k, ph.v, rows + 1, 256, wl.scale)
    log(f"  {len(rows)} rows sampled")
    check_close(host_f64(out[torch.from_numpy(rows).cuda()]), ref, f"long prompt g{hq // hkv}")


def test_prefill_long_prefix_key_split_sampled(pa, orc):
    """A 1024-token chunk over a 31744-token cached prefix read through the
    pools (block size 256), with and without the key-split workspace."""
    from paged_kv_attention_27_amd import workloads
    q_len, k_len, hq, hkv, bs = 1024, 32768, 16, 8, 256
    wl = workloads.synthetic(q_lens=[q_len], k_lens=[k_len], num_q_heads=hq, num_kv_heads=hkv,
                             block_size=bs, seed=92, q_scale=4.0, v_position=True)
    fx, ph = wl.prefix, wl.prefill
    log(f"[chunk {q_len} over {k_len} keys, Hq={hq} Hkv={hkv}]")
    kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    for phase in (fx, ph):
        slots = pa.pa_slot_mapping(phase.cu_seqlens_q, phase.seqlens_k, wl.block_tables, bs)
        pa.pa_store_kv(dev_bf16(phase.k), dev_bf16(phase.v), kc, vc, slots.cuda())
    ws = pa.pa_prefill_workspace(1, q_len, k_len, hq, hkv)
    assert ws.numel() > 16, "the key split was not planned"
    args = (dev_bf16(ph.q), None, None, kc, vc, dev_i32(wl.block_tables),
            dev_i32(ph.cu_seqlens_q), dev_i32(cu_of(ph.seqlens_k)), q_len, k_len, hkv, wl.scale)
    outs = {"key split": pa.pa_prefill_varlen(*args, workspace=ws),
            "unsplit": pa.pa_prefill_varlen(*args)}
    torch.cuda.synchronize()
    rows = _rows(q_len, 92)
    k_all = np.concatenate([fx.k, ph.k])
    v_all = np.concatenate([fx.v, ph.v])
    ref = _oracle_rows(orc, ph.q[rows], k_all, v_all, (k_len - q_len) + rows + 1, bs, wl.scale)
    log(f"  {len(rows)} rows sampled")
    idx = torch.from_numpy(rows).cuda()
    for label, out in outs.items():
        check_close(host_f64(out[idx]), ref, f"long prefix {label}")
