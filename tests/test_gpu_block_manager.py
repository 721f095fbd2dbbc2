"""Block tables and cached-prefix lengths from the host block manager driving the
GPU path: slot mapping -> KV store of the uncached tail -> chunked causal
prefill over the pools -> decode steps with the fused store.

A position's K/V here is a deterministic function of the salt and the whole
token prefix up to it (as a model's would be), so a prefix hit is only correct
if the shared block really holds that prefix's rows.  The reference attention
is the oracle over each sequence's own flat K/V (no pool, no tables), so it
does not depend on the manager at all; the pools are also compared bit for bit
with the rows every live sequence expects at every position.

Sources: block tables map logical to physical blocks and only ids move
("nano-vLLM offline" course, THE IMPORTANT DETAILS item 02); after a prefix hit
the query covers the uncached tail while keys cover the whole prompt ("Visual
atlas" ch.26); the decode token's K/V is written before attention ("nano-vLLM
offline" course, ACCURACY & SCOPE).
"""
import numpy as np
import pytest
import torch

from pipelines import check_close, cu_of, dev_bf16, dev_i32, host_f64, host_u16, log

pytestmark = pytest.mark.gpu

MASK = (1 << 64) - 1


class KV:
    """K/V rows of a position from (salt, tokens[:pos+1]), memoised by prefix hash."""

    def __init__(self, Hkv, d):
        self.Hkv, self.d, self.memo = Hkv, d, {}

    def rows(self, salt, toks, lo, hi):
        from paged_kv_attention_27_amd.workloads import f32_to_bf16_bits
        h = (salt * 0x9E3779B97F4A7C15 + 12345) & MASK
        k = np.empty((hi - lo, self.Hkv, self.d), np.uint16)
        v = np.empty_like(k)
        for p in range(hi):
            h = ((h ^ (toks[p] + 0x51ED27)) * 0x100000001B3) & MASK
            if p < lo:
                continue
            if h not in self.memo:
                g = np.random.default_rng(h)
                self.memo[h] = tuple(
                    f32_to_bf16_bits(g.standard_normal((self.Hkv, self.d), dtype=np.float32))
                    for _ in range(2))
            k[p - lo], v[p - lo] = self.memo[h]
        return k, v


@pytest.mark.parametrize("bs", [16, 64])
def test_block_manager_prefix_reuse_end_to_end(bs, orc):
    import paged_kv_attention_27_amd as pa
    from paged_kv_attention_27_amd.binding import BlockManager
    from paged_kv_attention_27_amd.workloads import BF16_NAN, normal_bf16
    Hq, Hkv, d = 8, 2, 128
    scale = float(np.float32(1.0 / np.sqrt(d)))
    maxb = -(-400 // bs)
    NB = max(3 * 1300 // bs, 40)
    rng = np.random.default_rng(4242 + bs)
    kv = KV(Hkv, d)
    kc = torch.full((NB, bs, Hkv, d), int(BF16_NAN), dtype=torch.int16, device="cuda")
    kc = kc.view(torch.bfloat16)
    vc = kc.clone()
    bm = BlockManager(NB, bs)
    systems = [[int(x) for x in rng.integers(0, 1000, size=n)] for n in (70, 130, 200)]
    live = []          # dicts: toks, salt, table (CPU int32 [maxb])
    stats = {"cached": 0}

    def tail(n):
        return [int(x) for x in rng.integers(0, 1000, size=n)]

    def admit(reqs, label):
        """Allocate, store the uncached tails and run one chunked prefill batch."""
        batch = []
        for toks, salt in reqs:
            table, cached = bm.allocate(toks, maxb, salt)
            stats["cached"] += cached
            batch.append(dict(toks=toks, salt=salt, table=table, cached=cached))
        n_new = [len(r["toks"]) - r["cached"] for r in batch]
        n_all = [len(r["toks"]) for r in batch]
        log(f"[bs{bs}] {label}: lens={n_all} cached={[r['cached'] for r in batch]}")
        cu_q, cu_k = cu_of(n_new), cu_of(n_all)
        tables = np.stack([r["table"].numpy() for r in batch])
        k_new, v_new, k_all, v_all = [], [], [], []
        for r in batch:
            kn, vn = kv.rows(r["salt"], r["toks"], r["cached"], len(r["toks"]))
            ka, va = kv.rows(r["salt"], r["toks"], 0, len(r["toks"]))
            k_new.append(kn), v_new.append(vn), k_all.append(ka), v_all.append(va)
        k_new, v_new = np.concatenate(k_new), np.concatenate(v_new)
        k_all, v_all = np.concatenate(k_all), np.concatenate(v_all)
        q = normal_bf16(rng, (int(cu_q[-1]), Hq, d))
        slots = pa.pa_slot_mapping(cu_q, np.array(n_all, np.int32), tables, bs)
        pa.pa_store_kv(dev_bf16(k_new), dev_bf16(v_new), kc, vc, slots.cuda())
        out = pa.pa_prefill_varlen(dev_bf16(q), None, None, kc, vc, dev_i32(tables),
                                   dev_i32(cu_q), dev_i32(cu_k), max(n_new), max(n_all), Hkv,
                                   scale)
        got = host_f64(out)
        ref = orc.attention(q, cu_q, k=k_all, v=v_all, cu_seqlens_k=cu_k, scale=scale)
        check_close(got, ref, f"bs{bs} {label} prefill")
        live.extend(batch)

    def decode_step(label):
        S = len(live)
        for r in live:
            r["toks"].append(int(rng.integers(0, 1000)))
            bm.append(r["toks"], r["table"], r["salt"])
        ctx = np.array([len(r["toks"]) for r in live], np.int32)
        tables = np.stack([r["table"].numpy() for r in live])
        slots = pa.pa_slot_mapping(np.arange(S + 1, dtype=np.int32), ctx, tables, bs)
        k_new = np.concatenate([kv.rows(r["salt"], r["toks"], len(r["toks"]) - 1,
                                        len(r["toks"]))[0] for r in live])
        v_new = np.concatenate([kv.rows(r["salt"], r["toks"], len(r["toks"]) - 1,
                                        len(r["toks"]))[1] for r in live])
        q = normal_bf16(rng, (S, Hq, d))
        out = pa.pa_decode_store(dev_bf16(q), dev_bf16(k_new), dev_bf16(v_new), slots.cuda(),
                                 kc, vc, dev_i32(tables), dev_i32(ctx), int(ctx.max()), scale)
        got = host_f64(out)
        k_all = np.concatenate([kv.rows(r["salt"], r["toks"], 0, len(r["toks"]))[0]
                                for r in live])
        v_all = np.concatenate([kv.rows(r["salt"], r["toks"], 0, len(r["toks"]))[1]
                                for r in live])
        ref = orc.attention(q, np.arange(S + 1, dtype=np.int32), k=k_all, v=v_all,
                            cu_seqlens_k=cu_of(ctx), scale=scale)
        check_close(got, ref, f"bs{bs} {label}")

    def check_pools(label):
        torch.cuda.synchronize()
        hk, hv = host_u16(kc), host_u16(vc)
        for r in live:
            n = len(r["toks"])
            ids = r["table"].numpy()[: -(-n // bs)]
            got_k = hk[ids].reshape(-1, Hkv, d)[:n]
            got_v = hv[ids].reshape(-1, Hkv, d)[:n]
            want_k, want_v = kv.rows(r["salt"], r["toks"], 0, n)
            assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v), \
                f"{label}: pool rows of a live sequence differ"
        log(f"[bs{bs}] {label}: pools hold every live sequence's rows")

    s0, s1, s2 = systems
    admit([(s0 + tail(30), 0), (s0 + tail(5), 0), (s1 + tail(64), 0), (s2 + tail(1), 0),
           (tail(50), 0)], "wave 1")
    check_pools("after wave 1")
    decode_step("decode 1")
    # two requests finish; their blocks are free but keep their content
    for i in (3, 1):
        bm.free(live.pop(i)["table"])
    fork = list(live[0]["toks"])
    admit([(s0 + tail(17), 0), (fork + tail(40), 0), (s1 + tail(9), 1), (s2 + tail(33), 0),
           (list(s1), 0)], "wave 2")
    check_pools("after wave 2")
    for step in range(2, 5):
        decode_step(f"decode {step}")
    check_pools("after decode")
    assert stats["cached"] >= 4 * bs, "the workload must exercise prefix hits"
    held = {}
    for r in live:
        for x in r["table"].tolist():
            if x >= 0:
                held[x] = held.get(x, 0) + 1
    assert bm.num_free() == NB - len(held)
    assert all(bm.ref_count(x) == c for x, c in held.items())
    for r in live:
        bm.free(r["table"])
    assert bm.num_free() == NB


def test_block_manager_prefix_prefill_tables(orc):
    """The shared-prefix chunked prefill shape (16 sequences behind one 512-token
    prefix, chunks U[64,1024], Hq16/Hkv8, block size 256) with every table and
    cached length produced by the block manager in one admission batch: the
    first request stores the prefix, the other fifteen hit it."""
    import paged_kv_attention_27_amd as pa
    from paged_kv_attention_27_amd.binding import BlockManager
    from paged_kv_attention_27_amd.workloads import BF16_NAN, normal_bf16
    Hq, Hkv, d, bs, NB, P = 16, 8, 128, 256, 128, 512
    scale = float(np.float32(1.0 / np.sqrt(d)))
    rng = np.random.default_rng(27003)
    prefix = [int(x) for x in rng.integers(0, 32000, size=P)]
    chunks = rng.integers(64, 1024, size=16, endpoint=True)
    reqs = [prefix + [int(x) for x in rng.integers(0, 32000, size=int(n))] for n in chunks]
    bm = BlockManager(NB, bs)
    maxb = -(-(P + 1024) // bs)
    alloc = [bm.allocate(r, maxb) for r in reqs]
    cached = [c for _, c in alloc]
    assert cached == [0] + [P] * 15
    tables = np.stack([t.numpy() for t, _ in alloc])
    assert (tables[1:, :2] == tables[0, :2]).all()
    assert bm.num_free() == NB - sum(-(-len(r) // bs) for r in reqs) + 2 * 15
    kv = KV(Hkv, d)
    n_all = [len(r) for r in reqs]
    n_new = [n - c for n, c in zip(n_all, cached)]
    cu_q, cu_k = cu_of(n_new), cu_of(n_all)
    rows = [kv.rows(0, r, 0, len(r)) for r in reqs]
    k_new = np.concatenate([k[c:] for (k, _), c in zip(rows, cached)])
    v_new = np.concatenate([v[c:] for (_, v), c in zip(rows, cached)])
    k_all = np.concatenate([k for k, _ in rows])
    v_all = np.concatenate([v for _, v in rows])
    q = normal_bf16(rng, (int(cu_q[-1]), Hq, d))
    kc = torch.full((NB, bs, Hkv, d), int(BF16_NAN), dtype=torch.int16,
                    device="cuda").view(torch.bfloat16)
    vc = kc.clone()
    log(f"prefix batch: new tokens {int(cu_q[-1])}, keys {int(cu_k[-1])}")
    slots = pa.pa_slot_mapping(cu_q, np.array(n_all, np.int32), tables, bs)
    pa.pa_store_kv(dev_bf16(k_new), dev_bf16(v_new), kc, vc, slots.cuda())
    out = pa.pa_prefill_varlen(dev_bf16(q), None, None, kc, vc, dev_i32(tables), dev_i32(cu_q),
                               dev_i32(cu_k), max(n_new), max(n_all), Hkv, scale)
    got = host_f64(out)
    ref = orc.attention(q, cu_q, k=k_all, v=v_all, cu_seqlens_k=cu_k, scale=scale)
    check_close(got, ref, "block-manager prefix prefill")
