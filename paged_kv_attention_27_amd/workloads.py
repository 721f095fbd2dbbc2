"""Seeded synthetic inputs for the paged-attention workloads.

This module draws inputs and nothing else: sequence lengths, physical block
permutations carved into block tables, and N(0,1) values rounded to bf16.  It
holds none of the attention arithmetic (no slot computation, no masking, no
softmax) and imports neither the HIP binding nor the CPU oracle, so both sides
of every parity test and the benchmark receive the very same arrays from it.

Workload shapes follow the pages' running example, Qwen3-0.6B's attention
heads (16 query heads, 8 KV heads, head_dim 128) with the source default block
size of 256 tokens ("nano-vLLM offline" course, ACCURACY & SCOPE: block size
256, a multiple of 256; "Visual atlas" ch.15: projection widths from the model
config).

Representation: bf16 tensors are numpy ``uint16`` arrays of their bit
patterns, index arrays are ``int32``.  Values are drawn as float32 N(0,1) and
rounded to bf16 round-to-nearest-even.  Pools start filled with the bf16 quiet
NaN 0x7FC0 wherever no token has been written, so a kernel that reads a slot
it should not read shows it in its output.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
_CHUNK = 1 << 22  # values per independently seeded chunk
_POOL = None


def _executor():
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=16)
    return _POOL


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) values as bf16 bits, drawn in fixed-size chunks.

    Each chunk has its own generator seeded from ``rng``, so the result does not
    depend on the number of threads used to fill it.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    seeds = rng.integers(0, 2**63 - 1, size=max(nchunks, 1), dtype=np.int64)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(int(seeds[i])))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[lo:hi] = f32_to_bf16_bits(x)

    list(_executor().map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclass
class Phase:
    """One batch of new tokens and the attention over them.

    ``q`` is [Tq, Hq, d]; ``k``/``v`` are the new tokens' rows [Tq, Hkv, d];
    sequence s owns rows cu_seqlens_q[s]..cu_seqlens_q[s+1] and has
    seqlens_k[s] keys in total once they are stored (the new ones are its last
    q_len positions).  ``paged`` says whether attention reads its keys from the
    pools (through the block tables) or from the flat k/v of this phase
    (``cu_seqlens_k``, no cache).
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_seqlens_q: np.ndarray
    seqlens_k: np.ndarray
    paged: bool
    cu_seqlens_k: Optional[np.ndarray] = None
    max_seqlen_q: int = 0
    max_seqlen_k: int = 0


@dataclass
class Workload:
    name: str
    description: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    block_tables: np.ndarray          # [S, max_blocks] int32, -1 = unused
    k_cache: np.ndarray               # [NB, bs, Hkv, d] bf16 bits, initial content
    v_cache: np.ndarray
    prefix: Optional[Phase] = None    # stored before the prefill (shared prefix)
    prefill: Optional[Phase] = None
    decode: Optional[Phase] = None
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return self.block_tables.shape[0]

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_tables.shape[1]


def _cu(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _tables(perm: np.ndarray, blocks_per_seq, max_blocks: int, shared=()) -> np.ndarray:
    """Carve consecutive runs of a block permutation into per-sequence tables.

    ``shared`` physical ids head every table (a prefix held by all sequences).
    """
    S = len(blocks_per_seq)
    bt = np.full((S, max_blocks), -1, dtype=np.int32)
    cursor = 0
    for s, nb in enumerate(blocks_per_seq):
        row = list(shared) + [int(x) for x in perm[cursor:cursor + nb]]
        cursor += nb
        bt[s, :len(row)] = row
    if cursor > len(perm):
        raise ValueError("pool too small for the drawn lengths")
    return bt


def _nan_pool(nb, bs, hkv, d):
    return np.full((nb, bs, hkv, d), BF16_NAN, dtype=np.uint16)


def _phase(rng, lengths, seqlens_k, Hq, Hkv, d, paged, values=True) -> Phase:
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    if values:
        q = normal_bf16(rng, (T, Hq, d))
        k = normal_bf16(rng, (T, Hkv, d))
        v = normal_bf16(rng, (T, Hkv, d))
    else:
        q = k = v = None
    cu = _cu(lengths)
    sk = np.asarray(seqlens_k, dtype=np.int32)
    return Phase(q=q, k=k, v=v, cu_seqlens_q=cu, seqlens_k=sk, paged=paged,
                 cu_seqlens_k=None if paged else cu.copy(),
                 max_seqlen_q=int(lengths.max()), max_seqlen_k=int(sk.max()))


def _blocks_for(n_tokens: int, bs: int) -> int:
    # capacity the block manager reserves for a sequence of n tokens
    return -(-int(n_tokens) // bs)


def _streams(seed: int):
    """Independent generators: metadata, pools, prefill, prefix, decode values.

    Each component has a stream of its own, so drawing (or skipping) one never
    shifts another.
    """
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(5)]


def config1(seed: int = 27001, values: bool = True) -> Workload:
    """4 sequences {17,256,300,511}: full causal prefill, then one decode step."""
    meta, _, r_pre, _, r_dec = _streams(seed)
    Hq, Hkv, d, bs, NB = 16, 8, 128, 256, 16
    L = np.array([17, 256, 300, 511])
    perm = meta.permutation(NB).astype(np.int32)
    nb = [_blocks_for(n + 1, bs) for n in L]  # room for the decode token
    bt = _tables(perm, nb, max(nb))
    prefill = _phase(r_pre, L, L, Hq, Hkv, d, paged=False, values=values)
    decode = _phase(r_dec, np.ones(len(L), np.int64), L + 1, Hq, Hkv, d, paged=True,
                    values=values)
    return Workload("c1_tiny_prefill_decode",
                    "4 seqs L={17,256,300,511}, Hq16/Hkv8/d128, bs256, 16-block pool; "
                    "store+prefill then one decode step",
                    Hq, Hkv, d, bs, NB, _scale(d), bt, _nan_pool(NB, bs, Hkv, d),
                    _nan_pool(NB, bs, Hkv, d), prefill=prefill, decode=decode)


def config2(seed: int = 27002, values: bool = True) -> Workload:
    """8 sequences, lengths U[100,1024], varlen causal prefill from flat K/V."""
    meta, _, r_pre, _, _ = _streams(seed)
    Hq, Hkv, d, bs, NB = 16, 8, 128, 256, 64
    L = meta.integers(100, 1024, size=8, endpoint=True)
    perm = meta.permutation(NB).astype(np.int32)
    nb = [_blocks_for(n, bs) for n in L]
    bt = _tables(perm, nb, max(nb))
    prefill = _phase(r_pre, L, L, Hq, Hkv, d, paged=False, values=values)
    return Workload("c2_varlen_prefill",
                    "8 seqs L~U[100,1024], Hq16/Hkv8/d128, bs256, store into 64-block pool; "
                    "causal prefill from flat K/V",
                    Hq, Hkv, d, bs, NB, _scale(d), bt, _nan_pool(NB, bs, Hkv, d),
                    _nan_pool(NB, bs, Hkv, d), prefill=prefill)


def config3(seed: int = 27003, values: bool = True) -> Workload:
    """16 sequences share a 512-token cached prefix; chunks U[64,1024] attend to it."""
    meta, _, r_pre, r_fix, _ = _streams(seed)
    Hq, Hkv, d, bs, NB, P = 16, 8, 128, 256, 128, 512
    Lq = meta.integers(64, 1024, size=16, endpoint=True)
    perm = meta.permutation(NB).astype(np.int32)
    n_shared = P // bs
    shared = perm[:n_shared]
    nb = [_blocks_for(P + n, bs) - n_shared for n in Lq]
    bt = _tables(perm[n_shared:], nb, n_shared + max(nb), shared=shared)
    prefill = _phase(r_pre, Lq, P + Lq, Hq, Hkv, d, paged=True, values=values)
    # the prefix is written once, as the first P positions of sequence 0
    prefix = _phase(r_fix, [P], [P], Hq, Hkv, d, paged=True, values=values)
    return Workload("c3_prefix_chunked_prefill",
                    "16 seqs, shared 512-token cached prefix (2 shared blocks) + chunk "
                    "q~U[64,1024]; Hq16/Hkv8/d128, bs256, 128-block pool; prefill reads pools",
                    Hq, Hkv, d, bs, NB, _scale(d), bt, _nan_pool(NB, bs, Hkv, d),
                    _nan_pool(NB, bs, Hkv, d), prefix=prefix, prefill=prefill,
                    extra={"prefix_len": P, "prefix_seq": 0})


def _history_pools(rng, bt, NB, bs, Hkv, d):
    """Pools whose blocks in use hold N(0,1) history; blocks never used hold NaN."""
    used = np.unique(bt[bt >= 0])
    kc = _nan_pool(NB, bs, Hkv, d)
    vc = _nan_pool(NB, bs, Hkv, d)
    # used blocks in ascending physical id, K first, then V
    kvals = normal_bf16(rng, (len(used), bs, Hkv, d))
    vvals = normal_bf16(rng, (len(used), bs, Hkv, d))
    kc[used] = kvals
    vc[used] = vvals
    return kc, vc


def _decode_config(name, desc, streams, ctx, Hq, Hkv, d, bs, NB, values) -> Workload:
    meta, r_pool, _, _, r_dec = streams
    S = len(ctx)
    perm = meta.permutation(NB).astype(np.int32)
    nb = [_blocks_for(c, bs) for c in ctx]
    bt = _tables(perm, nb, max(nb))
    if values:
        kc, vc = _history_pools(r_pool, bt, NB, bs, Hkv, d)
    else:
        kc = vc = None
    decode = _phase(r_dec, np.ones(S, np.int64), ctx, Hq, Hkv, d, paged=True, values=values)
    return Workload(name, desc, Hq, Hkv, d, bs, NB, _scale(d), bt, kc, vc, decode=decode)


def config4(seed: int = 27004, values: bool = True) -> Workload:
    """256 sequences decode, context U[128,4096] (new token included)."""
    streams = _streams(seed)
    ctx = streams[0].integers(128, 4096, size=256, endpoint=True).astype(np.int32)
    return _decode_config("c4_batched_decode",
                          "256 seqs, ctx~U[128,4096] incl. new token, Hq16/Hkv8/d128, bs256, "
                          "4096-block pool; store new K/V then paged decode",
                          streams, ctx, 16, 8, 128, 256, 4096, values)


def config5(seed: int = 27005, values: bool = True) -> Workload:
    """16 sequences x 32768 context, Hq=32 over Hkv=8 (group of 4)."""
    streams = _streams(seed)
    ctx = np.full(16, 32768, dtype=np.int32)
    return _decode_config("c5_long_decode",
                          "16 seqs x ctx 32768, Hq32/Hkv8/d128, bs256, 2048-block pool; "
                          "store new K/V then split-K paged decode",
                          streams, ctx, 32, 8, 128, 256, 2048, values)


def head_ratio_decode(num_kv_heads: int, seed: int = 27010, values: bool = True) -> Workload:
    """256-sequence decode with 8 Q heads over 8, 2 or 1 KV heads (MHA, GQA, MQA).

    Same lengths (ctx U[128,4096]) and values stream for every ratio, so the KV
    bytes read scale 8:2:1 ("Visual atlas" ch.18: with Q heads fixed at 8, the
    KV capacity of MHA, GQA and MQA is 8:2:1).
    """
    streams = _streams(seed)
    ctx = streams[0].integers(128, 4096, size=256, endpoint=True).astype(np.int32)
    name = {8: "mha", 2: "gqa", 1: "mqa"}.get(num_kv_heads, f"hkv{num_kv_heads}")
    return _decode_config(f"decode_hq8_{name}",
                          f"256 seqs, ctx~U[128,4096], Hq8/Hkv{num_kv_heads}/d128, bs256, "
                          "4096-block pool; store new K/V then paged decode",
                          streams, ctx, 8, num_kv_heads, 128, 256, 4096, values)


def _scale(d: int) -> float:
    # 1/sqrt(d) as the float32 both sides receive
    return float(np.float32(1.0 / math.sqrt(d)))


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def make(cfg_id: int, values: bool = True) -> Workload:
    """Workload of config 1..5; values=False draws only lengths and tables."""
    return CONFIGS[cfg_id](values=values)


def synthetic(q_lens, k_lens, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
              seed=0, paged=True, q_scale=1.0, q_zero=False, v_position=False,
              v_scale=1.0, extra_blocks=3, name="synthetic") -> Workload:
    """A small seeded problem with discriminating options for parity tests.

    Sequence s has k_lens[s] tokens of which the last q_lens[s] are new.  With
    ``paged`` the earlier k_lens[s] - q_lens[s] tokens form a ``prefix`` phase
    (cached history, stored first) and attention reads the pools; without it
    q_lens must equal k_lens and attention reads the flat k/v.
    Options: ``q_scale`` multiplies q (8 gives a peaky softmax), ``q_zero``
    makes every weight equal, ``v_position`` writes each value row's position
    into its first two elements as (j mod 16)/16 and ((j div 16) mod 16)/16,
    ``v_scale`` multiplies every value row (outputs then scale with it).
    """
    meta, _, r_pre, r_fix, _ = _streams(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    if (q_lens > k_lens).any() or (not paged and (q_lens != k_lens).any()):
        raise ValueError("need q_len <= k_len, and equal lengths without a cache")
    S = len(q_lens)
    Hq, Hkv, d, bs = num_q_heads, num_kv_heads, head_dim, block_size
    nb = [max(_blocks_for(n, bs), 1) for n in k_lens]
    NB = int(sum(nb)) + extra_blocks
    perm = meta.permutation(NB).astype(np.int32)
    bt = _tables(perm, nb, max(nb))
    prefill = _phase(r_pre, q_lens, k_lens, Hq, Hkv, d, paged=paged)
    hist_lens = k_lens - q_lens
    prefix = None
    if paged and hist_lens.sum() > 0:
        prefix = _phase(r_fix, hist_lens, hist_lens, Hq, Hkv, d, paged=True)
    if q_zero:
        prefill.q[:] = 0
    elif q_scale != 1.0:
        prefill.q[:] = f32_to_bf16_bits(bf16_bits_to_f32(prefill.q) * np.float32(q_scale))
    if v_position:
        for ph, first in ((prefix, np.zeros(S, np.int64)), (prefill, hist_lens)):
            if ph is None:
                continue
            for s in range(S):
                a, b = ph.cu_seqlens_q[s], ph.cu_seqlens_q[s + 1]
                j = first[s] + np.arange(b - a)
                ph.v[a:b, :, 0] = f32_to_bf16_bits(((j % 16) / 16.0).astype(np.float32))[:, None]
                ph.v[a:b, :, 1] = f32_to_bf16_bits((((j // 16) % 16) / 16.0).astype(np.float32))[:, None]
    if v_scale != 1.0:
        for ph in (prefix, prefill):
            if ph is not None:
                ph.v[:] = f32_to_bf16_bits(bf16_bits_to_f32(ph.v) * np.float32(v_scale))
    wl = Workload(name, "synthetic parity problem", Hq, Hkv, d, bs, NB, _scale(d), bt,
                  _nan_pool(NB, bs, Hkv, d), _nan_pool(NB, bs, Hkv, d), prefix=prefix,
                  prefill=prefill)
    wl.extra["prefix_per_seq"] = True
    return wl
