"""Host block manager with prefix caching (pa_bm_* in include/pa.h), on the CPU.

The rules checked come from the pages: blocks come from a pool reserved once
and are only handed out and returned ("nano-vLLM offline" course, THE
IMPORTANT DETAILS item 02); the manager keeps block ids, prefix hashes and
reference counts ("Nano-vLLM reading notes", key state and module boundaries);
only full blocks are shared and the trailing partial block is not
("nano-vLLM offline" course, ACCURACY & SCOPE); a freed block keeps its content
and can still be hit until it is reused ("Visual atlas" ch.25); cache identity
is more than a token substring ("Visual atlas" ch.28).

The stress test keeps its own model of what every pool block holds -- the salt
and the whole token prefix up to the block's end, since a position's K/V
depends on every token before it -- and checks that every cache hit hands out
a block whose content is exactly what the request would have written, that
writes only go to blocks with one holder, and that reference and free counts
always match the live tables.
"""
import numpy as np
import pytest

import paged_kv_attention_27_amd as pa
from paged_kv_attention_27_amd.binding import BlockManager, PaError


def table_ids(table):
    t = table.tolist()
    n = t.index(-1) if -1 in t else len(t)
    assert all(x == -1 for x in t[n:]), "padding must be -1 to the end"
    return t[:n]


def test_full_prefix_blocks_are_shared():
    bm = BlockManager(16, 4)
    a = list(range(100, 110))                              # 10 tokens: 2 full blocks + 2
    ta, ca = bm.allocate(a, 8)
    assert ca == 0 and len(table_ids(ta)) == 3
    b = a[:8] + [7, 8, 9]
    tb, cb = bm.allocate(b, 8)
    ia, ib = table_ids(ta), table_ids(tb)
    assert cb == 8 and ib[:2] == ia[:2] and ib[2] not in ia
    assert [bm.ref_count(x) for x in ia] == [2, 2, 1]
    assert bm.ref_count(ib[2]) == 1
    assert bm.num_free() == 16 - 4


def test_partial_block_is_not_shared():
    bm = BlockManager(16, 4)
    p = [5, 6, 7, 8, 9, 10]                                # one full block + 2 tokens
    t1, c1 = bm.allocate(p, 4)
    t2, c2 = bm.allocate(p, 4)
    assert c1 == 0 and c2 == 4
    assert table_ids(t1)[0] == table_ids(t2)[0]
    assert table_ids(t1)[1] != table_ids(t2)[1]


def test_last_prompt_block_is_always_computed():
    bm = BlockManager(16, 4)
    p = list(range(12))                                    # exactly 3 full blocks
    t1, _ = bm.allocate(p, 4)
    t2, c2 = bm.allocate(p, 4)
    assert c2 == 8 < len(p)
    i1, i2 = table_ids(t1), table_ids(t2)
    assert i2[:2] == i1[:2] and i2[2] != i1[2]
    assert bm.allocate([1, 2, 3], 1)[1] == 0               # prompt shorter than a block
    assert bm.allocate([], 2)[1] == 0


def test_salt_separates_caches():
    bm = BlockManager(16, 4)
    p = list(range(9))
    bm.allocate(p, 4, salt=1)
    assert bm.allocate(p, 4, salt=2)[1] == 0
    assert bm.allocate(p, 4, salt=1)[1] == 8


def test_key_chains_the_prefix():
    """Equal tokens in block 1 behind a different block 0 must not hit."""
    bm = BlockManager(16, 4)
    bm.allocate([1, 2, 3, 4, 50, 51, 52, 53, 0], 4)
    assert bm.allocate([9, 9, 9, 9, 50, 51, 52, 53, 0], 4)[1] == 0
    assert bm.allocate([1, 2, 3, 4, 50, 51, 52, 53, 1], 4)[1] == 8


def test_miss_then_later_blocks_fresh_and_registered():
    """After a miss at block 0 the later full blocks are fresh; they are still
    registered under their own prefix, so a third identical request hits them."""
    bm = BlockManager(32, 4)
    bm.allocate([1, 2, 3, 4, 5], 4)
    p = [7, 7, 7, 7, 8, 8, 8, 8, 9]
    t1, c1 = bm.allocate(p, 4)
    assert c1 == 0
    t2, c2 = bm.allocate(p, 4)
    assert c2 == 8 and table_ids(t2)[:2] == table_ids(t1)[:2]


def test_freed_blocks_still_hit_until_reused():
    bm = BlockManager(6, 4)
    p = list(range(9))                                     # 3 blocks
    t, _ = bm.allocate(p, 4)
    ids = table_ids(t)
    bm.free(t)
    assert bm.num_free() == 6 and all(bm.ref_count(x) == 0 for x in ids)
    assert bm.blocks_needed(p) == 3                        # hits on free blocks still take them
    t2, c2 = bm.allocate(p, 4)
    assert c2 == 8 and table_ids(t2)[:2] == ids[:2]
    bm.free(t2)
    # fill the pool with unrelated prompts: the freed cached blocks get reused
    tables = [bm.allocate([1000 + 10 * i + j for j in range(8)], 2)[0] for i in range(3)]
    assert bm.num_free() == 0
    for tt in tables:
        bm.free(tt)
    assert bm.allocate(p, 4)[1] == 0


def test_recycling_is_least_recently_freed_first():
    bm = BlockManager(4, 2)
    t1, _ = bm.allocate([1, 2, 3], 2)                      # blocks 0, 1
    t2, _ = bm.allocate([4, 5, 6], 2)                      # blocks 2, 3
    bm.free(t1)                                            # freed: 1 then 0 (reverse order)
    bm.free(t2)                                            # then 3, 2
    t3, _ = bm.allocate([9, 9, 9], 2)
    assert table_ids(t3) == [table_ids(t1)[1], table_ids(t1)[0]]


def test_exhaustion_takes_nothing():
    bm = BlockManager(4, 4)
    t, _ = bm.allocate(list(range(10)), 4)                 # 3 blocks
    with pytest.raises(PaError) as e:
        bm.allocate(list(range(100, 110)), 4)              # needs 3, 1 free
    assert e.value.status == 4
    assert bm.num_free() == 1
    assert [bm.ref_count(x) for x in table_ids(t)] == [1, 1, 1]
    # a request that shares the cached prefix only needs its own tail
    assert bm.blocks_needed(list(range(8)) + [55]) == 1
    t2, c2 = bm.allocate(list(range(8)) + [55], 4)
    assert c2 == 8 and bm.num_free() == 0


def test_append_grows_and_registers():
    bm = BlockManager(16, 4)
    toks = [3, 1, 4]
    t, _ = bm.allocate(toks, 4)
    assert len(table_ids(t)) == 1
    for x in [1, 5, 9, 2, 6, 5]:                           # positions 3..8
        toks.append(x)
        bm.append(toks, t)
    ids = table_ids(t)
    assert len(ids) == 3 and bm.num_free() == 13
    # blocks 0 and 1 filled during decode: a new prompt with that prefix hits them
    t2, c2 = bm.allocate(toks[:8] + [0], 4)
    assert c2 == 8 and table_ids(t2)[:2] == ids[:2]


def test_errors():
    bm = BlockManager(4, 4)
    t, _ = bm.allocate([1, 2, 3, 4, 5], 2)
    with pytest.raises(PaError) as e:
        bm.allocate(list(range(9)), 2)                     # table too short
    assert e.value.status == 2
    with pytest.raises(PaError):
        bm.append([1, 2, 3, 4, 5, 6, 7, 8, 9], t)          # position 8 needs a third entry
    with pytest.raises(PaError):
        bm.append([1, 2, 3, 4, 5], t)                      # position 4 opens block 1: already set
    bm.free(t)
    with pytest.raises(PaError):
        bm.free(t)                                         # not held any more
    with pytest.raises(PaError):
        bm.free([99])
    with pytest.raises(ValueError):
        BlockManager(0, 4)
    assert bm.ref_count(-1) == -1 and bm.ref_count(4) == -1
    # a full pool makes append report exhaustion and leave the table alone
    bm2 = BlockManager(1, 2)
    tt, _ = bm2.allocate([1, 2], 2)
    before = tt.clone()
    with pytest.raises(PaError) as e:
        bm2.append([1, 2, 3], tt)
    assert e.value.status == 4 and bool((tt == before).all())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_scheduler_invariants(seed):
    """A random mix of admissions with shared system prompts, decode appends and
    completions against a model of the pool's contents."""
    rng = np.random.default_rng(seed)
    NB, bs, maxb = 96, 4, 24
    bm = BlockManager(NB, bs)
    systems = [list(rng.integers(0, 50, size=int(rng.integers(3, 14)))) for _ in range(4)]
    content = {}                      # block id -> (salt, tuple of tokens up to its last stored slot)
    live = []                         # (tokens, table, salt)

    def write(tokens, table, salt, lo, hi):
        """The model of storing K/V for positions lo..hi-1 (a prefill or a decode step)."""
        ids = table.tolist()
        for p in range(lo, hi):
            blk = ids[p // bs]
            assert bm.ref_count(blk) == 1, "a write must go to a block with one holder"
            content[blk] = (salt, tuple(tokens[:p + 1]))

    def check_counts():
        held = {}
        for _, table, _ in live:
            for x in table_ids(table):
                held[x] = held.get(x, 0) + 1
        for x in range(NB):
            assert bm.ref_count(x) == held.get(x, 0)
        assert bm.num_free() == NB - len(held)

    for step in range(600):
        op = rng.random()
        if op < 0.35 or not live:
            salt = int(rng.integers(0, 2))
            toks = list(systems[int(rng.integers(0, 4))]) if rng.random() < 0.8 else []
            if live and rng.random() < 0.3:                # fork a running sequence's history
                toks = list(live[int(rng.integers(0, len(live)))][0])
            toks += list(rng.integers(0, 50, size=int(rng.integers(1, 12))))
            toks = [int(x) for x in toks][:maxb * bs - 8]
            need = bm.blocks_needed(toks, salt)
            if need > bm.num_free():
                with pytest.raises(PaError):
                    bm.allocate(toks, maxb, salt)
                check_counts()
                continue
            free_before = bm.num_free()
            table, cached = bm.allocate(toks, maxb, salt)
            assert bm.num_free() == free_before - need
            assert cached % bs == 0 and cached < len(toks)
            ids = table_ids(table)
            assert len(ids) == -(-len(toks) // bs)
            for b in range(cached // bs):                  # every hit holds exactly this prefix
                assert content.get(ids[b]) == (salt, tuple(toks[:(b + 1) * bs]))
            live.append((toks, table, salt))
            write(toks, table, salt, cached, len(toks))
        elif op < 0.8:
            toks, table, salt = live[int(rng.integers(0, len(live)))]
            if len(toks) >= maxb * bs:
                continue
            toks.append(int(rng.integers(0, 50)))
            pos = len(toks) - 1
            if pos % bs == 0 and bm.num_free() == 0:
                with pytest.raises(PaError):
                    bm.append(toks, table, salt)
                toks.pop()
                continue
            bm.append(toks, table, salt)
            write(toks, table, salt, pos, pos + 1)
        else:
            i = int(rng.integers(0, len(live)))
            _, table, _ = live.pop(i)
            bm.free(table)
        check_counts()
