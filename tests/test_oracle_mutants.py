"""Planted mistakes in copies of the oracle's source must each fail a pin (CPU only).

Every mutant is a one-line change of the kind a careful reader could still
make (an off-by-one mask, a top-left-anchored mask, an interleaved GQA head map,
a dropped scale or normaliser, V read from K, a wrong row, slot or sign).  The
copy is compiled with gcc into a temporary directory, loaded through the same
wrapper, and run against every pin in ``oracle_pins``: at least one must fail.
The real oracle itself is never modified.
"""
import os
import sys

import pytest

import oracle
from oracle import build as oracle_build
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")

MUTANTS = {
    "mask_off_by_one_short": ("int32_t last = off + i;", "int32_t last = off + i - 1;"),
    "mask_off_by_one_long": ("int32_t last = off + i;",
                             "int32_t last = off + i + 1 < k_len ? off + i + 1 : k_len - 1;"),
    "mask_top_left_tril": ("int32_t last = off + i;", "int32_t last = i;"),
    "gqa_interleaved": ("for (int32_t h = kvh * group; h < (kvh + 1) * group; ++h) {",
                        "for (int32_t h = kvh; h < q_heads; h += kv_heads) {"),
    "scale_dropped": ("S[j] = scale * dot;", "S[j] = dot;"),
    "normaliser_dropped": ("o[x] = acc / l;", "o[x] = acc;"),
    "normaliser_last_term_dropped": ("l += S[j];", "if (j < last) l += S[j];"),
    "exp_sign_flipped": ("S[j] = exp(S[j] - m);", "S[j] = exp(m - S[j]);"),
    "values_from_keys": ("acc += S[j] * V[(int64_t)j * head_dim + x];",
                         "acc += S[j] * K[(int64_t)j * head_dim + x];"),
    "head_dim_reversed": ("dot += qi[x] * K[(int64_t)j * head_dim + x];",
                          "dot += qi[x] * K[(int64_t)j * head_dim + (head_dim - 1 - x)];"),
    "query_head_is_kv_head": ("const uint16_t *qrow = q + (row * q_heads + h) * head_dim;",
                              "const uint16_t *qrow = q + (row * q_heads + kvh) * head_dim;"),
    "gather_offset_shifted": ("int64_t offset = j % block_size;",
                              "int64_t offset = (j + 1) % block_size;"),
    "flat_rows_ignore_cu": ("int64_t r = (int64_t)cu_seqlens_k[s] + j;", "int64_t r = j;"),
    "slot_uses_logical_block": ("slots[cu_seqlens_q[s] + i] = physical * block_size + offset;",
                                "slots[cu_seqlens_q[s] + i] = logical * block_size + offset;"),
    "slot_new_tokens_first": ("int32_t first = seqlens_k[s] - q_len;", "int32_t first = 0;"),
    "store_v_from_k": ("v_cache[dst] = v[src];", "v_cache[dst] = k[src];"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique/present"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new))
    lib = str(tmp_path / f"lib{name}.so")
    oracle_build.build(str(src), lib, extra_flags=["-Wno-error"])
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except Exception as e:  # AssertionError, or an error the mutant provokes
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin catches mutant {name}"
    # the brute force restates the definition; some other pin must catch it too
    assert any(not c.startswith("pin_brute_force") for c in caught), caught
    sys.stdout.write(f"{name} caught by {len(caught)} pin(s): {caught[:3]}\n")
