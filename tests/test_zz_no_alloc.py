"""pa_decode_noalloc (include/pa.h) against pa_decode, through the C-ABI.

The no-allocation variant keeps a split context's partials in the library's
fixed device scratch instead of a caller workspace; it runs the same kernels
with the same partitions, so its output must equal pa_decode's bit for bit,
and both must match the fp64 oracle within the parity tolerance.  Two calls in
a row on the same scratch, the second with a smaller problem, check that
nothing left by the first call leaks into the second.
"""
import numpy as np
import pytest
import torch

from pipelines import check_close, dev_bf16, dev_i32, host_f64, log, prefix_tables

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import paged_kv_attention_27_amd as pa
    pa.load()
    return pa


def _decode_problem(pa, orc, ctx, hq, hkv, seed):
    from paged_kv_attention_27_amd import workloads
    wl = workloads.synthetic(q_lens=[1] * len(ctx), k_lens=ctx, num_q_heads=hq,
                             num_kv_heads=hkv, seed=seed, q_scale=4.0)
    kc, vc = dev_bf16(wl.k_cache), dev_bf16(wl.v_cache)
    okc, ovc = wl.k_cache.copy(), wl.v_cache.copy()
    for ph, tables in ((wl.prefix, prefix_tables(wl)), (wl.prefill, wl.block_tables)):
        if ph is None:
            continue
        slots = pa.pa_slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, tables, wl.block_size)
        pa.pa_store_kv(dev_bf16(ph.k), dev_bf16(ph.v), kc, vc, slots.cuda())
        orc.store(ph.k, ph.v, orc.slot_mapping(ph.cu_seqlens_q, ph.seqlens_k, tables,
                                               wl.block_size), okc, ovc)
    ref = orc.decode(wl.prefill.q, okc, ovc, wl.block_tables, wl.prefill.seqlens_k, wl.scale)
    dev = dict(q=dev_bf16(wl.prefill.q), kc=kc, vc=vc, bt=dev_i32(wl.block_tables),
               ctx=dev_i32(wl.prefill.seqlens_k), max_ctx=int(max(ctx)), scale=wl.scale)
    return dev, ref


def _both(pa, d, part):
    out_ws = pa.pa_decode(d["q"], d["kc"], d["vc"], d["bt"], d["ctx"], d["max_ctx"], d["scale"],
                          partition_size=part)
    out_na = torch.full_like(out_ws, float("nan"))
    pa.pa_decode_noalloc(d["q"], d["kc"], d["vc"], d["bt"], d["ctx"], d["max_ctx"], d["scale"],
                         out_na, partition_size=part)
    torch.cuda.synchronize()
    return out_ws, out_na


def test_noalloc_matches_decode_twice(pa, orc):
    """Two calls in a row, the second smaller; each equals pa_decode bit for bit."""
    cases = [
        ("12 seqs up to 9000 keys, Hq32/Hkv8, 512-key partitions",
         [9000, 1, 257, 4096, 700, 8192, 33, 5000, 6001, 2, 1024, 7777], 32, 8, 512, 41),
        ("3 seqs up to 2000 keys, Hq8/Hkv1, 256-key partitions",
         [2000, 300, 1500], 8, 1, 256, 42),
    ]
    for label, ctx, hq, hkv, part, seed in cases:
        log(f"[no-alloc decode: {label}]")
        d, ref = _decode_problem(pa, orc, ctx, hq, hkv, seed)
        need = pa.pa_decode_workspace_size(len(ctx), hq, hkv, 128, max(ctx), part)
        assert 0 < need <= pa.NOALLOC_SCRATCH_BYTES
        assert pa.pa_decode_num_partitions(len(ctx), hq, hkv, max(ctx), part) > 1
        out_ws, out_na = _both(pa, d, part)
        assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16)), \
            "pa_decode_noalloc differs from pa_decode"
        check_close(host_f64(out_na), ref, label + " vs oracle")


def test_noalloc_default_partitions(pa, orc):
    """The library's own partition choice (a whole-sequence batch and a split one)."""
    for label, ctx, hq, hkv, seed in (("5 seqs, one partition each", [3, 800, 64, 1999, 256], 16, 8, 43),
                                      ("2 seqs of 20000 keys, split", [20000, 19000], 16, 2, 44)):
        log(f"[no-alloc decode: {label}]")
        d, ref = _decode_problem(pa, orc, ctx, hq, hkv, seed)
        out_ws, out_na = _both(pa, d, 0)
        assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16))
        check_close(host_f64(out_na), ref, label + " vs oracle")


def test_noalloc_rejects_oversized(pa):
    """A problem whose partials exceed the fixed scratch is refused before any launch."""
    from paged_kv_attention_27_amd.binding import PaError
    S, hq, hkv, ctx, part = 64, 32, 8, 65536, 256
    need = pa.pa_decode_workspace_size(S, hq, hkv, 128, ctx, part)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((S, hq, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 256, hkv, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((S, ctx // 256), dtype=torch.int32, device="cuda")
    lens = torch.ones(S, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(PaError) as e:
        pa.pa_decode_noalloc(q, kc, kc, bt, lens, ctx, 0.1, out, partition_size=part)
    assert e.value.status == 6
