"""GPU parity on the five workload configurations, through the C-ABI.

For each configuration the library and the oracle run the same phases on the
same seeded inputs; the pools after every store must be bit-identical (whole
pools compared, so a stray write anywhere fails) and the attention outputs
must satisfy max|err| <= 2e-2 and mean|err| <= 2e-3 against the fp64 oracle.
"""
import gc

import numpy as np
import pytest

from pipelines import check_close, gpu_pipeline, log, oracle_pipeline

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity(cfg, orc):
    import paged_kv_attention_27_amd as pa
    from paged_kv_attention_27_amd import workloads
    log(f"[config {cfg}] generating inputs")
    wl = workloads.make(cfg)
    log(f"[config {cfg}] {wl.name}: GPU pipeline")
    g = gpu_pipeline(pa, wl)
    log(f"[config {cfg}] oracle pipeline")
    o = oracle_pipeline(orc, wl)
    assert np.array_equal(g["k_cache"], o["k_cache"]), "k_cache differs after store"
    assert np.array_equal(g["v_cache"], o["v_cache"]), "v_cache differs after store"
    log(f"[config {cfg}] pools bit-identical")
    for phase in ("prefill", "decode"):
        if phase in o:
            check_close(g[phase], o[phase], f"config {cfg} {phase}")
    del g, o, wl
    gc.collect()
