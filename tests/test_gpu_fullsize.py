"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (library-chosen split size), checked against the oracle on sampled
(sequence, head) pairs that the oracle computes one by one, plus properties
that hold at any size (finite outputs, lse not below the log of the largest
single weight, which the oracle pins per sample)."""
import numpy as np
import pytest

import synth
from gpu_util import DeviceCase, compare, log, oracle_run

pytestmark = pytest.mark.gpu

WORKLOADS = [(2, {}), (3, {"window": 0}), (3, {"window": 4096}), (4, {}), (5, {})]
# the tiered workload's shape with an f16 cold tier, the window ring, four and sixteen queries per sequence,
# four queries over the block-sparse cache
EXTRA = {"tiered_f16": lambda: synth.tiered_f16_workload(0), "ring": synth.ring_workload,
         "multi_query": lambda: synth.multi_query_workload(4),
         "multi_query_16": lambda: synth.multi_query_workload(16),
         "sparse_multi_query": lambda: synth.sparse_multi_query_workload(4)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_quantized_kv_amd as dk
    dk.lib()
    yield


def _sampled(case, seed):
    import torch
    log(f"full-size {case.name}")
    dc = DeviceCase(case)
    out, lse = dc.run_np()
    del dc
    torch.cuda.empty_cache()
    p = case.params
    nbh = p["num_seqs"] * max(1, p.get("query_len", 1)) * p["num_heads"]
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(seed)
    pairs = np.unique(np.concatenate([[0, nbh - 1, p["num_heads"] - 1], rng.integers(0, nbh, 21)])).astype(np.int32)
    ref_o, ref_l = oracle_run(case, pairs=pairs)
    compare(out.reshape(nbh, -1)[pairs], lse.reshape(nbh)[pairs], ref_o, ref_l, what=f"{case.name} sampled")


@pytest.mark.parametrize("idx,kw", WORKLOADS, ids=["paged", "tiered_w0", "tiered_w4096", "long", "sparse"])
def test_full_size_sampled(idx, kw):
    _sampled(synth.workload(idx, **kw), idx)


@pytest.mark.parametrize("name", sorted(EXTRA))
def test_full_size_sampled_other_caches(name):
    _sampled(EXTRA[name](), 11)
