"""GPU parity of the sliding-window ring f16 cache (token t at slot t mod W,
the last W tokens resident) against the fp64 oracle."""
import numpy as np
import pytest

import synth
from gpu_util import DeviceCase, compare, log, oracle_run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_quantized_kv_amd as dk
    dk.lib()   # fail loudly if the library is missing
    yield


def _check(case, split_tokens=0, what=""):
    log(f"case {case.kind} {what} split_tokens={split_tokens}")
    og, lg = DeviceCase(case).run_np(split_tokens)
    orf, lrf = oracle_run(case)
    return compare(og, lg, orf, lrf, what=what)


@pytest.mark.parametrize("split_tokens", [0, 256])
def test_ring_small(split_tokens):
    c = synth.ring_case(401, 3, 32, 8, 128, 256, [1000, 100, 257], softcap=30.0)
    _check(c, split_tokens, what="ring W256 L1000/100/257")


def _rand_case(seed):
    rng = np.random.default_rng(90_000 + seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 4))
    W = int(rng.choice([1, 16, 50, 128, 512]))
    lens = rng.integers(0, 1500, size=B)
    if rng.random() < 0.3:
        lens[0] = int(rng.choice([0, 1, W - 1, W, W + 1]))
    qp = None
    if rng.random() < 0.4:
        qp = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    return synth.ring_case(seed, B, Hkv * G, Hkv, D, W, lens, q_pos=qp, causal=int(rng.random() < 0.8),
                           softcap=float(rng.choice([0.0, 0.0, 5.0, 50.0])),
                           scale=float(rng.choice([0.0, np.float32(rng.uniform(0.03, 0.3))])))


@pytest.mark.parametrize("seed", range(20))
def test_ring_random_sweep(seed):
    case = _rand_case(seed)
    st = int(np.random.default_rng(seed).choice([0, 0, 16, 48, 256]))
    p = case.params
    _check(case, split_tokens=st,
           what=f"seed{seed} B{p['num_seqs']} H{p['num_heads']}/{p['num_kv_heads']} D{p['head_dim']} "
                f"W{case.hot_window} cap{p['softcap']} lens{list(case.seq_lens)}")


def test_ring_unfilled_and_overwritten_slots_hold_nan():
    """Slots never written (L < W) hold NaN / Inf; tiles that straddle the ring's
    oldest resident token read whole slots of the wrapped ring and must mask them."""
    c = synth.ring_case(402, 3, 32, 8, 128, 96, [40, 500, 95], softcap=20.0)
    for b, L in enumerate(c.seq_lens):
        if L < c.hot_window:
            c.k_hot[b, int(L):] = np.nan
            c.v_hot[b, int(L):, ..., ::2] = np.inf
    _check(c, what="ring with NaN in unfilled slots")


def test_ring_earlier_query():
    qp = np.array([900, 20, 511], np.int32)
    c = synth.ring_case(403, 3, 16, 4, 128, 128, [1000, 700, 512], q_pos=qp, causal=1)
    _check(c, what="ring, query before the last token")
