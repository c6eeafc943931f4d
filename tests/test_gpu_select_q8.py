"""dflash2_select_q8 against the oracle: bit-exact tokens, slots, q rows and status."""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import assert_same_floats, poison_like, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


@pytest.fixture(scope="module")
def q8_books():
    say("quantizing the drafter-geometry codebooks to Q8")
    return wl.codebooks_q8(wl.CONFIGS[2])


def _dev_q8(cb):
    codes, sc, bi = cb
    return (torch.from_numpy(np.ascontiguousarray(codes)).cuda(), to_dev(sc), to_dev(bi))


def run_both(d2, ci, cv, gate, pq, sq, anchor, temp, seed, step, what=""):
    B, N, _ = ci.shape
    say(f"select_q8 {what} B={B} N={N} V={pq[0].shape[0]} R={pq[0].shape[1]}")
    tok = poison_like((B, N), torch.int32)
    sl = poison_like((B, N), torch.int32)
    q = poison_like((B, N, 16), torch.float32)
    st = poison_like((B,), torch.int32)
    d2.select_q8(to_dev(ci), to_dev(cv), to_dev(gate), _dev_q8(pq), _dev_q8(sq), to_dev(anchor),
                 to_dev(temp), seed, step, tokens=tok, slot=sl, q=q, status=st)
    torch.cuda.synchronize()
    g = [to_host(tok), to_host(sl), to_host(q), to_host(st)]
    o = orc.select_q8(ci, cv, gate, pq, sq, anchor, temp, seed, step)
    np.testing.assert_array_equal(g[0], o[0], err_msg=f"{what}: tokens")
    np.testing.assert_array_equal(g[1], o[1], err_msg=f"{what}: slot")
    assert_same_floats(g[2], o[2], f"{what}: q")
    np.testing.assert_array_equal(g[3], o[3], err_msg=f"{what}: status")
    return g


@pytest.mark.parametrize("R", [64, 192, 512])
def test_select_q8_small_ranks(d2, R):
    rng = np.random.default_rng(100 + R)
    V, B, N = 3000, 4, 7
    pq = wl.q8_quantize(rng.standard_normal((V, R)).astype(np.float32) / 4)
    sq = wl.q8_quantize(rng.standard_normal((V, R)).astype(np.float32) / 4)
    ci = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                   for _ in range(B)]).astype(np.int32)
    cv = (rng.standard_normal((B, N, 16)) * 2).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    an = rng.integers(0, V, size=B).astype(np.int32)
    for T in (0.0, 0.7):
        run_both(d2, ci, cv, g, pq, sq, an, np.full(B, T, np.float32), 9, 2, what=f"R={R} T={T}")


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_select_q8_drafter_geometry(d2, q8_books, T):
    cfg = wl.CONFIGS[2]
    pq, sq = q8_books
    draft = wl.draft_logits(cfg)
    ci, cv = orc.topk16(draft.reshape(-1), 1, cfg.N, 1, cfg.P * cfg.V, cfg.V, cfg.V)
    run_both(d2, ci, cv, wl.gate(cfg), pq, sq, wl.anchor(cfg), np.full(1, T, np.float32),
             cfg.seed, 3, what=f"config 2 T={T}")


def test_select_q8_serving_batch_and_bad_inputs(d2, q8_books):
    rng = np.random.default_rng(103)
    pq, sq = q8_books
    V, R = pq[0].shape
    B, N = 64, 7
    ci = rng.integers(0, V, size=(B, N, 16)).astype(np.int32)
    cv = (rng.standard_normal((B, N, 16)) * 2).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    an = rng.integers(0, V, size=B).astype(np.int32)
    temp = np.where(np.arange(B) % 2 == 0, 0.0, 1.0).astype(np.float32)
    ci[3, 2, 5] = V              # out of range
    an[7] = -1
    cv[9, 0, 0] = np.inf         # nonfinite value
    run_both(d2, ci, cv, g, pq, sq, an, temp, 21, 5, what="serving batch")
