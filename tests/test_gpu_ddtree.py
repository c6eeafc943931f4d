"""dflash2_ddtree against the oracle: bit-exact trees (parents, depths, slots, tokens,
scores) and status."""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import assert_same_floats, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def run_both(d2, ci, cv, g, A, Bc, an, budget, what):
    B, N, _ = ci.shape
    say(f"ddtree {what} B={B} N={N} budget={budget}")
    got = d2.ddtree(to_dev(ci), to_dev(cv), to_dev(g), to_dev(A), to_dev(Bc), to_dev(an), budget)
    torch.cuda.synchronize()
    got = [to_host(x) for x in got]
    want = orc.ddtree(ci, cv, g, A, Bc, an, budget)
    for name, x, y in zip(("parent", "depth", "slot", "token"), got[:4], want[:4]):
        np.testing.assert_array_equal(x, y, err_msg=f"{what}: {name}")
    assert_same_floats(got[4], want[4], f"{what}: score")
    np.testing.assert_array_equal(got[5], want[5], err_msg=f"{what}: status")
    return got


@pytest.mark.parametrize("budget", [1, 12, 64])
def test_ddtree_drafter_geometry(d2, budget):
    cfg = wl.CONFIGS[2]
    A, Bc = wl.codebooks(cfg)
    draft = wl.draft_logits(cfg)
    ci, cv = orc.topk16(draft.reshape(-1), 1, cfg.N, 1, cfg.P * cfg.V, cfg.V, cfg.V)
    run_both(d2, ci, cv, wl.gate(cfg), A, Bc, wl.anchor(cfg), budget, "config 2")


def test_ddtree_batch_widths_and_bad_inputs(d2):
    rng = np.random.default_rng(105)
    V, R, B = 2000, 256, 12
    A = wl.to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) / 4)
    Bc = wl.to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) / 4)
    for N, budget in ((1, 16), (3, 40), (15, 64), (2, 64)):
        ci = rng.integers(0, V, size=(B, N, 16)).astype(np.int32)
        cv = (rng.standard_normal((B, N, 16)) * 2).astype(np.float32)
        cv[1] = np.round(cv[1])          # ties between candidates
        g = rng.standard_normal((B, N, R)).astype(np.float32)
        an = rng.integers(0, V, size=B).astype(np.int32)
        ci[3, 0, 2] = -5                 # bad index
        cv[5, N - 1, 1] = np.nan         # nonfinite value
        run_both(d2, ci, cv, g, A, Bc, an, budget, f"N={N}")
