"""dflash2_select against the oracle: bit-exact tokens, slots, q rows and status."""
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
def full_codebooks():
    return {c: wl.codebooks(wl.CONFIGS[c]) for c in (2, 4)}


def run_both(d2, ci, cv, gate, A, Bc, anchor, temp, seed, step, what=""):
    B, N, _ = ci.shape
    say(f"select {what} B={B} N={N} V={A.shape[0]} R={A.shape[1]}")
    tok = poison_like((B, N), torch.int32)
    sl = poison_like((B, N), torch.int32)
    q = poison_like((B, N, 16), torch.float32)
    st = poison_like((B,), torch.int32)
    d2.select(to_dev(ci), to_dev(cv), to_dev(gate), to_dev(A), to_dev(Bc), to_dev(anchor),
              to_dev(temp), seed, step, tokens=tok, slot=sl, q=q, status=st)
    torch.cuda.synchronize()
    g = [to_host(tok), to_host(sl), to_host(q), to_host(st)]
    o = orc.select(ci, cv, gate, A, Bc, anchor, temp, seed, step)
    np.testing.assert_array_equal(g[0], o[0], err_msg=f"{what}: tokens")
    np.testing.assert_array_equal(g[1], o[1], err_msg=f"{what}: slot")
    assert_same_floats(g[2], o[2], f"{what}: q")
    np.testing.assert_array_equal(g[3], o[3], err_msg=f"{what}: status")
    return g


def candidates_from_draft(cfg, draft):
    """The selector's candidate input: the oracle's top-16 of draft rows 1..N."""
    B, P, V = draft.shape
    return orc.topk16(draft.reshape(-1), B, P - 1, 1, P * V, V, V)


def test_select_tiny_config(d2):
    cfg = wl.CONFIGS[1]
    draft = wl.draft_logits(cfg)
    ci, cv = candidates_from_draft(cfg, draft)
    A, Bc = wl.codebooks(cfg)
    g = wl.gate(cfg)
    an = wl.anchor(cfg)
    for T in (0.0, 0.7, 1.0, 2.5):
        for step in range(3):
            run_both(d2, ci, cv, g, A, Bc, an, np.full(1, T, np.float32), cfg.seed, step,
                     what=f"tiny T={T} step={step}")


@pytest.mark.parametrize("cfgno,T", [(2, 0.0), (2, 0.7), (4, 0.7)])
def test_select_drafter_geometry(d2, full_codebooks, cfgno, T):
    cfg = wl.CONFIGS[cfgno]
    A, Bc = full_codebooks[cfgno]
    seqs = [0, 5] if cfg.B > 1 else [0]
    draft = wl.draft_logits(cfg, seqs=seqs)
    ci, cv = candidates_from_draft(cfg, draft)
    g = wl.gate(cfg, seqs=seqs)
    an = wl.anchor(cfg)[seqs]
    run_both(d2, ci, cv, g, A, Bc, an, np.full(len(seqs), T, np.float32), cfg.seed, 4,
             what=f"config {cfgno} T={T}")


def test_select_mixed_serving_batch(d2, full_codebooks):
    rng = np.random.default_rng(41)
    A, Bc = full_codebooks[2]
    V, R = A.shape
    B, N = 64, 7
    ci = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                   for _ in range(B)]).astype(np.int32)
    cv = -np.sort(-(rng.standard_normal((B, N, 16)) * 2), axis=2).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    an = rng.integers(0, V, B).astype(np.int32)
    temps = np.where(np.arange(B) % 2 == 0, 0.0, 1.0).astype(np.float32)
    run_both(d2, ci, cv, g, A, Bc, an, temps, 0xDF20005, 9, what="B=64 mixed")


@pytest.mark.parametrize("R", [1, 2, 17, 64, 255, 512])
def test_select_ranks(d2, R):
    rng = np.random.default_rng(42 + R)
    B, N, V = 3, 7, 777
    ci = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                   for _ in range(B)]).astype(np.int32)
    cv = (rng.standard_normal((B, N, 16)) * 2).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    A = wl.to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    Bc = wl.to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    an = rng.integers(0, V, B).astype(np.int32)
    run_both(d2, ci, cv, g, A, Bc, an, np.array([0, 0.5, 1.5], np.float32), 77, 0, what=f"R={R}")


@pytest.mark.parametrize("N", [1, 2, 15])
def test_select_block_widths(d2, N):
    rng = np.random.default_rng(43 + N)
    B, V, R = 4, 3000, 32
    ci = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                   for _ in range(B)]).astype(np.int32)
    cv = (rng.standard_normal((B, N, 16)) * 2).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    A = wl.to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    Bc = wl.to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    an = rng.integers(0, V, B).astype(np.int32)
    run_both(d2, ci, cv, g, A, Bc, an, np.array([0, 1, 0, 0.3], np.float32), 78, 2, what=f"N={N}")


def test_select_rejections_and_ties(d2):
    rng = np.random.default_rng(44)
    B, N, V, R = 9, 7, 500, 16
    ci = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                   for _ in range(B)]).astype(np.int32)
    cv = np.round(rng.standard_normal((B, N, 16)) * 2).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    A = wl.to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    Bc = wl.to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    an = rng.integers(0, V, B).astype(np.int32)
    temps = np.zeros(B, np.float32)
    cv[0, 3, 4] = np.nan
    cv[1, 0, 0] = np.inf
    ci[2, 6, 15] = V                 # out of range
    an[3] = -5                       # out of range anchor
    g[4] = 0.0                       # no transition term: integer-valued ties everywhere
    temps[5] = np.nan                # invalid temperature: greedy, flagged
    temps[6] = 1e-45
    g[7, 2] = 1e30                   # overflowing scores
    temps[8] = 0.25
    ci[8, 1] = ci[8, 0]              # repeated candidate lists
    st = run_both(d2, ci, cv, g, A, Bc, an, temps, 79, 5, what="rejections")[3]
    assert st[0] & orc.ST_NONFINITE and st[1] & orc.ST_NONFINITE
    assert st[2] & orc.ST_BADTOKEN and st[3] & orc.ST_BADTOKEN
    assert st[5] & orc.ST_BADTEMP and st[6] & orc.ST_BADTEMP


def test_select_viterbi_ties_across_lane_groups(d2):
    # With no transition term every predecessor of a candidate scores dp[kp] + val[k], so
    # equal dp values tie; the path must take the first (smallest) predecessor and the first
    # maximal last candidate. Ties are placed across the 4-predecessor groups the kernel
    # reduces separately (3|4, 7|12, 0|15), and one sequence has integer values in {0, 1}.
    rng = np.random.default_rng(45)
    B, N, V, R = 6, 15, 700, 8
    ci = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                   for _ in range(B)]).astype(np.int32)
    cv = np.zeros((B, N, 16), np.float32)
    cv[1] = rng.integers(0, 2, (N, 16))
    cv[2, :, [3, 4]] = 1.0
    cv[3, :, [7, 12]] = 2.0
    cv[3, :, 9] = 1.0
    cv[4, :, [0, 15]] = -1.0
    cv[4, :, 1:15] = -2.0
    cv[5] = rng.standard_normal((N, 16)).astype(np.float32)
    g = np.zeros((B, N, R), np.float32)
    g[5] = rng.standard_normal((N, R))
    A = wl.to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    Bc = wl.to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    an = rng.integers(0, V, B).astype(np.int32)
    tok, sl, q, st = run_both(d2, ci, cv, g, A, Bc, an, np.zeros(B, np.float32), 80, 1,
                              what="viterbi ties")
    assert not st.any()
    assert np.all(sl[0] == 0) and np.all(sl[2] == 3) and np.all(sl[3] == 7) and np.all(sl[4] == 0)
