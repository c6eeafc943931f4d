"""dflash2_verify against the oracle: bit-exact accept counts, emitted tokens and status."""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import DEV, poison_like, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def _softmax_rows(logits, T):
    z = logits.astype(np.float64) / T
    z -= z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def make_proposals(rng, target_f, N, V, accept_prefix=None):
    """Candidates, q, slots and tokens for B sequences. With accept_prefix, the first
    accept_prefix[b] proposals of sequence b are the target rows' argmax (when it is among
    the candidates), so that greedy chains accept a known prefix."""
    B = target_f.shape[0]
    cand = np.empty((B, N, 16), np.int32)
    for b in range(B):
        for j in range(N):
            row = target_f[b, j]
            top = np.argsort(-row, kind="stable")[:8]            # some strong candidates
            rest = rng.choice(V, 24, replace=False)
            c = list(dict.fromkeys(list(top) + list(rest)))[:16]
            cand[b, j] = rng.permutation(np.array(c, np.int32))
    q = rng.dirichlet(np.ones(16), (B, N)).astype(np.float32)
    slot = np.array([[rng.choice(16, p=q[b, j] / q[b, j].sum()) for j in range(N)]
                     for b in range(B)], np.int32)
    if accept_prefix is not None:
        for b in range(B):
            for j in range(min(accept_prefix[b], N)):
                am = int(np.argmax(target_f[b, j]))
                hit = np.where(cand[b, j] == am)[0]
                if hit.size:
                    slot[b, j] = hit[0]
    tokens = np.take_along_axis(cand, slot[..., None], axis=2)[..., 0].astype(np.int32)
    return cand, q, slot, tokens


def run_both(d2, target, dtype_is_bf16, B, N, ss, rs, V, tokens, cand, q, slot, temp, seed, step,
             status0=None, what=""):
    say(f"verify {what} B={B} N={N} V={V} bf16={dtype_is_bf16}")
    st0 = np.zeros(B, np.int32) if status0 is None else status0
    tgt_dev = to_dev(np.ascontiguousarray(target).reshape(-1))
    st = to_dev(st0.copy())
    n_acc = poison_like((B,), torch.int32)
    out = poison_like((B, N + 1), torch.int32)
    d2.verify(tgt_dev, B, N, ss, rs, V, to_dev(tokens), to_dev(cand), to_dev(q), to_dev(slot),
              to_dev(temp), seed, step, st, n_accept=n_acc, out_tokens=out)
    torch.cuda.synchronize()
    g = (to_host(n_acc), to_host(out), to_host(st))
    o = orc.verify(np.ascontiguousarray(target).reshape(-1), B, N, ss, rs, V, tokens, cand, q,
                   slot, temp, seed, step, status=st0)
    for a, b_, name in zip(g, o, ("n_accept", "out_tokens", "status")):
        np.testing.assert_array_equal(a, b_, err_msg=f"{what}: {name}")
    return g


def test_verify_greedy_bf16_drafter_geometry(d2):
    cfg = wl.CONFIGS[2]
    draft = wl.draft_logits(cfg)
    target = wl.target_rows(cfg, draft)                     # bf16 logits [1, 8, V]
    tf = wl.bf16_bits_to_f32(target)
    rng = np.random.default_rng(31)
    for pref in range(0, 8):
        cand, q, slot, tok = make_proposals(rng, tf, 7, cfg.V, accept_prefix=[pref])
        n, out, st = run_both(d2, target, True, 1, 7, 8 * cfg.V, cfg.V, cfg.V, tok, cand, q, slot,
                              np.zeros(1, np.float32), cfg.seed, pref, what=f"greedy prefix {pref}")


def test_verify_greedy_f32_tiny(d2):
    cfg = wl.CONFIGS[1]
    draft = wl.draft_logits(cfg)
    target = wl.target_rows(cfg, draft)                     # f32 logits [1, 8, 1024]
    rng = np.random.default_rng(32)
    for pref in (0, 3, 7):
        cand, q, slot, tok = make_proposals(rng, target, 7, cfg.V, accept_prefix=[pref])
        run_both(d2, target, False, 1, 7, 8 * cfg.V, cfg.V, cfg.V, tok, cand, q, slot,
                 np.zeros(1, np.float32), cfg.seed, 0, what=f"greedy f32 prefix {pref}")


@pytest.mark.parametrize("V", [248320, 5003])
def test_verify_sampled(d2, V):
    rng = np.random.default_rng(33 + V)
    B, N, T = 6, 7, 0.7
    logits = (rng.standard_normal((B, N + 1, V)) * 2).astype(np.float32)
    p_t = _softmax_rows(logits, T)
    cand, q, slot, tok = make_proposals(rng, p_t, N, V, accept_prefix=[0, 2, 4, 7, 7, 1])
    # make some proposals likely to be accepted: q close to p_t on the candidates
    temps = np.full(B, T, np.float32)
    for step in range(3):
        run_both(d2, p_t, False, B, N, (N + 1) * V, V, V, tok, cand, q, slot, temps, 99, step,
                 what=f"sampled V={V} step {step}")


def test_verify_mixed_batch(d2):
    rng = np.random.default_rng(34)
    B, N, V = 16, 7, 30011
    logits = (rng.standard_normal((B, N + 1, V)) * 2).astype(np.float32)
    temps = np.where(np.arange(B) % 2 == 0, 0.0, 1.0).astype(np.float32)
    p_t = np.stack([_softmax_rows(logits[b], 1.0) for b in range(B)])
    cand, q, slot, tok = make_proposals(rng, p_t, N, V, accept_prefix=list(range(B)))
    run_both(d2, p_t, False, B, N, (N + 1) * V, V, V, tok, cand, q, slot, temps, 7, 3,
             what="mixed greedy/sampled")


def test_verify_all_accept_and_bonus(d2):
    # q equal to p_t on every candidate and the candidates hold all the mass: every proposal
    # is accepted and the bonus comes from row N
    rng = np.random.default_rng(35)
    B, N, V = 8, 7, 4096
    p_t = np.zeros((B, N + 1, V), np.float32)
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                     for _ in range(B)]).astype(np.int32)
    q = rng.dirichlet(np.ones(16), (B, N)).astype(np.float32)
    for b in range(B):
        for j in range(N):
            p_t[b, j, cand[b, j]] = q[b, j]
        p_t[b, N] = rng.dirichlet(np.ones(V))
    slot = rng.integers(0, 16, (B, N)).astype(np.int32)
    tok = np.take_along_axis(cand, slot[..., None], axis=2)[..., 0]
    n, out, st = run_both(d2, p_t, False, B, N, (N + 1) * V, V, V, tok, cand, q, slot,
                          np.ones(B, np.float32), 5, 0, what="all accept")
    assert np.all(n == N)


def test_verify_status_paths(d2):
    rng = np.random.default_rng(36)
    B, N, V = 10, 7, 2000
    logits = rng.standard_normal((B, N + 1, V)).astype(np.float32)
    p_t = np.stack([_softmax_rows(logits[b], 1.0) for b in range(B)])
    cand, q, slot, tok = make_proposals(rng, p_t, N, V, accept_prefix=[3] * B)
    temps = np.ones(B, np.float32)
    p_t[0, :, :] = 0.0                                    # zero mass everywhere
    p_t[1, 0, 5] = -0.25                                  # a negative probability
    p_t[2, 1, 7] = np.nan
    tok[3, 0] = -1                                        # no proposal: plain sample
    slot[4, 0] = (slot[4, 0] + 1) % 16                    # slot does not match the token
    temps[5] = np.nan                                     # invalid temperature: greedy
    temps[6] = -1.0
    temps[7] = 1e-45                                      # reciprocal overflows
    cand[8, 2, :] = cand[8, 2, 0]                         # duplicated candidates
    q[9, 0, :] = 2.0                                      # q out of range
    st0 = np.zeros(B, np.int32)
    st0[3] = 16                                           # OR-ed, never cleared
    n, out, st = run_both(d2, p_t, False, B, N, (N + 1) * V, V, V, tok, cand, q, slot, temps, 11,
                          2, status0=st0, what="status paths")
    assert st[0] & orc.ST_ZEROMASS
    assert st[4] & orc.ST_BADTOKEN
    assert st[5] & orc.ST_BADTEMP and st[6] & orc.ST_BADTEMP and st[7] & orc.ST_BADTEMP


def test_verify_sampling_on_bf16_target_falls_back_to_greedy(d2):
    cfg = wl.CONFIGS[2]
    draft = wl.draft_logits(cfg)
    target = wl.target_rows(cfg, draft)
    rng = np.random.default_rng(37)
    cand, q, slot, tok = make_proposals(rng, wl.bf16_bits_to_f32(target), 7, cfg.V, accept_prefix=[2])
    n, out, st = run_both(d2, target, True, 1, 7, 8 * cfg.V, cfg.V, cfg.V, tok, cand, q, slot,
                          np.full(1, 0.8, np.float32), 1, 0, what="bf16 sampled")
    assert st[0] & orc.ST_BADPROB


@pytest.mark.parametrize("N", [1, 15])
def test_verify_block_widths(d2, N):
    rng = np.random.default_rng(38 + N)
    B, V = 5, 3001
    logits = rng.standard_normal((B, N + 1, V)).astype(np.float32)
    p_t = np.stack([_softmax_rows(logits[b], 0.9) for b in range(B)])
    cand, q, slot, tok = make_proposals(rng, p_t, N, V, accept_prefix=[N, 0, 1, N, 2])
    temps = np.array([0, 0.9, 0.9, 0, 0.9], np.float32)
    run_both(d2, p_t, False, B, N, (N + 1) * V, V, V, tok, cand, q, slot, temps, 3, 1,
             what=f"N={N}")


def test_verify_lossless_on_gpu(d2):
    # V = 16 and the 16 candidates cover it; 2^20 single-proposal trials share one row pair
    # through a zero sequence stride; the first emitted token must follow p_t
    rng = np.random.default_rng(39)
    V, N = 16, 1
    p_t = rng.dirichlet(np.ones(V)).astype(np.float32)
    q_d = rng.dirichlet(np.ones(V)).astype(np.float32)
    target = np.stack([p_t, p_t])
    perm = rng.permutation(V).astype(np.int32)
    counts = np.zeros(V, np.int64)
    M = 1 << 20
    Bc = 1 << 16
    tgt_dev = to_dev(target.reshape(-1))
    for step in range(M // Bc):
        say(f"verify lossless chunk {step}")
        d = rng.choice(V, size=(Bc, N), p=q_d / q_d.sum()).astype(np.int32)
        slot = np.argsort(perm)[d].astype(np.int32)
        cand = np.ascontiguousarray(np.broadcast_to(perm, (Bc, N, 16)))
        q = np.ascontiguousarray(np.broadcast_to(q_d[perm], (Bc, N, 16)))
        st = torch.zeros(Bc, dtype=torch.int32, device=DEV)
        n, out, _ = d2.verify(tgt_dev, Bc - 1, N, 0, V, V, to_dev(d[:-1]), to_dev(cand[:-1]),
                              to_dev(q[:-1]), to_dev(slot[:-1]), torch.ones(Bc - 1, device=DEV),
                              17, step, st[:-1])
        first = to_host(out)[:, 0]
        counts += np.bincount(first, minlength=V)
        if step == 0:   # and the first chunk matches the oracle exactly
            o = orc.verify(target.reshape(-1), Bc - 1, N, 0, V, V, d[:-1], cand[:-1], q[:-1],
                           slot[:-1], np.ones(Bc - 1, np.float32), 17, step)
            np.testing.assert_array_equal(to_host(out), o[1])
    tot = counts.sum()
    e = tot * p_t.astype(np.float64)
    chi2 = float(((counts - e) ** 2 / e).sum())
    assert chi2 < 37.70, chi2
