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


def test_verify_lossless_every_position_on_gpu(d2):
    # N = 3 proposals, each slot with its own target row, candidate order and q; proposal j
    # drawn from slot j's q. Every chunk of trials is bit-exact against the oracle, and over
    # all 2^20 trials the token emitted at each block position k follows target row k among
    # the trials that reach k (so a residual or an accept test that used another slot's
    # candidates, q or row would fail).
    rng = np.random.default_rng(40)
    V, N = 16, 3
    rows = rng.dirichlet(np.ones(V), N + 1).astype(np.float32)
    qs = np.stack([0.5 * rows[j] + 0.5 * rng.dirichlet(np.ones(V)) for j in range(N)]).astype(np.float32)
    perms = np.stack([rng.permutation(V) for _ in range(N)]).astype(np.int32)
    qc = np.stack([qs[j][perms[j]] for j in range(N)]).astype(np.float32)
    M, Bc = 1 << 20, (1 << 16) - 1
    counts = np.zeros((N + 1, V), np.int64)
    reached = np.zeros(N + 1, np.int64)
    acc_hits = np.zeros(N, np.int64)
    tgt_dev = to_dev(rows.reshape(-1))
    done, step = 0, 0
    while done < M:
        B = min(Bc, M - done)
        say(f"verify every-position chunk {step} B={B}")
        d = np.stack([rng.choice(V, size=B, p=qs[j] / qs[j].sum()) for j in range(N)],
                     axis=1).astype(np.int32)
        slot = np.stack([np.argsort(perms[j])[d[:, j]] for j in range(N)], axis=1).astype(np.int32)
        cand = np.ascontiguousarray(np.broadcast_to(perms, (B, N, 16)))
        q = np.ascontiguousarray(np.broadcast_to(qc, (B, N, 16)))
        T = np.ones(B, np.float32)
        st = torch.zeros(B, dtype=torch.int32, device=DEV)
        n_dev, out_dev, _ = d2.verify(tgt_dev, B, N, 0, V, V, to_dev(d), to_dev(cand), to_dev(q),
                                      to_dev(slot), to_dev(T), 23, step, st)
        n, out = to_host(n_dev), to_host(out_dev)
        o = orc.verify(rows.reshape(-1), B, N, 0, V, V, d, cand, q, slot, T, 23, step)
        np.testing.assert_array_equal(n, o[0], err_msg=f"chunk {step}: n_accept")
        np.testing.assert_array_equal(out, o[1], err_msg=f"chunk {step}: out_tokens")
        assert not to_host(st).any()
        for k in range(N + 1):
            r = n >= k
            reached[k] += int(r.sum())
            counts[k] += np.bincount(out[r, k], minlength=V)
            if k < N:
                acc_hits[k] += int((n[r] > k).sum())
        done += B
        step += 1
    for k in range(N + 1):
        e = reached[k] * rows[k].astype(np.float64)
        chi2 = float(((counts[k] - e) ** 2 / e).sum())
        assert chi2 < 37.70, (k, chi2)
        if k < N:
            want = np.minimum(rows[k].astype(np.float64), qs[k]).sum()
            got = acc_hits[k] / reached[k]
            assert abs(got - want) < 5 * np.sqrt(want * (1 - want) / reached[k]), (k, got, want)


def _special_greedy_rows(rng, V, f32):
    """Six sequences of 8 rows whose maxima are decided by NaN, signed zeros, ties across
    lanes, waves, vectors and chunks, the ragged last chunk, and infinities."""
    B, R = 6, 8
    x = rng.standard_normal((B, R, V)).astype(np.float32)
    x[1] = -(np.abs(x[1]) + 1.0)
    x[4] = -np.inf
    bits = x.copy().view(np.uint32) if f32 else wl.to_bf16_bits(x)
    if f32:
        pnan, nnan, pz, nz, pinf = 0x7FC00001, 0xFFC00000, 0x00000000, 0x80000000, 0x7F800000
        big = int(np.float32(50.0).view(np.uint32))
    else:
        pnan, nnan, pz, nz, pinf = 0x7FC1, 0xFFC0, 0x0000, 0x8000, 0x7F80
        big = int(wl.to_bf16_bits(np.float32(50.0))[0])
    for r in range(R):
        # sequence 0: NaN of either sign, sometimes both, at random depths
        pos = rng.choice(V, 3, replace=False)
        if r % 3 != 1:
            bits[0, r, pos[0]] = pnan
        if r % 3 != 0:
            bits[0, r, pos[1]] = nnan
        # sequence 1: all negative but two zeros of opposite signs, in either order
        i1, i2 = sorted(rng.choice(V, 2, replace=False))
        bits[1, r, i1], bits[1, r, i2] = (nz, pz) if r % 2 == 0 else (pz, nz)
        # sequence 2: one maximum repeated at indices that differ by a lane, a vector, a
        # wave and a chunk
        a = int(rng.integers(0, V - 5000))
        for d in (0, 1, 4, 8, 256, 512, 1024, 2048, 4096)[r % 4:]:
            bits[2, r, a + d] = big
        # sequence 3: maximum at the very start, the very end, and chunk edges
        at = (0, V - 1, 2047, 2048, V - 2, 1023, 1024, V // 2)[r]
        bits[3, r, at] = big
        # sequence 4: all -inf, then +inf twice, then one finite value
        if r == 1:
            bits[4, r, [77, 70000]] = pinf
        elif r >= 2:
            bits[4, r, rng.integers(0, V)] = big
    return bits.view(np.float32) if f32 else bits


@pytest.mark.parametrize("f32", [False, True])
def test_verify_greedy_special_rows(d2, f32):
    # the proposals are each row's first element under the top-16 order (from the oracle's
    # top-16), so every row's decision is visible in n_accept / out_tokens; then each row
    # in turn gets a wrong proposal, so that its first element is the emitted token
    rng = np.random.default_rng(71 + f32)
    V, N = 248320, 7
    bits = _special_greedy_rows(rng, V, f32)
    B = bits.shape[0]
    first = np.stack([orc.topk16_rows(bits[b])[0][:, 0] for b in range(B)]).astype(np.int32)
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                     for _ in range(B)]).astype(np.int32)
    slot = rng.integers(0, 16, (B, N)).astype(np.int32)
    for b in range(B):
        for j in range(N):
            if first[b, j] not in cand[b, j]:
                cand[b, j, slot[b, j]] = first[b, j]
            slot[b, j] = int(np.where(cand[b, j] == first[b, j])[0][0])
    q = rng.dirichlet(np.ones(16), (B, N)).astype(np.float32)
    temps = np.zeros(B, np.float32)
    for wrong in [None] + list(range(N)):
        s = slot.copy()
        if wrong is not None:
            s[:, wrong] = (s[:, wrong] + 1) % 16
        tok = np.take_along_axis(cand, s[..., None], axis=2)[..., 0].astype(np.int32)
        n, out, st = run_both(d2, bits, not f32, B, N, (N + 1) * V, V, V, tok, cand, q, s, temps,
                              1, 0, what=f"greedy special rows f32={f32} wrong={wrong}")
        if wrong is None:
            assert np.all(n == N)


@pytest.mark.parametrize("sampled", [False, True])
def test_verify_width_cap(d2, sampled):
    # Verifying the first N_v of N = 7 proposals: the caller compacts the proposal arrays to
    # N_v columns on the device; the target is read in place from the full 8-row block
    # through its strides (rows 0..N_v). GPU and oracle must agree bit for bit.
    rng = np.random.default_rng(41 + sampled)
    B, N = 4, 7
    if sampled:
        V = 5003
        logits = (rng.standard_normal((B, N + 1, V)) * 2).astype(np.float32)
        target = np.stack([_softmax_rows(logits[b], 0.8) for b in range(B)])
        temps = np.full(B, 0.8, np.float32)
        tf = target
    else:
        cfg = wl.CONFIGS[2]
        V = cfg.V
        draft = wl.draft_logits(cfg)
        one = wl.target_rows(cfg, draft)[0]                  # bf16 logits [8, V]
        target = np.stack([np.roll(one, 977 * b, axis=1) for b in range(B)])
        temps = np.zeros(B, np.float32)
        tf = wl.bf16_bits_to_f32(target)
    cand, q, slot, tok = make_proposals(rng, tf, N, V, accept_prefix=[7, 3, 1, 5])
    tgt_dev = to_dev(np.ascontiguousarray(target).reshape(-1))
    full = [to_dev(a) for a in (tok, cand, q, slot)]
    for nv in (1, 3, 5):
        say(f"verify width cap N_v={nv} of {N}, sampled={sampled}")
        tok_c, cand_c, q_c, slot_c = (a[:, :nv].contiguous() for a in full)
        st = torch.zeros(B, dtype=torch.int32, device=DEV)
        n_acc = poison_like((B,), torch.int32)
        out = poison_like((B, nv + 1), torch.int32)
        d2.verify(tgt_dev, B, nv, (N + 1) * V, V, V, tok_c, cand_c, q_c, slot_c, to_dev(temps),
                  11, nv, st, n_accept=n_acc, out_tokens=out)
        torch.cuda.synchronize()
        o = orc.verify(np.ascontiguousarray(target).reshape(-1), B, nv, (N + 1) * V, V, V,
                       tok[:, :nv].copy(), cand[:, :nv].copy(), q[:, :nv].copy(),
                       slot[:, :nv].copy(), temps, 11, nv)
        for a, b_, name in zip((to_host(n_acc), to_host(out), to_host(st)), o,
                               ("n_accept", "out_tokens", "status")):
            np.testing.assert_array_equal(a, b_, err_msg=f"N_v={nv}: {name}")
        assert np.all(to_host(n_acc) <= nv)


@pytest.mark.parametrize("c", [2, 5])
def test_verify_all_accept_inputs(d2, c):
    # the workload's targets changed only at the proposals so that every proposal is
    # accepted: greedy sequences then read every row, sampled ones draw the bonus
    cfg = wl.CONFIGS[c]
    seqs = list(range(min(cfg.B, 12)))
    vi = wl.all_accept_verify_inputs(cfg, iset=0, seqs=seqs)
    B = len(seqs)
    for step in (0, 1):
        n, out, st = run_both(d2, vi.target, vi.target.dtype == np.uint16, B, cfg.N,
                              cfg.P * cfg.V, cfg.V, cfg.V, vi.tokens, vi.cand_idx, vi.q,
                              vi.slot, vi.temperature, cfg.seed, step,
                              what=f"all-accept config {c} step {step}")
        assert np.all(n == cfg.N) and not st.any()


def test_verify_repeated_calls_share_one_workspace(d2):
    # kernel 1 clears the accepted-chain row words and arrival counters that kernel 2 folds
    # into with atomics; calls that reuse one workspace, each accepting different prefixes,
    # must each match the oracle
    rng = np.random.default_rng(41)
    B, N, V = 48, 7, 30011
    ws = d2.workspace(d2.verify_workspace_bytes(B, N, V, d2.F32), DEV)
    ws.fill_(0xA5)                                          # stale contents, not zeros
    for call in range(10):
        logits = (rng.standard_normal((B, N + 1, V)) * 2).astype(np.float32)
        temps = np.where(rng.random(B) < 0.5, 0.0, 0.8).astype(np.float32)
        p_t = np.stack([_softmax_rows(logits[b], 0.8) for b in range(B)])
        pref = rng.integers(0, N + 1, B)
        cand, q, slot, tok = make_proposals(rng, p_t, N, V, accept_prefix=list(pref))
        say(f"verify shared workspace call {call}")
        st = torch.zeros(B, dtype=torch.int32, device=DEV)
        n_dev = poison_like((B,), torch.int32)
        o_dev = poison_like((B, N + 1), torch.int32)
        d2.verify(to_dev(p_t.reshape(-1)), B, N, (N + 1) * V, V, V, to_dev(tok), to_dev(cand),
                  to_dev(q), to_dev(slot), to_dev(temps), 13, call, st, n_accept=n_dev,
                  out_tokens=o_dev, ws=ws)
        torch.cuda.synchronize()
        o = orc.verify(p_t.reshape(-1), B, N, (N + 1) * V, V, V, tok, cand, q, slot, temps, 13,
                       call)
        np.testing.assert_array_equal(to_host(n_dev), o[0], err_msg=f"call {call}: n_accept")
        np.testing.assert_array_equal(to_host(o_dev), o[1], err_msg=f"call {call}: out_tokens")
        np.testing.assert_array_equal(to_host(st), o[2], err_msg=f"call {call}: status")
        assert (o[0][temps == 0] > 0).any()                 # some greedy chains go past row 0
