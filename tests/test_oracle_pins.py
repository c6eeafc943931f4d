"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a library routine, a differently formulated
brute force, a closed form, an error bound printed on the pages, or a statistical
invariant, chosen so that a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, a wrong tie rule) fails at least one of them. No GPU is needed.
"""
import itertools

import numpy as np
import pytest
import torch

from block_drafter_draft_amd.workloads import bf16_bits_to_f32, to_bf16_bits


# ----------------------------------------------------------------------------------------
# Philox4x64-10: numpy's Philox bit generator is the same published generator.
# ----------------------------------------------------------------------------------------

def _numpy_philox_block(ctr, key):
    # numpy advances its 256-bit counter before producing a block, so start one below.
    c = [int(x) for x in ctr]
    for w in range(4):
        if c[w] > 0:
            c[w] -= 1
            break
        c[w] = 2**64 - 1
    # (uint64 arrays: numpy's constructor rounds large Python ints through float64)
    bg = np.random.Philox(counter=np.array(c, dtype=np.uint64),
                          key=np.array([int(k) for k in key], dtype=np.uint64))
    return np.array(bg.random_raw(4), dtype=np.uint64)


def test_philox_matches_numpy(orc):
    rng = np.random.default_rng(7)
    cases = [([0, 0, 0, 0], [0, 0]), ([2**64 - 1] * 4, [2**64 - 1] * 2)]
    for _ in range(200):
        cases.append((rng.integers(0, 2**64, size=4, dtype=np.uint64),
                      rng.integers(0, 2**64, size=2, dtype=np.uint64)))
    for step, b, j in [(0, 0, 1), (5, 63, 8), (2**40 + 3, 12, 7)]:
        cases.append(([step, b, j, 0], [0xDF20002, 0]))
    for ctr, key in cases:
        assert np.array_equal(orc.philox4x64_10(ctr, key), _numpy_philox_block(ctr, key)), (ctr, key)


def test_philox_published_zero_vector(orc):
    # Random123's known answer for philox4x64-10 with zero counter and zero key.
    out = orc.philox4x64_10([0, 0, 0, 0], [0, 0])
    assert [int(x) for x in out] == [0x16554D9ECA36314C, 0xDB20FE9D672D0FDC,
                                     0xD7E772CEE186176B, 0x7E68B68AEC7BA23B]


# ----------------------------------------------------------------------------------------
# exp_c: accuracy against binary64 exp over a dense sweep of [-87, 0].
# ----------------------------------------------------------------------------------------

def _ulp_err(approx: np.ndarray, y: np.ndarray) -> np.ndarray:
    exact = np.exp(y.astype(np.float64))
    spacing = np.spacing(exact.astype(np.float32)).astype(np.float64)
    return np.abs(approx.astype(np.float64) - exact) / spacing


def test_exp_c_accuracy(orc):
    # every 61st binary32 pattern from -0 down to -87, plus the ends exhaustively
    lo_bits = np.float32(-87.0).view(np.uint32)
    bits = np.arange(np.uint32(0x80000000), lo_bits + 1, 61, dtype=np.uint64).astype(np.uint32)
    ends = np.concatenate([np.arange(0x80000000, 0x80000000 + 200000, dtype=np.uint64),
                           np.arange(lo_bits - 200000, lo_bits + 1, dtype=np.uint64)]).astype(np.uint32)
    y = np.concatenate([bits, ends]).view(np.float32)
    err = _ulp_err(orc.exp_c_array(y), y)
    assert err.max() <= 2.0, (err.max(), y[np.argmax(err)])
    assert np.mean(err) < 0.5


def test_exp_c_special_values(orc):
    assert orc.exp_c(0.0) == 1.0
    assert orc.exp_c(-0.0) == 1.0
    assert orc.exp_c(float("-inf")) == 0.0
    assert orc.exp_c(-87.0001) == 0.0
    assert orc.exp_c(-87.0) > 0.0
    # monotone non-decreasing on a dense grid
    y = np.linspace(-87, 0, 2_000_001, dtype=np.float32)
    e = orc.exp_c_array(y)
    assert np.all(np.diff(e) >= 0)


# ----------------------------------------------------------------------------------------
# Block attention
# ----------------------------------------------------------------------------------------

def _attn_inputs(rng, B, P, Hq, Hkv, D, S, dtype=np.float32):
    def mk(*shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return to_bf16_bits(x) if dtype == np.uint16 else x
    return mk(B, P, Hq, D), mk(B, P, Hkv, D), mk(B, P, Hkv, D), mk(B, S, Hkv, D), mk(B, S, Hkv, D)


def _as_f64(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def _attn_masked_bruteforce(q, kb, vb, kr, vr, L, W):
    """Materialise keys by absolute position and apply an explicit [P x keys] mask."""
    q, kb, vb, kr, vr = map(_as_f64, (q, kb, vb, kr, vr))
    B, P, Hq, D = q.shape
    S, Hkv = kr.shape[1], kr.shape[2]
    grp = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        Lb = int(L[b])
        first_kept = max(0, Lb - S)  # oldest context position still in the ring
        pos = np.arange(first_kept, Lb)
        keys = np.concatenate([kr[b, pos % S], kb[b]], axis=0)      # [n, Hkv, D]
        vals = np.concatenate([vr[b, pos % S], vb[b]], axis=0)
        is_blk = np.concatenate([np.zeros(len(pos), bool), np.ones(P, bool)])
        abs_pos = np.concatenate([pos, Lb + np.arange(P)])
        qpos = Lb + np.arange(P)
        mask = is_blk[None, :] | ((qpos[:, None] - abs_pos[None, :]) < W)   # [P, n]
        for h in range(Hq):
            g = h // grp
            s = q[b, :, h, :] @ keys[:, g, :].T / np.sqrt(D)                  # [P, n]
            s = np.where(mask, s, -np.inf)
            s -= s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w /= w.sum(axis=1, keepdims=True)
            out[b, :, h, :] = w @ vals[:, g, :]
    return out


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
@pytest.mark.parametrize("L,W,S", [(128, 64, 128), (3000, 64, 96), (9, 2048, 2048),
                                   (2047, 2048, 2048), (5, 3, 16), (0, 16, 16), (40, 1, 8)])
def test_attention_matches_masked_bruteforce(orc, dtype, L, W, S):
    rng = np.random.default_rng(L * 7 + W + S)
    B, P, Hq, Hkv, D = 2, 8, 4, 2, 64 if S != 2048 else 128
    q, kb, vb, kr, vr = _attn_inputs(rng, B, P, Hq, Hkv, D, S, dtype)
    Ls = np.array([L, max(0, L - 3)], np.int32)
    got = orc.block_attn(q, kb, vb, kr, vr, Ls, W)
    ref = _attn_masked_bruteforce(q, kb, vb, kr, vr, Ls, W)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_attention_full_window_is_sdpa(orc):
    # With every context key visible the op is plain noncausal GQA attention.
    rng = np.random.default_rng(3)
    B, P, Hq, Hkv, D, S, L = 2, 8, 8, 2, 64, 64, 50
    q, kb, vb, kr, vr = _attn_inputs(rng, B, P, Hq, Hkv, D, S)
    got = orc.block_attn(q, kb, vb, kr, vr, np.array([L, L], np.int32), W=10_000)
    keys = torch.from_numpy(np.concatenate([kr[:, :L], kb], axis=1)).double()   # [B,n,Hkv,D]
    vals = torch.from_numpy(np.concatenate([vr[:, :L], vb], axis=1)).double()
    rep = Hq // Hkv
    kk = keys.permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)                  # [B,Hq,n,D]
    vv = vals.permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    qq = torch.from_numpy(q).double().permute(0, 2, 1, 3)                        # [B,Hq,P,D]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).permute(0, 2, 1, 3)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_attention_invariants(orc):
    rng = np.random.default_rng(11)
    B, P, Hq, Hkv, D, S = 1, 8, 4, 1, 32, 32
    q, kb, vb, kr, vr = _attn_inputs(rng, B, P, Hq, Hkv, D, S)
    # constant value rows give that constant whatever the weights
    c = rng.standard_normal(D).astype(np.float32)
    vb_c = np.broadcast_to(c, vb.shape).copy()
    vr_c = np.broadcast_to(c, vr.shape).copy()
    out = orc.block_attn(q, kb, vb_c, kr, vr_c, np.array([30], np.int32), W=20)
    np.testing.assert_allclose(out, np.broadcast_to(c.astype(np.float64), out.shape), rtol=1e-12)
    # W = 1 hides every context key, which is the same as an empty context
    a = orc.block_attn(q, kb, vb, kr, vr, np.array([30], np.int32), W=1)
    b = orc.block_attn(q, kb, vb, kr, vr, np.array([0], np.int32), W=64)
    np.testing.assert_array_equal(a, b)
    # scale 0 gives the plain mean of the visible values; slot i sees (W-1-i) context keys
    L, W = 30, 10
    out = orc.block_attn(q, kb, vb, kr, vr, np.array([L], np.int32), W=W, scale=0.0)
    for i in range(P):
        vis = [kr_row % S for kr_row in range(L + i - W + 1, L)]
        mean = np.concatenate([vr[0, vis, 0], vb[0, :, 0]], axis=0).astype(np.float64).mean(0)
        np.testing.assert_allclose(out[0, i, 0], mean, rtol=1e-12)
    # keys outside the window do not matter, keys inside do
    kr2, vr2 = kr.copy(), vr.copy()
    kr2[0, (L - W) % S] += 5.0          # position L-W is outside every slot's window
    vr2[0, (L - W) % S] += 5.0
    np.testing.assert_array_equal(out, orc.block_attn(q, kb, vb, kr2, vr2, np.array([L], np.int32), W=W, scale=0.0))
    vr2[0, (L - 1) % S] += 5.0          # position L-1 is visible to every slot
    assert not np.array_equal(out, orc.block_attn(q, kb, vb, kr2, vr2, np.array([L], np.int32), W=W, scale=0.0))


# ----------------------------------------------------------------------------------------
# Dynamic two-tap conv
# ----------------------------------------------------------------------------------------

def _conv_inputs(rng, B=2, P=8, C=64):
    x = rng.standard_normal((B, P, C)).astype(np.float32)
    base = rng.uniform(-1, 1, (2, C)).astype(np.float32)
    delta = rng.uniform(-1, 1, (B, P, 2, C // 16)).astype(np.float32)
    return x, base, delta


def test_conv_identity_and_shift(orc):
    rng = np.random.default_rng(1)
    x, _, _ = _conv_inputs(rng)
    C = x.shape[2]
    zero = np.zeros((2, 8, 2, C // 16), np.float32)
    ident = np.stack([np.ones(C), np.zeros(C)]).astype(np.float32)
    np.testing.assert_array_equal(orc.dynconv2(x, ident, zero), x.astype(np.float64))
    shift = np.stack([np.zeros(C), np.ones(C)]).astype(np.float32)
    out = orc.dynconv2(x, shift, zero)
    np.testing.assert_array_equal(out[:, 1:], x[:, :-1].astype(np.float64))
    np.testing.assert_array_equal(out[:, 0], 0.0)


def test_conv_static_taps_is_depthwise_conv1d(orc):
    rng = np.random.default_rng(2)
    x, base, _ = _conv_inputs(rng, C=256)
    B, P, C = x.shape
    got = orc.dynconv2(x, base, np.zeros((B, P, 2, C // 16), np.float32))
    xt = torch.from_numpy(x).double().permute(0, 2, 1)                  # [B, C, P]
    # conv1d correlates: with one zero on the left, weight[...,0] meets x[i-1], weight[...,1] x[i]
    w = torch.from_numpy(np.stack([base[1], base[0]], axis=-1)).double().unsqueeze(1)   # [C,1,2]
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (1, 0)), w, groups=C)
    np.testing.assert_allclose(got, ref.permute(0, 2, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_conv_group_mapping_and_isolation(orc):
    rng = np.random.default_rng(3)
    x, base, delta = _conv_inputs(rng, C=128)
    B, P, C = x.shape
    # a dynamic coefficient on one group, with no base, touches exactly that group's channels
    d = np.zeros_like(delta)
    d[1, 4, 0, 5] = 2.0
    out = orc.dynconv2(x, np.zeros_like(base), d)
    nz = np.argwhere(out != 0)
    assert set(map(tuple, nz)) == {(1, 4, c) for c in range(80, 96) if x[1, 4, c] != 0}
    np.testing.assert_array_equal(out[1, 4, 80:96], 2.0 * x[1, 4, 80:96].astype(np.float64))
    # tap 1 of the same group reads the previous position
    d2 = np.zeros_like(delta)
    d2[0, 3, 1, 2] = 1.0
    out = orc.dynconv2(x, np.zeros_like(base), d2)
    np.testing.assert_array_equal(out[0, 3, 32:48], x[0, 2, 32:48].astype(np.float64))
    # block-boundary isolation: position 0 never sees anything but itself
    ref = orc.dynconv2(x, base, delta)
    x2 = x.copy()
    x2[1] += 1.0
    x2[0, 1:] += 1.0
    out = orc.dynconv2(x2, base, delta)
    np.testing.assert_array_equal(out[0, 0], ref[0, 0])
    # a change at position i reaches i and i+1 only
    x3 = x.copy()
    x3[0, 3] += 1.0
    diff = np.any(orc.dynconv2(x3, base, delta) != ref, axis=2)
    assert set(map(tuple, np.argwhere(diff))) <= {(0, 3), (0, 4)}


# ----------------------------------------------------------------------------------------
# Top-16
# ----------------------------------------------------------------------------------------

def _py_order_key(v, i):
    # (class, value, index): NaN first, then by value descending, then by index ascending
    if np.isnan(v):
        return (0, 0.0, i)
    return (1, -float(v), i)


def _py_top16(row):
    return sorted(range(len(row)), key=lambda i: _py_order_key(row[i], i))[:16]


def test_topk_matches_lexsort_and_torch(orc):
    rng = np.random.default_rng(4)
    rows = rng.standard_normal((6, 5000)).astype(np.float32)
    rows[3] = np.round(rows[3] * 4) / 4          # many ties
    rows[4] = np.round(rows[4])                  # heavy ties
    rows[5, ::7] = -0.0
    rows[5, 1::7] = 0.0
    idx, val = orc.topk16_rows(rows)
    for r in range(rows.shape[0]):
        order = np.lexsort((np.arange(rows.shape[1]), -rows[r]))[:16]
        np.testing.assert_array_equal(idx[r], order)
        np.testing.assert_array_equal(val[r], rows[r, order])
        t = torch.sort(torch.from_numpy(rows[r]), descending=True, stable=True).indices[:16]
        np.testing.assert_array_equal(idx[r], t.numpy())


def test_topk_edge_rows(orc):
    # four 4097-wide rows: NaNs, both infinities, ties across 512-element chunk boundaries,
    # and an all -inf row (the shapes of the pages' top-k edge test)
    V = 4097
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((4, V)).astype(np.float32)
    rows[0, [4000, 5, 2048, 511, 512]] = np.nan
    rows[0, [7, 3000]] = np.inf
    rows[0, [1, 2, 4096]] = -np.inf
    rows[1, :] = -1.0
    rows[1, [511, 512, 1023, 1024, 4095, 4096, 0]] = 3.0
    rows[1, [100, 600, 1100, 1600, 2100, 2600, 3100, 3600, 4000, 4050]] = 3.0
    rows[2, :] = -np.inf
    rows[3, ::2] = np.inf
    idx, val = orc.topk16_rows(rows)
    for r in range(4):
        want = _py_top16(rows[r])
        np.testing.assert_array_equal(idx[r], want)
    np.testing.assert_array_equal(idx[0, :5], [5, 511, 512, 2048, 4000])
    np.testing.assert_array_equal(idx[0, 5:7], [7, 3000])
    np.testing.assert_array_equal(idx[2], np.arange(16))
    np.testing.assert_array_equal(idx[3], np.arange(0, 32, 2))
    assert np.all(np.isneginf(val[2]))


def test_topk_bf16_widening_and_strides(orc):
    rng = np.random.default_rng(6)
    B, P, V = 3, 8, 1000
    logits = rng.standard_normal((B, P, V)).astype(np.float32)
    bits = to_bf16_bits(logits)
    widened = bf16_bits_to_f32(bits)
    idx, val = orc.topk16(bits, B, P - 1, 1, P * V, V, V)
    for b in range(B):
        for r in range(P - 1):
            want = _py_top16(widened[b, r + 1])
            np.testing.assert_array_equal(idx[b, r], want)
            np.testing.assert_array_equal(val[b, r], widened[b, r + 1, want])


def test_topk_tiny_bruteforce(orc):
    rng = np.random.default_rng(8)
    for trial in range(50):
        V = 16 + trial
        row = rng.integers(-3, 4, size=V).astype(np.float32)
        row[rng.integers(0, V, size=2)] = [np.nan, np.inf][trial % 2]
        idx, _ = orc.topk16_rows(row[None, :])
        np.testing.assert_array_equal(idx[0], _py_top16(row))


# ----------------------------------------------------------------------------------------
# Selector: lattice within the pages' rounding bound; best path by enumeration; walk
# ----------------------------------------------------------------------------------------

def _selector_inputs(rng, B, N, V, R, heavy=False):
    cand_idx = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                         for _ in range(B)]).astype(np.int32)
    cand_val = rng.normal(0, 2, (B, N, 16)).astype(np.float32)
    gate = rng.standard_normal((B, N, R)).astype(np.float32)
    if heavy:
        A = to_bf16_bits((0.25 * rng.standard_t(3, (V, R))).astype(np.float32))
        Bc = to_bf16_bits((0.25 * rng.standard_t(3, (V, R))).astype(np.float32))
    else:
        A = to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
        Bc = to_bf16_bits(rng.normal(0, 0.25, (V, R)).astype(np.float32))
    anchor = rng.integers(0, V, B).astype(np.int32)
    return cand_idx, cand_val, gate, A, Bc, anchor


@pytest.mark.parametrize("heavy", [False, True])
def test_selector_lattice_within_pages_bound(orc, heavy):
    rng = np.random.default_rng(9)
    B, N, V, R = 3, 7, 3000, 256
    ci, cv, g, A, Bc, an = _selector_inputs(rng, B, N, V, R, heavy)
    *_, lat = orc.select(ci, cv, g, A, Bc, an, np.zeros(B, np.float32), 1, 0, want_lattice=True)
    Af, Bf = bf16_bits_to_f32(A).astype(np.float64), bf16_bits_to_f32(Bc).astype(np.float64)
    u = 2.0 ** -24
    gam = (R + 2) * u / (1 - (R + 2) * u)
    worst = 0.0
    for b in range(B):
        for i in range(N):
            preds = [an[b]] if i == 0 else list(ci[b, i - 1])
            for kp, p in enumerate(preds):
                for k in range(16):
                    c = ci[b, i, k]
                    terms = Af[p] * g[b, i].astype(np.float64) * Bf[c]
                    ref = cv[b, i, k] + terms.sum()
                    bound = gam * np.abs(terms).sum() + 2 * u / (1 - u) * abs(ref)
                    err = abs(float(lat[b, i, kp, k]) - ref)
                    assert err <= bound, (b, i, kp, k, err, bound)
                    worst = max(worst, err / bound if bound else 0)
            if i == 0:
                assert np.all(lat[b, 0, 1:] == 0)
    assert worst < 1.0


def _best_paths_exhaustive(s1, s):
    K, N = s1.shape[0], s.shape[0] + 1
    best, arg = None, None
    for path in itertools.product(range(K), repeat=N):
        tot = float(s1[path[0]]) + sum(float(s[i - 1, path[i - 1], path[i]]) for i in range(1, N))
        # ties: the path that is smallest comparing the last slot first
        key = (-tot, tuple(reversed(path)))
        if best is None or key < best:
            best, arg = key, path
    return np.array(arg, np.int32), -best[0]


def test_viterbi_exhaustive_integer_scores(orc):
    rng = np.random.default_rng(10)
    for _ in range(400):
        K, N = 4, 3
        s1 = rng.integers(-3, 4, K).astype(np.float32)
        s = rng.integers(-3, 4, (N - 1, K, K)).astype(np.float32)
        want, _ = _best_paths_exhaustive(s1, s)
        np.testing.assert_array_equal(orc.viterbi(s1, s), want)


def test_viterbi_exhaustive_real_scores(orc):
    rng = np.random.default_rng(12)
    for _ in range(4):
        K, N = 16, 4
        s1 = rng.normal(0, 2, K).astype(np.float32)
        s = rng.normal(0, 2, (N - 1, K, K)).astype(np.float32)
        want, best = _best_paths_exhaustive(s1, s)
        got = orc.viterbi(s1, s)
        tot = float(s1[got[0]]) + sum(float(s[i - 1, got[i - 1], got[i]]) for i in range(1, N))
        assert abs(tot - best) < 1e-4
        np.testing.assert_array_equal(got, want)


def test_selector_zero_gate_is_per_slot_argmax(orc):
    rng = np.random.default_rng(13)
    B, N, V, R = 4, 7, 500, 16
    ci, cv, g, A, Bc, an = _selector_inputs(rng, B, N, V, R)
    cv = -np.sort(-cv, axis=2)                       # top-16 values arrive sorted
    cv[0, 2, 1] = cv[0, 2, 0]                        # a tie: the lower slot wins
    tokens, slot, q, st = orc.select(ci, cv, np.zeros_like(g), A, Bc, an,
                                     np.zeros(B, np.float32), 1, 0)
    np.testing.assert_array_equal(slot, 0)
    np.testing.assert_array_equal(tokens, ci[:, :, 0])
    np.testing.assert_array_equal(q[:, :, 0], 1.0)
    assert q.sum() == B * N and not st.any()


def _path_probs_fp64(s1, s, T):
    K, N = s1.shape[0], s.shape[0] + 1
    def sm(v):
        z = np.asarray(v, np.float64) / T
        z -= z.max()
        e = np.exp(z)
        return e / e.sum()
    probs = {}
    for path in itertools.product(range(K), repeat=N):
        p = sm(s1)[path[0]]
        for i in range(1, N):
            p *= sm(s[i - 1, path[i - 1]])[path[i]]
        probs[path] = p
    return probs


def test_walk_distribution_chi_square(orc):
    rng = np.random.default_rng(14)
    K, N, T = 4, 3, 0.7
    s1 = rng.normal(0, 1, K).astype(np.float32)
    s = rng.normal(0, 1, (N - 1, K, K)).astype(np.float32)
    probs = _path_probs_fp64(s1, s, T)
    assert abs(sum(probs.values()) - 1) < 1e-12
    M = 60_000
    u = (rng.integers(0, 2**24, (M, N)) * 2.0**-24).astype(np.float32)
    counts = {}
    invT = np.float32(1) / np.float32(T)
    for m in range(M):
        path, q = orc.walk(s1, s, float(invT), u[m])
        counts[tuple(path)] = counts.get(tuple(path), 0) + 1
        if m < 200:   # the returned q rows are the softmax of the row the walk stood on
            prev = None
            for i in range(N):
                row = s1 if i == 0 else s[i - 1, prev]
                z = row.astype(np.float64) / T
                e = np.exp(z - z.max())
                np.testing.assert_allclose(q[i], e / e.sum(), rtol=2e-6, atol=1e-7)
                prev = path[i]
    chi2 = sum((counts.get(p, 0) - M * pr) ** 2 / (M * pr) for p, pr in probs.items())
    assert chi2 < 103.4, chi2   # 63 degrees of freedom, alpha = 1e-3


def test_walk_inverse_cdf_edges(orc):
    s1 = np.array([0.0, -1e30, 0.0, 0.0], np.float32)   # slot 1 has a zero-weight candidate
    s = np.zeros((1, 4, 4), np.float32)
    path, q = orc.walk(s1, s, 1.0, np.array([0.0, 0.0], np.float32))
    assert path[0] == 0 and q[0, 1] == 0.0
    # u just below 1 picks the last candidate with weight
    path, _ = orc.walk(s1, s, 1.0, np.array([1 - 2**-24, 1 - 2**-24], np.float32))
    assert path[0] == 3 and path[1] == 3
    # a zero-weight first candidate is never chosen, even at u = 0
    s1z = np.array([-1e30, 0.0, 0.0, 0.0], np.float32)
    path, q = orc.walk(s1z, s, 1.0, np.array([0.0, 0.0], np.float32))
    assert path[0] == 1 and q[0, 0] == 0.0
    # inverse CDF: candidate k owns [C_{k-1}, C_k); four equal weights and u = 1/4 put
    # tau exactly on C_0, which belongs to candidate 1
    path, q = orc.walk(np.zeros(4, np.float32), s, 1.0, np.array([0.25, 0.75], np.float32))
    assert path[0] == 1 and path[1] == 3
    np.testing.assert_array_equal(q, 0.25)


def test_selector_rejects_nonfinite(orc):
    rng = np.random.default_rng(15)
    B, N, V, R = 3, 7, 400, 16
    ci, cv, g, A, Bc, an = _selector_inputs(rng, B, N, V, R)
    cv[1, 3, 5] = np.nan
    cv[2, 0, 0] = np.inf
    tokens, slot, q, st = orc.select(ci, cv, g, A, Bc, an, np.array([0, 0.5, 0], np.float32), 3, 1)
    assert st[0] == 0 and st[1] & orc.ST_NONFINITE and st[2] & orc.ST_NONFINITE
    assert np.all(tokens[1:] == -1) and np.all(slot[1:] == -1) and not q[1:].any()
    ci[0, 0, 0] = V   # out-of-range candidate
    _, _, _, st = orc.select(ci, cv, g, A, Bc, an, np.zeros(B, np.float32), 3, 1)
    assert st[0] & orc.ST_BADTOKEN


# ----------------------------------------------------------------------------------------
# Verify: lossless sampling (chi-square), special cases, greedy chain properties
# ----------------------------------------------------------------------------------------

def _verify_trials(orc, p_t, q_dist, M, seed, rng, N=1):
    """M independent single-proposal trials sharing one 16-token target row pair."""
    V = p_t.shape[-1]
    target = np.ascontiguousarray(np.broadcast_to(p_t, (N + 1, V)), dtype=np.float32)
    perm = rng.permutation(V).astype(np.int32)           # candidate order = a permutation
    cand_idx = np.ascontiguousarray(np.broadcast_to(perm, (M, N, 16)))
    qrow = q_dist[perm].astype(np.float32)
    q = np.ascontiguousarray(np.broadcast_to(qrow, (M, N, 16)))
    d = rng.choice(V, size=(M, N), p=q_dist / q_dist.sum()).astype(np.int32)
    inv = np.argsort(perm)
    slot = inv[d].astype(np.int32)
    n_acc, out, st = orc.verify(target, M, N, 0, V, V, d, cand_idx, q, slot,
                                np.ones(M, np.float32), seed, 0)
    return n_acc, out, st, d


def _chi2(counts, p, M):
    e = M * p
    m = e > 0
    assert counts[~m].sum() == 0
    return float(((counts[m] - e[m]) ** 2 / e[m]).sum())


@pytest.mark.parametrize("seed", [11, 12])
def test_verify_lossless_chi_square(orc, seed):
    rng = np.random.default_rng(seed)
    V, M = 16, 1_000_000
    p_t = rng.dirichlet(np.ones(V)).astype(np.float32)
    q_d = rng.dirichlet(np.ones(V)).astype(np.float32)
    n_acc, out, st, _ = _verify_trials(orc, p_t, q_d, M, seed, rng)
    assert not st.any()
    counts = np.bincount(out[:, 0], minlength=V)
    assert _chi2(counts, p_t.astype(np.float64), M) < 37.70     # 15 dof, alpha = 1e-3
    # the acceptance rate is sum_x min(p, q)
    want = np.minimum(p_t.astype(np.float64), q_d).sum()
    assert abs(n_acc.mean() - want) < 5 * np.sqrt(want * (1 - want) / M)


def _slotwise_trials(orc, rows, perms, qs, M, seed, rng):
    """M independent trials of one N-proposal block on a 16-token vocabulary. rows [N+1, V]
    are the target rows (row j-1 verifies proposal j, row N gives the bonus); slot j has its
    own candidate permutation perms[j] and its own draft distribution qs[j], and proposal j
    is drawn from qs[j]. Every trial shares the rows through a zero sequence stride."""
    N, V = qs.shape
    cand = np.ascontiguousarray(np.broadcast_to(perms, (M, N, 16))).astype(np.int32)
    qc = np.stack([qs[j][perms[j]] for j in range(N)]).astype(np.float32)
    q = np.ascontiguousarray(np.broadcast_to(qc, (M, N, 16)))
    d = np.stack([rng.choice(V, size=M, p=qs[j] / qs[j].sum()) for j in range(N)],
                 axis=1).astype(np.int32)
    slot = np.stack([np.argsort(perms[j])[d[:, j]] for j in range(N)], axis=1).astype(np.int32)
    n_acc, out, st = orc.verify(rows.astype(np.float32), M, N, 0, V, V, d, cand, q, slot,
                                np.ones(M, np.float32), seed, 0)
    return n_acc, out, st, (d, cand, q, slot)


@pytest.mark.parametrize("seed", [31, 32])
def test_verify_lossless_at_every_position(orc, seed):
    # "Geramy/LSE docs/DFLASH2.md", usage paragraph: the target checks every proposal of the
    # block by probability-ratio rejection and samples the residual on the first rejection.
    # Lossless means: for every block position k, the token the step emits there (the
    # accepted proposal k+1, the residual draw, or the bonus) follows target row k, over the
    # trials that reach position k (n_accept >= k). Each slot has its own target row, its own
    # candidate order and its own q, so a residual or an accept test that takes another
    # slot's candidates, q or row fails the chi-square at that position. The accept rate at
    # slot j+1, among trials that reach it, is sum_x min(p_j, q_{j+1}).
    rng = np.random.default_rng(seed)
    V, N, M = 16, 3, 1_000_000
    rows = rng.dirichlet(np.ones(V), N + 1)
    # q of slot j+1 leans on row j so that later positions are reached often
    qs = np.stack([0.5 * rows[j] + 0.5 * rng.dirichlet(np.ones(V)) for j in range(N)])
    perms = np.stack([rng.permutation(V) for _ in range(N)]).astype(np.int32)
    rows32 = rows.astype(np.float32)
    qs32 = qs.astype(np.float32)
    n_acc, out, st, _ = _slotwise_trials(orc, rows32, perms, qs32, M, seed, rng)
    assert not st.any()
    for k in range(N + 1):
        reach = n_acc >= k
        m = int(reach.sum())
        assert m > 100_000, (k, m)
        counts = np.bincount(out[reach, k], minlength=V)
        chi2 = _chi2(counts, rows32[k].astype(np.float64), m)
        assert chi2 < 37.70, (k, chi2)               # 15 dof, alpha = 1e-3
        if k < N:
            want = np.minimum(rows32[k].astype(np.float64), qs32[k]).sum()
            got = float((n_acc[reach] > k).mean())
            assert abs(got - want) < 5 * np.sqrt(want * (1 - want) / m), (k, got, want)


def test_verify_special_cases(orc):
    rng = np.random.default_rng(16)
    V, M = 16, 50_000
    p = rng.dirichlet(np.ones(V)).astype(np.float32)
    n_acc, out, st, d = _verify_trials(orc, p, p, M, 3, rng, N=3)
    assert np.all(n_acc == 3) and not st.any()
    np.testing.assert_array_equal(out[:, :3], d)
    # disjoint support: every proposal is rejected and the token follows p_t
    p2 = np.zeros(V, np.float32)
    p2[:8] = rng.dirichlet(np.ones(8))
    q2 = np.zeros(V, np.float32)
    q2[8:] = rng.dirichlet(np.ones(8))
    n_acc, out, st, _ = _verify_trials(orc, p2, q2, 200_000, 4, rng)
    assert np.all(n_acc == 0)
    assert _chi2(np.bincount(out[:, 0], minlength=V), p2.astype(np.float64), 200_000) < 37.70


def test_verify_bonus_comes_from_the_last_row(orc):
    # every proposal accepted (q = p_t); the bonus row differs from the others
    rng = np.random.default_rng(19)
    V, N, M = 16, 3, 2000
    p = rng.dirichlet(np.ones(V)).astype(np.float32)
    target = np.stack([p] * N + [np.eye(V, dtype=np.float32)[5]])
    perm = rng.permutation(V).astype(np.int32)
    ci = np.ascontiguousarray(np.broadcast_to(perm, (M, N, 16)))
    q = np.ascontiguousarray(np.broadcast_to(p[perm], (M, N, 16)))
    d = rng.choice(V, size=(M, N), p=p / p.sum()).astype(np.int32)
    slot = np.argsort(perm)[d].astype(np.int32)
    n_acc, out, st = orc.verify(target, M, N, 0, V, V, d, ci, q, slot, np.ones(M, np.float32), 9, 0)
    assert np.all(n_acc == N) and np.all(out[:, N] == 5) and not st.any()
    # greedy: the bonus is the last row's first element
    logits = rng.standard_normal((N + 1, V)).astype(np.float32)
    dg = logits[:N].argmax(axis=1)[None, :].astype(np.int32)
    n_acc, out, _ = orc.verify(logits, 1, N, 0, V, V, dg, ci[:1], q[:1], slot[:1],
                               np.zeros(1, np.float32), 9, 0)
    assert n_acc[0] == N and out[0, N] == logits[N].argmax()


def test_verify_zero_mass_and_bad_probabilities(orc):
    V, N = 32, 2
    target = np.zeros((1, N + 1, V), np.float32)
    ci = np.tile(np.arange(16, dtype=np.int32), (1, N, 1))
    q = np.full((1, N, 16), 1 / 16, np.float32)
    n_acc, out, st = orc.verify(target, 1, N, (N + 1) * V, V, V, np.array([[3, 4]], np.int32),
                                ci, q, np.array([[3, 4]], np.int32), np.ones(1, np.float32), 1, 0)
    assert n_acc[0] == 0 and out[0, 0] == 0 and st[0] & orc.ST_ZEROMASS
    target[0, 0, :] = 1 / V
    target[0, 0, 7] = -0.5
    _, _, st = orc.verify(target, 1, N, (N + 1) * V, V, V, np.array([[3, 4]], np.int32),
                          ci, q, np.array([[3, 4]], np.int32), np.ones(1, np.float32), 1, 0)
    assert st[0] & orc.ST_BADPROB


def test_verify_greedy_chain_properties(orc):
    rng = np.random.default_rng(17)
    B, N, V = 64, 7, 300
    rows = rng.standard_normal((B, N + 1, V)).astype(np.float32)
    am = rows.argmax(axis=2)
    d = rng.integers(0, V, (B, N)).astype(np.int32)
    # make a random-length prefix of each proposal chain match the target argmax
    for b in range(B):
        k = b % (N + 1)
        d[b, :k] = am[b, :k]
    n_acc, out, st = orc.verify(rows, B, N, (N + 1) * V, V, V, d, np.zeros((B, N, 16), np.int32),
                                np.zeros((B, N, 16), np.float32), np.zeros((B, N), np.int32),
                                np.zeros(B, np.float32), 0, 0)
    assert not st.any()
    for b in range(B):
        n = n_acc[b]
        np.testing.assert_array_equal(d[b, :n], am[b, :n])
        if n < N:
            assert d[b, n] != am[b, n]
        np.testing.assert_array_equal(out[b, :n], d[b, :n])
        assert out[b, n] == am[b, n]
        assert np.all(out[b, n + 1:] == -1)
    assert n_acc.max() == N


def test_verify_width_cap(orc):
    # Verifying only the first N_v < N proposals ("verify-width cap"): the same call with
    # N = N_v over the first N_v proposals and target rows 0..N_v of the full block.
    # Greedy, against the chain's definition written out: the accepted run is capped at N_v
    # and the token after it is the first argmax of row min(n, N_v).
    rng = np.random.default_rng(23)
    B, N, V = 48, 7, 200
    rows = rng.standard_normal((B, N + 1, V)).astype(np.float32)
    am = rows.argmax(axis=2)
    d = rng.integers(0, V, (B, N)).astype(np.int32)
    for b in range(B):
        d[b, :b % (N + 1)] = am[b, :b % (N + 1)]
    z16 = np.zeros((B, N, 16), np.int32)
    for nv in range(1, N):
        n_acc, out, st = orc.verify(rows, B, nv, (N + 1) * V, V, V, d[:, :nv].copy(),
                                    z16[:, :nv].copy(), z16[:, :nv].astype(np.float32),
                                    np.zeros((B, nv), np.int32), np.zeros(B, np.float32), 0, 0)
        assert not st.any() and out.shape == (B, nv + 1)
        for b in range(B):
            n = 0
            while n < nv and d[b, n] == am[b, n]:
                n += 1
            assert n_acc[b] == n
            np.testing.assert_array_equal(out[b, :n], d[b, :n])
            assert out[b, n] == am[b, n] and np.all(out[b, n + 1:] == -1)
    # Sampled: the uniforms are keyed by (step, sequence, row), so wherever the full-width
    # call stops before N_v the capped call gives the same result; where every one of the
    # N_v proposals is accepted, the token after them follows target row N_v.
    V, N, M = 16, 4, 40_000
    p = rng.dirichlet(np.ones(V)).astype(np.float32)
    r = rng.dirichlet(np.ones(V) * 0.5).astype(np.float32)
    for nv in (1, 2, 3):
        target = np.stack([p] * nv + [r] + [p] * (N - nv)).astype(np.float32)
        perm = rng.permutation(V).astype(np.int32)
        ci = np.ascontiguousarray(np.broadcast_to(perm, (M, N, 16)))
        qd = rng.dirichlet(np.ones(V)).astype(np.float32)
        q = np.ascontiguousarray(np.broadcast_to(qd[perm], (M, N, 16)))
        d = rng.choice(V, size=(M, N), p=qd / qd.sum()).astype(np.int32)
        slot = np.argsort(perm)[d].astype(np.int32)
        T = np.ones(M, np.float32)
        fn, fo, fs = orc.verify(target, M, N, 0, V, V, d, ci, q, slot, T, 77, 3)
        cn, co, cs = orc.verify(target, M, nv, 0, V, V, d[:, :nv].copy(), ci[:, :nv].copy(),
                                q[:, :nv].copy(), slot[:, :nv].copy(), T, 77, 3)
        assert not fs.any() and not cs.any()
        early = fn < nv
        np.testing.assert_array_equal(cn[early], fn[early])
        for b in np.nonzero(early)[0][:2000]:
            np.testing.assert_array_equal(co[b, :fn[b] + 1], fo[b, :fn[b] + 1])
        full = ~early
        assert np.all(cn[full] == nv)
        np.testing.assert_array_equal(co[full, :nv], d[full, :nv])
        k = int(full.sum())
        assert k > 2000
        assert _chi2(np.bincount(co[full, nv], minlength=V), r.astype(np.float64), k) < 37.70


def test_verify_one_hot_target_sampled_equals_greedy(orc):
    rng = np.random.default_rng(18)
    B, N, V = 32, 7, 64
    hot = rng.integers(0, V, (B, N + 1))
    target = np.zeros((B, N + 1, V), np.float32)
    np.put_along_axis(target, hot[..., None], 1.0, axis=2)
    ci = np.stack([np.stack([rng.permutation(V)[:16] for _ in range(N)]) for _ in range(B)]).astype(np.int32)
    slot = rng.integers(0, 16, (B, N)).astype(np.int32)
    for b in range(B):   # plant the target's choice in the draft for a prefix
        for j in range(b % (N + 1)):
            if hot[b, j] in ci[b, j]:
                slot[b, j] = int(np.where(ci[b, j] == hot[b, j])[0][0])
    d = np.take_along_axis(ci, slot[..., None], axis=2)[..., 0]
    q = rng.dirichlet(np.ones(16), (B, N)).astype(np.float32)
    g = orc.verify(target, B, N, (N + 1) * V, V, V, d, ci, q, slot, np.zeros(B, np.float32), 5, 0)
    s = orc.verify(target, B, N, (N + 1) * V, V, V, d, ci, q, slot, np.ones(B, np.float32), 5, 0)
    for a, b_ in zip(g, s):
        np.testing.assert_array_equal(a, b_)


# ----------------------------------------------------------------------------------------
# Printed live key counts ("Geramy/LSE docs/DFLASH2.md", native-test notes)
# ----------------------------------------------------------------------------------------

def _golden_rows(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append([int(x) for x in line.split()])
    return rows


def test_attention_live_counts_printed_on_the_pages(orc):
    # With zero queries every visible key gets the same weight 1/live. Value column 0 is 1
    # on block keys only, so the anchor's output there is P/live: the live count read back.
    for L, W, P, D, live in _golden_rows("lse_live_context_counts.txt"):
        S = max(W, 16)
        q = np.zeros((1, P, 1, D), np.float32)
        kb = np.zeros((1, P, 1, D), np.float32)
        kr = np.zeros((1, S, 1, D), np.float32)
        vb = np.zeros((1, P, 1, D), np.float32)
        vr = np.zeros((1, S, 1, D), np.float32)
        vb[..., 0] = 1.0
        out = orc.block_attn(q, kb, vb, kr, vr, np.array([L], np.int32), W)
        got = P / out[0, 0, 0, 0]
        assert abs(got - live) < 1e-9, (L, W, got, live)


# ----------------------------------------------------------------------------------------
# Output-head projection + top-16
# ----------------------------------------------------------------------------------------

def test_lmhead_logits_match_fsum_bruteforce(orc):
    # every logit against a correctly rounded sum (math.fsum) of the exact bf16 products,
    # computed element by element in plain Python; the absolute sums likewise
    import math
    rng = np.random.default_rng(81)
    M, C, V = 3, 128, 37
    h = to_bf16_bits(rng.standard_normal((M, C)).astype(np.float32) * 3)
    w = to_bf16_bits(rng.standard_normal((V, C)).astype(np.float32) / 8)
    L, A = orc.lmhead_logits(h, w, chunk=16)
    hf, wf = bf16_bits_to_f32(h).astype(float), bf16_bits_to_f32(w).astype(float)
    for m in range(M):
        for v in range(V):
            prods = [hf[m, c] * wf[v, c] for c in range(C)]
            exact = math.fsum(prods)
            assert abs(L[m, v] - exact) <= C * 2.0**-53 * math.fsum(abs(p) for p in prods)
            assert A[m, v] == pytest.approx(math.fsum(abs(p) for p in prods), rel=1e-14)


def test_lmhead_one_hot_head_selects_known_entries(orc):
    # weight row v = s_v * e_{c(v)}: logit[m, v] = s_v h[m, c(v)] exactly, so the top-16
    # is fixed by construction: rows planted with large products in a chosen order
    rng = np.random.default_rng(82)
    C, V, B, N = 256, 500, 2, 3
    hid = np.zeros((B, N + 1, C), np.float32)
    hid[:] = rng.uniform(-1, 1, size=hid.shape).astype(np.float32)
    col = rng.integers(0, C, size=V)
    scale = rng.choice([0.5, 0.25, -0.5], size=V).astype(np.float32)
    w = np.zeros((V, C), np.float32)
    w[np.arange(V), col] = scale
    chosen = rng.choice(V, size=16, replace=False)       # planted winners, best first
    for rank, v in enumerate(chosen):
        w[v] = 0
        w[v, 0] = 1.0
        w[v, 1] = float(64 - rank)                       # needs hid[., ., 1] = 1
    hid[:, :, 0] = 0.0
    hid[:, :, 1] = 1.0
    hb, wb = to_bf16_bits(hid), to_bf16_bits(w)
    idx, L, _ = orc.lmhead_topk16(hb, B, N, 1, (N + 1) * C, C, wb)
    for m in range(B * N):
        np.testing.assert_array_equal(idx.reshape(B * N, 16)[m], chosen)
        b, r = divmod(m, N)
        hv = bf16_bits_to_f32(hb[b, 1 + r]).astype(float)
        exact = bf16_bits_to_f32(wb).astype(float)[np.arange(V), col] * hv[col]
        exact[chosen] = [64 - k for k in range(16)]
        np.testing.assert_array_equal(L[m], exact)


def test_lmhead_topk_order_bruteforce_with_ties(orc):
    # small-integer data: the logits are exact integers with many ties; the top-16 must be
    # the first 16 of a plain Python sort by (-value, index)
    rng = np.random.default_rng(83)
    B, N, C, V = 2, 2, 64, 300
    hid = rng.integers(-2, 3, size=(B, N, C)).astype(np.float32)
    w = rng.integers(-1, 2, size=(V, C)).astype(np.float32)
    w[50] = w[7]                                          # duplicated rows tie exactly
    w[299] = w[7]
    idx, L, _ = orc.lmhead_topk16(to_bf16_bits(hid), B, N, 0, N * C, C, to_bf16_bits(w))
    for m in range(B * N):
        b, r = divmod(m, N)
        logits = [float(np.dot(hid[b, r].astype(np.int64), w[v].astype(np.int64))) for v in range(V)]
        want = sorted(range(V), key=lambda v: (-logits[v], v))[:16]
        np.testing.assert_array_equal(idx.reshape(-1, 16)[m], want)
        assert L[m].tolist() == logits


def test_lmhead_top16_order_specials(orc):
    x = np.array([1.0, np.nan, 3.0, -0.0, 0.0, 3.0, -np.inf, np.inf, np.nan] + [-5.0] * 10)
    np.testing.assert_array_equal(orc.top16_order_f64(x),
                                  [1, 8, 7, 2, 5, 0, 3, 4, 9, 10, 11, 12, 13, 14, 15, 16])


# ----------------------------------------------------------------------------------------
# Context-ring maintenance
# ----------------------------------------------------------------------------------------

def test_ring_update_against_an_ownership_model(orc):
    # An independent model keeps the committed sequence (content by position) and, per slot,
    # which position last wrote it. After every operation the ring must hold each position
    # of the next window that still owns its slot, and ST_RINGLOST must be set exactly when
    # a window position had lost its slot at the rewind.
    rng = np.random.default_rng(84)
    S, W, Pn = 12, 10, 4
    L = np.zeros(1, np.int32)
    kr = np.full((1, S, 1, 2), -1.0, np.float32)
    vr = kr.copy()
    hist = []                 # content id by position
    owner = [-1] * S          # position that last wrote each slot
    gen = 0
    for step in range(400):
        back = int(rng.choice([-1, 0, 0, 0, 1, 2, 3, 5, 40]))
        n = int(rng.integers(0, Pn + 1))
        gen += 1
        content = np.array([[[[gen * 100.0 + j, -gen * 100.0 - j]] for j in range(Pn)]], np.float32)
        # model
        Lb = len(hist)
        if back < 0:
            Lr, lost = 0, False
            owner = [-1] * S
        else:
            Lr = Lb - min(back, Lb)
            need = range(max(0, Lr - W + 1), Lr)
            lost = any(owner[p % S] != p for p in need)
        hist = hist[:Lr]
        for j in range(n):
            hist.append(gen * 100.0 + j)
            owner[(Lr + j) % S] = Lr + j
        # oracle
        L, kr, vr, st = orc.ring_update(content, -content, np.array([n], np.int32),
                                        np.array([back], np.int32), L, kr, vr, S, W)
        assert int(L[0]) == len(hist)
        assert bool(st[0] & orc.ST_RINGLOST) == lost, (step, back, Lb)
        for p in range(max(0, len(hist) - S), len(hist)):
            if owner[p % S] == p:
                assert kr[0, p % S, 0, 0] == hist[p] and vr[0, p % S, 0, 0] == -hist[p]


def test_ring_update_plain_appends_fill_slots_by_position(orc):
    # appends only: slot p mod S holds position p for the last S positions (closed form)
    S, W, Pn = 7, 5, 3
    L = np.array([0, 5], np.int32)
    kr = np.zeros((2, S, 1, 1), np.float32)
    vr = kr.copy()
    total = [0, 5]
    for step in range(20):
        n = np.array([step % (Pn + 1), (step * 2) % (Pn + 1)], np.int32)
        new = np.stack([np.arange(total[b], total[b] + Pn, dtype=np.float32).reshape(Pn, 1, 1)
                        for b in range(2)])
        L, kr, vr, st = orc.ring_update(new, new, n, np.zeros(2, np.int32), L, kr, vr, S, W)
        assert not st.any()
        for b in range(2):
            total[b] += int(n[b])
            assert int(L[b]) == total[b]
            for p in range(max(total[b] - S, 5 if b else 0), total[b]):
                assert kr[b, p % S, 0, 0] == p


def test_ring_update_counts_and_reset(orc):
    S, W, Pn = 8, 8, 4
    new = np.ones((3, Pn, 1, 1), np.float32)
    L, kr, vr, st = orc.ring_update(new, new, np.array([-1, 9, 2], np.int32),
                                    np.array([0, 0, -1], np.int32), np.array([5, 5, 100], np.int32),
                                    np.zeros((3, S, 1, 1), np.float32),
                                    np.zeros((3, S, 1, 1), np.float32), S, W)
    np.testing.assert_array_equal(L, [5, 9, 2])
    np.testing.assert_array_equal(st, [orc.ST_BADCOUNT, orc.ST_BADCOUNT, 0])


# ----------------------------------------------------------------------------------------
# Selector over affine-Q8 codebooks
# ----------------------------------------------------------------------------------------

def _exact_q8_rows(rng, V, R):
    """Q8 codebooks whose values are exact in bf16: per-group power-of-two scales, small
    integer-multiple biases and codes, with the equivalent bf16 rows built independently
    (binary64 arithmetic, then an exact conversion)."""
    G = R // 64
    # value = (code + k) * scale with code + k in [-32, 255]: 8 significant bits at most
    codes = rng.integers(0, 224, size=(V, R)).astype(np.uint8)
    sc = np.float32(2.0) ** rng.integers(-7, -4, size=(V, G)).astype(np.float32)
    bi = (rng.integers(-32, 33, size=(V, G)) * sc).astype(np.float32)
    vals = codes.astype(np.float64) * np.repeat(sc, 64, axis=1) + np.repeat(bi, 64, axis=1)
    bf = to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(bf).astype(np.float64), vals)  # exact
    return (codes, to_bf16_bits(sc), to_bf16_bits(bi)), bf


@pytest.mark.parametrize("T", [0.0, 0.8])
def test_select_q8_equals_bf16_select_on_exact_codebooks(orc, T):
    # with every dequantized value exact in bf16, the Q8 selector must reproduce the bf16
    # selector bit for bit (a wrong group, swapped scale/bias or a signed code would not)
    rng = np.random.default_rng(85)
    V, R, B, N = 500, 256, 3, 7
    pq, pb = _exact_q8_rows(rng, V, R)
    sq, sb = _exact_q8_rows(rng, V, R)
    ci = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                   for _ in range(B)]).astype(np.int32)
    cv = rng.standard_normal((B, N, 16)).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    an = rng.integers(0, V, size=B).astype(np.int32)
    temp = np.full(B, T, np.float32)
    a = orc.select_q8(ci, cv, g, pq, sq, an, temp, 5, 1, want_lattice=True)
    b = orc.select(ci, cv, g, pb, sb, an, temp, 5, 1, want_lattice=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_q8_quantizer_error_bound(orc):
    # the converter's convention (codes chosen against the stored bf16 scale and bias):
    # every dequantized value lies within half a step (plus the bias rounding) of the input
    rng = np.random.default_rng(86)
    from block_drafter_draft_amd.workloads import q8_quantize
    x = (rng.standard_normal((40, 256)) / 4).astype(np.float32)
    codes, sc, bi = q8_quantize(x)
    d = orc.q8_dequant(codes, sc, bi)
    s = np.repeat(bf16_bits_to_f32(sc), 64, axis=1)
    lo = np.repeat(np.abs(x.reshape(40, 4, 64)).max(axis=2), 64, axis=1)
    assert np.all(np.abs(d - x) <= 0.5 * s + lo * 2.0 ** -8 + 1e-7)


# ----------------------------------------------------------------------------------------
# log_c and the best-first draft tree
# ----------------------------------------------------------------------------------------

def test_log_c_accuracy(orc):
    # within 3 ulp of binary64 log over [1, 16] (the normaliser's range) and a wide sweep;
    # exactly 0 at 1, monotone on [1, 16]
    x = np.concatenate([np.linspace(1, 16, 200001), np.geomspace(1e-30, 1e30, 40001)]).astype(np.float32)
    got = orc.log_c_array(x).astype(np.float64)
    ref = np.log(x.astype(np.float64))
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 3 * np.maximum(ulp, 1e-45))
    assert orc.log_c(1.0) == 0.0
    seg = got[:200001]
    assert np.all(np.diff(seg) >= 0)


def _tree_inputs(rng, V=400, R=64, B=2, N=3):
    A = to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) / 4)
    Bc = to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) / 4)
    ci = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                   for _ in range(B)]).astype(np.int32)
    cv = (rng.standard_normal((B, N, 16)) * 1.5).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    an = rng.integers(0, V, size=B).astype(np.int32)
    return ci, cv, g, A, Bc, an


@pytest.mark.parametrize("budget", [1, 5, 17, 40])
def test_ddtree_is_the_top_budget_nodes(orc, budget):
    # Independent formulation: every node of the full tree (16 + 256 + 4096 at N = 3) with
    # its cumulative binary64 log-softmax score over the selector lattice; best-first with
    # a budget takes exactly the `budget` best nodes (scores only fall along a path), in
    # descending order, each with its own parent.
    rng = np.random.default_rng(87 + budget)
    ci, cv, g, A, Bc, an = _tree_inputs(rng)
    B, N = ci.shape[:2]
    par, dep, slt, tok, sc, st = orc.ddtree(ci, cv, g, A, Bc, an, budget)
    _, _, _, _, lat = orc.select(ci, cv, g, A, Bc, an, np.zeros(B, np.float32), 1, 0,
                                 want_lattice=True)
    for b in range(B):
        def ls(i, kp):   # binary64 log-softmax of lattice row kp of slot i
            row = lat[b, i - 1, kp].astype(np.float64)
            m = row.max()
            return row - m - np.log(np.exp(row - m).sum())
        nodes = []       # (score, path)
        frontier = [(0.0, ())]
        for i in range(1, N + 1):
            nxt = []
            for s0, path in frontier:
                kp = path[-1] if path else 0
                l = ls(i, kp)
                for k in range(16):
                    nxt.append((s0 + l[k], path + (k,)))
            nodes += nxt
            frontier = nxt
        nodes.sort(key=lambda z: -z[0])
        want = nodes[:budget]
        taken = {}
        for t in range(budget):
            path = want[t][1]
            assert dep[b, t] == len(path) and slt[b, t] == path[-1]
            assert par[b, t] == (taken[path[:-1]] if len(path) > 1 else -1)
            assert tok[b, t] == ci[b, len(path) - 1, path[-1]]
            assert abs(sc[b, t] - want[t][0]) < 1e-4
            taken[path] = t
    assert not st.any()


# ----------------------------------------------------------------------------------------
# Drafter projections: conv coefficients and the selector gate
# ----------------------------------------------------------------------------------------

def test_proj_addressing_with_one_hot_weights(orc):
    # every element of the (padded, strided) hidden buffer holds a distinct small integer
    # (exact in bf16); weight row o is s_o * e_{c(o)}, so y[b, r, o] must be exactly
    # s_o * buf[b*ss + (row0 + r)*rs + c(o)], each index computed here by hand
    rng = np.random.default_rng(91)
    B, N, row0, C, O = 3, 4, 2, 40, 29
    rs, ss = C + 8, (N + row0 + 1) * (C + 8) + 16
    buf = ((np.arange(B * ss) * 7) % 251 - 125).astype(np.float32)
    col = rng.integers(0, C, size=O)
    sc = rng.choice([1.0, -2.0, 0.5], size=O).astype(np.float32)
    w = np.zeros((O, C), np.float32)
    w[np.arange(O), col] = sc
    Y, A = orc.proj(to_bf16_bits(buf), B, N, row0, ss, rs, to_bf16_bits(w))
    assert Y.shape == (B, N, O)
    for b in range(B):
        for r in range(N):
            for o in range(O):
                want = float(sc[o]) * float(buf[b * ss + (row0 + r) * rs + int(col[o])])
                assert Y[b, r, o] == want and A[b, r, o] == abs(want)


def test_proj_matches_fsum_and_torch_linear(orc):
    # against a correctly rounded sum of the exact products (math.fsum), element by element,
    # and against torch's linear layer in binary64 (y = x W^T) on a non-square weight
    import math
    rng = np.random.default_rng(92)
    B, N, C, O = 2, 3, 72, 11
    h = to_bf16_bits(rng.standard_normal((B, N, C)).astype(np.float32) * 2)
    w = to_bf16_bits(rng.standard_normal((O, C)).astype(np.float32) / 4)
    Y, A = orc.proj(h.reshape(-1), B, N, 0, N * C, C, w)
    hf, wf = bf16_bits_to_f32(h).astype(float), bf16_bits_to_f32(w).astype(float)
    for b in range(B):
        for r in range(N):
            for o in range(O):
                prods = [hf[b, r, c] * wf[o, c] for c in range(C)]
                assert abs(Y[b, r, o] - math.fsum(prods)) <= C * 2.0**-53 * A[b, r, o]
    ref = torch.nn.functional.linear(torch.from_numpy(hf), torch.from_numpy(wf)).numpy()
    np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-12)


def test_conv_coeffs_layout(orc):
    # one projection of the sublayer input gives both convs' coefficients: weight row
    # (2 s + t) G + g is a one-hot on column c(s, t, g), so delta_s[b, i, t, g] must be
    # x[b, i, c(s, t, g)] exactly (s = 0: the conv before the sublayer, s = 1: after)
    rng = np.random.default_rng(93)
    B, P, C, G = 2, 8, 64, 4
    x = ((np.arange(B * P * C).reshape(B, P, C) * 5) % 199 - 99).astype(np.float32)
    col = rng.integers(0, C, size=(2, 2, G))
    w = np.zeros((4 * G, C), np.float32)
    for s, t, g in itertools.product(range(2), range(2), range(G)):
        w[(2 * s + t) * G + g, col[s, t, g]] = 1.0
    d_in, d_out = orc.conv_coeffs(to_bf16_bits(x), to_bf16_bits(w), G)
    assert d_in.shape == (B, P, 2, G) and d_in.dtype == np.float32
    for s, d in enumerate((d_in, d_out)):
        for b, i, t, g in itertools.product(range(B), range(P), range(2), range(G)):
            assert d[b, i, t, g] == x[b, i, col[s, t, g]]


def test_selector_gate_takes_slots_one_to_n(orc):
    # the gate of slot i comes from slot i's hidden row: rows are made distinct by a
    # constant per (b, slot) in column 0 and the weight reads only column 0
    B, P, C, R = 2, 8, 32, 16
    h = np.zeros((B, P, C), np.float32)
    for b in range(B):
        for i in range(P):
            h[b, i, 0] = 10 * b + i
    w = np.zeros((R, C), np.float32)
    w[:, 0] = np.arange(1, R + 1)
    g = orc.selector_gate(to_bf16_bits(h), to_bf16_bits(w))
    assert g.shape == (B, P - 1, R) and g.dtype == np.float32
    for b in range(B):
        for i in range(1, P):
            np.testing.assert_array_equal(g[b, i - 1], (10 * b + i) * np.arange(1, R + 1))


def _best_path_full_width(s1, s):
    """Brute force over all K^N paths (N = 7, K = 16: 268,435,456 of them): every path's
    score summed left to right in binary32 (the order the max-sum recursion adds in), the
    three-slot prefixes enumerated in a loop and the four-slot suffixes vectorised. s[i] is
    the transition from slot i + 1 to slot i + 2. Returns the best path, its score and the
    runner-up score."""
    K = s1.shape[0]
    f = np.float32
    a4, a5, a6, a7 = (a.ravel() for a in np.meshgrid(np.arange(K), np.arange(K), np.arange(K),
                                                      np.arange(K), indexing="ij"))
    t34 = s[2][:, a4]                                  # [K (k3), K^4]
    t45, t56, t67 = s[3][a4, a5], s[4][a5, a6], s[5][a6, a7]
    best, second, arg = -np.inf, -np.inf, None
    for k1 in range(K):
        for k2 in range(K):
            p2 = f(f(s1[k1]) + f(s[0][k1, k2]))
            for k3 in range(K):
                t = (f(p2 + s[1][k2, k3]) + t34[k3]).astype(f)
                t = (t + t45).astype(f)
                t = (t + t56).astype(f)
                t = (t + t67).astype(f)
                i = int(np.argmax(t))
                m = float(t[i])
                if m > best:
                    second = max(best, float(np.partition(t, -2)[-2]))
                    best = m
                    arg = (k1, k2, k3, int(a4[i]), int(a5[i]), int(a6[i]), int(a7[i]))
                else:
                    second = max(second, m)
    return np.array(arg, dtype=np.int32), best, second


@pytest.mark.parametrize("seed", [31, 32])
def test_viterbi_exhaustive_full_width(orc, seed):
    # the drafter's full shape, N = 7 slots of K = 16 candidates: the recursion's path must
    # be the path with the largest binary32 score among all 16^7 (real-valued scores, so
    # the maximum is unique; the test checks that it is)
    rng = np.random.default_rng(seed)
    K, N = 16, 7
    s1 = rng.normal(0, 2, K).astype(np.float32)
    s = rng.normal(0, 2, (N - 1, K, K)).astype(np.float32)
    want, best, second = _best_path_full_width(s1, s)
    assert best > second, "the maximum is not unique for this seed"
    np.testing.assert_array_equal(orc.viterbi(s1, s), want)
