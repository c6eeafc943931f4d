"""Every step entry point at the largest batch it accepts, with short rows so that the oracle
finishes in seconds: 65535 (sequence, position) rows for the conv and the top-16, 65535
sequences for select, verify and block attention. Attention is compared on sampled
sequences, each computed by the oracle on its own (sequences are independent); the others
are compared in full. Integer results bit for bit, floating results to the usual bounds."""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import assert_close_tol, assert_same_floats, poison_like, say, to_dev, to_host

pytestmark = pytest.mark.gpu

BF16_TOL = dict(max_abs=2e-2, rel_l2=1e-2)
MAX_ROWS = 65535


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def _cands(rng, B, N, V):
    """16 distinct indices per (sequence, slot): the first 16 of a random permutation."""
    perm = rng.permuted(np.tile(np.arange(V, dtype=np.int32), (B * N, 1)), axis=1)
    return np.ascontiguousarray(perm[:, :16]).reshape(B, N, 16)


def test_conv_at_the_row_limit(d2):
    B, P, C = 4369, 15, 48                      # B * P = 65535 rows
    assert B * P == MAX_ROWS
    rng = np.random.default_rng(501)
    x = rng.standard_normal((B, P, C)).astype(np.float32)
    base = rng.uniform(-1, 1, (2, C)).astype(np.float32)
    delta = rng.uniform(-1, 1, (B, P, 2, C // 16)).astype(np.float32)
    say(f"dynconv2 at the row limit B={B} P={P} C={C}")
    for xin, tol in ((x, dict(max_abs=1e-5, rel_l2=1e-6)), (wl.to_bf16_bits(x), BF16_TOL)):
        out = poison_like(xin.shape, torch.bfloat16 if xin.dtype == np.uint16 else torch.float32)
        d2.dynconv2(to_dev(xin), to_dev(base), to_dev(delta), out=out)
        torch.cuda.synchronize()
        assert_close_tol(to_host(out), orc.dynconv2(xin, base, delta), what="conv limit", **tol)
    with pytest.raises(d2.DFlash2Error):        # one row more is refused
        d2.dynconv2(to_dev(np.zeros((MAX_ROWS + 1, 1, 16), np.float32)),
                    to_dev(np.zeros((2, 16), np.float32)),
                    to_dev(np.zeros((MAX_ROWS + 1, 1, 2, 1), np.float32)))


def test_topk16_at_the_row_limit(d2):
    B, N, V = 4369, 15, 40                      # B * N = 65535 rows of a 16-position block
    P = N + 1
    rng = np.random.default_rng(502)
    # coarse values force many ties, which the total order breaks by index
    x = wl.to_bf16_bits(rng.integers(-6, 7, (B, P, V)).astype(np.float32) * np.float32(0.5))
    say(f"topk16 at the row limit B={B} N={N} V={V}")
    idx, val = d2.topk16(to_dev(x), B, N, 1, P * V, V, V)
    torch.cuda.synchronize()
    oi, ov = orc.topk16(x.reshape(-1), B, N, 1, P * V, V, V)
    np.testing.assert_array_equal(to_host(idx), oi)
    assert_same_floats(to_host(val), ov, "top-16 values")


def test_select_at_the_batch_limit(d2):
    B, N, V, R = MAX_ROWS, 2, 96, 8
    rng = np.random.default_rng(503)
    ci = _cands(rng, B, N, V)
    cv = rng.standard_normal((B, N, 16)).astype(np.float32)
    g = rng.standard_normal((B, N, R)).astype(np.float32)
    A = wl.to_bf16_bits(rng.normal(0, 0.5, (V, R)).astype(np.float32))
    Bc = wl.to_bf16_bits(rng.normal(0, 0.5, (V, R)).astype(np.float32))
    an = rng.integers(0, V, B).astype(np.int32)
    temp = np.where(np.arange(B) % 3 == 0, 0.0, 0.8).astype(np.float32)
    say(f"select at the batch limit B={B} N={N} V={V} R={R}")
    tok = poison_like((B, N), torch.int32)
    sl = poison_like((B, N), torch.int32)
    q = poison_like((B, N, 16), torch.float32)
    st = poison_like((B,), torch.int32)
    d2.select(to_dev(ci), to_dev(cv), to_dev(g), to_dev(A), to_dev(Bc), to_dev(an), to_dev(temp),
              17, 4, tokens=tok, slot=sl, q=q, status=st)
    torch.cuda.synchronize()
    o = orc.select(ci, cv, g, A, Bc, an, temp, 17, 4)
    np.testing.assert_array_equal(to_host(tok), o[0], err_msg="tokens")
    np.testing.assert_array_equal(to_host(sl), o[1], err_msg="slot")
    assert_same_floats(to_host(q), o[2], "q")
    np.testing.assert_array_equal(to_host(st), o[3], err_msg="status")


def test_verify_at_the_batch_limit(d2):
    B, N, V = MAX_ROWS, 2, 24
    rng = np.random.default_rng(504)
    logits = rng.standard_normal((B, N + 1, V)).astype(np.float32)
    z = np.exp(logits - logits.max(axis=-1, keepdims=True))
    p_t = (z / z.sum(axis=-1, keepdims=True)).astype(np.float32)
    ci = _cands(rng, B, N, V)
    q = rng.dirichlet(np.ones(16), (B, N)).astype(np.float32)
    slot = rng.integers(0, 16, (B, N)).astype(np.int32)
    tok = np.take_along_axis(ci, slot[..., None], axis=2)[..., 0].astype(np.int32)
    temp = np.where(np.arange(B) % 2 == 0, 0.0, 1.0).astype(np.float32)
    say(f"verify at the batch limit B={B} N={N} V={V}")
    st = torch.zeros(B, dtype=torch.int32, device="cuda")
    n_acc = poison_like((B,), torch.int32)
    out = poison_like((B, N + 1), torch.int32)
    d2.verify(to_dev(p_t.reshape(-1)), B, N, (N + 1) * V, V, V, to_dev(tok), to_dev(ci), to_dev(q),
              to_dev(slot), to_dev(temp), 23, 2, st, n_accept=n_acc, out_tokens=out)
    torch.cuda.synchronize()
    o = orc.verify(p_t.reshape(-1), B, N, (N + 1) * V, V, V, tok, ci, q, slot, temp, 23, 2)
    for a, b_, name in zip((to_host(n_acc), to_host(out), to_host(st)), o,
                           ("n_accept", "out_tokens", "status")):
        np.testing.assert_array_equal(a, b_, err_msg=name)
    assert 0 < to_host(n_acc).mean() < N


def test_block_attn_at_the_batch_limit(d2):
    # 65535 sequences of the streaming (D = 128) kernel, P = 2, one KV head and two query
    # heads, a 40-key window over a 48-row ring; ring contents come from a pool of 97
    # distinct sequences, context lengths vary per sequence (empty, short, wrapped)
    B, P, Hq, Hkv, D, S, W = MAX_ROWS, 2, 2, 1, 128, 48, 40
    rng = np.random.default_rng(505)
    pool = 97

    def mk(*shape):
        return wl.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    kr_p, vr_p = mk(pool, S, Hkv, D), mk(pool, S, Hkv, D)
    sel_pool = np.arange(B) % pool
    kr, vr = kr_p[sel_pool], vr_p[sel_pool]
    q, kb, vb = mk(B, P, Hq, D), mk(B, P, Hkv, D), mk(B, P, Hkv, D)
    L = rng.integers(0, 200, B).astype(np.int32)
    L[:4] = [0, 1, 39, 47]
    say(f"block_attn at the batch limit B={B} P={P} Hq={Hq} Hkv={Hkv} D={D} S={S} W={W}")
    out = poison_like(q.shape, torch.bfloat16)
    d2.block_attn(to_dev(q), to_dev(kb), to_dev(vb), to_dev(kr), to_dev(vr), to_dev(L), W, out=out)
    torch.cuda.synchronize()
    got = to_host(out)
    pick = np.unique(np.concatenate([np.arange(4), [B // 2, B - 2, B - 1],
                                     rng.choice(B, 249, replace=False)]))
    ref = orc.block_attn(q[pick], kb[pick], vb[pick], kr[pick], vr[pick], L[pick], W)
    assert_close_tol(got[pick], ref, what="attention at the batch limit", **BF16_TOL)
