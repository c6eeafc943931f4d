"""dflash2_block_attn and dflash2_dynconv2 against the binary64 oracle, within tolerance.

Tolerances: bf16 results within max-abs 2e-2 and rel-L2 1e-2 of the oracle; f32 results
within 1e-4 (attention: softmax in binary32 over at most a few thousand keys) and 1e-5
(conv: two products and one sum, each rounded once).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import assert_close_tol, poison_like, say, to_dev, to_host

pytestmark = pytest.mark.gpu

BF16_TOL = dict(max_abs=2e-2, rel_l2=1e-2)
F32_ATTN_TOL = dict(max_abs=1e-4, rel_l2=1e-5)


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def run_attn(d2, q, kb, vb, kr, vr, L, W, what, scale=None):
    B, P, Hq, D = q.shape
    say(f"block_attn {what} B={B} P={P} Hq={Hq} Hkv={kr.shape[2]} D={D} S={kr.shape[1]} W={W} L={list(L)[:4]}")
    out = poison_like(q.shape, torch.bfloat16 if q.dtype == np.uint16 else torch.float32)
    d2.block_attn(to_dev(q), to_dev(kb), to_dev(vb), to_dev(kr), to_dev(vr),
                  to_dev(np.asarray(L, np.int32)), W, scale=scale, out=out)
    torch.cuda.synchronize()
    got = to_host(out)
    ref = orc.block_attn(q, kb, vb, kr, vr, np.asarray(L, np.int32), W, scale=scale)
    tol = BF16_TOL if q.dtype == np.uint16 else F32_ATTN_TOL
    return assert_close_tol(got, ref, what=what, **tol)


def _rand_attn(rng, B, P, Hq, Hkv, D, S, bf16=True):
    def mk(*shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return wl.to_bf16_bits(x) if bf16 else x
    return mk(B, P, Hq, D), mk(B, P, Hkv, D), mk(B, P, Hkv, D), mk(B, S, Hkv, D), mk(B, S, Hkv, D)


def test_attn_tiny_config_f32(d2):
    cfg = wl.CONFIGS[1]
    q = wl.attn_q(cfg, 0)
    kb, vb = wl.attn_block_kv(cfg, 0)
    kr, vr = wl.attn_ring(cfg, 0)
    run_attn(d2, q, kb, vb, kr, vr, wl.ctx_len(cfg), cfg.W, "config 1")


def test_attn_drafter_geometry_b1(d2):
    cfg = wl.CONFIGS[2]
    for layer in (0, 4):
        q = wl.attn_q(cfg, layer)
        kb, vb = wl.attn_block_kv(cfg, layer)
        kr, vr = wl.attn_ring(cfg, layer)
        run_attn(d2, q, kb, vb, kr, vr, wl.ctx_len(cfg), cfg.W, f"config 2 layer {layer}")


def test_attn_varied_contexts(d2):
    # per-sequence contexts: partly empty windows, ring wrap, live counts 17 and 2055
    rng = np.random.default_rng(51)
    L = [0, 9, 512, 2047, 2048, 3000, 8192, 131071]
    q, kb, vb, kr, vr = _rand_attn(rng, len(L), 8, 32, 8, 128, 2048)
    run_attn(d2, q, kb, vb, kr, vr, L, 2048, "varied contexts")


@pytest.mark.parametrize("P,Hq,Hkv,D,S,W", [(8, 32, 8, 64, 300, 200), (16, 2, 1, 128, 64, 33),
                                           (8, 8, 8, 128, 40, 40), (3, 5, 1, 64, 100, 1),
                                           (2, 16, 2, 128, 17, 18), (8, 24, 8, 128, 2048, 2048),
                                           (8, 32, 8, 128, 511, 512), (4, 32, 8, 128, 1000, 1000)])
def test_attn_shapes(d2, P, Hq, Hkv, D, S, W):
    rng = np.random.default_rng(P * 131 + Hq * 7 + D + S + W)
    L = [0, 1, W - 2 if W > 2 else 0, W + 5, 3 * S + 7]
    q, kb, vb, kr, vr = _rand_attn(rng, len(L), P, Hq, Hkv, D, S)
    run_attn(d2, q, kb, vb, kr, vr, L, W, f"shape P{P} Hq{Hq} Hkv{Hkv} D{D} S{S} W{W}")


@pytest.mark.parametrize("B,P,Hq,Hkv,S,W", [(36, 8, 32, 8, 2048, 2048), (20, 5, 32, 16, 700, 600)])
def test_attn_large_batch_two_wave_workgroups(d2, B, P, Hq, Hkv, S, W):
    # more (sequence, KV head) pairs than compute units: the streaming kernel runs
    # workgroups of two waves, two per unit; contexts cover empty, short, ragged-tile,
    # wrapped-ring and full windows
    rng = np.random.default_rng(B * 17 + Hkv)
    base = [0, 1, 9, 31, 33, W - 2, W - 1, W, W + 5, 3 * S + 7, 131071]
    L = [base[i % len(base)] for i in range(B)]
    q, kb, vb, kr, vr = _rand_attn(rng, B, P, Hq, Hkv, 128, S)
    run_attn(d2, q, kb, vb, kr, vr, L, W, f"two-wave workgroups B{B} Hkv{Hkv}")


def test_attn_f32_shapes(d2):
    rng = np.random.default_rng(52)
    L = [0, 10, 100]
    q, kb, vb, kr, vr = _rand_attn(rng, 3, 8, 8, 1, 128, 96, bf16=False)
    run_attn(d2, q, kb, vb, kr, vr, L, 64, "f32 D128")
    # several 64-key tiles (307 keys, ragged), two KV heads, ring wrap-around
    rng = np.random.default_rng(53)
    q, kb, vb, kr, vr = _rand_attn(rng, 2, 8, 8, 2, 64, 512, bf16=False)
    run_attn(d2, q, kb, vb, kr, vr, [500, 900], 300, "f32 five tiles")


def test_attn_scale_and_large_values(d2):
    rng = np.random.default_rng(53)
    q, kb, vb, kr, vr = _rand_attn(rng, 2, 8, 32, 8, 128, 2048)
    run_attn(d2, q, kb, vb, kr, vr, [2500, 700], 2048, "scale 0.3", scale=0.3)
    q4 = wl.to_bf16_bits(wl.bf16_bits_to_f32(q) * 4)
    run_attn(d2, q4, kb, vb, kr, vr, [2500, 700], 2048, "peaked softmax")


def test_attn_serving_batch_sampled(d2):
    cfg = wl.CONFIGS[5]
    say("block_attn config 5 full batch (oracle on 3 sequences)")
    q = wl.attn_q(cfg, 2)
    kb, vb = wl.attn_block_kv(cfg, 2)
    kr, vr = wl.attn_ring(cfg, 2)
    L = wl.ctx_len(cfg)
    out = poison_like(q.shape, torch.bfloat16)
    d2.block_attn(to_dev(q), to_dev(kb), to_dev(vb), to_dev(kr), to_dev(vr), to_dev(L), cfg.W,
                  out=out)
    torch.cuda.synchronize()
    got = to_host(out)
    for b in (0, 31, 63):
        ref = orc.block_attn(q[b:b + 1], kb[b:b + 1], vb[b:b + 1], kr[b:b + 1], vr[b:b + 1],
                             L[b:b + 1], cfg.W)
        assert_close_tol(got[b:b + 1], ref, what=f"config 5 seq {b}", **BF16_TOL)


def test_attn_deterministic(d2):
    rng = np.random.default_rng(54)
    q, kb, vb, kr, vr = _rand_attn(rng, 4, 8, 32, 8, 128, 2048)
    L = to_dev(np.array([100, 2047, 4000, 9000], np.int32))
    args = [to_dev(a) for a in (q, kb, vb, kr, vr)]
    a = to_host(d2.block_attn(*args, L, 2048))
    b = to_host(d2.block_attn(*args, L, 2048))
    np.testing.assert_array_equal(a, b)


def test_attn_workspace_reuse(d2):
    # one workspace (filled with 0xFF first) for several calls of different contexts
    rng = np.random.default_rng(55)
    B, P, Hq, Hkv, D, S, W = 2, 8, 32, 8, 128, 2048, 2048
    need = d2.block_attn_workspace_bytes(B, P, Hq, Hkv, D, S, W, d2.BF16)
    assert need > 0
    ws = d2.workspace(need, "cuda:0")
    ws.fill_(0xFF)
    for call, L in enumerate(([3000, 17], [2047, 0], [5, 9000])):
        q, kb, vb, kr, vr = _rand_attn(rng, B, P, Hq, Hkv, D, S)
        say(f"block_attn workspace reuse call {call} L={L}")
        out = poison_like(q.shape, torch.bfloat16)
        d2.block_attn(to_dev(q), to_dev(kb), to_dev(vb), to_dev(kr), to_dev(vr),
                      to_dev(np.asarray(L, np.int32)), W, out=out, ws=ws)
        torch.cuda.synchronize()
        ref = orc.block_attn(q, kb, vb, kr, vr, np.asarray(L, np.int32), W)
        assert_close_tol(to_host(out), ref, what=f"reuse call {call}", **BF16_TOL)


# ------------------------------------------------------------------------------------------
# dynconv2
# ------------------------------------------------------------------------------------------

def run_conv(d2, x, base, delta, what, tol):
    B, P, C = x.shape
    say(f"dynconv2 {what} B={B} P={P} C={C}")
    out = poison_like(x.shape, torch.bfloat16 if x.dtype == np.uint16 else torch.float32)
    d2.dynconv2(to_dev(x), to_dev(base), to_dev(delta), out=out)
    torch.cuda.synchronize()
    got = to_host(out)
    ref = orc.dynconv2(x, base, delta)
    assert_close_tol(got, ref, what=what, **tol)
    return got


def test_conv_tiny_config_f32(d2):
    cfg = wl.CONFIGS[1]
    for site in range(cfg.sites):
        x, base, delta = wl.conv_inputs(cfg, site)
        run_conv(d2, x, base, delta, f"config 1 site {site}", dict(max_abs=1e-5, rel_l2=1e-6))


@pytest.mark.parametrize("cfgno", [2, 5])
def test_conv_drafter_width(d2, cfgno):
    cfg = wl.CONFIGS[cfgno]
    x, base, delta = wl.conv_inputs(cfg, 7)
    run_conv(d2, x, base, delta, f"config {cfgno}", BF16_TOL)


def test_conv_identity_is_exact(d2):
    rng = np.random.default_rng(55)
    B, P, C = 3, 8, 5120
    x = wl.to_bf16_bits(rng.standard_normal((B, P, C)).astype(np.float32))
    base = np.stack([np.ones(C), np.zeros(C)]).astype(np.float32)
    delta = np.zeros((B, P, 2, C // 16), np.float32)
    got = run_conv(d2, x, base, delta, "identity", BF16_TOL)
    np.testing.assert_array_equal(got, x)


@pytest.mark.parametrize("P,C", [(1, 16), (2, 48), (16, 256)])
def test_conv_shapes(d2, P, C):
    rng = np.random.default_rng(56 + P + C)
    B = 5
    x = rng.standard_normal((B, P, C)).astype(np.float32)
    base = rng.uniform(-1, 1, (2, C)).astype(np.float32)
    delta = rng.uniform(-1, 1, (B, P, 2, C // 16)).astype(np.float32)
    run_conv(d2, x, base, delta, f"f32 P{P} C{C}", dict(max_abs=1e-5, rel_l2=1e-6))
    run_conv(d2, wl.to_bf16_bits(x), base, delta, f"bf16 P{P} C{C}", BF16_TOL)


@pytest.mark.parametrize("B,P,C", [(40, 16, 4096), (128, 3, 1024), (26, 8, 5120), (33, 1, 4000),
                                   (300, 1, 528)])
def test_conv_large_batches(d2, B, P, C):
    # large batches (P up to 16, f32 and bf16, a ragged channel count): the same bounds,
    # and identity taps reproduce the input exactly. From 256 rows a thread takes two
    # positions: odd P and P = 1 leave the last pair half empty.
    rng = np.random.default_rng(90 + B + P)
    x = rng.standard_normal((B, P, C)).astype(np.float32)
    base = rng.uniform(-1, 1, (2, C)).astype(np.float32)
    delta = rng.uniform(-1, 1, (B, P, 2, C // 16)).astype(np.float32)
    run_conv(d2, x, base, delta, f"f32 large batch B{B} P{P} C{C}", dict(max_abs=1e-5, rel_l2=1e-6))
    xb = wl.to_bf16_bits(x)
    run_conv(d2, xb, base, delta, f"bf16 large batch B{B} P{P} C{C}", BF16_TOL)
    ident = np.stack([np.ones(C), np.zeros(C)]).astype(np.float32)
    got = run_conv(d2, xb, ident, np.zeros_like(delta), f"identity large batch B{B}", BF16_TOL)
    np.testing.assert_array_equal(got, xb)
