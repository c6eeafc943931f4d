"""dflash2_ring_update against the oracle: bit-exact rings, context lengths and status, over
random sequences of rewinds, resets and appends; then block attention over the updated
rings against the oracle's attention over the oracle's rings."""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import assert_close_tol, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def _bits(x, bf16):
    return wl.to_bf16_bits(x) if bf16 else x.astype(np.float32)


@pytest.mark.parametrize("bf16", [True, False])
def test_ring_update_random_operations(d2, bf16):
    rng = np.random.default_rng(95 + bf16)
    B, Pn, Hkv, D, S, W = 6, 8, 8, 128, 64, 64
    L = rng.integers(0, 200, size=B).astype(np.int32)
    kr = _bits(rng.standard_normal((B, S, Hkv, D)).astype(np.float32), bf16)
    vr = _bits(rng.standard_normal((B, S, Hkv, D)).astype(np.float32), bf16)
    st = np.zeros(B, np.int32)
    dL, dk, dv, ds = to_dev(L), to_dev(kr), to_dev(vr), to_dev(st)
    for step in range(24):
        new_k = _bits(rng.standard_normal((B, Pn, Hkv, D)).astype(np.float32), bf16)
        new_v = _bits(rng.standard_normal((B, Pn, Hkv, D)).astype(np.float32), bf16)
        n_new = rng.integers(0, Pn + 1, size=B).astype(np.int32)
        back = rng.choice([-1, 0, 0, 0, 1, 3, 7, 70], size=B).astype(np.int32)
        if step % 5 == 4:
            n_new[0] = Pn + 3          # clamped, flagged
            n_new[1] = -2
        say(f"ring_update step {step} bf16={bf16} n_new={n_new.tolist()} back={back.tolist()}")
        d2.ring_update(to_dev(new_k), to_dev(new_v), to_dev(n_new), to_dev(back), dL, dk, dv, W, ds)
        torch.cuda.synchronize()
        L, kr, vr, st = orc.ring_update(new_k, new_v, n_new, back, L, kr, vr, S, W, status=st)
        np.testing.assert_array_equal(to_host(dL), L, err_msg=f"ctx_len step {step}")
        np.testing.assert_array_equal(to_host(ds), st, err_msg=f"status step {step}")
        np.testing.assert_array_equal(to_host(dk), kr, err_msg=f"k_ring step {step}")
        np.testing.assert_array_equal(to_host(dv), vr, err_msg=f"v_ring step {step}")
    assert (st & orc.ST_RINGLOST).any() and (st & orc.ST_BADCOUNT).any()


def test_ring_update_then_attention(d2):
    # the rings a few commits leave behind are read by block attention exactly as the
    # oracle's attention reads the oracle's rings
    rng = np.random.default_rng(97)
    B, P, Hq, Hkv, D, S, W = 4, 8, 32, 8, 128, 2048, 2048
    L = np.array([0, 100, 2040, 5000], np.int32)
    kr = wl.to_bf16_bits(rng.standard_normal((B, S, Hkv, D)).astype(np.float32))
    vr = wl.to_bf16_bits(rng.standard_normal((B, S, Hkv, D)).astype(np.float32))
    dL, dk, dv = to_dev(L), to_dev(kr), to_dev(vr)
    st = np.zeros(B, np.int32)
    ds = to_dev(st)
    for step in range(3):
        nk = wl.to_bf16_bits(rng.standard_normal((B, P, Hkv, D)).astype(np.float32))
        nv = wl.to_bf16_bits(rng.standard_normal((B, P, Hkv, D)).astype(np.float32))
        n_new = np.array([8, 3, 5, 1], np.int32)
        back = np.array([0, 1, 0, 2], np.int32)
        d2.ring_update(to_dev(nk), to_dev(nv), to_dev(n_new), to_dev(back), dL, dk, dv, W, ds)
        L, kr, vr, st = orc.ring_update(nk, nv, n_new, back, L, kr, vr, S, W, status=st)
    torch.cuda.synchronize()
    q = wl.to_bf16_bits(rng.standard_normal((B, P, Hq, D)).astype(np.float32))
    kb = wl.to_bf16_bits(rng.standard_normal((B, P, Hkv, D)).astype(np.float32))
    vb = wl.to_bf16_bits(rng.standard_normal((B, P, Hkv, D)).astype(np.float32))
    say("block_attn over updated rings")
    out = d2.block_attn(to_dev(q), to_dev(kb), to_dev(vb), dk, dv, dL, W)
    torch.cuda.synchronize()
    ref = orc.block_attn(q, kb, vb, kr, vr, L, W)
    assert_close_tol(to_host(out), ref, what="attention after ring updates", max_abs=2e-2,
                     rel_l2=1e-2)
