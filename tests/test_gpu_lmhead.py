"""dflash2_lmhead_topk16 against the binary64 oracle.

The GPU sums binary32 products in its own order, so each logit may differ from the exact
one by up to gamma * sum_c |h_c w_c|, gamma = C u / (1 - C u), u = 2^-24 (the classical
bound for any summation order). The checks are therefore:
  - every reported value lies within that bound of the exact logit at its index;
  - the values are non-increasing, equal values by ascending index, indices distinct;
  - the set is a valid top-16 for some admissible rounding: for every chosen i and every
    unchosen j, exact_i + bound_i >= exact_j - bound_j.
With small-integer data every partial sum is exact, so the result must equal the oracle's
bit for bit, ties included.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import poison_like, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def run_gpu(d2, hid, B, N, row0, ss, rs, w):
    hd = to_dev(np.ascontiguousarray(hid).reshape(-1))
    wd = to_dev(np.ascontiguousarray(w))
    idx = poison_like((B, N, 16), torch.int32)
    val = poison_like((B, N, 16), torch.float32)
    d2.lmhead_topk16(hd, B, N, row0, ss, rs, wd, idx=idx, val=val)
    torch.cuda.synchronize()
    return to_host(idx).reshape(B * N, 16), to_host(val).reshape(B * N, 16)


def check_valid(gi, gv, L, A, C, what):
    u = 2.0 ** -24
    gamma = C * u / (1 - C * u)
    for m in range(gi.shape[0]):
        i, v = gi[m].astype(np.int64), gv[m].astype(np.float64)
        assert len(set(i.tolist())) == 16 and i.min() >= 0 and i.max() < L.shape[1], what
        bound = gamma * A[m] + 1e-30
        err = np.abs(v - L[m, i])
        assert np.all(err <= bound[i]), f"{what} row {m}: value error {err.max()} > bound"
        d = np.diff(v)
        assert np.all(d <= 0) and np.all(np.diff(i)[d == 0] > 0), f"{what} row {m}: order"
        chosen = np.zeros(L.shape[1], bool)
        chosen[i] = True
        lo = np.min(L[m, i] + bound[i])
        hi = np.max(np.where(chosen, -np.inf, L[m] - bound))
        assert lo >= hi, f"{what} row {m}: an excluded logit beats a chosen one ({hi} > {lo})"


def run_case(d2, hid, B, N, row0, ss, rs, w, what, exact=False):
    C = w.shape[1]
    say(f"lmhead_topk16 {what} B={B} N={N} C={C} V={w.shape[0]} row0={row0}")
    gi, gv = run_gpu(d2, hid, B, N, row0, ss, rs, w)
    oi, L, A = orc.lmhead_topk16(hid, B, N, row0, ss, rs, w)
    oi = oi.reshape(B * N, 16)
    if exact:
        np.testing.assert_array_equal(gi, oi, err_msg=what)
        np.testing.assert_array_equal(gv, np.take_along_axis(L, oi.astype(np.int64), 1).astype(np.float32),
                                      err_msg=what)
    else:
        check_valid(gi, gv, L, A, C, what)
    return gi, oi


def _rand(rng, shape, scale):
    return wl.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


@pytest.mark.parametrize("B,N,C,V", [(1, 7, 256, 1000), (2, 3, 128, 32), (1, 1, 384, 16),
                                     (5, 7, 512, 3001), (16, 7, 512, 3001), (19, 7, 256, 4097),
                                     (12, 4, 128, 16), (64, 7, 128, 700)])
def test_lmhead_small_shapes(d2, B, N, C, V):
    # up to 32 hidden rows: ragged last vocabulary block, a single block, V = 16; more
    # than 32 (the tiled kernel, 128 rows per pass): a ragged row tile, two and four passes,
    # a vocabulary smaller than one workgroup's eight blocks, and last block groups that
    # are only partly inside the vocabulary
    rng = np.random.default_rng(B * 1000 + N * 100 + C + V)
    hid = _rand(rng, (B, N + 1, C), 2.0)
    w = _rand(rng, (V, C), 1.0 / np.sqrt(C))
    run_case(d2, hid, B, N, 1, (N + 1) * C, C, w, f"small B{B} N{N} C{C} V{V}")


def test_lmhead_integer_data_is_exact_with_ties(d2):
    rng = np.random.default_rng(91)
    B, N, C, V = 3, 7, 640, 9000
    hid = wl.to_bf16_bits(rng.integers(-2, 3, size=(B, N, C)).astype(np.float32))
    w = rng.integers(-1, 2, size=(V, C)).astype(np.float32)
    w[[100, 4000, 8999]] = w[5]                            # exact ties across blocks and waves
    run_case(d2, hid, B, N, 0, N * C, C, wl.to_bf16_bits(w), "integer data", exact=True)


def test_lmhead_integer_data_many_rows_exact(d2):
    # the tiled kernel on exact data: 42 hidden rows, ties across workgroups
    rng = np.random.default_rng(93)
    B, N, C, V = 6, 7, 640, 9000
    hid = wl.to_bf16_bits(rng.integers(-2, 3, size=(B, N, C)).astype(np.float32))
    w = rng.integers(-1, 2, size=(V, C)).astype(np.float32)
    w[[31, 32, 4000, 8999]] = w[7]
    run_case(d2, hid, B, N, 0, N * C, C, wl.to_bf16_bits(w), "integer data, 42 rows", exact=True)


def test_lmhead_strides_and_broadcast(d2):
    # hidden rows with padding between rows and a zero sequence stride (all sequences
    # share one block of rows)
    rng = np.random.default_rng(92)
    B, N, C, V, pad = 3, 4, 256, 2000, 24
    buf = _rand(rng, (N + 2, C + pad), 2.0)
    w = _rand(rng, (V, C), 1.0 / 16)
    gi, _ = run_case(d2, buf, B, N, 2, 0, C + pad, w, "zero seq stride, padded rows")
    np.testing.assert_array_equal(gi[:N], gi[N:2 * N])


def test_lmhead_drafter_geometry(d2):
    # the drafter's head: C = 5120, V = 248320, the 7 proposal rows of one block
    cfg = wl.CONFIGS[2]
    say("lmhead_topk16 generating the 248320 x 5120 head")
    w = wl.head_weight(cfg)
    hid = wl.head_hidden(cfg)
    gi, oi = run_case(d2, hid, 1, cfg.N, 1, cfg.P * cfg.C, cfg.C, w, "drafter geometry")
    # with continuous data the order is essentially unambiguous
    assert (gi == oi).mean() > 0.95


def test_lmhead_drafter_geometry_batch16_sampled(d2):
    # 16 sequences x 7 proposal rows (one 128-row tile) on the drafter's head; the oracle
    # is evaluated on a sample of the 112 rows
    cfg = wl.CONFIGS[2]
    B, N, P, C = 16, cfg.N, cfg.P, cfg.C
    w = wl.head_weight(cfg)
    rng = np.random.default_rng(94)
    hid = _rand(rng, (B, P, C), float(np.sqrt(cfg.draft_var)))
    say(f"lmhead_topk16 drafter geometry B={B} N={N} C={C} V={w.shape[0]}")
    gi, gv = run_gpu(d2, hid, B, N, 1, P * C, C, w)
    sample = [0, 6, 31, 32, 63, 64, 95, 111]
    rows = np.stack([hid[m // N, 1 + m % N] for m in sample])
    oi, L, A = orc.lmhead_topk16(rows, 1, len(sample), 0, 0, C, w)
    check_valid(gi[sample], gv[sample], L, A, C, "drafter geometry B16 sample")
    assert (gi[sample] == oi.reshape(len(sample), 16)).mean() > 0.95
