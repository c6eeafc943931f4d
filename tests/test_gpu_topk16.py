"""dflash2_topk16 against the oracle: bit-exact indices and values."""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import DEV, assert_same_floats, poison_like, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def run_gpu(d2, host, B, N, row0, ss, rs, V, flat_len=None):
    dev = to_dev(np.ascontiguousarray(host).reshape(-1))
    idx = poison_like((B, N, 16), torch.int32)
    val = poison_like((B, N, 16), torch.float32)
    d2.topk16(dev, B, N, row0, ss, rs, V, idx=idx, val=val)
    torch.cuda.synchronize()
    return to_host(idx), to_host(val)


def check(d2, host, B, N, row0, ss, rs, V, what):
    say(f"topk16 {what} B={B} N={N} V={V} row0={row0} ss={ss} rs={rs} dtype={host.dtype}")
    gi, gv = run_gpu(d2, host, B, N, row0, ss, rs, V)
    oi, ov = orc.topk16(np.ascontiguousarray(host).reshape(-1), B, N, row0, ss, rs, V)
    np.testing.assert_array_equal(gi, oi, err_msg=what)
    assert_same_floats(gv, ov, what)


def test_topk16_tiny_config_f32(d2):
    cfg = wl.CONFIGS[1]
    draft = wl.draft_logits(cfg)                  # [1, 8, 1024] f32
    check(d2, draft, 1, 7, 1, 8 * cfg.V, cfg.V, cfg.V, "config 1")


def test_topk16_drafter_geometry_bf16(d2):
    cfg = wl.CONFIGS[2]
    draft = wl.draft_logits(cfg)                  # [1, 8, 248320] bf16
    check(d2, draft, 1, 7, 1, 8 * cfg.V, cfg.V, cfg.V, "config 2")


def test_topk16_quantised_ties_batch16(d2):
    cfg = wl.CONFIGS[4]
    draft = wl.draft_logits(cfg)                  # [16, 8, V] bf16, multiples of 0.25
    say("topk16 config 4 B=16 full")
    gi, gv = run_gpu(d2, draft, 16, 7, 1, 8 * cfg.V, cfg.V, cfg.V)
    for b in (0, 7, 15):                          # the oracle on a sample of sequences
        oi, ov = orc.topk16(np.ascontiguousarray(draft[b]).reshape(-1), 1, 7, 1, 0, cfg.V, cfg.V)
        np.testing.assert_array_equal(gi[b], oi[0], err_msg=f"seq {b}")
        assert_same_floats(gv[b], ov[0], f"seq {b}")
    # property on every row: values non-increasing, equal values in increasing index
    full = wl.bf16_bits_to_f32(draft[:, 1:])
    assert np.all(np.diff(gv, axis=2) <= 0)
    eq = np.diff(gv, axis=2) == 0
    assert np.all(np.diff(gi, axis=2)[eq] > 0)
    # the 16th value bounds the rest of the row
    kth = gv[:, :, 15]
    assert np.all((full > kth[..., None]).sum(axis=2) <= 15)


def _edge_rows(V=4097):
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((8, V)).astype(np.float32)
    rows[0, [4000, 5, 2048, 511, 512]] = np.nan
    rows[0, [7, 3000]] = np.inf
    rows[0, [1, 2, 4096]] = -np.inf
    rows[1, :] = -1.0
    rows[1, [511, 512, 1023, 1024, 4095, 4096, 0]] = 3.0
    rows[1, [100, 600, 1100, 1600, 2100, 2600, 3100, 3600, 4000, 4050]] = 3.0
    rows[2, :] = -np.inf
    rows[3, ::2] = np.inf
    rows[4, :] = 0.0
    rows[4, ::3] = -0.0
    rows[5, :] = np.sort(rng.standard_normal(V))[::-1]        # all the best in one chunk
    rows[6, :] = np.sort(rng.standard_normal(V))
    rows[7, :] = np.where(rng.random(V) < 0.5, 0.0, -0.0)
    rows[7, 17] = 1e-45                                        # one subnormal above the zeros
    return rows


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk16_edge_rows(d2, dtype):
    rows = _edge_rows()
    host = rows if dtype == "f32" else wl.to_bf16_bits(rows)
    n, V = rows.shape
    check(d2, host, 1, n, 0, 0, V, V, f"edge rows {dtype}")
    # each row on its own, as a batch of sequences
    check(d2, host, n, 1, 0, V, 0, V, f"edge rows as batch {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk16_negative_nans_and_zero_runs(d2, dtype):
    V = 9000
    rng = np.random.default_rng(21)
    rows = rng.standard_normal((4, V)).astype(np.float32)
    neg_nan = np.array([0xFFC00001], dtype=np.uint32).view(np.float32)[0]
    rows[0, [8191, 8192, 3]] = neg_nan                  # negative NaNs still come first
    rows[1, :] = 0.0                                   # ties across every chunk
    rows[2, 100:8000] = 7.0                            # a long run of a top value
    rows[3, ::97] = -np.inf
    host = rows if dtype == "f32" else wl.to_bf16_bits(rows)
    if dtype == "bf16":
        host[0, [8191, 8192, 3]] = 0xFFC1
    check(d2, host, 1, 4, 0, 0, V, V, f"neg-nan/zero runs {dtype}")


@pytest.mark.parametrize("V", [16, 17, 31, 1000, 2049, 4097, 65537])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk16_ragged_widths(d2, V, dtype):
    rng = np.random.default_rng(V)
    B, P = 3, 8
    x = (np.round(rng.standard_normal((B, P, V)) * 3) / 3).astype(np.float32)
    host = x if dtype == "f32" else wl.to_bf16_bits(x)
    # packed rows (strides multiples of V: aligned only when V*size is a multiple of 16)
    check(d2, host, B, P - 1, 1, P * V, V, V, f"ragged V={V}")


def test_topk16_strides_and_broadcast(d2):
    rng = np.random.default_rng(22)
    V, Vpad = 3000, 3008
    x = wl.to_bf16_bits(rng.standard_normal((4, 8, Vpad)).astype(np.float32))
    # padded row stride, row0 = 2, 5 rows per sequence
    check(d2, x, 4, 5, 2, 8 * Vpad, Vpad, V, "padded stride")
    # seq_stride 0 broadcasts one sequence to all
    check(d2, x, 3, 7, 1, 0, Vpad, V, "broadcast")
    # odd stride forces element-wise loads
    y = x.reshape(-1)[: 4 * 8 * 3001].copy()
    check(d2, y, 4, 7, 1, 8 * 3001, 3001, 3000, "odd stride")


def test_topk16_serving_batch(d2):
    rng = np.random.default_rng(23)
    B, P, V = 64, 8, 20000
    x = wl.to_bf16_bits((rng.standard_normal((B, P, V)) * 2).astype(np.float32))
    say("topk16 B=64 V=20000")
    gi, gv = run_gpu(d2, x, B, P - 1, 1, P * V, V, V)
    oi, ov = orc.topk16(x.reshape(-1), B, P - 1, 1, P * V, V, V)
    np.testing.assert_array_equal(gi, oi)
    assert_same_floats(gv, ov)


def test_topk16_deterministic(d2):
    cfg = wl.CONFIGS[2]
    draft = wl.draft_logits(cfg)
    a = run_gpu(d2, draft, 1, 7, 1, 8 * cfg.V, cfg.V, cfg.V)
    b = run_gpu(d2, draft, 1, 7, 1, 8 * cfg.V, cfg.V, cfg.V)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def _bf16(x):
    return wl.to_bf16_bits(np.asarray(x, np.float32))


@pytest.mark.parametrize("case", ["late_specials", "tie_plateau", "rising", "unaligned_long",
                                  "f32_late_specials"])
def test_topk16_long_rows_adversarial(d2, case):
    # Full-width rows whose decisive elements sit deep in the row, so that they meet the
    # running thresholds of many sub-chunks and workgroups: NaN (both signs, quiet and
    # signalling patterns) and infinities placed late, a plateau of equal maxima spread over
    # the whole row, values that rise along the row (every sub-chunk raises the threshold),
    # and a row length that is not a whole number of 16-byte vectors (the register-load path).
    seed = {"late_specials": 61, "tie_plateau": 62, "rising": 63, "unaligned_long": 64,
            "f32_late_specials": 65}[case]
    rng = np.random.default_rng(seed)
    V = 248317 if case == "unaligned_long" else 248320
    B, N = 8, 7
    x = rng.standard_normal((B, N + 1, V)).astype(np.float32) * 2.0
    if case == "tie_plateau":
        x = np.round(x)                            # few distinct values
        for b in range(B):
            for r in range(1, N + 1):
                pos = rng.choice(V, size=40, replace=False)
                x[b, r, pos] = 9.0                 # 40 equal maxima, ties by index
    elif case == "rising":
        x += np.linspace(0.0, 30.0, V, dtype=np.float32)[None, None, :]
    f32 = case.startswith("f32")
    host = x if f32 else _bf16(x)
    if case.endswith("late_specials"):
        if f32:
            pats = [0x7FC00000, 0xFFC00000, 0x7F800001, 0x7F800000, 0xFF800000, 0x80000000]
            bits = host.view(np.uint32)
        else:
            pats = [0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80, 0x8000]
            bits = host
        for b in range(B):
            for r in range(1, N + 1):
                pos = rng.choice(np.arange(V // 2, V), size=len(pats), replace=False)
                for p_, v_ in zip(pos, pats):
                    bits[b, r, p_] = v_
    check(d2, host, B, N, 1, (N + 1) * V, V, V, f"long rows {case}")


def test_topk16_shared_workspace(d2):
    # One workspace for many calls with different rows, starting from stale contents.
    B, N, V = 8, 7, 100003
    rng = np.random.default_rng(71)
    ws = d2.workspace(d2.topk16_workspace_bytes(B, N, V, d2.F32), DEV)
    ws.fill_(0xA5)
    for it in range(6):
        say(f"topk16 shared workspace call {it} B={B} N={N} V={V}")
        host = rng.standard_normal((B, N + 1, V)).astype(np.float32)
        if it % 2:
            host[:, :, ::7] = 0.5                 # a plateau of ties
        dev = to_dev(host.reshape(-1))
        idx = poison_like((B, N, 16), torch.int32)
        val = poison_like((B, N, 16), torch.float32)
        d2.topk16(dev, B, N, 1, (N + 1) * V, V, V, idx=idx, val=val, ws=ws)
        torch.cuda.synchronize()
        oi, ov = orc.topk16(host.reshape(-1), B, N, 1, (N + 1) * V, V, V)
        np.testing.assert_array_equal(to_host(idx), oi, err_msg=f"call {it}")
        assert_same_floats(to_host(val), ov, f"call {it}")


@pytest.mark.parametrize("V", [2097152, 2097153])
def test_topk16_most_lists_per_row(d2, V):
    # A single row long enough that its 512 workgroups write 2048 lists, which the merge
    # reads maxima first, and one element past that (513 workgroups).
    rng = np.random.default_rng(V % 97)
    host = _bf16(rng.standard_normal((1, 2, V)).astype(np.float32) * 3.0)
    check(d2, host, 1, 1, 1, 2 * V, V, V, f"most lists V={V}")
