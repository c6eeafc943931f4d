"""dflash2_proj against the binary64 oracle, and its outputs fed to the conv and selector.

The GPU sums exact bf16 products in binary32 in its own fixed order, so each output may
differ from the exact sum by at most gamma_C * sum_c |h_c w_c|, gamma_C = C u / (1 - C u),
u = 2^-24 (the classical bound for any summation order); the tests check every output
against it. With data on a coarse binary grid every partial sum is exact, so the result
must equal the oracle's bit for bit; the composition tests use such data so that the
conv and selector see exactly the oracle's coefficients and gate.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from helpers import assert_close_tol, assert_same_floats, poison_like, say, to_dev, to_host

pytestmark = pytest.mark.gpu

BF16_TOL = dict(max_abs=2e-2, rel_l2=1e-2)


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def _rand(rng, shape, scale):
    return wl.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def _grid(rng, shape, k=2, scale=2.0**-6):
    """Integers in [-k, k] times a power of two: exact in bf16, and sums of their products
    stay exact in binary32 for the sizes used here."""
    return wl.to_bf16_bits(rng.integers(-k, k + 1, size=shape).astype(np.float32) * np.float32(scale))


def run_gpu(d2, hid_flat, B, N, row0, ss, rs, w, out_shape=None, oss=None, ors=None):
    O, C = w.shape
    hd = to_dev(np.ascontiguousarray(hid_flat).reshape(-1))
    wd = to_dev(np.ascontiguousarray(w))
    if out_shape is None:
        out = poison_like((B, N, O), torch.float32)
        d2.proj(hd, B, N, row0, ss, rs, wd, out=out)
    else:
        out = poison_like(out_shape, torch.float32)
        d2.proj(hd, B, N, row0, ss, rs, wd, out=out, out_seq_stride=oss, out_row_stride=ors)
    torch.cuda.synchronize()
    return to_host(out)


def check_bound(got, Y, A, C, what):
    u = 2.0 ** -24
    gamma = C * u / (1 - C * u)
    assert np.all(np.isfinite(got)), f"{what}: nonfinite output"
    err = np.abs(got.astype(np.float64) - Y)
    bound = gamma * A + 1e-30
    worst = float((err / bound).max())
    assert np.all(err <= bound), f"{what}: error {err.max():.3g} exceeds the bound (x{worst:.2f})"


@pytest.mark.parametrize("B,N,row0,C,O,pad", [
    (1, 8, 0, 5120, 640, 0),      # one conv site's coefficients at the drafter width
    (1, 7, 1, 5120, 256, 0),      # selector gate: rows 1..7 of the block
    (2, 8, 0, 264, 23, 8),        # ragged contraction (8.25 steps) and output tile
    (3, 8, 0, 1024, 48, 0),       # 24 rows: two row tiles per wave
    (5, 7, 1, 512, 100, 16),      # 35 rows: four row tiles, ragged
    (16, 7, 1, 256, 16, 0),       # the tiny configuration's gate shape
    (1, 1, 0, 8, 1, 0),           # smallest call
    (64, 8, 0, 5120, 640, 0),     # batch 64 at the drafter width
    (256, 8, 0, 512, 640, 8),     # 2048 rows: enough 64 x 64 tiles for one kernel, no split
    (5, 8, 0, 264, 520, 8),       # 64 x 64 tiles with ragged features, rows and contraction
])
def test_proj_within_bound(d2, B, N, row0, C, O, pad):
    rng = np.random.default_rng(700 + B * 31 + C + O)
    rs = C + pad
    ss = (row0 + N) * rs + pad
    hid = _rand(rng, (B * ss,), 1.0)
    w = _rand(rng, (O, C), C ** -0.5)
    say(f"proj B={B} N={N} row0={row0} C={C} O={O} pad={pad}")
    got = run_gpu(d2, hid, B, N, row0, ss, rs, w)
    Y, A = orc.proj(hid, B, N, row0, ss, rs, w)
    check_bound(got, Y, A, C, f"proj B={B} N={N} C={C} O={O}")
    again = run_gpu(d2, hid, B, N, row0, ss, rs, w)
    assert_same_floats(again, got, "a second call")


@pytest.mark.parametrize("B,N,C,O", [(1, 8, 5120, 640), (7, 8, 264, 33), (3, 8, 1024, 48),
                                     (5, 8, 264, 520), (64, 8, 1024, 640)])
def test_proj_exact_on_grid_data(d2, B, N, C, O):
    rng = np.random.default_rng(800 + B + C)
    hid = _grid(rng, (B * N * C,))
    w = _grid(rng, (O, C))
    say(f"proj exact B={B} N={N} C={C} O={O}")
    got = run_gpu(d2, hid, B, N, 0, N * C, C, w)
    Y, _ = orc.proj(hid, B, N, 0, N * C, C, w)
    assert_same_floats(got, Y.astype(np.float32), "grid data")


def test_proj_broadcast_and_row_major_output(d2):
    # hidden sequence stride 0 (every sequence reads the same rows); outputs placed
    # row-major ([N, B, O] with padding), the padding left untouched
    rng = np.random.default_rng(901)
    B, N, C, O = 4, 7, 512, 40
    hid = _rand(rng, (N * C,), 1.0)
    w = _rand(rng, (O, C), C ** -0.5)
    oss, ors = O + 4, B * (O + 4) + 8
    say(f"proj broadcast B={B} N={N} C={C} O={O}")
    got = run_gpu(d2, hid, B, N, 0, 0, C, w, out_shape=(N * ors,), oss=oss, ors=ors)
    Y, A = orc.proj(hid, B, N, 0, 0, C, w)
    for b in range(B):
        for r in range(N):
            seg = got[b * oss + r * ors: b * oss + r * ors + O]
            check_bound(seg[None], Y[b, r][None], A[b, r][None], C, f"row {r} seq {b}")
            assert_same_floats(seg, got[r * ors: r * ors + O], "broadcast rows")
    written = np.zeros(got.shape, bool)
    for b in range(B):
        for r in range(N):
            written[b * oss + r * ors: b * oss + r * ors + O] = True
    assert np.all(got.view(np.uint32)[~written] == 0xFFFFFFFF), "padding was written"


def test_proj_coefficients_drive_the_conv(d2):
    # one projection of the sublayer input gives both convs' coefficients (two calls, the
    # weight offset by 2G rows); on grid data they equal the oracle's exactly, and the conv
    # driven by them matches the oracle conv driven by the oracle's coefficients
    rng = np.random.default_rng(902)
    B, P, C = 2, 8, 5120
    G = C // 16
    x = _grid(rng, (B, P, C))
    wd = _grid(rng, (4 * G, C))
    base = rng.uniform(-1, 1, (2, C)).astype(np.float32)
    say(f"proj -> dynconv2 B={B} P={P} C={C}")
    xd, wdd = to_dev(x), to_dev(wd)
    d_in = poison_like((B, P, 2, G), torch.float32)
    d_out = poison_like((B, P, 2, G), torch.float32)
    d2.proj(xd, B, P, 0, P * C, C, wdd[:2 * G], out=d_in.view(B, P, 2 * G))
    d2.proj(xd, B, P, 0, P * C, C, wdd[2 * G:], out=d_out.view(B, P, 2 * G))
    out = poison_like((B, P, C), torch.bfloat16)
    d2.dynconv2(xd, to_dev(base), d_in, out=out)
    torch.cuda.synchronize()
    o_in, o_out = orc.conv_coeffs(x, wd, G)
    assert_same_floats(to_host(d_in), o_in, "coefficients of the conv before the sublayer")
    assert_same_floats(to_host(d_out), o_out, "coefficients of the conv after the sublayer")
    assert_close_tol(to_host(out), orc.dynconv2(x, base, o_in), what="conv", **BF16_TOL)


@pytest.mark.parametrize("T", [0.0, 0.7])
def test_proj_gate_drives_the_selector(d2, T):
    # gate = projection of block rows 1..7; on grid data it equals the oracle's gate
    # exactly, so the selector's tokens, slots and q must match bit for bit
    cfg = wl.CONFIGS[2]
    rng = np.random.default_rng(903)
    B, P, C, R, V = 2, 8, cfg.C, cfg.R, 4096
    hid = _grid(rng, (B, P, C))
    wg = _grid(rng, (R, C), k=3, scale=2.0**-7)
    A = _rand(rng, (V, R), 0.25)
    Bc = _rand(rng, (V, R), 0.25)
    draft = wl.to_bf16_bits(rng.standard_normal((B, P, V)).astype(np.float32) * 2)
    ci, cv = orc.topk16(draft.reshape(-1), B, P - 1, 1, P * V, V, V)
    anchor = rng.integers(0, V, size=B).astype(np.int32)
    temp = np.full(B, T, np.float32)
    say(f"proj -> select B={B} C={C} R={R} T={T}")
    gate = poison_like((B, P - 1, R), torch.float32)
    d2.proj(to_dev(hid), B, P - 1, 1, P * C, C, to_dev(wg), out=gate)
    tok = poison_like((B, P - 1), torch.int32)
    sl = poison_like((B, P - 1), torch.int32)
    q = poison_like((B, P - 1, 16), torch.float32)
    st = poison_like((B,), torch.int32)
    d2.select(to_dev(ci), to_dev(cv), gate, to_dev(A), to_dev(Bc), to_dev(anchor),
              to_dev(temp), cfg.seed, 3, tokens=tok, slot=sl, q=q, status=st)
    torch.cuda.synchronize()
    og = orc.selector_gate(hid, wg)
    assert_same_floats(to_host(gate), og, "gate")
    o = orc.select(ci, cv, og, A, Bc, anchor, temp, cfg.seed, 3)
    np.testing.assert_array_equal(to_host(tok), o[0], err_msg="tokens")
    np.testing.assert_array_equal(to_host(sl), o[1], err_msg="slot")
    assert_same_floats(to_host(q), o[2], "q")
    np.testing.assert_array_equal(to_host(st), o[3], err_msg="status")


def test_proj_and_conv_replayed_in_a_graph(d2):
    # the split path (workspace partials, then the ordered reduction) captured with the conv
    # it feeds in one HIP graph; every replay, with the outputs scribbled over in between,
    # must equal the eager result bit for bit
    rng = np.random.default_rng(904)
    B, P, C = 1, 8, 5120
    G = C // 16
    x = to_dev(_rand(rng, (B, P, C), 1.0))
    w = to_dev(_rand(rng, (2 * G, C), C ** -0.5))
    base = to_dev(rng.uniform(-1, 1, (2, C)).astype(np.float32))
    delta = torch.empty((B, P, 2, G), dtype=torch.float32, device=x.device)
    out = torch.empty((B, P, C), dtype=torch.bfloat16, device=x.device)
    ws = d2.workspace(d2.proj_workspace_bytes(B, P, 2 * G, C), x.device)
    assert d2.proj_workspace_bytes(B, P, 2 * G, C) > 0          # the split path
    say("proj + dynconv2 graph replay B=1 C=5120")

    def run():
        d2.proj(x, B, P, 0, P * C, C, w, out=delta.view(B, P, 2 * G), ws=ws)
        d2.dynconv2(x, base, delta, out=out)

    run()
    torch.cuda.synchronize()
    want_d, want_o = to_host(delta), to_host(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        delta.fill_(float("nan"))
        out.view(torch.int16).fill_(-1)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same_floats(to_host(delta), want_d, f"coefficients, replay {rep}")
        np.testing.assert_array_equal(to_host(out), want_o, err_msg=f"conv, replay {rep}")
