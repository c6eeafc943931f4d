"""A whole draft-and-verify step on the GPU against an independent oracle chain.

The GPU step runs every stage through the C ABI; the oracle recomputes the chain from the
same inputs on its own (its top-16 feeds its selector, which feeds its verify). Integer
outputs (candidates, paths, slots, q rows, accept counts, emitted tokens, status) must be
bit-identical; attention and conv outputs must be within the bf16/f32 tolerances.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from block_drafter_draft_amd import workloads as wl
from block_drafter_draft_amd.step import DeviceInputs, StepRunner
from helpers import DEV, assert_close_tol, assert_same_floats, say, to_host

pytestmark = pytest.mark.gpu

BF16_TOL = dict(max_abs=2e-2, rel_l2=1e-2)


def _oracle_chain(cfg, si, step):
    B, P, N, V = cfg.B, cfg.P, cfg.N, cfg.V
    ci, cv = orc.topk16(si.draft.reshape(-1), B, N, 1, P * V, V, V)
    tok, slot, q, st = orc.select(ci, cv, si.gate, si.pred_cb, si.succ_cb, si.anchor,
                                  si.temperature, cfg.seed, step)
    n, out, st2 = orc.verify(si.target.reshape(-1), B, N, P * V, V, V, tok, ci, q, slot,
                             si.temperature, cfg.seed, step, status=st)
    return dict(cand_idx=ci, cand_val=cv, tokens=tok, slot=slot, q=q, n_accept=n,
                out_tokens=out, status=st2)


def _check_chain(o, ref, what):
    np.testing.assert_array_equal(to_host(o.cand_idx), ref["cand_idx"], err_msg=f"{what} cand_idx")
    assert_same_floats(to_host(o.cand_val), ref["cand_val"], f"{what} cand_val")
    for name in ("tokens", "slot", "n_accept", "out_tokens", "status"):
        np.testing.assert_array_equal(to_host(getattr(o, name)), ref[name], err_msg=f"{what} {name}")
    assert_same_floats(to_host(o.q), ref["q"], f"{what} q")


def _check_dense(cfg, si, o, seqs, layers, sites):
    tol_attn = BF16_TOL if cfg.act_bf16 else dict(max_abs=1e-4, rel_l2=1e-5)
    tol_conv = BF16_TOL if cfg.act_bf16 else dict(max_abs=1e-5, rel_l2=1e-6)
    sl = slice(None) if seqs is None else list(seqs)
    for layer in layers:
        got = to_host(o.attn[layer])[sl]
        ref = orc.block_attn(*(np.ascontiguousarray(a[layer][sl]) for a in
                               (si.q, si.k_blk, si.v_blk, si.k_ring, si.v_ring)),
                             si.ctx_len[sl], cfg.W)
        assert_close_tol(got, ref, what=f"attn layer {layer}", **tol_attn)
    for s in sites:
        got = to_host(o.conv[s])[sl]
        ref = orc.dynconv2(np.ascontiguousarray(si.conv_x[s][sl]), si.conv_base[s],
                           np.ascontiguousarray(si.conv_delta[s][sl]))
        assert_close_tol(got, ref, what=f"conv site {s}", **tol_conv)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfgno", [1, 2, 3, 4])
def test_step_matches_oracle(cfgno):
    cfg = wl.CONFIGS[cfgno]
    say(f"step config {cfgno}: generating inputs")
    si = wl.make_step_inputs(cfg)
    runner = StepRunner(cfg, [DeviceInputs(si, DEV)])
    step = 3
    say(f"step config {cfgno}: running")
    runner.run(0, step)
    torch.cuda.synchronize()
    ref = _oracle_chain(cfg, si, step)
    _check_chain(runner.out, ref, f"config {cfgno}")
    seqs = None if cfg.B <= 2 else [0, cfg.B // 2, cfg.B - 1]
    _check_dense(cfg, si, runner.out, seqs, range(cfg.layers), range(cfg.sites))
    print(f"config {cfgno}: mean accepted {to_host(runner.out.n_accept).mean():.3f} of {cfg.N}",
          flush=True)


@pytest.mark.timeout(600)
def test_step_serving_batch():
    cfg = wl.CONFIGS[5]
    say("step config 5: generating inputs")
    si = wl.make_step_inputs(cfg)
    runner = StepRunner(cfg, [DeviceInputs(si, DEV)])
    say("step config 5: running")
    runner.run(0, 1)
    torch.cuda.synchronize()
    ref = _oracle_chain(cfg, si, 1)
    _check_chain(runner.out, ref, "config 5")
    _check_dense(cfg, si, runner.out, [0, 33], [0, 4], [0, 19])


@pytest.mark.timeout(300)
def test_step_graph_replay_matches_eager():
    cfg = wl.CONFIGS[3]
    say("step graph replay: config 3")
    si = wl.make_step_inputs(cfg)
    runner = StepRunner(cfg, [DeviceInputs(si, DEV)])
    runner.run(0, 5)
    torch.cuda.synchronize()
    names = ("cand_idx", "cand_val", "tokens", "slot", "q", "status", "n_accept", "out_tokens")
    eager = {n: to_host(getattr(runner.out, n)).copy() for n in names}
    eager_attn = to_host(runner.out.attn[2]).copy()
    g = runner.capture(0, 5)
    for rep in range(3):
        for n in names:                       # scribble over the outputs between replays
            getattr(runner.out, n).view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            got = to_host(getattr(runner.out, n))
            if got.dtype == np.float32:
                assert_same_floats(got, eager[n], f"replay {rep} {n}")
            else:
                np.testing.assert_array_equal(got, eager[n], err_msg=f"replay {rep} {n}")
        np.testing.assert_array_equal(to_host(runner.out.attn[2]), eager_attn)
