"""One DFlash2 draft-and-verify step as a sequence of library calls on one stream.

A step is, per drafter layer, the dynamic conv around the attention sublayer (in and out)
and around the MLP sublayer (in and out) with the block attention between them ("[Spec
Decode] DFlash2: local convolution + candidate selector - #52816": the conv wraps each
sublayer in and out, 20 calls over five layers), then top-16 over draft rows 1..N, the
selector and the verify. The projections, MLP and LM head are outside the step, so the
attention and conv outputs do not feed the logits: every stage reads its own inputs.

`StepRunner` keeps all inputs of one or more input sets resident on the GPU, allocates
every output and workspace once, and can capture the whole step in a HIP graph. Nothing
here computes: it only orders the calls of the C ABI through the ctypes binding.
"""
from __future__ import annotations

import numpy as np
import torch

from . import dflash2 as d2
from . import workloads as wl


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


class DeviceInputs:
    """One input set of a configuration, resident in HBM."""

    def __init__(self, si: wl.StepInputs, device, cb_dev=None):
        self.cfg = si.cfg
        self.ctx_len = _dev(si.ctx_len, device)
        self.q = [_dev(a, device) for a in si.q]
        self.k_blk = [_dev(a, device) for a in si.k_blk]
        self.v_blk = [_dev(a, device) for a in si.v_blk]
        self.k_ring = [_dev(a, device) for a in si.k_ring]
        self.v_ring = [_dev(a, device) for a in si.v_ring]
        self.conv_x = [_dev(a, device) for a in si.conv_x]
        self.conv_base = [_dev(a, device) for a in si.conv_base]
        self.conv_delta = [_dev(a, device) for a in si.conv_delta]
        self.draft = _dev(si.draft, device)
        self.target = _dev(si.target, device)
        if cb_dev is None:
            cb_dev = (_dev(si.pred_cb, device), _dev(si.succ_cb, device))
        self.pred_cb, self.succ_cb = cb_dev
        self.gate = _dev(si.gate, device)
        self.anchor = _dev(si.anchor, device)
        self.temperature = _dev(si.temperature, device)


class StepOutputs:
    def __init__(self, cfg: wl.Config, device):
        B, P, N = cfg.B, cfg.P, cfg.N
        act = torch.bfloat16 if cfg.act_bf16 else torch.float32
        self.attn = [torch.empty((B, P, cfg.Hq, cfg.D), dtype=act, device=device)
                     for _ in range(cfg.layers)]
        self.conv = [torch.empty((B, P, cfg.C), dtype=act, device=device)
                     for _ in range(cfg.sites)]
        self.cand_idx = torch.empty((B, N, 16), dtype=torch.int32, device=device)
        self.cand_val = torch.empty((B, N, 16), dtype=torch.float32, device=device)
        self.tokens = torch.empty((B, N), dtype=torch.int32, device=device)
        self.slot = torch.empty((B, N), dtype=torch.int32, device=device)
        self.q = torch.empty((B, N, 16), dtype=torch.float32, device=device)
        self.status = torch.empty((B,), dtype=torch.int32, device=device)
        self.n_accept = torch.empty((B,), dtype=torch.int32, device=device)
        self.out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=device)


class StepRunner:
    def __init__(self, cfg: wl.Config, inputs: list[DeviceInputs], device="cuda:0"):
        self.cfg = cfg
        self.inputs = inputs
        self.device = device
        self.out = StepOutputs(cfg, device)
        B, P, N, V = cfg.B, cfg.P, cfg.N, cfg.V
        adt = d2.BF16 if cfg.act_bf16 else d2.F32
        tdt = d2.F32 if cfg.target_kind == "probs" else adt
        self.ws_attn = d2.workspace(
            d2.block_attn_workspace_bytes(B, P, cfg.Hq, cfg.Hkv, cfg.D, cfg.S, cfg.W, adt), device)
        self.ws_topk = d2.workspace(d2.topk16_workspace_bytes(B, N, V, adt), device)
        self.ws_sel = d2.workspace(d2.select_workspace_bytes(B, N), device)
        self.ws_ver = d2.workspace(d2.verify_workspace_bytes(B, N, V, tdt), device)
        self.graphs: dict[int, torch.cuda.CUDAGraph] = {}

    # the sublayers of layer l use conv sites 4l .. 4l+3 (attention in/out, MLP in/out)
    def run(self, iset: int = 0, step: int = 0):
        c, x, o = self.cfg, self.inputs[iset], self.out
        B, P, N, V = c.B, c.P, c.N, c.V
        for layer in range(c.layers):
            s0 = layer * c.conv_sites_per_layer
            d2.dynconv2(x.conv_x[s0], x.conv_base[s0], x.conv_delta[s0], out=o.conv[s0])
            d2.block_attn(x.q[layer], x.k_blk[layer], x.v_blk[layer], x.k_ring[layer],
                          x.v_ring[layer], x.ctx_len, c.W, out=o.attn[layer], ws=self.ws_attn)
            for s in range(s0 + 1, s0 + c.conv_sites_per_layer):
                d2.dynconv2(x.conv_x[s], x.conv_base[s], x.conv_delta[s], out=o.conv[s])
        d2.topk16(x.draft, B, N, 1, P * V, V, V, idx=o.cand_idx, val=o.cand_val, ws=self.ws_topk)
        d2.select(o.cand_idx, o.cand_val, x.gate, x.pred_cb, x.succ_cb, x.anchor, x.temperature,
                  c.seed, step, tokens=o.tokens, slot=o.slot, q=o.q, status=o.status,
                  ws=self.ws_sel)
        d2.verify(x.target, B, N, P * V, V, V, o.tokens, o.cand_idx, o.q, o.slot, x.temperature,
                  c.seed, step, o.status, n_accept=o.n_accept, out_tokens=o.out_tokens,
                  ws=self.ws_ver)

    def capture(self, iset: int = 0, step: int = 0) -> torch.cuda.CUDAGraph:
        """Capture one step of input set `iset` (its draws use counter `step`)."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run(iset, step)   # warm the launch path outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(iset, step)
        self.graphs[iset] = g
        return g
