#!/usr/bin/env python3
"""Draft+verify steps/s of the DFlash2 step on one MI355X.

One step is the whole hot path over one batch: per drafter layer the block attention and
its four dynamic-conv sites, then top-16 over the draft rows, the selector and the verify
(5 attention + 20 conv + 1 top-16 + 1 select + 1 verify calls of libdflash2). Inputs are
seeded synthetic tensors already resident in HBM; several input sets are rotated so that
the working set exceeds the 256 MiB last-level cache. Each step is one HIP-graph replay.

Prints one JSON line: throughput, a roofline record for the block-attention call (its
algorithmic bytes over its average duration, measured with HIP events on its stream), the
CPU oracle timed on a bounded sample on one host core, and separate records for the
output-head projection fused with the top-16, the selector over Q8 codebooks and the
best-first draft tree (none of them part of the step).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
LLC_BYTES = 256 << 20           # last-level (MALL) cache
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attn_bytes_flops(cfg, ctx_len):
    """Algorithmic bytes and FLOPs of one block-attention call: every visible context key
    and value of each (sequence, KV head) read once, the queries and block keys/values read
    once, the output written once; 4 * D FLOPs per (query row, visible key) pair."""
    esz = 2 if cfg.act_bf16 else 4
    per_key = cfg.Hkv * cfg.D * 2 * esz
    fixed = (2 * cfg.P * cfg.Hq * cfg.D + 2 * cfg.P * cfg.Hkv * cfg.D) * esz
    nbytes, flops = 0, 0
    for L in ctx_len:
        L = max(int(L), 0)
        nbytes += min(L, cfg.W - 1) * per_key + fixed
        for i in range(cfg.P):
            keys = min(L, max(0, cfg.W - 1 - i)) + cfg.P
            flops += 4 * cfg.D * cfg.Hq * keys
    return nbytes, flops


def set_bytes(cfg):
    esz = 2 if cfg.act_bf16 else 4
    ring = cfg.layers * 2 * cfg.B * cfg.S * cfg.Hkv * cfg.D * esz
    logits = cfg.B * cfg.P * cfg.V * (esz + (4 if cfg.target_kind == "probs" else esz))
    conv = cfg.sites * cfg.B * cfg.P * cfg.C * esz
    return ring + logits + conv


def stage_bytes(cfg, n_accept_sets):
    """Algorithmic bytes per call of each stage other than attention (what the method must
    move): conv reads x and writes out once, plus the coefficients and the base; top-16
    reads the N ranked logits rows once and writes the lists; the selector gathers the
    anchor's and each slot's predecessor rows of A and the slots' candidate rows of B,
    reads the gates and candidates; verify reads, per greedy sequence, the n + 1 target
    rows the argmax chain needs, and per sampled sequence the one row it draws from.
    n_accept_sets: the accept counts of each input set's step."""
    esz = 2 if cfg.act_bf16 else 4
    tsz = 4 if cfg.target_kind == "probs" else esz
    G = cfg.C // 16
    B, P, N, V, R = cfg.B, cfg.P, cfg.N, cfg.V, cfg.R
    conv = 2 * B * P * cfg.C * esz + B * P * 2 * G * 4 + 2 * cfg.C * 4
    topk = B * N * V * esz + B * N * 16 * 8
    select = B * ((1 + (N - 1) * 16 + N * 16) * R * 2 + N * R * 4 + N * 16 * 8)
    temps = cfg.temperatures()
    ver = []
    for n_acc in n_accept_sets:
        rows = sum(1 if temps[b] > 0 else int(n_acc[b]) + 1 for b in range(B))
        ver.append(rows * V * tsz + B * N * 16 * 8)
    return {"dynconv2": conv, "topk16": topk, "select": select, "verify": sum(ver) / len(ver)}


def traffic_record(workload):
    """HBM bytes per attention launch from the committed PMC summary, if it was taken on
    the current kernel source."""
    path = os.path.join(PROFILES, "block_attn_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "block_drafter_draft_amd", "csrc", "block_attn.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, seconds):
    """The oracle, as it stands, on one host core: whole steps of the same workload, one
    sequence at a time, for about `seconds`; scaled to steps/s of the full batch."""
    import numpy as np

    import oracle as orc
    from block_drafter_draft_amd import workloads as wl
    si = wl.make_step_inputs(cfg, iset=0)
    B, P, N, V = cfg.B, cfg.P, cfg.N, cfg.V
    t0 = time.perf_counter()
    seqs_done = 0
    while True:
        b = seqs_done % B
        sl = slice(b, b + 1)
        for layer in range(cfg.layers):
            orc.block_attn(*(np.ascontiguousarray(a[layer][sl]) for a in
                             (si.q, si.k_blk, si.v_blk, si.k_ring, si.v_ring)),
                           si.ctx_len[sl], cfg.W)
        for s in range(cfg.sites):
            orc.dynconv2(np.ascontiguousarray(si.conv_x[s][sl]), si.conv_base[s],
                         np.ascontiguousarray(si.conv_delta[s][sl]))
        ci, cv = orc.topk16(np.ascontiguousarray(si.draft[sl]).reshape(-1), 1, N, 1, P * V, V, V)
        tok, slot, q, st = orc.select(ci, cv, np.ascontiguousarray(si.gate[sl]), si.pred_cb,
                                      si.succ_cb, si.anchor[sl], si.temperature[sl], cfg.seed, 0)
        orc.verify(np.ascontiguousarray(si.target[sl]).reshape(-1), 1, N, P * V, V, V, tok, ci, q,
                   slot, si.temperature[sl], cfg.seed, 0, status=st)
        seqs_done += 1
        el = time.perf_counter() - t0
        if el >= seconds and seqs_done >= 1:
            break
    steps = seqs_done / B
    return {"value": steps / el, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{seqs_done} sequence(s) of full oracle steps ({steps:.3g} steps of batch "
                      f"{B}) in {el:.1f} s on one host core"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="input configuration (default: the drafter geometry at batch 1)")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets to rotate (default: enough to exceed the last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lmhead", action="store_true",
                    help="skip the separate output-head + top-16 and projection measurements")
    ap.add_argument("--no-q8", action="store_true",
                    help="skip the separate Q8-selector and draft-tree measurements")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the DFlash2 step shards by sequence with no "
              "exchange, and no multi-GPU path is implemented (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_drafter_draft_amd import dflash2 as d2
    from block_drafter_draft_amd import workloads as wl
    from block_drafter_draft_amd.step import DeviceInputs, StepRunner

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = "cuda:0"
    cfg = wl.CONFIGS[args.workload]
    nsets = args.sets or max(1, min(16, math.ceil(1.25 * LLC_BYTES / set_bytes(cfg))))
    log(f"workload {cfg.cfg} ({cfg.name}), {nsets} input set(s) of {set_bytes(cfg) / 1e6:.1f} MB")
    cb = wl.codebooks(cfg)
    cb_dev = None
    inputs = []
    for i in range(nsets):
        si = wl.make_step_inputs(cfg, iset=i, cb=cb)
        di = DeviceInputs(si, dev, cb_dev)
        cb_dev = (di.pred_cb, di.succ_cb)
        inputs.append(di)
        del si
    runner = StepRunner(cfg, inputs, dev)
    log("capturing graphs")
    graphs = [runner.capture(i, step=i) for i in range(nsets)]
    torch.cuda.synchronize()

    for k in range(args.warmup):
        graphs[k % nsets].replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for k in range(args.steps):
        graphs[k % nsets].replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps

    # steps with the host waiting for each step's tokens (a serving loop that must see them)
    sync_steps = min(args.steps, 200)
    host_out = torch.empty((cfg.B, cfg.N + 1), dtype=torch.int32, pin_memory=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(sync_steps):
        graphs[k % nsets].replay()
        host_out.copy_(runner.out.out_tokens, non_blocking=True)
        torch.cuda.synchronize()
    ms_sync = (time.perf_counter() - t1) * 1e3 / sync_steps

    # Per-stage durations: each stage's calls (rotating over input sets and layers or sites,
    # as in the step) are captured back to back in one graph, and replays of that graph are
    # bracketed by HIP events on the stream it runs on; duration = elapsed / calls.
    def timed(fn, calls, replays=6):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(calls):
                fn(r)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / (replays * calls)
        del g
        return ms

    o = runner.out
    B, P, N, V = cfg.B, cfg.P, cfg.N, cfg.V
    reps = max(20, 4 * nsets)
    # calls per timing graph: every input set once, over every layer (or site)
    attn_calls = nsets * cfg.layers
    conv_calls = nsets * cfg.sites

    def attn_call(r):
        x = inputs[r % nsets]
        layer = (r // nsets) % cfg.layers
        d2.block_attn(x.q[layer], x.k_blk[layer], x.v_blk[layer], x.k_ring[layer],
                      x.v_ring[layer], x.ctx_len, cfg.W, out=o.attn[layer], ws=runner.ws_attn)

    def conv_call(r):
        x = inputs[r % nsets]
        s = (r // nsets) % cfg.sites
        d2.dynconv2(x.conv_x[s], x.conv_base[s], x.conv_delta[s], out=o.conv[s])

    def topk_call(r):
        x = inputs[r % nsets]
        d2.topk16(x.draft, B, N, 1, P * V, V, V, idx=o.cand_idx, val=o.cand_val, ws=runner.ws_topk)

    def select_call(r):
        x = inputs[r % nsets]
        d2.select(o.cand_idx, o.cand_val, x.gate, x.pred_cb, x.succ_cb, x.anchor, x.temperature,
                  cfg.seed, r, tokens=o.tokens, slot=o.slot, q=o.q, status=o.status,
                  ws=runner.ws_sel)

    def verify_call(r):
        x = inputs[r % nsets]
        d2.verify(x.target, B, N, P * V, V, V, o.tokens, o.cand_idx, o.q, o.slot, x.temperature,
                  cfg.seed, r, o.status, n_accept=o.n_accept, out_tokens=o.out_tokens,
                  ws=runner.ws_ver)

    runner.run(0, 0)
    torch.cuda.synchronize()
    stage_ms = {"block_attn": timed(attn_call, attn_calls), "dynconv2": timed(conv_call, conv_calls),
                "topk16": timed(topk_call, reps), "select": timed(select_call, reps),
                "verify": timed(verify_call, reps)}
    attn_ms = stage_ms["block_attn"]
    # accept counts of every input set's step (the verify timing graph rotates the sets)
    n_acc_sets = []
    for i in range(nsets):
        runner.run(i, i)
        n_acc_sets.append(o.n_accept.cpu().numpy().copy())
    runner.run(0, 0)
    torch.cuda.synchronize()
    # the timing graph visits every input set equally often: average their byte counts
    per_set = [attn_bytes_flops(cfg, x.ctx_len.cpu().numpy()) for x in inputs]
    a_bytes = sum(p[0] for p in per_set) / len(per_set)
    a_flops = sum(p[1] for p in per_set) / len(per_set)
    achieved = a_bytes / (attn_ms * 1e-3) / 1e9
    traffic = traffic_record(cfg.cfg)
    mean_acc = float(o.n_accept.float().mean().item())
    # The launch chain: kernel launches per step (attention is one kernel without splits,
    # two with; top-16, select and verify are two each; conv one per site) and the per-node
    # floor of a graph of one-element fills, the cheapest kernel node there is.
    attn_k = 1 + (d2.block_attn_workspace_bytes(B, P, cfg.Hq, cfg.Hkv, cfg.D, cfg.S, cfg.W,
                                                d2.BF16 if cfg.act_bf16 else d2.F32) > 0)
    launches = cfg.layers * attn_k + cfg.sites + 2 + 2 + 2
    tiny = torch.empty(1, device=dev)
    node_floor_ms = timed(lambda r: tiny.fill_(float(r)), 64)
    sb = stage_bytes(cfg, n_acc_sets)
    stage_hbm = {"block_attn": {"bytes_per_call": a_bytes, "achieved": achieved,
                                "frac": achieved / HBM_PEAK_GBS}}
    for k, nb in sb.items():
        gbs = nb / (stage_ms[k] * 1e-3) / 1e9
        stage_hbm[k] = {"bytes_per_call": float(nb), "achieved": gbs, "frac": gbs / HBM_PEAK_GBS}

    # The output-head projection fused with the top-16 (a call outside the step): the
    # drafter's rows 1..N against a synthetic V x C bf16 head, ~N(0, 1/C), generated on the
    # device from a fixed seed. Its algorithmic bytes are one read of the head and of the
    # hidden rows.
    lmhead = None
    if not args.no_lmhead:
        gen = torch.Generator(device=dev)
        gen.manual_seed(0xDF2 + cfg.cfg)
        head = torch.randn((V, cfg.C), generator=gen, device=dev, dtype=torch.float32)
        head = (head * (1.0 / math.sqrt(cfg.C))).to(torch.bfloat16)
        hid = torch.from_numpy(wl.head_hidden(cfg).view(np.int16)).view(torch.bfloat16).to(dev)
        lm_idx = torch.empty((B, N, 16), dtype=torch.int32, device=dev)
        lm_val = torch.empty((B, N, 16), dtype=torch.float32, device=dev)
        lm_ws = d2.workspace(d2.lmhead_topk16_workspace_bytes(B, N, V, cfg.C), dev)

        def lm_call(r):
            d2.lmhead_topk16(hid, B, N, 1, P * cfg.C, cfg.C, head, idx=lm_idx, val=lm_val, ws=lm_ws)

        lm_call(0)
        torch.cuda.synchronize()
        lm_ms = timed(lm_call, 4, replays=3)
        lm_bytes = float(V * cfg.C * 2 + B * N * cfg.C * 2 + B * N * 16 * 8)
        lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
        lmhead = {"call": "dflash2_lmhead_topk16", "rows": B * N, "width": cfg.C, "vocab": V,
                  "us_per_call": lm_ms * 1e3, "bytes_per_call": lm_bytes, "achieved": lm_gbs,
                  "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lm_gbs / HBM_PEAK_GBS}
        del head

    # The drafter projections beside the step (calls outside it): per conv site, the
    # coefficients from one projection of the sublayer's input (2G of the sublayer's 4G
    # weight rows), and once per step the selector gate from block rows 1..N. Weights are
    # N(0, 1/C) bf16, drawn on the device; three copies of every weight rotate so that the
    # replays read them from HBM rather than the last-level cache. Algorithmic bytes: one
    # read of the weight rows and the hidden rows, one write of the outputs.
    proj = None
    if not args.no_lmhead and cfg.act_bf16:
        G, C = cfg.C // 16, cfg.C
        gen = torch.Generator(device=dev)
        gen.manual_seed(0xDF2F + cfg.cfg)
        ncopy = 3
        subs = cfg.layers * 2

        def rand_w(rows):
            return (torch.randn((rows, C), generator=gen, device=dev) * (1.0 / math.sqrt(C))).to(torch.bfloat16)
        wconv = [[rand_w(4 * G) for _ in range(subs)] for _ in range(ncopy)]
        wgate = [rand_w(cfg.R) for _ in range(ncopy)]
        dbuf = torch.empty((cfg.sites, B, P, 2 * G), dtype=torch.float32, device=dev)
        gbuf = torch.empty((B, N, cfg.R), dtype=torch.float32, device=dev)
        ghid = torch.from_numpy(wl.head_hidden(cfg).view(np.int16)).view(torch.bfloat16).to(dev)
        c_ws = d2.workspace(d2.proj_workspace_bytes(B, P, 2 * G, C), dev)
        g_ws = d2.workspace(d2.proj_workspace_bytes(B, N, cfg.R, C), dev)

        def coeff_call(r):
            x = inputs[r % nsets]
            site = r % cfg.sites
            sub, half = site // 2, site % 2
            w = wconv[(r // cfg.sites) % ncopy][sub][half * 2 * G:(half + 1) * 2 * G]
            d2.proj(x.conv_x[site - half], B, P, 0, P * C, C, w, out=dbuf[site], ws=c_ws)

        def gate_call(r):
            d2.proj(ghid, B, N, 1, P * C, C, wgate[r % ncopy], out=gbuf, ws=g_ws)

        coeff_call(0)
        gate_call(0)
        torch.cuda.synchronize()
        c_ms = timed(coeff_call, ncopy * cfg.sites)
        g_ms = timed(gate_call, ncopy * 4)
        c_bytes = float(2 * G * C * 2 + B * P * C * 2 + B * P * 2 * G * 4)
        g_bytes = float(cfg.R * C * 2 + B * N * C * 2 + B * N * cfg.R * 4)
        proj = {"call": "dflash2_proj",
                "conv_coeffs": {"rows": B * P, "outputs": 2 * G, "width": C,
                                "calls_per_step": cfg.sites, "us_per_call": c_ms * 1e3,
                                "bytes_per_call": c_bytes,
                                "achieved": c_bytes / (c_ms * 1e-3) / 1e9},
                "selector_gate": {"rows": B * N, "outputs": cfg.R, "width": C,
                                  "calls_per_step": 1, "us_per_call": g_ms * 1e3,
                                  "bytes_per_call": g_bytes,
                                  "achieved": g_bytes / (g_ms * 1e-3) / 1e9},
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        del wconv, wgate

    # The selector over affine-Q8 codebooks (a call outside the step): the workload's bf16
    # codebooks converted to Q8 (groups of 64), same candidates, gates and anchors.
    select_q8 = None
    if not args.no_q8 and cfg.R % 64 == 0:
        pq, sq = wl.q8_quantize(wl.bf16_bits_to_f32(cb[0])), wl.q8_quantize(wl.bf16_bits_to_f32(cb[1]))

        def q8_dev(t):
            codes = torch.from_numpy(np.ascontiguousarray(t[0])).to(dev)
            sc = torch.from_numpy(t[1].view(np.int16)).view(torch.bfloat16).to(dev)
            bi = torch.from_numpy(t[2].view(np.int16)).view(torch.bfloat16).to(dev)
            return codes, sc, bi
        pq_d, sq_d = q8_dev(pq), q8_dev(sq)
        del pq, sq

        def q8_call(r):
            x = inputs[r % nsets]
            d2.select_q8(o.cand_idx, o.cand_val, x.gate, pq_d, sq_d, x.anchor, x.temperature,
                         cfg.seed, r, tokens=o.tokens, slot=o.slot, q=o.q, status=o.status,
                         ws=runner.ws_sel)

        q8_call(0)
        torch.cuda.synchronize()
        select_q8 = {"call": "dflash2_select_q8", "us_per_call": timed(q8_call, reps) * 1e3,
                     "bf16_select_us_per_call": stage_ms["select"] * 1e3}
        del pq_d, sq_d

    # The best-first draft tree over the selector lattice (a call outside the step),
    # budget 12 (the pages' tree budget), same candidates, gates and anchors.
    ddtree = None
    if not args.no_q8:
        tree_out = None

        def tree_call(r):
            nonlocal tree_out
            x = inputs[r % nsets]
            tree_out = d2.ddtree(o.cand_idx, o.cand_val, x.gate, x.pred_cb, x.succ_cb, x.anchor,
                                 12, out=tree_out, ws=runner.ws_sel)

        tree_call(0)
        torch.cuda.synchronize()
        ddtree = {"call": "dflash2_ddtree", "budget": 12, "us_per_call": timed(tree_call, reps) * 1e3}

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    result = {
        "metric": "draft+verify steps/s at batch B (vocab 248320)",
        "value": args.steps / wall,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act_bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "block": P, "vocab": V, "q_heads": cfg.Hq,
                   "kv_heads": cfg.Hkv, "head_dim": cfg.D, "window": cfg.W, "width": cfg.C,
                   "selector_rank": cfg.R, "layers": cfg.layers, "conv_sites": cfg.sites,
                   "input_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "dflash2_block_attn (split + combine)",
                     "bytes_per_launch": a_bytes, "avg_launch_us": attn_ms * 1e3,
                     "mfma_tflops": a_flops / (attn_ms * 1e-3) / 1e12,
                     "mfma_frac": a_flops / (attn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "stage_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "stage_hbm": stage_hbm,
        "step_event_ms": ev_ms / args.steps,
        "ms_per_step_host_sync": ms_sync,
        "mean_accepted": mean_acc,
        "launch_chain": {"kernels_per_step": launches, "graph_node_floor_us": node_floor_ms * 1e3,
                         "floor_us_per_step": launches * node_floor_ms * 1e3},
        "cpu_baseline": None,
        "lmhead_topk16": lmhead,
        "proj": proj,
        "select_q8": select_q8,
        "ddtree": ddtree,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
