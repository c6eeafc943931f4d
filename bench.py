#!/usr/bin/env python3
"""Draft+verify steps/s of the DFlash2 step on one MI355X.

One step is the whole hot path over one batch: per drafter layer the block attention and
its four dynamic-conv sites, then top-16 over the draft rows, the selector and the verify
(5 attention + 20 conv + 1 top-16 + 1 select + 1 verify calls of libdflash2). Inputs are
seeded synthetic tensors already resident in HBM; several input sets are rotated where one
set would fit in the 256 MiB last-level cache. Each step is one HIP-graph replay.

The headline is the serving-shaped workload: batch 64, mixed greedy and sampled sequences,
contexts in [2048, 131072]. It prints one JSON line with throughput (steps per wall-clock
second, and the median / p10 / p90 step time from HIP events between replays), a roofline
record for the dominant kernel (block attention: its algorithmic bytes over its average
duration, measured with HIP events on its stream), per-stage durations and HBM fractions,
acceptance statistics, verify alone on inputs that accept every proposal, the CPU oracle
timed on a bounded sample on one pinned host core, host and clock details, a measured copy
ceiling, and records for the calls beside the step (output head + top-16, projections, Q8
selector, draft tree). The batch-1 drafter workload and the batch-16 sampled workload are
measured in the same run as extra records.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
LLC_BYTES = 256 << 20           # last-level (MALL) cache
COLD_PASS = 3                   # a loop over distinct inputs reads this many LLCs per pass
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


def verify_bytes(cfg, n_acc, temps):
    """Algorithmic bytes of one verify call: per greedy sequence the n + 1 target rows the
    argmax chain needs, per sampled sequence the one row it draws from, plus the proposals'
    candidate lists and q."""
    tsz = 4 if cfg.target_kind == "probs" else (2 if cfg.act_bf16 else 4)
    rows = sum(1 if temps[b] > 0 else int(n_acc[b]) + 1 for b in range(cfg.B))
    return rows * cfg.V * tsz + cfg.B * cfg.N * 16 * 8


def stage_bytes(cfg, n_accept_sets):
    """Algorithmic bytes per call of each stage other than attention (what the method must
    move): conv reads x and writes out once, plus the coefficients and the base; top-16
    reads the N ranked logits rows once and writes the lists; the selector gathers the
    anchor's and each slot's predecessor rows of A and the slots' candidate rows of B,
    reads the gates and candidates; verify as in verify_bytes.
    n_accept_sets: the accept counts of each input set's step."""
    esz = 2 if cfg.act_bf16 else 4
    G = cfg.C // 16
    B, P, N, V, R = cfg.B, cfg.P, cfg.N, cfg.V, cfg.R
    conv = 2 * B * P * cfg.C * esz + B * P * 2 * G * 4 + 2 * cfg.C * 4
    topk = B * N * V * esz + B * N * 16 * 8
    select = B * ((1 + (N - 1) * 16 + N * 16) * R * 2 + N * R * 4 + N * 16 * 8)
    temps = cfg.temperatures()
    ver = [verify_bytes(cfg, n_acc, temps) for n_acc in n_accept_sets]
    return {"dynconv2": conv, "topk16": topk, "select": select, "verify": sum(ver) / len(ver)}


def traffic_record(workload):
    """HBM bytes per attention launch from the committed PMC summary, if it was taken on
    the current kernel source and this workload."""
    path = os.path.join(PROFILES, "block_attn_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "block_drafter_draft_amd", "csrc", "block_attn.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model}


def gpu_clocks():
    """Current sclk / mclk and the power cap as rocm-smi reports them (read before this
    process touches the GPU; a child process, bounded in time). Under a profiler, whose
    preloaded library has initialised the GPU already, no child program is started."""
    if any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return {"skipped": "running under a profiler"}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showmaxpower",
                            "--json"], capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout)
    except Exception as e:  # noqa: BLE001 - a report field, never fatal
        return {"error": f"{type(e).__name__}: {e}"[:200]}
    out = {}
    for card, fields in data.items():
        if not isinstance(fields, dict):
            continue
        keep = {k: v for k, v in fields.items()
                if any(s in k.lower() for s in ("sclk", "mclk", "power", "fclk"))}
        out[card] = keep
    return out


def cpu_baseline(cfg, seconds):
    """The oracle, as it stands, on one pinned host core: whole steps of the same workload,
    one sequence at a time (inputs drawn per sequence, the same values as in the batch), for
    about `seconds`; scaled to steps/s of the full batch."""
    import oracle as orc
    from block_drafter_draft_amd import workloads as wl
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})
    try:
        cb = wl.codebooks(cfg)
        B, P, N, V = cfg.B, cfg.P, cfg.N, cfg.V
        el = 0.0
        seqs_done = 0
        while True:
            b = seqs_done % B
            si = wl.make_step_inputs(cfg, iset=0, cb=cb, seqs=[b])
            t0 = time.perf_counter()
            for layer in range(cfg.layers):
                orc.block_attn(si.q[layer], si.k_blk[layer], si.v_blk[layer], si.k_ring[layer],
                               si.v_ring[layer], si.ctx_len, cfg.W)
            for s in range(cfg.sites):
                orc.dynconv2(si.conv_x[s], si.conv_base[s], si.conv_delta[s])
            ci, cv = orc.topk16(si.draft.reshape(-1), 1, N, 1, P * V, V, V)
            tok, slot, q, st = orc.select(ci, cv, si.gate, si.pred_cb, si.succ_cb, si.anchor,
                                          si.temperature, cfg.seed, 0)
            orc.verify(si.target.reshape(-1), 1, N, P * V, V, V, tok, ci, q, slot,
                       si.temperature, cfg.seed, 0, status=st)
            el += time.perf_counter() - t0
            seqs_done += 1
            if el >= seconds:
                break
    finally:
        os.sched_setaffinity(0, set(allowed))
    steps = seqs_done / B
    return {"value": steps / el, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{seqs_done} sequence(s) of full oracle steps ({steps:.3g} steps of batch "
                      f"{B}) in {el:.1f} s of oracle time on host core {core} (input drawing "
                      f"not timed)"}


def pct(xs, p):
    xs = sorted(xs)
    if not xs:
        return None
    k = (len(xs) - 1) * p / 100.0
    lo, hi = math.floor(k), math.ceil(k)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


class Bench:
    def __init__(self, args, dev):
        import torch
        self.torch = torch
        self.args = args
        self.dev = dev

    # Per-stage durations: each stage's calls (rotating over input sets and layers or sites,
    # as in the step) are captured back to back in one graph, and replays of that graph are
    # bracketed by HIP events on the stream it runs on; duration = elapsed / calls.
    def timed(self, fn, calls, replays=6):
        torch = self.torch
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

    def graph_kernels(self, runner):
        """Kernel nodes in a HIP graph of one step, counted through the HIP runtime
        (hipGraphGetNodes / hipGraphNodeGetType) on a graph kept for inspection."""
        import ctypes
        torch = self.torch
        try:
            g = torch.cuda.CUDAGraph(keep_graph=True)
            with torch.cuda.graph(g):
                runner.run(0, 0)
            torch.cuda.synchronize()
            hip = ctypes.CDLL("libamdhip64.so")
            graph = ctypes.c_void_p(g.raw_cuda_graph())
            n = ctypes.c_size_t(0)
            if hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) != 0:
                return None
            nodes = (ctypes.c_void_p * n.value)()
            if hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) != 0:
                return None
            kernels = 0
            kind = ctypes.c_int(-1)
            for nd in nodes:
                if hip.hipGraphNodeGetType(ctypes.c_void_p(nd), ctypes.byref(kind)) != 0:
                    return None
                kernels += kind.value == 0       # hipGraphNodeTypeKernel
            del g
            return kernels
        except Exception as e:  # noqa: BLE001 - a report field, never fatal
            log(f"graph node count unavailable: {type(e).__name__}: {e}")
            return None

    def copy_ceiling(self):
        """A plain device copy of 1 GiB: (read + written bytes) / time."""
        torch = self.torch
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=self.dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        a.record()
        for _ in range(reps):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        gbs = 2 * n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
        del src, dst
        torch.cuda.empty_cache()
        return {"kernel": "device copy (torch)", "bytes_per_copy": 2 * n, "achieved": gbs,
                "unit": "GB/s", "frac_of_peak": gbs / HBM_PEAK_GBS}

    def workload(self, wid, steps, warmup, full, copy_gbs=None):
        """Measure one workload. `full` adds the roofline, the launch chain, the all-accept
        verify diagnostic and the calls beside the step."""
        import numpy as np
        torch = self.torch
        from block_drafter_draft_amd import dflash2 as d2
        from block_drafter_draft_amd import workloads as wl
        from block_drafter_draft_amd.step import DeviceInputs, StepRunner
        args, dev = self.args, self.dev
        cfg = wl.CONFIGS[wid]
        nsets = args.sets or max(1, min(32, math.ceil(COLD_PASS * LLC_BYTES / set_bytes(cfg))))
        log(f"workload {cfg.cfg} ({cfg.name}), {nsets} input set(s) of "
            f"{set_bytes(cfg) / 1e6:.1f} MB")
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

        for k in range(warmup):
            graphs[k % nsets].replay()
        torch.cuda.synchronize()
        log(f"timing {steps} steps")
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record()
        for k in range(steps):
            graphs[k % nsets].replay()
            evs[k + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = [evs[k].elapsed_time(evs[k + 1]) for k in range(steps)]
        ev_total = evs[0].elapsed_time(evs[-1])

        o = runner.out
        B, P, N, V = cfg.B, cfg.P, cfg.N, cfg.V
        reps = max(20, 4 * nsets)
        attn_calls = nsets * cfg.layers
        conv_calls = nsets * cfg.sites

        def attn_call(r):
            x = inputs[r % nsets]
            layer = (r // nsets) % cfg.layers
            d2.block_attn(x.q[layer], x.k_blk[layer], x.v_blk[layer], x.k_ring[layer],
                          x.v_ring[layer], x.ctx_len, cfg.W, out=o.attn[layer],
                          ws=runner.ws_attn)

        # accept counts of every input set's step, with the counter each graph uses
        n_acc_sets = []
        for i in range(nsets):
            runner.run(i, i)
            n_acc_sets.append(o.n_accept.cpu().numpy().copy())
        runner.run(0, 0)
        torch.cuda.synchronize()
        sb = stage_bytes(cfg, n_acc_sets)
        sb["verify"] = verify_bytes(cfg, n_acc_sets[0], cfg.temperatures())  # timed on set 0

        # In the step every stage reads its inputs from HBM: the step's working set is many
        # times the last-level cache. So that a loop of one stage's calls does the same,
        # each loop cycles through enough distinct copies of that stage's inputs (stacked,
        # the given sets first, then clones of them in turn) to read COLD_PASS times the
        # cache per pass.
        def n_cold(per_call_bytes):
            return max(1, math.ceil(COLD_PASS * LLC_BYTES / max(per_call_bytes, 1)))

        def stack(srcs, n):
            base = torch.stack(srcs)
            reps = -(-n // len(srcs))
            return base.repeat(reps, *([1] * (base.dim() - 1)))[:n].contiguous()

        sites = cfg.sites
        nc = n_cold(sb["dynconv2"])
        cx = stack([x.conv_x[s] for x in inputs for s in range(sites)], nc)
        cbase = stack([x.conv_base[s] for x in inputs for s in range(sites)], nc)
        cdel = stack([x.conv_delta[s] for x in inputs for s in range(sites)], nc)

        def conv_call(r):
            d2.dynconv2(cx[r % nc], cbase[r % nc], cdel[r % nc], out=o.conv[r % sites])

        nt = n_cold(sb["topk16"])
        drafts = stack([x.draft for x in inputs], nt)

        def topk_call(r):
            d2.topk16(drafts[r % nt], B, N, 1, P * V, V, V, idx=o.cand_idx, val=o.cand_val,
                      ws=runner.ws_topk)

        # the selector gathers codebook rows chosen by the candidates: copies of the
        # codebooks, and per call the candidate indices shifted by a multiple of a stride,
        # so that each call gathers other rows
        ncb = n_cold(inputs[0].pred_cb.numel() * inputs[0].pred_cb.element_size() * 2)
        cbs = [(inputs[0].pred_cb, inputs[0].succ_cb)] + [
            (inputs[0].pred_cb.clone(), inputs[0].succ_cb.clone()) for _ in range(ncb - 1)]
        ns = n_cold(sb["select"])
        cand0 = o.cand_idx.clone()
        shift = 7919 * torch.arange(ns, device=dev, dtype=torch.int64).view(-1, 1, 1, 1)
        cands = ((cand0.to(torch.int64).unsqueeze(0) + shift) % V).to(torch.int32)

        def select_call(r):
            x = inputs[r % nsets]
            pc, sc = cbs[r % ncb]
            d2.select(cands[r % ns], o.cand_val, x.gate, pc, sc, x.anchor,
                      x.temperature, cfg.seed, r, tokens=o.tokens, slot=o.slot, q=o.q,
                      status=o.status, ws=runner.ws_sel)

        nv = n_cold(sb["verify"])
        targets = stack([inputs[0].target], nv)

        def verify_call(r):
            x = inputs[0]
            d2.verify(targets[r % nv], B, N, P * V, V, V, o.tokens, o.cand_idx, o.q, o.slot,
                      x.temperature, cfg.seed, r, o.status, n_accept=o.n_accept,
                      out_tokens=o.out_tokens, ws=runner.ws_ver)

        torch.cuda.synchronize()
        stage_ms = {"block_attn": self.timed(attn_call, attn_calls),
                    "dynconv2": self.timed(conv_call, max(nc, conv_calls)),
                    "topk16": self.timed(topk_call, max(nt, reps)),
                    "select": self.timed(select_call, max(ns, ncb, reps))}
        runner.run(0, 0)  # verify reads set 0's own proposals
        stage_ms["verify"] = self.timed(verify_call, max(nv, reps))
        cold_copies = {"dynconv2": nc, "topk16": nt, "select": [ns, ncb], "verify": nv}
        del cx, cbase, cdel, drafts, cbs, cands, targets
        attn_ms = stage_ms["block_attn"]
        per_set = [attn_bytes_flops(cfg, x.ctx_len.cpu().numpy()) for x in inputs]
        a_bytes = sum(p[0] for p in per_set) / len(per_set)
        a_flops = sum(p[1] for p in per_set) / len(per_set)
        achieved = a_bytes / (attn_ms * 1e-3) / 1e9

        stage_hbm = {"block_attn": {"bytes_per_call": a_bytes, "achieved": achieved,
                                    "frac": achieved / HBM_PEAK_GBS}}
        for k, nb in sb.items():
            gbs = nb / (stage_ms[k] * 1e-3) / 1e9
            stage_hbm[k] = {"bytes_per_call": float(nb), "achieved": gbs,
                            "frac": gbs / HBM_PEAK_GBS}
        if copy_gbs:
            for v in stage_hbm.values():
                v["frac_of_copy"] = v["achieved"] / copy_gbs

        # Acceptance ("DFlash 2 on Qwen3.8-27B-FP8", methodology: acceptance length is one
        # plus accepted over drafts; the vLLM PR reports per-position accepted counts).
        temps = cfg.temperatures()
        allacc = np.concatenate(n_acc_sets)
        modes = np.tile(temps > 0, nsets)
        per_pos = [int((allacc > k).sum()) for k in range(N)]
        acceptance = {
            "blocks": int(allacc.size),
            "mean_accepted": float(allacc.mean()),
            "acceptance_length": 1.0 + float(allacc.mean()),
            "accepted_at_position": per_pos,
            "greedy_mean_accepted": float(allacc[~modes].mean()) if (~modes).any() else None,
            "sampled_mean_accepted": float(allacc[modes].mean()) if modes.any() else None,
        }

        rec = {
            "workload": cfg.name, "batch": B, "input_sets": nsets,
            "value": steps / wall, "unit": "steps/s", "ms_per_step": wall * 1e3 / steps,
            "step_ms": {"median": pct(step_ms, 50), "p10": pct(step_ms, 10),
                        "p90": pct(step_ms, 90), "event_mean": ev_total / steps},
            "stage_us": {k: v * 1e3 for k, v in stage_ms.items()},
            "stage_cold_copies": cold_copies,
            "stage_hbm": stage_hbm,
            "acceptance": acceptance,
        }
        if not full:
            del graphs, runner, inputs
            torch.cuda.empty_cache()
            return rec, cfg

        # steps with the host waiting for each step's tokens (a serving loop that must see them)
        sync_steps = min(steps, 200)
        host_out = torch.empty((B, N + 1), dtype=torch.int32, pin_memory=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for k in range(sync_steps):
            graphs[k % nsets].replay()
            host_out.copy_(runner.out.out_tokens, non_blocking=True)
            torch.cuda.synchronize()
        rec["ms_per_step_host_sync"] = (time.perf_counter() - t1) * 1e3 / sync_steps

        traffic = traffic_record(cfg.cfg)
        rec["roofline"] = {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "frac_of_copy": achieved / copy_gbs if copy_gbs else None,
            "kernel": "dflash2_block_attn", "bytes_per_launch": a_bytes,
            "avg_launch_us": attn_ms * 1e3,
            "mfma_tflops": a_flops / (attn_ms * 1e-3) / 1e12,
            "mfma_frac": a_flops / (attn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}

        # The launch chain: kernel launches per step and the per-node floor of a HIP graph
        # of one-element fills, the cheapest kernel node there is.
        rec["launch_chain"] = {"kernels_per_step": self.graph_kernels(runner)}
        tiny = torch.empty(1, device=dev)
        node_floor_ms = self.timed(lambda r: tiny.fill_(float(r)), 64)
        rec["launch_chain"]["graph_node_floor_us"] = node_floor_ms * 1e3
        kps = rec["launch_chain"]["kernels_per_step"]
        rec["launch_chain"]["floor_us_per_step"] = kps * node_floor_ms * 1e3 if kps else None

        # Verify alone where every proposal is accepted: greedy sequences then need all
        # N + 1 rows, sampled ones the bonus row. The other extreme from the step's targets.
        rec["verify_all_accept"] = None if args.no_all_accept else self._all_accept(cfg, wl, runner, reps, temps)
        if not args.no_lmhead:
            rec["lmhead_topk16"] = self._lmhead(cfg, wl)
            rec["proj"] = self._proj(cfg, wl, inputs, nsets) if cfg.act_bf16 else None
        if not args.no_q8:
            rec["select_q8"] = self._q8(cfg, wl, cb, inputs, runner, nsets, reps,
                                        stage_ms["select"])
            rec["ddtree"] = self._ddtree(cfg, inputs, runner, nsets, reps)
        del graphs, runner, inputs
        torch.cuda.empty_cache()
        return rec, cfg

    def _all_accept(self, cfg, wl, runner, reps, temps):
        import numpy as np
        torch, dev = self.torch, self.dev
        from block_drafter_draft_amd import dflash2 as d2
        B, P, N, V = cfg.B, cfg.P, cfg.N, cfg.V
        vi = wl.all_accept_verify_inputs(cfg)
        vt = torch.from_numpy(vi.target.view(np.int16) if vi.target.dtype == np.uint16
                              else vi.target)
        vt = (vt.view(torch.bfloat16) if vi.target.dtype == np.uint16 else vt).to(dev)
        vtok, vci, vq, vsl, vT = (torch.from_numpy(a).to(dev) for a in
                                  (vi.tokens, vi.cand_idx, vi.q, vi.slot, vi.temperature))
        vst = torch.zeros(B, dtype=torch.int32, device=dev)
        va_n = torch.empty(B, dtype=torch.int32, device=dev)
        va_out = torch.empty((B, N + 1), dtype=torch.int32, device=dev)

        def verify_acc_call(r):
            d2.verify(vt, B, N, P * V, V, V, vtok, vci, vq, vsl, vT, cfg.seed, r, vst,
                      n_accept=va_n, out_tokens=va_out, ws=runner.ws_ver)

        verify_acc_call(0)
        torch.cuda.synchronize()
        n_all = va_n.cpu().numpy()
        va_ms = self.timed(verify_acc_call, reps)
        va_bytes = verify_bytes(cfg, n_all, temps)
        return {
            "mean_accepted": float(n_all.mean()), "us_per_call": va_ms * 1e3,
            "bytes_per_call": float(va_bytes),
            "achieved": va_bytes / (va_ms * 1e-3) / 1e9,
            "frac": va_bytes / (va_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


    # The output-head projection fused with the top-16 (a call outside the step): the
    # drafter's rows 1..N against a synthetic V x C bf16 head, ~N(0, 1/C), generated on the
    # device from a fixed seed. Its algorithmic bytes are one read of the head and of the
    # hidden rows.
    def _lmhead(self, cfg, wl):
        import numpy as np
        torch, dev = self.torch, self.dev
        from block_drafter_draft_amd import dflash2 as d2
        B, P, N, V = cfg.B, cfg.P, cfg.N, cfg.V
        gen = torch.Generator(device=dev)
        gen.manual_seed(0xDF2 + cfg.cfg)
        head = torch.randn((V, cfg.C), generator=gen, device=dev, dtype=torch.float32)
        head = (head * (1.0 / math.sqrt(cfg.C))).to(torch.bfloat16)
        hid = torch.from_numpy(wl.head_hidden(cfg).view(np.int16)).view(torch.bfloat16).to(dev)
        lm_idx = torch.empty((B, N, 16), dtype=torch.int32, device=dev)
        lm_val = torch.empty((B, N, 16), dtype=torch.float32, device=dev)
        lm_ws = d2.workspace(d2.lmhead_topk16_workspace_bytes(B, N, V, cfg.C), dev)

        def lm_call(r):
            d2.lmhead_topk16(hid, B, N, 1, P * cfg.C, cfg.C, head, idx=lm_idx, val=lm_val,
                             ws=lm_ws)

        lm_call(0)
        torch.cuda.synchronize()
        lm_ms = self.timed(lm_call, 4, replays=3)
        lm_bytes = float(V * cfg.C * 2 + B * N * cfg.C * 2 + B * N * 16 * 8)
        lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
        del head
        return {"call": "dflash2_lmhead_topk16", "rows": B * N, "width": cfg.C, "vocab": V,
                "us_per_call": lm_ms * 1e3, "bytes_per_call": lm_bytes, "achieved": lm_gbs,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lm_gbs / HBM_PEAK_GBS}

    # The drafter projections beside the step (calls outside it): per conv site, the
    # coefficients from one projection of the sublayer's input (2G of the sublayer's 4G
    # weight rows), and once per step the selector gate from block rows 1..N. Weights are
    # N(0, 1/C) bf16, drawn on the device; three copies of every weight rotate so that the
    # replays read them from HBM rather than the last-level cache. Algorithmic bytes: one
    # read of the weight rows and the hidden rows, one write of the outputs.
    def _proj(self, cfg, wl, inputs, nsets):
        import numpy as np
        torch, dev = self.torch, self.dev
        from block_drafter_draft_amd import dflash2 as d2
        B, P, N = cfg.B, cfg.P, cfg.N
        G, C = cfg.C // 16, cfg.C
        gen = torch.Generator(device=dev)
        gen.manual_seed(0xDF2F + cfg.cfg)
        ncopy = 3
        subs = cfg.layers * 2

        def rand_w(rows):
            return (torch.randn((rows, C), generator=gen, device=dev)
                    * (1.0 / math.sqrt(C))).to(torch.bfloat16)
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
        c_ms = self.timed(coeff_call, ncopy * cfg.sites)
        g_ms = self.timed(gate_call, ncopy * 4)
        c_bytes = float(2 * G * C * 2 + B * P * C * 2 + B * P * 2 * G * 4)
        g_bytes = float(cfg.R * C * 2 + B * N * C * 2 + B * N * cfg.R * 4)
        del wconv, wgate
        return {"call": "dflash2_proj",
                "conv_coeffs": {"rows": B * P, "outputs": 2 * G, "width": C,
                                "calls_per_step": cfg.sites, "us_per_call": c_ms * 1e3,
                                "bytes_per_call": c_bytes,
                                "achieved": c_bytes / (c_ms * 1e-3) / 1e9},
                "selector_gate": {"rows": B * N, "outputs": cfg.R, "width": C,
                                  "calls_per_step": 1, "us_per_call": g_ms * 1e3,
                                  "bytes_per_call": g_bytes,
                                  "achieved": g_bytes / (g_ms * 1e-3) / 1e9},
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}

    # The selector over affine-Q8 codebooks (a call outside the step): the workload's bf16
    # codebooks converted to Q8 (groups of 64), same candidates, gates and anchors.
    def _q8(self, cfg, wl, cb, inputs, runner, nsets, reps, bf16_select_ms):
        import numpy as np
        torch, dev = self.torch, self.dev
        from block_drafter_draft_amd import dflash2 as d2
        if cfg.R % 64:
            return None
        o = runner.out
        pq = wl.q8_quantize(wl.bf16_bits_to_f32(cb[0]))
        sq = wl.q8_quantize(wl.bf16_bits_to_f32(cb[1]))

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
        return {"call": "dflash2_select_q8", "us_per_call": self.timed(q8_call, reps) * 1e3,
                "bf16_select_us_per_call": bf16_select_ms * 1e3}

    # The best-first draft tree over the selector lattice (a call outside the step),
    # budget 12 (the pages' tree budget), same candidates, gates and anchors.
    def _ddtree(self, cfg, inputs, runner, nsets, reps):
        from block_drafter_draft_amd import dflash2 as d2
        o = runner.out
        tree_out = None

        def tree_call(r):
            nonlocal tree_out
            x = inputs[r % nsets]
            tree_out = d2.ddtree(o.cand_idx, o.cand_val, x.gate, x.pred_cb, x.succ_cb, x.anchor,
                                 12, out=tree_out, ws=runner.ws_sel)

        tree_call(0)
        self.torch.cuda.synchronize()
        return {"call": "dflash2_ddtree", "budget": 12,
                "us_per_call": self.timed(tree_call, reps) * 1e3}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="input configuration of the headline (default: batch 64, serving)")
    ap.add_argument("--extra", default="2,3",
                    help="comma-separated workloads also measured in this run ('' for none)")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets to rotate (default: enough to exceed the last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lmhead", action="store_true",
                    help="skip the separate output-head + top-16 and projection measurements")
    ap.add_argument("--no-q8", action="store_true",
                    help="skip the separate Q8-selector and draft-tree measurements")
    ap.add_argument("--no-all-accept", action="store_true",
                    help="skip verify on all-accept inputs (keeps per-dispatch profiles of the "
                         "step's own verify calls unmixed)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the DFlash2 step shards by sequence with no "
              "exchange, and no multi-GPU path is implemented (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    clocks = gpu_clocks()          # before this process initialises the GPU
    host = host_info()

    import torch

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = "cuda:0"
    bench = Bench(args, dev)
    copy = bench.copy_ceiling()
    log(f"device copy {copy['achieved']:.0f} GB/s")
    rec, cfg = bench.workload(args.workload, args.steps, args.warmup, True, copy["achieved"])
    extra = {}
    for w in [int(x) for x in args.extra.split(",") if x.strip()]:
        if w == args.workload:
            continue
        r, c = bench.workload(w, args.steps, args.warmup, False, copy["achieved"])
        extra[c.name] = r

    result = {
        "metric": "draft+verify steps/s at batch B (vocab 248320)",
        "value": rec["value"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act_bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "block": cfg.P, "vocab": cfg.V,
                   "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.D,
                   "window": cfg.W, "width": cfg.C, "selector_rank": cfg.R,
                   "layers": cfg.layers, "conv_sites": cfg.sites,
                   "input_sets": rec["input_sets"]},
        "roofline": rec["roofline"],
        "step_ms": rec["step_ms"],
        "ms_per_step_host_sync": rec["ms_per_step_host_sync"],
        "stage_us": rec["stage_us"],
        "stage_cold_copies": rec["stage_cold_copies"],
        "stage_hbm": rec["stage_hbm"],
        "acceptance": rec["acceptance"],
        "mean_accepted": rec["acceptance"]["mean_accepted"],
        "verify_all_accept": rec["verify_all_accept"],
        "launch_chain": rec["launch_chain"],
        "copy_ceiling": copy,
        "host": host,
        "gpu_clocks": clocks,
        "cpu_baseline": None,
        "lmhead_topk16": rec.get("lmhead_topk16"),
        "proj": rec.get("proj"),
        "select_q8": rec.get("select_q8"),
        "ddtree": rec.get("ddtree"),
        "other_workloads": extra,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
