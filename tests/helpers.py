"""Shared helpers of the GPU parity tests (device transfer, comparisons, announcements)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from block_drafter_draft_amd.workloads import bf16_bits_to_f32

DEV = "cuda:0"


def say(msg: str):
    """Name the case on stdout before a GPU step, so a lost box still tells which one ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> GPU tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


# unit roundoff of the output format: the exact result itself is off by up to this much
# relative once it is stored as bf16 (or f32)
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24


def assert_close_tol(got: np.ndarray, ref: np.ndarray, max_abs: float, rel_l2: float, what=""):
    """Elementwise |got - ref| <= max_abs + u * |ref| with u the unit roundoff of got's format
    (storing the exact value alone costs up to u * |ref|: 0.031 at |ref| = 8 for bf16), and
    ||got - ref|| / ||ref|| <= rel_l2."""
    g = as_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: nonfinite output"
    u = U_BF16 if got.dtype == np.uint16 else U_F32
    err = np.abs(g - r)
    excess = err - (max_abs + u * np.abs(r))
    mae = float(err.max()) if err.size else 0.0
    worst = float(excess.max()) if err.size else -1.0
    rl2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    assert worst <= 0 and rl2 <= rel_l2, (
        f"{what}: max-abs {mae:.3g} (bound {max_abs} + {u:.3g}|ref|, worst excess {worst:.3g}), "
        f"rel-L2 {rl2:.3g} (<= {rel_l2})")
    return mae, rl2


def assert_same_floats(got: np.ndarray, want: np.ndarray, what=""):
    """Bit-identical binary32 arrays, except that any NaN matches any NaN."""
    g = np.asarray(got, np.float32)
    w = np.asarray(want, np.float32)
    assert g.shape == w.shape, what
    gn, wn = np.isnan(g), np.isnan(w)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    gb, wb = g.view(np.uint32), w.view(np.uint32)
    bad = (~gn) & (gb != wb)
    assert not bad.any(), f"{what}: {bad.sum()} values differ, first at {np.argwhere(bad)[0]}"


def poison_like(shape, dtype):
    """An output buffer filled with 0xFF bytes, so unwritten entries cannot look right."""
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xFF)
    return t
