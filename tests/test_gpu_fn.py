"""The library's exp_c and log_c on the GPU against the oracle's, bit for bit.

exp_c shapes every sampled selector walk (q over the 16 candidates) and, with log_c, the
draft tree's per-parent normalisation. Both are defined step by step, each step one
correctly rounded binary32 operation, so the GPU and the CPU must agree exactly:
  - exp_c on every binary32 input in [-87, -0] (the walk feeds it fl(fl(s - max) / T) <= 0),
    plus inputs below -87 and -inf, which both sides flush to 0;
  - log_c on every binary32 input in [1, 16] (the tree's normaliser Z = sum of 16 terms in
    (0, 1], one of them 1), plus every 97th normal positive binary32.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from helpers import DEV, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def _bits(f):
    return int(np.float32(f).view(np.uint32))


def _compare_range(d2, lo_bits, hi_bits, which, step=1):
    """Every step-th binary32 pattern in [lo_bits, hi_bits] (unsigned order), in chunks."""
    fn = orc.exp_c_array if which == 0 else orc.log_c_array
    total = 0
    for start in range(lo_bits, hi_bits + 1, CHUNK * step):
        end = min(start + CHUNK * step, hi_bits + 1)
        # the patterns as int32 (patterns >= 2^31 become negative int32), built on the device
        x64 = torch.arange(start, end, step, dtype=torch.int64, device=DEV)
        x64 = torch.where(x64 >= (1 << 31), x64 - (1 << 32), x64)
        x = x64.to(torch.int32).view(torch.float32)
        del x64
        got = d2.eval_fn(x, which).cpu().numpy()
        xh = x.cpu().numpy()
        want = fn(xh)
        bad = got.view(np.uint32) != want.view(np.uint32)
        if bad.any():
            i = int(np.argmax(bad))
            raise AssertionError(f"fn {which}: {int(bad.sum())} mismatches, first x={xh[i]!r} "
                                 f"(bits {xh.view(np.uint32)[i]:#x}): gpu {got[i]!r}, oracle {want[i]!r}")
        total += xh.size
    return total


def test_exp_c_every_input_in_domain(d2):
    lo, hi = _bits(-0.0), _bits(-87.0)
    say(f"exp_c exhaustive over [{lo:#x}, {hi:#x}]")
    n = _compare_range(d2, lo, hi, 0)
    assert n == hi - lo + 1


def test_exp_c_below_domain_flushes(d2):
    x = torch.tensor([-87.0001, -88.0, -100.0, -1e30, -3.4e38, float("-inf")],
                     dtype=torch.float32, device=DEV)
    say("exp_c below -87")
    got = d2.eval_fn(x, 0).cpu().numpy()
    want = orc.exp_c_array(x.cpu().numpy())
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.all(got == 0.0)


def test_log_c_every_input_in_1_16(d2):
    lo, hi = _bits(1.0), _bits(16.0)
    say(f"log_c exhaustive over [{lo:#x}, {hi:#x}]")
    n = _compare_range(d2, lo, hi, 1)
    assert n == hi - lo + 1


def test_log_c_sampled_normals(d2):
    say("log_c every 97th normal positive binary32")
    _compare_range(d2, _bits(1.1754944e-38), _bits(3.4028235e38), 1, step=97)
