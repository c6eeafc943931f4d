"""dflash2_select_noalloc (the selector without a workspace, for callers that cannot
allocate) against dflash2_select: bit-exact tokens, slots, q and status on two calls in a
row, the second smaller, and its size limit."""
import numpy as np
import pytest
import torch

from block_drafter_draft_amd import workloads as wl
from helpers import DEV, poison_like, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from block_drafter_draft_amd import dflash2
    return dflash2


def _inputs(rng, B, N, V, R):
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(N)])
                     for _ in range(B)]).astype(np.int32)
    val = np.sort(rng.standard_normal((B, N, 16)).astype(np.float32) * 2 + 8, axis=2)[..., ::-1]
    gate = rng.standard_normal((B, N, R)).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    temp = np.where(np.arange(B) % 3 == 0, 0.0, 0.5 + (np.arange(B) % 5) * 0.25).astype(np.float32)
    return cand, np.ascontiguousarray(val), gate, anchor, temp


def test_select_noalloc_matches_select(d2):
    rng = np.random.default_rng(71)
    V, R = 50_000, 256
    A = to_dev(wl.to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * 0.25))
    Bc = to_dev(wl.to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * 0.25))
    cap = d2.select_noalloc_max_bytes()
    big_b = cap // (7 * 16 * 16 * 4)                      # the largest batch at N = 7
    for call, (B, N, step) in enumerate(((big_b, 7, 5), (3, 5, 6))):
        say(f"select_noalloc call {call} B={B} N={N}")
        assert d2.select_workspace_bytes(B, N) <= cap
        cand, val, gate, anchor, temp = _inputs(rng, B, N, V, R)
        args = [to_dev(a) for a in (cand, val, gate)] + [A, Bc] + [to_dev(anchor), to_dev(temp)]
        outs = []
        for fn in ("select", "select_noalloc"):
            tok = poison_like((B, N), torch.int32)
            slot = poison_like((B, N), torch.int32)
            q = poison_like((B, N, 16), torch.float32)
            st = poison_like((B,), torch.int32)
            getattr(d2, fn)(*args, 0xABC, step, tokens=tok, slot=slot, q=q, status=st)
            torch.cuda.synchronize()
            outs.append([to_host(t) for t in (tok, slot, q, st)])
        for a, b, name in zip(outs[0], outs[1], ("tokens", "slot", "q", "status")):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b), (call, name)
        assert (outs[1][0] >= 0).all()


def test_select_noalloc_refuses_oversized(d2):
    cap = d2.select_noalloc_max_bytes()
    N = 7
    B = cap // (N * 16 * 16 * 4) + 1
    x = torch.zeros(16, dtype=torch.int32, device=DEV)
    rc = d2.lib().dflash2_select_noalloc(*([d2._ptr(x)] * 5), 1000, 16, d2._ptr(x), d2._ptr(x),
                                         0, 0, B, N, *([d2._ptr(x)] * 4),
                                         d2._stream(None))
    assert rc == d2.EWORKSPACE
