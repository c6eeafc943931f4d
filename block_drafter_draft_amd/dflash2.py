"""ctypes binding of libdflash2 (the C ABI in include/dflash2.h).

Argument marshalling only: every function takes torch tensors that already live on the
GPU, checks their dtypes and shapes against the call, and passes raw pointers, sizes and
the current HIP stream to the library. No step of the computation runs here, and there is
no fallback: importing this module raises if libdflash2.so has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash2.so")

BF16 = 0
F32 = 1

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
EWORKSPACE = -3
EHIP = -4

ST_NONFINITE = 1
ST_BADTOKEN = 2
ST_ZEROMASS = 4
ST_BADPROB = 8
ST_BADTEMP = 16
ST_RINGLOST = 32
ST_BADCOUNT = 64

K = 16

# name -> (argtypes, restype); mirrors include/dflash2.h
_vp, _i32, _i64, _u64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "dflash2_block_attn": ([_vp] * 7 + [_i32] * 7 + [_f32, _i32, _vp, _sz, _vp], _i32),
    "dflash2_block_attn_workspace_bytes": ([_i32] * 8, _sz),
    "dflash2_dynconv2": ([_vp] * 4 + [_i32] * 5 + [_vp], _i32),
    "dflash2_topk16": ([_vp, _i32, _i32, _i32, _i32, _i64, _i64, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "dflash2_topk16_workspace_bytes": ([_i32] * 4, _sz),
    "dflash2_lmhead_topk16": ([_vp, _i64, _i64, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "dflash2_lmhead_topk16_workspace_bytes": ([_i32] * 4, _sz),
    "dflash2_proj": ([_vp, _i64, _i64, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _i64, _i64, _vp, _sz, _vp], _i32),
    "dflash2_proj_workspace_bytes": ([_i32] * 4, _sz),
    "dflash2_select": ([_vp] * 5 + [_i32, _i32, _vp, _vp, _u64, _u64, _i32, _i32] + [_vp] * 5 + [_sz, _vp], _i32),
    "dflash2_select_workspace_bytes": ([_i32] * 2, _sz),
    "dflash2_select_noalloc": ([_vp] * 5 + [_i32, _i32, _vp, _vp, _u64, _u64, _i32, _i32] + [_vp] * 5, _i32),
    "dflash2_select_noalloc_max_bytes": ([], _sz),
    "dflash2_ddtree": ([_vp] * 5 + [_i32, _i32, _vp, _i32, _i32, _i32] + [_vp] * 7 + [_sz, _vp], _i32),
    "dflash2_ddtree_workspace_bytes": ([_i32] * 2, _sz),
    "dflash2_select_q8": ([_vp] * 9 + [_i32, _i32, _vp, _vp, _u64, _u64, _i32, _i32] + [_vp] * 5 + [_sz, _vp], _i32),
    "dflash2_verify": ([_vp, _i32, _i64, _i64, _i32] + [_vp] * 5 + [_u64, _u64, _i32, _i32] + [_vp] * 4 + [_sz, _vp], _i32),
    "dflash2_verify_workspace_bytes": ([_i32] * 4, _sz),
    "dflash2_ring_update": ([_vp] * 7 + [_i32] * 7 + [_vp, _vp], _i32),
    "dflash2_eval_fn": ([_vp, _vp, _i64, _i32, _vp], _i32),
    "dflash2_status_string": ([_i32], ctypes.c_char_p),
    "dflash2_version": ([], _i32),
}


class DFlash2Error(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m block_drafter_draft_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (argt, rest) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = rest
    return lib


_lib = _load()


def lib():
    return _lib


def status_string(code: int) -> str:
    return _lib.dflash2_status_string(code).decode()


def _check(rc: int, what: str):
    if rc != OK:
        raise DFlash2Error(f"{what}: {status_string(rc)} ({rc})")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("dflash2 tensors must be on the GPU")


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("dflash2 tensors must be contiguous")


def workspace(nbytes: int, device) -> torch.Tensor:
    """A byte buffer for the ws argument (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------------------


def block_attn_workspace_bytes(B, P, Hq, Hkv, D, S, W, dtype) -> int:
    return int(_lib.dflash2_block_attn_workspace_bytes(B, P, Hq, Hkv, D, S, W, dtype))


def block_attn(q, k_blk, v_blk, k_ring, v_ring, ctx_len, W, scale=None, out=None, ws=None,
               stream=None):
    _dev(q, k_blk, v_blk, k_ring, v_ring, ctx_len)
    _contig(q, k_blk, v_blk, k_ring, v_ring, ctx_len)
    B, P, Hq, D = q.shape
    S, Hkv = k_ring.shape[1], k_ring.shape[2]
    dt = _dtype(q)
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = block_attn_workspace_bytes(B, P, Hq, Hkv, D, S, W, dt)
    if ws is None and need:
        ws = workspace(need, q.device)
    rc = _lib.dflash2_block_attn(_ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_ring), _ptr(v_ring),
                                 _ptr(ctx_len), _ptr(out), B, P, Hq, Hkv, D, S, W, float(scale),
                                 dt, _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream))
    _check(rc, "dflash2_block_attn")
    return out


def dynconv2(x, base, delta, out=None, group=16, stream=None):
    _dev(x, base, delta)
    _contig(x, base, delta)
    B, P, C = x.shape
    if out is None:
        out = torch.empty_like(x)
    rc = _lib.dflash2_dynconv2(_ptr(x), _ptr(base), _ptr(delta), _ptr(out), B, P, C, group,
                               _dtype(x), _stream(stream))
    _check(rc, "dflash2_dynconv2")
    return out


def topk16_workspace_bytes(B, N, V, dtype) -> int:
    return int(_lib.dflash2_topk16_workspace_bytes(B, N, V, dtype))


def topk16(scores, B, N, row0, seq_stride, row_stride, V, idx=None, val=None, ws=None,
           stream=None):
    """Top-16 of rows row0..row0+N-1 of each sequence; strides in elements."""
    _dev(scores)
    dt = _dtype(scores)
    if idx is None:
        idx = torch.empty((B, N, K), dtype=torch.int32, device=scores.device)
    if val is None:
        val = torch.empty((B, N, K), dtype=torch.float32, device=scores.device)
    if ws is None:
        ws = workspace(topk16_workspace_bytes(B, N, V, dt), scores.device)
    rc = _lib.dflash2_topk16(_ptr(scores), dt, B, N, row0, seq_stride, row_stride, V, _ptr(idx),
                             _ptr(val), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "dflash2_topk16")
    return idx, val


def lmhead_topk16_workspace_bytes(B, N, V, C) -> int:
    return int(_lib.dflash2_lmhead_topk16_workspace_bytes(B, N, V, C))


def lmhead_topk16(hidden, B, N, row0, seq_stride, row_stride, weight, idx=None, val=None,
                  ws=None, stream=None):
    """Top-16 of hidden-row x output-head logits; hidden bf16 rows addressed by element
    strides, weight bf16 [V, C]."""
    _dev(hidden, weight)
    _contig(weight)
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    V, C = weight.shape
    dev = hidden.device
    if idx is None:
        idx = torch.empty((B, N, K), dtype=torch.int32, device=dev)
    if val is None:
        val = torch.empty((B, N, K), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(lmhead_topk16_workspace_bytes(B, N, V, C), dev)
    rc = _lib.dflash2_lmhead_topk16(_ptr(hidden), seq_stride, row_stride, row0, _ptr(weight), C,
                                    V, B, N, _ptr(idx), _ptr(val), _ptr(ws), ws.numel(),
                                    _stream(stream))
    _check(rc, "dflash2_lmhead_topk16")
    return idx, val


def proj_workspace_bytes(B, N, O, C) -> int:
    return int(_lib.dflash2_proj_workspace_bytes(B, N, O, C))


def proj(hidden, B, N, row0, seq_stride, row_stride, weight, out=None, out_seq_stride=None,
         out_row_stride=None, ws=None, stream=None):
    """out[b, r, o] = sum_c hidden[b*seq_stride + (row0+r)*row_stride + c] * weight[o, c] in
    binary32; hidden bf16 rows addressed by element strides, weight bf16 [O, C]. With no
    out given, a new f32 [B, N, O] tensor."""
    _dev(hidden, weight)
    _contig(weight)
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    O, C = weight.shape
    if out is None:
        out = torch.empty((B, N, O), dtype=torch.float32, device=hidden.device)
        out_seq_stride, out_row_stride = N * O, O
    else:
        _dev(out)
        if out.dtype != torch.float32:
            raise TypeError("out must be float32")
        if out_seq_stride is None or out_row_stride is None:
            _contig(out)
            out_seq_stride, out_row_stride = N * O, O
    need = proj_workspace_bytes(B, N, O, C)
    if ws is None and need:
        ws = workspace(need, hidden.device)
    rc = _lib.dflash2_proj(_ptr(hidden), seq_stride, row_stride, row0, _ptr(weight), C, O, B, N,
                           _ptr(out), out_seq_stride, out_row_stride, _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "dflash2_proj")
    return out


def eval_fn(x, which, out=None, stream=None):
    """The library's exp_c (which 0, x <= 0) or log_c (which 1, x > 0), elementwise, on a
    contiguous f32 tensor."""
    _dev(x)
    _contig(x)
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    if out is None:
        out = torch.empty_like(x)
    rc = _lib.dflash2_eval_fn(_ptr(x), _ptr(out), x.numel(), which, _stream(stream))
    _check(rc, "dflash2_eval_fn")
    return out


def select_workspace_bytes(B, N) -> int:
    return int(_lib.dflash2_select_workspace_bytes(B, N))


def select(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, temperature, seed, step,
           tokens=None, slot=None, q=None, status=None, ws=None, stream=None):
    _dev(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, temperature)
    _contig(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, temperature)
    B, N, _ = cand_idx.shape
    V, R = pred_cb.shape
    if pred_cb.dtype != torch.bfloat16 or succ_cb.dtype != torch.bfloat16:
        raise TypeError("codebooks must be bfloat16")
    dev = cand_idx.device
    tokens = torch.empty((B, N), dtype=torch.int32, device=dev) if tokens is None else tokens
    slot = torch.empty((B, N), dtype=torch.int32, device=dev) if slot is None else slot
    q = torch.empty((B, N, K), dtype=torch.float32, device=dev) if q is None else q
    status = torch.empty((B,), dtype=torch.int32, device=dev) if status is None else status
    if ws is None:
        ws = workspace(select_workspace_bytes(B, N), dev)
    rc = _lib.dflash2_select(_ptr(cand_idx), _ptr(cand_val), _ptr(gate), _ptr(pred_cb),
                             _ptr(succ_cb), V, R, _ptr(anchor), _ptr(temperature),
                             int(seed) & (2**64 - 1), int(step) & (2**64 - 1), B, N,
                             _ptr(tokens), _ptr(slot), _ptr(q), _ptr(status), _ptr(ws),
                             ws.numel(), _stream(stream))
    _check(rc, "dflash2_select")
    return tokens, slot, q, status


def select_noalloc_max_bytes() -> int:
    return int(_lib.dflash2_select_noalloc_max_bytes())


def select_noalloc(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, temperature, seed, step,
                   tokens, slot, q, status, stream=None):
    """dflash2_select without a workspace (the library's static lattice); every output is
    caller-provided so that the call allocates nothing."""
    _dev(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, temperature, tokens, slot, q, status)
    _contig(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, temperature, tokens, slot, q,
            status)
    B, N, _ = cand_idx.shape
    V, R = pred_cb.shape
    if pred_cb.dtype != torch.bfloat16 or succ_cb.dtype != torch.bfloat16:
        raise TypeError("codebooks must be bfloat16")
    rc = _lib.dflash2_select_noalloc(_ptr(cand_idx), _ptr(cand_val), _ptr(gate), _ptr(pred_cb),
                                     _ptr(succ_cb), V, R, _ptr(anchor), _ptr(temperature),
                                     int(seed) & (2**64 - 1), int(step) & (2**64 - 1), B, N,
                                     _ptr(tokens), _ptr(slot), _ptr(q), _ptr(status),
                                     _stream(stream))
    _check(rc, "dflash2_select_noalloc")
    return tokens, slot, q, status


def ddtree(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, budget, out=None, ws=None,
           stream=None):
    """Best-first draft tree; returns (parent, depth, slot, token, score, status)."""
    _dev(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor)
    _contig(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor)
    B, N, _ = cand_idx.shape
    V, R = pred_cb.shape
    if pred_cb.dtype != torch.bfloat16 or succ_cb.dtype != torch.bfloat16:
        raise TypeError("codebooks must be bfloat16")
    dev = cand_idx.device
    if out is None:
        out = tuple(torch.empty((B, budget), dtype=torch.int32, device=dev) for _ in range(4)) + (
            torch.empty((B, budget), dtype=torch.float32, device=dev),
            torch.empty((B,), dtype=torch.int32, device=dev))
    if ws is None:
        ws = workspace(int(_lib.dflash2_ddtree_workspace_bytes(B, N)), dev)
    rc = _lib.dflash2_ddtree(_ptr(cand_idx), _ptr(cand_val), _ptr(gate), _ptr(pred_cb),
                             _ptr(succ_cb), V, R, _ptr(anchor), B, N, budget,
                             *[_ptr(t) for t in out], _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "dflash2_ddtree")
    return out


def select_q8(cand_idx, cand_val, gate, pred_q8, succ_q8, anchor, temperature, seed, step,
              tokens=None, slot=None, q=None, status=None, ws=None, stream=None):
    """pred_q8 / succ_q8: (codes uint8 [V, R], scale bf16 [V, R/64], bias bf16 [V, R/64])."""
    _dev(cand_idx, cand_val, gate, anchor, temperature, *pred_q8, *succ_q8)
    _contig(cand_idx, cand_val, gate, anchor, temperature, *pred_q8, *succ_q8)
    B, N, _ = cand_idx.shape
    V, R = pred_q8[0].shape
    for cb in (pred_q8, succ_q8):
        if cb[0].dtype != torch.uint8 or cb[1].dtype != torch.bfloat16 or cb[2].dtype != torch.bfloat16:
            raise TypeError("Q8 codebooks: uint8 codes, bfloat16 scale and bias")
    dev = cand_idx.device
    tokens = torch.empty((B, N), dtype=torch.int32, device=dev) if tokens is None else tokens
    slot = torch.empty((B, N), dtype=torch.int32, device=dev) if slot is None else slot
    q = torch.empty((B, N, K), dtype=torch.float32, device=dev) if q is None else q
    status = torch.empty((B,), dtype=torch.int32, device=dev) if status is None else status
    if ws is None:
        ws = workspace(select_workspace_bytes(B, N), dev)
    rc = _lib.dflash2_select_q8(_ptr(cand_idx), _ptr(cand_val), _ptr(gate),
                                *[_ptr(a) for a in pred_q8], *[_ptr(a) for a in succ_q8], V, R,
                                _ptr(anchor), _ptr(temperature), int(seed) & (2**64 - 1),
                                int(step) & (2**64 - 1), B, N, _ptr(tokens), _ptr(slot), _ptr(q),
                                _ptr(status), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "dflash2_select_q8")
    return tokens, slot, q, status


def verify_workspace_bytes(B, N, V, dtype) -> int:
    return int(_lib.dflash2_verify_workspace_bytes(B, N, V, dtype))


def verify(target, B, N, seq_stride, row_stride, V, tokens, cand_idx, q, slot, temperature,
           seed, step, status, n_accept=None, out_tokens=None, ws=None, stream=None):
    """status is OR-ed in place (pass the selector's status, or zeros)."""
    _dev(target, tokens, cand_idx, q, slot, temperature, status)
    _contig(tokens, cand_idx, q, slot, temperature, status)
    dt = _dtype(target)
    dev = target.device
    n_accept = torch.empty((B,), dtype=torch.int32, device=dev) if n_accept is None else n_accept
    out_tokens = (torch.empty((B, N + 1), dtype=torch.int32, device=dev)
                  if out_tokens is None else out_tokens)
    if ws is None:
        ws = workspace(verify_workspace_bytes(B, N, V, dt), dev)
    rc = _lib.dflash2_verify(_ptr(target), dt, seq_stride, row_stride, V, _ptr(tokens),
                             _ptr(cand_idx), _ptr(q), _ptr(slot), _ptr(temperature),
                             int(seed) & (2**64 - 1), int(step) & (2**64 - 1), B, N,
                             _ptr(n_accept), _ptr(out_tokens), _ptr(status), _ptr(ws), ws.numel(),
                             _stream(stream))
    _check(rc, "dflash2_verify")
    return n_accept, out_tokens, status


def ring_update(new_k, new_v, n_new, back, ctx_len, k_ring, v_ring, W, status, stream=None):
    """Rewind (back >= 0) or reset (back < 0), then append n_new rows; ctx_len and the rings
    are updated in place, status is OR-ed."""
    _dev(new_k, new_v, n_new, back, ctx_len, k_ring, v_ring, status)
    _contig(new_k, new_v, n_new, back, ctx_len, k_ring, v_ring, status)
    B, Pn, Hkv, D = new_k.shape
    S = k_ring.shape[1]
    rc = _lib.dflash2_ring_update(_ptr(new_k), _ptr(new_v), _ptr(n_new), _ptr(back),
                                  _ptr(ctx_len), _ptr(k_ring), _ptr(v_ring), B, Pn, Hkv, D, S, W,
                                  _dtype(new_k), _ptr(status), _stream(stream))
    _check(rc, "dflash2_ring_update")
    return ctx_len, status
