"""CPU oracle for the DFlash2 block-draft-and-verify step.

TEST INFRASTRUCTURE ONLY. This package wraps ``dflash2_oracle.c``, the plain, slow,
single-threaded reference that the GPU library is checked against. Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it; the
product path (``block_drafter_draft_amd``) never does, and shares no code with it.

Each wrapper marshals numpy arrays into the C functions; the arithmetic and the citations
of the pages live in the C file. The exceptions are the output-head projection (the
``lmhead_*`` functions) and the drafter projections (``proj``, ``conv_coeffs``,
``selector_gate``), written here with numpy: a binary64 matrix product of the exact bf16
values (and, for the head, the top-16 order applied to its rows). Functions that are pinned
by tests are listed in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dflash2_oracle.c")
_LIB = os.path.join(_HERE, "libdflash2_oracle.so")

BF16 = 0
F32 = 1

ST_NONFINITE = 1
ST_BADTOKEN = 2
ST_ZEROMASS = 4
ST_BADPROB = 8
ST_BADTEMP = 16
ST_RINGLOST = 32
ST_BADCOUNT = 64

K = 16


def build() -> str:
    """Compile the oracle with gcc (no contraction, no fast-math, no vectorised libm)."""
    cmd = [
        "gcc", "-std=gnu11", "-O2", "-ffp-contract=off", "-fno-fast-math",
        "-fno-builtin", "-Wall", "-Wextra", "-Wno-unused-parameter",
        "-shared", "-fPIC", "-o", _LIB + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i32p, f32p, f64p, u16p, u64p = (ctypes.c_void_p,) * 6
        c_int, c_i64, c_u64, c_f32, c_f64 = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                             ctypes.c_float, ctypes.c_double)
        L.or_philox4x64_10.argtypes = [u64p, u64p, u64p]
        L.or_exp_c.argtypes = [c_f32]
        L.or_exp_c.restype = c_f32
        L.or_exp_c_many.argtypes = [f32p, f32p, c_i64]
        L.or_block_attn.argtypes = [vp, vp, vp, vp, vp, i32p, f64p] + [c_int] * 7 + [c_f64, c_int]
        L.or_dynconv2.argtypes = [vp, f32p, f32p, f64p] + [c_int] * 5
        L.or_topk16.argtypes = [vp, c_int, c_int, c_int, c_int, c_i64, c_i64, c_int, i32p, f32p]
        L.or_viterbi.argtypes = [c_int, c_int, f32p, f32p, i32p]
        L.or_walk.argtypes = [c_int, c_int, f32p, f32p, c_f32, f32p, i32p, f32p]
        L.or_select.argtypes = ([i32p, f32p, f32p, u16p, u16p, c_int, c_int, i32p, f32p,
                                 c_u64, c_u64, c_int, c_int, i32p, i32p, f32p, i32p, f32p])
        L.or_verify.argtypes = ([vp, c_int, c_i64, c_i64, c_int, i32p, i32p, f32p, i32p, f32p,
                                 c_u64, c_u64, c_int, c_int, i32p, i32p, i32p])
        L.or_select_q8.argtypes = ([i32p, f32p, f32p] + [vp] * 6 +
                                   [c_int, c_int, i32p, f32p, c_u64, c_u64, c_int, c_int,
                                    i32p, i32p, f32p, i32p, f32p])
        L.or_q8_dequant.argtypes = [vp, vp, vp, c_i64, c_int, f32p]
        L.or_log_c.argtypes = [c_f32]
        L.or_log_c.restype = c_f32
        L.or_log_c_many.argtypes = [f32p, f32p, c_i64]
        L.or_ddtree.argtypes = ([i32p, f32p, f32p, u16p, u16p, c_int, c_int, i32p, c_int, c_int,
                                 c_int, i32p, i32p, i32p, i32p, f32p, i32p])
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"expected float32 or bf16 bits (uint16), got {a.dtype}")


# ----------------------------------------------------------------------------------------
# Wrappers
# ----------------------------------------------------------------------------------------

def philox4x64_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint64).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64).reshape(2))
    out = np.zeros(4, dtype=np.uint64)
    lib().or_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def exp_c(y: float) -> float:
    return float(lib().or_exp_c(ctypes.c_float(y)))


def exp_c_array(y: np.ndarray) -> np.ndarray:
    yy = np.ascontiguousarray(y, dtype=np.float32).reshape(-1)
    out = np.empty_like(yy)
    lib().or_exp_c_many(_p(yy), _p(out), yy.size)
    return out.reshape(np.shape(y))


def block_attn(q, k_blk, v_blk, k_ring, v_ring, ctx_len, W, scale=None) -> np.ndarray:
    """Dense binary64 block attention. q [B,P,Hq,D]; blocks [B,P,Hkv,D]; rings [B,S,Hkv,D]."""
    B, P, Hq, D = q.shape
    S, Hkv = k_ring.shape[1], k_ring.shape[2]
    dt = _dtype_code(q)
    for a in (k_blk, v_blk, k_ring, v_ring):
        assert _dtype_code(a) == dt
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    arrs = [np.ascontiguousarray(a) for a in (q, k_blk, v_blk, k_ring, v_ring)]
    cl = np.ascontiguousarray(np.asarray(ctx_len, dtype=np.int32))
    out = np.zeros((B, P, Hq, D), dtype=np.float64)
    lib().or_block_attn(*[_p(a) for a in arrs], _p(cl), _p(out), B, P, Hq, Hkv, D, S, W,
                        float(scale), dt)
    return out


def dynconv2(x, base, delta, group=16) -> np.ndarray:
    """x [B,P,C] (f32 or bf16 bits); base [2,C] f32; delta [B,P,2,C/group] f32."""
    B, P, C = x.shape
    xx = np.ascontiguousarray(x)
    bb = np.ascontiguousarray(base, dtype=np.float32)
    dd = np.ascontiguousarray(delta, dtype=np.float32)
    out = np.zeros((B, P, C), dtype=np.float64)
    lib().or_dynconv2(_p(xx), _p(bb), _p(dd), _p(out), B, P, C, group, _dtype_code(x))
    return out


def topk16(scores, B, N, row0, seq_stride, row_stride, V):
    """Top-16 of rows row0..row0+N-1 of each sequence, from a flat buffer with element strides."""
    s = np.ascontiguousarray(scores).reshape(-1)
    idx = np.zeros((B, N, K), dtype=np.int32)
    val = np.zeros((B, N, K), dtype=np.float32)
    lib().or_topk16(_p(s), _dtype_code(s), B, N, row0, seq_stride, row_stride, V, _p(idx), _p(val))
    return idx, val


def topk16_rows(rows: np.ndarray):
    """Top-16 of each row of a 2-D array [n, V]."""
    n, V = rows.shape
    idx, val = topk16(rows, 1, n, 0, 0, V, V)
    return idx[0], val[0]


def viterbi(s1: np.ndarray, s: np.ndarray) -> np.ndarray:
    """s1 [K]; s [N-1, K, K] (from candidate kp of slot i-1 to k of slot i)."""
    Kk = s1.shape[0]
    N = s.shape[0] + 1
    a1 = np.ascontiguousarray(s1, dtype=np.float32)
    a = np.ascontiguousarray(s, dtype=np.float32) if N > 1 else np.zeros(1, np.float32)
    path = np.zeros(N, dtype=np.int32)
    lib().or_viterbi(Kk, N, _p(a1), _p(a), _p(path))
    return path


def walk(s1, s, invT: float, uniforms):
    Kk = s1.shape[0]
    N = s.shape[0] + 1
    a1 = np.ascontiguousarray(s1, dtype=np.float32)
    a = np.ascontiguousarray(s, dtype=np.float32) if N > 1 else np.zeros(1, np.float32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    path = np.zeros(N, dtype=np.int32)
    q = np.zeros((N, Kk), dtype=np.float32)
    lib().or_walk(Kk, N, _p(a1), _p(a), ctypes.c_float(invT), _p(u), _p(path), _p(q))
    return path, q


def select(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, temperature, seed, step,
           want_lattice=False):
    B, N, _ = cand_idx.shape
    V, R = pred_cb.shape
    ci = np.ascontiguousarray(cand_idx, dtype=np.int32)
    cv = np.ascontiguousarray(cand_val, dtype=np.float32)
    g = np.ascontiguousarray(gate, dtype=np.float32)
    A = np.ascontiguousarray(pred_cb, dtype=np.uint16)
    Bc = np.ascontiguousarray(succ_cb, dtype=np.uint16)
    an = np.ascontiguousarray(anchor, dtype=np.int32)
    T = np.ascontiguousarray(temperature, dtype=np.float32)
    tokens = np.zeros((B, N), np.int32)
    slot = np.zeros((B, N), np.int32)
    q = np.zeros((B, N, K), np.float32)
    status = np.zeros(B, np.int32)
    lat = np.zeros((B, N, K, K), np.float32) if want_lattice else None
    lib().or_select(_p(ci), _p(cv), _p(g), _p(A), _p(Bc), V, R, _p(an), _p(T),
                    ctypes.c_uint64(seed), ctypes.c_uint64(step), B, N, _p(tokens), _p(slot),
                    _p(q), _p(status), _p(lat))
    if want_lattice:
        return tokens, slot, q, status, lat
    return tokens, slot, q, status


def select_q8(cand_idx, cand_val, gate, pred_q8, succ_q8, anchor, temperature, seed, step,
              want_lattice=False):
    """The selector over affine-Q8 codebooks; pred_q8 / succ_q8 are (codes [V, R] uint8,
    scale [V, R/64] bf16 bits, bias [V, R/64] bf16 bits)."""
    B, N, _ = cand_idx.shape
    V, R = pred_q8[0].shape
    ci = np.ascontiguousarray(cand_idx, dtype=np.int32)
    cv = np.ascontiguousarray(cand_val, dtype=np.float32)
    g = np.ascontiguousarray(gate, dtype=np.float32)
    pa = [np.ascontiguousarray(a) for a in pred_q8]
    sa = [np.ascontiguousarray(a) for a in succ_q8]
    assert pa[0].dtype == np.uint8 and pa[1].dtype == np.uint16 and pa[2].dtype == np.uint16
    an = np.ascontiguousarray(anchor, dtype=np.int32)
    T = np.ascontiguousarray(temperature, dtype=np.float32)
    tokens = np.zeros((B, N), np.int32)
    slot = np.zeros((B, N), np.int32)
    q = np.zeros((B, N, K), np.float32)
    status = np.zeros(B, np.int32)
    lat = np.zeros((B, N, K, K), np.float32) if want_lattice else None
    lib().or_select_q8(_p(ci), _p(cv), _p(g), *[_p(a) for a in pa], *[_p(a) for a in sa], V, R,
                       _p(an), _p(T), ctypes.c_uint64(seed), ctypes.c_uint64(step), B, N,
                       _p(tokens), _p(slot), _p(q), _p(status), _p(lat))
    if want_lattice:
        return tokens, slot, q, status, lat
    return tokens, slot, q, status


def q8_dequant(codes, scale, bias) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(scale, dtype=np.uint16)
    bi = np.ascontiguousarray(bias, dtype=np.uint16)
    V, R = c.shape
    out = np.zeros((V, R), np.float32)
    lib().or_q8_dequant(_p(c), _p(sc), _p(bi), V, R, _p(out))
    return out


def verify(target, B, N, seq_stride, row_stride, V, tokens, cand_idx, q, slot, temperature,
           seed, step, status=None):
    """target is a flat (or shaped) f32 / bf16-bits buffer addressed by element strides."""
    t = np.ascontiguousarray(target).reshape(-1)
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    ci = np.ascontiguousarray(cand_idx, dtype=np.int32)
    qq = np.ascontiguousarray(q, dtype=np.float32)
    sl = np.ascontiguousarray(slot, dtype=np.int32)
    T = np.ascontiguousarray(temperature, dtype=np.float32)
    n_acc = np.zeros(B, np.int32)
    out = np.zeros((B, N + 1), np.int32)
    st = np.zeros(B, np.int32) if status is None else np.ascontiguousarray(status, dtype=np.int32).copy()
    lib().or_verify(_p(t), _dtype_code(t), seq_stride, row_stride, V, _p(tok), _p(ci), _p(qq),
                    _p(sl), _p(T), ctypes.c_uint64(seed), ctypes.c_uint64(step), B, N,
                    _p(n_acc), _p(out), _p(st))
    return n_acc, out, st


# ------------------------------------------------------------------------------------------
# Output-head projection fused with the top-16 ("Geramy/LSE docs/DFLASH2.md",
# drafter-geometry paragraph: the drafter shares the target's output head; "qwen35: DSpark
# speculative decoding (Qwen3.8-27B drafters) - #625", DFlash 2 commit: the selector takes
# the top-k head candidates of each block position).
# ------------------------------------------------------------------------------------------


def _bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def lmhead_logits(hidden_rows: np.ndarray, weight: np.ndarray, chunk: int = 8192):
    """logits[m, v] = sum_c h[m, c] w[v, c] for bf16-bit inputs hidden_rows [M, C] and
    weight [V, C], in binary64, and the sums of |h[m, c] w[v, c]|. Every product of two bf16
    values is exact in binary64 and the binary64 sum of C of them is within
    C * 2^-53 * abs_sum of the exact sum, far inside any binary32 result's error."""
    h = _bf16_to_f64(hidden_rows)
    ha = np.abs(h)
    M, V = h.shape[0], weight.shape[0]
    L = np.empty((M, V), dtype=np.float64)
    A = np.empty((M, V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        w = _bf16_to_f64(weight[v0:v0 + chunk])
        L[:, v0:v0 + w.shape[0]] = h @ w.T
        A[:, v0:v0 + w.shape[0]] = ha @ np.abs(w).T
    return L, A


def top16_order_f64(row: np.ndarray) -> np.ndarray:
    """Indices of the 16 first elements of a binary64 row under the top-16 order: every NaN
    by ascending index, then values descending (+inf first, -inf last; -0 equal to +0), equal
    values by ascending index."""
    x = np.asarray(row, dtype=np.float64)
    nan = np.isnan(x)
    idx = np.arange(x.shape[0])
    key = np.where(nan, 0.0, x) + 0.0               # -0 -> +0
    # lexsort: last key is primary; sort NaN first, then by -value, then by index
    order = np.lexsort((idx, -key, ~nan))
    return order[:K].astype(np.int32)


def lmhead_topk16(hidden, B, N, row0, seq_stride, row_stride, weight):
    """Top-16 of the output-head logits of rows row0..row0+N-1 of each sequence (hidden is
    a flat bf16-bit buffer addressed by element strides). Returns (idx [B,N,16],
    logits [B*N, V], abs_sums [B*N, V]); the reported values are logits at idx."""
    h = np.ascontiguousarray(hidden, dtype=np.uint16).reshape(-1)
    C = weight.shape[1]
    rows = np.stack([h[b * seq_stride + (row0 + r) * row_stride:
                       b * seq_stride + (row0 + r) * row_stride + C]
                     for b in range(B) for r in range(N)])
    L, A = lmhead_logits(rows, weight)
    idx = np.stack([top16_order_f64(L[m]) for m in range(B * N)]).reshape(B, N, K)
    return idx, L, A



# ------------------------------------------------------------------------------------------
# The drafter's projections on either side of the path ("[Spec Decode] DFlash2: local
# convolution + candidate selector - #52816", PR description: the dynamic conv wraps each
# sublayer in and out, its per-group coefficients coming from one projection of the
# sublayer's input; the selector's edge multiplies A[p] elementwise by a projection of the
# hidden state, project(h). "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) -
# #625", DFlash 2 commit: the conv's kernel projections and the selector's hproj).
# Readings: both are plain linear maps, no bias and no nonlinearity; a coefficient row of
# a sublayer is ordered (conv s, tap t, group g) -> (2 s + t) G + g, s = 0 the conv before
# the sublayer and s = 1 the one after; the selector gate of slot i is the projection of
# slot i's hidden row.
# ------------------------------------------------------------------------------------------


def gather_rows(hidden, B, N, row0, seq_stride, row_stride, C) -> np.ndarray:
    """Rows row0..row0+N-1 of each of the B sequences of a flat buffer addressed by element
    strides, as an array [B*N, C] (sequence-major)."""
    h = np.ascontiguousarray(hidden).reshape(-1)
    return np.stack([h[b * seq_stride + (row0 + r) * row_stride:
                       b * seq_stride + (row0 + r) * row_stride + C]
                     for b in range(B) for r in range(N)])


def proj(hidden, B, N, row0, seq_stride, row_stride, weight):
    """y[b, r, o] = sum_c hidden[b*seq_stride + (row0 + r)*row_stride + c] * weight[o, c] for
    bf16-bit hidden rows and a bf16-bit weight [O, C] (a linear layer's usual layout), in
    binary64 (the exact products summed; within C * 2^-53 * abs_sum of the exact sum).
    Returns (Y [B, N, O], A [B, N, O]) with A the sums of |h w|."""
    O, C = weight.shape
    rows = gather_rows(hidden, B, N, row0, seq_stride, row_stride, C)
    Y, A = lmhead_logits(rows, weight)
    return Y.reshape(B, N, O), A.reshape(B, N, O)


def conv_coeffs(x_in, w_delta, G):
    """The dynamic coefficients of the two convs around one sublayer, from one projection of
    the sublayer's input x_in [B, P, C] (bf16 bits) with w_delta [4 G, C] (bf16 bits):
    returns (delta_in, delta_out), each [B, P, 2, G] binary32 (the binary64 sums rounded
    once), in the layout the conv takes (tap-major within a position)."""
    B, P, C = x_in.shape
    Y, _ = proj(x_in.reshape(-1), B, P, 0, P * C, C, w_delta)
    d = Y.astype(np.float32).reshape(B, P, 2, 2, G)
    return np.ascontiguousarray(d[:, :, 0]), np.ascontiguousarray(d[:, :, 1])


def selector_gate(hidden, w_gate, N=None):
    """g[b, i-1] = project(h[b, i]) for block slots i = 1..N (slot 0, the anchor, is not
    scored), hidden [B, P, C] and w_gate [R, C] bf16 bits; binary32 [B, N, R]."""
    B, P, C = hidden.shape
    N = P - 1 if N is None else N
    Y, _ = proj(hidden.reshape(-1), B, N, 1, P * C, C, w_gate)
    return Y.astype(np.float32)

# ------------------------------------------------------------------------------------------
# Context-ring maintenance after verification ("Geramy/LSE docs/DFLASH2.md", native-test
# notes: cache rewind, replacement and reset). Position p of a sequence lives in ring slot
# p mod S.
# ------------------------------------------------------------------------------------------


def ring_update(new_k, new_v, n_new, back, ctx_len, k_ring, v_ring, S, W, status=None):
    """For each sequence: back < 0 resets it (L' = 0), else it is rewound by min(back, L)
    (flagging ST_RINGLOST when the rewound window max(0, L'-W+1) .. L'-1 is not empty and
    reaches below the oldest held position max(0, L-S)); then rows j < n_new go to slots (L'+j) mod S and the
    length becomes L' + n_new (a count outside [0, Pn] is clamped and flags ST_BADCOUNT).
    Returns new (ctx_len, k_ring, v_ring, status) arrays."""
    kr, vr = np.array(k_ring, copy=True), np.array(v_ring, copy=True)
    L = np.array(ctx_len, dtype=np.int32, copy=True)
    st = np.zeros(L.shape[0], np.int32) if status is None else np.array(status, np.int32, copy=True)
    B, Pn = new_k.shape[0], new_k.shape[1]
    for b in range(B):
        Lb = max(int(L[b]), 0)
        if int(back[b]) < 0:
            Lr = 0
        else:
            Lr = Lb - min(int(back[b]), Lb)
            need_lo = max(0, Lr - W + 1)
            if need_lo < Lr and need_lo < max(0, Lb - S):
                st[b] |= ST_RINGLOST
        n = int(n_new[b])
        if n < 0 or n > Pn:
            st[b] |= ST_BADCOUNT
            n = min(max(n, 0), Pn)
        for j in range(n):
            kr[b, (Lr + j) % S] = new_k[b, j]
            vr[b, (Lr + j) % S] = new_v[b, j]
        L[b] = Lr + n
    return L, kr, vr, st


def log_c(x: float) -> float:
    return float(lib().or_log_c(ctypes.c_float(x)))


def log_c_array(x: np.ndarray) -> np.ndarray:
    xs = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros_like(xs)
    lib().or_log_c_many(_p(xs), _p(out), xs.size)
    return out


def ddtree(cand_idx, cand_val, gate, pred_cb, succ_cb, anchor, budget):
    """Best-first draft tree over the selector lattice; returns (parent, depth, slot, token,
    score, status), the first five [B, budget]."""
    B, N, _ = cand_idx.shape
    V, R = pred_cb.shape
    ci = np.ascontiguousarray(cand_idx, dtype=np.int32)
    cv = np.ascontiguousarray(cand_val, dtype=np.float32)
    g = np.ascontiguousarray(gate, dtype=np.float32)
    A = np.ascontiguousarray(pred_cb, dtype=np.uint16)
    Bc = np.ascontiguousarray(succ_cb, dtype=np.uint16)
    an = np.ascontiguousarray(anchor, dtype=np.int32)
    par = np.zeros((B, budget), np.int32)
    dep = np.zeros((B, budget), np.int32)
    slt = np.zeros((B, budget), np.int32)
    tok = np.zeros((B, budget), np.int32)
    sc = np.zeros((B, budget), np.float32)
    st = np.zeros(B, np.int32)
    lib().or_ddtree(_p(ci), _p(cv), _p(g), _p(A), _p(Bc), V, R, _p(an), B, N, budget, _p(par),
                    _p(dep), _p(slt), _p(tok), _p(sc), _p(st))
    return par, dep, slt, tok, sc, st
