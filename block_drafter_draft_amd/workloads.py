"""Seeded synthetic workloads for the DFlash2 draft-and-verify step.

This module only draws inputs. It holds none of the step's arithmetic, and both the GPU
library's tests and the CPU oracle consume exactly the arrays it returns (bf16 values are
rounded once, here, and passed around as their 16-bit patterns).

Shapes follow the drafter geometry of the pages (block of 8 = anchor + 7 masks, 32 query
heads, 8 KV heads, head dim 128, 2048-position window, width 5120 with groups of 16, vocab
248320, top-16, rank-256 codebooks, 5 drafter layers with 4 conv sites each). Variances are
read as variances: N(0, 4) has standard deviation 2; the heavy-tailed codebooks are
0.25 * Student-t(3).

Every tensor has its own numpy stream keyed by (config seed, tensor id, layer or site,
sequence, input set), so any sequence can be regenerated on its own, and one sequence's
values do not depend on the batch size.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ------------------------------------------------------------------------------------------
# bf16 helpers (input construction only: one round-to-nearest-even narrowing)
# ------------------------------------------------------------------------------------------


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------------------------------
# Configurations
# ------------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    W: int
    C: int
    V: int
    R: int
    layers: int
    act_bf16: bool            # q/k/v and conv activations in bf16 (else f32)
    draft_var: float
    target_noise_var: float
    target_kind: str          # "logits" (greedy only, same dtype as draft) or "probs" (f32)
    temperature: tuple        # per-sequence rule: ("all", T) or ("alternate", T_even, T_odd)
    ctx: tuple                # ("fixed", L) or ("uniform", lo, hi)
    quantize_draft: float = 0.0  # draft logits rounded to multiples of this (0 = off)
    heavy_codebooks: bool = False
    P: int = 8
    group: int = 16
    conv_sites_per_layer: int = 4

    @property
    def N(self) -> int:
        return self.P - 1

    @property
    def G(self) -> int:
        return self.C // self.group

    @property
    def sites(self) -> int:
        return self.layers * self.conv_sites_per_layer

    @property
    def seed(self) -> int:
        """Philox seed of the step's random draws."""
        return 0xDF20000 + self.cfg

    def temperatures(self) -> np.ndarray:
        rule = self.temperature
        if rule[0] == "all":
            return np.full(self.B, rule[1], dtype=np.float32)
        t = np.empty(self.B, dtype=np.float32)
        t[0::2] = rule[1]
        t[1::2] = rule[2]
        return t


CONFIGS = {
    1: Config(1, "tiny-fp32-smoke", B=1, Hq=4, Hkv=1, D=64, S=128, W=64, C=256, V=1024, R=16,
              layers=1, act_bf16=False, draft_var=3.0, target_noise_var=1.0,
              target_kind="logits", temperature=("all", 0.0), ctx=("fixed", 128)),
    2: Config(2, "qwen3.8-27b-drafter-b1-greedy", B=1, Hq=32, Hkv=8, D=128, S=2048, W=2048,
              C=5120, V=248320, R=256, layers=5, act_bf16=True, draft_var=4.0,
              target_noise_var=1.5, target_kind="logits", temperature=("all", 0.0),
              ctx=("fixed", 3000)),
    3: Config(3, "b16-sampled-t0.7", B=16, Hq=32, Hkv=8, D=128, S=2048, W=2048, C=5120,
              V=248320, R=256, layers=5, act_bf16=True, draft_var=4.0, target_noise_var=1.5,
              target_kind="probs", temperature=("all", 0.7), ctx=("uniform", 512, 8192)),
    4: Config(4, "b16-low-acceptance", B=16, Hq=32, Hkv=8, D=128, S=2048, W=2048, C=5120,
              V=248320, R=256, layers=5, act_bf16=True, draft_var=4.0, target_noise_var=4.0,
              target_kind="probs", temperature=("all", 0.7), ctx=("uniform", 512, 8192),
              quantize_draft=0.25, heavy_codebooks=True),
    5: Config(5, "b64-serving-mixed", B=64, Hq=32, Hkv=8, D=128, S=2048, W=2048, C=5120,
              V=248320, R=256, layers=5, act_bf16=True, draft_var=4.0, target_noise_var=1.5,
              target_kind="probs", temperature=("alternate", 0.0, 1.0),
              ctx=("uniform", 2048, 131072)),
}

# tensor ids of the per-tensor streams
_T_CTX, _T_Q, _T_KBLK, _T_VBLK, _T_KRING, _T_VRING = 1, 2, 3, 4, 5, 6
_T_X, _T_BASE, _T_DELTA = 7, 8, 9
_T_DRAFT, _T_TNOISE, _T_PRED, _T_SUCC, _T_GATE, _T_ANCHOR = 10, 11, 12, 13, 14, 15
_T_HIDDEN, _T_HEAD = 16, 17
_T_CONVPROJ, _T_GATEPROJ = 18, 19
_T_BONUS, _T_ACCEPT = 20, 21


def _rng(cfg: Config, tensor: int, *more: int) -> np.random.Generator:
    return np.random.default_rng([1000 + cfg.cfg, tensor, *more])


def _normal(rng, shape, var=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        x *= np.float32(np.sqrt(var))
    return x


def _act(cfg: Config, x: np.ndarray) -> np.ndarray:
    return to_bf16_bits(x) if cfg.act_bf16 else x.astype(np.float32)


# ------------------------------------------------------------------------------------------
# Per-tensor generators. `seqs` selects sequences (default all); `iset` picks an input set
# (the benchmark rotates several so that its working set does not sit in the last-level
# cache).
# ------------------------------------------------------------------------------------------


def ctx_len(cfg: Config, iset: int = 0) -> np.ndarray:
    if cfg.ctx[0] == "fixed":
        return np.full(cfg.B, cfg.ctx[1], dtype=np.int32)
    lo, hi = cfg.ctx[1], cfg.ctx[2]
    return _rng(cfg, _T_CTX, iset).integers(lo, hi + 1, size=cfg.B, dtype=np.int64).astype(np.int32)


def _per_seq(cfg, tensor, layer, seqs, iset, shape, gen):
    seqs = range(cfg.B) if seqs is None else seqs
    return np.stack([gen(_rng(cfg, tensor, layer, b, iset), shape) for b in seqs])


def attn_q(cfg: Config, layer: int, seqs=None, iset: int = 0) -> np.ndarray:
    return _act(cfg, _per_seq(cfg, _T_Q, layer, seqs, iset, (cfg.P, cfg.Hq, cfg.D), _normal))


def attn_block_kv(cfg: Config, layer: int, seqs=None, iset: int = 0):
    shp = (cfg.P, cfg.Hkv, cfg.D)
    return (_act(cfg, _per_seq(cfg, _T_KBLK, layer, seqs, iset, shp, _normal)),
            _act(cfg, _per_seq(cfg, _T_VBLK, layer, seqs, iset, shp, _normal)))


def attn_ring(cfg: Config, layer: int, seqs=None, iset: int = 0):
    shp = (cfg.S, cfg.Hkv, cfg.D)
    return (_act(cfg, _per_seq(cfg, _T_KRING, layer, seqs, iset, shp, _normal)),
            _act(cfg, _per_seq(cfg, _T_VRING, layer, seqs, iset, shp, _normal)))


def conv_inputs(cfg: Config, site: int, seqs=None, iset: int = 0):
    """x [B,P,C] ~ N(0,1); base [2,C] ~ U(-1,1) (one per site); delta [B,P,2,G] ~ U(-1,1)."""
    x = _act(cfg, _per_seq(cfg, _T_X, site, seqs, iset, (cfg.P, cfg.C), _normal))
    base = _rng(cfg, _T_BASE, site).uniform(-1, 1, size=(2, cfg.C)).astype(np.float32)
    delta = _per_seq(cfg, _T_DELTA, site, seqs, iset, (cfg.P, 2, cfg.G),
                     lambda r, s: r.uniform(-1, 1, size=s).astype(np.float32))
    return x, base, delta


def draft_logits(cfg: Config, seqs=None, iset: int = 0) -> np.ndarray:
    """[B, P, V] draft logits: f32 for the tiny config, bf16 bits otherwise."""
    def gen(r, s):
        x = _normal(r, s, cfg.draft_var)
        if cfg.quantize_draft:
            x = (np.round(x / cfg.quantize_draft) * cfg.quantize_draft).astype(np.float32)
        return x
    x = _per_seq(cfg, _T_DRAFT, 0, seqs, iset, (cfg.P, cfg.V), gen)
    return _act(cfg, x)


def bonus_draft_row(cfg: Config, seqs=None, iset: int = 0) -> np.ndarray:
    """[B, 1, V] a draft-like row (same distribution, rounding and quantisation as the draft
    logits) for the position after the block, which no draft row predicts: the base of the
    target's bonus row."""
    def gen(r, s):
        x = _normal(r, s, cfg.draft_var)
        if cfg.quantize_draft:
            x = (np.round(x / cfg.quantize_draft) * cfg.quantize_draft).astype(np.float32)
        return x
    return _act(cfg, _per_seq(cfg, _T_BONUS, 0, seqs, iset, (1, cfg.V), gen))


def target_rows(cfg: Config, draft: np.ndarray, seqs=None, iset: int = 0) -> np.ndarray:
    """Target rows [B, P, V]: the draft row that predicts the same position plus noise, as
    logits (same dtype as the draft), or as f32 probabilities softmax(logits / T) (T = 1 for
    greedy sequences).

    Alignment: target row r verifies proposal r + 1, which the selector takes from the
    candidates of draft row r + 1, so target row r is built around draft row r + 1 (both
    score the token at block position r + 1). Row P - 1, the bonus row, predicts the position
    after the block; no draft row does, so its base is a draft-like row of its own stream."""
    seqs_l = list(range(cfg.B)) if seqs is None else list(seqs)
    d = bf16_bits_to_f32(draft) if draft.dtype == np.uint16 else draft
    bonus = bonus_draft_row(cfg, seqs_l, iset)
    bonus = bf16_bits_to_f32(bonus) if bonus.dtype == np.uint16 else bonus
    base = np.concatenate([d[:, 1:], bonus], axis=1).astype(np.float32)
    noise = _per_seq(cfg, _T_TNOISE, 0, seqs_l, iset, (cfg.P, cfg.V),
                     lambda r, s: _normal(r, s, cfg.target_noise_var))
    logits = base + noise
    if cfg.target_kind == "logits":
        return _act(cfg, logits)
    temps = cfg.temperatures()[seqs_l]
    out = np.empty(logits.shape, dtype=np.float32)
    for n, T in enumerate(temps):
        z = logits[n].astype(np.float64) / (float(T) if T > 0 else 1.0)
        z -= z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        out[n] = (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)
    return out


def codebooks(cfg: Config):
    """Predecessor and successor codebooks [V, R] as bf16 bits."""
    out = []
    for t in (_T_PRED, _T_SUCC):
        r = _rng(cfg, t)
        if cfg.heavy_codebooks:
            x = (0.25 * r.standard_t(3, size=(cfg.V, cfg.R))).astype(np.float32)
        else:
            x = _normal(r, (cfg.V, cfg.R), 1.0 / 16.0)
        out.append(to_bf16_bits(x))
    return out[0], out[1]


def q8_quantize(x: np.ndarray, group: int = 64):
    """Affine Q8 of rows [V, R] in groups of `group`: bf16 scale and bias per group, then
    codes in 0..255 chosen against the stored (bf16-rounded) scale and bias. Returns
    (codes uint8 [V, R], scale bf16 bits [V, R/group], bias bf16 bits [V, R/group]).
    This is input preparation (a converter's job), not part of the selector."""
    V, R = x.shape
    xg = x.astype(np.float32).reshape(V, R // group, group)
    lo, hi = xg.min(axis=2), xg.max(axis=2)
    scale = to_bf16_bits(np.maximum((hi - lo) / np.float32(255.0), np.float32(1e-8)))
    bias = to_bf16_bits(lo)
    s = bf16_bits_to_f32(scale)[..., None]
    z = bf16_bits_to_f32(bias)[..., None]
    codes = np.clip(np.rint((xg - z) / s), 0, 255).astype(np.uint8).reshape(V, R)
    return codes, scale, bias


def codebooks_q8(cfg: Config):
    """The bf16 codebooks of `codebooks`, converted to affine Q8 (groups of 64)."""
    A, Bc = codebooks(cfg)
    return q8_quantize(bf16_bits_to_f32(A)), q8_quantize(bf16_bits_to_f32(Bc))


def gate(cfg: Config, seqs=None, iset: int = 0) -> np.ndarray:
    return _per_seq(cfg, _T_GATE, 0, seqs, iset, (cfg.N, cfg.R), _normal)


def head_hidden(cfg: Config, seqs=None, iset: int = 0) -> np.ndarray:
    """Final hidden states [B, P, C] bf16 bits ~ N(0, draft_var), the rows the output head
    projects (rows 1..P-1 are the proposals)."""
    x = _per_seq(cfg, _T_HIDDEN, 0, seqs, iset, (cfg.P, cfg.C),
                 lambda r, s: _normal(r, s, cfg.draft_var))
    return to_bf16_bits(x)


def head_weight(cfg: Config, V: int | None = None, chunk: int = 16384) -> np.ndarray:
    """Output head [V, C] bf16 bits ~ N(0, 1/C), so that logits have variance about
    draft_var. Generated in row chunks (one stream per chunk) to bound host memory."""
    V = cfg.V if V is None else V
    out = np.empty((V, cfg.C), dtype=np.uint16)
    for c, v0 in enumerate(range(0, V, chunk)):
        v1 = min(V, v0 + chunk)
        out[v0:v1] = to_bf16_bits(_normal(_rng(cfg, _T_HEAD, c), (v1 - v0, cfg.C), 1.0 / cfg.C))
    return out


def conv_proj_weight(cfg: Config, layer: int, sub: int) -> np.ndarray:
    """Coefficient projection of one sublayer (sub 0: attention, 1: MLP) of a layer,
    [4 G, C] bf16 bits ~ N(0, 1/C): rows (conv s, tap t, group g) -> (2 s + t) G + g, s = 0
    the conv before the sublayer and s = 1 the one after."""
    G = cfg.C // 16
    return to_bf16_bits(_normal(_rng(cfg, _T_CONVPROJ, layer, sub), (4 * G, cfg.C), 1.0 / cfg.C))


def gate_proj_weight(cfg: Config) -> np.ndarray:
    """Selector gate projection [R, C] bf16 bits ~ N(0, 1/C)."""
    return to_bf16_bits(_normal(_rng(cfg, _T_GATEPROJ), (cfg.R, cfg.C), 1.0 / cfg.C))


def anchor(cfg: Config, iset: int = 0) -> np.ndarray:
    return _rng(cfg, _T_ANCHOR, iset).integers(0, cfg.V, size=cfg.B).astype(np.int32)


@dataclass
class StepInputs:
    """Everything one step consumes, as numpy arrays (bf16 as uint16 bit patterns)."""
    cfg: Config
    ctx_len: np.ndarray
    q: list = field(default_factory=list)        # per layer [B,P,Hq,D]
    k_blk: list = field(default_factory=list)    # per layer [B,P,Hkv,D]
    v_blk: list = field(default_factory=list)
    k_ring: list = field(default_factory=list)   # per layer [B,S,Hkv,D]
    v_ring: list = field(default_factory=list)
    conv_x: list = field(default_factory=list)   # per site [B,P,C]
    conv_base: list = field(default_factory=list)
    conv_delta: list = field(default_factory=list)
    draft: np.ndarray | None = None              # [B,P,V]
    target: np.ndarray | None = None             # [B,P,V]
    pred_cb: np.ndarray | None = None            # [V,R]
    succ_cb: np.ndarray | None = None
    gate: np.ndarray | None = None               # [B,N,R]
    anchor: np.ndarray | None = None             # [B]
    temperature: np.ndarray | None = None        # [B]


def make_step_inputs(cfg: Config, iset: int = 0, with_attention: bool = True,
                     with_codebooks: bool = True, cb=None, seqs=None) -> StepInputs:
    """All inputs of one step. `seqs` (a list of sequence indices) draws only those
    sequences, with exactly the values they have in the full batch."""
    sel = slice(None) if seqs is None else list(seqs)
    si = StepInputs(cfg=cfg, ctx_len=ctx_len(cfg, iset)[sel])
    if with_attention:
        for layer in range(cfg.layers):
            si.q.append(attn_q(cfg, layer, seqs, iset=iset))
            kb, vb = attn_block_kv(cfg, layer, seqs, iset=iset)
            si.k_blk.append(kb)
            si.v_blk.append(vb)
            kr, vr = attn_ring(cfg, layer, seqs, iset=iset)
            si.k_ring.append(kr)
            si.v_ring.append(vr)
    for site in range(cfg.sites):
        x, base, delta = conv_inputs(cfg, site, seqs, iset=iset)
        si.conv_x.append(x)
        si.conv_base.append(base)
        si.conv_delta.append(delta)
    si.draft = draft_logits(cfg, seqs, iset=iset)
    si.target = target_rows(cfg, si.draft, seqs, iset=iset)
    if with_codebooks:
        si.pred_cb, si.succ_cb = cb if cb is not None else codebooks(cfg)
    si.gate = gate(cfg, seqs, iset=iset)
    si.anchor = anchor(cfg, iset)[sel]
    si.temperature = cfg.temperatures()[sel]
    return si


@dataclass
class VerifyInputs:
    """Inputs of one verify call (bf16 as uint16 bit patterns)."""
    target: np.ndarray        # [B, P, V]
    tokens: np.ndarray        # [B, N]
    cand_idx: np.ndarray      # [B, N, 16]
    q: np.ndarray             # [B, N, 16]
    slot: np.ndarray          # [B, N]
    temperature: np.ndarray   # [B]


def all_accept_verify_inputs(cfg: Config, iset: int = 0, seqs=None) -> VerifyInputs:
    """Verify inputs under which every proposal of every sequence is accepted: the other
    extreme from the step's own targets, for the verify call alone.

    Per sequence and slot j: 16 distinct candidates, q ~ Dirichlet(1) over them, and the
    proposal drawn from q. The target rows are the workload's own (target_rows), changed
    only at each proposal: for a greedy sequence, row j-1 gets a strict maximum at d_j
    (logits: 2 |max| + 1; probabilities: the row scaled by 1/2 plus 1/2 at d_j); for a
    sampled sequence, row j-1 is scaled by 1 - q_j(d_j) and gets q_j(d_j) added at d_j, so
    that p_t(d_j) >= q_j(d_j) (the ratio test then always accepts). Row N is unchanged."""
    seqs_l = list(range(cfg.B)) if seqs is None else list(seqs)
    N, V = cfg.N, cfg.V
    draft = draft_logits(cfg, seqs_l, iset)
    target = target_rows(cfg, draft, seqs_l, iset)
    temps = cfg.temperatures()[seqs_l]
    B = len(seqs_l)
    cand = np.empty((B, N, 16), np.int32)
    q = np.empty((B, N, 16), np.float32)
    slot = np.empty((B, N), np.int32)
    for n, b in enumerate(seqs_l):
        r = _rng(cfg, _T_ACCEPT, 0, b, iset)
        for j in range(N):
            cand[n, j] = r.choice(V, 16, replace=False)
            q[n, j] = r.dirichlet(np.ones(16)).astype(np.float32)
            w = q[n, j].astype(np.float64)
            slot[n, j] = r.choice(16, p=w / w.sum())
    tokens = np.take_along_axis(cand, slot[..., None], axis=2)[..., 0].astype(np.int32)
    for n in range(B):
        for j in range(N):
            d = tokens[n, j]
            if target.dtype == np.uint16:           # bf16 logits: greedy
                row = bf16_bits_to_f32(target[n, j])
                top = float(np.max(np.abs(row)))
                target[n, j, d] = to_bf16_bits(np.array([2 * top + 1], np.float32))[0]
            elif temps[n] > 0:                      # probabilities, sampled
                qd = np.float32(q[n, j, slot[n, j]])
                row = target[n, j] * (np.float32(1) - qd)
                row[d] += qd
                target[n, j] = row
            elif cfg.target_kind == "probs":        # probabilities, greedy
                row = target[n, j] * np.float32(0.5)
                row[d] += np.float32(0.5)
                target[n, j] = row
            else:                                   # f32 logits: greedy
                top = float(np.max(np.abs(target[n, j])))
                target[n, j, d] = np.float32(2 * top + 1)
    return VerifyInputs(target=target, tokens=tokens, cand_idx=cand, q=q, slot=slot,
                        temperature=temps)
