"""The C ABI without a GPU: the library loads, exports every declared function, sizes its
workspaces and rejects bad arguments on the host before any launch.

Every call below is invalid in at least one argument that the host checks reject, so no
kernel is ever launched from these tests (they are safe on any machine).
"""
import ctypes
import os
import re

import pytest

from block_drafter_draft_amd import dflash2 as d2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash2_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_stages():
    names = _declared_functions()
    for stage in ("dflash2_block_attn", "dflash2_dynconv2", "dflash2_topk16", "dflash2_select",
                  "dflash2_verify"):
        assert stage in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(d2.LIB_PATH)
    names = _declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n
    # the binding describes exactly the declared functions
    assert sorted(d2.SIGNATURES) == names


def _declared_arg_counts():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(dflash2_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        args = m.group(2).strip()
        out[m.group(1)] = 0 if args in ("", "void") else args.count(",") + 1
    return out


def test_binding_argument_counts_match_header():
    counts = _declared_arg_counts()
    for name, (argt, _) in d2.SIGNATURES.items():
        assert len(argt) == counts[name], (name, len(argt), counts[name])


def test_version_and_status_strings():
    assert d2.lib().dflash2_version() >= 100
    for code in (d2.OK, d2.EINVAL, d2.EUNSUPPORTED, d2.EWORKSPACE, d2.EHIP, d2.ST_NONFINITE,
                 d2.ST_BADTOKEN, d2.ST_ZEROMASS, d2.ST_BADPROB, d2.ST_BADTEMP, d2.ST_RINGLOST,
                 d2.ST_BADCOUNT):
        s = d2.status_string(code)
        assert s and s != "unknown code"
    assert d2.status_string(12345) == "unknown code"


def test_constants_match_header():
    text = open(HEADER).read()
    for name, val in [("DFLASH2_BF16", d2.BF16), ("DFLASH2_F32", d2.F32),
                      ("DFLASH2_ST_NONFINITE", d2.ST_NONFINITE),
                      ("DFLASH2_ST_BADTOKEN", d2.ST_BADTOKEN),
                      ("DFLASH2_ST_ZEROMASS", d2.ST_ZEROMASS),
                      ("DFLASH2_ST_BADPROB", d2.ST_BADPROB), ("DFLASH2_ST_BADTEMP", d2.ST_BADTEMP),
                      ("DFLASH2_ST_RINGLOST", d2.ST_RINGLOST),
                      ("DFLASH2_ST_BADCOUNT", d2.ST_BADCOUNT)]:
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == val, name
    for name, val in [("DFLASH2_OK", d2.OK), ("DFLASH2_EINVAL", d2.EINVAL),
                      ("DFLASH2_EUNSUPPORTED", d2.EUNSUPPORTED),
                      ("DFLASH2_EWORKSPACE", d2.EWORKSPACE), ("DFLASH2_EHIP", d2.EHIP)]:
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == val, name


def test_workspace_sizes():
    L = d2.lib()
    V = 248320
    for B in (1, 16, 64):
        a = L.dflash2_block_attn_workspace_bytes(B, 8, 32, 8, 128, 2048, 2048, d2.BF16)
        assert a % 256 == 0 and (a > 0 or B == 64)   # one split per head needs none
        t = L.dflash2_topk16_workspace_bytes(B, 7, V, d2.BF16)
        assert t >= B * 7 * 16 * 8 and t % 256 == 0
        s = L.dflash2_select_workspace_bytes(B, 7)
        assert s >= B * 7 * 256 * 4
        v = L.dflash2_verify_workspace_bytes(B, 7, V, d2.F32)
        assert v > 0 and v % 256 == 0
    # f32 attention needs no workspace; bad shapes report 0
    assert L.dflash2_block_attn_workspace_bytes(1, 8, 4, 1, 64, 128, 64, d2.F32) == 0
    assert L.dflash2_topk16_workspace_bytes(0, 7, V, d2.BF16) == 0
    assert L.dflash2_select_workspace_bytes(1, 16) == 0
    assert L.dflash2_verify_workspace_bytes(1, 7, 8, d2.F32) == 0


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation
NUL = None


def test_topk16_rejects():
    L = d2.lib()
    V = 1000
    ok = dict(scores=FAKE, dt=d2.BF16, B=1, N=7, row0=1, ss=8 * V, rs=V, V=V, idx=FAKE, val=FAKE,
              ws=FAKE, wsb=1 << 20)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.dflash2_topk16(a["scores"], a["dt"], a["B"], a["N"], a["row0"], a["ss"], a["rs"],
                                a["V"], a["idx"], a["val"], a["ws"], a["wsb"], None)
    assert call(scores=NUL) == d2.EINVAL
    assert call(idx=NUL) == d2.EINVAL
    assert call(B=0) == d2.EINVAL
    assert call(N=0) == d2.EINVAL
    assert call(V=15) == d2.EINVAL
    assert call(row0=-1) == d2.EINVAL
    assert call(rs=-1) == d2.EINVAL
    assert call(dt=7) == d2.EUNSUPPORTED
    assert call(wsb=16) == d2.EWORKSPACE
    assert call(ws=ctypes.c_void_p(0x100008)) == d2.EWORKSPACE   # misaligned


def test_verify_rejects():
    L = d2.lib()
    V = 1000

    def call(target=FAKE, dt=d2.F32, ss=8 * V, rs=V, V=V, B=2, N=7, ws=FAKE, wsb=1 << 24, **kw):
        p = [kw.get(k, FAKE) for k in ("tokens", "cidx", "q", "slot", "temp")]
        o = [kw.get(k, FAKE) for k in ("nacc", "out", "status")]
        return L.dflash2_verify(target, dt, ss, rs, V, *p, 1, 0, B, N, *o, ws, wsb, None)
    assert call(target=NUL) == d2.EINVAL
    assert call(tokens=NUL) == d2.EINVAL
    assert call(status=NUL) == d2.EINVAL
    assert call(N=0) == d2.EINVAL
    assert call(N=16) == d2.EUNSUPPORTED
    assert call(V=10) == d2.EINVAL
    assert call(ss=-5) == d2.EINVAL
    assert call(dt=3) == d2.EUNSUPPORTED
    assert call(wsb=8) == d2.EWORKSPACE


def test_select_rejects():
    L = d2.lib()

    def call(V=1000, R=256, B=2, N=7, wsb=1 << 20, ws=FAKE, **kw):
        a = [kw.get(k, FAKE) for k in ("ci", "cv", "gate", "A", "Bc")]
        b = [kw.get(k, FAKE) for k in ("anchor", "temp")]
        o = [kw.get(k, FAKE) for k in ("tok", "slot", "q", "status")]
        return L.dflash2_select(*a, V, R, *b, 1, 0, B, N, *o, ws, wsb, None)
    assert call(ci=NUL) == d2.EINVAL
    assert call(status=NUL) == d2.EINVAL
    assert call(R=0) == d2.EINVAL
    assert call(R=513) == d2.EUNSUPPORTED
    assert call(N=16) == d2.EUNSUPPORTED
    assert call(B=0) == d2.EINVAL
    assert call(V=8) == d2.EINVAL
    assert call(wsb=4) == d2.EWORKSPACE


def test_block_attn_rejects():
    L = d2.lib()

    def call(B=1, P=8, Hq=32, Hkv=8, D=128, S=2048, W=2048, dt=d2.BF16, ws=FAKE, wsb=1 << 26, **kw):
        p = [kw.get(k, FAKE) for k in ("q", "kb", "vb", "kr", "vr", "cl", "out")]
        return L.dflash2_block_attn(*p, B, P, Hq, Hkv, D, S, W, 0.088, dt, ws, wsb, None)
    assert call(q=NUL) == d2.EINVAL
    assert call(out=NUL) == d2.EINVAL
    assert call(Hq=30) == d2.EINVAL          # not a multiple of Hkv
    assert call(P=1) == d2.EINVAL
    assert call(P=17) == d2.EINVAL
    assert call(S=100) == d2.EINVAL          # window keys would be overwritten
    assert call(D=96) == d2.EUNSUPPORTED
    assert call(Hq=64) == d2.EUNSUPPORTED     # 8 x 8 = 64 query rows > 32 for bf16
    assert call(dt=5) == d2.EUNSUPPORTED
    assert call(wsb=1024) == d2.EWORKSPACE
    assert call(ws=NUL) == d2.EWORKSPACE
    assert call(q=ctypes.c_void_p(0x100002)) == d2.EUNSUPPORTED   # misaligned bf16 rows


def test_dynconv2_rejects():
    L = d2.lib()

    def call(B=1, P=8, C=5120, group=16, dt=d2.BF16, **kw):
        p = [kw.get(k, FAKE) for k in ("x", "base", "delta", "out")]
        return L.dflash2_dynconv2(*p, B, P, C, group, dt, None)
    assert call(x=NUL) == d2.EINVAL
    assert call(B=0) == d2.EINVAL
    assert call(group=8) == d2.EUNSUPPORTED
    assert call(C=5128 + 4) == d2.EUNSUPPORTED
    assert call(dt=9) == d2.EUNSUPPORTED
    assert call(out=FAKE, x=FAKE) == d2.EINVAL     # in place is not allowed
    assert call(x=ctypes.c_void_p(0x100004), out=ctypes.c_void_p(0x200000)) == d2.EUNSUPPORTED


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        d2.dynconv2(torch.zeros(1, 8, 16), torch.zeros(2, 16), torch.zeros(1, 8, 2, 1))


def test_lmhead_topk16_rejects():
    L = d2.lib()

    def call(hid=FAKE, w=FAKE, C=5120, V=248320, B=1, N=7, row0=1, ss=8 * 5120, rs=5120,
             idx=FAKE, val=FAKE, ws=FAKE, wsb=1 << 30):
        return L.dflash2_lmhead_topk16(hid, ss, rs, row0, w, C, V, B, N, idx, val, ws, wsb, None)
    assert call(hid=NUL) == d2.EINVAL
    assert call(val=NUL) == d2.EINVAL
    assert call(B=0) == d2.EINVAL
    assert call(V=15) == d2.EINVAL
    assert call(row0=-1) == d2.EINVAL
    assert call(C=5000) == d2.EUNSUPPORTED            # not a multiple of 128
    assert call(rs=5121) == d2.EUNSUPPORTED           # row stride not a multiple of 8
    assert call(hid=ctypes.c_void_p(0x100008)) == d2.EUNSUPPORTED
    assert call(wsb=16) == d2.EWORKSPACE
    assert d2.lmhead_topk16_workspace_bytes(1, 7, 248320, 5120) > 0


def test_ring_update_rejects():
    L = d2.lib()

    def call(nk=FAKE, B=2, Pn=8, Hkv=8, D=128, S=2048, W=2048, dt=d2.BF16, status=FAKE, kr=FAKE):
        return L.dflash2_ring_update(nk, FAKE, FAKE, FAKE, FAKE, kr, FAKE, B, Pn, Hkv, D, S, W, dt,
                                     status, None)
    assert call(nk=NUL) == d2.EINVAL
    assert call(status=NUL) == d2.EINVAL
    assert call(B=0) == d2.EINVAL
    assert call(S=100, W=2048) == d2.EINVAL            # the ring cannot hold the window
    assert call(Pn=17) == d2.EUNSUPPORTED
    assert call(S=4, W=4, Pn=8) == d2.EUNSUPPORTED     # more new rows than slots
    assert call(dt=9) == d2.EUNSUPPORTED
    assert call(Hkv=1, D=3) == d2.EUNSUPPORTED         # rows not whole 16-byte pieces
    assert call(kr=ctypes.c_void_p(0x100008)) == d2.EUNSUPPORTED


def test_proj_rejects():
    L = d2.lib()

    def call(hid=FAKE, w=FAKE, C=5120, O=640, B=2, N=8, row0=0, ss=8 * 5120, rs=5120,
             out=FAKE, oss=8 * 640, ors=640, ws=FAKE, wsb=1 << 30):
        return L.dflash2_proj(hid, ss, rs, row0, w, C, O, B, N, out, oss, ors, ws, wsb, None)
    assert call(hid=NUL) == d2.EINVAL
    assert call(out=NUL) == d2.EINVAL
    assert call(B=0) == d2.EINVAL
    assert call(O=0) == d2.EINVAL
    assert call(row0=-1) == d2.EINVAL
    assert call(ss=-8) == d2.EINVAL
    assert call(ors=600) == d2.EINVAL                  # output rows would overlap
    assert call(oss=640) == d2.EINVAL                  # sequences would overlap
    assert call(C=5124) == d2.EUNSUPPORTED             # not a multiple of 8
    assert call(rs=5121) == d2.EUNSUPPORTED            # row stride not a multiple of 8
    assert call(w=ctypes.c_void_p(0x100008)) == d2.EUNSUPPORTED
    assert call(B=1 << 18, N=8) == d2.EUNSUPPORTED     # more than 2^20 rows
    assert call(wsb=16) == d2.EWORKSPACE               # small call: split contraction
    assert call(ws=NUL) == d2.EWORKSPACE
    assert d2.proj_workspace_bytes(2, 8, 640, 5120) > 0
    assert d2.proj_workspace_bytes(256, 8, 640, 5120) == 0  # enough output tiles already


def test_eval_fn_rejects():
    L = d2.lib()
    assert L.dflash2_eval_fn(NUL, FAKE, 16, 0, None) == d2.EINVAL
    assert L.dflash2_eval_fn(FAKE, NUL, 16, 0, None) == d2.EINVAL
    assert L.dflash2_eval_fn(FAKE, FAKE, -1, 0, None) == d2.EINVAL
    assert L.dflash2_eval_fn(FAKE, FAKE, 16, 2, None) == d2.EUNSUPPORTED
    assert L.dflash2_eval_fn(FAKE, FAKE, 0, 1, None) == d2.OK          # nothing to launch


def test_select_noalloc_rejects():
    L = d2.lib()
    p = ctypes.c_void_p(16)
    cap = L.dflash2_select_noalloc_max_bytes()
    assert cap == 4 << 20
    args = lambda B, N, first=p: [first] + [p] * 4 + [1000, 16, p, p, 0, 0, B, N] + [p] * 4 + [None]
    assert L.dflash2_select_noalloc(*args(1, 7, None)) == d2.EINVAL
    assert L.dflash2_select_noalloc(*args(0, 7)) == d2.EINVAL
    assert L.dflash2_select_noalloc(*args(1, 16)) == d2.EUNSUPPORTED
    over = cap // (7 * 16 * 16 * 4) + 1                   # one sequence past the static lattice
    assert L.dflash2_select_noalloc(*args(over, 7)) == d2.EWORKSPACE
