"""The C ABI on the host: the library loads, exports every symbol the header
declares, and every invalid argument returns its error code before any HIP
call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import speculative_decoding_verification_sample_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

FAKE = 0x10000  # a non-null, 256-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = sv.load()
    names = declared_functions()
    assert set(names) == set(sv.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert sv.status_string(code) and sv.status_string(code) != "unknown status"
    assert sv.status_string(-99) == "unknown status"


def test_workspace_bytes():
    for op, KN in ((0, 5), (1, 8), (2, 63)):
        for dt in (0, 1):
            n = sv.verify_workspace_bytes(op, 64, KN, 128256, dt, op == 1)
            assert n > 0 and n % 256 == 0
    assert sv.verify_workspace_bytes(1, 4, 4, 32000, 0, True) > sv.verify_workspace_bytes(1, 4, 4, 32000, 0, False)
    # invalid sizes -> 0
    assert sv.verify_workspace_bytes(1, 0, 4, 100, 0, False) == 0
    assert sv.verify_workspace_bytes(1, 1, 64, 100, 0, False) == 0
    assert sv.verify_workspace_bytes(2, 1, 65, 100, 0, False) == 0
    assert sv.verify_workspace_bytes(2, 1, 64, 100, 0, False) > 0
    assert sv.verify_workspace_bytes(1, 1, 4, 0, 0, False) == 0
    assert sv.verify_workspace_bytes(7, 1, 4, 100, 0, False) == 0
    assert sv.verify_workspace_bytes(1, 1, 4, 100, 5, False) == 0


def _sample(**kw):
    args = dict(t=FAKE, d=FAKE, dt=0, tok=FAKE, ua=FAKE, us=FAKE, T=1.0, top_p=1.0, B=2, K=3,
                V=100, acc=FAKE, out=FAKE, p=None, q=None, S=None, ws=FAKE, wsb=1 << 30,
                stream=None)
    args.update(kw)
    a = args
    return sv.load().spec_verify_sample(a["t"], a["d"], a["dt"], a["tok"], a["ua"], a["us"],
                                        a["T"], a["top_p"], a["B"], a["K"], a["V"], a["acc"],
                                        a["out"], a["p"], a["q"], a["S"], a["ws"], a["wsb"],
                                        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(t=None), -1), (dict(d=None), -1), (dict(tok=None), -1), (dict(ua=None), -1),
    (dict(us=None), -1), (dict(acc=None), -1), (dict(out=None), -1), (dict(ws=None), -1),
    (dict(B=0), -2), (dict(K=0), -2), (dict(K=64), -2), (dict(V=0), -2),
    (dict(T=0.0), -3), (dict(T=-1.0), -3), (dict(T=float("inf")), -3), (dict(T=float("nan")), -3),
    (dict(T=1e-45), -3), (dict(top_p=0.0), -3), (dict(top_p=1.5), -3), (dict(top_p=float("nan")), -3),
    (dict(dt=2), -3), (dict(wsb=16), -4), (dict(ws=FAKE + 8), -5), (dict(t=FAKE + 2), -5),
    (dict(d=FAKE + 1, dt=1), -5),
])
def test_sample_errors(kw, code):
    assert _sample(**kw) == code


def test_sample_workspace_exact_boundary():
    need = sv.verify_workspace_bytes(1, 2, 3, 100, 0, True)
    assert _sample(top_p=0.9, wsb=need - 1) == -4
    need_nop = sv.verify_workspace_bytes(1, 2, 3, 100, 0, False)
    assert need_nop < need
    assert _sample(top_p=1.0, wsb=need_nop - 1) == -4


def test_greedy_errors():
    L = sv.load()
    g = lambda **kw: L.spec_verify_greedy(kw.get("t", FAKE), kw.get("dt", 1), kw.get("tok", FAKE),
                                          kw.get("B", 2), kw.get("K", 3), kw.get("V", 100),
                                          kw.get("acc", FAKE), kw.get("out", FAKE),
                                          kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert g(t=None) == -1 and g(tok=None) == -1 and g(acc=None) == -1 and g(out=None) == -1
    assert g(B=0) == -2 and g(K=0) == -2 and g(K=64) == -2 and g(V=-5) == -2
    assert g(dt=9) == -3
    assert g(wsb=0) == -4
    assert g(ws=FAKE + 64) == -5 and g(t=FAKE + 1) == -5


def test_tree_errors():
    L = sv.load()
    tr = lambda **kw: L.spec_verify_tree(kw.get("t", FAKE), kw.get("dt", 1), kw.get("par", FAKE),
                                         kw.get("tok", FAKE), kw.get("mask", FAKE), kw.get("B", 2),
                                         kw.get("N", 63), kw.get("V", 100), kw.get("pl", FAKE),
                                         kw.get("pn", FAKE), kw.get("out", FAKE),
                                         kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    for name in ("t", "par", "tok", "mask", "pl", "pn", "out"):
        assert tr(**{name: None}) == -1, name
    assert tr(N=0) == -2 and tr(N=65) == -2 and tr(B=0) == -2
    assert tr(dt=-1) == -3
    assert tr(wsb=8) == -4
    assert tr(ws=FAKE + 128) == -5


def test_profile_args():
    L = sv.load()
    assert L.spec_profile_begin(0) == -3
    assert L.spec_profile_end(None, None) == -1


def test_binding_requires_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sv, "_lib", None)
    monkeypatch.setattr(sv, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        sv.load()


def _kv(**kw):
    a = dict(kv=FAKE, mirror=None, es=2, L=2, B=3, H=2, S=80, D=128, cl=FAKE, pl=FAKE,
             pn=FAKE, N=63, nl=FAKE, stream=None)
    a.update(kw)
    return sv.load().spec_kv_commit(a["kv"], a["mirror"], a["es"], a["L"], a["B"], a["H"],
                                    a["S"], a["D"], a["cl"], a["pl"], a["pn"], a["N"], a["nl"],
                                    a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kv=None), -1), (dict(cl=None), -1), (dict(pl=None), -1), (dict(nl=None), -1),
    (dict(es=3), -3), (dict(es=0), -3), (dict(kv=FAKE, mirror=FAKE), -3),
    (dict(L=0), -2), (dict(B=0), -2), (dict(H=0), -2), (dict(D=0), -2), (dict(N=0), -2),
    (dict(N=65), -2), (dict(S=62), -2),
    (dict(D=7), -5), (dict(kv=FAKE + 8), -5), (dict(mirror=FAKE + 4), -5),
    (dict(D=1024, es=4), -2),  # one head of the cycle exceeds a workgroup's registers
])
def test_kv_commit_errors(kw, code):
    assert _kv(**kw) == code


def test_mixed_errors():
    L = sv.load()
    call = lambda **kw: L.spec_verify_mixed(
        kw.get("t", FAKE), FAKE, 0, FAKE, FAKE, FAKE, kw.get("temps", FAKE), None, 2, 3, 100,
        FAKE, FAKE, None, None, None, FAKE, kw.get("wsb", 1 << 30), None)
    assert call(temps=None) == -1
    assert call(t=None) == -1
    assert call(wsb=0) == -4


def test_tree_merge_errors():
    L = sv.load()
    call = lambda **kw: L.spec_tree_merge(
        kw.get("p1", FAKE), FAKE, FAKE, kw.get("n1", 31), kw.get("p2", FAKE), FAKE, FAKE,
        kw.get("n2", 31), kw.get("B", 4), kw.get("op", FAKE), FAKE, kw.get("om", FAKE), None,
        None, None)
    for name in ("p1", "p2", "op", "om"):
        assert call(**{name: None}) == -1, name
    assert call(n1=33) == -2 and call(n1=-1) == -2 and call(B=0) == -2


def test_lmhead_errors():
    L = sv.load()
    # one 8-byte key per (row, 256-column vocabulary tile)
    assert L.spec_lmhead_workspace_bytes(2, 3, 128, 1000) == 2 * 4 * 4 * 8
    assert L.spec_lmhead_workspace_bytes(2, 3, 96, 1000) == 0
    call = lambda **kw: L.spec_lmhead_greedy(
        kw.get("h", FAKE), kw.get("w", FAKE), kw.get("t", FAKE), kw.get("B", 2), kw.get("K", 3),
        kw.get("d", 128), kw.get("V", 1000), FAKE, FAKE, None, kw.get("ws", FAKE),
        kw.get("wsb", 1 << 20), None)
    for name in ("h", "w", "t", "ws"):
        assert call(**{name: None}) == -1, name
    assert call(d=96) == -2 and call(d=0) == -2 and call(K=0) == -2 and call(K=64) == -2
    assert call(B=0) == -2 and call(V=0) == -2
    assert call(h=FAKE + 8) == -5 and call(ws=FAKE + 64) == -5
    assert call(wsb=10) == -4


def _sample_noalloc(**kw):
    args = dict(t=FAKE, d=FAKE, dt=0, tok=FAKE, ua=FAKE, us=FAKE, T=1.0, top_p=1.0, B=2, K=3,
                V=100, acc=FAKE, out=FAKE, p=None, q=None, S=None, stream=None)
    args.update(kw)
    a = args
    return sv.load().spec_verify_sample_noalloc(a["t"], a["d"], a["dt"], a["tok"], a["ua"],
                                                a["us"], a["T"], a["top_p"], a["B"], a["K"],
                                                a["V"], a["acc"], a["out"], a["p"], a["q"],
                                                a["S"], a["stream"])


def test_noalloc_host_errors():
    """Invalid arguments of the no-allocation call return their codes before
    any HIP call, as the workspace-taking call does; a call whose workspace
    would exceed the library's array returns SPEC_ERR_WORKSPACE."""
    assert _sample_noalloc(t=None) == -1
    assert _sample_noalloc(us=None) == -1
    assert _sample_noalloc(dt=7) == -3
    assert _sample_noalloc(T=0.0) == -3
    assert _sample_noalloc(T=float("nan")) == -3
    assert _sample_noalloc(top_p=0.0) == -3
    assert _sample_noalloc(top_p=1.5) == -3
    assert _sample_noalloc(K=64) == -2
    assert _sample_noalloc(B=0) == -2
    assert _sample_noalloc(t=FAKE + 2) == -5
    # sizes: the headline fits; top-p at the large-batch setting does not
    need = sv.verify_workspace_bytes(sv.SPEC_OP_SAMPLE, 64, 8, 128256, sv.SPEC_BF16, False)
    assert 0 < need <= sv.SPEC_SCRATCH_BYTES
    big = sv.verify_workspace_bytes(sv.SPEC_OP_SAMPLE, 256, 4, 152064, sv.SPEC_F32, True)
    assert big > sv.SPEC_SCRATCH_BYTES
    assert _sample_noalloc(B=256, K=4, V=152064, top_p=0.95) == -4
