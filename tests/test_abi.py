"""C-ABI checks that need no GPU: the library loads, exports every function the
public header declares, and rejects host-checkable bad arguments synchronously
(these paths return before any HIP call)."""
import ctypes as C
import os
import re

import pytest

import draft_token_verification_08_amd as sv
from draft_token_verification_08_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ["spec_verify_sample", "spec_verify_greedy", "mtp_shift_insert", "sv_workspace_bytes",
              "sv_workspace_clear", "sv_status_string", "sv_last_hip_error", "sv_softmax_rows_debug",
              "spec_verify_greedy_mtp", "spec_verify_sample_mtp", "spec_verify_sample_ex", "sv_sample_rows",
              "spec_verify_greedy_lmhead", "sv_lmhead_logits_debug", "sv_residual_weights_debug"]:
        assert f in names, names


def test_library_exports_every_declared_function():
    L = sv.lib()
    missing = [f for f in declared_functions() if not hasattr(L, f)]
    assert not missing, missing


def test_status_strings():
    L = sv.lib()
    for code in range(5):
        s = L.sv_status_string(code).decode()
        assert s.startswith("SV_")
    assert L.sv_last_hip_error().decode() == ""


def test_workspace_bytes():
    assert sv.sv_workspace_bytes(0, 4, 100, sv.SV_BF16) >= 256
    assert sv.sv_workspace_bytes(-1, 4, 100, sv.SV_BF16) == 0
    assert sv.sv_workspace_bytes(4, sv.SV_MAX_DRAFT + 1, 100, sv.SV_BF16) == 0
    assert sv.sv_workspace_bytes(4, 4, 0, sv.SV_BF16) == 0
    assert sv.sv_workspace_bytes(4, 4, 100, 7) == 0
    a = sv.sv_workspace_bytes(256, 4, 128256, sv.SV_BF16)
    b = sv.sv_workspace_bytes(1024, 8, 152064, sv.SV_BF16)
    assert 0 < a < b < 64 << 20
    assert a % 256 == 0 and b % 256 == 0


NULL = None


def _sample(**kw):
    args = dict(t=C.c_void_p(16), d=C.c_void_p(16), dt=sv.SV_BF16, x=C.c_void_p(16), L=C.c_void_p(16),
                T=C.c_void_p(16), u=C.c_void_p(16), B=4, n=4, V=1024, acc=C.c_void_p(16),
                emi=C.c_void_p(16), lse=NULL, fl=NULL, ws=C.c_void_p(256), wsb=1 << 20, s=NULL)
    args.update(kw)
    return sv.lib().spec_verify_sample(*args.values())


def test_sample_host_checks():
    assert _sample(B=0) == sv.SV_OK                       # no-op, nothing touched
    assert _sample(B=-1) == sv.SV_EINVAL
    assert _sample(n=-1) == sv.SV_EINVAL
    assert _sample(n=sv.SV_MAX_DRAFT + 1) == sv.SV_EINVAL
    assert _sample(V=0) == sv.SV_EINVAL
    assert _sample(dt=5) == sv.SV_EINVAL
    assert _sample(t=NULL) == sv.SV_EINVAL
    assert _sample(x=NULL) == sv.SV_EINVAL
    assert _sample(L=NULL) == sv.SV_EINVAL
    assert _sample(T=NULL) == sv.SV_EINVAL
    assert _sample(u=NULL) == sv.SV_EINVAL
    assert _sample(acc=NULL) == sv.SV_EINVAL
    assert _sample(emi=NULL) == sv.SV_EINVAL
    assert _sample(t=C.c_void_p(17)) == sv.SV_EALIGN
    assert _sample(acc=C.c_void_p(18)) == sv.SV_EALIGN
    assert _sample(ws=NULL) == sv.SV_EWORKSPACE
    assert _sample(wsb=16) == sv.SV_EWORKSPACE
    assert _sample(ws=C.c_void_p(264)) == sv.SV_EALIGN


def _greedy(**kw):
    args = dict(t=C.c_void_p(16), dt=sv.SV_F32, x=C.c_void_p(16), L=C.c_void_p(16), B=4, n=4, V=1024,
                acc=C.c_void_p(16), emi=C.c_void_p(16), fl=NULL, ws=C.c_void_p(256), wsb=1 << 20, s=NULL)
    args.update(kw)
    return sv.lib().spec_verify_greedy(*args.values())


def test_greedy_host_checks():
    assert _greedy(B=0) == sv.SV_OK
    assert _greedy(B=-3) == sv.SV_EINVAL
    assert _greedy(t=NULL) == sv.SV_EINVAL
    assert _greedy(x=NULL) == sv.SV_EINVAL
    assert _greedy(t=C.c_void_p(18)) == sv.SV_EALIGN
    assert _greedy(wsb=0) == sv.SV_EWORKSPACE


def _tree_sample(**kw):
    p = C.c_void_p(16)
    args = dict(t=p, d=p, dt=sv.SV_BF16, x=p, par=p, L=p, T=p, u=p, B=4, n=4, V=1024, R=2, acc=p, emi=p,
                path=NULL, fl=NULL, ws=C.c_void_p(256), wsb=1 << 20, s=NULL)
    args.update(kw)
    return sv.lib().spec_verify_tree_sample(*args.values())


def test_tree_sample_host_checks():
    # every case has one bad argument, so nothing is launched
    assert _tree_sample(B=0) == sv.SV_OK
    assert _tree_sample(B=-1) == sv.SV_EINVAL
    assert _tree_sample(n=sv.SV_MAX_DRAFT + 1) == sv.SV_EINVAL
    assert _tree_sample(R=-1) == sv.SV_EINVAL
    assert _tree_sample(R=4097) == sv.SV_EINVAL
    assert _tree_sample(d=NULL) == sv.SV_EINVAL           # draft logits required when n > 0
    assert _tree_sample(par=NULL) == sv.SV_EINVAL
    assert _tree_sample(x=NULL) == sv.SV_EINVAL
    assert _tree_sample(u=NULL) == sv.SV_EINVAL
    assert _tree_sample(par=C.c_void_p(18)) == sv.SV_EALIGN
    assert _tree_sample(ws=NULL) == sv.SV_EWORKSPACE
    assert _tree_sample(wsb=64) == sv.SV_EWORKSPACE


def test_tree_rounds_helper():
    assert sv.sv_tree_rounds([]) == 0
    assert sv.sv_tree_rounds(list(range(10))) == 0            # a chain: one child per node
    assert sv.sv_tree_rounds([0, 0, 0]) == 2                  # a star of 3
    assert sv.sv_tree_rounds([0, 0, 0, 1, 1, 2]) == 3         # 3 at the root, 2 below node 1
    assert sv.sv_tree_rounds([0, 0, 1, 1, 2, 2, 3, 3]) == 3   # binary tree of depth 3
    assert sv.sv_tree_rounds([0, 5, 0]) == 1                  # node 2's parent is not earlier: left out
    assert sv.sv_tree_rounds(_lib_tree_parents(25)) == 3      # the 26-node top-k tree


def _lib_tree_parents(n):
    from draft_token_verification_08_amd import synth
    return synth.tree_parents(n)


def test_mtp_host_checks():
    f = sv.lib().mtp_shift_insert
    p = C.c_void_p(16)
    assert f(p, NULL, NULL, 0, p, p, 0, 4, NULL) == sv.SV_OK
    assert f(p, NULL, NULL, 0, p, p, -1, 4, NULL) == sv.SV_EINVAL
    assert f(NULL, NULL, NULL, 0, p, p, 4, 4, NULL) == sv.SV_EINVAL
    assert f(p, p, NULL, 8, p, p, 4, 4, NULL) == sv.SV_EINVAL         # one hidden pointer only
    assert f(p, p, p, 0, p, p, 4, 4, NULL) == sv.SV_EINVAL            # hidden without H
    assert f(C.c_void_p(18), NULL, NULL, 0, p, p, 4, 4, NULL) == sv.SV_EALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libspecverify.so not found"):
        _lib.lib()


def test_vocabulary_limit():
    assert sv.sv_workspace_bytes(4, 4, 1024 * 2048, sv.SV_BF16) > 0
    assert sv.sv_workspace_bytes(4, 4, 1024 * 2048 + 1, sv.SV_BF16) == 0
    assert sv.sv_workspace_bytes(4, 4, 1024 * 1024 + 1, sv.SV_F32) == 0
    assert _sample(V=1024 * 2048 + 1) == sv.SV_EINVAL
    assert _greedy(V=1024 * 1024 + 1) == sv.SV_EINVAL


def test_sample_rows_host_checks():
    f = sv.lib().sv_sample_rows
    p = C.c_void_p(16)
    ws = C.c_void_p(256)
    args = lambda **kw: [kw.get(k, v) for k, v in dict(z=p, dt=sv.SV_BF16, R=2, ri=NULL, T=p, u=p, B=4, V=100,
                                                       tok=p, fl=NULL, st=NULL, ws=ws, wsb=1 << 20, s=NULL).items()]
    assert f(*args(B=0)) == sv.SV_OK
    assert f(*args(R=0)) == sv.SV_EINVAL
    assert f(*args(z=NULL)) == sv.SV_EINVAL
    assert f(*args(tok=NULL)) == sv.SV_EINVAL
    assert f(*args(ri=C.c_void_p(18))) == sv.SV_EALIGN
    assert f(*args(wsb=8)) == sv.SV_EWORKSPACE
    assert f(*args(st=C.c_void_p(18))) == sv.SV_EALIGN


def _addr(k):
    """Distinct fake device addresses (never dereferenced: host checks only)."""
    return C.c_void_p((1 << 40) + (k << 32))


def _greedy_mtp(**kw):
    args = dict(t=_addr(0), dt=sv.SV_BF16, x=_addr(1), L=_addr(2), B=4, n=4, V=1024, acc=_addr(3), emi=_addr(4),
                fl=NULL, tok=_addr(5), hs=_addr(6), hd=_addr(7), H=64, ws=_addr(8), wsb=1 << 20, s=NULL)
    args.update(kw)
    return sv.lib().spec_verify_greedy_mtp(*args.values())


def _sample_mtp(**kw):
    args = dict(t=_addr(0), d=_addr(9), dt=sv.SV_BF16, x=_addr(1), L=_addr(2), T=_addr(10), u=_addr(11), B=4, n=4,
                V=1024, acc=_addr(3), emi=_addr(4), lse=NULL, fl=NULL, tok=_addr(5), hs=_addr(6), hd=_addr(7),
                H=64, ws=_addr(8), wsb=1 << 20, s=NULL)
    args.update(kw)
    return sv.lib().spec_verify_sample_mtp(*args.values())


def test_fused_mtp_host_checks():
    for f in (_greedy_mtp, _sample_mtp):
        assert f(B=0) == sv.SV_OK
        assert f(tok=NULL) == sv.SV_EINVAL                     # tokens required
        assert f(hs=NULL) == sv.SV_EINVAL                      # one hidden pointer only
        assert f(hd=NULL) == sv.SV_EINVAL
        assert f(H=0) == sv.SV_EINVAL                          # hidden without H
        assert f(H=-1) == sv.SV_EINVAL
        assert f(tok=C.c_void_p((1 << 40) + (5 << 32) + 2)) == sv.SV_EALIGN
        assert f(hs=C.c_void_p((1 << 40) + (6 << 32) + 1)) == sv.SV_EALIGN
        # aliasing: the copy and the token shift run inside the verify kernels
        assert f(tok=_addr(4)) == sv.SV_EINVAL                 # tokens == emitted
        assert f(tok=C.c_void_p((1 << 40) + (1 << 32) + 8)) == sv.SV_EINVAL  # inside draft_tokens
        assert f(hd=_addr(0)) == sv.SV_EINVAL                  # hidden_dst over the target logits
        assert f(hd=_addr(8)) == sv.SV_EINVAL                  # hidden_dst over the workspace
        assert f(hd=C.c_void_p((1 << 40) + (6 << 32) + 256)) == sv.SV_EINVAL  # partial overlap with hidden_src
        assert f(hs=NULL, hd=NULL, H=0, wsb=8) == sv.SV_EWORKSPACE


def test_mtp_partial_overlap_rejected():
    f = sv.lib().mtp_shift_insert
    p = C.c_void_p(16)
    src = C.c_void_p(1 << 20)
    assert f(p, src, C.c_void_p((1 << 20) + 64), 64, p, p, 4, 4, NULL) == sv.SV_EINVAL


def _sample_ex(**kw):
    args = dict(t=_addr(0), d=_addr(9), dt=sv.SV_BF16, x=_addr(1), L=_addr(2), T=_addr(10), u=_addr(11),
                ds=_addr(12), B=4, n=4, V=1024, acc=_addr(3), emi=_addr(4), lse=NULL, fl=NULL, tok=NULL, hs=NULL,
                hd=NULL, H=0, ws=_addr(8), wsb=1 << 20, s=NULL)
    args.update(kw)
    return sv.lib().spec_verify_sample_ex(*args.values())


def test_sample_ex_host_checks():
    assert _sample_ex(B=0) == sv.SV_OK
    assert _sample_ex(d=NULL) == sv.SV_EINVAL                  # draft statistics still need the draft rows
    assert _sample_ex(ds=C.c_void_p((1 << 40) + (12 << 32) + 2)) == sv.SV_EALIGN
    assert _sample_ex(hs=_addr(6), hd=_addr(7), H=64) == sv.SV_EINVAL   # hidden buffers without tokens
    assert _sample_ex(tok=_addr(5), hd=_addr(12), hs=_addr(6), H=64) == sv.SV_EINVAL  # hidden_dst over draft_stats
    assert _sample_ex(wsb=8) == sv.SV_EWORKSPACE


def _lmhead(**kw):
    args = dict(h=_addr(0), w=_addr(9), H=128, x=_addr(1), L=_addr(2), B=4, n=4, V=1000, acc=_addr(3),
                emi=_addr(4), fl=NULL, tok=_addr(5), hd=_addr(7), ws=_addr(8), wsb=1 << 20, s=NULL)
    args.update(kw)
    return sv.lib().spec_verify_greedy_lmhead(*args.values())


def test_lmhead_host_checks():
    assert _lmhead(B=0) == sv.SV_OK
    assert _lmhead(H=100) == sv.SV_EINVAL                       # H not a multiple of 64
    assert _lmhead(H=0) == sv.SV_EINVAL
    assert _lmhead(V=0) == sv.SV_EINVAL
    assert _lmhead(n=sv.SV_MAX_DRAFT + 1) == sv.SV_EINVAL
    assert _lmhead(V=1 << 22, H=1 << 12) == sv.SV_EINVAL          # weight offsets beyond 32 bits of vectors
    assert _lmhead(h=NULL) == sv.SV_EINVAL
    assert _lmhead(w=NULL) == sv.SV_EINVAL
    assert _lmhead(tok=NULL) == sv.SV_EINVAL                     # hidden_dst needs the token step
    assert _lmhead(h=C.c_void_p((1 << 40) + 8)) == sv.SV_EALIGN  # 16-byte vectors
    assert _lmhead(w=C.c_void_p((1 << 40) + (9 << 32) + 8)) == sv.SV_EALIGN
    assert _lmhead(hd=C.c_void_p((1 << 40) + (7 << 32) + 8)) == sv.SV_EALIGN
    assert _lmhead(wsb=8) == sv.SV_EWORKSPACE
    assert _lmhead(tok=_addr(4)) == sv.SV_EINVAL                 # tokens == emitted
    assert _lmhead(hd=_addr(9)) == sv.SV_EINVAL                  # hidden_dst over the weight
    assert _lmhead(hd=C.c_void_p((1 << 40) + 4096)) == sv.SV_EINVAL  # partial overlap with hidden
    f = sv.lib().sv_lmhead_logits_debug
    assert f(_addr(0), _addr(9), 0, 64, 10, _addr(3), NULL) == sv.SV_OK
    assert f(_addr(0), _addr(9), 4, 96, 10, _addr(3), NULL) == sv.SV_EINVAL
    assert f(C.c_void_p((1 << 40) + 4), _addr(9), 4, 64, 10, _addr(3), NULL) == sv.SV_EALIGN
    assert f(_addr(0), _addr(9), 4, 64, 10, NULL, NULL) == sv.SV_EINVAL



def test_residual_debug_host_checks():
    f = sv.lib().sv_residual_weights_debug
    a = lambda **kw: [kw.get(k, v) for k, v in dict(t=_addr(0), d=_addr(1), dt=sv.SV_BF16, T=_addr(2), rows=4,
                                                     V=1000, w=_addr(3), tw=NULL, info=NULL, s=NULL).items()]
    assert f(*a(rows=0)) == sv.SV_OK
    assert f(*a(rows=-1)) == sv.SV_EINVAL
    assert f(*a(V=0)) == sv.SV_EINVAL
    assert f(*a(dt=3)) == sv.SV_EINVAL
    assert f(*a(d=NULL)) == sv.SV_EINVAL
    assert f(*a(w=NULL)) == sv.SV_EINVAL
    assert f(*a(tw=C.c_void_p((1 << 40) + 4))) == sv.SV_EALIGN
    assert f(*a(V=1024 * 2048 + 1)) == sv.SV_EINVAL


def test_noalloc_size_checks_touch_nothing():
    """The no-allocation entry point rejects sizes before any device call.  Data
    pointers are NULL: a call that passed a check could still launch nothing."""
    f = sv.lib().spec_verify_sample_ex_noalloc
    a = lambda **kw: [kw.get(k, v) for k, v in dict(
        t=NULL, d=NULL, dt=sv.SV_BF16, x=NULL, L=NULL, T=NULL, u=NULL, ds=NULL, B=4, n=4,
        V=1024, acc=NULL, emi=NULL, lse=NULL, fl=NULL, tok=NULL, hs=NULL, hd=NULL, H=0, s=NULL).items()]
    assert f(*a(B=0)) == sv.SV_OK
    assert f(*a(n=sv.SV_MAX_DRAFT + 1)) == sv.SV_EINVAL
    assert f(*a(V=0)) == sv.SV_EINVAL
    assert f(*a(dt=4)) == sv.SV_EINVAL
    big = sv.sv_workspace_bytes(32768, 8, 152064, sv.SV_BF16)
    assert big > 2 * (16 << 20), big
    assert f(*a(B=32768, n=8, V=152064)) == sv.SV_EWORKSPACE      # beyond SV_NOALLOC_SCRATCH_BYTES


def test_noalloc_capacity_as_documented():
    """The capacities the header states for the static workspace (16 MiB) are
    the largest batches whose sv_workspace_bytes fit it."""
    text = open(HEADER).read()
    cap = 16 << 20
    assert "SV_NOALLOC_SCRATCH_BYTES (16u << 20)" in text
    for B, n, V in ((5262, 8, 152064), (6422, 4, 128256)):
        assert f"{B} at n = {n}" in text or f"B up to {B} at n = {n}" in text, B
        assert sv.sv_workspace_bytes(B, n, V, sv.SV_BF16) <= cap < sv.sv_workspace_bytes(B + 1, n, V, sv.SV_BF16)
