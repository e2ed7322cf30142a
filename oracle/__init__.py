"""CPU oracle for the verify-and-sample step and the MTP shift/insert.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this package.  The GPU library and its Python binding never
import it.  The arithmetic lives in ``specverify_oracle.c`` (plain C, double
precision); this module only loads the shared object and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "specverify_oracle.c")
LIB = os.path.join(HERE, "libspecverify_oracle.so")

F32, BF16, F64 = 0, 1, 2
FLAG_LEN_CLAMPED, FLAG_TOKEN_OOR, FLAG_BAD_TEMP, FLAG_BAD_UNIFORM, FLAG_ZERO_RESIDUAL = 1, 2, 4, 8, 16
FLAG_ROW_CLAMPED = 32
FLAG_BAD_PARENT = 64


def build(out_path: str = LIB, plant: int = 0, sanitize: bool = False) -> str:
    """Compile the oracle with gcc.  ``plant`` > 0 builds a test-only variant that
    carries one deliberate mistake (used by negative-control tests);
    ``sanitize`` builds it with AddressSanitizer and UndefinedBehaviorSanitizer
    (load it in a process that preloads their runtimes)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-D_POSIX_C_SOURCE=200809L", SRC, "-o", out_path, "-lm", "-lpthread"]
    if plant:
        cmd.insert(1, f"-DSV_ORACLE_PLANT={int(plant)}")
    if sanitize:
        cmd[1:2] = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all"]
    subprocess.run(cmd, check=True)
    return out_path


class Oracle:
    """numpy-facing wrapper around one build of the oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(path)
        self.lib = C.CDLL(path)
        L = self.lib
        vp, i32p, f32p, f64p, u32p = C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p
        L.sv_oracle_verify_sample.argtypes = [vp, vp, C.c_int, i32p, i32p, f32p, f32p, C.c_int, C.c_int,
                                              C.c_int, i32p, i32p, f64p, f64p, f64p, u32p, C.c_int]
        L.sv_oracle_verify_sample.restype = C.c_int
        L.sv_oracle_verify_greedy.argtypes = [vp, C.c_int, i32p, i32p, C.c_int, C.c_int, C.c_int, i32p,
                                              i32p, u32p, C.c_int]
        L.sv_oracle_verify_greedy.restype = C.c_int
        L.sv_oracle_mtp_shift_insert.argtypes = [i32p, vp, vp, C.c_int, C.c_int, i32p, i32p, C.c_int, C.c_int]
        L.sv_oracle_mtp_shift_insert.restype = C.c_int
        L.sv_oracle_softmax_row.argtypes = [vp, C.c_int, C.c_int, C.c_double, f64p]
        L.sv_oracle_softmax_row.restype = C.c_double
        L.sv_oracle_argmax_row.argtypes = [vp, C.c_int, C.c_int]
        L.sv_oracle_argmax_row.restype = C.c_int
        L.sv_oracle_draw_weights.argtypes = [f64p, C.c_int, C.c_double, f64p]
        L.sv_oracle_draw_weights.restype = C.c_int
        L.sv_oracle_sample_rows.argtypes = [vp, C.c_int, C.c_int, i32p, f32p, f32p, C.c_int, C.c_int, i32p,
                                            u32p, C.c_int]
        L.sv_oracle_sample_rows.restype = C.c_int
        L.sv_oracle_lmhead_logits.argtypes = [vp, vp, C.c_int, C.c_int, C.c_int, i32p, C.c_int, f64p, C.c_int]
        L.sv_oracle_lmhead_logits.restype = C.c_int
        L.sv_oracle_verify_tree_greedy.argtypes = [vp, C.c_int, i32p, i32p, i32p, C.c_int, C.c_int, C.c_int,
                                                   i32p, i32p, i32p, u32p]
        L.sv_oracle_verify_tree_greedy.restype = C.c_int
        L.sv_oracle_verify_tree_sample.argtypes = [vp, vp, C.c_int, i32p, i32p, i32p, f32p, f32p, C.c_int, C.c_int,
                                                   C.c_int, C.c_int, i32p, i32p, i32p, f64p, f64p, u32p]
        L.sv_oracle_verify_tree_sample.restype = C.c_int
        L.sv_oracle_plant.argtypes = []
        L.sv_oracle_plant.restype = C.c_int

    # -- marshalling helpers -------------------------------------------------
    @staticmethod
    def _logits(a: np.ndarray):
        """Accept fp32 or float64 arrays, or bf16 bit patterns stored as uint16."""
        a = np.ascontiguousarray(a)
        if a.dtype == np.float32:
            return a, F32
        if a.dtype == np.float64:
            return a, F64
        if a.dtype == np.uint16:
            return a, BF16
        raise TypeError(f"logits must be float32, float64 or uint16 (bf16 bits), got {a.dtype}")

    @staticmethod
    def _p(a):
        return None if a is None else a.ctypes.data_as(C.c_void_p)

    @property
    def plant(self) -> int:
        return self.lib.sv_oracle_plant()

    # -- entry points --------------------------------------------------------
    def verify_sample(self, target, draft, draft_tokens, draft_lens, temperature, uniforms, threads=1):
        target, dt = self._logits(target)
        B, n1, V = target.shape
        n = n1 - 1
        if draft is not None:
            draft, dt2 = self._logits(draft)
            assert dt2 == dt and draft.shape == (B, n, V)
        draft_tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, n)
        draft_lens = np.ascontiguousarray(draft_lens, dtype=np.int32).reshape(B)
        temperature = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
        uniforms = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, n + 1)
        acc = np.empty(B, np.int32)
        emi = np.empty((B, n + 1), np.int32)
        lse = np.empty((B, 2 * n + 1), np.float64)
        am = np.empty((B, n), np.float64)
        dm = np.empty(B, np.float64)
        fl = np.empty(B, np.uint32)
        rc = self.lib.sv_oracle_verify_sample(
            self._p(target), self._p(draft), dt, self._p(draft_tokens), self._p(draft_lens),
            self._p(temperature), self._p(uniforms), B, n, V, self._p(acc), self._p(emi),
            self._p(lse), self._p(am), self._p(dm), self._p(fl), int(threads))
        if rc != 0:
            raise RuntimeError(f"sv_oracle_verify_sample failed: {rc}")
        return dict(accepted_len=acc, emitted=emi, row_lse=lse, accept_margin=am,
                    draw_margin=dm, seq_flags=fl)

    def verify_greedy(self, target, draft_tokens, draft_lens, threads=1):
        target, dt = self._logits(target)
        B, n1, V = target.shape
        n = n1 - 1
        draft_tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, n)
        draft_lens = np.ascontiguousarray(draft_lens, dtype=np.int32).reshape(B)
        acc = np.empty(B, np.int32)
        emi = np.empty((B, n + 1), np.int32)
        fl = np.empty(B, np.uint32)
        rc = self.lib.sv_oracle_verify_greedy(self._p(target), dt, self._p(draft_tokens),
                                              self._p(draft_lens), B, n, V, self._p(acc),
                                              self._p(emi), self._p(fl), int(threads))
        if rc != 0:
            raise RuntimeError(f"sv_oracle_verify_greedy failed: {rc}")
        return dict(accepted_len=acc, emitted=emi, seq_flags=fl)

    def verify_tree_greedy(self, target, draft_tokens, draft_parents, draft_lens):
        """Greedy tree verification (see sv_oracle_verify_tree_greedy)."""
        target, dt = self._logits(target)
        B, n1, V = target.shape
        n = n1 - 1
        x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, n)
        par = np.ascontiguousarray(draft_parents, dtype=np.int32).reshape(B, n)
        L = np.ascontiguousarray(draft_lens, dtype=np.int32).reshape(B)
        acc = np.empty(B, np.int32)
        emi = np.empty((B, n + 1), np.int32)
        path = np.empty((B, max(n, 1)), np.int32)[:, :n].copy()
        fl = np.empty(B, np.uint32)
        rc = self.lib.sv_oracle_verify_tree_greedy(self._p(target), dt, self._p(x), self._p(par), self._p(L), B, n,
                                                   V, self._p(acc), self._p(emi), self._p(path), self._p(fl))
        if rc != 0:
            raise RuntimeError(f"sv_oracle_verify_tree_greedy failed: {rc}")
        return dict(accepted_len=acc, emitted=emi, path=path, seq_flags=fl)

    def verify_tree_sample(self, target, draft, draft_tokens, draft_parents, draft_lens, temperature, uniforms,
                           max_rounds=None):
        """Sampling tree verification (see sv_oracle_verify_tree_sample);
        max_rounds None: no limit on the residual sums of a walk."""
        target, dt = self._logits(target)
        B, n1, V = target.shape
        n = n1 - 1
        draft, dt2 = self._logits(draft)
        assert dt2 == dt and draft.shape == (B, n, V)
        x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, n)
        par = np.ascontiguousarray(draft_parents, dtype=np.int32).reshape(B, n)
        L = np.ascontiguousarray(draft_lens, dtype=np.int32).reshape(B)
        T = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
        u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, n + 1)
        acc = np.empty(B, np.int32)
        emi = np.empty((B, n + 1), np.int32)
        path = np.empty((B, max(n, 1)), np.int32)[:, :n].copy()
        am = np.empty((B, n), np.float64)
        dm = np.empty(B, np.float64)
        fl = np.empty(B, np.uint32)
        rc = self.lib.sv_oracle_verify_tree_sample(self._p(target), self._p(draft), dt, self._p(x), self._p(par),
                                                   self._p(L), self._p(T), self._p(u), B, n, V,
                                                   -1 if max_rounds is None else int(max_rounds), self._p(acc),
                                                   self._p(emi), self._p(path), self._p(am), self._p(dm), self._p(fl))
        if rc != 0:
            raise RuntimeError(f"sv_oracle_verify_tree_sample failed: {rc}")
        return dict(accepted_len=acc, emitted=emi, path=path, accept_margin=am, draw_margin=dm, seq_flags=fl)

    def mtp_shift_insert(self, tokens, hidden_src, accepted_len, emitted, copy_hidden=True):
        """Returns (new_tokens, hidden_dst); inputs are not modified."""
        tok = np.array(tokens, dtype=np.int32, copy=True, order="C")
        B, n1 = tok.shape
        n = n1 - 1
        acc = np.ascontiguousarray(accepted_len, dtype=np.int32).reshape(B)
        emi = np.ascontiguousarray(emitted, dtype=np.int32).reshape(B, n1)
        if hidden_src is not None and copy_hidden:
            hs = np.ascontiguousarray(hidden_src)
            hd = np.zeros_like(hs)
            H = hs.shape[-1]
            rc = self.lib.sv_oracle_mtp_shift_insert(self._p(tok), self._p(hs), self._p(hd), H,
                                                     hs.dtype.itemsize, self._p(acc), self._p(emi), B, n)
        else:
            hd = None
            rc = self.lib.sv_oracle_mtp_shift_insert(self._p(tok), None, None, 0, 0, self._p(acc),
                                                     self._p(emi), B, n)
        if rc != 0:
            raise RuntimeError(f"sv_oracle_mtp_shift_insert failed: {rc}")
        return tok, hd

    def sample_rows(self, logits, temperature, uniforms, row_index=None, threads=1):
        """One token per sequence from logits[b][row_index[b]] (row 0 if None)."""
        logits, dt = self._logits(logits)
        B, R, V = logits.shape
        ri = None if row_index is None else np.ascontiguousarray(row_index, dtype=np.int32).reshape(B)
        temperature = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
        uniforms = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B)
        tok = np.empty(B, np.int32)
        fl = np.empty(B, np.uint32)
        rc = self.lib.sv_oracle_sample_rows(self._p(logits), dt, R, self._p(ri), self._p(temperature),
                                            self._p(uniforms), B, V, self._p(tok), self._p(fl), int(threads))
        if rc != 0:
            raise RuntimeError(f"sv_oracle_sample_rows failed: {rc}")
        return dict(tokens=tok, seq_flags=fl)

    def lmhead_logits(self, hidden, weight, rows=None, threads=1):
        """Logits of the target's logit projection in double: hidden [M, H] and
        weight [V, H] as bf16 bit patterns (uint16); rows selects hidden rows
        (all M when None).  Returns float64 [len(rows), V]."""
        h = np.ascontiguousarray(hidden, dtype=np.uint16)
        w = np.ascontiguousarray(weight, dtype=np.uint16)
        H = h.shape[-1]
        h = h.reshape(-1, H)
        M = h.shape[0]
        V = w.shape[0]
        assert w.shape == (V, H)
        r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32).reshape(-1)
        nrows = M if r is None else r.shape[0]
        out = np.empty((nrows, V), np.float64)
        rc = self.lib.sv_oracle_lmhead_logits(self._p(h), self._p(w), M, H, V, self._p(r), nrows,
                                              self._p(out), int(threads))
        if rc != 0:
            raise RuntimeError(f"sv_oracle_lmhead_logits failed: {rc}")
        return out

    def softmax_row(self, z, T):
        z, dt = self._logits(np.asarray(z).reshape(-1))
        V = z.shape[0]
        p = np.empty(V, np.float64)
        lse = self.lib.sv_oracle_softmax_row(self._p(z), dt, V, float(T), self._p(p))
        return lse, p

    def argmax_row(self, z):
        z, dt = self._logits(np.asarray(z).reshape(-1))
        return self.lib.sv_oracle_argmax_row(self._p(z), dt, z.shape[0])

    def draw_weights(self, w, u):
        w = np.ascontiguousarray(w, dtype=np.float64)
        m = np.zeros(1, np.float64)
        y = self.lib.sv_oracle_draw_weights(self._p(w), w.shape[0], float(u), self._p(m))
        return y, float(m[0])


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
