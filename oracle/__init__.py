"""fp64 CPU oracle of the speculative-sampling verify step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the GPU library and
its Python binding never do.  The arithmetic lives in ``oracle.c`` (plain C,
fp64, Neumaier sums); this file only marshals numpy arrays.

Parity pins: every exported function is pinned by ``tests/test_oracle_*.py``
against the pages' equations, closed forms, library routines and brute force
(see the header of ``oracle.c`` for the pages followed).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FLAG_A, FLAG_B, FLAG_D, FLAG_E = 1, 2, 4, 8
ACCEPT_BAND, CDF_BAND = 1e-5, 1e-12

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2, no fast-math)."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC",
                           "-shared", "-fno-fast-math", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


@contextlib.contextmanager
def using_library(path: str):
    """Route every call through another build of oracle.c for the duration
    (the mutation tests build copies with planted mistakes this way)."""
    global _lib
    saved = _lib
    _lib = _open(path)
    try:
        yield
    finally:
        _lib = saved


def _load():
    """The oracle library: liboracle.so next to oracle.c (built on first
    use), or the build ORACLE_LIB names (the sanitizer test runs the pins
    against an address/undefined-behaviour sanitizer build this way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(path):
                build()
        _lib = _open(path)
    return _lib


def _open(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_verify.restype = ctypes.c_int
    lib.oracle_verify.argtypes = [P, P, i32, i64, i32, P, P, P, P, i32, i32,
                                  P, P, P, P, P, P, P, P, P, P]
    lib.oracle_verify_probs.restype = ctypes.c_int
    lib.oracle_verify_probs.argtypes = [P, P, i64, i32, i32, i32, P, P, P, P, P, P, P]
    lib.oracle_softmax_rows.restype = ctypes.c_int
    lib.oracle_softmax_rows.argtypes = [P, i32, i64, i64, ctypes.c_double, P, P, P]
    lib.oracle_inverse_cdf.restype = i64
    lib.oracle_inverse_cdf.argtypes = [P, i64, ctypes.c_float, P, P]
    lib.oracle_verify_gathered.restype = ctypes.c_int
    lib.oracle_verify_gathered.argtypes = [P, P, i32, i64, i32, P, P, P, P, P, i32, i32,
                                           P, P, P, P, P, P, P, P]
    lib.oracle_draft_sample.restype = ctypes.c_int
    lib.oracle_draft_sample.argtypes = [P, i32, i64, i32, P, P, i32, i32, P, P, P, P]
    lib.oracle_commit.restype = ctypes.c_int
    lib.oracle_commit.argtypes = [P, P, P, i32, P, P, i32, P, P]
    lib.oracle_adapt_k.restype = ctypes.c_int
    lib.oracle_adapt_k.argtypes = [P, P, i32, i32, i32, P, P, P]
    lib.oracle_ngram_draft.restype = ctypes.c_int
    lib.oracle_ngram_draft.argtypes = [P, P, i32, i32, i32, i32, i32, P, P]
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(rows: np.ndarray) -> int:
    if rows.dtype == np.float32:
        return 0
    if rows.dtype == np.uint16:
        return 1
    raise TypeError(f"stored logits must be float32 or uint16 (bf16 bits), got {rows.dtype}")


def verify(w, diag: bool = False, threads: int = 1, seqs: tuple[int, int] | None = None,
           draft_probs: np.ndarray | None = None) -> dict:
    """Run the oracle over a ``workloads.Workload`` (or any object with the
    same fields).  Returns numpy arrays: tokens [total+B], n [B], flags [B]
    and, with ``diag``, alpha/px/qx [total], Z/gap [B], row_max/row_sum
    [2*total+B] (target rows first; not for the gathered form).  ``seqs`` =
    (b0, b1) limits the work to those sequences (other outputs stay at their
    fill values).  ``draft_probs`` [total] (fp32): the drafter's gathered
    q_i(x_i), used in the accept tests instead of the draft rows' softmax
    (oracle_verify_gathered)."""
    lib = _load()
    B, V = int(w.B), int(w.V)
    off = np.ascontiguousarray(w.offsets, np.int32)
    total = int(off[-1])
    target = np.ascontiguousarray(w.target)
    draft = np.ascontiguousarray(w.draft)
    if draft.size == 0:
        draft = np.zeros((1, V), target.dtype)
    dt = _dtype_code(target)
    tokens = np.ascontiguousarray(w.tokens, np.int32)
    unif = np.ascontiguousarray(w.uniforms, np.float32)
    temp = np.ascontiguousarray(w.temperature, np.float32)
    out = dict(tokens=np.full(total + B, -1, np.int32), n=np.full(B, -2, np.int32),
               flags=np.zeros(B, np.int32))
    if diag:
        out.update(alpha=np.full(total, np.nan), px=np.full(total, np.nan),
                   qx=np.full(total, np.nan), Z=np.full(B, np.nan), gap=np.full(B, np.nan),
                   row_max=np.full(2 * total + B, np.nan),
                   row_sum=np.full(2 * total + B, np.nan))
    b0, b1 = seqs if seqs is not None else (0, B)

    qg = None
    if draft_probs is not None:
        qg = np.ascontiguousarray(draft_probs, np.float32)
        if qg.size == 0:
            qg = np.zeros(1, np.float32)
        out.pop("row_max", None)
        out.pop("row_sum", None)

    def run(rng):
        lo, hi = rng
        if qg is None:
            rc = lib.oracle_verify(
                _ptr(target), _ptr(draft), dt, V, B, _ptr(off), _ptr(tokens), _ptr(unif),
                _ptr(temp), lo, hi, _ptr(out["tokens"]), _ptr(out["n"]), _ptr(out["flags"]),
                _ptr(out.get("alpha")), _ptr(out.get("px")), _ptr(out.get("qx")),
                _ptr(out.get("Z")), _ptr(out.get("gap")), _ptr(out.get("row_max")),
                _ptr(out.get("row_sum")))
        else:
            rc = lib.oracle_verify_gathered(
                _ptr(target), _ptr(draft), dt, V, B, _ptr(off), _ptr(tokens), _ptr(qg),
                _ptr(unif), _ptr(temp), lo, hi, _ptr(out["tokens"]), _ptr(out["n"]),
                _ptr(out["flags"]), _ptr(out.get("alpha")), _ptr(out.get("px")),
                _ptr(out.get("qx")), _ptr(out.get("Z")), _ptr(out.get("gap")))
        if rc != 0:
            raise RuntimeError(f"oracle_verify failed with code {rc}")

    if threads <= 1 or b1 - b0 <= 1:
        run((b0, b1))
    else:
        edges = np.linspace(b0, b1, min(threads, b1 - b0) + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, zip(edges[:-1], edges[1:])))
    return out


def verify_probs(P: np.ndarray, Q: np.ndarray, tokens: np.ndarray, uniforms: np.ndarray,
                 k: int, shared_rows: bool) -> dict:
    """Probability-domain verify (no softmax): uniform k over B sequences.
    shared_rows: P [k+1, V] and Q [k, V] serve every sequence; otherwise
    P [B*(k+1), V], Q [B*k, V].  tokens [B, k], uniforms [B, k+1]."""
    lib = _load()
    P = np.ascontiguousarray(P, np.float64)
    Q = np.ascontiguousarray(Q, np.float64)
    V = P.shape[-1]
    tokens = np.ascontiguousarray(tokens, np.int32).reshape(-1, k) if k else \
        np.zeros((len(uniforms), 0), np.int32)
    uniforms = np.ascontiguousarray(uniforms, np.float32).reshape(-1, k + 1)
    B = uniforms.shape[0]
    if Q.size == 0:
        Q = np.zeros((1, V))
    out = dict(tokens=np.full((B, k + 1), -1, np.int32), n=np.zeros(B, np.int32),
               flags=np.zeros(B, np.int32), Z=np.zeros(B), gap=np.zeros(B))
    rc = lib.oracle_verify_probs(_ptr(P), _ptr(Q), V, B, k, int(bool(shared_rows)),
                                 _ptr(tokens), _ptr(uniforms), _ptr(out["tokens"]),
                                 _ptr(out["n"]), _ptr(out["flags"]), _ptr(out["Z"]),
                                 _ptr(out["gap"]))
    if rc != 0:
        raise RuntimeError(f"oracle_verify_probs failed with code {rc}")
    return out


def softmax_rows(rows: np.ndarray, T: float):
    """Tempered softmax of stored rows [n, V] -> (p [n, V], m [n], S [n])."""
    lib = _load()
    rows = np.ascontiguousarray(rows)
    if rows.ndim == 1:
        rows = rows[None]
    n, V = rows.shape
    p = np.empty((n, V))
    m = np.empty(n)
    S = np.empty(n)
    rc = lib.oracle_softmax_rows(_ptr(rows), _dtype_code(rows), n, V, float(T), _ptr(p),
                                 _ptr(m), _ptr(S))
    if rc != 0:
        raise RuntimeError(f"oracle_softmax_rows failed with code {rc}")
    return p, m, S


def inverse_cdf(r: np.ndarray, u: float):
    """Inverse-CDF draw over a non-negative mass row -> (t, Z, gap)."""
    lib = _load()
    r = np.ascontiguousarray(r, np.float64)
    Z = ctypes.c_double()
    gap = ctypes.c_double()
    t = lib.oracle_inverse_cdf(_ptr(r), r.size, ctypes.c_float(np.float32(u)),
                               ctypes.byref(Z), ctypes.byref(gap))
    return int(t), Z.value, gap.value


def draft_sample(logits: np.ndarray, temperature, uniforms, threads: int = 1) -> dict:
    """Draft sampler over stored rows [rows, V] (fp32 or bf16 bits): per row
    the drawn token, its probability q(x) (fp64; 1 for greedy rows), flags
    (B: u Z within 1e-12 of a CDF boundary; E: bad temperature) and the
    boundary gap."""
    lib = _load()
    logits = np.ascontiguousarray(logits)
    if logits.ndim == 1:
        logits = logits[None]
    rows, V = logits.shape
    temp = np.ascontiguousarray(np.broadcast_to(np.asarray(temperature, np.float32), (rows,)))
    unif = np.ascontiguousarray(np.asarray(uniforms, np.float32).reshape(rows))
    out = dict(tokens=np.full(rows, -1, np.int32), probs=np.full(rows, np.nan),
               flags=np.zeros(rows, np.int32), gap=np.full(rows, np.nan))

    def run(rng):
        lo, hi = rng
        rc = lib.oracle_draft_sample(_ptr(logits), _dtype_code(logits), V, rows, _ptr(temp),
                                     _ptr(unif), lo, hi, _ptr(out["tokens"]), _ptr(out["probs"]),
                                     _ptr(out["flags"]), _ptr(out["gap"]))
        if rc != 0:
            raise RuntimeError(f"oracle_draft_sample failed with code {rc}")

    if threads <= 1 or rows <= 1:
        run((0, rows))
    else:
        edges = np.linspace(0, rows, min(threads, rows) + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, zip(edges[:-1], edges[1:])))
    return out


def commit(out_tokens, out_n, offsets, seq_tokens, seq_len):
    """One round's commit: returns (seq_tokens', seq_len', committed,
    committed_offsets); the inputs are not modified."""
    lib = _load()
    out_tokens = np.ascontiguousarray(out_tokens, np.int32)
    out_n = np.ascontiguousarray(out_n, np.int32)
    offsets = np.ascontiguousarray(offsets, np.int32)
    seq = np.array(seq_tokens, np.int32, copy=True, order="C")
    L = np.array(seq_len, np.int32, copy=True)
    B, max_len = seq.shape
    committed = np.full(max(1, int(offsets[-1]) + B), -1, np.int32)
    coff = np.zeros(B + 1, np.int32)
    rc = lib.oracle_commit(_ptr(out_tokens), _ptr(out_n), _ptr(offsets), B, _ptr(seq), _ptr(L),
                           max_len, _ptr(committed), _ptr(coff))
    if rc != 0:
        raise RuntimeError(f"oracle_commit failed with code {rc}")
    return seq, L, committed[:coff[-1]], coff


class AdaptK:
    """Adaptive draft length over rounds (oracle_adapt_k); holds the
    oracle's own per-sequence history."""

    def __init__(self, B: int, min_k: int = 1, max_k: int = 10, k0=None):
        self.B, self.min_k, self.max_k = B, min_k, max_k
        self.k = np.full(B, (min_k + max_k) // 2 if k0 is None else k0, np.int32)
        self.hist = np.zeros((B, 100))
        self.count = np.zeros(B, np.int32)

    def update(self, out_n, k_used) -> np.ndarray:
        lib = _load()
        out_n = np.ascontiguousarray(out_n, np.int32)
        k_used = np.ascontiguousarray(k_used, np.int32)
        rc = lib.oracle_adapt_k(_ptr(out_n), _ptr(k_used), self.B, self.min_k, self.max_k,
                                _ptr(self.hist), _ptr(self.count), _ptr(self.k))
        if rc != 0:
            raise RuntimeError(f"oracle_adapt_k failed with code {rc}")
        return self.k.copy()


def ngram_draft(seq_tokens, seq_len, ngram_max: int, ngram_min: int, k_max: int):
    """n-gram drafts: returns (draft_tokens packed, draft_offsets [B+1])."""
    lib = _load()
    seq = np.ascontiguousarray(seq_tokens, np.int32)
    L = np.ascontiguousarray(seq_len, np.int32)
    B, max_len = seq.shape
    toks = np.full(max(1, B * k_max), -1, np.int32)
    off = np.zeros(B + 1, np.int32)
    rc = lib.oracle_ngram_draft(_ptr(seq), _ptr(L), B, max_len, ngram_max, ngram_min, k_max,
                                _ptr(toks), _ptr(off))
    if rc != 0:
        raise RuntimeError(f"oracle_ngram_draft failed with code {rc}")
    return toks[:off[-1]], off
