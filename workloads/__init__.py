"""Seeded synthetic inputs for the speculative-sampling verify step.

This module is shared by the fp64 oracle tests, the GPU parity tests and the
benchmark.  It produces *inputs only*: target/draft logit rows, drafted tokens,
uniforms and per-sequence temperatures.  It holds none of the verify step's
arithmetic (no softmax, no acceptance ratio, no residual, no inverse CDF).
Draft tokens are drawn from the draft distribution with the Gumbel-max trick
(argmax of logits/T plus standard Gumbel noise), which samples from
softmax(logits/T) without forming it; greedy (T=0) sequences draft by argmax of
the draft logits, as the greedy branch of the drafting loop does on the page
"投机解码" (docs.ifdog.com), section 动手实践.

Layout (the same one the C ABI takes):
  * sequence b has k_b drafted tokens; ``offsets`` is the prefix sum of k_b;
  * target row for (b, i), i = 0..k_b, is row ``offsets[b] + b + i`` of
    ``target``; row i scores drafted token i and row k_b is the bonus row;
  * draft row for (b, i), i = 0..k_b-1, is row ``offsets[b] + i`` of ``draft``;
  * ``uniforms[offsets[b] + b + i]`` is the accept uniform of position i for
    i < k_b and the draw uniform for i = k_b.

Every random number comes from numpy's Philox bit generator keyed by
``SeedSequence([config_id, trial, b, role, i])``, so a row is reproducible on
its own and rows can be generated in parallel threads.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "CONFIGS", "Workload", "make_workload", "assemble", "bf16_round",
    "bf16_to_f32", "logits_as_f32", "stored_bytes_per_elem",
]

# Seed roles.
_ROLE_TARGET, _ROLE_DRAFT, _ROLE_GUMBEL, _ROLE_UNIF, _ROLE_SEQ = 0, 1, 2, 3, 4
_ROLE_CONFIG = 0xC0

# The five workload shapes (name -> recipe).  "kind" picks the target logit
# generator; "draft" picks how draft logits relate to target logits.
CONFIGS = {
    # B=1, k=4, V=32000 fp32, T=1; target iid N(0, 2^2); draft = target + N(0, 0.5^2)
    "c1": dict(cid=1, B=1, k=4, V=32000, dtype="f32", T=1.0,
               kind="gauss", draft="noise", sigma=(0.5, 0.5)),
    # B=1, k=5, V=128256 bf16 at T=1; Zipf-shaped targets; draft = target + N(0, 1)
    "c2": dict(cid=2, B=1, k=5, V=128256, dtype="bf16", T=1.0,
               kind="zipf", draft="noise", sigma=(1.0, 1.0)),
    # same logits as c2, greedy (T=0)
    "c2g": dict(cid=2, B=1, k=5, V=128256, dtype="bf16", T=0.0,
                kind="zipf", draft="noise", sigma=(1.0, 1.0)),
    # B=64, k=4, V=128256 bf16, T=0.7; per-sequence draft noise sigma ~ U[0.2, 2.0]
    "c3": dict(cid=3, B=64, k=4, V=128256, dtype="bf16", T=0.7,
               kind="zipf", draft="noise", sigma=(0.2, 2.0)),
    # B=256, k=8, V=152064 bf16, T=1; first half near-identical drafts
    # (noise 0.1), second half independent N(0, 2^2) draft logits
    "c4": dict(cid=4, B=256, k=8, V=152064, dtype="bf16", T=1.0,
               kind="gauss", draft="halves", sigma=(0.1, 0.1)),
    # B=512, k_b ~ U{1..10}, V=128256 bf16, T_b in {0, 0.6, 1.0};
    # draft noise sigma ~ U[0.1, 2.0]
    "c5": dict(cid=5, B=512, k=(1, 10), V=128256, dtype="bf16", T=(0.0, 0.6, 1.0),
               kind="zipf", draft="noise", sigma=(0.1, 2.0)),
}

_GAUSS_STD = 2.0          # target logits N(0, 2^2) (and independent drafts)
_ZIPF_A, _ZIPF_B, _ZIPF_JITTER = 8.0, 1.1, 0.3


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(list(key))))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def logits_as_f32(rows: np.ndarray) -> np.ndarray:
    """Stored logits (uint16 bf16 bits or float32) -> float32 values (exact)."""
    if rows.dtype == np.uint16:
        return bf16_to_f32(rows)
    return np.asarray(rows, dtype=np.float32)


def stored_bytes_per_elem(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


@dataclasses.dataclass
class Workload:
    name: str
    V: int
    B: int
    dtype: str                 # "f32" | "bf16"
    k: np.ndarray              # int32 [B]
    offsets: np.ndarray        # int32 [B+1]
    target: np.ndarray         # [total+B, V] float32 or uint16 (bf16 bits)
    draft: np.ndarray          # [total, V]   same dtype as target
    tokens: np.ndarray         # int32 [total]
    uniforms: np.ndarray       # float32 [total+B]
    temperature: np.ndarray    # float32 [B]
    sigma: np.ndarray          # float64 [B] draft-noise parameter (metadata)

    @property
    def total(self) -> int:
        return int(self.offsets[-1])

    @property
    def elem_bytes(self) -> int:
        return stored_bytes_per_elem(self.dtype)

    def target_row(self, b: int, i: int) -> int:
        return int(self.offsets[b]) + b + i

    def draft_row(self, b: int, i: int) -> int:
        return int(self.offsets[b]) + i

    def uniform_slot(self, b: int, i: int) -> int:
        return int(self.offsets[b]) + b + i

    def subset(self, seqs) -> "Workload":
        """A new workload holding only the listed sequences (copies rows)."""
        seqs = [int(s) for s in seqs]
        k = self.k[seqs].astype(np.int32)
        off = np.zeros(len(seqs) + 1, np.int32)
        off[1:] = np.cumsum(k)
        t_rows, d_rows, u_slots = [], [], []
        for b in seqs:
            kb = int(self.k[b])
            t_rows += [self.target_row(b, i) for i in range(kb + 1)]
            d_rows += [self.draft_row(b, i) for i in range(kb)]
            u_slots += [self.uniform_slot(b, i) for i in range(kb + 1)]
        d_idx = np.array(d_rows, dtype=np.int64)
        return Workload(
            name=f"{self.name}[subset]", V=self.V, B=len(seqs), dtype=self.dtype,
            k=k, offsets=off,
            target=self.target[np.array(t_rows, dtype=np.int64)],
            draft=self.draft[d_idx] if len(d_idx) else self.draft[:0],
            tokens=self.tokens[d_idx] if len(d_idx) else self.tokens[:0],
            uniforms=self.uniforms[np.array(u_slots, dtype=np.int64)],
            temperature=self.temperature[seqs].copy(), sigma=self.sigma[seqs].copy())


def assemble(target_rows, draft_rows, tokens, uniforms, temperature, k, dtype="f32",
             name="custom") -> Workload:
    """Build a workload from explicit arrays laid out as described above.

    ``target_rows``/``draft_rows`` are float arrays (values) or uint16 bf16
    bits; float values are stored as fp32 (dtype "f32") or rounded to bf16.
    """
    k = np.asarray(k, dtype=np.int32)
    off = np.zeros(len(k) + 1, np.int32)
    off[1:] = np.cumsum(k)
    V = int(np.asarray(target_rows).shape[1])

    def store(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:
            assert dtype == "bf16"
            return np.ascontiguousarray(a)
        a = np.ascontiguousarray(a, dtype=np.float32)
        return bf16_round(a) if dtype == "bf16" else a

    draft = np.asarray(draft_rows)
    if draft.size == 0:
        draft = np.zeros((0, V), np.float32)
    return Workload(
        name=name, V=V, B=len(k), dtype=dtype, k=k, offsets=off,
        target=store(target_rows).reshape(-1, V), draft=store(draft).reshape(-1, V),
        tokens=np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1),
        uniforms=np.ascontiguousarray(uniforms, dtype=np.float32).reshape(-1),
        temperature=np.ascontiguousarray(temperature, dtype=np.float32).reshape(-1),
        sigma=np.zeros(len(k)))


def _zipf_base(V: int) -> np.ndarray:
    r = np.arange(1, V + 1, dtype=np.float64)
    return (_ZIPF_A - _ZIPF_B * np.log(r)).astype(np.float32)


def make_workload(name: str, trial: int = 0, B: int | None = None, V: int | None = None,
                  k: int | None = None, threads: int | None = None,
                  shuffle_halves: bool = False) -> Workload:
    """Generate one of the named workloads.

    ``B``, ``V`` and ``k`` override the recipe's sizes (smaller parity cases
    keep the recipe's value distributions).  For "c4", ``shuffle_halves``
    assigns the near-identical / independent draft kinds to a random half of
    the sequences instead of the first / second half.
    """
    spec = CONFIGS[name]
    cid = spec["cid"]
    B = int(spec["B"] if B is None else B)
    V = int(spec["V"] if V is None else V)
    dtype = spec["dtype"]
    crng = _rng(cid, trial, _ROLE_CONFIG)

    # per-sequence k and T
    if k is not None:
        kk = np.full(B, int(k), np.int32)
    elif isinstance(spec["k"], tuple):
        lo, hi = spec["k"]
        kk = crng.integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        kk = np.full(B, spec["k"], np.int32)
    if isinstance(spec["T"], tuple):
        temps = np.asarray(spec["T"], np.float32)[crng.integers(0, len(spec["T"]), size=B)]
    else:
        temps = np.full(B, spec["T"], np.float32)
    off = np.zeros(B + 1, np.int32)
    off[1:] = np.cumsum(kk)
    total = int(off[-1])

    # per-sequence draft-noise sigma and draft kind
    sig = np.zeros(B)
    indep = np.zeros(B, bool)
    lo, hi = spec["sigma"]
    for b in range(B):
        sig[b] = lo if lo == hi else _rng(cid, trial, b, _ROLE_SEQ).uniform(lo, hi)
    if spec["draft"] == "halves":
        if shuffle_halves:
            perm = crng.permutation(B)
            indep[perm[B // 2:]] = True
        else:
            indep[B // 2:] = True
        sig[indep] = np.nan

    store_dt = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((total + B, V), store_dt)
    draft = np.empty((total, V), store_dt)
    tokens = np.empty(total, np.int32)
    uniforms = np.empty(total + B, np.float32)
    zbase = _zipf_base(V) if spec["kind"] == "zipf" else None

    def target_values(b, i):
        g = _rng(cid, trial, b, _ROLE_TARGET, i)
        if spec["kind"] == "gauss":
            return g.standard_normal(V, dtype=np.float32) * np.float32(_GAUSS_STD)
        vals = zbase + g.standard_normal(V, dtype=np.float32) * np.float32(_ZIPF_JITTER)
        out = np.empty(V, np.float32)
        out[g.permutation(V)] = vals      # rank r lands on a random token id
        return out

    def store(x):
        return bf16_round(x) if dtype == "bf16" else x

    def gen_sequence(b):
        kb = int(kk[b])
        base_t = int(off[b]) + b
        base_d = int(off[b])
        T = float(temps[b])
        for i in range(kb + 1):
            zt = target_values(b, i)
            target[base_t + i] = store(zt)
            if i == kb:
                break
            g = _rng(cid, trial, b, _ROLE_DRAFT, i)
            if indep[b]:
                zd = g.standard_normal(V, dtype=np.float32) * np.float32(_GAUSS_STD)
            else:
                zd = zt + g.standard_normal(V, dtype=np.float32) * np.float32(sig[b])
            draft[base_d + i] = store(zd)
            zd_stored = logits_as_f32(draft[base_d + i]).astype(np.float64)
            if T == 0.0:
                tokens[base_d + i] = int(np.argmax(zd_stored))
            else:
                e = _rng(cid, trial, b, _ROLE_GUMBEL, i).standard_exponential(V)
                tokens[base_d + i] = int(np.argmax(zd_stored / T - np.log(e)))
        uniforms[base_t:base_t + kb + 1] = _rng(cid, trial, b, _ROLE_UNIF).random(
            kb + 1, dtype=np.float32)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if B == 1 or nthreads == 1:
        for b in range(B):
            gen_sequence(b)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(gen_sequence, range(B)))
    return Workload(name=name, V=V, B=B, dtype=dtype, k=kk, offsets=off, target=target,
                    draft=draft, tokens=tokens, uniforms=uniforms, temperature=temps,
                    sigma=sig)
