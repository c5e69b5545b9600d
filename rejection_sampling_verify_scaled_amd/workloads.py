"""Seeded synthetic inputs for the speculative-decoding verify step.

This module is the only code shared by the CPU oracle's tests and the HIP
path's tests and benchmark.  It produces *inputs* only: logits shaped like the
workloads the pages describe (Llama-class V=128256, DeepSeek-class V=129280,
a Qwen-size V=152064, draft lengths K=1..8), draft tokens chosen the way a
drafter would choose them, per-request temperatures and the Philox seed.  It
contains none of the verify step's arithmetic (no acceptance test, no
residual, no race); the only probability computation here is the drafter's
own choice of x_t ~ softmax(draft_t / T), which happens before the verify
step and is outside it ("Decodificación Especulativa y EAGLE", section
"El Concepto", step 1: the draft model proposes x_1..x_K ~ q).

Packed layout (shared with the C ABI):
  * request b has K_b = offsets[b+1] - offsets[b] draft tokens;
  * target rows: K_b + 1 rows per request, request b's row t at offsets[b] + b + t;
  * draft rows: K_b rows per request, request b's row t at offsets[b] + t;
  * draft token t of request b at tokens[offsets[b] + t];
  * temperature[b] == 0 selects the greedy rule for request b.

bf16 logits are stored as their raw 16-bit patterns (numpy uint16), produced
from the float64 draw by rounding to float32 and then to bf16 with
round-to-nearest-even.  Both sides of every parity test read these exact bits.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_NAMES = {DTYPE_F32: "f32", DTYPE_BF16: "bf16"}

GEN_TAG = 0x5356  # first word of every generator seed sequence


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes and value distributions."""

    cfg: int                 # 1-based workload number
    name: str
    B: int
    K: Optional[int]         # fixed draft length, or None when ragged
    K_range: tuple           # (lo, hi) inclusive for ragged batches
    V: int
    dtype: int
    target_sigma: float
    peak_frac: float         # fraction of entries boosted per target row
    peak_boost: float
    draft_sigma: tuple       # per-request draft noise: ("cycle", values) | ("uniform", lo, hi)
    temperature: tuple       # ("split", T_first_half, T_second_half) | ("choice", values) | ("const", T)
    max_k: int

    @property
    def n_peaks(self) -> int:
        return int(round(self.peak_frac * self.V))


WORKLOADS = {
    1: Workload(1, "tiny B=1 K=4 V=32 f32", 1, 4, (4, 4), 32, DTYPE_F32,
                2.0, 0.0, 0.0, ("cycle", (0.5,)), ("const", 1.0), 4),
    2: Workload(2, "llama B=64 K=4 V=128256 bf16", 64, 4, (4, 4), 128256, DTYPE_BF16,
                3.0, 0.01, 8.0, ("cycle", (0.25, 0.5, 1.0, 2.0)), ("split", 1.0, 0.0), 4),
    3: Workload(3, "large-batch B=256 K=8 V=128256 f32", 256, 8, (8, 8), 128256, DTYPE_F32,
                2.0, 0.0, 0.0, ("cycle", (0.5, 1.0)), ("choice", (0.6, 0.8, 1.0)), 8),
    4: Workload(4, "mtp B=512 K=1 V=129280 bf16", 512, 1, (1, 1), 129280, DTYPE_BF16,
                3.0, 0.01, 8.0, ("cycle", (0.5,)), ("split", 1.0, 0.0), 1),
    5: Workload(5, "ragged B=1024 K=1..8 V=152064 bf16", 1024, None, (1, 8), 152064, DTYPE_BF16,
                3.0, 0.01, 8.0, ("uniform", 0.25, 2.0), ("choice", (0.0, 0.7, 1.0)), 8),
}


def philox_seed(cfg: int, step: int) -> int:
    """Philox key used for workload ``cfg`` at step ``step``."""
    return 1000 * cfg + step


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even), return uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round a float array to the storage dtype (float32 array, or bf16 bits)."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == DTYPE_F32:
        return x32
    if dtype == DTYPE_BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype}")


def storage_to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float64 view of stored logits (every bf16 / f32 value is a double)."""
    if dtype == DTYPE_F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == DTYPE_BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def _draft_choice(rng: np.random.Generator, draft_row_f64: np.ndarray, T: float) -> int:
    """The drafter's own token choice: argmax at T=0, else x ~ softmax(row/T)
    by inverse CDF (one uniform against the running sum of the weights)."""
    if T == 0.0:
        return int(np.argmax(draft_row_f64))
    z = draft_row_f64 / T
    c = np.cumsum(np.exp(z - z.max()))
    i = int(np.searchsorted(c, rng.random() * c[-1], side="right"))
    return min(i, draft_row_f64.shape[0] - 1)


@dataclasses.dataclass
class Batch:
    """A packed batch of verify inputs (host numpy arrays)."""

    dtype: int
    B: int
    V: int
    max_k: int
    target: np.ndarray       # [sum(K_b+1), V]  float32 or uint16(bf16 bits)
    draft: np.ndarray        # [sum(K_b), V]
    offsets: np.ndarray      # [B+1] int32
    tokens: np.ndarray       # [sum(K_b)] int32
    temperature: np.ndarray  # [B] float32
    seed: int
    sigma: np.ndarray        # [B] float64, draft noise per request (metadata)
    label: str = ""

    @property
    def n_draft_rows(self) -> int:
        return int(self.offsets[-1])

    @property
    def k(self) -> np.ndarray:
        return np.diff(self.offsets).astype(np.int64)

    def target_row(self, b: int, t: int) -> np.ndarray:
        return self.target[int(self.offsets[b]) + b + t]

    def draft_row(self, b: int, t: int) -> np.ndarray:
        return self.draft[int(self.offsets[b]) + t]


def _per_request_params(w: Workload, rng: np.random.Generator):
    B = w.B
    if w.K is None:
        k = rng.integers(w.K_range[0], w.K_range[1] + 1, size=B)
    else:
        k = np.full(B, w.K, dtype=np.int64)
    kind = w.draft_sigma[0]
    if kind == "cycle":
        vals = w.draft_sigma[1]
        sigma = np.array([vals[b % len(vals)] for b in range(B)], dtype=np.float64)
    elif kind == "uniform":
        sigma = rng.uniform(w.draft_sigma[1], w.draft_sigma[2], size=B)
    else:
        raise ValueError(kind)
    kind = w.temperature[0]
    if kind == "split":
        temp = np.where(np.arange(B) < B // 2, w.temperature[1], w.temperature[2])
    elif kind == "choice":
        temp = rng.choice(np.asarray(w.temperature[1], dtype=np.float64), size=B)
    elif kind == "const":
        temp = np.full(B, w.temperature[1])
    else:
        raise ValueError(kind)
    return k.astype(np.int64), sigma, temp.astype(np.float32)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_batch(cfg: int, step: int = 0, B: Optional[int] = None,
               temperature_override: Optional[float] = None,
               progress: bool = False, workers: Optional[int] = None) -> Batch:
    """Generate workload ``cfg`` (1..5) at ``step``; ``B`` may shrink the batch.

    Seeds: the per-request parameters (K_b, sigma_b, T_b) come from numpy PCG64
    ``default_rng([0x5356, cfg, step])``; request b's rows and draft tokens from
    its own stream ``default_rng([0x5356, cfg, step, b])``, so requests are
    generated independently (and in parallel).  The Philox key is
    ``1000*cfg + step``.  Target row t ~ N(0, sigma_t^2) with round(peak_frac*V)
    distinct entries (uniform without replacement) raised by peak_boost; draft
    row t = target row t (before rounding) + N(0, sigma_b^2); both rounded to
    the storage dtype.  Sampled requests draft x_t ~ softmax(draft_t / T_b),
    greedy requests (T_b = 0) draft argmax(draft_t).
    """
    w = WORKLOADS[cfg]
    rng = np.random.default_rng([GEN_TAG, cfg, step])
    k, sigma, temp = _per_request_params(w, rng)
    if B is not None and B < w.B:
        k, sigma, temp = k[:B], sigma[:B], temp[:B]
    Bn = k.shape[0]
    if temperature_override is not None:
        temp = np.full(Bn, temperature_override, dtype=np.float32)
    offsets = np.zeros(Bn + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(k)
    n_d = int(offsets[-1])
    n_t = n_d + Bn
    V = w.V
    sdt = np.float32 if w.dtype == DTYPE_F32 else np.uint16
    target = np.empty((n_t, V), dtype=sdt)
    draft = np.empty((n_d, V), dtype=sdt)
    tokens = np.empty(n_d, dtype=np.int32)
    n_pk = w.n_peaks

    def one(b: int) -> None:
        r = np.random.default_rng([GEN_TAG, cfg, step, b])
        kb = int(k[b])
        z = r.standard_normal((kb + 1, V), dtype=np.float32) * np.float32(w.target_sigma)
        if n_pk > 0:
            for t in range(kb + 1):
                z[t, r.choice(V, size=n_pk, replace=False)] += np.float32(w.peak_boost)
        d = z[:kb] + r.standard_normal((kb, V), dtype=np.float32) * np.float32(sigma[b])
        t0 = int(offsets[b]) + b
        target[t0:t0 + kb + 1] = to_storage(z, w.dtype)
        d0 = int(offsets[b])
        draft[d0:d0 + kb] = to_storage(d, w.dtype)
        for t in range(kb):
            tokens[d0 + t] = _draft_choice(r, storage_to_f64(draft[d0 + t], w.dtype),
                                           float(temp[b]))

    nw = workers or _workers()
    if nw == 1 or Bn < 8:
        for b in range(Bn):
            one(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(nw) as ex:
            for i, _ in enumerate(ex.map(one, range(Bn))):
                if progress and (i + 1) % 256 == 0:
                    print(f"  generated {i + 1}/{Bn} requests", flush=True)
    return Batch(dtype=w.dtype, B=Bn, V=V, max_k=w.max_k, target=target, draft=draft,
                 offsets=offsets.astype(np.int32), tokens=tokens, temperature=temp,
                 seed=philox_seed(cfg, step), sigma=sigma, label=w.name)


def make_custom_batch(rng: np.random.Generator, dtype: int, V: int, ks, temps,
                      target_sigma: float = 3.0, draft_sigma: float = 0.5,
                      seed: int = 12345, max_k: Optional[int] = None) -> Batch:
    """Small ad-hoc batch (any V, any per-request K and T) for edge-case tests."""
    ks = [int(x) for x in ks]
    temps = np.asarray(temps, dtype=np.float32)
    B = len(ks)
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(ks)
    n_d = int(offsets[-1])
    sdt = np.float32 if dtype == DTYPE_F32 else np.uint16
    target = np.empty((n_d + B, V), dtype=sdt)
    draft = np.empty((n_d, V), dtype=sdt)
    tokens = np.empty(n_d, dtype=np.int32)
    for b in range(B):
        kb = ks[b]
        z = rng.standard_normal((kb + 1, V)) * target_sigma
        d = z[:kb] + rng.standard_normal((kb, V)) * draft_sigma
        t0 = int(offsets[b]) + b
        target[t0:t0 + kb + 1] = to_storage(z, dtype)
        d0 = int(offsets[b])
        draft[d0:d0 + kb] = to_storage(d, dtype)
        for t in range(kb):
            T = float(temps[b]) if math.isfinite(float(temps[b])) and temps[b] > 0 else 0.0
            tokens[d0 + t] = _draft_choice(rng, storage_to_f64(draft[d0 + t], dtype), T)
    mk = max_k if max_k is not None else max(1, max(ks) if ks else 1)
    return Batch(dtype=dtype, B=B, V=V, max_k=mk, target=target, draft=draft,
                 offsets=offsets.astype(np.int32), tokens=tokens, temperature=temps,
                 seed=seed, sigma=np.full(B, draft_sigma), label="custom")


def subset_requests(batch: Batch, reqs) -> Batch:
    """Copy of ``batch`` restricted to the listed requests (re-packed)."""
    reqs = [int(r) for r in reqs]
    ks = [int(batch.offsets[b + 1] - batch.offsets[b]) for b in reqs]
    offsets = np.zeros(len(reqs) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(ks)
    t_rows = [batch.target[int(batch.offsets[b]) + b: int(batch.offsets[b + 1]) + b + 1]
              for b in reqs]
    d_rows = [batch.draft[int(batch.offsets[b]): int(batch.offsets[b + 1])] for b in reqs]
    toks = [batch.tokens[int(batch.offsets[b]): int(batch.offsets[b + 1])] for b in reqs]
    V = batch.V
    sdt = batch.target.dtype
    return Batch(dtype=batch.dtype, B=len(reqs), V=V, max_k=batch.max_k,
                 target=np.concatenate(t_rows) if t_rows else np.empty((0, V), sdt),
                 draft=np.concatenate(d_rows) if d_rows else np.empty((0, V), sdt),
                 offsets=offsets.astype(np.int32),
                 tokens=np.concatenate(toks).astype(np.int32) if toks else np.empty(0, np.int32),
                 temperature=batch.temperature[reqs].copy(), seed=batch.seed,
                 sigma=batch.sigma[reqs].copy(), label=batch.label + " (subset)")


def draft_step_rows(batch: Batch, t: int) -> np.ndarray:
    """Draft rows at draft step t, one per request ([B, V], storage dtype).

    Request b contributes its draft row t (row offsets[b] + t); a request with
    fewer than t + 1 drafts contributes its last draft row (or its first
    target row when it has none), so every request has a row."""
    rows = []
    for b in range(batch.B):
        k = int(batch.offsets[b + 1] - batch.offsets[b])
        if k > 0:
            rows.append(batch.draft[int(batch.offsets[b]) + min(t, k - 1)])
        else:
            rows.append(batch.target[int(batch.offsets[b]) + b])
    return np.stack(rows)


# ------------------------------------------------------------------ draft trees

@dataclasses.dataclass(frozen=True)
class TreeWorkload:
    """A synthetic draft-tree workload (EAGLE-style trees: a few candidates per
    level, a few levels; "Decodificación Especulativa y EAGLE", section on
    EAGLE's tree drafting, and the tree drawn in its tree-attention section)."""

    name: str
    B: int
    depth: tuple             # (lo, hi) inclusive levels below the root
    width: tuple             # (lo, hi) inclusive nodes per level
    V: int
    dtype: int
    target_sigma: float
    peak_frac: float
    peak_boost: float
    draft_sigma: tuple       # ("uniform", lo, hi) per request

    @property
    def max_nodes(self) -> int:
        return 1 + self.depth[1] * self.width[1]


TREE_WORKLOADS = {
    "tree-small": TreeWorkload("tree-small B=8 depth 3 width 3 V=1000 f32", 8, (3, 3), (3, 3),
                               1000, DTYPE_F32, 2.0, 0.01, 6.0, ("uniform", 0.25, 1.0)),
    "tree-eagle": TreeWorkload("tree-eagle B=16 depth 5 width 8 V=128256 bf16", 16, (5, 5),
                               (8, 8), 128256, DTYPE_BF16, 3.0, 0.01, 8.0,
                               ("uniform", 0.25, 2.0)),
    "tree-ragged": TreeWorkload("tree-ragged B=64 depth 2..6 width 2..8 V=152064 bf16", 64,
                                (2, 6), (2, 8), 152064, DTYPE_BF16, 3.0, 0.01, 8.0,
                                ("uniform", 0.25, 2.0)),
}


@dataclasses.dataclass
class TreeBatch:
    """A packed batch of draft trees (host numpy arrays).

    Request b owns nodes i = 0..N_b-1 at packed rows offsets[b] + i; node 0 is the
    root (parents / tokens entry -1), node i >= 1 has parents[offsets[b] + i] in
    [0, i) and token tokens[offsets[b] + i].  target[offsets[b] + i] is the target
    row after the path root..i."""

    dtype: int
    B: int
    V: int
    max_nodes: int
    target: np.ndarray       # [sum(N_b), V] float32 or uint16 (bf16 bits)
    offsets: np.ndarray      # [B+1] int32
    parents: np.ndarray      # [sum(N_b)] int32
    tokens: np.ndarray       # [sum(N_b)] int32
    label: str = ""


def make_tree_batch(name: str, step: int = 0, B: Optional[int] = None,
                    workers: Optional[int] = None) -> TreeBatch:
    """Generate a draft-tree workload by name.

    Seeds: tree shapes and noise levels from ``default_rng([0x5356, 0x7472, k, step])``
    (k = the workload's position in TREE_WORKLOADS), request b's rows and tokens
    from ``default_rng([0x5356, 0x7472, k, step, b])``.  Per request: D levels
    below the root and W nodes per level (uniform in the workload's ranges).
    Level l's W nodes hang under the nodes of level l - 1, which the drafter
    ranks by its own confidence (creation order): node j of level l goes to
    the parent of rank min(floor(G), W_prev - 1), G geometric with mean 1.5,
    so the leading nodes get most children.  Every node has a target row
    ~ N(0, sigma^2) with round(peak_frac V) entries raised by peak_boost.  A
    parent's children take, in order, the top tokens of the drafter's row for
    that parent (the parent's target row + N(0, sigma_b^2)): distinct
    sibling tokens, as a top-k expansion gives.  Rows are rounded to the
    storage dtype.  Nodes are numbered level by level.
    """
    w = TREE_WORKLOADS[name]
    k_id = list(TREE_WORKLOADS).index(name)
    rng = np.random.default_rng([GEN_TAG, 0x7472, k_id, step])
    Bn = w.B if B is None else min(B, w.B)
    depth = rng.integers(w.depth[0], w.depth[1] + 1, size=w.B)[:Bn]
    width = rng.integers(w.width[0], w.width[1] + 1, size=w.B)[:Bn]
    sigma = rng.uniform(w.draft_sigma[1], w.draft_sigma[2], size=w.B)[:Bn]
    sizes = 1 + depth * width
    offsets = np.zeros(Bn + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(sizes)
    n = int(offsets[-1])
    V = w.V
    sdt = np.float32 if w.dtype == DTYPE_F32 else np.uint16
    target = np.empty((n, V), dtype=sdt)
    parents = np.full(n, -1, dtype=np.int32)
    tokens = np.full(n, -1, dtype=np.int32)
    n_pk = int(round(w.peak_frac * V))

    def one(b: int) -> None:
        r = np.random.default_rng([GEN_TAG, 0x7472, k_id, step, b])
        D, W, o = int(depth[b]), int(width[b]), int(offsets[b])
        N = 1 + D * W
        z = r.standard_normal((N, V), dtype=np.float32) * np.float32(w.target_sigma)
        if n_pk > 0:
            for i in range(N):
                z[i, r.choice(V, size=n_pk, replace=False)] += np.float32(w.peak_boost)
        target[o:o + N] = to_storage(z, w.dtype)
        prev = [0]
        nxt = 1
        for _ in range(D):
            ranks = np.minimum(np.floor(r.geometric(1.0 / 1.5, size=W) - 1).astype(int),
                               len(prev) - 1)
            kids = {}
            for j in range(W):
                kids.setdefault(prev[int(ranks[j])], []).append(j)
            level = []
            for par in sorted(kids):
                cnt = len(kids[par])
                drow = storage_to_f64(target[o + par], w.dtype) + \
                    r.standard_normal(V) * float(sigma[b])
                top = np.argsort(-drow, kind="stable")[:cnt]
                for t in top:
                    parents[o + nxt] = par
                    tokens[o + nxt] = int(t)
                    level.append(nxt)
                    nxt += 1
            prev = level

    nw = workers or _workers()
    if nw == 1 or Bn < 8:
        for b in range(Bn):
            one(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(nw) as ex:
            list(ex.map(one, range(Bn)))
    return TreeBatch(dtype=w.dtype, B=Bn, V=V, max_nodes=w.max_nodes, target=target,
                     offsets=offsets.astype(np.int32), parents=parents, tokens=tokens,
                     label=w.name)
