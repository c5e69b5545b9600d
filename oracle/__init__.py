"""Float64 CPU oracle of the speculative-decoding verify step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  The C
source (``spec_oracle.c``) shares no code with the HIP implementation.

What it computes is stated in ``spec_oracle.c``: the exact accept / residual /
bonus rule and the greedy case of "Decodificación Especulativa y EAGLE"
(section "La Regla de Exactitud"), with randomness drawn from Philox4x32-10 by
counter, so that a result is a pure function of the inputs and the seed.
It also holds the draft-side sampler that precedes verification
(``draft_sample``: one token per request from softmax(z/T), or the argmax at
T = 0), the commit step that follows it (``commit_tokens``: the emitted
tokens appended to each request's token history), and greedy verification of
a draft tree (``tree_verify``: the longest accepted root-to-node path, then
the argmax of its last node's row).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "spec_oracle.c")
LIB = os.path.join(HERE, "liboracle_specverify.so")

F32, BF16, F64 = 0, 1, 2
FLAG_ACCEPT_NEAR_TIE = 1
FLAG_RACE_NEAR_TIE = 2
FLAG_RESIDUAL_EMPTY = 4


def build(force: bool = False, extra_flags=(), out: str = LIB, src: str = SRC) -> str:
    """Compile the oracle with gcc (plain IEEE float64, no contraction)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str = LIB):
    """Load (building first if needed) and declare the C entry points."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if path == LIB:
        build()
    lib = ctypes.CDLL(path)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_u01.argtypes = [ctypes.c_uint32]
    lib.oracle_u01.restype = ctypes.c_double
    lib.oracle_accept_uniform.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32]
    lib.oracle_accept_uniform.restype = ctypes.c_double
    lib.oracle_race_exponential.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32]
    lib.oracle_race_exponential.restype = ctypes.c_double
    vp = ctypes.c_void_p
    lib.oracle_spec_verify.argtypes = [
        ctypes.c_int, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        vp, vp, vp, ctypes.c_uint64, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_spec_verify.restype = ctypes.c_int
    lib.oracle_draft_exponential.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32]
    lib.oracle_draft_exponential.restype = ctypes.c_double
    lib.oracle_draft_sample.argtypes = [ctypes.c_int, vp, ctypes.c_int32, ctypes.c_int32, vp,
                                        ctypes.c_uint64, ctypes.c_int32, vp, vp, vp, vp]
    lib.oracle_draft_sample.restype = ctypes.c_int
    lib.oracle_commit_tokens.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                         vp, vp, ctypes.c_int64, vp, ctypes.c_int32, vp, vp]
    lib.oracle_commit_tokens.restype = ctypes.c_int
    lib.oracle_tree_verify_greedy.argtypes = [ctypes.c_int, vp, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp,
                                              vp]
    lib.oracle_tree_verify_greedy.restype = ctypes.c_int
    if path == LIB:
        _lib = lib
    return lib


def philox4x32_10(ctr, key, lib=None) -> np.ndarray:
    """Philox4x32-10 block for a 4-word counter and 2-word key."""
    lib = lib or load()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    lib.oracle_philox4x32_10(c, k, o)
    return np.array(list(o), dtype=np.uint32)


def u01(x: int, lib=None) -> float:
    return (lib or load()).oracle_u01(int(x) & 0xFFFFFFFF)


def accept_uniform(seed: int, b: int, t: int, lib=None) -> float:
    return (lib or load()).oracle_accept_uniform(seed, b, t)


def race_exponential(seed: int, b: int, pos: int, v: int, lib=None) -> float:
    return (lib or load()).oracle_race_exponential(seed, b, pos, v)


def default_threads() -> int:
    """Worker threads for request-parallel oracle runs: the cores this process may
    use, at most 16 (``ORACLE_THREADS`` overrides)."""
    env = os.environ.get("ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_logits(dtype: int, a):
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return np.ascontiguousarray(a, dtype=np.uint16)
    if dtype == F64:
        return np.ascontiguousarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def verify(dtype: int, target, draft, offsets, tokens, temperature, seed: int, V: int,
           max_k: int, reqs=None, lib=None, n_draft_rows=None, threads=None) -> dict:
    """Run the oracle over a packed batch (see the workload module for layout).

    Returns numpy arrays: accept_len [B], out_tokens [sum(K_b)+B], p_at / q_at
    [sum(K_b)] (float64), flags [B], race_best / race_gap [B].  With ``reqs``
    only the listed requests are evaluated (others keep accept_len == -2).

    Requests are independent, so ``threads`` > 1 (default: ``default_threads()``)
    splits them over worker threads, each calling the same C entry point on its
    own requests and writing their disjoint entries of the shared outputs (a
    ctypes call releases the GIL).  The result does not depend on ``threads``.
    """
    lib = lib or load()
    if dtype == F32:
        target = np.ascontiguousarray(target, dtype=np.float32)
        draft = None if draft is None else np.ascontiguousarray(draft, dtype=np.float32)
    elif dtype == BF16:
        target = np.ascontiguousarray(target, dtype=np.uint16)
        draft = None if draft is None else np.ascontiguousarray(draft, dtype=np.uint16)
    elif dtype == F64:
        target = np.ascontiguousarray(target, dtype=np.float64)
        draft = None if draft is None else np.ascontiguousarray(draft, dtype=np.float64)
    else:
        raise ValueError(f"unknown dtype {dtype}")
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    B = offsets.shape[0] - 1
    n_d = int(offsets[-1]) if n_draft_rows is None else int(n_draft_rows)
    if tokens.shape[0] == 0:
        tokens = np.zeros(1, dtype=np.int32)
    acc = np.full(B, -2, dtype=np.int32)
    out = np.full(n_d + B, -2, dtype=np.int32)
    p_at = np.full(max(n_d, 1), np.nan)
    q_at = np.full(max(n_d, 1), np.nan)
    flags = np.zeros(B, dtype=np.uint32)
    best = np.full(B, np.nan)
    gap = np.full(B, np.nan)
    r = None
    if reqs is not None:
        r = np.ascontiguousarray(reqs, dtype=np.int32)
    threads = default_threads() if threads is None else max(1, int(threads))

    def run(rr):
        return lib.oracle_spec_verify(dtype, _ptr(target), _ptr(draft), B, V, max_k, n_d,
                                      _ptr(offsets), _ptr(tokens), _ptr(temperature),
                                      ctypes.c_uint64(seed), _ptr(rr),
                                      0 if rr is None else rr.shape[0], _ptr(acc), _ptr(out),
                                      _ptr(p_at), _ptr(q_at), _ptr(flags), _ptr(best), _ptr(gap))

    n_req = B if r is None else r.shape[0]
    if threads == 1 or n_req < 2:
        rcs = [run(r)]
    else:
        every = np.arange(B, dtype=np.int32) if r is None else r
        # interleaved shards balance ragged batches (neighbouring requests differ in K_b)
        shards = [np.ascontiguousarray(every[i::threads]) for i in range(min(threads, n_req))]
        with ThreadPoolExecutor(len(shards)) as pool:
            rcs = list(pool.map(run, shards))
    if any(rc != 0 for rc in rcs):
        raise ValueError(f"oracle_spec_verify rejected its arguments (rc={rcs})")
    return dict(accept_len=acc, out_tokens=out, p_at=p_at[:n_d], q_at=q_at[:n_d],
                flags=flags, race_best=best, race_gap=gap)


def verify_batch(batch, reqs=None, greedy_only: bool = False, lib=None, threads=None) -> dict:
    """Oracle over a workload ``Batch``; ``greedy_only`` forces T=0 everywhere."""
    temp = np.zeros_like(batch.temperature) if greedy_only else batch.temperature
    return verify(batch.dtype, batch.target, None if greedy_only else batch.draft,
                  batch.offsets, batch.tokens, temp, batch.seed, batch.V, batch.max_k,
                  reqs=reqs, lib=lib, n_draft_rows=batch.n_draft_rows, threads=threads)


def draft_exponential(seed: int, b: int, step: int, v: int, lib=None) -> float:
    return (lib or load()).oracle_draft_exponential(seed, b, step, v)


def draft_sample(dtype: int, logits, temperature, seed: int, step: int, lib=None) -> dict:
    """Draft-side sampler over B rows of logits [B, V] (one row per request).

    Returns numpy arrays: tokens [B] (int32, -1 for a bad row or temperature),
    q_at [B] (float64 softmax probability of the drawn token, NaN at T == 0),
    flags [B] (bit 2: near tie in the race) and race_gap [B].
    """
    lib = lib or load()
    np_dt = {F32: np.float32, BF16: np.uint16, F64: np.float64}.get(dtype)
    if np_dt is None:
        raise ValueError(f"unknown dtype {dtype}")
    logits = np.ascontiguousarray(logits, dtype=np_dt)
    B, V = logits.shape
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    tokens = np.full(B, -2, dtype=np.int32)
    q_at = np.full(B, np.nan)
    flags = np.zeros(B, dtype=np.uint32)
    gap = np.full(B, np.nan)
    rc = lib.oracle_draft_sample(dtype, _ptr(logits), B, V, _ptr(temperature),
                                 ctypes.c_uint64(seed), step, _ptr(tokens), _ptr(q_at),
                                 _ptr(flags), _ptr(gap))
    if rc != 0:
        raise ValueError(f"oracle_draft_sample rejected its arguments (rc={rc})")
    return dict(tokens=tokens, q_at=q_at, flags=flags, race_gap=gap)


def commit_tokens(offsets, accept_len, out_tokens, seq_tokens, seq_len, max_k: int,
                  n_draft_rows=None, lib=None) -> dict:
    """Commit step: returns new copies of seq_tokens [B, capacity] and seq_len [B],
    with next_tokens [B] and status [B] (see spec_oracle.c)."""
    lib = lib or load()
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    accept_len = np.ascontiguousarray(accept_len, dtype=np.int32)
    out_tokens = np.ascontiguousarray(out_tokens, dtype=np.int32)
    seq = np.array(seq_tokens, dtype=np.int32, copy=True, order="C")
    lens = np.array(seq_len, dtype=np.int32, copy=True)
    B, cap = seq.shape
    n_d = int(offsets[-1]) if n_draft_rows is None else int(n_draft_rows)
    nxt = np.full(B, -3, dtype=np.int32)
    st = np.full(B, -3, dtype=np.int32)
    rc = lib.oracle_commit_tokens(B, max_k, n_d, _ptr(offsets), _ptr(accept_len), _ptr(out_tokens),
                                  _ptr(seq), cap, _ptr(lens), cap, _ptr(nxt), _ptr(st))
    if rc != 0:
        raise ValueError(f"oracle_commit_tokens rejected its arguments (rc={rc})")
    return dict(seq_tokens=seq, seq_len=lens, next_tokens=nxt, status=st)


def tree_verify(dtype: int, target, node_offsets, parents, tokens, V: int, max_nodes: int,
                n_rows=None, lib=None) -> dict:
    """Greedy tree verification (see oracle_tree_verify_greedy in spec_oracle.c):
    accept_len [B], out_tokens [n_rows], accept_nodes [n_rows]."""
    lib = lib or load()
    target = _as_logits(dtype, target)
    node_offsets = np.ascontiguousarray(node_offsets, dtype=np.int32)
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B = node_offsets.size - 1
    n = int(node_offsets[-1]) if n_rows is None else int(n_rows)
    acc = np.full(B, -3, dtype=np.int32)
    out = np.full(max(n, 1), -3, dtype=np.int32)
    nodes = np.full(max(n, 1), -3, dtype=np.int32)
    rc = lib.oracle_tree_verify_greedy(dtype, _ptr(target), B, V, max_nodes, n,
                                       _ptr(node_offsets), _ptr(parents), _ptr(tokens), _ptr(acc),
                                       _ptr(out), _ptr(nodes))
    if rc != 0:
        raise ValueError(f"oracle_tree_verify_greedy rejected its arguments (rc={rc})")
    return dict(accept_len=acc, out_tokens=out[:n], accept_nodes=nodes[:n])
