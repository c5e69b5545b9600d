"""Pins that tie the float64 oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load(path)``)
and raises AssertionError when the oracle disagrees with:
  * published known-answer vectors and an independent implementation (Philox);
  * library routines (scipy's softmax, numpy's first-occurrence argmax);
  * exact enumeration of the method's output law at tiny sizes, and the
    distribution-equivalence property of "Decodificación Especulativa y EAGLE",
    section "La Regla de Exactitud";
  * the closed form of section "Aceleración Esperada";
  * textbook results (exponential race = categorical sampling; temperature
    scaling invariance; identical draft and target always accept).
The same functions run against planted-mistake builds of the oracle in
test_oracle_mutants.py, to show that each plausible mistake fails a pin.
"""
from __future__ import annotations

import itertools
import math
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import scipy.special
import scipy.stats

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


# ------------------------------------------------------------------ Philox


def read_kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def pin_philox_kat(lib):
    for ctr, key, want in read_kat():
        got = oracle.philox4x32_10(ctr, key, lib=lib)
        assert list(got) == want, (ctr, key, [hex(x) for x in got], [hex(x) for x in want])


_REF_BIN = None


def rocrand_reference_binary():
    """Build (once per process) the host driver around rocRAND's Philox engine."""
    global _REF_BIN
    if _REF_BIN is None:
        d = tempfile.mkdtemp(prefix="philox_ref_")
        out = os.path.join(d, "philox_ref")
        subprocess.run(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-o", out,
                        os.path.join(HERE, "philox_rocrand_ref.cpp")], check=True)
        _REF_BIN = out
    return _REF_BIN


def pin_philox_rocrand(lib, n=4000, seed=7):
    rng = np.random.default_rng(seed)
    words = rng.integers(0, 2**32, size=(n, 6), dtype=np.uint64)
    # edge counters: zeros, all-ones, single bits, the counters the method uses
    edge = [[0, 0, 0, 0, 0, 0], [2**32 - 1] * 6, [1, 0, 0, 0, 0, 0], [0, 1, 0, 0, 0, 0],
            [0, 0, 1, 0, 0, 0], [0, 0, 0, 1, 0, 0], [0, 0, 0, 0, 1, 0], [0, 0, 0, 0, 0, 1],
            [0, 3, 1023, 1, 2002, 0], [38015, 4, 63, 0, 2000, 0]]
    words = np.concatenate([np.array(edge, dtype=np.uint64), words])
    text = "\n".join(" ".join(str(int(x)) for x in row) for row in words) + "\n"
    res = subprocess.run([rocrand_reference_binary()], input=text, capture_output=True,
                         text=True, check=True)
    ref = np.array([[int(x) for x in ln.split()] for ln in res.stdout.strip().splitlines()],
                   dtype=np.uint64)
    assert ref.shape == (words.shape[0], 4)
    for i, row in enumerate(words):
        got = oracle.philox4x32_10(row[:4], row[4:6], lib=lib)
        assert list(got) == list(ref[i]), (i, row, got, ref[i])


def pin_u01(lib):
    lo = oracle.u01(0, lib=lib)
    hi = oracle.u01(0xFFFFFFFF, lib=lib)
    assert lo == 2.0**-24 and hi == 1.0 - 2.0**-24
    rng = np.random.default_rng(3)
    xs = rng.integers(0, 2**32, size=2000, dtype=np.uint64)
    for x in xs:
        u = oracle.u01(int(x), lib=lib)
        assert 0.0 < u < 1.0
        assert float(np.float32(u)) == u  # exact in float32 too
        assert u == (2 * (int(x) >> 9) + 1) / 2**24
    # accept uniforms and race exponentials are U(0,1) / Exp(1) distributed
    us = np.array([oracle.accept_uniform(11, b, t, lib=lib) for b in range(500) for t in range(8)])
    assert scipy.stats.kstest(us, "uniform").pvalue > 1e-4
    es = np.array([oracle.race_exponential(11, b, 2, v, lib=lib)
                   for b in range(40) for v in range(100)])
    assert scipy.stats.kstest(es, "expon").pvalue > 1e-4


# ------------------------------------------------------------------ helpers


def pack_requests(rows_t, rows_d, toks):
    """Pack per-request target rows [K+1,V], draft rows [K,V], tokens [K]."""
    ks = [len(t) for t in toks]
    offsets = np.zeros(len(ks) + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(ks)
    target = np.concatenate(rows_t)
    V = target.shape[1]
    draft = np.concatenate(rows_d) if sum(ks) else np.zeros((0, V))
    tokens = np.concatenate([np.asarray(t, dtype=np.int32) for t in toks]) if sum(ks) \
        else np.zeros(0, np.int32)
    return target, draft, offsets, tokens


def emitted(res, offsets, b):
    n = int(res["accept_len"][b])
    base = int(offsets[b]) + b
    return tuple(int(x) for x in res["out_tokens"][base:base + n + 1])


def check_invariants(res, offsets, tokens, B):
    for b in range(B):
        n = int(res["accept_len"][b])
        k = int(offsets[b + 1] - offsets[b])
        assert 0 <= n <= k
        base = int(offsets[b]) + b
        out = res["out_tokens"][base:base + k + 1]
        assert list(out[:n]) == list(tokens[offsets[b]:offsets[b] + n])
        assert out[n] >= 0
        assert all(x == -1 for x in out[n + 1:])


# ------------------------------------------------------------------ library routines


def pin_softmax_vs_scipy(lib):
    """p(x_t), q(x_t) equal scipy's softmax(z / T) at x_t (float64 routine)."""
    rng = np.random.default_rng(5)
    for dtype in (oracle.F64, oracle.F32, oracle.BF16):
        for T in (1.0, 0.7, 2.5):
            V, K = 300, 3
            z = rng.normal(0, 3, size=(K + 1, V))
            d = z[:K] + rng.normal(0, 1, size=(K, V))
            if dtype == oracle.F32:
                zs, ds = z.astype(np.float32), d.astype(np.float32)
                z64, d64 = zs.astype(np.float64), ds.astype(np.float64)
            elif dtype == oracle.BF16:
                from rejection_sampling_verify_scaled_amd.workloads import (f32_to_bf16_bits,
                                                                              bf16_bits_to_f32)
                zs, ds = f32_to_bf16_bits(z.astype(np.float32)), f32_to_bf16_bits(d.astype(np.float32))
                z64 = bf16_bits_to_f32(zs).astype(np.float64)
                d64 = bf16_bits_to_f32(ds).astype(np.float64)
            else:
                zs, ds, z64, d64 = z, d, z, d
            toks = rng.integers(0, V, size=K).astype(np.int32)
            offsets = np.array([0, K], dtype=np.int32)
            res = oracle.verify(dtype, zs, ds, offsets, toks, np.array([T], np.float32), 9, V, K,
                                lib=lib)
            Tf = float(np.float32(T))
            for t in range(K):
                pt = scipy.special.softmax(z64[t] / Tf)[toks[t]]
                qt = scipy.special.softmax(d64[t] / Tf)[toks[t]]
                assert abs(res["p_at"][t] - pt) <= 1e-12 * max(pt, 1e-300) + 1e-300, (t, res["p_at"][t], pt)
                assert abs(res["q_at"][t] - qt) <= 1e-12 * max(qt, 1e-300) + 1e-300
    # closed forms: equal logits give 1/V; two tokens give the logistic function
    V = 7
    z = np.zeros((2, V))
    res = oracle.verify(oracle.F64, z, z[:1] + 0.0, np.array([0, 1], np.int32),
                        np.array([3], np.int32), np.array([1.0], np.float32), 1, V, 1, lib=lib)
    assert abs(res["p_at"][0] - 1.0 / V) < 1e-15
    a, bb = 1.3, -0.4
    z = np.array([[a, bb], [0.0, 0.0]])
    d = np.array([[0.0, 0.0]])
    res = oracle.verify(oracle.F64, z, d, np.array([0, 1], np.int32), np.array([0], np.int32),
                        np.array([1.0], np.float32), 1, 2, 1, lib=lib)
    assert abs(res["p_at"][0] - 1.0 / (1.0 + math.exp(bb - a))) < 1e-15
    assert abs(res["q_at"][0] - 0.5) < 1e-15


def greedy_rule(rows, toks):
    """The page's greedy case written with numpy.argmax (first occurrence)."""
    g = [int(np.argmax(np.where(np.isnan(r), -np.inf, r))) for r in rows]
    n = len(toks)
    for t in range(len(toks)):
        if g[t] != toks[t]:
            n = t
            break
    return n, g[n]


def pin_greedy_vs_numpy(lib):
    rng = np.random.default_rng(8)
    from rejection_sampling_verify_scaled_amd.workloads import f32_to_bf16_bits, bf16_bits_to_f32
    rows_t, rows_d, toks_all, ref = [], [], [], []
    V = 64
    for b in range(300):
        K = int(rng.integers(0, 6))
        z = rng.normal(0, 2, size=(K + 1, V)).astype(np.float32)
        for t in range(K + 1):
            if rng.random() < 0.6:  # plant ties at the maximum
                m = z[t].max() + 1.0
                idx = rng.choice(V, size=int(rng.integers(2, 5)), replace=False)
                z[t, idx] = m
        zb = f32_to_bf16_bits(z)
        z64 = bf16_bits_to_f32(zb).astype(np.float64)
        g = [int(np.argmax(r)) for r in z64]
        toks = []
        for t in range(K):
            r = rng.random()
            if r < 0.7:
                toks.append(g[t])
            elif r < 0.85:  # a tied-but-not-first index must be rejected
                ties = np.flatnonzero(z64[t] == z64[t].max())
                toks.append(int(ties[-1]))
            else:
                toks.append(int(rng.integers(0, V)))
        rows_t.append(zb)
        rows_d.append(np.zeros((K, V), np.uint16))
        toks_all.append(toks)
        ref.append(greedy_rule(z64, toks))
    target, draft, offsets, tokens = pack_requests(rows_t, rows_d, toks_all)
    B = len(ref)
    res = oracle.verify(oracle.BF16, target, None, offsets, tokens, np.zeros(B, np.float32),
                        3, V, 8, lib=lib)
    check_invariants(res, offsets, tokens, B)
    for b in range(B):
        n, y = ref[b]
        assert int(res["accept_len"][b]) == n, (b, res["accept_len"][b], n)
        assert emitted(res, offsets, b)[-1] == y


# ------------------------------------------------------------------ exact law


def rational_tables(rng, V, K, zero_p=True, zero_q=True):
    """Random rational distributions p_0..p_K and q_0..q_{K-1} over V tokens."""
    def dist(zero_at=None):
        w = [int(x) for x in rng.integers(1, 20, size=V)]
        if zero_at is not None:
            w[zero_at] = 0
        s = sum(w)
        return [Fraction(x, s) for x in w]
    p = [dist(0 if (zero_p and t % 2 == 0) else None) for t in range(K + 1)]
    q = [dist(V - 1 if (zero_q and t % 2 == 1) else None) for t in range(K)]
    return p, q


def exact_law(p, q, K, V):
    """Brute-force enumeration of the verify step's output law (Fractions).

    Drafts x_t ~ q_t; accept with probability min(1, p_t(x)/q_t(x)); on the
    first rejection emit a token from (p_t - q_t)+ normalised and stop; after
    K acceptances emit a bonus token from p_K.
    """
    law = {}

    def residual(t):
        r = [max(p[t][v] - q[t][v], Fraction(0)) for v in range(V)]
        s = sum(r)
        return [x / s for x in r]

    res = [residual(t) for t in range(K)]

    def walk(t, prefix, prob):
        if prob == 0:
            return
        if t == K:
            for v in range(V):
                if p[K][v]:
                    law[prefix + (v,)] = law.get(prefix + (v,), 0) + prob * p[K][v]
            return
        for x in range(V):
            if q[t][x] == 0:
                continue
            a = min(Fraction(1), p[t][x] / q[t][x])
            walk(t + 1, prefix + (x,), prob * q[t][x] * a)
            rej = prob * q[t][x] * (1 - a)
            if rej:
                for v in range(V):
                    if res[t][v]:
                        law[prefix + (v,)] = law.get(prefix + (v,), 0) + rej * res[t][v]

    walk(0, (), Fraction(1))
    return law


def check_law_is_target(law, p, q, K, V):
    """(i) first token ~ p_0; (ii) token j+1 given n >= j ~ p_j; (iii) P(n >= j) = prod alpha."""
    assert sum(law.values()) == 1
    alpha = [sum(min(p[t][v], q[t][v]) for v in range(V)) for t in range(K)]
    for j in range(K + 1):
        reach = sum(pr for seq, pr in law.items() if len(seq) >= j + 1)
        want = Fraction(1)
        for t in range(j):
            want *= alpha[t]
        assert reach == want, (j, reach, want)
        for v in range(V):
            pv = sum(pr for seq, pr in law.items() if len(seq) >= j + 1 and seq[j] == v)
            assert pv == reach * p[j][v], (j, v)


def sample_oracle(lib, p, q, K, V, N, T, seed, rng):
    """N independent requests sharing the tables; drafts drawn by numpy from q."""
    with np.errstate(divide="ignore"):
        zt = np.array([[T * math.log(float(x)) if x else -np.inf for x in row] for row in p])
        zd = np.array([[T * math.log(float(x)) if x else -np.inf for x in row] for row in q])
    qf = np.array([[float(x) for x in row] for row in q])
    target = np.tile(zt, (N, 1))
    draft = np.tile(zd, (N, 1)) if K else np.zeros((0, V))
    tokens = np.empty(N * K, dtype=np.int32)
    for t in range(K):
        tokens[t::K] = rng.choice(V, size=N, p=qf[t])
    offsets = (np.arange(N + 1) * K).astype(np.int32)
    res = oracle.verify(oracle.F64, target, draft, offsets, tokens,
                        np.full(N, T, np.float32), seed, V, K, lib=lib)
    check_invariants(res, offsets, tokens, N)
    counts = {}
    for b in range(N):
        s = emitted(res, offsets, b)
        counts[s] = counts.get(s, 0) + 1
    return counts


def tv(counts, law, N):
    keys = set(counts) | set(law)
    return 0.5 * sum(abs(counts.get(k, 0) / N - float(law.get(k, 0))) for k in keys)


def chi2_pvalue(counts, law, N):
    keys = sorted(law, key=lambda k: -float(law[k]))
    obs, exp_ = [], []
    acc_o = acc_e = 0.0
    for k in keys:  # pool cells so each has expected count >= 5
        acc_o += counts.get(k, 0)
        acc_e += float(law[k]) * N
        if acc_e >= 5:
            obs.append(acc_o)
            exp_.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0 and exp_:
        obs[-1] += acc_o
        exp_[-1] += acc_e
    extra = sum(c for k, c in counts.items() if k not in law)
    assert extra == 0, f"{extra} samples outside the support of the exact law"
    return scipy.stats.chisquare(obs, exp_).pvalue


def pin_exact_enumeration(lib, cases=((4, 2, 300_000, 0.7), (6, 3, 200_000, 1.0)),
                          seed=21):
    rng = np.random.default_rng(seed)
    for (V, K, N, T) in cases:
        p, q = rational_tables(rng, V, K)
        law = exact_law(p, q, K, V)
        check_law_is_target(law, p, q, K, V)
        counts = sample_oracle(lib, p, q, K, V, N, T, seed=1000 + V, rng=rng)
        pv = chi2_pvalue(counts, law, N)
        assert pv > 1e-5, (V, K, pv)
        # section "Ejercicios", exercise 1: total-variation distance to plain
        # target sampling below 0.01 -- the first emitted token against p_0
        hist = np.zeros(V)
        for s, c in counts.items():
            hist[s[0]] += c
        d = 0.5 * np.abs(hist / N - np.array([float(x) for x in p[0]])).sum()
        assert d < 0.01, (V, K, d)


def pin_plain_sampling(lib, V=8, N=400_000, T=1.3, seed=4):
    """K_b = 0 is plain sampling from softmax(z/T) (exponential-race textbook result)."""
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1.5, size=(1, V))
    Tf = float(np.float32(T))
    p = scipy.special.softmax(z[0] / Tf)
    target = np.tile(z, (N, 1))
    offsets = np.zeros(N + 1, dtype=np.int32)
    res = oracle.verify(oracle.F64, target, np.zeros((0, V)), offsets, np.zeros(0, np.int32),
                        np.full(N, T, np.float32), 77, V, 0, lib=lib)
    assert (res["accept_len"] == 0).all()
    y = res["out_tokens"]
    hist = np.bincount(y, minlength=V) / N
    assert 0.5 * np.abs(hist - p).sum() < 0.005
    assert scipy.stats.chisquare(hist * N, p * N).pvalue > 1e-5


# ------------------------------------------------------------------ closed form


def expected_tokens(alpha, K):
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def controlled_alpha_batch(rng, alpha, K, V, N, T=1.0):
    """Rows whose per-position acceptance probability is exactly alpha.

    q_t = alpha * p_t + (1 - alpha) * delta_w with p_t(w) = 0, so
    sum_v min(p_t(v), q_t(v)) = alpha.
    """
    w = V - 1
    rows_p = rng.dirichlet(np.ones(V - 1), size=K + 1)
    p = np.zeros((K + 1, V))
    p[:, :w] = rows_p
    q = alpha * p[:K].copy()
    q[:, w] += 1.0 - alpha
    with np.errstate(divide="ignore"):
        zt = T * np.log(p)
        zd = T * np.log(q)
    target = np.tile(zt, (N, 1))
    draft = np.tile(zd, (N, 1))
    tokens = np.empty(N * K, dtype=np.int32)
    for t in range(K):
        tokens[t::K] = rng.choice(V, size=N, p=q[t] / q[t].sum())
    offsets = (np.arange(N + 1) * K).astype(np.int32)
    return target, draft, offsets, tokens


def pin_closed_form(lib, N=100_000):
    with open(os.path.join(GOLDEN, "expected_tokens_closed_form.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                a, K, printed, dec = line.split()
                assert round(expected_tokens(float(a), int(K)), int(dec)) == float(printed)
    rng = np.random.default_rng(31)
    for alpha, K in ((0.8, 4), (0.5, 2), (0.9, 8), (0.7, 1)):
        V = 12
        target, draft, offsets, tokens = controlled_alpha_batch(rng, alpha, K, V, N)
        res = oracle.verify(oracle.F64, target, draft, offsets, tokens,
                            np.ones(N, np.float32), 4242 + K, V, K, lib=lib)
        L = res["accept_len"].astype(np.float64) + 1.0
        mean = L.mean()
        # exact variance of min(G, K+1) with P(L >= j+1) = alpha^j
        pj = np.array([alpha ** j for j in range(K + 1)])
        e1 = pj.sum()
        e2 = sum((2 * j + 1) * pj[j] for j in range(K + 1))
        se = math.sqrt((e2 - e1 * e1) / N)
        want = expected_tokens(alpha, K)
        assert abs(e1 - want) < 1e-12
        assert abs(mean - want) < 4.0 * se, (alpha, K, mean, want, se)


# ------------------------------------------------------------------ textbook invariants


def pin_temperature_invariance(lib):
    """Sampling at temperature T on z equals temperature 1 on z / T."""
    rng = np.random.default_rng(12)
    V, K, B = 40, 3, 400
    T = 2.0  # z / 2 is exact in float64
    z = rng.normal(0, 2, size=(B * (K + 1), V))
    d = rng.normal(0, 2, size=(B * K, V))
    offsets = (np.arange(B + 1) * K).astype(np.int32)
    toks = rng.integers(0, V, size=B * K).astype(np.int32)
    a = oracle.verify(oracle.F64, z, d, offsets, toks, np.full(B, T, np.float32), 5, V, K, lib=lib)
    b = oracle.verify(oracle.F64, z / T, d / T, offsets, toks, np.ones(B, np.float32), 5, V, K,
                      lib=lib)
    assert (a["accept_len"] == b["accept_len"]).all()
    assert (a["out_tokens"] == b["out_tokens"]).all()
    assert np.allclose(a["p_at"], b["p_at"], rtol=1e-13, atol=0)
    assert np.allclose(a["q_at"], b["q_at"], rtol=1e-13, atol=0)


def pin_identical_draft_accepts(lib):
    """q == p accepts every draft (r < 1 = p/q), so n = K and a bonus follows."""
    rng = np.random.default_rng(13)
    V, K, B = 50, 4, 300
    z = rng.normal(0, 2, size=(B * (K + 1), V))
    d = np.concatenate([z[b * (K + 1): b * (K + 1) + K] for b in range(B)])
    offsets = (np.arange(B + 1) * K).astype(np.int32)
    toks = rng.integers(0, V, size=B * K).astype(np.int32)
    res = oracle.verify(oracle.F64, z, d, offsets, toks, np.full(B, 0.9, np.float32), 6, V, K,
                        lib=lib)
    assert (res["accept_len"] == K).all()


def pin_disjoint_draft_rejects(lib):
    """q concentrated where p = 0 always rejects at t = 0, and the residual is p_0."""
    V, K, N = 6, 2, 200_000
    rng = np.random.default_rng(14)
    p0 = np.array([0.0, 0.1, 0.2, 0.3, 0.25, 0.15])
    with np.errstate(divide="ignore"):
        zt0 = np.log(p0)
    zt = np.stack([zt0, rng.normal(size=V), rng.normal(size=V)])
    zq = np.full((K, V), -np.inf)
    zq[:, 0] = 0.0
    target = np.tile(zt, (N, 1))
    draft = np.tile(zq, (N, 1))
    tokens = np.zeros(N * K, dtype=np.int32)
    offsets = (np.arange(N + 1) * K).astype(np.int32)
    res = oracle.verify(oracle.F64, target, draft, offsets, tokens, np.ones(N, np.float32), 8,
                        V, K, lib=lib)
    assert (res["accept_len"] == 0).all()
    y = res["out_tokens"][offsets[:-1] + np.arange(N)]
    hist = np.bincount(y, minlength=V) / N
    assert 0.5 * np.abs(hist - p0).sum() < 0.005


def pin_faults(lib):
    """Bad requests fail alone (accept_len = -1, tokens -1); others are unaffected."""
    rng = np.random.default_rng(15)
    V, K = 16, 2
    B = 8
    z = rng.normal(size=(B * (K + 1), V))
    d = rng.normal(size=(B * K, V))
    offsets = (np.arange(B + 1) * K).astype(np.int32)
    toks = rng.integers(0, V, size=B * K).astype(np.int32)
    temp = np.ones(B, np.float32)
    temp[4:] = 0.0
    toks[1 * K + 1] = V          # b=1: token out of range
    temp[2] = -1.0               # b=2: negative temperature
    temp[3] = np.nan             # b=3: NaN temperature
    z[5 * (K + 1) + 1, :] = -np.inf   # b=5 (greedy): a row with no finite maximum
    z[6 * (K + 1) + 0, 3] = np.nan    # b=6 (greedy): NaN entries never win
    z[6 * (K + 1) + 0, 4] = 100.0
    z[0 * (K + 1) + 2, 7] = np.nan    # b=0 (sampled): NaN in the bonus row
    res = oracle.verify(oracle.F64, z, d, offsets, toks, temp, 3, V, K, lib=lib)
    acc = res["accept_len"]
    for b in (0, 1, 2, 3, 5):
        assert acc[b] == -1, b
        base = offsets[b] + b
        assert (res["out_tokens"][base:base + K + 1] == -1).all()
    assert acc[4] >= 0 and acc[6] >= 0 and acc[7] >= 0
    assert int(res["out_tokens"][offsets[6] + 6]) == 4  # accepted draft or emitted argmax
    # a request whose K_b exceeds max_k fails without touching others
    offsets2 = np.array([0, 2, 5, 6], dtype=np.int32)
    z2 = rng.normal(size=(6 + 3, V))
    d2 = rng.normal(size=(6, V))
    t2 = rng.integers(0, V, size=6).astype(np.int32)
    res = oracle.verify(oracle.F64, z2, d2, offsets2, t2, np.ones(3, np.float32), 3, V, 2,
                        lib=lib)
    assert res["accept_len"][1] == -1
    assert res["accept_len"][0] >= 0 and res["accept_len"][2] >= 0


# ------------------------------------------------------------------ near ties and the empty residual
#
# The parity tests forgive a GPU mismatch only on a request the oracle flags,
# so the flags are pinned like any other output: cases built so that the
# quantity a flag measures is known by construction (independently of the
# oracle's arithmetic) must flag inside the window and must not outside it.
# The accept test and the race follow "Decodificacion Especulativa y EAGLE",
# section "La Regla de Exactitud"; the window widths are the oracle's stated
# reading (1e-6 relative).


def _two_token_row(p):
    """float64 logits of the two-token distribution (p, 1 - p)."""
    return np.array([math.log(p), math.log1p(-p)])


def pin_accept_near_tie_flag(lib, seed=31):
    """r*q(x) placed at a known relative distance delta from p(x) (V = 2, K = 1, T = 1):
    |delta| = 1e-9 flags, |delta| = 1e-3 does not, also for probabilities near 1e-8
    (the window is relative); delta > 0 accepts and delta < 0 rejects."""
    cases = [(1e-9, 0.4), (-1e-9, 0.4), (1e-3, 0.4), (-1e-3, 0.4), (1e-9, 2e-8), (1e-3, 2e-8),
             (-1e-3, 2e-8)]
    B = len(cases)
    rows_t, rows_d, toks = [], [], []
    for b, (delta, q) in enumerate(cases):
        r = oracle.accept_uniform(seed, b, 0, lib=lib)
        p = r * q * (1.0 + delta)
        rows_t.append(np.stack([_two_token_row(p), np.zeros(2)]))
        rows_d.append(_two_token_row(q)[None, :])
        toks.append([0])
    target, draft, offsets, tokens = pack_requests(rows_t, rows_d, toks)
    res = oracle.verify(oracle.F64, target, draft, offsets, tokens, np.ones(B, np.float32), seed,
                        2, 1, lib=lib)
    for b, (delta, q) in enumerate(cases):
        flagged = bool(res["flags"][b] & oracle.FLAG_ACCEPT_NEAR_TIE)
        assert flagged == (abs(delta) < 1e-6), (b, delta, q, int(res["flags"][b]))
        assert int(res["accept_len"][b]) == (1 if delta > 0 else 0), (b, delta)
        # the reported probabilities are the constructed ones
        assert abs(res["q_at"][b] - q) <= 1e-12 * q
        r = oracle.accept_uniform(seed, b, 0, lib=lib)
        assert abs(res["p_at"][b] - r * q * (1 + delta)) <= 1e-12 * q


def pin_bonus_race_near_tie_flag(lib, seed=32):
    """Bonus race (K = 0, V = 2): logits chosen so the two race keys differ by a known
    eps.  |eps| = 1e-9 flags, |eps| = 1e-4 does not; the winner follows the sign of
    eps and race_gap equals |eps|.  The same rows shifted by +1000, or at T = 0.25,
    give the same outcome: the window does not widen with a logit offset."""
    cases = []
    for shift in (0.0, 1000.0):
        for T in (1.0, 0.25):
            for eps in (1e-9, -1e-9, 1e-4, -1e-4):
                cases.append((eps, shift, T))
    B = len(cases)
    rows_t, temps = [], []
    for b, (eps, shift, T) in enumerate(cases):
        e0 = oracle.race_exponential(seed, b, 0, 0, lib=lib)
        e1 = oracle.race_exponential(seed, b, 0, 1, lib=lib)
        # key_v = z_v / T - lse - ln E_v, so key_0 - key_1 = (z_0 - z_1) / T - ln(E_0 / E_1)
        d = (math.log(e0 / e1) + eps) * T
        rows_t.append(np.array([[shift + d, shift]]))
        temps.append(T)
    target = np.concatenate(rows_t)
    offsets = np.zeros(B + 1, np.int32)
    res = oracle.verify(oracle.F64, target, np.zeros((0, 2)), offsets, np.zeros(0, np.int32),
                        np.array(temps, np.float32), seed, 2, 0, lib=lib)
    for b, (eps, shift, T) in enumerate(cases):
        flagged = bool(res["flags"][b] & oracle.FLAG_RACE_NEAR_TIE)
        assert flagged == (abs(eps) < 1e-6), (b, eps, shift, T, float(res["race_gap"][b]))
        assert int(res["accept_len"][b]) == 0
        assert int(res["out_tokens"][b]) == (0 if eps > 0 else 1), (b, eps)
        assert abs(res["race_gap"][b] - abs(eps)) <= 1e-12 * (1 + shift) / T, (b, eps)


def _residual_tie_case(lib, seed, b, eps, mass):
    """Rows of one K = 1, V = 3 request whose draft x = 2 is always rejected
    (target p_2 = 0 < r*q_2) and whose residual (p - q)+ lives on tokens 0 and 1
    with weights w_0, w_1 (w_0 + w_1 = mass) chosen so that the residual race
    keys ln w_v - ln E_v differ by eps."""
    e0 = oracle.race_exponential(seed, b, 0, 0, lib=lib)
    e1 = oracle.race_exponential(seed, b, 0, 1, lib=lib)
    rho = (e0 / e1) * math.exp(eps)        # w_0 / w_1
    w1 = mass / (1.0 + rho)
    w0 = mass - w1
    q = np.array([0.5, 0.5 - mass, mass])
    p = np.array([q[0] + w0, q[1] + w1, 0.0])
    with np.errstate(divide="ignore"):
        zt = np.log(p)
    return np.stack([zt, np.zeros(3)]), np.log(q)[None, :], [2]


def pin_residual_race_near_tie_flag(lib, seed=33):
    """Residual race with two positive weights whose keys differ by a known eps.
    At residual mass 0.3: |eps| = 1e-9 flags, 1e-4 does not.  At mass 2e-9 the keys
    sit near ln(1e-9) ~ -21, so the window 1e-6 * |best| is ~2e-5: eps = 5e-6 flags
    there (the window scales with |best| above 1) and eps = 1e-4 does not."""
    cases = [(1e-9, 0.3), (-1e-9, 0.3), (1e-4, 0.3), (-1e-4, 0.3), (5e-6, 2e-9), (-5e-6, 2e-9),
             (1e-4, 2e-9)]
    rows_t, rows_d, toks = [], [], []
    for b, (eps, mass) in enumerate(cases):
        t, d, x = _residual_tie_case(lib, seed, b, eps, mass)
        rows_t.append(t)
        rows_d.append(d)
        toks.append(x)
    target, draft, offsets, tokens = pack_requests(rows_t, rows_d, toks)
    B = len(cases)
    res = oracle.verify(oracle.F64, target, draft, offsets, tokens, np.ones(B, np.float32), seed,
                        3, 1, lib=lib)
    for b, (eps, mass) in enumerate(cases):
        assert int(res["accept_len"][b]) == 0, b
        assert not (res["flags"][b] & oracle.FLAG_RESIDUAL_EMPTY), b
        best = float(res["race_best"][b])
        window = 1e-6 * max(1.0, abs(best))
        assert (abs(eps) < window) == bool(res["flags"][b] & oracle.FLAG_RACE_NEAR_TIE), \
            (b, eps, mass, best, int(res["flags"][b]))
        assert int(res["out_tokens"][offsets[b] + b]) == (0 if eps > 0 else 1), (b, eps)
        # w_v = p_v - q_v loses ~1e-16 absolute to rounding, so ln w_v carries ~1e-16 / w_v
        assert abs(res["race_gap"][b] - abs(eps)) <= 1e-7 * abs(eps) + 1e-14 + 3e-16 / mass, \
            (b, eps)
    # the tiny-mass cases are inside the widened window only because |best| > 1
    assert all(abs(float(res["race_best"][b])) > 10 for b in (4, 5, 6))


def pin_residual_empty_fallback(lib, seed=34, B=96):
    """A rejection with an empty residual.  Target row (1, 0, -800) against draft row
    (1, 0, -700) at T = 1, draft token 2: in float64 the target's p_2 underflows to 0
    while q_2 ~ 1e-305 does not, p_0 = q_0 and p_1 = q_1 exactly, so (p - q)+ is
    zero everywhere.  The request must reject at t = 0, set the residual-empty flag,
    and draw from p_0 instead: the winner is argmax over v of ln p_v - ln E_v.  An
    identical draft row accepts its token 0 (control).  The cases include seeds where that
    winner differs both from the plain minimum of E (an unweighted race) and from
    the minimum of E over tokens 0 and 1."""
    zt = np.array([[1.0, 0.0, -800.0], [0.0, 0.0, 0.0]])
    zq = np.array([[1.0, 0.0, -700.0]])
    assert math.exp(-800.0 - math.log(math.e + 1)) == 0.0 and math.exp(-700.0 - 1.32) > 0.0
    rows_t = [zt] * B + [zt]
    rows_d = [zq] * B + [zt[:1]]
    toks = [[2]] * B + [[0]]
    target, draft, offsets, tokens = pack_requests(rows_t, rows_d, toks)
    res = oracle.verify(oracle.F64, target, draft, offsets, tokens, np.ones(B + 1, np.float32),
                        seed, 3, 1, lib=lib)
    with np.errstate(divide="ignore"):
        lp = np.log(scipy.special.softmax(zt[0]))
    differs_unweighted = differs_pair = 0
    for b in range(B):
        assert int(res["accept_len"][b]) == 0, b
        assert res["flags"][b] & oracle.FLAG_RESIDUAL_EMPTY, b
        e = np.array([oracle.race_exponential(seed, b, 0, v, lib=lib) for v in range(3)])
        with np.errstate(divide="ignore"):
            want = int(np.argmax(lp - np.log(e)))
        assert int(res["out_tokens"][offsets[b] + b]) == want, (b, want, e)
        differs_unweighted += want != int(np.argmin(e))
        differs_pair += want != int(np.argmin(e[:2]))
    assert differs_unweighted > 0 and differs_pair > 0
    assert int(res["accept_len"][B]) == 1 and res["flags"][B] == 0


# ------------------------------------------------------------------ draft-side sampler


def pin_draft_distribution(lib, V=8, N=400_000):
    """The draft sampler draws exactly from softmax(z / T) (exponential race), at two T."""
    rng = np.random.default_rng(21)
    z = rng.normal(0, 1.5, size=V)
    for T, seed in ((1.3, 5), (0.45, 6)):
        Tf = float(np.float32(T))
        p = scipy.special.softmax(z / Tf)
        res = oracle.draft_sample(oracle.F64, np.tile(z, (N, 1)), np.full(N, T, np.float32),
                                  seed, 3, lib=lib)
        hist = np.bincount(res["tokens"], minlength=V) / N
        assert 0.5 * np.abs(hist - p).sum() < 0.005, (T, hist, p)
        assert scipy.stats.chisquare(hist * N, p * N).pvalue > 1e-5
        # q(x) is the softmax probability of the drawn token
        assert np.allclose(res["q_at"], p[res["tokens"]], rtol=1e-12, atol=0)


def pin_draft_greedy(lib):
    """T = 0 takes the first maximum (numpy's argmax), ties included."""
    rng = np.random.default_rng(22)
    B, V = 300, 33
    z = rng.integers(-3, 4, size=(B, V)).astype(np.float64)  # many ties
    res = oracle.draft_sample(oracle.F64, z, np.zeros(B, np.float32), 1, 0, lib=lib)
    assert (res["tokens"] == np.argmax(z, axis=1)).all()
    assert np.isnan(res["q_at"]).all()


def pin_draft_streams(lib, V=5, N=200_000):
    """Draft steps are independent draws, and independent of the verify step's race.

    The joint law of the tokens drawn at steps 0 and 1 for the same requests is
    the product law; the step-0 token agrees with the verify step's K = 0
    plain sample (same seed, request and position) only as often as two
    independent draws do (sum p^2), so the draft stream is a separate stream.
    """
    rng = np.random.default_rng(23)
    z = rng.normal(0, 1.0, size=V)
    p = scipy.special.softmax(z)
    rows = np.tile(z, (N, 1))
    temp = np.ones(N, np.float32)
    a = oracle.draft_sample(oracle.F64, rows, temp, 9, 0, lib=lib)["tokens"]
    b = oracle.draft_sample(oracle.F64, rows, temp, 9, 1, lib=lib)["tokens"]
    joint = np.bincount(a * V + b, minlength=V * V)
    assert scipy.stats.chisquare(joint, np.outer(p, p).ravel() * N).pvalue > 1e-5
    v = oracle.verify(oracle.F64, rows, np.zeros((0, V)), np.zeros(N + 1, np.int32),
                      np.zeros(0, np.int32), temp, 9, V, 0, lib=lib)["out_tokens"]
    same = (a == v).mean()
    want = float((p * p).sum())
    assert abs(same - want) < 5 * math.sqrt(want * (1 - want) / N), (same, want)


def pin_draft_faults(lib):
    """A bad temperature or a row with no finite maximum gives -1 for that request only."""
    rng = np.random.default_rng(24)
    B, V = 6, 12
    z = rng.normal(size=(B, V))
    temp = np.array([1.0, -1.0, np.nan, np.inf, 0.7, 0.0], np.float32)
    z[4, :] = -np.inf
    res = oracle.draft_sample(oracle.F64, z, temp, 2, 0, lib=lib)
    assert list(res["tokens"][1:5]) == [-1, -1, -1, -1]
    assert 0 <= res["tokens"][0] < V and res["tokens"][5] == int(np.argmax(z[5]))


def pin_draft_race_near_tie_flag(lib, seed=35):
    """Draft race (V = 2) with keys built to differ by a known eps, as for the bonus
    race: 1e-9 flags, 1e-4 does not, the winner follows the sign of eps, and a
    +1000 logit shift or T = 0.25 changes nothing."""
    cases = [(eps, shift, T) for shift in (0.0, 1000.0) for T in (1.0, 0.25)
             for eps in (1e-9, -1e-9, 1e-4, -1e-4)]
    step = 3
    rows = []
    for b, (eps, shift, T) in enumerate(cases):
        e0 = oracle.draft_exponential(seed, b, step, 0, lib=lib)
        e1 = oracle.draft_exponential(seed, b, step, 1, lib=lib)
        rows.append([shift + (math.log(e0 / e1) + eps) * T, shift])
    res = oracle.draft_sample(oracle.F64, np.array(rows), np.array([c[2] for c in cases],
                              np.float32), seed, step, lib=lib)
    for b, (eps, shift, T) in enumerate(cases):
        assert bool(res["flags"][b] & oracle.FLAG_RACE_NEAR_TIE) == (abs(eps) < 1e-6), (b, eps)
        assert int(res["tokens"][b]) == (0 if eps > 0 else 1), (b, eps)
        assert abs(res["race_gap"][b] - abs(eps)) <= 1e-12 * (1 + shift) / T, (b, eps)


# ------------------------------------------------------------------ commit step


def pin_commit_example(lib):
    """A hand-checked batch: append, empty draft, failed verify, capacity overflow,
    and an append that fills the history exactly."""
    offsets = np.array([0, 2, 2, 5, 6, 7], np.int32)       # K = 2, 0, 3, 1, 1
    accept = np.array([1, 0, -1, 1, 1], np.int32)
    # packed outputs: request b's block of K_b + 1 starts at offsets[b] + b
    out = np.array([7, 9, -1, 4, -1, -1, -1, -1, 11, 12, 13, 14], np.int32)
    seq = np.array([[1, 2, 3, 0, 0, 0], [5, 0, 0, 0, 0, 0], [6, 6, 6, 6, 6, 0],
                    [8, 8, 8, 8, 8, 0], [2, 2, 2, 2, 0, 0]], np.int32)
    lens = np.array([3, 1, 5, 5, 4], np.int32)
    r = oracle.commit_tokens(offsets, accept, out, seq, lens, 3, lib=lib)
    assert r["seq_tokens"].tolist() == [[1, 2, 3, 7, 9, 0], [5, 4, 0, 0, 0, 0],
                                        [6, 6, 6, 6, 6, 0], [8, 8, 8, 8, 8, 0],
                                        [2, 2, 2, 2, 13, 14]]
    assert r["seq_len"].tolist() == [5, 2, 5, 5, 6]
    assert r["next_tokens"].tolist() == [9, 4, -1, -1, 14]
    assert r["status"].tolist() == [2, 1, -1, -2, 2]


def pin_commit_after_verify(lib):
    """Committing a verify result appends the accepted drafts, then the emitted token,
    and leaves every earlier token of the history in place."""
    rng = np.random.default_rng(25)
    B, V, cap = 50, 30, 40
    ks = rng.integers(0, 6, size=B)
    offsets = np.zeros(B + 1, np.int32)
    offsets[1:] = np.cumsum(ks)
    n_d = int(offsets[-1])
    z = rng.normal(0, 2, size=(n_d + B, V))
    d = z[np.concatenate([np.arange(offsets[b] + b, offsets[b] + b + ks[b]) for b in range(B)])
          .astype(int)] + rng.normal(0, 0.7, size=(n_d, V)) if n_d else np.zeros((0, V))
    toks = rng.integers(0, V, size=n_d).astype(np.int32)
    temps = rng.choice([0.0, 1.0], size=B).astype(np.float32)
    v = oracle.verify(oracle.F64, z, d, offsets, toks, temps, 17, V, 5, lib=lib)
    seq = rng.integers(0, V, size=(B, cap)).astype(np.int32)
    lens = rng.integers(0, cap - 5, size=B).astype(np.int32)
    r = oracle.commit_tokens(offsets, v["accept_len"], v["out_tokens"], seq, lens, 5, lib=lib)
    for b in range(B):
        n, L = int(v["accept_len"][b]), int(lens[b])
        assert r["status"][b] == n + 1 and r["seq_len"][b] == L + n + 1
        row = r["seq_tokens"][b]
        assert (row[:L] == seq[b, :L]).all() and (row[L + n + 1:] == seq[b, L + n + 1:]).all()
        assert (row[L:L + n] == toks[offsets[b]:offsets[b] + n]).all()
        assert row[L + n] == v["out_tokens"][offsets[b] + b + n] == r["next_tokens"][b]


# ------------------------------------------------------------------ tree verify


def read_tree_cases():
    """Cases of tests/golden/tree_example.txt: (name, parents, tokens, argmax spec,
    expected accept, out, nodes); parents and tokens with the root's -1 prepended."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "tree_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
                cases.append(cur)
            elif key in ("parents", "tokens"):
                cur[key] = [-1] + [int(v) for v in vals]
            elif key == "argmax":
                cur[key] = vals
            elif key == "accept":
                cur[key] = int(vals[0])
            else:
                cur[key] = [int(v) for v in vals]
    return cases


def pin_tree_page_example(lib):
    """The page's two-level tree, argmaxes fixed by hand, expected outputs by hand."""
    V = 10
    for c in read_tree_cases():
        N = len(c["parents"])
        rows = np.full((N, V), -1.0)
        for i, spec in enumerate(c["argmax"]):
            g = int(spec.rstrip("t"))
            rows[i, g] = 2.0
            if spec.endswith("t"):
                rows[i, g + 1] = 2.0
        r = oracle.tree_verify(oracle.F64, rows, [0, N], c["parents"], c["tokens"], V, N, lib=lib)
        assert r["accept_len"].tolist() == [c["accept"]], (c["name"], r["accept_len"])
        assert r["out_tokens"].tolist() == c["out"], (c["name"], r["out_tokens"])
        assert r["accept_nodes"].tolist() == c["nodes"], (c["name"], r["accept_nodes"])


def pin_tree_chain_is_linear(lib):
    """A tree whose node i has parent i - 1 is a linear draft: the same rows, tokens
    and outputs as the greedy linear verify (itself pinned above)."""
    rng = np.random.default_rng(41)
    V, B = 12, 120
    ks = rng.integers(0, 8, size=B)
    offs = np.zeros(B + 1, np.int32)
    offs[1:] = np.cumsum(ks + 1)
    rows = rng.normal(0, 1.5, size=(int(offs[-1]), V))
    g = rows.argmax(axis=1)
    lin_tok, parents, tree_tok = [], [], []
    for b in range(B):
        o = int(offs[b])
        for t in range(int(ks[b])):
            # mostly the target's argmax, so that long prefixes occur
            x = int(g[o + t]) if rng.random() < 0.75 else int(rng.integers(0, V))
            lin_tok.append(x)
            tree_tok.append(x)
            parents.append(t)
        parents.insert(len(parents) - int(ks[b]), -1)
        tree_tok.insert(len(tree_tok) - int(ks[b]), -1)
    doffs = np.zeros(B + 1, np.int32)
    doffs[1:] = np.cumsum(ks)
    lin = oracle.verify(oracle.F64, rows, None, doffs, np.array(lin_tok, np.int32),
                        np.zeros(B, np.float32), 0, V, 8, lib=lib)
    tree = oracle.tree_verify(oracle.F64, rows, offs, parents, tree_tok, V, 9, lib=lib)
    assert (tree["accept_len"] == lin["accept_len"]).all()
    assert (tree["out_tokens"] == lin["out_tokens"]).all()
    for b in range(B):
        o, n = int(offs[b]), int(lin["accept_len"][b])
        assert tree["accept_nodes"][o:o + n + 1].tolist() == list(range(n + 1))
        assert (tree["accept_nodes"][o + n + 1:int(offs[b + 1])] == -1).all()
    assert 0 < (lin["accept_len"] > 2).sum() < B


def tree_by_paths(rows, parents, tokens):
    """Brute force: every node's root path, accepted if each token on it is numpy's
    first-occurrence argmax of its parent's row; the longest such path wins, the
    lowest end node among equally long ones."""
    N = len(parents)
    best = (0, 0, [0])
    for i in range(N):
        path = [i]
        while path[-1] != 0:
            path.append(parents[path[-1]])
        path.reverse()
        if all(tokens[v] == int(np.argmax(rows[u])) for u, v in zip(path, path[1:])):
            if len(path) - 1 > best[0]:
                best = (len(path) - 1, i, path)
    d, c, path = best
    out = [tokens[v] for v in path[1:]] + [int(np.argmax(rows[c]))]
    return d, out + [-1] * (N - d - 1), path + [-1] * (N - d - 1)


def pin_tree_brute_force(lib):
    """Random trees of up to 14 nodes over a 4-token vocabulary (so that siblings often
    share tokens and several paths are accepted) against path enumeration."""
    rng = np.random.default_rng(43)
    V, B = 4, 300
    sizes = rng.integers(1, 15, size=B)
    offs = np.zeros(B + 1, np.int32)
    offs[1:] = np.cumsum(sizes)
    rows = rng.integers(-3, 3, size=(int(offs[-1]), V)).astype(np.float64)  # many ties
    parents, tokens, want = [], [], []
    for b in range(B):
        N = int(sizes[b])
        par = [-1] + [int(rng.integers(max(0, i - 3), i)) for i in range(1, N)]  # deep trees
        blk = rows[offs[b]:offs[b + 1]]
        # half the tokens planted on the first maximum of the parent's row
        tok = [-1] + [int(np.argmax(blk[par[i]])) if rng.random() < 0.5 else
                      int(rng.integers(0, V)) for i in range(1, N)]
        parents += par
        tokens += tok
        want.append(tree_by_paths(rows[offs[b]:offs[b + 1]], par, tok))
    r = oracle.tree_verify(oracle.F64, rows, offs, parents, tokens, V, 14, lib=lib)
    for b in range(B):
        o, o1 = int(offs[b]), int(offs[b + 1])
        d, out, nodes = want[b]
        assert r["accept_len"][b] == d, (b, r["accept_len"][b], d)
        assert r["out_tokens"][o:o1].tolist() == out, b
        assert r["accept_nodes"][o:o1].tolist() == nodes, b
    assert (r["accept_len"] >= 3).sum() > 10


def pin_tree_faults(lib):
    """Bad parents, bad tokens, non-finite rows and bad slices fail only their own
    request; a request whose slice is bad gets no output writes."""
    V = 6
    rows = np.zeros((30, V))
    rows[:, 2] = 1.0
    offs = [0, 3, 6, 9, 12, 15, 15, 18, 21, 30]
    parents = [-1, 0, 1] * 10
    tokens = [-1, 2, 2] * 10
    parents[5] = 2          # request 1: a node's parent is itself
    tokens[7] = V           # request 2: token outside the vocabulary
    rows[10] = np.nan       # request 3: a row with no finite maximum
    rows[13] = -np.inf      # request 4: likewise
    parents[19] = -5        # request 7: negative parent
    r = oracle.tree_verify(oracle.F64, rows, offs, parents, tokens, V, 8, lib=lib)
    assert r["accept_len"].tolist() == [2, -1, -1, -1, -1, -1, 2, -1, -1]
    out = r["out_tokens"]
    assert out[0:3].tolist() == [2, 2, 2] and out[15:18].tolist() == [2, 2, 2]
    assert r["accept_nodes"][15:18].tolist() == [0, 1, 2]
    for o, o1 in ((3, 6), (6, 9), (9, 12), (12, 15), (18, 21)):
        assert (out[o:o1] == -1).all() and (r["accept_nodes"][o:o1] == -1).all()
    # request 5 is empty (N = 0), request 8 has 9 nodes > max_nodes = 8: nothing written
    assert (out[21:30] == -3).all() and (r["accept_nodes"][21:30] == -3).all()


ALL_PINS = [pin_philox_kat, pin_philox_rocrand, pin_u01, pin_softmax_vs_scipy,
            pin_greedy_vs_numpy, pin_exact_enumeration, pin_plain_sampling, pin_closed_form,
            pin_temperature_invariance, pin_identical_draft_accepts, pin_disjoint_draft_rejects,
            pin_faults, pin_accept_near_tie_flag, pin_bonus_race_near_tie_flag,
            pin_residual_race_near_tie_flag, pin_residual_empty_fallback,
            pin_draft_distribution, pin_draft_greedy, pin_draft_streams,
            pin_draft_faults, pin_draft_race_near_tie_flag, pin_commit_example, pin_commit_after_verify,
            pin_tree_page_example, pin_tree_chain_is_linear, pin_tree_brute_force,
            pin_tree_faults]
