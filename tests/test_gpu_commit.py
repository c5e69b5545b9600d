"""GPU parity of the commit step (spec_commit_tokens) against the oracle: bit-exact.

The verify outputs fed to the commit step come from the oracle (uploaded as
inputs); an end-to-end case chains the GPU verify step into the GPU commit
step and compares with the oracle's chain on every request the verify
comparison itself accepts as exact.
"""
import numpy as np
import pytest

import oracle
from parity import run_gpu
from rejection_sampling_verify_scaled_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rejection_sampling_verify_scaled_amd import binding
    binding.load_library()
    yield


def gpu_commit(offsets, accept, out, seq, lens, max_k, capacity=None):
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    seq_d, lens_d = t(seq), t(lens)
    nxt, st = binding.spec_commit_tokens(t(offsets), t(accept), t(out), seq_d, lens_d, max_k,
                                         capacity=capacity)
    torch.cuda.synchronize()
    return dict(seq_tokens=seq_d.cpu().numpy(), seq_len=lens_d.cpu().numpy(),
                next_tokens=nxt.cpu().numpy(), status=st.cpu().numpy())


def same(a, b):
    for k in ("seq_tokens", "seq_len", "next_tokens", "status"):
        assert (a[k] == b[k]).all(), (k, np.nonzero(a[k] != b[k]))


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_commit_after_oracle_verify(cfg):
    """Workload batches: histories of random lengths, some near capacity."""
    b = W.make_batch(cfg, 0)
    reqs = None if b.B <= 64 else list(range(0, b.B, 8))
    v = oracle.verify_batch(b, reqs=reqs)
    acc = v["accept_len"].copy()
    acc[acc == -2] = -1  # requests the oracle skipped: treated as failed
    rng = np.random.default_rng(cfg)
    cap = 48
    seq = rng.integers(0, b.V, size=(b.B, cap)).astype(np.int32)
    lens = rng.integers(0, cap + 1, size=b.B).astype(np.int32)  # some overflow
    say(f"commit after oracle verify, workload {cfg}")
    ref = oracle.commit_tokens(b.offsets, acc, v["out_tokens"], seq, lens, b.max_k,
                               n_draft_rows=b.n_draft_rows)
    got = gpu_commit(b.offsets, acc, v["out_tokens"], seq, lens, b.max_k)
    same(got, ref)
    assert (ref["status"] == -2).any() and (ref["status"] > 0).any()


def test_commit_edge_cases():
    """Failed verify, n > K, bad slices, negative length, exact fill, K = 0."""
    offsets = np.array([0, 2, 2, 5, 6, 7, 9], np.int32)
    n_d, B = 9, 6
    accept = np.array([1, 0, -1, 1, 1, 3], np.int32)   # b5: n > K
    out = np.arange(100, 100 + n_d + B, dtype=np.int32)
    seq = np.zeros((B, 6), np.int32)
    lens = np.array([3, 1, 5, -1, 4, 0], np.int32)    # b3: negative length
    say("commit edge cases")
    ref = oracle.commit_tokens(offsets, accept, out, seq, lens, 3, n_draft_rows=n_d)
    same(gpu_commit(offsets, accept, out, seq, lens, 3), ref)
    assert ref["status"].tolist() == [2, 1, -1, -2, 2, -1]
    bad = offsets.copy()
    bad[2] = 9  # slices of b1 and b2 out of order
    ref = oracle.commit_tokens(bad, accept, out, seq, lens, 3, n_draft_rows=n_d)
    same(gpu_commit(bad, accept, out, seq, lens, 3), ref)


def test_verify_then_commit_on_gpu():
    """GPU verify -> GPU commit equals oracle verify -> oracle commit."""
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    b = W.make_batch(2, 3)
    d = binding.to_device_batch(b, "cuda")
    say("verify then commit")
    acc, out, _, _ = binding.spec_verify_sample(d["target"], d["draft"], d["offsets"],
                                                d["tokens"], d["temperature"], b.seed, b.max_k)
    rng = np.random.default_rng(5)
    cap = 40
    seq = rng.integers(0, b.V, size=(b.B, cap)).astype(np.int32)
    lens = rng.integers(0, 30, size=b.B).astype(np.int32)
    seq_d = torch.from_numpy(seq).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    nxt, st = binding.spec_commit_tokens(d["offsets"], acc, out, seq_d, lens_d, b.max_k)
    torch.cuda.synchronize()
    v = oracle.verify_batch(b)
    ref = oracle.commit_tokens(b.offsets, v["accept_len"], v["out_tokens"], seq, lens, b.max_k)
    ok = (v["flags"] == 0) | (b.temperature == 0)
    assert ok.sum() >= b.B - 1
    for k, g in (("seq_tokens", seq_d), ("seq_len", lens_d), ("next_tokens", nxt),
                 ("status", st)):
        assert (g.cpu().numpy()[ok] == ref[k][ok]).all(), k
