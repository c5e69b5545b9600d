"""One speculative-decoding step end to end on the GPU, against the oracle's chain.

The draft-side sampler is called once per draft position on that position's
draft rows and chooses the draft tokens. The verify step judges those tokens
against the target rows, and the commit step appends each request's emitted
tokens to its history. Every hand-off between the three steps stays on the
device. The oracle runs the same chain on the CPU.

Parity: a request whose draft tokens or verify outcome the oracle flags as a
near tie is allowed to differ (its later steps then see other inputs).
Every other request must match exactly: draft tokens, accept length,
emitted tokens, history, length, next token and status.
"""
import numpy as np
import pytest

import oracle
from rejection_sampling_verify_scaled_amd import workloads as W

pytestmark = pytest.mark.gpu

DRAFT_SEED = 4242


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


def upload_rows(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def gpu_chain(b, seq0, lens0, cap):
    """Draft K positions, verify, commit; everything on the device."""
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    d = binding.to_device_batch(b)
    ks = torch.from_numpy(np.diff(b.offsets).astype(np.int64)).cuda()
    starts = d["offsets"][:-1].long()
    tokens = torch.full((max(b.n_draft_rows, 1),), -7, dtype=torch.int32, device="cuda")
    for t in range(b.max_k):
        rows = upload_rows(W.draft_step_rows(b, t))
        tok, _ = binding.spec_draft_sample(rows, d["temperature"], DRAFT_SEED, t, want_q=False)
        live = ks > t
        tokens[starts[live] + t] = tok[live]
    tokens = tokens[:b.n_draft_rows]
    acc, out, _, _ = binding.spec_verify_sample(
        d["target"], d["draft"], d["offsets"], tokens, d["temperature"], b.seed, b.max_k)
    seq = torch.from_numpy(seq0.copy()).cuda()
    lens = torch.from_numpy(lens0.copy()).cuda()
    nxt, st = binding.spec_commit_tokens(d["offsets"], acc, out, seq, lens, b.max_k)
    torch.cuda.synchronize()
    return dict(draft_tokens=tokens.cpu().numpy(), accept_len=acc.cpu().numpy(),
                out_tokens=out.cpu().numpy(), seq_tokens=seq.cpu().numpy(),
                seq_len=lens.cpu().numpy(), next_tokens=nxt.cpu().numpy(),
                status=st.cpu().numpy())


def oracle_chain(b, seq0, lens0):
    tokens = np.full(b.n_draft_rows, -7, dtype=np.int32)
    draft_flag = np.zeros(b.B, dtype=bool)
    ks = np.diff(b.offsets)
    for t in range(b.max_k):
        r = oracle.draft_sample(b.dtype, W.draft_step_rows(b, t), b.temperature, DRAFT_SEED, t)
        for q in range(b.B):
            if ks[q] > t:
                tokens[b.offsets[q] + t] = r["tokens"][q]
                draft_flag[q] |= (r["flags"][q] & oracle.FLAG_RACE_NEAR_TIE) != 0
    v = oracle.verify(b.dtype, b.target, b.draft, b.offsets, tokens, b.temperature, b.seed, b.V,
                      b.max_k)
    c = oracle.commit_tokens(b.offsets, v["accept_len"], v["out_tokens"], seq0, lens0, b.max_k,
                             n_draft_rows=b.n_draft_rows)
    near_tie = oracle.FLAG_ACCEPT_NEAR_TIE | oracle.FLAG_RACE_NEAR_TIE
    flagged = draft_flag | ((b.temperature > 0) & ((v["flags"] & near_tie) != 0))
    return dict(draft_tokens=tokens, accept_len=v["accept_len"], out_tokens=v["out_tokens"],
                **c), flagged


@pytest.mark.parametrize("cfg,B", [(2, None), (4, 128), (5, 96)])
def test_decode_step_chain(cfg, B):
    say("decode step chain", cfg, B)
    b = W.make_batch(cfg, 0, B=B)
    rng = np.random.default_rng(cfg)
    cap = 64
    seq0 = rng.integers(0, b.V, size=(b.B, cap)).astype(np.int32)
    lens0 = rng.integers(0, cap - b.max_k - 1, size=b.B).astype(np.int32)
    got = gpu_chain(b, seq0, lens0, cap)
    want, flagged = oracle_chain(b, seq0, lens0)
    assert flagged.sum() <= 0.001 * (b.temperature > 0).sum(), flagged.sum()
    exact = ~flagged
    for q in np.flatnonzero(exact):
        o, o1 = int(b.offsets[q]), int(b.offsets[q + 1])
        assert (got["draft_tokens"][o:o1] == want["draft_tokens"][o:o1]).all(), q
        assert got["accept_len"][q] == want["accept_len"][q], q
        assert (got["out_tokens"][o + q:o1 + q + 1] == want["out_tokens"][o + q:o1 + q + 1]).all(), q
        for k in ("seq_len", "next_tokens", "status"):
            assert got[k][q] == want[k][q], (k, q)
        assert (got["seq_tokens"][q] == want["seq_tokens"][q]).all(), q
    # the chain did real work: some drafts accepted, some rejected
    n = want["accept_len"][exact]
    assert (n > 0).any() and (n < np.diff(b.offsets)[exact]).any()
    assert (want["status"][exact] == n + 1).all()
