"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph).

A serving loop replays one captured step instead of issuing its launches one
by one. The library's calls enqueue kernels only (no allocation, no memset,
no host synchronisation), and each call leaves its workspace zeroed for the
next one. So a captured call replays correctly.

Each case captures the call once, then replays it several times. Before every
replay, eager work overwrites the outputs, and a synchronisation follows it.
Every replay must reproduce the eager call's outputs exactly and leave the
workspace zeroed.
"""
import numpy as np
import pytest

from rejection_sampling_verify_scaled_amd import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 5


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


def capture_and_replay(run, outputs, workspace):
    """run() enqueues the call on the current stream, writing into `outputs`."""
    import torch
    run()  # eager reference
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    assert int(workspace.count_nonzero()) == 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream, as torch recommends
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in outputs:  # eager work between replays
            o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            if o.dtype.is_floating_point:
                assert torch.equal(torch.nan_to_num(o, nan=-1e30), torch.nan_to_num(r, nan=-1e30)), rep
            else:
                assert torch.equal(o, r), rep
        assert int(workspace.count_nonzero()) == 0, rep
    del g


def test_verify_sample_in_graph():
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    say("graph: spec_verify_sample, Llama-class batch")
    b = W.make_batch(2, 0)
    d = binding.to_device_batch(b)
    acc = torch.empty(b.B, dtype=torch.int32, device="cuda")
    out = torch.empty(b.n_draft_rows + b.B, dtype=torch.int32, device="cuda")
    pa = torch.empty(b.n_draft_rows, dtype=torch.float32, device="cuda")
    qa = torch.empty(b.n_draft_rows, dtype=torch.float32, device="cuda")
    ws = binding.new_workspace(b.B, b.V, b.max_k)

    def run():
        binding.spec_verify_sample(d["target"], d["draft"], d["offsets"], d["tokens"],
                                   d["temperature"], b.seed, b.max_k, accept_len=acc,
                                   out_tokens=out, p_at_draft=pa, q_at_draft=qa, workspace=ws)
    capture_and_replay(run, [acc, out, pa, qa], ws)


def test_early_exit_in_graph():
    """Two launches per call (the verify kernel, then the record clearing)."""
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    say("graph: spec_verify_sample_early_exit, ragged batch")
    b = W.make_batch(5, 0, B=128)
    d = binding.to_device_batch(b)
    acc = torch.empty(b.B, dtype=torch.int32, device="cuda")
    out = torch.empty(b.n_draft_rows + b.B, dtype=torch.int32, device="cuda")
    ws = torch.zeros(binding.early_exit_workspace_bytes(b.B, b.V, b.max_k), dtype=torch.uint8,
                     device="cuda")

    def run():
        binding.spec_verify_sample_early_exit(d["target"], d["draft"], d["offsets"], d["tokens"],
                                              d["temperature"], b.seed, b.max_k, accept_len=acc,
                                              out_tokens=out, workspace=ws)
    capture_and_replay(run, [acc, out], ws)


def test_decode_step_in_graph():
    """Draft sampler for every position, verify and commit captured as one graph.
    The histories advance on every replay, so they are reset eagerly before it."""
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    say("graph: draft sampler x K, verify, commit")
    b = W.make_batch(4, 0, B=64)
    d = binding.to_device_batch(b)
    rows = [torch.from_numpy(np.ascontiguousarray(W.draft_step_rows(b, t)).view(np.int16))
            .cuda().view(torch.bfloat16) for t in range(b.max_k)]
    ks = torch.from_numpy(np.diff(b.offsets).astype(np.int64)).cuda()
    starts = d["offsets"][:-1].long()
    cap = 32
    seq0 = torch.from_numpy(np.random.default_rng(3).integers(0, b.V, size=(b.B, cap))
                            .astype(np.int32)).cuda()
    lens0 = torch.full((b.B,), 5, dtype=torch.int32, device="cuda")
    tok = torch.empty(b.B, dtype=torch.int32, device="cuda")
    tokens = torch.empty(b.n_draft_rows, dtype=torch.int32, device="cuda")
    acc = torch.empty(b.B, dtype=torch.int32, device="cuda")
    out = torch.empty(b.n_draft_rows + b.B, dtype=torch.int32, device="cuda")
    seq = seq0.clone()
    lens = lens0.clone()
    nxt = torch.empty(b.B, dtype=torch.int32, device="cuda")
    st = torch.empty(b.B, dtype=torch.int32, device="cuda")
    dws = torch.zeros(binding.draft_workspace_bytes(b.B, b.V), dtype=torch.uint8, device="cuda")
    vws = binding.new_workspace(b.B, b.V, b.max_k)
    # fixed index tensors, so the capture holds no data-dependent shapes
    src = [torch.nonzero(ks > t).flatten() for t in range(b.max_k)]
    idx = [starts[src[t]] + t for t in range(b.max_k)]

    def run():
        for t in range(b.max_k):
            binding.spec_draft_sample(rows[t], d["temperature"], 777, t, tokens=tok,
                                      want_q=False, workspace=dws)
            tokens.index_copy_(0, idx[t], tok.index_select(0, src[t]))
        binding.spec_verify_sample(d["target"], d["draft"], d["offsets"], tokens,
                                   d["temperature"], b.seed, b.max_k, accept_len=acc,
                                   out_tokens=out, workspace=vws)
        binding.spec_commit_tokens(d["offsets"], acc, out, seq, lens, b.max_k, next_tokens=nxt,
                                   status=st)

    run()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (tokens, acc, out, seq, lens, nxt, st)]
    g = torch.cuda.CUDAGraph()
    seq.copy_(seq0)
    lens.copy_(lens0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(REPLAYS):
        seq.copy_(seq0)
        lens.copy_(lens0)
        for x in (tokens, acc, out, nxt, st):
            x.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, r in zip((tokens, acc, out, seq, lens, nxt, st), ref):
            assert torch.equal(x, r), rep
        assert int(dws.count_nonzero()) == 0 and int(vws.count_nonzero()) == 0, rep
    assert (acc >= 0).all() and (st == acc + 1).all()
