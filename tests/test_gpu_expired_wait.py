"""Expired waits, forced from the host side of the build (GPU).

libspecverify_spin0.so is the library built with every bounded wait cut to a
single load (SV_SPIN_LIMIT = 0), so a consumer that finds a hand-off slot not
yet written gives up at once.  Nothing faults or hangs: every wait still ends
and every kernel exits.  The contract being checked (the verify step's header):
a request whose wait expired reports accept_len = -1 and, for the verify step,
leaves its output tokens unwritten; every other request is exact against the
oracle; and after the workspace is zero-filled again the normal library gives
exact results on it.
"""
import os

import numpy as np
import pytest

import oracle
from parity import P_TOL, compare
from rejection_sampling_verify_scaled_amd import build as hip_build
from rejection_sampling_verify_scaled_amd import workloads as W

pytestmark = pytest.mark.gpu

SENTINEL = -9


def say(*a):
    print("[gpu-case]", *a, flush=True)


@pytest.fixture(scope="module")
def libs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rejection_sampling_verify_scaled_amd import binding
    assert os.path.exists(hip_build.LIB_SPIN0), (
        f"{hip_build.LIB_SPIN0} is missing: build it with "
        "`python -m rejection_sampling_verify_scaled_amd.build --all`")
    return binding.load_library(), binding.load_library(hip_build.LIB_SPIN0)


def outputs(batch):
    import torch
    n_d = batch.n_draft_rows
    return dict(acc=torch.full((batch.B,), SENTINEL, dtype=torch.int32, device="cuda"),
                out=torch.full((n_d + batch.B,), SENTINEL, dtype=torch.int32, device="cuda"),
                pa=torch.full((n_d,), float(SENTINEL), dtype=torch.float32, device="cuda"),
                qa=torch.full((n_d,), float(SENTINEL), dtype=torch.float32, device="cuda"))


def host(o):
    import torch
    torch.cuda.synchronize()
    return dict(accept_len=o["acc"].cpu().numpy(), out_tokens=o["out"].cpu().numpy(),
                p_at=o["pa"].cpu().numpy().astype(np.float64),
                q_at=o["qa"].cpu().numpy().astype(np.float64))


def split(batch, got, untouched_tokens):
    """Requests that expired (accept_len = -1) and the rest; checks the expired ones."""
    expired, done = [], []
    for b in range(batch.B):
        if int(got["accept_len"][b]) == -1:
            expired.append(b)
            if untouched_tokens:
                o0, o1 = int(batch.offsets[b]), int(batch.offsets[b + 1])
                assert (got["out_tokens"][o0 + b:o1 + b + 1] == SENTINEL).all(), b
        else:
            done.append(b)
    return expired, done


@pytest.mark.parametrize("mode", ["sample", "greedy"])
def test_verify_expired_waits(libs, mode):
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    lib, lib0 = libs
    b = W.make_batch(2, 0)
    d = binding.to_device_batch(b, "cuda")
    ws = binding.new_workspace(b.B, b.V, b.max_k)
    orc = oracle.verify_batch(b, greedy_only=mode == "greedy")

    def call(which):
        o = outputs(b)
        if mode == "greedy":
            binding.spec_verify_greedy(d["target"], d["offsets"], d["tokens"], b.max_k, o["acc"],
                                       o["out"], workspace=ws, lib=which)
        else:
            binding.spec_verify_sample(d["target"], d["draft"], d["offsets"], d["tokens"],
                                       d["temperature"], b.seed, b.max_k, o["acc"], o["out"],
                                       o["pa"], o["qa"], workspace=ws, lib=which)
        return host(o)

    say(f"verify {mode}, waits cut to one load")
    got = call(lib0)
    expired, done = split(b, got, untouched_tokens=True)
    print(f"{mode}: {len(expired)} of {b.B} requests expired")
    assert expired, "no wait expired: the test exercised nothing"
    compare(b, got, orc, reqs=done, greedy_only=mode == "greedy", check_pq=mode == "sample")
    say(f"verify {mode}, normal library on the re-zeroed workspace")
    ws.zero_()
    again = call(lib)
    compare(b, again, orc, greedy_only=mode == "greedy", check_pq=mode == "sample")
    assert int((ws != 0).sum().item()) == 0


def test_early_exit_expired_waits(libs):
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    lib, lib0 = libs
    b = W.make_batch(2, 0)
    d = binding.to_device_batch(b, "cuda")
    ws = torch.zeros(binding.early_exit_workspace_bytes(b.B, b.V, b.max_k), dtype=torch.uint8,
                     device="cuda")
    orc = oracle.verify_batch(b)

    def call(which):
        o = outputs(b)
        binding.spec_verify_sample_early_exit(d["target"], d["draft"], d["offsets"], d["tokens"],
                                              d["temperature"], b.seed, b.max_k, o["acc"],
                                              o["out"], o["pa"], o["qa"], workspace=ws, lib=which)
        return host(o)

    say("early exit, waits cut to one load")
    got = call(lib0)
    expired, done = split(b, got, untouched_tokens=False)
    print(f"early exit: {len(expired)} of {b.B} requests expired")
    assert expired
    compare(b, got, orc, reqs=done, check_pq=False)
    say("early exit, normal library on the re-zeroed workspace")
    ws.zero_()
    compare(b, call(lib), orc, check_pq=False)


def test_draft_expired_waits(libs):
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    lib, lib0 = libs
    b = W.make_batch(2, 0)
    rows = W.draft_step_rows(b, 1)
    x = torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(b.temperature).cuda()
    ws = torch.zeros(binding.draft_workspace_bytes(b.B, b.V), dtype=torch.uint8, device="cuda")
    ref = oracle.draft_sample(b.dtype, rows, b.temperature, b.seed, 1)
    say("draft sampler, waits cut to one load")
    tok, q = binding.spec_draft_sample(x, t, b.seed, 1, workspace=ws, lib=lib0)
    torch.cuda.synchronize()
    tok, q = tok.cpu().numpy(), q.cpu().numpy()
    expired = tok == -1
    print(f"draft: {int(expired.sum())} of {b.B} rows expired")
    assert expired.any()
    assert (tok[~expired] == ref["tokens"][~expired]).all()
    s = ~expired & (b.temperature > 0)
    assert (np.abs(q[s] - ref["q_at"][s]) <= P_TOL).all()
    assert np.isnan(q[expired]).all()
    say("draft sampler, normal library on the re-zeroed workspace")
    ws.zero_()
    tok, _ = binding.spec_draft_sample(x, t, b.seed, 1, workspace=ws, lib=lib)
    torch.cuda.synchronize()
    assert (tok.cpu().numpy() == ref["tokens"]).all()
    assert int((ws != 0).sum().item()) == 0


def test_tree_expired_waits(libs):
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    lib, lib0 = libs
    tb = W.make_tree_batch("tree-eagle")
    want = oracle.tree_verify(tb.dtype, tb.target, tb.offsets, tb.parents, tb.tokens, tb.V,
                              tb.max_nodes)
    tgt = torch.from_numpy(np.ascontiguousarray(tb.target).view(np.int16)).cuda().view(
        torch.bfloat16)
    offs = torch.from_numpy(tb.offsets).cuda()
    par = torch.from_numpy(tb.parents).cuda()
    tok = torch.from_numpy(tb.tokens).cuda()
    ws = torch.zeros(binding.tree_workspace_bytes(tb.B, tb.V, tb.max_nodes), dtype=torch.uint8,
                     device="cuda")
    say("tree, waits cut to one load")
    acc, out, nodes = binding.spec_verify_tree_greedy(tgt, offs, par, tok, tb.max_nodes,
                                                      workspace=ws, lib=lib0)
    torch.cuda.synchronize()
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    expired = acc == -1
    print(f"tree: {int(expired.sum())} of {tb.B} requests expired")
    assert expired.any()
    for b in range(tb.B):
        o, o1 = tb.offsets[b], tb.offsets[b + 1]
        if expired[b]:
            assert (out[o:o1] == -1).all(), b
        else:
            assert acc[b] == want["accept_len"][b] and (out[o:o1] == want["out_tokens"][o:o1]).all()
    say("tree, normal library on the re-zeroed workspace")
    ws.zero_()
    acc, out, _ = binding.spec_verify_tree_greedy(tgt, offs, par, tok, tb.max_nodes, workspace=ws,
                                                  lib=lib)
    torch.cuda.synchronize()
    assert (acc.cpu().numpy() == want["accept_len"]).all()
    assert (out.cpu().numpy() == want["out_tokens"]).all()
