"""The no-allocation verify entry point (spec_verify_sample_static) against
spec_verify_sample, through the C ABI.

Two calls in a row on the library's fixed device array, the second with a
smaller batch, must each give exactly what spec_verify_sample gives on the same
inputs with a fresh workspace (same kernel, so bit for bit), and both must meet
the oracle's match rules.  A size beyond the array is refused on the host.
"""
import numpy as np
import pytest

import oracle
from parity import compare, run_gpu
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


def run_static(batch, clear=False):
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    d = binding.to_device_batch(batch, "cuda")
    n_d = batch.n_draft_rows
    acc = torch.full((batch.B,), -9, dtype=torch.int32, device="cuda")
    out = torch.full((n_d + batch.B,), -9, dtype=torch.int32, device="cuda")
    pa = torch.empty(n_d, dtype=torch.float32, device="cuda")
    qa = torch.empty(n_d, dtype=torch.float32, device="cuda")
    binding.spec_verify_sample_static(d["target"], d["draft"], d["offsets"], d["tokens"],
                                      d["temperature"], batch.seed, batch.max_k, acc, out, pa, qa,
                                      clear_scratch=clear)
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(),
                p_at=pa.cpu().numpy().astype(np.float64), q_at=qa.cpu().numpy().astype(np.float64))


def same(a, b):
    assert np.array_equal(a["accept_len"], b["accept_len"])
    assert np.array_equal(a["out_tokens"], b["out_tokens"])
    assert np.array_equal(a["p_at"], b["p_at"], equal_nan=True)
    assert np.array_equal(a["q_at"], b["q_at"], equal_nan=True)


def test_static_scratch_matches_workspace_entry():
    big = W.make_batch(2, 0)                                        # B=64 K=4 V=128256 bf16
    rng = np.random.default_rng(77)
    ks = [int(x) for x in rng.integers(0, 9, size=12)]
    small = W.make_custom_batch(rng, W.DTYPE_F32, 40001, ks, rng.choice([0.0, 0.8, 1.0], size=12),
                                seed=5, max_k=8)                    # ragged, other dtype and V
    for name, b in (("llama B=64 K=4 bf16", big), ("ragged B=12 V=40001 f32", small)):
        say(f"static scratch: {name}")
        got = run_static(b)
        want = run_gpu(b, "sample")
        same(got, want)
        compare(b, got, oracle.verify_batch(b))
    say("static scratch: first batch again, with clear_scratch")
    same(run_static(big, clear=True), run_gpu(big, "sample"))


def test_static_scratch_refuses_oversize():
    import ctypes
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    lib = binding.load_library()
    B, V, K = 1024, 262144, 8
    need = lib.spec_verify_workspace_bytes(B, V, K)
    assert need > binding.SV_STATIC_SCRATCH_BYTES
    say("static scratch: oversize call (refused on the host, nothing launched)")
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(dummy.data_ptr())
    rc = lib.spec_verify_sample_static(p, p, binding.SV_BF16, B, V, K, B * K, p, p, p,
                                       ctypes.c_uint64(1), p, p, None, None, 0, None)
    assert rc == -6
    assert b"static scratch" in lib.spec_verify_status_string(rc)
