"""Shared helpers of the GPU parity tests: run a workload Batch through the C
ABI (via the ctypes binding) and compare it with the float64 oracle.

Match rules (see the design notes):
  * greedy requests: accept length and every token bit-exact;
  * sampled requests: accept length and tokens exact unless the oracle flags
    the request as a near-tie: |r*q - p| < 1e-6 * max(p, r*q) at an evaluated
    position (relative), or the two best race keys ln w - ln E within
    1e-6 * max(1, |best|); flagged requests stay under 0.1% of the sampled
    requests compared (no allowance of one);
  * p_t(x_t), q_t(x_t): within 1e-5 absolute of the oracle;
  * failed requests (accept_len == -1) must fail on both sides.
"""
from __future__ import annotations

import numpy as np

import oracle

P_TOL = 1e-5


def run_gpu(batch, mode="sample", device="cuda", workspace=None, want_pq=True):
    import torch
    from rejection_sampling_verify_scaled_amd import binding

    d = binding.to_device_batch(batch, device)
    if mode == "greedy":
        acc, out = binding.spec_verify_greedy(d["target"], d["offsets"], d["tokens"],
                                              batch.max_k, workspace=workspace)
        pa = qa = None
    else:
        n_d = batch.n_draft_rows
        pa = torch.empty(n_d, dtype=torch.float32, device=device) if want_pq else None
        qa = torch.empty(n_d, dtype=torch.float32, device=device) if want_pq else None
        acc, out, pa, qa = binding.spec_verify_sample(
            d["target"], d["draft"], d["offsets"], d["tokens"], d["temperature"], batch.seed,
            batch.max_k, p_at_draft=pa, q_at_draft=qa, workspace=workspace)
    torch.cuda.synchronize()
    res = dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy())
    if pa is not None:
        res["p_at"] = pa.cpu().numpy().astype(np.float64)
        res["q_at"] = qa.cpu().numpy().astype(np.float64)
    return res


class Tally:
    def __init__(self):
        self.sampled = 0
        self.greedy = 0
        self.failed = 0
        self.flagged = 0
        self.flagged_mismatch = 0
        self.max_p_err = 0.0

    def __repr__(self):
        return (f"Tally(sampled={self.sampled}, greedy={self.greedy}, failed={self.failed}, "
                f"flagged={self.flagged}, flagged_mismatch={self.flagged_mismatch}, "
                f"max_p_err={self.max_p_err:.3g})")


def compare(batch, gpu, orc, reqs=None, greedy_only=False, tally=None, check_pq=True):
    """Assert the match rules request by request; returns the Tally."""
    tally = tally or Tally()
    B = batch.B
    reqs = range(B) if reqs is None else reqs
    problems = []
    for b in reqs:
        b = int(b)
        o0, o1 = int(batch.offsets[b]), int(batch.offsets[b + 1])
        k = o1 - o0
        base = o0 + b
        g_acc, o_acc = int(gpu["accept_len"][b]), int(orc["accept_len"][b])
        if o_acc == -1:
            tally.failed += 1
            if g_acc != -1:
                problems.append((b, "oracle failed the request, GPU did not", g_acc))
            elif 0 <= o0 and o1 <= batch.n_draft_rows and 0 <= k <= batch.max_k:
                if not (gpu["out_tokens"][base:base + k + 1] == -1).all():
                    problems.append((b, "failed request has tokens"))
            continue
        T = 0.0 if greedy_only else float(batch.temperature[b])
        g_tok = gpu["out_tokens"][base:base + k + 1]
        o_tok = orc["out_tokens"][base:base + k + 1]
        same = g_acc == o_acc and (g_tok == o_tok).all()
        # invariants on the GPU output alone: prefix = drafts, then one token, then -1
        if not (0 <= g_acc <= k):
            problems.append((b, "accept_len out of range", g_acc))
        else:
            if not (g_tok[:g_acc] == batch.tokens[o0:o0 + g_acc]).all():
                problems.append((b, "emitted prefix differs from the drafts"))
            if not (0 <= g_tok[g_acc] < batch.V) or not (g_tok[g_acc + 1:] == -1).all():
                problems.append((b, "bad stop token / padding"))
        if T == 0.0:
            tally.greedy += 1
            if not same:
                problems.append((b, "greedy mismatch", g_acc, o_acc, list(g_tok), list(o_tok)))
            continue
        tally.sampled += 1
        flagged = int(orc["flags"][b]) & (oracle.FLAG_ACCEPT_NEAR_TIE | oracle.FLAG_RACE_NEAR_TIE)
        if flagged:
            tally.flagged += 1
            if not same:
                tally.flagged_mismatch += 1
        elif not same:
            problems.append((b, "sampled mismatch (unflagged)", g_acc, o_acc, list(g_tok),
                             list(o_tok), float(orc["race_gap"][b])))
        if check_pq and "p_at" in gpu and k > 0:
            for name in ("p_at", "q_at"):
                e = np.abs(gpu[name][o0:o1] - orc[name][o0:o1])
                tally.max_p_err = max(tally.max_p_err, float(e.max()))
                if not (e <= P_TOL).all():
                    problems.append((b, f"{name} off by {e.max():.3g}"))
    assert not problems, f"{len(problems)} problems, first: {problems[:5]}"
    check_flag_rate(tally)
    return tally


def check_flag_rate(tally):
    """Flagged (forgiven) sampled requests stay under 0.1% of those compared."""
    assert tally.flagged <= 0.001 * tally.sampled, tally
