"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Every case below copies the oracle's C source, plants one plausible mistake by
text substitution, builds the copy in a temporary directory and runs the pins
of tests/oracle_pins.py against it.  A mistake that no pin notices would mean
the pins cannot vouch for that part of the oracle.  The committed oracle is
never modified.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins as P

MUTANTS = {
    # residual drops the draft term: raced on p instead of (p - q)+
    "residual_without_q": ("double w = p - q;", "double w = p;"),
    # the lesson listing's slip: subtract the scalar q(x_t) from the vector p
    "residual_minus_scalar_q": (
        "double w = p - q;",
        "double w = p - exp(logit(in->draft, in->dtype, drow0 + n, V, "
        "in->tokens[off + n]) / T - lq[n]);"),
    # ratio test with its operands transposed
    "accept_transposed": ("if (!(r * q < p)) n = t;", "if (!(r * p < q)) n = t;"),
    # one uniform reused for every position
    "accept_uniform_reused": ("oracle_accept_uniform(in->seed, b, t)",
                              "oracle_accept_uniform(in->seed, b, 0)"),
    # draft logits not divided by the temperature
    "draft_untempered": (
        "lq[t] = row_lse(in->draft, in->dtype, drow0 + t, V, T);",
        "lq[t] = row_lse(in->draft, in->dtype, drow0 + t, V, 1.0);"),
    # the max shift of the log-sum-exp applied without the temperature
    "lse_shift_untempered": ("/ T - m / T);", "/ T - m);"),
    # greedy ties resolved to the last index
    "greedy_last_tie": ("if (z > m) {\n      m = z;\n      idx = v;",
                        "if (z >= m) {\n      m = z;\n      idx = v;"),
    # target rows addressed like draft rows (missing the per-request +b)
    "target_row_alignment": ("const int64_t trow0 = (int64_t)off + b;",
                             "const int64_t trow0 = (int64_t)off;"),
    # bonus drawn from the last drafted position instead of the one after it
    "bonus_wrong_row": ("key = logit(in->target, in->dtype, trow0 + n, V, v) / T - lp[n] - log(e);",
                        "key = logit(in->target, in->dtype, trow0 + (n > 0 ? n - 1 : 0), V, v)"
                        " / T - lp[n] - log(e);"),
    # bonus key left unnormalised (z / T - ln E): the near-tie window then grows with a
    # constant added to the logits
    "bonus_key_unshifted": ("/ T - lp[n] - log(e);", "/ T - log(e);"),
    # accept near-tie window 1000 times too wide
    "accept_flag_wide": ("fabs(r * q - p) < 1e-6 * fmax(p, r * q)",
                         "fabs(r * q - p) < 1e-3 * fmax(p, r * q)"),
    # accept near-tie window absolute instead of relative
    "accept_flag_absolute": ("fabs(r * q - p) < 1e-6 * fmax(p, r * q)", "fabs(r * q - p) < 1e-6"),
    # race near-tie window 1000 times too wide (verify step)
    "race_flag_wide": ("if (best - second < 1e-6 * fmax(1.0, fabs(best)) && o->flags)",
                       "if (best - second < 1e-3 * fmax(1.0, fabs(best)) && o->flags)"),
    # race near-tie window that does not scale with |best|
    "race_flag_unscaled": ("if (best - second < 1e-6 * fmax(1.0, fabs(best)) && o->flags)",
                           "if (best - second < 1e-6 * fmin(1.0, fabs(best)) && o->flags)"),
    # empty residual: the fallback race on p_n removed (nothing is drawn)
    "fallback_removed": ("if (residual && any_positive) {", "if (residual) {"),
    # empty residual detected with >=, so an all-zero residual counts as non-empty
    "residual_empty_test": ("if (p - q > 0.0) any_positive = 1;", "if (p - q >= 0.0) any_positive = 1;"),
    # empty residual: fallback races every token with equal weight
    "fallback_unweighted": ("        key = logit(in->target, in->dtype, trow0 + n, V, v) / T - lp[n] - log(e);",
                            "        key = residual ? -log(e) :\n"
                            "            logit(in->target, in->dtype, trow0 + n, V, v) / T - lp[n] - log(e);"),
    # exponential race with the wrong sign on the exponential variate
    "race_sign": ("key = log(w) - log(e);", "key = log(w) + log(e);"),
    # Philox: wrong multiplier in the first lane
    "philox_multiplier": ("uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;",
                          "uint64_t p0 = (uint64_t)M1 * (uint64_t)c0;"),
    # Philox: wrong key increment
    "philox_key_schedule": ("k1 += W1;", "k1 += W0;"),
    # draft sampler: exponential variate added instead of subtracted
    "draft_race_sign": ("/ T - lse - log(oracle_draft_exponential(seed, b, step, v));",
                        "/ T - lse + log(oracle_draft_exponential(seed, b, step, v));"),
    # draft sampler: key left unnormalised (z / T - ln E)
    "draft_key_unshifted": ("/ T - lse - log(oracle_draft_exponential(seed, b, step, v));",
                            "/ T - log(oracle_draft_exponential(seed, b, step, v));"),
    # draft sampler: the draft step left out of the counter
    "draft_step_ignored": ("(uint32_t)v >> 2, (uint32_t)step, (uint32_t)b, 2u",
                           "(uint32_t)v >> 2, 0u, (uint32_t)b, 2u"),
    # draft sampler: the verify race's stream tag reused
    "draft_stream_tag": ("(uint32_t)v >> 2, (uint32_t)step, (uint32_t)b, 2u",
                         "(uint32_t)v >> 2, (uint32_t)step, (uint32_t)b, 0u"),
    # draft sampler: temperature ignored in the race key
    "draft_untempered": ("logit(logits, dtype, b, V, v) / T - lse - log(",
                         "logit(logits, dtype, b, V, v) - lse - log("),
    # commit: the emitted token left out (only the accepted drafts appended)
    "commit_drops_emitted": ("for (int32_t i = 0; i <= n; ++i)\n      seq_tokens",
                             "for (int32_t i = 0; i < n; ++i)\n      seq_tokens"),
    # commit: the request's block read at the draft offset (missing + b)
    "commit_block_base": ("out_tokens[(int64_t)off + b + i]", "out_tokens[(int64_t)off + i]"),
    # commit: a history exactly at capacity rejected
    "commit_capacity": ("(int64_t)L + n + 1 > capacity", "(int64_t)L + n + 1 >= capacity"),
    # tree: a node's token compared with its own row instead of its parent's
    "tree_own_row": ("acc[i] = acc[par] && tokens[off + i] == g[par];",
                     "acc[i] = acc[par] && tokens[off + i] == g[i];"),
    # tree: a match under a rejected parent accepted
    "tree_parent_ignored": ("acc[i] = acc[par] && tokens[off + i] == g[par];",
                            "acc[i] = tokens[off + i] == g[par];"),
    # tree: equally deep accepted nodes resolved to the highest index
    "tree_last_tie": ("if (acc[i] && depth[i] > depth[c]) c = i;",
                      "if (acc[i] && depth[i] >= depth[c]) c = i;"),
    # tree: depth taken as the node index (right for chains only)
    "tree_depth_index": ("depth[i] = depth[par] + 1;", "depth[i] = i;"),
    # tree: the extra token taken from the parent of the chosen node
    "tree_bonus_row": ("(j == d ? g[c] : -1)", "(j == d ? g[path[d > 0 ? d - 1 : 0]] : -1)"),
    # uniform map that can return 0
    "u01_map": ("return (2.0 * (double)(x >> 9) + 1.0) / 16777216.0;",
                "return (double)(x >> 8) / 16777216.0;"),
}

# cheap pins first; the first failing pin ends a case
ORDER = [P.pin_philox_kat, P.pin_u01, P.pin_softmax_vs_scipy, P.pin_greedy_vs_numpy,
         P.pin_temperature_invariance, P.pin_identical_draft_accepts,
         P.pin_disjoint_draft_rejects, P.pin_faults, P.pin_accept_near_tie_flag,
         P.pin_bonus_race_near_tie_flag, P.pin_residual_race_near_tie_flag,
         P.pin_residual_empty_fallback, P.pin_plain_sampling,
         P.pin_exact_enumeration, P.pin_closed_form, P.pin_draft_greedy, P.pin_draft_faults,
         P.pin_draft_distribution, P.pin_draft_streams, P.pin_draft_race_near_tie_flag,
         P.pin_commit_example,
         P.pin_commit_after_verify, P.pin_tree_page_example, P.pin_tree_faults,
         P.pin_tree_chain_is_linear, P.pin_tree_brute_force]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new)
    d = tempfile.mkdtemp(prefix=f"mutant_{name}_")
    c_path = os.path.join(d, "mutant.c")
    so_path = os.path.join(d, "mutant.so")
    with open(c_path, "w") as f:
        f.write(src)
    oracle.build(force=True, out=so_path, src=c_path, extra_flags=("-w",))
    lib = oracle.load(so_path)
    caught = None
    for pin in ORDER:
        try:
            pin(lib)
        except Exception:  # an assertion, or a pin that cannot even digest the output
            caught = pin.__name__
            break
    assert caught is not None, f"no pin catches the planted mistake {name}"
    print(f"{name}: caught by {caught}")
