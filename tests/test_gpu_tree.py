"""GPU parity of greedy draft-tree verification (spec_verify_tree_greedy) against
the oracle: accept lengths, emitted tokens and accepted node indices bit-exact.

Cases: the page's tree example (golden fixture), the seeded tree workloads in
full, random trees of up to 64 nodes (chains reaching depth 63, stars, equal
sibling tokens, planted ties) over vocabularies that exercise the vector and
scalar load paths and ragged row tails, per-request faults, workspace reuse,
and a chain tree against the linear greedy verify on the GPU.
"""
import numpy as np
import pytest

import oracle
from oracle_pins import read_tree_cases
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


def upload_logits(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_tree(target, offsets, parents, tokens, max_nodes, workspace=None, want_nodes=True):
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    acc, out, nodes = binding.spec_verify_tree_greedy(
        upload_logits(target), t(offsets), t(parents), t(tokens), max_nodes,
        want_nodes=want_nodes, workspace=workspace)
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(),
                accept_nodes=None if nodes is None else nodes.cpu().numpy())


def check(got, want, offsets, checked_nodes=True):
    """Exact equality on every request whose slice is valid (the others only get
    accept_len = -1 and no writes)."""
    assert (got["accept_len"] == want["accept_len"]).all(), \
        np.nonzero(got["accept_len"] != want["accept_len"])
    for b in range(len(offsets) - 1):
        if want["accept_len"][b] == -1 and not (want["out_tokens"][offsets[b]:offsets[b + 1]]
                                                == -1).all():
            continue  # bad slice: nothing written on either side
        o, o1 = int(offsets[b]), int(offsets[b + 1])
        assert (got["out_tokens"][o:o1] == want["out_tokens"][o:o1]).all(), b
        if checked_nodes:
            assert (got["accept_nodes"][o:o1] == want["accept_nodes"][o:o1]).all(), b


def pack_trees(trees):
    offs = np.zeros(len(trees) + 1, np.int32)
    offs[1:] = np.cumsum([len(p) for p, _ in trees])
    parents = np.concatenate([np.asarray(p, np.int32) for p, _ in trees])
    tokens = np.concatenate([np.asarray(t, np.int32) for _, t in trees])
    return offs, parents, tokens


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16])
def test_tree_page_example(dtype):
    """The tree-attention section's tree: every hand-checked case, both dtypes."""
    say("tree page example", W.DTYPE_NAMES[dtype])
    V = 10
    cases = read_tree_cases()
    trees, rows = [], []
    for c in cases:
        N = len(c["parents"])
        r = np.full((N, V), -1.0, np.float32)
        for i, spec in enumerate(c["argmax"]):
            g = int(spec.rstrip("t"))
            r[i, g] = 2.0
            if spec.endswith("t"):
                r[i, g + 1] = 2.0
        rows.append(r)
        trees.append((c["parents"], c["tokens"]))
    offs, parents, tokens = pack_trees(trees)
    target = W.to_storage(np.concatenate(rows), dtype)
    got = run_tree(target, offs, parents, tokens, 7)
    for b, c in enumerate(cases):
        o, o1 = offs[b], offs[b + 1]
        assert got["accept_len"][b] == c["accept"], c["name"]
        assert got["out_tokens"][o:o1].tolist() == c["out"], c["name"]
        assert got["accept_nodes"][o:o1].tolist() == c["nodes"], c["name"]


@pytest.mark.parametrize("name", ["tree-small", "tree-eagle", "tree-ragged"])
def test_tree_workloads(name):
    say("tree workload", name)
    tb = W.make_tree_batch(name)
    want = oracle.tree_verify(tb.dtype, tb.target, tb.offsets, tb.parents, tb.tokens, tb.V,
                              tb.max_nodes)
    got = run_tree(tb.target, tb.offsets, tb.parents, tb.tokens, tb.max_nodes)
    check(got, want, tb.offsets)
    assert (want["accept_len"] >= 2).any()


def random_trees(rng, B, V, max_nodes, kinds, min_nodes=1):
    """Random trees with rows whose argmax is planted on a child's token often
    enough that deep paths occur; some siblings share tokens, some rows tie."""
    trees, rows = [], []
    for b in range(B):
        kind = kinds[b % len(kinds)]
        N = int(rng.integers(min_nodes, max_nodes + 1)) if kind != "full" else max_nodes
        if kind == "chain":
            par = [-1] + list(range(N - 1))
        elif kind == "star":
            par = [-1] + [0] * (N - 1)
        else:
            par = [-1] + [int(rng.integers(max(0, i - 4), i)) for i in range(1, N)]
        z = rng.normal(0, 2, size=(N, V))
        tok = [-1] * N
        for i in range(1, N):
            tok[i] = int(rng.integers(0, V))
        # plant: each parent's argmax on one of its children's tokens (97%),
        # sometimes tied with the next token (x still wins) or the previous
        # one (x loses)
        for u in range(N):
            kids = [i for i in range(1, N) if par[i] == u]
            if kids and rng.random() < 0.97:
                x = tok[kids[int(rng.integers(0, len(kids)))]]
                z[u, x] = z[u].max() + 1.0
                r = rng.random()
                if r < 0.15 and x + 1 < V:
                    z[u, x + 1] = z[u, x]
                elif r < 0.18 and x > 0:
                    z[u, x - 1] = z[u, x]
            if kids and len(kids) > 1 and rng.random() < 0.2:  # equal sibling tokens
                tok[kids[1]] = tok[kids[0]]
        trees.append((par, tok))
        rows.append(z)
    return trees, np.concatenate(rows)


@pytest.mark.parametrize("V,dtype", [(1, W.DTYPE_F32), (37, W.DTYPE_BF16), (4099, W.DTYPE_F32),
                                     (4099, W.DTYPE_BF16), (70000, W.DTYPE_BF16),
                                     (70000, W.DTYPE_F32), (262144, W.DTYPE_F32),
                                     (300007, W.DTYPE_BF16)])
def test_tree_random_shapes(V, dtype):
    say("tree random shapes", V, W.DTYPE_NAMES[dtype])
    rng = np.random.default_rng(V * 7 + dtype)
    B = 24 if V < 50000 else (12 if V < 200000 else 4)
    trees, z = random_trees(rng, B, V, 64, ["chain", "star", "random", "full"])
    offs, parents, tokens = pack_trees(trees)
    target = W.to_storage(z, dtype)
    want = oracle.tree_verify(dtype, target, offs, parents, tokens, V, 64)
    got = run_tree(target, offs, parents, tokens, 64)
    check(got, want, offs)
    if V > 1:
        assert want["accept_len"].max() >= 8  # chains reach deep


def test_tree_faults():
    """Bad parents, bad tokens, non-finite rows and bad slices fail only their own
    request."""
    say("tree faults")
    V = 300
    rng = np.random.default_rng(5)
    trees, z = random_trees(rng, 10, V, 12, ["chain", "random"], min_nodes=3)
    offs, parents, tokens = pack_trees(trees)
    z = z.astype(np.float32)
    # request 1: parent equal to the node; request 2: token outside V;
    # request 3: NaN row; request 4: all -inf row; request 6: negative parent
    def node(b, i):
        return int(offs[b]) + i
    for b in (1, 2, 3, 4, 6):
        assert offs[b + 1] - offs[b] >= 3, "fault requests need 3 nodes"
    parents[node(1, 2)] = 2
    tokens[node(2, 1)] = V
    z[node(3, 1)] = np.nan
    z[node(4, 2)] = -np.inf
    parents[node(6, 1)] = -3
    for dtype in (W.DTYPE_F32, W.DTYPE_BF16):
        target = W.to_storage(z, dtype)
        want = oracle.tree_verify(dtype, target, offs, parents, tokens, V, 12)
        got = run_tree(target, offs, parents, tokens, 12)
        check(got, want, offs)
        assert [int(want["accept_len"][b]) for b in (1, 2, 3, 4, 6)] == [-1] * 5
        assert (want["accept_len"][[0, 5, 7, 8, 9]] >= 0).all()
    # bad slices: an empty request and one larger than max_nodes
    offs2 = offs.copy()
    offs2[4] = offs2[3]  # request 3 empty, request 4 grows
    target = W.to_storage(z, W.DTYPE_F32)
    want = oracle.tree_verify(W.DTYPE_F32, target, offs2, parents, tokens, V, 12)
    got = run_tree(target, offs2, parents, tokens, 12)
    assert got["accept_len"][3] == -1 and want["accept_len"][3] == -1
    check(got, want, offs2)


def test_tree_without_node_output():
    say("tree without accept_nodes")
    tb = W.make_tree_batch("tree-small")
    want = oracle.tree_verify(tb.dtype, tb.target, tb.offsets, tb.parents, tb.tokens, tb.V,
                              tb.max_nodes)
    got = run_tree(tb.target, tb.offsets, tb.parents, tb.tokens, tb.max_nodes, want_nodes=False)
    assert got["accept_nodes"] is None
    check(got, want, tb.offsets, checked_nodes=False)


def test_tree_workspace_reuse():
    """One workspace across calls of different sizes; all-zero after each call."""
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    say("tree workspace reuse")
    ws = torch.zeros(binding.tree_workspace_bytes(40, 70000, 64), dtype=torch.uint8,
                     device="cuda")
    rng = np.random.default_rng(11)
    for B, V, mn, dtype in ((40, 70000, 64, W.DTYPE_BF16), (7, 5000, 20, W.DTYPE_F32),
                            (40, 70000, 64, W.DTYPE_F32), (3, 129, 5, W.DTYPE_BF16)):
        trees, z = random_trees(rng, B, V, mn, ["random", "chain"])
        offs, parents, tokens = pack_trees(trees)
        target = W.to_storage(z, dtype)
        want = oracle.tree_verify(dtype, target, offs, parents, tokens, V, mn)
        got = run_tree(target, offs, parents, tokens, mn, workspace=ws)
        check(got, want, offs)
        assert int(ws.count_nonzero()) == 0


def test_tree_chain_matches_linear_greedy():
    """A chain tree on the GPU gives the GPU linear greedy verify's outputs."""
    import torch
    from rejection_sampling_verify_scaled_amd import binding
    say("tree chain vs linear greedy")
    b = W.make_batch(2, 0, temperature_override=0.0)
    ks = np.diff(b.offsets)
    trees = [([-1] + list(range(int(k))), [-1] + b.tokens[b.offsets[i]:b.offsets[i + 1]].tolist())
             for i, k in enumerate(ks)]
    offs, parents, tokens = pack_trees(trees)
    got = run_tree(b.target, offs, parents, tokens, int(ks.max()) + 1)
    d = binding.to_device_batch(b)
    acc, out = binding.spec_verify_greedy(d["target"], d["offsets"], d["tokens"], b.max_k)
    torch.cuda.synchronize()
    assert (got["accept_len"] == acc.cpu().numpy()).all()
    assert (got["out_tokens"] == out.cpu().numpy()).all()
