"""C ABI checks that need no GPU: the library loads, exports what the header
declares, sizes workspaces, and rejects bad arguments before any HIP call."""
import ctypes
import os

import pytest

from rejection_sampling_verify_scaled_amd import binding


@pytest.fixture(scope="module")
def lib():
    # SPECVERIFY_HOST_TEST_LIB: another build of the same sources (the sanitizer
    # test points it at a host-side AddressSanitizer build)
    path = os.environ.get("SPECVERIFY_HOST_TEST_LIB")
    return binding.load_library(path) if path else binding.load_library()


def test_exports_every_declared_function(lib):
    names = binding.header_functions()
    assert {"spec_verify_greedy", "spec_verify_sample", "spec_verify_workspace_bytes",
            "spec_verify_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/spec_verify.h but not exported"


def test_every_declared_function_has_a_signature(lib):
    """The binding declares argument and result types for every entry point the
    header declares (ctypes would otherwise pass 64-bit sizes and pointers as int)."""
    for n in binding.header_functions():
        f = getattr(lib, n)
        assert f.argtypes is not None, f"{n} has no argtypes in the binding"
        assert f.restype is not None, f"{n} has no restype in the binding"


def test_workspace_bytes(lib):
    assert lib.spec_verify_workspace_bytes(64, 128256, 4) > 0
    assert lib.spec_verify_workspace_bytes(64, 128256, 4) % 256 == 0
    assert lib.spec_verify_workspace_bytes(1024, 152064, 8) >= \
        lib.spec_verify_workspace_bytes(64, 152064, 8)
    for bad in ((0, 10, 1), (1, 0, 1), (1, 10, -1), (1, 10, 9)):
        assert lib.spec_verify_workspace_bytes(*bad) == 0


def _fake(n):  # host addresses are fine: these calls must fail before touching them
    buf = (ctypes.c_char * n)()
    return ctypes.cast(buf, ctypes.c_void_p), buf


@pytest.mark.parametrize("case", ["null_target", "null_offsets", "null_out", "null_ws",
                                  "null_draft", "null_temp", "B0", "V0", "maxk9", "maxk_neg",
                                  "ndraft_neg", "dtype", "ws_small", "ws_misaligned"])
def test_sample_rejects_bad_arguments(lib, case):
    B, V, max_k, nd = 4, 64, 2, 8
    keep = []
    def p(n=4096):
        ptr, buf = _fake(n + 64)
        keep.append(buf)
        return ctypes.c_void_p((ptr.value + 15) // 16 * 16)
    ws_n = lib.spec_verify_workspace_bytes(B, V, max_k)
    args = dict(target=p(), draft=p(), dtype=1, B=B, V=V, max_k=max_k, nd=nd, offs=p(),
                toks=p(), temp=p(), seed=1, acc=p(), out=p(), pa=None, qa=None,
                ws=p(ws_n), ws_n=ws_n)
    expect = {"null_target": -1, "null_offsets": -1, "null_out": -1, "null_ws": -1,
              "null_draft": -1, "null_temp": -1, "B0": -2, "V0": -2, "maxk9": -2,
              "maxk_neg": -2, "ndraft_neg": -2, "dtype": -3, "ws_small": -4,
              "ws_misaligned": -4}[case]
    if case == "null_target": args["target"] = None
    if case == "null_offsets": args["offs"] = None
    if case == "null_out": args["out"] = None
    if case == "null_ws": args["ws"] = None
    if case == "null_draft": args["draft"] = None
    if case == "null_temp": args["temp"] = None
    if case == "B0": args["B"] = 0
    if case == "V0": args["V"] = 0
    if case == "maxk9": args["max_k"] = 9
    if case == "maxk_neg": args["max_k"] = -1
    if case == "ndraft_neg": args["nd"] = -1
    if case == "dtype": args["dtype"] = 7
    if case == "ws_small": args["ws_n"] = ws_n - 1
    if case == "ws_misaligned": args["ws"] = ctypes.c_void_p(args["ws"].value + 4)
    a = args
    rc = lib.spec_verify_sample(a["target"], a["draft"], a["dtype"], a["B"], a["V"], a["max_k"],
                                a["nd"], a["offs"], a["toks"], a["temp"], a["seed"], a["acc"],
                                a["out"], a["pa"], a["qa"], a["ws"], a["ws_n"], None)
    assert rc == expect, (case, rc)
    assert lib.spec_verify_status_string(rc)


def test_greedy_rejects_bad_arguments(lib):
    ptr, buf = _fake(1 << 16)
    base = ctypes.c_void_p((ptr.value + 15) // 16 * 16)
    ws = lib.spec_verify_workspace_bytes(2, 32, 1)
    assert lib.spec_verify_greedy(None, 1, 2, 32, 1, 2, base, base, base, base, base, ws,
                                  None) == -1
    assert lib.spec_verify_greedy(base, 1, 2, 32, 11, 2, base, base, base, base, base, ws,
                                  None) == -2
    assert lib.spec_verify_greedy(base, 5, 2, 32, 1, 2, base, base, base, base, base, ws,
                                  None) == -3
    assert lib.spec_verify_greedy(base, 1, 2, 32, 1, 2, base, base, base, base, base, 16,
                                  None) == -4


def test_draft_workspace_bytes(lib):
    assert lib.spec_draft_workspace_bytes(64, 128256) >= 64 * 63 * 16
    assert lib.spec_draft_workspace_bytes(0, 10) == 0
    assert lib.spec_draft_workspace_bytes(1, 0) == 0


@pytest.mark.parametrize("case", ["null_logits", "null_temp", "null_tokens", "null_ws", "B0",
                                  "V0", "step_neg", "dtype", "ws_small", "ws_misaligned"])
def test_draft_rejects_bad_arguments(lib, case):
    B, V = 4, 64
    keep = []
    def p(n=4096):
        ptr, buf = _fake(n + 64)
        keep.append(buf)
        return ctypes.c_void_p((ptr.value + 15) // 16 * 16)
    ws_n = lib.spec_draft_workspace_bytes(B, V)
    a = dict(logits=p(), dtype=1, B=B, V=V, temp=p(), seed=3, step=0, toks=p(), q=None,
             ws=p(ws_n), ws_n=ws_n)
    expect = {"null_logits": -1, "null_temp": -1, "null_tokens": -1, "null_ws": -1, "B0": -2,
              "V0": -2, "step_neg": -2, "dtype": -3, "ws_small": -4, "ws_misaligned": -4}[case]
    if case == "null_logits": a["logits"] = None
    if case == "null_temp": a["temp"] = None
    if case == "null_tokens": a["toks"] = None
    if case == "null_ws": a["ws"] = None
    if case == "B0": a["B"] = 0
    if case == "V0": a["V"] = 0
    if case == "step_neg": a["step"] = -1
    if case == "dtype": a["dtype"] = 7
    if case == "ws_small": a["ws_n"] = ws_n - 1
    if case == "ws_misaligned": a["ws"] = ctypes.c_void_p(a["ws"].value + 4)
    rc = lib.spec_draft_sample(a["logits"], a["dtype"], a["B"], a["V"], a["temp"],
                               ctypes.c_uint64(a["seed"]), a["step"], a["toks"], a["q"],
                               a["ws"], a["ws_n"], None)
    assert rc == expect


@pytest.mark.parametrize("case", ["null_offsets", "null_accept", "null_out", "null_seq",
                                  "null_len", "B0", "maxk_big", "ndraft_neg", "cap_neg",
                                  "stride_small"])
def test_commit_rejects_bad_arguments(lib, case):
    keep = []
    def p(n=4096):
        ptr, buf = _fake(n + 64)
        keep.append(buf)
        return ctypes.c_void_p((ptr.value + 15) // 16 * 16)
    a = dict(B=4, max_k=2, nd=8, offs=p(), acc=p(), out=p(), seq=p(), stride=32, lens=p(),
             cap=32)
    expect = {"null_offsets": -1, "null_accept": -1, "null_out": -1, "null_seq": -1,
              "null_len": -1, "B0": -2, "maxk_big": -2, "ndraft_neg": -2, "cap_neg": -2,
              "stride_small": -2}[case]
    if case == "null_offsets": a["offs"] = None
    if case == "null_accept": a["acc"] = None
    if case == "null_out": a["out"] = None
    if case == "null_seq": a["seq"] = None
    if case == "null_len": a["lens"] = None
    if case == "B0": a["B"] = 0
    if case == "maxk_big": a["max_k"] = 9
    if case == "ndraft_neg": a["nd"] = -1
    if case == "cap_neg": a["cap"] = -1
    if case == "stride_small": a["stride"] = 16
    rc = lib.spec_commit_tokens(a["B"], a["max_k"], a["nd"], a["offs"], a["acc"], a["out"],
                                a["seq"], a["stride"], a["lens"], a["cap"], None, None, None)
    assert rc == expect


def test_tree_workspace_bytes(lib):
    n = lib.spec_verify_tree_workspace_bytes(16, 128256, 41)
    assert n > 0 and n % 256 == 0
    # one partial per block of 8 float32 chunks (2048 tokens each):
    # 16 requests x 41 nodes x ceil(63 / 8) blocks x 8 bytes
    assert n >= 16 * 41 * 8 * 8
    for bad in ((0, 10, 1), (1, 0, 1), (1, 10, 0), (1, 10, binding.SV_TREE_MAX_NODES + 1)):
        assert lib.spec_verify_tree_workspace_bytes(*bad) == 0
    assert binding.SV_TREE_MAX_NODES == 64


@pytest.mark.parametrize("case", ["null_target", "null_offsets", "null_parents", "null_tokens",
                                  "null_accept", "null_out", "null_ws", "B0", "V0", "nodes0",
                                  "nodes_big", "rows_neg", "dtype", "ws_small", "ws_misaligned"])
def test_tree_rejects_bad_arguments(lib, case):
    keep = []

    def p(n=1 << 16):
        ptr, buf = _fake(n + 64)
        keep.append(buf)
        return ctypes.c_void_p((ptr.value + 15) // 16 * 16)
    a = dict(tgt=p(), dtype=binding.SV_BF16, B=2, V=100, nodes=8, rows=12, offs=p(), par=p(),
             tok=p(), acc=p(), out=p(), ws=p())
    a["ws_n"] = lib.spec_verify_tree_workspace_bytes(2, 100, 8)
    expect = {"null_target": -1, "null_offsets": -1, "null_parents": -1, "null_tokens": -1,
              "null_accept": -1, "null_out": -1, "null_ws": -1, "B0": -2, "V0": -2,
              "nodes0": -2, "nodes_big": -2, "rows_neg": -2, "dtype": -3, "ws_small": -4,
              "ws_misaligned": -4}[case]
    key = {"null_target": "tgt", "null_offsets": "offs", "null_parents": "par",
           "null_tokens": "tok", "null_accept": "acc", "null_out": "out", "null_ws": "ws"}
    if case in key: a[key[case]] = None
    if case == "B0": a["B"] = 0
    if case == "V0": a["V"] = 0
    if case == "nodes0": a["nodes"] = 0
    if case == "nodes_big": a["nodes"] = binding.SV_TREE_MAX_NODES + 1
    if case == "rows_neg": a["rows"] = -1
    if case == "dtype": a["dtype"] = 7
    if case == "ws_small": a["ws_n"] -= 8
    if case == "ws_misaligned": a["ws"] = ctypes.c_void_p(a["ws"].value + 4)
    rc = lib.spec_verify_tree_greedy(a["tgt"], a["dtype"], a["B"], a["V"], a["nodes"], a["rows"],
                                     a["offs"], a["par"], a["tok"], a["acc"], a["out"], None,
                                     a["ws"], a["ws_n"], None)
    assert rc == expect


def test_valu_rate_probe_rejects_bad_arguments():
    """The issue-rate probe library (a measurement build) loads and refuses bad
    arguments before any HIP call."""
    from rejection_sampling_verify_scaled_amd import build as hip_build
    if not os.path.exists(hip_build.LIB_RATES):
        pytest.skip("libspecverify_rates.so is not built (build.py --all)")
    rl = ctypes.CDLL(hip_build.LIB_RATES)
    f = rl.sv_valu_rate
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.POINTER(ctypes.c_float),
                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    f.restype = ctypes.c_int
    ms, bodies, mhz = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
    refs = (ctypes.byref(ms), ctypes.byref(bodies), ctypes.byref(mhz))
    assert f(-1, 256, 100.0, *refs) == -1
    assert f(6, 256, 100.0, *refs) == -1
    assert f(0, 0, 100.0, *refs) == -1
    assert f(0, 256, 100.0, None, None, None) == -1
