"""ctypes binding of libspecverify.so (the C ABI in include/spec_verify.h).

Argument marshalling only: tensors are checked against the shapes the kernels
and their grids assume, then their device pointers go to the C entry points,
which enqueue the HIP kernels on torch's current stream.  There is no
fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "spec_verify.h")

SV_F32 = 0
SV_BF16 = 1
SV_KMAX = 8
SV_TREE_MAX_NODES = 64
SV_STATIC_SCRATCH_BYTES = 16 << 20
STATUS = {0: "SV_OK", -1: "SV_ERR_NULL", -2: "SV_ERR_SHAPE", -3: "SV_ERR_DTYPE",
          -4: "SV_ERR_WORKSPACE", -5: "SV_ERR_LAUNCH", -6: "SV_ERR_SCRATCH"}


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, '?')}): {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library and declare its entry points (raises if absent)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m rejection_sampling_verify_scaled_amd.build`"
            " (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    i32, vp, sz, u64 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64
    lib.spec_verify_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify_greedy.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_greedy.restype = ctypes.c_int
    lib.spec_verify_sample.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, u64, vp, vp,
                                       vp, vp, vp, sz, vp]
    lib.spec_verify_sample.restype = ctypes.c_int
    lib.spec_verify_sample_static.argtypes = list(lib.spec_verify_sample.argtypes[:15]) + [i32, vp]
    lib.spec_verify_sample_static.restype = ctypes.c_int
    lib.spec_verify_sample_timed.argtypes = list(lib.spec_verify_sample.argtypes) + [vp, vp]
    lib.spec_verify_sample_timed.restype = ctypes.c_int
    lib.spec_verify_early_exit_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_verify_early_exit_workspace_bytes.restype = sz
    lib.spec_verify_sample_early_exit.argtypes = list(lib.spec_verify_sample.argtypes)
    lib.spec_verify_sample_early_exit.restype = ctypes.c_int
    lib.spec_draft_workspace_bytes.argtypes = [i32, i32]
    lib.spec_draft_workspace_bytes.restype = sz
    lib.spec_draft_sample.argtypes = [vp, i32, i32, i32, vp, u64, i32, vp, vp, vp, sz, vp]
    lib.spec_draft_sample.restype = ctypes.c_int
    lib.spec_commit_tokens.argtypes = [i32, i32, i32, vp, vp, vp, vp, ctypes.c_int64, vp, i32, vp,
                                       vp, vp]
    lib.spec_commit_tokens.restype = ctypes.c_int
    lib.spec_verify_tree_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_verify_tree_workspace_bytes.restype = sz
    lib.spec_verify_tree_greedy.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]
    lib.spec_verify_tree_greedy.restype = ctypes.c_int
    lib.spec_verify_status_string.argtypes = [ctypes.c_int]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def header_functions(header: str = HEADER):
    """Names of the functions include/spec_verify.h declares."""
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_(?:verify|draft|commit)_\w+)\s*\(", text)))


def workspace_bytes(B: int, V: int, max_k: int) -> int:
    return int(load_library().spec_verify_workspace_bytes(B, V, max_k))


def new_workspace(B: int, V: int, max_k: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for calls up to these sizes."""
    return torch.zeros(workspace_bytes(B, V, max_k), dtype=torch.uint8, device=device)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _check(t: torch.Tensor, name: str, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream_handle(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _prepare(target, offsets, tokens, max_k, accept_len, out_tokens, workspace):
    if target.dim() != 2:
        raise ValueError("target_logits must be 2-D [rows, V]")
    device = target.device
    if device.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    B = offsets.shape[0] - 1
    if B < 1:
        raise ValueError("need at least one request (offsets has B+1 entries)")
    V = target.shape[1]
    n_d = tokens.shape[0]
    _check(offsets, "draft_offsets", torch.int32, (B + 1,), device)
    _check(tokens, "draft_tokens", torch.int32, (n_d,), device)
    _check(target, "target_logits", target.dtype, (n_d + B, V), device)
    if not 0 <= max_k <= SV_KMAX:
        raise ValueError(f"max_k must be in [0, {SV_KMAX}]")
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=device)
    if out_tokens is None:
        out_tokens = torch.empty(n_d + B, dtype=torch.int32, device=device)
    _check(accept_len, "accept_len", torch.int32, (B,), device)
    _check(out_tokens, "out_tokens", torch.int32, (n_d + B,), device)
    need = workspace_bytes(B, V, max_k)
    if workspace is None:  # zero-filled once; every completed call leaves it zeroed
        workspace = torch.zeros(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    return B, V, n_d, accept_len, out_tokens, workspace


def spec_verify_greedy(target_logits: torch.Tensor, draft_offsets: torch.Tensor,
                       draft_tokens: torch.Tensor, max_k: int,
                       accept_len: Optional[torch.Tensor] = None,
                       out_tokens: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None, lib=None):
    """All-greedy verify; returns (accept_len [B], out_tokens [n_draft + B])."""
    lib = lib or load_library()
    B, V, n_d, accept_len, out_tokens, workspace = _prepare(
        target_logits, draft_offsets, draft_tokens, max_k, accept_len, out_tokens, workspace)
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    rc = lib.spec_verify_greedy(
        _ptr(target_logits), _dtype_code(target_logits), B, V, max_k, n_d, _ptr(draft_offsets),
        _ptr(draft_tokens), _ptr(accept_len), _ptr(out_tokens), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if rc != 0:
        raise SpecVerifyError("spec_verify_greedy", rc, lib.spec_verify_status_string(rc).decode())
    return accept_len, out_tokens


def spec_verify_sample(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                       draft_offsets: torch.Tensor, draft_tokens: torch.Tensor,
                       temperature: torch.Tensor, seed: int, max_k: int,
                       accept_len: Optional[torch.Tensor] = None,
                       out_tokens: Optional[torch.Tensor] = None,
                       p_at_draft: Optional[torch.Tensor] = None,
                       q_at_draft: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None, lib=None):
    """Mixed sampled / greedy verify; returns (accept_len, out_tokens, p_at, q_at)."""
    lib = lib or load_library()
    B, V, n_d, accept_len, out_tokens, workspace = _prepare(
        target_logits, draft_offsets, draft_tokens, max_k, accept_len, out_tokens, workspace)
    device = target_logits.device
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    _check(draft_logits, "draft_logits", target_logits.dtype, (n_d, V), device)
    _check(temperature, "temperature", torch.float32, (B,), device)
    for name, t in (("p_at_draft", p_at_draft), ("q_at_draft", q_at_draft)):
        if t is not None:
            _check(t, name, torch.float32, (n_d,), device)
    rc = lib.spec_verify_sample(
        _ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits), B, V, max_k, n_d,
        _ptr(draft_offsets), _ptr(draft_tokens), _ptr(temperature),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), _ptr(accept_len), _ptr(out_tokens),
        _ptr(p_at_draft), _ptr(q_at_draft), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if rc != 0:
        raise SpecVerifyError("spec_verify_sample", rc, lib.spec_verify_status_string(rc).decode())
    return accept_len, out_tokens, p_at_draft, q_at_draft


def spec_verify_sample_static(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                              draft_offsets: torch.Tensor, draft_tokens: torch.Tensor,
                              temperature: torch.Tensor, seed: int, max_k: int,
                              accept_len: torch.Tensor, out_tokens: torch.Tensor,
                              p_at_draft: Optional[torch.Tensor] = None,
                              q_at_draft: Optional[torch.Tensor] = None,
                              clear_scratch: bool = False, stream=None, lib=None):
    """spec_verify_sample on the library's fixed device array instead of a
    workspace: allocates nothing, so every output is passed in.  Returns
    (accept_len, out_tokens, p_at, q_at)."""
    lib = lib or load_library()
    if target_logits.dim() != 2 or target_logits.device.type != "cuda":
        raise ValueError("target_logits must be a 2-D tensor on a HIP device")
    device = target_logits.device
    B = draft_offsets.shape[0] - 1
    V = target_logits.shape[1]
    n_d = draft_tokens.shape[0]
    if B < 1:
        raise ValueError("need at least one request (offsets has B+1 entries)")
    if not 0 <= max_k <= SV_KMAX:
        raise ValueError(f"max_k must be in [0, {SV_KMAX}]")
    _check(draft_offsets, "draft_offsets", torch.int32, (B + 1,), device)
    _check(draft_tokens, "draft_tokens", torch.int32, (n_d,), device)
    _check(target_logits, "target_logits", target_logits.dtype, (n_d + B, V), device)
    _check(draft_logits, "draft_logits", target_logits.dtype, (n_d, V), device)
    _check(temperature, "temperature", torch.float32, (B,), device)
    _check(accept_len, "accept_len", torch.int32, (B,), device)
    _check(out_tokens, "out_tokens", torch.int32, (n_d + B,), device)
    for name, t in (("p_at_draft", p_at_draft), ("q_at_draft", q_at_draft)):
        if t is not None:
            _check(t, name, torch.float32, (n_d,), device)
    rc = lib.spec_verify_sample_static(
        _ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits), B, V, max_k, n_d,
        _ptr(draft_offsets), _ptr(draft_tokens), _ptr(temperature),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), _ptr(accept_len), _ptr(out_tokens),
        _ptr(p_at_draft), _ptr(q_at_draft), 1 if clear_scratch else 0, _stream_handle(stream))
    if rc != 0:
        raise SpecVerifyError("spec_verify_sample_static", rc,
                              lib.spec_verify_status_string(rc).decode())
    return accept_len, out_tokens, p_at_draft, q_at_draft


def early_exit_workspace_bytes(B: int, V: int, max_k: int) -> int:
    return int(load_library().spec_verify_early_exit_workspace_bytes(B, V, max_k))


def spec_verify_sample_early_exit(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                                  draft_offsets: torch.Tensor, draft_tokens: torch.Tensor,
                                  temperature: torch.Tensor, seed: int, max_k: int,
                                  accept_len: Optional[torch.Tensor] = None,
                                  out_tokens: Optional[torch.Tensor] = None,
                                  p_at_draft: Optional[torch.Tensor] = None,
                                  q_at_draft: Optional[torch.Tensor] = None,
                                  workspace: Optional[torch.Tensor] = None, stream=None, lib=None):
    """Early-exit verify (rows past each request's stop are not read); returns
    (accept_len, out_tokens, p_at, q_at) like spec_verify_sample, with p/q NaN
    past the stop."""
    lib = lib or load_library()
    B = draft_offsets.shape[0] - 1
    V = target_logits.shape[1]
    n_d = draft_tokens.shape[0]
    device = target_logits.device
    if workspace is None:
        workspace = torch.zeros(early_exit_workspace_bytes(B, V, max_k), dtype=torch.uint8,
                                device=device)
    B, V, n_d, accept_len, out_tokens, _ = _prepare(
        target_logits, draft_offsets, draft_tokens, max_k, accept_len, out_tokens, workspace)
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    _check(draft_logits, "draft_logits", target_logits.dtype, (n_d, V), device)
    _check(temperature, "temperature", torch.float32, (B,), device)
    for name, t in (("p_at_draft", p_at_draft), ("q_at_draft", q_at_draft)):
        if t is not None:
            _check(t, name, torch.float32, (n_d,), device)
    rc = lib.spec_verify_sample_early_exit(
        _ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits), B, V, max_k, n_d,
        _ptr(draft_offsets), _ptr(draft_tokens), _ptr(temperature),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), _ptr(accept_len), _ptr(out_tokens),
        _ptr(p_at_draft), _ptr(q_at_draft), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if rc != 0:
        raise SpecVerifyError("spec_verify_sample_early_exit", rc,
                              lib.spec_verify_status_string(rc).decode())
    return accept_len, out_tokens, p_at_draft, q_at_draft


def draft_workspace_bytes(B: int, V: int) -> int:
    return int(load_library().spec_draft_workspace_bytes(B, V))


def spec_draft_sample(draft_logits: torch.Tensor, temperature: torch.Tensor, seed: int,
                      step: int, tokens: Optional[torch.Tensor] = None,
                      q_at: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      want_q: bool = True, lib=None):
    """Draft-side sampler over rows [B, V]; returns (tokens [B] int32, q_at [B] or None)."""
    lib = lib or load_library()
    if draft_logits.dim() != 2 or not draft_logits.is_contiguous():
        raise ValueError("draft_logits must be a contiguous [B, V] tensor")
    B, V = draft_logits.shape
    device = draft_logits.device
    _check(temperature, "temperature", torch.float32, (B,), device)
    if tokens is None:
        tokens = torch.empty(B, dtype=torch.int32, device=device)
    _check(tokens, "tokens", torch.int32, (B,), device)
    if q_at is None and want_q:
        q_at = torch.empty(B, dtype=torch.float32, device=device)
    if q_at is not None:
        _check(q_at, "q_at", torch.float32, (B,), device)
    if workspace is None:
        workspace = torch.zeros(draft_workspace_bytes(B, V), dtype=torch.uint8, device=device)
    rc = lib.spec_draft_sample(
        _ptr(draft_logits), _dtype_code(draft_logits), B, V, _ptr(temperature),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), int(step), _ptr(tokens), _ptr(q_at),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if rc != 0:
        raise SpecVerifyError("spec_draft_sample", rc, lib.spec_verify_status_string(rc).decode())
    return tokens, q_at


def spec_commit_tokens(draft_offsets: torch.Tensor, accept_len: torch.Tensor,
                       out_tokens: torch.Tensor, seq_tokens: torch.Tensor,
                       seq_len: torch.Tensor, max_k: int, capacity: Optional[int] = None,
                       next_tokens: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None, stream=None, lib=None):
    """Append the verify step's emitted tokens to the histories seq_tokens [B, S]
    (in place) and advance seq_len [B]; returns (next_tokens [B], status [B])."""
    lib = lib or load_library()
    B = accept_len.shape[0]
    device = accept_len.device
    _check(draft_offsets, "draft_offsets", torch.int32, (B + 1,), device)
    _check(accept_len, "accept_len", torch.int32, (B,), device)
    if seq_tokens.dim() != 2 or seq_tokens.shape[0] != B or seq_tokens.dtype != torch.int32 \
            or seq_tokens.stride(1) != 1:
        raise ValueError("seq_tokens must be an int32 [B, S] tensor with unit column stride")
    _check(seq_len, "seq_len", torch.int32, (B,), device)
    n_d = out_tokens.shape[0] - B
    _check(out_tokens, "out_tokens", torch.int32, (n_d + B,), device)
    if next_tokens is None:
        next_tokens = torch.empty(B, dtype=torch.int32, device=device)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=device)
    cap = seq_tokens.shape[1] if capacity is None else int(capacity)
    rc = lib.spec_commit_tokens(B, max_k, n_d, _ptr(draft_offsets), _ptr(accept_len),
                                _ptr(out_tokens), _ptr(seq_tokens), seq_tokens.stride(0),
                                _ptr(seq_len), cap, _ptr(next_tokens), _ptr(status),
                                _stream_handle(stream))
    if rc != 0:
        raise SpecVerifyError("spec_commit_tokens", rc, lib.spec_verify_status_string(rc).decode())
    return next_tokens, status


def tree_workspace_bytes(B: int, V: int, max_nodes: int) -> int:
    return int(load_library().spec_verify_tree_workspace_bytes(B, V, max_nodes))


def spec_verify_tree_greedy(target_logits: torch.Tensor, node_offsets: torch.Tensor,
                            parents: torch.Tensor, tokens: torch.Tensor, max_nodes: int,
                            accept_len: Optional[torch.Tensor] = None,
                            out_tokens: Optional[torch.Tensor] = None,
                            accept_nodes: Optional[torch.Tensor] = None,
                            want_nodes: bool = True,
                            workspace: Optional[torch.Tensor] = None, stream=None, lib=None):
    """Greedy draft-tree verify; returns (accept_len [B], out_tokens [n_rows],
    accept_nodes [n_rows] or None)."""
    lib = lib or load_library()
    if target_logits.dim() != 2:
        raise ValueError("target_logits must be 2-D [rows, V]")
    device = target_logits.device
    if device.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    B = node_offsets.shape[0] - 1
    if B < 1:
        raise ValueError("need at least one request (node_offsets has B+1 entries)")
    n, V = target_logits.shape
    _check(target_logits, "target_logits", target_logits.dtype, (n, V), device)
    _check(node_offsets, "node_offsets", torch.int32, (B + 1,), device)
    _check(parents, "parents", torch.int32, (n,), device)
    _check(tokens, "tokens", torch.int32, (n,), device)
    if not 1 <= max_nodes <= SV_TREE_MAX_NODES:
        raise ValueError(f"max_nodes must be in [1, {SV_TREE_MAX_NODES}]")
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=device)
    if out_tokens is None:
        out_tokens = torch.empty(max(n, 1), dtype=torch.int32, device=device)[:n]
    if accept_nodes is None and want_nodes:
        accept_nodes = torch.empty(max(n, 1), dtype=torch.int32, device=device)[:n]
    _check(accept_len, "accept_len", torch.int32, (B,), device)
    _check(out_tokens, "out_tokens", torch.int32, (n,), device)
    if accept_nodes is not None:
        _check(accept_nodes, "accept_nodes", torch.int32, (n,), device)
    need = tree_workspace_bytes(B, V, max_nodes)
    if workspace is None:  # zero-filled once; every completed call leaves it zeroed
        workspace = torch.zeros(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    rc = lib.spec_verify_tree_greedy(
        _ptr(target_logits), _dtype_code(target_logits), B, V, max_nodes, n, _ptr(node_offsets),
        _ptr(parents), _ptr(tokens), _ptr(accept_len), _ptr(out_tokens), _ptr(accept_nodes),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if rc != 0:
        raise SpecVerifyError("spec_verify_tree_greedy", rc,
                              lib.spec_verify_status_string(rc).decode())
    return accept_len, out_tokens, accept_nodes


def to_device_tree_batch(tb, device="cuda"):
    """Upload a workloads.TreeBatch to the device."""
    import numpy as np
    if tb.target.dtype == np.uint16:
        target = torch.from_numpy(tb.target.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        target = torch.from_numpy(np.ascontiguousarray(tb.target, dtype=np.float32)).to(device)
    return dict(target=target.reshape(-1, tb.V),
                offsets=torch.from_numpy(tb.offsets).to(device),
                parents=torch.from_numpy(tb.parents).to(device),
                tokens=torch.from_numpy(tb.tokens).to(device))


def to_device_batch(batch, device="cuda"):
    """Upload a workloads.Batch to the device (bf16 bits reinterpreted as bfloat16)."""
    import numpy as np

    def logits(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    V = batch.V
    target = logits(batch.target)
    draft = logits(batch.draft) if batch.draft.shape[0] else logits(batch.draft.reshape(0, V))
    return dict(
        target=target.reshape(-1, V), draft=draft.reshape(-1, V),
        offsets=torch.from_numpy(batch.offsets).to(device),
        tokens=torch.from_numpy(batch.tokens).to(device),
        temperature=torch.from_numpy(batch.temperature).to(device))
