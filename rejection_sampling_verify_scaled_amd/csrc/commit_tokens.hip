// commit_tokens.hip -- gfx950 kernel and C ABI of the commit step after
// verification.
//
// What is computed is stated in include/spec_verify.h (spec_commit_tokens):
// each request's emitted tokens (its accepted drafts, then the replacement
// or bonus token) are appended to its token history on the device and its
// length advanced, so the serving loop never waits on the host for the
// verify step's outcome (Perplexity's page, section on MTP scheduling: a
// kernel writes the accepted tokens into their places).
//
// One thread per request: it reads the request's slice, accept_len and
// history length, copies the n + 1 emitted tokens, then writes the new
// length.  Only that thread touches the request's length, so there is no
// ordering hazard between readers and the writer.  Latency-bound: a few
// words per request.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "spec_verify.h"

namespace {

constexpr int kCommitThreads = 256;

struct CommitParams {
  int32_t B, max_k, n_draft_rows, capacity;
  int64_t seq_stride;
  const int32_t* offsets;     // [B+1]
  const int32_t* accept_len;  // [B]
  const int32_t* out_tokens;  // [n_draft_rows + B]
  int32_t* seq_tokens;        // [B][seq_stride]
  int32_t* seq_len;           // [B]
  int32_t* next_tokens;       // [B] or NULL
  int32_t* status;            // [B] or NULL
};

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitParams p) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kCommitThreads + threadIdx.x;
  if (b >= p.B) return;
  const int32_t off = p.offsets[b], off1 = p.offsets[b + 1], n = p.accept_len[b];
  const bool slice_ok =
      off >= 0 && off1 >= off && off1 <= p.n_draft_rows && off1 - off <= p.max_k;
  int32_t st, next = -1;
  if (!slice_ok || n < 0 || n > off1 - off) {
    st = -1;
  } else {
    const int32_t L = p.seq_len[b];
    if (L < 0 || static_cast<int64_t>(L) + n + 1 > p.capacity) {
      st = -2;
    } else {
      const int32_t* src = p.out_tokens + static_cast<int64_t>(off) + b;
      int32_t* dst = p.seq_tokens + b * p.seq_stride + L;
      for (int32_t i = 0; i <= n; ++i) dst[i] = src[i];
      next = src[n];
      p.seq_len[b] = L + n + 1;
      st = n + 1;
    }
  }
  if (p.next_tokens) p.next_tokens[b] = next;
  if (p.status) p.status[b] = st;
}

}  // namespace

extern "C" {

int spec_commit_tokens(int32_t B, int32_t max_k, int32_t n_draft_rows,
                       const int32_t* draft_offsets, const int32_t* accept_len,
                       const int32_t* out_tokens, int32_t* seq_tokens, int64_t seq_stride,
                       int32_t* seq_len, int32_t capacity, int32_t* next_tokens, int32_t* status,
                       void* stream) {
  if (!draft_offsets || !accept_len || !out_tokens || !seq_tokens || !seq_len)
    return SV_ERR_NULL;
  if (B < 1 || max_k < 0 || max_k > SV_KMAX || n_draft_rows < 0 || capacity < 0 ||
      seq_stride < capacity)
    return SV_ERR_SHAPE;
  CommitParams prm;
  prm.B = B;
  prm.max_k = max_k;
  prm.n_draft_rows = n_draft_rows;
  prm.capacity = capacity;
  prm.seq_stride = seq_stride;
  prm.offsets = draft_offsets;
  prm.accept_len = accept_len;
  prm.out_tokens = out_tokens;
  prm.seq_tokens = seq_tokens;
  prm.seq_len = seq_len;
  prm.next_tokens = next_tokens;
  prm.status = status;
  const uint32_t grid = static_cast<uint32_t>((B + kCommitThreads - 1) / kCommitThreads);
  hipLaunchKernelGGL(commit_kernel, dim3(grid), dim3(kCommitThreads), 0,
                     static_cast<hipStream_t>(stream), prm);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // extern "C"
