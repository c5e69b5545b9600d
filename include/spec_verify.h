/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-decoding verify step.
 *
 * The operation (pages: "Decodificación Especulativa y EAGLE", ai-engineering.academy
 * Phase 10 lesson 25; Perplexity, "Accelerating Sonar through speculation"):
 * a drafter proposed K_b tokens x_0..x_{K_b-1} for request b; the target model
 * scored the K_b + 1 positions in one forward pass.  This library decides how
 * many drafts to keep and which token follows them:
 *   - sampled requests (temperature T_b > 0), section "La Regla de Exactitud":
 *     with p_t = softmax(target_t / T_b), q_t = softmax(draft_t / T_b), accept
 *     x_t iff r_t * q_t(x_t) < p_t(x_t) for a uniform r_t, scanning t = 0, 1, ...
 *     and stopping at the first rejection n; the stop token is drawn from
 *     (p_n - q_n)+ normalised; if all K_b drafts pass, a bonus token is drawn
 *     from p_{K_b} (section "El Concepto", steps 3-4);
 *   - greedy requests (T_b == 0), same section, greedy case: accept x_t iff
 *     argmax p_t == x_t (lowest index on ties); the stop token is argmax p_n.
 * The blog post calls this the sampler that finds the accepted length and
 * samples one extra target token (section "Objetivo-Borrador").
 *
 * Randomness is a pure function of (seed, request index b, position, token):
 *   r_t        = U(Philox4x32-10(key = seed, counter = (0, t, b, 1)).word0)
 *   E_v (race) = -ln U(Philox4x32-10(key = seed, counter = (v >> 2, pos, b, 0)).word[v & 3])
 *   U(x)       = (2 * (x >> 9) + 1) * 2^-24,  key = (low 32 bits, high 32 bits) of seed
 * and every draw from a distribution w is the exponential race
 *   argmax_v (ln w_v - ln E_v)   (lowest v on exact ties),
 * so results do not depend on the launch shape or the GPU.
 *
 * Layout (packed, row-major, stride V elements; all DEVICE pointers unless noted):
 *   draft_offsets [B + 1] int32   K_b = draft_offsets[b+1] - draft_offsets[b]
 *   target_logits [n_draft_rows + B][V]  row t of request b at draft_offsets[b] + b + t,
 *                                 t = 0..K_b; row t is the target distribution
 *                                 after the prefix x_0..x_{t-1}
 *   draft_logits  [n_draft_rows][V]      row t of request b at draft_offsets[b] + t,
 *                                 the distribution x_t was drawn from
 *   draft_tokens  [n_draft_rows] int32   x_t of request b at draft_offsets[b] + t
 *   out_tokens    [n_draft_rows + B] int32 (output)  request b's slot i at
 *                                 draft_offsets[b] + b + i: x_0..x_{n-1}, then the
 *                                 stop token, then -1 up to i = K_b
 *   accept_len    [B] int32 (output)  n_b in [0, K_b] (accepted drafts; n_b + 1
 *                                 tokens are emitted), or -1 for a failed request
 *   Logits are float32 (SV_F32) or bfloat16 bit patterns (SV_BF16).
 *
 * Ownership: the caller owns every buffer, the workspace included.  The library
 * allocates nothing, keeps no host state between calls (apart from the device
 * address of spec_verify_sample_static's array), never synchronises, and
 * only enqueues one kernel on `stream` (a hipStream_t; NULL is the default
 * stream).  Outputs are valid once the stream reaches the end of the call's
 * work.  The workspace carries hand-off slots between the kernel's
 * workgroups: it must be zero-filled once before its first use (hipMemset),
 * and every call leaves it zero-filled again when it completes, so it can be
 * reused by later calls of any size up to the one it was sized for.  Two
 * calls that may run concurrently need separate workspaces.
 *
 * Errors: a negative return value means nothing was enqueued (except
 * SV_ERR_LAUNCH, which reports a launch failure).  accept_len[b] = -1 with
 * tokens left unwritten would mean a bounded wait inside the kernel expired
 * (the device stopped making progress); zero the workspace again after that.
 * Per-request problems found on the device -- K_b outside [0, max_k], a slice outside [0, n_draft_rows),
 * a draft token outside [0, V), a temperature that is negative, NaN or
 * infinite, a needed row whose maximum is not finite, or a NaN in a row that
 * a sampled request reads -- set accept_len[b] = -1 and fill request b's output
 * slots with -1 (when its slice is valid); other requests are unaffected.
 */
#ifndef SPEC_VERIFY_H_
#define SPEC_VERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_KMAX 8 /* largest per-request draft length */
#define SV_TREE_MAX_NODES 64 /* largest draft tree (root included), spec_verify_tree_greedy */
#define SV_STATIC_SCRATCH_BYTES ((size_t)16 << 20) /* fixed array of spec_verify_sample_static */

enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 };

enum sv_status {
  SV_OK = 0,
  SV_ERR_NULL = -1,      /* a required pointer is NULL */
  SV_ERR_SHAPE = -2,     /* B < 1, V < 1, max_k outside [0, SV_KMAX], n_draft_rows < 0,
                            or the launch grid would be too large */
  SV_ERR_DTYPE = -3,     /* dtype is not SV_F32 or SV_BF16 */
  SV_ERR_WORKSPACE = -4, /* workspace smaller than spec_verify_workspace_bytes() or
                            not 16-byte aligned */
  SV_ERR_LAUNCH = -5,    /* the HIP runtime rejected a kernel launch */
  SV_ERR_SCRATCH = -6    /* spec_verify_sample_static: spec_verify_workspace_bytes(B, V,
                            max_k) exceeds SV_STATIC_SCRATCH_BYTES */
};

/* Host function.  Bytes of device workspace a call with these sizes needs
 * (valid for both dtypes; zero-fill it before first use).  Returns 0 for sizes
 * the library rejects. */
size_t spec_verify_workspace_bytes(int32_t B, int32_t V, int32_t max_k);

/* All-greedy verify (every request follows the temperature-0 rule of section
 * "La Regla de Exactitud").  Draft logits are not needed and not read.
 *   target_logits  device, [n_draft_rows + B][V] of `dtype`
 *   dtype          SV_F32 or SV_BF16 (host scalar)
 *   B, V, max_k, n_draft_rows   host scalars; max_k bounds every K_b
 *   draft_offsets, draft_tokens, accept_len, out_tokens   device, see layout
 *   workspace      device, >= spec_verify_workspace_bytes(B, V, max_k) bytes
 *   stream         hipStream_t to enqueue on
 * Returns SV_OK or a negative sv_status. */
int spec_verify_greedy(const void* target_logits, int32_t dtype, int32_t B, int32_t V,
                       int32_t max_k, int32_t n_draft_rows, const int32_t* draft_offsets,
                       const int32_t* draft_tokens, int32_t* accept_len, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Mixed verify: requests with temperature[b] > 0 follow the sampled rule,
 * requests with temperature[b] == 0 the greedy rule (their draft rows are not
 * read, and their greedy results equal spec_verify_greedy's bit for bit).
 *   draft_logits   device, [n_draft_rows][V] of `dtype`
 *   temperature    device, [B] float32
 *   seed           host; Philox key (low word, high word)
 *   p_at_draft, q_at_draft   optional device outputs [n_draft_rows] float32:
 *                  p_t(x_t) and q_t(x_t) for every position of a sampled
 *                  request (also past its first rejection); NaN for greedy or
 *                  failed requests.  Either may be NULL.
 * Other arguments as for spec_verify_greedy. */
int spec_verify_sample(const void* target_logits, const void* draft_logits, int32_t dtype,
                       int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows,
                       const int32_t* draft_offsets, const int32_t* draft_tokens,
                       const float* temperature, uint64_t seed, int32_t* accept_len,
                       int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Measurement hook (not needed to serve): spec_verify_sample, plus two HIP
 * events (hipEvent_t handles created by the caller) recorded on `stream`
 * immediately before and after the library's kernel, so a benchmark can time
 * the kernel on the stream it runs on.  Both events must be valid.  Same
 * results as spec_verify_sample. */
int spec_verify_sample_timed(const void* target_logits, const void* draft_logits, int32_t dtype,
                             int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows,
                             const int32_t* draft_offsets, const int32_t* draft_tokens,
                             const float* temperature, uint64_t seed, int32_t* accept_len,
                             int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* event_start, void* event_end);

/* ---------------------------------------------------------------- no allocation */

/* For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  spec_verify_sample with the workspace replaced by a fixed
 * array in the library's device code: SV_STATIC_SCRATCH_BYTES (16 MiB) per
 * device, held by every device the library runs on until the process ends.  No call allocates (no hipMalloc, hipFree or
 * allocating library routine).  Same arguments, results and status codes as
 * spec_verify_sample, without workspace and workspace_bytes, plus:
 *   clear_scratch  host; nonzero enqueues a zero fill of the hand-off slots
 *                  this call uses before its kernel.  The first call on a
 *                  device always fills the whole array.  Every completed
 *                  call leaves the slots zero, so 0 is the normal value;
 *                  pass 1 after a call that returned accept_len = -1 from an
 *                  expired wait.
 * Sizes whose spec_verify_workspace_bytes(B, V, max_k) exceeds the array
 * (e.g. B = 1024 requests of max_k = 8 at V = 256k) return SV_ERR_SCRATCH
 * with nothing enqueued.  The slots start zero (the loader zero-fills the
 * array, and the first call fills it again); each call relies on the last
 * completed call on that device having left them zero.  All calls on one
 * device share the array: two calls that may overlap in time on one device
 * (different streams or host threads) race and give wrong results.  The
 * first call on a device looks up the array's device address with
 * hipGetSymbolAddress (with that device current) and keeps it for later
 * calls. */
int spec_verify_sample_static(const void* target_logits, const void* draft_logits, int32_t dtype,
                              int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows,
                              const int32_t* draft_offsets, const int32_t* draft_tokens,
                              const float* temperature, uint64_t seed, int32_t* accept_len,
                              int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                              int32_t clear_scratch, void* stream);

/* ---------------------------------------------------------------- early exit */

/* Host function.  Workspace bytes spec_verify_sample_early_exit needs (either
 * dtype); 0 for a bad shape.  The workspace must be zero-filled once when
 * allocated; completed calls keep it usable without further clearing (zero it
 * again after a call that reported accept_len = -1 from an expired wait). */
size_t spec_verify_early_exit_workspace_bytes(int32_t B, int32_t V, int32_t max_k);

/* Early-exit verify: the decision of spec_verify_sample without reading the
 * rows past each request's stop.  The ratio tests run left to right and stop
 * at the first rejection ("Decodificación Especulativa y EAGLE", section "La
 * Regla de Exactitud"; "El Concepto", steps 3-4), so target and draft rows
 * after the stop position cannot change the outcome; this entry point
 * streams a request's rows one position (stage) at a time and skips the
 * stages that start after the request's stop is decided.  A stage whose
 * previous decision is still pending when it starts streams anyway (on
 * speculation), so small batches stream their stages together.
 * Arguments, layout, ownership and status codes as for spec_verify_sample,
 * with these differences:
 *   - accept_len and out_tokens equal spec_verify_sample's (same Philox
 *     streams and race keys; a race near-tie may resolve differently, as
 *     between any two float orders of the same keys);
 *   - p_at_draft / q_at_draft are written for positions t <= n and are NaN
 *     for positions past the stop n, which are never evaluated;
 *   - a non-finite row past the stop is not read, so it does not fail the
 *     request (spec_verify_sample reads every row and fails it);
 *   - it trades parallelism inside a request for bytes: worthwhile for large
 *     batches whose requests mostly stop well before K_b, slower than
 *     spec_verify_sample for small ones (its stage decisions form a chain).
 *     On MI355X it pays once the full verify takes more than about 50 us:
 *     K = 8 fp32 from 32 requests of V = 128256, ragged K <= 8 bf16 from
 *     64 requests of V = 152064; at K = 1 the two are within a few us.
 * The workspace is the one sized by spec_verify_early_exit_workspace_bytes.
 * Unlike spec_verify_sample, each call enqueues two kernels on `stream`: the
 * verify kernel, then a small kernel that clears its decision records and
 * the partials of stages streamed on speculation past a stop.  As
 * for the other entry points, accept_len[b] = -1 with no fault found in the
 * request means a bounded wait expired; the workspace may then hold stale
 * hand-off slots, so zero it again before the next call.  Calls that overlap
 * in time need separate workspaces. */
int spec_verify_sample_early_exit(const void* target_logits, const void* draft_logits,
                                  int32_t dtype, int32_t B, int32_t V, int32_t max_k,
                                  int32_t n_draft_rows, const int32_t* draft_offsets,
                                  const int32_t* draft_tokens, const float* temperature,
                                  uint64_t seed, int32_t* accept_len, int32_t* out_tokens,
                                  float* p_at_draft, float* q_at_draft, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- draft side */

/* Host function.  Workspace bytes spec_draft_sample needs for B rows of V
 * logits (either dtype); 0 for B < 1 or V < 1.  The workspace must be
 * zero-filled once when allocated; every call leaves it zero again. */
size_t spec_draft_workspace_bytes(int32_t B, int32_t V);

/* Draft-side sampler: the drafting step that precedes verification draws
 * each draft token from softmax(q / T) ("Decodificación Especulativa y
 * EAGLE", section "El Concepto", step 1, and its listing's draft loop), or
 * takes the top token at T = 0 (Perplexity's draft-target scheme drafts
 * greedily).  One call draws one token for each of B requests, from row b of
 * draft_logits, at draft step `step`:
 *   temperature[b] == 0: tokens[b] = lowest index attaining the row maximum;
 *   temperature[b] > 0:  tokens[b] = argmax_v (z_v / T - ln E_v), ties to the
 *       lowest index, with E_v = -ln U_v and U_v from Philox4x32-10 keyed by
 *       `seed`, counter (v >> 2, step, b, 2), word v & 3, mapped to
 *       (2 (x >> 9) + 1) 2^-24.  An exponential race, so tokens[b] is an
 *       exact draw from softmax(z / T); stream tag 2 keeps these draws apart
 *       from the verify step's (tags 0 and 1).  Calling with step = t for
 *       t = 0..K-1 gives independent draft steps.
 *   draft_logits   device, [B][V] of `dtype`, row-major, contiguous
 *   temperature    device, [B] float32; negative, NaN or infinite values fail
 *                  that request (tokens[b] = -1)
 *   seed, step     host; step >= 0
 *   tokens         device out, [B] int32; -1 for a failed request: a bad
 *                  temperature, a row with no finite maximum, a NaN or +inf
 *                  logit in a sampled row, or an expired internal wait
 *   q_at           device out, optional [B] float32: softmax(z / T) at
 *                  tokens[b] for sampled requests, NaN for greedy or failed
 *                  ones; may be NULL
 *   workspace      device, >= spec_draft_workspace_bytes(B, V) bytes,
 *                  16-byte aligned, zero-filled at allocation; calls that
 *                  overlap in time need separate workspaces
 *   stream         hipStream_t; the call only enqueues work on it
 * Returns SV_OK, or a negative status with nothing enqueued (SV_ERR_NULL for
 * a missing required pointer, SV_ERR_SHAPE for B < 1, V < 1 or step < 0,
 * SV_ERR_DTYPE, SV_ERR_WORKSPACE, SV_ERR_LAUNCH). */
int spec_draft_sample(const void* draft_logits, int32_t dtype, int32_t B, int32_t V,
                      const float* temperature, uint64_t seed, int32_t step, int32_t* tokens,
                      float* q_at, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- commit step */

/* Commit step after verification: appends each request's emitted tokens to
 * its token history on the device, so the serving loop needs no host round
 * trip to learn the verify step's outcome (Perplexity's "Accelerating Sonar
 * through speculation", section on MTP scheduling: a kernel writes the
 * accepted tokens into their places).  For request b with
 * n = accept_len[b] and history length L = seq_len[b]:
 *   - n < 0 (a failed verify), n > K_b, or a slice outside the packed
 *     layout (draft_offsets as for the verify step, K_b <= max_k): the
 *     request is left unchanged, status[b] = -1;
 *   - L < 0 or L + n + 1 > capacity: unchanged, status[b] = -2;
 *   - otherwise out_tokens[draft_offsets[b] + b + i], i = 0..n (the
 *     accepted drafts, then the emitted token) are written to
 *     seq_tokens[b * seq_stride + L + i], seq_len[b] becomes L + n + 1,
 *     next_tokens[b] the last of them, status[b] = n + 1.
 * next_tokens[b] is -1 for a request left unchanged.  Each call appends
 * again: call it once per verify step.
 *   draft_offsets  device, [B+1] int32 (the verify step's)
 *   accept_len     device, [B] int32 (the verify step's output)
 *   out_tokens     device, [n_draft_rows + B] int32 (the verify step's output)
 *   seq_tokens     device in/out, [B][seq_stride] int32 token histories
 *   seq_len        device in/out, [B] int32 history lengths
 *   capacity       host; usable entries per history row (<= seq_stride)
 *   next_tokens, status   device out, optional [B] int32; either may be NULL
 *   stream         hipStream_t; the call only enqueues work on it
 * Returns SV_OK, or a negative status with nothing enqueued (SV_ERR_NULL for
 * a missing required pointer; SV_ERR_SHAPE for B < 1, max_k outside
 * [0, SV_KMAX], n_draft_rows < 0, capacity < 0 or seq_stride < capacity;
 * SV_ERR_LAUNCH). */
int spec_commit_tokens(int32_t B, int32_t max_k, int32_t n_draft_rows,
                       const int32_t* draft_offsets, const int32_t* accept_len,
                       const int32_t* out_tokens, int32_t* seq_tokens, int64_t seq_stride,
                       int32_t* seq_len, int32_t capacity, int32_t* next_tokens, int32_t* status,
                       void* stream);

/* Host function.  Static description of a status code. */
const char* spec_verify_status_string(int status);

/* ---------------------------------------------------------------- draft trees */

/* Host function.  Workspace bytes spec_verify_tree_greedy needs (either
 * dtype); 0 unless B >= 1, V >= 1 and 1 <= max_nodes <= SV_TREE_MAX_NODES.
 * The workspace must be zero-filled once when allocated; every call leaves it
 * zero again (unless a bounded wait expired, as for the verify step). */
size_t spec_verify_tree_workspace_bytes(int32_t B, int32_t V, int32_t max_nodes);

/* Greedy verification of a draft tree.  The drafter expanded several
 * candidates per position into a tree and the target scored every node in
 * one pass, each node attending only to its ancestors; the result is the
 * longest prefix along an accepted root-to-node path ("Decodificación
 * Especulativa y EAGLE", section on tree attention verification), followed by
 * one extra target token (Perplexity's post, section "EAGLE").  With the
 * greedy rule of section "La Regla de Exactitud" a node is accepted when its
 * parent is accepted and its token is the argmax of the parent's target row
 * (lowest index on ties).  Only the greedy rule is provided: the pages give
 * no rule for sampling over a tree.
 *
 * Layout (DEVICE pointers, packed like the linear verify's target rows):
 *   node_offsets  [B + 1] int32  request b owns nodes i = 0..N_b - 1,
 *                                N_b = node_offsets[b+1] - node_offsets[b]
 *   target_logits [n_rows][V]    row of node i at node_offsets[b] + i: the
 *                                target distribution after the path root..i
 *   parents       [n_rows] int32 parent of node i >= 1, in [0, i) (parents
 *                                are numbered before their children); the
 *                                root's entry (i = 0) is not read
 *   tokens        [n_rows] int32 draft token of node i >= 1, in [0, V); the
 *                                root's entry is not read (the root is the
 *                                last token already emitted)
 * Per request, with g_i the argmax of node i's row and c the accepted node
 * of greatest depth d (lowest index among equally deep ones; two exist only
 * when siblings share a token), path root = a_0, ..., a_d = c:
 *   accept_len[b]                    = d (drafts accepted; d + 1 tokens emitted)
 *   out_tokens[node_offsets[b] + j]  = token of a_{j+1} for j < d, g_c for j = d,
 *                                      -1 for d < j < N_b
 *   accept_nodes[node_offsets[b] + j] = a_j for j <= d, -1 after (optional:
 *                                      NULL skips it; the node indices tell the
 *                                      caller which KV-cache entries to keep)
 * Per-request failures set accept_len[b] = -1: a slice outside [0, n_rows),
 * N_b outside [1, max_nodes] (nothing else written); a parent outside
 * [0, i), a token outside [0, V), or a row whose maximum is not finite (the
 * request's out_tokens and accept_nodes entries set to -1).
 * Ownership, streams and the workspace as for spec_verify_greedy; the
 * workspace is the one sized by spec_verify_tree_workspace_bytes.  One
 * kernel is enqueued on `stream`.
 * Returns SV_OK, or a negative status with nothing enqueued (SV_ERR_NULL for
 * a missing required pointer; SV_ERR_SHAPE for B < 1, V < 1, max_nodes
 * outside [1, SV_TREE_MAX_NODES], n_rows < 0 or a grid too large;
 * SV_ERR_DTYPE; SV_ERR_WORKSPACE; SV_ERR_LAUNCH). */
int spec_verify_tree_greedy(const void* target_logits, int32_t dtype, int32_t B, int32_t V,
                            int32_t max_nodes, int32_t n_rows, const int32_t* node_offsets,
                            const int32_t* parents, const int32_t* tokens, int32_t* accept_len,
                            int32_t* out_tokens, int32_t* accept_nodes, void* workspace,
                            size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H_ */
