// spec_verify.hip -- gfx950 kernel and C ABI of the speculative-decoding verify step.
//
// What is computed is stated in include/spec_verify.h (the accept / residual /
// bonus rule of "Decodificación Especulativa y EAGLE", section "La Regla de
// Exactitud", and its greedy case).  How it runs on MI355X: one launch.
//
// Vocabulary chunks.  Every row is cut into chunks of 8 KiB (4096 bf16 or
// 2048 float32 logits).  Each workgroup does one task:
//   1. statistics of one group of a request's row-chunks (8 row-chunks in
//      row-major order when every request has max_k drafts, else one column
//      of m chunks across the request's rows): each wave streams whole
//      row-chunks (8 16-byte loads per lane, two row-chunks in flight) and
//      reduces each to one 8-byte partial: (max, sum of 2^((z - max) c)),
//      c = log2(e) / T, for the K+1 target and K draft rows of a sampled
//      request, or (max, lowest argmax index) for the K+1 target rows of a
//      greedy one;
//   2. race over one range of chunks of a sampled request: fold the partials
//      of all its rows (every race workgroup of the request does the same
//      fold in the same order, so all of them find the same values), gather
//      p_t(x_t) and q_t(x_t), draw r_t, find the first rejection n with a
//      wave ballot, then run the exponential race over its chunks of row n --
//      the residual (p_n - q_n)+ after a rejection, p_K otherwise.
// Grid order: a request's ngr race workgroups follow its statistics by lag
// requests' worth of statistics workgroups, so they usually find the
// partials ready and one request's race arithmetic overlaps the streaming
// of later ones.  The last workgroup of a request in grid order finishes it:
// the last statistics workgroup with items of a greedy request folds its
// argmaxes and writes the outputs; the last race workgroup of a sampled
// request folds the chunk winners and writes the outputs.  Each polls the
// slots of its siblings, which sit earlier in the grid.
//
// Hand-offs between workgroups use 8-byte slots in the workspace that are
// all-zero until written (a written slot never has all-zero bits: +0.0 is
// stored as -0.0).  Producers store with device-coherent (sc1) stores;
// consumers poll with device-coherent loads.  The finishing workgroup of a
// request writes every slot of that request back to zero, so the workspace
// is all-zero again after every call.  No agent-
// scope release/acquire fence is used (on gfx950 those write back or
// invalidate the XCD's whole L2).  A workgroup waits only for partials of
// workgroups earlier in the grid, and those store their partials before they
// wait for anything, so with in-order dispatch every wait ends.  Waits are
// also bounded (kSpinLimit polls); an expired wait reports accept_len = -1.
//
// Race keys: the winner maximises ln w_v - ln E_v, i.e. w_v / E_v.  Inside a
// thread and chunk, candidates are compared by cross-multiplication
// (w_a e_b > w_b e_a) with e = -log2 U = E / ln 2 (a common factor); a
// thread's best in a chunk becomes the float key w / e, and keys merge
// across threads, chunks and workgroups by (larger key, then lower index),
// an order-independent rule, so the winner does not depend on how chunks are
// grouped.  Weights are 2^((z - m) c) with m the row maximum, the exponent
// formed from the exact difference z - m (device_common.h), and the row's sum
// is formed relative to the same m, so m cancels exactly from p = w / sum.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <mutex>
#include <type_traits>
#include <cmath>
#include <cstdint>

#include "spec_verify.h"
#include "device_common.h"

namespace {

constexpr int kRowsMax = 2 * SV_KMAX + 1;         // row slots per request
constexpr int kFoldBlocks = 8;  // canonical blocks of a row per round of a fold
constexpr int kFoldSlotsPerThread = (kRowsMax * kFoldBlocks * kGroupItems + 255) / 256;
constexpr uint32_t kExpiredIdx = 0xFFFFFFFEu;  // race slot word: a wait expired
// s_sleep units (64 clocks each) between polling rounds of a fold
#ifndef SV_FOLD_SLEEP
#define SV_FOLD_SLEEP 1
#endif
// Workgroups of this kernel one CU holds at once (at most 96 VGPRs per lane:
// five waves per SIMD, so five 4-wave workgroups per CU).
constexpr int kWorkgroupsPerCu = 5;
// XCDs of an MI355X; the dispatcher deals workgroups to them round robin.
constexpr int kXcds = 8;

// Stage timestamps (a build with SV_TRACE defined only; the product build
// compiles them out).  Workgroup g records its role in word 0 of its record
// (kind | request << 8 | group << 32; kind 1: statistics, 2: race) and the
// wall clock (hipDeviceAttributeWallClockRate) at numbered stages in words
// 1..kTracePoints - 1; spec_verify_trace_copy reads the records back.
#ifdef SV_TRACE
constexpr int kTraceWgs = 1 << 16, kTracePoints = 10;
__device__ uint64_t sv_trace[kTraceWgs * kTracePoints];
#define SV_TRACE_HEAD(kind, b, grp)                                                      \
  do {                                                                                   \
    if (threadIdx.x == 0 && blockIdx.x < kTraceWgs)                                      \
      sv_trace[blockIdx.x * kTracePoints] = static_cast<uint64_t>(kind) |                \
                                            (static_cast<uint64_t>(b) << 8) |            \
                                            (static_cast<uint64_t>(grp) << 32);          \
  } while (0)
#define SV_STAMP(i)                                                                      \
  do {                                                                                   \
    if (threadIdx.x == 0 && blockIdx.x < kTraceWgs)                                      \
      sv_trace[blockIdx.x * kTracePoints + (i)] = wall_clock64();                        \
  } while (0)
#else
#define SV_TRACE_HEAD(kind, b, grp) \
  do {                              \
  } while (0)
#define SV_STAMP(i) \
  do {              \
  } while (0)
#endif

// ------------------------------------------------------------------ parameters

struct Params {
  const void* target;
  const void* draft;
  const int32_t* offsets;
  const int32_t* tokens;
  const float* temperature;  // NULL: every request greedy
  uint32_t k0, k1;           // Philox key
  int32_t B, V, max_k, n_draft_rows;
  int32_t nc;   // row-chunks per row
  int32_t flat; // 1: flat grouping (one 8-chunk block of one row per workgroup), 0: column
  int32_t m;    // column grouping: chunks per workgroup
  int32_t ng;   // workgroups per request: ceil(nc / m), or rows ceil(nc / 8) when flat
  int32_t mr;   // race chunks per race workgroup
  int32_t ngr;  // race workgroups per request, ceil(nc / mr) <= ng
  int32_t lag;  // request b's race workgroups follow the statistics of request b + lag
  uint64_t* part;    // [B][2 max_k + 1][nc] block (flat) or row-chunk (column) partials
  uint64_t* race;    // [B][ngr] race winner of each race workgroup
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_at;
  float* q_at;
};

// Per-request checks every workgroup can make from the request's scalars.
struct Req {
  int32_t off0, K;
  float T;
  bool slice_ok, temp_ok, greedy;
  __device__ bool valid() const { return slice_ok && temp_ok; }
  __device__ bool sampled() const { return slice_ok && temp_ok && !greedy; }
};

__device__ __forceinline__ Req load_req(const Params& p, int b) {
  Req r;
  r.off0 = p.offsets[b];
  const int32_t off1 = p.offsets[b + 1];
  // wrapping difference; it is K_b whenever off1 >= off0 >= 0, the only case used
  r.K = static_cast<int32_t>(static_cast<uint32_t>(off1) - static_cast<uint32_t>(r.off0));
  r.slice_ok = r.off0 >= 0 && off1 <= p.n_draft_rows && off1 >= r.off0 && r.K <= p.max_k;
  r.T = p.temperature ? p.temperature[b] : 0.f;
  r.greedy = r.T == 0.f;
  r.temp_ok = (r.T >= 0.f) && (r.T < INFINITY) && (r.greedy || r.K == 0 || p.draft != nullptr);
  return r;
}

// Outputs of a failed request whose slice is valid.
__device__ void write_fault(const Params& p, int b, const Req& r) {
  const int tid = threadIdx.x;
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  if (tid <= r.K) p.out_tokens[trow0 + tid] = -1;
  if (tid < r.K) {
    if (p.p_at) p.p_at[r.off0 + tid] = NAN;
    if (p.q_at) p.q_at[r.off0 + tid] = NAN;
  }
  if (tid == 0) p.accept_len[b] = -1;
}

// Row r of a request (r <= K target row r, else draft row r - K - 1) keeps its
// partials in row slot j.
__device__ __forceinline__ int row_slot(const Params& p, int K, int r) {
  return r <= K ? r : p.max_k + r - K;
}

// A row's statistics are folded over canonical blocks: chunks [8k, 8k + 8)
// of the row.  With flat grouping a statistics workgroup covers one block
// and leaves its merged partial in slot k of the row; with column grouping
// workgroups leave one partial per row-chunk (slot c) and the fold forms the
// blocks.  Both give the same floats, so results do not depend on the grid.
__device__ __forceinline__ int blocks_per_row(const Params& p) {
  return (p.nc + kGroupItems - 1) / kGroupItems;
}
__device__ __forceinline__ int slots_per_row(const Params& p) {
  return p.flat ? blocks_per_row(p) : p.nc;
}

__device__ __forceinline__ uint64_t* part_slot(const Params& p, int b, int j, int u) {
  return p.part + (static_cast<int64_t>(b) * (2 * p.max_k + 1) + j) * p.nc + u;
}

// Zeroes the partials of rows 0..nrows-1 of request b (the finishing
// workgroup, once every reader of them is done).
__device__ void clear_request(const Params& p, int b, int K, int nrows) {
  const int ns = slots_per_row(p);
  const int n = nrows * ns;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int r = i / ns;
    slot_store(part_slot(p, b, row_slot(p, K, r), i - r * ns), 0u);
  }
}

// The canonical block merge of n chunk partials in order: the largest
// maximum, then the sums moved to it and added in order (sampled); the larger
// maximum, then the lower index (greedy, exact in any order).
template <bool GREEDY>
__device__ __forceinline__ uint64_t merge_block(const uint64_t* part, int n, float cf) {
  float M = -INFINITY;
  int I = INT_MAX;
  if constexpr (GREEDY) {
    for (int i = 0; i < n; ++i) merge_argmax(M, I, slot_f(part[i]), static_cast<int>(slot_w(part[i])));
    return pack_slot(M, static_cast<uint32_t>(I));
  } else {
    for (int i = 0; i < n; ++i) M = fmaxf(M, slot_f(part[i]));
    const float mc = weight_ref(M);
    float S = 0.f;
    for (int i = 0; i < n; ++i) S += __uint_as_float(slot_w(part[i])) * rescale(slot_f(part[i]), cf, mc);
    return pack_slot(M, __float_as_uint(S));
  }
}

__device__ void finish_greedy(const Params& p, int b, const Req& r);

// One wave's row-chunks of request b in group cg, reduced to (max, sum)
// partials for a sampled request or (max, argmax) for a greedy one.
template <bool BF16, bool VEC, bool GREEDY>
__device__ void stats_items(const Params& p, int b, const Req& r, int cg, float cf) {
  __shared__ uint64_t sh_block[kGroupItems];  // flat grouping: the block's chunk partials
  constexpr int CHUNK = chunk_tokens(BF16);
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int K = r.K;
  const int nrows = GREEDY ? K + 1 : 2 * K + 1;
  // The request's (row, chunk) items are numbered row-major over the chunks
  // a group covers; item i is row i / span, chunk c0 + i % span.  Flat
  // grouping: group cg covers block k = cg mod (blocks per row) of row
  // cg / (blocks per row), chunks [8k, 8k + 8).  Column grouping: group cg
  // covers m chunks from cg m and takes all its rows x m items.
  int span, c0, i_lo, i_hi;
  if (p.flat) {
    const int bpr = blocks_per_row(p);
    const int row = cg / bpr;
    if (row >= nrows) return;  // (a greedy request's groups past its rows)
    c0 = (cg - row * bpr) * kGroupItems;
    span = min(kGroupItems, p.nc - c0);
    i_lo = row * span;
    i_hi = i_lo + span;
  } else {
    c0 = cg * p.m;
    span = min(p.m, p.nc - c0);
    i_lo = 0;
    i_hi = nrows * span;
  }
  // (the scalar-load path holds one row-chunk at a time: its loads are
  // 2-byte or 4-byte, so a row-chunk already takes many registers in flight)
  constexpr int IN_FLIGHT = VEC ? kItemsInFlight : 1;
  // wave w takes items 2w, 2w+1 of the group, then 8 further on
  for (int i0 = i_lo + wave * IN_FLIGHT; i0 < i_hi; i0 += kWaves * IN_FLIGHT) {
    uint4 buf[IN_FLIGHT][kItemVecs];
#pragma unroll
    for (int k = 0; k < IN_FLIGHT; ++k) {
      // issue every load before any math, on one code path: past the last
      // item the wave loads the last item again (the second load of the same
      // lines is served by the cache) and skips it below
      const int i = min(i0 + k, i_hi - 1);
      const int row = i / span;
      const int c = c0 + i - row * span;
      const bool tgt = row <= K;
      const int64_t prow = tgt ? static_cast<int64_t>(r.off0) + b + row
                               : static_cast<int64_t>(r.off0) + row - K - 1;
      load_item<BF16, VEC>(tgt ? p.target : p.draft, prow, p.V, static_cast<int64_t>(c) * CHUNK,
                           buf[k]);
    }
#pragma unroll
    for (int k = 0; k < IN_FLIGHT; ++k) {
      const int i = i0 + k;
      if (i < i_hi) {
        const int row = i / span;
        const int c = c0 + i - row * span;
        if (VEC && static_cast<int64_t>(c + 1) * CHUNK > p.V)
          mask_tail<BF16>(buf[k], p.V, static_cast<int64_t>(c) * CHUNK);
        const uint64_t v = GREEDY ? item_argmax<BF16>(buf[k], static_cast<int64_t>(c) * CHUNK)
                                  : item_stats<BF16>(buf[k], cf);
        if (lane == 0) {
          if (p.flat)
            sh_block[i - i_lo] = v;
          else
            slot_store(part_slot(p, b, row_slot(p, K, row), c), v);
        }
      }
    }
  }
  if (p.flat) {
    __syncthreads();
    if (threadIdx.x == 0) {
      const int row = i_lo / span;
      slot_store(part_slot(p, b, row_slot(p, K, row), c0 / kGroupItems),
                 merge_block<GREEDY>(sh_block, span, cf));
    }
  }
}

// Statistics of request b over the chunks of group cg.
template <bool BF16, bool VEC>
__device__ void stats_part(const Params& p, int b, int cg) {
  SV_TRACE_HEAD(1, b, cg);
  const Req r = load_req(p, b);
  SV_STAMP(2);  // the request's scalars loaded
  const int tid = threadIdx.x;
  if (!r.valid()) {
    if (cg == 0) {
      if (r.slice_ok)
        write_fault(p, b, r);
      else if (tid == 0)
        p.accept_len[b] = -1;
    }
    return;
  }
  if (r.greedy) {
    stats_items<BF16, VEC, true>(p, b, r, cg, 0.f);
    SV_STAMP(3);  // partials stored
    // the request's last workgroup with items finishes it (flat grouping
    // leaves the groups past a greedy request's (K+1) nc items empty)
    const int last = p.flat ? (r.K + 1) * blocks_per_row(p) - 1 : p.ng - 1;
    if (cg == last) finish_greedy(p, b, r);
  } else {
    stats_items<BF16, VEC, false>(p, b, r, cg, kLog2e / r.T);
    SV_STAMP(3);  // partials stored
  }
}

// ------------------------------------------------------------------ folding

struct FoldShared {
  uint64_t slots[kRowsMax * kFoldBlocks * kGroupItems];  // one round of partials, [row][slot]
  float m[kWaves][kRowsMax];
  float s[kWaves][kRowsMax];  // greedy: argmax index bits
  float row_m[kRowsMax];      // folded row maximum
  float row_ls[kRowsMax];     // sampled: log2 of the row sum; greedy: argmax index bits
  int bad;                    // 1: a row is not finite, 2: a wait expired
};

// One round of a fold: row = lane takes blocks blk0 + 2w, blk0 + 2w + 1
// (wave w) from the round's slots in LDS (nsr per row, spb per block; a
// block of chunk partials is merged with merge_block) into its running row
// statistics (M, S) or argmax (M, I).
template <bool GREEDY>
__device__ __forceinline__ void fold_round(const uint64_t* rs, int blk0, int nb, int nsr,
                                           int spb, float cf, float& M, float& S, int& I) {
  const int wave = wave_id();
  uint64_t bv[2] = {0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = 2 * wave + h;  // block within the round
    if (blk0 + j >= nb) continue;
    const int a = j * spb, n = min(spb, nsr - a);
    if (n <= 0) continue;
    bool have = true;
    for (int i = 0; i < n; ++i) have = have && rs[a + i] != 0u;
    if (have) bv[h] = spb == 1 ? rs[a] : merge_block<GREEDY>(rs + a, n, cf);
  }
  if constexpr (GREEDY) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (bv[h] != 0u) merge_argmax(M, I, slot_f(bv[h]), static_cast<int>(slot_w(bv[h])));
  } else {
    float bm = M;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (bv[h] != 0u) bm = fmaxf(bm, slot_f(bv[h]));
    const float bmc = weight_ref(bm);
    S *= rescale(M, cf, bmc);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (bv[h] != 0u) S += __uint_as_float(slot_w(bv[h])) * rescale(slot_f(bv[h]), cf, bmc);
    M = bm;
  }
}

// Folds the partials of rows 0..nrows-1 of request b, in rounds of
// kFoldBlocks canonical blocks per row (fold_round).  When the request has
// at most 64 slots (one round), wave 0 polls them all, one per lane, and
// stages them in LDS as they arrive.  Otherwise the workgroup first waits
// for the request's last slot (sampled), then per round loads the round's
// slots with adjacent threads on adjacent slots (few memory transactions),
// re-polls the slots still missing, and stages them in LDS.  At the end
// wave 0 merges the waves in order.  The order of every operation depends on
// nc only, so every workgroup that folds the same request, and every grid,
// gets the same floats.
template <bool GREEDY>
__device__ void fold_rows(const Params& p, int b, int K, int nrows, float cf, FoldShared& sh) {
  static_assert(kFoldBlocks == 2 * kWaves, "two blocks per wave per round");
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  if (tid == 0) sh.bad = 0;
  const bool active = lane < nrows;
  const int nb = blocks_per_row(p), ns = slots_per_row(p);
  const int spb = p.flat ? 1 : kGroupItems;  // slots per block
  float M = -INFINITY, S = 0.f;
  int I = INT_MAX;
  bool expired = false;
  if (nb <= kFoldBlocks && nrows * ns <= 64) {
    // one round: wave 0 polls every slot directly (a lane per slot)
    if (wave == 0) {
      const int n_slots = nrows * ns;
      const int q = min(lane, n_slots - 1);
      const int row = q / ns;
      uint64_t* slot = part_slot(p, b, row_slot(p, K, row), q - row * ns);
      uint64_t v = slot_load(slot);
      for (unsigned it = 0; __ballot(v == 0u) != 0u && it < kSpinLimit; ++it) {
        __builtin_amdgcn_s_sleep(SV_FOLD_SLEEP);
        if (v == 0u) v = slot_load(slot);
      }
      expired = __ballot(v == 0u) != 0u;
      if (lane < n_slots) sh.slots[lane] = v;
    }
    if constexpr (!GREEDY) SV_STAMP(3);  // race: the request's last partial seen
    __syncthreads();
    if (active) fold_round<GREEDY>(sh.slots + lane * ns, 0, nb, ns, spb, cf, M, S, I);
  } else {
    if constexpr (!GREEDY) {
      // A race workgroup may start long before the request's statistics are
      // in.  It first waits, with one lane, for the request's last slot,
      // which the last statistics workgroup in grid order writes, and only
      // then loads every slot: hundreds of racing workgroups each re-polling
      // hundreds of partials would load the memory system that the
      // statistics stream through.
      if (tid == 0) slot_wait(part_slot(p, b, row_slot(p, K, nrows - 1), ns - 1));
      SV_STAMP(3);  // race: the request's last partial seen
    }
    for (int blk0 = 0; blk0 < nb; blk0 += kFoldBlocks) {
      const int u0 = blk0 * spb;                       // the round's first slot
      const int nsr = min(kFoldBlocks * spb, ns - u0);  // slots per row this round
      const int n_slots = nrows * nsr;
      __syncthreads();  // the previous round's LDS reads are done
      uint64_t v[kFoldSlotsPerThread];
#pragma unroll
      for (int i = 0; i < kFoldSlotsPerThread; ++i) {  // issue every load before waiting on any
        // on one code path: past the round's last slot a thread loads that slot again
        const int q = min(tid + i * kThreads, n_slots - 1);
        const int row = q / nsr;
        v[i] = slot_load(part_slot(p, b, row_slot(p, K, row), u0 + q - row * nsr));
      }
      // re-poll every slot still missing together, one round trip per round
      uint32_t missing = 0u;
#pragma unroll
      for (int i = 0; i < kFoldSlotsPerThread; ++i)
        if (tid + i * kThreads < n_slots && v[i] == 0u) missing |= 1u << i;
      for (unsigned it = 0; missing != 0u && it < kSpinLimit; ++it) {
        __builtin_amdgcn_s_sleep(SV_FOLD_SLEEP);
#pragma unroll
        for (int i = 0; i < kFoldSlotsPerThread; ++i) {
          if (missing & (1u << i)) {
            const int q = tid + i * kThreads;
            const int row = q / nsr;
            v[i] = slot_load(part_slot(p, b, row_slot(p, K, row), u0 + q - row * nsr));
          }
        }
#pragma unroll
        for (int i = 0; i < kFoldSlotsPerThread; ++i)
          if ((missing & (1u << i)) && v[i] != 0u) missing &= ~(1u << i);
      }
      if (missing != 0u) expired = true;
#pragma unroll
      for (int i = 0; i < kFoldSlotsPerThread; ++i) {
        const int q = tid + i * kThreads;
        if (q < n_slots) sh.slots[q] = v[i];
      }
      __syncthreads();
      if (active) fold_round<GREEDY>(sh.slots + lane * nsr, blk0, nb, nsr, spb, cf, M, S, I);
    }
  }
  __syncthreads();  // sh.bad initialised
  if (expired) atomicOr(&sh.bad, 2);
  if (active) {
    sh.m[wave][lane] = M;
    sh.s[wave][lane] = GREEDY ? __int_as_float(I) : S;
  }
  __syncthreads();
  if (wave == 0 && active) {
    for (int w = 1; w < kWaves; ++w) {
      if constexpr (GREEDY)
        merge_argmax(M, I, sh.m[w][lane], __float_as_int(sh.s[w][lane]));
      else
        merge_stats(M, S, sh.m[w][lane], sh.s[w][lane], cf);
    }
    const bool finite_max = M > -INFINITY && M < INFINITY;
    if (!finite_max || (!GREEDY && !(S < INFINITY))) atomicOr(&sh.bad, 1);
    sh.row_m[lane] = M;
    sh.row_ls[lane] = GREEDY ? __int_as_float(I) : fast_log2(S);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ greedy finish

__device__ void finish_greedy(const Params& p, int b, const Req& r) {
  __shared__ FoldShared sh;
  __shared__ int sh_n;
  const int tid = threadIdx.x;
  __syncthreads();  // this workgroup's own partials are stored
  const int K = r.K;
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  int32_t x = 0;
  bool bad_token = false;
  if (tid < K) {
    x = p.tokens[r.off0 + tid];
    bad_token = x < 0 || x >= p.V;
  }
  fold_rows<true>(p, b, K, K + 1, 0.f, sh);
  SV_STAMP(4);  // greedy finisher: partials folded
  const bool any_bad_token = __syncthreads_or(bad_token);
  clear_request(p, b, K, K + 1);
  if (sh.bad & 2) {
    if (tid == 0) p.accept_len[b] = -1;
    return;
  }
  if (sh.bad || any_bad_token) {
    write_fault(p, b, r);
    return;
  }
  // first t < K whose draft differs from the argmax; the stop token is argmax row n
  const bool mismatch = tid < K && __float_as_int(sh.row_ls[tid]) != x;
  const uint64_t mask = __ballot(mismatch);
  if (tid == 0) sh_n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : K;
  __syncthreads();
  const int n = sh_n;
  if (tid <= K) {
    const int32_t y = __float_as_int(sh.row_ls[n]);
    p.out_tokens[trow0 + tid] = (tid < n) ? x : (tid == n ? y : -1);
  }
  if (tid < K) {
    if (p.p_at) p.p_at[r.off0 + tid] = NAN;
    if (p.q_at) p.q_at[r.off0 + tid] = NAN;
  }
  if (tid == 0) p.accept_len[b] = n;
  SV_STAMP(5);  // greedy outputs written
}

// ------------------------------------------------------------------ race

struct RaceRow {
  float mp, lsp, mq, lsq, cf;
  int n;
};

template <bool BF16, bool VEC>
__device__ __forceinline__ void load4(const void* rowp, int64_t v, int64_t vend, float out[4]) {
  if (VEC && v + 4 <= vend) {
    if constexpr (BF16) {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(rowp) + v);
      out[0] = bf16_lo(w.x);
      out[1] = bf16_hi(w.x);
      out[2] = bf16_lo(w.y);
      out[3] = bf16_hi(w.y);
    } else {
      const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(rowp) + v);
      out[0] = w.x;
      out[1] = w.y;
      out[2] = w.z;
      out[3] = w.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = (v + k < vend) ? load_logit<BF16>(rowp, v + k) : 0.f;
  }
}

// Race candidates of tokens 4g..4g+3 folded into this thread's best
// (bw / be, bidx); tokens arrive in increasing order, so a strict > keeps the
// lowest index on ties.  Bonus weights drop the row's common factor 2^-lsp.
template <bool RESIDUAL, bool FULL>
__device__ __forceinline__ void race_group(const float zp[4], const float zq[4],
                                           const RaceRow& rr, int64_t g, int64_t v_end,
                                           uint32_t b, uint32_t k0, uint32_t k1, float& bw,
                                           float& be, int& bidx) {
  const Philox4 r = philox_race(static_cast<uint32_t>(g), static_cast<uint32_t>(rr.n), b, 0u, k0, k1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int v = static_cast<int>(g) * 4 + k;
    if (!FULL && v >= v_end) break;
    const float e = -fast_log2(uniform_open01(r.w[k]));  // E / ln 2
    float w;
    if constexpr (RESIDUAL) {
      w = fast_exp2(log2_weight(zp[k], rr.cf, rr.mp) - rr.lsp) -
          fast_exp2(log2_weight(zq[k], rr.cf, rr.mq) - rr.lsq);
    } else {
      w = fast_exp2(log2_weight(zp[k], rr.cf, rr.mp));
    }
    if (w * be > bw * e) {
      bw = w;
      be = e;
      bidx = v;
    }
  }
}

// A thread's best as a float key for merging (-inf when it has none).
__device__ __forceinline__ float race_key(float bw, float be, int bidx) {
  return bidx == INT_MAX ? -INFINITY : bw / be;
}

// 4 logits at v (a multiple of 4) with one vector load (vector path only).
template <bool BF16>
__device__ __forceinline__ void load4v(const void* rowp, int64_t v, float out[4]) {
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(rowp) + v);
    out[0] = bf16_lo(w.x);
    out[1] = bf16_hi(w.x);
    out[2] = bf16_lo(w.y);
    out[3] = bf16_hi(w.y);
  } else {
    const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(rowp) + v);
    out[0] = w.x;
    out[1] = w.y;
    out[2] = w.z;
    out[3] = w.w;
  }
}

// Race over chunk c of row n: this thread's (key, index) merged into (key, idx).
// A chunk wholly inside the row (vector path) takes unconditional loads and no
// per-token bounds; the last chunk of a row checks every group and token.
template <bool BF16, bool VEC, bool RESIDUAL>
__device__ __forceinline__ void race_chunk(const Params& p, int b, int c, const void* prow,
                                           const void* qrow, const RaceRow& rr, float& key,
                                           int& idx) {
  constexpr int CHUNK = chunk_tokens(BF16);
  constexpr int G = CHUNK / (4 * kThreads);  // 4-token groups per thread
  const int tid = threadIdx.x;
  const int64_t v_end = min(static_cast<int64_t>(c + 1) * CHUNK, static_cast<int64_t>(p.V));
  const int64_t g0 = static_cast<int64_t>(c) * (CHUNK / 4);
  float zp[G][4], zq[G][4];
  float bw = 0.f, be = 1.f;  // any w > 0 beats the empty candidate
  int bi = INT_MAX;
  if (VEC && static_cast<int64_t>(c + 1) * CHUNK <= p.V) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {  // issue every load before any math
      const int64_t g = g0 + gi * kThreads + tid;
      load4v<BF16>(prow, g * 4, zp[gi]);
      if (RESIDUAL) load4v<BF16>(qrow, g * 4, zq[gi]);
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
      race_group<RESIDUAL, true>(zp[gi], zq[gi], rr, g0 + gi * kThreads + tid, v_end,
                                 static_cast<uint32_t>(b), p.k0, p.k1, bw, be, bi);
  } else {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int64_t g = g0 + gi * kThreads + tid;
#pragma unroll
      for (int k = 0; k < 4; ++k) zq[gi][k] = 0.f;
      if (g * 4 < v_end) {
        load4<BF16, VEC>(prow, g * 4, v_end, zp[gi]);
        if (RESIDUAL) load4<BF16, VEC>(qrow, g * 4, v_end, zq[gi]);
      }
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int64_t g = g0 + gi * kThreads + tid;
      if (g * 4 < v_end)
        race_group<RESIDUAL, false>(zp[gi], zq[gi], rr, g, v_end, static_cast<uint32_t>(b), p.k0,
                                    p.k1, bw, be, bi);
    }
  }
  merge_argmax(key, idx, race_key(bw, be, bi), bi);
}

// Race over two whole chunks c, c + 1 inside the row (vector path): every
// load of both is issued first, kept packed (4 logits per 8 bytes for bf16),
// so the second chunk's loads do not wait behind the first chunk's math.
// Each chunk still reduces to its own per-thread key, as in race_chunk.
template <bool BF16, bool RESIDUAL>
__device__ __forceinline__ void race_pair(const Params& p, int b, int c, const void* prow,
                                          const void* qrow, const RaceRow& rr, float& key,
                                          int& idx) {
  constexpr int CHUNK = chunk_tokens(BF16);
  constexpr int G = CHUNK / (4 * kThreads);
  using Raw = typename std::conditional<BF16, uint2, uint4>::type;
  const int tid = threadIdx.x;
  const Raw* pr = static_cast<const Raw*>(prow);
  const Raw* qr = static_cast<const Raw*>(qrow);
  Raw rp[2][G], rq[2][G];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int64_t g = static_cast<int64_t>(c + h) * (CHUNK / 4) + gi * kThreads + tid;
      rp[h][gi] = pr[g];
      if (RESIDUAL) rq[h][gi] = qr[g];
    }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float bw = 0.f, be = 1.f;
    int bi = INT_MAX;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int64_t g = static_cast<int64_t>(c + h) * (CHUNK / 4) + gi * kThreads + tid;
      float zp[4], zq[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
        zp[0] = bf16_lo(rp[h][gi].x);
        zp[1] = bf16_hi(rp[h][gi].x);
        zp[2] = bf16_lo(rp[h][gi].y);
        zp[3] = bf16_hi(rp[h][gi].y);
        if (RESIDUAL) {
          zq[0] = bf16_lo(rq[h][gi].x);
          zq[1] = bf16_hi(rq[h][gi].x);
          zq[2] = bf16_lo(rq[h][gi].y);
          zq[3] = bf16_hi(rq[h][gi].y);
        }
      } else {
        zp[0] = __uint_as_float(rp[h][gi].x);
        zp[1] = __uint_as_float(rp[h][gi].y);
        zp[2] = __uint_as_float(rp[h][gi].z);
        zp[3] = __uint_as_float(rp[h][gi].w);
        if (RESIDUAL) {
          zq[0] = __uint_as_float(rq[h][gi].x);
          zq[1] = __uint_as_float(rq[h][gi].y);
          zq[2] = __uint_as_float(rq[h][gi].z);
          zq[3] = __uint_as_float(rq[h][gi].w);
        }
      }
      race_group<RESIDUAL, true>(zp, zq, rr, g, static_cast<int64_t>(p.V),
                                 static_cast<uint32_t>(b), p.k0, p.k1, bw, be, bi);
    }
    merge_argmax(key, idx, race_key(bw, be, bi), bi);
  }
}

template <bool BF16, bool VEC>
__device__ void finish_sampled(const Params& p, int b, const Req& r, const RaceRow& rr,
                               bool bad, bool fold_expired, int32_t x);

// Race of sampled request b over the chunks of group cg.  x holds draft token
// t = threadIdx.x of request b for t < K (loaded at the start of the workgroup).
template <bool BF16, bool VEC>
__device__ void race_part(const Params& p, int b, int cg, const Req& r, int32_t x) {
  __shared__ FoldShared sh;
  __shared__ int sh_n;
  __shared__ float sh_key[kWaves];
  __shared__ int sh_idx[kWaves];
  const int tid = threadIdx.x;
  const int K = r.K;
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  const int64_t drow0 = r.off0;
  const int64_t esz = BF16 ? 2 : 4;
  const float cf = kLog2e / r.T;

  // gather z at x_t now, so the loads overlap the wait for the partials
  float zp = 0.f, zq = 0.f;
  bool bad_token = false;
  if (tid < K) {
    if (x < 0 || x >= p.V) {
      bad_token = true;
    } else {
      zp = load_logit<BF16>(p.target, (trow0 + tid) * p.V + x);
      zq = load_logit<BF16>(p.draft, (drow0 + tid) * p.V + x);
    }
  }
  fold_rows<false>(p, b, K, 2 * K + 1, cf, sh);
  SV_STAMP(4);  // race: partials folded
  const bool any_bad_token = __syncthreads_or(bad_token) != 0;
  const bool bad = (sh.bad & 1) || any_bad_token;
  const bool expired = (sh.bad & 2) != 0;

  RaceRow rr{};
  rr.cf = cf;
  float key = -INFINITY;
  int idx = INT_MAX;
  if (!bad && !expired) {
    // ratio test r_t * q_t(x_t) < p_t(x_t), left to right (wave 0 holds t < K <= 8)
    bool reject = false;
    if (tid < K) {
      const float pp =
          fast_exp2(log2_weight(zp, cf, sh.row_m[tid]) - sh.row_ls[tid]);
      const float qq = fast_exp2(log2_weight(zq, cf, sh.row_m[K + 1 + tid]) -
                                 sh.row_ls[K + 1 + tid]);
      const float u = uniform_open01(philox4x32_10(0u, tid, b, 1u, p.k0, p.k1).w[0]);
      reject = !(u * qq < pp);
      if (cg == 0) {
        if (p.p_at) p.p_at[drow0 + tid] = pp;
        if (p.q_at) p.q_at[drow0 + tid] = qq;
      }
    }
    const uint64_t mask = __ballot(reject);
    if (tid == 0) sh_n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : K;
    __syncthreads();
    // workgroup-uniform values read from LDS: keep them in scalar registers
    rr.n = uniform_int(sh_n);
    SV_STAMP(5);  // race: ratio tests done, n known
    rr.mp = uniform_float(sh.row_m[rr.n]);
    rr.lsp = uniform_float(sh.row_ls[rr.n]);
    if (rr.n < K) {
      rr.mq = uniform_float(sh.row_m[K + 1 + rr.n]);
      rr.lsq = uniform_float(sh.row_ls[K + 1 + rr.n]);
    }
    const void* prow = static_cast<const char*>(p.target) + (trow0 + rr.n) * p.V * esz;
    const int c_first = cg * p.mr;
    const int c_end = min(c_first + p.mr, p.nc);
    constexpr int CHUNK = chunk_tokens(BF16);
    int c = c_first;
    if (rr.n < K) {
      const void* qrow = static_cast<const char*>(p.draft) + (drow0 + rr.n) * p.V * esz;
      if (VEC)
        for (; c + 1 < c_end && static_cast<int64_t>(c + 2) * CHUNK <= p.V; c += 2)
          race_pair<BF16, true>(p, b, c, prow, qrow, rr, key, idx);
      for (; c < c_end; ++c) race_chunk<BF16, VEC, true>(p, b, c, prow, qrow, rr, key, idx);
    } else {
      if (VEC)
        for (; c + 1 < c_end && static_cast<int64_t>(c + 2) * CHUNK <= p.V; c += 2)
          race_pair<BF16, false>(p, b, c, prow, nullptr, rr, key, idx);
      for (; c < c_end; ++c) race_chunk<BF16, VEC, false>(p, b, c, prow, nullptr, rr, key, idx);
    }
  }
  SV_STAMP(6);  // race: this workgroup's chunks raced
  block_argmax(key, idx, sh_key, sh_idx);
  if (tid == 0)
    slot_store(p.race + static_cast<int64_t>(b) * p.ngr + cg,
               pack_slot(key, expired ? kExpiredIdx : static_cast<uint32_t>(idx)));
  SV_STAMP(7);  // race: winner stored
  // the request's last race workgroup finishes it
  if (cg == p.ngr - 1) finish_sampled<BF16, VEC>(p, b, r, rr, bad, expired, x);
}

// The last race workgroup of request b: folds the workgroup winners, writes
// the outputs and clears the request's slots.  x is draft token t = threadIdx.x
// (t < K), loaded when the workgroup started, so the outputs need no load.
template <bool BF16, bool VEC>
__device__ void finish_sampled(const Params& p, int b, const Req& r, const RaceRow& rr,
                               bool bad, bool fold_expired, int32_t x) {
  __shared__ float sh_key[kWaves];
  __shared__ int sh_idx[kWaves];
  __shared__ int sh_expired;
  const int tid = threadIdx.x;
  if (tid == 0) sh_expired = fold_expired ? 1 : 0;
  __syncthreads();
  float key = -INFINITY;
  int idx = INT_MAX;
  for (int i = tid; i < p.ngr; i += kThreads) {
    uint64_t* slot = p.race + static_cast<int64_t>(b) * p.ngr + i;
    const uint64_t v = slot_wait(slot);
    slot_store(slot, 0u);
    if (v == 0u || slot_w(v) == kExpiredIdx) {
      atomicOr(&sh_expired, 1);
      continue;
    }
    merge_argmax(key, idx, slot_f(v), static_cast<int>(slot_w(v)));
  }
  block_argmax(key, idx, sh_key, sh_idx);  // its barriers also publish sh_expired
  SV_STAMP(8);  // finisher: every winner collected
  clear_request(p, b, r.K, 2 * r.K + 1);
  if (sh_expired) {
    if (tid == 0) p.accept_len[b] = -1;
    return;
  }
  if (bad) {
    write_fault(p, b, r);
    return;
  }
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  if (idx == INT_MAX) {
    // no token had p > q (rounding can only cause this when p == q): race on p_n
    const int64_t esz = BF16 ? 2 : 4;
    const void* prow = static_cast<const char*>(p.target) + (trow0 + rr.n) * p.V * esz;
    float bw = 0.f, be = 1.f;
    int bi = INT_MAX;
    for (int64_t g = tid; g * 4 < p.V; g += kThreads) {
      float zp[4];
      const float zq[4] = {0.f, 0.f, 0.f, 0.f};
      load4<BF16, VEC>(prow, g * 4, p.V, zp);
      race_group<false, false>(zp, zq, rr, g, p.V, static_cast<uint32_t>(b), p.k0, p.k1, bw, be,
                               bi);
    }
    key = race_key(bw, be, bi);
    idx = bi;
    block_argmax(key, idx, sh_key, sh_idx);
  }
  const int n = rr.n;
  if (tid <= r.K) p.out_tokens[trow0 + tid] = (tid < n) ? x : (tid == n ? idx : -1);
  if (tid == 0) p.accept_len[b] = n;
  SV_STAMP(9);  // finisher: outputs written
}

// ------------------------------------------------------------------ kernel

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sv_verify(Params p) {
  // Grid order, with L = lag: the statistics of requests 0..L-1 (ng workgroups
  // each); then, for k = L..B-1, the statistics of request k followed by the
  // ngr race workgroups of request k - L; then the races of the last L
  // requests.  A request's races thus follow its statistics by about L ng
  // workgroups, and every race has workgroups of its own.
  const int g = blockIdx.x;
  const int L = p.lag, seg = p.ng + p.ngr;
  int b1 = p.B, cg = 0, b2 = -1, rc = 0;
  if (g < L * p.ng) {
    b1 = g / p.ng;
    cg = g - b1 * p.ng;
  } else if (g < L * p.ng + (p.B - L) * seg) {
    const int t = g - L * p.ng;
    const int k = L + t / seg;
    const int tt = t - (k - L) * seg;
    if (tt < p.ng) {
      b1 = k;
      cg = tt;
    } else {
      b2 = k - L;
      rc = tt - p.ng;
    }
  } else {
    const int t = g - L * p.ng - (p.B - L) * seg;
    b2 = p.B - L + t / p.ngr;
    rc = t - (b2 - (p.B - L)) * p.ngr;
  }
  SV_STAMP(1);  // workgroup started
  // the race request's draft tokens, loaded before anything waits
  Req r2{};
  bool race = false;
  int32_t x = 0;
  if (b2 >= 0 && b2 < p.B) {
    SV_TRACE_HEAD(2, b2, rc);
    r2 = load_req(p, b2);
    SV_STAMP(2);  // the request's scalars loaded
    race = r2.sampled();
    if (race && static_cast<int>(threadIdx.x) < r2.K) x = p.tokens[r2.off0 + threadIdx.x];
  }
  if (b1 < p.B) stats_part<BF16, VEC>(p, b1, cg);
  if (race) race_part<BF16, VEC>(p, b2, rc, r2, x);
}

// ------------------------------------------------------------------ host side

bool shape_ok(int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows) {
  return B >= 1 && V >= 1 && max_k >= 0 && max_k <= SV_KMAX && n_draft_rows >= 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }


size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct Layout {
  size_t part_off, race_off, total;
};

// Sized with the float32 chunk (the smaller one, so more chunks) so that
// either dtype fits.
Layout make_layout(int32_t B, int32_t V, int32_t max_k) {
  const size_t nc = static_cast<size_t>(ceil_div(V, chunk_tokens(false)));
  Layout L;
  L.part_off = 0;
  L.race_off = round256(static_cast<size_t>(B) * (2 * max_k + 1) * nc * sizeof(uint64_t));
  L.total = L.race_off + round256(static_cast<size_t>(B) * nc * sizeof(uint64_t));
  return L;
}

// Chunks per workgroup: enough rows x chunks that a workgroup streams about
// 64 KiB (8 row-chunks) when the request reads all its rows.
int chunks_per_workgroup(int rows, int nc) {
  int m = 1;
  while (m < 8 && rows * m < 8) m *= 2;
  return std::max(1, std::min(m, nc));
}

template <bool BF16, bool VEC>
int launch(const Params& prm, int64_t grid, hipStream_t stream, void* ev0, void* ev1) {
  if (ev0 && hipEventRecord(static_cast<hipEvent_t>(ev0), stream) != hipSuccess)
    return SV_ERR_LAUNCH;
  hipLaunchKernelGGL((sv_verify<BF16, VEC>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads),
                     0, stream, prm);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  if (ev1 && hipEventRecord(static_cast<hipEvent_t>(ev1), stream) != hipSuccess)
    return SV_ERR_LAUNCH;
  return SV_OK;
}

int dispatch(const void* target, const void* draft, int32_t dtype, int32_t B, int32_t V,
             int32_t max_k, int32_t n_draft_rows, const int32_t* offsets, const int32_t* tokens,
             const float* temperature, uint64_t seed, int32_t* accept_len, int32_t* out_tokens,
             float* p_at, float* q_at, void* workspace, size_t workspace_bytes, void* stream,
             bool all_greedy, void* ev0, void* ev1) {
  if (!target || !offsets || !accept_len || !out_tokens || !workspace) return SV_ERR_NULL;
  if (!all_greedy && (!temperature || (n_draft_rows > 0 && !draft))) return SV_ERR_NULL;
  if (n_draft_rows > 0 && !tokens) return SV_ERR_NULL;
  if (!shape_ok(B, V, max_k, n_draft_rows)) return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (workspace_bytes < spec_verify_workspace_bytes(B, V, max_k) || !aligned16(workspace))
    return SV_ERR_WORKSPACE;
  const bool bf16 = dtype == SV_BF16;
  const Layout L = make_layout(B, V, max_k);
  char* ws = static_cast<char*>(workspace);
  Params prm;
  prm.target = target;
  prm.draft = all_greedy ? nullptr : draft;
  prm.offsets = offsets;
  prm.tokens = tokens;
  prm.temperature = all_greedy ? nullptr : temperature;
  prm.k0 = static_cast<uint32_t>(seed);
  prm.k1 = static_cast<uint32_t>(seed >> 32);
  prm.B = B;
  prm.V = V;
  prm.max_k = max_k;
  prm.n_draft_rows = n_draft_rows;
  prm.nc = static_cast<int32_t>(ceil_div(V, chunk_tokens(bf16)));
  // Flat grouping when every request has max_k drafts: each workgroup then
  // streams one full round of row-chunks.  With ragged draft lengths it would
  // leave the shorter requests' surplus workgroups empty, so column grouping
  // (one chunk column of every row per workgroup) is used instead.
  const int rows = all_greedy ? max_k + 1 : 2 * max_k + 1;
  prm.flat = static_cast<int64_t>(n_draft_rows) == static_cast<int64_t>(B) * max_k;
  if (prm.flat) {
    prm.m = 1;
    // one canonical block (8 chunks of one row) per statistics workgroup
    prm.ng = static_cast<int32_t>(static_cast<int64_t>(rows) * ceil_div(prm.nc, kGroupItems));
    // race chunks per race workgroup: at least two, and enough that a
    // request has at most half as many race workgroups as statistics
    // workgroups.  Few rows per request (MTP, K = 1) then get wide races:
    // fewer workgroups folding the same partials, and fewer empty ones for
    // the greedy requests (B=512 K=1: 11 race workgroups per request -> 6,
    // 82.0 -> 77.8 us; B=64 K=4 and B=256 K=8 keep two chunks)
    prm.mr = static_cast<int32_t>(
        std::min<int64_t>(prm.nc, std::max<int64_t>(2, ceil_div(2 * prm.nc, prm.ng))));
  } else {
    prm.m = chunks_per_workgroup(rows, prm.nc);
    prm.ng = static_cast<int32_t>(ceil_div(prm.nc, prm.m));
    // about six chunks per race workgroup (B=1024 ragged: 494 -> 483 us
    // against four; five to eight measured within noise of six or worse)
    prm.mr = std::min(prm.nc, prm.m * std::max(1, 6 / prm.m));
  }
  prm.ngr = static_cast<int32_t>(ceil_div(prm.nc, prm.mr));
  // Workgroups go to the XCDs round robin by grid index, and a request's race
  // workgroups sit ng + ngr after the previous request's.  With fewer race
  // workgroups than XCDs and ng + ngr a multiple of the XCD count, every
  // request's races would run on the same few XCDs (B=512 K=1 with four race
  // workgroups of 8 or 9 chunks: 121-131 us, against 78-81 us with five or
  // six of 6 or 7 chunks), so the race is narrowed until they rotate.
  while (prm.ngr < kXcds && (prm.ng + prm.ngr) % kXcds == 0 && prm.mr > 1) {
    --prm.mr;
    prm.ngr = static_cast<int32_t>(ceil_div(prm.nc, prm.mr));
  }
  // Race placement.  A race workgroup polls, holding its slot, until its
  // request's statistics are in; placed too early it idles a slot the stream
  // needs, too late it starts the request's dependent chain late.  The lag,
  // in workgroups between a request's statistics and its races, was tuned
  // on MI355X: about 0.55 of a resident generation (5 workgroups per CU)
  // with flat grouping (0.45 -> 0.55 once the fold reads merged block
  // partials: B=64 K=4 29.35 -> 28.93 us, B=512 K=1 78.2 -> 77.5 us),
  // 1.2 with column grouping (ragged batches).  An
  // all-greedy call has no races: lag = B puts every statistics workgroup
  // first and the grid ends there.
  const int64_t resident = kWorkgroupsPerCu * device_compute_units();
  const int64_t lag_wgs = prm.flat ? resident * 11 / 20 : resident * 6 / 5;
  prm.lag = all_greedy ? B
                       : static_cast<int32_t>(std::min<int64_t>(
                             B, std::max<int64_t>(1, ceil_div(lag_wgs, prm.ng))));
  prm.part = reinterpret_cast<uint64_t*>(ws + L.part_off);
  prm.race = reinterpret_cast<uint64_t*>(ws + L.race_off);
  prm.accept_len = accept_len;
  prm.out_tokens = out_tokens;
  prm.p_at = p_at;
  prm.q_at = q_at;
  // all-greedy calls have no races, so no race-only tail
  // every request has ngr race workgroups (they find nothing to do for a
  // greedy request); an all-greedy call has none
  const int64_t grid = static_cast<int64_t>(B) * prm.ng +
                       (all_greedy ? 0 : static_cast<int64_t>(B) * prm.ngr);
  if (grid <= 0 || grid > INT32_MAX) return SV_ERR_SHAPE;
  const int64_t row_bytes = static_cast<int64_t>(V) * (bf16 ? 2 : 4);
  const bool vec = row_bytes % 16 == 0 && aligned16(target) && (!draft || aligned16(draft));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch<true, true>(prm, grid, s, ev0, ev1)
               : launch<true, false>(prm, grid, s, ev0, ev1);
  return vec ? launch<false, true>(prm, grid, s, ev0, ev1)
             : launch<false, false>(prm, grid, s, ev0, ev1);
}

// ------------------------------------------------------------------ static scratch
//
// Hand-off slots of spec_verify_sample_static, the variant for callers that
// cannot allocate device memory.  The array lives in the code object: every
// device the library runs on holds one copy of kScratchBytes until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = SV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

__global__ __launch_bounds__(kThreads) void sv_zero_fill(uint4* p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchSlot {
  void* ptr = nullptr;   // device address of `scratch` on this device
  bool cleared = false;  // a zero fill of the whole array has been enqueued
};

// Looks up (once per device, with that device current) the device address of
// `scratch`; enqueues a zero fill of the whole array on the first call on a
// device, or of the first `clear_bytes` bytes when `clear_bytes` > 0.
int static_scratch(hipStream_t stream, size_t clear_bytes, void** out) {
  constexpr int kMaxDevices = 64;
  static ScratchSlot slots[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(mu);
  ScratchSlot& sl = slots[dev];
  if (!sl.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_LAUNCH;
    sl.ptr = p;
  }
  if (!sl.cleared) clear_bytes = kScratchBytes;
  if (clear_bytes > 0) {
    const int64_t n = static_cast<int64_t>(round256(std::min(clear_bytes, kScratchBytes)) / 16);
    const int64_t grid = std::min<int64_t>(ceil_div(n, kThreads), 4 * device_compute_units());
    hipLaunchKernelGGL(sv_zero_fill, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream,
                       static_cast<uint4*>(sl.ptr), n);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    sl.cleared = true;
  }
  *out = sl.ptr;
  return SV_OK;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_bytes(int32_t B, int32_t V, int32_t max_k) {
  if (!shape_ok(B, V, max_k, 0)) return 0;
  return make_layout(B, V, max_k).total;
}

int spec_verify_greedy(const void* target_logits, int32_t dtype, int32_t B, int32_t V,
                       int32_t max_k, int32_t n_draft_rows, const int32_t* draft_offsets,
                       const int32_t* draft_tokens, int32_t* accept_len, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return dispatch(target_logits, nullptr, dtype, B, V, max_k, n_draft_rows, draft_offsets,
                  draft_tokens, nullptr, 0, accept_len, out_tokens, nullptr, nullptr, workspace,
                  workspace_bytes, stream, true, nullptr, nullptr);
}

int spec_verify_sample(const void* target_logits, const void* draft_logits, int32_t dtype,
                       int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows,
                       const int32_t* draft_offsets, const int32_t* draft_tokens,
                       const float* temperature, uint64_t seed, int32_t* accept_len,
                       int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return dispatch(target_logits, draft_logits, dtype, B, V, max_k, n_draft_rows, draft_offsets,
                  draft_tokens, temperature, seed, accept_len, out_tokens, p_at_draft,
                  q_at_draft, workspace, workspace_bytes, stream, false, nullptr, nullptr);
}

int spec_verify_sample_timed(const void* target_logits, const void* draft_logits, int32_t dtype,
                             int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows,
                             const int32_t* draft_offsets, const int32_t* draft_tokens,
                             const float* temperature, uint64_t seed, int32_t* accept_len,
                             int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* event_start, void* event_end) {
  if (!event_start || !event_end) return SV_ERR_NULL;
  return dispatch(target_logits, draft_logits, dtype, B, V, max_k, n_draft_rows, draft_offsets,
                  draft_tokens, temperature, seed, accept_len, out_tokens, p_at_draft,
                  q_at_draft, workspace, workspace_bytes, stream, false, event_start, event_end);
}

int spec_verify_sample_static(const void* target_logits, const void* draft_logits, int32_t dtype,
                              int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows,
                              const int32_t* draft_offsets, const int32_t* draft_tokens,
                              const float* temperature, uint64_t seed, int32_t* accept_len,
                              int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                              int32_t clear_scratch, void* stream) {
  if (!target_logits || !draft_offsets || !accept_len || !out_tokens || !temperature ||
      (n_draft_rows > 0 && (!draft_logits || !draft_tokens)))
    return SV_ERR_NULL;
  if (!shape_ok(B, V, max_k, n_draft_rows)) return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  const size_t need = spec_verify_workspace_bytes(B, V, max_k);
  if (need == 0 || need > kScratchBytes) return SV_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int rc = static_scratch(s, clear_scratch ? need : 0, &ws);
  if (rc != SV_OK) return rc;
  return dispatch(target_logits, draft_logits, dtype, B, V, max_k, n_draft_rows, draft_offsets,
                  draft_tokens, temperature, seed, accept_len, out_tokens, p_at_draft,
                  q_at_draft, ws, kScratchBytes, stream, false, nullptr, nullptr);
}

#ifdef SV_TRACE
// Trace build only (not part of the product ABI): copy the first n_words
// words of the stage records to host memory, or zero them all (reset).
int spec_verify_trace_copy(uint64_t* host, size_t n_words) {
  n_words = std::min(n_words, static_cast<size_t>(kTraceWgs) * kTracePoints);
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(sv_trace), n_words * sizeof(uint64_t)) ==
                 hipSuccess
             ? 0
             : -1;
}
int spec_verify_trace_reset(void) {
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(sv_trace)) != hipSuccess) return -1;
  return hipMemset(ptr, 0, sizeof(uint64_t) * kTraceWgs * kTracePoints) == hipSuccess ? 0 : -1;
}
int spec_verify_trace_points(void) { return kTracePoints; }
#endif

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "bad shape (B, V, max_k or n_draft_rows) or grid too large";
    case SV_ERR_DTYPE: return "unknown dtype";
    case SV_ERR_WORKSPACE: return "workspace too small or not 16-byte aligned";
    case SV_ERR_LAUNCH: return "kernel launch failed";
    case SV_ERR_SCRATCH:
      return "sizes need more hand-off slots than the static scratch holds "
             "(SV_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
