// spec_verify.hip -- gfx950 kernel and C ABI of the speculative-decoding verify step.
//
// What is computed is stated in include/spec_verify.h (the accept / residual /
// bonus rule of "Decodificación Especulativa y EAGLE", section "La Regla de
// Exactitud", and its greedy case).  How it runs on MI355X: one launch of
// persistent workgroups that take work items from per-list ticket counters.
//
// Work items of request b:
//   SA  statistics of a sampled request: one item per (row, 64 KiB V-chunk) of
//       its K+1 target and K draft rows.  Streams the chunk with 16-byte
//       loads and reduces it to one 8-byte partial (max, sum of
//       2^(z c - fl(max c))), c = log2(e) / T.
//   SG  statistics of a greedy request: (max, lowest argmax index) per chunk
//       of its K+1 target rows (draft rows are never read).
//   FA  finisher of a sampled request: folds the partials into per-row
//       (max, log2 sum), gathers p_t(x_t) and q_t(x_t), draws r_t, finds the
//       first rejection n with a wave ballot, and publishes n with the
//       statistics of row n.
//   R   race of a sampled request: one item per 4096-token chunk of row n, the
//       exponential race over the residual (p_n - q_n)+ after a rejection or
//       over p_K otherwise, plus one item that folds the chunk winners and
//       writes the outputs.
//   FG  finisher of a greedy request: first draft that differs from the row
//       argmax; writes the outputs.  Also reports a request whose slice or
//       temperature is invalid.
//
// Work lists: request b belongs to list b mod 8, served by the workgroups with
// blockIdx mod 8 equal to the list (on MI355X those sit on one XCD, so a
// request's hand-offs stay in one L2, though nothing relies on that).  Every
// workgroup of a list builds the same plan in LDS from the requests' offsets
// and temperatures: the list's items laid out by "time step" -- SA of the
// list's i-th request at step i, SG at step nloc + i (after every sampled
// request), FA at i + d1, R at i + d1 + d2, FG at the SG step + d3, and inside
// a step the order SA, SG, FA, R, FG.  The lags (about two generations of the
// list's workgroups) put consumers well after their producers, so finishing
// and races overlap the streaming of other rows.  A workgroup draws tickets
// from the list's counter and processes item ticket by ticket.
//
// Forward progress needs no assumption about dispatch or residency: an item
// only waits for items of the same list with smaller tickets, and a ticket is
// only handed out to a running workgroup, so by induction on the ticket every
// wait ends.  Waits are also bounded (kSpinLimit polls); an expired wait
// reports accept_len = -1.
//
// Hand-offs between workgroups use 8-byte slots in the workspace that are
// all-zero until written (a written slot never has all-zero bits: +0.0 is
// stored as -0.0).  Producers store with a device-coherent (sc1) store;
// consumers poll with device-coherent loads, then write the slot back to
// zero.  No agent-scope release/acquire fence is used (on gfx950 those write
// back or invalidate the XCD's whole L2).  The last workgroup of a list to
// exit resets the list's counters, so the workspace is all-zero again after
// every call.
//
// Race keys: the winner maximises ln w_v - ln E_v, i.e. w_v / E_v.  Inside a
// thread candidates are compared by cross-multiplication (w_a e_b > w_b e_a)
// with e = -log2 U = E / ln 2 (a common factor); a thread's best becomes the
// float key w / e for the merges across threads, waves and chunks.  Weights
// are 2^(z c - fl(m c)) with fl(m c) the rounded product for the row maximum
// m; the same rounded offset is used when the row's sum is formed, so it
// cancels exactly from p = w / sum.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;  // 4 wave64s per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kStatsVecs = 16;  // 16-byte loads per thread per statistics chunk
constexpr int kRaceGroups = 4;  // 4-token Philox groups per thread per race chunk
constexpr int kRaceChunk = kThreads * kRaceGroups * 4;  // tokens per race chunk
constexpr int kRowsMax = 2 * SV_KMAX + 1;               // row slots per request
constexpr int kRowsPerWave = (kRowsMax + kWaves - 1) / kWaves;
constexpr unsigned kSpinLimit = 1u << 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLists = 8;                       // work lists (one per XCD on MI355X)
constexpr int kMaxLocal = 512;                  // requests per list and launch
constexpr int kMaxSteps = 4 * kMaxLocal;        // time steps a list's plan can span
constexpr int kCounterStride = 16;              // 64-byte lines between counters

__host__ __device__ constexpr int elems_per_vec(bool bf16) { return bf16 ? 8 : 4; }
__host__ __device__ constexpr int stats_chunk(bool bf16) {
  return kThreads * kStatsVecs * elems_per_vec(bf16);
}

// ------------------------------------------------------------------ helpers

// threadIdx.x behind an empty asm: work items run in a loop, and without this
// the compiler hoists every per-thread address offset of every item kind out
// of the loop, where they stay live and triple the register footprint.
__device__ __forceinline__ int item_tid() {
  int t = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <bool BF16>
__device__ __forceinline__ float load_logit(const void* base, int64_t i) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
  } else {
    return static_cast<const float*>(base)[i];
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Philox4x32-10 (Salmon et al., SC'11): ten rounds, each two 32x32->64
// products; the key advances by the Weyl constants between rounds.
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t d = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t n0 = static_cast<uint32_t>(d >> 32) ^ c1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(a >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(d);
    c3 = static_cast<uint32_t>(a);
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// (2 * (x >> 9) + 1) * 2^-24, exact in float32, strictly inside (0, 1).
__device__ __forceinline__ float uniform_open01(uint32_t x) {
  return __fmaf_rn(static_cast<float>(x >> 9), 0x1p-23f, 0x1p-24f);
}

// fl(m * c): the row-maximum offset, rounded once (the build disables
// contraction), so every place that needs it gets the identical float.
__device__ __forceinline__ float scaled_max(float m, float cf) { return m * cf; }

// log2 of the unnormalised weight 2^(z c - fl(m c)).
__device__ __forceinline__ float scaled_logit(float z, float cf, float mc) {
  return __fmaf_rn(z, cf, -mc);
}

// (max, sum) pairs; a sum s is relative to fl(max * c).  Larger max wins and
// the other sum is rescaled by 2^(fl(m c) - fl(M c)).  A side with max == -inf
// contributes 0 * s, which keeps a NaN sum NaN.
__device__ __forceinline__ void merge_stats(float& m, float& s, float m2, float s2, float cf) {
  const float M = fmaxf(m, m2);
  const float Mc = scaled_max(M, cf);
  const float f1 = (m == -INFINITY) ? 0.f : fast_exp2(scaled_max(m, cf) - Mc);
  const float f2 = (m2 == -INFINITY) ? 0.f : fast_exp2(scaled_max(m2, cf) - Mc);
  s = s * f1 + s2 * f2;
  m = M;
}

// Larger value wins; equal values keep the lower index.
__device__ __forceinline__ void merge_argmax(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ __forceinline__ void wave_merge_stats(float& m, float& s, float cf) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    merge_stats(m, s, m2, s2, cf);
  }
}

__device__ __forceinline__ void wave_merge_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(v, o, 64);
    const int i2 = __shfl_xor(i, o, 64);
    merge_argmax(v, i, v2, i2);
  }
}

// All threads end with the workgroup's (key, idx) winner.
__device__ __forceinline__ void block_argmax(float& key, int& idx, float* sh_k, int* sh_i) {
  wave_merge_argmax(key, idx);
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  __syncthreads();
  if (lane == 0) {
    sh_k[wave] = key;
    sh_i[wave] = idx;
  }
  __syncthreads();
  key = sh_k[0];
  idx = sh_i[0];
  for (int w = 1; w < kWaves; ++w) merge_argmax(key, idx, sh_k[w], sh_i[w]);
}

// ------------------------------------------------------------------ hand-off slots

// (float, word) packed so a written slot is never all-zero bits.
__device__ __forceinline__ uint64_t pack_slot(float a, uint32_t b) {
  uint32_t ab = __float_as_uint(a);
  if (ab == 0u) ab = 0x80000000u;  // +0.0 -> -0.0 (equal as a number)
  return static_cast<uint64_t>(ab) | (static_cast<uint64_t>(b) << 32);
}
__device__ __forceinline__ float slot_f(uint64_t v) {
  return __uint_as_float(static_cast<uint32_t>(v));
}
__device__ __forceinline__ uint32_t slot_w(uint64_t v) { return static_cast<uint32_t>(v >> 32); }

__device__ __forceinline__ void slot_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t slot_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll until the slot is written; 0 if the bounded wait expires.
__device__ uint64_t slot_wait(const uint64_t* p) {
  uint64_t v = slot_load(p);
  for (unsigned it = 0; v == 0u && it < kSpinLimit; ++it) {
    __builtin_amdgcn_s_sleep(2);
    v = slot_load(p);
  }
  return v;
}

// Drain this thread's outstanding memory operations, so device-coherent
// stores made so far are visible before the next one.  The signal fences keep
// the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void drain_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------------------ workspace

enum : uint32_t { kStatusOk = 1, kStatusFault = 2 };

struct Layout {
  int J;    // row slots per request: target 0..max_k, then draft 0..max_k-1
  int nc1;  // statistics chunks per row
  int nc2;  // race chunks per row
  size_t count_off, stats_off, race_off, pub_off, total;
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

Layout make_layout(int32_t B, int32_t V, int32_t max_k, bool bf16) {
  Layout L;
  L.J = 2 * max_k + 1;
  L.nc1 = static_cast<int>(ceil_div(V, stats_chunk(bf16)));
  L.nc2 = static_cast<int>(ceil_div(V, kRaceChunk));
  L.count_off = 0;  // tickets [kLists] then exits [kLists], one 64-byte line each
  L.stats_off = round256(2 * kLists * kCounterStride * sizeof(uint32_t));
  // sized with the float32 chunk (the smaller one) so either dtype fits
  const size_t stats_bytes =
      static_cast<size_t>(B) * L.J * ceil_div(V, stats_chunk(false)) * sizeof(uint64_t);
  L.race_off = L.stats_off + round256(stats_bytes);
  L.pub_off = L.race_off + round256(static_cast<size_t>(B) * L.nc2 * sizeof(uint64_t));
  L.total = L.pub_off + round256(static_cast<size_t>(B) * 4 * sizeof(uint64_t));
  return L;
}

struct Params {
  const void* target;
  const void* draft;
  const int32_t* offsets;
  const int32_t* tokens;
  const float* temperature;  // NULL: every request greedy
  uint32_t k0, k1;           // Philox key
  int32_t b_begin, b_end;    // requests of this launch
  int32_t V, max_k, n_draft_rows, nc1, nc2, grid;
  uint32_t* counters;        // tickets [kLists], exits [kLists] (stride kCounterStride)
  uint64_t* part;            // [B][J][nc1] statistics partials
  uint64_t* race_part;       // [B][nc2] race chunk winners
  uint64_t* pub;             // [B][4] published record: (fl(m c), log2 sum) of target row n,
                             // the same of draft row n, (c, n), (1, status) -- last written
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_at;
  float* q_at;
};

// A request as the plan records it.
struct Req {
  int32_t off0, K;
  float T;
  bool slice_ok, temp_ok, greedy;
  __device__ bool sampled() const { return slice_ok && temp_ok && !greedy; }
  __device__ bool greedy_ok() const { return slice_ok && temp_ok && greedy; }
};

// Outputs of a failed request (its slice is valid).
__device__ void write_fault(const Params& p, int b, const Req& r) {
  const int tid = item_tid();
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  if (tid <= r.K) p.out_tokens[trow0 + tid] = -1;
  if (tid < r.K) {
    if (p.p_at) p.p_at[r.off0 + tid] = NAN;
    if (p.q_at) p.q_at[r.off0 + tid] = NAN;
  }
  if (tid == 0) p.accept_len[b] = -1;
}

// Row r of a request (target rows 0..K, then draft rows 0..K-1) to its slot.
__device__ __forceinline__ int row_slot(int max_k, int K, int r) {
  return r <= K ? r : max_k + r - K;
}

__device__ __forceinline__ uint64_t* part_slot(const Params& p, int b, int j, int c) {
  return p.part + (static_cast<int64_t>(b) * (2 * p.max_k + 1) + j) * p.nc1 + c;
}

// ------------------------------------------------------------------ plan

enum Kind : int { kSA = 0, kSG = 1, kFA = 2, kR = 3, kFG = 4, kKinds = 5 };

struct Plan {
  int32_t nloc;              // requests in this list
  int32_t steps;             // time steps
  int32_t total;             // items
  int32_t off[kKinds];       // time step of the list's first request, per kind
  int32_t off0[kMaxLocal];   // draft_offsets[b]
  int32_t info[kMaxLocal];   // K | slice_ok << 8 | temp_ok << 9 | greedy << 10
  float temp[kMaxLocal];
  int32_t P[kMaxSteps + 1];  // items before each time step
};

__device__ __forceinline__ Req make_req(int32_t info, int32_t off0, float T) {
  Req r;
  r.off0 = off0;
  r.K = info & 0xff;
  r.slice_ok = (info >> 8) & 1;
  r.temp_ok = (info >> 9) & 1;
  r.greedy = (info >> 10) & 1;
  r.T = T;
  return r;
}

// Request i of the plan, read by one thread.
__device__ __forceinline__ Req plan_req(const Plan& pl, int i) {
  return make_req(pl.info[i], pl.off0[i], pl.temp[i]);
}

// A value every lane of the wave holds, moved to a scalar register.  Plan
// entries read at a workgroup-uniform index are uniform, but the compiler
// cannot prove it for LDS loads; without this the item dispatch would be
// compiled as divergent control flow.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Request i of the plan, i uniform across the workgroup.
__device__ __forceinline__ Req plan_req_uniform(const Plan& pl, int i) {
  return make_req(uni(pl.info[i]), uni(pl.off0[i]), uni_f(pl.temp[i]));
}

__device__ __forceinline__ int kind_len(const Params& p, int kind, const Req& r) {
  switch (kind) {
    case kSA: return r.sampled() ? (2 * r.K + 1) * p.nc1 : 0;
    case kSG: return r.greedy_ok() ? (r.K + 1) * p.nc1 : 0;
    case kFA: return r.sampled() ? 1 : 0;
    case kR: return r.sampled() ? p.nc2 + 1 : 0;
    default: return r.sampled() ? 0 : 1;
  }
}

__device__ __forceinline__ int list_workgroups(const Params& p, int list) {
  return list < p.grid ? (p.grid - list + kLists - 1) / kLists : 0;
}

// Items of time step k (the request of kind j at step k is k - off[j]).
__device__ __forceinline__ int step_items(const Params& p, const Plan& pl, int k) {
  int n = 0;
  for (int j = 0; j < kKinds; ++j) {
    const int i = k - pl.off[j];
    if (i >= 0 && i < pl.nloc) n += kind_len(p, j, plan_req(pl, i));
  }
  return n;
}

// Every workgroup of a list computes the same plan.
__device__ void build_plan(const Params& p, int list, Plan& pl) {
  const int tid = threadIdx.x;
  const int first = p.b_begin + list;
  const int nloc = first < p.b_end ? (p.b_end - first + kLists - 1) / kLists : 0;
  int n_s = 0, n_g = 0, sum_s = 0, sum_g = 0;
  for (int i = tid; i < nloc; i += kThreads) {
    const int b = first + i * kLists;
    const int32_t o0 = p.offsets[b], o1 = p.offsets[b + 1];
    const int64_t K64 = static_cast<int64_t>(o1) - o0;
    const bool slice_ok = o0 >= 0 && o1 <= p.n_draft_rows && K64 >= 0 && K64 <= p.max_k;
    const int32_t K = slice_ok ? static_cast<int32_t>(K64) : 0;
    const float T = p.temperature ? p.temperature[b] : 0.f;
    const bool greedy = T == 0.f;
    const bool temp_ok = (T >= 0.f) && (T < INFINITY) && (greedy || K == 0 || p.draft != nullptr);
    const int Ks = K;
    pl.off0[i] = o0;
    pl.info[i] = Ks | (slice_ok << 8) | (temp_ok << 9) | (greedy << 10);
    pl.temp[i] = T;
    if (slice_ok && temp_ok) {
      if (greedy) {
        ++n_g;
        sum_g += (Ks + 1) * p.nc1;
      } else {
        ++n_s;
        sum_s += (2 * Ks + 1) * p.nc1;
      }
    }
  }
  // list totals
  __shared__ int sh_red[4][kWaves];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    n_s += __shfl_xor(n_s, o, 64);
    n_g += __shfl_xor(n_g, o, 64);
    sum_s += __shfl_xor(sum_s, o, 64);
    sum_g += __shfl_xor(sum_g, o, 64);
  }
  if ((tid & 63) == 0) {
    sh_red[0][tid >> 6] = n_s;
    sh_red[1][tid >> 6] = n_g;
    sh_red[2][tid >> 6] = sum_s;
    sh_red[3][tid >> 6] = sum_g;
  }
  __syncthreads();
  if (tid == 0) {
    int t[4] = {0, 0, 0, 0};
    for (int q = 0; q < 4; ++q)
      for (int w = 0; w < kWaves; ++w) t[q] += sh_red[q][w];
    const int64_t gen = list_workgroups(p, list);  // one generation of this list's workgroups
    const int64_t avg_s = std::max<int64_t>(1, t[2] / std::max(1, t[0]));
    const int64_t avg_g = std::max<int64_t>(1, t[3] / std::max(1, t[1]));
    const int64_t cap = 2 * static_cast<int64_t>(nloc);
    const int d1 = static_cast<int>(std::max<int64_t>(1, std::min(cap, ceil_div(2 * gen, avg_s))));
    const int d2 = static_cast<int>(
        std::max<int64_t>(1, std::min<int64_t>(nloc, ceil_div(gen, avg_s + p.nc2 + 1))));
    const int d3 = static_cast<int>(std::max<int64_t>(1, std::min(cap, ceil_div(2 * gen, avg_g))));
    pl.nloc = nloc;
    pl.off[kSA] = 0;
    pl.off[kSG] = t[0] > 0 ? nloc : 0;  // greedy statistics after the sampled ones
    pl.off[kFA] = d1;
    pl.off[kR] = d1 + d2;
    pl.off[kFG] = pl.off[kSG] + d3;
    int steps = 0;
    for (int j = 0; j < kKinds; ++j) steps = std::max(steps, pl.off[j] + nloc);
    pl.steps = nloc > 0 ? steps : 0;
  }
  __syncthreads();
  // P[k] = items before step k: per-thread runs of steps, then a block scan
  const int steps = pl.steps;
  const int per = (steps + kThreads - 1) / kThreads;
  const int k0 = tid * per, k1 = std::min(steps, k0 + per);
  int run = 0;
  for (int k = k0; k < k1; ++k) run += step_items(p, pl, k);
  int incl = run;  // inclusive scan of run across the workgroup
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if ((tid & 63) >= o) incl += v;
  }
  __shared__ int sh_wave[kWaves];
  if ((tid & 63) == 63) sh_wave[tid >> 6] = incl;
  __syncthreads();
  int base = incl - run;
  for (int w = 0; w < (tid >> 6); ++w) base += sh_wave[w];
  for (int k = k0; k < k1; ++k) {
    pl.P[k] = base;
    base += step_items(p, pl, k);
  }
  if (tid == kThreads - 1) {
    pl.P[steps] = base;
    pl.total = base;
  }
  __syncthreads();
}

// Ticket -> (kind, local request, index inside the request's items of that
// kind); t is uniform across the workgroup and so are the results.
__device__ void decode_ticket(const Params& p, const Plan& pl, int t, int& kind, int& i, int& o) {
  int lo = 0, hi = uni(pl.steps);  // largest k with P[k] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(pl.P[mid]) <= t)
      lo = mid;
    else
      hi = mid;
  }
  o = t - uni(pl.P[lo]);
  const int nloc = uni(pl.nloc);
  for (int j = 0; j < kKinds; ++j) {
    const int ii = lo - uni(pl.off[j]);
    if (ii < 0 || ii >= nloc) continue;
    const int len = kind_len(p, j, plan_req_uniform(pl, ii));
    if (o < len) {
      kind = j;
      i = ii;
      return;
    }
    o -= len;
  }
  kind = -1;  // unreachable for t < total
  i = 0;
}

// ------------------------------------------------------------------ statistics items

template <bool BF16, bool VEC, bool GREEDY>
__device__ void stats_item(const Params& p, int b, const Req& r, int row_r, int c) {
  constexpr int EPV = elems_per_vec(BF16);
  constexpr int CHUNK = stats_chunk(BF16);
  constexpr int PAIR = 2 * EPV;  // elements folded per online step
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  const void* base;
  int64_t row;
  if (row_r <= r.K) {
    base = p.target;
    row = static_cast<int64_t>(r.off0) + b + row_r;
  } else {
    base = p.draft;
    row = static_cast<int64_t>(r.off0) + row_r - r.K - 1;
  }
  const int64_t e0 = static_cast<int64_t>(c) * CHUNK;
  const int64_t e_end = (e0 + CHUNK < p.V) ? e0 + CHUNK : p.V;
  const int64_t rbase = row * static_cast<int64_t>(p.V);

  // issue every 16-byte load first; elements of vector u are
  // e0 + (u * kThreads + tid) * EPV + [0, EPV), increasing in u
  uint4 buf[kStatsVecs];
  if constexpr (VEC) {
    const uint4* rowv = reinterpret_cast<const uint4*>(static_cast<const char*>(base) +
                                                       rbase * (BF16 ? 2 : 4));
    const uint32_t ninf = BF16 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
      const int64_t e = e0 + (static_cast<int64_t>(u) * kThreads + tid) * EPV;
      buf[u] = (e < e_end) ? rowv[e / EPV] : make_uint4(ninf, ninf, ninf, ninf);
    }
  }
  auto unpack_pair = [&](int pi, float* xs) {
    if constexpr (VEC) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 v = buf[2 * pi + h];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        if constexpr (BF16) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            xs[h * 8 + 2 * k] = bf16_lo(w[k]);
            xs[h * 8 + 2 * k + 1] = bf16_hi(w[k]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) xs[h * 4 + k] = __uint_as_float(w[k]);
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          const int64_t e = e0 + (static_cast<int64_t>(2 * pi + h) * kThreads + tid) * EPV + k;
          xs[h * EPV + k] = (e < e_end) ? load_logit<BF16>(base, rbase + e) : -INFINITY;
        }
    }
  };

  __shared__ float sh_a[kWaves];
  __shared__ float sh_b[kWaves];
  uint64_t result = 0;
  if constexpr (GREEDY) {
    float best = -INFINITY;
    int idx = INT_MAX;
#pragma unroll
    for (int pi = 0; pi < kStatsVecs / 2; ++pi) {
      float xs[PAIR];
      unpack_pair(pi, xs);
#pragma unroll
      for (int k = 0; k < PAIR; ++k) {
        if (xs[k] > best) {
          best = xs[k];
          idx = static_cast<int>(e0 + (static_cast<int64_t>(2 * pi + k / EPV) * kThreads + tid) *
                                          EPV + k % EPV);
        }
      }
    }
    wave_merge_argmax(best, idx);
    if (lane == 0) {
      sh_a[wave] = best;
      sh_b[wave] = __int_as_float(idx);
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kWaves; ++w) merge_argmax(best, idx, sh_a[w], __float_as_int(sh_b[w]));
      result = pack_slot(best, static_cast<uint32_t>(idx));
    }
  } else {
    // online over pairs of vectors: (m, s) with s relative to fl(m c)
    const float cf = kLog2e / r.T;
    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int pi = 0; pi < kStatsVecs / 2; ++pi) {
      float xs[PAIR];
      unpack_pair(pi, xs);
      float pm = xs[0];
#pragma unroll
      for (int k = 1; k < PAIR; ++k) pm = fmaxf(pm, xs[k]);
      const float M = fmaxf(m, pm);
      // offset 0 when there is no finite max keeps a NaN visible in the sum
      const float Mc = (M == -INFINITY) ? 0.f : scaled_max(M, cf);
      if (m != -INFINITY) s *= fast_exp2(scaled_max(m, cf) - Mc);
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int k = 0; k < PAIR; k += 2) {
        a0 += fast_exp2(scaled_logit(xs[k], cf, Mc));
        a1 += fast_exp2(scaled_logit(xs[k + 1], cf, Mc));
      }
      s += a0 + a1;
      m = M;
    }
    wave_merge_stats(m, s, cf);
    if (lane == 0) {
      sh_a[wave] = m;
      sh_b[wave] = s;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kWaves; ++w) merge_stats(m, s, sh_a[w], sh_b[w], cf);
      result = pack_slot(m, __float_as_uint(s));
    }
  }
  if (tid == 0) slot_store(part_slot(p, b, row_slot(p.max_k, r.K, row_r), c), result);
}

// ------------------------------------------------------------------ finishers

// Waits for the partials of rows 0..nrows-1, folds them into sh_m / sh_ls and
// zeroes the slots.  Greedy: sh_ls holds the argmax index bits.  Sets *bad on
// a non-finite row, a NaN sum or an expired wait.
template <bool GREEDY>
__device__ void fold_partials(const Params& p, int b, int K, float cf, int nrows, float* sh_m,
                              float* sh_ls, int* bad) {
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  float a[kRowsPerWave], s[kRowsPerWave];
  int ia[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    a[i] = -INFINITY;
    s[i] = 0.f;
    ia[i] = INT_MAX;
  }
  bool expired = false;
  for (int c0 = 0; c0 < p.nc1; c0 += 64) {
    const int c = c0 + lane;
    // issue every slot load before waiting on any of them
    uint64_t v[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int row = wave + i * kWaves;
      v[i] = (row < nrows && c < p.nc1)
                 ? slot_load(part_slot(p, b, row_slot(p.max_k, K, row), c))
                 : 1u;
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int row = wave + i * kWaves;
      if (row < nrows && c < p.nc1) {
        uint64_t* slot = part_slot(p, b, row_slot(p.max_k, K, row), c);
        if (v[i] == 0u) v[i] = slot_wait(slot);
        if (v[i] == 0u) {
          expired = true;
          continue;
        }
        slot_store(slot, 0u);
        if (GREEDY) {
          if (slot_f(v[i]) > -INFINITY)
            merge_argmax(a[i], ia[i], slot_f(v[i]), static_cast<int>(slot_w(v[i])));
        } else {
          merge_stats(a[i], s[i], slot_f(v[i]), __uint_as_float(slot_w(v[i])), cf);
        }
      }
    }
  }
  if (expired) atomicOr(bad, 1);
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int row = wave + i * kWaves;
    if (GREEDY)
      wave_merge_argmax(a[i], ia[i]);
    else
      wave_merge_stats(a[i], s[i], cf);
    if (lane == 0 && row < nrows) {
      const bool finite_max = a[i] > -INFINITY && a[i] < INFINITY;
      if (GREEDY) {
        if (!finite_max) atomicOr(bad, 1);
        sh_ls[row] = __int_as_float(ia[i]);
      } else {
        if (!finite_max || !(s[i] < INFINITY)) atomicOr(bad, 1);
        sh_m[row] = a[i];
        sh_ls[row] = fast_log2(s[i]);
      }
    }
  }
}

template <bool BF16>
__device__ void finish_sampled(const Params& p, int b, const Req& r) {
  const int tid = item_tid();
  const int K = r.K;
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  const int64_t drow0 = r.off0;
  const float cf = kLog2e / r.T;

  __shared__ int sh_bad;
  __shared__ float sh_m[kRowsMax];
  __shared__ float sh_ls[kRowsMax];
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  int32_t x = 0;
  float zp = 0.f, zq = 0.f;
  if (tid < K) {
    x = p.tokens[r.off0 + tid];
    if (x < 0 || x >= p.V) {
      atomicOr(&sh_bad, 1);
    } else {  // gathered now, so the loads overlap the wait for the partials
      zp = load_logit<BF16>(p.target, (trow0 + tid) * p.V + x);
      zq = load_logit<BF16>(p.draft, (drow0 + tid) * p.V + x);
    }
  }
  fold_partials<false>(p, b, K, cf, 2 * K + 1, sh_m, sh_ls, &sh_bad);
  __syncthreads();

  uint64_t* pub = p.pub + 4 * static_cast<int64_t>(b);
  if (sh_bad) {
    write_fault(p, b, r);
    if (tid == 0) slot_store(pub + 3, pack_slot(1.f, kStatusFault));
    return;
  }
  // ratio test r_t * q_t(x_t) < p_t(x_t), left to right (wave 0 holds t < K <= 8)
  bool reject = false;
  if (tid < K) {
    const float pp = fast_exp2(scaled_logit(zp, cf, scaled_max(sh_m[tid], cf)) - sh_ls[tid]);
    const float qq =
        fast_exp2(scaled_logit(zq, cf, scaled_max(sh_m[K + 1 + tid], cf)) - sh_ls[K + 1 + tid]);
    const float u = uniform_open01(philox4x32_10(0u, tid, b, 1u, p.k0, p.k1).w[0]);
    reject = !(u * qq < pp);
    if (p.p_at) p.p_at[drow0 + tid] = pp;
    if (p.q_at) p.q_at[drow0 + tid] = qq;
  }
  const uint64_t mask = __ballot(reject);
  if (tid == 0) {
    const int n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : K;
    const float mcq = n < K ? scaled_max(sh_m[K + 1 + n], cf) : 0.f;
    const float lsq = n < K ? sh_ls[K + 1 + n] : 0.f;
    slot_store(pub + 0, pack_slot(scaled_max(sh_m[n], cf), __float_as_uint(sh_ls[n])));
    slot_store(pub + 1, pack_slot(mcq, __float_as_uint(lsq)));
    slot_store(pub + 2, pack_slot(cf, static_cast<uint32_t>(n)));
    drain_memory();
    slot_store(pub + 3, pack_slot(1.f, kStatusOk));
  }
}

// Greedy requests, and requests whose slice or temperature is invalid.
__device__ void finish_greedy(const Params& p, int b, const Req& r) {
  const int tid = item_tid();
  if (!r.slice_ok) {
    if (tid == 0) p.accept_len[b] = -1;
    return;
  }
  if (!r.temp_ok) {
    write_fault(p, b, r);
    return;
  }
  const int K = r.K;
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  __shared__ int sh_bad;
  __shared__ float sh_ls[kRowsMax];
  __shared__ int sh_n;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  int32_t x = 0;
  if (tid < K) {
    x = p.tokens[r.off0 + tid];
    if (x < 0 || x >= p.V) atomicOr(&sh_bad, 1);
  }
  fold_partials<true>(p, b, K, 0.f, K + 1, nullptr, sh_ls, &sh_bad);
  __syncthreads();
  if (sh_bad) {
    write_fault(p, b, r);
    return;
  }
  // first t < K whose draft differs from the argmax; the stop token is argmax row n
  const bool mismatch = tid < K && __float_as_int(sh_ls[tid]) != x;
  const uint64_t mask = __ballot(mismatch);
  if (tid == 0) sh_n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : K;
  __syncthreads();
  const int n = sh_n;
  if (tid <= K) {
    const int32_t y = __float_as_int(sh_ls[n]);
    p.out_tokens[trow0 + tid] = (tid < n) ? x : (tid == n ? y : -1);
  }
  if (tid < K) {
    if (p.p_at) p.p_at[r.off0 + tid] = NAN;
    if (p.q_at) p.q_at[r.off0 + tid] = NAN;
  }
  if (tid == 0) p.accept_len[b] = n;
}

// ------------------------------------------------------------------ race items

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

struct RaceRow {
  float mcp, lsp, mcq, lsq, cf;
  int n;
};

__device__ __forceinline__ RaceRow read_published(const uint64_t* pub) {
  RaceRow rr;
  const uint64_t w0 = slot_load(pub + 0), w1 = slot_load(pub + 1), w2 = slot_load(pub + 2);
  rr.mcp = slot_f(w0);
  rr.lsp = __uint_as_float(slot_w(w0));
  rr.mcq = slot_f(w1);
  rr.lsq = __uint_as_float(slot_w(w1));
  rr.cf = slot_f(w2);
  rr.n = static_cast<int>(slot_w(w2));
  return rr;
}

// Race candidates of tokens 4g..4g+3 folded into this thread's best
// (bw / be, bidx); tokens arrive in increasing order, so a strict > keeps the
// lowest index on ties.
__device__ __forceinline__ void race_group(const float zp[4], const float zq[4], bool residual,
                                           const RaceRow& rr, int64_t g, int64_t v_end,
                                           uint32_t b, uint32_t k0, uint32_t k1, float& bw,
                                           float& be, int& bidx) {
  const Philox4 r = philox4x32_10(static_cast<uint32_t>(g), static_cast<uint32_t>(rr.n), b, 0u,
                                  k0, k1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t v = g * 4 + k;
    if (v >= v_end) break;
    const float e = -fast_log2(uniform_open01(r.w[k]));  // E / ln 2
    float w = fast_exp2(scaled_logit(zp[k], rr.cf, rr.mcp) - rr.lsp);
    if (residual) w -= fast_exp2(scaled_logit(zq[k], rr.cf, rr.mcq) - rr.lsq);
    if (w * be > bw * e) {
      bw = w;
      be = e;
      bidx = static_cast<int>(v);
    }
  }
}

// A thread's best as a float key for merging (-inf when it has none).
__device__ __forceinline__ float race_key(float bw, float be, int bidx) {
  return bidx == INT_MAX ? -INFINITY : bw / be;
}

template <bool BF16, bool VEC>
__device__ void race_chunk(const Params& p, int b, const Req& r, int c) {
  const int tid = item_tid();
  const uint64_t* pub = p.pub + 4 * static_cast<int64_t>(b);
  __shared__ uint32_t sh_status;
  if (tid == 0) sh_status = slot_w(slot_wait(pub + 3));  // 0 if the wait expired
  __syncthreads();
  uint64_t* out = p.race_part + static_cast<int64_t>(b) * p.nc2 + c;
  if (sh_status != kStatusOk) {
    if (tid == 0) slot_store(out, pack_slot(-INFINITY, INT_MAX));
    return;
  }
  const RaceRow rr = read_published(pub);
  const int64_t esz = BF16 ? 2 : 4;
  const bool residual = rr.n < r.K;
  const void* prow =
      static_cast<const char*>(p.target) + (static_cast<int64_t>(r.off0) + b + rr.n) * p.V * esz;
  const void* qrow = residual ? static_cast<const char*>(p.draft) +
                                    (static_cast<int64_t>(r.off0) + rr.n) * p.V * esz
                              : nullptr;
  const int64_t v_begin = static_cast<int64_t>(c) * kRaceChunk;
  const int64_t v_end = (v_begin + kRaceChunk < p.V) ? v_begin + kRaceChunk : p.V;
  float zp[kRaceGroups][4], zq[kRaceGroups][4];
#pragma unroll
  for (int gi = 0; gi < kRaceGroups; ++gi) {  // issue every load before any math
    const int64_t g = v_begin / 4 + gi * kThreads + tid;
#pragma unroll
    for (int k = 0; k < 4; ++k) zq[gi][k] = 0.f;
    if (g * 4 < v_end) {
      load4<BF16, VEC>(prow, g * 4, v_end, zp[gi]);
      if (residual) load4<BF16, VEC>(qrow, g * 4, v_end, zq[gi]);
    }
  }
  float bw = 0.f, be = 1.f;  // any w > 0 beats the empty candidate
  int idx = INT_MAX;
#pragma unroll
  for (int gi = 0; gi < kRaceGroups; ++gi) {
    const int64_t g = v_begin / 4 + gi * kThreads + tid;
    if (g * 4 < v_end)
      race_group(zp[gi], zq[gi], residual, rr, g, v_end, b, p.k0, p.k1, bw, be, idx);
  }
  float key = race_key(bw, be, idx);
  __shared__ float sh_key[kWaves];
  __shared__ int sh_idx[kWaves];
  block_argmax(key, idx, sh_key, sh_idx);
  if (tid == 0) slot_store(out, pack_slot(key, static_cast<uint32_t>(idx)));
}

template <bool BF16, bool VEC>
__device__ void race_finish(const Params& p, int b, const Req& r) {
  const int tid = item_tid();
  __shared__ float sh_key[kWaves];
  __shared__ int sh_idx[kWaves];
  __shared__ int sh_expired;
  if (tid == 0) sh_expired = 0;
  __syncthreads();
  float key = -INFINITY;
  int idx = INT_MAX;
  for (int i = tid; i < p.nc2; i += kThreads) {
    uint64_t* slot = p.race_part + static_cast<int64_t>(b) * p.nc2 + i;
    const uint64_t v = slot_wait(slot);
    if (v == 0u) {
      atomicOr(&sh_expired, 1);
      continue;
    }
    slot_store(slot, 0u);
    merge_argmax(key, idx, slot_f(v), static_cast<int>(slot_w(v)));
  }
  block_argmax(key, idx, sh_key, sh_idx);  // its barriers also publish sh_expired
  uint64_t* pub = p.pub + 4 * static_cast<int64_t>(b);
  const uint32_t status = slot_w(slot_load(pub + 3));
  const RaceRow rr = read_published(pub);
  __syncthreads();  // every thread has read the record before it is cleared
  if (tid < 4) slot_store(pub + tid, 0u);
  if (sh_expired || status == 0u) {
    if (tid == 0) p.accept_len[b] = -1;
    return;
  }
  if (status != kStatusOk) return;  // the finisher wrote the failure
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  if (idx == INT_MAX) {
    // no token had p > q (rounding can only cause this when p == q): race on p_n
    const int64_t esz = BF16 ? 2 : 4;
    const void* prow = static_cast<const char*>(p.target) + (trow0 + rr.n) * p.V * esz;
    float bw = 0.f, be = 1.f;
    for (int64_t g = tid; g * 4 < p.V; g += kThreads) {
      float zp[4];
      const float zq[4] = {0.f, 0.f, 0.f, 0.f};
      load4<BF16, VEC>(prow, g * 4, p.V, zp);
      race_group(zp, zq, false, rr, g, p.V, b, p.k0, p.k1, bw, be, idx);
    }
    key = race_key(bw, be, idx);
    block_argmax(key, idx, sh_key, sh_idx);
  }
  const int n = rr.n;
  if (tid <= r.K) {
    const int32_t xt = (tid < n) ? p.tokens[r.off0 + tid] : 0;
    p.out_tokens[trow0 + tid] = (tid < n) ? xt : (tid == n ? idx : -1);
  }
  if (tid == 0) p.accept_len[b] = n;
}

// ------------------------------------------------------------------ kernel

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) void sv_verify(Params p) {
  const int tid = threadIdx.x;
  const int list = blockIdx.x % kLists;
  uint32_t* ticket = p.counters + list * kCounterStride;
  uint32_t* exits = p.counters + (kLists + list) * kCounterStride;
  __shared__ Plan pl;
  __shared__ uint32_t sh_t;
  uint32_t next = 0;
  if (tid == 0) next = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  build_plan(p, list, pl);  // overlaps the first ticket's round trip
  if (tid == 0) sh_t = next;
  __syncthreads();
  const uint32_t total = static_cast<uint32_t>(uni(pl.total));
  uint32_t t = static_cast<uint32_t>(uni(static_cast<int>(sh_t)));
  while (t < total) {
    // take the next ticket now; it is only read after this item
    if (tid == 0)
      next = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int kind, i, o;
    decode_ticket(p, pl, static_cast<int>(t), kind, i, o);
    const int b = p.b_begin + list + i * kLists;
    const Req r = plan_req_uniform(pl, i);
    switch (kind) {
      case kSA: stats_item<BF16, VEC, false>(p, b, r, o / p.nc1, o % p.nc1); break;
      case kSG: stats_item<BF16, VEC, true>(p, b, r, o / p.nc1, o % p.nc1); break;
      case kFA: finish_sampled<BF16>(p, b, r); break;
      case kR:
        if (o < p.nc2)
          race_chunk<BF16, VEC>(p, b, r, o);
        else
          race_finish<BF16, VEC>(p, b, r);
        break;
      case kFG: finish_greedy(p, b, r); break;
      default: break;
    }
    __syncthreads();
    if (tid == 0) sh_t = next;
    __syncthreads();
    t = static_cast<uint32_t>(uni(static_cast<int>(sh_t)));
  }
  // the list's last workgroup to leave resets its counters for the next call
  if (tid == 0) {
    const uint32_t left = __hip_atomic_fetch_add(exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (left + 1 == static_cast<uint32_t>(list_workgroups(p, list))) {
      __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ host side

bool shape_ok(int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows) {
  return B >= 1 && V >= 1 && max_k >= 0 && max_k <= SV_KMAX && n_draft_rows >= 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups that fit on the device at once (cached per device and kernel;
// a property of the device, not of any call).
template <bool BF16, bool VEC>
int resident_workgroups() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sv_verify<BF16, VEC>, kThreads, 0) !=
        hipSuccess)
      return 0;
    cache[dev] = std::max(1, cus * per_cu);
  }
  return cache[dev];
}

template <bool BF16, bool VEC>
int launch(Params prm, int32_t B, hipStream_t stream, void* ev0, void* ev1) {
  const int resident = resident_workgroups<BF16, VEC>();
  if (resident <= 0) return SV_ERR_LAUNCH;
  if (ev0 && hipEventRecord(static_cast<hipEvent_t>(ev0), stream) != hipSuccess)
    return SV_ERR_LAUNCH;
  // requests go in launches of at most kLists * kMaxLocal
  for (int32_t b0 = 0; b0 < B; b0 += kLists * kMaxLocal) {
    prm.b_begin = b0;
    prm.b_end = std::min<int32_t>(B, b0 + kLists * kMaxLocal);
    const int64_t nreq = prm.b_end - prm.b_begin;
    const int64_t items = nreq * ((2 * prm.max_k + 1) * prm.nc1 + prm.nc2 + 3);
    int64_t grid = std::min<int64_t>(resident, items);
    grid = std::max<int64_t>(kLists, (grid + kLists - 1) / kLists * kLists);
    prm.grid = static_cast<int32_t>(grid);
    hipLaunchKernelGGL((sv_verify<BF16, VEC>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads),
                       0, stream, prm);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  }
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
  const Layout L = make_layout(B, V, max_k, bf16);
  char* ws = static_cast<char*>(workspace);
  Params prm;
  prm.target = target;
  prm.draft = all_greedy ? nullptr : draft;
  prm.offsets = offsets;
  prm.tokens = tokens;
  prm.temperature = all_greedy ? nullptr : temperature;
  prm.k0 = static_cast<uint32_t>(seed);
  prm.k1 = static_cast<uint32_t>(seed >> 32);
  prm.b_begin = 0;
  prm.b_end = B;
  prm.V = V;
  prm.max_k = max_k;
  prm.n_draft_rows = n_draft_rows;
  prm.nc1 = L.nc1;
  prm.nc2 = L.nc2;
  prm.grid = 0;
  prm.counters = reinterpret_cast<uint32_t*>(ws + L.count_off);
  prm.part = reinterpret_cast<uint64_t*>(ws + L.stats_off);
  prm.race_part = reinterpret_cast<uint64_t*>(ws + L.race_off);
  prm.pub = reinterpret_cast<uint64_t*>(ws + L.pub_off);
  prm.accept_len = accept_len;
  prm.out_tokens = out_tokens;
  prm.p_at = p_at;
  prm.q_at = q_at;
  const int64_t row_bytes = static_cast<int64_t>(V) * (bf16 ? 2 : 4);
  const bool vec = row_bytes % 16 == 0 && aligned16(target) && (!draft || aligned16(draft));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch<true, true>(prm, B, s, ev0, ev1) : launch<true, false>(prm, B, s, ev0, ev1);
  return vec ? launch<false, true>(prm, B, s, ev0, ev1) : launch<false, false>(prm, B, s, ev0, ev1);
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_bytes(int32_t B, int32_t V, int32_t max_k) {
  if (!shape_ok(B, V, max_k, 0)) return 0;
  return make_layout(B, V, max_k, false).total;
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

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "bad shape (B, V, max_k or n_draft_rows) or grid too large";
    case SV_ERR_DTYPE: return "unknown dtype";
    case SV_ERR_WORKSPACE: return "workspace too small or not 16-byte aligned";
    case SV_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
