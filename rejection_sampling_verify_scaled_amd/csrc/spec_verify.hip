// spec_verify.hip -- gfx950 kernel and C ABI of the speculative-decoding verify step.
//
// What is computed is stated in include/spec_verify.h (the accept / residual /
// bonus rule of "Decodificación Especulativa y EAGLE", section "La Regla de
// Exactitud", and its greedy case).  How it runs on MI355X: one launch, two
// kinds of workgroup.
//
//   row-statistics workgroups, one per (request, row slot, V-chunk), first in
//     the grid.  Each streams its chunk with 16-byte loads and reduces it to
//     one 8-byte partial: (max, sum of 2^((z - max) * log2(e) / T)) for rows a
//     sampled request needs, (max, lowest argmax index) for rows of a greedy
//     request.  Draft rows of greedy requests are never read.  These carry
//     all of the HBM traffic.  The last of a request's workgroups to finish
//     (atomic counter; nobody waits) becomes the request's finisher: it folds
//     the partials into per-row (max, log2 sum), and
//       greedy:  finds the first draft that differs from the row argmax and
//                writes the request's outputs;
//       sampled: gathers p_t(x_t), q_t(x_t), draws r_t, finds the first
//                rejection n with a wave ballot, and publishes n with the
//                statistics of row n.
//   race workgroups, one per (sampled request, race chunk).  Each waits for
//     its request's publication, runs the exponential race over its chunk of
//     row n -- residual (p_n - q_n)+ after a rejection, bonus p_K otherwise --
//     and the last of them folds the chunk winners and writes the outputs.
//     Request b's race workgroups sit in the grid right after the row
//     statistics of request b + lag (lag ~ one residency's worth of
//     workgroups), so race arithmetic overlaps the streaming of later rows.
//
// Forward progress: a race workgroup only waits for row-statistics
// workgroups, which have lower indices and never wait, so with in-order
// dispatch the wait always ends.  The wait is also bounded (kSpinLimit polls);
// if it ever expired the request would report accept_len = -1.
//
// Cross-workgroup data (partials, published records, flags) moves only
// through device-coherent stores and loads (agent-scope relaxed atomics,
// i.e. sc1 accesses that bypass the per-XCD L2 for these lines), and each
// data store is drained (s_waitcnt) before the counter increment that
// announces it.  No agent-scope release/acquire fence is used: on gfx950
// those write back or invalidate the whole L2 of the XCD, which thousands of
// workgroups per call cannot afford.
//
// Race keys: the winner maximises ln w_v - ln E_v, i.e. w_v / E_v.  Inside a
// thread candidates are compared by cross-multiplication (w_a e_b > w_b e_a)
// with e = -log2 U = E / ln 2 (a common factor); a thread's best becomes the
// float key w / e for the merges across threads, waves and chunks.  Weights
// are 2^(z c - fl(m c)) with c = log2(e) / T, fl(m c) the rounded product
// for the row's maximum m; the same rounded offset is used when the row's
// sum is formed, so it cancels exactly from p = w / sum.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;  // 4 wave64s per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kStatsVecs = 8;   // 16-byte loads per thread per statistics chunk
constexpr int kRaceGroups = 4;  // 4-token Philox groups per thread per race chunk
constexpr int kRaceChunk = kThreads * kRaceGroups * 4;  // tokens per race chunk
constexpr int kRowsMax = 2 * SV_KMAX + 1;               // row slots per request
constexpr int kRowsPerWave = (kRowsMax + kWaves - 1) / kWaves;
constexpr unsigned kSpinLimit = 1u << 16;
#ifndef SV_RACE_LAG_SLOTS
#define SV_RACE_LAG_SLOTS 1536  // grid slots between a request's statistics and its race
#endif
constexpr float kLog2e = 1.4426950408889634f;

__host__ __device__ constexpr int elems_per_vec(bool bf16) { return bf16 ? 8 : 4; }
__host__ __device__ constexpr int stats_chunk(bool bf16) {
  return kThreads * kStatsVecs * elems_per_vec(bf16);
}

// ------------------------------------------------------------------ helpers

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

// fl(m * c): the row-maximum offset, rounded once and never contracted, so
// every place that needs it gets the identical float.
__device__ __forceinline__ float scaled_max(float m, float cf) { return __fmul_rn(m, cf); }

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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

// Device-coherent 8-byte store / load of a float2 (bypasses stale L2 lines).
__device__ __forceinline__ void store_coherent(float2* p, float2 v) {
  const uint64_t bits = static_cast<uint64_t>(__float_as_uint(v.x)) |
                        (static_cast<uint64_t>(__float_as_uint(v.y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 load_coherent(const float2* p) {
  const uint64_t bits = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(bits)),
                     __uint_as_float(static_cast<uint32_t>(bits >> 32)));
}

__device__ __forceinline__ void store_coherent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_coherent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Drain this thread's outstanding memory operations, so a device-coherent
// store is visible before the atomic that follows announces it.  The signal
// fences keep the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void drain_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint32_t count_one(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ workspace

enum : int32_t { kStatusOk = 0, kStatusFault = 1 };

// What a sampled request's finisher publishes for its race workgroups.
struct Published {
  int32_t n;       // first rejected position (K when every draft passed)
  int32_t status;  // kStatusOk / kStatusFault
  float mcp, lsp;  // target row n: fl(max * c) and log2 of its sum
  float mcq, lsq;  // draft row n (residual race only)
  float cf;        // log2(e) / T
  int32_t pad;
};
static_assert(sizeof(Published) == 4 * sizeof(float2), "Published moves as four float2");

__device__ __forceinline__ void publish(Published* dst, const Published& v) {
  const float2* src = reinterpret_cast<const float2*>(&v);
#pragma unroll
  for (int i = 0; i < 4; ++i) store_coherent(reinterpret_cast<float2*>(dst) + i, src[i]);
}

__device__ __forceinline__ Published read_published(const Published* src) {
  Published v;
  float2* dst = reinterpret_cast<float2*>(&v);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = load_coherent(reinterpret_cast<const float2*>(src) + i);
  return v;
}

// Data regions grow from the start of the workspace and depend on the call's
// sizes; the per-request counters sit in 16-byte slots at the end of the
// caller's buffer (slot b at end - 16 (b + 1)), so their addresses do not
// move between calls that share a buffer.
struct Layout {
  int J;    // row slots per request: target 0..max_k, then draft 0..max_k-1
  int nc1;  // statistics chunks per row
  int nc2;  // race chunks per row
  size_t stats_off, race_off, pub_off, data_end, total;
};

struct Counters {
  uint32_t done;       // finished row-statistics workgroups
  uint32_t ready;      // the finisher has published
  uint32_t race_done;  // finished race workgroups
  uint32_t pad;
};

__host__ __device__ inline int ceil_div(int64_t a, int64_t b) {
  return static_cast<int>((a + b - 1) / b);
}

inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

Layout make_layout(int32_t B, int32_t V, int32_t max_k, bool bf16) {
  Layout L;
  L.J = 2 * max_k + 1;
  L.nc1 = ceil_div(V, stats_chunk(bf16));
  L.nc2 = ceil_div(V, kRaceChunk);
  L.stats_off = 0;
  const size_t stats_bytes =
      static_cast<size_t>(B) * L.J * ceil_div(V, stats_chunk(false)) * sizeof(float2);
  L.race_off = round256(stats_bytes);
  L.pub_off = L.race_off + round256(static_cast<size_t>(B) * L.nc2 * sizeof(float2));
  L.data_end = L.pub_off + round256(static_cast<size_t>(B) * sizeof(Published));
  L.total = round256(L.data_end + static_cast<size_t>(B) * sizeof(Counters) + 16);
  return L;
}

struct Params {
  const void* target;
  const void* draft;
  const int32_t* offsets;
  const int32_t* tokens;
  const float* temperature;  // NULL: every request greedy
  uint32_t k0, k1;           // Philox key
  int32_t B, V, max_k, n_draft_rows, nc1, nc2;
  int32_t lag;      // request b's race follows the statistics of request b + lag
  int64_t S;        // statistics slots per request: (2 max_k + 1) * nc1
  float2* part;          // [B][J][nc1] row-statistics partials
  float2* race_part;     // [B][nc2] race chunk winners (key, index bits)
  Published* pub;        // [B]
  Counters* cnt_end;     // request b's counters at cnt_end[-1 - b]
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_at;
  float* q_at;
};

__device__ __forceinline__ Counters& counters(const Params& p, int b) { return p.cnt_end[-1 - b]; }

// Per-request checks every workgroup can make from the request's scalars.
struct Req {
  int32_t off0, K;
  float T;
  bool slice_ok, temp_ok, greedy;
};

__device__ __forceinline__ Req load_req(const Params& p, int b) {
  Req r;
  r.off0 = p.offsets[b];
  const int32_t off1 = p.offsets[b + 1];
  r.K = off1 - r.off0;
  r.slice_ok = r.off0 >= 0 && off1 <= p.n_draft_rows && r.K >= 0 && r.K <= p.max_k;
  r.T = p.temperature ? p.temperature[b] : 0.f;
  r.greedy = r.T == 0.f;
  r.temp_ok = (r.T >= 0.f) && (r.T < INFINITY) && (r.greedy || r.K == 0 || p.draft != nullptr);
  return r;
}

// Outputs of a failed request (its slice is valid).
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

// ------------------------------------------------------------------ finisher

template <bool BF16>
__device__ void finish_request(const Params& p, int b, const Req& r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = r.K;
  const int J = 2 * p.max_k + 1;
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  const int64_t drow0 = r.off0;
  const bool greedy = r.greedy;
  const float cf = greedy ? 0.f : kLog2e / r.T;
  const int nrows = greedy ? K + 1 : 2 * K + 1;  // rows 0..K target, K+1..2K draft 0..K-1

  __shared__ int sh_bad;
  __shared__ float sh_m[kRowsMax];
  __shared__ float sh_ls[kRowsMax];  // greedy: argmax index bits
  __shared__ int sh_n;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  int32_t x = 0;
  if (tid < K) {
    x = p.tokens[r.off0 + tid];
    if (x < 0 || x >= p.V) atomicOr(&sh_bad, 1);
  }

  // fold the partials: wave w takes rows w, w+4, ...; lanes take chunks
  float a[kRowsPerWave], s[kRowsPerWave];
  int ia[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    a[i] = -INFINITY;
    s[i] = 0.f;
    ia[i] = INT_MAX;
  }
  for (int c0 = 0; c0 < p.nc1; c0 += 64) {
    const int c = c0 + lane;
    float2 v[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int row = wave + i * kWaves;
      v[i] = make_float2(-INFINITY, 0.f);
      if (row < nrows && c < p.nc1) {
        const int j = (row <= K) ? row : p.max_k + 1 + (row - K - 1);
        v[i] = load_coherent(p.part + (static_cast<int64_t>(b) * J + j) * p.nc1 + c);
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (greedy) {
        if (v[i].x > -INFINITY) merge_argmax(a[i], ia[i], v[i].x, __float_as_int(v[i].y));
      } else {
        merge_stats(a[i], s[i], v[i].x, v[i].y, cf);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int row = wave + i * kWaves;
    if (greedy)
      wave_merge_argmax(a[i], ia[i]);
    else
      wave_merge_stats(a[i], s[i], cf);
    if (lane == 0 && row < nrows) {
      const bool finite_max = a[i] > -INFINITY && a[i] < INFINITY;
      if (greedy) {
        if (!finite_max) atomicOr(&sh_bad, 1);
        sh_ls[row] = __int_as_float(ia[i]);
      } else {
        if (!finite_max || !(s[i] < INFINITY)) atomicOr(&sh_bad, 1);
        sh_m[row] = a[i];
        sh_ls[row] = fast_log2(s[i]);
      }
    }
  }
  __syncthreads();

  if (sh_bad) {
    write_fault(p, b, r);
    if (tid == 0) {
      Counters& cn = counters(p, b);
      store_coherent_u32(&cn.done, 0u);
      if (!greedy) {
        Published pub = {};
        pub.status = kStatusFault;
        publish(p.pub + b, pub);
        drain_memory();
        store_coherent_u32(&cn.ready, 1u);
      }
    }
    return;
  }

  if (greedy) {
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
      if (p.p_at) p.p_at[drow0 + tid] = NAN;
      if (p.q_at) p.q_at[drow0 + tid] = NAN;
    }
    if (tid == 0) {
      p.accept_len[b] = n;
      store_coherent_u32(&counters(p, b).done, 0u);
    }
    return;
  }

  // ratio test r_t * q_t(x_t) < p_t(x_t), left to right (wave 0 holds t < K <= 8)
  bool reject = false;
  if (tid < K) {
    const float zp = load_logit<BF16>(p.target, (trow0 + tid) * p.V + x);
    const float zq = load_logit<BF16>(p.draft, (drow0 + tid) * p.V + x);
    const float pp =
        fast_exp2(scaled_logit(zp, cf, scaled_max(sh_m[tid], cf)) - sh_ls[tid]);
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
    Published pub;
    pub.n = n;
    pub.status = kStatusOk;
    pub.mcp = scaled_max(sh_m[n], cf);
    pub.lsp = sh_ls[n];
    pub.mcq = n < K ? scaled_max(sh_m[K + 1 + n], cf) : 0.f;
    pub.lsq = n < K ? sh_ls[K + 1 + n] : 0.f;
    pub.cf = cf;
    pub.pad = 0;
    publish(p.pub + b, pub);
    Counters& cn = counters(p, b);
    store_coherent_u32(&cn.done, 0u);
    drain_memory();
    store_coherent_u32(&cn.ready, 1u);
  }
}

// ------------------------------------------------------------------ row statistics

template <bool BF16, bool VEC>
__device__ void stats_slot(const Params& p, int b, int slot) {
  constexpr int EPV = elems_per_vec(BF16);
  constexpr int CHUNK = stats_chunk(BF16);
  const int J = 2 * p.max_k + 1;
  const int c = slot % p.nc1;
  const int j = slot / p.nc1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const Req r = load_req(p, b);
  if (!r.slice_ok || !r.temp_ok) return;  // reported by the request's race workgroup 0
  const void* base;
  int64_t row;
  if (j <= p.max_k) {
    if (j > r.K) return;
    base = p.target;
    row = static_cast<int64_t>(r.off0) + b + j;
  } else {
    const int t = j - p.max_k - 1;
    if (r.greedy || t >= r.K) return;
    base = p.draft;
    row = static_cast<int64_t>(r.off0) + t;
  }

  const int64_t e0 = static_cast<int64_t>(c) * CHUNK;
  const int64_t e_end = (e0 + CHUNK < p.V) ? e0 + CHUNK : p.V;

  // this thread's elements, in increasing index order
  float x[kStatsVecs * EPV];
  if constexpr (VEC) {
    const uint4* rowv = reinterpret_cast<const uint4*>(
        static_cast<const char*>(base) + row * static_cast<int64_t>(p.V) * (BF16 ? 2 : 4));
    uint4 buf[kStatsVecs];
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
      const int64_t e = e0 + (static_cast<int64_t>(u) * kThreads + tid) * EPV;
      if (e < e_end) {
        buf[u] = rowv[e / EPV];
      } else {
        const uint32_t ninf = BF16 ? 0xff80ff80u : 0xff800000u;
        buf[u] = make_uint4(ninf, ninf, ninf, ninf);
      }
    }
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
      const uint32_t w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
      if constexpr (BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[u * 8 + 2 * k] = bf16_lo(w[k]);
          x[u * 8 + 2 * k + 1] = bf16_hi(w[k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[u * 4 + k] = __uint_as_float(w[k]);
      }
    }
  } else {
    const int64_t rbase = row * static_cast<int64_t>(p.V);
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const int64_t e = e0 + (static_cast<int64_t>(u) * kThreads + tid) * EPV + k;
        x[u * EPV + k] = (e < e_end) ? load_logit<BF16>(base, rbase + e) : -INFINITY;
      }
    }
  }

  __shared__ float sh_a[kWaves];
  __shared__ float sh_b[kWaves];
  float2 result;
  if (r.greedy) {
    float best = -INFINITY;
    int idx = INT_MAX;
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const float v = x[u * EPV + k];
        if (v > best) {
          best = v;
          idx = static_cast<int>(e0 + (static_cast<int64_t>(u) * kThreads + tid) * EPV + k);
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
      result = make_float2(best, __int_as_float(idx));
    }
  } else {
    const float cf = kLog2e / r.T;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kStatsVecs * EPV; ++i) m = fmaxf(m, x[i]);
    // offset 0 when there is no finite max keeps a NaN visible in the sum
    const float mc = (m == -INFINITY) ? 0.f : scaled_max(m, cf);
    float acc[kStatsVecs];
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < EPV; ++k) sum += fast_exp2(scaled_logit(x[u * EPV + k], cf, mc));
      acc[u] = sum;
    }
#pragma unroll
    for (int h = kStatsVecs / 2; h >= 1; h >>= 1)
#pragma unroll
      for (int u = 0; u < h; ++u) acc[u] += acc[u + h];
    float s = acc[0];
    wave_merge_stats(m, s, cf);
    if (lane == 0) {
      sh_a[wave] = m;
      sh_b[wave] = s;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kWaves; ++w) merge_stats(m, s, sh_a[w], sh_b[w], cf);
      result = make_float2(m, s);
    }
  }

  __shared__ int sh_last;
  if (tid == 0) {
    store_coherent(p.part + (static_cast<int64_t>(b) * J + j) * p.nc1 + c, result);
    drain_memory();
    const uint32_t need = static_cast<uint32_t>((r.greedy ? r.K + 1 : 2 * r.K + 1) * p.nc1);
    sh_last = (count_one(&counters(p, b).done) + 1 == need) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;
  finish_request<BF16>(p, b, r);
}

// ------------------------------------------------------------------ race

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
// lowest index on ties.
__device__ __forceinline__ void race_group(const float zp[4], const float zq[4], bool residual,
                                           const Published& pub, int64_t g, int64_t v_end,
                                           uint32_t b, uint32_t k0, uint32_t k1, float& bw,
                                           float& be, int& bidx) {
  const Philox4 r = philox4x32_10(static_cast<uint32_t>(g), static_cast<uint32_t>(pub.n), b, 0u,
                                  k0, k1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t v = g * 4 + k;
    if (v >= v_end) break;
    const float e = -fast_log2(uniform_open01(r.w[k]));  // E / ln 2
    float w = fast_exp2(scaled_logit(zp[k], pub.cf, pub.mcp) - pub.lsp);
    if (residual) w -= fast_exp2(scaled_logit(zq[k], pub.cf, pub.mcq) - pub.lsq);
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
__device__ void race_slot(const Params& p, int b, int c) {
  const int tid = threadIdx.x;
  const Req r = load_req(p, b);
  if (!r.slice_ok) {
    if (c == 0 && tid == 0) p.accept_len[b] = -1;
    return;
  }
  if (!r.temp_ok) {
    if (c == 0) write_fault(p, b, r);
    return;
  }
  if (r.greedy) return;  // finished by its row-statistics finisher

  Counters& cn = counters(p, b);
  __shared__ int sh_flag;
  if (tid == 0) {
    unsigned it = 0;
    while (load_coherent_u32(&cn.ready) == 0u) {
      if (++it > kSpinLimit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    sh_flag = (it > kSpinLimit) ? 1 : 0;
  }
  __syncthreads();
  if (sh_flag) {
    if (c == 0 && tid == 0) p.accept_len[b] = -1;
    return;
  }
  const Published pub = read_published(p.pub + b);
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  const int64_t drow0 = r.off0;
  const int64_t esz = BF16 ? 2 : 4;
  const void* prow = static_cast<const char*>(p.target) + (trow0 + pub.n) * p.V * esz;
  const bool residual = pub.n < r.K;
  const void* qrow =
      residual ? static_cast<const char*>(p.draft) + (drow0 + pub.n) * p.V * esz : nullptr;

  __shared__ float sh_key[kWaves];
  __shared__ int sh_idx[kWaves];
  float key = -INFINITY;
  int idx = INT_MAX;
  if (pub.status == kStatusOk) {
    float bw = 0.f, be = 1.f;  // any w > 0 beats the empty candidate
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
#pragma unroll
    for (int gi = 0; gi < kRaceGroups; ++gi) {
      const int64_t g = v_begin / 4 + gi * kThreads + tid;
      if (g * 4 < v_end)
        race_group(zp[gi], zq[gi], residual, pub, g, v_end, b, p.k0, p.k1, bw, be, idx);
    }
    key = race_key(bw, be, idx);
    block_argmax(key, idx, sh_key, sh_idx);
  }

  __shared__ int sh_last;
  if (tid == 0) {
    if (pub.status == kStatusOk) {
      store_coherent(p.race_part + static_cast<int64_t>(b) * p.nc2 + c,
                     make_float2(key, __int_as_float(idx)));
      drain_memory();
    }
    sh_last = (count_one(&cn.race_done) + 1 == static_cast<uint32_t>(p.nc2)) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;

  if (pub.status == kStatusOk) {
    key = -INFINITY;
    idx = INT_MAX;
    for (int i = tid; i < p.nc2; i += kThreads) {
      const float2 w = load_coherent(p.race_part + static_cast<int64_t>(b) * p.nc2 + i);
      merge_argmax(key, idx, w.x, __float_as_int(w.y));
    }
    block_argmax(key, idx, sh_key, sh_idx);
    if (idx == INT_MAX) {
      // no token had p > q (rounding can only cause this when p == q): race on p_n
      float bw = 0.f, be = 1.f;
      for (int64_t g = tid; g * 4 < p.V; g += kThreads) {
        float zp[4];
        const float zq[4] = {0.f, 0.f, 0.f, 0.f};
        load4<BF16, VEC>(prow, g * 4, p.V, zp);
        race_group(zp, zq, false, pub, g, p.V, b, p.k0, p.k1, bw, be, idx);
      }
      key = race_key(bw, be, idx);
      block_argmax(key, idx, sh_key, sh_idx);
    }
    const int n = pub.n;
    if (tid <= r.K) {
      const int32_t xt = (tid < n) ? p.tokens[r.off0 + tid] : 0;
      p.out_tokens[trow0 + tid] = (tid < n) ? xt : (tid == n ? idx : -1);
    }
    if (tid == 0) p.accept_len[b] = n;
  }
  if (tid == 0) {
    store_coherent_u32(&cn.ready, 0u);
    store_coherent_u32(&cn.race_done, 0u);
  }
}

// ------------------------------------------------------------------ kernel

// Grid order (S statistics slots per request, nc2 race slots per request,
// d = min(lag, B)):
//   [stats 0] .. [stats d-1]
//   [stats d][race 0] [stats d+1][race 1] .. [stats B-1][race B-1-d]
//   [race B-d] .. [race B-1]
// so every race slot comes after all statistics slots of its request.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sv_verify(Params p) {
  const int64_t g = blockIdx.x;
  const int64_t d = p.lag < p.B ? p.lag : p.B;
  const int64_t head = d * p.S;
  const int64_t seg = p.S + p.nc2;
  const int64_t body = head + (p.B - d) * seg;
  if (g < head) {
    stats_slot<BF16, VEC>(p, static_cast<int>(g / p.S), static_cast<int>(g % p.S));
  } else if (g < body) {
    const int64_t k = (g - head) / seg, o = (g - head) % seg;
    if (o < p.S)
      stats_slot<BF16, VEC>(p, static_cast<int>(d + k), static_cast<int>(o));
    else
      race_slot<BF16, VEC>(p, static_cast<int>(k), static_cast<int>(o - p.S));
  } else {
    const int64_t h = g - body;
    race_slot<BF16, VEC>(p, static_cast<int>(p.B - d + h / p.nc2), static_cast<int>(h % p.nc2));
  }
}

// ------------------------------------------------------------------ host side

bool shape_ok(int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows) {
  return B >= 1 && V >= 1 && max_k >= 0 && max_k <= SV_KMAX && n_draft_rows >= 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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
  prm.B = B;
  prm.V = V;
  prm.max_k = max_k;
  prm.n_draft_rows = n_draft_rows;
  prm.nc1 = L.nc1;
  prm.nc2 = all_greedy ? 0 : L.nc2;
  prm.S = static_cast<int64_t>(L.J) * L.nc1;
  prm.lag = all_greedy ? B : ceil_div(SV_RACE_LAG_SLOTS, prm.S);
  prm.part = reinterpret_cast<float2*>(ws + L.stats_off);
  prm.race_part = reinterpret_cast<float2*>(ws + L.race_off);
  prm.pub = reinterpret_cast<Published*>(ws + L.pub_off);
  const uintptr_t end = (reinterpret_cast<uintptr_t>(ws) + workspace_bytes) & ~uintptr_t{15};
  prm.cnt_end = reinterpret_cast<Counters*>(end);
  if (reinterpret_cast<char*>(prm.cnt_end - B) < ws + L.data_end) return SV_ERR_WORKSPACE;
  prm.accept_len = accept_len;
  prm.out_tokens = out_tokens;
  prm.p_at = p_at;
  prm.q_at = q_at;
  const int64_t grid = static_cast<int64_t>(B) * (prm.S + prm.nc2);
  if (grid > INT32_MAX) return SV_ERR_SHAPE;
  const int64_t row_bytes = static_cast<int64_t>(V) * (bf16 ? 2 : 4);
  const bool vec = row_bytes % 16 == 0 && aligned16(target) && (!draft || aligned16(draft));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch<true, true>(prm, grid, s, ev0, ev1)
               : launch<true, false>(prm, grid, s, ev0, ev1);
  return vec ? launch<false, true>(prm, grid, s, ev0, ev1)
             : launch<false, false>(prm, grid, s, ev0, ev1);
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
