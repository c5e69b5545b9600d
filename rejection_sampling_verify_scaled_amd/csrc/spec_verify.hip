// spec_verify.hip -- gfx950 kernels and C ABI of the speculative-decoding verify step.
//
// What is computed is stated in include/spec_verify.h (the accept / residual /
// bonus rule of "Decodificación Especulativa y EAGLE", section "La Regla de
// Exactitud", and its greedy case).  How it runs on MI355X: two kernels on the
// caller's stream.
//
// sv_stats -- one workgroup per (row, 64 KiB chunk) of every target row and
// every draft row, in memory order.  A target row's loads are issued before
// anything else (its address needs no request data); the owner request of the
// row is found meanwhile by a binary search over a window of draft_offsets
// cached in LDS.  A draft row is loaded only if its owner samples (the draft
// rows of greedy requests are never read).  The chunk is reduced to one
// 8-byte partial: (max, sum of 2^(z c - fl(max c))), c = log2(e) / T, for a
// sampled request; (max, lowest argmax index) for a greedy one.  The workgroup
// whose chunk holds the logit at a draft token x_t hands that logit over (a
// "gather" slot); for a greedy request the token itself is handed over.
// The kernel is a plain streaming reduction: all loads of a workgroup are in
// flight at once and nothing waits on another workgroup.
//
// sv_finish -- per request, nc2 race workgroups (4096 tokens each) and one
// finishing workgroup, request-major.  Every statistic is complete when it
// starts (stream order).  A race workgroup of a sampled request folds the
// partials of all rows and the gathered logits (one round of loads), draws
// r_t, finds the first rejection n, and runs the exponential race over its
// chunk of the residual (p_n - q_n)+ (or of p_K when nothing was rejected).
// Every race workgroup repeats the same fold in the same order, so all find
// the same n.  The finishing workgroup folds the chunk winners, writes the
// outputs and zeroes every workspace slot of the request; for a greedy
// request it compares the row argmaxes with the drafts instead.  It is the
// only workgroup that waits (for the race workgroups of its own request,
// which precede it in dispatch order); the wait is bounded.
//
// Hand-off slots are 8 bytes and all-zero until written (a written slot never
// has all-zero bits: +0.0 is stored as -0.0), so the finishing workgroup can
// tell a missing value from a present one; accesses are device-coherent
// relaxed atomics (no agent-scope fence, which on gfx950 writes back or
// invalidates a whole L2).
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
constexpr int kWindow = 256;  // requests of draft_offsets a statistics job caches

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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
// gather slot kinds (high word)
enum : uint32_t { kGatherLogit = 1, kGatherBadToken = 2 };
constexpr uint32_t kIdxFailed = 0xffffffffu;  // race slot of a chunk that could not race

struct Layout {
  int J;    // row slots per request: target 0..max_k, then draft 0..max_k-1
  int nc1;  // statistics chunks per row
  int nc2;  // race chunks per row
  size_t stats_off, race_off, pub_off, gather_off, total;
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

Layout make_layout(int32_t B, int32_t V, int32_t max_k, bool bf16) {
  Layout L;
  L.J = 2 * max_k + 1;
  L.nc1 = static_cast<int>(ceil_div(V, stats_chunk(bf16)));
  L.nc2 = static_cast<int>(ceil_div(V, kRaceChunk));
  L.stats_off = 0;
  // sized with the float32 chunk (the smaller one) so either dtype fits
  const size_t stats_bytes =
      static_cast<size_t>(B) * L.J * ceil_div(V, stats_chunk(false)) * sizeof(uint64_t);
  L.race_off = round256(stats_bytes);
  L.pub_off = L.race_off + round256(static_cast<size_t>(B) * L.nc2 * sizeof(uint64_t));
  L.gather_off = L.pub_off + round256(static_cast<size_t>(B) * 4 * sizeof(uint64_t));
  L.total = L.gather_off + round256(static_cast<size_t>(B) * L.J * sizeof(uint64_t));
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
  uint64_t* part;            // [B][J][nc1] statistics partials
  uint64_t* race_part;       // [B][nc2] race chunk winners
  uint64_t* pub;             // [B][4] race record, written by race chunk 0: (fl(m c), log2 sum)
                             // of target row n, the same of draft row n, (c, n | status << 8)
  uint64_t* gather;          // [B][J] row j's logit at its draft token (or the token)
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_at;
  float* q_at;
};

// A request's scalars and the checks every job can make from them.
struct Req {
  int32_t off0, K;
  float T;
  bool slice_ok, temp_ok, greedy;
  __device__ bool sampled() const { return slice_ok && temp_ok && !greedy; }
  __device__ bool greedy_ok() const { return slice_ok && temp_ok && greedy; }
};

__device__ __forceinline__ Req make_req(const Params& p, int32_t o0, int32_t o1, float T) {
  Req r;
  const int64_t K64 = static_cast<int64_t>(o1) - o0;
  r.slice_ok = o0 >= 0 && o1 <= p.n_draft_rows && K64 >= 0 && K64 <= p.max_k;
  r.off0 = o0;
  r.K = r.slice_ok ? static_cast<int32_t>(K64) : 0;
  r.T = T;
  r.greedy = T == 0.f;
  r.temp_ok = (T >= 0.f) && (T < INFINITY) && (r.greedy || r.K == 0 || p.draft != nullptr);
  return r;
}

__device__ __forceinline__ Req load_req(const Params& p, int b) {
  return make_req(p, p.offsets[b], p.offsets[b + 1], p.temperature ? p.temperature[b] : 0.f);
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

__device__ __forceinline__ uint64_t* part_slot(const Params& p, int b, int j, int c) {
  return p.part + (static_cast<int64_t>(b) * (2 * p.max_k + 1) + j) * p.nc1 + c;
}

__device__ __forceinline__ uint64_t* gather_slot(const Params& p, int b, int j) {
  return p.gather + static_cast<int64_t>(b) * (2 * p.max_k + 1) + j;
}

// ------------------------------------------------------------------ statistics kernel

// Largest b in [lo, hi) with key(b) <= row, over global draft_offsets
// (key(b) = offsets[b] + b for target rows); -1 if none.  Used when the row
// is outside the cached window (very uneven K_b).
__device__ int search_global(const Params& p, bool target, int64_t row, int lo, int hi) {
  int ans = -1;
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    const int64_t key = static_cast<int64_t>(p.offsets[mid]) + (target ? mid : 0);
    if (key <= row) {
      ans = mid;
      lo = mid + 1;
    } else {
      hi = mid;
    }
  }
  return ans;
}

template <bool BF16, bool VEC>
__device__ __forceinline__ void load_chunk(const void* base, int64_t row, int64_t V, int64_t e0,
                                           int64_t e_end, uint4 (&buf)[kStatsVecs]) {
  constexpr int EPV = elems_per_vec(BF16);
  const int tid = threadIdx.x;
  const char* rowp = static_cast<const char*>(base) + row * V * (BF16 ? 2 : 4);
  if constexpr (VEC) {
    const uint4* rowv = reinterpret_cast<const uint4*>(rowp);
    const uint32_t ninf = BF16 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
      const int64_t e = e0 + (static_cast<int64_t>(u) * kThreads + tid) * EPV;
      buf[u] = (e < e_end) ? rowv[e / EPV] : make_uint4(ninf, ninf, ninf, ninf);
    }
  } else {
    // rows not 16-byte aligned: element loads at clamped indices (they stay
    // unconditional, so they issue back to back), -inf past the row end
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
      if (u % 4 == 0) asm volatile("" ::: "memory");  // bounds the loads in flight (registers)
      const int64_t e = e0 + (static_cast<int64_t>(u) * kThreads + tid) * EPV;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (BF16) {
          const uint16_t* rp = reinterpret_cast<const uint16_t*>(rowp);
          const int64_t i0 = e + 2 * q, i1 = e + 2 * q + 1;
          const uint32_t lo = rp[i0 < e_end ? i0 : e_end - 1];
          const uint32_t hi = rp[i1 < e_end ? i1 : e_end - 1];
          w[q] = (i0 < e_end ? lo : 0xff80u) | ((i1 < e_end ? hi : 0xff80u) << 16);
          asm volatile("" : "+v"(w[q]));  // hold packed pairs, not unpacked values
        } else {
          const uint32_t* rp = reinterpret_cast<const uint32_t*>(rowp);
          const int64_t i0 = e + q;
          const uint32_t x = rp[i0 < e_end ? i0 : e_end - 1];
          w[q] = i0 < e_end ? x : 0xff800000u;
        }
      }
      buf[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Element k of a thread's pair of vectors (2u, 2u + 1), as float.
template <bool BF16>
__device__ __forceinline__ void unpack_pair(const uint4 (&buf)[kStatsVecs], int pi,
                                            float* xs) {
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
}

// The loaded vectors behind an empty asm: each statistics path unpacks its
// own copy, so the compiler cannot unpack every element once for both paths
// ahead of the branch (that doubles the registers and costs occupancy).
__device__ __forceinline__ void launder(uint4 (&buf)[kStatsVecs]) {
#pragma unroll
  for (int u = 0; u < kStatsVecs; ++u)
    asm volatile("" : "+v"(buf[u].x), "+v"(buf[u].y), "+v"(buf[u].z), "+v"(buf[u].w));
}

// Greedy statistics of one chunk: (max, lowest index holding it).  The
// maximum first (NaN never wins), then the index, searched only by the
// threads whose own maximum it is.
template <bool BF16, bool VEC>
__device__ __forceinline__ void chunk_greedy(const Params& p, uint4 (&buf)[kStatsVecs], int64_t e0,
                                             int b, int j, int c) {
  constexpr int EPV = elems_per_vec(BF16);
  constexpr int PAIR = 2 * EPV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float best = -INFINITY;
#pragma unroll
  for (int pi = 0; pi < kStatsVecs / 2; ++pi) {
    float xs[PAIR];
    unpack_pair<BF16>(buf, pi, xs);
#pragma unroll
    for (int k = 0; k < PAIR; ++k) best = fmaxf(best, xs[k]);
  }
  float bm = best;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o, 64));
  __shared__ float sh_m[kWaves];
  __shared__ int sh_i[kWaves];
  if (lane == 0) sh_m[wave] = bm;
  __syncthreads();
  bm = fmaxf(fmaxf(sh_m[0], sh_m[1]), fmaxf(sh_m[2], sh_m[3]));
  int idx = INT_MAX;
  if (bm > -INFINITY && best == bm) {
    launder(buf);  // unpack again rather than keep every unpacked value alive
#pragma unroll
    for (int pi = kStatsVecs / 2 - 1; pi >= 0; --pi) {
      float xs[PAIR];
      unpack_pair<BF16>(buf, pi, xs);
#pragma unroll
      for (int k = PAIR - 1; k >= 0; --k)
        if (xs[k] == bm)
          idx = static_cast<int>(e0) + ((2 * pi + k / EPV) * kThreads + tid) * EPV + k % EPV;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) idx = min(idx, __shfl_xor(idx, o, 64));
  if (lane == 0) sh_i[wave] = idx;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kWaves; ++w) idx = min(idx, sh_i[w]);
    slot_store(part_slot(p, b, j, c), pack_slot(bm, static_cast<uint32_t>(idx)));
  }
}

// Sampled statistics of one chunk: (m, sum of 2^(z c - fl(m c))), online over
// pairs of vectors.  The thread holding the logit at the row's draft token
// hands it to the finish kernel (chunk 0 reports a token outside [0, V)).
template <bool BF16, bool VEC>
__device__ __forceinline__ void chunk_sampled(const Params& p, uint4 (&buf)[kStatsVecs],
                                              int64_t e0, int64_t e_end, int b, int j, int c,
                                              float cf, bool has_x, int32_t x) {
  constexpr int EPV = elems_per_vec(BF16);
  constexpr int PAIR = 2 * EPV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (has_x && x >= e0 && x < e_end) {
    const int xl = static_cast<int>(x - e0);
    if (tid == (xl / EPV) % kThreads) {
      const int ux = xl / (kThreads * EPV), k = xl % EPV;
      uint32_t wd = 0;
#pragma unroll
      for (int u = 0; u < kStatsVecs; ++u) {
        if (u == ux) {
          const uint32_t w4[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == (BF16 ? k / 2 : k)) wd = w4[q];
        }
      }
      const float z = BF16 ? ((k & 1) ? bf16_hi(wd) : bf16_lo(wd)) : __uint_as_float(wd);
      slot_store(gather_slot(p, b, j), pack_slot(z, kGatherLogit));
    }
  } else if (has_x && (x < 0 || x >= p.V) && c == 0 && tid == 0) {
    slot_store(gather_slot(p, b, j), pack_slot(0.f, kGatherBadToken));
  }
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int pi = 0; pi < kStatsVecs / 2; ++pi) {
    float xs[PAIR];
    unpack_pair<BF16>(buf, pi, xs);
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
  __shared__ float sh_m[kWaves];
  __shared__ float sh_s[kWaves];
  if (lane == 0) {
    sh_m[wave] = m;
    sh_s[wave] = s;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kWaves; ++w) merge_stats(m, s, sh_m[w], sh_s[w], cf);
    slot_store(part_slot(p, b, j, c), pack_slot(m, __float_as_uint(s)));
  }
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) void sv_stats(Params p) {
  constexpr int CHUNK = stats_chunk(BF16);
  const int tid = threadIdx.x;
  const int64_t n_target_rows = static_cast<int64_t>(p.n_draft_rows) + p.B;
  const int64_t g = blockIdx.x;
  const int64_t n_tc = n_target_rows * p.nc1;
  const bool is_target = g < n_tc;
  const int64_t gg = is_target ? g : g - n_tc;
  const int64_t row = gg / p.nc1;
  const int c = static_cast<int>(gg - row * p.nc1);
  const int64_t e0 = static_cast<int64_t>(c) * CHUNK;
  const int64_t e_end = (e0 + CHUNK < p.V) ? e0 + CHUNK : p.V;

  // window of draft_offsets (and temperatures) around the proportional guess;
  // these loads go first, so waiting for them does not wait for the row
  const int64_t n_rows = is_target ? n_target_rows : p.n_draft_rows;
  const int64_t guess = row * p.B / (n_rows > 0 ? n_rows : 1);
  const int w0 = static_cast<int>(
      std::max<int64_t>(0, std::min<int64_t>(guess - kWindow / 2, p.B - kWindow)));
  const int nw = std::min(kWindow, p.B - w0);  // requests w0 .. w0 + nw - 1, keys up to w0 + nw
  __shared__ int64_t sh_key[kWindow + 1];
  __shared__ float sh_T[kWindow];
  {
    const int i = tid;
    if (i <= nw) {
      const int bi = w0 + i;
      sh_key[i] = static_cast<int64_t>(p.offsets[bi]) + (is_target ? bi : 0);
      if (i < nw) sh_T[i] = p.temperature ? p.temperature[bi] : 0.f;
    }
    if (tid == 0 && nw == kWindow) {
      const int bi = w0 + kWindow;
      sh_key[kWindow] = static_cast<int64_t>(p.offsets[bi]) + (is_target ? bi : 0);
    }
  }
  // a target row's loads go out now: its address needs no request data
  uint4 buf[kStatsVecs];
  if (is_target) load_chunk<BF16, VEC>(p.target, row, p.V, e0, e_end, buf);
  __syncthreads();
  __shared__ int sh_b;
  if (tid == 0) {
    int bb = -1;
    if (nw > 0 && sh_key[0] <= row && row < sh_key[nw]) {
      int lo = 0, hi = nw;  // largest i with key <= row
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sh_key[mid] <= row)
          lo = mid;
        else
          hi = mid;
      }
      bb = w0 + lo;
    } else if (nw > 0) {
      bb = search_global(p, is_target, row, 0, p.B);
    }
    sh_b = bb;
  }
  __syncthreads();
  int b = sh_b;
  b = __builtin_amdgcn_readfirstlane(b);
  if (b < 0) return;
  Req r;
  if (b - w0 >= 0 && b - w0 < nw) {
    const int i = b - w0;
    const int64_t k0 = sh_key[i] - (is_target ? b : 0);
    const int64_t k1 = sh_key[i + 1] - (is_target ? b + 1 : 0);
    r = make_req(p, static_cast<int32_t>(k0), static_cast<int32_t>(k1), sh_T[i]);
  } else {
    r = load_req(p, b);
  }
  // the row's position in its request; rows no valid request needs are skipped
  const int64_t first = static_cast<int64_t>(r.off0) + (is_target ? b : 0);
  const int64_t t64 = row - first;
  const bool needed = is_target ? (r.slice_ok && r.temp_ok && t64 >= 0 && t64 <= r.K)
                                : (r.sampled() && t64 >= 0 && t64 < r.K);
  if (!needed) return;
  const int t = static_cast<int>(t64);
  const int j = is_target ? t : p.max_k + 1 + t;
  const bool greedy = is_target && r.greedy;
  // the draft token of this row, whose logit this chunk may hold
  const int32_t x = (!greedy && t < r.K) ? p.tokens[r.off0 + t] : -1;
  if (!is_target) load_chunk<BF16, VEC>(p.draft, row, p.V, e0, e_end, buf);
  if (greedy)
    chunk_greedy<BF16, VEC>(p, buf, e0, b, j, c);
  else
    chunk_sampled<BF16, VEC>(p, buf, e0, e_end, b, j, c, kLog2e / r.T, t < r.K, x);
}

// ------------------------------------------------------------------ finish kernel

// Partials of every row slot of request b (rows a request does not use are
// zero), loaded in one round; after the request's K is known, the used rows
// are folded into sh_m / sh_ls (greedy: sh_ls holds the argmax index bits).
// A missing partial or a non-finite row sets *bad.
template <bool GREEDY>
struct RowPartials {
  uint64_t v[kRowsPerWave][2];  // (row wave + 4 i, chunks lane and lane + 64)
};

template <bool GREEDY>
__device__ __forceinline__ void issue_partials(const Params& p, int b, int nslots,
                                               RowPartials<GREEDY>& rp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int j = wave + i * kWaves;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = lane + 64 * h;
      rp.v[i][h] = (j < nslots && c < p.nc1) ? slot_load(part_slot(p, b, j, c)) : 0u;
    }
  }
}

template <bool GREEDY>
__device__ void fold_rows(const Params& p, int b, const Req& r, int nrows, float cf,
                          RowPartials<GREEDY>& rp, float* sh_m, float* sh_ls, int* bad) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = r.K;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int j = wave + i * kWaves;
    // the request's row using slot j (target t = j <= K, draft t = j - max_k - 1 < K)
    const bool used = j <= K || (j > p.max_k && j - p.max_k - 1 < K);
    const int rrow = j <= K ? j : K + 1 + (j - p.max_k - 1);
    float a = -INFINITY, s = 0.f;
    int ia = INT_MAX;
    bool missing = false;
    if (used && rrow < nrows) {
      for (int c0 = 0; c0 < p.nc1; c0 += 64) {
        const int c = c0 + lane;
        if (c >= p.nc1) break;
        uint64_t v = c0 == 0 ? rp.v[i][0] : (c0 == 64 ? rp.v[i][1] : slot_load(part_slot(p, b, j, c)));
        if (v == 0u) {
          missing = true;
          continue;
        }
        if (GREEDY) {
          if (slot_f(v) > -INFINITY) merge_argmax(a, ia, slot_f(v), static_cast<int>(slot_w(v)));
        } else {
          merge_stats(a, s, slot_f(v), __uint_as_float(slot_w(v)), cf);
        }
      }
    }
    if (missing) atomicOr(bad, 1);
    if (GREEDY)
      wave_merge_argmax(a, ia);
    else
      wave_merge_stats(a, s, cf);
    if (lane == 0 && used && rrow < nrows) {
      const bool finite_max = a > -INFINITY && a < INFINITY;
      if (GREEDY) {
        if (!finite_max) atomicOr(bad, 1);
        sh_ls[rrow] = __int_as_float(ia);
      } else {
        if (!finite_max || !(s < INFINITY)) atomicOr(bad, 1);
        sh_m[rrow] = a;
        sh_ls[rrow] = fast_log2(s);
      }
    }
  }
}

// Zero every slot request b may have written.
__device__ void clear_request(const Params& p, int b, bool race) {
  const int tid = threadIdx.x;
  const int J = 2 * p.max_k + 1;
  for (int i = tid; i < J * p.nc1; i += kThreads) slot_store(part_slot(p, b, i / p.nc1, i % p.nc1), 0u);
  if (tid < J) slot_store(gather_slot(p, b, tid), 0u);
  if (race) {
    for (int i = tid; i < p.nc2; i += kThreads)
      slot_store(p.race_part + static_cast<int64_t>(b) * p.nc2 + i, 0u);
    if (tid < 3) slot_store(p.pub + 4 * static_cast<int64_t>(b) + tid, 0u);
  }
}

// Greedy requests, and requests whose slice or temperature is invalid.
__device__ void finish_greedy(const Params& p, int b, const Req& r, RowPartials<true>& rp) {
  const int tid = threadIdx.x;
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
  const int32_t x = tid < K ? p.tokens[r.off0 + tid] : 0;
  fold_rows<true>(p, b, r, K + 1, 0.f, rp, nullptr, sh_ls, &sh_bad);
  if (tid < K && (x < 0 || x >= p.V)) atomicOr(&sh_bad, 1);
  __syncthreads();
  clear_request(p, b, false);
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
    // clamped, unconditional element loads (they issue back to back)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x = load_logit<BF16>(rowp, v + k < vend ? v + k : vend - 1);
      out[k] = (v + k < vend) ? x : 0.f;
    }
  }
}

// What the race over row n needs: the rounded offsets fl(m c) and log2 sums of
// target row n and (after a rejection) draft row n.
struct RaceRow {
  float mcp, lsp, mcq, lsq, cf;
  int n;
};

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

// Race chunk c of a sampled request: fold, acceptance test, race.  Chunk 0
// also writes p_t(x_t), q_t(x_t) and the record the finishing workgroup
// needs, and the failure outputs if the request turns out invalid.
template <bool BF16, bool VEC>
__device__ void race_item(const Params& p, int b, const Req& r, int c, RowPartials<false>& rp) {
  const int tid = threadIdx.x;
  const int K = r.K;
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  const int64_t drow0 = r.off0;
  const float cf = kLog2e / r.T;
  __shared__ int sh_bad;
  __shared__ float sh_m[kRowsMax];
  __shared__ float sh_ls[kRowsMax];
  __shared__ int sh_n;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  uint64_t gp = 0, gq = 0;
  if (tid < K) {
    gp = slot_load(gather_slot(p, b, tid));
    gq = slot_load(gather_slot(p, b, p.max_k + 1 + tid));
  }
  fold_rows<false>(p, b, r, 2 * K + 1, cf, rp, sh_m, sh_ls, &sh_bad);
  float zp = 0.f, zq = 0.f;
  if (tid < K) {
    if (slot_w(gp) != kGatherLogit || slot_w(gq) != kGatherLogit) atomicOr(&sh_bad, 1);
    zp = slot_f(gp);
    zq = slot_f(gq);
  }
  __syncthreads();
  uint64_t* pub = p.pub + 4 * static_cast<int64_t>(b);
  uint64_t* out = p.race_part + static_cast<int64_t>(b) * p.nc2 + c;
  if (sh_bad) {
    if (c == 0) {
      write_fault(p, b, r);
      if (tid < 2) slot_store(pub + tid, pack_slot(0.f, 0u));
      if (tid == 0) slot_store(pub + 2, pack_slot(cf, kStatusFault << 8));
    }
    if (tid == 0) slot_store(out, pack_slot(-INFINITY, kIdxFailed));
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
    if (c == 0) {
      if (p.p_at) p.p_at[drow0 + tid] = pp;
      if (p.q_at) p.q_at[drow0 + tid] = qq;
    }
  }
  const uint64_t mask = __ballot(reject);
  if (tid == 0) sh_n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : K;
  __syncthreads();
  RaceRow rr;
  rr.n = sh_n;
  rr.cf = cf;
  rr.mcp = scaled_max(sh_m[rr.n], cf);
  rr.lsp = sh_ls[rr.n];
  const bool residual = rr.n < K;
  rr.mcq = residual ? scaled_max(sh_m[K + 1 + rr.n], cf) : 0.f;
  rr.lsq = residual ? sh_ls[K + 1 + rr.n] : 0.f;
  if (c == 0 && tid == 0) {
    slot_store(pub + 0, pack_slot(rr.mcp, __float_as_uint(rr.lsp)));
    slot_store(pub + 1, pack_slot(rr.mcq, __float_as_uint(rr.lsq)));
    slot_store(pub + 2, pack_slot(cf, static_cast<uint32_t>(rr.n) | (kStatusOk << 8)));
  }

  const int64_t esz = BF16 ? 2 : 4;
  const void* prow = static_cast<const char*>(p.target) + (trow0 + rr.n) * p.V * esz;
  const void* qrow =
      residual ? static_cast<const char*>(p.draft) + (drow0 + rr.n) * p.V * esz : nullptr;
  const int64_t v_begin = static_cast<int64_t>(c) * kRaceChunk;
  const int64_t v_end = (v_begin + kRaceChunk < p.V) ? v_begin + kRaceChunk : p.V;
  float lp[kRaceGroups][4], lq[kRaceGroups][4];
#pragma unroll
  for (int gi = 0; gi < kRaceGroups; ++gi) {  // issue every load before any math
    const int64_t g = v_begin / 4 + gi * kThreads + tid;
#pragma unroll
    for (int k = 0; k < 4; ++k) lq[gi][k] = 0.f;
    if (g * 4 < v_end) {
      load4<BF16, VEC>(prow, g * 4, v_end, lp[gi]);
      if (residual) load4<BF16, VEC>(qrow, g * 4, v_end, lq[gi]);
    }
  }
  float bw = 0.f, be = 1.f;  // any w > 0 beats the empty candidate
  int idx = INT_MAX;
#pragma unroll
  for (int gi = 0; gi < kRaceGroups; ++gi) {
    const int64_t g = v_begin / 4 + gi * kThreads + tid;
    if (g * 4 < v_end)
      race_group(lp[gi], lq[gi], residual, rr, g, v_end, b, p.k0, p.k1, bw, be, idx);
  }
  float key = race_key(bw, be, idx);
  __shared__ float sh_key[kWaves];
  __shared__ int sh_idx[kWaves];
  block_argmax(key, idx, sh_key, sh_idx);
  if (tid == 0) slot_store(out, pack_slot(key, static_cast<uint32_t>(idx)));
}

// Folds the chunk winners of a sampled request, writes its outputs and zeroes
// every slot the request used.  Waits (bounded) for the request's race chunks.
template <bool BF16, bool VEC>
__device__ void race_finish(const Params& p, int b, const Req& r) {
  const int tid = threadIdx.x;
  const int K = r.K;
  __shared__ float sh_key[kWaves];
  __shared__ int sh_idx[kWaves];
  __shared__ int sh_fail;
  __shared__ uint64_t sh_pub[3];
  if (tid == 0) sh_fail = 0;
  __syncthreads();
  uint64_t* pub = p.pub + 4 * static_cast<int64_t>(b);
  const int32_t x = (tid < K) ? p.tokens[r.off0 + tid] : 0;  // overlaps the waits
  if (tid < 3) {
    const uint64_t v = slot_wait(pub + tid);
    if (v == 0u) atomicOr(&sh_fail, 1);
    sh_pub[tid] = v;
  }
  float key = -INFINITY;
  int idx = INT_MAX;
  for (int i = tid; i < p.nc2; i += kThreads) {
    const uint64_t v = slot_wait(p.race_part + static_cast<int64_t>(b) * p.nc2 + i);
    if (v == 0u || slot_w(v) == kIdxFailed) {
      atomicOr(&sh_fail, 1);
      continue;
    }
    merge_argmax(key, idx, slot_f(v), static_cast<int>(slot_w(v)));
  }
  block_argmax(key, idx, sh_key, sh_idx);  // its barriers also publish sh_fail and sh_pub
  clear_request(p, b, true);
  RaceRow rr;
  rr.mcp = slot_f(sh_pub[0]);
  rr.lsp = __uint_as_float(slot_w(sh_pub[0]));
  rr.mcq = slot_f(sh_pub[1]);
  rr.lsq = __uint_as_float(slot_w(sh_pub[1]));
  rr.cf = slot_f(sh_pub[2]);
  rr.n = static_cast<int>(slot_w(sh_pub[2]) & 0xffu);
  const uint32_t status = slot_w(sh_pub[2]) >> 8;
  if (sh_pub[2] != 0u && status == kStatusFault) return;  // chunk 0 wrote the failure
  if (sh_fail) {
    if (tid == 0) p.accept_len[b] = -1;
    return;
  }
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
  if (tid <= K) p.out_tokens[trow0 + tid] = (tid < n) ? x : (tid == n ? idx : -1);
  if (tid == 0) p.accept_len[b] = n;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sv_finish(Params p) {
  const int64_t g = blockIdx.x;
  const int b = static_cast<int>(g / (p.nc2 + 1));
  const int s = static_cast<int>(g - static_cast<int64_t>(b) * (p.nc2 + 1));
  const Req r = load_req(p, b);
  if (s < p.nc2) {
    // the partials go out together with the request's scalars (one round trip)
    RowPartials<false> rp;
    issue_partials<false>(p, b, 2 * p.max_k + 1, rp);
    if (!r.sampled()) return;
    race_item<BF16, VEC>(p, b, r, s, rp);
  } else {
    RowPartials<true> rp;
    if (p.temperature) {
      if (r.sampled()) {
        race_finish<BF16, VEC>(p, b, r);
        return;
      }
    }
    issue_partials<true>(p, b, p.max_k + 1, rp);
    finish_greedy(p, b, r, rp);
  }
}

// ------------------------------------------------------------------ host side

bool shape_ok(int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows) {
  return B >= 1 && V >= 1 && max_k >= 0 && max_k <= SV_KMAX && n_draft_rows >= 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <bool BF16, bool VEC>
int launch(const Params& prm, int64_t grid1, int64_t grid2, hipStream_t stream, void* ev0,
           void* ev1) {
  if (ev0 && hipEventRecord(static_cast<hipEvent_t>(ev0), stream) != hipSuccess)
    return SV_ERR_LAUNCH;
  hipLaunchKernelGGL((sv_stats<BF16, VEC>), dim3(static_cast<uint32_t>(grid1)), dim3(kThreads), 0,
                     stream, prm);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  if (ev1 && hipEventRecord(static_cast<hipEvent_t>(ev1), stream) != hipSuccess)
    return SV_ERR_LAUNCH;
  hipLaunchKernelGGL((sv_finish<BF16, VEC>), dim3(static_cast<uint32_t>(grid2)), dim3(kThreads), 0,
                     stream, prm);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
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
  // every target row, then every draft row (none when every request is greedy)
  const int64_t grid1 = ((all_greedy ? 1 : 2) * static_cast<int64_t>(n_draft_rows) + B) *
                        static_cast<int64_t>(L.nc1);
  const int64_t grid2 = static_cast<int64_t>(B) * (L.nc2 + 1);
  if (grid1 > INT32_MAX || grid2 > INT32_MAX) return SV_ERR_SHAPE;
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
  prm.nc2 = L.nc2;
  prm.part = reinterpret_cast<uint64_t*>(ws + L.stats_off);
  prm.race_part = reinterpret_cast<uint64_t*>(ws + L.race_off);
  prm.pub = reinterpret_cast<uint64_t*>(ws + L.pub_off);
  prm.gather = reinterpret_cast<uint64_t*>(ws + L.gather_off);
  prm.accept_len = accept_len;
  prm.out_tokens = out_tokens;
  prm.p_at = p_at;
  prm.q_at = q_at;
  const int64_t row_bytes = static_cast<int64_t>(V) * (bf16 ? 2 : 4);
  const bool vec = row_bytes % 16 == 0 && aligned16(target) && (!draft || aligned16(draft));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch<true, true>(prm, grid1, grid2, s, ev0, ev1)
               : launch<true, false>(prm, grid1, grid2, s, ev0, ev1);
  return vec ? launch<false, true>(prm, grid1, grid2, s, ev0, ev1)
             : launch<false, false>(prm, grid1, grid2, s, ev0, ev1);
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
