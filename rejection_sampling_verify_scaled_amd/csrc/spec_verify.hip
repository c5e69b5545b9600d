// spec_verify.hip -- gfx950 kernel and C ABI of the speculative-decoding verify step.
//
// What is computed is stated in include/spec_verify.h (the accept / residual /
// bonus rule of "Decodificación Especulativa y EAGLE", section "La Regla de
// Exactitud", and its greedy case).  How it runs on MI355X: one launch whose
// workgroups each take one job from a fixed schedule.
//
// Jobs of request b:
//   SA  statistics of a sampled request: one job per (row, 64 KiB V-chunk) of
//       its K+1 target and K draft rows.  Streams the chunk with 16-byte
//       loads and reduces it to one 8-byte partial (max, sum of
//       2^(z c - fl(max c))), c = log2(e) / T, then stores it and exits.
//   FA  finisher of a sampled request: collects the partials, folds them into
//       per-row (max, log2 sum), gathers p_t(x_t) and q_t(x_t), draws r_t,
//       finds the first rejection n with a wave ballot, and publishes n with
//       the statistics of row n.
//   R   race of a sampled request: one job per 4096-token chunk of row n, the
//       exponential race over the residual (p_n - q_n)+ after a rejection or
//       over p_K otherwise, plus one job that folds the chunk winners and
//       writes the outputs.
//   SB  statistics of a greedy request: (max, lowest argmax index) per chunk
//       of its K+1 target rows (draft rows are never read).
//   FB  finisher of a greedy request: first draft that differs from the row
//       argmax; writes the outputs.  Also reports requests with a bad slice
//       or temperature.
// A job that does not apply to request b (e.g. SA of a greedy request) exits
// at once.
//
// Schedule: request b's SA jobs sit at "time" b, SB at B + b, FA at b + d1,
// R at b + d1 + d2 and FB at B + b + d3; the grid lists times in order and,
// inside a time, the jobs in the order SA, SB, FA, R, FB.  The lags are
// about two generations of resident workgroups, so every job comes well
// after the jobs it depends on, sampled requests stream first, and their
// finishing and races overlap the streaming of greedy requests and of later
// sampled requests.
//
// Hand-offs between workgroups use 8-byte slots in the workspace that are
// all-zero until written (a written slot never has all-zero bits: +0.0 is
// stored as -0.0).  Producers store with a device-coherent (sc1) store and
// exit; consumers poll with device-coherent loads, then write the slot back
// to zero, so the workspace is all-zero again after every call.  No
// agent-scope release/acquire fence is used (on gfx950 those write back or
// invalidate the XCD's whole L2).  A consumer only waits for jobs that come
// earlier in the grid; the earliest waiting job waits only for jobs that
// never wait, so with in-order dispatch every wait ends.  Waits are also
// bounded (kSpinLimit polls); an expired wait reports accept_len = -1.
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
// Consumers sit this many grid slots after their producers: about two
// generations of resident workgroups (5 per CU here), so a consumer is
// dispatched once its producers have finished rather than spinning beside
// them.
#ifndef SV_FINISH_LAG_SLOTS
#define SV_FINISH_LAG_SLOTS 4096  // statistics -> finisher
#endif
#ifndef SV_RACE_LAG_SLOTS
#define SV_RACE_LAG_SLOTS 2048  // finisher -> race
#endif

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
  size_t stats_off, race_off, pub_off, total;
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
  L.total = L.pub_off + round256(static_cast<size_t>(B) * 4 * sizeof(uint64_t));
  return L;
}

// Jobs in schedule order inside one time step.
enum Job : int { kSA = 0, kSB = 1, kFA = 2, kR = 3, kFB = 4, kJobs = 5 };

// A run of time steps with the same set of jobs present.
struct Region {
  int64_t g0;    // first grid slot
  int32_t k0;    // first time step
  int32_t seg;   // slots per time step
  int32_t mask;  // jobs present (bit per Job)
  int32_t pad;
};
constexpr int kMaxRegions = 12;

struct Params {
  const void* target;
  const void* draft;
  const int32_t* offsets;
  const int32_t* tokens;
  const float* temperature;  // NULL: every request greedy
  uint32_t k0, k1;           // Philox key
  int32_t B, V, max_k, n_draft_rows, nc1, nc2;
  uint64_t* part;       // [B][J][nc1] statistics partials
  uint64_t* race_part;  // [B][nc2] race chunk winners
  uint64_t* pub;        // [B][4] published record: (fl(m c), log2 sum) of target row n,
                        // the same of draft row n, (c, n), (1, status) -- last written
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_at;
  float* q_at;
  int32_t job_len[kJobs];  // slots each job kind takes per request
  int32_t job_off[kJobs];  // time step of request 0's job
  int32_t n_regions;
  Region reg[kMaxRegions];
};

// Per-request checks every job can make from the request's scalars.
struct Req {
  int32_t off0, K;
  float T;
  bool slice_ok, temp_ok, greedy;
  __device__ bool sampled() const { return slice_ok && temp_ok && !greedy; }
  __device__ bool greedy_ok() const { return slice_ok && temp_ok && greedy; }
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

// ------------------------------------------------------------------ statistics jobs

template <bool BF16, bool VEC>
__device__ void stats_job(const Params& p, int b, int slot, bool sampled_job) {
  constexpr int EPV = elems_per_vec(BF16);
  constexpr int CHUNK = stats_chunk(BF16);
  constexpr int PAIR = 2 * EPV;  // elements folded per online step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = slot % p.nc1;
  const int j = slot / p.nc1;

  const Req r = load_req(p, b);
  if (sampled_job ? !r.sampled() : !r.greedy_ok()) return;
  const void* base;
  int64_t row;
  if (j <= p.max_k) {
    if (j > r.K) return;
    base = p.target;
    row = static_cast<int64_t>(r.off0) + b + j;
  } else {
    const int t = j - p.max_k - 1;
    if (t >= r.K) return;
    base = p.draft;
    row = static_cast<int64_t>(r.off0) + t;
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
  if (r.greedy) {
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
  if (tid == 0) slot_store(part_slot(p, b, j, c), result);
}

// ------------------------------------------------------------------ finishers

// Waits for the partials of rows 0..nrows-1 (row r: slot j = r for r <= K,
// j = max_k + r - K for the draft rows), folds them into sh_m / sh_ls and
// zeroes the slots.  Greedy: sh_ls holds the argmax index bits.  Sets *bad on
// a non-finite row, a NaN sum or an expired wait.
template <bool GREEDY>
__device__ void fold_partials(const Params& p, int b, int K, float cf, int nrows, float* sh_m,
                              float* sh_ls, int* bad) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
      const int j = (row <= K) ? row : p.max_k + row - K;
      v[i] = (row < nrows && c < p.nc1) ? slot_load(part_slot(p, b, j, c)) : 1u;
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int row = wave + i * kWaves;
      if (row < nrows && c < p.nc1) {
        const int j = (row <= K) ? row : p.max_k + row - K;
        uint64_t* slot = part_slot(p, b, j, c);
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
__device__ void finish_sampled(const Params& p, int b) {
  const Req r = load_req(p, b);
  if (!r.sampled()) return;
  const int tid = threadIdx.x;
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

__device__ void finish_greedy(const Params& p, int b) {
  const Req r = load_req(p, b);
  const int tid = threadIdx.x;
  if (!r.slice_ok) {
    if (tid == 0) p.accept_len[b] = -1;
    return;
  }
  if (!r.temp_ok) {
    write_fault(p, b, r);
    return;
  }
  if (!r.greedy) return;
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

// ------------------------------------------------------------------ race jobs

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
__device__ void race_chunk(const Params& p, int b, int c) {
  const Req r = load_req(p, b);
  if (!r.sampled()) return;
  const int tid = threadIdx.x;
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
__device__ void race_finish(const Params& p, int b) {
  const Req r = load_req(p, b);
  if (!r.sampled()) return;
  const int tid = threadIdx.x;
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
__global__ __launch_bounds__(kThreads) void sv_verify(Params p) {
  const int64_t g = blockIdx.x;
  int ri = 0;
  while (ri + 1 < p.n_regions && g >= p.reg[ri + 1].g0) ++ri;
  const Region& R = p.reg[ri];
  const int64_t rel = g - R.g0;
  const int k = R.k0 + static_cast<int>(rel / R.seg);
  int o = static_cast<int>(rel % R.seg);
  for (int job = 0; job < kJobs; ++job) {
    if (!(R.mask & (1 << job))) continue;
    if (o >= p.job_len[job]) {
      o -= p.job_len[job];
      continue;
    }
    const int b = k - p.job_off[job];
    switch (job) {
      case kSA: stats_job<BF16, VEC>(p, b, o, true); break;
      case kFA: finish_sampled<BF16>(p, b); break;
      case kR:
        if (o < p.nc2)
          race_chunk<BF16, VEC>(p, b, o);
        else
          race_finish<BF16, VEC>(p, b);
        break;
      case kSB: stats_job<BF16, VEC>(p, b, o, false); break;
      default: finish_greedy(p, b); break;
    }
    return;
  }
}

// ------------------------------------------------------------------ host side

bool shape_ok(int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows) {
  return B >= 1 && V >= 1 && max_k >= 0 && max_k <= SV_KMAX && n_draft_rows >= 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Lays the jobs out in time steps (see the schedule at the top); returns the
// grid size, or -1 if it does not fit the region table.
int64_t build_schedule(Params& prm, int B, bool all_greedy) {
  const int J = 2 * prm.max_k + 1;
  int len[kJobs];
  len[kSA] = all_greedy ? 0 : J * prm.nc1;
  len[kSB] = (prm.max_k + 1) * prm.nc1;
  len[kFA] = all_greedy ? 0 : 1;
  len[kR] = all_greedy ? 0 : prm.nc2 + 1;
  len[kFB] = 1;
  const int gb = all_greedy ? 0 : B;  // greedy statistics start after the sampled ones
  const int64_t d1 = ceil_div(SV_FINISH_LAG_SLOTS, std::max(len[kSA], 1));
  const int64_t d2 = ceil_div(SV_RACE_LAG_SLOTS, std::max(len[kSA] + len[kSB], 1));
  const int64_t d3 = ceil_div(SV_FINISH_LAG_SLOTS, len[kSB]);
  const int64_t cap = 4 * static_cast<int64_t>(B);  // keeps every offset small
  int off[kJobs];
  off[kSA] = 0;
  off[kSB] = gb;
  off[kFA] = static_cast<int>(std::min(d1, cap));
  off[kR] = static_cast<int>(std::min(d1 + d2, cap));
  off[kFB] = static_cast<int>(gb + std::min(d3, cap));
  int bounds[2 * kJobs];
  int nb = 0;
  for (int j = 0; j < kJobs; ++j) {
    prm.job_len[j] = len[j];
    prm.job_off[j] = off[j];
    if (len[j] == 0) continue;
    bounds[nb++] = off[j];
    bounds[nb++] = off[j] + B;
  }
  std::sort(bounds, bounds + nb);
  nb = static_cast<int>(std::unique(bounds, bounds + nb) - bounds);
  int64_t g = 0;
  prm.n_regions = 0;
  for (int i = 0; i + 1 < nb; ++i) {
    const int ka = bounds[i], kb = bounds[i + 1];
    int mask = 0, seg = 0;
    for (int j = 0; j < kJobs; ++j)
      if (len[j] > 0 && off[j] <= ka && ka < off[j] + B) {
        mask |= 1 << j;
        seg += len[j];
      }
    if (seg == 0) continue;
    if (prm.n_regions == kMaxRegions) return -1;
    Region& R = prm.reg[prm.n_regions++];
    R.g0 = g;
    R.k0 = ka;
    R.seg = seg;
    R.mask = mask;
    R.pad = 0;
    g += static_cast<int64_t>(kb - ka) * seg;
  }
  return g;
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
  prm.nc2 = L.nc2;
  prm.part = reinterpret_cast<uint64_t*>(ws + L.stats_off);
  prm.race_part = reinterpret_cast<uint64_t*>(ws + L.race_off);
  prm.pub = reinterpret_cast<uint64_t*>(ws + L.pub_off);
  prm.accept_len = accept_len;
  prm.out_tokens = out_tokens;
  prm.p_at = p_at;
  prm.q_at = q_at;
  const int64_t grid = build_schedule(prm, B, all_greedy);
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
