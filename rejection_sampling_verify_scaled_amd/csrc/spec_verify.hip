// spec_verify.hip -- gfx950 kernels and C ABI of the speculative-decoding verify step.
//
// What is computed is stated in include/spec_verify.h (the accept / residual /
// bonus rule of "Decodificación Especulativa y EAGLE", section "La Regla de
// Exactitud", and its greedy case).  How it runs on MI355X:
//
//   launch 1, sv_row_stats -- one workgroup per (request, row slot, V-chunk).
//     Streams the chunk with 16-byte loads and reduces it to one 8-byte
//     partial: (max, sum of 2^((z - max) * log2(e) / T)) for rows a sampled
//     request needs, (max, lowest argmax index) for rows of a greedy request.
//     Draft rows of greedy requests are never read.  This launch carries all
//     of the HBM traffic and is bound by it.
//   launch 2, sv_accept_race -- one workgroup per (request, race chunk).
//     Every workgroup of a request folds the partials into per-row (max, lse),
//     gathers p_t(x_t), q_t(x_t), draws r_t and finds the first rejection n
//     with a wave ballot (redundantly, so no workgroup waits for another).  It
//     then runs the exponential race over its chunk of row n: residual
//     (p_n - q_n)+ after a rejection, bonus p_K otherwise.  The last
//     workgroup of a request to finish (atomic counter) folds the chunk
//     winners and writes the request's outputs.  Greedy requests are finished
//     by their first workgroup from the argmax partials.
//
// Race keys are kept in base-2 logs: key_v = log2 w_v - log2(-log2 U_v), a
// strictly increasing function of the natural-log key ln w_v - ln E_v, so the
// winner is the same token.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;                  // 4 wave64s per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kStatsVecs = 8;                  // 16-byte loads per thread per stats chunk
constexpr int kRaceGroups = 4;                 // 4-token Philox groups per thread per race chunk
constexpr int kRaceChunk = kThreads * kRaceGroups * 4;  // tokens per race chunk
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

// Larger max wins; a chunk's sum is rescaled to the common max.  A side with
// max == -inf contributes 0 * s, which keeps a NaN sum NaN.
__device__ __forceinline__ void merge_stats(float& m, float& s, float m2, float s2, float cf) {
  const float M = fmaxf(m, m2);
  const float f1 = (m == -INFINITY) ? 0.f : fast_exp2((m - M) * cf);
  const float f2 = (m2 == -INFINITY) ? 0.f : fast_exp2((m2 - M) * cf);
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

struct Layout {
  int J;        // row slots per request: target 0..max_k, then draft 0..max_k-1
  int nc1;      // stats chunks per row
  int nc2;      // race chunks per row
  size_t stats_off, race_off, count_off, total;
};

__host__ __device__ inline int ceil_div(int64_t a, int64_t b) {
  return static_cast<int>((a + b - 1) / b);
}

Layout make_layout(int32_t B, int32_t V, int32_t max_k, bool bf16) {
  Layout L;
  L.J = 2 * max_k + 1;
  L.nc1 = ceil_div(V, stats_chunk(bf16));
  L.nc2 = ceil_div(V, kRaceChunk);
  L.stats_off = 0;
  const size_t stats_bytes = static_cast<size_t>(B) * L.J * ceil_div(V, stats_chunk(false)) * 8;
  L.race_off = (stats_bytes + 255) / 256 * 256;
  const size_t race_bytes = static_cast<size_t>(B) * L.nc2 * 8;
  L.count_off = L.race_off + (race_bytes + 255) / 256 * 256;
  L.total = L.count_off + (static_cast<size_t>(B) * 4 + 255) / 256 * 256;
  return L;
}

// ------------------------------------------------------------------ launch 1

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sv_row_stats(
    const void* __restrict__ target, const void* __restrict__ draft,
    const int32_t* __restrict__ offsets, const float* __restrict__ temperature, int32_t B,
    int32_t V, int32_t max_k, int32_t n_draft_rows, int32_t nc1, float2* __restrict__ part,
    uint32_t* __restrict__ counters) {
  constexpr int EPV = elems_per_vec(BF16);
  constexpr int CHUNK = stats_chunk(BF16);
  const int J = 2 * max_k + 1;
  const int64_t bid = blockIdx.x;
  const int c = static_cast<int>(bid % nc1);
  const int j = static_cast<int>((bid / nc1) % J);
  const int b = static_cast<int>(bid / (static_cast<int64_t>(nc1) * J));
  const int tid = threadIdx.x;

  // launch 2 counts finished race chunks per request from zero
  if (bid == 0)
    for (int i = tid; i < B; i += kThreads) counters[i] = 0u;

  const int32_t off0 = offsets[b];
  const int32_t off1 = offsets[b + 1];
  const int32_t K = off1 - off0;
  if (off0 < 0 || off1 > n_draft_rows || K < 0 || K > max_k) return;
  const float T = temperature ? temperature[b] : 0.f;
  if (!(T >= 0.f) || !(T < INFINITY)) return;  // launch 2 reports the failure
  const bool greedy = (T == 0.f);
  const void* base;
  int64_t row;
  if (j <= max_k) {
    if (j > K) return;
    base = target;
    row = static_cast<int64_t>(off0) + b + j;
  } else {
    const int t = j - max_k - 1;
    if (greedy || t >= K || draft == nullptr) return;
    base = draft;
    row = static_cast<int64_t>(off0) + t;
  }

  const int64_t e0 = static_cast<int64_t>(c) * CHUNK;
  const int64_t e_end = (e0 + CHUNK < V) ? e0 + CHUNK : V;

  // gather this thread's elements in increasing index order
  float x[kStatsVecs * EPV];
  if constexpr (VEC) {
    const uint4* rowv = reinterpret_cast<const uint4*>(
        static_cast<const char*>(base) + row * static_cast<int64_t>(V) * (BF16 ? 2 : 4));
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
    const int64_t rbase = row * static_cast<int64_t>(V);
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
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float2 result;

  if (greedy) {
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
    const float cf = kLog2e / T;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kStatsVecs * EPV; ++i) m = fmaxf(m, x[i]);
    const float ms = (m == -INFINITY) ? 0.f : m;  // keeps NaN visible when no finite max
    float acc[kStatsVecs];
#pragma unroll
    for (int u = 0; u < kStatsVecs; ++u) {
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < EPV; ++k) a += fast_exp2((x[u * EPV + k] - ms) * cf);
      acc[u] = a;
    }
#pragma unroll
    for (int h = kStatsVecs / 2; h >= 1; h >>= 1)
#pragma unroll
      for (int u = 0; u < h; ++u) acc[u] += acc[u + h];
    float s = acc[0];
    if (m == -INFINITY) {
      // all of this thread's elements are -inf or NaN: s is 0 or NaN already
      m = -INFINITY;
    }
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
  if (tid == 0) part[(static_cast<int64_t>(b) * J + j) * nc1 + c] = result;
}

// ------------------------------------------------------------------ launch 2

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

// Race over tokens [v_begin, v_end) of one row.  residual: w_v = p_v - q_v
// (tokens with w_v <= 0 are out); otherwise log2 w_v = (z_v - mp) * cf.
template <bool BF16, bool VEC>
__device__ void race_span(const void* prow, const void* qrow, bool residual, float mp, float lsp,
                          float mq, float lsq, float cf, int64_t v_begin, int64_t v_end,
                          uint32_t pos, uint32_t b, uint32_t k0, uint32_t k1, float& best_key,
                          int& best_idx) {
  for (int64_t g = v_begin / 4 + threadIdx.x; g * 4 < v_end; g += kThreads) {
    const int64_t v = g * 4;
    float zp[4], zq[4];
    load4<BF16, VEC>(prow, v, v_end, zp);
    if (residual) load4<BF16, VEC>(qrow, v, v_end, zq);
    const Philox4 r = philox4x32_10(static_cast<uint32_t>(g), pos, b, 0u, k0, k1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (v + k >= v_end) break;
      const float e2 = -fast_log2(uniform_open01(r.w[k]));  // E / ln 2
      float lw;
      if (residual) {
        const float p = fast_exp2((zp[k] - mp) * cf - lsp);
        const float q = fast_exp2((zq[k] - mq) * cf - lsq);
        const float w = p - q;
        if (!(w > 0.f)) continue;
        lw = fast_log2(w);
      } else {
        lw = (zp[k] - mp) * cf;
      }
      const float key = lw - fast_log2(e2);
      if (key > best_key) {
        best_key = key;
        best_idx = static_cast<int>(v + k);
      }
    }
  }
}

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

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sv_accept_race(
    const void* __restrict__ target, const void* __restrict__ draft,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tokens,
    const float* __restrict__ temperature, uint32_t k0, uint32_t k1, int32_t V, int32_t max_k,
    int32_t n_draft_rows, int32_t nc1, int32_t nc2, const float2* __restrict__ part,
    float2* __restrict__ race_part, uint32_t* __restrict__ counters,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ p_at, float* __restrict__ q_at) {
  const int b = blockIdx.x / nc2;
  const int c = blockIdx.x % nc2;
  const int tid = threadIdx.x;
  const int J = 2 * max_k + 1;

  const int32_t off0 = offsets[b];
  const int32_t off1 = offsets[b + 1];
  const int32_t K = off1 - off0;
  if (off0 < 0 || off1 > n_draft_rows || K < 0 || K > max_k) {
    if (c == 0 && tid == 0) accept_len[b] = -1;
    return;
  }
  const float T = temperature ? temperature[b] : 0.f;
  const bool greedy = (T == 0.f);
  if (greedy && c != 0) return;
  const int64_t trow0 = static_cast<int64_t>(off0) + b;  // target row t: trow0 + t
  const int64_t drow0 = off0;                            // draft row t: drow0 + t

  __shared__ int sh_bad;
  __shared__ float sh_m[2 * SV_KMAX + 1];
  __shared__ float sh_ls[2 * SV_KMAX + 1];  // log2 of the row's scaled sum; greedy: argmax
  __shared__ int sh_n;
  __shared__ float sh_key[kWaves];
  __shared__ int sh_idx[kWaves];
  __shared__ int sh_last;

  if (tid == 0)
    sh_bad = (!(T >= 0.f) || !(T < INFINITY) || (!greedy && K > 0 && draft == nullptr)) ? 1 : 0;
  __syncthreads();
  const float cf = greedy ? 0.f : kLog2e / T;
  if (tid < K) {
    const int32_t x = tokens[off0 + tid];
    if (x < 0 || x >= V) atomicOr(&sh_bad, 1);
  }
  const int nrows = greedy ? K + 1 : 2 * K + 1;
  if (tid < nrows) {  // reads stay inside request b's partials even for a bad request
    // rows 0..K are target rows, rows K+1..2K draft rows 0..K-1
    const int j = (tid <= K) ? tid : (max_k + 1 + tid - K - 1);
    const float2* pp = part + (static_cast<int64_t>(b) * J + j) * nc1;
    if (greedy) {
      float best = -INFINITY;
      int idx = INT_MAX;
      for (int i = 0; i < nc1; ++i) {
        const float2 r = pp[i];
        merge_argmax(best, idx, r.x, __float_as_int(r.y));
      }
      if (!(best > -INFINITY && best < INFINITY)) atomicOr(&sh_bad, 1);
      sh_ls[tid] = __int_as_float(idx);
    } else {
      float m = -INFINITY, s = 0.f;
      for (int i = 0; i < nc1; ++i) {
        const float2 r = pp[i];
        merge_stats(m, s, r.x, r.y, cf);
      }
      if (!(m > -INFINITY && m < INFINITY) || !(s < INFINITY)) atomicOr(&sh_bad, 1);
      sh_m[tid] = m;
      sh_ls[tid] = fast_log2(s);
    }
  }
  __syncthreads();

  if (sh_bad) {
    if (c == 0) {
      if (tid <= K) out_tokens[trow0 + tid] = -1;
      if (tid < K) {
        if (p_at) p_at[drow0 + tid] = NAN;
        if (q_at) q_at[drow0 + tid] = NAN;
      }
      if (tid == 0) accept_len[b] = -1;
    }
    return;
  }

  if (greedy) {
    // first t < K whose draft differs from the argmax; stop token argmax row n
    bool mismatch = false;
    int32_t x = 0;
    if (tid < K) {
      x = tokens[off0 + tid];
      mismatch = (__float_as_int(sh_ls[tid]) != x);
    }
    const uint64_t mask = __ballot(mismatch);
    if (tid < 64 && tid == 0) sh_n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : K;
    __syncthreads();
    const int n = sh_n;
    if (tid <= K) {
      const int32_t y = __float_as_int(sh_ls[n]);
      out_tokens[trow0 + tid] = (tid < n) ? x : (tid == n ? y : -1);
    }
    if (tid < K) {
      if (p_at) p_at[drow0 + tid] = NAN;
      if (q_at) q_at[drow0 + tid] = NAN;
    }
    if (tid == 0) accept_len[b] = n;
    return;
  }

  // ratio test r_t * q_t(x_t) < p_t(x_t), left to right (wave 0 holds t < K <= 8)
  bool reject = false;
  int32_t x = 0;
  if (tid < K) {
    x = tokens[off0 + tid];
    const float zp = load_logit<BF16>(target, (trow0 + tid) * V + x);
    const float zq = load_logit<BF16>(draft, (drow0 + tid) * V + x);
    const float p = fast_exp2((zp - sh_m[tid]) * cf - sh_ls[tid]);
    const float q = fast_exp2((zq - sh_m[K + 1 + tid]) * cf - sh_ls[K + 1 + tid]);
    const float r = uniform_open01(philox4x32_10(0u, tid, b, 1u, k0, k1).w[0]);
    reject = !(r * q < p);
    if (c == 0) {
      if (p_at) p_at[drow0 + tid] = p;
      if (q_at) q_at[drow0 + tid] = q;
    }
  }
  const uint64_t mask = __ballot(reject);
  if (tid == 0) sh_n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : K;
  __syncthreads();
  const int n = sh_n;
  const bool residual = n < K;

  const void* prow = static_cast<const char*>(target) + (trow0 + n) * V * (BF16 ? 2 : 4);
  const void* qrow =
      residual ? static_cast<const char*>(draft) + (drow0 + n) * V * (BF16 ? 2 : 4) : nullptr;
  const float mp = sh_m[n], lsp = sh_ls[n];
  const float mq = residual ? sh_m[K + 1 + n] : 0.f;
  const float lsq = residual ? sh_ls[K + 1 + n] : 0.f;

  float key = -INFINITY;
  int idx = INT_MAX;
  const int64_t v_begin = static_cast<int64_t>(c) * kRaceChunk;
  const int64_t v_end = (v_begin + kRaceChunk < V) ? v_begin + kRaceChunk : V;
  race_span<BF16, VEC>(prow, qrow, residual, mp, lsp, mq, lsq, cf, v_begin, v_end, n, b, k0, k1,
                       key, idx);
  block_argmax(key, idx, sh_key, sh_idx);

  if (tid == 0) {
    race_part[static_cast<int64_t>(b) * nc2 + c] = make_float2(key, __int_as_float(idx));
    const uint32_t done = __hip_atomic_fetch_add(&counters[b], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh_last = (done == static_cast<uint32_t>(nc2 - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();

  // last workgroup of request b: fold the chunk winners
  key = -INFINITY;
  idx = INT_MAX;
  for (int i = tid; i < nc2; i += kThreads) {
    const float2 r = race_part[static_cast<int64_t>(b) * nc2 + i];
    merge_argmax(key, idx, r.x, __float_as_int(r.y));
  }
  block_argmax(key, idx, sh_key, sh_idx);
  if (idx == INT_MAX) {
    // no token had p > q (rounding can only cause this when p == q): race on p_n
    key = -INFINITY;
    race_span<BF16, VEC>(prow, nullptr, false, mp, lsp, 0.f, 0.f, cf, 0, V, n, b, k0, k1, key,
                         idx);
    block_argmax(key, idx, sh_key, sh_idx);
  }
  if (tid <= K) out_tokens[trow0 + tid] = (tid < n) ? x : (tid == n ? idx : -1);
  if (tid == 0) {
    accept_len[b] = n;
    counters[b] = 0u;
  }
}

// ------------------------------------------------------------------ host side

bool shape_ok(int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows) {
  return B >= 1 && V >= 1 && max_k >= 0 && max_k <= SV_KMAX && n_draft_rows >= 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <bool BF16, bool VEC>
int launch_all(const void* target, const void* draft, int32_t B, int32_t V, int32_t max_k,
               int32_t n_draft_rows, const int32_t* offsets, const int32_t* tokens,
               const float* temperature, uint64_t seed, int32_t* accept_len,
               int32_t* out_tokens, float* p_at, float* q_at, void* workspace,
               hipStream_t stream, bool all_greedy, void* const* events) {
  const Layout L = make_layout(B, V, max_k, BF16);
  char* ws = static_cast<char*>(workspace);
  float2* part = reinterpret_cast<float2*>(ws + L.stats_off);
  float2* race_part = reinterpret_cast<float2*>(ws + L.race_off);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + L.count_off);
  const int64_t grid1 = static_cast<int64_t>(B) * L.J * L.nc1;
  const int nc2 = all_greedy ? 1 : L.nc2;
  const int64_t grid2 = static_cast<int64_t>(B) * nc2;
  if (grid1 > INT32_MAX || grid2 > INT32_MAX) return SV_ERR_SHAPE;
  if (events && hipEventRecord(static_cast<hipEvent_t>(events[0]), stream) != hipSuccess)
    return SV_ERR_LAUNCH;
  hipLaunchKernelGGL((sv_row_stats<BF16, VEC>), dim3(static_cast<uint32_t>(grid1)),
                     dim3(kThreads), 0, stream, target, draft, offsets, temperature, B, V, max_k,
                     n_draft_rows, L.nc1, part, counters);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  if (events && hipEventRecord(static_cast<hipEvent_t>(events[1]), stream) != hipSuccess)
    return SV_ERR_LAUNCH;
  hipLaunchKernelGGL((sv_accept_race<BF16, VEC>), dim3(static_cast<uint32_t>(grid2)),
                     dim3(kThreads), 0, stream, target, draft, offsets, tokens, temperature,
                     static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), V, max_k,
                     n_draft_rows, L.nc1, nc2, part, race_part, counters, accept_len, out_tokens,
                     p_at, q_at);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  if (events && hipEventRecord(static_cast<hipEvent_t>(events[2]), stream) != hipSuccess)
    return SV_ERR_LAUNCH;
  return SV_OK;
}

int dispatch(const void* target, const void* draft, int32_t dtype, int32_t B, int32_t V,
             int32_t max_k, int32_t n_draft_rows, const int32_t* offsets, const int32_t* tokens,
             const float* temperature, uint64_t seed, int32_t* accept_len, int32_t* out_tokens,
             float* p_at, float* q_at, void* workspace, size_t workspace_bytes, void* stream,
             bool all_greedy, void* const* events) {
  if (!target || !offsets || !accept_len || !out_tokens || !workspace) return SV_ERR_NULL;
  if (!all_greedy && (!temperature || (n_draft_rows > 0 && !draft))) return SV_ERR_NULL;
  if (n_draft_rows > 0 && !tokens) return SV_ERR_NULL;
  if (!shape_ok(B, V, max_k, n_draft_rows)) return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (workspace_bytes < spec_verify_workspace_bytes(B, V, max_k) || !aligned16(workspace))
    return SV_ERR_WORKSPACE;
  const bool bf16 = dtype == SV_BF16;
  const int64_t row_bytes = static_cast<int64_t>(V) * (bf16 ? 2 : 4);
  const bool vec = row_bytes % 16 == 0 && aligned16(target) && (!draft || aligned16(draft));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16) {
    return vec ? launch_all<true, true>(target, draft, B, V, max_k, n_draft_rows, offsets, tokens,
                                        temperature, seed, accept_len, out_tokens, p_at, q_at,
                                        workspace, s, all_greedy, events)
               : launch_all<true, false>(target, draft, B, V, max_k, n_draft_rows, offsets,
                                         tokens, temperature, seed, accept_len, out_tokens, p_at,
                                         q_at, workspace, s, all_greedy, events);
  }
  return vec ? launch_all<false, true>(target, draft, B, V, max_k, n_draft_rows, offsets, tokens,
                                       temperature, seed, accept_len, out_tokens, p_at, q_at,
                                       workspace, s, all_greedy, events)
             : launch_all<false, false>(target, draft, B, V, max_k, n_draft_rows, offsets, tokens,
                                        temperature, seed, accept_len, out_tokens, p_at, q_at,
                                        workspace, s, all_greedy, events);
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
                  workspace_bytes, stream, true, nullptr);
}

int spec_verify_sample(const void* target_logits, const void* draft_logits, int32_t dtype,
                       int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows,
                       const int32_t* draft_offsets, const int32_t* draft_tokens,
                       const float* temperature, uint64_t seed, int32_t* accept_len,
                       int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return dispatch(target_logits, draft_logits, dtype, B, V, max_k, n_draft_rows, draft_offsets,
                  draft_tokens, temperature, seed, accept_len, out_tokens, p_at_draft,
                  q_at_draft, workspace, workspace_bytes, stream, false, nullptr);
}

int spec_verify_sample_timed(const void* target_logits, const void* draft_logits, int32_t dtype,
                             int32_t B, int32_t V, int32_t max_k, int32_t n_draft_rows,
                             const int32_t* draft_offsets, const int32_t* draft_tokens,
                             const float* temperature, uint64_t seed, int32_t* accept_len,
                             int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events) {
  if (!events || !events[0] || !events[1] || !events[2]) return SV_ERR_NULL;
  return dispatch(target_logits, draft_logits, dtype, B, V, max_k, n_draft_rows, draft_offsets,
                  draft_tokens, temperature, seed, accept_len, out_tokens, p_at_draft,
                  q_at_draft, workspace, workspace_bytes, stream, false, events);
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
