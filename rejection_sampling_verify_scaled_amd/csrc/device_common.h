// device_common.h -- gfx950 device helpers shared by the library's kernels:
// launch-shape constants, bf16 unpacking, Philox4x32-10, the open-interval
// uniform map, exp2-domain softmax arithmetic, wave and workgroup
// reductions, device-coherent hand-off slots, and the row-chunk loads and
// reductions (softmax statistics, argmax) of one wave.
//
// Included only by the library's .hip sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>

namespace {

constexpr int kThreads = 256;  // 4 wave64s per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kItemVecs = 8;                      // 16-byte loads per lane per row-chunk
constexpr int kItemsInFlight = 2;                 // row-chunks a wave loads before reducing
constexpr int kGroupItems = kWaves * kItemsInFlight;  // flat grouping: row-chunks per workgroup
constexpr int kChunkBytes = 64 * kItemVecs * 16;  // one row-chunk: 8 KiB
// Polls before a wait gives up.  A library built with a small limit (0: one
// load, no re-poll) makes the waits expire on purpose, so that the expired
// paths can be exercised: every wait still ends and every kernel exits.
#ifndef SV_SPIN_LIMIT
#define SV_SPIN_LIMIT (1u << 16)
#endif
constexpr unsigned kSpinLimit = SV_SPIN_LIMIT;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int ceil_div_dev(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int elems_per_vec(bool bf16) { return bf16 ? 8 : 4; }
__host__ __device__ constexpr int chunk_tokens(bool bf16) { return kChunkBytes / (bf16 ? 2 : 4); }

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

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = static_cast<uint64_t>(kPhiloxM0) * c0;
    const uint64_t d = static_cast<uint64_t>(kPhiloxM1) * c2;
    const uint32_t n0 = static_cast<uint32_t>(d >> 32) ^ c1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(a >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(d);
    c3 = static_cast<uint32_t>(a);
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// a ^ b ^ k in one instruction (gfx950's three-input bit operation; 0x96 is
// the truth table of three-way exclusive or).  k is wave-uniform.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

// The same generator for race counters (c0, c1, c2, c3) with c1, c2, c3 and
// the key wave-uniform (c3 is the stream tag).  Rounds 1-3 still mix uniform
// words (the compiler keeps those on the scalar unit); from round 4 on every
// word varies per lane and each output word takes one three-input xor.
__device__ __forceinline__ Philox4 philox_race(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = static_cast<uint64_t>(kPhiloxM0) * c0;
    const uint64_t d = static_cast<uint64_t>(kPhiloxM1) * c2;
    uint32_t n0, n2;
    if (r < 3) {
      n0 = static_cast<uint32_t>(d >> 32) ^ c1 ^ k0;
      n2 = static_cast<uint32_t>(a >> 32) ^ c3 ^ k1;
    } else {
      n0 = xor3(static_cast<uint32_t>(d >> 32), c1, k0);
      n2 = xor3(static_cast<uint32_t>(a >> 32), c3, k1);
    }
    c1 = static_cast<uint32_t>(d);
    c3 = static_cast<uint32_t>(a);
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// (2 * (x >> 9) + 1) * 2^-24, exact in float32, strictly inside (0, 1): the
// float 1 + (x >> 9) 2^-23 (one funnel shift puts x >> 9 under the exponent
// bits of 1.0) minus (1 - 2^-24); both lie in [0.5, 2], so the difference is
// exact (Sterbenz).
__device__ __forceinline__ float uniform_open01(uint32_t x) {
  const uint32_t one_plus = __builtin_amdgcn_alignbit(0x7Fu, x, 9u);  // 0x3F800000 | x >> 9
  return __uint_as_float(one_plus) - 0x1.fffffep-1f;
}

// Weights are 2^((z - m) c) for a reference m (a row's or a chunk's maximum)
// and c = log2(e) / T.  The exponent is formed from the difference z - m,
// which is exact in float32 for bfloat16 logits (and for float32 logits
// within a factor two of m), so its rounding is relative to the exponent
// itself: the weights of the tokens that matter keep float32 precision at any
// temperature, where 2^(z c - fl(m c)) would carry an error of about
// |m| c 2^-24 in every exponent.

// Reference for a maximum m: m itself, or 0 when there is no finite maximum
// (the weights of -inf logits are then 0 and a NaN stays visible).
__device__ __forceinline__ float weight_ref(float m) { return (m == -INFINITY) ? 0.f : m; }

// log2 of the unnormalised weight 2^((z - m) c).
__device__ __forceinline__ float log2_weight(float z, float cf, float m) { return (z - m) * cf; }

// 2^((m - M) c): a partial with maximum m moved to the reference M; 0 for a
// partial with no finite maximum (0 * s keeps a NaN sum NaN).
__device__ __forceinline__ float rescale(float m, float cf, float M) {
  return (m == -INFINITY) ? 0.f : fast_exp2((m - M) * cf);
}

// (max, sum) pairs; a sum s is relative to its max: s = sum 2^((z - max) c).
__device__ __forceinline__ void merge_stats(float& m, float& s, float m2, float s2, float cf) {
  const float M = fmaxf(m, m2);
  s = s * rescale(m, cf, M) + s2 * rescale(m2, cf, M);
  m = M;
}

// Larger value wins; equal values keep the lower index.
__device__ __forceinline__ void merge_argmax(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Exact wave reductions (max, argmax, min) through DPP: within each 16-lane
// row, lane i combines with lanes i-1, i-2, i-4, i-8 (row_shr), so lane 15 of
// a row holds the row's result; row_bcast:15 then carries rows 0 and 2 into
// rows 1 and 3, and row_bcast:31 carries row 1 into rows 2 and 3, leaving the
// wave's result in lane 63, which readlane makes wave-uniform.  Each step is
// a VALU operation on the register file, not a round trip through the LDS
// permute path.  A lane whose DPP source does not exist keeps its own value
// (combining a value with itself changes nothing, and keeps an all-NaN
// maximum NaN).  Called with every lane of the wave active.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_int(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_float(float v) {
  return __int_as_float(dpp_int<CTRL, ROW_MASK>(__float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_float<kDppRowShr1>(x));
  x = fmaxf(x, dpp_float<kDppRowShr2>(x));
  x = fmaxf(x, dpp_float<kDppRowShr4>(x));
  x = fmaxf(x, dpp_float<kDppRowShr8>(x));
  x = fmaxf(x, dpp_float<kDppRowBcast15, 0xa>(x));
  x = fmaxf(x, dpp_float<kDppRowBcast31, 0xc>(x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ int wave_min_int(int x) {
  x = min(x, dpp_int<kDppRowShr1>(x));
  x = min(x, dpp_int<kDppRowShr2>(x));
  x = min(x, dpp_int<kDppRowShr4>(x));
  x = min(x, dpp_int<kDppRowShr8>(x));
  x = min(x, dpp_int<kDppRowBcast15, 0xa>(x));
  x = min(x, dpp_int<kDppRowBcast31, 0xc>(x));
  return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ int wave_max_int(int x) {
  x = max(x, dpp_int<kDppRowShr1>(x));
  x = max(x, dpp_int<kDppRowShr2>(x));
  x = max(x, dpp_int<kDppRowShr4>(x));
  x = max(x, dpp_int<kDppRowShr8>(x));
  x = max(x, dpp_int<kDppRowBcast15, 0xa>(x));
  x = max(x, dpp_int<kDppRowBcast31, 0xc>(x));
  return __builtin_amdgcn_readlane(x, 63);
}

// Float sums keep the butterfly (its rounding order is the one the results
// were validated with).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ void dpp_merge_argmax(float& v, int& i) {
  const float v2 = dpp_float<CTRL, ROW_MASK>(v);
  const int i2 = dpp_int<CTRL, ROW_MASK>(i);
  merge_argmax(v, i, v2, i2);
}

// (max, sum) pairs through the same DPP steps.  Merging a pair with itself
// would double its sum, so a lane without a DPP source takes the empty pair
// (-inf, 0) instead; the sums are added in the DPP tree's order.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ void dpp_merge_stats(float& m, float& s, float cf) {
  const float m2 = __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(-INFINITY), __float_as_int(m), CTRL, ROW_MASK, 0xf, false));
  const float s2 = __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(0.f), __float_as_int(s), CTRL, ROW_MASK, 0xf, false));
  merge_stats(m, s, m2, s2, cf);
}

// Every lane ends with the wave's merged (max, sum).
__device__ __forceinline__ void wave_merge_stats(float& m, float& s, float cf) {
  dpp_merge_stats<kDppRowShr1>(m, s, cf);
  dpp_merge_stats<kDppRowShr2>(m, s, cf);
  dpp_merge_stats<kDppRowShr4>(m, s, cf);
  dpp_merge_stats<kDppRowShr8>(m, s, cf);
  dpp_merge_stats<kDppRowBcast15, 0xa>(m, s, cf);
  dpp_merge_stats<kDppRowBcast31, 0xc>(m, s, cf);
  m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 63));
  s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 63));
}

// Every lane ends with the wave's (value, lowest index) winner.
__device__ __forceinline__ void wave_merge_argmax(float& v, int& i) {
  dpp_merge_argmax<kDppRowShr1>(v, i);
  dpp_merge_argmax<kDppRowShr2>(v, i);
  dpp_merge_argmax<kDppRowShr4>(v, i);
  dpp_merge_argmax<kDppRowShr8>(v, i);
  dpp_merge_argmax<kDppRowBcast15, 0xa>(v, i);
  dpp_merge_argmax<kDppRowBcast31, 0xc>(v, i);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
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

// This wave's index in the workgroup, known to the compiler as wave-uniform
// (so per-wave decisions become scalar branches, not exec-masked ones).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A value every lane holds equally, moved to a scalar register.
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform_float(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
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
__device__ inline uint64_t slot_wait(const uint64_t* p) {
  uint64_t v = slot_load(p);
  for (unsigned it = 0; v == 0u && it < kSpinLimit; ++it) {
    __builtin_amdgcn_s_sleep(2);
    v = slot_load(p);
  }
  return v;
}

// ------------------------------------------------------------------ statistics

// One wave's share of a row-chunk: lane elements e0 + (u * 64 + lane) * EPV +
// [0, EPV), u = 0..NV-1 (NV = kItemVecs for a full row-chunk; a shorter
// chunk keeps the same layout with fewer vectors).  The vector path loads every vector from an
// in-row address (indices clamped to the row's last vector) on one code path,
// so the loads of several row-chunks stay in flight together; mask_tail then
// replaces the vectors past the row end with -inf.  The scalar path reads -inf
// past V itself.
template <bool BF16, bool VEC, int NV = kItemVecs>
__device__ __forceinline__ void load_item(const void* base, int64_t row, int V, int64_t e0,
                                          uint4* out) {
  constexpr int EPV = elems_per_vec(BF16);
  const int lane = threadIdx.x & 63;
  if constexpr (VEC) {
    const uint4* rowv = reinterpret_cast<const uint4*>(static_cast<const char*>(base) +
                                                       row * V * (BF16 ? 2 : 4));
    const int last = V / EPV - 1;
    const int i0 = static_cast<int>(e0 / EPV) + lane;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      // non-temporal: every logit is read once per call, so these lines are
      // not worth keeping in the caches (measured: B=256 K=8 fp32 374 -> 358 us)
      typedef unsigned int v4u __attribute__((ext_vector_type(4)));
      const v4u v =
          __builtin_nontemporal_load(reinterpret_cast<const v4u*>(rowv + min(i0 + u * 64, last)));
      out[u] = make_uint4(v.x, v.y, v.z, v.w);
    }
  } else {
    const uint32_t ninf = BF16 ? 0xff80ff80u : 0xff800000u;
    const int64_t rb = row * V;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int64_t e = e0 + static_cast<int64_t>(u * 64 + lane) * EPV;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (BF16) {
          const uint16_t* b16 = static_cast<const uint16_t*>(base);
          const uint32_t lo = (e + 2 * k < V) ? b16[rb + e + 2 * k] : 0xff80u;
          const uint32_t hi = (e + 2 * k + 1 < V) ? b16[rb + e + 2 * k + 1] : 0xff80u;
          w[k] = lo | (hi << 16);
        } else {
          w[k] = (e + k < V) ? __float_as_uint(static_cast<const float*>(base)[rb + e + k])
                             : ninf;
        }
      }
      out[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Vector path, row-chunk reaching past the row end: vectors past it become -inf.
template <bool BF16, int NV = kItemVecs>
__device__ __forceinline__ void mask_tail(uint4* buf, int V, int64_t e0) {
  constexpr int EPV = elems_per_vec(BF16);
  const uint32_t ninf = BF16 ? 0xff80ff80u : 0xff800000u;
  const int last = V / EPV - 1;
  const int i0 = static_cast<int>(e0 / EPV) + (threadIdx.x & 63);
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if (i0 + u * 64 > last) buf[u] = make_uint4(ninf, ninf, ninf, ninf);
}

template <bool BF16>
__device__ __forceinline__ void unpack(const uint4& v, float* xs) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xs[2 * k] = bf16_lo(w[k]);
      xs[2 * k + 1] = bf16_hi(w[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) xs[k] = __uint_as_float(w[k]);
  }
}

// Partial of one row-chunk held by the wave: (max, sum of 2^((z - max) c)).
// One pass: each vector's sum is formed relative to the vector's own maximum,
// then rescaled to the wave maximum.
template <bool BF16>
__device__ __forceinline__ uint64_t item_stats(const uint4* buf, float cf) {
  constexpr int EPV = elems_per_vec(BF16);
  float vm[kItemVecs], vs[kItemVecs];
#pragma unroll
  for (int u = 0; u < kItemVecs; ++u) {
    float xs[EPV];
    unpack<BF16>(buf[u], xs);
    float m = xs[0];
#pragma unroll
    for (int k = 1; k < EPV; ++k) m = fmaxf(m, xs[k]);
    // offset 0 when there is no finite max keeps a NaN visible in the sum
    const float mr = weight_ref(m);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < EPV; k += 2) {
      s0 += fast_exp2(log2_weight(xs[k], cf, mr));
      s1 += fast_exp2(log2_weight(xs[k + 1], cf, mr));
    }
    vm[u] = m;
    vs[u] = s0 + s1;
  }
  float mx = vm[0];
#pragma unroll
  for (int u = 1; u < kItemVecs; ++u) mx = fmaxf(mx, vm[u]);
  mx = wave_max(mx);
  const float Mr = weight_ref(mx);
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kItemVecs; ++u) s += vs[u] * rescale(vm[u], cf, Mr);
  s = wave_sum(s);
  return pack_slot(mx, __float_as_uint(s));
}

// Partial of one row-chunk for a greedy row: (max, lowest index attaining it).
// The wave maximum from per-vector maxima; then each lane takes the first of
// its vectors holding it (a backward scan keeps the last match, the lowest)
// and the first element of that vector equal to it.  NaN never matches.
template <bool BF16, int NV = kItemVecs>
__device__ __forceinline__ uint64_t item_argmax(const uint4* buf, int64_t e0) {
  constexpr int EPV = elems_per_vec(BF16);
  const int lane = threadIdx.x & 63;
  float vm[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float xs[EPV];
    unpack<BF16>(buf[u], xs);
    vm[u] = xs[0];
#pragma unroll
    for (int k = 1; k < EPV; ++k) vm[u] = fmaxf(vm[u], xs[k]);
  }
  float mx = vm[0];
#pragma unroll
  for (int u = 1; u < NV; ++u) mx = fmaxf(mx, vm[u]);
  mx = wave_max(mx);
  int us = -1;
  uint4 sel = buf[0];
#pragma unroll
  for (int u = NV - 1; u >= 0; --u) {
    if (vm[u] == mx) {
      us = u;
      sel = buf[u];
    }
  }
  int idx = INT_MAX;
  if (us >= 0) {
    float xs[EPV];
    unpack<BF16>(sel, xs);
    int ks = 0;
#pragma unroll
    for (int k = EPV - 1; k >= 0; --k)
      if (xs[k] == mx) ks = k;
    idx = static_cast<int>(e0) + (us * 64 + lane) * EPV + ks;
  }
  idx = wave_min_int(idx);
  return pack_slot(mx, static_cast<uint32_t>(idx));
}

// ------------------------------------------------------------------ host helpers

// Compute units of the current device, looked up once per device (launch
// shapes are sized from it: a resident generation is a few workgroups per CU).
inline int64_t device_compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace
