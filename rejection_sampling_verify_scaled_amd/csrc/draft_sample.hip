// draft_sample.hip -- gfx950 kernel and C ABI of the draft-side sampler.
//
// What is computed is stated in include/spec_verify.h (spec_draft_sample):
// the drafting step that precedes verification draws one token per request
// from softmax(z / T) of its draft row ("Decodificación Especulativa y
// EAGLE", section "El Concepto", step 1, and the listing's draft loop), or
// takes the row's argmax when T = 0 (the top-token drafting of Perplexity's
// draft-target scheme).
//
// One launch.  Row b is cut into chunks of NV 16-byte vectors per lane: 8 KiB
// (NV = 8, the verify kernel's row-chunk), 4 KiB (NV = 4) when full chunks
// would give the batch fewer than about four waves per SIMD for this
// arithmetic-bound pass, and 2 KiB (NV = 2) when half chunks would give it
// fewer than one.  Workgroup g serves request b = g / ng and the 4
// chunks cg * 4 + wave (cg = g mod ng, one chunk per wave).  A wave of a sampled request makes one pass over its chunk for the
// maximum, then a second pass that, per token, forms the weight
// w = 2^((z - m) c) (c = log2(e) / T, m the chunk maximum), adds it to
// the chunk's softmax sum and runs the exponential race: the token with the
// largest w / e wins, e = -log2 U from Philox4x32-10 on stream tag 2,
// counter (v >> 2, step, b, 2), word v & 3.  Candidates are compared by
// cross-multiplication; the chunk's winner becomes the log2-domain key
// log2(w / e), relative to the chunk maximum; the finisher moves each key to
// the row maximum M by adding (m - M) c before comparing.  A greedy wave
// reduces its chunk to (max, lowest argmax).  Each chunk leaves one or two
// 8-byte slots in the workspace; the request's last workgroup in grid order
// folds them (larger key, then lower index; softmax sums rescaled to the
// row maximum), gathers z at the winner for q(x), writes the outputs and
// zeroes the slots.  Hand-offs use the same device-coherent zero-slot
// protocol as the verify kernel; waits are bounded, and an expired wait
// gives token -1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "spec_verify.h"
#include "device_common.h"

namespace {

constexpr uint32_t kDraftTag = 2u;  // Philox stream tag of the draft sampler
// Half chunks below this many full-chunk waves (1024 SIMDs x 4): 64 bf16 rows
// of V = 128256 go from 10.6 to 10.0 us, while 256 fp32 rows keep full chunks
// (half chunks there: 35.4 -> 40.4 us, twice the partials to fold).
constexpr int64_t kHalfChunksBelow = 4096;
// Quarter chunks below this many half-chunk waves (one per SIMD): one sampled
// bf16 row of V = 128256 7.1 -> 6.4 us, eight 7.6 -> 6.8 us; from 32 rows on
// quarter chunks gain nothing.
constexpr int64_t kQuarterChunksBelow = 1024;

__host__ __device__ constexpr int draft_chunk_tokens(bool bf16, int nv) {
  return 64 * nv * elems_per_vec(bf16);
}

struct DraftParams {
  const void* logits;        // [B][V]
  const float* temperature;  // [B]
  uint32_t k0, k1;           // Philox key
  int32_t B, V, step;
  int32_t nc;          // chunks per row
  int32_t ng;          // workgroups per row, ceil(nc / 4)
  uint64_t* part;      // [B][nc][2]: statistics slot, race slot
  int32_t* tokens;     // [B]
  float* q_at;         // [B] or NULL
};

__device__ __forceinline__ uint64_t* stat_slot(const DraftParams& p, int b, int c) {
  return p.part + (static_cast<int64_t>(b) * p.nc + c) * 2;
}
__device__ __forceinline__ uint64_t* race_slot(const DraftParams& p, int b, int c) {
  return stat_slot(p, b, c) + 1;
}

// Statistics and race of one sampled chunk held by a wave (lane elements as
// in load_item).  Returns the statistics slot (max, sum relative to max) and
// sets the race slot (log2-domain key relative to the chunk maximum, index).
template <bool BF16, int NV>
__device__ __forceinline__ uint64_t chunk_race(const uint4* buf, int64_t e0, float cf, uint32_t b,
                                               uint32_t step, uint32_t k0, uint32_t k1,
                                               uint64_t& race) {
  constexpr int EPV = elems_per_vec(BF16);
  const int lane = threadIdx.x & 63;
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float xs[EPV];
    unpack<BF16>(buf[u], xs);
#pragma unroll
    for (int k = 0; k < EPV; ++k) mx = fmaxf(mx, xs[k]);
  }
  mx = wave_max(mx);
  // offset 0 when there is no finite max keeps a NaN visible in the sum
  const float mc = weight_ref(mx);
  float s = 0.f, bw = 0.f, be = 1.f;
  int bi = INT_MAX;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float xs[EPV];
    unpack<BF16>(buf[u], xs);
    const int64_t v0 = e0 + static_cast<int64_t>(u * 64 + lane) * EPV;
#pragma unroll
    for (int h = 0; h < EPV / 4; ++h) {
      const Philox4 r = philox_race(static_cast<uint32_t>((v0 >> 2) + h), step, b, kDraftTag, k0, k1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = fast_exp2(log2_weight(xs[4 * h + k], cf, mc));
        s += w;
        const float e = -fast_log2(uniform_open01(r.w[k]));  // E / ln 2
        if (w * be > bw * e) {
          bw = w;
          be = e;
          bi = static_cast<int>(v0) + 4 * h + k;
        }
      }
    }
  }
  s = wave_sum(s);
  float key = bi == INT_MAX ? -INFINITY : fast_log2(bw / be);
  wave_merge_argmax(key, bi);
  race = pack_slot(key, static_cast<uint32_t>(bi));
  return pack_slot(mx, __float_as_uint(s));
}

// Poll the slots a thread folds until all are written; false if a wait expired.
__device__ __forceinline__ bool wait_slots(uint64_t* const* slot, uint64_t* v, int n) {
  uint32_t missing = 0u;
  for (int i = 0; i < n; ++i) {
    v[i] = slot_load(slot[i]);
    if (v[i] == 0u) missing |= 1u << i;
  }
  for (unsigned it = 0; missing != 0u && it < kSpinLimit; ++it) {
    __builtin_amdgcn_s_sleep(1);
    for (int i = 0; i < n; ++i) {
      if (missing & (1u << i)) {
        v[i] = slot_load(slot[i]);
        if (v[i] != 0u) missing &= ~(1u << i);
      }
    }
  }
  return missing == 0u;
}

// The request's last workgroup: fold every chunk's slots, write the outputs,
// zero the slots.  Thread t folds chunks t, t + 256, ... in order; threads
// merge in a fixed tree (wave shuffles, then the waves in order).
template <bool BF16>
__device__ void draft_finish(const DraftParams& p, int b, float T) {
  __shared__ float sh_m[kWaves], sh_s[kWaves], sh_k[kWaves];
  __shared__ int sh_i[kWaves], sh_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const bool greedy = T == 0.f;
  const float cf = greedy ? 0.f : kLog2e / T;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  float M = -INFINITY, S = 0.f, key = -INFINITY;
  int idx = INT_MAX;
  bool expired = false;
  // pass 1: the statistics (and a greedy row's argmax).  A sampled row's race
  // keys are relative to their chunk maximum, so they are merged in pass 2,
  // once the row maximum is known; the thread's first chunk keeps its slots
  // in registers, later chunks (V above 256 chunks) are read again.
  uint64_t first_s = 0u, first_r = 0u;
  for (int c = tid; c < p.nc; c += kThreads) {
    uint64_t* slots[2] = {stat_slot(p, b, c), race_slot(p, b, c)};
    uint64_t v[2];
    if (!wait_slots(slots, v, greedy ? 1 : 2)) {
      expired = true;
      continue;
    }
    if (greedy) {
      merge_argmax(M, idx, slot_f(v[0]), static_cast<int>(slot_w(v[0])));
      slot_store(slots[0], 0u);
    } else {
      merge_stats(M, S, slot_f(v[0]), __uint_as_float(slot_w(v[0])), cf);
      if (c == tid) {
        first_s = v[0];
        first_r = v[1];
        slot_store(slots[0], 0u);
        slot_store(slots[1], 0u);
      }
    }
  }
  if (expired) atomicOr(&sh_bad, 1);
  // fixed-order DPP tree over each wave, then the waves in order
  if (greedy)
    wave_merge_argmax(M, idx);
  else
    wave_merge_stats(M, S, cf);
  if (lane == 0) {
    sh_m[wave] = M;
    sh_s[wave] = S;
    sh_i[wave] = idx;
  }
  __syncthreads();
  M = sh_m[0];
  S = sh_s[0];
  idx = sh_i[0];
  for (int w = 1; w < kWaves; ++w) {
    if (greedy)
      merge_argmax(M, idx, sh_m[w], sh_i[w]);
    else
      merge_stats(M, S, sh_m[w], sh_s[w], cf);
  }
  if (!greedy) {
    // pass 2: each chunk's key log2(w / e) + (m - M) c, relative to the row maximum
    idx = INT_MAX;
    for (int c = tid; c < p.nc; c += kThreads) {
      uint64_t vs = first_s, vr = first_r;
      if (c != tid) {
        vs = slot_load(stat_slot(p, b, c));
        vr = slot_load(race_slot(p, b, c));
        if (vs != 0u) {
          slot_store(stat_slot(p, b, c), 0u);
          slot_store(race_slot(p, b, c), 0u);
        }
      }
      if (vs == 0u || vr == 0u) continue;  // an expired wait (already reported)
      const float kc = slot_f(vr) + (slot_f(vs) - M) * cf;
      merge_argmax(key, idx, kc, static_cast<int>(slot_w(vr)));
    }
    block_argmax(key, idx, sh_k, sh_i);
  }
  if (tid != 0) return;
  const bool finite_max = M > -INFINITY && M < INFINITY;
  const bool ok = !sh_bad && finite_max && idx != INT_MAX && (greedy || S < INFINITY);
  p.tokens[b] = ok ? idx : -1;
  if (p.q_at) {
    float q = NAN;
    if (ok && !greedy) {
      const float zx = load_logit<BF16>(p.logits, static_cast<int64_t>(b) * p.V + idx);
      q = fast_exp2(log2_weight(zx, cf, M) - fast_log2(S));
    }
    p.q_at[b] = q;
  }
}

template <bool BF16, bool VEC, int NV>
__global__ __launch_bounds__(kThreads) void sd_sample(DraftParams p) {
  constexpr int CHUNK = draft_chunk_tokens(BF16, NV);
  const int g = blockIdx.x;
  const int b = g / p.ng;
  const int cg = g - b * p.ng;
  // the chunk's loads go out before the temperature arrives (one memory round
  // trip fewer per workgroup: one bf16 row 6.1 -> 6.0 us, eight 6.8 -> 6.5 us)
  const int c = cg * kWaves + wave_id();
  const int64_t e0 = static_cast<int64_t>(c) * CHUNK;
  uint4 buf[NV];
  if (c < p.nc) load_item<BF16, VEC, NV>(p.logits, b, p.V, e0, buf);
  const float T = p.temperature[b];
  // NaN, negative and infinite temperatures fail the request
  if (!(T >= 0.f && T < INFINITY)) {
    if (cg == p.ng - 1 && threadIdx.x == 0) {
      p.tokens[b] = -1;
      if (p.q_at) p.q_at[b] = NAN;
    }
    return;
  }
  if (c < p.nc) {
    if (VEC && e0 + CHUNK > p.V) mask_tail<BF16, NV>(buf, p.V, e0);
    const int lane = threadIdx.x & 63;
    if (T == 0.f) {
      const uint64_t v = item_argmax<BF16, NV>(buf, e0);
      if (lane == 0) slot_store(stat_slot(p, b, c), v);
    } else {
      uint64_t race;
      const uint64_t v = chunk_race<BF16, NV>(buf, e0, kLog2e / T, static_cast<uint32_t>(b),
                                          static_cast<uint32_t>(p.step), p.k0, p.k1, race);
      if (lane == 0) {
        slot_store(stat_slot(p, b, c), v);
        slot_store(race_slot(p, b, c), race);
      }
    }
  }
  if (cg == p.ng - 1) draft_finish<BF16>(p, b, T);
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Sized with the smallest chunk (float32, quarter length), so any launch fits.
size_t draft_workspace(int32_t B, int32_t V) {
  const int64_t nc = ceil_div64(V, draft_chunk_tokens(false, kItemVecs / 4));
  return static_cast<size_t>(B) * static_cast<size_t>(nc) * 2 * sizeof(uint64_t);
}

template <bool BF16, bool VEC, int NV>
int draft_launch(const DraftParams& prm, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((sd_sample<BF16, VEC, NV>), dim3(static_cast<uint32_t>(grid)),
                     dim3(kThreads), 0, stream, prm);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

template <bool BF16, bool VEC>
int draft_launch_nv(const DraftParams& prm, int64_t grid, int nv, hipStream_t stream) {
  if (nv == kItemVecs / 4) return draft_launch<BF16, VEC, kItemVecs / 4>(prm, grid, stream);
  if (nv == kItemVecs / 2) return draft_launch<BF16, VEC, kItemVecs / 2>(prm, grid, stream);
  return draft_launch<BF16, VEC, kItemVecs>(prm, grid, stream);
}

}  // namespace

extern "C" {

size_t spec_draft_workspace_bytes(int32_t B, int32_t V) {
  if (B < 1 || V < 1) return 0;
  return draft_workspace(B, V);
}

int spec_draft_sample(const void* draft_logits, int32_t dtype, int32_t B, int32_t V,
                      const float* temperature, uint64_t seed, int32_t step, int32_t* tokens,
                      float* q_at, void* workspace, size_t workspace_bytes, void* stream) {
  if (!draft_logits || !temperature || !tokens || !workspace) return SV_ERR_NULL;
  if (B < 1 || V < 1 || step < 0) return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (workspace_bytes < draft_workspace(B, V) ||
      (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return SV_ERR_WORKSPACE;
  const bool bf16 = dtype == SV_BF16;
  DraftParams prm;
  prm.logits = draft_logits;
  prm.temperature = temperature;
  prm.k0 = static_cast<uint32_t>(seed);
  prm.k1 = static_cast<uint32_t>(seed >> 32);
  prm.B = B;
  prm.V = V;
  prm.step = step;
  int nv = kItemVecs;
  if (static_cast<int64_t>(B) * ceil_div64(V, draft_chunk_tokens(bf16, nv)) < kHalfChunksBelow)
    nv = kItemVecs / 2;
  if (nv == kItemVecs / 2 &&
      static_cast<int64_t>(B) * ceil_div64(V, draft_chunk_tokens(bf16, nv)) < kQuarterChunksBelow)
    nv = kItemVecs / 4;
  prm.nc = static_cast<int32_t>(ceil_div64(V, draft_chunk_tokens(bf16, nv)));
  prm.ng = static_cast<int32_t>(ceil_div64(prm.nc, kWaves));
  prm.part = static_cast<uint64_t*>(workspace);
  prm.tokens = tokens;
  prm.q_at = q_at;
  const int64_t grid = static_cast<int64_t>(B) * prm.ng;
  if (grid > INT32_MAX) return SV_ERR_SHAPE;
  const int64_t row_bytes = static_cast<int64_t>(V) * (bf16 ? 2 : 4);
  const bool vec = row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(draft_logits) & 15u) == 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? draft_launch_nv<true, true>(prm, grid, nv, s)
               : draft_launch_nv<true, false>(prm, grid, nv, s);
  return vec ? draft_launch_nv<false, true>(prm, grid, nv, s)
             : draft_launch_nv<false, false>(prm, grid, nv, s);
}

}  // extern "C"
