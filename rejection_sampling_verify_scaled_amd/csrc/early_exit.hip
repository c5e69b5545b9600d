// early_exit.hip -- gfx950 kernel and C ABI of the early-exit verify step.
//
// Same decision as spec_verify_sample (include/spec_verify.h; "Decodificación
// Especulativa y EAGLE", section "La Regla de Exactitud"): the ratio tests run
// left to right and stop at the first rejection, so rows past it never
// influence the result.  This variant does not read them.  It trades
// parallelism inside a request for bytes: a request's rows are streamed one
// position (stage) at a time, and later stages are skipped once a stage
// rejects (sampled) or mismatches (greedy).
//
// One launch, stage-major.  The grid is max_k + 1 regions of ngs statistics
// workgroups per request, one region per stage s, and ngr race workgroups
// per request, in one of two layouts (below):
//   statistics (b, s), s < K_b: unless stage s - 1 is already decided and
//     stopped, stream target row s and, for a sampled request, draft row s
//     (8 row-chunks per workgroup, two in flight per wave), one 8-byte
//     partial per row-chunk.  A stage does not wait for the previous
//     stage's decision to stream: when that decision is still pending (small
//     batches, where the regions overlap in time) it streams on speculation.
//     A greedy request also streams target row K_b at s = K_b (its stop
//     token's row).  The stage's last workgroup with items then waits for
//     the decision of stage s - 1; after an acceptance it folds the partials
//     and decides: sampled -- p_s(x_s), q_s(x_s), r_s, accept iff
//     r_s q_s < p_s; greedy -- accept iff argmax equals x_s, else (or at
//     s = K_b) write the outputs.  After a stop it leaves the stage's
//     partials unread.  The decision goes to a record for (b, s), and a stop
//     is copied into the records of the later stages so their workgroups
//     exit without streaming.
//   race (b, s), sampled requests: after a rejection at s - 1, the residual
//     race over row s - 1 with the normalisers the decision carried; at
//     s = K_b after acceptances only, the bonus race over target row K_b
//     (keys in the log2 domain relative to each chunk's maximum, so it needs
//     no statistics of that row).  The last race workgroup folds the chunk
//     winners and writes the outputs.
// Layouts.  Races at the end (the default): the race workgroups of every
// request follow all statistics regions, and each finds its request's stop in
// the record of the request's last draft position (a stop is copied there).
// Races per region: region s also holds ngr race workgroups per request that
// race a rejection at s - 1 (or the bonus at s = K_b).  Most of these find
// nothing to do, and while a decision is pending they hold slots the stream
// needs; but when the batch's races are many and mostly bonus races (K = 1,
// more race workgroups than one resident generation), interleaving them with
// the last stage's statistics keeps their arithmetic beside streaming instead
// of in a tail of its own.  A region's workgroups find the previous stage's
// decisions ready when the regions are large (many requests); with small
// batches only the deciding workgroups and the races wait on them.
//
// Hand-offs use the zero-slot protocol of the verify kernel: a slot is
// written once per call and is all-zero until then.  Partials and race
// winners have one reader each, which zeroes them.  The decision records
// are read by many workgroups, so none of them can tell when the record is
// free, and the partials of a stage streamed on speculation past a stop
// have no reader; a small second kernel on the same stream zeroes the
// records and any partial still set after the verify kernel, so the
// workspace is all-zero again after every call.  A
// record's upper word is 1 (a payload of 0, such as a zero maximum, still
// reads as written).  All waits are bounded; an expired wait reports
// accept_len = -1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "spec_verify.h"
#include "device_common.h"

namespace {

// Chunks per race workgroup: 8, or 4 when a stage's race workgroups at 8
// would fill less than about half of a resident generation (fewer than
// kNarrowRaceBelow workgroups): a small batch then gets more race
// parallelism on its dependent chain (B=64 K=4 bf16: 57.3 -> 49.1 us), while
// large batches keep the wider races (B=256 K=8 fp32 at 4 chunks: 236 ->
// 293 us).  bf16 rows with max_k > 1 always race 4 chunks (16K tokens, as 8
// fp32 chunks): with the races after all statistics, ragged K <= 8 batches
// of B=128 run 79.5 -> 67.6 us and of B=1024 359 -> 355 us.
constexpr int kRaceChunks = 8;
constexpr int kRaceChunksNarrow = 4;
constexpr int64_t kNarrowRaceBelow = 512;
// XCDs of an MI355X; the dispatcher deals workgroups to them round robin.
constexpr int kEeXcds = 8;
constexpr int kStageRows = 2;      // a stage streams target row s and draft row s
constexpr int kDecSlots = 5;       // decision record: code, m_p, log2 S_p, m_q, log2 S_q
constexpr uint32_t kCont = 1u, kRej = 2u, kDone = 3u;  // decision codes (low byte)
// race slot index word of a bonus race that found its row non-finite (a NaN,
// a +inf maximum): the request fails, as the verify step fails a row whose
// softmax is not finite
constexpr uint32_t kBadRowIdx = 0xFFFFFFFEu;

struct EeParams {
  const void* target;
  const void* draft;
  const int32_t* offsets;
  const int32_t* tokens;
  const float* temperature;
  uint32_t k0, k1;
  int32_t B, V, max_k, n_draft_rows;
  int32_t nc;   // chunks per row
  int32_t ngs;  // statistics workgroups per (request, stage): ceil(2 nc / 8)
  int32_t rcw;  // race chunks per race workgroup (kRaceChunks, kRaceChunksNarrow or fewer)
  int32_t ngr;  // race workgroups per (request, region): ceil(nc / rcw)
  uint64_t* part;  // [B][max_k + 1][2][nc] stage partials
  uint64_t* race;  // [B][ngr] race winners
  uint64_t* dec;   // [B][max_k + 1][kDecSlots] decision records
  int32_t endrace; // 1: the race workgroups follow all statistics regions
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_at;
  float* q_at;
};

struct EeReq {
  int32_t off0, K;
  float T;
  bool valid, greedy;
};

// Request b's scalars, checked as the verify step checks them (slice inside
// the packed layout, K_b <= max_k, a finite non-negative temperature), then
// its draft tokens (inside the vocabulary); uniform, so the loads are scalar.
// A request whose drafts end before `stage` is not valid for that stage, and
// its tokens are not loaded (its workgroups of that region only exit).
__device__ EeReq ee_req_scalars(const EeParams& p, int b, int stage) {
  EeReq r;
  r.off0 = p.offsets[b];
  const int32_t off1 = p.offsets[b + 1];
  r.K = static_cast<int32_t>(static_cast<uint32_t>(off1) - static_cast<uint32_t>(r.off0));
  r.T = p.temperature[b];
  r.greedy = r.T == 0.f;
  const bool slice_ok =
      r.off0 >= 0 && off1 <= p.n_draft_rows && off1 >= r.off0 && r.K <= p.max_k;
  r.valid = slice_ok && r.T >= 0.f && r.T < INFINITY && stage <= r.K;
  return r;
}
__device__ void ee_req_tokens(const EeParams& p, EeReq& r) {
  bool ok = r.valid;
  if (ok) {
    for (int t = 0; t < r.K; ++t) {
      const int32_t x = p.tokens[r.off0 + t];
      ok = ok && x >= 0 && x < p.V;
    }
  }
  r.valid = ok;
}

__device__ __forceinline__ uint64_t* ee_part(const EeParams& p, int b, int s, int row, int c) {
  return p.part + ((static_cast<int64_t>(b) * (p.max_k + 1) + s) * kStageRows + row) * p.nc + c;
}
__device__ __forceinline__ uint64_t* ee_dec(const EeParams& p, int b, int s, int k) {
  return p.dec + (static_cast<int64_t>(b) * (p.max_k + 1) + s) * kDecSlots + k;
}
constexpr uint64_t kDecWritten = 1ull << 32;  // upper word of a written record
__device__ __forceinline__ void dec_store(const EeParams& p, int b, int s, int k, uint32_t v) {
  slot_store(ee_dec(p, b, s, k), kDecWritten | v);
}
// Payload of a record once written; false if the wait expired.
__device__ bool dec_wait(const EeParams& p, int b, int s, int k, uint32_t& v) {
  const uint64_t x = slot_wait(ee_dec(p, b, s, k));
  v = static_cast<uint32_t>(x);
  return x != 0u;
}

// A stop at stage s: the records of stages s..K-1 say so, so that the
// statistics workgroups of those stages exit without waiting.
__device__ void publish_stop(const EeParams& p, int b, int s, int K, uint32_t code) {
  for (int t = s + static_cast<int>(threadIdx.x); t < K; t += kThreads) dec_store(p, b, t, 0, code);
}

__device__ void ee_fault(const EeParams& p, int b, const EeReq& r, bool slice_ok) {
  const int tid = threadIdx.x;
  if (slice_ok) {
    const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
    if (tid <= r.K) p.out_tokens[trow0 + tid] = -1;
    if (tid < r.K) {
      if (p.p_at) p.p_at[r.off0 + tid] = NAN;
      if (p.q_at) p.q_at[r.off0 + tid] = NAN;
    }
  }
  if (tid == 0) p.accept_len[b] = -1;
}

// Outputs of a decided request: accept_len = n, tokens x_0..x_{n-1}, y, -1 padding;
// p/q past position n (never evaluated) are NaN, greedy requests have none.
__device__ void ee_outputs(const EeParams& p, int b, const EeReq& r, int n, int32_t y) {
  const int tid = threadIdx.x;
  const int64_t trow0 = static_cast<int64_t>(r.off0) + b;
  if (tid <= r.K) {
    const int32_t xt = tid < n ? p.tokens[r.off0 + tid] : 0;
    p.out_tokens[trow0 + tid] = tid < n ? xt : (tid == n ? y : -1);
  }
  if (tid < r.K && (r.greedy || tid > n)) {
    if (p.p_at) p.p_at[r.off0 + tid] = NAN;
    if (p.q_at) p.q_at[r.off0 + tid] = NAN;
  }
  if (tid == 0) p.accept_len[b] = n;
}

// ------------------------------------------------------------------ statistics of a stage

template <bool BF16, bool VEC, bool GREEDY>
__device__ void ee_stats(const EeParams& p, int b, int s, int j, const EeReq& r) {
  constexpr int CHUNK = chunk_tokens(BF16);
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int nrows = GREEDY ? 1 : kStageRows;
  const int i_lo = j * kGroupItems;
  const int i_hi = min(i_lo + kGroupItems, nrows * p.nc);
  const float cf = GREEDY ? 0.f : kLog2e / r.T;
  constexpr int IN_FLIGHT = VEC ? kItemsInFlight : 1;
  for (int i0 = i_lo + wave * IN_FLIGHT; i0 < i_hi; i0 += kWaves * IN_FLIGHT) {
    uint4 buf[IN_FLIGHT][kItemVecs];
#pragma unroll
    for (int k = 0; k < IN_FLIGHT; ++k) {
      const int i = min(i0 + k, i_hi - 1);
      const int row = i / p.nc;
      const int c = i - row * p.nc;
      const int64_t prow = row == 0 ? static_cast<int64_t>(r.off0) + b + s
                                    : static_cast<int64_t>(r.off0) + s;
      load_item<BF16, VEC>(row == 0 ? p.target : p.draft, prow, p.V,
                           static_cast<int64_t>(c) * CHUNK, buf[k]);
    }
#pragma unroll
    for (int k = 0; k < IN_FLIGHT; ++k) {
      const int i = i0 + k;
      if (i < i_hi) {
        const int row = i / p.nc;
        const int c = i - row * p.nc;
        if (VEC && static_cast<int64_t>(c + 1) * CHUNK > p.V)
          mask_tail<BF16>(buf[k], p.V, static_cast<int64_t>(c) * CHUNK);
        const uint64_t v = GREEDY ? item_argmax<BF16>(buf[k], static_cast<int64_t>(c) * CHUNK)
                                  : item_stats<BF16>(buf[k], cf);
        if (lane == 0) slot_store(ee_part(p, b, s, row, c), v);
      }
    }
  }
}

// The stage's last workgroup: fold the stage's partials (wave w < nrows folds
// row w: lane l takes chunks l, l + 64, ... in order, then a fixed DPP tree),
// then decide.
template <bool BF16>
__device__ void ee_decide(const EeParams& p, int b, int s, const EeReq& r) {
  __shared__ float sh_m[kStageRows], sh_s[kStageRows];
  __shared__ int sh_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int nrows = r.greedy ? 1 : kStageRows;
  const float cf = r.greedy ? 0.f : kLog2e / r.T;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  if (wave < nrows) {
    float M = -INFINITY, S = 0.f;
    int I = INT_MAX;
    bool expired = false;
    for (int c = lane; c < p.nc; c += 64) {
      uint64_t* slot = ee_part(p, b, s, wave, c);
      const uint64_t v = slot_wait(slot);
      if (v == 0u) {
        expired = true;
        continue;
      }
      slot_store(slot, 0u);
      if (r.greedy)
        merge_argmax(M, I, slot_f(v), static_cast<int>(slot_w(v)));
      else
        merge_stats(M, S, slot_f(v), __uint_as_float(slot_w(v)), cf);
    }
    if (r.greedy)
      wave_merge_argmax(M, I);
    else
      wave_merge_stats(M, S, cf);
    if (expired) atomicOr(&sh_bad, 2);
    if (lane == 0) {
      const bool finite = M > -INFINITY && M < INFINITY && (r.greedy || S < INFINITY);
      if (!finite) atomicOr(&sh_bad, 1);
      sh_m[wave] = M;
      sh_s[wave] = r.greedy ? __int_as_float(I) : S;
    }
  }
  __syncthreads();
  const int bad = sh_bad;
  if (bad) {
    // a stage that cannot be evaluated fails the request (an expired wait
    // reports -1 like a failure); later stages are told to stop
    publish_stop(p, b, s, r.K, kDone);
    ee_fault(p, b, r, true);
    return;
  }
  if (r.greedy) {
    const int32_t g = __float_as_int(sh_s[0]);
    const int32_t x = s < r.K ? p.tokens[r.off0 + s] : -1;
    if (s < r.K && g == x) {
      if (tid == 0) dec_store(p, b, s, 0, kCont);
    } else {
      publish_stop(p, b, s, r.K, kDone);
      ee_outputs(p, b, r, s, g);
    }
    return;
  }
  // sampled: ratio test at position s
  __shared__ int sh_rej;
  if (tid == 0) {
    const float mp = sh_m[0], lsp = fast_log2(sh_s[0]);
    const float mq = sh_m[1], lsq = fast_log2(sh_s[1]);
    const int32_t x = p.tokens[r.off0 + s];
    const float zp = load_logit<BF16>(p.target, (static_cast<int64_t>(r.off0) + b + s) * p.V + x);
    const float zq = load_logit<BF16>(p.draft, (static_cast<int64_t>(r.off0) + s) * p.V + x);
    const float pp = fast_exp2(log2_weight(zp, cf, mp) - lsp);
    const float qq = fast_exp2(log2_weight(zq, cf, mq) - lsq);
    const float u = uniform_open01(philox4x32_10(0u, s, b, 1u, p.k0, p.k1).w[0]);
    if (p.p_at) p.p_at[r.off0 + s] = pp;
    if (p.q_at) p.q_at[r.off0 + s] = qq;
    sh_rej = !(u * qq < pp);
    if (!sh_rej) {
      dec_store(p, b, s, 0, kCont);
    } else {
      dec_store(p, b, s, 1, __float_as_uint(mp));
      dec_store(p, b, s, 2, __float_as_uint(lsp));
      dec_store(p, b, s, 3, __float_as_uint(mq));
      dec_store(p, b, s, 4, __float_as_uint(lsq));
      dec_store(p, b, s, 0, kRej | (static_cast<uint32_t>(s) << 8));
    }
  }
  __syncthreads();
  // a rejection also stops the later stages (their races see a stop at s,
  // not at the stage before them, and do nothing)
  if (sh_rej) publish_stop(p, b, s + 1, r.K, kRej | (static_cast<uint32_t>(s) << 8));
}

// ------------------------------------------------------------------ races

struct EeRace {
  float cf, mp, lsp, mq, lsq;
  int n;
  bool residual;
};

// One chunk of the race held in registers (target chunk bp, draft chunk bq
// for the residual), folded into (key, idx): keys are log2(w / e) plus the
// weight reference, comparable across lanes and chunks.  The residual race's
// weights use the row statistics its decision carried.  The bonus race's row
// has no statistics pass: each lane keeps a running reference, the largest
// logit it has seen, and moves its best weight to a new reference when that
// grows (recomputed from the best logit, so the exponent stays an exact
// difference); the chunk is read once.  Its chunks are checked here as well:
// bad is set when the chunk holds a NaN or a +inf (the residual race's rows
// were checked by their stage's statistics).
template <bool BF16, bool RESIDUAL, int NV>
__device__ __forceinline__ void ee_race_chunk(const uint4* bp, const uint4* bq, int64_t e0,
                                              const EeRace& rr, uint32_t b, uint32_t k0,
                                              uint32_t k1, float& key, int& idx, bool& bad) {
  constexpr int EPV = elems_per_vec(BF16);
  const int lane = threadIdx.x & 63;
  float ref = 0.f, run = -INFINITY;  // bonus: weight reference, running maximum
  bool nan = false;
  float bw = 0.f, be = 1.f, bz = -INFINITY;
  int bi = INT_MAX;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float zp[EPV], zq[EPV];
    unpack<BF16>(bp[u], zp);
    if constexpr (RESIDUAL) {
      unpack<BF16>(bq[u], zq);
    } else {
      // (a NaN-propagating maximum: NaN if the vector holds one)
      float vm = zp[0];
#pragma unroll
      for (int k = 1; k < EPV; ++k) vm = __builtin_elementwise_maximum(vm, zp[k]);
      nan = nan || vm != vm;
      if (vm > run) {
        run = vm;
        ref = weight_ref(vm);
        bw = fast_exp2(log2_weight(bz, rr.cf, ref));  // 0 while there is no best
      }
    }
    const int64_t v0 = e0 + static_cast<int64_t>(u * 64 + lane) * EPV;
#pragma unroll
    for (int h = 0; h < EPV / 4; ++h) {
      const Philox4 ph = philox_race(static_cast<uint32_t>((v0 >> 2) + h),
                                     static_cast<uint32_t>(rr.n), b, 0u, k0, k1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float w;
        if constexpr (RESIDUAL) {
          w = fast_exp2(log2_weight(zp[4 * h + k], rr.cf, rr.mp) - rr.lsp) -
              fast_exp2(log2_weight(zq[4 * h + k], rr.cf, rr.mq) - rr.lsq);
        } else {
          w = fast_exp2(log2_weight(zp[4 * h + k], rr.cf, ref));
        }
        const float e = -fast_log2(uniform_open01(ph.w[k]));  // E / ln 2
        if (w * be > bw * e) {
          bw = w;
          be = e;
          bi = static_cast<int>(v0) + 4 * h + k;
          if constexpr (!RESIDUAL) bz = zp[4 * h + k];
        }
      }
    }
  }
  if constexpr (!RESIDUAL) bad = bad || __ballot(nan || run == INFINITY) != 0;
  // (log2 keys over an absolute offset: lanes and chunks share no reference)
  float kk = bi == INT_MAX ? -INFINITY : fast_log2(bw / be) + ref * rr.cf;
  wave_merge_argmax(kk, bi);
  merge_argmax(key, idx, kk, bi);
}

template <bool BF16, bool VEC>
__device__ void ee_race_range(const EeParams& p, int b, const EeReq& r, const EeRace& rr,
                              int c_lo, int c_hi, float& key, int& idx, bool& bad) {
  constexpr int CHUNK = chunk_tokens(BF16);
  const int wave = wave_id();
  const int64_t prow = static_cast<int64_t>(r.off0) + b + rr.n;
  const int64_t qrow = static_cast<int64_t>(r.off0) + rr.n;
  if constexpr (VEC && BF16) {
    for (int c = c_lo + wave; c < c_hi; c += kWaves) {
      uint4 bp[kItemVecs], bq[kItemVecs];
      const int64_t e0 = static_cast<int64_t>(c) * CHUNK;
      load_item<BF16, true>(p.target, prow, p.V, e0, bp);
      if (rr.residual) load_item<BF16, true>(p.draft, qrow, p.V, e0, bq);
      if (e0 + CHUNK > p.V) {
        mask_tail<BF16>(bp, p.V, e0);
        if (rr.residual) mask_tail<BF16>(bq, p.V, e0);
      }
      if (rr.residual)
        ee_race_chunk<BF16, true, kItemVecs>(bp, bq, e0, rr, static_cast<uint32_t>(b), p.k0, p.k1,
                                             key, idx, bad);
      else
        ee_race_chunk<BF16, false, kItemVecs>(bp, bp, e0, rr, static_cast<uint32_t>(b), p.k0,
                                              p.k1, key, idx, bad);
    }
  } else {
    // float32 rows and the scalar-load path take half a chunk at a time: a
    // float32 residual race then fits five waves per SIMD (B=256 K=8: 237 ->
    // 223 us), and the scalar path's element loads need many more registers
    // in flight than vector loads
    constexpr int NV = kItemVecs / 2, HALF = CHUNK / 2;
    for (int c = c_lo + wave; c < c_hi; c += kWaves) {
      for (int h = 0; h < 2; ++h) {
        const int64_t e0 = static_cast<int64_t>(c) * CHUNK + h * HALF;
        if (e0 >= p.V) break;
        uint4 bp[NV], bq[NV];
        load_item<BF16, VEC, NV>(p.target, prow, p.V, e0, bp);
        if (rr.residual) load_item<BF16, VEC, NV>(p.draft, qrow, p.V, e0, bq);
        if (VEC && e0 + HALF > p.V) {
          mask_tail<BF16, NV>(bp, p.V, e0);
          if (rr.residual) mask_tail<BF16, NV>(bq, p.V, e0);
        }
        if (rr.residual)
          ee_race_chunk<BF16, true, NV>(bp, bq, e0, rr, static_cast<uint32_t>(b), p.k0, p.k1, key,
                                        idx, bad);
        else
          ee_race_chunk<BF16, false, NV>(bp, bp, e0, rr, static_cast<uint32_t>(b), p.k0, p.k1,
                                         key, idx, bad);
      }
    }
  }
}

template <bool BF16, bool VEC>
__device__ void ee_race(const EeParams& p, int b, int s, int rc, const EeReq& r) {
  __shared__ float sh_k[kWaves];
  __shared__ int sh_i[kWaves];
  __shared__ int sh_expired;
  const int tid = threadIdx.x;
  EeRace rr{};
  rr.cf = kLog2e / r.T;
  if (s == 0) {
    if (r.K != 0) return;
    rr.n = 0;
    rr.residual = false;
  } else {
    uint32_t code = 0;
    if (!dec_wait(p, b, s - 1, 0, code)) {
      if (rc == p.ngr - 1 && tid == 0) p.accept_len[b] = -1;
      return;
    }
    const uint32_t kind = code & 0xFFu;
    if (kind == kRej && static_cast<int>(code >> 8) == s - 1) {
      rr.n = s - 1;
      rr.residual = true;
      uint32_t v[4];
      bool ok = true;
      for (int k = 0; k < 4; ++k) ok = dec_wait(p, b, s - 1, k + 1, v[k]) && ok;
      if (!ok) {
        if (rc == p.ngr - 1 && tid == 0) p.accept_len[b] = -1;
        return;
      }
      rr.mp = __uint_as_float(v[0]);
      rr.lsp = __uint_as_float(v[1]);
      rr.mq = __uint_as_float(v[2]);
      rr.lsq = __uint_as_float(v[3]);
    } else if (kind == kCont && s == r.K) {
      rr.n = s;
      rr.residual = false;
    } else {
      return;
    }
  }
  float key = -INFINITY;
  int idx = INT_MAX;
  bool bad = false;
  const int c_lo = rc * p.rcw, c_hi = min(c_lo + p.rcw, p.nc);
  ee_race_range<BF16, VEC>(p, b, r, rr, c_lo, c_hi, key, idx, bad);
  block_argmax(key, idx, sh_k, sh_i);
  bad = __syncthreads_or(bad) != 0;
  if (tid == 0)
    slot_store(p.race + static_cast<int64_t>(b) * p.ngr + rc,
               pack_slot(bad ? -INFINITY : key, bad ? kBadRowIdx : static_cast<uint32_t>(idx)));
  if (rc != p.ngr - 1) return;
  // the request's last race workgroup: fold the winners, write the outputs
  if (tid == 0) sh_expired = 0;
  __syncthreads();
  key = -INFINITY;
  idx = INT_MAX;
  for (int i = tid; i < p.ngr; i += kThreads) {
    uint64_t* slot = p.race + static_cast<int64_t>(b) * p.ngr + i;
    const uint64_t v = slot_wait(slot);
    slot_store(slot, 0u);
    if (v == 0u) {
      atomicOr(&sh_expired, 1);
      continue;
    }
    if (slot_w(v) == kBadRowIdx) {
      atomicOr(&sh_expired, 2);
      continue;
    }
    merge_argmax(key, idx, slot_f(v), static_cast<int>(slot_w(v)));
  }
  block_argmax(key, idx, sh_k, sh_i);  // its barriers also publish sh_expired
  if (sh_expired & 1) {
    if (tid == 0) p.accept_len[b] = -1;
    return;
  }
  // a bonus row with a NaN or a +inf maximum, or with no finite maximum (no
  // token has a positive weight), fails the request
  if ((sh_expired & 2) || (!rr.residual && idx == INT_MAX)) {
    ee_fault(p, b, r, true);
    return;
  }
  if (idx == INT_MAX) {
    // no token had p > q (rounding can only cause this when p == q): race on p_n
    EeRace rb = rr;
    rb.residual = false;
    key = -INFINITY;
    bool unused = false;
    ee_race_range<BF16, VEC>(p, b, r, rb, 0, p.nc, key, idx, unused);
    block_argmax(key, idx, sh_k, sh_i);
  }
  ee_outputs(p, b, r, rr.n, idx);
}

// ------------------------------------------------------------------ kernel

// bfloat16 rows: at most 128 VGPRs, four waves per SIMD; float32 rows: at
// most 96, five waves per SIMD (their races take half chunks)
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BF16 ? 4 : 5))) void sv_verify_ee(
    EeParams p) {
  const int g = blockIdx.x;
  int s, b, j;            // stage, request, group (j >= ngs: race group j - ngs)
  bool end_race = false;  // a race workgroup of the end region (s = 0 stands in)
  if (p.endrace) {
    const int region = p.B * p.ngs;
    const int n_stats = (p.max_k + 1) * region;
    if (g < n_stats) {
      s = g / region;
      const int t = g - s * region;
      b = t / p.ngs;
      j = t - b * p.ngs;
    } else {
      const int t = g - n_stats;
      s = 0;
      b = t / p.ngr;
      j = p.ngs + (t - b * p.ngr);
      end_race = true;
    }
  } else {
    const int per_req = p.ngs + p.ngr;
    const int region = p.B * per_req;
    s = g / region;
    const int t = g - s * region;
    b = t / per_req;
    j = t - b * per_req;
  }
  // A request that stopped before stage s has a stop in the record of stage
  // s - 1 (its own decision, or one copied by publish_stop), so the
  // workgroups of its later stages exit on that one load, issued beside the
  // request's scalars, rather than after the token check (which waits for
  // each token in turn).  A race workgroup still runs after a rejection at
  // s - 1 itself.
  const uint64_t d = s > 0 ? slot_load(ee_dec(p, b, s - 1, 0)) : 0u;
  EeReq r = ee_req_scalars(p, b, s);
  bool cont_prev = false;  // stage s - 1 is decided and accepted
  {
    const uint32_t code = static_cast<uint32_t>(d), kind = code & 0xFFu;
    const bool rejected_here = kind == kRej && static_cast<int>(code >> 8) == s - 1;
    if (d != 0u && kind != kCont && !(j >= p.ngs && rejected_here)) return;
    cont_prev = d != 0u && kind == kCont;
  }
  // Workgroups with nothing to do for this request also exit before its
  // token check.  (The request's faults are reported by workgroup 0 of
  // region 0, which always checks.)
  if (r.valid) {
    if (j < p.ngs) {
      // a sampled request has no statistics at s = K; groups past the items
      if (!r.greedy && s == r.K) return;
      const int n_items = (r.greedy ? 1 : kStageRows) * p.nc;
      if (j > (n_items + kGroupItems - 1) / kGroupItems - 1) return;
    } else {
      // a greedy request has no races; with races per region, region 0 races
      // only K = 0 requests, and after an acceptance at s - 1 only the bonus
      // stage s = K races
      if (r.greedy || (!end_race && ((s == 0 && r.K != 0) || (cont_prev && s < r.K)))) return;
    }
  }
  ee_req_tokens(p, r);
  if (!r.valid) {
    // (s = 0 never exceeds K_b, so region 0 sees every genuine failure)
    if (s == 0 && j == 0) {
      const int32_t off1 = p.offsets[b + 1];
      const bool slice_ok = r.off0 >= 0 && off1 <= p.n_draft_rows && off1 >= r.off0 &&
                            r.K <= p.max_k;
      ee_fault(p, b, r, slice_ok);
    }
    return;
  }
  if (s > r.K) return;
  if (j < p.ngs) {
    // statistics of stage s (a sampled request has none at s = K)
    if (!r.greedy && s == r.K) return;
    const int n_items = (r.greedy ? 1 : kStageRows) * p.nc;
    const int last = (n_items + kGroupItems - 1) / kGroupItems - 1;
    if (j > last) return;
    // stream without waiting for the decision of stage s - 1 (a stop already
    // published was seen above); small batches then stream their stages
    // together instead of one after another (B=16 K=8 fp32 62 -> 44 us,
    // B=64 ragged 80 -> 60 us, B=1024 ragged 414 -> 397 us)
    if (r.greedy)
      ee_stats<BF16, VEC, true>(p, b, s, j, r);
    else
      ee_stats<BF16, VEC, false>(p, b, s, j, r);
    if (j == last) {
      __syncthreads();
      if (s > 0) {
        // decide only after an acceptance at s - 1; after a stop the stage's
        // partials are left to ee_clear_records
        uint32_t code = 0;
        if (!dec_wait(p, b, s - 1, 0, code)) {
          if (threadIdx.x == 0) p.accept_len[b] = -1;
          return;
        }
        if ((code & 0xFFu) != kCont) return;
      }
      ee_decide<BF16>(p, b, s, r);
    }
  } else if (!r.greedy) {
    int sr = s;  // the race's stage: a rejection at sr - 1, or the bonus at sr = K
    if (end_race && r.K > 0) {
      // the request's stop, copied into the record of its last draft position
      uint32_t code = 0;
      if (!dec_wait(p, b, r.K - 1, 0, code)) {
        if (j - p.ngs == p.ngr - 1 && threadIdx.x == 0) p.accept_len[b] = -1;
        return;
      }
      const uint32_t kind = code & 0xFFu;
      if (kind == kCont)
        sr = r.K;
      else if (kind == kRej)
        sr = static_cast<int>(code >> 8) + 1;
      else
        return;  // stopped without a race (a failure)
    }
    ee_race<BF16, VEC>(p, b, sr, j - p.ngs, r);
  }
}

// ------------------------------------------------------------------ host side

int64_t ee_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }


struct EeLayout {
  size_t part_off, race_off, dec_off, total;
};

size_t ee_round256(size_t x) { return (x + 255) / 256 * 256; }

EeLayout ee_layout(int32_t B, int32_t V, int32_t max_k) {
  const size_t nc = static_cast<size_t>(ee_ceil_div(V, chunk_tokens(false)));
  const size_t S = static_cast<size_t>(max_k) + 1;
  EeLayout L;
  L.part_off = 0;
  L.race_off = ee_round256(static_cast<size_t>(B) * S * kStageRows * nc * sizeof(uint64_t));
  L.dec_off = L.race_off + ee_round256(static_cast<size_t>(B) * nc * sizeof(uint64_t));
  L.total = L.dec_off + ee_round256(static_cast<size_t>(B) * S * kDecSlots * sizeof(uint64_t));
  return L;
}

// After the verify kernel (same stream): zeroes the decision records and the
// stage partials (those streamed on speculation past a stop are still set;
// every other partial was zeroed by its reader).  Every slot takes a store,
// with no load first: one memory round trip (B=64 K=4 bf16 40.6 -> 39.9 us
// per call against loading each partial and storing the few still set).
__global__ __launch_bounds__(kThreads) void ee_clear_records(uint64_t* dec, int64_t n_dec,
                                                              uint64_t* part, int64_t n_part) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
       i < n_dec + n_part; i += static_cast<int64_t>(gridDim.x) * kThreads) {
    if (i < n_dec)
      dec[i] = 0u;
    else
      part[i - n_dec] = 0u;
  }
}

template <bool BF16, bool VEC>
int ee_launch(const EeParams& prm, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((sv_verify_ee<BF16, VEC>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads),
                     0, stream, prm);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  const int64_t n_dec = static_cast<int64_t>(prm.B) * (prm.max_k + 1) * kDecSlots;
  const int64_t n_part = static_cast<int64_t>(prm.B) * (prm.max_k + 1) * kStageRows * prm.nc;
  const int64_t clear_wgs = std::min<int64_t>(1024, (n_dec + n_part + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(ee_clear_records, dim3(static_cast<uint32_t>(clear_wgs)), dim3(kThreads), 0,
                     stream, prm.dec, n_dec, prm.part, n_part);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t spec_verify_early_exit_workspace_bytes(int32_t B, int32_t V, int32_t max_k) {
  if (B < 1 || V < 1 || max_k < 0 || max_k > SV_KMAX) return 0;
  return ee_layout(B, V, max_k).total;
}

int spec_verify_sample_early_exit(const void* target_logits, const void* draft_logits,
                                  int32_t dtype, int32_t B, int32_t V, int32_t max_k,
                                  int32_t n_draft_rows, const int32_t* draft_offsets,
                                  const int32_t* draft_tokens, const float* temperature,
                                  uint64_t seed, int32_t* accept_len, int32_t* out_tokens,
                                  float* p_at_draft, float* q_at_draft, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!target_logits || !draft_offsets || !accept_len || !out_tokens || !workspace ||
      !temperature)
    return SV_ERR_NULL;
  if (n_draft_rows > 0 && (!draft_logits || !draft_tokens)) return SV_ERR_NULL;
  if (B < 1 || V < 1 || max_k < 0 || max_k > SV_KMAX || n_draft_rows < 0) return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (workspace_bytes < spec_verify_early_exit_workspace_bytes(B, V, max_k) ||
      (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return SV_ERR_WORKSPACE;
  const bool bf16 = dtype == SV_BF16;
  const EeLayout L = ee_layout(B, V, max_k);
  char* ws = static_cast<char*>(workspace);
  EeParams prm;
  prm.target = target_logits;
  prm.draft = draft_logits;
  prm.offsets = draft_offsets;
  prm.tokens = draft_tokens;
  prm.temperature = temperature;
  prm.k0 = static_cast<uint32_t>(seed);
  prm.k1 = static_cast<uint32_t>(seed >> 32);
  prm.B = B;
  prm.V = V;
  prm.max_k = max_k;
  prm.n_draft_rows = n_draft_rows;
  prm.nc = static_cast<int32_t>(ee_ceil_div(V, chunk_tokens(bf16)));
  prm.ngs = static_cast<int32_t>(ee_ceil_div(static_cast<int64_t>(kStageRows) * prm.nc, kGroupItems));
  prm.rcw = static_cast<int64_t>(B) * ee_ceil_div(prm.nc, kRaceChunks) < kNarrowRaceBelow ||
                    (bf16 && max_k > 1)
                ? kRaceChunksNarrow
                : kRaceChunks;
  prm.ngr = static_cast<int32_t>(ee_ceil_div(prm.nc, prm.rcw));
  prm.part = reinterpret_cast<uint64_t*>(ws + L.part_off);
  prm.race = reinterpret_cast<uint64_t*>(ws + L.race_off);
  prm.dec = reinterpret_cast<uint64_t*>(ws + L.dec_off);
  prm.accept_len = accept_len;
  prm.out_tokens = out_tokens;
  prm.p_at = p_at_draft;
  prm.q_at = q_at_draft;
  // Races at the end unless they are mostly bonus races (K = 1) and more than
  // one resident generation: B=512 K=1 bf16 77.9 us per region against 93.5
  // at the end, while at the end B=1024 ragged K <= 8 runs 402 -> 355 us,
  // B=64 K=4 44.3 -> 40.3 us and B=64 K=1 31.8 -> 26.9 us.
  const int64_t resident = static_cast<int64_t>(bf16 ? 4 : 5) * device_compute_units();
  prm.endrace = max_k > 1 || static_cast<int64_t>(B) * prm.ngr <= resident;
  // With the races in every region, a request's statistics and races span
  // ngs + ngr workgroups, and the dispatcher deals workgroups to the XCDs
  // round robin by index: with fewer race workgroups than XCDs and a span that
  // is a multiple of the XCD count, every request's races would run on the
  // same few XCDs.  Narrower races rotate them (B=512 K=1 V=70000 bf16:
  // 93.3 -> 68.8 us; B=768 V=65600: 129.6 -> 92.4 us).
  while (!prm.endrace && prm.ngr < kEeXcds && (prm.ngs + prm.ngr) % kEeXcds == 0 &&
         prm.rcw > 1) {
    --prm.rcw;
    prm.ngr = static_cast<int32_t>(ee_ceil_div(prm.nc, prm.rcw));
  }
  const int64_t grid =
      prm.endrace ? static_cast<int64_t>(max_k + 1) * B * prm.ngs + static_cast<int64_t>(B) * prm.ngr
                  : static_cast<int64_t>(max_k + 1) * B * (prm.ngs + prm.ngr);
  if (grid > INT32_MAX) return SV_ERR_SHAPE;
  const int64_t row_bytes = static_cast<int64_t>(V) * (bf16 ? 2 : 4);
  const bool vec = row_bytes % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(target_logits) & 15u) == 0 &&
                   (!draft_logits || (reinterpret_cast<uintptr_t>(draft_logits) & 15u) == 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (bf16) return vec ? ee_launch<true, true>(prm, grid, st) : ee_launch<true, false>(prm, grid, st);
  return vec ? ee_launch<false, true>(prm, grid, st) : ee_launch<false, false>(prm, grid, st);
}

}  // extern "C"
