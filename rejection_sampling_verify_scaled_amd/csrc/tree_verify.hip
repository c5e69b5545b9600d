// tree_verify.hip -- gfx950 kernel and C ABI of greedy draft-tree verification.
//
// What is computed is stated in include/spec_verify.h (spec_verify_tree_greedy):
// the target scored every node of a draft tree in one pass, each node seeing
// only its ancestors ("Decodificación Especulativa y EAGLE", section on tree
// attention verification); a node is accepted when its parent is accepted and
// its token is the argmax of its parent's row (the greedy rule of section "La
// Regla de Exactitud"); the result is the deepest accepted node (lowest index
// among equals), the tokens on its root path, and the argmax of its own row
// as the extra target token (Perplexity's post, section "EAGLE").
//
// The work is the argmax of every node's row: HBM streaming, as for the
// greedy rows of the linear verify, with the same row-chunk reduction.  One
// launch; request b owns ng consecutive workgroups, workgroup j taking block
// j mod nb of node j / nb: 8 row-chunks (8 KiB each) of that node's row.  It
// merges them in LDS into one (max, argmax) partial per block (the merge is
// exact in any order), so a row leaves ceil(nc / 8) partials in the
// workspace instead of nc (16 EAGLE-style trees: 32.5 -> 30.4 us).  The
// request's last workgroup with items then
//   1. folds the partials of every node's row (up to 2048 partials staged in
//      LDS at a time; lane l holds row l and each wave scans a quarter),
//   2. runs the tree logic in one wave, lane i = node i (at most 64 nodes):
//      node i accepts its edge when token_i equals the argmax of its parent's
//      row; acceptance along the root path and the depth come from pointer
//      jumping over the parent links (6 rounds of lane shuffles for depth up
//      to 63), and a wave reduction picks the deepest accepted node;
//   3. marks the chosen path by walking up the parent links and writes the
//      outputs, one position per lane.
// Partials follow the zero-slot protocol of the verify kernel: written once
// per call, read and zeroed by the finishing workgroup, all waits bounded.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "spec_verify.h"
#include "device_common.h"

namespace {

constexpr int kFoldBlock = 2048;                     // partials staged in LDS per block
constexpr int kFoldPerThread = kFoldBlock / kThreads;  // 8
constexpr int kJumpRounds = 6;                       // 2^6 >= SV_TREE_MAX_NODES - 1 edges

static_assert(SV_TREE_MAX_NODES <= 64, "one wave holds a request's nodes");
static_assert(kFoldBlock % kThreads == 0, "fold block is a whole number of rounds");

struct TreeParams {
  const void* target;
  const int32_t* offsets;  // [B+1]
  const int32_t* parents;  // [n_rows]
  const int32_t* tokens;   // [n_rows]
  int32_t B, V, max_nodes, n_rows;
  int32_t nc;  // chunks per row
  int32_t nb;  // blocks per row: ceil(nc / 8), one partial each
  int32_t ng;  // workgroups per request: max_nodes * nb
  uint64_t* part;  // [B][max_nodes][nb] block partials
  int32_t* accept_len;
  int32_t* out_tokens;
  int32_t* accept_nodes;  // or NULL
};

__device__ __forceinline__ uint64_t* tree_part(const TreeParams& p, int b, int node, int c) {
  return p.part + (static_cast<int64_t>(b) * p.max_nodes + node) * p.nb + c;
}

// This workgroup's block: row-chunks [8 k, 8 k + 8) of node j / nb's row
// (k = j mod nb).  Wave w loads items 2w and 2w + 1 (both in flight) and
// reduces each to its (max, lowest argmax); the block's partials are merged
// in LDS and published as one.
template <bool BF16, bool VEC>
__device__ void tree_items(const TreeParams& p, int b, int32_t off, int j) {
  __shared__ uint64_t sh_block[kGroupItems];
  constexpr int CHUNK = chunk_tokens(BF16);
  constexpr int IN_FLIGHT = VEC ? kItemsInFlight : 1;
  const int lane = threadIdx.x & 63, wave = wave_id();
  // block k = j mod nb of node j / nb: its row's chunks [8 k, 8 k + 8)
  const int bnode = j / p.nb, bk = j - bnode * p.nb;
  const int i_lo = bnode * p.nc + bk * kGroupItems;
  const int i_hi = min(i_lo + kGroupItems, (bnode + 1) * p.nc);
  for (int i0 = i_lo + wave * IN_FLIGHT; i0 < i_hi; i0 += kWaves * IN_FLIGHT) {
    uint4 buf[IN_FLIGHT][kItemVecs];
#pragma unroll
    for (int k = 0; k < IN_FLIGHT; ++k) {
      // past the last item the wave loads the last item again and skips it
      const int i = min(i0 + k, i_hi - 1);
      const int node = i / p.nc;
      const int c = i - node * p.nc;
      load_item<BF16, VEC>(p.target, static_cast<int64_t>(off) + node, p.V,
                           static_cast<int64_t>(c) * CHUNK, buf[k]);
    }
#pragma unroll
    for (int k = 0; k < IN_FLIGHT; ++k) {
      const int i = i0 + k;
      if (i < i_hi) {
        const int node = i / p.nc;
        const int c = i - node * p.nc;
        if (VEC && static_cast<int64_t>(c + 1) * CHUNK > p.V)
          mask_tail<BF16>(buf[k], p.V, static_cast<int64_t>(c) * CHUNK);
        const uint64_t v = item_argmax<BF16>(buf[k], static_cast<int64_t>(c) * CHUNK);
        if (lane == 0) sh_block[i - i_lo] = v;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = -INFINITY;
    int mi = INT_MAX;
    for (int i = 0; i < i_hi - i_lo; ++i)
      merge_argmax(m, mi, slot_f(sh_block[i]), static_cast<int>(slot_w(sh_block[i])));
    slot_store(tree_part(p, b, bnode, bk), pack_slot(m, static_cast<uint32_t>(mi)));
  }
}

struct TreeShared {
  uint64_t slots[kFoldBlock];
  float wave_v[kWaves][SV_TREE_MAX_NODES];  // each wave's share of a block's rows
  int wave_i[kWaves][SV_TREE_MAX_NODES];
  float row_v[SV_TREE_MAX_NODES];  // folded row maximum
  int row_i[SV_TREE_MAX_NODES];    // lowest index attaining it
  int expired;
};

// Every node's row argmax, from the block partials (which are zeroed once
// read).  Rows are taken R at a time with all their blocks, R * nb <= 2048; a
// row of more than 2048 blocks is taken alone, 2048 blocks at a time.  In a block,
// lane l holds row l and wave w scans its quarter of the chunks from LDS (a
// chain of independent LDS reads, not of cross-lane shuffles); wave 0 then
// merges the four quarters in order into the running row results.
__device__ void fold_tree_rows(const TreeParams& p, int b, int N, TreeShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  if (tid < SV_TREE_MAX_NODES) {
    sh.row_v[tid] = -INFINITY;
    sh.row_i[tid] = INT_MAX;
  }
  if (tid == 0) sh.expired = 0;
  const int nb = p.nb;
  const int C = min(nb, kFoldBlock);
  const int R = max(1, kFoldBlock / C);
  bool expired = false;
  for (int r0 = 0; r0 < N; r0 += R) {
    const int rr = min(R, N - r0);
    for (int c0 = 0; c0 < nb; c0 += C) {
      const int cc = min(C, nb - c0);
      const int n_slots = rr * cc;
      __syncthreads();  // the previous block's LDS reads are done
      uint64_t v[kFoldPerThread];
#pragma unroll
      for (int k = 0; k < kFoldPerThread; ++k) {  // issue every load before waiting on any
        const int q = min(tid + k * kThreads, n_slots - 1);
        const int row = q / cc;
        v[k] = slot_load(tree_part(p, b, r0 + row, c0 + q - row * cc));
      }
      uint32_t missing = 0u;
#pragma unroll
      for (int k = 0; k < kFoldPerThread; ++k)
        if (tid + k * kThreads < n_slots && v[k] == 0u) missing |= 1u << k;
      for (unsigned it = 0; missing != 0u && it < kSpinLimit; ++it) {
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int k = 0; k < kFoldPerThread; ++k) {
          if (missing & (1u << k)) {
            const int q = tid + k * kThreads;
            const int row = q / cc;
            v[k] = slot_load(tree_part(p, b, r0 + row, c0 + q - row * cc));
            if (v[k] != 0u) missing &= ~(1u << k);
          }
        }
      }
      if (missing != 0u) expired = true;
#pragma unroll
      for (int k = 0; k < kFoldPerThread; ++k) {
        const int q = tid + k * kThreads;
        if (q < n_slots) {
          sh.slots[q] = v[k];
          if (v[k] != 0u) {  // read once: clear it for the next call
            const int row = q / cc;
            slot_store(tree_part(p, b, r0 + row, c0 + q - row * cc), 0u);
          }
        }
      }
      __syncthreads();
      const int cpw = (cc + kWaves - 1) / kWaves;
      const int cb = wave * cpw, ce = min(cb + cpw, cc);
      if (lane < rr) {
        float mv = -INFINITY;
        int mi = INT_MAX;
        const uint64_t* rs = sh.slots + lane * cc;
        for (int c = cb; c < ce; ++c) {
          const uint64_t x = rs[c];
          if (x != 0u) merge_argmax(mv, mi, slot_f(x), static_cast<int>(slot_w(x)));
        }
        sh.wave_v[wave][lane] = mv;
        sh.wave_i[wave][lane] = mi;
      }
      __syncthreads();
      if (wave == 0 && lane < rr) {
        float rv = sh.row_v[r0 + lane];
        int ri = sh.row_i[r0 + lane];
        for (int w = 0; w < kWaves; ++w) merge_argmax(rv, ri, sh.wave_v[w][lane], sh.wave_i[w][lane]);
        sh.row_v[r0 + lane] = rv;
        sh.row_i[r0 + lane] = ri;
      }
    }
  }
  if (expired) atomicOr(&sh.expired, 1);
  __syncthreads();
}

__device__ __forceinline__ int lane_int(int v, int src) { return __shfl(v, src, 64); }

// Fold, tree logic and outputs of request b (the request's last workgroup).
__device__ void tree_finish(const TreeParams& p, int b, int32_t off, int N) {
  __shared__ TreeShared sh;
  __syncthreads();  // this workgroup's own partials are stored
  fold_tree_rows(p, b, N, sh);
  if (wave_id() != 0) return;
  const int i = threadIdx.x & 63;
  const bool live = i < N;
  int par = 0, tok = -1, g = -1;
  bool bad = false;
  if (live) {
    const float gv = sh.row_v[i];
    g = sh.row_i[i];
    bad = !(gv > -INFINITY && gv < INFINITY);
    if (i >= 1) {
      par = p.parents[off + i];
      tok = p.tokens[off + i];
      bad = bad || par < 0 || par >= i || tok < 0 || tok >= p.V;
    }
  }
  if (__any(bad) || sh.expired) {
    if (live) {
      p.out_tokens[off + i] = -1;
      if (p.accept_nodes) p.accept_nodes[off + i] = -1;
    }
    if (i == 0) p.accept_len[b] = -1;
    return;
  }
  // edge i -> parent accepted when token_i is the parent's argmax
  const int g_par = lane_int(g, par);
  int acc = live && (i == 0 || tok == g_par) ? 1 : 0;
  int anc = par;  // root and idle lanes point at node 0
  int dep = (live && i > 0) ? 1 : 0;
  // pointer jumping: after round r, acc and dep cover the 2^(r+1) nearest
  // edges of the root path (or all of them), anc is the node above those
#pragma unroll
  for (int r = 0; r < kJumpRounds; ++r) {
    const int acc_a = lane_int(acc, anc);
    const int dep_a = lane_int(dep, anc);
    const int anc_a = lane_int(anc, anc);
    acc &= acc_a;
    dep += dep_a;
    anc = anc_a;
  }
  // deepest accepted node, lowest index among equals: maximise (depth, 63 - i)
  int key = (live && acc) ? ((dep + 1) << 8) | (63 - i) : 0;
  key = wave_max_int(key);
  const int c = 63 - (key & 255);
  const int d = (key >> 8) - 1;
  // mark the path root .. c (d + 1 nodes)
  bool on = false;
  int cur = c;
  for (int k = d; k >= 0; --k) {
    on = on || i == cur;
    cur = lane_int(par, cur);
  }
  if (live) {
    if (on) {
      if (i > 0) p.out_tokens[off + dep - 1] = tok;
      if (p.accept_nodes) p.accept_nodes[off + dep] = i;
    }
    if (i == c) p.out_tokens[off + d] = g;
    if (i > d) {
      p.out_tokens[off + i] = -1;
      if (p.accept_nodes) p.accept_nodes[off + i] = -1;
    }
  }
  if (i == 0) p.accept_len[b] = d;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void tv_verify(TreeParams p) {
  const int b = blockIdx.x / p.ng;
  const int j = blockIdx.x - b * p.ng;
  const int32_t off = p.offsets[b], off1 = p.offsets[b + 1];
  const int32_t N = static_cast<int32_t>(static_cast<uint32_t>(off1) - static_cast<uint32_t>(off));
  const bool slice_ok = off >= 0 && off1 <= p.n_rows && off1 >= off && N >= 1 && N <= p.max_nodes;
  if (!slice_ok) {
    if (j == 0 && threadIdx.x == 0) p.accept_len[b] = -1;
    return;
  }
  const int last = N * p.nb - 1;
  if (j > last) return;
  tree_items<BF16, VEC>(p, b, off, j);
  if (j == last) tree_finish(p, b, off, N);
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool tree_shape_ok(int32_t B, int32_t V, int32_t max_nodes) {
  return B >= 1 && V >= 1 && max_nodes >= 1 && max_nodes <= SV_TREE_MAX_NODES;
}

template <bool BF16, bool VEC>
int tv_launch(const TreeParams& prm, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((tv_verify<BF16, VEC>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads),
                     0, stream, prm);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

// Sized with the float32 chunk (more blocks per row) so either dtype fits.
size_t spec_verify_tree_workspace_bytes(int32_t B, int32_t V, int32_t max_nodes) {
  if (!tree_shape_ok(B, V, max_nodes)) return 0;
  const size_t nb = static_cast<size_t>(ceil_div64(ceil_div64(V, chunk_tokens(false)), kGroupItems));
  return (static_cast<size_t>(B) * max_nodes * nb * sizeof(uint64_t) + 255) / 256 * 256;
}

int spec_verify_tree_greedy(const void* target_logits, int32_t dtype, int32_t B, int32_t V,
                            int32_t max_nodes, int32_t n_rows, const int32_t* node_offsets,
                            const int32_t* parents, const int32_t* tokens, int32_t* accept_len,
                            int32_t* out_tokens, int32_t* accept_nodes, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!target_logits || !node_offsets || !parents || !tokens || !accept_len || !out_tokens ||
      !workspace)
    return SV_ERR_NULL;
  if (!tree_shape_ok(B, V, max_nodes) || n_rows < 0) return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (workspace_bytes < spec_verify_tree_workspace_bytes(B, V, max_nodes) || !aligned16(workspace))
    return SV_ERR_WORKSPACE;
  const bool bf16 = dtype == SV_BF16;
  TreeParams prm;
  prm.target = target_logits;
  prm.offsets = node_offsets;
  prm.parents = parents;
  prm.tokens = tokens;
  prm.B = B;
  prm.V = V;
  prm.max_nodes = max_nodes;
  prm.n_rows = n_rows;
  prm.nc = static_cast<int32_t>(ceil_div64(V, chunk_tokens(bf16)));
  prm.nb = static_cast<int32_t>(ceil_div64(prm.nc, kGroupItems));
  const int64_t ng = static_cast<int64_t>(max_nodes) * prm.nb;
  const int64_t grid = static_cast<int64_t>(B) * ng;
  if (ng > INT32_MAX || grid <= 0 || grid > INT32_MAX) return SV_ERR_SHAPE;
  prm.ng = static_cast<int32_t>(ng);
  prm.part = static_cast<uint64_t*>(workspace);
  prm.accept_len = accept_len;
  prm.out_tokens = out_tokens;
  prm.accept_nodes = accept_nodes;
  const int64_t row_bytes = static_cast<int64_t>(V) * (bf16 ? 2 : 4);
  const bool vec = row_bytes % 16 == 0 && aligned16(target_logits);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16) return vec ? tv_launch<true, true>(prm, grid, s) : tv_launch<true, false>(prm, grid, s);
  return vec ? tv_launch<false, true>(prm, grid, s) : tv_launch<false, false>(prm, grid, s);
}

}  // extern "C"
