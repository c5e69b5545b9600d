// valu_rates.hip -- issue rates of the VALU instruction classes the samplers
// use, measured on the device (a measurement library, not part of the
// verify path; built as libspecverify_rates.so).
//
// Each thread runs 16 independent chains of one operation for a fixed number
// of iterations over a grid of 8 workgroups of 256 threads per CU; the host
// times the launch with HIP events and workgroup 0 reads the shader clock
// (clock64) against the constant-rate wall clock (wall_clock64), so a rate
// can be stated per SIMD and clock cycle.  The operations, one per loop body:
//   0  v_fma_f32                      (a full-rate 32-bit operation)
//   1  v_exp_f32                      (transcendental)
//   2  v_log_f32                      (transcendental)
//   3  v_mad_u64_u32 + v_add_u32      (Philox4x32-10's 32 x 32 -> 64 product)
//   4  v_mul_lo_u32 + v_add_u32
//   5  v_xor_b32 + v_add_u32          (two full-rate integer operations)
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kChains = 16;

template <int OP>
__global__ __launch_bounds__(256) void valu_rate_kernel(float* out, unsigned long long* clk,
                                                        uint32_t seed, int iters) {
  float a[kChains];
  uint32_t u[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) {
    a[i] = static_cast<float>(threadIdx.x + i) * 1e-3f + 0.5f;
    u[i] = seed ^ (threadIdx.x * kChains + i);
  }
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
      if constexpr (OP == 0) {
        a[i] = __builtin_fmaf(a[i], 0.999f, 1e-4f);
      } else if constexpr (OP == 1) {
        a[i] = __builtin_amdgcn_exp2f(a[i]);
      } else if constexpr (OP == 2) {
        a[i] = __builtin_amdgcn_logf(a[i]);
      } else if constexpr (OP == 3) {
        const uint64_t pr = static_cast<uint64_t>(u[i]) * 0xD2511F53u;
        u[i] = static_cast<uint32_t>(pr >> 32) + static_cast<uint32_t>(pr);
      } else if constexpr (OP == 4) {
        u[i] = u[i] * 0x9E3779B9u + 0xBB67AE85u;
      } else {
        u[i] = (u[i] ^ 0x9E3779B9u) + 0xBB67AE85u;
      }
    }
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += a[i] + static_cast<float>(u[i] & 1u);
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = c1 - c0;
    clk[1] = w1 - w0;
  }
}

template <int OP>
hipError_t launch(int blocks, float* out, unsigned long long* clk, int iters) {
  hipLaunchKernelGGL(valu_rate_kernel<OP>, dim3(blocks), dim3(256), 0, nullptr, out, clk, 1u,
                     iters);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Runs operation `op` (0..5, above) three times on the current device and
// reports the fastest launch: *ms its duration, *bodies the loop bodies
// executed (threads x iterations x chains), *shader_mhz the shader clock seen
// by workgroup 0 (wall clock at wall_mhz MHz).  Returns 0, or -1 on a bad
// argument or a HIP error.
int sv_valu_rate(int op, int cu_count, double wall_mhz, float* ms, double* bodies,
                 double* shader_mhz) {
  if (op < 0 || op > 5 || cu_count < 1 || cu_count > 4096 || !ms || !bodies || !shader_mhz)
    return -1;
  const int blocks = cu_count * 8, iters = 4000;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  if (hipMalloc(&out, sizeof(float) * blocks * 256) != hipSuccess) return -1;
  if (hipMalloc(&clk, 2 * sizeof(unsigned long long)) != hipSuccess) {
    (void)hipFree(out);
    return -1;
  }
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  float best = 0.f;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) rc = -1;
  for (int rep = 0; rc == 0 && rep < 3; ++rep) {
    hipError_t e = hipEventRecord(e0, nullptr);
    if (e == hipSuccess) {
      switch (op) {
        case 0: e = launch<0>(blocks, out, clk, iters); break;
        case 1: e = launch<1>(blocks, out, clk, iters); break;
        case 2: e = launch<2>(blocks, out, clk, iters); break;
        case 3: e = launch<3>(blocks, out, clk, iters); break;
        case 4: e = launch<4>(blocks, out, clk, iters); break;
        default: e = launch<5>(blocks, out, clk, iters); break;
      }
    }
    if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
    if (e != hipSuccess) {
      rc = -1;
      break;
    }
    if (rep == 0 || t < best) best = t;
  }
  unsigned long long c[2] = {0, 0};
  if (rc == 0 && hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost) != hipSuccess) rc = -1;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  (void)hipFree(clk);
  if (rc != 0) return rc;
  *ms = best;
  *bodies = static_cast<double>(blocks) * 256.0 * iters * kChains;
  *shader_mhz = c[1] ? static_cast<double>(c[0]) / static_cast<double>(c[1]) * wall_mhz : 0.0;
  return 0;
}

}  // extern "C"
