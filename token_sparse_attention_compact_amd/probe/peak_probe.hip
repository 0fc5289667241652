// Attainable-peak probes (measurement only, not part of the HSA path):
//  * a register-only loop of v_mfma_f32_32x32x16_bf16 with four independent
//    accumulators per wavefront, eight wavefronts per workgroup: what the
//    matrix cores deliver at the clock they hold under MFMA load;
//  * a streaming copy (16-byte non-temporal loads and stores, four per
//    thread in flight): what HBM delivers to a plain read + write stream.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512, 1) void mfma_peak_kernel(float* __restrict__ out, int32_t iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each thread moves 4 x 16 bytes per round; rounds stride over the grid.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x) * 4 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + (int64_t)u * blockDim.x;
      if (j < n16) v[u] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + (int64_t)u * blockDim.x;
      if (j < n16) __builtin_nontemporal_store(v[u], dst + j);
    }
  }
}

}  // namespace

// Launches n_wg workgroups of 512 threads, each wavefront issuing 16 * iters
// MFMAs of 32x32x16 (32768 FLOP each).  out: n_wg * 512 floats (device).
// Returns 0, or -1 on bad arguments / -6 on a launch error.
extern "C" int hsa_probe_mfma_peak(int32_t n_wg, int32_t iters, float* out, void* stream) {
  if (n_wg <= 0 || iters <= 0 || out == nullptr) return -1;
  mfma_peak_kernel<<<n_wg, 512, 0, (hipStream_t)stream>>>(out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Copies n_bytes (a multiple of 16; both pointers 16-byte aligned) from src
// to dst on the device.  Returns 0, or -1 on bad arguments / -6 on a launch
// error.
extern "C" int hsa_probe_copy(const void* src, void* dst, int64_t n_bytes, void* stream) {
  if (src == nullptr || dst == nullptr || n_bytes <= 0 || n_bytes % 16 != 0 ||
      ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
    return -1;
  const int64_t n16 = n_bytes / 16;
  const int64_t per_block = 256 * 4;
  const int64_t blocks = (n16 + per_block - 1) / per_block;
  const unsigned grid = (unsigned)(blocks < 256 * 32 ? blocks : 256 * 32);
  copy_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
