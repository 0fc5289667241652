// Attainable-peak probes (measurement only, not part of the HSA path):
//  * a register-only loop of v_mfma_f32_32x32x16_bf16 with four independent
//    accumulators per wavefront, eight wavefronts per workgroup: what the
//    matrix cores deliver at the clock they hold under MFMA load, on one
//    repeated operand pair and on random operands taken in turn;
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

// The same loop with random operands: four (a, b) pairs of pseudo-random
// bf16 values per lane (random sign, exponent and mantissa, magnitudes in
// [0.5, 4)), used in turn, so that consecutive MFMAs switch their operand
// logic as a workload's do (the loop above repeats one pair, whose MFMAs
// switch little and draw less power, and the chip then holds a higher clock).
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(512, 1) void mfma_peak_random_kernel(float* __restrict__ out,
                                                                  int32_t iters) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t ha = probe_hash(tid * 64u + (uint32_t)(q * 16 + e));
      const uint32_t hb = probe_hash(tid * 64u + (uint32_t)(q * 16 + 8 + e) + 0x9e3779b9u);
      // bf16 bits: sign, exponent 126..128, 7 mantissa bits
      const uint16_t ba = (uint16_t)(((ha >> 31) << 15) | ((126u + (ha >> 8) % 3u) << 7) | (ha & 0x7fu));
      const uint16_t bb = (uint16_t)(((hb >> 31) << 15) | ((126u + (hb >> 8) % 3u) << 7) | (hb & 0x7fu));
      a[q][e] = __builtin_bit_cast(__bf16, ba);
      b[q][e] = __builtin_bit_cast(__bf16, bb);
    }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j >> 2) & 3], acc[j & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each thread moves U x 16 bytes per round (all U loads issued before the
// first store); rounds stride over the grid.
template <int U>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x) * U + threadIdx.x; i < n16; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * blockDim.x;
      if (j < n16) v[u] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
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

// As hsa_probe_mfma_peak, on random operands (four operand pairs per lane in turn).
extern "C" int hsa_probe_mfma_peak_random(int32_t n_wg, int32_t iters, float* out, void* stream) {
  if (n_wg <= 0 || iters <= 0 || out == nullptr) return -1;
  mfma_peak_random_kernel<<<n_wg, 512, 0, (hipStream_t)stream>>>(out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Copies n_bytes (a multiple of 16; both pointers 16-byte aligned) from src
// to dst on the device, each thread moving per_thread (4, 8 or 16) x 16 bytes
// per round, over at most max_blocks workgroups of 256 threads (0: as many as
// one round over the whole copy needs).  Returns 0, or -1 on bad arguments /
// -6 on a launch error.
extern "C" int hsa_probe_copy(const void* src, void* dst, int64_t n_bytes, int32_t per_thread,
                              int32_t max_blocks, void* stream) {
  if (src == nullptr || dst == nullptr || n_bytes <= 0 || n_bytes % 16 != 0 ||
      ((uintptr_t)src | (uintptr_t)dst) % 16 != 0 || max_blocks < 0 ||
      (per_thread != 4 && per_thread != 8 && per_thread != 16))
    return -1;
  const int64_t n16 = n_bytes / 16;
  const int64_t per_block = 256 * (int64_t)per_thread;
  int64_t blocks = (n16 + per_block - 1) / per_block;
  if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
  if (blocks > 0x7fffffff) blocks = 0x7fffffff;
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = (unsigned)blocks;
  if (per_thread == 4) copy_kernel<4><<<grid, 256, 0, s>>>((const u32x4*)src, (u32x4*)dst, n16);
  else if (per_thread == 8) copy_kernel<8><<<grid, 256, 0, s>>>((const u32x4*)src, (u32x4*)dst, n16);
  else copy_kernel<16><<<grid, 256, 0, s>>>((const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
