// Cached Euler update with the L1 relative-change score, one fused pass over
// all N tokens (cached Euler update, section 2.3; dynamic selection score,
// section 2.1).
//
// Active tokens (pos[n] >= 0) first score the fresh velocity
// against the cached one, then replace it; every token then advances by
// dsigma * v_hat.  Bandwidth-bound: per token 4 B of pos, C*4 B each of x
// (read and write) and v_hat (read), plus for active tokens C*4 B of v_new,
// C*4 B of v_hat written and 4 B of score.
#include "common.h"

namespace hsa {
namespace {

// C == 16: four lanes per token, each owning one float4 of the row, so every
// load and store instruction of a wavefront covers 1 KiB of contiguous memory.
// x, v_hat and pos are touched once per iteration and streamed with
// non-temporal loads and stores (kept out of the caches): 6.1 TB/s on a
// 3.8 GB working set on MI355X, against 4.9 TB/s with ordinary accesses;
// several tokens per lane (U > 1) measured slower.
// The score's two row sums are reduced over the four lanes with shuffles.
template <int U>
__global__ __launch_bounds__(256) void euler_kernel_c16(float* __restrict__ x, float* __restrict__ v_hat,
                                                        float* __restrict__ score,
                                                        const float* __restrict__ v_new,
                                                        const int32_t* __restrict__ pos, int32_t N,
                                                        float dsigma, float eps, int update_score) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;   // threads; tokens advance by stride/4
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int part = (int)(t0 & 3);
  int32_t n[U], p[U];
  f32x4 vh[U], xv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    n[u] = (int32_t)((t0 + u * stride) >> 2);
    const bool in = n[u] < N;
    p[u] = in ? __builtin_nontemporal_load(pos + n[u]) : -1;
    const f32x4* vp = reinterpret_cast<const f32x4*>(v_hat + (size_t)n[u] * 16) + part;
    const f32x4* xp = reinterpret_cast<const f32x4*>(x + (size_t)n[u] * 16) + part;
    vh[u] = in ? __builtin_nontemporal_load(vp) : f32x4{0.f, 0.f, 0.f, 0.f};
    xv[u] = in ? __builtin_nontemporal_load(xp) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (p[u] >= 0) {   // uniform across the four lanes of a token
      const f32x4 vn = *(reinterpret_cast<const f32x4*>(v_new + (size_t)p[u] * 16) + part);
      if (update_score) {
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          num += fabsf(vn[c] - vh[u][c]);
          den += fabsf(vh[u][c]);
        }
        num += __shfl_xor(num, 1, 4);
        den += __shfl_xor(den, 1, 4);
        num += __shfl_xor(num, 2, 4);
        den += __shfl_xor(den, 2, 4);
        if (part == 0) score[n[u]] = num / (den + eps);
      }
      vh[u] = vn;
      __builtin_nontemporal_store(vn, reinterpret_cast<f32x4*>(v_hat + (size_t)n[u] * 16) + part);
    }
    if (n[u] < N) {
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[u][c] = __builtin_fmaf(dsigma, vh[u][c], xv[u][c]);
      __builtin_nontemporal_store(xv[u], reinterpret_cast<f32x4*>(x + (size_t)n[u] * 16) + part);
    }
  }
}

// Any C that is a multiple of 4: the same pass with a runtime channel loop.
__global__ __launch_bounds__(256) void euler_kernel_any(float* __restrict__ x, float* __restrict__ v_hat,
                                                        float* __restrict__ score,
                                                        const float* __restrict__ v_new,
                                                        const int32_t* __restrict__ pos, int32_t N,
                                                        int32_t C, float dsigma, float eps,
                                                        int update_score) {
  const int32_t n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const int32_t p = pos[n];
  float* vh = v_hat + (size_t)n * C;
  float* xr = x + (size_t)n * C;
  if (p >= 0) {
    const float* vn = v_new + (size_t)p * C;
    if (update_score) {
      float num = 0.f, den = 0.f;
      for (int c = 0; c < C; ++c) {
        num += fabsf(vn[c] - vh[c]);
        den += fabsf(vh[c]);
      }
      score[n] = num / (den + eps);
    }
    for (int c = 0; c < C; ++c) vh[c] = vn[c];
  }
  for (int c = 0; c < C; ++c) xr[c] = __builtin_fmaf(dsigma, vh[c], xr[c]);
}

__global__ void gather_rows_kernel(const float* __restrict__ src, const int32_t* __restrict__ idx,
                                   float* __restrict__ dst, int32_t rows, int32_t C) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rows * C) return;
  const int32_t r = (int32_t)(t / C), c = (int32_t)(t % C);
  dst[t] = src[(size_t)idx[r] * C + c];
}

}  // namespace

hsa_status launch_euler(float* x, float* v_hat, float* score, const float* v_new,
                        const int32_t* pos, int32_t N, int32_t C, float dsigma, float eps,
                        int32_t update_score, hipStream_t s) {
  if (N == 0) return HSA_OK;
  if (C == 16) {
    constexpr int U = 1;
    const int64_t threads = (int64_t)N * 4;
    euler_kernel_c16<U><<<cdiv(threads, 256 * U), 256, 0, s>>>(x, v_hat, score, v_new, pos, N,
                                                               dsigma, eps, update_score);
  }
  else
    euler_kernel_any<<<cdiv(N, 256), 256, 0, s>>>(x, v_hat, score, v_new, pos, N, C, dsigma, eps,
                                                  update_score);
  return launch_status();
}

hsa_status launch_gather_rows(const float* src, const int32_t* idx, float* dst, int32_t rows,
                              int32_t C, hipStream_t s) {
  if (rows == 0) return HSA_OK;
  const int64_t total = (int64_t)rows * C;
  gather_rows_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(src, idx, dst, rows, C);
  return launch_status();
}

}  // namespace hsa
