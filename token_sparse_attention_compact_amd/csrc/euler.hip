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
// The score's two row sums are reduced over the four lanes with shuffles.
__global__ __launch_bounds__(256) void euler_kernel_c16(float* __restrict__ x, float* __restrict__ v_hat,
                                                        float* __restrict__ score,
                                                        const float* __restrict__ v_new,
                                                        const int32_t* __restrict__ pos, int32_t N,
                                                        float dsigma, float eps, int update_score) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t n = (int32_t)(t >> 2);
  const int part = (int)(t & 3);
  const bool in = n < N;
  const int32_t p = in ? pos[n] : -1;
  f32x4* vh_ptr = reinterpret_cast<f32x4*>(v_hat + (size_t)n * 16) + part;
  f32x4 vh = in ? *vh_ptr : f32x4{0.f, 0.f, 0.f, 0.f};
  if (p >= 0) {
    const f32x4 vn = *(reinterpret_cast<const f32x4*>(v_new + (size_t)p * 16) + part);
    if (update_score) {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        num += fabsf(vn[c] - vh[c]);
        den += fabsf(vh[c]);
      }
      // lanes 4k..4k+3 hold one token; p >= 0 is uniform across them
      num += __shfl_xor(num, 1, 4);
      den += __shfl_xor(den, 1, 4);
      num += __shfl_xor(num, 2, 4);
      den += __shfl_xor(den, 2, 4);
      if (part == 0) score[n] = num / (den + eps);
    }
    vh = vn;
    *vh_ptr = vn;
  }
  if (in) {
    f32x4* x_ptr = reinterpret_cast<f32x4*>(x + (size_t)n * 16) + part;
    f32x4 xv = *x_ptr;
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[c] = __builtin_fmaf(dsigma, vh[c], xv[c]);
    *x_ptr = xv;
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
  if (C == 16)
    euler_kernel_c16<<<cdiv((int64_t)N * 4, 256), 256, 0, s>>>(x, v_hat, score, v_new, pos, N,
                                                               dsigma, eps, update_score);
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
