// Row operations on the active rows: LayerNorm (pre-norm of every sub-layer),
// gather + embed of the active latents (the active rows enter the model,
// section 2.2 item 1) and final LayerNorm + unembed to the velocity.
// All three are bandwidth-bound; one 64-wide wavefront per row with float4
// accesses.  LayerNorm keeps the row in registers when D is a multiple of
// 256 (one read of the row from memory, statistics in float32 from the
// registers); otherwise, and in unembed, the statistics take two passes.
// LayerNorm and unembed optionally apply the timestep modulation
// LN(h) (1 + scale) + shift (MOD template flag; shift and scale are [D]
// vectors read as float4 from L2, the same for every row).
#include "common.h"

namespace hsa {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 wavefronts of 64 lanes

__device__ __forceinline__ void row_stats(const f32x4* hr, int nv, int lane, int D, float& mean,
                                          float& rstd) {
  float s = 0.f;
  for (int i = lane; i < nv; i += kWave) {
    const f32x4 v = hr[i];
    s += (v[0] + v[1]) + (v[2] + v[3]);
  }
  mean = wave_sum(s) / (float)D;
  float q = 0.f;
  for (int i = lane; i < nv; i += kWave) {
    const f32x4 v = hr[i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float d = v[c] - mean;
      q += d * d;
    }
  }
  const float var = wave_sum(q) / (float)D;
  rstd = 1.0f / sqrtf(var + kLnEps);
}

template <typename OutT>
__device__ __forceinline__ void store4(OutT* p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, f32x4 v) {
  bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4*>(p) = b;
}

// n (1 + scale) + shift on the float4 chunk at column 4*i.
template <bool MOD>
__device__ __forceinline__ f32x4 modulate4(f32x4 n, const ModVec& shift, const ModVec& scale,
                                           int32_t i) {
  if constexpr (MOD) {
    const f32x4 sh = load_mod4(shift, 4 * i);
    const f32x4 sc = load_mod4(scale, 4 * i);
#pragma unroll
    for (int c = 0; c < 4; ++c) n[c] = __builtin_fmaf(n[c], 1.0f + sc[c], sh[c]);
  }
  return n;
}

template <typename OutT, bool MOD>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ h,
                                                        OutT* __restrict__ out, int32_t rows,
                                                        int32_t D, ModVec shift, ModVec scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;
  const int nv = D / 4;
  const f32x4* hr = reinterpret_cast<const f32x4*>(h + (size_t)row * D);
  float mean, rstd;
  row_stats(hr, nv, lane, D, mean, rstd);
  OutT* orow = out + (size_t)row * D;
  for (int i = lane; i < nv; i += kWave) {
    f32x4 v = hr[i];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = (v[c] - mean) * rstd;
    store4<OutT>(orow + 4 * i, modulate4<MOD>(v, shift, scale, i));
  }
}

// Row in registers: lane l holds float4 chunks l, l+64, ..., l+64(NV-1).
// With MOD the block first combines shift and scale (base + add) once into
// LDS, so the four rows of the block read them from there.
template <typename OutT, int NV, bool MOD>
__global__ __launch_bounds__(256) void layernorm_reg_kernel(const float* __restrict__ h,
                                                            OutT* __restrict__ out, int32_t rows,
                                                            int32_t D, ModVec shift,
                                                            ModVec scale) {
  __shared__ f32x4 s_mod[MOD ? 2 * NV * kWave : 1];   // shift chunks, then scale chunks
  if constexpr (MOD) {
    for (int i = threadIdx.x; i < NV * kWave; i += kRowsPerBlock * kWave) {
      s_mod[i] = load_mod4(shift, 4 * i);
      s_mod[NV * kWave + i] = load_mod4(scale, 4 * i);
    }
    __syncthreads();
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;
  const f32x4* hr = reinterpret_cast<const f32x4*>(h + (size_t)row * D);
  f32x4 v[NV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = hr[lane + kWave * i];
    s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  }
  const float mean = wave_sum(s) / (float)D;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float d = v[i][c] - mean;
      q += d * d;
    }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)D + kLnEps);
  OutT* orow = out + (size_t)row * D;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    f32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = (v[i][c] - mean) * rstd;
    const int32_t c4 = lane + kWave * i;
    if constexpr (MOD) {
      const f32x4 sh = s_mod[c4], sc = s_mod[NV * kWave + c4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = __builtin_fmaf(o[c], 1.0f + sc[c], sh[c]);
    }
    store4<OutT>(orow + 4 * c4, o);
  }
}

template <typename OutT, bool MOD>
bool launch_layernorm_reg(const float* h, OutT* out, int32_t rows, int32_t D, int blocks,
                          ModVec shift, ModVec scale, hipStream_t s) {
  if (D % (4 * kWave) != 0) return false;
  switch (D / (4 * kWave)) {
#define HSA_LN_CASE(nv)                                                                  \
    case nv:                                                                             \
      layernorm_reg_kernel<OutT, nv, MOD><<<blocks, 256, 0, s>>>(h, out, rows, D, shift, \
                                                                 scale);                 \
      return true;
    HSA_LN_CASE(1) HSA_LN_CASE(2) HSA_LN_CASE(3) HSA_LN_CASE(4) HSA_LN_CASE(5) HSA_LN_CASE(6)
    HSA_LN_CASE(8) HSA_LN_CASE(10) HSA_LN_CASE(12) HSA_LN_CASE(16) HSA_LN_CASE(20) HSA_LN_CASE(24)
#undef HSA_LN_CASE
    default: return false;
  }
}

// h[j][d] = sum_c x[idx[j]][c] * w_in[d][c]
template <typename WT>
__global__ __launch_bounds__(256) void embed_kernel(const float* __restrict__ x,
                                                    const int32_t* __restrict__ idx,
                                                    const WT* __restrict__ w_in,
                                                    float* __restrict__ h, int32_t rows, int32_t C,
                                                    int32_t D) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rows * D) return;
  const int32_t j = (int32_t)(t / D), d = (int32_t)(t % D);
  const float* xr = x + (size_t)idx[j] * C;
  const WT* wr = w_in + (size_t)d * C;
  float acc = 0.f;
  for (int c = 0; c < C; ++c) acc = __builtin_fmaf(xr[c], to_f32(wr[c]), acc);
  h[t] = acc;
}

// C == 16: each lane produces 4 consecutive outputs of one row from the
// latent row (4 x float4, shared by the row's lanes through the cache) and
// four 16-channel weight rows, so the pass is a handful of vector loads per
// output quad instead of 32 scalar loads per output.
template <typename WT>
__global__ __launch_bounds__(256) void embed_kernel_c16(const float* __restrict__ x,
                                                        const int32_t* __restrict__ idx,
                                                        const WT* __restrict__ w_in,
                                                        float* __restrict__ h, int32_t rows,
                                                        int32_t D) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t quads = D / 4;
  if (t >= (int64_t)rows * quads) return;
  const int32_t j = (int32_t)(t / quads), d0 = (int32_t)(t % quads) * 4;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + (size_t)idx[j] * 16);
  float xv[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 v = xr[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) xv[4 * i + e] = v[e];
  }
  f32x4 out;
#pragma unroll
  for (int o = 0; o < 4; ++o) {
    const WT* wr = w_in + (size_t)(d0 + o) * 16;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc = __builtin_fmaf(xv[c], to_f32(wr[c]), acc);
    out[o] = acc;
  }
  *reinterpret_cast<f32x4*>(h + (size_t)j * D + d0) = out;
}

// v_new[j][c] = sum_d LN(h[j])[d] * w_out[c][d], C == CC known at compile time.
template <typename WT, int CC, bool MOD>
__global__ __launch_bounds__(256) void unembed_kernel(const float* __restrict__ h,
                                                      const WT* __restrict__ w_out,
                                                      float* __restrict__ v_new, int32_t rows,
                                                      int32_t D, ModVec shift, ModVec scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;
  const int nv = D / 4;
  const f32x4* hr = reinterpret_cast<const f32x4*>(h + (size_t)row * D);
  float mean, rstd;
  row_stats(hr, nv, lane, D, mean, rstd);
  float acc[CC];
#pragma unroll
  for (int c = 0; c < CC; ++c) acc[c] = 0.f;
  for (int i = lane; i < nv; i += kWave) {
    f32x4 v = hr[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (v[e] - mean) * rstd;
    v = modulate4<MOD>(v, shift, scale, i);
#pragma unroll
    for (int c = 0; c < CC; ++c) {
      const WT* w = w_out + (size_t)c * D + 4 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[c] = __builtin_fmaf(v[e], to_f32(w[e]), acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < CC; ++c) acc[c] = wave_sum(acc[c]);
  if (lane < CC) {
    float mine = 0.f;
#pragma unroll
    for (int c = 0; c < CC; ++c) mine = (lane == c) ? acc[c] : mine;
    v_new[(size_t)row * CC + lane] = mine;
  }
}

// Any C: one wave reduction per output channel.
template <typename WT, bool MOD>
__global__ __launch_bounds__(256) void unembed_kernel_any(const float* __restrict__ h,
                                                          const WT* __restrict__ w_out,
                                                          float* __restrict__ v_new, int32_t rows,
                                                          int32_t D, int32_t C, ModVec shift,
                                                          ModVec scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;
  const int nv = D / 4;
  const f32x4* hr = reinterpret_cast<const f32x4*>(h + (size_t)row * D);
  float mean, rstd;
  row_stats(hr, nv, lane, D, mean, rstd);
  for (int c = 0; c < C; ++c) {
    float acc = 0.f;
    for (int i = lane; i < nv; i += kWave) {
      f32x4 v = hr[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (v[e] - mean) * rstd;
      v = modulate4<MOD>(v, shift, scale, i);
      const WT* w = w_out + (size_t)c * D + 4 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(v[e], to_f32(w[e]), acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) v_new[(size_t)row * C + c] = acc;
  }
}

template <bool MOD>
void layernorm_dispatch(const float* h, void* out, int32_t rows, int32_t D, hsa_dtype dt,
                        ModVec shift, ModVec scale, hipStream_t s) {
  const int blocks = cdiv(rows, kRowsPerBlock);
  if (dt == HSA_BF16) {
    if (!launch_layernorm_reg<bf16, MOD>(h, (bf16*)out, rows, D, blocks, shift, scale, s))
      layernorm_kernel<bf16, MOD><<<blocks, 256, 0, s>>>(h, (bf16*)out, rows, D, shift, scale);
  } else {
    if (!launch_layernorm_reg<float, MOD>(h, (float*)out, rows, D, blocks, shift, scale, s))
      layernorm_kernel<float, MOD><<<blocks, 256, 0, s>>>(h, (float*)out, rows, D, shift, scale);
  }
}

template <bool MOD>
void unembed_dispatch(const float* h, const void* w_out, float* v_new, int32_t rows, int32_t D,
                      int32_t C, hsa_dtype dt, ModVec shift, ModVec scale, hipStream_t s) {
  const int blocks = cdiv(rows, kRowsPerBlock);
  if (C == 16) {
    if (dt == HSA_BF16)
      unembed_kernel<bf16, 16, MOD><<<blocks, 256, 0, s>>>(h, (const bf16*)w_out, v_new, rows, D,
                                                           shift, scale);
    else
      unembed_kernel<float, 16, MOD><<<blocks, 256, 0, s>>>(h, (const float*)w_out, v_new, rows,
                                                            D, shift, scale);
  } else {
    if (dt == HSA_BF16)
      unembed_kernel_any<bf16, MOD><<<blocks, 256, 0, s>>>(h, (const bf16*)w_out, v_new, rows, D,
                                                           C, shift, scale);
    else
      unembed_kernel_any<float, MOD><<<blocks, 256, 0, s>>>(h, (const float*)w_out, v_new, rows,
                                                            D, C, shift, scale);
  }
}

}  // namespace

hsa_status launch_layernorm(const float* h, void* out, int32_t rows, int32_t D, hsa_dtype dt,
                            ModVec shift, ModVec scale, hipStream_t s) {
  if (rows == 0) return HSA_OK;
  if (shift.present() && scale.present())
    layernorm_dispatch<true>(h, out, rows, D, dt, shift, scale, s);
  else
    layernorm_dispatch<false>(h, out, rows, D, dt, shift, scale, s);
  return launch_status();
}

hsa_status launch_embed(const float* x, const int32_t* idx, const void* w_in, float* h,
                        int32_t rows, int32_t C, int32_t D, hsa_dtype dt, hipStream_t s) {
  if (rows == 0) return HSA_OK;
  if (C == 16 && D % 4 == 0) {
    const int64_t total = (int64_t)rows * (D / 4);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (dt == HSA_BF16)
      embed_kernel_c16<bf16><<<blocks, 256, 0, s>>>(x, idx, (const bf16*)w_in, h, rows, D);
    else
      embed_kernel_c16<float><<<blocks, 256, 0, s>>>(x, idx, (const float*)w_in, h, rows, D);
    return launch_status();
  }
  const int64_t total = (int64_t)rows * D;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dt == HSA_BF16)
    embed_kernel<bf16><<<blocks, 256, 0, s>>>(x, idx, (const bf16*)w_in, h, rows, C, D);
  else
    embed_kernel<float><<<blocks, 256, 0, s>>>(x, idx, (const float*)w_in, h, rows, C, D);
  return launch_status();
}

hsa_status launch_unembed(const float* h, const void* w_out, float* v_new, int32_t rows,
                          int32_t D, int32_t C, hsa_dtype dt, ModVec shift, ModVec scale,
                          hipStream_t s) {
  if (rows == 0) return HSA_OK;
  if (shift.present() && scale.present())
    unembed_dispatch<true>(h, w_out, v_new, rows, D, C, dt, shift, scale, s);
  else
    unembed_dispatch<false>(h, w_out, v_new, rows, D, C, dt, shift, scale, s);
  return launch_status();
}

}  // namespace hsa
