// Row operations on the active rows: LayerNorm (pre-norm of every sub-layer),
// gather + embed of the active latents (the active rows enter the model,
// section 2.2 item 1) and final LayerNorm + unembed to the velocity.
// All three are bandwidth-bound.  LayerNorm: one 64-wide wavefront per row
// with float4 accesses, the row kept in registers when D is a multiple of
// 256 (one read of the row from memory, statistics in float32 from the
// registers), two passes otherwise.  Embed keeps each thread's weights in
// registers across a block of rows, the columns spread so that every SIMD
// carries the same share of the FMAs; unembed (D <= 1536) runs the projection
// on the fp32 matrix cores over shifted rows, other widths keep w_out in LDS
// and a row per wavefront in registers (or two passes per row).
// LayerNorm and unembed optionally apply the timestep modulation
// LN(h) (1 + scale) + shift (MOD template flag; shift and scale are [D]
// vectors read as float4 from L2, the same for every row).
#include <type_traits>

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

// C == 16: a thread owns 4 consecutive output columns and keeps their 4 x 16
// weights in registers for every row of its block.  The block's latent rows
// x[idx[j]] are gathered into LDS first (one round of loads for the block),
// so the row loop is 64 FMAs and one 16-byte store per output quad.
constexpr int kEmbedRows = 32;     // rows per block
constexpr int kEmbedThreads = 128; // output quads per block
template <typename WT>
__global__ __launch_bounds__(kEmbedThreads) void embed_kernel_c16(const float* __restrict__ x,
                                                                  const int32_t* __restrict__ idx,
                                                                  const WT* __restrict__ w_in,
                                                                  float* __restrict__ h,
                                                                  int32_t rows, int32_t D) {
  __shared__ f32x4 sx[kEmbedRows][4];
  const int32_t r0 = blockIdx.x * kEmbedRows;
  const int32_t nr = min(rows - r0, kEmbedRows);
  {
    const int t = threadIdx.x;   // 128 threads: row t/4, chunk t%4
    if (t / 4 < nr)
      sx[t / 4][t % 4] = reinterpret_cast<const f32x4*>(x + (size_t)idx[r0 + t / 4] * 16)[t % 4];
  }
  const int32_t q = blockIdx.y * kEmbedThreads + threadIdx.x;   // columns 4q .. 4q+3
  const bool col_ok = 4 * q < D;
  float w[4][16];
#pragma unroll
  for (int o = 0; o < 4; ++o)
#pragma unroll
    for (int c = 0; c < 16; ++c) w[o][c] = 0.f;
  if (col_ok) {
    // the 4 weight rows are 64 consecutive values: 16-byte loads
    constexpr int kPer = 16 / (int)sizeof(WT);
    const u32x4* wr = reinterpret_cast<const u32x4*>(w_in + (size_t)4 * q * 16);
#pragma unroll
    for (int i = 0; i < 64 / kPer; ++i) {
      const u32x4 raw = wr[i];
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int f = i * kPer + e;
        if constexpr (sizeof(WT) == 2) {
          const uint32_t word = raw[e >> 1];
          w[f >> 4][f & 15] = __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
        } else {
          w[f >> 4][f & 15] = __uint_as_float(raw[e]);
        }
      }
    }
  }
  __syncthreads();
  if (!col_ok) return;
  for (int32_t j = 0; j < nr; ++j) {
    float xv[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = sx[j][i];
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[4 * i + e] = v[e];
    }
    f32x4 out;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc = __builtin_fmaf(xv[c], w[o][c], acc);
      out[o] = acc;
    }
    *reinterpret_cast<f32x4*>(h + (size_t)(r0 + j) * D + 4 * q) = out;
  }
}

// C == 16, D == 512 P: a block of 256 threads takes kEmbedPairRows rows over
// all D columns; thread t owns the column pairs t + 256 p (p < P) and keeps
// their 2 x 16 weights in registers, so each of the chip's SIMDs issues the
// same share of the 16 D FMAs per row (D / 4 threads per row would leave half
// the SIMDs with a second wavefront at D = 1536); 8-byte stores, 512
// contiguous bytes per wavefront and store.
constexpr int kEmbedPairRows = 16;
template <typename WT, int P>
__global__ __launch_bounds__(256) void embed_pairs_kernel(const float* __restrict__ x,
                                                          const int32_t* __restrict__ idx,
                                                          const WT* __restrict__ w_in,
                                                          float* __restrict__ h, int32_t rows) {
  constexpr int D = 512 * P;
  __shared__ f32x4 sx[kEmbedPairRows][4];
  const int32_t r0 = blockIdx.x * kEmbedPairRows;
  const int32_t nr = min(rows - r0, kEmbedPairRows);
  const int t = threadIdx.x;
  const bool gx = t < 4 * nr;   // thread t gathers chunk t % 4 of row t / 4
  const int32_t src = gx ? idx[r0 + t / 4] : 0;
  float w[2 * P][16];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    // rows 2q, 2q + 1 of w_in (q = t + 256 p): 32 consecutive values
    constexpr int kPer = 16 / (int)sizeof(WT);
    const u32x4* wr = reinterpret_cast<const u32x4*>(w_in + (size_t)(t + 256 * p) * 32);
#pragma unroll
    for (int i = 0; i < 32 / kPer; ++i) {
      const u32x4 raw = wr[i];
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int f = i * kPer + e;
        if constexpr (sizeof(WT) == 2) {
          const uint32_t word = raw[e >> 1];
          w[2 * p + (f >> 4)][f & 15] = __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
        } else {
          w[2 * p + (f >> 4)][f & 15] = __uint_as_float(raw[e]);
        }
      }
    }
  }
  if (gx) sx[t / 4][t % 4] = reinterpret_cast<const f32x4*>(x + (size_t)src * 16)[t % 4];
  __syncthreads();
  for (int32_t j = 0; j < nr; ++j) {
    float xv[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = sx[j][i];
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[4 * i + e] = v[e];
    }
    float* hr = h + (size_t)(r0 + j) * D + 2 * t;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      f32x2 out;
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc = __builtin_fmaf(xv[c], w[2 * p + o][c], acc);
        out[o] = acc;
      }
      *reinterpret_cast<f32x2*>(hr + 512 * p) = out;
    }
  }
}

template <int O, int HALF>
__device__ __forceinline__ void reduce_halve(float (&a)[16], int lane) {
  const bool hi = (lane & O) != 0;
#pragma unroll
  for (int c = 0; c < HALF; ++c) {
    const float keep = hi ? a[c + HALF] : a[c];
    const float send = hi ? a[c] : a[c + HALF];
    a[c] = keep + __shfl_xor(send, O, kWave);
  }
}
__device__ __forceinline__ float reduce16(float (&a)[16], int lane) {
  reduce_halve<32, 8>(a, lane);
  reduce_halve<16, 4>(a, lane);
  reduce_halve<8, 2>(a, lane);
  reduce_halve<4, 1>(a, lane);
  float t = a[0];
  t += __shfl_xor(t, 2, kWave);
  t += __shfl_xor(t, 1, kWave);
  return t;
}

// C == 16, D = 256 NV: the block copies w_out [16][D] into LDS once (as
// float32, so the FMAs read it without conversions; D <= 2048); each
// of its 8 wavefronts then takes rows one at a time, held in registers (lane
// l: float4 chunks l, l+64, ...) with the next row's load in flight:
// statistics, normalisation and modulation there, the 16 dot products
// against the LDS weights, reduced with reduce16.
constexpr int kUnembedRows = 32;     // rows per block
constexpr int kUnembedWaves = 8;
template <typename WT, int NV, bool MOD>
__global__ __launch_bounds__(kUnembedWaves * kWave) void unembed_c16_reg_kernel(
    const float* __restrict__ h, const WT* __restrict__ w_out, float* __restrict__ v_new,
    int32_t rows, ModVec shift, ModVec scale) {
  constexpr int D = NV * 4 * kWave;
  __shared__ __attribute__((aligned(16))) float sw[16 * D];   // w_out as float32
  {
    // every 16-byte load of the weights issued before the first conversion
    constexpr int kPer = 16 / (int)sizeof(WT);                  // weights per load
    constexpr int kThreads = kUnembedWaves * kWave;
    constexpr int kLoads = (16 * D / kPer + kThreads - 1) / kThreads;
    const u32x4* src = reinterpret_cast<const u32x4*>(w_out);
    u32x4 raw[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int i = threadIdx.x + k * kThreads;
      if (i < 16 * D / kPer) raw[k] = src[i];
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int i = threadIdx.x + k * kThreads;
      if (i < 16 * D / kPer) {
        if constexpr (sizeof(WT) == 2) {
          f32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            lo[2 * e] = __uint_as_float(raw[k][e] << 16);
            lo[2 * e + 1] = __uint_as_float(raw[k][e] & 0xffff0000u);
            hi[2 * e] = __uint_as_float(raw[k][2 + e] << 16);
            hi[2 * e + 1] = __uint_as_float(raw[k][2 + e] & 0xffff0000u);
          }
          reinterpret_cast<f32x4*>(sw)[2 * i] = lo;
          reinterpret_cast<f32x4*>(sw)[2 * i + 1] = hi;
        } else {
          reinterpret_cast<u32x4*>(sw)[i] = raw[k];
        }
      }
    }
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int32_t r1 = min(rows, (int32_t)(blockIdx.x + 1) * kUnembedRows);
  int32_t row = blockIdx.x * kUnembedRows + wave;
  f32x4 nxt[NV];
  auto load_row = [&](int32_t r) {
    const f32x4* hr = reinterpret_cast<const f32x4*>(h + (size_t)r * D);
#pragma unroll
    for (int i = 0; i < NV; ++i) nxt[i] = hr[lane + kWave * i];
  };
  if (row < r1) load_row(row);
  __syncthreads();
  for (; row < r1; row += kUnembedWaves) {
    f32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = nxt[i];
    if (row + kUnembedWaves < r1) load_row(row + kUnembedWaves);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
    const float mean = wave_sum(s) / (float)D;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = v[i][e] - mean;
        q += d * d;
      }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)D + kLnEps);
    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.f;
    // A real loop over the row's chunks (v rotated down one chunk per pass),
    // so that the compiler issues one chunk's 16 weight reads at a time
    // instead of hoisting all of them.
#pragma unroll 1
    for (int i = 0; i < NV; ++i) {
      const int col = 4 * (lane + kWave * i);
      f32x4 n;
#pragma unroll
      for (int e = 0; e < 4; ++e) n[e] = (v[0][e] - mean) * rstd;
#pragma unroll
      for (int k = 0; k + 1 < NV; ++k) v[k] = v[k + 1];
      n = modulate4<MOD>(n, shift, scale, lane + kWave * i);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(sw + c * D + col);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[c] = __builtin_fmaf(n[e], w[e], acc[c]);
      }
    }
    const float sum = reduce16(acc, lane);
    if ((lane & 3) == 0) v_new[(size_t)row * 16 + ((lane >> 2) & 15)] = sum;
  }
}

// C == 16, D = 128 G (G even, D <= 1536), on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: D[16x16] += A[16x4] B[4x16]; lane l holds
// A[l%16][l/16], B[l/16][l%16] and D[4(l/16)+m][l%16], m = 0..3).  With
// K = h[r][0], mean - K = S1/D, S1 = sum(h - K), var = S2/D - (S1/D)^2,
// S2 = sum((h - K)^2) (shifted sums: no cancellation for rows far from 0),
// and w' = w (1 + scale):
//   v[r][c] = rstd_r (sum_d (h[r][d] - K) w'[c][d] - (S1/D) sum_d w'[c][d])
//             + sum_d shift_d w[c][d],
// the first sum on the matrix cores over (h - K), which also feeds S1 and S2.
// A block takes 32 rows: two 16-row tiles, each split over the two halves
// of D between two wavefronts (one per SIMD), whose partials meet in LDS.
// Step (e, t) of group g takes d = half + 64 g + 16 e + 4 (l/16) + t on both
// operands: one load instruction reads 64 contiguous bytes of each of 16 rows.
constexpr int kUnMmRows = 32;
template <typename WT, int G, bool MOD>
__global__ __launch_bounds__(256) void unembed_mfma_kernel(const float* __restrict__ h,
                                                           const WT* __restrict__ w_out,
                                                           float* __restrict__ v_new, int32_t rows,
                                                           ModVec shift, ModVec scale) {
  constexpr int D = 128 * G, DP = D + 4;   // LDS row pitch: the 16 weight rows on distinct banks
  __shared__ __attribute__((aligned(16))) float um_smem[16 * DP + 32 + 2 * 64 * 4 + 2 * 16 * 2 * 2];
  float* ws = um_smem;              // w' [16][DP]
  float* wsum = ws + 16 * DP;       // sum_d w'[c][d]
  float* bsum = wsum + 16;          // sum_d shift_d w[c][d]
  float* xacc = bsum + 16;          // [2 tiles][64 lanes][4]: the second half's partial products
  float* xst = xacc + 2 * 64 * 4;   // [2 tiles][16 rows][2]: its S1, S2
  float* st = xst + 2 * 16 * 2;     // [2 tiles][16 rows][2]: S1/D and rstd
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int tile = wave >> 1, kh = wave & 1;
  const int i = lane & 15, q = lane >> 4;
  const int32_t r0 = blockIdx.x * kUnMmRows + tile * 16;
  const float* hr = h + (size_t)min(r0 + i, rows - 1) * D;   // rows past the end: a copy, not stored
  // ---- the weights' loads first (L2-resident), then the first row loads of
  // this half: loads return in order, so the weights' conversion below waits
  // for its own loads only, while the rows stream in behind them
  // thread t: weight row c = t / 16, 16-byte chunks (t % 16) + 16 j
  const int c = tid >> 4;
  constexpr int kPer = 16 / (int)sizeof(WT);   // weights per 16-byte load
  constexpr int kChunks = D / kPer / 16;        // per thread
  u32x4 wraw[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j)
    wraw[j] = *reinterpret_cast<const u32x4*>(w_out + (size_t)c * D + kPer * ((tid & 15) + 16 * j));
  // the rows stream through a ring of LA groups (4 loads each): a wavefront
  // issues in order, so with every load of the half issued up front the
  // matrix-core chain could not start before the last load had been accepted
  // by the memory pipeline, and ran after the data instead of beside it
  const float K = hr[0];
  f32x4 hv[G][4];
  constexpr int LA = G < 4 ? G : 4;
  auto load_group = [&](int g) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      hv[g][e] = *reinterpret_cast<const f32x4*>(hr + kh * (D / 2) + 64 * g + 16 * e + 4 * q);
  };
#pragma unroll
  for (int g = 0; g < LA; ++g) load_group(g);
  {
    float ps = 0.f, pb = 0.f;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int d0 = kPer * ((tid & 15) + 16 * j);
      const u32x4 raw = wraw[j];
      float w[kPer];
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if constexpr (sizeof(WT) == 2)
          w[e] = __uint_as_float((e & 1) ? (raw[e >> 1] & 0xffff0000u) : (raw[e >> 1] << 16));
        else
          w[e] = __uint_as_float(raw[e]);
      }
#pragma unroll
      for (int e4 = 0; e4 < kPer; e4 += 4) {
        f32x4 o;
        if constexpr (MOD) {
          const f32x4 sh = load_mod4(shift, d0 + e4);
          const f32x4 sc = load_mod4(scale, d0 + e4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = w[e4 + e] * (1.0f + sc[e]);
            pb = __builtin_fmaf(sh[e], w[e4 + e], pb);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = w[e4 + e];
        }
        ps += (o[0] + o[1]) + (o[2] + o[3]);
        *reinterpret_cast<f32x4*>(ws + c * DP + d0 + e4) = o;
      }
    }
    // the 16 threads of row c are 16 consecutive lanes
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      ps += __shfl_xor(ps, o, kWave);
      pb += __shfl_xor(pb, o, kWave);
    }
    if ((tid & 15) == 0) {
      wsum[c] = ps;
      bsum[c] = pb;
    }
  }
  __syncthreads();
  // ---- this half's products and shifted sums
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float s1 = 0.f, s2 = 0.f;
  const float* wrow = ws + i * DP + kh * (D / 2) + 4 * q;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g + LA < G) load_group(g + LA);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 64 * g + 16 * e);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = hv[g][e][t] - K;
        s1 += a;
        s2 = __builtin_fmaf(a, a, s2);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, w4[t], acc, 0, 0, 0);
      }
    }
    if (LA < G) __builtin_amdgcn_sched_barrier(0);
  }
  // a row's sums over its four lanes (i, i + 16, i + 32, i + 48)
  s1 += __shfl_xor(s1, 16, kWave);
  s2 += __shfl_xor(s2, 16, kWave);
  s1 += __shfl_xor(s1, 32, kWave);
  s2 += __shfl_xor(s2, 32, kWave);
  if (kh == 1) {
    *reinterpret_cast<f32x4*>(xacc + (tile * 64 + lane) * 4) = acc;
    if (q == 0) {
      xst[(tile * 16 + i) * 2] = s1;
      xst[(tile * 16 + i) * 2 + 1] = s2;
    }
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const f32x4 o = *reinterpret_cast<const f32x4*>(xacc + (tile * 64 + lane) * 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] += o[m];
    if (q == 0) {
      s1 += xst[(tile * 16 + i) * 2];
      s2 += xst[(tile * 16 + i) * 2 + 1];
      const float mk = s1 / (float)D;                 // mean - K
      const float var = fmaxf(s2 / (float)D - mk * mk, 0.f);
      st[(tile * 16 + i) * 2] = mk;
      st[(tile * 16 + i) * 2 + 1] = 1.0f / sqrtf(var + kLnEps);
    }
  }
  // (LDS operations of one wavefront complete in order: no barrier)
  const float wc = wsum[i], bc = MOD ? bsum[i] : 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int rr = 4 * q + m;
    const float mk = st[(tile * 16 + rr) * 2], rs = st[(tile * 16 + rr) * 2 + 1];
    if (r0 + rr < rows) v_new[(size_t)(r0 + rr) * 16 + i] = rs * (acc[m] - mk * wc) + bc;
  }
}

template <typename WT, bool MOD>
bool launch_unembed_mfma(const float* h, const WT* w_out, float* v_new, int32_t rows, int32_t D,
                         ModVec shift, ModVec scale, hipStream_t s) {
  if (D % 256 != 0 || D > 1536) return false;   // wider: the row loads would not fit the registers
  const unsigned blocks = (unsigned)cdiv(rows, kUnMmRows);
  auto launch = [&](auto g) {
    constexpr int G = decltype(g)::value;
    unembed_mfma_kernel<WT, G, MOD><<<blocks, 256, 0, s>>>(h, w_out, v_new, rows, shift, scale);
  };
  switch (D / 128) {
    case 2: launch(std::integral_constant<int, 2>{}); break;
    case 4: launch(std::integral_constant<int, 4>{}); break;
    case 6: launch(std::integral_constant<int, 6>{}); break;
    case 8: launch(std::integral_constant<int, 8>{}); break;
    case 10: launch(std::integral_constant<int, 10>{}); break;
    default: launch(std::integral_constant<int, 12>{}); break;
  }
  return true;
}

template <typename WT, bool MOD>
bool launch_unembed_reg(const float* h, const WT* w_out, float* v_new, int32_t rows, int32_t D,
                        ModVec shift, ModVec scale, hipStream_t s) {
  if (D % (4 * kWave) != 0 || 16 * D * (int64_t)sizeof(float) > 128 * 1024) return false;
  const unsigned blocks = (unsigned)cdiv(rows, kUnembedRows);
  const int nv = D / (4 * kWave);
  if (nv < 1 || nv > 8) return false;
  auto launch = [&](auto nv_const) {
    unembed_c16_reg_kernel<WT, decltype(nv_const)::value, MOD>
        <<<blocks, kUnembedWaves * kWave, 0, s>>>(h, w_out, v_new, rows, shift, scale);
  };
  switch (nv) {
    case 1: launch(std::integral_constant<int, 1>{}); break;
    case 2: launch(std::integral_constant<int, 2>{}); break;
    case 3: launch(std::integral_constant<int, 3>{}); break;
    case 4: launch(std::integral_constant<int, 4>{}); break;
    case 5: launch(std::integral_constant<int, 5>{}); break;
    case 6: launch(std::integral_constant<int, 6>{}); break;
    case 7: launch(std::integral_constant<int, 7>{}); break;
    default: launch(std::integral_constant<int, 8>{}); break;
  }
  return true;
}

// Sum of v[0..15] over the wavefront, reduced and scattered: lane L returns the
// total of channel ((L >> 2) & 15) (four lanes hold each), in 17 exchanges
// instead of 16 full reductions: each halving step keeps the half of the
// channels that the lane's next address bit selects.
__device__ __forceinline__ float wave_sum16_scatter(const float (&v)[16]) {
  const int lane = threadIdx.x & (kWave - 1);
  float a[8];
  {
    const bool hi = (lane >> 5) & 1;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float keep = hi ? v[8 + k] : v[k], give = hi ? v[k] : v[8 + k];
      a[k] = keep + __shfl_xor(give, 32, kWave);
    }
  }
  float b[4];
  {
    const bool hi = (lane >> 4) & 1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float keep = hi ? a[4 + k] : a[k], give = hi ? a[k] : a[4 + k];
      b[k] = keep + __shfl_xor(give, 16, kWave);
    }
  }
  float c2[2];
  {
    const bool hi = (lane >> 3) & 1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float keep = hi ? b[2 + k] : b[k], give = hi ? b[k] : b[2 + k];
      c2[k] = keep + __shfl_xor(give, 8, kWave);
    }
  }
  float d;
  {
    const bool hi = (lane >> 2) & 1;
    const float keep = hi ? c2[1] : c2[0], give = hi ? c2[0] : c2[1];
    d = keep + __shfl_xor(give, 4, kWave);
  }
  d += __shfl_xor(d, 2, kWave);
  d += __shfl_xor(d, 1, kWave);
  return d;
}

// Channel held by lane L after wave_sum16_scatter: lane bits 5..2, as the
// halving steps on lane bits 5, 4, 3, 2 chose channel bits 3, 2, 1, 0.
__device__ __forceinline__ int scatter_channel(int lane) { return (lane >> 2) & 15; }

// C = 16, wide rows (D % 256 == 0, weights too large for the LDS forms): one
// pass over each row.  A wavefront takes kWideRows rows, so each weight load
// from the cache feeds that many rows.  With K = h[r][0], a = (h - K)(1 + scale)
// (a = h - K unmodulated), S1 = sum (h - K), S2 = sum (h - K)^2:
// v[r][c] = rstd (sum_d a w[c] - (S1 / D) sum_d (1 + scale) w[c]) + sum_d shift w[c],
// rstd = 1 / sqrt(S2 / D - (S1 / D)^2 + eps).  Rows far from zero lose nothing to
// cancellation since the sums are shifted by a value of the row.
constexpr int kWideRows = 4;
template <typename WT, bool MOD>
__global__ __launch_bounds__(256) void unembed_c16_wide_kernel(const float* __restrict__ h,
                                                               const WT* __restrict__ w_out,
                                                               float* __restrict__ v_new,
                                                               int32_t rows, int32_t D,
                                                               ModVec shift, ModVec scale) {
  constexpr int R = kWideRows;
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t r0 = (blockIdx.x * (256 / kWave) + threadIdx.x / kWave) * R;
  if (r0 >= rows) return;
  const int nr = min(R, rows - r0);
  const f32x4* hr[R];
  float K[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {   // rows past the end repeat the last one (not stored)
    hr[r] = reinterpret_cast<const f32x4*>(h + (size_t)(r0 + min(r, nr - 1)) * D);
    K[r] = h[(size_t)(r0 + min(r, nr - 1)) * D];
  }
  float acc[R][16], s1[R], s2[R], ws[16], bs[16];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    s1[r] = 0.f;
    s2[r] = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[r][c] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    ws[c] = 0.f;
    bs[c] = 0.f;
  }
  // Every load of a chunk is issued before any of its arithmetic (the rows'
  // chunks and sixteen weight loads in flight together): issued one at a time
  // with a wait each, the loads of a chunk would be a chain of cache round
  // trips.
  typedef typename std::conditional<sizeof(WT) == 2, u32x2, f32x4>::type WRaw;
  const int nv = D / 4;
  // a modulation vector's optional second term: read from the first when absent, weighted 0
  const float* sc_add = MOD && scale.add ? scale.add : scale.base;
  const float* sh_add = MOD && shift.add ? shift.add : shift.base;
  const float sc_on = MOD && scale.add ? 1.f : 0.f, sh_on = MOD && shift.add ? 1.f : 0.f;
  for (int i = lane; i < nv; i += kWave) {
    f32x4 hv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) hv[r] = hr[r][i];
    WRaw wr[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) wr[c] = *reinterpret_cast<const WRaw*>(w_out + (size_t)c * D + 4 * i);
    f32x4 g = {1.f, 1.f, 1.f, 1.f}, sh = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MOD) {   // base + (add or nothing), with no branch in the loop
      const f32x4 sc0 = *reinterpret_cast<const f32x4*>(scale.base + 4 * i);
      const f32x4 sc1 = *reinterpret_cast<const f32x4*>(sc_add + 4 * i);
      const f32x4 sh0 = *reinterpret_cast<const f32x4*>(shift.base + 4 * i);
      const f32x4 sh1 = *reinterpret_cast<const f32x4*>(sh_add + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[e] = 1.0f + __builtin_fmaf(sc_on, sc1[e], sc0[e]);
        sh[e] = __builtin_fmaf(sh_on, sh1[e], sh0[e]);
      }
    }
    f32x4 a[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = hv[r][e] - K[r];
        s1[r] += d;
        s2[r] = __builtin_fmaf(d, d, s2[r]);
        a[r][e] = MOD ? d * g[e] : d;
      }
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      f32x4 w;
      if constexpr (sizeof(WT) == 2) {
        w[0] = __uint_as_float(wr[c][0] << 16);
        w[1] = __uint_as_float(wr[c][0] & 0xffff0000u);
        w[2] = __uint_as_float(wr[c][1] << 16);
        w[3] = __uint_as_float(wr[c][1] & 0xffff0000u);
      } else {
        w = wr[c];
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r][c] = __builtin_fmaf(a[r][e], w[e], acc[r][c]);
      if constexpr (MOD) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ws[c] = __builtin_fmaf(g[e], w[e], ws[c]);
          bs[c] = __builtin_fmaf(sh[e], w[e], bs[c]);
        }
      } else {
        ws[c] += (w[0] + w[1]) + (w[2] + w[3]);
      }
    }
  }
  const int ch = scatter_channel(lane);
  const float wsum = wave_sum16_scatter(ws);
  const float bsum = MOD ? wave_sum16_scatter(bs) : 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float dot = wave_sum16_scatter(acc[r]);
    const float t1 = wave_sum(s1[r]), t2 = wave_sum(s2[r]);
    const float mk = t1 / (float)D;                           // mean - K
    const float var = fmaxf(t2 / (float)D - mk * mk, 0.f);
    const float rstd = 1.0f / sqrtf(var + kLnEps);
    if (r < nr && (lane & 3) == 0) v_new[(size_t)(r0 + r) * 16 + ch] = rstd * (dot - mk * wsum) + bsum;
  }
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
    if (dt == HSA_BF16 ? launch_unembed_mfma<bf16, MOD>(h, (const bf16*)w_out, v_new, rows, D, shift,
                                                        scale, s)
                       : launch_unembed_mfma<float, MOD>(h, (const float*)w_out, v_new, rows, D,
                                                         shift, scale, s))
      return;
    if (dt == HSA_BF16 ? launch_unembed_reg<bf16, MOD>(h, (const bf16*)w_out, v_new, rows, D, shift,
                                                       scale, s)
                       : launch_unembed_reg<float, MOD>(h, (const float*)w_out, v_new, rows, D,
                                                        shift, scale, s))
      return;
    if (D % 256 == 0) {
      const unsigned wblocks = (unsigned)cdiv(rows, (256 / kWave) * kWideRows);
      if (dt == HSA_BF16)
        unembed_c16_wide_kernel<bf16, MOD><<<wblocks, 256, 0, s>>>(h, (const bf16*)w_out, v_new,
                                                                    rows, D, shift, scale);
      else
        unembed_c16_wide_kernel<float, MOD><<<wblocks, 256, 0, s>>>(h, (const float*)w_out, v_new,
                                                                     rows, D, shift, scale);
      return;
    }
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
  if (C == 16 && D % 512 == 0 && D <= 2048) {
    const unsigned grid = (unsigned)cdiv(rows, kEmbedPairRows);
#define HSA_EMBED_CASE(P)                                                                           \
  case P:                                                                                          \
    if (dt == HSA_BF16)                                                                            \
      embed_pairs_kernel<bf16, P><<<grid, 256, 0, s>>>(x, idx, (const bf16*)w_in, h, rows);        \
    else                                                                                           \
      embed_pairs_kernel<float, P><<<grid, 256, 0, s>>>(x, idx, (const float*)w_in, h, rows);      \
    return launch_status();
    switch (D / 512) {
      HSA_EMBED_CASE(1) HSA_EMBED_CASE(2) HSA_EMBED_CASE(3) HSA_EMBED_CASE(4)
    }
#undef HSA_EMBED_CASE
  }
  if (C == 16 && D % 4 == 0) {
    const dim3 grid((unsigned)cdiv(rows, kEmbedRows), (unsigned)cdiv(D / 4, kEmbedThreads));
    if (dt == HSA_BF16)
      embed_kernel_c16<bf16><<<grid, kEmbedThreads, 0, s>>>(x, idx, (const bf16*)w_in, h, rows, D);
    else
      embed_kernel_c16<float><<<grid, kEmbedThreads, 0, s>>>(x, idx, (const float*)w_in, h, rows, D);
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
