// Optional Wan-style block features.  The pages evaluate HSA on Wan-family
// DiTs ("Not All Tokens Need 40 Steps", section 4) without defining their
// layers; include/hsa.h states the definitions implemented here:
//  - qk-RMSNorm and 3D rotary position embedding, fused into one in-place
//    pass over the fresh q rows and the K-cache rows of the active tokens
//    (right after the QKV projection scattered them), so the cache holds
//    normalised, rotated keys and the attention kernel is unchanged;
//  - the timestep MLP of the adaLN modulation (three small float32 GEMVs per
//    iteration; the modulation itself is applied inside the LayerNorm and
//    residual-epilogue kernels);
//  - the classifier-free guidance combine of the two branch velocities.
// All three are bandwidth- or latency-bound: one 64-wide wavefront per row,
// 16-byte vector accesses.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace hsa {
namespace {

constexpr int kRows = 4;  // rows (wavefronts) per 256-thread block
constexpr float kRmsEps = 1e-6f;
constexpr double kLn10000 = 9.210340371976184;

// 16-byte chunk of a row: 4 float32 or 8 bf16 values.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int N = 4;
  typedef f32x4 V;
};
template <> struct Chunk<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 V;
};

// Normalise (NORM) and rotate (ROPE) one row in place: x / sqrt(mean(x^2) +
// eps) * gain over D, then pair (2i, 2i+1) of every head turned by the angle
// whose (cos, sin) the wave's table cs holds for pair i of a head.  A 16-byte
// chunk never straddles two heads (Dh % 8 == 0).
template <typename T, bool NORM, bool ROPE>
__device__ __forceinline__ void norm_rotate_row(T* __restrict__ row, const float* __restrict__ gain,
                                                const float2* __restrict__ cs, int32_t D,
                                                int32_t Dh, int lane) {
  constexpr int CN = Chunk<T>::N;
  typedef typename Chunk<T>::V V;
  const int nch = D / CN;
  float rs = 1.0f;
  if constexpr (NORM) {
    float ss = 0.f;
    for (int c = lane; c < nch; c += kWave) {
      const V v = reinterpret_cast<const V*>(row)[c];
#pragma unroll
      for (int e = 0; e < CN; ++e) {
        const float x = to_f32(v[e]);
        ss = __builtin_fmaf(x, x, ss);
      }
    }
    rs = 1.0f / sqrtf(wave_sum(ss) / (float)D + kRmsEps);
  }
  for (int c = lane; c < nch; c += kWave) {
    V v = reinterpret_cast<const V*>(row)[c];
    float x[CN];
#pragma unroll
    for (int e = 0; e < CN; ++e) x[e] = to_f32(v[e]);
    if constexpr (NORM) {
#pragma unroll
      for (int g4 = 0; g4 < CN / 4; ++g4) {
        const f32x4 g = reinterpret_cast<const f32x4*>(gain + (size_t)c * CN)[g4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * g4 + e] = x[4 * g4 + e] * rs * g[e];
      }
    }
    if constexpr (ROPE) {
      const int pair0 = ((c * CN) % Dh) / 2;
#pragma unroll
      for (int pr = 0; pr < CN / 2; ++pr) {
        const float2 t = cs[pair0 + pr];
        const float a = x[2 * pr], b = x[2 * pr + 1];
        x[2 * pr] = a * t.x - b * t.y;
        x[2 * pr + 1] = a * t.y + b * t.x;
      }
    }
#pragma unroll
    for (int e = 0; e < CN; ++e) v[e] = from_f32<T>(x[e]);
    reinterpret_cast<V*>(row)[c] = v;
  }
}

// Both rows of a token at once, held in registers: D = 64 NCH CN (NCH chunks of
// 16 bytes per lane).  Each row is read once (its sum of squares and its
// transform from the same registers), and the two rows' loads are in flight
// together: for wide rows, where the loop form's second pass over a row no
// longer finds it in the cache.
template <typename T, bool NORM, bool ROPE, int NCH>
__device__ __forceinline__ void norm_rotate_rows_reg(T* __restrict__ qrow, T* __restrict__ krow,
                                                     const float* __restrict__ q_gain,
                                                     const float* __restrict__ k_gain,
                                                     const float2* __restrict__ cs, int32_t D,
                                                     int32_t Dh, int lane) {
  constexpr int CN = Chunk<T>::N;
  typedef typename Chunk<T>::V V;
  V v[2][NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    v[0][i] = reinterpret_cast<const V*>(qrow)[lane + kWave * i];
    v[1][i] = reinterpret_cast<const V*>(krow)[lane + kWave * i];
  }
  float rs[2] = {1.0f, 1.0f};
  if constexpr (NORM) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < CN; ++e) {
          const float x = to_f32(v[w][i][e]);
          ss = __builtin_fmaf(x, x, ss);
        }
      rs[w] = 1.0f / sqrtf(wave_sum(ss) / (float)D + kRmsEps);
    }
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const float* gain = w == 0 ? q_gain : k_gain;
    T* row = w == 0 ? qrow : krow;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + kWave * i;
      float x[CN];
#pragma unroll
      for (int e = 0; e < CN; ++e) x[e] = to_f32(v[w][i][e]);
      if constexpr (NORM) {
#pragma unroll
        for (int g4 = 0; g4 < CN / 4; ++g4) {
          const f32x4 g = reinterpret_cast<const f32x4*>(gain + (size_t)c * CN)[g4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * g4 + e] = x[4 * g4 + e] * rs[w] * g[e];
        }
      }
      if constexpr (ROPE) {
        const int pair0 = ((c * CN) % Dh) / 2;
#pragma unroll
        for (int pr = 0; pr < CN / 2; ++pr) {
          const float2 t = cs[pair0 + pr];
          const float a = x[2 * pr], b = x[2 * pr + 1];
          x[2 * pr] = a * t.x - b * t.y;
          x[2 * pr + 1] = a * t.y + b * t.x;
        }
      }
      V o;
#pragma unroll
      for (int e = 0; e < CN; ++e) o[e] = from_f32<T>(x[e]);
      reinterpret_cast<V*>(row)[c] = o;
    }
  }
}

// One wavefront per active token j: its q row j and its K-cache row idx[j].
// The token's rotation (cos, sin) per pair of a head is evaluated once into
// the wave's LDS table (one pair per lane, precise sincosf) and shared by all
// heads of both rows.
template <typename T, bool NORM, bool ROPE, int NCH>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    T* __restrict__ q, T* __restrict__ kc, const int32_t* __restrict__ idx, int32_t rows,
    int32_t D, int32_t Dh, const float* __restrict__ q_gain, const float* __restrict__ k_gain,
    int32_t grid_h, int32_t grid_w) {
  __shared__ float2 s_cs[kRows][64];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int32_t j = blockIdx.x * kRows + wid;
  const bool valid = j < rows;
  const int32_t tok = valid ? idx[j] : 0;
  if constexpr (ROPE) {
    // pair `lane` of a head: its axis (frame, row, column section) and
    // frequency 10000^(-j'/p), evaluated in double and rounded once
    const int P = Dh / 2;
    if (lane < P) {
      const int p_hw = P / 3;
      const int p_f = P - 2 * p_hw;
      int32_t pos;
      int jp, p;
      if (lane < p_f) {
        pos = tok / (grid_h * grid_w), jp = lane, p = p_f;
      } else if (lane < p_f + p_hw) {
        pos = (tok / grid_w) % grid_h, jp = lane - p_f, p = p_hw;
      } else {
        pos = tok % grid_w, jp = lane - p_f - p_hw, p = p_hw;
      }
      const float freq = (float)exp(-(double)jp / (double)p * kLn10000);
      float sn, cs;
      sincosf((float)pos * freq, &sn, &cs);
      s_cs[wid][lane] = make_float2(cs, sn);
    }
    __syncthreads();
  }
  if (!valid) return;
  if constexpr (NCH > 0) {
    norm_rotate_rows_reg<T, NORM, ROPE, NCH>(q + (size_t)j * D, kc + (size_t)tok * D, q_gain, k_gain,
                                             s_cs[wid], D, Dh, lane);
  } else {
    norm_rotate_row<T, NORM, ROPE>(q + (size_t)j * D, q_gain, s_cs[wid], D, Dh, lane);
    norm_rotate_row<T, NORM, ROPE>(kc + (size_t)tok * D, k_gain, s_cs[wid], D, Dh, lane);
  }
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// e1[r] = silu(w1[r] . s + b1[r]) with s the 256-wide timestep sinusoid of
// t = 1000 sigma: s[k] = cos(t w_k), s[128 + k] = sin(t w_k), w_k =
// 10000^(-k/128), each evaluated in double precision and rounded once.
__global__ __launch_bounds__(256) void time_stage1_kernel(float sigma,
                                                          const float* __restrict__ w1,
                                                          const float* __restrict__ b1,
                                                          float* __restrict__ e1, int32_t D) {
  __shared__ float s_sin[256];
  const int tid = threadIdx.x;
  {
    const double t = 1000.0 * (double)sigma;
    const int k = tid & 127;
    const double a = t * exp(-(double)k / 128.0 * kLn10000);
    s_sin[tid] = (float)(tid < 128 ? cos(a) : sin(a));
  }
  __syncthreads();
  const int lane = tid & (kWave - 1);
  const int32_t r = blockIdx.x * kRows + tid / kWave;
  if (r >= D) return;
  const f32x4 w = reinterpret_cast<const f32x4*>(w1 + (size_t)r * 256)[lane];
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(w[e], s_sin[4 * lane + e], acc);
  acc = wave_sum(acc);
  if (lane == 0) e1[r] = silu(acc + b1[r]);
}

// y[r] = w[r] . act(x) + b[r], act = silu (IN_SILU) or identity; n_in % 4 == 0.
template <bool IN_SILU>
__global__ __launch_bounds__(256) void gemv_bias_kernel(const float* __restrict__ w,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ b,
                                                        float* __restrict__ y, int32_t n_out,
                                                        int32_t n_in) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t r = blockIdx.x * kRows + threadIdx.x / kWave;
  if (r >= n_out) return;
  const f32x4* wr = reinterpret_cast<const f32x4*>(w + (size_t)r * n_in);
  const f32x4* xr = reinterpret_cast<const f32x4*>(x);
  float acc = 0.f;
  for (int c = lane; c < n_in / 4; c += kWave) {
    const f32x4 wv = wr[c];
    const f32x4 xv = xr[c];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_fmaf(wv[e], IN_SILU ? silu(xv[e]) : xv[e], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) y[r] = acc + b[r];
}

// v = v + g (v_cond - v), evaluated as g v_cond + (1 - g) v so that g = 1
// returns v_cond and g = 0 returns v exactly; float4 at a time (n % 4 == 0).
__global__ __launch_bounds__(256) void guidance_kernel(const f32x4* __restrict__ vc,
                                                       f32x4* __restrict__ v, int64_t n4,
                                                       float g) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 c = vc[i];
  f32x4 u = v[i];
  const float h = 1.0f - g;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = __builtin_fmaf(g, c[e], h * u[e]);
  v[i] = u;
}

template <typename T>
void qk_dispatch(T* q, T* kc, const int32_t* idx, int32_t rows, int32_t D, int32_t Dh, bool norm,
                 bool rope, const float* qg, const float* kg, int32_t gh, int32_t gw,
                 hipStream_t s) {
  const int blocks = cdiv(rows, kRows);
  // wide rows of 64 NCH 16-byte chunks (NCH 8, 10 or 12; bf16 D = 4096, 5120,
  // 6144): both rows held in registers.  Narrower rows take the loop form,
  // whose second read of a row hits the cache and which keeps more waves per
  // SIMD (D = 1536 bf16: 20.0 us loop form against 20.9 us in registers,
  // D = 5120: 202 against 162 us, at |A| = 8190 and 18900)
  const int nch = D / Chunk<T>::N;
  const int reg = nch % kWave == 0 ? nch / kWave : 0;
  auto run = [&](auto nc) {
    constexpr int NC = decltype(nc)::value;
    if (norm && rope)
      qk_norm_rope_kernel<T, true, true, NC><<<blocks, 256, 0, s>>>(q, kc, idx, rows, D, Dh, qg, kg, gh, gw);
    else if (norm)
      qk_norm_rope_kernel<T, true, false, NC><<<blocks, 256, 0, s>>>(q, kc, idx, rows, D, Dh, qg, kg, gh, gw);
    else
      qk_norm_rope_kernel<T, false, true, NC><<<blocks, 256, 0, s>>>(q, kc, idx, rows, D, Dh, qg, kg, gh, gw);
  };
  switch (reg) {
    case 8: run(std::integral_constant<int, 8>{}); break;
    case 10: run(std::integral_constant<int, 10>{}); break;
    case 12: run(std::integral_constant<int, 12>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
  }
}

}  // namespace

hsa_status launch_qk_norm_rope(void* q, void* kc, const int32_t* idx, int32_t rows, int32_t D,
                               int32_t Dh, hsa_dtype dt, bool norm, bool rope,
                               const float* q_gain, const float* k_gain, int32_t grid_h,
                               int32_t grid_w, hipStream_t s) {
  if (rows == 0 || (!norm && !rope)) return HSA_OK;
  if (Dh % 8 != 0 || Dh > 128 || D % Dh != 0) return HSA_ERR_SHAPE;
  if (dt == HSA_BF16)
    qk_dispatch<bf16>((bf16*)q, (bf16*)kc, idx, rows, D, Dh, norm, rope, q_gain, k_gain, grid_h,
                      grid_w, s);
  else
    qk_dispatch<float>((float*)q, (float*)kc, idx, rows, D, Dh, norm, rope, q_gain, k_gain, grid_h,
                       grid_w, s);
  return launch_status();
}

// e0 [6D] doubles as scratch: the first stage's output goes to its last D
// entries, which the third stage overwrites after the second has read them.
hsa_status launch_time_embed(float sigma, const float* w1, const float* b1, const float* w2,
                             const float* b2, const float* w3, const float* b3, int32_t D,
                             float* e, float* e0, hipStream_t s) {
  if (D % 4 != 0) return HSA_ERR_SHAPE;
  float* e1 = e0 + (size_t)5 * D;
  time_stage1_kernel<<<cdiv(D, kRows), 256, 0, s>>>(sigma, w1, b1, e1, D);
  gemv_bias_kernel<false><<<cdiv(D, kRows), 256, 0, s>>>(w2, e1, b2, e, D, D);
  gemv_bias_kernel<true><<<cdiv(6 * (int64_t)D, kRows), 256, 0, s>>>(w3, e, b3, e0, 6 * D, D);
  return launch_status();
}

hsa_status launch_guidance(const float* v_cond, float* v, int64_t n, float g, hipStream_t s) {
  if (n == 0) return HSA_OK;
  if (n % 4 != 0) return HSA_ERR_SHAPE;
  const int64_t n4 = n / 4;
  guidance_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const f32x4*>(v_cond), reinterpret_cast<f32x4*>(v), n4, g);
  return launch_status();
}

}  // namespace hsa
