// Internal helpers shared by the HIP kernels and the host API of libhsa.
// gfx950 (CDNA4) only: 64-wide wavefronts, bf16 MFMA (32x32x16 and 16x16x32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hsa.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace hsa {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLnEps = 1e-6f;

// ---- scalar conversions -------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// GELU, tanh form: 0.5 u (1 + tanh(z)) = u / (1 + exp(-2z)),
// z = sqrt(2/pi) (u + 0.044715 u^3).  exp via the hardware exp2.
__device__ __forceinline__ float gelu_tanh(float u) {
  const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
  const float z = k0 * (u + 0.044715f * u * u * u);
  const float e = __builtin_amdgcn_exp2f(-2.0f * kLog2e * z);
  return u / (1.0f + e);
}

// ---- wave reductions (64 lanes) -------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- host-side helpers ----------------------------------------------------
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hsa_status launch_status() {
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}
inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline size_t dtype_size(hsa_dtype t) { return t == HSA_BF16 ? 2 : 4; }

// ---- kernel launchers (one per .hip file), argument checks done by callers --
hsa_status launch_active_set(const uint8_t* group, int32_t N, uint32_t active_groups,
                             int32_t expected, int32_t* active_idx, int32_t* pos,
                             int32_t* n_active_dev, hipStream_t s);
hsa_status launch_select(const float* score, int32_t B, int32_t N, const int32_t* count,
                         int32_t K, uint8_t* group_out, hipStream_t s);
hsa_status launch_euler(float* x, float* v_hat, float* score, const float* v_new,
                        const int32_t* pos, int32_t N, int32_t C, float dsigma, float eps,
                        int32_t update_score, hipStream_t s);
hsa_status launch_gather_rows(const float* src, const int32_t* idx, float* dst, int32_t rows,
                              int32_t C, hipStream_t s);

// A float32 vector [n] given as base[i] + add[i] (add may be null), so that a
// block's modulation table row and the per-iteration timestep projection are
// combined where they are read.  base == null: the vector is absent.
struct ModVec {
  const float* base;
  const float* add;
  __host__ __device__ bool present() const { return base != nullptr; }
};
__device__ __forceinline__ f32x4 load_mod4(const ModVec& m, int32_t i) {
  f32x4 v = *reinterpret_cast<const f32x4*>(m.base + i);
  if (m.add) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(m.add + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += a[e];
  }
  return v;
}
__device__ __forceinline__ float load_mod(const ModVec& m, int32_t i) {
  return m.add ? m.base[i] + m.add[i] : m.base[i];
}

// LayerNorm, optionally modulated: LN(h) (1 + scale) + shift when both are present.
hsa_status launch_layernorm(const float* h, void* out, int32_t rows, int32_t D, hsa_dtype dt,
                            ModVec shift, ModVec scale, hipStream_t s);
hsa_status launch_embed(const float* x, const int32_t* idx, const void* w_in, float* h,
                        int32_t rows, int32_t C, int32_t D, hsa_dtype dt, hipStream_t s);
hsa_status launch_unembed(const float* h, const void* w_out, float* v_new, int32_t rows,
                          int32_t D, int32_t C, hsa_dtype dt, ModVec shift, ModVec scale,
                          hipStream_t s);

// Optional block features (wanfeat.hip).
hsa_status launch_qk_norm_rope(void* q, void* kc, const int32_t* idx, int32_t rows, int32_t D,
                               int32_t Dh, hsa_dtype dt, bool norm, bool rope,
                               const float* q_gain, const float* k_gain, int32_t grid_h,
                               int32_t grid_w, hipStream_t s);
hsa_status launch_time_embed(float sigma, const float* w1, const float* b1, const float* w2,
                             const float* b2, const float* w3, const float* b3, int32_t D,
                             float* e, float* e0, hipStream_t s);
hsa_status launch_guidance(const float* v_cond, float* v, int64_t n, float g, hipStream_t s);

// GEMM epilogues: out = a w^T followed by one of these.
enum Epilogue : int {
  EPI_STORE = 0,        // out[m][n] = acc                      (dtype)
  EPI_GELU = 1,         // out[m][n] = gelu(acc)                (dtype)
  EPI_RESID = 2,        // resid[m][n] += acc                   (float32)
  EPI_QKV_SCATTER = 3,  // n <  D: q[m][n];  n < 2D: kc[idx[m]][n-D];  else vc[idx[m]][n-2D]
  EPI_RESID_GATED = 4,  // resid[m][n] += gate[n] * acc          (float32)
};
struct EpiArgs {
  void* out;            // EPI_STORE / EPI_GELU output, EPI_QKV_SCATTER q output
  float* resid;         // EPI_RESID
  void* kc;             // EPI_QKV_SCATTER caches
  void* vc;
  const int32_t* idx;   // EPI_QKV_SCATTER row -> cache row
  int32_t D;            // EPI_QKV_SCATTER width of each of q, k, v
  ModVec gate;          // EPI_RESID_GATED, [N]
  int32_t gather_rows;  // EPI_QKV_SCATTER only: > 0 when row m of a is a[idx[m]] of an
                        // a with gather_rows rows; 0 when a is [M][K]
};
hsa_status launch_gemm(const void* a, const void* w, int32_t M, int32_t N, int32_t K,
                       hsa_dtype dt, int epi, const EpiArgs& ep, hipStream_t s);

size_t attn_workspace_bytes(int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh);
hsa_status launch_attention(const void* q, const void* k, const void* v, void* o,
                            int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh, float scale,
                            hsa_dtype dt, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace hsa
