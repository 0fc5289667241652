// GEMMs on the active rows: out = a w^T with a [M][K] (M = |A_i| active rows,
// ragged), w [N][K] out-major.  These carry every per-token linear map of the
// block that KV-cache synchronisation keeps to active tokens (section 2.2):
// the QKV projection (with the fresh K/V rows scattered into the per-layer
// cache, item 2), the attention out-projection, and the MLP.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on 128x128 output tiles, K in steps of
// 64 staged through double-buffered LDS (rows padded by 16 bytes so the
// 16-byte operand reads of 8 consecutive rows fall in distinct banks).  Four
// wavefronts per tile, each owning a 64x64 quarter as 2x2 MFMA blocks.
// Global loads of the next K step are issued before the MFMAs of the current
// one.  Epilogues are fused (store / GELU / residual add / QKV scatter).
//
// float32 path (small float32 workloads): LDS-tiled FMA GEMM, 64x64 tiles.
#include "common.h"

namespace hsa {
namespace {

template <int EPI, typename T>
__device__ __forceinline__ void epilogue(const EpiArgs& ep, int32_t N, int32_t row, int32_t col,
                                         float v) {
  if constexpr (EPI == EPI_STORE) {
    reinterpret_cast<T*>(ep.out)[(size_t)row * N + col] = from_f32<T>(v);
  } else if constexpr (EPI == EPI_GELU) {
    reinterpret_cast<T*>(ep.out)[(size_t)row * N + col] = from_f32<T>(gelu_tanh(v));
  } else if constexpr (EPI == EPI_RESID) {
    float* p = ep.resid + (size_t)row * N + col;
    *p = *p + v;
  } else {  // EPI_QKV_SCATTER
    const int32_t D = ep.D;
    const int32_t which = col / D;
    const int32_t c = col - which * D;
    if (which == 0) {
      reinterpret_cast<T*>(ep.out)[(size_t)row * D + c] = from_f32<T>(v);
    } else {
      const size_t r = (size_t)ep.idx[row];
      T* dst = reinterpret_cast<T*>(which == 1 ? ep.kc : ep.vc);
      dst[r * D + c] = from_f32<T>(v);
    }
  }
}

// ---------------------------------------------------------------- bf16 MFMA
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (16-byte pad)
constexpr int kGemmThreads = 256;

// XCD-aware tile order: consecutive workgroup ids land on different XCDs
// (round-robin over 8), so hand each XCD a contiguous run of tiles; within a
// run, tiles walk M fastest so concurrent workgroups share a column block of w.
__device__ __forceinline__ int32_t xcd_tile(int32_t bid, int32_t ntiles) {
  constexpr int32_t kXcd = 8;
  const int32_t per = ntiles / kXcd;
  const int32_t full = per * kXcd;
  if (bid >= full) return bid;  // leftover tail keeps its id
  return (bid % kXcd) * per + bid / kXcd;
}

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, int32_t M, int32_t N, int32_t K,
    EpiArgs ep) {
  __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * LDS_STRIDE];

  const int32_t tm = (M + BM - 1) / BM;
  const int32_t tn = (N + BN - 1) / BN;
  const int32_t tile = xcd_tile(blockIdx.x, tm * tn);
  const int32_t m0 = (tile % tm) * BM;
  const int32_t n0 = (tile / tm) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Global -> register staging: 4 chunks of 16 bytes per thread per operand.
  u32x4 ra[4], rb[4];
  auto load_tile = [&](int32_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kGemmThreads;
      const int r = c >> 3, kc = c & 7;
      const int32_t gm = m0 + r, gn = n0 + r;
      ra[i] = (gm < M) ? *reinterpret_cast<const u32x4*>(A + (size_t)gm * K + k0 + kc * 8)
                       : u32x4{0u, 0u, 0u, 0u};
      rb[i] = (gn < N) ? *reinterpret_cast<const u32x4*>(W + (size_t)gn * K + k0 + kc * 8)
                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kGemmThreads;
      const int r = c >> 3, kc = c & 7;
      *reinterpret_cast<u32x4*>(&sA[buf][r * LDS_STRIDE + kc * 8]) = ra[i];
      *reinterpret_cast<u32x4*>(&sB[buf][r * LDS_STRIDE + kc * 8]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
    const bf16* a_base = &sA[buf][(wm * 64 + frag_row) * LDS_STRIDE + frag_k];
    const bf16* b_base = &sB[buf][(wn * 64 + frag_row) * LDS_STRIDE + frag_k];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(a_base + i * 32 * LDS_STRIDE + ks * 16);
        bfr[i] = *reinterpret_cast<const bf16x8*>(b_base + i * 32 * LDS_STRIDE + ks * 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j][r]: row 8*(r/4) + 4*(lane/32) + r%4, column lane%32 of block (i, j).
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int32_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < M && col < N) epilogue<EPI, bf16>(ep, N, row, col, acc[i][j][r]);
      }
}

// ---------------------------------------------------------------- float32
constexpr int FT = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ W, int32_t M,
                                                       int32_t N, int32_t K, EpiArgs ep) {
  __shared__ float sA[FK][FT + 4];
  __shared__ float sB[FK][FT + 4];
  const int32_t m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  const int tid = threadIdx.x;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int32_t k0 = 0; k0 < K; k0 += FK) {
    const int32_t gk = k0 + lk;
    f32x4 va = {0.f, 0.f, 0.f, 0.f}, vb = {0.f, 0.f, 0.f, 0.f};
    if (m0 + lr < M && gk < K) va = *reinterpret_cast<const f32x4*>(A + (size_t)(m0 + lr) * K + gk);
    if (n0 + lr < N && gk < K) vb = *reinterpret_cast<const f32x4*>(W + (size_t)(n0 + lr) * K + gk);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sA[lk + e][lr] = va[e];
      sB[lk + e][lr] = vb[e];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; ++k) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sA[k][ty * 4]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&sB[k][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row < M && col < N) epilogue<EPI, float>(ep, N, row, col, acc[i][j]);
    }
}

template <int EPI>
hsa_status run(const void* a, const void* w, int32_t M, int32_t N, int32_t K, hsa_dtype dt,
               const EpiArgs& ep, hipStream_t s) {
  if (dt == HSA_BF16) {
    const int32_t tiles = cdiv(M, BM) * cdiv(N, BN);
    gemm_bf16_kernel<EPI><<<tiles, kGemmThreads, 0, s>>>((const bf16*)a, (const bf16*)w, M, N, K, ep);
  } else {
    dim3 grid(cdiv(N, FT), cdiv(M, FT));
    gemm_f32_kernel<EPI><<<grid, 256, 0, s>>>((const float*)a, (const float*)w, M, N, K, ep);
  }
  return launch_status();
}

}  // namespace

hsa_status launch_gemm(const void* a, const void* w, int32_t M, int32_t N, int32_t K,
                       hsa_dtype dt, int epi, const EpiArgs& ep, hipStream_t s) {
  if (M == 0 || N == 0) return HSA_OK;
  switch (epi) {
    case EPI_STORE: return run<EPI_STORE>(a, w, M, N, K, dt, ep, s);
    case EPI_GELU: return run<EPI_GELU>(a, w, M, N, K, dt, ep, s);
    case EPI_RESID: return run<EPI_RESID>(a, w, M, N, K, dt, ep, s);
    case EPI_QKV_SCATTER: return run<EPI_QKV_SCATTER>(a, w, M, N, K, dt, ep, s);
    default: return HSA_ERR_ARG;
  }
}

}  // namespace hsa
