// Dynamic token selection (section 2.1): tokens with the largest L1 relative
// change of velocity keep the full budget.  Tokens are ranked by (score
// descending, index ascending), NaN counting as +inf and -0 as +0; rank r goes
// to group k when count[0] + .. + count[k-1] <= r < count[0] + .. + count[k].
//
// Deterministic radix select, one workgroup of 1024 threads:
//   * each score maps to a 32-bit key that increases as the score decreases;
//   * for every group boundary b_k (k = 1..K-1) three histogram passes over
//     11/11/10 key bits find the key t_k of the token at rank b_k and the
//     number of tokens with key t_k that still rank before the boundary;
//   * a final pass in index order assigns groups; tokens whose key equals a
//     boundary key are split by their index-order position among those ties,
//     found with wavefront ballots and a running count.
// The result is unique, so it matches any correct implementation bit for bit.
#include "common.h"

namespace hsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;
constexpr int kMaxB = HSA_MAX_GROUPS - 1;

struct Counts {
  int32_t bound[kMaxB];  // b_k = count[0] + .. + count[k-1], k = 1..K-1
};

__device__ __forceinline__ uint32_t desc_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) u = 0x7f800000u;               // NaN ranks as +inf
  if ((u & 0x7fffffffu) == 0u) u = 0u;       // -0 ranks as +0
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // monotone in the score
  return ~asc;                                // larger score -> smaller key
}

// Exclusive scan of one int per thread over the workgroup.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* wave_tmp, int32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int32_t inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  if (lane == kWave - 1) wave_tmp[wave] = inc;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int32_t c = wave_tmp[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

__global__ __launch_bounds__(kThreads) void select_kernel(const float* __restrict__ score, int32_t N,
                                                          Counts cnt, int32_t nb,
                                                          uint8_t* __restrict__ group_out) {
  __shared__ int32_t hist[kMaxB][kBins];
  __shared__ int32_t wave_tmp[kWaves];
  __shared__ int32_t tie_tot[kMaxB][kWaves];
  __shared__ uint32_t s_prefix[kMaxB];
  __shared__ int32_t s_rem[kMaxB];
  const int tid = threadIdx.x;

  if (tid < kMaxB) {
    s_prefix[tid] = 0u;
    s_rem[tid] = (tid < nb) ? cnt.bound[tid] : 0;
  }
  // Boundaries at or past N have no token at that rank: nothing passes them.
  // ---- three radix passes ----
  const int shifts[3] = {21, 10, 0};
  const uint32_t digit_mask[3] = {0x7ffu, 0x7ffu, 0x3ffu};
  uint32_t mask = 0u;
  for (int pass = 0; pass < 3; ++pass) {
    for (int i = tid; i < kMaxB * kBins; i += kThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const int sh = shifts[pass];
    const uint32_t dm = digit_mask[pass];
    for (int32_t n = tid; n < N; n += kThreads) {
      const uint32_t key = desc_key(score[n]);
      for (int k = 0; k < nb; ++k) {
        if (cnt.bound[k] < N && (key & mask) == s_prefix[k])
          atomicAdd(&hist[k][(key >> sh) & dm], 1);
      }
    }
    __syncthreads();
    for (int k = 0; k < nb; ++k) {
      if (cnt.bound[k] >= N) continue;  // uniform across the workgroup
      const int32_t h0 = hist[k][2 * tid], h1 = hist[k][2 * tid + 1];
      int32_t tot;
      const int32_t before = block_exclusive_scan(h0 + h1, wave_tmp, &tot);
      const int32_t rem = s_rem[k];
      __syncthreads();
      if (before <= rem && rem < before + h0) {
        s_prefix[k] |= (uint32_t)(2 * tid) << sh;
        s_rem[k] = rem - before;
      } else if (before + h0 <= rem && rem < before + h0 + h1) {
        s_prefix[k] |= (uint32_t)(2 * tid + 1) << sh;
        s_rem[k] = rem - before - h0;
      }
      __syncthreads();
    }
    mask |= dm << sh;
  }

  // ---- assignment in index order ----
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t tkey[kMaxB];
  int32_t need[kMaxB], running[kMaxB];
  bool live[kMaxB];
#pragma unroll
  for (int k = 0; k < kMaxB; ++k) {
    live[k] = (k < nb) && (cnt.bound[k] < N);
    tkey[k] = s_prefix[k];
    need[k] = s_rem[k];
    running[k] = 0;
  }
  for (int32_t base = 0; base < N; base += kThreads) {
    const int32_t n = base + tid;
    const bool in = n < N;
    const uint32_t key = in ? desc_key(score[n]) : 0xffffffffu;
    int32_t tie_before[kMaxB];
#pragma unroll
    for (int k = 0; k < kMaxB; ++k) {
      if (k >= nb) break;
      const bool eq = in && live[k] && key == tkey[k];
      const uint64_t b = __ballot(eq);
      tie_before[k] = __popcll(b & lt_mask);
      if (lane == 0) tie_tot[k][wave] = __popcll(b);
    }
    __syncthreads();
    int g = 0;
#pragma unroll
    for (int k = 0; k < kMaxB; ++k) {
      if (k >= nb) break;
      int32_t woff = 0, ctot = 0;
      for (int w = 0; w < kWaves; ++w) {
        const int32_t c = tie_tot[k][w];
        woff += (w < wave) ? c : 0;
        ctot += c;
      }
      if (live[k]) {
        bool ge;
        if (key != tkey[k]) ge = key > tkey[k];
        else ge = (running[k] + woff + tie_before[k]) >= need[k];
        g += ge ? 1 : 0;
      }
      running[k] += ctot;
    }
    if (in) group_out[n] = (uint8_t)g;
    __syncthreads();
  }
}

__global__ void fill_u8_kernel(uint8_t* p, int32_t n, uint8_t v) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hsa_status launch_select(const float* score, int32_t N, const int32_t* count, int32_t K,
                         uint8_t* group_out, hipStream_t s) {
  if (N == 0) return HSA_OK;
  if (K == 1) {
    fill_u8_kernel<<<cdiv(N, 256), 256, 0, s>>>(group_out, N, 0);
    return launch_status();
  }
  Counts c{};
  int32_t acc = 0;
  for (int k = 0; k < K - 1; ++k) {
    acc += count[k];
    c.bound[k] = acc;
  }
  select_kernel<<<1, kThreads, 0, s>>>(score, N, c, K - 1, group_out);
  return launch_status();
}

}  // namespace hsa
