// Dynamic token selection (section 2.1): tokens with the largest L1 relative
// change of velocity keep the full budget.  Tokens are ranked by (score
// descending, index ascending), NaN counting as +inf and -0 as +0; rank r goes
// to group k when count[0] + .. + count[k-1] <= r < count[0] + .. + count[k].
//
// Deterministic radix select, one workgroup of 1024 threads per row of a
// [B][N] batch (independent selections with the same counts):
//   * each score maps to a 32-bit key that increases as the score decreases;
//     for rows of up to 32768 tokens the keys stay in registers (thread t
//     holds tokens 4 (t + 1024 j) + e), so the row crosses HBM once: 4N
//     bytes of scores in, N bytes of groups out;
//   * the first pass (top 11 key bits) histograms every key as it is loaded
//     and serves every group boundary b_k (k = 1..K-1) at once; two more
//     passes (11 and 10 bits) narrow each boundary to the key t_k of the token
//     at rank b_k and the number need_k of tokens with key t_k that still rank
//     before it (every boundary's histogram filled in the same sweep; only
//     keys in a boundary's bucket are counted);
//   * assignment: group = number of boundaries whose key the token's key
//     reaches.  When some need_k > 0, the ties with t_k are split by their
//     index-order position: ballots count them per (wavefront, 4096-token
//     chunk), and one wavefront scans those counts.
//   Longer rows take the same passes reading the scores from memory.
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

constexpr uint32_t kPad = 0xffffffffu;   // above every key desc_key produces (max 0xff800000)

// Bucket of this thread's two bins (2t, 2t+1) that holds rank rem, given the
// exclusive prefix `before` of the bins below them: records the digit, the
// rank left inside the bucket and the bucket's size.
__device__ __forceinline__ void take_bucket(int32_t before, int32_t h0, int32_t h1, int32_t rem,
                                            int sh, uint32_t* prefix, int32_t* rem_out,
                                            int32_t* size_out) {
  const int tid = threadIdx.x;
  if (before <= rem && rem < before + h0) {
    *prefix |= (uint32_t)(2 * tid) << sh;
    *rem_out = rem - before;
    *size_out = h0;
  } else if (before + h0 <= rem && rem < before + h0 + h1) {
    *prefix |= (uint32_t)(2 * tid + 1) << sh;
    *rem_out = rem - before - h0;
    *size_out = h1;
  }
}

// Group bytes of tokens n..n+3 (packed, token n in the low byte), n + e < N only.
__device__ __forceinline__ void store_groups(uint8_t* out, int32_t n, int32_t N, uint32_t packed,
                                             bool aligned4) {
  if (aligned4 && n + 3 < N) {
    *reinterpret_cast<uint32_t*>(out + n) = packed;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < N) out[n + e] = (uint8_t)(packed >> (8 * e));
  }
}

template <int V>   // float4 loads per thread: rows of up to 4 * V * kThreads tokens
__global__ __launch_bounds__(kThreads) void select_reg_kernel(const float* __restrict__ score,
                                                              int32_t N, Counts cnt, int32_t nb,
                                                              uint8_t* __restrict__ group_out) {
  __shared__ int32_t hist[kMaxB][kBins];   // one per boundary in passes 2-3; pass 1 uses [0]
  __shared__ int32_t wave_tmp[kWaves];
  __shared__ int32_t tie_pre[V * kWaves];  // ties per (chunk j, wavefront), then their prefix
  __shared__ uint32_t s_prefix[kMaxB];
  __shared__ int32_t s_rem[kMaxB];
  __shared__ int32_t s_size[kMaxB];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const float* row = score + (size_t)blockIdx.x * N;
  uint8_t* out = group_out + (size_t)blockIdx.x * N;
  auto live = [&](int k) { return k < nb && cnt.bound[k] < N; };   // a boundary at N: none pass

  for (int i = tid; i < kBins; i += kThreads) hist[0][i] = 0;
  if (tid < kMaxB) {
    s_prefix[tid] = 0u;
    s_rem[tid] = (tid < nb) ? cnt.bound[tid] : 0;
    s_size[tid] = 0;
  }
  __syncthreads();

  // ---- the row into registers as keys, with the pass-1 histogram (bits 31..21)
  uint32_t key[V][4];
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0u) {
    f32x4 raw[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int32_t n = 4 * (tid + j * kThreads);
      if (n + 3 < N) raw[j] = *reinterpret_cast<const f32x4*>(row + n);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int32_t n = 4 * (tid + j * kThreads);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        key[j][e] = (n + 3 < N) ? desc_key(raw[j][e]) : (n + e < N ? desc_key(row[n + e]) : kPad);
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int32_t n = 4 * (tid + j * kThreads);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j][e] = (n + e < N) ? desc_key(row[n + e]) : kPad;
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (key[j][e] != kPad) atomicAdd(&hist[0][key[j][e] >> 21], 1);
  {
    int32_t rem[kMaxB];
#pragma unroll
    for (int k = 0; k < kMaxB; ++k) rem[k] = __builtin_amdgcn_readfirstlane(s_rem[k]);
    __syncthreads();
    const int32_t h0 = hist[0][2 * tid], h1 = hist[0][2 * tid + 1];
    int32_t tot;
    const int32_t before = block_exclusive_scan(h0 + h1, wave_tmp, &tot);
#pragma unroll
    for (int k = 0; k < kMaxB; ++k)
      if (live(k)) take_bucket(before, h0, h1, rem[k], 21, &s_prefix[k], &s_rem[k], &s_size[k]);
    __syncthreads();
  }

  // ---- passes 2 and 3 (bits 20..10, 9..0), every boundary in one sweep
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int sh = pass == 0 ? 10 : 0;
    const uint32_t dm = pass == 0 ? 0x7ffu : 0x3ffu;
    const uint32_t mask = pass == 0 ? 0xffe00000u : 0xfffffc00u;   // bits already fixed
    uint32_t pre[kMaxB];
    int32_t rem[kMaxB];
#pragma unroll
    for (int k = 0; k < kMaxB; ++k) {
      pre[k] = __builtin_amdgcn_readfirstlane(live(k) ? s_prefix[k] : kPad);   // kPad & mask matches no key
      rem[k] = __builtin_amdgcn_readfirstlane(s_rem[k]);
      if (live(k))
        for (int i = tid; i < kBins; i += kThreads) hist[k][i] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t m = key[j][e] & mask;
#pragma unroll
        for (int k = 0; k < kMaxB; ++k)
          if (k < nb && m == pre[k]) atomicAdd(&hist[k][(key[j][e] >> sh) & dm], 1);
      }
    __syncthreads();
    for (int k = 0; k < nb; ++k) {
      if (!live(k)) continue;   // uniform across the workgroup
      const int32_t h0 = hist[k][2 * tid], h1 = hist[k][2 * tid + 1];
      int32_t tot;
      const int32_t before = block_exclusive_scan(h0 + h1, wave_tmp, &tot);
      take_bucket(before, h0, h1, rem[k], sh, &s_prefix[k], &s_rem[k], &s_size[k]);
    }
    __syncthreads();
  }

  // ---- assignment
  uint32_t tk[kMaxB];
  int32_t need[kMaxB];
#pragma unroll
  for (int k = 0; k < kMaxB; ++k) {
    tk[k] = __builtin_amdgcn_readfirstlane(live(k) ? s_prefix[k] : kPad);   // no key reaches kPad
    need[k] = __builtin_amdgcn_readfirstlane(live(k) ? s_rem[k] : 0);
  }
  uint32_t gp[V];   // 4 group bytes per chunk
#pragma unroll
  for (int j = 0; j < V; ++j) gp[j] = 0u;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int k = 0; k < kMaxB; ++k) {
    if (k >= nb) break;
    if (need[k] == 0) {   // every tie with t_k ranks at or past the boundary
#pragma unroll
      for (int j = 0; j < V; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) gp[j] += (key[j][e] != kPad && key[j][e] >= tk[k]) ? 1u << (8 * e) : 0u;
      continue;
    }
    // ties per (chunk, wavefront): index order is chunk-major, then wavefront,
    // lane and element
#pragma unroll
    for (int j = 0; j < V; ++j) {
      int32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += __popcll(__ballot(key[j][e] == tk[k]));
      if (lane == 0) tie_pre[j * kWaves + wave] = c;
    }
    __syncthreads();
    if (wave == 0) {   // exclusive scan of the V * kWaves counts, 64 lanes over runs
      constexpr int E = V * kWaves, PER = (E + kWave - 1) / kWave;
      int32_t v[PER], sum = 0;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int i = lane * PER + q;
        v[q] = i < E ? tie_pre[i] : 0;
        sum += v[q];
      }
      int32_t inc = sum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int32_t y = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += y;
      }
      int32_t run = inc - sum;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int i = lane * PER + q;
        if (i < E) tie_pre[i] = run;
        run += v[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < V; ++j) {
      int32_t before = tie_pre[j * kWaves + wave];
      bool eq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        eq[e] = key[j][e] == tk[k];
        before += __popcll(__ballot(eq[e]) & lt_mask);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ge = eq[e] ? before >= need[k] : (key[j][e] != kPad && key[j][e] > tk[k]);
        gp[j] += ge ? 1u << (8 * e) : 0u;
        before += eq[e] ? 1 : 0;
      }
    }
    __syncthreads();   // tie_pre is reused by the next boundary
  }
  const bool aligned4 = (reinterpret_cast<uintptr_t>(out) & 3u) == 0u;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int32_t n = 4 * (tid + j * kThreads);
    if (n < N) store_groups(out, n, N, gp[j], aligned4);
  }
}

// Rows past the register capacity: the same passes, reading the scores from
// memory each time (the row stays in L2 / the Infinity Cache between passes).
__global__ __launch_bounds__(kThreads) void select_mem_kernel(const float* __restrict__ score,
                                                              int32_t N, Counts cnt, int32_t nb,
                                                              uint8_t* __restrict__ group_out) {
  __shared__ int32_t hist[kBins];
  __shared__ int32_t wave_tmp[kWaves];
  __shared__ int32_t tie_tot[kMaxB][kWaves];
  __shared__ uint32_t s_prefix[kMaxB];
  __shared__ int32_t s_rem[kMaxB];
  __shared__ int32_t s_size[kMaxB];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const float* row = score + (size_t)blockIdx.x * N;
  uint8_t* out = group_out + (size_t)blockIdx.x * N;
  auto live = [&](int k) { return k < nb && cnt.bound[k] < N; };

  if (tid < kMaxB) {
    s_prefix[tid] = 0u;
    s_rem[tid] = (tid < nb) ? cnt.bound[tid] : 0;
  }
  const int shifts[3] = {21, 10, 0};
  const uint32_t digit_mask[3] = {0x7ffu, 0x7ffu, 0x3ffu};
  uint32_t mask = 0u;
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t dm = digit_mask[pass];
    for (int k = 0; k < nb; ++k) {
      if (!live(k)) continue;   // uniform across the workgroup
      for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix[k];
      const int32_t rem = s_rem[k];
      for (int32_t n = tid; n < N; n += kThreads) {
        const uint32_t key = desc_key(row[n]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> sh) & dm], 1);
      }
      __syncthreads();
      const int32_t h0 = hist[2 * tid], h1 = hist[2 * tid + 1];
      int32_t tot;
      const int32_t before = block_exclusive_scan(h0 + h1, wave_tmp, &tot);
      take_bucket(before, h0, h1, rem, sh, &s_prefix[k], &s_rem[k], &s_size[k]);
      __syncthreads();
    }
    mask |= dm << sh;
  }

  // assignment in index order, 1024 tokens at a time
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t tkey[kMaxB];
  int32_t need[kMaxB], running[kMaxB];
#pragma unroll
  for (int k = 0; k < kMaxB; ++k) {
    tkey[k] = live(k) ? s_prefix[k] : kPad;
    need[k] = s_rem[k];
    running[k] = 0;
  }
  for (int32_t base = 0; base < N; base += kThreads) {
    const int32_t n = base + tid;
    const bool in = n < N;
    const uint32_t key = in ? desc_key(row[n]) : kPad;
    int32_t tie_before[kMaxB];
#pragma unroll
    for (int k = 0; k < kMaxB; ++k) {
      if (k >= nb) break;
      const uint64_t b = __ballot(in && key == tkey[k]);
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
      if (live(k)) {
        const bool ge = key != tkey[k] ? key > tkey[k] : (running[k] + woff + tie_before[k]) >= need[k];
        g += ge ? 1 : 0;
      }
      running[k] += ctot;
    }
    if (in) out[n] = (uint8_t)g;
    __syncthreads();
  }
}

__global__ void fill_u8_kernel(uint8_t* p, int64_t n, uint8_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hsa_status launch_select(const float* score, int32_t B, int32_t N, const int32_t* count,
                         int32_t K, uint8_t* group_out, hipStream_t s) {
  if (N == 0 || B == 0) return HSA_OK;
  if (K == 1) {
    const int64_t n = (int64_t)B * N;
    fill_u8_kernel<<<cdiv(n, 256), 256, 0, s>>>(group_out, n, 0);
    return launch_status();
  }
  Counts c{};
  int32_t acc = 0;
  for (int k = 0; k < K - 1; ++k) {
    acc += count[k];
    c.bound[k] = acc;
  }
  if (N <= 4 * 8 * kThreads)
    select_reg_kernel<8><<<B, kThreads, 0, s>>>(score, N, c, K - 1, group_out);
  else
    select_mem_kernel<<<B, kThreads, 0, s>>>(score, N, c, K - 1, group_out);
  return launch_status();
}

}  // namespace hsa
