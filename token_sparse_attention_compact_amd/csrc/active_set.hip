// Active-set compaction: the activity rule of the token partitioning and
// scheduling section (2.1) and the "only active tokens" step of KV-cache
// synchronisation (2.2).  Token n is active at iteration i iff
// i mod (T / s_{g(n)}) == 0; the host folds that test into a per-group bit
// mask, so the kernel only looks up bit g(n).
//
// One workgroup of 1024 threads walks the token range in chunks of 4096
// (4 tokens per thread, one 32-bit load of group bytes).  Inside a chunk the
// order-preserving positions come from wavefront ballots (one per token slot)
// and a scan of the 16 wave totals in LDS; a running total carries across
// chunks.  Output order is ascending token index, so the result is unique and
// bit-exact.
//
// The launches that follow are sized by the host's closed-form |A_i|
// (`expected`).  Groups that do not hold exactly count[k] tokens (a caller
// error) must still leave every later access in bounds: entries past the
// actual count are filled with token 0, and tokens past `expected` are
// marked skipped.  *n_active receives the actual count.
#include "common.h"

namespace hsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kPerThread = 4;
constexpr int kChunk = kThreads * kPerThread;

__global__ __launch_bounds__(kThreads) void active_set_kernel(
    const uint8_t* __restrict__ group, int32_t N, uint32_t active_groups, int32_t expected,
    int32_t* __restrict__ active_idx, int32_t* __restrict__ pos, int32_t* __restrict__ n_active) {
  __shared__ int32_t wave_tot[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t running = 0;

  for (int32_t base = 0; base < N; base += kChunk) {
    const int32_t t0 = base + tid * kPerThread;
    bool f[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int32_t n = t0 + j;
      f[j] = (n < N) && ((active_groups >> group[n]) & 1u);
    }
    // Token (lane, j) precedes (lane', j') iff lane < lane' or (lane == lane' and j < j').
    int32_t before = 0, wtot = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const uint64_t b = __ballot(f[j]);
      before += __popcll(b & lt_mask);
      wtot += __popcll(b);
    }
    if (lane == 0) wave_tot[wave] = wtot;
    __syncthreads();
    int32_t wave_off = 0, chunk_tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int32_t c = wave_tot[w];
      wave_off += (w < wave) ? c : 0;
      chunk_tot += c;
    }
    int32_t p = running + wave_off + before;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int32_t n = t0 + j;
      if (n < N) {
        if (f[j] && p < expected) {
          active_idx[p] = n;
          pos[n] = p;
        } else {
          pos[n] = -1;
        }
        p += f[j] ? 1 : 0;
      }
    }
    running += chunk_tot;
    __syncthreads();  // wave_tot is rewritten by the next chunk
  }
  for (int32_t i = running + tid; i < expected; i += kThreads) active_idx[i] = 0;
  if (tid == 0) *n_active = running;
}

}  // namespace

hsa_status launch_active_set(const uint8_t* group, int32_t N, uint32_t active_groups,
                             int32_t expected, int32_t* active_idx, int32_t* pos,
                             int32_t* n_active_dev, hipStream_t s) {
  active_set_kernel<<<1, kThreads, 0, s>>>(group, N, active_groups, expected, active_idx, pos,
                                           n_active_dev);
  return launch_status();
}

}  // namespace hsa
