// Dynamic token selection (section 2.1): tokens with the largest L1 relative
// change of velocity keep the full budget.  Tokens are ranked by (score
// descending, index ascending), NaN counting as +inf and -0 as +0; rank r goes
// to group k when count[0] + .. + count[k-1] <= r < count[0] + .. + count[k].
//
// Deterministic radix select, one workgroup of 1024 threads per row of a
// [B][N] batch (independent selections with the same counts):
//   * each score maps to a 32-bit key that increases as the score decreases;
//     for rows of up to 32768 tokens thread t holds tokens 4 (t + 1024 j) + e,
//     so the row crosses HBM once: 4N bytes of scores in, N bytes of groups
//     out.  Persistent workgroups (one per CU) walk the rows of the batch,
//     loading the next row while the current one is ranked;
//   * the smallest and largest key give the bits every key shares, and the
//     digit passes start below them;
//   * one or two boundaries (K <= 3, select_lds_kernel): a first pass of a
//     12-bit digit over every key serves both boundaries; further 11-bit
//     passes only while a boundary's bucket holds more keys than a quarter
//     of its threads; then each bucket's keys go to an LDS list, which four
//     threads per key rank by comparing every pair (rank_in_list).  This
//     gives t_k, the key of the token at rank b_k, and need_k, the number of
//     tokens with key t_k that still rank before it;
//   * three to seven boundaries (select_reg_kernel): the same with an 11-bit
//     first pass into four histogram copies, narrowing passes while a bucket
//     exceeds 1024 keys, and each list finished by one wavefront
//     (finish_bucket);
//   * assignment: group = number of boundaries whose key the token's key
//     reaches.  When some need_k > 0, the ties with t_k are split by their
//     index-order position: ballots count them per (wavefront, 4096-token
//     chunk), and one wavefront scans those counts.
//   Longer rows take three fixed passes, reading the scores from memory.
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
  u = (f != f) ? 0x7f800000u : u;                  // NaN ranks as +inf
  u = (u == 0x80000000u) ? 0u : u;                 // -0 ranks as +0
  // monotone in the score: flip every bit of negatives, the sign bit of the rest
  const uint32_t asc = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return ~asc;                                     // larger score -> smaller key
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP (row shifts
// within rows of 16 lanes, then row broadcasts of lanes 15 and 31): no LDS
// traffic, unlike shuffles.  Lanes that a shift leaves without a source add 0.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return x;
}

// Smallest and largest value over the wavefront (the same DPP pattern; lanes
// without a source take the identity), returned to every lane.
__device__ __forceinline__ void wave_min_max(uint32_t& mn, uint32_t& mx) {
  int a = (int)mn, b = (int)mx;
  const int id_min = (int)0xffffffffu, id_max = 0;
#define HSA_DPP_STEP(ctrl, rows)                                                              \
  a = (int)min((uint32_t)a, (uint32_t)__builtin_amdgcn_update_dpp(id_min, a, ctrl, rows, 0xf, false)); \
  b = (int)max((uint32_t)b, (uint32_t)__builtin_amdgcn_update_dpp(id_max, b, ctrl, rows, 0xf, false));
  HSA_DPP_STEP(0x111, 0xf) HSA_DPP_STEP(0x112, 0xf) HSA_DPP_STEP(0x114, 0xf)
  HSA_DPP_STEP(0x118, 0xf) HSA_DPP_STEP(0x142, 0xa) HSA_DPP_STEP(0x143, 0xc)
#undef HSA_DPP_STEP
  mn = (uint32_t)__builtin_amdgcn_readlane(a, 63);
  mx = (uint32_t)__builtin_amdgcn_readlane(b, 63);
}

// Exclusive scan of one int per thread over the workgroup.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* wave_tmp, int32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int32_t inc = wave_incl_scan(v);
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

// The same for four bins 4t .. 4t + 3.
__device__ __forceinline__ void take_bucket4(int32_t before, const int32_t (&h)[4], int32_t rem,
                                             int sh, uint32_t* prefix, int32_t* rem_out,
                                             int32_t* size_out) {
  const int tid = threadIdx.x;
  int32_t run = before;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (run <= rem && rem < run + h[q]) {
      *prefix |= (uint32_t)(4 * tid + q) << sh;
      *rem_out = rem - run;
      *size_out = h[q];
    }
    run += h[q];
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

constexpr int kV = 8;          // float4 loads per thread: rows of up to 4 * kV * kThreads tokens
constexpr int kList = kThreads; // a bucket this small is copied to LDS and finished there
constexpr int kCopies = 4;     // first-pass histogram copies (by lane % 4): fewer same-address atomics
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// 16-byte buffer loads of a row's raw score bits (zero past its 4N bytes),
// thread t taking chunks t + 1024 j; 4-byte loads when the row is not
// 16-byte aligned (a batch with N % 4 != 0).
__device__ __forceinline__ void load_row_bits(const float* row, int32_t N, uint32_t (&raw)[kV][4]) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, N * 4, 0x00020000);
  const int tid = threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0u) {
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * (tid + j * kThreads), 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[j][e] = v[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        raw[j][e] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, 16 * (tid + j * kThreads) + 4 * e, 0, 0);
  }
}

// One wavefront finishes a boundary from the list of its bucket's keys
// (n <= kList entries; `fixed` the key bits the bucket shares, `lo` the
// number still free): while more than 64 keys remain in the bucket, a digit
// pass of up to 11 bits (histogram in `hist`, scanned by the wavefront: lane
// l sums bins 32 l .. 32 l + 31); then the remaining keys are gathered into
// `small` and ranked directly.  On return *prefix is the key t at the
// boundary's rank and *rem the number of keys equal to t that rank before it.
// Wavefront-local: LDS operations of one wavefront take effect in order.
__device__ __forceinline__ void finish_bucket(const uint32_t* list, int32_t n, int32_t* hist,
                                              uint32_t* small, uint32_t fixed, int lo,
                                              uint32_t* prefix, int32_t* rem_io) {
  constexpr int M = kList / kWave;   // list entries per lane, loaded once
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t pre = __builtin_amdgcn_readfirstlane(*prefix);
  int32_t rem = __builtin_amdgcn_readfirstlane(*rem_io);
  uint32_t c[M];
#pragma unroll
  for (int m = 0; m < M; ++m) c[m] = list[lane + kWave * m < n ? lane + kWave * m : 0];
  while (lo > 0) {   // lo == 0: every bit fixed, pre is t and rem its tie count
    int32_t total = 0;
#pragma unroll
    for (int m = 0; m < M; ++m)
      total += __popcll(__ballot(lane + kWave * m < n && (c[m] & fixed) == pre));
    if (total <= kWave) {   // gather the bucket's keys, one per lane, and rank them
      int32_t at = 0;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const bool in = lane + kWave * m < n && (c[m] & fixed) == pre;
        const uint64_t bal = __ballot(in);
        if (in) small[at + __popcll(bal & lt_mask)] = c[m];
        at += __popcll(bal);
      }
      const uint32_t x = lane < total ? small[lane] : 0u;
      int32_t less = 0, leq = 0;
      for (int i = 0; i < total; ++i) {   // i is uniform: the key of lane i from a register
        const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, i);
        less += y < x ? 1 : 0;
        leq += y <= x ? 1 : 0;
      }
      const bool hit = lane < total && less <= rem && rem < leq;   // x is the key at rank rem
      const int src = __builtin_ctzll(__ballot(hit));               // some lane holds it
      pre = (uint32_t)__builtin_amdgcn_readlane((int)x, src);
      rem = rem - __builtin_amdgcn_readlane(less, src);
      break;
    }
    const int width = lo < 11 ? lo : 11;
    const int sh = lo - width;
    const uint32_t dm = (1u << width) - 1u;
#pragma unroll
    for (int i = 0; i < kBins / kWave; i += 4)
      *reinterpret_cast<i32x4_t*>(&hist[32 * lane + i]) = i32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (lane + kWave * m < n && (c[m] & fixed) == pre) atomicAdd(&hist[(c[m] >> sh) & dm], 1);
    int32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kBins / kWave; i += 4) {
      const i32x4_t v = *reinterpret_cast<const i32x4_t*>(&hist[32 * lane + i]);
      sum += (v[0] + v[1]) + (v[2] + v[3]);
    }
    const int32_t inc = wave_incl_scan(sum);
    const int32_t excl = inc - sum;
    // the lane whose 32 bins hold rank rem; then 32 lanes scan those bins
    const int src = __builtin_ctzll(__ballot(excl <= rem && rem < inc));
    const int32_t left0 = rem - __builtin_amdgcn_readlane(excl, src);
    const int32_t hb = lane < 32 ? hist[32 * src + lane] : 0;
    const int32_t hinc = wave_incl_scan(hb);
    const int bin = __builtin_ctzll(__ballot(lane < 32 && left0 < hinc));   // first bin reaching rank
    pre |= (uint32_t)(32 * src + bin) << sh;
    rem = left0 - (__builtin_amdgcn_readlane(hinc, bin) - __builtin_amdgcn_readlane(hb, bin));
    fixed |= dm << sh;
    lo = sh;
  }
  if (lane == 0) {
    *prefix = pre;
    *rem_io = rem;
  }
}

// One lane adds v to the LDS counter *p; every lane gets the value before.
// (Written out so that the compiler does not rebuild it as a whole-wavefront
// atomic; the wait is inside the same statement.)
__device__ __forceinline__ int32_t lds_reserve(int32_t* p, int32_t v) {
  int32_t old = 0;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int32_t*)p;
    asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(old) : "v"(a), "v"(v) : "memory");
  }
  return __builtin_amdgcn_readfirstlane(old);
}

// Lanes below this one whose bit is set in m.
__device__ __forceinline__ int32_t lanes_below(uint64_t m) {
  return (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The threads t = 0, 1, .. of one boundary (whole wavefronts, four per key)
// rank the n keys of its list, whose slots from n on hold kPad: the four
// lanes 4i .. 4i + 3 take key i and a quarter of the list each, counting the
// keys below key i and those at most key i, then add their counts.  The key
// whose range [less, leq) holds rank rem is the boundary key t_k, and
// rem - less is the number of its ties ranked before the boundary; every lane
// holding t_k writes the same two values.  rem is read by the caller before
// any thread can write *rem_out.
__device__ __forceinline__ void rank_in_list(const uint32_t* list, int32_t n, int t, int32_t rem,
                                             uint32_t* prefix_out, int32_t* rem_out) {
  const int i = t >> 2, q = t & 3;
  const int32_t m = ((n + 15) >> 4) << 2;   // quarter length, a multiple of 4 (slots past n hold kPad)
  const uint32_t x = i < n ? list[i] : kPad;
  const uint32_t* part = list + q * m;
  int32_t less = 0, leq = 0;
  for (int r = 0; r < m; r += 4) {
    const u32x4 y = *reinterpret_cast<const u32x4*>(&part[r]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      less += y[e] < x ? 1 : 0;
      leq += y[e] <= x ? 1 : 0;
    }
  }
  // the four lanes of key i: quad permutations [1,0,3,2] then [2,3,0,1]
  less += __builtin_amdgcn_update_dpp(0, less, 0xb1, 0xf, 0xf, false);
  leq += __builtin_amdgcn_update_dpp(0, leq, 0xb1, 0xf, 0xf, false);
  less += __builtin_amdgcn_update_dpp(0, less, 0x4e, 0xf, 0xf, false);
  leq += __builtin_amdgcn_update_dpp(0, leq, 0x4e, 0xf, 0xf, false);
  if (q == 0 && i < n && less <= rem && rem < leq) {
    *prefix_out = x;
    *rem_out = rem - less;
  }
}

// Rows of up to 32768 tokens, keys in registers (thread t holds tokens
// 4 (t + 1024 j) + e), NB = K - 1 group boundaries known at compile time.
// Each workgroup takes rows blockIdx.x, blockIdx.x + gridDim.x, ...  Per row:
//  1. The smallest and largest key give the bits every key shares; the digit
//     passes start below them, so a narrow score distribution spreads over
//     the first pass's 2048 bins instead of a handful.
//  2. First pass: every key into one histogram (kept as four copies by lane
//     so that lanes of a wavefront collide less), serving every boundary.
//  3. While a boundary's bucket holds more than kList keys, another digit
//     pass over the registers, counting only the bucket's keys.
//  4. Then one sweep copies each boundary's bucket keys to an LDS list, and
//     wavefront k finishes boundary k from its list (finish_bucket): t_k is
//     the key at the boundary's rank and need_k the number of keys equal to
//     t_k that rank before it.
//  5. Assignment: group = number of boundaries whose key the token's key
//     reaches, ties with t_k split by their index-order position.
template <int NB>
__global__ __launch_bounds__(kThreads) void select_reg_kernel(const float* __restrict__ score,
                                                              int32_t B, int32_t N, Counts cnt,
                                                              uint8_t* __restrict__ group_out) {
  constexpr int kHist = NB > kCopies ? NB : kCopies;
  __shared__ int32_t hist[kHist][kBins];   // first pass: copies by lane; later: one per boundary
  __shared__ uint32_t s_list[NB][kList];
  __shared__ int32_t s_nlist[NB];
  __shared__ uint32_t s_small[NB][kWave];
  __shared__ int32_t wave_tmp[kWaves];
  __shared__ uint32_t red_min[kWaves], red_max[kWaves];
  __shared__ int32_t tie_pre[kV * kWaves];
  __shared__ uint32_t s_prefix[NB];   // key bits of boundary k's bucket (bits fixed so far)
  __shared__ int32_t s_rem[NB];       // the boundary's rank inside that bucket
  __shared__ int32_t s_size[NB];      // keys in that bucket
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto live = [&](int k) { return cnt.bound[k] < N; };   // a boundary at N: no token passes it

  for (int32_t b = blockIdx.x; b < B; b += gridDim.x) {
    // ---- this row's keys
    uint32_t key[kV][4];
    load_row_bits(score + (size_t)b * N, N, key);
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int32_t left = N - 4 * (tid + j * kThreads);   // tokens of this chunk inside the row
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j][e] = desc_key(__uint_as_float(key[j][e])) | (e < left ? 0u : kPad);
    }
    uint32_t kmin = kPad, kmax = 0u;
#pragma unroll
    for (int j = 0; j < kV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key[j][e] != kPad) {
          kmin = min(kmin, key[j][e]);
          kmax = max(kmax, key[j][e]);
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, kWave));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, kWave));
    }
    if (lane == 0) {
      red_min[wave] = kmin;
      red_max[wave] = kmax;
    }
#pragma unroll
    for (int c = 0; c < kCopies; ++c)
      for (int i = tid; i < kBins; i += kThreads) hist[c][i] = 0;
    if (tid < NB) {
      s_rem[tid] = cnt.bound[tid];
      s_size[tid] = N;
      s_nlist[tid] = 0;
    }
    __syncthreads();
    kmin = red_min[0];
    kmax = red_max[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      kmin = min(kmin, red_min[w]);
      kmax = max(kmax, red_max[w]);
    }
    // Slots past the row's end take the row's largest key: they sit after
    // every token (index >= N), so they rank after every real key equal to
    // it, and every boundary rank is < N: t_k and need_k are unchanged, and
    // no pass needs to tell them apart.  They are never stored.
#pragma unroll
    for (int j = 0; j < kV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j][e] = key[j][e] == kPad ? kmax : key[j][e];
    // bits below `lo` still differ between keys; every key has kmin's bits above
    const uint32_t diff = kmin ^ kmax;
    int lo = diff == 0u ? 0 : 32 - __clz(diff);
    uint32_t fixed = lo == 32 ? 0u : ~((1u << lo) - 1u);
    if (tid < NB) s_prefix[tid] = kmin & fixed;

    // ---- first pass over every key (all keys share the fixed bits)
    if (lo > 0) {
      const int width = lo < 11 ? lo : 11;
      const int sh = lo - width;
      const uint32_t dm = (1u << width) - 1u;
      int32_t* h = hist[lane & (kCopies - 1)];
#pragma unroll
      for (int j = 0; j < kV; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          atomicAdd(&h[(key[j][e] >> sh) & dm], 1);
      __syncthreads();
      int32_t h0 = 0, h1 = 0;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) {
        h0 += hist[c][2 * tid];
        h1 += hist[c][2 * tid + 1];
      }
      int32_t tot;
      const int32_t before = block_exclusive_scan(h0 + h1, wave_tmp, &tot);
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (live(k)) take_bucket(before, h0, h1, cnt.bound[k], sh, &s_prefix[k], &s_rem[k], &s_size[k]);
      fixed |= dm << sh;
      lo = sh;
    }
    __syncthreads();

    // ---- further passes over the registers while a bucket is larger than its
    // list; every live boundary narrows in each pass (they share `fixed`)
    while (lo > 0) {
      bool big[NB];
      uint32_t pre[NB];
      int32_t rem[NB];
      bool any = false;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        any = any || (live(k) && __builtin_amdgcn_readfirstlane(s_size[k]) > kList);
        big[k] = live(k);
        pre[k] = __builtin_amdgcn_readfirstlane(s_prefix[k]);
        rem[k] = __builtin_amdgcn_readfirstlane(s_rem[k]);
      }
      if (!any) break;
      const int width = lo < 11 ? lo : 11;
      const int sh = lo - width;
      const uint32_t dm = (1u << width) - 1u;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (big[k])
          for (int i = tid; i < kBins; i += kThreads) hist[k][i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kV; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t m = key[j][e] & fixed;
#pragma unroll
          for (int k = 0; k < NB; ++k)
            if (big[k] && m == pre[k]) atomicAdd(&hist[k][(key[j][e] >> sh) & dm], 1);
        }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (!big[k]) continue;   // uniform
        const int32_t h0 = hist[k][2 * tid], h1 = hist[k][2 * tid + 1];
        int32_t tot;
        const int32_t before = block_exclusive_scan(h0 + h1, wave_tmp, &tot);
        take_bucket(before, h0, h1, rem[k], sh, &s_prefix[k], &s_rem[k], &s_size[k]);
      }
      __syncthreads();
      fixed |= dm << sh;
      lo = sh;
    }

    // ---- every bucket holds at most kList keys, or every bit is fixed:
    // copy the buckets' keys to their lists: per chunk of 4 keys a wavefront
    // counts its bucket keys (ballots), reserves that much room, then writes.
    if (lo > 0) {
      uint32_t pre[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) pre[k] = __builtin_amdgcn_readfirstlane(s_prefix[k]);
#pragma unroll
      for (int j = 0; j < kV; ++j)
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          if (!live(k)) continue;
          uint64_t bal[4];
          int32_t cnt = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bal[e] = __ballot((key[j][e] & fixed) == pre[k]);
            cnt += __popcll(bal[e]);
          }
          if (cnt == 0) continue;   // uniform
          int32_t at = 0;
          if (lane == 0) at = atomicAdd(&s_nlist[k], cnt);
          at = __shfl(at, 0, kWave);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((bal[e] >> lane) & 1ull) s_list[k][at + __popcll(bal[e] & lt_mask)] = key[j][e];
            at += __popcll(bal[e]);
          }
        }
      __syncthreads();
      // wavefront k finishes boundary k from its list, no workgroup barrier
      if (wave < NB && live(wave))
        finish_bucket(s_list[wave], s_nlist[wave], hist[wave], s_small[wave], fixed, lo,
                      &s_prefix[wave], &s_rem[wave]);
      __syncthreads();
    }

    // ---- assignment: every bit of each boundary's key is fixed
    uint32_t tk[NB];
    int32_t need[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      tk[k] = live(k) ? __builtin_amdgcn_readfirstlane(s_prefix[k]) : kPad;   // no key reaches kPad
      need[k] = live(k) ? __builtin_amdgcn_readfirstlane(s_rem[k]) : 0;
    }
    uint32_t gp[kV];   // 4 group bytes per chunk
#pragma unroll
    for (int j = 0; j < kV; ++j) gp[j] = 0u;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (need[k] == 0) {   // every tie with t_k ranks at or past the boundary
#pragma unroll
        for (int j = 0; j < kV; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) gp[j] += key[j][e] >= tk[k] ? 1u << (8 * e) : 0u;
        continue;
      }
      // ties per (chunk, wavefront): index order is chunk-major, then wavefront,
      // lane and element
#pragma unroll
      for (int j = 0; j < kV; ++j) {
        int32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) c += __popcll(__ballot(key[j][e] == tk[k]));
        if (lane == 0) tie_pre[j * kWaves + wave] = c;
      }
      __syncthreads();
      if (wave == 0) {   // exclusive scan of the kV * kWaves counts, 64 lanes over runs
        constexpr int E = kV * kWaves, PER = (E + kWave - 1) / kWave;
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
      for (int j = 0; j < kV; ++j) {
        int32_t before = tie_pre[j * kWaves + wave];
        bool eq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          eq[e] = key[j][e] == tk[k];
          before += __popcll(__ballot(eq[e]) & lt_mask);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ge = eq[e] ? before >= need[k] : key[j][e] > tk[k];
          gp[j] += ge ? 1u << (8 * e) : 0u;
          before += eq[e] ? 1 : 0;
        }
      }
      __syncthreads();   // tie_pre is reused by the next boundary
    }
    uint8_t* out = group_out + (size_t)b * N;
    const bool aligned4 = (reinterpret_cast<uintptr_t>(out) & 3u) == 0u;
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int32_t n = 4 * (tid + j * kThreads);
      if (n < N) store_groups(out, n, N, gp[j], aligned4);
    }
    __syncthreads();   // the shared state is reset for the next row
  }
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from a buffer straight into LDS at lds_addr + 16 * lane,
// after every LDS read of this wavefront has returned (the loads may land on
// what those reads were reading).  The instruction has no register result;
// its completion is waited for with vmcnt(0).
__device__ __forceinline__ void lds_dma16_after_reads(uint32_t lds_addr, uint32_t voff, i32x4_t rsrc) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// One or two group boundaries (K <= 3, every workload here), rows of up to
// 32768 tokens: the same passes as select_reg_kernel.  Each workgroup takes
// rows blockIdx.x, blockIdx.x + gridDim.x, ...; slots past a row's end take
// the row's largest key.  The next row is read while this one is ranked:
//  * DMA (rows 16-byte aligned): the next row's scores go straight from HBM
//    into LDS (token order, 128 KiB; each wavefront loads exactly the chunks
//    its own threads read back), and the row being ranked is held as keys in
//    registers, so no pass reads LDS for keys;
//  * otherwise: the next row's scores load into registers and the row being
//    ranked sits in LDS as keys, which every pass reads from there.
template <int NB, bool DMA>
__global__ __launch_bounds__(kThreads) void select_lds_kernel(const float* __restrict__ score,
                                                              int32_t B, int32_t N, Counts cnt,
                                                              uint8_t* __restrict__ group_out) {
  static_assert(NB >= 1 && NB <= 2, "LDS holds two boundaries' histograms and lists");
  __shared__ __attribute__((aligned(16))) uint32_t s_key[4 * kV * kThreads];   // keys, or (DMA) the next row's scores
  __shared__ int32_t hist[2][kBins];   // first pass: one histogram of 4096 bins; later: one per boundary
  __shared__ __attribute__((aligned(16))) uint32_t s_list[NB][kList];
  __shared__ uint32_t s_small[NB][kWave];
  __shared__ int32_t wave_tmp[kWaves];
  __shared__ uint32_t red_min[kWaves], red_max[kWaves];
  __shared__ int32_t tie_pre[kV * kWaves];
  __shared__ uint32_t s_prefix[NB];
  __shared__ int32_t s_rem[NB], s_size[NB], s_nlist[NB];
  // The bounds in scalar registers, opaque to the compiler: a bound picked by
  // a k that differs between wavefronts must not become a load from the
  // kernel arguments (that load would wait for every load and store in
  // flight, the next row's prefetch included).
  int32_t bnd[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    bnd[k] = cnt.bound[k];
    asm volatile("" : "+s"(bnd[k]));
  }
  auto live = [&](int k) { return bnd[k] < N; };   // a boundary at N: no token passes it
  auto bound_of = [&](int k) { return NB == 1 || k == 0 ? bnd[0] : bnd[NB - 1]; };

  uint32_t raw[kV][4];   // the next row's scores, or (DMA) this row's keys
  uint32_t gp[kV];   // group bytes of the previous row, 4 per chunk, stored once
                     // this row's scores have arrived (so that no wait for the
                     // next row's loads also waits for these stores)
  const uint32_t s_key_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)s_key;
  // DMA: row r's scores into s_key, each wavefront its own threads' chunks
  auto dma_row = [&](int32_t r) {
    const uint64_t a = reinterpret_cast<uint64_t>(score + (size_t)r * N);
    const i32x4_t rsrc = {(int32_t)(uint32_t)a, (int32_t)(uint32_t)(a >> 32), N * 4, 0x00020000};
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
#pragma unroll
    for (int j = 0; j < kV; ++j)
      lds_dma16_after_reads(s_key_lds + 16u * (uint32_t)(w * kWave + j * kThreads),
                            16u * (uint32_t)(threadIdx.x + j * kThreads), rsrc);
  };
  if (blockIdx.x < (uint32_t)B) {
    if constexpr (DMA) dma_row(blockIdx.x);
    else load_row_bits(score + (size_t)blockIdx.x * N, N, raw);
  }
  for (int32_t b = blockIdx.x; b < B; b += gridDim.x) {
    // The thread id is made opaque per row, so that the addresses derived
    // from it are recomputed in each row instead of held in registers across
    // the whole loop (which would spill, and every spill reload waits for
    // the next row's loads in flight).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    auto keys4 = [&](int j) {
      if constexpr (DMA) return u32x4{raw[j][0], raw[j][1], raw[j][2], raw[j][3]};
      else return *reinterpret_cast<const u32x4*>(&s_key[4 * (tid + j * kThreads)]);
    };
    if constexpr (DMA) {   // this row's scores, landed in LDS while the previous row was ranked
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < kV; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&s_key[4 * (tid + j * kThreads)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[j][e] = v[e];
      }
    }
    // ---- keys, the smallest and largest; (DMA) the next row's loads go out
    uint32_t kmin = kPad, kmax = 0u;
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      if (4 * (j + 1) * kThreads <= N) {   // uniform: the whole chunk lies inside the row
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[j][e] = desc_key(__uint_as_float(raw[j][e]));
        kmin = min(kmin, min(min(raw[j][0], raw[j][1]), min(raw[j][2], raw[j][3])));
        kmax = max(kmax, max(max(raw[j][0], raw[j][1]), max(raw[j][2], raw[j][3])));
        continue;
      }
      const int32_t left = N - 4 * (tid + j * kThreads);   // tokens of this chunk inside the row
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        raw[j][e] = desc_key(__uint_as_float(raw[j][e])) | (e < left ? 0u : kPad);
        if (raw[j][e] != kPad) {
          kmin = min(kmin, raw[j][e]);
          kmax = max(kmax, raw[j][e]);
        }
      }
    }
    if constexpr (DMA) {
      if (b + (int32_t)gridDim.x < B) dma_row(b + gridDim.x);
    }
    if (b != (int32_t)blockIdx.x) {
      // the stores take an address that depends on every key, so that they
      // issue after this row's scores have arrived
      int32_t after_keys = 0;
      asm volatile("" : "+v"(after_keys) : "v"(kmin), "v"(kmax));
      uint8_t* prev = group_out + (size_t)(b - gridDim.x) * N + after_keys;
      const bool aligned4 = (reinterpret_cast<uintptr_t>(prev) & 3u) == 0u;
#pragma unroll
      for (int j = 0; j < kV; ++j) {
        const int32_t n = 4 * (tid + j * kThreads);
        if (aligned4 && 4 * (j + 1) * kThreads <= N)   // uniform
          *reinterpret_cast<uint32_t*>(prev + n) = gp[j];
        else if (n < N)
          store_groups(prev, n, N, gp[j], aligned4);
      }
    }
    wave_min_max(kmin, kmax);
    if (lane == 0) {
      red_min[wave] = kmin;
      red_max[wave] = kmax;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
      for (int i = tid; i < kBins; i += kThreads) hist[c][i] = 0;
#pragma unroll
    for (int k = 0; k < NB; ++k)
      for (int i = tid; i < kList; i += kThreads) s_list[k][i] = kPad;   // slots past a bucket's size
    if (tid < NB) {
      s_rem[tid] = bound_of(tid);
      s_size[tid] = N;
      s_nlist[tid] = 0;
    }
    __syncthreads();
    kmin = red_min[0];
    kmax = red_max[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      kmin = min(kmin, red_min[w]);
      kmax = max(kmax, red_max[w]);
    }
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      u32x4 v;
      const bool whole = 4 * (j + 1) * kThreads <= N;   // uniform
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (!whole && raw[j][e] == kPad) ? kmax : raw[j][e];
      if constexpr (DMA) {
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[j][e] = v[e];
      } else {
        *reinterpret_cast<u32x4*>(&s_key[4 * (tid + j * kThreads)]) = v;
      }
    }
    if constexpr (!DMA)
      if (b + (int32_t)gridDim.x < B) load_row_bits(score + (size_t)(b + gridDim.x) * N, N, raw);
    // bits below `lo` still differ between keys; every key has kmin's bits above
    const uint32_t diff = kmin ^ kmax;
    int lo = diff == 0u ? 0 : 32 - __clz(diff);
    uint32_t fixed = lo == 32 ? 0u : ~((1u << lo) - 1u);
    if (tid < NB) s_prefix[tid] = kmin & fixed;
    __syncthreads();

    // ---- first pass over every key: a 12-bit digit, both halves of `hist`
    // as one histogram of 4096 bins
    if (lo > 0) {
      const int width = lo < 12 ? lo : 12;
      const int sh = lo - width;
      const uint32_t dm = (1u << width) - 1u;
      int32_t* h = &hist[0][0];
#pragma unroll
      for (int j = 0; j < kV; ++j) {
        const u32x4 v = keys4(j);
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(&h[(v[e] >> sh) & dm], 1);
      }
      __syncthreads();
      const i32x4_t h4 = *reinterpret_cast<const i32x4_t*>(&h[4 * tid]);
      const int32_t hb[4] = {h4[0], h4[1], h4[2], h4[3]};
      int32_t tot;
      const int32_t before = block_exclusive_scan((hb[0] + hb[1]) + (hb[2] + hb[3]), wave_tmp, &tot);
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (live(k)) take_bucket4(before, hb, bnd[k], sh, &s_prefix[k], &s_rem[k], &s_size[k]);
      fixed |= dm << sh;
      lo = sh;
    }
    __syncthreads();

    // ---- further passes while a bucket is too large to be ranked directly
    // (four threads per key; every live boundary narrows in each pass, as
    // they share `fixed`)
    while (lo > 0) {
      uint32_t pre[NB];
      int32_t rem[NB];
      bool any = false;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        any = any || (live(k) && 4 * __builtin_amdgcn_readfirstlane(s_size[k]) > kThreads / NB);
        pre[k] = __builtin_amdgcn_readfirstlane(s_prefix[k]);
        rem[k] = __builtin_amdgcn_readfirstlane(s_rem[k]);
      }
      if (!any) break;
      const int width = lo < 11 ? lo : 11;
      const int sh = lo - width;
      const uint32_t dm = (1u << width) - 1u;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        for (int i = tid; i < kBins; i += kThreads) hist[k][i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kV; ++j) {
        const u32x4 v = keys4(j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int k = 0; k < NB; ++k)
            if (live(k) && (v[e] & fixed) == pre[k]) atomicAdd(&hist[k][(v[e] >> sh) & dm], 1);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (!live(k)) continue;   // uniform
        const int32_t h0 = hist[k][2 * tid], h1 = hist[k][2 * tid + 1];
        int32_t tot;
        const int32_t before = block_exclusive_scan(h0 + h1, wave_tmp, &tot);
        take_bucket(before, h0, h1, rem[k], sh, &s_prefix[k], &s_rem[k], &s_size[k]);
      }
      __syncthreads();
      fixed |= dm << sh;
      lo = sh;
    }

    // ---- the buckets' keys to their lists: per chunk of 4 keys a wavefront
    // counts its bucket keys (ballots), reserves that much room, then writes;
    // then each boundary's bucket is ranked (the bucket's size is s_size)
    if (lo > 0) {
      uint32_t pre[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) pre[k] = __builtin_amdgcn_readfirstlane(s_prefix[k]);
      const uint32_t span = lo == 32 ? 0xffffffffu : 1u << lo;   // lo == 32: no bit fixed, every key
#pragma unroll
      for (int j = 0; j < kV; ++j) {
        const u32x4 v = keys4(j);
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          if (!live(k)) continue;   // uniform
          bool in[4];
          uint64_t bal[4];
          int32_t c = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            in[e] = v[e] - pre[k] < span;   // the bucket: keys pre[k] .. pre[k] + span - 1
            bal[e] = __ballot(in[e]);
            c += __popcll(bal[e]);
          }
          if (c == 0) continue;   // uniform
          int32_t at = lds_reserve(&s_nlist[k], c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (in[e]) s_list[k][at + lanes_below(bal[e])] = v[e];
            at += __popcll(bal[e]);
          }
        }
      }
      // boundary k takes threads k * kThreads / NB ..: a bucket of up to a
      // quarter as many keys is ranked by comparing every pair, a larger one
      // by the part's first wavefront in digit passes
      constexpr int kPart = kThreads / NB;
      const int kb = tid / kPart, t = tid % kPart;
      const int32_t rem = __builtin_amdgcn_readfirstlane(s_rem[kb]);   // before any thread rewrites it
      __syncthreads();
      const int32_t n = __builtin_amdgcn_readfirstlane(s_nlist[kb]);
      if (bound_of(kb) < N) {
        if (4 * n <= kPart) {
          if (t < ((4 * n + kWave - 1) & ~(kWave - 1)))   // wavefronts holding a key
            rank_in_list(s_list[kb], n, t, rem, &s_prefix[kb], &s_rem[kb]);
        } else if (t < kWave) {
          finish_bucket(s_list[kb], n, hist[kb], s_small[kb], fixed, lo, &s_prefix[kb], &s_rem[kb]);
        }
      }
      __syncthreads();
    }

    // ---- assignment: every bit of each boundary's key is fixed.  A key
    // passes boundary k if it is above t_k, or equals t_k and does not rank
    // among the first need[k] ties (index order); with need[k] == 0 every
    // tie passes, so one compare per boundary settles every key.
    uint32_t tk[NB], thr[NB];
    int32_t need[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      tk[k] = live(k) ? __builtin_amdgcn_readfirstlane(s_prefix[k]) : kPad;   // no key reaches kPad
      need[k] = live(k) ? __builtin_amdgcn_readfirstlane(s_rem[k]) : 0;
      thr[k] = need[k] == 0 ? tk[k] : tk[k] + 1u;   // ties counted apart below
    }
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const u32x4 v = keys4(j);
      uint32_t g = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t c = 0u;
#pragma unroll
        for (int k = 0; k < NB; ++k) c += v[e] >= thr[k] ? 1u : 0u;
        g |= c << (8 * e);
      }
      gp[j] = g;
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (need[k] == 0) continue;   // uniform
      // ties per (chunk, wavefront): index order is chunk-major, then wavefront,
      // lane and element
#pragma unroll
      for (int j = 0; j < kV; ++j) {
        const u32x4 v = keys4(j);
        int32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) c += __popcll(__ballot(v[e] == tk[k]));
        if (lane == 0) tie_pre[j * kWaves + wave] = c;
      }
      __syncthreads();
      if (wave == 0) {   // exclusive scan of the kV * kWaves counts, 64 lanes over runs
        constexpr int E = kV * kWaves, PER = (E + kWave - 1) / kWave;
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
      for (int j = 0; j < kV; ++j) {
        const u32x4 v = keys4(j);
        int32_t before = tie_pre[j * kWaves + wave];
        bool eq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          eq[e] = v[e] == tk[k];
          before += __popcll(__ballot(eq[e]) & lt_mask);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gp[j] += (eq[e] && before >= need[k]) ? 1u << (8 * e) : 0u;
          before += eq[e] ? 1 : 0;
        }
      }
      __syncthreads();   // tie_pre is reused by the next boundary
    }
    __syncthreads();   // the shared state (keys included) is rewritten for the next row
  }
  // the last row's groups
  const int32_t last = blockIdx.x + ((B - 1 - (int32_t)blockIdx.x) / (int32_t)gridDim.x) * gridDim.x;
  if ((int32_t)blockIdx.x < B) {
    uint8_t* out = group_out + (size_t)last * N;
    const bool aligned4 = (reinterpret_cast<uintptr_t>(out) & 3u) == 0u;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int32_t n = 4 * (tid + j * kThreads);
      if (aligned4 && 4 * (j + 1) * kThreads <= N)   // uniform
        *reinterpret_cast<uint32_t*>(out + n) = gp[j];
      else if (n < N)
        store_groups(out, n, N, gp[j], aligned4);
    }
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

// ---------------------------------------------------------------- two rows per CU
// Batches of more rows than CUs (K <= 3, rows of up to 16384 * 2 tokens):
// two 512-thread workgroups per CU, each ranking its own row with 64 keys
// per thread in registers (thread t holds tokens 4 (t + 512 j) + e).  While
// one workgroup waits (its row's loads, a barrier, a block-wide scan, the
// ranking of a bucket) the other's sweeps keep the SIMDs busy.  The passes
// are those of select_lds_kernel: a 12-bit first digit below the row's
// shared key bits, 11-bit passes while a bucket is too large to rank
// directly, the buckets' keys to LDS lists ranked by two threads per key,
// one compare per key and boundary to assign, ties at t_k by index.
namespace two {

constexpr int kT = 512;
constexpr int kW = kT / kWave;       // wavefronts per workgroup
constexpr int kC = 16;               // 16-byte chunks per thread: rows of up to 4 kC kT = 32768 tokens
constexpr int kFirstBits = 14;       // first pass: 16384 bins (64 KB); later passes 2048 per boundary
constexpr int kBins = 1 << kFirstBits;
constexpr int kBinsPerThread = kBins / kT;   // 32, read as 8 16-byte vectors
constexpr int kL = 512;              // list slots per boundary

// 16-byte buffer loads of a row's raw score bits (zero past its 4N bytes);
// 4-byte loads when the row is not 16-byte aligned.
__device__ __forceinline__ void load_row(const float* row, int32_t N, uint32_t (&raw)[kC][4]) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, N * 4, 0x00020000);
  const int tid = threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0u) {
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * (tid + j * kT), 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[j][e] = v[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kC; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        raw[j][e] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, 16 * (tid + j * kT) + 4 * e, 0, 0);
  }
}

// A key whose ascending order is the score's descending order, as desc_key
// but with other codes: the negated score, both zeros as +0 (0 - f) and NaN as
// the negation of +inf (maxNum drops the NaN), mapped monotonically to an
// unsigned integer.  Two VALU float operations and two integer ones.
__device__ __forceinline__ uint32_t neg_key(float f) {
  float h;
  // written out: the compiler folds 0 - f into -f below maxNum (which may
  // take either zero) and would quiet the difference again before the max
  asm("v_sub_f32 %0, 0, %1\n\tv_max_f32 %0, 0xff800000, %0" : "=&v"(h) : "v"(f));
  const uint32_t u = __float_as_uint(h);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// 1 when x >= a + 1, else 0, for a < 0xffffffff: med3(x, a, a + 1) - a, with
// no carry flag (a compare and add-with-carry needs hazard wait states).
__device__ __forceinline__ uint32_t med3_u32(uint32_t x, uint32_t a, uint32_t a1) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(a), "v"(a1));
  return r;
}

// Exclusive prefix over the workgroup's threads (thread order) and the total.
__device__ int32_t block_scan(int32_t v, int32_t* wave_tmp, int32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int32_t inc = wave_incl_scan(v);
  if (lane == kWave - 1) wave_tmp[wave] = inc;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int32_t c = wave_tmp[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// rank_in_list with two threads per key: lanes 2i, 2i + 1 take key i and half
// of the list each (slots from n on hold kPad).
__device__ __forceinline__ void rank_in_list2(const uint32_t* list, int32_t n, int t, int32_t rem,
                                              uint32_t* prefix_out, int32_t* rem_out) {
  const int i = t >> 1, q = t & 1;
  const int32_t m = ((n + 7) >> 3) << 2;   // half length, a multiple of 4
  const uint32_t x = i < n ? list[i] : kPad;
  const uint32_t* part = list + q * m;
  int32_t less = 0, leq = 0;
  for (int r = 0; r < m; r += 4) {   // r uniform
    const u32x4 y = *reinterpret_cast<const u32x4*>(&part[r]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      less += y[e] < x ? 1 : 0;
      leq += y[e] <= x ? 1 : 0;
    }
  }
  // the two lanes of key i: quad permutation [1,0,3,2]
  less += __builtin_amdgcn_update_dpp(0, less, 0xb1, 0xf, 0xf, false);
  leq += __builtin_amdgcn_update_dpp(0, leq, 0xb1, 0xf, 0xf, false);
  if (q == 0 && i < n && less <= rem && rem < leq) {
    *prefix_out = x;
    *rem_out = rem - less;
  }
}

// Bucket of this thread's first-pass bins (kBinsPerThread t onward; bin i
// holds the keys with key >> sh == first + i) that holds rank rem, for the one
// thread whose bins hold it: the 4-bin group first, then the bin inside it
// (two rounds of reads, not one per bin).
__device__ void take_bucket_first(const int32_t* hist, int32_t before, int32_t rem, uint32_t first,
                                  int sh, uint32_t* prefix, int32_t* rem_out, int32_t* size_out) {
  const int tid = threadIdx.x;
  const int32_t* mine = hist + kBinsPerThread * tid;
  int32_t gsum[kBinsPerThread / 4];
#pragma unroll
  for (int g = 0; g < kBinsPerThread / 4; ++g) {
    const i32x4_t v = *reinterpret_cast<const i32x4_t*>(&mine[4 * g]);
    gsum[g] = (v[0] + v[1]) + (v[2] + v[3]);
  }
  int32_t run = before, grp = 0;
#pragma unroll
  for (int g = 0; g < kBinsPerThread / 4 - 1; ++g) {
    const bool past = run + gsum[g] <= rem;   // rank rem lies after group g
    grp += past ? 1 : 0;
    run += past ? gsum[g] : 0;
    if (!past) break;
  }
  const i32x4_t v = *reinterpret_cast<const i32x4_t*>(&mine[4 * grp]);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q == 3 || rem < run + v[q]) {
      *prefix = (first + (uint32_t)(kBinsPerThread * tid + 4 * grp + q)) << sh;
      *rem_out = rem - run;
      *size_out = v[q];
      return;
    }
    run += v[q];
  }
}

template <int NB>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(4))) void select_two_kernel(const float* __restrict__ score,
                                                           int32_t B, int32_t N, Counts cnt,
                                                           uint8_t* __restrict__ group_out) {
  static_assert(NB >= 1 && NB <= 2, "two boundaries' histograms fit the first pass's bins");
  __shared__ __attribute__((aligned(16))) int32_t hist[kBins];
  __shared__ __attribute__((aligned(16))) uint32_t s_list[NB][kL];
  __shared__ int32_t wave_tmp[kW];
  __shared__ uint32_t red_min[kW], red_max[kW];
  __shared__ int32_t tie_pre[kC * kW];
  __shared__ uint32_t s_prefix[NB];
  __shared__ int32_t s_rem[NB], s_size[NB], s_nlist[NB];
  constexpr int kPart = kT / NB;        // threads per boundary when ranking
  constexpr int kRankMax = kPart / 2;   // a bucket ranked directly: two threads per key
  static_assert(2 * ((kRankMax + 7) / 8) * 4 <= kL, "list slots cover both halves");
  int32_t bnd[NB];   // the bounds in scalar registers (see select_lds_kernel)
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    bnd[k] = cnt.bound[k];
    asm volatile("" : "+s"(bnd[k]));
  }
  auto live = [&](int k) { return bnd[k] < N; };
  auto bound_of = [&](int k) { return NB == 1 || k == 0 ? bnd[0] : bnd[NB - 1]; };

  for (int32_t b = blockIdx.x; b < B; b += gridDim.x) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t key[kC][4];
    load_row(score + (size_t)b * N, N, key);
    // chunks wholly inside the row: recomputed per row (kept opaque), not
    // sixteen flags held across the loop
    int32_t nfull = N / (4 * kT);
    asm volatile("" : "+s"(nfull));
    // ---- keys, the smallest and largest.  First 0x7fffffff - bits, one
    // instruction, the key of a score in [+0, +inf] (larger score, smaller
    // key, from kFastMin for +inf to kFastMax for +0); a row holding a
    // negative score, -0 or NaN shows in its range and is keyed again below.
    constexpr uint32_t kFastMin = 0x7fffffffu - 0x7f800000u, kFastMax = 0x7fffffffu;
    uint32_t kmin = kPad, kmax = 0u;
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      if (j < nfull) {   // uniform: the whole chunk lies inside the row
#pragma unroll
        for (int e = 0; e < 4; ++e) key[j][e] = kFastMax - key[j][e];
        kmin = min(kmin, min(min(key[j][0], key[j][1]), min(key[j][2], key[j][3])));
        kmax = max(kmax, max(max(key[j][0], key[j][1]), max(key[j][2], key[j][3])));
        continue;
      }
      const int32_t left = N - 4 * (tid + j * kT);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (e < left) {
          key[j][e] = kFastMax - key[j][e];
          kmin = min(kmin, key[j][e]);
          kmax = max(kmax, key[j][e]);
        } else {
          key[j][e] = kPad;
        }
      }
    }
    wave_min_max(kmin, kmax);
    if (lane == 0) {
      red_min[wave] = kmin;
      red_max[wave] = kmax;
    }
#pragma unroll
    for (int i = 0; i < kBins / (4 * kT); ++i)   // consecutive lanes, consecutive 16 bytes
      *reinterpret_cast<i32x4_t*>(&hist[4 * (i * kT + tid)]) = i32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < NB; ++k) s_list[k][tid] = kPad;   // slots past a bucket's size
    if (tid < NB) {
      s_rem[tid] = bound_of(tid);
      s_size[tid] = N;
      s_nlist[tid] = 0;
    }
    __syncthreads();
    kmin = red_min[0];
    kmax = red_max[0];
#pragma unroll
    for (int w = 1; w < kW; ++w) {
      kmin = min(kmin, red_min[w]);
      kmax = max(kmax, red_max[w]);
    }
    if (kmin < kFastMin || kmax > kFastMax) {   // uniform: keys of every score
      uint32_t mn = kPad, mx = 0u;
#pragma unroll
      for (int j = 0; j < kC; ++j) {
        const int32_t left = j < nfull ? 4 : N - 4 * (tid + j * kT);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e < left) {
            key[j][e] = neg_key(__uint_as_float(kFastMax - key[j][e]));
            mn = min(mn, key[j][e]);
            mx = max(mx, key[j][e]);
          }
        }
      }
      wave_min_max(mn, mx);
      __syncthreads();   // every wavefront has read the first range
      if (lane == 0) {
        red_min[wave] = mn;
        red_max[wave] = mx;
      }
      __syncthreads();
      kmin = red_min[0];
      kmax = red_max[0];
#pragma unroll
      for (int w = 1; w < kW; ++w) {
        kmin = min(kmin, red_min[w]);
        kmax = max(kmax, red_max[w]);
      }
    }
#pragma unroll
    for (int j = 0; j < kC; ++j)
      if (j >= nfull)   // uniform: slots past the row's end take its largest key
#pragma unroll
        for (int e = 0; e < 4; ++e) key[j][e] = key[j][e] == kPad ? kmax : key[j][e];
    kmin = __builtin_amdgcn_readfirstlane(kmin);
    kmax = __builtin_amdgcn_readfirstlane(kmax);
    // the bucket that holds a boundary is the keys with one value of
    // key >> lo: its bits above lo are `fixed`
    int lo = 0;
    uint32_t fixed = ~0u;
    if (tid < NB) s_prefix[tid] = kmin;   // every key equal: no pass

    // ---- first pass over every key: bin (key >> sh) - (kmin >> sh) of
    // kBins, sh the least shift that fits kmin .. kmax into them (so the bins
    // follow the keys' actual range, not their common bit prefix)
    if (kmin != kmax) {
      int sh = 32 - __clz(kmax - kmin) - kFirstBits;
      sh = sh < 0 ? 0 : sh;
      if ((kmax >> sh) - (kmin >> sh) >= (uint32_t)kBins) ++sh;
      const uint32_t first = kmin >> sh;
      // LDS byte address of bin (key >> sh) - first: one shift-and-add per key
      uint32_t at0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int32_t*)hist - 4u * first;
      asm volatile("" : "+s"(at0));   // kept an addend: one v_lshl_add per key
#pragma unroll
      for (int j = 0; j < kC; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __hip_atomic_fetch_add((__attribute__((address_space(3))) int32_t*)(uintptr_t)(at0 + 4u * (key[j][e] >> sh)),
                                 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __syncthreads();
      // this thread's bins, read in a lane-rotated order (the sum does not
      // care) so that one read spreads over the banks
      int32_t mine = 0;
#pragma unroll
      for (int i = 0; i < kBinsPerThread / 4; ++i) {
        const int r = (i + tid) & (kBinsPerThread / 4 - 1);
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(&hist[kBinsPerThread * tid + 4 * r]);
        mine += (v[0] + v[1]) + (v[2] + v[3]);
      }
      int32_t tot;
      const int32_t before = block_scan(mine, wave_tmp, &tot);
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (live(k) && before <= bnd[k] && bnd[k] < before + mine)
          take_bucket_first(hist, before, bnd[k], first, sh, &s_prefix[k], &s_rem[k], &s_size[k]);
      fixed = ~0u << sh;   // sh <= 19: the range spans at most 2^32 keys
      lo = sh;
    }
    __syncthreads();

    // ---- further passes while a bucket is too large to rank directly (every
    // live boundary narrows in each, as they share `fixed`)
    while (lo > 0) {
      uint32_t pre[NB];
      int32_t rem[NB];
      bool any = false;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        any = any || (live(k) && __builtin_amdgcn_readfirstlane(s_size[k]) > kRankMax);
        pre[k] = __builtin_amdgcn_readfirstlane(s_prefix[k]);
        rem[k] = __builtin_amdgcn_readfirstlane(s_rem[k]);
      }
      if (!any) break;
      const int width = lo < 11 ? lo : 11;
      const int sh = lo - width;
      const uint32_t dm = (1u << width) - 1u;
#pragma unroll
      for (int i = 0; i < NB * 2048 / (4 * kT); ++i)
        *reinterpret_cast<i32x4_t*>(&hist[4 * (i * kT + tid)]) = i32x4_t{0, 0, 0, 0};
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kC; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int k = 0; k < NB; ++k)
            if (live(k) && (key[j][e] & fixed) == pre[k]) atomicAdd(&hist[k * 2048 + ((key[j][e] >> sh) & dm)], 1);
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (!live(k)) continue;   // uniform
        const i32x4_t hv = *reinterpret_cast<const i32x4_t*>(&hist[k * 2048 + 4 * tid]);
        const int32_t h4[4] = {hv[0], hv[1], hv[2], hv[3]};
        int32_t tot;
        const int32_t before = block_scan((h4[0] + h4[1]) + (h4[2] + h4[3]), wave_tmp, &tot);
        take_bucket4(before, h4, rem[k], sh, &s_prefix[k], &s_rem[k], &s_size[k]);
      }
      __syncthreads();
      fixed |= dm << sh;
      lo = sh;
    }

    // ---- the buckets' keys to their lists (room reserved per chunk of 4
    // keys and wavefront), then each boundary's bucket ranked by two threads
    // per key
    if (lo > 0) {
      uint32_t top[NB];   // a bucket is the keys with one value of key >> lo
#pragma unroll
      for (int k = 0; k < NB; ++k) top[k] = (uint32_t)__builtin_amdgcn_readfirstlane(s_prefix[k]) >> lo;
#pragma unroll
      for (int j = 0; j < kC; ++j) {
        uint32_t kt[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) kt[e] = key[j][e] >> lo;   // lo < 32 after the first pass
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          if (!live(k)) continue;   // uniform
          bool in[4];
          uint64_t bal[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            in[e] = kt[e] == top[k];
            bal[e] = __ballot(in[e]);
          }
          if ((bal[0] | bal[1] | bal[2] | bal[3]) == 0ull) continue;   // uniform: the common case
          const int32_t c = (__popcll(bal[0]) + __popcll(bal[1])) + (__popcll(bal[2]) + __popcll(bal[3]));
          int32_t at = lds_reserve(&s_nlist[k], c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (bal[e] == 0ull) continue;   // uniform: no write issued for an empty element
            if (in[e]) s_list[k][at + lanes_below(bal[e])] = key[j][e];
            at += __popcll(bal[e]);
          }
        }
      }
      const int kb = tid / kPart, t = tid % kPart;
      const int32_t rem = __builtin_amdgcn_readfirstlane(s_rem[kb]);   // before any thread rewrites it
      __syncthreads();
      const int32_t n = __builtin_amdgcn_readfirstlane(s_nlist[kb]);
      if (bound_of(kb) < N && t < ((2 * n + kWave - 1) & ~(kWave - 1)))   // wavefronts holding a key
        rank_in_list2(s_list[kb], n, t, rem, &s_prefix[kb], &s_rem[kb]);
      __syncthreads();
    }

    // ---- assignment (as in select_lds_kernel)
    // key >= thr[k] counts boundary k (thr >= 1: keys of scores are at least
    // 0x007fffff in either form, a dead boundary's thr is kPad), as
    // med3(key, thr - 1, thr) - (thr - 1)
    uint32_t tk[NB], am[NB], ap[NB], asum = 0u;
    int32_t need[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      tk[k] = live(k) ? __builtin_amdgcn_readfirstlane(s_prefix[k]) : kPad;
      need[k] = live(k) ? __builtin_amdgcn_readfirstlane(s_rem[k]) : 0;
      const uint32_t thr = need[k] == 0 ? tk[k] : tk[k] + 1u;
      am[k] = thr - 1u;
      ap[k] = thr;
      asum += am[k];
    }
    // the four bytes at once: sum of med3 << 8e, less asum in every byte
    // (modulo 2^32; each byte's true sum is at most NB)
    uint32_t gp[kC];
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      uint32_t g = 0u - asum * 0x01010101u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int k = 0; k < NB; ++k) g += med3_u32(key[j][e], am[k], ap[k]) << (8 * e);
      gp[j] = g;
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (need[k] == 0) continue;   // uniform
      // ties per (chunk, wavefront): index order is chunk-major, then
      // wavefront, lane and element
#pragma unroll
      for (int j = 0; j < kC; ++j) {
        int32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) c += __popcll(__ballot(key[j][e] == tk[k]));
        if (lane == 0) tie_pre[j * kW + wave] = c;
      }
      __syncthreads();
      if (wave == 0) {   // exclusive scan of the kC * kW counts, 64 lanes over runs
        constexpr int E = kC * kW, PER = (E + kWave - 1) / kWave;
        int32_t v[PER], sum = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int i = lane * PER + q;
          v[q] = i < E ? tie_pre[i] : 0;
          sum += v[q];
        }
        const int32_t inc = wave_incl_scan(sum);
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
      for (int j = 0; j < kC; ++j) {
        int32_t before = tie_pre[j * kW + wave];
        bool eq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          eq[e] = key[j][e] == tk[k];
          before += __popcll(__ballot(eq[e]) & lt_mask);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gp[j] += (eq[e] && before >= need[k]) ? 1u << (8 * e) : 0u;
          before += eq[e] ? 1 : 0;
        }
      }
      __syncthreads();   // tie_pre is reused by the next boundary
    }
    uint8_t* out = group_out + (size_t)b * N;
    const bool aligned4 = (reinterpret_cast<uintptr_t>(out) & 3u) == 0u;
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const int32_t n = 4 * (tid + j * kT);
      if (aligned4 && j < nfull)   // uniform
        *reinterpret_cast<uint32_t*>(out + n) = gp[j];
      else if (n < N)
        store_groups(out, n, N, gp[j], aligned4);
    }
    __syncthreads();   // the shared state is reset for the next row
  }
}

}  // namespace two

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
  if (N <= 4 * kV * kThreads) {
    // one resident workgroup per CU; each walks rows with stride = grid
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const unsigned grid = (unsigned)(B < cus ? B : cus);
    if (B > cus && K - 1 <= 2) {
      // more rows than CUs: two 512-thread workgroups per CU, a row each
      const unsigned grid2 = (unsigned)(B < 2 * cus ? B : 2 * cus);
      if (K - 1 == 1)
        two::select_two_kernel<1><<<grid2, two::kT, 0, s>>>(score, B, N, c, group_out);
      else
        two::select_two_kernel<2><<<grid2, two::kT, 0, s>>>(score, B, N, c, group_out);
      return launch_status();
    }
    // rows start on 16-byte boundaries: the next row can be loaded into LDS directly
    const bool dma = N % 4 == 0 && (reinterpret_cast<uintptr_t>(score) & 15u) == 0;
    switch (K - 1) {
      case 1:
        if (dma) select_lds_kernel<1, true><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out);
        else select_lds_kernel<1, false><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out);
        break;
      case 2:
        if (dma) select_lds_kernel<2, true><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out);
        else select_lds_kernel<2, false><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out);
        break;
      case 3: select_reg_kernel<3><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out); break;
      case 4: select_reg_kernel<4><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out); break;
      case 5: select_reg_kernel<5><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out); break;
      case 6: select_reg_kernel<6><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out); break;
      default: select_reg_kernel<7><<<grid, kThreads, 0, s>>>(score, B, N, c, group_out); break;
    }
  } else
    select_mem_kernel<<<B, kThreads, 0, s>>>(score, N, c, K - 1, group_out);
  return launch_status();
}

}  // namespace hsa
