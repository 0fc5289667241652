// Active-query attention (KV-cache synchronisation, section 2.2 items 3-4):
// |A_i| query rows attend over all N rows of the per-layer K/V cache (fresh
// rows of active tokens and stale rows of skipped ones), so the work is
// O(|A_i| * N) instead of O(N^2).  No mask.
//
// bf16, Dh = 128: flash-style online softmax on v_mfma_f32_32x32x16_bf16.
//  * One workgroup = one head x 128 queries (4 wavefronts x 32); it streams
//    the head's K/V in tiles of 64 rows through double-buffered LDS, the next
//    tile's global loads in flight while the current one is consumed.
//  * Each wavefront computes S^T = K Q^T (keys as MFMA rows, its 32 queries
//    as columns), so a lane holds one query's scores: the row max and row
//    sum are in-lane except for one exchange between the two lane halves.
//  * P^T goes straight from the S^T accumulators into the B operand of
//    O^T = V^T P^T; the key order inside each 16-wide MFMA step follows the
//    accumulator layout, and the V^T operand is read in the same order from a
//    transposed copy of the V tile in LDS (chunks of 4 keys, XOR-swizzled by
//    the row so both the transposing writes and the operand reads spread
//    over the banks).
//  * exp2 with scale*log2(e) folded into one FMA; the running max is only
//    raised (and O, l rescaled) when a tile's max exceeds it by more than 8,
//    which is exact after the final division and keeps P <= 2^8.
//  * When |A_i| is small the KV range is split across workgroups; partial
//    (O, max, sum) are merged in a fixed split order (deterministic).
//  * Workgroup ids are remapped so each XCD runs a contiguous range of
//    (head, query tile) pairs: the workgroups sharing an XCD's L2 stream the
//    same head's K/V at the same time.
// Other head sizes / float32: a plain LDS-tiled kernel (float32 arithmetic).
#include "common.h"

namespace hsa {
namespace {

constexpr int kAttnThreads = 256;
constexpr int DH = 128;
constexpr int BKV = 64;
constexpr int BQ = 128;
constexpr int KSTR = DH + 8;              // bf16 per K row in LDS
constexpr int KCHUNKS = BKV * DH / 8 / kAttnThreads;  // 16-byte chunks per thread (= 4)
constexpr float kRescaleSlack = 8.0f;     // log2 units

__device__ __forceinline__ int32_t xcd_remap(int32_t bid, int32_t total) {
  constexpr int32_t kXcd = 8;
  const int32_t per = total / kXcd;
  const int32_t full = per * kXcd;
  if (bid >= full) return bid;
  return (bid % kXcd) * per + bid / kXcd;
}

// Swizzled 4-key chunk index of row d of the transposed V tile.
__device__ __forceinline__ int vt_chunk(int d, int kc) { return kc ^ ((d ^ (d >> 3)) & 15); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {  // low halves of a, b
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {  // high halves of a, b
  return (a >> 16) | (b & 0xffff0000u);
}

__global__ __launch_bounds__(kAttnThreads, 2) void attn_bf16_d128_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, float* __restrict__ part_o, float* __restrict__ part_ml, int32_t nA,
    int32_t nkv, int32_t H, float c, int32_t n_qt, int32_t splits, int32_t tiles_per_split) {
  __shared__ __attribute__((aligned(16))) bf16 sK[2][BKV * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 sVt[2][DH * BKV];

  const int32_t total = n_qt * H * splits;
  const int32_t t = xcd_remap(blockIdx.x, total);
  const int32_t qt = t % n_qt;
  const int32_t h = (t / n_qt) % H;
  const int32_t sp = t / (n_qt * H);
  const int32_t D = H * DH;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int32_t kv_begin = sp * tiles_per_split * BKV;
  const int32_t kv_end = min(nkv, kv_begin + tiles_per_split * BKV);
  const int32_t ntiles = (kv_end - kv_begin + BKV - 1) / BKV;

  // ---- Q^T fragments (B operand): lane = query column, 8 consecutive dims.
  const int32_t qi = qt * BQ + wave * 32 + l32;
  const bool q_ok = qi < nA;
  bf16x8 qf[DH / 16];
  {
    const bf16* qrow = q + (size_t)(q_ok ? qi : 0) * D + h * DH + half * 8;
#pragma unroll
    for (int dk = 0; dk < DH / 16; ++dk) {
      u32x4 raw = q_ok ? *reinterpret_cast<const u32x4*>(qrow + dk * 16) : u32x4{0u, 0u, 0u, 0u};
      qf[dk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- global -> register staging of one K/V tile
  u32x4 rk[KCHUNKS], rv[4];
  const int vdc = tid & 15;   // V: 8-dim chunk
  const int vkg = tid >> 4;   // V: group of 4 keys
  auto load_tile = [&](int32_t base) {
#pragma unroll
    for (int i = 0; i < KCHUNKS; ++i) {
      const int cidx = tid + i * kAttnThreads;
      const int r = cidx >> 4, ch = cidx & 15;
      const int32_t key = base + r;
      rk[i] = (key < kv_end) ? *reinterpret_cast<const u32x4*>(k + (size_t)key * D + h * DH + ch * 8)
                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t key = base + vkg * 4 + r;
      rv[r] = (key < kv_end) ? *reinterpret_cast<const u32x4*>(v + (size_t)key * D + h * DH + vdc * 8)
                             : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCHUNKS; ++i) {
      const int cidx = tid + i * kAttnThreads;
      const int r = cidx >> 4, ch = cidx & 15;
      *reinterpret_cast<u32x4*>(&sK[buf][r * KSTR + ch * 8]) = rk[i];
    }
    // transpose 4 keys x 8 dims -> 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int d = vdc * 8 + w * 2 + hi;
        u32x2 val;
        if (hi == 0) {
          val[0] = pack_lo(rv[0][w], rv[1][w]);
          val[1] = pack_lo(rv[2][w], rv[3][w]);
        } else {
          val[0] = pack_hi(rv[0][w], rv[1][w]);
          val[1] = pack_hi(rv[2][w], rv[3][w]);
        }
        *reinterpret_cast<u32x2*>(&sVt[buf][d * BKV + vt_chunk(d, vkg) * 4]) = val;
      }
    }
  };

  f32x16 acc_o[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  float m_run = -INFINITY;   // running max, log2 units (scaled)
  float l_run = 0.f;         // this lane's partial row sum

  if (ntiles > 0) {
    load_tile(kv_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int32_t base = kv_begin + it * BKV;
    if (it + 1 < ntiles) load_tile(base + BKV);

    // ---- S^T = K Q^T for 64 keys x 32 queries: two 32x32 blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const bf16* krow = &sK[buf][(kb * 32 + l32) * KSTR + half * 8];
#pragma unroll
      for (int dk = 0; dk < DH / 16; ++dk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + dk * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[dk], s[kb], 0, 0, 0);
      }
    }
    // s[kb][r] <-> key base + kb*32 + 8*(r/4) + 4*half + r%4, query l32
    if (base + BKV > kv_end) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t key = base + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= kv_end) s[kb][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mxs = mx * c;
    const bool need = mxs > m_run + kRescaleSlack;
    if (__ballot(need) != 0ull) {
      const float m_new = need ? mxs : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DH / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      m_run = m_new;
    }
    bf16x8 pb[4];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        bf16x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][jp * 8 + e], c, -m_run));
          lsum += p;
          pv[e] = (bf16)p;
        }
        pb[kb * 2 + jp] = pv;
      }
    l_run += lsum;

    // ---- O^T += V^T P^T: k-step ts covers keys kb*32 + 16*jp + {0..3, 8..11} + 4*half
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) {
      const int d = db * 32 + l32;
      const bf16* vrow = &sVt[buf][d * BKV];
#pragma unroll
      for (int ts = 0; ts < 4; ++ts) {
        const int kb = ts >> 1, jp = ts & 1;
        const int kc1 = 8 * kb + 4 * jp + half;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + vt_chunk(d, kc1) * 4);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + vt_chunk(d, kc1 + 2) * 4);
        const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw), pb[ts],
                                                             acc_o[db], 0, 0, 0);
      }
    }

    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!q_ok) return;
  // acc_o[db][r] <-> dim db*32 + 8*(r/4) + 4*half + r%4, query l32
  if (splits == 1) {
    const float inv = 1.0f / l_tot;
    bf16* orow = o + (size_t)qi * D + h * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = (bf16)(acc_o[db][4 * j + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * j + 4 * half) = w4;
      }
  } else {
    const size_t prow = ((size_t)(sp * H + h) * nA + qi);
    float* po = part_o + prow * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = acc_o[db][4 * j + e];
        *reinterpret_cast<f32x4*>(po + db * 32 + 8 * j + 4 * half) = w4;
      }
    if (half == 0) {
      part_ml[prow * 2 + 0] = m_run;
      part_ml[prow * 2 + 1] = l_tot;
    }
  }
}

// Merge split partials in split order: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         bf16* __restrict__ o, int32_t nA,
                                                         int32_t H, int32_t splits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)nA * H;
  const int64_t row = t / (HD / 4);
  const int d4 = (int)(t % (HD / 4)) * 4;
  if (row >= rows) return;
  const int32_t qi = (int32_t)(row / H), h = (int32_t)(row % H);
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[((size_t)(s * H + h) * nA + qi) * 2]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const size_t pr = (size_t)(s * H + h) * nA + qi;
    const float w = __builtin_amdgcn_exp2f(part_ml[pr * 2] - M);
    L += w * part_ml[pr * 2 + 1];
    const f32x4 po = *reinterpret_cast<const f32x4*>(part_o + pr * HD + d4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, po[e], acc[e]);
  }
  const float inv = 1.0f / L;
  bf16x4 w4;
#pragma unroll
  for (int e = 0; e < 4; ++e) w4[e] = (bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x4*>(o + (size_t)qi * H * HD + h * HD + d4) = w4;
}

// ---------------------------------------------------------------- plain path
// 64 queries x 4 sub-lanes per workgroup; each sub-lane owns HD/4 dims.
// K/V tiles of 32 rows in LDS as float32; exact online softmax per key.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_plain_kernel(const T* __restrict__ q,
                                                         const T* __restrict__ k,
                                                         const T* __restrict__ v,
                                                         T* __restrict__ o, int32_t nA,
                                                         int32_t nkv, int32_t H, float scale) {
  constexpr int TK = 32;
  constexpr int PER = HD / 4;
  __shared__ float sk[TK][HD];
  __shared__ float sv[TK][HD];
  const int tid = threadIdx.x;
  const int sub = tid & 3;
  const int32_t qi = blockIdx.x * 64 + (tid >> 2);
  const int32_t h = blockIdx.y;
  const int32_t D = H * HD;
  const bool q_ok = qi < nA;
  float qr[PER], acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    qr[e] = q_ok ? to_f32(q[(size_t)qi * D + h * HD + sub * PER + e]) * scale : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int32_t base = 0; base < nkv; base += TK) {
    __syncthreads();
    for (int i = tid; i < TK * HD; i += 256) {
      const int r = i / HD, cc = i % HD;
      const int32_t key = base + r;
      sk[r][cc] = key < nkv ? to_f32(k[(size_t)key * D + h * HD + cc]) : 0.f;
      sv[r][cc] = key < nkv ? to_f32(v[(size_t)key * D + h * HD + cc]) : 0.f;
    }
    __syncthreads();
    const int lim = min(TK, nkv - base);
    for (int r = 0; r < lim; ++r) {
      float sdot = 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) sdot = __builtin_fmaf(qr[e], sk[r][sub * PER + e], sdot);
      sdot += __shfl_xor(sdot, 1, 4);
      sdot += __shfl_xor(sdot, 2, 4);
      const float m_new = fmaxf(m, sdot);
      const float alpha = expf(m - m_new);
      const float p = expf(sdot - m_new);
      l = l * alpha + p;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(p, sv[r][sub * PER + e], acc[e] * alpha);
      m = m_new;
    }
  }
  if (!q_ok) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[(size_t)qi * D + h * HD + sub * PER + e] = from_f32<T>(acc[e] * inv);
}

struct SplitPlan {
  int32_t n_qt, splits, tiles_per_split;
};

SplitPlan plan_split(int32_t nA, int32_t nkv, int32_t H) {
  SplitPlan p;
  p.n_qt = cdiv(nA, BQ);
  const int32_t ntiles = cdiv(nkv, BKV);
  const int32_t base = p.n_qt * H;
  constexpr int32_t kTargetWgs = 1024;  // 2 resident workgroups on each of 256 CUs, x2
  int32_t s = 1;
  if (base < kTargetWgs / 2) s = min(16, cdiv(kTargetWgs, base));
  s = max(1, min(s, ntiles / 4));       // keep >= 4 tiles per split
  p.tiles_per_split = cdiv(ntiles, s);
  p.splits = cdiv(ntiles, p.tiles_per_split);
  return p;
}

bool use_mfma_path(int32_t Dh, hsa_dtype dt) { return dt == HSA_BF16 && Dh == 128; }

}  // namespace

size_t attn_workspace_bytes(int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh) {
  if (n_active <= 0 || n_kv <= 0) return 0;
  const SplitPlan p = plan_split(n_active, n_kv, H);
  if (p.splits <= 1) return 0;
  const size_t rows = (size_t)p.splits * H * n_active;
  return align_up(rows * Dh * sizeof(float), 256) + rows * 2 * sizeof(float);
}

hsa_status launch_attention(const void* q, const void* k, const void* v, void* o,
                            int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh, float scale,
                            hsa_dtype dt, void* ws, size_t ws_bytes, hipStream_t s) {
  if (n_active == 0) return HSA_OK;
  if (use_mfma_path(Dh, dt)) {
    const SplitPlan p = plan_split(n_active, n_kv, H);
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (p.splits > 1) {
      const size_t rows = (size_t)p.splits * H * n_active;
      if (ws == nullptr || ws_bytes < attn_workspace_bytes(n_active, n_kv, H, Dh))
        return HSA_ERR_WORKSPACE;
      part_o = (float*)ws;
      part_ml = (float*)((char*)ws + align_up(rows * Dh * sizeof(float), 256));
    }
    const int32_t total = p.n_qt * H * p.splits;
    attn_bf16_d128_kernel<<<total, kAttnThreads, 0, s>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, part_o, part_ml, n_active, n_kv,
        H, scale * kLog2e, p.n_qt, p.splits, p.tiles_per_split);
    if (p.splits > 1) {
      const int64_t threads = (int64_t)n_active * H * (DH / 4);
      attn_merge_kernel<DH><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(
          part_o, part_ml, (bf16*)o, n_active, H, p.splits);
    }
    return launch_status();
  }
  dim3 grid(cdiv(n_active, 64), H);
  if (dt == HSA_BF16) {
    if (Dh == 64)
      attn_plain_kernel<bf16, 64><<<grid, 256, 0, s>>>((const bf16*)q, (const bf16*)k, (const bf16*)v,
                                                       (bf16*)o, n_active, n_kv, H, scale);
    else
      return HSA_ERR_SHAPE;
  } else {
    if (Dh == 64)
      attn_plain_kernel<float, 64><<<grid, 256, 0, s>>>((const float*)q, (const float*)k,
                                                        (const float*)v, (float*)o, n_active, n_kv,
                                                        H, scale);
    else
      attn_plain_kernel<float, 128><<<grid, 256, 0, s>>>((const float*)q, (const float*)k,
                                                         (const float*)v, (float*)o, n_active,
                                                         n_kv, H, scale);
  }
  return launch_status();
}

}  // namespace hsa
