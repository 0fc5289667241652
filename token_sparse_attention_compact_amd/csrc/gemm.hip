// GEMMs on the active rows: out = a w^T with a [M][K] (M = |A_i| active rows,
// ragged), w [N][K] out-major.  These carry every per-token linear map of the
// block that KV-cache synchronisation keeps to active tokens (section 2.2):
// the QKV projection (with the fresh K/V rows scattered into the per-layer
// cache, item 2), the attention out-projection, and the MLP.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 (or 32x32x16) on 128x128, 128x192 or
// 256x256 output tiles, eight wavefronts each owning a block of MFMA tiles.
// K advances in steps of 64 through a 2-stage ring of LDS filled straight
// from HBM with buffer_load ... lds (no register staging; rows past M or N
// read as zero), each 16-byte chunk at an XOR-swizzled position of its
// 128-byte row so the operand reads hit distinct banks.  The next stage's
// loads are in flight while the current one feeds the MFMAs.  Epilogues are
// fused (store / GELU / residual add, plain or gated per column / QKV
// scatter) and work on quads of 4 consecutive output columns: the MFMA
// computes C^T blocks (w rows as MFMA rows), whose accumulator layout gives
// each lane runs of 4 consecutive columns of a row.
//
// float32 path (small float32 workloads): LDS-tiled FMA GEMM, 64x64 tiles.
// The QKV projection can read its rows gathered, a[idx[m]], from a larger
// matrix (the per-token hidden state), on both paths.
#include <type_traits>

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
  } else if constexpr (EPI == EPI_RESID_GATED) {
    float* p = ep.resid + (size_t)row * N + col;
    *p = *p + load_mod(ep.gate, col) * v;
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

// Epilogue on 4 consecutive output columns col..col+3 of one row (N % 4 == 0).
__device__ __forceinline__ float gelu_fast(float u) {
  const float z = 0.7978845608028654f * (u + 0.044715f * u * u * u);
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.0f * kLog2e * z));
}

template <int EPI>
__device__ __forceinline__ void epilogue4(const EpiArgs& ep, int32_t N, int32_t row, int32_t col,
                                          f32x4 v) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_GELU) {
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)(EPI == EPI_GELU ? gelu_fast(v[e]) : v[e]);
    *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(ep.out) + (size_t)row * N + col) = o;
  } else if constexpr (EPI == EPI_RESID) {
    f32x4* p = reinterpret_cast<f32x4*>(ep.resid + (size_t)row * N + col);
    f32x4 h = *p;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] += v[e];
    *p = h;
  } else if constexpr (EPI == EPI_RESID_GATED) {
    f32x4* p = reinterpret_cast<f32x4*>(ep.resid + (size_t)row * N + col);
    const f32x4 g = load_mod4(ep.gate, col);
    f32x4 h = *p;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] += g[e] * v[e];
    *p = h;
  } else {  // EPI_QKV_SCATTER: D % 4 == 0, so the 4 columns stay in one of q, k, v
    const int32_t D = ep.D;
    const int32_t which = col / D;
    const int32_t c = col - which * D;
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
    bf16* dst;
    if (which == 0) dst = reinterpret_cast<bf16*>(ep.out) + (size_t)row * D + c;
    else dst = reinterpret_cast<bf16*>(which == 1 ? ep.kc : ep.vc) + (size_t)ep.idx[row] * D + c;
    *reinterpret_cast<bf16x4*>(dst) = o;
  }
}

// ---------------------------------------------------------------- bf16 MFMA
constexpr int BK = 64;
constexpr int ROWB = BK * 2;                       // bytes per LDS row (128)

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Tile order.  Consecutive workgroup ids land on different XCDs (round-robin
// over 8), so each XCD is first handed a contiguous run of tile indices.  The
// index then walks the tiles in groups of GM row blocks, column-major inside a
// group: the ~32 workgroups an XCD runs at once cover a GM x (32/GM) block of
// tiles and share its GM row blocks of a and 32/GM column blocks of w in that
// XCD's L2, instead of streaming 32 row blocks of a that every column tile
// then reads again from HBM.
__device__ __forceinline__ void tile_coords(int32_t bid, int32_t tm, int32_t tn, int32_t gm,
                                            int32_t& mi, int32_t& ni) {
  constexpr int32_t kXcd = 8;
  const int32_t ntiles = tm * tn;
  const int32_t per = ntiles / kXcd;
  int32_t t = bid;
  if (bid < per * kXcd) t = (bid % kXcd) * per + bid / kXcd;   // leftover tail keeps its id
  const int32_t width = gm * tn;
  const int32_t group = t / width;
  const int32_t first_m = group * gm;
  const int32_t gsize = min(tm - first_m, gm);
  const int32_t r = t - group * width;
  mi = first_m + r % gsize;
  ni = r / gsize;
}

// Position of 16-byte chunk c (0..7) in LDS row r: XOR swizzle chosen so that
// 16-byte operand reads of 8 consecutive rows (32 banks) or of 16 consecutive
// rows (64 banks) at one chunk hit distinct banks.
__device__ __forceinline__ int gpos(int r, int c) { return c ^ (((r >> 1) ^ (r << 2)) & 7); }

__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}

// 16 bytes per lane from a buffer straight into LDS at lds_addr + 16*lane.
// Inline asm keeps the compiler from waiting for every in-flight load before
// each LDS read; completion is tracked with vmcnt before the barrier.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int VM>   // loads of this wave allowed in flight
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(VM) : "memory");
}

// Tile configuration: BM x BN output tile, WM x WN wavefronts (each owning a
// (BM/WM) x (BN/WN) block of MI x MI MFMA tiles), NST LDS stages of BK=64,
// tile groups of GM row blocks by default (the launch may pass another
// group size), at least MINB workgroups per CU (which caps the registers per
// lane: 128 at two 512-thread workgroups, 256 at one), MFMA shape MI:
// 16 = v_mfma_f32_16x16x32_bf16, 32 = v_mfma_f32_32x32x16_bf16.
template <int BM_, int BN_, int WM_, int WN_, int NST_, int GM_, int MINB_, int MI_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NST = NST_, GM = GM_;
  static constexpr int MINB = MINB_, MI = MI_;
  static_assert(MI == 16 || MI == 32, "MFMA shape");
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;        // per-wave block
  static constexpr int FM = TM / MI, FN = TN / MI;        // MFMA tiles per wave
  static constexpr int TILE_A = BM * ROWB, TILE_B = BN * ROWB;
  static constexpr int STAGE = TILE_A + TILE_B;
  static constexpr int LOADS_A = TILE_A / 16 / THREADS;
  static constexpr int LOADS_B = TILE_B / 16 / THREADS;
  static constexpr int LOADS = LOADS_A + LOADS_B;
  static_assert(LOADS_A * 16 * THREADS == TILE_A && LOADS_B * 16 * THREADS == TILE_B, "load split");
  static_assert(NST * STAGE <= 160 * 1024, "LDS");
};

template <class G, int EPI>
__global__ __launch_bounds__(G::THREADS, G::MINB) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, int32_t M, int32_t N, int32_t K,
    int32_t gm, EpiArgs ep) {
  constexpr int BM = G::BM, BN = G::BN, NST = G::NST;
  __shared__ __attribute__((aligned(1024))) char smem[NST * G::STAGE];
  static_assert(G::FM >= 1 && G::FN >= 1, "wave tile");
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  const int32_t tm = (M + BM - 1) / BM;
  const int32_t tn = (N + BN - 1) / BN;
  int32_t mi, ni;
  tile_coords(blockIdx.x, tm, tn, gm, mi, ni);
  const int32_t m0 = mi * BM;
  const int32_t n0 = ni * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / G::WN, wn = wave % G::WN;

  // DMA source offsets (bytes from the tile's k-slice base), fixed over k.
  // Load j of wave w fills 16-byte slots (j*WAVES + w)*64 + lane of a tile.
  // QKV may read its rows gathered from a larger matrix: row m of the tile is
  // a[idx[m]] (rows past M repeat the last active row; they are not stored).
  const bool gather = EPI == EPI_QKV_SCATTER && ep.gather_rows > 0;
  uint32_t voff_a[G::LOADS_A], voff_b[G::LOADS_B];
#pragma unroll
  for (int j = 0; j < G::LOADS_A; ++j) {
    const int sl = (j * G::WAVES + wave) * 64 + lane;
    const int r = sl >> 3, p = sl & 7;
    const uint32_t row_off = gather ? (uint32_t)ep.idx[min(m0 + r, M - 1)] * (uint32_t)K * 2u
                                    : (uint32_t)(r * K * 2);
    voff_a[j] = row_off + (uint32_t)(gpos(r, p) * 16);   // gpos(r, .) is an involution
  }
#pragma unroll
  for (int j = 0; j < G::LOADS_B; ++j) {
    const int sl = (j * G::WAVES + wave) * 64 + lane;
    const int r = sl >> 3, p = sl & 7;
    voff_b[j] = (uint32_t)(r * K * 2 + gpos(r, p) * 16);
  }
  const uint32_t bytes_a = gather ? (uint32_t)ep.gather_rows * (uint32_t)K * 2u
                                  : (uint32_t)(M - m0) * (uint32_t)K * 2u;
  const uint32_t bytes_b = (uint32_t)(min(N, n0 + BN) - n0) * (uint32_t)K * 2u;
  const char* a_base = reinterpret_cast<const char*>(A) + (gather ? 0 : (size_t)m0 * K * 2);
  const char* b_base = reinterpret_cast<const char*>(W) + (size_t)n0 * K * 2;

  auto issue = [&](int kt, int stage) {
    const uint32_t kb = (uint32_t)kt * BK * 2;
    const i32x4 ra = buffer_rsrc(a_base + kb, bytes_a - kb);
    const i32x4 rb = buffer_rsrc(b_base + kb, bytes_b - kb);
    const uint32_t sa = lds0 + stage * G::STAGE;
    const uint32_t sb = sa + G::TILE_A;
#pragma unroll
    for (int j = 0; j < G::LOADS_A; ++j)
      dma16(sa + (uint32_t)__builtin_amdgcn_readfirstlane((j * G::WAVES + wave) * 1024), voff_a[j], ra);
#pragma unroll
    for (int j = 0; j < G::LOADS_B; ++j)
      dma16(sb + (uint32_t)__builtin_amdgcn_readfirstlane((j * G::WAVES + wave) * 1024), voff_b[j], rb);
  };

  // Operand read offsets.  An MFMA step takes KSTEP = 512/MI values of k; its
  // 8-value operand run in a lane is row lr = lane % MI of the MI-row block at
  // 16-byte chunk (64/MI) * ks + lane / MI of the 128-byte LDS row.
  constexpr int MI = G::MI, KSTEP = 512 / MI, NKS = BK / KSTEP;
  const int lr = lane % MI, lc = lane / MI;
  uint32_t frag[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    frag[ks] = (uint32_t)(lr * ROWB + gpos(lr, (64 / MI) * ks + lc) * 16);

  typedef typename std::conditional<MI == 32, f32x16, f32x4>::type Acc;
  constexpr int NACC = MI * MI / 64;   // accumulator values per lane
  Acc acc[G::FM][G::FN];
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j)
#pragma unroll
      for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nk) issue(st, st);

  for (int kt = 0; kt < nk; ++kt) {
    // k-tile kt landed (later ones may be in flight) and is visible to every
    // wave; every wave is done with k-tile kt-1, whose stage is refilled next
    const int ahead = min(NST - 2, nk - 1 - kt);
    if (NST >= 4 && ahead >= 2) wait_barrier<2 * G::LOADS>();
    else if (NST >= 3 && ahead >= 1) wait_barrier<G::LOADS>();
    else wait_barrier<0>();
    if (kt + NST - 1 < nk) issue(kt + NST - 1, (kt + NST - 1) % NST);
    const char* sa = smem + (kt % NST) * G::STAGE;
    const char* a_frag = sa + (wm * G::TM) * ROWB;
    const char* b_frag = sa + G::TILE_A + (wn * G::TN) * ROWB;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 af[G::FM], bfr[G::FN];
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(a_frag + i * MI * ROWB + frag[ks]);
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(b_frag + j * MI * ROWB + frag[ks]);
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int j = 0; j < G::FN; ++j) {   // C^T block: w rows as MFMA rows, a rows as columns
          if constexpr (MI == 32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
    }
  }

  // acc[i][j][r] = C[row][col] with row = block (i) row lr and col = block (j)
  // column 8*(r/4) + 4*lc + r%4 (MI = 32) or 4*lc + r (MI = 16): each quad
  // r = 4g..4g+3 is 4 consecutive columns of one row.
  if constexpr (MI == 16 && BM <= 128) {
    // 128-row tiles go out through the LDS ring, free once every wave is past
    // the last k-slice: a wavefront's accumulators cover 32-byte pieces of 16
    // rows per store, so they are written to LDS in that layout and read back
    // as 16-byte chunks of whole rows, which leave in 1 KiB runs per store
    // instruction.  A pass stages whole wave-row blocks (TM rows): bf16
    // outputs in one pass, float32 residual tiles in one or two, each pass
    // read-add-written against the residual stream.  M = 8190 (128 x 192
    // tiles): QKV 119 -> 115, out-projection 45.2 -> 43.8, MLP up 233 -> 225
    // us, MLP down unchanged; on 256 x 256 tiles (two to four passes) the
    // direct stores below measured 2-4% faster, so those keep them.
    constexpr bool F32 = EPI == EPI_RESID || EPI == EPI_RESID_GATED;
    constexpr int ESZ = F32 ? 4 : 2;                  // staged bytes per value
    constexpr int PITCH = BN * ESZ + 16;              // staged row, padded against bank conflicts
    constexpr int FIT = NST * G::STAGE / (G::TM * PITCH);
    constexpr int WRP = FIT < G::WM ? FIT : G::WM;    // wave-row blocks per pass
    static_assert(WRP >= 1, "a wave-row block fits the ring");
    constexpr int PASSES = (G::WM + WRP - 1) / WRP;
    constexpr int PR = WRP * G::TM;                   // rows per pass
    constexpr int CPR = BN * ESZ / 16;                // 16-byte chunks per staged row
    constexpr int VPC = 16 / ESZ;                     // values per chunk
    // 16-byte bf16 stores need 16-byte aligned rows: widths a multiple of 8
    // and aligned bases, else two 8-byte stores per chunk
    bool a16 = false;
    if constexpr (EPI == EPI_QKV_SCATTER)
      a16 = ep.D % 8 == 0 && ((reinterpret_cast<uintptr_t>(ep.out) | reinterpret_cast<uintptr_t>(ep.kc) |
                               reinterpret_cast<uintptr_t>(ep.vc)) & 15u) == 0;
    else if constexpr (!F32)
      a16 = N % 8 == 0 && (reinterpret_cast<uintptr_t>(ep.out) & 15u) == 0;
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      if (wm / WRP == ps) {
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int j = 0; j < G::FN; ++j) {
            const int rl = (wm % WRP) * G::TM + i * MI + lr;
            const int cl = wn * G::TN + j * MI + 4 * lc;
            char* dst = smem + rl * PITCH + cl * ESZ;
            if constexpr (F32) {
              *reinterpret_cast<f32x4*>(dst) = acc[i][j];
            } else {
              bf16x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (bf16)(EPI == EPI_GELU ? gelu_fast(acc[i][j][e]) : acc[i][j][e]);
              *reinterpret_cast<bf16x4*>(dst) = o;
            }
          }
      }
      __syncthreads();
      const int rows = min(PR, BM - ps * PR);
      for (int c = tid; c < rows * CPR; c += G::THREADS) {
        const int rl = c / CPR, ch = c - rl * CPR;
        const int32_t r = m0 + ps * PR + rl;
        const int32_t col = n0 + ch * VPC;
        if (r >= M || col >= N) continue;
        const char* src = smem + rl * PITCH + ch * 16;
        if constexpr (F32) {   // N % 4 == 0: a chunk is all in or all out
          const f32x4 v = *reinterpret_cast<const f32x4*>(src);
          f32x4* hp = reinterpret_cast<f32x4*>(ep.resid + (size_t)r * N + col);
          f32x4 hv = *hp;
          if constexpr (EPI == EPI_RESID_GATED) {
            const f32x4 g = load_mod4(ep.gate, col);
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] += g[e] * v[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] += v[e];
          }
          *hp = hv;
        } else {
          const u32x4 v = *reinterpret_cast<const u32x4*>(src);
          auto dst_of = [&](int32_t cc) -> bf16* {   // output address of column cc of row r
            if constexpr (EPI == EPI_QKV_SCATTER) {
              const int32_t which = cc / ep.D, c0 = cc - which * ep.D;
              if (which == 0) return reinterpret_cast<bf16*>(ep.out) + (size_t)r * ep.D + c0;
              return reinterpret_cast<bf16*>(which == 1 ? ep.kc : ep.vc) + (size_t)ep.idx[r] * ep.D + c0;
            } else {
              return reinterpret_cast<bf16*>(ep.out) + (size_t)r * N + cc;
            }
          };
          const bool whole = a16 && col + 8 <= N && (EPI != EPI_QKV_SCATTER || col % ep.D + 8 <= ep.D);
          if (whole) {
            *reinterpret_cast<u32x4*>(dst_of(col)) = v;
          } else {   // unaligned rows, or the chunk ends the row or crosses from q to k or k to v
            *reinterpret_cast<u32x2*>(dst_of(col)) = u32x2{v[0], v[1]};
            if (col + 4 < N) *reinterpret_cast<u32x2*>(dst_of(col + 4)) = u32x2{v[2], v[3]};
          }
        }
      }
      if (ps + 1 < PASSES) __syncthreads();
    }
  } else {
    const int32_t row = m0 + wm * G::TM + lr;
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
#pragma unroll
        for (int g = 0; g < NACC / 4; ++g) {
          const int32_t r = row + i * MI;
          const int32_t col = n0 + wn * G::TN + j * MI + 8 * g + 4 * lc;
          if (r < M && col < N) {
            const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
            epilogue4<EPI>(ep, N, r, col, v);
          }
        }
  }
}

// Four tile shapes, chosen per GEMM shape (pick_cfg), all on the 16x16x32
// MFMA.  Measured on MI355X with interleaved runs over 4 rotating weight sets
// (TFLOP/s for QKV / out-projection / MLP up / MLP down, D 1536, FFN 8960):
//  * 128x192, 8 waves of 32x96 (80 KiB LDS, two workgroups per CU):
//    M = 8190: 1031 / 863 / 1040 / 1135, against 945 / 765 / 988 / 1110 for
//    the same pipeline on 256x192 tiles of 32x32x16 MFMAs.  The 16x16 shape
//    issues twice the operand reads per flop, but at 16 rows per block a
//    wave's tile needs half the accumulator registers of the 32x32 form of
//    the same block count, which leaves room for two workgroups per CU;
//    192 divides the stack's output widths (1536, 4608), so the tile count
//    is a whole number of rounds over the chip;
//  * 256x256, 8 waves of 64x128, one workgroup per CU (128 KiB): fewer,
//    larger tiles for large M: M = 32760: 983 / 746 / 1046 / 1160 against
//    1014 / 747 / 1017 / 1091 for 128x192;
//  * 128x128, 8 waves of 32x64 (64 KiB, two per CU): the most tiles when M
//    is small and the output is wide: M = 2048: 599 / 413 / 777 / 579
//    against 751 / 357 / 926 / 509 (128x192 / 256x256 columns);
//  * 128x64 (below): narrow outputs at small M.
// 256x192 and 128x128 tiles of 32x32x16 MFMAs, 256x128, 64x192 tiles,
// 4-wave layouts and 3-4 stage rings measured slower.
typedef GemmCfg<256, 256, 4, 2, 2, 4, 1, 16> CfgWide;
typedef GemmCfg<128, 192, 4, 2, 2, 4, 2, 16> CfgMain;
typedef GemmCfg<128, 128, 4, 2, 2, 8, 2, 16> CfgSmall;
// 128x64, 8 waves of 32x32 (48 KiB, two per CU): narrow outputs at small M,
// where the larger tiles leave CUs idle: M = 2048, N = 1536: out-projection
// 447 and MLP down 614 TFLOP/s against 408 and 572 on 128x128 tiles
// (M = 1638: 363 / 519 against 324 / 448); from M = 4095 the larger tiles win.
typedef GemmCfg<128, 64, 4, 2, 2, 8, 2, 16> CfgTiny;

enum { kCfgWide, kCfgMain, kCfgSmall, kCfgTiny };

// Row blocks per tile group of the 256x256 tiles.  Each layer's weights are
// read cold from HBM once per iteration: with wide outputs (QKV, MLP up) two
// row blocks per group keep more of W's column tiles streaming at once
// (interleaved runs over 8 rotating weight sets, 256-row tiles: MLP up
// 863 -> 931, QKV 878 -> 904 TFLOP/s); the narrow, long-K shapes
// (out-projection, MLP down) do best with four.
int32_t wide_group_rows(int32_t N) { return N > 2048 ? 2 : CfgWide::GM; }

// Cost model: a CU works through ceil(tiles / 256) tiles of its shape one
// after another (two co-resident workgroups share the CU's MFMA rate), so
// time ~ ceil(tiles / 256) * tile area / relative efficiency.  Ties go to
// the larger tile.  Outside the model: M <= 2048 with N <= 2048 (the
// out-projection and MLP down at <= 6.25% active) takes the 128x64 tile,
// which the model would rank below 128x128 but measured 7-16% faster there
// (more tiles for the chip; the measurements are at CfgTiny).
int pick_cfg(int32_t M, int32_t N) {
  if (M <= 2048 && N <= 2048) return kCfgTiny;
  constexpr int64_t kCus = 256;
  const struct { int id; int64_t bm, bn, eff; } c[3] = {
      {kCfgWide, 256, 256, 1025}, {kCfgMain, 128, 192, 1000}, {kCfgSmall, 128, 128, 900}};
  int best = kCfgWide;
  int64_t best_cost = -1;
  for (const auto& x : c) {
    const int64_t tiles = cdiv((int64_t)M, x.bm) * cdiv((int64_t)N, x.bn);
    const int64_t cost = cdiv(tiles, kCus) * x.bm * x.bn * 1000 / x.eff;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = x.id;
    }
  }
  return best;
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
  const bool gather = EPI == EPI_QKV_SCATTER && ep.gather_rows > 0;
  const int32_t arow = (m0 + lr < M && gather) ? ep.idx[m0 + lr] : m0 + lr;   // row of a
  float acc[4][4] = {};
  for (int32_t k0 = 0; k0 < K; k0 += FK) {
    const int32_t gk = k0 + lk;
    f32x4 va = {0.f, 0.f, 0.f, 0.f}, vb = {0.f, 0.f, 0.f, 0.f};
    if (m0 + lr < M && gk < K) va = *reinterpret_cast<const f32x4*>(A + (size_t)arow * K + gk);
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

template <class G, int EPI>
void launch_bf16(const void* a, const void* w, int32_t M, int32_t N, int32_t K, int32_t gm,
                 const EpiArgs& ep, hipStream_t s) {
  const int32_t tiles = cdiv(M, G::BM) * cdiv(N, G::BN);
  gemm_bf16_kernel<G, EPI><<<tiles, G::THREADS, 0, s>>>((const bf16*)a, (const bf16*)w, M, N, K, gm, ep);
}

template <int EPI>
hsa_status run(const void* a, const void* w, int32_t M, int32_t N, int32_t K, hsa_dtype dt,
               const EpiArgs& ep, hipStream_t s) {
  if (dt == HSA_BF16) {
    if (N % 4 != 0 || (EPI == EPI_QKV_SCATTER && ep.D % 4 != 0)) return HSA_ERR_SHAPE;
    switch (pick_cfg(M, N)) {
      case kCfgWide:
        launch_bf16<CfgWide, EPI>(a, w, M, N, K, wide_group_rows(N), ep, s);
        break;
      case kCfgMain: launch_bf16<CfgMain, EPI>(a, w, M, N, K, CfgMain::GM, ep, s); break;
      case kCfgSmall: launch_bf16<CfgSmall, EPI>(a, w, M, N, K, CfgSmall::GM, ep, s); break;
      default: launch_bf16<CfgTiny, EPI>(a, w, M, N, K, CfgTiny::GM, ep, s); break;
    }
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
    case EPI_RESID_GATED: return run<EPI_RESID_GATED>(a, w, M, N, K, dt, ep, s);
    default: return HSA_ERR_ARG;
  }
}

}  // namespace hsa
