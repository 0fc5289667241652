// Active-query attention (KV-cache synchronisation, section 2.2 items 3-4):
// |A_i| query rows attend over all N rows of the per-layer K/V cache (fresh
// rows of active tokens and stale rows of skipped ones), so the work is
// O(|A_i| * N) instead of O(N^2).  No mask.
//
// bf16, Dh = 128 or 64: flash-style online softmax on
// v_mfma_f32_32x32x16_bf16 (one kernel body, templated on the head width).
//  * One workgroup = one head x 256 queries (8 wavefronts x 32, two per SIMD
//    so one wave's softmax overlaps the other's MFMAs).  It streams the
//    head's K/V in tiles of 64 rows through a 4-stage LDS ring (128 KiB at
//    Dh = 128, 64 KiB at Dh = 64).
//  * Tiles move HBM -> LDS with buffer_load ... lds (no register staging, no
//    per-load VALU work; rows past the end read as zero).  Each 16-byte chunk
//    lands at an XOR-swizzled position of its 256-byte row, so the operand
//    reads below hit distinct banks (256-byte rows at Dh = 128, 128-byte at 64).
//  * Each wavefront computes S^T = K Q^T (keys as MFMA rows, its 32 queries
//    as columns): a lane holds one query's scores, so the row max and row
//    sum are in-lane except one exchange between the lane halves
//    (v_permlane32_swap).
//  * P^T goes from the S^T accumulators into the B operand of O^T = V^T P^T;
//    the key order of each 16-key MFMA step follows the accumulator layout.
//    The V^T operand is read from the row-major V tile with the transposing
//    LDS read ds_read_b64_tr_b16: per 16-lane group it takes a 4-key x
//    16-dim block and gives lane i dim i of those 4 keys.
//  * Inside each wavefront the loop is software-pipelined over 32-key
//    sub-tiles (two per LDS tile): one step issues the S^T MFMAs of sub-tile
//    u+1 and the PV MFMAs of sub-tile u-1 alternately (Dh/16 of each), with
//    the softmax of sub-tile u spread between them, so the MFMA unit always
//    has independent work while the VALU turns scores into probabilities.  One 32x32 score
//    block per sub-tile keeps the live registers within the 256 a wave may
//    hold at two waves per SIMD.
//  * Softmax in log2 units with little VALU work per score: Q is pre-scaled
//    by scale*log2(e) and each S^T accumulator is seeded with minus the
//    running max, so the MFMA itself yields s = c q.k - m and a probability
//    is one exp2 (plus a pack to bf16 shared by two).  The running max is
//    taken from the first sub-tile and raised only when a later one's
//    row-sum partial shows a probability far above 1 (no per-score max);
//    O and l are then rescaled, which is exact after the final division.
//    Row sums are float32 adds (v_dot2 over the packed pairs would be fewer
//    instructions but holds up the MFMA issue far more).
//  * Work items are (query tile, head) pairs.  When they do not fill whole
//    rounds of the chip, the first n_full items (whole rounds) run over the
//    full KV range and the remaining ones are split over the KV range into
//    `splits` parts, whose partials (O/l in bf16, max, sum) are merged in a
//    fixed split order (deterministic).  At 384 items on 256 CUs: 256 whole
//    items, then 128 items in two halves, so the chip stays full to the end
//    and only a third of the rows go through partials.
//  * Workgroup ids are remapped (within the whole and the split segment) so
//    each XCD runs a contiguous range of items: the workgroups sharing an
//    XCD's L2 stream the same head's K/V at the same time.
// float32: a plain LDS-tiled kernel (float32 arithmetic).
#include "common.h"

namespace hsa {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int NW = 8;                      // wavefronts per workgroup
constexpr int kAttnThreads = NW * 64;
constexpr int BKV = 64;                    // keys per tile (LDS stage)
constexpr int SUB = 32;                    // keys per sub-tile (one S^T MFMA block)
constexpr int BQ = NW * 32;                // queries per workgroup
constexpr int NST = 4;                     // LDS stages

// Head-width constants of the MFMA path (Dh = 128 or 64).
template <int DH_>
struct AttnShape {
  static constexpr int DH = DH_;
  static constexpr int ROWB = DH * 2;                        // bytes per K/V row of one head
  static constexpr int TILEB = BKV * ROWB;                   // bytes per K or V tile
  static constexpr int LOADS = TILEB / 16 / kAttnThreads;    // 16-byte loads per lane per tile
  static constexpr int NS = DH / 16;      // S^T MFMAs per sub-tile (16 dims each) = PV MFMAs
  static constexpr int NDB = DH / 32;     // 32-dim blocks of O^T
  static constexpr int EPS = 16 / NS;     // score elements a lane exponentiates per MFMA pair
  static_assert(LOADS * 16 * kAttnThreads == TILEB, "tile load split");
};
// Largest row-sum partial (32 probabilities of one query in one lane) a tile may
// reach before the running max is raised: it bounds every probability by 2^32.
constexpr float kRaiseSum = 4294967296.0f;

__device__ __forceinline__ int32_t xcd_remap(int32_t bid, int32_t total) {
  constexpr int32_t kXcd = 8;
  const int32_t per = total / kXcd;
  const int32_t full = per * kXcd;
  if (bid >= full) return bid;
  return (bid % kXcd) * per + bid / kXcd;
}

// Position of 16-byte chunk c within row r of a K / V tile in LDS (XOR
// swizzles, involutions in c).  Dh = 128 (16 chunks, 256-byte rows): K reads
// of 16 consecutive rows at one chunk, and the transposing V reads, hit
// distinct banks.  Dh = 64 (8 chunks, 128-byte rows): the K swizzle spreads 8
// or 16 consecutive rows at one chunk over distinct banks; the V swizzle swaps
// the halves of rows 2, 3 (mod 4) so the 4-key x 32-dim blocks of a
// transposing read cover all 64 banks.
template <int DH>
__device__ __forceinline__ int k_pos(int r, int c) {
  if constexpr (DH == 128) return c ^ (r & 15);
  else return c ^ (((r >> 1) ^ (r << 2)) & 7);
}
template <int DH>
__device__ __forceinline__ int v_pos(int r, int c) {
  if constexpr (DH == 128) return c ^ ((r & 3) << 2);
  else return c ^ (((r >> 1) & 1) << 2);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for `bytes` bytes from `base` (raw buffer, stride 0):
// loads at offsets >= bytes return zero.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}

// One 16-byte-per-lane buffer load straight into LDS at lds_addr + 16*lane.
// Written as inline asm so the compiler does not treat the LDS stage as
// written by an unknown DMA (it would wait for every load in flight before
// each LDS read); completion is tracked by hand with vmcnt before the barrier.
// The instruction has no register result.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Issue the loads of one K and one V tile (rows row0.. of head h) into LDS.
template <int DH>
__device__ __forceinline__ void issue_tile(const bf16* k, const bf16* v, int32_t row0, int32_t nkv,
                                           int32_t ldk, int32_t h, uint32_t sk, uint32_t sv,
                                           const uint32_t* voff_k, const uint32_t* voff_v,
                                           int wave) {
  const int32_t rows_left = nkv - row0;
  const uint32_t nbytes = rows_left > 0 ? (uint32_t)rows_left * (uint32_t)ldk * 2u : 0u;
  constexpr int LOADS = AttnShape<DH>::LOADS;
  const size_t off = ((size_t)row0 * ldk + (size_t)h * DH) * 2;
  const i32x4 rk = buffer_rsrc(reinterpret_cast<const char*>(k) + off, nbytes);
  const i32x4 rv = buffer_rsrc(reinterpret_cast<const char*>(v) + off, nbytes);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    // this wave's 1 KiB slice of the tile (wave-uniform: scalar for M0)
    const uint32_t blk = (uint32_t)__builtin_amdgcn_readfirstlane((j * NW + wave) * 1024);
    dma16(sk + blk, voff_k[j], rk);
    dma16(sv + blk, voff_v[j], rv);
  }
}

// One of the 2 LOADS loads of a K / V tile pair (part p: K for even p, V for
// odd p, slice p / 2), for loads spread over the MFMA stream of a step.
// Loads at or past nkv return zero (row0 = nkv: zero-byte loads).
struct TileLoads {
  i32x4 rk, rv;
  uint32_t sk, sv;
};
template <int DH>
__device__ __forceinline__ TileLoads tile_loads(const bf16* k, const bf16* v, int32_t row0,
                                                int32_t nkv, int32_t ldk, int32_t h, uint32_t sk,
                                                uint32_t sv) {
  const int32_t rows_left = nkv - row0;
  const uint32_t nbytes = rows_left > 0 ? (uint32_t)rows_left * (uint32_t)ldk * 2u : 0u;
  const size_t off = ((size_t)row0 * ldk + (size_t)h * DH) * 2;
  return TileLoads{buffer_rsrc(reinterpret_cast<const char*>(k) + off, nbytes),
                   buffer_rsrc(reinterpret_cast<const char*>(v) + off, nbytes), sk, sv};
}
__device__ __forceinline__ void tile_part(const TileLoads& t, int p, const uint32_t* voff_k,
                                          const uint32_t* voff_v, int wave) {
  const int j = p >> 1;
  const uint32_t blk = (uint32_t)__builtin_amdgcn_readfirstlane((j * NW + wave) * 1024);
  if (p & 1) dma16(t.sv + blk, voff_v[j], t.rv);
  else dma16(t.sk + blk, voff_k[j], t.rk);
}

// Wait until at most OUT tiles' loads of this wave are in flight, then
// synchronise the workgroup.  No memory fence: the only LDS writes are the
// tile loads, whose completion vmcnt reports.
template <int DH, int OUT>
__device__ __forceinline__ void wait_tiles_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(OUT * 2 * AttnShape<DH>::LOADS) : "memory");
}

template <int DH_>
__device__ __forceinline__ void attn_bf16_body(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, bf16* __restrict__ part_o, float* __restrict__ part_ml, int32_t nA,
    int32_t nkv, int32_t H, float c, int32_t n_qt, int32_t n_full, int32_t splits,
    int32_t tiles_per_split, char* smem) {
  typedef AttnShape<DH_> S;
  constexpr int DH = S::DH, ROWB = S::ROWB, TILEB = S::TILEB, LOADS = S::LOADS;
  constexpr int NS = S::NS, NDB = S::NDB, EPS = S::EPS;
  const char* const sK = smem;
  const uint32_t sK_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const uint32_t sV_lds = sK_lds + NST * TILEB;

  // item i = qt + n_qt * h; items below n_full whole, the rest in `splits`
  // parts (part sp of split item n_full + il at workgroup n_full + sp * L + il)
  const int32_t n_items = n_qt * H;
  const int32_t L = n_items - n_full;
  const int32_t bid = blockIdx.x;
  const bool split = bid >= n_full;
  const int32_t t = split ? xcd_remap(bid - n_full, L * splits) : xcd_remap(bid, n_full);
  const int32_t il = split ? t % L : 0;             // index among the split items
  const int32_t sp = split ? t / L : 0;
  const int32_t item = split ? n_full + il : t;
  const int32_t qt = item % n_qt;
  const int32_t h = item / n_qt;
  const int32_t D = H * DH;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int32_t kv_begin = split ? sp * tiles_per_split * BKV : 0;
  const int32_t kv_end = split ? min(nkv, kv_begin + tiles_per_split * BKV) : nkv;
  const int32_t ntiles = (kv_end - kv_begin + BKV - 1) / BKV;

  // ---- per-lane load offsets (bytes within a tile of this head), fixed for all tiles
  uint32_t voff_k[LOADS], voff_v[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int s = (j * NW + wave) * 64 + lane;   // 16-byte slot in the tile
    const int r = s / (ROWB / 16), p = s % (ROWB / 16);   // row, chunk
    voff_k[j] = (uint32_t)(r * D * 2 + k_pos<DH>(r, p) * 16);   // k_pos is an involution
    voff_v[j] = (uint32_t)(r * D * 2 + v_pos<DH>(r, p) * 16);
  }

  // ---- Q^T fragments (B operand): lane = query column, 8 consecutive dims
  const int32_t qi = qt * BQ + wave * 32 + l32;
  const bool q_ok = qi < nA;
  // pre-multiplied by c = scale * log2(e), so the MFMA yields scores in log2 units
  bf16x8 qf[DH / 16];
  {
    const bf16* qrow = q + (size_t)(q_ok ? qi : nA - 1) * D + h * DH + half * 8;
#pragma unroll
    for (int dk = 0; dk < DH / 16; ++dk) {
      const bf16x8 raw = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + dk * 16));
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[dk][e] = (bf16)((float)raw[e] * c);
    }
  }

  // ---- per-lane LDS read offsets
  // K (A operand of S^T): row kb*32 + l32, chunk 2*dk + half
  uint32_t koff[DH / 16];
#pragma unroll
  for (int dk = 0; dk < DH / 16; ++dk) koff[dk] = (uint32_t)(l32 * ROWB + k_pos<DH>(l32, 2 * dk + half) * 16);
  // V (transposing reads): 16-lane group g points at keys kbase + i/4, dims d0 + 4*(i%4)
  const int grp = lane >> 4, gi = lane & 15;
  const int vrow = 4 * (grp >> 1) + (gi >> 2);   // key within a 8-key step (plus 16*jp + 8*second + 32*kb)
  // LDS byte address of this lane's V read in stage 0, sub-tile 0, with the
  // V region's base (64 KiB at Dh = 128) folded in and hidden from the
  // compiler, so a read's stage and key offsets (< 64 KiB) go into the
  // instruction's offset field instead of an add per read
  uint32_t vrd[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db) {
    const int chunk = 4 * db + 2 * (grp & 1) + ((gi & 3) >> 1);
    vrd[db] = sV_lds + (uint32_t)(vrow * ROWB + v_pos<DH>(vrow, chunk) * 16 + 8 * (gi & 1));
    asm volatile("" : "+v"(vrd[db]));
  }

  f32x16 acc_o[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  float m_run;               // running max of this lane's query, log2 units
  float l_run = 0.f;         // this lane's partial row sum
  f32x16 negm;               // -m_run in every element: the seed of each S^T accumulator
  auto set_negm = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = -m_run;
  };

  // ---- phases of one sub-tile (32 keys: half hb of a 64-key LDS stage)
  // Scores are held relative to the running max: s = c q.k - m_run, which the
  // MFMA produces directly from an accumulator seeded with -m_run.
  // s[r] <-> key 8*(r/4) + 4*half + r%4 of the sub-tile, query l32.
  auto kfrag = [&](const char* kt, int dk) {
    return *reinterpret_cast<const bf16x8*>(kt + koff[dk]);
  };
  // keys past the end of this split's range (its last sub-tile only) get -inf
  auto mask_tail = [&](f32x16& s, int32_t base) {
    if (base + SUB > kv_end) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t key = base + 8 * (r >> 2) + 4 * half + (r & 3);
        if (key >= kv_end) s[r] = -INFINITY;
      }
    }
  };
  // this query's max over the sub-tile (the two lane halves hold half of its keys each)
  auto tile_max = [&](const f32x16& s) {
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  // The running max is not tracked per sub-tile: one whose scores rise far
  // above it shows in its row-sum partial (> kRaiseSum), and only then is the
  // max raised to the sub-tile's, with O, l and the (already shifted) scores
  // of this sub-tile and of the next one moved to the new reference.  Exact
  // after the final division; every probability stays <= 2^32.
  auto raise = [&](f32x16& s_cur, f32x16* s_nxt) {
    const float d = fmaxf(tile_max(s_cur), 0.f);
    const float alpha = __builtin_amdgcn_exp2f(-d);
    m_run += d;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s_cur[r] -= d;
      if (s_nxt != nullptr) (*s_nxt)[r] -= d;
    }
    set_negm();
  };
  // P^T = exp2(s) as bf16 MFMA fragments (packed pairs); row-sum partial in
  // float32 over two independent chains
  auto probs = [&](const f32x16& s, u32x4* pw) {
    float l2[2] = {-0.f, -0.f};   // -0 + x == x: the first adds fold away
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(s[r]);
      const float p1 = __builtin_amdgcn_exp2f(s[r + 1]);
      const bf16x2 pr = {(bf16)p0, (bf16)p1};
      pw[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pr);
      l2[(r >> 1) & 1] += p0 + p1;
    }
    return l2[0] + l2[1];
  };
  // O^T += V^T P^T over the sub-tile: k-step jp covers keys 16*jp + 4*half + {0..3, 8..11}
  auto vfrag = [&](uint32_t vt, int j) {   // vt: sub-tile offset in the V region; j: k-step
    const int jp = j / NDB, db = j % NDB;  // jp = j / NDB, dims block db = j % NDB
    const uint32_t a = vrd[db] + vt + 16 * jp * ROWB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(a + 8 * ROWB));
    const u32x4 raw = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                       __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
    return __builtin_bit_cast(bf16x8, raw);
  };
  auto accumulate = [&](uint32_t vt, const u32x4* pw) {
    bf16x8 vf[2];
    vf[0] = vfrag(vt, 0);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j + 1 < NS) vf[(j + 1) & 1] = vfrag(vt, j + 1);
      acc_o[j % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          vf[j & 1], __builtin_bit_cast(bf16x8, pw[j / NDB]), acc_o[j % NDB], 0, 0, 0);
    }
  };
  // LDS addresses of sub-tile u's K and V rows
  static_assert((NST & (NST - 1)) == 0, "ring of a power-of-two stages");
  auto k_sub = [&](int u) { return sK + ((u >> 1) & (NST - 1)) * TILEB + (u & 1) * SUB * ROWB; };
  auto v_sub = [&](int u) { return (uint32_t)(((u >> 1) & (NST - 1)) * TILEB + (u & 1) * SUB * ROWB); };

  // Q in registers before the LDS pipeline starts (a builtin, so the compiler's own
  // wait accounting sees it and adds no vmcnt waits for Q inside the loop)
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0), expcnt/lgkmcnt unconstrained
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < ntiles)
      issue_tile<DH>(k, v, kv_begin + st * BKV, nkv, D, h, sK_lds + st * TILEB, sV_lds + st * TILEB,
                 voff_k, voff_v, wave);

  // Software pipeline inside each wavefront over 32-key sub-tiles: step u
  // issues the 8 S^T MFMAs of sub-tile u+1 and the 8 PV MFMAs of sub-tile
  // u-1 alternately, with the exp2 / pack / row sum of one score element of
  // sub-tile u next to each, so the VALU work is spread evenly over the MFMA
  // stream.  Before the first sub-tile of a stage is scored, the workgroup
  // synchronises: that stage has landed and every wave is done with the
  // stage two back, which is refilled with the next tile (one load after
  // every second score MFMA of that step).  The LDS ring keeps two stages
  // resident and two in flight.
  // First K and V fragments of a step, read at the end of the one before
  // (kin / vin: this step takes them; kout / vout: this step reads them for
  // the next).  V of the next step's PV is always in a stage already waited
  // for; K of the next step's scores only when that step opens no stage
  // (after an odd step), so only odd steps read K ahead.
  bf16x8 kpre, vpre;
  auto step = [&](f32x16& s_cur, f32x16& s_nxt, u32x4* pw_cur, const u32x4* pw_prev, int u,
                  bool pv, bool kin, bool vin, bool kout, bool vout) {
    TileLoads tl;
    if (u & 1) {
      const int it = u >> 1;   // stage of sub-tile u; sub-tile u+1 opens stage it+1
      if (it + 2 < ntiles) wait_tiles_barrier<DH, 1>();
      else wait_tiles_barrier<DH, 0>();
      // the refill of the stage two back: tile it+NST-1, or past the last
      // tile zero-byte loads into that (free) stage, so the issue needs no
      // branch; its loads are spread over the step's MFMA slots below
      const int ns = (it + NST - 1) & (NST - 1);
      const int32_t r0 = it + NST - 1 < ntiles ? kv_begin + (it + NST - 1) * BKV : nkv;
      tl = tile_loads<DH>(k, v, r0, nkv, D, h, sK_lds + ns * TILEB, sV_lds + ns * TILEB);
    }
    const char* kt = k_sub(u + 1);
    const uint32_t vt = v_sub(u - 1);
    bf16x8 kf[2], vf[2];
    kf[0] = kin ? kpre : kfrag(kt, 0);
    if (pv) vf[0] = vin ? vpre : vfrag(vt, 0);
    float l2[2] = {-0.f, -0.f};   // -0 + x == x: the first adds fold away
    // slot j: S^T MFMA j of sub-tile u+1, the first EPS/2 exponentials of the
    // slot's score elements of sub-tile u, PV MFMA j of sub-tile u-1, the rest
    // of them with their bf16 packing and the row-sum adds
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j + 1 < NS) kf[(j + 1) & 1] = kfrag(kt, j + 1);
      s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j & 1], qf[j], j == 0 ? negm : s_nxt, 0, 0, 0);
      // one refill load after every second score MFMA of an odd step: a
      // wavefront issues in order, and the loads issued together at the
      // step's start held back the MFMAs behind them
      if ((u & 1) && j % 2 == 1 && j / 2 < 2 * LOADS) tile_part(tl, j / 2, voff_k, voff_v, wave);
      float p[EPS];
#pragma unroll
      for (int e = 0; e < EPS / 2; ++e) p[e] = __builtin_amdgcn_exp2f(s_cur[EPS * j + e]);
      if (pv) {
        if (j + 1 < NS) vf[(j + 1) & 1] = vfrag(vt, j + 1);
        acc_o[j % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            vf[j & 1], __builtin_bit_cast(bf16x8, pw_prev[j / NDB]), acc_o[j % NDB], 0, 0, 0);
      }
#pragma unroll
      for (int e = EPS / 2; e < EPS; ++e) p[e] = __builtin_amdgcn_exp2f(s_cur[EPS * j + e]);
#pragma unroll
      for (int pr = 0; pr < EPS / 2; ++pr) {
        const int r = EPS * j + 2 * pr;   // score elements r, r+1 of sub-tile u
        const bf16x2 pk = {(bf16)p[2 * pr], (bf16)p[2 * pr + 1]};
        pw_cur[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
        l2[(j * (EPS / 2) + pr) & 1] += p[2 * pr] + p[2 * pr + 1];
      }
    }
    if (vout) vpre = vfrag(v_sub(u), 0);
    if (kout) kpre = kfrag(k_sub(u + 2), 0);
    float lt = l2[0] + l2[1];
    if (__ballot(lt > kRaiseSum) != 0ull) {   // after PV(u-1): O is complete up to sub-tile u-1
      raise(s_cur, &s_nxt);
      lt = probs(s_cur, pw_cur);
    }
    l_run += lt;
  };

  f32x16 sa, sb;
  u32x4 pwa[2], pwb[2];   // P^T fragments (packed bf16 pairs) of two consecutive sub-tiles
  if (min(NST - 2, ntiles - 1) >= 2) wait_tiles_barrier<DH, 2>();
  else if (ntiles - 1 >= 1) wait_tiles_barrier<DH, 1>();
  else wait_tiles_barrier<DH, 0>();
  // first sub-tile: unshifted scores, whose max is the initial reference
  {
    const char* kt = k_sub(0);
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = 0.f;
#pragma unroll
    for (int dk = 0; dk < DH / 16; ++dk)
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(kt, dk), qf[dk], sa, 0, 0, 0);
  }
  mask_tail(sa, kv_begin);
  m_run = tile_max(sa);
#pragma unroll
  for (int r = 0; r < 16; ++r) sa[r] -= m_run;
  set_negm();
  // last sub-tile u: its softmax, then the PV of sub-tiles u-1 (if pv) and u
  auto finish = [&](f32x16& s_cur, u32x4* pw_cur, const u32x4* pw_prev, int u, bool pv) {
    mask_tail(s_cur, kv_begin + u * SUB);
    if (pv) accumulate(v_sub(u - 1), pw_prev);
    float lt = probs(s_cur, pw_cur);
    if (__ballot(lt > kRaiseSum) != 0ull) {
      raise(s_cur, nullptr);
      lt = probs(s_cur, pw_cur);
    }
    l_run += lt;
    accumulate(v_sub(u), pw_cur);
  };
  const int nsub = (kv_end - kv_begin + SUB - 1) / SUB;
  if (nsub == 1) {
    finish(sa, pwa, pwb, 0, false);
  } else {
    step(sa, sb, pwa, pwb, 0, false, false, false, false, true);
    int u = 1;
    // whole ring cycles (2 * NST sub-tiles) unrolled from u = 1 mod 2 * NST:
    // every stage offset is then a constant that the LDS reads carry as an
    // immediate, instead of address arithmetic in each step
    for (int cyc = 0; 2 * NST * cyc + 2 * NST + 1 < nsub; ++cyc) {
      const int u0 = 2 * NST * cyc + 1;
#pragma unroll
      for (int c = 0; c < 2 * NST; c += 2) {
        step(sb, sa, pwb, pwa, u0 + c, true, false, true, true, true);
        step(sa, sb, pwa, pwb, u0 + c + 1, true, true, true, false, true);
      }
      u = u0 + 2 * NST;
    }
    for (; u + 2 < nsub; u += 2) {
      step(sb, sa, pwb, pwa, u, true, false, true, true, true);
      step(sa, sb, pwa, pwb, u + 1, true, true, true, false, true);
    }
    // one step more when two sub-tiles remain; its scores and P^T are then
    // moved into the roles of the single finish below (a finish inlined once
    // per parity leaves the registers of the two copies in swapped roles,
    // which the allocator resolves with spills)
    if (u + 1 < nsub) {
      step(sb, sa, pwb, pwa, u, true, false, true, false, false);
      sb = sa;
      pwa[0] = pwb[0];
      pwa[1] = pwb[1];
      ++u;
    }
    finish(sb, pwb, pwa, u, true);
  }

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // zero-byte tile loads land before exit
  float l_tot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (!q_ok) return;
  // acc_o[db][r] <-> dim db*32 + 8*(r/4) + 4*half + r%4, query l32
  // acc_o[db][r] <-> dim db*32 + 8*(r/4) + 4*half + r%4, query l32; the
  // split partials are stored normalised (O / l, bf16) with their (m, l)
  const float inv = 1.0f / l_tot;
  // partial row of a split item: (part, split item, query within the tile)
  const size_t prow = ((size_t)sp * L + il) * BQ + (qi - qt * BQ);
  bf16* orow = split ? part_o + prow * DH : o + (size_t)qi * D + h * DH;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (bf16)(acc_o[db][4 * j + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * j + 4 * half) = w4;
    }
  if (split && half == 0) {
    part_ml[prow * 2 + 0] = m_run;
    part_ml[prow * 2 + 1] = l_tot;
  }
}

#define HSA_ATTN_ARGS                                                                        \
  const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,        \
      bf16 *__restrict__ o, bf16 *__restrict__ part_o, float *__restrict__ part_ml, int32_t nA, \
      int32_t nkv, int32_t H, float c, int32_t n_qt, int32_t n_full, int32_t splits,         \
      int32_t tiles_per_split

__global__ __launch_bounds__(kAttnThreads, 1) void attn_bf16_d128_kernel(HSA_ATTN_ARGS) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * NST * AttnShape<128>::TILEB];
  attn_bf16_body<128>(q, k, v, o, part_o, part_ml, nA, nkv, H, c, n_qt, n_full, splits,
                      tiles_per_split, smem);
}

__global__ __launch_bounds__(kAttnThreads, 1) void attn_bf16_d64_kernel(HSA_ATTN_ARGS) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * NST * AttnShape<64>::TILEB];
  attn_bf16_body<64>(q, k, v, o, part_o, part_ml, nA, nkv, H, c, n_qt, n_full, splits,
                     tiles_per_split, smem);
}
#undef HSA_ATTN_ARGS

// Merge split partials in split order: with weights w_s = l_s 2^(m_s - M),
// O = sum_s w_s (O_s / l_s) / sum_s w_s.  One thread per 8 dims of a query row
// of a split item (items n_full .. n_qt * H - 1): 16-byte partial reads and
// output writes.
template <int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(const bf16* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         bf16* __restrict__ o, int32_t nA,
                                                         int32_t H, int32_t n_qt, int32_t n_full,
                                                         int32_t splits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t L = n_qt * H - n_full;
  const int64_t rows = (int64_t)L * BQ;
  const int64_t row = t / (HD / 8);   // il * BQ + query within the tile
  const int d8 = (int)(t % (HD / 8)) * 8;
  if (row >= rows) return;
  const int32_t il = (int32_t)(row / BQ), qin = (int32_t)(row % BQ);
  const int32_t item = n_full + il;
  const int32_t qt = item % n_qt, h = item / n_qt;
  const int32_t qi = qt * BQ + qin;
  if (qi >= nA) return;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[((size_t)s * rows + row) * 2]);
  float Lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const size_t pr = (size_t)s * rows + row;
    const float w = __builtin_amdgcn_exp2f(part_ml[pr * 2] - M) * part_ml[pr * 2 + 1];
    Lsum += w;
    const bf16x8 po = *reinterpret_cast<const bf16x8*>(part_o + pr * HD + d8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w, (float)po[e], acc[e]);
  }
  const float inv = 1.0f / Lsum;
  bf16x8 w8;
#pragma unroll
  for (int e = 0; e < 8; ++e) w8[e] = (bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x8*>(o + (size_t)qi * H * HD + h * HD + d8) = w8;
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
  int32_t n_qt, n_full, splits, tiles_per_split;
  // partial rows: every part of every split item, BQ rows each
  int64_t part_rows(int32_t H) const {
    return splits > 1 ? (int64_t)splits * (n_qt * H - n_full) * BQ : 0;
  }
};

// One workgroup per CU at a time (128 KiB of LDS each).  Items (query tile,
// head) take `ntiles` KV tiles each.  Candidates: n_full items in whole
// rounds of 256 run unsplit, the remaining L items split into s parts; the
// cost is the rounds times the tiles per workgroup, plus one tile per
// partial row block merged.  The cheapest candidate wins; ties go to the
// fewest split items, then the fewest parts.  Every part covers >= 8 tiles.
SplitPlan plan_split(int32_t nA, int32_t nkv, int32_t H) {
  constexpr int32_t kCus = 256;
  SplitPlan p;
  p.n_qt = cdiv(nA, BQ);
  const int32_t ntiles = cdiv(nkv, BKV);
  const int32_t items = p.n_qt * H;
  const int32_t smax = max(1, min(16, ntiles / 8));
  int64_t best = -1;
  p.n_full = items;
  p.splits = 1;
  for (int32_t nf = (items / kCus) * kCus; nf >= 0; nf -= kCus) {
    const int32_t L = items - nf;
    for (int32_t s = 1; s <= smax; ++s) {
      if (L == 0 && s > 1) break;
      const int32_t tps = cdiv(ntiles, s);
      const int64_t cost = (int64_t)(nf / kCus) * ntiles + (int64_t)cdiv((int64_t)L * s, kCus) * tps +
                           (s > 1 ? (int64_t)L * s / kCus : 0);
      if (best < 0 || cost < best) {
        best = cost;
        p.n_full = nf;
        p.splits = s;
      }
    }
  }
  if (p.splits == 1) p.n_full = items;   // nothing split
  p.tiles_per_split = cdiv(ntiles, p.splits);
  p.splits = cdiv(ntiles, p.tiles_per_split);
  if (p.splits == 1) p.n_full = items;
  return p;
}

bool use_mfma_path(int32_t Dh, hsa_dtype dt) { return dt == HSA_BF16 && (Dh == 128 || Dh == 64); }

}  // namespace

size_t attn_workspace_bytes(int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh) {
  if (n_active <= 0 || n_kv <= 0) return 0;
  const SplitPlan p = plan_split(n_active, n_kv, H);
  if (p.splits <= 1) return 0;
  const size_t rows = (size_t)p.part_rows(H);
  return align_up(rows * Dh * sizeof(bf16), 256) + rows * 2 * sizeof(float);
}

hsa_status launch_attention(const void* q, const void* k, const void* v, void* o,
                            int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh, float scale,
                            hsa_dtype dt, void* ws, size_t ws_bytes, hipStream_t s) {
  if (n_active == 0) return HSA_OK;
  if (use_mfma_path(Dh, dt)) {
    const SplitPlan p = plan_split(n_active, n_kv, H);
    bf16* part_o = nullptr;
    float* part_ml = nullptr;
    if (p.splits > 1) {
      const size_t rows = (size_t)p.part_rows(H);
      if (ws == nullptr || ws_bytes < attn_workspace_bytes(n_active, n_kv, H, Dh))
        return HSA_ERR_WORKSPACE;
      part_o = (bf16*)ws;
      part_ml = (float*)((char*)ws + align_up(rows * Dh * sizeof(bf16), 256));
    }
    const int32_t total = p.n_full + (p.n_qt * H - p.n_full) * p.splits;
    if (Dh == 128)
      attn_bf16_d128_kernel<<<total, kAttnThreads, 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, part_o, part_ml, n_active,
          n_kv, H, scale * kLog2e, p.n_qt, p.n_full, p.splits, p.tiles_per_split);
    else
      attn_bf16_d64_kernel<<<total, kAttnThreads, 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, part_o, part_ml, n_active,
          n_kv, H, scale * kLog2e, p.n_qt, p.n_full, p.splits, p.tiles_per_split);
    if (p.splits > 1) {
      const int64_t threads = (int64_t)(p.n_qt * H - p.n_full) * BQ * (Dh / 8);
      const unsigned blocks = (unsigned)((threads + 255) / 256);
      if (Dh == 128)
        attn_merge_kernel<128><<<blocks, 256, 0, s>>>(part_o, part_ml, (bf16*)o, n_active, H, p.n_qt,
                                                       p.n_full, p.splits);
      else
        attn_merge_kernel<64><<<blocks, 256, 0, s>>>(part_o, part_ml, (bf16*)o, n_active, H, p.n_qt,
                                                      p.n_full, p.splits);
    }
    return launch_status();
  }
  dim3 grid(cdiv(n_active, 64), H);
  if (dt == HSA_BF16) {
    return HSA_ERR_SHAPE;   // bf16 takes the MFMA path for every supported head width
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

