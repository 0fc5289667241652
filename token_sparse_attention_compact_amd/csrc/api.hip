// Host side of libhsa: argument validation, workspace layout and the order
// of launches that makes one HSA iteration.  No device allocation, no device
// synchronisation: |A_i| is computed on the host in closed form from the
// group sizes (activity rule of section 2.1), so every launch size is known
// before anything runs.
#include <math.h>
#include <string.h>

#include "common.h"

using namespace hsa;

namespace {

constexpr int32_t kAbiVersion = HSA_ABI_VERSION;

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool valid_dtype(hsa_dtype t) { return t == HSA_F32 || t == HSA_BF16; }

constexpr int32_t kAllFeatures = HSA_FEAT_QK_NORM | HSA_FEAT_ROPE3D | HSA_FEAT_ADALN | HSA_FEAT_CFG;
bool has(const hsa_dims& d, int32_t feature) { return (d.features & feature) != 0; }

// bf16 GEMM and attention operands are read through buffer descriptors whose
// size and offsets are 32-bit: a whole operand must stay below 4 GiB.
bool fits_buffer(int64_t bytes) { return bytes < ((int64_t)1 << 32); }

hsa_status check_dims(const hsa_dims* d) {
  if (!d) return HSA_ERR_ARG;
  if (!valid_dtype(d->dtype)) return HSA_ERR_DTYPE;
  if (d->N <= 0 || d->C <= 0 || d->D <= 0 || d->H <= 0 || d->Dh <= 0 || d->F <= 0 || d->L <= 0 ||
      d->n_text < 0)
    return HSA_ERR_SHAPE;
  if (d->D != d->H * d->Dh) return HSA_ERR_SHAPE;
  if (d->Dh != 64 && d->Dh != 128) return HSA_ERR_SHAPE;
  if (d->C % 4 != 0) return HSA_ERR_SHAPE;
  if (d->dtype == HSA_BF16 && (d->D % 64 != 0 || d->F % 64 != 0)) return HSA_ERR_SHAPE;
  if (d->dtype == HSA_BF16 && !fits_buffer((int64_t)d->N * (d->D > d->F ? d->D : d->F) * 2))
    return HSA_ERR_SHAPE;
  if (d->dtype == HSA_F32 && (d->D % 4 != 0 || d->F % 4 != 0)) return HSA_ERR_SHAPE;
  if (d->features & ~kAllFeatures) return HSA_ERR_ARG;
  if ((d->features & HSA_FEAT_ROPE3D) &&
      (d->grid_f <= 0 || d->grid_h <= 0 || d->grid_w <= 0 ||
       (int64_t)d->grid_f * d->grid_h * d->grid_w != d->N))
    return HSA_ERR_SHAPE;
  if ((d->features & HSA_FEAT_CFG) && d->n_text <= 0) return HSA_ERR_ARG;
  return HSA_OK;
}

hsa_status check_schedule(const hsa_schedule* s, int32_t N) {
  if (!s) return HSA_ERR_ARG;
  if (s->T <= 0 || s->K < 1 || s->K > HSA_MAX_GROUPS || s->m < 0) return HSA_ERR_SCHEDULE;
  if (s->budget[0] != s->T) return HSA_ERR_SCHEDULE;
  int64_t sum = 0;
  for (int k = 0; k < s->K; ++k) {
    if (s->budget[k] <= 0 || s->T % s->budget[k] != 0) return HSA_ERR_SCHEDULE;
    if (s->count[k] < 0) return HSA_ERR_SCHEDULE;
    sum += s->count[k];
  }
  if (sum != N) return HSA_ERR_SCHEDULE;
  return HSA_OK;
}

bool in_window(const hsa_schedule* s, int32_t iter) { return iter < s->m || iter >= s->T - s->m; }

// Bit k set iff group k is active at `iter`.
uint32_t active_group_mask(const hsa_schedule* s, int32_t iter) {
  uint32_t mask = 0;
  for (int k = 0; k < s->K; ++k) {
    const int32_t period = s->T / s->budget[k];
    if (in_window(s, iter) || iter % period == 0) mask |= 1u << k;
  }
  return mask;
}

int32_t n_active_of(const hsa_schedule* s, int32_t iter) {
  const uint32_t mask = active_group_mask(s, iter);
  int32_t n = 0;
  for (int k = 0; k < s->K; ++k)
    if (mask & (1u << k)) n += s->count[k];
  return n;
}

#define CHECK_PTR(p)                        \
  do {                                      \
    if (!(p)) return HSA_ERR_ARG;           \
    if (!aligned16(p)) return HSA_ERR_ALIGN; \
  } while (0)

#define RETURN_IF(st)               \
  do {                              \
    const hsa_status _s = (st);     \
    if (_s != HSA_OK) return _s;    \
  } while (0)

// ---- workspace layout of hsa_step / hsa_block_forward ----
struct Layout {
  size_t h, a, q, o, u, v_new, n_active, attn, total;
  size_t attn_bytes;
  size_t temb;    // HSA_FEAT_ADALN: e [D] then e0 [6][D], float32
  size_t v_cond;  // HSA_FEAT_CFG: conditional-branch velocity [N][C], float32
};

size_t attn_ws_max(int32_t n_rows, int32_t n_kv, int32_t H, int32_t Dh) {
  // The split plan depends on the number of 128-query tiles; take the worst case.
  size_t best = 0;
  for (int32_t nq = 128; nq < n_rows + 128; nq += 128) {
    const int32_t rows = nq < n_rows ? nq : n_rows;
    const size_t b = attn_workspace_bytes(rows, n_kv, H, Dh);
    if (b > best) best = b;
  }
  return best;
}

Layout layout_of(const hsa_dims* d) {
  Layout L{};
  const size_t es = dtype_size(d->dtype);
  const size_t N = (size_t)d->N;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L.h = take(N * d->D * sizeof(float));
  L.a = take(N * d->D * es);
  L.q = take(N * d->D * es);
  L.o = take(N * d->D * es);
  L.u = take(N * d->F * es);
  L.v_new = take(N * d->C * sizeof(float));
  L.n_active = take(sizeof(int32_t));
  size_t ab = attn_ws_max(d->N, d->N, d->H, d->Dh);
  if (d->n_text > 0) {
    const size_t ax = attn_ws_max(d->N, d->n_text, d->H, d->Dh);
    if (ax > ab) ab = ax;
  }
  L.attn_bytes = ab;
  L.attn = take(ab > 0 ? ab : 16);
  L.temb = has(*d, HSA_FEAT_ADALN) ? take((size_t)7 * d->D * sizeof(float)) : 0;
  L.v_cond = has(*d, HSA_FEAT_CFG) ? take(N * d->C * sizeof(float)) : 0;
  L.total = off;
  return L;
}

hsa_status check_time_weights(const hsa_model* m) {
  CHECK_PTR(m->t_w1);
  CHECK_PTR(m->t_b1);
  CHECK_PTR(m->t_w2);
  CHECK_PTR(m->t_b2);
  CHECK_PTR(m->t_w3);
  CHECK_PTR(m->t_b3);
  CHECK_PTR(m->head_mod);
  return HSA_OK;
}

hsa_status check_model(const hsa_model* m) {
  if (!m) return HSA_ERR_ARG;
  RETURN_IF(check_dims(&m->dims));
  CHECK_PTR(m->w_in);
  CHECK_PTR(m->w_out);
  if (!m->blocks) return HSA_ERR_ARG;
  for (int l = 0; l < m->dims.L; ++l) {
    const hsa_block& b = m->blocks[l];
    CHECK_PTR(b.w_qkv);
    CHECK_PTR(b.w_o);
    CHECK_PTR(b.w_1);
    CHECK_PTR(b.w_2);
    CHECK_PTR(b.k_cache);
    CHECK_PTR(b.v_cache);
    if (m->dims.n_text > 0) {
      CHECK_PTR(b.w_qx);
      CHECK_PTR(b.w_ox);
      CHECK_PTR(b.k_text);
      CHECK_PTR(b.v_text);
    }
    if (has(m->dims, HSA_FEAT_QK_NORM)) {
      CHECK_PTR(b.q_gain);
      CHECK_PTR(b.k_gain);
    }
    if (has(m->dims, HSA_FEAT_ADALN)) CHECK_PTR(b.mod);
    if (has(m->dims, HSA_FEAT_CFG)) {
      CHECK_PTR(b.k_text_u);
      CHECK_PTR(b.v_text_u);
      CHECK_PTR(b.k_cache_u);
      CHECK_PTR(b.v_cache_u);
    }
  }
  if (has(m->dims, HSA_FEAT_ADALN)) RETURN_IF(check_time_weights(m));
  if (has(m->dims, HSA_FEAT_CFG) && !isfinite(m->cfg_scale)) return HSA_ERR_ARG;
  return HSA_OK;
}

// One block on nA active rows.  e0 [6][D]: timestep projection (adaLN only);
// branch 1: the unconditional text set and caches (guidance only).
hsa_status block_forward_impl(const hsa_model* m, int32_t layer, float* h,
                              const int32_t* active_idx, int32_t nA, const float* e0,
                              int32_t branch, char* ws, const Layout& L, hipStream_t s) {
  if (nA == 0) return HSA_OK;
  const hsa_dims& d = m->dims;
  const hsa_block& b = m->blocks[layer];
  const hsa_dtype dt = d.dtype;
  void* a = ws + L.a;
  void* q = ws + L.q;
  void* o = ws + L.o;
  void* u = ws + L.u;
  void* attn_ws = ws + L.attn;
  const float scale = 1.0f / sqrtf((float)d.Dh);
  const bool adaln = has(d, HSA_FEAT_ADALN);
  void* kc = branch ? b.k_cache_u : b.k_cache;
  void* vc = branch ? b.v_cache_u : b.v_cache;
  const void* kt = branch ? b.k_text_u : b.k_text;
  const void* vt = branch ? b.v_text_u : b.v_text;
  // row k of the block's modulation: mod[k] + e0[k] (absent without adaLN)
  auto mod = [&](int k) {
    return adaln ? ModVec{b.mod + (size_t)k * d.D, e0 + (size_t)k * d.D} : ModVec{nullptr, nullptr};
  };
  const ModVec none{nullptr, nullptr};
  const int epi_res = adaln ? EPI_RESID_GATED : EPI_RESID;

  // KV-cache synchronisation: QKV on active rows, fresh K/V scattered into the cache
  RETURN_IF(launch_layernorm(h, a, nA, d.D, dt, mod(0), mod(1), s));
  EpiArgs e_qkv{q, nullptr, kc, vc, active_idx, d.D, none};
  RETURN_IF(launch_gemm(a, b.w_qkv, nA, 3 * d.D, d.D, dt, EPI_QKV_SCATTER, e_qkv, s));
  // qk-RMSNorm / rotary embedding of the fresh q rows and cache rows
  const bool norm = has(d, HSA_FEAT_QK_NORM), rope = has(d, HSA_FEAT_ROPE3D);
  if (norm || rope)
    RETURN_IF(launch_qk_norm_rope(q, kc, active_idx, nA, d.D, d.Dh, dt, norm, rope, b.q_gain,
                                  b.k_gain, d.grid_h, d.grid_w, s));
  // active queries over all N cached rows
  RETURN_IF(launch_attention(q, kc, vc, o, nA, d.N, d.H, d.Dh, scale, dt, attn_ws, L.attn_bytes, s));
  EpiArgs e_res{nullptr, h, nullptr, nullptr, nullptr, 0, mod(2)};
  RETURN_IF(launch_gemm(o, b.w_o, nA, d.D, d.D, dt, epi_res, e_res, s));
  if (d.n_text > 0) {
    RETURN_IF(launch_layernorm(h, a, nA, d.D, dt, none, none, s));
    EpiArgs e_q{q, nullptr, nullptr, nullptr, nullptr, 0, none};
    RETURN_IF(launch_gemm(a, b.w_qx, nA, d.D, d.D, dt, EPI_STORE, e_q, s));
    RETURN_IF(launch_attention(q, kt, vt, o, nA, d.n_text, d.H, d.Dh, scale, dt, attn_ws,
                               L.attn_bytes, s));
    EpiArgs e_x{nullptr, h, nullptr, nullptr, nullptr, 0, none};
    RETURN_IF(launch_gemm(o, b.w_ox, nA, d.D, d.D, dt, EPI_RESID, e_x, s));
  }
  RETURN_IF(launch_layernorm(h, a, nA, d.D, dt, mod(3), mod(4), s));
  EpiArgs e_up{u, nullptr, nullptr, nullptr, nullptr, 0, none};
  RETURN_IF(launch_gemm(a, b.w_1, nA, d.F, d.D, dt, EPI_GELU, e_up, s));
  EpiArgs e_down{nullptr, h, nullptr, nullptr, nullptr, 0, mod(5)};
  RETURN_IF(launch_gemm(u, b.w_2, nA, d.D, d.F, dt, epi_res, e_down, s));
  return HSA_OK;
}

hsa_status check_gemm_shape(int32_t M, int32_t N, int32_t K, hsa_dtype dt) {
  if (!valid_dtype(dt)) return HSA_ERR_DTYPE;
  if (M < 0 || N <= 0 || K <= 0) return HSA_ERR_SHAPE;
  if (dt == HSA_BF16 && (K % 64 != 0 || N % 4 != 0)) return HSA_ERR_SHAPE;
  if (dt == HSA_BF16 && (!fits_buffer((int64_t)M * K * 2) || !fits_buffer((int64_t)N * K * 2)))
    return HSA_ERR_SHAPE;
  if (dt == HSA_F32 && K % 4 != 0) return HSA_ERR_SHAPE;
  return HSA_OK;
}

}  // namespace

extern "C" {

const char* hsa_status_str(int32_t status) {
  switch (status) {
    case HSA_OK: return "ok";
    case HSA_ERR_ARG: return "invalid argument (null pointer, negative size or bad flag)";
    case HSA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case HSA_ERR_DTYPE: return "unsupported dtype";
    case HSA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case HSA_ERR_WORKSPACE: return "workspace missing or too small";
    case HSA_ERR_HIP: return "HIP runtime error";
    case HSA_ERR_SCHEDULE: return "invalid schedule (budgets must divide T, budget[0] == T, counts sum to N)";
    case HSA_ERR_TOO_LARGE:
      return "problem needs more scratch than the allocation-free entry point's fixed array "
             "(HSA_NOALLOC_SCRATCH_BYTES); call the entry point that takes a workspace";
    default: return "unknown status";
  }
}

int32_t hsa_abi_version(void) { return kAbiVersion; }

hsa_status hsa_workspace_size(const hsa_dims* dims, size_t* bytes) {
  if (!bytes) return HSA_ERR_ARG;
  RETURN_IF(check_dims(dims));
  *bytes = layout_of(dims).total;
  return HSA_OK;
}

hsa_status hsa_attn_workspace_size(int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh,
                                   size_t* bytes) {
  if (!bytes) return HSA_ERR_ARG;
  if (n_active < 0 || n_kv <= 0 || H <= 0 || (Dh != 64 && Dh != 128)) return HSA_ERR_SHAPE;
  *bytes = attn_workspace_bytes(n_active, n_kv, H, Dh);
  return HSA_OK;
}

hsa_status hsa_select_workspace_size(int32_t N, int32_t K, size_t* bytes) {
  if (!bytes) return HSA_ERR_ARG;
  if (N < 0 || K < 1 || K > HSA_MAX_GROUPS) return HSA_ERR_SHAPE;
  *bytes = 0;
  return HSA_OK;
}

hsa_status hsa_n_active(const hsa_schedule* sched, int32_t iter, int32_t* n_active) {
  if (!sched || !n_active) return HSA_ERR_ARG;
  int64_t N = 0;
  for (int k = 0; k < sched->K && k < HSA_MAX_GROUPS; ++k) N += sched->count[k];
  RETURN_IF(check_schedule(sched, (int32_t)N));
  if (iter < 0 || iter >= sched->T) return HSA_ERR_ARG;
  *n_active = n_active_of(sched, iter);
  return HSA_OK;
}

hsa_status hsa_active_set(const uint8_t* group, int32_t N, const hsa_schedule* sched,
                          int32_t iter, int32_t* active_idx, int32_t* pos, int32_t* n_active_dev,
                          void* stream) {
  if (N <= 0) return HSA_ERR_SHAPE;
  RETURN_IF(check_schedule(sched, N));
  if (iter < 0 || iter >= sched->T) return HSA_ERR_ARG;
  if (!group || !active_idx || !pos || !n_active_dev) return HSA_ERR_ARG;
  if (!aligned16(active_idx) || !aligned16(pos)) return HSA_ERR_ALIGN;
  return launch_active_set(group, N, active_group_mask(sched, iter), n_active_of(sched, iter),
                           active_idx, pos, n_active_dev, as_stream(stream));
}

namespace {
hsa_status check_counts(int32_t N, const int32_t* count, int32_t K) {
  if (K < 1 || K > HSA_MAX_GROUPS) return HSA_ERR_SHAPE;
  if (!count) return HSA_ERR_ARG;
  int64_t sum = 0;
  for (int k = 0; k < K; ++k) {
    if (count[k] < 0) return HSA_ERR_SCHEDULE;
    sum += count[k];
  }
  return sum == N ? HSA_OK : HSA_ERR_SCHEDULE;
}
}  // namespace

hsa_status hsa_select(const float* score, int32_t N, const int32_t* count, int32_t K,
                      uint8_t* group_out, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (N <= 0 || K < 1 || K > HSA_MAX_GROUPS) return HSA_ERR_SHAPE;
  if (!score || !count || !group_out) return HSA_ERR_ARG;
  RETURN_IF(check_counts(N, count, K));
  return launch_select(score, 1, N, count, K, group_out, as_stream(stream));
}

hsa_status hsa_select_batch(const float* score, int32_t B, int32_t N, const int32_t* count,
                            int32_t K, uint8_t* group_out, void* stream) {
  if (B <= 0 || N <= 0 || K < 1 || K > HSA_MAX_GROUPS) return HSA_ERR_SHAPE;
  if ((int64_t)B * N > ((int64_t)1 << 38)) return HSA_ERR_SHAPE;   // grid limits of the fill path
  if (!score || !count || !group_out) return HSA_ERR_ARG;
  RETURN_IF(check_counts(N, count, K));
  return launch_select(score, B, N, count, K, group_out, as_stream(stream));
}

hsa_status hsa_euler(float* x, float* v_hat, float* score, const float* v_new, const int32_t* pos,
                     int32_t N, int32_t C, float dsigma, float eps, int32_t update_score,
                     void* stream) {
  if (N < 0 || C <= 0 || C % 4 != 0) return HSA_ERR_SHAPE;
  if (N == 0) return HSA_OK;
  CHECK_PTR(x);
  CHECK_PTR(v_hat);
  CHECK_PTR(score);
  CHECK_PTR(pos);
  if (v_new && !aligned16(v_new)) return HSA_ERR_ALIGN;
  if (update_score != 0 && update_score != 1) return HSA_ERR_ARG;
  // v_new may be NULL only when no token is active; the kernel reads it for pos >= 0.
  return launch_euler(x, v_hat, score, v_new, pos, N, C, dsigma, eps, update_score,
                      as_stream(stream));
}

hsa_status hsa_attn_active(const void* q, const void* k, const void* v, void* o,
                           int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh, float scale,
                           hsa_dtype dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return HSA_ERR_DTYPE;
  if (n_active < 0 || n_kv <= 0 || H <= 0 || (Dh != 64 && Dh != 128)) return HSA_ERR_SHAPE;
  if (dtype == HSA_BF16 && !fits_buffer((int64_t)n_kv * H * Dh * 2)) return HSA_ERR_SHAPE;
  if (n_active == 0) return HSA_OK;
  CHECK_PTR(q);
  CHECK_PTR(k);
  CHECK_PTR(v);
  CHECK_PTR(o);
  if (!(scale > 0.f) || !isfinite(scale)) return HSA_ERR_ARG;
  const size_t need = attn_workspace_bytes(n_active, n_kv, H, Dh);
  if (dtype == HSA_BF16 && need > 0) {
    if (!ws || ws_bytes < need) return HSA_ERR_WORKSPACE;
    if (!aligned16(ws)) return HSA_ERR_ALIGN;
  }
  return launch_attention(q, k, v, o, n_active, n_kv, H, Dh, scale, dtype, ws, ws_bytes,
                          as_stream(stream));
}

hsa_status hsa_layernorm(const float* h, void* out, int32_t rows, int32_t D, const float* shift,
                         const float* scale, hsa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return HSA_ERR_DTYPE;
  if (rows < 0 || D <= 0 || D % 4 != 0) return HSA_ERR_SHAPE;
  if ((shift == nullptr) != (scale == nullptr)) return HSA_ERR_ARG;
  if (rows == 0) return HSA_OK;
  CHECK_PTR(h);
  CHECK_PTR(out);
  if (shift) {
    CHECK_PTR(shift);
    CHECK_PTR(scale);
  }
  return launch_layernorm(h, out, rows, D, dtype, ModVec{shift, nullptr}, ModVec{scale, nullptr},
                          as_stream(stream));
}

hsa_status hsa_embed(const float* x, const int32_t* active_idx, const void* w_in, float* h,
                     int32_t n_active, int32_t C, int32_t D, hsa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return HSA_ERR_DTYPE;
  if (n_active < 0 || C <= 0 || D <= 0) return HSA_ERR_SHAPE;
  if (n_active == 0) return HSA_OK;
  CHECK_PTR(x);
  CHECK_PTR(active_idx);
  CHECK_PTR(w_in);
  CHECK_PTR(h);
  return launch_embed(x, active_idx, w_in, h, n_active, C, D, dtype, as_stream(stream));
}

hsa_status hsa_unembed(const float* h, const void* w_out, float* v_new, int32_t n_active,
                       int32_t D, int32_t C, const float* shift, const float* scale,
                       hsa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return HSA_ERR_DTYPE;
  if (n_active < 0 || C <= 0 || D <= 0 || D % 4 != 0) return HSA_ERR_SHAPE;
  if ((shift == nullptr) != (scale == nullptr)) return HSA_ERR_ARG;
  if (n_active == 0) return HSA_OK;
  CHECK_PTR(h);
  CHECK_PTR(w_out);
  CHECK_PTR(v_new);
  if (shift) {
    CHECK_PTR(shift);
    CHECK_PTR(scale);
  }
  return launch_unembed(h, w_out, v_new, n_active, D, C, dtype, ModVec{shift, nullptr},
                        ModVec{scale, nullptr}, as_stream(stream));
}

hsa_status hsa_linear(const void* a, const void* w, void* out, int32_t M, int32_t Nout, int32_t K,
                      int32_t act, hsa_dtype dtype, void* stream) {
  RETURN_IF(check_gemm_shape(M, Nout, K, dtype));
  if (act != 0 && act != 1) return HSA_ERR_ARG;
  if (M == 0) return HSA_OK;
  CHECK_PTR(a);
  CHECK_PTR(w);
  CHECK_PTR(out);
  EpiArgs e{out, nullptr, nullptr, nullptr, nullptr, 0, ModVec{nullptr, nullptr}};
  return launch_gemm(a, w, M, Nout, K, dtype, act ? EPI_GELU : EPI_STORE, e, as_stream(stream));
}

hsa_status hsa_linear_residual(const void* a, const void* w, float* h, int32_t M, int32_t Nout,
                               int32_t K, const float* gate, hsa_dtype dtype, void* stream) {
  RETURN_IF(check_gemm_shape(M, Nout, K, dtype));
  if (M == 0) return HSA_OK;
  CHECK_PTR(a);
  CHECK_PTR(w);
  CHECK_PTR(h);
  if (gate) CHECK_PTR(gate);
  EpiArgs e{nullptr, h, nullptr, nullptr, nullptr, 0, ModVec{gate, nullptr}};
  return launch_gemm(a, w, M, Nout, K, dtype, gate ? EPI_RESID_GATED : EPI_RESID, e,
                     as_stream(stream));
}

hsa_status hsa_qkv_scatter(const void* a, const int32_t* active_idx, int32_t gather,
                           const void* w_qkv, void* q_out, void* k_cache, void* v_cache,
                           int32_t n_active, int32_t N, int32_t D, hsa_dtype dtype, void* stream) {
  RETURN_IF(check_gemm_shape(n_active, 3 * D, D, dtype));
  if (n_active > N || N <= 0) return HSA_ERR_SHAPE;
  if (gather != 0 && gather != 1) return HSA_ERR_ARG;
  if (gather && dtype == HSA_BF16 && !fits_buffer((int64_t)N * D * 2)) return HSA_ERR_SHAPE;
  if (n_active == 0) return HSA_OK;
  CHECK_PTR(a);
  CHECK_PTR(active_idx);
  CHECK_PTR(w_qkv);
  CHECK_PTR(q_out);
  CHECK_PTR(k_cache);
  CHECK_PTR(v_cache);
  EpiArgs e{q_out, nullptr, k_cache, v_cache, active_idx, D, ModVec{nullptr, nullptr}, gather ? N : 0};
  return launch_gemm(a, w_qkv, n_active, 3 * D, D, dtype, EPI_QKV_SCATTER, e, as_stream(stream));
}

hsa_status hsa_qk_norm_rope(void* q, void* k_cache, const int32_t* active_idx, int32_t n_active,
                            const hsa_dims* dims, const float* q_gain, const float* k_gain,
                            void* stream) {
  RETURN_IF(check_dims(dims));
  if (n_active < 0 || n_active > dims->N) return HSA_ERR_SHAPE;
  const bool norm = has(*dims, HSA_FEAT_QK_NORM), rope = has(*dims, HSA_FEAT_ROPE3D);
  if (n_active == 0 || (!norm && !rope)) return HSA_OK;
  CHECK_PTR(q);
  CHECK_PTR(k_cache);
  CHECK_PTR(active_idx);
  if (norm) {
    CHECK_PTR(q_gain);
    CHECK_PTR(k_gain);
  }
  return launch_qk_norm_rope(q, k_cache, active_idx, n_active, dims->D, dims->Dh, dims->dtype, norm,
                             rope, q_gain, k_gain, dims->grid_h, dims->grid_w, as_stream(stream));
}

hsa_status hsa_time_embed(const hsa_model* model, float sigma, float* e, float* e0, void* stream) {
  if (!model) return HSA_ERR_ARG;
  RETURN_IF(check_dims(&model->dims));
  if (!has(model->dims, HSA_FEAT_ADALN)) return HSA_ERR_ARG;
  if (!isfinite(sigma)) return HSA_ERR_ARG;
  RETURN_IF(check_time_weights(model));
  CHECK_PTR(e);
  CHECK_PTR(e0);
  return launch_time_embed(sigma, model->t_w1, model->t_b1, model->t_w2, model->t_b2, model->t_w3,
                           model->t_b3, model->dims.D, e, e0, as_stream(stream));
}

hsa_status hsa_guidance(const float* v_cond, float* v, int32_t rows, int32_t C, float g,
                        void* stream) {
  if (rows < 0 || C <= 0 || C % 4 != 0) return HSA_ERR_SHAPE;
  if (!isfinite(g)) return HSA_ERR_ARG;
  if (rows == 0) return HSA_OK;
  CHECK_PTR(v_cond);
  CHECK_PTR(v);
  return launch_guidance(v_cond, v, (int64_t)rows * C, g, as_stream(stream));
}

hsa_status hsa_block_forward(const hsa_model* model, int32_t layer, float* h,
                             const int32_t* active_idx, int32_t n_active, const float* e0,
                             int32_t branch, void* ws, size_t ws_bytes, void* stream) {
  RETURN_IF(check_model(model));
  if (layer < 0 || layer >= model->dims.L) return HSA_ERR_ARG;
  if (n_active < 0 || n_active > model->dims.N) return HSA_ERR_SHAPE;
  if (branch != 0 && !(branch == 1 && has(model->dims, HSA_FEAT_CFG))) return HSA_ERR_ARG;
  if (n_active == 0) return HSA_OK;
  CHECK_PTR(h);
  CHECK_PTR(active_idx);
  CHECK_PTR(ws);
  if (has(model->dims, HSA_FEAT_ADALN)) CHECK_PTR(e0);
  const Layout L = layout_of(&model->dims);
  if (ws_bytes < L.total) return HSA_ERR_WORKSPACE;
  return block_forward_impl(model, layer, h, active_idx, n_active, e0, branch, (char*)ws, L,
                            as_stream(stream));
}

hsa_status hsa_step(const hsa_model* model, const hsa_schedule* sched, hsa_state* st,
                    int32_t iter, float sigma_i, float sigma_next, int32_t regroup,
                    const float* v_field, void* stream) {
  RETURN_IF(check_model(model));
  const hsa_dims& d = model->dims;
  RETURN_IF(check_schedule(sched, d.N));
  if (!st) return HSA_ERR_ARG;
  if (iter < 0 || iter >= sched->T) return HSA_ERR_ARG;
  if (regroup != 0 && regroup != 1) return HSA_ERR_ARG;
  CHECK_PTR(st->x);
  CHECK_PTR(st->v_hat);
  CHECK_PTR(st->score);
  CHECK_PTR(st->active_idx);
  CHECK_PTR(st->pos);
  CHECK_PTR(st->workspace);
  if (!st->group) return HSA_ERR_ARG;
  if (v_field && !aligned16(v_field)) return HSA_ERR_ALIGN;
  const Layout L = layout_of(&d);
  if (st->workspace_bytes < L.total) return HSA_ERR_WORKSPACE;

  hipStream_t s = as_stream(stream);
  char* ws = (char*)st->workspace;
  float* h = (float*)(ws + L.h);
  float* v_new = (float*)(ws + L.v_new);
  int32_t* n_dev = (int32_t*)(ws + L.n_active);

  // 1. regroup by the L1 relative change (before A_i is formed)
  if (regroup) RETURN_IF(launch_select(st->score, 1, d.N, sched->count, sched->K, st->group, s));
  // 2. active set; its size is known on the host in closed form
  const int32_t nA = n_active_of(sched, iter);
  RETURN_IF(launch_active_set(st->group, d.N, active_group_mask(sched, iter), nA, st->active_idx,
                              st->pos, n_dev, s));
  // 3. model on the active rows: timestep embedding of sigma_i (adaLN), then
  //    embed -> blocks -> unembed per guidance branch, then the combine
  if (nA > 0) {
    const bool adaln = has(d, HSA_FEAT_ADALN), cfg = has(d, HSA_FEAT_CFG);
    float* e = adaln ? (float*)(ws + L.temb) : nullptr;
    float* e0 = adaln ? e + d.D : nullptr;
    if (adaln)
      RETURN_IF(launch_time_embed(sigma_i, model->t_w1, model->t_b1, model->t_w2, model->t_b2,
                                  model->t_w3, model->t_b3, d.D, e, e0, s));
    const ModVec head_shift = adaln ? ModVec{model->head_mod, e} : ModVec{nullptr, nullptr};
    const ModVec head_scale =
        adaln ? ModVec{model->head_mod + d.D, e} : ModVec{nullptr, nullptr};
    float* v_cond = cfg ? (float*)(ws + L.v_cond) : nullptr;
    for (int branch = 0; branch < (cfg ? 2 : 1); ++branch) {
      RETURN_IF(launch_embed(st->x, st->active_idx, model->w_in, h, nA, d.C, d.D, d.dtype, s));
      for (int l = 0; l < d.L; ++l)
        RETURN_IF(block_forward_impl(model, l, h, st->active_idx, nA, e0, branch, ws, L, s));
      RETURN_IF(launch_unembed(h, model->w_out, (cfg && branch == 0) ? v_cond : v_new, nA, d.D,
                               d.C, d.dtype, head_shift, head_scale, s));
    }
    if (cfg) RETURN_IF(launch_guidance(v_cond, v_new, (int64_t)nA * d.C, model->cfg_scale, s));
    // 4. optional synthetic velocity in place of the model's
    if (v_field) RETURN_IF(launch_gather_rows(v_field, st->active_idx, v_new, nA, d.C, s));
  }
  // 5. cached Euler over all N tokens, score for active tokens from the second iteration on
  const float dsigma = sigma_next - sigma_i;
  return launch_euler(st->x, st->v_hat, st->score, v_new, st->pos, d.N, d.C, dsigma, 1e-6f,
                      iter >= 1 ? 1 : 0, s);
}

}  // extern "C"
