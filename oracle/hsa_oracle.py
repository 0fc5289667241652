"""CPU oracle for Heterogeneous Step Allocation (HSA): one global denoising iteration.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  The product path (the HIP
library and its Python binding) never does.

Plain, slow and meant to be read against the source pages: "Not All Tokens Need
40 Steps: Heterogeneous Step Allocation in Diffusion Transformers for Efficient
Video Generation" (gist.science technical summary; section numbers below refer
to it).  All arithmetic is float64.  Values are rounded only at the points where
the method's data are stored (latents, caches, activations handed from one
operation to the next): float32 in float32 workloads, bfloat16 for the
activations and caches of bfloat16 workloads (see `Store`).

Readings where the pages leave a step open:
  * iteration index i is 0-based, i in [0, T): every group is active at i = 0;
  * sigma_i = 1 - i/T;
  * block = pre-LayerNorm (no affine, eps 1e-6) multi-head self-attention
    (scale 1/sqrt(Dh), no mask, no biases), optional pre-LN cross-attention,
    pre-LN GELU(tanh) MLP, residual adds; embed C->D, unembed LN then D->C;
  * L1 relative change r_n = sum_c |v_new - v_hat| / (sum_c |v_hat| + eps),
    eps = 1e-6, updated for active tokens at i >= 1, +inf before;
  * regrouping ranks tokens by (score descending, index ascending), NaN as
    +inf and -0 as +0; the first n_1 go to G_1, the next n_2 to G_2, ...

Optional Wan-style block features (off by default).  The pages evaluate HSA on
Wan-family DiTs (section 4) but define none of the model's layers, so these
follow the published general definitions they name, and each reading below is
this module's own:
  * qk-RMSNorm: q and k rows, after projection, scaled by 1/sqrt(mean(x^2) +
    1e-6) over the whole model width D, times a learned gain [D];
  * 3D rotary embedding (RoFormer's rotation of coordinate pairs (2j, 2j+1)
    by angle pos * theta^(-j/p), theta = 10000), per head: the Dh/2 pairs
    split into a frame section of P - 2*floor(P/3) pairs, then height and
    width sections of floor(P/3) pairs each (P = Dh/2), each section
    rotated by the token's frame, row or column index in the latent grid,
    token n = (f * grid_h + y) * grid_w + x; applied after the RMSNorm, so
    the cache holds rotated keys;
  * adaLN timestep modulation: t = 1000 sigma_i (sigma_i as float32);
    sinusoid [cos(t w_k), sin(t w_k)], w_k = 10000^(-k/128), k < 128;
    e = W2 silu(W1 sinusoid + b1) + b2; e0 = W3 silu(e) + b3 -> [6][D];
    block table mod_l + e0 = (shift, scale, gate) for the attention branch,
    then for the MLP branch: LN(h)(1 + scale) + shift feeds the branch and
    gate multiplies its output before the residual add; cross-attention is
    neither modulated nor gated; the final LayerNorm takes (shift, scale) =
    head_mod + e;
  * classifier-free guidance, batch 2: the model runs once with the text
    condition and once with the unconditional text set, each branch with
    its own K/V caches (both on the same active rows), and the velocity is
    v_u + g (v_c - v_u); needs cross-attention.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

LN_EPS = 1e-6
SCORE_EPS = 1e-6
RMS_EPS = 1e-6
ROPE_THETA = 10000.0
T_FREQ = 256          # width of the timestep sinusoid
T_SCALE = 1000.0      # timestep value fed to the sinusoid: t = T_SCALE * sigma


# ----------------------------------------------------------------------------
# Storage rounding.
# ----------------------------------------------------------------------------

def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each element, returned as float64.

    Written with frexp/ldexp: a = f * 2^e with 0.5 <= |f| < 1; bfloat16 keeps
    8 significant bits, so the spacing of representable values near a is
    2^(e-8), but never below the subnormal spacing 2^-133 (bfloat16 has
    float32's exponent range and 7 stored fraction bits).  a is rounded to a
    multiple of that spacing with numpy's round-half-even.  Finite inputs
    only (the method produces no inf/NaN in activations).
    """
    a = np.asarray(a, dtype=np.float64)
    a32 = a.astype(np.float32).astype(np.float64)   # storage goes through fp32 first
    _, e = np.frexp(a32)
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.round(a32 / quantum) * quantum


def round_to_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


@dataclasses.dataclass
class Store:
    """Where values are rounded: `act` for GEMM operands, q/k/v/o, MLP hidden
    and the K/V caches; `res` for the residual stream, latents and velocities."""
    bf16: bool

    def act(self, a):
        return round_to_bf16(a) if self.bf16 else round_to_f32(a)

    def res(self, a):
        return round_to_f32(a)


# ----------------------------------------------------------------------------
# Token partitioning and scheduling (section 2.1) and phase window (2.4).
# ----------------------------------------------------------------------------

def active_mask(group: np.ndarray, budgets: Sequence[int], T: int, i: int,
                m: int = 0) -> np.ndarray:
    """Token n is active at iteration i iff i mod (T / s_{g(n)}) == 0.

    G_1 has s_1 = T (period 1) and is active every iteration.  With a phase
    window m > 0 every token is active in the first and last m iterations.
    """
    budgets = np.asarray(budgets, dtype=np.int64)
    assert budgets[0] == T and np.all(T % budgets == 0)
    if i < m or i >= T - m:
        return np.ones(group.shape[0], dtype=bool)
    period = T // budgets[group.astype(np.int64)]
    return (i % period) == 0


def active_set(group, budgets, T, i, m=0):
    """Ascending list A_i of active token indices and its inverse map
    pos[n] = j if A_i[j] == n, else -1 (section 2.2, item 1)."""
    mask = active_mask(group, budgets, T, i, m)
    idx = np.flatnonzero(mask).astype(np.int32)
    pos = np.full(group.shape[0], -1, dtype=np.int32)
    pos[idx] = np.arange(idx.size, dtype=np.int32)
    return idx, pos


def n_active_closed_form(counts, budgets, T, i, m=0) -> int:
    """|A_i| = sum_k n_k [i mod (T/s_k) == 0]; every token in the phase window."""
    if i < m or i >= T - m:
        return int(sum(counts))
    return int(sum(n for n, s in zip(counts, budgets) if i % (T // s) == 0))


# ----------------------------------------------------------------------------
# Dynamic token selection (section 2.1): rank by L1 relative change.
# ----------------------------------------------------------------------------

def select_groups(score: np.ndarray, counts: Sequence[int]) -> np.ndarray:
    """Group of each token: tokens ranked by (score desc, index asc); ranks
    [0, n_1) -> group 0, [n_1, n_1 + n_2) -> group 1, ...  NaN ranks as +inf,
    -0 as +0."""
    s = np.asarray(score, dtype=np.float32).astype(np.float64)
    s = np.where(np.isnan(s), np.inf, s)
    s = np.where(s == 0.0, 0.0, s)
    N = s.shape[0]
    assert sum(counts) == N
    order = np.lexsort((np.arange(N), -s))
    group = np.empty(N, dtype=np.uint8)
    start = 0
    for k, n in enumerate(counts):
        group[order[start:start + n]] = k
        start += n
    return group


def l1_relative_change(v_new: np.ndarray, v_old: np.ndarray, eps=SCORE_EPS) -> np.ndarray:
    """r = ||v_new - v_old||_1 / (||v_old||_1 + eps) per row, over channels."""
    v_new = np.asarray(v_new, np.float64)
    v_old = np.asarray(v_old, np.float64)
    num = np.abs(v_new - v_old).sum(axis=-1)
    den = np.abs(v_old).sum(axis=-1) + eps
    return num / den


# ----------------------------------------------------------------------------
# Model pieces.
# ----------------------------------------------------------------------------

def layer_norm(y: np.ndarray, eps=LN_EPS) -> np.ndarray:
    """(y - mean) / sqrt(var + eps) over the last axis, population variance, no affine."""
    y = np.asarray(y, np.float64)
    mu = y.mean(axis=-1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)
    return (y - mu) / np.sqrt(var + eps)


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    u = np.asarray(u, np.float64)
    return 0.5 * u * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (u + 0.044715 * u ** 3)))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, H: int, Dh: int,
              scale: Optional[float] = None) -> np.ndarray:
    """Multi-head softmax attention of M query rows over all Nk key/value rows.

    q: [M][H*Dh], k, v: [Nk][H*Dh] -> [M][H*Dh].  Per head h:
    o = softmax(q_h k_h^T * scale) v_h with the row max subtracted first.
    No mask: every query sees every row (section 2.2, item 3).
    """
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    M, Nk = q.shape[0], k.shape[0]
    out = np.empty((M, H * Dh), dtype=np.float64)
    for h in range(H):
        sl = slice(h * Dh, (h + 1) * Dh)
        s = (q[:, sl] @ k[:, sl].T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, sl] = p @ v[:, sl]
    return out


# ----------------------------------------------------------------------------
# Optional block features (readings in the module header).
# ----------------------------------------------------------------------------

def rms_norm(y: np.ndarray, gain: np.ndarray, eps=RMS_EPS) -> np.ndarray:
    """y / sqrt(mean(y^2) + eps) * gain over the last axis."""
    y = np.asarray(y, np.float64)
    return y / np.sqrt((y * y).mean(axis=-1, keepdims=True) + eps) * np.asarray(gain, np.float64)


def rope_sections(Dh: int) -> Tuple[int, int, int]:
    """Rotation pairs per head given to the frame, row and column axes."""
    P = Dh // 2
    p_hw = P // 3
    return P - 2 * p_hw, p_hw, p_hw


def token_coords(idx: np.ndarray, grid: Tuple[int, int, int]):
    """(frame, row, column) of tokens idx; n = (f * grid_h + y) * grid_w + x."""
    _, gh, gw = grid
    n = np.asarray(idx, np.int64)
    return n // (gh * gw), (n // gw) % gh, n % gw


def rope_angles(idx: np.ndarray, grid: Tuple[int, int, int], Dh: int,
                theta=ROPE_THETA) -> np.ndarray:
    """[len(idx)][Dh/2] rotation angle of each pair of a head: the frame
    section first, then rows, then columns; pair j of a section with p pairs
    turns by theta^(-j/p) per unit of that axis."""
    cols = []
    for pos, p in zip(token_coords(idx, grid), rope_sections(Dh)):
        freq = theta ** (-np.arange(p, dtype=np.float64) / p)
        cols.append(pos[:, None].astype(np.float64) * freq[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(x: np.ndarray, angles: np.ndarray, H: int, Dh: int) -> np.ndarray:
    """Rotate coordinate pair (2j, 2j+1) of every head of row r by angles[r][j]:
    (a, b) -> (a cos - b sin, a sin + b cos)."""
    x = np.asarray(x, np.float64)
    M = x.shape[0]
    xp = x.reshape(M, H, Dh // 2, 2)
    c = np.cos(angles)[:, None, :]
    s = np.sin(angles)[:, None, :]
    a, b = xp[..., 0], xp[..., 1]
    return np.stack((a * c - b * s, a * s + b * c), axis=-1).reshape(M, H * Dh)


def qk_transform(dims: Dims, x: np.ndarray, idx: np.ndarray, gain: Optional[np.ndarray]) -> np.ndarray:
    """What the enabled features do to stored q or k rows of tokens idx after
    the projection: RMSNorm over D with `gain`, then the 3D rotation."""
    y = np.asarray(x, np.float64)
    if dims.qk_norm:
        y = rms_norm(y, gain)
    if dims.rope3d:
        y = apply_rope(y, rope_angles(idx, dims.grid, dims.Dh), dims.H, dims.Dh)
    return y


def silu(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, np.float64)
    return u / (1.0 + np.exp(-u))


def timestep_sinusoid(sigma: float) -> np.ndarray:
    """[cos(t w_k) for k < 128] + [sin(t w_k) for k < 128], w_k = 10000^(-k/128),
    t = 1000 * sigma with sigma taken as the float32 the step receives."""
    t = T_SCALE * float(np.float32(sigma))
    half = T_FREQ // 2
    w = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
    return np.concatenate([np.cos(t * w), np.sin(t * w)])


def time_embedding(model: "Model", sigma: float):
    """(e [D], e0 [6][D]): e = W2 silu(W1 s + b1) + b2, e0 = W3 silu(e) + b3,
    s the timestep sinusoid; every stored vector float32."""
    tm = model.time
    s = round_to_f32(timestep_sinusoid(sigma))
    e1 = round_to_f32(silu(tm["t_w1"] @ s + tm["t_b1"]))
    e = round_to_f32(tm["t_w2"] @ e1 + tm["t_b2"])
    e0 = round_to_f32(tm["t_w3"] @ silu(e) + tm["t_b3"])
    return e, e0.reshape(6, model.dims.D)


def block_modulation(model: "Model", l: int, e0: np.ndarray) -> np.ndarray:
    """[6][D] = mod_l + e0: shift, scale, gate (attention), shift, scale, gate (MLP)."""
    return round_to_f32(model.blocks[l]["mod"] + e0)


def head_modulation(model: "Model", e: np.ndarray) -> np.ndarray:
    """[2][D] = head_mod + e: shift, scale of the final LayerNorm."""
    return round_to_f32(model.time["head_mod"] + np.asarray(e)[None, :])


def modulated_layer_norm(h: np.ndarray, shift: Optional[np.ndarray],
                         scale: Optional[np.ndarray]) -> np.ndarray:
    """LN(h) (1 + scale) + shift; plain LN when no modulation is given."""
    y = layer_norm(h)
    if scale is not None:
        y = y * (1.0 + np.asarray(scale, np.float64))
    if shift is not None:
        y = y + np.asarray(shift, np.float64)
    return y


def guidance(v_cond: np.ndarray, v_uncond: np.ndarray, g: float) -> np.ndarray:
    """Classifier-free guidance: v_u + g (v_c - v_u), stored float32."""
    vc = np.asarray(v_cond, np.float64)
    vu = np.asarray(v_uncond, np.float64)
    return round_to_f32(vu + np.float64(np.float32(g)) * (vc - vu))


@dataclasses.dataclass
class Dims:
    N: int
    C: int
    D: int
    H: int
    Dh: int
    F: int
    L: int
    bf16: bool
    n_text: int = 0
    qk_norm: bool = False
    rope3d: bool = False
    adaln: bool = False
    cfg: bool = False
    grid: Tuple[int, int, int] = (0, 0, 0)    # (frames, rows, columns) of the token grid


@dataclasses.dataclass
class Model:
    """Weights as float64 copies of the stored values, all out-major [out][in]:
    w_in [D][C], w_out [C][D]; per block w_qkv [3D][D], w_o [D][D], w_1 [F][D],
    w_2 [D][F]; cross-attention w_qx, w_ox [D][D] and per-layer text K/V."""
    dims: Dims
    w_in: np.ndarray
    w_out: np.ndarray
    blocks: List[Dict[str, np.ndarray]]
    time: Optional[Dict[str, np.ndarray]] = None   # adaLN: timestep MLP and head_mod
    cfg_scale: float = 1.0                         # guidance scale g

    @property
    def store(self) -> Store:
        return Store(self.dims.bf16)


def make_model(dims: Dims, io: Dict[str, np.ndarray], blocks: List[Dict[str, np.ndarray]],
               text: Optional[Dict[str, np.ndarray]] = None,
               time: Optional[Dict[str, np.ndarray]] = None,
               text_uncond: Optional[np.ndarray] = None, cfg_scale: float = 1.0) -> Model:
    """Blocks carry q_gain, k_gain [D] (qk_norm) and mod [6][D] (adaln) when
    those features are on; `time` holds the timestep MLP and head_mod (adaln);
    `text_uncond` [n_text][text_dim] is the unconditional text set (cfg)."""
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    bl = [{k: f64(v) for k, v in b.items()} for b in blocks]
    m = Model(dims, f64(io["w_in"]), f64(io["w_out"]), bl,
              None if time is None else {k: f64(v) for k, v in time.items()}, float(cfg_scale))
    if dims.qk_norm:
        assert all("q_gain" in b and "k_gain" in b for b in bl)
    if dims.rope3d:
        assert int(np.prod(dims.grid)) == dims.N
    if dims.adaln:
        assert time is not None and all("mod" in b for b in bl)
    if dims.cfg:
        assert dims.n_text > 0 and text_uncond is not None
    if dims.n_text:
        assert text is not None
        st = m.store
        E = st.act(f64(text["text"]) @ f64(text["w_t"]).T)   # text embedding, once per run
        for b in m.blocks:
            b["k_text"] = st.act(E @ b["w_kx"].T)
            b["v_text"] = st.act(E @ b["w_vx"].T)
        if dims.cfg:
            Eu = st.act(f64(text_uncond) @ f64(text["w_t"]).T)
            for b in m.blocks:
                b["k_text_u"] = st.act(Eu @ b["w_kx"].T)
                b["v_text_u"] = st.act(Eu @ b["w_vx"].T)
    return m


def embed(model: Model, x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """h = x[A] W_in^T, the residual stream of the active rows."""
    return model.store.res(np.asarray(x, np.float64)[idx] @ model.w_in.T)


def unembed(model: Model, h: np.ndarray, head_mod: Optional[np.ndarray] = None) -> np.ndarray:
    """v_new = LN(h) W_out^T (float32 velocities); with head_mod [2][D] the
    LayerNorm output is modulated by (shift, scale) first."""
    if head_mod is None:
        return round_to_f32(layer_norm(h) @ model.w_out.T)
    return round_to_f32(modulated_layer_norm(h, head_mod[0], head_mod[1]) @ model.w_out.T)


def block_forward(model: Model, l: int, h: np.ndarray, idx: np.ndarray,
                  k_cache: np.ndarray, v_cache: np.ndarray,
                  rows: Optional[np.ndarray] = None, mod: Optional[np.ndarray] = None,
                  branch: int = 0) -> np.ndarray:
    """One transformer block on the active rows with KV-cache synchronisation
    (section 2.2):
      1. only active rows go through the QKV projection;
      2. their fresh K/V overwrite rows A_i of this layer's cache (in place);
      3. active queries attend over all N cached rows, fresh and stale;
      4. out-projection, cross-attention and MLP run on active rows only.
    `rows` (indices into A_i) restricts steps 3-4 to a sample of the active
    rows; the cache update always covers every active row.  `mod` [6][D] is
    the block's timestep modulation (adaln), `branch` 1 selects the
    unconditional text set (cfg); k_cache/v_cache are that branch's caches.
    Returns the new residual rows ([len(rows)][D], or [|A|][D])."""
    d = model.dims
    st = model.store
    b = model.blocks[l]
    D = d.D
    idx = np.asarray(idx)
    h = np.asarray(h, np.float64)
    m = mod if mod is not None else [None] * 6
    a = st.act(modulated_layer_norm(h, m[0], m[1]))
    kv = a @ b["w_qkv"][D:].T
    k = st.act(kv[:, :D])
    if d.qk_norm or d.rope3d:
        k = st.act(qk_transform(d, k, idx, b.get("k_gain")))
    k_cache[idx] = k
    v_cache[idx] = st.act(kv[:, D:])
    q_tok = idx
    if rows is not None:
        h = h[rows]
        a = a[rows]
        q_tok = idx[rows]
    q = st.act(a @ b["w_qkv"][:D].T)
    if d.qk_norm or d.rope3d:
        q = st.act(qk_transform(d, q, q_tok, b.get("q_gain")))
    o = st.act(attention(q, k_cache, v_cache, d.H, d.Dh))
    y = o @ b["w_o"].T
    h = st.res(h + (y if m[2] is None else y * m[2]))
    if d.n_text:
        kt, vt = (b["k_text"], b["v_text"]) if branch == 0 else (b["k_text_u"], b["v_text_u"])
        ax = st.act(layer_norm(h))
        qx = st.act(ax @ b["w_qx"].T)
        ox = st.act(attention(qx, kt, vt, d.H, d.Dh))
        h = st.res(h + ox @ b["w_ox"].T)
    a2 = st.act(modulated_layer_norm(h, m[3], m[4]))
    u = st.act(gelu_tanh(a2 @ b["w_1"].T))
    y = u @ b["w_2"].T
    h = st.res(h + (y if m[5] is None else y * m[5]))
    return h


# ----------------------------------------------------------------------------
# Cached Euler update (section 2.3) with the L1 score of section 2.1.
# ----------------------------------------------------------------------------

def euler_update(x, v_hat, score, v_new, idx, dsigma, update_score, eps=SCORE_EPS):
    """Returns new (x, v_hat, score).

    For active tokens (rows idx, with fresh velocities v_new in the same order):
    if update_score, score = L1 relative change between v_new and the cached
    v_hat; then v_hat <- v_new.  Every token then advances by
    x <- x + dsigma * v_hat: fresh velocity if active, cached if skipped.
    """
    x = np.asarray(x, np.float64)
    v_hat = np.array(v_hat, np.float64)
    score = np.array(score, np.float64)
    v_new = np.asarray(v_new, np.float64)
    if update_score:
        score[idx] = round_to_f32(l1_relative_change(v_new, v_hat[idx], eps))
    v_hat[idx] = v_new
    x_new = round_to_f32(x + np.float64(dsigma) * v_hat)
    return x_new, round_to_f32(v_hat), round_to_f32(score)


# ----------------------------------------------------------------------------
# One HSA iteration and the sampling loop.
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Schedule:
    T: int
    budgets: List[int]
    counts: List[int]
    m: int = 0
    regroup: Sequence[int] = ()


@dataclasses.dataclass
class State:
    x: np.ndarray            # [N][C] float32 values
    v_hat: np.ndarray        # [N][C]
    score: np.ndarray        # [N]
    group: np.ndarray        # [N] uint8
    k_cache: np.ndarray      # [L][N][D]
    v_cache: np.ndarray      # [L][N][D]
    k_cache_u: Optional[np.ndarray] = None   # [L][N][D], unconditional branch (cfg)
    v_cache_u: Optional[np.ndarray] = None

    def copy(self) -> "State":
        return State(*(None if a is None else np.array(a) for a in
                       (getattr(self, f.name) for f in dataclasses.fields(self))))


def init_state(dims: Dims, x0: np.ndarray, group0: np.ndarray) -> State:
    N, C, D, L = dims.N, dims.C, dims.D, dims.L
    st = State(x=np.asarray(x0, np.float64).copy(),
               v_hat=np.zeros((N, C)), score=np.full(N, np.inf),
               group=np.asarray(group0, np.uint8).copy(),
               k_cache=np.zeros((L, N, D)), v_cache=np.zeros((L, N, D)))
    if dims.cfg:
        st.k_cache_u = np.zeros((L, N, D))
        st.v_cache_u = np.zeros((L, N, D))
    return st


def dsigma_f32(sigma_i, sigma_next) -> np.float32:
    """The Euler increment sigma_{i+1} - sigma_i as a float32 scalar."""
    return np.float32(np.float32(sigma_next) - np.float32(sigma_i))


def model_velocity(model: Model, state: State, x: np.ndarray, idx: np.ndarray,
                   sigma_i: float) -> np.ndarray:
    """Velocity of the active rows idx: embed -> L blocks (caches of `state`
    updated) -> unembed, once per guidance branch, combined under cfg."""
    d = model.dims
    mods, hmod = [None] * d.L, None
    if d.adaln:
        e, e0 = time_embedding(model, sigma_i)
        mods = [block_modulation(model, l, e0) for l in range(d.L)]
        hmod = head_modulation(model, e)
    out = []
    for branch in ((0, 1) if d.cfg else (0,)):
        kc, vc = (state.k_cache, state.v_cache) if branch == 0 else (state.k_cache_u, state.v_cache_u)
        h = embed(model, x, idx)
        for l in range(d.L):
            h = block_forward(model, l, h, idx, kc[l], vc[l], mod=mods[l], branch=branch)
        out.append(unembed(model, h, hmod))
    return guidance(out[0], out[1], model.cfg_scale) if d.cfg else out[0]


def hsa_iteration(model: Model, sched: Schedule, state: State, i: int,
                  sigma_i: float, sigma_next: float, regroup: bool,
                  v_field: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """One global iteration, in place on `state`:
      regroup (at the start of i, before A_i) -> A_i -> embed -> L blocks ->
      unembed (per guidance branch, then combined) -> cached Euler with score
      update.
    `v_field` ([N][C]) replaces the model's velocity for the active tokens in
    the Euler/score path when given (the model still runs).
    Returns the per-iteration intermediates (active list, pos, v_new)."""
    if regroup:
        state.group = select_groups(state.score, sched.counts)
    idx, pos = active_set(state.group, sched.budgets, sched.T, i, sched.m)
    v_new = model_velocity(model, state, state.x, idx, sigma_i)
    if v_field is not None:
        v_new = np.asarray(v_field, np.float64)[idx]
    state.x, state.v_hat, state.score = euler_update(
        state.x, state.v_hat, state.score, v_new, idx, dsigma_f32(sigma_i, sigma_next),
        update_score=(i >= 1))
    return {"active_idx": idx, "pos": pos, "v_new": v_new}


def sample(model: Model, sched: Schedule, state: State, sigma: np.ndarray,
           field=None, iters: Optional[Sequence[int]] = None) -> List[Dict[str, np.ndarray]]:
    """Run iterations (default 0..T-1), regrouping at the start of each
    iteration listed in sched.regroup."""
    trace = []
    for i in (range(sched.T) if iters is None else iters):
        vf = field(i) if field is not None else None
        trace.append(hsa_iteration(model, sched, state, i, sigma[i], sigma[i + 1],
                                   regroup=(i in set(sched.regroup)), v_field=vf))
    return trace


# ----------------------------------------------------------------------------
# Dense reference: the plain DiT forward over all N tokens, no cache, no
# active list.  With every s_k = T the HSA iteration must reduce to this.
# ----------------------------------------------------------------------------

def dense_velocity(model: Model, x: np.ndarray, sigma: float = 1.0) -> np.ndarray:
    """Every token through every block with no cache: q, k, v of all N rows
    computed afresh.  `sigma` feeds the timestep modulation (adaln)."""
    d = model.dims
    st = model.store
    D = d.D
    allt = np.arange(d.N)
    mods, hmod = [None] * d.L, None
    if d.adaln:
        e, e0 = time_embedding(model, sigma)
        mods = [block_modulation(model, l, e0) for l in range(d.L)]
        hmod = head_modulation(model, e)
    out = []
    for branch in ((0, 1) if d.cfg else (0,)):
        h = st.res(np.asarray(x, np.float64) @ model.w_in.T)
        for l, b in enumerate(model.blocks):
            m = mods[l] if mods[l] is not None else [None] * 6
            a = st.act(modulated_layer_norm(h, m[0], m[1]))
            q = st.act(a @ b["w_qkv"][:D].T)
            k = st.act(a @ b["w_qkv"][D:2 * D].T)
            v = st.act(a @ b["w_qkv"][2 * D:].T)
            if d.qk_norm or d.rope3d:
                q = st.act(qk_transform(d, q, allt, b.get("q_gain")))
                k = st.act(qk_transform(d, k, allt, b.get("k_gain")))
            y = st.act(attention(q, k, v, d.H, d.Dh)) @ b["w_o"].T
            h = st.res(h + (y if m[2] is None else y * m[2]))
            if d.n_text:
                kt, vt = (b["k_text"], b["v_text"]) if branch == 0 else (b["k_text_u"], b["v_text_u"])
                ax = st.act(layer_norm(h))
                qx = st.act(ax @ b["w_qx"].T)
                h = st.res(h + st.act(attention(qx, kt, vt, d.H, d.Dh)) @ b["w_ox"].T)
            a2 = st.act(modulated_layer_norm(h, m[3], m[4]))
            y = st.act(gelu_tanh(a2 @ b["w_1"].T)) @ b["w_2"].T
            h = st.res(h + (y if m[5] is None else y * m[5]))
        out.append(unembed(model, h, hmod))
    return guidance(out[0], out[1], model.cfg_scale) if d.cfg else out[0]


def dense_euler_sample(model: Model, x0: np.ndarray, sigma: np.ndarray, T: int) -> np.ndarray:
    """Plain Euler flow-matching loop: x_{i+1} = x_i + (sigma_{i+1} - sigma_i) v(x_i)."""
    x = round_to_f32(x0)
    for i in range(T):
        v = dense_velocity(model, x, sigma[i])
        x = round_to_f32(x + np.float64(dsigma_f32(sigma[i], sigma[i + 1])) * v)
    return x


def field_iteration(sched: Schedule, state: State, i: int, sigma_i: float, sigma_next: float,
                    regroup: bool, v_field: np.ndarray) -> Dict[str, np.ndarray]:
    """One iteration of the sampler state when a velocity field [N][C] replaces
    the model's prediction in the Euler/score path: regroup (section 2.1) ->
    A_i -> cached Euler with v_new = v_field[A_i] (section 2.3).  The model's
    caches are not touched here; x, v_hat, score and group evolve exactly as
    in hsa_iteration with the same v_field."""
    if regroup:
        state.group = select_groups(state.score, sched.counts)
    idx, pos = active_set(state.group, sched.budgets, sched.T, i, sched.m)
    v_new = np.asarray(v_field, np.float64)[idx]
    state.x, state.v_hat, state.score = euler_update(
        state.x, state.v_hat, state.score, v_new, idx, dsigma_f32(sigma_i, sigma_next),
        update_score=(i >= 1))
    return {"active_idx": idx, "pos": pos, "v_new": v_new}
