"""Seeded synthetic inputs for Heterogeneous Step Allocation (HSA) workloads.

This module is the only code that both the CPU oracle and the HIP path use.
It draws random numbers and shapes them into workloads; it contains none of
the method's arithmetic (no activity rule, no attention, no Euler step, no
selection).  Every generator is keyed by (config id, stream id) so that both
sides see byte-identical inputs.

Workload shapes follow the Wan-shaped DiT token grids of the HSA evaluation
("Not All Tokens Need 40 Steps", technical summary, section 4): a latent video
of t x h x w tokens, C latent channels, a stack of transformer blocks.
Weights are drawn N(0, 1/fan_in); latents, caches and hidden states N(0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# Random streams (one PCG64 stream per purpose, seed = 1000 * cfg + stream).
STREAM_WEIGHTS = 1
STREAM_X0 = 2
STREAM_GROUP0 = 3
STREAM_TEXT = 4
STREAM_CACHE = 5
STREAM_HIDDEN = 6
STREAM_ACTIVE = 7
STREAM_FIELD = 8
STREAM_STATE = 9
STREAM_FEATURES = 10

# Optional Wan-style block features a Config may switch on (names, not flags:
# each side maps them to its own representation).
FEATURES = ("qk_norm", "rope3d", "adaln", "cfg")


def rng(cfg: int, stream: int, sub: int = 0) -> np.random.Generator:
    """Counter-keyed generator: PCG64 seeded by (1000*cfg + stream, sub)."""
    return np.random.Generator(np.random.PCG64([1000 * cfg + stream, sub]))


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Used once on generated inputs so that the bf16 workloads hand both sides
    the same representable values.  NaN/inf do not occur in generated data.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: model shape, schedule and synthetic-input recipe."""
    cfg: int
    name: str
    grid: Tuple[int, int, int]          # (frames, h, w) token grid
    C: int                              # latent channels
    D: int                              # model width
    H: int                              # heads
    Dh: int                             # head dim
    F: int                              # MLP hidden width
    L: int                              # blocks
    dtype: str                          # "f32" or "bf16"
    T: int                              # global Euler iterations
    budgets: Tuple[int, ...]            # s_k, budgets[0] == T
    shares: Tuple[float, ...]           # token shares per group
    regroup: Tuple[int, ...]            # iterations that start with a regroup
    n_text: int = 0                     # text tokens for cross-attention (0: none)
    text_dim: int = 0                   # text embedding width
    m: int = 0                          # phase window (first/last m iterations full)
    features: Tuple[str, ...] = ()      # subset of FEATURES
    cfg_scale: float = 5.0              # guidance scale when "cfg" is on

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def K(self) -> int:
        return len(self.budgets)

    def counts(self) -> List[int]:
        """Exact group sizes: n_k = round_half_even(share_k * N) for k >= 2, n_1 the rest."""
        N = self.N
        rest = [int(np.round(s * N)) for s in self.shares[1:]]
        return [N - sum(rest)] + rest

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[int, Config] = {
    # Tiny DiT-lite, fp32.
    1: Config(1, "dit-lite-fp32", (4, 8, 8), C=16, D=128, H=2, Dh=64, F=512, L=1,
              dtype="f32", T=8, budgets=(8, 4), shares=(0.5, 0.5),
              regroup=(3, 4, 5, 6, 7)),
    # Single Wan-1.3B-shaped block, bf16 (stage benchmark and block parity).
    2: Config(2, "wan1.3b-block-bf16", (21, 30, 52), C=16, D=1536, H=12, Dh=128,
              F=8960, L=1, dtype="bf16", T=40, budgets=(40, 20, 10),
              shares=(0.25, 0.25, 0.5), regroup=(10, 20, 30)),
    # Wan-1.3B-shaped 30-block stack, bf16.
    3: Config(3, "wan1.3b-30blk-bf16", (21, 30, 52), C=16, D=1536, H=12, Dh=128,
              F=8960, L=30, dtype="bf16", T=40, budgets=(40, 20, 10),
              shares=(0.25, 0.25, 0.5), regroup=(10, 20, 30)),
    # Wan-14B-shaped 40-block stack with cross-attention, bf16.
    4: Config(4, "wan14b-40blk-xattn-bf16", (21, 45, 80), C=16, D=5120, H=40,
              Dh=128, F=13824, L=40, dtype="bf16", T=40, budgets=(40, 20, 10),
              shares=(0.25, 0.25, 0.5), regroup=(10, 20, 30), n_text=512,
              text_dim=4096),
    # Aggressive regime on the single-block model, synthetic velocity field.
    5: Config(5, "wan1.3b-block-churn-bf16", (21, 30, 52), C=16, D=1536, H=12,
              Dh=128, F=8960, L=1, dtype="bf16", T=40, budgets=(40, 10, 5),
              shares=(0.125, 0.375, 0.5), regroup=(10, 20, 30)),
}


def sigma_schedule(T: int) -> np.ndarray:
    """Linear sigma from 1 to 0 over T iterations, computed in fp64, stored fp32."""
    return (1.0 - np.arange(T + 1, dtype=np.float64) / T).astype(np.float32)


# ----------------------------------------------------------------------------
# Weights.  Layout: every linear map is stored out-major, [out][in], so that
# y = a @ W.T.  Variance is 1/fan_in.
# ----------------------------------------------------------------------------

def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def block_weights(c: Config, layer: int) -> Dict[str, np.ndarray]:
    """Weights of block `layer`: w_qkv [3D][D], w_o [D][D], w_1 [F][D], w_2 [D][F],
    and for cross-attention w_qx [D][D], w_kx [D][D], w_vx [D][D], w_ox [D][D]."""
    g = rng(c.cfg, STREAM_WEIGHTS, 1 + layer)
    D, F = c.D, c.F
    w = {
        "w_qkv": _normal(g, (3 * D, D), D ** -0.5),
        "w_o": _normal(g, (D, D), D ** -0.5),
        "w_1": _normal(g, (F, D), D ** -0.5),
        "w_2": _normal(g, (D, F), F ** -0.5),
    }
    if c.n_text:
        for k in ("w_qx", "w_kx", "w_vx", "w_ox"):
            w[k] = _normal(g, (D, D), D ** -0.5)
    if c.dtype == "bf16":
        w = {k: to_bf16_values(v) for k, v in w.items()}
    return w


def io_weights(c: Config) -> Dict[str, np.ndarray]:
    """Embed w_in [D][C] (latent -> width) and unembed w_out [C][D]."""
    g = rng(c.cfg, STREAM_WEIGHTS, 0)
    w = {"w_in": _normal(g, (c.D, c.C), c.C ** -0.5),
         "w_out": _normal(g, (c.C, c.D), c.D ** -0.5)}
    if c.dtype == "bf16":
        w = {k: to_bf16_values(v) for k, v in w.items()}
    return w


def text_inputs(c: Config) -> Dict[str, np.ndarray]:
    """Synthetic text tokens [n_text][text_dim] ~ N(0,1) and projection w_t [D][text_dim]."""
    g = rng(c.cfg, STREAM_TEXT)
    t = g.standard_normal((c.n_text, c.text_dim), dtype=np.float32)
    w_t = _normal(g, (c.D, c.text_dim), c.text_dim ** -0.5)
    if c.dtype == "bf16":
        t, w_t = to_bf16_values(t), to_bf16_values(w_t)
    return {"text": t, "w_t": w_t}


def text_inputs_uncond(c: Config) -> np.ndarray:
    """Second set of text tokens [n_text][text_dim] ~ N(0,1): the condition of the
    unconditional branch under classifier-free guidance (a stand-in for the
    encoded empty or negative prompt).  Projected by the same w_t."""
    t = rng(c.cfg, STREAM_TEXT, 1).standard_normal((c.n_text, c.text_dim), dtype=np.float32)
    return to_bf16_values(t) if c.dtype == "bf16" else t


# ----------------------------------------------------------------------------
# Optional block features.  Gains, modulation tables and the timestep MLP are
# float32 in both dtypes (they are small vectors, read once per row).
# ----------------------------------------------------------------------------

def feature_weights(c: Config, layer: int) -> Dict[str, np.ndarray]:
    """Per-block feature parameters:
      q_gain, k_gain [D]: RMSNorm gains of q and k, 1 + N(0, 0.1^2);
      mod [6][D]: learned modulation table (shift, scale, gate of the attention
        branch, then of the MLP branch), N(0, 0.1^2) with the gate rows
        centred on 1 so that both residual branches stay alive."""
    g = rng(c.cfg, STREAM_FEATURES, 1 + layer)
    D = c.D
    q_gain = 1.0 + _normal(g, (D,), 0.1)
    k_gain = 1.0 + _normal(g, (D,), 0.1)
    mod = _normal(g, (6, D), 0.1)
    mod[2] += 1.0
    mod[5] += 1.0
    return {"q_gain": q_gain.astype(np.float32), "k_gain": k_gain.astype(np.float32),
            "mod": mod.astype(np.float32)}


def time_weights(c: Config, t_freq: int = 256) -> Dict[str, np.ndarray]:
    """Timestep MLP and output-head modulation, out-major like every linear map:
      t_w1 [D][t_freq], t_b1 [D]; t_w2 [D][D], t_b2 [D]; t_w3 [6D][D], t_b3 [6D];
      head_mod [2][D] (shift, scale of the final LayerNorm).
    Scales keep the projected modulation around 0.1 in magnitude."""
    g = rng(c.cfg, STREAM_FEATURES, 0)
    D = c.D
    return {
        "t_w1": _normal(g, (D, t_freq), t_freq ** -0.5),
        "t_b1": _normal(g, (D,), 0.01),
        "t_w2": _normal(g, (D, D), D ** -0.5),
        "t_b2": _normal(g, (D,), 0.01),
        "t_w3": _normal(g, (6 * D, D), 0.3 * D ** -0.5),
        "t_b3": _normal(g, (6 * D,), 0.01),
        "head_mod": _normal(g, (2, D), 0.1),
    }


# ----------------------------------------------------------------------------
# Sampler state.
# ----------------------------------------------------------------------------

def x0(c: Config) -> np.ndarray:
    return rng(c.cfg, STREAM_X0).standard_normal((c.N, c.C), dtype=np.float32)


def group0(c: Config) -> np.ndarray:
    """Initial groups: a seeded random permutation cut by the exact counts."""
    counts = c.counts()
    perm = rng(c.cfg, STREAM_GROUP0).permutation(c.N)
    g = np.empty(c.N, dtype=np.uint8)
    start = 0
    for k, n in enumerate(counts):
        g[perm[start:start + n]] = k
        start += n
    return g


def mid_run_state(c: Config, sub: int = 0) -> Dict[str, np.ndarray]:
    """A state as it looks in the middle of a run: latents, cached velocities,
    finite scores, groups with the exact counts, and per-layer K/V caches.

    Used to start one-iteration parity runs from the same synthetic point on
    both sides.  Caches hold bf16-representable values in bf16 configs.
    """
    g = rng(c.cfg, STREAM_STATE, sub)
    N, C, D = c.N, c.C, c.D
    st = {
        "x": g.standard_normal((N, C), dtype=np.float32),
        "v_hat": g.standard_normal((N, C), dtype=np.float32),
        "score": np.abs(g.standard_normal(N, dtype=np.float32)),
        "group": group_from_perm(c, g.permutation(N)),
    }
    k = g.standard_normal((c.L, N, D), dtype=np.float32)
    v = g.standard_normal((c.L, N, D), dtype=np.float32)
    if c.dtype == "bf16":
        k, v = to_bf16_values(k), to_bf16_values(v)
    st["k_cache"], st["v_cache"] = k, v
    return st


def group_from_perm(c: Config, perm: np.ndarray) -> np.ndarray:
    g = np.empty(c.N, dtype=np.uint8)
    start = 0
    for k, n in enumerate(c.counts()):
        g[perm[start:start + n]] = k
        start += n
    return g


# ----------------------------------------------------------------------------
# Active-set patterns for the single-block sweep.
# ----------------------------------------------------------------------------

def n_active_for_fraction(N: int, f: float) -> int:
    return int(np.round(f * N))


def active_random(c: Config, n_active: int, sub: int = 0) -> np.ndarray:
    """Uniform draw without replacement, sorted ascending."""
    idx = rng(c.cfg, STREAM_ACTIVE, sub).choice(c.N, size=n_active, replace=False)
    return np.sort(idx).astype(np.int32)


def active_blob(c: Config, n_active: int, sub: int = 0) -> np.ndarray:
    """Contiguous spatial blobs: per frame the (h, w) tokens nearest a centre
    that drifts one token along w per frame; total exactly n_active, ties by index."""
    t_, h_, w_ = c.grid
    g = rng(c.cfg, STREAM_ACTIVE, 100 + sub)
    h0, w0 = g.integers(0, h_), g.integers(0, w_)
    n = np.arange(c.N)
    t = n // (h_ * w_)
    hh = (n // w_) % h_
    ww = n % w_
    dh = hh - h0
    dw = (ww - (w0 + t)) % w_
    dw = np.minimum(dw, w_ - dw)
    d2 = dh * dh + dw * dw
    order = np.lexsort((n, d2, t))          # per frame, nearest first
    per = np.full(t_, n_active // t_)
    per[: n_active % t_] += 1
    out = []
    start = 0
    for f in range(t_):
        cnt = h_ * w_
        sel = order[start:start + cnt][: per[f]]
        out.append(sel)
        start += cnt
    return np.sort(np.concatenate(out)).astype(np.int32)


def hidden_states(c: Config, rows: int, sub: int = 0) -> np.ndarray:
    h = rng(c.cfg, STREAM_HIDDEN, sub).standard_normal((rows, c.D), dtype=np.float32)
    return h


def kv_cache(c: Config, sub: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    g = rng(c.cfg, STREAM_CACHE, sub)
    k = g.standard_normal((c.N, c.D), dtype=np.float32)
    v = g.standard_normal((c.N, c.D), dtype=np.float32)
    if c.dtype == "bf16":
        k, v = to_bf16_values(k), to_bf16_values(v)
    return k, v


# ----------------------------------------------------------------------------
# Synthetic velocity field for the churn regime.
# ----------------------------------------------------------------------------

class ChurnField:
    """Slow background b*(1 + 0.002 i) plus a moving foreground blob of fresh
    N(0,1) draws covering ~15% of tokens (per frame the 234 (h, w) nearest a
    centre that moves one w-token per iteration, wrapping)."""

    def __init__(self, c: Config, blob_per_frame: int = 234):
        self.c = c
        self.b = rng(c.cfg, STREAM_FIELD, 0).standard_normal((c.N, c.C), dtype=np.float32)
        self.blob_per_frame = blob_per_frame

    def blob(self, i: int) -> np.ndarray:
        c = self.c
        t_, h_, w_ = c.grid
        n = np.arange(c.N)
        t = n // (h_ * w_)
        hh = (n // w_) % h_
        ww = n % w_
        dh = hh - h_ // 2
        dw = (ww - (w_ // 4 + i)) % w_
        dw = np.minimum(dw, w_ - dw)
        d2 = dh * dh + dw * dw
        order = np.lexsort((n, d2, t))
        sel = []
        for f in range(t_):
            sel.append(order[f * h_ * w_: f * h_ * w_ + self.blob_per_frame])
        return np.sort(np.concatenate(sel))

    def __call__(self, i: int) -> np.ndarray:
        v = (self.b * np.float32(1.0 + 0.002 * i)).astype(np.float32)
        idx = self.blob(i)
        v[idx] = rng(self.c.cfg, STREAM_FIELD, 1 + i).standard_normal(
            (idx.size, self.c.C), dtype=np.float32)
        return v


def small(c: Config, **kw) -> Config:
    """A reduced copy of a config (same structure, smaller shapes) for CPU-speed parity."""
    return c.with_(**kw)
