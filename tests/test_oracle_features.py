"""Pins for the oracle's optional Wan-style block features (qk-RMSNorm, 3D
rotary embedding, adaLN timestep modulation, classifier-free guidance).

The pages evaluate HSA on Wan-family models without defining their layers, so
each feature follows a published general definition (RMSNorm, RoFormer's
rotary embedding, sinusoidal timestep features, adaptive LayerNorm, guidance)
under the readings stated in the oracle's header.  Every check here ties the
oracle to something outside it: a torch library routine (CPU, float64), the
complex-number form of the rotation, numpy's index unravelling, closed forms
under crafted weights, invariants, or a reduction to the plain block that
test_oracle.py pins.  CPU only.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import synth
from oracle import hsa_oracle as O


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float64))


# ---------------------------------------------------------------- RMSNorm

def test_rms_norm_matches_torch():
    rs = np.random.default_rng(0)
    y = rs.standard_normal((7, 96)) * 3.0
    g = 1.0 + 0.1 * rs.standard_normal(96)
    ref = Fnn.rms_norm(t64(y), (96,), weight=t64(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(y, g), ref, rtol=1e-13, atol=1e-13)


def test_rms_norm_of_centred_row_is_layer_norm():
    # For a zero-mean row the mean square is the population variance.
    rs = np.random.default_rng(1)
    y = rs.standard_normal((5, 64))
    yc = y - y.mean(axis=1, keepdims=True)
    np.testing.assert_allclose(O.rms_norm(yc, np.ones(64)),
                               Fnn.layer_norm(t64(y), (64,), eps=1e-6).numpy(), rtol=1e-12, atol=1e-12)


def test_rms_norm_closed_forms():
    # constant row c: c / sqrt(c^2 + eps) * gain
    for c in (0.5, -2.0, 1e-4):
        got = O.rms_norm(np.full((1, 8), c), np.arange(1, 9, dtype=np.float64))
        np.testing.assert_allclose(got[0], c / math.sqrt(c * c + 1e-6) * np.arange(1, 9), rtol=1e-14)
    # scale invariance away from the eps floor
    rs = np.random.default_rng(2)
    y = rs.standard_normal((3, 32))
    np.testing.assert_allclose(O.rms_norm(7.5 * y, np.ones(32)), O.rms_norm(y, np.ones(32)),
                               rtol=1e-6)


# ---------------------------------------------------------------- 3D rotary embedding

def test_rope_sections_hand_values():
    # Dh/2 pairs: rows and columns get floor(P/3) each, frames the rest.
    assert O.rope_sections(128) == (22, 21, 21)
    assert O.rope_sections(64) == (12, 10, 10)
    assert O.rope_sections(16) == (4, 2, 2)


def test_token_coords_match_unravel_index():
    grid = (3, 5, 7)
    idx = np.arange(105)
    f, y, x = O.token_coords(idx, grid)
    uf, uy, ux = np.unravel_index(idx, grid)
    np.testing.assert_array_equal(f, uf)
    np.testing.assert_array_equal(y, uy)
    np.testing.assert_array_equal(x, ux)


def test_rope_angles_structure():
    grid = (4, 6, 8)
    Dh = 128
    pf, ph, pw = O.rope_sections(Dh)
    n = lambda f, y, x: np.array([(f * grid[1] + y) * grid[2] + x])
    # origin: no rotation anywhere
    assert np.all(O.rope_angles(n(0, 0, 0), grid, Dh) == 0)
    # one step along each axis touches only that axis's section; pair 0 of
    # the section turns by exactly one radian per step
    for axis, tok, lo, p in ((0, n(1, 0, 0), 0, pf), (1, n(0, 1, 0), pf, ph), (2, n(0, 0, 1), pf + ph, pw)):
        a = O.rope_angles(tok, grid, Dh)[0]
        mask = np.zeros(Dh // 2, bool)
        mask[lo:lo + p] = True
        assert np.all(a[~mask] == 0), axis
        assert a[lo] == 1.0
        # frequencies fall geometrically; p ratios multiply to 1/theta
        r = a[lo + 1:lo + p] / a[lo:lo + p - 1]
        np.testing.assert_allclose(r, r[0], rtol=1e-12)
        np.testing.assert_allclose(r[0] ** p, 1e-4, rtol=1e-12)
    # angles are linear in the coordinate: 3 steps = 3 x one step
    np.testing.assert_allclose(O.rope_angles(n(3, 5, 7), grid, Dh),
                               3 * O.rope_angles(n(1, 0, 0), grid, Dh) + 5 * O.rope_angles(n(0, 1, 0), grid, Dh)
                               + 7 * O.rope_angles(n(0, 0, 1), grid, Dh), rtol=1e-13)


def test_apply_rope_is_complex_multiplication():
    rs = np.random.default_rng(3)
    H, Dh, M = 3, 16, 9
    x = rs.standard_normal((M, H * Dh))
    ang = rs.uniform(-40, 40, (M, Dh // 2))
    xc = torch.view_as_complex(t64(x).view(M, H, Dh // 2, 2))
    rot = torch.polar(torch.ones(M, 1, Dh // 2, dtype=torch.float64), t64(ang)[:, None, :])
    ref = torch.view_as_real(xc * rot).reshape(M, H * Dh).numpy()
    np.testing.assert_allclose(O.apply_rope(x, ang, H, Dh), ref, rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    # <R(p1) q, R(p2) k> is unchanged when both positions move by the same offset
    rs = np.random.default_rng(4)
    grid, H, Dh = (6, 7, 9), 2, 64
    q = rs.standard_normal((1, H * Dh))
    k = rs.standard_normal((1, H * Dh))
    n = lambda f, y, x: np.array([(f * grid[1] + y) * grid[2] + x])

    def scores(p1, p2):
        rq = O.apply_rope(q, O.rope_angles(n(*p1), grid, Dh), H, Dh).reshape(H, Dh)
        rk = O.apply_rope(k, O.rope_angles(n(*p2), grid, Dh), H, Dh).reshape(H, Dh)
        return (rq * rk).sum(axis=1)

    base = scores((1, 2, 3), (4, 0, 5))
    for off in ((1, 1, 1), (0, 3, 0), (1, 0, 3), (0, 1, 2)):
        p1 = tuple(a + b for a, b in zip((1, 2, 3), off))
        p2 = tuple(a + b for a, b in zip((4, 0, 5), off))
        np.testing.assert_allclose(scores(p1, p2), base, rtol=1e-10, atol=1e-12)
    # and it does change with the relative position
    assert np.max(np.abs(scores((1, 2, 3), (4, 1, 5)) - base)) > 1e-3


def test_rope_preserves_head_norms():
    rs = np.random.default_rng(5)
    H, Dh = 4, 128
    grid = (5, 6, 7)
    idx = rs.integers(0, 210, 11)
    x = rs.standard_normal((11, H * Dh))
    y = O.apply_rope(x, O.rope_angles(idx, grid, Dh), H, Dh)
    np.testing.assert_allclose(np.linalg.norm(y.reshape(11, H, Dh), axis=2),
                               np.linalg.norm(x.reshape(11, H, Dh), axis=2), rtol=1e-12)


# ---------------------------------------------------------------- timestep modulation

def test_timestep_sinusoid_closed_forms():
    z = O.timestep_sinusoid(0.0)
    np.testing.assert_array_equal(z, np.r_[np.ones(128), np.zeros(128)])
    s = O.timestep_sinusoid(0.4375)          # exact in float32: t = 437.5
    np.testing.assert_allclose(s[:128] ** 2 + s[128:] ** 2, 1.0, rtol=1e-14)
    assert s[0] == math.cos(437.5) and s[128] == math.sin(437.5)
    # small t: recover each angle, check the geometric frequencies and t itself
    s = O.timestep_sinusoid(0.002)           # t = 1000 * float32(0.002)
    t = 1000.0 * float(np.float32(0.002))
    ang = np.arctan2(s[128:], s[:128])
    np.testing.assert_allclose(ang[0], t, rtol=1e-14)
    np.testing.assert_allclose(ang[1:] / ang[:-1], 10000.0 ** (-1 / 128), rtol=1e-10)


def _silu_ref(x):
    return x / (1.0 + math.exp(-x))


def _crafted_time(D, beta, alpha, gamma, b3):
    """Timestep MLP whose outputs have hand-derivable values."""
    return {"t_w1": np.zeros((D, 256)), "t_b1": np.full(D, beta),
            "t_w2": alpha * np.eye(D), "t_b2": np.full(D, gamma),
            "t_w3": np.tile(np.eye(D), (6, 1)), "t_b3": np.asarray(b3, np.float64),
            "head_mod": np.zeros((2, D))}


def _tiny_model(time=None, **dims_kw):
    D = 4
    dims = O.Dims(N=4, C=4, D=D, H=1, Dh=4, F=8, L=1, bf16=False, **dims_kw)
    m = O.Model(dims, np.zeros((D, 4)), np.zeros((4, D)), [{}], time=time)
    return m


def test_time_mlp_closed_form():
    D = 4
    b3 = np.arange(6 * D) * 0.01
    m = _tiny_model(_crafted_time(D, beta=math.log(3.0), alpha=2.0, gamma=-0.25, b3=b3), adaln=True)
    e, e0 = O.time_embedding(m, 0.3)
    e_ref = 2.0 * _silu_ref(math.log(3.0)) - 0.25          # silu(ln 3) = 0.75 ln 3
    np.testing.assert_allclose(e, np.float32(e_ref), rtol=1e-7)
    np.testing.assert_allclose(e0.ravel(), np.float32(_silu_ref(float(np.float32(e_ref))) + b3), rtol=1e-6)
    # the sinusoid reaches W1: rows picking cos(t) and sin(t)
    tm = _crafted_time(D, beta=0.0, alpha=1.0, gamma=0.0, b3=np.zeros(6 * D))
    tm["t_w1"][0, 0] = 1.0
    tm["t_w1"][1, 128] = 1.0
    m = _tiny_model(tm, adaln=True)
    e, _ = O.time_embedding(m, 0.3)
    t = 1000.0 * float(np.float32(0.3))
    np.testing.assert_allclose(e[:2], [_silu_ref(math.cos(t)), _silu_ref(math.sin(t))], rtol=1e-6)
    assert e[2] == 0.0 and e[3] == 0.0


def test_modulated_layer_norm_matches_torch():
    rs = np.random.default_rng(6)
    h = rs.standard_normal((5, 32)) * 2 + 1
    sh, sc = rs.standard_normal(32) * 0.1, rs.standard_normal(32) * 0.1
    ref = (Fnn.layer_norm(t64(h), (32,), eps=1e-6) * (1 + t64(sc)) + t64(sh)).numpy()
    np.testing.assert_allclose(O.modulated_layer_norm(h, sh, sc), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.modulated_layer_norm(h, np.zeros(32), np.zeros(32)),
                               Fnn.layer_norm(t64(h), (32,), eps=1e-6).numpy(), rtol=1e-12, atol=1e-12)
    # scale -1 leaves exactly the shift
    np.testing.assert_array_equal(O.modulated_layer_norm(h, sh, -np.ones(32)), np.tile(sh, (5, 1)))


def test_guidance_closed_forms():
    rs = np.random.default_rng(7)
    vc, vu = rs.standard_normal((3, 4)).astype(np.float32), rs.standard_normal((3, 4)).astype(np.float32)
    np.testing.assert_array_equal(O.guidance(vc, vu, 1.0), vc)
    np.testing.assert_array_equal(O.guidance(vc, vu, 0.0), vu)
    np.testing.assert_allclose(O.guidance(vc, vu, 2.0), 2 * vc.astype(np.float64) - vu, rtol=1e-6)


# ---------------------------------------------------------------- whole-model pins

FEATS = ("qk_norm", "rope3d", "adaln")


def _cfg(features=FEATS, **kw):
    base = dict(grid=(2, 4, 4), C=4, D=48, H=3, Dh=16, F=64, L=2, dtype="f32", T=8,
                budgets=(8, 4), shares=(0.5, 0.5), regroup=(3,), features=tuple(features))
    base.update(kw)
    return synth.CONFIGS[1].with_(**base)


def _model(c, drop=()):
    f = set(c.features) - set(drop)
    dims = O.Dims(N=c.N, C=c.C, D=c.D, H=c.H, Dh=c.Dh, F=c.F, L=c.L, bf16=(c.dtype == "bf16"),
                  n_text=c.n_text, qk_norm="qk_norm" in f, rope3d="rope3d" in f,
                  adaln="adaln" in f, cfg="cfg" in f, grid=c.grid)
    blocks = []
    for l in range(c.L):
        b = synth.block_weights(c, l)
        b.update(synth.feature_weights(c, l))
        blocks.append(b)
    text = synth.text_inputs(c) if c.n_text else None
    tu = synth.text_inputs_uncond(c) if c.n_text else None
    return O.make_model(dims, synth.io_weights(c), blocks, text, synth.time_weights(c), tu, c.cfg_scale)


def _torch_dense_velocity(c, x, sigma):
    """The featured DiT written with torch CPU float64 library ops: rms_norm,
    complex rotation, silu, layer_norm, scaled_dot_product_attention."""
    D, H, Dh = c.D, c.H, c.Dh
    f = set(c.features)
    io = synth.io_weights(c)
    tw = {k: t64(v) for k, v in synth.time_weights(c).items()}

    def freqs(p):   # 10000^(-j/p), j < p, in log space
        return torch.logspace(0, -4.0 * (p - 1) / p, p, base=10.0, dtype=torch.float64)

    gf, gh, gw = c.grid
    n = torch.arange(c.N)
    coords = (n // (gh * gw), (n // gw) % gh, n % gw)
    P = Dh // 2
    sec = (P - 2 * (P // 3), P // 3, P // 3)
    ang = torch.cat([torch.outer(pos.to(torch.float64), freqs(p)) for pos, p in zip(coords, sec)], dim=1)
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

    def qk(x, g):
        if "qk_norm" in f:
            x = Fnn.rms_norm(x, (D,), weight=g, eps=1e-6)
        if "rope3d" in f:
            x = torch.view_as_real(torch.view_as_complex(x.reshape(-1, H, P, 2)) * rot).reshape(-1, D)
        return x

    def mha(q, k, v):
        M, Nk = q.shape[0], k.shape[0]
        o = Fnn.scaled_dot_product_attention(q.view(M, H, Dh).transpose(0, 1),
                                             k.view(Nk, H, Dh).transpose(0, 1),
                                             v.view(Nk, H, Dh).transpose(0, 1))
        return o.transpose(0, 1).reshape(M, D)

    ln = lambda h: Fnn.layer_norm(h, (D,), eps=1e-6)
    e = e0 = None
    if "adaln" in f:
        t = 1000.0 * float(np.float32(sigma))
        fr = torch.logspace(0, -4.0 * 127 / 128, 128, base=10.0, dtype=torch.float64)
        s = torch.cat([torch.cos(t * fr), torch.sin(t * fr)])
        e = Fnn.linear(Fnn.silu(Fnn.linear(s, tw["t_w1"], tw["t_b1"])), tw["t_w2"], tw["t_b2"])
        e0 = Fnn.linear(Fnn.silu(e), tw["t_w3"], tw["t_b3"]).view(6, D)
    E = None
    if c.n_text:
        tx = synth.text_inputs(c)
        E = Fnn.linear(t64(tx["text"]), t64(tx["w_t"]))
        Eu = Fnn.linear(t64(synth.text_inputs_uncond(c)), t64(tx["w_t"]))
    outs = []
    for branch in ((0, 1) if "cfg" in f else (0,)):
        h = Fnn.linear(t64(x), t64(io["w_in"]))
        for l in range(c.L):
            w = synth.block_weights(c, l)
            fw = {k: t64(v) for k, v in synth.feature_weights(c, l).items()}
            mod = (fw["mod"] + e0) if e0 is not None else None
            a = ln(h) if mod is None else ln(h) * (1 + mod[1]) + mod[0]
            qkv = Fnn.linear(a, t64(w["w_qkv"]))
            q, k = qk(qkv[:, :D], fw["q_gain"]), qk(qkv[:, D:2 * D], fw["k_gain"])
            y = Fnn.linear(mha(q, k, qkv[:, 2 * D:]), t64(w["w_o"]))
            h = h + (y if mod is None else y * mod[2])
            if c.n_text:
                Ex = E if branch == 0 else Eu
                qx = Fnn.linear(ln(h), t64(w["w_qx"]))
                h = h + Fnn.linear(mha(qx, Fnn.linear(Ex, t64(w["w_kx"])), Fnn.linear(Ex, t64(w["w_vx"]))),
                                   t64(w["w_ox"]))
            a2 = ln(h) if mod is None else ln(h) * (1 + mod[4]) + mod[3]
            y = Fnn.linear(Fnn.gelu(Fnn.linear(a2, t64(w["w_1"])), approximate="tanh"), t64(w["w_2"]))
            h = h + (y if mod is None else y * mod[5])
        if e is not None:
            hm = tw["head_mod"] + e
            hn = ln(h) * (1 + hm[1]) + hm[0]
        else:
            hn = ln(h)
        outs.append(Fnn.linear(hn, t64(io["w_out"])))
    if "cfg" in f:
        return (outs[1] + float(np.float32(c.cfg_scale)) * (outs[0] - outs[1])).numpy()
    return outs[0].numpy()


@pytest.mark.parametrize("features,n_text", [
    (("qk_norm",), 0), (("rope3d",), 0), (("adaln",), 0), (FEATS, 0),
    (FEATS + ("cfg",), 8), (("cfg",), 8)])
def test_featured_dense_velocity_matches_torch_model(features, n_text):
    c = _cfg(features, n_text=n_text, text_dim=24 if n_text else 0)
    m = _model(c)
    x = synth.x0(c)
    for sigma in (1.0, 0.625):
        np.testing.assert_allclose(O.dense_velocity(m, x, sigma), _torch_dense_velocity(c, x, sigma),
                                   rtol=2e-4, atol=2e-5)


def test_featured_full_budget_reduces_to_dense_euler():
    # Every token active every iteration: HSA with caches, positions of the
    # active rows and per-iteration modulation equals the plain Euler loop.
    c = _cfg(FEATS + ("cfg",), n_text=8, text_dim=24, budgets=(8, 8), L=1)
    m = _model(c)
    sched = O.Schedule(T=8, budgets=[8, 8], counts=c.counts(), regroup=(3, 5))
    sigma = synth.sigma_schedule(8)
    st = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    O.sample(m, sched, st, sigma)
    ref = O.dense_euler_sample(m, synth.x0(c), sigma, 8)
    np.testing.assert_allclose(st.x, ref, rtol=1e-12, atol=1e-12)


def test_identity_modulation_is_the_plain_block():
    # shift = scale = 0 and unit gates: the adaLN block is the unmodulated block
    c = _cfg(("adaln",))
    m = _model(c)
    rs = np.random.default_rng(8)
    h = rs.standard_normal((10, c.D))
    idx = np.sort(rs.choice(c.N, 10, replace=False))
    kc1, vc1 = np.zeros((c.N, c.D)), np.zeros((c.N, c.D))
    kc2, vc2 = np.zeros((c.N, c.D)), np.zeros((c.N, c.D))
    ident = np.zeros((6, c.D))
    ident[2] = ident[5] = 1.0
    got = O.block_forward(m, 0, h, idx, kc1, vc1, mod=ident)
    ref = O.block_forward(m, 0, h, idx, kc2, vc2)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(kc1, kc2)
    # zero gates: the residual stream passes through, the caches still refresh
    zero = np.zeros((6, c.D))
    kc3, vc3 = np.zeros((c.N, c.D)), np.zeros((c.N, c.D))
    got = O.block_forward(m, 0, h, idx, kc3, vc3, mod=zero)
    np.testing.assert_array_equal(got, O.round_to_f32(h))
    np.testing.assert_array_equal(kc3, kc2)


def test_guidance_scale_one_is_the_conditional_model():
    c = _cfg(FEATS + ("cfg",), n_text=8, text_dim=24).with_(cfg_scale=1.0)
    with_cfg = _model(c)
    without = _model(c, drop=("cfg",))
    x = synth.x0(c)
    np.testing.assert_array_equal(O.dense_velocity(with_cfg, x, 0.5), O.dense_velocity(without, x, 0.5))


def test_guidance_with_equal_text_sets_keeps_caches_equal():
    c = _cfg(FEATS + ("cfg",), n_text=8, text_dim=24, L=1)
    m = _model(c)
    for b in m.blocks:
        b["k_text_u"], b["v_text_u"] = b["k_text"], b["v_text"]
    st = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    sched = O.Schedule(T=8, budgets=[8, 4], counts=c.counts())
    sigma = synth.sigma_schedule(8)
    tr = O.sample(m, sched, st, sigma, iters=range(3))
    np.testing.assert_array_equal(st.k_cache, st.k_cache_u)
    np.testing.assert_array_equal(st.v_cache, st.v_cache_u)
    ref = _model(c, drop=("cfg",))
    st2 = O.init_state(ref.dims, synth.x0(c), synth.group0(c))
    tr2 = O.sample(ref, sched, st2, sigma, iters=range(3))
    np.testing.assert_allclose(tr[-1]["v_new"], tr2[-1]["v_new"], rtol=1e-6, atol=1e-7)


def test_featured_row_sampled_block_equals_full_block():
    c = _cfg(FEATS)
    m = _model(c)
    rs = np.random.default_rng(9)
    idx = np.sort(rs.choice(c.N, 12, replace=False))
    h = rs.standard_normal((12, c.D))
    e, e0 = O.time_embedding(m, 0.75)
    mod = O.block_modulation(m, 0, e0)
    kc, vc = np.zeros((c.N, c.D)), np.zeros((c.N, c.D))
    full = O.block_forward(m, 0, h, idx, kc, vc, mod=mod)
    rows = np.array([0, 5, 11])
    kc2, vc2 = np.zeros((c.N, c.D)), np.zeros((c.N, c.D))
    part = O.block_forward(m, 0, h, idx, kc2, vc2, rows=rows, mod=mod)
    np.testing.assert_array_equal(part, full[rows])
    np.testing.assert_array_equal(kc2, kc)
