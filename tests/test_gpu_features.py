"""GPU parity of the optional Wan-style block features (qk-RMSNorm, 3D rotary
embedding, adaLN timestep modulation, classifier-free guidance batch 2)
against the CPU oracle, through the C ABI: each kernel on its own, one block,
whole sampling runs, and a Wan-1.3B-shaped block on sampled rows."""
import numpy as np
import pytest
import torch

import synth
from oracle import hsa_oracle as O
from tests.gpu_common import DEV, TOL_BF16, TOL_F32, assert_rows_close, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu

H = None
ALL = ("qk_norm", "rope3d", "adaln")


@pytest.fixture(scope="module", autouse=True)
def lib():
    global H
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from token_sparse_attention_compact_amd import hsa
    hsa.load()
    H = hsa
    yield hsa


def tdt(c):
    return torch.bfloat16 if c.dtype == "bf16" else torch.float32


def tol(c):
    return TOL_BF16 if c.dtype == "bf16" else TOL_F32


def oracle_dims(c):
    f = set(c.features)
    return O.Dims(N=c.N, C=c.C, D=c.D, H=c.H, Dh=c.Dh, F=c.F, L=c.L, bf16=(c.dtype == "bf16"),
                  n_text=c.n_text, qk_norm="qk_norm" in f, rope3d="rope3d" in f,
                  adaln="adaln" in f, cfg="cfg" in f, grid=c.grid)


def oracle_model(c):
    blocks = []
    for l in range(c.L):
        b = synth.block_weights(c, l)
        b.update(synth.feature_weights(c, l))
        blocks.append(b)
    text = synth.text_inputs(c) if c.n_text else None
    tu = synth.text_inputs_uncond(c) if c.n_text else None
    return O.make_model(oracle_dims(c), synth.io_weights(c), blocks, text, synth.time_weights(c), tu,
                        c.cfg_scale)


def device_model(c, k_cache=None, v_cache=None):
    """Device copy of the seeded weights with every feature parameter the
    config's features need; caches zero or given [L][N][D] (both branches)."""
    dt = tdt(c)
    f = set(c.features)
    dims = H.make_dims(c.N, c.C, c.D, c.H, c.Dh, c.F, c.L, c.n_text, dt, features=f, grid=c.grid)
    io = synth.io_weights(c)
    tx = synth.text_inputs(c) if c.n_text else None

    def project(text):
        E = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
        H.hsa_linear(dev(text, dt), dev(tx["w_t"], dt), E)
        return E

    E = project(tx["text"]) if c.n_text else None
    Eu = project(synth.text_inputs_uncond(c)) if "cfg" in f else None
    blocks = []
    for l in range(c.L):
        w = synth.block_weights(c, l)
        fw = synth.feature_weights(c, l)
        b = {k: dev(v, dt) for k, v in w.items() if k in ("w_qkv", "w_o", "w_1", "w_2", "w_qx", "w_ox")}
        cache = lambda src: (torch.zeros(c.N, c.D, dtype=dt, device=DEV) if src is None else dev(src[l], dt))
        b["k_cache"], b["v_cache"] = cache(k_cache), cache(v_cache)
        if c.n_text:
            for name, Ex in (("", E), ("_u", Eu)):
                if Ex is None:
                    continue
                b["k_text" + name] = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
                b["v_text" + name] = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
                H.hsa_linear(Ex, dev(w["w_kx"], dt), b["k_text" + name])
                H.hsa_linear(Ex, dev(w["w_vx"], dt), b["v_text" + name])
        if "cfg" in f:
            b["k_cache_u"], b["v_cache_u"] = cache(k_cache), cache(v_cache)
        b["q_gain"], b["k_gain"], b["mod"] = dev(fw["q_gain"]), dev(fw["k_gain"]), dev(fw["mod"])
        blocks.append(b)
    time = {k: dev(v) for k, v in synth.time_weights(c).items()}
    return H.DeviceModel(dims, dev(io["w_in"], dt), dev(io["w_out"], dt), blocks, time, c.cfg_scale)


def tiny(features, dtype="f32", Dh=64, H_=2, grid=(3, 5, 7), **kw):
    base = dict(grid=grid, C=16, D=H_ * Dh, H=H_, Dh=Dh, F=4 * H_ * Dh, L=1, dtype=dtype, T=8,
                budgets=(8, 4), shares=(0.5, 0.5), regroup=(3, 4, 5, 6, 7), features=tuple(features))
    base.update(kw)
    return synth.CONFIGS[1].with_(**base)


# ---------------------------------------------------------------- kernels

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dh,H_", [(64, 3), (128, 2), (128, 12), (64, 32), (128, 40)])
@pytest.mark.parametrize("features", [("qk_norm",), ("rope3d",), ("qk_norm", "rope3d")])
def test_qk_norm_rope_kernel(dtype, Dh, H_, features):
    """q rows and the K-cache rows of 61 active tokens (of 105 on a 3x5x7 grid,
    ragged against the 4-row blocks) against the oracle's RMSNorm + rotation;
    cache rows of skipped tokens stay bit-identical.  Widths D = 192, 256,
    1536 and 2048 (the loop form) and 5120 (bf16: both rows held in
    registers, 10 chunks of 16 bytes per lane; float32: the loop form)."""
    c = tiny(features, dtype, Dh=Dh, H_=H_)
    say(f"qk_norm_rope {dtype} Dh={Dh} {features}")
    dt = tdt(c)
    rs = np.random.default_rng(11)
    idx = np.sort(rs.choice(c.N, 61, replace=False)).astype(np.int32)
    q = rs.standard_normal((idx.size, c.D)).astype(np.float32) * 2
    kc = rs.standard_normal((c.N, c.D)).astype(np.float32) * 2
    fw = synth.feature_weights(c, 0)
    tq, tk = dev(q, dt), dev(kc, dt)
    q_in, k_in = host(tq), host(tk)                  # the stored values both sides start from
    dims = H.make_dims(c.N, c.C, c.D, c.H, c.Dh, c.F, 1, 0, dt, features=features, grid=c.grid)
    H.hsa_qk_norm_rope(tq, tk, dev(idx, torch.int32), idx.size, dims, dev(fw["q_gain"]), dev(fw["k_gain"]))
    torch.cuda.synchronize()
    od = oracle_dims(c)
    st = O.Store(c.dtype == "bf16")
    q_ref = st.act(O.qk_transform(od, q_in, idx, fw["q_gain"]))
    k_ref = st.act(O.qk_transform(od, k_in[idx], idx, fw["k_gain"]))
    bound = 5e-3 if dtype == "bf16" else 1e-5
    assert rel_l2(host(tq), q_ref) < bound
    kg = host(tk)
    assert rel_l2(kg[idx], k_ref) < bound
    skipped = np.setdiff1d(np.arange(c.N), idx)
    np.testing.assert_array_equal(kg[skipped], k_in[skipped])


@pytest.mark.parametrize("D", [128, 1536])
def test_time_embed_kernel(D):
    c = tiny(("adaln",), D=D, H_=D // 64)
    say(f"time_embed D={D}")
    om = oracle_model(c)
    m = device_model(c)
    e = torch.empty(D, device=DEV)
    e0 = torch.empty(6, D, device=DEV)
    for sigma in (1.0, 0.6, 0.025, 0.0):
        H.hsa_time_embed(m, sigma, e, e0)
        torch.cuda.synchronize()
        e_ref, e0_ref = O.time_embedding(om, sigma)
        assert rel_l2(host(e), e_ref) < 1e-5, sigma
        assert rel_l2(host(e0), e0_ref) < 1e-5, sigma


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,D", [(37, 256), (130, 1536), (9, 320), (70, 5120), (5, 2304)])
def test_modulated_layernorm_and_unembed(dtype, rows, D):
    """LN(h) (1 + scale) + shift into the model dtype, and the modulated final
    LayerNorm + unembed, on the register-resident (D % 256 == 0) and the
    two-pass (D = 320) LayerNorm paths; the unembed on its matrix-core
    (D <= 1536), one-pass wide-row (D = 2304, 5120, four rows per wavefront,
    ragged) and two-pass (D = 320) forms, every row within tolerance."""
    say(f"modulated LN {dtype} rows={rows} D={D}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    st = O.Store(dtype == "bf16")
    rs = np.random.default_rng(12)
    h = (rs.standard_normal((rows, D)) * 3 + 0.5).astype(np.float32)
    shift = (rs.standard_normal(D) * 0.2).astype(np.float32)
    scale = (rs.standard_normal(D) * 0.2).astype(np.float32)
    out = torch.empty(rows, D, dtype=dt, device=DEV)
    H.hsa_layernorm(dev(h), out, dev(shift), dev(scale))
    ref = st.act(O.modulated_layer_norm(h, shift, scale))
    assert rel_l2(host(out), ref) < (5e-3 if dtype == "bf16" else 1e-6)
    w_out = rs.standard_normal((16, D)).astype(np.float32) * D ** -0.5
    if dtype == "bf16":
        w_out = synth.to_bf16_values(w_out)
    vn = torch.empty(rows, 16, device=DEV)
    H.hsa_unembed(dev(h), dev(w_out, dt), vn, rows, dev(shift), dev(scale))
    ref = O.round_to_f32(O.modulated_layer_norm(h, shift, scale) @ w_out.astype(np.float64).T)
    assert_rows_close(host(vn), ref, 1e-5, "modulated unembed rows")


@pytest.mark.parametrize("dtype,M,N,K", [("bf16", 1030, 1536, 1536), ("bf16", 77, 300, 256),
                                         ("f32", 45, 132, 68)])
def test_gated_linear_residual(dtype, M, N, K):
    say(f"gated residual {dtype} {M}x{N}x{K}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rs = np.random.default_rng(13)
    a = rs.standard_normal((M, K)).astype(np.float32)
    w = (rs.standard_normal((N, K)) * K ** -0.5).astype(np.float32)
    if dtype == "bf16":
        a, w = synth.to_bf16_values(a), synth.to_bf16_values(w)
    h = rs.standard_normal((M, N)).astype(np.float32)
    gate = (1 + 0.3 * rs.standard_normal(N)).astype(np.float32)
    th = dev(h)
    H.hsa_linear_residual(dev(a, dt), dev(w, dt), th, gate=dev(gate))
    ref = O.round_to_f32(h + (a.astype(np.float64) @ w.astype(np.float64).T) * gate)
    assert rel_l2(host(th), ref) < 1e-6


def test_guidance_kernel():
    rs = np.random.default_rng(14)
    vc = rs.standard_normal((333, 16)).astype(np.float32)
    vu = rs.standard_normal((333, 16)).astype(np.float32)
    for g in (5.0, 1.0, 0.0, -1.5):
        tv = dev(vu)
        H.hsa_guidance(dev(vc), tv, g=g)
        got = host(tv)
        ref = O.guidance(vc, vu, g)
        np.testing.assert_allclose(got, ref, rtol=2e-6, atol=2e-6)
        if g in (1.0, 0.0):
            np.testing.assert_array_equal(got, vc if g == 1.0 else vu)


# ---------------------------------------------------------------- one block

@pytest.mark.parametrize("features,n_text,branch,Dh", [(ALL, 0, 0, 128), (ALL + ("cfg",), 16, 0, 128),
                                                       (ALL + ("cfg",), 16, 1, 128), (("rope3d",), 0, 0, 128),
                                                       (ALL, 0, 0, 64), (ALL + ("cfg",), 16, 1, 64)])
def test_featured_block_forward_bf16(features, n_text, branch, Dh):
    """One bf16 block (D 256 as 2x128 or 4x64 heads) on 211 of 640 tokens with
    stale cache rows, the timestep projection from the library, and the
    unconditional branch's text set and caches when branch == 1."""
    c = tiny(features, "bf16", Dh=Dh, H_=256 // Dh, grid=(2, 20, 16), n_text=n_text,
             text_dim=64 if n_text else 0)
    say(f"featured block bf16 {features} n_text={n_text} branch={branch} Dh={Dh}")
    om = oracle_model(c)
    kc, vc = synth.kv_cache(c)
    m = device_model(c, kc[None], vc[None])
    rs = np.random.default_rng(15)
    idx = np.sort(rs.choice(c.N, 211, replace=False)).astype(np.int32)
    h = rs.standard_normal((idx.size, c.D)).astype(np.float32)
    e0 = None
    mod = None
    if "adaln" in features:
        e = torch.empty(c.D, device=DEV)
        e0 = torch.empty(6, c.D, device=DEV)
        H.hsa_time_embed(m, 0.7, e, e0)
        _, oe0 = O.time_embedding(om, 0.7)
        mod = O.block_modulation(om, 0, oe0)
    ws = torch.empty(H.hsa_workspace_size(m.dims), dtype=torch.uint8, device=DEV)
    th = dev(h)
    H.hsa_block_forward(m, 0, th, dev(idx, torch.int32), idx.size, ws, e0=e0, branch=branch)
    torch.cuda.synchronize()
    kref, vref = kc.astype(np.float64), vc.astype(np.float64)
    ref = O.block_forward(om, 0, h, idx, kref, vref, mod=mod, branch=branch)
    assert rel_l2(host(th), ref) < 5e-3
    sfx = "_u" if branch else ""
    kg = host(m.blocks[0]["k_cache" + sfx])
    skipped = np.setdiff1d(np.arange(c.N), idx)
    np.testing.assert_array_equal(kg[skipped], kc[skipped])
    assert rel_l2(kg[idx], kref[idx]) < 5e-3
    assert rel_l2(host(m.blocks[0]["v_cache" + sfx])[idx], vref[idx]) < 5e-3
    if "cfg" in features:
        # the other branch's caches are untouched
        other = host(m.blocks[0]["k_cache" if branch else "k_cache_u"])
        np.testing.assert_array_equal(other, kc)


@pytest.mark.parametrize("frac", [0.25, 0.125])
def test_featured_block_full_size_sampled_rows(frac):
    """Wan-1.3B-shaped block (D 1536, 12x128 heads, F 8960, N = 32760 on the
    21x30x52 grid) with qk-RMSNorm, 3D rotation and timestep modulation, 25%
    or 12.5% of the tokens active at random: every active K/V row and 48
    sampled output rows against the oracle."""
    c = synth.CONFIGS[2].with_(features=ALL)
    nA = synth.n_active_for_fraction(c.N, frac)
    say(f"featured block full-size nA={nA}")
    om = oracle_model(c)
    kc, vc = synth.kv_cache(c)
    idx = synth.active_random(c, nA)
    h = synth.hidden_states(c, nA)
    m = device_model(c, kc[None], vc[None])
    e = torch.empty(c.D, device=DEV)
    e0 = torch.empty(6, c.D, device=DEV)
    H.hsa_time_embed(m, 0.45, e, e0)
    ws = torch.empty(H.hsa_workspace_size(m.dims), dtype=torch.uint8, device=DEV)
    th = dev(h)
    H.hsa_block_forward(m, 0, th, dev(idx, torch.int32), nA, ws, e0=e0)
    torch.cuda.synchronize()
    _, oe0 = O.time_embedding(om, 0.45)
    rows = np.sort(np.random.default_rng(5).choice(nA, 48, replace=False))
    kref, vref = kc.astype(np.float64), vc.astype(np.float64)
    ref = O.block_forward(om, 0, h, idx, kref, vref, rows=rows, mod=O.block_modulation(om, 0, oe0))
    assert_rows_close(host(th)[rows], ref, TOL_BF16, "block output rows")
    kg = host(m.blocks[0]["k_cache"])
    skipped = np.setdiff1d(np.arange(c.N), idx)
    np.testing.assert_array_equal(kg[skipped], kc[skipped])
    assert_rows_close(kg[idx], kref[idx], TOL_BF16, "K rows")
    assert_rows_close(host(m.blocks[0]["v_cache"])[idx], vref[idx], TOL_BF16, "V rows")


# ---------------------------------------------------------------- whole runs

def select_margin(score, counts):
    s = np.sort(np.asarray(score, np.float64))[::-1]
    gaps = []
    b = 0
    for n in counts[:-1]:
        b += n
        if 0 < b < s.size:
            hi, lo = s[b - 1], s[b]
            if np.isinf(hi):
                if hi != lo:
                    gaps.append(np.inf)
                continue
            gaps.append(abs(hi - lo) / max(abs(hi), 1e-30))
    return min(gaps) if gaps else np.inf


@pytest.mark.parametrize("features,n_text,empty,m", [(ALL, 0, False, 0), (ALL + ("cfg",), 8, False, 0),
                                                     (ALL + ("cfg",), 8, True, 0), (ALL + ("cfg",), 8, True, 2)])
def test_featured_step_full_run_f32(features, n_text, empty, m):
    """DiT-lite float32 on the 4x8x8 grid with the features on: all 8
    iterations (regrouping from i = 3 on) against the oracle, every state
    array after every iteration, both branches' caches under guidance.
    `empty`: budgets {8, 4, 2} with an empty full-budget group, so every odd
    iteration has no active token (the cached Euler step alone); `m`: phase
    window, the first and last m iterations run every token."""
    c = synth.CONFIGS[1].with_(features=features, n_text=n_text, text_dim=32 if n_text else 0, m=m)
    if empty:
        c = c.with_(budgets=(8, 4, 2), shares=(0.0, 0.5, 0.5))
    say(f"featured hsa_step fp32 full run {features}")
    om = oracle_model(c)
    dm = device_model(c)
    sched = H.make_schedule(c.T, c.budgets, c.counts(), m=c.m)
    osched = O.Schedule(c.T, list(c.budgets), c.counts(), m=c.m, regroup=c.regroup)
    sigma = synth.sigma_schedule(c.T)
    x0, g0 = synth.x0(c), synth.group0(c)
    st = H.DeviceState(dm.dims, dev(x0), dev(g0, torch.uint8))
    ost = O.init_state(om.dims, x0, g0)
    for i in range(c.T):
        if i in c.regroup:
            fin = np.isfinite(ost.score)
            dev_rel = np.max(np.abs(host(st.score)[fin] - ost.score[fin]) / np.abs(ost.score[fin]))
            assert select_margin(ost.score, c.counts()) > 10 * dev_rel
        H.hsa_step(dm, sched, st, i, float(sigma[i]), float(sigma[i + 1]), i in c.regroup)
        torch.cuda.synchronize()
        O.sample(om, osched, ost, sigma, iters=[i])
        np.testing.assert_array_equal(st.group.cpu().numpy(), ost.group)
        assert rel_l2(host(st.x), ost.x) < TOL_F32
        assert rel_l2(host(st.v_hat), ost.v_hat) < TOL_F32
        fin = np.isfinite(ost.score)
        np.testing.assert_array_equal(np.isfinite(host(st.score)), fin)
        if fin.any():
            assert rel_l2(host(st.score)[fin], ost.score[fin]) < TOL_F32
        assert rel_l2(host(dm.blocks[0]["k_cache"]), ost.k_cache[0]) < TOL_F32
        if "cfg" in features:
            assert rel_l2(host(dm.blocks[0]["k_cache_u"]), ost.k_cache_u[0]) < TOL_F32
            assert rel_l2(host(dm.blocks[0]["v_cache_u"]), ost.v_cache_u[0]) < TOL_F32


def test_featured_step_mid_run_bf16():
    """One 2-block bf16 iteration with every feature and guidance, from a
    synthetic mid-run state, regrouping first."""
    c = tiny(ALL + ("cfg",), "bf16", Dh=128, H_=2, grid=(2, 20, 16), n_text=16, text_dim=64, L=2,
             T=40, budgets=(40, 20, 10), shares=(0.25, 0.25, 0.5), regroup=(10, 20, 30))
    say("featured hsa_step mid-run bf16")
    i = 10
    om = oracle_model(c)
    s0 = synth.mid_run_state(c)
    m = device_model(c, s0["k_cache"], s0["v_cache"])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    st = H.DeviceState(m.dims, dev(s0["x"]), dev(s0["group"], torch.uint8), dev(s0["v_hat"]),
                       dev(s0["score"]))
    H.hsa_step(m, sched, st, i, float(sigma[i]), float(sigma[i + 1]), True)
    torch.cuda.synchronize()
    f64 = lambda a: np.asarray(a, np.float64)
    ost = O.State(f64(s0["x"]), f64(s0["v_hat"]), f64(s0["score"]), s0["group"].copy(),
                  f64(s0["k_cache"]), f64(s0["v_cache"]), f64(s0["k_cache"]), f64(s0["v_cache"]))
    out = O.hsa_iteration(om, O.Schedule(c.T, list(c.budgets), c.counts()), ost, i, sigma[i],
                          sigma[i + 1], True)
    np.testing.assert_array_equal(st.group.cpu().numpy(), ost.group)
    nA = out["active_idx"].size
    np.testing.assert_array_equal(st.active_idx[:nA].cpu().numpy(), out["active_idx"])
    a = out["active_idx"]
    skipped = np.setdiff1d(np.arange(c.N), a)
    # errors over the computed rows only (skipped rows are exact copies, checked below)
    assert_rows_close(host(st.x)[a], ost.x[a], TOL_BF16, "x")
    assert rel_l2(host(st.x)[a], ost.x[a]) < 1e-3
    assert_rows_close(host(st.v_hat)[a], ost.v_hat[a], TOL_BF16, "v_hat")
    assert_rows_close(host(st.score)[a][:, None], ost.score[a][:, None], TOL_BF16, "score")
    np.testing.assert_array_equal(host(st.v_hat)[skipped], s0["v_hat"][skipped])
    np.testing.assert_array_equal(host(st.score)[skipped], s0["score"][skipped])
    for l in range(c.L):
        for sfx, ref in (("", ost.k_cache), ("_u", ost.k_cache_u)):
            kg = host(m.blocks[l]["k_cache" + sfx])
            np.testing.assert_array_equal(kg[skipped], s0["k_cache"][l][skipped])
            assert_rows_close(kg[a], ref[l][a], TOL_BF16, f"layer {l} K{sfx} rows")


@pytest.mark.timeout(400)     # the oracle's side takes about a minute of host time
def test_featured_step_14b_shape():
    """The 14B-shaped block (N = 75600 on the 21x45x80 grid, D 5120, 40x128
    heads, F 13824, 512 text tokens) with every feature and guidance, one
    25%-active iteration from a synthetic mid-run state: properties that hold
    at any size, every active row's fresh K/V in both branches against the
    oracle, and the whole iteration (both branches, guidance, Euler) on 16
    sampled active tokens: their v_hat, x and score."""
    c = synth.CONFIGS[4].with_(L=1, features=ALL + ("cfg",))
    say("featured hsa_step 14B-shaped")
    i = 11
    om = oracle_model(c)
    s0 = synth.mid_run_state(c)
    m = device_model(c, s0["k_cache"], s0["v_cache"])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    st = H.DeviceState(m.dims, dev(s0["x"]), dev(s0["group"], torch.uint8), dev(s0["v_hat"]),
                       dev(s0["score"]))
    H.hsa_step(m, sched, st, i, float(sigma[i]), float(sigma[i + 1]), False)
    torch.cuda.synchronize()
    idx, pos = O.active_set(s0["group"], c.budgets, c.T, i)
    assert idx.size == 18900
    np.testing.assert_array_equal(st.active_idx[:idx.size].cpu().numpy(), idx)
    np.testing.assert_array_equal(st.pos.cpu().numpy(), pos)
    skipped = np.setdiff1d(np.arange(c.N), idx)
    ds = np.float32(np.float32(sigma[i + 1]) - np.float32(sigma[i]))
    xs = (s0["x"][skipped].astype(np.float64) + np.float64(ds) * s0["v_hat"][skipped]).astype(np.float32)
    np.testing.assert_array_equal(host(st.x)[skipped].astype(np.float32), xs)
    np.testing.assert_array_equal(host(st.v_hat)[skipped], s0["v_hat"][skipped])
    kc, kcu = host(m.blocks[0]["k_cache"]), host(m.blocks[0]["k_cache_u"])
    vc, vcu = host(m.blocks[0]["v_cache"]), host(m.blocks[0]["v_cache_u"])
    for a in (kc, kcu):
        np.testing.assert_array_equal(a[skipped], s0["k_cache"][0][skipped])
    for a in (vc, vcu):
        np.testing.assert_array_equal(a[skipped], s0["v_cache"][0][skipped])
    # text enters after self-attention: layer-0 fresh K/V are the same in both branches
    np.testing.assert_array_equal(kcu[idx], kc[idx])
    np.testing.assert_array_equal(vcu[idx], vc[idx])
    kg, vg = kc[idx], vc[idx]
    del kc, kcu, vc, vcu
    # the oracle: both branches on 16 sampled rows (every active row's K/V written)
    rows = np.sort(np.random.default_rng(3).choice(idx.size, 16, replace=False))
    tok = idx[rows]
    e, e0 = O.time_embedding(om, sigma[i])
    mod, hmod = O.block_modulation(om, 0, e0), O.head_modulation(om, e)
    h = O.embed(om, s0["x"], idx)
    say("oracle: conditional branch")
    kref, vref = s0["k_cache"][0].astype(np.float64), s0["v_cache"][0].astype(np.float64)
    v_c = O.unembed(om, O.block_forward(om, 0, h, idx, kref, vref, rows=rows, mod=mod, branch=0), hmod)
    assert_rows_close(kg, kref[idx], TOL_BF16, "K rows")
    assert_rows_close(vg, vref[idx], TOL_BF16, "V rows")
    # The unconditional branch writes the same layer-0 K/V rows (text enters after
    # self-attention), so its cache after the update is kref/vref: run its sampled
    # rows against that cache (block_forward rewrites only their own rows).
    say("oracle: unconditional branch")
    v_u = O.unembed(om, O.block_forward(om, 0, h[rows], tok, kref, vref, mod=mod, branch=1), hmod)
    del kref, vref
    v_new = O.guidance(v_c, v_u, om.cfg_scale)
    x_ref, vh_ref, sc_ref = O.euler_update(s0["x"][tok], s0["v_hat"][tok], s0["score"][tok], v_new,
                                           np.arange(rows.size), ds, update_score=True)
    e_v = assert_rows_close(host(st.v_hat)[tok], vh_ref, TOL_BF16, "v_hat")
    e_x = assert_rows_close(host(st.x)[tok], x_ref, TOL_BF16, "x")
    e_s = assert_rows_close(host(st.score)[tok][:, None], sc_ref[:, None], TOL_BF16, "score")
    say(f"sampled tokens: v_hat {e_v}, x {e_x}, score {e_s} (whole, worst row)")


def test_featured_step_graph_capture_replays_match_eager():
    """The featured iteration (timestep MLP, modulated LayerNorms, gated
    residuals, qk-norm + rotation pass, two guidance branches and the
    combine) enqueues kernels only, so it captures in a HIP graph: three
    replays from the same state, with other device work in between, each
    equal the eager iteration bit for bit."""
    c = tiny(ALL + ("cfg",), "bf16", Dh=128, H_=2, grid=(2, 20, 16), n_text=16, text_dim=64, L=2,
             T=40, budgets=(40, 20, 10), shares=(0.25, 0.25, 0.5), regroup=(10, 20, 30))
    say("featured hsa_step graph capture")
    i = 10
    s0 = synth.mid_run_state(c)
    m = device_model(c, s0["k_cache"], s0["v_cache"])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    st = H.DeviceState(m.dims, dev(s0["x"]), dev(s0["group"], torch.uint8), dev(s0["v_hat"]),
                       dev(s0["score"]))
    bufs = [st.x, st.v_hat, st.score, st.group] + [
        b[n] for b in m.blocks for n in ("k_cache", "v_cache", "k_cache_u", "v_cache_u")]
    init = [b.clone() for b in bufs]

    def restore():
        for b, v in zip(bufs, init):
            b.copy_(v)

    def step():
        H.hsa_step(m, sched, st, i, float(sigma[i]), float(sigma[i + 1]), True)

    restore()
    step()
    torch.cuda.synchronize()
    eager = [b.clone() for b in bufs]
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = torch.randn(512, 512, device=DEV)
    for rep in range(3):
        restore()
        other = other @ other.T / 512.0
        g.replay()
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            assert torch.equal(b, e), f"replay {rep} differs from the eager iteration"
