"""GPU parity of whole blocks and whole HSA iterations against the CPU oracle,
through the C ABI (hsa_block_forward, hsa_step)."""
import numpy as np
import pytest
import torch

import synth
from oracle import hsa_oracle as O
from tests.gpu_common import (DEV, TOL_BF16, TOL_F32, assert_rows_close, dev, host,
                              oracle_block_all_rows, rel_l2, say)

pytestmark = pytest.mark.gpu

H = None


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


def oracle_model(c):
    dims = O.Dims(N=c.N, C=c.C, D=c.D, H=c.H, Dh=c.Dh, F=c.F, L=c.L, bf16=(c.dtype == "bf16"),
                  n_text=c.n_text)
    text = synth.text_inputs(c) if c.n_text else None
    return O.make_model(dims, synth.io_weights(c), [synth.block_weights(c, l) for l in range(c.L)], text)


def device_model(c, om, k_cache=None, v_cache=None):
    """Device copy of the same seeded weights; caches zero or given [L][N][D]."""
    dt = tdt(c)
    dims = H.make_dims(c.N, c.C, c.D, c.H, c.Dh, c.F, c.L, c.n_text, dt)
    io = synth.io_weights(c)
    blocks = []
    for l in range(c.L):
        w = synth.block_weights(c, l)
        b = {k: dev(v, dt) for k, v in w.items() if k in ("w_qkv", "w_o", "w_1", "w_2", "w_qx", "w_ox")}
        b["k_cache"] = (torch.zeros(c.N, c.D, dtype=dt, device=DEV) if k_cache is None
                        else dev(k_cache[l], dt))
        b["v_cache"] = (torch.zeros(c.N, c.D, dtype=dt, device=DEV) if v_cache is None
                        else dev(v_cache[l], dt))
        if c.n_text:
            # text K/V: the oracle's once-per-run projection is recomputed here with the library
            tx = synth.text_inputs(c)
            E = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
            H.hsa_linear(dev(tx["text"], dt), dev(tx["w_t"], dt), E)
            b["k_text"] = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
            b["v_text"] = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
            H.hsa_linear(E, dev(w["w_kx"], dt), b["k_text"])
            H.hsa_linear(E, dev(w["w_vx"], dt), b["v_text"])
        blocks.append(b)
    return H.DeviceModel(dims, dev(io["w_in"], dt), dev(io["w_out"], dt), blocks)


def small_bf16(**kw):
    base = dict(grid=(2, 20, 16), C=16, D=256, H=2, Dh=128, F=512, L=2, dtype="bf16", T=40,
                budgets=(40, 20, 10), shares=(0.25, 0.25, 0.5), regroup=(10, 20, 30))
    base.update(kw)
    return synth.CONFIGS[3].with_(**base)


# ---------------------------------------------------------------- one block

@pytest.mark.parametrize("n_text,Dh", [(0, 128), (16, 128), (0, 64), (16, 64)])
def test_block_forward_small_bf16(n_text, Dh):
    c = small_bf16(L=1, n_text=n_text, text_dim=64 if n_text else 0, H=256 // Dh, Dh=Dh)
    say(f"block_forward small bf16 n_text={n_text} Dh={Dh}")
    om = oracle_model(c)
    kc, vc = synth.kv_cache(c)
    rs = np.random.default_rng(1)
    idx = np.sort(rs.choice(c.N, 211, replace=False)).astype(np.int32)
    h = rs.standard_normal((idx.size, c.D)).astype(np.float32)
    m = device_model(c, om, kc[None], vc[None])
    dims = m.dims
    ws = torch.empty(H.hsa_workspace_size(dims), dtype=torch.uint8, device=DEV)
    th = dev(h)
    H.hsa_block_forward(m, 0, th, dev(idx, torch.int32), idx.size, ws)
    kref, vref = kc.astype(np.float64), vc.astype(np.float64)
    ref = O.block_forward(om, 0, h, idx, kref, vref)
    assert rel_l2(host(th), ref) < TOL_BF16
    assert rel_l2(host(th), ref) < 5e-3
    k_gpu = host(m.blocks[0]["k_cache"])
    skipped = np.setdiff1d(np.arange(c.N), idx)
    np.testing.assert_array_equal(k_gpu[skipped], kc[skipped])
    assert rel_l2(k_gpu[idx], kref[idx]) < 5e-3
    assert rel_l2(host(m.blocks[0]["v_cache"])[idx], vref[idx]) < 5e-3


@pytest.mark.parametrize("frac,pattern", [(0.25, "random"), (0.25, "blob"), (0.125, "random"),
                                          (0.0625, "blob")])
def test_block_forward_full_size_sampled_rows(frac, pattern):
    """Wan-1.3B-shaped block (D 1536, 12x128 heads, F 8960) over N = 32760 cached
    rows, active rows drawn at random or as contiguous spatial blobs (per frame
    the tokens nearest a drifting centre): every active row's K/V goes through
    the oracle, the block output is checked on 48 sampled active rows."""
    c = synth.CONFIGS[2]
    nA = synth.n_active_for_fraction(c.N, frac)
    say(f"block_forward full-size nA={nA} {pattern}")
    om = oracle_model(c)
    kc, vc = synth.kv_cache(c)
    idx = synth.active_random(c, nA) if pattern == "random" else synth.active_blob(c, nA)
    assert idx.size == nA and np.all(np.diff(idx) > 0)
    h = synth.hidden_states(c, nA)
    m = device_model(c, om, kc[None], vc[None])
    ws = torch.empty(H.hsa_workspace_size(m.dims), dtype=torch.uint8, device=DEV)
    th = dev(h)
    H.hsa_block_forward(m, 0, th, dev(idx, torch.int32), nA, ws)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(nA, 48, replace=False))
    kref, vref = kc.astype(np.float64), vc.astype(np.float64)
    ref = O.block_forward(om, 0, h, idx, kref, vref, rows=rows)
    assert_rows_close(host(th)[rows], ref, TOL_BF16, "block output rows")
    k_gpu = host(m.blocks[0]["k_cache"])
    skipped = np.setdiff1d(np.arange(c.N), idx)
    np.testing.assert_array_equal(k_gpu[skipped], kc[skipped])
    assert_rows_close(k_gpu[idx], kref[idx], TOL_BF16, "K rows")
    assert_rows_close(host(m.blocks[0]["v_cache"])[idx], vref[idx], TOL_BF16, "V rows")


# ---------------------------------------------------------------- whole iterations

def run_gpu(c, m, sched, state, iters, sigma, field=None):
    for i in iters:
        vf = None if field is None else dev(field(i))
        H.hsa_step(m, sched, state, i, float(sigma[i]), float(sigma[i + 1]), i in set(c.regroup), vf)
    torch.cuda.synchronize()


def select_margin(score, counts):
    """Smallest relative gap between the scores on either side of a group boundary.
    A boundary between two +inf scores (tokens without a second prediction yet)
    is an exact tie on both sides, broken by token index: it has no margin to
    lose and is skipped."""
    s = np.sort(np.asarray(score, np.float64))[::-1]
    gaps = []
    b = 0
    for n in counts[:-1]:
        b += n
        if 0 < b < s.size:
            hi, lo = s[b - 1], s[b]
            if np.isinf(hi):
                if hi != lo:
                    gaps.append(np.inf)   # +inf against a finite score: no rounding can flip it
                continue
            gaps.append(abs(hi - lo) / max(abs(hi), 1e-30))
    return min(gaps) if gaps else np.inf


@pytest.mark.parametrize("variant", ["cfg1", "empty_active_sets", "static_groups", "regroup_every_2"])
def test_step_cfg1_full_run_f32(variant):
    """DiT-lite float32: 8 iterations, budgets {8,4}, regrouping from i = 3 on.
    Variants: an empty full-budget group (budgets {8,4,2}, shares 0/50/50:
    every odd iteration has |A_i| = 0 and is the cached Euler step alone);
    static groups (never regrouped); three groups regrouped every 2nd
    iteration (budgets {8,4,2})."""
    c = synth.CONFIGS[1]
    if variant == "empty_active_sets":
        c = c.with_(budgets=(8, 4, 2), shares=(0.0, 0.5, 0.5))
        assert c.counts()[0] == 0
    elif variant == "static_groups":
        c = c.with_(regroup=())
    elif variant == "regroup_every_2":
        c = c.with_(budgets=(8, 4, 2), shares=(0.25, 0.25, 0.5), regroup=(2, 4, 6))
    say(f"hsa_step cfg1 fp32 full run ({variant})")
    om = oracle_model(c)
    m = device_model(c, om)
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    osched = O.Schedule(c.T, list(c.budgets), c.counts(), regroup=c.regroup)
    sigma = synth.sigma_schedule(c.T)
    x0, g0 = synth.x0(c), synth.group0(c)
    st = H.DeviceState(m.dims, dev(x0), dev(g0, torch.uint8))
    ost = O.init_state(om.dims, x0, g0)
    for i in range(c.T):
        if i in c.regroup:
            # Both sides rank their own float32 scores: the decision is the same when the gap at
            # every group boundary exceeds the GPU/oracle score deviation by a wide margin.
            fin = np.isfinite(ost.score)
            dev_rel = np.max(np.abs(host(st.score)[fin] - ost.score[fin]) / np.abs(ost.score[fin]))
            assert select_margin(ost.score, c.counts()) > 10 * dev_rel
        run_gpu(c, m, sched, st, [i], sigma)
        O.sample(om, osched, ost, sigma, iters=[i])
        np.testing.assert_array_equal(st.group.cpu().numpy(), ost.group)
        assert rel_l2(host(st.x), ost.x) < TOL_F32
        assert rel_l2(host(st.v_hat), ost.v_hat) < TOL_F32
        fin = np.isfinite(ost.score)
        np.testing.assert_array_equal(np.isfinite(host(st.score)), fin)
        if fin.any():
            assert rel_l2(host(st.score)[fin], ost.score[fin]) < TOL_F32
        assert rel_l2(host(m.blocks[0]["k_cache"]), ost.k_cache[0]) < TOL_F32


def test_step_full_budget_is_dense_euler_f32():
    c = synth.CONFIGS[1].with_(budgets=(8, 8))
    om = oracle_model(c)
    m = device_model(c, om)
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    st = H.DeviceState(m.dims, dev(synth.x0(c)), dev(synth.group0(c), torch.uint8))
    run_gpu(c, m, sched, st, range(c.T), sigma)
    assert rel_l2(host(st.x), O.dense_euler_sample(om, synth.x0(c), sigma, c.T)) < TOL_F32


def test_step_constant_velocity_closed_form():
    c = synth.CONFIGS[1]
    om = oracle_model(c)
    m = device_model(c, om)
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    v = np.random.default_rng(4).standard_normal((c.N, c.C)).astype(np.float32)
    st = H.DeviceState(m.dims, dev(synth.x0(c)), dev(synth.group0(c), torch.uint8))
    run_gpu(c, m, sched, st, range(c.T), sigma, field=lambda i: v)
    expect = synth.x0(c).astype(np.float64) + (float(sigma[-1]) - float(sigma[0])) * v
    np.testing.assert_allclose(host(st.x), expect, rtol=0, atol=1e-5)


@pytest.mark.parametrize("i,regroup,Dh", [(10, True, 128), (11, False, 128), (12, False, 128),
                                          (10, True, 64)])
def test_step_mid_run_bf16(i, regroup, Dh):
    """One iteration from a synthetic mid-run state (caches, v_hat, scores, groups)."""
    c = small_bf16(Dh=Dh, H=256 // Dh)
    say(f"hsa_step mid-run bf16 i={i} Dh={Dh}")
    om = oracle_model(c)
    s0 = synth.mid_run_state(c)
    m = device_model(c, om, s0["k_cache"], s0["v_cache"])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    st = H.DeviceState(m.dims, dev(s0["x"]), dev(s0["group"], torch.uint8), dev(s0["v_hat"]),
                       dev(s0["score"]))
    H.hsa_step(m, sched, st, i, float(sigma[i]), float(sigma[i + 1]), regroup)
    torch.cuda.synchronize()
    ost = O.State(s0["x"].astype(np.float64), s0["v_hat"].astype(np.float64),
                  s0["score"].astype(np.float64), s0["group"].copy(),
                  s0["k_cache"].astype(np.float64), s0["v_cache"].astype(np.float64))
    osched = O.Schedule(c.T, list(c.budgets), c.counts())
    out = O.hsa_iteration(om, osched, ost, i, sigma[i], sigma[i + 1], regroup)
    np.testing.assert_array_equal(st.group.cpu().numpy(), ost.group)
    nA = out["active_idx"].size
    np.testing.assert_array_equal(st.active_idx[:nA].cpu().numpy(), out["active_idx"])
    np.testing.assert_array_equal(st.pos.cpu().numpy(), out["pos"])
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
        kg = host(m.blocks[l]["k_cache"])
        np.testing.assert_array_equal(kg[skipped], s0["k_cache"][l][skipped])
        assert_rows_close(kg[a], ost.k_cache[l][a], TOL_BF16, f"layer {l} K rows")
    # skipped tokens advance with their cached velocity, bit-for-bit as an FMA
    ds = np.float32(np.float32(sigma[i + 1]) - np.float32(sigma[i]))
    xs = (s0["x"][skipped].astype(np.float64) + np.float64(ds) * s0["v_hat"][skipped]).astype(np.float32)
    np.testing.assert_array_equal(host(st.x)[skipped].astype(np.float32), xs)


@pytest.mark.timeout(400)     # the oracle's side takes about a minute of host time
def test_step_full_size_iteration():
    """Wan-1.3B shapes (N 32760, D 1536, F 8960), 2 blocks, 25%-active iteration
    from a synthetic mid-run state.  Exact properties that hold at any size
    (active set, untouched skipped rows, skipped-token Euler), then the
    velocity against the oracle: layer 0 over all 8190 active rows (their
    outputs feed layer 1's fresh K/V), every active row's K/V in both layers,
    layer 1 + unembed + Euler on 64 sampled active rows; v_hat, x and score of
    those tokens and every compared row within the bf16 tolerance."""
    c = synth.CONFIGS[3].with_(L=2)
    say("hsa_step full-size iteration")
    i = 11
    om = oracle_model(c)
    s0 = synth.mid_run_state(c)
    m = device_model(c, om, s0["k_cache"], s0["v_cache"])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    st = H.DeviceState(m.dims, dev(s0["x"]), dev(s0["group"], torch.uint8), dev(s0["v_hat"]),
                       dev(s0["score"]))
    H.hsa_step(m, sched, st, i, float(sigma[i]), float(sigma[i + 1]), False)
    torch.cuda.synchronize()
    idx, pos = O.active_set(s0["group"], c.budgets, c.T, i)
    assert idx.size == 8190
    np.testing.assert_array_equal(st.active_idx[:idx.size].cpu().numpy(), idx)
    np.testing.assert_array_equal(st.pos.cpu().numpy(), pos)
    skipped = np.setdiff1d(np.arange(c.N), idx)
    np.testing.assert_array_equal(host(st.v_hat)[skipped], s0["v_hat"][skipped])
    np.testing.assert_array_equal(host(st.score)[skipped], s0["score"][skipped])
    ds = np.float32(np.float32(sigma[i + 1]) - np.float32(sigma[i]))
    xs = (s0["x"][skipped].astype(np.float64) + np.float64(ds) * s0["v_hat"][skipped]).astype(np.float32)
    np.testing.assert_array_equal(host(st.x)[skipped].astype(np.float32), xs)
    kg = [host(m.blocks[l]["k_cache"]) for l in range(c.L)]
    vg = [host(m.blocks[l]["v_cache"]) for l in range(c.L)]
    for l in range(c.L):
        np.testing.assert_array_equal(kg[l][skipped], s0["k_cache"][l][skipped])
        np.testing.assert_array_equal(vg[l][skipped], s0["v_cache"][l][skipped])
    # the oracle through the whole iteration
    say("oracle: layer 0 over all active rows")
    kc = [s0["k_cache"][l].astype(np.float64) for l in range(c.L)]
    vc = [s0["v_cache"][l].astype(np.float64) for l in range(c.L)]
    h1 = oracle_block_all_rows(O, om, 0, O.embed(om, s0["x"], idx), idx, kc[0], vc[0])
    rows = np.sort(np.random.default_rng(3).choice(idx.size, 64, replace=False))
    h2 = O.block_forward(om, 1, h1, idx, kc[1], vc[1], rows=rows)
    tok = idx[rows]
    x_ref, vh_ref, sc_ref = O.euler_update(s0["x"][tok], s0["v_hat"][tok], s0["score"][tok],
                                           O.unembed(om, h2), np.arange(rows.size), ds, update_score=True)
    for l in range(c.L):
        assert_rows_close(kg[l][idx], kc[l][idx], TOL_BF16, f"layer {l} K rows")
        assert_rows_close(vg[l][idx], vc[l][idx], TOL_BF16, f"layer {l} V rows")
    e_v = assert_rows_close(host(st.v_hat)[tok], vh_ref, TOL_BF16, "v_hat")
    e_x = assert_rows_close(host(st.x)[tok], x_ref, TOL_BF16, "x")
    e_s = assert_rows_close(host(st.score)[tok][:, None], sc_ref[:, None], TOL_BF16, "score")
    say(f"sampled tokens: v_hat {e_v}, x {e_x}, score {e_s} (whole, worst row)")
    # active tokens advance with their fresh velocity
    np.testing.assert_allclose(host(st.x)[idx], s0["x"][idx] + float(ds) * host(st.v_hat)[idx],
                               rtol=1e-5, atol=1e-6)


def test_zero_row_calls_are_no_ops():
    """|A_i| = 0 reaches every row-wise entry point as zero rows: each returns
    success and writes nothing."""
    D = 256
    sentinel = torch.full((4, D), 7.0, dtype=torch.bfloat16, device=DEV)
    q = torch.zeros(0, D, dtype=torch.bfloat16, device=DEV)
    kv = torch.randn(100, D, device=DEV).to(torch.bfloat16)
    o = sentinel[:0]
    H.hsa_attn_active(q, kv, kv, o, 2, 128)
    w = torch.randn(D, D, device=DEV).to(torch.bfloat16)
    H.hsa_linear(q, w, sentinel[:0])
    H.hsa_layernorm(torch.zeros(0, D, device=DEV), sentinel[:0])
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)


def test_step_graph_capture_replays_match_eager():
    """hsa_step enqueues kernels only (no allocation, copy, memset or
    synchronisation), so a caller can capture one iteration in a HIP graph.
    Three replays from the same starting state, with other device work in
    between, each equal the eager iteration bit for bit (regroup included)."""
    c = small_bf16()
    i = 10
    say("hsa_step graph capture")
    om = oracle_model(c)
    s0 = synth.mid_run_state(c)
    m = device_model(c, om, s0["k_cache"], s0["v_cache"])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    st = H.DeviceState(m.dims, dev(s0["x"]), dev(s0["group"], torch.uint8), dev(s0["v_hat"]),
                       dev(s0["score"]))
    bufs = [st.x, st.v_hat, st.score, st.group] + [b[n] for b in m.blocks for n in ("k_cache", "v_cache")]
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
        other = other @ other.T / 512.0        # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            assert torch.equal(b, e), f"replay {rep} differs from the eager iteration"


def test_step_full_size_is_deterministic():
    """Two runs of the same full-size iteration (N 32760, D 1536, F 8960,
    2 blocks, regrouping on, the attention's KV range split and merged) from
    the same state give bit-identical latents, velocities, scores, groups and
    caches: no kernel on the path accumulates in a run-dependent order."""
    c = synth.CONFIGS[3].with_(L=2)
    say("hsa_step full-size determinism")
    i = 11
    om = oracle_model(c)
    s0 = synth.mid_run_state(c)
    m = device_model(c, om, s0["k_cache"], s0["v_cache"])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    st = H.DeviceState(m.dims, dev(s0["x"]), dev(s0["group"], torch.uint8), dev(s0["v_hat"]),
                       dev(s0["score"]))
    bufs = [st.x, st.v_hat, st.score, st.group] + [b[n] for b in m.blocks for n in ("k_cache", "v_cache")]
    init = [b.clone() for b in bufs]
    runs = []
    for _ in range(2):
        for b, v in zip(bufs, init):
            b.copy_(v)
        H.hsa_step(m, sched, st, i, float(sigma[i]), float(sigma[i + 1]), True)
        torch.cuda.synchronize()
        runs.append([b.clone() for b in bufs])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    assert not torch.equal(runs[0][0], init[0])   # the iteration did move the latents
