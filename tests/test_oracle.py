"""Pins for the CPU oracle, independent of the oracle's own code.

Every check here ties an oracle function to something fixed outside it: a
hand-derived value from the pages' rules (tests/golden), a library routine that
computes the same textbook operation (torch on the CPU, float64), a closed form,
an invariant, or brute force on tiny inputs.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import synth
from oracle import hsa_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- activity rule

def test_activity_tables_golden():
    g = gold("activity_tables.json")
    for case in g["cases"]:
        T, budgets = case["T"], case["budgets"]
        for k, iters in enumerate(case["active_iters"]):
            group = np.array([k], dtype=np.uint8)
            got = [i for i in range(T) if O.active_mask(group, budgets, T, i)[0]]
            assert got == iters, (T, budgets, k)


def test_each_group_active_exactly_budget_times():
    # Static groups: a token of G_k runs exactly s_k of the T iterations.
    rs = np.random.default_rng(0)
    for T, budgets in [(8, [8, 4]), (40, [40, 20, 10]), (40, [40, 10, 5]), (12, [12, 6, 4, 3, 2, 1])]:
        group = rs.integers(0, len(budgets), 300).astype(np.uint8)
        runs = sum(O.active_mask(group, budgets, T, i).astype(int) for i in range(T))
        np.testing.assert_array_equal(runs, np.asarray(budgets)[group])


def test_active_set_list_and_inverse():
    rs = np.random.default_rng(1)
    group = rs.integers(0, 3, 1000).astype(np.uint8)
    for i in range(8):
        idx, pos = O.active_set(group, [40, 20, 10], 40, i)
        assert np.all(np.diff(idx) > 0)
        # brute force over tokens
        brute = [n for n in range(1000) if group[n] == 0 or (group[n] == 1 and i % 2 == 0)
                 or (group[n] == 2 and i % 4 == 0)]
        assert idx.tolist() == brute
        assert np.all(pos[idx] == np.arange(idx.size))
        assert np.all(pos[np.setdiff1d(np.arange(1000), idx)] == -1)
        counts = np.bincount(group, minlength=3)
        assert idx.size == O.n_active_closed_form(counts, [40, 20, 10], 40, i)


def test_n_active_closed_form_golden():
    g = gold("activity_tables.json")["n_active"]
    for i in range(g["T"]):
        assert O.n_active_closed_form(g["counts"], g["budgets"], g["T"], i) == g["by_i_mod_4"][str(i % 4)]


def test_phase_window():
    group = np.array([0, 1, 2] * 10, dtype=np.uint8)
    T, m = 40, 3
    for i in range(T):
        mask = O.active_mask(group, [40, 20, 10], T, i, m)
        if i < m or i >= T - m:
            assert mask.all()
        else:
            np.testing.assert_array_equal(mask, O.active_mask(group, [40, 20, 10], T, i, 0))


# ---------------------------------------------------------------- selection

def _scores(strs):
    return np.array([float(s) for s in strs], dtype=np.float32)


@pytest.mark.parametrize("name", ["select_adversarial.json", "select_ties.json"])
def test_select_golden(name):
    g = gold(name)
    got = O.select_groups(_scores(g["score"]), g["counts"])
    assert got.tolist() == g["group"]


def test_select_invariants_random():
    rs = np.random.default_rng(2)
    for trial in range(20):
        N = int(rs.integers(1, 400))
        K = int(rs.integers(1, 6))
        cuts = np.sort(rs.integers(0, N + 1, K - 1))
        counts = np.diff(np.concatenate([[0], cuts, [N]])).tolist()
        # few distinct values -> many ties across thresholds
        score = rs.integers(0, 7, N).astype(np.float32) * np.float32(0.25)
        g = O.select_groups(score, counts)
        assert np.bincount(g, minlength=K).tolist() == counts
        for k in range(K - 1):
            a, b = score[g == k], score[g == k + 1]
            if a.size and b.size:
                assert a.min() >= b.max()
                # equal scores split across the boundary: lower indices first
                tie = a.min()
                if b.max() == tie:
                    assert np.flatnonzero((g == k) & (score == tie)).max() < \
                        np.flatnonzero((g == k + 1) & (score == tie)).min()


def test_select_brute_force_rank():
    # rank(n) = #{m: s_m > s_n} + #{m < n: s_m == s_n}; group = which cut the rank falls in.
    rs = np.random.default_rng(3)
    N = 60
    score = rs.integers(0, 5, N).astype(np.float32)
    counts = [10, 20, 30]
    bounds = np.cumsum(counts)
    g = O.select_groups(score, counts)
    for n in range(N):
        rank = sum(1 for m in range(N) if score[m] > score[n] or (score[m] == score[n] and m < n))
        assert g[n] == int(np.searchsorted(bounds, rank, side="right"))


# ---------------------------------------------------------------- textbook pieces

def test_layer_norm_matches_torch():
    y = np.random.default_rng(4).standard_normal((7, 96)) * 3 + 1
    ref = Fnn.layer_norm(torch.from_numpy(y), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(y), ref, rtol=1e-12, atol=1e-12)


def test_gelu_matches_torch():
    u = np.linspace(-8, 8, 1001)
    ref = Fnn.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(u), ref, rtol=1e-12, atol=1e-14)


def test_bf16_rounding_matches_torch():
    rs = np.random.default_rng(5)
    a = np.concatenate([rs.standard_normal(5000) * 10 ** rs.uniform(-6, 6, 5000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0e-39, 65504.0]]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(a), ref)
    np.testing.assert_array_equal(synth.to_bf16_values(a).astype(np.float64), ref)


def test_attention_matches_torch_sdpa():
    rs = np.random.default_rng(6)
    H, Dh, M, Nk = 3, 16, 9, 37
    q, k, v = (rs.standard_normal((n, H * Dh)) for n in (M, Nk, Nk))
    got = O.attention(q, k, v, H, Dh)
    tq = torch.from_numpy(q).view(M, H, Dh).transpose(0, 1)
    tk = torch.from_numpy(k).view(Nk, H, Dh).transpose(0, 1)
    tv = torch.from_numpy(v).view(Nk, H, Dh).transpose(0, 1)
    ref = Fnn.scaled_dot_product_attention(tq, tk, tv).transpose(0, 1).reshape(M, H * Dh).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_attention_closed_forms():
    rs = np.random.default_rng(7)
    H, Dh, Nk = 2, 8, 50
    k, v = rs.standard_normal((Nk, H * Dh)), rs.standard_normal((Nk, H * Dh))
    # q = 0: uniform weights, output = mean of V rows
    o = O.attention(np.zeros((3, H * Dh)), k, v, H, Dh)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), rtol=1e-12)
    # all V rows equal c: output c
    c = rs.standard_normal(H * Dh)
    o = O.attention(rs.standard_normal((4, H * Dh)), k, np.tile(c, (Nk, 1)), H, Dh)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-12)
    # one dominant key: output its V row
    kk = np.zeros((Nk, H * Dh))
    kk[17] = 1.0
    q = np.full((1, H * Dh), 1e4)
    o = O.attention(q, kk, v, H, Dh)
    np.testing.assert_allclose(o[0], v[17], rtol=1e-12)
    # permuting K/V rows together leaves the output unchanged
    q = rs.standard_normal((5, H * Dh))
    perm = rs.permutation(Nk)
    np.testing.assert_allclose(O.attention(q, k[perm], v[perm], H, Dh), O.attention(q, k, v, H, Dh),
                               rtol=1e-12, atol=1e-13)
    # a single key/value row: output is that row
    np.testing.assert_allclose(O.attention(q, k[:1], v[:1], H, Dh), np.tile(v[0], (5, 1)), rtol=1e-12)


# ---------------------------------------------------------------- model definition vs torch

def _tiny_cfg(**kw):
    base = dict(grid=(2, 4, 4), C=4, D=32, H=2, Dh=16, F=64, L=2, dtype="f32", T=8,
                budgets=(8, 4), shares=(0.5, 0.5), regroup=(3,))
    base.update(kw)
    return synth.CONFIGS[1].with_(**base)


def _model(c):
    dims = O.Dims(N=c.N, C=c.C, D=c.D, H=c.H, Dh=c.Dh, F=c.F, L=c.L, bf16=(c.dtype == "bf16"),
                  n_text=c.n_text)
    blocks = [synth.block_weights(c, l) for l in range(c.L)]
    text = synth.text_inputs(c) if c.n_text else None
    return O.make_model(dims, synth.io_weights(c), blocks, text)


def _torch_dense_velocity(c, x):
    """The same DiT written with torch CPU float64 library ops."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    D, H, Dh = c.D, c.H, c.Dh
    io = synth.io_weights(c)
    h = Fnn.linear(t(x), t(io["w_in"]))

    def mha(q, k, v):
        M, Nk = q.shape[0], k.shape[0]
        o = Fnn.scaled_dot_product_attention(q.view(M, H, Dh).transpose(0, 1),
                                             k.view(Nk, H, Dh).transpose(0, 1),
                                             v.view(Nk, H, Dh).transpose(0, 1))
        return o.transpose(0, 1).reshape(M, D)

    E = None
    if c.n_text:
        tx = synth.text_inputs(c)
        E = Fnn.linear(t(tx["text"]), t(tx["w_t"]))
    for l in range(c.L):
        w = synth.block_weights(c, l)
        qkv = Fnn.linear(Fnn.layer_norm(h, (D,), eps=1e-6), t(w["w_qkv"]))
        h = h + Fnn.linear(mha(qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]), t(w["w_o"]))
        if c.n_text:
            qx = Fnn.linear(Fnn.layer_norm(h, (D,), eps=1e-6), t(w["w_qx"]))
            h = h + Fnn.linear(mha(qx, Fnn.linear(E, t(w["w_kx"])), Fnn.linear(E, t(w["w_vx"]))), t(w["w_ox"]))
        u = Fnn.gelu(Fnn.linear(Fnn.layer_norm(h, (D,), eps=1e-6), t(w["w_1"])), approximate="tanh")
        h = h + Fnn.linear(u, t(w["w_2"]))
    return Fnn.linear(Fnn.layer_norm(h, (D,), eps=1e-6), t(io["w_out"])).numpy()


@pytest.mark.parametrize("n_text", [0, 8])
def test_dense_velocity_matches_torch_model(n_text):
    c = _tiny_cfg(n_text=n_text, text_dim=24 if n_text else 0)
    m = _model(c)
    x = synth.x0(c)
    # float32 storage rounding on the oracle side: agreement to float32 precision
    np.testing.assert_allclose(O.dense_velocity(m, x), _torch_dense_velocity(c, x), rtol=1e-4, atol=1e-5)


def test_all_full_budget_reduces_to_dense_euler():
    # Every s_k = T: every token active every iteration; HSA must equal a plain Euler loop.
    c = _tiny_cfg(budgets=(8, 8), L=1)
    m = _model(c)
    sched = O.Schedule(T=8, budgets=[8, 8], counts=c.counts(), regroup=(3, 5))
    sigma = synth.sigma_schedule(8)
    st = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    O.sample(m, sched, st, sigma)
    ref = O.dense_euler_sample(m, synth.x0(c), sigma, 8)
    np.testing.assert_allclose(st.x, ref, rtol=1e-12, atol=1e-12)


def test_full_budget_oracle_matches_torch_euler():
    # Same invariant against the torch-written model: plain Euler with torch velocities.
    c = _tiny_cfg(budgets=(8, 8), L=1)
    m = _model(c)
    sched = O.Schedule(T=8, budgets=[8, 8], counts=c.counts())
    sigma = synth.sigma_schedule(8)
    st = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    O.sample(m, sched, st, sigma)
    x = synth.x0(c).astype(np.float64)
    for i in range(8):
        x = x + (float(sigma[i + 1]) - float(sigma[i])) * _torch_dense_velocity(c, x)
    np.testing.assert_allclose(st.x, x, rtol=1e-4, atol=1e-5)


# ---------------------------------------------------------------- cached Euler and score

def test_euler_hand_values():
    g = gold("euler_hand.json")
    C = g["C"]
    x = np.repeat(np.array(g["x"])[:, None], C, 1)
    vh = np.repeat(np.array(g["v_hat"])[:, None], C, 1)
    vn = np.repeat(np.array(g["v_new"])[:, None], C, 1)
    x2, vh2, s2 = O.euler_update(x, vh, np.array(g["score"]), vn, np.array(g["active"]),
                                 g["dsigma"], update_score=True)
    np.testing.assert_array_equal(x2[:, 0], g["expect_x"])
    np.testing.assert_array_equal(vh2[:, 0], g["expect_v_hat"])
    np.testing.assert_allclose(s2, g["expect_score"], rtol=1e-7)
    # no score update on the first iteration
    _, _, s3 = O.euler_update(x, vh, np.array(g["score"]), vn, np.array(g["active"]), g["dsigma"],
                              update_score=False)
    np.testing.assert_array_equal(s3, g["score"])


def test_constant_velocity_closed_form():
    # v(x) == v for every token and iteration: x_T = x_0 + (sigma_T - sigma_0) v under any grouping.
    c = _tiny_cfg(budgets=(8, 4), L=1)
    m = _model(c)
    sched = O.Schedule(T=8, budgets=[8, 4], counts=c.counts(), regroup=(3, 4, 5))
    sigma = synth.sigma_schedule(8)
    v = np.random.default_rng(8).standard_normal((c.N, c.C))
    st = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    O.sample(m, sched, st, sigma, field=lambda i: v)
    expect = synth.x0(c) + (float(sigma[8]) - float(sigma[0])) * v
    # telescoping sum of T float32-rounded steps
    np.testing.assert_allclose(st.x, expect, rtol=0, atol=8 * 4 * np.finfo(np.float32).eps * 8)


def test_skipped_tokens_advance_with_cached_velocity():
    c = _tiny_cfg(budgets=(8, 4), L=1)
    m = _model(c)
    sched = O.Schedule(T=8, budgets=[8, 4], counts=c.counts())
    sigma = synth.sigma_schedule(8)
    st = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    O.sample(m, sched, st, sigma, iters=[0])
    before = st.copy()
    out = O.hsa_iteration(m, sched, st, 1, sigma[1], sigma[2], regroup=False)
    skipped = np.setdiff1d(np.arange(c.N), out["active_idx"])
    assert skipped.size == c.counts()[1]
    ds = float(np.float32(sigma[2]) - np.float32(sigma[1]))
    np.testing.assert_array_equal(st.v_hat[skipped], before.v_hat[skipped])
    np.testing.assert_array_equal(st.score[skipped], before.score[skipped])
    np.testing.assert_allclose(st.x[skipped], before.x[skipped] + ds * before.v_hat[skipped], rtol=1e-6)
    # active tokens: fresh velocity, score = L1 relative change against the previous one
    a = out["active_idx"]
    np.testing.assert_array_equal(st.v_hat[a], out["v_new"])
    r = np.abs(out["v_new"] - before.v_hat[a]).sum(1) / (np.abs(before.v_hat[a]).sum(1) + 1e-6)
    np.testing.assert_allclose(st.score[a], r, rtol=1e-6)
    # caches of skipped tokens untouched, of active tokens rewritten
    np.testing.assert_array_equal(st.k_cache[:, skipped], before.k_cache[:, skipped])
    assert np.all(np.any(st.k_cache[:, a] != before.k_cache[:, a], axis=-1))


def test_empty_active_set_iteration():
    # A schedule whose full-budget group is empty: at odd i no group is active,
    # |A_i| = 0, and the iteration is the cached Euler step alone.
    c = _tiny_cfg(budgets=(8, 4, 2), shares=(0.0, 0.5, 0.5), L=1)
    assert c.counts()[0] == 0
    m = _model(c)
    sched = O.Schedule(T=8, budgets=[8, 4, 2], counts=c.counts())
    assert O.n_active_closed_form(c.counts(), [8, 4, 2], 8, 1) == 0
    sigma = synth.sigma_schedule(8)
    st = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    O.sample(m, sched, st, sigma, iters=[0])
    before = st.copy()
    out = O.hsa_iteration(m, sched, st, 1, sigma[1], sigma[2], regroup=False)
    assert out["active_idx"].size == 0
    ds = float(np.float32(sigma[2]) - np.float32(sigma[1]))
    np.testing.assert_array_equal(st.v_hat, before.v_hat)
    np.testing.assert_array_equal(st.score, before.score)
    np.testing.assert_array_equal(st.k_cache, before.k_cache)
    np.testing.assert_allclose(st.x, before.x + ds * before.v_hat, rtol=1e-6)


def test_cache_rows_hold_last_active_projection():
    # After each iteration, row n of layer l holds the K/V the token had at its last
    # active iteration; attention at i sees those stale rows for skipped tokens.
    c = _tiny_cfg(budgets=(8, 4, 2), shares=(0.25, 0.25, 0.5), L=2)
    m = _model(c)
    sched = O.Schedule(T=8, budgets=[8, 4, 2], counts=c.counts())
    sigma = synth.sigma_schedule(8)
    st = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    last_k = np.zeros_like(st.k_cache)
    for i in range(8):
        x_in = st.x.copy()
        idx, _ = O.active_set(st.group, sched.budgets, 8, i)
        # recompute this iteration's fresh K for the active rows, layer by layer, from scratch
        h = x_in[idx] @ m.w_in.T
        kc, vc = st.k_cache.copy(), st.v_cache.copy()
        for l in range(c.L):
            a = O.layer_norm(h)
            last_k[l][idx] = a @ m.blocks[l]["w_qkv"][c.D:2 * c.D].T
            h = O.block_forward(m, l, h, idx, kc[l], vc[l])
        O.hsa_iteration(m, sched, st, i, sigma[i], sigma[i + 1], regroup=False)
        np.testing.assert_allclose(st.k_cache, last_k, rtol=1e-5, atol=1e-6)


def _stale_block_case(seed=21):
    """A block with a partial active set over a cache whose skipped rows hold
    stale values unrelated to the current rows (KV-cache synchronisation,
    HSA summary section 2.2, items 2-3)."""
    c = _tiny_cfg(grid=(1, 4, 4), C=4, D=16, H=2, Dh=8, F=32, L=1)
    m = _model(c)
    rs = np.random.default_rng(seed)
    idx = np.array([1, 4, 6, 9, 13])
    h = rs.standard_normal((idx.size, c.D))
    k_cache = rs.standard_normal((c.N, c.D))
    v_cache = rs.standard_normal((c.N, c.D))
    return c, m, idx, h, k_cache, v_cache


def test_active_queries_attend_to_stale_rows_closed_form():
    # Active queries see every cached row: here one skipped token's stale key
    # dominates every active query's logits in every head, so the attention
    # output of each active row is that token's stale value row.  With W_o = I
    # and W_1 = 0 the block returns h + v_stale exactly (GELU(0) = 0), whatever
    # the fresh rows are.  Attending over the fresh rows alone gives their
    # values instead (all equal here), which this checks is not what happens.
    c, m, idx, _, k_cache, v_cache = _stale_block_case()
    D = c.D
    rs = np.random.default_rng(22)
    u = rs.standard_normal(D)
    # LayerNorm ignores scale and offset: every active row normalises to LN(u),
    # so all fresh q (and k, v) rows are equal.
    h = np.stack([(j + 1.5) * u + 0.25 * j for j in range(idx.size)])
    blk = m.blocks[0]
    blk["w_o"] = np.eye(D)
    blk["w_1"] = np.zeros_like(blk["w_1"])
    q = O.layer_norm(u[None, :]) @ blk["w_qkv"][:D].T
    stale = 11
    assert stale not in idx
    k_cache[:, :] = 0.0
    k_cache[stale] = 60.0 * q[0] / np.abs(q[0]).max() ** 2    # logit >= 60 / sqrt(Dh) per head
    v_stale = np.linspace(-2.0, 3.0, D)
    v_cache[stale] = v_stale
    out = O.block_forward(m, 0, h, idx, k_cache, v_cache)
    # every other logit is q.k_fresh (tiny next to the planted one) or 0
    np.testing.assert_allclose(out, h + v_stale[None, :], rtol=0, atol=1e-6)
    v_fresh = O.layer_norm(u[None, :]) @ blk["w_qkv"][2 * D:].T
    assert np.abs(out - (h + v_fresh)).max() > 0.5


def test_block_attention_over_stale_cache_matches_torch_sdpa():
    # Brute force with torch CPU float64 library ops: write the fresh K/V of the
    # active rows into a copy of the stale cache, then SDPA of the active
    # queries over all N rows, out-projection, MLP; compare the block's output.
    c, m, idx, h, k_cache, v_cache = _stale_block_case()
    D, H, Dh, N = c.D, c.H, c.Dh, c.N
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    w = m.blocks[0]
    ht = t(h)
    qkv = Fnn.linear(Fnn.layer_norm(ht, (D,), eps=1e-6), t(w["w_qkv"]))
    kc, vc = t(k_cache).clone(), t(v_cache).clone()
    kc[torch.from_numpy(idx)] = qkv[:, D:2 * D]
    vc[torch.from_numpy(idx)] = qkv[:, 2 * D:]
    M = idx.size
    o = Fnn.scaled_dot_product_attention(qkv[:, :D].view(M, H, Dh).transpose(0, 1),
                                         kc.view(N, H, Dh).transpose(0, 1),
                                         vc.view(N, H, Dh).transpose(0, 1))
    ht = ht + Fnn.linear(o.transpose(0, 1).reshape(M, D), t(w["w_o"]))
    u = Fnn.gelu(Fnn.linear(Fnn.layer_norm(ht, (D,), eps=1e-6), t(w["w_1"])), approximate="tanh")
    ref = (ht + Fnn.linear(u, t(w["w_2"]))).numpy()
    kc_o, vc_o = k_cache.copy(), v_cache.copy()
    out = O.block_forward(m, 0, h, idx, kc_o, vc_o)
    np.testing.assert_allclose(out, ref, rtol=1e-5, atol=1e-6)   # float32 storage on the oracle side
    np.testing.assert_allclose(kc_o, kc.numpy(), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(vc_o, vc.numpy(), rtol=1e-6, atol=1e-7)
    # the stale rows do move the result: attending over the fresh rows alone differs
    o_fresh = Fnn.scaled_dot_product_attention(qkv[:, :D].view(M, H, Dh).transpose(0, 1),
                                               qkv[:, D:2 * D].view(M, H, Dh).transpose(0, 1),
                                               qkv[:, 2 * D:].view(M, H, Dh).transpose(0, 1))
    assert (o_fresh - o).abs().max().item() > 0.1


def test_total_work_matches_budgets():
    # Over T iterations with static groups the number of token evaluations is sum_k n_k s_k:
    # attention work O(|A_i| N) summed over the run.
    c = synth.CONFIGS[3]
    counts = c.counts()
    total = sum(O.n_active_closed_form(counts, c.budgets, c.T, i) for i in range(c.T))
    assert total == sum(n * s for n, s in zip(counts, c.budgets))
    assert total / (c.N * c.T) == pytest.approx(0.5)
    c5 = synth.CONFIGS[5]
    t5 = sum(O.n_active_closed_form(c5.counts(), c5.budgets, c5.T, i) for i in range(c5.T))
    assert t5 / (c5.N * c5.T) == pytest.approx(0.28125)


def test_row_sampled_block_equals_full_block():
    c = _tiny_cfg(L=1)
    m = _model(c)
    rs = np.random.default_rng(9)
    idx = np.sort(rs.choice(c.N, 20, replace=False))
    h = rs.standard_normal((20, c.D))
    k0, v0 = rs.standard_normal((c.N, c.D)), rs.standard_normal((c.N, c.D))
    k1, v1 = k0.copy(), v0.copy()
    full = O.block_forward(m, 0, h, idx, k0, v0)
    rows = np.array([0, 7, 19])
    part = O.block_forward(m, 0, h, idx, k1, v1, rows=rows)
    np.testing.assert_array_equal(part, full[rows])
    np.testing.assert_array_equal(k0, k1)


def test_config_counts_exact():
    assert synth.CONFIGS[1].counts() == [128, 128]
    assert synth.CONFIGS[3].counts() == [8190, 8190, 16380]
    assert synth.CONFIGS[4].counts() == [18900, 18900, 37800]
    assert synth.CONFIGS[5].counts() == [4095, 12285, 16380]
    assert synth.n_active_for_fraction(32760, 0.0625) == 2048
    assert synth.n_active_for_fraction(32760, 0.05) == 1638


def test_field_iteration_matches_full_iteration_with_field():
    # With a velocity field in place of the model, the sampler state does not depend on the model.
    c = _tiny_cfg(budgets=(8, 4, 2), shares=(0.25, 0.25, 0.5), L=1)
    m = _model(c)
    sched = O.Schedule(T=8, budgets=[8, 4, 2], counts=c.counts(), regroup=(3, 5))
    sigma = synth.sigma_schedule(8)
    rs = np.random.default_rng(12)
    fields = [rs.standard_normal((c.N, c.C)) for _ in range(8)]
    a = O.init_state(m.dims, synth.x0(c), synth.group0(c))
    b = a.copy()
    for i in range(8):
        O.hsa_iteration(m, sched, a, i, sigma[i], sigma[i + 1], i in (3, 5), v_field=fields[i])
        O.field_iteration(sched, b, i, sigma[i], sigma[i + 1], i in (3, 5), fields[i])
        np.testing.assert_array_equal(a.x, b.x)
        np.testing.assert_array_equal(a.group, b.group)
        np.testing.assert_array_equal(a.score, b.score)


def test_churn_field_shape_and_blob():
    c = synth.CONFIGS[5]
    f = synth.ChurnField(c)
    blob = f.blob(3)
    assert blob.size == 21 * 234                      # 15% of 32760 tokens
    v3, v4 = f(3), f(4)
    bg = np.setdiff1d(np.arange(c.N), np.union1d(f.blob(3), f.blob(4)))
    # background changes by (1 + 0.002*4)/(1 + 0.002*3) - 1 ~ 0.2% per step
    r = np.abs(v4[bg] - v3[bg]).sum(1) / np.abs(v3[bg]).sum(1)
    np.testing.assert_allclose(r, 0.002 / 1.006, rtol=1e-4)
