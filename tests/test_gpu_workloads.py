"""GPU parity at the shapes of the larger workloads, through the C ABI:

* the Wan-14B-shaped stack: 40 heads x 128 (D 5120), MLP 13824, N = 75600
  cached rows, cross-attention to 512 text tokens on active rows only;
* the aggressive churn regime: budgets {40, 10, 5} at 12.5/37.5/50%, a
  synthetic velocity field replacing the model's velocity in the Euler /
  score / select path.

Outputs the oracle can compute one by one are checked on sampled rows;
integer results bit for bit; the regroup decision by validity of the ranking
(ties between equal-change background tokens are decided by rounding).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import hsa_oracle as O
from tests.gpu_common import DEV, TOL_BF16, assert_rows_close, dev, host, rel_l2, say

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


def bf(a):
    return synth.to_bf16_values(np.asarray(a, np.float32))


C4 = synth.CONFIGS[4]


def test_attention_14b_shape_sampled_rows():
    c = C4
    nA = c.counts()[0]   # 18900 = 25% of 75600
    say(f"attention 14B shape nA={nA} N={c.N}")
    kc, vc = synth.kv_cache(c)
    rs = np.random.default_rng(41)
    q = bf(rs.standard_normal((nA, c.D)))
    o = torch.empty(nA, c.D, dtype=torch.bfloat16, device=DEV)
    H.hsa_attn_active(dev(q, torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16), o, c.H, c.Dh)
    torch.cuda.synchronize()
    rows = np.sort(rs.choice(nA, 24, replace=False))
    ref = O.attention(q[rows], kc, vc, c.H, c.Dh)
    assert_rows_close(host(o)[rows], ref, TOL_BF16, "attention rows")


def test_cross_attention_14b_shape():
    c = C4
    nA = c.counts()[0]
    say(f"cross-attention 14B shape nA={nA} n_text={c.n_text}")
    rs = np.random.default_rng(42)
    q = bf(rs.standard_normal((nA, c.D)))
    kt = bf(rs.standard_normal((c.n_text, c.D)))
    vt = bf(rs.standard_normal((c.n_text, c.D)))
    o = torch.empty(nA, c.D, dtype=torch.bfloat16, device=DEV)
    H.hsa_attn_active(dev(q, torch.bfloat16), dev(kt, torch.bfloat16), dev(vt, torch.bfloat16), o, c.H, c.Dh)
    torch.cuda.synchronize()
    rows = np.sort(rs.choice(nA, 64, replace=False))
    assert_rows_close(host(o)[rows], O.attention(q[rows], kt, vt, c.H, c.Dh), TOL_BF16, "attention rows")


def test_block_forward_14b_shape_with_cross_attention():
    """One 14B-shaped block (self-attention over N = 75600 cached rows, cross-
    attention to the 512 projected text tokens, MLP 13824) on 1024 active
    rows; every active row's K/V goes through the oracle, 24 sampled rows are
    checked through the whole block."""
    c = C4.with_(L=1)
    nA = 1024
    say(f"block_forward 14B shape nA={nA}")
    dims = O.Dims(N=c.N, C=c.C, D=c.D, H=c.H, Dh=c.Dh, F=c.F, L=1, bf16=True, n_text=c.n_text)
    w = synth.block_weights(c, 0)
    tx = synth.text_inputs(c)
    om = O.make_model(dims, synth.io_weights(c), [w], tx)
    kc, vc = synth.kv_cache(c)
    idx = synth.active_random(c, nA)
    h = synth.hidden_states(c, nA)
    dt = torch.bfloat16
    E = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
    H.hsa_linear(dev(tx["text"], dt), dev(tx["w_t"], dt), E)          # text embedding, once per run
    kt = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
    vt = torch.empty(c.n_text, c.D, dtype=dt, device=DEV)
    H.hsa_linear(E, dev(w["w_kx"], dt), kt)
    H.hsa_linear(E, dev(w["w_vx"], dt), vt)
    blk = {k: dev(w[k], dt) for k in ("w_qkv", "w_o", "w_1", "w_2", "w_qx", "w_ox")}
    blk.update(k_cache=dev(kc, dt), v_cache=dev(vc, dt), k_text=kt, v_text=vt)
    io = synth.io_weights(c)
    m = H.DeviceModel(H.make_dims(c.N, c.C, c.D, c.H, c.Dh, c.F, 1, c.n_text, dt),
                      dev(io["w_in"], dt), dev(io["w_out"], dt), [blk])
    ws = torch.empty(H.hsa_workspace_size(m.dims), dtype=torch.uint8, device=DEV)
    th = dev(h)
    H.hsa_block_forward(m, 0, th, dev(idx, torch.int32), nA, ws)
    torch.cuda.synchronize()
    # the projected text K/V agree with the oracle's once-per-run projection
    assert rel_l2(host(kt), om.blocks[0]["k_text"]) < 5e-3
    rows = np.sort(np.random.default_rng(7).choice(nA, 24, replace=False))
    ref = O.block_forward(om, 0, h, idx, kc, vc, rows=rows)     # caches updated in place
    assert_rows_close(host(th)[rows], ref, TOL_BF16, "block output rows")
    k_gpu = host(m.blocks[0]["k_cache"])
    assert_rows_close(k_gpu[idx], kc[idx], TOL_BF16, "K rows")
    assert_rows_close(host(m.blocks[0]["v_cache"])[idx], vc[idx], TOL_BF16, "V rows")
    skipped = np.setdiff1d(np.arange(c.N), idx)[::97]
    np.testing.assert_array_equal(k_gpu[skipped], kc[skipped])


def test_churn_regime_euler_score_select():
    """Aggressive regime on the Wan-1.3B block: T = 40, budgets {40, 10, 5};
    the churn field replaces v_new.  Iterations 0..9 run through hsa_step (the
    model runs, its velocity is replaced) and match the oracle's sampler
    state; at iteration 10 the regroup must form a valid ranking of the
    scores, which match the oracle's."""
    c = synth.CONFIGS[5]
    say("churn regime T=40 budgets 40/10/5")
    field = synth.ChurnField(c)
    dt = torch.bfloat16
    io = synth.io_weights(c)
    w = synth.block_weights(c, 0)
    blk = {k: dev(w[k], dt) for k in ("w_qkv", "w_o", "w_1", "w_2")}
    blk.update(k_cache=torch.zeros(c.N, c.D, dtype=dt, device=DEV),
               v_cache=torch.zeros(c.N, c.D, dtype=dt, device=DEV))
    m = H.DeviceModel(H.make_dims(c.N, c.C, c.D, c.H, c.Dh, c.F, 1, 0, dt), dev(io["w_in"], dt),
                      dev(io["w_out"], dt), [blk])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    osched = O.Schedule(c.T, list(c.budgets), c.counts())
    sigma = synth.sigma_schedule(c.T)
    x0, g0 = synth.x0(c), synth.group0(c)
    st = H.DeviceState(m.dims, dev(x0), dev(g0, torch.uint8))
    ost = O.State(x0.astype(np.float64), np.zeros((c.N, c.C)), np.full(c.N, np.inf), g0.copy(),
                  np.zeros((0,)), np.zeros((0,)))
    for i in range(11):
        regroup = i == 10
        vf = field(i)
        if regroup:
            s_gpu = host(st.score).astype(np.float32)   # the scores the regroup ranks
        H.hsa_step(m, sched, st, i, float(sigma[i]), float(sigma[i + 1]), regroup, dev(vf))
        torch.cuda.synchronize()
        if regroup:
            g_gpu = st.group.cpu().numpy()
            # a valid ranking of the GPU's own scores: exact counts, ordered groups
            assert np.bincount(g_gpu, minlength=3).tolist() == c.counts()
            for k in range(2):
                a, b = s_gpu[g_gpu == k], s_gpu[g_gpu == k + 1]
                assert a.min() >= b.max()
            pre = ost.score.copy()
        out = O.field_iteration(osched, ost, i, sigma[i], sigma[i + 1], regroup, vf)
        if regroup:
            fin = np.isfinite(pre)
            assert rel_l2(s_gpu[fin], pre[fin]) < 1e-5
            # tokens whose score is clear of every boundary score by more than the
            # score tolerance are ranked the same on both sides: their group must match
            srt = np.sort(pre)[::-1]
            bounds = np.cumsum(c.counts())[:-1]
            t = srt[bounds]
            clear = np.all(np.abs(pre[:, None] - t[None, :]) > 1e-4 * np.abs(t[None, :]), axis=1)
            np.testing.assert_array_equal(g_gpu[clear], ost.group[clear])
            say(f"regroup: {clear.mean():.3f} of tokens clear of the boundaries, all agree; "
                f"overall agreement {np.mean(g_gpu == ost.group):.3f}")
        else:
            nA = out["active_idx"].size
            np.testing.assert_array_equal(st.active_idx[:nA].cpu().numpy(), out["active_idx"])
            np.testing.assert_array_equal(host(st.v_hat), ost.v_hat)
            assert rel_l2(host(st.x), ost.x) < 1e-6
            fin = np.isfinite(ost.score)
            np.testing.assert_array_equal(np.isfinite(host(st.score)), fin)
            if fin.any():
                assert rel_l2(host(st.score)[fin], ost.score[fin]) < 1e-5


def test_churn_regime_whole_sampling_run():
    """All 40 iterations of the aggressive regime (budgets {40, 10, 5}, churn
    field replacing v_new).  At each regroup (10, 20, 30) the GPU's grouping
    must be a valid ranking of its own scores and agree with the oracle on
    every token clear of a boundary; the oracle then adopts the GPU's groups
    (ties at a boundary may fall either way), so every other iteration is
    compared exactly: active sets bit for bit, v_hat exactly, x and scores
    to float32 rounding."""
    c = synth.CONFIGS[5]
    say("churn regime, 40 iterations")
    field = synth.ChurnField(c)
    dt = torch.bfloat16
    io = synth.io_weights(c)
    w = synth.block_weights(c, 0)
    blk = {k: dev(w[k], dt) for k in ("w_qkv", "w_o", "w_1", "w_2")}
    blk.update(k_cache=torch.zeros(c.N, c.D, dtype=dt, device=DEV),
               v_cache=torch.zeros(c.N, c.D, dtype=dt, device=DEV))
    m = H.DeviceModel(H.make_dims(c.N, c.C, c.D, c.H, c.Dh, c.F, 1, 0, dt), dev(io["w_in"], dt),
                      dev(io["w_out"], dt), [blk])
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    osched = O.Schedule(c.T, list(c.budgets), c.counts())
    sigma = synth.sigma_schedule(c.T)
    x0, g0 = synth.x0(c), synth.group0(c)
    st = H.DeviceState(m.dims, dev(x0), dev(g0, torch.uint8))
    ost = O.State(x0.astype(np.float64), np.zeros((c.N, c.C)), np.full(c.N, np.inf), g0.copy(),
                  np.zeros((0,)), np.zeros((0,)))
    bounds = np.cumsum(c.counts())[:-1]
    for i in range(c.T):
        regroup = i in c.regroup
        vf = field(i)
        H.hsa_step(m, sched, st, i, float(sigma[i]), float(sigma[i + 1]), regroup, dev(vf))
        torch.cuda.synchronize()
        pre = ost.score.copy()
        out = O.field_iteration(osched, ost, i, sigma[i], sigma[i + 1], regroup, vf)
        if regroup:
            g_gpu = st.group.cpu().numpy()
            assert np.bincount(g_gpu, minlength=len(c.counts())).tolist() == c.counts()
            srt = np.sort(pre)[::-1]
            t = srt[bounds]
            clear = np.all(np.abs(pre[:, None] - t[None, :]) > 1e-4 * np.abs(t[None, :]), axis=1)
            np.testing.assert_array_equal(g_gpu[clear], ost.group[clear])
            # continue from the GPU's grouping: redo the oracle's iteration with it
            ost.group = g_gpu.copy()
            ost.x[:] = xs_before
            ost.v_hat[:] = vh_before
            ost.score[:] = pre
            out = O.field_iteration(osched, ost, i, sigma[i], sigma[i + 1], False, vf)
        nA = out["active_idx"].size
        np.testing.assert_array_equal(st.active_idx[:nA].cpu().numpy(), out["active_idx"])
        np.testing.assert_array_equal(host(st.v_hat), ost.v_hat)
        assert rel_l2(host(st.x), ost.x) < 1e-6
        fin = np.isfinite(ost.score)
        np.testing.assert_array_equal(np.isfinite(host(st.score)), fin)
        if fin.any():
            assert rel_l2(host(st.score)[fin], ost.score[fin]) < 1e-5
        xs_before, vh_before = ost.x.copy(), ost.v_hat.copy()
