"""GPU parity of each HIP kernel against the CPU oracle, through the C ABI.

Integer results (active set, groups, scatter positions) must match bit for
bit; floating results within relative L2 1e-4 (float32) or 2e-2 (bfloat16).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import hsa_oracle as O
from tests.gpu_common import DEV, TOL_BF16, TOL_F32, assert_rows_close, dev, host, rel_l2, say

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


# ---------------------------------------------------------------- active set

@pytest.mark.parametrize("N", [1, 255, 4096, 4097, 32760, 75600])
def test_active_set_bit_exact(N):
    say(f"active_set N={N}")
    rs = np.random.default_rng(N)
    T, budgets = 40, [40, 20, 10]
    group = rs.integers(0, 3, N).astype(np.uint8)
    counts = np.bincount(group, minlength=3).tolist()
    sched = H.make_schedule(T, budgets, counts)
    g = dev(group, torch.uint8)
    idx = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    pos = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    nd = torch.zeros(1, dtype=torch.int32, device=DEV)
    for i in [0, 1, 2, 3, 4, 39]:
        H.hsa_active_set(g, sched, i, idx, pos, nd)
        torch.cuda.synchronize()
        ref_idx, ref_pos = O.active_set(group, budgets, T, i)
        nA = H.hsa_n_active(sched, i)
        assert nA == ref_idx.size == int(nd.item())
        np.testing.assert_array_equal(idx[:nA].cpu().numpy(), ref_idx)
        np.testing.assert_array_equal(pos.cpu().numpy(), ref_pos)


def test_active_set_groups_inconsistent_with_counts_stay_in_bounds():
    """Groups that do not hold count[k] tokens (a caller error): the device
    count reports the real |A_i|, while active_idx is written up to the
    closed-form |A_i| that sizes the later launches (padded with token 0,
    surplus tokens marked skipped), so nothing downstream reads an unwritten
    or out-of-range index."""
    N, T, budgets = 5000, 40, [40, 20, 10]
    rs = np.random.default_rng(11)
    group = rs.integers(0, 3, N).astype(np.uint8)
    real = np.bincount(group, minlength=3)
    for delta in (+300, -300):                       # schedule claims more / fewer full-budget tokens
        counts = [int(real[0] + delta), int(real[1] - delta), int(real[2])]
        sched = H.make_schedule(T, budgets, counts)
        idx = torch.full((N,), -7, dtype=torch.int32, device=DEV)
        pos = torch.full((N,), -7, dtype=torch.int32, device=DEV)
        nd = torch.zeros(1, dtype=torch.int32, device=DEV)
        i = 1                                        # only group 0 is active at odd i
        H.hsa_active_set(dev(group, torch.uint8), sched, i, idx, pos, nd)
        torch.cuda.synchronize()
        expected = H.hsa_n_active(sched, i)
        ref_idx, _ = O.active_set(group, budgets, T, i)
        assert int(nd.item()) == ref_idx.size == real[0]
        got = idx[:expected].cpu().numpy()
        assert np.all((got >= 0) & (got < N))
        k = min(expected, ref_idx.size)
        np.testing.assert_array_equal(got[:k], ref_idx[:k])
        assert np.all(got[k:] == 0)
        p = pos.cpu().numpy()
        assert np.all((p >= -1) & (p < expected))
        np.testing.assert_array_equal(np.flatnonzero(p >= 0), ref_idx[:k])


def test_active_set_phase_window():
    N, T = 1000, 40
    rs = np.random.default_rng(5)
    group = rs.integers(0, 3, N).astype(np.uint8)
    counts = np.bincount(group, minlength=3).tolist()
    sched = H.make_schedule(T, [40, 20, 10], counts, m=3)
    g = dev(group, torch.uint8)
    idx = torch.zeros(N, dtype=torch.int32, device=DEV)
    pos = torch.zeros(N, dtype=torch.int32, device=DEV)
    nd = torch.zeros(1, dtype=torch.int32, device=DEV)
    for i in [0, 2, 3, 5, 36, 37, 39]:
        H.hsa_active_set(g, sched, i, idx, pos, nd)
        ref_idx, ref_pos = O.active_set(group, [40, 20, 10], T, i, m=3)
        assert int(nd.item()) == ref_idx.size == H.hsa_n_active(sched, i)
        np.testing.assert_array_equal(pos.cpu().numpy(), ref_pos)


# ---------------------------------------------------------------- selection

def _select_case(score, counts):
    s = dev(score, torch.float32)
    out = torch.full((score.size,), 255, dtype=torch.uint8, device=DEV)
    H.hsa_select(s, counts, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), O.select_groups(score, counts))


@pytest.mark.parametrize("N,K", [(1, 1), (10, 2), (1000, 3), (1000, 8), (32760, 3), (75600, 3), (4099, 5)])
def test_select_bit_exact(N, K):
    say(f"select N={N} K={K}")
    rs = np.random.default_rng(N * 10 + K)
    cuts = np.sort(rs.integers(0, N + 1, K - 1))
    counts = np.diff(np.concatenate([[0], cuts, [N]])).astype(int).tolist()
    # continuous scores
    _select_case(np.abs(rs.standard_normal(N)).astype(np.float32), counts)
    # heavy ties and special values across the boundaries
    s = (rs.integers(0, 4, N) * 0.5).astype(np.float32)
    sp = rs.choice(N, size=min(N, 7), replace=False)
    s[sp] = np.array([np.nan, np.inf, -0.0, 0.0, -1.0, np.inf, np.nan], np.float32)[: sp.size]
    _select_case(s, counts)
    # all equal
    _select_case(np.full(N, 0.25, np.float32), counts)


def test_select_golden_fixtures():
    import json, os
    for name in ("select_adversarial.json", "select_ties.json"):
        g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", name)))
        s = np.array([float(x) for x in g["score"]], np.float32)
        out = torch.zeros(s.size, dtype=torch.uint8, device=DEV)
        H.hsa_select(dev(s), g["counts"], out)
        assert out.cpu().tolist() == g["group"]


def test_select_zero_count_groups():
    rs = np.random.default_rng(11)
    N = 3000
    s = rs.standard_normal(N).astype(np.float32)
    for counts in ([0, 1000, 2000], [1000, 0, 2000], [1000, 2000, 0], [3000, 0, 0], [0, 0, 3000]):
        _select_case(s, counts)


def _select_batch_case(score, counts):
    s = dev(score, torch.float32)
    out = torch.full(score.shape, 255, dtype=torch.uint8, device=DEV)
    H.hsa_select_batch(s, counts, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(score.shape[0]):
        np.testing.assert_array_equal(got[b], O.select_groups(score[b], counts), err_msg=f"row {b}")


@pytest.mark.parametrize("B,N,K", [(1, 1, 2), (3, 10, 2), (5, 1001, 3), (4, 1000, 8), (2, 4099, 5),
                                   (3, 32760, 3), (2, 32768, 4), (2, 40000, 3), (6, 513, 1),
                                   (5, 1000, 2), (300, 1000, 3), (260, 2052, 2), (270, 1001, 3),
                                   (3, 32768, 3), (2, 4, 2)])
def test_select_batch_bit_exact(B, N, K):
    """Each row of a batch against the oracle's selection of that row: rows
    staged in LDS (N <= 32768) and read from memory (N = 40000), rows whose
    start is not 16- or 4-byte aligned (N odd), ties and special values.
    More rows than CUs (B = 260..300): a workgroup ranks several rows, each
    loaded while the previous one is ranked (straight into LDS when rows are
    16-byte aligned, N % 4 == 0; into registers otherwise)."""
    say(f"select batch B={B} N={N} K={K}")
    rs = np.random.default_rng(B * 100000 + N * 10 + K)
    cuts = np.sort(rs.integers(0, N + 1, K - 1))
    counts = np.diff(np.concatenate([[0], cuts, [N]])).astype(int).tolist()
    _select_batch_case(rs.standard_normal((B, N)).astype(np.float32), counts)
    s = (rs.integers(0, 4, (B, N)) * 0.5).astype(np.float32)
    for b in range(B):
        sp = rs.choice(N, size=min(N, 7), replace=False)
        s[b, sp] = np.array([np.nan, np.inf, -0.0, 0.0, -1.0, -np.inf, np.nan], np.float32)[: sp.size]
    _select_batch_case(s, counts)
    # one row constant (every token ties with every boundary key), one row sorted ascending
    s2 = rs.standard_normal((B, N)).astype(np.float32)
    s2[0] = 0.25
    if B > 1:
        s2[1] = np.sort(s2[1])
    _select_batch_case(s2, counts)


def _score_rows(kind, rs, B, N):
    """B rows of N scores of one distribution family (float32)."""
    if kind == "uniform":
        return rs.random((B, N)).astype(np.float32)
    if kind == "abs_normal":
        return np.abs(rs.standard_normal((B, N))).astype(np.float32)
    if kind == "lognormal_wide":        # keys spread over many exponents
        return np.exp(rs.standard_normal((B, N)) * 8).astype(np.float32)
    if kind == "signed":                # both signs: the key's top bit differs
        return rs.standard_normal((B, N)).astype(np.float32)
    if kind == "narrow":                # all keys share their top 20-odd bits
        return (1.0 + rs.random((B, N)) * 1e-4).astype(np.float32)
    if kind == "few_values":            # heavy ties at every boundary
        return rs.integers(0, 5, (B, N)).astype(np.float32)
    if kind == "denormals":             # values below float32's normal range, and zeros of both signs
        s = (rs.random((B, N)) * 1e-39).astype(np.float32)
        s[:, ::7] = -0.0
        s[:, 3::11] = 0.0
        return s
    if kind == "sorted":                # the bucket's keys in one chunk of the row
        return np.sort(rs.random((B, N)), axis=1).astype(np.float32)
    if kind == "signed_zeros":          # 60% zeros of either sign: a boundary falls among them
        s = rs.random((B, N)).astype(np.float32)
        m = rs.random((B, N))
        s[m < 0.3] = 0.0
        s[(m >= 0.3) & (m < 0.6)] = -0.0
        return s
    if kind == "specials":              # NaN, +-inf, +-0 mixed into normal scores
        s = rs.standard_normal((B, N)).astype(np.float32)
        m = rs.random((B, N))
        s[m < 0.05] = np.nan
        s[(m >= 0.05) & (m < 0.08)] = np.inf
        s[(m >= 0.08) & (m < 0.1)] = -np.inf
        s[(m >= 0.1) & (m < 0.12)] = -0.0
        return s
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["uniform", "abs_normal", "lognormal_wide", "signed", "narrow",
                                  "few_values", "denormals", "signed_zeros", "sorted", "specials"])
def test_select_batch_distributions(kind):
    """Score distributions that drive the digit passes differently (wide and
    narrow key ranges, heavy ties, special values, denormals, a boundary among
    zeros of both signs, sorted rows),
    300 rows (more than the CUs: a workgroup ranks several rows, loading the
    next while it ranks the current one) at an aligned and a ragged row
    length, two and three groups; every row against the oracle."""
    rs = np.random.default_rng(sum(ord(ch) for ch in kind))
    for N, counts in ((2048, [512, 512, 1024]), (1999, [1000, 999])):
        score = _score_rows(kind, rs, 300, N)
        say(f"select distributions {kind} N={N}")
        _select_batch_case(score, counts)


def test_select_batch_rows_independent_and_match_single():
    """Row b of a batch equals hsa_select on that row alone, and a row's
    groups do not depend on the other rows."""
    rs = np.random.default_rng(5)
    B, N, counts = 4, 32760, [8190, 8190, 16380]
    score = np.abs(rs.standard_normal((B, N))).astype(np.float32)
    out = torch.empty((B, N), dtype=torch.uint8, device=DEV)
    H.hsa_select_batch(dev(score), counts, out)
    single = torch.empty(N, dtype=torch.uint8, device=DEV)
    for b in range(B):
        H.hsa_select(dev(score[b]), counts, single)
        assert torch.equal(out[b], single)
    score2 = score.copy()
    score2[1:] = -score2[1:]
    H.hsa_select_batch(dev(score2), counts, out)
    np.testing.assert_array_equal(out[0].cpu().numpy(), O.select_groups(score[0], counts))


def test_select_batch_full_size_sampled_rows():
    """The bench's batch (8192 videos of 32760 tokens, counts 8190 / 8190 /
    16380): every row's group sizes are exact, and sampled rows match the
    oracle's selection bit for bit."""
    B, N, counts = 8192, 32760, [8190, 8190, 16380]
    g = torch.Generator(device=DEV)
    g.manual_seed(8192)
    score = torch.rand((B, N), generator=g, device=DEV)
    out = torch.empty((B, N), dtype=torch.uint8, device=DEV)
    H.hsa_select_batch(score, counts, out)
    sizes = torch.stack([(out == k).sum(dim=1) for k in range(3)], dim=1)
    assert torch.equal(sizes.cpu(), torch.tensor([counts] * B))
    for b in (0, 1, 4095, 8191):
        np.testing.assert_array_equal(out[b].cpu().numpy(), O.select_groups(score[b].cpu().numpy(), counts))


# ---------------------------------------------------------------- cached Euler

@pytest.mark.parametrize("N,C", [(1, 16), (333, 16), (32760, 16), (100, 8)])
def test_euler_matches_oracle(N, C):
    say(f"euler N={N} C={C}")
    rs = np.random.default_rng(N + C)
    x = rs.standard_normal((N, C)).astype(np.float32)
    vh = rs.standard_normal((N, C)).astype(np.float32)
    sc = np.abs(rs.standard_normal(N)).astype(np.float32)
    act = np.sort(rs.choice(N, size=max(1, N // 3), replace=False)).astype(np.int32)
    pos = np.full(N, -1, np.int32)
    pos[act] = np.arange(act.size)
    vn = rs.standard_normal((act.size, C)).astype(np.float32)
    ds = np.float32(-0.025)
    for upd in (False, True):
        tx, tv, ts = dev(x), dev(vh), dev(sc)
        H.hsa_euler(tx, tv, ts, dev(vn), dev(pos, torch.int32), float(ds), upd)
        rx, rv, rsc = O.euler_update(x, vh, sc, vn, act, ds, update_score=upd)
        np.testing.assert_allclose(host(tx), rx, rtol=1e-6, atol=1e-6)
        np.testing.assert_array_equal(host(tv), rv)
        np.testing.assert_allclose(host(ts), rsc, rtol=2e-6, atol=0)
        skipped = np.setdiff1d(np.arange(N), act)
        np.testing.assert_array_equal(host(tv)[skipped], vh[skipped])
        np.testing.assert_array_equal(host(ts)[skipped], sc[skipped])


def test_euler_sweep_size_sampled_tokens():
    """The Euler pass at the largest size the bench sweeps (24M tokens, 25%
    active, device-generated inputs): 4096 sampled tokens, active and
    skipped, against the oracle's update of those tokens; skipped tokens'
    v_hat and score untouched everywhere."""
    N, C = 24 << 20, 16
    g = torch.Generator(device=DEV)
    g.manual_seed(24)
    x = torch.randn((N, C), generator=g, device=DEV)
    vh = torch.randn((N, C), generator=g, device=DEV)
    sc = torch.rand((N,), generator=g, device=DEV)
    nA = N // 4
    act = torch.randperm(N, generator=g, device=DEV)[:nA].sort().values.to(torch.int32)
    pos = torch.full((N,), -1, dtype=torch.int32, device=DEV)
    pos[act.long()] = torch.arange(nA, dtype=torch.int32, device=DEV)
    vn = torch.randn((nA, C), generator=g, device=DEV)
    x0, vh0, sc0 = x.clone(), vh.clone(), sc.clone()
    ds = np.float32(-0.025)
    H.hsa_euler(x, vh, sc, vn, pos, float(ds), True)
    torch.cuda.synchronize()
    active = pos >= 0
    assert torch.equal(vh[~active], vh0[~active]) and torch.equal(sc[~active], sc0[~active])
    rs = np.random.default_rng(24)
    tok = np.sort(rs.choice(N, 4096, replace=False))
    t = torch.from_numpy(tok).to(DEV)
    p = pos[t].cpu().numpy()
    rows = np.flatnonzero(p >= 0)
    rx, rv, rsc = O.euler_update(x0[t].cpu().numpy(), vh0[t].cpu().numpy(), sc0[t].cpu().numpy(),
                                 vn[torch.from_numpy(p[rows]).to(DEV).long()].cpu().numpy(),
                                 rows.astype(np.int32), ds, update_score=True)
    np.testing.assert_allclose(x[t].cpu().numpy(), rx, rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(vh[t].cpu().numpy(), rv)
    np.testing.assert_allclose(sc[t].cpu().numpy(), rsc, rtol=2e-6, atol=0)


def test_euler_hand_values():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "euler_hand.json")))
    C = g["C"]
    x = np.repeat(np.array(g["x"], np.float32)[:, None], C, 1)
    vh = np.repeat(np.array(g["v_hat"], np.float32)[:, None], C, 1)
    vn = np.repeat(np.array(g["v_new"], np.float32)[:, None], C, 1)
    pos = np.full(3, -1, np.int32)
    pos[g["active"]] = np.arange(len(g["active"]))
    tx, tv, ts = dev(x), dev(vh), dev(np.array(g["score"], np.float32))
    H.hsa_euler(tx, tv, ts, dev(vn), dev(pos, torch.int32), g["dsigma"], True)
    np.testing.assert_array_equal(host(tx)[:, 0], g["expect_x"])
    np.testing.assert_array_equal(host(tv)[:, 0], g["expect_v_hat"])
    np.testing.assert_allclose(host(ts), g["expect_score"], rtol=1e-6)


# ---------------------------------------------------------------- row ops

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_layernorm_embed_unembed(dtype):
    rs = np.random.default_rng(3)
    rows, D, C, N = 301, 1536, 16, 1000
    h = (rs.standard_normal((rows, D)) * 2 + 0.5).astype(np.float32)
    out = torch.empty(rows, D, dtype=dtype, device=DEV)
    H.hsa_layernorm(dev(h), out)
    ref = O.layer_norm(h)
    tol = 1e-5 if dtype == torch.float32 else 4e-3
    assert rel_l2(host(out), ref) < tol
    # embed (gather of active latents)
    x = rs.standard_normal((N, C)).astype(np.float32)
    w_in = rs.standard_normal((D, C)).astype(np.float32) / 4
    if dtype == torch.bfloat16:
        w_in = bf(w_in)
    idx = np.sort(rs.choice(N, rows, replace=False)).astype(np.int32)
    th = torch.empty(rows, D, device=DEV)
    H.hsa_embed(dev(x), dev(idx, torch.int32), rows, dev(w_in, dtype), th)
    assert rel_l2(host(th), x[idx].astype(np.float64) @ w_in.T.astype(np.float64)) < 1e-6
    # unembed
    w_out = rs.standard_normal((C, D)).astype(np.float32) / 40
    if dtype == torch.bfloat16:
        w_out = bf(w_out)
    vn = torch.empty(rows, C, device=DEV)
    H.hsa_unembed(dev(h), dev(w_out, dtype), vn, rows)
    assert rel_l2(host(vn), O.layer_norm(h) @ w_out.T.astype(np.float64)) < 1e-5


@pytest.mark.parametrize("D", [128, 256, 512, 1024, 1280, 1536, 2048, 2304, 5120])
@pytest.mark.parametrize("rows", [1, 17, 8190])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_embed_unembed_widths(D, rows, dtype):
    """Gather + embed (weights held per thread across a block of rows) and
    final LayerNorm + unembed (on the fp32 matrix cores when D <= 1536 is a
    multiple of 256; weights in LDS as float32 for D = 2048; one pass with
    four rows per wavefront for wider multiples of 256; the two-pass kernel
    otherwise), C = 16, row counts that leave partial blocks, every row
    within tolerance."""
    rs = np.random.default_rng(D + rows)
    C, N = 16, max(2 * rows, 64)
    x = rs.standard_normal((N, C)).astype(np.float32)
    w_in = rs.standard_normal((D, C)).astype(np.float32) / 4
    w_out = rs.standard_normal((C, D)).astype(np.float32) * D ** -0.5
    if dtype == torch.bfloat16:
        w_in, w_out = bf(w_in), bf(w_out)
    idx = np.sort(rs.choice(N, rows, replace=False)).astype(np.int32)
    th = torch.full((rows + 1, D), 5.0, device=DEV)     # one sentinel row past the end
    H.hsa_embed(dev(x), dev(idx, torch.int32), rows, dev(w_in, dtype), th[:rows])
    assert_rows_close(host(th)[:rows], x[idx].astype(np.float64) @ w_in.T.astype(np.float64), 1e-6,
                      "embed rows")
    assert torch.all(th[rows] == 5.0)
    h = (rs.standard_normal((rows, D)) * 2 + 0.5).astype(np.float32)
    vn = torch.full((rows + 1, C), 5.0, device=DEV)
    H.hsa_unembed(dev(h), dev(w_out, dtype), vn[:rows], rows)
    assert_rows_close(host(vn)[:rows], O.layer_norm(h) @ w_out.T.astype(np.float64), 1e-5,
                      "unembed rows")
    assert torch.all(vn[rows] == 5.0)


@pytest.mark.parametrize("D", [128, 256, 1536, 2000, 5120])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_layernorm_widths(D, dtype):
    """Row held in registers (D a multiple of 256) and the two-pass kernel
    (other widths), against the oracle's LayerNorm."""
    rs = np.random.default_rng(D)
    rows = 37
    h = (rs.standard_normal((rows, D)) * 3 - 1.5).astype(np.float32)
    out = torch.empty(rows, D, dtype=dtype, device=DEV)
    H.hsa_layernorm(dev(h), out)
    tol = 1e-5 if dtype == torch.float32 else 4e-3
    assert rel_l2(host(out), O.layer_norm(h)) < tol


# ---------------------------------------------------------------- GEMMs

@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (100, 384, 192), (300, 256, 128), (257, 200, 64),
                                   (1000, 1536, 1536),
                                   # each tile shape the library picks, ragged in M and N:
                                   # 256x256 (4000 x 4000), 128x192 (2100 x 4000, 1100 x 4000),
                                   # 128x128 (1000 x 4000, short and long K), 128x64 with
                                   # long K (1030 x 300)
                                   (4000, 4000, 128), (2100, 4000, 128), (1100, 4000, 128),
                                   (1000, 4000, 128), (1000, 4000, 4160), (1030, 300, 4160)])
def test_linear_bf16(M, N, K):
    say(f"linear bf16 M={M} N={N} K={K}")
    rs = np.random.default_rng(M * 7 + N + K)
    a = bf(rs.standard_normal((M, K)))
    w = bf(rs.standard_normal((N, K)) / np.sqrt(K))
    ref = a.astype(np.float64) @ w.T.astype(np.float64)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    H.hsa_linear(dev(a, torch.bfloat16), dev(w, torch.bfloat16), out, act=0)
    assert rel_l2(host(out), ref) < 5e-3
    H.hsa_linear(dev(a, torch.bfloat16), dev(w, torch.bfloat16), out, act=1)
    assert rel_l2(host(out), O.gelu_tanh(ref)) < 5e-3
    h0 = rs.standard_normal((M, N)).astype(np.float32)
    th = dev(h0)
    H.hsa_linear_residual(dev(a, torch.bfloat16), dev(w, torch.bfloat16), th)
    assert rel_l2(host(th), h0 + ref) < 1e-5


def test_linear_bf16_random_shapes():
    """Seeded random GEMM shapes (ragged M and N, K a multiple of 64) through
    every tile shape the library may pick, with each fused epilogue."""
    rs = np.random.default_rng(2024)
    for case in range(10):
        M = int(rs.integers(1, 3000))
        N = 4 * int(rs.integers(1, 1300))
        K = 64 * int(rs.integers(1, 40))
        say(f"linear bf16 random M={M} N={N} K={K}")
        a = bf(rs.standard_normal((M, K)))
        w = bf(rs.standard_normal((N, K)) / np.sqrt(K))
        ref = a.astype(np.float64) @ w.T.astype(np.float64)
        out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        act = case % 2
        H.hsa_linear(dev(a, torch.bfloat16), dev(w, torch.bfloat16), out, act=act)
        assert rel_l2(host(out), O.gelu_tanh(ref) if act else ref) < 5e-3, (M, N, K, act)
        h0 = rs.standard_normal((M, N)).astype(np.float32)
        th = dev(h0)
        H.hsa_linear_residual(dev(a, torch.bfloat16), dev(w, torch.bfloat16), th)
        assert rel_l2(host(th), h0 + ref) < 1e-5, (M, N, K)


def test_attention_random_shapes():
    """Seeded random attention shapes (query count, cache rows and heads; the
    split plan and the partial last tile vary with them) against the oracle."""
    rs = np.random.default_rng(77)
    for _ in range(8):
        nA = int(rs.integers(1, 1500))
        nkv = int(rs.integers(1, 9000))
        Hh = int(rs.integers(1, 4))
        say(f"attention random nA={nA} nkv={nkv} H={Hh}")
        _attn_case(nA, nkv, Hh, 128, torch.bfloat16, TOL_BF16, seed=int(rs.integers(0, 1000)))


@pytest.mark.parametrize("M,N,K", [(1, 64, 4), (77, 384, 128), (256, 512, 512), (130, 100, 36)])
def test_linear_f32(M, N, K):
    rs = np.random.default_rng(M + N + K)
    a = rs.standard_normal((M, K)).astype(np.float32)
    w = (rs.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    ref = a.astype(np.float64) @ w.T.astype(np.float64)
    out = torch.empty(M, N, device=DEV)
    H.hsa_linear(dev(a), dev(w), out, act=0)
    assert rel_l2(host(out), ref) < 1e-6
    H.hsa_linear(dev(a), dev(w), out, act=1)
    assert rel_l2(host(out), O.gelu_tanh(ref)) < 1e-5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_qkv_scatter_positions(dtype):
    rs = np.random.default_rng(21)
    N, D, nA = 700, 256, 233
    a = rs.standard_normal((nA, D)).astype(np.float32)
    w = (rs.standard_normal((3 * D, D)) / 16).astype(np.float32)
    if dtype == torch.bfloat16:
        a, w = bf(a), bf(w)
    idx = np.sort(rs.choice(N, nA, replace=False)).astype(np.int32)
    sentinel = -1024.0  # exactly representable in bfloat16 and float32
    kc = torch.full((N, D), sentinel, dtype=dtype, device=DEV)
    vc = torch.full((N, D), sentinel, dtype=dtype, device=DEV)
    q = torch.empty(nA, D, dtype=dtype, device=DEV)
    H.hsa_qkv_scatter(dev(a, dtype), dev(idx, torch.int32), nA, dev(w, dtype), q, kc, vc)
    ref = a.astype(np.float64) @ w.T.astype(np.float64)
    k_h, v_h = host(kc), host(vc)
    touched = np.flatnonzero(np.any(k_h != sentinel, axis=1))
    np.testing.assert_array_equal(touched, idx)           # positions: bit-exact
    np.testing.assert_array_equal(np.flatnonzero(np.any(v_h != sentinel, axis=1)), idx)
    assert np.all(k_h[np.setdiff1d(np.arange(N), idx)] == sentinel)
    tol = 5e-3 if dtype == torch.bfloat16 else 1e-6
    assert rel_l2(host(q), ref[:, :D]) < tol
    assert rel_l2(k_h[idx], ref[:, D:2 * D]) < tol
    assert rel_l2(v_h[idx], ref[:, 2 * D:]) < tol


@pytest.mark.parametrize("dtype,N,D,nA", [(torch.bfloat16, 700, 256, 233), (torch.float32, 700, 256, 233),
                                           (torch.bfloat16, 32760, 1536, 8190)])
def test_qkv_scatter_gather_mode(dtype, N, D, nA):
    """gather=1 reads the active rows a[active_idx[j]] straight from the [N][D]
    per-token matrix: bit-identical to the compact call on those rows
    (ragged 233-row case and the Wan-1.3B stage shape), and against the oracle
    on sampled rows."""
    say(f"qkv gather {dtype} N={N} D={D} nA={nA}")
    rs = np.random.default_rng(22)
    w = (rs.standard_normal((3 * D, D)) / np.sqrt(D)).astype(np.float32)
    if dtype == torch.bfloat16:
        w = bf(w)
    idx = np.sort(rs.choice(N, nA, replace=False)).astype(np.int32)
    ta = torch.randn(N, D, device=DEV).to(dtype)            # the per-token matrix
    ti, tw = dev(idx, torch.int32), dev(w, dtype)
    out = []
    for gather in (False, True):
        kc = torch.zeros(N, D, dtype=dtype, device=DEV)
        vc = torch.zeros(N, D, dtype=dtype, device=DEV)
        q = torch.empty(nA, D, dtype=dtype, device=DEV)
        a = ta if gather else ta[ti.long()].contiguous()
        H.hsa_qkv_scatter(a, ti, nA, tw, q, kc, vc, gather=gather)
        torch.cuda.synchronize()
        out.append((q, kc, vc))
    for x, y in zip(out[0], out[1]):
        assert torch.equal(x, y), "gathered rows differ from the compact call"
    rows = np.sort(rs.choice(nA, min(nA, 64), replace=False))
    ref = host(ta)[idx[rows]] @ w.astype(np.float64).T
    tol = 5e-3 if dtype == torch.bfloat16 else 1e-6
    q, kc, vc = out[1]
    assert rel_l2(host(q)[rows], ref[:, :D]) < tol
    assert rel_l2(host(kc)[idx[rows]], ref[:, D:2 * D]) < tol
    assert rel_l2(host(vc)[idx[rows]], ref[:, 2 * D:]) < tol


# ---------------------------------------------------------------- attention

def _attn_case(nA, nkv, Hh, Dh, dtype, tol, seed=0):
    rs = np.random.default_rng(seed + nA * 3 + nkv)
    q = rs.standard_normal((nA, Hh * Dh)).astype(np.float32)
    k = rs.standard_normal((nkv, Hh * Dh)).astype(np.float32)
    v = rs.standard_normal((nkv, Hh * Dh)).astype(np.float32)
    if dtype == torch.bfloat16:
        q, k, v = bf(q), bf(k), bf(v)
    o = torch.empty(nA, Hh * Dh, dtype=dtype, device=DEV)
    H.hsa_attn_active(dev(q, dtype), dev(k, dtype), dev(v, dtype), o, Hh, Dh)
    ref = O.attention(q, k, v, Hh, Dh)
    err = rel_l2(host(o), ref)
    assert err < tol, err
    return err


@pytest.mark.parametrize("Dh", [128, 64])
@pytest.mark.parametrize("nA,nkv", [(1, 1), (37, 63), (128, 64), (129, 65), (300, 1000), (64, 4097),
                                    (2, 20000), (700, 5000)])
def test_attention_bf16(nA, nkv, Dh):
    """The MFMA path at both head widths: ragged query and key counts, tails
    of one key, KV splits (long key ranges, few queries)."""
    say(f"attention bf16 Dh={Dh} nA={nA} nkv={nkv}")
    err = _attn_case(nA, nkv, 2 if Dh == 128 else 3, Dh, torch.bfloat16, TOL_BF16)
    assert err < 1e-2


@pytest.mark.parametrize("Dh", [128, 64])
def test_attention_bf16_whole_and_split_items(Dh):
    """More (query tile, head) items than one round of the chip: 24 heads x
    11 query tiles = 264 items, of which 256 run whole over the KV range and
    the last 8 (head 23, query tiles 3..10) in KV parts merged afterwards.
    Sampled rows against the oracle; every sampled row past query 768 takes
    head 23 from merged partials and the other heads from whole items."""
    nA, nkv, Hh = 2816, 4096, 24
    say(f"attention bf16 whole + split items Dh={Dh}")
    rs = np.random.default_rng(41 + Dh)
    q, k, v = (bf(rs.standard_normal((n, Hh * Dh))) for n in (nA, nkv, nkv))
    o = torch.empty(nA, Hh * Dh, dtype=torch.bfloat16, device=DEV)
    H.hsa_attn_active(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), o, Hh, Dh)
    rows = np.concatenate([np.arange(0, 8), rs.choice(np.arange(768, nA), 40, replace=False), [nA - 1]])
    assert_rows_close(host(o)[rows], O.attention(q[rows], k, v, Hh, Dh), TOL_BF16, "attention rows")


@pytest.mark.parametrize("nA,nkv,Hh", [(256 * 256, 4096, 1), (256 * 256 + 1, 4096, 1),
                                       (256 * 255 + 1, 4096, 1), (256 * 512 + 300, 2048, 1)])
def test_attention_bf16_split_plan_edges(nA, nkv, Hh):
    """Edges of the whole/split plan with one head: exactly one round of 256
    query-tile items (nothing split), one item more (that item, a last tile
    holding a single query, split over the KV range), one round with a
    ragged last tile, and two rounds plus a ragged item.  Sampled rows
    (first, around the tile and round boundaries, last) against the oracle."""
    say(f"attention bf16 plan edges nA={nA} nkv={nkv}")
    Dh = 128
    rs = np.random.default_rng(nA + nkv)
    q, k, v = (bf(rs.standard_normal((n, Hh * Dh))) for n in (nA, nkv, nkv))
    o = torch.empty(nA, Hh * Dh, dtype=torch.bfloat16, device=DEV)
    H.hsa_attn_active(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), o, Hh, Dh)
    rows = np.unique(np.clip(np.array([0, 1, 255, 256, 65535, 65536, nA - 2, nA - 1]), 0, nA - 1))
    assert_rows_close(host(o)[rows], O.attention(q[rows], k, v, Hh, Dh), TOL_BF16, "attention rows")


@pytest.mark.parametrize("nA,nkv,Dh", [(1, 1, 64), (77, 256, 64), (256, 256, 64), (50, 300, 128)])
def test_attention_f32(nA, nkv, Dh):
    _attn_case(nA, nkv, 2, Dh, torch.float32, 1e-5)


@pytest.mark.parametrize("Dh", [128, 64])
def test_attention_closed_forms_bf16(Dh):
    # q = 0 -> mean of V rows; all V rows equal -> that row
    nkv, Hh = 3000, 2
    rs = np.random.default_rng(9)
    k = bf(rs.standard_normal((nkv, Hh * Dh)))
    v = bf(rs.standard_normal((nkv, Hh * Dh)))
    o = torch.empty(5, Hh * Dh, dtype=torch.bfloat16, device=DEV)
    H.hsa_attn_active(dev(np.zeros((5, Hh * Dh)), torch.bfloat16), dev(k, torch.bfloat16),
                      dev(v, torch.bfloat16), o, Hh, Dh)
    assert rel_l2(host(o), np.broadcast_to(v.astype(np.float64).mean(0), (5, Hh * Dh))) < 2e-2
    c = bf(rs.standard_normal(Hh * Dh))
    H.hsa_attn_active(dev(bf(rs.standard_normal((5, Hh * Dh))), torch.bfloat16), dev(k, torch.bfloat16),
                      dev(np.tile(c, (nkv, 1)), torch.bfloat16), o, Hh, Dh)
    np.testing.assert_allclose(host(o), np.broadcast_to(c, (5, Hh * Dh)), rtol=8e-3, atol=1e-6)


def _softmax_range_case(pattern, nA, nkv, Hh=2, Dh=128, seed=5):
    """Inputs whose score maxima move far from where the first keys put them."""
    rs = np.random.default_rng(seed)
    D = Hh * Dh
    q = rs.standard_normal((nA, D))
    k = rs.standard_normal((nkv, D))
    v = rs.standard_normal((nkv, D))
    u = rs.standard_normal(D)
    u /= np.linalg.norm(u)
    if pattern == "spike":
        # a few keys far past the first tile align with every query: scores
        # ~ 4 * 200 / 2 heads = 400 above the rest (about 50 in log2 units)
        q += 4.0 * u
        for j in (nkv // 2 + 7, nkv - 3):
            k[j] += 200.0 * u
    elif pattern == "ramp":
        # key norms grow 9x along the cache: the row max keeps rising
        k *= (1.0 + 8.0 * np.arange(nkv) / nkv)[:, None]
        q *= 3.0
    elif pattern == "negative":
        # every score ~ -1600 (about -200 in log2 units): exp2 of the raw
        # scores would underflow; the probabilities are relative to the max
        q += 8.0 * u
        k -= 400.0 * u
    return bf(q), bf(k), bf(v)


@pytest.mark.parametrize("Dh", [128, 64])
@pytest.mark.parametrize("pattern", ["spike", "ramp", "negative"])
@pytest.mark.parametrize("nA,nkv", [(70, 5000), (300, 2113), (1, 9000)])
def test_attention_softmax_reference_moves(pattern, nA, nkv, Dh):
    """The running max is taken from the first keys and raised only when a
    later tile's probabilities grow far above 1: spikes, ramps and uniformly
    very negative scores against the oracle (several KV splits included)."""
    say(f"attention softmax range Dh={Dh} {pattern} nA={nA} nkv={nkv}")
    Hh = 2
    q, k, v = _softmax_range_case(pattern, nA, nkv, Hh, Dh)
    o = torch.empty(nA, Hh * Dh, dtype=torch.bfloat16, device=DEV)
    H.hsa_attn_active(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), o, Hh, Dh)
    out = host(o)
    assert np.all(np.isfinite(out))
    assert rel_l2(out, O.attention(q, k, v, Hh, Dh)) < TOL_BF16


@pytest.mark.parametrize("frac", [0.25, 0.0625, 1.0])
def test_attention_full_size_sampled_rows(frac):
    """Wan-1.3B-shaped layer: N = 32760 cached rows, 12 heads x 128, the launch
    configuration of the timed path; 64 sampled query rows against the oracle."""
    c = synth.CONFIGS[2]
    nA = synth.n_active_for_fraction(c.N, frac)
    say(f"attention full-size nA={nA}")
    kc, vc = synth.kv_cache(c)
    rs = np.random.default_rng(77)
    q = bf(rs.standard_normal((nA, c.D)))
    o = torch.empty(nA, c.D, dtype=torch.bfloat16, device=DEV)
    H.hsa_attn_active(dev(q, torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16), o,
                      c.H, c.Dh)
    rows = np.sort(rs.choice(nA, 64, replace=False))
    ref = O.attention(q[rows], kc, vc, c.H, c.Dh)
    assert_rows_close(host(o)[rows], ref, TOL_BF16, "attention rows")


@pytest.mark.parametrize("frac", [0.25, 0.0625])
def test_attention_full_size_64_wide_heads(frac):
    """64-wide heads at the full token count: N = 32760 cached rows, 32 heads x
    64 (D = 2048, the head layout of LTX-style DiTs); 64 sampled query rows
    against the oracle."""
    c = synth.CONFIGS[2].with_(D=2048, H=32, Dh=64)
    nA = synth.n_active_for_fraction(c.N, frac)
    say(f"attention full-size Dh=64 nA={nA}")
    kc, vc = synth.kv_cache(c)
    rs = np.random.default_rng(78)
    q = bf(rs.standard_normal((nA, c.D)))
    o = torch.empty(nA, c.D, dtype=torch.bfloat16, device=DEV)
    H.hsa_attn_active(dev(q, torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16), o,
                      c.H, c.Dh)
    rows = np.sort(rs.choice(nA, 64, replace=False))
    ref = O.attention(q[rows], kc, vc, c.H, c.Dh)
    assert_rows_close(host(o)[rows], ref, TOL_BF16, "attention rows")
