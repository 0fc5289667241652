"""Property tests of the oracle (hypothesis): each checks an oracle function
on generated small inputs against the definition written out a second,
independent way (plain Python loops over the definition in the HSA summary),
so a mistake in the vectorised oracle cannot hide behind its own formula.
CPU only."""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import hsa_oracle as O

SETTINGS = dict(max_examples=60, deadline=None)

# scores drawn from a small pool so that ties are common, with the special
# values the selection reading fixes (NaN as +inf, -0 as +0)
SCORE_POOL = [0.0, -0.0, 0.25, 0.5, 1.0, -1.0, 3.0, float("inf"), float("-inf"), float("nan")]


@st.composite
def scores_and_counts(draw):
    n = draw(st.integers(1, 40))
    score = draw(st.lists(st.sampled_from(SCORE_POOL), min_size=n, max_size=n))
    k = draw(st.integers(1, 5))
    cuts = sorted(draw(st.lists(st.integers(0, n), min_size=k - 1, max_size=k - 1)))
    counts = [b - a for a, b in zip([0] + cuts, cuts + [n])]
    return np.array(score, np.float32), counts


@settings(**SETTINGS)
@given(scores_and_counts())
def test_select_equals_rank_definition(args):
    """Dynamic selection (HSA summary 2.1): token n's rank is the number of
    tokens with a larger score plus the earlier tokens with an equal one; it
    joins the group whose cumulative count first exceeds that rank."""
    score, counts = args
    key = [math.inf if math.isnan(float(s)) else float(s) + 0.0 for s in score]   # -0 + 0 -> +0
    got = O.select_groups(score, counts)
    for n in range(len(key)):
        rank = sum(1 for m in range(len(key)) if key[m] > key[n] or (key[m] == key[n] and m < n))
        g, acc = 0, counts[0]
        while rank >= acc:
            g += 1
            acc += counts[g]
        assert got[n] == g


@st.composite
def schedules(draw):
    T = draw(st.sampled_from([4, 8, 12, 40]))
    divisors = [d for d in range(1, T + 1) if T % d == 0]
    k = draw(st.integers(1, 4))
    budgets = [T] + draw(st.lists(st.sampled_from(divisors), min_size=k - 1, max_size=k - 1))
    n = draw(st.integers(1, 30))
    group = np.array(draw(st.lists(st.integers(0, k - 1), min_size=n, max_size=n)), np.uint8)
    m = draw(st.integers(0, T // 2))
    # every iteration, with the phase window's edges drawn often
    edges = [j for j in (m - 1, m, T - m - 1, T - m) if 0 <= j < T]
    i = draw(st.one_of(st.integers(0, T - 1), st.sampled_from(edges))) if edges else draw(st.integers(0, T - 1))
    return T, budgets, group, i, m


@settings(**SETTINGS)
@given(schedules())
def test_active_set_equals_activity_rule(args):
    """Activity rule (HSA summary 2.1) and phase window (2.4): token n is
    active at i iff i lies in the first or last m iterations or the period
    T / s of its group divides i; the list is ascending, pos is its inverse,
    and |A_i| matches the closed form over the group sizes."""
    T, budgets, group, i, m = args
    idx, pos = O.active_set(group, budgets, T, i, m)
    want = [n for n in range(group.size)
            if i < m or i >= T - m or i % (T // budgets[int(group[n])]) == 0]
    assert idx.tolist() == want
    for n in range(group.size):
        assert pos[n] == (want.index(n) if n in want else -1)
    counts = [int((group == g).sum()) for g in range(len(budgets))]
    assert O.n_active_closed_form(counts, budgets, T, i, m) == len(want)


small_floats = st.floats(-2.0, 2.0, allow_nan=False, width=32)


@st.composite
def attention_inputs(draw):
    H = draw(st.integers(1, 2))
    Dh = draw(st.integers(1, 4))
    M = draw(st.integers(1, 3))
    Nk = draw(st.integers(1, 5))
    arr = lambda r, c: np.array(draw(st.lists(small_floats, min_size=r * c, max_size=r * c)),
                                np.float64).reshape(r, c)
    return H, Dh, arr(M, H * Dh), arr(Nk, H * Dh), arr(Nk, H * Dh)


@settings(**SETTINGS)
@given(attention_inputs())
def test_attention_equals_softmax_definition(args):
    """Active-query attention (HSA summary 2.2 items 3-4): for each query and
    head, the weights exp(q.k / sqrt(Dh)) over every key row, normalised,
    applied to the value rows; no mask and no max shift in this form."""
    H, Dh, q, k, v = args
    got = O.attention(q, k, v, H, Dh)
    for r in range(q.shape[0]):
        for h in range(H):
            cols = range(h * Dh, (h + 1) * Dh)
            w = [math.exp(sum(q[r, c] * k[j, c] for c in cols) / math.sqrt(Dh)) for j in range(k.shape[0])]
            z = sum(w)
            for c in cols:
                want = sum(w[j] * v[j, c] for j in range(k.shape[0])) / z
                assert abs(got[r, c] - want) <= 1e-12 * max(1.0, abs(want))


@st.composite
def euler_inputs(draw):
    N = draw(st.integers(1, 6))
    C = draw(st.integers(1, 3))
    arr = lambda r, c: np.array(draw(st.lists(small_floats, min_size=r * c, max_size=r * c)),
                                np.float32).reshape(r, c)
    x, vh = arr(N, C), arr(N, C)
    score = np.array(draw(st.lists(st.floats(0, 5, width=32), min_size=N, max_size=N)), np.float32)
    idx = np.array(sorted(draw(st.sets(st.integers(0, N - 1), max_size=N))), np.int32)
    vn = arr(idx.size, C)
    ds = draw(st.floats(-0.5, 0.0, width=32))
    upd = draw(st.booleans())
    return x, vh, score, vn, idx, ds, upd


@settings(**SETTINGS)
@given(euler_inputs())
def test_euler_equals_cached_update_definition(args):
    """Cached Euler step (HSA summary 2.3) with the L1 score (2.1): an active
    token's score becomes sum|v_new - v_hat| / (sum|v_hat| + eps) when scores
    are updated, its cached velocity becomes v_new; every token then moves by
    dsigma times its (fresh or cached) velocity."""
    x, vh, score, vn, idx, ds, upd = args
    gx, gv, gs = O.euler_update(x, vh, score, vn, idx, ds, upd)
    f32 = lambda a: float(np.float32(a))
    for n in range(x.shape[0]):
        act = list(idx).index(n) if n in idx else -1
        vel = [float(vn[act, c]) if act >= 0 else float(vh[n, c]) for c in range(x.shape[1])]
        s = float(score[n])
        if act >= 0 and upd:
            num = sum(abs(float(vn[act, c]) - float(vh[n, c])) for c in range(x.shape[1]))
            s = num / (sum(abs(float(vh[n, c])) for c in range(x.shape[1])) + O.SCORE_EPS)
        assert gs[n] == np.float32(f32(s)) or abs(gs[n] - s) <= 1e-6 * max(1.0, abs(s))
        for c in range(x.shape[1]):
            assert gv[n, c] == np.float32(vel[c])
            want = float(x[n, c]) + float(ds) * vel[c]
            assert abs(float(gx[n, c]) - want) <= 1e-6 * max(1.0, abs(want))
