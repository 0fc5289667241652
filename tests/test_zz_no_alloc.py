"""The allocation-free attention entry point (hsa_attn_active_noalloc) against
the entry point that takes a workspace (hsa_attn_active), through the C ABI:
two calls in a row on the Wan-1.3B-shaped layer (N = 32760 cached rows, 12
heads x 128), the second with fewer queries, each equal to hsa_attn_active
bit for bit and to the oracle on sampled rows; a call that needs more than
the fixed scratch is rejected before anything runs."""
import numpy as np
import pytest
import torch

import synth
from oracle import hsa_oracle as O
from tests.gpu_common import DEV, TOL_BF16, assert_rows_close, dev, host, say

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


def test_noalloc_attention_matches_workspace_entry_point():
    c = synth.CONFIGS[2]
    kc, vc = synth.kv_cache(c)
    k, v = dev(kc, torch.bfloat16), dev(vc, torch.bfloat16)
    rs = np.random.default_rng(91)
    for frac in (0.25, 0.05):     # 8190 then 1638 queries; both split the KV range
        nA = synth.n_active_for_fraction(c.N, frac)
        need = H.hsa_attn_workspace_size(nA, c.N, c.H, c.Dh)
        say(f"noalloc attention nA={nA} scratch {need} B")
        assert 0 < need <= H.NOALLOC_SCRATCH_BYTES
        q = synth.to_bf16_values(rs.standard_normal((nA, c.D)).astype(np.float32))
        tq = dev(q, torch.bfloat16)
        o_ws = torch.empty(nA, c.D, dtype=torch.bfloat16, device=DEV)
        o_na = torch.full((nA, c.D), 7.0, dtype=torch.bfloat16, device=DEV)
        H.hsa_attn_active(tq, k, v, o_ws, c.H, c.Dh)
        H.hsa_attn_active_noalloc(tq, k, v, o_na, c.H, c.Dh)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws)
        rows = np.sort(rs.choice(nA, 32, replace=False))
        assert_rows_close(host(o_na)[rows], O.attention(q[rows], kc, vc, c.H, c.Dh), TOL_BF16,
                          "attention rows")


def test_noalloc_attention_rejects_a_problem_past_its_scratch():
    # 200 heads x 128 over 75600 rows with 256 queries: every (query tile, head)
    # item is split 14 ways over the KV range, 180 MiB of partials.
    nA, nkv, Hh, Dh = 256, 75600, 200, 128
    assert H.hsa_attn_workspace_size(nA, nkv, Hh, Dh) > H.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(nA, Hh * Dh, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(nkv, Hh * Dh, dtype=torch.bfloat16, device=DEV)
    o = torch.full((nA, Hh * Dh), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(H.HsaError) as e:
        H.hsa_attn_active_noalloc(q, kv, kv, o, Hh, Dh)
    assert e.value.status == -8
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)      # nothing ran
