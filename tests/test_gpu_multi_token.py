"""Multi-token score/top-k over one history (csa_score_topk_multi; DS4X page,
«Packed prefill implementation»: batch score/top-k) on the GPU against the
oracle: every token's selection equals the oracle's exact top-k of its own
scores, rows and order, with the scores bit for bit."""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import long_context_sparse_score_amd as m

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


def _queries(T, H, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, 128)).astype(np.float32)
    w = rng.uniform(0.0, 1.0, (T, H)).astype(np.float32)
    return q, w


@pytest.mark.parametrize("n,T,H,k", [(0, 2, 8, 512), (300, 3, 8, 512), (5000, 4, 64, 512), (70001, 3, 64, 100),
                                     (262144, 8, 64, 512)])
def test_multi_token_matches_oracle(csa, orc, n, T, H, k):
    rows = gen.session(2, n_rows=n)["idx_rows"]
    q, w = _queries(T, H, n + T)
    sel, sel_score = csa.score_topk_multi(torch.from_numpy(rows).cuda(), torch.from_numpy(q).cuda(),
                                          torch.from_numpy(w).cuda(), k)
    torch.cuda.synchronize()
    sel, sel_score = sel.cpu().numpy(), sel_score.cpu().numpy()
    ref_sel, ref_score = orc.score_topk_multi(rows, q, w, k)
    assert np.array_equal(sel, ref_sel), [int(np.sum(sel[t] != ref_sel[t])) for t in range(T)]
    k_eff = min(k, n)
    assert np.array_equal(sel_score[:, :k_eff].view(np.uint32), ref_score[:, :k_eff].view(np.uint32))
    assert np.all(np.isneginf(sel_score[:, k_eff:]))


def test_multi_token_equals_single_token_calls(csa):
    s = gen.session(3)
    d = torch.from_numpy(s["idx_rows"]).cuda()
    q, w = _queries(4, 64, 9)
    sel, sel_score = csa.score_topk_multi(d, torch.from_numpy(q).cuda(), torch.from_numpy(w).cuda())
    for t in range(4):
        s1, sc1 = csa.topk(csa.score(d, torch.from_numpy(q[t]).cuda(), torch.from_numpy(w[t]).cuda()), 512)
        assert torch.equal(sel[t], s1) and torch.equal(sel_score[t].view(torch.int32), sc1.view(torch.int32))
