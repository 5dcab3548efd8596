"""Dense attention over every KV row (csa_dense_attn: the HCA layers' exact
score-split attention on the DS4X page, «What DS4X changes» and
«Optimization details») on the GPU against the oracle's dense attention.

Acceptance as for the selected-row attention: max |out - ref| <= 1e-3
max |ref| and lse within 1e-5, ref the oracle's fp64 attention over the
same rows.  Sizes cross the 32-row batches, the group boundaries (groups of
32 rows up to 8,192 rows, then of 64, 96, ... up to 512 rows), the 8,194 rows
of a ratio-128 layer at a 1M-token context and the largest accepted size.
"""
import numpy as np
import pytest
import torch

import gen
import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import long_context_sparse_score_amd as m

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


@pytest.fixture(scope="module")
def kv_big():
    s = gen.session(3, n_rows=1 << 17)  # the largest accepted size
    return s["kv_rows"], s["q_attn"], s["softmax_scale"]


def _check(csa, orc, rows, q, scale, heads_checked=None):
    out, lse = csa.dense_attn(torch.from_numpy(rows).cuda(), torch.from_numpy(q).cuda(), scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    hc = q.shape[0] if heads_checked is None else heads_checked
    ref_o, ref_l = orc.dense_attention(rows, q[:hc], scale)
    gu.check_attention(out[:hc], ref_o)
    if rows.shape[0]:
        assert np.allclose(lse[:hc], ref_l, rtol=1e-5, atol=1e-5)
    else:
        assert np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 100, 513, 2048, 8192, 8193, 8194, 20000])
def test_dense_attention_matches_oracle(csa, orc, kv_big, n):
    rows, q, scale = kv_big
    _check(csa, orc, np.ascontiguousarray(rows[:n]), q, scale)


@pytest.mark.parametrize("h", [1, 7, 20])
def test_dense_attention_head_counts(csa, orc, kv_big, h):
    rows, q, scale = kv_big
    _check(csa, orc, np.ascontiguousarray(rows[:3000]), np.ascontiguousarray(q[:h]), scale)


def test_dense_attention_largest_size(csa, orc, kv_big):
    # every head is computed; the oracle checks two of them (a head's output
    # depends on no other head)
    rows, q, scale = kv_big
    _check(csa, orc, rows, q, scale, heads_checked=2)


def test_dense_attention_rejects_oversized(csa):
    import ctypes

    fake = ctypes.c_void_p(4096)
    assert csa.lib.csa_dense_attn(fake, (1 << 17) + 1, fake, 64, 0.1, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert csa.lib.csa_dense_workspace_bytes((1 << 17) + 1) == 0
