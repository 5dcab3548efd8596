"""csa_decode_step_noalloc (the static per-device workspace) against
csa_decode_step (a caller's workspace): the same kernels, so the results must
be bit-identical, on two calls in a row, the second with fewer rows.  Also the
host-side rejection of a step too large for the static array."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import gen
import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import long_context_sparse_score_amd as m

    assert torch.cuda.is_available()
    return m


def _step(csa, s, noalloc):
    d = gu.to_dev(s)
    st = csa.DecodeStep([d], s["softmax_scale"], noalloc=noalloc)
    st()
    torch.cuda.synchronize()
    return {k: st.sessions[0][k].cpu().numpy() for k in ("sel", "sel_score", "out", "lse")}


@pytest.mark.parametrize("sizes", [(300_000, 5_000), (1 << 20, 700)])
def test_noalloc_matches_workspace_entry_point(csa, orc, sizes):
    for n in sizes:  # the second call is smaller: stale scratch must not leak into it
        s = gen.session(1, n_rows=n)
        print(f"noalloc step n_rows={n}", flush=True)
        a = _step(csa, s, noalloc=True)
        b = _step(csa, s, noalloc=False)
        for k in a:
            assert a[k].tobytes() == b[k].tobytes(), f"n={n}: {k} differs"
        if n <= 5_000:  # and against the oracle, to the usual bar
            ref_scores = orc.score(s["idx_rows"], s["q_idx"], s["w_idx"])
            ref_sel, ref_sel_score, _ = orc.topk(ref_scores, 512)
            gu.check_selection_exact(a["sel"], a["sel_score"], ref_sel, ref_sel_score, min(512, n))
            att, _ = orc.attention(s["kv_rows"], a["sel"][:min(512, n)], s["q_attn"], s["softmax_scale"])
            gu.check_attention(a["out"], att)


def test_noalloc_rejects_oversized_steps(csa):
    fake = ctypes.c_void_p(4096)  # never dereferenced: the size check comes first
    sess = (csa.Session * 16)()
    for i in range(16):
        sess[i] = csa.Session(fake, fake, 1 << 20, fake, fake, fake, fake, None, fake, None)
    assert csa.workspace_bytes(1 << 20, 16) > csa.SCRATCH_BYTES
    assert csa.lib.csa_decode_step_noalloc(sess, 16, 64, 64, 0.1, None) == csa.EWORKSPACE
    assert csa.lib.csa_decode_step_noalloc(sess, 0, 64, 64, 0.1, None) == csa.EINVAL
    assert csa.workspace_bytes(1 << 20, 1) <= csa.SCRATCH_BYTES
