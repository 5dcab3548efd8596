"""The element decode on the path that runs, bit for bit.

csa_sparse_attn over a single selected row must give exactly that row: with
one row the softmax weight is exp(0) = 1 and the sum of weights is 1, so by
the oracle's closed form (k = 1) out[h] is the decoded row.  With a one-hot
query (1.0 at dimension d of head h) and softmax scale 1 the logit is the
decoded value at d, and lse = logit + log(1) is that value exactly.  Together
these put every finite (E4M3 code, UE8M0 byte) pair and every finite FP16
code through the attention kernels' own decode: the codes' conversion on the
logit side and the P.V side, the block scale applied to the partial logits
and carried by the P.V weights.  (Rows with an infinite or NaN value give
NaN logits in the oracle as well, so they have no exact closed form.)

Full decode steps then run with every indexer and KV block at the extreme
scale bytes 0, 1, 2, 253 and 254, with the RoPE tail zeroed so the scaled
blocks set the output's magnitude, against the oracle to the usual bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gen
import gpu_util as gu
import pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import long_context_sparse_score_amd as m

    assert torch.cuda.is_available()
    return m


def _finite_e4m3_rows() -> np.ndarray:
    """One KV row per scale byte 0..254: the 448 non-RoPE slots cycle
    through every E4M3 code whose value at that scale is finite in fp32;
    RoPE zero."""
    vals = pins.lib_e4m3(np.arange(256))
    rows = np.zeros((255, 583), dtype=np.uint8)
    for s in range(255):
        dec = vals * 2.0 ** (s - 127)
        ok = np.nonzero(np.isfinite(dec) & (np.abs(dec) <= np.finfo(np.float32).max))[0]
        rows[s, :448] = ok[np.arange(448) % len(ok)].astype(np.uint8)
        rows[s, 576:583] = s
    return rows


def _finite_f16_rows() -> np.ndarray:
    """Every finite FP16 code, 64 per row in the RoPE tail (non-RoPE codes
    zero at scale byte 127)."""
    codes = np.arange(65536, dtype=np.uint32)
    codes = codes[((codes >> 10) & 31) != 31].astype("<u2")  # drop inf / NaN
    n = (len(codes) + 63) // 64
    tail = np.resize(codes, n * 64).reshape(n, 64)
    rows = np.zeros((n, 583), dtype=np.uint8)
    rows[:, 448:576] = tail.view(np.uint8).reshape(n, 128)
    rows[:, 576:583] = 127
    return rows


def _one_hot_calls(csa, rows, blocks):
    """For every row r and 64-dimension block c in `blocks`: csa_sparse_attn
    over sel = [r] with q[h] = e_{64c + h}, scale 1.  Returns out, lse."""
    dev = torch.device("cuda")
    kv = torch.from_numpy(rows).to(dev)
    ws = csa.alloc_workspace(0, 1, dev)
    eye = torch.zeros((len(blocks), 64, 512), dtype=torch.float32, device=dev)
    for i, c in enumerate(blocks):
        eye[i, torch.arange(64), 64 * c + torch.arange(64)] = 1.0
    sel = torch.arange(len(rows), dtype=torch.int32, device=dev)
    outs = torch.empty((len(rows), len(blocks), 64, 512), dtype=torch.float32, device=dev)
    lses = torch.empty((len(rows), len(blocks), 64), dtype=torch.float32, device=dev)
    for r in range(len(rows)):
        for i in range(len(blocks)):
            out, lse = csa.sparse_attn(kv, sel[r:r + 1], 1, eye[i], 1.0, ws=ws)
            outs[r, i] = out
            lses[r, i] = lse
    torch.cuda.synchronize()
    return outs.cpu().numpy(), lses.cpu().numpy()


def _check_exact(rows, blocks, outs, lses, orc):
    """Bit equality, except that a -0 value comes back as +0: the oracle's
    own attention forms 0 + 1 * v (and lse = logit + log(1)), which is +0 for
    v = -0 in IEEE arithmetic.  Reports every mismatch."""
    ref = orc.decode_kv(rows)
    assert np.all(np.isfinite(ref))
    ref = ref + np.float32(0.0)  # -0 -> +0
    bad_out, bad_lse = [], []
    for r in range(len(rows)):
        for i, c in enumerate(blocks):
            # P.V side: every head returns the whole decoded row
            got = outs[r, i] + np.float32(0.0)
            diff = np.nonzero((got.view(np.uint32) != ref[r][None, :].view(np.uint32)).any(axis=0))[0]
            if len(diff):
                bad_out.append((r, int(diff[0]), float(got[0, diff[0]]), float(ref[r, diff[0]]), len(diff)))
            # logit side: head h's lse is the decoded value at 64c + h
            want = ref[r, 64 * c:64 * c + 64]
            gl = lses[r, i] + np.float32(0.0)
            dl = np.nonzero(gl.view(np.uint32) != want.view(np.uint32))[0]
            if len(dl):
                bad_lse.append((r, int(64 * c + dl[0]), float(gl[dl[0]]), float(want[dl[0]]), len(dl)))
    msg = (f"out mismatches (row, first dim, got, want, count): {bad_out[:6]} ({len(bad_out)} rows); "
           f"lse mismatches (row, dim, got, want, count): {bad_lse[:6]} ({len(bad_lse)})")
    assert not bad_out and not bad_lse, msg


def test_single_row_attention_is_the_decoded_row_every_e4m3_code_and_scale(csa, orc):
    rows = _finite_e4m3_rows()
    blocks = list(range(8))
    outs, lses = _one_hot_calls(csa, rows, blocks)
    _check_exact(rows, blocks, outs, lses, orc)


def test_single_row_attention_every_finite_fp16_code(csa, orc):
    rows = _finite_f16_rows()
    blocks = [7]  # the RoPE dimensions 448..511
    outs, lses = _one_hot_calls(csa, rows, blocks)
    _check_exact(rows, blocks, outs, lses, orc)


@pytest.mark.parametrize("sbyte", [0, 1, 2, 253, 254])
def test_decode_step_extreme_scale_bytes(csa, orc, sbyte):
    """Every block of every row at scale byte `sbyte`.  Codes stay finite
    after scaling (at 253/254: E2M1 magnitudes <= 1, E4M3 subnormal codes);
    queries, head weights and the softmax scale are scaled by exact powers of
    two so that dot products, scores and logits stay in fp32's normal range
    while the decoded values sit at the ends of theirs."""
    n = 3000
    s = gen.session(1, n_rows=n)
    rng = np.random.default_rng(sbyte)
    big = sbyte >= 253
    idx = s["idx_rows"]
    if big:
        mag = rng.choice(np.array([0, 1, 2, 8, 9, 10], np.uint8), size=(n, 128))
        idx[:, :64] = mag[:, 0::2] | (mag[:, 1::2] << 4)
    idx[:, 64:68] = sbyte
    kv = s["kv_rows"]
    if big:
        kv[:, :448] = rng.integers(0, 8, size=(n, 448), dtype=np.uint8) | (rng.integers(0, 2, size=(n, 448),
                                                                                        dtype=np.uint8) << 7)
    kv[:, 448:576] = 0  # RoPE tail zero
    kv[:, 576:583] = sbyte
    qs, ws_, lg = (-30, -97, -8) if big else (30, 97, 0)
    s["q_idx"] = (s["q_idx"] * np.float32(2.0 ** qs)).astype(np.float32)
    s["w_idx"] = (s["w_idx"] * np.float32(2.0 ** ws_)).astype(np.float32)
    s["q_attn"] = (s["q_attn"] * np.float32(2.0 ** lg)).astype(np.float32)
    # logits O(1): |q . kv| is about 2^(s - 116 + lg) for the generator's
    # codes (about 128 N(0,1) at their stored scale) and 2^(s - 130 + lg) for
    # subnormal codes
    s["softmax_scale"] = float(np.float32(2.0 ** ((130 if big else 116) - sbyte - lg) / np.sqrt(512.0)))
    assert np.all(np.isfinite(orc.decode_kv(kv))) and np.all(np.isfinite(orc.decode_idx(idx)))
    print(f"extreme scale byte {sbyte}: n_rows={n}", flush=True)
    d = gu.to_dev(s)
    got = csa.decode_step([d], s["softmax_scale"])[0]
    torch.cuda.synchronize()
    got = {k: got[k].cpu().numpy() for k in ("sel", "sel_score", "out", "lse")}
    ref_scores = orc.score(idx, s["q_idx"], s["w_idx"])
    assert np.all(np.isfinite(ref_scores))
    ref_sel, ref_sel_score, _ = orc.topk(ref_scores, 512)
    info = gu.check_selection_exact(got["sel"], got["sel_score"], ref_sel, ref_sel_score, 512)
    att, lse = orc.attention(kv, got["sel"], s["q_attn"], s["softmax_scale"])
    assert np.max(np.abs(att)) > 0
    info["attn_rel_err"] = gu.check_attention(got["out"], att)
    assert np.allclose(got["lse"], lse, rtol=1e-5, atol=1e-5)
    print(f"  {info}, max|out| {np.max(np.abs(att)):.3e}")
