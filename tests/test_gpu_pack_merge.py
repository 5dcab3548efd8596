"""Packing new rows and merging attention results, on the GPU against the
oracle.

* csa_pack_rows writes new compressed / raw-ring rows in the 583-byte KV and
  68-byte indexer formats (DS4X page, «Packed cache ABI»); it must equal the
  oracle's packing byte for byte, over many binades, zero blocks, exact ties
  of both element grids, values that saturate, binary16 subnormals, signed
  zeros and overflow.
* csa_lse_merge joins two attention results over disjoint rows (the
  sliding-window ring and the selected compressed rows in one softmax): the
  decode step's attention merged with the dense attention over a 256-row
  ring equals the oracle's attention over the union of the rows (attention
  tolerance), and the merge itself equals the oracle's merge of the same
  inputs to fp32 rounding.
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


def _vals(rng, n, width):
    v = (rng.standard_normal((n, width)) * 2.0 ** rng.integers(-40, 40, (n, 1))).astype(np.float32)
    if n >= 8:
        v[0, :64] = 0.0                                                            # zero block
        v[1] = (rng.integers(-64, 65, width) * 0.0625).astype(np.float32)          # grid ties
        v[2] = (rng.integers(-16, 17, width) * 0.25).astype(np.float32)
        v[3] *= np.float32(2.0 ** -120)                                            # tiny blocks
        v[4, ::7] = np.float32(7.99) * v[4, ::7] / np.maximum(np.abs(v[4, ::7]), 1e-30)  # near the top of a binade
        v[5] = np.where(rng.random(width) < 0.5, -0.0, 0.0).astype(np.float32)     # signed zeros
    if width == 512 and n >= 8:
        v[6, 448:] = np.array([65504.0, 65519.0, 65520.0, -7e4, 2.0 ** -25, -3 * 2.0 ** -26, 6e-8, -0.0] * 8, np.float32)
        v[7, 448:] = (rng.standard_normal(64) * 1e-6).astype(np.float32)           # binary16 subnormals
    return v


@pytest.mark.parametrize("n", [1, 37, 1000])
def test_pack_matches_oracle(csa, orc, n):
    rng = np.random.default_rng(n)
    kv, idx = _vals(rng, n, 512), _vals(rng, n, 128)
    kr, ir = csa.pack_rows(torch.from_numpy(kv).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    kr, ir = kr.cpu().numpy(), ir.cpu().numpy()
    ref_k, ref_i = orc.pack_kv(kv), orc.pack_idx(idx)
    assert np.array_equal(kr, ref_k), np.argwhere(kr != ref_k)[:5]
    assert np.array_equal(ir, ref_i), np.argwhere(ir != ref_i)[:5]


def test_pack_one_format_and_in_place(csa, orc):
    rng = np.random.default_rng(3)
    kv = _vals(rng, 20, 512)
    cache = torch.zeros((50, 583), dtype=torch.uint8, device="cuda")
    csa.pack_rows(torch.from_numpy(kv).cuda(), None, kv_rows=cache[10:30])  # append at row 10
    torch.cuda.synchronize()
    c = cache.cpu().numpy()
    assert np.array_equal(c[10:30], orc.pack_kv(kv)) and not c[:10].any() and not c[30:].any()
    idx = _vals(rng, 9, 128)
    kr, ir = csa.pack_rows(None, torch.from_numpy(idx).cuda())
    assert kr is None and np.array_equal(ir.cpu().numpy(), orc.pack_idx(idx))


def test_packed_rows_decode_back(csa, orc):
    # rows packed on the GPU decode (oracle) to within the element grid's
    # error: half a spacing (at most 16 scale units below 512) or, for the
    # values the MX exponent rule leaves in [448, 512) scale units, the
    # saturation to 448 (under 64 units)
    rng = np.random.default_rng(4)
    kv = rng.standard_normal((64, 512)).astype(np.float32)
    kr, _ = csa.pack_rows(torch.from_numpy(kv).cuda(), None)
    d = orc.decode_kv(kr.cpu().numpy())
    sc = np.repeat(2.0 ** (kr.cpu().numpy()[:, 576:583].astype(np.float64) - 127), 64, axis=1)
    assert np.all(np.abs(d[:, :448] - kv[:, :448]) <= 64 * sc)
    assert np.allclose(d[:, 448:], kv[:, 448:], rtol=2.0 ** -11, atol=2.0 ** -25)


def test_merge_matches_oracle_merge(csa, orc):
    rng = np.random.default_rng(5)
    h = 13
    oa, ob = (rng.standard_normal((h, 512)).astype(np.float32) for _ in range(2))
    la, lb = (rng.uniform(-30, 30, h).astype(np.float32) for _ in range(2))
    la[0], lb[1], la[2], lb[2] = -np.inf, -np.inf, -np.inf, -np.inf  # empty sides
    t = [torch.from_numpy(x).cuda() for x in (oa, la, ob, lb)]
    out, lse = csa.lse_merge(*t)
    torch.cuda.synchronize()
    ro, rl = orc.lse_merge(oa, la, ob, lb)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.allclose(out, ro, rtol=1e-5, atol=1e-6)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.allclose(lse[fin], rl[fin], rtol=1e-6, atol=1e-5)
    assert np.array_equal(out[0], ob[0]) and np.array_equal(out[1], oa[1]) and np.all(out[2] == 0)


def test_decode_step_with_ring_equals_attention_over_the_union(csa, orc):
    # one softmax over the selected compressed rows and a 256-row raw ring
    s = gen.session(1)
    ring = gen.session(2, n_rows=256)["kv_rows"]
    d = gu.to_dev(s)
    out_c = csa.decode_step([d], s["softmax_scale"])[0]
    out_r, lse_r = csa.dense_attn(torch.from_numpy(ring).cuda(), d["q_attn"], s["softmax_scale"])
    out, lse = csa.lse_merge(out_c["out"], out_c["lse"], out_r, lse_r)
    torch.cuda.synchronize()
    sel = out_c["sel"].cpu().numpy()
    rows = np.concatenate([s["kv_rows"][sel], ring])
    ref_o, ref_l = orc.attention(rows, np.arange(rows.shape[0], dtype=np.int32), s["q_attn"], s["softmax_scale"])
    gu.check_attention(out.cpu().numpy(), ref_o)
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=1e-5, atol=1e-5)
