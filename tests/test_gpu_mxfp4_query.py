"""The MXFP4-quantized-query scorer on the GPU against the oracle.

The DS4X page ("What DS4X changes", "Optimization details") scores the
packed 68-byte rows with a block-scaled MXFP4 matrix product; the query is
quantized to MXFP4 first (the OCP MX v1.0 conversion, the oracle's reading).
Checked here, all bit for bit:
  * csa_quantize_query equals the oracle's quantizer on the hand-worked
    blocks and on adversarial queries;
  * the filter's brackets (one fp4 query operand, no residual) contain the
    oracle's score of the decoded quantized query;
  * the decode step with CSA_QUERY_MXFP4 selects exactly the oracle's top-512
    of that score (rows, order, scores), and its attention is within the
    tolerance of the oracle's attention over that selection.
"""
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

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


def _np(t):
    return t.detach().cpu().numpy()


def _adversarial_queries(rng, h):
    from test_filter_bound import adversarial_query

    q = adversarial_query(rng, h)
    q[0, :] = (rng.integers(-24, 25, 128) * 0.25).astype(np.float32)  # exact E2M1 ties at scale 1
    q[1 % h, 32:64] = 0.0                                              # a zero block
    q[2 % h, 64:96] = (rng.integers(-8, 9, 32) * 2.0 ** -140).astype(np.float32)  # subnormal block
    return q


def test_quantize_query_golden_blocks(csa, orc):
    gold = pins.fp4_query_golden()
    q = np.zeros((len(gold), 128), np.float32)
    for i, (_, _, vals, _) in enumerate(gold):
        q[i, 32 * (i % 4):32 * (i % 4) + 32] = vals
    got = _np(csa.quantize_query(torch.from_numpy(q).cuda()))
    assert np.array_equal(got, orc.quantize_query(q))
    codes = pins.unpack_codes(got)
    for i, (name, byte, _, want) in enumerate(gold):
        assert got[i, 64 + i % 4] == byte, name
        assert np.array_equal(codes[i, 32 * (i % 4):32 * (i % 4) + 32], want), name


@pytest.mark.parametrize("h", [1, 13, 64])
@pytest.mark.parametrize("seed", [1, 2])
def test_quantize_query_matches_oracle(csa, orc, h, seed):
    rng = np.random.default_rng(seed)
    q = _adversarial_queries(rng, h)
    got = _np(csa.quantize_query(torch.from_numpy(q).cuda()))
    ref = orc.quantize_query(q)
    assert np.array_equal(got, ref), int(np.sum(got != ref))
    # the library's own decode of the rows is the oracle's decoded query
    qhat = _np(csa.dequant_idx(torch.from_numpy(got).cuda()))
    assert pins.same_bits_or_nan(qhat, orc.quantized_query(q))


@pytest.mark.parametrize("case", ["normal", "adversarial"])
def test_mxfp4_brackets_contain_the_exact_score(csa, orc, case):
    rng = np.random.default_rng(3 + len(case))
    n = 40000
    if case == "normal":
        s = gen.session(1, n_rows=n)
        rows, q, w = s["idx_rows"], s["q_idx"], s["w_idx"]
    else:
        rows = pins.random_idx_rows(n, 9)
        rows[: n // 2, 64:68] = rng.integers(0, 253, size=(n // 2, 4))
        q = _adversarial_queries(rng, 64)
        w = (rng.uniform(-1, 1, 64) * 2.0 ** rng.integers(-20, 20, 64)).astype(np.float32)
    up, lo = csa.score_bounds(torch.from_numpy(rows).cuda(), torch.from_numpy(q).cuda(), torch.from_numpy(w).cuda(),
                              query_format="mxfp4")
    up, lo = _np(up), _np(lo)
    ref = orc.score(rows, orc.quantized_query(q), w).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.all(lo[finite] <= ref[finite]) and np.all(ref[finite] <= up[finite])
    width = (up - lo)[finite] / np.maximum(np.abs(ref[finite]), 1e-30)
    print(f"{case}: median bracket width / |score| {np.median(width):.2e}")
    if case == "normal":
        assert np.median(width) < 1e-2  # no query residual: only the fp32 sums' rounding


def _run(csa, sessions_np, scale):
    devs = [gu.to_dev(s) for s in sessions_np]
    out = csa.decode_step(devs, scale, query_format="mxfp4")
    torch.cuda.synchronize()
    return devs, [{k: _np(o[k]) for k in ("sel", "sel_score", "out", "lse")} for o in out]


def _check(orc, s, got):
    n = s["idx_rows"].shape[0]
    k_eff = min(512, n)
    qhat = orc.quantized_query(s["q_idx"])
    ref_scores = orc.score(s["idx_rows"], qhat, s["w_idx"])
    ref_sel, ref_sel_score, _ = orc.topk(ref_scores, 512)
    gu.check_selection_exact(got["sel"], got["sel_score"], ref_sel, ref_sel_score, k_eff)
    att, lse = orc.attention(s["kv_rows"], got["sel"][:k_eff], s["q_attn"], s["softmax_scale"])
    gu.check_attention(got["out"], att)
    if k_eff:
        assert np.allclose(got["lse"], lse, rtol=1e-5, atol=1e-5)
    else:
        assert np.all(np.isneginf(got["lse"])) and np.all(got["out"] == 0)


@pytest.mark.parametrize("n", [0, 1, 513, 2049, 70001])
def test_decode_step_mxfp4_small_histories(csa, orc, n):
    s = gen.session(0, n_rows=n)
    _, got = _run(csa, [s], s["softmax_scale"])
    _check(orc, s, got[0])


@pytest.mark.parametrize("cid", [0, 1, 3])
def test_decode_step_mxfp4_workloads(csa, orc, cid):
    s = gen.session(cid)
    _, got = _run(csa, [s], s["softmax_scale"])
    _check(orc, s, got[0])


def test_decode_step_mxfp4_sessions_and_heads(csa, orc):
    ss = [gen.session(1, s=i, n_rows=n, n_idx_heads=13, n_heads=20) for i, n in enumerate([3000, 0, 40000, 511])]
    _, got = _run(csa, ss, ss[0]["softmax_scale"])
    for s, g in zip(ss, got):
        _check(orc, s, g)


def test_decode_step_mxfp4_equals_library_pipeline(csa):
    # the same selection as csa_quantize_query -> csa_dequant_idx -> csa_score
    # -> csa_topk, bit for bit
    s = gen.session(1)
    devs, got = _run(csa, [s], s["softmax_scale"])
    d = devs[0]
    qhat = csa.dequant_idx(csa.quantize_query(d["q_idx"]))
    sel, sel_score = csa.topk(csa.score(d["idx_rows"], qhat, d["w_idx"]), 512)
    torch.cuda.synchronize()
    assert np.array_equal(got[0]["sel"], _np(sel))
    assert np.array_equal(got[0]["sel_score"].view(np.uint32), _np(sel_score).view(np.uint32))
