"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.  Needs an MI355X."""
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


def _np(t):
    return t.detach().cpu().numpy()


# ------------------------------------------------------------------ decode

def test_dequant_idx_every_code_scale_pair(csa, orc):
    rows = np.concatenate([pins.idx_rows_all_pairs(), gen.idx_rows(gen.seed(1), 0, 777)])
    got = _np(csa.dequant_idx(torch.from_numpy(rows).cuda()))
    assert pins.same_bits_or_nan(got, orc.decode_idx(rows))


def test_dequant_kv_every_code_scale_pair(csa, orc):
    rows = np.concatenate([pins.kv_rows_all_pairs(), gen.kv_rows(gen.seed(1), 0, 333)])
    got = _np(csa.dequant_kv(torch.from_numpy(rows).cuda()))
    assert pins.same_bits_or_nan(got, orc.decode_kv(rows))


def test_dequant_every_fp16_code(csa, orc):
    n = 65536 // 64
    rows = np.zeros((n, 583), dtype=np.uint8)
    rows[:, 448:576] = np.arange(65536, dtype="<u2").reshape(n, 64).view(np.uint8)
    got = _np(csa.dequant_kv(torch.from_numpy(rows).cuda()))
    assert pins.same_bits_or_nan(got, orc.decode_kv(rows))


# ------------------------------------------------------------------ top-k

def _tricky_scores(n, seed):
    rng = np.random.default_rng(seed)
    s = (rng.integers(-20, 60, n) * 0.25).astype(np.float32)  # heavy ties
    if n > 10:
        s[rng.integers(0, n, 3)] = np.nan
        s[rng.integers(0, n, 3)] = -0.0
        s[rng.integers(0, n, 2)] = -np.inf
        s[rng.integers(0, n, 2)] = np.inf
    return s


@pytest.mark.parametrize("n", [0, 1, 2, 100, 511, 512, 513, 2047, 2048, 2049, 5000, 70001, 3_000_001])
def test_topk_matches_oracle_exactly(csa, orc, n):
    s = _tricky_scores(n, n)
    for k in (512, 1, 37):
        sel, sel_score = csa.topk(torch.from_numpy(s).cuda(), k)
        ref_sel, ref_score, k_eff = orc.topk(s, k)
        assert np.array_equal(_np(sel), ref_sel), f"n={n} k={k}"
        assert pins.same_bits_or_nan(_np(sel_score)[:k_eff], ref_score[:k_eff])


@pytest.mark.parametrize("pattern", ["ascending", "descending", "one_tile", "two_values", "clustered"])
@pytest.mark.parametrize("n", [40000, 1 << 20])
def test_topk_adversarial_layouts(csa, orc, pattern, n):
    rng = np.random.default_rng(n % 1000 + len(pattern))
    if pattern == "ascending":  # every winner in the last tiles
        s = np.arange(n, dtype=np.float32)
    elif pattern == "descending":
        s = np.arange(n, 0, -1).astype(np.float32)
    elif pattern == "one_tile":  # all winners packed in one tile, ties inside it
        s = rng.standard_normal(n).astype(np.float32)
        s[n // 3:n // 3 + 700] = 100.0 + (np.arange(700) % 7).astype(np.float32)
    elif pattern == "two_values":
        s = np.where(rng.random(n) < 0.001, 2.0, 1.0).astype(np.float32)
    else:  # many near-equal values around the threshold
        s = (1000.0 + rng.integers(0, 3, n) * np.float32(2.0**-13)).astype(np.float32)
    sel, sel_score = csa.topk(torch.from_numpy(s).cuda(), 512)
    ref_sel, ref_score, _ = orc.topk(s, 512)
    assert np.array_equal(_np(sel), ref_sel)
    assert pins.same_bits_or_nan(_np(sel_score), ref_score)


def test_topk_all_ties_and_distinct(csa, orc):
    z = np.zeros(300000, np.float32)
    sel, _ = csa.topk(torch.from_numpy(z).cuda())
    assert np.array_equal(_np(sel), np.arange(512))
    s = np.random.default_rng(5).standard_normal(300000).astype(np.float32)
    sel, _ = csa.topk(torch.from_numpy(s).cuda())
    assert np.array_equal(_np(sel), orc.topk(s)[0])


# ------------------------------------------------------------------ score

@pytest.mark.parametrize("cid,n", [(0, 2048), (1, 32768), (0, 2049), (1, 6001), (0, 70001)])
def test_score_matches_oracle_bit_for_bit(csa, orc, cid, n):
    # csa_score evaluates the score definition in fp64 in the reference order
    # and rounds once: it equals the oracle bit for bit
    s = gen.session(cid, n_rows=n)
    d = gu.to_dev(s)
    got = _np(csa.score(d["idx_rows"], d["q_idx"], d["w_idx"]))
    ref = orc.score(s["idx_rows"], s["q_idx"], s["w_idx"])
    assert pins.same_bits_or_nan(got, ref), int(np.sum(got.view(np.uint32) != ref.view(np.uint32)))


def test_score_tiny_mixed_scales_and_adversarial_queries(csa, orc):
    from test_filter_bound import adversarial_query

    rows = pins.random_idx_rows(3000, 21)
    rng = np.random.default_rng(2)
    rows[:1000, 64:68] = rng.integers(0, 6, size=(1000, 4))  # subnormal decoded values
    rows[1000:1500, 64:68] = rng.integers(0, 250, size=(500, 4))  # wildly mixed blocks
    for q in (rng.standard_normal((8, 128)).astype(np.float32), adversarial_query(rng, 12)):
        w = (rng.uniform(-1, 1, q.shape[0]) * 2.0 ** rng.integers(-8, 8, q.shape[0])).astype(np.float32)
        got = _np(csa.score(torch.from_numpy(rows).cuda(), torch.from_numpy(q).cuda(), torch.from_numpy(w).cuda()))
        ref = orc.score(rows, q, w)
        assert pins.same_bits_or_nan(got, ref)


@pytest.mark.parametrize("case", ["normal", "adversarial", "extreme_scales"])
def test_filter_brackets_contain_the_exact_score(csa, orc, case):
    """The decode step's matrix-core filter (three fp6 query terms, fp32
    sums) and its rigorous bound: lower <= oracle score <= upper on every
    row, with adversarial queries (large in-block dynamic range, subnormal
    and zero blocks, values near the E2M3 rounding ties, huge heads) and
    every finite scale byte."""
    from test_filter_bound import adversarial_query

    rng = np.random.default_rng(len(case))
    n = 40000
    if case == "normal":
        s = gen.session(1, n_rows=n)
        rows, q, w = s["idx_rows"], s["q_idx"], s["w_idx"]
    else:
        rows = pins.random_idx_rows(n, 7)
        q = adversarial_query(rng, 64)
        w = (rng.uniform(-1, 1, 64) * 2.0 ** rng.integers(-20, 20, 64)).astype(np.float32)
        if case == "extreme_scales":
            rows[:, 64:68] = rng.integers(0, 256, size=(n, 4))
            rows[rows[:, 64:68].max(axis=1) == 255, 64:68] = 254  # no NaN scales
    up, lo = csa.score_bounds(torch.from_numpy(rows).cuda(), torch.from_numpy(q).cuda(), torch.from_numpy(w).cuda())
    up, lo = _np(up), _np(lo)
    ref = orc.score(rows, q, w).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.all(lo[finite] <= ref[finite]) and np.all(ref[finite] <= up[finite]), (
        int(np.sum(lo[finite] > ref[finite])), int(np.sum(ref[finite] > up[finite])))
    assert np.all(up >= lo)
    big = rows[:, 64:68].max(axis=1) >= 253  # bytes that can decode to infinity: unbounded brackets
    assert np.all(np.isposinf(up[big])) and np.all(np.isneginf(lo[big]))
    width = (up - lo)[~big] / np.maximum(np.abs(ref[~big]), 1e-30)
    print(f"{case}: median bracket width / |score| {np.median(width):.2e}")
    if case == "normal":
        assert np.median(width) < 5e-2  # a useful filter (about +-0.6% at these workloads), not a vacuous one


# ------------------------------------------------------------------ decode step

def _run_step(csa, sessions_np, scale):
    devs = [gu.to_dev(s) for s in sessions_np]
    out = csa.decode_step(devs, scale)
    torch.cuda.synchronize()
    return [{k: _np(o[k]) for k in ("sel", "sel_score", "out", "lse")} for o in out]


def _check_session(orc, s, got):
    """The selection equals the oracle's exactly (rows, order and scores, bit
    for bit: the candidates are rescored in the reference's arithmetic), and
    the attention over it is within the tolerance."""
    n = s["idx_rows"].shape[0]
    k_eff = min(512, n)
    ref_scores = orc.score(s["idx_rows"], s["q_idx"], s["w_idx"])
    ref_sel, ref_sel_score, _ = orc.topk(ref_scores, 512)
    info = gu.check_selection_exact(got["sel"], got["sel_score"], ref_sel, ref_sel_score, k_eff)
    att, lse = orc.attention(s["kv_rows"], got["sel"][:k_eff], s["q_attn"], s["softmax_scale"])
    info["attn_rel_err"] = gu.check_attention(got["out"], att)
    if k_eff:
        assert np.allclose(got["lse"], lse, rtol=1e-5, atol=1e-5)
    else:
        assert np.all(np.isneginf(got["lse"])) and np.all(got["out"] == 0)
    return info


@pytest.mark.parametrize("n", [0, 1, 7, 300, 511, 512, 513, 2048, 2049, 6001])
def test_decode_step_small_histories(csa, orc, n):
    s = gen.session(0, n_rows=n)
    got = _run_step(csa, [s], s["softmax_scale"])[0]
    _check_session(orc, s, got)


@pytest.mark.parametrize("cid", [0, 1, 2])
def test_decode_step_full_workload(csa, orc, cid):
    s = gen.session(cid)
    got = _run_step(csa, [s], s["softmax_scale"])[0]
    info = _check_session(orc, s, got)
    print(f"workload {gen.WORKLOADS[cid].name}: {info}")


def test_decode_step_frontier_1m(csa, orc):
    s = gen.session(3)
    got = _run_step(csa, [s], s["softmax_scale"])[0]
    info = _check_session(orc, s, got)
    print(f"workload {gen.WORKLOADS[3].name}: {info}")


def test_decode_step_sixteen_sessions(csa, orc):
    w = gen.WORKLOADS[4]
    ss = [gen.session(4, s=i) for i in range(w.n_sessions)]
    got = _run_step(csa, ss, ss[0]["softmax_scale"])
    for s, g in zip(ss, got):
        _check_session(orc, s, g)


def test_decode_step_ragged_sessions(csa, orc):
    sizes = [0, 5, 512, 513, 3000, 2048, 70000, 1]
    ss = [gen.session(1, s=i, n_rows=n) for i, n in enumerate(sizes)]
    got = _run_step(csa, ss, ss[0]["softmax_scale"])
    for s, g in zip(ss, got):
        _check_session(orc, s, g)


@pytest.mark.parametrize("n_idx_heads,n_heads", [(1, 1), (13, 20), (40, 64), (64, 7)])
def test_decode_step_head_counts(csa, orc, n_idx_heads, n_heads):
    # head groups only partly filled: dead indexer heads weigh zero, dead
    # attention heads are not written
    s = gen.session(1, n_rows=20000, n_idx_heads=n_idx_heads, n_heads=n_heads)
    got = _run_step(csa, [s], s["softmax_scale"])[0]
    assert got["out"].shape == (n_heads, 512)
    _check_session(orc, s, got)


@pytest.mark.parametrize("sizes", [[3000, 700], [3000, 700, 0], [513, 40000, 511, 1, 9000]])
def test_decode_step_session_counts(csa, orc, sizes):
    # two sessions: attention inside the selection kernel; three or more:
    # selection alone, then the attention with fewer row groups
    ss = [gen.session(1, s=i, n_rows=n) for i, n in enumerate(sizes)]
    got = _run_step(csa, ss, ss[0]["softmax_scale"])
    for s, g in zip(ss, got):
        _check_session(orc, s, g)


@pytest.mark.parametrize("n_rows", [None, 2_500_000])
def test_fused_equals_unfused(csa, n_rows):
    # 2.5M rows: more tile heads than the selection holds in registers
    s = gen.session(1) if n_rows is None else gen.session(1, n_rows=n_rows)
    d = gu.to_dev(s)
    step = csa.decode_step([dict(d)], s["softmax_scale"])[0]
    scores = csa.score(d["idx_rows"], d["q_idx"], d["w_idx"])
    sel, sel_score = csa.topk(scores, 512)
    out, lse = csa.sparse_attn(d["kv_rows"], sel, 512, d["q_attn"], s["softmax_scale"])
    torch.cuda.synchronize()
    assert torch.equal(step["sel"], sel) and torch.equal(step["sel_score"], sel_score)
    assert torch.equal(step["out"], out) and torch.equal(step["lse"], lse)
    # the selection is the exact top-512 of the GPU's own scores
    assert np.array_equal(_np(sel), gu.topk_keys_host(_np(scores), 512))


@pytest.mark.parametrize("pattern", ["one_stretch", "ascending", "descending", "clustered", "two_rows"])
def test_decode_step_adversarial_layouts(csa, orc, pattern):
    """The decode step (filter, tile heads, rescoring, selection) on score
    layouts built from the rows themselves: a row's scale bytes set its
    scores' magnitude, so the winners can be packed into one stretch of
    rows (whole tiles are then "full" and rescored row by row), sit at the
    end or the start, form clusters, or tie massively (two distinct rows).
    The selection must still be exactly the oracle's."""
    n = 60000
    s = gen.session(1, n_rows=n, seed_=91)
    idx = s["idx_rows"]
    r = np.arange(n)
    if pattern == "one_stretch":  # 700 consecutive rows eight times larger
        idx[:, 64:68] = 120
        idx[30000:30700, 64:68] = 123
    elif pattern == "ascending":  # every winner among the last rows
        idx[:, 64:68] = (110 + (20 * r) // n)[:, None]
    elif pattern == "descending":
        idx[:, 64:68] = (130 - (20 * r) // n)[:, None]
    elif pattern == "clustered":  # eight clusters of 90 rows
        idx[:, 64:68] = 118
        for c in range(8):
            idx[5000 + 7000 * c:5090 + 7000 * c, 64:68] = 121
    else:  # two distinct rows alternating: ties decided by the row index
        a, b = idx[3].copy(), idx[4].copy()
        idx[0::2] = a
        idx[1::2] = b
    print(f"adversarial layout {pattern}: n_rows={n}", flush=True)
    got = _run_step(csa, [s], s["softmax_scale"])[0]
    _check_session(orc, s, got)


def test_zero_cache_selects_first_rows(csa, orc):
    s = gen.session(1, n_rows=20000)
    s["idx_rows"] = np.zeros_like(s["idx_rows"])
    s["idx_rows"][:, 64:] = 127
    got = _run_step(csa, [s], s["softmax_scale"])[0]
    assert np.array_equal(got["sel"], np.arange(512))
    assert np.all(got["sel_score"] == 0)
    _check_session(orc, s, got)


def test_duplicate_rows_tie_break(csa, orc):
    s = gen.session(1, n_rows=9000)
    s["idx_rows"][:] = s["idx_rows"][17]
    got = _run_step(csa, [s], s["softmax_scale"])[0]
    assert np.array_equal(got["sel"], np.arange(512))
    _check_session(orc, s, got)


def test_sparse_attn_skips_invalid_entries(csa, orc):
    s = gen.session(0, n_rows=1000)
    d = gu.to_dev(s)
    sel = np.arange(0, 600, 3, dtype=np.int32)[:200]
    sel[[3, 50, 199]] = [-1, 1000, 2**31 - 1]
    out, lse = csa.sparse_attn(d["kv_rows"], torch.from_numpy(sel).cuda(), len(sel), d["q_attn"], s["softmax_scale"])
    valid = sel[(sel >= 0) & (sel < 1000)]
    ref, ref_lse = orc.attention(s["kv_rows"], valid, s["q_attn"], s["softmax_scale"])
    gu.check_attention(_np(out), ref)
    assert np.allclose(_np(lse), ref_lse, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("count", [33, 64, 65, 100, 512])
def test_sparse_attn_crowded_row_group(csa, orc, count):
    # every entry in one of the stand-alone attention's 32 row groups (the
    # top five bits of row * 0x9E3779B1), so that one workgroup stages many
    # 32-row rounds, the last one partial; plus the buffer's last row
    n = 20000
    s = gen.session(0, n_rows=n)
    d = gu.to_dev(s)
    rows = np.arange(n, dtype=np.uint64)
    group = ((rows * np.uint64(0x9E3779B1)) & np.uint64(0xFFFFFFFF)) >> np.uint64(27)
    g0 = np.nonzero(group == group[n - 1])[0]
    assert len(g0) >= count
    sel = np.random.default_rng(count).permutation(g0[g0 != n - 1])[:count - 1].astype(np.int32)
    sel = np.concatenate([sel, [n - 1]]).astype(np.int32)
    out, lse = csa.sparse_attn(d["kv_rows"], torch.from_numpy(sel).cuda(), len(sel), d["q_attn"], s["softmax_scale"])
    ref, ref_lse = orc.attention(s["kv_rows"], sel, s["q_attn"], s["softmax_scale"])
    gu.check_attention(_np(out), ref)
    assert np.allclose(_np(lse), ref_lse, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("n_rows,fmt", [(20000, "fp32"), (20000, "mxfp4"), (300, "fp32")])
def test_decode_step_timed_matches_untimed(csa, n_rows, fmt):
    """The timed decode step (stage events) does exactly the untimed step's
    work: identical outputs.  Every stage's event pair completes; stage 0's
    pair, recorded by the score kernel's launch at the kernel's own start
    and end, spans a positive time whenever the kernel runs (a short fp32
    history skips it, and its pair is then recorded back to back)."""
    s = gen.session(1, n_rows=n_rows)
    d = gu.to_dev(s)
    ref = csa.decode_step([dict(d)], s["softmax_scale"], query_format=fmt)[0]
    ref = {k: ref[k].clone() for k in ("sel", "sel_score", "out", "lse")}
    step = csa.DecodeStep([dict(d)], s["softmax_scale"], query_format=fmt)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(csa.STAGES))]
    step.timed(evs)
    torch.cuda.synchronize()
    got = step.sessions[0]
    for k, v in ref.items():
        assert torch.equal(got[k], v), k
    ms = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(len(csa.STAGES))]
    print(f"stage ms {ms}")
    assert all(m >= 0.0 for m in ms)
    if n_rows > 4096 or fmt == "mxfp4":
        assert ms[0] > 0.0


def test_deterministic(csa):
    s = gen.session(1, n_rows=40000)
    a = _run_step(csa, [s], s["softmax_scale"])[0]
    b = _run_step(csa, [s], s["softmax_scale"])[0]
    for k in a:
        assert a[k].tobytes() == b[k].tobytes()
