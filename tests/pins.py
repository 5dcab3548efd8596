"""Pins of the CPU oracle against things other than itself.

Each ``check_*`` function takes an ``oracle.Oracle`` and raises
``AssertionError`` on a mismatch.  They are used twice: on the real oracle
(test_oracle_pins.py) and on deliberately broken copies of its source
(test_oracle_mutants.py), which every plausible mistake must fail.

Independent references used here:
  * element decoding by library routines: ``torch.float8_e4m3fn``,
    ``torch.float8_e8m0fnu`` and ``numpy.float16`` (little-endian '<f2');
  * the E2M1 value table of the OCP MX v1.0 specification (golden file);
  * numbers printed on the DS4X page, "Packed cache ABI" (golden file);
  * hand-worked MXFP4 conversions of query blocks from the OCP MX v1.0
    definition (golden file) and a brute-force nearest-value search over the
    E2M1 table;
  * numpy float64 ``einsum`` for the score, Python ``sorted`` for the top-k,
    ``torch.nn.functional.scaled_dot_product_attention`` in float64 on the CPU
    for attention, plus closed-form special cases.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- golden files

def load_kv_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = float(v) if "." in v else int(v)
    return out


def e2m1_golden() -> np.ndarray:
    vals = {}
    with open(os.path.join(GOLDEN, "ocp_mx_e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                c, v = line.split()
                vals[int(c)] = float(v)
    mags = np.array([vals[c] for c in range(8)], dtype=np.float64)
    return np.concatenate([mags, -mags])  # codes 8..15 carry the sign bit


# ------------------------------------------------ library-based element decode

def lib_e4m3(codes) -> np.ndarray:
    t = torch.as_tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def lib_ue8m0(b) -> np.ndarray:
    t = torch.as_tensor(np.asarray(b, dtype=np.uint8)).view(torch.float8_e8m0fnu)
    return t.to(torch.float64).numpy()


def lib_f16(bits) -> np.ndarray:
    return np.asarray(bits, dtype="<u2").view("<f2").astype(np.float64)


def ref_decode_idx(rows: np.ndarray) -> np.ndarray:
    """Decode 68-byte indexer rows with the library references above."""
    rows = np.asarray(rows, dtype=np.uint8).reshape(-1, 68)
    codes = np.empty((rows.shape[0], 128), dtype=np.int64)
    codes[:, 0::2] = rows[:, :64] & 15
    codes[:, 1::2] = rows[:, :64] >> 4
    vals = e2m1_golden()[codes]
    scale = np.repeat(lib_ue8m0(rows[:, 64:68]), 32, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        return (vals * scale).astype(np.float32)


def ref_decode_kv(rows: np.ndarray) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8).reshape(-1, 583)
    out = np.empty((rows.shape[0], 512), dtype=np.float32)
    scale = np.repeat(lib_ue8m0(rows[:, 576:583]), 64, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        out[:, :448] = (lib_e4m3(rows[:, :448]) * scale).astype(np.float32)
    out[:, 448:] = np.ascontiguousarray(rows[:, 448:576]).view("<f2").astype(np.float32)
    return out


def same_bits_or_nan(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    an, bn = np.isnan(a), np.isnan(b)
    if not np.array_equal(an, bn):
        return False
    return np.array_equal(a[~an].view(np.uint32), b[~bn].view(np.uint32))


# ------------------------------------------------------------ row builders

def idx_rows_all_pairs() -> np.ndarray:
    """Rows that put every (E2M1 code, UE8M0 byte) pair through the decoder:
    row r uses scale byte r for all four blocks and codes cycling 0..15."""
    rows = np.zeros((256, 68), dtype=np.uint8)
    el = np.arange(128) % 16
    packed = (el[0::2] | (el[1::2] << 4)).astype(np.uint8)
    rows[:, :64] = packed
    rows[:, 64:68] = np.arange(256, dtype=np.uint8)[:, None]
    return rows


def kv_rows_all_pairs() -> np.ndarray:
    """Every (E4M3 byte, UE8M0 byte) pair: row r has scale byte r in all seven
    blocks and non-RoPE bytes cycling through 0..255; RoPE slots hold
    assorted FP16 codes (normal, subnormal, inf, NaN)."""
    rows = np.zeros((256, 583), dtype=np.uint8)
    rows[:, :448] = (np.arange(448) % 256).astype(np.uint8)[None, :]
    rows[:, 576:583] = np.arange(256, dtype=np.uint8)[:, None]
    rng = np.random.default_rng(7)
    f16 = rng.integers(0, 65536, size=(256, 64), dtype=np.uint32).astype("<u2")
    f16[:, :8] = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x7C00], dtype="<u2")
    f16[:, 8] = 0xFC00
    f16[:, 9] = 0x7E01
    rows[:, 448:576] = f16.view(np.uint8).reshape(256, 128)
    return rows


def random_idx_rows(n: int, seed: int) -> np.ndarray:
    """Random codes with mixed, moderate scales (bytes 120..134)."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, 256, size=(n, 68), dtype=np.uint8)
    rows[:, 64:68] = rng.integers(120, 135, size=(n, 4), dtype=np.uint8)
    return rows


def random_kv_rows(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, 256, size=(n, 583), dtype=np.uint8)
    codes = rows[:, :448]
    codes[(codes & 0x7F) == 0x7F] = 0x3F  # no NaN codes
    rows[:, 576:583] = rng.integers(120, 132, size=(n, 7), dtype=np.uint8)
    f16 = rng.standard_normal((n, 64)).astype("<f2")
    rows[:, 448:576] = f16.view(np.uint8).reshape(n, 128)
    return rows


# ------------------------------------------------------------------ checks

def check_tables(o) -> None:
    e2 = e2m1_golden()
    got = np.array([o.e2m1(c) for c in range(16)])
    assert np.array_equal(got, e2) and math.copysign(1, o.e2m1(8)) < 0, "E2M1 table"
    got = np.array([o.e4m3(c) for c in range(256)])
    ref = lib_e4m3(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "E4M3 NaN codes"
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)]), "E4M3 table"
    got = np.array([o.ue8m0(b) for b in range(256)])
    ref = lib_ue8m0(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "UE8M0 NaN"
    assert np.array_equal(got[:255], ref[:255]), "UE8M0 table"
    bits = np.arange(65536)
    got = np.array([o.f16(int(b)) for b in bits])
    ref = lib_f16(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "FP16 NaN"
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m]), "FP16 table"
    # spot values of the formats' definitions
    assert o.e4m3(0x7E) == 448.0 and o.e4m3(0x38) == 1.0 and o.e4m3(0x08) == 2.0**-6
    assert o.e4m3(0x01) == 2.0**-9
    assert o.ue8m0(127) == 1.0 and o.ue8m0(0) == 2.0**-127 and o.ue8m0(254) == 2.0**127
    assert o.f16(0x3C00) == 1.0 and o.f16(0x0001) == 2.0**-24 and o.f16(0x7BFF) == 65504.0


def check_decode(o) -> None:
    rows = idx_rows_all_pairs()
    assert same_bits_or_nan(o.decode_idx(rows), ref_decode_idx(rows)), "indexer row decode (code x scale grid)"
    rows = kv_rows_all_pairs()
    assert same_bits_or_nan(o.decode_kv(rows), ref_decode_kv(rows)), "KV row decode (code x scale grid)"
    # row stride and field positions: distinct random rows decode independently
    rows = random_idx_rows(5, 1)
    assert same_bits_or_nan(o.decode_idx(rows), ref_decode_idx(rows)), "indexer row stride"
    rows = random_kv_rows(5, 2)
    assert same_bits_or_nan(o.decode_kv(rows), ref_decode_kv(rows)), "KV row stride"


def ref_score(idx_rows, q_idx, w_idx) -> np.ndarray:
    k = ref_decode_idx(idx_rows).astype(np.float64)
    d = np.einsum("hi,ji->jh", np.asarray(q_idx, np.float64), k)
    s = (np.asarray(w_idx, np.float64)[None, :] * np.maximum(d, 0.0)).sum(axis=1)
    return s.astype(np.float32)


def check_score(o) -> None:
    rng = np.random.default_rng(11)
    for n, h in ((1, 1), (7, 2), (64, 3), (33, 8)):
        rows = random_idx_rows(n, 100 + n)
        q = rng.standard_normal((h, 128)).astype(np.float32)
        w = rng.uniform(0, 1, h).astype(np.float32)
        got = o.score(rows, q, w)
        ref = ref_score(rows, q, w)
        assert np.all(np.abs(got - ref) <= 2.0**-23 * np.abs(ref)), f"score n={n} H={h}"
    # H = 1, w = 1 with a positive dot product: the score is the plain dot
    rows = random_idx_rows(16, 5)
    k = ref_decode_idx(rows).astype(np.float64)
    q = np.sign(k[0]).astype(np.float32)[None, :]
    got = o.score(rows[:1], q, np.ones(1, np.float32))
    assert got[0] == np.float32(np.dot(q[0].astype(np.float64), k[0])), "H=1 plain dot"
    # w = 0 -> 0; the zero cache -> every score exactly +0
    assert np.all(o.score(rows, rng.standard_normal((4, 128)).astype(np.float32), np.zeros(4, np.float32)) == 0)
    zero = np.zeros((9, 68), dtype=np.uint8)
    zero[:, 64:] = 127
    s = o.score(zero, rng.standard_normal((4, 128)).astype(np.float32), np.ones(4, np.float32))
    assert np.all(s.view(np.uint32) == 0), "zero cache scores are +0"
    # a head whose dot is negative contributes nothing (ReLU), weights scale heads
    q2 = np.stack([q[0], -q[0]])
    got = o.score(rows[:1], q2, np.array([0.25, 1.0], np.float32))
    assert got[0] == np.float32(0.25 * np.dot(q[0].astype(np.float64), k[0])), "ReLU / weights"


def ref_topk(scores: np.ndarray, k: int):
    order = sorted(range(len(scores)), key=lambda j: (1 if math.isnan(scores[j]) else 0,
                                                       0.0 if math.isnan(scores[j]) else -float(scores[j]), j))
    return order[:k]


def check_topk(o) -> None:
    rng = np.random.default_rng(3)
    for n in (0, 1, 5, 511, 512, 513, 1500):
        s = rng.integers(0, 40, n).astype(np.float32) * 0.5  # many ties
        sel, ss, k_eff = o.topk(s, 512)
        ref = ref_topk(list(s), 512)
        assert k_eff == min(512, n)
        assert list(sel[:k_eff]) == ref, f"top-k n={n}"
        assert np.all(sel[k_eff:] == -1)
        assert np.array_equal(ss[:k_eff], s[ref]) if k_eff else True
    # zero cache: every score ties, rows 0..511 in order
    sel, _, _ = o.topk(np.zeros(4096, np.float32), 512)
    assert list(sel) == list(range(512)), "zero-cache tie break"
    # -0 ties with +0; NaN sorts after every number
    s = np.array([np.nan, -0.0, 0.0, -1.0, np.inf, np.nan], np.float32)
    sel, _, _ = o.topk(s, 6)
    assert list(sel) == [4, 1, 2, 3, 0, 5], "signed zero / NaN order"
    s = rng.standard_normal(3000).astype(np.float32)
    sel, _, _ = o.topk(s, 512)
    assert list(sel) == ref_topk(list(s), 512), "distinct scores"


def ref_attention(kv_rows, sel, q_attn, scale):
    kv = torch.from_numpy(ref_decode_kv(np.asarray(kv_rows)[np.asarray(sel)]).astype(np.float64))
    q = torch.from_numpy(np.asarray(q_attn, np.float64))
    h, n = q.shape[0], kv.shape[0]
    kvb = kv[None, None].expand(1, h, n, 512)
    o = torch.nn.functional.scaled_dot_product_attention(q[None, :, None, :], kvb, kvb,
                                                         scale=float(scale))[0, :, 0, :]
    logits = (q @ kv.T) * float(scale)
    lse = torch.logsumexp(logits, dim=1)
    return o.numpy(), lse.numpy()


def check_attention(o) -> None:
    rng = np.random.default_rng(9)
    rows = random_kv_rows(40, 4)
    scale = float(np.float32(1 / math.sqrt(512)))
    for nsel, h in ((1, 1), (3, 2), (17, 4), (40, 3)):
        sel = rng.permutation(40)[:nsel].astype(np.int32)
        q = rng.standard_normal((h, 512)).astype(np.float32)
        out, lse = o.attention(rows, sel, q, scale)
        ref_o, ref_l = ref_attention(rows, sel, q, scale)
        assert np.max(np.abs(out - ref_o)) <= 1e-6 * max(1e-30, np.max(np.abs(ref_o))), f"attention n_sel={nsel}"
        assert np.allclose(lse, ref_l, rtol=1e-6, atol=1e-6), "lse"
    kv = ref_decode_kv(rows)
    # one selected row: the output is that row exactly
    out, _ = o.attention(rows, np.array([7], np.int32), rng.standard_normal((2, 512)).astype(np.float32), scale)
    assert np.array_equal(out[0], kv[7]) and np.array_equal(out[1], kv[7]), "k=1"
    # q = 0: the output is the mean of the selected rows and lse = log(n)
    sel = np.array([1, 5, 9, 30], np.int32)
    out, lse = o.attention(rows, sel, np.zeros((1, 512), np.float32), scale)
    mean = kv[sel].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(out[0] - mean)) <= 1e-6 * np.max(np.abs(mean)), "q=0 mean"
    assert abs(lse[0] - math.log(4)) < 1e-6, "q=0 lse"
    # no row selected: zero output and lse = -inf
    out, lse = o.attention(rows, np.zeros(0, np.int32), np.ones((2, 512), np.float32), scale)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def check_dense_attention(o) -> None:
    """Attention over every row against float64 scaled_dot_product_attention
    over the library-decoded rows, and closed forms: one row gives that row,
    q = 0 gives the mean of all rows with lse = log n, no row gives 0 and
    -inf."""
    rng = np.random.default_rng(13)
    rows = random_kv_rows(300, 6)
    scale = float(np.float32(1 / math.sqrt(512)))
    for n, h in ((1, 1), (2, 3), (33, 2), (300, 4)):
        q = rng.standard_normal((h, 512)).astype(np.float32)
        out, lse = o.dense_attention(rows[:n], q, scale)
        ref_o, ref_l = ref_attention(rows[:n], np.arange(n), q, scale)
        assert np.max(np.abs(out - ref_o)) <= 1e-6 * max(1e-30, np.max(np.abs(ref_o))), f"dense n={n}"
        assert np.allclose(lse, ref_l, rtol=1e-6, atol=1e-6), "dense lse"
    kv = ref_decode_kv(rows)
    out, _ = o.dense_attention(rows[5:6], rng.standard_normal((2, 512)).astype(np.float32), scale)
    assert np.array_equal(out[0], kv[5]) and np.array_equal(out[1], kv[5]), "dense n=1"
    out, lse = o.dense_attention(rows[:77], np.zeros((1, 512), np.float32), scale)
    mean = kv[:77].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(out[0] - mean)) <= 1e-6 * np.max(np.abs(mean)), "dense q=0 mean"
    assert abs(lse[0] - math.log(77)) < 1e-6, "dense q=0 lse"
    out, lse = o.dense_attention(rows[:0], np.ones((2, 512), np.float32), scale)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def check_decode_step(o) -> None:
    """The whole step against the pipeline built from the independent
    references above (numpy score -> Python sort -> PyTorch attention), at a
    history shorter than 512 rows, one longer, and an empty one, with indexer
    and attention head counts that differ (so a swapped count or query
    cannot pass)."""
    rng = np.random.default_rng(17)
    scale = float(np.float32(1 / math.sqrt(512)))
    for n, h_idx, h in ((300, 3, 2), (700, 2, 3), (0, 2, 1)):
        idx = random_idx_rows(n, 40 + n)
        kv = random_kv_rows(n, 50 + n)
        q = rng.standard_normal((h_idx, 128)).astype(np.float32)
        w = rng.uniform(0, 1, h_idx).astype(np.float32)
        qa = rng.standard_normal((h, 512)).astype(np.float32)
        got = o.decode_step(idx, kv, q, w, qa, scale)
        k_eff = min(512, n)
        assert got["k_eff"] == k_eff
        s = ref_score(idx, q, w)
        sel = ref_topk(list(s), 512)
        assert list(got["sel"][:k_eff]) == sel, f"decode step selection n={n}"
        assert np.all(got["sel"][k_eff:] == -1) and np.all(np.isneginf(got["sel_score"][k_eff:]))
        assert np.array_equal(got["sel_score"][:k_eff], s[sel]), "decode step selected scores"
        if k_eff == 0:
            assert np.all(got["out"] == 0) and np.all(np.isneginf(got["lse"])), "empty history"
            continue
        ref_o, ref_l = ref_attention(kv, np.array(sel), qa, scale)
        assert np.max(np.abs(got["out"] - ref_o)) <= 1e-6 * np.max(np.abs(ref_o)), f"decode step attention n={n}"
        assert np.allclose(got["lse"], ref_l, rtol=1e-6, atol=1e-6), "decode step lse"


# ------------------------------------------------------- MXFP4 query quantizer

def fp4_query_golden() -> list:
    """Blocks of tests/golden/ocp_mx_fp4_query_blocks.txt: (name, scale byte,
    32 fp32 values, 32 codes)."""
    blocks, cur = [], None
    with open(os.path.join(GOLDEN, "ocp_mx_fp4_query_blocks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            t = line.split()
            if t[0] == "block":
                cur = [t[1], int(t[2]), np.zeros(32, np.float32), np.zeros(32, np.int64)]
                blocks.append(cur)
            else:
                i = int(t[0])
                v = float.fromhex(t[1]) if "x" in t[1] else float(t[1])
                cur[2][i] = np.float32(v)
                cur[3][i] = int(t[2])
    return blocks


def unpack_codes(rows: np.ndarray) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8).reshape(-1, 68)
    codes = np.empty((rows.shape[0], 128), dtype=np.int64)
    codes[:, 0::2] = rows[:, :64] & 15
    codes[:, 1::2] = rows[:, :64] >> 4
    return codes


def brute_force_fp4(v: np.ndarray):
    """The conversion by exhaustive search: for each block the exponent
    floor(log2 amax) (math.frexp) - 2 clamped to [-127, 127] (zero block:
    -127), for each element the E2M1 table entry at the least distance from
    v / 2^e, ties to the entry with an even code, sign from v's sign bit."""
    v = np.asarray(v, dtype=np.float32).reshape(-1, 32).astype(np.float64)
    table = e2m1_golden()[:8]
    codes = np.zeros(v.shape, dtype=np.int64)
    byte = np.zeros(v.shape[0], dtype=np.int64)
    for b in range(v.shape[0]):
        amax = float(np.max(np.abs(v[b])))
        e = -127 if amax == 0.0 else min(max(math.frexp(amax)[1] - 1 - 2, -127), 127)
        byte[b] = e + 127
        y = np.abs(v[b]) * 2.0 ** (-e)
        dist = np.abs(y[:, None] - table[None, :])           # [32][8]
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best
        even = cand & (np.arange(8)[None, :] % 2 == 0)
        mag = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
        codes[b] = mag | np.where(np.signbit(v[b]), 8, 0)
    return byte, codes


def check_quantize_query(o) -> None:
    # the hand-worked blocks, each placed at every block position of a head
    gold = fp4_query_golden()
    for pos in range(4):
        q = np.zeros((len(gold), 128), np.float32)
        for i, (_, _, vals, _) in enumerate(gold):
            q[i, 32 * pos:32 * pos + 32] = vals
        rows = o.quantize_query(q)
        codes = unpack_codes(rows)
        for i, (name, byte, _, want) in enumerate(gold):
            assert rows[i, 64 + pos] == byte, (name, pos, rows[i, 64 + pos], byte)
            assert np.array_equal(codes[i, 32 * pos:32 * pos + 32], want), (name, pos)
            other = [b for b in range(4) if b != pos]
            assert np.all(rows[i, 64 + np.array(other)] == 0), (name, pos)  # zero blocks: byte 0
    # random blocks over many binades against the exhaustive search
    rng = np.random.default_rng(11)
    q = (rng.standard_normal((16, 128)) * 2.0 ** rng.integers(-40, 40, (16, 128))).astype(np.float32)
    q[3] = (rng.integers(-16, 17, 128) * 0.25).astype(np.float32)  # many exact ties
    q[4, :32] = 0.0
    rows = o.quantize_query(q)
    byte, codes = brute_force_fp4(q)
    assert np.array_equal(rows[:, 64:68].reshape(-1), byte)
    assert np.array_equal(unpack_codes(rows).reshape(-1, 32), codes)
    # the decoded query is a fixed point of the conversion
    qhat = o.decode_idx(rows)
    assert np.array_equal(o.quantize_query(qhat), rows)


# ------------------------------------------------ packing new rows, the merge

def lib_e4m3_code(y: np.ndarray) -> np.ndarray:
    """E4M3 codes of |y| <= 464 by torch's float8_e4m3fn conversion (round to
    nearest even)."""
    t = torch.as_tensor(np.asarray(y, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().astype(np.int64)


def check_pack(o) -> None:
    rng = np.random.default_rng(21)
    n = 24
    v = (rng.standard_normal((n, 512)) * 2.0 ** rng.integers(-30, 30, (n, 1))).astype(np.float32)
    v[1, :64] = 0.0                                                     # a zero block
    v[2, 64:128] = (rng.integers(-15, 16, 64) * 0.0625).astype(np.float32)  # exact E4M3 ties at scale 2^-? blocks
    v[3, 448:] = (rng.standard_normal(64) * 1e-6).astype(np.float32)    # binary16 subnormals
    v[4, 448:] = (rng.standard_normal(64) * 3e4).astype(np.float32)     # binary16 overflow to infinity
    v[5, 448:] = np.array([65504.0, 65519.0, 65520.0, -65520.0, 2.0 ** -25, 3 * 2.0 ** -26] * 10 + [0.0, -0.0, 1.0, -1.0],
                          np.float32)
    rows = o.pack_kv(v)
    # RoPE part: numpy's IEEE binary16 conversion, bit for bit
    with np.errstate(over="ignore"):
        f16 = v[:, 448:].astype("<f2")
    assert np.array_equal(rows[:, 448:576], f16.view(np.uint8).reshape(n, 128)), "f16"
    # non-RoPE blocks: the scale byte by frexp, the codes by torch's E4M3
    for j in range(n):
        for b in range(7):
            x = v[j, 64 * b:64 * b + 64].astype(np.float64)
            amax = float(np.max(np.abs(x)))
            byte = 127 if amax == 0.0 else min(max(math.frexp(amax)[1] - 1 - 8 + 127, 0), 254)
            assert rows[j, 576 + b] == byte, ("e4m3 scale", j, b)
            y = x * 2.0 ** (127 - byte)
            want = lib_e4m3_code(np.clip(y, -448.0, 448.0))     # beyond 448: saturation
            want = np.where((want & 0x7F) == 0, 0, want)         # zeros stored as +0
            assert np.array_equal(rows[j, 64 * b:64 * b + 64].astype(np.int64), want), ("e4m3", j, b)
    # hand-worked E4M3 cases at scale byte 127 (block maximum in [256, 512))
    x = np.zeros((1, 512), np.float32)
    x[0, :9] = [480.0, 464.0, 1.0625, 1.1875, 0.0009765625, -0.00146484375, 300.0, -0.0009, -0.0029296875]
    r = o.pack_kv(x)
    assert r[0, 576] == 127
    # 480 and 464 saturate to 448 (0x7E); 1.0625 ties to 1.0 (0x38), 1.1875
    # to 1.25 (0x3A); 2^-10 ties between 0 and 2^-9 -> +0; -0.75 * 2^-9 ->
    # -2^-9 (0x81); 300 -> 288 = 2^8 * 1.125 (0x79); -0.0009 = -0.46 * 2^-9 ->
    # +0; -1.5 * 2^-9 ties between 2^-9 and 2^-8 -> -2^-8 (0x82)
    assert list(r[0, :9]) == [0x7E, 0x7E, 0x38, 0x3A, 0x00, 0x81, 0x79, 0x00, 0x82], list(r[0, :9])
    # the indexer format: exhaustive nearest-value search (zero block 127,
    # zeros as +0), and the generator's encoder (an independent
    # implementation of the same rule) on random rows
    vi = (rng.standard_normal((12, 128)) * 2.0 ** rng.integers(-40, 40, (12, 128))).astype(np.float32)
    vi[3, :32] = 0.0
    vi[4] = (rng.integers(-16, 17, 128) * 0.25).astype(np.float32)
    ri = o.pack_idx(vi)
    byte, codes = brute_force_fp4(vi)
    zero = np.max(np.abs(vi.reshape(-1, 32)), axis=1) == 0
    byte = np.where(zero, 127, byte)
    codes = np.where((codes & 7) == 0, 0, codes)
    assert np.array_equal(ri[:, 64:68].reshape(-1), byte), "idx scale"
    assert np.array_equal(unpack_codes(ri).reshape(-1, 32), codes), "idx codes"
    import gen as _gen
    g = _gen.lib()
    for j in range(4):
        gk = np.empty(583, np.uint8)
        g.csa_gen_pack_kv_row(np.ascontiguousarray(v[j]).ctypes.data, gk.ctypes.data)
        assert np.array_equal(gk, rows[j]), ("generator kv", j)
        gi = np.empty(68, np.uint8)
        g.csa_gen_pack_idx_row(np.ascontiguousarray(vi[j]).ctypes.data, gi.ctypes.data)
        assert np.array_equal(gi, ri[j]), ("generator idx", j)


def check_lse_merge(o) -> None:
    """Attention over two disjoint row sets merged equals attention over their
    union (an identity of the softmax); an empty side leaves the other."""
    rng = np.random.default_rng(23)
    rows = random_kv_rows(90, 8)
    scale = float(np.float32(1 / math.sqrt(512)))
    q = rng.standard_normal((5, 512)).astype(np.float32)
    sa = rng.permutation(90)
    A, B = sa[:50].astype(np.int32), sa[50:].astype(np.int32)
    oa, la = o.attention(rows, A, q, scale)
    ob, lb = o.attention(rows, B, q, scale)
    om, lm = o.lse_merge(oa, la, ob, lb)
    ref_o, ref_l = ref_attention(rows, np.concatenate([A, B]), q, scale)
    assert np.max(np.abs(om - ref_o)) <= 2e-6 * np.max(np.abs(ref_o)), "merge out"
    assert np.allclose(lm, ref_l, rtol=1e-6, atol=1e-6), "merge lse"
    # swapping the sides gives the same result
    om2, lm2 = o.lse_merge(ob, lb, oa, la)
    assert np.max(np.abs(om2 - om)) <= 1e-6 * np.max(np.abs(om)) and np.allclose(lm2, lm, rtol=1e-7, atol=1e-7)
    empty_o, empty_l = o.attention(rows, np.zeros(0, np.int32), q, scale)
    om, lm = o.lse_merge(oa, la, empty_o, empty_l)
    assert np.array_equal(om, oa) and np.array_equal(lm, la), "empty side"
    om, lm = o.lse_merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(om == 0) and np.all(np.isneginf(lm)), "both empty"


def check_score_topk_multi(o) -> None:
    """Each token's selection against float64 einsum scores and Python's
    sorted, over one shared history."""
    rng = np.random.default_rng(29)
    rows = random_idx_rows(700, 12)
    T, H, k = 3, 5, 40
    q = rng.standard_normal((T, H, 128)).astype(np.float32)
    w = rng.uniform(-1, 1, (T, H)).astype(np.float32)
    sel, sel_score = o.score_topk_multi(rows, q, w, k)
    for t in range(T):
        s = ref_score(rows, q[t], w[t])
        want = [j for _, j in sorted((-float(s[j]), j) for j in range(len(s)))][:k]
        assert list(sel[t]) == want, f"token {t}"
        assert np.array_equal(sel_score[t], s[want].astype(np.float32)), f"token {t} scores"


ALL_CHECKS = (check_tables, check_decode, check_score, check_topk, check_attention, check_decode_step,
              check_quantize_query, check_dense_attention, check_pack, check_lse_merge, check_score_topk_multi)
