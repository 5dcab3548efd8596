"""CPU oracle of the CSA decode step (numpy wrapper over ``csa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  The C source builds
its own decode tables from the OCP MX v1.0 / IEEE 754 definitions and shares
nothing with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "csa_oracle.c")
SO = os.path.join(_HERE, "libcsa_oracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(src: str = SRC, out: str = SO, verbose: bool = False) -> str:
    """Compile the oracle (always recompiles).  ``src``/``out`` let a test
    build a modified copy of the source elsewhere."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, "-I", _HERE, src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes binding of one compiled oracle library."""

    def __init__(self, so_path: str = SO):
        if so_path == SO and not os.path.exists(SO):
            build()
        L = ctypes.CDLL(so_path)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        for name in ("csa_oracle_e2m1", "csa_oracle_e4m3", "csa_oracle_ue8m0", "csa_oracle_f16"):
            getattr(L, name).restype = dbl
            getattr(L, name).argtypes = [i32]
        L.csa_oracle_decode_idx_rows.argtypes = [vp, i64, vp]
        L.csa_oracle_decode_kv_rows.argtypes = [vp, i64, vp]
        L.csa_oracle_score.argtypes = [vp, i64, vp, vp, i32, vp]
        L.csa_oracle_topk.restype = i64
        L.csa_oracle_topk.argtypes = [vp, i64, i32, vp, vp]
        L.csa_oracle_attention.restype = i32
        L.csa_oracle_attention.argtypes = [vp, i64, vp, i32, vp, i32, dbl, vp, vp]
        L.csa_oracle_quantize_query.argtypes = [vp, i32, vp]
        L.csa_oracle_score_topk_multi.restype = i32
        L.csa_oracle_score_topk_multi.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp]
        L.csa_oracle_pack_kv_rows.argtypes = [vp, i64, vp]
        L.csa_oracle_pack_idx_rows.argtypes = [vp, i64, vp]
        L.csa_oracle_lse_merge.argtypes = [vp, vp, vp, vp, i32, vp, vp]
        L.csa_oracle_dense_attention.restype = i32
        L.csa_oracle_dense_attention.argtypes = [vp, i64, vp, i32, dbl, vp, vp]
        L.csa_oracle_decode_step.restype = i32
        L.csa_oracle_decode_step.argtypes = [vp, vp, i64, vp, vp, i32, vp, i32, dbl, i32, vp, vp, vp, vp]
        self.L = L

    # -- tables
    def e2m1(self, code: int) -> float:
        return self.L.csa_oracle_e2m1(code)

    def e4m3(self, code: int) -> float:
        return self.L.csa_oracle_e4m3(code)

    def ue8m0(self, b: int) -> float:
        return self.L.csa_oracle_ue8m0(b)

    def f16(self, bits: int) -> float:
        return self.L.csa_oracle_f16(bits)

    # -- row decode
    def decode_idx(self, rows: np.ndarray) -> np.ndarray:
        rows = _rows(rows, 68)
        out = np.empty((rows.shape[0], 128), dtype=np.float32)
        self.L.csa_oracle_decode_idx_rows(_p(rows), rows.shape[0], _p(out))
        return out

    def decode_kv(self, rows: np.ndarray) -> np.ndarray:
        rows = _rows(rows, 583)
        out = np.empty((rows.shape[0], 512), dtype=np.float32)
        self.L.csa_oracle_decode_kv_rows(_p(rows), rows.shape[0], _p(out))
        return out

    # -- MXFP4 query
    def quantize_query(self, q) -> np.ndarray:
        """The query [h][128] quantized to MXFP4, packed as indexer rows [h][68]."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        assert q.ndim == 2 and q.shape[1] == 128
        rows = np.empty((q.shape[0], 68), dtype=np.uint8)
        self.L.csa_oracle_quantize_query(_p(q), q.shape[0], _p(rows))
        return rows

    def quantized_query(self, q) -> np.ndarray:
        """The MXFP4 query decoded back to fp32 (the query the quantized-query
        scorer scores with)."""
        return self.decode_idx(self.quantize_query(q))

    # -- score / select / attend
    def score(self, idx_rows, q_idx, w_idx) -> np.ndarray:
        idx_rows = _rows(idx_rows, 68)
        q_idx = np.ascontiguousarray(q_idx, dtype=np.float32)
        w_idx = np.ascontiguousarray(w_idx, dtype=np.float32)
        h = w_idx.shape[0]
        assert q_idx.shape == (h, 128)
        out = np.empty(idx_rows.shape[0], dtype=np.float32)
        self.L.csa_oracle_score(_p(idx_rows), idx_rows.shape[0], _p(q_idx), _p(w_idx), h, _p(out))
        return out

    def topk(self, scores, k: int = 512):
        scores = np.ascontiguousarray(scores, dtype=np.float32)
        sel = np.empty(k, dtype=np.int32)
        sel_score = np.empty(k, dtype=np.float32)
        k_eff = self.L.csa_oracle_topk(_p(scores), scores.shape[0], k, _p(sel), _p(sel_score))
        if k_eff < 0:
            raise MemoryError("oracle top-k")
        return sel, sel_score, int(k_eff)

    def attention(self, kv_rows, sel, q_attn, softmax_scale: float):
        kv_rows = _rows(kv_rows, 583)
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        q_attn = np.ascontiguousarray(q_attn, dtype=np.float32)
        h = q_attn.shape[0]
        assert q_attn.shape == (h, 512)
        out = np.empty((h, 512), dtype=np.float32)
        lse = np.empty(h, dtype=np.float32)
        rc = self.L.csa_oracle_attention(_p(kv_rows), kv_rows.shape[0], _p(sel), sel.shape[0], _p(q_attn), h,
                                         float(softmax_scale), _p(out), _p(lse))
        if rc != 0:
            raise ValueError(f"oracle attention failed ({rc})")
        return out, lse

    def score_topk_multi(self, idx_rows, q_idx, w_idx, k: int = 512):
        """Each token's exact top-k over the same rows: q_idx [T][H][128],
        w_idx [T][H] -> (sel [T][k], sel_score [T][k])."""
        idx_rows = _rows(idx_rows, 68)
        q_idx = np.ascontiguousarray(q_idx, dtype=np.float32)
        w_idx = np.ascontiguousarray(w_idx, dtype=np.float32)
        T, H = w_idx.shape
        assert q_idx.shape == (T, H, 128)
        sel = np.empty((T, k), dtype=np.int32)
        sel_score = np.empty((T, k), dtype=np.float32)
        rc = self.L.csa_oracle_score_topk_multi(_p(idx_rows), idx_rows.shape[0], _p(q_idx), _p(w_idx), T, H, k,
                                                _p(sel), _p(sel_score))
        if rc != 0:
            raise MemoryError("oracle multi-token top-k")
        return sel, sel_score

    def pack_kv(self, v) -> np.ndarray:
        """Rows of 512 values packed into 583-byte KV rows."""
        v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1, 512)
        rows = np.empty((v.shape[0], 583), dtype=np.uint8)
        self.L.csa_oracle_pack_kv_rows(_p(v), v.shape[0], _p(rows))
        return rows

    def pack_idx(self, v) -> np.ndarray:
        """Rows of 128 values packed into 68-byte indexer rows."""
        v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1, 128)
        rows = np.empty((v.shape[0], 68), dtype=np.uint8)
        self.L.csa_oracle_pack_idx_rows(_p(v), v.shape[0], _p(rows))
        return rows

    def lse_merge(self, out_a, lse_a, out_b, lse_b):
        """The merge of two attention results over disjoint rows."""
        out_a, out_b = (np.ascontiguousarray(x, dtype=np.float32) for x in (out_a, out_b))
        lse_a, lse_b = (np.ascontiguousarray(x, dtype=np.float32) for x in (lse_a, lse_b))
        h = lse_a.shape[0]
        out = np.empty((h, 512), dtype=np.float32)
        lse = np.empty(h, dtype=np.float32)
        self.L.csa_oracle_lse_merge(_p(out_a), _p(lse_a), _p(out_b), _p(lse_b), h, _p(out), _p(lse))
        return out, lse

    def dense_attention(self, kv_rows, q_attn, softmax_scale: float):
        """Softmax attention over every row."""
        kv_rows = _rows(kv_rows, 583)
        q_attn = np.ascontiguousarray(q_attn, dtype=np.float32)
        h = q_attn.shape[0]
        assert q_attn.shape == (h, 512)
        out = np.empty((h, 512), dtype=np.float32)
        lse = np.empty(h, dtype=np.float32)
        rc = self.L.csa_oracle_dense_attention(_p(kv_rows), kv_rows.shape[0], _p(q_attn), h, float(softmax_scale),
                                               _p(out), _p(lse))
        if rc != 0:
            raise ValueError(f"oracle dense attention failed ({rc})")
        return out, lse

    def decode_step(self, idx_rows, kv_rows, q_idx, w_idx, q_attn, softmax_scale: float, k: int = 512):
        idx_rows = _rows(idx_rows, 68)
        kv_rows = _rows(kv_rows, 583)
        n = idx_rows.shape[0]
        assert kv_rows.shape[0] == n
        q_idx = np.ascontiguousarray(q_idx, dtype=np.float32)
        w_idx = np.ascontiguousarray(w_idx, dtype=np.float32)
        q_attn = np.ascontiguousarray(q_attn, dtype=np.float32)
        hi, ha = w_idx.shape[0], q_attn.shape[0]
        sel = np.empty(k, dtype=np.int32)
        sel_score = np.empty(k, dtype=np.float32)
        out = np.empty((ha, 512), dtype=np.float32)
        lse = np.empty(ha, dtype=np.float32)
        rc = self.L.csa_oracle_decode_step(_p(idx_rows), _p(kv_rows), n, _p(q_idx), _p(w_idx), hi, _p(q_attn), ha,
                                           float(softmax_scale), k, _p(sel), _p(sel_score), _p(out), _p(lse))
        if rc != 0:
            raise ValueError(f"oracle decode step failed ({rc})")
        return {"sel": sel, "sel_score": sel_score, "out": out, "lse": lse, "k_eff": min(k, n)}


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _rows(a, width: int) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint8)
    if a.ndim == 1:
        a = a.reshape(-1, width)
    assert a.ndim == 2 and a.shape[1] == width, a.shape
    return a


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
