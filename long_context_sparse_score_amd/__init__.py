"""MI355X (gfx950) CSA decode step: Python binding of libcsa.so.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libcsa.so`` (C ABI in ``include/csa.h``).  PyTorch supplies device
memory and the current HIP stream.  There is no fallback: if the library is
missing or fails to load, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

IDX_ROW_BYTES = 68
KV_ROW_BYTES = 583
IDX_DIM = 128
KV_DIM = 512
TOPK = 512
MAX_HEADS = 64
MAX_SESSIONS = 64
ABI_VERSION = 2
STAGES = ("filter score + tile heads", "exact rescoring", "select + attention", "merge")
QUERY_FORMATS = {"fp32": 0, "mxfp4": 1}  # CSA_QUERY_FP32, CSA_QUERY_MXFP4

OK, EINVAL, EWORKSPACE, EDEVICE, EUNSUPPORTED = 0, -1, -2, -3, -4
SCRATCH_BYTES = 32 << 20  # CSA_SCRATCH_BYTES: the static workspace of csa_decode_step_noalloc


class CsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} ({status})")
        self.status = status


class Session(ctypes.Structure):
    """Mirror of ``csa_session`` in include/csa.h."""

    _fields_ = [
        ("idx_rows", ctypes.c_void_p),
        ("kv_rows", ctypes.c_void_p),
        ("n_rows", ctypes.c_int64),
        ("q_idx", ctypes.c_void_p),
        ("w_idx", ctypes.c_void_p),
        ("q_attn", ctypes.c_void_p),
        ("sel_idx", ctypes.c_void_p),
        ("sel_score", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.csa_abi_version.restype = ctypes.c_uint32
    L.csa_abi_version.argtypes = []
    L.csa_strerror.restype = ctypes.c_char_p
    L.csa_strerror.argtypes = [i32]
    L.csa_workspace_bytes.restype = sz
    L.csa_workspace_bytes.argtypes = [i64, i32]
    L.csa_score.restype = i32
    L.csa_score.argtypes = [vp, i64, vp, vp, i32, vp, vp, sz, vp]
    L.csa_score_bounds.restype = i32
    L.csa_score_bounds.argtypes = [vp, i64, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    L.csa_dense_workspace_bytes.restype = sz
    L.csa_dense_workspace_bytes.argtypes = [i64]
    L.csa_dense_attn.restype = i32
    L.csa_dense_attn.argtypes = [vp, i64, vp, i32, f32, vp, vp, vp, sz, vp]
    L.csa_score_topk_multi.restype = i32
    L.csa_score_topk_multi.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    L.csa_pack_rows.restype = i32
    L.csa_pack_rows.argtypes = [vp, vp, i64, vp, vp, vp]
    L.csa_lse_merge.restype = i32
    L.csa_lse_merge.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp]
    L.csa_quantize_query.restype = i32
    L.csa_quantize_query.argtypes = [vp, i32, vp, vp]
    L.csa_decode_step_ex.restype = i32
    L.csa_decode_step_ex.argtypes = [ctypes.POINTER(Session), i32, i32, i32, f32, i32, vp, sz, vp, vp]
    L.csa_topk.restype = i32
    L.csa_topk.argtypes = [vp, i64, i32, vp, vp, vp, sz, vp]
    L.csa_sparse_attn.restype = i32
    L.csa_sparse_attn.argtypes = [vp, i64, vp, i32, vp, i32, f32, vp, vp, vp, sz, vp]
    L.csa_decode_step.restype = i32
    L.csa_decode_step.argtypes = [ctypes.POINTER(Session), i32, i32, i32, f32, vp, sz, vp]
    L.csa_decode_step_noalloc.restype = i32
    L.csa_decode_step_noalloc.argtypes = [ctypes.POINTER(Session), i32, i32, i32, f32, vp]
    L.csa_decode_step_timed.restype = i32
    L.csa_decode_step_timed.argtypes = [ctypes.POINTER(Session), i32, i32, i32, f32, vp, sz, vp,
                                        ctypes.POINTER(ctypes.c_void_p)]
    L.csa_dequant_idx.restype = i32
    L.csa_dequant_idx.argtypes = [vp, i64, vp, vp]
    L.csa_dequant_kv.restype = i32
    L.csa_dequant_kv.argtypes = [vp, i64, vp, vp]
    if L.csa_abi_version() != ABI_VERSION:
        raise ImportError(f"libcsa.so ABI {L.csa_abi_version()} != {ABI_VERSION}")
    return L


lib = _load()


def strerror(status: int) -> str:
    return lib.csa_strerror(status).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise CsaError(status, where)


def _ptr(t: torch.Tensor | None, dtype: torch.dtype | None = None, name: str = "") -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr() if t.numel() else None


def _rows(t: torch.Tensor, width: int, name: str) -> int:
    """A packed row buffer [n][width] of bytes; returns n.  Checked on the host
    so that a mis-shaped buffer is refused before any launch."""
    if t.dtype != torch.uint8 or t.dim() != 2 or t.shape[1] != width:
        raise ValueError(f"{name}: expected a uint8 tensor of shape [n, {width}], got {t.dtype} {tuple(t.shape)}")
    return int(t.shape[0])


def _mat(t: torch.Tensor, cols: int, name: str, rows: int | None = None) -> int:
    """A float32 matrix [rows][cols]; returns its row count."""
    if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != cols or (rows is not None and t.shape[0] != rows):
        want = f"[{rows if rows is not None else 'h'}, {cols}]"
        raise ValueError(f"{name}: expected a float32 tensor of shape {want}, got {t.dtype} {tuple(t.shape)}")
    return int(t.shape[0])


def _vec(t: torch.Tensor, n: int, name: str, dtype=torch.float32) -> None:
    if t.dtype != dtype or t.dim() != 1 or t.shape[0] != n:
        raise ValueError(f"{name}: expected a {dtype} vector of length {n}, got {t.dtype} {tuple(t.shape)}")


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def workspace_bytes(max_rows_per_session: int, n_sessions: int = 1) -> int:
    return int(lib.csa_workspace_bytes(max_rows_per_session, n_sessions))


def alloc_workspace(max_rows_per_session: int, n_sessions: int = 1, device="cuda") -> torch.Tensor:
    nb = workspace_bytes(max_rows_per_session, n_sessions)
    if nb == 0:
        raise ValueError("workspace size out of range")
    return torch.empty(nb, dtype=torch.uint8, device=device)  # caching allocator: 256-B aligned


def score(idx_rows: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor, scores: torch.Tensor | None = None,
          ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    n = _rows(idx_rows, IDX_ROW_BYTES, "idx_rows")
    h = _mat(q_idx, IDX_DIM, "q_idx")
    _vec(w_idx, h, "w_idx")
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=idx_rows.device)
    _vec(scores, n, "scores")
    if ws is None:
        ws = alloc_workspace(n, 1, idx_rows.device)
    _check(lib.csa_score(_ptr(idx_rows, torch.uint8, "idx_rows"), n, _ptr(q_idx, torch.float32, "q_idx"),
                         _ptr(w_idx, torch.float32, "w_idx"), h, _ptr(scores, torch.float32, "scores"),
                         _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "csa_score")
    return scores


def _format(query_format: str) -> int:
    if query_format not in QUERY_FORMATS:
        raise ValueError(f"query_format: one of {sorted(QUERY_FORMATS)}, got {query_format!r}")
    return QUERY_FORMATS[query_format]


def score_bounds(idx_rows: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor, ws: torch.Tensor | None = None,
                 stream=None, query_format: str = "fp32"):
    """The decode step's filter: (upper, lower) with lower <= score <= upper
    for every row (csa_score_bounds; with query_format="mxfp4" the score of
    the quantized query)."""
    fmt = _format(query_format)
    n = _rows(idx_rows, IDX_ROW_BYTES, "idx_rows")
    h = _mat(q_idx, IDX_DIM, "q_idx")
    _vec(w_idx, h, "w_idx")
    up = torch.empty(n, dtype=torch.float32, device=idx_rows.device)
    lo = torch.empty(n, dtype=torch.float32, device=idx_rows.device)
    if ws is None:
        ws = alloc_workspace(n, 1, idx_rows.device)
    _check(lib.csa_score_bounds(_ptr(idx_rows, torch.uint8, "idx_rows"), n, _ptr(q_idx, torch.float32, "q_idx"),
                                _ptr(w_idx, torch.float32, "w_idx"), h, fmt, _ptr(up), _ptr(lo),
                                _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "csa_score_bounds")
    return up, lo


def quantize_query(q_idx: torch.Tensor, stream=None) -> torch.Tensor:
    """The indexer query [h][128] quantized to MXFP4, packed as rows [h][68]
    (csa_quantize_query)."""
    h = _mat(q_idx, IDX_DIM, "q_idx")
    rows = torch.empty((h, IDX_ROW_BYTES), dtype=torch.uint8, device=q_idx.device)
    _check(lib.csa_quantize_query(_ptr(q_idx, torch.float32, "q_idx"), h, _ptr(rows, torch.uint8), _stream(stream)),
           "csa_quantize_query")
    return rows


def topk(scores: torch.Tensor, k: int = TOPK, ws: torch.Tensor | None = None, stream=None):
    if scores.dtype != torch.float32 or scores.dim() != 1:
        raise ValueError(f"scores: expected a float32 vector, got {scores.dtype} {tuple(scores.shape)}")
    n = int(scores.shape[0])
    if ws is None:
        ws = alloc_workspace(n, 1, scores.device)
    sel = torch.empty(k, dtype=torch.int32, device=scores.device)
    sel_score = torch.empty(k, dtype=torch.float32, device=scores.device)
    _check(lib.csa_topk(_ptr(scores, torch.float32, "scores"), n, k, _ptr(sel, torch.int32), _ptr(sel_score),
                        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "csa_topk")
    return sel, sel_score


def sparse_attn(kv_rows: torch.Tensor, sel_idx: torch.Tensor, n_sel: int, q_attn: torch.Tensor, softmax_scale: float,
                ws: torch.Tensor | None = None, stream=None):
    n_rows = _rows(kv_rows, KV_ROW_BYTES, "kv_rows")
    h = _mat(q_attn, KV_DIM, "q_attn")
    if sel_idx.dtype != torch.int32 or sel_idx.dim() != 1 or not 0 <= n_sel <= min(TOPK, sel_idx.shape[0]):
        raise ValueError(f"sel_idx: expected an int32 vector holding n_sel={n_sel} <= {TOPK} entries, "
                         f"got {sel_idx.dtype} {tuple(sel_idx.shape)}")
    dev = q_attn.device
    if ws is None:
        ws = alloc_workspace(0, 1, dev)
    out = torch.empty((h, KV_DIM), dtype=torch.float32, device=dev)
    lse = torch.empty(h, dtype=torch.float32, device=dev)
    _check(lib.csa_sparse_attn(_ptr(kv_rows, torch.uint8, "kv_rows"), n_rows, _ptr(sel_idx, torch.int32, "sel"),
                               n_sel, _ptr(q_attn, torch.float32, "q_attn"), h, softmax_scale, _ptr(out), _ptr(lse),
                               _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "csa_sparse_attn")
    return out, lse


DENSE_MAX_ROWS = 1 << 17  # CSA_DENSE_MAX_ROWS


def dense_attn(kv_rows: torch.Tensor, q_attn: torch.Tensor, softmax_scale: float, ws: torch.Tensor | None = None,
               out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
    """Softmax attention over every KV row (csa_dense_attn)."""
    n = _rows(kv_rows, KV_ROW_BYTES, "kv_rows")
    if n > DENSE_MAX_ROWS:
        raise ValueError(f"kv_rows: at most {DENSE_MAX_ROWS} rows, got {n}")
    h = _mat(q_attn, KV_DIM, "q_attn")
    dev = q_attn.device
    if ws is None:
        ws = torch.empty(int(lib.csa_dense_workspace_bytes(n)), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((h, KV_DIM), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(h, dtype=torch.float32, device=dev)
    _mat(out, KV_DIM, "out", h)
    _vec(lse, h, "lse")
    _check(lib.csa_dense_attn(_ptr(kv_rows, torch.uint8, "kv_rows"), n, _ptr(q_attn, torch.float32, "q_attn"), h,
                              softmax_scale, _ptr(out, torch.float32), _ptr(lse, torch.float32),
                              _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "csa_dense_attn")
    return out, lse


def score_topk_multi(idx_rows: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor, k: int = TOPK,
                     ws: torch.Tensor | None = None, stream=None):
    """Exact top-k of every token's scores over one history
    (csa_score_topk_multi): q_idx [T][H][128], w_idx [T][H] -> (sel [T][k],
    sel_score [T][k])."""
    n = _rows(idx_rows, IDX_ROW_BYTES, "idx_rows")
    if q_idx.dim() != 3 or q_idx.shape[2] != IDX_DIM or w_idx.dim() != 2 or tuple(w_idx.shape) != tuple(q_idx.shape[:2]):
        raise ValueError(f"q_idx [T][H][128] and w_idx [T][H] expected, got {tuple(q_idx.shape)} {tuple(w_idx.shape)}")
    T, H = int(q_idx.shape[0]), int(q_idx.shape[1])
    dev = idx_rows.device
    if ws is None:
        ws = alloc_workspace(n, T, dev)
    sel = torch.empty((T, k), dtype=torch.int32, device=dev)
    sel_score = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib.csa_score_topk_multi(_ptr(idx_rows, torch.uint8, "idx_rows"), n, _ptr(q_idx, torch.float32, "q_idx"),
                                    _ptr(w_idx, torch.float32, "w_idx"), T, H, k, _ptr(sel), _ptr(sel_score),
                                    _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "csa_score_topk_multi")
    return sel, sel_score


def pack_rows(kv_vals: torch.Tensor | None = None, idx_vals: torch.Tensor | None = None, kv_rows=None, idx_rows=None,
              stream=None):
    """New rows in the packed formats (csa_pack_rows): kv_vals [n][512] ->
    583-byte rows, idx_vals [n][128] -> 68-byte rows.  Returns (kv_rows,
    idx_rows) (None where no values were given)."""
    if kv_vals is None and idx_vals is None:
        raise ValueError("pack_rows: kv_vals or idx_vals")
    n = None
    if kv_vals is not None:
        n = _mat(kv_vals, KV_DIM, "kv_vals")
        if kv_rows is None:
            kv_rows = torch.empty((n, KV_ROW_BYTES), dtype=torch.uint8, device=kv_vals.device)
        if _rows(kv_rows, KV_ROW_BYTES, "kv_rows") < n:
            raise ValueError("kv_rows: fewer rows than kv_vals")
    if idx_vals is not None:
        ni = _mat(idx_vals, IDX_DIM, "idx_vals")
        if n is not None and ni != n:
            raise ValueError("kv_vals and idx_vals disagree on the row count")
        n = ni
        if idx_rows is None:
            idx_rows = torch.empty((n, IDX_ROW_BYTES), dtype=torch.uint8, device=idx_vals.device)
        if _rows(idx_rows, IDX_ROW_BYTES, "idx_rows") < n:
            raise ValueError("idx_rows: fewer rows than idx_vals")
    if n == 0:
        return kv_rows, idx_rows
    _check(lib.csa_pack_rows(_ptr(kv_vals, torch.float32, "kv_vals"), _ptr(idx_vals, torch.float32, "idx_vals"), n,
                             _ptr(kv_rows, torch.uint8, "kv_rows"), _ptr(idx_rows, torch.uint8, "idx_rows"),
                             _stream(stream)), "csa_pack_rows")
    return kv_rows, idx_rows


def lse_merge(out_a: torch.Tensor, lse_a: torch.Tensor, out_b: torch.Tensor, lse_b: torch.Tensor, stream=None):
    """The attention over the union of two disjoint row sets from their two
    results (csa_lse_merge)."""
    h = _mat(out_a, KV_DIM, "out_a")
    _mat(out_b, KV_DIM, "out_b", h)
    _vec(lse_a, h, "lse_a")
    _vec(lse_b, h, "lse_b")
    out = torch.empty_like(out_a)
    lse = torch.empty_like(lse_a)
    _check(lib.csa_lse_merge(_ptr(out_a, torch.float32), _ptr(lse_a, torch.float32), _ptr(out_b, torch.float32),
                             _ptr(lse_b, torch.float32), h, _ptr(out), _ptr(lse), _stream(stream)), "csa_lse_merge")
    return out, lse


class DecodeStep:
    """Pre-marshalled csa_decode_step over fixed device buffers.

    ``sessions`` is a sequence of dicts with device tensors ``idx_rows``,
    ``kv_rows``, ``q_idx``, ``w_idx``, ``q_attn``; outputs ``sel``,
    ``sel_score``, ``out``, ``lse`` are allocated here.  ``__call__`` enqueues
    one decode step of every session on the current stream.  With
    ``noalloc=True`` no workspace is allocated and ``__call__`` runs
    csa_decode_step_noalloc (the library's static per-device workspace).
    ``query_format="mxfp4"`` scores the MXFP4-quantized indexer query
    (csa_decode_step_ex).
    """

    def __init__(self, sessions: Sequence[dict], softmax_scale: float, ws: torch.Tensor | None = None,
                 noalloc: bool = False, query_format: str = "fp32"):
        if not 1 <= len(sessions) <= MAX_SESSIONS:
            raise ValueError("1..64 sessions")
        self.sessions = list(sessions)
        self.n_idx_heads = _mat(sessions[0]["q_idx"], IDX_DIM, "q_idx")
        self.n_heads = _mat(sessions[0]["q_attn"], KV_DIM, "q_attn")
        if not (1 <= self.n_idx_heads <= MAX_HEADS and 1 <= self.n_heads <= MAX_HEADS):
            raise ValueError("1..64 indexer and attention heads")
        self.softmax_scale = float(softmax_scale)
        self.noalloc = bool(noalloc)
        self.query_format = _format(query_format)
        if self.noalloc and self.query_format != QUERY_FORMATS["fp32"]:
            raise ValueError("the no-allocation entry point scores the fp32 query only")
        dev = sessions[0]["q_attn"].device
        max_rows = max(_rows(s["idx_rows"], IDX_ROW_BYTES, "idx_rows") for s in sessions)
        if self.noalloc:
            self.ws = None
        else:
            self.ws = alloc_workspace(max_rows, len(sessions), dev) if ws is None else ws
        arr = (Session * len(sessions))()
        for i, s in enumerate(self.sessions):
            n = _rows(s["idx_rows"], IDX_ROW_BYTES, "idx_rows")
            if _rows(s["kv_rows"], KV_ROW_BYTES, "kv_rows") != n:
                raise ValueError("idx_rows and kv_rows disagree on n_rows")
            _mat(s["q_idx"], IDX_DIM, "q_idx", self.n_idx_heads)
            _vec(s["w_idx"], self.n_idx_heads, "w_idx")
            _mat(s["q_attn"], KV_DIM, "q_attn", self.n_heads)
            s.setdefault("sel", torch.empty(TOPK, dtype=torch.int32, device=dev))
            s.setdefault("sel_score", torch.empty(TOPK, dtype=torch.float32, device=dev))
            s.setdefault("out", torch.empty((self.n_heads, KV_DIM), dtype=torch.float32, device=dev))
            s.setdefault("lse", torch.empty(self.n_heads, dtype=torch.float32, device=dev))
            arr[i] = Session(_ptr(s["idx_rows"], torch.uint8, "idx_rows"), _ptr(s["kv_rows"], torch.uint8, "kv_rows"), n,
                             _ptr(s["q_idx"], torch.float32, "q_idx"), _ptr(s["w_idx"], torch.float32, "w_idx"),
                             _ptr(s["q_attn"], torch.float32, "q_attn"), _ptr(s["sel"], torch.int32, "sel"),
                             _ptr(s["sel_score"], torch.float32), _ptr(s["out"], torch.float32),
                             _ptr(s["lse"], torch.float32))
            _vec(s["sel"], TOPK, "sel", torch.int32)
            _vec(s["sel_score"], TOPK, "sel_score")
            _mat(s["out"], KV_DIM, "out", self.n_heads)
            _vec(s["lse"], self.n_heads, "lse")
        self._arr = arr

    def __call__(self, stream=None) -> None:
        if self.noalloc:
            _check(lib.csa_decode_step_noalloc(self._arr, len(self.sessions), self.n_idx_heads, self.n_heads,
                                               self.softmax_scale, _stream(stream)), "csa_decode_step_noalloc")
            return
        if self.query_format != QUERY_FORMATS["fp32"]:
            _check(lib.csa_decode_step_ex(self._arr, len(self.sessions), self.n_idx_heads, self.n_heads,
                                          self.softmax_scale, self.query_format, _ptr(self.ws, torch.uint8, "ws"),
                                          self.ws.numel(), _stream(stream), None), "csa_decode_step_ex")
            return
        _check(lib.csa_decode_step(self._arr, len(self.sessions), self.n_idx_heads, self.n_heads, self.softmax_scale,
                                   _ptr(self.ws, torch.uint8, "ws"), self.ws.numel(), _stream(stream)),
               "csa_decode_step")

    def timed(self, events: Sequence["torch.cuda.Event"], stream=None) -> None:
        """Same work as ``__call__`` (with a workspace); records ``events[2s]`` /
        ``events[2s+1]`` around stage s (STAGES) on the stream."""
        if self.ws is None:
            raise ValueError("timed steps need a workspace (noalloc=False)")
        if len(events) != 2 * len(STAGES):
            raise ValueError(f"need {2 * len(STAGES)} events")
        for e in events:
            if not e.cuda_event:  # torch creates the HIP event on its first record
                e.record()
        handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        _check(lib.csa_decode_step_ex(self._arr, len(self.sessions), self.n_idx_heads, self.n_heads,
                                      self.softmax_scale, self.query_format, _ptr(self.ws, torch.uint8, "ws"),
                                      self.ws.numel(), _stream(stream), handles), "csa_decode_step_ex")


def decode_step(sessions: Sequence[dict], softmax_scale: float, ws: torch.Tensor | None = None, stream=None,
                query_format: str = "fp32"):
    """One decode step over ``sessions`` (see DecodeStep); returns the session dicts with outputs."""
    step = DecodeStep(sessions, softmax_scale, ws, query_format=query_format)
    step(stream)
    return step.sessions


def dequant_idx(idx_rows: torch.Tensor, stream=None) -> torch.Tensor:
    n = idx_rows.shape[0]
    out = torch.empty((n, IDX_DIM), dtype=torch.float32, device=idx_rows.device)
    _check(lib.csa_dequant_idx(_ptr(idx_rows, torch.uint8, "idx_rows"), n, _ptr(out), _stream(stream)), "csa_dequant_idx")
    return out


def dequant_kv(kv_rows: torch.Tensor, stream=None) -> torch.Tensor:
    n = kv_rows.shape[0]
    out = torch.empty((n, KV_DIM), dtype=torch.float32, device=kv_rows.device)
    _check(lib.csa_dequant_kv(_ptr(kv_rows, torch.uint8, "kv_rows"), n, _ptr(out), _stream(stream)), "csa_dequant_kv")
    return out
