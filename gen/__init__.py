"""Seeded synthetic workloads for the CSA decode step.

Test and benchmark infrastructure shared by the CPU oracle side and the HIP
side.  It draws the random inputs and encodes them into the packed row formats
(68-byte MXFP4 indexer rows, 583-byte E4M3/FP16/UE8M0 KV rows, as laid out in
the DS4X README, "Packed cache ABI").  It contains none of the decode step's
arithmetic.  The C source is ``gen/csa_gen.c``; ``build()`` compiles it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libcsagen.so")
IDX_ROW_BYTES = 68
KV_ROW_BYTES = 583


@dataclass(frozen=True)
class Workload:
    """One decode-step workload: rows per session, indexer heads, sessions."""

    cid: int
    name: str
    n_rows: int
    n_idx_heads: int
    n_sessions: int
    n_heads: int = 64
    topk: int = 512


# Rows are compressed CSA rows (one per four context tokens).
WORKLOADS = [
    Workload(0, "tiny-2k-rows", 2048, 8, 1),
    Workload(1, "mid-32k-rows", 32768, 64, 1),
    Workload(2, "long-256k-rows", 262144, 64, 1),
    Workload(3, "frontier-1m-rows", 1048576, 64, 1),
    Workload(4, "batch16-64k-rows", 65536, 64, 16),
]


def build(verbose: bool = False) -> str:
    """Compile ``libcsagen.so`` (always recompiles)."""
    src = os.path.join(_HERE, "csa_gen.c")
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, _SO)
    return _SO


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.csa_gen_seed.restype = u64
        L.csa_gen_seed.argtypes = [i32]
        L.csa_gen_u64.restype = u64
        L.csa_gen_u64.argtypes = [u64, u64, u64]
        L.csa_gen_normal.restype = ctypes.c_float
        L.csa_gen_normal.argtypes = [u64, u64, u64]
        L.csa_gen_uniform.restype = ctypes.c_float
        L.csa_gen_uniform.argtypes = [u64, u64, u64]
        L.csa_gen_pack_idx_row.argtypes = [vp, vp]
        L.csa_gen_pack_kv_row.argtypes = [vp, vp]
        L.csa_gen_f16_bits.restype = ctypes.c_uint16
        L.csa_gen_f16_bits.argtypes = [ctypes.c_float]
        L.csa_gen_e4m3_bits.restype = ctypes.c_uint8
        L.csa_gen_e4m3_bits.argtypes = [ctypes.c_double]
        L.csa_gen_idx_rows.argtypes = [u64, i32, i64, i64, vp]
        L.csa_gen_kv_rows.argtypes = [u64, i32, i64, i64, vp]
        L.csa_gen_queries.argtypes = [u64, i32, i32, i32, vp, vp, vp]
        L.csa_gen_fnv1a64.restype = u64
        L.csa_gen_fnv1a64.argtypes = [vp, i64]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def seed(cid: int) -> int:
    return int(lib().csa_gen_seed(cid))


def idx_rows(seed_: int, session: int, n: int, row0: int = 0) -> np.ndarray:
    out = np.empty((n, IDX_ROW_BYTES), dtype=np.uint8)
    if n:
        lib().csa_gen_idx_rows(seed_, session, row0, n, _ptr(out))
    return out


def kv_rows(seed_: int, session: int, n: int, row0: int = 0) -> np.ndarray:
    out = np.empty((n, KV_ROW_BYTES), dtype=np.uint8)
    if n:
        lib().csa_gen_kv_rows(seed_, session, row0, n, _ptr(out))
    return out


def queries(seed_: int, session: int, n_idx_heads: int, n_heads: int = 64):
    q_idx = np.empty((n_idx_heads, 128), dtype=np.float32)
    w_idx = np.empty((n_idx_heads,), dtype=np.float32)
    q_attn = np.empty((n_heads, 512), dtype=np.float32)
    lib().csa_gen_queries(seed_, session, n_idx_heads, n_heads, _ptr(q_idx), _ptr(w_idx), _ptr(q_attn))
    return q_idx, w_idx, q_attn


def session(cid: int, s: int = 0, n_rows: int | None = None, seed_: int | None = None,
            n_idx_heads: int | None = None, n_heads: int | None = None) -> dict:
    """All inputs of session ``s`` of workload ``cid`` (optionally truncated to
    ``n_rows`` rows -- the generator is prefix-stable)."""
    w = WORKLOADS[cid]
    sd = seed(cid) if seed_ is None else seed_
    n = w.n_rows if n_rows is None else n_rows
    hi = w.n_idx_heads if n_idx_heads is None else n_idx_heads
    ha = w.n_heads if n_heads is None else n_heads
    q_idx, w_idx, q_attn = queries(sd, s, hi, ha)
    return {
        "idx_rows": idx_rows(sd, s, n),
        "kv_rows": kv_rows(sd, s, n),
        "q_idx": q_idx,
        "w_idx": w_idx,
        "q_attn": q_attn,
        "softmax_scale": float(np.float32(1.0 / np.sqrt(512.0))),
    }


def pack_idx_row(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.shape == (128,)
    row = np.empty(IDX_ROW_BYTES, dtype=np.uint8)
    lib().csa_gen_pack_idx_row(_ptr(v), _ptr(row))
    return row


def pack_kv_row(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.shape == (512,)
    row = np.empty(KV_ROW_BYTES, dtype=np.uint8)
    lib().csa_gen_pack_kv_row(_ptr(v), _ptr(row))
    return row


def digest(a: np.ndarray) -> int:
    a = np.ascontiguousarray(a)
    return int(lib().csa_gen_fnv1a64(_ptr(a), a.nbytes))
