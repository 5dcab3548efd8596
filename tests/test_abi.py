"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host (no compute call: these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


@pytest.fixture(scope="module")
def csa():
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "_csa_build", os.path.join(ROOT, "long_context_sparse_score_amd", "_build.py"))
    _build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(_build)  # by path: the package import needs the library
    if not os.path.exists(_build.LIB):
        _build.build()
    import long_context_sparse_score_amd as m

    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("csa_score", "csa_topk", "csa_sparse_attn", "csa_decode_step", "csa_workspace_bytes",
              "csa_abi_version", "csa_strerror"):
        assert f in names


def test_every_declared_symbol_is_exported(csa):
    lib = ctypes.CDLL(csa.LIB_PATH)
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing


def test_constants_match_header(csa):
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (CSA_[A-Z_0-9]+) (\d+)u?\b", text))
    assert int(consts["CSA_IDX_ROW_BYTES"]) == csa.IDX_ROW_BYTES == 68
    assert int(consts["CSA_KV_ROW_BYTES"]) == csa.KV_ROW_BYTES == 583
    assert int(consts["CSA_TOPK"]) == csa.TOPK == 512
    assert int(consts["CSA_ABI_VERSION"]) == csa.lib.csa_abi_version() == csa.ABI_VERSION
    assert int(consts["CSA_STAGES"]) == len(csa.STAGES)
    assert int(consts["CSA_QUERY_FP32"]) == csa.QUERY_FORMATS["fp32"]
    assert int(consts["CSA_QUERY_MXFP4"]) == csa.QUERY_FORMATS["mxfp4"]


def test_strerror_and_workspace(csa):
    for st in (0, -1, -2, -3, -4):
        assert csa.strerror(st) and csa.strerror(st) != "unknown status"
    assert csa.strerror(-99) == "unknown status"
    assert csa.workspace_bytes(0, 1) > 0
    assert csa.workspace_bytes(1 << 20, 1) >= (1 << 20) * 4
    assert csa.workspace_bytes(1 << 20, 16) > csa.workspace_bytes(1 << 20, 1)
    assert csa.workspace_bytes(1 << 20, 1) % 256 == 0
    assert csa.workspace_bytes(-1, 1) == 0
    assert csa.workspace_bytes(10, 0) == 0 and csa.workspace_bytes(10, 65) == 0
    assert csa.workspace_bytes((1 << 30) + 1, 1) == 0


def test_invalid_arguments_rejected_on_host(csa):
    L = csa.lib
    fake = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    assert L.csa_score(fake, 10, fake, fake, 0, fake, fake, 1 << 30, None) == csa.EINVAL  # 0 heads
    assert L.csa_score(fake, 10, fake, fake, 65, fake, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score(None, 10, fake, fake, 8, fake, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score(fake, -1, fake, fake, 8, fake, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score(fake, 10, fake, fake, 8, fake, fake, 16, None) == csa.EWORKSPACE
    odd = ctypes.c_void_p(4096 + 4)  # indexer rows must be 16-byte aligned
    assert L.csa_score(odd, 10, fake, fake, 8, fake, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score(fake, 10, odd, fake, 8, fake, fake, 1 << 30, None) == csa.EINVAL  # so must the query
    assert L.csa_topk(fake, 10, 0, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_topk(fake, 10, 513, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_topk(fake, 10, 8, None, None, fake, 1 << 30, None) == csa.EINVAL
    # workspace: too small, misaligned, missing
    assert L.csa_topk(fake, 10, 8, fake, None, fake, 16, None) == csa.EWORKSPACE
    assert L.csa_topk(fake, 10, 8, fake, None, ctypes.c_void_p(4096 + 8), 1 << 30, None) == csa.EWORKSPACE
    assert L.csa_topk(fake, 10, 8, fake, None, None, 1 << 30, None) == csa.EWORKSPACE
    assert L.csa_sparse_attn(fake, 10, fake, 513, fake, 8, 0.1, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_sparse_attn(fake, 10, fake, 4, fake, 0, 0.1, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_sparse_attn(fake, 10, None, 4, fake, 8, 0.1, fake, None, fake, 1 << 30, None) == csa.EINVAL
    sess = (csa.Session * 2)()
    assert L.csa_decode_step(sess, 0, 8, 64, 0.1, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_decode_step(sess, 65, 8, 64, 0.1, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_decode_step(sess, 2, 8, 64, 0.1, fake, 1 << 30, None) == csa.EINVAL  # null members
    assert L.csa_decode_step(None, 1, 8, 64, 0.1, fake, 1 << 30, None) == csa.EINVAL
    for i in range(2):
        sess[i] = csa.Session(fake, fake, 100, fake, fake, fake, fake, None, fake, None)
    assert L.csa_decode_step(sess, 2, 8, 0, 0.1, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_decode_step(sess, 2, 8, 64, 0.1, fake, 64, None) == csa.EWORKSPACE
    sess[1] = csa.Session(odd, fake, 100, fake, fake, fake, fake, None, fake, None)
    assert L.csa_decode_step(sess, 2, 8, 64, 0.1, fake, 1 << 30, None) == csa.EINVAL
    sess[1] = csa.Session(fake, fake, 100, odd, fake, fake, fake, None, fake, None)
    assert L.csa_decode_step(sess, 2, 8, 64, 0.1, fake, 1 << 30, None) == csa.EINVAL
    # the query-format entry points: unknown formats, bad queries, missing events
    for i in range(2):
        sess[i] = csa.Session(fake, fake, 100, fake, fake, fake, fake, None, fake, None)
    for fmt in (-1, 2, 7):
        assert L.csa_decode_step_ex(sess, 2, 8, 64, 0.1, fmt, fake, 1 << 30, None, None) == csa.EINVAL
        assert L.csa_score_bounds(fake, 10, fake, fake, 8, fmt, fake, fake, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_decode_step_ex(sess, 2, 8, 64, 0.1, 1, fake, 64, None, None) == csa.EWORKSPACE
    no_events = (ctypes.c_void_p * 8)()
    assert L.csa_decode_step_ex(sess, 2, 8, 64, 0.1, 1, fake, 1 << 30, None, no_events) == csa.EINVAL
    assert L.csa_dense_attn(fake, -1, fake, 8, 0.1, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_dense_attn(fake, (1 << 17) + 1, fake, 8, 0.1, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_dense_attn(fake, 100, fake, 0, 0.1, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_dense_attn(None, 100, fake, 8, 0.1, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_dense_attn(fake, 100, fake, 8, 0.1, fake, None, fake, 64, None) == csa.EWORKSPACE
    assert L.csa_dense_attn(fake, 100, fake, 8, 0.1, fake, None, ctypes.c_void_p(4096 + 8), 1 << 30, None) == csa.EWORKSPACE
    assert csa.lib.csa_dense_workspace_bytes(8194) > csa.lib.csa_dense_workspace_bytes(100) > 0
    assert L.csa_score_topk_multi(fake, 10, fake, fake, 0, 8, 512, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score_topk_multi(fake, 10, fake, fake, 65, 8, 512, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score_topk_multi(fake, 10, fake, fake, 4, 8, 513, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score_topk_multi(fake, 10, fake, fake, 4, 8, 0, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score_topk_multi(odd, 10, fake, fake, 4, 8, 512, fake, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score_topk_multi(fake, 10, fake, fake, 4, 8, 512, None, None, fake, 1 << 30, None) == csa.EINVAL
    assert L.csa_score_topk_multi(fake, 10, fake, fake, 4, 8, 512, fake, None, fake, 64, None) == csa.EWORKSPACE
    assert L.csa_pack_rows(None, None, 10, fake, fake, None) == csa.EINVAL
    assert L.csa_pack_rows(fake, None, 10, None, fake, None) == csa.EINVAL
    assert L.csa_pack_rows(None, fake, 10, fake, None, None) == csa.EINVAL
    assert L.csa_pack_rows(None, ctypes.c_void_p(4096 + 4), 10, fake, fake, None) == csa.EINVAL
    assert L.csa_pack_rows(fake, None, -1, fake, fake, None) == csa.EINVAL
    assert L.csa_lse_merge(fake, fake, fake, fake, 0, fake, ctypes.c_void_p(8192), None) == csa.EINVAL
    assert L.csa_lse_merge(fake, fake, fake, ctypes.c_void_p(8192), 8, fake, fake, None) == csa.EINVAL  # lse aliases lse_a
    assert L.csa_lse_merge(fake, None, fake, fake, 8, fake, ctypes.c_void_p(8192), None) == csa.EINVAL
    assert L.csa_quantize_query(fake, 0, fake, None) == csa.EINVAL
    assert L.csa_quantize_query(fake, 65, fake, None) == csa.EINVAL
    assert L.csa_quantize_query(odd, 8, fake, None) == csa.EINVAL
    assert L.csa_quantize_query(fake, 8, ctypes.c_void_p(4096 + 2), None) == csa.EINVAL
    assert L.csa_quantize_query(None, 8, fake, None) == csa.EINVAL


def test_noalloc_entry_point_rejects_oversized_steps_on_host(csa):
    L = csa.lib
    fake = ctypes.c_void_p(4096)  # never dereferenced: the size check comes first
    sess = (csa.Session * 16)()
    for i in range(16):
        sess[i] = csa.Session(fake, fake, 1 << 20, fake, fake, fake, fake, None, fake, None)
    assert csa.workspace_bytes(1 << 20, 16) > csa.SCRATCH_BYTES >= csa.workspace_bytes(1 << 20, 1)
    assert L.csa_decode_step_noalloc(sess, 16, 64, 64, 0.1, None) == csa.EWORKSPACE
    assert L.csa_decode_step_noalloc(sess, 0, 64, 64, 0.1, None) == csa.EINVAL
    assert L.csa_decode_step_noalloc(None, 1, 64, 64, 0.1, None) == csa.EINVAL
    sess[0] = csa.Session(fake, fake, -5, fake, fake, fake, fake, None, fake, None)
    assert L.csa_decode_step_noalloc(sess, 1, 64, 64, 0.1, None) == csa.EINVAL
    text = open(HEADER).read()
    assert "#define CSA_SCRATCH_BYTES (32u << 20)" in text and csa.SCRATCH_BYTES == 32 << 20


def test_binding_rejects_misshaped_tensors_before_any_launch(csa):
    import torch

    rows = torch.zeros((10, 68), dtype=torch.uint8)
    q = torch.zeros((8, 128), dtype=torch.float32)
    w = torch.zeros(8, dtype=torch.float32)
    kv = torch.zeros((10, 583), dtype=torch.uint8)
    qa = torch.zeros((4, 512), dtype=torch.float32)
    sel = torch.zeros(512, dtype=torch.int32)
    bad_calls = [
        lambda: csa.score(rows.view(-1), q, w),                   # flat row buffer
        lambda: csa.score(rows[:, :64], q, w),                    # wrong row width
        lambda: csa.score(rows, q[:, :64], w),                    # wrong query width
        lambda: csa.score(rows, q, w[:7]),                        # weights vs heads
        lambda: csa.score(rows, q.double(), w),                   # wrong dtype
        lambda: csa.topk(torch.zeros((4, 4)), 8),                 # not a vector
        lambda: csa.sparse_attn(kv.view(-1), sel, 4, qa, 0.1),    # flat KV buffer
        lambda: csa.sparse_attn(kv, sel, 4, qa[:, :100], 0.1),    # wrong query width
        lambda: csa.sparse_attn(kv, sel[:3], 4, qa, 0.1),         # fewer entries than n_sel
        lambda: csa.sparse_attn(kv, sel.long(), 4, qa, 0.1),      # wrong index dtype
        lambda: csa.DecodeStep([dict(idx_rows=rows, kv_rows=kv[:9], q_idx=q, w_idx=w, q_attn=qa)], 0.1),
        lambda: csa.DecodeStep([dict(idx_rows=rows, kv_rows=kv, q_idx=q, w_idx=w[:3], q_attn=qa)], 0.1),
        lambda: csa.DecodeStep([dict(idx_rows=rows, kv_rows=kv, q_idx=q, w_idx=w, q_attn=qa[:, :8])], 0.1),
    ]
    for i, call in enumerate(bad_calls):
        with pytest.raises(ValueError):
            call()
