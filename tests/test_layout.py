"""Row-format arithmetic pinned to the numbers printed on the DS4X page
("Packed cache ABI"; the F32 size from "Long-context synthetic decode")."""
import numpy as np

import gen
import pins

G = pins.load_kv_golden("ds4x_packed_cache_abi.txt")


def test_row_byte_counts():
    assert G["kv_e4m3_bytes"] + G["kv_rope_values"] * G["kv_rope_bytes_each"] + G["kv_scales"] == G["kv_row_bytes"]
    assert G["kv_e4m3_bytes"] + G["kv_rope_values"] == G["kv_row_elements"]
    assert G["kv_scales"] * G["kv_scale_block"] == G["kv_e4m3_bytes"]
    assert G["idx_values"] // 2 + G["idx_scales"] == G["idx_row_bytes"] == G["idx_code_bytes"] + G["idx_scales"]
    assert G["idx_scales"] * G["idx_scale_block"] == G["idx_values"]
    assert gen.IDX_ROW_BYTES == G["idx_row_bytes"] and gen.KV_ROW_BYTES == G["kv_row_bytes"]


def _kv_bytes(L, kv_row, idx_row):
    raw = G["layers"] * G["raw_ring_rows"] * kv_row
    comp = G["csa_layers"] * (L // G["csa_ratio"] + 2) * (kv_row + idx_row) + \
        G["hca_layers"] * (L // G["hca_ratio"] + 2) * kv_row
    return raw, comp, raw + comp


def test_allocation_formula_reproduces_page_totals():
    raw, comp, total = _kv_bytes(G["L"], G["kv_row_bytes"], G["idx_row_bytes"])
    assert raw == G["raw_rings_bytes"]
    assert comp == G["compressed_kv_and_indexer_bytes"]
    assert total == G["total_persistent_kv_bytes"]
    assert round(total / 2**30, 3) == G["total_persistent_kv_gib"]
    # a padded stride would not reproduce the printed total
    assert _kv_bytes(G["L"], 584, 68)[2] != G["total_persistent_kv_bytes"]
    assert _kv_bytes(G["L"], 583, 72)[2] != G["total_persistent_kv_bytes"]


def test_upstream_f32_size_pins_element_counts():
    L = G["L"]
    floats = (G["layers"] * G["raw_ring_rows"] * G["kv_row_elements"]
              + G["csa_layers"] * (L // 4 + 2) * (G["kv_row_elements"] + G["idx_values"])
              + G["hca_layers"] * (L // 128 + 2) * G["kv_row_elements"])
    assert round(4 * floats / 2**30, 2) == G["upstream_f32_gib_1m"]


def test_csa_rows_per_context():
    # one CSA row per four tokens plus two; 128K tokens -> 32,770 rows, 1M -> 262,146
    assert 131072 // 4 + 2 == 32770 and 1048576 // 4 + 2 == 262146
