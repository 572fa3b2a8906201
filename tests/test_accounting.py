"""The measurement accounting reproduces the numbers printed in the pages' footnotes."""
import json
import os

from sparse_mla_attention_score_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "footnote_accounting.json")))


def test_footnote_1_sparse_mla_accounting():
    f = GOLD["footnote_1"]
    K = f["rows_per_query"]
    assert acc.ROW_BYTES[1] == f["fp8_row_bytes"]
    assert acc.ROW_BYTES[1] + acc.ROW_INDEX_BYTES == f["bytes_per_selected_row"]
    assert round(K * f["bytes_per_selected_row"] / 1e6, 2) == f["row_bytes_per_query_MB"]
    assert acc.HEAD_IO_BYTES == f["bytes_per_head_for_bf16_query_and_output"]
    assert acc.FLOPS_PER_HEAD_ROW == f["flops_per_head_row"]
    for heads, key in ((8, "heads_8"), (64, "heads_64")):
        b = acc.sparse_mla_bytes(K, heads)
        fl = acc.sparse_mla_flops(K, heads)
        assert round(b / 1e6, 2) == f[key]["MB"]
        assert round(fl / 1e6, 1 if heads == 8 else 0) == f[key]["MFLOPs"]
        assert int(fl / b) == f[key]["flops_per_byte"]


def test_footnote_3_per_token_footprint():
    f = GOLD["footnote_3"]
    assert acc.IDX_KEY_BYTES[1] == f["indexer_key_bytes"] == f["indexer_fp8_values"] + f["indexer_scale_bytes"]
    per_tok = acc.kv_bytes_per_token(f["mla_layers"], f["indexer_layers"], f["mtp_bytes"])
    assert per_tok == f["bytes_per_token"]
    assert round(per_tok * f["tokens"] / 2 ** 30, 1) == f["GiB"]


def test_hot_buffer_rules():
    p1 = GOLD["part_1"]
    K = GOLD["part_2_topk"]["topk"]
    assert p1["hot_rows_default_multiple_of_topk"] * K == 4096
    assert (p1["mtp_num_speculative_tokens"] + 2) * K == 10240


def test_step_work_128k_config():
    w = acc.step_work([131072] * 64, 4, 2048, 1, 1, 1)
    # keys alone: 64 x 131072 x 132 B = 1107.3 MB; plus q, w in and top-K lists out
    assert w["indexer_bytes"] == 64 * (131072 * 132 + 4 * (32 * 128 * 2 + 32 * 4) + 4 * 2048 * 4)
    assert abs(w["gather_bytes"] / 1e6 - 381.7) < 0.1
    assert abs(w["attention_flops"] / 1e9 - 73.0) < 0.05


def test_sweep_bytes_are_keys_and_queries():
    # FP8: 128 codes + a 4-byte scale per key; per query 32 x 128 bf16 + 32 fp32 weights
    assert acc.sweep_bytes(131072, 4) == 131072 * 132 + 4 * (32 * 128 * 2 + 32 * 4)
    assert acc.sweep_bytes(8192, 1, idx_dtype=0) == 8192 * 256 + 32 * 128 * 2 + 32 * 4
    assert acc.indexer_bytes(131072, 4, 2048) - acc.sweep_bytes(131072, 4) == 4 * 2048 * 4
