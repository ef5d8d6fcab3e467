"""Pins of the KV-size formula against numbers the pages print."""
import json
import os

from oracle import kvsize

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_lecture10_kv_size_table():
    tab = json.load(open(os.path.join(GOLDEN, "kv_size_table.json")))
    for row in tab["rows"]:
        nbytes = kvsize.kv_cache_bytes_mha(row["layers"], row["d_model"], row["seq_len"],
                                           tab["bytes_per_elem"])
        assert nbytes == row["gib"] * 2**30, row
        # the head-count form gives the same bytes when n_kv_heads * head_dim = d_model
        heads = row["d_model"] // 128
        assert kvsize.kv_cache_bytes(row["layers"], heads, 128, row["seq_len"], 1,
                                     tab["bytes_per_elem"]) == nbytes


def test_kv_size_scales_with_kv_heads():
    # Tutorial §3: 32 query heads with 8 KV heads keeps a quarter of the MHA cache.
    mha = kvsize.kv_cache_bytes(32, 32, 128, 4096)
    gqa = kvsize.kv_cache_bytes(32, 8, 128, 4096)
    assert gqa * 4 == mha
    # Lecture 10 GQA table: group 8 -> 1/8; MQA -> 1/n_heads
    assert kvsize.kv_cache_bytes(80, 64 // 8, 128, 2048) * 8 == kvsize.kv_cache_bytes(80, 64, 128, 2048)
    assert kvsize.kv_cache_bytes(1, 1, 128, 100) * 32 == kvsize.kv_cache_bytes(1, 32, 128, 100)


def test_kv_size_is_linear_in_each_factor():
    base = kvsize.kv_cache_bytes(2, 3, 5, 7, 11, 2)
    assert base == 2 * 2 * 3 * 5 * 7 * 11 * 2
    assert kvsize.kv_cache_bytes(2, 3, 5, 14, 11, 2) == 2 * base
    assert kvsize.kv_cache_bytes(2, 3, 5, 7, 22, 2) == 2 * base
    assert kvsize.kv_cache_bytes(2, 3, 5, 7, 11, 4) == 2 * base


def test_blocks_needed():
    # Tutorial §7: ceil(token_count / block_size)
    assert [kvsize.blocks_needed(n) for n in (0, 1, 15, 16, 17, 32, 33)] == [0, 1, 1, 1, 2, 2, 3]
    assert kvsize.blocks_needed(131072) == 8192
