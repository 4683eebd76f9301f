"""The byte accounting behind every GB/s figure and roofline fraction
(bench.py's kv_bytes_per_token, side_cache_bytes_per_block, step_bytes),
pinned to the numbers the pages print (tests/golden/page_numbers.json) and to
per-workload totals that follow from them by multiplication.

* cpu-attn kernel card, introduction ("Measured on the boards"): 8 heads at
  head dimension 128, 8,192 tokens, the cache goes from 32 MB (f16) to 16 MB
  (int8 codes).
* Certified Sparse Attention via Perturbed Retrieval, appendix layout table,
  row "Keys and values": fp16 token-major, 256 B per row, 512 B per token.
* sparse_attn.md, "Method: Quest-style min/max block bounds": kmin[head_dim]
  and kmax[head_dim] per block in f16, i.e. 512 B per (block, KV head) at
  D = 128.
"""
import json
import os

import bench

HERE = os.path.dirname(os.path.abspath(__file__))
PAGES = json.load(open(os.path.join(HERE, "golden", "page_numbers.json")))
MiB = 2 ** 20


def test_cache_size_at_8192_tokens_matches_the_card():
    p = PAGES["int8_cache_bytes"]
    T, Hkv, D = p["tokens"], p["kv_heads"], p["head_dim"]
    f16 = T * Hkv * bench.kv_bytes_per_token("f16", D)
    assert f16 == p["f16_cache_MiB"] * MiB
    # int8: the codes (one byte per value) are the card's 16 MB; the two
    # float32 scales per (token, KV head) come on top
    i8 = T * Hkv * bench.kv_bytes_per_token("i8", D)
    assert i8 - T * Hkv * 8 == p["int8_codes_MiB"] * MiB


def test_token_and_row_bytes_match_the_layout_table():
    p = PAGES["f16_row_bytes"]
    assert bench.kv_bytes_per_token("f16", p["head_dim"]) == p["token_bytes_k_plus_v"]
    assert bench.kv_bytes_per_token("f16", p["head_dim"]) == 2 * p["row_bytes"]


def test_side_cache_bytes_per_block():
    p = PAGES["side_cache_bytes"]
    assert bench.side_cache_bytes_per_block(p["head_dim"]) == p["bytes_per_block_per_kv_head"]


def _quest_blocks(L, block, Hkv, n_sel):
    """n_sel attended blocks per KV head, all full (the last one too when L is
    a multiple of the block)."""
    return {(0, g): list(range(n_sel)) for g in range(Hkv)}


def test_workload_totals():
    # 32K f16 dense: 32,768 tokens x 8 KV heads x 512 B = 128 MiB
    d3 = bench.step_bytes([32768], 8, 32, 128, "f16", 64, None)
    assert d3["kv"] == 134_217_728 and d3["bounds"] == 0
    # 32K Quest: 131 of 512 blocks per KV head + the whole 2 MiB side cache
    q3 = bench.step_bytes([32768], 8, 32, 128, "f16", 64, _quest_blocks(32768, 64, 8, 131))
    assert q3["kv"] == 34_340_864 and q3["bounds"] == 2_097_152
    assert q3["kv"] + q3["bounds"] == 36_438_016
    # 262K int8 dense: 262,144 x 4 x 264 B
    d5 = bench.step_bytes([262144], 4, 32, 128, "i8", 64, None)
    assert d5["kv"] == 276_824_064
    # 262K int8 Quest: 517 of 4,096 blocks per KV head + 8 MiB side cache
    q5 = bench.step_bytes([262144], 4, 32, 128, "i8", 64, _quest_blocks(262144, 64, 4, 517))
    assert q5["kv"] == 34_940_928 and q5["bounds"] == 8_388_608
    assert q5["kv"] + q5["bounds"] == 43_329_536
    # 8K int8 dense: the card's shape with the two scales
    d2 = bench.step_bytes([8192], 8, 32, 128, "i8", 64, None)
    assert d2["kv"] == 17_301_504
    # query in, output out: float32 [B][H][D] each
    assert d3["q_out"] == 2 * 32 * 128 * 4
    assert d3["total"] == d3["kv"] + d3["q_out"]


def test_partial_last_block_is_clipped():
    # a 100-token sequence: blocks 0 (64 tokens) and 1 (36 tokens)
    r = bench.step_bytes([100], 1, 1, 128, "f16", 64, {(0, 0): [0, 1]})
    assert r["kv"] == 100 * 512
    assert r["bounds"] == 2 * 512
    r = bench.step_bytes([100], 1, 1, 128, "f16", 64, {(0, 0): [1]})
    assert r["kv"] == 36 * 512


def test_grouped_cache_bytes():
    """q8_0 / q4_0 / q5_0 (sparse_attn.md, "All-KV-types composition": blocks of 32
    values): per (token, KV head) the K and V rows hold D codes of 8 or 4 bits
    and an f16 scale per 32 channels -- 2 x (128 + 8) and 2 x (64 + 8) bytes at
    D = 128, i.e. 34 and 18 bytes per 32 values."""
    assert bench.kv_bytes_per_token("q8_0", 128) == 272
    assert bench.kv_bytes_per_token("q4_0", 128) == 144
    assert bench.kv_bytes_per_token("q8_0", 128) / 2 / 4 == 34
    assert bench.kv_bytes_per_token("q4_0", 128) / 2 / 4 == 18
    # q5_0: five bits per value (a nibble plus a fifth bit) and the f16 scale:
    # 20 + 2 = 22 bytes per 32 values, 2 x (64 + 16 + 8) per row at D = 128
    assert bench.kv_bytes_per_token("q5_0", 128) == 176
    assert bench.kv_bytes_per_token("q5_0", 128) / 2 / 4 == 22
    assert bench.kv_bytes_per_token("q5_0", 64) == 88


def test_scan4_index_bytes_match_the_layout_table():
    """The 4-bit scan reads 64 B of codes per token and, per block, three
    float32 values per channel; at the table's 128-token blocks those are 12 B
    per token (Certified Sparse Attention via Perturbed Retrieval, appendix
    layout table, rows "4-bit codes" and "Block scales").  The GQA-shared scan
    reads the codes once per KV head, a per-head scan G times."""
    p = PAGES["scan4_index_bytes"]
    D, blk = p["head_dim"], p["block_tokens_implied"]
    one_token = bench.scan4_index_bytes([blk], 1, D, blk) / blk
    assert one_token == p["codes_bytes_per_token"] + p["block_scales_bytes_per_token"]
    codes_only = bench.scan4_index_bytes([blk], 1, D, blk) - 3 * D * 4
    assert codes_only == p["codes_bytes_per_token"] * blk
    # 32K f16 workload: 32,768 tokens x 8 KV heads, 64-token blocks
    assert bench.scan4_index_bytes([32768], 8, 128, 64) == 32768 * 8 * 64 + 512 * 8 * 1536
    assert bench.scan4_index_bytes([32768], 8, 128, 64, reads_per_token=4) == \
        4 * 32768 * 8 * 64 + 512 * 8 * 1536
