"""Oracle check (a): the closed-form cache sizes against every number the
pages print (tests/golden/cache_sizes.json, each entry cited there)."""
import json
import os

import pytest

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_sizes.json")))
MiB, GiB, KiB = 2 ** 20, 2 ** 30, 2 ** 10


def test_huny_per_token_layer():
    g = GOLD["huny_table_per_token_layer"]
    s = g["settings"]
    assert O.kv_bytes_per_token_layer("mha", n_h=s["n_h"], d_h=s["d_h"], bytes_per=s["bytes"]) == g["mha_bytes"]
    assert O.kv_bytes_per_token_layer("gqa", groups=s["gqa_groups"], d_h=s["d_h"], bytes_per=s["bytes"]) == g["gqa_bytes"]
    assert O.kv_bytes_per_token_layer("mla", d_c=s["d_c"], d_r=s["d_r"], bytes_per=s["bytes"]) == g["mla_bytes"]
    assert round(g["mha_bytes"] / g["mla_bytes"]) == 57


def test_huny_4k_session_and_savings():
    g = GOLD["huny_table_4k_session"]
    s = GOLD["huny_table_per_token_layer"]["settings"]
    L, S = g["settings"]["layers"], g["settings"]["tokens"]
    mha = O.kv_cache_bytes("mha", layers=L, tokens=S, n_h=s["n_h"], d_h=s["d_h"])
    gqa = O.kv_cache_bytes("gqa", layers=L, tokens=S, groups=s["gqa_groups"], d_h=s["d_h"])
    mla = O.kv_cache_bytes("mla", layers=L, tokens=S, d_c=s["d_c"], d_r=s["d_r"])
    assert (mha, gqa, mla) == (g["mha_mib"] * MiB, g["gqa_mib"] * MiB, g["mla_mib"] * MiB)
    assert mha / GiB == g["mha_gib_printed"]
    assert round(100 * (1 - mla / mha), 2) == g["saving_mla_vs_mha_pct"]
    assert round(100 * (1 - gqa / mha), 2) == g["saving_gqa_vs_mha_pct"]
    assert round(100 * (1 - mla / gqa), 1) == g["saving_mla_vs_gqa_pct_table"]
    assert round(100 * (1 - mla / gqa), 2) == g["saving_mla_vs_gqa_pct_case1"]


def test_huny_32_sessions_units():
    # 32 x 7680 MiB = 245,760 MiB; the page prints it as "245GB" (MiB/1000).
    g = GOLD["huny_32_sessions"]
    s = GOLD["huny_table_per_token_layer"]["settings"]
    one = O.kv_cache_bytes("mha", layers=30, tokens=4096, n_h=s["n_h"], d_h=s["d_h"])
    total_mib = g["sessions"] * one / MiB
    assert total_mib == 245760
    assert int(total_mib // 1000) == g["printed_gb"]


def test_huny_latent_ratio():
    assert (128 * 128) // 512 == GOLD["huny_latent_ratio"]["ratio"]


def test_donmain_128k_60_layers():
    g = GOLD["donmain_128k_60_layers"]
    s = g["settings"]
    mha = O.kv_cache_bytes("mha", layers=s["layers"], tokens=s["tokens"], n_h=128, d_h=128)
    gqa = O.kv_cache_bytes("gqa", layers=s["layers"], tokens=s["tokens"], groups=8, d_h=128)
    mla = O.kv_cache_bytes("mla", layers=s["layers"], tokens=s["tokens"], d_c=512, d_r=64)
    assert mha == g["mha_dims"] * s["layers"] * s["tokens"] * s["bytes"]
    assert gqa == g["gqa8_dims"] * s["layers"] * s["tokens"] * s["bytes"]
    assert mla == g["mla_dims"] * s["layers"] * s["tokens"] * s["bytes"]
    # the printed values are binary GB, rounded loosely
    assert mha / GiB == g["mha_printed_gb"]
    assert gqa / GiB == g["gqa8_printed_gb"]
    assert mla / GiB == pytest.approx(g["mla_printed_gb"], abs=0.07)   # 8.4375 GiB


def test_donmain_mqa_floor_and_gqa_equiv():
    assert O.kv_bytes_per_token_layer("mqa", d_h=128, bytes_per=1) == GOLD["donmain_mqa_floor"]["dims"]
    mla = O.kv_bytes_per_token_layer("mla", d_c=512, d_r=64, bytes_per=1)
    per_head = O.kv_bytes_per_token_layer("gqa", groups=1, d_h=128, bytes_per=1)
    assert mla / per_head == GOLD["donmain_gqa_equiv"]["kv_heads_equiv"]


def test_donmain_tp4():
    g = GOLD["donmain_tp4"]
    assert O.kv_bytes_per_token_layer("gqa", groups=8, d_h=128, bytes_per=1) // 4 == g["gqa8_per_gpu_dims"]
    # the latent is not split by head: every rank keeps the full row
    assert O.kv_bytes_per_token_layer("mla", d_c=512, d_r=64, bytes_per=1) == g["mla_per_gpu_dims"]


def test_vllm_compression():
    g = GOLD["vllm_compression"]
    assert O.kv_bytes_per_token_layer("mha", n_h=128, d_h=128, bytes_per=1) == g["mha_dims"]
    assert O.kv_bytes_per_token_layer("mla", d_c=512, d_r=64, bytes_per=1) == g["mla_dims"]
    assert int(g["mha_dims"] / g["mla_dims"]) == g["printed_ratio_approx"]


def test_thaki_table():
    g = GOLD["thaki_table"]
    per_tok = {}
    for m in g["models"]:
        if m["kind"] == "mla":
            f = O.floats_per_token_all_layers("mla", layers=m["layers"], d_latent=m["d_latent"])
        else:
            f = O.floats_per_token_all_layers("gqa", layers=m["layers"], kv_heads=m["kv_heads"],
                                              d_head=m["d_head"])
        b = 2 * f
        per_tok[m["name"]] = b
        assert b == m["per_token_kib"] * KiB, m["name"]
        assert b * 131072 == m["ctx_128k_gib"] * GiB, m["name"]
    assert round(per_tok["Gemma 3 27B"] / per_tok["Llama 3 70B"], 2) == g["gemma_over_llama_printed"]
    assert round(per_tok["Gemma 3 27B"] / per_tok["DeepSeek V2"], 1) == g["gemma_over_deepseek_printed"]
    llama_mha = 2 * O.floats_per_token_all_layers("mha", layers=80, kv_heads=g["llama_query_heads"], d_head=128)
    assert llama_mha == g["llama_no_sharing_kib"] * KiB


def test_thaki_table_omits_rope_key():
    # The table's DeepSeek V2 row counts only d_c = 512; with the 64 RoPE dims
    # that the other pages cache (576 wide) the row is 67.5 KiB / 8.4375 GiB.
    with_rope = 2 * O.floats_per_token_all_layers("mla", layers=60, d_latent=576)
    assert with_rope == 67.5 * KiB
    assert with_rope * 131072 == 8.4375 * GiB
