"""Page arithmetic of the oracle against the numbers the pages print.

The expected values live in tests/golden/page_facts.json, each with the page
and section that prints it.
"""

import json
import os

import pytest

from oracle import pages as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")
FACTS = {f["name"]: f for f in json.load(open(GOLDEN))["facts"]}


def fact(name):
    return FACTS[name]["value"], FACTS[name]["inputs"]


PAGES = ("cs2680 Lecture 10", "inferenceinterviews.com", "llm-serving.xyz", "The inference server",
         "same page", "same paragraph", "same section")


def test_every_fact_has_a_source():
    for f in FACTS.values():
        assert any(p in f["source"] for p in PAGES), f["name"]


def test_bytes_per_token_and_pool():
    v, i = fact("kv_bytes_per_token_8b_shape")
    assert P.kv_bytes_per_token(**i) == v
    v, i = fact("kv_bytes_per_token_70b_shape")
    assert P.kv_bytes_per_token(**i) == v
    v, i = fact("page_bytes_8b_shape")
    assert P.page_bytes(**i) == v
    v, i = fact("pool_pages_512MiB")
    assert P.pool_pages(i["pool_bytes"], i["page_bytes"]) == v


def test_request_pages_round_up():
    v, i = fact("request_pages_2048_plus_257")
    assert P.pages_for_tokens(**i) == v
    v, i = fact("prompt_only_pages_2048")
    assert P.pages_for_tokens(**i) == v
    # the partial last page is a whole page: ceil, not round or floor
    assert P.pages_for_tokens(2305, 16) != round(2305 / 16)
    assert P.pages_for_tokens(2305, 16) != 2305 // 16


def test_shared_prefix_admission():
    v, i = fact("private_pages_per_request")
    assert P.private_pages(**i) == v
    v, i = fact("eight_shared_requests_pages")
    assert P.group_pages(**i) == v
    v, i = fact("seven_shared_requests_pages")
    assert P.group_pages(**i) == v
    v, i = fact("eight_unshared_requests_pages")
    assert P.unshared_pages(**i) == v
    v, i = fact("max_admitted_shared")
    assert P.max_admitted(i["pool_pages"], i["prefix_tokens"], i["total_tokens"],
                          i["block_tokens"], i["isolated"]) == v
    v, i = fact("max_admitted_isolated")
    assert P.max_admitted(i["pool_pages"], i["prefix_tokens"], i["total_tokens"],
                          i["block_tokens"], i["isolated"]) == v
    # 256 - 247 = 9 pages left, fewer than one more private reservation
    assert 256 - P.group_pages(7, 2048, 2305, 16) == 9 < P.private_pages(2048, 2305, 16)


def test_block_table_sizes():
    for name in ("block_table_entries_8k", "block_table_entries_8k_b64",
                 "block_table_entries_4k", "block_table_entries_4k_b64",
                 "block_table_entries_4k_b256"):
        v, i = fact(name)
        assert P.block_table_entries(**i) == v, name
    v, i = fact("block_table_bytes_8k_int32")
    assert P.block_table_bytes(**i) == v


@pytest.mark.parametrize("name", ["exercise3_table_entries_800",
                                  "exercise3_table_entries_20000"])
def test_exercise3_table_entries(name):
    v, i = fact(name)
    got = [P.block_table_entries(i["seq_len"], b) for b in i["block_tokens"]]
    assert got == v


def test_prefix_hits_are_whole_blocks():
    v, i = fact("prefix_hit_blocks_8000")
    assert P.prefix_hit_blocks(**i) == v
    v, i = fact("shared_system_prompt_blocks_2000")
    assert P.prefix_hit_blocks(**i) == v


def test_growth_takes_a_block_only_when_full():
    v, i = fact("growth_new_block_only_when_full")
    for L, n in v.items():
        assert P.blocks_after_growth(int(L), i["block_tokens"]) == n


def test_latent_cache_bytes():
    for name in ("mla_elements_per_token_layer", "mla_bytes_per_token_v3_fp8",
                 "mla_bytes_per_token_k3_bf16"):
        v, i = fact(name)
        assert P.latent_bytes_per_token(**i) == v
    # the printed ratio of the 70B shape's bytes per token to the latent cache's
    ratio = fact("kv_bytes_per_token_70b_shape")[0] / fact("mla_bytes_per_token_v3_fp8")[0]
    assert round(ratio, 1) == 9.3


def test_attention_flops_per_cached_token():
    for name in ("mla_attention_flops_per_cached_token",
                 "gqa70b_attention_flops_per_cached_token"):
        v, i = fact(name)
        assert P.attention_flops_per_cached_token(**i) == v
    # nine times the flops, as printed
    assert (fact("mla_attention_flops_per_cached_token")[0]
            // fact("gqa70b_attention_flops_per_cached_token")[0]) == 9
