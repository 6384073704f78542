"""Oracle: page and block-table arithmetic of a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Plain formulas, each the definition stated on the pages:
* bytes per token = 2 (K and V) x layers x KV heads x head dim x bytes per
  element [llm-serving.xyz "KV-cache systems", bytes-per-token equation;
  inferenceinterviews.com "Reserve the page a request has not written yet",
  "Separate the pool from its owners"].
* a page holds ``block`` tokens of every layer; a pool holds
  floor(pool bytes / page bytes) pages [same section].
* a request is charged whole pages, the last partial page included:
  ceil(tokens / block) [same page, worked arithmetic and the paragraph on
  the mostly-empty last page].
* complete shared-prefix pages are charged once per trust group; each
  request still pays its private pages [same page, "Charge shared pages
  once"].
* a block table has ceil(L / block) entries [llm-serving.xyz "KV-cache
  systems", block-table cost paragraph; cs2680 Lecture 10, §10.3 table].
* a prefix-cache hit reuses only complete matching blocks:
  floor(matched / block) [llm-serving.xyz "KV-cache systems", prefix-caching
  worked example].
* a latent (MLA) cache holds one latent of (compressed + positional)
  elements per token per layer, so bytes per token = (c + r) x layers x
  bytes per element [llm-serving.xyz "KV-cache systems", MLA section,
  cached-latent equation and the 34 KB/token figure].
* attention costs 4 x query heads x effective head dim flops per cached
  token per layer (a multiply-add for the score and one for the value, per
  head and dim) [same section, the costs paragraph].
"""

from __future__ import annotations


def ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int,
                       bytes_per_elem: int) -> int:
    return 2 * n_layers * n_kv_heads * head_dim * bytes_per_elem


def page_bytes(block_tokens: int, bytes_per_token: int) -> int:
    return block_tokens * bytes_per_token


def pool_pages(pool_bytes: int, page_bytes_: int) -> int:
    return int(pool_bytes) // int(page_bytes_)


def pages_for_tokens(tokens: int, block_tokens: int) -> int:
    return ceil_div(tokens, block_tokens)


def shared_prefix_pages(prefix_tokens: int, block_tokens: int) -> int:
    """Pages of a common prefix that can be shared: only complete pages."""
    return int(prefix_tokens) // int(block_tokens)


def private_pages(prefix_tokens: int, total_tokens: int,
                  block_tokens: int) -> int:
    """Pages a request owns alone when the complete prefix pages are shared."""
    return (pages_for_tokens(total_tokens, block_tokens)
            - shared_prefix_pages(prefix_tokens, block_tokens))


def group_pages(n_requests: int, prefix_tokens: int, total_tokens: int,
                block_tokens: int, groups: int = 1) -> int:
    """Pages charged for n requests split evenly over ``groups`` trust groups.

    Each group stores its shared prefix pages once; every request pays its
    private pages. With ``groups == n_requests`` nothing is shared.
    """
    if n_requests == 0:
        return 0
    shared = shared_prefix_pages(prefix_tokens, block_tokens)
    priv = private_pages(prefix_tokens, total_tokens, block_tokens)
    used_groups = min(groups, n_requests)
    return used_groups * shared + n_requests * priv


def unshared_pages(n_requests: int, total_tokens: int,
                   block_tokens: int) -> int:
    return n_requests * pages_for_tokens(total_tokens, block_tokens)


def max_admitted(pool_pages_: int, prefix_tokens: int, total_tokens: int,
                 block_tokens: int, isolated: bool = False) -> int:
    """Largest number of requests whose full reservation fits the pool."""
    n = 0
    while True:
        groups = n + 1 if isolated else 1
        need = group_pages(n + 1, prefix_tokens, total_tokens, block_tokens,
                           groups)
        if need > pool_pages_:
            return n
        n += 1


def block_table_entries(seq_len: int, block_tokens: int) -> int:
    return ceil_div(seq_len, block_tokens)


def block_table_bytes(seq_len: int, block_tokens: int, id_bytes: int) -> int:
    return block_table_entries(seq_len, block_tokens) * id_bytes


def prefix_hit_blocks(matched_tokens: int, block_tokens: int) -> int:
    return int(matched_tokens) // int(block_tokens)


def blocks_after_growth(seq_len: int, block_tokens: int) -> int:
    """Blocks a sequence holds at length L under on-demand growth."""
    return ceil_div(seq_len, block_tokens)


def latent_bytes_per_token(latent: int, rope: int, n_layers: int, bytes_per_elem: int) -> int:
    return (latent + rope) * n_layers * bytes_per_elem


def attention_flops_per_cached_token(n_q_heads: int, head_dim: int) -> int:
    return 4 * n_q_heads * head_dim
