"""Closed-form KV-cache sizes stated on the pages, as plain integer formulas.

* Bytes per token across all layers with grouped-query attention:
  2 (K and V) x layers x KV heads x head_dim x bytes per element
  ("PagedAttention deep dive", §1.1; Llama-3-8B: 2*32*8*128*2 = 131,072 B).
* Bytes for one sequence of T cached tokens:
  M_KV = 2 x L x T x H_KV x d_h x b ("vLLM inference principles", equation
  for M_KV and its symbol table; 2 GiB for L=32, T=4096, H_KV=32, d_h=128,
  b=2, and 0.5 GiB with H_KV=8).
* Bytes for a batch, counting every attention head (the page's worked example
  uses 32 heads, i.e. no GQA): batch x seq x layers x heads x head_dim x
  precision x 2 ("KV-Cache evolution", §2).
* Blocks a sequence occupies: ceil(seq_len / block_size) ("KV-cache sharing
  article", §5.1, pre-allocation code).
"""


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_bytes_per_token_per_layer(kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * kv_heads * head_dim * elem_bytes


def kv_bytes_sequence(layers: int, tokens: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * tokens * kv_heads * head_dim * elem_bytes


def kv_bytes_batch(batch: int, seq_len: int, layers: int, heads: int, head_dim: int,
                   elem_bytes: int) -> int:
    return batch * seq_len * layers * heads * head_dim * elem_bytes * 2


def blocks_needed(seq_len: int, block_size: int) -> int:
    return -(-seq_len // block_size)


def tokens_that_fit(budget_bytes: int, bytes_per_token: int) -> int:
    """Whole tokens whose KV fits in a byte budget."""
    return budget_bytes // bytes_per_token
