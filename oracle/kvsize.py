"""KV-cache size (oracle; test infrastructure only).

Tutorial §2 ("KV Cache 到底缓存了什么？", the KV memory estimate) and Lecture 10
("KV Cache 的内存占用") give the size of the cache as the product of: 2 (one
tensor for K and one for V), the number of layers, the batch size, the
sequence length, the number of KV heads, the head dimension and the bytes per
element.  Lecture 10 also writes it as 2 x layers x d_model x seq_len x bytes
for a model without GQA (n_heads x d_head = d_model).
"""


def kv_cache_bytes(n_layers, n_kv_heads, head_dim, seq_len, batch=1, bytes_per_elem=2):
    """Bytes of K plus V for ``batch`` sequences of ``seq_len`` tokens.

    The product written out as the Tutorial §2 estimate states it.  Integer
    arithmetic, so the result is exact.
    """
    return 2 * n_layers * batch * seq_len * n_kv_heads * head_dim * bytes_per_elem


def kv_cache_bytes_mha(n_layers, d_model, seq_len, bytes_per_elem=2):
    """Lecture 10's d_model form (no GQA: n_kv_heads x head_dim = d_model), batch 1."""
    return 2 * n_layers * d_model * seq_len * bytes_per_elem


def blocks_needed(n_tokens, block_size=16):
    """Number of fixed-size KV blocks that hold ``n_tokens`` tokens.

    Tutorial §7: the block manager reserves ceil(token_count / block_size) blocks.
    """
    return -(-n_tokens // block_size)
