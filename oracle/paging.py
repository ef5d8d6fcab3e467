"""Paged KV cache: block-table translation, de-paging, append, gather.

Oracle; test infrastructure only.

What the pages fix (Tutorial §7 "PagedAttention 如何解决显存碎片？"; Lecture 10
"PagedAttention 与 vLLM"; In-depth §2.1): the cache of a sequence is cut into
fixed blocks of 16 tokens; a per-sequence block table lists the physical block
that holds each logical block, so logical block i of a sequence whose table is
[17, 4, 29, 11] lives in physical block table[i].  Token t of the sequence is
therefore in physical block table[t // 16], at offset t % 16 inside it.

What the pages leave open is the element order inside a physical block.  The
cache format used throughout this project (and stated in include/paged_attn.h):

    k_cache[num_blocks, num_kv_heads, head_dim / x, 16, x]   x = 16 / element bytes
    v_cache[num_blocks, num_kv_heads, head_dim, 16]

so K of token t, KV head g is k_cache[table[t//16], g, :, t%16, :] read in (column,
element) order, and V of it is v_cache[table[t//16], g, :, t%16].  For int8 storage
one fp32 scale per (physical block, KV head) applies to each tensor:
k_scale[num_blocks, num_kv_heads], v_scale[num_blocks, num_kv_heads].

A "slot" is the flat index physical_block * 16 + offset of one token position.
"""

import numpy as np

from . import storage

BLOCK_SIZE = 16


def k_row(k_cache, blk, g, off):
    """Stored K row (head_dim elements) of one token: the 16-byte columns in order."""
    return np.asarray(k_cache[blk, g, :, off, :]).reshape(-1)


def token_location(table_row, t, block_size=BLOCK_SIZE):
    """(physical block, offset) of logical token ``t`` (Tutorial §7 block table)."""
    return int(table_row[t // block_size]), t % block_size


def slot_of(table_row, t, block_size=BLOCK_SIZE):
    """Flat slot index of logical token ``t``: physical_block * 16 + offset."""
    blk, off = token_location(table_row, t, block_size)
    return blk * block_size + off


def depage(k_cache, v_cache, kind, table_row, seq_len, g, k_scale=None, v_scale=None,
           block_size=BLOCK_SIZE):
    """Contiguous fp64 K and V ([seq_len, head_dim] each) of one sequence, KV head ``g``.

    Walks the sequence's logical tokens in order and reads each one from the
    physical block its table entry names (Tutorial §7), one token at a time --
    the plain definition, no blocking.  Decoding follows ``storage.decode``.
    """
    d = v_cache.shape[2]
    K = np.empty((seq_len, d), dtype=np.float64)
    V = np.empty((seq_len, d), dtype=np.float64)
    for t in range(seq_len):
        blk, off = token_location(table_row, t, block_size)
        ks = None if k_scale is None else k_scale[blk, g]
        vs = None if v_scale is None else v_scale[blk, g]
        K[t] = storage.decode(k_row(k_cache, blk, g, off), kind, ks)
        V[t] = storage.decode(v_cache[blk, g, :, off], kind, vs)
    return K, V


def depage_fast(k_cache, v_cache, kind, table_row, seq_len, g, k_scale=None, v_scale=None,
                block_size=BLOCK_SIZE):
    """Same result as ``depage``, with the token loop done by numpy fancy indexing.

    Used for large sequences; ``tests/test_oracle_paging.py`` checks it equals
    ``depage`` element for element.
    """
    t = np.arange(seq_len)
    blk = np.asarray(table_row)[t // block_size].astype(np.int64)
    off = t % block_size
    ks = None if k_scale is None else np.asarray(k_scale)[blk, g][:, None]
    vs = None if v_scale is None else np.asarray(v_scale)[blk, g][:, None]
    kc = np.asarray(k_cache)
    kr = kc[blk, g, :, off, :].reshape(seq_len, kc.shape[2] * kc.shape[4])
    K = storage.decode(kr, kind, ks)
    V = storage.decode(v_cache[blk, g, :, off], kind, vs)
    return K, V


def append(k_cache, v_cache, k_new, v_new, slot_mapping, block_size=BLOCK_SIZE):
    """Copies of the caches after writing each new token's K/V to its slot.

    Tutorial §2 and Lecture 10 ("KV Cache 原理"): each decode step computes the
    new token's K and V and appends them to the cache.  Token ``i`` of
    ``k_new``/``v_new`` ([T, num_kv_heads, head_dim], stored element type) goes
    to slot ``slot_mapping[i]``; a negative slot means "no write".  A bit copy:
    the stored elements are moved unchanged.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        blk, off = divmod(int(s), block_size)
        for g in range(kc.shape[1]):
            kc[blk, g, :, off, :] = np.asarray(k_new[i, g, :]).reshape(kc.shape[2], kc.shape[4])
            vc[blk, g, :, off] = v_new[i, g, :]
    return kc, vc


def gather(k_cache, v_cache, block_tables, seq_lens, k_out, v_out, block_size=BLOCK_SIZE):
    """Copies of ``k_out``/``v_out`` ([B, num_kv_heads, maxL, head_dim]) with each
    sequence's valid tokens copied out of the pool in logical order.

    Positions t >= seq_lens[b] are left as they were.  A bit copy of the stored
    elements, so int8 stays int8 (scales are not applied).
    """
    ko = np.array(k_out, copy=True)
    vo = np.array(v_out, copy=True)
    for b, L in enumerate(np.asarray(seq_lens).tolist()):
        for t in range(L):
            blk, off = token_location(block_tables[b], t, block_size)
            for g in range(ko.shape[1]):
                ko[b, g, t, :] = k_row(k_cache, blk, g, off)
                vo[b, g, t, :] = v_cache[blk, g, :, off]
    return ko, vo


def copy_blocks(k_cache, v_cache, pairs, k_scale=None, v_scale=None):
    """Copies of the caches (and int8 scales) after copying physical block ``src`` to
    ``dst`` for every pair: all KV heads' K and V of the block, bit for bit.

    This is the copy-on-write step of block sharing (devpress tutorial §7: blocks shared
    between sequences carry reference counts; a shared block that one sharer must write is
    first copied to a block of its own).  Pairs with a block outside the pool, or with
    src == dst, are skipped; every copy reads the pool as it was before the call (the
    destinations are fresh blocks that no pair reads).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ks = None if k_scale is None else np.array(k_scale, copy=True)
    vs = None if v_scale is None else np.array(v_scale, copy=True)
    nb = kc.shape[0]
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        if not (0 <= src < nb and 0 <= dst < nb) or src == dst:
            continue
        kc[dst] = k_cache[src]
        vc[dst] = v_cache[src]
        if ks is not None:
            ks[dst] = k_scale[src]
            vs[dst] = v_scale[src]
    return kc, vc, ks, vs
