"""Seeded synthetic inputs for paged GQA decode attention.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds NO attention arithmetic: it draws random numbers, rounds them to the
storage types, hands out pool blocks the way a KV block manager does, and
encodes int8 caches.  Everything it returns is a CPU ``torch`` tensor.

Cache format (the library's, see include/paged_attn.h):
    k_cache [num_blocks, num_kv_heads, head_dim / x, 16, x]   x = 16 / element bytes
    v_cache [num_blocks, num_kv_heads, head_dim, 16]
The generator works on token-major [num_blocks, num_kv_heads, 16, head_dim] arrays and
encodes them into that format as its last step (``encode_k`` / ``encode_v``).
    k_scale, v_scale [num_blocks, num_kv_heads] fp32 (int8 and fp8 caches; fp8 codes are
    stored as uint8 bytes)
    block_tables [B, max_blocks] int32 (unused entries = -1)
    seq_lens [B] int32, q [B, nq, Hq, d], slot_mapping [B] int64

Random K/V values are drawn for the whole physical pool at once (every slot of
every block), which gives the same distribution as drawing them per sequence
because each pool slot holds at most one token.  Slots and blocks that no
sequence uses are poisoned (NaN, or extreme int8 codes / NaN scales) so that a
kernel which reads them shows it in the result.
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import math

import torch

BLOCK_SIZE = 16


# --------------------------------------------------------------------------------------
# Block manager (host harness): the free-pool / block-table bookkeeping of the
# KVBlockManager sketched in the devpress tutorial §7, plus the reference counts and
# shared prefix entries that section lists as needed by a real system.
# --------------------------------------------------------------------------------------
class BlockAllocator:
    def __init__(self, total_blocks: int, block_size: int = BLOCK_SIZE, free_order=None):
        self.block_size = block_size
        self.total_blocks = total_blocks
        # blocks are handed out from the end of the free list
        self.free_blocks = list(range(total_blocks)) if free_order is None else list(free_order)
        self.block_tables = {}
        self.token_counts = {}
        self.refcount = [0] * total_blocks

    def _take(self):
        if not self.free_blocks:
            raise RuntimeError("KV cache pool exhausted")
        blk = self.free_blocks.pop()
        self.refcount[blk] += 1
        return blk

    def allocate(self, request_id, token_count: int):
        required = -(-token_count // self.block_size)
        if len(self.free_blocks) < required:
            raise RuntimeError("KV cache pool exhausted")
        self.block_tables[request_id] = [self._take() for _ in range(required)]
        self.token_counts[request_id] = token_count
        return self.block_tables[request_id]

    def fork(self, parent_id, child_id, shared_tokens: int, total_tokens: int):
        """Child shares the parent's first blocks (shared_tokens must fill whole
        blocks) and gets private blocks for the rest."""
        if shared_tokens % self.block_size:
            raise ValueError("a shared prefix must cover whole blocks")
        nshared = shared_tokens // self.block_size
        shared = self.block_tables[parent_id][:nshared]
        for blk in shared:
            self.refcount[blk] += 1
        required = -(-total_tokens // self.block_size) - nshared
        if len(self.free_blocks) < required:
            raise RuntimeError("KV cache pool exhausted")
        self.block_tables[child_id] = list(shared) + [self._take() for _ in range(required)]
        self.token_counts[child_id] = total_tokens
        return self.block_tables[child_id]

    def fork_all(self, parent_id, child_id):
        """Child shares every block of the parent, the partly filled last one included
        (parallel sampling from one prompt); the first of them to write into a shared
        block copies it (``append_token``)."""
        blocks = self.block_tables[parent_id]
        for blk in blocks:
            self.refcount[blk] += 1
        self.block_tables[child_id] = list(blocks)
        self.token_counts[child_id] = self.token_counts[parent_id]
        return self.block_tables[child_id]

    def append_token(self, request_id):
        """Account one more token and return its pool slot plus the block copy it needs:
        (slot, None), or (slot, (src, dst)) when the token lands in a block that other
        sequences still share, which the sequence first replaces by a private copy (the
        copy-on-write of devpress tutorial §7).  A full last block gets a new block."""
        blocks = self.block_tables[request_id]
        used = self.token_counts[request_id]
        copy = None
        if used >= len(blocks) * self.block_size:
            blocks.append(self._take())
        elif self.refcount[blocks[-1]] > 1:
            old = blocks[-1]
            blocks[-1] = self._take()
            self.refcount[old] -= 1
            copy = (old, blocks[-1])
        self.token_counts[request_id] = used + 1
        return blocks[used // self.block_size] * self.block_size + used % self.block_size, copy

    def release(self, request_id):
        for blk in self.block_tables.pop(request_id, []):
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free_blocks.append(blk)
        self.token_counts.pop(request_id, None)

    def occupancy(self):
        """Per physical block, how many leading slots hold a live token (0 = unused).
        A shared block counts as full when any owner fills it."""
        occ = [0] * self.total_blocks
        for rid, blocks in self.block_tables.items():
            n = self.token_counts[rid]
            for j, blk in enumerate(blocks):
                occ[blk] = max(occ[blk], min(self.block_size, n - j * self.block_size))
        return occ


# --------------------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str                      # "f32" | "bf16"
    kv_dtype: str                     # "f32" | "bf16" | "i8" | "fp8"
    lengths: Optional[Tuple[int, ...]] = None      # fixed context lengths, or
    length_range: Optional[Tuple[int, int]] = None  # inclusive uniform range
    lengths_are_cached: bool = False  # True: the step appends after these tokens
    num_q_pos: int = 1                # 1 = decode; >1 = causal verify rows
    append: bool = True               # the step writes one new token per sequence
    pool_blocks: Optional[int] = None  # None = exactly what the tables need
    shared_groups: int = 0            # groups of sequences sharing a prefix
    shared_group_size: int = 0
    shared_prefix_tokens: int = 0
    peaked_fraction: float = 0.0      # fraction of K slots scaled by peaked_factor
    peaked_factor: float = 8.0
    sliding_window: int = 0           # 0 = whole context; W = the W most recent tokens
    tree: bool = False                # the nq query positions form a speculative tree
    # outlier V scales (per-(block, head) scales exist because of outliers, in-depth guide
    # section 5.2): every sequence's first block has its V multiplied by this factor, and,
    # if v_outlier is set, element (token 0, dim v_outlier_dim) of that block's V set to
    # +-v_outlier (the sign alternating over sequences), before the 8-bit encoding
    v_first_block_factor: float = 1.0
    v_outlier: float = 0.0
    v_outlier_dim: int = 5
    seed: int = 0

    @property
    def group_size(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def sm_scale(self):
        return 1.0 / math.sqrt(self.head_dim)


CONFIGS = {
    # batch 4, 8q/2kv, d64, fp32; the listed lengths are cached before the step's append
    "tiny_fp32": Config("tiny_fp32", 4, 8, 2, 64, "f32", "f32", lengths=(37, 128, 200, 511),
                        lengths_are_cached=True, pool_blocks=256, seed=1000),
    # Llama-3-8B attention layer: 32q/8kv, d128, bf16, context U[512, 4096], batch 64
    "llama3_8b": Config("llama3_8b", 64, 32, 8, 128, "bf16", "bf16", length_range=(512, 4096),
                        seed=1001),
    # Llama-2-70B attention layer: 64q/8kv, 32 sequences of 4096; 6 groups of 5 share 2048
    "llama2_70b_prefix": Config("llama2_70b_prefix", 32, 64, 8, 128, "bf16", "bf16",
                                lengths=(4096,) * 32, shared_groups=6, shared_group_size=5,
                                shared_prefix_tokens=2048, seed=1002),
    # 128K-token contexts, batch 4, 32q/8kv; 1% of K positions x8 (peaked softmax)
    "long_128k": Config("long_128k", 4, 32, 8, 128, "bf16", "bf16", lengths=(131072,) * 4,
                        peaked_fraction=0.01, seed=1003),
    # speculative verify: 1 + 5 draft positions, causal, int8 KV, context U[1024, 8192]
    "verify_int8": Config("verify_int8", 32, 32, 8, 128, "bf16", "i8",
                          length_range=(1024, 8192), num_q_pos=6, append=False, seed=1004),
    # chunked prefill: a 256-token chunk of each of 4 prompts attends causally to the
    # prompt so far (Llama-3-8B layer shape), context U[2048, 8192] including the chunk
    "prefill_chunk": Config("prefill_chunk", 4, 32, 8, 128, "bf16", "bf16",
                            length_range=(2048, 8192), num_q_pos=256, append=False, seed=1007),
    # speculative tree verify: 64 candidates in a random tree per sequence, batch 32
    "tree_verify": Config("tree_verify", 32, 32, 8, 128, "bf16", "bf16",
                          length_range=(1024, 4096), num_q_pos=64, append=False, tree=True,
                          seed=1008),
    # fp8 e4m3 KV (per-(block, head) scales), the Llama-3-8B decode shape: half the bytes
    "llama3_8b_fp8": Config("llama3_8b_fp8", 64, 32, 8, 128, "bf16", "fp8",
                            length_range=(512, 4096), append=False, seed=1006),
    # sliding-window decode (Mistral-7B-shaped layer: 32q/8kv, d128, window 4096), batch
    # 64, context U[2048, 16384] so that most sequences run past the window
    "mistral_7b_window": Config("mistral_7b_window", 64, 32, 8, 128, "bf16", "bf16",
                                length_range=(2048, 16384), sliding_window=4096, seed=1005),
}


@dataclass
class Workload:
    cfg: Config
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    block_tables: torch.Tensor
    seq_lens: torch.Tensor            # tokens attended (after the step's append)
    slot_mapping: Optional[torch.Tensor]
    k_new: Optional[torch.Tensor]
    v_new: Optional[torch.Tensor]
    occupancy: torch.Tensor           # live slots per physical block
    meta: dict = field(default_factory=dict)
    tree_mask: Optional[torch.Tensor] = None   # [B, nq, nq] bool: candidate j visible to i

    @property
    def sm_scale(self):
        return self.cfg.sm_scale

    def kv_bytes(self):
        """Algorithmic bytes of K and V one pass over every sequence must read:
        each attended token's K and V once (plus the int8 scales of used blocks)."""
        c = self.cfg
        elem = {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1}[c.kv_dtype]
        toks = sum(self.visible_range(int(L))[1] - self.visible_range(int(L))[0]
                   for L in self.seq_lens.tolist())
        nbytes = toks * 2 * c.num_kv_heads * c.head_dim * elem
        if c.kv_dtype in ("i8", "fp8"):
            used = 0
            for L in self.seq_lens.tolist():
                lo, hi = self.visible_range(int(L))
                used += -(-hi // BLOCK_SIZE) - lo // BLOCK_SIZE if hi > lo else 0
            nbytes += used * 2 * c.num_kv_heads * 4
        return nbytes

    def visible_range(self, L):
        """Tokens [lo, L) that some query row of a sequence of L tokens attends (all of
        them, or with a sliding window of W the last W + nq - 1)."""
        c = self.cfg
        W = c.sliding_window
        return (max(0, L - W - c.num_q_pos + 1) if W > 0 else 0), L


_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _draw_lengths(cfg: Config, gen):
    if cfg.lengths is not None:
        L = list(cfg.lengths)[: cfg.batch]
        if len(L) != cfg.batch:
            raise ValueError("fixed lengths do not match the batch")
    else:
        lo, hi = cfg.length_range
        L = torch.randint(lo, hi + 1, (cfg.batch,), generator=gen).tolist()
    if cfg.lengths_are_cached:
        L = [x + 1 for x in L]
    return L


def _randn_pool(shape, gen, chunk_rows=1024):
    """N(0,1) fp32 tensor of ``shape``, drawn in chunks along dim 0."""
    out = torch.empty(shape, dtype=torch.float32)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=gen)
    return out


def generate(cfg, seed=None, *, poison=True, spare_blocks=0, shuffle_batch=False):
    """Build a seeded workload for ``cfg`` (a Config or a name in CONFIGS)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    gen = torch.Generator().manual_seed(seed)
    B, Hq, Hkv, d = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    lens = _draw_lengths(cfg, gen)

    # ---- block tables from a shuffled free pool -----------------------------------
    need = sum(-(-L // BLOCK_SIZE) for L in lens)
    if cfg.shared_groups:
        per_prefix = cfg.shared_prefix_tokens // BLOCK_SIZE
        need -= cfg.shared_groups * (cfg.shared_group_size - 1) * per_prefix
    NB = (cfg.pool_blocks if cfg.pool_blocks is not None else need) + spare_blocks
    free_order = torch.randperm(NB, generator=gen).tolist()
    alloc = BlockAllocator(NB, BLOCK_SIZE, free_order)
    b = 0
    for _ in range(cfg.shared_groups):
        leader = b
        alloc.allocate(leader, lens[leader])
        b += 1
        for _ in range(cfg.shared_group_size - 1):
            alloc.fork(leader, b, cfg.shared_prefix_tokens, lens[b])
            b += 1
    for bb in range(b, B):
        alloc.allocate(bb, lens[bb])
    # (at least one column: a batch of empty sequences still passes a table, all -1)
    max_blocks = max(1, max(len(alloc.block_tables[i]) for i in range(B)))
    tables = torch.full((B, max_blocks), -1, dtype=torch.int32)
    for i in range(B):
        row = alloc.block_tables[i]
        tables[i, : len(row)] = torch.tensor(row, dtype=torch.int32)
    occ = torch.tensor(alloc.occupancy(), dtype=torch.int32)

    # ---- K/V pool, token-major [NB, Hkv, 16, d] until encoded --------------------------
    k32 = _randn_pool((NB, Hkv, BLOCK_SIZE, d), gen)
    v32 = _randn_pool((NB, Hkv, BLOCK_SIZE, d), gen)
    if cfg.peaked_fraction > 0:
        nslots = NB * BLOCK_SIZE
        pick = torch.randperm(nslots, generator=gen)[: round(cfg.peaked_fraction * nslots)]
        blk, off = pick // BLOCK_SIZE, pick % BLOCK_SIZE
        k32[blk, :, off, :] *= cfg.peaked_factor
    if cfg.v_first_block_factor != 1.0 or cfg.v_outlier != 0.0:
        done = set()
        for i, L in enumerate(lens):
            if L <= 0 or alloc.block_tables[i][0] in done:
                continue
            blk = alloc.block_tables[i][0]
            done.add(blk)
            v32[blk] *= cfg.v_first_block_factor
            if cfg.v_outlier != 0.0:
                v32[blk, :, 0, cfg.v_outlier_dim] = cfg.v_outlier * (1 - 2 * (i % 2))
    q32 = torch.randn((B, cfg.num_q_pos, Hq, d), generator=gen)
    q = q32.to(_TORCH_DT[cfg.q_dtype])

    live = torch.arange(BLOCK_SIZE)[None, :] < occ[:, None]          # [NB, 16]
    k_scale = v_scale = None
    if cfg.kv_dtype in ("i8", "fp8"):
        enc = _quantise_int8 if cfg.kv_dtype == "i8" else _quantise_fp8
        k_tok, k_scale = enc(k32, live)
        v_tok, v_scale = enc(v32, live)
        if poison:
            # int8: extreme codes; fp8: NaN codes (any byte of an unused slot may be one)
            kp, vp = (127, -127) if cfg.kv_dtype == "i8" else (0x7F, 0xFF)
            for blk in (occ < BLOCK_SIZE).nonzero().flatten().tolist():
                n = int(occ[blk])
                k_tok[blk, :, n:, :] = kp
                v_tok[blk, :, n:, :] = vp
                if n == 0:
                    k_scale[blk] = float("nan")
                    v_scale[blk] = float("nan")
    else:
        dt = _TORCH_DT[cfg.kv_dtype]
        k_tok, v_tok = k32.to(dt), v32.to(dt)
        if poison:
            for blk in (occ < BLOCK_SIZE).nonzero().flatten().tolist():
                n = int(occ[blk])
                k_tok[blk, :, n:, :] = float("nan")
                v_tok[blk, :, n:, :] = float("nan")
    del k32, v32

    # ---- the step's new token: position L-1 of each sequence ------------------------
    slot_mapping = k_new = v_new = None
    if cfg.append:
        if cfg.kv_dtype in ("i8", "fp8"):
            raise ValueError("an 8-bit cache takes its new tokens through kv_append_quant")
        dt = _TORCH_DT[cfg.kv_dtype]
        k_new = torch.randn((B, Hkv, d), generator=gen).to(dt)
        v_new = torch.randn((B, Hkv, d), generator=gen).to(dt)
        slots = []
        for i, L in enumerate(lens):
            blk = alloc.block_tables[i][(L - 1) // BLOCK_SIZE]
            slots.append(blk * BLOCK_SIZE + (L - 1) % BLOCK_SIZE)
        slot_mapping = torch.tensor(slots, dtype=torch.int64)
        if poison:  # the slot the append must fill starts out as NaN
            for s in slots:
                blk, off = divmod(s, BLOCK_SIZE)
                k_tok[blk, :, off, :] = float("nan")
                v_tok[blk, :, off, :] = float("nan")
    k_cache, v_cache = encode_k(k_tok), encode_v(v_tok)
    del k_tok, v_tok

    tree_mask = None
    if cfg.tree:
        tree_mask = torch.stack([tree_mask_from_parents(random_tree(cfg.num_q_pos, gen))
                                 for _ in range(B)])
    wl = Workload(cfg, q, k_cache, v_cache, k_scale, v_scale, tables,
                  torch.tensor(lens, dtype=torch.int32), slot_mapping, k_new, v_new, occ,
                  meta={"seed": seed, "num_blocks": NB, "max_blocks": max_blocks,
                        "allocator": alloc}, tree_mask=tree_mask)
    if shuffle_batch:
        perm = torch.randperm(B, generator=gen)
        wl = permute_batch(wl, perm)
    return wl


def random_tree(n, gen):
    """Parent list of a random n-node candidate tree in tree order: node 0 is the root
    (parent -1) and node j > 0 hangs under a node drawn uniformly from 0 .. j - 1."""
    parents = [-1]
    for j in range(1, n):
        parents.append(int(torch.randint(0, j, (1,), generator=gen)))
    return parents


def tree_mask_from_parents(parents):
    """[n, n] bool: mask[i][j] is True when node j is node i or one of its ancestors."""
    n = len(parents)
    m = torch.zeros((n, n), dtype=torch.bool)
    for i in range(n):
        j = i
        while j >= 0:
            m[i, j] = True
            j = parents[j]
    return m


def tree_mask_words(mask):
    """Bit rows of a [B, nq, nq] bool mask as the library reads them: [B, nq, ceil(nq/32)]
    int32 words, bit j % 32 of word j // 32 of row i set when candidate j is visible."""
    B, nq, _ = mask.shape
    nw = -(-nq // 32)
    words = torch.zeros((B, nq, nw), dtype=torch.int64)
    for j in range(nq):
        words[:, :, j // 32] |= mask[:, :, j].to(torch.int64) << (j % 32)
    words = torch.where(words >= 2 ** 31, words - 2 ** 32, words)
    return words.to(torch.int32).contiguous()


def permute_batch(wl: Workload, perm):
    """The same workload with its sequences listed in order ``perm``."""
    p = torch.as_tensor(perm, dtype=torch.int64)
    return replace(
        wl, q=wl.q[p].contiguous(), block_tables=wl.block_tables[p].contiguous(),
        seq_lens=wl.seq_lens[p].contiguous(),
        slot_mapping=None if wl.slot_mapping is None else wl.slot_mapping[p].contiguous(),
        k_new=None if wl.k_new is None else wl.k_new[p].contiguous(),
        v_new=None if wl.v_new is None else wl.v_new[p].contiguous(),
        tree_mask=None if wl.tree_mask is None else wl.tree_mask[p].contiguous(),
        meta=dict({k: v for k, v in wl.meta.items() if k != "allocator"},
                  batch_perm=p.tolist()))


def relabel_blocks(wl: Workload, perm):
    """The same logical cache with physical block i moved to block perm[i]
    (data, scales and table entries move together)."""
    perm = torch.as_tensor(perm, dtype=torch.int64)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    def mv(x):
        return None if x is None else x[inv].contiguous()
    t = wl.block_tables.to(torch.int64)
    nt = torch.where(t >= 0, perm[t.clamp(min=0)], t).to(torch.int32)
    sm = None
    if wl.slot_mapping is not None:
        s = wl.slot_mapping
        sm = perm[s // BLOCK_SIZE] * BLOCK_SIZE + s % BLOCK_SIZE
    return replace(wl, k_cache=mv(wl.k_cache), v_cache=mv(wl.v_cache), k_scale=mv(wl.k_scale),
                   v_scale=mv(wl.v_scale), block_tables=nt, slot_mapping=sm,
                   occupancy=mv(wl.occupancy),
                   meta={k: v for k, v in wl.meta.items() if k != "allocator"})


def copy_pairs(wl: Workload, n: int, seed: int = 0):
    """[n, 2] int32 (src, dst) block pairs for a block copy: distinct sources drawn from the
    blocks that hold live tokens, distinct destinations from the blocks that hold none (so
    no destination is a source), as copy-on-write produces them."""
    gen = torch.Generator().manual_seed(seed)
    used = (wl.occupancy > 0).nonzero().flatten()
    free = (wl.occupancy == 0).nonzero().flatten()
    if n > used.numel() or n > free.numel():
        raise ValueError("not enough used or free blocks for the requested pairs")
    src = used[torch.randperm(used.numel(), generator=gen)[:n]]
    dst = free[torch.randperm(free.numel(), generator=gen)[:n]]
    return torch.stack([src, dst], dim=1).to(torch.int32).contiguous()


def _quantise_int8(x32, live):
    """Symmetric int8 encoding per (block, KV head) of a token-major [NB, H, 16, d] pool:
    scale = max|x| / 127 over the block's live slots, x_q = round-half-even(x / scale)
    clamped to [-127, 127] (Lecture 10's affine rule with zero point 0; In-depth §5.2
    per-head scales)."""
    m = live[:, None, :, None].expand_as(x32)
    amax = torch.where(m, x32.abs(), torch.zeros(())).amax(dim=(2, 3))      # [NB, H]
    scale = (amax / 127.0).to(torch.float32)
    safe = torch.where(scale > 0, scale, torch.ones(()))
    xq = torch.round(x32 / safe[:, :, None, None]).clamp_(-127, 127)
    xq = torch.where(scale[:, :, None, None] > 0, xq, torch.zeros(()))
    return xq.to(torch.int8), scale


def _quantise_fp8(x32, live):
    """e4m3 encoding per (block, KV head) of a token-major [NB, H, 16, d] pool: scale =
    max|x| / 448 over the block's live slots, codes = x / scale converted to torch's
    float8_e4m3fn (round to nearest even) after clamping to +-448, returned as uint8."""
    m = live[:, None, :, None].expand_as(x32)
    amax = torch.where(m, x32.abs(), torch.zeros(())).amax(dim=(2, 3))
    scale = (amax / 448.0).to(torch.float32)
    safe = torch.where(scale > 0, scale, torch.ones(()))
    y = (x32 / safe[:, :, None, None]).clamp_(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    codes = torch.where(scale[:, :, None, None] > 0, codes, torch.zeros((), dtype=torch.uint8))
    return codes, scale


def encode_k(k_tok):
    """Token-major K [NB, H, 16, d] -> the cache format [NB, H, d/x, 16, x], x = 16 / element
    bytes (each 16-byte column of the 16 tokens' rows contiguous)."""
    NB, H, T, d = k_tok.shape
    x = 16 // k_tok.element_size()
    return k_tok.reshape(NB, H, T, d // x, x).permute(0, 1, 3, 2, 4).contiguous()


def encode_v(v_tok):
    """Token-major V [NB, H, 16, d] -> the cache format [NB, H, d, 16]."""
    return v_tok.transpose(2, 3).contiguous()


def k_token_rows(k_cache):
    """The cache-format K pool viewed back as token-major [NB, H, 16, d] (a copy)."""
    NB, H, C, T, x = k_cache.shape
    return k_cache.permute(0, 1, 3, 2, 4).reshape(NB, H, T, C * x)


def scaled(cfg, **changes) -> Config:
    """A copy of a config with some fields changed (smaller parity cases)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    return replace(cfg, **changes)
