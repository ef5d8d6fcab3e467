"""Host harness: block manager semantics and the seeded workloads' structure."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import kvsize, paging


def test_allocator_semantics():
    a = W.BlockAllocator(10, 16)
    assert a.allocate("x", 33) == [9, 8, 7]          # ceil(33/16) blocks, popped from the end
    a.token_counts["x"] = 48
    a.append_token("x")                               # 48 tokens fill 3 blocks -> new block
    assert len(a.block_tables["x"]) == 4
    a.append_token("x")
    assert len(a.block_tables["x"]) == 4
    with pytest.raises(RuntimeError):
        a.allocate("y", 16 * 7)
    a.release("x")
    assert sorted(a.free_blocks) == list(range(10))
    b = W.BlockAllocator(2, 16)
    b.allocate("z", 32)
    with pytest.raises(RuntimeError):
        b.append_token("z")


def test_fork_shares_prefix_refcounted():
    a = W.BlockAllocator(20, 16)
    a.allocate(0, 64)
    a.fork(0, 1, 32, 64)
    assert a.block_tables[1][:2] == a.block_tables[0][:2]
    assert set(a.block_tables[1][2:]).isdisjoint(a.block_tables[0])
    a.release(0)
    assert a.block_tables[1][0] not in a.free_blocks      # still referenced
    a.release(1)
    assert sorted(a.free_blocks) == list(range(20))


def test_copy_on_write_on_the_first_write_into_a_shared_block():
    a = W.BlockAllocator(12, 16, free_order=list(range(12)))
    a.allocate(0, 37)                                 # blocks 11, 10, 9; 5 tokens in block 9
    a.fork_all(0, 1)
    assert a.block_tables[1] == [11, 10, 9] and a.refcount[9] == 2
    slot, copy = a.append_token(1)                    # writes position 37 into shared block 9
    assert copy == (9, 8) and a.block_tables[1] == [11, 10, 8]
    assert slot == 8 * 16 + 5
    assert a.refcount[9] == 1 and a.refcount[8] == 1 and a.refcount[11] == 2
    slot, copy = a.append_token(0)                    # block 9 is now the parent's alone
    assert copy is None and slot == 9 * 16 + 5
    for _ in range(10):                               # positions 38..47 stay in block 8
        assert a.append_token(1)[1] is None
    slot, copy = a.append_token(1)                    # position 48: a new block, no copy
    assert copy is None and a.block_tables[1] == [11, 10, 8, 7] and slot == 7 * 16
    a.release(0)
    assert a.refcount[11] == 1 and 9 in a.free_blocks and 11 not in a.free_blocks
    a.release(1)
    assert sorted(a.free_blocks) == list(range(12))
    b = W.BlockAllocator(8, 16)
    b.allocate(0, 32)                                  # two full blocks
    b.fork_all(0, 1)
    slot, copy = b.append_token(1)                     # full shared block: new block, no copy
    assert copy is None and b.block_tables[1][:2] == b.block_tables[0]


@pytest.mark.parametrize("name", ["tiny_fp32", "llama3_8b", "verify_int8"])
def test_tables_distinct_and_sized(name):
    wl = W.generate(name)
    seen = set()
    for b, L in enumerate(wl.seq_lens.tolist()):
        n = kvsize.blocks_needed(L)
        row = wl.block_tables[b].tolist()
        assert all(x >= 0 for x in row[:n]) and all(x == -1 for x in row[n:])
        assert seen.isdisjoint(row[:n])
        seen.update(row[:n])
    assert max(seen) < wl.k_cache.shape[0]


def test_tiny_config_lengths_and_append_slots():
    wl = W.generate("tiny_fp32")
    assert wl.seq_lens.tolist() == [38, 129, 201, 512]
    assert wl.block_tables.shape[0] == 4 and wl.k_cache.shape == (256, 2, 16, 16, 4)
    assert wl.v_cache.shape == (256, 2, 64, 16)
    for b, L in enumerate(wl.seq_lens.tolist()):
        assert int(wl.slot_mapping[b]) == paging.slot_of(wl.block_tables[b].tolist(), L - 1)
        blk, off = divmod(int(wl.slot_mapping[b]), 16)
        assert torch.isnan(W.k_token_rows(wl.k_cache)[blk, :, off, :]).all()  # only the append fills it
        assert torch.isnan(wl.v_cache[blk, :, :, off]).all()


def test_shared_prefix_structure():
    wl = W.generate("llama2_70b_prefix")
    t = wl.block_tables
    assert wl.k_cache.shape[0] == 5120
    for grp in range(6):
        rows = t[grp * 5: grp * 5 + 5]
        assert (rows[:, :128] == rows[0, :128]).all()
        priv = [set(r[128:].tolist()) for r in rows]
        for i in range(5):
            for j in range(i + 1, 5):
                assert priv[i].isdisjoint(priv[j])
    assert len(set(t.flatten().tolist())) == 5120


def test_peaked_positions():
    cfg = W.scaled("long_128k", lengths=(4096,) * 4)
    wl = W.generate(cfg)
    k = W.k_token_rows(wl.k_cache).float()
    big = (k.abs().amax(dim=(1, 3)) > 6.5)               # [NB, 16] slot-level
    frac = big.float().mean().item()
    assert 0.006 < frac < 0.014


def test_int8_encoding_invariants():
    wl = W.generate(W.scaled("verify_int8", batch=4, length_range=(20, 300)), poison=False)
    occ = wl.occupancy
    for cache, scale in ((W.k_token_rows(wl.k_cache), wl.k_scale),
                         (wl.v_cache.transpose(2, 3), wl.v_scale)):
        assert cache.dtype == torch.int8 and int(cache.abs().max()) <= 127
        for blk in range(cache.shape[0]):
            n = int(occ[blk])
            if n == 0:
                continue
            live = cache[blk, :, :n, :]
            # the largest-magnitude live element encodes to +-127 in every head
            assert (live.abs().amax(dim=(1, 2)) == 127).all()
            assert (scale[blk] > 0).all()


def test_int8_dequant_error_bound():
    cfg = W.scaled("verify_int8", batch=2, length_range=(40, 64))
    gen_a = W.generate(cfg, poison=False)
    # regenerate the fp32 pool the encoder saw (same seed, same draw order)
    g = torch.Generator().manual_seed(cfg.seed)
    W._draw_lengths(cfg, g)
    NB = gen_a.k_cache.shape[0]
    torch.randperm(NB, generator=g)
    k32 = W._randn_pool((NB, cfg.num_kv_heads, 16, cfg.head_dim), g)
    deq = W.k_token_rows(gen_a.k_cache).float() * gen_a.k_scale[:, :, None, None]
    err = (deq - k32).abs()
    bound = gen_a.k_scale[:, :, None, None] / 2 * (1 + 1e-6)
    live = (torch.arange(16)[None, :] < gen_a.occupancy[:, None])[:, None, :, None]
    assert bool(((err <= bound) | ~live).all())


def test_k_encoding_roundtrip():
    x = torch.arange(3 * 2 * 16 * 64, dtype=torch.float32).reshape(3, 2, 16, 64)
    for dt, xw in ((torch.float32, 4), (torch.bfloat16, 8), (torch.int8, 16)):
        t = (x % 100).to(dt)
        enc = W.encode_k(t)
        assert enc.shape == (3, 2, 64 // xw, 16, xw)
        # element k of token o at [k // x][o][k % x]
        assert enc[1, 1, 5 // xw, 7, 5 % xw] == t[1, 1, 7, 5]
        assert torch.equal(W.k_token_rows(enc), t)
    v = W.encode_v(x)
    assert v.shape == (3, 2, 64, 16) and v[2, 0, 9, 4] == x[2, 0, 4, 9]


def test_seeded_determinism():
    a = W.generate("tiny_fp32")
    b = W.generate("tiny_fp32")
    assert torch.equal(a.block_tables, b.block_tables)
    assert torch.equal(a.q, b.q)
    assert torch.equal(a.k_cache.nan_to_num(), b.k_cache.nan_to_num())


def test_relabel_moves_data_with_tables():
    wl = W.generate(W.scaled("tiny_fp32", head_dim=8))
    perm = torch.randperm(256, generator=torch.Generator().manual_seed(1))
    w2 = W.relabel_blocks(wl, perm)
    for b in range(4):
        L = int(wl.seq_lens[b])
        K1, V1 = paging.depage(wl.k_cache.numpy(), wl.v_cache.numpy(), "f32",
                               wl.block_tables[b].numpy(), L, 1)
        K2, V2 = paging.depage(w2.k_cache.numpy(), w2.v_cache.numpy(), "f32",
                               w2.block_tables[b].numpy(), L, 1)
        assert np.array_equal(K1, K2, equal_nan=True) and np.array_equal(V1, V2, equal_nan=True)


def test_v_scale_outliers():
    """An outlier element in each sequence's first block raises that block's V scale to
    outlier / 127 (int8) and leaves the block's other codes at 0; a first-block factor
    scales the first block's V scale by the factor."""
    base = dict(batch=4, length_range=(40, 200))
    big = W.generate(W.scaled("verify_int8", v_outlier=4e4, **base), poison=False)
    ref = W.generate(W.scaled("verify_int8", **base), poison=False)
    small = W.generate(W.scaled("verify_int8", v_first_block_factor=1e-4, **base), poison=False)
    v = big.v_cache.transpose(2, 3)                       # token-major codes
    for b in range(4):
        first = int(big.block_tables[b, 0])
        assert torch.allclose(big.v_scale[first], torch.full((8,), 4e4 / 127), rtol=1e-6)
        sign = 1 - 2 * (b % 2)
        assert (v[first, :, 0, 5] == 127 * sign).all()
        others = v[first].clone()
        others[:, 0, 5] = 0
        assert int(others.abs().max()) == 0                # N(0,1) values round to code 0
        r = small.v_scale[first] / ref.v_scale[first]
        assert torch.allclose(r, torch.full((8,), 1e-4), rtol=1e-5)
        # later blocks are untouched
        rest = big.block_tables[b, 1:int(-(-int(big.seq_lens[b]) // 16))].long()
        assert torch.equal(big.v_scale[rest], ref.v_scale[rest])
