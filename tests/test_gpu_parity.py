"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded
inputs.  Bit-exact for append and gather; for attention max |gpu - oracle| within 1e-5
(fp32 KV), 2e-3 (bf16 KV), 4e-3 (int8 KV)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention, paging, quant
from _helpers import (TOL, Dev, dims_of, gpu_append, gpu_attention, gpu_decode_step,
                      gpu_multi_query, max_err, oracle_attention, oracle_caches, raw, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import paged_gqa_decode_kv_amd as P
    assert torch.cuda.is_available()
    return P


def _bits(x):
    x = x.detach().cpu()
    if x.dtype == torch.float32:
        return x.view(torch.int32)
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16)
    return x


def _small(name, spare=7, **kw):
    base = dict(lengths=None, pool_blocks=None, shared_groups=0, shared_group_size=0,
                shared_prefix_tokens=0, lengths_are_cached=False, peaked_fraction=0.0)
    base.update(kw)
    return W.generate(W.scaled(name, **base), spare_blocks=spare)


def _assert_close(out, ref, tol, pairs=None, group=None, rel_dims=None):
    """max |out - ref| <= tol over the compared elements.  rel_dims: head dims that carry an
    outlier value; there fp16 weights round to 2^-12 of the outlier's magnitude, so the
    bound is tol * max(1, |ref|) (the other dims keep the absolute tol)."""
    if rel_dims is None:
        err = max_err(out, ref, pairs, group)
        say(f"  max abs err {err:.3e} (tol {tol:.0e})")
        assert err <= tol
        return
    assert pairs is None
    g = out.detach().cpu().numpy().astype(np.float64).reshape(ref.shape)
    assert np.isfinite(g).all(), "non-finite GPU output"
    diff = np.abs(g - ref)
    keep = np.ones(ref.shape[-1], bool)
    keep[list(rel_dims)] = False
    e_abs = float(diff[..., keep].max())
    e_rel = float((diff[..., ~keep] / np.maximum(1.0, np.abs(ref[..., ~keep]))).max())
    say(f"  max abs err {e_abs:.3e} off the outlier dims, max rel err {e_rel:.3e} on them "
        f"(tol {tol:.0e})")
    assert e_abs <= tol and e_rel <= tol


def _check_attention(P, wl, tol=None, split=None, pairs=None, append=True, balanced=None,
                     interleave=False, ref=None, rel_dims=None):
    """ref: the oracle's (out, lse) for this workload's caches (after the append when
    `append`), computed once by the caller when several modes are compared with it."""
    c = wl.cfg
    tol = TOL[c.kv_dtype] if tol is None else tol
    say(f"[case] {c.name} B={c.batch} Hq={c.num_q_heads} Hkv={c.num_kv_heads} d={c.head_dim} "
        f"nq={c.num_q_pos} kv={c.kv_dtype} split={split} balanced={balanced} "
        f"interleave={interleave} seed={wl.meta['seed']}")
    dv = Dev(wl, interleave)
    if append and wl.slot_mapping is not None:
        gpu_append(P, wl, dv)
    out, parts, out_lse = gpu_attention(P, wl, dv, split=split, balanced=balanced)
    torch.cuda.synchronize()
    if ref is None:
        kc, vc = oracle_caches(wl, appended=append)
        ref, ref_lse = oracle_attention(wl, kc, vc, pairs=pairs)
    else:
        ref, ref_lse = ref
    _assert_close(out, ref, tol, pairs, c.group_size, rel_dims)
    if out_lse is not None:
        g = out_lse.cpu().numpy().reshape(ref_lse.shape)
        r = ref_lse
        sel = np.isfinite(r)
        if pairs is not None:
            m = np.zeros(r.shape, bool)
            for b, kv in pairs:
                m[b, ..., kv * c.group_size:(kv + 1) * c.group_size] = True
            sel &= m
        assert np.all(np.abs(g[sel] - r[sel]) <= 1e-3 * np.maximum(1, np.abs(r[sel])))
        empty = r == -np.inf
        if pairs is None:
            assert np.all(g[empty] == -np.inf)
    return out, parts, dv


# ---- append and gather: bit exact -------------------------------------------------
@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("name,kw", [("tiny_fp32", {}),
                                     ("llama3_8b", dict(batch=9, length_range=(1, 300)))])
def test_kv_append_bit_exact(P, name, kw, interleave):
    wl = W.generate(W.scaled(name, **kw), spare_blocks=3) if kw else W.generate(name)
    say(f"[case] append {wl.cfg.name} interleave={interleave}")
    dv = Dev(wl, interleave)
    gpu_append(P, wl, dv)
    torch.cuda.synchronize()
    kc, vc = oracle_caches(wl, appended=True)
    gk, gv = dv.caches_host()
    assert np.array_equal(raw(gk).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(raw(gv).view(np.uint8), vc.view(np.uint8))


def test_kv_append_skips_negative_and_out_of_pool_slots(P):
    wl = W.generate(W.scaled("tiny_fp32", batch=4))
    say("[case] append with skipped slots")
    sm = wl.slot_mapping.clone()
    sm[1] = -1
    sm[2] = wl.k_cache.shape[0] * 16          # one past the pool
    dv = Dev(wl)
    dv.slot_mapping = sm.cuda()
    d = dims_of(P, wl)
    P.kv_append(d, dv.k_new, dv.v_new, dv.slot_mapping, 4, dv.k_cache, dv.v_cache)
    torch.cuda.synchronize()
    sm_or = sm.numpy().copy()
    sm_or[2] = -1
    kc, vc = paging.append(raw(wl.k_cache), raw(wl.v_cache), raw(wl.k_new), raw(wl.v_new), sm_or)
    assert np.array_equal(raw(dv.k_cache.cpu()).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(raw(dv.v_cache.cpu()).view(np.uint8), vc.view(np.uint8))


@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("name", ["tiny_fp32", "llama3_8b", "verify_int8", "llama3_8b_fp8"])
def test_kv_gather_bit_exact(P, name, interleave):
    wl = _small(name, batch=5, length_range=(0, 333), append=False)
    say(f"[case] gather {name} interleave={interleave}")
    dv = Dev(wl, interleave)
    c = wl.cfg
    maxL = int(wl.seq_lens.max()) + 3
    fill = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8,
            "fp8": torch.uint8}[c.kv_dtype]
    k_out = torch.full((c.batch, c.num_kv_heads, maxL, c.head_dim), 7, dtype=fill, device="cuda:0")
    v_out = k_out.clone()
    P.kv_gather(dims_of(P, wl, dv), dv.k_cache, dv.v_cache, dv.block_tables, dv.seq_lens, maxL,
                k_out, v_out)
    torch.cuda.synchronize()
    ko, vo = paging.gather(raw(wl.k_cache), raw(wl.v_cache), wl.block_tables.numpy(),
                           wl.seq_lens.numpy(), raw(k_out.cpu()), raw(v_out.cpu()))
    assert np.array_equal(raw(k_out.cpu()).view(np.uint8), ko.view(np.uint8))
    assert np.array_equal(raw(v_out.cpu()).view(np.uint8), vo.view(np.uint8))


# ---- block copy (copy-on-write): bit exact ---------------------------------------------
def _gpu_copy(P, wl, dv, pairs):
    pd = pairs.to("cuda:0")
    P.kv_copy_blocks(dims_of(P, wl, dv), pd, pairs.shape[0], dv.k_cache, dv.v_cache,
                     dv.k_scale, dv.v_scale)
    torch.cuda.synchronize()


def _check_pool(dv, kc, vc, ks=None, vs=None):
    gk, gv = dv.caches_host()
    assert np.array_equal(raw(gk).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(raw(gv).view(np.uint8), vc.view(np.uint8))
    if ks is not None:
        assert np.array_equal(raw(dv.k_scale).view(np.uint8), ks.view(np.uint8))
        assert np.array_equal(raw(dv.v_scale).view(np.uint8), vs.view(np.uint8))


@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("name", ["tiny_fp32", "llama3_8b", "verify_int8", "llama3_8b_fp8"])
def test_kv_copy_blocks_bit_exact(P, name, interleave):
    wl = _small(name, spare=12, batch=6, length_range=(1, 200), append=False)
    nb = wl.k_cache.shape[0]
    pairs = W.copy_pairs(wl, 9, seed=5)
    free = sorted(set((wl.occupancy == 0).nonzero().flatten().tolist()) -
                  set(pairs[:, 1].tolist()))
    skip = torch.tensor([[-1, free[0]], [int(pairs[0, 0]), nb], [free[1], free[1]],
                         [nb + 5, free[2]], [int(pairs[1, 0]), -7]], dtype=torch.int32)
    allp = torch.cat([pairs[:4], skip, pairs[4:]]).contiguous()
    say(f"[case] copy_blocks {name} interleave={interleave} pairs={allp.shape[0]} NB={nb}")
    dv = Dev(wl, interleave)
    _gpu_copy(P, wl, dv, allp)
    kc, vc, ks, vs = paging.copy_blocks(raw(wl.k_cache), raw(wl.v_cache), allp.numpy(),
                                        raw(wl.k_scale), raw(wl.v_scale))
    _check_pool(dv, kc, vc, ks, vs)
    # no pairs: nothing launched, nothing changed
    P.kv_copy_blocks(dims_of(P, wl, dv), allp.cuda(), 0, dv.k_cache, dv.v_cache, dv.k_scale,
                     dv.v_scale)
    torch.cuda.synchronize()
    _check_pool(dv, kc, vc, ks, vs)


@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("name", ["tiny_fp32", "llama3_8b"])
def test_copy_on_write_then_decode(P, name, interleave):
    """Parallel sampling: sequences fork with every block shared (the partly filled last
    one too); on the next token each writer of a still-shared block gets a private copy.
    GPU: block copy, append, decode attention; oracle: the same three steps."""
    from dataclasses import replace
    wl = _small(name, spare=16, lengths=[37, 50, 16, 129, 3], batch=5, append=False)
    c = wl.cfg
    alloc = wl.meta["allocator"]
    for parent, child in [(0, 5), (3, 6), (4, 7), (4, 8)]:
        alloc.fork_all(parent, child)
    B = 9
    slots, pairs = [0] * B, []
    for i in [5, 0, 6, 3, 7, 8, 4, 1, 2]:          # children write first: they copy
        slots[i], cp = alloc.append_token(i)
        if cp is not None:
            pairs.append(cp)
    assert len(pairs) == 4
    rows = [alloc.block_tables[i] for i in range(B)]
    tables = torch.full((B, max(map(len, rows))), -1, dtype=torch.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = torch.tensor(r, dtype=torch.int32)
    gen = torch.Generator().manual_seed(77)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    q = torch.randn((B, 1, c.num_q_heads, c.head_dim), generator=gen).to(dt[c.q_dtype])
    kn = torch.randn((B, c.num_kv_heads, c.head_dim), generator=gen).to(dt[c.kv_dtype])
    vn = torch.randn((B, c.num_kv_heads, c.head_dim), generator=gen).to(dt[c.kv_dtype])
    wl2 = replace(wl, cfg=replace(c, batch=B, lengths=None), q=q, block_tables=tables,
                  seq_lens=torch.tensor([alloc.token_counts[i] for i in range(B)],
                                        dtype=torch.int32),
                  slot_mapping=torch.tensor(slots, dtype=torch.int64), k_new=kn, v_new=vn)
    pt = torch.tensor(pairs, dtype=torch.int32)
    say(f"[case] copy-on-write {name} interleave={interleave} pairs={pairs}")
    dv = Dev(wl2, interleave)
    _gpu_copy(P, wl2, dv, pt)
    gpu_append(P, wl2, dv)
    out, _, _ = gpu_attention(P, wl2, dv)
    out_b, _, _ = gpu_attention(P, wl2, dv, balanced=0)
    torch.cuda.synchronize()
    kc, vc, _, _ = paging.copy_blocks(raw(wl.k_cache), raw(wl.v_cache), pt.numpy())
    kc, vc = paging.append(kc, vc, raw(kn), raw(vn), np.array(slots))
    _check_pool(dv, kc, vc)
    ref, _ = oracle_attention(wl2, kc, vc)
    for o in (out, out_b):
        err = max_err(o, ref)
        say(f"  max abs err {err:.3e}")
        assert err <= TOL[c.kv_dtype]
    # a child and its parent share every block but the last
    assert rows[5][:-1] == rows[0][:-1] and rows[5][-1] != rows[0][-1]


def test_kv_copy_blocks_full_llama3_8b_pool(P):
    """The benchmark's bulk copy: 2048 pairs on the Llama-3-8B pool, whole pool compared."""
    wl = W.generate(W.scaled("llama3_8b", append=False), spare_blocks=2048)
    pairs = W.copy_pairs(wl, 2048, seed=3)
    say(f"[case] copy_blocks full llama3_8b pairs=2048 NB={wl.k_cache.shape[0]}")
    dv = Dev(wl, True)
    _gpu_copy(P, wl, dv, pairs)
    kc, vc, _, _ = paging.copy_blocks(raw(wl.k_cache), raw(wl.v_cache), pairs.numpy())
    _check_pool(dv, kc, vc)


# ---- attention, small shapes (several tiles, ragged tails, edge cases) ---------------
def test_tiny_fp32_config(P):
    wl = W.generate("tiny_fp32")
    out, _, dv = _check_attention(P, wl)
    # the same cache read with the pre-append lengths
    say("[case] tiny_fp32 pre-append lengths")
    lens = wl.seq_lens - 1
    out2, _, _ = gpu_attention(P, wl, dv, seq_lens=lens.cuda())
    torch.cuda.synchronize()
    kc, vc = oracle_caches(wl)
    ref, _ = oracle_attention(wl, kc, vc, seq_lens=lens.numpy())
    assert max_err(out2, ref) <= 1e-5


CASES = [
    # name, overrides
    ("llama3_8b", dict(batch=6, length_range=(1, 700))),
    ("llama3_8b", dict(batch=5, length_range=(1, 300), head_dim=64, num_q_heads=16, num_kv_heads=2)),
    ("llama3_8b", dict(batch=3, length_range=(40, 400), num_q_heads=32, num_kv_heads=1)),   # MQA
    ("llama3_8b", dict(batch=3, length_range=(40, 400), num_q_heads=4, num_kv_heads=4)),    # MHA
    ("llama3_8b", dict(batch=2, length_range=(100, 300), num_q_heads=64, num_kv_heads=1)),  # 64 rows
    ("llama2_70b_prefix", dict(batch=4, length_range=(17, 520))),                          # G = 8
    ("tiny_fp32", dict(batch=5, length_range=(1, 400), head_dim=128, pool_blocks=None)),
    ("tiny_fp32", dict(batch=4, length_range=(1, 200), num_q_heads=12, num_kv_heads=4)),
    ("verify_int8", dict(batch=5, length_range=(6, 600))),
    ("verify_int8", dict(batch=4, length_range=(1, 300), head_dim=64, num_q_heads=8,
                         num_kv_heads=2)),
    ("verify_int8", dict(batch=4, length_range=(1, 300), num_q_pos=1)),
    ("verify_int8", dict(batch=4, length_range=(1, 40), num_q_pos=3, num_q_heads=16,
                         num_kv_heads=8)),
    ("llama3_8b", dict(batch=4, length_range=(1, 200), num_q_pos=4, append=False)),     # bf16 verify
    ("llama3_8b_fp8", dict(batch=6, length_range=(1, 700))),                            # fp8 KV
    ("llama3_8b_fp8", dict(batch=4, length_range=(1, 300), head_dim=64, num_q_heads=16,
                           num_kv_heads=2)),
    ("verify_int8", dict(batch=5, length_range=(6, 600), kv_dtype="fp8")),              # fp8 verify
]


@pytest.mark.parametrize("name,kw", CASES)
def test_attention_small(P, name, kw):
    wl = _small(name, **kw)
    _check_attention(P, wl)


# K and V tiles of one (block, head) side by side in one allocation (tile stride 2 tiles)
@pytest.mark.parametrize("name,kw", [CASES[0], CASES[2], CASES[6], CASES[8], CASES[12]])
def test_attention_small_interleaved(P, name, kw):
    wl = _small(name, **kw)
    _check_attention(P, wl, interleave=True)
    _check_attention(P, wl, interleave=True, balanced=0)
    _check_attention(P, wl, interleave=True, balanced=7)
    if wl.cfg.num_q_pos == 1:
        _check_attention(P, wl, interleave=True, split=(64, 16))


def test_empty_and_short_sequences(P):
    wl = _small("llama3_8b", batch=6, lengths=(0, 1, 15, 16, 17, 0), append=False)
    out, _, _ = _check_attention(P, wl)
    assert (out[0] == 0).all() and (out[5] == 0).all()


def test_verify_rows_that_see_nothing(P):
    wl = _small("verify_int8", batch=3, lengths=(3, 6, 1))
    out, _, _ = _check_attention(P, wl)
    assert (out[0, :3] == 0).all() and (out[2, :5] == 0).all()


@pytest.mark.parametrize("split", [(512, 16), (256, 3), (16, 400), (1024, 1)])
def test_split_merge_small(P, split):
    wl = _small("long_128k", batch=4, lengths=(3000, 1, 17, 4101), peaked_fraction=0.01)
    out, (po, pl), _ = _check_attention(P, wl, split=split)
    # partials against the oracle's per-partition results
    kc, vc = oracle_caches(wl)
    c = wl.cfg
    ro, rl = attention.paged_attention_partitions(
        raw(wl.q), "bf16", kc, vc, "bf16", wl.block_tables.numpy(), wl.seq_lens.numpy(),
        float(np.float32(wl.sm_scale)), split[0], split[1])
    po, pl = po.cpu().numpy(), pl.cpu().numpy()
    for b, L in enumerate(wl.seq_lens.tolist()):
        n = attention.partitions_used(L, *split)
        assert np.abs(po[b, :, :n] - ro[b, 0, :, :n]).max() <= 2e-3
        assert np.abs(pl[b, :, :n] - rl[b, 0, :, :n]).max() <= 1e-3


# ---- balanced mode: the batch's blocks dealt evenly over G workgroups -----------------
@pytest.mark.parametrize("G", [1, 3, 7, 64, 0])
@pytest.mark.parametrize("name,kw", [
    ("llama3_8b", dict(batch=6, length_range=(1, 700))),
    ("verify_int8", dict(batch=5, length_range=(1, 600))),
    ("tiny_fp32", dict(batch=5, length_range=(1, 400))),
])
def test_balanced_small(P, name, kw, G):
    wl = _small(name, **kw)
    _check_attention(P, wl, balanced=G)


@pytest.mark.parametrize("name,kw", [
    ("llama3_8b", dict(batch=3, length_range=(40, 400), num_q_heads=64, num_kv_heads=1)),  # 64 rows
    ("llama3_8b", dict(batch=6, lengths=(0, 1, 15, 16, 17, 0), append=False)),
    ("verify_int8", dict(batch=3, lengths=(3, 6, 1))),
    ("llama3_8b", dict(batch=4, length_range=(1, 200), num_q_pos=4, append=False)),
    ("llama2_70b_prefix", dict(batch=4, length_range=(17, 520), head_dim=64)),
])
def test_balanced_edge_cases(P, name, kw):
    wl = _small(name, **kw)
    _check_attention(P, wl, balanced=0)
    _check_attention(P, wl, balanced=5)


@pytest.mark.parametrize("G", [1, 2, 5, 33])
@pytest.mark.parametrize("name,kw", [
    ("llama3_8b", dict(num_q_pos=6)),                    # bf16, 24 rows
    ("verify_int8", dict()),                             # int8, 24 rows
    ("llama3_8b_fp8", dict(num_q_pos=6)),                # fp8, 24 rows
    ("tiny_fp32", dict(num_q_pos=7, head_dim=128)),      # fp32, 28 rows
    ("mistral_7b_window", dict(num_q_pos=6, sliding_window=300)),  # window: lists start late
    ("llama2_70b_prefix", dict(num_q_pos=3, head_dim=64)),         # d64, 8 heads a group: 24 rows
])
def test_balanced_two_tiles_workgroup_combine(P, name, kw, G):
    """Two row tiles per wave: a segment cut between waves of one workgroup is combined in
    LDS (later waves park their rows, the segment's first wave of the workgroup adds them at
    the end of its slice) and one partial per workgroup reaches the merge kernel.  Lengths
    from empty to several slices long, and workgroup counts from one (every segment combined
    on chip) to many (segments crossing several workgroups)."""
    wl = _small(name, batch=7, lengths=(0, 900, 17, 2000, 1, 333, 1200), append=False, **kw)
    _check_attention(P, wl, balanced=G)


@pytest.mark.parametrize("kv,G", [("bf16", 300), ("i8", 97), ("fp8", 512)])
def test_balanced_two_tiles_many_pieces(P, kv, G):
    """One long sequence on one KV head (24 rows) dealt over hundreds of workgroups: its one
    segment leaves one partial per workgroup, so the two-tile merge runs many rounds of
    four pieces a row (and the workgroup combine has every slice cut)."""
    kw = dict(batch=1, lengths=(6000,), num_q_heads=4, num_kv_heads=1, num_q_pos=6,
              append=False, kv_dtype=kv)
    wl = _small("llama3_8b", **kw)
    _check_attention(P, wl, balanced=G)


def test_balanced_workspace_errors(P):
    wl = _small("llama3_8b", batch=2, length_range=(1, 50), append=False)
    c = wl.cfg
    d = dims_of(P, wl)
    dv = Dev(wl)
    n = P.paged_attn_balanced_workspace_bytes(d, 1, 4)
    assert n > 0
    ws = torch.empty(n - 4, dtype=torch.uint8, device="cuda:0")
    out = torch.empty((c.batch, 1, c.num_q_heads, c.head_dim), device="cuda:0")
    with pytest.raises(P.PagedAttnError) as e:
        P.paged_attn_balanced(d, 1, dv.q, dv.k_cache, dv.v_cache, None, None, dv.block_tables,
                              dv.seq_lens, 0.1, 4, ws, out)
    assert e.value.status == -6
    assert P.paged_attn_balanced_workgroups(d, 1) >= 256
    with pytest.raises(P.PagedAttnError) as e:
        P.paged_attn_balanced_merge(d, 1, 4, ws, out)
    assert e.value.status == -6


# ---- quantising append into an int8 cache: bit exact --------------------------------------
def _rand_bf16(gen, shape, scale=1.0):
    return (torch.randn(shape, generator=gen) * scale).to(torch.bfloat16)


def _interleave_i8(kc, vc):
    nb, h = kc.shape[:2]
    tile = kc[0, 0].numel()
    comb = torch.empty((nb, h, 2, tile), dtype=torch.int8, device="cuda:0")
    comb[:, :, 0] = kc.reshape(nb, h, tile).cuda()
    comb[:, :, 1] = vc.reshape(nb, h, tile).cuda()
    return comb, comb.data_ptr() + tile, 2 * tile


@pytest.mark.parametrize("kind", ["i8", "fp8"])
@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("d,hkv", [(128, 8), (64, 2)])
def test_kv_append_quant_bit_exact(P, d, hkv, interleave, kind):
    gen = torch.Generator().manual_seed(d + hkv + interleave)
    nb, S, T = 40, 24, 20
    kc = torch.randint(-128, 128, (nb, hkv, d // 16, 16, 16), generator=gen, dtype=torch.int8)
    vc = torch.randint(-128, 128, (nb, hkv, d, 16), generator=gen, dtype=torch.int8)
    ks = torch.rand((nb, hkv), generator=gen)
    vs = torch.rand((nb, hkv), generator=gen)
    kst = _rand_bf16(gen, (S, hkv, 16, d), 2.0)
    vst = _rand_bf16(gen, (S, hkv, 16, d), 0.5)
    kn = _rand_bf16(gen, (T, hkv, d), 3.0)
    vn = _rand_bf16(gen, (T, hkv, d))
    kn[3, 1 % hkv, 5] = 200.0                                   # a token that raises the scale
    blocks = torch.randperm(nb, generator=gen)[:T]
    offs = torch.randint(0, 16, (T,), generator=gen)
    offs[:3] = torch.tensor([0, 15, 1])
    slots = (blocks * 16 + offs).to(torch.int64)
    rows = torch.randperm(S, generator=gen)[:T].to(torch.int32)
    slots[4], slots[5], rows[6], rows[7] = -1, nb * 16, -1, S    # skipped tokens
    say(f"[case] append_quant {kind} d={d} hkv={hkv} interleave={interleave}")
    if interleave:
        comb, vptr, stride = _interleave_i8(kc, vc)
        gk, gv = comb, vptr
    else:
        gk, gv, stride = kc.cuda(), vc.cuda(), 0
    dims = P.make_dims(1, hkv, hkv, d, 1, nb, "bf16", kind, kv_tile_stride=stride)
    dks, dvs, dkst, dvst = ks.cuda(), vs.cuda(), kst.cuda(), vst.cuda()
    P.kv_append_quant(dims, kn.cuda(), vn.cuda(), slots.cuda(), rows.cuda(), T, dkst, dvst, gk, gv,
                      dks, dvs)
    torch.cuda.synchronize()
    r = lambda x: x.view(torch.int16).numpy()
    ok, ov, oks, ovs, okst, ovst = quant.append_quant(
        kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), r(kst), r(vst), r(kn), r(vn),
        slots.numpy(), rows.numpy(), kind=kind)
    if interleave:
        hk = comb[:, :, 0].reshape(kc.shape).cpu().numpy()
        hv = comb[:, :, 1].reshape(vc.shape).cpu().numpy()
    else:
        hk, hv = gk.cpu().numpy(), gv.cpu().numpy()
    assert np.array_equal(hk, ok) and np.array_equal(hv, ov)
    assert np.array_equal(dks.cpu().numpy().view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(dvs.cpu().numpy().view(np.uint32), ovs.view(np.uint32))
    assert np.array_equal(r(dkst.cpu()), okst) and np.array_equal(r(dvst.cpu()), ovst)


@pytest.mark.parametrize("edge", [None, "q_range", "v_outlier"])
@pytest.mark.parametrize("kind", ["i8", "fp8"])
@pytest.mark.parametrize("balanced", [None, 0])
def test_int8_decode_steps_from_empty(P, balanced, kind, edge):
    """Sequences grow token by token from nothing through kv_append_quant (block
    boundaries crossed, scales growing), and decode attention reads the int8 cache after
    every step; the oracle does the same steps with its own quantising append.
    edge "q_range": the queries carry entries at +-1e5, +-1e-6 and +-1e30 (_extreme_q);
    "v_outlier": the first token of every sequence has V = +-4e4 at dim 5, so each first
    block's V scale sits ~1e4 above the later blocks' (checked relative to its magnitude on
    dim 5, absolute elsewhere)."""
    gen = torch.Generator().manual_seed(21)
    B, hq, hkv, d, steps = 5, 16, 4, 128, 37
    start = [0, 3, 15, 16, 30]                      # the step at which each sequence begins
    nb = 64
    alloc = W.BlockAllocator(nb, 16, free_order=torch.randperm(nb, generator=gen).tolist())
    for b in range(B):
        alloc.allocate(b, 0)
    kc = torch.zeros((nb, hkv, d // 16, 16, 16), dtype=torch.int8)
    vc = torch.zeros((nb, hkv, d, 16), dtype=torch.int8)
    ks, vs = torch.zeros((nb, hkv)), torch.zeros((nb, hkv))
    kst = torch.zeros((B, hkv, 16, d), dtype=torch.bfloat16)
    vst = torch.zeros_like(kst)
    r = lambda x: x.view(torch.int16).numpy()
    ora = [kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), r(kst), r(vst)]
    dev = [kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), kst.cuda(), vst.cuda()]
    rows = torch.arange(B, dtype=torch.int32)
    say(f"[case] {kind} decode steps from empty balanced={balanced}")
    for step in range(steps + max(start)):
        live = [b for b in range(B) if start[b] <= step < start[b] + steps]
        slots = torch.full((B,), -1, dtype=torch.int64)
        for b in live:
            slots[b] = alloc.append_token(b)[0]
        kn = _rand_bf16(gen, (B, hkv, d), 1.0 + step % 5)
        vn = _rand_bf16(gen, (B, hkv, d))
        if edge == "v_outlier":
            for b in live:
                if step == start[b]:
                    vn[b, :, 5] = 4e4 * (1 - 2 * (b % 2))
        dims = P.make_dims(B, hq, hkv, d, 8, nb, "bf16", kind)
        P.kv_append_quant(dims, kn.cuda(), vn.cuda(), slots.cuda(), rows.cuda(), B, dev[4], dev[5],
                          dev[0], dev[1], dev[2], dev[3])
        ora = list(quant.append_quant(*ora, r(kn), r(vn), slots.numpy(), rows.numpy(),
                                      kind=kind))
        if step % 6 != 5:
            continue
        tables = torch.full((B, 8), -1, dtype=torch.int32)
        for b in range(B):
            t = alloc.block_tables[b]
            tables[b, :len(t)] = torch.tensor(t, dtype=torch.int32)
        lens = torch.tensor([alloc.token_counts[b] for b in range(B)], dtype=torch.int32)
        q = _rand_bf16(gen, (B, 1, hq, d))
        if edge == "q_range":
            q = _extreme_q((B, 1, hq, d), 100 + step)
        out = torch.full((B, 1, hq, d), float("nan"), device="cuda:0")
        sm = float(np.float32(1 / np.sqrt(d)))
        if balanced is None:
            P.paged_decode_attn(dims, q.cuda(), dev[0], dev[1], dev[2], dev[3], tables.cuda(),
                                lens.cuda(), sm, out)
        else:
            G = P.paged_attn_balanced_workgroups(dims, 1)
            ws = torch.empty(P.paged_attn_balanced_workspace_bytes(dims, 1, G), dtype=torch.uint8,
                             device="cuda:0")
            P.paged_attn_balanced(dims, 1, q.cuda(), dev[0], dev[1], dev[2], dev[3], tables.cuda(),
                                  lens.cuda(), sm, G, ws, out)
            P.paged_attn_balanced_merge(dims, 1, G, ws, out)
        torch.cuda.synchronize()
        assert np.array_equal(dev[0].cpu().numpy(), ora[0]) and np.array_equal(dev[1].cpu().numpy(), ora[1])
        assert np.array_equal(dev[2].cpu().numpy(), ora[2]) and np.array_equal(dev[3].cpu().numpy(), ora[3])
        ref, _ = attention.paged_attention(r(q), "bf16", ora[0], ora[1], kind, tables.numpy(),
                                           lens.numpy(), sm, 1, ora[2], ora[3])
        say(f"  step {step} lens {lens.tolist()}")
        _assert_close(out, ref, TOL[kind], rel_dims=(5,) if edge == "v_outlier" else None)


# ---- 8-bit caches: the whole bf16 range of q, outlier V scales -----------------------------
def _extreme_q(shape, seed):
    """bf16 queries whose rows are, by (sequence + position + head) % 4: every entry +-1e5
    (scores ~1e5: one-hot attention), every entry +-1e-6 (uniform attention), a random half
    of the entries +-1e5 and the rest +-1e-6, every entry +-1e30 (scores ~1e32, still
    finite in fp32); random signs."""
    gen = torch.Generator().manual_seed(seed)
    B, nq, Hq, d = shape
    sign = torch.where(torch.rand(shape, generator=gen) < 0.5, -1.0, 1.0)
    mix = torch.rand(shape, generator=gen) < 0.5
    pat = ((torch.arange(B)[:, None, None] + torch.arange(nq)[None, :, None] +
            torch.arange(Hq)[None, None, :]) % 4)[..., None].expand(shape)
    mag = torch.where(pat == 0, 1e5, torch.where(pat == 1, 1e-6, torch.where(
        pat == 2, torch.where(mix, 1e5, 1e-6), torch.full(shape, 1e30))))
    return (sign * mag).to(torch.bfloat16)


@pytest.mark.parametrize("nq", [1, 6])
@pytest.mark.parametrize("kind", ["i8", "fp8"])
def test_8bit_extreme_q(P, kind, nq):
    """q entries far outside fp16's range (and far below its normal range) on int8 and fp8
    caches, in every mode: q.K runs on bf16 operands, so no query value is narrowed."""
    from dataclasses import replace
    wl = _small("verify_int8", batch=6, length_range=(1, 700), num_q_pos=nq, kv_dtype=kind)
    wl = replace(wl, q=_extreme_q(tuple(wl.q.shape), 31 + nq))
    kc, vc = oracle_caches(wl, appended=False)
    ref = oracle_attention(wl, kc, vc)
    _check_attention(P, wl, ref=ref)
    _check_attention(P, wl, balanced=0, ref=ref)
    _check_attention(P, wl, balanced=5, interleave=True, ref=ref)
    if nq == 1:
        _check_attention(P, wl, split=(64, 40), ref=ref)
    else:
        _check_multi_query(P, wl)


@pytest.mark.parametrize("case", ["big_first", "small_first"])
@pytest.mark.parametrize("kind", ["i8", "fp8"])
def test_8bit_v_scale_outliers(P, kind, case):
    """Every sequence's first block has a V scale ~1e4 above the later blocks' (one V
    element of +-4e4 at dim 5, the block's other values rounding to near zero) or 1e4 below
    them; queries x3 spread the scores so that much of the softmax mass sits in small
    weights.  The later blocks' weights must keep their precision whichever block a wave
    starts on."""
    from dataclasses import replace
    kw = dict(v_outlier=4e4) if case == "big_first" else dict(v_first_block_factor=1e-4)
    rel = (5,) if case == "big_first" else None
    for nq in (1, 6):
        wl = _small("verify_int8", batch=6, length_range=(17, 900), num_q_pos=nq,
                    kv_dtype=kind, **kw)
        wl = replace(wl, q=(wl.q.float() * 3).to(torch.bfloat16))
        kc, vc = oracle_caches(wl, appended=False)
        ref = oracle_attention(wl, kc, vc)
        _check_attention(P, wl, ref=ref, rel_dims=rel)
        _check_attention(P, wl, balanced=0, ref=ref, rel_dims=rel)
        _check_attention(P, wl, balanced=5, interleave=True, ref=ref, rel_dims=rel)
        if nq == 6:
            _check_multi_query(P, wl, rel_dims=rel)


# ---- multi-query rows: chunked prefill and speculative trees --------------------------------
def _check_multi_query(P, wl, interleave=False, pairs=None, rel_dims=None):
    c = wl.cfg
    say(f"[case] multi-query {c.name} B={c.batch} nq={c.num_q_pos} Hq={c.num_q_heads} "
        f"Hkv={c.num_kv_heads} d={c.head_dim} kv={c.kv_dtype} tree={wl.tree_mask is not None} "
        f"window={c.sliding_window} interleave={interleave} seed={wl.meta['seed']}")
    dv = Dev(wl, interleave)
    out, out_lse = gpu_multi_query(P, wl, dv)
    torch.cuda.synchronize()
    kc, vc = oracle_caches(wl, appended=False)
    ref, ref_lse = oracle_attention(wl, kc, vc, pairs=pairs, tree_mask=wl.tree_mask)
    _assert_close(out, ref, TOL[c.kv_dtype], pairs, c.group_size, rel_dims)
    g = out_lse.cpu().numpy()
    sel = np.isfinite(ref_lse)
    if pairs is not None:
        m = np.zeros(ref_lse.shape, bool)
        for b, kv in pairs:
            m[b, ..., kv * c.group_size:(kv + 1) * c.group_size] = True
        sel &= m
    else:
        assert np.all(g[ref_lse == -np.inf] == -np.inf)
    assert np.all(np.abs(g[sel] - ref_lse[sel]) <= 1e-3 * np.maximum(1, np.abs(ref_lse[sel])))


MQ_CASES = [
    ("prefill_chunk", dict(batch=3, num_q_pos=40, length_range=(40, 300), num_q_heads=8,
                           num_kv_heads=2)),
    ("prefill_chunk", dict(batch=2, num_q_pos=70, length_range=(1, 200), num_q_heads=4,
                           num_kv_heads=4, head_dim=64)),                    # L < nq rows
    ("prefill_chunk", dict(batch=3, num_q_pos=33, length_range=(33, 400), kv_dtype="i8")),
    ("prefill_chunk", dict(batch=3, num_q_pos=33, length_range=(33, 400), kv_dtype="fp8")),
    ("prefill_chunk", dict(batch=2, num_q_pos=24, length_range=(30, 300), q_dtype="f32",
                           kv_dtype="f32", num_q_heads=8, num_kv_heads=1)),
    ("prefill_chunk", dict(batch=3, num_q_pos=40, length_range=(40, 500), sliding_window=50)),
    ("tree_verify", dict(batch=4, num_q_pos=20, length_range=(20, 300))),
    ("tree_verify", dict(batch=3, num_q_pos=128, length_range=(1, 400), head_dim=64,
                         num_q_heads=4, num_kv_heads=2)),
    ("tree_verify", dict(batch=3, num_q_pos=64, length_range=(64, 300), kv_dtype="fp8")),
    ("tree_verify", dict(batch=3, num_q_pos=37, length_range=(30, 300), kv_dtype="i8",
                         num_q_heads=32, num_kv_heads=1)),
]


@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("name,kw", MQ_CASES)
def test_multi_query_small(P, name, kw, interleave):
    _check_multi_query(P, _small(name, **kw), interleave)


def test_multi_query_causal_mask_matches_causal_rows(P):
    """A lower-triangular candidate mask gives the same result as the causal rows."""
    wl = _small("prefill_chunk", batch=3, num_q_pos=48, length_range=(48, 300))
    say("[case] multi-query causal mask")
    dv = Dev(wl)
    nq = wl.cfg.num_q_pos
    causal = torch.tril(torch.ones((nq, nq), dtype=torch.bool)).expand(wl.cfg.batch, nq, nq)
    a, la = gpu_multi_query(P, wl, dv)
    b, lb = gpu_multi_query(P, wl, dv, tree=causal.contiguous())
    torch.cuda.synchronize()
    # (the two launches split a row tile's blocks over different numbers of waves, so only
    # the order of the fp32 sums differs)
    assert torch.allclose(a, b, rtol=0, atol=2e-5) and torch.allclose(la, lb, rtol=0, atol=2e-5)


def test_full_prefill_chunk(P):
    """The benchmark's chunked-prefill workload at full size, every output element."""
    _check_multi_query(P, W.generate("prefill_chunk"), interleave=True)


@pytest.mark.parametrize("half", [0, 1])
def test_full_tree_verify(P, half):
    """The benchmark's tree-verify workload at full size; every output element of one half
    of the batch per test (the oracle takes about a minute for the whole batch)."""
    wl = W.generate("tree_verify")
    pairs = [(b, g) for b in range(16 * half, 16 * half + 16) for g in range(8)]
    _check_multi_query(P, wl, interleave=True, pairs=pairs)


# ---- sliding window ------------------------------------------------------------------
def _poison_before_window(wl):
    """NaN every block wholly before the window of its sequence's first row (such blocks
    belong to that sequence only in these workloads): a kernel that reads one shows it."""
    from dataclasses import replace
    c = wl.cfg
    kc, vc = wl.k_cache.clone(), wl.v_cache.clone()
    ks = None if wl.k_scale is None else wl.k_scale.clone()
    vs = None if wl.v_scale is None else wl.v_scale.clone()
    n = 0
    for b, L in enumerate(wl.seq_lens.tolist()):
        lo = max(0, L - c.num_q_pos + 1 - c.sliding_window)
        for j in range(lo // 16):
            blk = int(wl.block_tables[b, j])
            if ks is not None:
                ks[blk] = float("nan")
                vs[blk] = float("nan")
            else:
                kc[blk] = float("nan")
                vc[blk] = float("nan")
            n += 1
    return replace(wl, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs), n


WINDOW_DECODE = [
    ("tiny_fp32", dict(batch=5, length_range=(1, 520), sliding_window=1)),
    ("tiny_fp32", dict(batch=5, length_range=(1, 520), sliding_window=100)),
    ("llama3_8b", dict(batch=7, length_range=(1, 600), sliding_window=16)),
    ("llama3_8b", dict(batch=7, length_range=(1, 600), sliding_window=37)),
    ("llama3_8b", dict(batch=6, length_range=(1, 900), sliding_window=256, num_q_heads=64,
                       num_kv_heads=1)),
    ("mistral_7b_window", dict(batch=5, length_range=(1, 1200), sliding_window=300)),
]


@pytest.mark.parametrize("mode", ["direct", "split", "balanced", "step"])
@pytest.mark.parametrize("name,kw", WINDOW_DECODE)
def test_sliding_window_decode(P, name, kw, mode):
    wl, npois = _poison_before_window(_small(name, **kw))
    say(f"[case] window {kw['sliding_window']} {mode} blocks poisoned {npois}")
    if mode == "direct":
        _check_attention(P, wl)
    elif mode == "split":
        _check_attention(P, wl, split=(64, 40))
        _check_attention(P, wl, split=(16, 200), interleave=True)
    elif mode == "balanced":
        _check_attention(P, wl, balanced=0)
        _check_attention(P, wl, balanced=5, interleave=True)
    else:
        _check_decode_step(P, wl, 0)
        _check_decode_step(P, wl, 3, interleave=True)


@pytest.mark.parametrize("mode", ["direct", "balanced"])
@pytest.mark.parametrize("name,kw", [
    ("verify_int8", dict(batch=5, length_range=(1, 500), sliding_window=20)),
    ("verify_int8", dict(batch=5, length_range=(1, 500), sliding_window=3)),
    ("verify_int8", dict(batch=4, length_range=(1, 400), sliding_window=64, kv_dtype="bf16")),
])
def test_sliding_window_verify(P, name, kw, mode):
    wl, npois = _poison_before_window(_small(name, **kw))
    say(f"[case] verify window {kw['sliding_window']} {mode} blocks poisoned {npois}")
    if mode == "direct":
        _check_attention(P, wl)
    else:
        _check_attention(P, wl, balanced=0)
        _check_attention(P, wl, balanced=7, interleave=True)


def test_sliding_window_full_mistral_7b(P):
    """The benchmark's sliding-window workload at full size (64 sequences of U[2048, 16384]
    tokens, window 4096) through the decode step, every output element."""
    _check_decode_step(P, W.generate("mistral_7b_window"), 0, interleave=True)


# ---- decode step: the append folded into the balanced attention launch ----------------
def _check_decode_step(P, wl, G=0, interleave=False, zero_lens=(), pairs=None, ref=None):
    c = wl.cfg
    say(f"[case] decode step {c.name} B={c.batch} Hq={c.num_q_heads} Hkv={c.num_kv_heads} "
        f"d={c.head_dim} kv={c.kv_dtype} G={G} interleave={interleave} zero={zero_lens} "
        f"seed={wl.meta['seed']}")
    lens = wl.seq_lens.clone()
    slots = wl.slot_mapping.numpy().copy()
    tables = wl.block_tables.numpy()
    for b, L in enumerate(lens.tolist()):      # the slot the kernel derives from the table
        assert slots[b] == paging.slot_of(tables[b], L - 1)
    for b in zero_lens:
        lens[b] = 0
        slots[b] = -1
    dv = Dev(wl, interleave)
    out, out_lse = gpu_decode_step(P, wl, dv, G, seq_lens=lens.cuda())
    torch.cuda.synchronize()
    kc, vc = paging.append(raw(wl.k_cache), raw(wl.v_cache), raw(wl.k_new), raw(wl.v_new), slots)
    gk, gv = dv.caches_host()
    assert np.array_equal(raw(gk).view(np.uint8), kc.view(np.uint8)), "K cache after the step"
    assert np.array_equal(raw(gv).view(np.uint8), vc.view(np.uint8)), "V cache after the step"
    if ref is None:
        ref, ref_lse = oracle_attention(wl, kc, vc, seq_lens=lens.numpy(), pairs=pairs)
    else:
        assert not zero_lens
        ref, ref_lse = ref
    err = max_err(out, ref, pairs, c.group_size)
    say(f"  max abs err {err:.3e} (tol {TOL[c.kv_dtype]:.0e})")
    assert err <= TOL[c.kv_dtype]
    g = out_lse.cpu().numpy().reshape(ref_lse.shape)
    sel = np.isfinite(ref_lse)
    if pairs is not None:
        m = np.zeros(ref_lse.shape, bool)
        for b, kv in pairs:
            m[b, ..., kv * c.group_size:(kv + 1) * c.group_size] = True
        sel &= m
    assert np.all(np.abs(g[sel] - ref_lse[sel]) <= 1e-3 * np.maximum(1, np.abs(ref_lse[sel])))
    for b in zero_lens:
        assert (out[b] == 0).all() and (out_lse[b] == -np.inf).all()


@pytest.mark.parametrize("G", [0, 5])
@pytest.mark.parametrize("name,kw", [
    ("llama3_8b", dict(batch=6, length_range=(1, 700))),
    ("llama3_8b", dict(batch=5, length_range=(1, 300), head_dim=64, num_q_heads=16, num_kv_heads=2)),
    ("llama3_8b", dict(batch=3, length_range=(40, 400), num_q_heads=32, num_kv_heads=1)),   # 32 rows
    ("llama3_8b", dict(batch=2, length_range=(100, 300), num_q_heads=64, num_kv_heads=1)),  # 2 row tiles
    ("llama2_70b_prefix", dict(batch=4, length_range=(17, 520))),
    ("tiny_fp32", dict(batch=5, length_range=(1, 400), head_dim=128)),
    ("tiny_fp32", dict(batch=4, length_range=(1, 200), num_q_heads=12, num_kv_heads=4)),
])
def test_decode_step_small(P, name, kw, G):
    wl = _small(name, **kw)
    _check_decode_step(P, wl, G)
    _check_decode_step(P, wl, G, interleave=True)


def test_decode_step_lengths_at_block_edges(P):
    # new token at offsets 0, 15 and 1 of a block; a sequence of one token; sequences of
    # length 0 append nothing and read nothing
    wl = _small("llama3_8b", batch=7, lengths=(1, 16, 17, 32, 33, 5, 200))
    _check_decode_step(P, wl, 0)
    _check_decode_step(P, wl, 3, zero_lens=(1, 5))


@pytest.mark.parametrize("B", [65, 300, 2048])
def test_large_batches(P, B):
    """Batches past the direct kernel's longest-first ranking (64 sequences) and past one
    chunk of the balanced kernel's prefix scan (256 sequences), up to its limit of 2048:
    direct, balanced and the decode step against the oracle on every output; contexts of
    1-60 tokens, so that some segments lie inside one wave's slice and others are cut
    over several."""
    wl = _small("llama3_8b", batch=B, length_range=(1, 60), num_q_heads=8, num_kv_heads=2,
                head_dim=64, spare=3)
    kc, vc = oracle_caches(wl)
    ref = oracle_attention(wl, kc, vc)
    _check_attention(P, wl, ref=ref)
    _check_attention(P, wl, balanced=0, interleave=True, ref=ref)
    _check_decode_step(P, wl, 0, interleave=True, ref=ref)


@pytest.mark.parametrize("name,kw", [
    ("llama3_8b_fp8", dict(batch=300, length_range=(1, 60), num_q_heads=8, num_kv_heads=2,
                           head_dim=64)),
    ("verify_int8", dict(batch=300, length_range=(6, 90))),   # 24 rows: two row tiles
])
def test_large_batches_8bit(P, name, kw):
    """The 8-bit caches (per-block scales staged with the table entries) and two row tiles
    per wave past one chunk of the prefix scan: direct and balanced against the oracle."""
    wl = _small(name, spare=3, **kw)
    kc, vc = oracle_caches(wl)
    ref = oracle_attention(wl, kc, vc)
    _check_attention(P, wl, ref=ref)
    _check_attention(P, wl, balanced=0, interleave=True, ref=ref)


@pytest.mark.parametrize("interleave", [False, True])
def test_decode_steps_back_to_back(P, interleave):
    """Six decode steps queued on one stream with no host synchronisation between them, as
    a serving loop (and the benchmark) issues them: every step appends a fresh token to
    each sequence and attends over it, all steps share one workspace, and each keeps its
    own output.  Step s + 1 reads the token step s wrote, and its attention kernel reuses
    the partial rows step s's merge reads, so stream order is what keeps them apart.  The
    oracle runs the same steps one after another with its own scatter."""
    S = 6
    wl = _small("llama3_8b", batch=10, length_range=(S + 1, 600))
    c = wl.cfg
    gen = torch.Generator().manual_seed(33)
    final = wl.seq_lens.numpy()
    tables = wl.block_tables.numpy()
    dv = Dev(wl, interleave)
    d = dims_of(P, wl, dv)
    G = P.paged_attn_balanced_workgroups(d, 1)
    ws = torch.full((P.paged_attn_balanced_workspace_bytes(d, 1, G),), 0xFF, dtype=torch.uint8,
                    device="cuda:0")
    sm = float(np.float32(wl.sm_scale))
    say(f"[case] {S} decode steps back to back B={c.batch} G={G} interleave={interleave}")
    steps = []
    for s in range(S):
        lens = (final - (S - 1) + s).astype(np.int32)
        q = _rand_bf16(gen, (c.batch, 1, c.num_q_heads, c.head_dim))
        kn = _rand_bf16(gen, (c.batch, c.num_kv_heads, c.head_dim), 1.0 + s % 3)
        vn = _rand_bf16(gen, (c.batch, c.num_kv_heads, c.head_dim))
        steps.append((lens, q, kn, vn, torch.from_numpy(lens).cuda(), q.cuda(), kn.cuda(),
                      vn.cuda()))
    outs = [torch.full((c.batch, 1, c.num_q_heads, c.head_dim), float("nan"), device="cuda:0")
            for _ in range(S)]
    torch.cuda.synchronize()
    for s, (_, _, _, _, dl, dq, dk, dvn) in enumerate(steps):
        P.paged_decode_step(d, dq, dk, dvn, dv.k_cache, dv.v_cache, dv.block_tables, dl, sm, G,
                            ws, outs[s])
        P.paged_attn_balanced_merge(d, 1, G, ws, outs[s])
    torch.cuda.synchronize()
    kc, vc = raw(wl.k_cache), raw(wl.v_cache)
    for s, (lens, q, kn, vn, *_) in enumerate(steps):
        slots = np.array([paging.slot_of(tables[b], int(lens[b]) - 1) for b in range(c.batch)])
        kc, vc = paging.append(kc, vc, raw(kn), raw(vn), slots)
        ref, _ = attention.paged_attention(raw(q), c.q_dtype, kc, vc, c.kv_dtype, tables, lens,
                                           sm, 1)
        say(f"  step {s}")
        _assert_close(outs[s], ref, TOL[c.kv_dtype])
    gk, gv = dv.caches_host()
    assert np.array_equal(raw(gk).view(np.uint8), kc.view(np.uint8)), "K cache after the steps"
    assert np.array_equal(raw(gv).view(np.uint8), vc.view(np.uint8)), "V cache after the steps"


def test_decode_step_int8_rejected(P):
    wl = _small("verify_int8", batch=2, length_range=(1, 50), num_q_pos=1)
    d = dims_of(P, wl)
    dv = Dev(wl)
    ws = torch.empty(P.paged_attn_balanced_workspace_bytes(d, 1, 4), dtype=torch.uint8,
                     device="cuda:0")
    out = torch.empty((2, 1, wl.cfg.num_q_heads, wl.cfg.head_dim), device="cuda:0")
    with pytest.raises(P.PagedAttnError) as e:
        P.paged_decode_step(d, dv.q, dv.q, dv.q, dv.k_cache, dv.v_cache, dv.block_tables,
                            dv.seq_lens, 0.1, 4, ws, out)
    assert e.value.status == -3


# ---- invariances, bit for bit --------------------------------------------------------
def test_block_relabel_and_batch_order_bit_identical(P):
    wl = _small("llama3_8b", batch=6, length_range=(1, 500), append=False)
    say("[case] relabel / shuffle invariance")
    out1, _, _ = gpu_attention(P, wl, Dev(wl))
    perm = torch.randperm(wl.k_cache.shape[0], generator=torch.Generator().manual_seed(5))
    out2, _, _ = gpu_attention(P, W.relabel_blocks(wl, perm), Dev(W.relabel_blocks(wl, perm)))
    bperm = torch.tensor([3, 0, 5, 1, 4, 2])
    wl3 = W.permute_batch(wl, bperm)
    out3, _, _ = gpu_attention(P, wl3, Dev(wl3))
    out4, _, _ = gpu_attention(P, wl, Dev(wl))
    torch.cuda.synchronize()
    assert torch.equal(_bits(out1), _bits(out2))
    assert torch.equal(_bits(out1[bperm]), _bits(out3))
    assert torch.equal(_bits(out1), _bits(out4))
    # the balanced mode deals logical positions, so a relabelled pool gives the same bits,
    # and so does a repeat (the merge order is fixed)
    wlr = W.relabel_blocks(wl, perm)
    b1, _, l1 = gpu_attention(P, wl, Dev(wl), balanced=0)
    b2, _, l2 = gpu_attention(P, wlr, Dev(wlr), balanced=0)
    b3, _, l3 = gpu_attention(P, wl, Dev(wl), balanced=0)
    torch.cuda.synchronize()
    assert torch.equal(_bits(b1), _bits(b2)) and torch.equal(_bits(b1), _bits(b3))
    assert torch.equal(_bits(l1), _bits(l2)) and torch.equal(_bits(l1), _bits(l3))


def test_multi_query_repeat_bit_identical(P):
    for name, kw in (("prefill_chunk", dict(batch=2, num_q_pos=40, length_range=(40, 400))),
                     ("tree_verify", dict(batch=3, num_q_pos=20, length_range=(20, 300)))):
        wl = _small(name, **kw)
        say(f"[case] multi-query repeat {name}")
        dv = Dev(wl)
        a, la = gpu_multi_query(P, wl, dv)
        b, lb = gpu_multi_query(P, wl, dv)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b)) and torch.equal(_bits(la), _bits(lb))


def test_split_count_invariance(P):
    wl = _small("llama3_8b", batch=3, length_range=(2000, 3000), append=False)
    say("[case] split count invariance")
    dv = Dev(wl)
    outs = [gpu_attention(P, wl, dv, split=s)[0] for s in [(256, 16), (512, 8), (2048, 2)]]
    outs.append(gpu_attention(P, wl, dv)[0])
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 1e-4


# ---- full-size configurations ---------------------------------------------------------
def test_full_llama3_8b_decode_step(P):
    wl = W.generate("llama3_8b")
    _check_decode_step(P, wl, 0)
    _check_decode_step(P, wl, 0, interleave=True)


def test_full_llama3_8b(P):
    wl = W.generate("llama3_8b")
    _check_attention(P, wl)
    _check_attention(P, wl, split=(512, 8))
    _check_attention(P, wl, balanced=0)
    _check_attention(P, wl, balanced=0, interleave=True)


def test_full_llama3_8b_fp8(P):
    wl = W.generate("llama3_8b_fp8")
    _check_attention(P, wl, balanced=0, interleave=True)
    _check_attention(P, wl, split=(512, 8))


@pytest.mark.parametrize("name,kw", [
    ("llama3_8b_fp8", dict(batch=6, length_range=(1, 700))),
    ("verify_int8", dict(batch=5, length_range=(6, 600), kv_dtype="fp8")),
    ("llama3_8b_fp8", dict(batch=6, length_range=(1, 700), sliding_window=40)),
])
def test_fp8_all_modes(P, name, kw):
    wl = _small(name, **kw)
    _check_attention(P, wl, interleave=True)
    _check_attention(P, wl, balanced=0)
    _check_attention(P, wl, balanced=5, interleave=True)
    if wl.cfg.num_q_pos == 1:
        _check_attention(P, wl, split=(64, 40))


def test_full_llama2_70b_shared_prefix(P):
    wl = W.generate("llama2_70b_prefix")
    _check_decode_step(P, wl, 0)
    _check_decode_step(P, wl, 0, interleave=True)      # the benchmark's launch
    _check_attention(P, wl)
    _check_attention(P, wl, balanced=0)
    wl2 = W.generate("llama2_70b_prefix", shuffle_batch=True)
    _check_attention(P, wl2)
    _check_attention(P, wl2, balanced=0, interleave=True)


def test_full_long_128k(P):
    """128K-token contexts at full size, every output element, in every mode that serves
    them; the oracle runs once (about 10 s) and is compared with each."""
    wl = W.generate("long_128k")
    kc, vc = oracle_caches(wl, appended=True)
    say("[case] long_128k oracle over all 32 (sequence, KV head) pairs")
    ref = oracle_attention(wl, kc, vc)
    del kc, vc
    _check_attention(P, wl, split=(2048, 64), ref=ref)
    _check_attention(P, wl, split=(4096, 8), ref=ref)   # the last partition absorbs the rest
    _check_attention(P, wl, balanced=0, ref=ref)
    _check_decode_step(P, wl, 0, interleave=True, ref=ref)   # the benchmark's launch


def test_full_verify_int8(P):
    wl = W.generate("verify_int8")
    _check_attention(P, wl)
    _check_attention(P, wl, balanced=0)
    _check_attention(P, wl, balanced=0, interleave=True)     # the benchmark's launch


def test_full_kv_append_quant_llama3_8b_int8(P):
    """The benchmark's quantising append: 64 tokens, one per sequence at the end of each
    Llama-3-8B-shaped sequence, into an int8 pool, whole pool and staging compared."""
    wl = W.generate(W.scaled("llama3_8b", kv_dtype="i8", append=False), spare_blocks=64)
    c = wl.cfg
    alloc = wl.meta["allocator"]
    slots = torch.tensor([alloc.append_token(b)[0] for b in range(c.batch)], dtype=torch.int64)
    gen = torch.Generator().manual_seed(7)
    h, d = c.num_kv_heads, c.head_dim
    kn = _rand_bf16(gen, (c.batch, h, d))
    vn = _rand_bf16(gen, (c.batch, h, d))
    kst = _rand_bf16(gen, (c.batch, h, 16, d))
    vst = _rand_bf16(gen, (c.batch, h, 16, d))
    rows = torch.arange(c.batch, dtype=torch.int32)
    say("[case] append_quant full llama3_8b int8")
    dims = P.make_dims(c.batch, c.num_q_heads, h, d, wl.block_tables.shape[1], wl.k_cache.shape[0],
                       "bf16", "i8")
    dk, dv_, dks, dvs = wl.k_cache.cuda(), wl.v_cache.cuda(), wl.k_scale.cuda(), wl.v_scale.cuda()
    dkst, dvst = kst.cuda(), vst.cuda()
    P.kv_append_quant(dims, kn.cuda(), vn.cuda(), slots.cuda(), rows.cuda(), c.batch, dkst, dvst,
                      dk, dv_, dks, dvs)
    torch.cuda.synchronize()
    r = lambda x: x.view(torch.int16).numpy()
    ok, ov, oks, ovs, okst, ovst = quant.append_quant(
        wl.k_cache.numpy(), wl.v_cache.numpy(), wl.k_scale.numpy(), wl.v_scale.numpy(), r(kst),
        r(vst), r(kn), r(vn), slots.numpy(), rows.numpy())
    assert np.array_equal(dk.cpu().numpy(), ok) and np.array_equal(dv_.cpu().numpy(), ov)
    # scales bit for bit (the untouched, poisoned entries keep their NaN patterns)
    assert np.array_equal(dks.cpu().numpy().view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(dvs.cpu().numpy().view(np.uint32), ovs.view(np.uint32))
    assert np.array_equal(r(dkst.cpu()), okst) and np.array_equal(r(dvst.cpu()), ovst)


# ---- HIP graph capture: the calls allocate nothing, set no memory and never sync --------
def test_decode_step_and_split_in_a_graph(P):
    """The decode step + merge and the split + lse_merge pair captured in one HIP graph
    (torch.cuda.graph, the library launching on the capturing stream) and replayed several
    times with eager work and synchronisations between replays: every replay must give
    exactly the eager results (the kernels are deterministic) and the same cache."""
    wl = _small("llama3_8b", batch=6, length_range=(1, 700))
    c = wl.cfg
    say(f"[case] graph replay {c.name} B={c.batch} seed={wl.meta['seed']}")
    dv = Dev(wl, interleave=True)
    d = dims_of(P, wl, dv)
    sm = float(np.float32(wl.sm_scale))
    G = P.paged_attn_balanced_workgroups(d, 1)
    ws = torch.empty((P.paged_attn_balanced_workspace_bytes(d, 1, G),), dtype=torch.uint8,
                     device="cuda:0")
    pt, maxp = 128, 8
    po = torch.empty((c.batch, c.num_q_heads, maxp, c.head_dim), device="cuda:0")
    pl = torch.empty((c.batch, c.num_q_heads, maxp), device="cuda:0")
    out1 = torch.empty((c.batch, 1, c.num_q_heads, c.head_dim), device="cuda:0")
    lse1 = torch.empty((c.batch, 1, c.num_q_heads), device="cuda:0")
    out2 = torch.empty((c.batch, c.num_q_heads, c.head_dim), device="cuda:0")

    def work():
        P.paged_decode_step(d, dv.q, dv.k_new, dv.v_new, dv.k_cache, dv.v_cache,
                            dv.block_tables, dv.seq_lens, sm, G, ws, out1, lse1)
        P.paged_attn_balanced_merge(d, 1, G, ws, out1, lse1)
        P.paged_decode_attn_split(d, dv.q, dv.k_cache, dv.v_cache, None, None, dv.block_tables,
                                  dv.seq_lens, sm, pt, maxp, po, pl)
        P.lse_merge(d, po, pl, dv.seq_lens, pt, maxp, out2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()                                   # eager, on the stream to be captured
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref1, ref_lse, ref2 = out1.clone(), lse1.clone(), out2.clone()
    cache = dv.comb.clone()
    kc, vc = oracle_caches(wl)
    ref, _ = oracle_attention(wl, kc, vc)
    assert max_err(out1, ref) <= TOL[c.kv_dtype] and max_err(out2[:, None], ref) <= TOL[c.kv_dtype]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for t in (out1, lse1, out2):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        assert torch.equal(out1, ref1) and torch.equal(out2, ref2)
        assert torch.equal(lse1, ref_lse)
        assert torch.equal(dv.comb.view(torch.int16), cache.view(torch.int16))  # (NaN poison)
        with torch.cuda.stream(side):            # eager work between the replays
            work()
        torch.cuda.synchronize()


# ---- seeded random sweep over shapes, element types and modes ---------------------------
def _sweep_case(i):
    """Case i of the sweep: a seeded draw of the shape, element type, lengths, query
    positions, window, layout and launch mode."""
    rng = np.random.default_rng(7000 + i)
    kv = str(rng.choice(["f32", "bf16", "bf16", "i8", "fp8"]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    nq = int(rng.choice([1, 1, 1, 2, 5, 6, 9]))
    batch = int(rng.integers(1, 9))
    lmax = int(rng.choice([40, 300, 700]))
    eight = kv in ("i8", "fp8")
    append = nq == 1 and not eight and bool(rng.integers(0, 2))
    window = int(rng.choice([0, 0, 0, 17, 64, 200]))
    tree = nq > 1 and window == 0 and bool(rng.integers(0, 2))
    kw = dict(batch=batch, num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=d,
              q_dtype="f32" if kv == "f32" else "bf16", kv_dtype=kv, num_q_pos=nq,
              length_range=(1 if append else 0, lmax), append=append,
              sliding_window=window, tree=tree, seed=7000 + i)
    modes = ["direct", "balanced"]
    if nq == 1:
        modes.append("split")
        if append:
            modes.append("step")
    if nq > 1:
        modes.append("multi")
    mode = modes[int(rng.integers(0, len(modes)))]
    if tree:
        mode = "multi"
    if append and rng.integers(0, 2):
        mode = "step"
    return kw, mode, bool(rng.integers(0, 2)), int(rng.choice([0, 1, 3, 7, 40]))


@pytest.mark.parametrize("i", range(512))
def test_random_sweep(P, i):
    kw, mode, interleave, G = _sweep_case(i)
    wl = _small("llama3_8b", **kw)
    say(f"[sweep {i}] mode={mode} G={G} {kw}")
    if mode == "step":
        _check_decode_step(P, wl, G, interleave=interleave)
    elif mode == "multi":
        _check_multi_query(P, wl, interleave=interleave)
    elif mode == "split":
        pt = int(np.random.default_rng(i).choice([16, 64, 256]))
        _check_attention(P, wl, split=(pt, 1 + int(wl.seq_lens.max()) // pt),
                         interleave=interleave)
    elif mode == "balanced":
        _check_attention(P, wl, balanced=G, interleave=interleave)
    else:
        _check_attention(P, wl, interleave=interleave)
