"""Pins of the oracle's storage decoding and paging against the pages and closed forms."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import paging, storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- storage decoding -------------------------------------------------------------
def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x3F81, 0x4049],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 2.0**-133, 1.0 + 2.0**-7, 3.140625]
    got = storage.bf16_bits_to_f64(bits)
    assert got.tolist() == want
    assert np.signbit(got[3])


def test_bf16_decode_matches_torch_widening():
    # a library routine: torch widens bf16 to fp64 exactly
    x = torch.randn(4096, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    got = storage.decode(x.view(torch.int16).numpy(), "bf16")
    assert np.array_equal(got, x.to(torch.float64).numpy())


def test_int8_decode_is_exact_product():
    q = np.array([-127, -1, 0, 1, 5, 127], dtype=np.int8)
    s = np.float32(0.0371)
    got = storage.decode(q, "i8", s)
    assert got.tolist() == [float(v) * float(s) for v in q.tolist()]
    with pytest.raises(ValueError):
        storage.decode(q, "i8")


# ---- block-table translation (Tutorial §7 worked example) ---------------------------
def test_worked_block_table():
    ex = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    A = ex["tables"]["A"]
    for logical, phys in ex["logical_to_physical_A"]:
        assert paging.token_location(A, logical * 16) == (phys, 0)
    for row in ex["token_checks_A"]:
        assert paging.token_location(A, row["token"]) == (row["block"], row["offset"])
        assert paging.slot_of(A, row["token"]) == row["slot"]
    B = ex["tables"]["B"]
    assert paging.token_location(B, 47) == (31, 15)


def _labelled_pool(NB, H, d, kind):
    """fp32 pool whose every element encodes its own (block, head, slot, dim) position,
    laid out as the header states: K [NB, H, d/4, 16, 4], V [NB, H, d, 16]."""
    kval = np.empty((NB, H, d // 4, 16, 4), np.float32)
    vval = np.empty((NB, H, d, 16), np.float32)
    for blk in range(NB):
        for g in range(H):
            for off in range(16):
                for k in range(d):
                    label = ((blk * 8 + g) * 16 + off) * 64.0 + k    # exact in fp32
                    kval[blk, g, k // 4, off, k % 4] = label
                    vval[blk, g, k, off] = -label
    return kval, vval


def test_depage_reads_documented_layout():
    # closed form: K[t, k] must be the element labelled (table[t//16], g, t%16, k)
    NB, H, d = 40, 3, 8
    kc, vc = _labelled_pool(NB, H, d, "f32")
    table = [17, 4, 29, 11]
    L = 55
    for g in range(H):
        K, V = paging.depage(kc, vc, "f32", table, L, g)
        for t in range(L):
            blk, off = table[t // 16], t % 16
            label = ((blk * 8 + g) * 16 + off) * 64.0
            assert K[t].tolist() == [label + k for k in range(d)]
            assert V[t].tolist() == [-(label + k) for k in range(d)]


@pytest.mark.parametrize("kind", ["f32", "bf16", "i8"])
def test_depage_fast_equals_depage(kind):
    rng = np.random.default_rng(3)
    NB, H, d = 64, 2, 16
    if kind == "f32":
        kc = rng.standard_normal((NB, H, d // 4, 16, 4)).astype(np.float32)
        vc = rng.standard_normal((NB, H, d, 16)).astype(np.float32)
        ks = vs = None
    elif kind == "bf16":
        kc = rng.integers(0, 2**16, (NB, H, d // 8, 16, 8)).astype(np.uint16)
        vc = rng.integers(0, 2**16, (NB, H, d, 16)).astype(np.uint16)
        kc[(kc & 0x7F80) == 0x7F80] = 0x3F80  # no inf/nan patterns
        vc[(vc & 0x7F80) == 0x7F80] = 0x3F80
        ks = vs = None
    else:
        kc = rng.integers(-127, 128, (NB, H, d // 16, 16, 16)).astype(np.int8)
        vc = rng.integers(-127, 128, (NB, H, d, 16)).astype(np.int8)
        ks = rng.random((NB, H)).astype(np.float32)
        vs = rng.random((NB, H)).astype(np.float32)
    table = rng.permutation(NB)[:10]
    for L in (0, 1, 16, 17, 150, 160):
        for g in range(H):
            a = paging.depage(kc, vc, kind, table, L, g, ks, vs)
            b = paging.depage_fast(kc, vc, kind, table, L, g, ks, vs)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_append_writes_slot_and_nothing_else():
    NB, H, d = 8, 2, 16
    kc, vc = _labelled_pool(NB, H, d, "f32")
    k_new = np.arange(3 * H * d, dtype=np.float32).reshape(3, H, d) + 0.5
    v_new = -k_new
    slots = np.array([5 * 16 + 3, -1, 0 * 16 + 15], dtype=np.int64)
    kc2, vc2 = paging.append(kc, vc, k_new, v_new, slots)
    for g in range(H):
        assert np.array_equal(paging.k_row(kc2, 5, g, 3), k_new[0, g])
        assert np.array_equal(paging.k_row(kc2, 0, g, 15), k_new[2, g])
    assert np.array_equal(vc2[5, :, :, 3], v_new[0]) and np.array_equal(vc2[0, :, :, 15], v_new[2])
    mask_k = np.ones(kc.shape, bool)
    mask_k[5, :, :, 3, :] = False
    mask_k[0, :, :, 15, :] = False
    mask_v = np.ones(vc.shape, bool)
    mask_v[5, :, :, 3] = False
    mask_v[0, :, :, 15] = False
    assert np.array_equal(kc2[mask_k], kc[mask_k]) and np.array_equal(vc2[mask_v], vc[mask_v])
    # the new token is what de-paging returns at its position
    table = [0, 5]
    K, V = paging.depage(kc2, vc2, "f32", table, 20, 1)
    assert np.array_equal(K[15], k_new[2, 1]) and np.array_equal(K[19], k_new[0, 1])
    assert np.array_equal(V[19], v_new[0, 1])


def test_gather_equals_depage():
    NB, H, d = 30, 2, 8
    kc, vc = _labelled_pool(NB, H, d, "f32")
    tables = np.array([[3, 7, 1, -1], [9, 2, 20, 21]], dtype=np.int32)
    lens = [40, 64]
    ko = np.full((2, H, 70, d), 7.0, np.float32)
    vo = np.full((2, H, 70, d), 7.0, np.float32)
    ko2, vo2 = paging.gather(kc, vc, tables, lens, ko, vo)
    for b in range(2):
        for g in range(H):
            K, V = paging.depage(kc, vc, "f32", tables[b], lens[b], g)
            assert np.array_equal(ko2[b, g, : lens[b]], K.astype(np.float32))
            assert np.array_equal(vo2[b, g, : lens[b]], V.astype(np.float32))
            assert (ko2[b, g, lens[b]:] == 7.0).all()


def test_copy_blocks_copies_whole_blocks_and_nothing_else():
    # closed form on the labelled pool: after copying 3 -> 10 and 7 -> 11, de-paging a
    # table that names block 10 (11) returns the labels of block 3 (7); skipped pairs
    # (out of the pool, src == dst) change nothing
    NB, H, d = 24, 3, 8
    kc, vc = _labelled_pool(NB, H, d, "f32")
    ks = np.arange(NB * H, dtype=np.float32).reshape(NB, H) + 0.25
    vs = -ks
    pairs = np.array([[3, 10], [7, 11], [-1, 5], [2, 99], [4, 4]], dtype=np.int32)
    kc2, vc2, ks2, vs2 = paging.copy_blocks(kc, vc, pairs, ks, vs)
    for dst, src in ((10, 3), (11, 7)):
        for g in range(H):
            K, V = paging.depage(kc2, vc2, "f32", [dst], 16, g)
            for t in range(16):
                label = ((src * 8 + g) * 16 + t) * 64.0
                assert K[t].tolist() == [label + k for k in range(d)]
                assert V[t].tolist() == [-(label + k) for k in range(d)]
        assert ks2[dst].tolist() == ks[src].tolist() and vs2[dst].tolist() == vs[src].tolist()
    keep = np.ones(NB, bool)
    keep[[10, 11]] = False
    assert np.array_equal(kc2[keep], kc[keep]) and np.array_equal(vc2[keep], vc[keep])
    assert np.array_equal(ks2[keep], ks[keep]) and np.array_equal(vs2[keep], vs[keep])


def test_copy_on_write_keeps_the_other_sharer_intact():
    # two sequences share a partly filled block; the writer gets a private copy first,
    # then appends into it: the other sharer still reads the old contents, the writer
    # reads the old tokens followed by its new one
    NB, H, d = 12, 2, 8
    kc, vc = _labelled_pool(NB, H, d, "f32")
    shared, private = 5, 9
    kc2, vc2, _, _ = paging.copy_blocks(kc, vc, [[shared, private]])
    k_new = np.full((1, H, d), 0.5, np.float32)
    kc3, vc3 = paging.append(kc2, vc2, k_new, -k_new, [private * 16 + 7])
    for g in range(H):
        Ka, _ = paging.depage(kc3, vc3, "f32", [shared], 8, g)    # the reader
        Kb, _ = paging.depage(kc3, vc3, "f32", [private], 8, g)   # the writer
        K0, _ = paging.depage(kc, vc, "f32", [shared], 8, g)
        assert np.array_equal(Ka, K0)
        assert np.array_equal(Kb[:7], K0[:7]) and (Kb[7] == 0.5).all()
