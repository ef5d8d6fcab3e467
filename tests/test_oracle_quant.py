"""Pins of the quantising-append oracle: closed forms of the int8 rule, rounding ties,
the generator's independent whole-block encoder, error bounds and what must stay
untouched."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import quant, storage


def _bf16_bits(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()


def test_quantise_closed_forms():
    # max |x| = 127 * 0.5 -> scale 0.5 exactly, and multiples of 0.5 encode exactly
    x = np.array([[63.5, -12.0, 0.5], [0.0, -63.5, 3.0]], np.float32)
    q, s = quant.quantise_i8(x)
    assert s == np.float32(0.5)
    assert np.array_equal(q, (x / 0.5).astype(np.int8))
    # ties go to even: with scale 1, 2.5 -> 2, 3.5 -> 4, -0.5 -> 0, -1.5 -> -2
    x = np.array([[127.0, 2.5, 3.5, -0.5, -1.5]], np.float32)
    q, s = quant.quantise_i8(x)
    assert s == 1.0 and q.tolist() == [[127, 2, 4, 0, -2]]
    # all zero -> scale 0, codes 0
    q, s = quant.quantise_i8(np.zeros((3, 4), np.float32))
    assert s == 0 and not q.any()
    # the largest magnitude always maps to +-127
    rng = np.random.default_rng(0)
    for _ in range(20):
        x = (rng.standard_normal((5, 16)) * rng.uniform(0.01, 100)).astype(np.float32)
        q, s = quant.quantise_i8(x)
        assert np.abs(q).max() == 127
        assert np.all(np.abs(q.astype(np.float64) * s - x) <= s / 2 * (1 + 1e-6))


def _empty_pool(nb, hkv, d, rows):
    kc = np.full((nb, hkv, d // 16, 16, 16), 99, np.int8)
    vc = np.full((nb, hkv, d, 16), -99, np.int8)
    ks = np.full((nb, hkv), np.nan, np.float32)
    vs = np.full((nb, hkv), np.nan, np.float32)
    kst = np.zeros((rows, hkv, 16, d), np.int16)
    vst = np.zeros((rows, hkv, 16, d), np.int16)
    return kc, vc, ks, vs, kst, vst


def test_token_by_token_equals_the_generators_whole_block_encoding():
    """16 appends into one block, one call each, leave exactly what the workload
    generator's own encoder (torch, whole block at once) makes of the same tokens; after
    every append the open block equals that encoder on its live tokens."""
    hkv, d, nb = 2, 32, 5
    rng = np.random.default_rng(1)
    toks = (rng.standard_normal((16, hkv, d)) * 3).astype(np.float32)
    toks[5, 1, 7] = 40.0                               # the scale grows mid-block
    kb, vb = _bf16_bits(toks), _bf16_bits(-2 * toks)
    state = _empty_pool(nb, hkv, d, rows=3)
    blk, row = 3, 2
    for t in range(16):
        state = quant.append_quant(*state, kb[t:t + 1], vb[t:t + 1], np.array([blk * 16 + t]),
                                   np.array([row]))
        kc, vc, ks, vs, _, _ = state
        x = storage.bf16_bits_to_f64(kb).astype(np.float32)          # [16, hkv, d]
        pool = torch.zeros((nb, hkv, 16, d))
        pool[blk] = torch.from_numpy(x).permute(1, 0, 2)
        live = torch.zeros((nb, 16), dtype=torch.bool)
        live[blk, :t + 1] = True
        ref_q, ref_s = W._quantise_int8(pool, live)
        ref_k = W.encode_k(ref_q)
        assert np.array_equal(kc[blk][:, :, :t + 1], ref_k[blk].numpy()[:, :, :t + 1]), t
        assert ks[blk].tolist() == ref_s[blk].tolist(), t
        vx = storage.bf16_bits_to_f64(vb).astype(np.float32)
        pool[blk] = torch.from_numpy(vx).permute(1, 0, 2)
        ref_vq, ref_vs = W._quantise_int8(pool, live)
        ref_v = W.encode_v(ref_vq)
        assert np.array_equal(vc[blk][:, :, :t + 1], ref_v[blk].numpy()[:, :, :t + 1]), t
        assert vs[blk].tolist() == ref_vs[blk].tolist(), t
        # slots after the last token and every other block are untouched
        assert (kc[blk][:, :, t + 1:] == 99).all() and (vc[blk][:, :, t + 1:] == -99).all()
        others = [b for b in range(nb) if b != blk]
        assert (kc[others] == 99).all() and np.isnan(ks[others]).all()


def test_negative_and_out_of_pool_slots_write_nothing():
    hkv, d, nb = 1, 16, 2
    state = _empty_pool(nb, hkv, d, rows=2)
    kb = _bf16_bits(np.ones((2, hkv, d)))
    out = quant.append_quant(*state, kb, kb, np.array([-1, nb * 16]), np.array([0, 1]))
    for a, b in zip(out, state):
        assert np.array_equal(a, b, equal_nan=True)
    kb = _bf16_bits(np.ones((2, hkv, d)))
    out = quant.append_quant(*state, kb, kb, np.array([3, 17]), np.array([-1, 2]))   # bad rows
    for a, b in zip(out, state):
        assert np.array_equal(a, b, equal_nan=True)


def test_staging_rows_are_per_sequence():
    """Two sequences with open blocks in different staging rows: each block is encoded from
    its own row only."""
    hkv, d, nb = 1, 16, 4
    state = _empty_pool(nb, hkv, d, rows=2)
    a = _bf16_bits(np.full((1, hkv, d), 1.0))
    b = _bf16_bits(np.full((1, hkv, d), 100.0))
    state = quant.append_quant(*state, a, a, np.array([1 * 16 + 0]), np.array([0]))
    state = quant.append_quant(*state, b, b, np.array([2 * 16 + 0]), np.array([1]))
    state = quant.append_quant(*state, a, a, np.array([1 * 16 + 1]), np.array([0]))
    kc, vc, ks, vs, kst, _ = state
    assert ks[1, 0] == np.float32(1.0) / np.float32(127) and ks[2, 0] == np.float32(100) / np.float32(127)
    assert (kc[1, 0, :, :2] == 127).all() and (kc[2, 0, :, 0] == 127).all()
    assert (kst[1, 0, 0] == b[0, 0]).all() and (kst[0, 0, 1] == a[0, 0]).all()
