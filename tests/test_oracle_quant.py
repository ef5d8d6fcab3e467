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


# ---- fp8 e4m3 --------------------------------------------------------------------------
def test_fp8_decode_matches_library_and_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    ours = storage.fp8_e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9
    assert ours[0x08] == 2.0 ** -6 and ours[0x07] == 7 * 2.0 ** -9 and ours[0xC0] == -2.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and not np.isnan(ours[0x79])
    assert ours[0x80] == 0.0 and np.signbit(ours[0x80])


def test_fp8_encode_rounding_and_saturation():
    # exact values, ties to even, subnormal ties, saturation, signs
    y = np.array([1.0, 448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 460.0,
                  1e6, -500.0, -1.0, 0.0, -0.0, 2.0 ** -6, 15 * 2.0 ** -10], np.float32)
    want = [0x38, 0x7E, 0x01, 0x00, 0x02, 0x38, 0x3A, 0x7E, 0x7E, 0xFE, 0xB8, 0x00, 0x80,
            0x08, 0x08]
    assert quant.fp8_e4m3_encode(y).tolist() == want
    # against the library's round-to-nearest-even conversion over the finite range,
    # including every midpoint between neighbouring e4m3 values
    rng = np.random.default_rng(4)
    mags = np.exp2(rng.uniform(-12, np.log2(448), 4000)).astype(np.float32)
    vals = storage.fp8_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    y = np.concatenate([mags, -mags, mids, -mids, vals.astype(np.float32)])
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quant.fp8_e4m3_encode(y), lib)


def test_fp8_quantise_invariants():
    rng = np.random.default_rng(5)
    for _ in range(10):
        x = (rng.standard_normal((7, 32)) * rng.uniform(1e-3, 50)).astype(np.float32)
        q, s = quant.quantise_fp8(x)
        assert s == np.float32(np.abs(x).max() / np.float32(448))
        assert np.abs(storage.fp8_e4m3_to_f64(q)).max() == 448.0
        deq = storage.decode(q, "fp8", s)
        # half a step of the e4m3 grid: 2^-4 relative (normal range), 2^-10 * scale below it
        assert np.all(np.abs(deq - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * 1.0001)


def test_fp8_token_by_token_equals_the_generators_whole_block_encoding():
    hkv, d, nb = 2, 32, 3
    rng = np.random.default_rng(6)
    toks = (rng.standard_normal((16, hkv, d)) * 2).astype(np.float32)
    toks[9, 0, 3] = -30.0
    kb = _bf16_bits(toks)
    state = _empty_pool(nb, hkv, d, rows=1)
    blk = 1
    for t in range(16):
        state = quant.append_quant(*state, kb[t:t + 1], kb[t:t + 1], np.array([blk * 16 + t]),
                                   np.array([0]), kind="fp8")
        kc, vc, ks, vs, _, _ = state
        x = storage.bf16_bits_to_f64(kb).astype(np.float32)
        pool = torch.zeros((nb, hkv, 16, d))
        pool[blk] = torch.from_numpy(x).permute(1, 0, 2)
        live = torch.zeros((nb, 16), dtype=torch.bool)
        live[blk, :t + 1] = True
        ref_q, ref_s = W._quantise_fp8(pool, live)
        ref_k = W.encode_k(ref_q)
        assert np.array_equal(kc[blk][:, :, :t + 1].view(np.uint8),
                              ref_k[blk].numpy()[:, :, :t + 1]), t
        assert ks[blk].tolist() == ref_s[blk].tolist(), t
        assert np.array_equal(vc[blk][:, :, :t + 1].view(np.uint8),
                              W.encode_v(ref_q)[blk].numpy()[:, :, :t + 1]), t


def test_fp8_attention_reads_decoded_values_times_scales():
    """paged attention over an fp8 cache equals attention over an fp32 cache holding
    value(code) * scale (the decode definition, checked against the library above)."""
    from oracle import attention
    wl = W.generate(W.scaled("llama3_8b_fp8", batch=3, length_range=(1, 90), num_q_heads=4,
                             num_kv_heads=2, head_dim=32), spare_blocks=2)
    r = lambda x: x.view(torch.int16).numpy()
    kc, vc = wl.k_cache.numpy(), wl.v_cache.numpy()
    ks, vs = wl.k_scale.numpy(), wl.v_scale.numpy()
    out, lse = attention.paged_attention(r(wl.q), "bf16", kc, vc, "fp8", wl.block_tables.numpy(),
                                         wl.seq_lens.numpy(), 0.17, 1, ks, vs)
    # (the products rounded to fp32: relative 2^-24, far inside the 1e-6 below)
    kd = (storage.fp8_e4m3_to_f64(kc) * ks[:, :, None, None, None]).astype(np.float32)
    vd = (storage.fp8_e4m3_to_f64(vc) * vs[:, :, None, None]).astype(np.float32)
    out2, lse2 = attention.paged_attention(r(wl.q), "bf16", kd, vd, "f32", wl.block_tables.numpy(),
                                           wl.seq_lens.numpy(), 0.17, 1)
    assert np.allclose(out, out2, rtol=0, atol=1e-6) and np.allclose(lse, lse2, rtol=0, atol=1e-6)
