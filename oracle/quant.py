"""Quantising append into an 8-bit paged cache, int8 or fp8 e4m3 (oracle; test
infrastructure only).

What is quantised, and how (Lecture 10 "Quantization 量化 / 基本概念": x_q =
round(x / scale) + zero_point, x = (x_q - zero_point) * scale, here symmetric with
zero_point = 0; in-depth guide §5.2: KV caches need per-head (or per-channel) scales
rather than one global scale): each (physical block, KV head) of K and of V carries one
fp32 scale

    scale = max |x| / 127        over the block's live tokens and every dim,
    x_q   = round-half-even(x / scale), clamped to [-127, 127]   (0 when scale == 0),

computed in fp32 (the values are bf16 inputs widened exactly to fp32; the division is
an fp32 division): the codes are integers decided by floating point, so the kernel makes
the same decisions in the same precision.

The pages say nothing about how tokens enter a block whose scale depends on all of its
tokens.  Reading taken: the open (partly filled) block of each sequence is kept beside
the cache in its input precision, in a staging row [Hkv][16][head_dim] (token-major
bf16).  Appending token t at offset o of its block writes t into staging offset o, then
re-encodes the block's live tokens 0..o from the staging row with the rule above and
writes their codes and the new scale into the cache.  So at every moment an int8 block
holds exactly the whole-block encoding of its live tokens (its scale is provisional
while the block is open and final once the 16th token is in), and the attention kernels
read it unchanged.

FP8 e4m3 variant (in-depth guide §5.2: an FP8 KV cache with per-head scaling factors
halves the cache at a small quality loss): the same per-(block, KV head) layout and
staging rule with

    scale = max |x| / 448       (448 = the largest finite e4m3 value),
    code  = e4m3(x / scale)     round to nearest, ties to even, saturating at +-448,

written here from the OCP e4m3 definition (see ``storage``).  A per-head calibrated
scale is the special case of every block of a head holding the same scale.
"""

import numpy as np

from . import storage

BLOCK_SIZE = 16
QMAX = 127
FP8_MAX = 448.0


def quantise_i8(x):
    """Encode the live tokens of one (block, head): x [n, d] fp32 -> (codes int8, scale fp32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(QMAX))
    if scale == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    q = np.rint(x / scale)                     # fp32 division, ties to even
    return np.clip(q, -QMAX, QMAX).astype(np.int8), scale


def fp8_e4m3_encode(y):
    """e4m3 bytes (uint8) of fp32 values y: round to nearest, ties to even, magnitudes at or
    above 448 saturate to 448; the sign bit is y's own (so -0.0 gives 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    out = np.zeros(y.shape, np.uint8)
    for ix in np.ndindex(*y.shape):
        v = float(y[ix])
        a = abs(v)
        if a >= FP8_MAX:
            code = 0x7E
        elif a < 2.0 ** -6:                     # subnormal grid m * 2^-9 (m = 8 is 2^-6)
            code = int(np.rint(a * 2.0 ** 9))
        else:
            e = int(np.floor(np.log2(a)))
            if 2.0 ** e > a:                    # guard log2 rounding
                e -= 1
            elif 2.0 ** (e + 1) <= a:
                e += 1
            r = int(np.rint(a * 2.0 ** (3 - e)))   # 8 .. 16, exact scaling, ties to even
            if r == 16:
                e, r = e + 1, 8
            code = min(((e + 7) << 3) | (r - 8), 0x7E)
        out[ix] = code | (0x80 if np.signbit(y[ix]) else 0)
    return out


def quantise_fp8(x):
    """Encode the live tokens of one (block, head) as e4m3: (codes uint8, scale fp32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(FP8_MAX))
    if scale == 0:
        return np.zeros(x.shape, np.uint8), np.float32(0)
    return fp8_e4m3_encode(x / scale), scale    # fp32 division


def append_quant(k_cache, v_cache, k_scale, v_scale, k_stage, v_stage, k_new, v_new,
                 slot_mapping, stage_rows, block_size=BLOCK_SIZE, kind="i8"):
    """Copies of (k_cache, v_cache, k_scale, v_scale, k_stage, v_stage) after appending
    token i of k_new / v_new ([T, Hkv, d] bf16 bit patterns) to slot slot_mapping[i],
    through staging row stage_rows[i].

    kind: "i8" or "fp8" (e4m3 codes stored as bytes).
    Caches: 8-bit in the project format (k [NB, Hkv, d/16, 16, 16], v [NB, Hkv, d, 16]);
    scales [NB, Hkv] fp32; staging [S, Hkv, 16, d] bf16 bit patterns.  A slot < 0 or
    outside the pool, or a staging row outside [0, S), writes nothing.  Tokens are taken
    in order; no two tokens of one call
    may fall into the same block (each one re-encodes the block from its staging row).
    """
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    ks, vs = np.array(k_scale, copy=True), np.array(v_scale, copy=True)
    kst, vst = np.array(k_stage, copy=True), np.array(v_stage, copy=True)
    nb, hkv = kc.shape[0], kc.shape[1]
    assert kst.shape[1:] == (hkv, block_size, kc.shape[2] * kc.shape[4])
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0 or s >= nb * block_size:
            continue
        blk, off = divmod(int(s), block_size)
        row = int(stage_rows[i])
        if row < 0 or row >= kst.shape[0]:
            continue
        for g in range(hkv):
            kst[row, g, off] = k_new[i, g]
            vst[row, g, off] = v_new[i, g]
            kx = storage.bf16_bits_to_f64(kst[row, g, :off + 1]).astype(np.float32)
            vx = storage.bf16_bits_to_f64(vst[row, g, :off + 1]).astype(np.float32)
            enc = quantise_i8 if kind == "i8" else quantise_fp8
            kq, ks[blk, g] = enc(kx)
            vq, vs[blk, g] = enc(vx)
            kq, vq = kq.view(kc.dtype), vq.view(vc.dtype)
            for t in range(off + 1):
                kc[blk, g, :, t, :] = kq[t].reshape(kc.shape[2], kc.shape[4])
                vc[blk, g, :, t] = vq[t]
    return kc, vc, ks, vs, kst, vst
