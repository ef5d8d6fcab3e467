"""Pins of the fp64 attention oracle: brute force, a library routine, closed forms,
GQA/MHA equivalence, block-relabel invariance, verify rows and the LSE merge."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention, paging, storage


def _brute(q, K, V, sigma):
    """Direct softmax without the max shift, in Python floats (tiny inputs only)."""
    L = len(K)
    s = [sigma * sum(q[k] * K[t][k] for k in range(len(q))) for t in range(L)]
    e = [math.exp(x) for x in s]
    z = sum(e)
    out = [sum(e[t] * V[t][k] for t in range(L)) / z for k in range(len(V[0]))]
    return out, math.log(z)


def test_attend_matches_brute_force():
    rng = np.random.default_rng(0)
    for L in (1, 2, 7, 33):
        q = rng.standard_normal((3, 5))
        K = rng.standard_normal((L, 5))
        V = rng.standard_normal((L, 5))
        out, lse = attention.attend(q, K, V, 0.4, [L, L, L])
        for r in range(3):
            o, l = _brute(q[r].tolist(), K.tolist(), V.tolist(), 0.4)
            assert np.allclose(out[r], o, rtol=0, atol=1e-13)
            assert abs(lse[r] - l) < 1e-12


def test_attend_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((6, 64))
    K = rng.standard_normal((300, 64))
    V = rng.standard_normal((300, 64))
    sigma = 1 / 8
    out, _ = attention.attend(q, K, V, sigma, [300] * 6)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(K)[None, None],
        torch.from_numpy(V)[None, None], scale=sigma)[0, 0].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_lse_matches_library_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 16))
    K = rng.standard_normal((50, 16)) * 6
    V = rng.standard_normal((50, 16))
    _, lse = attention.attend(q, K, V, 0.25, [50, 20])
    assert abs(lse[0] - logsumexp(0.25 * K @ q[0])) < 1e-12
    assert abs(lse[1] - logsumexp(0.25 * K[:20] @ q[1])) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(3)
    V = rng.standard_normal((40, 8))
    k = rng.standard_normal(8)
    K = np.tile(k, (40, 1))                       # identical keys -> mean of V
    out, lse = attention.attend(rng.standard_normal((2, 8)), K, V, 0.3, [40, 40])
    assert np.allclose(out, V.mean(0), atol=1e-14)
    out1, _ = attention.attend(rng.standard_normal((1, 8)), K[:1], V[:1], 0.3, [1])
    assert np.array_equal(out1[0], V[0])          # one token -> its value exactly
    Kd = rng.standard_normal((40, 8)) * 0.01      # one key dominates by far
    q = np.ones(8)
    Kd[17] = 100.0
    outd, _ = attention.attend(q[None], Kd, V, 1.0, [40])
    assert np.allclose(outd[0], V[17], atol=1e-12)
    oute, lsee = attention.attend(q[None], Kd, V, 1.0, [0])   # nothing visible
    assert (oute == 0).all() and lsee[0] == -np.inf


def _paged(wl, **kw):
    kind = wl.cfg.kv_dtype

    def raw(x):
        if x is None:
            return None
        return x.view(torch.int16).numpy() if x.dtype == torch.bfloat16 else x.numpy()
    return attention.paged_attention(
        raw(wl.q), wl.cfg.q_dtype, raw(wl.k_cache), raw(wl.v_cache), kind,
        wl.block_tables.numpy(), wl.seq_lens.numpy(), float(np.float32(wl.sm_scale)),
        wl.cfg.num_q_pos, raw(wl.k_scale), raw(wl.v_scale), **kw)


def _small(name, **kw):
    base = dict(batch=3, length_range=(1, 90), lengths=None, pool_blocks=None,
                shared_groups=0, shared_group_size=0, shared_prefix_tokens=0,
                lengths_are_cached=False, append=False)
    base.update(kw)
    return W.generate(W.scaled(name, **base), spare_blocks=5)


def test_gqa_equals_mha_with_replicated_kv():
    wl = _small("tiny_fp32", head_dim=16)
    G = wl.cfg.group_size
    out, lse = _paged(wl)
    # replicate each KV head G times in place -> an MHA cache with Hq KV heads
    rep = W.Workload(
        W.scaled(wl.cfg, num_kv_heads=wl.cfg.num_q_heads), wl.q,
        wl.k_cache.repeat_interleave(G, dim=1), wl.v_cache.repeat_interleave(G, dim=1),
        None, None, wl.block_tables, wl.seq_lens, None, None, None, wl.occupancy)
    out2, lse2 = _paged(rep)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_block_relabel_invariance():
    wl = _small("llama3_8b", head_dim=64, num_q_heads=8, num_kv_heads=2)
    perm = torch.randperm(wl.k_cache.shape[0], generator=torch.Generator().manual_seed(9))
    out, lse = _paged(wl)
    out2, lse2 = _paged(W.relabel_blocks(wl, perm))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_fast_and_slow_depage_give_same_attention():
    wl = _small("verify_int8", head_dim=64, num_q_heads=8, num_kv_heads=2)
    a = _paged(wl, fast=True)
    b = _paged(wl, fast=False)
    assert np.array_equal(a[0], b[0])


def test_verify_row_equals_decode_over_prefix():
    wl = _small("verify_int8", head_dim=32, num_q_heads=4, num_kv_heads=2,
                length_range=(20, 70))
    nq = wl.cfg.num_q_pos
    out, lse = _paged(wl)
    qd = storage.decode(wl.q.view(torch.int16).numpy(), "bf16")
    for b in range(wl.cfg.batch):
        L = int(wl.seq_lens[b])
        for i in range(nq):
            for h in range(wl.cfg.num_q_heads):
                g = h // wl.cfg.group_size
                K, V = paging.depage(wl.k_cache.numpy(), wl.v_cache.numpy(), "i8",
                                     wl.block_tables[b].numpy(), L - nq + 1 + i, g,
                                     wl.k_scale.numpy(), wl.v_scale.numpy())
                o, l = attention.attend(qd[b, i, h][None], K, V, float(np.float32(wl.sm_scale)),
                                        [len(K)])
                assert np.array_equal(o[0], out[b, i, h]) and l[0] == lse[b, i, h]


def test_verify_with_one_position_is_decode():
    wl = _small("verify_int8", head_dim=32, num_q_heads=4, num_kv_heads=1, num_q_pos=1)
    assert wl.cfg.num_q_pos == 1
    out, _ = _paged(wl)
    assert np.isfinite(out).all()
    lim = attention.row_limits(50, 1)
    assert lim == [50]
    assert attention.row_limits(50, 6) == [45, 46, 47, 48, 49, 50]


@pytest.mark.parametrize("pt,maxp", [(16, 100), (32, 3), (48, 100), (64, 1)])
def test_partition_merge_equals_unsplit(pt, maxp):
    wl = _small("llama3_8b", head_dim=32, num_q_heads=8, num_kv_heads=2, length_range=(1, 200))
    out, lse = _paged(wl)
    raw = lambda x: x.view(torch.int16).numpy()
    op, lp = attention.paged_attention_partitions(
        raw(wl.q), "bf16", raw(wl.k_cache), raw(wl.v_cache), "bf16", wl.block_tables.numpy(),
        wl.seq_lens.numpy(), float(np.float32(wl.sm_scale)), pt, maxp)
    n = np.array([attention.partitions_used(int(L), pt, maxp) for L in wl.seq_lens.tolist()])
    mo, ml = attention.lse_merge(op, lp, n[:, None, None])
    assert np.allclose(mo, out, rtol=0, atol=1e-13)
    assert np.allclose(ml, lse, rtol=0, atol=1e-12)


def test_merge_edge_cases():
    o = np.array([[[1.0, 2.0], [3.0, 4.0], [9.0, 9.0]]])
    lse = np.array([[-np.inf, 0.5, np.nan]])
    out, l = attention.lse_merge(o, lse, np.array([2]))
    assert np.array_equal(out[0], [3.0, 4.0]) and l[0] == 0.5
    out, l = attention.lse_merge(o, np.array([[-np.inf, -np.inf, 0.0]]), np.array([2]))
    assert (out == 0).all() and l[0] == -np.inf
    # two equal partitions average, lse adds log 2
    out, l = attention.lse_merge(o[:, :2], np.array([[1.0, 1.0]]))
    assert np.allclose(out[0], [2.0, 3.0]) and abs(l[0] - (1 + math.log(2))) < 1e-15


def test_partition_ranges():
    assert attention.partitions_used(0, 16, 4) == 0
    assert attention.partitions_used(17, 16, 4) == 2
    assert attention.partitions_used(1000, 16, 4) == 4
    assert attention.partition_range(1000, 3, 16, 4) == (48, 1000)
    assert attention.partition_range(40, 1, 16, 4) == (16, 32)
    assert attention.partition_range(40, 2, 16, 4) == (32, 40)


def test_verify_causal_closed_form():
    # Uniform attention (all keys equal) over values V[t] = t: query position i of
    # nq sits at absolute position p = L - nq + i and sees tokens 0..p, so its
    # output is the mean of 0..p = p / 2 in every dimension.
    L, nq, d, G = 37, 6, 4, 2
    tables = np.array([[2, 0, 1]], dtype=np.int32)
    kc = np.ones((3, 1, d // 4, 16, 4), np.float32)
    vc = np.zeros((3, 1, d, 16), np.float32)
    for t in range(48):
        vc[tables[0, t // 16], 0, :, t % 16] = t
    q = np.ones((1, nq, G, d), np.float32)
    out, lse = attention.paged_attention(q, "f32", kc, vc, "f32", tables, np.array([L]), 0.5, nq)
    for i in range(nq):
        p = L - nq + i
        assert np.allclose(out[0, i], p / 2, atol=1e-12)
        # lse of p+1 equal scores s = 0.5 * d
        assert abs(lse[0, i, 0] - (0.5 * d + math.log(p + 1))) < 1e-12


def test_sliding_window_closed_form():
    # Uniform attention over V[t] = t with a window of W tokens: the row at absolute
    # position p sees tokens max(0, p - W + 1) .. p, so its output is their mean
    # (lo + p) / 2 and its lse is s + log(p - lo + 1).
    L, nq, d, G = 37, 6, 4, 2
    tables = np.array([[2, 0, 1]], dtype=np.int32)
    kc = np.ones((3, 1, d // 4, 16, 4), np.float32)
    vc = np.zeros((3, 1, d, 16), np.float32)
    for t in range(48):
        vc[tables[0, t // 16], 0, :, t % 16] = t
    q = np.ones((1, nq, G, d), np.float32)
    for Wn in (1, 2, 5, 16, 17, 33, 34, 100):
        out, lse = attention.paged_attention(q, "f32", kc, vc, "f32", tables, np.array([L]),
                                             0.5, nq, window=Wn)
        for i in range(nq):
            p = L - nq + i
            lo = max(0, p - Wn + 1)
            assert np.allclose(out[0, i], (lo + p) / 2, atol=1e-12), (Wn, i)
            assert abs(lse[0, i, 0] - (0.5 * d + math.log(p - lo + 1))) < 1e-12


def test_sliding_window_of_one_is_own_value():
    wl = _small("tiny_fp32", head_dim=16, length_range=(1, 60))
    out, lse = _paged(wl, window=1)
    Kt = W.k_token_rows(wl.k_cache).numpy()              # [NB, Hkv, 16, d], by the generator
    q = wl.q.float().numpy().astype(np.float64)
    sig = float(np.float32(wl.sm_scale))
    G = wl.cfg.group_size
    for b in range(wl.cfg.batch):
        L = int(wl.seq_lens[b])
        blk = int(wl.block_tables[b, (L - 1) // 16])
        for h in range(wl.cfg.num_q_heads):
            v = wl.v_cache[blk, h // G, :, (L - 1) % 16].numpy()
            assert np.array_equal(out[b, 0, h], v.astype(np.float64))
            k = Kt[blk, h // G, (L - 1) % 16].astype(np.float64)
            assert abs(lse[b, 0, h] - sig * (q[b, 0, h] @ k)) < 1e-12


@pytest.mark.parametrize("Wn", [3, 16, 40])
def test_sliding_window_equals_full_attention_over_the_recent_tokens(Wn):
    """Brute force through another cache: each row's windowed result equals full attention
    over a fresh one-sequence pool that holds only that row's last Wn tokens, built from
    the generator's token-major values and re-encoded by it."""
    wl = _small("verify_int8", kv_dtype="bf16", head_dim=32, num_q_heads=4, num_kv_heads=2,
                length_range=(1, 80))
    c = wl.cfg
    nq = c.num_q_pos
    out, lse = _paged(wl, window=Wn)
    Kt = W.k_token_rows(wl.k_cache)                      # [NB, Hkv, 16, d] bf16
    Vt = wl.v_cache.transpose(2, 3)                      # [NB, Hkv, 16, d]
    raw = lambda x: x.view(torch.int16).numpy()
    for b in range(c.batch):
        L = int(wl.seq_lens[b])
        for i in range(nq):
            p = L - nq + i
            if p < 0:
                assert np.all(lse[b, i] == -np.inf)
                continue
            toks = list(range(max(0, p - Wn + 1), p + 1))
            nb = -(-len(toks) // 16)
            kt = torch.zeros((nb, c.num_kv_heads, 16, c.head_dim), dtype=torch.bfloat16)
            vt = torch.zeros_like(kt)
            for n, t in enumerate(toks):
                blk = int(wl.block_tables[b, t // 16])
                kt[n // 16, :, n % 16] = Kt[blk, :, t % 16]
                vt[n // 16, :, n % 16] = Vt[blk, :, t % 16]
            kc, vc = W.encode_k(kt), W.encode_v(vt)
            o2, l2 = attention.paged_attention(
                raw(wl.q[b:b + 1, i:i + 1]), "bf16", raw(kc), raw(vc), "bf16",
                np.arange(nb, dtype=np.int32)[None], np.array([len(toks)]),
                float(np.float32(wl.sm_scale)), 1)
            assert np.allclose(out[b, i], o2[0, 0], rtol=0, atol=1e-13)
            assert np.allclose(lse[b, i], l2[0, 0], rtol=0, atol=1e-12)


def test_sliding_window_at_least_the_context_is_full_attention():
    wl = _small("verify_int8", head_dim=32, num_q_heads=4, num_kv_heads=2, length_range=(1, 70))
    out, lse = _paged(wl)
    for Wn in (70, 71, 1000):
        o2, l2 = _paged(wl, window=Wn)
        assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    assert attention.row_starts(50, 3, 0) == [0, 0, 0]
    assert attention.row_starts(50, 3, 10) == [38, 39, 40]
    assert attention.row_starts(5, 3, 10) == [0, 0, 0]


# ---- multi-query rows: speculative trees and chunked prefill ---------------------------
def test_causal_tree_mask_is_the_verify_result():
    wl = _small("verify_int8", head_dim=32, num_q_heads=4, num_kv_heads=2, length_range=(1, 70))
    nq = wl.cfg.num_q_pos
    causal = torch.tril(torch.ones((nq, nq), dtype=torch.bool)).expand(wl.cfg.batch, nq, nq)
    out, lse = _paged(wl)
    out2, lse2 = _paged(wl, tree_mask=causal.numpy())
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_tree_closed_form():
    # uniform attention over V[t] = t: candidate i's output is the mean position of the
    # context tokens and of its ancestors-or-self
    nq, d, G = 7, 4, 2
    parents = [-1, 0, 0, 1, 1, 2, 5]
    mask = W.tree_mask_from_parents(parents).numpy()[None]
    tables = np.array([[2, 0, 1]], dtype=np.int32)
    kc = np.ones((3, 1, d // 4, 16, 4), np.float32)
    vc = np.zeros((3, 1, d, 16), np.float32)
    for t in range(48):
        vc[tables[0, t // 16], 0, :, t % 16] = t
    q = np.ones((1, nq, G, d), np.float32)
    for L in (7, 20, 40):
        out, lse = attention.paged_attention(q, "f32", kc, vc, "f32", tables, np.array([L]), 0.5,
                                             nq, tree_mask=mask)
        base = L - nq
        for i in range(nq):
            anc, j = [], i
            while j >= 0:
                anc.append(base + j)
                j = parents[j]
            vis = list(range(base)) + anc
            assert np.allclose(out[0, i], np.mean(vis), atol=1e-12), (L, i)
            assert abs(lse[0, i, 1] - (0.5 * d + math.log(len(vis)))) < 1e-12


def test_tree_row_equals_decode_over_its_path():
    """Brute force through another cache: candidate i's result equals decode attention
    over a fresh one-sequence pool holding the context and then the path root .. i."""
    wl = W.generate(W.scaled("tree_verify", batch=3, length_range=(20, 70), num_q_pos=12,
                             head_dim=32, num_q_heads=4, num_kv_heads=2, lengths=None),
                    spare_blocks=2)
    c = wl.cfg
    nq = c.num_q_pos
    out, lse = _paged(wl, tree_mask=wl.tree_mask.numpy())
    Kt = W.k_token_rows(wl.k_cache)
    Vt = wl.v_cache.transpose(2, 3)
    raw = lambda x: x.view(torch.int16).numpy()
    for b in range(c.batch):
        L = int(wl.seq_lens[b])
        for i in range(nq):
            toks = list(range(L - nq)) + [L - nq + j for j in range(nq) if wl.tree_mask[b, i, j]]
            nb = -(-len(toks) // 16)
            kt = torch.zeros((nb, c.num_kv_heads, 16, c.head_dim), dtype=torch.bfloat16)
            vt = torch.zeros_like(kt)
            for n, t in enumerate(toks):
                blk = int(wl.block_tables[b, t // 16])
                kt[n // 16, :, n % 16] = Kt[blk, :, t % 16]
                vt[n // 16, :, n % 16] = Vt[blk, :, t % 16]
            o2, l2 = attention.paged_attention(
                raw(wl.q[b:b + 1, i:i + 1]), "bf16", raw(W.encode_k(kt)), raw(W.encode_v(vt)),
                "bf16", np.arange(nb, dtype=np.int32)[None], np.array([len(toks)]),
                float(np.float32(wl.sm_scale)), 1)
            assert np.allclose(out[b, i], o2[0, 0], rtol=0, atol=1e-13)
            assert np.allclose(lse[b, i], l2[0, 0], rtol=0, atol=1e-12)


def test_tree_rows_that_see_nothing():
    # no context and a candidate whose row is empty: out 0, lse -inf
    nq, d = 3, 4
    mask = np.array([[[1, 0, 0], [0, 0, 0], [1, 1, 1]]], dtype=bool)
    kc = np.ones((1, 1, 1, 16, 4), np.float32)
    vc = np.ones((1, 1, d, 16), np.float32)
    out, lse = attention.paged_attention(np.ones((1, nq, 1, d), np.float32), "f32", kc, vc, "f32",
                                         np.array([[0]], np.int32), np.array([3]), 1.0, nq,
                                         tree_mask=mask)
    assert (out[0, 1] == 0).all() and lse[0, 1, 0] == -np.inf
    assert np.allclose(out[0, 0], 1.0) and np.allclose(out[0, 2], 1.0)
    assert W.tree_mask_words(torch.from_numpy(mask)).tolist() == [[[1], [0], [7]]]
