"""Shared helpers of the GPU parity tests: run a workload through the C ABI and through
the oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import workloads as W
from oracle import attention, paging

KIND = {"f32": "f32", "bf16": "bf16", "i8": "i8", "fp8": "fp8"}
TOL = {"f32": 1e-5, "bf16": 2e-3, "i8": 4e-3, "fp8": 4e-3}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def raw(x):
    """numpy view of a CPU tensor's stored elements (bf16 as int16 bit patterns)."""
    if x is None:
        return None
    x = x.cpu()
    return x.view(torch.int16).numpy() if x.dtype == torch.bfloat16 else x.numpy()


def dims_of(P, wl, dv=None):
    c = wl.cfg
    return P.make_dims(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim,
                       wl.block_tables.shape[1], wl.k_cache.shape[0], c.q_dtype, c.kv_dtype,
                       kv_tile_stride=0 if dv is None else dv.stride,
                       sliding_window=c.sliding_window)


class Dev:
    """Device copies of a workload's tensors.  With interleave=True the K and V tiles of
    each (block, KV head) sit side by side in one allocation [NB][Hkv][2][tile] (tile
    stride 2 * tile); k_cache is then that allocation and v_cache the address of its
    first V tile."""

    def __init__(self, wl, interleave=False):
        dev = torch.device("cuda:0")
        self.q = wl.q.to(dev)
        self.shape_k, self.shape_v = wl.k_cache.shape, wl.v_cache.shape
        self.stride = 0
        if interleave:
            nb, h = wl.k_cache.shape[:2]
            tile = wl.k_cache[0, 0].numel()
            self.comb = torch.empty((nb, h, 2, tile), dtype=wl.k_cache.dtype, device=dev)
            self.comb[:, :, 0] = wl.k_cache.reshape(nb, h, tile).to(dev)
            self.comb[:, :, 1] = wl.v_cache.reshape(nb, h, tile).to(dev)
            self.k_cache = self.comb
            self.v_cache = self.comb.data_ptr() + tile * self.comb.element_size()
            self.stride = 2 * tile
        else:
            self.k_cache = wl.k_cache.to(dev)
            self.v_cache = wl.v_cache.to(dev)
        self.k_scale = None if wl.k_scale is None else wl.k_scale.to(dev)
        self.v_scale = None if wl.v_scale is None else wl.v_scale.to(dev)
        self.block_tables = wl.block_tables.to(dev)
        self.seq_lens = wl.seq_lens.to(dev)
        self.slot_mapping = None if wl.slot_mapping is None else wl.slot_mapping.to(dev)
        self.k_new = None if wl.k_new is None else wl.k_new.to(dev)
        self.v_new = None if wl.v_new is None else wl.v_new.to(dev)

    def caches_host(self):
        """(K, V) on the host in the dense layout."""
        if self.stride:
            nb, h = self.shape_k[:2]
            return (self.comb[:, :, 0].reshape(self.shape_k).cpu(),
                    self.comb[:, :, 1].reshape(self.shape_v).cpu())
        return self.k_cache.cpu(), self.v_cache.cpu()


def gpu_append(P, wl, dv):
    d = dims_of(P, wl, dv)
    P.kv_append(d, dv.k_new, dv.v_new, dv.slot_mapping, wl.cfg.batch, dv.k_cache, dv.v_cache)


def gpu_attention(P, wl, dv, seq_lens=None, split=None, balanced=None):
    """Run decode / verify (or split + merge when split=(partition_tokens, max_partitions),
    or the balanced mode with `balanced` workgroups, 0 = the library's resident count).
    Returns (out, partials or None, out_lse or None)."""
    c = wl.cfg
    d = dims_of(P, wl, dv)
    lens = dv.seq_lens if seq_lens is None else seq_lens
    sm = float(np.float32(wl.sm_scale))
    out = torch.full((c.batch, c.num_q_pos, c.num_q_heads, c.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda:0")
    if balanced is not None:
        G = balanced or P.paged_attn_balanced_workgroups(d, c.num_q_pos)
        nbytes = P.paged_attn_balanced_workspace_bytes(d, c.num_q_pos, G)
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")   # no init needed
        out_lse = torch.full((c.batch, c.num_q_pos, c.num_q_heads), float("nan"), device="cuda:0")
        P.paged_attn_balanced(d, c.num_q_pos, dv.q, dv.k_cache, dv.v_cache, dv.k_scale,
                              dv.v_scale, dv.block_tables, lens, sm, G, ws, out, out_lse)
        P.paged_attn_balanced_merge(d, c.num_q_pos, G, ws, out, out_lse)
        return out, None, out_lse
    if split is None:
        if c.num_q_pos == 1:
            P.paged_decode_attn(d, dv.q, dv.k_cache, dv.v_cache, dv.k_scale, dv.v_scale,
                                dv.block_tables, lens, sm, out)
        else:
            P.paged_verify_attn(d, c.num_q_pos, dv.q, dv.k_cache, dv.v_cache, dv.k_scale,
                                dv.v_scale, dv.block_tables, lens, sm, out)
        return out, None, None
    pt, maxp = split
    part_out = torch.full((c.batch, c.num_q_heads, maxp, c.head_dim), float("nan"),
                          device="cuda:0")
    part_lse = torch.full((c.batch, c.num_q_heads, maxp), float("nan"), device="cuda:0")
    out_lse = torch.full((c.batch, c.num_q_heads), float("nan"), device="cuda:0")
    P.paged_decode_attn_split(d, dv.q, dv.k_cache, dv.v_cache, dv.k_scale, dv.v_scale,
                              dv.block_tables, lens, sm, pt, maxp, part_out, part_lse)
    P.lse_merge(d, part_out, part_lse, lens, pt, maxp, out, out_lse)
    return out, (part_out, part_lse), out_lse


def gpu_decode_step(P, wl, dv, G=0, seq_lens=None):
    """paged_decode_step + paged_attn_balanced_merge: append and decode attention in one
    attention launch.  Returns (out, out_lse)."""
    c = wl.cfg
    d = dims_of(P, wl, dv)
    lens = dv.seq_lens if seq_lens is None else seq_lens
    G = G or P.paged_attn_balanced_workgroups(d, 1)
    nbytes = P.paged_attn_balanced_workspace_bytes(d, 1, G)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = torch.full((c.batch, 1, c.num_q_heads, c.head_dim), float("nan"), device="cuda:0")
    out_lse = torch.full((c.batch, 1, c.num_q_heads), float("nan"), device="cuda:0")
    P.paged_decode_step(d, dv.q, dv.k_new, dv.v_new, dv.k_cache, dv.v_cache, dv.block_tables,
                        lens, float(np.float32(wl.sm_scale)), G, ws, out, out_lse)
    P.paged_attn_balanced_merge(d, 1, G, ws, out, out_lse)
    return out, out_lse


def gpu_multi_query(P, wl, dv, tree=None):
    """paged_multi_query_attn; tree=None: the workload's own mask if it has one.
    Returns (out, out_lse)."""
    import workloads as W
    c = wl.cfg
    d = dims_of(P, wl, dv)
    mask = wl.tree_mask if tree is None else tree
    words = None if mask is None else W.tree_mask_words(mask).to("cuda:0")
    out = torch.full((c.batch, c.num_q_pos, c.num_q_heads, c.head_dim), float("nan"),
                     device="cuda:0")
    out_lse = torch.full((c.batch, c.num_q_pos, c.num_q_heads), float("nan"), device="cuda:0")
    P.paged_multi_query_attn(d, c.num_q_pos, dv.q, dv.k_cache, dv.v_cache, dv.k_scale,
                             dv.v_scale, dv.block_tables, dv.seq_lens,
                             float(np.float32(wl.sm_scale)), out, out_lse, words)
    return out, out_lse


def oracle_caches(wl, appended=True):
    """Host caches as the oracle sees them (after the step's append, by the oracle's own
    scatter)."""
    kc, vc = raw(wl.k_cache), raw(wl.v_cache)
    if appended and wl.slot_mapping is not None:
        kc, vc = paging.append(kc, vc, raw(wl.k_new), raw(wl.v_new), wl.slot_mapping.numpy())
    return kc, vc


def oracle_attention(wl, kc, vc, seq_lens=None, pairs=None, tree_mask=None):
    c = wl.cfg
    lens = wl.seq_lens.numpy() if seq_lens is None else np.asarray(seq_lens)
    return attention.paged_attention(raw(wl.q), c.q_dtype, kc, vc, c.kv_dtype,
                                     wl.block_tables.numpy(), lens, float(np.float32(wl.sm_scale)),
                                     c.num_q_pos, raw(wl.k_scale), raw(wl.v_scale), pairs=pairs,
                                     window=c.sliding_window,
                                     tree_mask=None if tree_mask is None else tree_mask.numpy())


def max_err(gpu_out, ref, pairs=None, group=None):
    g = gpu_out.detach().cpu().numpy().astype(np.float64)
    if pairs is not None:
        sel = np.zeros(ref.shape, dtype=bool)
        for b, kv in pairs:
            sel[b, :, kv * group:(kv + 1) * group] = True
        diff = np.abs(g[sel] - ref[sel])
        assert np.isfinite(g[sel]).all(), "non-finite GPU output"
    else:
        assert np.isfinite(g).all(), "non-finite GPU output"
        diff = np.abs(g - ref)
    return float(diff.max()) if diff.size else 0.0
