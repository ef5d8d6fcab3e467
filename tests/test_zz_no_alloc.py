"""The allocation-free decode step, paged_decode_step_noalloc, through the C ABI against the
decode step with a caller workspace (paged_decode_step + paged_attn_balanced_merge): the same
kernels at the same launch shape, so outputs, log-sum-exps and the written caches must agree
bit for bit, and both within the bf16 tolerance of the oracle.  Two calls in a row share the
static scratch, the second with a smaller batch than the first."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import paging
from _helpers import TOL, Dev, dims_of, gpu_decode_step, max_err, oracle_attention, raw, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import paged_gqa_decode_kv_amd as P
    assert torch.cuda.is_available()
    return P


def _bits(x):
    return x.detach().cpu().view(torch.int32)


def _noalloc_step(P, wl, dv, G):
    c = wl.cfg
    out = torch.full((c.batch, 1, c.num_q_heads, c.head_dim), float("nan"), device="cuda:0")
    out_lse = torch.full((c.batch, 1, c.num_q_heads), float("nan"), device="cuda:0")
    P.paged_decode_step_noalloc(dims_of(P, wl, dv), dv.q, dv.k_new, dv.v_new, dv.k_cache,
                                dv.v_cache, dv.block_tables, dv.seq_lens,
                                float(np.float32(wl.sm_scale)), G, out, out_lse)
    return out, out_lse


def test_noalloc_decode_step_matches_the_workspace_step(P):
    cases = [
        # the benchmark's Llama-3-8B step: 64 sequences, 512 segments, library-default launch
        (W.generate("llama3_8b"), True, 0),
        # then a smaller batch on the same scratch, at two launch shapes
        (W.generate(W.scaled("llama3_8b", batch=9, length_range=(1, 700)), spare_blocks=3),
         False, 0),
        (W.generate(W.scaled("llama3_8b", batch=9, length_range=(1, 700)), spare_blocks=3),
         True, 5),
        # 32 query heads on one KV head: two row tiles, whose pieces are combined per
        # workgroup in the attention kernel and merged four rows a wave
        (W.generate(W.scaled("llama3_8b", batch=5, length_range=(1, 900), num_q_heads=32,
                             num_kv_heads=1), spare_blocks=3), True, 64),
        (W.generate(W.scaled("llama3_8b", batch=5, length_range=(1, 900), num_q_heads=32,
                             num_kv_heads=1), spare_blocks=3), False, 3),
    ]
    for wl, interleave, G in cases:
        c = wl.cfg
        G = G or P.paged_attn_balanced_workgroups(dims_of(P, wl), 1)
        need = P.paged_attn_balanced_workspace_bytes(dims_of(P, wl), 1, G)
        say(f"[case] noalloc decode step B={c.batch} G={G} interleave={interleave} "
            f"workspace {need} of {P.PA_NOALLOC_SCRATCH_BYTES} bytes")
        dv_ref = Dev(wl, interleave)
        ref_out, ref_lse = gpu_decode_step(P, wl, dv_ref, G)
        dv = Dev(wl, interleave)
        out, out_lse = _noalloc_step(P, wl, dv, G)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_out)), "output differs from the workspace step"
        assert torch.equal(_bits(out_lse), _bits(ref_lse)), "lse differs from the workspace step"
        gk, gv = dv.caches_host()
        rk, rv = dv_ref.caches_host()
        assert torch.equal(gk.view(torch.int16), rk.view(torch.int16))
        assert torch.equal(gv.view(torch.int16), rv.view(torch.int16))
        kc, vc = paging.append(raw(wl.k_cache), raw(wl.v_cache), raw(wl.k_new), raw(wl.v_new),
                               wl.slot_mapping.numpy())
        ref, _ = oracle_attention(wl, kc, vc)
        err = max_err(out, ref)
        say(f"  bit-identical to the workspace step; max abs err vs oracle {err:.3e}")
        assert err <= TOL[c.kv_dtype]


def test_noalloc_decode_step_refuses_more_than_its_scratch(P):
    wl = W.generate(W.scaled("llama3_8b", batch=9, length_range=(1, 100)), spare_blocks=3)
    d = dims_of(P, wl)
    G = 1 << 14          # 65,536 waves' partials do not fit in 16 MiB
    assert P.paged_attn_balanced_workspace_bytes(d, 1, G) > P.PA_NOALLOC_SCRATCH_BYTES
    dv = Dev(wl)
    with pytest.raises(P.PagedAttnError) as e:
        _noalloc_step(P, wl, dv, G)
    assert e.value.status == -10
