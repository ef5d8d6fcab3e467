"""ctypes binding of libpaged_attn.so (argument marshalling only).

Each function has the name of the C entry point it calls and takes the same arguments,
with torch tensors (or raw integer device addresses, or None for NULL) in place of
pointers.  All computation happens in the HIP kernels behind the C ABI; a non-zero
status raises PagedAttnError.  There is no fallback: if the library is missing, importing
this module fails.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpaged_attn.so")

PA_F32, PA_BF16, PA_I8, PA_FP8 = 0, 1, 2, 3
PA_OK = 0
PA_ERR_NULL, PA_ERR_DIMS, PA_ERR_DTYPE, PA_ERR_HEAD_DIM = -1, -2, -3, -4
PA_ERR_BLOCK_SIZE, PA_ERR_WORKSPACE, PA_ERR_LAUNCH, PA_ERR_PARTITION = -5, -6, -7, -8
PA_ERR_ALIGN, PA_ERR_SCRATCH = -9, -10
PA_NOALLOC_SCRATCH_BYTES = 16 << 20

_DTYPE_CODE = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int8: PA_I8,
               torch.float8_e4m3fn: PA_FP8,
               "f32": PA_F32, "bf16": PA_BF16, "i8": PA_I8, "fp8": PA_FP8}


class PagedAttnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {paged_status_string(status)} (status {status})")


class pa_dims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("q_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("kv_tile_stride", ctypes.c_int64),
                ("sliding_window", ctypes.c_int32)]


def _load(path=_LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python paged_gqa_decode_kv_amd/build.py`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    D = ctypes.POINTER(pa_dims)
    sig = {
        "kv_append": [D, P, P, P, I32, P, P, P],
        "paged_decode_attn": [D, P, P, P, P, P, P, P, F32, P, P],
        "paged_verify_attn": [D, I32, P, P, P, P, P, P, P, F32, P, P],
        "paged_decode_attn_split": [D, P, P, P, P, P, P, P, F32, I32, I32, P, P, P],
        "lse_merge": [D, P, P, P, I32, I32, P, P, P],
        "kv_gather": [D, P, P, P, P, I32, P, P, P],
        "paged_attn_balanced": [D, I32, P, P, P, P, P, P, P, F32, I32, P, ctypes.c_size_t, P, P, P],
        "paged_attn_balanced_workgroups": [D, I32],
        "paged_attn_balanced_merge": [D, I32, I32, P, ctypes.c_size_t, P, P, P],
        "paged_decode_step": [D, P, P, P, P, P, P, P, F32, I32, P, ctypes.c_size_t, P, P, P],
        "paged_decode_step_noalloc": [D, P, P, P, P, P, P, P, F32, I32, P, P, P],
        "kv_copy_blocks": [D, P, I32, P, P, P, P, P],
        "kv_append_quant": [D, P, P, P, P, I32, I32, P, P, P, P, P, P, P],
        "paged_multi_query_attn": [D, I32, P, P, P, P, P, P, P, P, F32, P, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.paged_split_workspace_bytes.argtypes = [D, I32]
    lib.paged_split_workspace_bytes.restype = ctypes.c_size_t
    lib.paged_attn_balanced_workspace_bytes.argtypes = [D, I32, I32]
    lib.paged_attn_balanced_workspace_bytes.restype = ctypes.c_size_t
    lib.paged_status_string.argtypes = [ctypes.c_int]
    lib.paged_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()
LIB_PATH = _LIB_PATH


def make_dims(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, num_blocks,
              q_dtype, kv_dtype, block_size=16, kv_tile_stride=0, sliding_window=0):
    """kv_tile_stride: elements between consecutive (block, KV head) tiles (0 = dense);
    sliding_window: tokens each row attends, ending at its own position (0 = all)."""
    return pa_dims(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                   max_blocks_per_seq, num_blocks, _DTYPE_CODE[q_dtype], _DTYPE_CODE[kv_dtype],
                   kv_tile_stride, sliding_window)


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    if not x.is_contiguous():
        raise ValueError("tensors passed to the C ABI must be contiguous")
    return ctypes.c_void_p(x.data_ptr())


# torch's current-stream handle without building a Stream object (torch.cuda.current_stream()
# took ~3.5 us a call, a third of an enqueue); the public call when the accessor is absent
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_raw_device = getattr(torch._C, "_cuda_getDevice", None)
_has_gpu = None


def _stream(stream):
    global _has_gpu
    if stream is not None:
        return ctypes.c_void_p(stream) if isinstance(stream, int) else ctypes.c_void_p(stream.cuda_stream)
    if _has_gpu is None:
        _has_gpu = torch.cuda.is_available()
    if not _has_gpu:
        return None
    if _raw_stream is not None and _raw_device is not None:
        return ctypes.c_void_p(_raw_stream(_raw_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, st):
    if st != PA_OK:
        raise PagedAttnError(fn, st)


def paged_status_string(status):
    return lib.paged_status_string(status).decode()


def kv_append(dims, k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, stream=None):
    _check("kv_append", lib.kv_append(ctypes.byref(dims), _p(k_new), _p(v_new), _p(slot_mapping),
                                      num_tokens, _p(k_cache), _p(v_cache), _stream(stream)))


def paged_decode_attn(dims, q, k_cache, v_cache, k_scale, v_scale, block_tables, seq_lens,
                      sm_scale, out, stream=None):
    _check("paged_decode_attn", lib.paged_decode_attn(
        ctypes.byref(dims), _p(q), _p(k_cache), _p(v_cache), _p(k_scale), _p(v_scale),
        _p(block_tables), _p(seq_lens), sm_scale, _p(out), _stream(stream)))


def paged_verify_attn(dims, num_q_pos, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                      seq_lens, sm_scale, out, stream=None):
    _check("paged_verify_attn", lib.paged_verify_attn(
        ctypes.byref(dims), num_q_pos, _p(q), _p(k_cache), _p(v_cache), _p(k_scale), _p(v_scale),
        _p(block_tables), _p(seq_lens), sm_scale, _p(out), _stream(stream)))


def paged_decode_attn_split(dims, q, k_cache, v_cache, k_scale, v_scale, block_tables, seq_lens,
                            sm_scale, partition_tokens, max_partitions, part_out, part_lse,
                            stream=None):
    _check("paged_decode_attn_split", lib.paged_decode_attn_split(
        ctypes.byref(dims), _p(q), _p(k_cache), _p(v_cache), _p(k_scale), _p(v_scale),
        _p(block_tables), _p(seq_lens), sm_scale, partition_tokens, max_partitions,
        _p(part_out), _p(part_lse), _stream(stream)))


def lse_merge(dims, part_out, part_lse, seq_lens, partition_tokens, max_partitions, out,
              out_lse=None, stream=None):
    _check("lse_merge", lib.lse_merge(
        ctypes.byref(dims), _p(part_out), _p(part_lse), _p(seq_lens), partition_tokens,
        max_partitions, _p(out), _p(out_lse), _stream(stream)))


def paged_split_workspace_bytes(dims, max_partitions):
    return lib.paged_split_workspace_bytes(ctypes.byref(dims), max_partitions)


def kv_gather(dims, k_cache, v_cache, block_tables, seq_lens, max_len, k_out, v_out, stream=None):
    _check("kv_gather", lib.kv_gather(ctypes.byref(dims), _p(k_cache), _p(v_cache),
                                      _p(block_tables), _p(seq_lens), max_len, _p(k_out),
                                      _p(v_out), _stream(stream)))


def paged_attn_balanced_workgroups(dims, num_q_pos):
    n = lib.paged_attn_balanced_workgroups(ctypes.byref(dims), num_q_pos)
    _check("paged_attn_balanced_workgroups", n if n < 0 else PA_OK)
    return n


def paged_attn_balanced_workspace_bytes(dims, num_q_pos, num_workgroups):
    return lib.paged_attn_balanced_workspace_bytes(ctypes.byref(dims), num_q_pos, num_workgroups)


def paged_attn_balanced(dims, num_q_pos, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                        seq_lens, sm_scale, num_workgroups, workspace, out, out_lse=None,
                        stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check("paged_attn_balanced", lib.paged_attn_balanced(
        ctypes.byref(dims), num_q_pos, _p(q), _p(k_cache), _p(v_cache), _p(k_scale), _p(v_scale),
        _p(block_tables), _p(seq_lens), sm_scale, num_workgroups, _p(workspace), nbytes, _p(out),
        _p(out_lse), _stream(stream)))


def kv_append_quant(dims, k_new, v_new, slot_mapping, stage_rows, num_tokens, k_stage, v_stage,
                    k_cache, v_cache, k_scale, v_scale, stream=None):
    """num_stage_rows is taken from k_stage's first dimension."""
    _check("kv_append_quant", lib.kv_append_quant(
        ctypes.byref(dims), _p(k_new), _p(v_new), _p(slot_mapping), _p(stage_rows), num_tokens,
        k_stage.shape[0], _p(k_stage), _p(v_stage), _p(k_cache), _p(v_cache), _p(k_scale),
        _p(v_scale), _stream(stream)))


def paged_multi_query_attn(dims, num_q_pos, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                           seq_lens, sm_scale, out, out_lse=None, tree_mask=None, stream=None):
    """tree_mask: int32 bit rows [B][nq][ceil(nq/32)] (workloads.tree_mask_words) or None."""
    _check("paged_multi_query_attn", lib.paged_multi_query_attn(
        ctypes.byref(dims), num_q_pos, _p(q), _p(k_cache), _p(v_cache), _p(k_scale), _p(v_scale),
        _p(block_tables), _p(seq_lens), _p(tree_mask), ctypes.c_float(sm_scale), _p(out),
        _p(out_lse), _stream(stream)))


def kv_copy_blocks(dims, block_pairs, num_pairs, k_cache, v_cache, k_scale=None, v_scale=None,
                   stream=None):
    _check("kv_copy_blocks", lib.kv_copy_blocks(
        ctypes.byref(dims), _p(block_pairs), num_pairs, _p(k_cache), _p(v_cache), _p(k_scale),
        _p(v_scale), _stream(stream)))


def paged_decode_step(dims, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, sm_scale,
                      num_workgroups, workspace, out, out_lse=None, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check("paged_decode_step", lib.paged_decode_step(
        ctypes.byref(dims), _p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache),
        _p(block_tables), _p(seq_lens), sm_scale, num_workgroups, _p(workspace), nbytes, _p(out),
        _p(out_lse), _stream(stream)))


def paged_decode_step_noalloc(dims, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens,
                              sm_scale, num_workgroups, out, out_lse=None, stream=None):
    _check("paged_decode_step_noalloc", lib.paged_decode_step_noalloc(
        ctypes.byref(dims), _p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache),
        _p(block_tables), _p(seq_lens), sm_scale, num_workgroups, _p(out), _p(out_lse),
        _stream(stream)))


def paged_attn_balanced_merge(dims, num_q_pos, num_workgroups, workspace, out, out_lse=None,
                              stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check("paged_attn_balanced_merge", lib.paged_attn_balanced_merge(
        ctypes.byref(dims), num_q_pos, num_workgroups, _p(workspace), nbytes, _p(out),
        _p(out_lse), _stream(stream)))
