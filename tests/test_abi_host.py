"""The C ABI on a host without a GPU: the library loads, exports every function the header
declares, and every argument check returns its status before any HIP call."""
import ctypes
import os
import re

import pytest

import paged_gqa_decode_kv_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const\s+char\s*\*)\s*\*?\s*"
                       r"(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["kv_append", "paged_decode_attn", "paged_verify_attn", "paged_decode_attn_split",
              "lse_merge", "paged_attn_balanced", "paged_attn_balanced_merge",
              "paged_attn_balanced_workspace_bytes", "paged_attn_balanced_workgroups",
              "paged_split_workspace_bytes", "kv_gather", "paged_status_string",
              "paged_decode_step", "kv_copy_blocks", "kv_append_quant",
              "paged_multi_query_attn", "paged_decode_step_noalloc"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(P.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def _dims(**kw):
    base = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=64, max_blocks_per_seq=4,
                num_blocks=16, q_dtype="bf16", kv_dtype="bf16")
    base.update(kw)
    return P.make_dims(**base)


FAKE = 0x1000  # a non-NULL address that is never dereferenced: every call below fails its checks


def _decode(d, q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, t=FAKE, lens=FAKE, out=FAKE):
    args = [ctypes.c_void_p(x) if x else None for x in (q, k, v, ks, vs, t, lens)]
    return P.lib.paged_decode_attn(ctypes.byref(d), *args, 0.125,
                                   ctypes.c_void_p(out) if out else None, None)


@pytest.mark.parametrize("change,status", [
    (dict(block_size=8), -5),
    (dict(head_dim=96), -4),
    (dict(num_seqs=0), -2),
    (dict(num_q_heads=6, num_kv_heads=4), -2),
    (dict(num_kv_heads=0), -2),
    (dict(max_blocks_per_seq=0), -2),
    (dict(num_blocks=0), -2),
    (dict(sliding_window=-1), -2),
    (dict(q_dtype="f32", kv_dtype="bf16"), -3),
    (dict(q_dtype="bf16", kv_dtype="f32"), -3),
    (dict(q_dtype="f32", kv_dtype="fp8"), -3),
    (dict(kv_dtype=7), -3),
])
def test_decode_dimension_and_type_checks(change, status):
    d = _dims()
    for k, v in change.items():
        setattr(d, k, {"f32": 0, "bf16": 1, "i8": 2, "fp8": 3}.get(v, v) if isinstance(v, str) else v)
    assert _decode(d) == status


def test_tile_stride_and_alignment_checks():
    for stride, status in [(16 * 64, 0), (32 * 64, 0), (16 * 64 - 8, -2), (16 * 64 + 4, -2),
                           (16 * 64 + 8, 0), (-1, -2)]:
        d = _dims(kv_tile_stride=stride)
        st = P.lib.kv_gather(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                             ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 0, ctypes.c_void_p(FAKE),
                             ctypes.c_void_p(FAKE), None)
        assert st == status, (stride, st)        # max_len 0: checks only, nothing launched
    d = _dims()
    assert _decode(d, q=FAKE + 8) == -9
    assert _decode(d, k=FAKE + 4) == -9
    assert _decode(d, v=FAKE + 2) == -9
    assert _decode(d, out=FAKE + 8) == -9


def test_copy_blocks_checks():
    d = _dims()
    f = ctypes.c_void_p(FAKE)
    assert P.lib.kv_copy_blocks(ctypes.byref(d), f, -1, f, f, None, None, None) == -2
    assert P.lib.kv_copy_blocks(ctypes.byref(d), f, 0, f, f, None, None, None) == 0
    assert P.lib.kv_copy_blocks(ctypes.byref(d), None, 3, f, f, None, None, None) == -1
    di8 = _dims(kv_dtype="i8")
    assert P.lib.kv_copy_blocks(ctypes.byref(di8), f, 3, f, f, None, None, None) == -1
    assert P.lib.kv_copy_blocks(ctypes.byref(d), f, 3, ctypes.c_void_p(FAKE + 4), f, None, None,
                                None) == -9


def test_null_pointer_checks():
    d = _dims()
    assert P.lib.paged_decode_attn(None, None, None, None, None, None, None, None, 0.1, None,
                                   None) == -1
    assert _decode(d, q=0) == -1
    assert _decode(d, lens=0) == -1
    assert _decode(d, out=0) == -1
    di8 = _dims(kv_dtype="i8")
    assert _decode(di8) == -1                 # int8 needs both scale arrays
    assert _decode(di8, ks=FAKE) == -1


def test_append_checks():
    d = _dims()
    f = ctypes.c_void_p(FAKE)
    assert P.lib.kv_append(ctypes.byref(d), f, f, f, -1, f, f, None) == -2
    assert P.lib.kv_append(ctypes.byref(d), f, f, f, 0, f, f, None) == 0     # nothing to do
    assert P.lib.kv_append(ctypes.byref(d), None, f, f, 4, f, f, None) == -1
    di8 = _dims(kv_dtype="i8")
    assert P.lib.kv_append(ctypes.byref(di8), f, f, f, 4, f, f, None) == -3


def test_verify_and_split_checks():
    d = _dims()
    f = ctypes.c_void_p(FAKE)
    assert P.lib.paged_verify_attn(ctypes.byref(d), 0, f, f, f, None, None, f, f, 0.1, f,
                                   None) == -2
    for pt, mp in [(0, 4), (24, 4), (-16, 4), (16, 0)]:
        assert P.lib.paged_decode_attn_split(ctypes.byref(d), f, f, f, None, None, f, f, 0.1,
                                             pt, mp, f, f, None) == -8
        assert P.lib.lse_merge(ctypes.byref(d), f, f, f, pt, mp, f, None, None) == -8
    assert P.lib.paged_decode_attn_split(ctypes.byref(d), f, f, f, None, None, f, f, 0.1, 32, 4,
                                         None, f, None) == -1
    assert P.lib.kv_gather(ctypes.byref(d), f, f, f, f, -1, f, f, None) == -2
    assert P.lib.kv_gather(ctypes.byref(d), f, f, f, f, 0, f, f, None) == 0


def test_balanced_checks_and_sizes():
    d = _dims()
    f = ctypes.c_void_p(FAKE)
    n = P.paged_attn_balanced_workspace_bytes(d, 1, 8)
    # prefix (3 ints -> 256 B) | lse (8 workgroups x 4 waves + 2*1*2 segments partials
    # x 16 rows) | rows (x 64 dims)
    npid = 8 * 4 + 2 * 2
    assert n == 256 + ((npid * 16 * 4 + 255) // 256) * 256 + npid * 16 * 64 * 4
    assert P.paged_attn_balanced_workspace_bytes(d, 6, 8) > n          # 24 rows -> 32-row tile
    assert P.paged_attn_balanced_workspace_bytes(d, 0, 8) == 0
    assert P.paged_attn_balanced_workspace_bytes(d, 1, 0) == 0
    big = _dims(num_seqs=4096)
    assert P.paged_attn_balanced_workspace_bytes(big, 1, 8) == 0       # more than 2048 sequences
    # flat block positions and tile indices must stay int32
    assert P.paged_attn_balanced_workspace_bytes(_dims(num_seqs=2048, max_blocks_per_seq=1 << 19),
                                                 1, 8) == 0
    assert P.paged_attn_balanced_workspace_bytes(_dims(num_blocks=1 << 30), 1, 8) == 0
    assert P.paged_attn_balanced_workspace_bytes(_dims(num_blocks=1 << 29), 1, 8) > 0
    call = P.lib.paged_attn_balanced
    assert call(ctypes.byref(d), 1, f, f, f, None, None, f, f, 0.1, 8, f, n - 1, f, None,
                None) == -6
    assert call(ctypes.byref(d), 1, f, f, f, None, None, f, f, 0.1, 8, ctypes.c_void_p(FAKE + 4),
                n, f, None, None) == -6                                 # misaligned
    assert call(ctypes.byref(d), 1, f, f, f, None, None, f, f, 0.1, 0, f, n, f, None, None) == -2
    assert P.lib.paged_attn_balanced_merge(ctypes.byref(d), 1, 8, f, n - 1, f, None, None) == -6
    assert P.lib.paged_split_workspace_bytes(ctypes.byref(d), 3) == 2 * 8 * 3 * (64 + 1) * 4


def test_status_strings():
    for st in range(0, -11, -1):
        assert P.paged_status_string(st) and P.paged_status_string(st) != "unknown status"
    assert P.paged_status_string(-99) == "unknown status"


def test_binding_raises_on_status():
    d = _dims(head_dim=80)
    with pytest.raises(P.PagedAttnError) as e:
        P.paged_decode_attn(d, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 0.1, FAKE)
    assert e.value.status == -4


def test_append_quant_checks():
    f = ctypes.c_void_p(FAKE)
    d = _dims(kv_dtype="i8")
    args = lambda n, rows=4, **kw: [kw.get(k, f) for k in ("kn", "vn", "sm", "sr")] + \
        [n, rows] + [kw.get(k, f) for k in ("kst", "vst", "kc", "vc", "ks", "vs")] + [None]
    assert P.lib.kv_append_quant(ctypes.byref(d), *args(0)) == 0
    assert P.lib.kv_append_quant(ctypes.byref(d), *args(-1)) == -2
    assert P.lib.kv_append_quant(ctypes.byref(d), *args(2, rows=-1)) == -2
    assert P.lib.kv_append_quant(ctypes.byref(d), *args(2, ks=None)) == -1
    assert P.lib.kv_append_quant(ctypes.byref(d), *args(2, kst=ctypes.c_void_p(FAKE + 2))) == -9
    db = _dims()
    assert P.lib.kv_append_quant(ctypes.byref(db), *args(2)) == -3
    d8 = _dims(kv_dtype="fp8")
    assert P.lib.kv_append_quant(ctypes.byref(d8), *args(0)) == 0
    assert P.lib.kv_append_quant(ctypes.byref(d8), *args(2, vs=None)) == -1
    # fp8 attention needs the scales like int8
    assert _decode(d8) == -1 and _decode(d8, ks=FAKE, vs=FAKE, out=FAKE + 8) == -9


def test_multi_query_checks():
    f = ctypes.c_void_p(FAKE)

    def call(d, nq, mask=None, out=FAKE):
        return P.lib.paged_multi_query_attn(ctypes.byref(d), nq, f, f, f, None, None, f, f, mask,
                                            ctypes.c_float(0.1), ctypes.c_void_p(out) if out else None,
                                            None, None)
    d = _dims()
    assert call(d, 0) == -2
    assert call(d, 4, out=None) == -1
    assert call(d, 4, out=FAKE + 4) == -9
    assert call(d, 129, mask=f) == -2                  # a mask covers at most 128 candidates
    assert call(_dims(sliding_window=8), 4, mask=f) == -2
    assert call(_dims(kv_dtype="i8"), 4) == -1         # 8-bit caches need their scales


def test_grid_limits_are_checked_before_any_launch():
    """Sizes whose grid would not fit the launch limits fail on the host (no HIP call)."""
    f = ctypes.c_void_p(FAKE)
    d = _dims(num_kv_heads=8, num_q_heads=8)
    # 2^31 - 1 pairs x 16 pieces per pair
    assert P.lib.kv_copy_blocks(ctypes.byref(d), f, 2 ** 31 - 1, f, f, None, None, None) == -2
    d8 = _dims(kv_dtype="i8", num_kv_heads=8, num_q_heads=8)
    assert P.lib.kv_append_quant(ctypes.byref(d8), f, f, f, f, 2 ** 31 - 1, 4, f, f, f, f, f, f,
                                 None) == -2
    big = _dims(num_q_heads=64, num_kv_heads=1)
    assert P.lib.paged_multi_query_attn(ctypes.byref(big), 2 ** 30, f, f, f, None, None, f, f, None,
                                        ctypes.c_float(0.1), f, None, None) == -2


def test_header_compiles_as_plain_c(tmp_path):
    """The ABI header is usable from C: a C99 translation unit that includes it, takes the
    address of every declared function and fills a pa_dims compiles warning-free."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = ["#include \"paged_attn.h\"", "#include <stddef.h>", "",
           "int main(void) {",
           "  pa_dims d = {0};",
           "  d.block_size = 16;",
           "  typedef void (*fn_t)(void);",
           "  const fn_t fns[] = {"]
    src += [f"    (fn_t)&{n}," for n in names]
    src += ["  };", "  return (int)(sizeof fns / sizeof fns[0]) - (int)d.block_size + 16 - "
            f"{len(names)};", "}"]
    c_file = tmp_path / "abi.c"
    c_file.write_text("\n".join(src) + "\n")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    for std in ("c99", "c11"):
        r = subprocess.run([cc, f"-std={std}", "-Wall", "-Wextra", "-pedantic", "-Werror",
                            "-I", inc, "-c", str(c_file), "-o", str(tmp_path / "abi.o")],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_noalloc_decode_step_checks():
    """The allocation-free decode step runs the decode step's host checks, and a call that
    needs more than the static scratch is refused, all before any HIP call."""
    f = ctypes.c_void_p(FAKE)

    def call(d, G=8, out=FAKE, k_new=FAKE):
        return P.lib.paged_decode_step_noalloc(
            ctypes.byref(d), f, ctypes.c_void_p(k_new) if k_new else None, f, f, f, f, f,
            ctypes.c_float(0.1), G, ctypes.c_void_p(out) if out else None, None, None)
    assert call(_dims(head_dim=80)) == -4
    assert call(_dims(kv_dtype="i8")) == -3
    assert call(_dims(), k_new=None) == -1
    assert call(_dims(), out=FAKE + 4) == -9
    assert call(_dims(), G=0) == -2
    # 2048 sequences x 8 KV heads: 16,384 segments of 16 rows x 128 dims, ~134 MB
    big = _dims(num_seqs=2048, num_q_heads=32, num_kv_heads=8, head_dim=128)
    assert P.paged_attn_balanced_workspace_bytes(big, 1, 256) > P.PA_NOALLOC_SCRATCH_BYTES
    assert call(big, G=256) == -10
    assert "scratch" in P.paged_status_string(-10)
