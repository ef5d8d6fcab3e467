"""Plant plausible mistakes in a scratch copy of the oracle (on the CPU) and check that
the oracle's pins catch every one of them."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (description, file, original text, planted text, pin file that must fail)
MUTATIONS = [
    ("GQA head mapping", "oracle/attention.py", "h = g * G + hg", "h = hg * (Hq // G) + g",
     "test_oracle_attention.py"),
    ("verify limit off by one", "oracle/attention.py", "seq_len - num_q_pos + 1 + i",
     "seq_len - num_q_pos + i", "test_oracle_attention.py"),
    ("softmax scale dropped", "oracle/attention.py", "s = sigma * (K[lo:lam] @ q_rows[r])",
     "s = (K[lo:lam] @ q_rows[r])", "test_oracle_attention.py"),
    ("lse without the max", "oracle/attention.py", "lse[r] = m + np.log(l)", "lse[r] = np.log(l)",
     "test_oracle_attention.py"),
    ("merge weight sign", "oracle/attention.py", "w = np.exp(lp[live] - M)",
     "w = np.exp(M - lp[live])", "test_oracle_attention.py"),
    ("last partition range", "oracle/attention.py", "hi = seq_len if p == n - 1 else",
     "hi = min(seq_len, (p + 1) * partition_tokens) if p == n - 1 else",
     "test_oracle_attention.py"),
    ("V read along the wrong axis", "oracle/paging.py",
     "V[t] = storage.decode(v_cache[blk, g, :, off]",
     "V[t] = storage.decode(v_cache[blk, g, off % v_cache.shape[2], :]", "test_oracle_paging.py"),
    ("fast V offset", "oracle/paging.py", "V = storage.decode(v_cache[blk, g, :, off], kind, vs)",
     "V = storage.decode(v_cache[blk, g, :, (off + 1) % block_size], kind, vs)",
     "test_oracle_paging.py"),
    ("K columns transposed", "oracle/paging.py",
     "return np.asarray(k_cache[blk, g, :, off, :]).reshape(-1)",
     "return np.asarray(k_cache[blk, g, :, off, :]).T.reshape(-1)", "test_oracle_paging.py"),
    ("fast K columns transposed", "oracle/paging.py",
     "kr = kc[blk, g, :, off, :].reshape(seq_len, kc.shape[2] * kc.shape[4])",
     "kr = kc[blk, g, :, off, :].transpose(0, 2, 1).reshape(seq_len, kc.shape[2] * kc.shape[4])",
     "test_oracle_paging.py"),
    ("append K columns transposed", "oracle/paging.py",
     "kc[blk, g, :, off, :] = np.asarray(k_new[i, g, :]).reshape(kc.shape[2], kc.shape[4])",
     "kc[blk, g, :, off, :] = np.asarray(k_new[i, g, :]).reshape(kc.shape[4], kc.shape[2]).T",
     "test_oracle_paging.py"),
    ("append V reversed", "oracle/paging.py", "vc[blk, g, :, off] = v_new[i, g, :]",
     "vc[blk, g, :, off] = v_new[i, g, ::-1]", "test_oracle_paging.py"),
    ("gather V reversed", "oracle/paging.py", "vo[b, g, t, :] = v_cache[blk, g, :, off]",
     "vo[b, g, t, :] = v_cache[blk, g, ::-1, off]", "test_oracle_paging.py"),
    ("slot off by one", "oracle/paging.py", "return blk * block_size + off",
     "return blk * block_size + off + 1", "test_oracle_paging.py"),
    ("table index shifted", "oracle/paging.py",
     "return int(table_row[t // block_size]), t % block_size",
     "return int(table_row[t // block_size - (t >= block_size)]), t % block_size",
     "test_oracle_paging.py"),
    ("bf16 shift", "oracle/storage.py", "<< np.uint32(16)", "<< np.uint32(15)",
     "test_oracle_paging.py"),
    ("int8 scale dropped", "oracle/storage.py",
     "return q * np.asarray(scale, dtype=np.float32).astype(np.float64)", "return q",
     "test_oracle_paging.py"),
    ("KV-size factor 2 dropped", "oracle/kvsize.py", "return 2 * n_layers * batch",
     "return n_layers * batch", "test_oracle_kvsize.py"),
    ("window one token too wide", "oracle/attention.py",
     "return [max(0, lam - window) for lam in", "return [max(0, lam - window - 1) for lam in",
     "test_oracle_attention.py"),
    ("window start of the last row for every row", "oracle/attention.py",
     "return [max(0, lam - window) for lam in row_limits(seq_len, num_q_pos)]",
     "return [max(0, seq_len - window)] * num_q_pos", "test_oracle_attention.py"),
    ("window start ignored", "oracle/attention.py",
     "lo = 0 if starts is None else max(0, int(starts[r]))", "lo = 0",
     "test_oracle_attention.py"),
    ("int8 scale over 128", "oracle/quant.py", "scale = np.float32(amax / np.float32(QMAX))",
     "scale = np.float32(amax / np.float32(128))", "test_oracle_quant.py"),
    ("int8 rounding toward zero", "oracle/quant.py", "q = np.rint(x / scale)",
     "q = np.trunc(x / scale)", "test_oracle_quant.py"),
    ("append re-encodes only the new token", "oracle/quant.py", "for t in range(off + 1):",
     "for t in range(off, off + 1):", "test_oracle_quant.py"),
    ("staging row ignored", "oracle/quant.py", "row = int(stage_rows[i])", "row = 0",
     "test_oracle_quant.py"),
    ("V encoded from the K staging", "oracle/quant.py",
     "vx = storage.bf16_bits_to_f64(vst[row, g, :off + 1])",
     "vx = storage.bf16_bits_to_f64(kst[row, g, :off + 1])", "test_oracle_quant.py"),
    ("fp8 exponent bias 8", "oracle/storage.py", "np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))",
     "np.ldexp(1.0 + m / 8.0, (e - 8).astype(np.int32))", "test_oracle_quant.py"),
    ("fp8 subnormal exponent", "oracle/storage.py", "np.ldexp(m / 8.0, -6))",
     "np.ldexp(m / 8.0, -7))", "test_oracle_quant.py"),
    ("fp8 saturates to the NaN code", "oracle/quant.py", "            code = 0x7E\n",
     "            code = 0x7F\n", "test_oracle_quant.py"),
    ("fp8 scale over 480", "oracle/quant.py", "scale = np.float32(amax / np.float32(FP8_MAX))",
     "scale = np.float32(amax / np.float32(480))", "test_oracle_quant.py"),
    ("fp8 ties away from zero", "oracle/quant.py", "r = int(np.rint(a * 2.0 ** (3 - e)))",
     "r = int(np.floor(a * 2.0 ** (3 - e) + 0.5))", "test_oracle_quant.py"),
    ("tree mask transposed", "oracle/attention.py",
     "vis = [tree_visible(L, nq, i, tree_mask[b][i]) for i in range(nq)]",
     "vis = [tree_visible(L, nq, i, [tree_mask[b][r][i] for r in range(nq)]) for i in range(nq)]",
     "test_oracle_attention.py"),
    ("tree context one token short", "oracle/attention.py", "ctx = list(range(max(0, base)))",
     "ctx = list(range(max(0, base - 1)))", "test_oracle_attention.py"),
    ("tree candidate shifted", "oracle/attention.py", "if mask_row[j] and base + j >= 0]",
     "if mask_row[j - 1] and base + j >= 0]", "test_oracle_attention.py"),
    ("copy direction swapped", "oracle/paging.py", "kc[dst] = k_cache[src]",
     "kc[src] = k_cache[dst]", "test_oracle_paging.py"),
    ("copy skips V", "oracle/paging.py", "vc[dst] = v_cache[src]", "pass",
     "test_oracle_paging.py"),
    ("copy skips scales", "oracle/paging.py", "ks[dst] = k_scale[src]", "pass",
     "test_oracle_paging.py"),
]


def _run(tmp_root, idx, mut):
    desc, path, old, new, pin = mut
    work = os.path.join(tmp_root, f"m{idx}")
    for d in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(work, d),
                        ignore=shutil.ignore_patterns("__pycache__"))
    target = os.path.join(work, path)
    text = open(target).read()
    assert old in text, f"mutation site gone: {desc}"
    open(target, "w").write(text.replace(old, new, 1))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", pin)], cwd=work, env=env, capture_output=True,
                       text=True, timeout=600)
    return desc, r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda im: _run(str(tmp_path), *im), enumerate(MUTATIONS)))
    survived = [d for d, rc in results if rc == 0]
    assert not survived, f"planted mistakes not caught: {survived}"
