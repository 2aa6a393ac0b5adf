"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
that the pins catch every one of them: evidence that the pins constrain each
step of the oracle, not just its overall shape."""
import importlib.util
import os
import shutil
import sys

import pytest

from oracle_pins import ALL_CHECKS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (file, exact original text, planted mistake)
MUTATIONS = [
    ("attention.py", "        kvh = h // groups\n        out[i] =", "        kvh = h % n_kv\n        out[i] ="),
    ("attention.py", "        kvh = h // groups\n        out[:, j, :]", "        kvh = h % n_kv\n        out[:, j, :]"),
    ("attention.py", "s = (keys[:n] @ q_rows[r]) * scale", "s = (keys[:n] @ q_rows[r])"),
    ("attention.py", "visible = np.array([ctx + i + 1 for i in rows])", "visible = np.array([ctx + i for i in rows])"),
    ("attention.py", "visible = np.full(len(rows), ctx + q_len)", "visible = np.full(len(rows), ctx)"),
    ("attention.py", "w = e / np.sum(e)", "w = e / n"),
    ("attention.py", "c = np.max(s)", "c = 0.0"),
    ("attention.py", "out[r] = w @ values[:n]", "out[r] = w @ keys[:n]"),
    ("attention.py", "out[r] = w @ values[:n]", "out[r] = w[::-1] @ values[:n]"),
    ("attention.py", "K = K * gather_scales(k_scale,", "K = K * gather_scales(v_scale,"),
    ("attention.py", "V = V * gather_scales(v_scale,", "V = V * gather_scales(k_scale,"),
    ("attention.py", "L = int(seq_lens[seq])", "L = int(seq_lens[seq]) - 1"),
    ("paging.py", "offset = pos % block_size", "offset = block_size - 1 - pos % block_size"),
    ("paging.py", "    block_size = cache.shape[2]\n    rows = []", "    block_size = 16\n    rows = []"),
    ("paging.py", "return list(kv_indices[kv_indptr[request]:kv_indptr[request + 1]])",
     "return list(kv_indices[kv_indptr[request]:kv_indptr[request + 1] + 1])"),
    ("paging.py", "physical_block = int(block_table[seq][pos // block_size])",
     "physical_block = int(block_table[seq][pos // block_size]) + 1"),
    ("paging.py", "rows.append(cache[block, :, p % block_size, :])", "rows.append(cache[block, :, (p + 1) % block_size, :])"),
    ("paging.py", "v_out[block, :, offset, :] = v_new[t]", "v_out[block, :, offset, :] = k_new[t]"),
    ("paging.py", "        if slot < 0:\n            continue\n", "        if slot < -1:\n            continue\n"),
    ("paging.py", "return 2 * n_layers * n_kv_heads * d_head * bytes_per_value",
     "return n_layers * n_kv_heads * d_head * bytes_per_value"),
    ("paging.py", "return blocks * block_size - seq_len", "return blocks * block_size - seq_len + 1"),
    ("codecs.py", "np.exp2(exp_field - 7.0)", "np.exp2(exp_field - 8.0)"),
    ("codecs.py", "subnormal = (man / 8.0) * 2.0 ** -6", "subnormal = (man / 8.0) * 2.0 ** -7"),
    ("codecs.py", "normal = (1.0 + man / 8.0)", "normal = (1.0 + man / 16.0)"),
    ("codecs.py", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("codecs.py", "val = np.where(sign == 1, -mag, mag)", "val = mag"),
    ("sharing.py", "                if self.ref[row[j]] > 1:", "                if self.ref[row[j]] >= 1:"),
    ("sharing.py", "                    self.release([row[j]])\n", ""),
    ("sharing.py", "out = [b for b, r in enumerate(self.ref) if r == 0][:n]",
     "out = [b for b, r in enumerate(self.ref) if r == 0][::-1][:n]"),
    ("sharing.py", "first, last = seq_len // block_size,", "first, last = (seq_len + 1) // block_size,"),
    ("sharing.py", "            self.ref[b] += 1", "            self.ref[b] += 2"),
    ("sharing.py", "        k[dst] = k_cache[src]", "        k[dst] = v_cache[src]"),
    ("sharing.py", "            vs[dst] = v_scale[src]", "            vs[dst] = k_scale[src]"),
    ("swap.py", "    parts += [_raw(v_cache[int(b)]).reshape(-1) for b in ids]",
     "    parts += [_raw(k_cache[int(b)]).reshape(-1) for b in ids]"),
    ("swap.py", "    parts = [_raw(k_cache[int(b)]).reshape(-1) for b in ids]",
     "    parts = [_raw(k_cache[int(b)]).reshape(-1) for b in ids[::-1]]"),
    ("swap.py", "        parts += [_raw(v_scale[int(b)]).reshape(-1) for b in ids]\n", ""),
    ("swap.py", "        off += n * size\n", "        off += size\n"),
    ("quant.py", "        codes[:n_old] = encode_e4m3fn(vals / new)\n", ""),
    ("quant.py", "np.float32(m / _F448)", "np.float32(m / np.float32(256.0))"),
    ("quant.py", "(codes[hi] % 2 == 0)", "(codes[hi] % 2 == 1)"),
    ("quant.py", "old = np.float32(scale) if n_old > 0 else np.float32(0.0)", "old = np.float32(0.0)"),
    ("quant.py", "n_old = min(max(ctx - j * B, 0), B)", "n_old = min(max(ctx - j * B - 1, 0), B)"),
    ("quant.py", "vals = e4m3fn_to_f64(codes[:n_old]).astype(np.float32) * old",
     "vals = e4m3fn_to_f64(codes[:n_old]).astype(np.float32) * new"),
]


def _load_mutant(tmp_path, idx, fname, old, new):
    src = os.path.join(ROOT, "oracle")
    name = f"oracle_mutant_{idx}"
    dst = tmp_path / name
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("__pycache__"))
    path = dst / fname
    text = path.read_text()
    assert text.count(old) == 1, f"mutation anchor must occur exactly once: {old!r}"
    path.write_text(text.replace(old, new))
    spec = importlib.util.spec_from_file_location(name, dst / "__init__.py", submodule_search_locations=[str(dst)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("idx", range(len(MUTATIONS)))
def test_pins_catch_planted_mistake(tmp_path, idx):
    fname, old, new = MUTATIONS[idx]
    mutant = _load_mutant(tmp_path, idx, fname, old, new)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(mutant)
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append((check.__name__, type(e).__name__))
    sys.modules.pop(f"oracle_mutant_{idx}", None)
    assert caught, f"no pin caught mutation {idx}: {fname}: {old!r} -> {new!r}"
