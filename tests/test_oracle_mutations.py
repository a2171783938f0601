"""The oracle's pins catch plausible mistakes.

For each oracle function, one plausible mistake (an off-by-one, a dropped
term, a wrong index, a wrong rounding) is planted in a temporary copy of
`oracle/`, and that function's pin file is run against the copy in a child
process: it must fail (pytest exit status 1: failed tests, not a collection
or usage error).  An unmodified copy must pass, so a broken harness cannot
count as a catch.  CPU only; nothing here touches the GPU path.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (label, oracle file, text, planted replacement, pin file)
MUTATIONS = [
    ("window bound", "attention.py", "return (d >= 0) & (d < window)", "return (d >= 0) & (d <= window)",
     "test_oracle_attention.py"),
    ("causal bound", "attention.py", "        return d >= 0\n", "        return d > 0\n", "test_oracle_attention.py"),
    ("softmax scale", "attention.py", "s = float(scale) * (q @ k.T)", "s = (q @ k.T)", "test_oracle_attention.py"),
    ("GQA head map", "attention.py", "return h // (Hq // Hkv)", "return h % Hkv", "test_oracle_attention.py"),
    ("INT8 K scale", "attention.py", "kk = np.concatenate([dequant_int8_b32(k_codes[b, g], k_scales[b, g], block)",
     "kk = np.concatenate([dequant_int8_b32(k_codes[b, g], v_scales[b, g], block)", "test_oracle_attention.py"),
    ("selected block index", "attention.py", "mask[r] |= np.isin(key_block, chosen)",
     "mask[r] |= np.isin(key_block, chosen + 1)", "test_oracle_attention.py"),
    ("INT8 rounding", "quant.py", "c = np.clip(np.rint(quot), -127, 127)", "c = np.clip(np.floor(quot + 0.5), -127, 127)",
     "test_oracle_quant.py"),
    ("INT8 scale divisor", "quant.py", "a / np.float32(127)", "a / np.float32(128)", "test_oracle_quant.py"),
    ("ring slot", "ring.py", "return np.asarray(pos, dtype=np.int64) % W", "return (np.asarray(pos, dtype=np.int64) + 1) % W",
     "test_oracle_select_ring.py"),
    ("strictly earlier blocks", "select.py", "key = np.where(kb_idx < qb_idx, -sc, np.inf)",
     "key = np.where(kb_idx <= qb_idx, -sc, np.inf)", "test_oracle_select_ring.py"),
    ("block score KV head", "select.py", "g = h // (Hq // Hkv)", "g = h % Hkv", "test_oracle_select_ring.py"),
    ("chunk ring slot", "chunk.py", "kl[j] = ring_k[b, :, p % W]", "kl[j] = ring_k[b, :, (p + 1) % W]",
     "test_oracle_chunk.py"),
    ("needed positions", "prefix.py", "for p in range(max(0, ell - W), ell)", "for p in range(max(0, ell - W + 1), ell)",
     "test_oracle_prefix.py"),
    ("block mean divisor", "sparse_decode.py", "(prod * np.float32(1.0 / BLOCK))", "(prod / np.float32(BLOCK - 1))",
     "test_oracle_sparse_decode.py"),
    ("sparse score KV head", "sparse_decode.py", "sc = means[b, g] @ q[b, h]", "sc = means[b, h % Hkv] @ q[b, h]",
     "test_oracle_sparse_decode.py"),
    ("kept block tokens", "sparse_decode.py", "visible[BLOCK * j:BLOCK * (j + 1)] = True",
     "visible[BLOCK * j + 1:BLOCK * (j + 1) + 1] = True", "test_oracle_sparse_decode.py"),
    ("pair count", "closed_forms.py", "return W * (W + 1) // 2 + (L - W) * W", "return W * (W - 1) // 2 + (L - W) * W",
     "test_oracle_select_ring.py"),
]

# Imports the (possibly mutated) copy before pytest runs, so every test module's
# `import oracle` gets it; then runs one pin file.
RUNNER = """
import sys
sys.path.insert(0, sys.argv[1])
import oracle
assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__
sys.path.insert(1, sys.argv[2])
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider"] + sys.argv[3:]))
"""


def _run(tmp, label, edit):
    copy = os.path.join(tmp, label.replace(" ", "_"))
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(copy, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    pins = sorted({m[4] for m in MUTATIONS})  # the control runs every pin file
    if edit is not None:
        fname, old, new, pin = edit
        pins = [pin]
        path = os.path.join(copy, "oracle", fname)
        text = open(path).read()
        assert text.count(old) == 1, (label, "mutation site not unique or missing")
        open(path, "w").write(text.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", RUNNER, copy, ROOT] + [os.path.join(ROOT, "tests", p) for p in pins],
                       cwd=copy, env=env, capture_output=True, text=True, timeout=600)
    return label, r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


def test_planted_mistakes_fail_their_pins(tmp_path):
    jobs = [("control", None)] + [(m[0], m[1:]) for m in MUTATIONS]
    with ThreadPoolExecutor(4) as ex:
        results = list(ex.map(lambda j: _run(str(tmp_path), *j), jobs))
    control = results[0]
    assert control[1] == 0, f"unmodified oracle fails its pins:\n{control[2]}"
    missed = [(label, rc, log) for label, rc, log in results[1:] if rc != 1]
    assert not missed, "\n".join(f"{label}: pytest exit {rc}\n{log}" for label, rc, log in missed)
