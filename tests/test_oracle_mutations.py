"""Mutation check of the oracle's pins (CPU only).

A copy of ``oracle/`` is taken into a temporary directory, one plausible
slip is planted in it (a flipped sign, an off-by-one mask bound, a dropped
term, a wrong head map or index, a transposed operand), and the pin suites
are run against the copy in a child process.  Each planted slip must make at
least one pin fail: that is what shows the pins constrain the oracle, rather
than restate it.  The real oracle is never modified.
"""

import os
import shutil
import subprocess
import sys
import concurrent.futures

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = [os.path.join(ROOT, "tests", n) for n in
        ("test_oracle_pins.py", "test_oracle_golden.py", "test_oracle_kvcache_pins.py")]

# (file under oracle/, exact text, replacement, what the slip is)
MUTATIONS = [
    ("attention.py", "u = t - slope * dist", "u = t + slope * dist",
     "ALiBi bias with the wrong sign"),
    ("attention.py", "dist = np.abs(rows[:, None] + (Sk - Sq) - cols[None, :])",
     "dist = np.abs(rows[:, None] - cols[None, :])",
     "ALiBi distance without the bottom-right offset"),
    ("attention.py", "else float(a[b, h])", "else float(a[h % a.shape[0], b % a.shape[1]])",
     "per-batch ALiBi table read transposed"),
    ("attention.py", "else float(a[b, h])", "else float(a.ravel()[h])",
     "per-batch ALiBi table read as its first row"),
    ("attention.py", "return h // (Hq // Hkv)", "return h % Hkv",
     "GQA head map h % Hkv instead of repeat_interleave"),
    ("attention.py", "t = softcap * np.tanh(s / softcap)", "t = softcap * np.tanh(s)",
     "softcap without the division by the cap"),
    ("attention.py", "ok &= j <= i + delta\n", "ok &= j <= i\n",
     "causal mask aligned top-left"),
    ("attention.py", "ok &= j >= i + delta - left", "ok &= j > i + delta - left",
     "left window bound exclusive"),
    ("attention.py", "ok &= j <= i + delta + right", "ok &= j < i + delta + right",
     "right window bound exclusive"),
    ("attention.py", "ok &= dq[:, None] == dk[None, :]", "ok &= dq[:, None] >= dk[None, :]",
     "document test as an ordering"),
    ("attention.py", "ok &= j < kv_len", "ok &= j <= kv_len",
     "cache length bound off by one"),
    ("attention.py", "lse = np.where(has, m + np.log(safe), _NEG_INF)",
     "lse = np.where(has, np.log(safe), _NEG_INF)",
     "log-sum-exp without the row maximum"),
    ("attention.py", "dU = P * (dP - delta[:, None])", "dU = P * dP",
     "backward without Delta"),
    ("attention.py", "dq[b, rows, h, :] = scale * (dS @ k_cols)",
     "dq[b, rows, h, :] = (dS @ k_cols)", "dQ without the softmax scale"),
    ("attention.py", "dk[b, lo:hi, g, :] += scale * (dS.T @ q_rows)",
     "dk[b, lo:hi, g, :] += (dS.T @ q_rows)", "dK without the softmax scale"),
    ("attention.py", "dv[b, lo:hi, g, :] += P.T @ do_rows", "dv[b, lo:hi, g, :] = P.T @ do_rows",
     "dV of a kv head not summed over its query heads"),
    ("attention.py", "dS = dU * (1.0 - np.tanh(s / softcap) ** 2)", "dS = dU",
     "softcap derivative dropped"),
    ("attention.py", "w = np.where(has, np.exp(np.where(has, lse_parts, 0.0) - m_safe), 0.0)",
     "w = np.where(has, np.exp(m_safe - np.where(has, lse_parts, 0.0)), 0.0)",
     "split-K combine weights inverted"),
    ("attention.py", "elif inside and tile.all():", "elif tile.all():",
     "a tile crossing the sequence end classified FULL"),
    ("attention.py", "hits = np.nonzero(cls[b, :, kb] == c)[0]",
     "hits = np.nonzero(cls[b, kb % nQ] == c)[0]", "transposed block lists read by row"),
    ("kvcache.py", "r = L + t\n", "r = L + t - 1\n", "append one row early"),
    ("kvcache.py", "out[r] = cache[int(block_table[b, r // page_size]), r % page_size]",
     "out[r] = cache[int(block_table[b, r % block_table.shape[1]]), r % page_size]",
     "paged cache page index taken modulo"),
]


def _run_pins(tmp, mutation):
    fname, old, new, what = mutation
    dst = os.path.join(tmp, "m%d" % MUTATIONS.index(mutation))
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    path = os.path.join(dst, "oracle", fname)
    src = open(path).read()
    assert src.count(old) == 1, "mutation target not found exactly once: %r" % old
    open(path, "w").write(src.replace(old, new))
    env = dict(os.environ)
    # the mutated copy comes first; the package under test (inputs) from ROOT
    env["PYTHONPATH"] = os.pathsep.join([dst, ROOT])
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "--rootdir", ROOT, *PINS], cwd=dst, env=env,
                       capture_output=True, text=True, timeout=600)
    imported = "oracle" in r.stdout  # traceback paths name the package
    return what, r.returncode, r.stdout[-1500:], imported


def test_every_planted_oracle_slip_fails_a_pin(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(4) as ex:
        results = list(ex.map(lambda m: _run_pins(str(tmp_path), m), MUTATIONS))
    survivors = [(what, out) for what, rc, out, _ in results if rc == 0]
    assert not survivors, "slips no pin caught:\n" + "\n".join(
        "%s\n%s" % (w, o) for w, o in survivors)
    # a failure must come from the tests, not from a broken harness
    for what, rc, out, _ in results:
        assert rc == 1, "%s: pytest exit %d (expected test failures)\n%s" % (what, rc, out)


def test_unmutated_copy_passes(tmp_path):
    """The harness itself: an unchanged copy of the oracle passes every pin
    (so the failures above come from the planted slips)."""
    dst = os.path.join(str(tmp_path), "clean")
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([dst, ROOT])
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "--rootdir", ROOT, *PINS,
                        "-k", "not every_planted"], cwd=dst, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    # the child really imported the copy
    probe = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.__file__)"],
                           cwd=dst, env=env, capture_output=True, text=True)
    assert probe.stdout.strip().startswith(dst), probe.stdout
