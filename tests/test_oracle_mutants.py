"""Planted mistakes in the oracle must be caught by its pins.

Each case below changes one line of a copy of oracle/spot_oracle.py into a
plausible mistake (a dropped scale, a wrong inequality, an inverted
permutation, ...) and runs the pin file that should catch it against that
copy, in a subprocess.  The case passes when the pins FAIL on the mutated
oracle.  An unmutated copy must pass the same pin files (the control), and
every planted line must still be found verbatim, so the list stays in step
with the oracle's source.  Everything runs on the CPU.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "spot_oracle.py")

PINS = "tests/test_oracle_pins.py"
ES = "tests/test_oracle_early_stop.py"
TAYLOR = "tests/test_oracle_taylor.py"
MXFP4 = "tests/test_oracle_mxfp4.py"
INT4 = "tests/test_oracle_int4.py"
S2O = "tests/test_oracle_s2o_map.py"
RLA = "tests/test_oracle_rla.py"

# (name, pin file, line fragment as written in the oracle, planted mistake)
MUTANTS = [
    ("RLA feature map with the attention scale", RLA,
     "return np.exp(np.asarray(x, dtype=np.float64))",
     "return np.exp(np.asarray(x, dtype=np.float64) / np.sqrt(np.shape(x)[-1]))"),
    ("RLA rest without the causal mask", RLA,
     "rest = np.arange(hi)[None, :] <= rows[:, None]", "rest = np.ones((rows.shape[0], hi), dtype=bool)"),
    ("RLA removes only the history keys it keeps", RLA,
     "rest[r_idx, phys[lim <= r]] = False", "rest[r_idx, phys[lim < 0]] = False"),
    ("RLA normalised by the feature mass", RLA,
     "out[h, rows] = w @ v[g, :hi]",
     "out[h, rows] = (w @ v[g, :hi]) / np.maximum(w.sum(axis=1, keepdims=True), 1e-300)"),
    ("RLA decode keeps the kept blocks", RLA,
     "rest[block_rows(int(t), block, T)] = False", "rest[block_rows(int(t), block, T)] = True"),
    ("history rows through the inverse permutation", PINS,
     "phys.append(perm[g, ts])", "phys.append(np.argsort(perm[g])[ts])"),
    ("exclusive top-p crossing", PINS, "c >= top_p", "c > top_p"),
    ("recency window one block too wide", PINS,
     "return (js < n_sink) | (js > i - n_recent)", "return (js < n_sink) | (js >= i - n_recent)"),
    ("decode recency window one block too wide", PINS,
     "return (ts < n_sink) | (ts > nt - 1 - n_recent)", "return (ts < n_sink) | (ts >= nt - 1 - n_recent)"),
    ("decode sink window one block too wide", PINS,
     "return (ts < n_sink) | (ts > nt - 1 - n_recent)", "return (ts <= n_sink) | (ts > nt - 1 - n_recent)"),
    ("decode recency window one block too narrow", PINS,
     "return (ts < n_sink) | (ts > nt - 1 - n_recent)", "return (ts < n_sink) | (ts > nt - n_recent)"),
    ("history key means without the permutation", PINS,
     "kp[g, i] = k[g, perm[g, rows]].mean(axis=0)", "kp[g, i] = k[g, rows].mean(axis=0)"),
    ("query means over one head of the group", PINS,
     "qbar[g, i] = q[g * G:(g + 1) * G, rows].mean(axis=(0, 1))", "qbar[g, i] = q[g, rows].mean(axis=0)"),
    ("strict causal mask", PINS,
     "visible = lim[None, :] <= rows[:, None]", "visible = lim[None, :] < rows[:, None]"),
    ("block score without the softmax scale", PINS,
     "s[g, i, :i + 1] = sm_scale * (kb @ qbar[g, i])", "s[g, i, :i + 1] = (kb @ qbar[g, i])"),
    ("indexer ReLU after the head weight", PINS,
     "s += idx_w[h] * np.maximum(dots, 0.0)", "s += np.maximum(idx_w[h] * dots, 0.0)"),
    ("key importance normalised by the heads only", PINS,
     "imp[g] /= G * rows.shape[0]", "imp[g] /= G"),
    ("keys sorted by ascending importance", PINS,
     "ts[np.lexsort((ts, -imp[g, ts]))]", "ts[np.lexsort((ts, imp[g, ts]))]"),
    ("decode logits without the softmax scale", PINS,
     "logits = sm_scale * (ks @ q[h])", "logits = (ks @ q[h])"),
    ("early stop against the mass before the block", ES,
     "acc = e_own.sum(axis=1)[:, None] + np.cumsum(gain, axis=1)\n                for ri, r in enumerate(rows):",
     "acc = e_own.sum(axis=1)[:, None] + np.cumsum(gain, axis=1) - gain\n                for ri, r in enumerate(rows):"),
    ("early stop drops the triggering block", ES,
     "n = int(below[0]) + 1 if below.size else n_h", "n = int(below[0]) if below.size else n_h"),
    ("Taylor term without the one half", TAYLOR,
     "np.log(1.0 + 0.5 * (vb @ (x * x)))", "np.log(1.0 + (vb @ (x * x)))"),
    ("Taylor term linear in the query", TAYLOR,
     "np.log(1.0 + 0.5 * (vb @ (x * x)))", "np.log(1.0 + 0.5 * (vb @ x))"),
    ("segment query mean over one head of the group", S2O,
     "rep_q[g, sg] = q[g * G:(g + 1) * G, sg * segment:min((sg + 1) * segment, L)].mean(axis=(0, 1))",
     "rep_q[g, sg] = q[g * G, sg * segment:min((sg + 1) * segment, L)].mean(axis=0)"),
    ("history map in ascending score order", S2O,
     "hmap[g, sg, :n] = ts[np.lexsort((ts, -c))]", "hmap[g, sg, :n] = ts[np.lexsort((ts, c))]"),
    ("history map ties by descending position", S2O,
     "hmap[g, sg, :n] = ts[np.lexsort((ts, -c))]", "hmap[g, sg, :n] = ts[np.lexsort((-ts, -c))]"),
    ("INT4 scale from max / 8", INT4,
     "scales = _round_bf16(np.abs(g).max(axis=1) / INT4_MAX)",
     "scales = _round_bf16(np.abs(g).max(axis=1) / (INT4_MAX + 1))"),
    ("INT4 scale not rounded to bf16", INT4,
     "scales = _round_bf16(np.abs(g).max(axis=1) / INT4_MAX)", "scales = np.abs(g).max(axis=1) / INT4_MAX"),
    ("INT4 ties away from zero", INT4,
     "codes = np.clip(np.rint(g / safe[:, None]), -INT4_MAX, INT4_MAX)",
     "codes = np.clip(np.trunc(g / safe[:, None] + np.copysign(0.5, g)), -INT4_MAX, INT4_MAX)"),
    ("INT4 ties upward", INT4,
     "codes = np.clip(np.rint(g / safe[:, None]), -INT4_MAX, INT4_MAX)",
     "codes = np.clip(np.floor(g / safe[:, None] + 0.5), -INT4_MAX, INT4_MAX)"),
    ("MXFP4 scale one power of two too large", MXFP4,
     "np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)", "np.clip(ex.astype(np.int64) - 1 - 1, -127, 127)"),
]


def _copy_tree(dst):
    """The oracle, the tests and the package's Python modules (no built library)."""
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(dst, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    pkg = os.path.join(dst, "block_sparse_attention_amd")
    os.makedirs(pkg)
    src = os.path.join(ROOT, "block_sparse_attention_amd")
    for f in os.listdir(src):
        if f.endswith(".py"):
            shutil.copy(os.path.join(src, f), pkg)


def _run_pins(tree, pin_file):
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", pin_file, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=tree, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, (r.stdout + r.stderr).strip().splitlines()[-1:]


def test_planted_oracle_mistakes_are_caught(tmp_path):
    source = open(ORACLE).read()
    for name, _, old, _ in MUTANTS:
        assert source.count(old) == 1, f"{name}: the planted line is no longer in the oracle: {old!r}"

    def job(k):
        tree = str(tmp_path / f"t{k}")
        _copy_tree(tree)
        if k < 0:   # control: every pin file on the unmutated copy
            return [_run_pins(tree, f) for f in sorted({m[1] for m in MUTANTS})]
        name, pin_file, old, new = MUTANTS[k]
        with open(os.path.join(tree, "oracle", "spot_oracle.py"), "w") as fh:
            fh.write(source.replace(old, new))
        return _run_pins(tree, pin_file)

    with ThreadPoolExecutor(max_workers=4) as ex:
        control = ex.submit(job, -1)
        results = list(ex.map(job, range(len(MUTANTS))))
    for code, tail in control.result():
        assert code == 0, f"pins fail on the unmutated copy: {tail}"
    # exit status 1: tests ran and failed (2 and above would be a broken run, not a catch)
    missed = [(m[0], code, tail) for m, (code, tail) in zip(MUTANTS, results) if code != 1]
    assert not missed, f"planted mistakes not caught by the pins: {missed}"
