"""The oracle's pins catch plausible mistakes (no GPU).

Each case plants one mistake in a copy of oracle/ under a temporary directory
and runs the pin files against that copy in a child process; the pins must fail.
A control case runs them against an unchanged copy and checks that the copy is
what the child imported.  Nothing here touches the repository's own oracle.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
PINS = [os.path.join(TESTS, f) for f in
        ("test_oracle_exact.py", "test_oracle_float.py", "test_oracle_history.py")]

# (name, file under oracle/, text, replacement)
MUTATIONS = [
    # eq. (4): the correction's sign, the decay, the state o is read from, the outer product
    ("flipped_sign", "gdn.py", "delta = beta[..., None] * (v - alpha[..., None] * Pk)",
     "delta = beta[..., None] * (v + alpha[..., None] * Pk)"),
    ("dropped_decay", "gdn.py", "S = alpha[..., None, None] * P + delta[..., :, None] * k[..., None, :]",
     "S = P + delta[..., :, None] * k[..., None, :]"),
    ("wrong_state_read", "gdn.py", "o = (S @ q[..., None])[..., 0]", "o = (P @ q[..., None])[..., 0]"),
    ("transposed_outer", "gdn.py", "S = alpha[..., None, None] * P + delta[..., :, None] * k[..., None, :]",
     "S = alpha[..., None, None] * P + k[..., :, None] * delta[..., None, :]"),
    # eq. (3) in the prefill: the decay inside the correction
    ("prefill_correction", "gdn.py", "corr = beta[..., None] * (v - alpha[..., None] * Sk)",
     "corr = beta[..., None] * (v - Sk)"),
    # eq. (9): the child's row not gathered from its parent's
    ("ancestry_not_gathered", "beam.py", "out[:, :t] = anc[parent, :t]",
     "out[:, :t] = anc[:parent.shape[0], :t]"),
    # the canonical order among equal scores
    ("tie_break_reversed", "beam.py", "order = np.lexsort((idx, -flat))[:K]",
     "order = np.lexsort((-idx, -flat))[:K]"),
    # scoring: log-softmax dropped, one head only
    ("log_softmax_dropped", "beam.py", "return cum[:, None] + log_softmax_rows(logits)",
     "return cum[:, None] + logits"),
    ("one_head_only", "beam.py", "z = np.sum(o, axis=0)", "z = o[0]"),
    # FullState: the children do not take their parents' states
    ("no_copy_on_reorder", "beam.py", "self.parent_states = self.child_states[:, parent]",
     "self.parent_states = self.child_states[:, :parent.shape[0]]"),
    # SID prefixes not gathered through the parents
    ("tokens_not_gathered", "beam.py", "tok[:, :t] = self.tokens[parent, :t]",
     "tok[:, :t] = self.tokens[:parent.shape[0], :t]"),
    # forced mode: the wrong candidate's score, or the step score without the prefix's
    ("forced_cum_wrong_token", "beam.py", "cum_next = score[fp, ft]", "cum_next = score[fp, ft[::-1]]"),
    ("forced_cum_not_cumulative", "beam.py", "cum_next = score[fp, ft]",
     "cum_next = score[fp, ft] - self.cum[fp]"),
    # grouped value heads: value head h on key head h % H_K instead of h // g
    ("group_tile_step", "run.py", 'return (np.repeat(x["q"].value.astype(np.float64), g, axis=0),',
     'return (np.tile(x["q"].value.astype(np.float64), (g, 1, 1)),'),
    ("group_tile_prefill", "run.py", 'k = np.repeat(p["k"].astype(np.float64), wl.group, axis=1)',
     'k = np.tile(p["k"].astype(np.float64), (1, wl.group, 1))'),
]


def _copy(tmp_path, mutation=None):
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("__pycache__"))
    if mutation is not None:
        _, fname, old, new = mutation
        f = dst / fname
        s = f.read_text()
        assert s.count(old) >= 1, f"mutation text not found in oracle/{fname}: {old}"
        f.write_text(s.replace(old, new, 1))
    return tmp_path


def _run_pins(tmp_path):
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]),
               PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS],
                          cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)


def test_unchanged_copy_passes_and_is_imported(tmp_path):
    base = _copy(tmp_path)
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(base), ROOT]))
    where = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.__file__)"],
                           cwd=str(base), env=env, capture_output=True, text=True, timeout=120)
    assert where.returncode == 0, where.stderr
    assert where.stdout.strip().startswith(str(base)), where.stdout
    r = _run_pins(base)
    assert r.returncode == 0, r.stdout[-3000:]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, mutation):
    r = _run_pins(_copy(tmp_path, mutation))
    assert r.returncode == 1, f"{mutation[0]}: the pins did not fail\n{r.stdout[-2000:]}"
