"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/sprint_oracle.py (in a
temporary directory, never in the tree) and runs tests/test_oracle_pins.py
against that copy; the pins must fail.  The mistakes are the kinds a reader
could make transcribing the pages: a wrong GQA index, scale or norm, the
wrong tie-break, >= for the strict threshold, swapped blend weights, a floor
for a ceiling, a dropped term, a wrong offset, truncation for round-to-even,
a sum for a mean, a missing bias, gate scale or SwiGLU factor, a top-2
gap taken to the smallest logit, to the next distinct logit or over
probabilities.  The unmutated
copy must pass, so a failure is the mistake's, not the harness's.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "sprint_oracle.py")

MUTATIONS = {
    "gqa_mod": ("g = (h * Hkv) // Hq", "g = h % Hkv"),
    "scale_1_over_D": ("scale = 1.0 / math.sqrt(D)", "scale = 1.0 / D"),
    "norm_no_sqrt": ('return np.sqrt(np.einsum("ij,ij->i", flat, flat))',
                     'return np.einsum("ij,ij->i", flat, flat)'),
    "norm_first_head": ("flat = K.reshape(K.shape[0], -1)", "flat = K[:, 0, :]"),
    "topk_tie_high": ("order = np.lexsort((pos, -score[pos]))",
                      "order = np.lexsort((-pos, -score[pos]))"),
    "tau_ge": ("n_hi = int(np.sum(conf[s, cand] > tau))", "n_hi = int(np.sum(conf[s, cand] >= tau))"),
    "blend_swap": ("return alpha * ibar + (1.0 - alpha) * conf",
                   "return (1.0 - alpha) * ibar + alpha * conf"),
    "min_accept_floor": ("return min(m, -(-m // steps_left))", "return min(m, m // steps_left)"),
    "argmax_last": ("amax = Z.argmax(axis=1)", "amax = Z.shape[1] - 1 - Z[:, ::-1].argmax(axis=1)"),
    "attn_no_block_keys": ("if Kb is not None:", "if False:"),
    "mean_over_all_seqs": ("mu = n[a:b].sum() / L", "mu = n.sum() / len(n)"),
    "append_drop_block": ("        parts.append(blk[s])\n", "        pass\n"),
    "append_offsets": ("cu_new = cu + n_blk * np.arange(nseq + 1, dtype=np.int64)",
                       "cu_new = cu + n_blk * np.arange(1, nseq + 2, dtype=np.int64)"),
    "bf16_truncate": ("bits = ((bits + 0x7FFF + lsb) >> 16) << 16", "bits = (bits >> 16) << 16"),
    "bf16_ties_up": ("bits = ((bits + 0x7FFF + lsb) >> 16) << 16",
                     "bits = ((bits + 0x8000) >> 16) << 16"),
    "layers_sum": ("return np.mean([key_norm_importance(K, cu_len) for K in K_layers], axis=0)",
                   "return np.sum([key_norm_importance(K, cu_len) for K in K_layers], axis=0)"),
    "layers_first_only": ("return np.mean([key_norm_importance(K, cu_len) for K in K_layers], axis=0)",
                          "return key_norm_importance(K_layers[0], cu_len)"),
    "silu_drop_z": ("return z / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))"),
    "route_no_bias": ("sel_score = s + np.asarray(bias, dtype=np.float64)[None, :]", "sel_score = s"),
    "route_gate_with_bias": ("gates[t] = route_scale * s[t, ids[t]] / s[t, ids[t]].sum()",
                             "gates[t] = route_scale * sel_score[t, ids[t]] / sel_score[t, ids[t]].sum()"),
    "route_no_scale": ("gates[t] = route_scale * s[t, ids[t]] / s[t, ids[t]].sum()",
                       "gates[t] = s[t, ids[t]] / s[t, ids[t]].sum()"),
    "route_tie_high": ("order = np.lexsort((np.arange(E), -sel_score[t]))",
                       "order = np.lexsort((-np.arange(E), -sel_score[t]))"),
    "swiglu_swapped": ("return (silu(g) * u) @ np.asarray(w_down, dtype=np.float64).T",
                       "return (g * silu(u)) @ np.asarray(w_down, dtype=np.float64).T"),
    "moe_no_gate": ("y[t] += gates[t, j] * expert_ffn(", "y[t] += expert_ffn("),
    "top2_gap_max_minus_min": ("return part[:, -1] - part[:, -2]",
                               "return part[:, -1] - part[:, 0]"),
    "top2_gap_distinct_runner_up": (
        "return part[:, -1] - part[:, -2]",
        "return part[:, -1] - np.where(part[:, -2] == part[:, -1], part[:, -3], part[:, -2])"),
    "top2_gap_probabilities": (
        "Z = np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T\n    if Z.shape[1] < 2:",
        "Z = np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T\n"
        "    Z = np.exp(Z - Z.max(axis=1, keepdims=True))\n    Z /= Z.sum(axis=1, keepdims=True)\n"
        "    if Z.shape[1] < 2:"),
}


def _run_pins(source: str) -> int:
    """Exit status of the pin tests run against `source` as the oracle."""
    with tempfile.TemporaryDirectory() as tmp:
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tmp, "oracle"),
                        ignore=shutil.ignore_patterns("__pycache__"))
        with open(os.path.join(tmp, "oracle", "sprint_oracle.py"), "w") as f:
            f.write(source)
        os.makedirs(os.path.join(tmp, "tests"))
        for name in ("conftest.py", "test_oracle_pins.py"):
            shutil.copy(os.path.join(ROOT, "tests", name), os.path.join(tmp, "tests", name))
        shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))
        os.makedirs(os.path.join(tmp, "sparse_prefix_kv_amd"))
        for name in ("__init__.py", "synth.py"):
            shutil.copy(os.path.join(ROOT, "sparse_prefix_kv_amd", name),
                        os.path.join(tmp, "sparse_prefix_kv_amd", name))
        r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                            "-p", "no:cacheprovider"], cwd=tmp, capture_output=True, text=True,
                           timeout=600)
        return r.returncode


def test_every_planted_mistake_fails_a_pin():
    src = open(ORACLE).read()
    for name, (old, _) in MUTATIONS.items():
        assert src.count(old) >= 1, f"mutation {name} no longer applies"
    cases = {"unmutated": src}
    cases.update({name: src.replace(old, new) for name, (old, new) in MUTATIONS.items()})
    with ThreadPoolExecutor(max_workers=6) as ex:
        status = dict(zip(cases, ex.map(_run_pins, cases.values())))
    assert status.pop("unmutated") == 0, "the pins fail on the unmutated oracle copy"
    missed = [name for name, rc in status.items() if rc == 0]
    assert not missed, f"mistakes no pin catches: {missed}"
