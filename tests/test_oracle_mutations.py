"""The oracle's pins catch planted mistakes (CPU only).

Each case copies the oracle, the input generators and the pin tests into a
temporary tree, plants one plausible mistake in the oracle's source there (a
swapped nibble order, a wrong sign, a dropped term, a broken tie rule, an
unstable permutation, a shifted combine slot, ...), and runs the pin tests of
that tree in a child process: every planted mistake must make a pin fail.
The repository's own files are never modified.  The unmutated copy must pass,
so that a failure means the mistake was caught and not that the copy is broken.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "moe_oracle.py")

# (name, text in oracle/moe_oracle.py, replacement)
MUTATIONS = [
    ("q4_nibble_order",
     "u[..., 0::2] = c & 0x0F\n    u[..., 1::2] = c >> 4",
     "u[..., 0::2] = c >> 4\n    u[..., 1::2] = c & 0x0F"),
    ("q4_offset_sign", "* (u - 8).astype(np.float64)", "* (8 - u).astype(np.float64)"),
    ("q2_crumb_order", "u[..., i::4] = (c >> (2 * i)) & 3", "u[..., (3 - i)::4] = (c >> (2 * i)) & 3"),
    ("router_bias_dropped", "l = l + np.asarray(b, np.float64)[None, :]", "l = l"),
    ("ties_to_higher_id",
     'order = np.argsort(-l, axis=-1, kind="stable")',
     'order = l.shape[-1] - 1 - np.argsort(-l[..., ::-1], axis=-1, kind="stable")'),
    ("weights_not_renormalised",
     "return z / z.sum(axis=-1, keepdims=True)",
     "return z / np.exp(np.asarray(logits, np.float64) - sel[..., :1]).sum(axis=-1, keepdims=True)"),
    ("permutation_reversed_within_expert",
     'sorted_pairs = np.argsort(flat, kind="stable").astype(np.int64)',
     "sorted_pairs = np.lexsort((-np.arange(flat.size), flat)).astype(np.int64)"),
    ("silu_sign", "return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    ("gate_and_up_swapped", "v = silu(g) * u", "v = silu(u) * g"),
    ("h_not_rounded", "h = round_act(v, act)", "h = v"),
    ("shared_expert_dropped", "shared_out = shared_out + sj", "shared_out = shared_out"),
    ("q3_high_bit_position",
     "high[..., i] = (g[..., 8 + i // 8] >> (i % 8)) & 1",
     "high[..., i] = (g[..., 8 + i % 4] >> (i // 4)) & 1"),
    ("q3_offset", "* (u - 4).astype(np.float64)", "* (u - 3).astype(np.float64)"),
    ("q3_low_and_high_swapped", "u = low + 4 * high", "u = 2 * low + high"),
    ("bf16_ties_away_from_zero",
     "keep = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16",
     "keep = ((bits + 0x8000) >> 16) << 16"),
    ("bf16_single_rounding_from_float64",
     "    return keep.astype(np.uint32).view(np.float32).astype(np.float64)",
     "    v = np.asarray(a, np.float64)\n"
     "    ulp = 2.0 ** (np.floor(np.log2(np.where(v == 0, 1.0, np.abs(v)))) - 7)\n"
     "    return np.round(v / ulp) * ulp"),
    ("residual_single_rounding_from_float64",
     "return round_bf16(round_f32(np.asarray(x, np.float64) + np.asarray(y, np.float64)))",
     "v = np.asarray(x, np.float64) + np.asarray(y, np.float64)\n"
     "    ulp = 2.0 ** (np.floor(np.log2(np.where(v == 0, 1.0, np.abs(v)))) - 7)\n"
     "    return np.round(v / ulp) * ulp"),
    ("combine_slot_shifted",
     "y = y + w[:, kk:kk + 1] * o_tk[:, kk, :]",
     "y = y + w[:, kk:kk + 1] * o_tk[:, (kk + 1) % o_tk.shape[1], :]"),
]

# the random brute-force sweep (200+ shapes) is the slow pin; the others are
# enough to catch every mistake above
PIN_SELECTION = "not random_tiny_shapes"


def make_tree(dst, mutation=None):
    for pkg in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, pkg), os.path.join(dst, pkg),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    for name in ("__init__.py", "conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), os.path.join(dst, "tests", name))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    if mutation is not None:
        old, new = mutation
        path = os.path.join(dst, "oracle", "moe_oracle.py")
        src = open(path).read()
        assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
        open(path, "w").write(src.replace(old, new))


def run_pins(tree):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q", "-p",
                        "no:cacheprovider", "-k", PIN_SELECTION], cwd=tree, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_unmutated_copy_passes(tmp_path):
    make_tree(str(tmp_path))
    rc, out = run_pins(str(tmp_path))
    assert rc == 0, out


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    assert open(ORACLE).read().count(old) == 1, f"{name}: anchor missing from the oracle"
    make_tree(str(tmp_path), (old, new))
    rc, out = run_pins(str(tmp_path))
    assert rc != 0, f"{name}: no pin failed\n{out}"
