"""The oracle's pins catch plausible mistakes: each case plants one in a copy of
the oracle (on the CPU, in a temporary directory) and runs the oracle's pin
tests against that copy, which must fail.

The mistakes are the kinds a hand-written implementation of the layer makes:
a dropped LoRA term or scale, gate and up swapped, a wrong sign or factor in
the SwiGLU derivative, a wrong operand in a LoRA gradient, a tie broken the
other way, a missing renormalisation, an inclusive scan, a wrong slot in the
combine. The unmutated copy must pass (so a failure means the pins saw the
mistake, not that the harness is broken).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_layer.py", "tests/test_oracle_route_permute.py",
             "tests/test_oracle_router_shared.py"]

# (name, text in oracle/moe_oracle.py, replacement)
MUTATIONS = [
    ("gate_up_lora_dropped", "h = X @ W1.T + s * (u_gu @ B1.T)", "h = X @ W1.T + 0 * (u_gu @ B1.T)"),
    ("gate_up_scale_dropped", "h = X @ W1.T + s * (u_gu @ B1.T)", "h = X @ W1.T + (u_gu @ B1.T)"),
    ("gate_up_swapped", "g, v = h[:, :I], h[:, I:]\n    a = g", "v, g = h[:, :I], h[:, I:]\n    a = g"),
    ("silu_without_gate", "a = g * _sigmoid(g) * v", "a = _sigmoid(g) * v"),
    ("down_lora_dropped", "y = a @ W2.T + s * (u_d @ B2.T)", "y = a @ W2.T"),
    ("swiglu_bwd_sign", "dg = da * v * sg * (1 + g * (1 - sg))", "dg = da * v * sg * (1 - g * (1 - sg))"),
    ("swiglu_bwd_up_factor", "dv = da * g * sg", "dv = da * sg"),
    ("dx_lora_dropped", "dx = dh @ W1 + s * (dhb @ A1)", "dx = dh @ W1"),
    ("db_d_wrong_operand", "db_d = s * (G.T @ u_d)", "db_d = s * (G.T @ u_gu)"),
    ("da_d_scale_dropped", "da_d = s * (gb.T @ a)", "da_d = gb.T @ a"),
    ("da_gu_scale_dropped", "da_gu = s * (dhb.T @ X)", "da_gu = dhb.T @ X"),
    ("db_gu_wrong_half", "db_gu = s * (dh.T @ u_gu)",
     "db_gu = s * (np.concatenate([dh[:, dh.shape[1] // 2:], dh[:, :dh.shape[1] // 2]], 1).T @ u_gu)"),
    ("tie_to_higher_index", "order = np.lexsort((idx, -logits), axis=-1)",
     "order = np.lexsort((-idx, -logits), axis=-1)"),
    ("renorm_missing", "            w = w / w.sum(axis=1, keepdims=True)", "            w = w"),
    ("sigmoid_renorm_missing", "w = sg / sg.sum(axis=1, keepdims=True)", "w = sg"),
    ("route_bwd_no_centering", "dl[rows, ids] = w * (dw - c)", "dl[rows, ids] = w * dw"),
    ("softmax_topk_bwd_no_centering", "dl = p * (dhat - c)", "dl = p * dhat"),
    ("sigmoid_bwd_missing_derivative", "dl[rows, ids] = sg * (1 - sg) * (dw - c)",
     "dl[rows, ids] = sg * (dw - c)"),
    ("inclusive_offsets", "offsets[1:] = np.cumsum(counts)", "offsets[1:] = np.cumsum(counts) - counts"),
    ("permute_unstable", 'sorted_pair = np.argsort(ids, kind="stable")',
     'sorted_pair = np.lexsort((-np.arange(ids.size), ids))'),
    ("gather_modulo", "np.asarray(x)[np.asarray(sorted_pair) // k]",
     "np.asarray(x)[np.asarray(sorted_pair) % np.asarray(x).shape[0]]"),
    ("combine_first_slot_weight", "Y += np.asarray(topk_w, dtype=dtype)[:, j:j + 1] * rows",
     "Y += np.asarray(topk_w, dtype=dtype)[:, 0:1] * rows"),
    ("combine_bwd_wrong_row", 'dw[:, j] = np.einsum("th,th->t", dY, y_perm[pos[:, j]])',
     'dw[:, j] = np.einsum("th,th->t", dY, y_perm[pos[:, 0]])'),
    ("unpermute_weighted", 'dx = combine(dx_perm, cache["inv_pos"], None, T, k, dtype)',
     'dx = combine(dx_perm, cache["inv_pos"], cache["w"], T, k, dtype)'),
    ("dw_gu_without_swiglu_derivative", 'out["dw_gu"] = dh.T @ X',
     'out["dw_gu"] = np.concatenate([da, da], axis=1).T @ X'),
    ("dw_d_scaled_by_lora_scale", 'out["dw_d"] = G.T @ a', 'out["dw_d"] = s * (G.T @ a)'),
    ("router_logits_negated", "return np.asarray(x, dtype) @ np.asarray(w_r, dtype).T",
     "return -(np.asarray(x, dtype) @ np.asarray(w_r, dtype).T)"),
    ("router_grad_dropped", 'g["dx"] = g["dx"] + router_input_grad(g["dlogits"], w_r, dtype)',
     'g["dx"] = g["dx"]'),
    ("router_grad_halved", "return np.asarray(dlogits, dtype) @ np.asarray(w_r, dtype)",
     "return np.asarray(dlogits, dtype) @ np.asarray(w_r, dtype) * 0.5"),
    ("shared_output_dropped", 'Y = Y + f["y"]', "Y = Y"),
    ("shared_dx_dropped", 'g["dx"] = g["dx"] + b["dx"]', 'g["dx"] = g["dx"]'),
    ("merge_scale_dropped", "out[name] = np.stack([W[e] + dtype(s) * (B[e] @ A[e])",
     "out[name] = np.stack([W[e] + (B[e] @ A[e])"),
    ("merge_base_dropped", "out[name] = np.stack([W[e] + dtype(s) * (B[e] @ A[e])",
     "out[name] = np.stack([dtype(s) * (B[e] @ A[e])"),
]

# Runs the pin tests with the oracle package taken from argv[1].
DRIVER = """
import sys
sys.path.insert(0, sys.argv[1])
import oracle  # the planted copy, cached before the tests put the repo on sys.path
assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__
import pytest
sys.exit(pytest.main(sys.argv[2:]))
"""


def run_pins(tmp_path, mutation):
    pkg = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg,
                    ignore=shutil.ignore_patterns("__pycache__"))
    if mutation is not None:
        old, new = mutation
        src = (pkg / "moe_oracle.py").read_text()
        assert src.count(old) == 1, f"mutation site not unique: {old!r}"
        (pkg / "moe_oracle.py").write_text(src.replace(old, new))
    args = [sys.executable, "-c", DRIVER, str(tmp_path), *PIN_TESTS, "-x", "-q",
            "-m", "not gpu", "-p", "no:cacheprovider"]
    return subprocess.run(args, cwd=ROOT, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes(tmp_path):
    r = run_pins(tmp_path, None)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, name, old, new):
    r = run_pins(tmp_path, (old, new))
    assert r.returncode == 1, f"planted mistake {name} not caught:\n{r.stdout[-1500:]}"
