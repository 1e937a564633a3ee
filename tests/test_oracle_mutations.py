"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's source (a
dropped term, a wrong sign, a wrong constant, swapped indices, a transposed
operand), loads that copy as a separate module, and checks that at least one
pin of ``test_oracle.py`` fails against it with an assertion.  A pin that
crashes (a TypeError, a shape error) does not count as a catch, and a guard
case runs every pin through the same harness against the unmutated oracle,
where all of them must pass.  The real oracle is untouched.
"""
import importlib.util
import inspect
import os
import sys
import types

import pytest

import tests.test_oracle as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "woq_oracle.py")

MUTATIONS = {
    "rint_to_floor": ("q = np.rint(np.divide(g, S32, dtype=np.float32))",
                      "q = np.floor(np.divide(g, S32, dtype=np.float32))"),
    "qmax_off_by_one": ("qmax = np.float32(half - 1)", "qmax = np.float32(half)"),
    "asym_range_levels": ("qu = np.float32(2 ** bits - 1)", "qu = np.float32(2 ** bits)"),
    "zero_point_sign": ("Zf = np.rint(np.divide(-mn, S32, dtype=np.float32))",
                        "Zf = np.rint(np.divide(mn, S32, dtype=np.float32))"),
    "zero_point_dropped": ("u = np.clip(q + Zf[:, :, None], 0, qu)", "u = np.clip(q, 0, qu)"),
    "sym_bias_dropped": ("u = (q + half).astype(np.uint8)", "u = (q + half - 1).astype(np.uint8)"),
    "zero_range_rule_dropped": ("r = np.where(r == 0, np.float32(1), r)", "r = r"),
    "pack_nibble_order": ("<< np.uint32(16 * h + 4 * t)\n", "<< np.uint32(8 * h + 4 * t)\n"),
    "pack3_pair_field": ("words[:, j, t // 5] |= u << np.uint32(16 * h + 3 * (t % 5))",
                         "words[:, j, t // 5] |= u << np.uint32(16 * h + 3 * (t % 4))"),
    "pack3_last_pair_bits": ("words[:, j, b] |= ((u >> np.uint32(b)) & 1) << np.uint32(16 * h + 15)",
                             "words[:, j, 2 - b] |= ((u >> np.uint32(b)) & 1) << np.uint32(16 * h + 15)"),
    "dequant_zero_dropped": ("return (q.codes.astype(np.float64) - Z) * S",
                             "return q.codes.astype(np.float64) * S"),
    "gemm_transposed": ("return X64 @ np.asarray(w_hat, dtype=np.float64).T",
                        "return (np.asarray(w_hat, dtype=np.float64) @ X64.T).T[:, ::-1]"),
    "gemm_scale_multiplied": ("X64 = X64 / np.asarray(act_scale", "X64 = X64 * np.asarray(act_scale"),
    "fold_divides": ("return np.multiply(w, s[None, :], dtype=np.float32)",
                     "return np.divide(w, s[None, :], dtype=np.float32)"),
    "awq_activation_not_divided": ("    y_q = gemm(X64, dequantize(q), s)\n", "    y_q = gemm(X64, dequantize(q), None)\n"),
    "awq_mean_not_absolute": ("return np.abs(np.asarray(X64, dtype=np.float64)).mean(axis=0)",
                              "return np.asarray(X64, dtype=np.float64).mean(axis=0)"),
    "awq_argmax": ("best = int(np.argmin(losses))", "best = int(np.argmax(losses))"),
    "awq_loss_not_squared": ("return float(np.sum((y_ref - y_q) ** 2))", "return float(np.sum(np.abs(y_ref - y_q)))"),
    "awq_alpha_grid_inclusive": ("return np.arange(n_grid, dtype=np.float64) / n_grid",
                                 "return np.arange(n_grid, dtype=np.float64) / (n_grid - 1)"),
    "gptq_error_not_scaled": ("err = (Wf[:, k] - w_hat) / U[k, k]", "err = (Wf[:, k] - w_hat)"),
    "gptq_update_sign": ("Wf[:, k + 1:] -= np.outer(err, U[k, k + 1:])", "Wf[:, k + 1:] += np.outer(err, U[k, k + 1:])"),
    "gptq_update_column_of_factor": ("Wf[:, k + 1:] -= np.outer(err, U[k, k + 1:])",
                                     "Wf[:, k + 1:] -= np.outer(err, U[k + 1:, k])"),
    "gptq_factor_not_transposed": ("U = np.linalg.cholesky(np.linalg.inv(H)).T", "U = np.linalg.cholesky(np.linalg.inv(H))"),
    "gptq_factor_of_hessian": ("U = np.linalg.cholesky(np.linalg.inv(H)).T", "U = np.linalg.cholesky(H).T"),
    "gptq_hessian_not_doubled": ("H = 2.0 * (X64.T @ X64)", "H = X64.T @ X64"),
    "gptq_dead_not_zeroed": ("Wf[:, dead] = 0.0", "Wf[:, dead] = Wf[:, dead]"),
    "gptq_params_from_original_weights": ("qg = quantize(Wf[:, k:k + group_size].astype(np.float32)",
                                          "qg = quantize(W[:, k:k + group_size].astype(np.float32)"),
    "scale_not_fp16": ("S = np.divide(a, qmax, dtype=np.float32).astype(np.float16)",
                       "S = np.divide(a, qmax, dtype=np.float32).astype(np.float16) * np.float16(1.0009765625)"),
    "rel_l2_squared": ("return float(num / den) if den > 0 else float(num)",
                       "return float((num / den) ** 2) if den > 0 else float(num)"),
    "reconstruction_loss_not_squared": ("return float(np.sum((X64 @ D.T) ** 2))",
                                        "return float(np.sum(np.abs(X64 @ D.T)))"),
    "bf16_bits_read_as_values": ("        return bf16_bits_to_f64(X)\n",
                                 "        return np.asarray(X).astype(np.float64)\n"),
    "awq_floor_1e-2": ("AWQ_SCALE_FLOOR = 1e-4", "AWQ_SCALE_FLOOR = 1e-2"),
    "gptq_error_not_propagated": ("Wf[:, k + 1:] -= np.outer(err, U[k, k + 1:])", "pass"),
}


def _mutant(name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found"
    src = src.replace(old, new)
    modname = f"woq_oracle_mutant_{name}"
    mod = types.ModuleType(modname)
    sys.modules[modname] = mod  # dataclasses look the module up by name
    try:
        exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    finally:
        del sys.modules[modname]
    return mod


def _pin_calls():
    """Every pin in test_oracle.py with each of its parameter combinations.
    A parametrize mark may name several arguments ("bits,asym,G"), whose
    values are then tuples."""
    calls = []
    for fname, fn in inspect.getmembers(pins, inspect.isfunction):
        if not fname.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        combos = [{}]
        for m in marks:
            if m.name != "parametrize":
                continue
            argnames, values = m.args[0], m.args[1]
            names = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else list(argnames)
            rows = [v if len(names) > 1 else (v,) for v in values]
            assert all(len(r) == len(names) for r in rows), fname
            combos = [dict(c, **dict(zip(names, r))) for c in combos for r in rows]
        assert set(inspect.signature(fn).parameters) == set(combos[0]), fname
        for c in combos:
            calls.append((fname, fn, c))
    return calls


def _run_pins():
    """(caught, crashed): pins that failed with an assertion, and pins that
    raised anything else."""
    caught, crashed = [], []
    for fname, fn, kwargs in _pin_calls():
        try:
            fn(**kwargs)
        except AssertionError:
            caught.append(fname)
        except Exception as e:  # noqa: BLE001 - reported, never counted as a catch
            crashed.append(f"{fname}: {type(e).__name__}: {e}")
    return caught, crashed


def test_every_pin_passes_on_the_unmutated_oracle_through_the_harness():
    caught, crashed = _run_pins()
    assert not caught and not crashed, (caught, crashed)
    assert len(_pin_calls()) >= 70


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    old, new = MUTATIONS[name]
    mutant = _mutant(name, old, new)
    monkeypatch.setattr(pins, "O", mutant)
    caught, crashed = _run_pins()
    assert caught, f"no pin caught mutation {name} with an assertion (crashes: {crashed})"
