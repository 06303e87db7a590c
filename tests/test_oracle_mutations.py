"""Mutation tests: plant a plausible mistake in the oracle's source, show a pin catches it.

Each mutant is the oracle module's source with one textual change (a dropped
term, a flipped sign, a transposed operand, a wrong reduction), executed as a
fresh module inside the ``oracle`` package and swapped in for the duration of
one pin.  CPU only.
"""
import inspect
import sys
import types

import pytest

import oracle

# the package re-exports functions named like their modules (oracle.prepare is the
# function), so take the modules themselves from sys.modules
GPTQ_MOD = sys.modules["oracle.gptq"]
HESS_MOD = sys.modules["oracle.hessian"]
PREP_MOD = sys.modules["oracle.prepare"]
QUANT_MOD = sys.modules["oracle.quantizer"]
DEQ_MOD = sys.modules["oracle.dequant"]
STACK_MOD = sys.modules["oracle.stack"]
AWQ_MOD = sys.modules["oracle.awq"]

import test_oracle_gptq as tg
import test_oracle_hessian_prepare as th
import test_oracle_quantizer as tq
import test_oracle_dequant as td
import test_oracle_stack as tst
import test_oracle_awq as tawq
import test_oracle_exact as tex


def _mutant(mod, old, new):
    src = inspect.getsource(mod)
    assert src.count(old) >= 1, old
    src = src.replace(old, new)
    m = types.ModuleType(mod.__name__ + "_mutant")
    m.__package__ = "oracle"
    sys.modules[m.__name__] = m  # dataclasses resolve their module through sys.modules
    try:
        exec(compile(src, m.__name__, "exec"), m.__dict__)
    finally:
        del sys.modules[m.__name__]
    return m


MUTANTS = [
    # (module, old text, new text, names to swap into ``oracle``, pin to run)
    (GPTQ_MOD, "W1[:, j + 1:] -= np.outer(e, U[c, c + 1:i1])",
     "W1[:, j + 1:] += np.outer(e, U[c, c + 1:i1])", ["gptq_quantize"],
     lambda gd: tg.test_cholesky_route_equals_literal_obs_route()),
    (GPTQ_MOD, "Wp[:, i1:] -= E @ U[i:i1, i1:]",
     "Wp[:, i1:] -= 0.0 * (E @ U[i:i1, i1:])", ["gptq_quantize"],
     lambda gd: tg.test_block_size_invariance()),
    (GPTQ_MOD, "W1[:, j + 1:] -= np.outer(e, U[c, c + 1:i1])",
     "W1[:, j + 1:] -= np.outer(e, U[c + 1:i1, c])", ["gptq_quantize"],
     lambda gd: tg.test_cholesky_route_equals_literal_obs_route()),
    (GPTQ_MOD, "e = (w - dequantize(q, scale, zero)) / U[c, c]",
     "e = (w - dequantize(q, scale, zero)) * U[c, c]", ["gptq_quantize"],
     lambda gd: tg.test_cholesky_route_equals_literal_obs_route()),
    (GPTQ_MOD, "cur = W1[:, j:j + glen] if G <= B else Wp[:, c:c + glen]",
     "cur = W[:, perm][:, c:c + glen]", ["gptq_quantize"],
     lambda gd: tg.test_cholesky_route_equals_literal_obs_route()),
    (QUANT_MOD, "zero = np.rint(r(r(-xmin * maxq) / span))",
     "zero = np.rint(r(r(xmin * maxq) / span))", ["group_params"],
     lambda gd: tq.test_codes_and_zero_in_range(4)),
    (QUANT_MOD, "scale = r(span / maxq)", "scale = r(span / (maxq + 1.0))",
     ["group_params"], lambda gd: tq.test_worked_example_minmax_int8(gd)),
    # the fp64 decision mode silently rounding to fp32 after all
    (QUANT_MOD, "return lambda x: np.asarray(x, dtype=np.float64)", "return f32",
     ["group_params"], lambda gd: tex.test_worked_example_exact(gd)),
    (QUANT_MOD, "return np.clip(np.rint(pre_round_value(w, scale, exact)) + zero, 0.0, maxq)",
     "return np.clip(np.floor(pre_round_value(w, scale, exact)) + zero, 0.0, maxq)",
     ["quantize_codes"], lambda gd: tex.test_exact_rtn_is_the_nearest_grid_point()),
    (PREP_MOD, "lam = float(perc_damp) * float(np.mean(np.diag(H)))",
     "lam = float(perc_damp) * float(np.sum(np.diag(H)))", ["prepare"],
     lambda gd: th.test_damping_closed_form_on_diagonal_S()),
    (PREP_MOD, "U = sla.cholesky(Hinv, lower=False)",
     "U = sla.cholesky(Hinv, lower=True)", ["prepare"],
     lambda gd: th.test_prepare_factor_properties()),
    (HESS_MOD, "S += X64.T @ X64", "S += X64.T @ X64 - np.diag(np.diag(X64.T @ X64)) * 0.5",
     ["hessian_S"], lambda gd: th.test_hessian_term_by_term()),
    (DEQ_MOD, "return s * (q - z)", "return s * (q + z)", ["dequant_matmul"],
     lambda gd: td.test_codes_at_zero_point_give_zero()),
    (DEQ_MOD, "return np.asarray(X, dtype=np.float64) @ Wq.T",
     "return np.asarray(X, dtype=np.float64) @ Wq[:, ::-1].T", ["dequant_matmul"],
     lambda gd: td.test_dequant_matmul_brute_force(4)),
    (DEQ_MOD, "s = np.asarray(scales, dtype=np.float64)[:, g]",
     "s = np.asarray(scales, dtype=np.float64)[:, np.sort(g)]", ["dequant_matmul"],
     lambda gd: td.test_dequant_matmul_brute_force(3)),
    (STACK_MOD, "h = to_bf16(silu(x @ gate.Wq.T) * (x @ up.Wq.T))",
     "h = to_bf16(silu(x @ np.asarray(Wg, np.float64).T) * (x @ up.Wq.T))", ["stack"],
     lambda gd: tst.test_hessians_come_from_the_quantized_network(False)),
    (STACK_MOD, "x_next = to_bf16(x + h @ down.Wq.T)", "x_next = to_bf16(h @ down.Wq.T)",
     ["stack"], lambda gd: tst.test_zero_weights_pass_the_input_through()),
    (STACK_MOD, "return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)",
     "return np.ldexp(np.rint(np.ldexp(m, 9)), e - 9)", ["stack"],
     lambda gd: tst.test_to_bf16_hand_values()),
    (AWQ_MOD, "        q, sc, z = quantize_groups(W * s, bits, G, sym)\n        D = dequant_groups(q, sc, z, G) / s - W",
     "        q, sc, z = quantize_groups(W / s, bits, G, sym)\n        D = dequant_groups(q, sc, z, G) * s - W",
     ["awq"], lambda gd: tawq.test_alpha_search_against_brute_force()),
    (AWQ_MOD, "D = dequant_groups(q, sc, z, G) / s - W", "D = dequant_groups(q, sc, z, G) - W",
     ["awq"], lambda gd: tawq.test_rescaling_preserves_the_output_when_nothing_is_rounded()),
    (AWQ_MOD, "best = int(np.argmin(losses))", "best = int(np.argmax(losses))", ["awq"],
     lambda gd: tawq.test_alpha_search_against_brute_force()),
    # awq_clip's group error without the 1/s rescaling of the inputs' second moments
    (AWQ_MOD, "Sp = S / np.outer(s, s)", "Sp = S", ["awq"],
     lambda gd: tawq.test_clip_group_error_over_tokens_with_rescaled_inputs()),
    # clip candidates that clamp the values instead of the range
    (AWQ_MOD, "        scale, zero = group_params(basis, bits, sym)\n        scales[:, k], zeros[:, k] = scale, zero\n        codes[:, g0:g1] = quantize_codes(v, scale[:, None], zero[:, None], bits)",
     "        scale, zero = group_params(v, bits, sym)\n        scales[:, k], zeros[:, k] = scale, zero\n        codes[:, g0:g1] = quantize_codes(basis, scale[:, None], zero[:, None], bits)",
     ["awq"], lambda gd: tawq.test_clip_parameters_come_from_the_clamped_range()),
]


@pytest.mark.parametrize("idx", range(len(MUTANTS)))
def test_pins_catch_planted_mistake(idx, monkeypatch, golden_dir):
    mod, old, new, names, pin = MUTANTS[idx]
    m = _mutant(mod, old, new)
    if mod is AWQ_MOD:
        monkeypatch.setattr(tawq, "awq", m)
        names = []
    if mod is STACK_MOD:
        # the stack pins call the module's functions by name and through oracle.stack
        monkeypatch.setattr(oracle, "stack", m)
        for nm in ("quantize_stack", "float_stack", "silu", "to_bf16"):
            monkeypatch.setattr(tst, nm, getattr(m, nm))
        names = []
    for nm in names:
        monkeypatch.setattr(oracle, nm, getattr(m, nm))
    # quantizer mutants must also reach the loop, which imported the name directly
    if mod is QUANT_MOD:
        for nm in names:
            monkeypatch.setattr(GPTQ_MOD, nm, getattr(m, nm))
    with pytest.raises(AssertionError):
        pin(golden_dir)


def test_unmutated_pins_pass(golden_dir):
    for _, _, _, _, pin in MUTANTS:
        pin(golden_dir)
