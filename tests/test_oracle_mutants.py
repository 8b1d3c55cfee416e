"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is the oracle's own source with one plausible mistake edited in
(a dropped term, a wrong sign, index or axis, a transposed operand); the pins
in ``tests/oracle_pins.py`` must reject every one of them.
"""
import inspect
import types

import pytest

import oracle.attention as ref
from tests import oracle_pins as pins

SRC = inspect.getsource(ref)

FWD_MUTANTS = {
    "dropped_scale": ("s = scale * (qh[rows] @ kh.T)", "s = (qh[rows] @ kh.T)"),
    "mask_includes_diagonal": ("s[j[None, :] > rows[:, None]] = -np.inf", "s[j[None, :] >= rows[:, None]] = -np.inf"),
    "mask_wrong_side": ("s[j[None, :] > rows[:, None]] = -np.inf", "s[j[None, :] < rows[:, None]] = -np.inf"),
    "q_k_swapped": ("s = scale * (qh[rows] @ kh.T)", "s = scale * (kh[rows] @ qh.T)"),
    "lse_drops_max": ("lse = m + np.log(l)", "lse = np.log(l)"),
    "lse_log2": ("lse = m + np.log(l)", "lse = m + np.log2(l)"),
    "unnormalised_p": ("p = e / l[:, None]", "p = e"),
    "normalised_wrong_axis": ("p = e / l[:, None]", "p = e / e.sum(axis=0)[None, :]"),
    "gqa_modulo_mapping": ("g = h // G\n            oh, lh", "g = h % Hkv\n            oh, lh"),
    "packed_lse_offset": ("lse[h, sl.start + r] = lh", "lse[h, r] = lh"),
    "exp_sign": ("e = np.exp(s - m[:, None])", "e = np.exp(m[:, None] - s)"),
}

BWD_MUTANTS = {
    "ds_sign_of_d": ("ds = p * (dp - d_row[:, None])", "ds = p * (dp + d_row[:, None])"),
    "d_uses_do_twice": ("d_row = np.sum(doh * oh, axis=1)", "d_row = np.sum(doh * doh, axis=1)"),
    "dq_drops_scale": ("dq = scale * (ds @ kh)", "dq = (ds @ kh)"),
    "dk_untransposed": ("dk = scale * (ds.T @ qh)", "dk = scale * (ds @ qh)"),
    "dv_untransposed": ("dv = p.T @ doh", "dv = p @ doh"),
    "dp_extra_scale": ("dp = doh @ vh.T", "dp = scale * (doh @ vh.T)"),
    "dk_group_overwrites": ("dks[:, g, :] += gk", "dks[:, g, :] = gk"),
    "dv_group_overwrites": ("dvs[:, g, :] += gv", "dvs[:, g, :] = gv"),
    "dq_uses_v": ("dq = scale * (ds @ kh)", "dq = scale * (ds @ vh)"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    fwd = lambda q, k, v, scale, causal, cu: mod.attention_forward(q, k, v, scale, causal, cu)
    bwd = lambda q, k, v, do, scale, causal, cu: mod.attention_backward(q, k, v, do, scale, causal, cu)
    return fwd, bwd


def _caught(pin_list, fwd, bwd):
    for pin in pin_list:
        try:
            pin(fwd, bwd)
        except Exception:
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_mutant_is_caught(name):
    fwd, bwd = _mutant(*FWD_MUTANTS[name])
    assert _caught(pins.ALL_FWD_PINS, fwd, bwd) is not None, f"mutant {name} passed every forward pin"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name):
    fwd, bwd = _mutant(*BWD_MUTANTS[name])
    order = [pins.pin_gradient_invariants, pins.pin_torch, pins.pin_reductions, pins.pin_finite_differences]
    assert _caught(order, fwd, bwd) is not None, f"mutant {name} passed every backward pin"


DQ_ROWS_MUTANTS = {
    "rows_ds_sign_of_d": ("ds_r = p_r * (dp_r - dd_r[:, None])", "ds_r = p_r * (dp_r + dd_r[:, None])"),
    "rows_d_uses_do_twice": ("dd_r = np.sum(do_r * o_r, axis=1)", "dd_r = np.sum(do_r * do_r, axis=1)"),
    "rows_drops_scale": ("return scale * (ds_r @ kh)", "return (ds_r @ kh)"),
    "rows_uses_v": ("return scale * (ds_r @ kh)", "return scale * (ds_r @ vh)"),
    "rows_unselected_do": ("do_r = doh[rows]", "do_r = doh[:len(rows)]"),
}


@pytest.mark.parametrize("name", sorted(DQ_ROWS_MUTANTS))
def test_dq_rows_mutant_is_caught(name):
    old, new = DQ_ROWS_MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        pins.pin_dq_rows(mod.head_backward_dq_rows)


SPLIT_MUTANTS = {
    "chunk_size_floor": ("c = -(-nk // n_splits)", "c = nk // n_splits"),
    "query_offset_sign": ("nk - nq, kb, ke)", "nq - nk, kb, ke)"),
    "chunk_mask_includes_diagonal": ("s[j[None, :] > (np.arange(nq) + q_off)[:, None]] = -np.inf",
                                     "s[j[None, :] >= (np.arange(nq) + q_off)[:, None]] = -np.inf"),
    "chunk_positions_local": ("j = np.arange(kb, ke)", "j = np.arange(0, ke - kb)"),
    "dead_rows_not_skipped": ("live = np.isfinite(s).any(axis=1)", "live = np.ones(nq, dtype=bool)"),
    "chunk_lse_drops_max": ("lse[live] = m + np.log(l)", "lse[live] = np.log(l)"),
    "merge_weight_sign": ("w = np.exp(lse_part - m_safe[None])", "w = np.exp(m_safe[None] - lse_part)"),
    "merge_unnormalised": ("coef = np.where(dead[None], 0.0, w / np.where(dead, 1.0, tot)[None])",
                           "coef = np.where(dead[None], 0.0, w)"),
    "merge_lse_drops_max": ("lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, tot)))",
                            "lse = np.where(dead, -np.inf, np.log(np.where(dead, 1.0, tot)))"),
    "merge_takes_max_part": ("o = np.einsum(\"pbhn,pbnhd->bnhd\", coef, o_part)",
                             "o = o_part[np.argmax(lse_part.max(axis=(1, 2, 3)))]"),
}


@pytest.mark.parametrize("name", sorted(SPLIT_MUTANTS))
def test_split_mutant_is_caught(name):
    old, new = SPLIT_MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        pins.pin_split(mod.attention_forward_split, mod.merge_partials)


FP8_MUTANTS = {
    "exponent_bias_8": ("(1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)",
                        "(1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 8.0)"),
    "subnormal_exponent": ("np.where(e == 0, m / 8.0 * 2.0 ** -6,", "np.where(e == 0, m / 8.0 * 2.0 ** -7,"),
    "mantissa_over_16": ("(1.0 + m / 8.0) * np.exp2", "(1.0 + m / 16.0) * np.exp2"),
    "nan_code_missed": ("return np.where((b & 0x7F) == 0x7F, np.nan, out)", "return out"),
    "sign_dropped": ("sign = np.where(b & 0x80, -1.0, 1.0)", "sign = np.where(b & 0x80, 1.0, 1.0)"),
    "q_descale_sequence_order": ("q[b] *= _token_descales(qd[b], q.shape[1])", "q[b] *= _token_descales(qd[-1 - b], q.shape[1])"),
    "k_scaled_by_q_descale": ("k[b] *= _token_descales(kd[b], k.shape[1])", "k[b] *= _token_descales(qd[b][:kd.shape[1]], k.shape[1])"),
    "packed_descale_first_sequence": ("q[cu[s]:cu[s + 1]] *= _token_descales(qd[s], L)", "q[cu[s]:cu[s + 1]] *= _token_descales(qd[0], L)"),
}

# Mistakes in the block-scaled dequantisation, each caught by pin_fp8_blocks.
FP8_BLOCK_MUTANTS = {
    "block_of_32_tokens": ("    block = np.arange(n_tokens) // FP8_SCALE_BLOCK",
                           "    block = np.minimum(np.arange(n_tokens) // 32, desc.shape[1] - 1)"),
    "block_off_by_one": ("    block = np.arange(n_tokens) // FP8_SCALE_BLOCK",
                         "    block = np.minimum((np.arange(n_tokens) + 1) // FP8_SCALE_BLOCK, desc.shape[1] - 1)"),
    "first_block_everywhere": ("    return desc[:, block].T", "    return desc[:, 0 * block].T"),
    "blocks_transposed": ("    return desc[:, block].T", "    return desc[:, block].T[::-1]"),
    "packed_block_from_global_position": (
        "            q[cu[s]:cu[s + 1]] *= _token_descales(qd[s], L)[:, :, None]",
        "            q[cu[s]:cu[s + 1]] *= _token_descales(qd[s], int(cu[s + 1]))[int(cu[s]):, :, None]"),
    "k_head_0_descales_for_every_head": ("            k[b] *= _token_descales(kd[b], k.shape[1])[:, :, None]",
                                       "            k[b] *= _token_descales(kd[b][:1].repeat(kd.shape[1], axis=0), k.shape[1])[:, :, None]"),
}


@pytest.mark.parametrize("name", sorted(FP8_BLOCK_MUTANTS))
def test_fp8_block_mutant_is_caught(name):
    old, new = FP8_BLOCK_MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    with pytest.raises(Exception):   # a wrong value (AssertionError) or a block index past the array
        pins.pin_fp8_blocks(mod.attention_forward_fp8)


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name):
    old, new = FP8_MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        pins.pin_fp8(mod.attention_forward_fp8, mod.e4m3_to_float)


ROWDOT_MUTANTS = {
    "rowdot_do_twice": ("d = np.sum(do * o, axis=-1)", "d = np.sum(do * do, axis=-1)"),
    "rowdot_sums_wrong_axis": ("d = np.sum(do * o, axis=-1)", "d = np.sum(do * o, axis=-2)"),
    "rowdot_packed_untransposed": ("    return d.T.copy()", "    return d.copy()"),
    "rowdot_uniform_swapped_axes": ("np.transpose(d, (0, 2, 1))", "np.transpose(d, (2, 1, 0))"),
}


@pytest.mark.parametrize("name", sorted(ROWDOT_MUTANTS))
def test_rowdot_mutant_is_caught(name):
    old, new = ROWDOT_MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    with pytest.raises(Exception):
        pins.pin_rowdot(mod.backward_rowdot)
