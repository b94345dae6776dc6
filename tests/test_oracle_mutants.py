"""The oracle pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/kda_oracle.c (on the CPU),
builds it, routes the oracle wrapper to that build and runs the pins: at
least one pin must fail.  This shows the pins constrain every part of the
oracle (orientation, decay, gate, delta rule, readout, conv, norm, null
rows, rounding), not only its happy path.  The packed call's q|k|v row split
lives in the Python wrapper, so its planted mistakes replace the wrapper.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_packed_fused as pf
from tests import test_oracle_pins as pins

MUTANTS = [
    ("state orientation transposed",
     "S[k][v] = load_elem(pool, dt, head_base + (size_t)v * KD + k);",
     "S[v][k] = load_elem(pool, dt, head_base + (size_t)v * KD + k);"),
    ("decay dropped", "S[k][j] *= decay[k];", "S[k][j] *= 1.0;"),
    ("decay indexed by value", "S[k][j] *= decay[k];", "S[k][j] *= decay[j];"),
    ("delta sign", "u[j] = v[j] - acc;", "u[j] = v[j] + acc;"),
    ("beta dropped from update", "S[k][j] += beta * kh[k] * u[j];", "S[k][j] += kh[k] * u[j];"),
    ("readout with k", "for (int k = 0; k < KD; ++k) acc += S[k][j] * qh[k];\n        o[j]",
     "for (int k = 0; k < KD; ++k) acc += S[k][j] * kh[k];\n        o[j]"),
    ("scale dropped", "o[j] = scale * acc;", "o[j] = acc;"),
    ("readout before update",
     "    /* S <- S + beta k u^T */\n    for (int k = 0; k < KD; ++k)\n        for (int j = 0; j < KD; ++j) S[k][j] += beta * kh[k] * u[j];\n",
     "    double Sn[KD][KD];\n    for (int k = 0; k < KD; ++k)\n        for (int j = 0; j < KD; ++j) Sn[k][j] = S[k][j] + beta * kh[k] * u[j];\n"),
    ("softplus sign", "log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    ("gate sign", "double g = -a * softplus", "double g = a * softplus"),
    ("A_log not exponentiated", "double a = exp(A_log_h);", "double a = A_log_h;"),
    ("dt_bias head offset", "gate_decay(gv, (double)A_log[hv], dt_bias + hv * KD, dec);",
     "gate_decay(gv, (double)A_log[hv], dt_bias, dec);"),
    ("beta not squashed", "b = sigmoid(bin);", "b = bin;"),
    ("q/k head not grouped", "const int64_t hk = hv / group;", "const int64_t hk = hv % H;"),
    ("precomputed decay taken as the gate", "for (int j = 0; j < KD; ++j) dec[j] = exp(gv[j]);",
     "for (int j = 0; j < KD; ++j) dec[j] = gv[j];"),
    ("correction without beta", "for (int j = 0; j < KD; ++j) corr[j] = beta * u[j];",
     "for (int j = 0; j < KD; ++j) corr[j] = u[j];"),
    ("gate cache holds the decay", "kg[cs * 2 * KD + KD + j] = gv[j];",
     "kg[cs * 2 * KD + KD + j] = dec[j];"),
    ("read-only pool written", "if (update_state) scatter_state(state, state_dtype, head_base, S);",
     "scatter_state(state, state_dtype, head_base, S);"),
    ("l2 norm dropped", "double inv = 1.0 / sqrt(ss + eps);", "double inv = 1.0;"),
    ("null row output not zero", "if (out64) out64[oi] = 0.0;\n                        if (out_bf16)",
     "if (out64) out64[oi] = 1.0;\n                        if (out_bf16)"),
    ("state not carried across tokens",
     "            for (int64_t t = t0; t < t1; ++t) {\n                size_t vq",
     "            for (int64_t t = t0; t < t1; ++t) {\n                gather_state(state, state_dtype, head_base, S);\n                size_t vq"),
    ("conv taps reversed", "weight[(grp * 4 + j) * HC + cc]", "weight[(grp * 4 + (3 - j)) * HC + cc]"),
    ("conv group ignored", "weight[(grp * 4 + j) * HC + cc]", "weight[j * HC + cc]"),
    ("conv cache not shifted", "cs[0 * C3 + c] = cs[1 * C3 + c];", "cs[0 * C3 + c] = cs[0 * C3 + c];"),
    ("silu dropped", "act[c] = y * sigmoid(y);", "act[c] = y;"),
    ("rms uses sum", "ms /= (double)KD;", "ms /= 1.0;"),
    ("norm gate not squashed", "sigmoid(bf16_to_f64(ogate[vec + j]))", "bf16_to_f64(ogate[vec + j])"),
    ("fused slot 0 live", "int null_row = idx <= 0 ||", "int null_row = idx < 0 ||"),
    ("packed fused starts from column 0",
     "int32_t src = (a >= 1 && a <= max_tokens) ? cols[a - 1] : -1;",
     "int32_t src = (a >= 1 && a <= max_tokens) ? cols[0] : -1;"),
    ("packed fused conv window not advanced", "                win[c] = win[C3 + c];\n",
     "                win[c] = win[c];\n"),
    ("packed fused checkpoint columns reversed", "int32_t dst = j < max_tokens ? cols[j] : -1;",
     "int32_t dst = j < max_tokens ? cols[max_tokens - 1 - j] : -1;"),
    ("packed fused state re-read every token",
     "        for (int64_t r = t0; r < t1; ++r) {\n            const int64_t j = r - t0;",
     "        for (int64_t r = t0; r < t1; ++r) {\n            for (int64_t h = 0; h < H; ++h)\n"
     "                gather_state(state, state_dtype, ((size_t)src * H + h) * head_elems, S[h]);\n"
     "            const int64_t j = r - t0;"),
    ("packed fused padding rows not zero", "        if (out64) out64[i] = 0.0;", "        if (out64) out64[i] = 1.0;"),
    ("packed fused slot 0 live", "if (src <= 0 || (int64_t)src >= num_slots || t1 <= t0) continue;",
     "if (src < 0 || (int64_t)src >= num_slots || t1 <= t0) continue;"),
    ("packed fused checkpoint skips slot filter",
     "if (dst > 0 && (int64_t)dst < num_slots) {\n                memcpy",
     "if (dst >= 0 && (int64_t)dst < num_slots) {\n                memcpy"),
    ("gate read from the sequence's first token",
     "for (int j = 0; j < KD; ++j) gv[j] = load_in(g, g_f32, vh + j);",
     "for (int j = 0; j < KD; ++j) gv[j] = load_in(g, g_f32, ((size_t)t0 * HV + hv) * KD + j);"),
    ("state gathered from the row position",
     "size_t head_base = ((size_t)idx * HV + hv) * head_elems;",
     "size_t head_base = ((size_t)(i % num_slots) * HV + hv) * head_elems;"),
    ("bf16 rounding truncates", "double q = nearbyint(m * 256.0);", "double q = trunc(m * 256.0);"),
    ("bf16 ties away", "double q = nearbyint(m * 256.0);", "double q = round(m * 256.0);"),
]

PINS = [
    pins.test_bf16_rounding_ties_and_double_rounding,
    lambda: pins.test_beta_zero_unit_decay_keeps_state_and_reads_out(pins.torch.float32),
    pins.test_beta_one_unit_decay_writes_value_exactly,
    pins.test_zero_state_closed_form,
    pins.test_decay_is_per_key_channel_along_the_contiguous_dim,
    pins.test_half_decay_special_value,
    pins.test_softplus_extremes,
    pins.test_null_rows_zero_output_and_untouched_slots,
    pins.test_two_tokens_orthogonal_keys_closed_form,
    pins.test_same_key_beta_one_overwrites,
    pins.test_product_form_cross_formulation,
    pins.test_beta_zero_tokens_read_out_the_cumulatively_decayed_state,
    pins.test_row_permutation_permutes_outputs_and_keeps_pool,
    pins.test_conv_one_hot_taps_reproduce_lagged_inputs,
    pins.test_conv_output_feeds_recurrence_as_qkv,
    pins.test_gated_rmsnorm_invariants,
    pins.test_fused_null_rows,
    pins.test_grouped_heads_equal_repeated_qk,
    pins.test_precomputed_gate_is_log_decay_per_key_channel,
    pins.test_precomputed_beta_is_used_as_is,
    pins.test_read_only_pool,
    pins.test_batched_form_equals_uniform_cu_seqlens,
    lambda: pins.test_verify_caches_rebuild_every_checkpoint("in_kernel"),
    lambda: pins.test_verify_caches_rebuild_every_checkpoint("precomputed"),
    pins.test_verify_caches_positions_and_null_rows,
    pf.test_chain_of_single_token_fused_calls,
    pf.test_single_token_rows_equal_the_fused_call,
    pf.test_conv_window_runs_across_tokens,
    pf.test_frozen_state_checkpoints_and_readout,
    pf.test_unit_decay_beta_one_stores_every_value,
    pf.test_bf16_checkpoints_round_an_unrounded_carry,
    pf.test_padding_null_sequences_and_checkpoint_columns,
]


PACKED_PINS = [
    pins.test_packed_row_split_zero_state_closed_form,
    pins.test_packed_equals_recurrent_on_hand_sliced_rows,
]

# Planted mistakes of the packed wrapper's row split: which third of the
# q|k|v row each of q, k and v is read from.
PACKED_MUTANTS = [
    ("packed k and v swapped", (0, 2, 1)),
    ("packed q and k swapped", (1, 0, 2)),
    ("packed v read from q", (0, 1, 0)),
]


def _packed_with_split(order):
    def packed(mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, state, state_indices):
        qkv = oracle.as_np(mixed_qkv)
        B = qkv.shape[0]
        H = np.asarray(oracle.as_np(A_log)).shape[0]
        HC = H * oracle.D
        q, k, v = (np.ascontiguousarray(qkv[:, j * HC:(j + 1) * HC]).reshape(B, H, oracle.D) for j in order)
        return oracle.recurrent(q, k, v, oracle.as_np(raw_gate).reshape(B, H, oracle.D),
                                oracle.as_np(raw_beta).reshape(B, H), A_log, dt_bias, state, state_indices)
    return packed


def test_packed_wrapper_as_written_passes():
    for pin in PACKED_PINS:
        pin()


@pytest.mark.parametrize("name,order", PACKED_MUTANTS, ids=[m[0] for m in PACKED_MUTANTS])
def test_planted_packed_split_mistake_is_caught(name, order, monkeypatch):
    monkeypatch.setattr(oracle, "packed", _packed_with_split(order))
    for pin in PACKED_PINS:
        with pytest.raises(AssertionError):
            pin()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert old in src, f"mutation anchor for '{name}' not found"
    mutated = src.replace(old, new)
    c = tmp_path / "mut.c"
    c.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-w", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    caught = []
    with oracle.using_library(str(so)):
        for pin in PINS:
            try:
                pin()
            except Exception:  # an assertion, or a shape/NaN error of the broken oracle
                caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"no pin catches the planted mistake '{name}'"
