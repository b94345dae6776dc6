"""Pins of the oracle's packed fused decode with T >= 1 tokens per sequence
("feat(kda): add fused speculative decode kernel": packed ragged rows from
query_start_loc, accepted-token commit, per-token conv and state
checkpoints, padding rows; its bf16-pool follow-up: the recurrence is carried
unrounded across the token loop and each checkpoint is rounded on store).

Each pin checks the oracle against something other than its own code path:
a chain of single-token fused calls written out here, closed forms of the
frozen-state and unit-decay cases, exact data movement of the conv window,
and the rounding of an fp64 carry.
"""
import math

import numpy as np
import torch

import oracle
from gated_delta_rule_decode_amd import synth

D = 128
SCALE = 1.0 / math.sqrt(D)
NEG_INF_BF16 = np.uint16(0xFF80)
POS_INF_BF16 = np.uint16(0x7F80)


def _np(t):
    return oracle.as_np(t)


def _case(seed, lengths, H=2, slots=48, max_tokens=None, **kw):
    return synth.packed_fused_case(seed, lengths=lengths, H=H, num_slots=slots, max_tokens=max_tokens, **kw)


def _run(c, **over):
    a = dict(x=c.x, weight=c.weight, conv_state=c.conv_state, raw_gate=c.raw_gate,
             raw_beta=c.raw_beta, A_log=c.A_log, dt_bias=c.dt_bias, state_indices=c.state_indices,
             state=c.state, output_gate=c.output_gate, norm_weight=c.norm_weight,
             query_start_loc=c.query_start_loc, num_accepted_tokens=c.num_accepted_tokens)
    a.update(over)
    return oracle.packed_fused(**a)


def _silu(y):
    return y / (1.0 + np.exp(-y))


def _unit(x, eps=oracle.L2_EPS):
    return x / math.sqrt(float((x * x).sum()) + eps)


def _live(c, si=None, acc=None):
    """(sequence, rows, start slot, checkpoint columns) of the live sequences."""
    si = _np(c.state_indices) if si is None else si
    acc = _np(c.num_accepted_tokens) if acc is None else acc
    qsl = _np(c.query_start_loc)
    S = c.state.shape[0]
    out = []
    for i in range(si.shape[0]):
        a = int(acc[i])
        src = int(si[i, a - 1]) if 1 <= a <= si.shape[1] else -1
        if 0 < src < S and qsl[i + 1] > qsl[i]:
            out.append((i, range(int(qsl[i]), int(qsl[i + 1])), src, si[i]))
    return out


def test_chain_of_single_token_fused_calls():
    """With an fp64 pool (no storage rounding) a sequence of T tokens equals
    T single-token fused calls on a working slot that starts as a copy of the
    accepted checkpoint, each followed by a copy of the working slot into
    that token's checkpoint column: outputs, pool and conv cache bit for bit."""
    c = _case(31, [3, 1, 4, 2], max_tokens=4)
    st = _np(c.state).astype(np.float64)
    cs = _np(c.conv_state).copy()
    r = _run(c, state=st, conv_state=cs)
    S = st.shape[0]
    pool = np.concatenate([st, np.zeros((1,) + st.shape[1:])])      # working slot W = S
    conv = np.concatenate([cs, np.zeros((1,) + cs.shape[1:], cs.dtype)])
    W = S
    x, gr, br, og = _np(c.x), _np(c.raw_gate), _np(c.raw_beta), _np(c.output_gate)
    live = _live(c)
    assert len(live) == 4
    for i, rows, src, cols in live:
        pool[W], conv[W] = pool[src], conv[src]
        for j, row in enumerate(rows):
            f = oracle.fused(x[row:row + 1], c.weight, conv, gr[row:row + 1], br[row:row + 1], c.A_log,
                             c.dt_bias, np.array([W], np.int32), pool, og[row:row + 1], c.norm_weight)
            pool, conv = f["state"], np.ascontiguousarray(f["conv_state"])
            np.testing.assert_array_equal(r["out64"][row], f["out64"][0])
            np.testing.assert_array_equal(r["act64"][row], f["act64"][0])
            if j < len(cols) and 0 < cols[j] < S:
                pool[cols[j]], conv[cols[j]] = pool[W], conv[W]
    np.testing.assert_array_equal(r["state"], pool[:S])
    np.testing.assert_array_equal(r["conv_state"], conv[:S])


def test_single_token_rows_equal_the_fused_call():
    """T=1 everywhere, one accepted token, column 0 = the fused call's index:
    the fused decode (fp32 pool, null rows 0 and -1 included) bit for bit."""
    fc = synth.fused_case(32, rows=6, H=2, num_slots=10, null_zero=1, null_neg=1)
    f = oracle.fused(fc.x, fc.weight, fc.conv_state, fc.raw_gate, fc.raw_beta, fc.A_log, fc.dt_bias,
                     fc.state_indices, fc.state, fc.output_gate, fc.norm_weight)
    r = oracle.packed_fused(fc.x, fc.weight, fc.conv_state, fc.raw_gate, fc.raw_beta, fc.A_log,
                            fc.dt_bias, _np(fc.state_indices).reshape(6, 1), fc.state, fc.output_gate,
                            fc.norm_weight, query_start_loc=np.arange(7, dtype=np.int32),
                            num_accepted_tokens=np.ones(6, np.int32))
    for key in ("out64", "out_bf16", "act64", "state", "conv_state"):
        np.testing.assert_array_equal(r[key], f[key], err_msg=key)


def test_conv_window_runs_across_tokens():
    """One-hot taps (q: tap 0, k: tap 2, v: tap 3): the pre-SiLU conv of token j
    is entry j+tap of [window (oldest first), x_0, x_1, ...]; the conv
    checkpoint after token j holds entries j+1..j+3 of that sequence."""
    H = 2
    c = _case(33, [4, 2, 3], H=H, max_tokens=4)
    HC = H * D
    taps = [0, 2, 3]
    w = np.zeros((3, 4, HC), np.float32)
    for grp, t in enumerate(taps):
        w[grp, t, :] = 1.0
    cs0 = _np(c.conv_state).copy()
    r = _run(c, weight=w, conv_state=cs0)
    x = oracle.bf16_to_f64(_np(c.x))
    for i, rows, src, cols in _live(c):
        seq = [oracle.bf16_to_f64(cs0[src, :, p]) for p in range(3)] + [x[row] for row in rows]
        for j, row in enumerate(rows):
            for grp, t in enumerate(taps):
                np.testing.assert_allclose(r["act64"][row, grp * HC:(grp + 1) * HC],
                                           _silu(seq[j + t][grp * HC:(grp + 1) * HC]), rtol=1e-14, atol=1e-300)
            for p in range(3):
                np.testing.assert_array_equal(oracle.bf16_to_f64(r["conv_state"][cols[j], :, p]), seq[j + 1 + p])


def test_frozen_state_checkpoints_and_readout():
    """Unit decay (A_log = -inf) and beta = 0 (logit -inf): every checkpoint
    slot equals the start state bit for bit; o = scale * S^T q_hat on that
    state and the output is the gated RMSNorm of o, both in closed form."""
    H = 2
    c = _case(34, [3, 2], H=H, max_tokens=3)
    A_log = torch.full((H,), -math.inf)
    braw = np.full(_np(c.raw_beta).shape, NEG_INF_BF16, np.uint16)
    st0 = _np(c.state).copy()
    r = _run(c, A_log=A_log, raw_beta=braw)
    og = oracle.bf16_to_f64(_np(c.output_gate))
    nw = _np(c.norm_weight).astype(np.float64)
    for i, rows, src, cols in _live(c):
        for j, row in enumerate(rows):
            np.testing.assert_array_equal(r["state"][cols[j]], st0[src])
            for h in range(H):
                P = st0[src, h].astype(np.float64)                       # [v][k]
                q = _unit(r["act64"][row, h * D:(h + 1) * D])
                o = SCALE * (P @ q)
                np.testing.assert_allclose(r["o_pre64"][row, h], o, rtol=1e-12, atol=1e-15)
                y = o / math.sqrt(float((o * o).mean()) + 1e-5) * nw / (1.0 + np.exp(-og[row, h]))
                np.testing.assert_allclose(r["out64"][row, h], y, rtol=1e-11, atol=1e-14)


def test_unit_decay_beta_one_stores_every_value():
    """Unit decay and beta = 1 with l2_eps = 0: after every token the state
    maps the normalised key to that token's value, k_hat^T S_j = v_j."""
    H = 2
    c = _case(35, [3, 4], H=H, max_tokens=4)
    A_log = torch.full((H,), -math.inf)
    braw = np.full(_np(c.raw_beta).shape, POS_INF_BF16, np.uint16)
    r = _run(c, A_log=A_log, raw_beta=braw, l2_eps=0.0, want_ckpt64=True)
    HC = H * D
    for i, rows, src, cols in _live(c):
        for row in rows:
            for h in range(H):
                k = r["act64"][row, HC + h * D:HC + (h + 1) * D]
                v = r["act64"][row, 2 * HC + h * D:2 * HC + (h + 1) * D]
                kv = r["ckpt64"][row, h] @ (k / math.sqrt(float((k * k).sum())))
                np.testing.assert_allclose(kv, v, rtol=0, atol=1e-12 * max(1.0, float(np.abs(v).max())))


def test_bf16_checkpoints_round_an_unrounded_carry():
    """bf16 pool: each checkpoint is the RNE rounding of the fp64 state after
    that token, and the carry is not re-rounded: outputs equal, bit for bit,
    those of an fp64 pool holding the same start values."""
    c = _case(36, [4, 3], max_tokens=4, state_dtype=torch.bfloat16)
    rb = _run(c, want_ckpt64=True)
    st64 = oracle.bf16_to_f64(_np(c.state))
    r64 = _run(c, state=st64, want_ckpt64=True)
    np.testing.assert_array_equal(rb["out64"], r64["out64"])
    np.testing.assert_array_equal(rb["ckpt64"], r64["ckpt64"])
    for i, rows, src, cols in _live(c):
        for j, row in enumerate(rows):
            np.testing.assert_array_equal(rb["state"][cols[j]], oracle.bf16_from_f64(rb["ckpt64"][row]))
            np.testing.assert_array_equal(r64["state"][cols[j]], r64["ckpt64"][row])
    # the carry matters: re-rounding the state after every token changes the last checkpoint
    seq_rows = _live(c)[0][1]
    assert not np.array_equal(rb["ckpt64"][seq_rows[-1]],
                              oracle.bf16_to_f64(oracle.bf16_from_f64(rb["ckpt64"][seq_rows[-1]])))


def test_padding_null_sequences_and_checkpoint_columns():
    """Sequence 0 runs past max_tokens (its 4th token writes nothing) and has
    column 1 set to the reserved slot 0 (not written); sequence 1 is empty; sequence 2 starts from column 2 and has column 1 set
    to -1 (that token writes nothing, the loop goes on); sequence 3 starts
    from slot 0 and sequence 4 has no accepted token (both null); two
    trailing rows belong to no sequence.  Null and trailing rows give +0,
    and only the written checkpoint slots change."""
    c = _case(37, [4, 0, 3, 1, 2], max_tokens=3, pad_rows=2)
    si = _np(c.state_indices).copy()
    acc = np.array([1, 1, 3, 1, 0], np.int32)
    si[0, 1] = 0
    si[2, 1] = -1
    si[3, 0] = 0
    st0, cs0 = _np(c.state).copy(), _np(c.conv_state).copy()
    r = _run(c, state_indices=si, num_accepted_tokens=acc)
    live_rows = set(range(0, 4)) | set(range(4, 7))
    for row in range(12):
        if row not in live_rows:
            assert not r["out64"][row].any() and not r["out_bf16"][row].any(), row
        else:
            assert np.abs(r["out64"][row]).max() > 0, row
    written = {int(si[0, 0]), int(si[0, 2]), int(si[2, 0]), int(si[2, 2])}
    for s in range(st0.shape[0]):
        same = np.array_equal(r["state"][s], st0[s]) and np.array_equal(r["conv_state"][s], cs0[s])
        assert same == (s not in written), s
    # the padded column changes nothing else: with a real slot there, the same
    # outputs and the same later checkpoint
    si2 = si.copy()
    si2[2, 1] = int(_np(c.state_indices)[2, 1])
    r2 = _run(c, state_indices=si2, num_accepted_tokens=acc)
    np.testing.assert_array_equal(r["out64"], r2["out64"])
    np.testing.assert_array_equal(r["state"][si[2, 2]], r2["state"][si[2, 2]])
