"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a closed
form of a special case, an invariant of the method, a library routine that a
special case reduces to, or an algebraically different formulation.  They are
chosen so that a dropped term, a wrong sign, a transposed operand or a wrong
index in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import synth

D = 128
SCALE = 1.0 / math.sqrt(D)
NEG_INF_BF16 = np.uint16(0xFF80)
POS_INF_BF16 = np.uint16(0x7F80)


def _np(t):
    return oracle.as_np(t)


def _bf16(x):
    return oracle.bf16_from_f64(np.asarray(x, np.float64))


def _unit(x):
    x = np.asarray(x, np.float64)
    return x / math.sqrt(float((x * x).sum()) + oracle.L2_EPS)


def _case(seed=1, n=3, H=2, slots=5, state_dtype=torch.float32, **kw):
    return synth.recurrent_case(seed, n_seqs=n, H=H, num_slots=slots,
                                state_dtype=state_dtype, **kw)


def _run(c, **over):
    args = dict(q=c.q, k=c.k, v=c.v, g=c.g, beta=c.beta, A_log=c.A_log,
                dt_bias=c.dt_bias, state=c.state, state_indices=c.state_indices,
                cu_seqlens=c.cu_seqlens)
    args.update(over)
    return oracle.recurrent(**args)


# ---- bf16 storage format --------------------------------------------------------

def test_bf16_rounding_matches_torch_on_fp32_values():
    """For fp32-representable values the direct fp64->bf16 rounding must equal
    the library's fp32->bf16 round-to-nearest-even (torch)."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
        np.array([0.0, -0.0, 1e-45, -1e-45, 1.17e-38, 3.3e38, -3.39e38]),
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_f64(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_rounding_ties_and_double_rounding():
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,            # tie, even stays at 1.0
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # tie, rounds up to the even code
        1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,  # just above the tie: up (fp32 first would tie to 1.0)
        -2.5: 0xC020,
        2.0 ** -133: 0x0001,                # smallest subnormal
        2.0 ** 128: 0x7F80,
        float.fromhex("0x1.FEp127"): 0x7F7F,                 # largest finite bf16
        float.fromhex("0x1.FFp127"): 0x7F80,  # tie above max: to even = inf
        float.fromhex("0x1.FEFp127"): 0x7F7F,   # below the tie: stays finite
    }
    got = oracle.bf16_from_f64(np.array(list(cases.keys())))
    np.testing.assert_array_equal(got, np.array(list(cases.values()), np.uint16))


# ---- invariants of the recurrence ----------------------------------------------------

@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_beta_zero_unit_decay_keeps_state_and_reads_out(state_dtype):
    """A_log=-inf makes every decay exactly 1 and beta logits -inf make beta 0:
    the state is unchanged bit for bit and o = scale * S^T q_hat."""
    c = _case(state_dtype=state_dtype)
    H = c.H
    A = torch.full((H,), -math.inf)
    braw = np.full((c.q.shape[0], H), NEG_INF_BF16)
    r = _run(c, A_log=A, beta=braw)
    np.testing.assert_array_equal(r["state"], _np(c.state))
    S = _np(c.state.float()).astype(np.float64)
    q = _np(c.q.float()).astype(np.float64)
    for i in range(c.q.shape[0]):
        slot = int(c.state_indices[i])
        for h in range(H):
            # pool holds [v][k]; S^T q in math orientation is pool @ q
            want = SCALE * (S[slot, h] @ _unit(q[i, h]))
            np.testing.assert_allclose(r["out64"][i, h], want, rtol=1e-12, atol=1e-15)


def test_beta_one_unit_decay_writes_value_exactly():
    """beta=1 with unit decay and eps=0: k_hat^T S' = v (the delta rule stores v
    under key k exactly)."""
    c = _case(seed=2)
    H = c.H
    r = _run(c, A_log=torch.full((H,), -math.inf),
             beta=np.full((c.q.shape[0], H), POS_INF_BF16),
             state=_np(c.state).astype(np.float64), l2_eps=0.0)
    k = _np(c.k.float()).astype(np.float64)
    v = _np(c.v.float()).astype(np.float64)
    for i in range(c.q.shape[0]):
        slot = int(c.state_indices[i])
        for h in range(H):
            kh = k[i, h] / np.linalg.norm(k[i, h])
            np.testing.assert_allclose(r["state"][slot, h] @ kh, v[i, h], rtol=0, atol=1e-12)


def test_zero_state_closed_form():
    """S=0: S' = beta k_hat v^T, o = scale * beta * (q_hat . k_hat) * v."""
    c = _case(seed=3)
    H = c.H
    st = np.zeros_like(_np(c.state), dtype=np.float64)
    r = _run(c, state=st)
    q = _np(c.q.float()).astype(np.float64)
    k = _np(c.k.float()).astype(np.float64)
    v = _np(c.v.float()).astype(np.float64)
    braw = oracle.bf16_to_f64(_np(c.beta))
    for i in range(c.q.shape[0]):
        slot = int(c.state_indices[i])
        for h in range(H):
            beta = 1.0 / (1.0 + math.exp(-braw[i, h]))
            qh, kh = _unit(q[i, h]), _unit(k[i, h])
            np.testing.assert_allclose(r["state"][slot, h], beta * np.outer(v[i, h], kh),
                                       rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(r["out64"][i, h], SCALE * beta * (qh @ kh) * v[i, h],
                                       rtol=1e-12, atol=1e-15)


def _packed_row_case(seed, B, H):
    """Random inputs of the packed T=1 call: bf16 q|k|v rows, raw gate and
    beta logits, gate parameters."""
    rng = np.random.default_rng(seed)
    HC = H * D
    return dict(mixed_qkv=_bf16(rng.standard_normal((B, 3 * HC))),
                raw_gate=_bf16(rng.standard_normal((B, HC))),
                raw_beta=_bf16(rng.standard_normal((B, H))),
                A_log=rng.uniform(-2.0, 0.0, H).astype(np.float32),
                dt_bias=(rng.standard_normal(HC) * 0.1).astype(np.float32))


def test_packed_row_split_zero_state_closed_form():
    """The packed call's projection row holds q at [0, H*128), k at
    [H*128, 2*H*128) and v at [2*H*128, 3*H*128), head-major inside each
    ("Serving-native packed Kimi K3 decode", and the Exact contract of the
    serving-native packed decode PR).  With a zero state the update is
    S' = beta k_hat v^T and o = scale beta (q_hat . k_hat) v; both are
    evaluated here from slices of the row taken by hand, so a q/k/v slice
    mix-up in the wrapper (k and v swapped, say) fails."""
    B, H = 3, 2
    HC = H * D
    c = _packed_row_case(11, B, H)
    idx = np.array([2, 0, 3], np.int32)
    st = np.zeros((4, H, D, D), np.float64)
    r = oracle.packed(c["mixed_qkv"], c["raw_gate"], c["raw_beta"], c["A_log"], c["dt_bias"], st, idx)
    x = oracle.bf16_to_f64(c["mixed_qkv"])
    braw = oracle.bf16_to_f64(c["raw_beta"])
    for b in range(B):
        for h in range(H):
            q = x[b, h * D:(h + 1) * D]
            k = x[b, HC + h * D:HC + (h + 1) * D]
            v = x[b, 2 * HC + h * D:2 * HC + (h + 1) * D]
            beta = 1.0 / (1.0 + math.exp(-braw[b, h]))
            qh, kh = _unit(q), _unit(k)
            np.testing.assert_allclose(r["state"][idx[b], h], beta * np.outer(v, kh), rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(r["out64"][b, h], SCALE * beta * (qh @ kh) * v, rtol=1e-12, atol=1e-15)
    assert not r["state"][1].any(), "a slot no row names stays zero"


def test_packed_equals_recurrent_on_hand_sliced_rows():
    """On a random pool with an inactive (-1) row, the packed call equals the
    recurrent call on q, k, v sliced by hand from the row (and the raw gate
    and beta reshaped to [B, H, 128] and [B, H]), bit for bit."""
    B, H = 4, 3
    HC = H * D
    c = _packed_row_case(12, B, H)
    rng = np.random.default_rng(13)
    st = (rng.standard_normal((6, H, D, D)) * 0.05).astype(np.float32)
    idx = np.array([5, -1, 0, 2], np.int32)
    got = oracle.packed(c["mixed_qkv"], c["raw_gate"], c["raw_beta"], c["A_log"], c["dt_bias"], st, idx)
    qkv = c["mixed_qkv"]
    want = oracle.recurrent(np.ascontiguousarray(qkv[:, 0:HC]).reshape(B, H, D),
                            np.ascontiguousarray(qkv[:, HC:2 * HC]).reshape(B, H, D),
                            np.ascontiguousarray(qkv[:, 2 * HC:3 * HC]).reshape(B, H, D),
                            c["raw_gate"].reshape(B, H, D), c["raw_beta"], c["A_log"], c["dt_bias"], st, idx)
    np.testing.assert_array_equal(got["out64"], want["out64"])
    np.testing.assert_array_equal(got["out_bf16"], want["out_bf16"])
    np.testing.assert_array_equal(got["state"], want["state"])
    assert not got["out64"][1].any()


def test_decay_is_per_key_channel_along_the_contiguous_dim():
    """beta=0, raw gate 0 and a dt_bias that varies over k: every stored
    element pool[v][k] is scaled by exp(-exp(A_log) * softplus(dt_bias[k]))
    -- the decay index is the contiguous (key) index of the pool."""
    c = _case(seed=4, n=2, H=2, slots=3)
    H = c.H
    A = torch.tensor([0.0, -0.7])
    dtb = torch.linspace(-3.0, 3.0, H * D, dtype=torch.float32)
    st = _np(c.state).astype(np.float64)
    r = _run(c, A_log=A, dt_bias=dtb, g=np.zeros((c.q.shape[0], H, D), np.uint16),
             beta=np.full((c.q.shape[0], H), NEG_INF_BF16), state=st)
    for i in range(c.q.shape[0]):
        slot = int(c.state_indices[i])
        for h in range(H):
            a = math.exp(float(A[h]))
            d = np.array([math.exp(-a * math.log1p(math.exp(float(dtb[h * D + kk]))))
                          for kk in range(D)])
            np.testing.assert_allclose(r["state"][slot, h], st[slot, h] * d[None, :],
                                       rtol=1e-13, atol=0)


def test_half_decay_special_value():
    """A_log=0 and raw+dt_bias=0 give g=-ln 2, i.e. decay exactly 1/2."""
    c = _case(seed=5, n=1, H=1, slots=1)
    st = _np(c.state).astype(np.float64)
    r = _run(c, A_log=torch.zeros(1), dt_bias=torch.zeros(D),
             g=np.zeros((1, 1, D), np.uint16), beta=np.full((1, 1), NEG_INF_BF16), state=st)
    np.testing.assert_allclose(r["state"], st / 2, rtol=1e-15, atol=0)


def test_softplus_extremes():
    """Large |raw| must not overflow: softplus(80) = 80 (+e^-80), softplus(-80) = e^-80."""
    c = _case(seed=6, n=1, H=1, slots=1)
    st = _np(c.state).astype(np.float64)
    for raw, sp in [(80.0, 80.0 + math.exp(-80.0)), (-80.0, math.exp(-80.0))]:
        r = _run(c, A_log=torch.full((1,), -3.0), dt_bias=torch.zeros(D),
                 g=np.full((1, 1, D), _bf16(raw)), beta=np.full((1, 1), NEG_INF_BF16), state=st)
        d = math.exp(-math.exp(-3.0) * sp)
        np.testing.assert_allclose(r["state"], st * d, rtol=1e-14, atol=0)


def test_qk_scale_invariance():
    """L2 normalisation: scaling q and k by c>0 leaves outputs and state
    unchanged up to the epsilon term."""
    c = _case(seed=7)
    r1 = _run(c, state=_np(c.state).astype(np.float64))
    q2 = _bf16(_np(c.q.float()).astype(np.float64) * 4.0)   # x4 is exact in bf16
    k2 = _bf16(_np(c.k.float()).astype(np.float64) * 0.25)
    r2 = _run(c, q=q2, k=k2, state=_np(c.state).astype(np.float64))
    # k/4 turns eps into 16*eps relative to sum k^2 (~128): a relative change of
    # the normalised key below 16e-6/128 ~ 1.3e-7, carried into o and S'.
    tol_o = 1e-6 * np.abs(r1["out64"]).max()
    tol_s = 1e-6 * np.abs(r1["state"]).max()
    np.testing.assert_allclose(r2["out64"], r1["out64"], rtol=0, atol=tol_o)
    np.testing.assert_allclose(r2["state"], r1["state"], rtol=0, atol=tol_s)


def test_null_rows_zero_output_and_untouched_slots():
    c = _case(seed=8, n=6, H=2, slots=8, indices="random", null_rows=2)
    idx = _np(c.state_indices).copy()
    idx[0] = 8          # out of range: treated as null as well
    r = _run(c, state_indices=idx)
    live = {int(s) for s in idx if 0 <= s < 8}
    for i, s in enumerate(idx):
        if not (0 <= s < 8):
            assert not r["out64"][i].any()
            assert not r["out_bf16"][i].any()
    for slot in range(8):
        same = np.array_equal(r["state"][slot], _np(c.state)[slot])
        assert same == (slot not in live)


def test_two_tokens_orthogonal_keys_closed_form():
    """Unit decay, zero state, orthogonal keys e0, e1 and beta logits 0
    (beta = 1/2): S2 = (1/2)(k1 v1^T + k2 v2^T) exactly, o2 = scale/2 (q.k1 v1 + q.k2 v2)."""
    H = 1
    e0 = np.zeros(D); e0[0] = 1.0
    e1 = np.zeros(D); e1[5] = 1.0
    rng = np.random.default_rng(3)
    qv = _bf16(rng.standard_normal((2, H, D)))
    vv = _bf16(rng.standard_normal((2, H, D)))
    kk = _bf16(np.stack([e0, e1])[:, None, :])
    cu = np.array([0, 2], np.int32)
    r = oracle.recurrent(qv, kk, vv, np.zeros((2, H, D), np.uint16), np.zeros((2, H), np.uint16),
                         np.full(H, -np.inf, np.float32), np.zeros(H * D, np.float32),
                         np.zeros((1, H, D, D)), np.array([0], np.int32), cu, l2_eps=0.0)
    v = oracle.bf16_to_f64(vv)
    q = oracle.bf16_to_f64(qv)
    S2 = 0.5 * (np.outer(v[0, 0], e0) + np.outer(v[1, 0], e1))   # [v][k]
    np.testing.assert_allclose(r["state"][0, 0], S2, rtol=0, atol=1e-15)
    qh = q[1, 0] / np.linalg.norm(q[1, 0])
    o2 = SCALE * 0.5 * (qh[0] * v[0, 0] + qh[5] * v[1, 0])
    np.testing.assert_allclose(r["out64"][1, 0], o2, rtol=1e-13, atol=1e-16)


def test_same_key_beta_one_overwrites():
    """Delta rule with beta = 1 and the same key twice: the second value
    replaces the first, o2 = scale (q_hat . k_hat) v2."""
    H = 1
    rng = np.random.default_rng(4)
    kk = _bf16(np.repeat(rng.standard_normal((1, H, D)), 2, axis=0))
    qv = _bf16(rng.standard_normal((2, H, D)))
    vv = _bf16(rng.standard_normal((2, H, D)))
    r = oracle.recurrent(qv, kk, vv, np.zeros((2, H, D), np.uint16),
                         np.full((2, H), POS_INF_BF16), np.full(H, -np.inf, np.float32),
                         np.zeros(H * D, np.float32), np.zeros((1, H, D, D)),
                         np.array([0], np.int32), np.array([0, 2], np.int32), l2_eps=0.0)
    k = oracle.bf16_to_f64(kk)[0, 0]
    kh = k / np.linalg.norm(k)
    q = oracle.bf16_to_f64(qv)[1, 0]
    v2 = oracle.bf16_to_f64(vv)[1, 0]
    np.testing.assert_allclose(r["state"][0, 0], np.outer(v2, kh), rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["out64"][1, 0], SCALE * (q @ kh) / np.linalg.norm(q) * v2,
                               rtol=1e-12, atol=1e-16)


def test_product_form_cross_formulation():
    """The loop oracle against the algebraically different product form
    S' = (I - beta k k^T) D S + beta k v^T (math orientation, K x V) over a
    ragged multi-token batch."""
    lengths = [3, 0, 2, 1]
    c = _case(seed=9, n=4, H=2, slots=6, indices="random", lengths=lengths)
    st = _np(c.state).astype(np.float64)
    r = _run(c, state=st)
    q = _np(c.q.float()).astype(np.float64)
    k = _np(c.k.float()).astype(np.float64)
    v = _np(c.v.float()).astype(np.float64)
    gr = _np(c.g.float()).astype(np.float64)
    br = _np(c.beta.float()).astype(np.float64)
    A = _np(c.A_log).astype(np.float64)
    dtb = _np(c.dt_bias).astype(np.float64)
    cu = _np(c.cu_seqlens)
    pool = st.copy()
    out = np.zeros((cu[-1], c.H, D))
    for i in range(4):
        slot = int(c.state_indices[i])
        for h in range(c.H):
            S = pool[slot, h].T.copy()            # K x V
            for t in range(cu[i], cu[i + 1]):
                x = gr[t, h] + dtb[h * D:(h + 1) * D]
                sp = np.logaddexp(0.0, x)
                dvec = np.exp(-np.exp(A[h]) * sp)
                beta = 0.5 * (1.0 + np.tanh(0.5 * br[t, h]))
                kh, qh = _unit(k[t, h]), _unit(q[t, h])
                S = (np.eye(D) - beta * np.outer(kh, kh)) @ (dvec[:, None] * S) \
                    + beta * np.outer(kh, v[t, h])
                out[t, h] = SCALE * (S.T @ qh)
            pool[slot, h] = S.T
    np.testing.assert_allclose(r["out64"], out, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(r["state"], pool, rtol=1e-10, atol=1e-14)


def test_beta_zero_tokens_read_out_the_cumulatively_decayed_state():
    """beta=0 over a ragged batch: no write ever happens, so after token t of a
    sequence the state is the initial one scaled by the product of that
    sequence's decays so far (per key channel), o_t = scale * q_hat_t^T of that
    state, and the final slot holds the product over all its tokens."""
    lengths = [4, 1, 0, 3]
    c = _case(seed=41, n=4, H=2, slots=6, indices="random", lengths=lengths)
    T, H = c.q.shape[0], c.H
    st = _np(c.state).astype(np.float64)
    r = _run(c, state=st, beta=np.full((T, H), NEG_INF_BF16))
    q = _np(c.q.float()).astype(np.float64)
    gr = _np(c.g.float()).astype(np.float64)
    A = _np(c.A_log).astype(np.float64)
    dtb = _np(c.dt_bias).astype(np.float64).reshape(H, D)
    cu = _np(c.cu_seqlens)
    want_pool = st.copy()
    for i in range(4):
        slot = int(c.state_indices[i])
        toks = np.arange(cu[i], cu[i + 1])
        if toks.size == 0:
            continue
        for h in range(H):
            # log-decay per token and key channel, summed along the sequence
            logd = -np.exp(A[h]) * np.logaddexp(0.0, gr[toks, h] + dtb[h])
            cum = np.exp(np.cumsum(logd, axis=0))          # [tokens, K]
            for j, t in enumerate(toks):
                S_t = st[slot, h] * cum[j][None, :]          # pool orientation [v][k]
                np.testing.assert_allclose(r["out64"][t, h], SCALE * (S_t @ _unit(q[t, h])),
                                           rtol=1e-11, atol=1e-16)
            want_pool[slot, h] = st[slot, h] * cum[-1][None, :]
    np.testing.assert_allclose(r["state"], want_pool, rtol=1e-11, atol=0)


def test_row_permutation_permutes_outputs_and_keeps_pool():
    """Rows are independent: permuting the rows of a call together with their
    slot indices permutes the outputs and leaves every slot of the pool (and
    the conv cache of the fused call) bit for bit the same."""
    c = _case(seed=42, n=7, H=2, slots=10, indices="random", null_rows=2)
    st = _np(c.state).astype(np.float64)
    perm = np.array([3, 6, 0, 5, 1, 4, 2])
    r1 = _run(c, state=st)
    r2 = _run(c, state=st, q=_np(c.q)[perm], k=_np(c.k)[perm], v=_np(c.v)[perm],
              g=_np(c.g)[perm], beta=_np(c.beta)[perm], state_indices=_np(c.state_indices)[perm])
    np.testing.assert_array_equal(r2["out64"], r1["out64"][perm])
    np.testing.assert_array_equal(r2["state"], r1["state"])

    f = _fcase(seed=43, rows=5, H=2, slots=8)
    fperm = np.array([4, 2, 0, 3, 1])
    idx = np.array([3, 0, 7, -1, 5], np.int32)
    f1 = _frun(f, state_indices=idx)
    rows = lambda a: _np(a)[fperm]  # noqa: E731
    f2 = _frun(f, x=rows(f.x), raw_gate=rows(f.raw_gate), raw_beta=rows(f.raw_beta),
               output_gate=rows(f.output_gate), state_indices=idx[fperm])
    np.testing.assert_array_equal(f2["out64"].reshape(5, -1), f1["out64"].reshape(5, -1)[fperm])
    np.testing.assert_array_equal(f2["state"], f1["state"])
    np.testing.assert_array_equal(f2["conv_state"], f1["conv_state"])


def test_varlen_equals_successive_single_steps():
    """A T-token packed step equals T successive T=1 calls (fp64 state: exact),
    and the checkpoints are the successive states."""
    lengths = [4, 0, 1, 3]
    c = _case(seed=10, n=4, H=2, slots=5, indices="random", lengths=lengths)
    st = _np(c.state).astype(np.float64)
    r = _run(c, state=st, ckpt_dtype=oracle.F64)
    cu = _np(c.cu_seqlens)
    idx = _np(c.state_indices)
    pool = st.copy()
    for t_step in range(max(lengths)):
        sel = [i for i in range(4) if lengths[i] > t_step]
        toks = [cu[i] + t_step for i in sel]
        rs = oracle.recurrent(_np(c.q)[toks], _np(c.k)[toks], _np(c.v)[toks], _np(c.g)[toks],
                              _np(c.beta)[toks], c.A_log, c.dt_bias, pool, idx[sel])
        pool = rs["state"]
        np.testing.assert_array_equal(rs["out64"], r["out64"][toks])
        for j, t in enumerate(toks):
            np.testing.assert_array_equal(r["ckpt"][t], pool[idx[sel][j]])
    np.testing.assert_array_equal(r["state"], pool)


def test_empty_sequences_write_nothing():
    c = _case(seed=11, n=3, H=1, slots=4, indices="random", lengths=[0, 0, 0])
    r = _run(c)
    np.testing.assert_array_equal(r["state"], _np(c.state))
    assert r["out64"].size == 0


def test_fp32_state_rounding_is_nearest():
    c = _case(seed=12, n=2, H=1, slots=2)
    r64 = _run(c, state=_np(c.state).astype(np.float64))
    r32 = _run(c)
    np.testing.assert_array_equal(r32["state"], r64["state"].astype(np.float32))
    rb = _run(c, state=_np(c.state.to(torch.bfloat16)))
    rb64 = _run(c, state=oracle.bf16_to_f64(_np(c.state.to(torch.bfloat16))))
    np.testing.assert_array_equal(rb["state"], oracle.bf16_from_f64(rb64["state"]))
    np.testing.assert_array_equal(r32["out_bf16"], oracle.bf16_from_f64(r32["out64"]))


# ---- fused decode: conv, SiLU, gated RMSNorm -------------------------------------------

def _fcase(seed=20, rows=3, H=2, slots=6, **kw):
    return synth.fused_case(seed, rows=rows, H=H, num_slots=slots, **kw)


def _frun(c, **over):
    a = dict(x=c.x, weight=c.weight, conv_state=c.conv_state, raw_gate=c.raw_gate,
             raw_beta=c.raw_beta, A_log=c.A_log, dt_bias=c.dt_bias,
             state_indices=c.state_indices, state=c.state, output_gate=c.output_gate,
             norm_weight=c.norm_weight)
    a.update(over)
    return oracle.fused(**a)


def _silu(y):
    return y / (1.0 + np.exp(-y))


def test_conv_one_hot_taps_reproduce_lagged_inputs():
    """A one-hot conv weight at tap j makes the pre-SiLU conv output the input
    lagged by 3-j; after three calls the cache holds the last three inputs.
    Each of the q, k, v groups uses a different tap to pin the group index."""
    H, rows = 2, 2
    c = _fcase(seed=21, rows=rows, H=H, slots=4)
    C3 = 3 * H * D
    taps = [0, 2, 3]
    w = np.zeros((3, 4, H * D), np.float32)
    for grp, j in enumerate(taps):
        w[grp, j, :] = 1.0
    cs = _np(c.conv_state).copy()
    idx = _np(c.state_indices).copy()
    idx[:] = [1, 3]
    hist = [oracle.bf16_to_f64(cs[idx, :, p]) for p in range(3)]   # oldest first
    rng = np.random.default_rng(5)
    st = _np(c.state)
    for call in range(3):
        x = _bf16(rng.standard_normal((rows, C3)))
        r = _frun(c, x=x, weight=w, conv_state=cs, state=st, state_indices=idx)
        cs, st = r["conv_state"], r["state"]
        hist.append(oracle.bf16_to_f64(x))
        for grp, j in enumerate(taps):
            lagged = hist[-4 + j][:, grp * H * D:(grp + 1) * H * D]
            np.testing.assert_allclose(r["act64"][:, grp * H * D:(grp + 1) * H * D],
                                       _silu(lagged), rtol=1e-14, atol=1e-300)
    for p in range(3):
        np.testing.assert_array_equal(oracle.bf16_to_f64(cs[idx, :, p]), hist[3 + p])


def test_conv_output_feeds_recurrence_as_qkv():
    """The fused recurrence equals the plain recurrence on the conv activations
    (zero state so that S' = beta k_hat v^T is a closed form of act)."""
    H = 2
    c = _fcase(seed=22, rows=2, H=H, slots=3)
    idx = np.array([1, 2], np.int32)
    st = np.zeros((3, H, D, D))
    r = _frun(c, state=st, state_indices=idx)
    act = r["act64"]
    braw = oracle.bf16_to_f64(_np(c.raw_beta))
    for b in range(2):
        for h in range(H):
            q = act[b, h * D:(h + 1) * D]
            k = act[b, H * D + h * D:H * D + (h + 1) * D]
            v = act[b, 2 * H * D + h * D:2 * H * D + (h + 1) * D]
            beta = 1.0 / (1.0 + math.exp(-braw[b, h]))
            qh, kh = _unit(q), _unit(k)
            np.testing.assert_allclose(r["state"][idx[b], h], beta * np.outer(v, kh),
                                       rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(r["o_pre64"][b, h], SCALE * beta * (qh @ kh) * v,
                                       rtol=1e-12, atol=1e-15)


def test_gated_rmsnorm_invariants():
    H = 2
    c = _fcase(seed=23, rows=3, H=H, slots=5)
    eps = 1e-5
    # gate = +inf (sigmoid 1) and unit weight: mean(y^2) = ms / (ms + eps)
    r = _frun(c, output_gate=np.full((3, H, D), POS_INF_BF16), norm_weight=np.ones(D, np.float32))
    ms = (r["o_pre64"] ** 2).mean(-1)
    np.testing.assert_allclose((r["out64"] ** 2).mean(-1), ms / (ms + eps), rtol=1e-12)
    # y is o scaled per head by a positive constant, times w * sigmoid(gate) elementwise
    r = _frun(c)
    gate = oracle.bf16_to_f64(_np(c.output_gate))
    w = _np(c.norm_weight).astype(np.float64)
    ratio = r["out64"] / (w * (1.0 / (1.0 + np.exp(-gate)))) / r["o_pre64"]
    np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-12)
    np.testing.assert_allclose(ratio[..., 0], 1.0 / np.sqrt(ms + eps), rtol=1e-12)
    # gate = -inf: output exactly zero
    r = _frun(c, output_gate=np.full((3, H, D), NEG_INF_BF16))
    assert not np.abs(r["out64"]).any()


def test_fused_null_rows():
    """Non-positive indices (slot 0 is reserved) and out-of-range ones are null:
    zero output, neither cache touched."""
    c = _fcase(seed=24, rows=4, H=1, slots=6)
    idx = np.array([0, 3, -1, 6], np.int32)
    r = _frun(c, state_indices=idx)
    for b in (0, 2, 3):
        assert not r["out64"][b].any() and not r["out_bf16"][b].any()
    cs0, st0 = _np(c.conv_state), _np(c.state)
    for s in range(6):
        assert np.array_equal(r["state"][s], st0[s]) == (s != 3)
        assert np.array_equal(r["conv_state"][s], cs0[s]) == (s != 3)


# ---- grouped value heads, precomputed gate, read-only pool, batched form ----------------

def _gqa_case(seed, n=3, H=2, group=3, slots=5, lengths=None):
    """Inputs with HV = group * H value heads (q, k at H heads)."""
    HV = H * group
    c = synth.recurrent_case(seed, n_seqs=n, H=HV, num_slots=slots, indices="random",
                             lengths=lengths)
    T = c.q.shape[0]
    q = _np(c.q)[:, :H].copy()
    k = _np(c.k)[:, :H].copy()
    return c, q, k, HV


def test_grouped_heads_equal_repeated_qk():
    """HV = 3H value heads reading q/k head hv // 3 equal an equal-head run on
    q and k repeated three times along the head axis (exactly)."""
    for lengths in (None, [2, 0, 3]):
        c, q, k, HV = _gqa_case(30, lengths=lengths)
        a = oracle.recurrent(q, k, c.v, c.g, c.beta, c.A_log, c.dt_bias, _np(c.state).astype(np.float64),
                             c.state_indices, c.cu_seqlens, ckpt_dtype=oracle.F64)
        qr, kr = np.repeat(q, 3, axis=1), np.repeat(k, 3, axis=1)
        b = oracle.recurrent(qr, kr, c.v, c.g, c.beta, c.A_log, c.dt_bias, _np(c.state).astype(np.float64),
                             c.state_indices, c.cu_seqlens, ckpt_dtype=oracle.F64)
        for key in ("out64", "state", "ckpt"):
            np.testing.assert_array_equal(a[key], b[key])
        # and the grouping is hv // group, not hv % H: heads 0..2 share q/k head 0
        c1 = oracle.recurrent(np.stack([q[:, 1], q[:, 0]], 1), np.stack([k[:, 1], k[:, 0]], 1), c.v,
                              c.g, c.beta, c.A_log, c.dt_bias, _np(c.state).astype(np.float64),
                              c.state_indices, c.cu_seqlens)
        assert not np.array_equal(c1["out64"][:, :3], a["out64"][:, :3])
        np.testing.assert_array_equal(c1["out64"][:, :3], oracle.recurrent(
            np.repeat(q[:, 1:2], 2, 1), np.repeat(k[:, 1:2], 2, 1), c.v, c.g, c.beta, c.A_log,
            c.dt_bias, _np(c.state).astype(np.float64), c.state_indices, c.cu_seqlens)["out64"][:, :3])


def test_precomputed_gate_is_log_decay_per_key_channel():
    """Precomputed mode: beta = 0 and a log-decay varying over k scale every
    pool element [v][k] by exp(g_k) (library exp)."""
    c = _case(seed=31, n=2, H=2, slots=3)
    T, H = c.q.shape[0], c.H
    gpre = np.tile(np.linspace(-4.0, 0.0, D, dtype=np.float32), (T, H, 1))
    st = _np(c.state).astype(np.float64)
    r = oracle.recurrent(c.q, c.k, c.v, gpre, np.zeros((T, H), np.float32), None, None, st,
                         c.state_indices, gate="precomputed")
    d = np.array([math.exp(float(x)) for x in gpre[0, 0]])
    for i in range(T):
        slot = int(c.state_indices[i])
        np.testing.assert_allclose(r["state"][slot], st[slot] * d[None, None, :], rtol=1e-15, atol=0)


def test_precomputed_beta_is_used_as_is():
    """Precomputed mode: beta = 1 with unit decay stores v under k exactly;
    zero state with beta = 0.25 gives S' = 0.25 k_hat v^T."""
    c = _case(seed=32, n=3, H=2, slots=4)
    T, H = c.q.shape[0], c.H
    zeros = np.zeros((T, H, D), np.float32)
    r = oracle.recurrent(c.q, c.k, c.v, zeros, np.ones((T, H), np.float32), None, None,
                         _np(c.state).astype(np.float64), c.state_indices, gate="precomputed",
                         l2_eps=0.0)
    k = _np(c.k.float()).astype(np.float64)
    v = _np(c.v.float()).astype(np.float64)
    for i in range(T):
        slot = int(c.state_indices[i])
        for h in range(H):
            kh = k[i, h] / np.linalg.norm(k[i, h])
            np.testing.assert_allclose(r["state"][slot, h] @ kh, v[i, h], rtol=0, atol=1e-12)
    r = oracle.recurrent(c.q, c.k, c.v, zeros, np.full((T, H), 0.25, np.float32), None, None,
                         np.zeros((4, H, D, D)), c.state_indices, gate="precomputed")
    for i in range(T):
        slot = int(c.state_indices[i])
        for h in range(H):
            np.testing.assert_allclose(r["state"][slot, h], 0.25 * np.outer(v[i, h], _unit(k[i, h])),
                                       rtol=1e-12, atol=1e-15)


def test_precomputed_gate_matches_in_kernel_gate_values():
    """Feeding the in-kernel gate's own values (computed here with library
    exp/log1p, rounded to fp32) as precomputed inputs reproduces the
    in-kernel run to fp32 input rounding."""
    c = _case(seed=33, n=3, H=2, slots=4)
    graw = oracle.bf16_to_f64(_np(c.g))
    dtb = _np(c.dt_bias).astype(np.float64).reshape(c.H, D)
    A = _np(c.A_log).astype(np.float64)
    x = graw + dtb[None]
    sp = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
    gpre = (-np.exp(A)[None, :, None] * sp).astype(np.float32)
    bpre = (1.0 / (1.0 + np.exp(-oracle.bf16_to_f64(_np(c.beta))))).astype(np.float32)
    st = _np(c.state).astype(np.float64)
    a = oracle.recurrent(c.q, c.k, c.v, c.g, c.beta, c.A_log, c.dt_bias, st, c.state_indices)
    b = oracle.recurrent(c.q, c.k, c.v, gpre, bpre, None, None, st, c.state_indices, gate="precomputed")
    np.testing.assert_allclose(b["out64"], a["out64"], rtol=0, atol=1e-8)
    np.testing.assert_allclose(b["state"], a["state"], rtol=0, atol=1e-7)


def test_read_only_pool():
    """update_state=False: the pool is bit-identical afterwards; outputs and
    checkpoints equal those of the state-updating call."""
    c = _case(seed=34, n=4, H=2, slots=6, indices="random", lengths=[3, 0, 2, 1], null_rows=1)
    a = _run(c, ckpt_dtype=oracle.F32)
    b = _run(c, ckpt_dtype=oracle.F32, update_state=False)
    np.testing.assert_array_equal(b["state"], _np(c.state))
    np.testing.assert_array_equal(b["out64"], a["out64"])
    np.testing.assert_array_equal(b["ckpt"], a["ckpt"])
    assert not np.array_equal(a["state"], _np(c.state))


def test_batched_form_equals_uniform_cu_seqlens():
    """tokens_per_seq = T without cu_seqlens equals cu_seqlens = [0, T, 2T, ...]."""
    c = _case(seed=35, n=3, H=2, slots=4, indices="random", lengths=[4, 4, 4])
    a = _run(c, ckpt_dtype=oracle.F32)
    b = _run(c, cu_seqlens=None, tokens_per_seq=4, ckpt_dtype=oracle.F32)
    for key in ("out64", "state", "ckpt"):
        np.testing.assert_array_equal(a[key], b[key])


# ---- verify caches: per-token corrections and raw key | gate -----------------------------

def _commit_from_caches(S0, corr, kg, n, gate, A_log=None, dt_bias=None, eps=oracle.L2_EPS):
    """Rebuild the state after the first n tokens of one (slot, head) from the
    caches alone: S_t = D_t S_{t-1} + k_hat_t c_t^T (math orientation K x V)."""
    S = S0.T.copy()
    for t in range(n):
        kraw, graw = kg[t, :D], kg[t, D:]
        kh = kraw / math.sqrt(float((kraw * kraw).sum()) + eps)
        if gate == "in_kernel":
            x = graw + dt_bias
            d = np.exp(-math.exp(A_log) * (np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))))
        else:
            d = np.exp(graw)
        S = d[:, None] * S + np.outer(kh, corr[t])
    return S.T


@pytest.mark.parametrize("gate", ["in_kernel", "precomputed"])
def test_verify_caches_rebuild_every_checkpoint(gate):
    """From the initial state and the two caches alone, every prefix state of
    every live sequence is rebuilt: the correction is exactly the vector the
    delta rule adds along k_hat, and kg holds the key and gate the step used."""
    lengths = [3, 0, 4, 1]
    c = synth.recurrent_case(40, n_seqs=4, H=6, HV=6, num_slots=7, indices="random",
                             lengths=lengths, null_rows=0, gate=gate)
    st0 = _np(c.state).astype(np.float64)
    r = oracle.recurrent(c.q, c.k, c.v, c.g, c.beta, c.A_log, c.dt_bias, st0, c.state_indices,
                         c.cu_seqlens, want_ckpt64=True, gate=gate, update_state=False, t_max=4)
    cu = _np(c.cu_seqlens)
    idx = _np(c.state_indices)
    for i in range(4):
        s = int(idx[i])
        for h in range(6):
            for n in range(1, lengths[i] + 1):
                S = _commit_from_caches(st0[s, h], r["corr"][s, h], r["kg"][s, h], n, gate,
                                        None if gate != "in_kernel" else float(_np(c.A_log)[h]),
                                        None if gate != "in_kernel" else
                                        _np(c.dt_bias)[h * D:(h + 1) * D].astype(np.float64))
                np.testing.assert_allclose(S, r["ckpt64"][cu[i] + n - 1, h], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(r["state"], st0)


def test_verify_caches_positions_and_null_rows():
    """Tokens at positions >= t_max are not recorded; null sequences record
    nothing; the key half of kg is the raw (unnormalised) key of the q/k head."""
    c = synth.recurrent_case(41, n_seqs=3, H=2, HV=4, num_slots=5, indices="random",
                             lengths=[3, 2, 1])
    idx = _np(c.state_indices).copy()
    idx[2] = -1
    r = oracle.recurrent(c.q, c.k, c.v, c.g, c.beta, c.A_log, c.dt_bias,
                         _np(c.state).astype(np.float64), idx, c.cu_seqlens, t_max=2)
    k = oracle.bf16_to_f64(_np(c.k))
    s0, s1 = int(idx[0]), int(idx[1])
    np.testing.assert_array_equal(r["kg"][s0, 3, 1, :D], k[1, 3 // 2])
    assert np.abs(r["corr"][s0, :, :2]).min(axis=-1).max() > 0  # positions 0, 1 recorded
    live = {s0, s1}
    for s in range(5):
        if s not in live:
            assert not r["corr"][s].any() and not r["kg"][s].any()
