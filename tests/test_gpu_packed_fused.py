"""GPU parity of packed_fused_kda_decode (T >= 1 tokens per sequence,
accepted-token start column, per-token conv and state checkpoints) against
the fp64 oracle, and its consistency with fused_kda_decode.

Bars: bf16 outputs and fp32/bf16 checkpoints as for every other call; conv
checkpoints (pure data movement of bf16 inputs), untouched slots and
padding rows bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import fused_kda_decode, packed_fused_kda_decode, synth
from tests import parity as P

pytestmark = pytest.mark.gpu
D = 128
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[case]", *a, flush=True)


def np_(t):
    return None if t is None else oracle.as_np(t.detach().cpu())


def gpu_call(c, *, si=None, acc=None, qsl=None, out=None, ws="auto"):
    return packed_fused_kda_decode(c.x, c.weight, c.conv_state, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias,
                                   c.state_indices if si is None else si, c.state, c.output_gate,
                                   c.norm_weight, output=out,
                                   query_start_loc=c.query_start_loc if qsl is None else qsl,
                                   num_accepted_tokens=c.num_accepted_tokens if acc is None else acc,
                                   workspace=ws)


def ref_call(c, st0, cs0, *, si=None, acc=None):
    return oracle.packed_fused(np_(c.x), np_(c.weight), cs0, np_(c.raw_gate), np_(c.raw_beta), np_(c.A_log),
                               np_(c.dt_bias), np_(c.state_indices) if si is None else si, st0,
                               np_(c.output_gate), np_(c.norm_weight), query_start_loc=np_(c.query_start_loc),
                               num_accepted_tokens=np_(c.num_accepted_tokens) if acc is None else acc)


def check_all(c, out, want, st0):
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
    assert np.array_equal(np_(c.conv_state), want["conv_state"]), "conv cache differs"
    # slots the oracle leaves alone are bit-identical on the GPU as well
    unchanged = [s for s in range(st0.shape[0]) if np.array_equal(want["state"][s], st0[s])]
    g = P.bits(c.state.cpu())
    assert torch.equal(g[unchanged], P.bits(torch.from_numpy(st0) if st0.dtype != np.uint16
                                            else torch.from_numpy(st0.view(np.int16)))[unchanged])


@pytest.mark.parametrize("ws", ["auto", None], ids=["split", "unsplit"])
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_ragged_random_accepted(state_dtype, ws):
    say(f"packed fused ragged H=4 {state_dtype} workspace={ws} seed=8000")
    c = synth.packed_fused_case(8000, lengths=[3, 1, 0, 5, 2], H=4, num_slots=40, max_tokens=5,
                                state_dtype=state_dtype, device=DEV, pad_rows=2)
    st0, cs0 = np_(c.state).copy(), np_(c.conv_state).copy()
    want = ref_call(c, st0, cs0)
    out = torch.full((1, c.x.shape[0], 4, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    gpu_call(c, out=out, ws=ws)
    torch.cuda.synchronize()
    check_all(c, out, want, st0)


@pytest.mark.parametrize("ws", ["auto", None], ids=["split", "unsplit"])
def test_padding_null_sequences_and_checkpoint_columns(ws):
    """The oracle pin's layout on the GPU: a sequence longer than max_tokens,
    a slot-0 and a -1 checkpoint column, an empty sequence, a slot-0 start,
    no accepted token, and two trailing rows (outputs pre-filled with NaN)."""
    say(f"packed fused padding/null H=4 fp32 workspace={ws} seed=8100")
    c = synth.packed_fused_case(8100, lengths=[4, 0, 3, 1, 2], H=4, num_slots=24, max_tokens=3,
                                device=DEV, pad_rows=2)
    si = c.state_indices.clone()
    si[0, 1] = 0
    si[2, 1] = -1
    si[3, 0] = 0
    acc = torch.tensor([1, 1, 3, 1, 0], dtype=torch.int32, device=DEV)
    st0, cs0 = np_(c.state).copy(), np_(c.conv_state).copy()
    want = ref_call(c, st0, cs0, si=np_(si), acc=np_(acc))
    out = torch.full((1, 12, 4, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    gpu_call(c, si=si, acc=acc, out=out, ws=ws)
    torch.cuda.synchronize()
    check_all(c, out, want, st0)
    o = out.reshape(12, -1)
    for row in (7, 8, 9, 10, 11):
        assert torch.equal(P.bits(o[row].cpu()), torch.zeros(4 * D, dtype=torch.int16)), row


@pytest.mark.parametrize("rows", [37, 128])
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_single_token_rows_equal_fused_decode(state_dtype, rows):
    """One token per row, start column = the fused call's index: the state and
    conv caches equal fused_kda_decode's bit for bit (the per-row arithmetic
    is the same).  At 128 rows x 8 heads both calls use 8 value rows per lane
    and the outputs are bitwise equal too; at 37 rows the packed call splits
    each head over two workgroups, whose RMS sum is added in another order,
    so outputs may differ by one bf16 ulp."""
    say(f"packed fused T=1 vs fused_kda_decode H=8 rows={rows} {state_dtype} seed=8200")
    fc = synth.fused_case(8200, rows=rows, H=8, num_slots=192, state_dtype=state_dtype, device=DEV,
                          null_zero=2, null_neg=2)
    st0, cs0 = fc.state.clone(), fc.conv_state.clone()
    o_f = fused_kda_decode(fc.x, fc.weight, fc.conv_state, fc.raw_gate, fc.raw_beta, fc.A_log, fc.dt_bias,
                           fc.state_indices, fc.state, fc.output_gate, fc.norm_weight)
    s_f, c_f = fc.state.clone(), fc.conv_state.clone()
    fc.state.copy_(st0)
    fc.conv_state.copy_(cs0)
    o_p = packed_fused_kda_decode(fc.x, fc.weight, fc.conv_state, fc.raw_gate, fc.raw_beta, fc.A_log,
                                  fc.dt_bias, fc.state_indices.reshape(rows, 1), fc.state, fc.output_gate,
                                  fc.norm_weight,
                                  query_start_loc=torch.arange(rows + 1, dtype=torch.int32, device=DEV),
                                  num_accepted_tokens=torch.ones(rows, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(P.bits(s_f), P.bits(fc.state))
    assert torch.equal(P.bits(c_f), P.bits(fc.conv_state))
    if rows == 128:
        assert torch.equal(P.bits(o_f), P.bits(o_p))
    else:
        a = o_f.float().cpu().numpy().astype(np.float64).ravel()
        b = o_p.float().cpu().numpy().astype(np.float64).ravel()
        assert np.all(np.abs(a - b) <= P.bf16_ulp(a)), "outputs differ by more than one bf16 ulp"


def test_tokens_equal_chained_single_token_calls_bitwise():
    """fp32 pool: the register carry is the fp32 state a single-token call
    would store and reload, so T tokens in one call equal T one-token calls
    that start from the previous token's checkpoint slot, bit for bit."""
    say("packed fused T tokens vs chained T=1 calls H=4 fp32 seed=8300")
    lengths = [4, 2, 3]
    c = synth.packed_fused_case(8300, lengths=lengths, H=4, num_slots=32, max_tokens=4, device=DEV)
    st0, cs0 = c.state.clone(), c.conv_state.clone()
    out = gpu_call(c)
    s_all, c_all = c.state.clone(), c.conv_state.clone()
    c.state.copy_(st0)
    c.conv_state.copy_(cs0)
    si = c.state_indices.cpu()
    acc = c.num_accepted_tokens.cpu()
    qsl = c.query_start_loc.cpu()
    one = torch.ones(1, dtype=torch.int32, device=DEV)
    q01 = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    outs = torch.empty_like(out)
    for i, n in enumerate(lengths):
        prev = int(si[i, int(acc[i]) - 1])
        for j in range(n):
            r = int(qsl[i]) + j
            dst = int(si[i, j])
            if dst != prev:  # the one-token call updates its slot in place
                c.state[dst].copy_(c.state[prev])
                c.conv_state[dst].copy_(c.conv_state[prev])
            o = packed_fused_kda_decode(c.x[r:r + 1], c.weight, c.conv_state, c.raw_gate[r:r + 1],
                                        c.raw_beta[r:r + 1], c.A_log, c.dt_bias,
                                        torch.tensor([[dst]], dtype=torch.int32, device=DEV), c.state,
                                        c.output_gate[r:r + 1], c.norm_weight, query_start_loc=q01,
                                        num_accepted_tokens=one)
            outs[0, r] = o[0, 0]
            prev = dst
    torch.cuda.synchronize()
    assert torch.equal(P.bits(out), P.bits(outs))
    written = {int(si[i, j]) for i, n in enumerate(lengths) for j in range(n)}
    for s in written:
        assert torch.equal(P.bits(s_all[s]), P.bits(c.state[s])), s
        assert torch.equal(P.bits(c_all[s]), P.bits(c.conv_state[s])), s


def test_graph_replay_reads_metadata_on_device():
    """Capture once, then replay with new query_start_loc / num_accepted_tokens
    / state_indices values (a zero-length sequence, other accepted counts):
    every replay equals an eager call with the same values."""
    say("packed fused graph replay with changed metadata H=4 seed=8400")
    c = synth.packed_fused_case(8400, lengths=[2, 2, 2], H=4, num_slots=40, max_tokens=3, device=DEV)
    st0, cs0 = c.state.clone(), c.conv_state.clone()
    out = torch.zeros((1, 6, 4, D), dtype=torch.bfloat16, device=DEV)
    qsl, acc, si = c.query_start_loc.clone(), c.num_accepted_tokens.clone(), c.state_indices.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu_call(c, si=si, acc=acc, qsl=qsl, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_call(c, si=si, acc=acc, qsl=qsl, out=out)
    variants = [([0, 2, 4, 6], [1, 2, 3]), ([0, 1, 1, 3], [3, 1, 2]), ([0, 2, 2, 2], [2, 2, 1])]
    for q, a in variants * 2:
        qsl.copy_(torch.tensor(q, dtype=torch.int32))
        acc.copy_(torch.tensor(a, dtype=torch.int32))
        c.state.copy_(st0)
        c.conv_state.copy_(cs0)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_g, s_g, c_g = out.clone(), c.state.clone(), c.conv_state.clone()
        c.state.copy_(st0)
        c.conv_state.copy_(cs0)
        o_e = gpu_call(c, si=si, acc=acc, qsl=qsl)
        torch.cuda.synchronize()
        assert torch.equal(P.bits(o_g), P.bits(o_e)), (q, a)
        assert torch.equal(P.bits(s_g), P.bits(c.state)), (q, a)
        assert torch.equal(P.bits(c_g), P.bits(c.conv_state)), (q, a)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_speculative_workload_h12_n128_t5(state_dtype):
    """The pages' speculative benchmark shape: H=12, 128 sequences of 5 tokens,
    one accepted token, against the oracle on every element."""
    say(f"packed fused H=12 N=128 T=5 {state_dtype} seed=8500")
    N, T = 128, 5
    c = synth.packed_fused_case(8500, lengths=[T] * N, H=12, num_slots=N * T + 1, max_tokens=T,
                                state_dtype=state_dtype, device=DEV, accepted="one")
    st0, cs0 = np_(c.state).copy(), np_(c.conv_state).copy()
    want = ref_call(c, st0, cs0)
    out = gpu_call(c)
    torch.cuda.synchronize()
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
    assert np.array_equal(np_(c.conv_state), want["conv_state"])


@pytest.mark.parametrize("ws", ["auto", None], ids=["split", "unsplit"])
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_start_columns_past_the_first_eight(state_dtype, ws):
    """max_tokens 12: start columns 9 and 12 (past the first 8 columns, which
    the kernel prefetches with the accepted count) and 1, sequences of 10, 12
    and 3 tokens (two chunks of 8)."""
    say(f"packed fused start columns > 8 H=4 {state_dtype} workspace={ws} seed=8150")
    c = synth.packed_fused_case(8150, lengths=[10, 12, 3], H=4, num_slots=48, max_tokens=12,
                                state_dtype=state_dtype, device=DEV, pad_rows=1)
    acc = torch.tensor([9, 12, 1], dtype=torch.int32, device=DEV)
    st0, cs0 = np_(c.state).copy(), np_(c.conv_state).copy()
    want = ref_call(c, st0, cs0, acc=np_(acc))
    out = torch.full((1, c.x.shape[0], 4, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    gpu_call(c, acc=acc, out=out, ws=ws)
    torch.cuda.synchronize()
    check_all(c, out, want, st0)
