"""Independent calls on separate streams, in flight together, give exactly
what they give one after another: the library keeps no hidden state between
calls (the packed fused call gets a workspace of its own on its stream, as
its documentation requires for concurrent calls).
"""
import pytest
import torch

from gated_delta_rule_decode_amd import (PackedFusedWorkspace, fused_kda_decode, packed_fused_kda_decode,
                                         recurrent_kda, synth)
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


def make_calls():
    rc = synth.recurrent_case(9950, n_seqs=64, H=8, num_slots=96, device=DEV, indices="random", null_rows=3)
    fc = synth.fused_case(9951, rows=48, H=8, num_slots=64, device=DEV, null_zero=2, null_neg=2)
    pc = synth.packed_fused_case(9952, lengths=[5, 3, 0, 6], H=8, num_slots=40, max_tokens=6, device=DEV)
    ws = PackedFusedWorkspace(DEV)
    r4 = lambda t: t.reshape(64, 1, *t.shape[1:])  # noqa: E731

    def rec():
        return recurrent_kda(r4(rc.q), r4(rc.k), r4(rc.v), r4(rc.g), rc.beta.reshape(64, 1, 8), rc.A_log,
                             rc.dt_bias, initial_state=rc.state, state_indices=rc.state_indices)

    def fused():
        return fused_kda_decode(fc.x, fc.weight, fc.conv_state, fc.raw_gate, fc.raw_beta, fc.A_log, fc.dt_bias,
                                fc.state_indices, fc.state, fc.output_gate, fc.norm_weight)

    def packed_fused():
        return packed_fused_kda_decode(pc.x, pc.weight, pc.conv_state, pc.raw_gate, pc.raw_beta, pc.A_log,
                                       pc.dt_bias, pc.state_indices, pc.state, pc.output_gate, pc.norm_weight,
                                       query_start_loc=pc.query_start_loc,
                                       num_accepted_tokens=pc.num_accepted_tokens, workspace=ws)

    buffers = [rc.state, fc.state, fc.conv_state, pc.state, pc.conv_state]
    return [rec, fused, packed_fused], buffers


def test_concurrent_streams_equal_serial_calls():
    say("three independent calls on three streams vs serial, seeds 9950-9952")
    calls, buffers = make_calls()
    start = [b.clone() for b in buffers]
    torch.cuda.synchronize()
    serial = [P.bits(f()).clone() for f in calls]
    torch.cuda.synchronize()
    after_serial = [P.bits(b).clone() for b in buffers]
    for rounds in range(3):
        for b, s in zip(buffers, start):
            b.copy_(s)
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream() for _ in calls]
        outs = []
        for st, f in zip(streams, calls):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                outs.append(f())
        torch.cuda.synchronize()
        for i, (o, s) in enumerate(zip(outs, serial)):
            assert torch.equal(P.bits(o), s), f"call {i} output differs when run concurrently (round {rounds})"
        for i, (b, s) in enumerate(zip(buffers, after_serial)):
            assert torch.equal(P.bits(b), s), f"buffer {i} differs when run concurrently (round {rounds})"
