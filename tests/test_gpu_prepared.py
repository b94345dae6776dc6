"""Prepared calls (``prepare``) on the GPU: the same results as the eager
calls, bit for bit, on the current and on another stream, and inside a
captured graph replayed with new inputs written into the bound buffers."""
import pytest
import torch

from gated_delta_rule_decode_amd import packed_kda_decode, prepare, recurrent_kda, synth
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


def test_prepared_packed_equals_eager_on_two_streams():
    say("prepared packed H=12 B=24 bf16 seed=9300")
    c = synth.packed_case(9300, B=24, H=12, num_slots=64, device=DEV, null_rows=3)
    st0 = c.state.clone()
    out = torch.empty((24, 1, 12, D), dtype=torch.bfloat16, device=DEV)
    call = prepare(packed_kda_decode, c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                   c.state_indices, output=out)
    torch.cuda.synchronize()
    assert torch.equal(P.bits(c.state), P.bits(st0)), "prepare must not launch"
    assert call() is out
    torch.cuda.synchronize()
    got_o, got_s = out.clone(), c.state.clone()
    c.state.copy_(st0)
    want = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state, c.state_indices)
    torch.cuda.synchronize()
    assert torch.equal(P.bits(got_o), P.bits(want)) and torch.equal(P.bits(got_s), P.bits(c.state))
    c.state.copy_(st0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    call(stream=side)
    torch.cuda.synchronize()
    assert torch.equal(P.bits(out), P.bits(want)) and torch.equal(P.bits(got_s), P.bits(c.state))


def test_prepared_recurrent_in_a_graph_with_new_inputs():
    """A prepared T=1 call captured into a graph; each replay, after new
    token inputs and slot indices are copied into the bound buffers, equals
    an eager call on the same values."""
    B, H, S = 16, 8, 48
    say(f"prepared recurrent in a graph B={B} H={H} seed=9310")
    c = synth.recurrent_case(9310, n_seqs=B, H=H, num_slots=S, device=DEV, indices="random")
    r = lambda t: t.reshape(B, 1, *t.shape[1:])  # noqa: E731
    bufs = [r(c.q).clone(), r(c.k).clone(), r(c.v).clone(), r(c.g).clone(), r(c.beta).clone()]
    idx = c.state_indices.clone()
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
    call = prepare(recurrent_kda, *bufs, c.A_log, c.dt_bias, initial_state=c.state, state_indices=idx, output=out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9311)
    for rep in range(3):
        for b in bufs:
            b.copy_(torch.randn(b.shape, generator=gen, device=DEV).to(b.dtype))
        idx.copy_(torch.randperm(S, generator=gen, device=DEV)[:B].to(torch.int32))
        st0 = c.state.clone()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, s_g = out.clone(), c.state.clone()
        c.state.copy_(st0)
        o_e = recurrent_kda(*bufs, c.A_log, c.dt_bias, initial_state=c.state, state_indices=idx)
        torch.cuda.synchronize()
        assert torch.equal(P.bits(o_g), P.bits(o_e)), f"replay {rep}: outputs differ"
        assert torch.equal(P.bits(s_g), P.bits(c.state)), f"replay {rep}: pools differ"
