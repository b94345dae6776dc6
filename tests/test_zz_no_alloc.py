"""The allocation-free packed fused entry point (kda_packed_fused_decode_noalloc)
against the workspace entry point (kda_packed_fused_decode) and the fp64
oracle, through the C ABI.

Two calls in a row, the second smaller (so the library's scratch array holds
the first call's contents when the second starts): each splits its heads, and
each equals the workspace entry point bit for bit (same geometry, same
kernel) and the oracle within the parity bar.  A call whose split would need
more scratch than the library holds is rejected before anything runs.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import (KDAError, PackedFusedWorkspace, packed_fused_kda_decode,
                                         packed_fused_kda_decode_noalloc, synth)
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
    return oracle.as_np(t.detach().cpu())


def _args(c):
    return (c.x, c.weight, c.conv_state, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state_indices, c.state,
            c.output_gate, c.norm_weight)


def test_noalloc_equals_the_workspace_entry_point_on_two_calls():
    for seed, lengths, dtype in ((9100, [5, 3, 4], torch.float32), (9101, [2], torch.bfloat16)):
        say(f"noalloc packed fused H=12 lengths={lengths} {dtype} seed={seed}")
        c = synth.packed_fused_case(seed, lengths=lengths, H=12, num_slots=32, max_tokens=5, state_dtype=dtype,
                                    device=DEV, pad_rows=1)
        st0, cs0 = c.state.clone(), c.conv_state.clone()
        want = oracle.packed_fused(np_(c.x), np_(c.weight), np_(cs0).copy(), np_(c.raw_gate), np_(c.raw_beta),
                                   np_(c.A_log), np_(c.dt_bias), np_(c.state_indices), np_(st0).copy(),
                                   np_(c.output_gate), np_(c.norm_weight), query_start_loc=np_(c.query_start_loc),
                                   num_accepted_tokens=np_(c.num_accepted_tokens))
        rows = c.x.shape[0]
        out_n = torch.full((1, rows, 12, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        packed_fused_kda_decode_noalloc(*_args(c), output=out_n, query_start_loc=c.query_start_loc,
                                        num_accepted_tokens=c.num_accepted_tokens)
        torch.cuda.synchronize()
        s_n, c_n = c.state.clone(), c.conv_state.clone()
        P.check_bf16_out(out_n, want["out64"])
        P.check_state(s_n, want["state"])
        assert np.array_equal(np_(c_n), want["conv_state"]), "conv cache differs from the oracle"
        c.state.copy_(st0)
        c.conv_state.copy_(cs0)
        ws = PackedFusedWorkspace(DEV)
        out_w = packed_fused_kda_decode(*_args(c), query_start_loc=c.query_start_loc,
                                        num_accepted_tokens=c.num_accepted_tokens, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(P.bits(out_n), P.bits(out_w)), "outputs differ from the workspace entry point"
        assert torch.equal(P.bits(s_n), P.bits(c.state)), "pools differ from the workspace entry point"
        assert torch.equal(P.bits(c_n), P.bits(c.conv_state)), "conv caches differ from the workspace entry point"
        assert int(ws.counters.abs().sum()) == 0


def test_noalloc_rejects_a_split_larger_than_its_scratch():
    """One sequence of 700 tokens at H=12 splits its heads (12 pairs) and
    would need 700*12 > 8192 (row, head) pairs of outputs: KDA_ERR_SHAPE,
    and nothing is written."""
    say("noalloc packed fused oversized split H=12 lengths=[700] seed=9102")
    c = synth.packed_fused_case(9102, lengths=[700], H=12, num_slots=4, max_tokens=2, device=DEV)
    st0, cs0 = c.state.clone(), c.conv_state.clone()
    out = torch.zeros((1, 700, 12, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(KDAError) as e:
        packed_fused_kda_decode_noalloc(*_args(c), output=out, query_start_loc=c.query_start_loc,
                                        num_accepted_tokens=c.num_accepted_tokens)
    assert e.value.code == "KDA_ERR_SHAPE"
    torch.cuda.synchronize()
    assert torch.equal(P.bits(st0), P.bits(c.state)) and torch.equal(P.bits(cs0), P.bits(c.conv_state))
    assert not P.bits(out).any()
