"""Split heads in packed_fused_kda_decode ("feat(kda): add fused speculative
decode kernel" workload at small batch): with a workspace, few (sequence,
head) pairs spread each head over 4 or 2 workgroups, and the last part of
a head to finish applies the gated RMSNorm to all of it.

Checked against the fp64 oracle on every element, against the unsplit
kernel (pools and conv caches bit for bit; outputs within one bf16 ulp, since
only the summation order of the RMS norm differs), for counters that are
zero after every call, and for one workspace shared by calls of different
sizes (the second smaller), sequences longer than one chunk of tokens
included.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import PackedFusedWorkspace, packed_fused_kda_decode, synth
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


def gpu_call(c, ws):
    return packed_fused_kda_decode(c.x, c.weight, c.conv_state, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias,
                                   c.state_indices, c.state, c.output_gate, c.norm_weight,
                                   query_start_loc=c.query_start_loc, num_accepted_tokens=c.num_accepted_tokens,
                                   workspace=ws)


def ref_call(c, st0, cs0):
    return oracle.packed_fused(np_(c.x), np_(c.weight), cs0, np_(c.raw_gate), np_(c.raw_beta), np_(c.A_log),
                               np_(c.dt_bias), np_(c.state_indices), st0, np_(c.output_gate),
                               np_(c.norm_weight), query_start_loc=np_(c.query_start_loc),
                               num_accepted_tokens=np_(c.num_accepted_tokens))


def check_vs_oracle(c, out, want):
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
    assert np.array_equal(np_(c.conv_state), want["conv_state"]), "conv cache differs"


def within_one_ulp(a_t, b_t):
    a = a_t.float().cpu().numpy().astype(np.float64).ravel()
    b = b_t.float().cpu().numpy().astype(np.float64).ravel()
    return bool(np.all(np.abs(a - b) <= P.bf16_ulp(a)))


@pytest.mark.parametrize("N", [1, 3, 8])
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_split_matches_oracle_and_unsplit(state_dtype, N):
    """H=12, N sequences of 5 tokens with random accepted counts (the small
    batches of the speculative benchmark: 4-, 4- and 2-way splits with a
    bf16 pool, 4-, 2-way and unsplit with fp32)."""
    say(f"packed fused split H=12 N={N} T=5 {state_dtype} seed={8600 + N}")
    c = synth.packed_fused_case(8600 + N, lengths=[5] * N, H=12, num_slots=5 * N + 1, max_tokens=5,
                                state_dtype=state_dtype, device=DEV)
    st0, cs0 = c.state.clone(), c.conv_state.clone()
    want = ref_call(c, np_(st0).copy(), np_(cs0).copy())
    ws = PackedFusedWorkspace(DEV)
    out_s = gpu_call(c, ws)
    torch.cuda.synchronize()
    check_vs_oracle(c, out_s, want)
    assert int(ws.counters.abs().sum()) == 0, "arrival counters not left at zero"
    s_s, c_s = c.state.clone(), c.conv_state.clone()
    c.state.copy_(st0)
    c.conv_state.copy_(cs0)
    out_u = gpu_call(c, None)
    torch.cuda.synchronize()
    assert torch.equal(P.bits(s_s), P.bits(c.state)), "split and unsplit pools differ"
    assert torch.equal(P.bits(c_s), P.bits(c.conv_state)), "split and unsplit conv caches differ"
    assert within_one_ulp(out_u, out_s), "split and unsplit outputs differ by more than one bf16 ulp"


def test_workspace_shared_by_calls_of_different_sizes():
    """One workspace, three calls in a row: 8 sequences, then a ragged batch
    with an empty sequence, then two long sequences (9 and 12 tokens, past
    one chunk of 8, max_tokens 6 so late tokens write no checkpoint)."""
    ws = PackedFusedWorkspace(DEV)
    for seed, lengths, tmax, dtype in ((8700, [5] * 8, 5, torch.float32),
                                       (8701, [2, 0, 6, 1], 6, torch.bfloat16),
                                       (8702, [9, 12], 6, torch.float32)):
        say(f"packed fused shared workspace H=8 lengths={lengths} {dtype} seed={seed}")
        c = synth.packed_fused_case(seed, lengths=lengths, H=8, num_slots=64, max_tokens=tmax,
                                    state_dtype=dtype, device=DEV, pad_rows=1)
        want = ref_call(c, np_(c.state).copy(), np_(c.conv_state).copy())
        out = gpu_call(c, ws)
        torch.cuda.synchronize()
        check_vs_oracle(c, out, want)
        assert int(ws.counters.abs().sum()) == 0, "arrival counters not left at zero"


def test_repeated_calls_give_identical_results():
    """The same call five times from the same inputs: outputs, pool and conv
    cache bit for bit the same each time (no state leaks through the
    workspace from one call to the next)."""
    say("packed fused split repeated H=12 N=4 seed=8800")
    c = synth.packed_fused_case(8800, lengths=[5, 3, 7, 2], H=12, num_slots=40, max_tokens=7, device=DEV)
    st0, cs0 = c.state.clone(), c.conv_state.clone()
    ws = PackedFusedWorkspace(DEV)
    first = None
    for _ in range(5):
        c.state.copy_(st0)
        c.conv_state.copy_(cs0)
        out = gpu_call(c, ws)
        torch.cuda.synchronize()
        got = (P.bits(out).clone(), P.bits(c.state).clone(), P.bits(c.conv_state).clone())
        if first is None:
            first = got
        else:
            assert all(torch.equal(a, b) for a, b in zip(first, got))
    assert int(ws.counters.abs().sum()) == 0


@pytest.mark.parametrize("H", [12, 24])  # 4- and 2-way splits
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_checkpoints_into_the_start_slot(state_dtype, H):
    """Every part of a split head reads the start slot's q and k conv
    windows, so checkpoints written back into that slot must wait for all of
    them: sequences whose every column is the start slot, whose start column
    is repeated later, and whose later column (not the start) is reused."""
    say(f"packed fused split checkpoints into the start slot H={H} {state_dtype} seed=8900")
    lengths = [5, 4, 6, 3, 5]
    c = synth.packed_fused_case(8900, lengths=lengths, H=H, num_slots=64, max_tokens=6,
                                state_dtype=state_dtype, device=DEV)
    si = c.state_indices.clone()
    acc = torch.tensor([1, 2, 3, 1, 4], dtype=torch.int32, device=DEV)
    si[0, :] = si[0, 0]            # all columns = the start slot
    si[1, 3] = si[1, 1]            # start column (a=2) written again at token 3
    si[2, 4] = si[2, 5]            # a reused column that is not the start
    si[3, 2] = si[3, 0]            # a=1: tokens 0 and 2 both land in the start slot
    c.state_indices.copy_(si)
    c.num_accepted_tokens.copy_(acc)
    st0, cs0 = c.state.clone(), c.conv_state.clone()
    want = ref_call(c, np_(st0).copy(), np_(cs0).copy())
    out = gpu_call(c, PackedFusedWorkspace(DEV))
    torch.cuda.synchronize()
    check_vs_oracle(c, out, want)
    s_s, c_s = c.state.clone(), c.conv_state.clone()
    c.state.copy_(st0)
    c.conv_state.copy_(cs0)
    out_u = gpu_call(c, None)
    torch.cuda.synchronize()
    assert torch.equal(P.bits(s_s), P.bits(c.state))
    assert torch.equal(P.bits(c_s), P.bits(c.conv_state))
    assert within_one_ulp(out_u, out)


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations(seed):
    """Seeded random packed fused calls against the oracle, split and
    unsplit: H in 1..24, 1..12 sequences of 0..11 tokens, 1..9 checkpoint
    columns, accepted counts in 0..columns+1 (0 and columns+1 make a sequence
    null), some columns repeating the start slot or set to 0/-1, 0..2 padding
    rows, fp32 or bf16 pools."""
    import random
    rng = random.Random(5000 + seed)
    H = rng.choice([1, 2, 4, 8, 12, 16, 24])
    N = rng.randint(1, 12)
    lengths = [rng.choice([0, 1, 2, 3, 5, 8, 9, 11]) for _ in range(N)]
    T_max = rng.randint(1, 9)
    dtype = rng.choice([torch.float32, torch.bfloat16])
    pad = rng.randint(0, 2)
    say(f"packed fused random seed={seed} H={H} lengths={lengths} max_tokens={T_max} {dtype} pad={pad}")
    c = synth.packed_fused_case(5000 + seed, lengths=lengths, H=H, num_slots=N * T_max + 8, max_tokens=T_max,
                                state_dtype=dtype, device=DEV, pad_rows=pad)
    si = c.state_indices.clone()
    acc = torch.tensor([rng.randint(0, T_max + 1) for _ in range(N)], dtype=torch.int32)
    for i in range(N):
        r = rng.random()
        a = int(acc[i])
        if r < 0.2 and 1 <= a <= T_max:
            si[i, rng.randrange(T_max)] = si[i, a - 1]       # a column repeats the start slot
        elif r < 0.35:
            si[i, rng.randrange(T_max)] = rng.choice([0, -1])  # a column that checkpoints nothing
    c.state_indices.copy_(si)
    c.num_accepted_tokens.copy_(acc.to(DEV))
    st0, cs0 = c.state.clone(), c.conv_state.clone()
    want = ref_call(c, np_(st0).copy(), np_(cs0).copy())
    results = []
    for ws in (PackedFusedWorkspace(DEV), None):
        c.state.copy_(st0)
        c.conv_state.copy_(cs0)
        out = gpu_call(c, ws)
        torch.cuda.synchronize()
        check_vs_oracle(c, out, want)
        results.append((out.clone(), P.bits(c.state).clone(), P.bits(c.conv_state).clone()))
        if ws is not None:
            assert int(ws.counters.abs().sum()) == 0
    (o_s, s_s, c_s), (o_u, s_u, c_u) = results
    assert torch.equal(s_s, s_u) and torch.equal(c_s, c_u), "split and unsplit caches differ"
    assert within_one_ulp(o_u, o_s)


@pytest.mark.parametrize("ws_kind", ["explicit", "auto"])
def test_captured_call_survives_a_larger_eager_call(ws_kind):
    """A small split call is captured into a graph; then a larger eager call
    makes the workspace grow (the explicit workspace is the same object; the
    default one is the capture stream's, grown here by an eager call on that
    stream), and other allocations of the freed sizes follow; every replay of
    the graph still matches the oracle."""
    say(f"packed fused graph capture then workspace growth ws={ws_kind} H=12 N=2 seed=8950")
    small = synth.packed_fused_case(8950, lengths=[5, 4], H=12, num_slots=16, max_tokens=5, device=DEV)
    st0, cs0 = small.state.clone(), small.conv_state.clone()
    want = ref_call(small, np_(st0).copy(), np_(cs0).copy())
    ws = PackedFusedWorkspace(DEV) if ws_kind == "explicit" else "auto"
    out = torch.zeros((1, small.x.shape[0], 12, D), dtype=torch.bfloat16, device=DEV)

    def call():
        packed_fused_kda_decode(small.x, small.weight, small.conv_state, small.raw_gate, small.raw_beta,
                                small.A_log, small.dt_bias, small.state_indices, small.state, small.output_gate,
                                small.norm_weight, output=out, query_start_loc=small.query_start_loc,
                                num_accepted_tokens=small.num_accepted_tokens, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        call()
    big = synth.packed_fused_case(8951, lengths=[5] * 8, H=12, num_slots=48, max_tokens=5,
                                  state_dtype=torch.bfloat16, device=DEV)
    want_big = ref_call(big, np_(big.state).copy(), np_(big.conv_state).copy())
    for rep in range(3):
        if rep == 1:
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):  # the capture stream's default workspace grows
                out_big = gpu_call(big, ws)  # 96 pairs of a bf16 pool: a 2-way split with more rows
            torch.cuda.synchronize()
            check_vs_oracle(big, out_big, want_big)
            junk = [torch.full((n,), 7.0, device=DEV) for n in (24, 12 * 10 * D, 96, 40 * 12 * D)]
        small.state.copy_(st0)
        small.conv_state.copy_(cs0)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        check_vs_oracle(small, out, want)
    del junk
