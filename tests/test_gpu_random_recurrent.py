"""Seeded random recurrent_kda calls against the fp64 oracle ("flashinfer.
kda_decode" function table and Frozen / speculative-verify mode): T=1 or
ragged, H and grouped value heads, in-kernel or precomputed gate (bf16 or
fp32), null rows, fp32 or bf16 pools, with or without per-token
checkpoints, verify caches and a read-only pool, drawn from a fixed seed per
case so that combinations the hand-written tests do not pair up are
covered too.  Bars as everywhere: bf16 outputs 2e-3 + 2^-8|ref|, fp32 state
1e-4, bf16 state 4e-3, caches as in the verify tests.
"""
import random

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import recurrent_kda, synth
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


@pytest.mark.parametrize("seed", range(24))
def test_random_recurrent_calls(seed):
    rng = random.Random(6000 + seed)
    H = rng.choice([1, 2, 4, 8, 16])
    HV = H * rng.choice([1, 1, 2, 4])
    N = rng.randint(1, 24)
    ragged = rng.random() < 0.6
    lengths = [rng.randint(0, 7) for _ in range(N)] if ragged else None
    if ragged and sum(lengths) == 0:
        lengths[0] = 1
    state_dtype = rng.choice([torch.float32, torch.bfloat16])
    gate = rng.choice(["in_kernel", "precomputed"])
    gate_dtype = rng.choice([torch.float32, torch.bfloat16])
    read_only = rng.random() < 0.3
    ckpt = ragged and rng.random() < 0.5
    t_max = rng.choice([0, 0, 2, 4]) if ragged else rng.choice([0, 1])
    kg_dtype = rng.choice([torch.float32, torch.bfloat16])
    null_rows = rng.randint(0, min(3, N - 1)) if N > 1 else 0
    declared = None  # a read-only ragged call may declare its longest sequence (up to 16 take the WY product)
    if ragged and read_only and rng.random() < 0.6:
        if rng.random() < 0.5:
            lengths = [rng.randint(0, 16) for _ in range(N)]
            if sum(lengths) == 0:
                lengths[0] = 1
        declared = max(lengths) + rng.choice([0, 0, 1, 4])
    S = N + 8
    say(f"random recurrent seed={seed} H={H} HV={HV} N={N} lengths={lengths} {state_dtype} gate={gate}/"
        f"{gate_dtype} read_only={read_only} ckpt={ckpt} t_max={t_max} null_rows={null_rows} "
        f"max_seqlen={declared}")
    c = synth.recurrent_case(6000 + seed, n_seqs=N, H=H, HV=HV, num_slots=S, state_dtype=state_dtype, device=DEV,
                             indices="random", lengths=lengths, null_rows=null_rows, gate=gate,
                             gate_dtype=gate_dtype)
    T = c.q.shape[0]
    st0 = c.state.clone()
    want = oracle.recurrent(np_(c.q), np_(c.k), np_(c.v), np_(c.g), np_(c.beta), np_(c.A_log), np_(c.dt_bias),
                            np_(st0), np_(c.state_indices), np_(c.cu_seqlens) if ragged else None,
                            gate=gate, update_state=not read_only, t_max=t_max or None,
                            ckpt_dtype=(oracle.BF16 if state_dtype == torch.bfloat16 else oracle.F32) if ckpt
                            else None)
    shp = (lambda t: t.reshape(1, T, *t.shape[1:])) if ragged else (lambda t: t.reshape(T, 1, *t.shape[1:]))
    ck = torch.zeros((T, HV, D, D), dtype=state_dtype, device=DEV) if ckpt else None
    corr = torch.zeros((S, HV, t_max, D), dtype=torch.float32, device=DEV) if t_max else None
    kg = torch.zeros((S, HV, t_max, 2 * D), dtype=kg_dtype, device=DEV) if t_max else None
    out = recurrent_kda(shp(c.q), shp(c.k), shp(c.v), shp(c.g), shp(c.beta), c.A_log, c.dt_bias,
                        initial_state=c.state, state_indices=c.state_indices,
                        cu_seqlens=c.cu_seqlens if ragged else None, intermediate_states=ck,
                        disable_state_update=read_only, correction_cache=corr, kg_cache=kg, max_seqlen=declared)
    torch.cuda.synchronize()
    P.check_bf16_out(out, want["out64"])
    if read_only:
        assert torch.equal(P.bits(st0), P.bits(c.state)), "read-only pool changed"
    else:
        P.check_state(c.state, want["state"])
    if ckpt:
        idx = c.state_indices.cpu().numpy()
        cu = c.cu_seqlens.cpu().numpy()
        live = np.zeros(T, bool)  # checkpoints of live sequences' tokens
        for i in range(N):
            if 0 <= idx[i] < S:
                live[cu[i]:cu[i + 1]] = True
        if live.any():
            P.check_state(ck[torch.from_numpy(live).to(DEV)], want["ckpt"][live], what="checkpoints")
    if t_max:
        got_c = corr.cpu().numpy().astype(np.float64)
        assert np.abs(got_c - want["corr"]).max() <= P.F32_STATE_ATOL, "correction cache"
        if kg_dtype == torch.float32:
            assert np.array_equal(kg.cpu().numpy(), want["kg"].astype(np.float32)), "kg cache"
        else:
            got = P.bits(kg.cpu()).numpy().astype(np.uint16)
            rec = np.abs(want["kg"]).sum(-1) > 0  # recorded rows; zero elsewhere on both sides
            assert np.array_equal(got[rec], oracle.bf16_from_f64(want["kg"])[rec]), "kg cache (bf16)"
            assert np.all(got[~rec] == 0)


@pytest.mark.parametrize("seed", range(12))
def test_random_batched_calls(seed):
    """The batched [B, T, ...] form with 2..16 tokens: read-only calls
    without checkpoints take the WY verify kernel's matrix product, the rest
    the token loop; both against the oracle with the same bars."""
    rng = random.Random(6100 + seed)
    H = rng.choice([1, 2, 4, 8])
    HV = H * rng.choice([1, 2, 3])
    N = rng.randint(1, 20)
    T = rng.randint(2, 16)
    state_dtype = rng.choice([torch.float32, torch.bfloat16])
    gate = rng.choice(["in_kernel", "precomputed"])
    gate_dtype = rng.choice([torch.float32, torch.bfloat16])
    read_only = rng.random() < 0.7
    ckpt = rng.random() < 0.25
    t_max = rng.choice([0, 1, T, T + 3])
    kg_dtype = rng.choice([torch.float32, torch.bfloat16])
    null_rows = rng.randint(0, min(2, N - 1)) if N > 1 else 0
    S = N + 6
    say(f"random batched seed={seed} H={H} HV={HV} N={N} T={T} {state_dtype} gate={gate}/{gate_dtype} "
        f"read_only={read_only} ckpt={ckpt} t_max={t_max} null_rows={null_rows}")
    c = synth.recurrent_case(6100 + seed, n_seqs=N, H=H, HV=HV, num_slots=S, state_dtype=state_dtype, device=DEV,
                             indices="random", lengths=[T] * N, null_rows=null_rows, gate=gate,
                             gate_dtype=gate_dtype)
    st0 = c.state.clone()
    want = oracle.recurrent(np_(c.q), np_(c.k), np_(c.v), np_(c.g), np_(c.beta), np_(c.A_log), np_(c.dt_bias),
                            np_(st0), np_(c.state_indices), None, gate=gate, update_state=not read_only,
                            tokens_per_seq=T, t_max=t_max or None,
                            ckpt_dtype=(oracle.BF16 if state_dtype == torch.bfloat16 else oracle.F32) if ckpt
                            else None)
    shp = lambda t: t.reshape(N, T, *t.shape[1:])  # noqa: E731
    ck = torch.zeros((N * T, HV, D, D), dtype=state_dtype, device=DEV) if ckpt else None
    corr = torch.zeros((S, HV, t_max, D), dtype=torch.float32, device=DEV) if t_max else None
    kg = torch.zeros((S, HV, t_max, 2 * D), dtype=kg_dtype, device=DEV) if t_max else None
    out = recurrent_kda(shp(c.q), shp(c.k), shp(c.v), shp(c.g), shp(c.beta), c.A_log, c.dt_bias,
                        initial_state=c.state, state_indices=c.state_indices, intermediate_states=ck,
                        disable_state_update=read_only, correction_cache=corr, kg_cache=kg)
    torch.cuda.synchronize()
    P.check_bf16_out(out, want["out64"])
    if read_only:
        assert torch.equal(P.bits(st0), P.bits(c.state)), "read-only pool changed"
    else:
        P.check_state(c.state, want["state"])
    if ckpt:
        idx = c.state_indices.cpu().numpy()
        live = np.repeat([0 <= i < S for i in idx], T)
        if live.any():
            P.check_state(ck[torch.from_numpy(live).to(DEV)], want["ckpt"][live], what="checkpoints")
    if t_max:
        got_c = corr.cpu().numpy().astype(np.float64)
        assert np.abs(got_c - want["corr"]).max() <= P.F32_STATE_ATOL, "correction cache"
        if kg_dtype == torch.float32:
            assert np.array_equal(kg.cpu().numpy(), want["kg"].astype(np.float32)), "kg cache"
        else:
            got = P.bits(kg.cpu()).numpy().astype(np.uint16)
            rec = np.abs(want["kg"]).sum(-1) > 0
            assert np.array_equal(got[rec], oracle.bf16_from_f64(want["kg"])[rec]), "kg cache (bf16)"
            assert np.all(got[~rec] == 0)
