"""GPU parity of the wider recurrent_kda modes against the fp64 oracle:
grouped value heads (HV a multiple of H), the precomputed-gate mode, the
uniform batched [B, T, ...] form and the read-only (speculative verify)
pool."""
import math

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


def run(c, *, form, ckpt=False, read_only=False, tps=None):
    """form: 't1' ([B,1,..]), 'ragged' ([1,T,..] + cu_seqlens), 'batched' ([B,T,..])."""
    T = c.q.shape[0]
    if form == "t1":
        shp = lambda t: t.reshape(T, 1, *t.shape[1:])  # noqa: E731
        cu = None
    elif form == "ragged":
        shp = lambda t: t.reshape(1, T, *t.shape[1:])  # noqa: E731
        cu = c.cu_seqlens
    else:
        B = T // tps
        shp = lambda t: t.reshape(B, tps, *t.shape[1:])  # noqa: E731
        cu = None
    HV = c.v.shape[1]
    ck = torch.zeros((T, HV, D, D), dtype=c.state.dtype, device=DEV) if ckpt else None
    out = recurrent_kda(shp(c.q), shp(c.k), shp(c.v), shp(c.g), shp(c.beta), c.A_log, c.dt_bias,
                        initial_state=c.state, state_indices=c.state_indices, cu_seqlens=cu,
                        intermediate_states=ck, disable_state_update=read_only)
    torch.cuda.synchronize()
    return out, ck


def ref(c, st, *, ckpt_dtype=None, read_only=False, tps=1, ragged=False):
    return oracle.recurrent(np_(c.q), np_(c.k), np_(c.v), np_(c.g), np_(c.beta), np_(c.A_log),
                            np_(c.dt_bias), st, np_(c.state_indices),
                            np_(c.cu_seqlens) if ragged else None, ckpt_dtype=ckpt_dtype,
                            gate="in_kernel" if c.A_log is not None else "precomputed",
                            update_state=not read_only, tokens_per_seq=tps)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("H,HV", [(4, 16), (2, 6), (16, 32)])
def test_grouped_value_heads_t1(H, HV, state_dtype):
    say(f"grouped heads T=1 H={H} HV={HV} {state_dtype} seed=6000")
    N = 37
    c = synth.recurrent_case(6000 + HV, n_seqs=N, H=H, HV=HV, num_slots=64, state_dtype=state_dtype,
                             device=DEV, indices="random", null_rows=3)
    st0 = c.state.clone()
    want = ref(c, np_(st0))
    out, _ = run(c, form="t1")
    assert tuple(out.shape) == (N, 1, HV, D)
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
    live = sorted(int(i) for i in c.state_indices.tolist() if i >= 0)
    assert set(P.changed_slots(st0, c.state)) <= set(live)


def test_grouped_value_heads_ragged_with_checkpoints():
    say("grouped heads ragged H=4 HV=12 bf16 seed=6100")
    lengths = [3, 0, 5, 1, 2, 4]
    c = synth.recurrent_case(6100, n_seqs=6, H=4, HV=12, num_slots=9, state_dtype=torch.bfloat16,
                             device=DEV, indices="random", lengths=lengths, null_rows=1)
    want = ref(c, np_(c.state), ckpt_dtype=oracle.BF16, ragged=True)
    out, ck = run(c, form="ragged", ckpt=True)
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
    P.check_state(ck, want["ckpt"], "checkpoints")


@pytest.mark.parametrize("gate_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("form", ["t1", "ragged"])
def test_precomputed_gate(form, gate_dtype):
    say(f"precomputed gate {form} {gate_dtype} seed=6200")
    lengths = None if form == "t1" else [2, 4, 0, 3]
    n = 29 if form == "t1" else 4
    c = synth.recurrent_case(6200, n_seqs=n, H=8, num_slots=40, device=DEV, indices="random",
                             lengths=lengths, gate="precomputed", gate_dtype=gate_dtype, null_rows=1)
    assert c.A_log is None
    want = ref(c, np_(c.state), ckpt_dtype=oracle.F32, ragged=form == "ragged")
    out, ck = run(c, form=form, ckpt=form == "ragged")
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
    if ck is not None:
        P.check_state(ck, want["ckpt"], "checkpoints")


def test_precomputed_unit_decay_beta_one_stores_value():
    say("precomputed gate g=0 beta=1 seed=6250")
    c = synth.recurrent_case(6250, n_seqs=8, H=4, num_slots=8, device=DEV, gate="precomputed")
    c.g.zero_()
    c.beta.fill_(1.0)
    T = 8
    recurrent_kda(c.q.reshape(T, 1, 4, D), c.k.reshape(T, 1, 4, D), c.v.reshape(T, 1, 4, D),
                  c.g.reshape(T, 1, 4, D), c.beta.reshape(T, 1, 4), initial_state=c.state,
                  state_indices=c.state_indices, l2_eps=0.0)
    torch.cuda.synchronize()
    kh = c.k.double() / c.k.double().norm(dim=-1, keepdim=True)
    kS = (c.state.double() * kh[:, :, None, :]).sum(-1)
    assert (kS - c.v.double()).abs().max().item() <= 1e-4


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_batched_form_matches_ragged_bitwise(state_dtype):
    """[B, T, ...] without cu_seqlens equals the ragged call with uniform lengths."""
    say(f"batched form B=12 T=4 {state_dtype} seed=6300")
    B, T = 12, 4
    c = synth.recurrent_case(6300, n_seqs=B, H=4, HV=8, num_slots=20, state_dtype=state_dtype,
                             device=DEV, indices="random", lengths=[T] * B, null_rows=2)
    st0 = c.state.clone()
    o_r, k_r = run(c, form="ragged", ckpt=True)
    s_r = c.state.clone()
    c.state.copy_(st0)
    o_b, k_b = run(c, form="batched", ckpt=True, tps=T)
    assert tuple(o_b.shape) == (B, T, 8, D)
    assert torch.equal(P.bits(o_r.reshape(-1)), P.bits(o_b.reshape(-1)))
    assert torch.equal(P.bits(k_r), P.bits(k_b))
    assert torch.equal(P.bits(s_r), P.bits(c.state))
    want = ref(c, np_(st0), ckpt_dtype=oracle.F32 if state_dtype == torch.float32 else oracle.BF16,
               tps=T)
    P.check_bf16_out(o_b, want["out64"])
    P.check_state(c.state, want["state"])


@pytest.mark.parametrize("B", [3, 8, 12])
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_updating_batched_token_loop_geometries(state_dtype, B):
    """Updating batched calls without checkpoints, H=32, 3 tokens: 96, 256
    and 384 (sequence, head) items, i.e. 4 value-row splits (fp32 pool up
    to 383 items), 2 splits (bf16 from 96 items, fp32 at 384), against the
    oracle, with random slots and null rows."""
    say(f"updating batched T=3 H=32 B={B} {state_dtype} seed={6400 + B}")
    T = 3
    c = synth.recurrent_case(6400 + B, n_seqs=B, H=32, num_slots=B + 4, state_dtype=state_dtype,
                             device=DEV, indices="random", lengths=[T] * B, null_rows=1)
    st0 = c.state.clone()
    o, _ = run(c, form="batched", tps=T)
    want = ref(c, np_(st0), tps=T)
    P.check_bf16_out(o, want["out64"])
    P.check_state(c.state, want["state"])


@pytest.mark.parametrize("form", ["t1", "ragged", "batched"])
def test_read_only_pool(form):
    """disable_state_update: the pool is bit-identical afterwards; outputs and
    checkpoints match the oracle's read-only run (= the updating run's)."""
    say(f"read-only pool {form} seed=6400")
    if form == "t1":
        c = synth.recurrent_case(6400, n_seqs=33, H=6, num_slots=40, device=DEV, indices="random",
                                 null_rows=3)
        tps, lengths = 1, None
    elif form == "ragged":
        lengths = [16, 3, 0, 9, 1, 16, 7]
        c = synth.recurrent_case(6401, n_seqs=7, H=6, num_slots=10, device=DEV, indices="random",
                                 lengths=lengths, null_rows=1, state_dtype=torch.bfloat16)
        tps = 1
    else:
        tps = 16
        c = synth.recurrent_case(6402, n_seqs=5, H=2, HV=6, num_slots=8, device=DEV,
                                 indices="random", lengths=[tps] * 5)
    st0 = c.state.clone()
    want = ref(c, np_(st0), ckpt_dtype=oracle.F32 if c.state.dtype == torch.float32 else oracle.BF16,
               read_only=True, tps=tps, ragged=form == "ragged")
    out, ck = run(c, form=form, ckpt=form != "t1", read_only=True, tps=tps)
    assert torch.equal(P.bits(st0), P.bits(c.state)), "a read-only pool was written"
    P.check_bf16_out(out, want["out64"])
    if ck is not None:
        P.check_state(ck, want["ckpt"], "checkpoints")
    # same outputs as the state-updating call
    out2, _ = run(c, form=form, tps=tps)
    assert torch.equal(P.bits(out.reshape(-1)), P.bits(out2.reshape(-1)))
