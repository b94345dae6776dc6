"""Write guards: every buffer an entry point writes (outputs, state pools,
conv caches, checkpoints, verify caches) is the middle of a larger
allocation whose margins hold a canary pattern; after the call the margins
must be bit-identical.  Index sets include null rows (-1, and 0 for the
fused calls), indices >= num_slots, padding columns and empty sequences, so
every kernel's bounds handling is exercised next to poisoned memory.
"""
import pytest
import torch

from gated_delta_rule_decode_amd import (PackedFusedWorkspace, fused_kda_decode, packed_fused_kda_decode,
                                         packed_kda_decode, recurrent_kda, synth)
from tests import parity as P

pytestmark = pytest.mark.gpu
D = 128
DEV = "cuda:0"
PAD = 4096  # canary elements on each side


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[case]", *a, flush=True)


class Guarded:
    """A tensor of `shape` in the middle of a flat allocation with canaries."""

    def __init__(self, shape, dtype, fill=None, pad=PAD):
        n = 1
        for s in shape:
            n *= s
        self.flat = torch.empty(n + 2 * pad, dtype=dtype, device=DEV)
        bits = P.bits(self.flat)
        bits.copy_(torch.arange(bits.numel(), device=DEV).remainder(251).add(0x1234).to(bits.dtype))
        self.ref = self.flat.clone()
        self.pad, self.n = pad, n
        self.t = self.flat[pad:pad + n].view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what):
        got, ref = P.bits(self.flat), P.bits(self.ref)
        assert torch.equal(got[:self.pad], ref[:self.pad]), f"{what}: wrote below its buffer"
        assert torch.equal(got[self.pad + self.n:], ref[self.pad + self.n:]), f"{what}: wrote past its buffer"


def guarded_pool(state):
    """The pool as a view into a larger allocation (guard slots on both sides)."""
    return Guarded(tuple(state.shape), state.dtype, fill=state, pad=2 * state[0].numel())


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_recurrent_t1_guards(state_dtype):
    say(f"guards recurrent T=1 {state_dtype}")
    N, H, S = 24, 4, 32
    c = synth.recurrent_case(9500, n_seqs=N, H=H, num_slots=S, state_dtype=state_dtype, device=DEV,
                             indices="random", null_rows=3)
    idx = c.state_indices.clone()
    idx[[1, 7]] = torch.tensor([S, S + 5], dtype=torch.int32, device=DEV)  # past the pool: null rows
    pool = guarded_pool(c.state)
    out = Guarded((N, 1, H, D), torch.bfloat16)
    r = lambda t: t.reshape(N, 1, *t.shape[1:])  # noqa: E731
    recurrent_kda(r(c.q), r(c.k), r(c.v), r(c.g), c.beta.reshape(N, 1, H), c.A_log, c.dt_bias,
                  initial_state=pool.t, state_indices=idx, output=out.t)
    torch.cuda.synchronize()
    pool.check("state pool")
    out.check("output")


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_recurrent_ragged_checkpoint_and_cache_guards(state_dtype):
    say(f"guards ragged + checkpoints + verify caches {state_dtype}")
    lengths = [3, 0, 5, 1, 2, 4]
    H, S, TM = 4, 16, 3
    c = synth.recurrent_case(9600, n_seqs=len(lengths), H=H, num_slots=S, state_dtype=state_dtype,
                             device=DEV, indices="random", lengths=lengths, null_rows=1)
    idx = c.state_indices.clone()
    idx[3] = S + 2
    T = sum(lengths)
    pool = guarded_pool(c.state)
    out = Guarded((1, T, H, D), torch.bfloat16)
    ck = Guarded((T, H, D, D), state_dtype)
    corr = Guarded((S, H, TM, D), torch.float32)
    kg = Guarded((S, H, TM, 2 * D), torch.bfloat16)
    r = lambda t: t.reshape(1, T, *t.shape[1:])  # noqa: E731
    recurrent_kda(r(c.q), r(c.k), r(c.v), r(c.g), r(c.beta), c.A_log, c.dt_bias, initial_state=pool.t,
                  state_indices=idx, cu_seqlens=c.cu_seqlens, output=out.t, intermediate_states=ck.t,
                  correction_cache=corr.t, kg_cache=kg.t)
    torch.cuda.synchronize()
    for g, n in ((pool, "state pool"), (out, "output"), (ck, "checkpoints"), (corr, "correction cache"),
                 (kg, "kg cache")):
        g.check(n)


@pytest.mark.parametrize("state_dtype,T,TM", [(torch.float32, 8, 5), (torch.bfloat16, 3, 6), (torch.float32, 2, 3)])
def test_verify_wy_guards(state_dtype, T, TM):
    """Read-only batched calls of a few tokens (the WY verify kernel; fp32
    pools of up to 4 tokens take its 4x4x1 products): output and both verify
    caches guarded, the pool guarded and unchanged, with a null row and an
    index past the pool."""
    say(f"guards WY verify T={T} cache {TM} {state_dtype}")
    n, H, HV, S = 6, 2, 4, 12
    c = synth.recurrent_case(9650 + T, n_seqs=n, H=H, HV=HV, num_slots=S, state_dtype=state_dtype, device=DEV,
                             indices="random", lengths=[T] * n, null_rows=1)
    idx = c.state_indices.clone()
    idx[2] = S + 3
    pool = guarded_pool(c.state)
    before = pool.t.clone()
    out = Guarded((n, T, HV, D), torch.bfloat16)
    corr = Guarded((S, HV, TM, D), torch.float32)
    kg = Guarded((S, HV, TM, 2 * D), torch.float32)
    b = lambda t: t.reshape(n, T, *t.shape[1:])  # noqa: E731
    recurrent_kda(b(c.q), b(c.k), b(c.v), b(c.g), b(c.beta), c.A_log, c.dt_bias, initial_state=pool.t,
                  state_indices=idx, output=out.t, disable_state_update=True, correction_cache=corr.t,
                  kg_cache=kg.t)
    torch.cuda.synchronize()
    for g, nm in ((pool, "state pool"), (out, "output"), (corr, "correction cache"), (kg, "kg cache")):
        g.check(nm)
    assert torch.equal(P.bits(pool.t), P.bits(before)), "read-only pool changed"


def test_packed_decode_guards():
    say("guards packed decode H=12 bf16")
    B, H, S = 40, 12, 64
    pc = synth.packed_case(9700, B=B, H=H, num_slots=S, device=DEV, null_rows=4)
    idx = pc.state_indices.clone()
    idx[5] = S
    pool = guarded_pool(pc.state)
    out = Guarded((B, 1, H, D), torch.bfloat16)
    packed_kda_decode(pc.mixed_qkv, pc.raw_gate, pc.raw_beta, pc.A_log, pc.dt_bias, pool.t, idx, output=out.t)
    torch.cuda.synchronize()
    pool.check("state pool")
    out.check("output")


def test_fused_decode_guards():
    say("guards fused decode H=8")
    rows, H, S = 20, 8, 32
    fc = synth.fused_case(9800, rows=rows, H=H, num_slots=S, device=DEV, null_zero=2, null_neg=2)
    idx = fc.state_indices.clone()
    idx[3] = S + 1
    pool = guarded_pool(fc.state)
    C3 = 3 * H * D
    cs = Guarded((S, 3, C3), torch.bfloat16, fill=fc.conv_state.transpose(1, 2), pad=3 * C3 * 2)
    conv = cs.t.transpose(1, 2)  # logical [S, C3, 3], strides [3*C3, 1, C3]
    out = Guarded((1, rows, H, D), torch.bfloat16)
    fused_kda_decode(fc.x, fc.weight, conv, fc.raw_gate, fc.raw_beta, fc.A_log, fc.dt_bias, idx, pool.t,
                     fc.output_gate, fc.norm_weight, output=out.t)
    torch.cuda.synchronize()
    pool.check("state pool")
    cs.check("conv cache")
    out.check("output")


@pytest.mark.parametrize("split", [False, True], ids=["unsplit", "split"])
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_packed_fused_guards(state_dtype, split):
    say(f"guards packed fused {state_dtype} split={split}")
    H, S = 4, 48
    c = synth.packed_fused_case(9900, lengths=[4, 0, 3, 1, 2], H=H, num_slots=S, max_tokens=3,
                                state_dtype=state_dtype, device=DEV, pad_rows=2)
    si = c.state_indices.clone()
    si[0, 1] = 0
    si[2, 1] = -1
    si[3, 0] = S + 3        # start slot past the pool: null sequence
    si[4, 1] = S            # checkpoint column past the pool: not written
    acc = torch.tensor([1, 1, 3, 1, 1], dtype=torch.int32, device=DEV)
    rows = c.x.shape[0]
    pool = guarded_pool(c.state)
    C3 = 3 * H * D
    cs = Guarded((S, 3, C3), torch.bfloat16, fill=c.conv_state.transpose(1, 2), pad=3 * C3 * 2)
    out = Guarded((1, rows, H, D), torch.bfloat16)
    ws = None
    if split:  # the split workspace, exactly sized, between canaries too
        ws = PackedFusedWorkspace(DEV)
        cnt = Guarded((5 * H,), torch.int32, fill=torch.zeros(5 * H, dtype=torch.int32))
        part = Guarded((rows * H * D,), torch.float32)
        ws.counters, ws.partials = cnt.t, part.t
    packed_fused_kda_decode(c.x, c.weight, cs.t.transpose(1, 2), c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, si,
                            pool.t, c.output_gate, c.norm_weight, output=out.t, query_start_loc=c.query_start_loc,
                            num_accepted_tokens=acc, workspace=ws)
    torch.cuda.synchronize()
    pool.check("state pool")
    cs.check("conv cache")
    out.check("output")
    if split:
        cnt.check("split counters")
        part.check("split partials")
        assert int(cnt.t.abs().sum()) == 0, "split counters not left at zero"
