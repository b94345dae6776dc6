"""Parity of the HIP path (through the C ABI) with the fp64 oracle on MI355X.

Every case prints its name, seed and shape before it touches the GPU.
Inputs come from the seeded generators in gated_delta_rule_decode_amd.synth;
the oracle gets host copies of exactly the tensors the kernels read.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import (KDAError, fused_kda_decode, packed_kda_decode,
                                         recurrent_kda, synth)

from tests import parity as P

pytestmark = pytest.mark.gpu
D = 128
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_decode_amd._lib as L
    assert L.load().kda_check_device(0) == 0, "device 0 is not a gfx950"


def say(*a):
    print("[case]", *a, flush=True)


def np_(t):
    return oracle.as_np(P.host(t))


# ------------------------------------------------------------------ helpers ----

def run_recurrent_case(c, *, ckpt=False, n_tokens=None):
    """Run recurrent_kda on device copies of case c; return (out, state, ckpt)."""
    g = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    T = c.q.shape[0]
    if c.cu_seqlens is None:
        shp = lambda t: t.reshape(T, 1, *t.shape[1:])  # noqa: E731
    else:
        shp = lambda t: t.reshape(1, T, *t.shape[1:])  # noqa: E731
    state = c.state if c.state.is_cuda else g(c.state)
    ck = torch.zeros((T, c.H, D, D), dtype=state.dtype, device=DEV) if ckpt else None
    out = recurrent_kda(shp(g(c.q)), shp(g(c.k)), shp(g(c.v)), shp(g(c.g)), shp(g(c.beta)),
                        g(c.A_log), g(c.dt_bias), initial_state=state,
                        state_indices=g(c.state_indices), cu_seqlens=g(c.cu_seqlens),
                        intermediate_states=ck)
    torch.cuda.synchronize()
    return out, state, ck


def oracle_recurrent(c, state_host, ckpt_dtype=None):
    return oracle.recurrent(np_(c.q), np_(c.k), np_(c.v), np_(c.g), np_(c.beta), np_(c.A_log),
                            np_(c.dt_bias), state_host, np_(c.state_indices),
                            None if c.cu_seqlens is None else np_(c.cu_seqlens),
                            ckpt_dtype=ckpt_dtype)


# ---------------------------------------------------- config: tiny recurrent ----

def test_recurrent_t1_tiny_identity():
    """recurrent_kda T=1: N=4, H=4, fp32 state, identity indices (seed 0)."""
    say("recurrent T=1 tiny N=4 H=4 fp32 seed=0")
    c = synth.recurrent_case(0, n_seqs=4, H=4, num_slots=4)
    want = oracle_recurrent(c, np_(c.state))
    out, state, _ = run_recurrent_case(c)
    e1 = P.check_bf16_out(out, want["out64"])
    e2 = P.check_state(state, want["state"])
    say(f"out err {e1:.3e} state err {e2:.3e}")


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,H", [(1, 1), (3, 5), (31, 2), (64, 7)])
def test_recurrent_t1_shapes(N, H, state_dtype):
    """Several tiles and ragged sizes; random unique slots with null rows and
    an out-of-range index; untouched slots stay bit-identical."""
    say(f"recurrent T=1 N={N} H={H} {state_dtype} seed={100 + N}")
    slots = N + 9
    c = synth.recurrent_case(100 + N, n_seqs=N, H=H, num_slots=slots, state_dtype=state_dtype,
                             indices="random", null_rows=N // 4)
    if N >= 3:
        c.state_indices[1] = slots + 3  # beyond the pool: null
    before = c.state.clone()
    want = oracle_recurrent(c, np_(c.state))
    out, state, _ = run_recurrent_case(c)
    P.check_bf16_out(out, want["out64"])
    P.check_state(state, want["state"])
    live = sorted({int(i) for i in c.state_indices.tolist() if 0 <= i < slots})
    assert set(P.changed_slots(before.to(DEV), state)) <= set(live)
    o = P.bits(out.cpu().reshape(N, H, D))
    for i, s in enumerate(c.state_indices.tolist()):
        if not (0 <= s < slots):
            assert not o[i].any(), "null rows must produce +0"


# ------------------------------------------- config: packed H=12 bf16 serving ----

@pytest.mark.parametrize("B,nulls,row_pad", [(64, 8, 0), (64, 8, 64), (256, 32, 0), (512, 64, 0)])
def test_packed_h12_bf16(B, nulls, row_pad):
    """packed_kda_decode T=1, H=12, bf16 pool [1024,12,128,128], unique slots
    in [1,1024), 1/8 of the rows -1: B=64 with a plain and a padded QKV row
    stride, and the two batch sizes the benchmark times (B=256 and B=512,
    the launch geometry of its packed sweep)."""
    seed = 2000 + B
    say(f"packed H=12 B={B} bf16 row_pad={row_pad} nulls={nulls} seed={seed}")
    c = synth.packed_case(seed, B=B, H=12, num_slots=1024, device=DEV, null_rows=nulls, row_pad=row_pad)
    idx = c.state_indices.cpu()
    live = sorted(int(i) for i in idx.tolist() if i >= 0)
    assert len(live) == B - nulls
    before_live = c.state[torch.tensor(live, device=DEV)].cpu()
    pool_before = c.state.clone()
    sub = {s: j for j, s in enumerate(live)}
    # oracle on the touched slots only (remapped indices)
    idx_sub = np.array([sub.get(int(i), -1) for i in idx.tolist()], np.int32)
    want = oracle.packed(P.host(c.mixed_qkv), P.host(c.raw_gate), P.host(c.raw_beta),
                         P.host(c.A_log), P.host(c.dt_bias), oracle.as_np(before_live), idx_sub)
    out = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                            c.state_indices)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (B, 1, 12, D)
    e1 = P.check_bf16_out(out, want["out64"])
    e2 = P.check_state(c.state[live], want["state"])
    assert set(P.changed_slots(pool_before, c.state)) <= set(live)
    untouched = torch.ones(1024, dtype=torch.bool)
    untouched[live] = False
    ut = torch.nonzero(untouched).flatten().to(DEV)
    assert torch.equal(P.bits(c.state.index_select(0, ut)), P.bits(pool_before.index_select(0, ut)))
    o = out.reshape(B, -1)
    assert not P.bits(o[idx.to(DEV) < 0]).any(), "inactive rows must be +0"
    say(f"out err {e1:.3e} state err {e2:.3e}")


# ------------------------------------ config: H=32 fp32 pool, batch sweep --------

@pytest.fixture(scope="module")
def pool_h32():
    say("allocating fp32 pool [4096,32,128,128] (8 GiB), seed=1000")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1000)
    pool = synth._randn_big(gen, (4096, 32, D, D), DEV, 0.05, torch.float32)
    yield pool
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [1, 8, 32, 128, 256, 512])
def test_recurrent_h32_fp32_sweep(pool_h32, B):
    """T=1 recurrence, H=32, fp32 pool [4096,32,128,128], random unique slots;
    every output and every touched slot against the oracle, every other slot
    bit-identical."""
    say(f"recurrent T=1 H=32 fp32 B={B} seed={1000 + B}")
    H = 32
    c = synth.recurrent_case(1000 + B, n_seqs=B, H=H, num_slots=1, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1000 + B)
    idx = synth.unique_slots(gen, B, 0, 4096, DEV)
    live = idx.tolist()
    touched_before = pool_h32.index_select(0, idx).cpu()
    marker = pool_h32[:, 0, 0, :2].clone()  # cheap fingerprint of every slot
    want = oracle.recurrent(np_(c.q), np_(c.k), np_(c.v), np_(c.g), np_(c.beta), np_(c.A_log),
                            np_(c.dt_bias), oracle.as_np(touched_before), np.arange(B, dtype=np.int32))
    out = recurrent_kda(c.q.reshape(B, 1, H, D), c.k.reshape(B, 1, H, D), c.v.reshape(B, 1, H, D),
                        c.g.reshape(B, 1, H, D), c.beta.reshape(B, 1, H), c.A_log, c.dt_bias,
                        initial_state=pool_h32, state_indices=idx)
    torch.cuda.synchronize()
    e1 = P.check_bf16_out(out, want["out64"])
    e2 = P.check_state(pool_h32.index_select(0, idx), want["state"])
    m2 = pool_h32[:, 0, 0, :2]
    diff = torch.nonzero((P.bits(m2) != P.bits(marker)).any(dim=1)).flatten().tolist()
    assert set(diff) <= set(live)
    say(f"out err {e1:.3e} state err {e2:.3e}")


def test_recurrent_h32_untouched_slots_bitwise(pool_h32):
    """Full-pool bitwise check around one B=256 call."""
    say("recurrent H=32 fp32 B=256 full-pool untouched check seed=1256")
    B, H = 256, 32
    c = synth.recurrent_case(1256, n_seqs=B, H=H, num_slots=1, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    idx = synth.unique_slots(gen, B, 0, 4096, DEV)
    before = pool_h32.clone()
    recurrent_kda(c.q.reshape(B, 1, H, D), c.k.reshape(B, 1, H, D), c.v.reshape(B, 1, H, D),
                  c.g.reshape(B, 1, H, D), c.beta.reshape(B, 1, H), c.A_log, c.dt_bias,
                  initial_state=pool_h32, state_indices=idx)
    torch.cuda.synchronize()
    changed = P.changed_slots(before, pool_h32)
    assert set(changed) <= set(idx.tolist())
    assert len(changed) == B
    del before


def test_row_permutation_at_full_size_is_bitwise(pool_h32):
    """Rows are independent at any size: the full B=256, H=32 fp32 call with
    its rows and slot indices permuted gives the permuted outputs and the same
    touched slots, bit for bit (checks every output and slot of the launch
    the benchmark times, where the oracle compares the same call)."""
    say("recurrent H=32 fp32 B=256 row permutation bitwise seed=1300")
    B, H = 256, 32
    c = synth.recurrent_case(1300, n_seqs=B, H=H, num_slots=1, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1300)
    idx = synth.unique_slots(gen, B, 0, 4096, DEV)
    perm = torch.randperm(B, generator=gen, device=DEV)
    before = pool_h32.index_select(0, idx)
    r4 = lambda t: t.reshape(B, 1, *t.shape[1:])  # noqa: E731
    args = [r4(c.q), r4(c.k), r4(c.v), r4(c.g), r4(c.beta)]
    out1 = recurrent_kda(*args, c.A_log, c.dt_bias, initial_state=pool_h32, state_indices=idx)
    torch.cuda.synchronize()
    after1 = pool_h32.index_select(0, idx)
    pool_h32.index_copy_(0, idx.long(), before)
    out2 = recurrent_kda(*[a[perm].contiguous() for a in args], c.A_log, c.dt_bias, initial_state=pool_h32,
                         state_indices=idx[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(P.bits(out2), P.bits(out1[perm]))
    assert torch.equal(P.bits(pool_h32.index_select(0, idx)), P.bits(after1))
    del before, after1


def test_packed_row_permutation_b512_is_bitwise():
    """The same for packed_kda_decode at H=12, B=512, bf16, 64 inactive rows."""
    say("packed H=12 B=512 bf16 row permutation bitwise seed=2512")
    B = 512
    c = synth.packed_case(2512, B=B, H=12, num_slots=1024, device=DEV, null_rows=64)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(2512)
    perm = torch.randperm(B, generator=gen, device=DEV)
    pool0 = c.state.clone()
    out1 = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state, c.state_indices)
    torch.cuda.synchronize()
    pool1 = c.state.clone()
    c.state.copy_(pool0)
    out2 = packed_kda_decode(c.mixed_qkv[perm].contiguous(), c.raw_gate[perm].contiguous(),
                             c.raw_beta[perm].contiguous(), c.A_log, c.dt_bias, c.state,
                             c.state_indices[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(P.bits(out2), P.bits(out1[perm]))
    assert torch.equal(P.bits(c.state), P.bits(pool1))
    del pool0, pool1


# --------------------------------------------------- config: fused decode -------

@pytest.mark.parametrize("state_dtype,rows,H,slots", [
    (torch.float32, 256, 32, 2048),
    (torch.bfloat16, 37, 12, 64),
    (torch.float32, 5, 8, 16),
])
def test_fused_decode(state_dtype, rows, H, slots):
    """fused_kda_decode: conv+SiLU -> KDA -> gated RMSNorm; unique slots in
    [1, slots), 8 zero + 8 negative null rows (fewer for small cases)."""
    nz = min(8, rows // 4)
    seed = 3000 + rows
    say(f"fused rows={rows} H={H} slots={slots} {state_dtype} seed={seed}")
    c = synth.fused_case(seed, rows=rows, H=H, num_slots=slots, state_dtype=state_dtype, device=DEV,
                         null_zero=nz, null_neg=nz, slot_pad=8 if rows < 100 else 0)
    idx = c.state_indices.cpu()
    live = sorted(int(i) for i in idx.tolist() if i > 0)
    sub = {s: j + 1 for j, s in enumerate(live)}   # slot 0 of the sub-pool stays reserved
    idx_sub = np.array([sub.get(int(i), int(i)) for i in idx.tolist()], np.int32)
    sel = torch.tensor([0] + live, device=DEV)
    st_sub = c.state.index_select(0, sel).cpu()
    cs_sub = c.conv_state.index_select(0, sel).cpu()
    st_before, cs_before = c.state.clone(), c.conv_state.clone()
    want = oracle.fused(P.host(c.x), P.host(c.weight), oracle.as_np(cs_sub), P.host(c.raw_gate),
                        P.host(c.raw_beta), P.host(c.A_log), P.host(c.dt_bias), idx_sub,
                        oracle.as_np(st_sub), P.host(c.output_gate), P.host(c.norm_weight))
    out = fused_kda_decode(c.x, c.weight, c.conv_state, c.raw_gate.reshape(1, rows, H, D),
                           c.raw_beta.reshape(1, rows, H), c.A_log, c.dt_bias, c.state_indices,
                           c.state, c.output_gate, c.norm_weight)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (1, rows, H, D)
    e1 = P.check_bf16_out(out, want["out64"], "fused out")
    e2 = P.check_state(c.state.index_select(0, sel[1:]), want["state"][1:])
    got_cs = c.conv_state.index_select(0, sel[1:]).cpu()
    want_cs = torch.from_numpy(np.ascontiguousarray(want["conv_state"][1:]).view(np.int16))
    assert torch.equal(got_cs.contiguous().view(torch.int16), want_cs), "conv cache must be bit-exact"
    assert P.changed_slots(st_before, c.state) == live
    cs_changed = torch.nonzero((P.bits(cs_before) != P.bits(c.conv_state)).reshape(slots, -1).any(1))
    assert sorted(cs_changed.flatten().tolist()) == live
    null = idx <= 0
    assert not P.bits(out.reshape(rows, -1)[null.to(DEV)]).any()
    say(f"fused out err {e1:.3e} state err {e2:.3e}")


# ------------------------------------------- config: ragged packed T>=2 ----------

@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_varlen_h16_n64(state_dtype):
    """recurrent_kda packed T>=2: H=16, N=64, lengths U{0..6} (empty allowed),
    per-token checkpoints, pool [N+1,16,128,128], sequence i in slot i+1."""
    N, H = 64, 16
    lengths = synth.ragged_lengths(4000, N, 0, 6)
    say(f"varlen H=16 N=64 {state_dtype} T_tot={sum(lengths)} seed=4000")
    c = synth.recurrent_case(4000, n_seqs=N, H=H, num_slots=N + 1, state_dtype=state_dtype,
                             device=DEV, lengths=lengths, slot_lo=1)
    before = c.state.clone()
    cdt = oracle.F32 if state_dtype == torch.float32 else oracle.BF16
    want = oracle_recurrent(c, np_(c.state), ckpt_dtype=cdt)
    out, state, ck = run_recurrent_case(c, ckpt=True)
    e1 = P.check_bf16_out(out, want["out64"])
    e2 = P.check_state(state, want["state"])
    e3 = P.check_state(ck, want["ckpt"], "checkpoints")
    assert torch.equal(P.bits(state[0]), P.bits(before[0])), "slot 0 must be untouched"
    live = [i + 1 for i in range(N) if lengths[i] > 0]
    assert P.changed_slots(before, state) == live
    say(f"varlen out err {e1:.3e} state err {e2:.3e} ckpt err {e3:.3e}")


def test_varlen_equals_successive_t1_calls_bitwise():
    """A T-token ragged call equals T successive T=1 calls, bit for bit with an
    fp32 pool (same per-row arithmetic on the device)."""
    N, H = 6, 3
    lengths = [3, 0, 1, 4, 2, 0]
    say("varlen vs successive T=1 calls fp32 seed=4100")
    c = synth.recurrent_case(4100, n_seqs=N, H=H, num_slots=N + 2, device=DEV, lengths=lengths,
                             indices="random")
    pool_a = c.state.clone()
    pool_b = c.state.clone()
    c.state = pool_a
    out_a, _, ck = run_recurrent_case(c, ckpt=True)
    cu = c.cu_seqlens.cpu().tolist()
    idx = c.state_indices
    out_b = torch.zeros_like(out_a).reshape(-1, H, D)
    for step in range(max(lengths)):
        sel = [i for i in range(N) if lengths[i] > step]
        toks = torch.tensor([cu[i] + step for i in sel], device=DEV)
        n = len(sel)
        o = recurrent_kda(c.q[toks].reshape(n, 1, H, D), c.k[toks].reshape(n, 1, H, D),
                          c.v[toks].reshape(n, 1, H, D), c.g[toks].reshape(n, 1, H, D),
                          c.beta[toks].reshape(n, 1, H), c.A_log, c.dt_bias, initial_state=pool_b,
                          state_indices=idx[torch.tensor(sel, device=DEV)].contiguous())
        out_b[toks] = o.reshape(n, H, D)
        for j, i in enumerate(sel):
            assert torch.equal(P.bits(ck[cu[i] + step]), P.bits(pool_b[int(idx[i])]))
    torch.cuda.synchronize()
    assert torch.equal(P.bits(out_a.reshape(-1, H, D)), P.bits(out_b))
    assert torch.equal(P.bits(pool_a), P.bits(pool_b))


def test_varlen_all_empty_and_zero_tokens():
    say("varlen all-empty sequences seed=4200")
    c = synth.recurrent_case(4200, n_seqs=4, H=2, num_slots=6, device=DEV, lengths=[0, 0, 0, 0],
                             indices="random")
    before = c.state.clone()
    out, state, _ = run_recurrent_case(c)
    assert out.numel() == 0
    assert torch.equal(P.bits(before), P.bits(state))


# ------------------------------------------------- invariants on the device --------

@pytest.mark.parametrize("kind", ["t1", "varlen", "fused"])
def test_bf16_store_is_rne_of_the_fp32_computation(kind):
    """With beta = 0 every state element becomes s * decay: one fp32 multiply
    whose value does not depend on how lanes split the key channels.  Starting
    from the same bf16-representable state, a bf16 pool must then end as the
    round-to-nearest-even (torch's fp32->bf16 conversion) of what an fp32
    pool ends with, and so must the ragged call's checkpoints.  Outputs
    (whose dot products the two layouts sum in different orders) must agree
    to one bf16 ulp."""
    say(f"bf16 store rounding vs fp32 pool ({kind}) seed=5100")
    if kind == "fused":
        c = synth.fused_case(5100, rows=9, H=4, num_slots=12, state_dtype=torch.bfloat16, device=DEV,
                             null_zero=1, null_neg=1)
        c.raw_beta.fill_(-math.inf)
        s32 = c.state.float()
        cs32 = c.conv_state.clone()
        args = lambda st, cs: (c.x, c.weight, cs, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias,  # noqa: E731
                               c.state_indices, st, c.output_gate, c.norm_weight)
        o16 = fused_kda_decode(*args(c.state, c.conv_state))
        o32 = fused_kda_decode(*args(s32, cs32))
        torch.cuda.synchronize()
        assert torch.equal(P.bits(c.state), P.bits(s32.to(torch.bfloat16)))
        a, b = o16.double().cpu().numpy(), o32.double().cpu().numpy()
        assert np.all(np.abs(a - b) <= P.bf16_ulp(b) + 1e-30)
        return
    lengths = None if kind == "t1" else [2, 0, 3, 1, 2]
    c = synth.recurrent_case(5100, n_seqs=5, H=3, num_slots=8, state_dtype=torch.bfloat16,
                             device=DEV, lengths=lengths, indices="random", null_rows=1)
    c.beta.fill_(-math.inf)
    c32 = synth.RecurrentCase(**{**c.__dict__, "state": c.state.float()})
    o16, s16, k16 = run_recurrent_case(c, ckpt=kind == "varlen")
    o32, s32, k32 = run_recurrent_case(c32, ckpt=kind == "varlen")
    assert torch.equal(P.bits(s16), P.bits(s32.to(torch.bfloat16)))
    if kind == "varlen":
        assert torch.equal(P.bits(k16), P.bits(k32.to(torch.bfloat16)))
        cu = c.cu_seqlens.tolist()
        for i, s in enumerate(c.state_indices.tolist()):
            if s < 0:  # a null sequence writes no checkpoint
                assert not P.bits(k16[cu[i]:cu[i + 1]]).any()
    a, b = o16.double().cpu().numpy(), o32.double().cpu().numpy()
    assert np.all(np.abs(a - b) <= P.bf16_ulp(b) + 1e-30)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_beta_zero_unit_decay_leaves_state_bitwise(state_dtype):
    say(f"invariant beta=0 unit decay {state_dtype} seed=5000")
    N, H = 16, 4
    c = synth.recurrent_case(5000, n_seqs=N, H=H, num_slots=N, state_dtype=state_dtype, device=DEV,
                             indices="random")
    c.A_log.fill_(-math.inf)
    c.beta.fill_(-math.inf)
    before = c.state.clone()
    want = oracle_recurrent(c, np_(c.state))
    out, state, _ = run_recurrent_case(c)
    assert torch.equal(P.bits(before), P.bits(state))
    P.check_bf16_out(out, want["out64"])


def test_beta_one_unit_decay_stores_value():
    say("invariant beta=1 unit decay eps=0 seed=5001")
    N, H = 8, 4
    c = synth.recurrent_case(5001, n_seqs=N, H=H, num_slots=N, device=DEV)
    c.A_log.fill_(-math.inf)
    c.beta.fill_(math.inf)
    T = N
    out = recurrent_kda(c.q.reshape(T, 1, H, D), c.k.reshape(T, 1, H, D), c.v.reshape(T, 1, H, D),
                        c.g.reshape(T, 1, H, D), c.beta.reshape(T, 1, H), c.A_log, c.dt_bias,
                        initial_state=c.state, state_indices=c.state_indices, l2_eps=0.0)
    torch.cuda.synchronize()
    k = c.k.double()
    kh = k / k.norm(dim=-1, keepdim=True)
    S = c.state.double()  # [slot][h][v][k]; slot i == row i
    kS = (S * kh[:, :, None, :]).sum(-1)
    err = (kS - c.v.double()).abs().max().item()
    say(f"max |k^T S' - v| = {err:.3e}")
    assert err <= 1e-4
    assert out.isfinite().all()


def test_null_only_batch():
    say("all rows null seed=5002")
    c = synth.packed_case(5002, B=5, H=3, num_slots=8, device=DEV, state_dtype=torch.float32)
    c.state_indices.fill_(-1)
    before = c.state.clone()
    out = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                            c.state_indices)
    torch.cuda.synchronize()
    assert not P.bits(out).any()
    assert torch.equal(P.bits(before), P.bits(c.state))


def test_padded_slot_stride_pool():
    """Pool slots with padding between them (arbitrary positive slot stride)."""
    say("packed padded slot stride seed=5003")
    H, B, S = 4, 10, 12
    c = synth.packed_case(5003, B=B, H=H, num_slots=S, device=DEV, state_dtype=torch.float32,
                          null_rows=2)
    pad = 4096 + 12  # elements; keeps 16-byte alignment
    store = torch.full((S, H * D * D + pad), 7.0, device=DEV)
    pool = store[:, :H * D * D].view(S, H, D, D)
    pool.copy_(c.state)
    want = oracle.packed(P.host(c.mixed_qkv), P.host(c.raw_gate), P.host(c.raw_beta), P.host(c.A_log),
                         P.host(c.dt_bias), np_(c.state), np_(c.state_indices))
    out = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, pool,
                            c.state_indices)
    torch.cuda.synchronize()
    P.check_bf16_out(out, want["out64"])
    P.check_state(pool, want["state"])
    assert bool((store[:, H * D * D:] == 7.0).all()), "padding between slots was written"


def test_determinism_and_noncurrent_stream():
    say("determinism + side stream seed=5004")
    c = synth.packed_case(5004, B=40, H=12, num_slots=64, device=DEV, null_rows=3)
    s0 = c.state.clone()
    o1 = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                           c.state_indices)
    st1 = c.state.clone()
    c.state.copy_(s0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2 = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                               c.state_indices)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(P.bits(o1), P.bits(o2))
    assert torch.equal(P.bits(st1), P.bits(c.state))


def test_graph_replay_with_changed_inputs_and_indices():
    """Capture one packed decode into a HIP graph and replay it with new
    inputs and new indices copied into the captured buffers; every replay
    matches an eager call and the oracle."""
    say("hip graph replay packed H=12 B=16 bf16 seed=5005")
    B, H, S = 16, 12, 48
    c = synth.packed_case(5005, B=B, H=H, num_slots=S, device=DEV, null_rows=2)
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                          c.state_indices, output=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                          c.state_indices, output=out)
    torch.cuda.synchronize()
    for rep in range(3):
        n = synth.packed_case(6000 + rep, B=B, H=H, num_slots=S, device=DEV, null_rows=rep + 1)
        c.mixed_qkv.copy_(n.mixed_qkv)
        c.raw_gate.copy_(n.raw_gate)
        c.raw_beta.copy_(n.raw_beta)
        c.state_indices.copy_(n.state_indices)
        st0 = c.state.clone()
        torch.cuda.synchronize()
        want = oracle.packed(P.host(c.mixed_qkv), P.host(c.raw_gate), P.host(c.raw_beta),
                             P.host(c.A_log), P.host(c.dt_bias), np_(st0), np_(c.state_indices))
        graph.replay()
        torch.cuda.synchronize()
        got_out, got_state = out.clone(), c.state.clone()
        # eager on the same inputs
        c.state.copy_(st0)
        eager = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                                  c.state_indices)
        torch.cuda.synchronize()
        assert torch.equal(P.bits(got_out), P.bits(eager)), f"replay {rep} != eager"
        assert torch.equal(P.bits(got_state), P.bits(c.state)), f"replay {rep} state != eager"
        P.check_bf16_out(got_out, want["out64"], f"replay {rep}")
        P.check_state(got_state, want["state"], f"replay {rep} state")


def test_lower_bound_gate_is_rejected():
    say("unsupported bounded gate")
    c = synth.packed_case(5006, B=2, H=12, num_slots=4, device=DEV)
    with pytest.raises(KDAError) as ei:
        packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state,
                          c.state_indices, lower_bound=-5.0)
    assert ei.value.code == "KDA_ERR_UNSUPPORTED"


def test_512_step_drift_against_fp64():
    """512 chained T=1 decode steps on the same slots (fp32 pool on the GPU vs
    an fp64 pool in the oracle).  The pages give no bound; the drift is
    reported and checked against the fp32 state tolerance."""
    say("512-step drift H=4 N=4 seed=5007")
    N, H, steps = 4, 4, 512
    c = synth.recurrent_case(5007, n_seqs=N, H=H, num_slots=N, device=DEV)
    ref = np_(c.state).astype(np.float64)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(5007)
    worst_o = 0.0
    for step in range(steps):
        q = torch.randn((N, H, D), generator=gen).to(torch.bfloat16)
        k = torch.randn((N, H, D), generator=gen).to(torch.bfloat16)
        v = torch.randn((N, H, D), generator=gen).to(torch.bfloat16)
        g = torch.randn((N, H, D), generator=gen).to(torch.bfloat16)
        b = torch.randn((N, H), generator=gen).to(torch.bfloat16)
        w = oracle.recurrent(q, k, v, g, b, np_(c.A_log), np_(c.dt_bias), ref, np_(c.state_indices))
        ref = w["state"]
        out = recurrent_kda(q.reshape(N, 1, H, D).to(DEV), k.reshape(N, 1, H, D).to(DEV),
                            v.reshape(N, 1, H, D).to(DEV), g.reshape(N, 1, H, D).to(DEV),
                            b.reshape(N, 1, H).to(DEV), c.A_log, c.dt_bias, initial_state=c.state,
                            state_indices=c.state_indices)
        if step % 64 == 63 or step == steps - 1:
            o = out.float().cpu().numpy().reshape(N, H, D)
            worst_o = max(worst_o, float(np.abs(o - w["out64"]).max()))
    torch.cuda.synchronize()
    drift = float(np.abs(c.state.double().cpu().numpy() - ref).max())
    say(f"after {steps} steps: max |state - fp64| = {drift:.3e}, sampled max |out - fp64| = {worst_o:.3e}")
    assert drift <= 1e-4
    assert worst_o <= 2e-3


def test_varlen_graph_replay_with_changed_cu_seqlens():
    """The ragged call reads cu_seqlens and state_indices on the device at
    every launch: a captured graph replayed with other lengths (same token
    total, trailing empty sequences, a null sequence) matches eager calls."""
    say("hip graph replay varlen H=4 N=6 seed=5200")
    N, H, T = 6, 4, 12
    c = synth.recurrent_case(5200, n_seqs=N, H=H, num_slots=10, device=DEV,
                             lengths=[2, 2, 2, 2, 2, 2], indices="random")
    r1 = lambda t: t.reshape(1, T, *t.shape[1:])  # noqa: E731
    out = torch.zeros((1, T, H, D), dtype=torch.bfloat16, device=DEV)
    ck = torch.zeros((T, H, D, D), dtype=torch.float32, device=DEV)
    call = lambda st, o, k: recurrent_kda(  # noqa: E731
        r1(c.q), r1(c.k), r1(c.v), r1(c.g), r1(c.beta), c.A_log, c.dt_bias, initial_state=st,
        state_indices=c.state_indices, cu_seqlens=c.cu_seqlens, n_tokens=T, output=o,
        intermediate_states=k)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(c.state.clone(), out, ck)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(c.state, out, ck)
    torch.cuda.synchronize()
    layouts = [([0, 1, 2, 9, 12, 12, 12], [3, -1, 5, 0, 7, 8]),
               ([0, 0, 6, 6, 12, 12, 12], [1, 2, 3, 4, 5, 6]),
               ([0, 12, 12, 12, 12, 12, 12], [9, -1, -1, 2, 3, 4])]
    for rep, (cu, idx) in enumerate(layouts):
        c.cu_seqlens.copy_(torch.tensor(cu, dtype=torch.int32))
        c.state_indices.copy_(torch.tensor(idx, dtype=torch.int32))
        st0 = c.state.clone()
        out.zero_()
        ck.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g_out, g_st, g_ck = out.clone(), c.state.clone(), ck.clone()
        e_st = st0.clone()
        e_out = torch.zeros_like(out)
        e_ck = torch.zeros_like(ck)
        call(e_st, e_out, e_ck)
        torch.cuda.synchronize()
        assert torch.equal(P.bits(g_out), P.bits(e_out)), f"replay {rep}: output"
        assert torch.equal(P.bits(g_st), P.bits(e_st)), f"replay {rep}: state"
        assert torch.equal(P.bits(g_ck), P.bits(e_ck)), f"replay {rep}: checkpoints"
        want = oracle.recurrent(np_(c.q), np_(c.k), np_(c.v), np_(c.g), np_(c.beta), np_(c.A_log),
                                np_(c.dt_bias), np_(st0), np.array(idx, np.int32),
                                np.array(cu, np.int32), ckpt_dtype=oracle.F32)
        P.check_bf16_out(g_out, want["out64"], f"replay {rep}")
        P.check_state(g_st, want["state"], f"replay {rep} state")
        P.check_state(g_ck, want["ckpt"], f"replay {rep} checkpoints")


def test_fused_graph_replay():
    say("hip graph replay fused H=8 rows=6 seed=5300")
    rows, H, S = 6, 8, 12
    c = synth.fused_case(5300, rows=rows, H=H, num_slots=S, device=DEV, null_zero=1, null_neg=1)
    out = torch.empty((1, rows, H, D), dtype=torch.bfloat16, device=DEV)
    call = lambda: fused_kda_decode(c.x, c.weight, c.conv_state, c.raw_gate, c.raw_beta, c.A_log,  # noqa: E731
                                    c.dt_bias, c.state_indices, c.state, c.output_gate,
                                    c.norm_weight, output=out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        n = synth.fused_case(5400 + rep, rows=rows, H=H, num_slots=S, device=DEV, null_zero=1,
                             null_neg=rep)
        c.x.copy_(n.x)
        c.state_indices.copy_(n.state_indices)
        st0, cs0 = c.state.clone(), c.conv_state.clone()
        torch.cuda.synchronize()
        want = oracle.fused(P.host(c.x), P.host(c.weight), P.host(cs0), P.host(c.raw_gate),
                            P.host(c.raw_beta), P.host(c.A_log), P.host(c.dt_bias),
                            P.host(c.state_indices), np_(st0), P.host(c.output_gate),
                            P.host(c.norm_weight))
        graph.replay()
        torch.cuda.synchronize()
        P.check_bf16_out(out, want["out64"], f"fused replay {rep}")
        P.check_state(c.state, want["state"], f"fused replay {rep} state")
        got_cs = c.conv_state.cpu().contiguous().view(torch.int16)
        want_cs = torch.from_numpy(np.ascontiguousarray(want["conv_state"]).view(np.int16))
        assert torch.equal(got_cs, want_cs), f"fused replay {rep}: conv cache"


@pytest.mark.parametrize("row_pad", [1, 3])
def test_packed_odd_row_strides_and_independent_gate_strides(row_pad):
    """Zero-copy views: an odd QKV row stride (2-byte aligned rows) and raw
    gate / beta views with their own row strides."""
    say(f"packed odd strides row_pad={row_pad} seed=5500")
    B, H, S = 13, 12, 40
    c = synth.packed_case(5500 + row_pad, B=B, H=H, num_slots=S, device=DEV, null_rows=2,
                          row_pad=row_pad)
    gate_wide = torch.randn((B, H * D + 5), device=DEV).to(torch.bfloat16)
    beta_wide = torch.randn((B, H + 7), device=DEV).to(torch.bfloat16)
    rg, rb = gate_wide[:, 2:2 + H * D], beta_wide[:, 3:3 + H]
    assert rg.stride(0) == H * D + 5 and rb.stride(0) == H + 7
    want = oracle.packed(P.host(c.mixed_qkv), P.host(rg), P.host(rb), P.host(c.A_log),
                         P.host(c.dt_bias), np_(c.state), np_(c.state_indices))
    out = packed_kda_decode(c.mixed_qkv, rg, rb, c.A_log, c.dt_bias, c.state, c.state_indices)
    torch.cuda.synchronize()
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
