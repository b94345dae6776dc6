"""GPU parity of the WY verify kernel ("flashinfer.kda_decode", Frozen /
speculative-verify mode): read-only calls without checkpoints and with at
most 16 tokens per sequence (batched, or ragged with the longest sequence
declared), where the tokens' products with the slot's initial state are one
matrix product per head and the rest a forward substitution.  Against the
fp64 oracle on every output, cache entry and pool bit: token counts 2..16,
ragged lengths 0..16, fp32 and bf16 pools, in-kernel and precomputed gates
(bf16 and fp32), grouped value heads, null rows and an index past the pool,
caches shorter than, equal to and longer than the token count, decays so
strong that the cumulative decay underflows, and a sequence longer than the
declared length (its tokens past it give zeros and record nothing).
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import _lib, recurrent_kda, synth
from tests import parity as P
from tests.test_gpu_verify import call, check_caches, np_, recorded_mask, reference

pytestmark = pytest.mark.gpu
D = 128
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[case]", *a, flush=True)


def wy_plan_kernel(n, T, H, HV, slots, bf16):
    """Kernel family the library plans for a read-only batched call of this shape."""
    import ctypes
    a = _lib.RecurrentArgs()
    a.struct_size = ctypes.sizeof(_lib.RecurrentArgs)
    a.n_seqs, a.n_tokens, a.H, a.HV, a.K, a.V = n, n * T, H, HV, D, D
    base = 1 << 36
    nxt = [base]

    def take(nb):
        p = nxt[0]
        nxt[0] += (nb + 4096 + 255) & ~255
        return p
    for f, hh in (("q", H), ("k", H), ("v", HV), ("g", HV)):
        setattr(a, f, take(n * T * hh * D * 2))
        setattr(a, f + "_stride", hh * D)
    a.beta, a.beta_stride = take(n * T * HV * 2), HV
    a.A_log, a.dt_bias = take(HV * 4), take(HV * D * 4)
    a.scale, a.l2_eps = 0.08838834764831845, 1e-6
    a.state = take(slots * HV * D * D * (2 if bf16 else 4))
    a.state_dtype = a.ckpt_dtype = 1 if bf16 else 0
    a.num_slots, a.slot_stride = slots, HV * D * D
    a.state_indices = take(n * 4)
    a.out = take(n * T * HV * D * 2)
    a.g_dtype = a.beta_dtype = 1
    a.tokens_per_seq, a.flags = T, 1
    plan = _lib.LaunchPlan()
    plan.struct_size = ctypes.sizeof(_lib.LaunchPlan)
    assert _lib.load().kda_recurrent_plan(ctypes.byref(a), ctypes.byref(plan)) == 0
    return plan.kernel


CASES = [  # T, state dtype, gate, gate dtype, H, HV, cache length
    (2, torch.float32, "in_kernel", torch.bfloat16, 4, 4, 2),
    (2, torch.bfloat16, "in_kernel", torch.bfloat16, 4, 4, 3),
    (3, torch.bfloat16, "in_kernel", torch.bfloat16, 4, 8, 5),
    (4, torch.float32, "precomputed", torch.float32, 2, 8, 3),
    (3, torch.float32, "in_kernel", torch.bfloat16, 2, 4, 4),
    (4, torch.bfloat16, "precomputed", torch.float32, 4, 4, 4),
    (5, torch.bfloat16, "precomputed", torch.bfloat16, 4, 4, 5),
    (6, torch.float32, "in_kernel", torch.float32, 8, 8, 8),
    (7, torch.float32, "precomputed", torch.float32, 4, 12, 7),
    (8, torch.bfloat16, "in_kernel", torch.bfloat16, 4, 8, 8),
    (8, torch.float32, "in_kernel", torch.bfloat16, 6, 12, 6),
    (9, torch.float32, "in_kernel", torch.float32, 4, 4, 9),
    (10, torch.bfloat16, "in_kernel", torch.bfloat16, 2, 4, 16),
    (11, torch.bfloat16, "precomputed", torch.float32, 4, 8, 6),
    (12, torch.float32, "in_kernel", torch.bfloat16, 4, 8, 12),
    (12, torch.bfloat16, "in_kernel", torch.float32, 8, 8, 12),
    (13, torch.float32, "precomputed", torch.bfloat16, 4, 12, 5),
    (16, torch.bfloat16, "precomputed", torch.float32, 4, 4, 9),
    (16, torch.float32, "in_kernel", torch.bfloat16, 8, 8, 16),
    (16, torch.bfloat16, "in_kernel", torch.bfloat16, 4, 8, 16),
]


@pytest.mark.parametrize("T,state_dtype,gate,gate_dtype,H,HV,t_max", CASES,
                         ids=[f"T{c[0]}-{'bf16' if c[1] == torch.bfloat16 else 'fp32'}-{c[2]}-H{c[4]}HV{c[5]}"
                              f"-tmax{c[6]}" for c in CASES])
def test_wy_verify_against_oracle(T, state_dtype, gate, gate_dtype, H, HV, t_max):
    seed = 7600 + 10 * T + HV
    n, slots = 11, 24
    say(f"WY verify T={T} {state_dtype} gate={gate}/{gate_dtype} H={H} HV={HV} t_max={t_max} seed={seed}")
    assert wy_plan_kernel(n, T, H, HV, slots, state_dtype == torch.bfloat16) == 5
    c = synth.recurrent_case(seed, n_seqs=n, H=H, HV=HV, num_slots=slots, state_dtype=state_dtype, device=DEV,
                             indices="random", lengths=[T] * n, null_rows=2, gate=gate, gate_dtype=gate_dtype)
    c.state_indices[4] = slots + 5  # past the pool: null
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=t_max, ragged=False, read_only=True, tps=T)
    kg_dtype = torch.float32 if T % 2 else torch.bfloat16
    out, corr, kg, _ = call(c, form="batched", t_max=t_max, kg_dtype=kg_dtype, read_only=True, tps=T)
    assert torch.equal(P.bits(st0), P.bits(c.state)), "read-only pool changed"
    e1 = P.check_bf16_out(out, want["out64"])
    e2 = check_caches(corr, kg, want, recorded_mask(c, [T] * n, t_max))
    idx = c.state_indices.cpu().numpy()
    o = P.bits(out.reshape(n, T, HV, D).cpu())
    for i in range(n):
        if not (0 <= idx[i] < slots):
            assert not o[i].any(), "null rows must produce +0"
    say(f"out err {e1:.3e} corr err {e2:.3e}")


@pytest.mark.parametrize("T,state_dtype", [(2, torch.float32), (4, torch.float32), (6, torch.float32),
                                           (6, torch.bfloat16), (11, torch.float32), (16, torch.float32)])
def test_wy_verify_with_underflowing_decay(T, state_dtype):
    """Log-decays of -20..-90 per token: the cumulative decay underflows to
    zero in fp32 within a token or two; outputs and corrections stay finite
    and match the oracle (every product form: fp32 4x4x1 at 2 and 4 tokens,
    16x16x4 at 6, the bf16 split at 11 (12 token slots) and 16, bf16 pools)."""
    n, H, slots = 7, 4, 12
    say(f"WY verify underflowing decay T={T} H={H} {state_dtype} seed=7700")
    c = synth.recurrent_case(7700, n_seqs=n, H=H, num_slots=slots, state_dtype=state_dtype, device=DEV,
                             indices="random", lengths=[T] * n, gate="precomputed", gate_dtype=torch.float32)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7700)
    c.g.copy_(-(20.0 + 70.0 * torch.rand(c.g.shape, generator=gen, device=DEV)))
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=T, ragged=False, read_only=True, tps=T)
    out, corr, kg, _ = call(c, form="batched", t_max=T, kg_dtype=torch.float32, read_only=True, tps=T)
    assert torch.isfinite(out.float()).all() and torch.isfinite(corr).all()
    P.check_bf16_out(out, want["out64"])
    check_caches(corr, kg, want, recorded_mask(c, [T] * n, T))


def test_wy_and_sequential_forms_agree():
    """The same tokens through the WY read-only kernel and through the
    sequential token loop (an updating call on a copy of the pool) give
    outputs within the bf16 bar of each other, and the read-only call leaves
    its pool untouched."""
    T, n, H = 4, 16, 8
    say(f"WY vs sequential T={T} H={H} seed=7800")
    c = synth.recurrent_case(7800, n_seqs=n, H=H, num_slots=20, device=DEV, indices="random", lengths=[T] * n)
    st0 = c.state.clone()
    shp = lambda t: t.reshape(n, T, *t.shape[1:])  # noqa: E731
    args = [shp(c.q), shp(c.k), shp(c.v), shp(c.g), shp(c.beta), c.A_log, c.dt_bias]
    o_wy = recurrent_kda(*args, initial_state=c.state, state_indices=c.state_indices,
                            disable_state_update=True)
    pool2 = st0.clone()
    o_seq = recurrent_kda(*args, initial_state=pool2, state_indices=c.state_indices)
    torch.cuda.synchronize()
    assert torch.equal(P.bits(st0), P.bits(c.state))
    want = oracle.recurrent(np_(c.q), np_(c.k), np_(c.v), np_(c.g), np_(c.beta), np_(c.A_log), np_(c.dt_bias),
                            np_(st0), np_(c.state_indices), None, update_state=False, tokens_per_seq=T)
    P.check_bf16_out(o_wy, want["out64"])
    P.check_bf16_out(o_seq, want["out64"])
    diff = (o_wy.float() - o_seq.float()).abs().max().item()
    assert diff <= 2 * P.OUT_ATOL, diff
    assert np.isfinite(diff)


def test_wy_verify_graph_replay_with_new_inputs_and_indices():
    """A captured read-only T=4 call replays with new token inputs and slot
    indices written into its buffers (metadata is read on the device):
    every replay equals the same call made eagerly, bit for bit."""
    T, n, H, slots = 4, 12, 4, 40
    say(f"WY verify graph replay T={T} H={H} seed=7900")
    c = synth.recurrent_case(7900, n_seqs=n, H=H, num_slots=slots, device=DEV, indices="random", lengths=[T] * n)
    shp = lambda t: t.reshape(n, T, *t.shape[1:])  # noqa: E731
    bufs = [shp(c.q).clone(), shp(c.k).clone(), shp(c.v).clone(), shp(c.g).clone(), shp(c.beta).clone()]
    idx = c.state_indices.clone()
    out = torch.empty((n, T, H, D), dtype=torch.bfloat16, device=DEV)

    def run(o):
        return recurrent_kda(*bufs, c.A_log, c.dt_bias, initial_state=c.state, state_indices=idx, output=o,
                             disable_state_update=True)
    run(out)  # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(out)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7901)
    for rep in range(3):
        for b in bufs:
            b.copy_(torch.randn(b.shape, generator=gen, device=DEV).to(b.dtype))
        idx.copy_(torch.randperm(slots, generator=gen, device=DEV)[:n].to(torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(out)
        run(eager)
        torch.cuda.synchronize()
        assert torch.equal(P.bits(out), P.bits(eager)), f"replay {rep} differs from the eager call"


def ragged_plan_kernel(lengths, H, HV, slots, bf16, max_seqlen):
    """Kernel family planned for a read-only ragged call declaring max_seqlen."""
    import ctypes
    n, T = len(lengths), int(sum(lengths))
    a = _lib.RecurrentArgs()
    a.struct_size = ctypes.sizeof(_lib.RecurrentArgs)
    a.n_seqs, a.n_tokens, a.H, a.HV, a.K, a.V = n, T, H, HV, D, D
    base, step = 1 << 36, 1 << 28
    for i, f in enumerate(("q", "k", "v", "g", "beta", "A_log", "dt_bias", "state", "state_indices", "cu_seqlens",
                           "out")):
        setattr(a, f, base + i * step)
    a.q_stride = a.k_stride = H * D
    a.v_stride = a.g_stride = HV * D
    a.beta_stride = HV
    a.scale, a.l2_eps = 0.08838834764831845, 1e-6
    a.state_dtype = a.ckpt_dtype = 1 if bf16 else 0
    a.num_slots, a.slot_stride = slots, HV * D * D
    a.g_dtype = a.beta_dtype = 1
    a.tokens_per_seq, a.flags = max_seqlen, 1
    plan = _lib.LaunchPlan()
    plan.struct_size = ctypes.sizeof(_lib.LaunchPlan)
    assert _lib.load().kda_recurrent_plan(ctypes.byref(a), ctypes.byref(plan)) == 0, _lib.load().kda_last_error()
    return plan.kernel


RAGGED = [  # max_seqlen, state dtype, gate, gate dtype, H, HV, cache length, seed
    (3, torch.float32, "in_kernel", torch.bfloat16, 4, 4, 3, 7610),
    (6, torch.bfloat16, "in_kernel", torch.bfloat16, 4, 8, 4, 7611),
    (8, torch.float32, "precomputed", torch.float32, 2, 8, 8, 7612),
    (12, torch.bfloat16, "precomputed", torch.bfloat16, 4, 4, 12, 7613),
    (10, torch.float32, "in_kernel", torch.bfloat16, 4, 8, 10, 7616),
    (16, torch.float32, "in_kernel", torch.bfloat16, 4, 8, 7, 7614),
    (16, torch.bfloat16, "in_kernel", torch.float32, 8, 8, 16, 7615),
]


@pytest.mark.parametrize("L,state_dtype,gate,gate_dtype,H,HV,t_max,seed", RAGGED,
                         ids=[f"L{c[0]}-{'bf16' if c[1] == torch.bfloat16 else 'fp32'}-{c[2]}-HV{c[5]}" for c in RAGGED])
def test_ragged_verify_against_oracle(L, state_dtype, gate, gate_dtype, H, HV, t_max, seed):
    """Ragged read-only calls (cu_seqlens) declaring their longest sequence:
    lengths 0..L (one sequence exactly L), null rows and an index past the
    pool, verify caches; every output, cache entry and pool bit against the
    oracle."""
    import random
    rng = random.Random(seed)
    n, slots = 12, 30
    lengths = [rng.randint(0, L) for _ in range(n)]
    lengths[rng.randrange(n)] = L
    say(f"ragged WY verify L={L} lengths={lengths} {state_dtype} gate={gate}/{gate_dtype} H={H} HV={HV} "
        f"t_max={t_max} seed={seed}")
    assert ragged_plan_kernel(lengths, H, HV, slots, state_dtype == torch.bfloat16, L) == 5
    c = synth.recurrent_case(seed, n_seqs=n, H=H, HV=HV, num_slots=slots, state_dtype=state_dtype, device=DEV,
                             indices="random", lengths=lengths, null_rows=2, gate=gate, gate_dtype=gate_dtype)
    c.state_indices[3] = slots + 2  # past the pool: null
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=t_max, ragged=True, read_only=True)
    out, corr, kg, _ = call(c, form="ragged", t_max=t_max, kg_dtype=torch.float32, read_only=True, max_seqlen=L)
    assert torch.equal(P.bits(st0), P.bits(c.state)), "read-only pool changed"
    e1 = P.check_bf16_out(out, want["out64"])
    e2 = check_caches(corr, kg, want, recorded_mask(c, lengths, t_max))
    say(f"out err {e1:.3e} corr err {e2:.3e}")


def test_ragged_verify_sequence_longer_than_declared():
    """A ragged read-only call declaring 4 tokens with one sequence of 7: its
    first 4 tokens and every other sequence match the oracle; its tokens 4..6
    give +0 and record nothing in the caches."""
    lengths = [3, 7, 0, 4, 2]
    n, H, slots, t_max = len(lengths), 4, 12, 8
    say(f"ragged WY verify with a sequence past the declared length lengths={lengths} seed=7620")
    c = synth.recurrent_case(7620, n_seqs=n, H=H, num_slots=slots, device=DEV, indices="random", lengths=lengths)
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=t_max, ragged=True, read_only=True)
    out, corr, kg, _ = call(c, form="ragged", t_max=t_max, kg_dtype=torch.float32, read_only=True, max_seqlen=4)
    cu = c.cu_seqlens.cpu().numpy()
    over = np.zeros(int(cu[-1]), bool)
    over[cu[1] + 4:cu[2]] = True  # tokens 4..6 of sequence 1
    o = out.reshape(-1, H, D)
    assert not P.bits(o[torch.from_numpy(over).to(DEV)]).any(), "tokens past the declared length must be +0"
    P.check_bf16_out(o[torch.from_numpy(~over).to(DEV)], want["out64"][~over])
    recorded = [min(x, 4) for x in lengths]
    check_caches(corr, kg, {"corr": want["corr"], "kg": want["kg"]}, recorded_mask(c, recorded, t_max))
    assert torch.equal(P.bits(st0), P.bits(c.state))


def test_wy_verify_t16_with_underflowing_decay():
    """Sixteen tokens with log-decays of -20..-90 each: the cumulative decay
    underflows within a token or two; outputs and corrections stay finite and
    match the oracle (batched, bf16 pool)."""
    T, n, H, slots = 16, 5, 4, 8
    say(f"WY verify underflowing decay T={T} H={H} seed=7710")
    c = synth.recurrent_case(7710, n_seqs=n, H=H, num_slots=slots, state_dtype=torch.bfloat16, device=DEV,
                             indices="random", lengths=[T] * n, gate="precomputed", gate_dtype=torch.float32)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7710)
    c.g.copy_(-(20.0 + 70.0 * torch.rand(c.g.shape, generator=gen, device=DEV)))
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=T, ragged=False, read_only=True, tps=T)
    out, corr, kg, _ = call(c, form="batched", t_max=T, kg_dtype=torch.float32, read_only=True, tps=T)
    assert torch.isfinite(out.float()).all() and torch.isfinite(corr).all()
    P.check_bf16_out(out, want["out64"])
    check_caches(corr, kg, want, recorded_mask(c, [T] * n, T))


STRIDED = [  # T, state dtype, ragged
    (4, torch.float32, False),
    (8, torch.float32, False),
    (16, torch.float32, False),
    (16, torch.bfloat16, False),
    (12, torch.float32, True),
]


@pytest.mark.parametrize("T,state_dtype,ragged", STRIDED,
                         ids=[f"T{c[0]}-{'bf16' if c[1] == torch.bfloat16 else 'fp32'}-{'ragged' if c[2] else 'batched'}"
                              for c in STRIDED])
def test_wy_verify_with_strided_inputs(T, state_dtype, ragged):
    """Token inputs read through padded row strides: q, k, v and the gate
    as column blocks of one bf16 row per token (with padding between
    tokens), beta as the first HV entries of a wider row.  The kernel
    addresses a sequence's rows by 32-bit offsets from its first row; the
    results equal the oracle on the same values, and the pool is untouched."""
    import random
    n, H, HV, slots, t_max = 6, 4, 8, 16, T
    seed = 7800 + T + (1 if ragged else 0)
    if ragged:
        rng = random.Random(seed)
        lengths = [rng.randint(0, T) for _ in range(n)]
        lengths[0] = T
    else:
        lengths = [T] * n
    say(f"WY verify strided inputs T={T} {state_dtype} ragged={ragged} lengths={lengths} seed={seed}")
    c = synth.recurrent_case(seed, n_seqs=n, H=H, HV=HV, num_slots=slots, state_dtype=state_dtype, device=DEV,
                             indices="random", lengths=lengths, null_rows=1, gate="in_kernel",
                             gate_dtype=torch.bfloat16)
    Tt = c.q.shape[0]
    HC, VC = H * D, HV * D
    row = 2 * HC + 2 * VC + 96  # q | k | v | g | padding
    buf = torch.full((Tt, row), float("nan"), dtype=torch.bfloat16, device=DEV)
    q = buf[:, :HC].view(Tt, H, D)
    k = buf[:, HC:2 * HC].view(Tt, H, D)
    v = buf[:, 2 * HC:2 * HC + VC].view(Tt, HV, D)
    g = buf[:, 2 * HC + VC:2 * HC + 2 * VC].view(Tt, HV, D)
    for dst, src in ((q, c.q), (k, c.k), (v, c.v), (g, c.g)):
        dst.copy_(src)
    bbuf = torch.full((Tt, HV + 24), float("nan"), dtype=torch.bfloat16, device=DEV)
    beta = bbuf[:, :HV]
    beta.copy_(c.beta)
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=t_max, ragged=ragged, read_only=True, tps=1 if ragged else T)
    corr = torch.full((slots, HV, t_max, D), -777.0, dtype=torch.float32, device=DEV)
    if ragged:
        shp = lambda t: t.view(1, Tt, *t.shape[1:])  # noqa: E731
        out = recurrent_kda(shp(q), shp(k), shp(v), shp(g), shp(beta), c.A_log, c.dt_bias, initial_state=c.state,
                            state_indices=c.state_indices, cu_seqlens=c.cu_seqlens, disable_state_update=True,
                            correction_cache=corr, max_seqlen=T)
    else:
        shp = lambda t: t.view(n, T, *t.shape[1:])  # noqa: E731
        out = recurrent_kda(shp(q), shp(k), shp(v), shp(g), shp(beta), c.A_log, c.dt_bias, initial_state=c.state,
                            state_indices=c.state_indices, disable_state_update=True, correction_cache=corr)
    torch.cuda.synchronize()
    assert torch.equal(P.bits(st0), P.bits(c.state)), "read-only pool changed"
    e1 = P.check_bf16_out(out.reshape(Tt, HV, D), want["out64"])
    m = recorded_mask(c, lengths, t_max)
    got = corr.cpu().numpy().astype(np.float64)
    mm = np.broadcast_to(m[:, None, :], got.shape[:3])
    assert np.abs(got[mm] - want["corr"][mm]).max() <= P.F32_STATE_ATOL
    assert np.all(got[~mm] == -777.0)
    say(f"out err {e1:.3e}")
