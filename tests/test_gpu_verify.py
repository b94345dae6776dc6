"""GPU parity of the speculative-verify caches ("flashinfer.kda_decode",
Frozen / speculative-verify mode) against the fp64 oracle.

correction_cache [num_slots, HV, T_max, 128] holds beta*u of token j of the
sequence in that slot and kg_cache [num_slots, HV, T_max, 256] its raw key |
raw gate.  Recorded entries: corrections within the fp32 state tolerance
(1e-4), key|gate bit-exact (they are inputs copied, or rounded once to bf16
with round-to-nearest-even).  Entries that nothing records (free slots,
positions >= T_max, null and empty sequences) keep a sentinel bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import recurrent_kda, synth
from tests import parity as P

pytestmark = pytest.mark.gpu
D = 128
DEV = "cuda:0"
SENTINEL = 7.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[case]", *a, flush=True)


def np_(t):
    return None if t is None else oracle.as_np(t.detach().cpu())


def recorded_mask(c, lengths, t_max):
    """[num_slots, T_max] True where some live sequence records token j."""
    S = c.state.shape[0]
    mask = np.zeros((S, t_max), bool)
    idx = c.state_indices.cpu().numpy()
    for i, n in enumerate(lengths):
        if 0 <= idx[i] < S:
            mask[idx[i], :min(n, t_max)] = True
    return mask


def call(c, *, form, t_max, kg_dtype, read_only, ckpt=False, tps=None, max_seqlen=None):
    T, HV = c.q.shape[0], c.v.shape[1]
    S = c.state.shape[0]
    corr = torch.full((S, HV, t_max, D), SENTINEL, dtype=torch.float32, device=DEV)
    kg = torch.full((S, HV, t_max, 2 * D), SENTINEL, dtype=kg_dtype, device=DEV)
    if form == "t1":
        shp = lambda t: t.reshape(T, 1, *t.shape[1:])  # noqa: E731
        cu = None
    elif form == "ragged":
        shp = lambda t: t.reshape(1, T, *t.shape[1:])  # noqa: E731
        cu = c.cu_seqlens
    else:
        shp = lambda t: t.reshape(T // tps, tps, *t.shape[1:])  # noqa: E731
        cu = None
    ck = torch.zeros((T, HV, D, D), dtype=c.state.dtype, device=DEV) if ckpt else None
    out = recurrent_kda(shp(c.q), shp(c.k), shp(c.v), shp(c.g), shp(c.beta), c.A_log, c.dt_bias,
                        initial_state=c.state, state_indices=c.state_indices, cu_seqlens=cu,
                        intermediate_states=ck, disable_state_update=read_only,
                        correction_cache=corr, kg_cache=kg, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    return out, corr, kg, ck


def reference(c, st0, *, t_max, ragged, read_only, tps=1, ckpt_dtype=None):
    return oracle.recurrent(np_(c.q), np_(c.k), np_(c.v), np_(c.g), np_(c.beta), np_(c.A_log),
                            np_(c.dt_bias), st0, np_(c.state_indices),
                            np_(c.cu_seqlens) if ragged else None,
                            gate="in_kernel" if c.A_log is not None else "precomputed",
                            update_state=not read_only, tokens_per_seq=tps, t_max=t_max,
                            ckpt_dtype=ckpt_dtype)


def check_caches(corr, kg, want, mask):
    """mask [num_slots, T_max]: recorded positions (all value heads)."""
    got_c = corr.cpu().numpy().astype(np.float64)
    m = np.broadcast_to(mask[:, None, :], got_c.shape[:3])
    assert m.any()
    err = np.abs(got_c[m] - want["corr"][m])
    worst = float(err.max())
    assert worst <= P.F32_STATE_ATOL, f"correction_cache: max err {worst:.3e} > 1e-4"
    assert np.all(got_c[~m] == SENTINEL), "correction_cache written where nothing records"
    if kg.dtype == torch.float32:
        got_k = kg.cpu().numpy()
        want_k = want["kg"].astype(np.float32)
        assert np.array_equal(got_k[m], want_k[m]), "kg_cache differs from raw key | gate"
        assert np.all(got_k[~m] == SENTINEL)
    else:
        got_k = P.bits(kg.cpu()).numpy().astype(np.uint16)
        want_k = oracle.bf16_from_f64(want["kg"])
        assert np.array_equal(got_k[m], want_k[m]), "kg_cache (bf16) differs from raw key | gate"
        sent = P.bits(torch.tensor([SENTINEL], dtype=torch.bfloat16)).numpy().astype(np.uint16)[0]
        assert np.all(got_k[~m] == sent)
    return worst


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("kg_dtype", [torch.float32, torch.bfloat16])
def test_verify_ragged_read_only(state_dtype, kg_dtype):
    say(f"verify caches ragged read-only {state_dtype} kg {kg_dtype} seed=7000")
    lengths = [4, 0, 3, 6, 1, 4, 2]
    t_max = 4
    c = synth.recurrent_case(7000, n_seqs=len(lengths), H=4, HV=8, num_slots=16, state_dtype=state_dtype,
                             device=DEV, indices="random", lengths=lengths, null_rows=2)
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=t_max, ragged=True, read_only=True)
    out, corr, kg, _ = call(c, form="ragged", t_max=t_max, kg_dtype=kg_dtype, read_only=True)
    assert torch.equal(P.bits(st0), P.bits(c.state)), "read-only pool changed"
    P.check_bf16_out(out, want["out64"])
    check_caches(corr, kg, want, recorded_mask(c, lengths, t_max))


@pytest.mark.parametrize("kg_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("form", ["t1", "batched"])
def test_verify_precomputed_gate(form, kg_dtype):
    """fp32 log-decay gates: kept exactly in an fp32 kg cache, rounded once
    (RNE) in a bf16 one."""
    say(f"verify caches precomputed fp32 gate {form} kg {kg_dtype} seed=7100")
    tps = 1 if form == "t1" else 3
    n = 23 if form == "t1" else 9
    lengths = None if form == "t1" else [tps] * n
    c = synth.recurrent_case(7100, n_seqs=n, H=8, num_slots=32, device=DEV, indices="random",
                             lengths=lengths, gate="precomputed", gate_dtype=torch.float32, null_rows=2)
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=2, ragged=False, read_only=False, tps=tps)
    out, corr, kg, _ = call(c, form=form, t_max=2, kg_dtype=kg_dtype, read_only=False, tps=tps)
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
    check_caches(corr, kg, want, recorded_mask(c, [tps] * n, 2))


def test_verify_caches_rebuild_gpu_checkpoints():
    """Property at the verify workload's head count: the GPU's own caches and
    the initial state rebuild the GPU's per-token checkpoints,
    S_j = diag(exp(g_j)) S_{j-1} + k_hat_j c_j^T (precomputed gate)."""
    say("verify caches rebuild checkpoints H=32 B=16 T=4 seed=7200")
    B, T, H = 16, 4, 32
    c = synth.recurrent_case(7200, n_seqs=B, H=H, num_slots=64, device=DEV, indices="random",
                             lengths=[T] * B, gate="precomputed", gate_dtype=torch.float32)
    st0 = c.state.clone()
    out, corr, kg, ck = call(c, form="batched", t_max=T, kg_dtype=torch.float32, read_only=True,
                             ckpt=True, tps=T)
    idx = c.state_indices.long()
    S = st0[idx].double()                         # [B, H, v, k]
    kgd = kg[idx].double()                        # [B, H, T, 256]
    cd = corr[idx].double()                       # [B, H, T, 128] (indexed by v)
    ckd = ck.double().reshape(B, T, H, D, D)
    worst = 0.0
    for j in range(T):
        kraw = kgd[:, :, j, :D]
        kh = kraw / torch.sqrt((kraw * kraw).sum(-1, keepdim=True) + 1e-6)
        dec = torch.exp(kgd[:, :, j, D:])
        S = S * dec[:, :, None, :] + cd[:, :, j, :, None] * kh[:, :, None, :]
        worst = max(worst, (S - ckd[:, j]).abs().max().item())
    assert worst <= 1e-4, worst


def test_verify_full_workload_b64_t4_h32():
    """The verify workload itself (64 sequences x 4 draft tokens, 32 heads,
    fp32 pool of 128 slots, read only) against the oracle, every element."""
    say("verify caches B=64 T=4 H=32 read-only seed=7300")
    B, T, H = 64, 4, 32
    c = synth.recurrent_case(7300, n_seqs=B, H=H, num_slots=128, device=DEV, indices="random",
                             lengths=[T] * B)
    st0 = c.state.clone()
    want = reference(c, np_(st0), t_max=T, ragged=False, read_only=True, tps=T)
    out, corr, kg, _ = call(c, form="batched", t_max=T, kg_dtype=torch.float32, read_only=True, tps=T)
    P.check_bf16_out(out, want["out64"])
    assert torch.equal(P.bits(st0), P.bits(c.state))
    check_caches(corr, kg, want, recorded_mask(c, [T] * B, T))
