"""On the GPU: the facade refuses a host tensor in place of any device tensor
argument of the four calls, before the library is reached (ValueError naming
the argument), and the call with every tensor on the device runs."""
import pytest
import torch

from gated_delta_rule_decode_amd import (fused_kda_decode, packed_fused_kda_decode, packed_kda_decode,
                                         recurrent_kda, synth)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _recurrent():
    c = synth.recurrent_case(11, n_seqs=3, H=2, num_slots=4, lengths=[2, 0, 3], device=DEV)
    T = c.q.shape[0]
    u = lambda t: t.unsqueeze(0)  # noqa: E731
    return recurrent_kda, dict(q=u(c.q), k=u(c.k), v=u(c.v), g=u(c.g), beta=u(c.beta), A_log=c.A_log,
                               dt_bias=c.dt_bias, initial_state=c.state, state_indices=c.state_indices,
                               cu_seqlens=c.cu_seqlens,
                               output=torch.empty((1, T, 2, D), dtype=torch.bfloat16, device=DEV))


def _packed():
    c = synth.packed_case(12, B=3, H=2, num_slots=4, null_rows=1, device=DEV)
    return packed_kda_decode, dict(mixed_qkv=c.mixed_qkv, raw_gate=c.raw_gate, raw_beta=c.raw_beta,
                                   A_log=c.A_log, dt_bias=c.dt_bias, state=c.state,
                                   state_indices=c.state_indices,
                                   output=torch.empty((3, 1, 2, D), dtype=torch.bfloat16, device=DEV))


def _fused_common(c, rows):
    return dict(x=c.x, weight=c.weight, conv_state=c.conv_state, raw_gate=c.raw_gate, raw_beta=c.raw_beta,
                A_log=c.A_log, dt_bias=c.dt_bias, state_indices=c.state_indices, state=c.state,
                output_gate=c.output_gate, norm_weight=c.norm_weight,
                output=torch.empty((1, rows, 2, D), dtype=torch.bfloat16, device=DEV))


def _fused():
    c = synth.fused_case(13, rows=3, H=2, num_slots=5, null_zero=1, device=DEV)
    return fused_kda_decode, _fused_common(c, 3)


def _packed_fused():
    c = synth.packed_fused_case(14, lengths=[2, 1], H=2, num_slots=8, max_tokens=2, device=DEV)
    args = _fused_common(c, 3)
    args.update(query_start_loc=c.query_start_loc, num_accepted_tokens=c.num_accepted_tokens)
    return packed_fused_kda_decode, args


@pytest.mark.parametrize("make", [_recurrent, _packed, _fused, _packed_fused], ids=["recurrent", "packed", "fused",
                                                                                     "packed_fused"])
def test_host_tensor_arguments_are_refused_on_the_gpu(make):
    print("[case]", make.__name__, flush=True)
    fn, args = make()
    fn(**args)
    torch.cuda.synchronize()
    names = [n for n, t in args.items() if isinstance(t, torch.Tensor)]
    assert len(names) >= 8
    for name in names:
        if name == "output":
            continue  # a host output would simply be the one written to host memory: refused below too
        before = {n: t.clone() for n, t in args.items() if isinstance(t, torch.Tensor)}
        bad = dict(args)
        bad[name] = args[name].cpu()
        with pytest.raises(ValueError) as e:
            fn(**bad)
        assert name in str(e.value) or "HIP" in str(e.value), f"{name}: {e.value}"
        torch.cuda.synchronize()
        for n, t in before.items():
            assert torch.equal(t, args[n]), f"{n} changed although the call with a host {name} was refused"
    bad = dict(args)
    bad["output"] = args["output"].cpu()
    with pytest.raises(ValueError):
        fn(**bad)
