"""The Python facade refuses a tensor argument that is not on the call's HIP
device before anything reaches the library (CPU only).

A host tensor's address handed to a kernel would fault the GPU instead of
raising, so every tensor argument of the four calls is checked.  Here the
facade's device type is switched to "cpu" so that a whole call can be built
from host tensors: with every tensor on the host the call passes validation
and reaches the library loader (replaced by one that raises a sentinel, so
nothing can launch); with any one tensor moved to another device (the meta
device) the call raises ValueError naming that argument and never reaches
the loader.  Prepared calls (``prepare``) launch exactly the struct an eager
call builds.
"""
import ctypes

import pytest
import torch

from gated_delta_rule_decode_amd import _lib, api, synth


class Reached(Exception):
    pass


@pytest.fixture(autouse=True)
def _host_device_type(monkeypatch):
    monkeypatch.setattr(api, "_DEVICE_TYPE", "cpu")

    def load(*a, **k):
        raise Reached()

    monkeypatch.setattr(_lib, "load", load)


def _meta(t):
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device="meta")


def _recurrent_args():
    c = synth.recurrent_case(1, n_seqs=3, H=2, num_slots=4, lengths=[2, 0, 3])
    T = c.q.shape[0]
    args = dict(q=c.q.unsqueeze(0), k=c.k.unsqueeze(0), v=c.v.unsqueeze(0), g=c.g.unsqueeze(0),
                beta=c.beta.unsqueeze(0), A_log=c.A_log, dt_bias=c.dt_bias, initial_state=c.state,
                state_indices=c.state_indices, cu_seqlens=c.cu_seqlens,
                output=torch.empty((1, T, 2, 128), dtype=torch.bfloat16),
                intermediate_states=torch.empty((T, 2, 128, 128), dtype=torch.float32),
                correction_cache=torch.empty((4, 2, 3, 128), dtype=torch.float32),
                kg_cache=torch.empty((4, 2, 3, 256), dtype=torch.float32))
    return api.recurrent_kda, args, "q"


def _packed_args():
    c = synth.packed_case(2, B=3, H=2, num_slots=4, null_rows=1)
    args = dict(mixed_qkv=c.mixed_qkv, raw_gate=c.raw_gate, raw_beta=c.raw_beta, A_log=c.A_log,
                dt_bias=c.dt_bias, state=c.state, state_indices=c.state_indices,
                output=torch.empty((3, 1, 2, 128), dtype=torch.bfloat16))
    return api.packed_kda_decode, args, "mixed_qkv"


def _fused_common(c, rows):
    return dict(x=c.x, weight=c.weight, conv_state=c.conv_state, raw_gate=c.raw_gate, raw_beta=c.raw_beta,
                A_log=c.A_log, dt_bias=c.dt_bias, state_indices=c.state_indices, state=c.state,
                output_gate=c.output_gate, norm_weight=c.norm_weight,
                output=torch.empty((1, rows, 2, 128), dtype=torch.bfloat16))


def _fused_args():
    c = synth.fused_case(3, rows=3, H=2, num_slots=5, null_zero=1)
    return api.fused_kda_decode, _fused_common(c, 3), "x"


def _packed_fused_args():
    c = synth.packed_fused_case(4, lengths=[2, 1], H=2, num_slots=8, max_tokens=2)
    args = _fused_common(c, 3)
    args.update(query_start_loc=c.query_start_loc, num_accepted_tokens=c.num_accepted_tokens, workspace=None)
    return api.packed_fused_kda_decode, args, "x"


CALLS = [_recurrent_args, _packed_args, _fused_args, _packed_fused_args]


@pytest.mark.parametrize("make", CALLS, ids=lambda f: f.__name__.strip("_").replace("_args", ""))
def test_host_tensors_reach_the_library_only_when_all_are_on_the_device(make):
    fn, args, _ = make()
    with pytest.raises(Reached):
        fn(**args)
    tensors = [n for n, t in args.items() if isinstance(t, torch.Tensor)]
    assert len(tensors) >= 8
    for name in tensors:
        bad = dict(args)
        bad[name] = _meta(args[name])
        with pytest.raises(ValueError) as e:
            fn(**bad)
        assert "meta" in str(e.value), f"{name}: {e.value}"


@pytest.mark.parametrize("make", CALLS, ids=lambda f: f.__name__.strip("_").replace("_args", ""))
def test_a_call_off_the_hip_device_type_is_refused(make, monkeypatch):
    monkeypatch.setattr(api, "_DEVICE_TYPE", "cuda")
    fn, args, first = make()
    with pytest.raises(ValueError, match="HIP"):
        fn(**args)


class RecordingLib:
    """Stands in for the library: records each entry point call's struct."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(ref, *rest):
            st = ctypes.cast(ref, ctypes.POINTER(_STRUCTS[name])).contents if name in _STRUCTS else None
            self.calls.append((name, bytes(st) if st is not None else None))
            return 0
        return fn


_STRUCTS = {"kda_recurrent": _lib.RecurrentArgs, "kda_packed_decode": _lib.PackedArgs,
            "kda_fused_decode": _lib.FusedArgs, "kda_packed_fused_decode": _lib.PackedFusedArgs,
            "kda_packed_fused_decode_noalloc": _lib.PackedFusedArgs}


@pytest.mark.parametrize("make", CALLS, ids=lambda f: f.__name__.strip("_").replace("_args", ""))
def test_prepared_call_launches_the_eager_struct(make, monkeypatch):
    """prepare() validates and builds the struct without launching; each
    call of the PreparedCall launches the same entry point with exactly the
    struct an eager call builds, and the prepared call keeps its tensors."""
    rec = RecordingLib()
    monkeypatch.setattr(_lib, "load", lambda *a, **k: rec)
    monkeypatch.setattr(api, "_launch", lambda fn, ref, dev, stream=None: fn(ref))
    fn, args, _ = make()
    call = api.prepare(fn, **args)
    assert rec.calls == [] and isinstance(call, api.PreparedCall)
    out = call()
    call()
    assert out is call.output and len(rec.calls) == 2 and rec.calls[0] == rec.calls[1]
    fn(**args)
    assert rec.calls[2] == rec.calls[0], "the prepared struct differs from the eager one"
    held = [t for t in args.values() if isinstance(t, torch.Tensor)]
    assert all(any(t is k for k in call._keep[1].values()) for t in held)


def test_max_seqlen_is_the_ragged_calls_declared_bound(monkeypatch):
    """``max_seqlen`` (the longest sequence a ragged read-only call declares,
    which selects the matrix-product verify form) reaches the library as
    tokens_per_seq; without it a ragged call passes 0 (undeclared); it is
    refused on the batched form and when negative."""
    rec = RecordingLib()
    monkeypatch.setattr(_lib, "load", lambda *a, **k: rec)
    monkeypatch.setattr(api, "_launch", lambda fn, ref, dev, stream=None: fn(ref))
    fn, args, _ = _recurrent_args()
    args = {k: v for k, v in args.items() if k not in ("intermediate_states",)}

    def tps_of(**kw):
        rec.calls.clear()
        fn(**args, disable_state_update=True, **kw)
        st = _lib.RecurrentArgs.from_buffer_copy(rec.calls[-1][1])
        return st.tokens_per_seq, st.flags

    assert tps_of() == (0, _lib.FLAG_NO_STATE_UPDATE)
    assert tps_of(max_seqlen=3) == (3, _lib.FLAG_NO_STATE_UPDATE)
    assert tps_of(max_seqlen=16)[0] == 16
    with pytest.raises(ValueError, match="max_seqlen"):
        fn(**args, max_seqlen=-1)
    c = synth.recurrent_case(5, n_seqs=2, H=2, num_slots=4, lengths=[3, 3])
    r = lambda t: t.reshape(2, 3, *t.shape[1:])  # noqa: E731
    batched = dict(q=r(c.q), k=r(c.k), v=r(c.v), g=r(c.g), beta=r(c.beta), A_log=c.A_log, dt_bias=c.dt_bias,
                   initial_state=c.state, state_indices=c.state_indices)
    with pytest.raises(ValueError, match="ragged"):
        fn(**batched, max_seqlen=3)
    rec.calls.clear()
    fn(**batched, disable_state_update=True)
    assert _lib.RecurrentArgs.from_buffer_copy(rec.calls[-1][1]).tokens_per_seq == 3
