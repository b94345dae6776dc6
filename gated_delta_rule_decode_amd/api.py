"""Python facade of libkda_mi355x.so (torch tensors in, C ABI underneath).

Only argument marshalling happens here: shapes, strides and dtypes are read
from the tensors, the output is allocated when the caller passes none, and
the call goes to the C library on the caller's current HIP stream.  Every
step of the decode runs in the library's gfx950 kernels; there is no
PyTorch or CPU fallback.

Call names and argument order follow the flashinfer KDA decode pages
("flashinfer.kda_decode" function table, "flashinfer.kda_decode.
fused_kda_decode" signature).  Deliberate differences: ``lower_bound``
defaults to None (the pages do not define the bounded gate, so passing a
number raises), and there is no ``backend`` / ``state_indices_mode``
selector because there is exactly one implementation.
"""
from __future__ import annotations

import ctypes
import math
import threading

import torch

from . import _lib

D = 128
_SCALE = 1.0 / math.sqrt(D)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _launch(fn, ref, dev, stream=None):
    """Call the library entry point `fn` with the argument struct `ref` on
    `stream` (default: the device's current stream), with `dev` current."""
    h = (torch.cuda.current_stream(dev) if stream is None else stream).cuda_stream
    if torch.cuda.current_device() == dev.index:
        rc = fn(ref, h)
    else:
        with torch.cuda.device(dev):
            rc = fn(ref, h)
    if rc:
        _lib.check(rc)


class PreparedCall:
    """One validated library call bound to its tensors (see ``prepare``).

    Calling it enqueues the same kernel with the same arguments again, on
    the device's current stream or the given one; the kernel reads the
    tensors' contents at that time.  It holds references to every tensor the
    call uses, which must stay where they are (no reallocation, no resize).
    Returns the call's output tensor."""

    __slots__ = ("_fn", "_args", "_ref", "_keep", "device", "output")

    def __init__(self, fn, args, device, output, keep):
        self._fn = fn
        self._args = args
        self._ref = ctypes.byref(args)
        self._keep = keep
        self.device = device
        self.output = output

    def __call__(self, stream=None):
        _launch(self._fn, self._ref, self.device, stream)
        return self.output


_PREPARING = threading.local()


def prepare(fn, *args, **kwargs):
    """Validate one call of ``fn`` (recurrent_kda, packed_kda_decode,
    fused_kda_decode, packed_fused_kda_decode or
    packed_fused_kda_decode_noalloc) with these arguments, without launching
    it, and return a PreparedCall that launches it.  The argument checks and
    the marshalling into the library's struct happen once here; each launch
    is then one library call (for eager serving loops whose buffers stay in
    place).  An output the call would allocate is allocated here, once."""
    _PREPARING.on = True
    try:
        call = fn(*args, **kwargs)
    finally:
        _PREPARING.on = False
    _need(isinstance(call, PreparedCall), lambda: f"{getattr(fn, '__name__', fn)} cannot be prepared")
    call._keep = (args, kwargs, call._keep)
    return call


def _run(name, a, dev, output, keep=()):
    """Launch entry point `name` with struct `a`, or, inside ``prepare``,
    return the PreparedCall that would."""
    fn = getattr(_lib.load(), name)
    if getattr(_PREPARING, "on", False):
        return PreparedCall(fn, a, dev, output, keep)
    _launch(fn, ctypes.byref(a), dev)
    return output


def _need(cond, msg):
    """Raise ValueError(msg) unless cond; msg may be a callable that builds
    the message (so that a passing check formats nothing)."""
    if not cond:
        raise ValueError(msg() if callable(msg) else msg)


def _state_dtype(state):
    if state.dtype == torch.float32:
        return _lib.DTYPE_F32
    if state.dtype == torch.bfloat16:
        return _lib.DTYPE_BF16
    raise ValueError(f"state dtype must be float32 or bfloat16, got {state.dtype}")


# Every tensor argument must live on one HIP device: a host tensor's address
# handed to a kernel would make the GPU fault instead of raising.
_DEVICE_TYPE = "cuda"


def _check_devices(ref, **named):
    """ref and every non-None tensor in ``named`` on ref's device, which must
    be a HIP device.  Returns that device."""
    dev = ref.device
    _need(dev.type == _DEVICE_TYPE, lambda: f"tensors must be on a HIP ({_DEVICE_TYPE}) device, got {dev}")
    # (on a HIP device: is_cuda and the device index, both plain attributes,
    # rather than a torch.device object per tensor)
    hip, index = dev.type == "cuda", ref.get_device()
    for name, t in named.items():
        if t is not None:
            _need(isinstance(t, torch.Tensor) and ((t.is_cuda and t.get_device() == index) if hip else t.device == dev),
                  lambda: f"{name} must be a tensor on {dev}, "
                  f"got {t.device if isinstance(t, torch.Tensor) else type(t).__name__}")
    return dev


def _check_pool(state, H):
    _need(state.dim() == 4 and tuple(state.shape[1:]) == (H, D, D),
          lambda: f"state must be [num_slots, {H}, 128, 128], got {tuple(state.shape)}")
    _need(state.stride(3) == 1 and state.stride(2) == D and state.stride(1) == D * D,
          "each slot's [H, 128, 128] block must be contiguous")


def _check_indices(idx, n):
    _need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.numel() == n,
          lambda: f"state_indices must be a contiguous int32 tensor with {n} elements")


def _gate_mode(lower_bound):
    if lower_bound is None:
        return _lib.GATE_SOFTPLUS, 0.0
    # Forwarded so the library reports KDA_ERR_UNSUPPORTED with its reason.
    return _lib.GATE_LOWER_BOUND, float(lower_bound)


def _dtype_code(t, name):
    if t.dtype == torch.bfloat16:
        return _lib.DTYPE_BF16
    if t.dtype == torch.float32:
        return _lib.DTYPE_F32
    raise ValueError(f"{name} must be bfloat16 or float32, got {t.dtype}")


def _tokens(t, name, heads, width, ragged):
    """(n_tokens, tokens_per_seq, token stride) of a per-token input whose
    inner [heads, width] block (or [heads] when width is None) is contiguous.
    Accepted: [T, ...]; [B, T, ...] (T tokens per sequence, T=1 is plain
    decode; the [B, T] dims must collapse to one stride); [1, T, ...] with
    cu_seqlens."""
    shape, st = t.shape, t.stride()
    inner = 1 if width is None else 2
    if width is None:
        _need(shape[-1] == heads and st[-1] == 1, lambda: f"{name} must end in a contiguous [{heads}] dim")
    else:
        _need(shape[-1] == width and shape[-2] == heads and st[-1] == 1 and st[-2] == width,
              lambda: f"{name} must end in a contiguous [{heads}, {width}] block")
    nlead = len(shape) - inner
    if nlead == 1:
        return shape[0], 1, st[0]
    _need(nlead == 2, lambda: f"{name} has an unsupported rank")
    B, T = shape[0], shape[1]
    if ragged:
        _need(B == 1, lambda: f"{name} must be [1, T, ...] with cu_seqlens")
        return T, 1, st[1]
    if T == 1:
        return B, 1, st[0]
    _need(st[0] == T * st[1], lambda: f"{name}: the [B, T] dims must collapse to one token stride")
    return B * T, T, st[1]


def recurrent_kda(q, k, v, g, beta, A_log=None, dt_bias=None, *, initial_state, state_indices,
                  cu_seqlens=None, n_tokens=None, scale=None, output=None, intermediate_states=None,
                  lower_bound=None, use_qk_l2norm_in_kernel=True, use_gate_in_kernel=None,
                  disable_state_update=False, l2_eps=1e-6, correction_cache=None, kg_cache=None,
                  max_seqlen=None):
    """Recurrent KDA decode ("flashinfer.kda_decode" function table).

    Forms: T=1 (q [B, 1, H, 128] or [B, H, 128]); batched T tokens per
    sequence (q [B, T, H, 128]); packed ragged (q [1, T, H, 128] with
    ``cu_seqlens`` int32 [N+1], empty sequences allowed; ``n_tokens`` defaults
    to T).  q, k have H heads; v, g [.., HV, 128] and beta [.., HV] have HV
    value heads, HV a multiple of H (value head hv reads q/k head
    hv // (HV // H)).  With ``use_gate_in_kernel`` (the default when A_log is
    given) g is the raw gate and beta the logits, A_log fp32 [HV] and
    dt_bias fp32 [HV*128]; otherwise g is the log-decay and beta is beta
    itself (bf16 or fp32 each).  The pool ``initial_state`` [num_slots, HV,
    128, 128] (fp32 or bf16) is updated in place at ``state_indices`` (int32,
    negative = null row) unless ``disable_state_update``.
    ``intermediate_states`` (optional, [T, HV, 128, 128], pool dtype) receives
    the state after every token.  Verify caches ("Frozen / speculative-verify
    mode"), each optional and indexed by pool slot: ``correction_cache`` fp32
    [num_slots, HV, T_max, 128] receives beta*u of token j of the sequence
    in that slot, ``kg_cache`` [num_slots, HV, T_max, 256] (fp32 or bf16) its
    raw key | raw gate; tokens j >= T_max and null rows record nothing.
    ``max_seqlen`` (ragged form only): the caller's bound on every sequence's
    length; a read-only call without intermediate states that declares at
    most 16 runs as one matrix product per head, and there the tokens of a
    longer sequence past the bound give zeros and record nothing.
    Returns the bf16 output [.., HV, 128].
    """
    _need(use_qk_l2norm_in_kernel, "only the in-kernel q/k L2 normalisation is implemented")
    _check_devices(q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt_bias, initial_state=initial_state,
                   state_indices=state_indices, cu_seqlens=cu_seqlens, output=output,
                   intermediate_states=intermediate_states, correction_cache=correction_cache,
                   kg_cache=kg_cache)
    if use_gate_in_kernel is None:
        use_gate_in_kernel = A_log is not None
    H = q.shape[-2]
    HV = v.shape[-2]
    state = initial_state
    _check_pool(state, HV)
    N = state_indices.numel()
    _check_indices(state_indices, N)
    ragged = cu_seqlens is not None
    if ragged:
        _need(cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous() and cu_seqlens.numel() == N + 1,
              "cu_seqlens must be a contiguous int32 tensor with N+1 elements")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t.dtype == torch.bfloat16, lambda: f"{name} must be a bf16 tensor")
    T, tps, sq = _tokens(q, "q", H, D, ragged)
    views = [_tokens(t, n, hh, D, ragged) for n, t, hh in (("k", k, H), ("v", v, HV), ("g", g, HV))]
    views.append(_tokens(beta, "beta", HV, None, ragged))
    for (Tn, tpn, _), n in zip(views, ("k", "v", "g", "beta")):
        _need(Tn == T and tpn == tps, lambda: f"{n} does not have the token layout of q")
    if ragged and n_tokens is not None:
        T = int(n_tokens)
    if ragged:
        _need(max_seqlen is None or int(max_seqlen) >= 0, "max_seqlen must be non-negative")
        tps = 0 if max_seqlen is None else int(max_seqlen)
    else:
        _need(max_seqlen is None, "max_seqlen applies to the ragged (cu_seqlens) form only")
    if use_gate_in_kernel:
        _need(A_log is not None and dt_bias is not None, "the in-kernel gate needs A_log and dt_bias")
        _need(g.dtype == torch.bfloat16 and beta.dtype == torch.bfloat16,
              "with the in-kernel gate, g and beta are bf16")
        _need(A_log.dtype == torch.float32 and A_log.is_contiguous() and A_log.numel() == HV,
              "A_log must be contiguous fp32 [HV]")
        _need(dt_bias.dtype == torch.float32 and dt_bias.is_contiguous() and dt_bias.numel() == HV * D,
              "dt_bias must be contiguous fp32 [HV*128]")
        gm, lb = _gate_mode(lower_bound)
    else:
        _need(lower_bound is None, "lower_bound applies to the in-kernel gate only")
        gm, lb = _lib.GATE_PRECOMPUTED, 0.0
    out_shape = tuple(v.shape)
    if output is None:
        output = torch.empty(out_shape, dtype=torch.bfloat16, device=q.device)
    else:
        _need(output.dtype == torch.bfloat16 and output.is_contiguous() and output.numel() == T * HV * D,
              "output must be a contiguous bf16 tensor with T*HV*128 elements")
    ck = intermediate_states
    if ck is not None:
        _need(ck.dtype == state.dtype and ck.is_contiguous() and ck.numel() == T * HV * D * D,
              "intermediate_states must be contiguous [T, HV, 128, 128] in the pool dtype")
    t_max = None
    for name, c, w in (("correction_cache", correction_cache, D), ("kg_cache", kg_cache, 2 * D)):
        if c is None:
            continue
        _need(c.is_contiguous() and c.dim() == 4 and c.shape[0] == state.shape[0]
              and c.shape[1] == HV and c.shape[3] == w,
              lambda: f"{name} must be contiguous [num_slots, HV, T_max, {w}]")
        _need(t_max is None or c.shape[2] == t_max, "the verify caches must share T_max")
        t_max = c.shape[2]
    if correction_cache is not None:
        _need(correction_cache.dtype == torch.float32, "correction_cache must be fp32")
    a = _lib.RecurrentArgs()
    a.struct_size = ctypes.sizeof(_lib.RecurrentArgs)
    a.n_seqs, a.n_tokens, a.H, a.HV, a.K, a.V = N, T, H, HV, D, D
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.q_stride = sq
    a.k_stride, a.v_stride, a.g_stride, a.beta_stride = (vw[2] for vw in views)
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.scale = _SCALE if scale is None else float(scale)
    a.l2_eps = float(l2_eps)
    a.gate_mode, a.lower_bound = gm, lb
    a.state, a.state_dtype, a.ckpt_dtype = _ptr(state), _state_dtype(state), _state_dtype(state)
    a.num_slots, a.slot_stride = state.shape[0], state.stride(0)
    a.state_indices = _ptr(state_indices)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.checkpoints = _ptr(ck)
    a.out = _ptr(output)
    a.g_dtype, a.beta_dtype = _dtype_code(g, "g"), _dtype_code(beta, "beta")
    a.tokens_per_seq = tps
    a.flags = _lib.FLAG_NO_STATE_UPDATE if disable_state_update else 0
    a.correction_cache, a.kg_cache = _ptr(correction_cache), _ptr(kg_cache)
    a.kg_dtype = _dtype_code(kg_cache, "kg_cache") if kg_cache is not None else _lib.DTYPE_F32
    a.cache_t_max = t_max or 0
    return _run("kda_recurrent", a, q.device, output)


def packed_kda_decode(mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, state, state_indices,
                      output=None, *, lower_bound=None):
    """Packed T=1 decode ("Serving-native packed Kimi K3 decode").

    mixed_qkv bf16 [B, 3*H*128] (q|k|v, channel-contiguous, any row stride),
    raw_gate bf16 [B, H*128], raw_beta bf16 [B, H], A_log fp32 [H],
    dt_bias fp32 [H*128], state [num_slots, H, 128, 128] (bf16 or fp32),
    state_indices int32 [B] (-1 inactive).  Returns bf16 [B, 1, H, 128].
    """
    _check_devices(mixed_qkv, raw_gate=raw_gate, raw_beta=raw_beta, A_log=A_log, dt_bias=dt_bias, state=state,
                   state_indices=state_indices, output=output)
    H = A_log.numel()
    B = mixed_qkv.shape[0]
    _check_pool(state, H)
    _check_indices(state_indices, B)
    _need(mixed_qkv.dtype == torch.bfloat16 and mixed_qkv.dim() == 2 and mixed_qkv.shape[1] == 3 * H * D
          and mixed_qkv.stride(1) == 1, "mixed_qkv must be bf16 [B, 3*H*128] with contiguous channels")
    rg = raw_gate.reshape(B, H * D) if raw_gate.is_contiguous() else raw_gate
    _need(rg.dtype == torch.bfloat16 and rg.dim() == 2 and tuple(rg.shape) == (B, H * D) and rg.stride(1) == 1,
          "raw_gate must be bf16 [B, H*128] with contiguous channels")
    rb = raw_beta.reshape(B, H) if raw_beta.is_contiguous() else raw_beta
    _need(rb.dtype == torch.bfloat16 and rb.dim() == 2 and tuple(rb.shape) == (B, H) and rb.stride(1) == 1,
          "raw_beta must be bf16 [B, H]")
    _need(A_log.dtype == torch.float32 and A_log.is_contiguous(), "A_log must be contiguous fp32 [H]")
    _need(dt_bias.dtype == torch.float32 and dt_bias.is_contiguous() and dt_bias.numel() == H * D,
          "dt_bias must be contiguous fp32 [H*128]")
    if output is None:
        output = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=mixed_qkv.device)
    else:
        _need(output.dtype == torch.bfloat16 and output.is_contiguous() and output.numel() == B * H * D,
              "output must be contiguous bf16 [B, 1, H, 128]")
    gm, lb = _gate_mode(lower_bound)
    a = _lib.PackedArgs()
    a.struct_size = ctypes.sizeof(_lib.PackedArgs)
    a.B, a.H = B, H
    a.mixed_qkv, a.qkv_stride = _ptr(mixed_qkv), mixed_qkv.stride(0)
    a.raw_gate, a.gate_stride = _ptr(rg), rg.stride(0)
    a.raw_beta, a.beta_stride = _ptr(rb), rb.stride(0)
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.gate_mode, a.lower_bound = gm, lb
    a.state, a.state_dtype = _ptr(state), _state_dtype(state)
    a.num_slots, a.slot_stride = state.shape[0], state.stride(0)
    a.state_indices = _ptr(state_indices)
    a.out = _ptr(output)
    return _run("kda_packed_decode", a, mixed_qkv.device, output)


def _fused_inputs(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias, state, output_gate,
                  norm_weight, norm_eps, output):
    """Checks shared by the fused calls; returns (H, rows, raw_gate, raw_beta,
    output_gate as (address, row stride) pairs, output)."""
    _check_devices(x, weight=weight, conv_state=conv_state, raw_gate=raw_gate, raw_beta=raw_beta, A_log=A_log,
                   dt_bias=dt_bias, state=state, output_gate=output_gate, norm_weight=norm_weight, output=output)
    H = A_log.numel()
    HC = H * D
    rows = x.shape[0]
    _check_pool(state, H)
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.shape[1] == 3 * HC and x.stride(1) == 1,
          "x must be bf16 [rows, 3*H*128] with contiguous channels")
    _need(weight.dtype == torch.float32 and weight.is_contiguous() and tuple(weight.shape) == (3, 4, HC),
          "weight must be contiguous fp32 [3, 4, H*128]")
    _need(conv_state.dtype == torch.bfloat16 and conv_state.dim() == 3
          and tuple(conv_state.shape[1:]) == (3 * HC, 3) and conv_state.stride(1) == 1
          and conv_state.stride(2) == 3 * HC, "conv_state must be bf16 [num_slots, 3*H*128, 3] "
          "with strides [slot_stride, 1, 3*H*128]")
    _need(conv_state.shape[0] == state.shape[0], "state and conv_state must have the same num_slots")

    def rows2d(t, name, width):
        """(address, row stride) of a [rows, width] bf16 input (any contiguous
        tensor of rows*width elements, or a 2-D one with contiguous rows)."""
        _need(t.dtype == torch.bfloat16, lambda: f"{name} must be bf16")
        if t.is_contiguous() and t.numel() == rows * width:
            return _ptr(t), width
        _need(t.dim() == 2 and tuple(t.shape) == (rows, width) and t.stride(1) == 1,
              lambda: f"{name} must be [rows, {width}] with a contiguous inner dimension")
        return _ptr(t), t.stride(0)

    rg = rows2d(raw_gate, "raw_gate", HC)
    rb = rows2d(raw_beta, "raw_beta", H)
    og = rows2d(output_gate, "output_gate", HC)
    _need(norm_weight.dtype == torch.float32 and norm_weight.is_contiguous() and norm_weight.numel() == D,
          "norm_weight must be contiguous fp32 [128]")
    _need(A_log.dtype == torch.float32 and A_log.is_contiguous(), "A_log must be contiguous fp32 [H]")
    _need(dt_bias.dtype == torch.float32 and dt_bias.is_contiguous() and dt_bias.numel() == HC,
          "dt_bias must be contiguous fp32 [H*128]")
    _need(norm_eps >= 0, "norm_eps must be non-negative")
    if output is None:
        output = torch.empty((1, rows, H, D), dtype=torch.bfloat16, device=x.device)
    else:
        _need(output.dtype == torch.bfloat16 and output.is_contiguous() and output.numel() == rows * HC,
              "output must be contiguous bf16 [1, rows, H, 128]")
    return H, rows, rg, rb, og, output


def fused_kda_decode(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias, state_indices,
                     state, output_gate, norm_weight, lower_bound=None, norm_eps=1e-5, output=None):
    """Fused decode ("flashinfer.kda_decode.fused_kda_decode"): width-4
    depthwise causal conv + SiLU over x, one KDA update, gated RMSNorm.

    x bf16 [rows, 3*H*128]; weight fp32 [3, 4, H*128]; conv_state bf16
    [num_slots, 3*H*128, 3] with strides [slot_stride, 1, 3*H*128]; raw_gate
    bf16 [1, rows, H, 128] or [rows, H, 128]; raw_beta bf16 [1, rows, H] or
    [rows, H]; state_indices int32 [rows] (non-positive = null); state
    [num_slots, H, 128, 128] fp32/bf16; output_gate bf16 [rows, H, 128] or
    [1, rows, H, 128]; norm_weight fp32 [128].  Returns bf16 [1, rows, H, 128].
    """
    _check_devices(x, state_indices=state_indices)
    H, rows, rg, rb, og, output = _fused_inputs(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias,
                                                state, output_gate, norm_weight, norm_eps, output)
    _check_indices(state_indices, rows)
    gm, lb = _gate_mode(lower_bound)
    a = _lib.FusedArgs()
    a.struct_size = ctypes.sizeof(_lib.FusedArgs)
    a.rows, a.H = rows, H
    a.x, a.x_stride = _ptr(x), x.stride(0)
    a.weight = _ptr(weight)
    a.conv_state, a.conv_slot_stride = _ptr(conv_state), conv_state.stride(0)
    a.raw_gate, a.gate_stride = rg
    a.raw_beta, a.beta_stride = rb
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.gate_mode, a.lower_bound = gm, lb
    a.state_indices = _ptr(state_indices)
    a.state, a.state_dtype = _ptr(state), _state_dtype(state)
    a.num_slots, a.slot_stride = state.shape[0], state.stride(0)
    a.output_gate, a.ogate_stride = og
    a.norm_weight, a.norm_eps = _ptr(norm_weight), float(norm_eps)
    a.out = _ptr(output)
    return _run("kda_fused_decode", a, x.device, output)


class PackedFusedWorkspace:
    """Workspace that lets packed_fused_kda_decode spread the work of one
    (sequence, head) over several workgroups when there are few of them:
    int32 arrival counters (zero between calls; the kernel leaves them zero)
    and fp32 unnormalised outputs.  It grows on demand, by at least doubling,
    and never frees a buffer it has handed out: a graph captured with an
    earlier, smaller buffer keeps using that memory when it is replayed.
    Calls that share one workspace must not overlap in time (use one per
    stream when calls run concurrently)."""

    def __init__(self, device):
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.counters = torch.zeros(0, dtype=torch.int32, device=self.device)
        self.partials = torch.empty(0, dtype=torch.float32, device=self.device)
        self._retired = []  # buffers replaced by larger ones, kept allocated

    def reserve(self, n_seqs, H, n_rows):
        nc, npart = n_seqs * H, max(n_rows, 1) * H * D
        if self.counters.numel() < nc:
            self._retired.append(self.counters)
            self.counters = torch.zeros(max(nc, 2 * self.counters.numel()), dtype=torch.int32, device=self.device)
        if self.partials.numel() < npart:
            self._retired.append(self.partials)
            self.partials = torch.empty(max(npart, 2 * self.partials.numel()), dtype=torch.float32,
                                        device=self.device)
        return self.counters, self.partials


# Default workspaces, one per (device, stream), so that calls on different
# streams never share arrival counters.  A call captured into a graph uses
# the workspace of its capture stream; if that workspace has to grow during
# the capture, the new buffers are allocated in the capture (a warm-up call on
# the capture stream avoids that).  Old buffers are never freed, so a graph
# keeps valid memory however the workspace grows later.
_AUTO_WORKSPACE = {}


def _auto_workspace(device):
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _AUTO_WORKSPACE.get(key)
    if ws is None:
        ws = _AUTO_WORKSPACE[key] = PackedFusedWorkspace(dev)
    return ws


def _packed_fused_args(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias, state_indices, state,
                       output_gate, norm_weight, lower_bound, norm_eps, output, query_start_loc,
                       num_accepted_tokens):
    """Checked argument struct of the packed fused calls (no split scratch
    set); returns (args, output, N, H, rows)."""
    _check_devices(x, state_indices=state_indices, query_start_loc=query_start_loc,
                   num_accepted_tokens=num_accepted_tokens)
    H, rows, rg, rb, og, output = _fused_inputs(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias,
                                                state, output_gate, norm_weight, norm_eps, output)
    si = state_indices if state_indices.dim() == 2 else state_indices.reshape(-1, 1)
    _need(si.dtype == torch.int32 and si.dim() == 2 and si.stride(1) == 1,
          "state_indices must be an int32 tensor [N, max_tokens] with contiguous columns")
    N, max_tokens = si.shape
    for name, t, n in (("query_start_loc", query_start_loc, N + 1), ("num_accepted_tokens", num_accepted_tokens, N)):
        _need(t.dtype == torch.int32 and t.is_contiguous() and t.numel() == n,
              lambda: f"{name} must be a contiguous int32 tensor with {n} elements")
    gm, lb = _gate_mode(lower_bound)
    a = _lib.PackedFusedArgs()
    a.struct_size = ctypes.sizeof(_lib.PackedFusedArgs)
    a.n_rows, a.n_seqs, a.H, a.max_tokens = rows, N, H, max_tokens
    a.x, a.x_stride = _ptr(x), x.stride(0)
    a.weight = _ptr(weight)
    a.conv_state, a.conv_slot_stride = _ptr(conv_state), conv_state.stride(0)
    a.raw_gate, a.gate_stride = rg
    a.raw_beta, a.beta_stride = rb
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.gate_mode, a.lower_bound = gm, lb
    a.state_indices, a.indices_stride = _ptr(si), si.stride(0)
    a.query_start_loc, a.num_accepted_tokens = _ptr(query_start_loc), _ptr(num_accepted_tokens)
    a.state, a.state_dtype = _ptr(state), _state_dtype(state)
    a.num_slots, a.slot_stride = state.shape[0], state.stride(0)
    a.output_gate, a.ogate_stride = og
    a.norm_weight, a.norm_eps = _ptr(norm_weight), float(norm_eps)
    a.out = _ptr(output)
    return a, output, N, H, rows


def packed_fused_kda_decode(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias, state_indices,
                            state, output_gate, norm_weight, lower_bound=None, norm_eps=1e-5, output=None,
                            *, query_start_loc, num_accepted_tokens, workspace="auto"):
    """Packed fused decode with T >= 1 tokens per sequence ("feat(kda): add
    fused speculative decode kernel").

    The fused step (conv + SiLU, KDA, gated RMSNorm) over packed rows: x
    [rows, 3*H*128], raw_gate, raw_beta, output_gate per row as in
    fused_kda_decode.  ``query_start_loc`` int32 [N+1] (non-decreasing): the
    rows of sequence i; ``state_indices`` int32 [N, max_tokens] (or [N]):
    column j is the slot that receives the conv window and the state after
    token j (non-positive: not written); ``num_accepted_tokens`` int32 [N]:
    sequence i starts from the slot in column num_accepted_tokens[i] - 1 (a
    non-positive start slot makes the sequence null).  Rows of null sequences
    and rows outside every sequence give zeros.  A bf16 pool holds each
    checkpoint rounded; the recurrence itself stays fp32 across the tokens.
    ``workspace``: "auto" (a PackedFusedWorkspace per device and stream; a
    captured call uses its capture stream's), a PackedFusedWorkspace, or
    None (one workgroup per (sequence, head)); only calls that split their
    heads take workspace memory.
    Returns bf16 [1, rows, H, 128].
    """
    a, output, N, H, rows = _packed_fused_args(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias,
                                               state_indices, state, output_gate, norm_weight, lower_bound,
                                               norm_eps, output, query_start_loc, num_accepted_tokens)
    if isinstance(workspace, str):
        _need(workspace == "auto", 'workspace must be "auto", a PackedFusedWorkspace or None')
        workspace = _auto_workspace(x.device)
    lib = _lib.load()
    if workspace is not None:
        _need(isinstance(workspace, PackedFusedWorkspace) and workspace.device == x.device,
              "workspace must be a PackedFusedWorkspace on the device of x")
        # only a call that would split its heads takes (and may grow) the workspace
        cb, pb = ctypes.c_int64(), ctypes.c_int64()
        _lib.check(lib.kda_packed_fused_workspace(ctypes.byref(a), ctypes.byref(cb), ctypes.byref(pb)))
        if cb.value:
            cnt, part = workspace.reserve(N, H, rows)
            a.split_counters, a.split_partials = _ptr(cnt), _ptr(part)
    return _run("kda_packed_fused_decode", a, x.device, output, keep=(workspace,))


def packed_fused_kda_decode_noalloc(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias, state_indices,
                                    state, output_gate, norm_weight, lower_bound=None, norm_eps=1e-5, *,
                                    output, query_start_loc, num_accepted_tokens):
    """packed_fused_kda_decode for callers that cannot allocate: nothing is
    allocated, neither here (``output`` is required) nor in the library,
    whose split heads use a scratch array it holds per device.  Calls on one
    device must not overlap in time (they share that array).  A call that
    would split its heads over more than 1024 (sequence, head) pairs or 8192
    (row, head) pairs is rejected (KDAError, KDA_ERR_SHAPE)."""
    _need(output is not None, "output is required: this call allocates nothing")
    a, output, _, _, _ = _packed_fused_args(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias,
                                            state_indices, state, output_gate, norm_weight, lower_bound,
                                            norm_eps, output, query_start_loc, num_accepted_tokens)
    return _run("kda_packed_fused_decode_noalloc", a, x.device, output)
