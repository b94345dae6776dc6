"""Seeded synthetic inputs for the KDA decode workloads.

This module only draws random tensors with the shapes, dtypes and value
distributions of the KDA decode workloads (Kimi-Linear / Kimi K3 serving
decode shapes). It holds none of the method's arithmetic: no gate, norm,
convolution or recurrence is evaluated here. Both the HIP path (through the
package facade) and the fp64 oracle consume the same tensors.

Distributions (all draws are from one ``torch.Generator`` seeded with the
given seed, on the requested device):

* q, k, v, raw gate, beta logits, packed QKV, x, output gate: bf16 ~ N(0, 1)
* A_log: fp32 ~ U(-2, 0);  dt_bias: fp32 ~ N(0, 0.1)
* recurrent state: N(0, 0.05) stored as fp32 or bf16
* conv weight: fp32 ~ N(0, 0.5);  conv cache: bf16 ~ N(0, 1)
* norm weight: fp32 ~ U(0.5, 1.5)

Every sigma is a standard deviation (``randn * sigma``).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

D = 128  # head dimension K = V = 128 on every page of the method


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(gen, shape, device, sigma=1.0, dtype=torch.bfloat16):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(dtype)


def _uniform(gen, shape, device, lo, hi):
    t = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def _randn_big(gen, shape, device, sigma, dtype):
    """N(0, sigma) fill of a possibly huge tensor, drawn in chunks to bound
    the fp32 staging memory."""
    out = torch.empty(shape, device=device, dtype=dtype)
    flat = out.view(-1)
    chunk = 1 << 27
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        t = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        t.mul_(sigma)
        flat[s:e].copy_(t)
    return out


def unique_slots(gen, n, lo, hi, device):
    """n distinct int32 slot indices drawn uniformly from [lo, hi)."""
    if n > hi - lo:
        raise ValueError("not enough slots for unique indices")
    perm = torch.randperm(hi - lo, generator=gen, device=device)[:n]
    return (perm + lo).to(torch.int32)


def gate_params(gen, H, device):
    A_log = _uniform(gen, (H,), device, -2.0, 0.0)
    dt_bias = _randn(gen, (H * D,), device, 0.1, torch.float32)
    return A_log, dt_bias


@dataclass
class RecurrentCase:
    q: torch.Tensor          # bf16 [T, H, 128]   (T = n_tokens)
    k: torch.Tensor
    v: torch.Tensor          # bf16 [T, HV, 128]
    g: torch.Tensor          # raw gate bf16 [T, HV, 128] (or precomputed log-decay)
    beta: torch.Tensor       # logits bf16 [T, HV] (or precomputed beta)
    A_log: torch.Tensor      # fp32 [HV] (None for a precomputed gate)
    dt_bias: torch.Tensor    # fp32 [HV*128] (None for a precomputed gate)
    state: torch.Tensor      # [num_slots, HV, 128, 128] fp32 or bf16
    state_indices: torch.Tensor  # int32 [n_seqs]
    cu_seqlens: torch.Tensor | None  # int32 [n_seqs+1] or None (T=1)

    @property
    def H(self):
        return self.q.shape[1]


def recurrent_case(seed, *, n_seqs, H, num_slots, state_dtype=torch.float32,
                   device="cpu", indices="identity", lengths=None,
                   null_rows=0, slot_lo=0, HV=None, gate="in_kernel",
                   gate_dtype=torch.float32):
    """Inputs of a recurrent KDA call.

    ``lengths`` None means T=1 (one token per sequence, no cu_seqlens);
    otherwise a list of per-sequence token counts (zero allowed).
    ``indices``: "identity" (slot i for sequence i, shifted by slot_lo) or
    "random" (unique slots from [slot_lo, num_slots)). ``null_rows`` rows
    chosen at random are set to -1.  ``HV`` value heads (default H; q and k
    keep H heads).  ``gate="precomputed"`` draws the log-decay g ~ U(-3, 0)
    and beta ~ U(0, 1) directly, in ``gate_dtype``.
    """
    if HV is not None and HV != H:
        return _grouped_case(seed, n_seqs=n_seqs, H=H, HV=HV, num_slots=num_slots,
                             state_dtype=state_dtype, device=device, indices=indices,
                             lengths=lengths, null_rows=null_rows, slot_lo=slot_lo, gate=gate,
                             gate_dtype=gate_dtype)
    if gate != "in_kernel":
        return _grouped_case(seed, n_seqs=n_seqs, H=H, HV=H, num_slots=num_slots,
                             state_dtype=state_dtype, device=device, indices=indices,
                             lengths=lengths, null_rows=null_rows, slot_lo=slot_lo, gate=gate,
                             gate_dtype=gate_dtype)
    gen = _gen(seed, device)
    if lengths is None:
        n_tokens = n_seqs
        cu = None
    else:
        assert len(lengths) == n_seqs
        n_tokens = int(sum(lengths))
        cu = torch.zeros(n_seqs + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        cu = cu.to(device)
    q = _randn(gen, (n_tokens, H, D), device)
    k = _randn(gen, (n_tokens, H, D), device)
    v = _randn(gen, (n_tokens, H, D), device)
    g = _randn(gen, (n_tokens, H, D), device)
    beta = _randn(gen, (n_tokens, H), device)
    A_log, dt_bias = gate_params(gen, H, device)
    state = _randn_big(gen, (num_slots, H, D, D), device, 0.05, state_dtype)
    if indices == "identity":
        idx = (torch.arange(n_seqs, device=device) + slot_lo).to(torch.int32)
    else:
        idx = unique_slots(gen, n_seqs, slot_lo, num_slots, device)
    if null_rows:
        rows = torch.randperm(n_seqs, generator=gen, device=device)[:null_rows]
        idx[rows] = -1
    return RecurrentCase(q, k, v, g, beta, A_log, dt_bias, state, idx, cu)


def _grouped_case(seed, *, n_seqs, H, HV, num_slots, state_dtype, device, indices, lengths,
                  null_rows, slot_lo, gate, gate_dtype):
    gen = _gen(seed, device)
    if lengths is None:
        n_tokens, cu = n_seqs, None
    else:
        n_tokens = int(sum(lengths))
        cu = torch.zeros(n_seqs + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        cu = cu.to(device)
    q = _randn(gen, (n_tokens, H, D), device)
    k = _randn(gen, (n_tokens, H, D), device)
    v = _randn(gen, (n_tokens, HV, D), device)
    if gate == "in_kernel":
        g = _randn(gen, (n_tokens, HV, D), device)
        beta = _randn(gen, (n_tokens, HV), device)
        A_log, dt_bias = gate_params(gen, HV, device)
    else:
        g = _uniform(gen, (n_tokens, HV, D), device, -3.0, 0.0).to(gate_dtype)
        beta = _uniform(gen, (n_tokens, HV), device, 0.0, 1.0).to(gate_dtype)
        A_log = dt_bias = None
    state = _randn_big(gen, (num_slots, HV, D, D), device, 0.05, state_dtype)
    if indices == "identity":
        idx = (torch.arange(n_seqs, device=device) + slot_lo).to(torch.int32)
    else:
        idx = unique_slots(gen, n_seqs, slot_lo, num_slots, device)
    if null_rows:
        rows = torch.randperm(n_seqs, generator=gen, device=device)[:null_rows]
        idx[rows] = -1
    return RecurrentCase(q, k, v, g, beta, A_log, dt_bias, state, idx, cu)


@dataclass
class PackedCase:
    mixed_qkv: torch.Tensor  # bf16 [B, 3*H*128] (row stride may exceed width)
    raw_gate: torch.Tensor   # bf16 [B, H*128]
    raw_beta: torch.Tensor   # bf16 [B, H]
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    state: torch.Tensor      # [num_slots, H, 128, 128]
    state_indices: torch.Tensor


def packed_case(seed, *, B, H, num_slots, state_dtype=torch.bfloat16,
                device="cpu", null_rows=0, slot_lo=1, row_pad=0):
    """Packed T=1 decode inputs: post-convolution q|k|v rows plus raw gate
    and beta logits. ``row_pad`` extra bf16 elements per QKV row give a
    padded production row stride (the tensors are views)."""
    gen = _gen(seed, device)
    W = 3 * H * D
    qkv_full = _randn(gen, (B, W + row_pad), device)
    mixed_qkv = qkv_full[:, :W]
    raw_gate = _randn(gen, (B, H * D), device)
    raw_beta = _randn(gen, (B, H), device)
    A_log, dt_bias = gate_params(gen, H, device)
    state = _randn_big(gen, (num_slots, H, D, D), device, 0.05, state_dtype)
    idx = unique_slots(gen, B, slot_lo, num_slots, device)
    if null_rows:
        rows = torch.randperm(B, generator=gen, device=device)[:null_rows]
        idx[rows] = -1
    return PackedCase(mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, state, idx)


@dataclass
class FusedCase:
    x: torch.Tensor            # bf16 [rows, 3*H*128]
    weight: torch.Tensor       # fp32 [3, 4, H*128]
    conv_state: torch.Tensor   # bf16 [num_slots, 3*H*128, 3], strides [ss, 1, 3*H*128]
    raw_gate: torch.Tensor     # bf16 [rows, H, 128]
    raw_beta: torch.Tensor     # bf16 [rows, H]
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    state_indices: torch.Tensor
    state: torch.Tensor        # [num_slots, H, 128, 128]
    output_gate: torch.Tensor  # bf16 [rows, H, 128]
    norm_weight: torch.Tensor  # fp32 [128]


def conv_cache(gen, num_slots, C, device, slot_pad=0):
    """Conv cache in the sequence-dimension layout: logical shape
    [num_slots, C, 3] with strides [slot_stride, 1, C]; the slot stride is
    3*C + slot_pad elements."""
    ss = 3 * C + slot_pad
    store = _randn_big(gen, (num_slots * ss,), device, 1.0, torch.bfloat16)
    return torch.as_strided(store, (num_slots, C, 3), (ss, 1, C))


def fused_case(seed, *, rows, H, num_slots, state_dtype=torch.float32,
               device="cpu", null_zero=0, null_neg=0, slot_pad=0):
    gen = _gen(seed, device)
    C = 3 * H * D
    x = _randn(gen, (rows, C), device)
    weight = _randn(gen, (3, 4, H * D), device, 0.5, torch.float32)
    cs = conv_cache(gen, num_slots, C, device, slot_pad)
    raw_gate = _randn(gen, (rows, H, D), device)
    raw_beta = _randn(gen, (rows, H), device)
    A_log, dt_bias = gate_params(gen, H, device)
    idx = unique_slots(gen, rows, 1, num_slots, device)
    n_null = null_zero + null_neg
    if n_null:
        r = torch.randperm(rows, generator=gen, device=device)[:n_null]
        idx[r[:null_zero]] = 0
        idx[r[null_zero:]] = -1
    state = _randn_big(gen, (num_slots, H, D, D), device, 0.05, state_dtype)
    ogate = _randn(gen, (rows, H, D), device)
    norm_weight = _uniform(gen, (D,), device, 0.5, 1.5)
    return FusedCase(x, weight, cs, raw_gate, raw_beta, A_log, dt_bias, idx,
                     state, ogate, norm_weight)


def ragged_lengths(seed, n_seqs, lo=0, hi=6):
    """Per-sequence token counts ~ U{lo..hi} (empty sequences allowed)."""
    gen = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, (n_seqs,), generator=gen).tolist()



@dataclass
class PackedFusedCase:
    x: torch.Tensor            # bf16 [rows, 3*H*128] (rows = sum(lengths) + pad_rows)
    weight: torch.Tensor       # fp32 [3, 4, H*128]
    conv_state: torch.Tensor   # bf16 [num_slots, 3*H*128, 3], strides [ss, 1, 3*H*128]
    raw_gate: torch.Tensor     # bf16 [rows, H, 128]
    raw_beta: torch.Tensor     # bf16 [rows, H]
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    state_indices: torch.Tensor        # int32 [N, max_tokens]
    query_start_loc: torch.Tensor      # int32 [N+1]
    num_accepted_tokens: torch.Tensor  # int32 [N], 1..max_tokens
    state: torch.Tensor        # [num_slots, H, 128, 128]
    output_gate: torch.Tensor  # bf16 [rows, H, 128]
    norm_weight: torch.Tensor  # fp32 [128]
    lengths: list


def packed_fused_case(seed, *, lengths, H, num_slots, max_tokens=None, state_dtype=torch.float32,
                      device="cpu", accepted="random", pad_rows=0, slot_pad=0):
    """Packed speculative rows: sequence i owns lengths[i] consecutive rows;
    every (sequence, column) gets its own slot from [1, num_slots) (so no
    two sequences share a slot); num_accepted_tokens ~ U{1..max_tokens}
    ("random") or all 1 ("one"); pad_rows trailing rows belong to no
    sequence."""
    N = len(lengths)
    T_max = int(max_tokens or max(max(lengths), 1))
    rows = int(sum(lengths)) + pad_rows
    gen = _gen(seed, device)
    C = 3 * H * D
    x = _randn(gen, (rows, C), device)
    weight = _randn(gen, (3, 4, H * D), device, 0.5, torch.float32)
    cs = conv_cache(gen, num_slots, C, device, slot_pad)
    raw_gate = _randn(gen, (rows, H, D), device)
    raw_beta = _randn(gen, (rows, H), device)
    A_log, dt_bias = gate_params(gen, H, device)
    idx = unique_slots(gen, N * T_max, 1, num_slots, device).reshape(N, T_max)
    if accepted == "random":
        acc = torch.randint(1, T_max + 1, (N,), generator=gen, device=device).to(torch.int32)
    else:
        acc = torch.ones(N, dtype=torch.int32, device=device)
    qsl = torch.zeros(N + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    state = _randn_big(gen, (num_slots, H, D, D), device, 0.05, state_dtype)
    ogate = _randn(gen, (rows, H, D), device)
    norm_weight = _uniform(gen, (D,), device, 0.5, 1.5)
    return PackedFusedCase(x, weight, cs, raw_gate, raw_beta, A_log, dt_bias, idx, qsl.to(device),
                           acc, state, ogate, norm_weight, list(lengths))
