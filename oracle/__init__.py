"""fp64 CPU oracle of the KDA decode step (ctypes wrapper of kda_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the package smoke
check and by the benchmark's cpu_baseline leg, never by the product path.
It shares no code with the HIP path; it imports neither the package nor its
C library.

Every function takes host arrays (numpy, or CPU torch tensors which are
viewed as numpy without arithmetic), copies what it updates, and returns
the results.  bf16 data travel as their uint16 bit patterns.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

F32, BF16, F64 = 0, 1, 2
D = 128
SCALE = 1.0 / math.sqrt(D)   # fixed output scale (packed decode exact contract)
L2_EPS = 1e-6                # fixed L2 epsilon (packed decode exact contract)

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 (no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load(path=None):
    global _lib
    if _lib is None:
        if path is None:
            path = _LIB
            if not os.path.exists(path):
                build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        Dbl = ctypes.c_double
        Int = ctypes.c_int
        lib.kdao_recurrent.restype = Int
        lib.kdao_recurrent.argtypes = [I64, I64, I64, P, P, P, P, P, P, P, Dbl, Dbl,
                                       P, P, I64, Int, P, P, P, Int, P, P]
        lib.kdao_recurrent2.restype = Int
        lib.kdao_recurrent2.argtypes = [I64, I64, I64, I64, P, P, P, P, Int, P, Int, Int, P, P,
                                        Dbl, Dbl, P, I64, P, I64, Int, P, Int, P, P, Int, P, P]
        lib.kdao_recurrent3.restype = Int
        lib.kdao_recurrent3.argtypes = [I64, I64, I64, I64, P, P, P, P, Int, P, Int, Int, P, P,
                                        Dbl, Dbl, P, I64, P, I64, Int, P, Int, P, P, Int, P, P,
                                        I64, P, P]
        lib.kdao_fused.restype = Int
        lib.kdao_fused.argtypes = [I64, I64, P, P, I64, P, I64, P, P, P, P, P, Int, P,
                                   P, P, Dbl, Dbl, Dbl, P, P, P, P]
        lib.kdao_packed_fused.restype = Int
        lib.kdao_packed_fused.argtypes = [I64, I64, I64, I64, P, P, I64, P, I64, P, P, P, P, P, P,
                                          P, Int, P, P, P, Dbl, Dbl, Dbl, P, P, P, P, P]
        lib.kdao_bf16_from_f64_n.restype = None
        lib.kdao_bf16_from_f64_n.argtypes = [P, P, I64]
        _lib = lib
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Temporarily route every call to another build of kda_oracle.c (used by
    the tests that plant mistakes in copies of the oracle)."""
    global _lib
    saved = _lib
    _lib = None
    try:
        _load(path)
        yield
    finally:
        _lib = saved


# ---- array helpers (no arithmetic) -------------------------------------------

def as_np(x):
    """numpy view of a CPU array / tensor; bf16 tensors become uint16 bits."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x
    import torch  # only for converting CPU tensors
    t = x.detach()
    if t.device.type != "cpu":
        raise ValueError("the oracle takes host arrays")
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def _c(a, dtype):
    a = np.ascontiguousarray(as_np(a))
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported state dtype {a.dtype}")


_NP_OF = {F32: np.float32, BF16: np.uint16, F64: np.float64}


def bf16_from_f64(x) -> np.ndarray:
    """Round doubles to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().kdao_bf16_from_f64_n(_ptr(x), _ptr(out), x.size)
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- entry points --------------------------------------------------------------

def _gate_input(a, what):
    a = np.ascontiguousarray(as_np(a))
    if a.dtype == np.uint16:
        return a, 0
    if a.dtype == np.float32:
        return a, 1
    raise TypeError(f"{what} must be bf16 (uint16 bits) or float32, got {a.dtype}")


def recurrent(q, k, v, g, beta, A_log, dt_bias, state, state_indices,
              cu_seqlens=None, *, scale=SCALE, l2_eps=L2_EPS, ckpt_dtype=None,
              want_ckpt64=False, gate="in_kernel", update_state=True, tokens_per_seq=1,
              t_max=None):
    """Recurrent KDA: T=1, uniform batches of tokens_per_seq tokens, or ragged
    (cu_seqlens given).

    q, k: bf16 [T, H, 128]; v: bf16 [T, HV, 128] (HV a multiple of H; value
    head hv reads q/k head hv // (HV // H)); g: [T, HV, 128] and beta: [T, HV],
    bf16 bits or float32.  gate="in_kernel": g is the raw gate, beta logits,
    A_log fp32 [HV] and dt_bias fp32 [HV*128] are used; gate="precomputed": g
    is the log-decay and beta is beta itself (A_log, dt_bias may be None).
    state [slots, HV, 128, 128] (fp32, bf16 bits or float64), state_indices
    int32 [N].  update_state=False leaves the pool as it was (read-only verify).
    t_max: also return the verify caches corr [slots, HV, t_max, 128] (the
    correction beta*u of each token) and kg [slots, HV, t_max, 256] (raw key |
    raw gate), in float64, zero where nothing was recorded.
    Returns dict(out64, out_bf16, state, ckpt, ckpt64, corr, kg).
    """
    q = _c(q, np.uint16); k = _c(k, np.uint16); v = _c(v, np.uint16)
    g, g_f32 = _gate_input(g, "g")
    beta, b_f32 = _gate_input(beta, "beta")
    mode = {"in_kernel": 0, "precomputed": 1}[gate]
    A_log = None if A_log is None else _c(A_log, np.float32)
    dt_bias = None if dt_bias is None else _c(dt_bias, np.float32)
    if mode == 0 and (A_log is None or dt_bias is None):
        raise ValueError("the in-kernel gate needs A_log and dt_bias")
    st = np.array(as_np(state), copy=True, order="C")
    sdt = _dtype_code(st)
    idx = _c(state_indices, np.int32)
    cu = None if cu_seqlens is None else _c(cu_seqlens, np.int32)
    T, H = q.shape[0], q.shape[1]
    HV = v.shape[1]
    N = idx.shape[0]
    assert k.shape == q.shape and v.shape == (T, HV, D) and g.shape == (T, HV, D)
    assert beta.shape == (T, HV) and st.shape[1:] == (HV, D, D)
    out64 = np.zeros((T, HV, D), np.float64)
    outb = np.zeros((T, HV, D), np.uint16)
    ckpt = None
    cdt = 0
    if ckpt_dtype is not None:
        cdt = ckpt_dtype
        ckpt = np.zeros((T, HV, D, D), _NP_OF[cdt])
    ck64 = np.zeros((T, HV, D, D), np.float64) if want_ckpt64 else None
    corr = kg = None
    tm = 0
    if t_max is not None:
        tm = int(t_max)
        corr = np.zeros((st.shape[0], HV, tm, D), np.float64)
        kg = np.zeros((st.shape[0], HV, tm, 2 * D), np.float64)
    rc = _load().kdao_recurrent3(T, N, H, HV, _ptr(q), _ptr(k), _ptr(v), _ptr(g), g_f32,
                                 _ptr(beta), b_f32, mode, _ptr(A_log), _ptr(dt_bias),
                                 float(scale), float(l2_eps), _ptr(cu), int(tokens_per_seq),
                                 _ptr(idx), st.shape[0], sdt, _ptr(st), 1 if update_state else 0,
                                 _ptr(out64), _ptr(outb), cdt, _ptr(ckpt), _ptr(ck64),
                                 tm, _ptr(corr), _ptr(kg))
    if rc != 0:
        raise ValueError(f"kdao_recurrent3 rejected its arguments ({rc})")
    return dict(out64=out64, out_bf16=outb, state=st, ckpt=ckpt, ckpt64=ck64, corr=corr, kg=kg)


def packed(mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, state, state_indices):
    """Packed T=1 decode: split the q|k|v projection row (q at [0, H*128),
    k at [H*128, 2*H*128), v at [2*H*128, 3*H*128)) and run the recurrence
    with the fixed scale and L2 epsilon; -1 rows are inactive."""
    qkv = as_np(mixed_qkv)
    B = qkv.shape[0]
    H = np.asarray(as_np(A_log)).shape[0]
    HC = H * D
    q = qkv[:, 0:HC].reshape(B, H, D)
    k = qkv[:, HC:2 * HC].reshape(B, H, D)
    v = qkv[:, 2 * HC:3 * HC].reshape(B, H, D)
    g = as_np(raw_gate).reshape(B, H, D)
    beta = as_np(raw_beta).reshape(B, H)
    return recurrent(q, k, v, g, beta, A_log, dt_bias, state, state_indices)


def fused(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias, state_indices,
          state, output_gate, norm_weight, *, norm_eps=1e-5, scale=SCALE,
          l2_eps=L2_EPS):
    """Fused decode: conv + SiLU, one KDA token, gated RMSNorm.

    conv_state is the logical [slots, 3*H*128, 3] cache; it is handed to C as
    a contiguous [slots, 3, 3*H*128] copy (position-major, the pages' layout).
    Returns dict(out64, out_bf16, o_pre64, act64, state, conv_state) where
    conv_state is again logical [slots, 3*H*128, 3].
    """
    xa = _c(x, np.uint16)
    rows, C3 = xa.shape
    H = C3 // (3 * D)
    cs_log = as_np(conv_state)                       # [slots, C3, 3]
    cs = np.ascontiguousarray(np.transpose(cs_log, (0, 2, 1)))  # [slots, 3, C3]
    st = np.array(as_np(state), copy=True, order="C")
    sdt = _dtype_code(st)
    w = _c(weight, np.float32)
    gr = _c(as_np(raw_gate).reshape(rows, H, D), np.uint16)
    br = _c(as_np(raw_beta).reshape(rows, H), np.uint16)
    og = _c(as_np(output_gate).reshape(rows, H, D), np.uint16)
    nw = _c(norm_weight, np.float32)
    idx = _c(state_indices, np.int32)
    A_log = _c(A_log, np.float32); dt_bias = _c(dt_bias, np.float32)
    out64 = np.zeros((rows, H, D), np.float64)
    outb = np.zeros((rows, H, D), np.uint16)
    opre = np.zeros((rows, H, D), np.float64)
    act = np.zeros((rows, C3), np.float64)
    rc = _load().kdao_fused(rows, H, _ptr(xa), _ptr(w), cs.shape[0], _ptr(cs), 3 * C3,
                            _ptr(gr), _ptr(br), _ptr(A_log), _ptr(dt_bias), _ptr(idx),
                            sdt, _ptr(st), _ptr(og), _ptr(nw), float(norm_eps),
                            float(scale), float(l2_eps), _ptr(out64), _ptr(outb),
                            _ptr(opre), _ptr(act))
    if rc != 0:
        raise ValueError(f"kdao_fused rejected its arguments ({rc})")
    return dict(out64=out64, out_bf16=outb, o_pre64=opre, act64=act, state=st,
                conv_state=np.transpose(cs, (0, 2, 1)))


def packed_fused(x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias, state_indices,
                 state, output_gate, norm_weight, *, query_start_loc, num_accepted_tokens,
                 norm_eps=1e-5, scale=SCALE, l2_eps=L2_EPS, want_ckpt64=False):
    """Packed fused decode with T >= 1 tokens per sequence.

    x [rows, 3*H*128]; raw_gate [rows, H, 128]; raw_beta [rows, H];
    output_gate [rows, H, 128]; state_indices int32 [N, max_tokens] (column j:
    the slot for the checkpoint after token j; the sequence starts from column
    num_accepted_tokens[i] - 1); query_start_loc int32 [N+1]; conv_state the
    logical [slots, 3*H*128, 3] cache.  Returns dict(out64, out_bf16,
    o_pre64, act64, state, conv_state, ckpt64).
    """
    xa = _c(x, np.uint16)
    rows, C3 = xa.shape
    H = C3 // (3 * D)
    cs_log = as_np(conv_state)
    cs = np.ascontiguousarray(np.transpose(cs_log, (0, 2, 1)))  # [slots, 3, C3]
    st = np.array(as_np(state), copy=True, order="C")
    sdt = _dtype_code(st)
    w = _c(weight, np.float32)
    gr = _c(as_np(raw_gate).reshape(rows, H, D), np.uint16)
    br = _c(as_np(raw_beta).reshape(rows, H), np.uint16)
    og = _c(as_np(output_gate).reshape(rows, H, D), np.uint16)
    nw = _c(norm_weight, np.float32)
    si = _c(state_indices, np.int32)
    if si.ndim == 1:
        si = si.reshape(-1, 1)
    N, max_tokens = si.shape
    qsl = _c(query_start_loc, np.int32)
    acc = _c(num_accepted_tokens, np.int32)
    assert qsl.shape == (N + 1,) and acc.shape == (N,)
    A_log = _c(A_log, np.float32); dt_bias = _c(dt_bias, np.float32)
    out64 = np.zeros((rows, H, D), np.float64)
    outb = np.zeros((rows, H, D), np.uint16)
    opre = np.zeros((rows, H, D), np.float64)
    act = np.zeros((rows, C3), np.float64)
    ck64 = np.zeros((rows, H, D, D), np.float64) if want_ckpt64 else None
    rc = _load().kdao_packed_fused(rows, N, H, max_tokens, _ptr(xa), _ptr(w), cs.shape[0], _ptr(cs),
                                   3 * C3, _ptr(gr), _ptr(br), _ptr(A_log), _ptr(dt_bias), _ptr(si),
                                   _ptr(qsl), _ptr(acc), sdt, _ptr(st), _ptr(og), _ptr(nw),
                                   float(norm_eps), float(scale), float(l2_eps), _ptr(out64),
                                   _ptr(outb), _ptr(opre), _ptr(act), _ptr(ck64))
    if rc != 0:
        raise ValueError(f"kdao_packed_fused rejected its arguments ({rc})")
    return dict(out64=out64, out_bf16=outb, o_pre64=opre, act64=act, state=st,
                conv_state=np.transpose(cs, (0, 2, 1)), ckpt64=ck64)
