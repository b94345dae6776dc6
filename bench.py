#!/usr/bin/env python3
"""Benchmark of the KDA decode hot path on one MI355X.

Default workload (the headline line): recurrent_kda T=1, H=HV=32, K=V=128,
fp32 state pool [4096, 32, 128, 128] (8 GiB) ~N(0, 0.05), B=256 rows on
random unique slots, bf16 inputs ~N(0,1), A_log ~U(-2,0), dt_bias
~N(0,0.1), softplus gate, scale 1/sqrt(128).  One step = one kernel launch
that gathers, updates and scatters the 256 x 32 head states.

Printed: one JSON line with rows/s (value), the live roofline of the
kernel (HIP events on the launch stream over the timed region), the fp64
oracle timed on the host cores over a bounded sample (cpu_baseline), and
the other workloads of the path (batch sweeps, packed H=12 bf16, fused,
ragged) with their own timings.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode rows/sec and achieved state HBM GB/s (% of peak), H=12/32, B=1..512"
HBM_PEAK_GBPS = 8000.0
D = 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_recurrent_t1_h32_fp32_b256.json")
# the sources that decide what the measured kernel does: its code and its launch policy
KERNEL_SRCS = [os.path.join(ROOT, "gated_delta_rule_decode_amd", "csrc", n) for n in ("kda_kernels.hip", "kda_api.cpp")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ byte model ----
# Algorithmic HBM bytes (each byte the method must move once):
#   per live (row, head), T=1: state read + write 2*128*128*s, q,k,v 3*256 B,
#   raw gate 256 B, beta 2 B, output 256 B; per row the 4-byte index; per call
#   A_log and dt_bias.  Null rows move their index and output only.

def t1_bytes(B_live, B_null, H, state_bytes):
    per_head = 2 * D * D * state_bytes + 3 * 2 * D + 2 * D + 2 + 2 * D
    return (B_live * (H * per_head + 4) + B_null * (4 + H * 2 * D) + H * 4 + H * D * 4)


def t1_state_bytes(B_live, H, state_bytes):
    return B_live * H * 2 * D * D * state_bytes


def fused_bytes(R_live, R_null, H, state_bytes):
    C3 = 3 * H * D
    per_row = (H * 2 * D * D * state_bytes      # state read + write
               + C3 * 2                           # x
               + 2 * 3 * C3 * 2                   # conv cache read 3 positions + write 3
               + H * D * 2 + H * 2                # raw gate, beta
               + H * D * 2 + H * D * 2 + 4)       # output gate, output, index
    return R_live * per_row + R_null * (4 + H * D * 2) + 12 * H * D * 4 + H * 4 + H * D * 4 + D * 4


def modes_bytes(n_live_seqs, tokens, H, HV, state_bytes, *, write_state=True, gate_bytes=2,
                beta_bytes=2, gate_params=True):
    """Recurrent call with HV value heads over H q/k heads: per live (sequence,
    value head) the state is read (and written unless read-only); per token
    q, k per q/k head and v, g, beta, output per value head."""
    head = D * D * state_bytes
    b = n_live_seqs * HV * head * (2 if write_state else 1)
    b += tokens * (H * 2 * D * 2 + HV * (D * 2 + D * gate_bytes + beta_bytes + D * 2))
    b += n_live_seqs * 4 + (HV * 4 + HV * D * 4 if gate_params else 0)
    return b


def packed_fused_bytes(N, T, H, state_bytes):
    """Packed fused call, N live sequences of T tokens: per (sequence, head)
    the state and the conv window are read once and written once per token
    (checkpoints); per token and head x, raw gate, beta, output gate and
    output; per sequence its metadata; per call the weights."""
    head = D * D * state_bytes
    win = 3 * 3 * D * 2
    per_item = head + T * head + win + T * win + T * (3 * D * 2 + D * 2 + 2 + D * 2 + D * 2)
    return N * H * per_item + N * (8 + 4 * T) + 4 + 12 * H * D * 4 + H * D * 4 + H * 4 + D * 4


def varlen_bytes(lengths, H, state_bytes, ckpt=True):
    live_seqs = sum(1 for n in lengths if n > 0)
    T = sum(lengths)
    head = D * D * state_bytes
    b = live_seqs * H * 2 * head + T * H * (4 * 2 * D + 2 + 2 * D)
    if ckpt:
        b += T * H * head
    return b + (len(lengths) + 1) * 4 + len(lengths) * 4 + H * 4 + H * D * 4


# ---------------------------------------------------------- CPU baseline ----

_SAMPLE = None  # (inputs per worker) set in the parent before the pool forks


def _oracle_slice(w):
    import oracle
    q, k, v, g, beta, A_log, dt_bias, st, idx = _SAMPLE[w]
    oracle.recurrent(q, k, v, g, beta, A_log, dt_bias, st, idx)
    return q.shape[0]


def cpu_baseline(budget_s=12.0, rows_per_worker=8, H=32):
    """The fp64 oracle as it stands, on the host cores, over a bounded sample
    of the headline workload (T=1, H=32, fp32 state): each worker process
    decodes its own 8 rows on their own slots, repeatedly, until the budget
    is spent.  Inputs are drawn once in the parent (seeded) before the pool
    forks; nothing here touches the GPU."""
    global _SAMPLE
    import multiprocessing as mp

    import oracle
    from gated_delta_rule_decode_amd import synth
    workers = max(1, min(16, os.cpu_count() or 1))
    sample = []
    for w in range(workers):
        c = synth.recurrent_case(9000 + w, n_seqs=rows_per_worker, H=H, num_slots=rows_per_worker)
        sample.append(tuple(oracle.as_np(t) for t in (c.q, c.k, c.v, c.g, c.beta, c.A_log,
                                                      c.dt_bias, c.state, c.state_indices)))
    _SAMPLE = sample
    # one thread first (this process), then every worker
    t0, one = time.perf_counter(), 0
    while time.perf_counter() - t0 < 2.0:
        one += _oracle_slice(0)
    one_rate = one / (time.perf_counter() - t0)
    ctx = mp.get_context("fork")
    done_rows = 0
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_slice, range(workers))  # warm the workers up
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            done_rows += sum(pool.map(_oracle_slice, range(workers)))
        wall = time.perf_counter() - t0
    _SAMPLE = None
    return {"value": done_rows / wall, "unit": "rows/s", "cores": workers, "kind": "oracle",
            "sample": f"{done_rows} rows of T=1 H=32 fp32-state decode ({done_rows * H} head "
                      f"updates) in {wall:.1f} s: {workers} worker processes, each repeating "
                      f"its own {rows_per_worker} rows; gcc -O2 fp64 oracle",
            "single_thread_rows_per_s": one_rate}


# ---------------------------------------------------------- GPU helpers ----

def sha256_of(paths):
    """sha256 over the concatenated bytes of the files."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(bytes_per_launch):
    """HBM traffic measured with rocprofv3 counters, if it was taken on the
    current kernel source and launch policy."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_sha256") != sha256_of(KERNEL_SRCS):
            return None
        return float(t["hbm_bytes_per_launch"])
    except Exception:
        return None


def launch_plan(c, idx, pool, out_t, B, H):
    """Launch geometry the library picks for the headline call (host-only query)."""
    import ctypes

    from gated_delta_rule_decode_amd import _lib
    a = _lib.RecurrentArgs()
    a.struct_size = ctypes.sizeof(_lib.RecurrentArgs)
    a.n_seqs, a.n_tokens, a.H, a.HV, a.K, a.V = B, B, H, H, D, D
    a.q, a.k, a.v, a.g, a.beta = (c.q.data_ptr(), c.k.data_ptr(), c.v.data_ptr(), c.g.data_ptr(),
                                  c.beta.data_ptr())
    a.q_stride = a.k_stride = a.v_stride = a.g_stride = H * D
    a.beta_stride = H
    a.A_log, a.dt_bias = c.A_log.data_ptr(), c.dt_bias.data_ptr()
    a.scale, a.l2_eps = 1.0 / math.sqrt(D), 1e-6
    a.state, a.state_dtype, a.ckpt_dtype = pool.data_ptr(), 0, 0
    a.num_slots, a.slot_stride = pool.shape[0], pool.stride(0)
    a.state_indices = idx.data_ptr()
    a.out = out_t.data_ptr()
    a.g_dtype = a.beta_dtype = _lib.DTYPE_BF16
    a.tokens_per_seq = 1
    p = _lib.LaunchPlan()
    rc = _lib.load().kda_recurrent_plan(ctypes.byref(a), ctypes.byref(p))
    if rc != 0:
        return {"rows_per_block": None, "grid_x": None}
    return {"rows_per_block": p.rows_per_block, "grid_x": p.grid_x}


class Timer:
    """HIP events on the launch stream around a region."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream

    def run(self, fn, n):
        torch = self.torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record(self.stream)
        for _ in range(n):
            fn()
        e.record(self.stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n * 1e3  # us per call


# --------------------------------------------------------- other workloads ----

def n_sets(state_bytes_per_call, available, lo=4, cycle=1 << 30):
    """Disjoint slot sets to rotate over so that one cycle touches at least
    `cycle` bytes of state (L2 is 8 x 4 MiB, the MALL 256 MiB): every call
    then finds its state cold, as with a flush before each launch."""
    need = -(-cycle // max(1, state_bytes_per_call))
    return int(max(min(lo, available), min(need, available)))


def rotating(torch, timer, calls, reps=8):
    """Average GPU time per call of `calls` (each touching its own slots, so
    consecutive calls find their state cold in L2 and the MALL), captured once
    into a HIP graph and replayed back to back: host launch overhead does not
    enter the measurement."""
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for f in calls:
            f()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):  # the warm-up stream: its default workspaces are sized
        for f in calls:
            f()
    graph.replay()
    torch.cuda.synchronize()
    return timer.run(graph.replay, reps) / len(calls)


def extra_workloads(torch, dev, timer, pool32, only=None, packed_b=None, packed_fused_n=None):
    from gated_delta_rule_decode_amd import (fused_kda_decode, packed_fused_kda_decode, packed_kda_decode,
                                             recurrent_kda, synth)
    out = {}
    want = lambda name: only is None or only in name  # noqa: E731
    g2 = torch.Generator(device=dev)
    g2.manual_seed(7)
    # slot order of the T=1 mode and verify workloads on the headline pool
    mperm = torch.randperm(pool32.shape[0], generator=g2, device=dev).to(torch.int32)
    H = 32
    SLOTS = pool32.shape[0]
    if want("recurrent_t1_h32_fp32"):
        # H=32 fp32 batch sweep on the 8 GiB pool: disjoint slot sets per B, a
        # cycle of >= 1 GiB of state
        sweep = []
        g2 = torch.Generator(device=dev)
        for Bs in (1, 8, 32, 128, 256, 512):
            cs = synth.recurrent_case(1000 + Bs, n_seqs=Bs, H=H, num_slots=1, device=dev)
            g2.manual_seed(1000 + Bs)
            perm = torch.randperm(SLOTS, generator=g2, device=dev).to(torch.int32)
            o = torch.empty((Bs, 1, H, D), dtype=torch.bfloat16, device=dev)
            r4 = lambda t, n=Bs: t.reshape(n, 1, H, D)  # noqa: E731
            calls = []
            for j in range(n_sets(Bs * H * D * D * 4, SLOTS // Bs)):
                ids = perm[j * Bs:(j + 1) * Bs].contiguous()
                calls.append(lambda cs=cs, ids=ids, o=o, r4=r4, n=Bs: recurrent_kda(
                    r4(cs.q), r4(cs.k), r4(cs.v), r4(cs.g), cs.beta.reshape(n, 1, H), cs.A_log,
                    cs.dt_bias, initial_state=pool32, state_indices=ids, output=o))
            t_us = rotating(torch, timer, calls)
            bts = t1_bytes(Bs, 0, H, 4)
            sweep.append({"B": Bs, "us": t_us, "rows_per_s": Bs / (t_us * 1e-6),
                          "state_GBps": t1_state_bytes(Bs, H, 4) / (t_us * 1e-6) / 1e9,
                          "GBps": bts / (t_us * 1e-6) / 1e9,
                          "frac": bts / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS})
            log(f"H=32 fp32 B={Bs}: {t_us:.1f} us, {sweep[-1]['GBps']:.0f} GB/s")
        out["recurrent_t1_h32_fp32"] = sweep

    if want("packed_t1_h12_bf16"):
        # packed H=12, bf16 pool [8192,12,128,128] (3 GiB), 1/8 of the rows inactive,
        # disjoint slot sets per B, a cycle of >= 1 GiB of state
        pcase = synth.packed_case(2000, B=512, H=12, num_slots=8192, device=dev)
        pperm = torch.randperm(8192 - 1, generator=g2, device=dev).to(torch.int32) + 1
        sweep = []
        for Bs in packed_b or (1, 8, 16, 31, 32, 64, 128, 256, 512):
            nnull = Bs // 8
            o = torch.empty((Bs, 1, 12, D), dtype=torch.bfloat16, device=dev)
            calls = []
            for j in range(n_sets((Bs - nnull) * 12 * D * D * 2, 8191 // Bs, lo=8)):
                ids = pperm[j * Bs:(j + 1) * Bs].clone()
                ids[:nnull] = -1
                calls.append(lambda ids=ids, o=o, n=Bs: packed_kda_decode(
                    pcase.mixed_qkv[:n], pcase.raw_gate[:n], pcase.raw_beta[:n], pcase.A_log,
                    pcase.dt_bias, pcase.state, ids, output=o))
            t_us = rotating(torch, timer, calls)
            live = Bs - nnull
            bts = t1_bytes(live, nnull, 12, 2)
            sweep.append({"B": Bs, "live": live, "us": t_us, "rows_per_s": live / (t_us * 1e-6),
                          "state_GBps": t1_state_bytes(live, 12, 2) / (t_us * 1e-6) / 1e9,
                          "GBps": bts / (t_us * 1e-6) / 1e9,
                          "frac": bts / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS})
            log(f"packed H=12 bf16 B={Bs} ({live} live): {t_us:.1f} us, {sweep[-1]['GBps']:.0f} GB/s")
        out["packed_t1_h12_bf16"] = sweep
        del pcase
        torch.cuda.empty_cache()

    if want("fused_h32_rows256_fp32"):
        # fused, rows=256, H=32, fp32 pool [2048,32,128,128], 16 null rows; two
        # disjoint slot sets
        fc = synth.fused_case(3000, rows=256, H=32, num_slots=2048, device=dev, null_zero=8, null_neg=8)
        idx2 = fc.state_indices.clone()
        live_mask = idx2 > 0
        free = torch.ones(2048, dtype=torch.bool, device=dev)
        free[0] = False
        free[idx2[live_mask].long()] = False
        spare = torch.nonzero(free).flatten()[:int(live_mask.sum())].to(torch.int32)
        idx2[live_mask] = spare
        o = torch.empty((1, 256, 32, D), dtype=torch.bfloat16, device=dev)
        calls = [lambda ids=ids: fused_kda_decode(fc.x, fc.weight, fc.conv_state, fc.raw_gate, fc.raw_beta,
                                                  fc.A_log, fc.dt_bias, ids, fc.state, fc.output_gate,
                                                  fc.norm_weight, output=o)
                 for ids in (fc.state_indices, idx2)]
        t_us = rotating(torch, timer, calls)
        bts = fused_bytes(240, 16, 32, 4)
        out["fused_h32_rows256_fp32"] = {"us": t_us, "rows_per_s": 240 / (t_us * 1e-6),
                                         "GBps": bts / (t_us * 1e-6) / 1e9,
                                         "frac": bts / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        log(f"fused H=32 rows=256: {t_us:.1f} us, {bts / (t_us * 1e-6) / 1e9:.0f} GB/s")
        del fc
        torch.cuda.empty_cache()

    if want("varlen_h16_n64_fp32_ckpt"):
        # ragged T>=2: H=16, N=64, lengths U{0..6}, fp32 checkpoints; the pool has
        # 16 disjoint slot sets (1 GiB of state per cycle)
        lengths = synth.ragged_lengths(4000, 64, 0, 6)
        vc = synth.recurrent_case(4000, n_seqs=64, H=16, num_slots=16 * 64 + 1, device=dev,
                                  lengths=lengths, slot_lo=1)
        T = sum(lengths)
        ck = torch.empty((T, 16, D, D), dtype=torch.float32, device=dev)
        o = torch.empty((1, T, 16, D), dtype=torch.bfloat16, device=dev)
        r1 = lambda t: t.reshape(1, T, *t.shape[1:])  # noqa: E731
        calls = [lambda ids=(vc.state_indices + 64 * j).contiguous(): recurrent_kda(
            r1(vc.q), r1(vc.k), r1(vc.v), r1(vc.g), r1(vc.beta), vc.A_log, vc.dt_bias,
            initial_state=vc.state, state_indices=ids, cu_seqlens=vc.cu_seqlens, output=o,
            intermediate_states=ck) for j in range(16)]
        t_us = rotating(torch, timer, calls)
        bts = varlen_bytes(lengths, 16, 4)
        out["varlen_h16_n64_fp32_ckpt"] = {"us": t_us, "tokens": T, "tokens_per_s": T / (t_us * 1e-6),
                                           "GBps": bts / (t_us * 1e-6) / 1e9,
                                           "frac": bts / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        log(f"varlen H=16 N=64 T={T}: {t_us:.1f} us, {bts / (t_us * 1e-6) / 1e9:.0f} GB/s")
        del vc, ck
        torch.cuda.empty_cache()

    def modes_entry(name, calls, bts, rows):
        t = rotating(torch, timer, calls)
        out[name] = {"us": t, "rows_per_s": rows / (t * 1e-6), "GBps": bts / (t * 1e-6) / 1e9,
                     "frac": bts / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        log(f"{name}: {t:.1f} us, {out[name]['GBps']:.0f} GB/s")

    B = 256
    o1 = torch.empty((B, 1, 32, D), dtype=torch.bfloat16, device=dev)
    r = lambda t: t.reshape(B, 1, *t.shape[1:])  # noqa: E731
    if want("grouped_t1_h16_hv32_fp32_b256"):
        # grouped value heads: H=16 q/k heads, HV=32 value heads, fp32 pool, T=1, B=256
        gc = synth.recurrent_case(7000, n_seqs=B, H=16, HV=32, num_slots=1, device=dev)
        calls = [lambda ids=mperm[j * B:(j + 1) * B].contiguous(): recurrent_kda(
            r(gc.q), r(gc.k), r(gc.v), r(gc.g), r(gc.beta), gc.A_log, gc.dt_bias, initial_state=pool32,
            state_indices=ids, output=o1) for j in range(4)]
        modes_entry("grouped_t1_h16_hv32_fp32_b256", calls, modes_bytes(B, B, 16, 32, 4), B)

    if want("precomputed_t1_h32_fp32_b256"):
        # precomputed gate (fp32 log-decay and beta), H=32, fp32 pool, T=1, B=256
        pc = synth.recurrent_case(7100, n_seqs=B, H=32, num_slots=1, device=dev, gate="precomputed")
        calls = [lambda ids=mperm[j * B:(j + 1) * B].contiguous(): recurrent_kda(
            r(pc.q), r(pc.k), r(pc.v), r(pc.g), r(pc.beta), initial_state=pool32, state_indices=ids,
            output=o1) for j in range(4)]
        modes_entry("precomputed_t1_h32_fp32_b256", calls,
                    modes_bytes(B, B, 32, 32, 4, gate_bytes=4, beta_bytes=4, gate_params=False), B)

    Bv, Tv = 64, 4
    vv = synth.recurrent_case(7200, n_seqs=Bv, H=32, num_slots=1, device=dev, lengths=[Tv] * Bv)
    ov = torch.empty((Bv, Tv, 32, D), dtype=torch.bfloat16, device=dev)
    rb = lambda t: t.reshape(Bv, Tv, *t.shape[1:])  # noqa: E731
    if want("verify_readonly_b64_t4_h32_fp32"):
        # speculative verify: read-only pool, batched [64, 4, 32, 128], H=32 fp32
        calls = [lambda ids=mperm[j * Bv:(j + 1) * Bv].contiguous(): recurrent_kda(
            rb(vv.q), rb(vv.k), rb(vv.v), rb(vv.g), rb(vv.beta), vv.A_log, vv.dt_bias,
            initial_state=pool32, state_indices=ids, output=ov, disable_state_update=True)
            for j in range(8)]
        modes_entry("verify_readonly_b64_t4_h32_fp32", calls,
                    modes_bytes(Bv, Bv * Tv, 32, 32, 4, write_state=False), Bv)

    if want("verify_caches_b64_t4_h32_fp32"):
        # the same verify call recording the per-token corrections (fp32) and raw
        # key | gate (fp32) into slot-indexed caches
        corr = torch.empty((SLOTS, 32, Tv, D), dtype=torch.float32, device=dev)
        kgc = torch.empty((SLOTS, 32, Tv, 2 * D), dtype=torch.float32, device=dev)
        calls = [lambda ids=mperm[j * Bv:(j + 1) * Bv].contiguous(): recurrent_kda(
            rb(vv.q), rb(vv.k), rb(vv.v), rb(vv.g), rb(vv.beta), vv.A_log, vv.dt_bias,
            initial_state=pool32, state_indices=ids, output=ov, disable_state_update=True,
            correction_cache=corr, kg_cache=kgc) for j in range(8)]
        modes_entry("verify_caches_b64_t4_h32_fp32", calls,
                    modes_bytes(Bv, Bv * Tv, 32, 32, 4, write_state=False) + Bv * Tv * 32 * 3 * D * 4, Bv)
        del corr, kgc
        torch.cuda.empty_cache()

    if want("verify_tsweep_b64_h32_fp32"):
        # read-only batched calls B=64 H=32 fp32 over the token count (the WY
        # verify kernel takes 2..16 tokens): the state read is the same for every T
        sweep = []
        for Tv2 in (2, 6, 8, 12, 16):
            vt = synth.recurrent_case(7200 + Tv2, n_seqs=Bv, H=32, num_slots=1, device=dev, lengths=[Tv2] * Bv)
            ot = torch.empty((Bv, Tv2, 32, D), dtype=torch.bfloat16, device=dev)
            rt = lambda t, n=Tv2: t.reshape(Bv, n, *t.shape[1:])  # noqa: E731
            calls = [lambda ids=mperm[j * Bv:(j + 1) * Bv].contiguous(), vt=vt, ot=ot, rt=rt: recurrent_kda(
                rt(vt.q), rt(vt.k), rt(vt.v), rt(vt.g), rt(vt.beta), vt.A_log, vt.dt_bias,
                initial_state=pool32, state_indices=ids, output=ot, disable_state_update=True)
                for j in range(8)]
            t_us = rotating(torch, timer, calls)
            bts = modes_bytes(Bv, Bv * Tv2, 32, 32, 4, write_state=False)
            sweep.append({"B": Bv, "T": Tv2, "us": t_us, "GBps": bts / (t_us * 1e-6) / 1e9,
                          "frac": bts / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS})
            log(f"verify read-only B={Bv} T={Tv2} H=32 fp32: {t_us:.1f} us, {sweep[-1]['GBps']:.0f} GB/s")
        out["verify_tsweep_b64_h32_fp32"] = sweep

    if want("verify_tsweep_b64_h32_bf16"):
        # the same read-only batched calls on a bf16 pool [4096,32,128,128]
        gb = torch.Generator(device=dev)
        gb.manual_seed(7201)
        pool16 = synth._randn_big(gb, (SLOTS, 32, D, D), dev, 0.05, torch.bfloat16)
        sweep = []
        for Tv2 in (2, 4, 8, 16):
            vt = synth.recurrent_case(7200 + Tv2, n_seqs=Bv, H=32, num_slots=1, device=dev, lengths=[Tv2] * Bv)
            ot = torch.empty((Bv, Tv2, 32, D), dtype=torch.bfloat16, device=dev)
            rt = lambda t, n=Tv2: t.reshape(Bv, n, *t.shape[1:])  # noqa: E731
            calls = [lambda ids=mperm[j * Bv:(j + 1) * Bv].contiguous(), vt=vt, ot=ot, rt=rt: recurrent_kda(
                rt(vt.q), rt(vt.k), rt(vt.v), rt(vt.g), rt(vt.beta), vt.A_log, vt.dt_bias,
                initial_state=pool16, state_indices=ids, output=ot, disable_state_update=True)
                for j in range(16)]
            t_us = rotating(torch, timer, calls)
            bts = modes_bytes(Bv, Bv * Tv2, 32, 32, 2, write_state=False)
            sweep.append({"B": Bv, "T": Tv2, "us": t_us, "GBps": bts / (t_us * 1e-6) / 1e9,
                          "frac": bts / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS})
            log(f"verify read-only B={Bv} T={Tv2} H=32 bf16: {t_us:.1f} us, {sweep[-1]['GBps']:.0f} GB/s")
        out["verify_tsweep_b64_h32_bf16"] = sweep
        del pool16
        torch.cuda.empty_cache()

    if want("verify_ragged_b64_h32_fp32"):
        # read-only ragged calls (cu_seqlens), B=64 H=32 fp32, lengths U{1..8},
        # the longest declared (8): the WY verify kernel
        lengths = synth.ragged_lengths(7300, Bv, 1, 8)
        rc_ = synth.recurrent_case(7300, n_seqs=Bv, H=32, num_slots=1, device=dev, lengths=lengths)
        Tr = sum(lengths)
        orr = torch.empty((1, Tr, 32, D), dtype=torch.bfloat16, device=dev)
        r1 = lambda t: t.reshape(1, Tr, *t.shape[1:])  # noqa: E731
        calls = [lambda ids=mperm[j * Bv:(j + 1) * Bv].contiguous(): recurrent_kda(
            r1(rc_.q), r1(rc_.k), r1(rc_.v), r1(rc_.g), r1(rc_.beta), rc_.A_log, rc_.dt_bias,
            initial_state=pool32, state_indices=ids, cu_seqlens=rc_.cu_seqlens, output=orr,
            disable_state_update=True, max_seqlen=max(lengths)) for j in range(8)]
        modes_entry("verify_ragged_b64_h32_fp32", calls, modes_bytes(Bv, Tr, 32, 32, 4, write_state=False), Bv)

    if want("eager_host"):
        # host cost per call: eager facade calls and prepared calls launched
        # back to back (wall clock per call: the larger of the host's and the
        # GPU's time per call) next to graph replays of the same calls
        import time
        from gated_delta_rule_decode_amd import prepare

        def wall(fns, m=3000):
            for f in fns:
                f()
            torch.cuda.synchronize()
            t = time.perf_counter()
            for i in range(m):
                fns[i % len(fns)]()
            torch.cuda.synchronize()
            return (time.perf_counter() - t) / m * 1e6

        rows = []
        pk = synth.packed_case(2100, B=256, H=12, num_slots=4096, device=dev)
        rk = synth.recurrent_case(1100, n_seqs=256, H=H, num_slots=1, device=dev)
        g3 = torch.Generator(device=dev)
        g3.manual_seed(11)
        pperm2 = torch.randperm(4095, generator=g3, device=dev).to(torch.int32) + 1
        for Bs in (1, 8, 256):
            o = torch.empty((Bs, 1, 12, D), dtype=torch.bfloat16, device=dev)
            pargs = [(pk.mixed_qkv[:Bs], pk.raw_gate[:Bs], pk.raw_beta[:Bs], pk.A_log, pk.dt_bias, pk.state,
                      pperm2[j * Bs:(j + 1) * Bs].contiguous())
                     for j in range(n_sets(Bs * 12 * D * D * 2, 4095 // Bs, lo=8))]
            eager = [lambda a=a: packed_kda_decode(*a, output=o) for a in pargs]
            prep = [prepare(packed_kda_decode, *a, output=o) for a in pargs]
            row = {"call": "packed_kda_decode H=12 bf16", "B": Bs, "graph_us": rotating(torch, timer, eager),
                   "eager_us": wall(eager), "prepared_us": wall(prep)}
            rows.append(row)
            log(f"eager/prepared/graph packed H=12 B={Bs}: {row['eager_us']:.1f} / {row['prepared_us']:.1f} / "
                f"{row['graph_us']:.1f} us per call")
            o2 = torch.empty((Bs, 1, H, D), dtype=torch.bfloat16, device=dev)
            r4 = lambda t, n=Bs: t[:n].reshape(n, 1, *t.shape[1:])  # noqa: E731
            rargs = [((r4(rk.q), r4(rk.k), r4(rk.v), r4(rk.g), r4(rk.beta), rk.A_log, rk.dt_bias),
                      mperm[j * Bs:(j + 1) * Bs].contiguous())
                     for j in range(n_sets(Bs * H * D * D * 4, SLOTS // Bs, lo=8))]
            eager = [lambda a=a, ids=ids: recurrent_kda(*a, initial_state=pool32, state_indices=ids, output=o2)
                     for a, ids in rargs]
            prep = [prepare(recurrent_kda, *a, initial_state=pool32, state_indices=ids, output=o2) for a, ids in rargs]
            row = {"call": "recurrent_kda T=1 H=32 fp32", "B": Bs, "graph_us": rotating(torch, timer, eager),
                   "eager_us": wall(eager), "prepared_us": wall(prep)}
            rows.append(row)
            log(f"eager/prepared/graph recurrent H=32 B={Bs}: {row['eager_us']:.1f} / {row['prepared_us']:.1f} / "
                f"{row['graph_us']:.1f} us per call")
        out["eager_host"] = rows
        del pk, rk
        torch.cuda.empty_cache()

    if want("packed_fused_t5_accept1"):
        # packed fused speculative decode, T=5 tokens per sequence, one accepted
        # token; disjoint checkpoint-slot sets per call
        pf = []
        for Hs, Ns_list in ((12, (1, 8, 32, 128)), (24, (8, 128))):
            Ns_list = tuple(n for n in Ns_list if packed_fused_n is None or n in packed_fused_n)
            if not Ns_list:
                continue
            for sdt, sb in ((torch.float32, 4), (torch.bfloat16, 2)):
                T = 5
                pool_slots = 4 * 128 * T + 1
                pc = synth.packed_fused_case(8500 + Hs, lengths=[T] * 128, H=Hs, num_slots=pool_slots,
                                             max_tokens=T, state_dtype=sdt, device=dev, accepted="one")
                g2.manual_seed(8500 + Hs)
                pperm = torch.randperm(pool_slots - 1, generator=g2, device=dev).to(torch.int32) + 1
                for Ns in Ns_list:
                    rows = Ns * T
                    o = torch.empty((1, rows, Hs, D), dtype=torch.bfloat16, device=dev)
                    qsl = (torch.arange(Ns + 1, dtype=torch.int32, device=dev) * T).contiguous()
                    acc = torch.ones(Ns, dtype=torch.int32, device=dev)
                    nset = n_sets(Ns * Hs * (1 + T) * D * D * sb, (pool_slots - 1) // (Ns * T))
                    calls = [lambda ids=pperm[k * Ns * T:(k + 1) * Ns * T].reshape(Ns, T).contiguous(), o=o, rows=rows,
                             qsl=qsl, acc=acc: packed_fused_kda_decode(
                                 pc.x[:rows], pc.weight, pc.conv_state, pc.raw_gate[:rows], pc.raw_beta[:rows], pc.A_log,
                                 pc.dt_bias, ids, pc.state, pc.output_gate[:rows], pc.norm_weight, output=o,
                                 query_start_loc=qsl, num_accepted_tokens=acc)
                             for k in range(nset)]
                    t_us = rotating(torch, timer, calls)
                    bts = packed_fused_bytes(Ns, T, Hs, sb)
                    pf.append({"H": Hs, "N": Ns, "T": T, "state": "bf16" if sb == 2 else "fp32", "us": t_us,
                               "GBps": bts / (t_us * 1e-6) / 1e9, "frac": bts / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS})
                    log(f"packed fused H={Hs} N={Ns} T={T} {pf[-1]['state']}: {t_us:.1f} us, "
                        f"{pf[-1]['GBps']:.0f} GB/s")
                del pc
                torch.cuda.empty_cache()
        out["packed_fused_t5_accept1"] = pf
    return out


def stream_ceilings(torch, dev, timer):
    """Reference HBM streams timed with PyTorch's own kernels on 1 GiB
    working sets (GB/s of bytes moved): what a read-modify-write stream, a
    write-only stream and the packed fused call's one read to five writes of
    64 KiB blocks reach on this device without any of this library's code."""
    n = 1 << 28  # fp32 elements: 1 GiB
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    res = {}

    def rate(fn, nbytes, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        return nbytes / (timer.run(fn, reps) * 1e-6) / 1e9

    res["write_only_fill_GBps"] = rate(lambda: b.fill_(2.0), 4 * n)
    res["copy_GBps"] = rate(lambda: b.copy_(a), 8 * n)
    res["inplace_rmw_GBps"] = rate(lambda: a.mul_(1.0), 8 * n)
    blk = 1 << 14  # fp32 elements: 64 KiB blocks
    nblk = (n // 6) // blk
    src = a[: nblk * blk].view(nblk, 1, blk)
    dst = b[: nblk * 5 * blk].view(nblk, 5, blk) if 5 * nblk * blk <= n else None
    if dst is not None:
        res["one_read_five_writes_64KiB_GBps"] = rate(lambda: dst.copy_(src.expand(nblk, 5, blk)), 6 * 4 * nblk * blk)
    del a, b
    torch.cuda.empty_cache()
    for k, v in res.items():
        log(f"ceiling {k}: {v:.0f}")
    return res


FLOORS_LIB = os.path.join(ROOT, "libkda_floors.so")


def access_floors(torch, dev, timer, pool32):
    """The floor each benchmarked access pattern sets on this chip: kernels of
    bench_floors.hip that move exactly a workload's state bytes in its access
    pattern (random slots, tile per workgroup, lane layout) with one FMA per
    element and nothing else, timed like the workloads (graph replays over
    rotating slot sets).  Run after the workloads: the in-place floors
    rewrite the slots they touch."""
    if not os.path.exists(FLOORS_LIB):
        log("floors: libkda_floors.so is not built (build() compiles it); skipped")
        return None
    lib = ctypes.CDLL(FLOORS_LIB)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.floor_read_heads.argtypes = [vp, vp, vp, ci, ci, ci, vp]
    lib.floor_rmw_slices.argtypes = [vp, vp, ci, ci, ci, ci, vp]

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"floor probe launch failed ({rc})")

    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    res = {}
    perm = torch.randperm(pool32.shape[0], generator=g, device=dev).to(torch.int32)
    Bv, H = 64, 32
    sums = torch.empty(Bv * H, device=dev)
    for layout, name in ((0, "whole_rows"), (1, "matrix_core_order")):
        calls = [lambda ids=perm[j * Bv:(j + 1) * Bv].contiguous(), layout=layout: ok(lib.floor_read_heads(
            pool32.data_ptr(), ids.data_ptr(), sums.data_ptr(), Bv, H, layout, cur())) for j in range(8)]
        us = rotating(torch, timer, calls)
        nb = Bv * H * D * D * 4
        res[f"verify_state_read_b64_h32_fp32_{name}"] = {"us": us, "GBps": nb / (us * 1e-6) / 1e9}
        log(f"floor verify state read ({name}): {us:.1f} us, {nb / (us * 1e-6) / 1e9:.0f} GB/s")
    B = 256
    calls = [lambda ids=perm[j * B:(j + 1) * B].contiguous(): ok(lib.floor_rmw_slices(
        pool32.data_ptr(), ids.data_ptr(), B, H, D * D * 4, 8192, cur())) for j in range(pool32.shape[0] // B)]
    us = rotating(torch, timer, calls)
    nb = 2 * B * H * D * D * 4
    res["headline_state_rmw_b256_h32_fp32_8KiB"] = {"us": us, "GBps": nb / (us * 1e-6) / 1e9}
    log(f"floor headline state RMW: {us:.1f} us, {nb / (us * 1e-6) / 1e9:.0f} GB/s")
    SL, Hp = 8192, 12
    poolb = torch.zeros((SL, Hp, D, D), dtype=torch.bfloat16, device=dev)
    permb = torch.randperm(SL, generator=g, device=dev).to(torch.int32)
    for Bp in (256, 512):
        live = Bp - Bp // 8
        sets = []
        for j in range(8):
            ids = permb[j * Bp:(j + 1) * Bp].clone()
            ids[live:] = -1
            sets.append(ids.contiguous())
        nb = 2 * live * Hp * D * D * 2
        for sb in (4096, 8192, 16384, 32768, 4096, 8192):
            calls = [lambda ids=ids, sb=sb, Bp=Bp: ok(lib.floor_rmw_slices(
                poolb.data_ptr(), ids.data_ptr(), Bp, Hp, D * D * 2, sb, cur())) for ids in sets]
            us = rotating(torch, timer, calls)
            res[f"packed_state_rmw_b{Bp}_h12_bf16_{sb // 1024}KiB"] = {"us": us, "GBps": nb / (us * 1e-6) / 1e9}
            log(f"floor packed H=12 bf16 B={Bp} state RMW, {sb // 1024} KiB tiles: {us:.1f} us, "
                f"{nb / (us * 1e-6) / 1e9:.0f} GB/s")
    del poolb
    torch.cuda.empty_cache()
    # packed fused N=128 T=5 (one accepted token): each head read from the
    # sequence's first slot and written to its five checkpoint slots
    lib.floor_read1_write_k.argtypes = [vp, vp, ci, ci, ci, ci, vp]
    N, T = 128, 5
    slots = 4 * N * T + 1
    for hb, dt, name in ((D * D * 4, torch.float32, "fp32"), (D * D * 2, torch.bfloat16, "bf16")):
        poolf = torch.zeros((slots, Hp, D, D), dtype=dt, device=dev)
        pp = torch.randperm(slots - 1, generator=g, device=dev).to(torch.int32) + 1
        calls = [lambda ids=pp[k * N * T:(k + 1) * N * T].contiguous(), hb=hb, poolf=poolf: ok(lib.floor_read1_write_k(
            poolf.data_ptr(), ids.data_ptr(), N, Hp, hb, T, cur())) for k in range((slots - 1) // (N * T))]
        us = rotating(torch, timer, calls)
        nb = N * Hp * (1 + T) * hb
        res[f"packed_fused_state_read1_write5_n128_h12_{name}"] = {"us": us, "GBps": nb / (us * 1e-6) / 1e9}
        log(f"floor packed fused H=12 N=128 T=5 {name} state (1 read, 5 writes): {us:.1f} us, "
            f"{nb / (us * 1e-6) / 1e9:.0f} GB/s")
        del poolf
        torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ main ----

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--B", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--extra-only", default=None,
                    help="run only the extra workloads whose name contains this text (for profiling)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="also run a 1 GiB device copy (for counter scaling under rocprofv3)")
    ap.add_argument("--no-floors", action="store_true", help="skip the access-pattern floors (bench_floors.hip)")
    ap.add_argument("--ceilings", action="store_true",
                    help="also time reference HBM streams with PyTorch's own kernels (write-only, copy, "
                         "in-place read-modify-write, one read to five writes in 64 KiB blocks)")
    ap.add_argument("--packed-fused-n", default=None,
                    help="comma-separated sequence counts of the packed fused sweep (default: all)")
    ap.add_argument("--packed-b", default=None,
                    help="comma-separated batch sizes of the packed H=12 bf16 sweep (default: all; "
                         "the small sizes replay thousands of calls per cycle, too many for a counter pass)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(requested --gpus {args.gpus}); the decode shards with no communication "
              f"(rows or heads per GPU), so run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline()
        log(f"cpu baseline {cpu['value']:.1f} rows/s on {cpu['cores']} cores")

    import torch

    from gated_delta_rule_decode_amd import (fused_kda_decode, packed_kda_decode, recurrent_kda,
                                             synth)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    timer = Timer(torch, stream)
    log("device:", torch.cuda.get_device_name(dev))

    # ---- headline: recurrent T=1, H=32, fp32 pool [4096,32,128,128], B ----
    H, B, SLOTS = 32, args.B, 4096
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + B)
    log(f"building fp32 pool [{SLOTS},{H},128,128] ...")
    pool = synth._randn_big(gen, (SLOTS, H, D, D), dev, 0.05, torch.float32)
    c = synth.recurrent_case(1000 + B, n_seqs=B, H=H, num_slots=1, device=dev)
    idx = synth.unique_slots(gen, B, 0, SLOTS, dev)
    q4 = lambda t: t.reshape(B, 1, H, D)  # noqa: E731
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=dev)
    qq, kk, vv, gg, bb = q4(c.q), q4(c.k), q4(c.v), q4(c.g), c.beta.reshape(B, 1, H)

    def step():
        recurrent_kda(qq, kk, vv, gg, bb, c.A_log, c.dt_bias, initial_state=pool,
                      state_indices=idx, output=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps ...")
    t_wall0 = time.perf_counter()
    us = timer.run(step, args.steps)
    t_wall = time.perf_counter() - t_wall0
    bytes_launch = t1_bytes(B, 0, H, 4)
    state_bytes = t1_state_bytes(B, H, 4)
    achieved = bytes_launch / (us * 1e-6) / 1e9
    log(f"B={B}: {us:.1f} us/step, {achieved:.0f} GB/s algorithmic "
        f"({100 * achieved / HBM_PEAK_GBPS:.1f}% of 8 TB/s), wall {t_wall:.3f}s")

    # per-launch distribution (after the timed region, not part of `value`)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
    for a_ev, b_ev in evs:
        a_ev.record(stream)
        step()
        b_ev.record(stream)
    torch.cuda.synchronize()
    per = sorted(a_ev.elapsed_time(b_ev) * 1e3 for a_ev, b_ev in evs)
    dist = {"n": len(per), "median_us": per[len(per) // 2], "p10_us": per[len(per) // 10],
            "p90_us": per[(9 * len(per)) // 10]}
    log(f"per-launch: median {dist['median_us']:.1f} us, p10 {dist['p10_us']:.1f}, p90 {dist['p90_us']:.1f}")

    if args.copy_calibrate:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        cus = timer.run(lambda: dst.copy_(src), 10)
        log(f"copy 1 GiB -> 1 GiB: {cus:.1f} us, {2 * (1 << 30) / (cus * 1e-6) / 1e9:.0f} GB/s")
        del src, dst

    ceilings = stream_ceilings(torch, dev, timer) if args.ceilings else None

    traffic_bytes = load_traffic(bytes_launch)
    plan = launch_plan(c, idx, pool, out, B, H)
    result = {
        "metric": METRIC,
        "value": B * 1e6 / us,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": us / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded N(0,1) bf16 inputs, N(0,0.05) state)",
        "config": {"workload": f"recurrent_kda T=1 H=HV=32 K=V=128 fp32 state pool "
                               f"[4096,32,128,128], B={B} random unique slots, softplus gate",
                   "B": B, "H": H, "state_dtype": "fp32", "num_slots": SLOTS},
        "state_GBps": state_bytes / (us * 1e-6) / 1e9,
        "launch_distribution": dist,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if traffic_bytes is None else traffic_bytes / (us * 1e-6) / 1e9,
                     "traffic_bytes_per_launch": traffic_bytes,
                     "algorithmic_bytes_per_launch": bytes_launch,
                     "kernel": f"kda_recurrent_kernel (T=1, fp32 state, {plan['rows_per_block']} value "
                               f"rows per workgroup, {plan['grid_x']} workgroups)",
                     "practical_ceiling_GBps": 6600.0,
                     "practical_ceiling": "in-place read-modify-write probe over 1 GiB, 4 KiB per workgroup, "
                                          "nontemporal dwordx4 (measured on this MI355X)"},
        "cpu_baseline": cpu,
    }
    if ceilings is not None:
        result["ceilings"] = ceilings

    if not args.no_extra:
        packed_b = tuple(int(b) for b in args.packed_b.split(",")) if args.packed_b else None
        packed_fused_n = tuple(int(n) for n in args.packed_fused_n.split(",")) if args.packed_fused_n else None
        result["workloads"] = extra_workloads(torch, dev, timer, pool, args.extra_only, packed_b, packed_fused_n)
    if not args.no_floors and not args.extra_only:
        floors = access_floors(torch, dev, timer, pool)
        if floors is not None:
            result["floors"] = floors

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
