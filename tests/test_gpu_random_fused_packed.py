"""Seeded random fused_kda_decode and packed_kda_decode calls against the
fp64 oracle ("flashinfer.kda_decode.fused_kda_decode" Parameters;
"Serving-native packed Kimi K3 decode"): random head counts and row counts,
null rows (0 and -1 for the fused call, -1 for the packed one) and indices
past the pool, padded QKV rows and padded conv-cache slots, fp32 or bf16
pools, every output, pool slot and conv-cache entry compared (the oracle
runs on the whole small pool).
"""
import random

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_decode_amd import fused_kda_decode, packed_kda_decode, synth
from tests import parity as P

pytestmark = pytest.mark.gpu
D = 128
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("seed", range(8))
def test_random_fused_calls(seed):
    rng = random.Random(7000 + seed)
    H = rng.choice([1, 2, 4, 8, 12, 32])
    rows = rng.randint(1, 48)
    slots = rows + rng.randint(1, 8)
    nz = rng.randint(0, rows // 3)
    nn = rng.randint(0, (rows - nz) // 3)
    dtype = rng.choice([torch.float32, torch.bfloat16])
    pad = rng.choice([0, 0, 16])
    say(f"random fused seed={seed} H={H} rows={rows} slots={slots} nulls={nz}+{nn} {dtype} slot_pad={pad}")
    c = synth.fused_case(7000 + seed, rows=rows, H=H, num_slots=slots, state_dtype=dtype, device=DEV,
                         null_zero=nz, null_neg=nn, slot_pad=pad)
    idx = c.state_indices.clone()
    if rows > 2 and rng.random() < 0.5:
        idx[rng.randrange(rows)] = slots + rng.randint(0, 5)  # past the pool: null
    c.state_indices.copy_(idx)
    want = oracle.fused(P.host(c.x), P.host(c.weight), oracle.as_np(c.conv_state.cpu()), P.host(c.raw_gate),
                        P.host(c.raw_beta), P.host(c.A_log), P.host(c.dt_bias), P.host(idx),
                        oracle.as_np(c.state.cpu()), P.host(c.output_gate), P.host(c.norm_weight))
    out = fused_kda_decode(c.x, c.weight, c.conv_state, c.raw_gate.reshape(1, rows, H, D),
                           c.raw_beta.reshape(1, rows, H), c.A_log, c.dt_bias, c.state_indices, c.state,
                           c.output_gate, c.norm_weight)
    torch.cuda.synchronize()
    P.check_bf16_out(out, want["out64"], "fused out")
    P.check_state(c.state, want["state"])
    got_cs = c.conv_state.cpu().contiguous().view(torch.int16)
    want_cs = torch.from_numpy(np.ascontiguousarray(want["conv_state"]).view(np.int16))
    assert torch.equal(got_cs, want_cs), "conv cache must be bit-exact"


@pytest.mark.parametrize("seed", range(8))
def test_random_packed_calls(seed):
    rng = random.Random(7100 + seed)
    H = rng.choice([1, 2, 4, 8, 12, 16])
    B = rng.randint(1, 64)
    slots = B + rng.randint(1, 16)
    nulls = rng.randint(0, B // 4)
    dtype = rng.choice([torch.float32, torch.bfloat16])
    row_pad = rng.choice([0, 0, 8, 24])
    say(f"random packed seed={seed} H={H} B={B} slots={slots} nulls={nulls} {dtype} row_pad={row_pad}")
    c = synth.packed_case(7100 + seed, B=B, H=H, num_slots=slots, state_dtype=dtype, device=DEV,
                          null_rows=nulls, row_pad=row_pad)
    idx = c.state_indices.clone()
    if B > 2 and rng.random() < 0.5:
        idx[rng.randrange(B)] = slots + rng.randint(0, 5)  # past the pool: null
    c.state_indices.copy_(idx)
    want = oracle.packed(P.host(c.mixed_qkv), P.host(c.raw_gate), P.host(c.raw_beta), P.host(c.A_log),
                         P.host(c.dt_bias), oracle.as_np(c.state.cpu()), P.host(idx))
    out = packed_kda_decode(c.mixed_qkv, c.raw_gate, c.raw_beta, c.A_log, c.dt_bias, c.state, c.state_indices)
    torch.cuda.synchronize()
    P.check_bf16_out(out, want["out64"])
    P.check_state(c.state, want["state"])
