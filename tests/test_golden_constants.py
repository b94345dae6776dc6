"""The oracle and the binding use the constants the pages print in the call
contracts (tests/golden/contract_constants.json, each value cited): head
dimension, fixed scale, L2 epsilon, RMSNorm epsilon default, conv width and
the null-row conventions.  CPU only."""
import inspect
import json
import math
import os

import numpy as np

import oracle
from gated_delta_rule_decode_amd import api

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "contract_constants.json")))


def test_oracle_constants_are_the_contract_values():
    assert oracle.D == GOLDEN["head_dim"]["value"]
    expr = GOLDEN["scale"]["expr"]
    assert expr.startswith("1/sqrt(") and expr.endswith(")")
    assert oracle.SCALE == 1.0 / math.sqrt(float(expr[len("1/sqrt("):-1]))
    assert oracle.L2_EPS == GOLDEN["l2_eps"]["value"]


def test_norm_eps_defaults_are_the_contract_value():
    want = GOLDEN["norm_eps_default"]["value"]
    for fn in (api.fused_kda_decode, api.packed_fused_kda_decode, oracle.fused, oracle.packed_fused):
        assert inspect.signature(fn).parameters["norm_eps"].default == want, fn.__name__


def test_conv_width_and_null_conventions_in_the_oracle():
    """The fused call takes 4 taps (weight [3, 4, H*128]) over a cache of the
    3 previous positions, which a live row shifts by one with x appended;
    index 0 is null for the fused call and -1 inactive for the packed call
    (zero outputs, caches untouched)."""
    H, W = 1, GOLDEN["conv_width"]["value"]
    rng = np.random.default_rng(1)
    C = 3 * H * 128
    x = rng.standard_normal((2, C)).astype(np.float32)
    bf = lambda a: oracle.bf16_from_f64(np.asarray(a, np.float64))  # noqa: E731
    weight = np.zeros((3, W, H * 128), np.float32)
    weight[:, 0, :] = 1.0
    cache = bf(rng.standard_normal((3, C, W - 1)))         # [slots, channels, W-1 positions], oldest first
    state = np.zeros((3, H, 128, 128), np.float32)
    gate = bf(np.zeros((2, H, 128)))
    beta = bf(np.zeros((2, H)))
    res = oracle.fused(bf(x), weight, cache.copy(), gate, beta, np.zeros(H, np.float32),
                       np.zeros(H * 128, np.float32), np.array([1, 0], np.int32), state,
                       bf(np.full((2, H, 128), 20.0)), np.ones(128, np.float32))
    shifted = oracle.bf16_to_f64(res["conv_state"][1])     # [channels, W-1]
    assert np.array_equal(shifted[:, :W - 2], oracle.bf16_to_f64(cache[1, :, 1:]))
    assert np.array_equal(shifted[:, W - 2], oracle.bf16_to_f64(bf(x[0])))
    assert np.all(res["out64"][1] == 0), "index 0 must be null for the fused call"
    assert np.array_equal(res["conv_state"][0], cache[0]) and np.array_equal(res["conv_state"][2], cache[2])
    qkv = bf(rng.standard_normal((2, 3 * H * 128)))
    pk = oracle.packed(qkv, bf(rng.standard_normal((2, H * 128))), bf(rng.standard_normal((2, H))),
                       np.zeros(H, np.float32), np.zeros(H * 128, np.float32),
                       rng.standard_normal((2, H, 128, 128)).astype(np.float32),
                       np.array([GOLDEN["packed_inactive_index"]["value"], 1], np.int32))
    assert np.all(pk["out64"][0] == 0), "index -1 must be inactive for the packed call"
