"""Host-only checks of the C ABI: the library loads, exports every entry point
include/kda.h declares, and validates arguments from host metadata alone
(the *_plan entry points never touch a device, so fake device addresses are
fine here)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
D = 128


def lib():
    return _lib.load()


def test_header_symbols_exported():
    text = open(HEADER).read()
    declared = re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", text)
    assert set(declared) == set(_lib.EXPORTS)
    L = lib()
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    L = lib()
    assert L.kda_version() == 6
    for code in _lib.STATUS:
        assert L.kda_status_string(code).decode()
    assert L.kda_status_string(12345).decode() == "unknown status"


def test_struct_layouts_match_header():
    """The C side rejects any struct_size other than its own sizeof, so a
    valid plan call proves the ctypes mirrors have the C layout."""
    r = rec_args()
    assert plan_rec(r)[0] == 0
    r.struct_size += 8
    assert plan_rec(r)[0] == -10
    p = packed_args()
    assert plan_packed(p)[0] == 0
    f = fused_args()
    assert plan_fused(f)[0] == 0


# ---- fake address space: disjoint, 16-byte aligned "device" buffers --------------

class Arena:
    def __init__(self):
        self.next = 1 << 32

    def take(self, nbytes):
        a = self.next
        self.next += (nbytes + 4096 + 255) & ~255
        return a


def rec_args(N=4, H=4, T=None, slots=8, bf16=False, varlen=False, HV=None, tps=1):
    A = Arena()
    HV = H if HV is None else HV
    T = N * tps if T is None else T
    a = _lib.RecurrentArgs()
    a.struct_size = ctypes.sizeof(_lib.RecurrentArgs)
    a.n_seqs, a.n_tokens, a.H, a.HV, a.K, a.V = N, T, H, HV, D, D
    for f, hh in (("q", H), ("k", H), ("v", HV), ("g", HV)):
        setattr(a, f, A.take(T * hh * D * 2))
        setattr(a, f + "_stride", hh * D)
    a.beta = A.take(T * HV * 2)
    a.beta_stride = HV
    a.A_log = A.take(HV * 4)
    a.dt_bias = A.take(HV * D * 4)
    a.scale, a.l2_eps = 0.08838834764831845, 1e-6
    es = 2 if bf16 else 4
    a.state = A.take(slots * HV * D * D * es)
    a.state_dtype = a.ckpt_dtype = 1 if bf16 else 0
    a.num_slots, a.slot_stride = slots, HV * D * D
    a.state_indices = A.take(N * 4)
    if varlen:
        a.cu_seqlens = A.take((N + 1) * 4)
    a.out = A.take(T * HV * D * 2)
    a.g_dtype = a.beta_dtype = 1
    a.tokens_per_seq = 0 if varlen else tps  # ragged: no declared longest sequence
    return a


def packed_args(B=8, H=12, slots=16):
    A = Arena()
    a = _lib.PackedArgs()
    a.struct_size = ctypes.sizeof(_lib.PackedArgs)
    a.B, a.H = B, H
    a.mixed_qkv, a.qkv_stride = A.take(B * 3 * H * D * 2), 3 * H * D
    a.raw_gate, a.gate_stride = A.take(B * H * D * 2), H * D
    a.raw_beta, a.beta_stride = A.take(B * H * 2), H
    a.A_log, a.dt_bias = A.take(H * 4), A.take(H * D * 4)
    a.state, a.state_dtype = A.take(slots * H * D * D * 2), 1
    a.num_slots, a.slot_stride = slots, H * D * D
    a.state_indices = A.take(B * 4)
    a.out = A.take(B * H * D * 2)
    return a


def fused_args(rows=4, H=8, slots=16):
    A = Arena()
    C3 = 3 * H * D
    a = _lib.FusedArgs()
    a.struct_size = ctypes.sizeof(_lib.FusedArgs)
    a.rows, a.H = rows, H
    a.x, a.x_stride = A.take(rows * C3 * 2), C3
    a.weight = A.take(12 * H * D * 4)
    a.conv_state, a.conv_slot_stride = A.take(slots * 3 * C3 * 2), 3 * C3
    a.raw_gate, a.gate_stride = A.take(rows * H * D * 2), H * D
    a.raw_beta, a.beta_stride = A.take(rows * H * 2), H
    a.A_log, a.dt_bias = A.take(H * 4), A.take(H * D * 4)
    a.state_indices = A.take(rows * 4)
    a.state, a.state_dtype = A.take(slots * H * D * D * 4), 0
    a.num_slots, a.slot_stride = slots, H * D * D
    a.output_gate, a.ogate_stride = A.take(rows * H * D * 2), H * D
    a.norm_weight, a.norm_eps = A.take(D * 4), 1e-5
    a.out = A.take(rows * H * D * 2)
    return a


def plan_rec(a):
    p = _lib.LaunchPlan()
    rc = lib().kda_recurrent_plan(ctypes.byref(a), ctypes.byref(p))
    return rc, p


def plan_packed(a):
    p = _lib.LaunchPlan()
    rc = lib().kda_packed_plan(ctypes.byref(a), ctypes.byref(p))
    return rc, p


def plan_fused(a):
    p = _lib.LaunchPlan()
    rc = lib().kda_fused_plan(ctypes.byref(a), ctypes.byref(p))
    return rc, p


def err():
    return lib().kda_last_error().decode()


# ---- launch geometry ---------------------------------------------------------------------

@pytest.mark.parametrize("N,H,bf16,vsplit", [(1, 32, False, 8), (4, 32, False, 4), (8, 32, False, 2), (6, 32, False, 4), (9, 32, False, 4),
                                             (10, 32, False, 8), (20, 12, False, 2), (7, 32, False, 2),
                                             (12, 32, False, 8), (256, 32, False, 8), (8, 12, False, 8),
                                             (16, 12, False, 4), (512, 12, True, 4), (64, 12, True, 2),
                                             (42, 12, True, 2), (96, 12, True, 2), (128, 12, True, 4),
                                             (16, 12, True, 4), (20, 12, True, 2),
                                             (1, 12, True, 8), (8, 12, True, 4), (4, 4, False, 8)])
def test_recurrent_plan_geometry(N, H, bf16, vsplit):
    rc, p = plan_rec(rec_args(N=N, H=H, slots=max(N, 8), bf16=bf16))
    assert rc == 0, err()
    assert p.vsplit == vsplit
    assert p.rows_per_block * p.vsplit == D
    assert p.grid_x == (N * H * vsplit + 7) // 8 * 8 and p.block == 256 and p.items == N * H
    assert p.kernel == 1


@pytest.mark.parametrize("N,H,bf16,read_only,vsplit", [
    (2, 32, False, False, 4), (2, 47, False, False, 4), (2, 48, False, False, 4), (8, 12, False, False, 4),
    (8, 32, False, False, 4), (12, 32, False, False, 2), (31, 32, False, False, 2), (32, 32, False, False, 1),
    (64, 16, False, False, 1), (64, 32, False, False, 1),
    (2, 47, False, True, 4), (2, 48, False, True, 2), (8, 32, False, True, 2), (32, 32, False, True, 1),
    (2, 47, True, False, 4), (2, 48, True, False, 2), (8, 32, True, False, 2), (32, 32, True, False, 1)])
def test_token_loop_plan_geometry(N, H, bf16, read_only, vsplit):
    """The token loop splits a head over workgroups only while the grid is
    small; an updating fp32 pool keeps 4 splits up to more items."""
    a = rec_args(N=N, H=H, T=3 * N, slots=max(N, 8), bf16=bf16, varlen=True)
    if read_only:
        a.flags = _lib.FLAG_NO_STATE_UPDATE
    rc, p = plan_rec(a)
    assert rc == 0, err()
    assert (p.kernel, p.vsplit, p.rows_per_block) == (2, vsplit, D // vsplit)
    assert p.grid_x == (N * H * vsplit + 7) // 8 * 8


@pytest.mark.parametrize("bf16,vsplit", [(False, 4), (True, 1)])
def test_token_loop_with_checkpoints_plan_geometry(bf16, vsplit):
    """A token loop writing fp32 checkpoints streams them in 32-row tiles at
    any size; bf16 checkpoints keep the size rule (whole heads at 1024 items)."""
    a = rec_args(N=64, H=16, T=190, slots=65, varlen=True, bf16=bf16)
    A = Arena()
    A.next = 1 << 40
    a.checkpoints = A.take(190 * 16 * D * D * (2 if bf16 else 4))
    rc, p = plan_rec(a)
    assert rc == 0, err()
    assert (p.kernel, p.vsplit, p.rows_per_block) == (2, vsplit, D // vsplit)


def test_varlen_and_fused_plans():
    rc, p = plan_rec(rec_args(N=64, H=16, T=190, slots=65, varlen=True))
    assert rc == 0, err()
    assert p.kernel == 2
    rc, p = plan_fused(fused_args(rows=256, H=32, slots=2048))
    assert rc == 0, err()
    assert (p.kernel, p.grid_x, p.vsplit, p.rows_per_block) == (3, 256 * 32, 1, 128)


def test_packed_plan_matches_recurrent():
    rc, p = plan_packed(packed_args(B=64, H=12, slots=1024))
    assert rc == 0, err()
    assert p.items == 64 * 12 and p.kernel == 1


# ---- validation -----------------------------------------------------------------------------

def expect(rc_p, code, fragment=""):
    rc = rc_p[0]
    assert rc == code, (rc, err())
    assert fragment in err()


def test_recurrent_validation_errors():
    a = rec_args(); a.q = 0
    expect(plan_rec(a), -1)
    a = rec_args(); a.K = 64
    expect(plan_rec(a), -7, "K=64")
    a = rec_args(); a.HV = 6
    expect(plan_rec(a), -7, "HV")
    a = rec_args(); a.n_tokens = 5
    expect(plan_rec(a), -2, "n_tokens")
    a = rec_args(); a.n_seqs = 0; a.n_tokens = 0
    expect(plan_rec(a), -2)
    a = rec_args(); a.state_dtype = 7
    expect(plan_rec(a), -3)
    a = rec_args(); a.q_stride = 100
    expect(plan_rec(a), -4)
    a = rec_args(); a.beta_stride = 1
    expect(plan_rec(a), -4)
    a = rec_args(); a.slot_stride = 4 * D * D - 4
    expect(plan_rec(a), -4)
    a = rec_args(); a.slot_stride = 4 * D * D + 1
    expect(plan_rec(a), -5)
    a = rec_args(); a.state += 4
    expect(plan_rec(a), -5)
    a = rec_args(); a.out += 2
    expect(plan_rec(a), -5)
    a = rec_args(); a.q += 1
    expect(plan_rec(a), -5)
    a = rec_args(); a.gate_mode = 1; a.lower_bound = -5.0
    expect(plan_rec(a), -7, "lower_bound")
    a = rec_args(); a.l2_eps = -1.0
    expect(plan_rec(a), -2)
    a = rec_args(); a.num_slots = 0
    expect(plan_rec(a), -2)


def test_recurrent_alias_detection():
    a = rec_args(); a.out = a.q
    expect(plan_rec(a), -6, "out overlaps")
    a = rec_args(); a.state = a.q - 16 * 4 * D * 0  # state starts where q starts
    expect(plan_rec(a), -6)
    a = rec_args(varlen=True, T=4); a.checkpoints = a.state; a.ckpt_dtype = 0
    expect(plan_rec(a), -6, "checkpoints")
    a = rec_args(); a.out = a.state + 16
    expect(plan_rec(a), -6)


def test_checkpoint_rules():
    a = rec_args(varlen=True, T=6)
    a.checkpoints = 1 << 40
    a.ckpt_dtype = 1
    expect(plan_rec(a), -7, "checkpoints")
    a.ckpt_dtype = 0
    assert plan_rec(a)[0] == 0, err()


def test_empty_varlen_is_valid():
    a = rec_args(N=3, T=0, varlen=True)
    a.q = a.k = a.v = a.g = a.beta = a.out = 0
    assert plan_rec(a)[0] == 0, err()


def test_packed_validation():
    a = packed_args(); a.qkv_stride = 3 * 12 * D - 1
    expect(plan_packed(a), -4)
    a = packed_args(); a.mixed_qkv = 0
    expect(plan_packed(a), -1)
    a = packed_args(); a.B = 0
    expect(plan_packed(a), -2)
    a = packed_args(); a.gate_mode = 1
    expect(plan_packed(a), -7)
    a = packed_args(); a.struct_size = 8
    expect(plan_packed(a), -10)


def test_fused_validation():
    a = fused_args(); a.conv_slot_stride = 10
    expect(plan_fused(a), -4)
    a = fused_args(); a.out = a.x
    expect(plan_fused(a), -6)
    a = fused_args(); a.conv_state = a.state
    expect(plan_fused(a), -6, "conv_state")
    a = fused_args(); a.norm_eps = -1.0
    expect(plan_fused(a), -2)
    a = fused_args(); a.norm_weight = 0
    expect(plan_fused(a), -1)
    a = fused_args(); a.state_dtype = 1
    assert plan_fused(a)[0] == 0, err()
    a = fused_args(); a.gate_mode = 1
    expect(plan_fused(a), -7)


def test_device_check_without_gpu_is_an_error_not_a_crash():
    """On a host without a GPU the device query fails cleanly."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib().kda_check_device(0) == -8


# ---- grouped value heads, precomputed gate, batched form, read-only pool --------

def test_grouped_heads_plan():
    rc, p = plan_rec(rec_args(N=64, H=4, HV=16, slots=64))
    assert rc == 0, err()
    assert p.items == 64 * 16 and p.kernel == 1
    a = rec_args(N=4, H=4, HV=16)
    a.v_stride = 4 * D  # v holds HV heads
    expect(plan_rec(a), -4, "v/g")
    a = rec_args(N=4, H=4, HV=16)
    a.beta_stride = 4
    expect(plan_rec(a), -4, "beta_stride")


def test_precomputed_gate_needs_no_gate_params():
    a = rec_args()
    a.gate_mode = 2
    a.A_log = a.dt_bias = 0
    a.g_dtype = a.beta_dtype = 0  # fp32 inputs; the arena left room for them
    assert plan_rec(a)[0] == 0, err()
    a = rec_args()
    a.A_log = 0
    expect(plan_rec(a), -1)
    a = rec_args()
    a.g_dtype = 5
    expect(plan_rec(a), -3)


def test_batched_form_and_flags():
    rc, p = plan_rec(rec_args(N=8, tps=4))
    assert rc == 0, err()
    assert p.kernel == 2  # token loop
    a = rec_args(N=8, tps=4)
    a.n_tokens = 31
    expect(plan_rec(a), -2, "tokens_per_seq")
    a = rec_args()
    a.flags = 2
    expect(plan_rec(a), -7, "flags")
    a = rec_args()
    a.flags = 1
    assert plan_rec(a)[0] == 0, err()


@pytest.mark.parametrize("tps", [2, 3, 4, 5, 8, 9, 12, 16])
@pytest.mark.parametrize("bf16", [False, True])
def test_read_only_batched_calls_take_a_verify_kernel(tps, bf16):
    """Read-only batched calls with 2..16 tokens and no checkpoints run as one
    matrix product per head on the WY verify kernel (family 5), one workgroup
    of 256 threads per head."""
    a = rec_args(N=64, H=32, tps=tps, slots=128, bf16=bf16)
    a.flags = 1
    rc, p = plan_rec(with_caches(a, t_max=tps))
    assert rc == 0, err()
    assert (p.kernel, p.vsplit, p.rows_per_block, p.block) == (5, 1, D, 256)
    assert p.grid_x == 64 * 32 and p.items == 64 * 32


@pytest.mark.parametrize("declared", [1, 3, 8, 16])
def test_read_only_ragged_calls_declaring_their_length_take_the_wy_verify_kernel(declared):
    """A read-only ragged call that declares its longest sequence (at most 16
    tokens) in tokens_per_seq runs as one matrix product per head."""
    a = rec_args(N=8, T=24, varlen=True)
    a.flags, a.tokens_per_seq = 1, declared
    rc, p = plan_rec(a)
    assert rc == 0, err()
    assert (p.kernel, p.vsplit, p.grid_x) == (5, 1, 8 * 4)


def test_calls_outside_the_wy_verify_kernel_keep_the_token_loop():
    """Updating pools, more than 16 tokens, ragged rows without a declared
    length (or one above 16) and checkpoints stay on the sequential token
    loop (family 2); T=1 on the T=1 kernel."""
    a = rec_args(N=8, tps=4)
    assert plan_rec(a)[1].kernel == 2  # updating
    a = rec_args(N=8, tps=17)
    a.flags = 1
    assert plan_rec(a)[1].kernel == 2  # 17 tokens
    a = rec_args(N=8, T=24, varlen=True)
    a.flags = 1
    assert plan_rec(a)[1].kernel == 2  # ragged, no declared length
    a.tokens_per_seq = 17
    assert plan_rec(a)[1].kernel == 2  # ragged, declared above 16
    a = rec_args(N=8, T=24, varlen=True)
    a.tokens_per_seq = 4
    assert plan_rec(a)[1].kernel == 2  # ragged, declared, but updating
    a = rec_args(N=8, tps=8)
    a.flags = 1
    a.q_stride += 4
    a.k_stride += 4
    a.k += 2
    assert plan_rec(a)[0] == 0 and plan_rec(a)[1].kernel == 5  # q/k rows need no alignment
    a = rec_args(N=8, tps=4)
    a.flags = 1
    A = Arena()
    A.next = 1 << 40
    a.checkpoints = A.take(32 * 4 * D * D * 4)
    assert plan_rec(a)[1].kernel == 2  # checkpoints
    a = rec_args(N=8)
    a.flags = 1
    assert plan_rec(a)[1].kernel == 1  # one token
    for f in ("q", "k", "v", "g", "beta"):
        # an input whose last token row of a sequence lies 2^31 bytes or more
        # past the first (the verify kernel's 32-bit row offsets)
        a = rec_args(N=8, tps=4)
        a.flags = 1
        es = 4 if f == "beta" else 2  # beta as fp32, the others bf16
        if f == "beta":
            a.beta_dtype = 0
        stride = (1 << 31) // (3 * es) + 1  # 3 rows past the first: just beyond 2^31 bytes
        setattr(a, f + "_stride", stride)
        A = Arena()
        A.next = 1 << 44
        setattr(a, f, A.take(32 * stride * 4))
        assert plan_rec(a)[0] == 0, err()
        assert plan_rec(a)[1].kernel == 2, f
        setattr(a, f + "_stride", stride - 4096)  # within 2^31: the verify kernel again
        assert plan_rec(a)[1].kernel == 5, f


def test_read_only_pool_still_may_not_alias_outputs():
    a = rec_args(varlen=True, T=4)
    a.flags = 1
    a.out = a.state
    expect(plan_rec(a), -6, "state")


def with_caches(a, t_max=4, kg_dtype=0, corr=True, kg=True):
    A = Arena()
    A.next = 1 << 40  # far from rec_args' buffers
    rows = a.num_slots * a.HV * t_max
    a.correction_cache = A.take(rows * D * 4) if corr else None
    a.kg_cache = A.take(rows * 2 * D * (4 if kg_dtype == 0 else 2)) if kg else None
    a.kg_dtype, a.cache_t_max = kg_dtype, t_max
    return a


def test_verify_cache_rules():
    for kw in ({}, {"kg_dtype": 1}, {"corr": False}, {"kg": False}):
        a = with_caches(rec_args(varlen=True, T=8), **kw)
        a.flags = 1
        assert plan_rec(a)[0] == 0, (kw, err())
    assert plan_rec(with_caches(rec_args()))[0] == 0, err()  # T=1 with caches
    expect(plan_rec(with_caches(rec_args(), t_max=0)), -2, "cache_t_max")
    expect(plan_rec(with_caches(rec_args(), kg_dtype=7)), -3, "kg_dtype")
    a = with_caches(rec_args())
    a.correction_cache += 4
    expect(plan_rec(a), -5, "correction_cache")
    a = with_caches(rec_args())
    a.correction_cache = a.state  # a cache may not overlap the pool
    expect(plan_rec(a), -6, "state")
    a = with_caches(rec_args())
    a.kg_cache = a.correction_cache + 64  # nor the other cache
    expect(plan_rec(a), -6, "cache")
    a = with_caches(rec_args(), corr=False)
    a.kg_cache = a.q  # nor an input
    expect(plan_rec(a), -6, "kg_cache")


def packed_fused_args(rows=10, N=3, T=4, H=12, slots=32, bf16=False):
    A = Arena()
    C3 = 3 * H * D
    a = _lib.PackedFusedArgs()
    a.struct_size = ctypes.sizeof(_lib.PackedFusedArgs)
    a.n_rows, a.n_seqs, a.H, a.max_tokens = rows, N, H, T
    a.x, a.x_stride = A.take(rows * C3 * 2), C3
    a.weight = A.take(12 * H * D * 4)
    a.conv_state, a.conv_slot_stride = A.take(slots * 3 * C3 * 2), 3 * C3
    a.raw_gate, a.gate_stride = A.take(rows * H * D * 2), H * D
    a.raw_beta, a.beta_stride = A.take(rows * H * 2), H
    a.A_log, a.dt_bias = A.take(H * 4), A.take(H * D * 4)
    a.state_indices, a.indices_stride = A.take(N * T * 4), T
    a.query_start_loc = A.take((N + 1) * 4)
    a.num_accepted_tokens = A.take(N * 4)
    es = 2 if bf16 else 4
    a.state, a.state_dtype = A.take(slots * H * D * D * es), 1 if bf16 else 0
    a.num_slots, a.slot_stride = slots, H * D * D
    a.output_gate, a.ogate_stride = A.take(rows * H * D * 2), H * D
    a.norm_weight, a.norm_eps = A.take(D * 4), 1e-5
    a.out = A.take(rows * H * D * 2)
    return a


def plan_pf(a):
    p = _lib.LaunchPlan()
    rc = lib().kda_packed_fused_plan(ctypes.byref(a), ctypes.byref(p))
    return rc, p


def test_packed_fused_plan_and_validation():
    rc, p = plan_pf(packed_fused_args())
    assert rc == 0, err()
    assert (p.kernel, p.grid_x, p.block, p.rows_per_block) == (4, 3 * 12, 512, 128)
    rc, p = plan_pf(packed_fused_args(N=128, T=5, rows=640, slots=700))
    assert rc == 0, err()
    assert (p.grid_x, p.block) == (128 * 12, 256)
    assert plan_pf(packed_fused_args(bf16=True))[0] == 0, err()
    a = packed_fused_args(rows=0)  # no rows at all: every sequence is empty
    a.x = a.raw_gate = a.raw_beta = a.output_gate = a.out = None
    assert plan_pf(a)[0] == 0, err()
    a = packed_fused_args()
    a.struct_size -= 8
    expect(plan_pf(a), -10)
    expect(plan_pf(packed_fused_args(N=0)), -2, "n_seqs")
    expect(plan_pf(packed_fused_args(T=0)), -2, "max_tokens")
    a = packed_fused_args()
    a.indices_stride = 3
    expect(plan_pf(a), -4, "indices_stride")
    a = packed_fused_args()
    a.gate_mode = 1
    expect(plan_pf(a), -7)
    a = packed_fused_args()
    a.query_start_loc = None
    expect(plan_pf(a), -1)
    a = packed_fused_args()
    a.out += 2
    expect(plan_pf(a), -5, "out")
    a = packed_fused_args()
    a.out = a.x  # output over an input
    expect(plan_pf(a), -6)
    a = packed_fused_args()
    a.conv_state = a.state  # the two caches may not overlap
    expect(plan_pf(a), -6)
    a = packed_fused_args()
    a.query_start_loc = a.state_indices  # metadata over metadata is fine (both read-only)
    assert plan_pf(a)[0] == 0, err()


def with_split(a, rows, N, H):
    A = Arena()
    A.next = 1 << 40  # clear of the other buffers
    a.split_counters = A.take(N * H * 4)
    a.split_partials = A.take(max(rows, 1) * H * D * 4)
    return a


@pytest.mark.parametrize("bf16,cases", [
    (True, ((1, 12, 4, 512), (3, 12, 4, 512), (5, 12, 4, 512), (6, 12, 2, 512), (8, 12, 2, 512),
            (10, 12, 2, 512), (11, 12, 1, 512), (32, 12, 1, 512), (128, 12, 1, 256), (1, 64, 2, 512),
            (2, 64, 1, 512))),
    (False, ((1, 12, 4, 512), (2, 12, 4, 512), (3, 12, 2, 512), (6, 12, 2, 512), (7, 12, 1, 512),
             (8, 12, 1, 512), (32, 12, 1, 512), (128, 12, 1, 256), (1, 64, 2, 512), (2, 64, 1, 512))),
])
def test_packed_fused_split_plan(bf16, cases):
    """With the split workspace, few (sequence, head) pairs spread each head
    over 4 or 2 workgroups (grid = pairs x split, 128/split value rows each;
    bf16 pools split up to more pairs than fp32 ones); many pairs, or no
    workspace, keep one workgroup per pair."""
    for N, H, vs, block in cases:
        rows = 5 * N
        args = packed_fused_args(rows=rows, N=N, T=5, H=H, slots=2 * N + 2, bf16=bf16)
        rc, p = plan_pf(with_split(args, rows, N, H))
        assert rc == 0, err()
        assert (p.vsplit, p.grid_x, p.block, p.rows_per_block, p.items) == (vs, N * H * vs, block, 128 // vs, N * H)
        rc, p = plan_pf(packed_fused_args(rows=rows, N=N, T=5, H=H, slots=2 * N + 2, bf16=bf16))
        assert rc == 0 and p.vsplit == 1 and p.grid_x == N * H, err()


def test_packed_fused_split_validation():
    a = with_split(packed_fused_args(), 10, 3, 12)
    a.split_partials = None  # both or neither
    expect(plan_pf(a), -1, "split_counters and split_partials")
    a = with_split(packed_fused_args(), 10, 3, 12)
    a.split_counters = None
    expect(plan_pf(a), -1, "split_counters and split_partials")
    a = with_split(packed_fused_args(), 10, 3, 12)
    a.split_partials += 4  # 16-byte alignment
    expect(plan_pf(a), -5, "split_partials")
    a = with_split(packed_fused_args(), 10, 3, 12)
    a.split_counters += 2
    expect(plan_pf(a), -5, "split_counters")
    a = with_split(packed_fused_args(), 10, 3, 12)
    a.split_partials = a.out  # scratch over the output
    expect(plan_pf(a), -6, "split_partials")
    a = with_split(packed_fused_args(), 10, 3, 12)
    a.split_counters = a.query_start_loc  # counters are written: not over metadata
    expect(plan_pf(a), -6, "split_counters")
    a = with_split(packed_fused_args(), 10, 3, 12)
    a.split_counters = a.split_partials + 10 * 12 * D * 4 - 4  # last partial = first counter
    expect(plan_pf(a), -6, "split_counters")


def test_sizes_that_would_overflow_are_rejected():
    """Extents are computed without wrap-around: strides and sizes whose
    buffers would exceed 2^48 bytes are errors, never silently small ranges."""
    a = rec_args()
    a.slot_stride = (1 << 44) + 16
    expect(plan_rec(a), -4, "slot_stride")
    a = rec_args()
    a.q_stride = 1 << 62
    expect(plan_rec(a), -2, "2^48")
    a = rec_args(varlen=True, T=8)
    a.n_seqs = 2 ** 31 - 1
    assert plan_rec(a)[0] < 0
    a = with_caches(rec_args())
    a.num_slots, a.cache_t_max = 1 << 20, 2 ** 31 - 1   # 2^53 cache rows
    expect(plan_rec(a), -2, "2^48")
    f = packed_fused_args()
    f.indices_stride = 1 << 61
    expect(plan_pf(f), -2, "2^48")


def test_validation_is_thread_safe_and_errors_are_thread_local():
    """Eight host threads call the plan entry points at once (ctypes drops the
    GIL around foreign calls), half with a valid argument set and half with
    an invalid one: every thread sees its own status and its own message."""
    import threading
    L = lib()
    errors = []

    def worker(bad, n=400):
        try:
            for _ in range(n):
                a = rec_args(N=8, H=4)
                if bad:
                    a.H = 0
                p = _lib.LaunchPlan()
                rc = L.kda_recurrent_plan(ctypes.byref(a), ctypes.byref(p))
                msg = L.kda_last_error().decode()
                if bad and (rc != -2 or "H" not in msg):
                    errors.append(("bad", rc, msg))
                if not bad and (rc != 0 or msg != ""):
                    errors.append(("good", rc, msg))
        except Exception as e:  # pragma: no cover - reported below
            errors.append(("exception", repr(e)))

    threads = [threading.Thread(target=worker, args=(i % 2 == 1,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]


def test_noalloc_entry_point_refuses_caller_scratch():
    """The allocation-free packed fused entry point takes its split scratch
    from the library: caller scratch pointers are refused, and so is a NULL
    or mis-sized argument struct, all before any HIP call."""
    L = lib()
    assert L.kda_packed_fused_decode_noalloc(None, None) == -1
    a = _lib.PackedFusedArgs()
    a.struct_size = ctypes.sizeof(_lib.PackedFusedArgs) + 8
    assert L.kda_packed_fused_decode_noalloc(ctypes.byref(a), None) == -10
    a.struct_size = ctypes.sizeof(_lib.PackedFusedArgs)
    a.split_counters = 1 << 32
    assert L.kda_packed_fused_decode_noalloc(ctypes.byref(a), None) == -7
    assert b"split_counters" in L.kda_last_error()


def test_packed_fused_workspace_sizes():
    """kda_packed_fused_workspace reports the split scratch a call would use:
    N*H*4 bytes of counters and rows*H*128*4 of outputs when the plan with a
    workspace splits its heads, nothing when it would not (many pairs), and
    an error (sizes 0) for invalid arguments or caller scratch pointers."""
    L = lib()

    def sizes(a):
        cb, pb = ctypes.c_int64(-1), ctypes.c_int64(-1)
        rc = L.kda_packed_fused_workspace(ctypes.byref(a), ctypes.byref(cb), ctypes.byref(pb))
        return rc, cb.value, pb.value

    for N, H, bf16 in ((1, 12, False), (3, 12, True), (8, 12, True), (128, 12, False), (2, 64, False)):
        a = packed_fused_args(rows=5 * N, N=N, T=5, H=H, slots=2 * N + 2, bf16=bf16)
        rc, cb, pb = sizes(a)
        assert rc == 0, err()
        vs = plan_pf(with_split(packed_fused_args(rows=5 * N, N=N, T=5, H=H, slots=2 * N + 2, bf16=bf16),
                                5 * N, N, H))[1].vsplit
        if vs > 1:
            assert (cb, pb) == (N * H * 4, 5 * N * H * D * 4), (N, H, bf16)
        else:
            assert (cb, pb) == (0, 0), (N, H, bf16)
    a = packed_fused_args(N=0)
    assert sizes(a) == (-2, 0, 0)
    a = with_split(packed_fused_args(N=1, rows=5), 5, 1, 12)
    assert sizes(a)[0] == -7 and b"must be NULL" in L.kda_last_error()
