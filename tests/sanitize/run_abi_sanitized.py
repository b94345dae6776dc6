"""Run inside a process with libasan preloaded: load the sanitized host-only
build of the validation layer in place of the real library, run the ABI test
module against it, then fuzz every *_plan entry point with random argument
structs.  Any sanitizer report aborts the process with a non-zero status."""
import ctypes
import os
import random
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from gated_delta_rule_decode_amd import _lib  # noqa: E402

lib = _lib.load(sys.argv[1])

import pytest  # noqa: E402

rc = pytest.main(["-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")])
if rc != 0:
    sys.exit(rc)

rng = random.Random(1234)
INTS = [0, 1, -1, 2, 3, 4, 7, 8, 12, 16, 31, 32, 64, 127, 128, 129, 255, 256, 1023, 1024, 4096, 65535,
        2 ** 31 - 1, -(2 ** 31)]
I64S = INTS + [2 ** 40, 2 ** 62, -(2 ** 62), 2 ** 63 - 1, -(2 ** 63)]


def rand_field(ctype):
    if ctype in (ctypes.c_void_p,):
        return rng.choice([None, 16, 4096, 1 << 32, (1 << 32) + 2, (1 << 32) + 1, 1 << 47,
                           rng.randrange(1, 1 << 47)])
    if ctype is ctypes.c_float:
        return rng.choice([0.0, 1.0, -1.0, 1e-6, 1e-5, float("inf"), float("nan"), 0.0883883])
    if ctype is ctypes.c_int64:
        return rng.choice(I64S)
    if ctype is ctypes.c_uint32:
        return rng.choice([0, 1, 2, 3, 0xFFFFFFFF])
    return rng.choice(INTS)


plans = [(_lib.RecurrentArgs, lib.kda_recurrent_plan), (_lib.PackedArgs, lib.kda_packed_plan),
         (_lib.FusedArgs, lib.kda_fused_plan), (_lib.PackedFusedArgs, lib.kda_packed_fused_plan)]
seen = set()
for cls, fn in plans:
    for i in range(3000):
        a = cls()
        for name, ctype in cls._fields_:
            setattr(a, name, rand_field(ctype))
        if i % 2 == 0:
            a.struct_size = ctypes.sizeof(cls)  # reach the field checks past the ABI check
        p = _lib.LaunchPlan()
        r = fn(ctypes.byref(a), ctypes.byref(p) if i % 3 else None)
        assert r <= 0, r
        seen.add((cls.__name__, r))
        lib.kda_last_error()
# mutations of valid argument sets reach the deeper checks (aliasing, alignment, caches)
sys.path.insert(0, os.path.join(ROOT, "tests"))
import test_abi as T  # noqa: E402

makers = [
    (lambda: T.rec_args(), lib.kda_recurrent_plan),
    (lambda: T.rec_args(varlen=True, T=12, bf16=True), lib.kda_recurrent_plan),
    (lambda: T.rec_args(N=8, tps=4, HV=8), lib.kda_recurrent_plan),
    (lambda: T.with_caches(T.rec_args(varlen=True, T=8)), lib.kda_recurrent_plan),
    (lambda: T.packed_args(), lib.kda_packed_plan),
    (lambda: T.fused_args(), lib.kda_fused_plan),
    (lambda: T.packed_fused_args(), lib.kda_packed_fused_plan),
    (lambda: T.with_split(T.packed_fused_args(), 10, 3, 12), lib.kda_packed_fused_plan),
]
for make, fn in makers:
    base = make()
    fields = [f for f in type(base)._fields_ if f[0] != "struct_size"]
    for i in range(3000):
        a = make()
        for name, ctype in rng.sample(fields, rng.randint(1, 3)):
            v = rand_field(ctype)
            if ctype is ctypes.c_void_p and v is not None and rng.random() < 0.5:
                # point into (or next to) another buffer of the same call: aliasing paths
                other = getattr(a, rng.choice([f for f, t in fields if t is ctypes.c_void_p])) or 0
                v = other + rng.choice([0, 2, 16, 4096, -16])
                v = v if v > 0 else None
            setattr(a, name, v)
        p = _lib.LaunchPlan()
        r = fn(ctypes.byref(a), ctypes.byref(p))
        assert r <= 0, r
        seen.add((type(a).__name__, r))
print("fuzzed plan calls; status codes seen:", sorted(seen))
