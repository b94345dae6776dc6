"""The public header is a C header: it compiles as strict C99 with gcc, and
every argument struct has exactly the layout the Python binding's ctypes
mirrors assume (each field's offset and the struct's size), so a field added
to one and not the other, or in another order, fails here and not as a
silent misread on the device.  The C program also links the built library
and calls kda_version() (no device access).  CPU only.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

from gated_delta_rule_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = [("kda_launch_plan", _lib.LaunchPlan), ("kda_recurrent_args", _lib.RecurrentArgs),
           ("kda_packed_args", _lib.PackedArgs), ("kda_fused_args", _lib.FusedArgs),
           ("kda_packed_fused_args", _lib.PackedFusedArgs)]


def c_program():
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "kda.h"', "int main(void) {"]
    for cname, cls in STRUCTS:
        lines.append(f'    printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            lines.append(f'    printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines.append('    printf("version %d\\n", kda_version());')
    lines.append("    return 0;\n}")
    return "\n".join(lines) + "\n"


@pytest.fixture(scope="module")
def c_layout(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    d = tmp_path_factory.mktemp("hdr")
    src, exe = d / "layout.c", d / "layout"
    src.write_text(c_program())
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", libdir, "-l:libkda_mi355x.so", f"-Wl,-rpath,{libdir}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    out = {}
    for line in run.stdout.splitlines():
        parts = line.split()
        out[tuple(parts[:-1])] = int(parts[-1])
    return out


def test_header_compiles_as_c99_and_links(c_layout):
    assert c_layout[("version",)] == _lib.load().kda_version()


@pytest.mark.parametrize("cname,cls", STRUCTS, ids=[s[0] for s in STRUCTS])
def test_ctypes_mirror_matches_the_c_layout(c_layout, cname, cls):
    assert c_layout[(cname, "size")] == ctypes.sizeof(cls), f"{cname}: size differs"
    for field, _ in cls._fields_:
        assert c_layout[(cname, field)] == getattr(cls, field).offset, f"{cname}.{field}: offset differs"
