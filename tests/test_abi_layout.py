"""The ctypes structures of the binding match include/ua.h field by field:
a C program built from the header with the host compiler prints every
field's offset and each structure's size, and the binding must agree."""
import ctypes
import os
import shutil
import subprocess

import pytest

from varlen_attention_serving_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRUCTS = {"ua_problem_desc_t": B.ua_problem_desc_t, "ua_run_args_t": B.ua_run_args_t,
           "ua_plan_info_t": B.ua_plan_info_t, "ua_merge_args_t": B.ua_merge_args_t}


def _c_layout(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "ua.h"', "int main(void) {"]
    for name, cls in STRUCTS.items():
        lines.append(f'    printf("{name} size %zu\\n", sizeof({name}));')
        for field, _ in cls._fields_:
            lines.append(f'    printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines += ["    return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return {tuple(l.split()[:2]): int(l.split()[2]) for l in out.splitlines()}


def test_binding_structs_match_the_header(tmp_path):
    c = _c_layout(tmp_path)
    for name, cls in STRUCTS.items():
        assert c[(name, "size")] == ctypes.sizeof(cls), name
        for field, _ in cls._fields_:
            assert c[(name, field)] == getattr(cls, field).offset, (name, field)
