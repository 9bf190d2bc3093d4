"""The ctypes structs of the binding lay out exactly as the C ABI's structs
(include/dgpass.h): size and the offset of every field, read from a small C
program compiled against the header with gcc.  A field added to one side only
would otherwise shift the others silently."""
import ctypes as C
import os
import shutil
import subprocess

import pytest

from block_diffusion_lm_denoise_amd import dgpass

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRUCTS = ("dg_config", "dg_layer_weights", "dg_weights", "dg_model", "dg_kv", "dg_taps",
           "dg_renoise_args")


def _c_layout(tmp_path):
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "dgpass.h"', "int main(void) {"]
    for name in STRUCTS:
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for f, _ in getattr(dgpass, name)._fields_:
            lines.append(f'  printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = {}
    for line in out.splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    return got


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_binding_structs_match_the_header(tmp_path):
    c = _c_layout(tmp_path)
    for name in STRUCTS:
        cls = getattr(dgpass, name)
        assert C.sizeof(cls) == c[(name, "size")], name
        for f, _ in cls._fields_:
            assert getattr(cls, f).offset == c[(name, f)], f"{name}.{f}"
