"""Checks on the HIP sources that need no GPU.

The kernels read their problem descriptors through a function that copies
every field into scalar registers one by one (find_problem in skinny.hip,
find_tiled in tiled.hip).  A field added to a descriptor but not to that copy
is read uninitialised on the device: undefined behaviour, which the compiler
may turn into anything (a windowed kernel whose branch on such a field lost
its barriers and never finished).  These tests hold the copies complete.
"""
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "weight_only_int4_group_amd", "csrc")


def _strip_comments(text):
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.sub(r"//[^\n]*", "", text)


def struct_fields(text, name):
    """Field names of `struct name { ... };` (plain declarations only)."""
    m = re.search(r"struct\s+" + name + r"\s*\{(.*?)\};", text, flags=re.S)
    assert m, f"struct {name} not found"
    fields = []
    for decl in m.group(1).split(";"):
        decl = decl.strip()
        if not decl:
            continue
        for i, piece in enumerate(decl.split(",")):
            ident = re.findall(r"[A-Za-z_]\w*", piece.replace("*", " "))
            assert ident, decl
            fields.append(ident[-1])
    return fields


def function_body(text, signature_regex):
    m = re.search(signature_regex, text)
    assert m, signature_regex
    i = text.index("{", m.end() - 1)
    depth = 0
    for j in range(i, len(text)):
        depth += {"{": 1, "}": -1}.get(text[j], 0)
        if depth == 0:
            return text[i:j + 1]
    raise AssertionError("unbalanced braces")


@pytest.mark.parametrize("source,struct,func", [
    ("skinny.hip", "Problem", r"Problem\s+find_problem\s*\([^)]*\)\s*\{"),
    ("tiled.hip", "TiledProblem", r"TiledProblem\s+find_tiled\s*\([^)]*\)\s*\{"),
])
def test_descriptor_copy_is_complete(source, struct, func):
    text = _strip_comments(open(os.path.join(CSRC, source)).read())
    fields = struct_fields(text, struct)
    body = function_body(text, func)
    assigned = set(re.findall(r"\bP\.(\w+)\s*=", body))
    missing = [f for f in fields if f not in assigned]
    assert not missing, f"{source}: {struct} fields not copied by the lookup: {missing}"
    assert len(fields) >= 15  # the parse saw the whole struct


def test_field_parser_sees_comma_lists():
    fields = struct_fields("struct T { const int *a, *b; int M, N;  float x; };", "T")
    assert fields == ["a", "b", "M", "N", "x"]


def _device_asm(source, tmp_path):
    """Device-only assembly of one library source, built with the library's flags."""
    import subprocess
    from weight_only_int4_group_amd import build
    flags = [f for f in build.compile_flags() if f not in ("-fPIC", "-shared")]
    out = str(tmp_path / (source + ".s"))
    res = subprocess.run([build.hipcc(), *flags, "--cuda-device-only", "-S",
                          os.path.join(CSRC, source), "-o", out], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _kernel_metadata(asm):
    """(name, private segment bytes, VGPR spills, SGPR spills) of every kernel in the
    assembly's metadata block."""
    kernels = []
    for block in asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        field = lambda key: int(re.search(r"\." + key + r":\s+(\d+)", block).group(1))
        kernels.append((name, field("private_segment_fixed_size"), field("vgpr_spill_count"),
                        field("sgpr_spill_count")))
    return kernels


@pytest.mark.parametrize("source", ["skinny.hip", "tiled.hip", "pack.hip", "outliers.hip",
                                    "gptq.hip", "spec.hip"])
def test_kernels_keep_everything_in_registers(source, tmp_path):
    """Every kernel compiles without register spills and without a private
    (per-lane scratch) segment.  A kernel whose accumulators land in scratch
    memory still computes the right values, so the GPU tests do not see it; it
    only runs several times slower (an instance whose helper lambdas were not
    inlined kept its accumulators there and took 19x the time)."""
    kernels = _kernel_metadata(_device_asm(source, tmp_path))
    assert kernels, f"{source}: no kernels found"
    bad = [k for k in kernels if k[1] or k[2] or k[3]]
    assert not bad, f"{source}: (kernel, private bytes, VGPR spills, SGPR spills): {bad}"
