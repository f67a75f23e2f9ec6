"""Host-only checks of the C ABI (no kernel is launched).

The library must load and export every function include/dgattn.h declares, and reject
malformed arguments with the documented status before any launch.  The argument checks pass
made-up device addresses into the real entry points, so they run in a child process that sees
no GPU (tests/abi_checks.py): if a check ever regressed, the call would fail to launch there
instead of running a kernel on an unmapped address.
"""
import json
import os
import re
import subprocess
import sys

import pytest

import gqa_flash_attention_dg_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgattn.h")
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import abi_checks  # noqa: E402

CHECK_NAMES = [f.__name__ for f in abi_checks.CHECKS]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dg.LIB_PATH):
        from gqa_flash_attention_dg_amd import build
        build.build()
    return dg.lib()


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(dg.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


@pytest.fixture(scope="module")
def isolated_results(L):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="",
               CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "abi_checks.py")], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("name", CHECK_NAMES)
def test_argument_checks_without_a_gpu(isolated_results, name):
    assert isolated_results.get(name) == "ok", isolated_results.get(name)


def prototypes():
    """{name: (return type, [parameter types])} of every function include/dgattn.h declares,
    with parameter names dropped and spacing normalised (`const float*`)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    out = {}
    for ret, name, params in re.findall(
            r"^\s*((?:const\s+)?\w+\s*\*?)\s*(\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.M | re.S):
        types = []
        for p in (x.strip() for x in params.split(",")):
            if p == "void" or not p:
                continue
            p = re.sub(r"\s+", " ", p.replace("*", " * ")).strip()
            words = p.split(" ")
            if words[-1] != "*" and len(words) > 1:
                words = words[:-1]                      # drop the parameter name
            types.append(" ".join(words).replace(" *", "*"))
        out[name] = (re.sub(r"\s+", " ", ret.replace("*", " *")).strip().replace(" *", "*"), types)
    return out


# The boundary calls in the form the method's hot path is specified with: headnorm + rope in
# place, split-GQA attention with an optional split-KV workspace, rel-pos attention (no
# workspace), and the error message.
BOUNDARY = {
    "dg_headnorm_rope": ("int", ["float*", "const float*", "const float*", "int", "int", "int",
                                 "int", "unsigned", "float", "void*"]),
    "dg_attn_split_gqa_workspace_size": ("size_t", ["int"] * 6),
    "dg_attn_split_gqa": ("int", ["const float*"] * 5 + ["float*"] + ["int"] * 6 +
                          ["float", "int", "void*", "size_t", "void*"]),
    "relpos_flash_attn": ("int", ["const float*"] * 3 + ["float*"] + ["int"] * 4 +
                          ["float", "void*"]),
    "dg_last_error": ("const char*", []),
}


@pytest.mark.parametrize("name", sorted(BOUNDARY))
def test_header_keeps_the_boundary_prototypes(name):
    assert prototypes()[name] == BOUNDARY[name]


def test_binding_argument_counts_match_the_header(L):
    for name, (_, params) in prototypes().items():
        argtypes = getattr(L, name).argtypes
        assert argtypes is not None and len(argtypes) == len(params), (name, argtypes, params)


def test_binding_refuses_bad_tensors_before_the_call():
    import torch
    x = torch.zeros(8)
    with pytest.raises(ValueError):
        dg._ptr(x, "x", 4)                                  # CPU tensor
    with pytest.raises(TypeError):
        dg._ptr(torch.zeros(8, dtype=torch.float64), "x", 4)
