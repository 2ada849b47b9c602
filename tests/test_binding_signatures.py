"""The ctypes binding declares, for every C entry point, as many arguments as
include/fm.h does (checked on the CPU: no library call is made)."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_arity():
    src = open(os.path.join(ROOT, "include", "fm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(fm_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", src, re.S):
        args = m.group(2).strip()
        out[m.group(1)] = 0 if args in ("", "void") else args.count(",") + 1
    return out


def binding_sigs():
    txt = open(os.path.join(ROOT, "quantized_state_space_fwht_amd", "binding.py")).read()
    start = txt.index("_SIGS = {")
    end = txt.index("\n}\n", start)
    env = {"ctypes": ctypes, "_c_i64": ctypes.c_int64, "_c_i32": ctypes.c_int32,
           "_c_sz": ctypes.c_size_t, "_vp": ctypes.c_void_p}
    for cls in ("LayerDesc", "StaticParams", "QParams", "LayerTaps", "LayerWeights", "Cache",
                "CacheNarrow", "LayerOpts"):
        env[cls] = type(cls, (ctypes.Structure,), {"_fields_": []})
    exec(txt[start:end + 2], env)
    return env["_SIGS"]


def test_binding_arity_matches_header():
    decl = header_arity()
    sigs = binding_sigs()
    bad = {k: (len(v[1]), decl.get(k)) for k, v in sigs.items() if decl.get(k) != len(v[1])}
    assert not bad, bad
    assert set(decl) == set(sigs), set(decl) ^ set(sigs)
