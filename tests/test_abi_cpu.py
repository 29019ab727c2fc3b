"""CPU-side checks of the C ABI: the library loads and exports every symbol zl.h declares."""
import ctypes
import os
import re

import coalesced_varlen_attention_amd as z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "zl.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zl_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("zl_plan_build", "zl_attn_fwd", "zl_attn_bwd", "zl_lse_merge", "zl_plan_info", "zl_plan_destroy",
              "zl_last_error", "zl_plan_group", "zl_plan_tiles"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(z.lib_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"libzl.so lacks {missing}"


def test_last_error_is_a_string():
    assert isinstance(z.lib().zl_last_error(), bytes)
