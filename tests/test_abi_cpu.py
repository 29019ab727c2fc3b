"""CPU-side checks of the C ABI: the library loads and exports every symbol zl.h declares, and the
binding's ctypes structs have the header's layout."""
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


def test_binding_structs_match_the_header(tmp_path):
    """The ctypes mirrors of zl_segment, zl_plan_info_t and zl_group_info_t have the header's size
    and field offsets (zl_plan_info fills sizeof(zl_plan_info_t) bytes of the caller's struct):
    a C program compiled against include/zl.h prints them."""
    import ctypes
    import subprocess
    import coalesced_varlen_attention_amd as z
    structs = {"zl_segment": z._Segment, "zl_plan_info_t": z._PlanInfo, "zl_group_info_t": z._GroupInfo}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "zl.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(ROOT, "include")
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, stdout=subprocess.PIPE, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            cname, field, val = line.split()
            got[(cname, field)] = int(val)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), f"{cname}: size differs from the binding"
        for field, _ in cls._fields_:
            assert got[(cname, field)] == getattr(cls, field).offset, f"{cname}.{field}: offset differs"


def test_missing_library_raises(monkeypatch, tmp_path):
    """Without libzl.so the binding raises on first use (plan building included): there is no
    fallback path."""
    import pytest
    monkeypatch.setattr(z, "_LIB", None)
    monkeypatch.setattr(z, "_LIB_PATH", str(tmp_path / "libzl.so"))
    with pytest.raises(ImportError, match="no fallback"):
        z.lib()
    with pytest.raises(ImportError, match="no fallback"):
        z.Plan([64], [64], [1], [(0, 0, 1, 0, 64, 0, 64, -1)], 64, host_only=True)
