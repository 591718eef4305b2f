"""The C-ABI library loads and exports every function include/aatc.h declares (no GPU)."""
import ctypes
import os
import re

import quantized_attention_klt_amd as q

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "aatc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aatc_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(q.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_versions_and_status_strings():
    assert q.version() == 1 and q.layout_version() == 2
    assert q.status_string(0) == "ok"
    assert q.status_string(-6) == "capacity"
