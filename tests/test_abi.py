"""The C-ABI library loads and exports every entry point include/bh.h declares.
No compute call is made (these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bh.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bh_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import barnes_hut_tree_amd as bh
    if not os.path.exists(bh.LIB_PATH):
        pytest.skip("libbh.so not built")
    return bh.load_library()


def test_header_declares_the_api():
    syms = declared_symbols()
    for name in ("bh_create", "bh_build", "bh_gravity", "bh_sync", "bh_destroy"):
        assert name in syms


def test_library_exports_every_declared_symbol(lib):
    import barnes_hut_tree_amd as bh
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(bh.EXPORTS)


def test_status_strings(lib):
    import barnes_hut_tree_amd as bh
    for code in (bh.BH_OK, bh.BH_ERR_INVALID, bh.BH_ERR_OOM, bh.BH_ERR_HIP, bh.BH_ERR_CAPACITY,
                 bh.BH_ERR_NONFINITE, bh.BH_ERR_NOT_BUILT, bh.BH_ERR_CONTENTION):
        s = bh.status_string(code)
        assert s and s != "unknown status"
    assert bh.status_string(12345) == "unknown status"


def test_create_rejects_bad_arguments_before_touching_the_device(lib):
    import barnes_hut_tree_amd as bh
    h = ctypes.c_void_p()
    assert lib.bh_create(None, 10, 0, None) == bh.BH_ERR_INVALID
    assert lib.bh_create(ctypes.byref(h), -1, 0, None) == bh.BH_ERR_INVALID
    assert lib.bh_create(ctypes.byref(h), 1 << 31, 0, None) == bh.BH_ERR_INVALID
    for kb, B, curve, res in ((31, 16, 0, 0), (63, 0, 0, 0), (63, 257, 0, 0), (63, 16, 2, 0),
                              (63, 16, 0, 1)):
        p = bh._Params(kb, B, 0, curve, res)
        assert lib.bh_create(ctypes.byref(h), 10, 0, ctypes.byref(p)) == bh.BH_ERR_INVALID
    assert lib.bh_build(None, None, 0, None) == bh.BH_ERR_INVALID
    assert lib.bh_gravity(None, None, 0, 0.5, 1.0, 0.0, None, None) == bh.BH_ERR_INVALID
    assert lib.bh_destroy(None) == bh.BH_OK
    assert lib.bh_direct(None, -1, None, -1, 1.0, 0.0, None, None) == bh.BH_ERR_INVALID
    assert lib.bh_direct(None, 4, None, 4, 1.0, 0.0, None, None) == bh.BH_ERR_INVALID
    assert lib.bh_direct(None, 0, None, 0, 1.0, -1.0, None, None) == bh.BH_ERR_INVALID
    assert lib.bh_direct(None, 0, None, 0, 1.0, 0.0, None, None) == bh.BH_OK


def test_product_path_has_no_cpu_fallback():
    # the package must not import the oracle or fall back to CPU code
    pkg = os.path.join(ROOT, "barnes_hut_tree_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), errors="replace").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f
