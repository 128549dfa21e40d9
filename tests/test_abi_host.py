"""C-ABI library: it loads, exports every symbol the header declares, and rejects
bad arguments on the host before any HIP call (CPU only: no kernel runs here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "expsketch.h")


def _lib():
    from exp_density_sketching_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from exp_density_sketching_amd import build
        build.build()
    return _binding.raw()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("sketch_create", "sketch_update", "sketch_merge", "sketch_query",
                     "exact_attend", "sketch_destroy", "sketch_reset", "sketch_state",
                     "sk_strerror"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"libexpsketch.so does not export {name}"


def test_binding_covers_every_declared_symbol():
    from exp_density_sketching_amd import _binding
    assert sorted(_binding.EXPORTED) == declared_functions()


def test_strerror_and_version():
    lib = _lib()
    assert lib.sk_strerror(0) == b"ok"
    assert lib.sk_strerror(-1) == b"invalid argument"
    assert lib.sk_strerror(-3) == b"sketch shapes differ"
    assert lib.sk_strerror(12345) == b"unknown status"
    assert lib.sk_version() >= 100


@pytest.mark.parametrize("d,dv,p,h", [(3, 4, 2, 1), (4, 6, 2, 1), (2, 4, 2, 1),
                                      (256, 4, 1, 1), (4, 4, -1, 1), (4, 4, 17, 1),
                                      (4, 4, 2, 0)])
def test_create_rejects_bad_shapes(d, dv, p, h):
    lib = _lib()
    out = ctypes.c_void_p(1234)
    assert lib.sketch_create(d, dv, p, h, None, ctypes.byref(out)) == -1
    assert out.value is None


def test_create_rejects_null_out_and_huge_state():
    lib = _lib()
    assert lib.sketch_create(4, 4, 2, 1, None, None) == -1
    out = ctypes.c_void_p()
    # 128^16 * 129 floats: refused before any allocation
    assert lib.sketch_create(128, 128, 16, 1, None, ctypes.byref(out)) == -2
    assert out.value is None


def test_create_ex_checks_the_layout():
    lib = _lib()
    out = ctypes.c_void_p(1234)
    assert lib.sketch_create_ex(4, 4, 2, 1, 2, None, ctypes.byref(out)) == -1   # layout
    assert out.value is None
    assert lib.sketch_create_ex(4, 4, 8, 1, 1, None, ctypes.byref(out)) == -1   # p > 7
    assert lib.sketch_create_ex(4, 4, 2, 1, -1, None, ctypes.byref(out)) == -1
    # C(135, 7) ~ 1.6e11 multiset rows: refused before any allocation
    assert lib.sketch_create_ex(128, 128, 7, 1, 1, None, ctypes.byref(out)) == -2
    assert out.value is None


def test_null_handles_are_rejected():
    lib = _lib()
    assert lib.sketch_destroy(None) == 0
    assert lib.sketch_reset(None) == -1
    assert lib.sketch_update(None, None, None, 5) == -1
    assert lib.sketch_merge(None, None) == -1
    assert lib.sketch_query(None, None, 3, None, None) == -1
    assert lib.sketch_export(None, None) == -1
    assert lib.sketch_state(None, None, None, None, None) == -1
    assert lib.sketch_info(None, None, None, None, None, None, None) == -1
    assert lib.sketch_set_stream(None, None) == -1
    assert lib.sketch_layout(None, None, None) == -1
    assert lib.sketch_update_path(None, None) == -1
    assert lib.sketch_set_center(None, None) == -1
    assert lib.sketch_step(None, None, None, None, None, None) == -1


def test_exact_rejects_bad_arguments():
    lib = _lib()
    # unsupported d, negative n or m, null pointers with work to do
    assert lib.exact_attend(None, None, 4, 3, 4, 1, None, 1, None, None, None) == -1
    assert lib.exact_attend(None, None, -1, 4, 4, 1, None, 1, None, None, None) == -1
    assert lib.exact_attend(None, None, 4, 4, 4, 1, None, -2, None, None, None) == -1
    assert lib.exact_attend(None, None, 4, 4, 4, 0, None, 1, None, None, None) == -1
    assert lib.exact_attend(None, None, 4, 4, 4, 1, None, 1, None, None, None) == -1
    # m == 0 is an empty call
    assert lib.exact_attend(None, None, 4, 4, 4, 1, None, 0, None, None, None) == 0


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle and has no CPU compute path."""
    pkg = os.path.join(ROOT, "exp_density_sketching_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn
            assert "numpy" not in src or fn == "build.py", fn


def test_noalloc_exact_rejects_on_the_host():
    lib = _lib()
    fake = ctypes.c_void_p(4096)          # never dereferenced: refused before any HIP call
    assert lib.exact_attend_noalloc(None, None, 4, 3, 4, 1, None, 1, None, None, None) == -1
    assert lib.exact_attend_noalloc(None, None, 4, 4, 4, 1, None, 1, None, None, None) == -1
    assert lib.exact_attend_noalloc(None, None, 4, 4, 4, 1, None, 0, None, None, None) == 0
    # 32 heads x 2048 queries x (2 + 64) floats > 4,194,304: beyond the scratch
    assert lib.exact_attend_noalloc(fake, fake, 32, 4, 64, 32, fake, 2048, fake, fake,
                                    None) == -5
    assert lib.sk_strerror(-5) == b"request exceeds the fixed scratch buffer"


def test_coreset_create_rejects_on_the_host():
    lib = _lib()
    out = ctypes.c_void_p(1234)
    for args in [(3, 4, 2, 1, 64, 0.25), (4, 4, 17, 1, 64, 0.25), (4, 4, 2, 0, 64, 0.25),
                 (4, 4, 2, 1, 100, 0.25), (4, 4, 2, 1, 32, 0.25), (4, 4, 2, 1, 4096, 0.25),
                 (4, 4, 2, 1, 64, 0.0), (4, 4, 2, 1, 64, -1.0), (4, 4, 2, 1, 64, float("nan"))]:
        assert lib.coreset_create(*args, 0, None, ctypes.byref(out)) == -1, args
        assert out.value is None
    assert lib.coreset_create(4, 4, 2, 1, 64, 0.25, 0, None, None) == -1
    assert lib.coreset_destroy(None) == 0
    assert lib.coreset_update(None, None, None, 3) == -1
    assert lib.coreset_merge(None, None) == -1
    assert lib.coreset_query(None, None, 1, None, None) == -1
    assert lib.coreset_info(None, None, None, None) == -1
    assert lib.coreset_export(None, None, None, None) == -1
    assert lib.coreset_reset(None) == -1
    assert lib.coreset_set_stream(None, None) == -1
