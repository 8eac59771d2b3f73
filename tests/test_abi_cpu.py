"""CPU checks of the C-ABI library: it loads, exports every symbol that
include/absa.h declares, and rejects bad arguments before any HIP call (so
these run without a GPU). No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

import sampled_block_sparse_amd as absa
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "absa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(absa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_interface():
    names = declared_functions()
    for required in ("absa_plan_create", "absa_plan_from_scores", "absa_plan_import",
                     "absa_plan_info", "absa_plan_export", "absa_plan_export_intermediate",
                     "absa_sparse_attention", "absa_dense_attention", "absa_plan_destroy",
                     "absa_status_string", "absa_last_error", "absa_plan_params_init",
                     "absa_plan_scores", "absa_sparse_attention_noalloc"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = absa.get_lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", absa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (absa_\w+)", out))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_c():
    src = '#include "absa.h"\nint main(void){absa_plan_params p; return (int)absa_plan_params_init(&p);}\n'
    path = os.path.join(ROOT, "_build_header_check.c")
    try:
        with open(path, "w") as f:
            f.write(src)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I",
                        os.path.join(ROOT, "include"), path], check=True)
    finally:
        os.remove(path)


def test_status_strings():
    assert absa.absa_status_string(0) == "ABSA_OK"
    assert absa.absa_status_string(5) == "ABSA_ERR_PLAN_MISMATCH"
    assert absa.absa_status_string(99) == "ABSA_UNKNOWN_STATUS"


def test_params_init_defaults():
    lib = absa.get_lib()
    p = absa._Params()
    assert lib.absa_plan_params_init(ctypes.byref(p)) == 0
    assert (p.query_block, p.kv_block, p.n_clusters, p.kmeans_iters) == (128, 4, 8, 4)
    assert (p.keep_intermediates, p.sampling, p.fused) == (0, 0, 0)
    assert lib.absa_plan_params_init(None) == absa.ABSA_ERR_INVALID_ARG


def test_params_struct_matches_header():
    """The binding's params struct has the C layout (size and field offsets
    as the compiler lays out include/absa.h)."""
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f[0] for f in absa._Params._fields_]
    body = "".join(f'printf("%zu ", offsetof(absa_plan_params, {f}));' for f in fields)
    src = ('#include <stdio.h>\n#include <stddef.h>\n#include "absa.h"\n'
           f'int main(void){{{body} printf("%zu", sizeof(absa_plan_params)); return 0;}}\n')
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "layout.c")
        exe = os.path.join(tmp, "layout")
        open(c, "w").write(src)
        subprocess.run([cc, "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                              check=True).stdout.split()]
    want = [getattr(absa._Params, f).offset for f in fields] + [ctypes.sizeof(absa._Params)]
    assert got == want


_FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: every call below fails validation


def _create(**kw):
    lib = absa.get_lib()
    p = absa._Params()
    lib.absa_plan_params_init(ctypes.byref(p))
    p.budget_blocks = 10
    shape = dict(B=1, H=2, N=1024, d=64, dtype=absa.ABSA_BF16)
    q = kw.pop("q", _FAKE)
    for key in list(kw):
        if hasattr(p, key):
            setattr(p, key, kw.pop(key))
    shape.update(kw)
    out = ctypes.c_void_p(123)
    st = lib.absa_plan_create(q, _FAKE, shape["dtype"], shape["B"], shape["H"], shape["N"],
                              shape["d"], ctypes.byref(p), None, ctypes.byref(out))
    assert out.value in (None, 0)
    return st


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), absa.ABSA_ERR_INVALID_ARG),
    (dict(d=96), absa.ABSA_ERR_UNSUPPORTED),
    (dict(d=32), absa.ABSA_ERR_UNSUPPORTED),
    (dict(N=1026), absa.ABSA_ERR_UNSUPPORTED),
    (dict(N=0), absa.ABSA_ERR_UNSUPPORTED),
    (dict(N=(1 << 21) + 4), absa.ABSA_ERR_UNSUPPORTED),
    (dict(B=0), absa.ABSA_ERR_INVALID_ARG),
    (dict(H=-1), absa.ABSA_ERR_INVALID_ARG),
    (dict(dtype=7), absa.ABSA_ERR_UNSUPPORTED),
    (dict(budget_blocks=0), absa.ABSA_ERR_INVALID_ARG),
    (dict(budget_blocks=257), absa.ABSA_ERR_INVALID_ARG),
    (dict(query_block=64), absa.ABSA_ERR_UNSUPPORTED),
    (dict(kv_block=8), absa.ABSA_ERR_UNSUPPORTED),
    (dict(n_clusters=0), absa.ABSA_ERR_UNSUPPORTED),
    (dict(n_clusters=17), absa.ABSA_ERR_UNSUPPORTED),
    (dict(kmeans_iters=0), absa.ABSA_ERR_INVALID_ARG),
    (dict(sampling=2), absa.ABSA_ERR_INVALID_ARG),
    (dict(sampling=-1), absa.ABSA_ERR_INVALID_ARG),
    # the fused plan path: at most 8 clusters, rows of at most 20,224 blocks,
    # no retained intermediates
    (dict(fused=1, n_clusters=9), absa.ABSA_ERR_UNSUPPORTED),
    (dict(fused=1, N=4 * 20225, budget_blocks=10), absa.ABSA_ERR_UNSUPPORTED),
    (dict(fused=1, keep_intermediates=1), absa.ABSA_ERR_UNSUPPORTED),
    # the score kernels put B*H on the grid's second dimension
    (dict(B=2, H=40000, N=128, budget_blocks=1), absa.ABSA_ERR_UNSUPPORTED),
])
def test_plan_create_rejects(kw, status):
    assert _create(**kw) == status
    assert absa.absa_last_error() != ""


def test_other_calls_reject_before_device_work():
    lib = absa.get_lib()
    out = ctypes.c_void_p()
    assert lib.absa_plan_create(_FAKE, _FAKE, 0, 1, 1, 1024, 64, None, None,
                                ctypes.byref(out)) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_plan_create(_FAKE, _FAKE, 0, 1, 1, 1024, 64, None, None,
                                None) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_plan_from_scores(None, 1, 1, 1024, 64, 10, 0, 0, None,
                                     ctypes.byref(out)) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_plan_from_scores(_FAKE, 1, 1, 1024, 64, 0, 0, 0, None,
                                     ctypes.byref(out)) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_plan_from_scores(_FAKE, 1, 1, 1000, 80, 10, 0, 0, None,
                                     ctypes.byref(out)) == absa.ABSA_ERR_UNSUPPORTED
    assert lib.absa_plan_from_scores(_FAKE, 1, 1, 1024, 64, 10, 0, 5, None,
                                     ctypes.byref(out)) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_sparse_attention(None, _FAKE, _FAKE, _FAKE, _FAKE, 0, 1, 1, 1024, 64,
                                     None) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_dense_attention(_FAKE, _FAKE, None, _FAKE, 0, 1, 1, 1024, 64,
                                    None) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_dense_attention(_FAKE, _FAKE, _FAKE, _FAKE, 0, 1, 1, 1024, 48,
                                    None) == absa.ABSA_ERR_UNSUPPORTED
    assert lib.absa_dense_attention(_FAKE, _FAKE, _FAKE, _FAKE, 3, 1, 1, 1024, 64,
                                    None) == absa.ABSA_ERR_UNSUPPORTED
    assert lib.absa_plan_info(None, None, None, None, None) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_plan_export(None, None, None, None, None) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_plan_export_intermediate(None, 0, 0, 0, None) == absa.ABSA_ERR_INVALID_ARG
    ptr = ctypes.c_void_p(7)
    assert lib.absa_plan_scores(None, ctypes.byref(ptr)) == absa.ABSA_ERR_INVALID_ARG
    assert lib.absa_sparse_attention_noalloc(None, _FAKE, _FAKE, _FAKE, _FAKE, 0, 1, 1, 1024, 64,
                                             None) == absa.ABSA_ERR_INVALID_ARG
    lib.absa_plan_destroy(None)     # no-op


def _import(rowptr, idx, logw, N=64, d=64):
    import numpy as np
    rowptr = np.asarray(rowptr, np.int64)
    idx = np.asarray(idx, np.int32)
    logw = np.asarray(logw, np.float32)
    out = ctypes.c_void_p()
    st = absa.get_lib().absa_plan_import(rowptr.ctypes.data_as(ctypes.c_void_p),
                                         idx.ctypes.data_as(ctypes.c_void_p),
                                         logw.ctypes.data_as(ctypes.c_void_p), None,
                                         1, 1, N, d, None, ctypes.byref(out))
    return st


@pytest.mark.parametrize("rowptr,idx,logw", [
    ([1, 2], [0, 1], [0.0, 0.0]),              # rowptr[0] != 0
    ([0, 2], [1, 1], [0.0, 0.0]),              # not strictly ascending
    ([0, 2], [3, 1], [0.0, 0.0]),              # descending
    ([0, 1], [16], [0.0]),                     # index >= M (M = 16)
    ([0, 1], [-1], [0.0]),                     # negative index
    ([0, 1], [0], [float("inf")]),             # non-finite log-weight
    ([0, 17], list(range(17)), [0.0] * 17),    # more than M blocks
])
def test_plan_import_rejects(rowptr, idx, logw):
    assert _import(rowptr, idx, logw) == absa.ABSA_ERR_INVALID_ARG
    assert absa.absa_last_error()


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        absa.absa_dense_attention(q, q, q)


@pytest.mark.parametrize("what", ["short rowptr", "long rowptr", "short idx", "short logw",
                                  "short p"])
def test_binding_checks_import_lengths(what):
    """The C import reads rowptr[0..rows] and rowptr[rows] entries of the
    other arrays (it has no length arguments): the binding rejects arrays of
    the wrong length before calling it. B=1, H=2, N=256: rows = 4."""
    import numpy as np
    rowptr = np.array([0, 2, 3, 3, 5], np.int64)
    idx = np.array([0, 5, 1, 7, 9], np.int32)
    logw = np.zeros(5, np.float32)
    p = np.ones(5)
    if what == "short rowptr":
        rowptr = rowptr[:3]
    elif what == "long rowptr":
        rowptr = np.append(rowptr, 5)
    elif what == "short idx":
        idx = idx[:4]
    elif what == "short logw":
        logw = logw[:2]
    else:
        p = p[:4]
    with pytest.raises(ValueError):
        absa.absa_plan_import(rowptr, idx, logw, p, 1, 2, 256, 64)
