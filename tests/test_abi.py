"""The C-ABI library loads and exports every symbol include/cdb.h declares;
host-side validation works without a GPU (no compute calls here)."""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "continuous_depth_batching_amd", "libcdb.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        subprocess.check_call([sys.executable, "-m", "continuous_depth_batching_amd.build"], cwd=ROOT)
    from continuous_depth_batching_amd import _lib
    return _lib


def declared_functions():
    src = open(os.path.join(ROOT, "include", "cdb.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cdb_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    decl = declared_functions()
    assert decl, "no declarations found"
    assert sorted(lib.EXPORTS) == decl
    for name in decl:
        assert hasattr(lib.lib, name), name


def test_strerror_and_version(lib):
    assert lib.lib.cdb_strerror(lib.CDB_EINVAL) == b"invalid argument"
    assert b"gfx950" in lib.lib.cdb_version()


def _dims(lib, **kw):
    base = dict(vocab=512, hidden=256, n_heads=4, head_dim=64, ffn=1024, n_prelude=0, n_core=2, n_coda=0,
                r_max=8, dtype=lib.CDB_FP32, kv_layout=lib.CDB_KV_DEPTH, inject=0, rms_eps=1e-6,
                rope_theta=10000.0, gate_bias=0.0, gate_threshold=0.0)
    base.update(kw)
    return lib.cdb_dims(**base)


def test_workspace_bytes_grows_with_rows(lib):
    d = _dims(lib)
    a = lib.lib.cdb_workspace_bytes(C.byref(d), 4, 64, 64)
    b = lib.lib.cdb_workspace_bytes(C.byref(d), 64, 64, 64)
    assert 0 < a < b


def test_invalid_dims_rejected_on_host(lib):
    for bad in (dict(r_max=0), dict(r_max=300), dict(head_dim=48), dict(dtype=7), dict(hidden=250),
                dict(kv_layout=4), dict(n_core=0), dict(gate_kind=2),
                dict(kv_layout=2, r_max=1)):
        d = _dims(lib, **bad)
        assert lib.lib.cdb_workspace_bytes(C.byref(d), 4, 64, 64) == 0, bad
    # every KV layout and both gate kinds are accepted
    for ok in (dict(kv_layout=1), dict(kv_layout=2), dict(kv_layout=lib.CDB_KV_DEPTH_COPY),
               dict(gate_kind=1, conv_threshold=0.3)):
        d = _dims(lib, **ok)
        assert lib.lib.cdb_workspace_bytes(C.byref(d), 4, 64, 64) > 0, ok
    # bf16 supports the Ouro and Huginn head widths
    for hd, nh in ((128, 2), (96, 2)):
        d = _dims(lib, dtype=lib.CDB_BF16, head_dim=hd, n_heads=nh, hidden=192 if hd == 96 else 256)
        assert lib.lib.cdb_workspace_bytes(C.byref(d), 4, 64, 64) > 0


def test_init_rejects_null_arguments_before_any_gpu_call(lib):
    out = C.c_void_p(123)
    rc = lib.lib.cdb_init(None, None, None, None, None, None, C.byref(out))
    assert rc == lib.CDB_EINVAL and out.value is None
    assert b"dims" in lib.lib.cdb_last_error()
    d = _dims(lib)
    rc = lib.lib.cdb_init(C.byref(d), None, None, None, None, None, C.byref(out))
    assert rc == lib.CDB_EINVAL


def test_calls_on_null_context_fail_cleanly(lib):
    assert lib.lib.cdb_core_step(None, None, 1) == lib.CDB_ESTATE
    assert lib.lib.cdb_sync(None) == lib.CDB_ESTATE
    lib.lib.cdb_destroy(None)


def test_pack_weight_rejects_bad_shapes_on_host(lib):
    L = lib
    dummy = C.c_void_p(0x1000)
    other = C.c_void_p(0x100000)
    # rows not a multiple of 16, cols not a multiple of the k-step, bad dtype, NULL, overlap
    assert L.lib.cdb_pack_weight(L.CDB_BF16, dummy, other, 15, 64, None) == L.CDB_EINVAL
    assert L.lib.cdb_pack_weight(L.CDB_BF16, dummy, other, 16, 48, None) == L.CDB_EINVAL
    assert L.lib.cdb_pack_weight(L.CDB_FP32, dummy, other, 16, 24, None) == L.CDB_EINVAL
    assert L.lib.cdb_pack_weight(7, dummy, other, 16, 64, None) == L.CDB_EINVAL
    assert L.lib.cdb_pack_weight(L.CDB_BF16, None, other, 16, 64, None) == L.CDB_EINVAL
    assert L.lib.cdb_pack_weight(L.CDB_BF16, dummy, C.c_void_p(0x1000 + 64), 16, 64, None) == L.CDB_EINVAL


def test_init_static_rejects_maxima_beyond_its_scratch(lib):
    """cdb_init_static (the entry point for callers that cannot allocate)
    refuses maxima whose workspace exceeds its 128 MiB static scratch, on the
    host, before any GPU call (the pointers below are never dereferenced)."""
    L = lib
    d = _dims(lib, vocab=49152, hidden=2048, n_heads=16, head_dim=128, ffn=5632, n_core=24, r_max=4,
              dtype=L.CDB_BF16)
    need = L.lib.cdb_workspace_bytes(C.byref(d), 256, 8192, 4096)
    assert need > 128 << 20
    fake = C.c_void_p(0x10000)
    kv = L.cdb_kv(16, 1, fake, fake, None, None, fake, fake, 1, 256)
    pools = L.cdb_pools(fake, None, None, 4, None, 0, 256, 8192, 4096)
    seqs = L.cdb_seqs(fake, fake, fake, fake, 4)
    lay = (L.cdb_layer * 24)(*[L.cdb_layer(fake, fake, fake, fake, fake, fake) for _ in range(24)])
    wts = L.cdb_weights(fake, None, lay, None, fake, fake, fake)
    ctx = C.c_void_p()
    rc = L.lib.cdb_init_static(C.byref(d), C.byref(wts), C.byref(kv), C.byref(pools), C.byref(seqs), None,
                               C.byref(ctx))
    assert rc == L.CDB_ENOMEM and not ctx.value
    assert b"static scratch" in L.lib.cdb_last_error()
    # a caller workspace is not accepted by this entry point
    pools2 = L.cdb_pools(fake, None, None, 4, fake, 1 << 30, 4, 16, 4096)
    rc = L.lib.cdb_init_static(C.byref(d), C.byref(wts), C.byref(kv), C.byref(pools2), C.byref(seqs), None,
                               C.byref(ctx))
    assert rc == L.CDB_EINVAL and not ctx.value
