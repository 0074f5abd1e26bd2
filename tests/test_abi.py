"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments before touching
the GPU (no compute calls here; these run without a GPU)."""

import ctypes
import os
import re

import pytest

import block_sparse_attention_ibcs_amd as ab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ab_attn.h")


def _lib():
    try:
        return ab.load_library()
    except ImportError as e:
        pytest.fail(f"libabattn.so not built: {e}")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ab_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert set(_declared_functions()) == set(ab.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.ab_abi_version() == 1


def test_status_strings():
    lib = _lib()
    for code in range(0, -9, -1):
        assert lib.ab_status_str(code)
    assert lib.ab_status_str(-99) == b"unknown status"


def _desc(**kw):
    base = dict(B=1, H=12, N=32760, d=128, dtype=ab.AB_BF16, q_block=128, k_block=32, n_clusters=8, kmeans_iters=4)
    base.update(kw)
    return ab.Desc(**base)


def test_workspace_size_covers_tables():
    d = _desc()
    n = ab.ab_score_workspace_size(d)
    heads = 12
    nqb, nkb = 256, 1024
    ell = heads * nqb * nkb * 8 * 4
    cent = heads * nqb * 8 * 128 * (4 + 2)
    assert n >= ell + cent
    assert n < ell + cent + 64 * 1024 * 1024  # the partial tables are small


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(d=96), -2),
        (dict(N=0), -2),
        (dict(B=0), -2),
        (dict(dtype=7), -5),
        (dict(q_block=32), -3),
        (dict(k_block=48), -3),
        (dict(k_block=256), -3),
        (dict(n_clusters=0), -3),
        (dict(n_clusters=129), -3),
        (dict(kmeans_iters=0), -3),
        (dict(kmeans_iters=65), -3),
        (dict(N=1 << 25), -2),
        (dict(N=1 << 23, k_block=128), -2),  # one bf16 d=128 head of K is 2 GiB
        (dict(N=1 << 22, k_block=128, dtype=1), -2),  # one fp32 d=128 head is 2 GiB
    ],
)
def test_validation_errors(kw, code):
    lib = _lib()
    cd = _desc(**kw).c()
    assert lib.ab_score_workspace_size(ctypes.byref(cd)) == 0
    fake = ctypes.c_void_p(256)
    rc = lib.ab_score(ctypes.byref(cd), fake, fake, fake, fake, 1 << 40, None)
    assert rc == code
    assert lib.ab_last_error()
    rc = lib.ab_attn_fwd(ctypes.byref(cd), fake, fake, fake, fake, fake, fake, fake, None, None)
    assert rc == code


def test_null_and_workspace_errors():
    lib = _lib()
    cd = _desc().c()
    fake = ctypes.c_void_p(256)
    need = lib.ab_score_workspace_size(ctypes.byref(cd))
    assert lib.ab_score(None, fake, fake, fake, fake, need, None) == -1
    assert lib.ab_score(ctypes.byref(cd), None, fake, fake, fake, need, None) == -1
    assert lib.ab_score(ctypes.byref(cd), fake, fake, fake, fake, need - 1, None) == -6
    assert b"workspace" in lib.ab_last_error()
    assert lib.ab_score(ctypes.byref(cd), fake, fake, fake, ctypes.c_void_p(256 + 16), need, None) == -6
    assert lib.ab_attn_fwd(ctypes.byref(cd), fake, fake, None, fake, fake, fake, fake, None, None) == -1
    assert lib.ab_score_debug(ctypes.byref(cd), fake, None, None, None, None) == -1


@pytest.mark.parametrize("density", [0.0, -0.5, 1.0000001, float("nan"), float("inf")])
def test_density_errors(density):
    lib = _lib()
    cd = _desc().c()
    fake = ctypes.c_void_p(256)
    rc = lib.ab_sample(ctypes.byref(cd), fake, ctypes.c_double(density), 0, fake, fake, fake, None, None)
    assert rc == -4
    assert b"density" in lib.ab_last_error()


@pytest.mark.parametrize("density", [0.0, float("nan"), 2.0])
def test_topk_density_errors(density):
    lib = _lib()
    cd = _desc().c()
    fake = ctypes.c_void_p(256)
    assert lib.ab_sample_topk(ctypes.byref(cd), fake, ctypes.c_double(density), fake, fake, fake, None, None) == -4


def test_systematic_validation():
    lib = _lib()
    fake = ctypes.c_void_p(256)
    cd = _desc().c()
    assert lib.ab_sample_systematic(ctypes.byref(cd), fake, ctypes.c_double(0.0), 0, fake, fake, fake, None, None) == -4
    assert lib.ab_sample_systematic(ctypes.byref(cd), fake, ctypes.c_double(0.1), 0, None, fake, fake, None, None) == -1
    cd = _desc(N=16385 * 16, k_block=16).c()
    assert lib.ab_sample_systematic(ctypes.byref(cd), fake, ctypes.c_double(0.1), 0, fake, fake, fake, None, None) == -2


def test_topk_rejects_long_rows_and_nulls():
    lib = _lib()
    fake = ctypes.c_void_p(256)
    # 16385 sub-blocks of 16 keys: one more than the top-K kernel takes
    cd = _desc(N=16385 * 16, k_block=16).c()
    assert lib.ab_sample_topk(ctypes.byref(cd), fake, ctypes.c_double(0.1), fake, fake, fake, None, None) == -2
    assert b"16384" in lib.ab_last_error()
    cd = _desc(N=16384 * 16, k_block=16).c()
    assert lib.ab_sample_topk(ctypes.byref(cd), None, ctypes.c_double(0.1), fake, fake, fake, None, None) == -1
    assert lib.ab_sample_topk(ctypes.byref(cd), fake, ctypes.c_double(0.1), fake, None, fake, None, None) == -1


def test_python_binding_rejects_host_tensors():
    import torch

    d = _desc(H=1, N=256, d=64, dtype=ab.AB_F32, q_block=64, k_block=16, n_clusters=4)
    q = torch.zeros(1, 1, 256, 64)
    with pytest.raises(ValueError):
        ab.ab_score(d, q, q, workspace=torch.zeros(16, dtype=torch.uint8))


def test_fp8_workspace_and_validation():
    """FP8 entry points: workspace size (one fp32 per head and key sub-block plus one
    per head), and every argument error caught before any device work."""
    lib = _lib()
    cd = _desc().c()
    need = lib.ab_fp8_workspace_size(ctypes.byref(cd))
    assert need == 1 * 12 * (1024 + 1) * 4
    assert lib.ab_fp8_workspace_size(ctypes.byref(_desc(d=96).c())) == 0
    fake = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(256 + 8)

    def prep(desc, ptrs=None, ws_bytes=need):
        p = ptrs or [fake] * 12  # q k v qcode qscale kcode kscale vcode vmean vscale vmean_scaled ws
        return lib.ab_fp8_prepare(ctypes.byref(desc), *p[:12], ws_bytes, None)

    assert prep(_desc(dtype=ab.AB_F32).c()) == -5
    assert prep(_desc(d=96).c()) == -2
    for i in range(12):
        p = [fake] * 12
        p[i] = None
        assert prep(cd, p) == -1, i
    for i in (0, 1, 2, 3, 5, 7, 10, 11):  # the 16-byte aligned operands
        p = [fake] * 12
        p[i] = odd
        assert prep(cd, p) == -2, i
    assert prep(cd, ws_bytes=need - 1) == -6
    assert b"workspace" in lib.ab_last_error()

    def attn(desc, ptrs=None):
        p = ptrs or [fake] * 12  # qcode qscale kcode kscale vcode vscale vmean_scaled idx weights counts out lse
        return lib.ab_attn_fwd_fp8(ctypes.byref(desc), *p, None)

    assert attn(_desc(dtype=ab.AB_F32).c()) == -5
    assert attn(_desc(d=64).c()) == -3
    assert attn(_desc(q_block=64).c()) == -3
    assert b"d = 128" in lib.ab_last_error()
    for i in range(11):  # every pointer but lse is required
        p = [fake] * 12
        p[i] = None
        assert attn(cd, p) == -1, i
    for i in (0, 2, 4, 6, 10):
        p = [fake] * 12
        p[i] = odd
        assert attn(cd, p) == -2, i


def test_intra_lists_validation():
    """INTRA pattern lists: layer and neighbourhood-size checks, NULL outputs."""
    lib = _lib()
    cd = _desc().c()
    fake = ctypes.c_void_p(256)
    assert lib.ab_intra_lists(ctypes.byref(cd), 2, 0, fake, fake, fake, None, None) == -3
    assert lib.ab_intra_lists(ctypes.byref(cd), -1, 0, fake, fake, fake, None, None) == -3
    for L in (64, 192, -128, (1 << 30) + 128):  # below q_block, not a multiple of it, negative, too large
        assert lib.ab_intra_lists(ctypes.byref(cd), 0, L, fake, fake, fake, fake, None) == -3, L
    assert b"partition_tokens" in lib.ab_last_error()
    assert lib.ab_intra_lists(ctypes.byref(cd), 1, 2048, None, fake, fake, None, None) == -1
    assert lib.ab_intra_lists(ctypes.byref(cd), 1, 0, fake, fake, None, fake, None) == -1
    assert lib.ab_intra_lists(ctypes.byref(_desc(q_block=32).c()), 0, 0, fake, fake, fake, None, None) == -3


def test_attn_fwd_ordered_validation():
    lib = _lib()
    cd = _desc().c()
    fake = ctypes.c_void_p(256)
    args = [fake] * 8  # q k v idx weights counts row_order out
    for i in range(8):
        a = list(args)
        a[i] = None
        assert lib.ab_attn_fwd_ordered(ctypes.byref(cd), *a, None, None) == -1, i
    a = list(args)
    a[0] = ctypes.c_void_p(256 + 8)
    assert lib.ab_attn_fwd_ordered(ctypes.byref(cd), *a, None, None) == -2
    assert lib.ab_attn_fwd_ordered(ctypes.byref(_desc(d=96).c()), *args, None, None) == -2


def test_score_noalloc_host_validation():
    """ab_score_noalloc checks its arguments on the host: NULL pointers, a bad
    descriptor, and a head that needs more scratch than the library's fixed array
    (rejected before any device call, so this runs without a GPU)."""
    lib = ab.load_library()
    good = ab.Desc(1, 2, 1000, 128, ab.AB_BF16, 128, 32, 8).c()
    fake = ctypes.c_void_p(4096)
    assert lib.ab_score_noalloc(ctypes.byref(good), None, fake, fake, None) == -1
    bad = ab.Desc(1, 2, 1000, 96, ab.AB_BF16, 128, 32, 8).c()
    assert lib.ab_score_noalloc(ctypes.byref(bad), fake, fake, fake, None) == -2
    big = ab.Desc(1, 1, 1 << 20, 128, ab.AB_BF16, 128, 16, 8).c()
    assert lib.ab_score_noalloc(ctypes.byref(big), fake, fake, fake, None) == -6
    msg = lib.ab_last_error().decode()
    assert "allocation-free" in msg and str(256 << 20) in msg
