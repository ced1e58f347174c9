"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every entry point
include/llsa.h declares, and every validation error is returned before anything is enqueued.
Fake device pointers are never dereferenced: each call below fails validation first."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llsa.h")

abi = pytest.importorskip("hierarchical_top_sparse_amd._abi")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(abi._LIB_PATH):
        pytest.fail("libllsa.so is not built (python -m hierarchical_top_sparse_amd.build)")
    return abi.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int32_t|const char\*)\s+(llsa_\w+)\(", text, re.M)))


def test_header_declares_every_bound_symbol():
    assert _declared() == sorted(abi.exported_symbols())


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.llsa_abi_version() == abi.LLSA_ABI_VERSION == 5
    for code in range(8):
        assert L.llsa_status_str(code)
    assert L.llsa_status_str(99) == b"unknown status"


def _p(**kw):
    base = dict(batch=1, heads=2, height=64, width=64, levels=2)
    base.update(kw)
    return abi.Problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(height=256, width=256, levels=3, dtype=abi.LLSA_BF16), 0),
    (dict(height=128, width=256, levels=3), 0),
    (dict(width=48), 2),                    # not a power of two
    (dict(height=16, width=8), 2),          # fewer than 256 tokens
    (dict(height=2, width=256, levels=1), 2),   # a side shorter than a 4x4 tile
    (dict(height=4096, width=4096, levels=1), 2),  # more than 2^23 tokens
    (dict(levels=3), 2),                    # N % B^L != 0
    (dict(topk=33), 2),                     # above the 32 supported
    (dict(levels=2, topk=9, height=32, width=64), 2),  # K > N / B^L = 8
    (dict(topk=0), 2),
    (dict(enrich_levels=-1), 2),
    (dict(coarse_unit_weight=2), 2),
    (dict(enrich_levels=5, coarse_unit_weight=1), 0),   # clamped to the L - 1 coarse levels
    (dict(coarse_exclude_overlap=2), 2),
    (dict(coarse_exclude_overlap=1), 0),
    (dict(head_dim=128), 0),
    (dict(head_dim=128, dtype=abi.LLSA_BF16, height=256, width=256, levels=3), 0),
    (dict(head_dim=96), 4),
    (dict(head_dim=32), 4),
    (dict(block=256), 4),                   # a power of 4 but not implemented
    (dict(block=64, levels=1), 0),          # 8x8 tiles: 64 blocks of 64 tokens, K = 8
    (dict(block=64, levels=2), 2),          # N / 64^2 = 1 < K
    (dict(block=64, levels=1, topk=9), 4),  # 9 picks cover 36 16-token blocks (> 32)
    (dict(block=8), 2),                     # not a square tile
    (dict(levels=0), 2),
    (dict(levels=7), 2),
    (dict(enrich=2), 2),
    (dict(scale=-1.0), 2),
    (dict(dtype=5), 3),
    (dict(layout=7), 3),
    (dict(batch=0), 2),
])
def test_check_status(L, kw, status):
    p = _p(**kw)
    assert abi.llsa_check(p) == status, abi.llsa_last_error()
    if status:
        assert abi.llsa_last_error()


FAKE = 0x10000          # aligned, never dereferenced
MISALIGNED = 0x10008


def test_entry_points_reject_null_and_misaligned(L):
    p = ctypes.byref(_p().c())
    assert L.llsa_reorder(p, None, ctypes.c_void_p(FAKE), 0, None) == 1
    assert L.llsa_reorder(p, ctypes.c_void_p(MISALIGNED), ctypes.c_void_p(FAKE), 0, None) == 6
    assert L.llsa_reorder(p, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 0, None) == 2
    assert L.llsa_reorder(p, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 64), 3, None) == 2
    assert L.llsa_pool(p, None, None, None, None, None, None, None) == 1
    null6 = (ctypes.c_void_p * 6)()
    assert L.llsa_select(p, null6, null6, null6, 2, 1, None) == 1
    assert L.llsa_select(p, null6, null6, null6, 3, 1, None) == 2
    assert L.llsa_attn_fwd(p, None, None, None, null6, null6, null6, None, None, None) == 1
    bf = ctypes.byref(_p(dtype=abi.LLSA_F32).c())
    assert L.llsa_attn_bwd(bf, *([ctypes.c_void_p(FAKE)] * 5), null6, null6, null6, null6,
                           null6, *([ctypes.c_void_p(FAKE)] * 4), 1 << 30, None) == 4


def test_workspace_queries(L):
    f, b = abi.llsa_workspace_bytes(_p(dtype=abi.LLSA_BF16))
    assert f == 0 and b > 0
    a256 = lambda x: (x + 255) // 256 * 256
    # up to 64 tiles of 4096 entries (the radix path): each tile's sorted rows and its column
    # bounds (cols + 1); one tile needs none
    assert abi.llsa_index_transpose_workspace(6, 4096, 4096, 8) == (
        a256(4 * 6 * 8 * 4096) + a256(4 * 6 * 8 * 4097))
    assert abi.llsa_index_transpose_workspace(3, 256, 256, 8) == 0
    # more tiles (the bitonic path): two code buffers + per-run column bounds (cols + 1) and
    # run starts (cols): 80 tiles of 4096 merge into 20 runs of 16384 (at most 32 runs)
    assert abi.llsa_index_transpose_workspace(1, 40960, 500, 8) == (
        2 * a256(4 * 40960 * 8) + a256(4 * 20 * 501) + a256(4 * 20 * 500))
    out = ctypes.c_size_t()
    assert L.llsa_index_transpose_workspace(1, 0, 4, 8, ctypes.byref(out)) == 2
    # the bitonic path's 32-bit codes: (cols + 1) * 2^ceil(log2 rows) <= 2^32
    assert L.llsa_index_transpose_workspace(1, 1 << 20, 1 << 13, 8, ctypes.byref(out)) == 2
    # the radix path has no such limit
    assert L.llsa_index_transpose_workspace(1, 1 << 15, 1 << 18, 8, ctypes.byref(out)) == 0
    # workspace too small / missing (two tiles need one), NULL pointers
    fake = ctypes.c_void_p(FAKE)
    assert L.llsa_index_transpose(1, 1024, 16, 8, fake, fake, fake, None, 0, None) == 5
    assert L.llsa_index_transpose(1, 1024, 16, 8, fake, fake, fake, fake, 8, None) == 5
    assert L.llsa_index_transpose(1, 16, 16, 8, None, fake, fake, fake, 4096, None) == 1
    # every level at once: the sum of the radix levels' needs, NULL pointers refused
    p = _p(height=256, width=256, levels=3, dtype=abi.LLSA_BF16)
    assert abi.llsa_index_transpose_levels_workspace(p) == (
        a256(4 * 2 * 8 * 4096) + a256(4 * 2 * 8 * 4097))
    lv = (ctypes.c_void_p * 6)(FAKE, FAKE, None)
    full = (ctypes.c_void_p * 6)(FAKE, FAKE, FAKE)
    assert L.llsa_index_transpose_levels(ctypes.byref(p.c()), full, full, lv, fake, 1 << 30,
                                         None) == 1
    assert L.llsa_index_transpose_levels(ctypes.byref(p.c()), full, full, full, None, 0,
                                         None) == 5


def test_backward_rejects_too_many_coarse_keys(L):
    p = _p(height=1024, width=1024, levels=4, topk=16, dtype=abi.LLSA_BF16)
    assert abi.llsa_check(p) == 0
    fake = ctypes.c_void_p(FAKE)
    null6 = (ctypes.c_void_p * 6)()
    st = L.llsa_attn_bwd(ctypes.byref(p.c()), *([fake] * 5), null6, null6, null6, null6, null6,
                         *([fake] * 4), 1 << 30, None)
    assert st == 4 and b"coarse" in L.llsa_last_error()


def test_dense_baseline_validation(L):
    f = ctypes.c_void_p(FAKE)
    # n must be a multiple of 128, head_dim 64, pointers present
    assert L.llsa_dense_attn_fwd(2, 1000, 64, 0.0, f, f, f, f, f, None) == 2
    assert L.llsa_dense_attn_fwd(2, 1024, 128, 0.0, f, f, f, f, f, None) == 4
    assert L.llsa_dense_attn_fwd(0, 1024, 64, 0.0, f, f, f, f, f, None) == 2
    assert L.llsa_dense_attn_fwd(2, 1024, 64, -1.0, f, f, f, f, f, None) == 2
    assert L.llsa_dense_attn_fwd(2, 1024, 64, 0.0, None, f, f, f, f, None) == 1
    assert L.llsa_dense_attn_fwd(2, 1024, 64, 0.0, f, f, f, f, ctypes.c_void_p(MISALIGNED),
                                 None) == 6
    assert L.llsa_dense_attn_bwd(2, 1024, 64, 0.0, *([f] * 8), None, None) == 1
    assert L.llsa_dense_attn_bwd(2, 64, 64, 0.0, *([f] * 9), None) == 2


def test_mask_comparator_validation(L):
    f = ctypes.c_void_p(FAKE)
    one = _p(height=128, width=128, levels=1, topk=32, dtype=abi.LLSA_BF16)
    assert abi.llsa_check(one) == 0
    # coarse keys (levels 2 with enrich) are not supported by the mask-based backward
    two = _p(height=128, width=128, levels=2, topk=8, dtype=abi.LLSA_BF16)
    assert L.llsa_block_mask(ctypes.byref(two.c()), f, f, None) == 4
    assert L.llsa_attn_bwd_masked(ctypes.byref(two.c()), *([f] * 11), 1 << 30, None) == 4
    # fp32 is not supported; missing / misaligned pointers; workspace too small
    f32 = _p(height=128, width=128, levels=1, topk=32, dtype=abi.LLSA_F32)
    assert L.llsa_block_mask(ctypes.byref(f32.c()), f, f, None) == 4
    assert L.llsa_block_mask(ctypes.byref(one.c()), None, f, None) == 1
    assert L.llsa_block_mask(ctypes.byref(one.c()), f, ctypes.c_void_p(MISALIGNED), None) == 6
    assert L.llsa_attn_bwd_masked(ctypes.byref(one.c()), *([f] * 6), None, *([f] * 4), 1 << 30,
                                  None) == 1
    assert L.llsa_attn_bwd_masked(ctypes.byref(one.c()), *([f] * 11), 4, None) == 5
    # a mask over 2^34 bytes: 1024x1024 pixels, n_1 = 65536, 8 heads -> 2^35
    big = _p(batch=1, heads=8, height=1024, width=1024, levels=1, topk=8, dtype=abi.LLSA_BF16)
    assert abi.llsa_check(big) == 0
    assert L.llsa_block_mask(ctypes.byref(big.c()), f, f, None) == 2


def test_block64_pool_needs_level_one(L):
    """With 8x8 blocks level 2 is pooled from level 1, so a tensor's level 1 must be stored."""
    f = ctypes.c_void_p(FAKE)
    p = _p(height=256, width=256, levels=2, dtype=abi.LLSA_BF16, block=64)
    assert abi.llsa_check(p) == 0
    lv_missing = (ctypes.c_void_p * 6)(None, FAKE)
    assert L.llsa_pool(ctypes.byref(p.c()), None, f, None, None, lv_missing, None, None) == 1
    assert b"level 1" in L.llsa_last_error()
    lv_bad = (ctypes.c_void_p * 6)(MISALIGNED, FAKE)
    assert L.llsa_pool(ctypes.byref(p.c()), None, f, None, None, lv_bad, None, None) == 6


def test_backward_rejects_more_than_2_19_tokens(L):
    """The level-1 transpose packs (key block, query block) in 32 bits: N <= 2^19 per head."""
    f = ctypes.c_void_p(FAKE)
    null6 = (ctypes.c_void_p * 6)()
    big = _p(height=1024, width=1024, levels=3, dtype=abi.LLSA_BF16, enrich=0)
    assert abi.llsa_check(big) == 0
    st = L.llsa_attn_bwd(ctypes.byref(big.c()), *([f] * 5), null6, null6, null6, null6, null6,
                         *([f] * 4), 1 << 30, None)
    assert st == 4 and b"2^19" in L.llsa_last_error()


def test_calibration_validation(L):
    f = ctypes.c_void_p(FAKE)
    assert L.llsa_calib_copy(f, ctypes.c_void_p(FAKE + 4096), 0, None) == 2
    assert L.llsa_calib_copy(f, ctypes.c_void_p(FAKE + 4096), 24, None) == 2
    assert L.llsa_calib_copy(None, f, 64, None) == 1
    assert L.llsa_calib_copy(f, f, 64, None) == 2
    assert L.llsa_calib_mfma(f, 0, 16, None) == 2
    assert L.llsa_calib_mfma(f, 4, 0, None) == 2
    assert L.llsa_calib_mfma(None, 4, 16, None) == 1


def test_pool_select_validation(L):
    """Q and K are required with all their levels (the selection reads them); V is optional."""
    f = ctypes.c_void_p(FAKE)
    p = ctypes.byref(_p(height=64, width=64, levels=2).c())
    lv2 = (ctypes.c_void_p * 6)(FAKE, FAKE)
    lv_missing1 = (ctypes.c_void_p * 6)(None, FAKE)
    assert L.llsa_pool_select(p, None, f, f, lv2, lv2, lv2, lv2, None) == 1
    assert L.llsa_pool_select(p, f, None, f, lv2, lv2, lv2, lv2, None) == 1
    assert L.llsa_pool_select(p, f, f, None, lv2, None, None, lv2, None) == 1
    assert L.llsa_pool_select(p, f, f, None, lv_missing1, lv2, None, lv2, None) == 1
    assert b"q level 1" in L.llsa_last_error()
    assert L.llsa_pool_select(p, f, f, None, lv2, lv2, None, lv_missing1, None) == 1
    assert L.llsa_pool_select(p, ctypes.c_void_p(MISALIGNED), f, None, lv2, lv2, None, lv2,
                              None) == 6
    lv_bad = (ctypes.c_void_p * 6)(FAKE, MISALIGNED)
    assert L.llsa_pool_select(p, f, f, f, lv2, lv2, lv_bad, lv2, None) == 6
    bad = ctypes.byref(_p(height=64, width=64, levels=2, topk=0).c())
    assert L.llsa_pool_select(bad, f, f, f, lv2, lv2, lv2, lv2, None) == 2


hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

_INT = st.one_of(st.integers(-4, 70), st.integers(-2 ** 31, 2 ** 31 - 1))
_SIDE = st.one_of(st.sampled_from([0, 1, 2, 4, 8, 16, 24, 64, 128, 256, 1024, 4096, 8192, -16]),
                  st.integers(-2 ** 31, 2 ** 31 - 1))


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(batch=_INT, heads=_INT, height=_SIDE, width=_SIDE, levels=_INT, topk=_INT, enrich=_INT,
       head_dim=st.sampled_from([0, 32, 64, 128, -64]),
       block=st.sampled_from([0, 1, 4, 8, 16, 32, 64, 256, -16]),
       scale=st.floats(width=32), dtype=_INT, layout=_INT, enrich_levels=_INT,
       unit_weight=_INT, exclude=_INT)
def test_check_never_accepts_what_the_kernels_cannot_run(L, batch, heads, height, width, levels,
                                                         topk, enrich, head_dim, block, scale,
                                                         dtype, layout, enrich_levels,
                                                         unit_weight, exclude):
    """Any problem: llsa_check returns a defined status without faulting, and every problem it
    accepts satisfies the limits the kernels rely on and has a sane backward workspace."""
    p = abi.Problem(batch=batch, heads=heads, height=height, width=width, levels=levels,
                    topk=topk, enrich=enrich, head_dim=head_dim, block=block, scale=scale,
                    dtype=dtype, layout=layout, enrich_levels=enrich_levels,
                    coarse_unit_weight=unit_weight, coarse_exclude_overlap=exclude)
    status = abi.llsa_check(p)
    assert 0 <= status <= 7
    if status:
        assert abi.llsa_last_error()
        return
    n = height * width
    assert batch >= 1 and heads >= 1 and head_dim in (64, 128) and block in (16, 64)
    assert 256 <= n <= 1 << 23 and batch * heads * n < 1 << 31
    assert n % block ** levels == 0 and 1 <= topk <= min(32, n // block ** levels)
    assert topk * block // 16 <= 32
    assert dtype in (abi.LLSA_F32, abi.LLSA_BF16) and scale >= 0
    f, b = abi.llsa_workspace_bytes(p)
    assert f == 0 and 0 < b < 1 << 44


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(batch=st.integers(1, 8), heads=st.integers(1, 16),
       height=st.sampled_from([4, 8, 16, 64, 256, 1024, 2048]),
       width=st.sampled_from([4, 8, 16, 64, 256, 1024, 2048]), levels=st.integers(1, 4),
       topk=st.integers(1, 33), enrich=st.integers(0, 1), block=st.sampled_from([16, 64]),
       dtype=st.integers(0, 1), layout=st.integers(0, 1), enrich_levels=st.integers(0, 4),
       unit_weight=st.integers(0, 1), exclude=st.integers(0, 1))
def test_check_and_workspace_on_nearly_valid_problems(L, batch, heads, height, width, levels,
                                                      topk, enrich, block, dtype, layout,
                                                      enrich_levels, unit_weight, exclude):
    """Mostly valid problems: accepted exactly when the documented limits hold, and then the
    backward workspace covers D (4 bytes per token) and grows with the problem."""
    p = abi.Problem(batch=batch, heads=heads, height=height, width=width, levels=levels,
                    topk=topk, enrich=enrich, block=block, dtype=dtype, layout=layout,
                    enrich_levels=enrich_levels, coarse_unit_weight=unit_weight,
                    coarse_exclude_overlap=exclude)
    n = height * width
    ok = (256 <= n <= 1 << 23 and n % block ** levels == 0
          and topk <= min(32, n // block ** levels) and topk * block // 16 <= 32
          and batch * heads * n < 1 << 31)
    status = abi.llsa_check(p)
    assert (status == 0) == ok, (status, abi.llsa_last_error())
    if ok:
        f, b = abi.llsa_workspace_bytes(p)
        assert f == 0 and b >= 4 * batch * heads * n


def test_head128_limits(L):
    """128-channel heads: the attention runs in bf16 only, the mask-based comparator has 64
    channels only (both refused before anything is enqueued)."""
    f = ctypes.c_void_p(FAKE)
    lv = (ctypes.c_void_p * 6)(FAKE, FAKE)
    f32 = _p(head_dim=128, dtype=abi.LLSA_F32)
    assert abi.llsa_check(f32) == 0
    assert L.llsa_attn_fwd(ctypes.byref(f32.c()), f, f, f, lv, lv, lv, f, f, None) == 4
    assert b"bf16" in L.llsa_last_error()
    m = _p(head_dim=128, height=128, width=128, levels=1, topk=32, dtype=abi.LLSA_BF16)
    assert L.llsa_block_mask(ctypes.byref(m.c()), f, f, None) == 4
    # the backward workspace grows with the head width
    p64 = _p(height=256, width=256, levels=3, dtype=abi.LLSA_BF16)
    p128 = _p(height=256, width=256, levels=3, dtype=abi.LLSA_BF16, head_dim=128)
    assert abi.llsa_workspace_bytes(p128)[1] > abi.llsa_workspace_bytes(p64)[1]
