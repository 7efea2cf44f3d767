"""The C ABI library: exported symbols and host-side validation (no GPU needed).

Only calls that return before any device work are made here.
"""
import ctypes
import os
import re

import pytest

import dynamic_sparse_attention_index_amd as vs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vs_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vs_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vs.LIB_PATH):
        pytest.skip("library not built")
    return vs.lib()


def test_header_symbols_exported(L):
    names = _declared()
    assert set(names) == set(vs.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_debug_build_exports_and_reports(L):
    """The bounds-checked build exports the same symbols and says so; the
    release build reports no checks and no count without touching a device."""
    assert L.vs_debug_bounds_enabled() == 0
    n = ctypes.c_int32(7)
    assert L.vs_debug_bounds_count(ctypes.byref(n), 1, None) == 0 and n.value == 0
    assert L.vs_debug_bounds_count(None, 0, None) == vs.VS_ERR_ARG
    if not os.path.exists(vs.DEBUG_LIB_PATH):
        pytest.skip("debug library not built")
    with vs.use_library(vs.DEBUG_LIB_PATH) as D:
        for name in _declared():
            assert hasattr(D, name), name
        assert D.vs_debug_bounds_enabled() == 1
        assert vs.lib() is D
    assert vs.lib() is L


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert vs.status_string(code) and vs.status_string(code) != "unknown status"
    assert vs.status_string(123) == "unknown status"


def _fake_tensor(addr, H, N, D, dtype=vs.VS_BF16):
    return vs.VsTensor(addr, dtype, H, N, D, N * D, D)


def _mask(L, Hq=4, Hkv=2, N=1024, kind="contig", P=1, cap=100):
    lay = vs.layout(kind, P, N)
    nbytes = L.vs_mask_bytes(Hq, Hkv, lay, cap)
    assert nbytes > 0
    m = vs.VsMask()
    fake = 0x10000000  # never dereferenced: vs_mask_init only computes addresses
    assert L.vs_mask_init(ctypes.byref(m), fake, nbytes, Hq, Hkv, lay, cap) == 0
    return m, lay, nbytes, fake


def test_mask_init_layout(L):
    m, lay, nbytes, base = _mask(L)
    ptrs = [m.tile_ptr, m.tile_col, m.csc_ptr, m.csc_row, m.vloc, m.vloc_cnt, m.vcum, m.vert_end,
            m.slash_bits, m.n_active, m.status]
    assert all(base <= p < base + nbytes and (p - base) % 256 == 0 for p in ptrs)
    assert ptrs == sorted(ptrs) and len(set(ptrs)) == len(ptrs)
    assert (m.QB, m.KB, m.T, m.W) == (16, 16, 16, 1)
    m2 = vs.VsMask()
    assert L.vs_mask_init(ctypes.byref(m2), base, nbytes - 1, 4, 2, lay, 100) == vs.VS_ERR_WORKSPACE


def test_layout_validation(L):
    assert L.vs_mask_bytes(4, 2, vs.layout("striped", 3, 64 * 10), 10) == 0      # N % (64 P) != 0
    assert L.vs_mask_bytes(4, 2, vs.layout("zigzag", 2, 64 * 6), 10) == 0        # N % (128 P) != 0
    assert L.vs_mask_bytes(4, 2, vs.layout("zigzag", 2, 64 * 8), 10) > 0
    assert L.vs_mask_bytes(4, 2, vs.layout("striped1", 4, 64 * 8), 10) > 0
    assert L.vs_mask_bytes(4, 2, vs.layout("striped1", 4, 64 * 6), 10) == 0      # N % (64 P) != 0
    assert L.vs_mask_bytes(4, 2, vs.layout("striped1", 33, 64 * 33), 10) == 0    # one-position stripes: P <= 32
    m = vs.VsMask()
    assert L.vs_mask_init(ctypes.byref(m), 0x10000000, 1 << 20, 3, 2, vs.layout("contig", 1, 1024), 10) \
        == vs.VS_ERR_ARG                                                           # Hq % Hkv != 0


def test_fwd_validation_before_device_work(L):
    m, lay, _, _ = _mask(L)
    m.rank = 0
    m.src = 0
    q = _fake_tensor(0x20000000, 4, 1024, 128)
    k = _fake_tensor(0x30000000, 2, 1024, 128)
    o, lse = ctypes.c_void_p(0x40000000), ctypes.c_void_p(0x50000000)
    null = _fake_tensor(None, 4, 1024, 128)
    assert L.vs_attn_fwd(null, k, k, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_ARG
    bad_n = _fake_tensor(0x20000000, 4, 1000, 128)
    assert L.vs_attn_fwd(bad_n, k, k, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_ARG
    d96q, d96k = _fake_tensor(0x20000000, 4, 1024, 96), _fake_tensor(0x30000000, 2, 1024, 96)
    assert L.vs_attn_fwd(d96q, d96k, d96k, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_UNSUPPORTED
    mis = _fake_tensor(0x20000002, 4, 1024, 128)
    assert L.vs_attn_fwd(mis, k, k, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_UNSUPPORTED
    f32k = _fake_tensor(0x30000000, 2, 1024, 128, vs.VS_F32)
    assert L.vs_attn_fwd(q, f32k, f32k, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_ARG
    assert L.vs_attn_fwd(q, k, k, ctypes.byref(m), -1.0, o, lse, 0, None) == vs.VS_ERR_ARG
    assert L.vs_attn_fwd(q, k, k, ctypes.byref(m), 0.1, o, lse, 2, None) == vs.VS_ERR_ARG
    assert L.vs_attn_fwd(q, k, k, ctypes.byref(m), 0.1, None, lse, 0, None) == vs.VS_ERR_ARG
    m.rank = -1                                            # mask never built
    assert L.vs_attn_fwd(q, k, k, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_ARG


def test_stripe1_attention_validation(L):
    """One-position stripes run on the head-dim-128 bf16/fp16 kernels only; the
    head-pair and resident-ring forms refuse the layout before device work."""
    m, lay, _, _ = _mask(L, kind="striped1", P=4, N=1024)
    m.rank = 0
    m.src = 0
    q64 = _fake_tensor(0x20000000, 4, 256, 64)
    k64 = _fake_tensor(0x30000000, 2, 256, 64)
    o, lse, st = ctypes.c_void_p(0x40000000), ctypes.c_void_p(0x50000000), ctypes.c_void_p(0x60000000)
    assert L.vs_attn_fwd(q64, k64, k64, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_UNSUPPORTED
    q = _fake_tensor(0x20000000, 4, 256, 128)
    k = _fake_tensor(0x30000000, 2, 256, 128)
    assert L.vs_attn_fwd_packed(q, k, k, ctypes.byref(m), 0.1, o, lse, 0, st, None) == vs.VS_ERR_UNSUPPORTED
    k_all = _fake_tensor(0x30000000, 2, 1024, 128)
    assert L.vs_attn_fwd_ring(q, k_all, k_all, ctypes.byref(m), 1, 0.1, o, lse, 0, None) == vs.VS_ERR_UNSUPPORTED


def test_sequence_beyond_the_lds_bitmap_refused(L):
    """2^20 tokens is the longest sequence the head-dim-128 attention kernels
    take (a head's slash bitmap, 512 words, lives in LDS); one block more is
    refused before device work."""
    N = (1 << 20) + 64
    m, lay, _, _ = _mask(L, Hq=2, Hkv=1, N=N)
    m.rank = 0
    m.src = 0
    q = _fake_tensor(0x20000000, 2, N, 128)
    k = _fake_tensor(0x30000000, 1, N, 128)
    o, lse = ctypes.c_void_p(0x40000000), ctypes.c_void_p(0x50000000)
    assert L.vs_attn_fwd(q, k, k, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_UNSUPPORTED
    p = ctypes.c_void_p(0x60000000)
    assert L.vs_attn_bwd(q, k, k, q, p, p, ctypes.byref(m), 0.1, p, p, p, None) == vs.VS_ERR_UNSUPPORTED


def test_block_mask_and_index_validation(L):
    m, lay, _, _ = _mask(L, kind="striped", P=4, N=1024)
    p = ctypes.c_void_p(0x60000000)
    assert L.vs_block_mask(p, p, 1024, p, p, 16, 4, 0, ctypes.byref(m), None) == vs.VS_ERR_ARG   # rank >= P
    assert L.vs_block_mask(p, p, 1024, p, p, 16, 0, -1, ctypes.byref(m), None) == vs.VS_ERR_ARG
    assert L.vs_block_mask(None, p, 1024, p, p, 16, 0, 0, ctypes.byref(m), None) == vs.VS_ERR_ARG
    q = _fake_tensor(0x20000000, 16, 64, 128)
    k = _fake_tensor(0x30000000, 2, 4096, 128)
    lay = vs.layout("contig", 1, 4096)
    ws = L.vs_index_workspace_size(16, 2, 4096, 128, 64)
    assert ws > 0
    args = [p] * 6
    assert L.vs_index_build(q, k, lay, 0.1, 0.9, *args, p, ws - 1, None) == vs.VS_ERR_WORKSPACE
    q65 = _fake_tensor(0x20000000, 16, 65, 128)
    assert L.vs_index_build(q65, k, lay, 0.1, 0.9, *args, p, ws, None) == vs.VS_ERR_UNSUPPORTED
    k3 = _fake_tensor(0x30000000, 3, 4096, 128)
    assert L.vs_index_build(q, k3, lay, 0.1, 0.9, *args, p, ws, None) == vs.VS_ERR_ARG
    kshort = _fake_tensor(0x30000000, 2, 2048, 128)
    assert L.vs_index_build(q, kshort, lay, 0.1, 0.9, *args, p, ws, None) == vs.VS_ERR_ARG
    # one-position stripes: the index takes the keys in global order
    s1 = vs.layout("striped1", 4, 4096)
    assert L.vs_index_build(q, k, s1, 0.1, 0.9, *args, p, ws, None) == vs.VS_ERR_UNSUPPORTED
    k_local = _fake_tensor(0x30000000, 2, 1024, 128)
    assert L.vs_index_rank_stats(q, k_local, s1, 0, 0.1, p, p, ws, None) == vs.VS_ERR_UNSUPPORTED


def test_rank_index_validation(L):
    """Per-rank index calls: host checks return before any device work."""
    p = ctypes.c_void_p(0x60000000)
    q = _fake_tensor(0x20000000, 16, 64, 128)
    lay = vs.layout("striped", 4, 4096)
    k_local = _fake_tensor(0x30000000, 2, 1024, 128)
    ws = L.vs_index_workspace_size(16, 2, 4096, 128, 64)
    assert L.vs_index_rank_stats(q, k_local, lay, 4, 0.1, p, p, ws, None) == vs.VS_ERR_ARG      # rank >= P
    assert L.vs_index_rank_stats(q, k_local, lay, -1, 0.1, p, p, ws, None) == vs.VS_ERR_ARG
    assert L.vs_index_rank_stats(q, k_local, lay, 0, 0.1, None, p, ws, None) == vs.VS_ERR_ARG   # no stats
    assert L.vs_index_rank_stats(q, k_local, lay, 0, 0.1, p, p, ws - 1, None) == vs.VS_ERR_WORKSPACE
    k_global = _fake_tensor(0x30000000, 2, 4096, 128)                                           # not a shard
    assert L.vs_index_rank_stats(q, k_global, lay, 0, 0.1, p, p, ws, None) == vs.VS_ERR_ARG
    assert L.vs_index_rank_mass(q, k_local, lay, 1, 0.1, None, p, p, p, ws, None) == vs.VS_ERR_ARG
    assert L.vs_index_rank_mass(q, k_local, lay, 1, 0.0, p, p, p, p, ws, None) == vs.VS_ERR_ARG  # scale
    for bad in (float("nan"), float("inf"), -0.5):
        assert L.vs_index_rank_mass(q, k_local, lay, 1, bad, p, p, p, p, ws, None) == vs.VS_ERR_ARG
    sws = L.vs_index_select_workspace_size(16, 4096)
    assert sws > 0 and L.vs_index_select_workspace_size(0, 4096) == 0
    assert L.vs_index_select(p, p, 16, 4096, 0.9, p, p, p, None, p, sws, None) == vs.VS_ERR_ARG
    assert L.vs_index_select(p, p, 0, 4096, 0.9, p, p, p, p, p, sws, None) == vs.VS_ERR_ARG
    assert L.vs_index_select(p, p, 16, 4096, 0.9, p, p, p, p, None, sws, None) == vs.VS_ERR_ARG
    assert L.vs_index_select(p, p, 16, 4000, 0.9, p, p, p, p, p, sws, None) == vs.VS_ERR_UNSUPPORTED
    assert L.vs_index_select(p, p, 16, 4096, 0.9, p, p, p, p, p, sws - 1, None) == vs.VS_ERR_WORKSPACE
    B = L.vs_index_select_budget
    assert B(p, p, 16, 4096, 3, 0.9, 1, 1, p, p, p, p, p, sws, None) == vs.VS_ERR_ARG            # unknown budget
    assert B(p, p, 16, 4096, -1, 0.9, 1, 1, p, p, p, p, p, sws, None) == vs.VS_ERR_ARG
    assert B(p, p, 16, 4096, vs.VS_BUDGET_TOP_K, 0.9, 8, 8, p, None, p, p, p, sws, None) == vs.VS_ERR_ARG
    assert B(p, p, 16, 4000, vs.VS_BUDGET_TOP_K, 0.9, 8, 8, p, p, p, p, p, sws, None) == vs.VS_ERR_UNSUPPORTED
    assert B(p, p, 16, 4096, vs.VS_BUDGET_JOINT_TOP_P, float("nan"), 0, 0, p, p, p, p, p, sws, None) == vs.VS_ERR_ARG
    assert B(p, p, 16, 4096, vs.VS_BUDGET_JOINT_TOP_P, 0.9, 0, 0, p, p, p, p, p, sws - 1, None) == vs.VS_ERR_WORKSPACE


def test_bwd_and_merge_validation(L):
    m, lay, _, _ = _mask(L)
    m.rank = m.src = 0
    q = _fake_tensor(0x20000000, 4, 1024, 128)
    k = _fake_tensor(0x30000000, 2, 1024, 128)
    p = ctypes.c_void_p(0x40000000)
    dq_mis = ctypes.c_void_p(0x40000004)
    assert L.vs_attn_bwd(q, k, k, q, p, p, ctypes.byref(m), 0.1, dq_mis, p, p, None) == vs.VS_ERR_UNSUPPORTED
    assert L.vs_attn_bwd(q, k, k, q, None, p, ctypes.byref(m), 0.1, p, p, p, None) == vs.VS_ERR_ARG
    assert L.vs_merge_lse(p, p, p, p, 4, 1024, 96, None) == vs.VS_ERR_UNSUPPORTED
    assert L.vs_merge_lse(None, p, p, p, 4, 1024, 128, None) == vs.VS_ERR_ARG
    assert L.vs_merge_lse(p, p, p, p, 4, 0, 128, None) == vs.VS_OK          # nothing to do


def test_dense_buffer_arguments_must_be_contiguous():
    """The ABI's plain float* arrays are dense; the binding refuses a strided view
    before anything is launched."""
    import torch
    with pytest.raises(vs.VsError):
        vs._cptr(torch.zeros(4, 8)[:, :4])
    assert vs._cptr(torch.zeros(4, 8)).value is not None


def test_f16_validation_before_device_work(L):
    """fp16 operands: attention at D = 128 only, never mixed with bf16, never
    for the index; the conversion call checks its buffers on the host."""
    m, lay, _, _ = _mask(L)
    m.rank = m.src = 0
    q16 = _fake_tensor(0x20000000, 4, 1024, 128, vs.VS_F16)
    k16 = _fake_tensor(0x30000000, 2, 1024, 128, vs.VS_F16)
    kb = _fake_tensor(0x30000000, 2, 1024, 128)
    o, lse = ctypes.c_void_p(0x40000000), ctypes.c_void_p(0x50000000)
    assert L.vs_attn_fwd(q16, kb, kb, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_ARG
    q64 = _fake_tensor(0x20000000, 4, 1024, 64, vs.VS_F16)
    k64 = _fake_tensor(0x30000000, 2, 1024, 64, vs.VS_F16)
    assert L.vs_attn_fwd(q64, k64, k64, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_UNSUPPORTED
    p = ctypes.c_void_p(0x40000000)
    assert L.vs_attn_bwd(q16, k16, k16, _fake_tensor(0x20000000, 4, 1024, 128), p, p, ctypes.byref(m), 0.1,
                         p, p, p, None) == vs.VS_ERR_ARG
    assert L.vs_attn_bwd_prep(p, q64, p, None) == vs.VS_ERR_UNSUPPORTED
    bad = _fake_tensor(0x20000000, 4, 1024, 128, 7)
    assert L.vs_attn_fwd(bad, bad, bad, ctypes.byref(m), 0.1, o, lse, 0, None) == vs.VS_ERR_ARG
    # the index has no fp16 kernels
    ws = ctypes.c_void_p(0x60000000)
    ql = _fake_tensor(0x20000000, 4, 64, 128, vs.VS_F16)
    assert L.vs_index_build(ql, _fake_tensor(0x30000000, 2, 1024, 128, vs.VS_F16), vs.layout("contig", 1, 1024),
                            0.1, 0.9, p, p, p, p, p, p, ws, 1 << 30, None) == vs.VS_ERR_UNSUPPORTED
    a, b, st = ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x30000000), ctypes.c_void_p(0x40000000)
    assert L.vs_convert_f16(None, b, 64, st, None) == vs.VS_ERR_ARG
    assert L.vs_convert_f16(a, b, 64, None, None) == vs.VS_ERR_ARG
    assert L.vs_convert_f16(a, b, -8, st, None) == vs.VS_ERR_ARG
    assert L.vs_convert_f16(a, b, 12, st, None) == vs.VS_ERR_UNSUPPORTED
    assert L.vs_convert_f16(ctypes.c_void_p(0x20000002), b, 64, st, None) == vs.VS_ERR_UNSUPPORTED
    assert L.vs_convert_f16(a, b, 0, st, None) == vs.VS_OK                 # nothing to do


def test_group_packed_and_fused_prep_validation(L):
    """Host checks of the per-kv-head selection, the head-pair forward and the
    fused delta / fp16 dO copy; nothing reaches the device."""
    p = ctypes.c_void_p(0x40000000)
    ws = ctypes.c_void_p(0x60000000)
    # per-kv-head selection
    assert L.vs_index_select_group_workspace_size(8, 3, 1024) == 0          # 8 % 3 != 0
    wsz = L.vs_index_select_group_workspace_size(8, 2, 1024)
    assert wsz > 0
    assert L.vs_index_select_group(p, p, 8, 3, 1024, 0.9, p, p, p, p, ws, wsz, None) == vs.VS_ERR_ARG
    assert L.vs_index_select_group(None, p, 8, 2, 1024, 0.9, p, p, p, p, ws, wsz, None) == vs.VS_ERR_ARG
    assert L.vs_index_select_group(p, p, 8, 2, 1000, 0.9, p, p, p, p, ws, wsz, None) == vs.VS_ERR_UNSUPPORTED
    assert L.vs_index_select_group(p, p, 8, 2, 1024, 0.9, p, p, p, p, ws, wsz - 1, None) == vs.VS_ERR_WORKSPACE
    # head-pair forward
    m, lay, _, _ = _mask(L, Hq=4, Hkv=2)
    m.rank = m.src = 0
    q = _fake_tensor(0x20000000, 4, 1024, 128, vs.VS_F16)
    k = _fake_tensor(0x30000000, 2, 1024, 128, vs.VS_F16)
    o, lse, st = ctypes.c_void_p(0x40000000), ctypes.c_void_p(0x50000000), ctypes.c_void_p(0x58000000)
    assert L.vs_attn_fwd_packed(q, k, k, ctypes.byref(m), 0.1, o, lse, 0, None, None) == vs.VS_ERR_ARG
    assert L.vs_attn_fwd_packed(q, k, k, ctypes.byref(m), 0.1, o, lse, 2, st, None) == vs.VS_ERR_ARG
    q32 = _fake_tensor(0x20000000, 4, 1024, 64, vs.VS_F32)
    k32 = _fake_tensor(0x30000000, 2, 1024, 64, vs.VS_F32)
    assert L.vs_attn_fwd_packed(q32, k32, k32, ctypes.byref(m), 0.1, o, lse, 0, st, None) == vs.VS_ERR_UNSUPPORTED
    m3, _, _, _ = _mask(L, Hq=3, Hkv=1)                   # three q heads per kv head: no pairs
    m3.rank = m3.src = 0
    q3 = _fake_tensor(0x20000000, 3, 1024, 128, vs.VS_F16)
    k3 = _fake_tensor(0x30000000, 1, 1024, 128, vs.VS_F16)
    assert L.vs_attn_fwd_packed(q3, k3, k3, ctypes.byref(m3), 0.1, o, lse, 0, st, None) == vs.VS_ERR_UNSUPPORTED
    # fused delta and fp16 dO copy
    a16 = ctypes.c_void_p(0x20000000)
    assert L.vs_attn_bwd_prep_f16(p, a16, a16, 4, 1024, 128, p, None, None) == vs.VS_ERR_ARG
    assert L.vs_attn_bwd_prep_f16(p, a16, a16, 0, 1024, 128, p, st, None) == vs.VS_ERR_ARG
    assert L.vs_attn_bwd_prep_f16(p, a16, a16, 4, 1024, 96, p, st, None) == vs.VS_ERR_UNSUPPORTED
    assert L.vs_attn_bwd_prep_f16(p, ctypes.c_void_p(0x20000002), a16, 4, 1024, 128, p, st,
                                  None) == vs.VS_ERR_UNSUPPORTED


def test_index_noalloc_rejects_beyond_scratch(L):
    """The entry point without a workspace refuses an index whose workspace
    would exceed its 16 MiB per-GPU scratch, before any device work."""
    N, Hq, Hkv, D = 1 << 20, 512, 64, 128
    assert vs.index_workspace_size(Hq, Hkv, N, D) > 16 << 20
    lay = vs.layout("contig", 1, N)
    fake = 0x10000000   # never dereferenced: the size check returns first
    q = _fake_tensor(fake, Hq, 64, D)
    k = _fake_tensor(fake, Hkv, N, D)
    assert L.vs_index_build_noalloc(q, k, lay, 0.088, 0.9, fake, fake, fake, fake, fake, fake, None) == \
        vs.VS_ERR_WORKSPACE
    # and the largest supported shape fits
    assert vs.index_workspace_size(128, 16, N, D) <= 16 << 20
