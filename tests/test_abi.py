"""CPU checks of the C ABI: the library loads, exports every declared entry
point, agrees with the oracle on the scheme's constants, and rejects bad
arguments on the host before anything would be enqueued.  No kernel runs."""

import ctypes
import os
import re

import pytest

import bit_quantized_attention_sage_amd as sage
from oracle import constants as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage_attn.h")
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sage.LIB_PATH):
        pytest.skip("libsage_attn.so not built")
    return sage.load()


def declared_functions():
    """Every function declared by include/*.h."""
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(sage_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("sage_attn_quantize", "sage_attn_fwd", "sage_attn_fwd_quantized",
                 "sage_attn_workspace_bytes", "sage_attn_quant_layout", "sage_attn_debug_scores_i32",
                 "sage_attn_quantize_frames", "sage_attn_quantize_frames_batched",
                 "sage_w8a8_quantize_weight", "sage_w8a8_quantize_act",
                 "sage_w8a8_gemm", "sage_w8a8_sizes"):
        assert must in names


def test_binding_limits_match_the_header():
    text = open(HEADER).read()
    for name in ("SAGE_MAX_BATCH", "SAGE_MAX_SPLITS", "SAGE_MAX_MASK_CHUNKS"):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(sage, name), name


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(sage.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_constants_agree_with_oracle(lib):
    for name in ("BQ", "BK", "VB", "QMAX", "TAU", "PSHIFT_FP8", "PSHIFT_16", "KMEAN_CHUNK"):
        assert sage.sage_attn_constant(name) == getattr(oc, name), name
    with pytest.raises(sage.SageError):
        sage.sage_attn_constant("NOPE")


def _desc(**kw):
    base = dict(B=1, H=2, Nq=100, Nkv=300, d=128, dtype=sage.SAGE_BF16)
    base.update(kw)
    return sage.Desc(**base)


def _status(desc):
    n = ctypes.c_size_t()
    return sage.load().sage_attn_workspace_bytes(desc.ptr, ctypes.byref(n)), n.value


def test_valid_desc_and_workspace(lib):
    st, n = _status(_desc())
    assert st == 0 and n > 0
    # the largest key lengths whose per-head K/V slices the kernel can address
    for nkv, d in ((8388480, 128), (16776960, 64)):
        st, n = _status(_desc(Nkv=nkv, d=d))
        assert st == 0 and n > 2 * nkv * d, sage.load().sage_attn_last_error()
    st8, n8 = _status(_desc(pv_mode=sage.SAGE_PV_FP8))
    assert st8 == 0 and n8 != n


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), 7), (dict(B=0), 2), (dict(Nq=0), 2), (dict(dtype=5), 3), (dict(pv_mode=3), 3),
    (dict(frame_len=-1), 6), (dict(kv_splits=99), 2), (dict(B=1, kv_len=[301]), 6),
    (dict(B=1, kv_len=[0]), 6), (dict(B=1, frame_len=50, kv_len=[120], q_pos0=[30]), 6),
    (dict(q_stride=(100 * 128 * 2, 100 * 128, 127)), 4), (dict(B=129), 7),
    (dict(sm_scale=float("nan")), 2),
    # one head's 16-bit V^T reaches 2^31 bytes (32-bit buffer offsets)
    (dict(Nkv=8388481), 2), (dict(Nkv=16777089, d=64), 2),
    # frame cache and window
    (dict(frame_stride=64, Nkv=320), 6),                                   # no frame_len
    (dict(frame_len=50, frame_stride=100, Nkv=300), 6),                    # not a multiple of 64
    (dict(frame_len=100, frame_stride=64, Nkv=320), 6),                    # shorter than a frame
    (dict(frame_len=50, frame_stride=64, Nkv=300), 2),                     # Nkv not whole frames
    (dict(frame_len=50, window_frames=2), 6),                              # window without a cache
    (dict(frame_len=50, frame_stride=64, Nkv=320, Nq=50, kv_len=[260]), 6),  # beyond 5 frames
    (dict(frame_len=50, frame_stride=64, Nkv=320, Nq=50, window_frames=-1), 6),
])
def test_bad_descriptors_are_rejected(lib, kw, code):
    st, _ = _status(_desc(**kw))
    assert st == code, sage.load().sage_attn_last_error()
    assert sage.load().sage_attn_last_error()


def test_per_head_mode_layout_and_validation(lib):
    """SAGE_PV_AUTO: a 16-bit sized V^T slot per head, the E8M0 region and
    the head lists; refused over a frame cache; its attention call needs the
    stats buffer (where the lists live)."""
    assert sage.SAGE_PV_AUTO == oc.PV_AUTO
    st16, n16 = _status(_desc())
    st8, n8 = _status(_desc(pv_mode=sage.SAGE_PV_FP8))
    sta, na = _status(_desc(pv_mode=sage.SAGE_PV_AUTO))
    assert st16 == st8 == sta == 0 and na > n16 > n8
    d = _desc(pv_mode=sage.SAGE_PV_AUTO)
    b = sage.sage_quant_bufs()
    fake = 1 << 20
    L = sage.load()
    assert L.sage_attn_quant_layout(d.ptr, ctypes.c_void_p(fake), na, ctypes.byref(b)) == 0
    assert b.v_e8m0 and b.stats and b.v_e8m0 - b.v_t >= 2 * 2 * 384 * 128
    assert b.pv_layout == sage.SAGE_PV_AUTO
    b.stats = None
    assert L.sage_attn_fwd_quantized(d.ptr, ctypes.byref(b), ctypes.c_void_p(fake), None) == 1
    assert "stats" in L.sage_attn_last_error().decode()
    # buffers carved for a single P.V mode have smaller V slots and no head
    # lists: a per-head call refuses them before anything is enqueued
    d8 = _desc(pv_mode=sage.SAGE_PV_FP8)
    b8 = sage.sage_quant_bufs()
    assert L.sage_attn_quant_layout(d8.ptr, ctypes.c_void_p(fake), n8, ctypes.byref(b8)) == 0
    assert b8.pv_layout == sage.SAGE_PV_FP8
    assert L.sage_attn_fwd_quantized(d.ptr, ctypes.byref(b8), ctypes.c_void_p(fake), None) == 8
    assert L.sage_attn_quantize(d.ptr, ctypes.c_void_p(fake), ctypes.c_void_p(fake), ctypes.c_void_p(fake),
                                ctypes.byref(b8), None) == 8
    assert _status(_desc(pv_mode=sage.SAGE_PV_AUTO, frame_len=50, frame_stride=64, Nkv=320, Nq=50))[0] == 7


def test_version_mismatch(lib):
    d = _desc()
    d.c.abi_version = 7
    assert _status(d)[0] == 9


def test_null_and_small_workspace_rejected(lib):
    d = _desc()
    b = sage.sage_quant_bufs()
    L = sage.load()
    assert L.sage_attn_quant_layout(d.ptr, None, 0, ctypes.byref(b)) == 8
    assert L.sage_attn_quant_layout(d.ptr, ctypes.c_void_p(256), 16, ctypes.byref(b)) == 8
    assert L.sage_attn_quant_layout(d.ptr, ctypes.c_void_p(257), 1 << 40, ctypes.byref(b)) == 5
    assert L.sage_attn_quantize(d.ptr, None, None, None, ctypes.byref(b), None) == 1
    assert L.sage_attn_fwd_quantized(d.ptr, ctypes.byref(b), None, None) == 1
    assert L.sage_attn_fwd(d.ptr, None, None, None, None, None, 0, None) == 8


def test_layout_is_host_only_and_aligned(lib):
    d = _desc(pv_mode=sage.SAGE_PV_FP8)
    st, n = _status(d)
    b = sage.sage_quant_bufs()
    fake = 1 << 20  # never dereferenced: layout only does pointer arithmetic
    assert sage.load().sage_attn_quant_layout(d.ptr, ctypes.c_void_p(fake), n, ctypes.byref(b)) == 0
    ptrs = [b.q_codes, b.q_scale, b.k_codes, b.k_scale, b.k_mean, b.chan_shift, b.v_t, b.v_e8m0, b.stats]
    assert all(p % 256 == 0 and fake <= p < fake + n for p in ptrs)
    assert len(set(ptrs)) == len(ptrs)


def test_auto_splits(lib):
    # 24 heads x 16 query tiles leave the 256 CUs short of work: split the keys
    d = sage.Desc(1, 24, 2040, 34680, 128, sage.SAGE_BF16, frame_len=2040)
    assert sage.sage_attn_kv_splits(d) > 1
    big = sage.Desc(1, 40, 75600, 75600, 128, sage.SAGE_BF16)
    assert sage.sage_attn_kv_splits(big) == 1
    fixed = sage.Desc(1, 2, 1024, 1024, 64, sage.SAGE_F16, kv_splits=3)
    assert sage.sage_attn_kv_splits(fixed) == 3


def test_frame_cache_desc_and_quantize_frames_validation(lib):
    ok = _desc(frame_len=50, frame_stride=64, Nkv=320, Nq=50, kv_len=[250], sink_frames=1, window_frames=2)
    assert _status(ok)[0] == 0
    d = _desc(frame_len=50, frame_stride=64, Nkv=320, Nq=50)
    d.c.reserved = 3
    assert _status(d)[0] == 7
    # argument checks of sage_attn_quantize_frames (host-only; nothing enqueued)
    n = sage.sage_attn_workspace_bytes(ok)
    ws = (ctypes.c_uint8 * (n + 256))()
    base = (ctypes.addressof(ws) + 255) // 256 * 256
    bufs = sage.sage_quant_bufs()
    assert lib.sage_attn_quant_layout(ok.ptr, ctypes.c_void_p(base), n, ctypes.byref(bufs)) == 0
    fake = ctypes.c_void_p(base)  # aligned; never dereferenced on these error paths
    st = lib.sage_attn_quantize_frames(ok.ptr, None, fake, fake, 4, 2, ctypes.byref(bufs), None)
    assert st == 2 and b"inside" in lib.sage_attn_last_error()
    assert lib.sage_attn_quantize_frames(ok.ptr, None, fake, fake, -1, 1, ctypes.byref(bufs), None) == 2
    plain = _desc()
    n2 = sage.sage_attn_workspace_bytes(plain)
    ws2 = (ctypes.c_uint8 * (n2 + 256))()
    base2 = (ctypes.addressof(ws2) + 255) // 256 * 256
    bufs2 = sage.sage_quant_bufs()
    assert lib.sage_attn_quant_layout(plain.ptr, ctypes.c_void_p(base2), n2, ctypes.byref(bufs2)) == 0
    f2 = ctypes.c_void_p(base2)
    assert lib.sage_attn_quantize_frames(plain.ptr, None, f2, f2, 0, 1, ctypes.byref(bufs2), None) == 7


def test_quantize_frames_batched_validation(lib):
    d = _desc(B=2, frame_len=50, frame_stride=64, Nkv=320, Nq=50, kv_len=[250, 150])
    assert _status(d)[0] == 0
    n = sage.sage_attn_workspace_bytes(d)
    ws = (ctypes.c_uint8 * (n + 256))()
    base = (ctypes.addressof(ws) + 255) // 256 * 256
    bufs = sage.sage_quant_bufs()
    assert lib.sage_attn_quant_layout(d.ptr, ctypes.c_void_p(base), n, ctypes.byref(bufs)) == 0
    fake = ctypes.c_void_p(base)  # aligned; never dereferenced on these error paths
    arr = ctypes.c_int32 * 2
    qfb = lib.sage_attn_quantize_frames_batched
    assert qfb(d.ptr, None, fake, fake, None, 1, ctypes.byref(bufs), None) == 1
    st = qfb(d.ptr, None, fake, fake, arr(4, 5), 1, ctypes.byref(bufs), None)  # batch 1: frame 5 of 5
    assert st == 2 and b"batch 1" in lib.sage_attn_last_error()
    assert qfb(d.ptr, None, fake, fake, arr(0, -1), 1, ctypes.byref(bufs), None) == 2
    assert qfb(d.ptr, None, fake, fake, arr(0, 0), 0, ctypes.byref(bufs), None) == 2
    plain = _desc(B=2)
    n2 = sage.sage_attn_workspace_bytes(plain)
    ws2 = (ctypes.c_uint8 * (n2 + 256))()
    base2 = (ctypes.addressof(ws2) + 255) // 256 * 256
    bufs2 = sage.sage_quant_bufs()
    assert lib.sage_attn_quant_layout(plain.ptr, ctypes.c_void_p(base2), n2, ctypes.byref(bufs2)) == 0
    f2 = ctypes.c_void_p(base2)
    assert qfb(plain.ptr, None, f2, f2, arr(0, 0), 1, ctypes.byref(bufs2), None) == 7


def test_block_mask_validation(lib):
    d = _desc()
    d.c.block_mask = 4096      # a device address; never read on the host
    assert _status(d)[0] == 0
    cache = _desc(frame_len=50, frame_stride=64, Nkv=320, Nq=50)
    cache.c.block_mask = 4096
    assert _status(cache)[0] == 7 and b"contiguous" in lib.sage_attn_last_error()
    big = sage.Desc(1, 1, 128, 64 * 4096 + 1, 128, sage.SAGE_BF16)
    big.c.block_mask = 4096
    assert _status(big)[0] == 7
    ok = sage.Desc(1, 1, 128, 64 * 4096, 128, sage.SAGE_BF16)
    ok.c.block_mask = 4096
    assert _status(ok)[0] == 0


def test_block_mask_binding_checks_its_shape():
    import torch
    m = torch.ones((1, 2, 1, 3), dtype=torch.uint8)
    sage.Desc(1, 2, 100, 150, 64, sage.SAGE_F16, block_mask=m)
    with pytest.raises(ValueError):
        sage.Desc(1, 2, 100, 150, 64, sage.SAGE_F16, block_mask=m[:, :, :, :2])
    with pytest.raises(ValueError):
        sage.Desc(1, 2, 100, 150, 64, sage.SAGE_F16, block_mask=m.bool())


def _w8(**kw):
    base = dict(M=300, N=256, K=384, dtype=sage.SAGE_BF16)
    base.update(kw)
    return sage.W8A8Desc(**base)


def test_w8a8_sizes_and_validation(lib):
    xq, xs, wq, ws = sage.sage_w8a8_sizes(_w8())
    assert (xq, xs, wq, ws) == (384 * 384, 3 * 384 * 4, 256 * 384, 2 * 3 * 4)
    for kw, code in [(dict(N=200), 2), (dict(K=100), 2), (dict(M=0), 2), (dict(dtype=4), 3),
                     (dict(x_stride=200), 4), (dict(y_stride=260), 4), (dict(M=1 << 22, K=1024), 2)]:
        n = ctypes.c_size_t()
        st = lib.sage_w8a8_sizes(_w8(**kw).ptr, ctypes.byref(n), None, None, None)
        assert st == code, (kw, st, lib.sage_attn_last_error())
    d = _w8()
    d.c.abi_version = 1
    assert lib.sage_w8a8_sizes(d.ptr, None, None, None, None) == 9
    d = _w8()
    assert lib.sage_w8a8_gemm(d.ptr, None, None, None, None, None, None, None) == 1
    fake = ctypes.c_void_p(4096 + 8)  # misaligned; never dereferenced
    ok = ctypes.c_void_p(4096)
    assert lib.sage_w8a8_gemm(d.ptr, ok, ok, ok, ok, None, fake, None) == 5
    assert lib.sage_w8a8_quantize_act(d.ptr, fake, ok, ok, None) == 5


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No CPU fallback: without the built library, loading it (which every
    entry point does first) raises."""
    monkeypatch.setattr(sage, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        sage.load(str(tmp_path / "libsage_attn.so"))


def test_split_capacity_covers_a_growing_frame_cache(lib):
    """A frame cache's workspace is carved once, while its kv_len grows step
    by step and the library's split count with it (B1 H1, 2040-token frames
    in 2048-slot strides, 1 -> 5 frames).  The carved partial region holds
    room for every later step; a call that needs more splits than were
    carved fails with SAGE_E_WORKSPACE before anything is enqueued (host
    validation only: the pointers below are never dereferenced)."""
    F, FS, nf = 2040, 2048, 5

    def desc(frames, **kw):
        return sage.Desc(1, 1, F, nf * FS, 128, sage.SAGE_BF16, frame_len=F, frame_stride=FS,
                         kv_len=[frames * F], **kw)

    L = sage.load()
    fake = 1 << 32
    first = desc(1)
    bufs = sage.sage_quant_bufs()
    n = sage.sage_attn_workspace_bytes(first)
    assert L.sage_attn_quant_layout(first.ptr, ctypes.c_void_p(fake), n, ctypes.byref(bufs)) == 0
    seen = [sage.sage_attn_kv_splits(desc(f)) for f in range(1, nf + 1)]
    assert len(set(seen)) > 1                        # the split count does grow with the cache
    assert max(seen) <= bufs.partial_splits
    part_end = bufs.partial + bufs.partial_splits * 1 * 1 * 2048 * (128 + 2) * 4
    assert part_end <= fake + n                      # and the region really is that large
    # carved for 2 forced splits, called with 16: rejected on the host
    small = desc(1, kv_splits=2)
    n2 = sage.sage_attn_workspace_bytes(small)
    b2 = sage.sage_quant_bufs()
    assert L.sage_attn_quant_layout(small.ptr, ctypes.c_void_p(fake), n2, ctypes.byref(b2)) == 0
    assert b2.partial_splits == 2
    big = desc(5, kv_splits=16)
    st = L.sage_attn_fwd_quantized(big.ptr, ctypes.byref(b2), ctypes.c_void_p(fake), None)
    assert st == 8 and b"16 KV splits" in L.sage_attn_last_error()
    # one split needs no partial region at all
    one = desc(1, kv_splits=1)
    b1 = sage.sage_quant_bufs()
    assert L.sage_attn_quant_layout(one.ptr, ctypes.c_void_p(fake), sage.sage_attn_workspace_bytes(one),
                                    ctypes.byref(b1)) == 0
    assert b1.partial is None and b1.partial_splits == 1
