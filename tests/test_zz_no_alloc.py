"""The allocation-free entry point, sage_attn_fwd_quantized_noalloc, for
callers that cannot allocate device memory: its output equals
sage_attn_fwd_quantized's bit for bit (the same kernels; only the split-KV
partials live in the library's device scratch instead of the workspace), on
two calls in a row, the second with a smaller input, both with KV splits so
that the scratch is really used; a call whose partials exceed the scratch
is refused on the host; and a streaming step captured into a HIP graph
replays like the workspace entry point."""

import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage

pytestmark = pytest.mark.gpu

SCRATCH = 128 << 20


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).cuda()


def _pair(B, H, Nq, Nkv, d, pv_mode, splits, seed, F=0, kv_len=None, outlier_heads=()):
    q, k, v = _rand((B, H, Nq, d), seed), _rand((B, H, Nkv, d), seed + 1), _rand((B, H, Nkv, d), seed + 2)
    for h in outlier_heads:                 # (per-head mode: those heads take 16-bit P.V)
        k[:, h, :, 3] *= 8
    o_ref, o_na = torch.empty_like(q), torch.full_like(q, float("nan"))
    desc = sage.Desc.for_tensors(q, k, v, o_ref, pv_mode=pv_mode, kv_splits=splits, frame_len=F, kv_len=kv_len)
    assert sage.sage_attn_kv_splits(desc) == splits
    need = splits * B * H * desc.Nq_pad * (d + 2) * 4
    assert 0 < need <= SCRATCH
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)
    sage.sage_attn_fwd_quantized(desc, bufs, o_ref)
    nb = sage.sage_quant_bufs.from_buffer_copy(bufs)
    nb.partial = None                       # the entry point needs no partial region
    nb.partial_splits = 1
    sage.sage_attn_fwd_quantized_noalloc(desc, nb, o_na)
    torch.cuda.synchronize()
    print(f"  B{B} H{H} Nq{Nq} Nkv{Nkv} d{d} pv{pv_mode} splits {splits}: scratch bytes {need}, "
          f"equal {torch.equal(o_ref, o_na)}", flush=True)
    return o_ref, o_na


@pytest.mark.parametrize("pv_mode", [0, 1, 2], ids=["pv16", "pvfp8", "pvauto"])
def test_noalloc_equals_workspace_entry_point(lib, pv_mode):
    # a streaming-sized call, then a smaller one: the second reads only what it wrote
    o1, n1 = _pair(1, 24, 2040, 34680, 128, pv_mode, 4, 10 + pv_mode, F=2040, kv_len=[34680],
                   outlier_heads=(1, 5, 23))
    assert torch.equal(o1, n1)
    o2, n2 = _pair(2, 3, 300, 2500, 64, pv_mode, 3, 20 + pv_mode, outlier_heads=(0,))
    assert torch.equal(o2, n2)


def test_noalloc_rejects_partials_beyond_the_scratch(lib):
    """Host validation: 16 splits of B4 H24 Nq 4096 d 128 need 208 MB of
    partials (> 128 MiB): SAGE_E_WORKSPACE, nothing enqueued."""
    d = sage.Desc(4, 24, 4096, 8192, 128, sage.SAGE_BF16, kv_splits=16)
    b = sage.sage_quant_bufs()
    st = sage.load().sage_attn_fwd_quantized_noalloc(d.ptr, ctypes.byref(b), ctypes.c_void_p(1 << 20), None)
    assert st == 8 and b"device scratch" in sage.load().sage_attn_last_error()


def _capture(fn):
    """Warm fn up on a side stream (the scratch address is looked up on a
    device's first call), then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("pv_mode", [0, 1], ids=["pv16", "pvfp8"])
def test_noalloc_streaming_step_replays_from_a_graph(lib, pv_mode):
    """The use the entry point exists for: a frame-cache attention step (4 KV
    splits, partials in the device scratch) captured once into a HIP graph
    and replayed four times, the cache's current frame and the queries
    quantized again eagerly between replays; every replay equals the
    workspace entry point run eagerly on the same buffers, bit for bit."""
    B, H, F, FS, nf, d = 1, 4, 200, 256, 6, 128
    q = _rand((B, H, F, d), 40 + pv_mode)
    k, v = _rand((B, H, nf * F, d), 41), _rand((B, H, nf * F, d), 42)
    o_na, o_ref = torch.full_like(q, float("nan")), torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o_ref, nkv=nf * FS, pv_mode=pv_mode, frame_len=F, frame_stride=FS,
                                 kv_len=[nf * F], q_pos0=[(nf - 1) * F], kv_splits=4)
    assert sage.sage_attn_kv_splits(desc) == 4
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)      # the cache, once
    nb = sage.sage_quant_bufs.from_buffer_copy(bufs)
    nb.partial = None
    nb.partial_splits = 1
    kk, vv = k[:, :, (nf - 1) * F:], v[:, :, (nf - 1) * F:]
    d2 = sage.Desc.for_tensors(q, kk, vv, nkv=nf * FS, pv_mode=pv_mode, frame_len=F, frame_stride=FS)
    g = _capture(lambda: sage.sage_attn_fwd_quantized_noalloc(desc, nb, o_na))
    for r in range(4):
        q.copy_(_rand((B, H, F, d), 50 + r))
        kk.copy_(_rand((B, H, F, d), 60 + r))
        vv.copy_(_rand((B, H, F, d), 70 + r))
        sage.sage_attn_quantize_frames(d2, q, kk, vv, nf - 1, 1, bufs)
        o_na.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        sage.sage_attn_fwd_quantized(desc, bufs, o_ref)
        torch.cuda.synchronize()
        print(f"  replay {r}: equal {torch.equal(o_na, o_ref)}", flush=True)
        assert torch.isfinite(o_ref).all() and torch.equal(o_na, o_ref)
