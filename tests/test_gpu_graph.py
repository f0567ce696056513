"""Capture of the library's calls into a HIP graph (torch.cuda.CUDAGraph).

Short streaming steps are dominated by launch overhead unless they are
replayed from a captured graph (Vidu S1 blog, section "Infra": CUDA graphs
for the real-time loop).  Every entry point enqueues kernels on the caller's
stream only -- no allocation, no synchronization, no memset -- so a call can
be captured.  Each test captures a call sequence once, replays it several
times with eager work and synchronizations in between (new inputs written in
place, the output cleared), and checks every replay bit-for-bit against the
same sequence run eagerly on the same inputs.
"""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
from oracle.constants import PV_16, PV_FP8, PV_AUTO

pytestmark = pytest.mark.gpu


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).cuda()


def _capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
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


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
def test_drop_in_call_replays_like_eager(lib, pv_mode):
    """sage_attn_fwd (quantize + fused kernel + split combine, 3 KV splits)."""
    B, H, Nq, Nkv, d = 1, 4, 500, 3000, 128
    q, k, v = _rand((B, H, Nq, d), 1), _rand((B, H, Nkv, d), 2, 2.0), _rand((B, H, Nkv, d), 3)
    o = torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o, pv_mode=pv_mode, kv_splits=3)
    assert sage.sage_attn_kv_splits(desc) == 3
    ws = sage.new_workspace(desc, q.device)
    g = _capture(lambda: sage.sage_attn_fwd(desc, q, k, v, o, ws))
    for r in range(4):
        # new inputs, written in place between replays (eager work)
        q.copy_(_rand((B, H, Nq, d), 10 + r))
        v.mul_(-1 if r % 2 else 1)
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = o.clone()
        ref = torch.empty_like(q)
        ws_ref = sage.new_workspace(desc, q.device)
        sage.sage_attn_fwd(desc, q, k, v, ref, ws_ref)
        torch.cuda.synchronize()
        print(f"  replay {r}: equal {torch.equal(got, ref)}", flush=True)
        assert torch.equal(got, ref)


def test_per_head_mode_replays_like_eager(lib):
    """sage_attn_fwd in the per-head P.V mode (head lists built on the device,
    one fused-kernel launch per mode, 2 KV splits).  Between replays the
    inputs change which heads carry an outlier K channel, so each replay
    must take its head split from the device, not from the capture."""
    B, H, Nq, Nkv, d = 1, 4, 400, 1500, 128
    q, k, v = _rand((B, H, Nq, d), 21), _rand((B, H, Nkv, d), 22), _rand((B, H, Nkv, d), 23)
    base = k.clone()
    o = torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o, pv_mode=PV_AUTO, kv_splits=2)
    ws = sage.new_workspace(desc, q.device)
    g = _capture(lambda: sage.sage_attn_fwd(desc, q, k, v, o, ws))
    for r, heads in enumerate([[0], [1, 3], [], [0, 1, 2, 3]]):
        k.copy_(base)
        for h in heads:
            k[0, h, :, 17] *= 8                  # an outlier channel: 16-bit P.V for that head
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = o.clone()
        ref = torch.empty_like(q)
        ws_ref = sage.new_workspace(desc, q.device)
        sage.sage_attn_fwd(desc, q, k, v, ref, ws_ref)
        torch.cuda.synchronize()
        moved = (sage.quant_views(desc, ws, sage.sage_attn_quant_layout(desc, ws))["chan_shift"] != 0)
        split = moved.any(dim=-1)[0].nonzero().flatten().tolist()
        print(f"  replay {r}: 16-bit heads {split}, equal {torch.equal(got, ref)}", flush=True)
        assert split == heads
        assert torch.equal(got, ref)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
def test_streaming_step_replays_like_eager(lib, pv_mode):
    """One streaming step over a frame cache of three sessions with their own
    lengths: each session's current frame appended (sage_attn_quantize_frames
    _batched, queries included) and the fused kernel with 3 KV splits plus
    the combine.  The cache is quantized once beforehand; each replay
    re-appends new frame contents written in place."""
    B, H, d, F, FS, nf = 3, 2, 128, 100, 128, 8
    frames = [8, 6, 3]                          # frames each session holds, its current one included
    kv_len = [f * F for f in frames]
    q_pos0 = [(f - 1) * F for f in frames]
    q = _rand((B, H, F, d), 20)
    k = _rand((B, H, nf * F, d), 21, 1.5)
    v = _rand((B, H, nf * F, d), 22)
    for b in range(B):
        k[b, :, kv_len[b]:] = 0
        v[b, :, kv_len[b]:] = 0
    o = torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o, nkv=nf * FS, pv_mode=pv_mode, frame_len=F, frame_stride=FS,
                                 kv_len=kv_len, q_pos0=q_pos0, kv_splits=3, sink_frames=1, window_frames=3)
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)           # the cache, quantized once
    torch.cuda.synchronize()
    f0 = [f - 1 for f in frames]
    kk = torch.stack([k[b, :, f0[b] * F:(f0[b] + 1) * F] for b in range(B)]).contiguous()
    vv = torch.stack([v[b, :, f0[b] * F:(f0[b] + 1) * F] for b in range(B)]).contiguous()
    d2 = sage.Desc.for_tensors(q, kk, vv, nkv=nf * FS, pv_mode=pv_mode, frame_len=F, frame_stride=FS)

    def step():
        sage.sage_attn_quantize_frames_batched(d2, q, kk, vv, f0, 1, bufs)
        sage.sage_attn_fwd_quantized(desc, bufs, o)

    snapshot = ws.clone()
    g = _capture(step)
    for r in range(4):
        q.copy_(_rand((B, H, F, d), 30 + r))
        kk.copy_(_rand((B, H, F, d), 40 + r, 1.5))
        vv.copy_(_rand((B, H, F, d), 50 + r))
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, got_ws = o.clone(), ws.clone()
        # the same step eagerly, on a copy of the cache as it was before the step
        ws_ref = snapshot.clone()
        bufs_ref = sage.sage_attn_quant_layout(desc, ws_ref)
        ref = torch.empty_like(q)
        sage.sage_attn_quantize_frames_batched(d2, q, kk, vv, f0, 1, bufs_ref)
        sage.sage_attn_fwd_quantized(desc, bufs_ref, ref)
        torch.cuda.synchronize()
        qv_got = sage.quant_views(desc, got_ws, sage.sage_attn_quant_layout(desc, got_ws))
        qv_ref = sage.quant_views(desc, ws_ref, bufs_ref)
        for name in ("q_codes", "q_scale", "k_codes", "k_scale", "v_t"):
            assert torch.equal(qv_got[name], qv_ref[name]), name
        print(f"  replay {r}: equal {torch.equal(got, ref)}", flush=True)
        assert torch.equal(got, ref)
        ws.copy_(snapshot)                     # back to the cache before the step (eager work)
