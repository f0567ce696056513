"""GPU parity of the frame cache (whole frames quantized once into padded
slots) and the sliding window with sink frames, through the C ABI.

Streaming decoding attends within a fixed window -- sink frames, the most
recent history frames and the current frame -- over cached history (Vidu S1
blog, section "Infra").  Bit-exact: every quantized operand in its cache
slots, and appending frames one at a time against the same frozen mean and
exponents gives the same buffers as quantizing the whole cache.  Outputs:
every element within the derived bound of gpu_util of the oracle's
emulation with the same KV splits (each batch's chunk list cut into the
library's split count), cosine >= 0.999 against float64 windowed
attention."""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
import workloads
from oracle import quant, emulate, attention, codecs
from oracle.constants import PV_16, PV_FP8, BK
from gpu_util import host, assert_close, cosine, NAME_DT, KERNEL_SLACK

pytestmark = pytest.mark.gpu


def _rand(shape, dtype, seed, scale=1.0, offset=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * scale
    if offset is not None:
        x = x + offset
    return x.to(dtype)


def _inputs(B, H, Nq, ntok, d, dt, seed):
    q = _rand((B, H, Nq, d), dt, seed)
    k = _rand((B, H, ntok, d), dt, seed + 1, offset=_rand((1, H, 1, d), torch.float32, seed + 2) * 1.5)
    v = _rand((B, H, ntok, d), dt, seed + 3)
    return q, k, v


def _frozen(Q, K):
    mu = quant.k_mean(K)
    return mu, quant.channel_shift(Q, K, mu)


def _run(q, k, v, pv_mode, F, FS, nslots, S=0, W=0, kv_len=None, q_pos0=None, splits=0, mu=None, a=None):
    o = torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o, nkv=nslots, pv_mode=pv_mode, frame_len=F, frame_stride=FS,
                                 sink_frames=S, window_frames=W, kv_len=kv_len, q_pos0=q_pos0,
                                 kv_splits=splits,
                                 k_mean_in=torch.from_numpy(mu).cuda() if mu is not None else None,
                                 chan_shift_in=torch.from_numpy(a.astype(np.int8)).cuda() if a is not None else None)
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)
    sage.sage_attn_fwd_quantized(desc, bufs, o)
    torch.cuda.synchronize()
    return o, desc, ws, bufs


def emulate_cache(Q, K, V, pv_mode, dtype, F, FS, S, W, kv_len, q_pos0, mu, a, nsplit, rows=None):
    """(O64, aux) of the frame-cache emulation with the kernel's slack."""
    o64, _, aux = emulate.emulate_frame_cache(Q, K, V, pv_mode, dtype, F, FS, S, W, kv_len, q_pos0, mu, a,
                                              nsplit, rows=rows, slack=KERNEL_SLACK)
    return o64, aux


def check_cache_operands(views, Q, K, V, mu, a, F, FS, pv_mode):
    """Every quantized operand of a frame cache holding the whole frames of
    K, V (frames 0 ..) bit-exactly against the oracle; slots past them zero."""
    B, H, Nq, d = Q.shape
    nf = K.shape[2] // F
    np.testing.assert_array_equal(views["chan_shift"].cpu().numpy(), a.astype(np.int8))
    kc, dk = quant.quantize_k_frames(K, mu, a, F, FS)
    gk = views["k_codes"].cpu().numpy()
    np.testing.assert_array_equal(gk[:, :, :nf * FS], kc)
    assert not gk[:, :, nf * FS:].any()
    np.testing.assert_array_equal(views["k_scale"].cpu().numpy()[:, :, :nf * FS // BK], dk)
    qc, dq = quant.quantize_q(Q, a)
    np.testing.assert_array_equal(views["q_codes"].cpu().numpy()[:, :, :Nq], qc)
    np.testing.assert_array_equal(views["q_scale"].cpu().numpy()[:, :, :dq.shape[2]], dq)
    untiled = views["v_t"].cpu().permute(0, 1, 2, 4, 3).reshape(B, H, -1, d).numpy()
    if pv_mode == PV_FP8:
        vc, ve = quant.quantize_v_fp8_frames(V, F, FS)
        np.testing.assert_array_equal(untiled.astype(np.uint8)[:, :, :nf * FS], vc)
        ge = views["v_e8m0"].cpu().numpy()
        nch = ge.shape[2]
        g5 = ge.reshape(B, H, nch, 2, 32, 4)[..., : d // 32].transpose(0, 1, 2, 3, 5, 4).reshape(B, H, 2 * nch, d)
        np.testing.assert_array_equal(g5[:, :, :nf * FS // 32], (ve + 127).astype(np.uint8))
    else:
        ref = codecs.bf16_bits(quant.to_frame_slots(V, F, FS))
        np.testing.assert_array_equal(untiled.view(np.uint16)[:, :, :nf * FS], ref)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_frame_cache_quantize_bit_exact(lib, pv_mode):
    B, H, d, F, FS, nf = 2, 2, 128, 200, 256, 5
    q, k, v = _inputs(B, H, F, nf * F, d, torch.bfloat16, 61)
    Q, K, V = host(q), host(k), host(v)
    mu, a = _frozen(Q, K)
    _, desc, ws, bufs = _run(q.cuda(), k.cuda(), v.cuda(), pv_mode, F, FS, nf * FS, mu=mu, a=a)
    check_cache_operands(sage.quant_views(desc, ws, bufs), Q, K, V, mu, a, F, FS, pv_mode)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_append_frames_equals_full_quantize(lib, pv_mode):
    B, H, d, F, FS, nf = 2, 3, 64, 100, 128, 6
    q, k, v = _inputs(B, H, F, nf * F, d, torch.float16, 62)
    Q, K = host(q), host(k)
    mu, a = _frozen(Q, K)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    _, desc, ws_full, bufs_full = _run(q, k, v, pv_mode, F, FS, nf * FS, mu=mu, a=a)
    full = sage.quant_views(desc, ws_full, bufs_full)
    ws = torch.zeros_like(ws_full)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    inc = sage.quant_views(desc, ws, bufs)
    inc["k_mean"].copy_(torch.from_numpy(mu))
    inc["chan_shift"].copy_(torch.from_numpy(a.astype(np.int8)))
    # frames 0..2 together, then 3 and 4 one at a time, the last with the queries
    for f0, nfr in ((0, 3), (3, 1), (4, 1), (5, 1)):
        kk = k[:, :, f0 * F:(f0 + nfr) * F]
        vv = v[:, :, f0 * F:(f0 + nfr) * F]
        d2 = sage.Desc.for_tensors(q, kk, vv, nkv=nf * FS, pv_mode=pv_mode, frame_len=F, frame_stride=FS)
        sage.sage_attn_quantize_frames(d2, q if f0 == 5 else None, kk, vv, f0, nfr, bufs)
    torch.cuda.synchronize()
    for name in full:
        if name in ("k_mean", "chan_shift"):
            continue
        assert torch.equal(full[name], inc[name]), name


CASES = [
    # (B, H, Nq, d, dtype, F, FS, frames cached, q frame0, S, W, splits)
    (1, 2, 200, 128, torch.bfloat16, 200, 256, 8, 7, 1, 3, 0),    # sink + window, padded frames
    (1, 2, 200, 128, torch.bfloat16, 200, 256, 8, 7, 1, 3, 3),    # ... with forced KV splits
    (2, 2, 200, 128, torch.bfloat16, 100, 128, 8, 6, 2, 2, 0),    # queries span two frames (tiles straddle)
    (1, 2, 200, 128, torch.bfloat16, 200, 256, 6, 5, 0, 0, 0),    # no window: causal over the padded cache
    (1, 1, 64, 128, torch.bfloat16, 64, 64, 2, 1, 4, 1, 0),       # query frame inside the sinks
    (1, 2, 150, 64, torch.float16, 150, 192, 9, 8, 2, 1, 2),      # d = 64, fp16, short window
    # queries over six frames: three 256-row work items (the last half empty),
    # tile boundaries inside frames, forced splits of each item's chunk list
    (1, 2, 600, 128, torch.bfloat16, 100, 128, 12, 6, 1, 2, 3),
    # no sinks: a work item's list starts with window frames that its later
    # rows do not see (their running max meets masked chunks first)
    (1, 2, 600, 128, torch.bfloat16, 100, 128, 12, 6, 0, 2, 0),
    (1, 2, 600, 64, torch.float16, 100, 128, 12, 6, 0, 1, 2),
]


def _cid(c):
    return f"B{c[0]}H{c[1]}q{c[2]}d{c[3]}{NAME_DT[c[4]]}F{c[5]}FS{c[6]}n{c[7]}S{c[9]}W{c[10]}s{c[11]}"


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_per_batch_appends_equal_full_quantize(lib, pv_mode):
    """Each batch appends its frames at its own place
    (sage_attn_quantize_frames_batched): three calls of two frames, batch b
    starting at frame (2b, 2b + 2, 2b + 4) mod 6, fill every batch's six
    frames in a different order; the buffers equal one whole-cache
    quantization byte for byte."""
    B, H, d, F, FS, nf = 3, 2, 128, 100, 128, 6
    q, k, v = _inputs(B, H, F, nf * F, d, torch.bfloat16, 63)
    Q, K = host(q), host(k)
    mu, a = _frozen(Q, K)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    _, desc, ws_full, bufs_full = _run(q, k, v, pv_mode, F, FS, nf * FS, mu=mu, a=a)
    full = sage.quant_views(desc, ws_full, bufs_full)
    ws = torch.zeros_like(ws_full)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    inc = sage.quant_views(desc, ws, bufs)
    inc["k_mean"].copy_(torch.from_numpy(mu))
    inc["chan_shift"].copy_(torch.from_numpy(a.astype(np.int8)))
    for call in range(3):
        f0 = [(2 * b + 2 * call) % nf for b in range(B)]
        kk = torch.stack([k[b, :, f0[b] * F:(f0[b] + 2) * F] for b in range(B)]).contiguous()
        vv = torch.stack([v[b, :, f0[b] * F:(f0[b] + 2) * F] for b in range(B)]).contiguous()
        d2 = sage.Desc.for_tensors(q, kk, vv, nkv=nf * FS, pv_mode=pv_mode, frame_len=F, frame_stride=FS)
        sage.sage_attn_quantize_frames_batched(d2, q if call == 2 else None, kk, vv, f0, 2, bufs)
    torch.cuda.synchronize()
    for name in full:
        if name in ("k_mean", "chan_shift"):
            continue
        assert torch.equal(full[name], inc[name]), name


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
@pytest.mark.parametrize("case", CASES, ids=[_cid(c) for c in CASES])
def test_window_parity(lib, case, pv_mode):
    B, H, Nq, d, dt, F, FS, nf, qf0, S, W, splits = case
    print(f"window case {_cid(case)} pv {pv_mode}", flush=True)
    q, k, v = _inputs(B, H, Nq, nf * F, d, dt, sum(map(ord, _cid(case))) + pv_mode)
    Q, K, V = host(q), host(k), host(v)
    mu, a = _frozen(Q, K)
    kv_len, q_pos0 = [nf * F] * B, [qf0 * F] * B
    o, desc, _, _ = _run(q.cuda(), k.cuda(), v.cuda(), pv_mode, F, FS, nf * FS, S, W, kv_len, q_pos0,
                         splits, mu, a)
    nsplit = sage.sage_attn_kv_splits(desc)
    o64, aux = emulate_cache(Q, K, V, pv_mode, NAME_DT[dt], F, FS, S, W, kv_len, q_pos0, mu, a, nsplit)
    og = host(o)
    print(f"  splits {nsplit}")
    assert_close(og, o64, aux, NAME_DT[dt], pv_mode, nsplit)
    ref = attention.attention_fp64(Q, K, V, frame_len=F, kv_len=kv_len, q_pos0=q_pos0, sink_frames=S,
                                   window_frames=W)
    cs = cosine(og, ref)
    print(f"  cosine vs fp64 windowed attention {cs:.6f} (emulation {cosine(o64, ref):.6f})")
    assert cs >= 0.999


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
def test_window_ragged_batches(lib, pv_mode, splits):
    """Batches with their own cache lengths, two of them ending inside a frame
    (the current frame only partly written), queries spanning frames, one
    sink frame and a two-frame window."""
    B, H, Nq, d, dt, F, FS, nf, S, W = 3, 2, 250, 128, torch.bfloat16, 100, 128, 10, 1, 2
    kv_len, q_pos0 = [1000, 763, 540], [750, 513, 290]
    print(f"ragged window batches pv {pv_mode} splits {splits}", flush=True)
    q, k, v = _inputs(B, H, Nq, nf * F, d, dt, 4100 + 10 * pv_mode + splits)
    Q, K, V = host(q), host(k), host(v)
    mu, a = _frozen(Q, K)
    o, desc, _, _ = _run(q.cuda(), k.cuda(), v.cuda(), pv_mode, F, FS, nf * FS, S, W, kv_len, q_pos0,
                         splits, mu, a)
    nsplit = sage.sage_attn_kv_splits(desc)
    o64, aux = emulate_cache(Q, K, V, pv_mode, "bf16", F, FS, S, W, kv_len, q_pos0, mu, a, nsplit)
    og = host(o)
    print(f"  splits {nsplit}")
    assert np.isfinite(og).all()
    assert_close(og, o64, aux, "bf16", pv_mode, nsplit)
    ref = attention.attention_fp64(Q, K, V, frame_len=F, kv_len=kv_len, q_pos0=q_pos0, sink_frames=S,
                                   window_frames=W)
    cs = cosine(og, ref)
    print(f"  cosine vs fp64 windowed attention {cs:.6f} (emulation {cosine(o64, ref):.6f})")
    assert cs >= 0.999


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_cache_without_padding_or_window_equals_contiguous(lib, pv_mode):
    """Frames of a multiple of 64 tokens, no padding, no window: the cache
    launch visits the same chunks with the same masks as the contiguous one,
    so the outputs are identical."""
    B, H, d, F, nf, Nq = 2, 2, 128, 256, 5, 256
    q, k, v = _inputs(B, H, Nq, nf * F, d, torch.bfloat16, 63)
    Q, K = host(q), host(k)
    mu, a = _frozen(Q, K)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    kv, qp = [nf * F, 3 * F], [(nf - 1) * F, 2 * F]
    o1, _, _, _ = _run(q, k, v, pv_mode, F, F, nf * F, kv_len=kv, q_pos0=qp, splits=1, mu=mu, a=a)
    o2 = torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o2, pv_mode=pv_mode, frame_len=F, kv_len=kv, q_pos0=qp, kv_splits=1,
                                 k_mean_in=torch.from_numpy(mu).cuda(),
                                 chan_shift_in=torch.from_numpy(a.astype(np.int8)).cuda())
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)
    sage.sage_attn_fwd_quantized(desc, bufs, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.slow
@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
def test_window_workload_parity(lib, pv_mode):
    """The window workload at full size (B1 H24, 41 cached 2040-token frames at
    a stride of 2048 slots, queries = frame 40, 1 sink + 16 window frames) in
    the launch configuration bench.py times: the whole cache quantized once
    (the library computes the mean and exponents), the current frame and the
    queries quantized again through sage_attn_quantize_frames, then attention
    with the library-chosen KV splits.  Bit-exact operands on all heads;
    outputs of 3 seeded heads on sampled rows against the emulation, cosine
    against float64 windowed attention."""
    w = workloads.get("window", pv_mode=pv_mode)
    print(f"workload window pv {pv_mode}", flush=True)
    x = workloads.make(w, "cuda")
    q, k, v = x["q"], x["k"], x["v"]
    o = torch.empty_like(q)
    F, FS, S, W = w.frame_len, w.frame_stride, w.sink_frames, w.window_frames
    kvl, qp = w.kv_lens(), w.q_pos0s()
    desc = sage.Desc.for_tensors(q, k, v, o, nkv=w.Nkv, pv_mode=pv_mode, frame_len=F, frame_stride=FS,
                                 sink_frames=S, window_frames=W, kv_len=kvl, q_pos0=qp)
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)
    fq = qp[0] // F
    kk, vv = k[:, :, fq * F:(fq + 1) * F], v[:, :, fq * F:(fq + 1) * F]
    d2 = sage.Desc.for_tensors(q, kk, vv, nkv=w.Nkv, pv_mode=pv_mode, frame_len=F, frame_stride=FS)
    sage.sage_attn_quantize_frames(d2, q, kk, vv, fq, 1, bufs)
    sage.sage_attn_fwd_quantized(desc, bufs, o)
    torch.cuda.synchronize()
    views = sage.quant_views(desc, ws, bufs)
    Q, K, V = host(q), host(k), host(v)
    mu = quant.k_mean(K)
    np.testing.assert_array_equal(views["k_mean"].cpu().numpy(), mu)
    a = quant.channel_shift(Q, K, mu)
    check_cache_operands(views, Q, K, V, mu, a, F, FS, pv_mode)
    hs = sorted(np.random.default_rng(2000).choice(w.H, 3, replace=False).tolist())
    rows = workloads.sample_rows(w, 96)
    nsplit = sage.sage_attn_kv_splits(desc)
    Qh, Kh, Vh = Q[:, hs], K[:, hs], V[:, hs]
    o64, aux = emulate_cache(Qh, Kh, Vh, pv_mode, w.dtype, F, FS, S, W, kvl, qp, mu[:, hs], a[:, hs], nsplit,
                             rows=rows)
    og = host(o[:, hs])[:, :, rows]
    print(f"  heads {hs} splits {nsplit}:", flush=True)
    assert_close(og, o64, aux, w.dtype, pv_mode, nsplit, max_abs=2e-3)
    ref = attention.attention_fp64(Qh, Kh, Vh, frame_len=F, kv_len=kvl, q_pos0=qp, rows=rows,
                                   sink_frames=S, window_frames=W)
    cs = cosine(og, ref)
    print(f"  cosine vs fp64 windowed attention {cs:.6f}", flush=True)
    assert cs >= 0.999
