"""GPU parity of the per-head P.V mode (SAGE_PV_AUTO) through the C ABI.

Each (b,h) runs FP8 P.V when its channel-balance exponents are all 0 and
16-bit P.V when some channel was moved (an outlier channel of K); the library
lists the heads of each mode on the device and runs one launch per mode.
Checked: every quantized operand bit-exact (V per head in its own format, in
its 16-bit sized slot), every output element within the derived bound of
gpu_util of the oracle's emulation with each head in the mode the oracle's
rule gives it, cosine >= 0.999 against float64 attention -- with ragged
batches, frames, forced KV splits, a block mask, and the degenerate lists
(every head in one mode, so the other launch has no work).
"""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
from oracle import attention, emulate, quant
from oracle.constants import PV_16, PV_FP8, PV_AUTO
from gpu_util import (run_gpu, host, check_quantized, emulate_like_gpu, assert_close, cosine, NAME_DT,
                      KERNEL_SLACK)

pytestmark = pytest.mark.gpu


def _inputs(B, H, Nq, Nkv, d, dt, seed, outliers, kv_len=None):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g)
    k = torch.randn((B, H, Nkv, d), generator=g) + torch.randn((1, H, 1, d), generator=g)
    v = torch.randn((B, H, Nkv, d), generator=g)
    for b, h, c in outliers:
        k[b, h, :, c] *= 8
    if kv_len is not None:
        for b in range(B):
            k[b, :, kv_len[b]:] = 0
            v[b, :, kv_len[b]:] = 0
    return q.to(dt), k.to(dt), v.to(dt)


CASES = [
    # (B, H, Nq, Nkv, d, dtype, F, kv_len, q_pos0, splits, outlier (b, h, channel)s)
    (1, 4, 777, 777, 128, torch.bfloat16, 0, None, None, 0, [(0, 1, 5), (0, 2, 77)]),
    (2, 3, 300, 1000, 64, torch.float16, 250, [1000, 731], None, 3, [(0, 0, 9), (1, 2, 40), (1, 2, 41)]),
    (1, 2, 520, 1500, 128, torch.bfloat16, 0, None, None, 2, [(0, 0, 3), (0, 1, 100)]),   # all 16-bit
    (2, 2, 256, 640, 128, torch.bfloat16, 0, [640, 333], None, 0, []),                      # all FP8
]


def _cid(c):
    return f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}{NAME_DT[c[5]]}F{c[6]}s{c[9]}o{len(c[10])}"


@pytest.mark.parametrize("case", CASES, ids=[_cid(c) for c in CASES])
def test_auto_parity(lib, case):
    B, H, Nq, Nkv, d, dt, F, kv_len, q_pos0, splits, outl = case
    print(f"auto case {_cid(case)}", flush=True)
    q, k, v = _inputs(B, H, Nq, Nkv, d, dt, sum(map(ord, _cid(case))), outl, kv_len)
    out, views, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), PV_AUTO, F, kv_len, q_pos0, splits)
    Q, K, V = host(q), host(k), host(v)
    check_quantized(views, Q, K, V, PV_AUTO, NAME_DT[dt], kv_len)
    o64, aux = emulate_like_gpu(Q, K, V, PV_AUTO, NAME_DT[dt], desc, F, kv_len, q_pos0)
    want = np.full((B, H), PV_FP8)
    for b, h, _ in outl:
        want[b, h] = PV_16
    np.testing.assert_array_equal(aux["pv_modes"], want)
    og = host(out)
    print(f"  modes {aux['pv_modes'].tolist()} splits {aux['splits']}", flush=True)
    assert_close(og, o64, aux, NAME_DT[dt], PV_AUTO)
    ref = attention.attention_fp64(Q, K, V, frame_len=F, kv_len=kv_len, q_pos0=q_pos0)
    cs = cosine(og, ref)
    print(f"  cosine vs fp64 {cs:.6f} (emulation {cosine(o64, ref):.6f})", flush=True)
    assert cs >= 0.999


@pytest.mark.parametrize("single", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
def test_auto_matches_the_single_mode_paths(lib, single):
    """Where the rule puts every head in one mode, the per-head path (head
    list + that mode's launch; the other launch has no heads) writes exactly
    the bytes of the single-mode call."""
    outl = [(0, 0, 1), (0, 1, 2), (0, 2, 3)] if single == PV_16 else []
    q, k, v = (t.cuda() for t in _inputs(1, 3, 400, 900, 128, torch.bfloat16, 91, outl))
    oa = run_gpu(q, k, v, PV_AUTO)[0]
    os_ = run_gpu(q, k, v, single)[0]
    assert torch.equal(oa.view(torch.int16), os_.view(torch.int16))


def test_auto_block_sparse(lib):
    """Per-head mode under a block mask (the sparse path), forced splits."""
    B, H, Nq, Nkv, d = 1, 3, 300, 1000, 128
    q, k, v = _inputs(B, H, Nq, Nkv, d, torch.bfloat16, 17, [(0, 2, 64)])
    M = (np.random.default_rng(5).random((B, H, 3, 16)) < 0.4).astype(np.uint8)
    M[0, 0, 0, :] = 0
    o = torch.full_like(q, float("nan")).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    desc = sage.Desc.for_tensors(qd, kd, vd, o, pv_mode=PV_AUTO, kv_splits=2,
                                 block_mask=torch.from_numpy(M).cuda())
    ws = sage.new_workspace(desc, qd.device)
    sage.sage_attn_fwd(desc, qd, kd, vd, o, ws)
    torch.cuda.synchronize()
    Q, K, V = host(q), host(k), host(v)
    o64, _, aux = emulate.emulate_block_sparse(Q, K, V, PV_AUTO, "bf16", M, 2, slack=KERNEL_SLACK)
    np.testing.assert_array_equal(aux["pv_modes"], [[PV_FP8, PV_FP8, PV_16]])
    og = host(o)
    assert_close(og, o64, aux, "bf16", PV_AUTO, 2)
    ref = attention.attention_fp64(Q, K, V, block_mask=M)
    assert cosine(og, ref) >= 0.999


def test_auto_many_heads(lib):
    """More (b,h) pairs than the head-list kernel's 256 threads (B 2 x H 150 =
    300): its running counts carry over from one pass of 256 heads to the
    next, in batch order (the longer batch first)."""
    B, H, N, d = 2, 150, 128, 64
    outl = [(0, 3, 1), (0, 149, 2), (1, 0, 3), (1, 105, 4), (1, 106, 5), (1, 149, 63)]
    kv_len = [100, 128]                      # batch 1 is listed first
    q, k, v = _inputs(B, H, N, N, d, torch.float16, 33, outl, kv_len)
    out, views, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), PV_AUTO, 0, kv_len, None, 0)
    Q, K, V = host(q), host(k), host(v)
    check_quantized(views, Q, K, V, PV_AUTO, "f16", kv_len)
    o64, aux = emulate_like_gpu(Q, K, V, PV_AUTO, "f16", desc, 0, kv_len)
    # (128 Gaussian tokens can by chance give some other channel a range
    # ratio of 2: the oracle's modes decide, and V's layout and the outputs
    # show that the GPU took the same ones)
    assert all(aux["pv_modes"][b, h] == PV_16 for b, h, _ in outl)
    print(f"  16-bit heads: {int((aux['pv_modes'] == PV_16).sum())} of {B * H}", flush=True)
    assert_close(host(out), o64, aux, "f16", PV_AUTO)


def test_auto_degenerate_heads(lib):
    """Heads whose exponents are 0 by definition take FP8 P.V: Q = 0 (every
    row's output is the mean of the visible V^ rows) and K constant along
    the keys (K~ = 0: zero codes and scales); beside them one head with an
    outlier channel (16-bit P.V) and one ordinary head (FP8)."""
    B, H, N, d = 1, 4, 333, 128
    q, k, v = _inputs(B, H, N, N, d, torch.bfloat16, 71, [(0, 2, 9)])
    q[0, 0] = 0
    k[0, 1] = k[0, 1, :1].expand(N, d)
    out, views, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), PV_AUTO)
    Q, K, V = host(q), host(k), host(v)
    check_quantized(views, Q, K, V, PV_AUTO, "bf16")
    assert not views["k_codes"][0, 1].any()
    o64, aux = emulate_like_gpu(Q, K, V, PV_AUTO, "bf16", desc)
    np.testing.assert_array_equal(aux["pv_modes"], [[PV_FP8, PV_FP8, PV_16, PV_FP8]])
    og = host(out)
    assert_close(og, o64, aux, "bf16", PV_AUTO)
    # Q = 0: every row is the mean of the (FP8-rounded) V rows
    vhat = quant.dequant_v_fp8(*quant.quantize_v_fp8(V)[:2])[0, 0]
    np.testing.assert_allclose(o64[0, 0], np.broadcast_to(vhat.mean(axis=0), (N, d)), rtol=0, atol=1e-12)
