"""GPU parity of the streaming steps over a quantize-once frame cache at full
size, in the launch configuration bench.py times (Vidu S1 blog, section
"Infra": each step quantizes only the new frame and attends over the cache).

stream-cache: B1 H24, 17 frames of 2040 tokens at a stride of 2048 slots,
queries = frame 16.  batched-cache: B8 H24, each session with its own cache
of 5-33 frames, queries = each session's last frame.  As in bench.py: the
whole cache is quantized once (the library computes the mean and the
channel exponents, then frozen), then one step -- the current frame of
every session and the queries appended (sage_attn_quantize_frames or its
batched form), and the fused kernel with the library-chosen KV splits.

Checks on two seeded heads of every session: the frozen mean and
exponents, the Q and K codes and scales and the V layout (16-bit) or e4m3
codes and E8M0 scales (FP8) bit-exact against the oracle over every cache
slot; outputs on sampled rows within the derived bound of gpu_util of the
oracle's frame-cache emulation with the same splits and max-abs <= 2e-3;
cosine >= 0.999 against float64 attention over the sample."""

import numpy as np
import pytest
import torch

import bench
import bit_quantized_attention_sage_amd as sage
import workloads
from oracle import attention, codecs, emulate, quant
from oracle.constants import BK, PV_16, PV_FP8
from gpu_util import host, assert_close, cosine, KERNEL_SLACK

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _check_operands(views, hs, Q, K, V, mu, a, w, kvl, pv_mode):
    F, FS, n = w.frame_len, w.frame_stride, w.Nkv
    np.testing.assert_array_equal(views["k_mean"][:, hs].cpu().numpy(), mu)
    np.testing.assert_array_equal(views["chan_shift"][:, hs].cpu().numpy(), a.astype(np.int8))
    qc, dq = quant.quantize_q(Q, a)
    np.testing.assert_array_equal(views["q_codes"][:, hs].cpu().numpy()[:, :, :w.Nq], qc)
    np.testing.assert_array_equal(views["q_scale"][:, hs].cpu().numpy()[:, :, :dq.shape[2]], dq)
    kc, dk = quant.quantize_k_frames(K, mu, a, F, FS, n_slots=n, kv_len=kvl)
    np.testing.assert_array_equal(views["k_codes"][:, hs].cpu().numpy()[:, :, :n], kc)
    np.testing.assert_array_equal(views["k_scale"][:, hs].cpu().numpy()[:, :, :n // BK], dk)
    B, H2, d = Q.shape[0], len(hs), Q.shape[3]
    untiled = views["v_t"][:, hs].cpu().permute(0, 1, 2, 4, 3).reshape(B, H2, -1, d).numpy()
    if pv_mode == PV_FP8:
        vc, ve = quant.quantize_v_fp8_frames(V, F, FS, n_slots=n, kv_len=kvl)
        np.testing.assert_array_equal(untiled.astype(np.uint8)[:, :, :n], vc)
        ge = views["v_e8m0"][:, hs].cpu().numpy()
        nch = ge.shape[2]
        g5 = ge.reshape(B, H2, nch, 2, 32, 4)[..., : d // 32].transpose(0, 1, 2, 3, 5, 4).reshape(B, H2, 2 * nch, d)
        np.testing.assert_array_equal(g5[:, :, :n // 32], (ve + 127).astype(np.uint8))
    else:
        # (keys past a session's kv_len are zero in the inputs, so whole
        # frames placed into their slots are that session's cache)
        ref = codecs.bf16_bits(quant.to_frame_slots(V, F, FS, n_slots=n))
        np.testing.assert_array_equal(untiled.view(np.uint16)[:, :, :n], ref)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
@pytest.mark.parametrize("name", ["stream-cache", "batched-cache"])
def test_cache_workload_parity(lib, name, pv_mode):
    w = workloads.get(name, pv_mode=pv_mode)
    print(f"workload {name} pv {pv_mode}", flush=True)
    x = workloads.make(w, "cuda")
    q, k, v = x["q"], x["k"], x["v"]
    o = torch.empty_like(q)
    kvl, qp = w.kv_lens(), w.q_pos0s()
    desc = sage.Desc.for_tensors(q, k, v, o, nkv=w.Nkv, pv_mode=pv_mode, frame_len=w.frame_len,
                                 frame_stride=w.frame_stride, kv_len=kvl, q_pos0=qp)
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)          # the cache, once
    append, attend = bench.step_parts(sage, w, desc, q, k, v, o, bufs, None)
    append()                                              # one step
    attend()
    torch.cuda.synchronize()
    views = sage.quant_views(desc, ws, bufs)
    hs = sorted(np.random.default_rng(3000 + pv_mode).choice(w.H, 2, replace=False).tolist())
    Q, K, V = host(q[:, hs]), host(k[:, hs]), host(v[:, hs])
    mu = quant.k_mean(K, kvl)
    a = quant.channel_shift(Q, K, mu, kvl)
    _check_operands(views, hs, Q, K, V, mu, a, w, kvl, pv_mode)
    rows = workloads.sample_rows(w, 64)
    nsplit = sage.sage_attn_kv_splits(desc)
    o64, _, aux = emulate.emulate_frame_cache(Q, K, V, pv_mode, w.dtype, w.frame_len, w.frame_stride, 0, 0,
                                              kvl, qp, mu, a, nsplit, rows=rows, slack=KERNEL_SLACK)
    og = host(o[:, hs])[:, :, rows]
    print(f"  heads {hs} splits {nsplit}:", flush=True)
    assert_close(og, o64, aux, w.dtype, pv_mode, nsplit, max_abs=2e-3)
    ref = attention.attention_fp64(Q, K, V, frame_len=w.frame_len, kv_len=kvl, q_pos0=qp, rows=rows)
    cs = cosine(og, ref)
    print(f"  cosine vs fp64 {cs:.6f} (emulation {cosine(o64, ref):.6f})", flush=True)
    assert cs >= 0.999
