"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same inputs, compare.  Test infrastructure only."""

import numpy as np
import torch

import bit_quantized_attention_sage_amd as sage
from oracle import quant, emulate, attention, codecs
from oracle.constants import BK, PV_FP8

SAGE_DT = {torch.float16: sage.SAGE_F16, torch.bfloat16: sage.SAGE_BF16}
NAME_DT = {torch.float16: "f16", torch.bfloat16: "bf16"}


def run_gpu(q, k, v, pv_mode, frame_len=0, kv_len=None, q_pos0=None, kv_splits=0, sm_scale=0.0,
            k_mean_in=None):
    """Quantize + attend through the C ABI; returns (out, quantized views, desc)."""
    o = torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o, pv_mode=pv_mode, frame_len=frame_len, kv_len=kv_len,
                                 q_pos0=q_pos0, kv_splits=kv_splits, sm_scale=sm_scale,
                                 k_mean_in=k_mean_in)
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)
    sage.sage_attn_fwd_quantized(desc, bufs, o)
    torch.cuda.synchronize()
    return o, sage.quant_views(desc, ws, bufs), desc, ws, bufs


def host(t):
    return t.detach().float().cpu().numpy()


def split_ranges(kv_len_b, S):
    n = -(-int(kv_len_b) // BK)
    return [(s * n // S, (s + 1) * n // S) for s in range(S)]


def check_quantized(views, Q, K, V, pv_mode, dtype, kv_len=None, mu_in=None):
    """Bit-exact comparison of every quantized operand with the oracle."""
    B, H, Nq, d = Q.shape
    Nkv = K.shape[2]
    mu = quant.k_mean(K, kv_len) if mu_in is None else mu_in
    if mu_in is None:
        np.testing.assert_array_equal(views["k_mean"].cpu().numpy(), mu)
    a = quant.channel_shift(Q, K, mu, kv_len)
    np.testing.assert_array_equal(views["chan_shift"].cpu().numpy().astype(np.int64), a)
    qc, dq = quant.quantize_q(Q, a)
    kc, dk = quant.quantize_k(K, mu, kv_len, a)
    gq = views["q_codes"].cpu().numpy()
    np.testing.assert_array_equal(gq[:, :, :Nq], qc)
    assert not gq[:, :, Nq:].any()
    np.testing.assert_array_equal(views["q_scale"].cpu().numpy()[:, :, :dq.shape[2]], dq)
    gk = views["k_codes"].cpu().numpy()
    np.testing.assert_array_equal(gk[:, :, :Nkv], kc)
    assert not gk[:, :, Nkv:].any()
    gks = views["k_scale"].cpu().numpy()
    np.testing.assert_array_equal(gks[:, :, :dk.shape[2]], dk)
    assert not gks[:, :, dk.shape[2]:].any()
    vt = views["v_t"].cpu()
    untiled = vt.permute(0, 1, 2, 4, 3).reshape(B, H, -1, d)
    if pv_mode == PV_FP8:
        vc, ve, e8 = quant.quantize_v_fp8(V, kv_len)
        g = untiled.numpy().astype(np.uint8)
        np.testing.assert_array_equal(g[:, :, :Nkv], vc)
        assert not g[:, :, Nkv:].any()
        # per chunk: byte [32k + r][cb] is block 2*chunk + k, channel 32*cb + r
        ge = views["v_e8m0"].cpu().numpy()                      # [B,H,nch,64,4]
        nch = ge.shape[2]
        g5 = ge.reshape(B, H, nch, 2, 32, 4)[..., : d // 32]     # [B,H,nch,k,r,cb]
        ge_std = g5.transpose(0, 1, 2, 3, 5, 4).reshape(B, H, 2 * nch, d)
        np.testing.assert_array_equal(ge_std[:, :, :e8.shape[2]], e8)
    else:
        g = untiled.numpy().view(np.uint16)
        vv = V.copy()
        kvl = kv_len if kv_len is not None else [Nkv] * B
        for b in range(B):
            vv[b, :, kvl[b]:] = 0
        ref_bits = codecs.bf16_bits(vv) if dtype == "bf16" else vv.astype(np.float16).view(np.uint16)
        np.testing.assert_array_equal(g[:, :, :Nkv], ref_bits)
        assert not g[:, :, Nkv:].any()
    return mu


def emulate_like_gpu(Q, K, V, pv_mode, dtype, desc, frame_len=0, kv_len=None, q_pos0=None, rows=None,
                     sm_scale=None, mu=None):
    """The oracle's emulation with the same KV split boundaries as the GPU launch."""
    B = Q.shape[0]
    S = sage.sage_attn_kv_splits(desc)
    kvl = list(kv_len) if kv_len is not None else [K.shape[2]] * B
    qp = list(q_pos0) if q_pos0 is not None else None
    outs = []
    for b in range(B):
        splits = split_ranges(kvl[b], S) if S > 1 else None
        o64, _ = emulate.emulate_from_inputs(
            Q[b:b + 1], K[b:b + 1], V[b:b + 1], pv_mode, dtype, sm_scale=sm_scale, frame_len=frame_len,
            kv_len=[kvl[b]], q_pos0=[qp[b]] if qp else None, rows=rows, splits=splits,
            mu=None if mu is None else mu[b:b + 1])
        outs.append(o64)
    return np.concatenate(outs, axis=0)


def ulp16(x, dtype):
    """Spacing of the 16-bit output type at |x| (bf16: 8-bit significand,
    fp16: 11-bit significand with subnormal spacing 2^-24)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    if dtype == "bf16":
        return np.exp2(e - 7)
    return np.exp2(np.maximum(e, -14) - 10)


# Accumulation of the scaled FP8 matrix-core products (measured on gfx950 with
# one-wave probes of v_mfma_scale_f32_32x32x64_f8f6f4): products are summed in
# groups of 8 consecutive K indices, aligned to the group's largest product
# with 13 fractional bits; bits below that are dropped (terms 2^-14 of the
# group maximum vanish, terms 2^-13 survive).  A group therefore loses less
# than 7 * 2^-13 of its largest |product|.  The 16-bit MFMAs showed no such
# loss (float32 rounding of the running sum only).
FP8_ACC = 7 * 2.0 ** -13


def compare_output(out_gpu, o64, dtype, pv_mode, o_abs=None):
    """Compare the GPU output with the emulation's unrounded float64 result.

    The GPU output is that value computed in float32 and rounded (RNE) to the
    16-bit output type, so each element may differ by half a spacing of that
    type (plus float32 accumulation noise); the acceptance bar is max-abs
    <= 2e-3, widened to that half spacing where the type itself is coarser.
    In FP8 mode the matrix cores' grouped accumulation (FP8_ACC) perturbs
    acc = sum p~ v and l = sum p~ by at most FP8_ACC * sum p~ |v| and
    FP8_ACC * l, so O = acc / l moves by at most FP8_ACC * (a + |O|) with
    a = sum p~ |v| / l, which is the emulation's output for |V| (o_abs); that
    much is added to the bar when o_abs is given.
    Returns (max_abs, worst excess over the per-element bound, fraction of
    elements beyond the tight rounding-only bound, relative L2 error, its
    bound: ulp/sqrt(12) of the type, plus 1e-3 in FP8 mode for the grouped
    accumulation)."""
    diff = np.abs(out_gpu - o64)
    half = 0.5 * ulp16(o64, dtype) * (1 + 2.0 ** -8)
    tol = np.maximum(2e-3, half + 1e-6)
    if pv_mode == PV_FP8 and o_abs is not None:
        tol = np.maximum(2e-3, half + 1e-6 + FP8_ACC * (o_abs + np.abs(o64)))
    excess = float((diff - tol).max())
    tight = half + 1e-5 * float(np.abs(o64).max())
    frac = float(np.mean(diff > tight))
    rel = float(np.linalg.norm(out_gpu - o64) / max(np.linalg.norm(o64), 1e-30))
    rel_bound = (2.0 ** -7 if dtype == "bf16" else 2.0 ** -10) / np.sqrt(12) * 1.1
    if pv_mode == PV_FP8:
        rel_bound += 1e-3
    return float(diff.max()), excess, frac, rel, rel_bound


def cosine(a, b):
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))
