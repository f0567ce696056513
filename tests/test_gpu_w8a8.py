"""GPU parity of the per-block W8A8 linear layer (Vidu S1 blog, section
"Infra"; TurboDiffusion digests), through the C ABI.

* Codes and scales of X (per row and 128-channel group) and W (per 128 x 128
  tile) are bit-exact against the oracle.
* Y against the oracle's float64 value of the same quantized product: the
  GPU rounds each block's scale fp32(dx dw) once, adds each block into a
  float32 sum with one FMA and adds the bias, which stays within
  (K/128 + 2) 2^-24 (sum of |block terms| + |bias|) of the exact value; the
  16-bit output then adds half a spacing.  Cosine against the unquantized
  float64 product >= 0.999 (the inputs carry x8 activation-channel outliers)."""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
import workloads
from oracle import w8a8
from gpu_util import host, ulp16, cosine

pytestmark = pytest.mark.gpu

DT = {torch.bfloat16: "bf16", torch.float16: "f16"}


def _inputs(M, N, K, dt, seed, outliers=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    if outliers:
        idx = torch.randperm(K, generator=g)[:outliers]
        x[:, idx] *= 8
    w = torch.randn((N, K), generator=g) * 0.05
    b = torch.randn((N,), generator=g) * 0.1
    return x.to(dt), w.to(dt), b.to(dt)


def _gpu(x, w, bias, y=None):
    d = sage.W8A8Desc.for_tensors(x, w, y)
    xq, xs, wq, ws = sage.w8a8_buffers(d, x.device)
    if y is None:
        y = torch.full((x.shape[0], w.shape[0]), float("nan"), dtype=x.dtype, device=x.device)
    sage.sage_w8a8_quantize_weight(d, w, wq, ws)
    sage.sage_w8a8_quantize_act(d, x, xq, xs)
    sage.sage_w8a8_gemm(d, xq, xs, wq, ws, bias, y)
    torch.cuda.synchronize()
    return y, xq, xs, wq, ws


def check_y(yg, y64, mag, bias, K, dtype):
    """Per-element bound above; returns (max |err|, worst excess)."""
    babs = np.abs(np.asarray(bias, np.float64))[None, :] if bias is not None else 0.0
    e32 = (K // 128 + 2) * 2.0 ** -24 * (mag + babs)
    bound = e32 + 0.5 * ulp16(np.abs(y64) + e32, dtype) * (1 + 2.0 ** -8) + 1e-30
    err = np.abs(yg.astype(np.float64) - y64)
    return float(err.max()), float((err - bound).max())


CASES = [
    # (M, N, K, dtype, bias, outlier channels, x row stride pad, y row stride pad)
    (300, 256, 384, torch.bfloat16, True, 4, 0, 0),
    (1, 128, 128, torch.float16, False, 0, 0, 0),
    (517, 640, 1024, torch.bfloat16, True, 10, 64, 24),   # half a feature tile, strided rows
    (128, 512, 2048, torch.float16, True, 20, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"M{c[0]}N{c[1]}K{c[2]}{DT[c[3]]}" for c in CASES])
def test_w8a8_parity(lib, case):
    M, N, K, dt, has_bias, outl, xpad, ypad = case
    print(f"w8a8 case {case[:4]}", flush=True)
    x, w, b = _inputs(M, N, K, dt, M * 7 + N + K, outl)
    x[min(2, M - 1), 128:256] = 0                          # an all-zero activation group
    xs_full = torch.zeros((M, K + xpad), dtype=dt)
    xs_full[:, :K] = x
    xd = xs_full.cuda()[:, :K]
    y = torch.full((M, N + ypad), float("nan"), dtype=dt, device="cuda")[:, :N]
    bias = b.cuda() if has_bias else None
    yg, xq, xsc, wq, wsc = _gpu(xd, w.cuda(), bias, y)
    X, W, B = host(x), host(w), host(b)
    oxq, odx = w8a8.quantize_act(X)
    owq, odw = w8a8.quantize_weight(W)
    np.testing.assert_array_equal(xq.cpu().numpy()[:M], oxq)
    assert not xq.cpu().numpy()[M:].any()
    np.testing.assert_array_equal(xsc.cpu().numpy()[:, :M], odx.T)
    assert not xsc.cpu().numpy()[:, M:].any()
    np.testing.assert_array_equal(wq.cpu().numpy(), owq)
    np.testing.assert_array_equal(wsc.cpu().numpy(), odw)
    y64, mag = w8a8.gemm_exact(oxq, odx, owq, odw, B if has_bias else None)
    mx, excess = check_y(host(yg), y64, mag, B if has_bias else None, K, DT[dt])
    ref = w8a8.linear_fp64(X, W, B if has_bias else None)
    cs = cosine(host(yg), ref)
    print(f"  max-abs vs exact quantized product {mx:.3e} (excess {excess:.2e}); cosine vs fp64 {cs:.6f}",
          flush=True)
    assert excess <= 0
    assert cs >= 0.999
    assert torch.isnan(y.as_strided((M, ypad), (N + ypad, 1), N)).all() if ypad else True  # padding untouched


def test_w8a8_repeatable(lib):
    x, w, b = _inputs(260, 256, 512, torch.bfloat16, 5)
    y1 = _gpu(x.cuda(), w.cuda(), b.cuda())[0]
    y2 = _gpu(x.cuda(), w.cuda(), b.cuda())[0]
    assert torch.equal(y1, y2)


@pytest.mark.slow
def test_w8a8_workload_parity(lib):
    """The linear workload at full size (75600 tokens, 5120 -> 13824) in the
    launch configuration bench.py times: codes and scales bit-exact on
    sampled rows and weight tiles, Y on sampled rows."""
    wl = workloads.get("linear")
    print("workload linear", flush=True)
    t = workloads.make_linear(wl, "cuda")
    x, w, b = t["x"], t["w"], t["bias"]
    yg, xq, xsc, wq, wsc = _gpu(x, w, b)
    rows = workloads.sample_rows(wl, 64)
    X = host(x[rows])
    oxq, odx = w8a8.quantize_act(X)
    np.testing.assert_array_equal(xq[rows].cpu().numpy(), oxq)
    np.testing.assert_array_equal(xsc[:, rows].cpu().numpy(), odx.T)
    W = host(w)
    owq, odw = w8a8.quantize_weight(W)
    np.testing.assert_array_equal(wq.cpu().numpy(), owq)
    np.testing.assert_array_equal(wsc.cpu().numpy(), odw)
    B = host(b)
    y64, mag = w8a8.gemm_exact(oxq, odx, owq, odw, B)
    yr = host(yg[rows])
    mx, excess = check_y(yr, y64, mag, B, wl.K, wl.dtype)
    cs = cosine(yr, w8a8.linear_fp64(X, W, B))
    print(f"  max-abs {mx:.3e} excess {excess:.2e} cosine vs fp64 {cs:.6f}", flush=True)
    assert excess <= 0
    assert cs >= 0.999
