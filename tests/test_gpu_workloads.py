"""GPU parity on the five workloads at their full sizes, in the launch
configuration bench.py times (library-chosen KV splits).

* Every quantized operand (K mean, channel shifts, Q/K codes and scales, V
  layout or FP8 codes and E8M0 scales) is compared bit-exactly with the oracle
  on the FULL tensors, one batch at a time.
* Outputs are compared on sampled rows (the oracle computes them one by one):
  every element within the derived bound of gpu_util of the emulation with
  the same KV splits, max-abs <= 2e-3 against it, and cosine >= 0.999
  against float64 attention over the sample, for the P.V mode each workload
  is reported with and for the other mode where the scheme reaches 0.999.
"""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
import workloads
from oracle import attention
from oracle.constants import PV_FP8
from gpu_util import host, check_quantized, assert_close, cosine, KERNEL_SLACK

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# (workload, P.V mode (the workload's own first), heads sampled for outputs
# (seeded choice), rows per head)
LARGE_FP8_REASON = ("FP8 P.V on the large workload misses cosine 0.999 by the scheme itself: the "
                    "emulation reaches 0.99865 on 40 heads x 32 rows (kernel 0.99794 on its outlier "
                    "heads 0-1); INT8 scores of the 24 outlier-channel heads cost 7.5e-4 of 1 - cos and "
                    "e4m3 P and V another 7e-4 (accuracy decomposition in the design notes)")
CASES = [("tiny", 1, None, None), ("tiny", 0, None, None), ("small", 1, 3, 96), ("small", 0, 2, 64),
         ("large", 2, 6, 48), ("large", 0, 6, 48),
         pytest.param("large", 1, 4, 48, marks=pytest.mark.skip(reason=LARGE_FP8_REASON)),
         ("stream", 1, 3, 96), ("stream", 0, 2, 64), ("batched", 1, 2, 48), ("batched", 0, 2, 32)]


def _cid(c):
    c = c.values if hasattr(c, "values") else c
    return c[0] + {0: "-pv16", 1: "-pvfp8", 2: "-pvauto"}[c[1]]


@pytest.mark.parametrize("name,pv,heads,R", CASES, ids=[_cid(c) for c in CASES])
def test_workload_parity(lib, name, pv, heads, R):
    w = workloads.get(name, pv_mode=pv)
    print(f"workload {name} pv_mode {w.pv_mode}", flush=True)
    x = workloads.make(w, "cuda")
    q, k, v = x["q"], x["k"], x["v"]
    o = torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o, pv_mode=w.pv_mode, frame_len=w.frame_len,
                                 kv_len=w.kv_len, q_pos0=w.q_pos0)
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)
    sage.sage_attn_fwd_quantized(desc, bufs, o)
    torch.cuda.synchronize()
    views = sage.quant_views(desc, ws, bufs)
    kvl, qp = w.kv_lens(), w.q_pos0s()
    rows = workloads.sample_rows(w, R) if R else None
    S = sage.sage_attn_kv_splits(desc)
    num = den_a = den_b = 0.0
    for b in range(w.B):
        # full-tensor bit-exact quantized operands of batch b
        vb = {key: t[b:b + 1] for key, t in views.items()}
        Q, K, V = host(q[b:b + 1]), host(k[b:b + 1]), host(v[b:b + 1])
        check_quantized(vb, Q, K, V, w.pv_mode, w.dtype, [kvl[b]])
        # sampled outputs of a few heads
        hs = list(range(w.H)) if heads is None else \
            sorted(np.random.default_rng(1000 + b).choice(w.H, heads, replace=False).tolist())
        if name == "batched" and b not in (0, w.B - 1):
            continue
        Qh, Kh, Vh = Q[:, hs], K[:, hs], V[:, hs]
        o64, aux = _emulate(Qh, Kh, Vh, w, kvl[b], qp[b], rows, S)
        og = host(o[b:b + 1, hs])
        og = og if rows is None else og[:, :, rows]
        print(f"  b{b} heads {hs}:", flush=True)
        assert_close(og, o64, aux, w.dtype, w.pv_mode, S, max_abs=2e-3)
        ref = attention.attention_fp64(Qh, Kh, Vh, frame_len=w.frame_len, kv_len=[kvl[b]],
                                       q_pos0=[qp[b]], rows=rows)
        num += float((og.astype(np.float64) * ref).sum())
        den_a += float((og.astype(np.float64) ** 2).sum())
        den_b += float((ref ** 2).sum())
        del Q, K, V
    cos = num / np.sqrt(den_a * den_b)
    print(f"  cosine vs fp64 over the sample: {cos:.6f}", flush=True)
    assert cos >= 0.999


def _emulate(Q, K, V, w, kv_b, qp_b, rows, S):
    from oracle import emulate
    o64, _, aux = emulate.emulate_from_inputs(Q, K, V, w.pv_mode, w.dtype, frame_len=w.frame_len,
                                              kv_len=[kv_b], q_pos0=[qp_b], rows=rows,
                                              splits=emulate.split_ranges(kv_b, S), slack=KERNEL_SLACK)
    return o64, aux
