"""GPU parity on the five workloads at their full sizes, in the launch
configuration bench.py times (library-chosen KV splits).

* Every quantized operand (K mean, channel shifts, Q/K codes and scales, V
  layout or FP8 codes and E8M0 scales) is compared bit-exactly with the oracle
  on the FULL tensors, one batch at a time.
* Outputs are compared on sampled rows (the oracle computes them one by one):
  within max(2e-3, half an output-type spacing) of the emulation with the same
  KV splits, and cosine >= 0.999 against float64 attention over the sample
  for the P.V mode each workload is reported with.
"""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
import workloads
from oracle import attention
from oracle.constants import PV_FP8
from gpu_util import (host, check_quantized, emulate_like_gpu, compare_output, cosine, split_ranges)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# (workload, number of heads sampled for outputs (seeded choice), rows per head)
CASES = [("tiny", None, None), ("small", 3, 96), ("large", 6, 48), ("stream", 3, 96), ("batched", 2, 48)]


@pytest.mark.parametrize("name,heads,R", CASES, ids=[c[0] for c in CASES])
def test_workload_parity(lib, name, heads, R):
    w = workloads.get(name)
    print(f"workload {name}", flush=True)
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
        o64, _ = _emulate(Qh, Kh, Vh, w, kvl[b], qp[b], rows, S)
        o_abs = _emulate(Qh, Kh, np.abs(Vh), w, kvl[b], qp[b], rows, S)[0] if w.pv_mode == PV_FP8 else None
        og = host(o[b:b + 1, hs])
        og = og if rows is None else og[:, :, rows]
        mx, excess, frac, rel, rel_bound = compare_output(og, o64, w.dtype, w.pv_mode, o_abs)
        print(f"  b{b} heads {hs}: max-abs {mx:.2e} excess {excess:.2e} beyond-rounding {frac:.2e} "
              f"rel-L2 {rel:.2e}", flush=True)
        assert excess <= 0
        assert rel <= rel_bound
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
    splits = split_ranges(kv_b, S) if S > 1 else None
    return emulate.emulate_from_inputs(Q, K, V, w.pv_mode, w.dtype, frame_len=w.frame_len, kv_len=[kv_b],
                                       q_pos0=[qp_b], rows=rows, splits=splits)
