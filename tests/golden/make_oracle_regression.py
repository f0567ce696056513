"""Write oracle_regression.json: the oracle's results on small seeded cases,
kept so that any later change to the oracle's arithmetic fails
tests/test_oracle_golden.py and has to be made, and justified, on purpose.

These values come from the oracle itself.  They guard it against drift;
they do not pin it (the pins are the closed forms, brute-force cases and
invariants of the test_oracle_* files).  The pages print no operator-level
worked example, so no value stored here is the pages'.  This script calls
only oracle/ and torch's seeded CPU generator (for the inputs).

    python tests/golden/make_oracle_regression.py
"""
import hashlib
import json
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import attention, emulate, quant, w8a8          # noqa: E402
from oracle.constants import PV_16, PV_FP8                   # noqa: E402

OUT = os.path.join(HERE, "oracle_regression.json")

# attention case: ragged against both tile sizes, a frame mask, K offset
ATTN = dict(B=1, H=2, Nq=70, Nkv=150, d=64, frame_len=48, kv_len=[150], q_pos0=[80], seed=2024)
ROWS = [0, 15, 33, 47, 48, 69]
# linear-layer case: a ragged row count, two weight tiles, three channel groups
LIN = dict(M=130, N=256, K=384, seed=2025)
LIN_ROWS = [0, 64, 129]


def attn_inputs(c=ATTN):
    """bf16 Q, K (+0.7), V as float32 arrays, from torch's seeded CPU generator."""
    g = torch.Generator().manual_seed(c["seed"])
    q = torch.randn(c["B"], c["H"], c["Nq"], c["d"], generator=g)
    k = torch.randn(c["B"], c["H"], c["Nkv"], c["d"], generator=g) + 0.7
    v = torch.randn(c["B"], c["H"], c["Nkv"], c["d"], generator=g)
    return tuple(t.to(torch.bfloat16).float().numpy() for t in (q, k, v))


def lin_inputs(c=LIN):
    g = torch.Generator().manual_seed(c["seed"])
    x = torch.randn(c["M"], c["K"], generator=g)
    w = torch.randn(c["N"], c["K"], generator=g) * 0.02
    b = torch.randn(c["N"], generator=g) * 0.1
    return tuple(t.to(torch.bfloat16).float().numpy() for t in (x, w, b))


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def hexes(a):
    return [float(x).hex() for x in np.asarray(a, dtype=np.float64).ravel()]


def attention_record():
    c = ATTN
    Q, K, V = attn_inputs()
    mu = quant.k_mean(K, c["kv_len"])
    a = quant.channel_shift(Q, K, mu, c["kv_len"])
    qc, dq = quant.quantize_q(Q, a)
    kc, dk = quant.quantize_k(K, mu, c["kv_len"], a)
    vc, ve, _ = quant.quantize_v_fp8(V, c["kv_len"])
    rec = {"k_mean": hexes(mu), "chan_shift": np.asarray(a).astype(int).ravel().tolist(),
           "q_codes_sha256": sha(qc.astype(np.int8)), "q_scale": hexes(dq),
           "k_codes_sha256": sha(kc.astype(np.int8)), "k_scale": hexes(dk),
           "v_e4m3_sha256": sha(vc.astype(np.uint8)), "v_e8m0_sha256": sha(ve.astype(np.uint8))}
    kw = dict(frame_len=c["frame_len"], kv_len=c["kv_len"], q_pos0=c["q_pos0"], rows=ROWS)
    for pv, name in ((PV_16, "pv16"), (PV_FP8, "pvfp8")):
        o64 = emulate.emulate_from_inputs(Q, K, V, pv, "bf16", **kw)[0]
        rec[f"emulated_{name}"] = hexes(o64)
    rec["fp64_attention"] = hexes(attention.attention_fp64(Q, K, V, **kw))
    return rec


def linear_record():
    X, W, b = lin_inputs()
    xq, dx = w8a8.quantize_act(X)
    wq, dw = w8a8.quantize_weight(W)
    y = w8a8.gemm_exact(xq, dx, wq, dw, b)[0]
    return {"x_codes_sha256": sha(np.asarray(xq).astype(np.int8)), "x_scale_sha256": sha(np.asarray(dx, np.float32)),
            "w_codes_sha256": sha(np.asarray(wq).astype(np.int8)), "w_scale": hexes(dw),
            "y_rows": hexes(np.asarray(y)[LIN_ROWS])}


def build():
    return {"note": "written by make_oracle_regression.py from the oracle alone: a drift guard, not a pin",
            "attention": {"case": ATTN, "rows": ROWS, **attention_record()},
            "linear": {"case": LIN, "rows": LIN_ROWS, **linear_record()}}


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(build(), f, indent=1)
        f.write("\n")
    print(OUT)
