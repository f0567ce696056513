"""GPU parity over a seeded sweep of random small shapes, through the C ABI.

Each case draws batch, heads, query and key lengths (not multiples of the
128-row and 64-key tiles), per-batch key lengths, head dim, input type, P.V
mode, an optional frame length with per-batch query positions (the
frame-block-causal mask of streaming generation over a KV cache, Vidu S1
blog, sections "模型架构" and "训练方法"), forced or library-chosen KV splits
and an optional block mask (tile skipping, same blog, section "Infra").  For every case: each quantized operand bit-exact
against the oracle's quantizer, every output element within the derived
bound of gpu_util of the oracle's emulation with the same splits, and the
cosine against float64 attention no worse than the emulation's.

A worst difference-to-bound ratio close to 1 is expected: the emulation is
float64 before the final rounding, and the bound's last term is half a
spacing of the 16-bit output type, which a round-to-nearest output reaches
wherever the other terms are small."""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
from oracle import emulate, attention
from oracle.constants import PV_16, PV_FP8, PV_AUTO
from gpu_util import host, check_quantized, emulate_like_gpu, assert_close, cosine, KERNEL_SLACK

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw_case(seed):
    """One random case; plain data so that the id names it completely."""
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    dt = "bf16" if rng.random() < 0.6 else "f16"
    pv = int(rng.choice([PV_16, PV_FP8]))
    Nq = int(rng.integers(1, 600))
    Nkv = int(rng.integers(1, 1400))
    F = 0
    if rng.random() < 0.5:
        Nkv = max(Nkv, Nq)
        F = int(rng.integers(16, 400))
    kv = [int(rng.integers(max(1, Nq if F else 1), Nkv + 1)) for _ in range(B)]
    if rng.random() < 0.3:
        kv[0] = Nkv                                   # one batch at the full length
    qp = None
    if F and rng.random() < 0.6:
        qp = [int(rng.integers(0, kv[b] - Nq + 1)) for b in range(B)]
    splits = int(rng.choice([0, 0, 1, 2, 3, 5]))
    density = float(rng.choice([0.2, 0.6])) if (rng.random() < 0.35) else 0.0
    qscale = float(rng.choice([1.0, 3.0]))
    return dict(seed=seed, B=B, H=H, d=d, dt=dt, pv=pv, Nq=Nq, Nkv=Nkv, F=F, kv=kv, qp=qp, splits=splits,
                density=density, qscale=qscale)


def case_id(c):
    s = (f"r{c['seed']}-B{c['B']}H{c['H']}q{c['Nq']}k{c['Nkv']}d{c['d']}{c['dt']}"
         f"pv{c['pv']}F{c['F']}s{c['splits']}")
    return s + (f"m{c['density']}" if c["density"] else "")


CASES = [draw_case(i) for i in range(N_CASES)]


def draw_auto_case(i):
    """A random case in the per-head P.V mode, with a x8 K channel in about
    half of the (b,h) pairs, so that both head lists are usually filled."""
    c = draw_case(100 + i)
    c["pv"] = PV_AUTO
    rng = np.random.default_rng(9500 + i)
    c["outliers"] = [(b, h, int(rng.integers(0, c["d"]))) for b in range(c["B"]) for h in range(c["H"])
                     if rng.random() < 0.5]
    return c


AUTO_CASES = [draw_auto_case(i) for i in range(8)]
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _inputs(c):
    g = torch.Generator().manual_seed(7100 + c["seed"])
    dt = TORCH_DT[c["dt"]]
    q = (torch.randn(c["B"], c["H"], c["Nq"], c["d"], generator=g) * c["qscale"]).to(dt)
    k = torch.randn(c["B"], c["H"], c["Nkv"], c["d"], generator=g) + 0.7
    for b, h, ch in c.get("outliers", ()):
        k[b, h, :, ch] *= 8
    k = k.to(dt)
    v = torch.randn(c["B"], c["H"], c["Nkv"], c["d"], generator=g).to(dt)
    M = None
    if c["density"]:
        rng = np.random.default_rng(7200 + c["seed"])
        M = (rng.random((c["B"], c["H"], -(-c["Nq"] // 128), -(-c["Nkv"] // 64))) < c["density"])
        M = M.astype(np.uint8)
    return q, k, v, M


def _run(q, k, v, c, M):
    """Quantize, then the fused kernel, as two calls through the C ABI."""
    o = torch.full_like(q, float("nan"))
    desc = sage.Desc.for_tensors(q, k, v, o, pv_mode=c["pv"], frame_len=c["F"], kv_len=c["kv"],
                                 q_pos0=c["qp"], kv_splits=c["splits"],
                                 block_mask=torch.from_numpy(M).cuda() if M is not None else None)
    ws = sage.new_workspace(desc, q.device)
    bufs = sage.sage_attn_quant_layout(desc, ws)
    sage.sage_attn_quantize(desc, q, k, v, bufs)
    sage.sage_attn_fwd_quantized(desc, bufs, o)
    torch.cuda.synchronize()
    return o, sage.quant_views(desc, ws, bufs), desc


def test_cases_are_varied():
    """The sweep reaches every branch it is meant to: both types, modes, head
    dims, frames on and off, forced splits, masks, ragged key lengths."""
    seen = lambda key: {c[key] for c in CASES}
    assert seen("dt") == {"bf16", "f16"} and seen("pv") == {PV_16, PV_FP8} and seen("d") == {64, 128}
    assert any(c["F"] for c in CASES) and any(not c["F"] for c in CASES)
    assert any(c["splits"] > 1 for c in CASES) and any(c["density"] for c in CASES)
    assert any(c["qp"] is not None for c in CASES)
    assert any(min(c["kv"]) < c["Nkv"] for c in CASES)


@pytest.mark.parametrize("c", CASES + AUTO_CASES, ids=[case_id(c) for c in CASES + AUTO_CASES])
def test_random_shape_parity(lib, c):
    print(f"random case {case_id(c)} kv {c['kv']} q_pos0 {c['qp']}", flush=True)
    q, k, v, M = _inputs(c)
    o, views, desc = _run(q.cuda(), k.cuda(), v.cuda(), c, M)
    Q, K, V = host(q), host(k), host(v)
    check_quantized(views, Q, K, V, c["pv"], c["dt"], c["kv"])
    nsplit = sage.sage_attn_kv_splits(desc)
    if M is None:
        o64, aux = emulate_like_gpu(Q, K, V, c["pv"], c["dt"], desc, c["F"], c["kv"], c["qp"])
    else:
        o64, _, aux = emulate.emulate_block_sparse(Q, K, V, c["pv"], c["dt"], M, nsplit, c["F"], c["kv"],
                                                   c["qp"], slack=KERNEL_SLACK)
    og = host(o)
    assert np.isfinite(og).all()
    print(f"  splits {nsplit}", flush=True)
    assert_close(og, o64, aux, c["dt"], c["pv"], nsplit)
    ref = attention.attention_fp64(Q, K, V, frame_len=c["F"], kv_len=c["kv"], q_pos0=c["qp"], block_mask=M)
    live = np.any(ref != 0, axis=-1)
    if live.any():
        cs, ce = cosine(og[live], ref[live]), cosine(o64[live], ref[live])
        print(f"  cosine vs fp64 {cs:.6f} (emulation {ce:.6f})", flush=True)
        assert cs >= ce - 1e-4
