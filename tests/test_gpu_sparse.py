"""GPU parity of block-sparse attention (tiles dropped by a caller-given mask
are skipped: sparse attention built on SageAttention, Vidu S1 blog, section
"Infra"), through the C ABI.

Every output element within the derived bound of gpu_util of the oracle's
emulation with the same KV splits (the batch's chunk grid cut as without a
mask; each tile visits its kept chunks inside its part); rows with no kept
visible key exactly 0; cosine against float64 attention under the same
mask; an all-kept mask gives byte-identical outputs to the dense path."""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
import workloads
from oracle import emulate, attention
from oracle.constants import PV_16, PV_FP8, PV_AUTO
from gpu_util import host, assert_close, cosine, NAME_DT, KERNEL_SLACK

pytestmark = pytest.mark.gpu


def _rand(shape, dtype, seed, offset=0.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) + offset).to(dtype)


def _mask(B, H, Nq, Nkv, density, seed):
    rng = np.random.default_rng(seed)
    return (rng.random((B, H, -(-Nq // 128), -(-Nkv // 64))) < density).astype(np.uint8)


def _emulate(Q, K, V, pv_mode, dtype, M, nsplit, F=0, kv=None, qp=None, rows=None):
    o64, _, aux = emulate.emulate_block_sparse(Q, K, V, pv_mode, dtype, M, nsplit, F, kv, qp, rows=rows,
                                               slack=KERNEL_SLACK)
    return o64, aux


def _run(q, k, v, pv_mode, M, frame_len=0, kv_len=None, q_pos0=None, splits=0):
    o = torch.full_like(q, float("nan"))
    desc = sage.Desc.for_tensors(q, k, v, o, pv_mode=pv_mode, frame_len=frame_len, kv_len=kv_len, q_pos0=q_pos0,
                                 kv_splits=splits,
                                 block_mask=torch.from_numpy(M).cuda() if M is not None else None)
    ws = sage.new_workspace(desc, q.device)
    sage.sage_attn_fwd(desc, q, k, v, o, ws)
    torch.cuda.synchronize()
    return o, desc


CASES = [
    # (B, H, Nq, Nkv, d, dtype, F, kv_len, q_pos0, density, splits)
    (1, 2, 300, 1000, 128, torch.bfloat16, 0, None, None, 0.4, 0),
    (1, 2, 300, 1000, 128, torch.bfloat16, 0, None, None, 0.4, 3),            # forced splits
    (2, 2, 256, 1300, 128, torch.bfloat16, 250, [1300, 900], [1044, 600], 0.5, 0),  # frames, ragged
    (1, 3, 200, 700, 64, torch.float16, 0, None, None, 0.15, 2),              # d 64, empty tiles
    (1, 1, 256, 64 * 1500, 128, torch.bfloat16, 0, [64 * 1500 - 37], None, 0.05, 0),  # long list
]


def _cid(c):
    return f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}{NAME_DT[c[5]]}F{c[6]}p{c[9]}s{c[10]}"


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
@pytest.mark.parametrize("case", CASES, ids=[_cid(c) for c in CASES])
def test_sparse_parity(lib, case, pv_mode):
    B, H, Nq, Nkv, d, dt, F, kv, qp, density, splits = case
    print(f"sparse case {_cid(case)} pv {pv_mode}", flush=True)
    seed = sum(map(ord, _cid(case))) + pv_mode
    q = _rand((B, H, Nq, d), dt, seed)
    k = _rand((B, H, Nkv, d), dt, seed + 1, offset=0.7)
    v = _rand((B, H, Nkv, d), dt, seed + 2)
    M = _mask(B, H, Nq, Nkv, density, seed + 3)
    M[0, 0, 0, :] = 0                      # one query tile with nothing kept
    if M.shape[2] > 1:
        M[0, -1, 1, :] = 0
        M[0, -1, 1, 0] = 1                 # one with a single kept block
    o, desc = _run(q.cuda(), k.cuda(), v.cuda(), pv_mode, M, F, kv, qp, splits)
    nsplit = sage.sage_attn_kv_splits(desc)
    Q, K, V = host(q), host(k), host(v)
    o64, aux = _emulate(Q, K, V, pv_mode, NAME_DT[dt], M, nsplit, F, kv, qp)
    og = host(o)
    zero = ~np.any(o64 != 0, axis=-1)      # rows with no kept visible key
    assert zero[0, 0, :min(128, Nq)].all()
    assert not og[zero].any()
    print(f"  splits {nsplit} zero rows {int(zero.sum())}", flush=True)
    assert_close(og, o64, aux, NAME_DT[dt], pv_mode, nsplit)
    ref = attention.attention_fp64(Q, K, V, frame_len=F, kv_len=kv, q_pos0=qp, block_mask=M)
    cs = cosine(og, ref)
    print(f"  cosine vs fp64 under the mask {cs:.6f} (emulation {cosine(o64, ref):.6f})", flush=True)
    assert cs >= 0.999


@pytest.mark.parametrize("splits", [0, 2])
@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
def test_rows_whose_kept_blocks_lie_in_later_frames(lib, pv_mode, splits):
    """One query tile over two frames (rows 0-63 in frame 2, rows 64-127 in
    frame 3).  Head 0 keeps only frame 3's key block: the rows of frame 2
    have no visible kept key and output 0; head 1 also keeps frame 1's
    block, which every row sees."""
    B, H, Nq, Nkv, d, dt, F = 1, 2, 128, 256, 128, torch.bfloat16, 64
    kv, qp = [256], [128]
    print(f"sparse later-frame blocks pv {pv_mode} splits {splits}", flush=True)
    q = _rand((B, H, Nq, d), dt, 610 + pv_mode)
    k = _rand((B, H, Nkv, d), dt, 611, offset=0.7)
    v = _rand((B, H, Nkv, d), dt, 612)
    M = np.zeros((B, H, 1, 4), dtype=np.uint8)
    M[:, :, 0, 3] = 1
    M[:, 1, 0, 1] = 1
    o, desc = _run(q.cuda(), k.cuda(), v.cuda(), pv_mode, M, F, kv, qp, splits)
    nsplit = sage.sage_attn_kv_splits(desc)
    Q, K, V = host(q), host(k), host(v)
    o64, aux = _emulate(Q, K, V, pv_mode, "bf16", M, nsplit, F, kv, qp)
    og = host(o)
    assert np.isfinite(og).all()
    assert not og[0, 0, :64].any() and not o64[0, 0, :64].any()
    assert og[0, 0, 64:].any() and og[0, 1].any(axis=-1).all()
    print(f"  splits {nsplit}", flush=True)
    assert_close(og, o64, aux, "bf16", pv_mode, nsplit)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8], ids=["pv16", "pvfp8"])
def test_paired_blocks_with_lists_of_different_lengths(lib, pv_mode):
    """One workgroup walks two query blocks, each over its own kept key
    blocks, for as many steps as the longer list has.  Head 0: block 0 keeps
    every key block, block 1 none (its rows output 0); head 1 the other way
    round; head 2: block 0 keeps one key block, block 1 all but one; head 3:
    the last block (rows 256-299) alone in its pair."""
    B, H, Nq, Nkv, d, dt = 1, 4, 300, 1000, 128, torch.bfloat16
    print(f"sparse paired lists pv {pv_mode}", flush=True)
    q = _rand((B, H, Nq, d), dt, 710 + pv_mode)
    k = _rand((B, H, Nkv, d), dt, 711, offset=0.7)
    v = _rand((B, H, Nkv, d), dt, 712)
    M = np.zeros((B, H, 3, 16), dtype=np.uint8)
    M[0, 0, 0, :] = 1
    M[0, 1, 1, :] = 1
    M[0, 2, 0, 5] = 1
    M[0, 2, 1, :] = 1
    M[0, 2, 1, 9] = 0
    M[0, 3, 2, ::3] = 1
    o, desc = _run(q.cuda(), k.cuda(), v.cuda(), pv_mode, M)
    nsplit = sage.sage_attn_kv_splits(desc)
    Q, K, V = host(q), host(k), host(v)
    o64, aux = _emulate(Q, K, V, pv_mode, "bf16", M, nsplit)
    og = host(o)
    assert np.isfinite(og).all()
    assert not og[0, 0, 128:256].any() and not og[0, 1, :128].any() and not og[0, 3, :256].any()
    assert og[0, 0, :128].any(axis=-1).all() and og[0, 1, 128:256].any(axis=-1).all()
    assert og[0, 2, :256].any(axis=-1).all() and og[0, 3, 256:].any(axis=-1).all()
    print(f"  splits {nsplit}", flush=True)
    assert_close(og, o64, aux, "bf16", pv_mode, nsplit)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_all_kept_mask_equals_dense(lib, pv_mode):
    """With every tile kept and one work item per tile, the sparse launch
    visits the same chunks in the same order as the dense one."""
    B, H, Nq, Nkv, d, F = 2, 2, 300, 900, 128, 150
    q = _rand((B, H, Nq, d), torch.bfloat16, 81).cuda()
    k = _rand((B, H, Nkv, d), torch.bfloat16, 82).cuda()
    v = _rand((B, H, Nkv, d), torch.bfloat16, 83).cuda()
    kv, qp = [900, 700], [600, 350]
    ones = np.ones((B, H, 3, 15), np.uint8)
    o1, _ = _run(q, k, v, pv_mode, ones, F, kv, qp, splits=1)
    o2, _ = _run(q, k, v, pv_mode, None, F, kv, qp, splits=1)
    assert torch.equal(o1, o2)


SPARSE_FP8_REASON = ("FP8 P.V on the sparse workload (the large workload's outlier-channel heads) misses "
                     "cosine 0.999 by the scheme itself, as on the large workload: 0.99861 on the bench's sample")


@pytest.mark.slow
@pytest.mark.parametrize("pv_mode", [PV_16, PV_AUTO, pytest.param(PV_FP8, marks=pytest.mark.skip(reason=SPARSE_FP8_REASON))],
                         ids=["pv16", "pvauto", "pvfp8"])
def test_sparse_workload_parity(lib, pv_mode):
    """The sparse workload at full size (the large workload with 25% of its
    tiles kept) in the launch configuration bench.py times; outputs of 3
    seeded heads on sampled rows."""
    w = workloads.get("sparse", pv_mode=pv_mode)
    print(f"workload sparse pv {pv_mode}", flush=True)
    x = workloads.make(w, "cuda")
    q, k, v = x["q"], x["k"], x["v"]
    M = workloads.block_mask(w)
    o = torch.empty_like(q)
    desc = sage.Desc.for_tensors(q, k, v, o, pv_mode=w.pv_mode, block_mask=torch.from_numpy(M).cuda())
    ws = sage.new_workspace(desc, q.device)
    sage.sage_attn_fwd(desc, q, k, v, o, ws)
    torch.cuda.synchronize()
    hs = sorted(np.random.default_rng(3000).choice(w.H, 3, replace=False).tolist())
    rows = workloads.sample_rows(w, 48)
    nsplit = sage.sage_attn_kv_splits(desc)
    Q, K, V = host(q[:, hs]), host(k[:, hs]), host(v[:, hs])
    Mh = M[:, hs]
    o64, aux = _emulate(Q, K, V, w.pv_mode, w.dtype, Mh, nsplit, rows=rows)
    og = host(o[:, hs])[:, :, rows]
    print(f"  heads {hs} splits {nsplit}:", flush=True)
    assert_close(og, o64, aux, w.dtype, w.pv_mode, nsplit, max_abs=2e-3)
    ref = attention.attention_fp64(Q, K, V, rows=rows, block_mask=Mh)
    cs = cosine(og, ref)
    print(f"  cosine vs fp64 under the mask {cs:.6f}", flush=True)
    assert cs >= 0.999
