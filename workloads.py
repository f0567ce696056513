"""Seeded synthetic inputs shaped like video-DiT attention.

This module only draws random numbers; it holds none of the quantized
attention's arithmetic.  Both the CPU oracle (through the tests and the bench's
CPU leg) and the HIP library consume what it produces.

The pages' workloads are video-diffusion transformers: 5-second 480p/720p
clips (TurboDiffusion digests on the reportify page) and a 540p frame-by-frame
stream with a KV cache (Vidu S1 blog, sections "Infra" and "评测 benchmark").
Their latents and models are not available, so these seeded Gaussian tensors
stand in for them, with the token grids of such clips:

  tiny     B1 H2  N 1024             d64  fp16  K += per-channel offset ~ N(0, 2^2)
  small    B1 H12 N 32760 (21x30x52) d128 bf16  K += per-channel bias ~ N(0, 3)
  large    B1 H40 N 75600 (21x45x80) d128 bf16  51 of the 40*128 (head, channel)
                                                 K channels scaled x8 (1%)
  stream   B1 H24 Nq 2040 (34x60 frame), Nkv 34680 = 16 cached frames + itself,
           d128 bf16, frame-block-causal mask with F = 2040
  batched  B8 H24 Nq 2040, each session's cache L_b ~ U{4..32} frames plus its
           own frame (kv_len = (L_b+1)*2040), KV allocated for 33 frames,
           d128 bf16, frame-block-causal
  window   streaming step over a frame cache (Vidu S1 blog, section "Infra":
           a fixed window of sink frames, recent history and the current
           frame): B1 H24 d128 bf16, 2040-token frames at a stride of 2048
           cache slots, 48 frames allocated, frames 0..40 cached, the
           queries are frame 40; 1 sink frame and a 16-frame window, so each
           query sees 18 frames (36720 keys).  The pages give no window
           length; 16 frames matches the stream workload's history.
  sparse   the large workload with a block mask over its (128-query,
           64-key) tiles keeping exactly 25% of each query tile's key
           blocks (296 of 1182), drawn uniformly and independently per
           (head, query tile) -- a stand-in
           for the sparse branch of sparse attention built on SageAttention
           (Vidu S1 blog, section "Infra"), whose predictor the pages do not
           give.
  linear   the per-block W8A8 linear layer on the large workload's tokens:
           X [75600, 5120] (1% of channels x8, as activation outliers),
           W [13824, 5120] ~ N(0, 0.02^2), bias ~ N(0, 0.1^2), bf16 -- the
           shape of a 14B-class video DiT's feed-forward up-projection (the
           pages' 14B text/image-to-video models; TurboDiffusion digests).
  stream-cache, batched-cache
           the stream and batched workloads over a quantize-once frame
           cache (2048-slot frame stride, every earlier frame visible): a
           step appends each session's current frame (its new keys and
           values) and quantizes the queries, then attends over the cache
           -- the cache is not re-quantized every step.

P.V mode of each workload (bench.py's default for it): the fastest mode that
meets both accuracy bars (cosine >= 0.999 against float64 attention, max-abs
<= 2e-3 against the oracle's emulation) on the workload, measured at full
size -- FP8 everywhere except large and sparse, whose outlier-channel heads
keep FP8 below 0.999: they run the per-head mode (FP8 on the heads without
an outlier channel, 16-bit on the others).  Any mode can be asked for.

Values are N(0,1) float32, then rounded to the 16-bit dtype.  Each (tensor,
batch, head) slice has its own seed, so any subset of heads can be drawn on
its own; the small per-config draws (offsets, outlier channels, cache
lengths) use numpy's default_rng and do not depend on the device.
"""

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

FRAME = 2040  # tokens per 34x60 latent frame


@dataclass
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    d: int
    dtype: str                 # 'f16' | 'bf16'
    pv_mode: int               # 0: 16-bit P.V, 1: FP8 P.V, 2: per head (FP8 unless an outlier channel)
    frame_len: int = 0
    kv_len: list = None        # per batch; None -> Nkv for all
    q_pos0: list = None        # per batch; None -> default
    seed: int = 0
    k_offset_std: float = 0.0
    outlier_frac: float = 0.0
    outlier_gain: float = 8.0
    frame_stride: int = 0      # > 0: K/V live in a frame cache of Nkv slots
    sink_frames: int = 0
    window_frames: int = 0
    block_density: float = 0.0  # > 0: block mask keeping this share of tiles
    extra: dict = field(default_factory=dict)

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    def kv_lens(self):
        return list(self.kv_len) if self.kv_len is not None else [self.Nkv] * self.B

    @property
    def kv_tokens(self):
        """Rows of the K and V input tensors: Nkv, or with a frame cache the
        longest batch's tokens (whole frames, before the slot layout)."""
        return max(self.kv_lens()) if self.frame_stride else self.Nkv

    def q_pos0s(self):
        if self.q_pos0 is not None:
            return list(self.q_pos0)
        if self.frame_len == 0:
            return [0] * self.B
        return [kv - self.Nq for kv in self.kv_lens()]

    def row_keys(self, b, rows=None, h=None):
        """Visible keys of each query row (all rows when None) of batch b; with
        a block mask, of head h (summed over heads when h is None)."""
        kv, qp = self.kv_lens()[b], self.q_pos0s()[b]
        i = np.arange(self.Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
        if self.block_density:
            M = block_mask(self)[b]                                    # [H, nqt, nkc]
            end = np.minimum(kv, ((qp + i) // self.frame_len + 1) * self.frame_len) if self.frame_len \
                else np.full(len(i), kv, dtype=np.int64)
            # kept keys of a row: the kept blocks' keys below its end; rows of
            # one query tile with the same end share the count
            nkc = M.shape[2]
            pairs, inv = np.unique(np.stack([i // 128, end]), axis=1, return_inverse=True)
            width = np.minimum(64, np.maximum(0, pairs[1][:, None] - 64 * np.arange(nkc)[None, :]))
            hs = range(self.H) if h is None else [h]
            per = sum((M[hh][pairs[0]].astype(np.int64) * width).sum(axis=1) for hh in hs)
            return per[np.ravel(inv)].astype(np.int64)
        if self.window_frames:
            F = self.frame_len
            fq = (qp + i) // F
            n = np.zeros(len(i), np.int64)
            for f in range(int(fq.max()) + 1):
                seen = (f <= fq) & ((f < self.sink_frames) | (f >= fq - self.window_frames))
                n += seen * max(0, min(F, kv - f * F))
            return n
        if self.frame_len:
            return np.minimum(kv, ((qp + i) // self.frame_len + 1) * self.frame_len)
        return np.full(len(i), kv, dtype=np.int64)

    def visible_pairs(self):
        """Number of visible (query, key) pairs over all batches and heads."""
        if self.block_density:
            return sum(int(self.row_keys(b).sum()) for b in range(self.B))
        return self.H * sum(int(self.row_keys(b).sum()) for b in range(self.B))

    def ops(self):
        """Algorithmic operations: 4*d per visible pair (QK^T and P.V)."""
        return 4 * self.d * self.visible_pairs()


def get(name, **override):
    """The named workload (see module docstring), fields overridable."""
    if name == "linear":
        return get_linear(name, **override)
    if name == "tiny":
        w = Workload("tiny", 1, 2, 1024, 1024, 64, "f16", 1, seed=101, k_offset_std=2.0)
    elif name == "small":
        w = Workload("small", 1, 12, 32760, 32760, 128, "bf16", 1, seed=202,
                     k_offset_std=float(np.sqrt(3.0)))
    elif name == "large":
        w = Workload("large", 1, 40, 75600, 75600, 128, "bf16", 2, seed=303,
                     outlier_frac=0.01)
    elif name == "stream":
        w = Workload("stream", 1, 24, FRAME, 17 * FRAME, 128, "bf16", 1,
                     frame_len=FRAME, kv_len=[17 * FRAME], q_pos0=[16 * FRAME], seed=404)
    elif name == "batched":
        L = np.random.default_rng(505).integers(4, 33, 8)
        kv = [int((x + 1) * FRAME) for x in L]
        w = Workload("batched", 8, 24, FRAME, 33 * FRAME, 128, "bf16", 1,
                     frame_len=FRAME, kv_len=kv, q_pos0=[int(x * FRAME) for x in L],
                     seed=505)
    elif name == "window":
        w = Workload("window", 1, 24, FRAME, 48 * 2048, 128, "bf16", 1,
                     frame_len=FRAME, kv_len=[41 * FRAME], q_pos0=[40 * FRAME], seed=606,
                     frame_stride=2048, sink_frames=1, window_frames=16)
    elif name == "sparse":
        w = Workload("sparse", 1, 40, 75600, 75600, 128, "bf16", 2, seed=303,
                     outlier_frac=0.01, block_density=0.25)
    elif name == "stream-cache":
        w = Workload("stream-cache", 1, 24, FRAME, 17 * 2048, 128, "bf16", 1,
                     frame_len=FRAME, kv_len=[17 * FRAME], q_pos0=[16 * FRAME], seed=404,
                     frame_stride=2048)
    elif name == "batched-cache":
        L = np.random.default_rng(505).integers(4, 33, 8)
        w = Workload("batched-cache", 8, 24, FRAME, 33 * 2048, 128, "bf16", 1,
                     frame_len=FRAME, kv_len=[int((x + 1) * FRAME) for x in L],
                     q_pos0=[int(x * FRAME) for x in L], seed=505, frame_stride=2048)
    else:
        raise KeyError(name)
    for k, v in override.items():
        setattr(w, k, v)
    return w


NAMES = ("tiny", "small", "large", "stream", "batched", "window", "sparse", "linear", "stream-cache",
         "batched-cache")


_MASKS = {}


def block_mask(w):
    """The workload's block mask: uint8 numpy [B, H, ceil(Nq/128), ceil(Nkv/64)]
    that keeps, for every (batch, head, query tile), exactly
    round(block_density * ceil(Nkv/64)) key blocks chosen uniformly without
    replacement (seeded; None without a density) -- a fixed share per query
    tile, as a top-k block selection keeps."""
    if not w.block_density:
        return None
    key = (w.seed, w.B, w.H, w.Nq, w.Nkv, w.block_density)
    if key not in _MASKS:
        rng = np.random.default_rng(w.seed * 7 + 3)
        shape = (w.B, w.H, -(-w.Nq // 128), -(-w.Nkv // 64))
        keep = int(round(w.block_density * shape[-1]))
        r = rng.random(shape, dtype=np.float32)
        m = np.zeros(shape, dtype=np.uint8)
        if keep > 0:
            np.put_along_axis(m, np.argpartition(r, keep - 1, axis=-1)[..., :keep], 1, axis=-1)
        _MASKS[key] = m
    return _MASKS[key]


@dataclass
class LinearWorkload:
    name: str
    M: int
    N: int
    K: int
    dtype: str
    seed: int
    outlier_frac: float = 0.0
    frame_len: int = 0        # (for sample_rows)

    @property
    def Nq(self):
        return self.M

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    def ops(self):
        """2 M N K: one multiply and one add per term of X W^T."""
        return 2 * self.M * self.N * self.K


def get_linear(name, **override):
    if name != "linear":
        raise KeyError(name)
    w = LinearWorkload("linear", 75600, 13824, 5120, "bf16", seed=707, outlier_frac=0.01)
    for k, v in override.items():
        setattr(w, k, v)
    return w


def make_linear(w, device="cpu"):
    """X [M,K], W [N,K], bias [N] of a linear workload on ``device``."""
    out = {}
    for name, shape, std in (("x", (w.M, w.K), 1.0), ("w", (w.N, w.K), 0.02), ("bias", (w.N,), 0.1)):
        g = torch.Generator(device=device)
        g.manual_seed(_slice_seed(w.seed, name, 0, 0))
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
        if name == "x" and w.outlier_frac:
            n = int(round(w.outlier_frac * w.K))
            idx = np.random.default_rng(w.seed * 7 + 4).choice(w.K, size=n, replace=False)
            t[:, torch.from_numpy(idx).to(device)] *= 8
        out[name] = t.to(w.torch_dtype)
    return out


def _slice_seed(seed, tensor, b, h):
    s = hashlib.sha256(f"{seed}:{tensor}:{b}:{h}".encode()).digest()
    return int.from_bytes(s[:8], "little") & ((1 << 63) - 1)


def k_offsets(w):
    """Per-(head, channel) K offsets [H, d] float32 (zeros if none)."""
    if w.k_offset_std == 0:
        return np.zeros((w.H, w.d), np.float32)
    rng = np.random.default_rng(w.seed * 7 + 1)
    return (rng.standard_normal((w.H, w.d)) * w.k_offset_std).astype(np.float32)


def outlier_channels(w):
    """Sorted flat (head*d + channel) indices of the scaled K channels."""
    if w.outlier_frac == 0:
        return np.zeros(0, np.int64)
    n = int(round(w.outlier_frac * w.H * w.d))
    rng = np.random.default_rng(w.seed * 7 + 2)
    return np.sort(rng.choice(w.H * w.d, size=n, replace=False))


def make(w, device="cpu", heads=None, batches=None, tensors="qkv"):
    """Draw the inputs of workload ``w`` on ``device``.

    Returns a dict with 'q' [B,H,Nq,d], 'k' and 'v' [B,H,kv_tokens,d] in the
    workload's 16-bit dtype (only the requested tensors), restricted to the
    given heads / batches when those are lists.  Key positions at or beyond
    kv_len[b] are zero.
    """
    heads = list(range(w.H)) if heads is None else list(heads)
    batches = list(range(w.B)) if batches is None else list(batches)
    off = torch.from_numpy(k_offsets(w))
    gain = torch.ones(w.H * w.d)
    gain[torch.from_numpy(outlier_channels(w))] = w.outlier_gain
    gain = gain.view(w.H, w.d)
    kvl = w.kv_lens()
    out = {}
    for name in tensors:
        n = w.Nq if name == "q" else w.kv_tokens
        t = torch.empty((len(batches), len(heads), n, w.d), dtype=w.torch_dtype, device=device)
        for bi, b in enumerate(batches):
            for hi, h in enumerate(heads):
                g = torch.Generator(device=device)
                g.manual_seed(_slice_seed(w.seed, name, b, h))
                x = torch.randn((n, w.d), generator=g, device=device, dtype=torch.float32)
                if name == "k":
                    x = x * gain[h].to(device) + off[h].to(device)
                if name != "q" and kvl[b] < n:
                    x[kvl[b]:] = 0
                t[bi, hi] = x.to(w.torch_dtype)
        out[name] = t
    return out


def sample_rows(w, R=512, seed=0):
    """R query rows per (b,h) for sampled checks: always row 0, the last row,
    rows on both sides of every 128-token Q block edge near the ends, and of
    the frame edges; the rest drawn without replacement (seeded)."""
    n = w.Nq
    if R >= n:
        return np.arange(n)
    must = {0, n - 1, 127, 128, min(n - 1, 255), n - 128 if n > 128 else 0}
    if w.frame_len:
        for f in range(w.frame_len, n, w.frame_len):
            must.update({f - 1, f})
    must = sorted(x for x in must if 0 <= x < n)
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(n), must)
    pick = rng.choice(rest, size=max(0, R - len(must)), replace=False)
    return np.sort(np.concatenate([np.asarray(must, np.int64), pick]))
