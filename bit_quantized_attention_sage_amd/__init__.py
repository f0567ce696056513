"""Python binding of libsage_attn.so: argument marshalling only.

Every step of the quantized attention runs in the HIP kernels behind the C ABI
declared in include/sage_attn.h; this module only turns torch tensors (device
memory and streams) into the plain pointers and sizes that ABI takes.  There
is no fallback: when the library is missing, every call raises.

Functions named like the C entry points take the same arguments (a
``Desc`` in place of ``const sage_attn_desc*``).  ``attention`` is the
one-line drop-in for exact attention (the pages' "one line of code" swap, in
the podcast notes' section "37:54 One line of code, twice the speed").
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsage_attn.so")

SAGE_ATTN_ABI_VERSION = 4
SAGE_F16, SAGE_BF16 = 0, 1
SAGE_PV_16, SAGE_PV_FP8, SAGE_PV_AUTO = 0, 1, 2
SAGE_FLAG_DEBUG_SYNC = 0x1
SAGE_MAX_BATCH = 128
SAGE_MAX_SPLITS = 16
SAGE_MAX_MASK_CHUNKS = 4096
STATUS = {0: "SAGE_OK", 1: "SAGE_E_NULL", 2: "SAGE_E_SHAPE", 3: "SAGE_E_DTYPE", 4: "SAGE_E_STRIDE",
          5: "SAGE_E_ALIGN", 6: "SAGE_E_MASK", 7: "SAGE_E_UNSUPPORTED", 8: "SAGE_E_WORKSPACE",
          9: "SAGE_E_VERSION", 10: "SAGE_E_HIP"}

_i64x3 = ctypes.c_int64 * 3


class sage_attn_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32), ("pv_mode", ctypes.c_int32),
                ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("Nkv", ctypes.c_int32), ("d", ctypes.c_int32), ("frame_len", ctypes.c_int32),
                ("kv_splits", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("q_stride", _i64x3), ("k_stride", _i64x3), ("v_stride", _i64x3), ("o_stride", _i64x3),
                ("kv_len", ctypes.POINTER(ctypes.c_int32)), ("q_pos0", ctypes.POINTER(ctypes.c_int32)),
                ("k_mean_in", ctypes.c_void_p), ("frame_stride", ctypes.c_int32),
                ("sink_frames", ctypes.c_int32), ("window_frames", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("chan_shift_in", ctypes.c_void_p),
                ("block_mask", ctypes.c_void_p)]


class sage_quant_bufs(ctypes.Structure):
    _fields_ = [("q_codes", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k_codes", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("k_mean", ctypes.c_void_p), ("chan_shift", ctypes.c_void_p),
                ("v_t", ctypes.c_void_p), ("v_e8m0", ctypes.c_void_p), ("stats", ctypes.c_void_p),
                ("partial", ctypes.c_void_p), ("partial_splits", ctypes.c_int32), ("pv_layout", ctypes.c_int32)]


class SageError(RuntimeError):
    def __init__(self, status, fn, detail):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status


class sage_w8a8_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32), ("M", ctypes.c_int32),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("x_stride", ctypes.c_int64), ("w_stride", ctypes.c_int64), ("y_stride", ctypes.c_int64),
                ("flags", ctypes.c_uint32)]


_lib = None
_DESC_P = ctypes.POINTER(sage_attn_desc)
_WDESC_P = ctypes.POINTER(sage_w8a8_desc)
_BUFS_P = ctypes.POINTER(sage_quant_bufs)


def load(path=None):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m bit_quantized_attention_sage_amd.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "sage_attn_abi_version": (ctypes.c_int, []),
        "sage_attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "sage_attn_last_error": (ctypes.c_char_p, []),
        "sage_attn_constant": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double)]),
        "sage_attn_kv_splits": (ctypes.c_int, [_DESC_P, ctypes.POINTER(ctypes.c_int32)]),
        "sage_attn_workspace_bytes": (ctypes.c_int, [_DESC_P, ctypes.POINTER(ctypes.c_size_t)]),
        "sage_attn_quant_layout": (ctypes.c_int, [_DESC_P, ctypes.c_void_p, ctypes.c_size_t, _BUFS_P]),
        "sage_attn_quantize": (ctypes.c_int, [_DESC_P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              _BUFS_P, ctypes.c_void_p]),
        "sage_attn_quantize_frames_batched": (ctypes.c_int, [_DESC_P, ctypes.c_void_p, ctypes.c_void_p,
                                                             ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
                                                             ctypes.c_int32, _BUFS_P, ctypes.c_void_p]),
        "sage_attn_quantize_frames": (ctypes.c_int, [_DESC_P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_int32, ctypes.c_int32, _BUFS_P, ctypes.c_void_p]),
        "sage_attn_fwd_quantized": (ctypes.c_int, [_DESC_P, _BUFS_P, ctypes.c_void_p, ctypes.c_void_p]),
        "sage_attn_fwd_quantized_noalloc": (ctypes.c_int, [_DESC_P, _BUFS_P, ctypes.c_void_p, ctypes.c_void_p]),
        "sage_attn_fwd": (ctypes.c_int, [_DESC_P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
        "sage_attn_debug_scores_i32": (ctypes.c_int, [_DESC_P, _BUFS_P, ctypes.POINTER(ctypes.c_int32),
                                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
        "sage_attn_debug_convert": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_int64, ctypes.c_void_p]),
        "sage_w8a8_sizes": (ctypes.c_int, [_WDESC_P] + [ctypes.POINTER(ctypes.c_size_t)] * 4),
        "sage_w8a8_quantize_weight": (ctypes.c_int, [_WDESC_P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_void_p]),
        "sage_w8a8_quantize_act": (ctypes.c_int, [_WDESC_P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p]),
        "sage_w8a8_gemm": (ctypes.c_int, [_WDESC_P] + [ctypes.c_void_p] * 7),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.sage_attn_abi_version() != SAGE_ATTN_ABI_VERSION:
        raise RuntimeError("libsage_attn.so ABI version mismatch")
    _lib = lib
    return lib


def _check(status, fn):
    if status != 0:
        raise SageError(status, fn, load().sage_attn_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


class Desc:
    """A sage_attn_desc plus the host arrays it points to (kept alive here)."""

    def __init__(self, B, H, Nq, Nkv, d, dtype, pv_mode=SAGE_PV_16, frame_len=0, kv_len=None,
                 q_pos0=None, sm_scale=0.0, kv_splits=0, flags=0, k_mean_in=None,
                 q_stride=None, k_stride=None, v_stride=None, o_stride=None,
                 frame_stride=0, sink_frames=0, window_frames=0, chan_shift_in=None, block_mask=None):
        c = sage_attn_desc()
        c.abi_version = SAGE_ATTN_ABI_VERSION
        c.dtype = dtype
        c.pv_mode = pv_mode
        c.B, c.H, c.Nq, c.Nkv, c.d = B, H, Nq, Nkv, d
        c.frame_len = frame_len
        c.kv_splits = kv_splits
        c.sm_scale = sm_scale
        c.flags = flags
        c.q_stride = _i64x3(*(q_stride or (H * Nq * d, Nq * d, d)))
        c.k_stride = _i64x3(*(k_stride or (H * Nkv * d, Nkv * d, d)))
        c.v_stride = _i64x3(*(v_stride or (H * Nkv * d, Nkv * d, d)))
        c.o_stride = _i64x3(*(o_stride or (H * Nq * d, Nq * d, d)))
        self._kv = (ctypes.c_int32 * B)(*kv_len) if kv_len is not None else None
        self._qp = (ctypes.c_int32 * B)(*q_pos0) if q_pos0 is not None else None
        c.kv_len = ctypes.cast(self._kv, ctypes.POINTER(ctypes.c_int32)) if self._kv else None
        c.q_pos0 = ctypes.cast(self._qp, ctypes.POINTER(ctypes.c_int32)) if self._qp else None
        self._k_mean_in = k_mean_in
        c.k_mean_in = k_mean_in.data_ptr() if k_mean_in is not None else None
        c.frame_stride, c.sink_frames, c.window_frames, c.reserved = frame_stride, sink_frames, window_frames, 0
        self._chan_shift_in = chan_shift_in
        c.chan_shift_in = chan_shift_in.data_ptr() if chan_shift_in is not None else None
        if block_mask is not None and (block_mask.dtype != torch.uint8 or not block_mask.is_contiguous()
                                       or tuple(block_mask.shape) != (B, H, (Nq + 127) // 128, (Nkv + 63) // 64)):
            raise ValueError("block_mask must be a contiguous uint8 [B, H, ceil(Nq/128), ceil(Nkv/64)] tensor")
        self._block_mask = block_mask
        c.block_mask = block_mask.data_ptr() if block_mask is not None else None
        self.c = c
        self.frame_stride, self.sink_frames, self.window_frames = frame_stride, sink_frames, window_frames
        self.B, self.H, self.Nq, self.Nkv, self.d = B, H, Nq, Nkv, d
        self.dtype, self.pv_mode, self.frame_len = dtype, pv_mode, frame_len
        self.Nq_pad = (Nq + 127) // 128 * 128
        self.Nkv_pad = (Nkv + 127) // 128 * 128

    @property
    def ptr(self):
        return ctypes.byref(self.c)

    @classmethod
    def for_tensors(cls, q, k, v, o=None, nkv=None, **kw):
        """Describe [B,H,N,d] tensors (channel dim contiguous, any b/h/n strides).
        nkv: the key length Nkv when it is not k's (a frame cache: its slot count)."""
        B, H, Nq, d = q.shape
        Nkv = k.shape[2] if nkv is None else nkv
        for t in (q, k, v) + ((o,) if o is not None else ()):
            if t.stride(3) != 1:
                raise ValueError("the channel dimension must be contiguous")
        if q.dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("q, k, v must be float16 or bfloat16")
        dt = SAGE_F16 if q.dtype == torch.float16 else SAGE_BF16
        st = lambda t: tuple(t.stride()[:3])  # noqa: E731
        return cls(B, H, Nq, Nkv, d, dt, q_stride=st(q), k_stride=st(k), v_stride=st(v),
                   o_stride=st(o) if o is not None else None, **kw)


def sage_attn_constant(name):
    v = ctypes.c_double()
    _check(load().sage_attn_constant(name.encode(), ctypes.byref(v)), "sage_attn_constant")
    return v.value


def sage_attn_kv_splits(desc):
    s = ctypes.c_int32()
    _check(load().sage_attn_kv_splits(desc.ptr, ctypes.byref(s)), "sage_attn_kv_splits")
    return s.value


def sage_attn_workspace_bytes(desc):
    n = ctypes.c_size_t()
    _check(load().sage_attn_workspace_bytes(desc.ptr, ctypes.byref(n)), "sage_attn_workspace_bytes")
    return n.value


def sage_attn_quant_layout(desc, ws):
    b = sage_quant_bufs()
    _check(load().sage_attn_quant_layout(desc.ptr, ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                         ctypes.byref(b)), "sage_attn_quant_layout")
    return b


def sage_attn_quantize(desc, q, k, v, bufs, stream=None):
    _check(load().sage_attn_quantize(desc.ptr, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                     ctypes.c_void_p(v.data_ptr()), ctypes.byref(bufs), _stream(stream)),
           "sage_attn_quantize")


def sage_attn_quantize_frames(desc, q, k, v, frame0, nframes, bufs, stream=None):
    """Quantize frames [frame0, frame0 + nframes) of new keys/values (k, v:
    [B,H,nframes*frame_len,d], desc's k/v strides) into the frame cache, and
    the queries q unless None, against the mean and exponents in bufs."""
    _check(load().sage_attn_quantize_frames(desc.ptr, ctypes.c_void_p(q.data_ptr() if q is not None else None),
                                            ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                            int(frame0), int(nframes), ctypes.byref(bufs), _stream(stream)),
           "sage_attn_quantize_frames")


def sage_attn_quantize_frames_batched(desc, q, k, v, frame0, nframes, bufs, stream=None):
    """As sage_attn_quantize_frames, batch b appending its nframes new frames
    (rows [0, nframes*frame_len) of its k, v) at frame frame0[b] of its cache."""
    f0 = (ctypes.c_int32 * len(frame0))(*[int(f) for f in frame0])
    _check(load().sage_attn_quantize_frames_batched(
        desc.ptr, ctypes.c_void_p(q.data_ptr() if q is not None else None), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), f0, int(nframes), ctypes.byref(bufs), _stream(stream)),
        "sage_attn_quantize_frames_batched")


def sage_attn_fwd_quantized(desc, bufs, o, stream=None):
    _check(load().sage_attn_fwd_quantized(desc.ptr, ctypes.byref(bufs), ctypes.c_void_p(o.data_ptr()),
                                          _stream(stream)), "sage_attn_fwd_quantized")


def sage_attn_fwd_quantized_noalloc(desc, bufs, o, stream=None):
    """sage_attn_fwd_quantized with its split-KV partials in the library's
    device scratch: no workspace partial region is needed."""
    _check(load().sage_attn_fwd_quantized_noalloc(desc.ptr, ctypes.byref(bufs), ctypes.c_void_p(o.data_ptr()),
                                                  _stream(stream)), "sage_attn_fwd_quantized_noalloc")


def sage_attn_fwd(desc, q, k, v, o, ws, stream=None):
    _check(load().sage_attn_fwd(desc.ptr, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream(stream)),
           "sage_attn_fwd")


def sage_attn_debug_scores_i32(desc, bufs, tiles, out, stream=None):
    """tiles: list of (b*H + h, q0, k0); out: int32 device tensor [n, 32, 64]."""
    flat = [int(x) for t in tiles for x in t]
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    _check(load().sage_attn_debug_scores_i32(desc.ptr, ctypes.byref(bufs), arr, len(tiles),
                                         ctypes.c_void_p(out.data_ptr()), _stream(stream)),
           "sage_attn_debug_scores_i32")


def sage_attn_debug_convert(kind, x, out, stream=None):
    _check(load().sage_attn_debug_convert(kind, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                          x.numel(), _stream(stream)), "sage_attn_debug_convert")


def new_workspace(desc, device="cuda"):
    """A device workspace of the size sage_attn_fwd needs (256-byte aligned)."""
    n = sage_attn_workspace_bytes(desc)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def quant_views(desc, ws, bufs):
    """Torch views of the quantized operands inside workspace ``ws``."""
    base = ws.data_ptr()
    B, H, d = desc.B, desc.H, desc.d

    def view(ptr, n, dtype, shape):
        off = ptr - base
        esz = torch.empty(0, dtype=dtype).element_size()
        return ws[off:off + n * esz].view(dtype).view(*shape)

    fp8 = desc.pv_mode == SAGE_PV_FP8
    auto = desc.pv_mode == SAGE_PV_AUTO
    # SAGE_PV_AUTO: raw bytes, Nkv_pad * d * 2 per head (a 16-bit head's
    # values, or an FP8 head's codes in the first half)
    vt_shape = (B, H, desc.Nkv_pad * d * 2) if auto else (B, H, desc.Nkv_pad // 64, d, 64)
    out = {
        "q_codes": view(bufs.q_codes, B * H * desc.Nq_pad * d, torch.int8, (B, H, desc.Nq_pad, d)),
        "q_scale": view(bufs.q_scale, B * H * desc.Nq_pad // 128, torch.float32, (B, H, desc.Nq_pad // 128)),
        "k_codes": view(bufs.k_codes, B * H * desc.Nkv_pad * d, torch.int8, (B, H, desc.Nkv_pad, d)),
        "k_scale": view(bufs.k_scale, B * H * desc.Nkv_pad // 64, torch.float32, (B, H, desc.Nkv_pad // 64)),
        "k_mean": view(bufs.k_mean, B * H * d, torch.float32, (B, H, d)),
        "chan_shift": view(bufs.chan_shift, B * H * d, torch.int8, (B, H, d)),
        "v_t": view(bufs.v_t, B * H * desc.Nkv_pad * d * (2 if auto else 1),
                    torch.uint8 if fp8 or auto else torch.int16, vt_shape),
    }
    if fp8 or auto:
        out["v_e8m0"] = view(bufs.v_e8m0, B * H * desc.Nkv_pad // 64 * 256, torch.uint8,
                             (B, H, desc.Nkv_pad // 64, 64, 4))
    return out


def attention(q, k, v, pv_mode=SAGE_PV_16, frame_len=0, kv_len=None, q_pos0=None, sm_scale=0.0,
              kv_splits=0, k_mean_in=None, out=None, workspace=None, stream=None):
    """Quantized attention on [B,H,N,d] fp16/bf16 device tensors; returns O.

    A drop-in for softmax(Q K^T * sm_scale) V with an optional
    frame-block-causal mask (frame_len > 0) against a KV cache of kv_len[b]
    valid keys.  Allocates the output and workspace with torch when not given.
    """
    if out is None:
        out = torch.empty_like(q)
    desc = Desc.for_tensors(q, k, v, out, pv_mode=pv_mode, frame_len=frame_len, kv_len=kv_len,
                            q_pos0=q_pos0, sm_scale=sm_scale, kv_splits=kv_splits, k_mean_in=k_mean_in)
    ws = workspace if workspace is not None else new_workspace(desc, q.device)
    sage_attn_fwd(desc, q, k, v, out, ws, stream)
    return out


# ---------------------------------------------------------------- W8A8 linear
class W8A8Desc:
    """A sage_w8a8_desc for Y [M,N] = X [M,K] W [N,K]^T (+ bias)."""

    def __init__(self, M, N, K, dtype, x_stride=None, w_stride=None, y_stride=None, flags=0):
        c = sage_w8a8_desc()
        c.abi_version = SAGE_ATTN_ABI_VERSION
        c.dtype = dtype
        c.M, c.N, c.K, c.reserved = M, N, K, 0
        c.x_stride = K if x_stride is None else x_stride
        c.w_stride = K if w_stride is None else w_stride
        c.y_stride = N if y_stride is None else y_stride
        c.flags = flags
        self.c = c
        self.M, self.N, self.K, self.dtype = M, N, K, dtype
        self.M_pad = (M + 127) // 128 * 128

    @property
    def ptr(self):
        return ctypes.byref(self.c)

    @classmethod
    def for_tensors(cls, x, w, y=None, **kw):
        """Describe X [M,K] and W [N,K] (rows contiguous in the channel dim)."""
        M, K = x.shape
        N = w.shape[0]
        for t in (x, w) + ((y,) if y is not None else ()):
            if t.stride(1) != 1:
                raise ValueError("rows must be contiguous")
        if x.dtype not in (torch.float16, torch.bfloat16) or w.dtype != x.dtype:
            raise ValueError("x and w must share float16 or bfloat16")
        dt = SAGE_F16 if x.dtype == torch.float16 else SAGE_BF16
        return cls(M, N, K, dt, x_stride=x.stride(0), w_stride=w.stride(0),
                   y_stride=y.stride(0) if y is not None else None, **kw)


def sage_w8a8_sizes(desc):
    """(xq, x_scale, wq, w_scale) sizes in bytes."""
    v = [ctypes.c_size_t() for _ in range(4)]
    _check(load().sage_w8a8_sizes(desc.ptr, *[ctypes.byref(x) for x in v]), "sage_w8a8_sizes")
    return tuple(x.value for x in v)


def w8a8_buffers(desc, device="cuda"):
    """Device tensors for the quantized operands: xq [M_pad,K] int8,
    x_scale [K/128, M_pad] float32, wq [N,K] int8, w_scale [N/128, K/128] float32."""
    M_pad, N, K = desc.M_pad, desc.N, desc.K
    return (torch.empty((M_pad, K), dtype=torch.int8, device=device),
            torch.empty((K // 128, M_pad), dtype=torch.float32, device=device),
            torch.empty((N, K), dtype=torch.int8, device=device),
            torch.empty((N // 128, K // 128), dtype=torch.float32, device=device))


def sage_w8a8_quantize_weight(desc, w, wq, w_scale, stream=None):
    _check(load().sage_w8a8_quantize_weight(desc.ptr, ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(wq.data_ptr()),
                                            ctypes.c_void_p(w_scale.data_ptr()), _stream(stream)),
           "sage_w8a8_quantize_weight")


def sage_w8a8_quantize_act(desc, x, xq, x_scale, stream=None):
    _check(load().sage_w8a8_quantize_act(desc.ptr, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(xq.data_ptr()),
                                         ctypes.c_void_p(x_scale.data_ptr()), _stream(stream)),
           "sage_w8a8_quantize_act")


def sage_w8a8_gemm(desc, xq, x_scale, wq, w_scale, bias, y, stream=None):
    _check(load().sage_w8a8_gemm(desc.ptr, ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(x_scale.data_ptr()),
                                 ctypes.c_void_p(wq.data_ptr()), ctypes.c_void_p(w_scale.data_ptr()),
                                 ctypes.c_void_p(bias.data_ptr() if bias is not None else None),
                                 ctypes.c_void_p(y.data_ptr()), _stream(stream)), "sage_w8a8_gemm")
