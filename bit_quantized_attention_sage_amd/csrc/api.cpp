// C ABI of the quantized attention library: argument validation, workspace
// layout, launch planning.  Host code only; every kernel is enqueued on the
// caller's stream and nothing here allocates or synchronizes (unless
// SAGE_FLAG_DEBUG_SYNC is set).  See include/sage_attn.h for the contract.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <exception>
#include <string>

#include "kernels.h"
#include "../../include/sage_w8a8.h"

namespace {

thread_local std::string g_last_error;

sage_status fail(sage_status status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
int64_t pad128(int64_t n) { return (n + 127) / 128 * 128; }

struct Plan {
  int B, H, Nq, Nkv, d, Nq_pad, Nkv_pad, splits, frame_len, dtype, pv_mode;
  int splits_cap;  // KV splits the workspace's partial region holds room for
  int frame_stride, sink_frames, window_frames;
  uint32_t cpf_magic;
  const uint8_t* block_mask;
  int mask_nkc;
  float sigma;
  sage::BatchInfo bi;
  int order[sage::MAXB_ARGS];
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Key chunks that query tile t (rows [t*rows, t*rows + rows)) of batch b
// visits (the fused kernel's list).
int tile_chunks(const Plan& p, int b, int t, int rows) {
  const int kv = p.bi.kv_len[b], qp = p.bi.q_pos0[b], F = p.frame_len;
  const int first = t * rows, last = std::min(t * rows + rows, p.Nq) - 1;
  if (p.frame_stride == 0) {
    const int end = F > 0 ? std::min(kv, ((qp + last) / F + 1) * F) : kv;
    return (end + 63) / 64;
  }
  const int cpf = p.frame_stride / 64;
  const int fq_lo = (qp + first) / F, fq_hi = (qp + last) / F;
  const int end = (fq_hi * p.frame_stride + std::min(F, kv - fq_hi * F) + 63) / 64;
  if (p.window_frames == 0) return end;
  const int a0 = std::min(std::min(p.sink_frames, fq_hi + 1) * cpf, end);
  const int b1 = std::max(std::min(std::max(p.sink_frames, fq_lo - p.window_frames) * cpf, end), a0);
  return a0 + (end - b1);
}

// KV splits per query tile.  Work items (batch, head, split, tile) run as
// rounds of SLOTS resident workgroups: 256-row ping-pong tiles, one per CU
// (under a block mask each of its two 128-row blocks walks its own kept
// chunks).  The estimated time of s splits is
// ceil(items / SLOTS) x (mean chunks per item + a prologue and epilogue of
// about 3 chunk steps), plus for s > 1 the combine pass (reads s fp32
// partial outputs; one chunk step of a workgroup takes about 1.5 us at
// d = 128, half that at d = 64).  Enough tiles for 4 rounds: no split.
int choose_splits(const Plan& p) {
  const int SLOTS = 256, rows = 256;
  const int nqt = (p.Nq + rows - 1) / rows;
  const int64_t items1 = static_cast<int64_t>(p.B) * p.H * nqt;
  if (items1 >= 4 * SLOTS) return 1;
  double total = 0.0;
  int longest = 1;
  for (int b = 0; b < p.B; ++b)
    for (int t = 0; t < nqt; ++t) {
      const int n = tile_chunks(p, b, t, rows);
      total += n;
      longest = std::max(longest, n);
    }
  const double mean = total / (static_cast<double>(p.B) * nqt);
  const double chunk_us = 1.5 * p.d / 128.0;
  int best = 1;
  double best_cost = 0.0;
  for (int s = 1; s <= SAGE_MAX_SPLITS && s <= std::max(1, longest / 8); ++s) {
    const int64_t items = items1 * s;
    double cost = static_cast<double>((items + SLOTS - 1) / SLOTS) * (mean / s + 3.0);
    if (s > 1) {
      const double bytes = static_cast<double>(s) * p.B * p.H * p.Nq_pad * (p.d + 2) * 4.0;
      cost += bytes / 4e12 / (chunk_us * 1e-6) + 4.0;
    }
    if (s == 1 || cost < 0.98 * best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

// Validate *d and fill *p.  Pure host code; touches no device memory.
sage_status make_plan(const sage_attn_desc* d, Plan* p) {
  if (!d) return fail(SAGE_E_NULL, "desc is NULL");
  if (d->abi_version != SAGE_ATTN_ABI_VERSION)
    return fail(SAGE_E_VERSION, "abi_version " + std::to_string(d->abi_version) + " != " +
                                    std::to_string(SAGE_ATTN_ABI_VERSION));
  if (d->dtype != SAGE_F16 && d->dtype != SAGE_BF16) return fail(SAGE_E_DTYPE, "dtype must be SAGE_F16 or SAGE_BF16");
  if (d->pv_mode != SAGE_PV_16 && d->pv_mode != SAGE_PV_FP8 && d->pv_mode != SAGE_PV_AUTO)
    return fail(SAGE_E_DTYPE, "pv_mode must be SAGE_PV_16, SAGE_PV_FP8 or SAGE_PV_AUTO");
  if (d->pv_mode == SAGE_PV_AUTO && d->frame_stride != 0)
    return fail(SAGE_E_UNSUPPORTED, "SAGE_PV_AUTO needs contiguous keys (frame_stride 0)");
  if (d->d != 64 && d->d != 128) return fail(SAGE_E_UNSUPPORTED, "head dim d must be 64 or 128");
  if (d->B < 1 || d->H < 1 || d->Nq < 1 || d->Nkv < 1) return fail(SAGE_E_SHAPE, "B, H, Nq and Nkv must be >= 1");
  if (d->B > SAGE_MAX_BATCH) return fail(SAGE_E_UNSUPPORTED, "B > SAGE_MAX_BATCH");
  if (d->Nq > (1 << 28) || d->Nkv > (1 << 28)) return fail(SAGE_E_SHAPE, "sequence length too large");
  // The attention kernel addresses one head's staged K and V (16-bit V^T:
  // Nkv_pad * d * 2 bytes) through buffer resources with 32-bit offsets.
  if (pad128(d->Nkv) * d->d * 2 > 0x7FFFFFFF)
    return fail(SAGE_E_SHAPE, "Nkv too large: ceil(Nkv/128)*128 * d * 2 must stay below 2^31");
  const int64_t bh = static_cast<int64_t>(d->B) * d->H;
  if (bh * pad128(d->Nq) / 128 * SAGE_MAX_SPLITS > 0x7FFFFFFF) return fail(SAGE_E_SHAPE, "too many work items");
  if (d->frame_len < 0) return fail(SAGE_E_MASK, "frame_len must be >= 0");
  if (d->reserved != 0) return fail(SAGE_E_UNSUPPORTED, "reserved must be 0");
  if (d->block_mask) {
    if (d->frame_stride != 0) return fail(SAGE_E_UNSUPPORTED, "a block mask needs contiguous keys (frame_stride 0)");
    if ((d->Nkv + 63) / 64 > SAGE_MAX_MASK_CHUNKS)
      return fail(SAGE_E_UNSUPPORTED, "a block mask allows at most SAGE_MAX_MASK_CHUNKS key blocks");
  }
  if (d->frame_stride < 0) return fail(SAGE_E_MASK, "frame_stride must be >= 0");
  if (d->frame_stride != 0) {
    if (d->frame_len <= 0) return fail(SAGE_E_MASK, "a frame cache needs frame_len > 0");
    if (d->frame_stride % 64 != 0 || d->frame_stride < d->frame_len || d->frame_stride >= 131072)
      return fail(SAGE_E_MASK, "frame_stride must be a multiple of 64, >= frame_len and < 131072");
    if (d->Nkv % d->frame_stride != 0) return fail(SAGE_E_SHAPE, "Nkv must be a multiple of frame_stride");
    if (d->Nkv >= (1 << 26)) return fail(SAGE_E_SHAPE, "a frame cache holds fewer than 2^26 slots");
  }
  if (d->sink_frames < 0 || d->window_frames < 0) return fail(SAGE_E_MASK, "sink_frames and window_frames must be >= 0");
  if ((d->window_frames > 0 || d->sink_frames > 0) && d->frame_stride == 0)
    return fail(SAGE_E_MASK, "sink/window frames need the frame cache (frame_stride > 0)");
  if (d->kv_splits < 0 || d->kv_splits > SAGE_MAX_SPLITS) return fail(SAGE_E_SHAPE, "kv_splits out of range");
  if (!(d->sm_scale >= 0.f) || isinf(d->sm_scale)) return fail(SAGE_E_SHAPE, "sm_scale must be finite and >= 0");
  const int64_t* strides[4] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i)
      if (strides[t][i] < 0 || strides[t][i] % 8 != 0)
        return fail(SAGE_E_STRIDE, std::string(names[t]) + "_stride[" + std::to_string(i) +
                                       "] must be a non-negative multiple of 8 elements");
  p->B = d->B;
  p->H = d->H;
  p->Nq = d->Nq;
  p->Nkv = d->Nkv;
  p->d = d->d;
  p->Nq_pad = static_cast<int>(pad128(d->Nq));
  p->Nkv_pad = static_cast<int>(pad128(d->Nkv));
  p->frame_len = d->frame_len;
  p->frame_stride = d->frame_stride;
  p->sink_frames = d->sink_frames;
  p->window_frames = d->window_frames;
  p->cpf_magic = 0;
  p->block_mask = d->block_mask;
  p->mask_nkc = (d->Nkv + 63) / 64;
  if (d->frame_stride > 64) {  // one chunk per frame needs no division
    const uint64_t cpf = static_cast<uint64_t>(d->frame_stride / 64);
    p->cpf_magic = static_cast<uint32_t>(((uint64_t{1} << 32) + cpf - 1) / cpf);
  }
  p->dtype = d->dtype;
  p->pv_mode = d->pv_mode;
  memset(&p->bi, 0, sizeof(p->bi));
  const int kv_cap = d->frame_stride > 0 ? d->Nkv / d->frame_stride * d->frame_len : d->Nkv;
  for (int b = 0; b < d->B; ++b) {
    const int kv = d->kv_len ? d->kv_len[b] : kv_cap;
    if (kv < 1 || kv > kv_cap)
      return fail(SAGE_E_MASK, "kv_len[" + std::to_string(b) +
                                   "] must be in [1, Nkv] (frame cache: tokens of Nkv/frame_stride frames)");
    int qp = 0;
    if (d->frame_len > 0) {
      qp = d->q_pos0 ? d->q_pos0[b] : kv - d->Nq;
      if (qp < 0 || static_cast<int64_t>(qp) + d->Nq > kv)
        return fail(SAGE_E_MASK, "q_pos0[" + std::to_string(b) + "] must satisfy 0 <= q_pos0 and q_pos0 + Nq <= kv_len");
    }
    p->bi.kv_len[b] = kv;
    p->bi.q_pos0[b] = qp;
  }
  for (int b = 0; b < sage::MAXB_ARGS; ++b) p->order[b] = b < d->B ? b : 0;
  std::stable_sort(p->order, p->order + d->B,
                   [&](int x, int y) { return p->bi.kv_len[x] > p->bi.kv_len[y]; });
  const double sm = d->sm_scale > 0.f ? static_cast<double>(d->sm_scale)
                                      : static_cast<double>(static_cast<float>(1.0 / sqrt(static_cast<double>(d->d))));
  p->sigma = static_cast<float>(sm * 1.4426950408889634);
  p->splits = d->kv_splits > 0 ? d->kv_splits : choose_splits(*p);
  // Room in the workspace for the split count of this desc and for the one
  // it would take with every batch at its full key length, so that a frame
  // cache carved once stays usable as its kv_len grows.
  p->splits_cap = p->splits;
  if (d->kv_splits == 0) {
    Plan full = *p;
    for (int b = 0; b < d->B; ++b) {
      full.bi.kv_len[b] = kv_cap;
      if (d->frame_len > 0 && !d->q_pos0) full.bi.q_pos0[b] = kv_cap - d->Nq;
    }
    p->splits_cap = std::max(p->splits, choose_splits(full));
  }
  return SAGE_OK;
}

struct Layout {
  size_t q_codes, q_scale, k_codes, k_scale, k_mean, chan_shift, v_t, v_e8m0, stats, partial, total;
  size_t ksum, kmax, kmin, qamax, pick;  // offsets inside stats
};

Layout layout_of(const Plan& p) {
  Layout L{};
  const size_t bh = static_cast<size_t>(p.B) * p.H;
  const size_t nck = (p.Nkv + sage::KMEAN_CHUNK - 1) / sage::KMEAN_CHUNK;
  const size_t ncq = (p.Nq + sage::KMEAN_CHUNK - 1) / sage::KMEAN_CHUNK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.q_codes = take(bh * p.Nq_pad * p.d);
  L.q_scale = take(bh * (p.Nq_pad / 128) * 4);
  L.k_codes = take(bh * p.Nkv_pad * p.d);
  L.k_scale = take(bh * (p.Nkv_pad / 64) * 4);
  L.k_mean = take(bh * p.d * 4);
  L.chan_shift = take(bh * p.d);
  L.v_t = take(bh * p.Nkv_pad * p.d * (p.pv_mode == SAGE_PV_FP8 ? 1 : 2));
  L.v_e8m0 = take(p.pv_mode != SAGE_PV_16 ? bh * (p.Nkv_pad / 64) * 256 : 0);
  L.ksum = 0;
  L.kmax = align_up(bh * nck * p.d * 8);
  L.kmin = L.kmax + align_up(bh * nck * p.d * 4);
  L.qamax = L.kmin + align_up(bh * nck * p.d * 4);
  L.pick = L.qamax + align_up(bh * ncq * p.d * 4);
  L.stats = take(L.pick + (p.pv_mode == SAGE_PV_AUTO ? 2 * (1 + bh) * 4 : 0));
  L.partial = take(p.splits_cap > 1 ? static_cast<size_t>(p.splits_cap) * bh * p.Nq_pad * (p.d + 2) * 4 : 0);
  L.total = off;
  return L;
}

sage_quant_bufs bufs_of(const Layout& L, const Plan& p, void* ws) {
  char* base = static_cast<char*>(ws);
  sage_quant_bufs b{};
  b.q_codes = reinterpret_cast<int8_t*>(base + L.q_codes);
  b.q_scale = reinterpret_cast<float*>(base + L.q_scale);
  b.k_codes = reinterpret_cast<int8_t*>(base + L.k_codes);
  b.k_scale = reinterpret_cast<float*>(base + L.k_scale);
  b.k_mean = reinterpret_cast<float*>(base + L.k_mean);
  b.chan_shift = reinterpret_cast<int8_t*>(base + L.chan_shift);
  b.v_t = base + L.v_t;
  b.v_e8m0 = p.pv_mode != SAGE_PV_16 ? reinterpret_cast<uint8_t*>(base + L.v_e8m0) : nullptr;
  b.stats = base + L.stats;
  b.partial = p.splits_cap > 1 ? base + L.partial : nullptr;
  b.partial_splits = p.splits_cap > 1 ? p.splits_cap : 1;
  b.pv_layout = p.pv_mode;
  return b;
}

sage_status check_bufs(const sage_quant_bufs* b, const Plan& p, bool need_stats) {
  if (!b) return fail(SAGE_E_NULL, "bufs is NULL");
  if (!b->q_codes || !b->q_scale || !b->k_codes || !b->k_scale || !b->k_mean || !b->chan_shift || !b->v_t)
    return fail(SAGE_E_NULL, "a quantized-operand buffer is NULL");
  if (p.pv_mode != SAGE_PV_16 && !b->v_e8m0) return fail(SAGE_E_NULL, "v_e8m0 is NULL in FP8 and AUTO modes");
  if ((need_stats || p.pv_mode == SAGE_PV_AUTO) && !b->stats)
    return fail(SAGE_E_NULL, need_stats ? "stats buffer is NULL" : "stats buffer is NULL (SAGE_PV_AUTO keeps its head lists there)");
  if (p.pv_mode == SAGE_PV_AUTO && b->pv_layout != SAGE_PV_AUTO)
    return fail(SAGE_E_WORKSPACE, "SAGE_PV_AUTO needs buffers carved for it (bufs->pv_layout " +
                                      std::to_string(b->pv_layout) + ")");
  if (p.pv_mode == SAGE_PV_AUTO && (reinterpret_cast<uintptr_t>(b->stats) & 3u))
    return fail(SAGE_E_ALIGN, "stats must be 4-byte aligned");
  if (p.splits > 1 && !need_stats) {
    if (!b->partial) return fail(SAGE_E_NULL, "partial buffer is NULL with kv_splits > 1");
    if (p.splits > b->partial_splits)
      return fail(SAGE_E_WORKSPACE, "this call needs " + std::to_string(p.splits) +
                                        " KV splits but bufs->partial holds " + std::to_string(b->partial_splits) +
                                        ": carve the workspace for this desc (or its full key length)");
  }
  if (!aligned16(b->q_codes) || !aligned16(b->k_codes) || !aligned16(b->v_t) ||
      (b->v_e8m0 && !aligned16(b->v_e8m0)) || (b->partial && !aligned16(b->partial)))
    return fail(SAGE_E_ALIGN, "quantized-operand buffers must be 16-byte aligned");
  return SAGE_OK;
}

sage_status finish(hipError_t e, const sage_attn_desc* d, hipStream_t st) {
  if (e == hipSuccess && d && (d->flags & SAGE_FLAG_DEBUG_SYNC)) {
    e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(SAGE_E_HIP, std::string("HIP error: ") + hipGetErrorString(e));
  return SAGE_OK;
}

sage::AttnLaunch attn_launch_of(const Plan& p, const sage_quant_bufs& b, void* o, const sage_attn_desc* d) {
  sage::AttnLaunch L{};
  L.dtype = p.dtype;
  L.pv_mode = p.pv_mode;
  L.d = p.d;
  L.B = p.B;
  L.H = p.H;
  L.Nq = p.Nq;
  L.Nkv = p.Nkv;
  L.Nq_pad = p.Nq_pad;
  L.Nkv_pad = p.Nkv_pad;
  L.frame_len = p.frame_len;
  L.splits = p.splits;
  L.frame_stride = p.frame_stride;
  L.sink_frames = p.sink_frames;
  L.window_frames = p.window_frames;
  L.cpf_magic = p.cpf_magic;
  L.block_mask = p.block_mask;
  L.mask_nkc = p.mask_nkc;
  L.sigma = p.sigma;
  L.bi = p.bi;
  for (int i = 0; i < sage::MAXB_ARGS; ++i) L.order[i] = p.order[i];
  L.bufs = b;
  L.o = o;
  for (int i = 0; i < 3; ++i) L.os[i] = d->o_stride[i];
  L.vt_hb = static_cast<int64_t>(p.Nkv_pad) * p.d * (p.pv_mode == SAGE_PV_FP8 ? 1 : 2);
  L.pick = p.pv_mode == SAGE_PV_AUTO ? reinterpret_cast<int*>(static_cast<char*>(b.stats) + layout_of(p).pick)
                                     : nullptr;
  return L;
}

sage_status quantize_impl(const sage_attn_desc* desc, const void* q, const void* k, const void* v,
                          int frames_only, int frame0, const int32_t* frame0s, int nframes,
                          const sage_quant_bufs* bufs, void* stream) {
  try {
    Plan p;
    sage_status s = make_plan(desc, &p);
    if (s != SAGE_OK) return s;
    if ((!frames_only && !q) || !k || !v) return fail(SAGE_E_NULL, "q, k and v must be non-NULL");
    if ((q && !aligned16(q)) || !aligned16(k) || !aligned16(v))
      return fail(SAGE_E_ALIGN, "q, k and v must be 16-byte aligned");
    if ((s = check_bufs(bufs, p, true)) != SAGE_OK) return s;
    if (desc->k_mean_in && (reinterpret_cast<uintptr_t>(desc->k_mean_in) & 3u))
      return fail(SAGE_E_ALIGN, "k_mean_in must be 4-byte aligned");
    if (frames_only) {
      if (p.frame_stride == 0) return fail(SAGE_E_UNSUPPORTED, "sage_attn_quantize_frames needs a frame cache");
      if (frame0s) {
        if (nframes < 1) return fail(SAGE_E_SHAPE, "nframes must be positive");
        for (int b = 0; b < p.B; ++b)
          if (frame0s[b] < 0 || static_cast<int64_t>(frame0s[b]) * p.frame_stride +
                                    static_cast<int64_t>(nframes) * p.frame_stride > p.Nkv)
            return fail(SAGE_E_SHAPE, "batch " + std::to_string(b) +
                                          ": frames [frame0, frame0 + nframes) must lie inside the Nkv cache slots");
      } else if (frame0 < 0 || nframes < 1 || static_cast<int64_t>(frame0) * p.frame_stride +
                                                   static_cast<int64_t>(nframes) * p.frame_stride > p.Nkv) {
        return fail(SAGE_E_SHAPE, "frames [frame0, frame0 + nframes) must lie inside the Nkv cache slots");
      }
    }
    sage::QuantLaunch L{};
    L.chan_shift_in = desc->chan_shift_in;
    L.frame_len = p.frame_len;
    L.frame_stride = p.frame_stride;
    L.frames_only = frames_only;
    L.frame0 = frame0s ? -1 : frame0;
    L.nframes = nframes;
    L.dtype = p.dtype;
    L.pv_mode = p.pv_mode;
    L.d = p.d;
    L.B = p.B;
    L.H = p.H;
    L.Nq = p.Nq;
    L.Nkv = p.Nkv;
    L.Nq_pad = p.Nq_pad;
    L.Nkv_pad = p.Nkv_pad;
    L.q = q;
    L.k = k;
    L.v = v;
    for (int i = 0; i < 3; ++i) {
      L.qs[i] = desc->q_stride[i];
      L.ks[i] = desc->k_stride[i];
      L.vs[i] = desc->v_stride[i];
    }
    L.k_mean_in = desc->k_mean_in;
    L.bi = p.bi;
    if (frame0s)
      for (int b = 0; b < p.B; ++b) L.bi.frame0[b] = frame0s[b];
    L.bufs = *bufs;
    const Layout lay = layout_of(p);
    char* st = static_cast<char*>(bufs->stats);
    L.stat_ksum = reinterpret_cast<double*>(st + lay.ksum);
    L.stat_kmax = reinterpret_cast<float*>(st + lay.kmax);
    L.stat_kmin = reinterpret_cast<float*>(st + lay.kmin);
    L.stat_qamax = reinterpret_cast<float*>(st + lay.qamax);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish(sage::launch_quantize(L, hs), desc, hs);
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status w8a8_plan(const sage_w8a8_desc* d, sage::W8A8Launch* L) {
  if (!d) return fail(SAGE_E_NULL, "desc is NULL");
  if (d->abi_version != SAGE_ATTN_ABI_VERSION)
    return fail(SAGE_E_VERSION, "abi_version " + std::to_string(d->abi_version) + " != " +
                                    std::to_string(SAGE_ATTN_ABI_VERSION));
  if (d->dtype != SAGE_F16 && d->dtype != SAGE_BF16) return fail(SAGE_E_DTYPE, "dtype must be SAGE_F16 or SAGE_BF16");
  if (d->reserved != 0) return fail(SAGE_E_UNSUPPORTED, "reserved must be 0");
  if (d->M < 1 || d->N < SAGE_W8A8_GROUP || d->K < SAGE_W8A8_GROUP || d->N % SAGE_W8A8_GROUP || d->K % SAGE_W8A8_GROUP)
    return fail(SAGE_E_SHAPE, "M >= 1; N and K positive multiples of 128");
  const int64_t mpad = pad128(d->M);
  if (mpad * d->K >= (int64_t{1} << 31) || static_cast<int64_t>(d->N) * d->K >= (int64_t{1} << 31))
    return fail(SAGE_E_SHAPE, "M_pad * K and N * K must be below 2^31");
  if (d->x_stride < d->K || d->w_stride < d->K || d->y_stride < d->N || d->x_stride % 8 || d->w_stride % 8 ||
      d->y_stride % 8)
    return fail(SAGE_E_STRIDE, "row strides must cover a row and be multiples of 8 elements");
  L->dtype = d->dtype;
  L->M = d->M;
  L->M_pad = static_cast<int>(mpad);
  L->N = d->N;
  L->K = d->K;
  L->xs = d->x_stride;
  L->ws = d->w_stride;
  L->ys = d->y_stride;
  return SAGE_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

sage_status finish_w8a8(hipError_t e, const sage_w8a8_desc* d, hipStream_t st) {
  if (e == hipSuccess && (d->flags & SAGE_FLAG_DEBUG_SYNC)) {
    e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(SAGE_E_HIP, hipGetErrorString(e));
  return SAGE_OK;
}

}  // namespace

extern "C" {

int sage_attn_abi_version(void) { return SAGE_ATTN_ABI_VERSION; }

const char* sage_attn_status_string(sage_status s) {
  switch (s) {
    case SAGE_OK: return "ok";
    case SAGE_E_NULL: return "null pointer";
    case SAGE_E_SHAPE: return "bad shape";
    case SAGE_E_DTYPE: return "bad dtype or pv_mode";
    case SAGE_E_STRIDE: return "bad stride";
    case SAGE_E_ALIGN: return "misaligned pointer";
    case SAGE_E_MASK: return "inconsistent mask parameters";
    case SAGE_E_UNSUPPORTED: return "unsupported configuration";
    case SAGE_E_WORKSPACE: return "workspace missing or too small";
    case SAGE_E_VERSION: return "ABI version mismatch";
    case SAGE_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* sage_attn_last_error(void) { return g_last_error.c_str(); }

sage_status sage_attn_constant(const char* name, double* value) {
  if (!name || !value) return fail(SAGE_E_NULL, "name/value is NULL");
  const struct { const char* n; double v; } table[] = {
      {"BQ", sage::BQ}, {"BK", sage::BK}, {"VB", sage::VB}, {"QMAX", sage::QMAX},
      {"TAU", sage::TAU}, {"PSHIFT_FP8", sage::PSHIFT_FP8}, {"PSHIFT_16", sage::PSHIFT_16},
      {"KMEAN_CHUNK", sage::KMEAN_CHUNK}};
  for (const auto& e : table)
    if (strcmp(e.n, name) == 0) {
      *value = e.v;
      return SAGE_OK;
    }
  return fail(SAGE_E_UNSUPPORTED, std::string("unknown constant ") + name);
}

sage_status sage_attn_kv_splits(const sage_attn_desc* desc, int32_t* splits) {
  try {
    if (!splits) return fail(SAGE_E_NULL, "splits is NULL");
    Plan p;
    const sage_status s = make_plan(desc, &p);
    if (s != SAGE_OK) return s;
    *splits = p.splits;
    return SAGE_OK;
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_attn_workspace_bytes(const sage_attn_desc* desc, size_t* bytes) {
  try {
    if (!bytes) return fail(SAGE_E_NULL, "bytes is NULL");
    Plan p;
    const sage_status s = make_plan(desc, &p);
    if (s != SAGE_OK) return s;
    *bytes = layout_of(p).total;
    return SAGE_OK;
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_attn_quant_layout(const sage_attn_desc* desc, void* ws, size_t ws_bytes, sage_quant_bufs* out) {
  try {
    if (!out) return fail(SAGE_E_NULL, "out is NULL");
    Plan p;
    const sage_status s = make_plan(desc, &p);
    if (s != SAGE_OK) return s;
    const Layout L = layout_of(p);
    if (!ws) return fail(SAGE_E_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % ALIGN) return fail(SAGE_E_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < L.total)
      return fail(SAGE_E_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, needs " + std::to_string(L.total));
    *out = bufs_of(L, p, ws);
    return SAGE_OK;
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_attn_quantize(const sage_attn_desc* desc, const void* q, const void* k, const void* v,
                               const sage_quant_bufs* bufs, void* stream) {
  return quantize_impl(desc, q, k, v, 0, 0, nullptr, 0, bufs, stream);
}

sage_status sage_attn_quantize_frames(const sage_attn_desc* desc, const void* q, const void* k, const void* v,
                                      int32_t frame0, int32_t nframes, const sage_quant_bufs* bufs, void* stream) {
  return quantize_impl(desc, q, k, v, 1, frame0, nullptr, nframes, bufs, stream);
}

sage_status sage_attn_quantize_frames_batched(const sage_attn_desc* desc, const void* q, const void* k,
                                              const void* v, const int32_t* frame0, int32_t nframes,
                                              const sage_quant_bufs* bufs, void* stream) {
  if (!frame0) return fail(SAGE_E_NULL, "frame0 is NULL");
  return quantize_impl(desc, q, k, v, 1, 0, frame0, nframes, bufs, stream);
}

sage_status sage_attn_fwd_quantized(const sage_attn_desc* desc, const sage_quant_bufs* bufs, void* o,
                                    void* stream) {
  try {
    Plan p;
    sage_status s = make_plan(desc, &p);
    if (s != SAGE_OK) return s;
    if (!o) return fail(SAGE_E_NULL, "o is NULL");
    if (!aligned16(o)) return fail(SAGE_E_ALIGN, "o must be 16-byte aligned");
    if ((s = check_bufs(bufs, p, false)) != SAGE_OK) return s;
    const sage::AttnLaunch L = attn_launch_of(p, *bufs, o, desc);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish(sage::launch_attention(L, hs), desc, hs);
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_attn_fwd_quantized_noalloc(const sage_attn_desc* desc, const sage_quant_bufs* bufs, void* o,
                                            void* stream) {
  try {
    Plan p;
    sage_status s = make_plan(desc, &p);
    if (s != SAGE_OK) return s;
    if (!o) return fail(SAGE_E_NULL, "o is NULL");
    if (!aligned16(o)) return fail(SAGE_E_ALIGN, "o must be 16-byte aligned");
    const size_t need = p.splits > 1 ? static_cast<size_t>(p.splits) * p.B * p.H * p.Nq_pad * (p.d + 2) * 4 : 0;
    if (need > sage::SCRATCH_BYTES)
      return fail(SAGE_E_WORKSPACE, "split-KV partials need " + std::to_string(need) +
                                        " bytes, more than the " + std::to_string(sage::SCRATCH_BYTES) +
                                        "-byte device scratch of sage_attn_fwd_quantized_noalloc");
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (hs) {
      int sdev = 0, cur = 0;
      hipError_t e = hipStreamGetDevice(hs, &sdev);
      if (e == hipSuccess) e = hipGetDevice(&cur);
      if (e != hipSuccess) return fail(SAGE_E_HIP, std::string("HIP error: ") + hipGetErrorString(e));
      if (sdev != cur) return fail(SAGE_E_UNSUPPORTED, "the stream must belong to the current device");
    }
    sage_quant_bufs b = bufs ? *bufs : sage_quant_bufs{};
    b.partial = nullptr;
    b.partial_splits = 1;
    if (need > 0) {
      void* ptr = nullptr;
      const hipError_t e = sage::scratch_address(&ptr);
      if (e != hipSuccess) return fail(SAGE_E_HIP, std::string("device scratch: ") + hipGetErrorString(e));
      b.partial = ptr;
      b.partial_splits = p.splits;
    }
    if ((s = check_bufs(bufs ? &b : nullptr, p, false)) != SAGE_OK) return s;
    const sage::AttnLaunch L = attn_launch_of(p, b, o, desc);
    return finish(sage::launch_attention(L, hs), desc, hs);
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_attn_fwd(const sage_attn_desc* desc, const void* q, const void* k, const void* v, void* o,
                          void* ws, size_t ws_bytes, void* stream) {
  sage_quant_bufs b;
  sage_status s = sage_attn_quant_layout(desc, ws, ws_bytes, &b);
  if (s != SAGE_OK) return s;
  if (!o) return fail(SAGE_E_NULL, "o is NULL");
  if (!aligned16(o)) return fail(SAGE_E_ALIGN, "o must be 16-byte aligned");
  s = sage_attn_quantize(desc, q, k, v, &b, stream);
  if (s != SAGE_OK) return s;
  return sage_attn_fwd_quantized(desc, &b, o, stream);
}

sage_status sage_attn_debug_scores_i32(const sage_attn_desc* desc, const sage_quant_bufs* bufs,
                                      const int32_t* tiles, int32_t ntiles, int32_t* out, void* stream) {
  try {
    Plan p;
    sage_status s = make_plan(desc, &p);
    if (s != SAGE_OK) return s;
    if (!tiles || !out) return fail(SAGE_E_NULL, "tiles/out is NULL");
    if (ntiles < 0) return fail(SAGE_E_SHAPE, "ntiles < 0");
    if (!bufs || !bufs->q_codes || !bufs->k_codes) return fail(SAGE_E_NULL, "codes are NULL");
    if (!aligned16(bufs->q_codes) || !aligned16(bufs->k_codes) || !aligned16(out))
      return fail(SAGE_E_ALIGN, "codes and out must be 16-byte aligned");
    for (int i = 0; i < ntiles; ++i) {
      const int bh = tiles[3 * i], q0 = tiles[3 * i + 1], k0 = tiles[3 * i + 2];
      if (bh < 0 || bh >= p.B * p.H || q0 < 0 || q0 % 32 || q0 + 32 > p.Nq_pad || k0 < 0 || k0 % 64 ||
          k0 + 64 > p.Nkv_pad)
        return fail(SAGE_E_SHAPE, "tile " + std::to_string(i) + " out of range");
    }
    const sage::AttnLaunch L = attn_launch_of(p, *bufs, nullptr, desc);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish(sage::launch_debug_scores(L, tiles, ntiles, out, hs), desc, hs);
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_attn_debug_convert(int kind, const float* in, void* out, int64_t n, void* stream) {
  try {
    if (kind < 0 || kind > 3) return fail(SAGE_E_UNSUPPORTED, "kind must be 0, 1, 2 or 3");
    if (n < 0) return fail(SAGE_E_SHAPE, "n < 0");
    if (n == 0) return SAGE_OK;
    if (!in || !out) return fail(SAGE_E_NULL, "in/out is NULL");
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish(sage::launch_convert(kind, in, out, n, hs), nullptr, hs);
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

// ---------------------------------------------------------------- W8A8 linear
sage_status sage_w8a8_sizes(const sage_w8a8_desc* desc, size_t* xq_bytes, size_t* x_scale_bytes,
                            size_t* wq_bytes, size_t* w_scale_bytes) {
  try {
    sage::W8A8Launch L{};
    const sage_status s = w8a8_plan(desc, &L);
    if (s != SAGE_OK) return s;
    const size_t nkb = static_cast<size_t>(L.K) / SAGE_W8A8_GROUP;
    if (xq_bytes) *xq_bytes = static_cast<size_t>(L.M_pad) * L.K;
    if (x_scale_bytes) *x_scale_bytes = nkb * L.M_pad * 4;
    if (wq_bytes) *wq_bytes = static_cast<size_t>(L.N) * L.K;
    if (w_scale_bytes) *w_scale_bytes = static_cast<size_t>(L.N) / SAGE_W8A8_GROUP * nkb * 4;
    return SAGE_OK;
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_w8a8_quantize_weight(const sage_w8a8_desc* desc, const void* w, int8_t* wq, float* w_scale, void* stream) {
  try {
    sage::W8A8Launch L{};
    const sage_status s = w8a8_plan(desc, &L);
    if (s != SAGE_OK) return s;
    if (!w || !wq || !w_scale) return fail(SAGE_E_NULL, "w, wq and w_scale must be non-NULL");
    if (!aligned16(w) || !aligned16(wq) || !aligned4(w_scale)) return fail(SAGE_E_ALIGN, "w, wq 16-byte and w_scale 4-byte aligned");
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish_w8a8(sage::launch_w8a8_quant_weight(L, w, wq, w_scale, hs), desc, hs);
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_w8a8_quantize_act(const sage_w8a8_desc* desc, const void* x, int8_t* xq, float* x_scale, void* stream) {
  try {
    sage::W8A8Launch L{};
    const sage_status s = w8a8_plan(desc, &L);
    if (s != SAGE_OK) return s;
    if (!x || !xq || !x_scale) return fail(SAGE_E_NULL, "x, xq and x_scale must be non-NULL");
    if (!aligned16(x) || !aligned16(xq) || !aligned4(x_scale)) return fail(SAGE_E_ALIGN, "x, xq 16-byte and x_scale 4-byte aligned");
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish_w8a8(sage::launch_w8a8_quant_act(L, x, xq, x_scale, hs), desc, hs);
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

sage_status sage_w8a8_gemm(const sage_w8a8_desc* desc, const int8_t* xq, const float* x_scale, const int8_t* wq,
                   const float* w_scale, const void* bias, void* y, void* stream) {
  try {
    sage::W8A8Launch L{};
    const sage_status s = w8a8_plan(desc, &L);
    if (s != SAGE_OK) return s;
    if (!xq || !x_scale || !wq || !w_scale || !y) return fail(SAGE_E_NULL, "xq, x_scale, wq, w_scale and y must be non-NULL");
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || (bias && !aligned16(bias)) || !aligned4(x_scale) ||
        !aligned4(w_scale))
      return fail(SAGE_E_ALIGN, "xq, wq, y, bias 16-byte and scales 4-byte aligned");
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish_w8a8(sage::launch_w8a8_gemm(L, xq, x_scale, wq, w_scale, bias, y, hs), desc, hs);
  } catch (const std::exception& e) {
    return fail(SAGE_E_HIP, e.what());
  }
}

}  // extern "C"
