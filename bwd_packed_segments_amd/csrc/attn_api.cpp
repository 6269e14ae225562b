// C ABI of the attention library: host-side validation, workspace layout,
// route choice and kernel launches.  Validation makes no HIP call, so every
// argument error is reported (and nothing launched) even without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "bps_args.hpp"
#include "bps_attn.h"

namespace {

using bps::ChunkSum;

thread_local std::string g_err;

attn_status fail(attn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Plan {
  bool meta = false;
  int sides = 0;
  bool fast_candidate = false;
  bool check_eq = false;
  bool derive_pos_q = false, derive_pos_kv = false;
  int nch_q = 0, nch_kv = 0;
  float scale = 0.f;
  size_t off_route = 0, off_run_q = 0, off_pos_q = 0, off_sum_q = 0, off_qord = 0, off_kord = 0;
  size_t off_run_kv = 0, off_pos_kv = 0, off_sum_kv = 0;
  size_t off_delta = 0, off_lse2 = 0;
  bool fused = false;           // ATTN_FUSED_BWD: dQ partials in the workspace
  size_t off_dqp = 0;
  int kv_split = 1;             // workgroups per key tile in dK/dV (partials when > 1)
  size_t off_dkvp = 0;
  size_t ws_fwd = 0, ws_bwd = 0;
};

// Longest-walk-first tile orders (tile_order_kernel) for non-causal
// attention whose rows are expected on the general route (separate KV
// metadata, or the route forced).  Measured: cross 4K 1.23 -> 1.13 ms per
// step.  Self-attention rows normally take the fast route, and causal walks
// already come longest first in the fixed order; there the order measured
// no gain while its kernel and the dependent load of the tile index at the
// start of every workgroup cost time.
bool ordered_tiles(const attn_desc* d, const Plan& p) {
  return !d->causal && (p.sides == 2 || (d->flags & ATTN_FORCE_GENERAL));
}

bool supported_dims(int dtype, int dqk, int dv) {
  if (dtype == ATTN_BF16) return (dqk == 64 || dqk == 128 || dqk == 192) && (dv == 64 || dv == 128);
  if (dtype == ATTN_FP32) return (dqk == 64 || dqk == 128) && (dv == 64 || dv == 128);
  return false;
}

attn_status check_strides(const char* name, const attn_strides& s, int vec) {
  if (s.batch < 0 || s.token < 0 || s.head < 0)
    return fail(ATTN_E_INVALID, "%s strides must be non-negative", name);
  if (s.batch % vec || s.token % vec || s.head % vec)
    return fail(ATTN_E_UNSUPPORTED, "%s strides must be multiples of %d elements (16-byte rows)", name, vec);
  return ATTN_OK;
}

// A tensor the library writes (O; dQ, dK, dV, which take the strides of Q,
// K, V) must not map two elements to one address, or several workgroups
// would store to the same memory.  With the head dim contiguous, that holds
// when the outer axes, taken in increasing stride, each step over the whole
// span of the axes inside them (axes of extent 1 aside).
attn_status check_disjoint(const char* name, const attn_strides& s, int B, int S, int H, int D) {
  struct Ax { int64_t stride; int64_t ext; } ax[3] = {{s.batch, B}, {s.token, S}, {s.head, H}};
  std::sort(ax, ax + 3, [](const Ax& x, const Ax& y) { return x.stride < y.stride; });
  int64_t span = D;   // elements covered by the axes inside the current one
  for (const Ax& a : ax) {
    if (a.ext <= 1) continue;
    if (a.stride < span)
      return fail(ATTN_E_UNSUPPORTED, "%s strides (batch %lld, token %lld, head %lld) overlap: the library writes "
                  "through them (outputs must not alias)", name, (long long)s.batch, (long long)s.token,
                  (long long)s.head);
    span = a.stride * (a.ext - 1) + span;
  }
  return ATTN_OK;
}

attn_status make_plan(const attn_desc* d, const attn_segments* seg, Plan* p, bool allow_split = true) {
  if (!d) return fail(ATTN_E_INVALID, "desc is NULL");
  if (d->B < 1 || d->Sq < 0 || d->Skv < 0 || d->Hq < 1 || d->Hkv < 1 || d->Dqk < 1 || d->Dv < 1)
    return fail(ATTN_E_INVALID, "sizes must be positive (B=%d Sq=%d Skv=%d Hq=%d Hkv=%d Dqk=%d Dv=%d)", d->B,
                d->Sq, d->Skv, d->Hq, d->Hkv, d->Dqk, d->Dv);
  if (d->Hq % d->Hkv) return fail(ATTN_E_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", d->Hq, d->Hkv);
  if (d->dtype != ATTN_BF16 && d->dtype != ATTN_FP32) return fail(ATTN_E_INVALID, "unknown dtype %d", d->dtype);
  if (!supported_dims(d->dtype, d->Dqk, d->Dv))
    return fail(ATTN_E_UNSUPPORTED, "head dims (Dqk=%d, Dv=%d) not built for dtype %d", d->Dqk, d->Dv, d->dtype);
  if (d->causal != 0 && d->causal != 1) return fail(ATTN_E_INVALID, "causal must be 0 or 1");
  if (!std::isfinite(d->scale) || d->scale < 0.f) return fail(ATTN_E_INVALID, "scale must be finite and >= 0");
  if (d->flags & ~static_cast<uint32_t>(ATTN_FORCE_GENERAL | ATTN_REVERSE_SCHEDULE | ATTN_FUSED_BWD | ATTN_LOG_ROUTE))
    return fail(ATTN_E_INVALID, "unknown flag bits 0x%x", d->flags);
  p->fused = (d->flags & ATTN_FUSED_BWD) != 0;
  if (p->fused && (d->dtype != ATTN_BF16 || d->Dqk > 128 || d->Dv > 128))
    return fail(ATTN_E_UNSUPPORTED, "the fused backward is built for bf16 with Dqk, Dv <= 128 (dtype %d, Dqk=%d, Dv=%d)",
                d->dtype, d->Dqk, d->Dv);
  const long long rows = (long long)d->B * d->Hq * (long long)(d->Sq > d->Skv ? d->Sq : d->Skv);
  if (rows > (1LL << 31) - 1) return fail(ATTN_E_UNSUPPORTED, "B*H*S exceeds 2^31");
  const int vec = d->dtype == ATTN_BF16 ? 8 : 4;
  attn_status st;
  if ((st = check_strides("q", d->q, vec)) != ATTN_OK) return st;
  if ((st = check_strides("k", d->k, vec)) != ATTN_OK) return st;
  if ((st = check_strides("v", d->v, vec)) != ATTN_OK) return st;
  if (d->k.token > bps::kMaxKvTokenStride || d->v.token > bps::kMaxKvTokenStride)
    return fail(ATTN_E_UNSUPPORTED, "k and v token strides must not exceed %lld elements (got %lld, %lld)",
                (long long)bps::kMaxKvTokenStride, (long long)d->k.token, (long long)d->v.token);
  if ((st = check_strides("o", d->o, vec)) != ATTN_OK) return st;
  if ((st = check_disjoint("o (and dO)", d->o, d->B, d->Sq, d->Hq, d->Dv)) != ATTN_OK) return st;
  p->scale = d->scale == 0.f ? 1.f / std::sqrt(static_cast<float>(d->Dqk)) : d->scale;

  p->meta = seg != nullptr;
  if (!p->meta) {
    if (d->causal && d->Sq != d->Skv)
      return fail(ATTN_E_UNSUPPORTED, "causal attention without segment metadata needs Sq == Skv (%d != %d)",
                  d->Sq, d->Skv);
  } else {
    if (!seg->ids_q) return fail(ATTN_E_INVALID, "segment metadata given without ids_q");
    if (!seg->ids_kv && seg->pos_kv)
      return fail(ATTN_E_INVALID, "pos_kv given without ids_kv (ids and pos must come in pairs)");
    const bool self = !seg->ids_kv || (seg->ids_kv == seg->ids_q && seg->pos_kv == seg->pos_q);
    if (self && d->Sq != d->Skv)
      return fail(ATTN_E_INVALID, "self-attention metadata (no separate ids_kv) needs Sq == Skv (%d != %d)",
                  d->Sq, d->Skv);
    p->sides = self ? 1 : 2;
    const bool forced = (d->flags & ATTN_FORCE_GENERAL) != 0;
    p->check_eq = !self && d->Sq == d->Skv && !forced;
    p->fast_candidate = !forced && (self || p->check_eq);
    p->derive_pos_q = seg->pos_q == nullptr;
    p->derive_pos_kv = !self && seg->pos_kv == nullptr;
    p->nch_q = (d->Sq + bps::kChunk - 1) / bps::kChunk;
    p->nch_kv = (d->Skv + bps::kChunk - 1) / bps::kChunk;
  }

  size_t off = 0;
  if (p->meta) {
    const size_t B = d->B;
    p->off_route = off; off = align_up(off + B * sizeof(int));
    p->off_run_q = off; off = align_up(off + B * d->Sq * sizeof(int2));
    if (p->derive_pos_q) { p->off_pos_q = off; off = align_up(off + B * d->Sq * sizeof(int)); }
    p->off_sum_q = off; off = align_up(off + B * p->nch_q * sizeof(ChunkSum));
    if (p->sides == 2) {
      p->off_run_kv = off; off = align_up(off + B * d->Skv * sizeof(int2));
      if (p->derive_pos_kv) { p->off_pos_kv = off; off = align_up(off + B * d->Skv * sizeof(int)); }
      p->off_sum_kv = off; off = align_up(off + B * p->nch_kv * sizeof(ChunkSum));
    }
    if (ordered_tiles(d, *p)) {
      p->off_qord = off; off = align_up(off + B * (((size_t)d->Sq + 127) / 128) * sizeof(int));
      p->off_kord = off; off = align_up(off + B * (((size_t)d->Skv + 127) / 128) * sizeof(int));
    }
  }
  p->ws_fwd = off;
  const size_t nrow = (size_t)d->B * d->Hq * d->Sq;
  p->off_delta = off; off = align_up(off + nrow * sizeof(float));
  p->off_lse2 = off; off = align_up(off + nrow * sizeof(float));
  if (p->fused) {
    // One fp32 partial of 32 queries x Dqk per (batch row, query head, key
    // tile of 128, query block of 32), query blocks padded to whole 64-row tiles.
    const size_t n_kt = ((size_t)d->Skv + 127) / 128, nqb = 2 * (((size_t)d->Sq + 63) / 64);
    p->off_dqp = off;
    off = align_up(off + (size_t)d->B * d->Hq * n_kt * nqb * 32 * d->Dqk * sizeof(float));
  }
  // bf16 dK/dV with fewer than two workgroups per CU (256 CUs): split each
  // key tile's walk over query tiles between 2 to 4 workgroups, about three
  // per CU in all, so the longest walk no longer sets the time alone; the
  // parts are fp32 partials summed in split order by a second kernel.
  // (Cross 4K, 256 key tiles: 0.92 / 0.73 / 0.62 / 0.73 ms for 1 / 2 / 3 / 4
  // parts.)
  const size_t n_kt = ((size_t)d->Skv + 127) / 128, nkvb = (size_t)d->B * d->Hkv * n_kt;
  const int split = (allow_split && nkvb > 0 && nkvb < 512)
                        ? (int)std::min<size_t>(4, std::max<size_t>(2, (768 + nkvb / 2) / nkvb))
                        : 1;
  if (d->dtype == ATTN_BF16 && nkvb > 0 && split > 1) {
    p->kv_split = split;
    p->off_dkvp = off;
    off = align_up(off + nkvb * p->kv_split * 128 * (size_t)(d->Dqk + d->Dv) * sizeof(float));
  }
  p->ws_bwd = off;
  return ATTN_OK;
}

bool need_nonnull(const void* ptr, long long elems) { return elems > 0 && ptr == nullptr; }

bps::Strides strides_of(const attn_strides& s) { return bps::Strides{s.batch, s.token, s.head}; }

bps::AttnShape shape_of(const attn_desc* d, const Plan& p) {
  bps::AttnShape s;
  s.B = d->B; s.Sq = d->Sq; s.Skv = d->Skv; s.Hq = d->Hq; s.Hkv = d->Hkv;
  s.causal = d->causal;
  s.reverse = (d->flags & ATTN_REVERSE_SCHEDULE) ? 1 : 0;
  s.has_meta = p.meta ? 1 : 0;
  s.scale = p.scale;
  s.scale_log2 = p.scale * bps::kLog2e;
  return s;
}

// Launches the metadata preparation and fills the kernels' view of it.
attn_status prepare_segments(const attn_desc* d, const attn_segments* seg, const Plan& p, char* ws,
                             hipStream_t st, bps::SegView* view, bool launch = true) {
  *view = bps::SegView{};
  if (!p.meta) return ATTN_OK;
  bps::SegMetaArgs m{};
  m.B = d->B; m.Sq = d->Sq; m.Skv = d->Skv;
  m.sides = p.sides;
  m.check_eq = p.check_eq ? 1 : 0;
  m.force_general = (d->flags & ATTN_FORCE_GENERAL) ? 1 : 0;
  m.ids[0] = seg->ids_q;
  m.pos_in[0] = seg->pos_q;
  m.pos_out[0] = p.derive_pos_q ? reinterpret_cast<int*>(ws + p.off_pos_q) : nullptr;
  m.run[0] = reinterpret_cast<int2*>(ws + p.off_run_q);
  m.sum[0] = reinterpret_cast<ChunkSum*>(ws + p.off_sum_q);
  m.nch[0] = p.nch_q;
  if (p.sides == 2) {
    m.ids[1] = seg->ids_kv;
    m.pos_in[1] = seg->pos_kv;
    m.pos_out[1] = p.derive_pos_kv ? reinterpret_cast<int*>(ws + p.off_pos_kv) : nullptr;
    m.run[1] = reinterpret_cast<int2*>(ws + p.off_run_kv);
    m.sum[1] = reinterpret_cast<ChunkSum*>(ws + p.off_sum_kv);
    m.nch[1] = p.nch_kv;
  } else {
    m.ids[1] = m.ids[0];
    m.pos_in[1] = m.pos_in[0];
    m.pos_out[1] = nullptr;
    m.run[1] = m.run[0];
    m.sum[1] = m.sum[0];
    m.nch[1] = m.nch[0];
  }
  m.route = reinterpret_cast<int*>(ws + p.off_route);

  view->ids_q = seg->ids_q;
  view->pos_q = p.derive_pos_q ? m.pos_out[0] : seg->pos_q;
  view->run_q = m.run[0];
  view->sum_q = m.sum[0];
  view->nch_q = p.nch_q;
  if (p.sides == 2) {
    view->ids_kv = seg->ids_kv;
    view->pos_kv = p.derive_pos_kv ? m.pos_out[1] : seg->pos_kv;
    view->run_kv = m.run[1];
    view->sum_kv = m.sum[1];
    view->nch_kv = p.nch_kv;
  } else {
    view->ids_kv = view->ids_q;
    view->pos_kv = view->pos_q;
    view->run_kv = view->run_q;
    view->sum_kv = view->sum_q;
    view->nch_kv = view->nch_q;
  }
  view->route = m.route;
  const bool ordered = ordered_tiles(d, p);
  if (ordered) {
    view->qord = reinterpret_cast<int*>(ws + p.off_qord);
    view->kord = reinterpret_cast<int*>(ws + p.off_kord);
  }
  if (!launch || d->B == 0 || (d->Sq == 0 && d->Skv == 0)) return ATTN_OK;
  hipError_t e = bps::launch_seg_meta(m, st);
  if (e != hipSuccess) return fail(ATTN_E_DEVICE, "segment metadata kernel: %s", hipGetErrorString(e));
  if (!ordered) return ATTN_OK;
  bps::TileOrderArgs o{};
  o.B = d->B; o.Sq = d->Sq; o.Skv = d->Skv; o.causal = d->causal;
  o.seg = *view;
  o.qord = reinterpret_cast<int*>(ws + p.off_qord);
  o.kord = reinterpret_cast<int*>(ws + p.off_kord);
  e = bps::launch_tile_order(o, st);
  if (e != hipSuccess) return fail(ATTN_E_DEVICE, "tile order kernel: %s", hipGetErrorString(e));
  return ATTN_OK;
}

// Head-dim pairs built for each element type (must match build.py).
#define BPS_BF16_DIMS(X) X(64, 64) X(64, 128) X(128, 64) X(128, 128) X(192, 64) X(192, 128)
#define BPS_FP32_DIMS(X) X(64, 64) X(64, 128) X(128, 64) X(128, 128)

template <typename T, int DQK, int DV, bool VAR>
hipError_t run_bwd_phases(int phases, const bps::BwdArgs& a, hipStream_t st) {
  hipError_t e = hipSuccess;
  if ((phases & ATTN_BWD_PREPARE) && (e = bps::launch_bwd_delta<T, DQK, DV, VAR>(a, st)) != hipSuccess) return e;
  if ((phases & ATTN_BWD_DKDV) && (e = bps::launch_bwd_dkdv<T, DQK, DV, VAR>(a, st)) != hipSuccess) return e;
  if ((phases & ATTN_BWD_DQ) && (e = bps::launch_bwd_dq<T, DQK, DV, VAR>(a, st)) != hipSuccess) return e;
  return e;
}

template <typename T, int DQK, int DV>
hipError_t run_fwd(int vm, const bps::FwdArgs& a, hipStream_t st) {
  if (vm == 2) return bps::launch_fwd<T, DQK, DV, 2>(a, st);
  if (vm == 1) return bps::launch_fwd<T, DQK, DV, 1>(a, st);
  return bps::launch_fwd<T, DQK, DV, 0>(a, st);
}

// var_delta: the prepare kernel writes the sink-gradient terms; var_attn:
// dK/dV and dQ apply a bias or a soft cap.  A sink alone needs neither: it
// enters the backward only through the saved LSE.
template <typename T, int DQK, int DV>
hipError_t run_bwd(int phases, bool var_delta, bool var_attn, const bps::BwdArgs& a, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (phases & ATTN_BWD_PREPARE) {
    e = var_delta ? run_bwd_phases<T, DQK, DV, true>(ATTN_BWD_PREPARE, a, st)
                  : run_bwd_phases<T, DQK, DV, false>(ATTN_BWD_PREPARE, a, st);
    if (e != hipSuccess) return e;
  }
  const int rest = phases & (ATTN_BWD_DKDV | ATTN_BWD_DQ);
  if (rest)
    e = var_attn ? run_bwd_phases<T, DQK, DV, true>(rest, a, st) : run_bwd_phases<T, DQK, DV, false>(rest, a, st);
  return e;
}

hipError_t dispatch_fwd(int dtype, int dqk, int dv, int vm, const bps::FwdArgs& a, hipStream_t st) {
#define BPS_FWD_BF16(DQK, DV) \
  if (dqk == DQK && dv == DV) return run_fwd<bps::bf16, DQK, DV>(vm, a, st);
#define BPS_FWD_FP32(DQK, DV) \
  if (dqk == DQK && dv == DV) return run_fwd<float, DQK, DV>(vm, a, st);
  if (dtype == ATTN_BF16) {
    BPS_BF16_DIMS(BPS_FWD_BF16)
  } else {
    BPS_FP32_DIMS(BPS_FWD_FP32)
  }
#undef BPS_FWD_BF16
#undef BPS_FWD_FP32
  return hipErrorInvalidValue;
}

hipError_t dispatch_bwd(int phases, int dtype, int dqk, int dv, bool var_delta, bool var_attn,
                        const bps::BwdArgs& a, hipStream_t st) {
#define BPS_BWD_BF16(DQK, DV) \
  if (dqk == DQK && dv == DV) return run_bwd<bps::bf16, DQK, DV>(phases, var_delta, var_attn, a, st);
#define BPS_BWD_FP32(DQK, DV) \
  if (dqk == DQK && dv == DV) return run_bwd<float, DQK, DV>(phases, var_delta, var_attn, a, st);
  if (dtype == ATTN_BF16) {
    BPS_BF16_DIMS(BPS_BWD_BF16)
  } else {
    BPS_FP32_DIMS(BPS_BWD_FP32)
  }
#undef BPS_BWD_BF16
#undef BPS_BWD_FP32
  return hipErrorInvalidValue;
}

int route_of(const Plan& p) {
  if (!p.meta) return ATTN_ROUTE_DENSE;
  return p.fast_candidate ? ATTN_ROUTE_FAST : ATTN_ROUTE_GENERAL;
}

// ATTN_LOG_ROUTE: after the metadata preparation of `call`, wait for the
// stream and report on stderr every batch row that the device moved from the
// requested fast route to the general route (debug only: it synchronises).
attn_status log_route(const attn_desc* d, const Plan& p, const char* ws, hipStream_t hs, const char* call) {
  if (!(d->flags & ATTN_LOG_ROUTE) || !p.meta || !p.fast_candidate || d->B == 0) return ATTN_OK;
  hipError_t e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return fail(ATTN_E_DEVICE, "route log: %s", hipGetErrorString(e));
  int32_t rows[256];
  const int32_t* src = reinterpret_cast<const int32_t*>(ws + p.off_route);
  int moved = 0;
  for (int b0 = 0; b0 < d->B; b0 += 256) {
    const int nb = std::min(256, d->B - b0);
    e = hipMemcpy(rows, src + b0, nb * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(ATTN_E_DEVICE, "route log: %s", hipGetErrorString(e));
    for (int i = 0; i < nb; ++i) {
      if (rows[i] == ATTN_ROUTE_FAST) continue;
      ++moved;
      std::fprintf(stderr, "bps_attn: %s: batch row %d takes the general route (fast route requested; the "
                   "device check of Q and KV metadata failed)\n", call, b0 + i);
    }
  }
  if (moved) std::fprintf(stderr, "bps_attn: %s: %d of %d batch rows on the general route\n", call, moved, d->B);
  return ATTN_OK;
}

attn_status check_ws(void* ws, size_t have, size_t need) {
  if (have < need) return fail(ATTN_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", have, need);
  if (need > 0 && ws == nullptr) return fail(ATTN_E_WORKSPACE, "workspace pointer is NULL (%zu bytes required)", need);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(ATTN_E_WORKSPACE, "workspace must be 256-byte aligned");
  return ATTN_OK;
}

attn_status check_align(const char* name, const void* ptr, int dtype) {
  (void)dtype;
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(ATTN_E_UNSUPPORTED, "%s must be 16-byte aligned", name);
  return ATTN_OK;
}

// ---------------------------------------------------------------- ring

// Elements a [B, S, H, D] tensor with these strides spans (first to last
// element), rounded up to 128 so consecutive partial copies stay aligned.
size_t span_of(const attn_strides& st, int B, int S, int H, int D) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0) return 0;
  const size_t n = (size_t)(B - 1) * st.batch + (size_t)(S - 1) * st.token + (size_t)(H - 1) * st.head + D;
  return (n + 127) & ~static_cast<size_t>(127);
}

struct RingPlan {
  int cp = 0, lq = 0, lkv = 0;
  attn_desc sd{};              // descriptor of one (Q shard, KV shard) step
  size_t esize = 0;
  size_t span_q = 0, span_k = 0, span_v = 0, span_o = 0;
  size_t off_ids_q = 0, off_pos_q = 0, off_ids_kv = 0, off_pos_kv = 0;
  size_t off_lse = 0;          // fwd: partial LSEs; bwd: shard-major LSE
  size_t off_p0 = 0;           // fwd: partial O; bwd: partial dQ
  size_t off_p1 = 0, off_p2 = 0;   // bwd: partial dK, dV
  size_t off_sub = 0, sub_bytes = 0;
  size_t ws = 0;
};

attn_status make_ring_plan(const attn_desc* d, const attn_segments* seg, int cp, bool bwd, RingPlan* rp) {
  Plan p;
  attn_status st = make_plan(d, seg, &p);
  if (st != ATTN_OK) return st;
  if (cp < 1) return fail(ATTN_E_INVALID, "cp must be at least 1 (got %d)", cp);
  if (p.fused) return fail(ATTN_E_UNSUPPORTED, "the ring emulation does not take ATTN_FUSED_BWD");
  if (d->Sq % cp || d->Skv % cp)
    return fail(ATTN_E_INVALID, "Sq (%d) and Skv (%d) must be multiples of cp (%d)", d->Sq, d->Skv, cp);
  rp->cp = cp;
  rp->lq = d->Sq / cp;
  rp->lkv = d->Skv / cp;
  rp->sd = *d;
  rp->sd.Sq = rp->lq;
  rp->sd.Skv = rp->lkv;
  rp->esize = d->dtype == ATTN_BF16 ? 2 : 4;
  rp->span_q = span_of(d->q, d->B, d->Sq, d->Hq, d->Dqk);
  rp->span_k = span_of(d->k, d->B, d->Skv, d->Hkv, d->Dqk);
  rp->span_v = span_of(d->v, d->B, d->Skv, d->Hkv, d->Dv);
  rp->span_o = span_of(d->o, d->B, d->Sq, d->Hq, d->Dv);
  // Every step carries metadata in separate Q and KV buffers (sizes only
  // depend on that, so placeholder pointers serve for the query).
  attn_segments probe{reinterpret_cast<const int32_t*>(256), reinterpret_cast<const int32_t*>(512),
                      reinterpret_cast<const int32_t*>(768), reinterpret_cast<const int32_t*>(1024)};
  Plan sp;
  if ((st = make_plan(&rp->sd, &probe, &sp)) != ATTN_OK) return st;
  rp->sub_bytes = bwd ? sp.ws_bwd : sp.ws_fwd;
  const size_t B = d->B;
  size_t off = 0;
  rp->off_ids_q = off; off = align_up(off + B * d->Sq * 4);
  rp->off_pos_q = off; off = align_up(off + B * d->Sq * 4);
  rp->off_ids_kv = off; off = align_up(off + B * d->Skv * 4);
  rp->off_pos_kv = off; off = align_up(off + B * d->Skv * 4);
  const size_t nlse = B * d->Hq * d->Sq;
  if (!bwd) {
    rp->off_lse = off; off = align_up(off + (size_t)cp * nlse * 4);
    rp->off_p0 = off; off = align_up(off + (size_t)cp * rp->span_o * rp->esize);
  } else {
    rp->off_lse = off; off = align_up(off + nlse * 4);
    rp->off_p0 = off; off = align_up(off + (size_t)cp * rp->span_q * rp->esize);
    rp->off_p1 = off; off = align_up(off + (size_t)cp * rp->span_k * rp->esize);
    rp->off_p2 = off; off = align_up(off + (size_t)cp * rp->span_v * rp->esize);
  }
  rp->off_sub = off; off = align_up(off + rp->sub_bytes);
  rp->ws = off;
  return ATTN_OK;
}

// Shard-major metadata of both sides in the workspace (global positions).
attn_status ring_metadata(const attn_desc* d, const attn_segments* seg, const RingPlan& rp, char* ws,
                          hipStream_t hs) {
  bps::RingMetaArgs m{};
  m.B = d->B; m.Sq = d->Sq; m.Skv = d->Skv; m.cp = rp.cp;
  if (seg) {
    const bool self = seg->ids_kv == nullptr;
    m.ids[0] = seg->ids_q;
    m.pos[0] = seg->pos_q;
    m.ids[1] = self ? seg->ids_q : seg->ids_kv;
    m.pos[1] = self ? seg->pos_q : seg->pos_kv;
  }
  m.ids_out[0] = reinterpret_cast<int*>(ws + rp.off_ids_q);
  m.pos_out[0] = reinterpret_cast<int*>(ws + rp.off_pos_q);
  m.ids_out[1] = reinterpret_cast<int*>(ws + rp.off_ids_kv);
  m.pos_out[1] = reinterpret_cast<int*>(ws + rp.off_pos_kv);
  hipError_t e = bps::launch_ring_meta(m, hs);
  if (e != hipSuccess) return fail(ATTN_E_DEVICE, "ring metadata kernel: %s", hipGetErrorString(e));
  return ATTN_OK;
}

// Step (rank r, ring step t): Q shard r against KV shard (r - t) mod cp.
struct RingStep {
  attn_desc d;
  attn_segments seg;
  int s;
};

RingStep ring_step(const RingPlan& rp, int B, char* ws, int r, int t) {
  RingStep x;
  x.d = rp.sd;
  if (t > 0) x.d.flags |= ATTN_FORCE_GENERAL;   // rotated steps: general route
  x.s = (r - t + rp.cp) % rp.cp;
  const size_t oq = (size_t)r * B * rp.lq, okv = (size_t)x.s * B * rp.lkv;
  x.seg.ids_q = reinterpret_cast<const int32_t*>(ws + rp.off_ids_q) + oq;
  x.seg.pos_q = reinterpret_cast<const int32_t*>(ws + rp.off_pos_q) + oq;
  x.seg.ids_kv = reinterpret_cast<const int32_t*>(ws + rp.off_ids_kv) + okv;
  x.seg.pos_kv = reinterpret_cast<const int32_t*>(ws + rp.off_pos_kv) + okv;
  return x;
}

const char* cadd(const void* base, size_t elems, size_t esize) {
  return static_cast<const char*>(base) + elems * esize;
}
char* madd(void* base, size_t elems, size_t esize) { return static_cast<char*>(base) + elems * esize; }


// ------------------------------------------------------------ variants

// Workspace and checks of the variant arguments (attn_variant).  The plain
// workspace layout of make_plan is a prefix of the variant one.
struct VarPlan {
  bool on = false;            // any variant requested: the VAR kernels run
  bool dbias_partial = false; // one bias slab for several batch rows: fp32 partials, then a sum
  size_t n_ml = 0;            // max-logit partials per head
  size_t off_ml = 0, off_dsink = 0, off_dbias = 0;
  size_t ws_fwd = 0, ws_bwd = 0;
};

attn_status make_var_plan(const attn_desc* d, const Plan& p, const attn_variant* var, VarPlan* vp) {
  vp->ws_fwd = p.ws_fwd;
  vp->ws_bwd = p.ws_bwd;
  if (!var) return ATTN_OK;
  if (!std::isfinite(var->softcap) || var->softcap < 0.f)
    return fail(ATTN_E_INVALID, "softcap must be finite and >= 0");
  if (p.fused && (var->bias || var->softcap > 0.f))
    return fail(ATTN_E_UNSUPPORTED, "the fused backward is not built for a bias or a soft cap");
  if (var->bias && var->bias_batch != 1 && var->bias_batch != d->B)
    return fail(ATTN_E_INVALID, "bias_batch must be 1 or B (%d), got %d", d->B, var->bias_batch);
  if (var->dbias && !var->bias) return fail(ATTN_E_INVALID, "dbias requested without a bias");
  if (var->dsink && !var->sink) return fail(ATTN_E_INVALID, "dsink requested without sink logits");
  if ((var->bias && reinterpret_cast<uintptr_t>(var->bias) % 16) ||
      (var->dbias && reinterpret_cast<uintptr_t>(var->dbias) % 16))
    return fail(ATTN_E_UNSUPPORTED, "bias and dbias must be 16-byte aligned");
  if ((var->sink && reinterpret_cast<uintptr_t>(var->sink) % 4) ||
      (var->max_logit && reinterpret_cast<uintptr_t>(var->max_logit) % 4) ||
      (var->dsink && reinterpret_cast<uintptr_t>(var->dsink) % 4))
    return fail(ATTN_E_INVALID, "sink, max_logit and dsink must be 4-byte aligned");
  vp->on = var->bias || var->softcap > 0.f || var->sink || var->max_logit || var->dbias || var->dsink;
  if (!vp->on) return ATTN_OK;
  size_t off = p.ws_fwd;
  if (var->max_logit) {
    const size_t n_qt = (d->Sq + 127) / 128;   // forward query tiles of 128 rows, 4 waves each
    vp->n_ml = (size_t)d->B * n_qt * 4;
    vp->off_ml = off;
    off = align_up(off + vp->n_ml * d->Hq * sizeof(float));
  }
  vp->ws_fwd = off;
  off = p.ws_bwd;
  const size_t nrow = (size_t)d->B * d->Hq * d->Sq;
  if (var->dsink) {
    vp->off_dsink = off;
    off = align_up(off + nrow * sizeof(float));
  }
  vp->dbias_partial = var->dbias && var->bias_batch == 1 && d->B > 1;
  if (vp->dbias_partial) {
    vp->off_dbias = off;
    off = align_up(off + nrow * (size_t)d->Skv * sizeof(float));
  }
  vp->ws_bwd = off;
  return ATTN_OK;
}

bps::VarView var_view(const attn_desc* d, const attn_variant* var, const VarPlan& vp, char* ws, bool bwd) {
  bps::VarView v{};
  if (!vp.on) return v;
  const int64_t slab = (int64_t)d->Hq * d->Sq * d->Skv;
  v.bias = var->bias;
  v.bias_b = (var->bias && var->bias_batch > 1) ? slab : 0;
  v.softcap = var->softcap;
  v.cap_k = var->softcap > 0.f ? 2.f * bps::kLog2e / var->softcap : 0.f;
  v.cap_l2 = var->softcap * bps::kLog2e;
  v.cap_inv = var->softcap > 0.f ? 1.f / v.cap_l2 : 0.f;
  v.sink = var->sink;
  if (!bwd) {
    v.ml_part = var->max_logit ? reinterpret_cast<float*>(ws + vp.off_ml) : nullptr;
    return v;
  }
  if (var->dbias) {
    v.dbias = vp.dbias_partial ? static_cast<void*>(ws + vp.off_dbias) : var->dbias;
    v.dbias_f32 = vp.dbias_partial ? 1 : 0;
    v.dbias_b = (vp.dbias_partial || var->bias_batch > 1) ? slab : 0;
  }
  v.dsink_row = var->dsink ? reinterpret_cast<float*>(ws + vp.off_dsink) : nullptr;
  return v;
}

// ------------------------------------------------------------ scratch of attn_bwd_noalloc

// The workspace of attn_bwd_noalloc: a file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  Host code
// never uses the array's name as an address: its device address is looked
// up once per device, with that device current, and kept here.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

attn_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_E_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(ATTN_E_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

attn_status fwd_impl(const attn_desc* d, const attn_segments* seg, const attn_variant* var, const void* q,
                     const void* k, const void* v, void* o, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream, int32_t* route_out) {
  try {
    Plan p;
    attn_status st = make_plan(d, seg, &p);
    if (st != ATTN_OK) return st;
    VarPlan vp;
    if ((st = make_var_plan(d, p, var, &vp)) != ATTN_OK) return st;
    const long long nq = (long long)d->B * d->Sq * d->Hq, nkv = (long long)d->B * d->Skv * d->Hkv;
    if (need_nonnull(q, nq) || need_nonnull(o, nq) || need_nonnull(lse, nq))
      return fail(ATTN_E_INVALID, "q, o and lse must not be NULL");
    if (need_nonnull(k, nkv) || need_nonnull(v, nkv)) return fail(ATTN_E_INVALID, "k and v must not be NULL");
    if ((st = check_align("q", q, d->dtype)) || (st = check_align("k", k, d->dtype)) ||
        (st = check_align("v", v, d->dtype)) || (st = check_align("o", o, d->dtype)))
      return st;
    if ((st = check_ws(workspace, workspace_bytes, vp.ws_fwd)) != ATTN_OK) return st;
    if (route_out) *route_out = route_of(p);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    bps::FwdArgs a{};
    a.s = shape_of(d, p);
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.sq = strides_of(d->q); a.sk = strides_of(d->k); a.sv = strides_of(d->v); a.so = strides_of(d->o);
    a.var = var_view(d, var, vp, ws, false);
    if (d->Sq > 0) {
      if ((st = prepare_segments(d, seg, p, ws, hs, &a.seg)) != ATTN_OK) return st;
      if ((st = log_route(d, p, ws, hs, "forward")) != ATTN_OK) return st;
      const int vm = !vp.on ? 0 : (var->bias != nullptr || var->softcap > 0.f) ? 2 : 1;
      hipError_t e = dispatch_fwd(d->dtype, d->Dqk, d->Dv, vm, a, hs);
      if (e != hipSuccess) return fail(ATTN_E_DEVICE, "forward launch: %s", hipGetErrorString(e));
    }
    if (vp.on && var->max_logit) {
      hipError_t e = bps::launch_max_logit_reduce(a.var.ml_part, vp.n_ml, d->Hq, var->max_logit, hs);
      if (e != hipSuccess) return fail(ATTN_E_DEVICE, "max-logit launch: %s", hipGetErrorString(e));
    }
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_DEVICE, "unexpected host exception");
  }
}

attn_status bwd_impl(int32_t phases, const attn_desc* d, const attn_segments* seg, const attn_variant* var,
                     const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream,
                     int32_t* route_out, bool allow_split = true, bool use_scratch = false) {
  try {
    if (phases <= 0 || (phases & ~ATTN_BWD_ALL))
      return fail(ATTN_E_INVALID, "phases must be a nonzero combination of ATTN_BWD_* bits (got %d)", phases);
    Plan p;
    attn_status st = make_plan(d, seg, &p, allow_split);
    if (st != ATTN_OK) return st;
    VarPlan vp;
    if ((st = make_var_plan(d, p, var, &vp)) != ATTN_OK) return st;
    const long long nq = (long long)d->B * d->Sq * d->Hq, nkv = (long long)d->B * d->Skv * d->Hkv;
    if (need_nonnull(dout, nq)) return fail(ATTN_E_INVALID, "dout must not be NULL");
    if ((phases & ATTN_BWD_PREPARE) && (need_nonnull(o, nq) || need_nonnull(lse, nq)))
      return fail(ATTN_E_INVALID, "o and lse must not be NULL");
    if ((phases & (ATTN_BWD_DKDV | ATTN_BWD_DQ)) && (need_nonnull(q, nq) || need_nonnull(k, nkv) || need_nonnull(v, nkv)))
      return fail(ATTN_E_INVALID, "q, k and v must not be NULL");
    if ((phases & ATTN_BWD_DQ) && need_nonnull(dq, nq)) return fail(ATTN_E_INVALID, "dq must not be NULL");
    if ((phases & ATTN_BWD_DKDV) && (need_nonnull(dk, nkv) || need_nonnull(dv, nkv)))
      return fail(ATTN_E_INVALID, "dk and dv must not be NULL");
    if ((st = check_align("q", q, d->dtype)) || (st = check_align("k", k, d->dtype)) ||
        (st = check_align("v", v, d->dtype)) || (st = check_align("o", o, d->dtype)) ||
        (st = check_align("dout", dout, d->dtype)) || (st = check_align("dq", dq, d->dtype)) ||
        (st = check_align("dk", dk, d->dtype)) || (st = check_align("dv", dv, d->dtype)))
      return st;
    if ((phases & ATTN_BWD_DQ) && (st = check_disjoint("q (and dQ)", d->q, d->B, d->Sq, d->Hq, d->Dqk)) != ATTN_OK)
      return st;
    if ((phases & ATTN_BWD_DKDV) &&
        ((st = check_disjoint("k (and dK)", d->k, d->B, d->Skv, d->Hkv, d->Dqk)) != ATTN_OK ||
         (st = check_disjoint("v (and dV)", d->v, d->B, d->Skv, d->Hkv, d->Dv)) != ATTN_OK))
      return st;
    if (use_scratch) {   // attn_bwd_noalloc: every argument checked; now the device's scratch array
      if (vp.ws_bwd > kScratchBytes)
        return fail(ATTN_E_WORKSPACE, "this backward needs %zu bytes of scratch; attn_bwd_noalloc holds %zu "
                    "(B * Hq * Sq up to about 4 million rows): use attn_bwd with a workspace", vp.ws_bwd,
                    kScratchBytes);
      if ((st = scratch_of_current_device(&workspace)) != ATTN_OK) return st;
      workspace_bytes = kScratchBytes;
    }
    if ((st = check_ws(workspace, workspace_bytes, vp.ws_bwd)) != ATTN_OK) return st;
    if (route_out) *route_out = route_of(p);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    bps::BwdArgs a{};
    a.s = shape_of(d, p);
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.sq = strides_of(d->q); a.sk = strides_of(d->k); a.sv = strides_of(d->v); a.so = strides_of(d->o);
    a.delta = reinterpret_cast<float*>(ws + p.off_delta);
    a.lse2 = reinterpret_cast<float*>(ws + p.off_lse2);
    a.dqp = p.fused ? reinterpret_cast<float*>(ws + p.off_dqp) : nullptr;
    a.kv_split = p.kv_split;
    a.dkvp = p.kv_split > 1 ? reinterpret_cast<float*>(ws + p.off_dkvp) : nullptr;
    a.var = var_view(d, var, vp, ws, true);
    const bool prep = (phases & ATTN_BWD_PREPARE) != 0;
    const size_t esize = d->dtype == ATTN_BF16 ? 2 : 4;
    const size_t slab = (size_t)d->Hq * d->Sq * d->Skv;
    hipError_t e = hipSuccess;
    // Variants, before the attention kernels: the dbias target starts at zero
    // (dK/dV writes only the tiles it visits).
    if (prep && vp.on && var->dbias) {
      e = vp.dbias_partial ? bps::launch_zero_fill(a.var.dbias, (size_t)d->B * slab * sizeof(float), hs)
                           : bps::launch_zero_fill(var->dbias, (size_t)var->bias_batch * slab * esize, hs);
      if (e != hipSuccess) return fail(ATTN_E_DEVICE, "dbias fill launch: %s", hipGetErrorString(e));
    }
    if (!(d->Sq == 0 && d->Skv == 0)) {
      if ((st = prepare_segments(d, seg, p, ws, hs, &a.seg, prep)) != ATTN_OK) return st;
      if (prep && (st = log_route(d, p, ws, hs, "backward")) != ATTN_OK) return st;
      const bool var_attn = vp.on && (var->bias != nullptr || var->softcap > 0.f);
      const bool var_delta = vp.on && var->dsink != nullptr;
      e = dispatch_bwd(phases, d->dtype, d->Dqk, d->Dv, var_delta, var_attn, a, hs);
      if (e != hipSuccess) return fail(ATTN_E_DEVICE, "backward launch: %s", hipGetErrorString(e));
    }
    // Variants, after: the per-head sink gradient (from the prepare phase's
    // per-row terms) and the sum of the dbias partials over batch rows.
    if (prep && vp.on && var->dsink) {
      e = bps::launch_dsink_reduce(a.var.dsink_row, d->B, d->Hq, d->Sq, var->dsink, hs);
      if (e != hipSuccess) return fail(ATTN_E_DEVICE, "dsink launch: %s", hipGetErrorString(e));
    }
    if ((phases & ATTN_BWD_DKDV) && vp.dbias_partial) {
      e = bps::launch_dbias_reduce(d->dtype == ATTN_BF16, static_cast<const float*>(a.var.dbias), d->B, slab,
                                   var->dbias, hs);
      if (e != hipSuccess) return fail(ATTN_E_DEVICE, "dbias sum launch: %s", hipGetErrorString(e));
    }
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_DEVICE, "unexpected host exception");
  }
}

}  // namespace

extern "C" {

size_t attn_fwd_workspace_size(const attn_desc* desc, const attn_segments* seg) {
  Plan p;
  return make_plan(desc, seg, &p) == ATTN_OK ? p.ws_fwd : 0;
}

size_t attn_bwd_workspace_size(const attn_desc* desc, const attn_segments* seg) {
  Plan p;
  return make_plan(desc, seg, &p) == ATTN_OK ? p.ws_bwd : 0;
}

attn_status attn_fwd(const attn_desc* d, const attn_segments* seg, const void* q, const void* k, const void* v,
                     void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                     int32_t* route_out) {
  return fwd_impl(d, seg, nullptr, q, k, v, o, lse, workspace, workspace_bytes, stream, route_out);
}

attn_status attn_bwd_phase(int32_t phases, const attn_desc* d, const attn_segments* seg, const void* q,
                           const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
                           void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream,
                           int32_t* route_out) {
  return bwd_impl(phases, d, seg, nullptr, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream,
                  route_out);
}

attn_status attn_bwd(const attn_desc* d, const attn_segments* seg, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, void* stream, int32_t* route_out) {
  return attn_bwd_phase(ATTN_BWD_ALL, d, seg, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                        stream, route_out);
}

attn_status attn_bwd_noalloc(const attn_desc* d, const attn_segments* seg, const void* q, const void* k,
                             const void* v, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                             void* dv, void* stream, int32_t* route_out) {
  try {
    if (d && (d->flags & ATTN_FUSED_BWD))
      return fail(ATTN_E_UNSUPPORTED, "attn_bwd_noalloc does not take ATTN_FUSED_BWD");
    return bwd_impl(ATTN_BWD_ALL, d, seg, nullptr, q, k, v, o, lse, dout, dq, dk, dv, nullptr, 0, stream,
                    route_out, /*allow_split=*/false, /*use_scratch=*/true);
  } catch (...) {
    return fail(ATTN_E_DEVICE, "unexpected host exception");
  }
}

size_t attn_fwd_ex_workspace_size(const attn_desc* desc, const attn_segments* seg, const attn_variant* var) {
  Plan p;
  VarPlan vp;
  if (make_plan(desc, seg, &p) != ATTN_OK || make_var_plan(desc, p, var, &vp) != ATTN_OK) return 0;
  return vp.ws_fwd;
}

size_t attn_bwd_ex_workspace_size(const attn_desc* desc, const attn_segments* seg, const attn_variant* var) {
  Plan p;
  VarPlan vp;
  if (make_plan(desc, seg, &p) != ATTN_OK || make_var_plan(desc, p, var, &vp) != ATTN_OK) return 0;
  return vp.ws_bwd;
}

attn_status attn_fwd_ex(const attn_desc* d, const attn_segments* seg, const attn_variant* var, const void* q,
                        const void* k, const void* v, void* o, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream, int32_t* route_out) {
  return fwd_impl(d, seg, var, q, k, v, o, lse, workspace, workspace_bytes, stream, route_out);
}

attn_status attn_bwd_ex_phase(int32_t phases, const attn_desc* d, const attn_segments* seg, const attn_variant* var,
                              const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, void* stream, int32_t* route_out) {
  return bwd_impl(phases, d, seg, var, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream,
                  route_out);
}

attn_status attn_bwd_ex(const attn_desc* d, const attn_segments* seg, const attn_variant* var, const void* q,
                        const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
                        void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream,
                        int32_t* route_out) {
  return bwd_impl(ATTN_BWD_ALL, d, seg, var, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream,
                  route_out);
}

attn_status attn_debug_mask(const attn_desc* d, const attn_segments* seg, uint8_t* mask_out, int32_t* route_rows,
                            void* workspace, size_t workspace_bytes, void* stream) {
  try {
    Plan p;
    attn_status st = make_plan(d, seg, &p);
    if (st != ATTN_OK) return st;
    if (need_nonnull(mask_out, (long long)d->B * d->Sq * d->Skv))
      return fail(ATTN_E_INVALID, "mask_out must not be NULL");
    if ((st = check_ws(workspace, workspace_bytes, p.ws_fwd)) != ATTN_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    bps::MaskArgs a{};
    a.B = d->B; a.Sq = d->Sq; a.Skv = d->Skv; a.causal = d->causal; a.has_meta = p.meta ? 1 : 0;
    a.mask = mask_out;
    a.route_rows = route_rows;
    if ((st = prepare_segments(d, seg, p, static_cast<char*>(workspace), hs, &a.seg)) != ATTN_OK) return st;
    hipError_t e = bps::launch_debug_mask(a, hs);
    if (e != hipSuccess) return fail(ATTN_E_DEVICE, "mask launch: %s", hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_DEVICE, "unexpected host exception");
  }
}

attn_status attn_route_rows(const attn_desc* d, const attn_segments* seg, const void* workspace,
                            size_t workspace_bytes, int32_t* route_rows, void* stream) {
  try {
    Plan p;
    attn_status st = make_plan(d, seg, &p);
    if (st != ATTN_OK) return st;
    if (need_nonnull(route_rows, d->B)) return fail(ATTN_E_INVALID, "route_rows must not be NULL");
    if (p.meta && (st = check_ws(const_cast<void*>(workspace), workspace_bytes, p.ws_fwd)) != ATTN_OK) return st;
    const int* src = p.meta ? reinterpret_cast<const int*>(static_cast<const char*>(workspace) + p.off_route) : nullptr;
    hipError_t e = bps::launch_route_rows(src, d->B, route_rows, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_E_DEVICE, "route copy launch: %s", hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_DEVICE, "unexpected host exception");
  }
}

size_t attn_ring_fwd_workspace_size(const attn_desc* desc, const attn_segments* seg, int32_t cp) {
  RingPlan rp;
  return make_ring_plan(desc, seg, cp, false, &rp) == ATTN_OK ? rp.ws : 0;
}

size_t attn_ring_bwd_workspace_size(const attn_desc* desc, const attn_segments* seg, int32_t cp) {
  RingPlan rp;
  return make_ring_plan(desc, seg, cp, true, &rp) == ATTN_OK ? rp.ws : 0;
}

attn_status attn_ring_fwd(const attn_desc* d, const attn_segments* seg, int32_t cp, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  try {
    RingPlan rp;
    attn_status st = make_ring_plan(d, seg, cp, false, &rp);
    if (st != ATTN_OK) return st;
    const long long nq = (long long)d->B * d->Sq * d->Hq, nkv = (long long)d->B * d->Skv * d->Hkv;
    if (need_nonnull(q, nq) || need_nonnull(o, nq) || need_nonnull(lse, nq))
      return fail(ATTN_E_INVALID, "q, o and lse must not be NULL");
    if (need_nonnull(k, nkv) || need_nonnull(v, nkv)) return fail(ATTN_E_INVALID, "k and v must not be NULL");
    if ((st = check_align("q", q, d->dtype)) || (st = check_align("k", k, d->dtype)) ||
        (st = check_align("v", v, d->dtype)) || (st = check_align("o", o, d->dtype)))
      return st;
    if ((st = check_ws(workspace, workspace_bytes, rp.ws)) != ATTN_OK) return st;
    if (d->Sq == 0) return ATTN_OK;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    if ((st = ring_metadata(d, seg, rp, ws, hs)) != ATTN_OK) return st;
    const size_t es = rp.esize;
    float* lse_parts = reinterpret_cast<float*>(ws + rp.off_lse);
    const size_t nl = (size_t)d->B * d->Hq * rp.lq;
    for (int t = 0; t < cp; ++t)
      for (int r = 0; r < cp; ++r) {
        const RingStep x = ring_step(rp, d->B, ws, r, t);
        const size_t rq = (size_t)r * rp.lq, rkv = (size_t)x.s * rp.lkv;
        st = attn_fwd(&x.d, &x.seg, cadd(q, rq * d->q.token, es), cadd(k, rkv * d->k.token, es),
                      cadd(v, rkv * d->v.token, es), madd(ws + rp.off_p0, t * rp.span_o + rq * d->o.token, es),
                      lse_parts + ((size_t)t * cp + r) * nl, ws + rp.off_sub, rp.sub_bytes, stream, nullptr);
        if (st != ATTN_OK) return st;
      }
    bps::RingMergeArgs m{};
    m.B = d->B; m.Sq = d->Sq; m.Hq = d->Hq; m.Dv = d->Dv; m.cp = cp;
    m.o_parts = ws + rp.off_p0;
    m.part_elems = rp.span_o;
    m.lse_parts = lse_parts;
    m.o = o; m.lse = lse;
    m.so = strides_of(d->o);
    hipError_t e = bps::launch_ring_merge(d->dtype == ATTN_BF16, m, hs);
    if (e != hipSuccess) return fail(ATTN_E_DEVICE, "ring merge: %s", hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_DEVICE, "unexpected host exception");
  }
}

attn_status attn_ring_bwd(const attn_desc* d, const attn_segments* seg, int32_t cp, const void* q, const void* k,
                          const void* v, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                          void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    RingPlan rp;
    attn_status st = make_ring_plan(d, seg, cp, true, &rp);
    if (st != ATTN_OK) return st;
    const long long nq = (long long)d->B * d->Sq * d->Hq, nkv = (long long)d->B * d->Skv * d->Hkv;
    if (need_nonnull(q, nq) || need_nonnull(o, nq) || need_nonnull(lse, nq) || need_nonnull(dout, nq) ||
        need_nonnull(dq, nq))
      return fail(ATTN_E_INVALID, "q, o, lse, dout and dq must not be NULL");
    if (need_nonnull(k, nkv) || need_nonnull(v, nkv) || need_nonnull(dk, nkv) || need_nonnull(dv, nkv))
      return fail(ATTN_E_INVALID, "k, v, dk and dv must not be NULL");
    if ((st = check_align("q", q, d->dtype)) || (st = check_align("k", k, d->dtype)) ||
        (st = check_align("v", v, d->dtype)) || (st = check_align("o", o, d->dtype)) ||
        (st = check_align("dout", dout, d->dtype)) || (st = check_align("dq", dq, d->dtype)) ||
        (st = check_align("dk", dk, d->dtype)) || (st = check_align("dv", dv, d->dtype)))
      return st;
    if ((st = check_disjoint("q (and dQ)", d->q, d->B, d->Sq, d->Hq, d->Dqk)) != ATTN_OK ||
        (st = check_disjoint("k (and dK)", d->k, d->B, d->Skv, d->Hkv, d->Dqk)) != ATTN_OK ||
        (st = check_disjoint("v (and dV)", d->v, d->B, d->Skv, d->Hkv, d->Dv)) != ATTN_OK)
      return st;
    if ((st = check_ws(workspace, workspace_bytes, rp.ws)) != ATTN_OK) return st;
    if (d->Sq == 0 && d->Skv == 0) return ATTN_OK;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    if ((st = ring_metadata(d, seg, rp, ws, hs)) != ATTN_OK) return st;
    float* lse_sh = reinterpret_cast<float*>(ws + rp.off_lse);
    bps::RingLseArgs la{d->B, d->Hq, d->Sq, cp, lse, lse_sh};
    hipError_t e = bps::launch_ring_lse_shards(la, hs);
    if (e != hipSuccess) return fail(ATTN_E_DEVICE, "ring LSE shards: %s", hipGetErrorString(e));
    const size_t es = rp.esize;
    const size_t nl = (size_t)d->B * d->Hq * rp.lq;
    for (int t = 0; t < cp; ++t)
      for (int r = 0; r < cp; ++r) {
        const RingStep x = ring_step(rp, d->B, ws, r, t);
        const size_t rq = (size_t)r * rp.lq, rkv = (size_t)x.s * rp.lkv;
        st = attn_bwd(&x.d, &x.seg, cadd(q, rq * d->q.token, es), cadd(k, rkv * d->k.token, es),
                      cadd(v, rkv * d->v.token, es), cadd(o, rq * d->o.token, es), lse_sh + (size_t)r * nl,
                      cadd(dout, rq * d->o.token, es), madd(ws + rp.off_p0, t * rp.span_q + rq * d->q.token, es),
                      madd(ws + rp.off_p1, t * rp.span_k + rkv * d->k.token, es),
                      madd(ws + rp.off_p2, t * rp.span_v + rkv * d->v.token, es), ws + rp.off_sub, rp.sub_bytes,
                      stream, nullptr);
        if (st != ATTN_OK) return st;
      }
    const int bf = d->dtype == ATTN_BF16;
    bps::RingReduceArgs ra{d->B, d->Sq, d->Hq, d->Dqk, cp, ws + rp.off_p0, rp.span_q, dq, strides_of(d->q)};
    if ((e = bps::launch_ring_reduce(bf, ra, hs)) != hipSuccess)
      return fail(ATTN_E_DEVICE, "ring reduce dq: %s", hipGetErrorString(e));
    ra = bps::RingReduceArgs{d->B, d->Skv, d->Hkv, d->Dqk, cp, ws + rp.off_p1, rp.span_k, dk, strides_of(d->k)};
    if ((e = bps::launch_ring_reduce(bf, ra, hs)) != hipSuccess)
      return fail(ATTN_E_DEVICE, "ring reduce dk: %s", hipGetErrorString(e));
    ra = bps::RingReduceArgs{d->B, d->Skv, d->Hkv, d->Dv, cp, ws + rp.off_p2, rp.span_v, dv, strides_of(d->v)};
    if ((e = bps::launch_ring_reduce(bf, ra, hs)) != hipSuccess)
      return fail(ATTN_E_DEVICE, "ring reduce dv: %s", hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_DEVICE, "unexpected host exception");
  }
}

const char* attn_last_error(void) { return g_err.c_str(); }

const char* attn_version(void) { return "bps_attn 0.1 (gfx950)"; }

}  // extern "C"
