// Segment metadata preparation (runs before every attention kernel that has
// THD metadata) and the mask dump used by the tests.
//
// Per batch row and per side (Q, and KV when its metadata are separate) one
// 1024-thread workgroup scans the row of segment ids:
//   * run start and end of every token's contiguous id run (the device form
//     of the cu_seqlens-style ragged offsets of TransformerEngine PR 2358,
//     review of the ragged offset tensor); (0, 0) for padding (id 0);
//   * positions derived from ids when none are given (offset inside the run,
//     the helper of "[JAX] Fix batcher in FusedAttn primitive ...",
//     Description);
//   * one summary per 32 tokens (ids, positions, run bounds of the tokens
//     with a nonzero id) used by the kernels to skip or fully accept tiles;
//   * on the Q side, whether the fast (boundary-only) route is exact for the
//     row: Q and KV metadata equal, runs of nonzero ids increasing, positions
//     equal to run offsets ("[JAX] Align fused attn backward output gradient
//     sharding ...", Changes 3 and 4).  The route can only fall back to the
//     general path here, never the other way.
#include "bps_args.hpp"

namespace bps {

namespace {

constexpr int kSegThreads = 1024;
constexpr int kSegItems = 8;
constexpr int kSegRound = kSegThreads * kSegItems;
constexpr int kSegWaves = kSegThreads / 64;

__device__ inline int op_max(int a, int b) { return a > b ? a : b; }
__device__ inline int op_min(int a, int b) { return a < b ? a : b; }
// Token index i clamped into [0, S) (S >= 1): loads of a round are issued
// unconditionally at clamped indices and out-of-row items ignore the value,
// so no load sits behind a per-lane branch.
__device__ inline int clamp_tok(int i, int S) { return i < 0 ? 0 : (i < S ? i : S - 1); }

// One thread's tokens base .. base + 7 of a row.  All of a row passes
// through one CU, so the loads and stores are 16 bytes per lane where the
// row start is 16-byte aligned (base is a multiple of 8) and the eight
// tokens are inside the row; elsewhere element accesses (loads at clamped
// indices, stores only inside the row).
__device__ inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
__device__ inline void load8(const int* p, int base, int S, bool vec, int (&o)[kSegItems]) {
  if (vec && base + kSegItems <= S) {
    const int4 x = *reinterpret_cast<const int4*>(p + base);
    const int4 y = *reinterpret_cast<const int4*>(p + base + 4);
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
  } else {
#pragma unroll
    for (int k = 0; k < kSegItems; ++k) o[k] = p[clamp_tok(base + k, S)];
  }
}
__device__ inline void store8(int* p, int base, int S, bool vec, const int (&v)[kSegItems]) {
  if (vec && base + kSegItems <= S) {
    *reinterpret_cast<int4*>(p + base) = make_int4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<int4*>(p + base + 4) = make_int4(v[4], v[5], v[6], v[7]);
  } else {
#pragma unroll
    for (int k = 0; k < kSegItems; ++k)
      if (base + k < S) p[base + k] = v[k];
  }
}
__device__ inline void store8_run(int2* p, int base, int S, bool vec, const int (&x)[kSegItems],
                                  const int (&y)[kSegItems]) {
  if (vec && base + kSegItems <= S) {
#pragma unroll
    for (int k = 0; k < kSegItems; k += 2)
      *reinterpret_cast<int4*>(p + base + k) = make_int4(x[k], y[k], x[k + 1], y[k + 1]);
  } else {
#pragma unroll
    for (int k = 0; k < kSegItems; ++k)
      if (base + k < S) p[base + k] = make_int2(x[k], y[k]);
  }
}

// Exclusive scan over the threads of the workgroup: forward combines the
// values of threads before this one, reverse those after it.  Returns the
// exclusive result and stores the combination of all threads in *total.
template <bool MAXOP, bool REVERSE>
__device__ int block_excl_scan(int v, int* wsum, int identity, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = REVERSE ? __shfl_down(x, d) : __shfl_up(x, d);
    bool take = REVERSE ? (lane + d < 64) : (lane >= d);
    if (take) x = MAXOP ? op_max(x, y) : op_min(x, y);
  }
  int excl = REVERSE ? __shfl_down(x, 1) : __shfl_up(x, 1);
  if (REVERSE ? (lane == 63) : (lane == 0)) excl = identity;
  if (REVERSE ? (lane == 0) : (lane == 63)) wsum[wave] = x;
  __syncthreads();
  int pre = identity, tot = identity;
#pragma unroll
  for (int w = 0; w < kSegWaves; ++w) {
    int s = wsum[w];
    tot = MAXOP ? op_max(tot, s) : op_min(tot, s);
    if (REVERSE ? (w > wave) : (w < wave)) pre = MAXOP ? op_max(pre, s) : op_min(pre, s);
  }
  __syncthreads();
  *total = tot;
  return MAXOP ? op_max(pre, excl) : op_min(pre, excl);
}

__global__ __launch_bounds__(kSegThreads) void seg_meta_kernel(SegMetaArgs a) {
  const int b = blockIdx.x;
  const int side = blockIdx.y;
  const int S = side ? a.Skv : a.Sq;
  const size_t row = (size_t)b * S;
  const int* ids = a.ids[side] + row;
  const int* pos_in = a.pos_in[side] ? a.pos_in[side] + row : nullptr;
  int* pos_out = a.pos_out[side] ? a.pos_out[side] + row : nullptr;
  int2* run = a.run[side] + row;
  ChunkSum* sum = a.sum[side] + (size_t)b * a.nch[side];
  const int nch = a.nch[side];
  const bool eq_check = side == 0 && a.check_eq;
  const int* ids_kv = eq_check ? a.ids[1] + row : nullptr;
  const int* pos_kv = (eq_check && a.pos_in[1]) ? a.pos_in[1] + row : nullptr;

  __shared__ int wsum[4][kSegWaves];
  const int t = threadIdx.x;
  const int lane = t & 63;
  int ok = 1;
  int carry_start = -1;
  int carry_nz = INT32_MIN;
  // Phase 1's last round is the round phase 2 starts with: its ids, next
  // id, positions and run starts stay in registers.
  int rs_last[kSegItems], id_last[kSegItems], pin_last[kSegItems], next_last = 0;
  const bool vec_ids = al16(ids), vec_run = al16(run);
  const bool vec_pin = pos_in && al16(pos_in), vec_pout = pos_out && al16(pos_out);
  const bool vec_ikv = ids_kv && al16(ids_kv), vec_pkv = pos_kv && al16(pos_kv);
  const int nrounds = (S + kSegRound - 1) / kSegRound;

  // Phase 1, left to right: run starts, derived positions, fast-route checks.
  for (int rd = 0; rd < nrounds; ++rd) {
    const int base = rd * kSegRound + t * kSegItems;
    int id[kSegItems];
    int st[kSegItems];
    // Every load of the round is issued here, before the scans' barriers
    // (which loads cannot move across), and waited for once.
    const int prev_v = ids[clamp_tok(base - 1, S)];
    const int next_v = ids[clamp_tok(base + kSegItems, S)];
    int prev = (base > 0 && base - 1 < S) ? prev_v : 0;
    load8(ids, base, S, vec_ids, id);
    int pin[kSegItems], ikv[kSegItems], pkv[kSegItems];
    if (pos_in) load8(pos_in, base, S, vec_pin, pin);
    if (eq_check) load8(ids_kv, base, S, vec_ikv, ikv);
    if (pos_kv) load8(pos_kv, base, S, vec_pkv, pkv);
    int st_local = -1;
    int nz_local = INT32_MIN;
#pragma unroll
    for (int k = 0; k < kSegItems; ++k) {
      const int i = base + k;
      const bool in = i < S;
      if (!in) id[k] = 0;
      const int pid = k == 0 ? prev : id[k - 1];
      if (in && (i == 0 || id[k] != pid)) st_local = i;
      st[k] = st_local;
      if (in && id[k] != 0) nz_local = op_max(nz_local, id[k]);
    }
    int tot;
    const int pre_start = op_max(carry_start, block_excl_scan<true, false>(st_local, wsum[0], -1, &tot));
    carry_start = op_max(carry_start, tot);
    const int pre_nz = op_max(carry_nz, block_excl_scan<true, false>(nz_local, wsum[1], INT32_MIN, &tot));
    carry_nz = op_max(carry_nz, tot);
    bool seen_nz = pre_nz != INT32_MIN;
    int running_nz = pre_nz;
    int rsv[kSegItems];
#pragma unroll
    for (int k = 0; k < kSegItems; ++k) {
      const int i = base + k;
      rsv[k] = st[k] >= 0 ? st[k] : pre_start;
      if (i < S) {
        const int rs = rsv[k];
        const int dpos = i - rs;
        if (id[k] != 0) {
          if (id[k] == INT32_MIN) ok = 0;
          if (rs == i && seen_nz && id[k] <= running_nz) ok = 0;
          running_nz = seen_nz ? op_max(running_nz, id[k]) : id[k];
          seen_nz = true;
        }
        const int p = pos_in ? pin[k] : dpos;
        if (pos_in && id[k] != 0 && p != dpos) ok = 0;
        if (eq_check) {
          const int pk = pos_kv ? pkv[k] : dpos;
          if (ikv[k] != id[k] || pk != p) ok = 0;
        }
      }
    }
    // The round's stores last, back to back (a store waited for before the
    // next token's work would cost a round trip per token again).
    int dpv[kSegItems], zero[kSegItems];
#pragma unroll
    for (int k = 0; k < kSegItems; ++k) {
      rs_last[k] = rsv[k];
      id_last[k] = id[k];
      pin_last[k] = pos_in ? pin[k] : 0;
      dpv[k] = base + k - rsv[k];
      zero[k] = 0;
    }
    next_last = base + kSegItems < S ? next_v : 0;
    if (pos_out) store8(pos_out, base, S, vec_pout, dpv);
    store8_run(run, base, S, vec_run, rsv, zero);
  }

  // Phase 2, right to left: run ends, final run bounds, 32-token summaries.
  int carry_end = INT32_MAX;
  for (int rd = nrounds - 1; rd >= 0; --rd) {
    const int base = rd * kSegRound + t * kSegItems;
    int id[kSegItems], en[kSegItems], rsv[kSegItems], pin[kSegItems];
    int next;
    if (rd == nrounds - 1) {
#pragma unroll
      for (int k = 0; k < kSegItems; ++k) {
        id[k] = id_last[k];
        rsv[k] = rs_last[k];
        pin[k] = pin_last[k];
      }
      next = next_last;
    } else {   // a whole round: ids, positions and run starts (this thread's own phase-1 stores)
      load8(ids, base, S, vec_ids, id);
      const int next_v = ids[clamp_tok(base + kSegItems, S)];
#pragma unroll
      for (int k = 0; k < kSegItems; ++k) rsv[k] = run[clamp_tok(base + k, S)].x;
      if (pos_in) load8(pos_in, base, S, vec_pin, pin);
#pragma unroll
      for (int k = 0; k < kSegItems; ++k)
        if (base + k >= S) id[k] = 0;
      next = base + kSegItems < S ? next_v : 0;
    }
    int en_local = INT32_MAX;
#pragma unroll
    for (int k = kSegItems - 1; k >= 0; --k) {
      const int i = base + k;
      if (i < S) {
        const int nid = k == kSegItems - 1 ? next : id[k + 1];
        if (i == S - 1 || id[k] != nid) en_local = i + 1;
      }
      en[k] = en_local;
    }
    int tot;
    const int pre_end = op_min(carry_end, block_excl_scan<false, true>(en_local, wsum[2], INT32_MAX, &tot));
    carry_end = op_min(carry_end, tot);

    int cnt = 0, idmin = INT32_MAX, idmax = INT32_MIN, pmin = INT32_MAX, pmax = INT32_MIN;
    int smin = INT32_MAX, smax = INT32_MIN, emin = INT32_MAX, emax = INT32_MIN;
    int rev[kSegItems];
#pragma unroll
    for (int k = 0; k < kSegItems; ++k) {
      const int i = base + k;
      rev[k] = en[k] != INT32_MAX ? en[k] : pre_end;
      if (i < S && id[k] != 0) {
        const int rs = rsv[k];
        const int re = rev[k];
        const int p = pos_in ? pin[k] : i - rs;
        ++cnt;
        idmin = op_min(idmin, id[k]); idmax = op_max(idmax, id[k]);
        pmin = op_min(pmin, p); pmax = op_max(pmax, p);
        smin = op_min(smin, rs); smax = op_max(smax, rs);
        emin = op_min(emin, re); emax = op_max(emax, re);
      }
    }
    int rso[kSegItems], reo[kSegItems];
#pragma unroll
    for (int k = 0; k < kSegItems; ++k) {
      rso[k] = id[k] != 0 ? rsv[k] : 0;
      reo[k] = id[k] != 0 ? rev[k] : 0;
    }
    store8_run(run, base, S, vec_run, rso, reo);
    // 4 consecutive threads cover one 32-token chunk.
#pragma unroll
    for (int d = 1; d < 4; d <<= 1) {
      cnt += __shfl_xor(cnt, d);
      idmin = op_min(idmin, __shfl_xor(idmin, d)); idmax = op_max(idmax, __shfl_xor(idmax, d));
      pmin = op_min(pmin, __shfl_xor(pmin, d)); pmax = op_max(pmax, __shfl_xor(pmax, d));
      smin = op_min(smin, __shfl_xor(smin, d)); smax = op_max(smax, __shfl_xor(smax, d));
      emin = op_min(emin, __shfl_xor(emin, d)); emax = op_max(emax, __shfl_xor(emax, d));
    }
    const int chunk = (rd * kSegRound + t * kSegItems) / kChunk;
    if ((lane & 3) == 0 && chunk < nch) {
      ChunkSum c;
      c.cnt = cnt; c.idmin = idmin; c.idmax = idmax; c.posmin = pmin;
      c.posmax = pmax; c.smin = smin; c.smax = smax; c.emin = emin;
      c.emax = emax; c.pad0 = 0; c.pad1 = 0; c.pad2 = 0;
      sum[chunk] = c;
    }
  }

  const int all_ok = __syncthreads_and(ok);
  if (side == 0 && t == 0) {
    const bool fast_candidate = !a.force_general && (a.sides == 1 || a.check_eq);
    a.route[b] = (fast_candidate && all_ok) ? kRouteFast : kRouteGeneral;
  }
}

__global__ __launch_bounds__(256) void debug_mask_kernel(MaskArgs a) {
  const size_t total = (size_t)a.B * a.Sq * a.Skv;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < total; x += (size_t)gridDim.x * blockDim.x) {
    const int j = (int)(x % a.Skv);
    const int i = (int)((x / a.Skv) % a.Sq);
    const int b = (int)(x / ((size_t)a.Skv * a.Sq));
    const int route = a.has_meta ? a.seg.route[b] : kRouteDense;
    TokMeta qi = q_meta(route, a.seg, b, a.Sq, i);
    TokMeta kj = route == kRouteGeneral ? kv_meta(route, a.seg, b, a.Skv, j) : TokMeta{0, 0};
    a.mask[x] = allowed(route, a.causal != 0, a.Skv, i, j, qi, kj) ? 1 : 0;
  }
  if (a.route_rows && blockIdx.x == 0) {
    for (int b = threadIdx.x; b < a.B; b += blockDim.x)
      a.route_rows[b] = a.has_meta ? a.seg.route[b] : kRouteDense;
  }
}

// Longest-walk-first tile orders for rows on the general route.  There
// the walk of a tile (the key tiles a query tile visits, or the query tiles
// a key tile is visited by) depends on where the segments fall, not on the
// tile's position, and the fixed order can leave long walks for last.  One
// workgroup per (batch row, side) counts the visited units of every tile of
// 128 (key or query units of 64, classified from the 32-token summaries as
// the attention kernels classify them) and ranks the tiles by that count,
// longest first, ties by index.  Rows on the fast route keep the fixed
// order (measured faster there: their walks follow the segment layout
// closely and neighbouring tiles share K/V or Q/dO in L2).  The order only
// changes which workgroup runs when; each tile's arithmetic is the same.
constexpr int kOrdThreads = 1024;
constexpr int kOrdTiles = 1024;   // tiles of 128 per row and side
constexpr int kOrdUnits = 2048;   // walk units of 64 per row and side

__global__ __launch_bounds__(kOrdThreads) void tile_order_kernel(TileOrderArgs t) {
  __shared__ TileSum tsum[kOrdTiles];
  __shared__ TileSum usum[kOrdUnits];
  __shared__ int lo_u[kOrdTiles], hi_u[kOrdTiles], len[kOrdTiles];
  const int b = blockIdx.x;
  const bool qside = blockIdx.y == 0;   // query tiles over key units, else key tiles over query units
  const int tid = threadIdx.x;
  const bool causal = t.causal != 0;
  const int route = t.seg.route[b];
  const int n_t = ((qside ? t.Sq : t.Skv) + 127) / 128;
  const int n_u = ((qside ? t.Skv : t.Sq) + 63) / 64;
  int* ord = (qside ? t.qord : t.kord) + (size_t)b * n_t;
  if (route != kRouteGeneral || n_t > kOrdTiles || n_u > kOrdUnits) {   // the fixed order
    for (int r = tid; r < n_t; r += kOrdThreads) ord[r] = (qside && causal) ? n_t - 1 - r : r;
    return;
  }
  const int nch_t = qside ? t.seg.nch_q : t.seg.nch_kv;
  const int nch_u = qside ? t.seg.nch_kv : t.seg.nch_q;
  const ChunkSum* row_t = (qside ? t.seg.sum_q : t.seg.sum_kv) + (size_t)b * nch_t;
  const ChunkSum* row_u = (qside ? t.seg.sum_kv : t.seg.sum_q) + (size_t)b * nch_u;
  for (int i = tid; i < n_t; i += kOrdThreads) {
    const TileSum ts = tile_sum(row_t, nch_t, i * 128, 128);
    int lo, hi;
    if (qside) kv_range(route, causal, t.Skv, i * 128, 128, ts, lo, hi);
    else q_range(route, causal, t.Sq, i * 128, 128, ts, lo, hi);
    tsum[i] = ts;
    lo_u[i] = lo / 64;
    hi_u[i] = (hi + 63) / 64;
    len[i] = 0;
  }
  for (int j = tid; j < n_u; j += kOrdThreads) usum[j] = tile_sum(row_u, nch_u, j * 64, 64);
  __syncthreads();
  // Every (tile, unit) pair in the tile's range, spread over all threads.
  for (int p = tid; p < n_t * n_u; p += kOrdThreads) {
    const int i = p / n_u, j = p - i * n_u;
    if (j < lo_u[i] || j >= hi_u[i]) continue;
    const int c = qside ? classify_tile(route, causal, t.Skv, i * 128, 128, j * 64, 64, tsum[i], usum[j])
                        : classify_tile(route, causal, t.Skv, j * 64, 64, i * 128, 128, usum[j], tsum[i]);
    if (c != kTileSkip) atomicAdd(&len[i], 1);
  }
  __syncthreads();
  for (int i = tid; i < n_t; i += kOrdThreads) {
    const int li = len[i];
    int r = 0;
    for (int u = 0; u < n_t; ++u) r += (len[u] > li) | ((len[u] == li) & (u < i));
    ord[r] = i;
  }
}

// The route each batch row took (route NULL: no metadata, every row dense).
__global__ __launch_bounds__(256) void route_rows_kernel(const int* route, int B, int* out) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x)
    out[b] = route ? route[b] : kRouteDense;
}

}  // namespace

hipError_t launch_route_rows(const int* route, int B, int* out, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  const int blocks = (B + 255) / 256 < 1024 ? (B + 255) / 256 : 1024;
  hipLaunchKernelGGL(route_rows_kernel, dim3(blocks), dim3(256), 0, st, route, B, out);
  return hipGetLastError();
}

hipError_t launch_seg_meta(const SegMetaArgs& a, hipStream_t st) {
  dim3 grid(a.B, a.sides);
  hipLaunchKernelGGL(seg_meta_kernel, grid, dim3(kSegThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tile_order(const TileOrderArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(tile_order_kernel, dim3(a.B, 2), dim3(kOrdThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_debug_mask(const MaskArgs& a, hipStream_t st) {
  const size_t total = (size_t)a.B * a.Sq * a.Skv;
  size_t blocks = (total + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(debug_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace bps
