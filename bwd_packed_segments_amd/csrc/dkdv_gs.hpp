// dK/dV with the work split by gradient (bf16, head dims 64 or 128).
//
// A workgroup owns 128 keys of one (batch row, key/value head) and walks, in
// one sequential loop, the query heads of its GQA group and the 32-query
// phases that may attend its keys (descending query tiles, heads inner, as
// the other dK/dV kernel).  Eight waves, two per SIMD, in pairs that own the
// same 32 keys:
//   * the P wave (waves 0-3) holds K, computes S = Q K^T and
//     P = exp2(S scale log2 e - LSE2), applies the mask, passes P to its
//     partner through LDS and accumulates dV^T += dO^T P one phase later;
//   * the dS wave (waves 4-7) holds V, computes dP = dO V^T and, one phase
//     later, dS = P (dP - Delta) with its partner's P, and accumulates
//     dK^T += Q^T dS.
// In every interval between two barriers each wave of a pair runs 16 MFMAs
// (P wave: dV of the previous phase, S of this one; dS wave: dK of the
// previous phase, dP of this one) and its own share of the softmax-gradient
// arithmetic, so the exponentials of one wave run beside the products of
// the other on the same SIMD.
//
// Q, dO, LSE2 and Delta of a phase are fetched straight into one of NB phase
// buffers in LDS, LA = NB - 2 intervals ahead, with buffer loads whose
// per-lane offsets are fixed for the whole walk (the phase moves only the
// scalar offset).  The interval loop is unrolled NB times, so that every LDS
// address is a per-lane offset computed once plus an immediate.  Every
// dK/dV element is a sum in a fixed order inside one workgroup, written once
// at the end: nothing depends on the order in which workgroups run
// (maxdiffusion PR 485, Code Review of the dkv kernel).
#pragma once

#include <type_traits>

#include "bps_args.hpp"
#include "lds_tile.hpp"

namespace bps {

template <int DQK, int DV>
struct DkvGsCfg {
  static constexpr int BN = 128;   // keys per workgroup: 4 key blocks of 32
  static constexpr int BQ = 32;    // queries per phase
  static constexpr int NB = 4;     // phase buffers
  static constexpr int LA = NB - 2;   // phases fetched ahead of the one in use
  static constexpr int Q_BYTES = BQ * DQK * 2;
  static constexpr int DO_BYTES = BQ * DV * 2;
  static constexpr int TILE_BYTES = Q_BYTES + DO_BYTES;   // Q and dO tiles of one phase buffer
  static constexpr int XKB_BYTES = 4 * 64 * 16;            // P of one key block: 4 float4 per lane
  static constexpr int XSLOT_BYTES = 4 * XKB_BYTES;
  static constexpr int SIDE_BYTES = BQ * 4 * 4;            // LSE2, Delta, metadata (a, b)
  static constexpr int XCH_OFF = NB * TILE_BYTES;
  static constexpr int SIDE_OFF = XCH_OFF + 2 * XSLOT_BYTES;
  static constexpr int CLS_OFF = SIDE_OFF + NB * SIDE_BYTES;
  static constexpr int LDS_BYTES = CLS_OFF + kClassCap;
  static constexpr int QW = BQ * DQK / 8 / 64;   // waves that fetch the Q tile (one 16-byte chunk per lane)
  static constexpr int DW = BQ * DV / 8 / 64;    // waves that fetch the dO tile (the last DW waves)
  static constexpr bool ENABLED = (DQK == 64 || DQK == 128) && (DV == 64 || DV == 128) && LDS_BYTES <= 160 * 1024;
};

// Byte offset of this lane's natural operand fragment t (row n, elements
// 16 t + 8 hf) in a [32 x D] bf16 tile.
template <int D>
__device__ inline uint32_t gs_row_off(int n, int hf, int t) {
  return (uint32_t)TileFmt<bf16, D>::off(n, 16 * t + 8 * hf) * 2;
}
// Byte offset of this lane's transposed read p (0: rows y, 1: rows y + 8) of
// column block d in a [32 x D] tile, rows 0..15 (frag_tr with x0 = 32 d,
// y0 = 0; y0 = 16 adds 16 D elements).
template <int D>
__device__ inline uint32_t gs_tr_off(int lane, int d, int p) {
  const int G = lane >> 4, i = lane & 15, hf = G >> 1;
  const int x = 32 * d + 16 * (G & 1) + 4 * (i & 3);
  const int y = 4 * hf + (i >> 2) + 8 * p;
  return (uint32_t)TileFmt<bf16, D>::off(y, x) * 2;
}

template <int DQK, int DV>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
    attn_bwd_dkdv_gs_kernel(BwdArgs a) {
  using C = DkvGsCfg<DQK, DV>;
  using T = bf16;
  using E = Elem<T>;
  using F8 = bf16x8;
  constexpr int BN = C::BN, BQ = C::BQ, NB = C::NB, LA = C::LA;
  static_assert(NB % 2 == 0, "exchange slots follow the buffer index");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  unsigned char* const cls_tab = reinterpret_cast<unsigned char*>(smem + C::CLS_OFF);

  const AttnShape& s = a.s;
  const bool causal = s.causal != 0;
  const int n_kt = (s.Skv + BN - 1) / BN;
  const int g = s.Hq / s.Hkv;
  const int nblocks = s.B * s.Hkv * n_kt;
  int L = logical_block(nblocks, s.reverse);
  const int rank = L % n_kt;
  L /= n_kt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  const int k0 = k_tile_of(a.seg, b, rank, n_kt) * BN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool pwave = wave < 4;
  const int kb = wave & 3;
  const int kj = k0 + kb * 32 + n;

  const int route = s.has_meta ? a.seg.route[b] : kRouteDense;
  TileSum ks{};
  const ChunkSum* sum_q_row = nullptr;
  if (route != kRouteDense) {
    ks = tile_sum(a.seg.sum_kv + (size_t)b * a.seg.nch_kv, a.seg.nch_kv, k0, BN);
    sum_q_row = a.seg.sum_q + (size_t)b * a.seg.nch_q;
  }
  int lo, hi;
  q_range(route, causal, s.Sq, k0, BN, ks, lo, hi);
  const int t_hi = (hi + BQ - 1) / BQ;
  const int ntiles = t_hi - lo / BQ;
  auto classify = [&](int u) -> int {
    const int q0 = (t_hi - 1 - u) * BQ;
    TileSum qs{};
    if (route != kRouteDense) qs = tile_sum(sum_q_row, a.seg.nch_q, q0, BQ);
    return classify_tile(route, causal, s.Skv, q0, BQ, k0, BN, qs, ks);
  };
  const bool tabled = route != kRouteDense;
  if (tabled) {
    fill_classes(cls_tab, ntiles, tid, 512, classify);
    __syncthreads();
  }
  auto tile_class = [&](int u) -> int { return (tabled && u < kClassCap) ? (int)cls_tab[u] : classify(u); };

  // Walk position: tile ordinal u (query tile t_hi - 1 - u), head hh of the
  // group, the tile's class.  u >= ntiles: past the end.
  struct Ph {
    int u, hh, cls;
  };
  auto seek = [&](int u) -> Ph {
    for (; u < ntiles; ++u) {
      const int c = tile_class(u);
      if (c != kTileSkip) return Ph{u, 0, c};
    }
    return Ph{ntiles, 0, kTileSkip};
  };
  auto advance = [&](const Ph& p) -> Ph {
    if (p.u >= ntiles) return p;
    if (p.hh + 1 < g) return Ph{p.u, p.hh + 1, p.cls};
    return seek(p.u + 1);
  };

  // ---------------------------------------------------------------- loads
  // This lane's 16-byte chunk of the Q and dO tiles: physical slot sl holds
  // logical chunk swz(r, sl % NC) of row r (see TileLoad).  Byte offsets of
  // a batch row's Q / dO fit in 32 bits (checked by the host).
  using FQ = TileFmt<T, DQK>;
  using FD = TileFmt<T, DV>;
  const bool q_loader = wave < C::QW;
  const bool d_loader = wave >= 8 - C::DW;
  const int q_sl = tid;
  const int d_sl = tid - (8 - C::DW) * 64;
  const int q_r = q_sl / FQ::NC, q_c = FQ::swz(q_r, q_sl % FQ::NC);
  const int d_r = d_sl / FD::NC, d_c = FD::swz(d_r, d_sl % FD::NC);
  const uint32_t q_ts = (uint32_t)a.sq.t * 2, q_hs = (uint32_t)a.sq.h * 2;   // bytes per token / head
  const uint32_t d_ts = (uint32_t)a.so.t * 2, d_hs = (uint32_t)a.so.h * 2;
  const uint32_t q_voff = (uint32_t)q_r * q_ts + (uint32_t)q_c * 16;
  const uint32_t d_voff = (uint32_t)d_r * d_ts + (uint32_t)d_c * 16;
  const T* const qb_ptr = static_cast<const T*>(a.q) + b * a.sq.b;
  const T* const db_ptr = static_cast<const T*>(a.dout) + b * a.so.b;
  const __amdgpu_buffer_rsrc_t q_rsrc = raw_rsrc(qb_ptr);
  const __amdgpu_buffer_rsrc_t d_rsrc = raw_rsrc(db_ptr);
  // LDS byte addresses (M0 values) of this wave's chunks in buffer 0.
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(BPS_LDS char*)smem);
  const uint32_t q_m0 = lds0 + (uint32_t)((q_sl & ~63) * 16);
  const uint32_t d_m0 = lds0 + C::Q_BYTES + (uint32_t)((d_sl & ~63) * 16);
  const uint32_t side_m0 = lds0 + C::SIDE_OFF;
  // Side rows: lanes 0-31 LSE2, 32-63 Delta of the phase's 32 queries
  // (wave 0); lanes 0-31 metadata a, 32-63 metadata b (wave 1).
  const size_t hrow0 = ((size_t)b * s.Hq + (size_t)hkv * g) * s.Sq;   // row of (b, first head of the group, query 0)
  const float* const side_src = (hf ? a.delta : a.lse2) + hrow0 + n;
  const int* meta_src = nullptr;
  if (route == kRouteFast) meta_src = reinterpret_cast<const int*>(a.seg.run_q + (size_t)b * s.Sq + n) + hf;
  else if (route == kRouteGeneral) meta_src = (hf ? a.seg.pos_q : a.seg.ids_q) + (size_t)b * s.Sq + n;
  const int meta_step = route == kRouteFast ? 2 : 1;   // ints per token

  // Fetches phase p into buffer BI; returns the vector memory operations
  // this wave left in flight.
  auto issue = [&](const Ph& p, auto bic) -> int {
    constexpr int BI = decltype(bic)::value;
    const int q0 = (t_hi - 1 - p.u) * BQ;
    const int hh = p.hh;
    const size_t rowx = (size_t)hh * s.Sq + q0;
    char* const tile = smem + BI * C::TILE_BYTES;
    float* const side = reinterpret_cast<float*>(smem + C::SIDE_OFF + BI * C::SIDE_BYTES);
    if (q0 + BQ <= s.Sq) {
      int nfl = 0;
      if (q_loader) {
        lds_load16(q_rsrc, q_m0 + BI * C::TILE_BYTES, q_voff, (uint32_t)(hkv * g + hh) * q_hs + (uint32_t)q0 * q_ts);
        ++nfl;
      }
      if (d_loader) {
        lds_load16(d_rsrc, d_m0 + BI * C::TILE_BYTES, d_voff, (uint32_t)(hkv * g + hh) * d_hs + (uint32_t)q0 * d_ts);
        ++nfl;
      }
      if (wave == 0) {
        lds_load4(side_src + rowx, side_m0 + BI * C::SIDE_BYTES);
        ++nfl;
      } else if (wave == 1 && route != kRouteDense) {
        lds_load4(meta_src + (size_t)q0 * meta_step, side_m0 + BI * C::SIDE_BYTES + 2 * BQ * 4);
        ++nfl;
      }
      return nfl;
    }
    // The last, partial phase: through registers, zeros (LSE2 = +inf, so
    // P = 0) for rows past Sq.
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int h = hkv * g + hh;
    if (q_loader) {
      u32x4v v = u32x4v{0u, 0u, 0u, 0u};
      if (q0 + q_r < s.Sq)
        v = *reinterpret_cast<const u32x4v*>(qb_ptr + h * a.sq.h + (int64_t)(q0 + q_r) * a.sq.t + q_c * 8);
      *reinterpret_cast<u32x4v*>(tile + q_sl * 16) = v;
    }
    if (d_loader) {
      u32x4v v = u32x4v{0u, 0u, 0u, 0u};
      if (q0 + d_r < s.Sq)
        v = *reinterpret_cast<const u32x4v*>(db_ptr + h * a.so.h + (int64_t)(q0 + d_r) * a.so.t + d_c * 8);
      *reinterpret_cast<u32x4v*>(tile + C::Q_BYTES + d_sl * 16) = v;
    }
    const bool in = q0 + n < s.Sq;
    if (wave == 0) {
      side[lane] = in ? side_src[rowx] : (hf ? 0.f : INFINITY);
    } else if (wave == 1 && route != kRouteDense) {
      const TokMeta t = in ? q_meta(route, a.seg, b, s.Sq, q0 + n) : TokMeta{0, 0};
      reinterpret_cast<int*>(side)[2 * BQ + lane] = hf ? t.b : t.a;
    }
    return 0;
  };

  // ---------------------------------------------------------------- state
  const float c2 = s.scale_log2;
  constexpr int NKV = DQK > DV ? DQK / 16 : DV / 16;
  constexpr int NACC = DQK > DV ? DQK / 32 : DV / 32;
  constexpr int NACC_P = DV / 32, NACC_D = DQK / 32;
  F8 kvf[NKV];        // P wave: K fragments; dS wave: V fragments
  f32x16 acc[NACC];   // P wave: dV^T; dS wave: dK^T
#pragma unroll
  for (int d = 0; d < NACC; ++d) acc[d] = f32x16{};
  TokMeta km{0, 0};
  {
    const T* kp = static_cast<const T*>(a.k) + b * a.sk.b + hkv * a.sk.h;
    const T* vp = static_cast<const T*>(a.v) + b * a.sv.b + hkv * a.sv.h;
    if (pwave) {
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t)
        kvf[t] = kj < s.Skv ? E::load8(kp + kj * a.sk.t + 16 * t + 8 * hf) : E::zero8();
      if (route == kRouteGeneral) km = kv_meta(route, a.seg, b, s.Skv, kj);
    } else {
#pragma unroll
      for (int t = 0; t < DV / 16; ++t)
        kvf[t] = kj < s.Skv ? E::load8(vp + kj * a.sv.t + 16 * t + 8 * hf) : E::zero8();
    }
  }
  F8 pbf[2];               // P wave: P of the previous phase (bf16, B operand of dV)
  f32x16 dpa = f32x16{};   // dS wave: dP of the previous phase
  pbf[0] = E::zero8();
  pbf[1] = E::zero8();

  // Per-lane LDS byte offsets, fixed for the walk.  P wave: rows of the Q
  // tile (S) and transposed reads of the dO tile (dV); dS wave: rows of the
  // dO tile (dP) and transposed reads of the Q tile (dK).
  constexpr int DR = DQK > DV ? DQK : DV;
  uint32_t roff[DR / 16];
  uint32_t troff[DR / 32][2];
  if (pwave) {
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t) roff[t] = gs_row_off<DQK>(n, hf, t);
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int p = 0; p < 2; ++p) troff[d][p] = C::Q_BYTES + gs_tr_off<DV>(lane, d, p);
  } else {
#pragma unroll
    for (int t = 0; t < DV / 16; ++t) roff[t] = C::Q_BYTES + gs_row_off<DV>(n, hf, t);
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
      for (int p = 0; p < 2; ++p) troff[d][p] = gs_tr_off<DQK>(lane, d, p);
  }
  char* const xlane = smem + C::XCH_OFF + kb * C::XKB_BYTES + lane * 16;   // + slot, + 1 KB per float4
  const char* const slane = smem + C::SIDE_OFF + 16 * hf;                     // + buffer, + 32 B per group

  auto rd_row = [&](int BI, int t) -> F8 {
    return *reinterpret_cast<const F8*>(smem + BI * C::TILE_BYTES + roff[t]);
  };
  // Transposed fragment (column block d, query rows 16 s2 ..) of buffer BI's
  // tile at D elements per row.
  auto rd_tr = [&](int BI, int D, int d, int s2) -> F8 {
    const char* base = smem + BI * C::TILE_BYTES + 16 * s2 * D * 2;
    const bf16x4v x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)(base + troff[d][0]));
    const bf16x4v y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)(base + troff[d][1]));
    return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  };

  // P wave, this interval's phase in buffer BI: S, P, mask, P to exchange
  // slot BI & 1.
  auto p_front = [&](const Ph& p, auto bic) {
    constexpr int BI = decltype(bic)::value;
    F8 qa[DQK / 16];
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t) qa[t] = rd_row(BI, t);
    f32x16 sa = f32x16{};
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t) sa = mma(qa[t], kvf[t], sa);
    const char* sl = slane + BI * C::SIDE_BYTES;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + 32 * grp);
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[4 * grp + i] = fast_exp2(fmaf(sa[4 * grp + i], c2, -l4[i]));
    }
    if (p.cls == kTilePart) {
      const int q0 = (t_hi - 1 - p.u) * BQ;
      const int* qm = reinterpret_cast<const int*>(smem + C::SIDE_OFF + BI * C::SIDE_BYTES) + 2 * BQ;
      mask_tile<false>(sa, 0.f, route, causal, s.Skv, kj, km, q0, hf, qm, qm + BQ, 0);
    }
    char* x = xlane + (BI & 1) * C::XSLOT_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4*>(x + j * 1024) = f32x4{sa[4 * j], sa[4 * j + 1], sa[4 * j + 2], sa[4 * j + 3]};
    pbf[0] = E::cvt8(slots8(sa, 0));
    pbf[1] = E::cvt8(slots8(sa, 1));
  };
  // P wave, the previous interval's phase in buffer BI: dV^T += dO^T P.
  auto p_back = [&](auto bic) {
    constexpr int BI = decltype(bic)::value;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d = 0; d < NACC_P; ++d) acc[d] = mma(rd_tr(BI, DV, d, s2), pbf[s2], acc[d]);
  };
  // dS wave, the previous interval's phase in buffer BI (P in exchange slot
  // BI & 1): dS = P (dP - Delta), dK^T += Q^T dS.
  auto d_back = [&](auto bic) {
    constexpr int BI = decltype(bic)::value;
    const char* x = xlane + (BI & 1) * C::XSLOT_BYTES;
    const char* sl = slane + BI * C::SIDE_BYTES + BQ * 4;   // Delta
    f32x16 ds;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 p4 = *reinterpret_cast<const f32x4*>(x + j * 1024);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(sl + 32 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) ds[4 * j + i] = p4[i] * (dpa[4 * j + i] - d4[i]);
    }
    const F8 dsf0 = E::cvt8(slots8(ds, 0));
    const F8 dsf1 = E::cvt8(slots8(ds, 1));
#pragma unroll
    for (int d = 0; d < NACC_D; ++d) acc[d] = mma(rd_tr(BI, DQK, d, 0), dsf0, acc[d]);
#pragma unroll
    for (int d = 0; d < NACC_D; ++d) acc[d] = mma(rd_tr(BI, DQK, d, 1), dsf1, acc[d]);
  };
  // dS wave, this interval's phase in buffer BI: dP = dO V^T.
  auto d_front = [&](auto bic) {
    constexpr int BI = decltype(bic)::value;
    F8 da[DV / 16];
#pragma unroll
    for (int t = 0; t < DV / 16; ++t) da[t] = rd_row(BI, t);
    dpa = f32x16{};
#pragma unroll
    for (int t = 0; t < DV / 16; ++t) dpa = mma(da[t], kvf[t], dpa);
  };

  // ---------------------------------------------------------------- walk
  // Interval i (between barriers i - 1 and i) works on phase i (front, in
  // buffer i % NB) and phase i - 1 (back) and fetches phase i + LA into the
  // buffer phase i - 2 used, which barrier i - 1 freed.  At its end each wave
  // waits for the loads of the interval before (needed in interval i + 1)
  // and keeps its own in flight.
  Ph prev{ntiles, 0, kTileSkip};
  Ph cur = seek(0);
  Ph ahead[LA];
  ahead[0] = advance(cur);
#pragma unroll
  for (int j = 1; j < LA; ++j) ahead[j] = advance(ahead[j - 1]);
  if (cur.u < ntiles) issue(cur, std::integral_constant<int, 0>{});
  if (LA >= 2 && ahead[0].u < ntiles) issue(ahead[0], std::integral_constant<int, 1>{});
  static_assert(LA == 2, "prologue fetches phases 0 and 1");
  wait_vm();
  __syncthreads();

  auto step = [&](auto bic) -> bool {
    constexpr int BI = decltype(bic)::value;
    constexpr int BP = (BI + NB - 1) % NB;   // buffer of the previous phase
    if (cur.u >= ntiles && prev.u >= ntiles) return false;
    int nfl = 0;
    if (ahead[LA - 1].u < ntiles) nfl = issue(ahead[LA - 1], std::integral_constant<int, (BI + LA) % NB>{});
    if (pwave) {
      if (prev.u < ntiles) p_back(std::integral_constant<int, BP>{});
      if (cur.u < ntiles) p_front(cur, std::integral_constant<int, BI>{});
    } else {
      if (prev.u < ntiles) d_back(std::integral_constant<int, BP>{});
      if (cur.u < ntiles) d_front(std::integral_constant<int, BI>{});
    }
    // LDS stores (exchange, partial-phase tiles) done; loads of the previous
    // interval landed, this interval's left in flight.
    if (nfl == 3) wait_vm_keep<3>();
    else if (nfl == 2) wait_vm_keep<2>();
    else if (nfl == 1) wait_vm_keep<1>();
    else wait_vm_keep<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    prev = cur;
    cur = ahead[0];
#pragma unroll
    for (int j = 0; j + 1 < LA; ++j) ahead[j] = ahead[j + 1];
    ahead[LA - 1] = advance(ahead[LA - 1]);
    return true;
  };
  static_assert(NB == 4, "the loop below is unrolled four times");
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{}) &&
         step(std::integral_constant<int, 2>{}) && step(std::integral_constant<int, 3>{})) {
  }
  wait_vm();

  if (kj < s.Skv) {
    if (pwave) {
      T* dvp = static_cast<T*>(a.dv) + b * a.sv.b + kj * a.sv.t + hkv * a.sv.h;
#pragma unroll
      for (int d = 0; d < NACC_P; ++d)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const f32x4 v = f32x4{acc[d][4 * grp], acc[d][4 * grp + 1], acc[d][4 * grp + 2], acc[d][4 * grp + 3]};
          *reinterpret_cast<typename E::P4*>(dvp + d * 32 + 8 * grp + 4 * hf) = E::cvt4(v);
        }
    } else {
      T* dkp = static_cast<T*>(a.dk) + b * a.sk.b + kj * a.sk.t + hkv * a.sk.h;
#pragma unroll
      for (int d = 0; d < NACC_D; ++d)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const f32x4 v =
              f32x4{acc[d][4 * grp], acc[d][4 * grp + 1], acc[d][4 * grp + 2], acc[d][4 * grp + 3]} * s.scale;
          *reinterpret_cast<typename E::P4*>(dkp + d * 32 + 8 * grp + 4 * hf) = E::cvt4(v);
        }
    }
  }
}

}  // namespace bps
