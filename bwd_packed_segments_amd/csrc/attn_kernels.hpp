// Fused attention forward and backward kernels for gfx950 (CDNA4).
//
// Forward (one workgroup = 4 waves = 128 queries of one (batch row, query
// head)): the workgroup loops over the key/value tiles its queries may
// attend, in ascending order, with K and V^T staged in LDS (double
// buffered); each wave keeps its 32 queries' Q fragments in registers and
// computes S^T = K Q^T with bf16 MFMA so that a query's scores sit in one
// lane pair, runs the online softmax (running max and sum; exp2 with
// log2(e) folded into the scale) and accumulates O^T += V^T P^T.  This is
// the tiled online-softmax method of FlashAttention / FlashAttention-2
// (Dao et al.) mapped onto 64-wide waves and 32x32 MFMA tiles.
//
// Backward, in three kernels and without atomics:
//   * bwd_delta: Delta = rowsum(dO * O) and LSE in base 2 (+inf for rows
//     that attend nothing, so their probabilities come out as exact zeros);
//   * bwd_dkdv: one workgroup per (batch row, key/value head, 128 keys)
//     keeps dK^T and dV^T in registers and walks, in a sequential loop, the
//     query heads of its GQA group and then the query tiles that may attend
//     its keys; every dK/dV element is written once at the end.  The review
//     of maxdiffusion PR 485 (Code Review of the dkv and fused backward
//     kernels) is why: accumulation must never lean on the execution order
//     of grid blocks, only on loops inside one kernel instance;
//   * bwd_dq: one workgroup per (batch row, query head, 128 queries)
//     recomputes S and dP for each key tile in ascending order and keeps dQ
//     in registers, so dQ is deterministic (maxdiffusion PR 485, Code Review
//     of the dq kernel: sequential in-kernel loops instead of grid-order
//     aliasing).
//
// Tiles are classified per (query tile, key tile) from the 32-token metadata
// summaries: skipped when no pair may attend, processed without a mask when
// every pair may, and masked element by element otherwise.  Partial tiles at
// the ends of the sequences are bounds-checked and zero-filled, which plays
// the role of the dynamic last-block slicing of maxdiffusion PR 485 (Key
// Features, mask-free KV padding).
#pragma once

#include <type_traits>

#include "bps_args.hpp"
#include "lds_tile.hpp"

namespace bps {

// Tile classes of a workgroup's walk, kept in LDS.  On the metadata routes
// classifying a tile reads the 32-token summaries from global memory, a
// round trip the loop would otherwise wait for on every step; instead the
// workgroup classifies the first kClassCap tiles of its walk at once (each
// thread a few, one round trip in all).  Tiles past the table (very long
// walks) are classified when reached.
constexpr int kClassCap = 1024;

template <typename F>
__device__ inline void fill_classes(unsigned char* tab, int n, int tid, int nthreads, F classify_walk) {
  const int m = min(n, kClassCap);
  for (int i = tid; i < m; i += nthreads) tab[i] = static_cast<unsigned char>(classify_walk(i));
}

// LDS staging: two buffers when two workgroups with two buffers fit in the
// 160 KB of a CU, otherwise one; two waves per SIMD when two workgroups fit.
template <typename T, int STAGE>
struct Staging {
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr int NBUF = (4 * STAGE <= LDS_MAX) ? 2 : 1;
  static constexpr int WAVES_PER_EU = (sizeof(T) == 2 && 2 * NBUF * STAGE <= LDS_MAX) ? 2 : 1;
};

// Segment ids and positions of BN keys (general route) into LDS: direct
// loads by waves 0 and 1 when the whole tile exists, else staged with zeros.
template <int BN>
__device__ inline void stage_kv_meta(const SegView& sv, int b, int Skv, int k0, int* kid, int tid, bool direct) {
  static_assert(BN == 64, "one wave per metadata row");
  const size_t row = (size_t)b * Skv + k0;
  if (direct) {
    if (tid < 64) __builtin_amdgcn_global_load_lds(sv.ids_kv + row + tid, (BPS_LDS void*)kid, 4, 0, 0);
    else if (tid < 128) __builtin_amdgcn_global_load_lds(sv.pos_kv + row + (tid - 64), (BPS_LDS void*)(kid + BN), 4, 0, 0);
  } else if (tid < 2 * BN) {
    const int j = tid & (BN - 1);
    const bool in = k0 + j < Skv;
    kid[tid] = in ? (tid < BN ? sv.ids_kv[row + j] : sv.pos_kv[row + j]) : 0;
  }
}

// ------------------------------------------------------------ variants

// Bias values of one 32x32 tile, kept in the element type until used
// (slot r is v[r / 4][r % 4]); all zero without a bias.
template <typename T>
struct BiasTile {
  typename Elem<T>::P4 v[4];
};

// Bias of a tile with keys in rows (S^T in the forward and dQ kernels):
// slot r holds key kbase + rmap(hf, r) of brow, the bias row of the lane's
// query (NULL: no bias, or a query past Sq).  Slots 4g..4g+3 are four
// consecutive keys, loaded at once when rows are aligned (Skv a multiple
// of 4).
template <typename T>
__device__ inline BiasTile<T> bias_keys(const T* brow, int kbase, int Skv, int hf) {
  using P4 = typename Elem<T>::P4;
  BiasTile<T> b;
#pragma unroll
  for (int g = 0; g < 4; ++g) b.v[g] = P4{};
  if (brow == nullptr) return b;
  if (kbase + 32 <= Skv && (Skv & 3) == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) b.v[g] = *reinterpret_cast<const P4*>(brow + kbase + 8 * g + 4 * hf);
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kbase + rmap(hf, r);
      if (j < Skv) b.v[r >> 2][r & 3] = brow[j];
    }
  }
  return b;
}

// The same with queries in rows (S in the dK/dV kernels): slot r holds
// query ibase + rmap(hf, r) of bcol, the bias column of the lane's key
// (queries Skv elements apart; NULL: no bias, or a key past Skv).
template <typename T>
__device__ inline BiasTile<T> bias_queries(const T* bcol, int ibase, int Sq, int Skv, int hf) {
  using P4 = typename Elem<T>::P4;
  BiasTile<T> b;
#pragma unroll
  for (int g = 0; g < 4; ++g) b.v[g] = P4{};
  if (bcol == nullptr) return b;
  if (ibase + 32 <= Sq) {
#pragma unroll
    for (int r = 0; r < 16; ++r) b.v[r >> 2][r & 3] = bcol[(size_t)(ibase + rmap(hf, r)) * Skv];
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = ibase + rmap(hf, r);
      if (i < Sq) b.v[r >> 2][r & 3] = bcol[(size_t)i * Skv];
    }
  }
  return b;
}

// Raw scores of a tile -> base-2 variant logits, in place: x = raw * scale
// + bias (natural units), soft-capped to softcap * tanh(x / softcap) when a
// cap is set, times log2(e).  tanh(y) = 1 - 2 / (exp(2y) + 1), which
// saturates to +-1 as |y| grows, so a capped logit is always finite.  The
// branch is uniform, taken once per tile.
template <typename T>
__device__ inline void var_logits(f32x16& x, const BiasTile<T>& bias, const VarView& v, float scale) {
  if (v.softcap > 0.f) {
    const float sk = scale * v.cap_k;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float bk = static_cast<float>(bias.v[r >> 2][r & 3]) * v.cap_k;
      const float t = 1.f - 2.f * __builtin_amdgcn_rcpf(fast_exp2(fmaf(x[r], sk, bk)) + 1.f);
      x[r] = t * v.cap_l2;
    }
  } else {
    const float sl2 = scale * kLog2e;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = fmaf(x[r], sl2, static_cast<float>(bias.v[r >> 2][r & 3]) * kLog2e);
  }
}

// dS/dx at a base-2 logit s2 under soft-capping: 1 - tanh^2, with tanh =
// s2 / (softcap log2 e); a masked logit (-inf) gives 0.
__device__ inline float softcap_dx(float s2, const VarView& v) {
  const float t = s2 * v.cap_inv;
  return fmaxf(1.f - t * t, 0.f);
}

// Softmax gradient of a dK/dV tile (queries in rows) from base-2 variant
// logits sa and dP in pa: sa <- P = exp2(sa - LSE2), pa <- dLoss/dx =
// P (dP - Delta) dS/dx; lse2 and delta are the tile's 32 rows in LDS.  The
// soft-cap branch is uniform, taken once per tile.
__device__ inline void var_softgrad(f32x16& sa, f32x16& pa, const float* lse2, const float* delta, const VarView& v,
                                    int hf) {
  if (v.softcap > 0.f) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + 8 * grp + 4 * hf);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(delta + 8 * grp + 4 * hf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        const float s2 = sa[r];
        sa[r] = fast_exp2(s2 - l4[i]);
        pa[r] = sa[r] * (pa[r] - d4[i]) * softcap_dx(s2, v);
      }
    }
  } else {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + 8 * grp + 4 * hf);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(delta + 8 * grp + 4 * hf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        sa[r] = fast_exp2(sa[r] - l4[i]);
        pa[r] = sa[r] * (pa[r] - d4[i]);
      }
    }
  }
}

// dLoss/dx of a dK/dV tile (queries in rows, the lane's key fixed) into the
// dbias target; col is the element offset of (batch row, head, query 0, key).
template <typename T>
__device__ inline void var_store_dx(const f32x16& dx, const VarView& v, size_t col, int ibase, int Sq, int Skv,
                                    int hf) {
  if (v.dbias_f32) {
    float* p = static_cast<float*>(v.dbias) + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = ibase + rmap(hf, r);
      if (i < Sq) p[(size_t)i * Skv] = dx[r];
    }
  } else {
    T* p = static_cast<T*>(v.dbias) + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = ibase + rmap(hf, r);
      if (i < Sq) p[(size_t)i * Skv] = static_cast<T>(dx[r]);
    }
  }
}

// ------------------------------------------------------------ forward

// W waves of 32 queries each, over HP query heads of one GQA group (W / HP
// waves per head).  Four waves and one head (two workgroups per CU) by
// default.  Eight waves load each key/value tile once for twice the
// queries, which halves the load instructions per product: as two heads of
// a GQA group over the same 128 queries (the masks are those of one head),
// or, without a group to share, as one head over 256 queries for bf16
// without segment metadata or causal mask, where wide query tiles cost no
// extra masked work (measured: 4 % less forward time on an 18,900 x 75,600
// shard, but 4-8 % more on the 8K causal workload).
template <typename T, int DQK, int DV, int W = 4, int HP = 1>
struct FwdCfg {
  static constexpr int QW = W / HP;     // waves per head
  static constexpr int BM = 32 * QW;
  static constexpr int BN = 64;
  static constexpr int THREADS = 64 * W;
  static constexpr int K_BYTES = BN * DQK * (int)sizeof(T);
  static constexpr int V_BYTES = BN * DV * (int)sizeof(T);
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES + 2 * BN * 4;
  static constexpr int NBUF = W == 8 ? 2 : Staging<T, STAGE_BYTES>::NBUF;
  static constexpr int WAVES_PER_EU = W == 8 ? 2 : Staging<T, STAGE_BYTES>::WAVES_PER_EU;
  static constexpr bool WIDE_OK = sizeof(T) == 2 && 2 * STAGE_BYTES <= 160 * 1024;
};

// VM: 0 plain; 1 sink and max logit only (scores stay raw); 2 any variant,
// with the scores turned into bias / soft-cap logits.
template <typename T, int DQK, int DV, int VM, int W = 4, int HP = 1>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(FwdCfg<T, DQK, DV, W, HP>::WAVES_PER_EU)))
    attn_fwd_kernel(FwdArgs a) {
  constexpr bool VAR = VM != 0;      // sink, max logit
  constexpr bool XFORM = VM == 2;    // bias, soft cap
  using C = FwdCfg<T, DQK, DV, W, HP>;
  using E = Elem<T>;
  using F8 = typename E::F8;
  constexpr int BM = C::BM, BN = C::BN, QW = C::QW;
  __shared__ __attribute__((aligned(1024))) char smem[C::NBUF * C::STAGE_BYTES];

  const AttnShape& s = a.s;
  const bool causal = s.causal != 0;
  const int n_qt = (s.Sq + BM - 1) / BM;
  const int g = s.Hq / s.Hkv;
  const int ngh = g / HP;            // head groups of HP per KV head
  const int nblocks = s.B * s.Hkv * ngh * n_qt;
  int L = logical_block(nblocks, s.reverse);
  const int hgp = L % ngh;
  L /= ngh;
  const int qrank = L % n_qt;
  L /= n_qt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  const int qt = BM == 128 ? q_tile_of(a.seg, b, qrank, n_qt, causal) : (causal ? n_qt - 1 - qrank : qrank);
  const int q0 = qt * BM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int h = hkv * g + hgp * HP + wave / QW;   // this wave's query head
  const int wq = wave % QW;                        // this wave's 32 rows of the tile
  const int qi = q0 + wq * 32 + n;

  const T* qp = static_cast<const T*>(a.q) + b * a.sq.b + h * a.sq.h;
  const T* kp = static_cast<const T*>(a.k) + b * a.sk.b + hkv * a.sk.h;
  const T* vp = static_cast<const T*>(a.v) + b * a.sv.b + hkv * a.sv.h;

  F8 qf[DQK / 16];
#pragma unroll
  for (int t = 0; t < DQK / 16; ++t)
    qf[t] = qi < s.Sq ? E::load8(qp + qi * a.sq.t + 16 * t + 8 * hf) : E::zero8();

  const int route = s.has_meta ? a.seg.route[b] : kRouteDense;
  const bool general = route == kRouteGeneral;
  const TokMeta qm = q_meta(route, a.seg, b, s.Sq, qi);
  TileSum qs{};
  const ChunkSum* sum_kv_row = nullptr;
  if (route != kRouteDense) {
    qs = tile_sum(a.seg.sum_q + (size_t)b * a.seg.nch_q, a.seg.nch_q, q0, BM);
    sum_kv_row = a.seg.sum_kv + (size_t)b * a.seg.nch_kv;
  }
  int lo, hi;
  kv_range(route, causal, s.Skv, q0, BM, qs, lo, hi);
  const int t_lo = lo / BN;
  const int t_hi = (hi + BN - 1) / BN;

  auto classify = [&](int kt) -> int {
    TileSum ks{};
    if (route != kRouteDense) ks = tile_sum(sum_kv_row, a.seg.nch_kv, kt * BN, BN);
    return classify_tile(route, causal, s.Skv, q0, BM, kt * BN, BN, qs, ks);
  };
  __shared__ unsigned char cls_tab[kClassCap];
  const bool tabled = route != kRouteDense;
  if (tabled) {
    fill_classes(cls_tab, t_hi - t_lo, tid, C::THREADS, [&](int i) { return classify(t_lo + i); });
    __syncthreads();
  }
  auto next_tile = [&](int kt, int& cls) -> int {
    for (int k = kt; k < t_hi; ++k) {
      cls = (tabled && k - t_lo < kClassCap) ? (int)cls_tab[k - t_lo] : classify(k);
      if (cls != kTileSkip) return k;
    }
    cls = kTileSkip;
    return t_hi;
  };
  auto stage = [&](int buf) { return smem + buf * C::STAGE_BYTES; };
  auto issue = [&](int kt, int buf) {
    T* Ks = reinterpret_cast<T*>(stage(buf));
    T* Vs = Ks + BN * DQK;
    int* kid = reinterpret_cast<int*>(Vs + BN * DV);
    const int k0 = kt * BN;
    const int nvalid = min(BN, s.Skv - k0);
    if (nvalid == BN) {
      TileLoad<T, BN, DQK, C::THREADS>::direct(kp + k0 * a.sk.t, a.sk.t, Ks, tid);
      TileLoad<T, BN, DV, C::THREADS>::direct(vp + k0 * a.sv.t, a.sv.t, Vs, tid);
    } else {
      TileLoad<T, BN, DQK, C::THREADS>::staged(kp + k0 * a.sk.t, a.sk.t, nvalid, Ks, tid);
      TileLoad<T, BN, DV, C::THREADS>::staged(vp + k0 * a.sv.t, a.sv.t, nvalid, Vs, tid);
    }
    if (general) stage_kv_meta<BN>(a.seg, b, s.Skv, k0, kid, tid, nvalid == BN);
  };

  // The scores stay raw (c2 folds in the scale) unless a bias or a soft cap
  // changes them; then they are turned into base-2 logits first (c2 = 1).
  const float c2 = XFORM ? 1.f : s.scale_log2;
  float m = -INFINITY;   // reference max of the scores (rescaled lazily)
  float l = 0.f;         // this lane half's partial sum of exp2((s - m) * c2)
  float mxe = -INFINITY; // exact max of this query's allowed scores
  const T* brow = nullptr;
  if constexpr (XFORM) {
    if (a.var.bias != nullptr && qi < s.Sq)
      brow = static_cast<const T*>(a.var.bias) + b * a.var.bias_b + ((size_t)h * s.Sq + qi) * s.Skv;
  }
  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};

  int cls;
  int kt = next_tile(t_lo, cls);
  int buf = 0;
  if (kt < t_hi) issue(kt, 0);
  wait_vm();
  __syncthreads();

  while (kt < t_hi) {
    int ncls;
    const int nkt = next_tile(kt + 1, ncls);
    if (C::NBUF == 2 && nkt < t_hi) issue(nkt, buf ^ 1);

    const T* Ks = reinterpret_cast<const T*>(stage(buf));
    const T* Vs = Ks + BN * DQK;
    const int* kid = reinterpret_cast<const int*>(Vs + BN * DV);
    const int k0 = kt * BN;

    // S^T = K Q^T for the tile's 64 keys (two 32-key blocks).  For bf16 the
    // K fragments are read two k-steps ahead (a ring of three), pinned in
    // that order with scheduling groups: left alone, the compiler reads each
    // pair just before its products and waits a full LDS round trip every
    // step (measured: 0.7-0.9 % less forward time on the 8K GQA workload;
    // the same change in dQ and in the dK/dV producers made them 3-4 %
    // slower).
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    if constexpr (sizeof(T) != 2) {
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          sacc[blk] = mma(frag_row<T, DQK>(Ks, blk * 32 + n, 16 * t + 8 * hf), qf[t], sacc[blk]);
    } else {
      constexpr int NT = DQK / 16;
      F8 kr[3][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) kr[t][blk] = frag_row<T, DQK>(Ks, blk * 32 + n, 16 * t + 8 * hf);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + 2 < NT) {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
            kr[(t + 2) % 3][blk] = frag_row<T, DQK>(Ks, blk * 32 + n, 16 * (t + 2) + 8 * hf);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) sacc[blk] = mma(kr[t % 3][blk], qf[t], sacc[blk]);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
    if constexpr (XFORM) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        var_logits<T>(sacc[blk], bias_keys<T>(brow, k0 + blk * 32, s.Skv, hf), a.var, s.scale);
    }

    if (cls == kTilePart) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        mask_tile<true>(sacc[blk], -INFINITY, route, causal, s.Skv, qi, qm, k0 + blk * 32, hf, kid, kid + BN, blk * 32);
    }

    // Online softmax with a lazily updated reference max: the accumulators
    // are rescaled only when the running max grows by more than 2^8 in
    // probability terms, so most tiles skip the O rescale entirely.
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
    mx = wave_xor32_max(mx);
    if constexpr (VAR) mxe = fmaxf(mxe, mx);
    const bool grow = mx > m && (m == -INFINITY || (mx - m) * c2 > 8.f);
    if (__any(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = grow ? fast_exp2((m - m_new) * c2) : 1.f;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;
      m = m_new;
    }
    const float mc = (m == -INFINITY ? 0.f : m) * c2;
    float rs = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[blk][r], c2, -mc));
        sacc[blk][r] = p;
        rs += p;
      }
    l += rs;

    // O^T += V^T P^T, V^T read from the row-major V tile by transpose loads.
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const F8 pf = E::cvt8(slots8(sacc[blk], s2));
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
          o[d] = mma(frag_tr<T, DV>(Vs, d * 32, blk * 32 + 16 * s2, lane), pf, o[d]);
      }

    if (C::NBUF == 1) {
      __syncthreads();
      if (nkt < t_hi) issue(nkt, buf);
    }
    wait_vm();
    __syncthreads();
    if (C::NBUF == 2) buf ^= 1;
    kt = nkt;
    cls = ncls;
  }

  // Epilogue: O = O^T / l, LSE = m * scale + ln(l); empty rows give O = 0,
  // LSE = -inf.
  const float lt = wave_xor32_sum(l);
  float inv = lt > 0.f ? 1.f / lt : 0.f;
  float lse = lt > 0.f ? m * s.scale + logf(lt) : -INFINITY;
  if constexpr (VAR) {
    // In base-2 units the reference is m * c2.  The sink adds
    // exp2(sink2 - ref) to the sum of terms; the reference moves to the
    // larger of the two so that no term overflows.  A row with no allowed
    // key then has O = 0 and LSE = sink.
    const float m2 = m * c2;
    float ref = m2, tot = lt, alpha = 1.f;
    if (a.var.sink != nullptr) {
      const float s2 = a.var.sink[h] * kLog2e;
      if (lt > 0.f) {
        ref = fmaxf(m2, s2);
        alpha = fast_exp2(m2 - ref);
        tot = lt * alpha + fast_exp2(s2 - ref);
      } else {
        ref = s2;
        alpha = 0.f;
        tot = 1.f;
      }
    }
    inv = tot > 0.f ? alpha / tot : 0.f;
    lse = tot > 0.f ? ref * kLn2 + logf(tot) : -INFINITY;
    if (a.var.ml_part != nullptr) {
      float wm = qi < s.Sq ? mxe : -INFINITY;
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) wm = fmaxf(wm, __shfl_xor(wm, d));
      if (lane == 0) a.var.ml_part[(((size_t)h * s.B + b) * n_qt + qt) * 4 + wq] = wm * (c2 * kLn2);
    }
  }
  if (qi < s.Sq) {
    T* op = static_cast<T*>(a.o) + b * a.so.b + qi * a.so.t + h * a.so.h;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 x = f32x4{o[d][4 * grp], o[d][4 * grp + 1], o[d][4 * grp + 2], o[d][4 * grp + 3]} * inv;
        *reinterpret_cast<typename E::P4*>(op + d * 32 + 8 * grp + 4 * hf) = E::cvt4(x);
      }
    if (hf == 0) a.lse[((size_t)b * s.Hq + h) * s.Sq + qi] = lse;
  }
}

// ------------------------------------------------------------ backward: Delta

template <typename T, int DV, bool VAR>
__global__ void __launch_bounds__(256) attn_bwd_delta_kernel(BwdArgs a) {
  using E = Elem<T>;
  using F8 = typename E::F8;
  constexpr int PARTS = 8;                 // lanes per row
  constexpr int CH = DV / 8 / PARTS;       // 8-element chunks per lane
  const AttnShape& s = a.s;
  const size_t rows = (size_t)s.B * s.Sq * s.Hq;
  const size_t row = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / PARTS;
  const int part = threadIdx.x % PARTS;
  float acc = 0.f;
  int b = 0, i = 0, h = 0;
  if (row < rows) {
    h = (int)(row % s.Hq);
    i = (int)((row / s.Hq) % s.Sq);
    b = (int)(row / ((size_t)s.Hq * s.Sq));
    const T* op = static_cast<const T*>(a.o) + b * a.so.b + i * a.so.t + h * a.so.h;
    const T* dp = static_cast<const T*>(a.dout) + b * a.so.b + i * a.so.t + h * a.so.h;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int off = (c * PARTS + part) * 8;
      const F8 x = E::load8(op + off);
      const F8 y = E::load8(dp + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
    }
  }
#pragma unroll
  for (int d = 1; d < PARTS; d <<= 1) acc += __shfl_xor(acc, d);
  if (row < rows && part == 0) {
    const size_t x = ((size_t)b * s.Hq + h) * s.Sq + i;
    a.delta[x] = acc;
    const float lse = a.lse[x];
    const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
    a.lse2[x] = lse2;
    // The sink's share of the row, exp(sink - LSE), times -Delta: this
    // row's term of dLoss/dsink.
    if constexpr (VAR) {
      if (a.var.dsink_row != nullptr) a.var.dsink_row[x] = -fast_exp2(a.var.sink[h] * kLog2e - lse2) * acc;
    }
  }
}

// ------------------------------------------------------------ backward: dQ

// W waves of 32 queries each over HP query heads, as for the forward:
// eight waves as two heads of a GQA group, or as 256-query tiles of one
// head for bf16 without metadata or causal mask.
template <typename T, int DQK, int DV, int W = 4, int HP = 1>
struct DqCfg {
  static constexpr int QW = W / HP;
  static constexpr int BM = 32 * QW;
  static constexpr int BN = 64;
  static constexpr int THREADS = 64 * W;
  static constexpr int K_BYTES = BN * DQK * (int)sizeof(T);
  static constexpr int V_BYTES = BN * DV * (int)sizeof(T);
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES + 2 * BN * 4;
  static constexpr int NBUF = W == 8 ? 2 : Staging<T, STAGE_BYTES>::NBUF;
  // Q, dO fragments and the dQ accumulator outgrow half the register file
  // for wide heads.
  static constexpr int WAVES_PER_EU =
      (DQK > 128 || DQK + DV > 256) ? 1 : (W == 8 ? 2 : Staging<T, STAGE_BYTES>::WAVES_PER_EU);
  static constexpr bool WIDE_OK = sizeof(T) == 2 && DQK <= 128 && DQK + DV <= 256 && 2 * STAGE_BYTES <= 160 * 1024;
};

template <typename T, int DQK, int DV, bool VAR, int W = 4, int HP = 1>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(DqCfg<T, DQK, DV, W, HP>::WAVES_PER_EU)))
    attn_bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<T, DQK, DV, W, HP>;
  using E = Elem<T>;
  using F8 = typename E::F8;
  constexpr int BM = C::BM, BN = C::BN, QW = C::QW;
  __shared__ __attribute__((aligned(1024))) char smem[C::NBUF * C::STAGE_BYTES];

  const AttnShape& s = a.s;
  const bool causal = s.causal != 0;
  const int n_qt = (s.Sq + BM - 1) / BM;
  const int g = s.Hq / s.Hkv;
  const int ngh = g / HP;            // head groups of HP per KV head
  const int nblocks = s.B * s.Hkv * ngh * n_qt;
  int L = logical_block(nblocks, s.reverse);
  const int hgp = L % ngh;
  L /= ngh;
  const int qrank = L % n_qt;
  L /= n_qt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  const int qt = BM == 128 ? q_tile_of(a.seg, b, qrank, n_qt, causal) : (causal ? n_qt - 1 - qrank : qrank);
  const int q0 = qt * BM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int h = hkv * g + hgp * HP + wave / QW;   // this wave's query head
  const int qi = q0 + (wave % QW) * 32 + n;

  const T* qp = static_cast<const T*>(a.q) + b * a.sq.b + h * a.sq.h;
  const T* dop = static_cast<const T*>(a.dout) + b * a.so.b + h * a.so.h;
  const T* kp = uniform_ptr(static_cast<const T*>(a.k) + b * a.sk.b + hkv * a.sk.h);
  const T* vp = uniform_ptr(static_cast<const T*>(a.v) + b * a.sv.b + hkv * a.sv.h);

  F8 qf[DQK / 16];
  F8 dof[DV / 16];
#pragma unroll
  for (int t = 0; t < DQK / 16; ++t)
    qf[t] = qi < s.Sq ? E::load8(qp + qi * a.sq.t + 16 * t + 8 * hf) : E::zero8();
#pragma unroll
  for (int t = 0; t < DV / 16; ++t)
    dof[t] = qi < s.Sq ? E::load8(dop + qi * a.so.t + 16 * t + 8 * hf) : E::zero8();
  const size_t rowx = ((size_t)b * s.Hq + h) * s.Sq + qi;
  const float lse2 = qi < s.Sq ? a.lse2[rowx] : INFINITY;
  const float delta = qi < s.Sq ? a.delta[rowx] : 0.f;

  const int route = s.has_meta ? a.seg.route[b] : kRouteDense;
  const bool general = route == kRouteGeneral;
  const TokMeta qm = q_meta(route, a.seg, b, s.Sq, qi);
  TileSum qs{};
  const ChunkSum* sum_kv_row = nullptr;
  if (route != kRouteDense) {
    qs = tile_sum(a.seg.sum_q + (size_t)b * a.seg.nch_q, a.seg.nch_q, q0, BM);
    sum_kv_row = a.seg.sum_kv + (size_t)b * a.seg.nch_kv;
  }
  int lo, hi;
  kv_range(route, causal, s.Skv, q0, BM, qs, lo, hi);
  const int t_lo = lo / BN;
  const int t_hi = (hi + BN - 1) / BN;
  auto classify = [&](int kt) -> int {
    TileSum ks{};
    if (route != kRouteDense) ks = tile_sum(sum_kv_row, a.seg.nch_kv, kt * BN, BN);
    return classify_tile(route, causal, s.Skv, q0, BM, kt * BN, BN, qs, ks);
  };
  __shared__ unsigned char cls_tab[kClassCap];
  const bool tabled = route != kRouteDense;
  if (tabled) {
    fill_classes(cls_tab, t_hi - t_lo, tid, C::THREADS, [&](int i) { return classify(t_lo + i); });
    __syncthreads();
  }
  auto next_tile = [&](int kt, int& cls) -> int {
    for (int k = kt; k < t_hi; ++k) {
      cls = (tabled && k - t_lo < kClassCap) ? (int)cls_tab[k - t_lo] : classify(k);
      if (cls != kTileSkip) return k;
    }
    cls = kTileSkip;
    return t_hi;
  };
  auto stage = [&](int buf) { return smem + buf * C::STAGE_BYTES; };
  auto issue = [&](int kt, int buf) {
    T* Ks = reinterpret_cast<T*>(stage(buf));
    T* Vs = Ks + BN * DQK;
    int* kid = reinterpret_cast<int*>(Vs + BN * DV);
    const int k0 = kt * BN;
    const int nvalid = min(BN, s.Skv - k0);
    if (nvalid == BN) {
      TileLoad<T, BN, DQK, C::THREADS, true>::direct(kp + k0 * a.sk.t, a.sk.t, Ks, tid);
      TileLoad<T, BN, DV, C::THREADS, true>::direct(vp + k0 * a.sv.t, a.sv.t, Vs, tid);
    } else {
      TileLoad<T, BN, DQK, C::THREADS, true>::staged(kp + k0 * a.sk.t, a.sk.t, nvalid, Ks, tid);
      TileLoad<T, BN, DV, C::THREADS, true>::staged(vp + k0 * a.sv.t, a.sv.t, nvalid, Vs, tid);
    }
    if (general) stage_kv_meta<BN>(a.seg, b, s.Skv, k0, kid, tid, nvalid == BN);
  };

  const float c2 = s.scale_log2;
  const T* brow = nullptr;
  if constexpr (VAR) {
    if (a.var.bias != nullptr && qi < s.Sq)
      brow = static_cast<const T*>(a.var.bias) + b * a.var.bias_b + ((size_t)h * s.Sq + qi) * s.Skv;
  }
  f32x16 dqa[DQK / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dqa[d] = f32x16{};

  // Per-lane LDS byte offsets inside a stage, fixed for the walk (bf16): K
  // rows and V rows (fragment t of row n of the first 32-key block) and the
  // transposed K reads (column block d, rows y and y + 8 of the first
  // 16-row group).  The key block and the stage add immediates: the loop is
  // unrolled over the two stages.
  uint32_t kro[DQK / 16], vro[DV / 16], ktr[DQK / 32][2];
  if constexpr (sizeof(T) == 2) {
    using FK = TileFmt<T, DQK>;
    using FV = TileFmt<T, DV>;
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t) kro[t] = (uint32_t)FK::off(n, 16 * t + 8 * hf) * 2;
#pragma unroll
    for (int t = 0; t < DV / 16; ++t) vro[t] = (uint32_t)(BN * DQK * 2 + FV::off(n, 16 * t + 8 * hf) * 2);
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int G = lane >> 4, i = lane & 15;
        ktr[d][p] = (uint32_t)FK::off(4 * (G >> 1) + (i >> 2) + 8 * p, 32 * d + 16 * (G & 1) + 4 * (i & 3)) * 2;
      }
  }
  // Natural operand fragment t of row blk * 32 + n of the K (V) tile in
  // stage ST; transposed K fragment (column block d, rows y0 ..).
  auto rd_k = [&](auto stc, int blk, int t) __attribute__((always_inline)) -> F8 {
    constexpr int ST = decltype(stc)::value;
    const T* Ks = reinterpret_cast<const T*>(stage(ST));
    if constexpr (sizeof(T) == 2)
      return *reinterpret_cast<const F8*>(smem + ST * C::STAGE_BYTES + blk * 32 * DQK * 2 + kro[t]);
    else
      return frag_row<T, DQK>(Ks, blk * 32 + n, 16 * t + 8 * hf);
  };
  auto rd_v = [&](auto stc, int blk, int t) __attribute__((always_inline)) -> F8 {
    constexpr int ST = decltype(stc)::value;
    const T* Vs = reinterpret_cast<const T*>(stage(ST)) + BN * DQK;
    if constexpr (sizeof(T) == 2)
      return *reinterpret_cast<const F8*>(smem + ST * C::STAGE_BYTES + blk * 32 * DV * 2 + vro[t]);
    else
      return frag_row<T, DV>(Vs, blk * 32 + n, 16 * t + 8 * hf);
  };
  auto rd_ktr = [&](auto stc, int d, int y0) __attribute__((always_inline)) -> F8 {
    constexpr int ST = decltype(stc)::value;
    const T* Ks = reinterpret_cast<const T*>(stage(ST));
    if constexpr (sizeof(T) == 2) {
      const char* base = smem + ST * C::STAGE_BYTES + y0 * DQK * 2;
      const bf16x4v x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)(base + ktr[d][0]));
      const bf16x4v y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)(base + ktr[d][1]));
      return F8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    } else {
      return frag_tr<T, DQK>(Ks, d * 32, y0, lane);
    }
  };

  int cls;
  int kt = next_tile(t_lo, cls);
  if (kt < t_hi) issue(kt, 0);
  wait_vm();
  __syncthreads();

  // One key tile in stage ST (the next one fetched into the other stage).
  auto step = [&](auto stc) __attribute__((always_inline)) -> bool {
    constexpr int ST = decltype(stc)::value;
    if (kt >= t_hi) return false;
    int ncls;
    const int nkt = next_tile(kt + 1, ncls);
    if (C::NBUF == 2 && nkt < t_hi) issue(nkt, ST ^ 1);

    const T* Vs = reinterpret_cast<const T*>(stage(ST)) + BN * DQK;
    const int* kid = reinterpret_cast<const int*>(Vs + BN * DV);
    const int k0 = kt * BN;

#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      // S^T and dP^T for 32 keys x this wave's 32 queries.
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) sacc = mma(rd_k(stc, blk, t), qf[t], sacc);
#pragma unroll
      for (int t = 0; t < DV / 16; ++t) pacc = mma(rd_v(stc, blk, t), dof[t], pacc);
      if constexpr (VAR) {
        // Variant logits, masked to -inf, then P and dLoss/dx = P (dP -
        // Delta) dS/dx in one pass.
        var_logits<T>(sacc, bias_keys<T>(brow, k0 + blk * 32, s.Skv, hf), a.var, s.scale);
        if (cls == kTilePart)
          mask_tile<true>(sacc, -INFINITY, route, causal, s.Skv, qi, qm, k0 + blk * 32, hf, kid, kid + BN, blk * 32);
        if (a.var.softcap > 0.f) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float s2 = sacc[r];
            sacc[r] = fast_exp2(s2 - lse2) * (pacc[r] - delta) * softcap_dx(s2, a.var);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(sacc[r] - lse2) * (pacc[r] - delta);
        }
      } else {
        // P = exp2(S * scale * log2e - LSE2); dS = P * (dP - Delta).
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(fmaf(sacc[r], c2, -lse2));
        if (cls == kTilePart)
          mask_tile<true>(sacc, 0.f, route, causal, s.Skv, qi, qm, k0 + blk * 32, hf, kid, kid + BN, blk * 32);
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = sacc[r] * (pacc[r] - delta);
      }
      // dQ^T += K^T dS^T, K^T read from the row-major K tile by transpose loads.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const F8 dsf = E::cvt8(slots8(sacc, s2));
#pragma unroll
        for (int d = 0; d < DQK / 32; ++d) dqa[d] = mma(rd_ktr(stc, d, blk * 32 + 16 * s2), dsf, dqa[d]);
      }
    }

    if (C::NBUF == 1) {
      __syncthreads();
      if (nkt < t_hi) issue(nkt, ST);
    }
    wait_vm();
    __syncthreads();
    kt = nkt;
    cls = ncls;
    return true;
  };
  if constexpr (C::NBUF == 2) {
    while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
    }
  } else {
    while (step(std::integral_constant<int, 0>{})) {
    }
  }

  if (qi < s.Sq) {
    T* dqp = static_cast<T*>(a.dq) + b * a.sq.b + qi * a.sq.t + h * a.sq.h;
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 x = f32x4{dqa[d][4 * grp], dqa[d][4 * grp + 1], dqa[d][4 * grp + 2], dqa[d][4 * grp + 3]} * s.scale;
        *reinterpret_cast<typename E::P4*>(dqp + d * 32 + 8 * grp + 4 * hf) = E::cvt4(x);
      }
  }
}

// ------------------------------------------------------------ backward: dK, dV

template <typename T, int DQK, int DV>
struct DkvCfg {
  static constexpr int BN = 128;   // keys per workgroup (32 per wave)
  // Queries per step: two 32-row blocks, one for wide heads and fp32 (the
  // transposed operands of a step are held in registers).
  static constexpr int BM = (sizeof(T) == 4 || DQK > 128 || DQK + DV > 256) ? 32 : 64;
  static constexpr int Q_BYTES = BM * DQK * (int)sizeof(T);
  static constexpr int DO_BYTES = BM * DV * (int)sizeof(T);
  static constexpr int SIDE_BYTES = BM * 4 * 4;   // lse2, delta, metadata (a, b)
  static constexpr int STAGE_BYTES = Q_BYTES + DO_BYTES + SIDE_BYTES;
  // Three buffers: the loads for step x + 2 are issued when step x ends, so
  // they have a whole step to land (one workgroup per CU, see below).
  static constexpr int NBUF = (3 * STAGE_BYTES <= 160 * 1024) ? 3 : 1;
  // K, V fragments and the dK, dV accumulators alone take 192 registers per
  // lane; with the rest this kernel needs more than 256, so one wave per SIMD.
  static constexpr int WAVES_PER_EU = 1;
};

template <typename T, int DQK, int DV, bool VAR>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DkvCfg<T, DQK, DV>::WAVES_PER_EU)))
    attn_bwd_dkdv_kernel(BwdArgs a) {
  using C = DkvCfg<T, DQK, DV>;
  using E = Elem<T>;
  using F8 = typename E::F8;
  constexpr int BM = C::BM, BN = C::BN;
  static_assert(BM == 32 || BM == 64, "one wave per side row");
  __shared__ __attribute__((aligned(1024))) char smem[C::NBUF * C::STAGE_BYTES];

  const AttnShape& s = a.s;
  const bool causal = s.causal != 0;
  const int n_kt = (s.Skv + BN - 1) / BN;
  const int g = s.Hq / s.Hkv;
  const int nblocks = s.B * s.Hkv * n_kt;
  int L = logical_block(nblocks, s.reverse);
  const int krank = L % n_kt;
  L /= n_kt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  const int kt = k_tile_of(a.seg, b, krank, n_kt);   // fixed order: low key tiles (the longest causal walks) first
  const int k0 = kt * BN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int kj = k0 + wave * 32 + n;

  const T* kp = static_cast<const T*>(a.k) + b * a.sk.b + hkv * a.sk.h;
  const T* vp = static_cast<const T*>(a.v) + b * a.sv.b + hkv * a.sv.h;
  F8 kf[DQK / 16];
  F8 vf[DV / 16];
#pragma unroll
  for (int t = 0; t < DQK / 16; ++t)
    kf[t] = kj < s.Skv ? E::load8(kp + kj * a.sk.t + 16 * t + 8 * hf) : E::zero8();
#pragma unroll
  for (int t = 0; t < DV / 16; ++t)
    vf[t] = kj < s.Skv ? E::load8(vp + kj * a.sv.t + 16 * t + 8 * hf) : E::zero8();

  const int route = s.has_meta ? a.seg.route[b] : kRouteDense;
  const bool general = route == kRouteGeneral;
  const TokMeta km = general ? kv_meta(route, a.seg, b, s.Skv, kj) : TokMeta{0, 0};
  TileSum ks{};
  const ChunkSum* sum_q_row = nullptr;
  if (route != kRouteDense) {
    ks = tile_sum(a.seg.sum_kv + (size_t)b * a.seg.nch_kv, a.seg.nch_kv, k0, BN);
    sum_q_row = a.seg.sum_q + (size_t)b * a.seg.nch_q;
  }
  int lo, hi;
  q_range(route, causal, s.Sq, k0, BN, ks, lo, hi);
  const int t_lo = lo / BM;
  const int t_hi = (hi + BM - 1) / BM;
  const int ntiles = t_hi - t_lo;
  const int nsteps = g * ntiles;

  // Steps walk the query tiles from the last one down, and the query heads
  // of the group inside each tile: workgroups of one key/value head then
  // read the same query tiles at about the same time (L2 reuse).
  auto tile_of = [&](int x) { return t_hi - 1 - x / g; };
  auto classify = [&](int qt) -> int {
    TileSum qs{};
    if (route != kRouteDense) qs = tile_sum(sum_q_row, a.seg.nch_q, qt * BM, BM);
    return classify_tile(route, causal, s.Skv, qt * BM, BM, k0, BN, qs, ks);
  };
  __shared__ unsigned char cls_tab[kClassCap];
  const bool tabled = route != kRouteDense;
  if (tabled) {
    fill_classes(cls_tab, ntiles, tid, 256, [&](int u) { return classify(t_hi - 1 - u); });
    __syncthreads();
  }
  auto next_step = [&](int x, int& cls) -> int {
    while (x < nsteps) {
      const int u = x / g;
      cls = (tabled && u < kClassCap) ? (int)cls_tab[u] : classify(tile_of(x));
      if (cls != kTileSkip) return x;
      x = (u + 1) * g;   // the whole tile is skipped for every head
    }
    cls = kTileSkip;
    return nsteps;
  };

  // Q, dO and the per-row side data of a step go straight from global memory
  // to LDS (through registers with zero fill for the last, partial tile).
  // Returns whether the loads are still in flight.
  auto issue = [&](int x, char* st) -> bool {
    T* Qs = reinterpret_cast<T*>(st);
    T* dOs = Qs + BM * DQK;
    float* side = reinterpret_cast<float*>(dOs + BM * DV);
    const int h = hkv * g + x % g;
    const int i0 = tile_of(x) * BM;
    const int nvalid = min(BM, s.Sq - i0);
    const T* qg = static_cast<const T*>(a.q) + b * a.sq.b + h * a.sq.h + i0 * a.sq.t;
    const T* dg = static_cast<const T*>(a.dout) + b * a.so.b + h * a.so.h + i0 * a.so.t;
    const size_t rowx = ((size_t)b * s.Hq + h) * s.Sq + i0;
    const size_t rowm = (size_t)b * s.Sq + i0;
    if (nvalid == BM) {
      TileLoad<T, BM, DQK, 256>::direct(qg, a.sq.t, Qs, tid);
      TileLoad<T, BM, DV, 256>::direct(dg, a.so.t, dOs, tid);
      // wave 0: LSE in base 2, wave 1: Delta, waves 2 and 3: row metadata
      const int* src;
      if (wave == 0) src = reinterpret_cast<const int*>(a.lse2 + rowx) + lane;
      else if (wave == 1) src = reinterpret_cast<const int*>(a.delta + rowx) + lane;
      else if (route == kRouteFast) src = reinterpret_cast<const int*>(a.seg.run_q + rowm + lane) + (wave - 2);
      else if (route == kRouteGeneral) src = (wave == 2 ? a.seg.ids_q : a.seg.pos_q) + rowm + lane;
      else src = nullptr;
      if (src && lane < BM) __builtin_amdgcn_global_load_lds(src, (BPS_LDS void*)(side + wave * BM), 4, 0, 0);
      return true;
    }
    TileLoad<T, BM, DQK, 256>::staged(qg, a.sq.t, nvalid, Qs, tid);
    TileLoad<T, BM, DV, 256>::staged(dg, a.so.t, nvalid, dOs, tid);
    const int r = lane;
    const bool in = r < nvalid;
    if (r < BM) {
      if (wave == 0) {
        side[r] = in ? a.lse2[rowx + r] : INFINITY;
      } else if (wave == 1) {
        side[BM + r] = in ? a.delta[rowx + r] : 0.f;
      } else {
        const TokMeta t = in ? q_meta(route, a.seg, b, s.Sq, i0 + r) : TokMeta{0, 0};
        reinterpret_cast<int*>(side)[wave * BM + r] = wave == 2 ? t.a : t.b;
      }
    }
    return false;
  };

  const float c2 = s.scale_log2;
  f32x16 dka[DQK / 32];
  f32x16 dva[DV / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dka[d] = f32x16{};
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) dva[d] = f32x16{};

  // One step over BM queries of one head.  The two 32-query blocks are
  // interleaved: block 1's S and dP products are issued before block 0's
  // softmax gradient, and block 0's dV and dK products before block 1's, so
  // the matrix cores have independent work while the VALU runs (one wave per
  // SIMD: nothing else would fill those cycles).  part: the tile needs the
  // element mask.
  auto compute = [&](const char* st, int x, bool part) {
    const T* Qs = reinterpret_cast<const T*>(st);
    const T* dOs = Qs + BM * DQK;
    const float* lse2s = reinterpret_cast<const float*>(dOs + BM * DV);
    const float* deltas = lse2s + BM;
    const int* qma = reinterpret_cast<const int*>(lse2s + 2 * BM);
    const int* qmb = qma + BM;
    const int i0 = tile_of(x) * BM;
    constexpr int NQB = BM / 32;
    const T* bcol = nullptr;   // variants: bias column of this lane's key
    size_t dcol = 0;           // and its offset in the dbias target
    if constexpr (VAR) {
      const size_t col = (size_t)(hkv * g + x % g) * s.Sq * s.Skv + kj;
      if (a.var.bias != nullptr && kj < s.Skv) bcol = static_cast<const T*>(a.var.bias) + b * a.var.bias_b + col;
      dcol = b * a.var.dbias_b + col;
    }

    auto sdp = [&](int qb, f32x16& sa, f32x16& pa, BiasTile<T>& bq) {
      if constexpr (VAR) bq = bias_queries<T>(bcol, i0 + qb * 32, s.Sq, s.Skv, hf);   // in flight under the products
      F8 qa[DQK / 16], da[DV / 16];
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) qa[t] = frag_row<T, DQK>(Qs, qb * 32 + n, 16 * t + 8 * hf);
#pragma unroll
      for (int t = 0; t < DV / 16; ++t) da[t] = frag_row<T, DV>(dOs, qb * 32 + n, 16 * t + 8 * hf);
      sa = f32x16{};
      pa = f32x16{};
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) sa = mma(qa[t], kf[t], sa);
#pragma unroll
      for (int t = 0; t < DV / 16; ++t) pa = mma(da[t], vf[t], pa);
    };
    // P = exp2(S * scale * log2e - LSE2), dS = P * (dP - Delta); returns the
    // bf16 operands of the dV and dK products.
    auto softgrad = [&](int qb, f32x16& sa, f32x16& pa, const BiasTile<T>& bq, F8* pf, F8* dsf) {
      if constexpr (VAR) {
        // Variant logits, masked to -inf, then P and dLoss/dx = P (dP -
        // Delta) dS/dx in one pass; dx also goes to the dbias target.
        var_logits<T>(sa, bq, a.var, s.scale);
        if (part) mask_tile<false>(sa, -INFINITY, route, causal, s.Skv, kj, km, i0 + qb * 32, hf, qma, qmb, qb * 32);
        var_softgrad(sa, pa, lse2s + qb * 32, deltas + qb * 32, a.var, hf);
        if (a.var.dbias != nullptr && kj < s.Skv) var_store_dx<T>(pa, a.var, dcol, i0 + qb * 32, s.Sq, s.Skv, hf);
      } else {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + qb * 32 + 8 * grp + 4 * hf);
#pragma unroll
          for (int i = 0; i < 4; ++i) sa[4 * grp + i] = fast_exp2(fmaf(sa[4 * grp + i], c2, -l4[i]));
        }
        if (part) mask_tile<false>(sa, 0.f, route, causal, s.Skv, kj, km, i0 + qb * 32, hf, qma, qmb, qb * 32);
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(deltas + qb * 32 + 8 * grp + 4 * hf);
#pragma unroll
          for (int i = 0; i < 4; ++i) pa[4 * grp + i] = sa[4 * grp + i] * (pa[4 * grp + i] - d4[i]);
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        pf[s2] = E::cvt8(slots8(sa, s2));
        dsf[s2] = E::cvt8(slots8(pa, s2));
      }
    };
    // dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by transpose reads).
    auto dvdk = [&](int qb, const F8* pf, const F8* dsf) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
          dva[d] = mma(frag_tr<T, DV>(dOs, d * 32, qb * 32 + 16 * s2, lane), pf[s2], dva[d]);
#pragma unroll
        for (int d = 0; d < DQK / 32; ++d)
          dka[d] = mma(frag_tr<T, DQK>(Qs, d * 32, qb * 32 + 16 * s2, lane), dsf[s2], dka[d]);
      }
    };

    f32x16 s0, p0;
    F8 pf0[2], dsf0[2];
    BiasTile<T> b0;
    sdp(0, s0, p0, b0);
    if constexpr (NQB == 2) {
      f32x16 s1, p1;
      F8 pf1[2], dsf1[2];
      BiasTile<T> b1;
      sdp(1, s1, p1, b1);
      softgrad(0, s0, p0, b0, pf0, dsf0);
      dvdk(0, pf0, dsf0);
      softgrad(1, s1, p1, b1, pf1, dsf1);
      dvdk(1, pf1, dsf1);
    } else {
      softgrad(0, s0, p0, b0, pf0, dsf0);
      dvdk(0, pf0, dsf0);
    }
  };

  // Loads in flight per thread after a direct issue (the side row load is
  // left out: waiting for one op fewer than issued still covers it, since
  // it is the youngest).
  constexpr int kBatch = TileLoad<T, BM, DQK, 256>::PER + TileLoad<T, BM, DV, 256>::PER;
  int cls;
  int x = next_step(0, cls);
  if constexpr (C::NBUF == 3) {
    int ncls;
    const int nx = next_step(x + 1, ncls);
    if (x < nsteps) issue(x, smem);
    if (nx < nsteps) issue(nx, smem + C::STAGE_BYTES);
    wait_vm();
    __syncthreads();
    int bi = 0;        // buffer of step x
    int nnx = nx, nncls = ncls;
    while (x < nsteps) {
      char* cur = smem + bi * C::STAGE_BYTES;
      compute(cur, x, cls == kTilePart);
      // Step after next into the buffer read in the previous step.
      int n2cls;
      const int n2 = nnx < nsteps ? next_step(nnx + 1, n2cls) : nsteps;
      bool inflight = false;
      if (n2 < nsteps) inflight = issue(n2, smem + (bi == 0 ? 2 : bi - 1) * C::STAGE_BYTES);
      if (inflight) wait_vm_keep<kBatch>();
      else wait_vm();
      __syncthreads();
      bi = bi == 2 ? 0 : bi + 1;
      x = nnx;
      cls = nncls;
      nnx = n2;
      nncls = n2cls;
    }
  } else {
    if (x < nsteps) issue(x, smem);
    wait_vm();
    __syncthreads();
    while (x < nsteps) {
      int ncls;
      const int nx = next_step(x + 1, ncls);
      compute(smem, x, cls == kTilePart);
      __syncthreads();
      if (nx < nsteps) issue(nx, smem);
      wait_vm();
      __syncthreads();
      x = nx;
      cls = ncls;
    }
  }

  if (kj < s.Skv) {
    T* dkp = static_cast<T*>(a.dk) + b * a.sk.b + kj * a.sk.t + hkv * a.sk.h;
    T* dvp = static_cast<T*>(a.dv) + b * a.sv.b + kj * a.sv.t + hkv * a.sv.h;
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 v = f32x4{dka[d][4 * grp], dka[d][4 * grp + 1], dka[d][4 * grp + 2], dka[d][4 * grp + 3]} * s.scale;
        *reinterpret_cast<typename E::P4*>(dkp + d * 32 + 8 * grp + 4 * hf) = E::cvt4(v);
      }
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 v = f32x4{dva[d][4 * grp], dva[d][4 * grp + 1], dva[d][4 * grp + 2], dva[d][4 * grp + 3]};
        *reinterpret_cast<typename E::P4*>(dvp + d * 32 + 8 * grp + 4 * hf) = E::cvt4(v);
      }
  }
}

// ------------------------------------------------------------ backward: dK, dV, warp-specialized

// bf16 with head dims up to 128: eight waves, two per SIMD.  Waves 0-3
// (producers) each own 32 keys: they hold the K and V fragments, compute S
// and dP for 32 queries, turn them into P and dS (bf16) and pass those
// through LDS.  Waves 4-7 (consumers) own the same 32 keys: they hold the dK
// and dV accumulators and run the dV += dO^T P and dK += Q^T dS products one
// 32-query phase behind.  Producer and consumer of a key block share a SIMD,
// so the producers' softmax-gradient VALU work overlaps the consumers'
// matrix work, and each role fits half the register file.  The query tiles
// are walked and classified exactly as in the kernel above, and every dK/dV
// element is still written once, at the end, by its consumer wave.
//
// DQP (the fused backward, for bf16 with Dqk <= 128): the producers also
// store dS of each phase transposed, as a [128 keys x 32 queries] bf16 tile,
// and each consumer wave then forms one 32-column block of the phase's dQ
// partial, dS (32 x 128) times K (128 keys x 32 columns, held in registers),
// and writes it to the dqp workspace.  No dQ value depends on the order in
// which workgroups run: each partial is written by one wave, and the dQ
// phase adds them up in ascending key-tile order.
template <typename T, int DQK, int DV, bool DQP = false>
struct DkvWsCfg {
  static constexpr int BN = 128;   // keys per workgroup: 4 key blocks of 32
  static constexpr int BM = 64;    // queries per step: 2 phases of 32
  static constexpr int THREADS = 512;
  static constexpr int Q_BYTES = BM * DQK * (int)sizeof(T);
  static constexpr int DO_BYTES = BM * DV * (int)sizeof(T);
  static constexpr int SIDE_BYTES = BM * 4 * 4;
  static constexpr int STAGE_BYTES = Q_BYTES + DO_BYTES + SIDE_BYTES;
  static constexpr int XSLOT_BYTES = 4 * 4 * 64 * 16;   // 4 key blocks x (P, P, dS, dS) x 64 lanes x 16 B
  static constexpr int DST_BYTES = DQP ? BN * 32 * (int)sizeof(T) : 0;   // dS^T tile of one phase
  static constexpr int LDS_BYTES = 3 * STAGE_BYTES + 2 * XSLOT_BYTES + 2 * DST_BYTES;
  static constexpr bool ENABLED = sizeof(T) == 2 && DQK <= 192 && DV <= 128 && LDS_BYTES <= 160 * 1024 &&
                                  (!DQP || DQK <= 128);
  static constexpr int PART = 32 * DQK;   // floats of one dQ partial (32 queries x Dqk)
};

template <typename T, int DQK, int DV, bool VAR, bool DQP = false, bool SPLIT = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
    attn_bwd_dkdv_ws_kernel(BwdArgs a) {
  using C = DkvWsCfg<T, DQK, DV, DQP>;
  static_assert(!DQP || (!VAR && C::ENABLED), "the fused backward has no variant kernels");
  using E = Elem<T>;
  using F8 = typename E::F8;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  char* xch = smem + 3 * C::STAGE_BYTES;
  char* dsx = xch + 2 * C::XSLOT_BYTES;   // DQP: dS^T tiles of the two exchange slots

  const AttnShape& s = a.s;
  const bool causal = s.causal != 0;
  const int n_kt = (s.Skv + BN - 1) / BN;
  const int g = s.Hq / s.Hkv;
  const int nsplit = SPLIT ? a.kv_split : 1;   // a separate instance, so the unsplit code stays lean
  const int nblocks = s.B * s.Hkv * n_kt * nsplit;
  int L = logical_block(nblocks, s.reverse);
  const int split = L % nsplit;
  L /= nsplit;
  const int rank = L % n_kt;
  L /= n_kt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  // The key tile.  Only the split instance takes the longest-walk-first
  // order: the unsplit one keeps the fixed order, whose tile index the
  // compiler recomputes from the block index instead of holding it (a loaded
  // index costs it SGPR spill reloads, measured 3 % slower on packed 8K).
  const int krank = SPLIT ? k_tile_of(a.seg, b, rank, n_kt) : rank;
  const int k0 = krank * BN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool producer = wave < 4;
  const int kb = wave & 3;                 // key block of this wave
  const int ptid = tid & 255;              // thread index among producers (loads)
  const int kj = k0 + kb * 32 + n;

  const int route = s.has_meta ? a.seg.route[b] : kRouteDense;
  const bool general = route == kRouteGeneral;
  TileSum ks{};
  const ChunkSum* sum_q_row = nullptr;
  if (route != kRouteDense) {
    ks = tile_sum(a.seg.sum_kv + (size_t)b * a.seg.nch_kv, a.seg.nch_kv, k0, BN);
    sum_q_row = a.seg.sum_q + (size_t)b * a.seg.nch_q;
  }
  int lo, hi;
  q_range(route, causal, s.Sq, k0, BN, ks, lo, hi);
  const int t_hi = (hi + BM - 1) / BM;
  const int ntiles = t_hi - lo / BM;
  // This workgroup's part of the walk: tiles [u0, u1) in walk order, steps
  // [x0, nsteps) (all of it unless the walk is split).
  const int u0 = split * ntiles / nsplit, u1 = (split + 1) * ntiles / nsplit;
  const int x0 = g * u0;
  const int nsteps = g * u1;
  auto tile_of = [&](int x) { return t_hi - 1 - x / g; };
  auto classify = [&](int qt) -> int {
    TileSum qs{};
    if (route != kRouteDense) qs = tile_sum(sum_q_row, a.seg.nch_q, qt * BM, BM);
    return classify_tile(route, causal, s.Skv, qt * BM, BM, k0, BN, qs, ks);
  };
  __shared__ unsigned char cls_tab[kClassCap];
  const bool tabled = route != kRouteDense;
  if (tabled) {
    fill_classes(cls_tab, ntiles, tid, C::THREADS, [&](int u) { return classify(t_hi - 1 - u); });
    __syncthreads();
  }
  auto next_step = [&](int x, int& cls) -> int {
    while (x < nsteps) {
      const int u = x / g;
      cls = (tabled && u < kClassCap) ? (int)cls_tab[u] : classify(tile_of(x));
      if (cls != kTileSkip) return x;
      x = (u + 1) * g;
    }
    cls = kTileSkip;
    return nsteps;
  };

  // Producer loads of one step (Q, dO, side rows) into a stage buffer;
  // returns whether they are still in flight.
  auto issue = [&](int x, char* st) -> bool {
    T* Qs = reinterpret_cast<T*>(st);
    T* dOs = Qs + BM * DQK;
    float* side = reinterpret_cast<float*>(dOs + BM * DV);
    const int h = hkv * g + x % g;
    const int i0 = tile_of(x) * BM;
    const int nvalid = min(BM, s.Sq - i0);
    const T* qg = static_cast<const T*>(a.q) + b * a.sq.b + h * a.sq.h + i0 * a.sq.t;
    const T* dg = static_cast<const T*>(a.dout) + b * a.so.b + h * a.so.h + i0 * a.so.t;
    const size_t rowx = ((size_t)b * s.Hq + h) * s.Sq + i0;
    const size_t rowm = (size_t)b * s.Sq + i0;
    if (nvalid == BM) {
      TileLoad<T, BM, DQK, 256>::direct(qg, a.sq.t, Qs, ptid);
      TileLoad<T, BM, DV, 256>::direct(dg, a.so.t, dOs, ptid);
      const int* src;
      if (wave == 0) src = reinterpret_cast<const int*>(a.lse2 + rowx) + lane;
      else if (wave == 1) src = reinterpret_cast<const int*>(a.delta + rowx) + lane;
      else if (route == kRouteFast) src = reinterpret_cast<const int*>(a.seg.run_q + rowm + lane) + (wave - 2);
      else if (route == kRouteGeneral) src = (wave == 2 ? a.seg.ids_q : a.seg.pos_q) + rowm + lane;
      else src = nullptr;
      if (src) __builtin_amdgcn_global_load_lds(src, (BPS_LDS void*)(side + wave * BM), 4, 0, 0);
      return true;
    }
    TileLoad<T, BM, DQK, 256>::staged(qg, a.sq.t, nvalid, Qs, ptid);
    TileLoad<T, BM, DV, 256>::staged(dg, a.so.t, nvalid, dOs, ptid);
    const bool in = lane < nvalid;
    if (wave == 0) {
      side[lane] = in ? a.lse2[rowx + lane] : INFINITY;
    } else if (wave == 1) {
      side[BM + lane] = in ? a.delta[rowx + lane] : 0.f;
    } else {
      const TokMeta t = in ? q_meta(route, a.seg, b, s.Sq, i0 + lane) : TokMeta{0, 0};
      reinterpret_cast<int*>(side)[wave * BM + lane] = wave == 2 ? t.a : t.b;
    }
    return false;
  };
  auto xfrag = [&](int slot, int f) {
    return reinterpret_cast<F8*>(xch + slot * C::XSLOT_BYTES) + ((kb * 4 + f) * 64 + lane);
  };

  const float c2 = s.scale_log2;
  F8 kf[DQK / 16];
  F8 vf[DV / 16];
  TokMeta km{0, 0};
  f32x16 dka[DQK / 32];
  f32x16 dva[DV / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dka[d] = f32x16{};
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) dva[d] = f32x16{};
  if (producer) {
    const T* kp = static_cast<const T*>(a.k) + b * a.sk.b + hkv * a.sk.h;
    const T* vp = static_cast<const T*>(a.v) + b * a.sv.b + hkv * a.sv.h;
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t)
      kf[t] = kj < s.Skv ? E::load8(kp + kj * a.sk.t + 16 * t + 8 * hf) : E::zero8();
#pragma unroll
    for (int t = 0; t < DV / 16; ++t)
      vf[t] = kj < s.Skv ? E::load8(vp + kj * a.sv.t + 16 * t + 8 * hf) : E::zero8();
    if (general) km = kv_meta(route, a.seg, b, s.Skv, kj);
  }
  // DQP: consumer wave kb's B operands of dQ = dS K, column block kb: for
  // keys k0 + 16 t + cmap(hf, e), column 32 kb + n (the key order of the
  // transposed dS^T reads).
  constexpr int NKT = DQP ? BN / 16 : 1;
  F8 kq[NKT];
  const bool dq_wave = DQP && !producer && kb < DQK / 32;
  if constexpr (DQP) {
    if (dq_wave) {
      const T* kp = static_cast<const T*>(a.k) + b * a.sk.b + hkv * a.sk.h + 32 * kb + n;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = k0 + 16 * t + 8 * (e >> 2) + 4 * hf + (e & 3);
          kq[t][e] = key < s.Skv ? kp[(int64_t)key * a.sk.t] : T(0.f);
        }
    }
  }

  // Producer phase: S, dP for queries qb*32.. of step x, then P and dS (bf16)
  // into exchange slot `slot`.
  auto produce = [&](const char* st, int x, int qb, bool part, int slot) {
    const T* Qs = reinterpret_cast<const T*>(st);
    const T* dOs = Qs + BM * DQK;
    const float* lse2s = reinterpret_cast<const float*>(dOs + BM * DV);
    const float* deltas = lse2s + BM;
    const int* qma = reinterpret_cast<const int*>(lse2s + 2 * BM);
    const int* qmb = qma + BM;
    // Variants: this phase's bias goes in flight before the products.
    int ib = 0;
    size_t col = 0;
    BiasTile<T> bq;
    if constexpr (VAR) {
      ib = tile_of(x) * BM + qb * 32;
      col = (size_t)(hkv * g + x % g) * s.Sq * s.Skv + kj;
      const T* bcol = (a.var.bias != nullptr && kj < s.Skv)
                          ? static_cast<const T*>(a.var.bias) + b * a.var.bias_b + col : nullptr;
      bq = bias_queries<T>(bcol, ib, s.Sq, s.Skv, hf);
    }
    F8 qa[DQK / 16], da[DV / 16];
    f32x16 sa = f32x16{}, pa = f32x16{};
    // Plain instance: exponentials of S taken with the dP products, and
    // (Dqk <= 128) Delta read during them.
    constexpr bool PRE = !VAR && !DQP;
    constexpr bool PRE_DELTA = PRE && DQK <= 128;
    f32x4 dl[4];
    if constexpr (PRE) {
      // Every Q fragment of S is read before the first product, so the S
      // chain runs back to back instead of waiting one LDS round trip per
      // product; the dO fragments and LSE values are read between the S
      // products, the exponentials of S run between the dP products, and
      // (Dqk <= 128) the Delta values are read with them: read after the
      // products, they cost two LDS round trips at the end of every phase
      // (same host: dK/dV 2.48-2.50 against 2.62-2.67 ms on the 8K causal
      // GQA workload; with Dqk = 192 it was 5 % slower, so that keeps the
      // late reads).
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) qa[t] = frag_row<T, DQK>(Qs, qb * 32 + n, 16 * t + 8 * hf);
      __builtin_amdgcn_sched_group_barrier(0x100, DQK / 16, 0);
      f32x4 l4[4];
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) {
        sa = mma(qa[t], kf[t], sa);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (t < DV / 16) {
          da[t] = frag_row<T, DV>(dOs, qb * 32 + n, 16 * t + 8 * hf);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (t >= DQK / 16 - 4) {
          const int grp = t - (DQK / 16 - 4);
          l4[grp] = *reinterpret_cast<const f32x4*>(lse2s + qb * 32 + 8 * grp + 4 * hf);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
#pragma unroll
      for (int t = DQK / 16; t < DV / 16; ++t) da[t] = frag_row<T, DV>(dOs, qb * 32 + n, 16 * t + 8 * hf);
      // The S and dP chains are scheduled apart, so that the Delta reads
      // below cannot take the place of the Q fragment reads ahead of S.
      if constexpr (PRE_DELTA) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < DV / 16; ++t) {
        pa = mma(da[t], vf[t], pa);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (PRE_DELTA) {
          if (t < 4) {
            dl[t] = *reinterpret_cast<const f32x4*>(deltas + qb * 32 + 8 * t + 4 * hf);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
#pragma unroll
        for (int grp = t * 4 / (DV / 16); grp < (t + 1) * 4 / (DV / 16); ++grp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sa[4 * grp + i] = fast_exp2(fmaf(sa[4 * grp + i], c2, -l4[grp][i]));
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) qa[t] = frag_row<T, DQK>(Qs, qb * 32 + n, 16 * t + 8 * hf);
#pragma unroll
      for (int t = 0; t < DV / 16; ++t) da[t] = frag_row<T, DV>(dOs, qb * 32 + n, 16 * t + 8 * hf);
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) sa = mma(qa[t], kf[t], sa);
#pragma unroll
      for (int t = 0; t < DV / 16; ++t) pa = mma(da[t], vf[t], pa);
    }
    if constexpr (VAR) {
      // Variant logits, masked to -inf, then P and dLoss/dx = P (dP - Delta)
      // dS/dx in one pass; dx also goes to the dbias target.
      var_logits<T>(sa, bq, a.var, s.scale);
      if (part) mask_tile<false>(sa, -INFINITY, route, causal, s.Skv, kj, km, ib, hf, qma, qmb, qb * 32);
      var_softgrad(sa, pa, lse2s + qb * 32, deltas + qb * 32, a.var, hf);
      if (a.var.dbias != nullptr && kj < s.Skv) var_store_dx<T>(pa, a.var, b * a.var.dbias_b + col, ib, s.Sq, s.Skv, hf);
    } else {
      if constexpr (!PRE) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + qb * 32 + 8 * grp + 4 * hf);
#pragma unroll
          for (int i = 0; i < 4; ++i) sa[4 * grp + i] = fast_exp2(fmaf(sa[4 * grp + i], c2, -l4[i]));
        }
      }
      if (part) mask_tile<false>(sa, 0.f, route, causal, s.Skv, kj, km, tile_of(x) * BM + qb * 32, hf, qma, qmb, qb * 32);
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 d4;
        if constexpr (PRE_DELTA) d4 = dl[grp];
        else d4 = *reinterpret_cast<const f32x4*>(deltas + qb * 32 + 8 * grp + 4 * hf);
#pragma unroll
        for (int i = 0; i < 4; ++i) pa[4 * grp + i] = sa[4 * grp + i] * (pa[4 * grp + i] - d4[i]);
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      *xfrag(slot, s2) = E::cvt8(slots8(sa, s2));
      *xfrag(slot, 2 + s2) = E::cvt8(slots8(pa, s2));
    }
    if constexpr (DQP) {
      // dS^T[key kb * 32 + n][query rmap(hf, r)]: four runs of 4 queries.
      T* dst = reinterpret_cast<T*>(dsx + slot * C::DST_BYTES);
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        *reinterpret_cast<typename E::P4*>(dst + TileFmt<T, 32>::off(kb * 32 + n, 8 * grp + 4 * hf)) =
            E::cvt4(f32x4{pa[4 * grp], pa[4 * grp + 1], pa[4 * grp + 2], pa[4 * grp + 3]});
    }
  };
  // Consumer phase: dV^T += dO^T P, dK^T += Q^T dS for queries qb*32.. of
  // the stage (dO^T and Q^T by transpose reads).
  auto consume = [&](const char* st, int x, int qb, int slot) {
    const T* Qs = reinterpret_cast<const T*>(st);
    const T* dOs = Qs + BM * DQK;
    F8 pf[2], dsf[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      pf[s2] = *xfrag(slot, s2);
      dsf[s2] = *xfrag(slot, 2 + s2);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
        dva[d] = mma(frag_tr<T, DV>(dOs, d * 32, qb * 32 + 16 * s2, lane), pf[s2], dva[d]);
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d)
        dka[d] = mma(frag_tr<T, DQK>(Qs, d * 32, qb * 32 + 16 * s2, lane), dsf[s2], dka[d]);
    }
    if constexpr (DQP) {
      if (dq_wave) {
        // Partial of queries tile_of(x) * BM + qb * 32 .. + 31, columns
        // 32 kb .. + 31, over this workgroup's keys in ascending order.
        const T* dst = reinterpret_cast<const T*>(dsx + slot * C::DST_BYTES);
        f32x16 qacc = f32x16{};
#pragma unroll
        for (int t = 0; t < NKT; ++t) qacc = mma(frag_tr<T, 32>(dst, 0, 16 * t, lane), kq[t], qacc);
        const int h = hkv * g + x % g;
        const int nqb = 2 * ((s.Sq + BM - 1) / BM);
        const size_t part = (((size_t)b * s.Hq + h) * n_kt + krank) * nqb + tile_of(x) * 2 + qb;
        f32x4* out = reinterpret_cast<f32x4*>(a.dqp + part * C::PART + (size_t)(kb * 64 + lane) * 16);
#pragma unroll
        for (int grp = 0; grp < 4; ++grp)
          out[grp] = f32x4{qacc[4 * grp], qacc[4 * grp + 1], qacc[4 * grp + 2], qacc[4 * grp + 3]};
      }
    }
  };

  // Phase schedule, computed identically by both roles.  Step k (in walk
  // order, skipped tiles left out) lives in stage buffer k % 3 and takes two
  // phases (32 queries each).  In phase j the producers handle phase j and
  // the consumers phase j - 1; every wave passes one barrier per phase.  In
  // the second phase of step k the producers issue the loads of step k + 2
  // (into the buffer of step k - 1, which the consumers finished a phase
  // earlier) and wait for those of step k + 1.
  struct Sched {
    int x, cls, nx, ncls, buf, qb;
  };
  auto sched_init = [&]() {
    Sched t;
    t.x = next_step(x0, t.cls);
    t.nx = t.x < nsteps ? next_step(t.x + 1, t.ncls) : nsteps;
    t.buf = 0;
    t.qb = 0;
    return t;
  };
  auto sched_next = [&](Sched& t) {
    if (t.qb == 0) {
      t.qb = 1;
      return;
    }
    t.qb = 0;
    t.x = t.nx;
    t.cls = t.ncls;
    t.buf = t.buf == 2 ? 0 : t.buf + 1;
    t.nx = t.x < nsteps ? next_step(t.x + 1, t.ncls) : nsteps;
  };
  constexpr int kBatch = TileLoad<T, BM, DQK, 256>::PER + TileLoad<T, BM, DV, 256>::PER;

  if (producer) {
    // The producers' chain (products, exponentials, dS) is the critical path
    // of a phase; at a higher wave priority their instructions win issue
    // over the consumers' when both are ready on a SIMD (measured: 7-8 %
    // less time than equal priorities on the 8K causal GQA workload).
    __builtin_amdgcn_s_setprio(3);
    Sched t = sched_init();
    if (t.x < nsteps) issue(t.x, smem);
    if (t.nx < nsteps) issue(t.nx, smem + C::STAGE_BYTES);
    wait_vm();
    __syncthreads();
    int slot = 0;
    while (t.x < nsteps) {
      bool inflight = false;
      int n2 = nsteps, n2cls = kTileSkip;
      if (t.qb == 1 && t.nx < nsteps) {
        n2 = next_step(t.nx + 1, n2cls);
        if (n2 < nsteps) inflight = issue(n2, smem + (t.buf == 0 ? 2 : t.buf - 1) * C::STAGE_BYTES);
      }
      produce(smem + t.buf * C::STAGE_BYTES, t.x, t.qb, t.cls == kTilePart, slot);
      if (t.qb == 1) {       // step k + 1 must be in LDS before its first phase
        if (inflight) wait_vm_keep<kBatch>();
        else wait_vm();
      }
      __syncthreads();
      slot ^= 1;
      // Moving on to the next step, the step after it is the look-ahead of
      // this step's second phase, already worked out above (working it out
      // again here put one more walk-and-classify between every two steps:
      // same host, dK/dV 1.2 % slower on the 8K causal GQA workload and
      // 4 % on the cross workload).
      if (t.qb == 1) {
        t.qb = 0;
        t.x = t.nx;
        t.cls = t.ncls;
        t.buf = t.buf == 2 ? 0 : t.buf + 1;
        t.nx = n2;
        t.ncls = n2cls;
      } else {
        t.qb = 1;
      }
    }
    wait_vm();
    __syncthreads();   // the consumers' last phase
  } else {
    Sched t = sched_init();
    __syncthreads();   // prologue loads
    __syncthreads();   // phase 0: the producers' first phase
    int slot = 0;
    while (t.x < nsteps) {
      consume(smem + t.buf * C::STAGE_BYTES, t.x, t.qb, slot);
      __syncthreads();
      slot ^= 1;
      sched_next(t);
    }
  }

  if (SPLIT) {
    // fp32 partials, float4-index-major so that every store instruction
    // writes 1 KB of contiguous memory.
    if (!producer) {
      constexpr int NF4 = 4 * (DQK / 32 + DV / 32);
      f32x4* out = reinterpret_cast<f32x4*>(a.dkvp) +
                   (((((size_t)b * s.Hkv + hkv) * n_kt + krank) * nsplit + split) * 4 + kb) * NF4 * 64 + lane;
      int i = 0;
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp, ++i)
          out[i * 64] = f32x4{dka[d][4 * grp], dka[d][4 * grp + 1], dka[d][4 * grp + 2], dka[d][4 * grp + 3]};
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp, ++i)
          out[i * 64] = f32x4{dva[d][4 * grp], dva[d][4 * grp + 1], dva[d][4 * grp + 2], dva[d][4 * grp + 3]};
    }
  } else if (!producer && kj < s.Skv) {
    T* dkp = static_cast<T*>(a.dk) + b * a.sk.b + kj * a.sk.t + hkv * a.sk.h;
    T* dvp = static_cast<T*>(a.dv) + b * a.sv.b + kj * a.sv.t + hkv * a.sv.h;
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 v = f32x4{dka[d][4 * grp], dka[d][4 * grp + 1], dka[d][4 * grp + 2], dka[d][4 * grp + 3]} * s.scale;
        *reinterpret_cast<typename E::P4*>(dkp + d * 32 + 8 * grp + 4 * hf) = E::cvt4(v);
      }
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 v = f32x4{dva[d][4 * grp], dva[d][4 * grp + 1], dva[d][4 * grp + 2], dva[d][4 * grp + 3]};
        *reinterpret_cast<typename E::P4*>(dvp + d * 32 + 8 * grp + 4 * hf) = E::cvt4(v);
      }
  }
}

// ------------------------------------------------------------ backward: split dK/dV walks

// dK (times the softmax scale) and dV of one key tile from the kv_split
// partials of its split walk, added in split order.  One wave per 32-key
// block, each lane the C-layout values the consumer wave held; blockIdx.y
// picks 4 of the tile's float4 slots per lane, so that the grid has enough
// waves and each lane enough loads in flight (all splits' loads are issued
// first, at a clamped split index, and only the real ones are added).
constexpr int kReduceSlots = 4;   // float4 slots per lane and workgroup
constexpr int kReduceMaxSplit = 4;

template <int DQK, int DV>
constexpr int dkdv_reduce_chunks() {
  return 4 * (DQK / 32 + DV / 32) / kReduceSlots;
}

template <typename T, int DQK, int DV>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_reduce_kernel(BwdArgs a) {
  using E = Elem<T>;
  constexpr int BN = DkvWsCfg<T, DQK, DV>::BN;
  constexpr int NF4 = 4 * (DQK / 32 + DV / 32);
  static_assert(NF4 % kReduceSlots == 0, "slots split evenly");
  const AttnShape& s = a.s;
  const int nsplit = a.kv_split;
  const int n_kt = (s.Skv + BN - 1) / BN;
  int L = blockIdx.x;
  const int krank = L % n_kt;
  L /= n_kt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  const int kb = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int kj = krank * BN + kb * 32 + n;
  const int i0 = blockIdx.y * kReduceSlots;
  const size_t stride = (size_t)4 * NF4 * 64;   // between the partials of consecutive splits
  const f32x4* part = reinterpret_cast<const f32x4*>(a.dkvp) +
                      (((size_t)b * s.Hkv + hkv) * n_kt + krank) * nsplit * stride + (size_t)kb * NF4 * 64 + lane;
  if (kj >= s.Skv) return;
  f32x4 x[kReduceMaxSplit][kReduceSlots];
#pragma unroll
  for (int sp = 0; sp < kReduceMaxSplit; ++sp)
#pragma unroll
    for (int j = 0; j < kReduceSlots; ++j) x[sp][j] = part[(sp < nsplit ? sp : 0) * stride + (i0 + j) * 64];
  T* dkp = static_cast<T*>(a.dk) + b * a.sk.b + kj * a.sk.t + hkv * a.sk.h;
  T* dvp = static_cast<T*>(a.dv) + b * a.sv.b + kj * a.sv.t + hkv * a.sv.h;
#pragma unroll
  for (int j = 0; j < kReduceSlots; ++j) {
    f32x4 v = x[0][j];
#pragma unroll
    for (int sp = 1; sp < kReduceMaxSplit; ++sp)
      if (sp < nsplit) v += x[sp][j];
    const int i = i0 + j;
    const int d = (i >> 2) % (DQK / 32), grp = i & 3;
    if (i < 4 * (DQK / 32))
      *reinterpret_cast<typename E::P4*>(dkp + d * 32 + 8 * grp + 4 * hf) = E::cvt4(v * s.scale);
    else
      *reinterpret_cast<typename E::P4*>(dvp + ((i >> 2) - DQK / 32) * 32 + 8 * grp + 4 * hf) = E::cvt4(v);
  }
}

// ------------------------------------------------------------ backward: dQ of the fused pass

// dQ of one (batch row, query head, block of 32 queries) as the sum of the
// partials the fused dK/dV kernel wrote, over key tiles in ascending order,
// then times the softmax scale.  The key tiles that wrote a partial for the
// block are found with the same range and tile classification as that
// kernel's walk; a block no key tile visited gets dQ = 0.  One wave per
// 32-column block; each lane owns the 16 values of its C-layout slot.
template <typename T, int DQK>
__global__ void __launch_bounds__(2 * DQK) attn_bwd_dq_reduce_kernel(BwdArgs a) {
  using W = DkvWsCfg<T, DQK, 128, true>;
  constexpr int BM = W::BM, BN = W::BN;
  const AttnShape& s = a.s;
  const int nqb = 2 * ((s.Sq + BM - 1) / BM);
  const int n_kt = (s.Skv + BN - 1) / BN;
  int L = blockIdx.x;
  const int qblk = L % nqb;
  L /= nqb;
  const int h = L % s.Hq;
  const int b = L / s.Hq;
  const int qt = qblk >> 1;
  const int j = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool causal = s.causal != 0;

  const int route = s.has_meta ? a.seg.route[b] : kRouteDense;
  TileSum qs{};
  if (route != kRouteDense) qs = tile_sum(a.seg.sum_q + (size_t)b * a.seg.nch_q, a.seg.nch_q, qt * BM, BM);
  const float* part = a.dqp + (((size_t)b * s.Hq + h) * n_kt * nqb + qblk) * W::PART + (size_t)(j * 64 + lane) * 16;
  f32x16 acc = f32x16{};
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BN;
    TileSum ks{};
    if (route != kRouteDense) ks = tile_sum(a.seg.sum_kv + (size_t)b * a.seg.nch_kv, a.seg.nch_kv, k0, BN);
    int lo, hi;
    q_range(route, causal, s.Sq, k0, BN, ks, lo, hi);
    if (qt < lo / BM || qt >= (hi + BM - 1) / BM) continue;
    if (classify_tile(route, causal, s.Skv, qt * BM, BM, k0, BN, qs, ks) == kTileSkip) continue;
    const f32x4* p = reinterpret_cast<const f32x4*>(part + (size_t)kt * nqb * W::PART);
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 v = p[grp];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[4 * grp + i] += v[i];
    }
  }
  T* dq = static_cast<T*>(a.dq) + b * a.sq.b + h * a.sq.h + 32 * j + n;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = qblk * 32 + rmap(hf, r);
    if (i < s.Sq) dq[(int64_t)i * a.sq.t] = T(acc[r] * s.scale);
  }
}

}  // namespace bps

#include "dkdv_gs.hpp"
#include "fwd_pp.hpp"
#include "dq_hp.hpp"

namespace bps {

// ------------------------------------------------------------ launchers

// The gradient-split dK/dV kernel addresses Q and dO of one batch row with
// 32-bit buffer offsets: every byte of a row's tensor must lie within 2 GB
// of its start.
inline bool gs_offsets_fit(const BwdArgs& a, int dqk, int dv) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t q = ((int64_t)(a.s.Hq - 1) * a.sq.h + (int64_t)(a.s.Sq - 1) * a.sq.t + dqk) * 2;
  const int64_t o = ((int64_t)(a.s.Hq - 1) * a.so.h + (int64_t)(a.s.Sq - 1) * a.so.t + dv) * 2;
  return a.sq.h >= 0 && a.sq.t >= 0 && a.so.h >= 0 && a.so.t >= 0 && q < lim && o < lim;
}

template <typename T, int DQK, int DV, int VM>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  using C = FwdCfg<T, DQK, DV>;
  const int n_qt = (a.s.Sq + C::BM - 1) / C::BM;
  const long long nblocks = (long long)a.s.B * a.s.Hq * n_qt;
  if (nblocks <= 0) return hipSuccess;
  if constexpr (VM == 0 && FwdCfg<T, DQK, DV, 8>::WIDE_OK) {
    if ((a.s.Hq / a.s.Hkv) % 2 == 0) {   // head pairs of a GQA group
      if constexpr (sizeof(T) == 2 && FwdPpCfg<DQK, DV>::ENABLED) {
        if (fwd_pp_offsets_fit(a, DQK, DV)) {   // the two heads half a step apart
          using CP = FwdPpCfg<DQK, DV>;
          const long long nbp = (long long)a.s.B * (a.s.Hq / 2) * ((a.s.Sq + CP::BM - 1) / CP::BM);
          hipLaunchKernelGGL((attn_fwd_pp_kernel<DQK, DV>), dim3((unsigned)nbp), dim3(CP::THREADS), 0, st, a);
          return hipGetLastError();
        }
      }
      using C8 = FwdCfg<T, DQK, DV, 8, 2>;
      const long long nb8 = (long long)a.s.B * (a.s.Hq / 2) * ((a.s.Sq + C8::BM - 1) / C8::BM);
      hipLaunchKernelGGL((attn_fwd_kernel<T, DQK, DV, 0, 8, 2>), dim3((unsigned)nb8), dim3(C8::THREADS), 0, st, a);
      return hipGetLastError();
    }
    if (!a.s.has_meta && !a.s.causal) {
      using C8 = FwdCfg<T, DQK, DV, 8>;
      const long long nb8 = (long long)a.s.B * a.s.Hq * ((a.s.Sq + C8::BM - 1) / C8::BM);
      hipLaunchKernelGGL((attn_fwd_kernel<T, DQK, DV, 0, 8>), dim3((unsigned)nb8), dim3(C8::THREADS), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_fwd_kernel<T, DQK, DV, VM>), dim3((unsigned)nblocks), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

template <typename T, int DQK, int DV, bool VAR>
hipError_t launch_bwd_delta(const BwdArgs& a, hipStream_t st) {
  const size_t rows = (size_t)a.s.B * a.s.Sq * a.s.Hq;
  if (rows == 0) return hipSuccess;
  const size_t blocks = (rows * 8 + 255) / 256;
  hipLaunchKernelGGL((attn_bwd_delta_kernel<T, DV, VAR>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The fused backward (a.dqp set) is built for bf16 with Dqk, Dv <= 128 and
// no bias or soft cap; the host checks this before any launch.
template <typename T, int DQK, int DV>
constexpr bool kFusedBwd = sizeof(T) == 2 && DQK <= 128 && DV <= 128 &&
                           DkvWsCfg<T, DQK, DV, true>::ENABLED;

template <typename T, int DQK, int DV, bool VAR>
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t st) {
  const int n_kt = (a.s.Skv + DkvCfg<T, DQK, DV>::BN - 1) / DkvCfg<T, DQK, DV>::BN;
  const long long nblocks = (long long)a.s.B * a.s.Hkv * n_kt;
  if (nblocks <= 0) return hipSuccess;
  if (a.kv_split < 1 || a.kv_split > kReduceMaxSplit ||
      (a.kv_split > 1 && (!DkvWsCfg<T, DQK, DV>::ENABLED || a.dkvp == nullptr)))
    return hipErrorInvalidValue;
  const unsigned nws = (unsigned)(nblocks * a.kv_split);
  const bool split = a.kv_split > 1;
  if (a.dqp != nullptr) {
    if constexpr (!VAR && kFusedBwd<T, DQK, DV>) {
      static_assert(DkvWsCfg<T, DQK, DV, true>::BN == DkvCfg<T, DQK, DV>::BN, "same key tiling");
      if (split)
        hipLaunchKernelGGL((attn_bwd_dkdv_ws_kernel<T, DQK, DV, false, true, true>), dim3(nws), dim3(512), 0, st, a);
      else
        hipLaunchKernelGGL((attn_bwd_dkdv_ws_kernel<T, DQK, DV, false, true>), dim3(nws), dim3(512), 0, st, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else if constexpr (DkvWsCfg<T, DQK, DV>::ENABLED) {
    static_assert(DkvWsCfg<T, DQK, DV>::BN == DkvCfg<T, DQK, DV>::BN, "same key tiling");
    if constexpr (!VAR && sizeof(T) == 2 && DkvGsCfg<DQK, DV>::ENABLED) {
      // Gradient-split kernel for GQA groups (same-host A/B, dK/dV: 2.46 against
      // 2.52-2.55 ms on the 8K causal GQA workload; without a group to walk it
      // was slower: 0.163 against 0.155 ms on BSHD 2K, 65.0 against 62.2 ms on
      // the 18,900 x 75,600 shard, and no faster on packed 8K).
      static_assert(DkvGsCfg<DQK, DV>::BN == DkvCfg<T, DQK, DV>::BN, "same key tiling");
      if (!split && a.s.Hq / a.s.Hkv >= 2 && gs_offsets_fit(a, DQK, DV)) {
        hipLaunchKernelGGL((attn_bwd_dkdv_gs_kernel<DQK, DV>), dim3(nws), dim3(512), 0, st, a);
        return hipGetLastError();
      }
    }
    if (split)
      hipLaunchKernelGGL((attn_bwd_dkdv_ws_kernel<T, DQK, DV, VAR, false, true>), dim3(nws), dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_ws_kernel<T, DQK, DV, VAR>), dim3(nws), dim3(512), 0, st, a);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DQK, DV, VAR>), dim3((unsigned)nblocks), dim3(256), 0, st, a);
  }
  if constexpr (DkvWsCfg<T, DQK, DV>::ENABLED) {
    if (a.kv_split > 1) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_bwd_dkdv_reduce_kernel<T, DQK, DV>),
                         dim3((unsigned)nblocks, (unsigned)dkdv_reduce_chunks<DQK, DV>()), dim3(256), 0, st, a);
    }
  }
  return hipGetLastError();
}

template <typename T, int DQK, int DV, bool VAR>
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st) {
  if (a.dqp != nullptr) {
    if constexpr (!VAR && kFusedBwd<T, DQK, DV>) {
      const long long nb = (long long)a.s.B * a.s.Hq * 2 * ((a.s.Sq + 63) / 64);
      if (nb <= 0) return hipSuccess;
      hipLaunchKernelGGL((attn_bwd_dq_reduce_kernel<T, DQK>), dim3((unsigned)nb), dim3(2 * DQK), 0, st, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  const int n_qt = (a.s.Sq + DqCfg<T, DQK, DV>::BM - 1) / DqCfg<T, DQK, DV>::BM;
  const long long nblocks = (long long)a.s.B * a.s.Hq * n_qt;
  if (nblocks <= 0) return hipSuccess;
  if constexpr (!VAR && DqCfg<T, DQK, DV, 8>::WIDE_OK) {
    if ((a.s.Hq / a.s.Hkv) % 2 == 0) {   // head pairs of a GQA group
      if constexpr (sizeof(T) == 2 && DqHpCfg<DQK, DV>::ENABLED) {
        const int64_t lim = (int64_t)1 << 31;
        if (a.sk.t >= 0 && a.sv.t >= 0 && ((int64_t)(a.s.Skv - 1) * a.sk.t + DQK) * 2 < lim &&
            ((int64_t)(a.s.Skv - 1) * a.sv.t + DV) * 2 < lim) {   // rotated blocks, three stages
          using CP = DqHpCfg<DQK, DV>;
          const long long nbp = (long long)a.s.B * (a.s.Hq / 2) * ((a.s.Sq + CP::BM - 1) / CP::BM);
          hipLaunchKernelGGL((attn_bwd_dq_hp_kernel<DQK, DV>), dim3((unsigned)nbp), dim3(CP::THREADS), 0, st, a);
          return hipGetLastError();
        }
      }
      using C8 = DqCfg<T, DQK, DV, 8, 2>;
      const long long nb8 = (long long)a.s.B * (a.s.Hq / 2) * ((a.s.Sq + C8::BM - 1) / C8::BM);
      hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DQK, DV, false, 8, 2>), dim3((unsigned)nb8), dim3(C8::THREADS), 0, st,
                         a);
      return hipGetLastError();
    }
    if (!a.s.has_meta && !a.s.causal) {
      using C8 = DqCfg<T, DQK, DV, 8>;
      const long long nb8 = (long long)a.s.B * a.s.Hq * ((a.s.Sq + C8::BM - 1) / C8::BM);
      hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DQK, DV, false, 8>), dim3((unsigned)nb8), dim3(C8::THREADS), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DQK, DV, VAR>), dim3((unsigned)nblocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace bps
