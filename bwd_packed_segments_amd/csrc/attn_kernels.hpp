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

#include "bps_args.hpp"

namespace bps {

// ------------------------------------------------------------ tile staging

// Loads a [ROWS x D] tile (rows past nvalid read as zero) with consecutive
// threads along a row, and stores it row-major into LDS.
template <typename T, int ROWS, int D, int THREADS>
struct RowTile {
  using E = Elem<T>;
  using F8 = typename E::F8;
  static constexpr int UNITS = ROWS * (D / 8);
  static constexpr int PER = UNITS / THREADS;
  static_assert(UNITS % THREADS == 0, "tile must split evenly over the workgroup");
  F8 r[PER];

  __device__ void load(const T* base, int64_t row_stride, int nvalid, int tid) {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int u = tid + x * THREADS;
      const int row = u / (D / 8);
      const int c8 = u % (D / 8);
      r[x] = row < nvalid ? E::load8(base + row * row_stride + c8 * 8) : E::zero8();
    }
  }
  __device__ void store(T* lds, int stride, int tid) const {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int u = tid + x * THREADS;
      const int row = u / (D / 8);
      const int c8 = u % (D / 8);
      *reinterpret_cast<F8*>(lds + row * stride + c8 * 8) = r[x];
    }
  }
};

// Loads a [ROWS x D] tile as row pairs so that it can also be stored
// transposed: T[d][perm(row)], where perm swaps bits 2 and 3 of the row
// index inside every group of 16 (the order the MFMA operands want).
template <typename T, int ROWS, int D, int THREADS>
struct PairTile {
  using E = Elem<T>;
  using F8 = typename E::F8;
  using P2 = typename E::P2;
  static constexpr int PAIRS = ROWS / 2;
  static constexpr int UNITS = PAIRS * (D / 8);
  static constexpr int PER = UNITS / THREADS;
  static_assert(UNITS % THREADS == 0, "tile must split evenly over the workgroup");
  static_assert(THREADS % PAIRS == 0, "row pairs must tile the workgroup");
  F8 r0[PER], r1[PER];

  __device__ static void unit(int u, int& pr, int& c8) {
    pr = u % PAIRS;
    c8 = u / PAIRS;
  }
  __device__ void load(const T* base, int64_t row_stride, int nvalid, int tid) {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      int pr, c8;
      unit(tid + x * THREADS, pr, c8);
      const int row = 2 * pr;
      r0[x] = row < nvalid ? E::load8(base + row * row_stride + c8 * 8) : E::zero8();
      r1[x] = row + 1 < nvalid ? E::load8(base + (row + 1) * row_stride + c8 * 8) : E::zero8();
    }
  }
  __device__ void store_rows(T* lds, int stride, int tid) const {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      int pr, c8;
      unit(tid + x * THREADS, pr, c8);
      *reinterpret_cast<F8*>(lds + (2 * pr) * stride + c8 * 8) = r0[x];
      *reinterpret_cast<F8*>(lds + (2 * pr + 1) * stride + c8 * 8) = r1[x];
    }
  }
  __device__ void store_t(T* lds, int stride, int tid) const {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      int pr, c8;
      unit(tid + x * THREADS, pr, c8);
      const int row = 2 * pr;
      const int col = (row & ~15) | perm16(row & 15);
      T* dst = lds + (c8 * 8) * stride + col;
      *reinterpret_cast<P2*>(dst + 0 * stride) = E::template pair<0>(r0[x], r1[x]);
      *reinterpret_cast<P2*>(dst + 1 * stride) = E::template pair<1>(r0[x], r1[x]);
      *reinterpret_cast<P2*>(dst + 2 * stride) = E::template pair<2>(r0[x], r1[x]);
      *reinterpret_cast<P2*>(dst + 3 * stride) = E::template pair<3>(r0[x], r1[x]);
      *reinterpret_cast<P2*>(dst + 4 * stride) = E::template pair<4>(r0[x], r1[x]);
      *reinterpret_cast<P2*>(dst + 5 * stride) = E::template pair<5>(r0[x], r1[x]);
      *reinterpret_cast<P2*>(dst + 6 * stride) = E::template pair<6>(r0[x], r1[x]);
      *reinterpret_cast<P2*>(dst + 7 * stride) = E::template pair<7>(r0[x], r1[x]);
    }
  }
};

template <typename T>
__device__ inline typename Elem<T>::F8 lds8(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::F8*>(p);
}

// Key tiles a query tile visits: [lo, hi) in tokens, per route.
__device__ inline void kv_range(int route, bool causal, int Skv, int q0, int nq, const TileSum& qs, int& lo,
                                int& hi) {
  lo = 0;
  hi = Skv;
  if (route == kRouteDense) {
    if (causal) hi = min(hi, q0 + nq);
  } else if (route == kRouteFast) {
    if (qs.cnt == 0) {
      hi = 0;
    } else {
      lo = qs.smin;
      hi = min(hi, qs.emax);
      if (causal) hi = min(hi, q0 + nq);
    }
  }
  if (hi < lo) hi = lo;
}

// Query tiles a key tile is visited by: [lo, hi) in tokens, per route.
__device__ inline void q_range(int route, bool causal, int Sq, int k0, int nk, const TileSum& ks, int& lo,
                               int& hi) {
  lo = 0;
  hi = Sq;
  if (route == kRouteDense) {
    if (causal) lo = k0;
  } else if (route == kRouteFast) {
    if (ks.cnt == 0) {
      hi = 0;
    } else {
      lo = ks.smin;
      hi = min(hi, ks.emax);
      if (causal) lo = max(lo, k0);
    }
  }
  if (hi < lo) hi = lo;
}

// ------------------------------------------------------------ forward

template <typename T, int DQK, int DV>
struct FwdCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int THREADS = 256;
  static constexpr int NBUF = sizeof(T) == 2 ? 2 : 1;
  static constexpr int KSTR = DQK + 8;
  static constexpr int VTSTR = BN + 8;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int VT_ELEMS = DV * VTSTR;
  static constexpr int META_BYTES = 2 * BN * 4;
  static constexpr int STAGE_BYTES = (K_ELEMS + VT_ELEMS) * (int)sizeof(T) + META_BYTES;
  static constexpr int WAVES_PER_EU = (NBUF * STAGE_BYTES * 2 <= 160 * 1024) ? 2 : 1;
};

template <typename T, int DQK, int DV>
__global__ void __launch_bounds__(256)
    attn_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<T, DQK, DV>;
  using E = Elem<T>;
  using F8 = typename E::F8;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(16))) char smem[C::NBUF * C::STAGE_BYTES];

  const AttnShape& s = a.s;
  const bool causal = s.causal != 0;
  const int n_qt = (s.Sq + BM - 1) / BM;
  const int g = s.Hq / s.Hkv;
  const int nblocks = s.B * s.Hq * n_qt;
  int L = logical_block(nblocks, s.reverse);
  const int hg = L % g;
  L /= g;
  const int qrank = L % n_qt;
  L /= n_qt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  const int h = hkv * g + hg;
  const int qt = causal ? (n_qt - 1 - qrank) : qrank;
  const int q0 = qt * BM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int qi = q0 + wave * 32 + n;

  const T* qp = static_cast<const T*>(a.q) + b * a.sq.b + h * a.sq.h;
  const T* kp = static_cast<const T*>(a.k) + b * a.sk.b + hkv * a.sk.h;
  const T* vp = static_cast<const T*>(a.v) + b * a.sv.b + hkv * a.sv.h;

  F8 qf[DQK / 16];
#pragma unroll
  for (int t = 0; t < DQK / 16; ++t)
    qf[t] = qi < s.Sq ? E::load8(qp + qi * a.sq.t + 16 * t + 8 * hf) : E::zero8();

  const int route = s.has_meta ? a.seg.route[b] : kRouteDense;
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
  auto next_tile = [&](int kt, int& cls) -> int {
    for (int k = kt; k < t_hi; ++k) {
      cls = classify(k);
      if (cls != kTileSkip) return k;
    }
    cls = kTileSkip;
    return t_hi;
  };

  RowTile<T, BN, DQK, 256> kreg;
  PairTile<T, BN, DV, 256> vreg;
  const bool general = route == kRouteGeneral;
  int kid_r = 0, kpos_r = 0;
  auto load_tile = [&](int kt) {
    const int k0 = kt * BN;
    const int nvalid = min(BN, s.Skv - k0);
    kreg.load(kp + k0 * a.sk.t, a.sk.t, nvalid, tid);
    vreg.load(vp + k0 * a.sv.t, a.sv.t, nvalid, tid);
    if (general && tid < BN) {
      const int j = k0 + tid;
      kid_r = j < s.Skv ? a.seg.ids_kv[(size_t)b * s.Skv + j] : 0;
      kpos_r = j < s.Skv ? a.seg.pos_kv[(size_t)b * s.Skv + j] : 0;
    }
  };
  auto stage_ptr = [&](int buf) { return smem + buf * C::STAGE_BYTES; };
  auto store_tile = [&](int buf) {
    char* st = stage_ptr(buf);
    T* Ks = reinterpret_cast<T*>(st);
    T* VT = Ks + C::K_ELEMS;
    int* kid = reinterpret_cast<int*>(VT + C::VT_ELEMS);
    kreg.store(Ks, C::KSTR, tid);
    vreg.store_t(VT, C::VTSTR, tid);
    if (general && tid < BN) {
      kid[tid] = kid_r;
      kid[BN + tid] = kpos_r;
    }
  };

  const float c2 = s.scale_log2;
  float m = -INFINITY;
  float l = 0.f;
  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};

  int cls;
  int kt = next_tile(t_lo, cls);
  int buf = 0;
  if (kt < t_hi) {
    load_tile(kt);
    store_tile(0);
  }
  __syncthreads();

  while (kt < t_hi) {
    int ncls;
    const int nkt = next_tile(kt + 1, ncls);
    if (nkt < t_hi) load_tile(nkt);

    const char* st = stage_ptr(buf);
    const T* Ks = reinterpret_cast<const T*>(st);
    const T* VT = Ks + C::K_ELEMS;
    const int* kid = reinterpret_cast<const int*>(VT + C::VT_ELEMS);
    const int k0 = kt * BN;

    // S^T = K Q^T for the tile's 64 keys (two 32-key blocks).
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const F8 ka = lds8<T>(Ks + (blk * 32 + n) * C::KSTR + 16 * t + 8 * hf);
        sacc[blk] = mma(ka, qf[t], sacc[blk]);
      }
    }

    if (cls == kTilePart) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int kk = blk * 32 + 8 * grp + 4 * hf;
          i32x4 ids4 = i32x4{0, 0, 0, 0}, pos4 = i32x4{0, 0, 0, 0};
          if (general) {
            ids4 = *reinterpret_cast<const i32x4*>(kid + kk);
            pos4 = *reinterpret_cast<const i32x4*>(kid + BN + kk);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = k0 + kk + i;
            if (!allowed(route, causal, s.Skv, qi, j, qm, TokMeta{ids4[i], pos4[i]}))
              sacc[blk][4 * grp + i] = -INFINITY;
          }
        }
      }
    }

    // Online softmax: running max and sum per query (lane pair n, n + 32).
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
    mx = wave_xor32_max(mx);
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float mc = m_use * c2;
    const float alpha = fast_exp2((m - m_use) * c2);
    float rs = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[blk][r], c2, -mc));
        sacc[blk][r] = p;
        rs += p;
      }
    l = l * alpha + rs;
    m = m_new;
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;
    }

    // O^T += V^T P^T.
    F8 pf[2][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) pf[blk][s2] = E::cvt8(slots8(sacc[blk], s2));
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const F8 va = lds8<T>(VT + (d * 32 + n) * C::VTSTR + blk * 32 + 16 * s2 + 8 * hf);
          o[d] = mma(va, pf[blk][s2], o[d]);
        }
    }

    if (C::NBUF == 1) __syncthreads();
    if (nkt < t_hi) store_tile(C::NBUF == 2 ? buf ^ 1 : buf);
    __syncthreads();
    if (C::NBUF == 2) buf ^= 1;
    kt = nkt;
    cls = ncls;
  }

  // Epilogue: O = O^T / l, LSE = m * scale + ln(l); empty rows give O = 0,
  // LSE = -inf.
  const float lt = wave_xor32_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qi < s.Sq) {
    T* op = static_cast<T*>(a.o) + b * a.so.b + qi * a.so.t + h * a.so.h;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 x = f32x4{o[d][4 * grp], o[d][4 * grp + 1], o[d][4 * grp + 2], o[d][4 * grp + 3]} * inv;
        *reinterpret_cast<typename E::P4*>(op + d * 32 + 8 * grp + 4 * hf) = E::cvt4(x);
      }
    if (hf == 0)
      a.lse[((size_t)b * s.Hq + h) * s.Sq + qi] = lt > 0.f ? m * s.scale + logf(lt) : -INFINITY;
  }
}

// ------------------------------------------------------------ backward: Delta

template <typename T, int DV>
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
    a.lse2[x] = lse == -INFINITY ? INFINITY : lse * kLog2e;
  }
}

// ------------------------------------------------------------ backward: dQ

template <typename T, int DQK, int DV>
struct DqCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int KSTR = DQK + 8;
  static constexpr int KTSTR = BN + 8;
  static constexpr int VSTR = DV + 8;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int KT_ELEMS = DQK * KTSTR;
  static constexpr int V_ELEMS = BN * VSTR;
  static constexpr int META_BYTES = 2 * BN * 4;
  static constexpr int STAGE_BYTES = (K_ELEMS + KT_ELEMS + V_ELEMS) * (int)sizeof(T) + META_BYTES;
  static constexpr int NBUF = (2 * STAGE_BYTES <= 160 * 1024) ? 2 : 1;
};

template <typename T, int DQK, int DV>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<T, DQK, DV>;
  using E = Elem<T>;
  using F8 = typename E::F8;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(16))) char smem[C::NBUF * C::STAGE_BYTES];

  const AttnShape& s = a.s;
  const bool causal = s.causal != 0;
  const int n_qt = (s.Sq + BM - 1) / BM;
  const int g = s.Hq / s.Hkv;
  const int nblocks = s.B * s.Hq * n_qt;
  int L = logical_block(nblocks, s.reverse);
  const int hg = L % g;
  L /= g;
  const int qrank = L % n_qt;
  L /= n_qt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  const int h = hkv * g + hg;
  const int qt = causal ? (n_qt - 1 - qrank) : qrank;
  const int q0 = qt * BM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int qi = q0 + wave * 32 + n;

  const T* qp = static_cast<const T*>(a.q) + b * a.sq.b + h * a.sq.h;
  const T* dop = static_cast<const T*>(a.dout) + b * a.so.b + h * a.so.h;
  const T* kp = static_cast<const T*>(a.k) + b * a.sk.b + hkv * a.sk.h;
  const T* vp = static_cast<const T*>(a.v) + b * a.sv.b + hkv * a.sv.h;

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
  auto next_tile = [&](int kt, int& cls) -> int {
    for (int k = kt; k < t_hi; ++k) {
      cls = classify(k);
      if (cls != kTileSkip) return k;
    }
    cls = kTileSkip;
    return t_hi;
  };

  PairTile<T, BN, DQK, 256> kreg;
  RowTile<T, BN, DV, 256> vreg;
  const bool general = route == kRouteGeneral;
  int kid_r = 0, kpos_r = 0;
  auto load_tile = [&](int kt) {
    const int k0 = kt * BN;
    const int nvalid = min(BN, s.Skv - k0);
    kreg.load(kp + k0 * a.sk.t, a.sk.t, nvalid, tid);
    vreg.load(vp + k0 * a.sv.t, a.sv.t, nvalid, tid);
    if (general && tid < BN) {
      const int j = k0 + tid;
      kid_r = j < s.Skv ? a.seg.ids_kv[(size_t)b * s.Skv + j] : 0;
      kpos_r = j < s.Skv ? a.seg.pos_kv[(size_t)b * s.Skv + j] : 0;
    }
  };
  auto stage_ptr = [&](int buf) { return smem + buf * C::STAGE_BYTES; };
  auto store_tile = [&](int buf) {
    char* st = stage_ptr(buf);
    T* Ks = reinterpret_cast<T*>(st);
    T* KT = Ks + C::K_ELEMS;
    T* Vs = KT + C::KT_ELEMS;
    int* kid = reinterpret_cast<int*>(Vs + C::V_ELEMS);
    kreg.store_rows(Ks, C::KSTR, tid);
    kreg.store_t(KT, C::KTSTR, tid);
    vreg.store(Vs, C::VSTR, tid);
    if (general && tid < BN) {
      kid[tid] = kid_r;
      kid[BN + tid] = kpos_r;
    }
  };

  const float c2 = s.scale_log2;
  f32x16 dqa[DQK / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dqa[d] = f32x16{};

  int cls;
  int kt = next_tile(t_lo, cls);
  int buf = 0;
  if (kt < t_hi) {
    load_tile(kt);
    store_tile(0);
  }
  __syncthreads();

  while (kt < t_hi) {
    int ncls;
    const int nkt = next_tile(kt + 1, ncls);
    if (nkt < t_hi) load_tile(nkt);

    const char* st = stage_ptr(buf);
    const T* Ks = reinterpret_cast<const T*>(st);
    const T* KT = Ks + C::K_ELEMS;
    const T* Vs = KT + C::KT_ELEMS;
    const int* kid = reinterpret_cast<const int*>(Vs + C::V_ELEMS);
    const int k0 = kt * BN;

    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    f32x16 pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        sacc[blk] = mma(lds8<T>(Ks + (blk * 32 + n) * C::KSTR + 16 * t + 8 * hf), qf[t], sacc[blk]);
#pragma unroll
    for (int t = 0; t < DV / 16; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        pacc[blk] = mma(lds8<T>(Vs + (blk * 32 + n) * C::VSTR + 16 * t + 8 * hf), dof[t], pacc[blk]);

    // P = exp2(S * scale * log2e - LSE2); dS = P * (dP - Delta).
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int kk = blk * 32 + 8 * grp + 4 * hf;
        i32x4 ids4 = i32x4{0, 0, 0, 0}, pos4 = i32x4{0, 0, 0, 0};
        if (cls == kTilePart && general) {
          ids4 = *reinterpret_cast<const i32x4*>(kid + kk);
          pos4 = *reinterpret_cast<const i32x4*>(kid + BN + kk);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * grp + i;
          float p = fast_exp2(fmaf(sacc[blk][r], c2, -lse2));
          if (cls == kTilePart && !allowed(route, causal, s.Skv, qi, k0 + kk + i, qm, TokMeta{ids4[i], pos4[i]}))
            p = 0.f;
          sacc[blk][r] = p * (pacc[blk][r] - delta);
        }
      }
    }

    // dQ^T += K^T dS^T.
    F8 dsf[2][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) dsf[blk][s2] = E::cvt8(slots8(sacc[blk], s2));
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          dqa[d] = mma(lds8<T>(KT + (d * 32 + n) * C::KTSTR + blk * 32 + 16 * s2 + 8 * hf), dsf[blk][s2], dqa[d]);

    if (C::NBUF == 1) __syncthreads();
    if (nkt < t_hi) store_tile(C::NBUF == 2 ? buf ^ 1 : buf);
    __syncthreads();
    if (C::NBUF == 2) buf ^= 1;
    kt = nkt;
    cls = ncls;
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
  static constexpr int BM = 64;    // queries per step
  static constexpr int QSTR = DQK + 8;
  static constexpr int QTSTR = BM + 8;
  static constexpr int DOSTR = DV + 8;
  static constexpr int DOTSTR = BM + 8;
  static constexpr int Q_ELEMS = BM * QSTR;
  static constexpr int QT_ELEMS = DQK * QTSTR;
  static constexpr int DO_ELEMS = BM * DOSTR;
  static constexpr int DOT_ELEMS = DV * DOTSTR;
  static constexpr int SIDE_BYTES = BM * 4 * 4;   // lse2, delta, meta (a, b)
  static constexpr int STAGE_BYTES = (Q_ELEMS + QT_ELEMS + DO_ELEMS + DOT_ELEMS) * (int)sizeof(T) + SIDE_BYTES;
  static constexpr int NBUF = (2 * STAGE_BYTES <= 160 * 1024) ? 2 : 1;
};

template <typename T, int DQK, int DV>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_kernel(BwdArgs a) {
  using C = DkvCfg<T, DQK, DV>;
  using E = Elem<T>;
  using F8 = typename E::F8;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(16))) char smem[C::NBUF * C::STAGE_BYTES];

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
  const int kt = krank;      // causal: low key tiles are the heaviest and come first
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

  auto classify = [&](int qt) -> int {
    TileSum qs{};
    if (route != kRouteDense) qs = tile_sum(sum_q_row, a.seg.nch_q, qt * BM, BM);
    return classify_tile(route, causal, s.Skv, qt * BM, BM, k0, BN, qs, ks);
  };
  // Steps run over (query head in group, query tile) in a fixed order.
  auto next_step = [&](int step, int& cls) -> int {
    for (int x = step; x < g * ntiles; ++x) {
      cls = classify(t_lo + x % ntiles);
      if (cls != kTileSkip) return x;
    }
    cls = kTileSkip;
    return g * ntiles;
  };

  PairTile<T, BM, DQK, 256> qreg;
  PairTile<T, BM, DV, 256> doreg;
  float side_r = 0.f;
  int meta_r = 0;
  auto load_step = [&](int x) {
    const int h = hkv * g + x / ntiles;
    const int i0 = (t_lo + x % ntiles) * BM;
    const int nvalid = min(BM, s.Sq - i0);
    qreg.load(static_cast<const T*>(a.q) + b * a.sq.b + h * a.sq.h + i0 * a.sq.t, a.sq.t, nvalid, tid);
    doreg.load(static_cast<const T*>(a.dout) + b * a.so.b + h * a.so.h + i0 * a.so.t, a.so.t, nvalid, tid);
    // threads 0..63: lse2, 64..127: delta, 128..191: meta a, 192..255: meta b
    const int r = tid & (BM - 1);
    const int i = i0 + r;
    const int which = tid / BM;
    if (which < 2) {
      const size_t x2 = ((size_t)b * s.Hq + h) * s.Sq + i;
      side_r = i < s.Sq ? (which == 0 ? a.lse2[x2] : a.delta[x2]) : (which == 0 ? INFINITY : 0.f);
    } else {
      const TokMeta t = q_meta(route, a.seg, b, s.Sq, i);
      meta_r = which == 2 ? t.a : t.b;
    }
  };
  auto stage_ptr = [&](int buf) { return smem + buf * C::STAGE_BYTES; };
  auto store_step = [&](int buf) {
    char* st = stage_ptr(buf);
    T* Qs = reinterpret_cast<T*>(st);
    T* QT = Qs + C::Q_ELEMS;
    T* dOs = QT + C::QT_ELEMS;
    T* dOT = dOs + C::DO_ELEMS;
    float* side = reinterpret_cast<float*>(dOT + C::DOT_ELEMS);
    qreg.store_rows(Qs, C::QSTR, tid);
    qreg.store_t(QT, C::QTSTR, tid);
    doreg.store_rows(dOs, C::DOSTR, tid);
    doreg.store_t(dOT, C::DOTSTR, tid);
    if (tid < 2 * BM)
      side[tid] = side_r;
    else
      reinterpret_cast<int*>(side)[tid] = meta_r;
  };

  const float c2 = s.scale_log2;
  f32x16 dka[DQK / 32];
  f32x16 dva[DV / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dka[d] = f32x16{};
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) dva[d] = f32x16{};

  int cls;
  int x = next_step(0, cls);
  int buf = 0;
  if (x < g * ntiles) {
    load_step(x);
    store_step(0);
  }
  __syncthreads();

  while (x < g * ntiles) {
    int ncls;
    const int nx = next_step(x + 1, ncls);
    if (nx < g * ntiles) load_step(nx);

    const char* st = stage_ptr(buf);
    const T* Qs = reinterpret_cast<const T*>(st);
    const T* QT = Qs + C::Q_ELEMS;
    const T* dOs = QT + C::QT_ELEMS;
    const T* dOT = dOs + C::DO_ELEMS;
    const float* lse2s = reinterpret_cast<const float*>(dOT + C::DOT_ELEMS);
    const float* deltas = lse2s + BM;
    const int* qma = reinterpret_cast<const int*>(lse2s + 2 * BM);
    const int* qmb = qma + BM;
    const int i0 = (t_lo + x % ntiles) * BM;

#pragma unroll
    for (int qb = 0; qb < BM / 32; ++qb) {
      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys.
      f32x16 sa = f32x16{}, pa = f32x16{};
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) sa = mma(lds8<T>(Qs + (qb * 32 + n) * C::QSTR + 16 * t + 8 * hf), kf[t], sa);
#pragma unroll
      for (int t = 0; t < DV / 16; ++t) pa = mma(lds8<T>(dOs + (qb * 32 + n) * C::DOSTR + 16 * t + 8 * hf), vf[t], pa);
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int rr = qb * 32 + 8 * grp + 4 * hf;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + rr);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(deltas + rr);
        i32x4 ma = i32x4{0, 0, 0, 0}, mb = i32x4{0, 0, 0, 0};
        if (cls == kTilePart && route != kRouteDense) {
          ma = *reinterpret_cast<const i32x4*>(qma + rr);
          mb = *reinterpret_cast<const i32x4*>(qmb + rr);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * grp + i;
          float p = fast_exp2(fmaf(sa[r], c2, -l4[i]));
          if (cls == kTilePart && !allowed(route, causal, s.Skv, i0 + rr + i, kj, TokMeta{ma[i], mb[i]}, km))
            p = 0.f;
          sa[r] = p;
          pa[r] = p * (pa[r] - d4[i]);
        }
      }
      F8 pf[2], dsf[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        pf[s2] = E::cvt8(slots8(sa, s2));
        dsf[s2] = E::cvt8(slots8(pa, s2));
      }
      // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries.
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          dva[d] = mma(lds8<T>(dOT + (d * 32 + n) * C::DOTSTR + qb * 32 + 16 * s2 + 8 * hf), pf[s2], dva[d]);
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          dka[d] = mma(lds8<T>(QT + (d * 32 + n) * C::QTSTR + qb * 32 + 16 * s2 + 8 * hf), dsf[s2], dka[d]);
    }

    if (C::NBUF == 1) __syncthreads();
    if (nx < g * ntiles) store_step(C::NBUF == 2 ? buf ^ 1 : buf);
    __syncthreads();
    if (C::NBUF == 2) buf ^= 1;
    x = nx;
    cls = ncls;
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

// ------------------------------------------------------------ launchers

template <typename T, int DQK, int DV>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  using C = FwdCfg<T, DQK, DV>;
  const int n_qt = (a.s.Sq + C::BM - 1) / C::BM;
  const long long nblocks = (long long)a.s.B * a.s.Hq * n_qt;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_kernel<T, DQK, DV>), dim3((unsigned)nblocks), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

template <typename T, int DQK, int DV>
hipError_t launch_bwd_delta(const BwdArgs& a, hipStream_t st) {
  const size_t rows = (size_t)a.s.B * a.s.Sq * a.s.Hq;
  if (rows == 0) return hipSuccess;
  const size_t blocks = (rows * 8 + 255) / 256;
  hipLaunchKernelGGL((attn_bwd_delta_kernel<T, DV>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int DQK, int DV>
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t st) {
  const int n_kt = (a.s.Skv + DkvCfg<T, DQK, DV>::BN - 1) / DkvCfg<T, DQK, DV>::BN;
  const long long nblocks = (long long)a.s.B * a.s.Hkv * n_kt;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DQK, DV>), dim3((unsigned)nblocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int DQK, int DV>
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st) {
  const int n_qt = (a.s.Sq + DqCfg<T, DQK, DV>::BM - 1) / DqCfg<T, DQK, DV>::BM;
  const long long nblocks = (long long)a.s.B * a.s.Hq * n_qt;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DQK, DV>), dim3((unsigned)nblocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace bps
