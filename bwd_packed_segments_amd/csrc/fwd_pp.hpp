// Forward over two query heads of a GQA group, the heads half a step apart
// (bf16).
//
// A workgroup takes the same 128 queries of two query heads that share a
// key/value head, four waves per head, so every SIMD runs one wave of each
// head.  Run in step, both waves of a SIMD would issue their products at the
// same time (competing for the matrix pipe while the vector unit idles) and
// then their softmax at the same time.  Here every wave runs the same loop,
//   step j:  [O += V_{j-1}^T P_{j-1}^T, S_j = K_j Q^T]   [softmax of S_j -> P_j]
//            (matrix block)                               (vector block)
// but the waves of head A reach the workgroup barrier after the vector block
// and those of head B after the matrix block.  Between two barriers head A
// thus runs its matrix block and then its vector block, head B its vector
// block and then its matrix block, and on every SIMD one wave's
// exponentials run beside the other's products.  The arithmetic of each head
// is that of the plain forward (same products in the same order, same
// softmax), so the results are bitwise the same.
//
// In the interval that ends at barrier j both heads read K_j and V_{j-1};
// meanwhile K_{j+1} and V_j are fetched (head A at the start of its step j,
// head B right after its barrier j - 1) with direct-to-LDS buffer loads
// whose per-lane offsets are fixed (the tile moves only the scalar offset).
// K_j and V_j share stage j % 2; the key metadata of the masks (general
// route) sit in a ring of three slots indexed by walk position, since head
// B masks tile j one interval after head A.  The walk over key tiles, their classes and masks are those
// of the plain forward.
#pragma once

#include <type_traits>

#include "bps_args.hpp"
#include "lds_tile.hpp"

namespace bps {

template <int DQK, int DV>
struct FwdPpCfg {
  static constexpr int BM = 128;   // queries per head
  static constexpr int BN = 64;    // keys per step
  static constexpr int THREADS = 512;
  static constexpr int K_BYTES = BN * DQK * 2;
  static constexpr int V_BYTES = BN * DV * 2;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int KID_OFF = 2 * STAGE;       // 3 x (ids, positions) of 64 keys
  static constexpr int KID_BYTES = 2 * BN * 4;
  static constexpr int LDS_BYTES = KID_OFF + 3 * KID_BYTES;
  static constexpr int KPER = BN * DQK / 8 / THREADS;   // 16-byte chunks per thread of a K tile
  static constexpr int VPER = BN * DV / 8 / THREADS;
  static constexpr bool ENABLED = (DQK == 64 || DQK == 128) && (DV == 64 || DV == 128) && KPER >= 1 &&
                                  VPER >= 1 && LDS_BYTES + kClassCap <= 160 * 1024;
};

// Byte offsets below 2^31 for every key row the buffer loads may address
// (per batch row and key/value head).
inline bool fwd_pp_offsets_fit(const FwdArgs& a, int dqk, int dv) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t k = ((int64_t)(a.s.Skv - 1) * a.sk.t + dqk) * 2;
  const int64_t v = ((int64_t)(a.s.Skv - 1) * a.sv.t + dv) * 2;
  return a.sk.t >= 0 && a.sv.t >= 0 && k < lim && v < lim;
}

template <int DQK, int DV>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
    attn_fwd_pp_kernel(FwdArgs a) {
  using C = FwdPpCfg<DQK, DV>;
  using T = bf16;
  using E = Elem<T>;
  using F8 = bf16x8;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  __shared__ unsigned char cls_tab[kClassCap];

  const AttnShape& s = a.s;
  const bool causal = s.causal != 0;
  const int n_qt = (s.Sq + BM - 1) / BM;
  const int g = s.Hq / s.Hkv;
  const int ngh = g / 2;
  const int nblocks = s.B * s.Hkv * ngh * n_qt;
  int L = logical_block(nblocks, s.reverse);
  const int hgp = L % ngh;
  L /= ngh;
  const int qrank = L % n_qt;
  L /= n_qt;
  const int hkv = L % s.Hkv;
  const int b = L / s.Hkv;
  const int qt = q_tile_of(a.seg, b, qrank, n_qt, causal);
  const int q0 = qt * BM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool late = wave >= 4;   // head B
  const int h = hkv * g + hgp * 2 + (wave >= 4 ? 1 : 0);
  const int qi = q0 + (wave & 3) * 32 + n;

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

  auto classify = [&](int kt) __attribute__((always_inline)) -> int {
    TileSum ks{};
    if (route != kRouteDense) ks = tile_sum(sum_kv_row, a.seg.nch_kv, kt * BN, BN);
    return classify_tile(route, causal, s.Skv, q0, BM, kt * BN, BN, qs, ks);
  };
  const bool tabled = route != kRouteDense;
  if (tabled) {
    fill_classes(cls_tab, t_hi - t_lo, tid, C::THREADS, [&](int i) { return classify(t_lo + i); });
    __syncthreads();
  }
  auto next_tile = [&](int kt, int& cls) __attribute__((always_inline)) -> int {
    for (int k = kt; k < t_hi; ++k) {
      cls = (tabled && k - t_lo < kClassCap) ? (int)cls_tab[k - t_lo] : classify(k);
      if (cls != kTileSkip) return k;
    }
    cls = kTileSkip;
    return t_hi;
  };

  // ---------------------------------------------------------------- loads
  // Chunk x of this thread: row r, physical slot sl holds the logical chunk
  // the swizzle puts there.  Byte offsets of a key row fit in 32 bits
  // (checked by the host).
  using FK = TileFmt<T, DQK>;
  using FV = TileFmt<T, DV>;
  const __amdgpu_buffer_rsrc_t k_rsrc = raw_rsrc(uniform_ptr(kp));
  const __amdgpu_buffer_rsrc_t v_rsrc = raw_rsrc(uniform_ptr(vp));
  const uint32_t k_ts = (uint32_t)a.sk.t * 2, v_ts = (uint32_t)a.sv.t * 2;
  uint32_t k_voff[C::KPER], v_voff[C::VPER];
#pragma unroll
  for (int x = 0; x < C::KPER; ++x) {
    const int sl = x * C::THREADS + tid, r = sl / FK::NC;
    k_voff[x] = (uint32_t)r * k_ts + (uint32_t)FK::swz(r, sl % FK::NC) * 16;
  }
#pragma unroll
  for (int x = 0; x < C::VPER; ++x) {
    const int sl = x * C::THREADS + tid, r = sl / FV::NC;
    v_voff[x] = (uint32_t)r * v_ts + (uint32_t)FV::swz(r, sl % FV::NC) * 16;
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(BPS_LDS char*)smem);
  const uint32_t wave_m0 = (uint32_t)(wave * 64 * 16);   // this wave's 1 KB of a chunk row
  auto kid_of = [&](int ks) __attribute__((always_inline)) {   // metadata slot ks of the ring of three
    return reinterpret_cast<int*>(smem + C::KID_OFF + ks * C::KID_BYTES);
  };

  // K tile kt into stage ST, its key metadata (general route) into slot ks
  // of the ring.
  auto issue_k = [&](int kt, auto stc, int ks) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    const int k0 = kt * BN;
    const int nvalid = min(BN, s.Skv - k0);
    if (nvalid == BN) {
      const uint32_t m0 = lds0 + (uint32_t)(ST * C::STAGE) + wave_m0;
#pragma unroll
      for (int x = 0; x < C::KPER; ++x) lds_load16(k_rsrc, m0 + x * C::THREADS * 16, k_voff[x], (uint32_t)k0 * k_ts);
      if (general && wave < 2) {
        const int* src = (wave == 0 ? a.seg.ids_kv : a.seg.pos_kv) + (size_t)b * s.Skv + k0 + lane;
        lds_load4(src, lds0 + (uint32_t)(C::KID_OFF + ks * C::KID_BYTES + wave * BN * 4));
      }
    } else {
      TileLoad<T, BN, DQK, C::THREADS>::staged(kp + k0 * a.sk.t, a.sk.t, nvalid,
                                               reinterpret_cast<T*>(smem + ST * C::STAGE), tid);
      if (general && tid < 2 * BN) {
        const int j = tid & (BN - 1);
        const size_t row = (size_t)b * s.Skv + k0 + j;
        kid_of(ks)[tid] = k0 + j < s.Skv ? (tid < BN ? a.seg.ids_kv[row] : a.seg.pos_kv[row]) : 0;
      }
    }
  };
  // V tile kt into stage ST.
  auto issue_v = [&](int kt, auto stc) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    const int k0 = kt * BN;
    const int nvalid = min(BN, s.Skv - k0);
    if (nvalid == BN) {
      const uint32_t m0 = lds0 + (uint32_t)(ST * C::STAGE + C::K_BYTES) + wave_m0;
#pragma unroll
      for (int x = 0; x < C::VPER; ++x) lds_load16(v_rsrc, m0 + x * C::THREADS * 16, v_voff[x], (uint32_t)k0 * v_ts);
    } else {
      TileLoad<T, BN, DV, C::THREADS>::staged(vp + k0 * a.sv.t, a.sv.t, nvalid,
                                              reinterpret_cast<T*>(smem + ST * C::STAGE + C::K_BYTES), tid);
    }
  };

  // ---------------------------------------------------------------- math
  // Per-lane LDS byte offsets, fixed: K rows (fragment t of row n) and V^T
  // (column block d, rows y and y + 8 of each 16-row group); tile rows and
  // stages move only immediates.
  uint32_t roff[DQK / 16];
  uint32_t troff[DV / 32][2];
#pragma unroll
  for (int t = 0; t < DQK / 16; ++t) roff[t] = (uint32_t)FK::off(n, 16 * t + 8 * hf) * 2;
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int G = lane >> 4, i = lane & 15;
      const int x = 32 * d + 16 * (G & 1) + 4 * (i & 3);
      const int y = 4 * (G >> 1) + (i >> 2) + 8 * p;
      troff[d][p] = C::K_BYTES + (uint32_t)FV::off(y, x) * 2;
    }

  const float c2 = s.scale_log2;
  float m = -INFINITY;   // reference max of the scores (rescaled lazily)
  float l = 0.f;         // this lane half's partial sum
  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};
  f32x16 sacc[2];
  F8 pf[2][2];

  auto rd_k = [&](int st, int blk, int t) __attribute__((always_inline)) -> F8 {
    return *reinterpret_cast<const F8*>(smem + st * C::STAGE + blk * 32 * DQK * 2 + roff[t]);
  };
  auto rd_vt = [&](int st, int d, int y0) __attribute__((always_inline)) -> F8 {
    const char* base = smem + st * C::STAGE + y0 * DV * 2;
    const bf16x4v x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)(base + troff[d][0]));
    const bf16x4v y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)(base + troff[d][1]));
    return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  };
  // S^T = K Q^T for a tile's 64 keys in stage st, K fragments two k-steps
  // ahead (order pinned with scheduling groups).
  auto scores = [&](int st) __attribute__((always_inline)) {
    constexpr int NT = DQK / 16;
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    F8 kr[3][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) kr[t][blk] = rd_k(st, blk, t);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t + 2 < NT) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) kr[(t + 2) % 3][blk] = rd_k(st, blk, t + 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) sacc[blk] = mma(kr[t % 3][blk], qf[t], sacc[blk]);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };
  // O^T += V^T P^T with the tile's V in stage st.
  auto values = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) o[d] = mma(rd_vt(st, d, blk * 32 + 16 * s2), pf[blk][s2], o[d]);
  };
  // Mask (partial tiles), online softmax, P in bf16 as the B operands of
  // the value product.
  auto softmax = [&](int kt, int cls, int ks) __attribute__((always_inline)) {
    if (cls == kTilePart) {
      const int* kid = kid_of(ks);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        mask_tile<true>(sacc[blk], -INFINITY, route, causal, s.Skv, qi, qm, kt * BN + blk * 32, hf, kid, kid + BN,
                        blk * 32);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
    mx = wave_xor32_max(mx);
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
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) pf[blk][s2] = E::cvt8(slots8(sacc[blk], s2));
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    wait_vm();
    __syncthreads();
  };

  // ---------------------------------------------------------------- walk
  // Tiles j, j+1, j+2 of the walk (t_hi: past the end) and their classes.
  int c0, c1, c2t;
  int kt0 = next_tile(t_lo, c0);
  int kt1 = kt0 < t_hi ? next_tile(kt0 + 1, c1) : (c1 = kTileSkip, t_hi);
  int kt2 = kt1 < t_hi ? next_tile(kt1 + 1, c2t) : (c2t = kTileSkip, t_hi);
  int ks0 = 0;   // metadata slot of tile j (walk position j mod 3)
  if (kt0 < t_hi) issue_k(kt0, std::integral_constant<int, 0>{}, 0);
  barrier();
  if (late) {   // head B's share of step 0's fetches
    if (kt1 < t_hi) issue_k(kt1, std::integral_constant<int, 1>{}, 1);
    if (kt0 < t_hi) issue_v(kt0, std::integral_constant<int, 0>{});
  }

  bool prev = false;   // tile j - 1 exists (its value product is due)
  // Step j with j % 2 == P: tile j in stage P, tile j - 1 in stage P ^ 1.
  auto step = [&](auto pc) __attribute__((always_inline)) -> bool {
    constexpr int P = decltype(pc)::value;
    constexpr int Q = P ^ 1;
    if (kt0 >= t_hi && !prev) return false;
    const int ks1 = ks0 == 2 ? 0 : ks0 + 1;
    if (!late) {
      if (kt1 < t_hi) issue_k(kt1, std::integral_constant<int, Q>{}, ks1);
      if (kt0 < t_hi) issue_v(kt0, std::integral_constant<int, P>{});
    }
    if (prev) values(Q);
    if (kt0 < t_hi) scores(P);
    if (late) {
      barrier();
      if (kt2 < t_hi) issue_k(kt2, std::integral_constant<int, P>{}, ks1 == 2 ? 0 : ks1 + 1);
      if (kt1 < t_hi) issue_v(kt1, std::integral_constant<int, Q>{});
    }
    if (kt0 < t_hi) softmax(kt0, c0, ks0);
    if (!late) barrier();
    prev = kt0 < t_hi;
    kt0 = kt1;
    c0 = c1;
    kt1 = kt2;
    c1 = c2t;
    if (kt2 < t_hi) kt2 = next_tile(kt2 + 1, c2t);
    ks0 = ks1;
    return true;
  };
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
  wait_vm();

  // Epilogue: O = O^T / l, LSE = m * scale + ln(l); empty rows give O = 0,
  // LSE = -inf.
  const float lt = wave_xor32_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? m * s.scale + logf(lt) : -INFINITY;
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

}  // namespace bps
