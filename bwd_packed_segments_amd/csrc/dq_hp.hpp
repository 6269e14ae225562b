// dQ over two query heads of a GQA group with the blocks of the loop rotated
// (bf16, no variants).
//
// A workgroup takes the same 128 queries of two query heads that share a
// key/value head, four waves per head; each key/value tile is loaded once
// for both.  Per 32-key block of a key tile a wave forms S^T and dP^T
// (products), then P = exp2(S scale log2 e - LSE2) and dS = P (dP - Delta)
// (vector work), then dQ^T += K^T dS^T (products that need the vector
// result).  Taken in that order, every block's dQ products wait for its
// vector work, which waits for its S^T and dP^T.  Here the loop is rotated:
//   [dQ of the previous 32-key block, S^T and dP^T of this block] [vector work of this block]
// so 24 independent products run back to back between two stretches of
// vector work.  The products and their order per head are those of the plain
// dQ kernel, so dQ is bitwise the same.  (Offsetting the two heads by half a
// step, so that one wave's vector work would run beside the other's
// products, measured no gain: 1.440 against 1.403 ms on the 8K GQA workload.)
//
// Between two barriers a workgroup touches key tiles j - 1 (the dQ products
// of its last block) and j, so K/V and the key metadata of the masks sit in
// three LDS stages while tile j + 1 is fetched, with inline-asm buffer loads
// whose per-lane offsets are fixed (the tile moves only the scalar offset;
// the compiler then inserts no wait for them before LDS reads).  The loop is
// unrolled over the three stages, so every LDS address is a lane offset
// plus an immediate.
#pragma once

#include <type_traits>

#include "bps_args.hpp"
#include "lds_tile.hpp"

namespace bps {

template <int DQK, int DV>
struct DqHpCfg {
  static constexpr int BM = 128;   // queries per head
  static constexpr int BN = 64;    // keys per step
  static constexpr int THREADS = 512;
  static constexpr int NS = 3;     // K/V stages
  static constexpr int K_BYTES = BN * DQK * 2;
  static constexpr int V_BYTES = BN * DV * 2;
  static constexpr int KID_BYTES = 2 * BN * 4;
  static constexpr int STAGE = K_BYTES + V_BYTES + KID_BYTES;
  static constexpr int LDS_BYTES = NS * STAGE;
  static constexpr int KPER = BN * DQK / 8 / THREADS;
  static constexpr int VPER = BN * DV / 8 / THREADS;
  static constexpr bool ENABLED = (DQK == 64 || DQK == 128) && (DV == 64 || DV == 128) && KPER >= 1 &&
                                  VPER >= 1 && LDS_BYTES + kClassCap <= 160 * 1024;
};

template <int DQK, int DV>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
    attn_bwd_dq_hp_kernel(BwdArgs a) {
  using C = DqHpCfg<DQK, DV>;
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
  const int h = hkv * g + hgp * 2 + (wave >= 4 ? 1 : 0);
  const int qi = q0 + (wave & 3) * 32 + n;

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
  const uint32_t wave_m0 = (uint32_t)(wave * 64 * 16);

  // Key tile kt (K, V and, on the general route, the key metadata) into
  // stage ST; this thread's share.
  auto issue = [&](int kt, auto stc) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    const int k0 = kt * BN;
    const int nvalid = min(BN, s.Skv - k0);
    char* st = smem + ST * C::STAGE;
    if (nvalid == BN) {
      const uint32_t m0 = lds0 + (uint32_t)(ST * C::STAGE) + wave_m0;
#pragma unroll
      for (int x = 0; x < C::KPER; ++x) lds_load16(k_rsrc, m0 + x * C::THREADS * 16, k_voff[x], (uint32_t)k0 * k_ts);
#pragma unroll
      for (int x = 0; x < C::VPER; ++x)
        lds_load16(v_rsrc, m0 + C::K_BYTES + x * C::THREADS * 16, v_voff[x], (uint32_t)k0 * v_ts);
      if (general && wave < 2) {
        const int* src = (wave == 0 ? a.seg.ids_kv : a.seg.pos_kv) + (size_t)b * s.Skv + k0 + lane;
        lds_load4(src, lds0 + (uint32_t)(ST * C::STAGE + C::K_BYTES + C::V_BYTES + wave * BN * 4));
      }
    } else {
      TileLoad<T, BN, DQK, C::THREADS, true>::staged(kp + k0 * a.sk.t, a.sk.t, nvalid, reinterpret_cast<T*>(st), tid);
      TileLoad<T, BN, DV, C::THREADS, true>::staged(vp + k0 * a.sv.t, a.sv.t, nvalid,
                                                    reinterpret_cast<T*>(st + C::K_BYTES), tid);
      if (general && tid < 2 * BN) {
        const int j = tid & (BN - 1);
        const size_t row = (size_t)b * s.Skv + k0 + j;
        reinterpret_cast<int*>(st + C::K_BYTES + C::V_BYTES)[tid] =
            k0 + j < s.Skv ? (tid < BN ? a.seg.ids_kv[row] : a.seg.pos_kv[row]) : 0;
      }
    }
  };

  // ---------------------------------------------------------------- math
  // Per-lane LDS byte offsets inside a stage, fixed for the walk: K rows and
  // V rows (fragment t of row n of the first 32-key block) and transposed K
  // reads (column block d, rows y and y + 8 of the first 16-row group).
  uint32_t kro[DQK / 16], vro[DV / 16], ktr[DQK / 32][2];
#pragma unroll
  for (int t = 0; t < DQK / 16; ++t) kro[t] = (uint32_t)FK::off(n, 16 * t + 8 * hf) * 2;
#pragma unroll
  for (int t = 0; t < DV / 16; ++t) vro[t] = (uint32_t)(C::K_BYTES + FV::off(n, 16 * t + 8 * hf) * 2);
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int G = lane >> 4, i = lane & 15;
      ktr[d][p] = (uint32_t)FK::off(4 * (G >> 1) + (i >> 2) + 8 * p, 32 * d + 16 * (G & 1) + 4 * (i & 3)) * 2;
    }

  const float c2 = s.scale_log2;
  f32x16 dqa[DQK / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dqa[d] = f32x16{};
  f32x16 sacc, pacc;   // S^T and dP^T of the current 32-key block
  F8 dsf[2];           // dS^T of the last 32-key block, the B operands of its dQ product

  // S^T and dP^T of block blk of the tile in stage ST.
  auto front = [&](auto stc, int blk) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    sacc = f32x16{};
    pacc = f32x16{};
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t)
      sacc = mma(*reinterpret_cast<const F8*>(smem + ST * C::STAGE + blk * 32 * DQK * 2 + kro[t]), qf[t], sacc);
#pragma unroll
    for (int t = 0; t < DV / 16; ++t)
      pacc = mma(*reinterpret_cast<const F8*>(smem + ST * C::STAGE + blk * 32 * DV * 2 + vro[t]), dof[t], pacc);
  };
  // dQ^T += K^T dS^T of block blk of the tile in stage ST.
  auto back = [&](auto stc, int blk) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const char* base = smem + ST * C::STAGE + (blk * 32 + 16 * s2) * DQK * 2;
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d) {
        const bf16x4v x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)(base + ktr[d][0]));
        const bf16x4v y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)(base + ktr[d][1]));
        dqa[d] = mma(F8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]}, dsf[s2], dqa[d]);
      }
    }
  };
  // P, mask, dS of block blk of key tile kt (class cls, metadata in stage ST).
  auto grad = [&](auto stc, int kt, int cls, int blk) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(fmaf(sacc[r], c2, -lse2));
    if (cls == kTilePart) {
      const int* kid = reinterpret_cast<const int*>(smem + ST * C::STAGE + C::K_BYTES + C::V_BYTES);
      mask_tile<true>(sacc, 0.f, route, causal, s.Skv, qi, qm, kt * BN + blk * 32, hf, kid, kid + BN, blk * 32);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = sacc[r] * (pacc[r] - delta);
    dsf[0] = E::cvt8(slots8(sacc, 0));
    dsf[1] = E::cvt8(slots8(sacc, 1));
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    wait_vm();
    __syncthreads();
  };

  // ---------------------------------------------------------------- walk
  int c0, c1;
  int kt0 = next_tile(t_lo, c0);
  int kt1 = kt0 < t_hi ? next_tile(kt0 + 1, c1) : (c1 = kTileSkip, t_hi);
  if (kt0 < t_hi) issue(kt0, std::integral_constant<int, 0>{});
  barrier();

  bool prev = false;   // tile j - 1 exists (the dQ product of its last block is due)
  // Step j with j % 3 == ST: tile j in stage ST, j - 1 in SP, j + 1 (fetched
  // meanwhile) in SN.
  auto step = [&](auto stc) __attribute__((always_inline)) -> bool {
    constexpr int ST = decltype(stc)::value;
    constexpr int SN = (ST + 1) % 3, SP = (ST + 2) % 3;
    if (kt0 >= t_hi && !prev) return false;
    const bool cur = kt0 < t_hi;
    if (kt1 < t_hi) issue(kt1, std::integral_constant<int, SN>{});
    if (prev) back(std::integral_constant<int, SP>{}, 1);
    if (cur) {
      front(stc, 0);
      grad(stc, kt0, c0, 0);
      back(stc, 0);
      front(stc, 1);
      grad(stc, kt0, c0, 1);
    }
    barrier();
    prev = cur;
    kt0 = kt1;
    c0 = c1;
    if (kt1 < t_hi) kt1 = next_tile(kt1 + 1, c1);
    return true;
  };
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{}) &&
         step(std::integral_constant<int, 2>{})) {
  }
  wait_vm();

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

}  // namespace bps
