// Device-side building blocks shared by the attention kernels (gfx950).
//
// MFMA conventions used everywhere (v_mfma_f32_32x32x16_bf16, wave64;
// lane l, n = l % 32, hf = l / 32):
//   A operand (32 rows x 16 k):  lane holds A[n][k(hf, e)], e = 0..7
//   B operand (16 k x 32 cols):  lane holds B[k(hf, e)][n]
//   C/D (32 x 32, fp32):         lane holds C[rmap(hf, r)][n], r = 0..15,
//                                rmap(hf, r) = 8 * (r / 4) + 4 * hf + r % 4
// The hardware pairs the k slots of A and B; only the C layout is fixed by
// the instruction.  Fragments loaded from memory along a contiguous axis use
// k(hf, e) = 8 hf + e.  A C tile fed back as a B operand (k = rows of C)
// uses, for k-step s of a 32-row block, k(hf, e) = 16 s + cmap(hf, e) with
// cmap(hf, e) = 8 * (e / 4) + 4 * hf + e % 4; the matching A operand is read
// from a transposed LDS tile whose column order within each group of 16 is
// the permutation that swaps bits 2 and 3 of the index (perm16 below), so
// that those 8 values are contiguous.
//
// fp32 tensors use v_mfma_f32_32x32x2_f32 eight times per 16-wide k step
// with the same per-lane fragment layout, so every kernel is written once
// for both element types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bps {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ element traits

template <typename T> struct Elem;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <> struct Elem<bf16> {
  typedef bf16x8 F8;   // one operand fragment (8 elements)
  typedef uint32_t P2; // two elements (transposed LDS stores)
  typedef bf16x4 P4;   // four elements (output stores)
  __device__ static F8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static F8 zero8() { return F8{}; }
  __device__ static F8 cvt8(const f32x8& x) { return __builtin_convertvector(x, bf16x8); }
  __device__ static P4 cvt4(const f32x4& x) { return __builtin_convertvector(x, bf16x4); }
  // Element e of a next to element e of b, as one 32-bit word.
  template <int e>
  __device__ static P2 pair(const F8& a, const F8& b) {
    const u32x4 wa = __builtin_bit_cast(u32x4, a);
    const u32x4 wb = __builtin_bit_cast(u32x4, b);
    return (e & 1) ? ((wa[e >> 1] >> 16) | (wb[e >> 1] & 0xFFFF0000u))
                   : ((wa[e >> 1] & 0xFFFFu) | (wb[e >> 1] << 16));
  }
};

template <> struct Elem<float> {
  typedef f32x8 F8;
  typedef f32x2 P2;
  typedef f32x4 P4;
  __device__ static F8 load8(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return F8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  __device__ static F8 zero8() { return F8{}; }
  __device__ static F8 cvt8(const f32x8& x) { return x; }
  __device__ static P4 cvt4(const f32x4& x) { return x; }
  template <int e>
  __device__ static P2 pair(const F8& a, const F8& b) { return P2{a[e], b[e]}; }
};

__device__ inline f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline f32x16 mma(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// Row of the C layout held in accumulator slot r by lane half hf.
__device__ __host__ constexpr int rmap(int hf, int r) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// Column order inside a 16-wide group of a transposed LDS tile.
__device__ __host__ constexpr int perm16(int x) { return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1); }

// Take the 8 fp32 values of accumulator slots 8s..8s+7 as one operand.
__device__ inline f32x8 slots8(const f32x16& c, int s) {
  return s == 0 ? f32x8{c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7]}
                : f32x8{c[8], c[9], c[10], c[11], c[12], c[13], c[14], c[15]};
}

__device__ inline float wave_xor32_max(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float wave_xor32_sum(float x) {
  return x + __shfl_xor(x, 32);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ segment metadata

constexpr int kChunk = 32;   // tokens per metadata summary

// Largest token stride (elements) of k and v: the dQ kernel addresses its
// key/value tile rows with 32-bit offsets.
constexpr int64_t kMaxKvTokenStride = (int64_t)1 << 24;

// Summary of kChunk consecutive tokens of one batch row, over the tokens
// that carry a nonzero segment id (cnt of them).  s/e are the bounds
// [start, end) of the contiguous id run holding each token.
struct ChunkSum {
  int cnt, idmin, idmax, posmin;
  int posmax, smin, smax, emin;
  int emax, pad0, pad1, pad2;
};

struct TileSum {
  int cnt, idmin, idmax, posmin, posmax, smin, smax, emin, emax;
};

// Metadata views prepared on the device before the attention kernels run.
struct SegView {
  const int* ids_q;      // [B, Sq]
  const int* pos_q;      // [B, Sq] given or derived
  const int* ids_kv;     // [B, Skv]
  const int* pos_kv;     // [B, Skv]
  const int2* run_q;     // [B, Sq] (start, end) of the id run; (0, 0) for id 0
  const int2* run_kv;    // [B, Skv]
  const ChunkSum* sum_q;   // [B, nch_q]
  const ChunkSum* sum_kv;  // [B, nch_kv]
  const int* route;      // [B] 1 fast, 2 general
  int nch_q, nch_kv;
  // Per batch row, the order in which workgroups take tiles, longest walk
  // first: query tiles of 128 (forward and dQ) and key tiles of 128 (dK/dV).
  // NULL: the fixed order (causal: the tiles with the longest causal walks
  // first).
  const int* qord;       // [B, ceil(Sq / 128)]
  const int* kord;       // [B, ceil(Skv / 128)]
};

// Query tile of 128 that the workgroup of rank r in batch row b takes.
__device__ inline int q_tile_of(const SegView& sv, int b, int r, int n_qt, bool causal) {
  if (sv.qord) return sv.qord[(size_t)b * n_qt + r];
  return causal ? n_qt - 1 - r : r;
}
// Key tile of 128 that the workgroup of rank r in batch row b takes.
__device__ inline int k_tile_of(const SegView& sv, int b, int r, int n_kt) {
  return sv.kord ? sv.kord[(size_t)b * n_kt + r] : r;
}

enum { kRouteDense = 0, kRouteFast = 1, kRouteGeneral = 2 };
enum { kTileSkip = 0, kTileFull = 1, kTilePart = 2 };

__device__ inline TileSum tile_sum(const ChunkSum* row, int nch, int x0, int len) {
  TileSum t;
  t.cnt = 0;
  t.idmin = INT32_MAX; t.idmax = INT32_MIN;
  t.posmin = INT32_MAX; t.posmax = INT32_MIN;
  t.smin = INT32_MAX; t.smax = INT32_MIN;
  t.emin = INT32_MAX; t.emax = INT32_MIN;
  int c0 = x0 / kChunk;
  int c1 = (x0 + len + kChunk - 1) / kChunk;
  if (c1 > nch) c1 = nch;
  for (int c = c0; c < c1; ++c) {
    const ChunkSum s = row[c];
    if (s.cnt == 0) continue;
    t.cnt += s.cnt;
    t.idmin = min(t.idmin, s.idmin); t.idmax = max(t.idmax, s.idmax);
    t.posmin = min(t.posmin, s.posmin); t.posmax = max(t.posmax, s.posmax);
    t.smin = min(t.smin, s.smin); t.smax = max(t.smax, s.smax);
    t.emin = min(t.emin, s.emin); t.emax = max(t.emax, s.emax);
  }
  return t;
}

// Tile of queries [r0, r0+nr) against keys [c0, c0+nc): skip (no allowed
// pair), full (every pair allowed) or partial (per-element mask).
// Conservative: "skip" and "full" are claimed only when certain.
__device__ inline int classify_tile(int route, bool causal, int Skv, int r0, int nr, int c0, int nc,
                                    const TileSum& qs, const TileSum& ks) {
  if (route == kRouteDense) {
    if (causal && c0 > r0 + nr - 1) return kTileSkip;
    if (c0 + nc > Skv) return kTilePart;
    if (causal && c0 + nc - 1 > r0) return kTilePart;
    return kTileFull;
  }
  if (qs.cnt == 0 || ks.cnt == 0) return kTileSkip;
  if (route == kRouteFast) {
    if (c0 + nc <= qs.smin || c0 >= qs.emax) return kTileSkip;
    if (causal && c0 > r0 + nr - 1) return kTileSkip;
    if (qs.cnt == nr && qs.smax <= c0 && qs.emin >= c0 + nc && (!causal || c0 + nc - 1 <= r0))
      return kTileFull;
    return kTilePart;
  }
  if (qs.idmax < ks.idmin || ks.idmax < qs.idmin) return kTileSkip;
  if (causal && ks.posmin > qs.posmax) return kTileSkip;
  if (qs.cnt == nr && ks.cnt == nc && qs.idmin == qs.idmax && ks.idmin == ks.idmax &&
      qs.idmin == ks.idmin && (!causal || ks.posmax <= qs.posmin))
    return kTileFull;
  return kTilePart;
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

// Per-token metadata used by the element mask: (run start, run end) on the
// fast route, (segment id, position) on the general route.
struct TokMeta {
  int a, b;
};

// The element mask.  i, j are token indices inside the batch row; rows past
// Sq and keys past Skv carry empty metadata (fast: (0,0); general: id 0).
// One branch-free predicate per route; the kernels pick the route and the
// causal flag once per tile and apply the predicate with selects.
template <bool CAUSAL>
__device__ inline bool allowed_dense(int Skv, int i, int j) {
  return (j < Skv) & (!CAUSAL | (j <= i));
}
template <bool CAUSAL>
__device__ inline bool allowed_fast(int i, int j, TokMeta qi) {   // qi = run [start, end) of query i
  return (j >= qi.a) & (j < qi.b) & (!CAUSAL | (j <= i));
}
template <bool CAUSAL>
__device__ inline bool allowed_general(TokMeta qi, TokMeta kj) {  // (segment id, position)
  return (qi.a != 0) & (qi.a == kj.a) & (!CAUSAL | (kj.b <= qi.b));
}

__device__ inline bool allowed(int route, bool causal, int Skv, int i, int j, TokMeta qi, TokMeta kj) {
  if (route == kRouteDense) return causal ? allowed_dense<true>(Skv, i, j) : allowed_dense<false>(Skv, i, j);
  if (route == kRouteFast) return causal ? allowed_fast<true>(i, j, qi) : allowed_fast<false>(i, j, qi);
  return causal ? allowed_general<true>(qi, kj) : allowed_general<false>(qi, kj);
}

// Masks one 32x32 accumulator tile held in the C layout: slot r of lane
// (n, hf) is row rmap(hf, r).  KEYS_IN_ROWS: rows are keys kbase + rmap and
// the lane's query is fixed (S^T in the forward and dQ kernels); otherwise
// rows are queries ibase + rmap and the lane's key is fixed (S in the dK/dV
// kernel).  Per-row metadata of the varying side comes from LDS
// (meta_a/meta_b, indexed like the rows, offset by moff); masked slots get
// `fill`.
template <bool KEYS_IN_ROWS, bool CAUSAL>
__device__ inline void mask_tile_route(f32x16& x, float fill, int route, int Skv, int fixed_tok, TokMeta fixed,
                                       int base, int hf, const int* meta_a, const int* meta_b, int moff) {
  if (route == kRouteDense) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = base + rmap(hf, r);
      const bool ok = KEYS_IN_ROWS ? allowed_dense<CAUSAL>(Skv, fixed_tok, v) : allowed_dense<CAUSAL>(Skv, v, fixed_tok);
      x[r] = ok ? x[r] : fill;
    }
  } else if (route == kRouteFast) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      i32x4 ma = i32x4{0, 0, 0, 0}, mb = i32x4{0, 0, 0, 0};
      if (!KEYS_IN_ROWS) {
        ma = *reinterpret_cast<const i32x4*>(meta_a + moff + 8 * grp + 4 * hf);
        mb = *reinterpret_cast<const i32x4*>(meta_b + moff + 8 * grp + 4 * hf);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        const int v = base + rmap(hf, r);
        const bool ok = KEYS_IN_ROWS ? allowed_fast<CAUSAL>(fixed_tok, v, fixed)
                                     : allowed_fast<CAUSAL>(v, fixed_tok, TokMeta{ma[i], mb[i]});
        x[r] = ok ? x[r] : fill;
      }
    }
  } else {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const i32x4 ma = *reinterpret_cast<const i32x4*>(meta_a + moff + 8 * grp + 4 * hf);
      const i32x4 mb = *reinterpret_cast<const i32x4*>(meta_b + moff + 8 * grp + 4 * hf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        const bool ok = KEYS_IN_ROWS ? allowed_general<CAUSAL>(fixed, TokMeta{ma[i], mb[i]})
                                     : allowed_general<CAUSAL>(TokMeta{ma[i], mb[i]}, fixed);
        x[r] = ok ? x[r] : fill;
      }
    }
  }
}

template <bool KEYS_IN_ROWS>
__device__ inline void mask_tile(f32x16& x, float fill, int route, bool causal, int Skv, int fixed_tok, TokMeta fixed,
                                 int base, int hf, const int* meta_a, const int* meta_b, int moff) {
  if (causal)
    mask_tile_route<KEYS_IN_ROWS, true>(x, fill, route, Skv, fixed_tok, fixed, base, hf, meta_a, meta_b, moff);
  else
    mask_tile_route<KEYS_IN_ROWS, false>(x, fill, route, Skv, fixed_tok, fixed, base, hf, meta_a, meta_b, moff);
}

__device__ inline TokMeta q_meta(int route, const SegView& sv, int b, int Sq, int i) {
  if (route == kRouteDense || i >= Sq) return TokMeta{0, 0};
  size_t x = (size_t)b * Sq + i;
  if (route == kRouteFast) {
    int2 r = sv.run_q[x];
    return TokMeta{r.x, r.y};
  }
  return TokMeta{sv.ids_q[x], sv.pos_q[x]};
}

__device__ inline TokMeta kv_meta(int route, const SegView& sv, int b, int Skv, int j) {
  if (route == kRouteDense || j >= Skv) return TokMeta{0, 0};
  size_t x = (size_t)b * Skv + j;
  if (route == kRouteFast) {
    int2 r = sv.run_kv[x];
    return TokMeta{r.x, r.y};
  }
  return TokMeta{sv.ids_kv[x], sv.pos_kv[x]};
}

// ------------------------------------------------------------ scheduling

// Maps the hardware workgroup index to a logical one.  Workgroups are
// handed to the 8 XCDs round robin; when the grid is a multiple of 8 the
// logical index gives each XCD one contiguous run of work (so workgroups that
// read the same K/V head share that XCD's L2).  reverse flips the order
// (tests: results must not depend on the schedule).
__device__ inline int logical_block(int nblocks, int reverse) {
  int i = blockIdx.x;
  int L = i;
  if ((nblocks & 7) == 0) L = (i & 7) * (nblocks >> 3) + (i >> 3);
  return reverse ? nblocks - 1 - L : L;
}

}  // namespace bps
