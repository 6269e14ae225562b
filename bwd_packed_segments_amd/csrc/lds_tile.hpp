// LDS tiles for the attention kernels (gfx950).
//
// A tile holds ROWS rows of D elements, row-major without padding.  Rows are
// split into 16-byte chunks and, for bf16, chunk c of row r is stored at
// chunk c ^ f(r) with f(r) = 4 (r % 4) + (r / 4) % 4 (inside each group of
// 16 chunks).  Two kinds of reads hit the same tile without bank conflicts:
//   * natural operand reads (ds_read_b128): 32 lanes read 16 bytes of 32
//     consecutive rows at the same logical chunk, which f spreads over all
//     banks;
//   * transposed operand reads (ds_read_b64_tr_b16, new in gfx950): each
//     16-lane group reads four rows times 32 bytes; f places the four rows'
//     chunk groups in different banks.
// The transposed read delivers, in every group of 16 lanes, element b of the
// 4-element rows addressed by lanes a, a+4, a+8 and a+12 to lane 4a + b
// (checked on the device with an in-bounds probe).  Pointing lane i of a
// group at tile[y + i / 4][x + 4 (i % 4)] therefore hands each lane four
// consecutive rows of one column: one MFMA A operand of a transposed tile
// in two reads.
//
// Tiles are filled straight from global memory with global_load_lds_dwordx4
// (16 bytes per lane, written at the wave's LDS base + 16 * lane), so no
// registers stage the data; the lane that owns physical slot s fetches the
// logical chunk that the swizzle puts there.  A tile with rows past the end
// of the sequence is filled through registers instead, with zeros for the
// missing rows.
#pragma once

#include "bps_common.hpp"

namespace bps {

#define BPS_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x4v __attribute__((__vector_size__(4 * sizeof(__bf16))));

template <typename T, int D>
struct TileFmt {
  static constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  static constexpr int NC = D / EPC;                // chunks per row
  static_assert(D % EPC == 0, "row must be whole chunks");

  // Physical chunk of logical chunk c in row r (an involution).
  __device__ static int swz(int r, int c) {
    if constexpr (sizeof(T) != 2) {
      return c;
    } else if constexpr (NC % 16 == 0) {
      return c ^ (4 * (r & 3) + ((r >> 2) & 3));
    } else if constexpr (NC == 8) {
      return c ^ (2 * (r & 3) + ((r >> 2) & 1));
    } else if constexpr (NC == 4) {
      // 64-byte rows (the fused backward's dS^T tile): transposed reads of 4
      // consecutive rows cover 256 contiguous bytes whatever f is; f = bits
      // 2-3 of the row halves the conflicts of column-wise 8-byte stores.
      return c ^ ((r >> 2) & 3);
    } else {
      static_assert(NC == 24, "unsupported row width");
      const int f = 4 * (r & 3) + ((r >> 2) & 3);
      return c < 16 ? (c ^ f) : (c ^ (f & 7));
    }
  }
  // Element offset of element e of row r.
  __device__ static int off(int r, int e) { return r * D + swz(r, e / EPC) * EPC + (e % EPC); }
};

// Natural operand fragment: 8 elements of row r starting at element e
// (e a multiple of 8).
template <typename T, int D>
__device__ inline typename Elem<T>::F8 frag_row(const T* tile, int r, int e) {
  using F = TileFmt<T, D>;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const typename Elem<T>::F8*>(tile + F::off(r, e));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(tile + F::off(r, e));
    const f32x4 b = *reinterpret_cast<const f32x4*>(tile + F::off(r, e + 4));
    return typename Elem<T>::F8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// Transposed operand fragment: lane (n, hf) gets tile[y0 + cmap(hf, e)][x0 + n]
// for e = 0..7, cmap(hf, e) = 8 (e / 4) + 4 hf + e % 4 (the k order of an
// MFMA C tile fed back as a B operand).
template <typename T, int D>
__device__ inline typename Elem<T>::F8 frag_tr(const T* tile, int x0, int y0, int lane) {
  using F = TileFmt<T, D>;
  if constexpr (sizeof(T) == 2) {
    const int G = lane >> 4;
    const int i = lane & 15;
    const int hf = G >> 1;
    const int x = x0 + 16 * (G & 1) + 4 * (i & 3);
    const int y = y0 + 4 * hf + (i >> 2);
    const BPS_LDS bf16x4v* p0 = (const BPS_LDS bf16x4v*)(tile + F::off(y, x));
    const BPS_LDS bf16x4v* p1 = (const BPS_LDS bf16x4v*)(tile + F::off(y + 8, x));
    const bf16x4v a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)p0);
    const bf16x4v b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BPS_LDS bf16x4v*)p1);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    const int n = lane & 31;
    const int hf = lane >> 5;
    typename Elem<T>::F8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[F::off(y0 + 8 * (e >> 2) + 4 * hf + (e & 3), x0 + n)];
    return v;
  }
}

// Raw buffer resource over a byte range starting at p (gfx9 format word 3).
__device__ inline __amdgpu_buffer_rsrc_t raw_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, -1, 0x00020000);
}

// Direct-to-LDS loads written as inline assembly.  Each lane's data lands
// at the wave's LDS base (M0) + lane * size.  The compiler does not see
// these as LDS writes, so it does not wait for them before every LDS read
// that follows (its alias analysis cannot tell the phase buffers apart);
// the kernel waits for them itself (vmcnt) before the barrier that
// publishes a buffer.  They write no registers.
// lds and soff must be wave-uniform (they are moved to scalar registers).
__device__ inline void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}
__device__ inline void lds_load4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
               : "memory");
}

// A workgroup-uniform pointer, held in scalar registers (the buffer
// resource of a scalar-operand load must be).
template <typename P>
__device__ inline const P* uniform_ptr(const P* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<const P*>(((uint64_t)hi << 32) | lo);
}

// Fills a [ROWS x D] tile from global memory rows base + r * row_stride.
// OFF32: lane offsets in 32-bit arithmetic (the caller guarantees
// ROWS * row_stride < 2^31 elements); a kernel short of registers keeps one
// register per load instead of a pair.
template <typename T, int ROWS, int D, int THREADS, bool OFF32 = false>
struct TileLoad {
  using F = TileFmt<T, D>;
  using E = Elem<T>;
  static constexpr int SLOTS = ROWS * F::NC;
  static constexpr int PER = SLOTS / THREADS;
  static_assert(SLOTS % THREADS == 0, "tile must split evenly over the workgroup");

  // All ROWS rows exist: direct global -> LDS loads (completion tracked by
  // vmcnt; wait with s_waitcnt before the barrier that publishes the tile).
  __device__ static void direct(const T* base, int64_t row_stride, T* tile, int tid) {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int s = x * THREADS + tid;
      const int r = s / F::NC;
      const int c = F::swz(r, s % F::NC);
      const T* g = OFF32 ? base + ((uint32_t)r * (uint32_t)row_stride + (uint32_t)(c * F::EPC))
                         : base + r * row_stride + c * F::EPC;
      T* wave_base = tile + (x * THREADS + (tid & ~63)) * F::EPC;
      __builtin_amdgcn_global_load_lds(g, (BPS_LDS void*)wave_base, 16, 0, 0);
    }
  }
  // Rows from nvalid on are zero: ordinary loads, then LDS stores.
  __device__ static void staged(const T* base, int64_t row_stride, int nvalid, T* tile, int tid) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int s = x * THREADS + tid;
      const int r = s / F::NC;
      const int c = F::swz(r, s % F::NC);
      u32x4v v = u32x4v{0u, 0u, 0u, 0u};
      if (r < nvalid)
        v = *reinterpret_cast<const u32x4v*>(OFF32 ? base + ((uint32_t)r * (uint32_t)row_stride + (uint32_t)(c * F::EPC))
                                                   : base + r * row_stride + c * F::EPC);
      *reinterpret_cast<u32x4v*>(tile + s * F::EPC) = v;
    }
  }
};

// The same tile through registers: load() issues the global loads (zeros for
// rows from nvalid on), store() writes the swizzled chunks to LDS later, so
// the loads overlap whatever runs in between.
template <typename T, int ROWS, int D, int THREADS>
struct TileRegs {
  using F = TileFmt<T, D>;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  static constexpr int PER = ROWS * F::NC / THREADS;
  static_assert((ROWS * F::NC) % THREADS == 0, "tile must split evenly over the workgroup");
  u32x4v r[PER];

  __device__ void load(const T* base, int64_t row_stride, int nvalid, int tid) {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int s = x * THREADS + tid;
      const int row = s / F::NC;
      const int c = F::swz(row, s % F::NC);
      r[x] = row < nvalid ? *reinterpret_cast<const u32x4v*>(base + row * row_stride + c * F::EPC)
                          : u32x4v{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(T* tile, int tid) const {
#pragma unroll
    for (int x = 0; x < PER; ++x) *reinterpret_cast<u32x4v*>(tile + (x * THREADS + tid) * F::EPC) = r[x];
  }
};

// Waits for this thread's outstanding global->LDS loads.
__device__ inline void wait_vm() { __builtin_amdgcn_s_waitcnt(0); }

// Waits until at most N vector memory operations of this thread are
// outstanding (they complete in issue order), leaving the N youngest in
// flight.  gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and
// lgkmcnt 11:8 (set to their maximum, i.e. not waited for).
template <int N>
__device__ inline void wait_vm_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace bps
