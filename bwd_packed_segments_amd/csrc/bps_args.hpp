// Kernel argument blocks and launcher declarations shared by the host
// dispatcher (attn_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bps_common.hpp"

namespace bps {

struct Strides {
  int64_t b, t, h;   // elements
};

struct AttnShape {
  int B, Sq, Skv, Hq, Hkv;
  int causal;
  int reverse;       // reverse the workgroup schedule
  int has_meta;
  float scale;       // softmax scale (natural)
  float scale_log2;  // scale * log2(e)
};

// Attention variants (attn_fwd_ex / attn_bwd_ex).  Logits are
// x = scale * <q, k> + bias, soft-capped to softcap * tanh(x / softcap) when
// softcap > 0; the sink adds exp(sink[h]) to every query's softmax
// denominator.  Read only by the kernels instantiated with VAR = true.
struct VarView {
  const void* bias;      // [Bb, Hq, Sq, Skv] element type of q, contiguous; NULL: none
  int64_t bias_b;        // batch stride of bias in elements (0: one slab for every batch row)
  float softcap;         // 0: no soft-capping
  float cap_k;           // 2 log2(e) / softcap: exp2 argument of tanh
  float cap_l2;          // softcap * log2(e): tanh value -> base-2 logit
  float cap_inv;         // 1 / cap_l2
  const float* sink;     // [Hq] natural-log sink logits, or NULL
  float* ml_part;        // forward: [Hq][B][query tiles][4 waves] base-e maxima, or NULL
  void* dbias;           // backward: where dK/dV writes dLoss/dx, or NULL
  int dbias_f32;         // dbias is an fp32 array of per-batch-row partials
  int64_t dbias_b;       // batch stride of dbias in elements
  float* dsink_row;      // backward: [B, Hq, Sq] -exp(sink - LSE) * Delta, or NULL
};

struct FwdArgs {
  AttnShape s;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  Strides sq, sk, sv, so;
  SegView seg;
  VarView var;
};

struct BwdArgs {
  AttnShape s;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  Strides sq, sk, sv, so;
  float* delta;      // [B, Hq, Sq] workspace: rowsum(dO * O)
  float* lse2;       // [B, Hq, Sq] workspace: LSE * log2(e), +inf for empty rows
  // Fused backward (NULL: separate dK/dV and dQ kernels).  The dK/dV kernel
  // also writes, per (batch row, query head, key tile of 128, query block
  // of 32), the fp32 partial sum dS K over that key tile (unscaled) in MFMA
  // C layout, [Dqk / 32 column blocks][64 lanes][16]; the dQ phase sums the
  // partials of each query block over key tiles in ascending order.
  float* dqp;        // [B, Hq, ceil(Skv / 128), 2 ceil(Sq / 64), 32 Dqk] workspace
  SegView seg;
  VarView var;
  // Split dK/dV walks (bf16 kernels): with kv_split > 1, kv_split workgroups
  // share each key tile's walk over query tiles (contiguous, nearly equal
  // parts) and write fp32 partials of dK (unscaled) and dV, which a second
  // kernel adds up in split order.  Small grids (fewer than two workgroups
  // per CU) otherwise leave the time to the longest walk alone.
  int kv_split;      // 1: one workgroup per key tile, dK/dV written directly
  float* dkvp;       // [B, Hkv, ceil(Skv / 128), kv_split, 128 (Dqk + Dv)] workspace
};

struct SegMetaArgs {
  int B, Sq, Skv;
  int sides;          // 1: KV metadata are Q's; 2: separate KV metadata
  int check_eq;       // compare Q and KV metadata elementwise (side 0)
  int force_general;
  const int* ids[2];
  const int* pos_in[2];   // NULL: derive from ids
  int* pos_out[2];        // derived positions (when pos_in is NULL)
  int2* run[2];
  ChunkSum* sum[2];
  int nch[2];
  int* route;             // [B]
};

// Longest-walk-first tile orders of every batch row (qord, kord in seg).
struct TileOrderArgs {
  int B, Sq, Skv, causal;
  SegView seg;
  int* qord;   // [B, ceil(Sq / 128)]
  int* kord;   // [B, ceil(Skv / 128)]
};

struct MaskArgs {
  int B, Sq, Skv, causal, has_meta;
  SegView seg;
  uint8_t* mask;    // [B, Sq, Skv]
  int* route_rows;  // [B] or NULL
};

// One-GPU ring emulation (ring.hip).
struct RingMetaArgs {
  int B, Sq, Skv, cp;
  const int* ids[2];   // source [B, S] per side (Q, KV); NULL: id 1, position = index
  const int* pos[2];   // NULL with ids given: derived on the whole row
  int* ids_out[2];     // [cp][B][S / cp]
  int* pos_out[2];
};

struct RingLseArgs {
  int B, Hq, Sq, cp;
  const float* lse;    // [B, Hq, Sq]
  float* lse_out;      // [cp][B][Hq][Sq / cp]
};

struct RingMergeArgs {
  int B, Sq, Hq, Dv, cp;
  const void* o_parts;      // cp partial outputs with the layout of o
  size_t part_elems;        // elements between consecutive partials
  const float* lse_parts;   // [t][rank][B][Hq][Sq / cp]
  void* o;
  float* lse;               // [B, Hq, Sq]
  Strides so;
};

struct RingReduceArgs {
  int B, S, H, D, nparts;
  const void* parts;        // nparts partials with the layout of out
  size_t part_elems;
  void* out;
  Strides st;
};

hipError_t launch_ring_meta(const RingMetaArgs& a, hipStream_t st);
hipError_t launch_ring_lse_shards(const RingLseArgs& a, hipStream_t st);
hipError_t launch_ring_merge(int dtype_bf16, const RingMergeArgs& a, hipStream_t st);
hipError_t launch_ring_reduce(int dtype_bf16, const RingReduceArgs& a, hipStream_t st);

// Launchers (defined in the kernel translation units).  Each returns the
// result of hipGetLastError() after its launches.
hipError_t launch_seg_meta(const SegMetaArgs& a, hipStream_t st);
hipError_t launch_debug_mask(const MaskArgs& a, hipStream_t st);
// Longest-walk-first tile orders (after launch_seg_meta on the same stream).
hipError_t launch_tile_order(const TileOrderArgs& a, hipStream_t st);
// out[b] = route[b] for b < B (route NULL: kRouteDense everywhere).
hipError_t launch_route_rows(const int* route, int B, int* out, hipStream_t st);

// VAR / VM select the kernels that apply the variants of VarView (forward
// VM: 0 plain, 1 sink and max logit only, 2 bias or soft cap as well).
template <typename T, int DQK, int DV, int VM>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);
template <typename T, int DQK, int DV, bool VAR>
hipError_t launch_bwd_delta(const BwdArgs& a, hipStream_t st);
template <typename T, int DQK, int DV, bool VAR>
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t st);
template <typename T, int DQK, int DV, bool VAR>
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st);

// Variant reductions (variant.hip).
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st);
// max_logit[h] = max over the n partials ml_part[h * n ...] (-inf when n == 0).
hipError_t launch_max_logit_reduce(const float* ml_part, size_t n, int Hq, float* max_logit, hipStream_t st);
// dsink[h] = sum over b, i of rows[(b * Hq + h) * Sq + i], in a fixed order.
hipError_t launch_dsink_reduce(const float* rows, int B, int Hq, int Sq, float* dsink, hipStream_t st);
// out[e] = sum over b < B of parts[b * n + e] in order b = 0, 1, ..., converted to the element type.
hipError_t launch_dbias_reduce(int dtype_bf16, const float* parts, int B, size_t n, void* out, hipStream_t st);

}  // namespace bps
