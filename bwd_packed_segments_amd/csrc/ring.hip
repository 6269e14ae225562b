// Kernels of the one-GPU ring (context-parallel) emulation: shard-major
// segment metadata with global positions, the log-sum-exp merge of the ring
// steps' partial outputs, and the fixed-order sum of their partial
// gradients.
//
// The ring-attention backward on the maxdiffusion page (Summary and Key
// Features: custom ring attention backward) rotates K, V, dK and dV between
// devices and accumulates the local dQ; the TransformerEngine page on fused
// attention sharding (Changes 3) sends every rotated ring step down the
// general metadata path.  On one GPU the devices are emulated by shards of
// the token axis; these kernels do the parts of a ring step that are not
// attention itself.
#include "bps_args.hpp"

namespace bps {

// One workgroup per (batch row, side).  Writes ids and positions of the row
// into shard-major arrays out[shard][b][S / cp].  Without source ids every
// token gets id 1 and its index as position (so a causal position compare is
// the index compare); without source positions they are derived on the whole
// row: the offset of the token inside its run of equal ids.
__global__ void __launch_bounds__(256) ring_meta_kernel(RingMetaArgs a) {
  const int side = blockIdx.y;
  const int b = blockIdx.x;
  const int S = side == 0 ? a.Sq : a.Skv;
  const int len = S / a.cp;
  const int* ids = a.ids[side];
  const int* pos = a.pos[side];
  int* ids_out = a.ids_out[side];
  int* pos_out = a.pos_out[side];
  const size_t row = (size_t)b * S;
  auto out_index = [&](int i) { return ((size_t)(i / len) * a.B + b) * len + (i % len); };

  if (ids == nullptr || pos != nullptr) {
    for (int i = threadIdx.x; i < S; i += blockDim.x) {
      const size_t o = out_index(i);
      ids_out[o] = ids ? ids[row + i] : 1;
      pos_out[o] = ids ? pos[row + i] : i;
    }
    return;
  }
  // Derived positions: start(i) = max{ j <= i : j == 0 or ids[j] != ids[j-1] }
  // as a prefix max over contiguous chunks of the row, one chunk per thread.
  __shared__ int carry[256];
  const int T = blockDim.x;
  const int chunk = (S + T - 1) / T;
  const int c0 = min(S, (int)threadIdx.x * chunk);
  const int c1 = min(S, c0 + chunk);
  int local = -1;
  for (int i = c0; i < c1; ++i)
    if (i == 0 || ids[row + i] != ids[row + i - 1]) local = i;
  carry[threadIdx.x] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = -1;
    for (int t = 0; t < T; ++t) {
      const int v = carry[t];
      carry[t] = run;   // exclusive prefix max
      run = max(run, v);
    }
  }
  __syncthreads();
  int start = carry[threadIdx.x];
  for (int i = c0; i < c1; ++i) {
    if (i == 0 || ids[row + i] != ids[row + i - 1]) start = i;
    const size_t o = out_index(i);
    ids_out[o] = ids[row + i];
    pos_out[o] = i - start;
  }
}

// Copies LSE [B, Hq, Sq] into shard-major [cp][B][Hq][Sq / cp].
__global__ void __launch_bounds__(256) ring_lse_shards_kernel(RingLseArgs a) {
  const size_t n = (size_t)a.B * a.Hq * a.Sq;
  const int len = a.Sq / a.cp;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(x % a.Sq);
    const size_t bh = x / a.Sq;
    const int h = (int)(bh % a.Hq);
    const int b = (int)(bh / a.Hq);
    a.lse_out[(((size_t)(i / len) * a.B + b) * a.Hq + h) * len + (i % len)] = a.lse[x];
  }
}

// Merge of the ring steps' partial outputs for one (b, i, h) and 8 output
// features per thread: LSE = log sum_t exp(LSE_t), O = sum_t exp(LSE_t - LSE)
// O_t (a row no step attended keeps O = 0, LSE = -inf).  Partial t of O has
// the layout of O itself at o_parts + t * part_elems; partial LSEs are
// [t][rank][B][Hq][Sq / cp].
template <typename T>
__global__ void __launch_bounds__(256) ring_merge_kernel(RingMergeArgs a) {
  using E = Elem<T>;
  const int chunks = a.Dv / 8;
  const size_t n = (size_t)a.B * a.Sq * a.Hq * chunks;
  const int len = a.Sq / a.cp;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(x % chunks);
    size_t y = x / chunks;
    const int h = (int)(y % a.Hq);
    y /= a.Hq;
    const int i = (int)(y % a.Sq);
    const int b = (int)(y / a.Sq);
    const int r = i / len, il = i % len;
    float mx = -INFINITY;
    for (int t = 0; t < a.cp; ++t)
      mx = fmaxf(mx, a.lse_parts[((((size_t)t * a.cp + r) * a.B + b) * a.Hq + h) * len + il]);
    float sum = 0.f;
    if (mx != -INFINITY)
      for (int t = 0; t < a.cp; ++t)
        sum += expf(a.lse_parts[((((size_t)t * a.cp + r) * a.B + b) * a.Hq + h) * len + il] - mx);
    const float lse = mx == -INFINITY ? -INFINITY : mx + logf(sum);
    f32x8 acc{};
    const size_t off = (size_t)b * a.so.b + (size_t)i * a.so.t + (size_t)h * a.so.h + 8 * c;
    if (mx != -INFINITY) {
      for (int t = 0; t < a.cp; ++t) {
        const float lt = a.lse_parts[((((size_t)t * a.cp + r) * a.B + b) * a.Hq + h) * len + il];
        if (lt == -INFINITY) continue;
        const float wgt = expf(lt - lse);
        const typename E::F8 v = E::load8(static_cast<const T*>(a.o_parts) + t * a.part_elems + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wgt * (float)v[e];
      }
    }
    T* dst = static_cast<T*>(a.o) + off;
    const f32x4 lo{acc[0], acc[1], acc[2], acc[3]}, hi{acc[4], acc[5], acc[6], acc[7]};
    *reinterpret_cast<typename E::P4*>(dst) = E::cvt4(lo);
    *reinterpret_cast<typename E::P4*>(dst + 4) = E::cvt4(hi);
    if (c == 0) a.lse[((size_t)b * a.Hq + h) * a.Sq + i] = lse;
  }
}

// out = sum_t part_t in the order t = 0, 1, ..., accumulated in fp32; the
// parts have the layout of out at parts + t * part_elems.
template <typename T>
__global__ void __launch_bounds__(256) ring_reduce_kernel(RingReduceArgs a) {
  using E = Elem<T>;
  const int chunks = a.D / 8;
  const size_t n = (size_t)a.B * a.S * a.H * chunks;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(x % chunks);
    size_t y = x / chunks;
    const int h = (int)(y % a.H);
    y /= a.H;
    const int i = (int)(y % a.S);
    const int b = (int)(y / a.S);
    const size_t off = (size_t)b * a.st.b + (size_t)i * a.st.t + (size_t)h * a.st.h + 8 * c;
    f32x8 acc{};
    for (int t = 0; t < a.nparts; ++t) {
      const typename E::F8 v = E::load8(static_cast<const T*>(a.parts) + t * a.part_elems + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
    }
    T* dst = static_cast<T*>(a.out) + off;
    const f32x4 lo{acc[0], acc[1], acc[2], acc[3]}, hi{acc[4], acc[5], acc[6], acc[7]};
    *reinterpret_cast<typename E::P4*>(dst) = E::cvt4(lo);
    *reinterpret_cast<typename E::P4*>(dst + 4) = E::cvt4(hi);
  }
}

namespace {
unsigned grid_for(size_t n) {
  const size_t blocks = (n + 255) / 256;
  return (unsigned)(blocks < 65536 ? (blocks ? blocks : 1) : 65536);
}
}  // namespace

hipError_t launch_ring_meta(const RingMetaArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_meta_kernel, dim3((unsigned)a.B, 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ring_lse_shards(const RingLseArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.B * a.Hq * a.Sq;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_lse_shards_kernel, dim3(grid_for(n)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ring_merge(int dtype_bf16, const RingMergeArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.B * a.Sq * a.Hq * (a.Dv / 8);
  if (n == 0) return hipSuccess;
  if (dtype_bf16) hipLaunchKernelGGL(ring_merge_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(ring_merge_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ring_reduce(int dtype_bf16, const RingReduceArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.B * a.S * a.H * (a.D / 8);
  if (n == 0) return hipSuccess;
  if (dtype_bf16) hipLaunchKernelGGL(ring_reduce_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(ring_reduce_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace bps
