// Small kernels around the attention variants: zero fill of the dbias
// target, the per-head reductions of the maximum logit and of the sink
// gradient, and the fixed-order sum of per-batch-row dbias partials when one
// bias slab is shared by every batch row.
//
// The variants themselves are named, not defined, by the TransformerEngine
// pages ("[JAX] Align fused attn backward output gradient sharding ...",
// Changes 5 and Diagram: max-logit and score-mod cases, optional bias
// gradients; "[JAX] Make all jax attention calls use non-packed common
// calls": a linked change adding sink attention).  Every reduction here runs
// in one fixed order, so results are bitwise reproducible.
#include "bps_args.hpp"

namespace bps {

namespace {

unsigned grid_for(size_t n) {
  const size_t blocks = (n + 255) / 256;
  return (unsigned)(blocks < 65536 ? (blocks ? blocks : 1) : 65536);
}

// bytes is a multiple of 2; p is 16-byte aligned.
__global__ void __launch_bounds__(256) zero_fill_kernel(char* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t t0 = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  for (size_t x = t0; x < n16; x += stride) reinterpret_cast<uint4*>(p)[x] = uint4{0u, 0u, 0u, 0u};
  const size_t tail = (bytes - n16 * 16) / 2;
  if (t0 < tail) reinterpret_cast<unsigned short*>(p + n16 * 16)[t0] = 0;
}

// One workgroup per head.
__global__ void __launch_bounds__(256) max_logit_kernel(const float* part, size_t n, float* out) {
  __shared__ float red[256];
  const float* p = part + (size_t)blockIdx.x * n;
  float m = -INFINITY;
  for (size_t x = threadIdx.x; x < n; x += blockDim.x) m = fmaxf(m, p[x]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

// One workgroup per head: thread t adds the rows' terms t, t + 256, ... of
// the flattened (batch row, query) sequence in order, then a fixed tree.
__global__ void __launch_bounds__(256) dsink_kernel(const float* rows, int B, int Hq, int Sq, float* out) {
  __shared__ float red[256];
  const int h = blockIdx.x;
  const size_t n = (size_t)B * Sq;
  float acc = 0.f;
  for (size_t x = threadIdx.x; x < n; x += blockDim.x) {
    const size_t b = x / Sq, i = x % Sq;
    acc += rows[(b * Hq + h) * Sq + i];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[h] = red[0];
}

template <typename T>
__global__ void __launch_bounds__(256) dbias_reduce_kernel(const float* parts, int B, size_t n, T* out) {
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    float acc = 0.f;
    for (int b = 0; b < B; ++b) acc += parts[(size_t)b * n + x];
    out[x] = static_cast<T>(acc);
  }
}

}  // namespace

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(grid_for(bytes / 16 > 8 ? bytes / 16 : 8)), dim3(256), 0, st,
                     static_cast<char*>(p), bytes);
  return hipGetLastError();
}

hipError_t launch_max_logit_reduce(const float* ml_part, size_t n, int Hq, float* max_logit, hipStream_t st) {
  if (Hq <= 0) return hipSuccess;
  hipLaunchKernelGGL(max_logit_kernel, dim3((unsigned)Hq), dim3(256), 0, st, ml_part, n, max_logit);
  return hipGetLastError();
}

hipError_t launch_dsink_reduce(const float* rows, int B, int Hq, int Sq, float* dsink, hipStream_t st) {
  if (Hq <= 0) return hipSuccess;
  hipLaunchKernelGGL(dsink_kernel, dim3((unsigned)Hq), dim3(256), 0, st, rows, B, Hq, Sq, dsink);
  return hipGetLastError();
}

hipError_t launch_dbias_reduce(int dtype_bf16, const float* parts, int B, size_t n, void* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (dtype_bf16)
    hipLaunchKernelGGL(dbias_reduce_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, st, parts, B, n,
                       static_cast<bf16*>(out));
  else
    hipLaunchKernelGGL(dbias_reduce_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, parts, B, n,
                       static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace bps
