// kda_state.hip -- state pool init / load / store (pure bandwidth kernels).
//
// A state is one fp32 dk x dv matrix per (slot, head); the pool is
// [num_slots, H, dk, dv].  The memory these states carry is the whole cache
// of the operator (heqinghuang "From GPT2 to Kimi3, Explained", section 09:
// the returned state is the cache), so saving and restoring it is a plain copy
// by slot index.
#include "kda_common.h"

namespace kda {

namespace {

constexpr int kThreads = 256;

// Zero a contiguous range of float4.
__global__ __launch_bounds__(kThreads) void zero_kernel(float4* __restrict__ p, size_t n4) {
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * kThreads)
    p[i] = z;
}

// dense[i] <-> pool[slot(i)], one state = per4 float4 (H * dk * dv / 4).
template <bool kToPool>
__global__ __launch_bounds__(kThreads) void gather_scatter_kernel(
    float4* __restrict__ pool, int32_t num_slots, const int32_t* __restrict__ slots, int32_t n,
    float4* __restrict__ dense, size_t per4) {
  const size_t total = (size_t)n * per4;
  for (size_t e = blockIdx.x * (size_t)kThreads + threadIdx.x; e < total;
       e += (size_t)gridDim.x * kThreads) {
    const size_t i = e / per4, off = e - i * per4;
    const int32_t slot = slots ? slots[i] : (int32_t)i;
    if (slot < 0 || slot >= num_slots) continue;
    float4* ps = pool + (size_t)slot * per4 + off;
    float4* pd = dense + i * per4 + off;
    if (kToPool) *ps = *pd;
    else *pd = *ps;
  }
}

// dst[slot(i)] = src[i], or zero when src is NULL, for i < n; one state is per
// floats (slot i when slots is NULL; slots outside [0, num_slots) are skipped).
// Plain float accesses: the callers' buffers are only element-aligned.
__global__ __launch_bounds__(kThreads) void state_fill_kernel(float* __restrict__ dst,
                                                              int32_t num_slots,
                                                              const int32_t* __restrict__ slots,
                                                              int32_t n,
                                                              const float* __restrict__ src,
                                                              size_t per) {
  const size_t total = (size_t)n * per;
  for (size_t e = blockIdx.x * (size_t)kThreads + threadIdx.x; e < total;
       e += (size_t)gridDim.x * kThreads) {
    const size_t i = e / per, off = e - i * per;
    const int32_t slot = slots ? slots[i] : (int32_t)i;
    if (slot < 0 || slot >= num_slots) continue;
    dst[(size_t)slot * per + off] = src ? src[e] : 0.f;
  }
}

// S_out = M S_in + B for one (entry, head) and a block of kAffCols columns:
// the effect of a segment on its incoming state is affine, and composing it is
// the exchange step of context-parallel prefill (heqinghuang "From GPT2 to
// Kimi3, Explained", section 10: the state is the only thing one chunk passes to
// the next; a run of chunks passes it through a product of transition matrices
// plus the state written inside it).  fp32 FMAs in key order; the S_in block is
// staged in LDS, rows of M are read by all column lanes at once.
constexpr int kAffCols = 32;
__global__ __launch_bounds__(kThreads) void affine_kernel(const float* __restrict__ M,
                                                          const float* __restrict__ S_in,
                                                          const float* B, float* S_out, int dk,
                                                          int dv, int col_blocks) {
  extern __shared__ float sin_blk[];  // [dk][kAffCols]
  const int cb = blockIdx.x % col_blocks;
  const size_t eh = blockIdx.x / col_blocks;  // entry * H + head
  const int c0 = cb * kAffCols;
  const int ncols = min(kAffCols, dv - c0);
  const float* Sm = S_in + eh * (size_t)dk * dv;
  const float* Mm = M + eh * (size_t)dk * dk;
  for (int e = threadIdx.x; e < dk * kAffCols; e += kThreads) {
    const int r = e / kAffCols, c = e - r * kAffCols;
    sin_blk[e] = c < ncols ? Sm[(size_t)r * dv + c0 + c] : 0.f;
  }
  __syncthreads();
  const int c = threadIdx.x % kAffCols;
  for (int r = threadIdx.x / kAffCols; r < dk; r += kThreads / kAffCols) {
    float acc = 0.f;
    const float* mrow = Mm + (size_t)r * dk;
    for (int kk = 0; kk < dk; ++kk) acc = fmaf(mrow[kk], sin_blk[kk * kAffCols + c], acc);
    if (c < ncols) {
      const size_t i = eh * (size_t)dk * dv + (size_t)r * dv + c0 + c;
      S_out[i] = acc + B[i];
    }
  }
}

int grid_for(size_t n4) {
  size_t blocks = (n4 + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

kda_status_t launch_state_init(float* states, size_t n_floats, hipStream_t stream) {
  const size_t n4 = n_floats / 4;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n4)), dim3(kThreads), 0, stream,
                     reinterpret_cast<float4*>(states), n4);
  return check_launch("zero_kernel");
}

kda_status_t launch_state_fill(float* dst, int32_t num_slots, const int32_t* slots, int32_t n,
                               const float* src, size_t per_state_floats, hipStream_t stream) {
  hipLaunchKernelGGL(state_fill_kernel, dim3(grid_for((size_t)n * per_state_floats)),
                     dim3(kThreads), 0, stream, dst, num_slots, slots, n, src, per_state_floats);
  return check_launch("state_fill_kernel");
}

kda_status_t launch_state_affine(int32_t n, int H, int dk, int dv, const float* M,
                                 const float* S_in, const float* B, float* S_out,
                                 hipStream_t stream) {
  const int col_blocks = (dv + kAffCols - 1) / kAffCols;
  hipLaunchKernelGGL(affine_kernel, dim3((unsigned)((size_t)n * H * col_blocks)), dim3(kThreads),
                     (size_t)dk * kAffCols * sizeof(float), stream, M, S_in, B, S_out, dk, dv,
                     col_blocks);
  return check_launch("affine_kernel");
}

kda_status_t launch_state_copy(bool to_pool, float* states, int32_t num_slots,
                               const int32_t* slots, int32_t n, float* dense,
                               size_t per_state_floats, hipStream_t stream) {
  const size_t per4 = per_state_floats / 4;
  const int grid = grid_for((size_t)n * per4);
  if (to_pool)
    hipLaunchKernelGGL(gather_scatter_kernel<true>, dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<float4*>(states), num_slots, slots, n,
                       reinterpret_cast<float4*>(dense), per4);
  else
    hipLaunchKernelGGL(gather_scatter_kernel<false>, dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<float4*>(states), num_slots, slots, n,
                       reinterpret_cast<float4*>(dense), per4);
  return check_launch("gather_scatter_kernel");
}

}  // namespace kda
