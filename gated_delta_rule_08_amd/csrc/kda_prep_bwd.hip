// kda_prep_bwd.hip -- the backward from raw projections: the input preparation
// (q, k = normalize(SiLU(.)), floored log-sigmoid gate, sigmoid write strength;
// heqinghuang "From GPT2 to Kimi3, Explained", section 09; engineermaxxing
// "From GPT-2 to Kimi K3", ch. 06b) materialised for the chunked backward, and
// the chain rule of those maps applied to its gradients:
//   y = x / max(|x|, 1e-12), x = silu(z):  dx = (dy - y (y.dy)) / |x| (I / 1e-12 below
//   the floor), dz = dx * s (1 + z (1 - s)), s = sigmoid(z);
//   g = max(log sigmoid(a), g_min):  da = dg * sigmoid(-a) where the floor is not taken;
//   beta = sigmoid(b):  db = dbeta * s (1 - s).
// One wave per (token, head) row of d = 128 channels, two channels per lane.
#include "kda_common.h"

namespace kda {

kda_status_t launch_chunk_mfma_bwd(const kda_shape_t* sh, int32_t T, int32_t N, const int32_t* cu,
                                   const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* states, int32_t num_slots,
                                   const int32_t* slots, uint32_t flags, const void* d_o,
                                   const float* d_final, void* dq, void* dk, void* dv, float* dg,
                                   float* dbeta, float* d_initial, void* workspace,
                                   hipStream_t stream);
size_t chunk_mfma_bwd_workspace_bytes(int H, int32_t T, int32_t N);

namespace {

constexpr int kPD = 128;          // channels per row
constexpr int kRowsPerBlock = 4;  // one wave per row
constexpr int kGateChannel = 0, kGateScalar = 1, kGateNone = 2;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float lo_f(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_f(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

template <int kGate, bool kAdd>
__global__ __launch_bounds__(64 * kRowsPerBlock) void prepare_kernel(
    int64_t rows, const uint16_t* __restrict__ q_raw, const uint16_t* __restrict__ k_raw,
    const uint16_t* __restrict__ a_raw, const uint16_t* __restrict__ b_raw, float gate_min,
    uint16_t* __restrict__ q, uint16_t* __restrict__ k, float* __restrict__ g,
    float* __restrict__ beta) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const size_t i = (size_t)row * kPD + 2 * lane;
  {
    const uint32_t r = *reinterpret_cast<const uint32_t*>(q_raw + i);
    const float x0 = silu(lo_f(r)), x1 = silu(hi_f(r));
    const float inv = inv_norm(wave_sum(x0 * x0 + x1 * x1));
    *reinterpret_cast<uint32_t*>(q + i) = pack2(x0 * inv, x1 * inv);
  }
  {
    const uint32_t r = *reinterpret_cast<const uint32_t*>(k_raw + i);
    const float x0 = silu(lo_f(r)), x1 = silu(hi_f(r));
    const float inv = inv_norm(wave_sum(x0 * x0 + x1 * x1));
    *reinterpret_cast<uint32_t*>(k + i) = pack2(x0 * inv, x1 * inv);
  }
  if (kGate == kGateChannel) {
    const uint32_t r = *reinterpret_cast<const uint32_t*>(a_raw + i);
    *reinterpret_cast<float2*>(g + i) = make_float2(fmaxf(log_sigmoid(lo_f(r)), gate_min),
                                                    fmaxf(log_sigmoid(hi_f(r)), gate_min));
  } else if (kGate == kGateScalar) {
    if (lane == 0) g[row] = fmaxf(log_sigmoid(bf16_to_f32(a_raw[row])), gate_min);
  }
  if (!kAdd && lane == 0) beta[row] = sigmoid(bf16_to_f32(b_raw[row]));
}

// dz for one row: the normaliser's projection, then SiLU's derivative
__device__ __forceinline__ void norm_silu_bwd(const uint16_t* raw, const uint16_t* dy, uint16_t* dz,
                                              size_t i) {
  const uint32_t r = *reinterpret_cast<const uint32_t*>(raw + i);
  const uint32_t d = *reinterpret_cast<const uint32_t*>(dy + i);
  const float z0 = lo_f(r), z1 = hi_f(r);
  const float s0 = sigmoid(z0), s1 = sigmoid(z1);
  const float x0 = z0 * s0, x1 = z1 * s1;
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float inv = inv_norm(ss);
  const float y0 = x0 * inv, y1 = x1 * inv, d0 = lo_f(d), d1 = hi_f(d);
  const float dot = ss > 1e-24f ? wave_sum(y0 * d0 + y1 * d1) : 0.f;  // uniform branch
  const float dx0 = (d0 - y0 * dot) * inv, dx1 = (d1 - y1 * dot) * inv;
  *reinterpret_cast<uint32_t*>(dz + i) =
      pack2(dx0 * s0 * (1.f + z0 * (1.f - s0)), dx1 * s1 * (1.f + z1 * (1.f - s1)));
}

template <int kGate, bool kAdd>
__global__ __launch_bounds__(64 * kRowsPerBlock) void prepare_bwd_kernel(
    int64_t rows, const uint16_t* __restrict__ q_raw, const uint16_t* __restrict__ k_raw,
    const uint16_t* __restrict__ a_raw, const uint16_t* __restrict__ b_raw, float gate_min,
    const uint16_t* __restrict__ dq, const uint16_t* __restrict__ dk, const float* __restrict__ dg,
    const float* __restrict__ dbeta, uint16_t* __restrict__ dq_raw, uint16_t* __restrict__ dk_raw,
    uint16_t* __restrict__ da_raw, uint16_t* __restrict__ db_raw) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const size_t i = (size_t)row * kPD + 2 * lane;
  norm_silu_bwd(q_raw, dq, dq_raw, i);
  norm_silu_bwd(k_raw, dk, dk_raw, i);
  if (kGate == kGateChannel) {
    const uint32_t r = *reinterpret_cast<const uint32_t*>(a_raw + i);
    const float2 d = *reinterpret_cast<const float2*>(dg + i);
    const float a0 = lo_f(r), a1 = hi_f(r);
    const float p0 = log_sigmoid(a0) >= gate_min ? sigmoid(-a0) : 0.f;
    const float p1 = log_sigmoid(a1) >= gate_min ? sigmoid(-a1) : 0.f;
    *reinterpret_cast<uint32_t*>(da_raw + i) = pack2(d.x * p0, d.y * p1);
  } else if (kGate == kGateScalar) {
    if (lane == 0) {
      const float a = bf16_to_f32(a_raw[row]);
      da_raw[row] = f32_to_bf16(log_sigmoid(a) >= gate_min ? dg[row] * sigmoid(-a) : 0.f);
    }
  }
  if (!kAdd && lane == 0) {
    const float s = sigmoid(bf16_to_f32(b_raw[row]));
    db_raw[row] = f32_to_bf16(dbeta[row] * s * (1.f - s));
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace past the backward's own: prepared q, k (bf16), g, beta (fp32) and the
// gradients of the prepared inputs (dq, dk bf16; dg, dbeta fp32).
struct RawWs {
  uint16_t* q;
  uint16_t* k;
  float* g;
  float* beta;
  uint16_t* dq;
  uint16_t* dk;
  float* dg;
  float* dbeta;
};

size_t raw_extra_bytes(int H, int32_t T) {
  const size_t rows = (size_t)T * H;
  return 2 * align256(rows * kPD * 2) + align256(rows * kPD * 4) + align256(rows * 4) +
         2 * align256(rows * kPD * 2) + align256(rows * kPD * 4) + align256(rows * 4);
}

RawWs carve_raw(void* base, int H, int32_t T) {
  const size_t rows = (size_t)T * H;
  uint8_t* p = static_cast<uint8_t*>(base);
  RawWs r;
  r.q = reinterpret_cast<uint16_t*>(p); p += align256(rows * kPD * 2);
  r.k = reinterpret_cast<uint16_t*>(p); p += align256(rows * kPD * 2);
  r.g = reinterpret_cast<float*>(p); p += align256(rows * kPD * 4);
  r.beta = reinterpret_cast<float*>(p); p += align256(rows * 4);
  r.dq = reinterpret_cast<uint16_t*>(p); p += align256(rows * kPD * 2);
  r.dk = reinterpret_cast<uint16_t*>(p); p += align256(rows * kPD * 2);
  r.dg = reinterpret_cast<float*>(p); p += align256(rows * kPD * 4);
  r.dbeta = reinterpret_cast<float*>(p);
  return r;
}

template <int kGate, bool kAdd>
kda_status_t launch_raw_pair(bool forward, int64_t rows, const void* q_raw, const void* k_raw,
                             const void* a_raw, const void* b_raw, float gate_min, const RawWs& r,
                             void* dq_raw, void* dk_raw, void* da_raw, void* db_raw,
                             hipStream_t stream) {
  const unsigned grid = (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const uint16_t* qr = static_cast<const uint16_t*>(q_raw);
  const uint16_t* kr = static_cast<const uint16_t*>(k_raw);
  const uint16_t* ar = static_cast<const uint16_t*>(a_raw);
  const uint16_t* br = static_cast<const uint16_t*>(b_raw);
  if (forward)
    hipLaunchKernelGGL((prepare_kernel<kGate, kAdd>), dim3(grid), dim3(64 * kRowsPerBlock), 0,
                       stream, rows, qr, kr, ar, br, gate_min, r.q, r.k, r.g, r.beta);
  else
    hipLaunchKernelGGL((prepare_bwd_kernel<kGate, kAdd>), dim3(grid), dim3(64 * kRowsPerBlock), 0,
                       stream, rows, qr, kr, ar, br, gate_min, r.dq, r.dk, r.dg, r.dbeta,
                       static_cast<uint16_t*>(dq_raw), static_cast<uint16_t*>(dk_raw),
                       static_cast<uint16_t*>(da_raw), static_cast<uint16_t*>(db_raw));
  return check_launch(forward ? "prepare_kernel" : "prepare_bwd_kernel");
}

kda_status_t launch_raw(uint32_t flags, bool forward, int64_t rows, const void* q_raw,
                        const void* k_raw, const void* a_raw, const void* b_raw, float gate_min,
                        const RawWs& r, void* dq_raw, void* dk_raw, void* da_raw, void* db_raw,
                        hipStream_t s) {
  const bool add = flags & KDA_ADDITIVE;
#define KDA_RAW(G, A) \
  launch_raw_pair<G, A>(forward, rows, q_raw, k_raw, a_raw, b_raw, gate_min, r, dq_raw, dk_raw, da_raw, db_raw, s)
  if (flags & KDA_GATE_SCALAR) return add ? KDA_RAW(kGateScalar, true) : KDA_RAW(kGateScalar, false);
  if (flags & KDA_GATE_NONE) return add ? KDA_RAW(kGateNone, true) : KDA_RAW(kGateNone, false);
  return add ? KDA_RAW(kGateChannel, true) : KDA_RAW(kGateChannel, false);
#undef KDA_RAW
}

}  // namespace

size_t chunk_mfma_bwd_raw_workspace_bytes(int H, int32_t T, int32_t N) {
  return chunk_mfma_bwd_workspace_bytes(H, T, N) + raw_extra_bytes(H, T);
}

kda_status_t launch_chunk_mfma_bwd_raw(const kda_shape_t* sh, int32_t T, int32_t N,
                                       const int32_t* cu, const void* q_raw, const void* k_raw,
                                       const void* v, const void* gate_logits,
                                       const void* beta_logits, float gate_min,
                                       const float* states, int32_t num_slots,
                                       const int32_t* slots, uint32_t flags, const void* d_o,
                                       const float* d_final, void* dq_raw, void* dk_raw, void* dv,
                                       void* dgate_logits, void* dbeta_logits, float* d_initial,
                                       void* workspace, hipStream_t stream) {
  const int H = sh->num_heads;
  const int64_t rows = (int64_t)T * H;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  const RawWs r = carve_raw(base + chunk_mfma_bwd_workspace_bytes(H, T, N), H, T);
  kda_status_t st = launch_raw(flags, true, rows, q_raw, k_raw, gate_logits, beta_logits, gate_min,
                               r, nullptr, nullptr, nullptr, nullptr, stream);
  if (st != KDA_OK) return st;
  const bool none = flags & KDA_GATE_NONE, add = flags & KDA_ADDITIVE;
  st = launch_chunk_mfma_bwd(sh, T, N, cu, r.q, r.k, v, none ? nullptr : r.g, add ? nullptr : r.beta,
                             states, num_slots, slots, flags, d_o, d_final, r.dq, r.dk, dv,
                             none ? nullptr : r.dg, add ? nullptr : r.dbeta, d_initial, workspace,
                             stream);
  if (st != KDA_OK) return st;
  return launch_raw(flags, false, rows, q_raw, k_raw, gate_logits, beta_logits, gate_min, r,
                    dq_raw, dk_raw, dgate_logits, dbeta_logits, stream);
}

}  // namespace kda
