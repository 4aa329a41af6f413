// kda_chunk_small.hip -- chunkwise prefill in fp32 arithmetic for small heads.
//
// One workgroup per (sequence, head) walks the sequence chunk by chunk.  Inside
// a chunk of C tokens entering with state S (G = running sum of the log-gates
// inside the chunk, Gam_r = exp(G_r)):
//   A_kk[r,j] = beta_r sum_c k_r[c] k_j[c] exp(G_r[c] - G_j[c])   (j < r)
//   A_qk[r,j] =        sum_c q_r[c] k_j[c] exp(G_r[c] - G_j[c])   (j <= r)
//   T = (I + A_kk)^-1                       (forward substitution)
//   U = T Diag(beta) (V - (K*Gam) S)        the corrected values of the chunk
//   O = (Q*Gam) S + A_qk U                  state read + in-chunk attention
//   S <- Diag(Gam_C) S + (K*exp(G_C - G))^T U
// This is the within-chunk triangular system of engineermaxxing "From GPT-2 to
// Kimi K3", ch. 04e (chunked delta rule, forward substitution) with the running
// per-channel decay products folded through it, which heqinghuang "From GPT2
// to Kimi3, Explained", section 11 describes for the gated rule.  Unrolling the
// recurrence across the chunk gives exactly these formulas, so the result is
// the sequential rule re-ordered, not an approximation.
//
// Everything is fp32 on the vector ALUs with the chunk staged in LDS: this path
// serves the fp32 contract (1e-4 relative) and small heads, where launch
// latency dominates.  A partial last chunk is padded with neutral tokens
// (q = k = v = 0, beta = 0, g = 0), which leave state and outputs unchanged.
//
// Variants (flags): a scalar gate per (token, head) is staged as the same
// value on every channel; without a gate G = 0; the additive write (u = v)
// drops the correction, so A_kk = 0 (T = I) and the right-hand side is V.
#include "kda_common.h"

namespace kda {

namespace {

constexpr int kSmallThreads = 256;

template <int D, int C, typename IO>
__global__ __launch_bounds__(kSmallThreads) void chunk_small_kernel(
    const int32_t* __restrict__ cu, int32_t T, const IO* __restrict__ q,
    const IO* __restrict__ k, const IO* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float* __restrict__ states, int32_t num_slots,
    const int32_t* __restrict__ slots, uint32_t flags, IO* __restrict__ o, int H) {
  __shared__ float Qs[C][D];   // q, later q * Gam
  __shared__ float Ks[C][D];   // k, later k * exp(G_C - G)
  __shared__ float Vs[C][D];   // v, later beta (v - (k*Gam) S)
  __shared__ float Gs[C][D];   // cumulative log-gate, later k*Gam, later U
  __shared__ float Ss[D][D];   // running state
  __shared__ float Akk[C][C], Aqk[C][C], Tm[C][C];
  __shared__ float bs[C], glast[D];

  const int n = blockIdx.x / H;
  const int h = blockIdx.x - n * H;
  const int tid = threadIdx.x;
  const int start = clamp_tok(cu[n], T);
  int end = clamp_tok(cu[n + 1], T);
  if (end < start) end = start;
  const int slot = slots ? slots[n] : n;
  const bool slot_ok = slot >= 0 && slot < num_slots && states != nullptr;
  float* Sg = slot_ok ? states + ((size_t)slot * H + h) * (size_t)(D * D) : nullptr;

  for (int e = tid; e < D * D; e += kSmallThreads)
    Ss[e / D][e % D] = (slot_ok && (flags & KDA_READ_INITIAL_STATE)) ? Sg[e] : 0.f;

  const bool gate_none = flags & KDA_GATE_NONE, gate_scalar = flags & KDA_GATE_SCALAR;
  const bool additive = flags & KDA_ADDITIVE;
  for (int t0 = start; t0 < end; t0 += C) {
    const int c = min(C, end - t0);
    __syncthreads();
    for (int e = tid; e < C * D; e += kSmallThreads) {
      const int r = e / D, d = e % D;
      const bool ok = r < c;
      const size_t gi = ((size_t)(t0 + r) * H + h) * D + d;
      Qs[r][d] = ok ? io_traits<IO>::load(q, gi) : 0.f;
      Ks[r][d] = ok ? io_traits<IO>::load(k, gi) : 0.f;
      Vs[r][d] = ok ? io_traits<IO>::load(v, gi) : 0.f;
      Gs[r][d] = ok && !gate_none ? (gate_scalar ? g[(size_t)(t0 + r) * H + h] : g[gi]) : 0.f;
    }
    for (int r = tid; r < C; r += kSmallThreads)
      bs[r] = r < c ? (additive ? 1.f : beta[(size_t)(t0 + r) * H + h]) : 0.f;
    __syncthreads();

    // running sum of the log-gates along the chunk, per key channel
    for (int d = tid; d < D; d += kSmallThreads) {
      float run = 0.f;
      for (int r = 0; r < C; ++r) { run += Gs[r][d]; Gs[r][d] = run; }
      glast[d] = run;
    }
    __syncthreads();

    // gated Gram products inside the chunk
    for (int p = tid; p < C * C; p += kSmallThreads) {
      const int r = p / C, j = p % C;
      float kk = 0.f, qk = 0.f;
      if (j <= r) {
        for (int d = 0; d < D; ++d) {
          const float e = fast_exp(Gs[r][d] - Gs[j][d]);
          const float kj = Ks[j][d] * e;
          kk += Ks[r][d] * kj;
          qk += Qs[r][d] * kj;
        }
      }
      Akk[r][j] = j < r && !additive ? bs[r] * kk : 0.f;
      Aqk[r][j] = qk;
    }
    __syncthreads();

    // T = (I + A_kk)^-1 by forward substitution, one column per thread
    for (int j = tid; j < C; j += kSmallThreads) {
      for (int i = 0; i < C; ++i) {
        float x;
        if (i < j) x = 0.f;
        else if (i == j) x = 1.f;
        else {
          x = 0.f;
          for (int m = j; m < i; ++m) x -= Akk[i][m] * Tm[m][j];
        }
        Tm[i][j] = x;
      }
    }
    // gate the operands: q*Gam, k*Gam (into Gs), k*exp(G_C - G) (into Ks)
    for (int e = tid; e < C * D; e += kSmallThreads) {
      const int r = e / D, d = e % D;
      const float G = Gs[r][d];
      const float gam = fast_exp(G);
      const float kv = Ks[r][d];
      Qs[r][d] *= gam;
      Gs[r][d] = kv * gam;
      Ks[r][d] = kv * fast_exp(glast[d] - G);
    }
    __syncthreads();

    // right-hand side beta (v - (k*Gam) S), in place of v
    for (int e = tid; e < C * D; e += kSmallThreads) {
      const int r = e / D, col = e % D;
      float acc = 0.f;
      if (!additive) {
        for (int d = 0; d < D; ++d) acc += Gs[r][d] * Ss[d][col];
        Vs[r][col] = bs[r] * (Vs[r][col] - acc);
      }
    }
    __syncthreads();

    // U = T rhs, in place of k*Gam
    for (int e = tid; e < C * D; e += kSmallThreads) {
      const int r = e / D, col = e % D;
      float acc = 0.f;
      for (int j = 0; j <= r; ++j) acc += Tm[r][j] * Vs[j][col];
      Gs[r][col] = acc;
    }
    __syncthreads();

    // outputs: state read + in-chunk attention over the corrected values
    for (int e = tid; e < c * D; e += kSmallThreads) {
      const int r = e / D, col = e % D;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc += Qs[r][d] * Ss[d][col];
      for (int j = 0; j <= r; ++j) acc += Aqk[r][j] * Gs[j][col];
      io_traits<IO>::store(o, ((size_t)(t0 + r) * H + h) * D + col, acc);
    }
    __syncthreads();

    // fold the chunk into the state
    for (int e = tid; e < D * D; e += kSmallThreads) {
      const int d = e / D, col = e % D;
      float acc = fast_exp(glast[d]) * Ss[d][col];
      for (int j = 0; j < C; ++j) acc += Ks[j][d] * Gs[j][col];
      Ss[d][col] = acc;
    }
  }
  __syncthreads();
  if (slot_ok && (flags & KDA_WRITE_FINAL_STATE))
    for (int e = tid; e < D * D; e += kSmallThreads) Sg[e] = Ss[e / D][e % D];
}

template <int D, int C, typename IO>
kda_status_t launch_dc(int32_t T, int32_t N, const int32_t* cu, const void* q, const void* k,
                       const void* v, const float* g, const float* beta, float* states,
                       int32_t num_slots, const int32_t* slots, uint32_t flags, void* o, int H,
                       hipStream_t stream) {
  hipLaunchKernelGGL((chunk_small_kernel<D, C, IO>), dim3((unsigned)N * H), dim3(kSmallThreads),
                     0, stream, cu, T, static_cast<const IO*>(q), static_cast<const IO*>(k),
                     static_cast<const IO*>(v), g, beta, states, num_slots, slots, flags,
                     static_cast<IO*>(o), H);
  return check_launch("chunk_small_kernel");
}

template <typename IO>
kda_status_t launch_io(int d, int C, int32_t T, int32_t N, const int32_t* cu, const void* q,
                       const void* k, const void* v, const float* g, const float* beta,
                       float* states, int32_t num_slots, const int32_t* slots, uint32_t flags,
                       void* o, int H, hipStream_t s) {
#define KDA_SMALL_CASE(DD, CC)                                                               \
  if (d == DD && C == CC)                                                                    \
    return launch_dc<DD, CC, IO>(T, N, cu, q, k, v, g, beta, states, num_slots, slots, flags, \
                                 o, H, s);
  KDA_SMALL_CASE(16, 16) KDA_SMALL_CASE(16, 32) KDA_SMALL_CASE(16, 64)
  KDA_SMALL_CASE(32, 16) KDA_SMALL_CASE(32, 32) KDA_SMALL_CASE(32, 64)
  KDA_SMALL_CASE(64, 16) KDA_SMALL_CASE(64, 32) KDA_SMALL_CASE(64, 64)
  KDA_SMALL_CASE(128, 16) KDA_SMALL_CASE(128, 32)
#undef KDA_SMALL_CASE
  return KDA_ERR_UNSUPPORTED;
}

}  // namespace

bool chunk_small_supported(int dk, int dv, int chunk) {
  if (dk != dv) return false;
  if (dk == 16 || dk == 32 || dk == 64) return chunk == 16 || chunk == 32 || chunk == 64;
  if (dk == 128) return chunk == 16 || chunk == 32;
  return false;
}

kda_status_t launch_chunk_small(const kda_shape_t* sh, int32_t chunk, int32_t T, int32_t N,
                                const int32_t* cu, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, float* states,
                                int32_t num_slots, const int32_t* slots, uint32_t flags, void* o,
                                hipStream_t stream) {
  if (sh->io_dtype == KDA_BF16)
    return launch_io<uint16_t>(sh->dk, chunk, T, N, cu, q, k, v, g, beta, states, num_slots,
                               slots, flags, o, sh->num_heads, stream);
  return launch_io<float>(sh->dk, chunk, T, N, cu, q, k, v, g, beta, states, num_slots, slots,
                          flags, o, sh->num_heads, stream);
}

}  // namespace kda
