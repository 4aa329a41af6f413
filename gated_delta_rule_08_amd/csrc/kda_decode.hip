// kda_decode.hip -- one decode step of the gated delta rule against resident states.
//
// Per (sequence b, head h), with S the resident fp32 dk x dv state:
//   Sbar = Diag(exp(g)) S            fade each key channel (row of S)
//   w    = Sbar^T k,  y = Sbar^T q    two reads of the faded state
//   u    = beta (v - w)               the correction
//   S    = Sbar + k u^T               written back in place
//   o    = S^T q = y + (k . q) u      read after the write
// (dev.to "From GPT-2 to Kimi K3", blocks 4-5: fade, read, correct against the
// faded state, one retention factor per key channel; heqinghuang "From GPT2 to
// Kimi3, Explained", section 09: output read after the write.)
//
// Variants (flags, uniform per launch): a scalar gate per (sequence, head)
// (Gated DeltaNet), no gate (DeltaNet), and the additive write u = v without
// the correction (gated linear attention): engineermaxxing ch. 05c and 02g.
//
// The step is a streaming read-modify-write of the state: each state is read
// from HBM once and written once, and the token vectors are tiny, so the kernel
// is bound by HBM bandwidth (engineermaxxing ch. 02b: a decode step reads the
// d x d state and writes it back).  Mapping: one workgroup per (b, h) and
// slice of DVW state columns (the columns of S evolve independently given k,
// q, beta and the gate, and the reductions run over rows, so slices need no
// exchange; two 64-column slices per state at d = 128 stream best); thread
// (row group rg, column quad cq) keeps rows rg, rg + RG, ... of columns
// 4cq .. 4cq+3 of the slice in registers, so every wave load instruction
// covers whole row segments (coalesced 16-byte accesses).  The reductions over
// key channels combine the row groups through LDS.
#include "kda_common.h"

namespace kda {

namespace {

// kRaw: q and k are raw projections (SiLU, then unit length), the gate and the
// write strength are bf16 logits (log-decay = max(log sigmoid, gate_min),
// beta = sigmoid): the input preparation fused into the step.
//
// kPersist: the grid is a fixed number of workgroups that walk the items (b, h,
// column slice) with a stride of the grid size, and each issues the next item's
// state loads before it works on the current one, so that its reads of item
// i + 1 overlap its reduction and writes of item i.  On the MI355X this form,
// with two waves per SIMD (two workgroups per CU resident), streams the state
// faster than one item per workgroup at a higher occupancy: the number of
// concurrent read streams, not latency hiding, sets the rate.
template <int DK, int DV, int BLOCK, typename IO, int DVW = DV, bool kRaw = false,
          bool kPersist = false>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(kPersist ? 2 : 1, kPersist ? 2 : 8)))
void decode_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const void* __restrict__ gp, const void* __restrict__ bp, float gate_min,
    float* __restrict__ states, int32_t num_slots, const int32_t* __restrict__ slots,
    uint32_t flags, IO* __restrict__ o, int H, int items) {
  const float* g = static_cast<const float*>(gp);
  const float* beta = static_cast<const float*>(bp);
  const uint16_t* g16 = static_cast<const uint16_t*>(gp);
  const uint16_t* b16 = static_cast<const uint16_t*>(bp);
  constexpr int NCQ = DVW / 4;     // column quads of this workgroup
  constexpr int RG = BLOCK / NCQ;  // row groups
  constexpr int RPT = DK / RG;     // rows per thread
  static_assert(DV % 4 == 0 && BLOCK % NCQ == 0 && DK % RG == 0, "bad decode tiling");
  static_assert(BLOCK >= DK && BLOCK >= DVW, "one token element per thread");
  constexpr int NSPLIT = DV / DVW;

  const int tid = threadIdx.x;
  const int cq = tid % NCQ;
  const int rg = tid / NCQ;
  const bool gate_none = flags & KDA_GATE_NONE, gate_scalar = flags & KDA_GATE_SCALAR;
  const bool additive = flags & KDA_ADDITIVE;

  __shared__ float ks[DK], qs[DK], as[DK], vs[DV], us[DV];
  __shared__ float4 wred[RG][NCQ];
  __shared__ float4 yred[RG][NCQ];
  __shared__ float kq_sh;

  // state slice of an item (nullptr when its slot is out of range: skipped)
  auto slice = [&](int it) -> float* {
    const int bh = it / NSPLIT, b = bh / H, h = bh - b * H;
    const int slot = slots ? slots[b] : b;
    if (slot < 0 || slot >= num_slots) return nullptr;
    return states + ((size_t)slot * H + h) * (size_t)(DK * DV) + (it - bh * NSPLIT) * DVW;
  };
  auto load_state = [&](const float* S, f32x4_t* s) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      s[i] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4_t*>(S + (size_t)(rg + RG * i) * DV + 4 * cq));
  };

  int item = blockIdx.x;
  f32x4_t s[RPT], sn[RPT];
  float* S = item < items ? slice(item) : nullptr;
  if (S) load_state(S, s);  // 1. the state loads first (the only large traffic)
  for (; item < items; item += gridDim.x) {
    const int bh = item / NSPLIT;
    const int c_base = (item - bh * NSPLIT) * DVW;
    const int nxt = item + gridDim.x;
    float* Sn = kPersist && nxt < items ? slice(nxt) : nullptr;
    if (S) {  // uniform across the workgroup
      // 2. this item's token vectors, issued before the next item's state loads so
      // that waiting for them does not wait for those
      const size_t tk = (size_t)bh * DK, tv = (size_t)bh * DV;
      float kv = 0.f, qv = 0.f, gv = 0.f, vv = 0.f;
      if (tid < DK) {
        kv = io_traits<IO>::load(k, tk + tid);
        qv = io_traits<IO>::load(q, tk + tid);
        const size_t gi = gate_scalar ? (size_t)bh : tk + tid;
        gv = gate_none ? 0.f : kRaw ? bf16_to_f32(g16[gi]) : g[gi];
      }
      if (tid < DVW) vv = io_traits<IO>::load(v, tv + c_base + tid);
      if (Sn) load_state(Sn, sn);
      if (tid < DK) {
        ks[tid] = kRaw ? silu(kv) : kv;
        qs[tid] = kRaw ? silu(qv) : qv;
        as[tid] = gate_none ? 1.f
                : kRaw      ? fast_exp(fmaxf(log_sigmoid(gv), gate_min))
                            : fast_exp(gv);
      }
      if (tid < DVW) vs[tid] = vv;
      __syncthreads();
      if (kRaw) {  // unit-length q and k (the first wave), seen by all after the barrier
        if (tid < 64) {
          float sk = 0.f, sq = 0.f;
          for (int i = tid; i < DK; i += 64) { sk += ks[i] * ks[i]; sq += qs[i] * qs[i]; }
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) {
            sk += __shfl_xor(sk, off, 64);
            sq += __shfl_xor(sq, off, 64);
          }
          const float ik = inv_norm(sk), iq = inv_norm(sq);
          for (int i = tid; i < DK; i += 64) { ks[i] *= ik; qs[i] *= iq; }
        }
        __syncthreads();
      }

      // k . q, reduced by the first wave
      if (tid < 64) {
        float p = 0.f;
        for (int i = tid; i < DK; i += 64) p += ks[i] * qs[i];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) p += __shfl_xor(p, off, 64);
        if (tid == 0) kq_sh = p;
      }

      // 3. fade and partial reads over this thread's rows
      float4 w = make_float4(0.f, 0.f, 0.f, 0.f), y = w;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float a = as[r], kr = ks[r], qr = qs[r];
        s[i] *= a;
        w.x += kr * s[i][0]; w.y += kr * s[i][1]; w.z += kr * s[i][2]; w.w += kr * s[i][3];
        y.x += qr * s[i][0]; y.y += qr * s[i][1]; y.z += qr * s[i][2]; y.w += qr * s[i][3];
      }
      wred[rg][cq] = w;
      yred[rg][cq] = y;
      __syncthreads();

      // 4. finish the reductions, form the correction and the output
      if (rg == 0) {
        float4 W = wred[0][cq], Y = yred[0][cq];
#pragma unroll
        for (int j = 1; j < RG; ++j) {
          const float4 a = wred[j][cq], c = yred[j][cq];
          W.x += a.x; W.y += a.y; W.z += a.z; W.w += a.w;
          Y.x += c.x; Y.y += c.y; Y.z += c.z; Y.w += c.w;
        }
        const float kq = kq_sh;
        const int c0 = 4 * cq;
        float u0 = vs[c0 + 0], u1 = vs[c0 + 1], u2 = vs[c0 + 2], u3 = vs[c0 + 3];
        if (!additive) {  // the correction against the faded read
          const float bt = kRaw ? sigmoid(bf16_to_f32(b16[bh])) : beta[bh];
          u0 = bt * (u0 - W.x); u1 = bt * (u1 - W.y); u2 = bt * (u2 - W.z); u3 = bt * (u3 - W.w);
        }
        us[c0 + 0] = u0; us[c0 + 1] = u1; us[c0 + 2] = u2; us[c0 + 3] = u3;
        io_traits<IO>::store(o, tv + c_base + c0 + 0, Y.x + kq * u0);
        io_traits<IO>::store(o, tv + c_base + c0 + 1, Y.y + kq * u1);
        io_traits<IO>::store(o, tv + c_base + c0 + 2, Y.z + kq * u2);
        io_traits<IO>::store(o, tv + c_base + c0 + 3, Y.w + kq * u3);
      }
      __syncthreads();

      // 5. write the updated state in place: S = Sbar + k u^T
      const float4 u4 = *reinterpret_cast<const float4*>(&us[4 * cq]);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float kr = ks[r];
        f32x4_t t = s[i];
        t[0] += kr * u4.x; t[1] += kr * u4.y; t[2] += kr * u4.z; t[3] += kr * u4.w;
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(S + (size_t)r * DV + 4 * cq));
      }
      if (!kPersist) return;
      __syncthreads();  // LDS is reused by the next item
    } else if (Sn) {
      load_state(Sn, sn);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = sn[i];
    S = Sn;
  }
}

// kPersist: a grid of kPersistPerCu workgroups per CU walking the items
constexpr int kPersistPerCu = 8;

template <int D, int BLOCK, typename IO, int DVW = D, bool kPersist = false>
kda_status_t launch_typed(int32_t batch, int H, const void* q, const void* k, const void* v,
                          const void* g, const void* beta, bool raw, float gate_min, float* states,
                          int32_t num_slots, const int32_t* slots, uint32_t flags, void* o,
                          hipStream_t stream) {
  const int items = batch * H * (D / DVW);
  unsigned grid = (unsigned)items;
  if (kPersist) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
      int x = 0;
      if (hipDeviceGetAttribute(&x, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && x > 0)
        ncu = x;
    }
    grid = (unsigned)min(items, kPersistPerCu * ncu);
  }
  if (raw)
    hipLaunchKernelGGL((decode_kernel<D, D, BLOCK, IO, DVW, true, kPersist>), dim3(grid), dim3(BLOCK),
                       0, stream, static_cast<const IO*>(q), static_cast<const IO*>(k),
                       static_cast<const IO*>(v), g, beta, gate_min, states, num_slots, slots,
                       flags, static_cast<IO*>(o), H, items);
  else
    hipLaunchKernelGGL((decode_kernel<D, D, BLOCK, IO, DVW, false, kPersist>), dim3(grid), dim3(BLOCK),
                       0, stream, static_cast<const IO*>(q), static_cast<const IO*>(k),
                       static_cast<const IO*>(v), g, beta, gate_min, states, num_slots, slots,
                       flags, static_cast<IO*>(o), H, items);
  return check_launch("decode_kernel");
}

template <typename IO>
kda_status_t launch_io(int d, int32_t batch, int H, const void* q, const void* k, const void* v,
                       const void* g, const void* beta, bool raw, float gate_min, float* states,
                       int32_t num_slots, const int32_t* slots, uint32_t flags, void* o,
                       hipStream_t stream) {
  switch (d) {
    case 16: return launch_typed<16, 64, IO>(batch, H, q, k, v, g, beta, raw, gate_min, states, num_slots, slots, flags, o, stream);
    case 32: return launch_typed<32, 64, IO>(batch, H, q, k, v, g, beta, raw, gate_min, states, num_slots, slots, flags, o, stream);
    case 64: return launch_typed<64, 128, IO>(batch, H, q, k, v, g, beta, raw, gate_min, states, num_slots, slots, flags, o, stream);
    case 128: return launch_typed<128, 256, IO, 64, true>(batch, H, q, k, v, g, beta, raw, gate_min, states, num_slots, slots, flags, o, stream);
    default: return KDA_ERR_UNSUPPORTED;
  }
}

}  // namespace

bool decode_supported(int dk, int dv) {
  return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

kda_status_t launch_decode(const kda_shape_t* sh, int32_t batch, const void* q, const void* k,
                           const void* v, const void* g, const void* beta, bool raw,
                           float gate_min, float* states, int32_t num_slots, const int32_t* slots,
                           uint32_t flags, void* o, hipStream_t stream) {
  if (sh->io_dtype == KDA_BF16)
    return launch_io<uint16_t>(sh->dk, batch, sh->num_heads, q, k, v, g, beta, raw, gate_min,
                               states, num_slots, slots, flags, o, stream);
  if (raw) return KDA_ERR_UNSUPPORTED;  // raw projections are bf16
  return launch_io<float>(sh->dk, batch, sh->num_heads, q, k, v, g, beta, false, gate_min, states,
                          num_slots, slots, flags, o, stream);
}

}  // namespace kda
