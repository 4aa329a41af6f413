// kda_chunk_mfma.hip -- chunkwise prefill for dk = dv = 128, chunk = 64, bf16 I/O,
// on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 state and accumulation.
//
// The chunk algebra (one head, chunk of C = 64 tokens entering with state S;
// G = running sum of the per-channel log-gates inside the chunk, Gam = exp(G)):
//   A_kk[r,j] = beta_r sum_c k_r[c] k_j[c] exp(G_r[c] - G_j[c])   (j < r)
//   A_qk[r,j] =        sum_c q_r[c] k_j[c] exp(G_r[c] - G_j[c])   (j <= r)
//   T  = (I + A_kk)^-1
//   W  = T Diag(beta) (K*Gam),  Ut = T Diag(beta) V
//   U  = Ut - W S                                   (corrected values)
//   O  = (Q*Gam) S + A_qk U                         (state read + in-chunk part)
//   S' = Diag(Gam_C) S + (K*exp(G_C - G))^T U       (fold the chunk into S)
// This is the triangular-solve ("WY") packaging of the chunked delta rule
// (engineermaxxing "From GPT-2 to Kimi K3", ch. 04e; heqinghuang "From GPT2 to
// Kimi3, Explained", section 10) with the running per-channel decay products
// folded through it (heqinghuang section 11; engineermaxxing ch. 05d keeps
// them as sums of logs).  It equals the sequential recurrence up to rounding.
//
// Work split (launches on the caller's stream):
//  1. index: per-sequence chunk counts and offsets (sanitised, one thread); up
//     to 384 sequences the prep builds them itself and this launch is skipped.
//  2. prep:  persistent workgroups over the (chunk, head) items, fully parallel
//     over chunks.  It
//     computes everything that does not depend on the incoming state: the
//     gated Gram blocks, the triangular inverse (fp32), W, Ut, Q*Gam,
//     (K*exp(G_C-G))^T, A_qk and Gam_C, and stores the MFMA operands in the
//     exact per-lane order the scan consumes (one 16-byte load per lane).
//  3. scan:  waves own tiles of 16 state columns of one (sequence, head); the
//     columns of S evolve independently given k, beta and g, so the state is
//     split over waves.  Each wave keeps its 128-row slice of S as MFMA
//     accumulators for the whole sequence and walks the chunks in order: the
//     only loop-carried dependency of the method (heqinghuang section 10: the
//     only sequential loop is over chunks).  The waves of a workgroup share
//     each chunk's operands through LDS.  With few chains, dedicated loader
//     waves copy the operands so the compute waves never wait on the copies,
//     and output waves of their own form the outputs one step behind the state
//     waves (a store wave writes them); with many chains, one workgroup per
//     head fetches them once per chunk.
//
// Numerics of the gated Gram products: exp(G_r - G_j) is split at the first
// row s of the 16-row block of r as exp(G_r - G_s) * exp(G_s - G_j).  For j in
// an earlier block both factors are <= 1.  For the diagonal block the second
// factor is >= 1 and bounded by exp(spread), spread = max_c (G_s - G_{s+15});
// when the spread exceeds kMaxSpread that diagonal block is computed element
// by element in fp32 instead (exact, slow, only for extreme decay).
#include "kda_common.h"

namespace kda {

namespace {

constexpr int C = 64;     // chunk
constexpr int D = 128;    // dk = dv
// bf16 LDS row stride (elements) of the prep's K, Q, V tiles: 272 bytes, so that a
// row piece of 8 elements is one 16-byte write and the row reads of the Gram
// operands (16 rows x 4 lane groups) fall on distinct banks in each half-wave
constexpr int KP = D + 8;
constexpr int GP = D + 4;  // fp32 LDS row stride for G
constexpr int AP = C + 4;  // fp32 LDS row stride for A_kk and T
constexpr float kMaxSpread = 80.f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Per chunk-head operand blocks in the workspace (bytes).
constexpr size_t kWnBytes = 4 * 4 * 64 * 16;   // -W      A operand, M=rows,  K=dk
constexpr size_t kQgBytes = 4 * 4 * 64 * 16;   // Q*Gam   A operand, M=rows,  K=dk
constexpr size_t kKdBytes = 8 * 2 * 64 * 16;   // Kd^T    A operand, M=dk,    K=rows
constexpr size_t kAqBytes = 4 * 2 * 64 * 16;   // A_qk    A operand, M=rows,  K=rows
constexpr size_t kUtBytes = 2 * 8 * 64 * 16;   // Ut      accumulator layout, bf16, row tiles in pairs
constexpr size_t kGcBytes = D * 4;             // Gam_C   fp32
// Written by the backward's forward state pass for the gradient kernel:
constexpr size_t kScBytes = 8 * 4 * 64 * 16;   // S at chunk start, B operand (K=dk, N=dv), bf16
constexpr size_t kUcBytes = 8 * 2 * 64 * 16;   // U, B operand (K=rows, N=dv), bf16
// Backward only (the reverse scan's A operands use the Kd^T / A_qk block sizes;
// the gradient kernel reads T^T as bf16 operand tiles and M_kk as fp32 16 x 16 tiles):
//   kdr  Kd        A operand, M=rows, K=dk      wt   -W^T    A operand, M=dk, K=rows
//   qgt  (Q*Gam)^T A operand, M=dk,   K=rows    aqt  A_qk^T  A operand, M=rows j, K=rows r
//   dsc  dL/dS at chunk end and duc dL/dU, laid out as S and U above.
constexpr size_t kMkBytes = C * C * 4;        // M_kk fp32, 16x16 tiles [R*4 + J][row][column]
constexpr size_t kTmBytes = 8 * 64 * 16;       // T^T bf16 A-operand tiles [m*2 + s2][lane]

// Chains (sequence-heads) up to which each head's state is split over eight
// workgroups of 16 columns whose state wave does only the state recurrence and
// a wave beside it forms the outputs: with few chains the serial chain of chunk
// steps is the critical path, so work is moved off it.
constexpr int kSplitMaxChains = 32;
bool split_outputs(int32_t N, int H) { return (int64_t)N * H <= kSplitMaxChains; }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 16x16x4: lane l supplies A[l%16][l/16] and B[l/16][l%16]; the result
// layout is that of the bf16 instruction (rows 4(l/16)+jj, column l%16).
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// K index held in slot q (0..7) of lane group g of a 32-deep MFMA operand.
// Slots 0-3 cover 4g..4g+3 and slots 4-7 cover 16+4g..16+4g+3: this is the row
// order in which two stacked 16x16 accumulator tiles sit in a lane, so an
// accumulator pair converts to a B operand without moving data across lanes.
__device__ __forceinline__ int kpos(int g, int q) { return q < 4 ? 4 * g + q : 12 + 4 * g + q; }

typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 pack8(const float* f) {
  f32x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = f[i];
  return __builtin_convertvector(v, bf16x8);  // v_cvt_pk_bf16_f32, round to nearest even
}
__device__ __forceinline__ bf16x8 pack_acc(f32x4 lo, f32x4 hi) {
  const f32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_convertvector(v, bf16x8);
}

// The two accumulator tiles that pack_acc packed, back in fp32 (exact: bf16 -> fp32).
__device__ __forceinline__ void unpack_acc(bf16x8 p, f32x4& lo, f32x4& hi) {
  const u32x4 w = __builtin_bit_cast(u32x4, p);
  lo = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
             __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
  hi = f32x4{__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
             __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u)};
}

// The 8 values a lane holds for K-block s: elements 32s+4g .. +3 and 32s+16+4g .. +3
// of a padded LDS row (bf16 or fp32), read as two vector loads.
__device__ __forceinline__ void runs_bf(const uint16_t* row, int s, int g, float out[8]) {
  const uint2 a = *reinterpret_cast<const uint2*>(row + 32 * s + 4 * g);
  const uint2 b = *reinterpret_cast<const uint2*>(row + 32 * s + 16 + 4 * g);
  const uint32_t w[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void runs_f32(const float* row, int s, int g, float out[8]) {
  const float4 a = *reinterpret_cast<const float4*>(row + 32 * s + 4 * g);
  const float4 b = *reinterpret_cast<const float4*>(row + 32 * s + 16 + 4 * g);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

struct Workspace {
  int32_t* seq_start;
  int32_t* seq_end;
  int32_t* seq_nch;
  int32_t* chunk_off;  // [N + 1]
  uint8_t* wn;
  uint8_t* qg;
  uint8_t* kd;
  uint8_t* aq;
  uint8_t* ut;
  uint8_t* gc;
  uint8_t* sc;         // split outputs and backward only (else null)
  uint8_t* uc;
  uint8_t* sink;       // 256 B target of stores for rows past a sequence's end
  // backward only (else null)
  uint8_t* kdr;
  uint8_t* wt;
  uint8_t* qgt;
  uint8_t* aqt;
  uint8_t* mkk;
  uint8_t* tm;
  uint8_t* dsc;
  uint8_t* duc;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t header_bytes(int32_t N) { return align256(sizeof(int32_t) * (size_t)(4 * N + 1)); }

size_t nchunks_max(int32_t T, int32_t N) { return (size_t)T / C + (size_t)N; }

Workspace carve(void* base, int32_t T, int32_t N, int H, bool bwd = false) {
  Workspace w;
  uint8_t* p = static_cast<uint8_t*>(base);
  int32_t* hdr = reinterpret_cast<int32_t*>(p);
  w.seq_start = hdr;
  w.seq_end = hdr + N;
  w.seq_nch = hdr + 2 * N;
  w.chunk_off = hdr + 3 * N;
  p += header_bytes(N);
  const size_t ci = nchunks_max(T, N) * (size_t)H;
  // Q*Gam and A_qk in the forward scans' layouts serve only the forward outputs;
  // the backward reads neither
  w.qg = w.aq = nullptr;
  w.wn = p; p += align256(ci * kWnBytes);
  if (!bwd) { w.qg = p; p += align256(ci * kQgBytes); }
  w.kd = p; p += align256(ci * kKdBytes);
  if (!bwd) { w.aq = p; p += align256(ci * kAqBytes); }
  w.ut = p; p += align256(ci * kUtBytes);
  w.gc = p; p += align256(ci * kGcBytes);
  w.sc = w.uc = nullptr;
  w.kdr = w.wt = w.qgt = w.aqt = w.mkk = w.tm = w.dsc = w.duc = nullptr;
  if (bwd) {
    w.sc = p; p += align256(ci * kScBytes);
    w.uc = p; p += align256(ci * kUcBytes);
  }
  if (bwd) {
    w.kdr = p; p += align256(ci * kKdBytes);
    w.wt = p; p += align256(ci * kKdBytes);
    w.qgt = p; p += align256(ci * kKdBytes);
    w.aqt = p; p += align256(ci * kAqBytes);
    w.mkk = p; p += align256(ci * kMkBytes);
    w.tm = p; p += align256(ci * kTmBytes);
    w.dsc = p; p += align256(ci * kScBytes);
    w.duc = p; p += align256(ci * kUcBytes);
  }
  w.sink = p;
  return w;
}

// ------------------------------------------------------------------ 1. index
// Sanitised bounds: start = clamp(cu[n]), end = clamp(cu[n+1]) >= start; the
// running chunk total is capped at the workspace capacity, so malformed
// offsets can never address memory outside the buffers.
__global__ void index_kernel(const int32_t* __restrict__ cu, int32_t N, int32_t T, int32_t cap,
                             Workspace w) {
  if (threadIdx.x != 0) return;
  int32_t run = 0;
  for (int32_t n = 0; n < N; ++n) {
    const int32_t s = clamp_tok(cu[n], T);
    int32_t e = clamp_tok(cu[n + 1], T);
    if (e < s) e = s;
    int32_t nch = (e - s + C - 1) / C;
    if (nch > cap - run) {
      nch = cap - run;
      e = s + nch * C < e ? s + nch * C : e;
    }
    w.seq_start[n] = s;
    w.seq_end[n] = e;
    w.seq_nch[n] = nch;
    w.chunk_off[n] = run;
    run += nch;
  }
  w.chunk_off[N] = run;
}

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its outstanding global loads and stores (which __syncthreads' fence would
// drain).  The empty asm after the barrier keeps the compiler from moving
// later LDS accesses above it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ 2. prep
// Persistent workgroups of 8 waves; each walks (chunk, head) items with a
// stride of the grid size.  The global loads of the next item are issued into
// registers before the current item is computed, so they overlap its compute.
constexpr int kPrepWaves = 8;

// The prep keeps the running gate sums in base-2 units, G * log2(e), so that every
// decay factor exp(G_a - G_b) is one hardware exp2 of a difference.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr int kPrepThreads = 64 * kPrepWaves;

struct PrepSmem {
  uint16_t K[C][KP];
  uint16_t Q[C][KP];
  uint16_t V[C][KP];
  float G[C][GP];        // running gate sums, in base-2 units (G * log2 e)
  float A[C][AP];        // beta-scaled strictly lower A_kk (backward: A_qk^T above it)
  float Tm[C][AP];       // (I + A_kk)^-1
  float tot[4][D];       // per-quarter column totals of the running gate sums
  float es[4][D];        // exp(G) at the first row of each 16-row block
  float spr[kPrepWaves]; // per-wave maxima of the in-block gate spread
  float bs[C];
  bf16x8 rk[16][64];     // row-side Gram operands [R * 4 + s][lane]: k_r exp(G_r - G_sR)
  bf16x8 rq[16][64];     //                                         q_r exp(G_r - G_sR)
  // sequence header built by the prep itself (up to kFuseMaxSeqs sequences)
  int32_t hs[384];       // sanitised sequence starts
  int32_t he[384];       // sanitised ends
  int32_t ho[385];       // chunk offsets (prefix sums of chunk counts, capped)
};
static_assert(sizeof(PrepSmem) <= 160 * 1024, "the prep's LDS");
// Up to this many sequences the prep builds the sequence header in LDS itself
// (and workgroup 0 publishes it for the later launches), so no separate index
// launch precedes it.
constexpr int kFuseMaxSeqs = 384;

// One item's inputs between the global loads and the LDS staging.  The gate is
// held by thread (channel tid % 128, quarter tid / 128) down its 16 rows, so the
// running sums over the rows are formed in registers.
struct PrepIn {
  uint4 k[2], q[2], v[2];
  float g[16];        // the gate of this thread's channel at rows 16 quarter + i (scalar gate: the row's)
  float beta;
  // raw projections (kRaw): bf16 logits kept as loaded, converted at staging
  uint16_t gl[16];    // gate logits, per channel or scalar, of the same entries
  uint16_t b16;       // write-strength logit
};

// Gate variants of the prep, fixed at compile time so that the prefetch of the
// next item has no data-dependent register moves (which would wait for it).
constexpr int kGateChannel = 0, kGateScalar = 1, kGateNone = 2;

struct ItemPos {
  int gc, h, t0, c;  // chunk, head, first token, valid rows (>= 1)
};

// The header arrays are read through const __restrict__ pointers with
// wave-uniform indices, so the compiler uses scalar loads: their waits do not
// include the workgroup's outstanding vector loads and stores.
struct Header {
  const int32_t* __restrict__ seq_start;
  const int32_t* __restrict__ seq_end;
  const int32_t* __restrict__ chunk_off;
};

__device__ __forceinline__ ItemPos locate(const Header& hd, int N, int H, int item) {
  ItemPos p;
  p.gc = item / H;
  p.h = item - p.gc * H;
  int lo = 0, hi = N - 1;  // the sequence owning chunk gc (largest n with chunk_off[n] <= gc)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (hd.chunk_off[mid] <= p.gc) lo = mid; else hi = mid - 1;
  }
  p.t0 = hd.seq_start[lo] + (p.gc - hd.chunk_off[lo]) * C;
  p.c = min(C, hd.seq_end[lo] - p.t0);
  return p;
}

// Heads up to which the prep's 32-bit row offsets (row < 64 times H * D elements)
// are exact; the host refuses more before any launch.
constexpr int kMaxHeads = 65536;

// The position of a workgroup-uniform item in scalar registers (values read from
// LDS are vector registers to the compiler), so that the row addresses built on it
// are a scalar base plus a 32-bit lane offset.
__device__ __forceinline__ ItemPos uniform_pos(ItemPos p) {
  p.gc = __builtin_amdgcn_readfirstlane(p.gc);
  p.h = __builtin_amdgcn_readfirstlane(p.h);
  p.t0 = __builtin_amdgcn_readfirstlane(p.t0);
  p.c = __builtin_amdgcn_readfirstlane(p.c);
  return p;
}

// The same lookup in the header the prep built in LDS.
__device__ __forceinline__ ItemPos locate_lds(const PrepSmem& sm, int N, int H, int item) {
  ItemPos p;
  p.gc = item / H;
  p.h = item - p.gc * H;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sm.ho[mid] <= p.gc) lo = mid; else hi = mid - 1;
  }
  p.t0 = sm.hs[lo] + (p.gc - sm.ho[lo]) * C;
  p.c = min(C, sm.he[lo] - p.t0);
  return uniform_pos(p);
}

// The sequence header (as index_kernel builds it) for N <= kFuseMaxSeqs, by the
// whole workgroup: chunk counts, their prefix sums by a scan over the waves,
// capped at the workspace capacity.  Workgroup 0 also stores it to the workspace.
__device__ __forceinline__ void build_header(PrepSmem& sm, const int32_t* __restrict__ cu, int32_t N,
                                             int32_t T, int32_t cap, const Workspace& w,
                                             bool publish, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  int32_t s = 0, e = 0, nch = 0;
  if (tid < N) {
    s = clamp_tok(cu[tid], T);
    e = clamp_tok(cu[tid + 1], T);
    if (e < s) e = s;
    nch = (e - s + C - 1) / C;
  }
  // inclusive scan of nch inside the wave, then over the wave totals
  int32_t incl = nch;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sm.ho[kFuseMaxSeqs - kPrepWaves + wave] = incl;  // wave totals, scratch
  __syncthreads();
  int32_t base = 0;
  for (int x = 0; x < wave; ++x) base += sm.ho[kFuseMaxSeqs - kPrepWaves + x];
  __syncthreads();
  const int32_t excl = base + incl - nch;
  if (tid < N) {
    const int32_t off = min(excl, cap), end = min(excl + nch, cap);
    const int32_t n2 = end - off;
    const int32_t e2 = s + n2 * C < e ? s + n2 * C : e;
    sm.hs[tid] = s;
    sm.he[tid] = e2;
    sm.ho[tid] = off;
    if (tid == N - 1) sm.ho[N] = end;
    if (publish) {
      w.seq_start[tid] = s;
      w.seq_end[tid] = e2;
      w.seq_nch[tid] = n2;
      w.chunk_off[tid] = off;
      if (tid == N - 1) w.chunk_off[N] = end;
    }
  }
  __syncthreads();
}

// Rows past the end of the sequence read the last valid row (zeroed at staging).
// Variants: a scalar gate is read once per row and staged on every channel; no
// gate reads nothing (G = 0); the additive write reads no beta (beta = 1, and
// the correction is dropped later).  kRaw: q, k are raw projections and the
// gate and write strength are bf16 logits (prepared at staging).
// The next item's loads, in four parts that the item loop issues at four
// points of the current item: all of them at once would hold the wave at the
// issue until the CU's memory pipeline takes them.  Part 0: k, q; part 1: v,
// beta; parts 2 and 3: the first and last eight of the thread's 16 gate rows
// (one channel each; a wave reads 64 consecutive channels of a row).
// The per-head rows of q, k, v and the channel gates are read once: non-temporal
// loads, which do not displace what the caches hold (on a cold call that also
// spares the write-back of the dirty lines they would evict).  beta and a scalar
// gate are one value per token and head, so one 128-byte line holds a token's
// values for many heads and the items of those heads share it: plain loads.
typedef unsigned int ntu32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load4(const void* p) {
  const ntu32x4 x = __builtin_nontemporal_load(reinterpret_cast<const ntu32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
template <typename T>
__device__ __forceinline__ T nt_load(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ T nt_load16(const T* p) {  // any 16-byte operand tile
  static_assert(sizeof(T) == 16, "16-byte loads");
  return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const ntu32x4*>(p)));
}

template <int kGate, bool kAdd, bool kRaw, int kPart>
__device__ __forceinline__ void prep_load_part(PrepIn& in, const ItemPos& p, const uint16_t* q,
                                               const uint16_t* k, const uint16_t* v,
                                               const void* gp, const void* bp, int H, int tid) {
  const float* g = static_cast<const float*>(gp);
  const float* beta = static_cast<const float*>(bp);
  const uint16_t* g16 = static_cast<const uint16_t*>(gp);
  const uint16_t* b16 = static_cast<const uint16_t*>(bp);
  // a scalar base at the chunk's first row, plus 32-bit lane offsets (rows < 64,
  // H * D < 2^24 elements, so the 24-bit multiply is exact and offsets fit)
  const uint32_t rowstride = (uint32_t)H * D;
  const size_t base = ((size_t)p.t0 * H + p.h) * D;
  const size_t bbase = (size_t)p.t0 * H + p.h;
  if constexpr (kPart <= 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + kPrepThreads * i, r = u >> 4, cc = (u & 15) * 8;
      const uint32_t gi = __umul24((uint32_t)min(r, p.c - 1), rowstride) + cc;
      if constexpr (kPart == 0) {
        in.k[i] = nt_load4(k + base + gi);
        in.q[i] = nt_load4(q + base + gi);
      } else {
        in.v[i] = nt_load4(v + base + gi);
      }
    }
    if constexpr (kPart == 1 && !kAdd) {
      const uint32_t bi = __umul24((uint32_t)min(tid & 63, p.c - 1), (uint32_t)H);
      if (kRaw) in.b16 = b16[bbase + bi];
      else in.beta = beta[bbase + bi];
    }
  } else {
    const int col = tid & (D - 1), qt = tid >> 7;
#pragma unroll
    for (int i = 8 * (kPart - 2); i < 8 * (kPart - 2) + 8; ++i) {
      const uint32_t row = (uint32_t)min(16 * qt + i, p.c - 1);
      if (kGate == kGateScalar) {
        const uint32_t gi = __umul24(row, (uint32_t)H);
        if (kRaw) in.gl[i] = g16[bbase + gi];
        else in.g[i] = g[bbase + gi];
      } else if (kGate == kGateChannel) {
        const uint32_t gi = __umul24(row, rowstride) + col;
        if (kRaw) in.gl[i] = nt_load(g16 + base + gi);
        else in.g[i] = nt_load(g + base + gi);
      }
    }
  }
}

template <int kGate, bool kAdd, bool kRaw>
__device__ __forceinline__ void prep_load(PrepIn& in, const ItemPos& p, const uint16_t* q,
                                          const uint16_t* k, const uint16_t* v, const void* gp,
                                          const void* bp, int H, int tid) {
  prep_load_part<kGate, kAdd, kRaw, 0>(in, p, q, k, v, gp, bp, H, tid);
  prep_load_part<kGate, kAdd, kRaw, 1>(in, p, q, k, v, gp, bp, H, tid);
  prep_load_part<kGate, kAdd, kRaw, 2>(in, p, q, k, v, gp, bp, H, tid);
  prep_load_part<kGate, kAdd, kRaw, 3>(in, p, q, k, v, gp, bp, H, tid);
}

// normalize(silu(x)) of one row held by the 16 lanes of a lane group, 8 channels
// per lane (bf16 in, bf16 out)
__device__ __forceinline__ uint4 prepare_row8(uint4 raw) {
  const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
  float f[8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = silu(__uint_as_float(wv[j] << 16));
    f[2 * j + 1] = silu(__uint_as_float(wv[j] & 0xffff0000u));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float inv = inv_norm(ss);
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = (uint32_t)f32_to_bf16(f[2 * j] * inv) | ((uint32_t)f32_to_bf16(f[2 * j + 1] * inv) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// normalize(silu(x)) of an item's raw q and k rows, in their load registers (the 16
// lanes of a row group hold one row, so every lane takes part)
__device__ __forceinline__ void prep_raw_qk(PrepIn& in) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    in.k[i] = prepare_row8(in.k[i]);
    in.q[i] = prepare_row8(in.q[i]);
  }
}

template <int kGate, bool kAdd, bool kRaw>
__device__ __forceinline__ void prep_stage(PrepSmem& sm, const PrepIn& in, int c, int tid,
                                           float gate_min) {
  const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + kPrepThreads * i, r = u >> 4, cc = (u & 15) * 8;
    const bool ok = r < c;
    // kRaw: q and k arrive prepared (prep_raw_qk, during the previous item)
    const uint4 kk = in.k[i];
    const uint4 qq = in.q[i];
    const uint4 a = ok ? kk : z4, b = ok ? qq : z4, d = ok ? in.v[i] : z4;
    *reinterpret_cast<uint4*>(&sm.K[r][cc]) = a;
    *reinterpret_cast<uint4*>(&sm.Q[r][cc]) = b;
    *reinterpret_cast<uint4*>(&sm.V[r][cc]) = d;
  }
  const float bt = kAdd ? 1.f : kRaw ? sigmoid(bf16_to_f32(in.b16)) : in.beta;
  if (tid < C) sm.bs[tid] = tid < c ? bt : 0.f;
  // the two blocks above the diagonal that the W / Ut products read, (0,1) and (2,3);
  // the inverse writes every block on and below the diagonal
  {
    const int blk = tid >> 8, e = tid & 255;
    sm.Tm[32 * blk + (e >> 4)][32 * blk + 16 + (e & 15)] = 0.f;
  }
}

// The log-gate of this thread's entry i (channel tid % 128, row 16 (tid / 128) + i),
// zero past the end of the sequence (neutral padding).
template <int kGate, bool kRaw>
__device__ __forceinline__ float prep_gate(const PrepIn& in, int i, int row, int c, float gate_min) {
  if (kGate == kGateNone || row >= c) return 0.f;
  return kRaw ? fmaxf(log_sigmoid(bf16_to_f32(in.gl[i])), gate_min) : in.g[i];
}

__device__ __forceinline__ float ld_bf(const uint16_t* row, int c) { return bf16_to_f32(row[c]); }

// Gram block pair (R, J), J <= R: raw A[r][j] for r in block R (lane row li),
// j = 16J + 4lg + jj, for keys (acck) and queries (accq).  The row side comes
// scaled from LDS; the key side k_j exp(G_sR - G_j) is formed here.  `wide`:
// the gate spread inside block R exceeds kMaxSpread, so the diagonal pair is
// summed element by element in fp32 (exact, slow, only for extreme decay).
__device__ __forceinline__ void gram_pair(const PrepSmem& sm, int R, int J, bool wide, int li,
                                          int lg, int lane, f32x4& acck, f32x4& accq) {
  const int sR = 16 * R, r = sR + li, j = 16 * J + li;
  acck = f32x4{0.f, 0.f, 0.f, 0.f};
  accq = acck;
  if (J != R || !wide) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float gs[8], kj[8], gj[8], fa[8];
      runs_f32(sm.G[sR], s, lg, gs);
      runs_bf(sm.K[j], s, lg, kj);
      runs_f32(sm.G[j], s, lg, gj);
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i] = kj[i] * exp2_fast(gs[i] - gj[i]);  // rows j: exp(G_s - G_j)
      const bf16x8 ak = pack8(fa);
      acck = mfma(ak, sm.rk[R * 4 + s][lane], acck);
      accq = mfma(ak, sm.rq[R * 4 + s][lane], accq);
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int jd = sR + 4 * lg + jj;
      float kk = 0.f, qk = 0.f;
      if (jd <= r) {
        for (int cc = 0; cc < D; ++cc) {
          const float e = exp2_fast(sm.G[r][cc] - sm.G[jd][cc]);
          const float kv = ld_bf(sm.K[jd], cc) * e;
          kk += ld_bf(sm.K[r], cc) * kv;
          qk += ld_bf(sm.Q[r], cc) * kv;
        }
      }
      acck[jj] = kk;
      accq[jj] = qk;
    }
  }
}

// One workgroup of the prep: items wg, wg + nwg, ... in chunk-major order.
template <int kGate, bool kAdd, bool kRaw, bool kBwd>
__device__ __forceinline__ void prep_role(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta, float gate_min, int32_t N, int H,
    const Workspace& w, const Header& hd, const int32_t* __restrict__ cu, int32_t T, int32_t cap,
    bool fused, uint8_t* smem_raw, int wg, int nwg) {
  // the additive write (u = v) has no correction: A_kk = 0, so T = I, W = 0, Ut = V
  constexpr bool additive = kAdd;
  PrepSmem& sm = *reinterpret_cast<PrepSmem*>(smem_raw);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  // The first item's loads are issued before the sequence header is known, for the
  // position the item has when the batch is one sequence from token 0 (chunk wg / H
  // of head wg % H, rows clamped inside [0, T)), so that they overlap the header's own
  // loads; a workgroup whose item turns out to lie elsewhere loads it again.
  PrepIn in;
  ItemPos spec;
  spec.gc = wg / H;
  spec.h = wg - spec.gc * H;
  spec.t0 = spec.gc * C;
  spec.c = spec.t0 < T ? min(C, T - spec.t0) : 0;
  if (spec.c > 0) prep_load<kGate, kAdd, kRaw>(in, spec, q, k, v, g, beta, H, tid);
  if (fused) build_header(sm, cu, N, T, cap, w, wg == 0, tid);
  auto where = [&](int it) { return fused ? locate_lds(sm, N, H, it) : locate(hd, N, H, it); };
  const int total = (fused ? sm.ho[N] : hd.chunk_off[N]) * H;
  int item = wg;
  if (item >= total) {  // uniform
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load left in flight
    return;
  }

  ItemPos pos = where(item);
  if (spec.c == 0 || pos.t0 != spec.t0 || pos.c != spec.c || pos.h != spec.h)
    prep_load<kGate, kAdd, kRaw>(in, pos, q, k, v, g, beta, H, tid);
  // Wait for the first item here, so that inside the loop the wait for the
  // prefetched registers only has to cover the loads, not the stores issued
  // after them.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if constexpr (kRaw) prep_raw_qk(in);

  for (; item < total; item += nwg) {
    const size_t ci = (size_t)item;  // items are numbered chunk-major: ci = gc * H + h
    const int c = pos.c;
    // the next item's position, looked up here so that its header reads are not
    // on the path of the first prefetch
    const int next = item + nwg;
    const bool prefetch = next < total;
    if (prefetch) pos = where(next);
    lds_barrier();  // the previous item is done with LDS
    prep_stage<kGate, kAdd, kRaw>(sm, in, c, tid, gate_min);

    // ---- running sum of the log-gates down each channel: each thread sums its
    // channel's 16 rows of one quarter in registers, then adds the quarters before it
    {
      const int col = tid & 127, qt = tid >> 7;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = prep_gate<kGate, kRaw>(in, i, 16 * qt + i, c, gate_min) * kLog2e;
#pragma unroll
      for (int i = 1; i < 16; ++i) x[i] += x[i - 1];
      sm.tot[qt][col] = x[15];
      lds_barrier();
      float base = 0.f;
      for (int j = 0; j < qt; ++j) base += sm.tot[j][col];
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.G[16 * qt + i][col] = x[i] + base;
      sm.es[qt][col] = exp2_fast(x[0] + base);
      float sp = x[0] - x[15];  // spread of this channel inside block qt
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sp = fmaxf(sp, __shfl_xor(sp, off, 64));
      if (lane == 0) sm.spr[wave] = sp;  // waves 2qt and 2qt + 1 cover block qt
    }
    // The next item's loads overlap this item's compute, issued in four parts
    // (here, before the Gram blocks, before the diagonal inverse, before the
    // off-diagonal blocks), not at the top of the item where the previous
    // item's output stores still occupy the memory pipeline.
    if (prefetch) prep_load_part<kGate, kAdd, kRaw, 0>(in, pos, q, k, v, g, beta, H, tid);
    lds_barrier();

    // ---- row-side Gram operands and Q*Gam, two (block R, K-block s) units per lane
    {
      uint16_t* qg_out = kBwd ? nullptr : reinterpret_cast<uint16_t*>(w.qg + ci * kQgBytes);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int R = (tid >> 8) + 2 * x, s = wave & 3, r = 16 * R + li;
        float kr[8], qr[8], gr[8], gs[8], e0[8], fk[8], fq[8], fg[8];
        runs_bf(sm.K[r], s, lg, kr);
        runs_bf(sm.Q[r], s, lg, qr);
        runs_f32(sm.G[r], s, lg, gr);
        runs_f32(sm.G[16 * R], s, lg, gs);
        runs_f32(sm.es[R], s, lg, e0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float f = exp2_fast(gr[i] - gs[i]);  // exp(G_r - G_sR) <= 1
          fk[i] = kr[i] * f;
          fq[i] = qr[i] * f;
          fg[i] = fq[i] * e0[i];                    // q_r exp(G_r)
        }
        sm.rk[R * 4 + s][lane] = pack8(fk);
        sm.rq[R * 4 + s][lane] = pack8(fq);
        if constexpr (!kBwd)
          *reinterpret_cast<bf16x8*>(qg_out + ((size_t)(R * 4 + s) * 64 + lane) * 8) = pack8(fg);
      }
    }
    lds_barrier();

    if (prefetch) prep_load_part<kGate, kAdd, kRaw, 1>(in, pos, q, k, v, g, beta, H, tid);

    // The backward's (Q*Gam)^T and Kd operand tiles need K, Q and G only.  Unit b < 16:
    // (Q*Gam)^T as the reverse scan's A operand (M = channel, K = row), channel tile
    // b >> 1, K half b & 1; unit b >= 16: Kd as an A operand (M = row, K = channel),
    // tile b - 16.  Waves that the Gram round and the last off-diagonal distance leave
    // idle take units 12-15 and 28-31; the item's tail takes the other 24.
    auto bwd_unit = [&](int b) {
      if (b < 16) {
        const int ch = 16 * (b >> 1) + li, s2 = b & 1;
        float qv[8], gv[8], fq[8];
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
          const int j = 32 * s2 + kpos(lg, qq);
          qv[qq] = ld_bf(sm.Q[j], ch);
          gv[qq] = sm.G[j][ch];
        }
        __builtin_amdgcn_sched_barrier(0);  // the reads together, then the arithmetic
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) fq[qq] = qv[qq] * exp2_fast(gv[qq]);
        *reinterpret_cast<bf16x8*>(w.qgt + ci * kKdBytes + ((size_t)b * 64 + lane) * 16) = pack8(fq);
      } else {
        const int opi = b - 16, m = opi >> 2, sk = opi & 3, r = 16 * m + li;
        float kv[8], gl[8], gv[8], fk[8];
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
          const int cc = 32 * sk + kpos(lg, qq);
          kv[qq] = ld_bf(sm.K[r], cc);
          gl[qq] = sm.G[C - 1][cc];
          gv[qq] = sm.G[r][cc];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) fk[qq] = kv[qq] * exp2_fast(gl[qq] - gv[qq]);
        *reinterpret_cast<bf16x8*>(w.kdr + ci * kKdBytes + ((size_t)opi * 64 + lane) * 16) = pack8(fk);
      }
    };
    constexpr bool kEarlyUnits = kBwd && !kAdd;

    const int wv = __builtin_amdgcn_readfirstlane(wave);  // scalar role choices
    // The operands of the last phase that do not involve T, for channel tile
    // `tile` and K half s2 (unit u = 2 tile + s2): Kd^T (stored), (beta K Gam)^T
    // and beta V in MFMA-operand order (ob, ov), parked in the LDS of the row-side
    // Gram operands once nothing reads those any more (after the Gram blocks).
    auto form_operands = [&](int u, bf16x8& ob, bf16x8& ov) {
      const int tile = u >> 1, s2 = u & 1, ch = 16 * tile + li;
      // every read first, then the arithmetic: one LDS round trip, not one per row
      const float gl = sm.G[C - 1][ch];
      const float4 b0 = *reinterpret_cast<const float4*>(&sm.bs[32 * s2 + 4 * lg]);
      const float4 b1 = *reinterpret_cast<const float4*>(&sm.bs[32 * s2 + 16 + 4 * lg]);
      float kv[8], gv[8], vv[8];
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        const int j = 32 * s2 + kpos(lg, qq);
        kv[qq] = ld_bf(sm.K[j], ch);
        gv[qq] = sm.G[j][ch];
        vv[qq] = ld_bf(sm.V[j], ch);
      }
      __builtin_amdgcn_sched_barrier(0);
      const float bj[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float fb[8], fd[8], fv[8];
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        fb[qq] = bj[qq] * kv[qq] * exp2_fast(gv[qq]);
        fd[qq] = kv[qq] * exp2_fast(gl - gv[qq]);
        fv[qq] = bj[qq] * vv[qq];  // B operand of Ut for value tile `tile`
      }
      uint16_t* kd_out = reinterpret_cast<uint16_t*>(w.kd + ci * kKdBytes);
      *reinterpret_cast<bf16x8*>(kd_out + ((size_t)u * 64 + lane) * 8) = pack8(fd);
      ob = pack8(fb);
      ov = pack8(fv);
    };
    auto park = [&](int u, const bf16x8& ob, const bf16x8& ov) {
      sm.rk[u][lane] = ob;
      sm.rq[u][lane] = ov;
    };
    // the forward's units 0-3, formed by waves 6 and 7 beside the diagonal inverse
    // (the Gram blocks may still read the LDS they go to) and parked at distance 1
    constexpr bool kFwdEarly = !kAdd && !kBwd;
    bf16x8 held[4];

    // ---- gated Gram blocks, then the diagonal blocks of T = (I + A_kk)^-1.
    // T_JJ = (I + A_JJ)^-1 by right-looking forward substitution (wave J, lane =
    // column): once x[m] is final it is eliminated from every later row at once,
    // so the dependency chain is 15 steps deep.
    {
      uint16_t* aq_out = kBwd ? nullptr : reinterpret_cast<uint16_t*>(w.aq + ci * kAqBytes);
      auto gram = [&](int R, int J) {
        f32x4 acck, accq;
        const bool wide = fmaxf(sm.spr[2 * R], sm.spr[2 * R + 1]) > kMaxSpread * kLog2e;
        gram_pair(sm, R, J, wide, li, lg, lane, acck, accq);
        const int r = 16 * R + li;
        const float br = sm.bs[r];
        float4 arow;
        float qv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 16 * J + 4 * lg + jj;
          (&arow.x)[jj] = j < r && !additive ? br * acck[jj] : 0.f;
          qv[jj] = j <= r ? accq[jj] : 0.f;
        }
        *reinterpret_cast<float4*>(&sm.A[r][16 * J + 4 * lg]) = arow;
        if constexpr (kBwd) {
          // M_kk (unscaled, strictly lower) for the gradient of beta, 16 x 16 tiles
          // [R * 4 + J][row][column], each written as one contiguous 1 KiB block
          float4 mrow;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) (&mrow.x)[jj] = 16 * J + 4 * lg + jj < r ? acck[jj] : 0.f;
          *reinterpret_cast<float4*>(w.mkk + ci * kMkBytes + (size_t)(((R * 4 + J) * 16 + li) * 16 + 4 * lg) * 4) = mrow;
          // A_qk^T into the upper triangle of A (row j, column r >= j), which the
          // triangular solve never reads; for the diagonal block this follows the
          // A_kk row's zeros in the same wave, so these values stay
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int j = 16 * J + 4 * lg + jj;
            if (j <= r) sm.A[j][r] = qv[jj];
          }
        }
        // A_qk as the forward scan's A operand: [m = R][s' = J / 2][lane][slots (J & 1) * 4 ..]
        if constexpr (!kBwd) {
          uint16_t* dst = aq_out + ((size_t)(R * 2 + (J >> 1)) * 64 + lane) * 8 + (J & 1) * 4;
          *reinterpret_cast<uint2*>(dst) =
              make_uint2((uint32_t)f32_to_bf16(qv[0]) | ((uint32_t)f32_to_bf16(qv[1]) << 16),
                         (uint32_t)f32_to_bf16(qv[2]) | ((uint32_t)f32_to_bf16(qv[3]) << 16));
        }
      };
      auto invert_diag = [&](int J) {
        if (lane < 16) {
          const int sJ = 16 * J;
          float x[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = i == lane ? 1.f : 0.f;
#pragma unroll
          for (int m = 0; m < 15; ++m)
#pragma unroll
            for (int i = m + 1; i < 16; ++i) x[i] -= sm.A[sJ + i][sJ + m] * x[m];
#pragma unroll
          for (int i = 0; i < 16; ++i) sm.Tm[sJ + i][sJ + lane] = x[i];
        }
      };
      auto zero_aq_upper = [&]() {
        // blocks above the diagonal stored by the scan: (R, J) = (0,1), (2,3)
        if constexpr (kBwd) return;
        const uint2 z = make_uint2(0, 0);
        *reinterpret_cast<uint2*>(aq_out + ((size_t)(0 * 2 + 0) * 64 + lane) * 8 + 4) = z;
        *reinterpret_cast<uint2*>(aq_out + ((size_t)(2 * 2 + 1) * 64 + lane) * 8 + 4) = z;
      };
      if constexpr (!kAdd) {
        // Round 1: wave w < 4 forms the diagonal pair (w, w), waves 4..7 the
        // pairs (1,0) (2,1) (3,2) (2,0).  Round 2: waves 0..3 invert their own
        // diagonal block (no barrier: the wave wrote it itself, and a wave's LDS
        // accesses are done in order) while waves 4 and 5 form (3,1) and (3,0),
        // which only the second and third off-diagonal distances need.
        if (wv < 4) {
          gram(wv, wv);
        } else {
          const int x = wv - 4;
          gram(x == 3 ? 2 : x + 1, x == 3 ? 0 : x);
        }
        if (wv == 7) zero_aq_upper();
        if (wv < 4) {
          invert_diag(wv);
        } else if (wv < 6) {
          gram(3, 5 - wv);  // wave 4: (3,1), wave 5: (3,0)
        } else if constexpr (kEarlyUnits) {
          bwd_unit(12 + 2 * (wv - 6));
          bwd_unit(13 + 2 * (wv - 6));
        } else {
          form_operands(2 * (wv - 6), held[0], held[1]);
          form_operands(2 * (wv - 6) + 1, held[2], held[3]);
        }
        if (prefetch) prep_load_part<kGate, kAdd, kRaw, 2>(in, pos, q, k, v, g, beta, H, tid);
      } else {
        // The additive write (A_kk = 0, so T = I) takes the 10 pairs in the order
        // (3,3) (3,2) (3,1) (3,0) (2,2) (2,1) (2,0) (1,1) (1,0) (0,0), computed
        // rather than read from a table (a memory read would wait for the next
        // item's prefetched loads), and invert after a barrier.
        for (int pi = wv; pi < 10; pi += kPrepWaves) {
          const int R = pi < 4 ? 3 : pi < 7 ? 2 : pi < 9 ? 1 : 0;
          const int J = pi < 4 ? 3 - pi : pi < 7 ? 6 - pi : pi < 9 ? 8 - pi : 0;
          gram(R, J);
        }
        if (wv == 7) zero_aq_upper();
        lds_barrier();
        if (prefetch) prep_load_part<kGate, kAdd, kRaw, 2>(in, pos, q, k, v, g, beta, H, tid);
        if (wv < 4) invert_diag(wv);
      }
    }
    lds_barrier();
    if (prefetch) prep_load_part<kGate, kAdd, kRaw, 3>(in, pos, q, k, v, g, beta, H, tid);
    // Off-diagonal blocks by distance L = R - J, the blocks of one distance in
    // parallel (one wave each): T_RJ = -T_RR X with X = sum_{J<=K<R} A_RK T_KJ,
    // both products on fp32 MFMA.  The second product takes X straight from the
    // accumulators: at step jj lane group g contributes contraction index 4g+jj.
    // The waves a distance leaves idle form the 16 operand units meanwhile.  The
    // forward: units 0-3 formed earlier are parked at distance 1, which forms none
    // (its blocks are the shortest), 4-9 at 2 (waves 2-7), 10-15 at 3 (waves 1-6).
    // The other variants: units 0-4 at distance 1 (waves 3-7), 5-10 at 2 (waves
    // 2-7), 11-15 at 3 (waves 1-5).
#pragma unroll
    for (int L = 1; L < 4; ++L) {
      if (wv >= 4 - L) {
        if constexpr (kFwdEarly) {
          if (L == 1) {
            if (wv >= 6) {
              park(2 * (wv - 6), held[0], held[1]);
              park(2 * (wv - 6) + 1, held[2], held[3]);
            }
          } else {
            const int u = (L == 2 ? 4 : 10) + wv - (4 - L);
            if (u < 16) {
              bf16x8 ob, ov;
              form_operands(u, ob, ov);
              park(u, ob, ov);
            }
          }
        } else {
          const int u = (L == 1 ? 0 : L == 2 ? 5 : 11) + wv - (4 - L);
          if (u < 16) {
            bf16x8 ob, ov;
            form_operands(u, ob, ov);
            park(u, ob, ov);
          } else if constexpr (kEarlyUnits) {  // waves 6 and 7 at distance 3
            bwd_unit(28 + 2 * (wv - 6));
            bwd_unit(29 + 2 * (wv - 6));
          }
        }
      } else {
        const int J = wv, R = J + L;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        for (int Kb = J; Kb < R; ++Kb)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            x = mfma_f32(sm.A[16 * R + li][16 * Kb + 4 * kb + lg],
                         sm.Tm[16 * Kb + 4 * kb + lg][16 * J + li], x);
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) t = mfma_f32(sm.Tm[16 * R + li][16 * R + 4 * lg + jj], x[jj], t);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sm.Tm[16 * R + 4 * lg + jj][16 * J + li] = -t[jj];
      }
      lds_barrier();
    }

    if constexpr (kBwd) {
      // T^T for the gradient kernel, as the A operand of dR = T^T dU there (M = row
      // r, K = row j, kpos order): bf16 tiles [m * 2 + s2][lane], wave = m * 2 + s2.
      // Tiles m >= 2, s2 = 0 are zero (T is lower triangular) and not stored.
      const int m = wave >> 1, s2 = wave & 1;
      if (m < 2 || s2 == 1) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = sm.Tm[32 * s2 + kpos(lg, e)][16 * m + li];
        *reinterpret_cast<bf16x8*>(w.tm + ci * kTmBytes + ((size_t)wave * 64 + lane) * 16) = pack8(f);
      }
    }

    // ---- W, Ut, Kd^T, Gam_C in the scan's operand order; wave = channel tile = value tile
    {
      bf16x8 tt[4][2];  // T tiles: A operand (M = r) of Ut and B operand (N = r) of W^T
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (m < 2 && s2 == 1) continue;  // T is lower triangular: zero block
          const float* trow = &sm.Tm[16 * m + li][32 * s2 + 4 * lg];
          const float4 a = *reinterpret_cast<const float4*>(trow);
          const float4 b = *reinterpret_cast<const float4*>(trow + 16);
          const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          tt[m][s2] = pack8(f);
        }
      const int tile = wave;
      // (beta K Gam)^T (A operand of W^T) and beta V (B operand of Ut) for channel
      // tile `tile`, formed during the off-diagonal blocks
      bf16x8 abkg[2], bv[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        abkg[s2] = sm.rk[tile * 2 + s2][lane];
        bv[s2] = sm.rq[tile * 2 + s2][lane];
      }
      // -W: [m = nt][s = tile / 2][lane][slots (tile & 1) * 4 ..]
      uint16_t* wn_out = reinterpret_cast<uint16_t*>(w.wn + ci * kWnBytes);
      bf16x8* ut_out = reinterpret_cast<bf16x8*>(w.ut + ci * kUtBytes);
      f32x4 ut_even = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma(abkg[0], tt[nt][0], acc);
        if (nt >= 2) acc = mfma(abkg[1], tt[nt][1], acc);
        uint16_t* dst = wn_out + ((size_t)(nt * 4 + (tile >> 1)) * 64 + lane) * 8 + (tile & 1) * 4;
        if (additive) acc = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<uint2*>(dst) =
            make_uint2((uint32_t)f32_to_bf16(-acc[0]) | ((uint32_t)f32_to_bf16(-acc[1]) << 16),
                       (uint32_t)f32_to_bf16(-acc[2]) | ((uint32_t)f32_to_bf16(-acc[3]) << 16));
        // Ut = T Diag(beta) V, value tile `tile`, accumulator layout; row tiles 2mp and
        // 2mp + 1 share one bf16 piece [mp][tile][lane] (the scans round U to bf16 for
        // their products as well)
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        u = mfma(tt[nt][0], bv[0], u);
        if (nt >= 2) u = mfma(tt[nt][1], bv[1], u);
        if (nt & 1) ut_out[((size_t)(nt >> 1) * 8 + tile) * 64 + lane] = pack_acc(ut_even, u);
        else ut_even = u;
      }
      if (tid < D) reinterpret_cast<float*>(w.gc + ci * kGcBytes)[tid] = exp2_fast(sm.G[C - 1][tid]);
      // the next item's raw q and k (loaded during this item) are prepared here,
      // where the vector ALU has room, rather than at its staging
      if constexpr (kRaw) {
        if (prefetch) prep_raw_qk(in);
      }
      if constexpr (kBwd) {
        // -W^T (M = channel, K = row): W tiles with rows in the accumulator, packed in pairs
        f32x4 wr[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          wr[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
          wr[nt] = mfma(tt[nt][0], abkg[0], wr[nt]);
          if (nt >= 2) wr[nt] = mfma(tt[nt][1], abkg[1], wr[nt]);
        }
        if (additive) wr[0] = wr[1] = wr[2] = wr[3] = f32x4{0.f, 0.f, 0.f, 0.f};  // W = 0
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          *reinterpret_cast<bf16x8*>(w.wt + ci * kKdBytes + ((size_t)(tile * 2 + s2) * 64 + lane) * 16) =
              pack_acc(-wr[2 * s2], -wr[2 * s2 + 1]);
      }
    }
    if constexpr (kBwd) {
      // the reverse pass's other operands, from LDS only
      {
        // A_qk^T as the reverse scan's A operand (M = row j, K = row r, kpos
        // order) from the upper triangle of A, one tile per wave; columns r < j
        // hold A_kk there and are zero in A_qk^T
        const int m = wave >> 1, s2 = wave & 1, j = 16 * m + li;
        const float4 a = *reinterpret_cast<const float4*>(&sm.A[j][32 * s2 + 4 * lg]);
        const float4 b = *reinterpret_cast<const float4*>(&sm.A[j][32 * s2 + 16 + 4 * lg]);
        float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (32 * s2 + kpos(lg, e) < j) f[e] = 0.f;
        *reinterpret_cast<bf16x8*>(w.aqt + ci * kAqBytes + ((size_t)wave * 64 + lane) * 16) = pack8(f);
      }
      // the units not taken earlier: 24 (three per wave), or all 32 (four per wave)
      if constexpr (kEarlyUnits) {
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          const int idx = 3 * wv + x;
          bwd_unit(idx < 12 ? idx : idx + 4);
        }
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) bwd_unit(x < 2 ? 2 * wv + x : 16 + 2 * wv + (x - 2));
      }
    }
  }
}

// LDS use (≈ 159 KiB) allows one workgroup (two waves per SIMD) per CU.
template <int kGate, bool kAdd, bool kRaw, bool kBwd>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta, float gate_min, int32_t N, int H,
    Workspace w, const int32_t* __restrict__ seq_start, const int32_t* __restrict__ seq_end,
    const int32_t* __restrict__ chunk_off, const int32_t* __restrict__ cu, int32_t T, int32_t cap,
    int fused) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  const Header hd{seq_start, seq_end, chunk_off};
  prep_role<kGate, kAdd, kRaw, kBwd>(q, k, v, g, beta, gate_min, N, H, w, hd, cu, T, cap,
                                     fused != 0, smem_raw, blockIdx.x, gridDim.x);
}

// What the prep needs to build the sequence header itself (fused = 1) instead of
// reading the one index_kernel wrote.
struct PrepIndex {
  const int32_t* cu;
  int32_t T;
  int32_t cap;
  int fused;
};

template <int kGate, bool kAdd, bool kRaw, bool kBwd = false>
kda_status_t launch_prep(unsigned grid, const void* q, const void* k, const void* v, const void* g,
                         const void* beta, float gate_min, int32_t N, int H, const Workspace& w,
                         const PrepIndex& ix, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};  // devices on which the limit is raised
  kda_status_t st = allow_dynamic_lds(reinterpret_cast<const void*>(prep_kernel<kGate, kAdd, kRaw, kBwd>),
                                      sizeof(PrepSmem), lds_set, "hipFuncSetAttribute(prep)");
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL((prep_kernel<kGate, kAdd, kRaw, kBwd>), dim3(grid), dim3(kPrepThreads),
                     sizeof(PrepSmem), stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), g, beta,
                     gate_min, N, H, w, w.seq_start, w.seq_end, w.chunk_off, ix.cu, ix.T, ix.cap,
                     ix.fused);
  return check_launch("prep_kernel");
}

template <bool kRaw>
kda_status_t launch_prep_variant(uint32_t flags, unsigned grid, const void* q, const void* k,
                                 const void* v, const void* g, const void* beta, float gate_min,
                                 int32_t N, int H, const Workspace& w, const PrepIndex& ix,
                                 hipStream_t s) {
  const bool add = flags & KDA_ADDITIVE;
#define KDA_PREP(G, A) launch_prep<G, A, kRaw>(grid, q, k, v, g, beta, gate_min, N, H, w, ix, s)
  if (flags & KDA_GATE_SCALAR) return add ? KDA_PREP(kGateScalar, true) : KDA_PREP(kGateScalar, false);
  if (flags & KDA_GATE_NONE) return add ? KDA_PREP(kGateNone, true) : KDA_PREP(kGateNone, false);
  return add ? KDA_PREP(kGateChannel, true) : KDA_PREP(kGateChannel, false);
#undef KDA_PREP
}

// ------------------------------------------------------------------ 3. scan
// A workgroup of WAVES waves owns 16 * NT * WAVES state columns of one
// (sequence n, head h); each wave owns NT tiles of 16 columns.  The per-chunk
// operands that every column needs (-W, Q*Gam, Kd^T, A_qk), the workgroup's
// Ut tiles and Gam_C are copied from the workspace into LDS with direct
// global->LDS loads, double buffered: the copy for chunk c+1 is in flight
// while chunk c is computed from the other buffer.  More waves per workgroup
// share one copy; more tiles per wave reuse each operand register for NT
// MFMAs, so fewer LDS bytes are read per unit of work.
//
// Block index b -> head_lin = b % NH, group = b / NH, so the column groups of
// a head land on the same XCD when NH is a multiple of 8 (workgroups are dealt
// to XCDs round-robin) and share its L2.
template <int WAVES, int NT>
struct ScanBuf {
  static constexpr int kTiles = WAVES * NT;  // 16-column tiles per workgroup
  // Ut goes through LDS when both buffers fit; otherwise each wave loads its
  // own Ut tiles into registers one chunk ahead.
  static constexpr bool kUtInLds = kTiles <= 4;
  bf16x8 wn[16][64];                        // [m*4 + s][lane]
  bf16x8 qg[16][64];                        // [m*4 + s][lane]
  bf16x8 kd[16][64];                        // [t*2 + s'][lane]
  bf16x8 aq[8][64];                         // [m*2 + s'][lane]
  bf16x8 ut[2][kUtInLds ? kTiles : 1][64];  // [row tile pair][local column tile][lane]
  f32x4 gc[32];                             // Gam_C
};

__device__ __forceinline__ void dma16(const uint8_t* src, void* lds_dst) {
  // each lane copies 16 bytes; lane i lands at lds_dst + 16 i
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// Copies of chunk `ci` into `dst`, in two parts: part 0 = -W and Q*Gam, part 1 =
// Kd^T, A_qk, Ut (when in LDS) and Gam_C.  Pieces of 1 KiB are dealt to waves.
template <int WAVES, int NT, int PART>
__device__ __forceinline__ void issue_chunk(const Workspace& w, size_t ci, int group,
                                            ScanBuf<WAVES, NT>* dst, int wave, int lane) {
  constexpr int kTiles = WAVES * NT;
  const int off = lane * 16;
  if (PART == 0) {
    const uint8_t* wn = w.wn + ci * kWnBytes;
    const uint8_t* qg = w.qg + ci * kQgBytes;
#pragma unroll
    for (int i = 0; i < (32 + WAVES - 1) / WAVES; ++i) {
      const int p = wave + WAVES * i;  // wave-uniform
      if (p < 16) dma16(wn + p * 1024 + off, &dst->wn[p][0]);
      else if (p < 32) dma16(qg + (p - 16) * 1024 + off, &dst->qg[p - 16][0]);
    }
  } else {
    constexpr int kPieces = 24 + (ScanBuf<WAVES, NT>::kUtInLds ? 2 * kTiles : 0);
    const uint8_t* kd = w.kd + ci * kKdBytes;
    const uint8_t* aq = w.aq + ci * kAqBytes;
    const uint8_t* ut = w.ut + ci * kUtBytes;
#pragma unroll
    for (int i = 0; i < (kPieces + WAVES - 1) / WAVES; ++i) {
      const int p = wave + WAVES * i;  // wave-uniform
      if (p < 16) dma16(kd + p * 1024 + off, &dst->kd[p][0]);
      else if (p < 24) dma16(aq + (p - 16) * 1024 + off, &dst->aq[p - 16][0]);
      else if (p < kPieces) {
        const int q = p - 24, mp = q / kTiles, tl = q % kTiles;
        dma16(ut + (size_t)((mp * 8 + group * kTiles + tl) * 64) * 16 + off, &dst->ut[mp][tl][0]);
      }
    }
    if (wave == WAVES - 1 && lane < 32) dma16(w.gc + ci * kGcBytes + off, &dst->gc[0]);
  }
}

template <int WAVES, int NT>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(1, 1))) void scan_kernel(
    int32_t N, int H, Workspace w, float* __restrict__ states, int32_t num_slots,
    const int32_t* __restrict__ slots, uint32_t flags, uint16_t* __restrict__ o) {
  using Buf = ScanBuf<WAVES, NT>;
  // Two separately declared buffers (not one indexed array): the compiler can
  // then see that the copies into one never alias reads of the other and does
  // not wait for the copies before unrelated LDS accesses.
  constexpr int kCols = 16 * WAVES * NT;     // columns of this workgroup
  __shared__ Buf buf0, buf1;
  __shared__ uint16_t out0[C][kCols], out1[C][kCols];  // staged bf16 outputs of a chunk
  const int NH = N * H;
  const int head_lin = blockIdx.x % NH;
  const int group = blockIdx.x / NH;
  const int n = head_lin / H, h = head_lin - n * H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  int col[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) col[i] = 16 * (group * WAVES * NT + wave * NT + i) + li;

  const int start = w.seq_start[n], end = w.seq_end[n], nch = w.seq_nch[n];
  const int cbase = w.chunk_off[n];
  const int slot = slots ? slots[n] : n;
  const bool slot_ok = states != nullptr && slot >= 0 && slot < num_slots;
  float* Sg = slot_ok ? states + ((size_t)slot * H + h) * (size_t)(D * D) : nullptr;

  // state slices: S[i][t] lane holds rows 16t + 4lg + jj of column col[i]
  f32x4 S[NT][8];
  if (slot_ok && (flags & KDA_READ_INITIAL_STATE)) {  // uniform branch; all loads in flight
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) S[i][t][jj] = Sg[(size_t)(16 * t + 4 * lg + jj) * D + col[i]];
  } else {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t) S[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Outputs of chunk c are staged as bf16 in an LDS tile and stored, as whole
  // 16-byte row pieces, early in chunk c + 1 so that they retire while it
  // computes.  Pieces of rows past the sequence end go to the workspace sink,
  // which keeps the stores free of branches.
  constexpr int kRowPieces = kCols / 8;      // 16-byte pieces per row
  constexpr int kStores = C * kRowPieces / (64 * WAVES);
  static_assert(C * kRowPieces % (64 * WAVES) == 0, "store split");
  auto store_rows = [&](const uint16_t (*ob)[kCols], int base) {
#pragma unroll
    for (int x = 0; x < kStores; ++x) {
      const int u = tid + 64 * WAVES * x;
      const int r = u / kRowPieces, pc = u % kRowPieces, tok = base + r;
      uint4* dst = tok < end
          ? reinterpret_cast<uint4*>(o + ((size_t)tok * H + h) * D + 16 * group * WAVES * NT + 8 * pc)
          : reinterpret_cast<uint4*>(w.sink) + (tid & 15);
      *dst = *reinterpret_cast<const uint4*>(&ob[r][8 * pc]);
    }
  };

  constexpr bool kUtInLds = Buf::kUtInLds;
  bf16x8 Unext[NT][2];
  auto load_ut = [&](size_t ci) {  // this wave's Ut tiles, straight into registers
    const bf16x8* ut = reinterpret_cast<const bf16x8*>(w.ut + ci * kUtBytes);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) Unext[i][mp] = ut[(mp * 8 + (col[i] >> 4)) * 64 + lane];
  };

  // One chunk: compute from B (copied during the previous chunk), copy the next
  // chunk into Bn, store the outputs of the previous chunk (staged in Bn).
  auto chunk_step = [&](const Buf& B, Buf& Bn, uint16_t (*ob)[kCols], const uint16_t (*obn)[kCols],
                        int lc) {
    // chunk lc has landed (this wave's copies; only the previous chunk's output
    // stores may still be in flight), then all waves' copies are visible and
    // every wave is done with Bn
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    const bool more = lc + 1 < nch;
    const size_t ci_next = (size_t)(cbase + lc + 1) * H + h;
    f32x4 U[NT][4];
    if (!kUtInLds) {
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int mp = 0; mp < 2; ++mp) unpack_acc(Unext[i][mp], U[i][2 * mp], U[i][2 * mp + 1]);
      if (more) load_ut(ci_next);
    }

    // Operands of this chunk: LDS -> registers in batches issued ahead of the
    // MFMAs that consume them (the scheduling barriers keep the compiler from
    // interleaving one read per MFMA); the copies for the next chunk are issued
    // in two parts after each batch of reads.
    bf16x8 a_wn[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) a_wn[x] = B.wn[x][lane];
    if (kUtInLds) {
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int mp = 0; mp < 2; ++mp)
          unpack_acc(B.ut[mp][kUtInLds ? wave * NT + i : 0][lane], U[i][2 * mp], U[i][2 * mp + 1]);
    }
    bf16x8 sb[NT][4];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) sb[i][s] = pack_acc(S[i][2 * s], S[i][2 * s + 1]);
    bf16x8 a_qg[16], a_aq[6];
#pragma unroll
    for (int x = 0; x < 16; ++x) a_qg[x] = B.qg[x][lane];
#pragma unroll
    for (int x = 0; x < 6; ++x) a_aq[x] = B.aq[x < 2 ? 2 * x : x + 2][lane];  // [0],[2],[4..7]
    __builtin_amdgcn_sched_barrier(0);
    // the previous chunk's outputs (staged in obn), early: they retire during this chunk
    if (lc > 0) store_rows(obn, start + (lc - 1) * C);
    if (more) issue_chunk<WAVES, NT, 0>(w, ci_next, group, &Bn, wave, lane);
    __builtin_amdgcn_sched_barrier(0);

    // U = Ut - W S   (consecutive MFMAs go to different accumulators)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < NT; ++i) U[i][m] = mfma(a_wn[m * 4 + s], sb[i][s], U[i][m]);
    // O, first part: (Q*Gam) S
    f32x4 O[NT][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < NT; ++i) O[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < NT; ++i) O[i][m] = mfma(a_qg[m * 4 + s], sb[i][s], O[i][m]);
    bf16x8 a_kd[16];
    f32x4 gcv[8];
#pragma unroll
    for (int x = 0; x < 16; ++x) a_kd[x] = B.kd[x][lane];
#pragma unroll
    for (int t = 0; t < 8; ++t) gcv[t] = B.gc[4 * t + lg];
    __builtin_amdgcn_sched_barrier(0);
    if (more) issue_chunk<WAVES, NT, 1>(w, ci_next, group, &Bn, wave, lane);
    __builtin_amdgcn_sched_barrier(0);

    bf16x8 ub[NT][2];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      ub[i][0] = pack_acc(U[i][0], U[i][1]);
      ub[i][1] = pack_acc(U[i][2], U[i][3]);
#pragma unroll
      for (int t = 0; t < 8; ++t) S[i][t] = S[i][t] * gcv[t];
    }
    // S' = Diag(Gam_C) S + Kd^T U  (the chain's critical path: issued first)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < NT; ++i) S[i][t] = mfma(a_kd[t * 2 + s2], ub[i][s2], S[i][t]);
    // O += A_qk U   (A_qk rows 0-31 have no entries in columns 32-63)
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      O[i][0] = mfma(a_aq[0], ub[i][0], O[i][0]);
      O[i][1] = mfma(a_aq[1], ub[i][0], O[i][1]);
      O[i][2] = mfma(a_aq[2], ub[i][0], O[i][2]);
      O[i][3] = mfma(a_aq[4], ub[i][0], O[i][3]);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      O[i][2] = mfma(a_aq[3], ub[i][1], O[i][2]);
      O[i][3] = mfma(a_aq[5], ub[i][1], O[i][3]);
    }

    // stage this chunk's outputs (bf16) in ob, stored during the next chunk
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          ob[16 * m + 4 * lg + jj][16 * (wave * NT + i) + li] = f32_to_bf16(O[i][m][jj]);
  };

  if (nch > 0) {
    issue_chunk<WAVES, NT, 0>(w, (size_t)cbase * H + h, group, &buf0, wave, lane);
    issue_chunk<WAVES, NT, 1>(w, (size_t)cbase * H + h, group, &buf0, wave, lane);
    if (!kUtInLds) load_ut((size_t)cbase * H + h);
  }
  for (int lc = 0; lc < nch; lc += 2) {
    chunk_step(buf0, buf1, out0, out1, lc);
    if (lc + 1 < nch) chunk_step(buf1, buf0, out1, out0, lc + 1);
  }
  if (nch > 0) {
    lds_barrier();
    store_rows((nch - 1) & 1 ? out1 : out0, start + (nch - 1) * C);
  }

  if (slot_ok && (flags & KDA_WRITE_FINAL_STATE)) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Sg[(size_t)(16 * t + 4 * lg + jj) * D + col[i]] = S[i][t][jj];
  }
}

// State-only warp-specialised scan: the backward's forward state pass.  Per
// chunk only the state recurrence is on the serial path: U = Ut - W S and S' =
// Diag(Gam_C) S + Kd^T U.  The compute waves store the bf16 MFMA operands they
// form anyway, S at the chunk start and U, for the gradient kernel.  The loaders
// copy -W, Kd^T, the workgroup's Ut tiles and Gam_C.  (The forward's few-chains
// scan, scan_out_kernel, keeps the same ring and forms the outputs instead.)
constexpr int kStateRing = 3;

template <int CW, int NT>
struct StateLds {
  static constexpr int kTiles = CW * NT;
  struct Buf {
    bf16x8 wn[16][64];         // [m*4 + s][lane]
    bf16x8 kd[16][64];         // [t*2 + s'][lane]
    bf16x8 ut[2][kTiles][64];  // [row tile pair][local column tile][lane]
    f32x4 gc[32];              // Gam_C
  };
  Buf buf[kStateRing];  // ring: the copies run kStateRing - 1 chunks ahead of the compute wave
  uint8_t sink[1024];   // target of the L2 warming loads (never read)
};

// s_waitcnt vmcnt(n) for a wave-uniform n <= 23 (the count is an immediate; its
// bits 5:4 sit in bits 15:14 of the encoding)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    case 15: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
    case 16: __builtin_amdgcn_s_waitcnt(0x4F70); break;
    case 17: __builtin_amdgcn_s_waitcnt(0x4F71); break;
    case 18: __builtin_amdgcn_s_waitcnt(0x4F72); break;
    case 19: __builtin_amdgcn_s_waitcnt(0x4F73); break;
    case 20: __builtin_amdgcn_s_waitcnt(0x4F74); break;
    case 21: __builtin_amdgcn_s_waitcnt(0x4F75); break;
    case 22: __builtin_amdgcn_s_waitcnt(0x4F76); break;
    default: __builtin_amdgcn_s_waitcnt(0x4F77); break;
  }
}

// kWarm (the backward's paired launch): wave CW + LW, beside the LW loaders,
// pulls the dO rows of the reverse pass's chunks into the caches, four of its
// chunks per step of this pass (which runs about twice as fast), waiting for
// none of them until its end, so that the reverse pass, which reads them as
// scattered 32-byte pieces, does not find them in HBM.
template <int CW, int NT, int LW, bool kWarm = false>
__device__ __forceinline__ void scan_state_role(int blk, uint8_t* smem_raw, int32_t N, int H,
                                                const Workspace& w, float* __restrict__ states,
                                                int32_t num_slots,
                                                const int32_t* __restrict__ slots, uint32_t flags,
                                                const uint16_t* __restrict__ d_o = nullptr) {
  using L = StateLds<CW, NT>;
  using Buf = typename L::Buf;
  constexpr int kTiles = L::kTiles;
  L& sl = *reinterpret_cast<L*>(smem_raw);
  const int NH = N * H;
  const int head_lin = blk % NH;
  const int group = blk / NH;
  const int n = head_lin / H, h = head_lin - n * H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int nch = w.seq_nch[n];
  const int cbase = w.chunk_off[n];

  if (kWarm && __builtin_amdgcn_readfirstlane(wave) == CW + LW) {
    // --------------------------------------------------------- dO warming
    // Lanes: chunk 4 lc + l / 16 of the reverse order (chunk nch - 1 - that),
    // row 8 group + (l % 16) / 2 of the head, its 128-byte line l % 2.
    auto warm = [&](int lc) {
      const int chunk = max(nch - 1 - (4 * lc + (lane >> 4)), 0);
      const int t0 = w.seq_start[n] + chunk * C;
      const int last = min(C, w.seq_end[n] - t0) - 1;
      const int row = min(8 * group + ((lane & 15) >> 1), last);
      dma16(reinterpret_cast<const uint8_t*>(d_o + ((size_t)(t0 + row) * H + h) * D + 64 * (lane & 1)),
            &sl.sink[0]);
    };
    if (nch > 0) warm(0);
    lds_barrier();
    for (int lc = 0; lc < nch; ++lc) {
      if (4 * (lc + 1) < nch) warm(lc + 1);
      lds_barrier();
    }
    wait_vm(0);  // no load into LDS outlives the wave
    return;
  }
  if (wave >= CW) {
    // ------------------------------------------------------------ loaders
    const int lw = wave - CW;
    const int off = lane * 16;
    constexpr int kPieces = 32 + 2 * kTiles;  // 1 KiB pieces of a chunk's operands
    auto issue = [&](size_t ci, Buf* dst) {
      const uint8_t* wn = w.wn + ci * kWnBytes;
      const uint8_t* kd = w.kd + ci * kKdBytes;
      const uint8_t* ut = w.ut + ci * kUtBytes;
#pragma unroll
      for (int i = 0; i < (kPieces + LW - 1) / LW; ++i) {
        const int p = lw + LW * i;  // wave-uniform
        if (p < 16) dma16(wn + p * 1024 + off, &dst->wn[p][0]);
        else if (p < 32) dma16(kd + (p - 16) * 1024 + off, &dst->kd[p - 16][0]);
        else if (p < kPieces) {
          const int x = p - 32, mp = x / kTiles, tl = x % kTiles;
          dma16(ut + (size_t)((mp * 8 + group * kTiles + tl) * 64) * 16 + off, &dst->ut[mp][tl][0]);
        }
      }
      if (lw == LW - 1 && lane < 32) dma16(w.gc + ci * kGcBytes + off, &dst->gc[0]);
    };
    // copies this wave issues per chunk: its pieces, plus Gam_C for the last wave
    const int mine = (kPieces - lw + LW - 1) / LW + (lw == LW - 1 ? 1 : 0);
    constexpr int kAhead = kStateRing - 1;  // chunks in flight beyond the current one
    static_assert(((kPieces + LW - 1) / LW + 1) * (kAhead - 1) <= 15, "graded wait range");
    // Chunk c is in buf[c % kStateRing].  At the end of the step before chunk lc,
    // chunks up to lc + kAhead - 1 have been issued; waiting for all but this
    // wave's newest (in-flight chunks - 1) x `mine` copies means chunk lc has
    // landed while the later ones stay in flight.
    for (int c = 0; c < kAhead && c < nch; ++c) issue((size_t)(cbase + c) * H + h, &sl.buf[c]);
    wait_vm(mine * (min(nch, kAhead) - 1 > 0 ? min(nch, kAhead) - 1 : 0));  // chunk 0 landed
    lds_barrier();
    for (int lc = 0; lc < nch; ++lc) {
      // chunk lc + 1 must land by the end of this step; lc + 2 .. lc + kAhead may fly
      const int nxt = lc + kAhead;
      if (nxt < nch) issue((size_t)(cbase + nxt) * H + h, &sl.buf[nxt % kStateRing]);
      const int newest = min(nch - 1, nxt) - (lc + 1);  // chunks issued after lc + 1
      wait_vm(newest > 0 ? mine * newest : 0);
      lds_barrier();
    }
    return;
  }

  // -------------------------------------------------------------- compute
  int ctile[NT], col[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    ctile[i] = group * kTiles + wave * NT + i;
    col[i] = 16 * ctile[i] + li;
  }
  const int slot = slots ? slots[n] : n;
  const bool slot_ok = states != nullptr && slot >= 0 && slot < num_slots;
  float* Sg = slot_ok ? states + ((size_t)slot * H + h) * (size_t)(D * D) : nullptr;
  f32x4 S[NT][8];
  if (slot_ok && (flags & KDA_READ_INITIAL_STATE)) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) S[i][t][jj] = Sg[(size_t)(16 * t + 4 * lg + jj) * D + col[i]];
  } else {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t) S[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  lds_barrier();

  auto chunk_step = [&](const Buf& B, size_t ci) {
    f32x4 U[NT][4];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int mp = 0; mp < 2; ++mp)
        unpack_acc(B.ut[mp][wave * NT + i][lane], U[i][2 * mp], U[i][2 * mp + 1]);
    bf16x8 a_wn[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) a_wn[x] = B.wn[x][lane];
    bf16x8 sb[NT][4];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) sb[i][s] = pack_acc(S[i][2 * s], S[i][2 * s + 1]);
    bf16x8 a_kd[16];
    f32x4 gcv[8];
#pragma unroll
    for (int x = 0; x < 16; ++x) a_kd[x] = B.kd[x][lane];
#pragma unroll
    for (int t = 0; t < 8; ++t) gcv[t] = B.gc[4 * t + lg];
    __builtin_amdgcn_sched_barrier(0);
    bf16x8* sc = reinterpret_cast<bf16x8*>(w.sc + ci * kScBytes);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) sc[(ctile[i] * 4 + s) * 64 + lane] = sb[i][s];
    // U = Ut - W S   (consecutive MFMAs go to different accumulators)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < NT; ++i) U[i][m] = mfma(a_wn[m * 4 + s], sb[i][s], U[i][m]);
    bf16x8 ub[NT][2];
    bf16x8* uc = reinterpret_cast<bf16x8*>(w.uc + ci * kUcBytes);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      ub[i][0] = pack_acc(U[i][0], U[i][1]);
      ub[i][1] = pack_acc(U[i][2], U[i][3]);
      uc[(ctile[i] * 2 + 0) * 64 + lane] = ub[i][0];
      uc[(ctile[i] * 2 + 1) * 64 + lane] = ub[i][1];
#pragma unroll
      for (int t = 0; t < 8; ++t) S[i][t] = S[i][t] * gcv[t];
    }
    // S' = Diag(Gam_C) S + Kd^T U
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < NT; ++i) S[i][t] = mfma(a_kd[t * 2 + s2], ub[i][s2], S[i][t]);
    lds_barrier();
  };
  for (int lc = 0; lc < nch; ++lc)
    chunk_step(sl.buf[lc % kStateRing], (size_t)(cbase + lc) * H + h);

  if (slot_ok && (flags & KDA_WRITE_FINAL_STATE)) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Sg[(size_t)(16 * t + 4 * lg + jj) * D + col[i]] = S[i][t][jj];
  }
}

// State scan with the outputs formed beside it.  A workgroup owns NCT tiles of 16
// state columns of one (sequence, head) (the columns evolve independently, so
// the workgroups of a head need no exchange).  Waves 0..NCT-1 carry one column
// tile of the state each, as in scan_state_role, and per chunk c leave S_c (at
// the chunk start) and U_c in LDS as the bf16 B operands they form anyway; the
// next two waves form the rows 0-31 and 32-63 of O_c = (Q*Gam)_c S_c +
// A_qk,c U_c one step later, with the MFMA order of the single-pass scan, from
// Q*Gam and A_qk tiles that they load from the workspace into registers two
// chunks ahead, and leave their outputs in LDS as bf16 rows, which the next wave
// stores as 16-byte row pieces one step later; the other waves keep a ring of the
// chain's operands filled.  Nothing of S or U goes through memory, and no
// separate output launch re-reads the chunk operands.
constexpr int kScanOutThreads = 512;

template <int NCT>
struct ScanOutLds {
  // NCT = 1: four buffers, and the state wave reads chunk c's operands at the end
  // of step c - 1 (they land while it waits at the barrier); NCT = 2: three
  // buffers (the LDS holds no more), read at the top of the step.
  static constexpr int kRing = NCT == 1 ? 4 : 3;
  static constexpr bool kPipe = NCT == 1;
  // one chunk's operands; 1 KiB pieces in the loaders' order (Gam_C is padded to
  // a whole piece so that every lane of its loader stores)
  struct Buf {
    bf16x8 wn[16][64];      // [m*4 + s][lane]
    bf16x8 kd[16][64];      // [t*2 + s'][lane]
    bf16x8 ut[2][NCT][64];  // [row tile pair][this group's column tile][lane]
    f32x4 gc[32];           // Gam_C
    f32x4 gc_pad[32];
  };
  Buf buf[kRing];
  bf16x8 xs[2][6 * NCT][64];  // per chunk parity: S_c as 4 B operands per tile (K = dk), then U_c as 2
  uint16_t ob[2][C][16 * NCT];  // per chunk parity: the output waves' bf16 outputs of the chunk
};

template <int NCT>
__device__ __forceinline__ void scan_out_role(int blk, uint8_t* smem_raw, int32_t N, int H,
                                              const Workspace& w, float* __restrict__ states,
                                              int32_t num_slots, const int32_t* __restrict__ slots,
                                              uint32_t flags, uint16_t* __restrict__ o) {
  using L = ScanOutLds<NCT>;
  using Buf = typename L::Buf;
  constexpr int kOutRing = L::kRing;
  constexpr bool kPipe = L::kPipe;
  constexpr int kOutWave0 = NCT, kOutWaves = 2;
  constexpr int kStoreWave = kOutWave0 + kOutWaves;
  constexpr int LW = kScanOutThreads / 64 - kStoreWave - 1;
  L& sl = *reinterpret_cast<L*>(smem_raw);
  const int NH = N * H;
  const int head_lin = blk % NH;
  const int group = blk / NH;  // NCT consecutive 16-column tiles of the state
  const int n = head_lin / H, h = head_lin - n * H;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = w.seq_nch[n];
  const int cbase = w.chunk_off[n];

  const int start = w.seq_start[n], end = w.seq_end[n];
  if (wave >= kStoreWave) {
    // -------------------------------------------------- copies (and stores)
    // Pieces of 1 KiB, dealt to the copy waves in turn: 0-15 -W, 16-31 Kd^T, then
    // this group's 2 NCT Ut pieces, then Gam_C (512 B, copied twice so that every
    // lane has a part).  A buffer holds them in this order, piece p at byte
    // 1024 p.  The copies go straight to LDS, kRing - 1 chunks ahead: a chunk's
    // copies take longer than one chunk step to land, and a CU takes them in
    // faster the more waves issue them.
    const int lw = wave - kStoreWave;
    constexpr int kCopyWaves = LW + 1;
    constexpr int kUt0 = 32, kGc = kUt0 + 2 * NCT, kPieces = kGc + 1;
    constexpr int kPer = (kPieces + kCopyWaves - 1) / kCopyWaves;
    const int mine = (kPieces - lw + kCopyWaves - 1) / kCopyWaves;  // this wave's pieces
    static_assert(sizeof(Buf) == kPieces * 1024, "piece p at byte 1024 p");
    // per piece: its array's address at chunk-head 0, that array's stride per
    // chunk-head, and the lane's byte offset (fixed for the wave)
    const uint8_t* pbase[kPer];
    uint32_t pstride[kPer], ploff[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = lw + kCopyWaves * i;  // wave-uniform
      if (p < 16) {
        pbase[i] = w.wn + p * 1024;
        pstride[i] = (uint32_t)kWnBytes;
      } else if (p < 32) {
        pbase[i] = w.kd + (p - 16) * 1024;
        pstride[i] = (uint32_t)kKdBytes;
      } else if (p < kGc) {
        const int mp = (p - kUt0) / NCT, ct = (p - kUt0) % NCT;
        pbase[i] = w.ut + (size_t)(mp * 8 + group * NCT + ct) * 1024;
        pstride[i] = (uint32_t)kUtBytes;
      } else {
        pbase[i] = w.gc;
        pstride[i] = (uint32_t)kGcBytes;
      }
      ploff[i] = (uint32_t)(p < kGc ? lane : (lane & 31)) * 16;
    }
    auto issue = [&](int c) {
      const size_t ci = (size_t)(cbase + c) * H + h;
      uint8_t* dst = reinterpret_cast<uint8_t*>(&sl.buf[c % kOutRing]);
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lw + kCopyWaves * i < kPieces)
          dma16(pbase[i] + ci * pstride[i] + ploff[i], dst + (lw + kCopyWaves * i) * 1024);
    };
    // Wave kStoreWave also stores the outputs: chunk c's, staged by the output
    // waves during step c + 1, go out as 16-byte row pieces during step c + 2 (the
    // staging tile has a slot per chunk parity), so the output waves never wait
    // on a store.  Every lane stores (rows past the sequence end into the
    // workspace sink), so that the waits below count the stores exactly.
    constexpr int kRowPieces = 2 * NCT;  // 16-byte pieces per output row
    const bool stores = lw == 0;
    auto store_chunk = [&](int c) {
      const int t0 = start + c * C, rows = min(C, end - t0);
#pragma unroll
      for (int xx = 0; xx < kRowPieces; ++xx) {
        const int pc = lane + 64 * xx, r = pc / kRowPieces, piece = pc % kRowPieces;
        const uint4 v4 = *reinterpret_cast<const uint4*>(&sl.ob[c & 1][r][8 * piece]);
        uint4* dst = r < rows
            ? reinterpret_cast<uint4*>(o + ((size_t)(t0 + r) * H + h) * D + 16 * NCT * group + 8 * piece)
            : reinterpret_cast<uint4*>(w.sink) + (lane & 15);
        *dst = v4;
      }
    };
    // Chunk c + kLead must have landed by the barrier that ends step c (kPipe: the
    // state wave reads chunk c + 2 at the end of step c + 1), so each wait leaves
    // only the newest chunk's copies (and the step's stores) in flight.
    constexpr int kAhead = kOutRing - 1;
    constexpr int kLead = kPipe ? 2 : 1;
    static_assert(kPer * (kAhead - kLead) + kRowPieces <= 23, "graded wait range");
    for (int c = 0; c < kAhead && c < nch; ++c) issue(c);
    wait_vm(mine * (min(nch, kAhead) - min(nch, kLead)));  // chunks before kLead landed
    lds_barrier();
    for (int lc = 0; lc < nch; ++lc) {
      const int nxt = lc + kAhead;
      if (nxt < nch) issue(nxt);
      const bool st = stores && lc >= 2;
      if (st) store_chunk(lc - 2);
      // chunk lc + kLead landed
      wait_vm(mine * (min(nch, nxt + 1) - min(nch, lc + kLead + 1)) + (st ? kRowPieces : 0));
      lds_barrier();
    }
    if (stores && nch >= 2) store_chunk(nch - 2);
    lds_barrier();  // the last chunk's outputs are staged
    if (stores && nch >= 1) store_chunk(nch - 1);
    return;
  }

  if (wave >= kOutWave0) {
    // ------------------------------------------------------------ outputs
    // rows 32 hf .. 32 hf + 31 of every column tile; chunk c's Q*Gam and A_qk tiles
    // sit in register set c % 2, loaded at step c - 1.  A_qk tiles (block row R,
    // column half s'): half 0 needs (0,0) (1,0); half 1 needs (2,0) (2,1) (3,0)
    // (3,1) (rows 0-31 have no entries in columns 32-63).
    const int hf = wave - kOutWave0;
    bf16x8 qg0[8], aq0[4], qg1[8], aq1[4];
    auto load_ops = [&](bf16x8* qgr, bf16x8* aqr, int c) {
      const size_t ci = (size_t)(cbase + c) * H + h;
      const bf16x8* qg = reinterpret_cast<const bf16x8*>(w.qg + ci * kQgBytes) + 8 * hf * 64;
      const bf16x8* aq = reinterpret_cast<const bf16x8*>(w.aq + ci * kAqBytes);
#pragma unroll
      for (int x = 0; x < 8; ++x) qgr[x] = qg[x * 64 + lane];
      // four tiles on both halves (half 0 uses the first two), so that the waits
      // for a register set count the same loads on both
#pragma unroll
      for (int x = 0; x < 4; ++x) aqr[x] = aq[(hf ? 4 + x : 2 * x) * 64 + lane];
    };
    // rows of O_c from slot c % 2 of the exchange and the operand tiles qgr, aqr
    auto out_chunk = [&](const bf16x8* qgr, const bf16x8* aqr, int c) {
      const bf16x8(*x)[64] = sl.xs[c & 1];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        bf16x8 sb[4], ub[2];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) sb[s2] = x[4 * ct + s2][lane];
        ub[0] = x[4 * NCT + 2 * ct][lane];
        ub[1] = x[4 * NCT + 2 * ct + 1][lane];
        f32x4 O[2];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) O[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) O[mm] = mfma(qgr[mm * 4 + s2], sb[s2], O[mm]);
        if (hf == 0) {
          O[0] = mfma(aqr[0], ub[0], O[0]);
          O[1] = mfma(aqr[1], ub[0], O[1]);
        } else {
          O[0] = mfma(aqr[0], ub[0], O[0]);
          O[1] = mfma(aqr[2], ub[0], O[1]);
          O[0] = mfma(aqr[1], ub[1], O[0]);
          O[1] = mfma(aqr[3], ub[1], O[1]);
        }
        // stage as bf16 rows for the store wave
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            sl.ob[c & 1][32 * hf + 16 * mm + 4 * lg + jj][16 * ct + li] = f32_to_bf16(O[mm][jj]);
      }
    };
    // loads on every path (past the last chunk: the last again), so that the wait
    // for one register set counts the other set's loads
    const int last = nch - 1;
    if (nch > 0) {
      load_ops(qg0, aq0, 0);
      load_ops(qg1, aq1, min(1, last));
    }
    lds_barrier();
    // after the barrier that ends chunk c: O_c, then chunk c + 2's tiles into the set
    // just used; unrolled by two so that every register set is named
    for (int c = 0; c < nch; c += 2) {
      lds_barrier();  // end of chunk c
      out_chunk(qg0, aq0, c);
      load_ops(qg0, aq0, min(c + 2, last));
      if (c + 1 < nch) {
        lds_barrier();  // end of chunk c + 1
        out_chunk(qg1, aq1, c + 1);
        load_ops(qg1, aq1, min(c + 3, last));
      }
    }
    lds_barrier();  // the last chunk's outputs are staged for the store wave
    return;
  }

  // ------------------------------------------------------ state (wave ct < NCT)
  const int ct = wave;
  const int col = 16 * (NCT * group + ct) + li;
  const int slot = slots ? slots[n] : n;
  const bool slot_ok = states != nullptr && slot >= 0 && slot < num_slots;
  float* Sg = slot_ok ? states + ((size_t)slot * H + h) * (size_t)(D * D) : nullptr;
  f32x4 S[8];
  if (slot_ok && (flags & KDA_READ_INITIAL_STATE)) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) S[t][jj] = Sg[(size_t)(16 * t + 4 * lg + jj) * D + col];
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  lds_barrier();
  f32x4 U[4];
  bf16x8 a_wn[16], a_kd[16];
  f32x4 gcv[8];
  auto read_ops = [&](int c) {
    const Buf& B = sl.buf[c % kOutRing];
    unpack_acc(B.ut[0][ct][lane], U[0], U[1]);
    unpack_acc(B.ut[1][ct][lane], U[2], U[3]);
#pragma unroll
    for (int xx = 0; xx < 16; ++xx) a_wn[xx] = B.wn[xx][lane];
#pragma unroll
    for (int xx = 0; xx < 16; ++xx) a_kd[xx] = B.kd[xx][lane];
#pragma unroll
    for (int t = 0; t < 8; ++t) gcv[t] = B.gc[4 * t + lg];
  };
  if (kPipe && nch > 0) read_ops(0);
  for (int lc = 0; lc < nch; ++lc) {
    if (!kPipe) read_ops(lc);
    bf16x8(*x)[64] = sl.xs[lc & 1];
    bf16x8 sb[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) sb[s2] = pack_acc(S[2 * s2], S[2 * s2 + 1]);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) x[4 * ct + s2][lane] = sb[s2];
    // U = Ut - W S   (consecutive MFMAs go to different accumulators)
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
      for (int m = 0; m < 4; ++m) U[m] = mfma(a_wn[m * 4 + s2], sb[s2], U[m]);
    bf16x8 ub[2];
    ub[0] = pack_acc(U[0], U[1]);
    ub[1] = pack_acc(U[2], U[3]);
    x[4 * NCT + 2 * ct][lane] = ub[0];
    x[4 * NCT + 2 * ct + 1][lane] = ub[1];
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] = S[t] * gcv[t];
    // S' = Diag(Gam_C) S + Kd^T U
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t) S[t] = mfma(a_kd[t * 2 + s2], ub[s2], S[t]);
    if constexpr (kPipe) {
      // the next chunk's operands, issued after this chunk's products: they land
      // while the wave waits at the barrier (which waits for its LDS writes only)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the exchange tiles are written
      if (lc + 1 < nch) read_ops(lc + 1);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      lds_barrier();
    }
  }
  lds_barrier();  // the closing barrier of the output and store waves
  if (slot_ok && (flags & KDA_WRITE_FINAL_STATE)) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Sg[(size_t)(16 * t + 4 * lg + jj) * D + col] = S[t][jj];
  }
}

template <int NCT>
__global__ __launch_bounds__(kScanOutThreads) void scan_out_kernel(
    int32_t N, int H, Workspace w, float* __restrict__ states, int32_t num_slots,
    const int32_t* __restrict__ slots, uint32_t flags, uint16_t* __restrict__ o) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  scan_out_role<NCT>(blockIdx.x, smem_raw, N, H, w, states, num_slots, slots, flags, o);
}

// NCT tiles of 16 columns per workgroup: N * H * 8 / NCT workgroups.
template <int NCT>
kda_status_t launch_scan_out(int32_t N, int H, const Workspace& w, float* states,
                             int32_t num_slots, const int32_t* slots, uint32_t flags, void* o,
                             hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  kda_status_t st = allow_dynamic_lds(reinterpret_cast<const void*>(scan_out_kernel<NCT>),
                                      sizeof(ScanOutLds<NCT>), lds_set, "hipFuncSetAttribute(scan)");
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL(scan_out_kernel<NCT>, dim3((unsigned)(N * H * (D / (16 * NCT)))),
                     dim3(kScanOutThreads), sizeof(ScanOutLds<NCT>), stream, N, H, w, states,
                     num_slots, slots, flags, static_cast<uint16_t*>(o));
  return check_launch("scan_out_kernel");
}

template <int WAVES, int NT>
kda_status_t launch_scan(int32_t N, int H, const Workspace& w, float* states, int32_t num_slots,
                         const int32_t* slots, uint32_t flags, void* o, hipStream_t stream) {
  constexpr int kGroups = D / (16 * WAVES * NT);
  hipLaunchKernelGGL((scan_kernel<WAVES, NT>), dim3((unsigned)(N * H * kGroups)), dim3(64 * WAVES),
                     0, stream, N, H, w, states, num_slots, slots, flags, static_cast<uint16_t*>(o));
  return check_launch("scan_kernel");
}

// ------------------------------------------------------------------ 4. backward
// The pages stop at the forward pass; the gradient is reverse-mode
// differentiation of the chunk algebra above.  With X = dL/dS at a chunk's end,
//   reverse pass   dU = A_qk^T dO + Kd X,   X <- (Q*Gam)^T dO + Diag(Gam_C) X - W^T dU
// (the transpose of the forward pass U = Ut - W S, S <- Diag(Gam_C) S + Kd^T U), and
// inside a chunk, with R = Diag(beta)(V - (K*Gam) S) and U = (I + A_kk)^-1 R:
//   dR = T^T dU,  dA_kk = -dR U^T,  dV = Diag(beta) dR,  Z = dR S^T,
//   dA_qk = dO U^T,  d(Q*Gam) = dO S^T,  dKd = U X^T,  dGam_C = rowsum(X * S),
// and the decayed products A_qk, M_kk send their cotangents to q, k and the
// cumulative gates.  The forward state pass runs first (the state-only scan
// stores S at every chunk start and U); the reverse pass stores X and dU; the
// gradient kernel then handles every (chunk, head) independently.

// Reverse pass: 8 workgroups of 16 value columns per (sequence, head), chunks
// walked from the last to the first.  Wave 0 carries X = dL/dS; the other seven
// keep a ring of kGradRing chunk buffers filled, two chunks ahead of it:
//  * waves 3..6 copy Kd, -W^T and Gam_C into LDS with direct global->LDS
//    loads, two chunks ahead; wave 7 copies the chunk's dO rows (this
//    workgroup's columns, 64 rows 32 bytes each) kDoAhead chunks ahead into a
//    ring of their own, and with them pulls the lines of that chunk's blocks
//    into L2 (the forward pass beside it pulls the dO rows earlier still).  A
//    wave's loads complete in issue order, so rows copied far ahead need a wave
//    that waits for nothing issued after them;
//  * waves 1 and 2 form the chunk's products that do not depend on X, for this
//    workgroup's columns: A_qk^T dO (the start of dU) and (Q*Gam)^T dO (X's
//    increment), from operand tiles they load into registers a step ahead and
//    the dO rows in LDS, and write them to LDS in the accumulator layout.
// Wave 0 then does the two products on the chain per chunk, as the forward pass.
// The role and piece of a wave are taken from a scalar copy of its index, so
// each choice is a branch, never a lane mask (a matrix instruction in a
// masked-off block still writes its accumulator, and the copies' waits count
// every issued load).
constexpr int kGradRing = 3;
constexpr int kDoAhead = 5;        // dO rows are copied this many chunks ahead of wave 0
constexpr int kDoRing = kDoAhead;  // chunk c's dO rows in slot c % kDoRing
struct GradScanLds {
  struct Buf {
    bf16x8 kdr[16][64];   // Kd      [m*4 + s][lane]   (M = rows, K = dk)
    bf16x8 wt[16][64];    // -W^T    [t*2 + s2][lane]  (M = dk, K = rows)
    f32x4 p[4][64];       // A_qk^T dO      [m][lane]  (rows 16m + 4lg + jj, column li)
    f32x4 r[8][64];       // (Q*Gam)^T dO   [t][lane]  (channels 16t + 4lg + jj)
    f32x4 gc[32];         // Gam_C
  };
  Buf buf[kGradRing];
  uint16_t dob[kDoRing][C][16];  // dO rows, this workgroup's 16 columns
  uint8_t sink[1024];            // target of the L2 prefetch loads (never read)
};

__device__ __forceinline__ void scan_grad_role(int blk, uint8_t* smem_raw, int32_t N, int H,
                                               const Workspace& w, const uint16_t* __restrict__ d_o,
                                               const float* __restrict__ d_final,
                                               float* __restrict__ d_initial) {
  using Buf = GradScanLds::Buf;
  GradScanLds& sl = *reinterpret_cast<GradScanLds*>(smem_raw);
  const int NH = N * H;
  const int head_lin = blk % NH;
  const int group = blk / NH;
  const int n = head_lin / H, h = head_lin - n * H;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = w.seq_nch[n];
  const int cbase = w.chunk_off[n];
  const int s_start = w.seq_start[n], s_end = w.seq_end[n];
  // the k-th chunk processed is chunk nch - 1 - k, in buffer k % kGradRing
  auto chunk_ci = [&](int k) { return (size_t)(cbase + nch - 1 - k) * H + h; };

  if (wave == 1 || wave == 2) {
    // ------------------------------------------------------ product waves
    // wave mw: (Q*Gam)^T dO for channel tiles 4mw .. 4mw + 3 and A_qk^T dO for
    // row tiles 2mw, 2mw + 1 (both K halves; those of row tiles 2, 3 with K
    // rows 0..31 are stored zeros)
    const int mw = wave - 1;
    struct Ops {
      bf16x8 qa[8];   // (Q*Gam)^T tiles [t*2 + s2], t = 4mw + x / 2
      bf16x8 aq[4];   // A_qk^T tiles [m*2 + s2], m = 2mw + x / 2
    };
    auto load = [&](int k, Ops& o) {
      const size_t ci = chunk_ci(k);
      const bf16x8* qgt = reinterpret_cast<const bf16x8*>(w.qgt + ci * kKdBytes);
      const bf16x8* aqt = reinterpret_cast<const bf16x8*>(w.aqt + ci * kAqBytes);
#pragma unroll
      for (int x = 0; x < 8; ++x) o.qa[x] = qgt[(8 * mw + x) * 64 + lane];
#pragma unroll
      for (int x = 0; x < 4; ++x) o.aq[x] = aqt[(4 * mw + x) * 64 + lane];
    };
    auto emit = [&](const Ops& o, int k, Buf& dst) {
      // dO as a B operand: K = row (kpos order), N = column li
      const uint16_t(&rows)[C][16] = sl.dob[k % kDoRing];
      bf16x8 dob[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = rows[32 * s2 + kpos(lg, e)][li];
        dob[s2] = __builtin_bit_cast(bf16x8, t);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma(o.qa[2 * x], dob[0], acc);
        acc = mfma(o.qa[2 * x + 1], dob[1], acc);
        dst.r[4 * mw + x][lane] = acc;
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma(o.aq[2 * x], dob[0], acc);
        acc = mfma(o.aq[2 * x + 1], dob[1], acc);
        dst.p[2 * mw + x][lane] = acc;
      }
    };
    if (nch == 0) {
      lds_barrier();
      lds_barrier();
      return;
    }
    // Chunk k + 1's products are written during step k while chunk k + 2's
    // operand tiles load; the two register sets alternate.  The loads are
    // issued on every step (the last steps re-load the last chunk), so the
    // wait before a product always leaves exactly one set in flight.
    Ops o0, o1;
    load(0, o0);
    load(min(1, nch - 1), o1);
    lds_barrier();  // dO rows of chunks 0 and 1 landed
    emit(o0, 0, sl.buf[0]);
    lds_barrier();
    for (int k = 0; k < nch; k += 2) {
      load(min(k + 2, nch - 1), o0);
      if (k + 1 < nch) emit(o1, k + 1, sl.buf[(k + 1) % kGradRing]);
      lds_barrier();
      if (k + 1 < nch) {
        load(min(k + 3, nch - 1), o1);
        if (k + 2 < nch) emit(o0, k + 2, sl.buf[(k + 2) % kGradRing]);
        lds_barrier();
      }
    }
    return;
  }
  if (wave == 7) {
    // ------------------------------------------------- dO rows, L2 prefetch
    // dO: two pieces per chunk, rows 0..31 and 32..63, lane -> row lane / 2, 8 columns.
    // With them, the chunk's operand blocks are pulled into L2 for the copies
    // that follow kDoAhead - 2 steps later: every 128-byte line of the head's
    // Kd, -W^T, (Q*Gam)^T (two 64-line units each), A_qk^T, dO rows (two units:
    // the lines holding columns 0..63 and 64..127) and Gam_C (4 lines), ten
    // units of one load each (lane -> line), units 2g and 2g + 1 by column
    // group g < 5 of the head (the eight groups share the L2 of one XCD).
    const int npf = group < 5 ? 2 : 0;
    auto issue_do = [&](int k) {
      const int t0 = s_start + (nch - 1 - k) * C;
      const int last = min(C, s_end - t0) - 1;  // rows past the end re-read the last row
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int row = min(32 * half + (lane >> 1), last);
        const uint16_t* src = d_o + ((size_t)(t0 + row) * H + h) * D + 16 * group + 8 * (lane & 1);
        dma16(reinterpret_cast<const uint8_t*>(src), &sl.dob[k % kDoRing][32 * half][0]);
      }
      if (npf) {
        const size_t ci = chunk_ci(k);
        const size_t line = (size_t)lane * 128;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int unit = 2 * group + x;  // scalar
          const uint8_t* src;
          if (unit < 2) src = w.kdr + ci * kKdBytes + unit * 8192 + line;
          else if (unit < 4) src = w.wt + ci * kKdBytes + (unit - 2) * 8192 + line;
          else if (unit < 6) src = w.qgt + ci * kKdBytes + (unit - 4) * 8192 + line;
          else if (unit == 6) src = w.aqt + ci * kAqBytes + line;
          else if (unit < 9) {
            const int row = min(lane, last);
            src = reinterpret_cast<const uint8_t*>(d_o + ((size_t)(t0 + row) * H + h) * D + 64 * (unit - 7));
          } else {
            src = w.gc + ci * kGcBytes + (size_t)min(lane, 3) * 128;
          }
          dma16(src, &sl.sink[0]);
        }
      }
    };
    static_assert(2 + 4 * (kDoAhead - 2) <= 23, "graded wait range");
    if (nch == 0) {
      lds_barrier();
      lds_barrier();
      return;
    }
    // loads issued after chunk j's dO rows, up to chunk `newest`
    auto after = [&](int j, int newest) { return npf + (2 + npf) * max(newest - j, 0); };
    const int first = min(nch, kDoAhead);
    for (int k = 0; k < first; ++k) issue_do(k);
    wait_vm(after(min(1, nch - 1), first - 1));  // dO rows of chunks 0 and 1 landed
    lds_barrier();
    lds_barrier();
    for (int k = 0; k < nch; ++k) {
      // by the end of this step chunk k + 2's dO rows have landed; later ones may fly
      if (k + kDoAhead < nch) issue_do(k + kDoAhead);
      wait_vm(k + 2 < nch ? after(k + 2, min(nch - 1, k + kDoAhead)) : 0);
      lds_barrier();
    }
    return;
  }
  if (wave >= 3) {
    // --------------------------------------------------------- copy waves
    // the 32 pieces of Kd and -W^T are dealt round-robin to the four waves,
    // Gam_C (half a piece) goes with the last
    const int cw = wave - 3;
    const int off = lane * 16;
    const int nrest = cw == 3 ? 9 : 8;
    auto issue = [&](int k, Buf* dst) {
      const size_t ci = chunk_ci(k);
      const uint8_t* kdr = w.kdr + ci * kKdBytes;
      const uint8_t* wt = w.wt + ci * kKdBytes;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = cw + 4 * i;  // scalar
        if (p < 16) dma16(kdr + p * 1024 + off, &dst->kdr[p][0]);
        else dma16(wt + (p - 16) * 1024 + off, &dst->wt[p - 16][0]);
      }
      if (cw == 3 && lane < 32) dma16(w.gc + ci * kGcBytes + off, &dst->gc[0]);
    };
    if (nch == 0) {
      lds_barrier();
      lds_barrier();
      return;
    }
    issue(0, &sl.buf[0]);
    if (nch > 1) issue(1, &sl.buf[1]);
    lds_barrier();
    wait_vm(nch > 1 ? nrest : 0);  // chunk 0 landed
    lds_barrier();
    for (int k = 0; k < nch; ++k) {
      // chunk k + 1 must land by the end of this step; k + 2 may fly
      if (k + 2 < nch) {
        issue(k + 2, &sl.buf[(k + 2) % kGradRing]);
        wait_vm(nrest);
      } else {
        wait_vm(0);
      }
      lds_barrier();
    }
    return;
  }

  // -------------------------------------------------------------- compute
  const int col = 16 * group + li;
  f32x4 X[8];
  const size_t sb = ((size_t)n * H + h) * (size_t)(D * D);
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      X[t][jj] = d_final ? d_final[sb + (size_t)(16 * t + 4 * lg + jj) * D + col] : 0.f;
  lds_barrier();
  lds_barrier();

  for (int k = 0; k < nch; ++k) {
    const Buf& B = sl.buf[k % kGradRing];
    const size_t ci = chunk_ci(k);
    bf16x8 xb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xb[s] = pack_acc(X[2 * s], X[2 * s + 1]);
    bf16x8* dsc = reinterpret_cast<bf16x8*>(w.dsc + ci * kScBytes);
#pragma unroll
    for (int s = 0; s < 4; ++s) dsc[(group * 4 + s) * 64 + lane] = xb[s];
    // dU = A_qk^T dO + Kd X
    f32x4 dU[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) dU[m] = B.p[m][lane];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m) dU[m] = mfma(B.kdr[m * 4 + s][lane], xb[s], dU[m]);
    bf16x8 ub[2];
    bf16x8* duc = reinterpret_cast<bf16x8*>(w.duc + ci * kUcBytes);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      ub[s2] = pack_acc(dU[2 * s2], dU[2 * s2 + 1]);
      duc[(group * 2 + s2) * 64 + lane] = ub[s2];
    }
    // X <- Diag(Gam_C) X + (Q*Gam)^T dO - W^T dU
#pragma unroll
    for (int t = 0; t < 8; ++t) X[t] = X[t] * B.gc[4 * t + lg] + B.r[t][lane];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t) X[t] = mfma(B.wt[t * 2 + s2][lane], ub[s2], X[t]);
    lds_barrier();
  }
  if (d_initial) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) d_initial[sb + (size_t)(16 * t + 4 * lg + jj) * D + col] = X[t][jj];
  }
}

// The forward state pass and the reverse pass need nothing from each other (the
// reverse pass carries dL/dS without S), so one launch runs both side by side:
// blocks [0, 8 N H) walk the chunks forward, the rest backward.
constexpr int kScanPairThreads = 64 * 8;
__global__ __launch_bounds__(kScanPairThreads) void scan_pair_kernel(
    int32_t N, int H, Workspace w, float* __restrict__ states, int32_t num_slots,
    const int32_t* __restrict__ slots, uint32_t flags, const uint16_t* __restrict__ d_o,
    const float* __restrict__ d_final, float* __restrict__ d_initial) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  const int nf = N * H * (D / 16);
  if ((int)blockIdx.x < nf)
    scan_state_role<1, 1, 6, true>(blockIdx.x, smem_raw, N, H, w, states, num_slots, slots, flags, d_o);
  else
    scan_grad_role(blockIdx.x - nf, smem_raw, N, H, w, d_o, d_final, d_initial);
}

// Gradient kernel: one workgroup of 8 waves per (chunk, head).  Phases:
//  0  stage K, Q, the gates (running sums) and beta; the T^T operand tiles to registers
//  1  two halves of 64 value columns: dR = T^T dU (-> dV, dbeta), then
//     Z = dR S^T, d(Q*Gam) = dO S^T, dKd = U X^T, dA_qk = dO U^T, dR U^T, dGam_C
//  2  elementwise terms of dq, dk, dG; dbeta terms; dA_qk and dM = beta dA_kk to LDS
//  3  the decayed products: blocks below the diagonal on MFMA with the decay split
//     at a block boundary (both factors <= 1), diagonal blocks on MFMA when the
//     block's gate spread allows it, else element by element
//  4  reverse running sum of dG (the gates are running sums), stores.
// Lane layout of the per-element results: rows 16m + 4lg + jj (m = 0..3),
// channel 16 * wave + li.
constexpr int kGradThreads = 512;
constexpr int KB = D + 8;  // bf16 row pitch of K, Q (16-byte aligned rows)
constexpr int HB = 72;     // bf16 row pitch of 64-column tiles

struct GradSmem {
  uint16_t K[C][KB];   // k (phase 4: dk staging)
  uint16_t Q[C][KB];   // q (phase 4: dq staging)
  float G[C][GP];      // running gate sums (phase 4: dG)
  float bs[C];
  float db[C];         // dbeta
  float dgl[D];        // dG of the chunk's last row from Gam_C
  float spr[kGradThreads / 64];
  union {
    uint16_t dR[C][KB];   // phase 1: all 128 value columns
  } x;
  union {
    struct {
      uint16_t dO[C][HB];
      uint16_t U[C][HB];
      uint16_t S[D][HB];
      uint16_t dS[D][HB];
    } h;                  // phase 1
    struct {
      uint16_t dAq[C][HB];
      uint16_t dAqT[C][HB];
      uint16_t dM[C][HB];
      uint16_t dMT[C][HB];
    } a;                  // phases 2-3
    float tot[4][D];      // running sums (phases 0 and 4)
  } y;
};

// Workspace blocks the gradient kernel reads.
struct GradWs {
  const uint8_t* tm;
  const uint8_t* mkk;
  const uint8_t* sc;
  const uint8_t* uc;
  const uint8_t* dsc;
  const uint8_t* duc;
};

// v[i] summed over the 16 lanes of a row group (lanes li = 0..15); lane li
// returns the sum of index li.  A butterfly that halves the values carried at
// every step: 15 shuffles instead of 64.
__device__ __forceinline__ float row_sum16_transposed(const float (&v)[16], int li) {
  float a[8], b[4], c2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool hi = li & 8;
    a[i] = (hi ? v[i + 8] : v[i]) + __shfl_xor(hi ? v[i] : v[i + 8], 8, 64);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool hi = li & 4;
    b[i] = (hi ? a[i + 4] : a[i]) + __shfl_xor(hi ? a[i] : a[i + 4], 4, 64);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bool hi = li & 2;
    c2[i] = (hi ? b[i + 2] : b[i]) + __shfl_xor(hi ? b[i] : b[i + 2], 2, 64);
  }
  const bool hi = li & 1;
  return (hi ? c2[1] : c2[0]) + __shfl_xor(hi ? c2[0] : c2[1], 1, 64);
}

// Workgroup barrier after which every LDS value is re-read: the empty asm keeps
// the compiler from carrying values loaded before it (which would only raise
// register pressure: LDS reads are cheap).
__device__ __forceinline__ void block_sync() {
  __syncthreads();
  asm volatile("" ::: "memory");
}

// x where ok, else all-zero bits: a per-component mask (a select of whole vectors
// can be lowered through private memory).
__device__ __forceinline__ uint4 keep_if(uint4 x, bool ok) {
  const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
  return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ float bfv(uint16_t b) { return bf16_to_f32(b); }

// Variants (compile time): kGate = kGateScalar reads a [T, H] gate and returns dg
// [T, H] (the channel sum of the per-channel gradient: the gate is broadcast over
// channels); kGateNone reads and returns no gate; kAdd (u = v, no beta): U = V,
// so T = I, W = 0, dV = dU, and the terms through (K*Gam) S and A_kk vanish.
template <int kGate, bool kAdd>
__global__ __launch_bounds__(kGradThreads) void grad_kernel(
    int32_t N, int H, GradWs w, const int32_t* __restrict__ seq_start,
    const int32_t* __restrict__ seq_end, const int32_t* __restrict__ chunk_off,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const uint16_t* __restrict__ d_o,
    uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  GradSmem& sm = *reinterpret_cast<GradSmem*>(smem_raw);
  float pb[16];  // dbeta partials of rows 16m + 4lg + jj at [4m + jj], over this lane's columns
#pragma unroll
  for (int i = 0; i < 16; ++i) pb[i] = 0.f;
  const Header hd{seq_start, seq_end, chunk_off};
  const int item = blockIdx.x;
  if (item >= hd.chunk_off[N] * H) return;  // uniform
  const ItemPos pos = locate(hd, N, H, item);
  const size_t ci = (size_t)item;
  const int c = pos.c;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const size_t row0 = (size_t)pos.t0 * H + pos.h;  // token-row of the chunk's first row
  const size_t rs = (size_t)H;                     // token-row stride

  // ---- 0. staging (rows past the end are zero).  Loads are issued for every
  // row (rows past the end re-read the last row) and the zeros are selected
  // afterwards, so that no load sits behind a branch and they overlap.
  {
    uint4 kx[2], qx[2];
    uint4 gx[4];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int u = tid + kGradThreads * x, r = min(u >> 4, c - 1), cc = (u & 15) * 8;
      const size_t gi = (row0 + r * rs) * D + cc;
      kx[x] = nt_load4(k + gi);
      qx[x] = nt_load4(q + gi);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int u = tid + kGradThreads * x, r = min(u >> 5, c - 1), cc = (u & 31) * 4;
      if (kGate == kGateChannel) {
        gx[x] = nt_load4(g + (row0 + r * rs) * D + cc);
      } else if (kGate == kGateScalar) {
        const uint32_t b = __float_as_uint(g[row0 + r * rs]);
        gx[x] = make_uint4(b, b, b, b);
      } else {
        gx[x] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int u = tid + kGradThreads * x, r = u >> 4, cc = (u & 15) * 8;
      *reinterpret_cast<uint4*>(&sm.K[r][cc]) = keep_if(kx[x], r < c);
      *reinterpret_cast<uint4*>(&sm.Q[r][cc]) = keep_if(qx[x], r < c);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int u = tid + kGradThreads * x, r = u >> 5, cc = (u & 31) * 4;
      *reinterpret_cast<uint4*>(&sm.G[r][cc]) = keep_if(gx[x], r < c);
    }
  }
  if (tid < C) {
    const float bt = kAdd ? 1.f : beta[row0 + min(tid, c - 1) * rs];
    sm.bs[tid] = tid < c ? bt : 0.f;
    sm.db[tid] = 0.f;
  }
  if (tid < D) sm.dgl[tid] = 0.f;
  // T^T as the A operand of dR = T^T dU (M = row r, K = row j, kpos order), tiles
  // stored by the prep; T^T is zero for K rows 0..31 of row tiles 2 and 3.
  bf16x8 tT[4][2];
  {
    const bf16x8* tmt = reinterpret_cast<const bf16x8*>(w.tm + ci * kTmBytes);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        if (m < 2 || s2 == 1) tT[m][s2] = nt_load16(tmt + (m * 2 + s2) * 64 + lane);
  }
  block_sync();
  {
    const int col = tid & 127, qt = tid >> 7;
    float xs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) xs[i] = sm.G[16 * qt + i][col];
#pragma unroll
    for (int i = 1; i < 16; ++i) xs[i] += xs[i - 1];
    sm.y.tot[qt][col] = xs[15];
    block_sync();
    float base = 0.f;
    for (int j = 0; j < qt; ++j) base += sm.y.tot[j][col];
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.G[16 * qt + i][col] = xs[i] + base;
    float sp = xs[0] - xs[15];  // gate spread of this channel inside block qt
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sp = fmaxf(sp, __shfl_xor(sp, off, 64));
    if (lane == 0) sm.spr[wave] = sp;  // waves 2qt and 2qt + 1 cover block qt
  }
  block_sync();  // the running sums are read before the tile area is reused

  // ---- 1. dR = T^T dU for value column tile `wave` (dU straight from the reverse
  // pass), then dV = Diag(beta) dR and the dbeta term rowsum(dR * V)
  {
    const bf16x8* duc = reinterpret_cast<const bf16x8*>(w.duc + ci * kUcBytes);
    const bf16x8 dub0 = nt_load16(duc + (wave * 2 + 0) * 64 + lane);
    const bf16x8 dub1 = nt_load16(duc + (wave * 2 + 1) * 64 + lane);
    const int cg = 16 * wave + li;
    uint16_t vx[4][4];  // V at this lane's dR positions, loaded before any is used
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        vx[m][jj] = nt_load(v + (row0 + min(16 * m + 4 * lg + jj, c - 1) * rs) * D + cg);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f32x4 r2 = {0.f, 0.f, 0.f, 0.f};
      if (m < 2) r2 = mfma(tT[m][0], dub0, r2);
      r2 = mfma(tT[m][1], dub1, r2);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * m + 4 * lg + jj;
        const float x = r2[jj];
        sm.x.dR[r][cg] = f32_to_bf16(x);
        if (!kAdd) pb[4 * m + jj] += r < c ? x * bf16_to_f32(vx[m][jj]) : 0.f;  // += dR V
        if (r < c) dv[(row0 + r * rs) * D + cg] = f32_to_bf16(sm.bs[r] * x);
      }
    }
  }

  // the two halves of the value columns
  f32x4 aZ[4], aQ[4], aK[4], aAq[2], aAk[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) aZ[m] = aQ[m] = aK[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  aAq[0] = aAq[1] = aAk[0] = aAk[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dgc = 0.f;  // rowsum(X * S) for channel tid >> 2, over this thread's columns
  const u16x8* uc = reinterpret_cast<const u16x8*>(w.uc + ci * kUcBytes);
  const u16x8* sc = reinterpret_cast<const u16x8*>(w.sc + ci * kScBytes);
  const u16x8* dsc = reinterpret_cast<const u16x8*>(w.dsc + ci * kScBytes);
  for (int hf = 0; hf < 2; ++hf) {
    {
      const int r = tid >> 3, cc = (tid & 7) * 8;
      const uint4 x = nt_load4(d_o + (row0 + min(r, c - 1) * rs) * D + 64 * hf + cc);
      *reinterpret_cast<uint4*>(&sm.y.h.dO[r][cc]) = keep_if(x, r < c);
    }
    {
      // U from the B-operand layout: [column tile][row half][lane], rows in kpos order
      const int ctl = tid >> 7, s2 = (tid >> 6) & 1, ln = tid & 63;
      const u16x8 u8 = nt_load16(uc + ((4 * hf + ctl) * 2 + s2) * 64 + ln);
      const int cl = 16 * ctl + (ln & 15), g4 = ln >> 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.y.h.U[32 * s2 + kpos(g4, e)][cl] = u8[e];
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      // S and X from [column tile][row block of 32][lane], rows in kpos order
      const int u = tid + kGradThreads * x, ctl = u >> 8, s = (u >> 6) & 3, ln = u & 63;
      const size_t idx = (size_t)((4 * hf + ctl) * 4 + s) * 64 + ln;
      const u16x8 s8 = nt_load16(sc + idx), d8 = nt_load16(dsc + idx);
      const int cl = 16 * ctl + (ln & 15), g4 = ln >> 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 32 * s + kpos(g4, e);
        sm.y.h.S[r][cl] = s8[e];
        sm.y.h.dS[r][cl] = d8[e];
      }
    }
    block_sync();
    // products over the half's 64 columns; plain operands, K = column
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int cc = 32 * ks + 8 * lg, ccg = 64 * hf + cc;
      const bf16x8 bS = lds8(&sm.y.h.S[16 * wave + li][cc]);
      const bf16x8 bX = lds8(&sm.y.h.dS[16 * wave + li][cc]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        aZ[m] = mfma(lds8(&sm.x.dR[16 * m + li][ccg]), bS, aZ[m]);
        aQ[m] = mfma(lds8(&sm.y.h.dO[16 * m + li][cc]), bS, aQ[m]);
        aK[m] = mfma(lds8(&sm.y.h.U[16 * m + li][cc]), bX, aK[m]);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int tt = wave + 8 * x, R = tt >> 2, J = tt & 3;
        if (J <= R) {
          const bf16x8 bU = lds8(&sm.y.h.U[16 * J + li][cc]);
          aAq[x] = mfma(lds8(&sm.y.h.dO[16 * R + li][cc]), bU, aAq[x]);
          aAk[x] = mfma(lds8(&sm.x.dR[16 * R + li][ccg]), bU, aAk[x]);
        }
      }
    }
    {
      const int i = tid >> 2, c0 = (tid & 3) * 16;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) s += bfv(sm.y.h.S[i][c0 + e]) * bfv(sm.y.h.dS[i][c0 + e]);
      dgc += s;
    }
    block_sync();  // the tiles are read before the next half (or phase 2) overwrites them
  }
  dgc += __shfl_xor(dgc, 1, 64);
  dgc += __shfl_xor(dgc, 2, 64);
  if ((tid & 3) == 0) atomicAdd(&sm.dgl[tid >> 2], dgc * fast_exp(sm.G[C - 1][tid >> 2]));

  // ---- 2. elementwise terms
  const int ich = 16 * wave + li;
  const float GC = sm.G[C - 1][ich];
  f32x4 oq[4], okk[4], oG[4];
  float kdsum = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * m + 4 * lg + jj;
      const float Gr = sm.G[r][ich], gam = fast_exp(Gr), ed = fast_exp(GC - Gr);
      const float kr = bfv(sm.K[r][ich]), qr = bfv(sm.Q[r][ich]), br = sm.bs[r];
      const float z = aZ[m][jj], dqg = aQ[m][jj], dkd = aK[m][jj];
      const float dkg = kAdd ? 0.f : -br * z;  // no (K*Gam) S term in the additive write
      const float kdv = kr * ed;
      oq[m][jj] = dqg * gam;
      okk[m][jj] = dkg * gam + dkd * ed;
      oG[m][jj] = (dqg * qr + dkg * kr) * gam - dkd * kdv;
      kdsum += dkd * kdv;
      if (!kAdd) pb[4 * m + jj] -= kr * gam * z;  // dbeta_r -= sum_i (K*Gam)[r,i] Z[r,i]
    }
  kdsum += __shfl_xor(kdsum, 16, 64);
  kdsum += __shfl_xor(kdsum, 32, 64);
  if (lg == 0) atomicAdd(&sm.dgl[ich], kdsum);
  {
    const float* mk = reinterpret_cast<const float*>(w.mkk + ci * kMkBytes);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int tt = wave + 8 * x, R = tt >> 2, J = tt & 3, j = 16 * J + li;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * R + 4 * lg + jj;
        const bool low = J <= R;
        const float aq = low && j <= r ? aAq[x][jj] : 0.f;
        const float ak = !kAdd && low && j < r ? -aAk[x][jj] : 0.f;   // dA_kk = -(dR U^T)
        const float mv = !kAdd && low && j < r ? nt_load(mk + ((R * 4 + J) * 16 + 4 * lg + jj) * 16 + li) : 0.f;
        // dbeta_r += sum_j dA_kk[r,j] M_kk[r,j]; R is 0 or 1 (x = 0), 2 or 3 (x = 1)
        const float add = ak * mv;
        pb[8 * x + jj] += (R & 1) ? 0.f : add;
        pb[8 * x + 4 + jj] += (R & 1) ? add : 0.f;
        const uint16_t bq = f32_to_bf16(aq), bm = f32_to_bf16(sm.bs[r] * ak);
        sm.y.a.dAq[r][j] = bq;
        sm.y.a.dAqT[j][r] = bq;
        sm.y.a.dM[r][j] = bm;
        sm.y.a.dMT[j][r] = bm;
      }
    }
  }
  atomicAdd(&sm.db[16 * (li >> 2) + 4 * lg + (li & 3)], row_sum16_transposed(pb, li));
  block_sync();

  // ---- 3. decayed products
  // Row side: out row r of block R gets sum_j dA[r,j] k_j exp(G_r - G_j); split at
  // ref = 16R: exp(G_r - G_ref) <= 1 and exp(G_ref - G_j) <= 1 for j < ref, <= the
  // block's spread for the diagonal block (included only when that is safe).
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    const int ref = 16 * R;
    const bool diag = fmaxf(sm.spr[2 * R], sm.spr[2 * R + 1]) <= kMaxSpread;
    const int jend = diag ? ref + 16 : ref;  // K rows j < jend (R = 0 without diag: none)
    f32x4 accq = {0.f, 0.f, 0.f, 0.f}, acck = {0.f, 0.f, 0.f, 0.f};
    const float Gref = sm.G[ref][ich];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks >= ref + 16) continue;  // compile-time: no row of this K step is used
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * ks + 8 * lg + e;  // < 64: loaded for every lane, masked after
        const float kj = bfv(sm.K[j][ich]);
        const float ex = fast_exp(fminf(Gref - sm.G[j][ich], 88.f));
        f[e] = j < jend ? kj * ex : 0.f;
      }
      const bf16x8 b = pack8(f);
      accq = mfma(lds8(&sm.y.a.dAq[16 * R + li][32 * ks + 8 * lg]), b, accq);
      acck = mfma(lds8(&sm.y.a.dM[16 * R + li][32 * ks + 8 * lg]), b, acck);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = ref + 4 * lg + jj;
      const float fr = fast_exp(sm.G[r][ich] - Gref);
      const float xq = accq[jj] * fr, xk = acck[jj] * fr;
      oq[R][jj] += xq;
      okk[R][jj] += xk;
      oG[R][jj] += bfv(sm.Q[r][ich]) * xq + bfv(sm.K[r][ich]) * xk;
    }
  }
  // Column side: out row j of block J gets sum_r (dA_qk[r,j] q_r + dM[r,j] k_r)
  // exp(G_r - G_j); split at ref = 16J + 15.
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    const int ref = 16 * J + 15;
    const bool diag = fmaxf(sm.spr[2 * J], sm.spr[2 * J + 1]) <= kMaxSpread;
    const int rbeg = diag ? 16 * J : ref + 1;  // K rows r >= rbeg (J = 3 without diag: none)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const float Gref = sm.G[ref][ich];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks + 32 <= 16 * J) continue;  // compile-time: no row of this K step is used
      float fq[8], fk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 32 * ks + 8 * lg + e;  // < 64: loaded for every lane, masked after
        const bool ok = r >= rbeg;
        const float qr = bfv(sm.Q[r][ich]), kr = bfv(sm.K[r][ich]);
        const float ex = fast_exp(fminf(sm.G[r][ich] - Gref, 88.f));
        fq[e] = ok ? qr * ex : 0.f;
        fk[e] = ok ? kr * ex : 0.f;
      }
      acc = mfma(lds8(&sm.y.a.dAqT[16 * J + li][32 * ks + 8 * lg]), pack8(fq), acc);
      acc = mfma(lds8(&sm.y.a.dMT[16 * J + li][32 * ks + 8 * lg]), pack8(fk), acc);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 16 * J + 4 * lg + jj;
      const float x = acc[jj] * fast_exp(Gref - sm.G[j][ich]);
      okk[J][jj] += x;
      oG[J][jj] -= bfv(sm.K[j][ich]) * x;
    }
  }
  // Diagonal blocks with a gate spread too wide for the split: exact decay per
  // element (rare; kept rolled so that it does not add to the register load of
  // the common path).
#pragma unroll 1
  for (int m = 0; m < 4; ++m) {
    if (fmaxf(sm.spr[2 * m], sm.spr[2 * m + 1]) <= kMaxSpread) continue;  // uniform
    float aq4[4], ak4[4], ag4[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * m + 4 * lg + jj;
      const float Gr = sm.G[r][ich], kr = bfv(sm.K[r][ich]), qr = bfv(sm.Q[r][ich]);
      float sq = 0.f, sk = 0.f, scol = 0.f;
#pragma unroll 1
      for (int x = 0; x < 16; ++x) {
        const int j = 16 * m + x;
        const float Gj = sm.G[j][ich];
        // row side (j <= r) and column side (this lane's row as the column, j > r)
        const float er = fast_exp(fminf(Gr - Gj, 0.f));
        const float ec = fast_exp(fminf(Gj - Gr, 0.f));
        const float kj = bfv(sm.K[j][ich]), qj = bfv(sm.Q[j][ich]);
        if (j <= r) {
          sq += bfv(sm.y.a.dAq[r][j]) * kj * er;
          sk += bfv(sm.y.a.dM[r][j]) * kj * er;
        } else {
          scol += (bfv(sm.y.a.dAq[j][r]) * qj + bfv(sm.y.a.dM[j][r]) * kj) * ec;
        }
      }
      scol += bfv(sm.y.a.dAq[r][r]) * qr;  // the diagonal entry (exp(0) = 1)
      aq4[jj] = sq;
      ak4[jj] = sk + scol;
      ag4[jj] = qr * sq + kr * sk - kr * scol;
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
      if (mm == m) {  // uniform branch: compile-time register indices
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          oq[mm][jj] += aq4[jj];
          okk[mm][jj] += ak4[jj];
          oG[mm][jj] += ag4[jj];
        }
      }
  }
  block_sync();  // every read of K, Q, G and the dA tiles is done

  // ---- 4. dG -> dg by a reverse running sum; dq, dk staged for row stores
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * m + 4 * lg + jj;
      sm.G[r][ich] = oG[m][jj] + (r == C - 1 ? sm.dgl[ich] : 0.f);
      sm.K[r][ich] = f32_to_bf16(okk[m][jj]);
      sm.Q[r][ich] = f32_to_bf16(oq[m][jj]);
    }
  block_sync();
  if (kGate == kGateChannel) {
    const int col = tid & 127, qt = tid >> 7;
    float xs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) xs[i] = sm.G[16 * qt + i][col];
#pragma unroll
    for (int i = 14; i >= 0; --i) xs[i] += xs[i + 1];
    sm.y.tot[qt][col] = xs[0];
    block_sync();
    float base = 0.f;
    for (int j = qt + 1; j < 4; ++j) base += sm.y.tot[j][col];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * qt + i;
      if (r < c) dg[(row0 + r * rs) * D + col] = xs[i] + base;
    }
  } else if (kGate == kGateScalar) {
    // the channel sum of dG per row (8 threads per row), then the reverse running sum
    // over the 64 rows in one wave
    const int r = tid >> 3, part = tid & 7;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += sm.G[r][16 * part + i];
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    sum += __shfl_xor(sum, 4, 64);
    if (part == 0) sm.y.tot[0][r] = sum;
    block_sync();
    if (wave == 0) {
      float x = sm.y.tot[0][lane];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {  // suffix sum: lane l adds lane l + o
        const float y = __shfl_down(x, o, 64);
        if (lane + o < 64) x += y;
      }
      if (lane < c) dg[row0 + lane * rs] = x;
    }
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int u = tid + kGradThreads * x, r = u >> 4, cc = (u & 15) * 8;
    if (r < c) {
      const size_t gi = (row0 + r * rs) * D + cc;
      *reinterpret_cast<uint4*>(dk + gi) = *reinterpret_cast<const uint4*>(&sm.K[r][cc]);
      *reinterpret_cast<uint4*>(dq + gi) = *reinterpret_cast<const uint4*>(&sm.Q[r][cc]);
    }
  }
  if (!kAdd && tid < c) dbeta[row0 + tid * rs] = sm.db[tid];
}

}  // namespace

bool chunk_mfma_supported(int dk, int dv, int chunk, int io_dtype) {
  return dk == D && dv == D && chunk == C && io_dtype == KDA_BF16;
}

size_t chunk_mfma_workspace_bytes(int H, int32_t T, int32_t N) {
  const size_t ci = nchunks_max(T, N) * (size_t)H;
  return header_bytes(N) + align256(ci * kWnBytes) + align256(ci * kQgBytes) +
         align256(ci * kKdBytes) + align256(ci * kAqBytes) + align256(ci * kUtBytes) +
         align256(ci * kGcBytes) + 256;
}

kda_status_t launch_chunk_mfma(const kda_shape_t* sh, int32_t T, int32_t N, const int32_t* cu,
                               const void* q, const void* k, const void* v, const void* g,
                               const void* beta, bool raw, float gate_min, float* states,
                               int32_t num_slots, const int32_t* slots, uint32_t flags, void* o,
                               void* workspace, hipStream_t stream) {
  const int H = sh->num_heads;
  if (H > kMaxHeads) {
    set_error("kda_chunk_fwd: at most %d heads are supported (got %d)", kMaxHeads, H);
    return KDA_ERR_UNSUPPORTED;
  }
  Workspace w = carve(workspace, T, N, H);
  const size_t cap = nchunks_max(T, N);
  const size_t items = cap * (size_t)H;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int x = 0;
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && x > 0) ncu = x;
  }
  // few sequences: the prep builds the sequence header itself (no index launch)
  const PrepIndex ix{cu, T, (int32_t)cap, N <= kFuseMaxSeqs ? 1 : 0};
  kda_status_t st = KDA_OK;
  if (!ix.fused) {
    hipLaunchKernelGGL(index_kernel, dim3(1), dim3(64), 0, stream, cu, N, T, (int32_t)cap, w);
    st = check_launch("index_kernel");
    if (st != KDA_OK) return st;
  }
  // persistent prep: one workgroup per CU, each walks items with a grid stride
  const unsigned grid = (unsigned)(items < (size_t)ncu ? items : (size_t)ncu);
  st = raw ? launch_prep_variant<true>(flags, grid, q, k, v, g, beta, gate_min, N, H, w, ix, stream)
           : launch_prep_variant<false>(flags, grid, q, k, v, g, beta, gate_min, N, H, w, ix, stream);
  if (st != KDA_OK) return st;
  // Few chains: the serial chain of chunk steps is the critical path; each
  // head's state is split over 8 warp-specialised workgroups of 16 columns whose
  // state wave carries only the state while waves beside it form the outputs.
  // Up to one workgroup per CU at 4 per head: the same scan with 32 columns (two
  // state waves) per workgroup.  Many chains: one workgroup of 4 waves x 32
  // columns per head, which fetches each chunk's shared operands once.
  if (split_outputs(N, H))
    return launch_scan_out<1>(N, H, w, states, num_slots, slots, flags, o, stream);
  if ((size_t)N * H * 4 <= (size_t)ncu)
    return launch_scan_out<2>(N, H, w, states, num_slots, slots, flags, o, stream);
  return launch_scan<4, 2>(N, H, w, states, num_slots, slots, flags, o, stream);
}

size_t chunk_mfma_bwd_workspace_bytes(int H, int32_t T, int32_t N) {
  const size_t ci = nchunks_max(T, N) * (size_t)H;
  // carve(..., bwd = true): no Q*Gam or A_qk in the forward scans' layouts
  return header_bytes(N) + align256(ci * kWnBytes) + align256(ci * kKdBytes) +
         align256(ci * kUtBytes) + align256(ci * kGcBytes) + align256(ci * kScBytes) +
         align256(ci * kUcBytes) +
         3 * align256(ci * kKdBytes) + align256(ci * kAqBytes) + align256(ci * kMkBytes) +
         align256(ci * kTmBytes) + align256(ci * kScBytes) + align256(ci * kUcBytes) + 256;
}

kda_status_t launch_chunk_mfma_bwd(const kda_shape_t* sh, int32_t T, int32_t N, const int32_t* cu,
                                   const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* states, int32_t num_slots,
                                   const int32_t* slots, uint32_t flags, const void* d_o,
                                   const float* d_final, void* dq, void* dk, void* dv, float* dg,
                                   float* dbeta, float* d_initial, void* workspace,
                                   hipStream_t stream) {
  const int H = sh->num_heads;
  if (H > kMaxHeads) {
    set_error("kda_chunk_bwd: at most %d heads are supported (got %d)", kMaxHeads, H);
    return KDA_ERR_UNSUPPORTED;
  }
  Workspace w = carve(workspace, T, N, H, true);
  const size_t cap = nchunks_max(T, N);
  const size_t items = cap * (size_t)H;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int x = 0;
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && x > 0) ncu = x;
  }
  const PrepIndex ix{cu, T, (int32_t)cap, N <= kFuseMaxSeqs ? 1 : 0};
  kda_status_t st = KDA_OK;
  if (!ix.fused) {
    hipLaunchKernelGGL(index_kernel, dim3(1), dim3(64), 0, stream, cu, N, T, (int32_t)cap, w);
    st = check_launch("index_kernel");
    if (st != KDA_OK) return st;
  }
  // chunk operands of the forward pass plus the transposed ones of the reverse pass
  const unsigned grid = (unsigned)(items < (size_t)ncu ? items : (size_t)ncu);
  const bool add = flags & KDA_ADDITIVE;
  const int gate = (flags & KDA_GATE_SCALAR) ? kGateScalar : (flags & KDA_GATE_NONE) ? kGateNone
                                                                                    : kGateChannel;
#define KDA_BWD_PREP(G, A) launch_prep<G, A, false, true>(grid, q, k, v, g, beta, 0.f, N, H, w, ix, stream)
  st = gate == kGateScalar ? (add ? KDA_BWD_PREP(kGateScalar, true) : KDA_BWD_PREP(kGateScalar, false))
     : gate == kGateNone   ? (add ? KDA_BWD_PREP(kGateNone, true) : KDA_BWD_PREP(kGateNone, false))
                           : (add ? KDA_BWD_PREP(kGateChannel, true) : KDA_BWD_PREP(kGateChannel, false));
#undef KDA_BWD_PREP
  if (st != KDA_OK) return st;
  // forward state pass (S at every chunk start, U) and reverse pass (dL/dS at every chunk
  // end, dL/dU) in one launch
  constexpr int kGroups = D / 16;
  constexpr size_t kPairLds =
      sizeof(StateLds<1, 1>) > sizeof(GradScanLds) ? sizeof(StateLds<1, 1>) : sizeof(GradScanLds);
  static std::atomic<uint64_t> lds_pair{0};
  st = allow_dynamic_lds(reinterpret_cast<const void*>(scan_pair_kernel), kPairLds, lds_pair,
                         "hipFuncSetAttribute(scan pair)");
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL(scan_pair_kernel, dim3((unsigned)(2 * N * H * kGroups)),
                     dim3(kScanPairThreads), kPairLds, stream, N, H, w, const_cast<float*>(states),
                     num_slots, slots, flags & KDA_READ_INITIAL_STATE,
                     static_cast<const uint16_t*>(d_o), d_final, d_initial);
  st = check_launch("scan_pair_kernel");
  if (st != KDA_OK) return st;
  // gradients of every (chunk, head)
  auto launch_grad = [&](auto kern, std::atomic<uint64_t>& done) -> kda_status_t {
    kda_status_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), sizeof(GradSmem), done,
                                       "hipFuncSetAttribute(grad)");
    if (e != KDA_OK) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(kGradThreads), sizeof(GradSmem), stream, N,
                       H, GradWs{w.tm, w.mkk, w.sc, w.uc, w.dsc, w.duc}, w.seq_start, w.seq_end,
                       w.chunk_off, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), g, beta, static_cast<const uint16_t*>(d_o),
                       static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk),
                       static_cast<uint16_t*>(dv), dg, dbeta);
    return KDA_OK;
  };
  static std::atomic<uint64_t> lg[6] = {{0}, {0}, {0}, {0}, {0}, {0}};
  st = gate == kGateScalar ? (add ? launch_grad(grad_kernel<kGateScalar, true>, lg[0])
                                  : launch_grad(grad_kernel<kGateScalar, false>, lg[1]))
     : gate == kGateNone   ? (add ? launch_grad(grad_kernel<kGateNone, true>, lg[2])
                                  : launch_grad(grad_kernel<kGateNone, false>, lg[3]))
                           : (add ? launch_grad(grad_kernel<kGateChannel, true>, lg[4])
                                  : launch_grad(grad_kernel<kGateChannel, false>, lg[5]));
  if (st != KDA_OK) return st;
  return check_launch("grad_kernel");
}

}  // namespace kda
