// kda_api.cpp -- the C ABI of libkda.so: host-side validation and dispatch.
//
// Every entry point validates its arguments before anything is enqueued; on
// any error it returns a status, records a message for kda_last_error() and
// writes nothing.  The library allocates no device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include "kda_common.h"

namespace kda {

// launchers defined next to their kernels
kda_status_t launch_state_init(float* states, size_t n_floats, hipStream_t stream);
kda_status_t launch_state_copy(bool to_pool, float* states, int32_t num_slots,
                               const int32_t* slots, int32_t n, float* dense,
                               size_t per_state_floats, hipStream_t stream);
kda_status_t launch_state_fill(float* dst, int32_t num_slots, const int32_t* slots, int32_t n,
                               const float* src, size_t per_state_floats, hipStream_t stream);
kda_status_t launch_state_affine(int32_t n, int H, int dk, int dv, const float* M,
                                 const float* S_in, const float* B, float* S_out,
                                 hipStream_t stream);
bool decode_supported(int dk, int dv);
kda_status_t launch_decode(const kda_shape_t* sh, int32_t batch, const void* q, const void* k,
                           const void* v, const void* g, const void* beta, bool raw,
                           float gate_min, float* states, int32_t num_slots, const int32_t* slots,
                           uint32_t flags, void* o, hipStream_t stream);
bool chunk_small_supported(int dk, int dv, int chunk);
kda_status_t launch_chunk_small(const kda_shape_t* sh, int32_t chunk, int32_t T, int32_t N,
                                const int32_t* cu, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, float* states,
                                int32_t num_slots, const int32_t* slots, uint32_t flags, void* o,
                                hipStream_t stream);
bool chunk_mfma_supported(int dk, int dv, int chunk, int io_dtype);
size_t chunk_mfma_workspace_bytes(int H, int32_t T, int32_t N);
kda_status_t launch_chunk_mfma(const kda_shape_t* sh, int32_t T, int32_t N, const int32_t* cu,
                               const void* q, const void* k, const void* v, const void* g,
                               const void* beta, bool raw, float gate_min, float* states,
                               int32_t num_slots, const int32_t* slots, uint32_t flags, void* o,
                               void* workspace, hipStream_t stream);

kda_status_t noalloc_scratch(void** out);

size_t chunk_mfma_bwd_workspace_bytes(int H, int32_t T, int32_t N);
kda_status_t launch_chunk_mfma_bwd(const kda_shape_t* sh, int32_t T, int32_t N, const int32_t* cu,
                                   const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* states, int32_t num_slots,
                                   const int32_t* slots, uint32_t flags, const void* d_o,
                                   const float* d_final, void* dq, void* dk, void* dv, float* dg,
                                   float* dbeta, float* d_initial, void* workspace,
                                   hipStream_t stream);

size_t chunk_mfma_bwd_raw_workspace_bytes(int H, int32_t T, int32_t N);
kda_status_t launch_chunk_mfma_bwd_raw(const kda_shape_t* sh, int32_t T, int32_t N,
                                       const int32_t* cu, const void* q_raw, const void* k_raw,
                                       const void* v, const void* gate_logits,
                                       const void* beta_logits, float gate_min,
                                       const float* states, int32_t num_slots,
                                       const int32_t* slots, uint32_t flags, const void* d_o,
                                       const float* d_final, void* dq_raw, void* dk_raw, void* dv,
                                       void* dgate_logits, void* dbeta_logits, float* d_initial,
                                       void* workspace, hipStream_t stream);

namespace {
thread_local char g_last_error[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

kda_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KDA_OK;
  set_error("%s: %s", what, hipGetErrorString(e));
  return KDA_ERR_HIP;
}

namespace {
// Per-launch timing between kda_launch_timer_begin and kda_launch_timer_end:
// event 0 is recorded by begin, event i + 1 after the i-th launch.
struct LaunchTimer {
  hipStream_t stream = nullptr;
  hipEvent_t ev[KDA_LAUNCH_TIMER_MAX + 1] = {};
  const char* name[KDA_LAUNCH_TIMER_MAX] = {};
  int created = 0;
  int n = 0;
  hipError_t err = hipSuccess;
};
thread_local LaunchTimer* t_timer = nullptr;

void timer_free(LaunchTimer* t) {
  for (int i = 0; i < t->created; ++i) (void)hipEventDestroy(t->ev[i]);
  delete t;
}
}  // namespace

kda_status_t allow_dynamic_lds(const void* fn, size_t bytes, std::atomic<uint64_t>& done,
                               const char* what) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, what);
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return KDA_OK;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return hip_status(e, what);
  if (bit) done.fetch_or(bit, std::memory_order_release);
  return KDA_OK;
}

kda_status_t check_launch(const char* what) {
  const kda_status_t st = hip_status(hipGetLastError(), what);
  LaunchTimer* t = t_timer;
  if (st == KDA_OK && t && t->n < KDA_LAUNCH_TIMER_MAX) {
    const hipError_t e = hipEventRecord(t->ev[t->n + 1], t->stream);
    if (e != hipSuccess && t->err == hipSuccess) t->err = e;
    t->name[t->n++] = what;
  }
  return st;
}

namespace {

kda_status_t invalid(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return KDA_ERR_INVALID_ARGUMENT;
}

kda_status_t unsupported(const char* what, const kda_shape_t* sh, int chunk) {
  set_error("%s: unsupported (dk=%d, dv=%d, chunk=%d, io_dtype=%d)", what, sh->dk, sh->dv, chunk,
            sh->io_dtype);
  return KDA_ERR_UNSUPPORTED;
}

kda_status_t check_shape(const kda_shape_t* sh, const char* what) {
  if (!sh) return invalid("%s: shape is NULL", what);
  if (sh->num_heads <= 0) return invalid("%s: num_heads must be >= 1 (got %d)", what, sh->num_heads);
  if (sh->dk <= 0 || sh->dv <= 0) return invalid("%s: dk and dv must be >= 1", what);
  if (sh->io_dtype != KDA_FP32 && sh->io_dtype != KDA_BF16)
    return invalid("%s: io_dtype must be KDA_FP32 or KDA_BF16 (got %d)", what, sh->io_dtype);
  return KDA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr uint32_t kStateFlags = KDA_READ_INITIAL_STATE | KDA_WRITE_FINAL_STATE;
constexpr uint32_t kVariantFlags = KDA_GATE_SCALAR | KDA_GATE_NONE | KDA_ADDITIVE;

// The variant bits: at most one gate bit.
kda_status_t check_variant(uint32_t flags, const char* what) {
  if ((flags & KDA_GATE_SCALAR) && (flags & KDA_GATE_NONE))
    return invalid("%s: KDA_GATE_SCALAR and KDA_GATE_NONE are exclusive", what);
  return KDA_OK;
}

// g and beta as the variant reads them: g not read with KDA_GATE_NONE, beta not
// read with KDA_ADDITIVE; a per-channel g is read as 16-byte vectors of fp32
// (8-byte vectors of bf16 logits when raw).
kda_status_t check_gate_beta(uint32_t flags, const void* g, const void* beta, bool raw,
                             const char* what) {
  if (!(flags & KDA_GATE_NONE)) {
    const int a = (flags & KDA_GATE_SCALAR) ? (raw ? 2 : 4) : (raw ? 8 : 16);
    if (!g) return invalid("%s: %s is NULL", what, raw ? "gate_logits" : "g");
    if (!aligned(g, a)) return invalid("%s: the gate must be %d-byte aligned", what, a);
  }
  if (!(flags & KDA_ADDITIVE)) {
    if (!beta) return invalid("%s: %s is NULL", what, raw ? "beta_logits" : "beta");
    if (!aligned(beta, raw ? 2 : 4)) return invalid("%s: beta is misaligned", what);
  }
  return KDA_OK;
}

bool chunk_supported(const kda_shape_t* sh, int chunk) {
  return chunk_mfma_supported(sh->dk, sh->dv, chunk, sh->io_dtype) ||
         chunk_small_supported(sh->dk, sh->dv, chunk);
}

}  // namespace
}  // namespace kda

using namespace kda;

extern "C" {

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error; }

int32_t kda_chunk_fwd_supported(int32_t dk, int32_t dv, int32_t chunk, int32_t io_dtype) {
  if (io_dtype != KDA_FP32 && io_dtype != KDA_BF16) return 0;
  return (chunk_mfma_supported(dk, dv, chunk, io_dtype) || chunk_small_supported(dk, dv, chunk))
             ? 1 : 0;
}

size_t kda_chunk_fwd_workspace_bytes(const kda_shape_t* sh, int32_t chunk, int32_t total_tokens,
                                     int32_t num_seqs) {
  if (!sh || sh->num_heads <= 0 || total_tokens < 0 || num_seqs < 0) return 0;
  if (chunk_mfma_supported(sh->dk, sh->dv, chunk, sh->io_dtype))
    return chunk_mfma_workspace_bytes(sh->num_heads, total_tokens, num_seqs);
  return 0;
}

namespace {

// noalloc: the scratch is the library's own device array (kda_chunk_fwd_noalloc),
// looked up only once every argument has been validated.
kda_status_t chunk_fwd_impl(const char* W, const kda_shape_t* sh, int32_t chunk,
                            int32_t total_tokens, int32_t num_seqs, const int32_t* cu_seqlens,
                            const void* q, const void* k, const void* v, const void* g,
                            const void* beta, bool raw, float gate_min, float* states,
                            int32_t num_slots, const int32_t* state_slots, uint32_t flags,
                            void* o, void* workspace, size_t workspace_bytes, void* stream,
                            bool noalloc = false) {
  kda_status_t st = check_shape(sh, W);
  if (st != KDA_OK) return st;
  if (total_tokens < 0 || num_seqs < 0)
    return invalid("%s: total_tokens and num_seqs must be >= 0", W);
  if (flags & ~(kStateFlags | kVariantFlags))
    return invalid("%s: unknown flag bits 0x%x", W, flags & ~(kStateFlags | kVariantFlags));
  st = check_variant(flags, W);
  if (st != KDA_OK) return st;
  if (chunk <= 0) return invalid("%s: chunk must be >= 1 (got %d)", W, chunk);
  if (raw && gate_min != gate_min) return invalid("%s: gate_min is NaN", W);
  if (raw ? !chunk_mfma_supported(sh->dk, sh->dv, chunk, sh->io_dtype) : !chunk_supported(sh, chunk))
    return unsupported(W, sh, chunk);
  if (num_seqs == 0) return KDA_OK;
  if (total_tokens == 0) {
    // Every sequence is empty and ends in the state it starts from (zero without
    // an initial state), so only a final-state write alone changes the pool.
    if ((flags & kStateFlags) != KDA_WRITE_FINAL_STATE) return KDA_OK;
    if (!states) return invalid("%s: states is NULL but flags request state I/O", W);
    if (num_slots <= 0) return invalid("%s: num_slots must be >= 1 with state I/O", W);
    if (!state_slots && num_slots < num_seqs)
      return invalid("%s: num_slots (%d) < num_seqs (%d) with implicit slots", W, num_slots,
                     num_seqs);
    return launch_state_fill(states, num_slots, state_slots, num_seqs, nullptr,
                             (size_t)sh->num_heads * sh->dk * sh->dv,
                             static_cast<hipStream_t>(stream));
  }
  if (!cu_seqlens) return invalid("%s: cu_seqlens is NULL", W);
  if (!q || !k || !v || !o) return invalid("%s: a tensor pointer is NULL", W);
  st = check_gate_beta(flags, g, beta, raw, W);
  if (st != KDA_OK) return st;
  if (flags & kStateFlags) {
    if (!states) return invalid("%s: states is NULL but flags request state I/O", W);
    if (num_slots <= 0) return invalid("%s: num_slots must be >= 1 with state I/O", W);
    if (!state_slots && num_slots < num_seqs)
      return invalid("%s: num_slots (%d) < num_seqs (%d) with implicit slots", W, num_slots,
                     num_seqs);
  }
  // the MFMA path reads q, k, v and writes o in 16-byte row pieces
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (states && !aligned(states, 16)))
    return invalid("%s: q, k, v, o and states must be 16-byte aligned", W);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (chunk_mfma_supported(sh->dk, sh->dv, chunk, sh->io_dtype)) {
    const size_t need = chunk_mfma_workspace_bytes(sh->num_heads, total_tokens, num_seqs);
    if (noalloc) {
      if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) {
        set_error("%s: the call needs %zu bytes of scratch, the library's array holds %zu "
                  "(KDA_NOALLOC_SCRATCH_BYTES): split it into smaller calls, or pass a "
                  "workspace to kda_chunk_fwd", W, need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
        return KDA_ERR_WORKSPACE_TOO_SMALL;
      }
      st = noalloc_scratch(&workspace);
      if (st != KDA_OK) return st;
      workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need) {
      set_error("%s: workspace of %zu bytes needed, %zu given", W, need, workspace_bytes);
      return KDA_ERR_WORKSPACE_TOO_SMALL;
    }
    if (!aligned(workspace, 256)) return invalid("%s: workspace must be 256-byte aligned", W);
    return launch_chunk_mfma(sh, total_tokens, num_seqs, cu_seqlens, q, k, v, g, beta, raw,
                             gate_min, states, num_slots, state_slots, flags, o, workspace, s);
  }
  return launch_chunk_small(sh, chunk, total_tokens, num_seqs, cu_seqlens, q, k, v,
                            static_cast<const float*>(g), static_cast<const float*>(beta),
                            (flags & kStateFlags) ? states : nullptr, num_slots, state_slots,
                            flags, o, s);
}

kda_status_t decode_impl(const char* W, const kda_shape_t* sh, int32_t batch, const void* q,
                         const void* k, const void* v, const void* g, const void* beta, bool raw,
                         float gate_min, float* states, int32_t num_slots,
                         const int32_t* state_slots, uint32_t flags, void* o, void* stream) {
  kda_status_t st = check_shape(sh, W);
  if (st != KDA_OK) return st;
  if (batch < 0) return invalid("%s: batch must be >= 0", W);
  if (flags & ~kVariantFlags)
    return invalid("%s: unknown flag bits 0x%x", W, flags & ~kVariantFlags);
  st = check_variant(flags, W);
  if (st != KDA_OK) return st;
  if (raw && gate_min != gate_min) return invalid("%s: gate_min is NaN", W);
  if (!decode_supported(sh->dk, sh->dv) || (raw && sh->io_dtype != KDA_BF16))
    return unsupported(W, sh, 0);
  if (batch == 0) return KDA_OK;
  if (!q || !k || !v || !o || !states) return invalid("%s: a tensor pointer is NULL", W);
  st = check_gate_beta(flags, g, beta, raw, W);
  if (st != KDA_OK) return st;
  if (num_slots <= 0) return invalid("%s: num_slots must be >= 1", W);
  if (!state_slots && num_slots < batch)
    return invalid("%s: num_slots (%d) < batch (%d) with implicit slots", W, num_slots, batch);
  if (!aligned(states, 16)) return invalid("%s: states must be 16-byte aligned", W);
  return launch_decode(sh, batch, q, k, v, g, beta, raw, gate_min, states, num_slots, state_slots,
                       flags, o, static_cast<hipStream_t>(stream));
}

}  // namespace

kda_status_t kda_chunk_fwd(const kda_shape_t* sh, int32_t chunk, int32_t total_tokens,
                           int32_t num_seqs, const int32_t* cu_seqlens, const void* q,
                           const void* k, const void* v, const float* g, const float* beta,
                           float* states, int32_t num_slots, const int32_t* state_slots,
                           uint32_t flags, void* o, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return chunk_fwd_impl("kda_chunk_fwd", sh, chunk, total_tokens, num_seqs, cu_seqlens, q, k, v,
                        g, beta, false, 0.f, states, num_slots, state_slots, flags, o, workspace,
                        workspace_bytes, stream);
}

kda_status_t kda_chunk_fwd_noalloc(const kda_shape_t* sh, int32_t chunk, int32_t total_tokens,
                                   int32_t num_seqs, const int32_t* cu_seqlens, const void* q,
                                   const void* k, const void* v, const float* g,
                                   const float* beta, float* states, int32_t num_slots,
                                   const int32_t* state_slots, uint32_t flags, void* o,
                                   void* stream) {
  return chunk_fwd_impl("kda_chunk_fwd_noalloc", sh, chunk, total_tokens, num_seqs, cu_seqlens,
                        q, k, v, g, beta, false, 0.f, states, num_slots, state_slots, flags, o,
                        nullptr, 0, stream, true);
}

kda_status_t kda_chunk_fwd_raw(const kda_shape_t* sh, int32_t chunk, int32_t total_tokens,
                               int32_t num_seqs, const int32_t* cu_seqlens, const void* q_raw,
                               const void* k_raw, const void* v, const void* gate_logits,
                               const void* beta_logits, float gate_min, float* states,
                               int32_t num_slots, const int32_t* state_slots, uint32_t flags,
                               void* o, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl("kda_chunk_fwd_raw", sh, chunk, total_tokens, num_seqs, cu_seqlens, q_raw,
                        k_raw, v, gate_logits, beta_logits, true, gate_min, states, num_slots,
                        state_slots, flags, o, workspace, workspace_bytes, stream);
}

kda_status_t kda_decode_step(const kda_shape_t* sh, int32_t batch, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, float* states,
                             int32_t num_slots, const int32_t* state_slots, void* o,
                             void* stream) {
  return kda_decode_step_ex(sh, batch, q, k, v, g, beta, states, num_slots, state_slots, 0u, o,
                            stream);
}

kda_status_t kda_decode_step_ex(const kda_shape_t* sh, int32_t batch, const void* q,
                                const void* k, const void* v, const float* g, const float* beta,
                                float* states, int32_t num_slots, const int32_t* state_slots,
                                uint32_t flags, void* o, void* stream) {
  return decode_impl("kda_decode_step", sh, batch, q, k, v, g, beta, false, 0.f, states,
                     num_slots, state_slots, flags, o, stream);
}

kda_status_t kda_decode_step_raw(const kda_shape_t* sh, int32_t batch, const void* q_raw,
                                 const void* k_raw, const void* v, const void* gate_logits,
                                 const void* beta_logits, float gate_min, float* states,
                                 int32_t num_slots, const int32_t* state_slots, uint32_t flags,
                                 void* o, void* stream) {
  return decode_impl("kda_decode_step_raw", sh, batch, q_raw, k_raw, v, gate_logits, beta_logits,
                     true, gate_min, states, num_slots, state_slots, flags, o, stream);
}

kda_status_t kda_state_init(const kda_shape_t* sh, float* states, int32_t num_slots,
                            void* stream) {
  const char* W = "kda_state_init";
  kda_status_t st = check_shape(sh, W);
  if (st != KDA_OK) return st;
  if (num_slots < 0) return invalid("%s: num_slots must be >= 0", W);
  if (num_slots == 0) return KDA_OK;
  if (!states) return invalid("%s: states is NULL", W);
  const size_t per = (size_t)sh->num_heads * sh->dk * sh->dv;
  if (per % 4 != 0 || !aligned(states, 16))
    return invalid("%s: H*dk*dv must be a multiple of 4 and states 16-byte aligned", W);
  return launch_state_init(states, per * (size_t)num_slots, static_cast<hipStream_t>(stream));
}

static kda_status_t state_copy(const char* W, bool to_pool, const kda_shape_t* sh, float* states,
                               int32_t num_slots, const int32_t* slots, int32_t n, float* dense,
                               void* stream) {
  kda_status_t st = check_shape(sh, W);
  if (st != KDA_OK) return st;
  if (n < 0 || num_slots < 0) return invalid("%s: n and num_slots must be >= 0", W);
  if (n == 0) return KDA_OK;
  if (!states || !dense) return invalid("%s: states or dense buffer is NULL", W);
  if (!slots && num_slots < n)
    return invalid("%s: num_slots (%d) < n (%d) with implicit slots", W, num_slots, n);
  const size_t per = (size_t)sh->num_heads * sh->dk * sh->dv;
  if (per % 4 != 0 || !aligned(states, 16) || !aligned(dense, 16))
    return invalid("%s: H*dk*dv must be a multiple of 4 and buffers 16-byte aligned", W);
  return launch_state_copy(to_pool, states, num_slots, slots, n, dense, per,
                           static_cast<hipStream_t>(stream));
}

kda_status_t kda_state_load(const kda_shape_t* sh, float* states, int32_t num_slots,
                            const int32_t* slots, int32_t n, const float* src, void* stream) {
  return state_copy("kda_state_load", true, sh, states, num_slots, slots, n,
                    const_cast<float*>(src), stream);
}

kda_status_t kda_state_store(const kda_shape_t* sh, const float* states, int32_t num_slots,
                             const int32_t* slots, int32_t n, float* dst, void* stream) {
  return state_copy("kda_state_store", false, sh, const_cast<float*>(states), num_slots, slots, n,
                    dst, stream);
}

kda_status_t kda_state_affine(const kda_shape_t* sh, int32_t n, const float* M,
                              const float* S_in, const float* B, float* S_out, void* stream) {
  const char* W = "kda_state_affine";
  kda_status_t st = check_shape(sh, W);
  if (st != KDA_OK) return st;
  if (n < 0) return invalid("%s: n must be >= 0", W);
  if (sh->dk > 256) return unsupported(W, sh, 0);
  if (n == 0) return KDA_OK;
  if (!M || !S_in || !B || !S_out) return invalid("%s: a tensor pointer is NULL", W);
  if (!aligned(M, 4) || !aligned(S_in, 4) || !aligned(B, 4) || !aligned(S_out, 4))
    return invalid("%s: tensors must be 4-byte aligned", W);
  const size_t per = (size_t)sh->num_heads * sh->dk * sh->dv * sizeof(float);
  const size_t perm = (size_t)sh->num_heads * sh->dk * sh->dk * sizeof(float);
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(S_out), o1 = o0 + (size_t)n * per;
  auto overlaps = [&](const void* p, size_t bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + (size_t)n * bytes;
    return a0 < o1 && o0 < a1;
  };
  if (overlaps(M, perm) || overlaps(S_in, per) || (B != S_out && overlaps(B, per)))
    return invalid("%s: S_out overlaps M or S_in (only S_out == B is allowed)", W);
  return launch_state_affine(n, sh->num_heads, sh->dk, sh->dv, M, S_in, B, S_out,
                             static_cast<hipStream_t>(stream));
}

size_t kda_chunk_bwd_workspace_bytes(const kda_shape_t* sh, int32_t chunk, int32_t total_tokens,
                                     int32_t num_seqs) {
  if (!sh || sh->num_heads <= 0 || total_tokens < 0 || num_seqs < 0) return 0;
  if (!chunk_mfma_supported(sh->dk, sh->dv, chunk, sh->io_dtype)) return 0;
  return chunk_mfma_bwd_workspace_bytes(sh->num_heads, total_tokens, num_seqs);
}

}  // extern "C"

namespace {

// Validation shared by kda_chunk_bwd and kda_chunk_bwd_raw (raw: bf16 logits for
// g and beta, bf16 gradients of them).
kda_status_t chunk_bwd_impl(const char* W, const kda_shape_t* sh, int32_t chunk,
                            int32_t total_tokens, int32_t num_seqs, const int32_t* cu_seqlens,
                            const void* q, const void* k, const void* v, const void* g,
                            const void* beta, bool raw, float gate_min, const float* states,
                            int32_t num_slots, const int32_t* state_slots, uint32_t flags,
                            const void* d_o, const float* d_final_state, void* dq, void* dk,
                            void* dv, void* dg, void* dbeta, float* d_initial_state,
                            void* workspace, size_t workspace_bytes, void* stream) {
  kda_status_t st = check_shape(sh, W);
  if (st != KDA_OK) return st;
  if (total_tokens < 0 || num_seqs < 0)
    return invalid("%s: total_tokens and num_seqs must be >= 0", W);
  const uint32_t allowed = KDA_READ_INITIAL_STATE | kVariantFlags;
  if (flags & ~allowed)
    return invalid("%s: flags other than KDA_READ_INITIAL_STATE and the variant bits (0x%x)", W,
                   flags & ~allowed);
  st = check_variant(flags, W);
  if (st != KDA_OK) return st;
  if (chunk <= 0) return invalid("%s: chunk must be >= 1 (got %d)", W, chunk);
  if (raw && gate_min != gate_min) return invalid("%s: gate_min is NaN", W);
  if (!chunk_mfma_supported(sh->dk, sh->dv, chunk, sh->io_dtype)) return unsupported(W, sh, chunk);
  if (num_seqs == 0) return KDA_OK;
  if (total_tokens == 0) {
    // Every sequence is empty and passes its state through unchanged, so
    // dL/dS0 = dL/dS_final (zero when no final-state gradient is given).
    if (!d_initial_state) return KDA_OK;
    if (!aligned(d_initial_state, 4) || (d_final_state && !aligned(d_final_state, 4)))
      return invalid("%s: the state gradients must be 4-byte aligned", W);
    return launch_state_fill(d_initial_state, num_seqs, nullptr, num_seqs, d_final_state,
                             (size_t)sh->num_heads * sh->dk * sh->dv,
                             static_cast<hipStream_t>(stream));
  }
  if (!cu_seqlens) return invalid("%s: cu_seqlens is NULL", W);
  if (!q || !k || !v || !d_o || !dq || !dk || !dv) return invalid("%s: a tensor pointer is NULL", W);
  st = check_gate_beta(flags, g, beta, raw, W);
  if (st != KDA_OK) return st;
  if (!(flags & KDA_GATE_NONE) && !dg) return invalid("%s: the gate gradient is NULL", W);
  if (!(flags & KDA_ADDITIVE) && !dbeta) return invalid("%s: the beta gradient is NULL", W);
  if (flags & KDA_READ_INITIAL_STATE) {
    if (!states) return invalid("%s: states is NULL but KDA_READ_INITIAL_STATE is set", W);
    if (num_slots <= 0) return invalid("%s: num_slots must be >= 1 with initial states", W);
    if (!state_slots && num_slots < num_seqs)
      return invalid("%s: num_slots (%d) < num_seqs (%d) with implicit slots", W, num_slots,
                     num_seqs);
  }
  const size_t ga = raw ? 2 : 4;  // element size of the gate and beta gradients
  // q, k, v and d_o are read, dq and dk written, in 16-byte row pieces
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_o, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 2) || (dg && !aligned(dg, raw ? 8 : 4)) ||
      (dbeta && !aligned(dbeta, ga)) || (states && !aligned(states, 16)) ||
      (d_final_state && !aligned(d_final_state, 4)) ||
      (d_initial_state && !aligned(d_initial_state, 4)))
    return invalid("%s: q, k, v, d_o, dq, dk, states must be 16-byte aligned, the rest "
                   "element-aligned", W);
  const size_t need = raw ? chunk_mfma_bwd_raw_workspace_bytes(sh->num_heads, total_tokens, num_seqs)
                          : chunk_mfma_bwd_workspace_bytes(sh->num_heads, total_tokens, num_seqs);
  if (!workspace || workspace_bytes < need) {
    set_error("%s: workspace of %zu bytes needed, %zu given", W, need, workspace_bytes);
    return KDA_ERR_WORKSPACE_TOO_SMALL;
  }
  if (!aligned(workspace, 256)) return invalid("%s: workspace must be 256-byte aligned", W);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (raw)
    return launch_chunk_mfma_bwd_raw(sh, total_tokens, num_seqs, cu_seqlens, q, k, v, g, beta,
                                     gate_min, states, num_slots, state_slots, flags, d_o,
                                     d_final_state, dq, dk, dv, dg, dbeta, d_initial_state,
                                     workspace, s);
  return launch_chunk_mfma_bwd(sh, total_tokens, num_seqs, cu_seqlens, q, k, v,
                               static_cast<const float*>(g), static_cast<const float*>(beta),
                               states, num_slots, state_slots, flags, d_o, d_final_state, dq, dk,
                               dv, static_cast<float*>(dg), static_cast<float*>(dbeta),
                               d_initial_state, workspace, s);
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_bwd(const kda_shape_t* sh, int32_t chunk, int32_t total_tokens,
                           int32_t num_seqs, const int32_t* cu_seqlens, const void* q,
                           const void* k, const void* v, const float* g, const float* beta,
                           const float* states, int32_t num_slots, const int32_t* state_slots,
                           uint32_t flags, const void* d_o, const float* d_final_state, void* dq,
                           void* dk, void* dv, float* dg, float* dbeta, float* d_initial_state,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl("kda_chunk_bwd", sh, chunk, total_tokens, num_seqs, cu_seqlens, q, k, v, g,
                        beta, false, 0.f, states, num_slots, state_slots, flags, d_o,
                        d_final_state, dq, dk, dv, dg, dbeta, d_initial_state, workspace,
                        workspace_bytes, stream);
}

size_t kda_chunk_bwd_raw_workspace_bytes(const kda_shape_t* sh, int32_t chunk,
                                         int32_t total_tokens, int32_t num_seqs) {
  if (!sh || sh->num_heads <= 0 || total_tokens < 0 || num_seqs < 0) return 0;
  if (!chunk_mfma_supported(sh->dk, sh->dv, chunk, sh->io_dtype)) return 0;
  return chunk_mfma_bwd_raw_workspace_bytes(sh->num_heads, total_tokens, num_seqs);
}

kda_status_t kda_chunk_bwd_raw(const kda_shape_t* sh, int32_t chunk, int32_t total_tokens,
                               int32_t num_seqs, const int32_t* cu_seqlens, const void* q_raw,
                               const void* k_raw, const void* v, const void* gate_logits,
                               const void* beta_logits, float gate_min, const float* states,
                               int32_t num_slots, const int32_t* state_slots, uint32_t flags,
                               const void* d_o, const float* d_final_state, void* dq_raw,
                               void* dk_raw, void* dv, void* dgate_logits, void* dbeta_logits,
                               float* d_initial_state, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return chunk_bwd_impl("kda_chunk_bwd_raw", sh, chunk, total_tokens, num_seqs, cu_seqlens, q_raw,
                        k_raw, v, gate_logits, beta_logits, true, gate_min, states, num_slots,
                        state_slots, flags, d_o, d_final_state, dq_raw, dk_raw, dv, dgate_logits,
                        dbeta_logits, d_initial_state, workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" {

kda_status_t kda_launch_timer_begin(void* stream) {
  using namespace kda;
  if (t_timer) return invalid("kda_launch_timer_begin: a timer is already active on this thread");
  LaunchTimer* t = new (std::nothrow) LaunchTimer;
  if (!t) return invalid("kda_launch_timer_begin: out of host memory");
  t->stream = static_cast<hipStream_t>(stream);
  for (int i = 0; i <= KDA_LAUNCH_TIMER_MAX; ++i) {
    const hipError_t e = hipEventCreate(&t->ev[i]);
    if (e != hipSuccess) {
      timer_free(t);
      return hip_status(e, "kda_launch_timer_begin: hipEventCreate");
    }
    t->created = i + 1;
  }
  const hipError_t e = hipEventRecord(t->ev[0], t->stream);
  if (e != hipSuccess) {
    timer_free(t);
    return hip_status(e, "kda_launch_timer_begin: hipEventRecord");
  }
  t_timer = t;
  return KDA_OK;
}

kda_status_t kda_launch_timer_end(float* ms, const char** names, int32_t capacity,
                                  int32_t* launches) {
  using namespace kda;
  LaunchTimer* t = t_timer;
  if (!t) return invalid("kda_launch_timer_end: no timer is active on this thread");
  t_timer = nullptr;
  kda_status_t st = KDA_OK;
  if (capacity < 0 || (capacity > 0 && (!ms || !names)))
    st = invalid("kda_launch_timer_end: capacity < 0, or ms / names NULL with capacity > 0");
  else if (t->err != hipSuccess)
    st = hip_status(t->err, "kda_launch_timer_end: hipEventRecord");
  if (st == KDA_OK) {
    hipError_t e = hipEventSynchronize(t->ev[t->n]);
    if (e != hipSuccess) st = hip_status(e, "kda_launch_timer_end: hipEventSynchronize");
    for (int i = 0; st == KDA_OK && i < t->n && i < capacity; ++i) {
      float x = 0.f;
      e = hipEventElapsedTime(&x, t->ev[i], t->ev[i + 1]);
      if (e != hipSuccess) st = hip_status(e, "kda_launch_timer_end: hipEventElapsedTime");
      ms[i] = x;
      names[i] = t->name[i];
    }
  }
  if (launches) *launches = t->n;
  timer_free(t);
  return st;
}

}  // extern "C"
