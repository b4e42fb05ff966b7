// C ABI of libkda (declared in include/kda.h): argument validation, workspace
// sizing and dispatch to the kernel launchers. No device work is enqueued
// unless every argument checks out.
#include "kda.h"
#include "kda_internal.h"
#include "kda_plan.h"

#include <float.h>
#include <limits.h>
#include <string.h>

#include <initializer_list>

namespace {

bool supported_dims(int32_t Dk, int32_t Dv) { return Dk == Dv && (Dk == 16 || Dk == 128); }

// An enum argument as the int a C caller passed. A C enum is an int, but in
// C++ a value outside the enumerators' range may not be read as the enum type,
// so the argument's bytes are read instead (by reference: no enum-typed load).
template <typename E>
int enum_code(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int c;
  memcpy(&c, &e, sizeof c);
  return c;
}

// Validates cu_seqlens_host; on success returns total tokens and prefill
// blocks (kda::kBlockTokens tokens each).
bool scan_lengths(const int32_t* cu, int32_t num_seqs, int64_t* tokens, int64_t* blocks) {
  if (!cu || num_seqs < 0 || cu[0] != 0) return false;
  int64_t c = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    if (cu[n + 1] < cu[n]) return false;
    c += (cu[n + 1] - cu[n] + kda::kBlockTokens - 1) / kda::kBlockTokens;
  }
  *tokens = cu[num_seqs];
  *blocks = c;
  return c <= INT32_MAX;
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Lowest decay floor the prefill accepts: a chunk's decayed keys span a
// factor of up to exp(-16 g_min) (k / P_r with P_r >= exp(16 g_min) inside
// each 16-token chunk), which must stay inside the fp32 / bf16 normal range
// (2^126) with margin.
constexpr float kMinGateFloor = KDA_PREFILL_MIN_G_FLOOR;
static_assert(KDA_CHUNK * -KDA_PREFILL_MIN_G_FLOOR * 1.4426950408889634f < 120.f,
              "decay span of a chunk");

// Options: NULL, or known flag bits, a known gate layout and a usable epsilon.
bool options_ok(const kda_options* opt) {
  if (!opt) return true;
  const uint32_t known = KDA_FE_L2NORM_QK | KDA_FE_GATE_LOGITS | KDA_FE_BETA_LOGITS;
  if (opt->flags & ~known) return false;
  if (opt->gate != KDA_GATE_CHANNEL && opt->gate != KDA_GATE_HEAD && opt->gate != KDA_GATE_NONE) return false;
  if (opt->gate == KDA_GATE_NONE && (opt->flags & KDA_FE_GATE_LOGITS)) return false;
  if (opt->segments < 0 || opt->segments > KDA_MAX_SEGMENTS) return false;
  return opt->norm_eps >= 0.f && opt->norm_eps <= FLT_MAX;
}
int32_t gate_of(const kda_options* opt) { return opt ? opt->gate : KDA_GATE_CHANNEL; }

// Decode multiplies the state by alpha = exp(clamp(g, g_min, 0)) directly, so
// any finite floor at or below 0 is usable.
bool decode_floor_ok(float g_min) { return g_min >= -FLT_MAX && g_min <= 0.f; }

kda_status prefill_impl(const void* q, const void* k, const void* v, int dtype, const float* g,
                        const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                        int32_t num_seqs, int32_t H, int32_t Dk, int32_t Dv, float scale, float g_min,
                        const float* initial_state, float* final_state, int32_t ckpt_interval,
                        float* checkpoints, void* o, void* workspace, size_t workspace_bytes,
                        bool use_scratch, const kda_options* opt, hipStream_t stream);

// Every tensor pointer must be 16-byte aligned (NULL passes).
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if ((uintptr_t)p & 15) return false;
  return true;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status status) {
  switch (enum_code(status)) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: unsupported head size or dtype";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime error";
  }
  return "KDA: unknown status";
}

int64_t kda_prefill_num_checkpoints(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                    int32_t ckpt_interval) {
  int64_t tokens, blocks;
  if (!scan_lengths(cu_seqlens_host, num_seqs, &tokens, &blocks)) return -1;
  if (ckpt_interval <= 0) return 0;
  int64_t total = 0;
  for (int32_t n = 0; n < num_seqs; ++n)
    total += (cu_seqlens_host[n + 1] - cu_seqlens_host[n]) / ckpt_interval;
  return total;
}

size_t kda_prefill_workspace_size_window(int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk,
                                         int32_t Dv, int64_t window_blocks) {
  if (num_seqs < 0 || total_tokens < 0 || H <= 0 || !supported_dims(Dk, Dv) || window_blocks <= 0) return 0;
  // shapes the prefill refuses (token-heads or 16-column slices past INT32_MAX)
  if (total_tokens > INT32_MAX || total_tokens * H > INT32_MAX || (int64_t)num_seqs * H * (Dv / 16) > INT32_MAX)
    return 0;
  // sum_n ceil(L_n / 32) <= sum_n (L_n / 32 + 1) for any lengths with this total
  const int64_t max_blocks = total_tokens / kda::kBlockTokens + num_seqs;
  if (max_blocks > INT32_MAX) return 0;
  const bool windowed = window_blocks < max_blocks;
  return kda::prefill_layout(num_seqs, max_blocks, H, Dk, windowed ? window_blocks : max_blocks, windowed).total;
}

size_t kda_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk,
                                  int32_t Dv) {
  if (H <= 0 || !supported_dims(Dk, Dv)) return 0;
  const size_t cap_bytes = num_seqs == 1 ? (size_t)KDA_PREFILL_SINGLE_SEQ_WINDOW_BYTES
                                         : (size_t)KDA_PREFILL_RECORD_CAP_BYTES;
  const int64_t cap = (int64_t)(cap_bytes / (kda::record_bytes(Dk) * (size_t)H));
  return kda_prefill_workspace_size_window(num_seqs, total_tokens, H, Dk, Dv, cap > 1 ? cap : 1);
}

kda_status kda_prefill_chunked(const void* q, const void* k, const void* v, kda_dtype dtype,
                               const float* g, const float* beta, const int32_t* cu_seqlens,
                               const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                               int32_t Dk, int32_t Dv, float scale, float g_min,
                               const float* initial_state, float* final_state,
                               int32_t ckpt_interval, float* checkpoints, void* o,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl(q, k, v, enum_code(dtype), g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, Dk, Dv,
                      scale, g_min, initial_state, final_state, ckpt_interval, checkpoints, o, workspace,
                      workspace_bytes, false, nullptr, stream);
}

}  // extern "C"

namespace {

// The prefill behind both workspace conventions: the caller's workspace, or
// (use_scratch) the library's static per-device scratch, looked up only after
// every argument and the size have been checked.
kda_status prefill_impl(const void* q, const void* k, const void* v, int dtype, const float* g,
                        const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                        int32_t num_seqs, int32_t H, int32_t Dk, int32_t Dv, float scale, float g_min,
                        const float* initial_state, float* final_state, int32_t ckpt_interval,
                        float* checkpoints, void* o, void* workspace, size_t workspace_bytes,
                        bool use_scratch, const kda_options* opt, hipStream_t stream) {
  if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_UNSUPPORTED;
  if (!options_ok(opt)) return KDA_ERR_INVALID_ARG;
  const bool need_g = gate_of(opt) != KDA_GATE_NONE;
  if (!supported_dims(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
  int64_t tokens, blocks;
  if (H <= 0 || num_seqs < 0 || !cu_seqlens || !scan_lengths(cu_seqlens_host, num_seqs, &tokens, &blocks))
    return KDA_ERR_INVALID_ARG;
  if (!(g_min >= kMinGateFloor && g_min <= 0.f)) return KDA_ERR_INVALID_ARG;
  if ((int64_t)num_seqs * H * (Dv / 16) > INT32_MAX || tokens * (int64_t)H > INT32_MAX)
    return KDA_ERR_INVALID_ARG;
  if (tokens > 0 && (!q || !k || !v || (need_g && !g) || !beta || !o)) return KDA_ERR_INVALID_ARG;
  if (ckpt_interval < 0 || (ckpt_interval > 0 && ckpt_interval % KDA_CHUNK != 0))
    return KDA_ERR_INVALID_ARG;
  const int64_t nck = kda_prefill_num_checkpoints(cu_seqlens_host, num_seqs, ckpt_interval);
  if (nck > 0 && !checkpoints) return KDA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, g, beta, cu_seqlens, initial_state, final_state, checkpoints, o}))
    return KDA_ERR_INVALID_ARG;
  if (num_seqs == 0) return KDA_OK;
  // segments per sequence: the library's choice (0), off (1), or forced
  // (where the workspace holds the segment states)
  const int32_t req = opt ? opt->segments : 0;
  if (req >= 2 && !kda::segments_allowed(num_seqs, H, Dk)) return KDA_ERR_INVALID_ARG;
  // Record windows: all of the call's records at once if the workspace holds
  // them, else windows of as many blocks as it holds, evened out.
  // A window also keeps the prep grid's second dimension (its blocks) within
  // kMaxWindowBlocks.
  constexpr int64_t kMaxWindowBlocks = 65535;
  // A single sequence runs in windows of about
  // KDA_PREFILL_SINGLE_SEQ_WINDOW_BYTES of records even when the workspace
  // holds more: every window then still holds all of its (sequence, head)
  // pairs, and part of each window's records is still in the memory-side
  // cache when the chain reads them.
  const size_t rec_bytes = kda::record_bytes(Dk) * (size_t)H;
  int64_t max_window = kMaxWindowBlocks;
  if (num_seqs == 1) {
    const int64_t w1 = (int64_t)((size_t)KDA_PREFILL_SINGLE_SEQ_WINDOW_BYTES / rec_bytes);
    max_window = w1 < 1 ? 1 : (w1 < max_window ? w1 : max_window);
  }
  if (use_scratch) workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
  // (every sequence empty: no records, the tables only)
  int64_t window = 1;
  if (blocks == 0) {
    if (workspace_bytes < kda::prefill_layout(num_seqs, 0, H, Dk, 0, false).total) return KDA_ERR_WORKSPACE;
  } else {
    window = kda::plan::choose_window(blocks, workspace_bytes,
                                      kda::prefill_layout(num_seqs, blocks, H, Dk, blocks, false).total,
                                      kda::prefill_layout(num_seqs, blocks, H, Dk, 0, true).total, rec_bytes,
                                      max_window);
    if (window < 1) return KDA_ERR_WORKSPACE;
  }
  if (use_scratch) {
    // the scratch of the device the work runs on: the stream's, which must be
    // the current one (the array's address is looked up with it current)
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &dev) != hipSuccess) return KDA_ERR_HIP;
    if (dev != cur) return KDA_ERR_INVALID_ARG;
    if (kda::noalloc_scratch(&workspace) != hipSuccess) return KDA_ERR_HIP;
  }
  if (!workspace || ((uintptr_t)workspace & 255)) return KDA_ERR_WORKSPACE;

  kda::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.cu_seqlens = cu_seqlens; a.cu_seqlens_host = cu_seqlens_host;
  a.num_seqs = num_seqs; a.H = H; a.D = Dk;
  a.total_tokens = tokens; a.total_blocks = blocks; a.window_blocks = window;
  a.num_checkpoints = nck > 0 ? nck : 0;
  a.scale = scale; a.g_min = g_min;
  a.fe_flags = opt ? opt->flags : 0u; a.fe_eps = opt ? opt->norm_eps : 0.f;
  a.gate = gate_of(opt);
  a.segments = req;
  a.initial_state = initial_state; a.final_state = final_state;
  a.ckpt_interval = nck > 0 ? ckpt_interval : 0;
  a.checkpoints = checkpoints;
  a.o = o; a.workspace = workspace;
  a.bf16 = dtype == KDA_BF16;
  a.stream = stream;
  return from_hip(kda::launch_prefill(a));
}

}  // namespace

extern "C" {

kda_status kda_prefill_chunked_ex(const void* q, const void* k, const void* v, kda_dtype dtype,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                                  int32_t Dk, int32_t Dv, float scale, float g_min,
                                  const float* initial_state, float* final_state,
                                  int32_t ckpt_interval, float* checkpoints, void* o,
                                  void* workspace, size_t workspace_bytes,
                                  const kda_options* opt, hipStream_t stream) {
  return prefill_impl(q, k, v, enum_code(dtype), g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, Dk, Dv, scale,
                      g_min, initial_state, final_state, ckpt_interval, checkpoints, o, workspace,
                      workspace_bytes, false, opt, stream);
}

kda_status kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v, kda_dtype dtype,
                                       const float* g, const float* beta, const int32_t* cu_seqlens,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                                       int32_t Dk, int32_t Dv, float scale, float g_min,
                                       const float* initial_state, float* final_state,
                                       int32_t ckpt_interval, float* checkpoints, void* o,
                                       const kda_options* opt, hipStream_t stream) {
  return prefill_impl(q, k, v, enum_code(dtype), g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, Dk, Dv, scale,
                      g_min, initial_state, final_state, ckpt_interval, checkpoints, o, nullptr, 0, true,
                      opt, stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, kda_dtype dtype,
                           const float* g, const float* beta, float* state, void* o, int32_t N,
                           int32_t H, int32_t Dk, int32_t Dv, float scale, float g_min,
                           hipStream_t stream) {
  const int dt = enum_code(dtype);
  if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_UNSUPPORTED;
  if (!supported_dims(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
  if (N < 0 || H <= 0 || (int64_t)N * H > INT32_MAX) return KDA_ERR_INVALID_ARG;
  if (!decode_floor_ok(g_min)) return KDA_ERR_INVALID_ARG;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, g, beta, state, o})) return KDA_ERR_INVALID_ARG;
  kda::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
  a.N = N; a.H = H; a.D = Dk;
  a.T = 1; a.accept = nullptr;
  a.scale = scale; a.g_min = g_min;
  a.bf16 = dt == KDA_BF16;
  a.stream = stream;
  return from_hip(kda::launch_decode(a));
}

kda_status kda_decode_tokens(const void* q, const void* k, const void* v, kda_dtype dtype,
                             const float* g, const float* beta, float* state,
                             const int32_t* accept, void* o, int32_t N, int32_t T, int32_t H,
                             int32_t Dk, int32_t Dv, float scale, float g_min,
                             const kda_options* opt, hipStream_t stream) {
  const int dt = enum_code(dtype);
  if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_UNSUPPORTED;
  if (!options_ok(opt)) return KDA_ERR_INVALID_ARG;
  const bool need_g = gate_of(opt) != KDA_GATE_NONE;
  if (!supported_dims(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
  if (T < 1 || T > KDA_DECODE_MAX_TOKENS) return KDA_ERR_INVALID_ARG;
  if (!decode_floor_ok(g_min)) return KDA_ERR_INVALID_ARG;
  if (N < 0 || H <= 0 || (int64_t)N * H > INT32_MAX || (int64_t)N * T * H > INT32_MAX)
    return KDA_ERR_INVALID_ARG;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || (need_g && !g) || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, g, beta, state, o})) return KDA_ERR_INVALID_ARG;
  kda::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
  a.N = N; a.H = H; a.D = Dk;
  a.T = T; a.accept = accept;
  a.scale = scale; a.g_min = g_min;
  a.fe_flags = opt ? opt->flags : 0u; a.fe_eps = opt ? opt->norm_eps : 0.f;
  a.gate = gate_of(opt);
  a.bf16 = dt == KDA_BF16;
  a.stream = stream;
  return from_hip(kda::launch_decode(a));
}

}  // extern "C"
