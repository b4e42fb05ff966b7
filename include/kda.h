/*
 * kda.h -- C ABI of libkda: Kimi Delta Attention (KDA) prefill and decode on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [K3-SA] "LLM - Semianalysis, Kimi K3 아키텍처" (charstring.tistory.com/2557)
 *   [K3-DD] "MoonshotAI/Kimi-K3 딥다이브" (fiv.co.kr/repos/kimi-k3-deep-dive.html)
 *
 * The operation (per sequence n and head h, token by token; [K3-SA] 배경 /
 * Background: delta rule on the L2 value-retrieval loss, Gated DeltaNet's
 * forget gate turned into a diagonal, i.e. one decay per key channel;
 * [K3-DD] 4-1 KDA, first bullet: the per-channel decay has a lower bound):
 *
 *     alpha_t = exp(clamp(g_t, g_min, 0))            per key channel
 *     S'      = Diag(alpha_t) S_{t-1}
 *     S_t     = S' + beta_t k_t (v_t - S'^T k_t)^T   = (I - b k k^T) S' + b k v^T
 *     o_t     = scale * S_t^T q_t                     (read out after the update)
 *
 * S is a Dk x Dv fp32 matrix (row = key channel, Dv contiguous). Prefill
 * evaluates this recurrence in chunks of 16 tokens with dense products inside
 * a chunk and a recurrence between chunks ([K3-SA] Methods 1) FlashKDA;
 * [K3-DD] 4-1 KDA, second bullet); decode runs one step directly ([K3-SA]
 * Methods 1) FlashKDA, first bullet). Both give the recurrence's result up to
 * floating-point rounding; the MFMA operands of prefill are bf16 (with a
 * two-term bf16 split where precision needs it), accumulation is fp32 and the
 * state is always fp32.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller, row-major
 *     and contiguous, 16-byte aligned. Only the *_host arrays are host memory.
 *   - Supported head sizes: Dk == Dv == D with D in {16, 128}; anything else
 *     returns KDA_ERR_UNSUPPORTED.
 *   - All work is enqueued on `stream` (NULL = the default stream) and the
 *     calls are asynchronous. The library allocates nothing and keeps no
 *     global state, with one exception: kda_prefill_chunked_noalloc's static
 *     per-device scratch (see there).
 *   - Arguments are validated before any device work; on an error status no
 *     work has been enqueued. A fault inside a kernel surfaces later, as
 *     KDA_ERR_HIP from a later call or as an error of the caller's sync.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* null required pointer, bad size, bad cu_seqlens */
  KDA_ERR_UNSUPPORTED = 2, /* head size or dtype this build does not handle  */
  KDA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  KDA_ERR_HIP = 4          /* a HIP runtime call failed (launch or earlier)  */
} kda_status;

/* Storage type of q, k, v and o. g, beta and every state are always fp32. */
typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

/* Chunk length of the prefill ([K3-DD] 4-1 KDA, second bullet: 16-token
 * tiles): every product of the chunked form works on 16-token tiles, and
 * checkpoint intervals are multiples of it. (The sequential chain advances
 * two chunks per step; that is internal and changes no result beyond
 * rounding.) */
#define KDA_CHUNK 16

/* Lowest decay floor (g_min) the prefill accepts: inside each 16-token chunk
 * the decayed keys span a factor up to exp(-16 g_min), which must stay inside
 * the fp32 / bf16 normal range with margin (exp(80) at -5; alpha >= 0.0067).
 * ln 0.5 (the configurations here) is far above it. Decode has no such
 * limit. */
#define KDA_PREFILL_MIN_G_FLOOR (-5.0f)

/* Options of the extended entry points (kda_prefill_chunked_ex,
 * kda_decode_tokens). A NULL pointer means all defaults: the KDA gate and no
 * front end.
 *
 * gate: layout of g, i.e. which member of the delta-rule family runs
 * ([K3-SA] Background: DeltaNet is the delta rule; Gated DeltaNet adds one
 * LSTM-style forget gate; KDA turns that gate into a diagonal, one decay per
 * key channel):
 *   KDA_GATE_CHANNEL  g [.., H, Dk]: one log-decay per key channel (KDA)
 *   KDA_GATE_HEAD     g [.., H]: one log-decay per token and head (Gated
 *                     DeltaNet); S' = alpha S. The floor applies as for KDA.
 *   KDA_GATE_NONE     no decay (DeltaNet); g is not read and may be NULL.
 * A scalar decay commutes with the erase step, so GDN is exactly KDA with
 * every channel given the same log-decay, and DeltaNet is KDA with g = 0.
 *
 * flags: the optional front end, the step just before the recurrence, fused
 * into the kernels that first read q, k, g and beta (no separate pass over
 * them). Each flag replaces one input convention:
 *   KDA_FE_L2NORM_QK   q and k are raw; each (token, head) row x is used as
 *                      x / sqrt(sum_i x_i^2 + norm_eps), computed in fp32
 *                      (the operator's inputs are unit-norm keys and queries;
 *                      [K3-SA] Background: the delta rule as a step on the L2
 *                      value-retrieval loss)
 *   KDA_FE_GATE_LOGITS g holds raw gate logits a; the log-decay is
 *                      g = -softplus(a) = -ln(1 + e^a), then floored at g_min
 *                      as always ([K3-DD] 4-1 KDA, first bullet: a lower
 *                      bound on each key channel's decay). Invalid with
 *                      KDA_GATE_NONE.
 *   KDA_FE_BETA_LOGITS beta holds raw logits b; the write strength is
 *                      sigmoid(b) = 1 / (1 + e^-b)
 */
#define KDA_FE_L2NORM_QK 1u
#define KDA_FE_GATE_LOGITS 2u
#define KDA_FE_BETA_LOGITS 4u
typedef enum { KDA_GATE_CHANNEL = 0, KDA_GATE_HEAD = 1, KDA_GATE_NONE = 2 } kda_gate;
/* segments (prefill only): a long sequence's recurrence split into segments
 * that run side by side ([K3-DD] 4-1 KDA names "KDA Context Parallelism"; the
 * split rests on the recurrence being linear in the state):
 *   pass 1: segment 0 runs in full; every middle segment p runs from a zero
 *           state (its local state) and, with zero values, from the identity
 *           (its transition M_p);
 *   scan:   S_in(p) = M_{p-1} S_in(p-1) + local(p-1);
 *   pass 2: segments 1 .. P-1 run in full from S_in(p).
 * Each segment holds whole 32-token blocks; a call in record windows (see
 * kda_prefill_workspace_size) splits each window's part of a sequence. It
 * pays when the chain would otherwise leave most compute units idle: few
 * sequences times heads. A
 * value of 0 lets the library choose (1 for most shapes); 1 turns it off;
 * 2 .. KDA_MAX_SEGMENTS forces that many segments per sequence. Forcing is
 * accepted only where the workspace holds the segment states:
 * num_seqs * H * (Dv / 16) <= KDA_SEGMENT_SLICE_LIMIT. */
#define KDA_MAX_SEGMENTS 16
#define KDA_SEGMENT_SLICE_LIMIT 80
typedef struct {
  uint32_t flags;   /* OR of KDA_FE_*; other bits are invalid */
  float norm_eps;   /* >= 0 and finite; used only with KDA_FE_L2NORM_QK */
  int32_t gate;     /* a kda_gate value */
  int32_t segments; /* 0 = library's choice, 1 = off, 2 .. KDA_MAX_SEGMENTS (prefill) */
} kda_options;

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status status);

/* Number of state checkpoints a prefill call writes:
 * sum_n floor(L_n / ckpt_interval), L_n = cu_seqlens_host[n+1] - cu_seqlens_host[n].
 * Returns 0 when ckpt_interval <= 0, -1 when the arguments are invalid. */
int64_t kda_prefill_num_checkpoints(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                    int32_t ckpt_interval);

/* Bytes of device workspace for kda_prefill_chunked on num_seqs sequences of
 * total_tokens packed tokens with H heads (0 if the arguments are invalid
 * or describe a call kda_prefill_chunked refuses: total_tokens * H or
 * num_seqs * H * (Dv / 16) above INT32_MAX). The workspace holds
 * per-sequence and per-block tables (16 bytes per 32-token block) and the
 * per-block decayed operands of the chunked form ("records": 47 KiB per
 * 32-token block and head at D = 128, about 1.5 KiB per token and head),
 * sized for the most blocks any split of total_tokens into num_seqs
 * sequences can have, total_tokens / 32 + num_seqs. The record space
 * is capped at KDA_PREFILL_RECORD_CAP_BYTES: a call with more records runs in
 * windows of consecutive blocks, preparing and consuming one window's records
 * at a time, so the workspace stops growing with T there (the tables still
 * grow by 16 bytes per block). Where segments may be used
 * (num_seqs * H * (Dv / 16) <= KDA_SEGMENT_SLICE_LIMIT) it also holds three
 * fp32 Dk x Dv states per sequence, head and segment; with windows, two fp32
 * Dk x Dv states per head carry the sequence that crosses a window edge. Its
 * contents are scratch and need no initialisation.
 * A single sequence (num_seqs == 1) runs in windows of about
 * KDA_PREFILL_SINGLE_SEQ_WINDOW_BYTES of records whatever the workspace
 * holds: each window still holds all of its heads, and part of its records is
 * still in the 256 MB memory-side cache when they are read. With several
 * sequences a window can hold only some of the (sequence, head) pairs, so
 * they run in one window up to the cap. */
#define KDA_PREFILL_RECORD_CAP_BYTES (8ull << 30)
#define KDA_PREFILL_SINGLE_SEQ_WINDOW_BYTES (1ull << 30)
size_t kda_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk,
                                  int32_t Dv);

/* Bytes of device workspace that runs the same prefill with records for at
 * most window_blocks blocks (of every head) at a time (0 if the arguments are
 * invalid or window_blocks < 1). A window of at least total_tokens / 32 +
 * num_seqs blocks is one window (no carry states). The prefill accepts any
 * workspace of at least this size for window_blocks = 1 and chooses its
 * windows from the bytes it is given: all records at once if they fit, else
 * windows of as many blocks as fit, evened out over the call. Results do not
 * depend on the windows (each block's arithmetic is the same), except that
 * the segment-parallel scan, when used, splits each window's part of a
 * sequence instead of the whole sequence. */
size_t kda_prefill_workspace_size_window(int32_t num_seqs, int64_t total_tokens, int32_t H,
                                         int32_t Dk, int32_t Dv, int64_t window_blocks);

/* Chunked prefill over packed variable-length sequences.
 *
 * Inputs (T = cu_seqlens_host[num_seqs] packed tokens):
 *   q, k        [T, H, Dk]  dtype      (q, k are used as given: no normalisation)
 *   v           [T, H, Dv]  dtype
 *   g           [T, H, Dk]  fp32 log-decay, clamped to [g_min, 0] on load
 *   beta        [T, H]      fp32
 *   cu_seqlens       [num_seqs + 1] int32, DEVICE copy of the offsets
 *   cu_seqlens_host  [num_seqs + 1] int32, HOST copy: cu[0] = 0,
 *                    non-decreasing. It is validated and sizes the launches
 *                    (grids, checkpoint count) without a device-to-host copy.
 *                    PRECONDITION: both copies hold the same values. The
 *                    kernels read the device copy (so a captured graph can
 *                    replay with new offsets of the same totals) and clamp
 *                    every offset they derive from it to the host copy's
 *                    total tokens and checkpoint count, so copies that differ
 *                    give wrong results but no access outside the buffers.
 *                    A sequence of length 0 is allowed (its final state equals
 *                    its initial state, it has no outputs).
 *   scale       readout scale (1.0 reproduces o_t = S_t^T q_t)
 *   g_min       decay floor in log space (ln 0.5 for the configurations here;
 *               [K3-DD] 4-1 KDA, first bullet); must lie in
 *               [KDA_PREFILL_MIN_G_FLOOR, 0]
 *   initial_state  [num_seqs, H, Dk, Dv] fp32, or NULL for zero states
 * Outputs:
 *   o              [T, H, Dv] dtype
 *   final_state    [num_seqs, H, Dk, Dv] fp32, or NULL to skip
 *   checkpoints    fp32 [kda_prefill_num_checkpoints(...), H, Dk, Dv], ordered
 *                  by (sequence, index within the sequence): checkpoint j >= 1 of
 *                  sequence n is the state after its first j * ckpt_interval
 *                  tokens, so any checkpoint is a valid initial_state for
 *                  resuming ([K3-SA] Methods 3) KV cache efficiency: the
 *                  recurrent state is kept only at sparse token intervals).
 *                  Ignored when ckpt_interval == 0.
 *   ckpt_interval  0 (no checkpoints) or a positive multiple of KDA_CHUNK.
 *   workspace      device scratch, 256-byte aligned, of workspace_bytes >=
 *                  kda_prefill_workspace_size_window(num_seqs, T, H, Dk, Dv, 1)
 *                  bytes; kda_prefill_workspace_size(num_seqs, T, H, Dk, Dv)
 *                  bytes run the call in the fewest windows up to the record
 *                  cap (one window below it).
 * initial_state may alias final_state (the state is read before it is written).
 * Errors: KDA_ERR_INVALID_ARG (null required pointer, negative sizes,
 * malformed cu_seqlens_host, bad ckpt_interval, g_min outside
 * [KDA_PREFILL_MIN_G_FLOOR, 0]), KDA_ERR_UNSUPPORTED,
 * KDA_ERR_WORKSPACE, KDA_ERR_HIP (launch failure). */
kda_status kda_prefill_chunked(const void* q, const void* k, const void* v, kda_dtype dtype,
                               const float* g, const float* beta, const int32_t* cu_seqlens,
                               const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                               int32_t Dk, int32_t Dv, float scale, float g_min,
                               const float* initial_state, float* final_state,
                               int32_t ckpt_interval, float* checkpoints, void* o,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kda_prefill_chunked with options `opt` (see kda_options): the gate layout
 * (KDA, Gated DeltaNet or DeltaNet) and the optional front end (q, k, g and
 * beta may be raw: unnormalised keys and queries, gate and write logits).
 * g is [T, H, Dk], [T, H] or unused (may be NULL) by opt->gate. Same
 * arguments, layouts, outputs and errors otherwise, plus KDA_ERR_INVALID_ARG
 * for unknown flag bits, an unknown gate, KDA_FE_GATE_LOGITS with
 * KDA_GATE_NONE, or a negative or non-finite norm_eps. opt = NULL is exactly
 * kda_prefill_chunked. */
kda_status kda_prefill_chunked_ex(const void* q, const void* k, const void* v, kda_dtype dtype,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                                  int32_t Dk, int32_t Dv, float scale, float g_min,
                                  const float* initial_state, float* final_state,
                                  int32_t ckpt_interval, float* checkpoints, void* o,
                                  void* workspace, size_t workspace_bytes,
                                  const kda_options* opt, hipStream_t stream);

/* kda_prefill_chunked_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, results and errors, without the workspace.
 * The workspace is a static device array of KDA_NOALLOC_SCRATCH_BYTES that
 * every GPU running this call holds from its first use until the process
 * ends; the call itself allocates nothing.
 *   - The call runs in record windows of as many blocks as the scratch holds
 *     (see kda_prefill_workspace_size_window), so any length fits; only calls
 *     whose tables and one block per head exceed it
 *     (kda_prefill_workspace_size_window(..., 1) > KDA_NOALLOC_SCRATCH_BYTES)
 *     return KDA_ERR_WORKSPACE, before any device work.
 *   - stream must belong to the current device (else KDA_ERR_INVALID_ARG).
 *   - Every call on one GPU uses the same scratch, and its contents are left
 *     from the last call (the prefill needs no initialised workspace). Calls
 *     that overlap on one GPU race: calls from several host threads or on
 *     several streams of one GPU must be ordered by the caller.
 * Errors: as kda_prefill_chunked_ex, plus KDA_ERR_HIP when the scratch's
 * device address cannot be looked up. */
#define KDA_NOALLOC_SCRATCH_BYTES (256u << 20)
kda_status kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v, kda_dtype dtype,
                                       const float* g, const float* beta, const int32_t* cu_seqlens,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                                       int32_t Dk, int32_t Dv, float scale, float g_min,
                                       const float* initial_state, float* final_state,
                                       int32_t ckpt_interval, float* checkpoints, void* o,
                                       const kda_options* opt, hipStream_t stream);

/* One recurrent decode step for N independent sequences ([K3-SA] Methods 1)
 * FlashKDA, first bullet: decode runs the state update directly; about 7 D^2
 * FLOPs and 8 D^2 bytes of fp32 state traffic per head-token).
 *   q, k   [N, H, Dk] dtype;  v [N, H, Dv] dtype
 *   g      [N, H, Dk] fp32 log-decay (clamped to [g_min, 0]);  beta [N, H] fp32
 *   state  [N, H, Dk, Dv] fp32, read and updated IN PLACE
 *   o      [N, H, Dv] dtype
 * g_min must lie in [-FLT_MAX, 0] (any finite floor; decode has no lower
 * limit, since it multiplies the state by alpha directly).
 * Errors: KDA_ERR_INVALID_ARG (null pointer, negative N, H <= 0, g_min
 * outside [-FLT_MAX, 0] or NaN), KDA_ERR_UNSUPPORTED, KDA_ERR_HIP. */
kda_status kda_decode_step(const void* q, const void* k, const void* v, kda_dtype dtype,
                           const float* g, const float* beta, float* state, void* o,
                           int32_t N, int32_t H, int32_t Dk, int32_t Dv, float scale,
                           float g_min, hipStream_t stream);

/* Most tokens per sequence that kda_decode_tokens takes in one call. */
#define KDA_DECODE_MAX_TOKENS 16

/* T consecutive recurrent steps per sequence in one call (1 <= T <=
 * KDA_DECODE_MAX_TOKENS): the draft tokens of a speculative-decoding step
 * ([K3-SA] Experiments, serving bullets: the day-0 serving recipes use DSpark
 * speculative decoding), or several decode tokens at once. Each step is the
 * recurrence of kda_decode_step; the fp32 state is read once and written at
 * most once per call, so the state traffic stays 8 D^2 bytes per head however
 * many tokens the call holds.
 *   q, k   [N, T, H, Dk] dtype (token t of sequence n is row n*T + t)
 *   v      [N, T, H, Dv] dtype
 *   g      [N, T, H, Dk] fp32 log-decay (clamped to [g_min, 0]); [N, T, H]
 *          with KDA_GATE_HEAD; unused (may be NULL) with KDA_GATE_NONE
 *   beta   [N, T, H] fp32
 *   state  [N, H, Dk, Dv] fp32, read, and updated IN PLACE to the state after
 *          the first accept[n] tokens of sequence n
 *   accept device int32 [N] or NULL (NULL commits all T tokens). Values are
 *          clamped to [0, T]; 0 leaves that sequence's state unchanged. A
 *          verify pass therefore runs with accept = 0, and once the accepted
 *          prefix length a_n is known a second call with accept = a_n on the
 *          same inputs commits exactly that prefix.
 *   o      [N, T, H, Dv] dtype, output of every token whatever accept holds
 *   opt    gate layout and front end (see kda_options), or NULL for the
 *          KDA gate with inputs used as given
 * Errors: KDA_ERR_INVALID_ARG (null required pointer, T outside
 * [1, KDA_DECODE_MAX_TOKENS], negative N, H <= 0, bad options, g_min as in
 * kda_decode_step),
 * KDA_ERR_UNSUPPORTED, KDA_ERR_HIP. */
kda_status kda_decode_tokens(const void* q, const void* k, const void* v, kda_dtype dtype,
                             const float* g, const float* beta, float* state,
                             const int32_t* accept, void* o, int32_t N, int32_t T, int32_t H,
                             int32_t Dk, int32_t Dv, float scale, float g_min,
                             const kda_options* opt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
