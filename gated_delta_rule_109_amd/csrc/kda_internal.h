// Host-side interface between the C ABI (kda_api.hip) and the kernel launchers.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Tokens per prefill block: the chain takes one step per two 16-token chunks.
constexpr int kBlockTokens = 32;
// Most tokens one decode call processes per sequence.
constexpr int kMaxTokens = KDA_DECODE_MAX_TOKENS;

struct DecodeArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  float* state;
  void* o;
  int32_t N, H, D;
  int32_t T;                  // tokens per sequence (1 for a plain decode step)
  const int32_t* accept;      // device [N] tokens to commit, or NULL (= T)
  float scale, g_min;
  uint32_t fe_flags = 0;      // KDA_FE_* (0: inputs used as given)
  float fe_eps = 0.f;
  int32_t gate = KDA_GATE_CHANNEL;  // layout of g (kda_gate)
  bool bf16;
  hipStream_t stream;
};

struct PrefillArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  const int32_t* cu_seqlens;       // device
  const int32_t* cu_seqlens_host;  // host, validated
  int32_t num_seqs, H, D;
  int64_t total_tokens;
  int64_t total_blocks;       // sum_n ceil(L_n / kBlockTokens), from the host copy
  int64_t window_blocks;      // blocks per record window (total_blocks: one window)
  int64_t num_checkpoints;    // from the host copy: checkpoints past it are not written
  float scale, g_min;
  uint32_t fe_flags = 0;      // KDA_FE_* (0: inputs used as given)
  float fe_eps = 0.f;
  int32_t gate = KDA_GATE_CHANNEL;  // layout of g (kda_gate)
  int32_t segments = 0;       // kda_options.segments: 0 library's choice, 1 off, >= 2 forced
  const float* initial_state;
  float* final_state;
  int32_t ckpt_interval;
  float* checkpoints;
  void* o;
  void* workspace;
  bool bf16;
  hipStream_t stream;
};

// Workspace layout of the prefill (all offsets 256-byte aligned). The block
// records exist for one window of window_blocks blocks (of every head) at a
// time; a call whose records do not fit the workspace at once runs window by
// window, carrying the state of the sequence that crosses each window edge.
struct PrefillLayout {
  size_t seq_blk_off;     // int32 [N + 1]
  size_t seq_ck_off;      // int32 [N + 1]
  size_t blk_info;        // int2  [total_blocks] (first token, valid tokens)
  int64_t win_slots;      // most windows the tables hold (one per block)
  size_t win_base;        // int32 [win_slots + 1] first entry of each window in win_order
  int64_t order_cap;      // entries of win_order: N + win_slots
  size_t win_order;       // int32 [order_cap] each window's sequences, longest part first
  size_t segs;            // fp32 [N][KDA_MAX_SEGMENTS][H][3][D][D] segment states, or 0
  size_t carry;           // fp32 [2][H][D][D] window carry states, or 0 (one window)
  size_t records;         // per (block, head) operand records of one window
  size_t record_bytes;    // bytes of one record
  size_t total;
};

PrefillLayout prefill_layout(int32_t num_seqs, int64_t total_blocks, int32_t H, int32_t D,
                             int64_t window_blocks, bool windowed);

// Bytes of one block record (one 32-token block of one head).
size_t record_bytes(int D);

// Whether the workspace holds segment states for this shape.
inline bool segments_allowed(int32_t num_seqs, int32_t H, int32_t D) {
  return (int64_t)num_seqs * H * (D / 16) <= KDA_SEGMENT_SLICE_LIMIT;
}
// The library's choice of segments per sequence: the largest P >= 3 whose
// chain workgroups (pass 1: 2P - 3 units per head, pass 2: P - 1) fit one per
// compute unit, with at least two blocks per segment of the longest
// sequence; else 1.
int32_t auto_segments(int32_t num_seqs, int32_t H, int32_t D, int64_t max_blocks);

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);

// Device address of the static scratch (KDA_NOALLOC_SCRATCH_BYTES) on the
// current device, looked up on the first call per device and kept.
hipError_t noalloc_scratch(void** ptr);

}  // namespace kda
