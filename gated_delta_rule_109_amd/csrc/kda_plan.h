// Index arithmetic of the prefill plan: how sequences map to 32-token blocks,
// block records and checkpoint slots. The plan and chain kernels call these
// functions on the device; a host check calls the same functions on the CPU.
//
// The kernels read the device copy of cu_seqlens, while the launches (grids,
// workspace, checkpoint count) are sized from the host copy. Every quantity
// derived from the device copy is clamped to the host copy's totals
// (total_tokens rows, total_blocks records, num_checkpoints slots), so copies
// that differ give wrong results but never an access outside the buffers.
//
// The includer provides __host__ / __device__ (hip_runtime.h does).
#pragma once

#include <stdint.h>

namespace kda {
namespace plan {

constexpr int kBT = 32;   // tokens per block

// Rows [s0, s1) of sequence n, clamped into [0, total].
__host__ __device__ inline void clamp_seq(const int32_t* cu, int n, int64_t total, int& s0, int& s1) {
  int64_t a = cu[n], b = cu[n + 1];
  a = a < 0 ? 0 : (a > total ? total : a);
  b = b < a ? a : (b > total ? total : b);
  s0 = (int)a;
  s1 = (int)b;
}

// Blocks of a sequence of len tokens (the last one may be ragged).
__host__ __device__ inline int seq_blocks(int len) { return (len + kBT - 1) / kBT; }

// a + b saturated at cap (a, b, cap >= 0). Associative on nonnegative values,
// so a parallel scan with it equals the sequential saturated prefix sum.
__host__ __device__ inline int sat_add(int a, int b, int cap) {
  return (int64_t)a + b > cap ? cap : a + b;
}

// Last n in [0, N) with off[n] <= c (off non-decreasing, off[0] = 0 <= c):
// the sequence that owns block c, skipping empty sequences.
__host__ __device__ inline int owner_of(const int32_t* off, int N, int c) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// First row and valid rows of block j of a sequence with rows [s0, s1).
// A block past the sequence's rows (only when the two copies differ) reads one
// valid row: t0 + cnt <= total always holds for total > 0.
__host__ __device__ inline void block_rows(int s0, int s1, int j, int64_t total, int& t0, int& cnt) {
  int64_t t = (int64_t)s0 + (int64_t)kBT * j;
  t0 = (int)(t < total - 1 ? t : total - 1);
  const int r = s1 - t0;
  cnt = r < 1 ? 1 : (r > kBT ? kBT : r);
}

// Blocks [blk0, blk1) of segment seg of P of a sequence of seq_nblk blocks
// whose records start at record blk_off, kept inside total_blocks records.
__host__ __device__ inline void segment_blocks(int seq_nblk, int seg, int P, int blk_off,
                                               int total_blocks, int& blk0, int& blk1) {
  const int bps = (seq_nblk + P - 1) / P;
  int room = total_blocks - blk_off;
  room = room < 0 ? 0 : room;
  int b0 = seg * bps < seq_nblk ? seg * bps : seq_nblk;
  b0 = b0 < room ? b0 : room;
  int b1 = b0 + bps < seq_nblk ? b0 + bps : seq_nblk;
  b1 = b1 < room ? b1 : room;
  blk0 = b0;
  blk1 = b1;
}

}  // namespace plan
}  // namespace kda
