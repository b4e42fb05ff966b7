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

// ---- record windows -----------------------------------------------------------
// The records of blocks [c0, c1) = [w W, min((w + 1) W, total_blocks)) of the
// global block list exist during window w of nwin = ceil(total_blocks / W)
// only. A sequence with records [g0, g1) (g0 = off[n], g1 = off[n + 1]) takes
// part in windows [win_lo, win_hi]; an empty one (g0 = g1) only in the window
// holding position g0 (the last window if g0 = total_blocks). Both ends are
// non-decreasing in n and win_hi(n) <= win_lo(n + 1), so the sequences of a
// window are a contiguous range and all windows together list at most
// N + nwin - 1 (sequence, window) pairs.
__host__ __device__ inline void window_range(int w, int W, int total_blocks, int& c0, int& c1) {
  const int64_t a = (int64_t)w * W, b = a + W;
  c0 = (int)(a < total_blocks ? a : total_blocks);
  c1 = (int)(b < total_blocks ? b : total_blocks);
}
__host__ __device__ inline int win_lo_at(int64_t g0, int W, int nwin) {
  const int64_t w = g0 / W;
  return (int)(w < nwin - 1 ? w : nwin - 1);
}
__host__ __device__ inline int win_hi_at(int64_t g0, int64_t g1, int W, int nwin) {
  if (g1 <= g0) return win_lo_at(g0, W, nwin);
  const int64_t w = (g1 - 1) / W;
  return (int)(w < nwin - 1 ? w : nwin - 1);
}
__host__ __device__ inline int win_lo(const int32_t* off, int n, int W, int nwin) {
  return win_lo_at(off[n], W, nwin);
}
__host__ __device__ inline int win_hi(const int32_t* off, int n, int W, int nwin) {
  return win_hi_at(off[n], off[n + 1], W, nwin);
}

// First sequence of window w and the number of sequences in it.
__host__ __device__ inline void window_seqs(const int32_t* off, int N, int W, int nwin, int w, int& first,
                                            int& count) {
  int lo = 0, hi = N;   // first n with win_hi(n) >= w
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (win_hi(off, mid, W, nwin) >= w) hi = mid; else lo = mid + 1;
  }
  first = lo;
  lo = 0, hi = N;       // first n with win_lo(n) > w
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (win_lo(off, mid, W, nwin) > w) hi = mid; else lo = mid + 1;
  }
  count = lo > first ? lo - first : 0;
}

// Blocks [p0, p1) of a sequence with records [g0, g1) that lie in the window's
// records [c0, c1), as indices within the sequence (p0 = p1 if none).
__host__ __device__ inline void window_part(int g0, int g1, int c0, int c1, int& p0, int& p1) {
  const int a = g0 > c0 ? g0 : c0, b = g1 < c1 ? g1 : c1;
  p0 = a < b ? a - g0 : 0;
  p1 = a < b ? b - g0 : 0;
}

// Blocks [b0, b1) of segment seg of P of np blocks.
__host__ __device__ inline void part_segment(int np, int seg, int P, int& b0, int& b1) {
  const int bps = (np + P - 1) / P;
  b0 = seg * bps < np ? seg * bps : np;
  b1 = b0 + bps < np ? b0 + bps : np;
}

// Blocks per record window for a call of blocks >= 1 blocks: all of them if
// they fit the workspace at once (one_window_bytes: tables and every record)
// and blocks <= max_window; else as many as fit beside fixed_bytes (tables
// and carry states) at block_bytes each (a block of every head), at most
// max_window, evened out over the windows. 0 if not one block fits.
inline int64_t choose_window(int64_t blocks, uint64_t workspace_bytes, uint64_t one_window_bytes,
                             uint64_t fixed_bytes, uint64_t block_bytes, int64_t max_window) {
  if (blocks <= max_window && workspace_bytes >= one_window_bytes) return blocks;
  if (workspace_bytes < fixed_bytes || block_bytes == 0) return 0;
  int64_t w = (int64_t)((workspace_bytes - fixed_bytes) / block_bytes);
  if (w < 1) return 0;
  w = w < max_window ? w : max_window;
  const int64_t nwin = (blocks + w - 1) / w;
  return (blocks + nwin - 1) / nwin;
}

// Host walk over the windows in order, from the host copy of cu_seqlens
// (exact per-sequence block counts, so the offsets need no table): calls
// visit(w, c0, c1, first, count, longest) for every window, with the window's
// first sequence, its number of sequences and its longest part in blocks.
// The sequences it counts per window are those window_seqs finds for offsets
// computed from the same copy.
template <typename Visit>
inline void walk_windows(const int32_t* cu_host, int N, int total_blocks, int W, int nwin, Visit visit) {
  auto nb = [&](int n) { return (int64_t)seq_blocks(cu_host[n + 1] - cu_host[n]); };
  int nf = 0;            // first sequence whose last window is not before w
  int64_t off_nf = 0;    // its first record
  for (int w = 0; w < nwin; ++w) {
    int c0, c1;
    window_range(w, W, total_blocks, c0, c1);
    while (nf < N && win_hi_at(off_nf, off_nf + nb(nf), W, nwin) < w) off_nf += nb(nf++);
    int count = 0;
    int64_t longest = 0, off = off_nf;
    for (int n = nf; n < N && win_lo_at(off, W, nwin) <= w; ++n) {
      const int64_t g1 = off + nb(n);
      const int64_t part = (g1 < c1 ? g1 : c1) - (off > c0 ? off : c0);
      longest = part > longest ? part : longest;
      ++count;
      off = g1;
    }
    visit(w, c0, c1, nf, count, (int)longest);
  }
}

}  // namespace plan
}  // namespace kda
