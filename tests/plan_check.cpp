// Host check of the prefill plan's index arithmetic (csrc/kda_plan.h), run by
// tests/test_plan.py on the CPU. It evaluates what the plan and chain kernels
// compute from a device cu_seqlens copy, for seeded host / device pairs and
// record windows of one block, a few blocks and the whole call, and checks
// that
//   - with equal copies the tables are the exact per-sequence blocks, rows
//     and checkpoint offsets; the windows' parts cover every sequence once,
//     each sequence starts and ends in exactly one window, the state one
//     window carries out is the one the next carries in, and the host's
//     window walk (which sizes the grids) agrees with the plan's tables;
//   - with copies that differ (shifted, shuffled, negative, past the total,
//     decreasing) every record, row, checkpoint slot and order-table entry
//     touched stays inside what the host copy sized, and at most one
//     sequence crosses each window edge;
// and that the window a call takes from its workspace (choose_window) fits
// it, respects the largest window, is evened out, and is refused only when
// not one block fits.
// The plan kernel's scan is a parallel prefix sum with plan::sat_add, which is
// associative on nonnegative values, so the sequential prefix here is what it
// computes.
#define __host__
#define __device__
#include "../gated_delta_rule_109_amd/csrc/kda_plan.h"

#include <algorithm>
#include <stdio.h>
#include <stdlib.h>
#include <vector>

using namespace kda::plan;

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {   // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static int rint_in(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }

static int failures = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      if (failures < 20) {                                 \
        fprintf(stderr, "FAIL %s: ", #cond);               \
        fprintf(stderr, __VA_ARGS__);                      \
        fprintf(stderr, "\n");                             \
      }                                                    \
      ++failures;                                          \
    }                                                      \
  } while (0)

// One case: returns the number of checks made.
static long run_case(const std::vector<int32_t>& host, const std::vector<int32_t>& dev, int interval,
                     bool same) {
  const int N = (int)host.size() - 1;
  const int64_t T = host[N];
  int total_blocks = 0, nck = 0;
  for (int n = 0; n < N; ++n) {
    total_blocks += seq_blocks(host[n + 1] - host[n]);
    nck += interval > 0 ? (host[n + 1] - host[n]) / interval : 0;
  }
  long checks = 0;
  // plan: saturated exclusive prefix sums of the clamped lengths
  std::vector<int32_t> blk_off(N + 1), ck_off(N + 1);
  int cb = 0, ck = 0;
  for (int n = 0; n < N; ++n) {
    int s0, s1;
    clamp_seq(dev.data(), n, T, s0, s1);
    CHECK(0 <= s0 && s0 <= s1 && s1 <= T, "seq %d rows [%d, %d) of %lld", n, s0, s1, (long long)T);
    blk_off[n] = cb;
    ck_off[n] = ck;
    cb = sat_add(cb, seq_blocks(s1 - s0), total_blocks);
    ck = sat_add(ck, interval > 0 ? (s1 - s0) / interval : 0, nck);
    ++checks;
  }
  blk_off[N] = cb;
  ck_off[N] = ck;
  for (int n = 0; n < N; ++n) {
    CHECK(0 <= blk_off[n] && blk_off[n] <= blk_off[n + 1] && blk_off[n + 1] <= total_blocks,
          "block offsets of seq %d", n);
    CHECK(0 <= ck_off[n] && ck_off[n] <= ck_off[n + 1] && ck_off[n + 1] <= nck, "checkpoint offsets of seq %d", n);
    if (same) {
      int eb = 0, ec = 0;
      for (int m = 0; m < n; ++m) {
        eb += seq_blocks(host[m + 1] - host[m]);
        ec += interval > 0 ? (host[m + 1] - host[m]) / interval : 0;
      }
      CHECK(blk_off[n] == eb && ck_off[n] == ec, "exact offsets of seq %d", n);
    }
    checks += 2;
  }
  // blk_info of every record (the prep kernel reads rows [t0, t0 + cnt))
  for (int c = 0; c < total_blocks; ++c) {
    const int n = owner_of(blk_off.data(), N, c);
    CHECK(0 <= n && n < N && blk_off[n] <= c, "owner of block %d", c);
    int s0, s1, t0, cnt;
    clamp_seq(dev.data(), n, T, s0, s1);
    block_rows(s0, s1, c - blk_off[n], T, t0, cnt);
    CHECK(0 <= t0 && 1 <= cnt && cnt <= kBT && t0 + cnt <= T, "rows of block %d: %d + %d of %lld", c, t0, cnt,
          (long long)T);
    if (same) {
      // block c is block j of sequence n: rows s0 + 32 j .. min(s1, s0 + 32 j + 32)
      const int j = c - blk_off[n];
      CHECK(j < seq_blocks(s1 - s0) && t0 == s0 + kBT * j && cnt == (s1 - t0 < kBT ? s1 - t0 : kBT),
            "exact rows of block %d", c);
    }
    checks += 2;
  }
  // Record windows of W blocks: the plan's per-window tables and the chain's
  // units, for a single window (W >= total_blocks) and for several.
  const int Ws[3] = {total_blocks > 0 ? total_blocks : 1, rint_in(1, 4), rint_in(1, 40)};
  for (int W : Ws) {
    const int nwin = total_blocks > 0 ? (total_blocks + W - 1) / W : 1;
    const int order_cap = N + (total_blocks > 1 ? total_blocks : 1);
    // plan: sequences per window, saturated prefix sums, longest-first order
    std::vector<int32_t> win_base(nwin + 1), order(order_cap, -1);
    int acc = 0;
    for (int w = 0; w < nwin; ++w) {
      int first, count;
      window_seqs(blk_off.data(), N, W, nwin, w, first, count);
      CHECK(0 <= first && first + count <= N, "window %d sequences [%d, +%d)", w, first, count);
      win_base[w] = acc;
      acc = sat_add(acc, count, order_cap);
      ++checks;
    }
    win_base[nwin] = acc;
    CHECK(acc <= N + nwin - 1, "window pairs %d > N + nwin - 1 = %d", acc, N + nwin - 1);
    for (int e = 0; e < acc; ++e) {
      const int w = owner_of(win_base.data(), nwin, e);
      int first, count, c0, c1;
      window_seqs(blk_off.data(), N, W, nwin, w, first, count);
      window_range(w, W, total_blocks, c0, c1);
      const int i = e - win_base[w];
      CHECK(0 <= i && i < count, "entry %d of window %d", i, w);
      const int n = first + i;
      int p0, p1;
      window_part(blk_off[n], blk_off[n + 1], c0, c1, p0, p1);
      int rank = 0;
      for (int m = first; m < first + count; ++m) {
        int q0, q1;
        window_part(blk_off[m], blk_off[m + 1], c0, c1, q0, q1);
        rank += q1 - q0 > p1 - p0 || (q1 - q0 == p1 - p0 && m < n);
      }
      CHECK(win_base[w] + rank < order_cap && order[win_base[w] + rank] == -1, "order slot of window %d", w);
      order[win_base[w] + rank] = n;
      checks += 2;
    }
    // host walk (launch grids) against the plan's windows
    walk_windows(host.data(), N, total_blocks, W, nwin, [&](int w, int c0, int c1, int first, int count, int longest) {
      int f2, n2, a0, a1;
      window_range(w, W, total_blocks, a0, a1);
      CHECK(a0 == c0 && a1 == c1, "window %d range", w);
      // the window's records fit the W blocks per head the workspace holds,
      // and the windows tile the block list
      CHECK(0 <= c0 && c0 <= c1 && c1 <= total_blocks && c1 - c0 <= W && c0 == w * W, "window %d: [%d, %d)", w,
            c0, c1);
      CHECK(w + 1 < nwin || c1 == total_blocks, "last window ends at %d of %d", c1, total_blocks);
      if (same) {
        window_seqs(blk_off.data(), N, W, nwin, w, f2, n2);
        CHECK(f2 == first && n2 == count, "host walk of window %d: %d +%d, plan %d +%d", w, first, count, f2, n2);
        int lg = 0;
        for (int m = first; m < first + count; ++m) {
          int q0, q1;
          window_part(blk_off[m], blk_off[m + 1], c0, c1, q0, q1);
          lg = q1 - q0 > lg ? q1 - q0 : lg;
        }
        CHECK(lg == longest, "longest part of window %d", w);
      }
      checks += 2;
    });
    // chain units of every window and segment count
    std::vector<int> covered(N, 0), starts(N, 0), ends(N, 0), listed(N, 0);
    int prev_out_seq = -1;   // the sequence the previous window carried out
    for (int w = 0; w < nwin; ++w) {
      int c0, c1;
      window_range(w, W, total_blocks, c0, c1);
      const int cnt = win_base[w + 1] - win_base[w];
      int carry_in = 0, carry_out = 0, in_seq = -1, out_seq = -1;
      for (int r = 0; r < cnt; ++r) {
        const int n = order[win_base[w] + r];
        CHECK(0 <= n && n < N, "unit %d of window %d", r, w);
        if (n < 0 || n >= N) continue;
        int s0, s1;
        clamp_seq(dev.data(), n, T, s0, s1);
        const int seq_len = s1 - s0, g0 = blk_off[n], g1 = blk_off[n + 1];
        int p0, p1;
        window_part(g0, g1, c0, c1, p0, p1);
        // every listed sequence has blocks in the window, or is an empty one
        // listed in this window only
        if (same) CHECK(p1 > p0 || g0 == g1, "seq %d listed in window %d without blocks there", n, w);
        if (p0 == p1 && g0 != g1) continue;   // not in this window (differing copies only)
        if (same) {
          listed[n] += g0 == g1;
          covered[n] += p1 - p0;
          starts[n] += p0 == 0;
          ends[n] += g0 + p1 == g1;
        }
        if (p0 != 0) ++carry_in, in_seq = n;
        if (g0 + p1 != g1) ++carry_out, out_seq = n;
        for (int P = 1; P <= 16; P += (P == 1 ? 2 : 5)) {
          int segcov = 0;
          for (int seg = 0; seg < P; ++seg) {
            int b0, b1;
            part_segment(p1 - p0, seg, P, b0, b1);
            const int blk0 = p0 + b0, blk1 = p0 + b1, nblk = blk1 - blk0;
            segcov += nblk;
            if (nblk > 0) {
              // records of the unit inside the window's records of its head
              CHECK(g0 + blk0 - c0 >= 0 && g0 + blk1 - c0 <= c1 - c0, "records of seq %d window %d seg %d/%d", n,
                    w, seg, P);
              const int seg_off = kBT * blk0;
              const int len_raw = seq_len - seg_off < kBT * nblk ? seq_len - seg_off : kBT * nblk;
              const int len = len_raw > 0 ? len_raw : 0;
              if (len > 0) CHECK(s0 + seg_off >= 0 && s0 + seg_off + len <= T, "rows of seq %d window %d", n, w);
              if (interval > 0)
                for (int e = 16; e <= len; e += 16)
                  if ((seg_off + e) % interval == 0) {
                    const int idx = (seg_off + e) / interval - 1;
                    CHECK(idx >= 0 && ck_off[n] >= 0, "checkpoint index of seq %d", n);
                    if (same) CHECK(ck_off[n] + idx < nck, "exact checkpoint slot of seq %d", n);
                  }
              if (same && len_raw <= 0) CHECK(false, "empty rows in a nonempty segment of seq %d", n);
            }
            checks += 2;
          }
          CHECK(segcov == p1 - p0, "segments of seq %d cover its part in window %d", n, w);
        }
      }
      // at most one sequence crosses each window edge
      CHECK(carry_in <= 1 && carry_out <= 1, "window %d: %d carried in, %d out", w, carry_in, carry_out);
      // the state a window carries out is the one the next window carries in
      if (same) CHECK(in_seq == prev_out_seq, "window %d carries in seq %d, window before out %d", w, in_seq,
                      prev_out_seq);
      prev_out_seq = out_seq;
      checks += 2;
    }
    if (same)
      for (int n = 0; n < N; ++n) {
        CHECK(covered[n] == seq_blocks(host[n + 1] - host[n]), "windows cover seq %d: %d blocks", n, covered[n]);
        CHECK(starts[n] == 1 && ends[n] == 1, "seq %d starts %d times, ends %d times", n, starts[n], ends[n]);
        if (host[n + 1] == host[n]) CHECK(listed[n] == 1, "empty seq %d listed %d times", n, listed[n]);
        checks += 2;
      }
  }
  return checks;
}

// The record window a call takes from its workspace (choose_window): one
// window when everything fits, else the most blocks that fit beside the
// tables and carry states, evened out, never past max_window, and 0 only
// when not one block fits.
static long check_windows() {
  long checks = 0;
  for (int it = 0; it < 200000; ++it) {
    const int64_t blocks = rint_in(1, 6000);
    const uint64_t block_bytes = (uint64_t)rint_in(1, 1 << 20);
    const uint64_t tables = (uint64_t)rint_in(0, 1 << 16), carry = (uint64_t)rint_in(0, 1 << 20);
    const uint64_t one = tables + (uint64_t)blocks * block_bytes, fixed = tables + carry;
    const int64_t max_window = it % 3 == 0 ? 65535 : rint_in(1, 8000);
    const uint64_t ws = it % 5 == 0 ? one : (uint64_t)((double)(rnd() % 1000) / 500.0 * (double)one);
    const int64_t w = choose_window(blocks, ws, one, fixed, block_bytes, max_window);
    if (blocks <= max_window && ws >= one) {
      CHECK(w == blocks, "one window: %lld of %lld", (long long)w, (long long)blocks);
    } else if (ws < fixed || (ws - fixed) / block_bytes < 1) {
      CHECK(w == 0, "nothing fits, got %lld", (long long)w);
    } else {
      const int64_t raw = std::min<int64_t>((int64_t)((ws - fixed) / block_bytes), max_window);
      const int64_t nwin = (blocks + w - 1) / w;
      CHECK(w >= 1 && w <= max_window && w <= raw, "window %lld (raw %lld, max %lld)", (long long)w,
            (long long)raw, (long long)max_window);
      CHECK(fixed + (uint64_t)w * block_bytes <= ws, "window %lld does not fit", (long long)w);
      CHECK(w * (nwin - 1) < blocks && blocks <= w * nwin, "windows of %lld over %lld blocks", (long long)w,
            (long long)blocks);
      CHECK(nwin == (blocks + raw - 1) / raw, "evening changed the window count");
      CHECK(blocks - w * (nwin - 1) > w - nwin, "last window of %lld blocks, others %lld",
            (long long)(blocks - w * (nwin - 1)), (long long)w);   // evened out
    }
    ++checks;
  }
  return checks;
}

int main() {
  long checks = check_windows(), cases = 0;
  for (int it = 0; it < 4000; ++it) {
    const int N = rint_in(1, 12);
    const int mode = it % 8;
    std::vector<int32_t> host(N + 1, 0);
    for (int n = 0; n < N; ++n) {
      const int r = rint_in(0, 9);
      const int len = r == 0 ? 0 : (r < 3 ? rint_in(1, 40) : rint_in(0, 400));
      host[n + 1] = host[n] + len;
    }
    const int interval = (it % 3 == 0) ? 0 : 16 * rint_in(1, 6);
    std::vector<int32_t> dev = host;
    switch (mode) {
      case 0: break;                                                      // equal copies
      case 1: for (auto& x : dev) x += rint_in(-50, 50); break;           // shifted
      case 2: for (auto& x : dev) x = rint_in(-100, 2 * (host[N] + 1)); break;   // arbitrary
      case 3: for (auto& x : dev) x *= 3; break;                          // past the total
      case 4: for (int n = 0; n <= N; ++n) dev[n] = host[N - n]; break;   // decreasing
      case 5: dev[rint_in(0, N)] = rint_in(0, 1) ? 0x7fffffff : (int32_t)0x80000000; break;
      case 6: for (int n = 1; n <= N; ++n) dev[n] = dev[n - 1] + rint_in(0, 600); break;   // other lengths
      case 7: dev[0] = rint_in(1, 64); break;                             // cu[0] != 0
    }
    checks += run_case(host, dev, interval, mode == 0);
    ++cases;
  }
  // a sequence far longer than the total (int64 row arithmetic)
  {
    std::vector<int32_t> host = {0, 64, 96}, dev = {0, 0x7fff0000, 0x7fffffff};
    checks += run_case(host, dev, 32, false);
    ++cases;
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok %ld cases %ld checks\n", cases, checks);
  return 0;
}
