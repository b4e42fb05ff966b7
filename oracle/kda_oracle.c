/*
 * KDA oracle: plain fp64 token-by-token recurrence on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the correctness reference for the
 * HIP library; it shares no code, header, table or helper with it. Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg load it.
 * Nothing on the product path may call it.
 *
 * Pages cited (by title and section):
 *   [K3-SA] "LLM - Semianalysis, Kimi K3 아키텍처" (charstring.tistory.com/2557)
 *   [K3-DD] "MoonshotAI/Kimi-K3 딥다이브" (fiv.co.kr/repos/kimi-k3-deep-dive.html)
 *
 * What is computed, per sequence n and head h, token by token:
 *   [K3-SA, 배경/Background]: linear attention folds all past keys/values
 *   into one state matrix S; DeltaNet updates S by a step that reduces the
 *   squared L2 error of retrieving v_t with key k_t; Gated DeltaNet adds a
 *   forget gate; KDA turns that gate into a diagonal matrix, i.e. one decay
 *   per key channel.  [K3-DD, 4-1 KDA, first bullet]: the per-channel decay
 *   has a lower bound.  The plainest reading of these, used here:
 *
 *     alpha_t = exp(clamp(g_t, g_min, 0))             (Dk, per key channel)
 *     S'      = Diag(alpha_t) S_{t-1}                  (gate first)
 *     S_t     = S' + beta_t k_t (v_t - S'^T k_t)^T     (one gradient step of
 *                size beta_t on 1/2 ||S^T k_t - v_t||^2 = (I - b k k^T)S' + b k v^T)
 *     o_t     = scale * S_t^T q_t                      (read out after update)
 *
 *   [K3-SA, Methods 1) FlashKDA]: decode runs exactly this recurrence, one
 *   token at a time; prefill only reorganises it into chunks.
 *   [K3-SA, Methods 3) KV cache efficiency] and the Conclusion table's
 *   prefix-caching row: the recurrent state is saved only at sparse token
 *   intervals; here a checkpoint is S after every ckpt_interval tokens of a
 *   sequence, counted from that sequence's first token in the call.
 *
 * Parity status: every function here is pinned by the CPU test suite (exact
 * rational brute force, a dense transition-matrix form, closed forms and
 * invariants).
 *
 * Layouts (row-major, contiguous):
 *   q, k, g : [T_tot, H, Dk]  float  (values exactly as the device sees them)
 *   v       : [T_tot, H, Dv]  float
 *   beta    : [T_tot, H]      float
 *   states  : [N, H, Dk, Dv]  double
 *   ckpts   : [sum_n floor(L_n / I), H, Dk, Dv] double, sequence-major
 *   o       : [T_tot, H, Dv]  double
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_NO_MEM = 2 };

static double clamp_gate(double g, double g_min) {
  if (g < g_min) g = g_min;
  if (g > 0.0) g = 0.0;
  return g;
}

/* One token of the recurrence on S (Dk x Dv, row = key channel). u is Dv
 * scratch. Writes o_t (Dv) if o is not NULL. */
static void token_step(double* S, double* u, int Dk, int Dv,
                       const float* q, const float* k, const float* v,
                       const float* g, double beta, double scale, double g_min,
                       double* o) {
  /* gate: S' = Diag(alpha) S */
  for (int c = 0; c < Dk; ++c) {
    double a = exp(clamp_gate((double)g[c], g_min));
    double* row = S + (size_t)c * Dv;
    for (int j = 0; j < Dv; ++j) row[j] *= a;
  }
  /* retrieval with the gated state: u = S'^T k */
  for (int j = 0; j < Dv; ++j) u[j] = 0.0;
  for (int c = 0; c < Dk; ++c) {
    double kc = (double)k[c];
    const double* row = S + (size_t)c * Dv;
    for (int j = 0; j < Dv; ++j) u[j] += row[j] * kc;
  }
  /* delta write: S = S' + k (beta (v - u))^T */
  for (int j = 0; j < Dv; ++j) u[j] = beta * ((double)v[j] - u[j]);
  for (int c = 0; c < Dk; ++c) {
    double kc = (double)k[c];
    double* row = S + (size_t)c * Dv;
    for (int j = 0; j < Dv; ++j) row[j] += kc * u[j];
  }
  /* readout from the updated state: o = scale S^T q */
  if (o) {
    for (int j = 0; j < Dv; ++j) o[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
      double qc = (double)q[c];
      const double* row = S + (size_t)c * Dv;
      for (int j = 0; j < Dv; ++j) o[j] += row[j] * qc;
    }
    for (int j = 0; j < Dv; ++j) o[j] *= scale;
  }
}

/* Number of checkpoints a call emits: sum_n floor(L_n / ckpt_interval). */
int64_t kda_oracle_num_checkpoints(const int64_t* cu_seqlens, int32_t num_seqs,
                                   int64_t ckpt_interval) {
  if (ckpt_interval <= 0) return 0;
  int64_t total = 0;
  for (int32_t n = 0; n < num_seqs; ++n)
    total += (cu_seqlens[n + 1] - cu_seqlens[n]) / ckpt_interval;
  return total;
}

int kda_oracle_prefill(const float* q, const float* k, const float* v,
                       const float* g, const float* beta,
                       const int64_t* cu_seqlens, int32_t num_seqs, int32_t H,
                       int32_t Dk, int32_t Dv, double scale, double g_min,
                       const double* initial_state, double* final_state,
                       int64_t ckpt_interval, double* checkpoints, double* o,
                       int32_t num_threads) {
  if (!q || !k || !v || !g || !beta || !cu_seqlens || num_seqs < 0 || H <= 0 ||
      Dk <= 0 || Dv <= 0 || ckpt_interval < 0 || (ckpt_interval > 0 && !checkpoints))
    return ORACLE_BAD_ARG;
  if (cu_seqlens[0] != 0) return ORACLE_BAD_ARG;
  for (int32_t n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return ORACLE_BAD_ARG;

  /* first checkpoint slot of each sequence */
  int64_t* ck_base = (int64_t*)malloc(sizeof(int64_t) * (size_t)(num_seqs + 1));
  if (!ck_base) return ORACLE_NO_MEM;
  ck_base[0] = 0;
  for (int32_t n = 0; n < num_seqs; ++n)
    ck_base[n + 1] = ck_base[n] + (ckpt_interval > 0
                                       ? (cu_seqlens[n + 1] - cu_seqlens[n]) / ckpt_interval
                                       : 0);
  const int64_t units = (int64_t)num_seqs * H;
  const size_t ssz = (size_t)Dk * Dv;
  int err = ORACLE_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < units; ++unit) {
    const int32_t n = (int32_t)(unit / H), h = (int32_t)(unit % H);
    double* S = (double*)malloc(sizeof(double) * (ssz + (size_t)Dv));
    if (!S) {
#pragma omp atomic write
      err = ORACLE_NO_MEM;
      continue;
    }
    double* u = S + ssz;
    if (initial_state)
      memcpy(S, initial_state + (size_t)unit * ssz, sizeof(double) * ssz);
    else
      memset(S, 0, sizeof(double) * ssz);
    const int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1];
    int64_t ck = ck_base[n];
    for (int64_t t = t0; t < t1; ++t) {
      const size_t th = (size_t)t * H + h;
      token_step(S, u, Dk, Dv, q + th * Dk, k + th * Dk, v + th * Dv, g + th * Dk,
                 (double)beta[th], scale, g_min, o ? o + th * Dv : NULL);
      if (ckpt_interval > 0 && (t - t0 + 1) % ckpt_interval == 0) {
        memcpy(checkpoints + ((size_t)ck * H + h) * ssz, S, sizeof(double) * ssz);
        ++ck;
      }
    }
    if (final_state) memcpy(final_state + (size_t)unit * ssz, S, sizeof(double) * ssz);
    free(S);
  }
  free(ck_base);
  return err;
}

/* One decode token for each of N sequences: state_in -> state_out, o.
 * Same step as prefill [K3-SA, Methods 1) FlashKDA: decode runs the
 * recurrence directly]. q,k,g: [N,H,Dk]; v: [N,H,Dv]; beta: [N,H];
 * states: [N,H,Dk,Dv] double; o: [N,H,Dv] double. state_out may alias
 * state_in. */
int kda_oracle_decode(const float* q, const float* k, const float* v,
                      const float* g, const float* beta, const double* state_in,
                      double* state_out, double* o, int32_t N, int32_t H,
                      int32_t Dk, int32_t Dv, double scale, double g_min,
                      int32_t num_threads) {
  if (!q || !k || !v || !g || !beta || !state_in || !state_out || !o || N < 0 ||
      H <= 0 || Dk <= 0 || Dv <= 0)
    return ORACLE_BAD_ARG;
  const int64_t units = (int64_t)N * H;
  const size_t ssz = (size_t)Dk * Dv;
  int err = ORACLE_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t unit = 0; unit < units; ++unit) {
    double* S = (double*)malloc(sizeof(double) * (ssz + (size_t)Dv));
    if (!S) {
#pragma omp atomic write
      err = ORACLE_NO_MEM;
      continue;
    }
    memcpy(S, state_in + (size_t)unit * ssz, sizeof(double) * ssz);
    token_step(S, S + ssz, Dk, Dv, q + (size_t)unit * Dk, k + (size_t)unit * Dk,
               v + (size_t)unit * Dv, g + (size_t)unit * Dk, (double)beta[unit],
               scale, g_min, o + (size_t)unit * Dv);
    memcpy(state_out + (size_t)unit * ssz, S, sizeof(double) * ssz);
    free(S);
  }
  return err;
}

/* Threads the OpenMP runtime would use (for reporting the CPU baseline). */
int32_t kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}
