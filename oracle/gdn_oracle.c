/*
 * gdn_oracle.c -- plain, slow, fp64 CPU reference of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, constant or helper with
 * the HIP library.
 *
 * What it computes (per lane, per layer, per value head h, independently):
 *
 *   The gated delta rule of Yang, Kautz & Hatamizadeh, "Gated Delta Networks:
 *   Improving Mamba2 with Delta Rule" (ICLR 2025), Sec. 3 (the gated delta
 *   rule), with the state S as a dv x dk matrix that maps keys to values:
 *
 *     khat_t = k_t / sqrt(sum_j k_tj^2 + eps)   (only when l2norm != 0)
 *     qhat_t = q_t / sqrt(sum_j q_tj^2 + eps)   (only when l2norm != 0)
 *     alpha_t = exp(g_t)
 *     p_t     = alpha_t * S_{t-1} khat_t              (prediction)
 *     u_t     = beta_t * (v_t - p_t)                  (delta)
 *     S_t     = alpha_t * S_{t-1} + u_t khat_t^T      (rank-1 write)
 *     o_t     = scale * S_t qhat_t                    (output reads S_t)
 *
 *   Value head h reads key head floor(h / (h_v / h_k)).
 *
 *   ReplaySSM commit (NInfer technical review, blog.123qwe.co.kr post 4624,
 *   section "Architecture 3: speculative decoding and ReplaySSM"): the state
 *   that a commit of m accepted window tokens produces is the state after the
 *   first m steps from the untouched window checkpoint S_0, i.e. S_m; m = 0
 *   leaves S_0 as it is.  The oracle reaches S_m by running the rule for m
 *   steps -- records are an implementation device and do not appear here.
 *
 *   Draft trees (the first page, the description of the MC engine: draft
 *   trees used together with DFlash2): the window is a tree of T nodes in
 *   an order where every node comes after its parent; node t's state is one
 *   step of the rule from its parent's state (from S_0 for the root), and a
 *   commit of an accepted root-to-node path is the state after the steps of
 *   the path's nodes, in order, from S_0.
 *
 *   Chunked prefill (same review, section "Architecture 2: context byte pool
 *   and prefix reuse", the context_cache.checkpoint_interval setting): the
 *   oracle runs the same rule token by token over the whole sequence and
 *   copies the state out after every multiple of the checkpoint interval.
 *   Chunking and the WY/UT block form are implementation devices that reach
 *   the same values; they do not appear here.
 *
 * Storage: S[j][i] holds the matrix entry S_ij (row i = value index in
 * 0..dv-1, column j = key index in 0..dk-1), i.e. key-major with the value
 * index contiguous.  This is only a layout; the arithmetic above is the
 * definition.
 *
 * Parallelism: OpenMP over independent (layer, lane, head) chains only.  No
 * blocking, fusion or reordering inside a chain.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_EPS 1e-6

/* Normalise x (length n) into out: out = x / sqrt(sum x^2 + eps), or copy. */
static void l2_normalise(const double* x, int n, int l2norm, double* out) {
  if (!l2norm) {
    for (int j = 0; j < n; ++j) out[j] = x[j];
    return;
  }
  double ss = 0.0;
  for (int j = 0; j < n; ++j) ss += x[j] * x[j];
  double inv = 1.0 / sqrt(ss + ORACLE_EPS);
  for (int j = 0; j < n; ++j) out[j] = x[j] * inv;
}

/*
 * One step of the gated delta rule on a single head's state S (dk x dv
 * storage, S[j*dv + i] = S_ij).  Writes o (length dv) when o != NULL.
 * kh, qh are already normalised.  work has room for dv doubles.
 */
static void gdr_step(int dk, int dv, double* S, const double* kh,
                     const double* qh, const double* v, double beta, double g,
                     double scale, double* o, double* work) {
  const double alpha = exp(g);
  double* u = work;
  /* p_i = alpha * sum_j S_ij khat_j ; u_i = beta * (v_i - p_i) */
  for (int i = 0; i < dv; ++i) {
    double acc = 0.0;
    for (int j = 0; j < dk; ++j) acc += S[(size_t)j * dv + i] * kh[j];
    double p = alpha * acc;
    u[i] = beta * (v[i] - p);
  }
  /* S_ij <- alpha * S_ij + u_i * khat_j */
  for (int j = 0; j < dk; ++j)
    for (int i = 0; i < dv; ++i)
      S[(size_t)j * dv + i] = alpha * S[(size_t)j * dv + i] + u[i] * kh[j];
  /* o_i = scale * sum_j S_ij qhat_j (post-update state) */
  if (o) {
    for (int i = 0; i < dv; ++i) {
      double acc = 0.0;
      for (int j = 0; j < dk; ++j) acc += S[(size_t)j * dv + i] * qh[j];
      o[i] = scale * acc;
    }
  }
}

/*
 * Speculative-window verify, oracle form.
 *
 * Layouts (all fp64, contiguous, row-major in the order written):
 *   q, k   [n_layers][n_lanes][t_max][h_k][d_k]
 *   v      [n_layers][n_lanes][t_max][h_v][d_v]
 *   beta,g [n_layers][n_lanes][t_max][h_v]
 *   S0     [n_layers][n_lanes][h_v][d_k][d_v]       (read only)
 *   o      [n_layers][n_lanes][t_max][h_v][d_v]     rows t >= T_lane untouched
 *   states [n_layers][n_lanes][t_max][h_v][d_k][d_v] nullable; S_1..S_T
 * t_lane[lane] in 1..t_max is the window length of each lane.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_verify(int n_layers, int n_lanes, int h_v, int h_k, int d_k,
                  int d_v, int t_max, const int32_t* t_lane, const double* q,
                  const double* k, const double* v, const double* beta,
                  const double* g, const double* S0, double scale, int l2norm,
                  double* o, double* states) {
  if (n_layers < 1 || n_lanes < 1 || h_v < 1 || h_k < 1 || d_k < 1 ||
      d_v < 1 || t_max < 1 || h_v % h_k != 0)
    return -1;
  for (int n = 0; n < n_lanes; ++n)
    if (t_lane[n] < 0 || t_lane[n] > t_max) return -1;
  const int group = h_v / h_k;
  const long n_chains = (long)n_layers * n_lanes * h_v;
  const size_t hs = (size_t)d_k * d_v;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long c = 0; c < n_chains; ++c) {
    const int h = (int)(c % h_v);
    const int lane = (int)((c / h_v) % n_lanes);
    const int layer = (int)(c / ((long)h_v * n_lanes));
    const int kh_idx = h / group;
    const long ll = (long)layer * n_lanes + lane;
    double* S = (double*)malloc(hs * sizeof(double));
    double* kh = (double*)malloc((size_t)d_k * sizeof(double));
    double* qh = (double*)malloc((size_t)d_k * sizeof(double));
    double* work = (double*)malloc((size_t)d_v * sizeof(double));
    if (!S || !kh || !qh || !work) {
      bad = 1;
    } else {
      memcpy(S, S0 + ((size_t)ll * h_v + h) * hs, hs * sizeof(double));
      for (int t = 0; t < t_lane[lane]; ++t) {
        const size_t tok = (size_t)ll * t_max + t;
        l2_normalise(k + (tok * h_k + kh_idx) * d_k, d_k, l2norm, kh);
        l2_normalise(q + (tok * h_k + kh_idx) * d_k, d_k, l2norm, qh);
        gdr_step(d_k, d_v, S, kh, qh, v + (tok * h_v + h) * d_v,
                 beta[tok * h_v + h], g[tok * h_v + h], scale,
                 o + (tok * h_v + h) * d_v, work);
        if (states)
          memcpy(states + (tok * h_v + h) * hs, S, hs * sizeof(double));
      }
    }
    free(S); free(kh); free(qh); free(work);
  }
  return bad ? -2 : 0;
}

/*
 * Commit, oracle form: S (same layout as S0 above) is replaced, for every
 * lane with m_lane[lane] > 0, by the state after the first m_lane[lane] window
 * steps from the S it holds on entry.  Lanes with m = 0 are left untouched.
 */
int oracle_commit(int n_layers, int n_lanes, int h_v, int h_k, int d_k,
                  int d_v, int t_max, const int32_t* m_lane, const double* q,
                  const double* k, const double* v, const double* beta,
                  const double* g, double* S, int l2norm) {
  if (n_layers < 1 || n_lanes < 1 || h_v < 1 || h_k < 1 || d_k < 1 ||
      d_v < 1 || t_max < 1 || h_v % h_k != 0)
    return -1;
  for (int n = 0; n < n_lanes; ++n)
    if (m_lane[n] < 0 || m_lane[n] > t_max) return -1;
  const int group = h_v / h_k;
  const long n_chains = (long)n_layers * n_lanes * h_v;
  const size_t hs = (size_t)d_k * d_v;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long c = 0; c < n_chains; ++c) {
    const int h = (int)(c % h_v);
    const int lane = (int)((c / h_v) % n_lanes);
    const int layer = (int)(c / ((long)h_v * n_lanes));
    const int kh_idx = h / group;
    const long ll = (long)layer * n_lanes + lane;
    if (m_lane[lane] == 0) continue;
    double* kh = (double*)malloc((size_t)d_k * sizeof(double));
    double* qh = (double*)malloc((size_t)d_k * sizeof(double));
    double* work = (double*)malloc((size_t)d_v * sizeof(double));
    if (!kh || !qh || !work) {
      bad = 1;
    } else {
      double* Sh = S + ((size_t)ll * h_v + h) * hs;
      for (int t = 0; t < m_lane[lane]; ++t) {
        const size_t tok = (size_t)ll * t_max + t;
        l2_normalise(k + (tok * h_k + kh_idx) * d_k, d_k, l2norm, kh);
        l2_normalise(q + (tok * h_k + kh_idx) * d_k, d_k, l2norm, qh);
        gdr_step(d_k, d_v, Sh, kh, qh, v + (tok * h_v + h) * d_v,
                 beta[tok * h_v + h], g[tok * h_v + h], 1.0, NULL, work);
      }
    }
    free(kh); free(qh); free(work);
  }
  return bad ? -2 : 0;
}

/*
 * Draft-tree verify, oracle form.  Layouts as oracle_verify; parent is
 * int32 [n_lanes][t_max]: parent[t] in -1..t-1 (-1: the node hangs off S_0).
 * Node t's state is one step of the rule applied to its parent's state;
 * states (nullable) receives every node's state.
 */
int oracle_verify_tree(int n_layers, int n_lanes, int h_v, int h_k, int d_k,
                       int d_v, int t_max, const int32_t* t_lane,
                       const int32_t* parent, const double* q,
                       const double* k, const double* v, const double* beta,
                       const double* g, const double* S0, double scale,
                       int l2norm, double* o, double* states) {
  if (n_layers < 1 || n_lanes < 1 || h_v < 1 || h_k < 1 || d_k < 1 ||
      d_v < 1 || t_max < 1 || h_v % h_k != 0)
    return -1;
  for (int n = 0; n < n_lanes; ++n) {
    if (t_lane[n] < 0 || t_lane[n] > t_max) return -1;
    for (int t = 0; t < t_lane[n]; ++t) {
      const int p = parent[(size_t)n * t_max + t];
      if (p < -1 || p >= t) return -1;
    }
  }
  const int group = h_v / h_k;
  const long n_chains = (long)n_layers * n_lanes * h_v;
  const size_t hs = (size_t)d_k * d_v;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long c = 0; c < n_chains; ++c) {
    const int h = (int)(c % h_v);
    const int lane = (int)((c / h_v) % n_lanes);
    const int layer = (int)(c / ((long)h_v * n_lanes));
    const int kh_idx = h / group;
    const long ll = (long)layer * n_lanes + lane;
    double* node = (double*)malloc((size_t)t_max * hs * sizeof(double));
    double* kh = (double*)malloc((size_t)d_k * sizeof(double));
    double* qh = (double*)malloc((size_t)d_k * sizeof(double));
    double* work = (double*)malloc((size_t)d_v * sizeof(double));
    if (!node || !kh || !qh || !work) {
      bad = 1;
    } else {
      for (int t = 0; t < t_lane[lane]; ++t) {
        const int p = parent[(size_t)lane * t_max + t];
        double* S = node + (size_t)t * hs;
        memcpy(S, p < 0 ? S0 + ((size_t)ll * h_v + h) * hs
                        : node + (size_t)p * hs, hs * sizeof(double));
        const size_t tok = (size_t)ll * t_max + t;
        l2_normalise(k + (tok * h_k + kh_idx) * d_k, d_k, l2norm, kh);
        l2_normalise(q + (tok * h_k + kh_idx) * d_k, d_k, l2norm, qh);
        gdr_step(d_k, d_v, S, kh, qh, v + (tok * h_v + h) * d_v,
                 beta[tok * h_v + h], g[tok * h_v + h], scale,
                 o + (tok * h_v + h) * d_v, work);
        if (states)
          memcpy(states + (tok * h_v + h) * hs, S, hs * sizeof(double));
      }
    }
    free(node); free(kh); free(qh); free(work);
  }
  return bad ? -2 : 0;
}

/*
 * Commit of an accepted path, oracle form: for every lane with
 * m_lane[lane] > 0, S is advanced by the steps of nodes path[lane][0..m-1]
 * in that order (path int32 [n_lanes][t_max], node indices).
 */
int oracle_commit_path(int n_layers, int n_lanes, int h_v, int h_k, int d_k,
                       int d_v, int t_max, const int32_t* m_lane,
                       const int32_t* path, const double* q, const double* k,
                       const double* v, const double* beta, const double* g,
                       double* S, int l2norm) {
  if (n_layers < 1 || n_lanes < 1 || h_v < 1 || h_k < 1 || d_k < 1 ||
      d_v < 1 || t_max < 1 || h_v % h_k != 0)
    return -1;
  for (int n = 0; n < n_lanes; ++n) {
    if (m_lane[n] < 0 || m_lane[n] > t_max) return -1;
    for (int j = 0; j < m_lane[n]; ++j) {
      const int node = path[(size_t)n * t_max + j];
      if (node < 0 || node >= t_max) return -1;
    }
  }
  const int group = h_v / h_k;
  const long n_chains = (long)n_layers * n_lanes * h_v;
  const size_t hs = (size_t)d_k * d_v;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long c = 0; c < n_chains; ++c) {
    const int h = (int)(c % h_v);
    const int lane = (int)((c / h_v) % n_lanes);
    const int layer = (int)(c / ((long)h_v * n_lanes));
    const int kh_idx = h / group;
    const long ll = (long)layer * n_lanes + lane;
    if (m_lane[lane] == 0) continue;
    double* kh = (double*)malloc((size_t)d_k * sizeof(double));
    double* qh = (double*)malloc((size_t)d_k * sizeof(double));
    double* work = (double*)malloc((size_t)d_v * sizeof(double));
    if (!kh || !qh || !work) {
      bad = 1;
    } else {
      double* Sh = S + ((size_t)ll * h_v + h) * hs;
      for (int j = 0; j < m_lane[lane]; ++j) {
        const size_t tok = (size_t)ll * t_max + path[(size_t)lane * t_max + j];
        l2_normalise(k + (tok * h_k + kh_idx) * d_k, d_k, l2norm, kh);
        l2_normalise(q + (tok * h_k + kh_idx) * d_k, d_k, l2norm, qh);
        gdr_step(d_k, d_v, Sh, kh, qh, v + (tok * h_v + h) * d_v,
                 beta[tok * h_v + h], g[tok * h_v + h], 1.0, NULL, work);
      }
    }
    free(kh); free(qh); free(work);
  }
  return bad ? -2 : 0;
}

/*
 * KDA, the sibling rule with a decay per key channel (Kimi Delta Attention,
 * Kimi Linear, 2025; the review names its recurrent state and a kda_replay
 * op contract beside gdn_replay).  With alpha_t a d_k vector,
 *     S'_t = S_{t-1} diag(alpha_t)          (column j scaled by alpha_tj)
 *     p_t  = S'_t khat_t
 *     u_t  = beta_t (v_t - p_t)
 *     S_t  = S'_t + u_t khat_t^T
 *     o_t  = scale * S_t qhat_t
 * alpha_tj = exp(g_tj).  g is [..][h_v][d_k] (per value head and channel).
 */
static void kda_step(int dk, int dv, double* S, const double* kh,
                     const double* qh, const double* v, double beta,
                     const double* g, double scale, double* o, double* work) {
  double* u = work;
  /* S' = S diag(alpha) */
  for (int j = 0; j < dk; ++j) {
    const double a = exp(g[j]);
    for (int i = 0; i < dv; ++i) S[(size_t)j * dv + i] *= a;
  }
  /* p = S' khat; u = beta (v - p) */
  for (int i = 0; i < dv; ++i) {
    double acc = 0.0;
    for (int j = 0; j < dk; ++j) acc += S[(size_t)j * dv + i] * kh[j];
    u[i] = beta * (v[i] - acc);
  }
  /* S = S' + u khat^T */
  for (int j = 0; j < dk; ++j)
    for (int i = 0; i < dv; ++i) S[(size_t)j * dv + i] += u[i] * kh[j];
  if (o) {
    for (int i = 0; i < dv; ++i) {
      double acc = 0.0;
      for (int j = 0; j < dk; ++j) acc += S[(size_t)j * dv + i] * qh[j];
      o[i] = scale * acc;
    }
  }
}

/*
 * KDA window verify (states nullable) and, with o == NULL and m_lane != NULL,
 * commit: S advanced by the first m_lane[lane] steps.  Layouts as
 * oracle_verify except g: [n_layers][n_lanes][t_max][h_v][d_k].
 */
int oracle_kda(int n_layers, int n_lanes, int h_v, int h_k, int d_k, int d_v,
               int t_max, const int32_t* t_lane, const int32_t* m_lane,
               const double* q, const double* k, const double* v,
               const double* beta, const double* g, double* S, double scale,
               int l2norm, double* o, double* states) {
  if (n_layers < 1 || n_lanes < 1 || h_v < 1 || h_k < 1 || d_k < 1 ||
      d_v < 1 || t_max < 1 || h_v % h_k != 0)
    return -1;
  for (int n = 0; n < n_lanes; ++n) {
    const int steps = m_lane ? m_lane[n] : t_lane[n];
    if (steps < 0 || steps > t_max) return -1;
  }
  const int group = h_v / h_k;
  const long n_chains = (long)n_layers * n_lanes * h_v;
  const size_t hs = (size_t)d_k * d_v;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long c = 0; c < n_chains; ++c) {
    const int h = (int)(c % h_v);
    const int lane = (int)((c / h_v) % n_lanes);
    const int layer = (int)(c / ((long)h_v * n_lanes));
    const int kh_idx = h / group;
    const long ll = (long)layer * n_lanes + lane;
    const int steps = m_lane ? m_lane[lane] : t_lane[lane];
    double* Sw = (double*)malloc(hs * sizeof(double));
    double* kh = (double*)malloc((size_t)d_k * sizeof(double));
    double* qh = (double*)malloc((size_t)d_k * sizeof(double));
    double* work = (double*)malloc((size_t)d_v * sizeof(double));
    if (!Sw || !kh || !qh || !work) {
      bad = 1;
    } else {
      double* Sh = S + ((size_t)ll * h_v + h) * hs;
      memcpy(Sw, Sh, hs * sizeof(double));
      for (int t = 0; t < steps; ++t) {
        const size_t tok = (size_t)ll * t_max + t;
        l2_normalise(k + (tok * h_k + kh_idx) * d_k, d_k, l2norm, kh);
        l2_normalise(q + (tok * h_k + kh_idx) * d_k, d_k, l2norm, qh);
        kda_step(d_k, d_v, Sw, kh, qh, v + (tok * h_v + h) * d_v,
                 beta[tok * h_v + h], g + (tok * h_v + h) * d_k, scale,
                 m_lane ? NULL : o + (tok * h_v + h) * d_v, work);
        if (states && !m_lane)
          memcpy(states + (tok * h_v + h) * hs, Sw, hs * sizeof(double));
      }
      if (m_lane) memcpy(Sh, Sw, hs * sizeof(double));
    }
    free(Sw); free(kh); free(qh); free(work);
  }
  return bad ? -2 : 0;
}

/*
 * Prefill, oracle form: one sequence of seq_len tokens, token by token.
 *   q, k   [seq_len][h_k][d_k]
 *   v      [seq_len][h_v][d_v]
 *   beta,g [seq_len][h_v]
 *   S_init [h_v][d_k][d_v]   nullable: zero state
 *   o      [seq_len][h_v][d_v]
 *   ckpt   [seq_len / ckpt_interval][h_v][d_k][d_v]  nullable; the state
 *          after token ckpt_interval * (c + 1), for every such multiple
 *          that is <= seq_len
 *   S_final[h_v][d_k][d_v]
 */
int oracle_prefill(int seq_len, int h_v, int h_k, int d_k, int d_v,
                   int ckpt_interval, const double* q, const double* k,
                   const double* v, const double* beta, const double* g,
                   const double* S_init, double scale, int l2norm, double* o,
                   double* ckpt, double* S_final) {
  if (seq_len < 0 || h_v < 1 || h_k < 1 || d_k < 1 || d_v < 1 ||
      h_v % h_k != 0 || (ckpt && ckpt_interval < 1))
    return -1;
  const int group = h_v / h_k;
  const size_t hs = (size_t)d_k * d_v;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < h_v; ++h) {
    const int kh_idx = h / group;
    double* S = S_final + (size_t)h * hs;
    double* kh = (double*)malloc((size_t)d_k * sizeof(double));
    double* qh = (double*)malloc((size_t)d_k * sizeof(double));
    double* work = (double*)malloc((size_t)d_v * sizeof(double));
    if (!kh || !qh || !work) {
      bad = 1;
    } else {
      if (S_init)
        memcpy(S, S_init + (size_t)h * hs, hs * sizeof(double));
      else
        memset(S, 0, hs * sizeof(double));
      for (int t = 0; t < seq_len; ++t) {
        l2_normalise(k + ((size_t)t * h_k + kh_idx) * d_k, d_k, l2norm, kh);
        l2_normalise(q + ((size_t)t * h_k + kh_idx) * d_k, d_k, l2norm, qh);
        gdr_step(d_k, d_v, S, kh, qh, v + ((size_t)t * h_v + h) * d_v,
                 beta[(size_t)t * h_v + h], g[(size_t)t * h_v + h], scale,
                 o + ((size_t)t * h_v + h) * d_v, work);
        if (ckpt && (t + 1) % ckpt_interval == 0) {
          const size_t c = (size_t)((t + 1) / ckpt_interval - 1);
          memcpy(ckpt + (c * h_v + h) * hs, S, hs * sizeof(double));
        }
      }
    }
    free(kh); free(qh); free(work);
  }
  return bad ? -2 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the OpenMP loops over independent chains (the CPU
 * baseline is timed at one thread and at all cores).  Not arithmetic: every
 * chain runs the same loop nest whatever the count. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
