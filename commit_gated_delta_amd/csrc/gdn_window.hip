// gdn_window.hip -- speculative-window verify and ReplaySSM commit for gfx950.
//
// The path, per (layer, lane, value head) and window of T <= t_max tokens:
//   verify  hold the head's S0 in registers, run the gated delta rule
//           (Gated DeltaNet, ICLR 2025, Sec. 3) token by token, write
//           o_t = scale * S_t qhat_t and compact per-token records.  S0 in
//           memory is never written.
//   commit  reload S0, replay the first m records with the same per-step
//           instruction sequence (gdn_step.h), store S_m in place
//           (ReplaySSM section of the NInfer technical review,
//           blog.123qwe.co.kr post 4624).
//
// Arithmetic of one step, with raw key k and query q (the L2 norms are
// folded into scalars so the raw bf16 values can be used as exact f32
// operands) and the state in the scaled form S = c * St of gdn_step.h:
//   rk = 1/sqrt(|k|^2 + 1e-6), rq likewise     (1 when normalisation is off)
//   alpha = exp(g);  c <- c * alpha            (folded into St if out of range)
//   P_i   = sum_j St_ij k_j                     (dk-reduction)
//   p_i   = (c * rk) * P_i                      (= alpha * (S_{t-1} khat)_i)
//   ut_i  = (beta * (v_i - p_i)) * (rk / c)     (= u_i * rk / c)
//   St_ij <- fma(ut_i, k_j, St_ij)              (S = alpha S + u khat^T)
//   o_i   = (scale * rq * c) * sum_j St_ij q_j
// Records per token: per value head the scale step (phi, c) as a float2 --
// phi the factor folded into St before the token (1 when none), c the scale
// after it -- ut (f32 per value head and column) and the raw key row widened
// to f32 (per key head).  Commit replays the same folds and St_ij <-
// fma(ut_i, k_j, St_ij) from exactly these values and stores S_m = c * St, so
// its result is bitwise the state verify held after the same token.
//
// Work decomposition (CDNA4, wave64):
//   One 256-thread workgroup per (layer, lane, value head, block of 64 value
//   columns).  Lane x of every wave owns column i = 64*cb + x; wave w owns
//   key rows j in [w*dk/4, (w+1)*dk/4).  A lane keeps its dk/4 state entries
//   in VGPRs for the whole window (32 at dk = 128), which leaves room for
//   eight waves per SIMD to hide memory latency.
//   Per token, one pass over the held entries forms the partial sums of
//   St k (prediction) and St q (output) from the state before the token's
//   write; the four wave partials meet in LDS behind one barrier; the
//   output uses S_t q = c_t (St_{t-1} q + ut (k . q)); a second pass applies
//   the write.  The key and query values of a wave's rows are the same for
//   all its lanes: they come in through scalar loads (SGPRs), bf16 pairs
//   unpacked with two scalar ALU ops, and every multiply-add takes them as
//   its SGPR operand -- no LDS broadcast traffic on the hot loop.
//   A prologue computes the norms, k . q and the whole scale sequence of
//   the window once and leaves the per-token scalars in LDS.
//   State loads/stores: for a fixed row j the 64 lanes of a wave touch 64
//   consecutive f32 -- one 256-byte transaction per instruction.
//   Blocks are dealt to the 8 XCDs round-robin; the block -> item map gives
//   each XCD a contiguous item range, so the workgroups that read one key
//   row (two value heads, two column blocks) share an L2.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <tuple>
#include <utility>

#include <type_traits>

#include "gdn_step.h"
#include "gdn_window_common.h"

namespace gdn {
// ------------------------------------------------------------- records
struct RecLayout {
  size_t k, u, scale, total;
};

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static RecLayout rec_layout(const gdn_dims& d) {
  RecLayout r;
  const size_t ntok = (size_t)d.n_layers * d.n_lanes * d.t_max;
  r.k = 0;
  r.u = align256(ntok * d.h_k * d.d_k * sizeof(float));
  r.scale = r.u + align256(ntok * d.h_v * d.d_v * sizeof(float));
  r.total = r.scale + align256(ntok * d.h_v * sizeof(float2));
  return r;
}

// ------------------------------------------------------------- verify
// Per-token scalars of one window, computed once in the prologue and shared
// through LDS:
//   f1 = c_t * rk_t           (prediction:  p = f1 * P)
//   f2 = rk_t / c_t           (record:      ut = beta (v - p) * f2)
//   f3 = scale * rq_t * c_t   (output:      o = f3 * (sum_j St_ij q_j
//                                                     + ut * (k_t . q_t)),
//                              St before the write: S_t q = c_t (St + ut k^T) q)
//   phi = c_{t-1} * alpha_t when the scale is folded into St at token t
//         (then c_t = 1), else 1 (a fold factor is never 1: a fold happens
//         only when the product leaves [2^-32, 2^32]; alpha = 0 folds by 0)
// c_t (the scale after token t) and phi are recorded for commit, which
// replays them instead of recomputing the scale sequence.
struct StepScalars {
  float f1, f2, f3, phi;
  float beta, c, kq, pad;  // kq = k_t . q_t (raw rows)
};

// Replay of m recorded tokens on the held state (the commit of the
// ReplaySSM section): the same fold, write and materialisation as
// commit_kernel, in the same order, on the same values.  Returns the scale
// of the state after the last replayed token.
// node_of(t) is the record index of the t-th replayed step (t itself for a
// window, the t-th node of the accepted path for a draft tree).
template <int R, typename NodeOf>
__device__ __forceinline__ float replay(float (&s)[R], const float* __restrict__ k0,
                                        const float* __restrict__ u0,
                                        const float2* __restrict__ c0, int m,
                                        int j0, int ic, size_t kq_step,
                                        size_t vo_step, int Hv, NodeOf node_of) {
  // the records of step t+1 are requested before step t is applied
  const int n0 = node_of(0);
  float2 fc = c0[n0 * Hv];
  float ut = u0[n0 * vo_step + (uint32_t)ic];
  RowWords<float, R> kw;
  kw.load(k0 + n0 * kq_step, j0);
  float c = 1.0f;
  for (int t = 0; t < m; ++t) {
    const int nt = node_of(t + 1 < m ? t + 1 : t);
    const float2 fc_n = c0[nt * Hv];
    const float ut_n = u0[nt * vo_step + (uint32_t)ic];
    RowWords<float, R> kw_n;
    kw_n.load(k0 + nt * kq_step, j0);
    if (fc.x != 1.f) fold_scale<R>(s, fc.x);
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = state_update(s[r], ut, kw.at(r));
    c = fc.y;
    fc = fc_n;
    ut = ut_n;
    kw = kw_n;
  }
  return c;
}

// Records of up to kTok tokens staged in LDS for the fused replay.
template <int DK>
struct ReplayStage {
  static constexpr int kTok = 16;
  float k[kTok][DK];     // raw key rows (this workgroup's key head)
  float u[kTok][kWave];  // ut of this workgroup's 64 columns
  float2 sc[kTok];       // (phi, c)
};

// The replay of the fused commit + verify.  The whole workgroup first loads
// the records of up to kTok tokens into LDS (one wait for all of them), then
// every wave applies them to its rows with the same operations, in the same
// order and on the same values as replay(), so the result is bitwise the
// same as gdn_commit's.  pk, pu, pc point at token 0 of this lane-layer
// (key head, value head); all loads are clamped to valid tokens and columns.
template <int DK, int R>
__device__ __forceinline__ float replay_staged(
    float (&s)[R], ReplayStage<DK>& st, const float* __restrict__ pk,
    const float* __restrict__ pu, const float2* __restrict__ pc, int m,
    int j0, int x, int cb, int dv, size_t kq_step, size_t vo_step, int Hv) {
  constexpr int kTok = ReplayStage<DK>::kTok;
  constexpr int kK4 = kTok * DK / 4;  // float4 slots of the key rows
  const int tid = (int)threadIdx.x;
  float c = 1.0f;
  for (int t0 = 0; t0 < m; t0 += kTok) {
    const int nb = m - t0 < kTok ? m - t0 : kTok;
    float4 kreg[(kK4 + kBlock - 1) / kBlock];
    float ureg[kTok * kWave / kBlock];
#pragma unroll
    for (int rep = 0; rep < (kK4 + kBlock - 1) / kBlock; ++rep) {
      const int e = tid + rep * kBlock;
      int tok = e / (DK / 4);
      tok = tok < nb ? tok : nb - 1;
      kreg[rep] = reinterpret_cast<const float4*>(
          pk + (t0 + tok) * kq_step)[e % (DK / 4)];
    }
#pragma unroll
    for (int rep = 0; rep < kTok * kWave / kBlock; ++rep) {
      const int e = tid + rep * kBlock;
      int tok = e / kWave;
      tok = tok < nb ? tok : nb - 1;
      int col = cb * kWave + e % kWave;
      col = col < dv ? col : dv - 1;
      ureg[rep] = pu[(t0 + tok) * vo_step + (uint32_t)col];
    }
    const float2 sreg = pc[(size_t)(t0 + (tid < nb ? tid : nb - 1)) * Hv];
#pragma unroll
    for (int rep = 0; rep < (kK4 + kBlock - 1) / kBlock; ++rep) {
      const int e = tid + rep * kBlock;
      if (e < kK4) reinterpret_cast<float4*>(&st.k[0][0])[e] = kreg[rep];
    }
#pragma unroll
    for (int rep = 0; rep < kTok * kWave / kBlock; ++rep)
      (&st.u[0][0])[tid + rep * kBlock] = ureg[rep];
    if (tid < kTok) st.sc[tid] = sreg;
    __syncthreads();
    for (int t = 0; t < nb; ++t) {
      const float2 fc = st.sc[t];
      const float phi = __int_as_float(
          __builtin_amdgcn_readfirstlane(__float_as_int(fc.x)));
      if (phi != 1.f) fold_scale<R>(s, phi);
      const float ut = st.u[t][x];
      const float4* kr = reinterpret_cast<const float4*>(&st.k[t][j0]);
#pragma unroll
      for (int r4 = 0; r4 < R / 4; ++r4) {
        const float4 kk = kr[r4];
        s[4 * r4 + 0] = state_update(s[4 * r4 + 0], ut, kk.x);
        s[4 * r4 + 1] = state_update(s[4 * r4 + 1], ut, kk.y);
        s[4 * r4 + 2] = state_update(s[4 * r4 + 2], ut, kk.z);
        s[4 * r4 + 3] = state_update(s[4 * r4 + 3], ut, kk.w);
      }
      c = fc.y;
    }
    __syncthreads();  // the next batch overwrites the stage
  }
  return c;
}

// REPLAY = false: gdn_verify (S is only read).  REPLAY = true: the fused
// gdn_commit_verify -- replay the previous window's accepted prefix from S,
// store the committed state S_m in place, then verify the new window from
// the state still held in registers (the committed values, bit for bit).
// TREE: a draft-tree window.  Node t steps from the state of its parent
// tree.v[lane * T + t] (S0 for kNoParent).  Nodes come in an order where a
// parent precedes its children; when node t's parent is not node t-1, every
// wave rebuilds the parent's state: S0 again, then the recorded steps of the
// root-to-parent path (fold, ut from LDS, the raw key row) -- exactly the
// operations a commit of that path performs, so the state at every node is
// bitwise what gdn_commit_path reproduces.
// Six waves per SIMD (at most 80 VGPRs) for windows; draft trees at d_k of
// 64 and 128 keep a second copy of the held state while they rebuild a
// parent's state, and spill at 80 VGPRs (a 32-node tree verify took 3.36 ms
// with 104 spilled VGPRs, 1.79 ms with none), so they get more registers,
// and so do the variants that write every intermediate state at d_k = 128
// (36 spilled VGPRs at 80).
template <int DK, bool DBG, typename TIn, bool REPLAY, bool TREE>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(
    TREE ? (DK == 128 ? 2 : DK == 64 ? 4 : 6) : (DBG && DK == 128 ? 4 : 6))))
void verify_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ g, float* S,
    float* __restrict__ o, float* __restrict__ rec_k,
    float* __restrict__ rec_u, float2* __restrict__ rec_scale,
    float* __restrict__ dbg, WinDims d, LaneTable tl, float scale,
    int l2norm, PrevRecords prev,
    std::conditional_t<TREE, TreeTable, NoTable> tree) {
  constexpr int R = DK / kWaves;  // key rows per wave
  __shared__ float nrm[3][GDN_MAX_T];  // rk_t, rq_t, k_t . q_t (raw)
  __shared__ StepScalars sc[GDN_MAX_T];
  // draft trees: ut of every node (this workgroup's columns) and the
  // root-to-node path of every node
  __shared__ float uth[TREE ? kTreeMaxT : 1][kWave];
  __shared__ uint8_t plist[TREE ? kTreeMaxT * (kTreeMaxT + 1) / 2 : 1];
  __shared__ uint16_t pstart[TREE ? kTreeMaxT : 1];

  int item = xcd_item(blockIdx.x, gridDim.x);
  const int cb = item % d.ncb;
  item /= d.ncb;
  const int h = item % d.Hv;
  item /= d.Hv;
  const int lane = item % d.N;
  const int layer = item / d.N;
  const int T = tl.v[lane];
  const int m_prev = REPLAY ? prev.m.v[lane] : 0;
  if (T == 0 && m_prev == 0) return;
  // parent of node t (t - 1 in a plain window; -1: steps from S0)
  auto parent_of = [&](int t) -> int {
    if constexpr (TREE) {
      const int p = tree.v[lane * d.T + t];
      return p == kNoParent ? -1 : p;
    } else {
      return t - 1;
    }
  };

  const int w = uniform((int)threadIdx.x / kWave);
  const int x = (int)threadIdx.x % kWave;
  const int j0 = w * R;
  const int i = cb * kWave + x;
  const bool act = i < d.dv;
  const int ic = act ? i : d.dv - 1;
  const int kh = h / d.group;
  const bool key_writer = (h % d.group == 0) && cb == 0;
  const size_t ll = (size_t)layer * d.N + lane;
  const size_t dv = (size_t)d.dv;
  // uniform row bases (token 0 of this lane-layer); per-lane offsets are
  // 32-bit column indices, so addresses are scalar base + lane offset
  const size_t kq_step = (size_t)d.Hk * DK;            // per token, q/k
  const size_t vo_step = (size_t)d.Hv * dv;            // per token, v/o/u
  const TIn* __restrict__ k0 = k + ((ll * d.T) * d.Hk + kh) * (size_t)DK;
  const TIn* __restrict__ q0 = q + ((ll * d.T) * d.Hk + kh) * (size_t)DK;
  const TIn* __restrict__ v0 = v + ((ll * d.T) * d.Hv + h) * dv;
  float* __restrict__ o0 = o + ((ll * d.T) * d.Hv + h) * dv;
  float* __restrict__ u0 = rec_u + ((ll * d.T) * d.Hv + h) * dv;

  float s[R];  // scaled state St (rows j0..j0+R-1, column i); S = c * St
  float* const Sh = S + ((ll * d.Hv + h) * (size_t)DK + j0) * dv;
  {
#pragma unroll
    for (int r = 0; r < R; ++r)
      s[r] = __builtin_nontemporal_load(Sh + (uint32_t)(r * d.dv + ic));
    if constexpr (REPLAY) {
      if (m_prev > 0) {
        __shared__ ReplayStage<DK> stage;
        const float c = replay_staged<DK, R>(
            s, stage, prev.k + ((ll * d.T) * d.Hk + kh) * (size_t)DK,
            prev.u + ((ll * d.T) * d.Hv + h) * dv,
            prev.scale + (ll * d.T) * d.Hv + h, m_prev, j0, x, cb, d.dv,
            kq_step, vo_step, d.Hv);
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = materialise(c, s[r]);
        if (act) {
#pragma unroll
          for (int r = 0; r < R; ++r)
            __builtin_nontemporal_store(s[r], Sh + (uint32_t)(r * d.dv + i));
        }
      }
    }
  }
  if (REPLAY && T == 0) return;

  // ---- prologue 1: per token (16 lanes each, 4 tokens per wave pass):
  // |k_t|^2, |q_t|^2 and k_t.q_t over the whole row; the key record rows
  for (int base = 4 * w; base < T; base += 16) {  // base is wave-uniform
    const int t = base + x / 16;
    const int tt = t < T ? t : T - 1;
    const int sub = x % 16;
    float kk[8], skk, sqq, skq;
    row_moments<TIn>(k0 + tt * kq_step, q0 + tt * kq_step, DK, sub, kk, skk,
                     sqq, skq);
    if (t < T) {
      if (sub == 0) {
        nrm[0][t] = l2norm ? inv_norm(skk) : 1.0f;
        nrm[1][t] = l2norm ? inv_norm(sqq) : 1.0f;
        nrm[2][t] = skq;
      }
      if (key_writer && 8 * sub < DK) {
        float4* dst = reinterpret_cast<float4*>(
            rec_k + ((ll * d.T + t) * d.Hk + kh) * (size_t)DK + 8 * sub);
        dst[0] = make_float4(kk[0], kk[1], kk[2], kk[3]);
        dst[1] = make_float4(kk[4], kk[5], kk[6], kk[7]);
      }
    }
  }
  __syncthreads();
  // ---- prologue 2 (one wave, chosen per workgroup to spread the work over
  // the SIMDs): lane t holds token t's gates; the scales c_t are an
  // inclusive prefix product of alpha over the lanes.  If a prefix leaves
  // [2^-32, 2^32] the scale is folded; that rare case walks the tokens in
  // order in one lane instead.
  if (w == (int)(blockIdx.x & 3)) {
    const int tt = x < T ? x : T - 1;
    const size_t gi = (ll * d.T + tt) * d.Hv + h;
    const float a_t = x < T ? __expf(g[gi]) : 1.0f;
    const float b_t = beta[gi];
    float c = a_t;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float y = __shfl_up(c, off, kWave);
      if (x >= off) c *= y;
    }
    const bool out = !(c >= kScaleLo && c <= kScaleHi);
    float phi = 1.f;
    if (TREE || __builtin_amdgcn_ballot_w64(out && x < T) != 0) {
      // sequential walk with folds (lane 0), results spread back by lane;
      // in a tree each node continues its parent's scale
      __shared__ float seq_c[GDN_MAX_T], seq_f[GDN_MAX_T], seq_a[GDN_MAX_T];
      if (x < T) seq_a[x] = a_t;
      __builtin_amdgcn_wave_barrier();
      if (x == 0) {
        [[maybe_unused]] int used = 0;
        for (int t = 0; t < T; ++t) {
          const int par = parent_of(t);
          const float cc = par < 0 ? 1.0f : seq_c[par];
          float cn, fo = 1.f;
          if (scale_step(cc, seq_a[t], cn)) {
            fo = cn;
            cn = 1.0f;
          }
          seq_c[t] = cn;
          seq_f[t] = fo;
          if constexpr (TREE) {  // root-to-node path of node t
            pstart[t] = (uint16_t)used;
            if (par >= 0) {
              // copy the parent's path (it ends with par), then append t
              int j = pstart[par];
              while (true) {
                const int u = plist[j++];
                plist[used++] = (uint8_t)u;
                if (u == par) break;
              }
            }
            plist[used++] = (uint8_t)t;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (x < T) {
        c = seq_c[x];
        phi = seq_f[x];
      }
    }
    if (x < T) {
      const float rk = nrm[0][x], rq = nrm[1][x];
      StepScalars z;
      z.f1 = c * rk;
      z.f2 = rk * __builtin_amdgcn_rcpf(c);
      z.f3 = scale * rq * c;
      z.phi = phi;
      z.beta = b_t;
      z.c = c;
      z.kq = nrm[2][x];
      z.pad = 0.f;
      sc[x] = z;
      if (cb == 0) rec_scale[gi] = make_float2(phi, c);
    }
  }
  __syncthreads();

  // ---- the window: one LDS exchange per token.  One pass over the state
  // forms the partials of St k (prediction) and St q (output, from the state
  // before the write); after the exchange a second pass applies the write.
  __shared__ float2 red[2][kWaves][kWave];
  RowWords<TIn, R> kw, qw;
  kw.load(k0, j0);
  qw.load(q0, j0);
  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    if constexpr (TREE) {
      const int par = parent_of(t);
      if (t > 0 && par != t - 1) {
        // rebuild the parent's state from S0 and its recorded path
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = Sh[(uint32_t)(r * d.dv + ic)];
        if (par >= 0) {
          for (int j = pstart[par];; ++j) {
            const int u = uniform(plist[j]);
            const float phu = sc[u].phi;
            if (phu != 1.f) fold_scale<R>(s, phu);
            const float utu = uth[u][x];
            RowWords<TIn, R> ku;
            ku.load(k0 + u * kq_step, j0);
#pragma unroll
            for (int r = 0; r < R; ++r) s[r] = state_update(s[r], utu, ku.at(r));
            if (u == par) break;
          }
        }
      }
    }
    const float vi = load_in(v0 + t * vo_step, (uint32_t)ic);
    const StepScalars z = sc[t];
    if (z.phi != 1.f) fold_scale<R>(s, z.phi);

    float kv[R];
    float a0 = 0.f, b0 = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kv[r] = kw.at(r);
      a0 = __builtin_fmaf(s[r], kv[r], a0);
      b0 = __builtin_fmaf(s[r], qw.at(r), b0);
    }
    red[buf][w][x] = make_float2(a0, b0);
    __syncthreads();
    const float2 r0 = red[buf][0][x], r1 = red[buf][1][x];
    const float2 r2 = red[buf][2][x], r3 = red[buf][3][x];
    // key and query rows of the next token: requested after the partials
    // are read (scalar and LDS loads share one wait counter), in flight
    // during the write pass
    if (t + 1 < T) {
      kw.load(k0 + (t + 1) * kq_step, j0);
      qw.load(q0 + (t + 1) * kq_step, j0);
    }
    const float P = (r0.x + r1.x) + (r2.x + r3.x);
    const float PQ = (r0.y + r1.y) + (r2.y + r3.y);
    const float p = z.f1 * P;
    const float ut = (z.beta * (vi - p)) * z.f2;
    const int owner = t % kWaves;  // wave that writes this token's outputs
    if (w == owner && act) {
      u0[t * vo_step + (uint32_t)i] = ut;
      __builtin_nontemporal_store(z.f3 * __builtin_fmaf(ut, z.kq, PQ),
                                  o0 + t * vo_step + (uint32_t)i);
    }
    if constexpr (TREE) {
      if (w == owner) uth[t][x] = ut;  // read back after a later barrier
    }

    // rank-1 write
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = state_update(s[r], ut, kv[r]);
    if (DBG && act) {
      float* __restrict__ dp =
          dbg + (((ll * d.T + t) * d.Hv + h) * (size_t)DK + j0) * dv;
#pragma unroll
      for (int r = 0; r < R; ++r)
        dp[(uint32_t)(r * d.dv + i)] = materialise(z.c, s[r]);
    }
  }
}

// ------------------------------------------------------------- commit
// PATH: the replayed steps are the accepted nodes path.v[a * T + t] of a
// draft tree (a: the lane's index among the active lanes), not 0..m-1.
template <int DK, bool PATH>
__global__ __launch_bounds__(kBlock) void commit_kernel(
    const float* __restrict__ rec_k, const float* __restrict__ rec_u,
    const float2* __restrict__ rec_scale, float* __restrict__ S, WinDims d,
    CommitTable ct, std::conditional_t<PATH, TreeTable, NoTable> path) {
  constexpr int R = DK / kWaves;
  int item = xcd_item(blockIdx.x, gridDim.x);
  const int cb = item % d.ncb;
  item /= d.ncb;
  const int h = item % d.Hv;
  item /= d.Hv;
  const int a = item % ct.n_act;  // items: (layer, active lane, head, cb)
  const int layer = item / ct.n_act;
  const int lane = ct.lane[a];
  const int m = ct.m[a];

  const int w = uniform((int)threadIdx.x / kWave);
  const int x = (int)threadIdx.x % kWave;
  const int j0 = w * R;
  const int i = cb * kWave + x;
  const bool act = i < d.dv;
  const int ic = act ? i : d.dv - 1;
  const int kh = h / d.group;
  const size_t ll = (size_t)layer * d.N + lane;
  const size_t dv = (size_t)d.dv;
  float* __restrict__ Sh = S + ((ll * d.Hv + h) * (size_t)DK + j0) * dv;
  const float* __restrict__ k0 = rec_k + ((ll * d.T) * d.Hk + kh) * (size_t)DK;
  const float* __restrict__ u0 = rec_u + ((ll * d.T) * d.Hv + h) * dv;
  const float2* __restrict__ c0 = rec_scale + (ll * d.T) * d.Hv + h;
  const size_t kq_step = (size_t)d.Hk * DK, vo_step = (size_t)d.Hv * dv;

  float s[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    s[r] = __builtin_nontemporal_load(Sh + (uint32_t)(r * d.dv + ic));
  const float c = replay<R>(s, k0, u0, c0, m, j0, ic, kq_step, vo_step, d.Hv,
                            [&](int t) -> int {
                              if constexpr (PATH) return path.v[a * d.T + t];
                              else return t;
                            });
  if (act) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      __builtin_nontemporal_store(materialise(c, s[r]),
                                  Sh + (uint32_t)(r * d.dv + i));
  }
}

// ------------------------------------------------------------- host side
static thread_local char g_last_error[256] = "";

void set_error(const char* msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
}

template <int DK, bool DBG, typename TIn, bool REPLAY, bool TREE, typename Tab>
static hipError_t launch_verify_t(const WinDims& w, const LaneTable& tl,
                                  const VerifyArgs& a, const PrevRecords& pr,
                                  const Tab& tree, hipStream_t st) {
  const int blocks = w.NL * w.N * w.Hv * w.ncb;
  return launch(verify_kernel<DK, DBG, TIn, REPLAY, TREE>, dim3(blocks),
                dim3(kBlock), st, (const TIn*)a.q, (const TIn*)a.k,
                (const TIn*)a.v, a.beta, a.g, a.S, a.o, a.rk, a.ru, a.ra,
                a.dbg, w, tl, a.scale, a.l2, pr, tree);
}

template <bool DBG, typename TIn, bool REPLAY, bool TREE, typename Tab>
static hipError_t launch_verify_d(const WinDims& w, const LaneTable& tl,
                                  const VerifyArgs& a, const PrevRecords& pr,
                                  const Tab& tree, hipStream_t st) {
  switch (w.dk) {
    case 16: return launch_verify_t<16, DBG, TIn, REPLAY, TREE>(w, tl, a, pr, tree, st);
    case 32: return launch_verify_t<32, DBG, TIn, REPLAY, TREE>(w, tl, a, pr, tree, st);
    case 64: return launch_verify_t<64, DBG, TIn, REPLAY, TREE>(w, tl, a, pr, tree, st);
    default: return launch_verify_t<128, DBG, TIn, REPLAY, TREE>(w, tl, a, pr, tree, st);
  }
}

template <bool REPLAY, bool TREE = false, typename Tab = NoTable>
static hipError_t launch_verify(const WinDims& w, const LaneTable& tl,
                                int in_dtype, const VerifyArgs& a,
                                const PrevRecords& pr, hipStream_t st,
                                const Tab& tree = Tab()) {
  if (in_dtype == GDN_BF16)
    return a.dbg ? launch_verify_d<true, uint16_t, REPLAY, TREE>(w, tl, a, pr, tree, st)
                 : launch_verify_d<false, uint16_t, REPLAY, TREE>(w, tl, a, pr, tree, st);
  return a.dbg ? launch_verify_d<true, float, REPLAY, TREE>(w, tl, a, pr, tree, st)
               : launch_verify_d<false, float, REPLAY, TREE>(w, tl, a, pr, tree, st);
}

// Checks shared by gdn_verify and gdn_commit_verify; fills the lane table
// and the kernel arguments.  *any = 0 when every t_lane is 0.
static int verify_setup(const char* fn, const gdn_dims* dims,
                        const int32_t* t_lane, const void* q, const void* k,
                        const void* v, int in_dtype, const float* beta,
                        const float* g, const float* S, float* o,
                        void* records, float* dbg_states, float scale,
                        int flags, LaneTable& tl, VerifyArgs& a, int* any) {
  char msg[128];
  int rc = check_dims(dims);
  if (rc != GDN_OK) return rc;
  if (!t_lane || !q || !k || !v || !beta || !g || !S || !o || !records) {
    snprintf(msg, sizeof(msg), "%s: required pointer is NULL", fn);
    return fail(GDN_EINVAL, msg);
  }
  if (in_dtype != GDN_BF16 && in_dtype != GDN_F32) {
    snprintf(msg, sizeof(msg), "%s: unknown in_dtype", fn);
    return fail(GDN_EINVAL, msg);
  }
  if (flags & ~(GDN_FLAG_L2NORM_QK | GDN_FLAG_TOKENWISE)) {
    snprintf(msg, sizeof(msg), "%s: unknown flag bits", fn);
    return fail(GDN_EINVAL, msg);
  }
  // q/k rows are read as dwords (bf16 pairs) or f32
  if (misaligned(q, 4) || misaligned(k, 4) ||
      misaligned(v, in_dtype == GDN_BF16 ? 2 : 4) || misaligned(beta, 4) ||
      misaligned(g, 4) || misaligned(S, 4) || misaligned(o, 4) ||
      misaligned(records, 256) || (dbg_states && misaligned(dbg_states, 4))) {
    snprintf(msg, sizeof(msg), "%s: misaligned pointer", fn);
    return fail(GDN_EINVAL, msg);
  }
  const gdn_dims& d = *dims;
  memset(&tl, 0, sizeof(tl));
  *any = 0;
  for (int n = 0; n < d.n_lanes; ++n) {
    if (t_lane[n] < 0 || t_lane[n] > d.t_max) {
      snprintf(msg, sizeof(msg), "%s: t_lane out of 0..t_max", fn);
      return fail(GDN_EINVAL, msg);
    }
    tl.v[n] = (uint8_t)t_lane[n];
    *any |= t_lane[n];
  }
  const RecLayout L = rec_layout(d);
  char* rb = (char*)records;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.S = const_cast<float*>(S);
  a.o = o;
  a.rk = (float*)(rb + L.k);
  a.ru = (float*)(rb + L.u);
  a.ra = (float2*)(rb + L.scale);
  a.dbg = dbg_states;
  a.scale = scale;
  a.l2 = (flags & GDN_FLAG_L2NORM_QK) ? 1 : 0;
  a.f32 = in_dtype == GDN_F32 ? 1 : 0;
  return GDN_OK;
}

}  // namespace gdn

using namespace gdn;

extern "C" size_t gdn_records_bytes(const gdn_dims* dims) {
  if (check_dims(dims) != GDN_OK) return 0;
  return rec_layout(*dims).total;
}

extern "C" int gdn_verify(const gdn_dims* dims, const int32_t* t_lane,
                          const void* q, const void* k, const void* v,
                          int in_dtype, const float* beta, const float* g,
                          const float* S, float* o, void* records,
                          float* dbg_states, float scale, int flags,
                          void* stream) {
  LaneTable tl;
  VerifyArgs a;
  int any = 0;
  int rc = verify_setup("gdn_verify", dims, t_lane, q, k, v, in_dtype, beta, g,
                        S, o, records, dbg_states, scale, flags, tl, a, &any);
  if (rc != GDN_OK) return rc;
  if (!any) return GDN_OK;
  PrevRecords none;
  memset(&none, 0, sizeof(none));
  hipError_t e =
      !(flags & GDN_FLAG_TOKENWISE) && mverify_eligible(*dims, in_dtype, a, false)
          ? launch_mverify(win_dims(*dims), tl, a, none, false,
                           (hipStream_t)stream)
          : launch_verify<false>(win_dims(*dims), tl, in_dtype, a, none,
                                 (hipStream_t)stream);
  return hip_status(e, "gdn_verify launch");
}

extern "C" int gdn_commit(const gdn_dims* dims, const int32_t* m_lane,
                          const int32_t* t_lane, const void* records,
                          float* S, void* stream) {
  int rc = check_dims(dims);
  if (rc != GDN_OK) return rc;
  if (!m_lane || !t_lane || !records || !S)
    return fail(GDN_EINVAL, "gdn_commit: required pointer is NULL");
  if (misaligned(records, 256) || misaligned(S, 4))
    return fail(GDN_EINVAL, "gdn_commit: misaligned pointer");
  const gdn_dims& d = *dims;
  CommitTable ct;
  rc = commit_lanes("gdn_commit", d, m_lane, t_lane, ct);
  if (rc != GDN_OK) return rc;
  if (ct.n_act == 0) return GDN_OK;
  const WinDims w = win_dims(d);
  const RecLayout L = rec_layout(d);
  const char* rb = (const char*)records;
  const float* rk = (const float*)(rb + L.k);
  const float* ru = (const float*)(rb + L.u);
  const float2* ra = (const float2*)(rb + L.scale);
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(d.n_layers * ct.n_act * d.h_v * w.ncb);
  hipError_t e;
  const NoTable none{};
  switch (d.d_k) {
    case 16: e = launch(commit_kernel<16, false>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct, none); break;
    case 32: e = launch(commit_kernel<32, false>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct, none); break;
    case 64: e = launch(commit_kernel<64, false>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct, none); break;
    default: e = launch(commit_kernel<128, false>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct, none); break;
  }
  return hip_status(e, "gdn_commit launch");
}

// Host checks of a draft-tree window: sizes that fit the kernel-argument
// table, and parent[t] in -1..t-1 for every node of every lane.
static int tree_table(const char* fn, const gdn_dims& d, const int32_t* t_lane,
                      const int32_t* parent, TreeTable& tab) {
  char msg[128];
  if (d.t_max > kTreeMaxT || d.n_lanes * d.t_max > kTreeCells) {
    snprintf(msg, sizeof(msg), "%s: tree windows need t_max <= %d and "
             "n_lanes * t_max <= %d", fn, kTreeMaxT, kTreeCells);
    return fail(GDN_EUNSUPPORTED, msg);
  }
  if (!parent) {
    snprintf(msg, sizeof(msg), "%s: parent is NULL", fn);
    return fail(GDN_EINVAL, msg);
  }
  memset(&tab, kNoParent, sizeof(tab));
  for (int n = 0; n < d.n_lanes; ++n) {
    const int T = t_lane[n] < 0 ? 0 : t_lane[n];
    for (int t = 0; t < T && t < d.t_max; ++t) {
      const int p = parent[n * d.t_max + t];
      if (p < -1 || p >= t) {
        snprintf(msg, sizeof(msg), "%s: parent[%d][%d] = %d is not in -1..%d",
                 fn, n, t, p, t - 1);
        return fail(GDN_EINVAL, msg);
      }
      tab.v[n * d.t_max + t] = p < 0 ? kNoParent : (uint8_t)p;
    }
  }
  return GDN_OK;
}

extern "C" int gdn_verify_tree(const gdn_dims* dims, const int32_t* t_lane,
                               const int32_t* parent, const void* q,
                               const void* k, const void* v, int in_dtype,
                               const float* beta, const float* g,
                               const float* S, float* o, void* records,
                               float* dbg_states, float scale, int flags,
                               void* stream) {
  LaneTable tl;
  VerifyArgs a;
  int any = 0;
  int rc = verify_setup("gdn_verify_tree", dims, t_lane, q, k, v, in_dtype,
                        beta, g, S, o, records, dbg_states, scale, flags, tl,
                        a, &any);
  if (rc != GDN_OK) return rc;
  TreeTable tab;
  rc = tree_table("gdn_verify_tree", *dims, t_lane, parent, tab);
  if (rc != GDN_OK) return rc;
  if (!any) return GDN_OK;
  PrevRecords none;
  memset(&none, 0, sizeof(none));
  hipError_t e =
      !(flags & GDN_FLAG_TOKENWISE) && mverify_eligible(*dims, in_dtype, a, true)
          ? launch_mverify_tree(win_dims(*dims), tl, a, tab,
                                (hipStream_t)stream)
          : launch_verify<false, true>(win_dims(*dims), tl, in_dtype, a, none,
                                       (hipStream_t)stream, tab);
  return hip_status(e, "gdn_verify_tree launch");
}

extern "C" int gdn_commit_path(const gdn_dims* dims, const int32_t* m_lane,
                               const int32_t* path, const int32_t* t_lane,
                               const int32_t* parent, const void* records,
                               float* S, void* stream) {
  int rc = check_dims(dims);
  if (rc != GDN_OK) return rc;
  if (!m_lane || !path || !t_lane || !records || !S)
    return fail(GDN_EINVAL, "gdn_commit_path: required pointer is NULL");
  if (misaligned(records, 256) || misaligned(S, 4))
    return fail(GDN_EINVAL, "gdn_commit_path: misaligned pointer");
  const gdn_dims& d = *dims;
  TreeTable parents;
  rc = tree_table("gdn_commit_path", d, t_lane, parent, parents);
  if (rc != GDN_OK) return rc;
  CommitTable ct;
  rc = commit_lanes("gdn_commit_path", d, m_lane, t_lane, ct);
  if (rc != GDN_OK) return rc;
  // the accepted nodes of each active lane must be a root-to-node path
  TreeTable nodes;
  memset(&nodes, 0, sizeof(nodes));
  for (int a_i = 0; a_i < ct.n_act; ++a_i) {
    const int n = ct.lane[a_i], m = ct.m[a_i];
    int prev = -1;
    for (int j = 0; j < m; ++j) {
      const int node = path[n * d.t_max + j];
      const int par = (node >= 0 && node < t_lane[n])
                          ? (parents.v[n * d.t_max + node] == kNoParent
                                 ? -1
                                 : parents.v[n * d.t_max + node])
                          : -2;
      if (par == -2 || par != prev)
        return fail(GDN_EINVAL,
                    "gdn_commit_path: path is not a root-to-node path of the tree");
      nodes.v[a_i * d.t_max + j] = (uint8_t)node;
      prev = node;
    }
  }
  if (ct.n_act == 0) return GDN_OK;
  const WinDims w = win_dims(d);
  const RecLayout L = rec_layout(d);
  const char* rb = (const char*)records;
  const float* rk = (const float*)(rb + L.k);
  const float* ru = (const float*)(rb + L.u);
  const float2* ra = (const float2*)(rb + L.scale);
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(d.n_layers * ct.n_act * d.h_v * w.ncb);
  hipError_t e;
  switch (d.d_k) {
    case 16: e = launch(commit_kernel<16, true>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct, nodes); break;
    case 32: e = launch(commit_kernel<32, true>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct, nodes); break;
    case 64: e = launch(commit_kernel<64, true>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct, nodes); break;
    default: e = launch(commit_kernel<128, true>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct, nodes); break;
  }
  return hip_status(e, "gdn_commit_path launch");
}

extern "C" int gdn_commit_verify(const gdn_dims* dims, const int32_t* m_prev,
                                 const int32_t* t_prev,
                                 const void* records_prev,
                                 const int32_t* t_lane, const void* q,
                                 const void* k, const void* v, int in_dtype,
                                 const float* beta, const float* g, float* S,
                                 float* o, void* records, float* dbg_states,
                                 float scale, int flags, void* stream) {
  LaneTable tl;
  VerifyArgs a;
  int any = 0;
  int rc = verify_setup("gdn_commit_verify", dims, t_lane, q, k, v, in_dtype,
                        beta, g, S, o, records, dbg_states, scale, flags, tl,
                        a, &any);
  if (rc != GDN_OK) return rc;
  if (!m_prev || !t_prev)
    return fail(GDN_EINVAL, "gdn_commit_verify: required pointer is NULL");
  const gdn_dims& d = *dims;
  CommitTable ct;
  rc = commit_lanes("gdn_commit_verify", d, m_prev, t_prev, ct);
  if (rc != GDN_OK) return rc;
  PrevRecords pr;
  memset(&pr, 0, sizeof(pr));
  if (ct.n_act > 0) {
    if (!records_prev)
      return fail(GDN_EINVAL, "gdn_commit_verify: records_prev is NULL");
    if (misaligned(records_prev, 256))
      return fail(GDN_EINVAL, "gdn_commit_verify: misaligned pointer");
    const RecLayout L = rec_layout(d);
    const char* p0 = (const char*)records_prev;
    const char* p1 = (const char*)records;
    if (p0 < p1 + L.total && p1 < p0 + L.total)
      return fail(GDN_EINVAL,
                  "gdn_commit_verify: records and records_prev overlap");
    pr.k = (const float*)(p0 + L.k);
    pr.u = (const float*)(p0 + L.u);
    pr.scale = (const float2*)(p0 + L.scale);
    for (int n = 0; n < d.n_lanes; ++n) pr.m.v[n] = (uint8_t)m_prev[n];
  }
  // Workgroups of one launch differ in cost by lane: a lane with m_prev > 0
  // also writes its committed state and replays m_prev records.  The
  // matrix-core kernel takes the lanes in decreasing order of that cost
  // within each XCD's share of the work, so that the cheap workgroups fill
  // the end of the launch (longest processing time first).
  {
    int ord[GDN_MAX_LANES];
    auto cost = [&](int n) {
      const int m = ct.n_act > 0 ? (int)pr.m.v[n] : 0;
      return (m > 0 ? 1024 : 0) + 32 * m + t_lane[n];
    };
    for (int i = 0; i < d.n_lanes; ++i) {  // stable insertion sort
      int j = i;
      for (; j > 0 && cost(ord[j - 1]) < cost(i); --j) ord[j] = ord[j - 1];
      ord[j] = i;
    }
    for (int n = 0; n < d.n_lanes; ++n) pr.order.v[n] = (uint8_t)ord[n];
  }
  if (!any && ct.n_act == 0) return GDN_OK;
  hipError_t e = !(flags & GDN_FLAG_TOKENWISE) &&
                          mverify_eligible(d, in_dtype, a, false)
                      ? launch_mverify(win_dims(d), tl, a, pr, true,
                                       (hipStream_t)stream)
                      : launch_verify<true>(win_dims(d), tl, in_dtype, a, pr,
                                            (hipStream_t)stream);
  return hip_status(e, "gdn_commit_verify launch");
}

extern "C" const char* gdn_strerror(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument";
    case GDN_EUNSUPPORTED: return "unsupported configuration";
    case GDN_EWORKSPACE: return "workspace too small";
    case GDN_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* gdn_last_error(void) { return g_last_error; }
