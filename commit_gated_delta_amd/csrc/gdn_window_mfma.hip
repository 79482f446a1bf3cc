// gdn_window_mfma.hip -- speculative-window verify, draft-tree verify and
// the fused commit + verify on the gfx950 matrix cores, for d_k = 128 and
// d_v a multiple of 128, bf16 or f32 inputs (f32 key / query rows enter the
// products as three bf16 parts, see Frag): windows of at most 16 tokens (the
// shapes of the speculative-decoding section of the NInfer technical review,
// blog.123qwe.co.kr post 4624) as one block, longer windows (up to 64
// tokens) in blocks of 16, draft trees of up to 32 nodes in blocks of 16.
// Other shapes, and
// calls with GDN_FLAG_TOKENWISE, take gdn_window.hip.
//
// The window is one chunk of the block (WY/UT) form of the rule: Yang et
// al., "Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length" (NeurIPS 2024), Sec. 3, with the per-token decay of Gated DeltaNet
// (ICLR 2025, Sec. 3).  With the window's start state H (d_k x d_v, key-major
// as stored), raw key / query rows k_t, q_t (t = 0..15), their inverse norms
// rk_t, rq_t, and dec(t, s) = exp(g_{s+1} + ... + g_t) the decay from token s
// to token t (A_t = dec(t, -1) the decay since the window start):
//   L_ts = beta_t rk_t rk_s dec(t, s) (k_t . k_s)            s < t
//   T    = (I + L)^-1                                     (unit lower)
//   P_ts = scale rq_t rk_s dec(t, s) (q_t . k_s)             s <= t
//   X_t  = beta_t v_t - beta_t A_t rk_t (K H)_t
//   U    = T X                          (row t: the delta u_t of token t)
//   O_t  = scale rq_t A_t (Q H)_t + (P U)_t      (o_t = scale S_t qhat_t)
// Unrolling the token-by-token rule over the window gives exactly these
// expressions.  The decays come from sums of the gates inside segments
// that end at a gate whose exponential is 0 in f32 (g < -128, g = -inf): a
// decay across such a token is 0, and no difference of two infinite sums
// is ever formed.
//
// Records: the same records as gdn_window.hip -- raw key rows as f32, the
// scale step (phi, c) of every token (the lazy-decay scale sequence of
// gdn_step.h, with its folds) and ut_t = u_t rk_t / c_t -- so gdn_commit
// replays them unchanged.  The state that verify holds after token t is, by
// definition here, the replay of its own first t + 1 records: the debug
// states are produced exactly so (the same fold, fma and materialisation,
// in the same order, on the same values as commit), hence commit(m) is
// bitwise the debug state m - 1.  The outputs come from the chunk form, so
// they agree with the replayed states to rounding, not bit for bit.
//
// Work decomposition: one 256-thread workgroup per (layer, lane, value head,
// block of 128 value columns); wave w owns 32 columns.  Lane l (g4 = l/16,
// n = l%16) holds the state entries of rows 32 ks + 8 g4 + e (ks = 0..3,
// e = 0..7) at its two columns 2n, 2n + 1: for every row the 16 lanes of a
// group read 128 contiguous bytes.  Those eight rows are exactly the lane's
// B operand of v_mfma_f32_16x16x32_bf16 for k-step ks, after a split of
// every f32 entry into bf16 hi + lo (x = hi + lo + ~2^-17 |x|): K H and
// Q H take 32 MFMAs per wave against the exact bf16 key / query rows.
// Every wave also forms the window's 16 x 16 matrices itself (K K^T and
// K Q^T on MFMA, the gates, L, P and T), so the four waves never wait for
// each other; T comes from a right-looking substitution in the wave's own
// LDS tile.  T X and P U run on v_mfma_f32_16x16x4_f32, whose B operand is
// the D layout of the previous product (k-slot g4 of step e is token
// 4 g4 + e).  The small loads (rows, gates) are issued before the 64 KB of
// state, so that everything but the state products overlaps its latency.
//
// The fused call first replays the previous window's accepted prefix on the
// state it loads, with the commit's operations, and stores it; a draft tree
// replaces the causal mask by the ancestor relation (see mverify_kernel).
// MB (windows of more than 16 tokens): block b runs from the held state,
// which then moves on by the block's rank-1 writes summed in one product on
// the matrix cores (St += K^T Ut over the block's records, f32 accurate);
// block b + 1 starts from it, its K H and Q H scaled by the scale of block
// b's last token.  The held state so agrees with the token-by-token replay
// of the records (which commit stores, and which the debug states are)
// to rounding; the sequential replay between blocks cost 0.1 ms per block
// boundary at 8 lanes x 48 layers, the product about a tenth of that.
// MFMA layouts: gdn_mfma_util.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <type_traits>

#include "gdn_mfma_util.h"
#include "gdn_step.h"
#include "gdn_window_common.h"

namespace gdn {
namespace wm {

constexpr int kDK = 128;        // key rows
constexpr int kKS = kDK / 32;   // k-steps of the bf16 products
constexpr int kTok = 16;        // window tokens: one 16-row MFMA tile
constexpr int kCB = 128;        // value columns per workgroup
constexpr int kLS = 20;         // padded row of a 16 x 16 LDS matrix
constexpr int kUS = 33;         // padded row of a wave's ut tile
constexpr float kReset = -128.f;  // exp(g) rounds to 0 in f32 below this

// Records of the previous window, staged for the fused replay.
struct Stage {
  float k[kTok][kDK];  // raw key rows
  float u[kTok][kCB];  // ut of this workgroup's columns
  f32x2 sc[kTok + 1];  // (phi, c); slot kTok: discarded writes
};
// The window's raw key / query / value rows (bf16 or f32, as given) and
// gates, staged once per workgroup (every wave reads its A fragments and
// per-token gates from here).
template <typename In>
struct RowLds {
  __attribute__((aligned(16))) In k[kTok][kDK];
  __attribute__((aligned(16))) In q[kTok][kDK];
  __attribute__((aligned(16))) In v[kTok][kCB];  // this block's columns
  float g[kTok + 1], b[kTok + 1];  // slot kTok: discarded writes
};
// The bf16 A fragment of eight staged entries: the raw words for bf16 rows;
// for f32 rows three parts, x = h + m + l + O(2^-25 |x|) (each bf16,
// rounded to nearest even): a product of two f32 rows keeps f32 accuracy
// only with all three (with two, a dot product of 128 terms that cancel
// loses about four bits of its 16).
struct Frag {
  u32x4 h, m, l;
};
__device__ __forceinline__ Frag frag8(const uint16_t* p) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  return Frag{*reinterpret_cast<const u32x4*>(p), z, z};
}
__device__ __forceinline__ Frag frag8(const float* p) {
  float x[8];
  row8(p, x);
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t r;
    split2(x[2 * i], x[2 * i + 1], h[i], r);
    m[i] = r;
    const float ra = x[2 * i] - lo_f(h[i]) - lo_f(r);
    const float rb = x[2 * i + 1] - hi_f(h[i]) - hi_f(r);
    const f32x2 y = {ra, rb};
    l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
  }
  return Frag{u32x4{h[0], h[1], h[2], h[3]}, u32x4{m[0], m[1], m[2], m[3]},
              u32x4{l[0], l[1], l[2], l[3]}};
}
// Draft trees of more than 16 nodes: what later blocks need of a node (its
// path aggregate -- segment sum G, deepest zero-decay node R, scale c, fold
// phi, ancestor set -- its inverse key norm and raw key row), and per wave
// the deltas U of every block but the last, in the D layout of T X.
template <typename In>
struct TreeLds {
  __attribute__((aligned(16))) In k[GDN_MAX_T][kDK];
  __attribute__((aligned(16))) f32x4 U[kWaves][GDN_MAX_T / kTok - 1][2][kWave];
  float G[GDN_MAX_T], c[GDN_MAX_T], phi[GDN_MAX_T], rk[GDN_MAX_T];
  int R[GDN_MAX_T];
  uint32_t alo[GDN_MAX_T], ahi[GDN_MAX_T];
};
// Debug states of such trees: every node's ut tile, per wave.
struct TreeDbgLds {
  float Us[kWaves][GDN_MAX_T * kUS];
};
// Debug states of a window of several blocks: the token-by-token replay
// state, carried from block to block (entry 2 (8 ks + e) + cs of thread tid).
struct SeqLds {
  float s[2 * 8 * kKS][kBlock];
};
// A wave's private LDS: L transposed, T, and (debug states only) its ut tile.
struct WaveLds {
  __attribute__((aligned(16))) float Lt[kTok * kLS];
  __attribute__((aligned(16))) float Ts[kTok * kLS];
  __attribute__((aligned(16))) float vec[6][kTok];  // per-token factors
  float Us[kTok * kUS];
};

// TREE: a draft-tree window (no fused replay).  Node t steps from the state
// of its parent (S0 for a root); the block form holds with the causal mask
// replaced by the ancestor relation: L_ts and P_ts are nonzero only for s an
// ancestor (or, for P, t itself), dec(t, s) is the decay along the path from
// s to t, and the scale sequence continues the parent's scale.  A parent
// precedes its children, so L stays strictly lower triangular.  A tree of
// several blocks (MB) is solved from the root state throughout, by block
// forward substitution of the whole system: block b's nodes take
// X_b -= L_bb' U_b' and O_b += P_bb' U_b' from every earlier block b'
// (their keys, path aggregates and, per wave, U kept in LDS); the held
// state never moves.
template <bool REPLAY, bool DBG, bool TREE, bool MB, bool F32>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(DBG || F32 || (MB && (REPLAY || TREE)) ? 2 : 3)))
void mverify_kernel(
    const std::conditional_t<F32, float, uint16_t>* __restrict__ q,
    const std::conditional_t<F32, float, uint16_t>* __restrict__ k,
    const std::conditional_t<F32, float, uint16_t>* __restrict__ v,
    const float* __restrict__ beta,
    const float* __restrict__ g, float* S, float* __restrict__ o,
    float* __restrict__ rec_k, float* __restrict__ rec_u,
    float2* __restrict__ rec_scale, float* __restrict__ dbg, WinDims d,
    LaneTable tl, float scale, int l2norm, PrevRecords prev,
    std::conditional_t<TREE, TreeTable, NoTable> tree) {
  static_assert(!(TREE && REPLAY), "draft trees have no fused replay");
  using In = std::conditional_t<F32, float, uint16_t>;
  constexpr int kEl = 16 / (int)sizeof(In);  // entries per 16-byte piece
  constexpr int kPc = F32 ? 2 : 1;           // pieces per thread and row
  __shared__ WaveLds wl[kWaves];
  __shared__ RowLds<In> rows;
  __shared__ std::conditional_t<REPLAY, Stage, char> stage;
  __shared__ std::conditional_t<DBG && MB && !TREE, SeqLds, char> seq;
  __shared__ std::conditional_t<TREE && MB, TreeLds<In>, char> tn;
  __shared__ std::conditional_t<TREE && MB && DBG, TreeDbgLds, char> tdbg;

  const int nc = d.dv / kCB;
  int item = xcd_item(blockIdx.x, gridDim.x);
  const int cb = item % nc;
  item /= nc;
  const int h = item % d.Hv;
  item /= d.Hv;
  // (layer, lane): an XCD's share is a range of layers (xcd_item); in the
  // fused call its workgroups go lane by lane in prev.order (costliest
  // lanes first), every layer of a lane together
  int lane, layer;
  if (REPLAY && gridDim.x % 8 == 0 && d.NL % 8 == 0) {
    const int lx = d.NL / 8;
    const int x = item / (lx * d.N), j = item % (lx * d.N);
    lane = table_byte(prev.order, j / lx);
    layer = x * lx + j % lx;
  } else {
    lane = item % d.N;
    layer = item / d.N;
  }
  const int T = table_byte(tl, lane);
  const int m_prev = REPLAY ? table_byte(prev.m, lane) : 0;
  if (T == 0 && m_prev == 0) return;

  const int tid = (int)threadIdx.x;
  const int w = uniform(tid / kWave);
  const int l = tid % kWave;
  const int g4 = l >> 4, n = l & 15;
  const int kh = h / d.group;
  const int dv = d.dv;
  const int c0 = kCB * cb + 32 * w + 2 * n;  // this lane's columns c0, c0 + 1
  const size_t ll = (size_t)layer * d.N + lane;
  const size_t tok0 = ll * d.T;              // token 0 of this lane-layer
  const size_t kq_step = (size_t)d.Hk * kDK;  // per token: q, k, key records
  const size_t vo_step = (size_t)d.Hv * dv;   // per token: v, o, ut records
  const In* __restrict__ k0 = k + (tok0 * d.Hk + kh) * kDK;
  const In* __restrict__ q0 = q + (tok0 * d.Hk + kh) * kDK;
  const In* __restrict__ v0 = v + (tok0 * d.Hv + h) * (size_t)dv;
  const size_t gh0 = tok0 * d.Hv + h;  // gate index of token 0 (step Hv)
  float* const Sh = S + (ll * d.Hv + h) * (size_t)kDK * dv;
  // The head's state through a buffer resource: row 32 ks + 8 g4 + e is the
  // uniform byte offset of row 32 ks + e (an SGPR) plus this lane's offset
  // (one VGPR for all 32 accesses); accesses past the head's rows would
  // read 0 and write nothing.
  const uint32_t soff = (uint32_t)(8 * g4 * dv + c0) * 4u;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      Sh, 0, kDK * dv * (int)sizeof(float), kBufWord3);
  auto sload = [&](int r) -> f32x2 {
    return __builtin_bit_cast(
        f32x2, __builtin_amdgcn_raw_buffer_load_b64(srs, soff, r * dv * 4, kNT));
  };
  auto sstore = [&](int r, f32x2 x) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), srs,
                                          soff, r * dv * 4, kNT);
  };
  auto srow = [&](float* base, int r) -> f32x2* {
    return reinterpret_cast<f32x2*>(
        reinterpret_cast<char*>(base + (size_t)r * dv) + soff);
  };
  WaveLds& W = wl[w];

  // ---- the window's rows, staged cooperatively: thread (rt, rp) loads one
  // 16-byte piece of key row rt, of query row rt and of value row rt (this
  // block's columns), threads 0..15 the gates of token tid.  All of it is
  // requested before the state, so that everything but the state products
  // overlaps the state's latency.  Tokens at or past T read token 0 and are
  // replaced by zeros.
  const int rt = tid >> 4, rp = tid & 15;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  u32x4 kr[kPc], qr[kPc], vr[kPc];
  float gl, bl;
  // the rows of the block of tokens tb .. tb + Tb - 1: thread (rt, rp) the
  // 16-byte pieces rp (and rp + 16 for f32 rows) of key row rt, of query row
  // rt and of value row rt (this workgroup's columns), threads 0..15 the
  // gates of token tid; tokens at or past Tb read the block's first token
  // and are replaced by zeros
  auto load_rows = [&](int tb, int Tb) {
    const bool rv = rt < Tb;
    const int tr = tb + (rv ? rt : 0);
#pragma unroll
    for (int p = 0; p < kPc; ++p) {
      const int pe = kEl * (rp + 16 * p);
      kr[p] = *reinterpret_cast<const u32x4*>(k0 + (uint32_t)(tr * kq_step) + pe);
      qr[p] = *reinterpret_cast<const u32x4*>(q0 + (uint32_t)(tr * kq_step) + pe);
      kr[p] = rv ? kr[p] : z4;
      qr[p] = rv ? qr[p] : z4;
    }
    const int tg = tb + (tid < Tb ? tid : 0);
    gl = g[gh0 + (size_t)tg * d.Hv];
    bl = beta[gh0 + (size_t)tg * d.Hv];
#pragma unroll
    for (int p = 0; p < kPc; ++p) {
      vr[p] = *reinterpret_cast<const u32x4*>(
          v0 + (uint32_t)(tr * vo_step) + kCB * cb + kEl * (rp + 16 * p));
      vr[p] = rv ? vr[p] : z4;
    }
  };
  auto stage_rows = [&](int tb, int Tb) {
    const bool rv = rt < Tb;
#pragma unroll
    for (int p = 0; p < kPc; ++p) {
      const int pe = kEl * (rp + 16 * p);
      *reinterpret_cast<u32x4*>(&rows.k[rt][pe]) = kr[p];
      *reinterpret_cast<u32x4*>(&rows.q[rt][pe]) = qr[p];
      *reinterpret_cast<u32x4*>(&rows.v[rt][pe]) = vr[p];
      if constexpr (TREE && MB)
        *reinterpret_cast<u32x4*>(&tn.k[tb + rt][pe]) = kr[p];
    }
    // every thread stores (threads past kTok into the discarded slot): a
    // store under a branch lets the compiler sink the gate loads into it,
    // behind the state requests, and wait for the whole state there
    const int gs = tid < kTok ? tid : kTok;
    rows.g[gs] = tid < Tb ? gl : 0.f;
    rows.b[gs] = tid < Tb ? bl : 0.f;
    // the key record rows (raw rows as f32): thread (rt, rp) writes its
    // pieces; done here so that the pieces are dead past the staging
    if (cb == 0 && h % d.group == 0 && rv) {
      float* __restrict__ dst = rec_k + (tok0 * d.Hk + kh) * kDK +
                                (uint32_t)((tb + rt) * kq_step);
      if constexpr (F32) {
#pragma unroll
        for (int p = 0; p < kPc; ++p)
          *reinterpret_cast<u32x4*>(dst + kEl * (rp + 16 * p)) = kr[p];
      } else {
        const u32x4 kw = kr[0];
        reinterpret_cast<float4*>(dst + 8 * rp)[0] =
            make_float4(lo_f(kw[0]), hi_f(kw[0]), lo_f(kw[1]), hi_f(kw[1]));
        reinterpret_cast<float4*>(dst + 8 * rp)[1] =
            make_float4(lo_f(kw[2]), hi_f(kw[2]), lo_f(kw[3]), hi_f(kw[3]));
      }
    }
  };
  // the first block's rows are requested before the state, so that
  // everything but the state products overlaps the state's latency
  const int T0 = MB ? (T < kTok ? T : kTok) : T;
  load_rows(0, T0);
  auto frag_k = [&](int ks) { return frag8(&rows.k[n][32 * ks + 8 * g4]); };
  auto frag_q = [&](int ks) { return frag8(&rows.q[n][32 * ks + 8 * g4]); };

  // ---- the state: rows 32 ks + 8 g4 + e, columns c0 and c0 + 1
  f32x2 s2[kKS][8];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      s2[ks][e] = sload(32 * ks + e);
  // keep the state requests here, right behind the small loads: the
  // scheduler would otherwise sink them below the first uses of the small
  // loads and wait for those first
  __builtin_amdgcn_sched_barrier(0);
  stage_rows(0, T0);
  __syncthreads();

  // ---- fused commit: the accepted prefix of the previous window, replayed
  // on the held state with exactly the operations of gdn_commit (fold,
  // fma per entry, materialisation) and stored.  The records come in
  // through LDS: two float4 of key rows and two of ut per thread, and the
  // scale steps.
  if constexpr (REPLAY) {
    if (m_prev > 0) {
      const float* __restrict__ pk = prev.k + (tok0 * d.Hk + kh) * kDK;
      const float* __restrict__ pu =
          prev.u + (tok0 * d.Hv + h) * (size_t)dv + kCB * cb;
      // the records arrive in chunks of kTok tokens (one chunk for windows
      // of at most kTok tokens)
      const int nrc = MB ? (m_prev + kTok - 1) / kTok : 1;
      int mc = m_prev;
      for (int rc = 0; rc < nrc; ++rc) {
        const int r0 = rc * kTok;
        mc = MB ? (m_prev - r0 < kTok ? m_prev - r0 : kTok) : m_prev;
        if (MB && rc > 0) __syncthreads();  // the previous chunk is applied
        f32x4 kst[2], ust[2];
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
          const int e = tid + kBlock * rep;  // float4 slot: token e/32
          int tok = e >> 5;
          tok = r0 + (tok < mc ? tok : mc - 1);
          kst[rep] = *reinterpret_cast<const f32x4*>(
              pk + (uint32_t)(tok * kq_step) + 4 * (e & 31));
          ust[rep] = *reinterpret_cast<const f32x4*>(
              pu + (uint32_t)(tok * vo_step) + 4 * (e & 31));
        }
        const int ts = r0 + (tid < mc ? tid : mc - 1);
        const f32x2 scst = *reinterpret_cast<const f32x2*>(
            prev.scale + gh0 + (size_t)ts * d.Hv);
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
          const int e = tid + kBlock * rep;
          reinterpret_cast<f32x4*>(&stage.k[0][0])[e] = kst[rep];
          reinterpret_cast<f32x4*>(&stage.u[0][0])[e] = ust[rep];
        }
        // every thread stores (past kTok into the discarded slot), so that
        // the scale load is not sunk behind the record loads into a branch
        stage.sc[tid < kTok ? tid : kTok] = scst;
        __syncthreads();
        // one step: fold (when the record has one), then the rank-1 write
        auto step = [&](int t, bool may_fold) {
          const f32x2 fc = stage.sc[t];
          const f32x2 uc =
              *reinterpret_cast<const f32x2*>(&stage.u[t][32 * w + 2 * n]);
          f32x4 kc[2 * kKS];
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) {
            kc[2 * ks] =
                *reinterpret_cast<const f32x4*>(&stage.k[t][32 * ks + 8 * g4]);
            kc[2 * ks + 1] =
                *reinterpret_cast<const f32x4*>(&stage.k[t][32 * ks + 8 * g4 + 4]);
          }
          if (may_fold) {
            const float ph = __int_as_float(
                __builtin_amdgcn_readfirstlane(__float_as_int(fc[0])));
            if (ph != 1.f) {
#pragma unroll
              for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  s2[ks][e][0] = ph * s2[ks][e][0];
                  s2[ks][e][1] = ph * s2[ks][e][1];
                }
            }
          }
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float kv = kc[2 * ks + e / 4][e % 4];
              s2[ks][e][0] = state_update(s2[ks][e][0], uc[0], kv);
              s2[ks][e][1] = state_update(s2[ks][e][1], uc[1], kv);
            }
        };
        // folds are rare: a prefix without one runs a branch-free loop
        const bool any_fold =
            __builtin_amdgcn_ballot_w64(l < mc && stage.sc[l < kTok ? l : 0][0] != 1.f) != 0;
        if (any_fold) {
#pragma unroll 1
          for (int t = 0; t < mc; ++t) step(t, true);
        } else {
#pragma unroll
          for (int t = 0; t < kTok; ++t) {
            if (t >= mc) break;
            step(t, false);
          }
        }
      }
      const float cf = stage.sc[mc - 1][1];
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s2[ks][e][0] = materialise(cf, s2[ks][e][0]);
          s2[ks][e][1] = materialise(cf, s2[ks][e][1]);
          sstore(32 * ks + e, s2[ks][e]);
        }
    }
    if (T == 0) return;
  }
  // the window in blocks of kTok tokens (one block unless MB): block tb
  // starts from the held state, the scaled replay state of the tokens
  // before it with scale c_in
  float c_in = 1.0f;
  for (int tb = 0;; tb += kTok) {
    const int Tb = MB ? (T - tb < kTok ? T - tb : kTok) : T;
    if (MB && tb > 0) {
      // plain verify requested this block's rows during the previous block;
      // the fused call (more registers live there) requests them here
      if constexpr (REPLAY) load_rows(tb, Tb);
      __syncthreads();  // every wave is done with the previous block's rows
      stage_rows(tb, Tb);
      __syncthreads();
    }
    const float gt = rows.g[n], bt = rows.b[n];
    Frag Kf[kKS], Qf[kKS];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      Kf[ks] = frag_k(ks);
      Qf[ks] = frag_q(ks);
    }

    // ---- inverse norms of token n (sums over the lane's row pieces, then
    // over the four groups)
    float skk = 0.f, sqq = 0.f;
    if constexpr (F32) {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        float kx[8], qx[8];
        row8(&rows.k[n][32 * ks + 8 * g4], kx);
        row8(&rows.q[n][32 * ks + 8 * g4], qx);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          skk = __builtin_fmaf(kx[i], kx[i], skk);
          sqq = __builtin_fmaf(qx[i], qx[i], sqq);
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const u32x4 kw = Kf[ks].h, qw = Qf[ks].h;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          skk = __builtin_fmaf(lo_f(kw[p]), lo_f(kw[p]), skk);
          skk = __builtin_fmaf(hi_f(kw[p]), hi_f(kw[p]), skk);
          sqq = __builtin_fmaf(lo_f(qw[p]), lo_f(qw[p]), sqq);
          sqq = __builtin_fmaf(hi_f(qw[p]), hi_f(qw[p]), sqq);
        }
      }
    }
    skk += __shfl_xor(skk, 16, kWave);
    sqq += __shfl_xor(sqq, 16, kWave);
    skk += __shfl_xor(skk, 32, kWave);
    sqq += __shfl_xor(sqq, 32, kWave);
    const float rk = l2norm ? __builtin_amdgcn_rsqf(skk + 1e-6f) : 1.0f;
    const float rq = l2norm ? __builtin_amdgcn_rsqf(sqq + 1e-6f) : 1.0f;


    // ---- K K^T and K Q^T: lane (g4, n), entry e = (k_{4g4+e} . k_n) and
    // (k_{4g4+e} . q_n) -- row n, column s = 4 g4 + e of the A layout of the
    // f32 products below
    f32x4 KK = {0.f, 0.f, 0.f, 0.f}, KQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      KK = mma_bf16(Kf[ks].h, Kf[ks].h, KK);
      KQ = mma_bf16(Kf[ks].h, Qf[ks].h, KQ);
      if constexpr (F32) {  // the part products of order at most 2^-16
        KK = mma_bf16(Kf[ks].h, Kf[ks].m, KK);
        KK = mma_bf16(Kf[ks].m, Kf[ks].h, KK);
        KK = mma_bf16(Kf[ks].h, Kf[ks].l, KK);
        KK = mma_bf16(Kf[ks].m, Kf[ks].m, KK);
        KK = mma_bf16(Kf[ks].l, Kf[ks].h, KK);
        KQ = mma_bf16(Kf[ks].h, Qf[ks].m, KQ);
        KQ = mma_bf16(Kf[ks].m, Qf[ks].h, KQ);
        KQ = mma_bf16(Kf[ks].h, Qf[ks].l, KQ);
        KQ = mma_bf16(Kf[ks].m, Qf[ks].m, KQ);
        KQ = mma_bf16(Kf[ks].l, Qf[ks].h, KQ);
      }
    }

    // ---- gates of token n, within each 16-lane group: segmented sums Gs
    // (restarting after the last token R <= n whose decay is 0) and the scale
    // sequence c of gdn_step.h (prefix products of alpha, folded when out of
    // [2^-32, 2^32]; that rare case walks the tokens in order)
    const bool tv = n < Tb;
    const float a_t = tv ? __expf(gt) : 1.0f;
    float Gs, c, phi = 1.f;
    int R;         // deepest zero-decay token or node on the path (window index)
    uint32_t anc;  // bit s: token tb + s is a strict ancestor of token tb + n
    [[maybe_unused]] uint64_t ancx = 0;  // trees: strict ancestors in earlier blocks
    if constexpr (TREE) {
      // pointer jumping over the ancestor chain: lane n holds the aggregate
      // of the path segment (J, n] (segment sum and deepest zero-decay node,
      // ancestor set, product of the decays) and combines it with the one that
      // lane J holds for (J', J], all lanes at once; parents precede their
      // children, so a segment inside the block has at most 16 nodes and four
      // jumps reach its first node.  On a chain this is the window's scan,
      // step for step.  In a tree of several blocks the segment then meets
      // the aggregate of its first node's parent, a node of an earlier block
      // (ext), kept in LDS.
      int J = -1, ext = -1;
      for (int t = 0; t < Tb; ++t) {
        const int par = tree_parent(tree, lane * d.T + tb + t);
        J = n == t ? (par >= tb ? par - tb : -1) : J;
        ext = n == t ? (par >= tb ? -1 : par) : ext;
      }
      const bool reset = gt < kReset;
      Gs = reset ? 0.f : gt;
      R = reset ? tb + n : -1;
      anc = 0u;
      c = a_t;
#pragma unroll
      for (int step = 0; step < 4; ++step) {
        const int src = J < 0 ? 0 : J;
        const float Gy = __shfl(Gs, src, 16);
        const int Ry = __shfl(R, src, 16);
        const uint32_t ay = (uint32_t)__shfl((int)anc, src, 16);
        const float cy = __shfl(c, src, 16);
        const int Jy = __shfl(J, src, 16);
        const int ey = __shfl(ext, src, 16);
        if (J >= 0) {
          Gs = R < 0 ? Gy + Gs : Gs;
          R = R > Ry ? R : Ry;
          anc = anc | ay | (1u << J);
          c *= cy;
          J = Jy;
          ext = ey;
        }
      }
      if constexpr (MB) {
        if (ext >= 0) {
          Gs = R < 0 ? tn.G[ext] + Gs : Gs;
          R = R > tn.R[ext] ? R : tn.R[ext];
          ancx = ((uint64_t)tn.ahi[ext] << 32 | tn.alo[ext]) | (1ull << ext);
          c *= tn.c[ext];
        }
      }
      // the scale sequence of gdn_step.h needs a fold somewhere (rare): walk
      // the nodes in index order, each continuing its parent's scale
      const bool out = !(c >= kScaleLo && c <= kScaleHi);
      if (__builtin_amdgcn_ballot_w64(out && tv) != 0) {
        for (int t = 0; t < Tb; ++t) {
          const int par = tree_parent(tree, lane * d.T + tb + t);
          float cp = 1.0f;
          if (par >= tb) cp = lane_value(c, par - tb);
          if constexpr (MB) {
            if (par >= 0 && par < tb) cp = tn.c[par];
          }
          float cn, fo = 1.f;
          if (scale_step(cp, lane_value(a_t, t), cn)) {
            fo = cn;
            cn = 1.0f;
          }
          if (n == t) {
            c = cn;
            phi = fo;
          }
        }
      }
    } else {
      const bool reset = gt < kReset;
      Gs = reset ? 0.f : gt;
      R = reset ? tb + n : -1;
      anc = (1u << n) - 1u;
      c = a_t;
      // inclusive scans over the 16 lanes of each row by DPP row shifts; a
      // lane without a source reads the identity (0, -1, 1)
      auto scan_step = [&](auto ctrl) {
        constexpr int kCtrl = decltype(ctrl)::value;
        const float ys = row_shift<kCtrl>(Gs, 0.f);
        const int yR = row_shift_int<kCtrl>(R, -1);
        const float yc = row_shift<kCtrl>(c, 1.f);
        Gs = R < 0 ? ys + Gs : Gs;
        R = R > yR ? R : yR;
        c *= yc;
      };
      scan_step(std::integral_constant<int, 0x111>{});  // row_shr:1
      scan_step(std::integral_constant<int, 0x112>{});  // row_shr:2
      scan_step(std::integral_constant<int, 0x114>{});  // row_shr:4
      scan_step(std::integral_constant<int, 0x118>{});  // row_shr:8
      // the scale continues from the previous block's last token
      if constexpr (MB) c = c_in * c;
      const bool out = !(c >= kScaleLo && c <= kScaleHi);
      if (__builtin_amdgcn_ballot_w64(out && tv) != 0) {
        float cc = c_in;
        for (int t = 0; t < Tb; ++t) {
          float cn, fo = 1.f;
          if (scale_step(cc, lane_value(a_t, t), cn)) {
            fo = cn;
            cn = 1.0f;
          }
          if (n == t) {
            c = cn;
            phi = fo;
          }
          cc = cn;
        }
      }
    }
    const float A = R >= 0 ? 0.f : __expf(Gs);
    if constexpr (TREE && MB) {
      // this block's nodes, for the blocks after it (and its debug replay)
      if (w == 0 && l < Tb) {
        const uint64_t a64 = ancx | ((uint64_t)anc << tb);
        tn.G[tb + n] = Gs;
        tn.R[tb + n] = R;
        tn.c[tb + n] = c;
        tn.phi[tb + n] = phi;
        tn.rk[tb + n] = rk;
        tn.alo[tb + n] = (uint32_t)a64;
        tn.ahi[tb + n] = (uint32_t)(a64 >> 32);
      }
    }
    const float f2 = rk * __builtin_amdgcn_rcpf(c);  // ut = u * f2
    const float so = scale * rq * A;                 // on (Q H)_n
    const float xb = bt * A * rk;                    // on (K H)_n

    // ---- per-token factors through the wave's LDS: lane (g4, n) reads those
    // of the tokens 4 g4 .. 4 g4 + 3 as one float4 each
    if (l < kTok) {
      W.vec[0][n] = rk;
      W.vec[1][n] = Gs;
      W.vec[2][n] = bt;
      W.vec[3][n] = xb;
      W.vec[4][n] = so;
      W.vec[5][n] = f2;
    }
    wave_lds_sync();
    auto vec4 = [&](int i) {
      return *reinterpret_cast<const f32x4*>(&W.vec[i][4 * g4]);
    };
    // ---- L and P entries of row n, columns s = 4 g4 + e
    float PA[4];
    {
      const float bk = bt * rk, sq = scale * rq;
      const f32x4 rk4 = vec4(0), gs4 = vec4(1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 4 * g4 + e;
        const float rks = rk4[e];
        const float Gss = gs4[e];
        const bool below = (anc >> s) & 1u;  // s a strict ancestor of n
        const bool on_path = below || s == n;
        const float dx = __expf(Gs - Gss);
        const float dec = (on_path && tb + s >= R) ? dx : 0.f;
        const float lv = bk * rks * KK[e] * dec;
        W.Lt[s * kLS + n] = below ? lv : 0.f;  // L[n][s], transposed
        PA[e] = on_path ? sq * rks * KQ[e] * dec : 0.f;
      }
    }
    wave_lds_sync();
    // ---- T = (I + L)^-1: lane n < 16 of group 0 solves column n by
    // right-looking substitution (once t_x is known it updates every later
    // row), then the columns meet in LDS to be read back as row pieces
    if (l < kTok) {
      float acc[kTok];
#pragma unroll
      for (int r = 0; r < kTok; ++r) acc[r] = 0.f;
#pragma unroll
      for (int x = 0; x < kTok; ++x) {
        const float tx = x == n ? 1.f : (x < n ? 0.f : -acc[x]);
        W.Ts[x * kLS + n] = tx;
#pragma unroll
        for (int r = x + 1; r < kTok; ++r)
          acc[r] = __builtin_fmaf(W.Lt[x * kLS + r], tx, acc[r]);
      }
    }
    wave_lds_sync();
    const float4 TA = *reinterpret_cast<const float4*>(&W.Ts[n * kLS + 4 * g4]);

    // the key / query fragments are read again from the staged rows: the
    // first copies died after K K^T and the norms, so they held no registers
    // through the solve, and no global round trip follows the state's arrival

    // ---- K H and Q H: per k-step, the eight rows of each column split into
    // bf16 hi and lo, two MFMAs each against the exact key / query pieces
    f32x4 KH[2], QH[2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      KH[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
      QH[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      uint32_t h0[4], lo0[4], h1[4], lo1[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        split2(s2[ks][2 * p][0], s2[ks][2 * p + 1][0], h0[p], lo0[p]);
        split2(s2[ks][2 * p][1], s2[ks][2 * p + 1][1], h1[p], lo1[p]);
      }
      const u32x4 H0 = {h0[0], h0[1], h0[2], h0[3]};
      const u32x4 L0 = {lo0[0], lo0[1], lo0[2], lo0[3]};
      const u32x4 H1 = {h1[0], h1[1], h1[2], h1[3]};
      const u32x4 L1 = {lo1[0], lo1[1], lo1[2], lo1[3]};
      const Frag kf = frag_k(ks), qf = frag_q(ks);
      KH[0] = mma_bf16(kf.h, H0, KH[0]);
      KH[1] = mma_bf16(kf.h, H1, KH[1]);
      QH[0] = mma_bf16(qf.h, H0, QH[0]);
      QH[1] = mma_bf16(qf.h, H1, QH[1]);
      KH[0] = mma_bf16(kf.h, L0, KH[0]);
      KH[1] = mma_bf16(kf.h, L1, KH[1]);
      QH[0] = mma_bf16(qf.h, L0, QH[0]);
      QH[1] = mma_bf16(qf.h, L1, QH[1]);
      if constexpr (F32) {  // the rows' m and l parts (state hi, lo)
        KH[0] = mma_bf16(kf.m, H0, KH[0]);
        KH[1] = mma_bf16(kf.m, H1, KH[1]);
        QH[0] = mma_bf16(qf.m, H0, QH[0]);
        QH[1] = mma_bf16(qf.m, H1, QH[1]);
        KH[0] = mma_bf16(kf.m, L0, KH[0]);
        KH[1] = mma_bf16(kf.m, L1, KH[1]);
        QH[0] = mma_bf16(qf.m, L0, QH[0]);
        QH[1] = mma_bf16(qf.m, L1, QH[1]);
        KH[0] = mma_bf16(kf.l, H0, KH[0]);
        KH[1] = mma_bf16(kf.l, H1, KH[1]);
        QH[0] = mma_bf16(qf.l, H0, QH[0]);
        QH[1] = mma_bf16(qf.l, H1, QH[1]);
      }
    }
    const bool more = MB && tb + kTok < T;
    if constexpr (MB) {
      // past the first block the held state is the scaled replay state:
      // S = c_in * St
#pragma unroll
      for (int cs = 0; cs < 2; ++cs)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          KH[cs][e] *= c_in;
          QH[cs][e] *= c_in;
        }
    }

    // ---- X, U = T X, O = diag(so) Q H + P U, ut = U f2 (rows t = 4 g4 + e)
    const f32x4 bte = vec4(2), xbe = vec4(3), soe = vec4(4), f2e = vec4(5);
    // values of the tokens 4 g4 + e at columns c0, c0 + 1
    float va[4], vb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (F32) {
        const f32x2 x = *reinterpret_cast<const f32x2*>(
            &rows.v[4 * g4 + e][32 * w + 2 * n]);
        va[e] = x[0];
        vb[e] = x[1];
      } else {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(
            &rows.v[4 * g4 + e][32 * w + 2 * n]);
        va[e] = lo_f(x);
        vb[e] = hi_f(x);
      }
    }
    f32x4 X[2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool te = 4 * g4 + e < Tb;
      const float x0 = __builtin_fmaf(-xbe[e], KH[0][e], bte[e] * va[e]);
      const float x1 = __builtin_fmaf(-xbe[e], KH[1][e], bte[e] * vb[e]);
      X[0][e] = te ? x0 : 0.f;
      X[1][e] = te ? x1 : 0.f;
    }
    // ---- draft trees of several blocks: the ancestors in earlier blocks,
    // by block forward substitution of the whole window's system (every node
    // is solved from the root state H): X_b -= L_bb' U_b' and O_b +=
    // P_bb' U_b' for each earlier block b', with L_bb' and P_bb' the
    // ancestor-masked, path-decayed entries between the blocks' nodes
    [[maybe_unused]] f32x4 Oc[2] = {f32x4{0.f, 0.f, 0.f, 0.f},
                                    f32x4{0.f, 0.f, 0.f, 0.f}};
    if constexpr (TREE && MB) {
      const float bk = bt * rk, sq = scale * rq;
      const uint32_t alo = (uint32_t)ancx, ahi = (uint32_t)(ancx >> 32);
#pragma unroll 1
      for (int bp = 0; bp < tb / kTok; ++bp) {
        // lane (g4, n), entry e: (k_s . k_t) and (k_s . q_t) for node
        // s = 16 bp + 4 g4 + e and node t = tb + n
        f32x4 KKx = {0.f, 0.f, 0.f, 0.f}, KQx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          const Frag fb = frag8(&tn.k[kTok * bp + n][32 * ks + 8 * g4]);
          const Frag kf = frag_k(ks), qf = frag_q(ks);
          KKx = mma_bf16(fb.h, kf.h, KKx);
          KQx = mma_bf16(fb.h, qf.h, KQx);
          if constexpr (F32) {  // the part products of order at most 2^-16
            KKx = mma_bf16(fb.h, kf.m, KKx);
            KKx = mma_bf16(fb.m, kf.h, KKx);
            KKx = mma_bf16(fb.h, kf.l, KKx);
            KKx = mma_bf16(fb.m, kf.m, KKx);
            KKx = mma_bf16(fb.l, kf.h, KKx);
            KQx = mma_bf16(fb.h, qf.m, KQx);
            KQx = mma_bf16(fb.m, qf.h, KQx);
            KQx = mma_bf16(fb.h, qf.l, KQx);
            KQx = mma_bf16(fb.m, qf.m, KQx);
            KQx = mma_bf16(fb.l, qf.h, KQx);
          }
        }
        float La[4], Pa[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sg = kTok * bp + 4 * g4 + e;
          const bool an = (((sg < 32 ? alo >> sg : ahi >> (sg - 32))) & 1u) != 0;
          const float dec = (an && sg >= R) ? __expf(Gs - tn.G[sg]) : 0.f;
          const float rks = tn.rk[sg];
          La[e] = bk * rks * KKx[e] * dec;
          Pa[e] = sq * rks * KQx[e] * dec;
        }
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
          const f32x4 Ub = tn.U[w][bp][cs][l];
          f32x4 Xc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            Xc = mma_f32(La[e], Ub[e], Xc);
            Oc[cs] = mma_f32(Pa[e], Ub[e], Oc[cs]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) X[cs][e] -= Xc[e];
        }
      }
    }
    const float ta[4] = {TA.x, TA.y, TA.z, TA.w};
    f32x4 U[2], O[2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      U[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) U[cs] = mma_f32(ta[e], X[cs][e], U[cs]);
#pragma unroll
      for (int e = 0; e < 4; ++e) O[cs][e] = soe[e] * QH[cs][e];
#pragma unroll
      for (int e = 0; e < 4; ++e) O[cs] = mma_f32(PA[e], U[cs][e], O[cs]);
      if constexpr (TREE && MB) O[cs] += Oc[cs];
    }
    if constexpr (TREE && MB) {
      if (tb + kTok < T) {
        tn.U[w][tb / kTok][0][l] = U[0];
        tn.U[w][tb / kTok][1][l] = U[1];
      }
    }
    float* __restrict__ o0 = o + ((tok0 + tb) * d.Hv + h) * (size_t)dv;
    float* __restrict__ u0 = rec_u + ((tok0 + tb) * d.Hv + h) * (size_t)dv;
    float ut[2][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * g4 + e;
      ut[0][e] = U[0][e] * f2e[e];
      ut[1][e] = U[1][e] * f2e[e];
      if (t < Tb) {
        const uint32_t off = (uint32_t)(t * vo_step) + c0;
        // outputs are not read again by this path: nontemporal stores keep
        // them from displacing the records and rows in the caches (verify
        // 0.206 -> 0.188 ms at 8 lanes x 48 layers, T = 16)
        __builtin_nontemporal_store(f32x2{O[0][e], O[1][e]},
                                    reinterpret_cast<f32x2*>(o0 + off));
        *reinterpret_cast<float2*>(u0 + off) = make_float2(ut[0][e], ut[1][e]);
      }
    }
    if (cb == 0 && w == 0 && l < Tb)
      rec_scale[gh0 + (size_t)(tb + l) * d.Hv] = make_float2(phi, c);
    // the next block's rows, requested here so that their latency overlaps
    // the state's update below (plain verify: T = 33 0.46 -> 0.43 ms at
    // 8 lanes x 48 layers; the fused call lost 3 % this way)
    if constexpr (!REPLAY)
      if (more) load_rows(tb + kTok, T - tb - kTok < kTok ? T - tb - kTok : kTok);
    // ---- debug states: the replay of this window's own records on the
    // start state (the committed state in the fused call), token by token; in
    // a draft tree, node t's state is the replay of the records on its path.
    // In a window of several blocks the replay runs on its own copy of the
    // state, carried from block to block through LDS (the held state moves
    // on by the block products below), so that it stays the token-by-token
    // replay of every record before it.
    if constexpr (DBG) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        W.Us[(4 * g4 + e) * kUS + 2 * n] = ut[0][e];
        W.Us[(4 * g4 + e) * kUS + 2 * n + 1] = ut[1][e];
      }
      wave_lds_sync();
      // record r applied to st: the fold, then the rank-1 write
      auto apply = [&](f32x2 (&st)[kKS][8], int r) {
        const float ph = lane_value(phi, r);
        if (ph != 1.f) {
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              st[ks][e][0] = ph * st[ks][e][0];
              st[ks][e][1] = ph * st[ks][e][1];
            }
        }
        const float ua = W.Us[r * kUS + 2 * n], ub = W.Us[r * kUS + 2 * n + 1];
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          // the block's raw key rows, still staged in LDS
          float kx[8];
          row8(&rows.k[r][32 * ks + 8 * g4], kx);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kv = kx[e];
            st[ks][e][0] = state_update(st[ks][e][0], ua, kv);
            st[ks][e][1] = state_update(st[ks][e][1], ub, kv);
          }
        }
      };
      auto emit = [&](const f32x2 (&st)[kKS][8], int t) {
        const float ct = lane_value(c, t);
        float* __restrict__ dp =
            dbg + (((tok0 + tb + t) * d.Hv + h) * (size_t)kDK) * dv;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *srow(dp, 32 * ks + e) =
                f32x2{materialise(ct, st[ks][e][0]), materialise(ct, st[ks][e][1])};
      };
      if constexpr (TREE && MB) {
        // the path's records over every block: ut tiles, keys, folds and
        // ancestor sets of all nodes so far from LDS
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tdbg.Us[w][(tb + 4 * g4 + e) * kUS + 2 * n] = ut[0][e];
          tdbg.Us[w][(tb + 4 * g4 + e) * kUS + 2 * n + 1] = ut[1][e];
        }
        __syncthreads();  // this block's node records (wave 0) are in place
        auto apply_node = [&](f32x2 (&st)[kKS][8], int r) {
          const float ph = tn.phi[r];
          if (ph != 1.f) {
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                st[ks][e][0] = ph * st[ks][e][0];
                st[ks][e][1] = ph * st[ks][e][1];
              }
          }
          const float ua = tdbg.Us[w][r * kUS + 2 * n];
          const float ub = tdbg.Us[w][r * kUS + 2 * n + 1];
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) {
            float kx[8];
            row8(&tn.k[r][32 * ks + 8 * g4], kx);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              st[ks][e][0] = state_update(st[ks][e][0], ua, kx[e]);
              st[ks][e][1] = state_update(st[ks][e][1], ub, kx[e]);
            }
          }
        };
#pragma unroll 1
        for (int t = 0; t < Tb; ++t) {
          const uint64_t path = ((uint64_t)tn.ahi[tb + t] << 32 | tn.alo[tb + t]) |
                                (1ull << (tb + t));
          f32x2 sd[kKS][8];
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) sd[ks][e] = s2[ks][e];
#pragma unroll 1
          for (int r = 0; r <= tb + t; ++r)
            if ((path >> r) & 1ull) apply_node(sd, r);
          emit(sd, t);
        }
      } else if constexpr (TREE) {
#pragma unroll 1
        for (int t = 0; t < T; ++t) {
          const uint32_t path = (uint32_t)lane_int((int)anc, t) | (1u << t);
          f32x2 sd[kKS][8];
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) sd[ks][e] = s2[ks][e];
#pragma unroll 1
          for (int r = 0; r <= t; ++r)
            if ((path >> r) & 1u) apply(sd, r);
          emit(sd, t);
        }
      } else if constexpr (MB) {
        f32x2 sd[kKS][8];
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sd[ks][e] = tb == 0 ? s2[ks][e]
                                : f32x2{seq.s[2 * (8 * ks + e)][tid],
                                        seq.s[2 * (8 * ks + e) + 1][tid]};
#pragma unroll 1
        for (int t = 0; t < Tb; ++t) {
          apply(sd, t);
          emit(sd, t);
        }
        if (more) {
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              seq.s[2 * (8 * ks + e)][tid] = sd[ks][e][0];
              seq.s[2 * (8 * ks + e) + 1][tid] = sd[ks][e][1];
            }
        }
      } else {
#pragma unroll 1
        for (int t = 0; t < Tb; ++t) {
          apply(s2, t);
          emit(s2, t);
        }
      }
    }
    // ---- the held state after the block, for the next one: the block's
    // rank-1 writes summed in one product, St += K^T Ut (key rows as the A
    // operand, the records ut as B), on v_mfma_f32_16x16x32_bf16.  The 32
    // k-slots of lane group g carry tokens 4 g .. 4 g + 3 twice, once for
    // each of two operand parts: ut enters as three bf16 parts, f32 key rows
    // as three as well (the six part products of order at most 2^-16),
    // bf16 key rows exactly.  Result row 4 g + i of tile (ks, half) is state
    // row 32 ks + 8 g + 4 half + i, so each lane receives exactly the
    // entries it holds.  Folds inside the block (rare) scale the start state
    // by the product of the block's phi and each ut_t by the phi after
    // token t: the closed form of the fold-then-write steps.
    if (!TREE && more) {
      float ub[2][4];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs)
#pragma unroll
        for (int e = 0; e < 4; ++e) ub[cs][e] = ut[cs][e];
      if (__builtin_amdgcn_ballot_w64(phi != 1.f) != 0) {
        float pall = 1.f, pf[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll 1
        for (int t = 0; t < Tb; ++t) {
          const float pt = lane_value(phi, t);
          pall *= pt;
#pragma unroll
          for (int e = 0; e < 4; ++e) pf[e] = t > 4 * g4 + e ? pf[e] * pt : pf[e];
        }
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            s2[ks][e][0] = pall * s2[ks][e][0];
            s2[ks][e][1] = pall * s2[ks][e][1];
          }
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
#pragma unroll
          for (int e = 0; e < 4; ++e) ub[cs][e] *= pf[e];
      }
      // ut of tokens 4 g4 .. 4 g4 + 3 in three parts (h, m, l), packed pairs
      u32x4 B1[2], B2[2];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        uint32_t ph[2], pm[2], pl[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float a = ub[cs][2 * i], b = ub[cs][2 * i + 1];
          split2(a, b, ph[i], pm[i]);
          const f32x2 y = {a - lo_f(ph[i]) - lo_f(pm[i]),
                           b - hi_f(ph[i]) - hi_f(pm[i])};
          pl[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
        }
        if constexpr (F32) {
          B1[cs] = u32x4{ph[0], ph[1], pm[0], pm[1]};  // [h, m]
          B2[cs] = u32x4{pl[0], pl[1], ph[0], ph[1]};  // [l, h]
        } else {
          B1[cs] = u32x4{ph[0], ph[1], pm[0], pm[1]};  // [h, m]
          B2[cs] = u32x4{pl[0], pl[1], 0u, 0u};        // [l, 0]
        }
      }
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          // key entry kx of tokens 4 g4 + j: the lane's A row
          const int kx = 32 * ks + 8 * (n >> 2) + 4 * half + (n & 3);
          f32x4 D[2];
          if constexpr (F32) {
            uint32_t ah[2], am[2], al[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const float a = rows.k[4 * g4 + 2 * i][kx];
              const float b = rows.k[4 * g4 + 2 * i + 1][kx];
              split2(a, b, ah[i], am[i]);
              const f32x2 y = {a - lo_f(ah[i]) - lo_f(am[i]),
                               b - hi_f(ah[i]) - hi_f(am[i])};
              al[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
            }
            const u32x4 Ahh = {ah[0], ah[1], ah[0], ah[1]};
            const u32x4 Amm = {am[0], am[1], am[0], am[1]};
            const u32x4 Ahl = {ah[0], ah[1], al[0], al[1]};
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
              D[cs] = mma_bf16(Ahh, B1[cs], f32x4{0.f, 0.f, 0.f, 0.f});
              D[cs] = mma_bf16(Amm, B1[cs], D[cs]);
              D[cs] = mma_bf16(Ahl, B2[cs], D[cs]);
            }
          } else {
            uint32_t a[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
              a[i] = (uint32_t)rows.k[4 * g4 + 2 * i][kx] |
                     ((uint32_t)rows.k[4 * g4 + 2 * i + 1][kx] << 16);
            const u32x4 A = {a[0], a[1], a[0], a[1]};
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
              D[cs] = mma_bf16(A, B1[cs], f32x4{0.f, 0.f, 0.f, 0.f});
              D[cs] = mma_bf16(A, B2[cs], D[cs]);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s2[ks][4 * half + i][0] += D[0][i];
            s2[ks][4 * half + i][1] += D[1][i];
          }
        }
    }
    if (!more) break;
    // a chain's next block continues the scale; a tree's nodes continue
    // their parents' scales (its blocks all start from the root state)
    if constexpr (!TREE) c_in = lane_value(c, Tb - 1);
  }
}

template <bool REPLAY, bool DBG, bool TREE, bool MB, bool F32 = false,
          typename Tab>
static hipError_t launch_t(const WinDims& w, const LaneTable& tl,
                           const VerifyArgs& a, const PrevRecords& pr,
                           const Tab& tree, hipStream_t st) {
  using In = std::conditional_t<F32, float, uint16_t>;
  const int blocks = w.NL * w.N * w.Hv * (w.dv / kCB);
  return launch(mverify_kernel<REPLAY, DBG, TREE, MB, F32>, dim3(blocks),
                dim3(kBlock), st, (const In*)a.q, (const In*)a.k,
                (const In*)a.v, a.beta, a.g, a.S, a.o, a.rk, a.ru, a.ra,
                a.dbg, w, tl, a.scale, a.l2, pr, tree);
}

}  // namespace wm

bool mverify_eligible(const gdn_dims& d, int in_dtype, const VerifyArgs& a,
                      bool tree) {
  auto al = [](const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; };
  return (in_dtype == GDN_BF16 || in_dtype == GDN_F32) &&
         d.d_k == wm::kDK && d.d_v % wm::kCB == 0 &&
         d.t_max <= GDN_MAX_T && al(a.q, 16) &&
         al(a.k, 16) && al(a.v, 4) && al(a.S, 8) && al(a.o, 8) &&
         (a.dbg == nullptr || al(a.dbg, 8));
}

template <bool MB, bool F32>
static hipError_t launch_window(const WinDims& w, const LaneTable& tl,
                                const VerifyArgs& a, const PrevRecords& pr,
                                bool replay, hipStream_t st) {
  const NoTable none{};
  if (replay)
    return a.dbg ? wm::launch_t<true, true, false, MB, F32>(w, tl, a, pr, none, st)
                 : wm::launch_t<true, false, false, MB, F32>(w, tl, a, pr, none, st);
  return a.dbg ? wm::launch_t<false, true, false, MB, F32>(w, tl, a, pr, none, st)
               : wm::launch_t<false, false, false, MB, F32>(w, tl, a, pr, none, st);
}

hipError_t launch_mverify(const WinDims& w, const LaneTable& tl,
                          const VerifyArgs& a, const PrevRecords& pr,
                          bool replay, hipStream_t st) {
  const bool mb = w.T > wm::kTok;  // windows of several blocks
  if (a.f32)
    return mb ? launch_window<true, true>(w, tl, a, pr, replay, st)
              : launch_window<false, true>(w, tl, a, pr, replay, st);
  return mb ? launch_window<true, false>(w, tl, a, pr, replay, st)
            : launch_window<false, false>(w, tl, a, pr, replay, st);
}

hipError_t launch_mverify_tree(const WinDims& w, const LaneTable& tl,
                               const VerifyArgs& a, const TreeTable& tree,
                               hipStream_t st) {
  PrevRecords none;
  memset(&none, 0, sizeof(none));
  if (w.T > wm::kTok) {  // trees of more than 16 nodes: several blocks
    if (a.f32)
      return a.dbg ? wm::launch_t<false, true, true, true, true>(w, tl, a, none, tree, st)
                   : wm::launch_t<false, false, true, true, true>(w, tl, a, none, tree, st);
    return a.dbg ? wm::launch_t<false, true, true, true>(w, tl, a, none, tree, st)
                 : wm::launch_t<false, false, true, true>(w, tl, a, none, tree, st);
  }
  if (a.f32)
    return a.dbg ? wm::launch_t<false, true, true, false, true>(w, tl, a, none, tree, st)
                 : wm::launch_t<false, false, true, false, true>(w, tl, a, none, tree, st);
  return a.dbg ? wm::launch_t<false, true, true, false>(w, tl, a, none, tree, st)
               : wm::launch_t<false, false, true, false>(w, tl, a, none, tree, st);
}

}  // namespace gdn
