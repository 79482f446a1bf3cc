// gdn_kda_mfma.hip -- KDA verify (the per-channel-decay sibling of the rule)
// on the gfx950 matrix cores, for bf16 or f32 inputs and d_k = d_v = 128: a
// window of at most 16 tokens as one block, longer windows (up to 64 tokens)
// in blocks of 16, each block from the state the blocks before it leave
// (their decay-then-write steps in closed form, the writes summed in one
// matrix-core product; equal to the commit's token-by-token replay to f32
// rounding).  Other shapes, and
// calls with GDN_FLAG_TOKENWISE, take gdn_kda.hip.
//
// The rule (Kimi Delta Attention of Kimi Linear, 2025; the NInfer technical
// review, blog.123qwe.co.kr post 4624, names its state and a kda_replay op
// contract) in the stored orientation H = S^T (d_k x d_v):
//   H'_t = diag(alpha_t) H_{t-1},  u_t = beta_t (v_t - H'_t^T khat_t),
//   H_t  = H'_t + khat_t u_t^T,    o_t = scale H_t^T qhat_t,
// alpha_t = exp(g_t) a d_k vector.  Over a window, with C_t = alpha_0 ...
// alpha_t (per channel, from the window start) and E_ts = alpha_{s+1} ...
// alpha_t (E_tt = 1), unrolling gives the block form
//   L_ts = beta_t rk_t rk_s sum_j k_tj k_sj E_tsj            s < t
//   P_ts = scale rq_t rk_s sum_j q_tj k_sj E_tsj             s <= t
//   X_t  = beta_t v_t - beta_t rk_t ((k_t . C_t) H)          (. : per channel)
//   U    = (I + L)^-1 X,   O_t = scale rq_t ((q_t . C_t) H) + (P U)_t,
// with raw rows k, q and their inverse norms rk, rq.  The decayed products
// E are formed by running products of alpha (never a quotient), so a zero
// decay is exact and nothing overflows.
//
// Records: the same records as gdn_kda.hip (raw key rows f32, ut_t = u_t rk_t,
// alpha per channel), so gdn_kda_commit replays them unchanged; the debug
// states are the replay of these records (decay multiply, then the fma, as
// commit does), so commit(m) is bitwise the debug state m - 1.
//
// Work: one 256-thread workgroup per (layer, lane, value head); wave w owns
// value columns 32w..32w+31 with the state layout of gdn_window_mfma.hip.
// The workgroup stages the window's key / query rows and decays in LDS and
// forms the decay-weighted Gram matrices L and P once: thread (s, cq) runs
// the running product E_ts over its 8 channels for t = s..15 and the 16
// channel slices meet by DPP row reductions.  Every wave then solves T
// = (I + L)^-1 in its own LDS tile and runs (k . C) H and (q . C) H on
// v_mfma_f32_16x16x32_bf16 with both operands split into bf16 hi + lo (three
// passes: hi hi, hi lo, lo hi), T X and P U on v_mfma_f32_16x16x4_f32.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <type_traits>

#include "gdn_mfma_util.h"
#include "gdn_window_common.h"

namespace gdn {
namespace wk {
using namespace wm;

constexpr int kD = 128;        // d_k = d_v
constexpr int kKS = kD / 32;   // k-steps of the bf16 products
constexpr int kTok = 16;       // window tokens
constexpr int kLS = 20;        // padded row of a 16 x 16 LDS matrix
constexpr int kUS = 33;        // padded row of a wave's ut tile

template <typename In>
struct KdaLds {
  __attribute__((aligned(16))) In k[kTok][kD];  // raw key rows (bf16 or f32)
  __attribute__((aligned(16))) In q[kTok][kD];  // raw query rows
  __attribute__((aligned(16))) float a[kTok][kD];     // alpha_t
  __attribute__((aligned(16))) float c[kTok][kD];     // C_t
  __attribute__((aligned(16))) float Lt[kTok * kLS];  // L transposed
  __attribute__((aligned(16))) float P[kTok * kLS];   // P[t][s]
  float beta[kTok], rk[kTok], rq[kTok];
};
// A fragments of (k . C) H and (q . C) H: [k-step][k hi, k lo, q hi, q lo]
// [lane], 16 KiB.  Without debug states they overlay the decays a and C
// (16 KiB, dead once L, P and the fragments are formed); the debug replay
// still reads a, so there they have their own space.
typedef u32x4 AFrags[kKS][4][kWave];
static_assert(sizeof(AFrags) == 2 * sizeof(float) * kTok * kD, "overlay size");
struct KdaWave {
  __attribute__((aligned(16))) float Ts[kTok * kLS];
  float Us[kTok * kUS];
};
// Windows of several blocks: E_t = alpha_{t+1} ... alpha_15 per channel (the
// decay from token t to the end of the block), and for debug states the
// token-by-token replay state carried from block to block (entry
// 2 (8 ks + e) + cs of thread tid).
struct KdaSuffix {
  __attribute__((aligned(16))) float e[kTok][kD];
};
struct KdaSeq {
  float s[2 * 8 * kKS][kBlock];
};

// Sum over the 16 lanes of a DPP row (every lane of the row gets it).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Eight bf16 of a raw row widened to f32 (exact).
__device__ __forceinline__ void widen8(u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    x[2 * p] = lo_f(w[p]);
    x[2 * p + 1] = hi_f(w[p]);
  }
}

template <bool DBG, bool MB, bool F32>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2)))
void mkda_kernel(const std::conditional_t<F32, float, uint16_t>* __restrict__ q,
                 const std::conditional_t<F32, float, uint16_t>* __restrict__ k,
                 const std::conditional_t<F32, float, uint16_t>* __restrict__ v,
                 const float* __restrict__ beta,
                 const float* __restrict__ g, const float* S,
                 float* __restrict__ o, float* __restrict__ rec_k,
                 float* __restrict__ rec_u, float* __restrict__ rec_a,
                 float* __restrict__ dbg, WinDims d, LaneTable tl, float scale,
                 int l2norm) {
  using In = std::conditional_t<F32, float, uint16_t>;
  constexpr int kEl = 16 / (int)sizeof(In);  // entries per 16-byte piece
  constexpr int kPc = F32 ? 2 : 1;           // pieces per thread and row
  __shared__ KdaLds<In> sh;
  __shared__ KdaWave wv[kWaves];
  // the replay of the debug states and between the blocks of a long
  // window reads the decays a: the fragments then have their own space
  __shared__ std::conditional_t<DBG || MB, AFrags, char> af_own;
  __shared__ std::conditional_t<MB, KdaSuffix, char> suf;
  __shared__ std::conditional_t<DBG && MB, KdaSeq, char> seq;
  AFrags& Af = *reinterpret_cast<AFrags*>(DBG || MB ? (void*)&af_own : (void*)&sh.a[0][0]);

  int item = xcd_item(blockIdx.x, gridDim.x);
  const int h = item % d.Hv;
  item /= d.Hv;
  const int lane = item % d.N;
  const int layer = item / d.N;
  const int T = table_byte(tl, lane);
  if (T == 0) return;

  const int tid = (int)threadIdx.x;
  const int w = uniform(tid / kWave);
  const int l = tid % kWave;
  const int g4 = l >> 4, n = l & 15;
  const int kh = h / d.group;
  const int c0 = 32 * w + 2 * n;  // this lane's columns c0, c0 + 1
  const size_t ll = (size_t)layer * d.N + lane;
  const size_t tok0 = ll * d.T;
  const size_t kq_step = (size_t)d.Hk * kD;  // per token: q, k, key records
  const size_t vo_step = (size_t)d.Hv * kD;  // per token: v, o, ut records
  const size_t g_step = (size_t)d.Hv * kD;   // per token: g, alpha records
  const In* __restrict__ k0 = k + (tok0 * d.Hk + kh) * kD;
  const In* __restrict__ q0 = q + (tok0 * d.Hk + kh) * kD;
  const In* __restrict__ v0 = v + (tok0 * d.Hv + h) * (size_t)kD;
  const float* __restrict__ g0 = g + (tok0 * d.Hv + h) * (size_t)kD;
  KdaWave& W = wv[w];

  // ---- window rows first (one 16-byte piece of k and q, two float4 of the
  // gates per thread, the value words), then the state, so that everything
  // before the state products overlaps its latency.  Tokens at or past T
  // read token 0 and become k = q = 0, alpha = 1, beta = 0.
  const int rt = tid >> 4, rp = tid & 15;  // row token, 16-byte piece
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  u32x4 kr[kPc], qr[kPc];  // pieces rp (and rp + 16 for f32 rows)
  f32x4 gr[2];
  float bl;
  float va[4], vb[4];  // values of the tokens 4 g4 + e at columns c0, c0 + 1
  // the rows of the block of tokens tb .. tb + Tb - 1
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
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int e = tid + kBlock * rep;  // float4 slot: token e / 32
      const int t = e >> 5;
      gr[rep] = *reinterpret_cast<const f32x4*>(
          g0 + (uint32_t)((tb + (t < Tb ? t : 0)) * g_step) + 4 * (e & 31));
    }
    bl = beta[(tok0 + tb + (tid < Tb ? tid : 0)) * d.Hv + h];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * g4 + e;
      const In* vp = v0 + (uint32_t)((tb + (t < Tb ? t : 0)) * vo_step) + c0;
      float x0, x1;
      if constexpr (F32) {
        const f32x2 x = *reinterpret_cast<const f32x2*>(vp);
        x0 = x[0];
        x1 = x[1];
      } else {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(vp);
        x0 = lo_f(x);
        x1 = hi_f(x);
      }
      va[e] = t < Tb ? x0 : 0.f;
      vb[e] = t < Tb ? x1 : 0.f;
    }
  };
  const int T0 = MB ? (T < kTok ? T : kTok) : T;
  load_rows(0, T0);

  const uint32_t soff = (uint32_t)(8 * g4 * kD + c0) * 4u;
  const auto srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(S) + (ll * d.Hv + h) * (size_t)kD * kD, 0,
      kD * kD * (int)sizeof(float), kBufWord3);
  f32x2 s2[kKS][8];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      s2[ks][e] = __builtin_bit_cast(
          f32x2, __builtin_amdgcn_raw_buffer_load_b64(
                     srs, soff, (32 * ks + e) * kD * 4, kNT));
  __builtin_amdgcn_sched_barrier(0);

  // ---- stage the rows, the decays and beta; write the key and decay records
  auto stage_rows = [&](int tb, int Tb) {
    const bool rv = rt < Tb;
#pragma unroll
    for (int p = 0; p < kPc; ++p) {
      *reinterpret_cast<u32x4*>(&sh.k[rt][kEl * (rp + 16 * p)]) = kr[p];
      *reinterpret_cast<u32x4*>(&sh.q[rt][kEl * (rp + 16 * p)]) = qr[p];
    }
    if (rv && h % d.group == 0) {
      float* __restrict__ dst = rec_k + (tok0 * d.Hk + kh) * kD +
                                (uint32_t)((tb + rt) * kq_step);
      if constexpr (F32) {
#pragma unroll
        for (int p = 0; p < kPc; ++p)
          *reinterpret_cast<u32x4*>(dst + kEl * (rp + 16 * p)) = kr[p];
      } else {
        float kx[8];
        widen8(kr[0], kx);
        reinterpret_cast<float4*>(dst + 8 * rp)[0] = make_float4(kx[0], kx[1], kx[2], kx[3]);
        reinterpret_cast<float4*>(dst + 8 * rp)[1] = make_float4(kx[4], kx[5], kx[6], kx[7]);
      }
    }
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int e = tid + kBlock * rep;
      const int t = e >> 5;
      f32x4 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = t < Tb ? __expf(gr[rep][i]) : 1.0f;
      *reinterpret_cast<f32x4*>(&sh.a[t][4 * (e & 31)]) = a;
      if (t < Tb)
        *reinterpret_cast<f32x4*>(rec_a + (tok0 * d.Hv + h) * (size_t)kD +
                                  (uint32_t)((tb + t) * g_step) + 4 * (e & 31)) = a;
    }
    if (tid < kTok) sh.beta[tid] = tid < Tb ? bl : 0.f;
  };
  stage_rows(0, T0);
  __syncthreads();

  // the window in blocks of kTok tokens (one block unless MB), each from
  // the held state the blocks before it leave
  for (int tb = 0;; tb += kTok) {
    const int Tb = MB ? (T - tb < kTok ? T - tb : kTok) : T;
    if (MB && tb > 0) {
      load_rows(tb, Tb);
      __syncthreads();  // every wave is done with the previous block
      stage_rows(tb, Tb);
      __syncthreads();
    }
    // ---- C_t per channel (threads 0..127) and the inverse norms (threads
    // 128..255: eight per token, 16 entries each)
    if (tid < kD) {
      float cc = 1.0f;
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        cc = cc * sh.a[t][tid];
        sh.c[t][tid] = cc;
      }
      if constexpr (MB) {
        float ee = 1.0f;
#pragma unroll
        for (int t = kTok - 1; t >= 0; --t) {
          suf.e[t][tid] = ee;
          ee = ee * sh.a[t][tid];
        }
      }
    } else {
      const int u = tid - kD, t = u >> 3, pc = u & 7;

      float skk = 0.f, sqq = 0.f;
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        float kx[8], qx[8];
        row8(&sh.k[t][16 * pc + 8 * hlf], kx);
        row8(&sh.q[t][16 * pc + 8 * hlf], qx);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          skk = __builtin_fmaf(kx[i], kx[i], skk);
          sqq = __builtin_fmaf(qx[i], qx[i], sqq);
        }
      }
      // eight consecutive lanes: two quad swaps and the half-row mirror
      skk += dpp<0xB1>(skk);
      sqq += dpp<0xB1>(sqq);
      skk += dpp<0x4E>(skk);
      sqq += dpp<0x4E>(sqq);
      skk += dpp<0x141>(skk);
      sqq += dpp<0x141>(sqq);
      if (pc == 0) {
        sh.rk[t] = l2norm ? __builtin_amdgcn_rsqf(skk + 1e-6f) : 1.0f;
        sh.rq[t] = l2norm ? __builtin_amdgcn_rsqf(sqq + 1e-6f) : 1.0f;
      }
    }
    __syncthreads();

    // ---- L and P: thread (s, cq) runs E_ts over channels 8 cq .. 8 cq + 7 for
    // t = s .. 15; the 16 channel slices of a row meet by a DPP row sum.  Wave
    // w holds the rows s = 4w .. 4w + 3, so its loop starts at t = 4w (every
    // entry before that is above the diagonal: P's are zeroed here, L's are
    // never read)
    {
      const int s = tid >> 4, cq = tid & 15;
      if (cq == 0)
        for (int t = 0; t < 4 * w; ++t) sh.P[t * kLS + s] = 0.f;
      float ksv[8];
      row8(&sh.k[s][8 * cq], ksv);
      float E[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) E[i] = 1.0f;
      const float rks = sh.rk[s];
      // rows past the block's tokens: L and P stay exactly 0 (T is then the
      // identity there and U, X vanish), without their running products
      if (cq == 0)
        for (int t = Tb > 4 * w ? Tb : 4 * w; t < kTok; ++t) {
          sh.Lt[s * kLS + t] = 0.f;
          sh.P[t * kLS + s] = 0.f;
        }
#pragma unroll 1
      for (int t = 4 * w; t < Tb; ++t) {
        float kt[8], qt[8];
        row8(&sh.k[t][8 * cq], kt);
        row8(&sh.q[t][8 * cq], qt);
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(&sh.a[t][8 * cq]);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(&sh.a[t][8 * cq + 4]);
        const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        float aL = 0.f, aP = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          E[i] = t > s ? E[i] * av[i] : E[i];
          const float ke = ksv[i] * E[i];
          aL = __builtin_fmaf(kt[i], ke, aL);
          aP = __builtin_fmaf(qt[i], ke, aP);
        }
        aL = row_sum16(aL);
        aP = row_sum16(aP);
        if (cq == 0) {
          const float lv = sh.beta[t] * sh.rk[t] * rks * aL;
          sh.Lt[s * kLS + t] = t > s ? lv : 0.f;  // L[t][s]
          const float pv = scale * sh.rq[t] * rks * aP;
          sh.P[t * kLS + s] = t >= s ? pv : 0.f;
        }
      }
    }
    // ---- the decayed key and query rows of token n (entries 32 ks + 8 g4 ..
    // + 7) split into bf16 hi + lo: the A fragments of (k . C) H and (q . C) H
    // are the same for every wave, so wave w forms k-step w once for all
    u32x4 af[4];
    {
      const int j0 = 32 * w + 8 * g4;
      float kx[8], qx[8];
      row8(&sh.k[n][j0], kx);
      row8(&sh.q[n][j0], qx);
      const f32x4 ca = *reinterpret_cast<const f32x4*>(&sh.c[n][j0]);
      const f32x4 cb = *reinterpret_cast<const f32x4*>(&sh.c[n][j0 + 4]);
      const float cv[8] = {ca[0], ca[1], ca[2], ca[3], cb[0], cb[1], cb[2], cb[3]};
      uint32_t kh4[4], kl4[4], qh4[4], ql4[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        split2(kx[2 * p] * cv[2 * p], kx[2 * p + 1] * cv[2 * p + 1], kh4[p], kl4[p]);
        split2(qx[2 * p] * cv[2 * p], qx[2 * p + 1] * cv[2 * p + 1], qh4[p], ql4[p]);
      }
      af[0] = u32x4{kh4[0], kh4[1], kh4[2], kh4[3]};
      af[1] = u32x4{kl4[0], kl4[1], kl4[2], kl4[3]};
      af[2] = u32x4{qh4[0], qh4[1], qh4[2], qh4[3]};
      af[3] = u32x4{ql4[0], ql4[1], ql4[2], ql4[3]};
    }
    __syncthreads();  // L, P complete; a and C read for the last time
#pragma unroll
    for (int x = 0; x < 4; ++x) Af[w][x][l] = af[x];
    __syncthreads();

    // ---- T = (I + L)^-1 in each wave's tile (lane n < 16 of group 0 solves
    // column n by right-looking substitution)
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
          acc[r] = __builtin_fmaf(sh.Lt[x * kLS + r], tx, acc[r]);
      }
    }
    wave_lds_sync();
    const f32x4 TA = *reinterpret_cast<const f32x4*>(&W.Ts[n * kLS + 4 * g4]);
    const f32x4 PA = *reinterpret_cast<const f32x4*>(&sh.P[n * kLS + 4 * g4]);

    // ---- (k . C) H and (q . C) H: per k-step, the decayed rows of token n
    // (entries 32 ks + 8 g4 .. + 7) and the state split into bf16 hi + lo
    f32x4 KH[2], QH[2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      KH[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
      QH[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const u32x4 KAh = Af[ks][0][l], KAl = Af[ks][1][l];
      const u32x4 QAh = Af[ks][2][l], QAl = Af[ks][3][l];
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
      KH[0] = mma_bf16(KAh, H0, KH[0]);
      KH[1] = mma_bf16(KAh, H1, KH[1]);
      QH[0] = mma_bf16(QAh, H0, QH[0]);
      QH[1] = mma_bf16(QAh, H1, QH[1]);
      KH[0] = mma_bf16(KAh, L0, KH[0]);
      KH[1] = mma_bf16(KAh, L1, KH[1]);
      QH[0] = mma_bf16(QAh, L0, QH[0]);
      QH[1] = mma_bf16(QAh, L1, QH[1]);
      KH[0] = mma_bf16(KAl, H0, KH[0]);
      KH[1] = mma_bf16(KAl, H1, KH[1]);
      QH[0] = mma_bf16(QAl, H0, QH[0]);
      QH[1] = mma_bf16(QAl, H1, QH[1]);
    }

    // ---- X, U = T X, O = diag(scale rq) (q . C) H + P U, ut = U rk
    f32x4 X[2];
    float rke[4], sqe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * g4 + e;
      const float bt = sh.beta[t];
      rke[e] = sh.rk[t];
      sqe[e] = scale * sh.rq[t];
      const float xb = bt * rke[e];
      const float x0 = __builtin_fmaf(-xb, KH[0][e], bt * va[e]);
      const float x1 = __builtin_fmaf(-xb, KH[1][e], bt * vb[e]);
      X[0][e] = t < Tb ? x0 : 0.f;
      X[1][e] = t < Tb ? x1 : 0.f;
    }
    f32x4 U[2], O[2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      U[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) U[cs] = mma_f32(TA[e], X[cs][e], U[cs]);
#pragma unroll
      for (int e = 0; e < 4; ++e) O[cs][e] = sqe[e] * QH[cs][e];
#pragma unroll
      for (int e = 0; e < 4; ++e) O[cs] = mma_f32(PA[e], U[cs][e], O[cs]);
    }
    float* __restrict__ o0 = o + ((tok0 + tb) * d.Hv + h) * (size_t)kD;
    float* __restrict__ u0 = rec_u + ((tok0 + tb) * d.Hv + h) * (size_t)kD;
    float ut[2][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * g4 + e;
      ut[0][e] = U[0][e] * rke[e];
      ut[1][e] = U[1][e] * rke[e];
      if (t < Tb) {
        const uint32_t off = (uint32_t)(t * vo_step) + c0;
        // outputs are not read again by this path: nontemporal stores
        __builtin_nontemporal_store(f32x2{O[0][e], O[1][e]},
                                    reinterpret_cast<f32x2*>(o0 + off));
        *reinterpret_cast<float2*>(u0 + off) = make_float2(ut[0][e], ut[1][e]);
      }
    }

    // ---- debug states: the records replayed token by token on the start
    // state with commit's operations (decay multiply, then the fma).  In a
    // window of several blocks the replay runs on its own copy of the state,
    // carried from block to block through LDS (the held state moves on by
    // the block product below).
    const bool more = MB && tb + kTok < T;
    if constexpr (DBG) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        W.Us[(4 * g4 + e) * kUS + 2 * n] = ut[0][e];
        W.Us[(4 * g4 + e) * kUS + 2 * n + 1] = ut[1][e];
      }
      wave_lds_sync();
      auto replay = [&](f32x2 (&st)[kKS][8]) {
#pragma unroll 1
        for (int t = 0; t < Tb; ++t) {
          const float ua = W.Us[t * kUS + 2 * n], ub = W.Us[t * kUS + 2 * n + 1];
          float* __restrict__ dp =
              dbg + ((tok0 + tb + t) * d.Hv + h) * (size_t)kD * kD;
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) {
            const int j0 = 32 * ks + 8 * g4;
            float kx[8];
            row8(&sh.k[t][j0], kx);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float a = sh.a[t][j0 + e];
              st[ks][e][0] = st[ks][e][0] * a;
              st[ks][e][1] = st[ks][e][1] * a;
              st[ks][e][0] = __builtin_fmaf(ua, kx[e], st[ks][e][0]);
              st[ks][e][1] = __builtin_fmaf(ub, kx[e], st[ks][e][1]);
              *reinterpret_cast<f32x2*>(dp + (size_t)(j0 + e) * kD + c0) = st[ks][e];
            }
          }
        }
      };
      if constexpr (MB) {
        f32x2 sd[kKS][8];
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sd[ks][e] = tb == 0 ? s2[ks][e]
                                : f32x2{seq.s[2 * (8 * ks + e)][tid],
                                        seq.s[2 * (8 * ks + e) + 1][tid]};
        replay(sd);
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
        replay(s2);
      }
    }
    // ---- the held state after the block, for the next one: the closed form
    // of the block's decay-then-write steps, St = diag(C_15) St + sum_t
    // diag(E_t) k_t ut_t^T, the sum as one product on
    // v_mfma_f32_16x16x32_bf16 with the decayed key rows k_t . E_t as the
    // A operand and the records ut as B, each in three bf16 parts (the six
    // part products of order at most 2^-16).  The 32 k-slots of lane group g
    // carry tokens 4 g .. 4 g + 3 twice, once per operand part; result row
    // 4 g + i of tile (ks, half) is state row 32 ks + 8 g + 4 half + i, the
    // entries the lane holds.  Decays enter only as running products, so
    // alpha = 0 channels stay exact.
    if constexpr (MB) if (more) {
      u32x4 B1[2], B2[2];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        uint32_t ph[2], pm[2], pl[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float a = ut[cs][2 * i], b = ut[cs][2 * i + 1];
          split2(a, b, ph[i], pm[i]);
          const f32x2 y = {a - lo_f(ph[i]) - lo_f(pm[i]),
                           b - hi_f(ph[i]) - hi_f(pm[i])};
          pl[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
        }
        B1[cs] = u32x4{ph[0], ph[1], pm[0], pm[1]};  // [h, m]
        B2[cs] = u32x4{pl[0], pl[1], ph[0], ph[1]};  // [l, h]
      }
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        // the block's decay of the lane's state rows 32 ks + 8 g4 + e
        const f32x4 c0v = *reinterpret_cast<const f32x4*>(&sh.c[kTok - 1][32 * ks + 8 * g4]);
        const f32x4 c1v = *reinterpret_cast<const f32x4*>(&sh.c[kTok - 1][32 * ks + 8 * g4 + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s2[ks][e][0] *= c0v[e];
          s2[ks][e][1] *= c0v[e];
          s2[ks][e + 4][0] *= c1v[e];
          s2[ks][e + 4][1] *= c1v[e];
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          // key entry kx of tokens 4 g4 + j, decayed to the block's end
          const int kx = 32 * ks + 8 * (n >> 2) + 4 * half + (n & 3);
          uint32_t ah[2], am[2], al[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int t0 = 4 * g4 + 2 * i;
            float ka, kb;
            if constexpr (F32) {
              ka = sh.k[t0][kx];
              kb = sh.k[t0 + 1][kx];
            } else {
              ka = lo_f((uint32_t)sh.k[t0][kx]);
              kb = lo_f((uint32_t)sh.k[t0 + 1][kx]);
            }
            const float a = ka * suf.e[t0][kx], b = kb * suf.e[t0 + 1][kx];
            split2(a, b, ah[i], am[i]);
            const f32x2 y = {a - lo_f(ah[i]) - lo_f(am[i]),
                             b - hi_f(ah[i]) - hi_f(am[i])};
            al[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
          }
          const u32x4 Ahh = {ah[0], ah[1], ah[0], ah[1]};
          const u32x4 Amm = {am[0], am[1], am[0], am[1]};
          const u32x4 Ahl = {ah[0], ah[1], al[0], al[1]};
          f32x4 D[2];
#pragma unroll
          for (int cs = 0; cs < 2; ++cs) {
            D[cs] = mma_bf16(Ahh, B1[cs], f32x4{0.f, 0.f, 0.f, 0.f});
            D[cs] = mma_bf16(Amm, B1[cs], D[cs]);
            D[cs] = mma_bf16(Ahl, B2[cs], D[cs]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s2[ks][4 * half + i][0] += D[0][i];
            s2[ks][4 * half + i][1] += D[1][i];
          }
        }
      }
    }
    if (!more) break;

  }
}

template <bool DBG, bool MB, bool F32>
static hipError_t launch_t(const WinDims& w, const LaneTable& tl,
                           const void* q, const void* k, const void* v,
                           const float* beta, const float* g, const float* S,
                           float* o, float* rk, float* ru, float* ra,
                           float* dbg, float scale, int l2, hipStream_t st) {
  const int blocks = w.NL * w.N * w.Hv;
  using In = std::conditional_t<F32, float, uint16_t>;
  return launch(mkda_kernel<DBG, MB, F32>, dim3(blocks), dim3(kBlock), st,
                (const In*)q, (const In*)k, (const In*)v,
                beta, g, S, o, rk, ru, ra, dbg, w, tl, scale, l2);
}

}  // namespace wk

bool mkda_eligible(const gdn_dims& d, int in_dtype, const void* q,
                   const void* k, const void* v, const float* g,
                   const float* S, const float* o, const float* dbg) {
  auto al = [](const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; };
  return (in_dtype == GDN_BF16 || in_dtype == GDN_F32) && d.d_k == wk::kD &&
         d.d_v == wk::kD && d.t_max <= GDN_MAX_T && al(q, 16) && al(k, 16) &&
         al(v, in_dtype == GDN_F32 ? 8 : 4) &&
         al(g, 16) && al(S, 8) && al(o, 8) && (dbg == nullptr || al(dbg, 8));
}

template <bool F32>
static hipError_t launch_kda(const WinDims& w, const LaneTable& tl,
                             const void* q, const void* k, const void* v,
                             const float* beta, const float* g, const float* S,
                             float* o, float* rk, float* ru, float* ra,
                             float* dbg, float scale, int l2, hipStream_t st) {
  if (w.T > wk::kTok)  // windows of several blocks
    return dbg ? wk::launch_t<true, true, F32>(w, tl, q, k, v, beta, g, S, o,
                                               rk, ru, ra, dbg, scale, l2, st)
               : wk::launch_t<false, true, F32>(w, tl, q, k, v, beta, g, S, o,
                                                rk, ru, ra, dbg, scale, l2, st);
  return dbg ? wk::launch_t<true, false, F32>(w, tl, q, k, v, beta, g, S, o, rk,
                                              ru, ra, dbg, scale, l2, st)
             : wk::launch_t<false, false, F32>(w, tl, q, k, v, beta, g, S, o,
                                               rk, ru, ra, dbg, scale, l2, st);
}

hipError_t launch_mkda(const WinDims& w, const LaneTable& tl, bool f32,
                       const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* S,
                       float* o, float* rk, float* ru, float* ra, float* dbg,
                       float scale, int l2, hipStream_t st) {
  return f32 ? launch_kda<true>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg,
                                scale, l2, st)
             : launch_kda<false>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg,
                                 scale, l2, st);
}

}  // namespace gdn
