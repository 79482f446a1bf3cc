// gdn_kda.hip -- verify and ReplaySSM commit for the per-channel-decay
// sibling of the gated delta rule (KDA, Kimi Delta Attention of Kimi Linear,
// 2025; the NInfer technical review, blog.123qwe.co.kr post 4624, names its
// recurrent state beside GDN's and a kda_replay op contract).
//
// Per (layer, lane, value head), state S (d_v x d_k), window token t:
//   alpha_t = exp(g_t)                     (a d_k vector: one decay per key channel)
//   S'      = S diag(alpha_t)              (column j scaled by alpha_tj)
//   u_t     = beta_t (v_t - S' khat_t)
//   S_t     = S' + u_t khat_t^T
//   o_t     = scale * S_t qhat_t
// A per-channel decay does not factor out of the state as one scale, so the
// state is decayed in place: per element and token one multiply (decay), one
// FMA for the prediction, one for the output and one for the write.  With
// raw k and q (norms folded into scalars, as in gdn_window.hip):
//   St_ij <- St_ij * alpha_j
//   P_i = sum_j St_ij k_j ;  p_i = rk P_i ;  ut_i = beta (v_i - p_i) rk
//   o_i = scale rq (sum_j St_ij q_j + ut_i (k . q))   (state before the write)
//   St_ij <- fma(ut_i, k_j, St_ij)
// Records per token: the raw key row (f32, per key head), ut (f32, per value
// head and column) and alpha (f32, per value head and channel).  Commit
// replays the same multiply and FMA per element on exactly these values, so
// commit(m) is bitwise the state verify held after token m (the ReplaySSM
// requirement of the review's section "Architecture 3").
//
// Decomposition as gdn_window.hip: one 256-thread workgroup per (layer,
// lane, value head, block of 64 value columns), wave w owns key rows
// 32w..32w+31 of d_k = 128 (lane = column), keys and queries through scalar
// loads.  The decays of a wave's rows differ per row but are the same for
// all its lanes: lanes 0..R-1 compute them one token ahead (exp of the
// loaded gate) into LDS, where the next token reads them back as broadcasts
// after the token's exchange barrier.
#include "gdn_window_common.h"

namespace gdn {

struct KdaRecLayout {
  size_t k, u, alpha, total;
};

static KdaRecLayout kda_rec_layout(const gdn_dims& d) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  KdaRecLayout r;
  const size_t ntok = (size_t)d.n_layers * d.n_lanes * d.t_max;
  r.k = 0;
  r.u = al(ntok * d.h_k * d.d_k * sizeof(float));
  r.alpha = r.u + al(ntok * d.h_v * d.d_v * sizeof(float));
  r.total = r.alpha + al(ntok * d.h_v * d.d_k * sizeof(float));
  return r;
}

// Per-token scalars of a KDA window (LDS).
struct KdaScalars {
  float rk, f3, beta, kq;  // f3 = scale * rq; kq = k_t . q_t (raw)
};

// Six waves per SIMD (at most 80 VGPRs); the variant that writes every
// intermediate state gets two (60 spilled VGPRs at 80, 18 at 128).
template <int DK, bool DBG, typename TIn>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(DBG ? 2 : 6)))
void kda_verify_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ g, const float* __restrict__ S,
    float* __restrict__ o, float* __restrict__ rec_k,
    float* __restrict__ rec_u, float* __restrict__ rec_a,
    float* __restrict__ dbg, WinDims d, LaneTable tl, float scale,
    int l2norm) {
  constexpr int R = DK / kWaves;
  __shared__ KdaScalars sc[GDN_MAX_T];
  __shared__ float2 red[2][kWaves][kWave];
  __shared__ __align__(16) float al[2][kWaves][R];  // decays of token t (and t+1)

  int item = xcd_item(blockIdx.x, gridDim.x);
  const int cb = item % d.ncb;
  item /= d.ncb;
  const int h = item % d.Hv;
  item /= d.Hv;
  const int lane = item % d.N;
  const int layer = item / d.N;
  const int T = tl.v[lane];
  if (T == 0) return;

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
  const size_t kq_step = (size_t)d.Hk * DK;   // per token, q/k
  const size_t vo_step = (size_t)d.Hv * dv;   // per token, v/o/u
  const size_t g_step = (size_t)d.Hv * DK;    // per token, g/alpha
  const TIn* __restrict__ k0 = k + ((ll * d.T) * d.Hk + kh) * (size_t)DK;
  const TIn* __restrict__ q0 = q + ((ll * d.T) * d.Hk + kh) * (size_t)DK;
  const TIn* __restrict__ v0 = v + ((ll * d.T) * d.Hv + h) * dv;
  const float* __restrict__ g0 = g + ((ll * d.T) * d.Hv + h) * (size_t)DK;
  float* __restrict__ a0r = rec_a + ((ll * d.T) * d.Hv + h) * (size_t)DK;
  float* __restrict__ o0 = o + ((ll * d.T) * d.Hv + h) * dv;
  float* __restrict__ u0 = rec_u + ((ll * d.T) * d.Hv + h) * dv;

  float s[R];  // state entries (rows j0..j0+R-1, column i)
  {
    const float* __restrict__ Sh = S + ((ll * d.Hv + h) * (size_t)DK + j0) * dv;
#pragma unroll
    for (int r = 0; r < R; ++r)
      s[r] = __builtin_nontemporal_load(Sh + (uint32_t)(r * d.dv + ic));
  }

  // ---- prologue: norms, k . q, key records (16 lanes per token)
  for (int base = 4 * w; base < T; base += 16) {
    const int t = base + x / 16;
    const int tt = t < T ? t : T - 1;
    const int sub = x % 16;
    float kk[8], skk, sqq, skq;
    row_moments<TIn>(k0 + tt * kq_step, q0 + tt * kq_step, DK, sub, kk, skk,
                     sqq, skq);
    if (t < T) {
      if (sub == 0) {
        const size_t gi = (ll * d.T + t) * d.Hv + h;
        KdaScalars z;
        z.rk = l2norm ? inv_norm(skk) : 1.0f;
        z.f3 = scale * (l2norm ? inv_norm(sqq) : 1.0f);
        z.beta = beta[gi];
        z.kq = skq;
        sc[t] = z;
      }
      if (key_writer && 8 * sub < DK) {
        float4* dst = reinterpret_cast<float4*>(
            rec_k + ((ll * d.T + t) * d.Hk + kh) * (size_t)DK + 8 * sub);
        dst[0] = make_float4(kk[0], kk[1], kk[2], kk[3]);
        dst[1] = make_float4(kk[4], kk[5], kk[6], kk[7]);
      }
    }
  }
  // decays of token 0 (lanes 0..R-1 of every wave: its own rows; the other
  // lanes load copies, so that no load sits in a divergent branch)
  {
    const float a = __expf(g0[j0 + x % R]);
    if (x < R) {
      al[0][w][x] = a;
      if (cb == 0) a0r[j0 + x] = a;
    }
  }
  // gate of token 1, in flight during token 0
  float g_next = g0[(T > 1 ? 1 : 0) * g_step + j0 + x % R];
  __syncthreads();

  RowWords<TIn, R> kw, qw;
  kw.load(k0, j0);
  qw.load(q0, j0);
  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    const float vi = load_in(v0 + t * vo_step, (uint32_t)ic);
    const KdaScalars z = sc[t];
    float av[R];
#pragma unroll
    for (int r4 = 0; r4 < R / 4; ++r4) {
      const float4 a4 = *reinterpret_cast<const float4*>(&al[buf][w][4 * r4]);
      av[4 * r4 + 0] = a4.x;
      av[4 * r4 + 1] = a4.y;
      av[4 * r4 + 2] = a4.z;
      av[4 * r4 + 3] = a4.w;
    }
    float kv[R];
    float pa = 0.f, pb = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = s[r] * av[r];  // S' = S diag(alpha)
      kv[r] = kw.at(r);
      pa = __builtin_fmaf(s[r], kv[r], pa);
      pb = __builtin_fmaf(s[r], qw.at(r), pb);
    }
    red[buf][w][x] = make_float2(pa, pb);
    // decays of the next token, published by this token's barrier
    {
      const float a = __expf(g_next);
      if (x < R && t + 1 < T) {
        al[buf ^ 1][w][x] = a;
        if (cb == 0) a0r[(t + 1) * g_step + j0 + x] = a;
      }
      g_next = g0[(t + 2 < T ? t + 2 : T - 1) * g_step + j0 + x % R];
    }
    __syncthreads();
    const float2 r0 = red[buf][0][x], r1 = red[buf][1][x];
    const float2 r2 = red[buf][2][x], r3 = red[buf][3][x];
    if (t + 1 < T) {
      kw.load(k0 + (t + 1) * kq_step, j0);
      qw.load(q0 + (t + 1) * kq_step, j0);
    }
    const float P = (r0.x + r1.x) + (r2.x + r3.x);
    const float PQ = (r0.y + r1.y) + (r2.y + r3.y);
    const float p = z.rk * P;
    const float ut = (z.beta * (vi - p)) * z.rk;
    const int owner = t % kWaves;
    if (w == owner && act) {
      u0[t * vo_step + (uint32_t)i] = ut;
      __builtin_nontemporal_store(z.f3 * __builtin_fmaf(ut, z.kq, PQ),
                                  o0 + t * vo_step + (uint32_t)i);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = __builtin_fmaf(ut, kv[r], s[r]);
    if (DBG && act) {
      float* __restrict__ dp =
          dbg + (((ll * d.T + t) * d.Hv + h) * (size_t)DK + j0) * dv;
#pragma unroll
      for (int r = 0; r < R; ++r) dp[(uint32_t)(r * d.dv + i)] = s[r];
    }
  }
}

template <int DK>
// Six waves per SIMD: the LDS stage lets the compiler hoist every row read
// of a token, which at the default limit halves the occupancy.
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void kda_commit_kernel(
    const float* __restrict__ rec_k, const float* __restrict__ rec_u,
    const float* __restrict__ rec_a, float* __restrict__ S, WinDims d,
    CommitTable ct) {
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
  const float* __restrict__ a0 = rec_a + ((ll * d.T) * d.Hv + h) * (size_t)DK;
  const size_t kq_step = (size_t)d.Hk * DK, vo_step = (size_t)d.Hv * dv;
  const size_t g_step = (size_t)d.Hv * DK;

  float s[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    s[r] = __builtin_nontemporal_load(Sh + (uint32_t)(r * d.dv + ic));
  // The key rows (this workgroup's key head) and decay rows (its value
  // head) of up to kStageTok tokens are staged in LDS with one cooperative
  // load and one wait; the replay then reads them as broadcasts.  ut of
  // token t+1 is requested before token t is applied.  The operations and
  // their order per entry are those of the verify's state update.
  constexpr int kStageTok = 16;
  constexpr int kRow4 = DK / 4;                        // float4 per row
  constexpr int kRep = 2 * kStageTok * kRow4 / kBlock;  // loads per thread
  static_assert(2 * kStageTok * kRow4 % kBlock == 0, "staging split");
  __shared__ float4 st_k[kStageTok][kRow4];
  __shared__ float4 st_a[kStageTok][kRow4];
  const int tid = (int)threadIdx.x;
  float ut = u0[(uint32_t)ic];
  for (int t0 = 0; t0 < m; t0 += kStageTok) {
    const int nb = m - t0 < kStageTok ? m - t0 : kStageTok;
    float4 reg[kRep];
#pragma unroll
    for (int rep = 0; rep < kRep; ++rep) {
      const int e = tid + rep * kBlock;
      const int which = e / (kStageTok * kRow4);  // 0: key row, 1: decay row
      const int idx = e % (kStageTok * kRow4);
      int tok = idx / kRow4;
      tok = tok < nb ? tok : nb - 1;
      const int c4 = idx % kRow4;
      const float* src = which ? a0 + (size_t)(t0 + tok) * g_step
                               : k0 + (size_t)(t0 + tok) * kq_step;
      reg[rep] = reinterpret_cast<const float4*>(src)[c4];
    }
#pragma unroll
    for (int rep = 0; rep < kRep; ++rep) {
      const int e = tid + rep * kBlock;
      const int which = e / (kStageTok * kRow4);
      const int idx = e % (kStageTok * kRow4);
      (which ? &st_a[0][0] : &st_k[0][0])[idx] = reg[rep];
    }
    __syncthreads();
    for (int t = 0; t < nb; ++t) {
      const int tg = t0 + t;
      const int nt = tg + 1 < m ? tg + 1 : tg;
      const float ut_n = u0[nt * vo_step + (uint32_t)ic];
      const float4* kr = &st_k[t][j0 / 4];
      const float4* ar = &st_a[t][j0 / 4];
#pragma unroll
      for (int r4 = 0; r4 < R / 4; ++r4) {
        const float4 kk = kr[r4], aa = ar[r4];
        s[4 * r4 + 0] = __builtin_fmaf(ut, kk.x, s[4 * r4 + 0] * aa.x);
        s[4 * r4 + 1] = __builtin_fmaf(ut, kk.y, s[4 * r4 + 1] * aa.y);
        s[4 * r4 + 2] = __builtin_fmaf(ut, kk.z, s[4 * r4 + 2] * aa.z);
        s[4 * r4 + 3] = __builtin_fmaf(ut, kk.w, s[4 * r4 + 3] * aa.w);
      }
      ut = ut_n;
    }
    __syncthreads();  // the next batch overwrites the stage
  }
  if (act) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      __builtin_nontemporal_store(s[r], Sh + (uint32_t)(r * d.dv + i));
  }
}

template <int DK, bool DBG, typename TIn>
static hipError_t launch_kda_verify(const WinDims& w, const LaneTable& tl,
                                    const void* q, const void* k, const void* v,
                                    const float* beta, const float* g,
                                    const float* S, float* o, float* rk,
                                    float* ru, float* ra, float* dbg,
                                    float scale, int l2, hipStream_t st) {
  const int blocks = w.NL * w.N * w.Hv * w.ncb;
  return launch(kda_verify_kernel<DK, DBG, TIn>, dim3(blocks), dim3(kBlock), st,
                (const TIn*)q, (const TIn*)k, (const TIn*)v, beta, g, S, o, rk,
                ru, ra, dbg, w, tl, scale, l2);
}

}  // namespace gdn

using namespace gdn;

extern "C" size_t gdn_kda_records_bytes(const gdn_dims* dims) {
  if (check_dims(dims) != GDN_OK || dims->d_k != 128) return 0;
  return kda_rec_layout(*dims).total;
}

extern "C" int gdn_kda_verify(const gdn_dims* dims, const int32_t* t_lane,
                              const void* q, const void* k, const void* v,
                              int in_dtype, const float* beta, const float* g,
                              const float* S, float* o, void* records,
                              float* dbg_states, float scale, int flags,
                              void* stream) {
  int rc = check_dims(dims);
  if (rc != GDN_OK) return rc;
  if (dims->d_k != 128)
    return fail(GDN_EUNSUPPORTED, "gdn_kda_verify: d_k must be 128");
  if (!t_lane || !q || !k || !v || !beta || !g || !S || !o || !records)
    return fail(GDN_EINVAL, "gdn_kda_verify: required pointer is NULL");
  if (in_dtype != GDN_BF16 && in_dtype != GDN_F32)
    return fail(GDN_EINVAL, "gdn_kda_verify: unknown in_dtype");
  if (flags & ~(GDN_FLAG_L2NORM_QK | GDN_FLAG_TOKENWISE))
    return fail(GDN_EINVAL, "gdn_kda_verify: unknown flag bits");
  if (misaligned(q, 4) || misaligned(k, 4) ||
      misaligned(v, in_dtype == GDN_BF16 ? 2 : 4) || misaligned(beta, 4) ||
      misaligned(g, 4) || misaligned(S, 4) || misaligned(o, 4) ||
      misaligned(records, 256) || (dbg_states && misaligned(dbg_states, 4)))
    return fail(GDN_EINVAL, "gdn_kda_verify: misaligned pointer");
  const gdn_dims& d = *dims;
  LaneTable tl;
  memset(&tl, 0, sizeof(tl));
  int any = 0;
  for (int n = 0; n < d.n_lanes; ++n) {
    if (t_lane[n] < 0 || t_lane[n] > d.t_max)
      return fail(GDN_EINVAL, "gdn_kda_verify: t_lane out of 0..t_max");
    tl.v[n] = (uint8_t)t_lane[n];
    any |= t_lane[n];
  }
  if (!any) return GDN_OK;
  const WinDims w = win_dims(d);
  const KdaRecLayout L = kda_rec_layout(d);
  char* rb = (char*)records;
  float* rk = (float*)(rb + L.k);
  float* ru = (float*)(rb + L.u);
  float* ra = (float*)(rb + L.alpha);
  hipStream_t st = (hipStream_t)stream;
  const int l2 = (flags & GDN_FLAG_L2NORM_QK) ? 1 : 0;
  hipError_t e;
  if (!(flags & GDN_FLAG_TOKENWISE) &&
      mkda_eligible(d, in_dtype, q, k, v, g, S, o, dbg_states))
    e = launch_mkda(w, tl, in_dtype == GDN_F32, q, k, v, beta, g, S, o, rk, ru,
                    ra, dbg_states, scale, l2, st);
  else if (in_dtype == GDN_BF16)
    e = dbg_states
            ? launch_kda_verify<128, true, uint16_t>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg_states, scale, l2, st)
            : launch_kda_verify<128, false, uint16_t>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, nullptr, scale, l2, st);
  else
    e = dbg_states
            ? launch_kda_verify<128, true, float>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg_states, scale, l2, st)
            : launch_kda_verify<128, false, float>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, nullptr, scale, l2, st);
  return hip_status(e, "gdn_kda_verify launch");
}

extern "C" int gdn_kda_commit(const gdn_dims* dims, const int32_t* m_lane,
                              const int32_t* t_lane, const void* records,
                              float* S, void* stream) {
  int rc = check_dims(dims);
  if (rc != GDN_OK) return rc;
  if (dims->d_k != 128)
    return fail(GDN_EUNSUPPORTED, "gdn_kda_commit: d_k must be 128");
  if (!m_lane || !t_lane || !records || !S)
    return fail(GDN_EINVAL, "gdn_kda_commit: required pointer is NULL");
  if (misaligned(records, 256) || misaligned(S, 4))
    return fail(GDN_EINVAL, "gdn_kda_commit: misaligned pointer");
  const gdn_dims& d = *dims;
  CommitTable ct;
  rc = commit_lanes("gdn_kda_commit", d, m_lane, t_lane, ct);
  if (rc != GDN_OK) return rc;
  if (ct.n_act == 0) return GDN_OK;
  const WinDims w = win_dims(d);
  const KdaRecLayout L = kda_rec_layout(d);
  const char* rb = (const char*)records;
  const dim3 grid(d.n_layers * ct.n_act * d.h_v * w.ncb);
  hipError_t e = launch(kda_commit_kernel<128>, grid, dim3(kBlock),
                        (hipStream_t)stream, (const float*)(rb + L.k),
                        (const float*)(rb + L.u), (const float*)(rb + L.alpha),
                        S, w, ct);
  return hip_status(e, "gdn_kda_commit launch");
}
