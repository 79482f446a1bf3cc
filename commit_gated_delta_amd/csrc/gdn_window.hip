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
// Records per token: alpha (f32 per value head), ut (f32 per value head and
// column) and the raw key row widened to f32 (per key head).  Commit replays
// the same scale steps and St_ij <- fma(ut_i, k_j, St_ij) from exactly these
// values and stores S_m = c * St, so its result is bitwise the state verify
// held after the same token.
//
// Work decomposition (CDNA4, wave64):
//   One 256-thread workgroup per (layer, lane, value head, block of 64 value
//   columns).  Lane x of every wave owns column i = 64*cb + x; wave w owns
//   key rows j in [w*dk/4, (w+1)*dk/4).  A lane keeps its dk/4 state entries
//   in VGPRs for the whole window (32 at dk = 128), which leaves room for
//   eight waves per SIMD to hide memory latency.
//   Both reductions over j are a register chain inside the lane plus a sum
//   of four wave partials through LDS (two barriers per token).  The key and
//   query values of a wave's rows are the same for all its lanes: they come
//   in through scalar loads (SGPRs), bf16 pairs unpacked with two scalar ALU
//   ops, and every multiply-add takes them as its SGPR operand -- no LDS
//   broadcast traffic on the hot loop.
//   The norms: wave 0 reduces |k|^2 and wave 1 reduces |q|^2 over the whole
//   row (one dword per lane and a wave reduction) while the others work;
//   the results travel with the first LDS exchange.
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

#include "gdn.h"
#include "gdn_internal.h"
#include "gdn_step.h"

namespace gdn {

constexpr int kWave = 64;
constexpr int kWaves = 4;  // waves per workgroup: d_k rows split four ways
constexpr int kBlock = kWave * kWaves;

struct WinDims {
  int NL, N, Hv, Hk, dk, dv, T;
  int group;  // h_v / h_k
  int ncb;    // column blocks of 64 per head
};

struct LaneTable {
  uint8_t v[GDN_MAX_LANES];
};

struct CommitTable {
  int n_act;  // lanes with m > 0, listed first in lane[] / m[]
  uint8_t lane[GDN_MAX_LANES];
  uint8_t m[GDN_MAX_LANES];
};

// ------------------------------------------------------------- records
struct RecLayout {
  size_t k, u, alpha, total;
};

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static RecLayout rec_layout(const gdn_dims& d) {
  RecLayout r;
  const size_t ntok = (size_t)d.n_layers * d.n_lanes * d.t_max;
  r.k = 0;
  r.u = align256(ntok * d.h_k * d.d_k * sizeof(float));
  r.alpha = r.u + align256(ntok * d.h_v * d.d_v * sizeof(float));
  r.total = r.alpha + align256(ntok * d.h_v * sizeof(float));
  return r;
}

// ------------------------------------------------------------- helpers
__device__ __forceinline__ float load_in(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);  // bf16 -> f32 is exact
}
__device__ __forceinline__ float load_in(const float* p, size_t i) {
  return p[i];
}

__device__ __forceinline__ int uniform(int x) {
  return __builtin_amdgcn_readfirstlane(x);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the 64 lanes, the same value in every lane: butterflies inside
// each 16-lane row through DPP (quad swaps, half-row and row mirrors), then
// the four row sums in a fixed order.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

// Block b runs on XCD b % 8.  XCD x gets the item range [x*n/8, (x+1)*n/8).
__device__ __forceinline__ int xcd_item(int b, int n) {
  constexpr int kXcd = 8;
  if (n % kXcd != 0) return b;
  return (b % kXcd) * (n / kXcd) + b / kXcd;
}

// Raw row words of this wave's key rows: bf16 pairs (R/2 dwords) or f32 (R
// dwords).  The addresses are wave-uniform, so these are scalar loads.
template <typename TIn, int R>
struct RowWords {
  static constexpr int kN = sizeof(TIn) == 2 ? R / 2 : R;
  uint32_t w[kN];
  __device__ __forceinline__ void load(const TIn* __restrict__ row, int j0) {
    const uint32_t* dw =
        reinterpret_cast<const uint32_t*>(row) + (sizeof(TIn) == 2 ? j0 / 2 : j0);
#pragma unroll
    for (int n = 0; n < kN; ++n) w[n] = dw[n];
  }
  // entry r as f32 (bf16 widening is exact)
  __device__ __forceinline__ float at(int r) const {
    if constexpr (sizeof(TIn) == 2)
      return (r & 1) ? __uint_as_float(w[r / 2] & 0xffff0000u)
                     : __uint_as_float(w[r / 2] << 16);
    else
      return __uint_as_float(w[r]);
  }
};

// |row|^2 over the whole row (n <= 128 entries; lane x holds entries 2x and
// 2x+1, returned through lo/hi so that the caller can copy the row out).
__device__ __forceinline__ float row_sumsq(const uint16_t* __restrict__ row,
                                           int n, int x, float& lo,
                                           float& hi) {
  lo = hi = 0.f;
  if (2 * x < n) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[x];
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  }
  return wave_sum(__builtin_fmaf(hi, hi, lo * lo));
}
__device__ __forceinline__ float row_sumsq(const float* __restrict__ row,
                                           int n, int x, float& lo,
                                           float& hi) {
  lo = hi = 0.f;
  if (2 * x < n) {
    const float2 p = reinterpret_cast<const float2*>(row)[x];
    lo = p.x;
    hi = p.y;
  }
  return wave_sum(__builtin_fmaf(hi, hi, lo * lo));
}

__device__ __forceinline__ float inv_norm(float ss) {
  return __builtin_amdgcn_rsqf(ss + 1e-6f);
}

// ------------------------------------------------------------- verify
template <int DK, bool DBG, typename TIn>
__global__ __launch_bounds__(kBlock) void verify_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ g, const float* __restrict__ S,
    float* __restrict__ o, float* __restrict__ rec_k,
    float* __restrict__ rec_u, float* __restrict__ rec_alpha,
    float* __restrict__ dbg, WinDims d, LaneTable tl, float scale,
    int l2norm) {
  constexpr int R = DK / kWaves;  // key rows per wave
  __shared__ float red_p[kWaves][kWave];
  __shared__ float red_o[kWaves][kWave];
  __shared__ float norm_s[2];

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
  const bool key_writer = (h % d.group == 0) && cb == 0 && w == 0;
  const size_t ll = (size_t)layer * d.N + lane;
  const size_t dv = (size_t)d.dv;

  float s[R];  // scaled state St (rows j0..j0+R-1, column i); S = c * St
  {
    const float* Sh = S + ((ll * d.Hv + h) * (size_t)DK + j0) * dv + ic;
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = __builtin_nontemporal_load(Sh + r * dv);
  }
  float c = 1.0f;

  for (int t = 0; t < T; ++t) {
    const size_t tok = ll * d.T + t;
    const size_t krow = (tok * d.Hk + kh) * (size_t)DK;
    const size_t gi = tok * d.Hv + h;
    RowWords<TIn, R> kw, qw;
    kw.load(k + krow, j0);
    qw.load(q + krow, j0);
    const float vi = load_in(v, gi * dv + ic);

    // norms (wave 0: key, wave 1: query) and the key record row
    if (w == 0 && (l2norm || key_writer)) {
      float lo, hi;
      const float ss = row_sumsq(k + krow, DK, x, lo, hi);
      if (x == 0) norm_s[0] = l2norm ? inv_norm(ss) : 1.0f;
      if (key_writer && 2 * x < DK)
        reinterpret_cast<float2*>(rec_k + krow)[x] = make_float2(lo, hi);
    } else if (w == 1 && l2norm) {
      float lo, hi;
      const float ss = row_sumsq(q + krow, DK, x, lo, hi);
      if (x == 0) norm_s[1] = inv_norm(ss);
    }

    const float alpha = __expf(g[gi]);
    float cn;
    if (scale_step(c, alpha, cn)) {
      fold_scale<R>(s, cn);
      cn = 1.0f;
    }

    // partial of P_i = sum_j St_ij k_j over this wave's rows (4 chains)
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      a0 = __builtin_fmaf(s[r + 0], kw.at(r + 0), a0);
      a1 = __builtin_fmaf(s[r + 1], kw.at(r + 1), a1);
      a2 = __builtin_fmaf(s[r + 2], kw.at(r + 2), a2);
      a3 = __builtin_fmaf(s[r + 3], kw.at(r + 3), a3);
    }
    red_p[w][x] = (a0 + a1) + (a2 + a3);
    __syncthreads();
    const float P = (red_p[0][x] + red_p[1][x]) + (red_p[2][x] + red_p[3][x]);
    const float rk = l2norm ? norm_s[0] : 1.0f;
    const float rq = l2norm ? norm_s[1] : 1.0f;
    // p = alpha * (S_{t-1} khat) = (c_t * rk) * P;  ut = u * rk / c_t
    const float p = (cn * rk) * P;
    const float ut = (beta[gi] * (vi - p)) * (rk * __builtin_amdgcn_rcpf(cn));
    if (w == 0) {
      if (act) rec_u[gi * dv + i] = ut;
      if (cb == 0 && x == 0) rec_alpha[gi] = alpha;
    }

    // rank-1 write, then the output partial on the new state
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      s[r + 0] = state_update(s[r + 0], ut, kw.at(r + 0));
      s[r + 1] = state_update(s[r + 1], ut, kw.at(r + 1));
      s[r + 2] = state_update(s[r + 2], ut, kw.at(r + 2));
      s[r + 3] = state_update(s[r + 3], ut, kw.at(r + 3));
      o0 = __builtin_fmaf(s[r + 0], qw.at(r + 0), o0);
      o1 = __builtin_fmaf(s[r + 1], qw.at(r + 1), o1);
      o2 = __builtin_fmaf(s[r + 2], qw.at(r + 2), o2);
      o3 = __builtin_fmaf(s[r + 3], qw.at(r + 3), o3);
    }
    red_o[w][x] = (o0 + o1) + (o2 + o3);
    c = cn;
    if (DBG && act) {
      float* dp = dbg + (gi * (size_t)DK + j0) * dv + i;
#pragma unroll
      for (int r = 0; r < R; ++r) dp[r * dv] = materialise(c, s[r]);
    }
    __syncthreads();
    if (w == 0 && act) {
      const float osum =
          (red_o[0][x] + red_o[1][x]) + (red_o[2][x] + red_o[3][x]);
      o[gi * dv + i] = (scale * rq * c) * osum;
    }
  }
}

// ------------------------------------------------------------- commit
template <int DK>
__global__ __launch_bounds__(kBlock) void commit_kernel(
    const float* __restrict__ rec_k, const float* __restrict__ rec_u,
    const float* __restrict__ rec_alpha, float* __restrict__ S, WinDims d,
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
  float* Sh = S + ((ll * d.Hv + h) * (size_t)DK + j0) * dv + ic;

  float s[R];
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = __builtin_nontemporal_load(Sh + r * dv);
  float c = 1.0f;

  // the records of token t+1 are requested before token t is applied
  size_t tok = ll * d.T;
  float alpha = rec_alpha[tok * d.Hv + h];
  float ut = rec_u[(tok * d.Hv + h) * dv + ic];
  RowWords<float, R> kw;
  kw.load(rec_k + (tok * d.Hk + kh) * (size_t)DK, j0);
  for (int t = 0; t < m; ++t) {
    const size_t nt = ll * d.T + (t + 1 < m ? t + 1 : t);
    const float alpha_n = rec_alpha[nt * d.Hv + h];
    const float ut_n = rec_u[(nt * d.Hv + h) * dv + ic];
    RowWords<float, R> kw_n;
    kw_n.load(rec_k + (nt * d.Hk + kh) * (size_t)DK, j0);
    float cn;
    if (scale_step(c, alpha, cn)) {
      fold_scale<R>(s, cn);
      cn = 1.0f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = state_update(s[r], ut, kw.at(r));
    c = cn;
    alpha = alpha_n;
    ut = ut_n;
    kw = kw_n;
  }
  if (act) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      __builtin_nontemporal_store(materialise(c, s[r]), Sh + r * dv);
  }
}

// ------------------------------------------------------------- host side
static thread_local char g_last_error[256] = "";

void set_error(const char* msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
}

static int fail(int status, const char* what) {
  set_error(what);
  return status;
}

// Launch through hipLaunchKernel so that the status returned is this
// launch's own (hipGetLastError could report an earlier, unrelated error).
template <typename... KArgs, typename... Args>
static hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block,
                         hipStream_t st, Args&&... args) {
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... v) {
    int n = 0;
    ((ptrs[n++] = (void*)&v), ...);
  }, vals);
  return hipLaunchKernel((const void*)kern, grid, block, ptrs, 0, st);
}

static int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GDN_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what,
           hipGetErrorString(e));
  return GDN_EHIP;
}

static int check_dims(const gdn_dims* p) {
  if (!p) return fail(GDN_EINVAL, "dims is NULL");
  const gdn_dims& d = *p;
  if (d.n_layers < 1 || d.n_lanes < 1 || d.n_lanes > GDN_MAX_LANES ||
      d.h_v < 1 || d.h_k < 1 || d.h_v % d.h_k != 0 || d.d_k < 1 ||
      d.d_v < 1 || d.d_v > 1024 || d.t_max < 1 || d.t_max > GDN_MAX_T)
    return fail(GDN_EINVAL, "dims out of range");
  if (d.d_k != 16 && d.d_k != 32 && d.d_k != 64 && d.d_k != 128)
    return fail(GDN_EUNSUPPORTED, "d_k must be 16, 32, 64 or 128");
  const double ntok = (double)d.n_layers * d.n_lanes * d.t_max;
  const double big = ntok * (double)d.h_v * d.d_k * d.d_v;  // dbg states
  if (big > 9.0e15) return fail(GDN_EINVAL, "sizes overflow");
  const double blocks = (double)d.n_layers * d.n_lanes * d.h_v *
                        ((d.d_v + kWave - 1) / kWave);
  if (blocks > (double)INT_MAX) return fail(GDN_EINVAL, "grid too large");
  return GDN_OK;
}

static bool misaligned(const void* p, size_t a) {
  return ((uintptr_t)p % a) != 0;
}

static WinDims win_dims(const gdn_dims& d) {
  WinDims w;
  w.NL = d.n_layers;
  w.N = d.n_lanes;
  w.Hv = d.h_v;
  w.Hk = d.h_k;
  w.dk = d.d_k;
  w.dv = d.d_v;
  w.T = d.t_max;
  w.group = d.h_v / d.h_k;
  w.ncb = (d.d_v + kWave - 1) / kWave;
  return w;
}

template <int DK, bool DBG, typename TIn>
static hipError_t launch_verify_t(const WinDims& w, const LaneTable& tl,
                                  const void* q, const void* k, const void* v,
                                  const float* beta, const float* g,
                                  const float* S, float* o, float* rk,
                                  float* ru, float* ra, float* dbg,
                                  float scale, int l2, hipStream_t st) {
  const int blocks = w.NL * w.N * w.Hv * w.ncb;
  return launch(verify_kernel<DK, DBG, TIn>, dim3(blocks), dim3(kBlock), st,
                (const TIn*)q, (const TIn*)k, (const TIn*)v, beta, g, S, o, rk,
                ru, ra, dbg, w, tl, scale, l2);
}

template <bool DBG, typename TIn>
static hipError_t launch_verify_d(const WinDims& w, const LaneTable& tl,
                                  const void* q, const void* k, const void* v,
                                  const float* beta, const float* g,
                                  const float* S, float* o, float* rk,
                                  float* ru, float* ra, float* dbg,
                                  float scale, int l2, hipStream_t st) {
  switch (w.dk) {
    case 16: return launch_verify_t<16, DBG, TIn>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg, scale, l2, st);
    case 32: return launch_verify_t<32, DBG, TIn>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg, scale, l2, st);
    case 64: return launch_verify_t<64, DBG, TIn>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg, scale, l2, st);
    default: return launch_verify_t<128, DBG, TIn>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg, scale, l2, st);
  }
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
  int rc = check_dims(dims);
  if (rc != GDN_OK) return rc;
  if (!t_lane || !q || !k || !v || !beta || !g || !S || !o || !records)
    return fail(GDN_EINVAL, "gdn_verify: required pointer is NULL");
  if (in_dtype != GDN_BF16 && in_dtype != GDN_F32)
    return fail(GDN_EINVAL, "gdn_verify: unknown in_dtype");
  if (flags & ~GDN_FLAG_L2NORM_QK)
    return fail(GDN_EINVAL, "gdn_verify: unknown flag bits");
  // q/k rows are read as dwords (bf16 pairs) or f32
  if (misaligned(q, 4) || misaligned(k, 4) ||
      misaligned(v, in_dtype == GDN_BF16 ? 2 : 4) || misaligned(beta, 4) ||
      misaligned(g, 4) || misaligned(S, 4) || misaligned(o, 4) ||
      misaligned(records, 256) || (dbg_states && misaligned(dbg_states, 4)))
    return fail(GDN_EINVAL, "gdn_verify: misaligned pointer");
  const gdn_dims& d = *dims;
  LaneTable tl;
  memset(&tl, 0, sizeof(tl));
  int any = 0;
  for (int n = 0; n < d.n_lanes; ++n) {
    if (t_lane[n] < 0 || t_lane[n] > d.t_max)
      return fail(GDN_EINVAL, "gdn_verify: t_lane out of 0..t_max");
    tl.v[n] = (uint8_t)t_lane[n];
    any |= t_lane[n];
  }
  if (!any) return GDN_OK;

  const WinDims w = win_dims(d);
  const RecLayout L = rec_layout(d);
  char* rb = (char*)records;
  float* rk = (float*)(rb + L.k);
  float* ru = (float*)(rb + L.u);
  float* ra = (float*)(rb + L.alpha);
  hipStream_t st = (hipStream_t)stream;
  const int l2 = (flags & GDN_FLAG_L2NORM_QK) ? 1 : 0;
  hipError_t e;
  if (in_dtype == GDN_BF16) {
    e = dbg_states
            ? launch_verify_d<true, uint16_t>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg_states, scale, l2, st)
            : launch_verify_d<false, uint16_t>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, nullptr, scale, l2, st);
  } else {
    e = dbg_states
            ? launch_verify_d<true, float>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, dbg_states, scale, l2, st)
            : launch_verify_d<false, float>(w, tl, q, k, v, beta, g, S, o, rk, ru, ra, nullptr, scale, l2, st);
  }
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
  memset(&ct, 0, sizeof(ct));
  int n_act = 0;
  for (int n = 0; n < d.n_lanes; ++n) {
    if (t_lane[n] < 0 || t_lane[n] > d.t_max)
      return fail(GDN_EINVAL, "gdn_commit: t_lane out of 0..t_max");
    if (m_lane[n] < 0 || m_lane[n] > t_lane[n])
      return fail(GDN_EINVAL, "gdn_commit: m_lane out of 0..t_lane");
    if (m_lane[n] > 0) {
      ct.lane[n_act] = (uint8_t)n;
      ct.m[n_act] = (uint8_t)m_lane[n];
      ++n_act;
    }
  }
  if (n_act == 0) return GDN_OK;
  ct.n_act = n_act;
  const WinDims w = win_dims(d);
  const RecLayout L = rec_layout(d);
  const char* rb = (const char*)records;
  const float* rk = (const float*)(rb + L.k);
  const float* ru = (const float*)(rb + L.u);
  const float* ra = (const float*)(rb + L.alpha);
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(d.n_layers * n_act * d.h_v * w.ncb);
  hipError_t e;
  switch (d.d_k) {
    case 16: e = launch(commit_kernel<16>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct); break;
    case 32: e = launch(commit_kernel<32>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct); break;
    case 64: e = launch(commit_kernel<64>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct); break;
    default: e = launch(commit_kernel<128>, grid, dim3(kBlock), st, rk, ru, ra, S, w, ct); break;
  }
  return hip_status(e, "gdn_commit launch");
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
