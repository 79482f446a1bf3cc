// gdn_window_common.h -- pieces shared by the window kernels (gated delta
// rule and its per-channel-decay sibling): sizes, lane tables, device
// helpers and host-side launch plumbing.  Included by gdn_window.hip and
// gdn_kda.hip only.
#pragma once
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <tuple>
#include <type_traits>

#include "gdn.h"
#include "gdn_internal.h"

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

// Records of the previous window, replayed by the fused commit + verify
// before the new window starts (unused by a plain verify).
struct PrevRecords {
  const float* k;
  const float* u;
  const float2* scale;
  LaneTable m;      // accepted prefix per lane
  LaneTable order;  // lanes by decreasing work (rank -> lane), see below
};

// Host-side arguments of a verify launch.
struct VerifyArgs {
  const void *q, *k, *v;
  const float *beta, *g;
  float* S;
  float* o;
  float *rk, *ru;
  float2* ra;
  float* dbg;
  float scale;
  int l2;
  int f32;  // inputs are f32 (else bf16)
};

// Draft trees (windows where a node steps from its parent's state): the
// parents of every lane's nodes, or for a commit the accepted nodes of every
// active lane, as bytes in the kernel arguments.
constexpr int kTreeMaxT = 32;     // nodes per tree window
constexpr int kTreeCells = 2048;  // n_lanes * t_max
constexpr uint8_t kNoParent = 255;
struct TreeTable {
  uint8_t v[kTreeCells];  // [lane * t_max + t]: parent, or kNoParent
};
struct NoTable {};

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

// Entries 2x and 2x+1 of a row of n <= 128 entries as f32 (0 past the end).
__device__ __forceinline__ void row_pair(const uint16_t* __restrict__ row,
                                         int n, int x, float& lo, float& hi) {
  lo = hi = 0.f;
  if (2 * x < n) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[x];
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  }
}
__device__ __forceinline__ void row_pair(const float* __restrict__ row, int n,
                                         int x, float& lo, float& hi) {
  lo = hi = 0.f;
  if (2 * x < n) {
    const float2 p = reinterpret_cast<const float2*>(row)[x];
    lo = p.x;
    hi = p.y;
  }
}

__device__ __forceinline__ float inv_norm(float ss) {
  return __builtin_amdgcn_rsqf(ss + 1e-6f);
}


// |k|^2, |q|^2 and k.q of one row, 16 lanes per row: lane `sub` holds the
// entries 8*sub .. 8*sub+7 (zeros past the end) and the sums are reduced
// over the 16-lane DPP row, so every lane of the row returns them.
template <typename TIn>
__device__ __forceinline__ void row_moments(const TIn* __restrict__ krow,
                                            const TIn* __restrict__ qrow,
                                            int n, int sub, float (&kk)[8],
                                            float& skk, float& sqq,
                                            float& skq) {
  float qq[8];
  if (8 * sub < n) {
    if constexpr (sizeof(TIn) == 2) {
      const uint4 kr = *reinterpret_cast<const uint4*>(krow + 8 * sub);
      const uint4 qr = *reinterpret_cast<const uint4*>(qrow + 8 * sub);
      const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
      const uint32_t qw[4] = {qr.x, qr.y, qr.z, qr.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk[2 * e] = __uint_as_float(kw[e] << 16);
        kk[2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
        qq[2 * e] = __uint_as_float(qw[e] << 16);
        qq[2 * e + 1] = __uint_as_float(qw[e] & 0xffff0000u);
      }
    } else {
      const float4 k0 = *reinterpret_cast<const float4*>(krow + 8 * sub);
      const float4 k1 = *reinterpret_cast<const float4*>(krow + 8 * sub + 4);
      const float4 q0 = *reinterpret_cast<const float4*>(qrow + 8 * sub);
      const float4 q1 = *reinterpret_cast<const float4*>(qrow + 8 * sub + 4);
      kk[0] = k0.x; kk[1] = k0.y; kk[2] = k0.z; kk[3] = k0.w;
      kk[4] = k1.x; kk[5] = k1.y; kk[6] = k1.z; kk[7] = k1.w;
      qq[0] = q0.x; qq[1] = q0.y; qq[2] = q0.z; qq[3] = q0.w;
      qq[4] = q1.x; qq[5] = q1.y; qq[6] = q1.z; qq[7] = q1.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) kk[e] = qq[e] = 0.f;
  }
  skk = sqq = skq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    skk = __builtin_fmaf(kk[e], kk[e], skk);
    sqq = __builtin_fmaf(qq[e], qq[e], sqq);
    skq = __builtin_fmaf(kk[e], qq[e], skq);
  }
  skk += dpp<0xB1>(skk); sqq += dpp<0xB1>(sqq); skq += dpp<0xB1>(skq);
  skk += dpp<0x4E>(skk); sqq += dpp<0x4E>(sqq); skq += dpp<0x4E>(skq);
  skk += dpp<0x141>(skk); sqq += dpp<0x141>(sqq); skq += dpp<0x141>(skq);
  skk += dpp<0x140>(skk); sqq += dpp<0x140>(sqq); skq += dpp<0x140>(skq);
}

// ------------------------------------------------------------- host side
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
  char msg[256];
  snprintf(msg, sizeof(msg), "%s: %s", what, hipGetErrorString(e));
  set_error(msg);
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

// Lane table of a commit: m_lane[n] in 0..t_lane[n] <= t_max.
static int commit_lanes(const char* fn, const gdn_dims& d,
                        const int32_t* m_lane, const int32_t* t_lane,
                        CommitTable& ct) {
  char msg[128];
  memset(&ct, 0, sizeof(ct));
  int n_act = 0;
  for (int n = 0; n < d.n_lanes; ++n) {
    if (t_lane[n] < 0 || t_lane[n] > d.t_max) {
      snprintf(msg, sizeof(msg), "%s: t_lane out of 0..t_max", fn);
      return fail(GDN_EINVAL, msg);
    }
    if (m_lane[n] < 0 || m_lane[n] > t_lane[n]) {
      snprintf(msg, sizeof(msg), "%s: m_lane out of 0..t_lane", fn);
      return fail(GDN_EINVAL, msg);
    }
    if (m_lane[n] > 0) {
      ct.lane[n_act] = (uint8_t)n;
      ct.m[n_act] = (uint8_t)m_lane[n];
      ++n_act;
    }
  }
  ct.n_act = n_act;
  return GDN_OK;
}

// The matrix-core verify (gdn_window_mfma.hip): whether a call can take it
// (bf16 or f32 windows of up to GDN_MAX_T tokens, draft trees of up to 16
// nodes), and its launch (replay = the fused commit + verify).
__attribute__((visibility("hidden"))) bool mverify_eligible(
    const gdn_dims& d, int in_dtype, const VerifyArgs& a, bool tree);
__attribute__((visibility("hidden"))) hipError_t launch_mverify(
    const WinDims& w, const LaneTable& tl, const VerifyArgs& a,
    const PrevRecords& pr, bool replay, hipStream_t st);
// The matrix-core verify of a draft-tree window.
__attribute__((visibility("hidden"))) hipError_t launch_mverify_tree(
    const WinDims& w, const LaneTable& tl, const VerifyArgs& a,
    const TreeTable& tree, hipStream_t st);

// The matrix-core KDA verify (gdn_kda_mfma.hip; f32: the inputs are f32,
// else bf16).
__attribute__((visibility("hidden"))) bool mkda_eligible(
    const gdn_dims& d, int in_dtype, const void* q, const void* k,
    const void* v, const float* g, const float* S, const float* o,
    const float* dbg);
__attribute__((visibility("hidden"))) hipError_t launch_mkda(
    const WinDims& w, const LaneTable& tl, bool f32, const void* q,
    const void* k, const void* v, const float* beta, const float* g,
    const float* S, float* o, float* rk, float* ru, float* ra, float* dbg,
    float scale, int l2, hipStream_t st);

}  // namespace gdn
