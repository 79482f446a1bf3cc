// gdn_state.hip -- recurrent-state snapshot and restore for gfx950.
//
// When memory runs short, the engine described in the NInfer technical
// review (blog.123qwe.co.kr post 4624, section "Architecture 2: context byte
// pool and prefix reuse") pauses active requests and later brings them back
// either by replaying their tokens or from a snapshot of their state; a
// pinned host budget holds such context.  For the gated-delta layers the
// continuation state of a request (a lane) is its f32 state S in every layer
// and value head.  These kernels gather the state of chosen lanes into a
// compact lane-major snapshot (one contiguous block per lane, in device or
// pinned host memory) and scatter a snapshot back into chosen lanes.  Both
// are exact copies.
//
// Layouts (f32):
//   S         [n_layers][n_lanes][h_v][d_k][d_v]   (the state the window
//                                                   kernels read and write)
//   snapshot  [n_sel][n_layers][h_v][d_k][d_v]
// One layer of one lane is a contiguous span of h_v*d_k*d_v floats in both,
// so every workgroup copies 64 KiB of one span with 16-byte vector accesses
// (streaming, non-temporal: a snapshot is written once and not read soon).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdns {

constexpr int kThreads = 256;
constexpr int kSpanChunk = 16384;  // floats per workgroup (64 KiB)

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct CopyPlan {
  int n_sel, n_layers, n_lanes;
  int chunks;   // workgroups per span
  long span;    // floats per (lane, layer)
  int gather;   // 1: S -> snapshot, 0: snapshot -> S
  int lane[GDN_MAX_LANES];
};

__global__ __launch_bounds__(kThreads) void copy_kernel(const f32x4* __restrict__ src,
                                                       f32x4* __restrict__ dst,
                                                       CopyPlan p) {
  const int b = blockIdx.x;
  const int ch = b % p.chunks;
  const int sl = b / p.chunks;  // (sel, layer)
  const int sel = sl / p.n_layers, layer = sl % p.n_layers;
  const long in_state = ((long)layer * p.n_lanes + p.lane[sel]) * p.span;
  const long in_snap = ((long)sel * p.n_layers + layer) * p.span;
  const long so = p.gather ? in_state : in_snap;
  const long d_o = p.gather ? in_snap : in_state;
  const long base = (long)ch * kSpanChunk;
  long n = p.span - base;
  if (n > kSpanChunk) n = kSpanChunk;
  const int n4 = (int)(n / 4);
  const f32x4* __restrict__ s4 = src + (so + base) / 4;
  f32x4* __restrict__ d4 = dst + (d_o + base) / 4;
  constexpr int kPer = kSpanChunk / 4 / kThreads;  // 16 vectors per thread
  if (n4 == kSpanChunk / 4) {
    // a full chunk: all loads of the thread in flight before the stores
    f32x4 r[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      r[u] = __builtin_nontemporal_load(s4 + threadIdx.x + u * kThreads);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      __builtin_nontemporal_store(r[u], d4 + threadIdx.x + u * kThreads);
  } else {
    for (int e = threadIdx.x; e < n4; e += kThreads)
      __builtin_nontemporal_store(__builtin_nontemporal_load(s4 + e), d4 + e);
  }
}

static thread_local char g_msg[160];

static int fail(int status, const char* msg) {
  gdn::set_error(msg);
  return status;
}

static int run(const gdn_dims* dims, int32_t n_sel, const int32_t* lanes,
               const float* src, float* dst, int gather, void* stream,
               const char* fn) {
  if (!dims) return fail(GDN_EINVAL, "state copy: dims is NULL");
  const gdn_dims& d = *dims;
  if (d.n_layers < 1 || d.n_lanes < 1 || d.n_lanes > GDN_MAX_LANES ||
      d.h_v < 1 || d.d_k < 1 || d.d_v < 1) {
    snprintf(g_msg, sizeof(g_msg), "%s: dims out of range", fn);
    return fail(GDN_EINVAL, g_msg);
  }
  if (n_sel < 0 || n_sel > d.n_lanes) {
    snprintf(g_msg, sizeof(g_msg), "%s: n_sel out of 0..n_lanes", fn);
    return fail(GDN_EINVAL, g_msg);
  }
  if (n_sel == 0) return GDN_OK;
  if (!lanes || !src || !dst) {
    snprintf(g_msg, sizeof(g_msg), "%s: required pointer is NULL", fn);
    return fail(GDN_EINVAL, g_msg);
  }
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) {
    snprintf(g_msg, sizeof(g_msg), "%s: pointers must be 16-byte aligned", fn);
    return fail(GDN_EINVAL, g_msg);
  }
  const long span = (long)d.h_v * d.d_k * d.d_v;
  if (span % 4 != 0) {
    snprintf(g_msg, sizeof(g_msg), "%s: h_v*d_k*d_v must be a multiple of 4", fn);
    return fail(GDN_EUNSUPPORTED, g_msg);
  }
  CopyPlan p;
  p.n_sel = n_sel;
  p.n_layers = d.n_layers;
  p.n_lanes = d.n_lanes;
  p.span = span;
  p.chunks = (int)((span + kSpanChunk - 1) / kSpanChunk);
  p.gather = gather;
  bool seen[GDN_MAX_LANES] = {};
  for (int j = 0; j < n_sel; ++j) {
    if (lanes[j] < 0 || lanes[j] >= d.n_lanes) {
      snprintf(g_msg, sizeof(g_msg), "%s: lane index out of range", fn);
      return fail(GDN_EINVAL, g_msg);
    }
    // two snapshot blocks written into one lane would race
    if (!gather && seen[lanes[j]]) {
      snprintf(g_msg, sizeof(g_msg), "%s: a lane is restored twice", fn);
      return fail(GDN_EINVAL, g_msg);
    }
    seen[lanes[j]] = true;
    p.lane[j] = lanes[j];
  }
  const double blocks = (double)n_sel * d.n_layers * p.chunks;
  if (blocks > (double)INT_MAX) {
    snprintf(g_msg, sizeof(g_msg), "%s: too many blocks", fn);
    return fail(GDN_EINVAL, g_msg);
  }
  const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
  f32x4* d4 = reinterpret_cast<f32x4*>(dst);
  void* args[] = {(void*)&s4, (void*)&d4, (void*)&p};
  hipError_t e = hipLaunchKernel((const void*)copy_kernel, dim3((unsigned)blocks),
                                 dim3(kThreads), args, 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    snprintf(g_msg, sizeof(g_msg), "%s launch: %s", fn, hipGetErrorString(e));
    return fail(GDN_EHIP, g_msg);
  }
  return GDN_OK;
}

}  // namespace gdns

extern "C" int gdn_state_snapshot(const gdn_dims* dims, int32_t n_sel,
                                  const int32_t* lanes, const float* S,
                                  float* snapshot, void* stream) {
  return gdns::run(dims, n_sel, lanes, S, snapshot, 1, stream,
                   "gdn_state_snapshot");
}

extern "C" int gdn_state_restore(const gdn_dims* dims, int32_t n_sel,
                                 const int32_t* lanes, const float* snapshot,
                                 float* S, void* stream) {
  return gdns::run(dims, n_sel, lanes, snapshot, S, 0, stream,
                   "gdn_state_restore");
}
