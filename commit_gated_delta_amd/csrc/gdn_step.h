// gdn_step.h -- the per-step state transition shared by verify and commit.
//
// Gated delta rule (Gated DeltaNet, ICLR 2025, Sec. 3) on one state element:
//   S_ij <- alpha_t * S_ij + u_ti * khat_tj
//
// The state is held in scaled form S = c * St, with one f32 scale c per
// head ("lazy decay"): the decay multiplies only c (c <- c * alpha_t) and the
// rank-1 write becomes a single fused multiply-add on St,
//   St_ij <- fma(ut_i, k_j, St_ij),   ut = u_t * rk / c  (rk: 1/|k_t|),
// so a token costs three VALU operations per element (prediction, write,
// output) instead of four.  When c leaves [2^-32, 2^32] -- after many small
// decays, or alpha = 0 exactly -- it is folded into St (St <- c * St, c <- 1)
// before the token is applied.  Verify takes these decisions and records,
// per token, the fold factor (1 when none; a real fold factor is never 1,
// and alpha = 0 folds by 0) and the scale after the token;
// commit replays the recorded values instead of recomputing them.  The
// explicit state is materialised as S = c * St (one rounded product per
// element).
//
// Verify and commit both run exactly these functions, in the same token
// order, on the same recorded (phi, c, ut, k) values, so the state that
// commit(m) stores is bit-for-bit the state verify held after token m: the
// "transitions equal in finite precision" requirement of the ReplaySSM
// section of the NInfer technical review (blog.123qwe.co.kr post 4624).
// The library is compiled with -ffp-contract=off, so the compiler neither
// fuses nor splits any of these operations.
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

constexpr float kScaleLo = 0x1p-32f;
constexpr float kScaleHi = 0x1p32f;

// New scale after decay alpha; true when it must be folded into St now.
__device__ __forceinline__ bool scale_step(float c, float alpha, float& cn) {
  cn = c * alpha;
  return !(cn >= kScaleLo && cn <= kScaleHi);
}

// Fold the scale into the state entries this thread holds.
template <int R>
__device__ __forceinline__ void fold_scale(float (&s)[R], float cn) {
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = cn * s[r];
}

// The rank-1 write on one scaled state entry.
__device__ __forceinline__ float state_update(float st, float ut, float k) {
  return __builtin_fmaf(ut, k, st);
}

// Explicit state entry from the scaled form.
__device__ __forceinline__ float materialise(float c, float st) {
  return c * st;
}

}  // namespace gdn
