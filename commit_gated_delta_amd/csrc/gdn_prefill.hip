// gdn_prefill.hip -- chunked prefill of the gated delta rule on gfx950 MFMA.
//
// Block (WY/UT) form of the rule over chunks of C = 16, 32 or 64 tokens, each
// chunk in a 64-row tile (rows past a short chunk are inert, see ws_bytes):
// Yang et al.,
// "Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length" (NeurIPS 2024), Sec. 3 (the UT transform), with the per-token decay
// of Gated DeltaNet (ICLR 2025).  In the stored orientation H = S^T (d_k x d_v)
// and for one chunk with rows i, j = 0..63, chunk-start state H and
//   rk_i, rq_i   inverse L2 norms of the raw key / query rows (1 if off)
//   G_i          = g_0 + ... + g_i (within the chunk), gamma_i = exp(G_i)
//   L_ij         = beta_i rk_i rk_j (k_i . k_j) exp(G_i - G_j)      j < i
//   T            = (I + L)^-1                          (unit lower triangular)
//   P_ij         = rq_i rk_j (q_i . k_j) exp(G_i - G_j)              j <= i
// the chunk advances as
//   X      = diag(beta) V - diag(beta gamma rk) (K H)
//   V_new  = T X                              (the actual deltas u_i, rows)
//   O      = diag(gamma rq) (Q H) + P V_new   (times the output scale)
//   H'     = gamma_63 H + K^T diag(rk exp(G_63 - G)) V_new
// Unrolling the token-by-token rule inside one chunk gives exactly these
// expressions; only the evaluation order differs.  G is summed in segments
// that restart after a gate whose exponential is 0 in f32 (g < -128, g =
// -inf): every decay across such a gate is exactly 0 (the state before it
// is forgotten, alpha = 0), and no difference of two infinite or huge sums
// is formed.
//
// Kernels:
//   p1  one workgroup per (sequence, chunk, value head), all chunks in
//       parallel: K K^T and Q K^T on bf16 MFMA (raw bf16 operands are exact),
//       L and P built on the f32 accumulators, T by blocked forward
//       substitution (16x16 diagonal blocks by column recurrences, then the
//       off-diagonal blocks block-row by block-row).  T and P are written to
//       the workspace as split bf16 pairs (hi = bf16(x), lo = bf16(x - hi)),
//       with the per-row scale vectors.
//   p2  one workgroup per (sequence, value head, 16-column tile of d_v),
//       sequential over the chunks, with one wave per role: the state chain
//       (the d_k x 16 state tile in f32 MFMA accumulators of one wave), two
//       output waves and one staging wave (details at p2 below).  Products
//       with an f32 operand use split bf16: two passes against an exact bf16
//       operand (K H, Q H, K^T V'), three passes f32 x f32 (T X, P V_new);
//       about 2^-17 relative error per product.  The state is never rounded
//       below f32, so a run resumed from a checkpoint is bitwise the straight
//       run.  The output O of each chunk is produced here too (no separate
//       pass).
//   Checkpoints: the state after every token count that is a positive
//   multiple of the interval (context_cache.checkpoint_interval, NInfer
//   technical review, blog.123qwe.co.kr post 4624, section "Architecture 2").
//   segments  a batch of at most kSegMaxHeads sequence-heads runs as
//       segments of kSeg tokens: P2 passes give each segment's transition
//       and offset, seg_scan_kernel chains them, a last P2 pass produces the
//       outputs (details in the segments section below).
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Lane l of a wave holds
//   A[l%16][8*(l/16) + e], B[8*(l/16) + e][l%16]   (e = 0..7, bf16)
//   D[4*(l/16) + e][l%16]                          (e = 0..3, f32).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdnp {

constexpr int kC = 64;     // chunk length
constexpr int kD = 128;    // d_k = d_v
constexpr int kTile = 16;  // value columns per p2 workgroup
constexpr int kThreads = 256;
constexpr float kReset = -128.f;  // exp(g) rounds to 0 in f32 below this

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

struct PDims {
  int n_seqs, L, Hv, Hk, group, n_chunks;  // n_seqs parts of L tokens
  // A P2 launch runs n_seqs parts; part s is piece s % segs of sequence
  // s / segs (segs = 1: every part a whole sequence).  Piece j starts at
  // token j * L of its sequence of seq_L tokens (seq_chunks chunks); the
  // last piece of each sequence has L_last <= L tokens.  P1 takes whole
  // sequences (segs = 1, seq_L = L_last = L).
  int segs, seq_L, seq_chunks, L_last;
  int chunk;          // tokens per chunk: 16, 32 or 64 (<= kC)
  int ckpt_interval;  // 0: no checkpoints
  float scale;
  int l2norm;
};

// Template arguments of the p2 roles for a segmented prefill (see
// seg_scan_kernel): a chain with V taken as zero, or started from the
// identity instead of S_init; output waves that only warm L2.  p2_kernel's
// own argument is 0 (the plain pass) or kModePair (two chains of one
// segment tile side by side, see p2_kernel).
enum { kModeVZero = 1, kModeNoOut = 2, kModeIdentity = 4, kModePair = 8 };

// Workspace per (sequence, chunk, value head).  T and P are stored as MFMA
// A-operand fragments, 1 KiB each (lane l: 16 bytes at l*16, so one load or
// copy instruction of a wave moves 1 KiB of consecutive bytes).  Both are
// lower triangular, so of the (row block mi, k-step kb) pairs of 16 rows x
// 32 columns only six are nonzero: pair index pair_of(mi, kb) for
// (0,0) (1,0) (2,0) (2,1) (3,0) (3,1); each pair has a hi and a lo fragment
// (slots 2*pair and 2*pair + 1).  Lane l of a fragment holds row
// 16*mi + l%16 and, with g = l/16, columns 32*kb + 4g + 0..3 and
// 32*kb + 16 + 4g + 0..3 (order "pi").
// The pi order matches the MFMA result layout: a lane's result rows
// 4g + 0..3 of two adjacent 16-row blocks are exactly the contraction entries
// that the lane supplies in pi order, so results feed the next product from
// registers (the contraction is a sum; both operands use the same order).
struct WsLayout {
  static constexpr size_t kSlot = 64 * 16;
  static constexpr size_t kT = 0;              // 12 slots
  static constexpr size_t kP = 12 * kSlot;     // 12 slots
  static constexpr size_t kVec = 24 * kSlot;   // float [4][64]: sb sk so sd
  static constexpr size_t kGc = kVec + 4 * kC * sizeof(float);  // {gamma_63, 0, 0, 0}
  static constexpr size_t kBytes = (kGc + 16 + 255) & ~size_t(255);
};

__host__ __device__ constexpr int pair_of(int mi, int kb) {
  return mi < 2 ? mi : 2 * mi - 2 + kb;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two f32 values as packed bf16 pairs: hi = bf16(x) and lo = bf16(x - hi)
// (round to nearest even, v_cvt_pk_bf16_f32); x = hi + lo + ~2^-17 |x|.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi,
                                       uint32_t& lo) {
  const f32x2 x = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  const f32x2 xh = {__uint_as_float(hi << 16),
                    __uint_as_float(hi & 0xffff0000u)};
  const f32x2 r = {x[0] - xh[0], x[1] - xh[1]};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// Split-bf16 words of two result tiles in pi order: elements 0..3 from tile
// t0, 4..7 from tile t1.
__device__ __forceinline__ void split_pi(const f32x4& t0, const f32x4& t1,
                                         uint32_t (&hi)[4], uint32_t (&lo)[4]) {
  split2(t0[0], t0[1], hi[0], lo[0]);
  split2(t0[2], t0[3], hi[1], lo[1]);
  split2(t1[0], t1[1], hi[2], lo[2]);
  split2(t1[2], t1[3], hi[3], lo[3]);
}

__device__ __forceinline__ float bf16_f(u16 b) {
  return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b,
                                      f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// ------------------------------------------------------------------ p1
// Wave w owns the rows i = 16w..16w+15 of the chunk.  It computes the tiles
// (j-block nt <= w, i-block w) of K K^T and K Q^T with K rows as the A
// operand (K staged once in LDS, Q fragments loaded into registers); in the MFMA
// result layout a lane then holds, for its row i, four consecutive columns
// j of each tile -- exactly the lane's part of a pi-order A fragment of P,
// which is split and written without passing through LDS.  L goes to LDS
// transposed (Lt[j][i]) for the inversion.  The squared key norms are the
// diagonal of K K^T; the query norms come from the wave's Q fragments.
__global__ __launch_bounds__(kThreads) void p1_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k,
    const float* __restrict__ beta, const float* __restrict__ g,
    uint8_t* __restrict__ ws, PDims d) {
  constexpr int KS = kD + 8;  // padded bf16 row of K
  constexpr int FS = kC + 1;  // padded f32 row of T
  constexpr int LS = kC + 4;  // padded f32 row of Lt, 16-byte aligned
  __shared__ __attribute__((aligned(16))) u16 Ks[kC * KS];      // K rows; later T
  __shared__ __attribute__((aligned(16))) float Lt[kC * LS];  // L transposed
  float* Ts = reinterpret_cast<float*>(Ks);  // written once K is consumed
  static_assert(sizeof(float) * kC * FS <= sizeof(u16) * kC * KS, "alias");
  __shared__ float rk_s[kC], rq_s[kC], G_s[kC], b_s[kC];
  __shared__ int R_s[kC];  // last reset at or before the token, -1 if none

  const int bid = blockIdx.x;
  const int h = bid % d.Hv;
  const int c = (bid / d.Hv) % d.n_chunks;
  const int s = bid / (d.Hv * d.n_chunks);
  const int kh = h / d.group;
  const int t0 = c * d.chunk;
  const int nv = min(d.chunk, d.L - t0);  // valid rows of this chunk
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int l = tid % 64;
  const int n = l % 16, g4 = l / 16;

  // ---- K rows to LDS, Q fragments of block w to registers.  Rows past the
  // end of the sequence are read from the last valid row (no branch around
  // the loads): they only meet beta = 0, or feed output rows that are not
  // stored.
  const int last = nv - 1;
  const size_t rs = (size_t)d.Hk * kD;  // row stride
  const u16* kbase = k + (((size_t)s * d.L + t0) * d.Hk + kh) * kD;
  const u16* qbase = q + (((size_t)s * d.L + t0) * d.Hk + kh) * kD + 8 * g4;
  uint4 QW[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    QW[ks] = *reinterpret_cast<const uint4*>(qbase + min(16 * w + n, last) * rs + 32 * ks);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = it * kThreads + tid;  // 1024 pieces of 8 bf16
    const int row = idx / 16, col = (idx % 16) * 8;
    *reinterpret_cast<uint4*>(&Ks[row * KS + col]) =
        *reinterpret_cast<const uint4*>(kbase + min(row, last) * rs + col);
  }
  if (tid < kC) {
    const size_t gi = ((size_t)s * d.L + t0 + min(tid, last)) * d.Hv + h;
    const float bb = (tid < nv) ? beta[gi] : 0.f;
    const float gg = (tid < nv) ? g[gi] : 0.f;
    b_s[tid] = bb;
    // segmented inclusive prefix sum of g over the chunk (wave 0), fixed
    // order.  A gate below kReset (its exponential is 0 in f32; g = -inf
    // included) starts a new segment and adds 0, so every decay between two
    // tokens of one segment is exp of a difference of finite sums, and a
    // decay across a reset is exactly 0 (never inf - inf).  Without resets
    // this is the plain prefix sum.
    const bool reset = gg < kReset;
    float x = reset ? 0.f : gg;
    int head = reset ? 1 : 0;
    int lr = reset ? tid : -1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      const int hy = __shfl_up(head, off, 64);
      const int ly = __shfl_up(lr, off, 64);
      if (tid >= off) {
        if (!head) x += y;
        head |= hy;
        lr = max(lr, ly);
      }
    }
    G_s[tid] = x;
    R_s[tid] = lr;
  }
  __syncthreads();  // K rows, b, G in LDS

  // ---- AK[nt] = (K K^T)[16nt + 4g4 + e][16w + n], AQ[nt] = (K Q^T)[...]
  f32x4 AK[4], AQ[4];
  uint4 KW[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    KW[ks] = *reinterpret_cast<const uint4*>(&Ks[(16 * w + n) * KS + 32 * ks + 8 * g4]);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    AK[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    AQ[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nt <= w) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&Ks[(16 * nt + n) * KS + 32 * ks + 8 * g4]));
        AK[nt] = mfma(a, as_bf16x8(KW[ks]), AK[nt]);
        AQ[nt] = mfma(a, as_bf16x8(QW[ks]), AQ[nt]);
      }
    }
  }
  // ---- inverse norms of the rows i = 16w + n: |k_i|^2 is the diagonal of
  // the tile nt = w (lane with 4*g4 + e = n); |q_i|^2 from the Q fragments
  {
    float sq = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t wd[4] = {QW[ks].x, QW[ks].y, QW[ks].z, QW[ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(wd[e] << 16), hi = __uint_as_float(wd[e] & 0xffff0000u);
        sq = __builtin_fmaf(lo, lo, sq);
        sq = __builtin_fmaf(hi, hi, sq);
      }
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    float kk = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      if (nt == w) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * g4 + e == n) kk = AK[nt][e];
      }
    if (g4 == n / 4) rk_s[16 * w + n] = d.l2norm ? __builtin_amdgcn_rsqf(kk + 1e-6f) : 1.0f;
    if (g4 == 0) rq_s[16 * w + n] = d.l2norm ? __builtin_amdgcn_rsqf(sq + 1e-6f) : 1.0f;
  }
  __syncthreads();  // norms, b, G in LDS

  // ---- L (strict lower, to LDS transposed) and P (lower with diagonal,
  // kept in registers) for row i = 16w + n, columns j = 16nt + 4g4 + e.  The
  // decay is formed for every entry (its exponent clamped to 0 above the
  // diagonal, where the entry is 0), so no branch surrounds the exponential.
  uint8_t* wsb = ws + ((size_t)bid) * WsLayout::kBytes;
  {
    const int i = 16 * w + n;
    const float Gi = G_s[i], bki = b_s[i] * rk_s[i], sqi = d.scale * rq_s[i];
    const int Ri = R_s[i];
    f32x4 pv[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      pv[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (nt <= w) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * nt + 4 * g4 + e;
          const float rkj = rk_s[j];
          // 0 across a reset between j and i
          const float dec = Ri <= j ? __expf(j <= i ? Gi - G_s[j] : 0.f) : 0.f;
          const float lraw = bki * rkj * AK[nt][e] * dec;
          const float praw = sqi * rkj * AQ[nt][e] * dec;
          Lt[j * LS + i] = (j < i) ? lraw : 0.f;
          pv[nt][e] = (j <= i) ? praw : 0.f;
        }
      }
    }
    // P fragments, pi order: columns 32kb + 4g4 + 0..3 (tile 2kb) and
    // 32kb + 16 + 4g4 + 0..3 (tile 2kb + 1)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb == 1 && w < 2) break;
      uint32_t hi[4], lo[4];
      split_pi(pv[2 * kb], pv[2 * kb + 1], hi, lo);
      uint4* pdst = reinterpret_cast<uint4*>(wsb + WsLayout::kP) + 2 * pair_of(w, kb) * 64 + l;
      pdst[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      pdst[64] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  __syncthreads();  // Lt complete

  // ---- T = (I + L)^-1, step 1: the four 16x16 diagonal blocks.  Wave b,
  // lane jj < 16 computes column jj of block b by right-looking
  // substitution: once t_x is known, it updates the partial sums of every
  // later row, so the dependent chain is one FMA per row instead of a dot
  // product per row.  (The other lanes stay idle: every lane reads the same
  // L entries, and fewer active lanes draw less LDS bandwidth.)
  if (l < 16) {
    const int b0 = 16 * w, jj = l;
    float acc[16], t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const float tx = (x == jj) ? 1.f : ((x < jj) ? 0.f : -acc[x]);
      t[x] = tx;
      const float* colx = &Lt[(b0 + x) * LS + b0];  // L[b0 + r][b0 + x]
#pragma unroll
      for (int r = x + 1; r < 16; ++r) acc[r] = __builtin_fmaf(colx[r], tx, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ts[(b0 + r) * FS + b0 + jj] = t[r];
  }
  __syncthreads();

  // ---- step 2: block rows 1..3, T_ib = -T_ii sum_{m=b}^{i-1} L_im T_mb, on
  // f32 MFMA (v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][l/16] and
  // B[l/16][l%16] and holds D[4*(l/16) + e][l%16]); wave b computes block
  // (i, b), the product Y = sum L_im T_mb goes through the wave's own LDS
  // tile to become the B operand of T_ii Y.
  __shared__ float Ys[4][16 * 17];
  for (int bi = 1; bi < 4; ++bi) {
    if (w < bi) {
      const int bb = w, nn = l & 15, g4 = l >> 4;
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
      for (int m = bb; m < bi; ++m) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kr = 16 * m + 4 * ks + g4;
          Y = __builtin_amdgcn_mfma_f32_16x16x4f32(Lt[kr * LS + 16 * bi + nn],
                                                   Ts[kr * FS + 16 * bb + nn], Y, 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Ys[bb][(4 * g4 + e) * 17 + nn] = Y[e];
      // the wave's own Ys block is read back by the same wave only
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      f32x4 Tv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        Tv = __builtin_amdgcn_mfma_f32_16x16x4f32(Ts[(16 * bi + nn) * FS + 16 * bi + 4 * ks + g4],
                                                  Ys[bb][(4 * ks + g4) * 17 + nn], Tv, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ts[(16 * bi + 4 * g4 + e) * FS + 16 * bb + nn] = -Tv[e];
    }
    __syncthreads();
  }

  // ---- write T (pi order) as split bf16 fragments, and the row vectors
  {
    const int i = 16 * w + l % 16;
    for (int kb = 0; kb < (w >= 2 ? 2 : 1); ++kb) {
      const int pr = pair_of(w, kb);
      uint4* tdst = reinterpret_cast<uint4*>(wsb + WsLayout::kT) + 2 * pr * 64 + l;
      uint32_t hi[4], lo[4];
      const int ja = 32 * kb + 4 * g4, jb = ja + 16;
      // columns jb lie in the strictly upper block (0,1) or (2,3) of T,
      // which is zero and never written
      const bool zb = (w == 0 && kb == 0) || (w == 2 && kb == 1);
      split2(Ts[i * FS + ja], Ts[i * FS + ja + 1], hi[0], lo[0]);
      split2(Ts[i * FS + ja + 2], Ts[i * FS + ja + 3], hi[1], lo[1]);
      split2(zb ? 0.f : Ts[i * FS + jb], zb ? 0.f : Ts[i * FS + jb + 1], hi[2], lo[2]);
      split2(zb ? 0.f : Ts[i * FS + jb + 2], zb ? 0.f : Ts[i * FS + jb + 3], hi[3], lo[3]);
      tdst[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      tdst[64] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  if (tid < kC) {
    const int i = tid;
    // decays from the chunk start (gamma) and to the chunk end, 0 across a
    // reset
    const float Gc = G_s[kC - 1];
    const int Rc = R_s[kC - 1];
    const float gam = R_s[i] < 0 ? __expf(G_s[i]) : 0.f;
    float* vec = reinterpret_cast<float*>(wsb + WsLayout::kVec);
    vec[i] = b_s[i];                                  // sb: beta
    vec[kC + i] = b_s[i] * gam * rk_s[i];             // sk: beta gamma rk
    vec[2 * kC + i] = gam * rq_s[i] * d.scale;        // so: gamma rq scale
    vec[3 * kC + i] = Rc <= i ? rk_s[i] * __expf(Gc - G_s[i]) : 0.f;  // sd: rk exp(G_63 - G_i)
    if (i == 0)
      *reinterpret_cast<float4*>(wsb + WsLayout::kGc) =
          make_float4(Rc < 0 ? __expf(Gc) : 0.f, 0.f, 0.f, 0.f);
  }
}

// ------------------------------------------------------------------ p2
// One workgroup of four waves per (sequence, value head, 16-column tile of
// d_v), sequential over the chunks.  The work is split by role so that the
// chunk-to-chunk recurrence never waits on global memory or on other waves:
//   wave 0  the state chain.  Holds the 128 x 16 f32 state tile H in MFMA
//           result registers and per chunk computes K H, X, V_new = T X and
//           H' = gamma_63 H + K^T diag(sd) V_new.  Every operand comes from
//           LDS (read one stage ahead) or from its own registers (pi order,
//           see WsLayout).  It publishes H and V_new to LDS for the output
//           waves.
//   wave 1, 2  O = diag(so) Q H + P V_new for row blocks {0, 3} / {1, 2},
//           with Q and P loaded straight into registers one chunk ahead.
//   wave 3  stages the chain's operands (K rows, T fragments, the V tile,
//           the row vectors) into LDS two chunks ahead.
// Several waves issue global loads because one wave alone draws only about
// a quarter of what a CU can take from L2.  One barrier per chunk.  Interval
// c (between barriers) holds the second half of chunk c on the chain
// (V_new -> H') and the first half of chunk c + 1 (K H -> X -> V_new), while
// the output waves produce O of chunk c.  Every LDS buffer rotates over
// three chunks (c, c + 1 in use, c + 2 being written).
constexpr int kP2Threads = 256;

typedef short v4s __attribute__((ext_vector_type(4)));

// Staged K rows: row stride kKS (padded against bank conflicts) and, inside
// each 32-column block, the 4-column groups stored in the order
// 0 4 1 5 2 6 3 7, so that the pi-order A fragment of K H (columns
// 32*kb + 4g + 0..3 and 32*kb + 16 + 4g + 0..3) is one 16-byte read at
// 32*kb + 8g.  kpos(col) is the stored position of a column.
constexpr int kKS = kD + 8;
__host__ __device__ constexpr int kpos(int col) {
  return (col & ~31) + 4 * (((col >> 2) & 3) * 2 + ((col >> 4) & 1)) + (col & 3);
}
constexpr int kSVS = kC + 4;  // row stride of the transposed sb V tile (f32)
constexpr int kWarm = 5;      // chunks ahead that the output waves warm L2 for

// LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group g, lane
// i receives element i%4 of the 8 bytes addressed by lane 16g + 4e + i/4 as
// its element e (e = 0..3).
__device__ __forceinline__ uint2 tr_read(const u16* p) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ bf16x8 frag(uint2 a, uint2 b) {
  return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}

__device__ __forceinline__ bf16x8 words(const uint32_t (&x)[4]) {
  return as_bf16x8(make_uint4(x[0], x[1], x[2], x[3]));
}

// Operands staged into LDS by the staging wave, in flight from one interval
// to the next.
struct KvTransit {
  uint4 k[16];  // 64 K rows x 128 columns
  uint4 t[12];  // the T fragments
  uint4 v[2];   // 64 rows x 16 columns of V
  float sb[2];  // sb of the two V rows of the lane
  uint4 vec;    // the row vectors
  uint4 gc;     // gamma_63
};


// Per-chunk operands of an output wave (row blocks mA with one k-step, mB
// with two).
struct OutOps {
  uint4 qa[4], qb[4];  // Q A fragments (natural order)
  uint4 p[3][2];       // P fragments, pi order (hi, lo): (mA,0), (mB,0), (mB,1)
};

// LDS of a p2 workgroup, shared by the role functions below.
struct P2Lds {
  __attribute__((aligned(16))) u16 Kr[3][kC * kKS];       // K rows (kpos order)
  __attribute__((aligned(16))) uint4 Tf[3][12][64];       // T fragments
  __attribute__((aligned(16))) float SVt[3][kTile * kSVS]; // diag(sb) V, [col][row]
  __attribute__((aligned(16))) float Vec[3][4 * kC + 4];  // sb sk so sd, gamma
  __attribute__((aligned(16))) uint4 Hf[3][8][64];        // H (natural B)
  __attribute__((aligned(16))) float Vf[3][2][64][8];     // V_new f32 (pi-order B rows)
};
__shared__ P2Lds p2lds;

// A pointer argument made wave-uniform, rebuilt as a global-memory pointer
// (cast back to a generic pointer, which address-space inference turns into
// global loads and stores rather than flat ones).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  typedef T __attribute__((address_space(1))) GlobalT;
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  GlobalT* gp = reinterpret_cast<GlobalT*>(((uint64_t)hi << 32) | lo);
  return (T*)gp;
}

__device__ __forceinline__ PDims uniform_dims(const PDims& a) {
  PDims r;
  r.n_seqs = __builtin_amdgcn_readfirstlane(a.n_seqs);
  r.L = __builtin_amdgcn_readfirstlane(a.L);
  r.Hv = __builtin_amdgcn_readfirstlane(a.Hv);
  r.Hk = __builtin_amdgcn_readfirstlane(a.Hk);
  r.group = __builtin_amdgcn_readfirstlane(a.group);
  r.n_chunks = __builtin_amdgcn_readfirstlane(a.n_chunks);
  r.chunk = __builtin_amdgcn_readfirstlane(a.chunk);
  r.segs = __builtin_amdgcn_readfirstlane(a.segs);
  r.seq_L = __builtin_amdgcn_readfirstlane(a.seq_L);
  r.seq_chunks = __builtin_amdgcn_readfirstlane(a.seq_chunks);
  r.L_last = __builtin_amdgcn_readfirstlane(a.L_last);
  r.ckpt_interval = __builtin_amdgcn_readfirstlane(a.ckpt_interval);
  r.scale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.scale)));
  r.l2norm = __builtin_amdgcn_readfirstlane(a.l2norm);
  return r;
}

// Where part s of a P2 launch lies: its first token and first chunk
// within the whole batch, and its length.
struct PartPos {
  size_t t0, c0;
  int len;
};
__device__ __forceinline__ PartPos part_pos(const PDims& d, int s) {
  const int seq = s / d.segs, j = s - seq * d.segs;
  PartPos p;
  p.t0 = (size_t)seq * d.seq_L + (size_t)j * d.L;
  p.c0 = (size_t)seq * d.seq_chunks + (size_t)j * d.n_chunks;
  p.len = j == d.segs - 1 ? d.L_last : d.L;
  return p;
}

// The two roles are separate functions so that the compiler allocates
// registers for each on its own (inlined into one kernel, the barriers that
// both roles execute get merged and the state of both roles is kept live
// at once).
template <int MODE>
static __device__ __attribute__((noinline)) void p2_chain(
    const u16* q_, const u16* k_, const u16* v_, const uint8_t* ws_,
    const float* S_init_, float* S_final_, float* o_, float* ckpt_,
    const PDims d_, const int tile_, const int h_, const int s_, const int kh_) {
  // arguments of a device function arrive in VGPRs: make their uniformity
  // explicit so that addresses and branches stay scalar
  const u16* __restrict__ q = uniform_ptr(q_);
  const u16* __restrict__ k = uniform_ptr(k_);
  const u16* __restrict__ v = uniform_ptr(v_);
  const uint8_t* __restrict__ ws = uniform_ptr(ws_);
  const float* __restrict__ S_init = uniform_ptr(S_init_);
  float* __restrict__ S_final = uniform_ptr(S_final_);
  float* __restrict__ o = uniform_ptr(o_);
  float* __restrict__ ckpt = uniform_ptr(ckpt_);
  const PDims d = uniform_dims(d_);
  const int tile = __builtin_amdgcn_readfirstlane(tile_);
  const int h = __builtin_amdgcn_readfirstlane(h_);
  const int s = __builtin_amdgcn_readfirstlane(s_);
  const int kh = __builtin_amdgcn_readfirstlane(kh_);
  (void)q; (void)k; (void)v; (void)S_init; (void)S_final; (void)o; (void)ckpt; (void)kh;
  auto& Kr = p2lds.Kr;
  auto& Tf = p2lds.Tf;
  auto& SVt = p2lds.SVt;
  auto& Vec = p2lds.Vec;
  auto& Hf = p2lds.Hf;
  auto& Vf = p2lds.Vf;
  const int l = threadIdx.x % 64;
  const int n = l % 16;   // result column inside the tile
  const int g = l / 16;   // lane group
  const int col = kTile * tile + n;
  // the last piece of a sequence may be shorter (segmented prefill)
  const PartPos pp = part_pos(d, s);
  const int Ls = pp.len;
  const int nch = (Ls + d.chunk - 1) / d.chunk;
  // per-sequence bases; element offsets below fit in 32 bits (host check)
  const u16* __restrict__ qs = q + pp.t0 * d.Hk * kD;
  const u16* __restrict__ kseq = k + pp.t0 * d.Hk * kD;
  const u16* __restrict__ vs = v + pp.t0 * d.Hv * kD;
  float* __restrict__ os = o + pp.t0 * d.Hv * kD;
  const uint8_t* __restrict__ wss =
      ws + (pp.c0 * d.Hv + h) * WsLayout::kBytes;
  const size_t ws_chunk = (size_t)d.Hv * WsLayout::kBytes;
  (void)qs; (void)kseq; (void)vs; (void)os; (void)wss; (void)ws_chunk;
  (void)Kr; (void)Tf; (void)SVt; (void)Vec; (void)Hf; (void)Vf; (void)col;
  // ================================================================ chain
  // H[mb]: state rows dk = 16*mb + 4g + e, column col
  f32x4 H[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * mb + 4 * g + e;
      if constexpr ((MODE & kModeIdentity) != 0)
        H[mb][e] = r == col ? 1.f : 0.f;
      else
        H[mb][e] = S_init ? S_init[(((size_t)s * d.Hv + h) * kD + r) * kD + col] : 0.f;
    }
  uint32_t hw[4][4], lw[4][4];  // split H, pi order per 32-row k-step
  f32x4 VN[4];                  // V_new rows 16*mi + 4g + e

  // Lane constants: element offsets of the K pieces inside one buffer.
  // K H A fragment (mj, kb): row 16*mj + n, stored columns 32*kb + 8g + 0..7,
  //   at ka + 16*kKS*mj + 32*kb.
  // K^T pieces (transposing reads, columns 16*mb + 4*(n%4) + 0..3 of row
  //   32*kb + 16*s + 4g + n/4), at kt + (32*kb + 16*s)*kKS + kpos(16*mb).
  const int ka = n * kKS + 8 * g;
  const int kt = (4 * g + (n >> 2)) * kKS + 8 * (n & 3);

  // H as natural B fragments for the output waves, 32 rows (pair pq of
  // 16-row blocks) at a time: rows 16*mb + 4g + e of a 32-row k-step are B
  // rows 8*gp + ep with gp = 2*(mb%2) + g/2 and ep = 4*(g%2) + e
  auto publish_pair = [&](auto pb, int pq) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int gp = 2 * t + (g >> 1);
      uint2* dh = reinterpret_cast<uint2*>(&Hf[pb][2 * pq][16 * gp + n]) + (g & 1);
      uint2* dl = reinterpret_cast<uint2*>(&Hf[pb][2 * pq + 1][16 * gp + n]) + (g & 1);
      *dh = make_uint2(hw[pq][2 * t], hw[pq][2 * t + 1]);
      *dl = make_uint2(lw[pq][2 * t], lw[pq][2 * t + 1]);
    }
  };
  // Operand fragments are read from LDS well before the MFMAs that use them
  // (an LDS read takes about as long as four to six MFMAs):
  //   KA[kb]  A fragments of K H (for the next chunk, during H')
  //   KT[kb]  A fragments of K^T for H' (k-step 0 after K H of the chunk,
  //           k-step 1 at the start of H')
  //   TF[pr]  T fragments (during the last k-steps of K H)
  bf16x8 KA[4][4], KT[2][8], TF[6][2];
  f32x4 KH[4], SV[4], SK[4];
  auto sched_fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // ask the scheduler to alternate one MFMA with up to three VALU
  // instructions and one LDS access, n times, over the region before the
  // next fence: VALU work then issues while the MFMAs run
  auto interleave = [](auto n) {
#pragma unroll
    for (int i = 0; i < decltype(n)::value; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);
    }
  };
  auto read_KA = [&](auto B, int kb0, int kb1) {
    const u16* K = Kr[B];
#pragma unroll
    for (int kb = kb0; kb < kb1; ++kb)
#pragma unroll
      for (int mj = 0; mj < 4; ++mj)
        KA[kb][mj] = as_bf16x8(*reinterpret_cast<const uint4*>(&K[ka + 16 * kKS * mj + 32 * kb]));
  };
  auto read_KT = [&](auto B, int kb) {
    const u16* K = Kr[B];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      KT[kb][mb] = frag(tr_read(&K[kt + 32 * kb * kKS + kpos(16 * mb)]),
                        tr_read(&K[kt + (32 * kb + 16) * kKS + kpos(16 * mb)]));
  };
  // T fragments and the row data of X (sb V and sk) of the chunk in buffer B
  auto read_front_ops = [&](auto B) {
#pragma unroll
    for (int pr = 0; pr < 6; ++pr) {
      TF[pr][0] = as_bf16x8(Tf[B][2 * pr][l]);
      TF[pr][1] = as_bf16x8(Tf[B][2 * pr + 1][l]);
    }
#pragma unroll
    for (int mj = 0; mj < 4; ++mj) {
      if constexpr ((MODE & kModeVZero) != 0)
        SV[mj] = f32x4{0.f, 0.f, 0.f, 0.f};
      else
        SV[mj] = *reinterpret_cast<const f32x4*>(&SVt[B][n * kSVS + 16 * mj + 4 * g]);
      SK[mj] = *reinterpret_cast<const f32x4*>(&Vec[B][kC + 16 * mj + 4 * g]);
    }
  };
  // K H, k-step kb (H split hw/lw, both passes)
  auto kh_step = [&](int kb) {
    const bf16x8 bh = words(hw[kb]), bl = words(lw[kb]);
#pragma unroll
    for (int mj = 0; mj < 4; ++mj) KH[mj] = mfma(KA[kb][mj], bh, KH[mj]);
#pragma unroll
    for (int mj = 0; mj < 4; ++mj) KH[mj] = mfma(KA[kb][mj], bl, KH[mj]);
  };
  // the chunk in buffer B from K H (complete) to V_new, published in f32
  // for the output waves (same row mapping as publish_pair); X is split and
  // multiplied by T one k-step at a time
  auto finish_front = [&](auto B) {
    constexpr int bb = decltype(B)::value;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) VN[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 X[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int mj = 2 * kb + t;
#pragma unroll
        for (int e = 0; e < 4; ++e) X[t][e] = __builtin_fmaf(-SK[mj][e], KH[mj][e], SV[mj][e]);
      }
      uint32_t xh[4], xl[4];
      split_pi(X[0], X[1], xh, xl);
      const bf16x8 bh = words(xh), bl = words(xl);
#pragma unroll
      for (int pass = 0; pass < 3; ++pass)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          if (kb == 1 && mi < 2) continue;
          const int pr = pair_of(mi, kb);
          VN[mi] = mfma(TF[pr][pass == 2 ? 1 : 0], pass == 1 ? bl : bh, VN[mi]);
        }
    }
    interleave(std::integral_constant<int, 18>{});
    // V_new for the output waves as pi-order B fragments: lane l holds rows
    // 32*kb + 4g + 0..3 and 32*kb + 16 + 4g + 0..3 (f32)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      *reinterpret_cast<f32x4*>(&Vf[bb][mi >> 1][l][4 * (mi & 1)]) = VN[mi];
  };

  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  typedef std::integral_constant<int, 2> B2;
  __syncthreads();  // chunks 0 and 1 staged
  // chunk 0 up to V_new
  read_KA(B0{}, 0, 4);
  read_front_ops(B0{});
#pragma unroll
  for (int pq = 0; pq < 4; ++pq) {
    split_pi(H[2 * pq], H[2 * pq + 1], hw[pq], lw[pq]);
    publish_pair(B0{}, pq);
  }
#pragma unroll
  for (int mj = 0; mj < 4; ++mj) KH[mj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) kh_step(kb);
  read_KT(B0{}, 0);
  finish_front(B0{});
  __syncthreads();
  // One interval: chunk c from V_new to H_{c+1}, software-pipelined with
  // chunk c + 1 up to V_new: each 32-row pair of H_{c+1} is split and
  // published and its K H k-step issued while the next pair's MFMAs run.
  // The buffers of chunk c and c + 1 are compile-time constants (the loop
  // is unrolled by three), so every LDS address is a lane constant plus an
  // immediate.  After the last chunk the second half runs on stale buffers
  // and its results are never read (no branch in the MFMA stream).
  auto step = [&](int c, auto B, auto NB) {
    const float* vc = Vec[B];
    const float gc = vc[4 * kC];
    f32x4 s0[2], s1[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s0[kb] = *reinterpret_cast<const f32x4*>(&vc[3 * kC + 32 * kb + 4 * g]);
      s1[kb] = *reinterpret_cast<const f32x4*>(&vc[3 * kC + 32 * kb + 16 + 4 * g]);
    }
    read_KT(B, 1);
    read_KA(NB, 0, 1);
    sched_fence();
    // D = diag(sd) V_new, split per k-step
    uint32_t dh[2][4], dl[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 D0, D1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        D0[e] = s0[kb][e] * VN[2 * kb][e];
        D1[e] = s1[kb][e] * VN[2 * kb + 1][e];
      }
      split_pi(D0, D1, dh[kb], dl[kb]);
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) H[mb][e] = gc * H[mb][e];
    // H' k-step 0 (tokens 0..31) for every row block
#pragma unroll
    for (int pq = 0; pq < 4; ++pq)
#pragma unroll
      for (int pass = 0; pass < 2; ++pass)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int mb = 2 * pq + t;
          H[mb] = mfma(KT[0][mb], words(pass ? dl[0] : dh[0]), H[mb]);
        }
    interleave(std::integral_constant<int, 16>{});
    sched_fence();
    read_KA(NB, 1, 4);
    sched_fence();
#pragma unroll
    for (int mj = 0; mj < 4; ++mj) KH[mj] = f32x4{0.f, 0.f, 0.f, 0.f};
    // H' k-step 1 pair by pair; pair pq - 1 is split, published and its
    // K H k-step issued behind pair pq's MFMAs
#pragma unroll
    for (int pq = 0; pq < 4; ++pq) {
#pragma unroll
      for (int pass = 0; pass < 2; ++pass)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int mb = 2 * pq + t;
          H[mb] = mfma(KT[1][mb], words(pass ? dl[1] : dh[1]), H[mb]);
        }
      if (pq >= 1) {
        split_pi(H[2 * pq - 2], H[2 * pq - 1], hw[pq - 1], lw[pq - 1]);
        publish_pair(NB, pq - 1);
        kh_step(pq - 1);
      }
      if (pq == 3) {
        interleave(std::integral_constant<int, 28>{});
        sched_fence();
        read_front_ops(NB);
        sched_fence();
      }
    }
    split_pi(H[6], H[7], hw[3], lw[3]);
    publish_pair(NB, 3);
    kh_step(3);
    const int t0 = c * d.chunk, nv = min(d.chunk, Ls - t0);
    // checkpoint after token t0 + nv when it is a multiple of the interval
    if (d.ckpt_interval > 0 && ckpt && (t0 + nv) % d.ckpt_interval == 0) {
      const int idx = (t0 + nv) / d.ckpt_interval - 1;
      const int n_ck = d.L / d.ckpt_interval;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * mb + 4 * g + e;
          ckpt[((((size_t)s * n_ck + idx) * d.Hv + h) * kD + r) * kD + col] = H[mb][e];
        }
    }
    sched_fence();
    read_KT(NB, 0);
    sched_fence();
    finish_front(NB);
    __syncthreads();
  };
  for (int c = 0; c < nch; c += 3) {
    step(c, B0{}, B1{});
    if (c + 1 < nch) step(c + 1, B1{}, B2{});
    if (c + 2 < nch) step(c + 2, B2{}, B0{});
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * mb + 4 * g + e;
      S_final[(((size_t)s * d.Hv + h) * kD + r) * kD + col] = H[mb][e];
    }
}

// Loads are unconditional: rows past the end of the sequence are read from
// the last valid row.  Their values never reach a result: P1 gives such rows
// beta = 0 (so X, V_new and their state contributions are 0), and their
// output rows are not stored.

// Staging wave: the K rows, the T fragments, sb V and the row vectors of
// chunk c + 2 are written to LDS in interval c (loaded during interval
// c - 1).
static __device__ __attribute__((noinline)) void p2_stage(
    const u16* q_, const u16* k_, const u16* v_, const uint8_t* ws_,
    const float* S_init_, float* S_final_, float* o_, float* ckpt_,
    const PDims d_, const int tile_, const int h_, const int s_, const int kh_) {
  const u16* __restrict__ q = uniform_ptr(q_);
  const u16* __restrict__ k = uniform_ptr(k_);
  const u16* __restrict__ v = uniform_ptr(v_);
  const uint8_t* __restrict__ ws = uniform_ptr(ws_);
  float* __restrict__ o = uniform_ptr(o_);
  const PDims d = uniform_dims(d_);
  const int tile = __builtin_amdgcn_readfirstlane(tile_);
  const int h = __builtin_amdgcn_readfirstlane(h_);
  const int s = __builtin_amdgcn_readfirstlane(s_);
  const int kh = __builtin_amdgcn_readfirstlane(kh_);
  (void)S_init_; (void)S_final_; (void)ckpt_;
  const int l = threadIdx.x % 64;
  const int n = l % 16;
  const int g = l / 16;
  const int col = kTile * tile + n;
  // the last piece of a sequence may be shorter (segmented prefill)
  const PartPos pp = part_pos(d, s);
  const int Ls = pp.len;
  const int nch = (Ls + d.chunk - 1) / d.chunk;
  const u16* __restrict__ qs = q + pp.t0 * d.Hk * kD;
  const u16* __restrict__ kseq = k + pp.t0 * d.Hk * kD;
  const u16* __restrict__ vs = v + pp.t0 * d.Hv * kD;
  float* __restrict__ os = o + pp.t0 * d.Hv * kD;
  const uint8_t* __restrict__ wss =
      ws + (pp.c0 * d.Hv + h) * WsLayout::kBytes;
  const size_t ws_chunk = (size_t)d.Hv * WsLayout::kBytes;
  (void)qs; (void)kseq; (void)vs; (void)os; (void)col; (void)g; (void)kh;
  auto& Kr = p2lds.Kr;
  auto& Tf = p2lds.Tf;
  auto& SVt = p2lds.SVt;
  auto& Vec = p2lds.Vec;
  auto load = [&](int c, KvTransit& tr) {
    const int t0 = c * d.chunk;
    const int last = min(d.chunk, Ls - t0) - 1;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int idx = it * 64 + l;
      const int row = idx >> 4, pc = idx & 15;
      tr.k[it] = *reinterpret_cast<const uint4*>(
          kseq + ((uint32_t)(t0 + min(row, last)) * d.Hk + kh) * kD + 8 * pc);
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int row = 32 * it + (l >> 1);
      tr.v[it] = *reinterpret_cast<const uint4*>(
          vs + ((uint32_t)(t0 + min(row, last)) * d.Hv + h) * kD + kTile * tile + 8 * (l & 1));
    }
    const uint8_t* wc = wss + (size_t)c * ws_chunk;
#pragma unroll
    for (int x = 0; x < 12; ++x) tr.t[x] = reinterpret_cast<const uint4*>(wc + WsLayout::kT)[x * 64 + l];
#pragma unroll
    for (int it = 0; it < 2; ++it)
      tr.sb[it] = reinterpret_cast<const float*>(wc + WsLayout::kVec)[32 * it + (l >> 1)];
    tr.vec = reinterpret_cast<const uint4*>(wc + WsLayout::kVec)[l];
    tr.gc = *reinterpret_cast<const uint4*>(wc + WsLayout::kGc);
  };
  auto store = [&](int buf, const KvTransit& tr) {
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int idx = it * 64 + l;
      const int row = idx >> 4, pc = idx & 15;
      const uint4 x = tr.k[it];
      // columns 8*pc + 0..3 and 8*pc + 4..7 land in separate groups
      *reinterpret_cast<uint2*>(&Kr[buf][row * kKS + kpos(8 * pc)]) = make_uint2(x.x, x.y);
      *reinterpret_cast<uint2*>(&Kr[buf][row * kKS + kpos(8 * pc + 4)]) = make_uint2(x.z, x.w);
    }
#pragma unroll
    for (int x = 0; x < 12; ++x) Tf[buf][x][l] = tr.t[x];
    // sb V, transposed to [column][row]
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int row = 32 * it + (l >> 1);
      const uint32_t w[4] = {tr.v[it].x, tr.v[it].y, tr.v[it].z, tr.v[it].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t b = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
        SVt[buf][(8 * (l & 1) + e) * kSVS + row] = tr.sb[it] * __uint_as_float(b);
      }
    }
    reinterpret_cast<uint4*>(Vec[buf])[l] = tr.vec;
    if (l == 0) reinterpret_cast<uint4*>(Vec[buf])[kC] = tr.gc;
  };
  KvTransit tr;
  load(0, tr);
  store(0, tr);
  if (nch > 1) {
    load(1, tr);
    store(1, tr);
  }
  if (nch > 2) load(2, tr);
  __syncthreads();  // chunks 0 and 1 staged
  __syncthreads();  // chain: chunk 0 up to V_new
  for (int c = 0; c < nch; ++c) {
    if (c + 2 < nch) store((c + 2) % 3, tr);
    load(min(c + 3, nch - 1), tr);  // unconditional, see p2_out
    __syncthreads();
  }
}

// Output wave ow (0 or 1): O = diag(so) Q H + P V_new for row blocks
// mA = ow (P has one k-step there) and mB = 3 - ow (two).  The output waves
// also warm L2 for chunk c + kWarm: the eight workgroups of a head (same
// XCD, same L2) each touch one eighth of the cache lines that the head's
// workgroups will load for that chunk, one dword per lane, so that the
// loads issued one or two chunks ahead find their data in L2.
template <int MODE>
static __device__ __attribute__((noinline)) void p2_out(
    const u16* q_, const u16* k_, const u16* v_, const uint8_t* ws_,
    const float* S_init_, float* S_final_, float* o_, float* ckpt_,
    const PDims d_, const int tile_, const int h_, const int s_, const int kh_, const int ow) {
  const u16* __restrict__ q = uniform_ptr(q_);
  const u16* __restrict__ k = uniform_ptr(k_);
  const u16* __restrict__ v = uniform_ptr(v_);
  const uint8_t* __restrict__ ws = uniform_ptr(ws_);
  float* __restrict__ o = uniform_ptr(o_);
  const PDims d = uniform_dims(d_);
  const int tile = __builtin_amdgcn_readfirstlane(tile_);
  const int h = __builtin_amdgcn_readfirstlane(h_);
  const int s = __builtin_amdgcn_readfirstlane(s_);
  const int kh = __builtin_amdgcn_readfirstlane(kh_);
  (void)S_init_; (void)S_final_; (void)ckpt_;
  const int l = threadIdx.x % 64;
  const int n = l % 16;
  const int g = l / 16;
  const int col = kTile * tile + n;
  // the last piece of a sequence may be shorter (segmented prefill)
  const PartPos pp = part_pos(d, s);
  const int Ls = pp.len;
  const int nch = (Ls + d.chunk - 1) / d.chunk;
  const u16* __restrict__ qs = q + pp.t0 * d.Hk * kD;
  const u16* __restrict__ kseq = k + pp.t0 * d.Hk * kD;
  const u16* __restrict__ vs = v + pp.t0 * d.Hv * kD;
  float* __restrict__ os = o + pp.t0 * d.Hv * kD;
  const uint8_t* __restrict__ wss =
      ws + (pp.c0 * d.Hv + h) * WsLayout::kBytes;
  const size_t ws_chunk = (size_t)d.Hv * WsLayout::kBytes;
  (void)qs; (void)kseq; (void)vs; (void)os; (void)col; (void)g; (void)kh;
  auto& Vec = p2lds.Vec;
  auto& Hf = p2lds.Hf;
  auto& Vf = p2lds.Vf;
  const int mA = ow, mB = 3 - ow;
  const int prA = pair_of(mA, 0), prB = pair_of(mB, 0);
  // L2 warm-up line of this lane: index u over the lines a head loads per
  // chunk (K rows 128, Q rows 128, V rows 128, workspace block), taken by
  // workgroup `tile` as u = 128*tile + 64*ow + l (lines past the end are
  // clamped to the last one)
  const int u = 128 * tile + 64 * ow + l;
  auto warm_at = [&](int c, int u) -> uint32_t {
    const int t0 = c * d.chunk;
    const int last = min(d.chunk, Ls - t0) - 1;
    const int row = min((u & 127) >> 1, last), half = u & 1;
    const uint32_t* p;
    if (u < 128)
      p = reinterpret_cast<const uint32_t*>(kseq + ((uint32_t)(t0 + row) * d.Hk + kh) * kD + 64 * half);
    else if (u < 256)
      p = reinterpret_cast<const uint32_t*>(qs + ((uint32_t)(t0 + row) * d.Hk + kh) * kD + 64 * half);
    else if (u < 384)
      p = reinterpret_cast<const uint32_t*>(vs + ((uint32_t)(t0 + row) * d.Hv + h) * kD + 64 * half);
    else
      p = reinterpret_cast<const uint32_t*>(
          wss + (size_t)c * ws_chunk + min((size_t)(u - 384) * 128, WsLayout::kBytes - 4));
    return *p;
  };
  auto warm = [&](int c) { return warm_at(c, u); };
  auto ops_load = [&](int c, OutOps& op) {
    const int t0 = c * d.chunk;
    const int last = min(d.chunk, Ls - t0) - 1;
    const uint32_t ra = ((uint32_t)(t0 + min(16 * mA + n, last)) * d.Hk + kh) * kD + 8 * g;
    const uint32_t rb = ((uint32_t)(t0 + min(16 * mB + n, last)) * d.Hk + kh) * kD + 8 * g;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      op.qa[kb] = *reinterpret_cast<const uint4*>(qs + ra + 32 * kb);
      op.qb[kb] = *reinterpret_cast<const uint4*>(qs + rb + 32 * kb);
    }
    const uint4* psrc = reinterpret_cast<const uint4*>(wss + (size_t)c * ws_chunk + WsLayout::kP);
    const int prs[3] = {prA, prB, prB + 1};
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      op.p[x][0] = psrc[2 * prs[x] * 64 + l];
      op.p[x][1] = psrc[(2 * prs[x] + 1) * 64 + l];
    }
  };
  auto outputs = [&](int c, const OutOps& op) {
    const int hb = c % 3, bb = c % 3;
    const int t0 = c * d.chunk, nv = min(d.chunk, Ls - t0);
    f32x4 QA = {0.f, 0.f, 0.f, 0.f}, QB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8 bh = as_bf16x8(Hf[hb][2 * kb][l]);
      const bf16x8 bl = as_bf16x8(Hf[hb][2 * kb + 1][l]);
      const bf16x8 aa = as_bf16x8(op.qa[kb]), ab = as_bf16x8(op.qb[kb]);
      QA = mfma(aa, bh, QA);
      QB = mfma(ab, bh, QB);
      QA = mfma(aa, bl, QA);
      QB = mfma(ab, bl, QB);
    }
    const f32x4 soA = *reinterpret_cast<const f32x4*>(&Vec[bb][2 * kC + 16 * mA + 4 * g]);
    const f32x4 soB = *reinterpret_cast<const f32x4*>(&Vec[bb][2 * kC + 16 * mB + 4 * g]);
    f32x4 OA, OB;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      OA[e] = soA[e] * QA[e];
      OB[e] = soB[e] * QB[e];
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&Vf[hb][kb][l][0]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&Vf[hb][kb][l][4]);
      uint32_t hi[4], lo[4];
      split2(v0[0], v0[1], hi[0], lo[0]);
      split2(v0[2], v0[3], hi[1], lo[1]);
      split2(v1[0], v1[1], hi[2], lo[2]);
      split2(v1[2], v1[3], hi[3], lo[3]);
      const bf16x8 vh = words(hi), vl = words(lo);
      const bf16x8 ph = as_bf16x8(op.p[1 + kb][0]), pl = as_bf16x8(op.p[1 + kb][1]);
      OB = mfma(ph, vh, OB);
      OB = mfma(ph, vl, OB);
      OB = mfma(pl, vh, OB);
      if (kb == 0) {
        const bf16x8 qh = as_bf16x8(op.p[0][0]), ql = as_bf16x8(op.p[0][1]);
        OA = mfma(qh, vh, OA);
        OA = mfma(qh, vl, OA);
        OA = mfma(ql, vh, OA);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ra = 16 * mA + 4 * g + e, rb = 16 * mB + 4 * g + e;
      if (ra < nv) os[((uint32_t)(t0 + ra) * d.Hv + h) * kD + col] = OA[e];
      if (rb < nv) os[((uint32_t)(t0 + rb) * d.Hv + h) * kD + col] = OB[e];
    }
  };

  if constexpr ((MODE & kModeNoOut) != 0) {
    // the barriers and the L2 warm-up of both output waves' lines
    __syncthreads();
    __syncthreads();
    uint32_t w0 = 0, w1 = 0;
    for (int c = 0; c < nch; ++c) {
      const int cw = min(c + kWarm, nch - 1);
      const uint32_t w2 = warm_at(cw, u) ^ warm_at(cw, u + 64);
      asm volatile("" ::"v"(w0));
      w0 = w1;
      w1 = w2;
      __syncthreads();
    }
    asm volatile("" ::"v"(w0), "v"(w1));
    return;
  }
  OutOps A, B;
  ops_load(0, A);
  __syncthreads();  // chunks 0 and 1 staged
  __syncthreads();  // chain: chunk 0 up to V_new
  // interval c: warm L2 for chunk c + kWarm, load the output operands of
  // chunk c + 1, then O of chunk c.  Loads are issued unconditionally, past
  // the last chunk for the last chunk again (a load under a branch makes the
  // compiler wait for every outstanding load where the branches join); a
  // warm-up value is consumed two intervals later, when it has long arrived.
  uint32_t w0 = 0, w1 = 0;
  auto interval = [&](int c, const OutOps& cur, OutOps& nxt) {
    const uint32_t w2 = warm(min(c + kWarm, nch - 1));
    ops_load(min(c + 1, nch - 1), nxt);
    outputs(c, cur);
    asm volatile("" ::"v"(w0));
    w0 = w1;
    w1 = w2;
    __syncthreads();
  };
  for (int c = 0; c < nch; c += 2) {
    interval(c, A, B);
    if (c + 1 < nch) interval(c + 1, B, A);
  }
  asm volatile("" ::"v"(w0), "v"(w1));
}

template <int MODE>
__global__ __launch_bounds__(kP2Threads) void p2_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k,
    const u16* __restrict__ v, const uint8_t* __restrict__ ws,
    const float* __restrict__ S_init, float* __restrict__ S_final,
    float* __restrict__ o, float* __restrict__ ckpt, PDims d) {
  // block -> (sequence, head, tile); the tiles of a head share one XCD
  const int nb = gridDim.x;
  int b = blockIdx.x;
  if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
  const int tile = b % (kD / kTile);
  const int h = (b / (kD / kTile)) % d.Hv;
  const int s = b / ((kD / kTile) * d.Hv);
  const int kh = h / d.group;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  if constexpr (MODE == kModePair) {
    // One segment and column tile, two chains on one staging: wave 0 runs
    // the chain from the identity with V taken as zero (its end state, the
    // segment's transition A_s, goes to S_final), wave 1 the chain from zero
    // (the offset B_s, to the array passed as o: a pair pass writes no
    // outputs).  Wave 2 only warms L2.  Both chains publish H and V_new to
    // the same LDS buffers, which nothing reads in this pass.
    if (w == 0)
      p2_chain<kModeIdentity | kModeVZero>(q, k, v, ws, nullptr, S_final, o,
                                           nullptr, d, tile, h, s, kh);
    else if (w == 1)
      p2_chain<0>(q, k, v, ws, nullptr, o, o, nullptr, d, tile, h, s, kh);
    else if (w == 2)
      p2_out<kModeNoOut>(q, k, v, ws, S_init, S_final, o, ckpt, d, tile, h, s, kh, 0);
    else
      p2_stage(q, k, v, ws, S_init, S_final, o, ckpt, d, tile, h, s, kh);
  } else {
    if (w == 0)
      p2_chain<0>(q, k, v, ws, S_init, S_final, o, ckpt, d, tile, h, s, kh);
    else if (w < 3)
      p2_out<0>(q, k, v, ws, S_init, S_final, o, ckpt, d, tile, h, s, kh, w - 1);
    else
      p2_stage(q, k, v, ws, S_init, S_final, o, ckpt, d, tile, h, s, kh);
  }
}

// ------------------------------------------------------------ segments
// Sequence-parallel prefill of a batch with few sequence-heads.  The P2
// chains are sequential over the chunks, and n_seqs sequences of h_v heads
// make only 8 n_seqs h_v of them: with fewer chains than CUs the chip idles.  The state after
// a segment of kSeg tokens is affine in the state before it,
// H_end = A_s H_start + B_s (stored orientation, A_s d_k x d_k): A_s is the
// chain run from the identity with V taken as zero, B_s the chain run from
// zero.  So the prefill runs as
//   P1 over the whole sequences;
//   P2 on every segment but the last of each sequence as kModePair: in
//     one workgroup per segment and column tile, the chain from the
//     identity with V taken as zero (giving A_s) and the chain from zero
//     (giving B_s) share one staging of the segment's operands;
//   seg_scan_kernel: H_0 = S_init, H_{s+1} = A_s H_s + B_s;
//   P2 on every segment from H_s, producing the outputs;
//   seg_place_kernel: checkpoints and S_final.
// The segments start at multiples of kSeg, which divides the checkpoint
// interval, so every checkpoint is a segment boundary and holds the scanned
// state that the next segment started from.  A prefill resumed from a
// checkpoint cuts its segments at the same tokens, starts its scan from that
// state and repeats the same operations: it reproduces the rest bit for bit.
constexpr int kSeg = 4096;       // tokens per segment (a multiple of every chunk)
constexpr int kSegMaxHeads = 8;  // sequences x heads: at most 64 chains, a quarter of the CUs

// The scan H_{s+1} = A_s H_s + B_s (s = 0..S-2, per head) is a chain of
// dense 128 x 128 x 128 products, run on the matrix cores with f32-grade
// accuracy: each f32 operand is split into three bf16 parts, x = x1 + x2 +
// x3 + O(2^-27 |x|), and the product takes the six part products of order
// at most 2^-16 (a1 h1, a1 h2, a2 h1, a1 h3, a2 h2, a3 h1) with f32
// accumulation; the dropped ones are below 2^-24 of |a||h|.
//
// One workgroup of eight waves per (head, 16-column tile of d_v); wave w
// produces row block w (rows 16w..16w+15).  The 128 contraction indices run
// as four k-steps p of 32, k-step p pairing H rows 32p + 4q + e (k-slot
// 8q + e) and 32p + 16 + 4q + e (k-slot 8q + 4 + e) for q = 0..3, e = 0..3:
// the rows that lane 16q + n holds in the result tiles of waves 2p and
// 2p + 1 (row 16 w + 4q + e, column n).  So each wave publishes its new rows
// as one half of k-step p's B fragments, and the A fragment of lane 16q + n
// is A_s[16w + n][32p + 4q + 0..3] and A_s[16w + n][32p + 16 + 4q + 0..3]:
// two float4 loads.  Step s loads A_{s+1} and B_{s+1} while its MFMAs run
// and splits A_{s+1} after them; one barrier per step.  Measured on this
// chain, the loads' latency from L2 and beyond, not the MFMAs, sets the
// step time.
constexpr int kScanLevels = 3;
constexpr int kScanWaves = kD / 16;
constexpr int kScanFrags = 4 * kScanLevels;  // per lane: (k-step, level)

// Three-level bf16 split of two f32 values, packed as bf16 pairs.
__device__ __forceinline__ void split3(float a, float b, uint32_t& w1,
                                       uint32_t& w2, uint32_t& w3) {
  uint32_t r;
  split2(a, b, w1, r);
  const float ra = a - __uint_as_float(w1 << 16) - __uint_as_float(r << 16);
  const float rb = b - __uint_as_float(w1 & 0xffff0000u) - __uint_as_float(r & 0xffff0000u);
  w2 = r;
  const f32x2 x = {ra, rb};
  w3 = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// Per sequence: Hs[0] is S_init (zero when absent), Hs[s + 1] = A_s Hs[s]
// + B_s.  A and B hold S - 1 entries per sequence, Hs S, each entry Hv
// states (sequence-major).  One workgroup per (sequence, head, tile).
__global__ __launch_bounds__(64 * kScanWaves) void seg_scan_kernel(
    const float* __restrict__ A, const float* __restrict__ B,
    const float* __restrict__ S_init, float* __restrict__ Hs, int S, int Hv) {
  __shared__ uint4 Hb[2][4][kScanLevels][64];  // [buffer][k-step][level][lane]
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if (nb % 8 == 0) bid = (bid % 8) * (nb / 8) + bid / 8;  // a head's tiles on one XCD
  const int sh = bid / (kD / kTile), c0 = kTile * (bid % (kD / kTile));
  const int seq = sh / Hv, h = sh % Hv;
  const int w = threadIdx.x / 64, l = threadIdx.x % 64, q = l / 16, n = l % 16;
  const size_t head = (size_t)kD * kD;
  // entry x of this sequence's transitions / offsets and of its states
  auto ab = [&](int x) { return (size_t)((seq * (S - 1) + x) * Hv + h) * head; };
  auto hs = [&](int x) { return (size_t)((seq * S + x) * Hv + h) * head; };
  // element e of this lane's result tile: row 16w + 4q + e, column c0 + n
  auto at = [&](int e) -> size_t {
    return (size_t)(16 * w + 4 * q + e) * kD + c0 + n;
  };
  // this wave's rows as half (w % 2) of the B fragments of k-step w / 2
  auto publish = [&](int buf, const f32x4& t) {
    uint32_t w1[2], w2[2], w3[2];
    split3(t[0], t[1], w1[0], w2[0], w3[0]);
    split3(t[2], t[3], w1[1], w2[1], w3[1]);
    reinterpret_cast<uint2*>(&Hb[buf][w / 2][0][l])[w % 2] = make_uint2(w1[0], w1[1]);
    reinterpret_cast<uint2*>(&Hb[buf][w / 2][1][l])[w % 2] = make_uint2(w2[0], w2[1]);
    reinterpret_cast<uint2*>(&Hb[buf][w / 2][2][l])[w % 2] = make_uint2(w3[0], w3[1]);
  };
  {
    const float* Si = S_init ? S_init + (size_t)sh * head : nullptr;
    float* H0 = Hs + hs(0);
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = Si ? Si[at(e)] : 0.f;
      H0[at(e)] = x[e];
    }
    publish(0, x);
  }
  auto load = [&](int sg, float4 (&ra)[8], float (&rb)[4]) {
    const float* row = A + ab(sg) + (size_t)(16 * w + n) * kD;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      ra[2 * p] = *reinterpret_cast<const float4*>(row + 32 * p + 4 * q);
      ra[2 * p + 1] = *reinterpret_cast<const float4*>(row + 32 * p + 16 + 4 * q);
    }
    const float* Bs = B + ab(sg);
#pragma unroll
    for (int e = 0; e < 4; ++e) rb[e] = Bs[at(e)];
  };
  auto split = [&](const float4 (&ra)[8], uint4 (&fa)[kScanFrags]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float4 x0 = ra[2 * p], x1 = ra[2 * p + 1];
      uint32_t w1[4], w2[4], w3[4];
      split3(x0.x, x0.y, w1[0], w2[0], w3[0]);
      split3(x0.z, x0.w, w1[1], w2[1], w3[1]);
      split3(x1.x, x1.y, w1[2], w2[2], w3[2]);
      split3(x1.z, x1.w, w1[3], w2[3], w3[3]);
      fa[kScanLevels * p + 0] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
      fa[kScanLevels * p + 1] = make_uint4(w2[0], w2[1], w2[2], w2[3]);
      fa[kScanLevels * p + 2] = make_uint4(w3[0], w3[1], w3[2], w3[3]);
    }
  };
  // step sg: A_s split in a, B_s in b; leaves A_{s+1} split in na, B_{s+1}
  // in nbv (the last step reloads its own: no branch around the loads)
  auto step = [&](int sg, const uint4 (&a)[kScanFrags], const float (&b)[4],
                  uint4 (&na)[kScanFrags], float (&nbv)[4]) {
    const int cur = sg & 1;
    float4 ra[8];
    load(min(sg + 1, S - 2), ra, nbv);
    __builtin_amdgcn_sched_barrier(0);  // loads issued before the MFMAs
    // two accumulators (even and odd k-steps), smallest parts first
    f32x4 t = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bf16x8 h1 = as_bf16x8(Hb[cur][p][0][l]);
      const bf16x8 h2 = as_bf16x8(Hb[cur][p][1][l]);
      const bf16x8 h3 = as_bf16x8(Hb[cur][p][2][l]);
      const uint4* f = a + kScanLevels * p;
      const bf16x8 a1 = as_bf16x8(f[0]), a2 = as_bf16x8(f[1]), a3 = as_bf16x8(f[2]);
      f32x4& acc = (p & 1) ? u : t;
      acc = mfma(a3, h1, acc);
      acc = mfma(a2, h2, acc);
      acc = mfma(a1, h3, acc);
      acc = mfma(a2, h1, acc);
      acc = mfma(a1, h2, acc);
      acc = mfma(a1, h1, acc);
    }
    __builtin_amdgcn_sched_barrier(0);
    split(ra, na);
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = (t[e] + u[e]) + b[e];
    float* Hn = Hs + hs(sg + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) Hn[at(e)] = t[e];
    publish(cur ^ 1, t);
    __syncthreads();  // H_{s+1} complete in the other buffer
  };
  uint4 a0[kScanFrags], a1[kScanFrags];
  float b0[4], b1[4];
  if (S > 1) {
    float4 ra[8];
    load(0, ra, b0);
    split(ra, a0);
  }
  __syncthreads();  // H_0 published
  for (int sg = 0; sg + 1 < S; sg += 2) {
    step(sg, a0, b0, a1, b1);
    if (sg + 2 < S) step(sg + 1, a1, b1, a0, b0);
  }
}

// Checkpoints and S_final of a segmented prefill, one workgroup per
// (sequence, job, head).  Job j < n_ck is checkpoint j, the state at token
// (j + 1) * interval: the start state of segment b = (j + 1) * segs_per_ck
// (the scanned state), or the last segment's end state when b = S (the end
// of the sequence).  Job n_ck is S_final, the last segment's end state.
__global__ __launch_bounds__(256) void seg_place_kernel(
    const float* __restrict__ Hs, const float* __restrict__ Send,
    float* __restrict__ ckpt, float* __restrict__ S_final, int n_ck,
    int segs_per_ck, int S, int Hv) {
  const int h = blockIdx.x % Hv, job = (blockIdx.x / Hv) % (n_ck + 1);
  const int seq = blockIdx.x / (Hv * (n_ck + 1));
  const size_t head = (size_t)kD * kD;
  const float* src = Send + ((size_t)(seq * S + S - 1) * Hv + h) * head;
  float* dst = S_final + ((size_t)seq * Hv + h) * head;
  if (job < n_ck) {
    const int b = (job + 1) * segs_per_ck;
    if (b < S) src = Hs + ((size_t)(seq * S + b) * Hv + h) * head;
    dst = ckpt + ((size_t)(seq * n_ck + job) * Hv + h) * head;
  }
  for (int x = threadIdx.x; x < kD * kD; x += 256) dst[x] = src[x];
}

// ------------------------------------------------------------------ host
static int fail(int status, const char* msg) {
  gdn::set_error(msg);
  return status;
}

static int hip_fail(const char* what, hipError_t e) {
  char buf[256];
  snprintf(buf, sizeof(buf), "%s: %s", what, hipGetErrorString(e));
  gdn::set_error(buf);
  return GDN_EHIP;
}

static bool misaligned(const void* p, size_t a) {
  return ((uintptr_t)p % a) != 0;
}

// Chunks of 16 and 32 tokens run in the 64-row tiles of both kernels with
// the rows past the chunk inert, exactly as the tail chunk of a sequence:
// their loads repeat the last valid row, P1 gives them beta = 0 and gate 0,
// so their X, V_new and D rows are exact zeros and T is the identity on
// them (L has zero rows there); they add nothing to the state and their
// output rows are never stored.
static size_t p1_bytes(int32_t n_seqs, int32_t L, int32_t Hv, int32_t C) {
  const size_t n_chunks = ((size_t)L + C - 1) / C;
  return (size_t)n_seqs * n_chunks * Hv * WsLayout::kBytes;
}

// Sizes for which a prefill may run in segments (few sequence-heads, more
// than one segment); whether it does also depends on the checkpoint
// interval and the flags (use_segments).
static bool segment_sizes(int32_t n_seqs, int32_t L, int32_t Hv) {
  return (int64_t)n_seqs * Hv <= kSegMaxHeads && L > kSeg;
}

static bool use_segments(int32_t n_seqs, int32_t L, int32_t Hv,
                         const float* checkpoints, int32_t ckpt_interval,
                         int flags) {
  return segment_sizes(n_seqs, L, Hv) && !(flags & GDN_FLAG_PREFILL_ONE_CHAIN) &&
         (!checkpoints || ckpt_interval % kSeg == 0);
}

// Segment buffers after the P1 workspace, each sequence-major with Hv
// states per entry: A_s and B_s of every segment but the last of each
// sequence, the scanned start state and the end state of every segment.
struct SegLayout {
  int S;  // segments per sequence
  size_t a, b, hs, send, end;
  SegLayout(int32_t n_seqs, int32_t L, int32_t Hv, size_t p1) {
    const size_t st = (size_t)n_seqs * Hv * kD * kD * sizeof(float);
    S = (L + kSeg - 1) / kSeg;
    a = (p1 + 255) & ~size_t(255);
    b = a + (size_t)(S - 1) * st;
    hs = b + (size_t)(S - 1) * st;
    send = hs + (size_t)S * st;
    end = send + (size_t)S * st;
  }
};

static size_t ws_bytes(int32_t n_seqs, int32_t L, int32_t Hv, int32_t C) {
  const size_t p1 = p1_bytes(n_seqs, L, Hv, C);
  return segment_sizes(n_seqs, L, Hv) ? SegLayout(n_seqs, L, Hv, p1).end : p1;
}

static int check_sizes(int32_t n_seqs, int32_t L, int32_t Hv, int32_t Hk,
                       int32_t dk, int32_t dv, int32_t C) {
  if (n_seqs < 1 || L < 1 || Hv < 1 || Hk < 1 || Hv % Hk != 0 || C < 1) {
    return fail(GDN_EINVAL, "prefill: sizes out of range");
  }
  if (C != 16 && C != 32 && C != kC) {
    return fail(GDN_EUNSUPPORTED, "prefill: chunk must be 16, 32 or 64");
  }
  if (dk != kD || dv != kD) {
    return fail(GDN_EUNSUPPORTED, "prefill: d_k = d_v = 128 only");
  }
  if ((double)L * Hv * kD >= 2147483648.0 || (double)L * Hk * kD >= 2147483648.0)
    return fail(GDN_EUNSUPPORTED, "prefill: seq_len x heads x 128 must stay below 2^31");
  const double blocks = (double)n_seqs * ((L + C - 1) / C) * Hv;
  const double elems = (double)n_seqs * L * Hv * kD;
  if (blocks > (double)INT_MAX || elems > 4.0e15) {
    return fail(GDN_EINVAL, "prefill: sizes overflow");
  }
  return GDN_OK;
}

}  // namespace gdnp

using namespace gdnp;

extern "C" size_t gdn_prefill_workspace_bytes(int32_t n_seqs, int32_t seq_len,
                                              int32_t h_v, int32_t h_k,
                                              int32_t d_k, int32_t d_v,
                                              int32_t chunk) {
  if (check_sizes(n_seqs, seq_len, h_v, h_k, d_k, d_v, chunk) != GDN_OK) return 0;
  return ws_bytes(n_seqs, seq_len, h_v, chunk);
}

// Workspace of the entry point that allocates nothing: a fixed device
// array, one copy per GPU, held until the process ends.  Host code never
// names it directly (on the host the name is only a stand-in); it takes the
// per-device address that hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = (size_t)GDN_PREFILL_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace gdnp {

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, looked up once per
// device with that device current.
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("prefill scratch: hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) {
    return fail(GDN_EUNSUPPORTED, "prefill scratch: device index out of range");
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      return hip_fail("prefill scratch: hipGetSymbolAddress",
                      e != hipSuccess ? e : hipErrorInvalidSymbol);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

// Every argument check except those of the workspace pointer; no HIP call.
static int check_args(int32_t n_seqs, int32_t seq_len, int32_t h_v,
                      int32_t h_k, int32_t d_k, int32_t d_v, int32_t chunk,
                      int32_t ckpt_interval, const void* q, const void* k,
                      const void* v, int in_dtype, const float* beta,
                      const float* g, const float* S_init, float* S_final,
                      float* o, float* checkpoints, size_t ws_size,
                      int flags) {
  int rc = check_sizes(n_seqs, seq_len, h_v, h_k, d_k, d_v, chunk);
  if (rc != GDN_OK) return rc;
  if (!q || !k || !v || !beta || !g || !S_final || !o) {
    return fail(GDN_EINVAL, "prefill: required pointer is NULL");
  }
  if (in_dtype != GDN_BF16) {
    return fail(in_dtype == GDN_F32 ? GDN_EUNSUPPORTED : GDN_EINVAL, "prefill: bf16 inputs only");
  }
  if (flags & ~(GDN_FLAG_L2NORM_QK | GDN_FLAG_PREFILL_ONE_CHAIN)) {
    return fail(GDN_EINVAL, "prefill: unknown flag bits");
  }
  if (checkpoints && (ckpt_interval < chunk || ckpt_interval % chunk != 0)) {
    return fail(GDN_EINVAL, "prefill: ckpt_interval must be a positive multiple of the chunk");
  }
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 2) ||
      misaligned(beta, 4) || misaligned(g, 4) || misaligned(S_final, 4) ||
      misaligned(o, 4) || (S_init && misaligned(S_init, 4)) ||
      (checkpoints && misaligned(checkpoints, 4))) {
    return fail(GDN_EINVAL, "prefill: misaligned pointer");
  }
  if (ws_size < ws_bytes(n_seqs, seq_len, h_v, chunk)) {
    return fail(GDN_EWORKSPACE, "prefill: workspace too small");
  }
  return GDN_OK;
}

static int launch_p2(int mode, const PDims& dd, int n_seqs, const u16* qq,
                     const u16* kk, const u16* vv, const uint8_t* ws,
                     const float* S_init, float* S_final, float* o,
                     float* checkpoints, hipStream_t st) {
  PDims d = dd;
  d.n_seqs = n_seqs;
  void* args[] = {(void*)&qq, (void*)&kk, (void*)&vv, (void*)&ws,
                  (void*)&S_init, (void*)&S_final, (void*)&o,
                  (void*)&checkpoints, (void*)&d};
  const void* fn = mode == kModePair ? (const void*)p2_kernel<kModePair>
                                     : (const void*)p2_kernel<0>;
  hipError_t e = hipLaunchKernel(fn,
                                 dim3(n_seqs * d.Hv * (kD / kTile)),
                                 dim3(kP2Threads), args, 0, st);
  return e == hipSuccess ? GDN_OK : hip_fail("prefill p2 launch", e);
}

// Launches P1 and P2, or the segmented passes (arguments already checked).
static int prefill_launch(
    int32_t n_seqs, int32_t seq_len, int32_t h_v, int32_t h_k, int32_t chunk,
    int32_t ckpt_interval, const void* q, const void* k, const void* v,
    const float* beta, const float* g, const float* S_init, float* S_final,
    float* o, float* checkpoints, void* workspace, float scale, int flags,
    void* stream) {
  PDims dd;
  dd.n_seqs = n_seqs;
  dd.L = seq_len;
  dd.Hv = h_v;
  dd.Hk = h_k;
  dd.group = h_v / h_k;
  dd.chunk = chunk;
  dd.n_chunks = (seq_len + chunk - 1) / chunk;
  dd.segs = 1;
  dd.seq_L = seq_len;
  dd.seq_chunks = dd.n_chunks;
  dd.L_last = seq_len;
  dd.ckpt_interval = checkpoints ? ckpt_interval : 0;
  dd.scale = scale;
  dd.l2norm = (flags & GDN_FLAG_L2NORM_QK) ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;

  const u16* qq = (const u16*)q;
  const u16* kk = (const u16*)k;
  const u16* vv = (const u16*)v;
  uint8_t* wsb = (uint8_t*)workspace;
  {
    void* args[] = {(void*)&qq, (void*)&kk, (void*)&beta, (void*)&g,
                    (void*)&wsb, (void*)&dd};
    hipError_t e = hipLaunchKernel((const void*)p1_kernel,
                                   dim3(n_seqs * dd.n_chunks * h_v),
                                   dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return hip_fail("prefill p1 launch", e);
  }
  if (!use_segments(n_seqs, seq_len, h_v, checkpoints, ckpt_interval, flags)) {
    return launch_p2(0, dd, n_seqs, qq, kk, vv, wsb, S_init, S_final, o,
                     checkpoints, st);
  }
  // Segments: P2 runs the segments of every sequence as parts of kSeg
  // tokens (the last one of each sequence may be shorter); the P1
  // workspace is indexed by (sequence, chunk), which part_pos follows.
  const SegLayout sl(n_seqs, seq_len, h_v, p1_bytes(n_seqs, seq_len, h_v, chunk));
  const int S = sl.S, tail = seq_len - (S - 1) * kSeg;
  float* A = reinterpret_cast<float*>(wsb + sl.a);
  float* B = reinterpret_cast<float*>(wsb + sl.b);
  float* Hs = reinterpret_cast<float*>(wsb + sl.hs);
  float* Send = reinterpret_cast<float*>(wsb + sl.send);
  PDims ds = dd;
  ds.L = kSeg;
  ds.n_chunks = kSeg / chunk;
  ds.segs = S - 1;
  ds.L_last = kSeg;
  ds.ckpt_interval = 0;
  // A_s to S_final's place, B_s to o's (see p2_kernel)
  int rc = launch_p2(kModePair, ds, n_seqs * (S - 1), qq, kk, vv, wsb, nullptr,
                     A, B, nullptr, st);
  if (rc != GDN_OK) return rc;
  {
    void* args[] = {(void*)&A, (void*)&B, (void*)&S_init, (void*)&Hs,
                    (void*)&S, (void*)&h_v};
    hipError_t e = hipLaunchKernel((const void*)seg_scan_kernel,
                                   dim3(n_seqs * h_v * (kD / kTile)),
                                   dim3(64 * kScanWaves), args, 0, st);
    if (e != hipSuccess) return hip_fail("prefill segment scan launch", e);
  }
  // the outputs of every segment, the last one of each sequence with its
  // own length
  ds.segs = S;
  ds.L_last = tail;
  rc = launch_p2(0, ds, n_seqs * S, qq, kk, vv, wsb, Hs, Send, o, nullptr, st);
  if (rc != GDN_OK) return rc;
  {
    int n_ck = checkpoints ? seq_len / ckpt_interval : 0;
    int per = checkpoints ? ckpt_interval / kSeg : 1;
    float* ck = checkpoints;
    void* args[] = {(void*)&Hs, (void*)&Send, (void*)&ck, (void*)&S_final,
                    (void*)&n_ck, (void*)&per, (void*)&S, (void*)&h_v};
    hipError_t e = hipLaunchKernel((const void*)seg_place_kernel,
                                   dim3(n_seqs * (n_ck + 1) * h_v), dim3(256),
                                   args, 0, st);
    if (e != hipSuccess) return hip_fail("prefill segment placement launch", e);
  }
  return GDN_OK;
}

}  // namespace gdnp

extern "C" int gdn_prefill_chunked(
    int32_t n_seqs, int32_t seq_len, int32_t h_v, int32_t h_k, int32_t d_k,
    int32_t d_v, int32_t chunk, int32_t ckpt_interval, const void* q,
    const void* k, const void* v, int in_dtype, const float* beta,
    const float* g, const float* S_init, float* S_final, float* o,
    float* checkpoints, void* workspace, size_t ws_size, float scale,
    int flags, void* stream) {
  int rc = check_args(n_seqs, seq_len, h_v, h_k, d_k, d_v, chunk,
                      ckpt_interval, q, k, v, in_dtype, beta, g, S_init,
                      S_final, o, checkpoints, ws_size, flags);
  if (rc != GDN_OK) return rc;
  if (!workspace) return fail(GDN_EINVAL, "prefill: required pointer is NULL");
  if (misaligned(workspace, 256)) {
    return fail(GDN_EINVAL, "prefill: misaligned pointer");
  }
  return prefill_launch(n_seqs, seq_len, h_v, h_k, chunk, ckpt_interval, q, k,
                        v, beta, g, S_init, S_final, o, checkpoints, workspace,
                        scale, flags, stream);
}

extern "C" int gdn_prefill_chunked_noalloc(
    int32_t n_seqs, int32_t seq_len, int32_t h_v, int32_t h_k, int32_t d_k,
    int32_t d_v, int32_t chunk, int32_t ckpt_interval, const void* q,
    const void* k, const void* v, int in_dtype, const float* beta,
    const float* g, const float* S_init, float* S_final, float* o,
    float* checkpoints, float scale, int flags, void* stream) {
  int rc = check_sizes(n_seqs, seq_len, h_v, h_k, d_k, d_v, chunk);
  if (rc != GDN_OK) return rc;
  if (ws_bytes(n_seqs, seq_len, h_v, chunk) > kScratchBytes) {
    return fail(GDN_EWORKSPACE,
                "prefill (no-alloc): the workspace for these sizes exceeds the "
                "library's fixed scratch array (GDN_PREFILL_SCRATCH_BYTES)");
  }
  rc = check_args(n_seqs, seq_len, h_v, h_k, d_k, d_v, chunk, ckpt_interval, q,
                  k, v, in_dtype, beta, g, S_init, S_final, o, checkpoints,
                  kScratchBytes, flags);
  if (rc != GDN_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != GDN_OK) return rc;
  return prefill_launch(n_seqs, seq_len, h_v, h_k, chunk, ckpt_interval, q, k,
                        v, beta, g, S_init, S_final, o, checkpoints, ws, scale,
                        flags, stream);
}
