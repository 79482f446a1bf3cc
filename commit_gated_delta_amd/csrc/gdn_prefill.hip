// gdn_prefill.hip -- chunked prefill of the gated delta rule on gfx950 MFMA.
//
// Block (WY/UT) form of the rule over chunks of C = 64 tokens: Yang et al.,
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
// expressions; only the evaluation order differs.
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
//       sequential over the chunks; the d_k x 16 state tile stays in f32 MFMA
//       accumulators (wave w holds rows 32w..32w+31).  Products with an f32
//       operand use split bf16: two passes against an exact bf16 operand
//       (K H, Q H, K^T V'), three passes f32 x f32 (T X, P V_new); about
//       2^-17 relative error per product.  The state is never rounded below
//       f32, so a run resumed from a checkpoint is bitwise the straight run.
//       The output O of each chunk is produced here too (no separate pass).
//   Checkpoints: the state after every token count that is a positive
//   multiple of the interval (context_cache.checkpoint_interval, NInfer
//   technical review, blog.123qwe.co.kr post 4624, section "Architecture 2").
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Lane l of a wave holds
//   A[l%16][8*(l/16) + e], B[8*(l/16) + e][l%16]   (e = 0..7, bf16)
//   D[4*(l/16) + e][l%16]                          (e = 0..3, f32).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdnp {

constexpr int kC = 64;     // chunk length
constexpr int kD = 128;    // d_k = d_v
constexpr int kTile = 16;  // value columns per p2 workgroup
constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

struct PDims {
  int n_seqs, L, Hv, Hk, group, n_chunks;
  int ckpt_interval;  // 0: no checkpoints
  float scale;
  int l2norm;
};

// Workspace per (sequence, chunk, value head).  T and P are stored as MFMA
// A-operand fragments in the order p2 reads them: for wave w, piece x (T hi,
// T lo for k-step 0, the same for k-step 1, then P likewise) and lane l, 16
// bytes holding row 16w + l%16, columns 32*ks + 8*(l/16) + 0..7, at
// ((w*8 + x)*64 + l)*16 -- one load instruction of a wave reads 1 KiB of
// consecutive bytes.
struct WsLayout {
  static constexpr size_t kFrag = 4 * 64 * 8 * 16;               // 32 KiB
  static constexpr size_t kVec = kFrag;      // float [64][4]: sb sk so sd
  static constexpr size_t kGc = kVec + kC * 4 * sizeof(float);   // float
  static constexpr size_t kBytes = (kGc + sizeof(float) + 255) & ~size_t(255);
};

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
__global__ __launch_bounds__(kThreads) void p1_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k,
    const float* __restrict__ beta, const float* __restrict__ g,
    uint8_t* __restrict__ ws, PDims d) {
  constexpr int KS = kD + 8;  // padded LDS row (bf16) against bank conflicts
  constexpr int FS = kC + 1;  // padded f32 row
  __shared__ __attribute__((aligned(16))) u16 Ks[kC * KS];
  __shared__ __attribute__((aligned(16))) u16 Qs[kC * KS];  // later: P (f32)
  __shared__ float Ls[kC * FS];                             // L (f32)
  __shared__ float rk_s[kC], rq_s[kC], G_s[kC], b_s[kC];
  float* Ts = reinterpret_cast<float*>(Ks);  // T (f32) once K is consumed
  float* Ps = reinterpret_cast<float*>(Qs);
  static_assert(sizeof(float) * kC * FS <= sizeof(u16) * kC * KS, "alias");

  const int bid = blockIdx.x;
  const int h = bid % d.Hv;
  const int c = (bid / d.Hv) % d.n_chunks;
  const int s = bid / (d.Hv * d.n_chunks);
  const int kh = h / d.group;
  const int t0 = c * kC;
  const int nv = min(kC, d.L - t0);  // valid rows of this chunk
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int l = tid % 64;

  // ---- load K, Q rows (bf16) to LDS.  Rows past the end of the sequence
  // are read from the last valid row (no branch around the loads): they only
  // meet beta = 0, or feed output rows that are not stored.
  const int last = nv - 1;
  for (int it = 0; it < 4; ++it) {
    const int idx = it * kThreads + tid;  // 1024 pieces of 8 bf16
    const int row = idx / 16, col = (idx % 16) * 8;
    const size_t off =
        (((size_t)s * d.L + t0 + min(row, last)) * d.Hk + kh) * kD + col;
    *reinterpret_cast<uint4*>(&Ks[row * KS + col]) =
        *reinterpret_cast<const uint4*>(k + off);
    *reinterpret_cast<uint4*>(&Qs[row * KS + col]) =
        *reinterpret_cast<const uint4*>(q + off);
  }
  if (tid < kC) {
    const size_t gi = ((size_t)s * d.L + t0 + min(tid, last)) * d.Hv + h;
    const float bb = (tid < nv) ? beta[gi] : 0.f;
    const float gg = (tid < nv) ? g[gi] : 0.f;
    b_s[tid] = bb;
    // inclusive prefix sum of g over the chunk (wave 0), fixed order
    float x = gg;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (tid >= off) x += y;
    }
    G_s[tid] = x;
  }
  __syncthreads();

  // ---- norms: four threads per row, 32 entries each
  {
    const int row = tid / 4, part = tid % 4;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float kv = bf16_f(Ks[row * KS + part * 32 + e]);
      const float qv = bf16_f(Qs[row * KS + part * 32 + e]);
      sk = __builtin_fmaf(kv, kv, sk);
      sq = __builtin_fmaf(qv, qv, sq);
    }
    sk += dpp<0xB1>(sk);  // quad_perm [1,0,3,2]
    sk += dpp<0x4E>(sk);  // quad_perm [2,3,0,1]
    sq += dpp<0xB1>(sq);
    sq += dpp<0x4E>(sq);
    if (part == 0) {
      rk_s[row] = d.l2norm ? __builtin_amdgcn_rsqf(sk + 1e-6f) : 1.0f;
      rq_s[row] = d.l2norm ? __builtin_amdgcn_rsqf(sq + 1e-6f) : 1.0f;
    }
  }

  // ---- A = K K^T and B = Q K^T: wave w owns rows 16w..16w+15
  f32x4 accA[4], accB[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    accA[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accB[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  {
    const int arow = 16 * w + l % 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = 32 * ks + 8 * (l / 16);
      const bf16x8 ak = as_bf16x8(*reinterpret_cast<const uint4*>(&Ks[arow * KS + kk]));
      const bf16x8 aq = as_bf16x8(*reinterpret_cast<const uint4*>(&Qs[arow * KS + kk]));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int brow = 16 * nt + l % 16;  // B[kk][j] = K[j][kk]
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(&Ks[brow * KS + kk]));
        accA[nt] = mfma(ak, b, accA[nt]);
        accB[nt] = mfma(aq, b, accB[nt]);
      }
    }
  }
  __syncthreads();  // every wave is done with Ks / Qs; norms and G are in LDS

  // ---- L (strict lower) and P (lower with diagonal) in f32
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int j = 16 * nt + l % 16;
    const float rkj = rk_s[j], Gj = G_s[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * (l / 16) + e;
      const float dec = __expf(G_s[i] - Gj);
      const float lv = (j < i) ? b_s[i] * rk_s[i] * rkj * accA[nt][e] * dec : 0.f;
      const float pv =
          (j <= i) ? d.scale * rq_s[i] * rkj * accB[nt][e] * dec : 0.f;
      Ls[i * FS + j] = lv;
      Ps[i * FS + j] = pv;
    }
  }
  __syncthreads();

  // ---- T = (I + L)^-1, step 1: the four 16x16 diagonal blocks.
  // Wave b, lane jj < 16: column jj of block b by forward substitution.
  if (l < 16) {
    const int b0 = 16 * w, jj = l;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int x = 0; x < r; ++x)
        acc = __builtin_fmaf(Ls[(b0 + r) * FS + b0 + x], t[x], acc);
      t[r] = (r == jj) ? 1.f : ((r < jj) ? 0.f : -acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ts[(b0 + r) * FS + b0 + jj] = t[r];
  }
  // zero the strictly upper blocks
  for (int idx = tid; idx < kC * kC; idx += kThreads) {
    const int i = idx / kC, j = idx % kC;
    if (j / 16 > i / 16) Ts[i * FS + j] = 0.f;
  }
  __syncthreads();

  // ---- step 2: block rows 1..3.  T_ib = -T_ii sum_{m=b}^{i-1} L_im T_mb;
  // wave b computes block (i, b); lane: column cc = l%16, rows 4*(l/16)+e.
  __shared__ float Ys[4][16 * 17];
  for (int bi = 1; bi < 4; ++bi) {
    if (w < bi) {
      const int bb = w, cc = l % 16, r0 = 4 * (l / 16);
      float y[4] = {0.f, 0.f, 0.f, 0.f};
      for (int m = bb; m < bi; ++m) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float tv = Ts[(16 * m + x) * FS + 16 * bb + cc];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            y[e] = __builtin_fmaf(Ls[(16 * bi + r0 + e) * FS + 16 * m + x], tv, y[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Ys[bb][(r0 + e) * 17 + cc] = y[e];
      // the wave's own Ys block is read back by the same wave only
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      float tvals[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float yv = Ys[bb][x * 17 + cc];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tvals[e] = __builtin_fmaf(Ts[(16 * bi + r0 + e) * FS + 16 * bi + x], yv, tvals[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Ts[(16 * bi + r0 + e) * FS + 16 * bb + cc] = -tvals[e];
    }
    __syncthreads();
  }

  // ---- write T, P (split bf16, fragment order) and the row vectors
  uint8_t* wsb = ws + ((size_t)bid) * WsLayout::kBytes;
  {
    const int i = 16 * w + l % 16;
    uint4* dst = reinterpret_cast<uint4*>(wsb) + (size_t)w * 8 * 64 + l;
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
      const float* M = mat ? Ps : Ts;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int j0 = 32 * ks + 8 * (l / 16);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          split2(M[i * FS + j0 + 2 * e], M[i * FS + j0 + 2 * e + 1], hi[e], lo[e]);
        dst[(mat * 4 + ks * 2 + 0) * 64] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        dst[(mat * 4 + ks * 2 + 1) * 64] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
    }
  }
  if (tid < kC) {
    const int i = tid;
    const float Gc = G_s[kC - 1];
    const float gam = __expf(G_s[i]);
    float4 v;
    v.x = b_s[i];                                // sb: beta
    v.y = b_s[i] * gam * rk_s[i];                // sk: beta gamma rk
    v.z = gam * rq_s[i] * d.scale;               // so: gamma rq scale
    v.w = rk_s[i] * __expf(Gc - G_s[i]);         // sd: rk exp(G_63 - G_i)
    reinterpret_cast<float4*>(wsb + WsLayout::kVec)[i] = v;
    if (i == 0) *reinterpret_cast<float*>(wsb + WsLayout::kGc) = __expf(Gc);
  }
}

// ------------------------------------------------------------------ p2
// Per-chunk operands that a lane prefetches one chunk ahead.
struct Pre {
  uint4 q[4];     // A fragments of the lane's Q row (4 k-steps)
  uint4 tp[8];    // A fragments of T and P (WsLayout order)
  uint32_t v[4];  // bf16 V[row 16w + 4*(l/16) + e][column], in the low half
  float4 vec[4];  // sb sk so sd of those rows
  float gc;
};

__device__ __forceinline__ uint2 pack4(const uint32_t (&x)[4], int e0) {
  return make_uint2(x[e0], x[e0 + 1]);
}

__global__ __launch_bounds__(kThreads) void p2_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k,
    const u16* __restrict__ v, const uint8_t* __restrict__ ws,
    const float* __restrict__ S_init, float* __restrict__ S_final,
    float* __restrict__ o, float* __restrict__ ckpt, PDims d) {
  constexpr int KS = kD + 8;   // Kr row stride (bf16)
  constexpr int TS = kC + 8;   // Kt / column-major tile row stride (bf16)
  constexpr int HS = kD + 8;   // Hb row stride (bf16)
  // double buffers (chunk parity) for the K copies and the state operand
  __shared__ __attribute__((aligned(16))) u16 Kr[2][kC * KS];      // K rows
  __shared__ __attribute__((aligned(16))) u16 Kt[2][kD * TS];      // K^T
  __shared__ __attribute__((aligned(16))) u16 Hb[2][2][kTile * HS];// H hi/lo [n][dk]
  __shared__ __attribute__((aligned(16))) u16 Xb[2][kTile * TS];   // X hi/lo [n][j]
  __shared__ __attribute__((aligned(16))) u16 Vb[2][kTile * TS];   // V_new hi/lo
  __shared__ __attribute__((aligned(16))) u16 Db[2][kTile * TS];   // sd V_new hi/lo
  // Kt holds K^T with the 8-entry groups of each row XOR-swizzled by
  // (dk / 8) % 8, so that the transposing stores of one wave spread over the
  // LDS banks while every 8-entry group stays 16-byte aligned for the reads.
  auto kt_at = [&](int dk, int j) {
    return dk * TS + 8 * ((j >> 3) ^ ((dk >> 3) & 7)) + (j & 7);
  };

  // block -> (sequence, head, tile); the tiles of a head share one XCD
  const int nb = gridDim.x;
  int b = blockIdx.x;
  if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
  const int tile = b % (kD / kTile);
  const int h = (b / (kD / kTile)) % d.Hv;
  const int s = b / ((kD / kTile) * d.Hv);
  const int kh = h / d.group;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int l = tid % 64;
  const int n = l % 16;       // column inside the tile (C/D/B layouts)
  const int q4 = l / 16;      // 0..3
  const int col = kTile * tile + n;
  const int nch = d.n_chunks;

  // per-sequence bases; element offsets below fit in 32 bits (host check)
  const u16* __restrict__ qs = q + (size_t)s * d.L * d.Hk * kD;
  const u16* __restrict__ kseq = k + (size_t)s * d.L * d.Hk * kD;
  const u16* __restrict__ vs = v + (size_t)s * d.L * d.Hv * kD;
  float* __restrict__ os = o + (size_t)s * d.L * d.Hv * kD;
  const uint8_t* __restrict__ wss =
      ws + ((size_t)s * nch * d.Hv + h) * WsLayout::kBytes;
  const size_t ws_chunk = (size_t)d.Hv * WsLayout::kBytes;

  // state fragments: wave w holds dk rows 32w + 16*mt + 4*q4 + e, column n
  f32x4 H[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 32 * w + 16 * mt + 4 * q4 + e;
      H[mt][e] = S_init ? S_init[(((size_t)s * d.Hv + h) * kD + r) * kD + col] : 0.f;
    }

  auto write_H = [&](int buf) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      uint32_t hi[2], lo[2];
      split2(H[mt][0], H[mt][1], hi[0], lo[0]);
      split2(H[mt][2], H[mt][3], hi[1], lo[1]);
      const int r = 32 * w + 16 * mt + 4 * q4;
      *reinterpret_cast<uint2*>(&Hb[buf][0][n * HS + r]) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2*>(&Hb[buf][1][n * HS + r]) = make_uint2(lo[0], lo[1]);
    }
  };

  // Loads are unconditional: rows past the end of the sequence are read from
  // the last valid row instead.  Their values never reach a result: P1 gives
  // such rows beta = 0, so X, V_new and their state contributions are 0, and
  // their output rows are not stored.  (A load under a branch would make the
  // compiler wait for it at the end of the branch, which defeats the
  // one-chunk-ahead prefetch.)
  auto prefetch = [&](int c, Pre& p) {
    const int t0 = c * kC;
    const int last = min(kC, d.L - t0) - 1;
    const uint4* wf = reinterpret_cast<const uint4*>(wss + (size_t)c * ws_chunk) +
                      w * 8 * 64 + l;
    const uint32_t qoff =
        ((uint32_t)(t0 + min(16 * w + n, last)) * d.Hk + kh) * kD + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      p.q[ks] = *reinterpret_cast<const uint4*>(qs + qoff + 32 * ks);
#pragma unroll
    for (int x = 0; x < 8; ++x) p.tp[x] = wf[x * 64];
    const float4* vec = reinterpret_cast<const float4*>(
        wss + (size_t)c * ws_chunk + WsLayout::kVec);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * w + 4 * q4 + e;
      p.v[e] = vs[((uint32_t)(t0 + min(r, last)) * d.Hv + h) * kD + col];
      p.vec[e] = vec[r];
    }
    p.gc = *reinterpret_cast<const float*>(wss + (size_t)c * ws_chunk + WsLayout::kGc);
  };

  // raw K pieces of one chunk, for the row-major and transposed LDS copies
  uint4 kr[4];
  auto load_K = [&](int c) {
    const int t0 = c * kC;
    const int last = min(kC, d.L - t0) - 1;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * kThreads + tid;
      const int row = idx / 16, cc = (idx % 16) * 8;
      kr[it] = *reinterpret_cast<const uint4*>(
          kseq + ((uint32_t)(t0 + min(row, last)) * d.Hk + kh) * kD + cc);
    }
  };

  auto stage_K = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * kThreads + tid;
      const int row = idx / 16, cc = (idx % 16) * 8;
      *reinterpret_cast<uint4*>(&Kr[buf][row * KS + cc]) = kr[it];
      const u16* e8 = reinterpret_cast<const u16*>(&kr[it]);
#pragma unroll
      for (int e = 0; e < 8; ++e) Kt[buf][kt_at(cc + e, row)] = e8[e];
    }
  };

  // Every global load is issued about one chunk before its data is used: at
  // the top of chunk c one explicit wait covers the operands of chunk c
  // (issued during chunk c-1) and the K rows of chunk c+1 (issued at the top
  // of chunk c-1); nothing later in the chunk reads a register that is still
  // being loaded.
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

  // one chunk: uses `cur`, prefetches chunk c+1 into `nxt`
  auto chunk = [&](int c, const Pre& cur, Pre& nxt) {
    const int buf = c & 1;
    const int t0 = c * kC;
    const int nv = min(kC, d.L - t0);
    wait_loads();
    // K of chunk c+1 into the other buffers (last read in chunk c-1, before
    // the barrier that ended it); visible to chunk c+1 after this chunk's
    // barriers
    if (c + 1 < nch) stage_K(buf ^ 1);
    if (c + 2 < nch) load_K(c + 2);

    // ---- K H and Q H for rows 16w..16w+15 (2 passes: H hi, H lo)
    f32x4 KH = {0.f, 0.f, 0.f, 0.f}, QH = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = 32 * ks + 8 * q4;
      const bf16x8 ak = as_bf16x8(*reinterpret_cast<const uint4*>(&Kr[buf][(16 * w + n) * KS + kk]));
      const bf16x8 aq = as_bf16x8(cur.q[ks]);
      const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(&Hb[buf][0][n * HS + kk]));
      const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(&Hb[buf][1][n * HS + kk]));
      KH = mfma(ak, bh, KH);
      QH = mfma(aq, bh, QH);
      KH = mfma(ak, bl, KH);
      QH = mfma(aq, bl, QH);
    }
    // operands of chunk c+1 (issued while the MFMAs above run)
    if (c + 1 < nch) prefetch(c + 1, nxt);

    // ---- X = sb V - sk (K H), to LDS as split bf16 (column-major)
    {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = cur.vec[e].x * __uint_as_float(cur.v[e] << 16) - cur.vec[e].y * KH[e];
      uint32_t hi[2], lo[2];
      split2(x[0], x[1], hi[0], lo[0]);
      split2(x[2], x[3], hi[1], lo[1]);
      const int r = 16 * w + 4 * q4;
      *reinterpret_cast<uint2*>(&Xb[0][n * TS + r]) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2*>(&Xb[1][n * TS + r]) = make_uint2(lo[0], lo[1]);
    }
    __syncthreads();

    // ---- V_new = T X (3 passes); T is lower triangular: k-step 1 (rows
    // 32..63 of X) only matters for waves 2 and 3
    f32x4 VN = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks == 1 && w < 2) break;
      const int kk = 32 * ks + 8 * q4;
      const bf16x8 xh = as_bf16x8(*reinterpret_cast<const uint4*>(&Xb[0][n * TS + kk]));
      const bf16x8 xl = as_bf16x8(*reinterpret_cast<const uint4*>(&Xb[1][n * TS + kk]));
      const bf16x8 th = as_bf16x8(cur.tp[2 * ks]), tl = as_bf16x8(cur.tp[2 * ks + 1]);
      VN = mfma(th, xh, VN);
      VN = mfma(th, xl, VN);
      VN = mfma(tl, xh, VN);
    }
    {
      uint32_t hi[2], lo[2], dh[2], dl[2];
      split2(VN[0], VN[1], hi[0], lo[0]);
      split2(VN[2], VN[3], hi[1], lo[1]);
      split2(cur.vec[0].w * VN[0], cur.vec[1].w * VN[1], dh[0], dl[0]);
      split2(cur.vec[2].w * VN[2], cur.vec[3].w * VN[3], dh[1], dl[1]);
      const int r = 16 * w + 4 * q4;
      *reinterpret_cast<uint2*>(&Vb[0][n * TS + r]) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2*>(&Vb[1][n * TS + r]) = make_uint2(lo[0], lo[1]);
      *reinterpret_cast<uint2*>(&Db[0][n * TS + r]) = make_uint2(dh[0], dh[1]);
      *reinterpret_cast<uint2*>(&Db[1][n * TS + r]) = make_uint2(dl[0], dl[1]);
    }
    __syncthreads();

    // ---- O = so (Q H) + P V_new (3 passes), rows 16w..16w+15
    {
      f32x4 O;
#pragma unroll
      for (int e = 0; e < 4; ++e) O[e] = cur.vec[e].z * QH[e];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1 && w < 2) break;
        const int kk = 32 * ks + 8 * q4;
        const bf16x8 vh = as_bf16x8(*reinterpret_cast<const uint4*>(&Vb[0][n * TS + kk]));
        const bf16x8 vl = as_bf16x8(*reinterpret_cast<const uint4*>(&Vb[1][n * TS + kk]));
        const bf16x8 ph = as_bf16x8(cur.tp[4 + 2 * ks]), pl = as_bf16x8(cur.tp[5 + 2 * ks]);
        O = mfma(ph, vh, O);
        O = mfma(ph, vl, O);
        O = mfma(pl, vh, O);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + 4 * q4 + e;
        if (r < nv) os[((uint32_t)(t0 + r) * d.Hv + h) * kD + col] = O[e];
      }
    }

    // ---- H' = gamma_63 H + K^T (sd V_new)  (2 passes), rows 32w..32w+31
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = cur.gc * H[mt][e];
      const int arow = 32 * w + 16 * mt + n;  // dk index
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kk = 32 * ks + 8 * q4;
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&Kt[buf][kt_at(arow, kk)]));
        const bf16x8 dh = as_bf16x8(*reinterpret_cast<const uint4*>(&Db[0][n * TS + kk]));
        const bf16x8 dl = as_bf16x8(*reinterpret_cast<const uint4*>(&Db[1][n * TS + kk]));
        acc = mfma(a, dh, acc);
        acc = mfma(a, dl, acc);
      }
      H[mt] = acc;
    }

    // ---- checkpoint after token t0 + nv when it is a multiple of the interval
    if (d.ckpt_interval > 0 && ckpt && (t0 + nv) % d.ckpt_interval == 0) {
      const int idx = (t0 + nv) / d.ckpt_interval - 1;
      const int n_ck = d.L / d.ckpt_interval;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 32 * w + 16 * mt + 4 * q4 + e;
          ckpt[((((size_t)s * n_ck + idx) * d.Hv + h) * kD + r) * kD + col] = H[mt][e];
        }
    }

    // the state operand of chunk c+1 goes to the other buffer (last read in
    // chunk c-1)
    if (c + 1 < nch) write_H(buf ^ 1);
    __syncthreads();
  };

  Pre A, B;
  load_K(0);
  wait_loads();
  stage_K(0);
  prefetch(0, A);
  if (nch > 1) load_K(1);
  write_H(0);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    chunk(c, A, B);
    if (c + 1 < nch) chunk(c + 1, B, A);
  }

#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 32 * w + 16 * mt + 4 * q4 + e;
      S_final[(((size_t)s * d.Hv + h) * kD + r) * kD + col] = H[mt][e];
    }
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

static size_t ws_bytes(int32_t n_seqs, int32_t L, int32_t Hv) {
  const size_t n_chunks = ((size_t)L + kC - 1) / kC;
  return (size_t)n_seqs * n_chunks * Hv * WsLayout::kBytes;
}

static int check_sizes(int32_t n_seqs, int32_t L, int32_t Hv, int32_t Hk,
                       int32_t dk, int32_t dv) {
  if (n_seqs < 1 || L < 1 || Hv < 1 || Hk < 1 || Hv % Hk != 0) {
    return fail(GDN_EINVAL, "prefill: sizes out of range");
  }
  if (dk != kD || dv != kD) {
    return fail(GDN_EUNSUPPORTED, "prefill: d_k = d_v = 128 only");
  }
  if ((double)L * Hv * kD >= 2147483648.0 || (double)L * Hk * kD >= 2147483648.0)
    return fail(GDN_EUNSUPPORTED, "prefill: seq_len x heads x 128 must stay below 2^31");
  const double blocks = (double)n_seqs * ((L + kC - 1) / kC) * Hv;
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
                                              int32_t d_k, int32_t d_v) {
  if (check_sizes(n_seqs, seq_len, h_v, h_k, d_k, d_v) != GDN_OK) return 0;
  return ws_bytes(n_seqs, seq_len, h_v);
}

extern "C" int gdn_prefill_chunked(
    int32_t n_seqs, int32_t seq_len, int32_t h_v, int32_t h_k, int32_t d_k,
    int32_t d_v, int32_t ckpt_interval, const void* q, const void* k,
    const void* v, int in_dtype, const float* beta, const float* g,
    const float* S_init, float* S_final, float* o, float* checkpoints,
    void* workspace, size_t ws_size, float scale, int flags, void* stream) {
  int rc = check_sizes(n_seqs, seq_len, h_v, h_k, d_k, d_v);
  if (rc != GDN_OK) return rc;
  if (!q || !k || !v || !beta || !g || !S_final || !o || !workspace) {
    return fail(GDN_EINVAL, "prefill: required pointer is NULL");
  }
  if (in_dtype != GDN_BF16) {
    return fail(in_dtype == GDN_F32 ? GDN_EUNSUPPORTED : GDN_EINVAL, "prefill: bf16 inputs only");
  }
  if (flags & ~GDN_FLAG_L2NORM_QK) {
    return fail(GDN_EINVAL, "prefill: unknown flag bits");
  }
  if (checkpoints && (ckpt_interval < kC || ckpt_interval % kC != 0)) {
    return fail(GDN_EINVAL, "prefill: ckpt_interval must be a positive multiple of 64");
  }
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 2) ||
      misaligned(beta, 4) || misaligned(g, 4) || misaligned(S_final, 4) ||
      misaligned(o, 4) || misaligned(workspace, 256) ||
      (S_init && misaligned(S_init, 4)) ||
      (checkpoints && misaligned(checkpoints, 4))) {
    return fail(GDN_EINVAL, "prefill: misaligned pointer");
  }
  if (ws_size < ws_bytes(n_seqs, seq_len, h_v)) {
    return fail(GDN_EWORKSPACE, "prefill: workspace too small");
  }
  PDims dd;
  dd.n_seqs = n_seqs;
  dd.L = seq_len;
  dd.Hv = h_v;
  dd.Hk = h_k;
  dd.group = h_v / h_k;
  dd.n_chunks = (seq_len + kC - 1) / kC;
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
  {
    const uint8_t* wsc = wsb;
    void* args[] = {(void*)&qq, (void*)&kk, (void*)&vv, (void*)&wsc,
                    (void*)&S_init, (void*)&S_final, (void*)&o,
                    (void*)&checkpoints, (void*)&dd};
    hipError_t e = hipLaunchKernel((const void*)p2_kernel,
                                   dim3(n_seqs * h_v * (kD / kTile)),
                                   dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return hip_fail("prefill p2 launch", e);
  }
  return GDN_OK;
}
