/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated-delta speculative-decoding path.
 *
 * The operations, all asynchronous on the caller's HIP stream:
 *
 *   gdn_verify           advance every (layer, lane, value head) recurrent
 *                        state S0 over a draft window of T <= t_max tokens by
 *                        the gated delta rule, write the outputs o_t = S_t q_t
 *                        and compact per-step transition records.  S0 itself
 *                        is never written.
 *   gdn_commit           ReplaySSM commit: replay the first m records of each
 *                        lane from the untouched S0 and store S_m in place.
 *   gdn_verify_tree,     the same for a draft tree (node t steps from its
 *   gdn_commit_path      parent) and the commit of an accepted path.
 *   gdn_commit_verify    both in one launch: commit the previous window's
 *                        accepted prefix, then verify the next window from
 *                        the committed state without reading it again.
 *   gdn_kda_verify,      verify and commit of the per-channel-decay sibling
 *   gdn_kda_commit       (KDA), same window protocol.
 *   gdn_state_snapshot,  copy the recurrent state of chosen lanes out to a
 *   gdn_state_restore    compact snapshot (device or pinned host memory) and
 *                        back, for requests that are paused and resumed.
 *   gdn_prefill_chunked  run the same recurrence over a long sequence in
 *                        chunks and emit fp32 state checkpoints at every
 *                        multiple of the checkpoint interval.
 *   gdn_prefill_chunked_noalloc  the same with the library's fixed scratch
 *                        array as workspace, for callers that cannot
 *                        allocate.
 *
 * The rule (Yang, Kautz & Hatamizadeh, "Gated Delta Networks: Improving
 * Mamba2 with Delta Rule", ICLR 2025, Sec. 3), per value head with state S
 * (a d_v x d_k matrix mapping keys to values):
 *
 *   khat = k / sqrt(|k|^2 + 1e-6), qhat likewise  (when GDN_FLAG_L2NORM_QK)
 *   alpha_t = exp(g_t)
 *   u_t = beta_t * (v_t - alpha_t * S_{t-1} khat_t)
 *   S_t = alpha_t * S_{t-1} + u_t khat_t^T
 *   o_t = scale * S_t qhat_t
 *
 * Value head h reads key head h / (h_v / h_k).
 *
 * The window protocol follows the NInfer technical review (blog.123qwe.co.kr
 * post 4624): section "Architecture 3: speculative decoding and ReplaySSM"
 * (one checkpoint plus compact records, replay of the accepted prefix from the
 * same S0, equality of the transitions in finite precision rather than over
 * the reals; 1..5 or 1..15 drafts plus the anchor token) and section
 * "Architecture 1: engine split by ownership" (results are provisional until
 * the real prefix is fixed; only then is the model state committed, so a
 * round that is cancelled simply never calls commit).  At most 8 active
 * requests per engine (the review's "key facts" table) -- the library takes
 * up to GDN_MAX_LANES.
 *
 * Storage layouts (row-major, outermost first; "bf16|f32" = in_dtype):
 *   q, k    [n_layers][n_lanes][t_max][h_k][d_k]       bf16|f32
 *   v       [n_layers][n_lanes][t_max][h_v][d_v]       bf16|f32
 *   beta, g [n_layers][n_lanes][t_max][h_v]            f32
 *   S       [n_layers][n_lanes][h_v][d_k][d_v]         f32 (S[.][j][i] = S_ij)
 *   o       [n_layers][n_lanes][t_max][h_v][d_v]       f32
 * Token rows t >= T_lane[lane] of q, k, v, beta, g are not read and the
 * matching rows of o are not written.
 *
 * Ownership: the caller allocates every buffer (device memory unless stated
 * "host"); the library allocates, frees and synchronises nothing and keeps no
 * state between calls, except the fixed scratch array that
 * gdn_prefill_chunked_noalloc uses as its workspace.  All pointers to device memory must be 4-byte aligned
 * (16-byte aligned for best speed).
 *
 * Errors: every argument error is found on the host, before any HIP call, and
 * returned as a negative gdn_status; nothing is launched then.  A launch
 * failure returns GDN_EHIP.  No C++ exception crosses this interface.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_MAX_LANES 256 /* lanes per call */
#define GDN_MAX_T 64      /* window tokens per lane (the pages use <= 16) */

typedef enum {
  GDN_OK = 0,
  GDN_EINVAL = -1,       /* bad argument (null pointer, range, shape) */
  GDN_EUNSUPPORTED = -2, /* valid but not built (e.g. d_k not in {16,32,64,128}) */
  GDN_EWORKSPACE = -3,   /* workspace too small */
  GDN_EHIP = -4          /* a HIP launch or runtime call failed */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

enum {
  GDN_FLAG_L2NORM_QK = 1,        /* normalise q and k inside the kernels */
  GDN_FLAG_PREFILL_ONE_CHAIN = 2, /* gdn_prefill_chunked*: never in segments */
  GDN_FLAG_TOKENWISE = 4         /* the verify calls: always token by token */
};

typedef struct {
  int32_t n_layers; /* >= 1: independent layers batched in one call       */
  int32_t n_lanes;  /* 1..GDN_MAX_LANES: requests (execution lanes)        */
  int32_t h_v;      /* >= 1 value heads                                    */
  int32_t h_k;      /* >= 1 key heads, h_v % h_k == 0                      */
  int32_t d_k;      /* key head dim: 16, 32, 64 or 128                     */
  int32_t d_v;      /* value head dim: 1..1024                             */
  int32_t t_max;    /* 1..GDN_MAX_T: window stride (anchor + drafts)       */
} gdn_dims;

/*
 * Bytes of the opaque record buffer that gdn_verify fills and gdn_commit
 * reads for these dims.  Returns 0 for invalid dims.  The records of one
 * verify stay valid until the next gdn_verify into the same buffer; S must
 * not be modified between a verify and its commit.
 *
 * Record contents (the "compact records that caused the transitions" of the
 * ReplaySSM section): per (layer, lane, token) the raw key rows widened to
 * f32 (f32 [h_k][d_k]); per value head the decay in scaled form, a float2
 * (phi, c) where c is the running state scale after this token and phi
 * the factor folded into the stored state before it (1 when none, 0 when
 * alpha_t = 0); and the
 * delta vectors with key norm and scale folded in,
 * u_t / (sqrt(|k_t|^2 + 1e-6) * c) (f32 [h_v][d_v]).  About 24.8 KB per
 * token per lane-layer at 32/16 heads of dim 128, against 2 MiB for a full
 * per-token state snapshot.
 */
size_t gdn_records_bytes(const gdn_dims* dims);

/*
 * Speculative-window verify (ReplaySSM section of the review).
 *   t_lane      host int32[n_lanes], 0..t_max: window length of each lane
 *               (0 = idle lane, nothing read or written for it).
 *   q, k, v     device, in_dtype; beta, g device f32 (layouts above).
 *   S           device f32, the window checkpoint S0; read only.
 *   o           device f32 outputs o_t = scale * S_t qhat_t.
 *   records     device, gdn_records_bytes(dims) bytes, written.
 *   dbg_states  device f32 [n_layers][n_lanes][t_max][h_v][d_k][d_v] or
 *               NULL: when given, every intermediate state S_1..S_T, as the
 *               kernel holds it (for tests; costs 64 KiB per head per token).
 *               With d_k = 128 and d_v a multiple of 128 the window is
 *               evaluated in blocks of 16 tokens (the chunked
 *               WY/UT form of the delta rule, Yang et al., NeurIPS 2024,
 *               Sec. 3) on the matrix cores, each block from the state the
 *               blocks before it leave (their rank-1 writes summed in one
 *               matrix-core product, equal to the token-by-token replay of
 *               their records to rounding); its intermediate states are
 *               then defined as the token-by-token replay of its own
 *               records, which is what dbg_states receives (asking for them
 *               changes neither o nor the records).
 *   scale       multiplies o only (1.0f for o_t = S_t q_t).
 *   flags       GDN_FLAG_L2NORM_QK, GDN_FLAG_TOKENWISE (evaluate token by
 *               token at every shape: verify then holds each intermediate
 *               state itself), or 0.
 *   stream      hipStream_t (NULL = the null stream).
 */
int gdn_verify(const gdn_dims* dims, const int32_t* t_lane, const void* q,
               const void* k, const void* v, int in_dtype, const float* beta,
               const float* g, const float* S, float* o, void* records,
               float* dbg_states, float scale, int flags, void* stream);

/*
 * ReplaySSM commit (ReplaySSM section of the review): for every lane with
 * m_lane[lane] > 0, replay records[0:m] from S (which must still hold the S0
 * that the matching gdn_verify read) and store S_m into S in place.  Lanes
 * with m = 0 are neither read nor written.  Commit never folds replayed
 * steps into a block product: it applies the recorded steps one token at a
 * time.  S_m is bit-for-bit the state written to dbg_states for token m:
 *   - on the token-by-token verify (d_k < 128, d_v not a multiple of
 *     128, or GDN_FLAG_TOKENWISE) that is the state verify held
 *     after its m-th token, formed by the same per-step instruction
 *     sequence;
 *   - on the block-form verify (d_k = 128, d_v a multiple of 128),
 *     which never forms per-token states, it is the replay of verify's
 *     records with commit's own operations.  There the emitted deltas and outputs
 *     agree with the rule applied to those replayed states to within about
 *     3e-7 (deltas) and 5e-6 (outputs) relative, not bit for bit.
 *   m_lane   host int32[n_lanes], 0..t_lane[lane]
 *   t_lane   host int32[n_lanes], as passed to the matching gdn_verify
 *   records  device, as filled by that gdn_verify
 *   S        device f32, in: S0, out: S_m
 */
int gdn_commit(const gdn_dims* dims, const int32_t* m_lane,
               const int32_t* t_lane, const void* records, float* S,
               void* stream);

/*
 * Draft-tree verify and accepted-path commit.  The speculative window of a
 * lane is a tree of draft tokens (draft trees are used together with DFlash2
 * by the engine the first page describes): node t steps from the state of
 * its parent, not from node t-1.  Records are per node, in the layout of
 * gdn_verify; commit replays the accepted root-to-node path from S0, and its
 * result is bit for bit the state verify held at the path's last node (the
 * ReplaySSM requirement, per node).
 *   parent   host int32 [n_lanes][t_max]: parent[n][t] in -1..t-1 for
 *            t < t_lane[n] (-1: the node steps from S0); nodes are ordered so
 *            that a parent precedes its children.  With d_k = 128 and d_v a
 *            multiple of 128 (and without GDN_FLAG_TOKENWISE) the tree is
 *            evaluated as block products on the matrix cores (the causal
 *            mask of the chunked form replaced by the ancestor relation;
 *            trees of more than 16 nodes in two blocks of 16, the second
 *            solved against its ancestors in the first) and any order costs
 *            the same; the debug state of a node is then the replay of the
 *            records on its root path, and asking for it changes neither o
 *            nor the records.  Otherwise depth-first order is cheapest: verify rebuilds
 *            the parent's state (S0 plus the path's recorded steps) whenever
 *            parent[t] != t - 1.
 *   path     host int32 [n_lanes][t_max]: the first m_lane[n] entries are the
 *            accepted nodes, root first, each the parent of the next.
 *   other arguments as for gdn_verify / gdn_commit.
 * Supported: t_max <= 32 and n_lanes * t_max <= 2048 (GDN_EUNSUPPORTED
 * otherwise); a bad parent or a path that is not a root-to-node chain is
 * GDN_EINVAL.
 */
int gdn_verify_tree(const gdn_dims* dims, const int32_t* t_lane,
                    const int32_t* parent, const void* q, const void* k,
                    const void* v, int in_dtype, const float* beta,
                    const float* g, const float* S, float* o, void* records,
                    float* dbg_states, float scale, int flags, void* stream);
int gdn_commit_path(const gdn_dims* dims, const int32_t* m_lane,
                    const int32_t* path, const int32_t* t_lane,
                    const int32_t* parent, const void* records, float* S,
                    void* stream);

/*
 * Fused commit + verify: the ReplaySSM commit of the previous window
 * followed by the verify of the next one, in one launch.  Equivalent, bit
 * for bit in S, o and records, to
 *   gdn_commit(dims, m_prev, t_prev, records_prev, S, stream);
 *   gdn_verify(dims, t_lane, q, k, v, in_dtype, beta, g, S, o, records,
 *              dbg_states, scale, flags, stream);
 * but the committed state S_m is passed from the replay to the new window in
 * registers, so the state is read once and written once per round instead of
 * read twice and written once (the commit mechanism of the ReplaySSM section,
 * with verify's separate read of S0 removed).
 *   m_prev, t_prev  host int32[n_lanes]: the previous window's accepted
 *                   prefix (0..t_prev) and length; m_prev = 0 leaves the
 *                   lane's S as it is
 *   records_prev    device, the previous gdn_verify / gdn_commit_verify
 *                   records (may be NULL when every m_prev is 0); must not
 *                   overlap records
 *   S               device f32, in: the previous window's S0, out: S_m
 *                   (the new window's S0, never advanced by the new window)
 *   other arguments as for gdn_verify.  A lane with t_lane = 0 and
 *   m_prev > 0 is committed only.
 * Errors: those of gdn_commit and gdn_verify, and GDN_EINVAL when the two
 * record buffers overlap.
 */
int gdn_commit_verify(const gdn_dims* dims, const int32_t* m_prev,
                      const int32_t* t_prev, const void* records_prev,
                      const int32_t* t_lane, const void* q, const void* k,
                      const void* v, int in_dtype, const float* beta,
                      const float* g, float* S, float* o, void* records,
                      float* dbg_states, float scale, int flags, void* stream);

/*
 * Workspace bytes that gdn_prefill_chunked needs for these sizes and chunk
 * length (0 for invalid or unsupported sizes).
 */
size_t gdn_prefill_workspace_bytes(int32_t n_seqs, int32_t seq_len,
                                   int32_t h_v, int32_t h_k, int32_t d_k,
                                   int32_t d_v, int32_t chunk);

/*
 * Chunked prefill of the gated delta rule with periodic state checkpoints
 * (interval default 8192 tokens: context_cache.checkpoint_interval in the
 * review's section "Architecture 2: context byte pool and prefix reuse").
 * Each chunk of `chunk` tokens is one step of the WY/UT block form of Yang
 * et al., "Parallelizing Linear Transformers with the Delta Rule over
 * Sequence Length" (NeurIPS 2024), extended with the per-token decay of
 * Gated DeltaNet; the state is carried in f32 from chunk to chunk (the
 * review's run configuration sets the prefill chunk as a parameter).
 *   n_seqs       >= 1 independent sequences of equal length seq_len >= 1
 *   chunk        tokens per block step: 16, 32 or 64 (GDN_EUNSUPPORTED
 *                otherwise; 64 is fastest: shorter chunks run in the same
 *                64-row tiles with the rows past the chunk inert)
 *   q, k         device [n_seqs][seq_len][h_k][d_k] in_dtype
 *   v            device [n_seqs][seq_len][h_v][d_v] in_dtype
 *   beta, g      device f32 [n_seqs][seq_len][h_v]
 *   S_init       device f32 [n_seqs][h_v][d_k][d_v] or NULL (zero state)
 *   S_final      device f32 [n_seqs][h_v][d_k][d_v], the state after the
 *                last token (may alias S_init)
 *   o            device f32 [n_seqs][seq_len][h_v][d_v]
 *   checkpoints  device f32 [n_seqs][seq_len / ckpt_interval][h_v][d_k][d_v]
 *                or NULL: the state after every token count that is a
 *                positive multiple of ckpt_interval
 *   ckpt_interval  positive multiple of chunk
 *   workspace    device, ws_bytes >= gdn_prefill_workspace_bytes(...);
 *                scratch owned by the caller, contents undefined on return
 *   scale        as for gdn_verify
 *   flags        GDN_FLAG_L2NORM_QK, GDN_FLAG_PREFILL_ONE_CHAIN, or 0
 * Segments: the chunk steps form one sequential chain per (head, 16 value
 * columns), so a batch with few sequence-heads leaves most of the GPU idle.
 * Sequences of more than 4,096 tokens with n_seqs * h_v <= 8 therefore run
 * in segments of 4,096 tokens, when checkpoints are off or their interval
 * is a multiple of 4,096.  Each sequence's results are bit for bit those of
 * the same sequence prefilled alone.  The state at a segment's end is
 * affine in its start state (the rule is linear in the state, so the maps
 * of consecutive tokens compose): each segment's
 * transition and offset are formed in parallel, scanned (f32-grade
 * products on the matrix cores), and the
 * segments then produce their outputs from the scanned start states.  The
 * results agree with the one-chain evaluation to rounding, not bit for bit;
 * checkpoints sit on segment boundaries, so a resumed prefill still
 * reproduces the rest bit for bit.  GDN_FLAG_PREFILL_ONE_CHAIN keeps the
 * one chain.  The workspace query includes room for the segments whenever
 * the sizes allow them.
 * Supported: d_k == d_v == 128, in_dtype == GDN_BF16 (q, k, v enter the
 * matrix cores as bf16; GDN_F32 returns GDN_EUNSUPPORTED).  The state,
 * decays and every accumulation are f32.  S_final and every checkpoint are
 * exactly the state the same call would pass on from that token, so a
 * prefill resumed from a checkpoint reproduces the rest bit for bit.
 * Errors: GDN_EINVAL for bad sizes or NULL required pointers,
 * GDN_EWORKSPACE when ws_bytes is too small, GDN_EHIP when a launch fails.
 */
int gdn_prefill_chunked(int32_t n_seqs, int32_t seq_len, int32_t h_v,
                        int32_t h_k, int32_t d_k, int32_t d_v, int32_t chunk,
                        int32_t ckpt_interval, const void* q, const void* k,
                        const void* v, int in_dtype, const float* beta,
                        const float* g, const float* S_init, float* S_final,
                        float* o, float* checkpoints, void* workspace,
                        size_t ws_bytes, float scale, int flags, void* stream);

/*
 * gdn_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is a fixed array inside
 * the library, GDN_PREFILL_SCRATCH_BYTES per GPU (each GPU the library runs
 * on holds its own copy until the process ends); this entry point calls no
 * allocator.  Every call on one GPU uses that GPU's array, so calls that
 * overlap in time on one GPU (different streams, or several host threads
 * without ordering) race and give undefined results: order them on one
 * stream or with events.  Nothing in the array needs to start at zero.
 * Sizes whose workspace (gdn_prefill_workspace_bytes) exceeds the array
 * return GDN_EWORKSPACE.  Arguments, results and the other errors are those
 * of gdn_prefill_chunked; the results are bit for bit the same.
 */
#define GDN_PREFILL_SCRATCH_BYTES (64u << 20)
int gdn_prefill_chunked_noalloc(int32_t n_seqs, int32_t seq_len, int32_t h_v,
                                int32_t h_k, int32_t d_k, int32_t d_v,
                                int32_t chunk, int32_t ckpt_interval,
                                const void* q,
                                const void* k, const void* v, int in_dtype,
                                const float* beta, const float* g,
                                const float* S_init, float* S_final, float* o,
                                float* checkpoints, float scale, int flags,
                                void* stream);

/*
 * KDA: the sibling rule with one decay per key channel (Kimi Delta
 * Attention, Kimi Linear, 2025; the review names its recurrent state beside
 * GDN's and a kda_replay op contract).  Per value head, with
 * alpha_t = exp(g_t) a d_k vector:
 *   S'_t = S_{t-1} diag(alpha_t),  u_t = beta_t (v_t - S'_t khat_t),
 *   S_t = S'_t + u_t khat_t^T,     o_t = scale * S_t qhat_t.
 * gdn_kda_verify / gdn_kda_commit have the contract of gdn_verify /
 * gdn_commit (S0 untouched by verify; commit(m) bitwise equal to verify's
 * state after token m) with these differences:
 *   g        device f32 [n_layers][n_lanes][t_max][h_v][d_k] (per channel)
 *   records  gdn_kda_records_bytes(dims) bytes: per token the raw key rows
 *            (f32 [h_k][d_k]), u_t / sqrt(|k_t|^2 + 1e-6) (f32 [h_v][d_v])
 *            and alpha_t (f32 [h_v][d_k])
 * Supported: d_k == 128 (GDN_EUNSUPPORTED otherwise; gdn_kda_records_bytes
 * returns 0).  For bf16 or f32 inputs with d_v = 128 (and without
 * GDN_FLAG_TOKENWISE) the window is evaluated in blocks of 16 tokens with
 * channel-weighted decays, each block from the state the blocks before it
 * leave (their writes summed in one matrix-core product, equal to the
 * token-by-token replay of their records to rounding); dbg_states then
 * receives the replay of its records, and asking for it changes neither o
 * nor the records (as for gdn_verify).
 */
size_t gdn_kda_records_bytes(const gdn_dims* dims);
int gdn_kda_verify(const gdn_dims* dims, const int32_t* t_lane,
                   const void* q, const void* k, const void* v, int in_dtype,
                   const float* beta, const float* g, const float* S, float* o,
                   void* records, float* dbg_states, float scale, int flags,
                   void* stream);
int gdn_kda_commit(const gdn_dims* dims, const int32_t* m_lane,
                   const int32_t* t_lane, const void* records, float* S,
                   void* stream);

/*
 * Recurrent-state snapshot and restore.  Under memory pressure the review's
 * engine pauses active requests and brings them back by replay or from a
 * snapshot, with a pinned host budget for such context (NInfer technical
 * review, section "Architecture 2: context byte pool and prefix reuse").
 * gdn_state_snapshot gathers the f32 state of n_sel lanes into a compact
 * lane-major snapshot; gdn_state_restore scatters a snapshot into lanes
 * (any lanes: a paused request may resume in another lane).  Exact copies.
 *   dims      as for gdn_verify (t_max and h_k are not used)
 *   n_sel     0..n_lanes lanes to copy (0: nothing is launched)
 *   lanes     host int32[n_sel], each in 0..n_lanes-1; restore rejects a
 *             lane listed twice
 *   S         device f32 [n_layers][n_lanes][h_v][d_k][d_v] (16-byte aligned)
 *   snapshot  f32 [n_sel][n_layers][h_v][d_k][d_v], device memory or pinned
 *             host memory (hipHostMalloc), 16-byte aligned; entry j holds
 *             lane lanes[j]
 * Errors: GDN_EINVAL for bad sizes, indices or pointers, GDN_EUNSUPPORTED
 * when h_v*d_k*d_v is not a multiple of 4, GDN_EHIP when the launch fails.
 */
int gdn_state_snapshot(const gdn_dims* dims, int32_t n_sel,
                       const int32_t* lanes, const float* S, float* snapshot,
                       void* stream);
int gdn_state_restore(const gdn_dims* dims, int32_t n_sel,
                      const int32_t* lanes, const float* snapshot, float* S,
                      void* stream);

/* Static description of a status code; never NULL. */
const char* gdn_strerror(int status);

/*
 * Detail of the most recent failing call on the calling thread (which
 * argument was rejected, or the HIP error string of a failed launch).  The
 * string is owned by the library and stays valid until the next failing call
 * on the same thread; never NULL.
 */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H_ */
