/*
 * vdn_local_attn.h -- C ABI of the MI355X (gfx950) local-window attention
 * forward pass: the local Softmax branch of VDN-H3 hybrid video attention.
 *
 * The operation (openi.cn "VDN-MiniMax-H3", section "technical principles:
 * local exact, remote compressed"; nav.superapi.store "VDN-MiniMax-H3 -
 * OpenVDN's Open-Source Video Generation Acceleration Solution", section
 * "Technical Principles", items "Local Softmax Branch", "Text Dual-Branch
 * Injection" and "Gated Fusion Mechanism"):
 *
 *   The sequence holds F latent frames of T tokens each (frame-major), then
 *   N text tokens: S = F*T + N.  Frames are grouped into blocks of
 *   `block_frames` consecutive frames starting at frame 0 (the last block may
 *   be short).  A video query of block b attends, with exact softmax, to
 *     - every token of blocks b-1, b, b+1 (clipped to the video),
 *     - every token of frames 0 and F-1 (boundary anchors, visible to all),
 *     - every text token.
 *   A text query attends to all S tokens.  With s = scale * q.k, the output is
 *   o_i = sum_j softmax_j(s_ij) v_j over the query's key set, optionally
 *   multiplied by sigmoid(gate[b, i, h]).  block_frames >= F gives plain full
 *   attention (the dense baseline).
 *
 * Conventions shared by every entry point:
 *   - Return value: VDN_OK (0) or a negative vdn_status_t.  On error a message
 *     is available from vdn_last_error() on the calling thread.  No C++
 *     exception crosses this boundary.
 *   - Sizes are plain ints; token offsets in outputs are int64.
 *   - Host-only functions never touch the GPU and may be called without one.
 */
#ifndef VDN_LOCAL_ATTN_H
#define VDN_LOCAL_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Canonical key lists never need more than 3 intervals ([0,T), the block
 * window, and [(F-1)T, S)); output arrays reserve this many slots. */
#define VDN_MAX_KEY_INTERVALS 4
/* Largest number of query blocks (frame blocks + 1 text block) the forward
 * kernel accepts: F <= 63 * block_frames. */
#define VDN_MAX_QUERY_BLOCKS 64

typedef enum {
  VDN_BF16 = 0,      /* bfloat16 q/k/v                                          */
  VDN_FP8_E4M3 = 1   /* OCP float8 e4m3fn q/k/v with per-head fp32 scales       */
} vdn_dtype_t;

typedef enum {
  VDN_OK = 0,
  VDN_ERR_INVALID_ARG = -1, /* non-positive size, negative n_text, NULL pointer,
                               or output aliasing an input                      */
  VDN_ERR_UNSUPPORTED = -2, /* head_dim not in {64,128}, unknown dtype, fp8
                               without scales or with head_dim != 128, too many
                               query blocks                                     */
  VDN_ERR_ALIGNMENT = -3,   /* q/k/v/out not 16-byte aligned, gate/lse/scales
                               not 4-byte aligned                               */
  VDN_ERR_OVERFLOW = -4,    /* S or a tensor's element count does not fit the
                               kernel's index types, or 128 token strides
                               (128 * heads * head_dim * element bytes) reach
                               2^32 bytes (the tiled kernels' 32-bit per-lane
                               DMA offsets)                                     */
  VDN_ERR_HIP = -5,         /* a HIP runtime call failed (message has details) */
  VDN_ERR_CAPACITY = -6     /* a host output array, or the fixed scratch of
                               vdn_local_attn_bwd_noalloc, is too small          */
} vdn_status_t;

/*
 * Forward pass, asynchronous on `hip_stream`.
 *
 *   q, k, v   device, [batch, S, heads, head_dim] contiguous, dtype `dtype`
 *             (S = F*tokens_per_frame + n_text; video tokens frame-major,
 *             then text tokens).
 *   gate      device, [batch, S, heads] fp32 logits, or NULL for no gate.
 *             The output row is multiplied by 1/(1+exp(-gate)).
 *   out       device, [batch, S, heads, head_dim] bfloat16, written in full.
 *   F, tokens_per_frame, n_text, block_frames
 *             frames (>=1), tokens per frame (>=1), text tokens (>=0),
 *             frames per block (>=1; >= F selects full attention).
 *   heads, head_dim, dtype
 *             heads (>=1); head_dim 64 or 128 (fp8: 128 only); VDN_BF16 or
 *             VDN_FP8_E4M3.
 *   batch     samples (>=1).
 *   qkv_scales device fp32 [3][heads] (q, k, v scale of each head) for fp8:
 *             the real value of a code c of head h is c * scale[h].
 *             Must be NULL for bf16.
 *   softmax_scale  score scale; <= 0 selects 1/sqrt(head_dim).
 *   lse       device fp32 [batch, heads, S] or NULL: natural-log
 *             log-sum-exp of the scaled scores over each query's key set.
 *   hip_stream a hipStream_t, or NULL for the default stream.
 *
 * Ownership: every buffer belongs to the caller and must stay alive until the
 * work on `hip_stream` completes.  The call allocates no device memory and
 * does not synchronise.  `out` and `lse` must not overlap q, k, v, gate or
 * each other.  Arguments are validated before any HIP call; a launch failure
 * returns VDN_ERR_HIP.
 *
 * Shared state: the forward kernels run one resident workgroup per compute
 * unit, each taking query tiles from per-XCD work queues.  Their claim
 * counters live in the library's static device memory (no allocation), one
 * set per launch handed out in rotation from 4096 sets per device and
 * process, and each launch leaves its set zero when it ends.  So at most 4096
 * forward launches may be in flight at once per device and process, and a
 * launch recorded into a HIP graph must not run concurrently with another
 * replay of itself (replays in stream order are fine).  The first call on a
 * device looks up the counters' address and the kernel's occupancy (host
 * queries, cached); make it outside stream capture.
 */
int vdn_local_attn_fwd(const void* q, const void* k, const void* v,
                       const float* gate, void* out,
                       int F, int tokens_per_frame, int n_text, int block_frames,
                       int heads, int head_dim, int dtype,
                       int batch, const float* qkv_scales, float softmax_scale,
                       float* lse, void* hip_stream);

/*
 * Backward pass (bf16 inputs only), asynchronous on `hip_stream`: the
 * gradients of vdn_local_attn_fwd's output with respect to q, k, v and the
 * gate logits, for an upstream gradient `dout`.  Derivative of the forward
 * operation above (chain rule through the gate, the softmax and the two
 * products).
 *
 *   q, k, v, gate, F .. block_frames, heads, head_dim, batch, softmax_scale
 *             as for the forward (dtype VDN_BF16, head_dim 64 or 128).
 *   out       device, [batch, S, heads, head_dim] bfloat16: the forward's
 *             output for these inputs.
 *   lse       device fp32 [batch, heads, S]: the forward's log-sum-exp.
 *   dout      device, [batch, S, heads, head_dim] bfloat16.
 *   dq, dk, dv device, [batch, S, heads, head_dim] bfloat16, written in full.
 *   dgate     device fp32 [batch, S, heads], written in full; must be NULL
 *             exactly when gate is NULL.
 *   workspace device fp32, 2 * batch * heads * S floats of caller-owned
 *             scratch (per-row constants); contents on return unspecified.
 *
 * Ownership and errors as for the forward: no allocation, no
 * synchronisation, validation before any HIP call.  The outputs and the
 * workspace must not overlap each other or any input.
 */
int vdn_local_attn_bwd(const void* q, const void* k, const void* v,
                       const float* gate, const void* out, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv,
                       float* dgate, int F, int tokens_per_frame, int n_text,
                       int block_frames, int heads, int head_dim, int batch,
                       float softmax_scale, float* workspace, void* hip_stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * backward pass with the per-row constants in a fixed scratch array that the
 * library holds on each GPU it runs on (32 MiB, kept until the process ends)
 * instead of a caller workspace.  Arguments, layout, ownership and errors as
 * for vdn_local_attn_bwd without `workspace`, plus:
 *   - batch * heads * S above 4194304 rows returns VDN_ERR_CAPACITY before
 *     any HIP call;
 *   - the call allocates nothing and calls no allocating routine; on its
 *     first use on a device it looks up the array's address there
 *     (hipGetSymbolAddress; a failure returns VDN_ERR_HIP);
 *   - every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (different streams, or threads) race and must be
 *     serialised by the caller.  Nothing in the array needs clearing: the
 *     first kernel of the pass writes every row it later reads.
 */
int vdn_local_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                               const float* gate, const void* out, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv,
                               float* dgate, int F, int tokens_per_frame, int n_text,
                               int block_frames, int heads, int head_dim, int batch,
                               float softmax_scale, void* hip_stream);

/*
 * Complement linear branch, forward (bf16), asynchronous on `hip_stream`.
 * openi.cn "VDN-MiniMax-H3", section "technical principles: local exact,
 * remote compressed": the linear branch summarises the context before and
 * after a block's window, leaving out the window frames and the boundary
 * anchors; nav.superapi.store "VDN-MiniMax-H3 - OpenVDN's Open-Source Video
 * Generation Acceleration Solution", Technical Principles, "Hybrid Attention
 * Architecture": long-range attention of linear cost.  Plain linear attention
 * with the feature map phi(x) = elu(x) + 1 (the pages fix no feature map and
 * do not define their frame-level state update; this is the plain form):
 *
 *   for a video query i of frame block b, with K_lin(b) the video tokens of
 *   frames f, 1 <= f <= F-2, outside the window of blocks b-1..b+1,
 *     out_i = sum_j (phi(q_i).phi(k_j)) v_j / sum_j phi(q_i).phi(k_j),
 *   j over K_lin(b); out_i = 0 for text queries and when K_lin(b) is empty.
 *   Together with vdn_local_attn_fwd's key sets this splits every
 *   (query, key) pair between the two branches.
 *
 *   q, k, v   device, [batch, S, heads, head_dim] bfloat16, S = F*T + N.
 *   out       device, same shape, bfloat16, written in full.
 *   F .. block_frames, heads, batch  as for vdn_local_attn_fwd.
 *   head_dim  64 or 128.  batch * heads <= 65535.
 *   workspace device, caller-owned scratch of at least workspace_bytes >=
 *             vdn_linear_branch_workspace_bytes(...) bytes, 256-byte aligned;
 *             holds per-frame and per-block states; contents on return
 *             unspecified.
 *
 * Internally the products run on bf16 MFMA with fp32 accumulation: phi(k),
 * phi(q) and the per-block state are rounded to bf16; the normaliser sum of
 * phi(k) is accumulated in fp32 and enters the final product as two bf16
 * parts (hi + lo, about 2^-17 of its value).  No allocation, no synchronisation, validation before any HIP call;
 * out and the workspace must not overlap each other or an input.
 */
int vdn_linear_branch_fwd(const void* q, const void* k, const void* v,
                          void* out, int F, int tokens_per_frame, int n_text,
                          int block_frames, int heads, int head_dim, int batch,
                          void* workspace, int64_t workspace_bytes,
                          void* hip_stream);

/* Host only.  Workspace bytes vdn_linear_branch_fwd needs for this shape
 * (B*H*(F-2)*(D*D+D) fp32 frame states, B*H*nb*D*D bf16 block states and
 * B*H*nb*D fp32 normalisers, each region rounded up to 256 bytes), or a
 * negative vdn_status_t. */
int64_t vdn_linear_branch_workspace_bytes(int F, int tokens_per_frame,
                                          int n_text, int block_frames,
                                          int heads, int head_dim, int batch);

/*
 * Two-branch fusion, asynchronous on `hip_stream` (openi.cn "VDN-MiniMax-H3",
 * section "technical principles": the linear branch's output is
 * RMS-normalised, then multiplied by its own content-dependent sigmoid gate,
 * and the branches are added; the output projections that follow are not
 * part of this call).  Per token t (a row of heads * head_dim values):
 *
 *   out[t] = soft_out[t] + sigmoid(gate_lin[t, h]) * lin_out[t]
 *            * norm_weight / sqrt(mean(lin_out[t]^2) + eps),
 *
 * the mean over all heads * head_dim values of the token, h the head of each
 * value.  soft_out is the softmax branch's output with its own gate already
 * applied (vdn_local_attn_fwd with a gate).
 *
 *   soft_out, lin_out  device, [tokens, heads, head_dim] bfloat16.
 *   gate_lin           device fp32 [tokens, heads] logits.
 *   norm_weight        device fp32 [heads * head_dim].
 *   out                device, [tokens, heads, head_dim] bfloat16; may be
 *                      the soft_out buffer itself, otherwise must not overlap
 *                      an input.
 *   head_dim           a multiple of 8; heads * head_dim <= 8192.
 *   eps                finite, > 0 (a token whose linear row is all zeros
 *                      then gets a linear term of exactly 0).
 * bf16 buffers and norm_weight 16-byte aligned, gate_lin 4-byte aligned.
 * tokens == 0 is a no-op.  No allocation, no synchronisation.
 */
int vdn_hybrid_fuse(const void* soft_out, const void* lin_out,
                    const float* gate_lin, const float* norm_weight, float eps,
                    void* out, int64_t tokens, int heads, int head_dim,
                    void* hip_stream);

/*
 * The hybrid attention output in one call, asynchronous on `hip_stream`: the
 * complement linear branch of q, k, v (as vdn_linear_branch_fwd), then the
 * local softmax branch (as vdn_local_attn_fwd, bf16) whose epilogue adds the
 * linear branch exactly as vdn_hybrid_fuse does (openi.cn "VDN-MiniMax-H3",
 * section "technical principles"):
 *
 *   out[t] = softmax branch with its gate[t]
 *            + sigmoid(gate_lin[t, h]) * lin[t] * norm_weight
 *              / sqrt(mean(lin[t]^2) + eps),
 *
 * summed in fp32 and rounded to bf16 once (the two-call path rounds the
 * softmax branch first).  The mean of squares comes from the linear branch's
 * values before their rounding.
 *
 *   q, k, v, gate, F .. block_frames, heads, head_dim, batch, softmax_scale,
 *   lse      as for vdn_local_attn_fwd (bf16, head_dim 64 or 128; gate and
 *            lse may be NULL).
 *   gate_lin device fp32 [batch, S, heads] logits of the linear branch's gate.
 *   norm_weight device fp32 [heads * head_dim], 16-byte aligned.
 *   eps      finite, > 0 (an all-zero linear row then contributes exactly 0).
 *   out      device, [batch, S, heads, head_dim] bfloat16.
 *   workspace device, caller-owned, at least vdn_hybrid_attn_workspace_bytes
 *            bytes, 256-byte aligned; holds the linear branch's states, its
 *            output and its per-(token, head) sums of squares.
 * Validation before any HIP call; no allocation, no synchronisation.  The
 * workspace must not overlap any input or output, and out and lse must not
 * overlap gate_lin or norm_weight.
 */
int vdn_hybrid_attn_fwd(const void* q, const void* k, const void* v,
                        const float* gate, const float* gate_lin,
                        const float* norm_weight, float eps, void* out,
                        int F, int tokens_per_frame, int n_text,
                        int block_frames, int heads, int head_dim, int batch,
                        float softmax_scale, float* lse, void* workspace,
                        int64_t workspace_bytes, void* hip_stream);

/* Host only.  Workspace bytes vdn_hybrid_attn_fwd needs for this shape (the
 * linear branch's, plus batch * S * heads * (2 * head_dim + 4), each part
 * rounded up to 256 bytes), or a negative vdn_status_t. */
int64_t vdn_hybrid_attn_workspace_bytes(int F, int tokens_per_frame,
                                        int n_text, int block_frames,
                                        int heads, int head_dim, int batch);

/*
 * Host only.  Number of query blocks for a geometry: ceil(F/block_frames)
 * frame blocks, plus one text block when n_text > 0.  The grouping of
 * latent frames into blocks of consecutive frames is the one of openi.cn
 * "VDN-MiniMax-H3", technical principles (five frames per block there).  Returns the count
 * (>= 1) or a negative vdn_status_t.
 */
int vdn_local_attn_num_query_blocks(int F, int tokens_per_frame, int n_text,
                                    int block_frames);

/*
 * Host only.  The canonical key structure of every query block, in the
 * kernel's block order (frame blocks by index, then text).  It is the key
 * set rule at the top of this header written as token intervals (openi.cn
 * "VDN-MiniMax-H3", technical principles: own block and its neighbours,
 * first/last-frame anchors; nav.superapi.store, Technical Principles,
 * "Local Softmax Branch" and "Text Dual-Branch Injection": text keys seen
 * by every frame):
 *   query_rows    [capacity][2] int64: half-open query token range of each
 *                 block (may be NULL);
 *   key_intervals [capacity][VDN_MAX_KEY_INTERVALS][2] int64: sorted,
 *                 disjoint, non-touching half-open key token intervals; unused
 *                 slots are -1 (may be NULL).
 *   *n_qblocks    receives the number of blocks written.
 * Returns VDN_ERR_CAPACITY (and sets *n_qblocks) if capacity is too small.
 */
int vdn_local_attn_key_intervals(int F, int tokens_per_frame, int n_text,
                                 int block_frames, int64_t* query_rows,
                                 int64_t* key_intervals, int capacity,
                                 int* n_qblocks);

/*
 * Host only.  Closed-form counts per (sample, head): *allowed = number of
 * (query, key) pairs attended; *anchor_added = video pairs present only
 * because the key frame is an anchor (frame 0 or F-1) outside the window.
 * These are the quantities behind the anchors' share of the attended pairs
 * quoted in nav.superapi.store, Technical Principles, "Local Softmax
 * Branch", and behind the softmax/linear split of openi.cn "VDN-MiniMax-H3",
 * technical principles (same key set rule as above).
 */
int vdn_local_attn_count_pairs(int F, int tokens_per_frame, int n_text,
                               int block_frames, int64_t* allowed,
                               int64_t* anchor_added);

/*
 * Host only.  The per-(sample, head) query-tile work list (longest key list
 * first; ties by block index, then row).  The pages define no work
 * decomposition; each tile's key list is that of its block under the rule
 * above (openi.cn "VDN-MiniMax-H3", technical principles), and the order is
 * this implementation's: entries [capacity][4] int32 =
 * {query block, first row, rows, keys}, tiles of `tile_m` rows that never
 * straddle a block boundary.  *n_entries receives the count;
 * VDN_ERR_CAPACITY if capacity is too small.  The kernels concatenate these
 * lists over (sample, head) and give each of the 8 XCDs one contiguous
 * eighth, in order; a list that spans several eighths is dealt over them
 * (entry s to the (s mod k)-th), and the last tiles of an eighth may run as
 * two halves of tile_m / 2 rows (schedule only: the results agree up to
 * rounding; the bf16 forward splits a half's keys between two waves and
 * merges their rows, which rounds differently from one wave).
 */
int vdn_local_attn_tile_schedule(int F, int tokens_per_frame, int n_text,
                                 int block_frames, int tile_m, int32_t* out,
                                 int capacity, int* n_entries);

/*
 * Host only.  The key side of the structure, used by the backward pass: the
 * same key set rule (openi.cn "VDN-MiniMax-H3", technical principles) read
 * from the keys' side, with keys grouped by the query rows that see them
 * (frame blocks by index with their
 * non-anchor frames, skipped when empty; then the anchor-frame and text keys,
 * skipped when empty):
 *   key_intervals   [capacity][VDN_MAX_KEY_INTERVALS][2] int64: the group's
 *                   keys, canonical as above, unused slots -1 (may be NULL);
 *   query_intervals [capacity][VDN_MAX_KEY_INTERVALS][2] int64: the query
 *                   rows that see every key of the group (may be NULL).
 *   *n_kblocks      receives the number of groups.
 * Returns VDN_ERR_CAPACITY (and sets *n_kblocks) if capacity is too small.
 */
int vdn_local_attn_key_blocks(int F, int tokens_per_frame, int n_text,
                              int block_frames, int64_t* key_intervals,
                              int64_t* query_intervals, int capacity,
                              int* n_kblocks);

/* Query rows per tile used by the forward kernel for a head_dim / dtype pair
 * (so callers can reproduce its schedule with vdn_local_attn_tile_schedule),
 * or a negative vdn_status_t.  An implementation parameter: no passage of
 * the pages defines it. */
int vdn_local_attn_kernel_tile_m(int head_dim, int dtype);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next call into this library on the same thread. */
const char* vdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VDN_LOCAL_ATTN_H */
