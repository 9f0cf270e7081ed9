/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta-rule library.
 *
 * The library computes chunked Gated DeltaNet linear attention for prefill and a
 * single-token decode step.  Per sequence n and value head h, with key/query head
 * hk = h % Hk (the GQA head replication hv % Hk described on the page
 * "Exp 2026-07-13 -- Linear-Attention Scans on the NPU", section 4), the state
 * S (Dv x Dk, fp32) evolves token by token as
 *
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t * v_t k_t^T,
 *     o_t = S_t q_t,               alpha_t = exp(g_t),
 *
 * i.e. the state is updated with k_t, v_t first and the output is then read with
 * q_t from the updated state ("Empowering Hybrid Attention Models on NPUs",
 * section 2.1).  Prefill evaluates this exactly (up to rounding) with the chunkwise
 * Map-Reduce-Map decomposition of that page (operators #1 Gate, #2 KKT, #3 Solve,
 * #4 W/U, #5 H, #6 O), chunk-first ordered and with the inverse factored out of
 * the W product as in its section 5.  No scaling is applied to q.
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller, row-major and
 *     contiguous.  q, k, v, o and the states are 16-byte aligned (the decode steps
 *     take v and o 4-byte aligned); g and beta 4-byte aligned, except a per-key-channel
 *     g (16-byte); cu_seqlens 4-byte; workspaces 256-byte.  The library allocates and
 *     frees no device memory and keeps no pointer after the call returns; the one
 *     device memory it holds is the static scratch of gdn_prefill_split_noalloc.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 *     call returns without synchronising.  Inputs are never written.
 *   - Argument errors are detected on the host before anything is enqueued; the
 *     call then returns a non-OK status, launches nothing and records a message
 *     retrievable with gdn_last_error() (thread-local).  A failed kernel launch
 *     returns GDN_ERR_DEVICE.  No C++ exception crosses this interface.
 *   - The contents of cu_seqlens (device memory) are a precondition the kernels do
 *     not check: with the environment variable GDN_CHECK set (to anything but "" or
 *     "0"), every prefill entry point first reads cu_seqlens back (ordered after the
 *     work already on `stream`, then waiting for it) and returns
 *     GDN_ERR_INVALID_ARGUMENT unless cu[0] = 0, cu is nondecreasing and
 *     cu[N] = T_tot; not for use under stream capture.
 *   - Supported shapes: Dk = Dv = 128; chunk_size 64, and also 32 and 128 for the
 *     scalar-gate two-launch paths (gdn_prefill_split*, gdn_prefill_seg); anything
 *     else returns GDN_ERR_UNSUPPORTED.
 *   - Value range with bf16 or fp16 I/O (every prefill entry point): the per-chunk
 *     products (v = U - W S^T, P, U, W and the decayed keys and queries) and the
 *     state's 16-bit copy that the recurrence multiplies with are fp16, whose largest
 *     finite value is 65504.  Results are within tolerance while the entries of v,
 *     of the states (initial, final and in between) and of o stay below about 6e4 in
 *     magnitude and g <= 0 (a decay: alpha = exp(g) in (0, 1], as the pages define
 *     it).  Beyond that the outputs may hold inf or NaN; no error is reported.  fp32
 *     I/O (gdn_prefill) and the decode steps keep fp32 throughout.
 */
#ifndef GDN_MI355X_GDN_H
#define GDN_MI355X_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1,  /* null/misaligned pointer, bad size or head counts    */
    GDN_ERR_UNSUPPORTED = 2,       /* valid request this build does not implement         */
    GDN_ERR_DEVICE = 3             /* the HIP runtime reported an error on launch          */
} gdn_status;

typedef enum gdn_dtype {
    GDN_F32 = 0,   /* q, k, v, o stored as IEEE fp32; all arithmetic in fp32                   */
    GDN_BF16 = 1,  /* q, k, v, o stored as bf16; fp32 accumulation and state, 16-bit products  */
    GDN_F16 = 2    /* q, k, v, o stored as fp16; fp32 accumulation and state, fp16 products    */
} gdn_dtype;

/*
 * Input prologue flags (bitwise or) of gdn_prefill_fused and gdn_decode_step_fused: the
 * steps that turn a linear-attention layer's projection outputs into the recurrence's
 * inputs, applied inside the kernels' load path.  "Empowering Hybrid Attention Models on
 * NPUs", section 7 (the full-layer implementation notes before 7.1), counts a layer's
 * input projections as part of it and fuses their operators; these are the elementwise
 * and per-row steps between those projections and the recurrence.
 */
typedef enum gdn_prologue_flags {
    GDN_PROLOGUE_QK_L2NORM = 1,     /* q, k rows (per token and key head) divided by
                                       max(||x||_2, 1e-12), computed in fp32           */
    GDN_PROLOGUE_BETA_SIGMOID = 2,  /* beta = 1 / (1 + exp(-x)) of the beta argument    */
    GDN_PROLOGUE_G_SOFTPLUS = 4     /* g = -softplus(x) = -log(1 + exp(x)) of the g
                                       argument, so the decay exp(g) lies in (0, 1)     */
} gdn_prologue_flags;

/*
 * gdn_prefill -- packed variable-length chunked prefill.
 *
 * Operation: the recurrence above over every sequence of a packed batch, each
 * sequence starting from its own initial state ("Empowering Hybrid Attention Models
 * on NPUs", section 3: the online stage takes Q/K/V, gates and an initial state and
 * returns outputs plus updated states for later decoding).  Chunks of `chunk_size`
 * tokens restart at every sequence start; a sequence's last chunk may be short.
 *
 *   q, k           [T_tot, Hk, Dk]  io_dtype      queries / keys, per key head
 *   v              [T_tot, Hv, Dv]  io_dtype      values, per value head
 *   g              [T_tot, Hv]      fp32          natural log of the decay alpha
 *                                                 (finite, <= 0; see the value range)
 *   beta           [T_tot, Hv]      fp32          delta-rule write strength
 *   initial_state  [N, Hv, Dv, Dk]  fp32 or NULL  NULL means zero states
 *   cu_seqlens     [N+1]            int32 device  cu[0] = 0, nondecreasing,
 *                                                 cu[N] = T_tot (precondition,
 *                                                 checked only under GDN_CHECK); may
 *                                                 be NULL only when N == 1
 *   N, T_tot       number of sequences (>= 1) and packed tokens (>= 0)
 *   Hk, Hv         key and value head counts, Hv % Hk == 0
 *   Dk, Dv         head dimensions (128)
 *   chunk_size     64
 *   io_dtype       storage type of q, k, v and o
 *   o              [T_tot, Hv, Dv]  io_dtype      written; must not alias an input
 *   final_state    [N, Hv, Dv, Dk]  fp32 or NULL  written when non-NULL; may alias
 *                                                 initial_state exactly (in-place)
 *   stream         hipStream_t or NULL
 *
 * A sequence of length 0 gets final_state = initial_state (or zeros).
 */
gdn_status gdn_prefill(const void *q, const void *k, const void *v,
                       const float *g, const float *beta,
                       const float *initial_state, const int32_t *cu_seqlens,
                       int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                       int32_t Dk, int32_t Dv, int32_t chunk_size, gdn_dtype io_dtype,
                       void *o, float *final_state, void *stream);

/*
 * gdn_decode_step -- one token per sequence, state updated in place (the
 * token-by-token recurrence that serves decoding: "Empowering Hybrid Attention
 * Models on NPUs", section 2.1).
 *
 *   q, k     [B, Hk, Dk]      io_dtype
 *   v        [B, Hv, Dv]      io_dtype
 *   g, beta  [B, Hv]          fp32
 *   state    [B, Hv, Dv, Dk]  fp32, read and overwritten
 *   o        [B, Hv, Dv]      io_dtype, written
 */
gdn_status gdn_decode_step(const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float *state,
                           int32_t B, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                           gdn_dtype io_dtype, void *o, void *stream);

/*
 * gdn_prefill_fused -- gdn_prefill with the input prologue applied in the kernel's load
 * path: `prologue` is a bitwise or of gdn_prologue_flags, and q, k, g, beta are the
 * values before the selected steps (unnormalised q/k rows, beta and g logits).  The L2
 * norms are taken in fp32 from the stored q/k and folded into the kernel's per-row
 * factors, so q and k themselves enter the products unchanged.  io_dtype GDN_BF16 or
 * GDN_F16 (GDN_F32 returns GDN_ERR_UNSUPPORTED); unknown flag bits return
 * GDN_ERR_INVALID_ARGUMENT.  Everything else as gdn_prefill.
 */
gdn_status gdn_prefill_fused(const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                             int32_t Dk, int32_t Dv, int32_t chunk_size, gdn_dtype io_dtype,
                             uint32_t prologue, void *o, float *final_state, void *stream);

/*
 * gdn_decode_step_fused -- gdn_decode_step with the input prologue (any io_dtype).
 */
gdn_status gdn_decode_step_fused(const void *q, const void *k, const void *v,
                                 const float *g, const float *beta, float *state,
                                 int32_t B, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                                 gdn_dtype io_dtype, uint32_t prologue, void *o, void *stream);

/*
 * Per-key-channel decay (KDA).  The gate of this variant of the delta rule is "fine
 * grained": one decay per key channel instead of one per head, so its cumulative gate
 * is Dk times larger ("Empowering Hybrid Attention Models on NPUs", section 2.1, and
 * section 7.5 on peak memory).  The scalar alpha_t above becomes Diag(a_t) acting on
 * the key index of S, applied where alpha_t is (before the erase):
 *
 *     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,               a_t[j] = exp(g_t[j]).
 *
 * With every channel's g equal this is the gated delta rule above.
 *
 * gdn_kda_workspace_size -- device bytes gdn_kda_prefill needs as workspace for these
 * sizes: one 72,192-byte tile per value head and chunk slot, with T_tot / 64 + N slots
 * (enough for any packing of N sequences into T_tot tokens).  Host pointer `bytes`.
 */
gdn_status gdn_kda_workspace_size(int32_t N, int32_t T_tot, int32_t Hv, int32_t chunk_size,
                                  size_t *bytes);

/*
 * gdn_kda_prefill -- packed variable-length chunked prefill with a per-key-channel
 * decay.  Arguments and conventions as for gdn_prefill, except:
 *
 *   g              [T_tot, Hv, Dk]  fp32          natural log of each key channel's
 *                                                 decay (finite, <= 0: the chunked
 *                                                 form multiplies decays of up to 64
 *                                                 tokens and relies on each being <= 1);
 *                                                 16-byte aligned
 *   io_dtype       GDN_BF16 or GDN_F16 (GDN_F32 returns GDN_ERR_UNSUPPORTED)
 *   workspace      device scratch owned by the caller, at least
 *                  gdn_kda_workspace_size(...) bytes, 256-byte aligned, overlapping no
 *                  other argument; its contents on entry are ignored and on return are
 *                  unspecified.  May be NULL when T_tot == 0.  Two calls in flight at
 *                  once must not share a workspace.
 *   workspace_bytes  its size in bytes
 *
 * Two kernels run in order on `stream`: one per (chunk, value head) that forms the
 * chunk's decay-weighted grams, T = (I + A)^-1, the products W = T diag(beta) K_decayed
 * and U = T diag(beta) V, and the decayed keys/queries into the workspace, then the
 * chunk-by-chunk state recurrence that reads them.
 */
gdn_status gdn_kda_prefill(const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           const float *initial_state, const int32_t *cu_seqlens,
                           int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                           int32_t Dk, int32_t Dv, int32_t chunk_size, gdn_dtype io_dtype,
                           void *workspace, size_t workspace_bytes,
                           void *o, float *final_state, void *stream);

/*
 * gdn_kda_decode_step -- one token per sequence with a per-key-channel decay, state
 * updated in place.  As gdn_decode_step, except g is [B, Hv, Dk] fp32, 16-byte aligned.
 * All three io_dtype values are supported.
 */
gdn_status gdn_kda_decode_step(const void *q, const void *k, const void *v,
                               const float *g, const float *beta, float *state,
                               int32_t B, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                               gdn_dtype io_dtype, void *o, void *stream);

/*
 * gdn_prefill_split -- gdn_prefill in two launches, with a caller-owned workspace: the
 * state-independent Map phases of every chunk of every value head first, all at once
 * (#1 Gate, #2 KKT and the Q K^T gram, #3 Solve: "Empowering Hybrid Attention Models on
 * NPUs", section 2.1, Figure 1(b)), then the chunk-by-chunk state recurrence that reads
 * their results.  Same results as gdn_prefill up to rounding; the faster of the two when
 * the (sequence, value head) pairs times 8 value-channel slices are fewer than the GPU's
 * compute units (gdn_prefill repeats the map work for each slice on the recurrence's
 * critical path).  Arguments as for gdn_prefill, plus:
 *
 *   chunk_size     32, 64 or 128 tokens per chunk (others return GDN_ERR_UNSUPPORTED);
 *                  the result does not depend on it beyond rounding.  64 is the fastest
 *                  on MI355X: 32 doubles the chain's serial steps, 128 quadruples the
 *                  intra-chunk products and the map's solve.
 *   io_dtype       GDN_BF16 or GDN_F16 (GDN_F32 returns GDN_ERR_UNSUPPORTED)
 *   workspace      device scratch owned by the caller, at least
 *                  gdn_prefill_split_workspace_size(...) bytes, 256-byte aligned,
 *                  overlapping no other argument; contents on entry ignored, on return
 *                  unspecified; may be NULL when T_tot == 0; not shared by two calls
 *                  in flight at once.
 *   workspace_bytes  its size in bytes
 *
 * gdn_prefill_split_workspace_size -- the workspace bytes for these sizes and chunk length:
 * one tile per value head and chunk slot (T_tot / chunk_size + N slots) of
 * C * 1024 + (C / 32) (C / 32 + 1) * 1024 + 512 bytes for C = chunk_size (72,192 at
 * C = 64, as for gdn_kda_workspace_size).  Host pointer `bytes`.
 */
gdn_status gdn_prefill_split_workspace_size(int32_t N, int32_t T_tot, int32_t Hv,
                                            int32_t chunk_size, size_t *bytes);
gdn_status gdn_prefill_split(const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                             int32_t Dk, int32_t Dv, int32_t chunk_size, gdn_dtype io_dtype,
                             void *workspace, size_t workspace_bytes,
                             void *o, float *final_state, void *stream);

/*
 * gdn_prefill_split_noalloc -- gdn_prefill_split for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same kernels and results, with the workspace taken from a
 * static array of GDN_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held from the
 * library's first use on that GPU until the process ends.  The call allocates nothing.
 * Arguments as for gdn_prefill_split without workspace / workspace_bytes.
 *
 *   Sizes whose gdn_prefill_split_workspace_size exceeds GDN_NOALLOC_SCRATCH_BYTES
 *   (96 MiB: e.g. 64-token chunks of up to 1394 (chunk slot, value head) pairs, which
 *   holds T_tot = 4096 at Hv = 16) return GDN_ERR_UNSUPPORTED before anything runs.
 *   Every call on one GPU uses that GPU's one array: two calls that overlap in time on
 *   the same GPU (different streams, or host threads without ordering) race and give
 *   undefined results.  Calls ordered on one stream are safe; nothing needs clearing
 *   between them.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
gdn_status gdn_prefill_split_noalloc(const void *q, const void *k, const void *v,
                                     const float *g, const float *beta,
                                     const float *initial_state, const int32_t *cu_seqlens,
                                     int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                                     int32_t Dk, int32_t Dv, int32_t chunk_size, gdn_dtype io_dtype,
                                     void *o, float *final_state, void *stream);

/*
 * gdn_prefill_split_fused -- gdn_prefill_split with the input prologue applied in the map
 * kernel's load path, as gdn_prefill_fused does for gdn_prefill: `prologue` is a bitwise
 * or of gdn_prologue_flags (unknown bits return GDN_ERR_INVALID_ARGUMENT), and q, k, g,
 * beta are then the raw inputs of the selected steps.  Workspace as for
 * gdn_prefill_split.  With prologue = 0 it is gdn_prefill_split.
 */
gdn_status gdn_prefill_split_fused(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta,
                                   const float *initial_state, const int32_t *cu_seqlens,
                                   int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                                   int32_t Dk, int32_t Dv, int32_t chunk_size, gdn_dtype io_dtype,
                                   uint32_t prologue, void *workspace, size_t workspace_bytes,
                                   void *o, float *final_state, void *stream);

/*
 * gdn_prefill_seg -- gdn_prefill_split with each sequence's state recurrence split into
 * `segments` runs of whole chunks that execute at the same time: the Chunk-Seg-Seg
 * mapping ("Empowering Hybrid Attention Models on NPUs", section 4, Figure 7), in which
 * extra pre-computation lets the Reduce run over segments concurrently.  The chunk state
 * map is affine (S -> S M + B), so each later segment runs twice side by side, from a zero
 * state and from the identity, and two more launches join them: the start state of
 * segment s + 1 is S_in(s) X_s + S0(s), with X_s the segment's product of M, and its
 * outputs gain E S_in(s)^T.  Same results as gdn_prefill_split up to rounding
 * (bit-identical with segments = 1); the faster one when few (sequence, head) pairs leave
 * compute units idle during the recurrence, since the serial chain shortens by the factor
 * `segments` at 2 segments - 1 times the recurrence's workgroups.  Arguments as for
 * gdn_prefill_split, plus:
 *
 *   segments       1 .. 256 segments per sequence (chunks [s nc / segments,
 *                  (s + 1) nc / segments) of a sequence of nc chunks form segment s; a
 *                  segment may be empty)
 *   workspace      at least gdn_prefill_seg_workspace_size(...) bytes, with the same
 *                  rules as gdn_prefill_split's
 *
 * gdn_prefill_seg_workspace_size -- gdn_prefill_split_workspace_size plus two fp16
 * [T_tot, Hv, Dv] output buffers and, per (sequence, head, segment), two fp32 and one
 * fp16 Dk x Dk states.
 *
 * gdn_prefill_seg_choose -- a segment count for these sizes on the current device: the
 * largest with one recurrence workgroup per compute unit, N * Hv * W * (2 segments - 1)
 * <= compute units, where W is the recurrence's workgroups per (sequence, head): 4 (32
 * value channels each) for chunk_size 32 or 64, 8 for 128; and at least 4 chunks per
 * segment on average; 1 means "use gdn_prefill_split".  Reads the device's compute-unit count (GDN_ERR_DEVICE if that
 * fails).  Host pointer `segments`.
 */
gdn_status gdn_prefill_seg_workspace_size(int32_t N, int32_t T_tot, int32_t Hv,
                                          int32_t chunk_size, int32_t segments, size_t *bytes);
gdn_status gdn_prefill_seg_choose(int32_t N, int32_t T_tot, int32_t Hv, int32_t chunk_size,
                                  int32_t *segments);
gdn_status gdn_prefill_seg(const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           const float *initial_state, const int32_t *cu_seqlens,
                           int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                           int32_t Dk, int32_t Dv, int32_t chunk_size, int32_t segments,
                           gdn_dtype io_dtype, void *workspace, size_t workspace_bytes,
                           void *o, float *final_state, void *stream);

/*
 * gdn_kda_prefill_seg -- gdn_kda_prefill with each sequence's recurrence run as
 * `segments` concurrent segments, as gdn_prefill_seg does for the scalar gate (the chunk
 * state map with a per-key-channel decay is affine too, S -> S (Diag(gl) - W^T Kl) +
 * U^T Kl).  Arguments as for gdn_kda_prefill plus `segments`; chunk_size 64; workspace at
 * least gdn_prefill_seg_workspace_size(N, T_tot, Hv, 64, segments) bytes.
 */
gdn_status gdn_kda_prefill_seg(const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                               int32_t Dk, int32_t Dv, int32_t chunk_size, int32_t segments,
                               gdn_dtype io_dtype, void *workspace, size_t workspace_bytes,
                               void *o, float *final_state, void *stream);

/*
 * gdn_prefill_plan -- the launch shape gdn_prefill would use for these sizes,
 * without launching anything: the width of the value-channel slice each workgroup
 * owns (the column-wise split of S, "Empowering Hybrid Attention Models on NPUs",
 * section 4, Figure 8(b)), the number of workgroups, the LDS bytes and the threads
 * per workgroup.  Any output pointer may be NULL.  Host pointers.
 */
gdn_status gdn_prefill_plan(int32_t N, int32_t Hv, int32_t Dv, gdn_dtype io_dtype,
                            int32_t *dv_per_workgroup, int32_t *workgroups,
                            int32_t *lds_bytes, int32_t *threads_per_workgroup);

/*
 * gdn_prefill_auto_plan / gdn_prefill_auto -- the prefill (with the input prologue when
 * `prologue` is nonzero) through whichever of this library's prefill paths is fastest
 * for these sizes on the current device, with 64-token chunks: the one-launch kernel of
 * gdn_prefill / gdn_prefill_fused, the two launches of gdn_prefill_split /
 * gdn_prefill_split_fused, or the segmented gdn_prefill_seg ("Empowering Hybrid
 * Attention Models on NPUs", section 4: the Chunk-Seg-Seg mapping for few heads and long
 * sequences).  Same results as gdn_prefill up to rounding.
 *
 * gdn_prefill_auto_plan reads the device's compute-unit count and returns, through the
 * non-NULL pointers, the path (gdn_prefill_path), the segment count (1 unless
 * GDN_PATH_SEG) and the workspace bytes gdn_prefill_auto needs for these sizes (0 for
 * GDN_PATH_ONE_LAUNCH; workspace_bytes must be non-NULL).  fp32 I/O always takes the
 * one-launch path; 16-bit I/O takes a two-launch path when their chain's N * Hv * 4
 * workgroups (two 16-channel slices each, 64-token chunks) fit the compute units in one
 * round, or when N > 1, and the segmented one when gdn_prefill_seg_choose gives at least
 * three segments and prologue is 0.
 *
 * gdn_prefill_auto takes gdn_prefill_fused's arguments (chunk_size is 64) plus a
 * caller-owned workspace of at least the planned bytes on the same device (256-byte
 * aligned, overlapping no other argument, not shared by two calls in flight; NULL when
 * the plan needs none); it plans again and runs the chosen entry point, which checks its
 * arguments and returns their statuses.
 */
typedef enum gdn_prefill_path {
    GDN_PATH_ONE_LAUNCH = 0,   /* gdn_prefill / gdn_prefill_fused          */
    GDN_PATH_SPLIT = 1,        /* gdn_prefill_split / gdn_prefill_split_fused */
    GDN_PATH_SEG = 2           /* gdn_prefill_seg                          */
} gdn_prefill_path;
gdn_status gdn_prefill_auto_plan(int32_t N, int32_t T_tot, int32_t Hv, gdn_dtype io_dtype,
                                 uint32_t prologue, int32_t *path, int32_t *segments,
                                 size_t *workspace_bytes);
gdn_status gdn_prefill_auto(const void *q, const void *k, const void *v,
                            const float *g, const float *beta,
                            const float *initial_state, const int32_t *cu_seqlens,
                            int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv,
                            int32_t Dk, int32_t Dv, gdn_dtype io_dtype, uint32_t prologue,
                            void *workspace, size_t workspace_bytes,
                            void *o, float *final_state, void *stream);

/* Static English name of a status code. */
const char *gdn_status_string(gdn_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_MI355X_GDN_H */
