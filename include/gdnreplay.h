/*
 * gdnreplay.h - C ABI of libgdnreplay: Gated DeltaNet span replay on AMD
 * Instinct MI355X (gfx950).
 *
 * Sources (cited by title and section):
 *   [TR]  "Tail-Replay: Escaping the Curse of Linear Attention in Prefix
 *         Caching for Hybrid LLMs" (notes page on arXiv 2608.30310v2).
 *   [SPC] "Sparse prefix caching for hybrid and recurrent LLM serving"
 *         (arXiv 2605.05219).
 *
 * The operation ([TR] §2.3, eq. (1)).  Per (request, head) a state S of
 * d_v x d_k float32 values (row-major, d_k contiguous) is carried through the
 * tokens of a span.  The key operator acts from the right, which is the only
 * reading that type-checks for a rectangular state ([TR] §2.3):
 *     S_i = alpha_i S_{i-1} (I - beta_i k_i k_i^T) + beta_i v_i k_i^T
 *         = alpha_i S_{i-1} + beta_i (v_i - alpha_i S_{i-1} k_i) k_i^T,
 * and every token of the span produces o_i = S_i q_i from the updated state.
 * With GDN_NORMALIZE_K (GDN_NORMALIZE_Q) each key (query) is first divided by
 * its L2 norm, computed in float32; a zero vector stays zero.
 *
 * Packed token layout, shared by every call (element types per gdn_dtype):
 *   q, k   [rows][H][d_k]      v, o   [rows][H][d_v]      alpha, beta  [rows][H]
 * Request b owns rows tok_offset[b] .. tok_offset[b+1]-1; row tok_offset[b]
 * holds the token at 1-based position first_pos[b] of that request
 * (first_pos == NULL means 1 for every request), so a caller may store a whole
 * prefix or only the rows a span needs.  A "position" c counts tokens: the
 * state "at c" is the state after the c-th token.
 * States: state_out [B][H][d_v][d_k] float32; checkpoint stores
 * [B][M][H][d_v][d_k] float32.
 *
 * Conventions for all entry points:
 *  - Device pointers (q, k, v, alpha, beta, o, state_out, ckpt_states) must
 *    be device memory of the current HIP device; arguments prefixed h_ are
 *    host arrays, read during the call only.  q, k, v, alpha, beta and o must
 *    be aligned to their element size and the float32 state buffers to 16
 *    bytes (GDN_ERR_INVALID_ARGUMENT otherwise).  The chunked kernel also
 *    needs 16-byte aligned q, k, v and o; a call whose rows are not runs on
 *    the per-token kernel instead (GDN_ERR_UNSUPPORTED under
 *    GDN_KERNEL_CHUNKED).  The caller owns every buffer.
 *    The library allocates nothing, keeps no device state beyond its code
 *    object and never synchronises: work is queued on `stream` (NULL = the
 *    null stream) and results are ready when that stream has drained.
 *  - Only the rows of a span are read from q, k, v, alpha, beta; o is written
 *    on the rows of the span only (other rows are left untouched); o == NULL
 *    skips the outputs (q may then be NULL).  Neither o nor a state written
 *    by the call may share memory with the rows of q, k, v, alpha or beta
 *    between the first and the last span row (GDN_ERR_INVALID_ARGUMENT).
 *  - Thread-safe: calls keep no shared mutable state (the error text is
 *    thread-local).
 *  - Errors: GDN_ERR_INVALID_ARGUMENT / GDN_ERR_UNSUPPORTED are detected on the
 *    host before anything is queued; GDN_ERR_HIP reports a failed launch.  In
 *    every error case gdn_last_error() describes it.  A fault inside a kernel
 *    surfaces at the caller's synchronisation of `stream`.
 */
#ifndef GDNREPLAY_H
#define GDNREPLAY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1,
    GDN_ERR_UNSUPPORTED = 2,
    GDN_ERR_HIP = 3
} gdn_status;

/* Element type of q, k, v, alpha, beta and o.  States are always float32. */
typedef enum gdn_dtype { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 } gdn_dtype;

/* gdn_shape.flags */
#define GDN_NORMALIZE_K 1u        /* divide each key by its L2 norm before use   */
#define GDN_NORMALIZE_Q 2u        /* divide each query by its L2 norm before use */
#define GDN_KERNEL_RECURRENT 256u /* force the per-token float32 kernel          */
#define GDN_KERNEL_CHUNKED 512u   /* require the chunked matrix-core kernel (bf16, d_k = d_v = 128, GDN_NORMALIZE_K) */

/* Largest number of checkpoint positions per request (emission and resume). */
#define GDN_MAX_CHECKPOINTS 192

typedef struct gdn_shape {
    int32_t B;      /* requests, >= 0                                  */
    int32_t H;      /* heads, >= 1                                     */
    int32_t dk;     /* key width: 16, 32, 64 or 128                    */
    int32_t dv;     /* value width: 16, 32, 64 or 128                  */
    int32_t dtype;  /* gdn_dtype                                       */
    uint32_t flags; /* GDN_NORMALIZE_K | GDN_NORMALIZE_Q | GDN_KERNEL_* */
} gdn_shape;

/* Library version string, e.g. "libgdnreplay 0.1.0 gfx950". */
const char *gdn_version(void);

/* Text of the last error reported on this thread ("" if none). */
const char *gdn_last_error(void);

/*
 * Which kernel the entry points would run for this shape (with 16-byte
 * aligned q, k, v and o): 0 = the per-token float32 kernel, 1 = the chunked
 * matrix-core kernel, -1 = the shape (or a GDN_KERNEL_* request in its flags)
 * is not supported.  Host only.
 */
int32_t gdn_kernel_for(const gdn_shape *shape);

/*
 * Tail length k = ceil(r m) with r = r_num / r_den, in exact integer
 * arithmetic, capped at m ([TR] §2.1 symbol table; §2.2: m = 10000 and r = 5%
 * replay positions 9501..10000).  Returns -1 if m < 0, r_num < 0 or r_den <= 0.
 * Host only.
 */
int64_t gdn_tail_len(int64_t m, int64_t r_num, int64_t r_den);

/*
 * Deepest checkpoint at or before depth ([SPC] §3): returns the 1-based index
 * j of the largest pos[j-1] <= depth, or 0 when none qualifies (recompute from
 * the zero state, the implicit c_0 = 0).  pos must hold M strictly increasing
 * positions >= 1.  Returns -1 if pos is NULL with M > 0, M < 0, depth < 0 or
 * pos is not strictly increasing.  Host only.
 */
int32_t gdn_select_checkpoint(const int64_t *pos, int32_t M, int64_t depth);

/*
 * Zero-start tail replay ([TR] §2.2): for each request b, k_b = ceil(r m_b)
 * and the state is rebuilt from zero over positions m_b - k_b + 1 .. m_b.
 *   h_m        host [B], m_b >= 0 (m_b = 0 gives k_b = 0 and a zero state)
 *   r_num/r_den  replay ratio r, r_num >= 0, r_den > 0
 *   state_out  device [B][H][d_v][d_k] float32: the replayed state at m_b
 *   o          device, nullable: outputs on the replayed rows
 *   h_k_out    host [B], nullable: receives k_b
 * The rows of positions m_b - k_b + 1 .. m_b must be stored.
 */
gdn_status gdn_tail_replay(const gdn_shape *shape,
                           const void *q, const void *k, const void *v,
                           const void *alpha, const void *beta,
                           const int64_t *h_tok_offset, const int64_t *h_first_pos,
                           const int64_t *h_m, int64_t r_num, int64_t r_den,
                           float *state_out, void *o, int64_t *h_k_out,
                           hipStream_t stream);

/*
 * Tail replay of a group of L linear-attention layers ([TR] §2.2 step 3: the
 * tail passes through the group's layers in turn; §2.3: each later layer takes
 * the earlier layer's outputs), under identity mixing: layer l + 1 (l >= 0)
 * takes layer l's bf16 / fp32 outputs on the replayed rows as its q = k = v.  Every layer
 * replays the same span k_b = ceil(r m_b) from zero.  Results are, bit for bit,
 * those of L calls of gdn_tail_replay chained that way.  Where that sequence
 * would run the chunked kernel with more workgroups than CUs on every layer, all
 * layers of a launch's requests run in one launch, each workgroup taking its
 * (request, head) through the layers in turn.  Otherwise the layers are
 * launched one after the other.
 *   L          1..4 layers; needs d_k = d_v
 *   q, k, v    layer 0's inputs (as for gdn_tail_replay; q non-NULL)
 *   alpha, beta  host arrays of L device pointers: each layer's gates, laid
 *              out like the inputs
 *   state_out  device [L][B][H][d_v][d_k] float32: each layer's state at m_b
 *   o          device [L][rows][H][d_v] (rows = h_tok_offset[B], the inputs'
 *              element type): each layer's outputs on the replayed rows (other
 *              rows are not written); must not overlap state_out
 *   h_k_out    host [B], nullable: receives k_b
 * Errors: those of gdn_tail_replay; GDN_ERR_INVALID_ARGUMENT for L outside
 * 1..4, NULL alpha / beta arrays, a NULL o or state_out, or o overlapping
 * state_out; GDN_ERR_UNSUPPORTED for d_k != d_v.  All layers are checked
 * before any launch.
 */
gdn_status gdn_tail_replay_group(const gdn_shape *shape, int32_t L,
                                 const void *q, const void *k, const void *v,
                                 const void *const *alpha, const void *const *beta,
                                 const int64_t *h_tok_offset, const int64_t *h_first_pos,
                                 const int64_t *h_m, int64_t r_num, int64_t r_den,
                                 float *state_out, void *o, int64_t *h_k_out,
                                 hipStream_t stream);

/*
 * Tail replay overlapped with the host-to-device transfer of the attention
 * layers' KV cache ([TR] §2.5, "transfer and replay overlap": the replay needs
 * only the tail inputs, so the KV copy and the replay run on separate streams
 * and join before the new suffix is processed).  In this order it queues
 *   1. hipMemcpyAsync(kv_dst, kv_src, kv_bytes, host to device) on copy_stream
 *      (skipped when kv_bytes = 0), then hipEventRecord(copy_done, copy_stream);
 *   2. the replay of gdn_tail_replay (same arguments, same results) on stream;
 *   3. hipStreamWaitEvent(stream, copy_done): later work on `stream` sees both.
 * kv_src should be pinned host memory (hipHostMalloc) for the copy to run
 * asynchronously; kv_dst is device memory of kv_bytes; copy_done is an event
 * created by the caller (the library creates and keeps none).  The streams
 * should be distinct for the two to overlap.  Errors: those of gdn_tail_replay,
 * GDN_ERR_INVALID_ARGUMENT for a NULL copy_done or a NULL kv_dst / kv_src with
 * kv_bytes > 0; every argument of both the replay and the copy is checked
 * before step 1, so none of these queues anything.  GDN_ERR_HIP when a
 * runtime call fails (earlier steps may have been queued).
 */
typedef struct ihipEvent_t *hipEvent_t;
gdn_status gdn_tail_replay_with_h2d(const gdn_shape *shape,
                                    const void *q, const void *k, const void *v,
                                    const void *alpha, const void *beta,
                                    const int64_t *h_tok_offset, const int64_t *h_first_pos,
                                    const int64_t *h_m, int64_t r_num, int64_t r_den,
                                    float *state_out, void *o, int64_t *h_k_out,
                                    void *kv_dst, const void *kv_src, size_t kv_bytes,
                                    hipStream_t stream, hipStream_t copy_stream,
                                    hipEvent_t copy_done);

/*
 * Resume from a sparse checkpoint ([SPC] §3): for each request b,
 * j_b = gdn_select_checkpoint(h_ckpt_pos + b*M, M, h_depth[b]); the scan
 * starts from ckpt_states[b][j_b - 1] (or from zero when j_b = 0) and
 * recomputes positions c_{j_b} + 1 .. depth_b.  A depth equal to a checkpoint
 * copies that state bit-for-bit; depth 0 gives the zero state.
 *   h_ckpt_pos   host [B][M], strictly increasing per request, >= 1
 *   ckpt_states  device [B][M][H][d_v][d_k] float32 (read only); may be NULL
 *                if no request selects a checkpoint
 *   h_depth      host [B], >= 0
 *   state_out    device [B][H][d_v][d_k]: the state at depth_b.  It may alias
 *                the selected slot ckpt_states[b][j_b - 1] exactly.
 *   h_j_out      host [B], nullable: receives j_b
 * The rows of positions c_{j_b} + 1 .. depth_b must be stored.
 */
gdn_status gdn_resume(const gdn_shape *shape,
                      const void *q, const void *k, const void *v,
                      const void *alpha, const void *beta,
                      const int64_t *h_tok_offset, const int64_t *h_first_pos,
                      const int64_t *h_ckpt_pos, int32_t M, const float *ckpt_states,
                      const int64_t *h_depth, float *state_out, void *o,
                      int32_t *h_j_out, hipStream_t stream);

/*
 * Full prefill with checkpoint emission ([SPC] §3: a state is kept at every
 * checkpoint position): for each request b the scan runs from the zero state over all its
 * N_b = tok_offset[b+1] - tok_offset[b] rows (first_pos must be NULL or 1) and
 * writes the state after position h_ckpt_pos[b][i] to ckpt_states[b][i].
 *   h_ckpt_pos   host [B][M], strictly increasing per request, in [1, N_b]
 *   ckpt_states  device [B][M][H][d_v][d_k] float32 (written); may be NULL if M = 0
 *   state_out    device [B][H][d_v][d_k]: the state at N_b
 */
gdn_status gdn_prefill_emit_checkpoints(const gdn_shape *shape,
                                        const void *q, const void *k, const void *v,
                                        const void *alpha, const void *beta,
                                        const int64_t *h_tok_offset,
                                        const int64_t *h_first_pos,
                                        const int64_t *h_ckpt_pos, int32_t M,
                                        float *ckpt_states, float *state_out, void *o,
                                        hipStream_t stream);

/*
 * Workspace bytes of gdn_prefill_emit_checkpoints_split for this shape:
 * 4 B H d_v d_k float32 values (0 for an invalid shape).  Host only.
 */
size_t gdn_prefill_split_workspace_bytes(const gdn_shape *shape);

/*
 * The same prefill with emission as gdn_prefill_emit_checkpoints (same
 * arguments and results, up to rounding), for batches with few (request,
 * head) pairs: each span of at least 768 tokens is cut into three segments
 * (boundaries floor(N/3) and floor(2N/3), rounded down to a multiple of 32)
 * so that three times as many workgroups share the GPU.  It uses the exact
 * split of [TR] §2.3: the state after a segment is S_start P + S^, with P the
 * product of the segment's transitions and S^ its zero-start replay.
 *   1. segment 0 runs from zero with its outputs and emissions, while the
 *      zero-start replay S^_1 and the product P_1 of segment 1 are formed (P_1
 *      is the scan of segment 1 with v = 0 started from the identity);
 *   2. S_start(2) = S_end(0) P_1 + S^_1 (float32);
 *   3. segments 1 and 2 run from their start states with their outputs and
 *      emissions.
 * Shorter spans run in one pass in step 1.  Needs d_k = d_v.
 *   workspace  device, >= gdn_prefill_split_workspace_bytes(shape) bytes,
 *              owned by the caller, overwritten; must not overlap state_out
 *              or ckpt_states.
 * Errors: those of gdn_prefill_emit_checkpoints; GDN_ERR_UNSUPPORTED for
 * d_k != d_v; GDN_ERR_INVALID_ARGUMENT for a NULL, small or overlapping
 * workspace.  Nothing is queued when an error is returned before step 1.
 */
gdn_status gdn_prefill_emit_checkpoints_split(const gdn_shape *shape,
                                              const void *q, const void *k, const void *v,
                                              const void *alpha, const void *beta,
                                              const int64_t *h_tok_offset,
                                              const int64_t *h_first_pos,
                                              const int64_t *h_ckpt_pos, int32_t M,
                                              float *ckpt_states, float *state_out, void *o,
                                              void *workspace, size_t workspace_bytes,
                                              hipStream_t stream);

/* Scratch bytes behind gdn_prefill_emit_checkpoints_split_noalloc, per GPU. */
#define GDN_SPLIT_SCRATCH_BYTES (32u << 20)

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * split prefill as gdn_prefill_emit_checkpoints_split (same arguments except
 * the workspace, same kernels, same results bit for bit), with its workspace
 * taken from a fixed array of GDN_SPLIT_SCRATCH_BYTES (32 MiB) in the
 * library's code object instead of from the caller.
 *  - Limit: gdn_prefill_split_workspace_bytes(shape) = 4 B H d_v d_k floats
 *    must not exceed GDN_SPLIT_SCRATCH_BYTES (B H <= 128 at d_k = d_v = 128),
 *    else GDN_ERR_UNSUPPORTED and nothing is queued.
 *  - Each GPU the library runs on holds its own copy of the array until the
 *    process ends; the first call on a device looks up its address
 *    (hipGetSymbolAddress, no allocation).  Nothing here calls hipMalloc,
 *    hipFree or an allocating routine.
 *  - Every call on a GPU shares that GPU's array and leaves its contents
 *    behind; nothing in it has to start at zero (every value read was written
 *    earlier in the same call).  Calls that overlap on one GPU (other streams,
 *    other threads) race on the array: the caller must order them, e.g. on
 *    one stream.
 * Errors: those of gdn_prefill_emit_checkpoints_split (except the workspace
 * ones); GDN_ERR_HIP if the array's address cannot be taken.
 */
gdn_status gdn_prefill_emit_checkpoints_split_noalloc(const gdn_shape *shape,
                                                      const void *q, const void *k, const void *v,
                                                      const void *alpha, const void *beta,
                                                      const int64_t *h_tok_offset,
                                                      const int64_t *h_first_pos,
                                                      const int64_t *h_ckpt_pos, int32_t M,
                                                      float *ckpt_states, float *state_out, void *o,
                                                      hipStream_t stream);

/*
 * Checkpoint placement ([SPC] §3 problem statement, §4 Theorems 1 and 2).
 * Host only, double precision, no device work.  A depth distribution p is an
 * array of N + 1 non-negative finite weights p[0..N] (p[0] is the weight of
 * a miss, d = 0; p need not sum to one).  Positions are M strictly increasing
 * integers in [1, N]; the implicit c_0 = 0 is the zero state.
 */

/*
 * Expected recomputation R(p, C) = sum_{d=0}^{N} p[d] (d - max({0} u {c_i <= d}))
 * ([SPC] §3, the gap form R(p, g) with c_i the partial sums of g).  Returns
 * -1.0 if p is NULL, N < 0, M < 0, pos is NULL with M > 0, a weight is negative
 * or not finite, or the positions are not strictly increasing in [1, N].
 */
double gdn_expected_recompute(const double *p, int64_t N, const int64_t *pos, int32_t M);

/*
 * Balanced placement ([SPC] §4 Theorem 1: optimal for p uniform on 1..N):
 * pos_out[i-1] = floor(i (N + 1) / (M + 1)), i = 1..M, so the M + 1 gaps
 * (summing to N + 1) differ by at most one.  pos_out: host [M].  Returns 0, or
 * -1 if N < 0, M < 0, M > N or pos_out is NULL with M > 0.
 */
int32_t gdn_balanced_checkpoints(int64_t N, int32_t M, int64_t *pos_out);

/*
 * Optimal placement for any p ([SPC] §4 Theorem 2): M positions minimising
 * R(p, C), by the dynamic programme over the last checkpoint with the convex
 * hull trick, O(N M) time and 4 M (N + 2) bytes of host memory (allocated and
 * freed inside the call).  Where several placements reach the minimum any one
 * of them is returned.
 *   p         host [N + 1]
 *   pos_out   host [M] (written), strictly increasing in [1, N]
 *   cost_out  host, nullable: receives the minimal R(p, C)
 * Errors: GDN_ERR_INVALID_ARGUMENT for a NULL p or pos_out (M > 0), N < 1,
 * M outside 0..N, or a negative or non-finite weight; GDN_ERR_UNSUPPORTED
 * when N + 2 or M (N + 2) exceeds 2^28.
 */
gdn_status gdn_plan_checkpoints(const double *p, int64_t N, int32_t M, int64_t *pos_out,
                                double *cost_out);

#ifdef __cplusplus
}
#endif

#endif /* GDNREPLAY_H */
