/*
 * sb.h -- C ABI of libsb: source projection of a vocab-sharded output head
 * on one AMD Instinct MI355X (gfx950).
 *
 * The head computes logits z = X . W for hidden rows X [B, H] (bf16) and a
 * head weight W [H, V] (bf16) whose vocabulary is split into k contiguous
 * lanes, lane i holding vocab columns [off_i, off_{i+1}).  Three result
 * surfaces are offered, following the SemBridge paper ("SemBridge: Compiling
 * Consumer Observations into Cross-Stack Communication Plans"):
 *
 *  - token-only (sb_project_tokens): section 2.3 and section 5.2 -- a
 *    deterministic token request applies the sampler (argmax) at the source
 *    and ships int32 token IDs; section 6 / Figure 1 -- one result per lane
 *    ("argmax x k"), and all plans deliver the same token ID;
 *  - log-probability (sb_project_logprobs): section 3.2 / 3.4 -- the surface
 *    keeps the complete logits plus token IDs; here the logsumexp per row, the
 *    selected-token log-probability and, on request, the complete fp32
 *    log-probabilities;
 *  - full-logit plan (sb_full_logits): section 5.2 / section 6 -- the logits
 *    are sliced by lane, the shards reconstructed into the complete tensor
 *    (the destination-local AllGather, here a device-local copy), then argmax.
 *
 * Semantics common to every call
 *  - Token IDs are int32 GLOBAL vocabulary indices.  The registered projection
 *    is greedy argmax over the fp32 logits; among equal maxima the LOWEST
 *    global index wins (section 3.1: a projection operator declares
 *    deterministic tie-breaking).
 *  - Logits are fp32 sums of exact bf16 x bf16 products.  The order in which
 *    each logit is accumulated depends only on (B, H, V), never on the
 *    surface, the lane split or the column position, so the three calls
 *    return bit-identical logits and IDs for the same inputs.
 *  - lse is an online sum over 128-column tiles.  A lane's tile grid starts on
 *    the cache line that holds the lane's first column, so lse (and sel_lp and
 *    the complete log-probs) can differ in the last bits between shard
 *    placements that differ modulo 128 bytes; for the same placement it is
 *    reproduced exactly.
 *  - Non-finite values: the argmax puts a NaN above every number (all NaNs
 *    equal, so the lowest-index NaN wins, as numpy's and torch's argmax do)
 *    and +inf above every finite value, so every ID, and every lane's ID, is
 *    one of the row's columns whatever the inputs.  NaN and infinities in x
 *    or w reach the fp32 logits by IEEE rules (NaN * anything and 0 * inf
 *    give NaN).  lse, sel_lp and the complete log-probs of a row holding a
 *    NaN or +inf logit are NaN; of a row of -inf only, unspecified.  Finite
 *    inputs whose sums overflow fp32 are outside the contract
 *    (|logit| < FLT_MAX).
 *
 * Ownership and threading
 *  - The caller allocates every device buffer.  The library allocates no
 *    device memory and is thread-safe.  The only things it keeps between
 *    calls are a per-device note of the kernels whose LDS limit it has
 *    raised (hipFuncSetAttribute, once per device and kernel) and, for
 *    sb_project_tokens_static, each device's address of its static array.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream).  Inputs are read-only.  Every device pointer of a
 *    call must be memory the stream's device can access (its own, or a
 *    peer's with peer access enabled); the library does not check this, as
 *    a per-call pointer query would cost more than a decode call's launch.
 *    Outputs must not overlap inputs, the workspace or each other.
 *  - The workspace is scratch owned by the call until its work completes on
 *    the stream: its contents on entry do not matter, and nothing in it is
 *    valid afterwards.  Every workspace starts with the same fixed region
 *    (8,192 bytes) of per-tile counters for heads split into K slices (see
 *    below); a call on a split head clears the counters it uses on `stream`
 *    before its head kernel runs (by a small clearing launch, or by the
 *    hidden-row copy for 33 <= B <= 64), so a workspace sized for the
 *    largest call serves calls of any shape, surface or entry point in any
 *    order.  Two calls that use one workspace at the same time (on different
 *    streams without ordering) race and give undefined results.
 *  - A head of fewer than 128 vocabulary tiles of 128 columns (B <= 64) splits
 *    each tile's hidden sum into up to 8 slices that run as separate
 *    workgroups, and one of 257 to 352 tiles (B <= 16, H >= 4065) into 2;
 *    the slice partials are added in slice order.  The split depends on
 *    (B, H, V) only, so the guarantees above still hold.
 *
 * Errors
 *  - Validation is synchronous: on any error status nothing is enqueued and
 *    no output is touched (missing facts select no silent fallback; section
 *    3.4's rule that an unavailable fact selects the materialising plan is
 *    left to the caller, who may call sb_full_logits).
 *  - SB_ERR_HIP reports a failed kernel launch (hipGetLastError); work may
 *    then be partially enqueued.
 */
#ifndef SB_H
#define SB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sb_status {
    SB_OK = 0,
    SB_ERR_NULL = -1,        /* a required pointer is NULL                     */
    SB_ERR_SHAPE = -2,       /* B < 0, H < 0, V < 1, or a leading dim too small */
    SB_ERR_LANES = -3,       /* k < 1, k > SB_MAX_LANES, or lane offsets not
                                strictly increasing from 0 to V               */
    SB_ERR_ALIGN = -4,       /* x, w[i], an fp32 output or the workspace not
                                16-byte aligned; ldx, ldw not multiples of 8;
                                a logits / log-probs leading dim not a
                                multiple of 4                                  */
    SB_ERR_WORKSPACE = -5,   /* workspace smaller than sb_workspace_bytes()   */
    SB_ERR_UNSUPPORTED = -6, /* V > 2^30; or 40 shard rows or 64 rows of x
                                span 4 GiB or more; or, for 65 <= B <= 128,
                                128 rows of x
                                do; or, for B >= 129, 72 shard rows or 256
                                rows of x do; or a launch of the call would
                                need 2^32 work items or more in one grid
                                dimension (B >= 2^24 always does; for
                                B >= 129 roughly B * V >= 5.5e11)          */
    SB_ERR_HIP = -7,         /* a HIP launch failed                            */
    /* not a status: widens the enumeration to every 32-bit int, so that
       sb_status_string() may be given any value a caller holds */
    SB_STATUS_RANGE_MAX_ = 0x7FFFFFFF
} sb_status;

#define SB_MAX_LANES 64

/* Result surfaces, used to size the workspace. */
typedef enum sb_surface {
    SB_SURF_TOKENS = 0,         /* sb_project_tokens                          */
    SB_SURF_LOGPROBS = 1,       /* sb_project_logprobs, logprobs == NULL      */
    SB_SURF_LOGPROBS_FULL = 2,  /* sb_project_logprobs, logprobs != NULL      */
    SB_SURF_FULL_LOGITS = 3     /* sb_full_logits (includes the lane shards)  */
} sb_surface;

/*
 * The head.  All shapes in elements.
 *   B        rows (decode batch / prefill tokens); B == 0 is a valid no-op
 *   H        hidden size (K of the product); H == 0 gives all-zero logits
 *   V        vocabulary size, >= 1
 *   k        number of vocab lanes, 1..SB_MAX_LANES
 *   lane_off HOST array of k+1 int32: 0 = off_0 < off_1 < ... < off_k = V
 *   x        DEVICE pointer, bf16 [B][ldx] row-major, 16-byte aligned
 *   ldx      row stride of x, >= H, multiple of 8
 *   w        HOST array of k DEVICE pointers; w[i] is lane i's shard, bf16
 *            [H][ldw] row-major, column j of the shard = vocab column
 *            off_i + j; 16-byte aligned.  A single [H][V] allocation is
 *            passed as w[i] = base + off_i with ldw = V (then every off_i
 *            must be a multiple of 8).
 *   ldw      row stride of every shard, >= max_i (off_{i+1} - off_i),
 *            multiple of 8
 */
typedef struct sb_head_desc {
    int32_t B, H, V, k;
    const int32_t *lane_off;
    const void *x;
    int64_t ldx;
    const void *const *w;
    int64_t ldw;
} sb_head_desc;

/*
 * Bytes of device workspace a call on `desc` with the given surface needs
 * (0 if none).  Returns 0 and sets *status (if not NULL) to an error code when
 * the descriptor is invalid.  Host-only; enqueues nothing.
 */
size_t sb_workspace_bytes(const sb_head_desc *desc, int surface, sb_status *status);

/*
 * Token-only surface (source projection, SemBridge section 5.2 / section 6):
 * ids[b] = lowest global index of max_v z[b][v].  Each lane reduces to one
 * (max, lowest-index) result per row inside the GEMM epilogue; the per-lane
 * results are combined in ascending lane order.  The full logits are never
 * written to memory.  Launches: the head kernel, which writes one (max,
 * lowest index) pair per (row, 128-column tile) into the workspace, then a
 * combine kernel (one workgroup per row) that folds them, lane by lane; for
 * 33 <= B <= 64 the head kernel is preceded by a copy of x into the
 * workspace in fragment order, and a head split into K slices by the
 * clearing of its slice counters (done by that copy where there is one).
 *   ids  DEVICE int32 [B]
 *   ws   DEVICE workspace of >= sb_workspace_bytes(desc, SB_SURF_TOKENS)
 *        bytes, 16-byte aligned
 */
sb_status sb_project_tokens(const sb_head_desc *desc, int32_t *ids,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * sb_project_tokens for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launches and bit-identical ids, with the workspace
 * taken from a static device array inside the library instead of an
 * argument.  The array holds SB_STATIC_SCRATCH_BYTES bytes on every device
 * the library runs on and stays allocated until the process ends; this call
 * allocates nothing.  Its address is looked up once per device, on the first
 * call there.
 *   ids     DEVICE int32 [B]
 *   stream  as for every call; the array used is the one of the stream's
 *           device
 * Returns SB_ERR_WORKSPACE when the call needs more than
 * SB_STATIC_SCRATCH_BYTES of workspace (sb_workspace_bytes(desc,
 * SB_SURF_TOKENS); for example B = 2048 rows at V = 151936 need about 20 MB).
 * Every call on a device shares that device's array and leaves its last
 * contents there: calls on one device whose work overlaps in time (two
 * streams, or two threads, without ordering between them) race and give
 * undefined results.
 */
#define SB_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
sb_status sb_project_tokens_static(const sb_head_desc *desc, int32_t *ids, void *stream);

/*
 * Token surface plus each lane's own result (SemBridge Figure 1 caption and
 * section 5.2: under source projection every lane ships one int32 result per
 * row).  Same launches and same ids as sb_project_tokens; in addition
 *   lane_ids[b][i] = lowest global index of the maximum of z[b][v] over lane
 *                    i's columns (DEVICE int32 [B][k], or NULL)
 *   lane_max[b][i] = that maximum (DEVICE fp32 [B][k], or NULL; -0 is
 *                    reported as +0)
 * ids[b] is lane_ids[b][j] for the first lane j whose lane_max is largest.
 *   ws  >= sb_workspace_bytes(desc, SB_SURF_TOKENS)
 */
sb_status sb_project_lane_results(const sb_head_desc *desc, int32_t *ids,
                                  int32_t *lane_ids, float *lane_max,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * Log-probability surface (SemBridge section 3.2 / 3.4: complete logits plus
 * token IDs), computed with an online per-lane logsumexp:
 *   ids[b]         as sb_project_tokens (bit-identical)
 *   lse[b]         = log sum_v exp(z[b][v])                       (fp32)
 *   sel_lp[b]      = z[b][ids[b]] - lse[b]   (optional, may be NULL)
 *   logprobs[b][v] = z[b][v] - lse[b]        (optional, may be NULL; fp32
 *                    [B][ldlp], ldlp >= V and a multiple of 4, 16-byte
 *                    aligned)
 *   ws  >= sb_workspace_bytes(desc, logprobs ? SB_SURF_LOGPROBS_FULL
 *                                            : SB_SURF_LOGPROBS)
 */
sb_status sb_project_logprobs(const sb_head_desc *desc, int32_t *ids,
                              float *lse, float *sel_lp, float *logprobs,
                              int64_t ldlp, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * Full-logit plan (SemBridge section 5.2 / section 6, the layout-directed
 * baseline): every lane writes its fp32 logit shard [B][V_i] into the
 * workspace, the shards are reconstructed into logits [B][ldl] (the
 * destination-local AllGather, a device-local copy here), then, if ids is not
 * NULL, a row argmax (lowest index on ties) yields the token IDs.
 *   logits DEVICE fp32 [B][ldl], ldl >= V and a multiple of 4, 16-byte aligned
 *   ids    DEVICE int32 [B] or NULL
 *   ws     >= sb_workspace_bytes(desc, SB_SURF_FULL_LOGITS)
 */
sb_status sb_full_logits(const sb_head_desc *desc, float *logits, int64_t ldl,
                         int32_t *ids, void *ws, size_t ws_bytes, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Partial completion (SemBridge section 6.4, Exact Shards and Partial
 * Completion; section 3.6, reduction obligations).  The MLP down projection is
 * row parallel: lane i holds a distinct activation shard X_i [B][K_i] and the
 * matching weight rows W_i [K_i][N], and produces the incomplete full-width
 * partial P_i = X_i . W_i (fp32 sums of exact bf16 x bf16 products).  The
 * registered elementwise operator completes the partials before the output
 * is exposed:  out = op(...op(op(P_0, P_1), P_2)..., P_{k-1})  (ascending
 * lane order).  Each P_i is accumulated in an order fixed by the shapes
 * alone (1024-row chunks summed in a fixed order), so repeated calls give
 * bit-identical outputs.  SB_RED_MIN and SB_RED_MAX propagate NaN (IEEE
 * 754-2019 minimum and maximum, as numpy's and torch's elementwise ones):
 * an output is NaN when any lane's partial there is NaN.
 * ---------------------------------------------------------------------------
 */
typedef enum sb_reduce_op {
    SB_RED_SUM = 0,
    SB_RED_PROD = 1,
    SB_RED_MIN = 2,
    SB_RED_MAX = 3
} sb_reduce_op;

/*
 *   B       rows (tokens); B == 0 is a valid no-op; the chunked GEMM's
 *           launch of about ceil(K_i / 1024) * ceil(N / 128) * ceil(B / 64)
 *           workgroups of 256 work items, summed over lanes, must hold fewer
 *           than 2^32 work items (else SB_ERR_UNSUPPORTED)
 *   N       output width (the model's hidden size), >= 1
 *   k       lanes, 1..SB_MAX_LANES
 *   lane_k  HOST array of k+1 int32 offsets of the reduction dimension:
 *           0 = lane_k[0] < lane_k[1] < ... < lane_k[k]; K_i = lane_k[i+1] -
 *           lane_k[i]
 *   x       HOST array of k DEVICE pointers; x[i] is bf16 [B][ldx], columns
 *           [0, K_i) used; 16-byte aligned
 *   ldx     row stride of every x[i], >= max K_i, multiple of 8
 *   w       HOST array of k DEVICE pointers; w[i] is bf16 [K_i][ldw], columns
 *           [0, N) used; 16-byte aligned
 *   ldw     row stride of every w[i], >= N, multiple of 8
 */
typedef struct sb_partial_desc {
    int32_t B, N, k;
    const int32_t *lane_k;
    const void *const *x;
    int64_t ldx;
    const void *const *w;
    int64_t ldw;
} sb_partial_desc;

/*
 * Bytes of device workspace sb_partial_complete needs on `desc`: the head
 * calls' fixed counter region, which this call leaves untouched, then the
 * fp32 chunk partials.  0 for B == 0.
 * Returns 0 and sets *status on an invalid descriptor (statuses as for the
 * head; SB_ERR_LANES for bad lane_k).
 */
size_t sb_partial_workspace_bytes(const sb_partial_desc *desc, sb_status *status);

/*
 * out[b][n] = op over lanes (ascending) of P_i[b][n].
 *   op   one of sb_reduce_op (anything else: SB_ERR_SHAPE)
 *   out  DEVICE fp32 [B][ldo], ldo >= N and a multiple of 4, 16-byte aligned
 *   ws   >= sb_partial_workspace_bytes(desc) bytes, 16-byte aligned
 * Two kernel launches: the chunked partial GEMM and the lane reduction.
 */
sb_status sb_partial_complete(const sb_partial_desc *desc, int op, float *out, int64_t ldo,
                              void *ws, size_t ws_bytes, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *sb_status_string(sb_status status);

#ifdef __cplusplus
}
#endif

#endif /* SB_H */
