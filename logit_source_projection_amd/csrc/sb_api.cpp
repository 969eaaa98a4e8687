// libsb C ABI: argument validation, workspace layout and kernel dispatch.
//
// Follows the SemBridge paper's rule that preconditions are validated before
// anything is lowered and invalid contracts are rejected (section 3.5, static
// validation): every check here runs on the host before the first launch, so
// an error status means nothing was enqueued.
#include "../../include/sb.h"

#include <stdint.h>
#include <string.h>

#include "kernels.h"

namespace {

constexpr size_t kRegionAlign = 256;
// Column counts and grid sizes over the vocabulary are 32-bit with room for
// a chunk's rounding.
constexpr int32_t kMaxVocab = 1 << 30;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Every workspace starts with the same fixed region: the per-tile counters of
// a head split into K slices.  A call on a split head clears the counters it
// uses before its head kernel runs (a.zero), so the workspace's contents on
// entry never matter.
constexpr size_t kCtrBytes = sbk::kMaxSplitTiles * sizeof(uint32_t);
static_assert(kCtrBytes == 8192, "the size include/sb.h states for the counter region");

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validation of the head descriptor (shapes, lanes, alignment, limits).
sb_status check_desc(const sb_head_desc *d)
{
    if (!d || !d->lane_off || !d->w)
        return SB_ERR_NULL;
    if (d->B < 0 || d->H < 0 || d->V < 1)
        return SB_ERR_SHAPE;
    if (d->k < 1 || d->k > SB_MAX_LANES)
        return SB_ERR_LANES;
    if (d->lane_off[0] != 0 || d->lane_off[d->k] != d->V)
        return SB_ERR_LANES;
    int64_t maxv = 0;
    for (int i = 0; i < d->k; ++i) {
        if (d->lane_off[i + 1] <= d->lane_off[i])
            return SB_ERR_LANES;
        const int64_t vi = (int64_t)d->lane_off[i + 1] - d->lane_off[i];
        if (vi > maxv)
            maxv = vi;
    }
    if (d->B > 0 && d->H > 0) {
        if (!d->x)
            return SB_ERR_NULL;
        for (int i = 0; i < d->k; ++i)
            if (!d->w[i])
                return SB_ERR_NULL;
    }
    if (d->ldx < d->H || d->ldw < maxv)
        return SB_ERR_SHAPE;
    if (d->B > 0 && d->H > 0) {
        if (!aligned16(d->x) || (d->ldx % 8) != 0 || (d->ldw % 8) != 0)
            return SB_ERR_ALIGN;
        for (int i = 0; i < d->k; ++i)
            if (!aligned16(d->w[i]))
                return SB_ERR_ALIGN;
    }
    if (d->V > kMaxVocab)
        return SB_ERR_UNSUPPORTED;
    // Per-step buffer offsets are 32-bit: 40 hidden rows of a shard and one
    // row group of x must span less than 4 GiB; for the large-batch kernel
    // (B >= 65) a K stage of a shard (32 rows up to 128 rows, else 64; plus 8)
    // and one block of x (128 rows up to 128 rows, else 256).
    const int64_t lim = (int64_t)1 << 32;
    if ((int64_t)(sbk::kStepK + 8) * d->ldw * 2 >= lim ||
        (int64_t)(sbk::kRowBlock * sbk::kMaxMB) * d->ldx * 2 >= lim)
        return SB_ERR_UNSUPPORTED;
    if (d->B >= sbk::kLargeBatch &&
        ((int64_t)(sbk::large_step_k(d->B) + 8) * d->ldw * 2 >= lim ||
         (int64_t)sbk::large_block_rows(d->B) * d->ldx * 2 >= lim))
        return SB_ERR_UNSUPPORTED;
    // every launch fits one grid (fewer than 2^32 work items per dimension);
    // among others this bounds B below 2^24, the combine's one workgroup per row
    if (sbk::head_launch_items(d->B, d->H, d->V, d->lane_off, d->k) >= lim)
        return SB_ERR_UNSUPPORTED;
    return SB_OK;
}

int lane_width(const sb_head_desc *d, int i) { return d->lane_off[i + 1] - d->lane_off[i]; }

int shard_ld(int vi) { return (vi + 3) & ~3; }

struct Layout {
    int T = 0;            // tile capacity: row stride of the (row, tile) regions
    int nchunks = 0;      // full-logit argmax chunks per row
    int kslices = 1;      // K slices of the head GEMM (one row group only)
    size_t kctr = 0, kpart = 0, xp = 0, pair = 0, mse = 0;
    size_t shard[SB_MAX_LANES] = {}, partial = 0;
    size_t total = 0;
};

Layout layout(const sb_head_desc *d, int surface)
{
    Layout L;
    // Sized for the largest tile shift, so that the workspace size does not
    // depend on where the shards sit in memory.
    for (int i = 0; i < d->k; ++i)
        L.T += sbk::lane_tiles(lane_width(d, i), sbk::kMaxShift);
    L.nchunks = (d->V + sbk::kArgmaxChunk - 1) / sbk::kArgmaxChunk;
    const size_t B = (size_t)d->B;
    size_t at = 0;
    if (B == 0)
        return L;
    const int rpg = sbk::rows_per_group(d->B);
    const bool lse = surface == SB_SURF_LOGPROBS || surface == SB_SURF_LOGPROBS_FULL;
    L.kctr = 0;
    at = kCtrBytes;
    L.kslices = sbk::k_slices(d->B, d->H, d->V);
    if (L.kslices > 1) {
        // partial tiles of the K slices: T x kslices tiles of rows per group x kTileN fp32
        L.kpart = at;
        at = align_up(at + (size_t)L.T * L.kslices * rpg * sbk::kTileN * sizeof(float),
                      kRegionAlign);
    }
    if (const size_t xpb = sbk::packed_hidden_bytes(d->B, d->H)) {
        // the hidden rows packed per K step (33-64 rows)
        L.xp = at;
        at = align_up(at + xpb, kRegionAlign);
    }
    switch (surface) {
    case SB_SURF_TOKENS:
    case SB_SURF_LOGPROBS:
    case SB_SURF_LOGPROBS_FULL:
        // (row, tile) results, folded by the combine launch
        L.pair = at;
        at = align_up(at + B * L.T * sizeof(int2), kRegionAlign);
        if (lse) {
            L.mse = at;
            at = align_up(at + B * L.T * sizeof(float2), kRegionAlign);
        }
        break;
    case SB_SURF_FULL_LOGITS:
        for (int i = 0; i < d->k; ++i) {
            L.shard[i] = at;
            at = align_up(at + B * (size_t)shard_ld(lane_width(d, i)) * sizeof(float),
                          kRegionAlign);
        }
        L.partial = at;
        at = align_up(at + B * L.nchunks * sizeof(int2), kRegionAlign);
        break;
    default:
        break;
    }
    L.total = at;
    return L;
}

template <typename T>
T *region(void *ws, size_t off)
{
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

void fill_lanes(const sb_head_desc *d, sbk::LaneTable &t)
{
    memset(&t, 0, sizeof t);
    t.k = d->k;
    int tiles = 0;
    for (int i = 0; i < d->k; ++i) {
        t.w[i] = static_cast<const uint16_t *>(d->w[i]);
        t.off[i] = d->lane_off[i];
        t.tile0[i] = tiles;
        // columns between the start of the cache line holding the shard's
        // first column and that column, in whole 16-byte units (at most
        // kMaxShift; a base that is not 16-byte aligned is only accepted
        // when nothing is read from it)
        const uintptr_t line_off = reinterpret_cast<uintptr_t>(d->w[i]) % sbk::kLineBytes;
        t.shift[i] = (int32_t)(line_off / 16 * 8);
        tiles += sbk::lane_tiles(lane_width(d, i), t.shift[i]);
    }
    t.off[d->k] = d->lane_off[d->k];
    t.tile0[d->k] = tiles;
}

void fill_args(const sb_head_desc *d, const Layout &L, sbk::HeadArgs &a)
{
    fill_lanes(d, a.lanes);
    a.x = static_cast<const uint16_t *>(d->x);
    a.ldx = d->ldx;
    a.ldw = d->ldw;
    a.B = d->B;
    a.H = d->H;
    a.V = d->V;
    a.T = L.T;
    a.pair = nullptr;
    a.mse = nullptr;
    a.out = nullptr;
    a.ldo = 0;
    a.kslices = L.kslices;
    a.slice_steps = sbk::slice_steps(d->H, L.kslices);
    a.kpart = nullptr;
    a.kctr = nullptr;
    a.xp = nullptr;
    memset(&a.zero, 0, sizeof a.zero);
}

// The words the head launch needs at zero: the slice counters of a split
// head.  Call after the regions are set.
void set_zero(sbk::HeadArgs &a)
{
    if (a.kctr) {
        a.zero.p[0] = a.kctr;
        a.zero.n[0] = a.lanes.tile0[a.lanes.k];
    }
}

// The K-slice regions of a split head and the packed hidden rows of 33-64
// rows (each a no-op where the call has none).
void set_slices(const Layout &L, void *ws, sbk::HeadArgs &a)
{
    if (L.kslices > 1) {
        a.kpart = region<float>(ws, L.kpart);
        a.kctr = region<uint32_t>(ws, L.kctr);
    }
    if (L.xp)
        a.xp = region<uint16_t>(ws, L.xp);
}

sb_status check_ws(const Layout &L, void *ws, size_t ws_bytes)
{
    if (L.total == 0)
        return SB_OK;
    if (!ws)
        return SB_ERR_NULL;
    if (ws_bytes < L.total)
        return SB_ERR_WORKSPACE;
    if (!aligned16(ws))
        return SB_ERR_ALIGN;
    return SB_OK;
}


// Token surface, optionally with the per-lane results.
sb_status project_tokens(const sb_head_desc *desc, int32_t *ids, int32_t *lane_ids,
                         float *lane_max, void *ws, size_t ws_bytes, void *stream)
{
    sb_status st = check_desc(desc);
    if (st != SB_OK)
        return st;
    if (desc->B == 0)
        return SB_OK;
    if (!ids)
        return SB_ERR_NULL;
    const Layout L = layout(desc, SB_SURF_TOKENS);
    if ((st = check_ws(L, ws, ws_bytes)) != SB_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    sbk::HeadArgs a;
    fill_args(desc, L, a);
    a.pair = region<int2>(ws, L.pair);
    set_slices(L, ws, a);
    set_zero(a);
    const hipError_t e = a.B >= sbk::kLargeBatch ? sbk::launch_head_gemm_large(a, sbk::kEpiPair, s)
                                                  : sbk::launch_head_gemm(a, sbk::kEpiPair, s);
    if (e != hipSuccess ||
        sbk::launch_combine(a.pair, nullptr, a.lanes, a.B, a.T, ids, nullptr, nullptr, lane_ids,
                            lane_max, s) != hipSuccess)
        return SB_ERR_HIP;
    return SB_OK;
}

// ---------------------------------------------------------------------------
// Partial completion
// ---------------------------------------------------------------------------
sb_status check_partial(const sb_partial_desc *d)
{
    if (!d || !d->lane_k || !d->x || !d->w)
        return SB_ERR_NULL;
    if (d->B < 0 || d->N < 1)
        return SB_ERR_SHAPE;
    if (d->k < 1 || d->k > SB_MAX_LANES || d->lane_k[0] != 0)
        return SB_ERR_LANES;
    int64_t maxk = 0;
    for (int i = 0; i < d->k; ++i) {
        if (d->lane_k[i + 1] <= d->lane_k[i])
            return SB_ERR_LANES;
        const int64_t ki = (int64_t)d->lane_k[i + 1] - d->lane_k[i];
        if (ki > maxk)
            maxk = ki;
    }
    if (d->B > 0)
        for (int i = 0; i < d->k; ++i)
            if (!d->x[i] || !d->w[i])
                return SB_ERR_NULL;
    if (d->ldx < maxk || d->ldw < d->N)
        return SB_ERR_SHAPE;
    if (d->B > 0) {
        if ((d->ldx % 8) != 0 || (d->ldw % 8) != 0)
            return SB_ERR_ALIGN;
        for (int i = 0; i < d->k; ++i)
            if (!aligned16(d->x[i]) || !aligned16(d->w[i]))
                return SB_ERR_ALIGN;
    }
    // per-chunk buffer offsets are 32-bit: a chunk of weight rows and one row
    // group of an activation shard must span less than 4 GiB
    const int64_t lim = (int64_t)1 << 32;
    if ((int64_t)(sbk::kPartChunk + 8) * d->ldw * 2 >= lim ||
        (int64_t)(sbk::kRowBlock * sbk::kMaxMB) * d->ldx * 2 >= lim)
        return SB_ERR_UNSUPPORTED;
    // the chunked GEMM's launch fits one grid
    int64_t chunks = 0;
    for (int i = 0; i < d->k; ++i)
        chunks += ((int64_t)d->lane_k[i + 1] - d->lane_k[i] + sbk::kPartChunk - 1) /
                  sbk::kPartChunk;
    if (sbk::partial_launch_items(d->B, d->N, (int32_t)chunks) >= lim)
        return SB_ERR_UNSUPPORTED;
    return SB_OK;
}

int partial_chunks(const sb_partial_desc *d)
{
    int n = 0;
    for (int i = 0; i < d->k; ++i)
        n += (d->lane_k[i + 1] - d->lane_k[i] + sbk::kPartChunk - 1) / sbk::kPartChunk;
    return n;
}

// The chunk partials sit after the head calls' counter region, so that one
// workspace can serve both kinds of call.
size_t partial_bytes(const sb_partial_desc *d)
{
    if (d->B == 0)
        return 0;  // nothing is read or written
    return kCtrBytes + align_up((size_t)partial_chunks(d) * (size_t)d->B *
                                     (size_t)shard_ld(d->N) * sizeof(float),
                                 kRegionAlign);
}

}  // namespace

extern "C" {

size_t sb_workspace_bytes(const sb_head_desc *desc, int surface, sb_status *status)
{
    sb_status st = check_desc(desc);
    if (st == SB_OK && (surface < SB_SURF_TOKENS || surface > SB_SURF_FULL_LOGITS))
        st = SB_ERR_SHAPE;
    if (status)
        *status = st;
    if (st != SB_OK)
        return 0;
    return layout(desc, surface).total;
}

sb_status sb_project_tokens(const sb_head_desc *desc, int32_t *ids, void *ws, size_t ws_bytes,
                            void *stream)
{
    return project_tokens(desc, ids, nullptr, nullptr, ws, ws_bytes, stream);
}

sb_status sb_project_tokens_static(const sb_head_desc *desc, int32_t *ids, void *stream)
{
    sb_status st = check_desc(desc);
    if (st != SB_OK)
        return st;
    if (desc->B == 0)
        return SB_OK;
    if (!ids)
        return SB_ERR_NULL;
    const Layout L = layout(desc, SB_SURF_TOKENS);
    if (L.total > sbk::kStaticScratchBytes)
        return SB_ERR_WORKSPACE;
    // the stream's device (the current one for the null stream)
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess)
        return SB_ERR_HIP;
    void *ws = nullptr;
    if (sbk::static_scratch(dev, &ws) != hipSuccess)
        return SB_ERR_HIP;
    return project_tokens(desc, ids, nullptr, nullptr, ws, sbk::kStaticScratchBytes, stream);
}

sb_status sb_project_lane_results(const sb_head_desc *desc, int32_t *ids, int32_t *lane_ids,
                                  float *lane_max, void *ws, size_t ws_bytes, void *stream)
{
    return project_tokens(desc, ids, lane_ids, lane_max, ws, ws_bytes, stream);
}

sb_status sb_project_logprobs(const sb_head_desc *desc, int32_t *ids, float *lse, float *sel_lp,
                              float *logprobs, int64_t ldlp, void *ws, size_t ws_bytes,
                              void *stream)
{
    sb_status st = check_desc(desc);
    if (st != SB_OK)
        return st;
    if (desc->B == 0)
        return SB_OK;
    if (!ids || !lse)
        return SB_ERR_NULL;
    if (logprobs) {
        if (ldlp < desc->V)
            return SB_ERR_SHAPE;
        if (!aligned16(logprobs) || (ldlp % 4) != 0)
            return SB_ERR_ALIGN;
    }
    const Layout L = layout(desc, logprobs ? SB_SURF_LOGPROBS_FULL : SB_SURF_LOGPROBS);
    if ((st = check_ws(L, ws, ws_bytes)) != SB_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    sbk::HeadArgs a;
    fill_args(desc, L, a);
    a.pair = region<int2>(ws, L.pair);
    a.mse = region<float2>(ws, L.mse);
    set_slices(L, ws, a);
    set_zero(a);
    a.out = logprobs;
    a.ldo = ldlp;
    const int epi = logprobs ? sbk::kEpiPairLseOut : sbk::kEpiPairLse;
    const hipError_t e = a.B >= sbk::kLargeBatch ? sbk::launch_head_gemm_large(a, epi, s)
                                                  : sbk::launch_head_gemm(a, epi, s);
    if (e != hipSuccess ||
        sbk::launch_combine(a.pair, a.mse, a.lanes, a.B, a.T, ids, lse, sel_lp, nullptr, nullptr,
                            s) != hipSuccess)
        return SB_ERR_HIP;
    if (logprobs && sbk::launch_normalize(logprobs, ldlp, lse, a.B, a.V, s) != hipSuccess)
        return SB_ERR_HIP;
    return SB_OK;
}

sb_status sb_full_logits(const sb_head_desc *desc, float *logits, int64_t ldl, int32_t *ids,
                         void *ws, size_t ws_bytes, void *stream)
{
    sb_status st = check_desc(desc);
    if (st != SB_OK)
        return st;
    if (desc->B == 0)
        return SB_OK;
    if (!logits)
        return SB_ERR_NULL;
    if (ldl < desc->V)
        return SB_ERR_SHAPE;
    if (!aligned16(logits) || (ldl % 4) != 0)
        return SB_ERR_ALIGN;
    const Layout L = layout(desc, SB_SURF_FULL_LOGITS);
    if ((st = check_ws(L, ws, ws_bytes)) != SB_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    sbk::HeadArgs a;
    fill_args(desc, L, a);
    for (int i = 0; i < desc->k; ++i) {
        a.lanes.shard[i] = region<float>(ws, L.shard[i]);
        a.lanes.shard_ld[i] = shard_ld(lane_width(desc, i));
    }
    set_slices(L, ws, a);
    set_zero(a);
    const hipError_t e = a.B >= sbk::kLargeBatch ? sbk::launch_head_gemm_large(a, sbk::kEpiShard, s)
                                                  : sbk::launch_head_gemm(a, sbk::kEpiShard, s);
    if (e != hipSuccess)
        return SB_ERR_HIP;
    if (sbk::launch_reconstruct(a.lanes, a.B, logits, ldl, s) != hipSuccess)
        return SB_ERR_HIP;
    if (ids && sbk::launch_row_argmax(logits, ldl, a.B, a.V, region<int2>(ws, L.partial), ids,
                                      s) != hipSuccess)
        return SB_ERR_HIP;
    return SB_OK;
}

size_t sb_partial_workspace_bytes(const sb_partial_desc *desc, sb_status *status)
{
    const sb_status st = check_partial(desc);
    if (status)
        *status = st;
    return st == SB_OK ? partial_bytes(desc) : 0;
}

sb_status sb_partial_complete(const sb_partial_desc *desc, int op, float *out, int64_t ldo,
                              void *ws, size_t ws_bytes, void *stream)
{
    sb_status st = check_partial(desc);
    if (st != SB_OK)
        return st;
    if (op < SB_RED_SUM || op > SB_RED_MAX)
        return SB_ERR_SHAPE;
    if (desc->B == 0)
        return SB_OK;
    if (!out)
        return SB_ERR_NULL;
    if (ldo < desc->N)
        return SB_ERR_SHAPE;
    if (!aligned16(out) || (ldo % 4) != 0)
        return SB_ERR_ALIGN;
    const size_t need = partial_bytes(desc);
    if (!ws)
        return SB_ERR_NULL;
    if (ws_bytes < need)
        return SB_ERR_WORKSPACE;
    if (!aligned16(ws))
        return SB_ERR_ALIGN;
    sbk::PartialArgs a;
    memset(&a, 0, sizeof a);
    a.k = desc->k;
    int chunks = 0;
    for (int i = 0; i < desc->k; ++i) {
        a.x[i] = static_cast<const uint16_t *>(desc->x[i]);
        a.w[i] = static_cast<const uint16_t *>(desc->w[i]);
        a.K[i] = desc->lane_k[i + 1] - desc->lane_k[i];
        a.chunk0[i] = chunks;
        chunks += (a.K[i] + sbk::kPartChunk - 1) / sbk::kPartChunk;
    }
    a.chunk0[desc->k] = chunks;
    a.ldx = desc->ldx;
    a.ldw = desc->ldw;
    a.B = desc->B;
    a.N = desc->N;
    a.T = (desc->N + sbk::kTileN - 1) / sbk::kTileN;
    a.part = reinterpret_cast<float *>(static_cast<char *>(ws) + kCtrBytes);
    a.ldp = shard_ld(desc->N);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (sbk::launch_partial_gemm(a, s) != hipSuccess ||
        sbk::launch_partial_reduce(a, op, out, ldo, s) != hipSuccess)
        return SB_ERR_HIP;
    return SB_OK;
}

const char *sb_status_string(sb_status status)
{
    switch (status) {
    case SB_OK:
        return "ok";
    case SB_ERR_NULL:
        return "a required pointer is NULL";
    case SB_ERR_SHAPE:
        return "invalid shape or leading dimension";
    case SB_ERR_LANES:
        return "invalid lane count or lane offsets";
    case SB_ERR_ALIGN:
        return "pointer or leading dimension not aligned";
    case SB_ERR_WORKSPACE:
        return "workspace too small";
    case SB_ERR_UNSUPPORTED:
        return "size beyond the supported limits";
    case SB_ERR_HIP:
        return "HIP launch failed";
    case SB_STATUS_RANGE_MAX_:
        break;
    }
    return "unknown status";
}

}  // extern "C"
