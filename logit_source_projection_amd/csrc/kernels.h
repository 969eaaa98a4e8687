// Internal launch interface of libsb's HIP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbk {

constexpr int kMaxLanes = 64;
constexpr int kTileN = 128;     // vocab columns per workgroup tile
constexpr int kStepK = 32;      // hidden rows per MFMA step (16x16x32 bf16)
constexpr int kWaves = 4;       // waves per workgroup; K steps interleaved over them
constexpr int kRowBlock = 16;   // rows per MFMA row block
constexpr int kMaxMB = 4;       // row blocks per workgroup
constexpr int kArgmaxChunk = 8192;  // columns per workgroup in the full-logit argmax
constexpr int kLineBytes = 128;     // L2 cache line
// A lane's tile grid starts up to this many columns before its first column,
// so that tiles begin on a cache line (shard bases are 16-byte aligned).
constexpr int kMaxShift = (kLineBytes - 16) / 2;

// Epilogue variants of the head GEMM.
enum Epilogue : int {
    kEpiPair = 0,        // (max, lowest index) per (row, tile)
    kEpiPairLse = 1,     // + (tile max, sum exp(y - tile max)) per (row, tile)
    kEpiPairLseOut = 2,  // + fp32 logits written at their global column
    kEpiShard = 3        // fp32 logits written to per-lane shards only
};

// Per-lane tables, passed by value as a kernel argument.
struct LaneTable {
    const uint16_t *w[kMaxLanes];  // lane i's shard base (bf16 bits)
    float *shard[kMaxLanes];       // lane i's fp32 shard (kEpiShard)
    int32_t off[kMaxLanes + 1];    // vocab offsets
    int32_t tile0[kMaxLanes + 1];  // first tile of lane i (prefix sums)
    // Tile t of lane i covers lane columns [t*kTileN - shift[i], +kTileN):
    // shift[i] (a multiple of 8, at most kMaxShift) puts every tile but the
    // first on a cache-line boundary, so that neighbouring tiles, which run
    // on different XCDs, never fetch the same line.  Columns before the
    // lane's first are loaded from column 0 and dropped.
    int32_t shift[kMaxLanes];
    int32_t shard_ld[kMaxLanes];   // row stride of lane i's shard
    int32_t k;
};

// Up to three ranges of 32-bit words that a call clears before its head
// kernel touches them (the slice counters of a split head).
struct ZeroRanges {
    uint32_t *p[3];
    int32_t n[3];  // words; 0 = unused
};

struct HeadArgs {
    LaneTable lanes;
    const uint16_t *x;   // bf16 [B][ldx]
    int64_t ldx;
    int64_t ldw;
    int32_t B, H, V;
    int32_t T;           // row stride of the pair workspaces (>= lanes.tile0[k])
    int2 *pair;          // [B][T] {float bits of the tile max, its lowest global index}
    float2 *mse;         // [B][T] {tile max, sum exp(y - tile max)} (log-prob surfaces)
    float *out;          // [B][ldo] fp32 logits at global columns (kEpiPairLseOut)
    int64_t ldo;
    // K slices (head_gemm_kernel, one row group): the hidden steps of every
    // tile are split into kslices contiguous runs of slice_steps steps, one
    // workgroup each; each writes its partial tile to kpart and the last to
    // finish a tile adds the kslices partials in slice order.
    int32_t kslices;             // 1 = no split
    int32_t slice_steps;         // kStepK-row steps per slice, a multiple of kWaves
    float *kpart;                // [T][kslices][row blocks][2][threads][4] fp32 partial tiles
    uint32_t *kctr;              // [T] per-tile slice counters, cleared before the launch
    // Hidden rows packed per K step for 33-64 rows (one row group of four
    // blocks): [steps][4][64 lanes] 16-byte units, written by the call.
    uint16_t *xp;
    // Words the head launch needs at zero: cleared by a launch of its own
    // before the head kernel (by the hidden-row pack for 33-64 rows).
    ZeroRanges zero;
};

// Bytes of the packed hidden rows of a call (0 where X is read directly).
inline size_t packed_hidden_bytes(int B, int H)
{
    return (B > 2 * kRowBlock && B <= kRowBlock * kMaxMB && H > 0)
               ? (size_t)((H + kStepK - 1) / kStepK) * kMaxMB * 1024
               : 0;
}

// Tiles of a lane of vi columns whose grid starts `shift` columns early.
inline int lane_tiles(int vi, int shift) { return (vi + shift + kTileN - 1) / kTileN; }

// Rows per workgroup row group for a batch of B rows: one, two or four
// 16-row MFMA blocks, so that up to 64 rows read each weight tile once (more
// rows run as further row groups, dispatched right after each other on the
// same weight tile).
inline int rows_per_group(int B)
{
    return B <= kRowBlock ? kRowBlock : (B <= 2 * kRowBlock ? 2 * kRowBlock : kMaxMB * kRowBlock);
}

// K slices for a head of few tiles.  One workgroup streams one 128-column
// tile at a few tens of GB/s, so a head of fewer than kSplitBelowTiles tiles
// leaves most of the 256 CUs idle.  Such a head splits every tile's hidden
// steps into slices of at least kMinSliceSteps steps, up to kMaxSlices of
// them, so that about kSplitTarget workgroups (one per CU) run.  Larger heads
// are not split, except just past one tile per CU (below): one workgroup per
// tile streamed fastest from 128 tiles up in timings of 1 to 8 slices (a
// split adds a partial-tile write and a fold per slice).  The split depends
// on (B, H, V) only -- not on the lane split or the shard placement -- so
// every surface and every lane split of a head sums each logit in the same
// order.
constexpr int kSplitBelowTiles = 128;
constexpr int kSplitTarget = 256;
constexpr int kMinSliceSteps = 16;
constexpr int kMaxSlices = 8;
// Just past one tile per CU (kSplitTarget < tiles <= kSplitPairMaxTiles),
// one 16-row block and at least kSplitPairMinSteps hidden steps: two slices
// per tile, so that no CU streams two whole tiles while others idle (timed
// at H = 5120: 4-7 % faster from 264 to 320 tiles, 1 % at 352, slower at
// 256 and from 391 tiles on).
constexpr int kSplitPairMaxTiles = 352;
constexpr int kSplitPairMinSteps = 128;
constexpr int kMaxSplitTiles = 2048;  // tile capacity of the slice counters
static_assert(kSplitBelowTiles + 2 * kMaxLanes <= kMaxSplitTiles &&
                  kSplitPairMaxTiles + 2 * kMaxLanes <= kMaxSplitTiles,
              "a split head's tiles, shifted lanes included, fit the counters");
inline int k_slices(int B, int H, int V)
{
    if (B <= 0 || B > kRowBlock * kMaxMB || H <= 0 || V <= 0)
        return 1;
    const int tiles = (V + kTileN - 1) / kTileN;
    const int nsteps = (H + kStepK - 1) / kStepK;
    int s;
    if (tiles < kSplitBelowTiles) {
        s = (kSplitTarget + tiles - 1) / tiles;
        s = s < kMaxSlices ? s : kMaxSlices;
        s = s < nsteps / kMinSliceSteps ? s : nsteps / kMinSliceSteps;
    } else if (B <= kRowBlock && tiles > kSplitTarget && tiles <= kSplitPairMaxTiles &&
               nsteps >= kSplitPairMinSteps) {
        s = 2;
    } else {
        return 1;
    }
    if (s <= 1)
        return 1;
    // whole multiples of kWaves steps per slice, and no empty slice
    const int per = ((nsteps + s - 1) / s + kWaves - 1) / kWaves * kWaves;
    return (nsteps + per - 1) / per;
}
inline int slice_steps(int H, int slices)
{
    const int nsteps = (H + kStepK - 1) / kStepK;
    return slices <= 1 ? nsteps : ((nsteps + slices - 1) / slices + kWaves - 1) / kWaves * kWaves;
}

// Launch the head GEMM (B <= 128) with the given epilogue: the (row, tile)
// pairs (every epilogue but kEpiShard; launch_combine folds them) and the
// logits or shards.  a.zero is cleared first, on the same stream.
hipError_t launch_head_gemm(const HeadArgs &a, int epi, hipStream_t s);

// Batches of at least this many rows (more than one 64-row group) use the
// large-batch head GEMM for every surface: from 65 to 128 rows with 128-row
// blocks (bench.py, alternated with the earlier kernel of two 128-column tiles
// per 64-row group: 9-12 % faster on the dense and MoE heads), from 129 rows
// with 256-row blocks (128-row blocks there read the weight once per block
// row and ran 9-20 % slower from 160 to 2048 rows).
constexpr int kLargeBatch = 65;
// Block rows and K stage depth of the large-batch kernel (its 32-bit buffer
// offsets reach large_block_rows(B) rows of x and at most kLargeStepK rows of
// a shard).  Up to kLargeSmallMax rows it runs 128-row blocks with
// kLargeSmallStepK-deep stages in a three-stage LDS ring, beyond that
// kLargeRows-row blocks with kLargeStepK-deep stages in two.
constexpr int kLargeRows = 256;
constexpr int kLargeSmallMax = 128;
constexpr int kLargeStepK = 64;
constexpr int kLargeStages = 2;
constexpr int kLargeSmallStepK = 32;
constexpr int kLargeSmallStages = 3;
inline int large_block_rows(int B) { return B <= kLargeSmallMax ? 128 : kLargeRows; }
inline int large_step_k(int B) { return B <= kLargeSmallMax ? kLargeSmallStepK : kLargeStepK; }

// Large-batch head GEMM: writes the (row, tile) results (and logits /
// shards); ids / lse / sel_lp come from launch_combine afterwards.
hipError_t launch_head_gemm_large(const HeadArgs &a, int epi, hipStream_t s);

// Fold the (row, tile) workspaces into ids / lse / sel_lp and the per-lane
// results lane_ids / lane_max ([B][k]; any may be NULL except ids).  One
// workgroup per row; tiles folded lane by lane in ascending order, lanes
// folded in ascending order.
hipError_t launch_combine(const int2 *pair, const float2 *mse, const LaneTable &lanes,
                          int32_t B, int32_t T, int32_t *ids, float *lse,
                          float *sel_lp, int32_t *lane_ids, float *lane_max, hipStream_t s);

// lp[b][v] -= lse[b] over [B][V] (row stride ld).
hipError_t launch_normalize(float *lp, int64_t ld, const float *lse, int32_t B,
                            int32_t V, hipStream_t s);

// Reconstruct the complete [B][ldl] logits from the per-lane shards.
hipError_t launch_reconstruct(const LaneTable &lanes, int32_t B, float *logits,
                              int64_t ldl, hipStream_t s);

// Row argmax (lowest index on ties) of logits [B][ldl] over V columns; needs a
// workspace of B * ceil(V / kArgmaxChunk) int2.
hipError_t launch_row_argmax(const float *logits, int64_t ldl, int32_t B, int32_t V,
                             int2 *partial, int32_t *ids, hipStream_t s);

// Launch limits.  A HIP launch holds fewer than 2^32 work items in each grid
// dimension and at most kMaxGridRows workgroups in y and z.  The launches with
// one row per y index (normalize, reconstruct, row argmax, partial reduce) run
// over longer batches in slices of kMaxGridRows rows; every other launch must
// fit in one grid, which validation checks with the functions below.
constexpr int kMaxGridRows = 65535;
// Work items of the largest x dimension of any launch a head call on B rows
// with these lane offsets makes, counted for the widest tile shifts, so that
// the bound does not depend on where the shards sit.
int64_t head_launch_items(int32_t B, int32_t H, int32_t V, const int32_t *lane_off, int32_t k);
// The same for a partial-completion call of B rows, N output columns and
// `chunks` reduction chunks.
int64_t partial_launch_items(int32_t B, int32_t N, int32_t chunks);

// ---------------------------------------------------------------------------
// Partial completion: lane i holds an activation shard X_i [B][K_i] and the
// matching weight rows W_i [K_i][N]; its partial is P_i = X_i . W_i, and a
// registered elementwise operator completes the k partials in lane order.
// ---------------------------------------------------------------------------
constexpr int kPartChunk = 1024;  // reduction rows per workgroup (split K)

enum ReduceOp : int { kRedSum = 0, kRedProd = 1, kRedMin = 2, kRedMax = 3 };

struct PartialArgs {
    const uint16_t *x[kMaxLanes];   // lane i's activation shard, bf16 [B][ldx]
    const uint16_t *w[kMaxLanes];   // lane i's weight rows, bf16 [K_i][ldw]
    int32_t K[kMaxLanes];           // reduction rows of lane i
    int32_t chunk0[kMaxLanes + 1];  // first chunk of lane i (prefix sums of ceil(K_i / kPartChunk))
    int64_t ldx, ldw;
    int32_t B, N, k;
    int32_t T;                      // 128-column tiles of the output
    float *part;                    // [chunks][B][ldp] fp32 chunk partials
    int64_t ldp;
};

// Chunk partials: part[c][b][n] = sum over the chunk's reduction rows.
hipError_t launch_partial_gemm(const PartialArgs &a, hipStream_t s);

// out[b][n] = op over lanes (ascending) of the sum over the lane's chunks
// (ascending).
hipError_t launch_partial_reduce(const PartialArgs &a, int op, float *out, int64_t ldo,
                                 hipStream_t s);

// ---------------------------------------------------------------------------
// Static device scratch for the token call that allocates nothing
// (sb_project_tokens_static): one array per device, held until the process
// ends.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;

// The device address of the current device's scratch array, looked up once
// per device (hipGetSymbolAddress with that device current) and kept.
hipError_t static_scratch(int device, void **ptr);

}  // namespace sbk
