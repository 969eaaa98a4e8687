// HIP kernels of libsb for CDNA4 (gfx950).
//
// Head GEMM z = X . W over k vocab lanes, with fused epilogues that reduce
// each (row, 128-column tile) to a (max, lowest global index) pair and an
// online (max, sum-exp) pair, or write the fp32 logits.  The SemBridge paper
// (section 5.2, section 6, Figure 1) ships one argmax result per lane instead
// of the lane's logits; here every lane is reduced inside the GEMM epilogue
// and the per-tile results are folded afterwards (combine kernel).
//
// Mainloop design (decode shapes are HBM-bound: every weight byte is used by
// B <= 64 rows only):
//   * one workgroup = 4 waves = one 128-column tile of one lane, rows
//     [m0, m0 + 16*MB) with MB = 1, 2 or 4, so that up to 64 rows read each
//     weight tile once;
//   * W is row-major along the vocabulary (column-contiguous), while the
//     16x16x32 bf16 MFMA wants 8 consecutive K values per lane.  Each lane
//     loads 8 rows x 8 columns (eight 16-byte loads, 256-byte contiguous
//     segments per 16 lanes) and transposes them in registers with v_perm;
//     MFMA number c of a step then covers the strided column set
//     {c0 + 8n + c : n = 0..15}, so after the eight MFMAs a lane holds eight
//     consecutive columns of four rows;
//   * K steps of 32 rows are interleaved over the 4 waves (wave w takes steps
//     w, w+4, ...); every wave keeps its own fp32 accumulators and the four
//     partial tiles are added in wave order 0+1+2+3 through LDS.  Each logit
//     is therefore accumulated in an order fixed by H alone (by B, H and V
//     for a head split into K slices), independent of the lane split, the
//     column position and the epilogue;
//   * buffer loads with per-step rebased resources: rows beyond H and
//     columns beyond the lane's end read as zero without faulting;
//   * weight loads are non-temporal when one row group covers the batch
//     (every weight byte is then read exactly once), and use the default
//     policy when further row groups re-read the tile through the L2;
//   * a lane's tiles start on 128-byte lines, so that no line is shared by
//     two tiles.
#include "kernels.h"

#include <atomic>
#include <algorithm>

#include <float.h>
#include <limits.h>

namespace sbk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = kWaves * 64;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// Cache policy of the weight loads: kPolicyStream marks them non-temporal
// (each weight byte is read by one workgroup only and should not displace
// the hidden rows, which every workgroup re-reads); kPolicyShared keeps the
// default policy, for tiles that several row groups read through the L2.
constexpr int kPolicyShared = 0;
constexpr int kPolicyStream = 2;  // the nt bit of the buffer instruction

template <int POL>
__device__ __forceinline__ u32x4 load16w(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, POL));
}

// (value, index) order: larger value first, then lower index.
// Raises a kernel's dynamic-LDS limit on the current device, once per device
// (the attribute is held per device; devices past 63 set it on every call).
// Concurrent first calls may both set it, which is harmless.
static hipError_t raise_lds_limit(const void *kernel, int bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

// The order of the argmax over (value, index): NaN above every number (the
// convention of numpy's and torch's argmax), then the order of the floats
// (+inf above every finite value, -0 equal to +0), and between equal values
// -- all NaNs count as equal -- the lower index.  It is a total order, so
// the result does not depend on the order of the fold, and every row's ID is
// one of its columns whatever its values.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2)
{
    const bool n1 = v1 != v1, n2 = v2 != v2;
    if (n1 || n2)
        return n1 && (!n2 || i1 < i2);
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// better() for a candidate whose index is higher than the current best's.
__device__ __forceinline__ bool above(float v, float best)
{
    return v > best || (v != v && best == best);
}

// The same order on values known to hold no NaN: one compare.  The head
// epilogues use it unless a wave finds a NaN among its values (any_nan8).
__device__ __forceinline__ bool better_num(float v1, int i1, float v2, int i2)
{
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Whether any of eight values is NaN: a NaN-propagating maximum of all of
// them (v_maximum3_f32, four instructions) compared with itself.
__device__ __forceinline__ bool any_nan8(float a, float b, float c, float d, float e, float f,
                                         float g, float h)
{
    const float m = __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c),
        __builtin_elementwise_maximum(__builtin_elementwise_maximum(d, e),
                                      __builtin_elementwise_maximum(__builtin_elementwise_maximum(f, g), h)));
    return m != m;
}

// Online logsumexp merge of (m2, s2) into (m1, s1); -inf marks "empty".
__device__ __forceinline__ void lse_merge(float &m1, float &s1, float m2, float s2)
{
    if (m2 == -INFINITY)
        return;
    if (m1 == -INFINITY) {
        m1 = m2;
        s1 = s2;
        return;
    }
    if (m2 > m1) {
        s1 = s1 * __expf(m1 - m2) + s2;
        m1 = m2;
    } else {
        s1 = s1 + s2 * __expf(m2 - m1);
    }
}

// Cross-lane reductions inside the 16-lane rows of a wave use DPP moves (a
// VALU operand modifier: no LDS traffic, no address registers).  Four steps
// pair each lane with one in the other half of a group of 2, 4, 8 and 16
// lanes: quad swaps by 1 and by 2, then the mirror of each 8-lane half and of
// the 16-lane row.  Both reductions below are symmetric in their two
// operands (floating-point addition commutes; the (max, lowest index) choice
// is a total order), so every lane of a row ends with the same bits.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i of its 8-lane half
constexpr int kDppMirror = 0x140;      // lane i <- lane 15 - i of its row

template <int CTRL>
__device__ __forceinline__ int dpp_int(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_float(float v)
{
    return __int_as_float(dpp_int<CTRL>(__float_as_int(v)));
}

template <int CTRL, bool NAN_AWARE>
__device__ __forceinline__ void best_step(float &bv, int &bi)
{
    const float ov = dpp_float<CTRL>(bv);
    const int oi = dpp_int<CTRL>(bi);
    if (NAN_AWARE ? better(ov, oi, bv, bi) : better_num(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
    }
}

// (max, lowest index) over each 16-lane row; every lane gets its row's.
// NAN_AWARE = false only where the wave holds no NaN.
template <bool NAN_AWARE = true>
__device__ __forceinline__ void row16_best(float &bv, int &bi)
{
    best_step<kDppQuadXor1, NAN_AWARE>(bv, bi);
    best_step<kDppQuadXor2, NAN_AWARE>(bv, bi);
    best_step<kDppHalfMirror, NAN_AWARE>(bv, bi);
    best_step<kDppMirror, NAN_AWARE>(bv, bi);
}

// The (max, lowest index) of each 16-lane row of a head epilogue, over the
// eight values y0..y7 of each thread at global columns gcol.. (the first
// nvalid of them real columns): the plain comparison, or, when any value
// of the wave is NaN, the NaN-aware order.  The branch is uniform over the
// wave, so the DPP steps see every lane of their rows.
__device__ __forceinline__ void tile_best(float y0, float y1, float y2, float y3, float y4,
                                          float y5, float y6, float y7, int nvalid, int gcol,
                                          float &bv, int &bi)
{
    const float y[8] = {y0, y1, y2, y3, y4, y5, y6, y7};
    bv = -INFINITY;
    bi = INT_MAX;
    if (nvalid > 0) {
        bv = y[0];
        bi = gcol;
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(any_nan8(y0, y1, y2, y3, y4, y5, y6, y7)) == 0,
                         1)) {
#pragma unroll
        for (int j = 1; j < 8; ++j)
            if (j < nvalid && y[j] > bv) {
                bv = y[j];
                bi = gcol + j;
            }
        row16_best<false>(bv, bi);
    } else {
#pragma unroll
        for (int j = 1; j < 8; ++j)
            if (j < nvalid && above(y[j], bv)) {
                bv = y[j];
                bi = gcol + j;
            }
        row16_best<true>(bv, bi);
    }
}

// Sum over each 16-lane row; every lane gets its row's.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_float<kDppQuadXor1>(v);
    v += dpp_float<kDppQuadXor2>(v);
    v += dpp_float<kDppHalfMirror>(v);
    v += dpp_float<kDppMirror>(v);
    return v;
}

template <int CTRL>
__device__ __forceinline__ void lse_step(float &m, float &s)
{
    lse_merge(m, s, dpp_float<CTRL>(m), dpp_float<CTRL>(s));
}

// Over the whole wave: the rows by DPP, then the four row results (lanes 0,
// 16, 32, 48) read as wave-uniform values and merged in row order.
__device__ __forceinline__ void wave_best(float &bv, int &bi)
{
    row16_best(bv, bi);
    float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
    int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
        const int oi = __builtin_amdgcn_readlane(bi, 16 * r);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
    bv = v;
    bi = i;
}

// Online logsumexp (m, s) over the whole wave, as wave_best.
__device__ __forceinline__ void wave_lse(float &m, float &s)
{
    lse_step<kDppQuadXor1>(m, s);
    lse_step<kDppQuadXor2>(m, s);
    lse_step<kDppHalfMirror>(m, s);
    lse_step<kDppMirror>(m, s);
    float wm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
    float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 0));
#pragma unroll
    for (int r = 1; r < 4; ++r)
        lse_merge(wm, ws, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16 * r)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 16 * r)));
    m = wm;
    s = ws;
}

// Results read by another workgroup of the same launch are written through
// to memory (the sc0 and sc1 bits of the store: never left dirty in an XCD's
// L2), so publishing them needs only a wait for store completion -- no L2
// write-back fence in every workgroup.
constexpr int kPolicyWriteThrough = 1 | 16;  // sc0 | sc1 of a buffer instruction

__device__ __forceinline__ void store16_through(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                const float *v)
{
    const u32x4 u = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(u, r, voff, 0, kPolicyWriteThrough);
}

// All of this wave's memory operations have completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ int find_lane(const LaneTable &t, int tile)
{
    int lane = 0;
    while (lane + 1 < t.k && t.tile0[lane + 1] <= tile)
        ++lane;
    return lane;
}

template <int MB>
struct Frags {
    u32x4 w[8];
    u32x4 x[MB];
};

// XP: xbase holds the hidden rows packed per step (pack_hidden_kernel), MB KB
// per step, and xvo[mb] = (64 mb + lane) * 16.
template <int MB, int POL, bool XP = false>
__device__ __forceinline__ void load_step(Frags<MB> &f, const uint16_t *wbase, int64_t wbytes,
                                          const uint16_t *xbase, int64_t xbytes, int k0,
                                          int64_t ldw, const uint32_t (&wvo)[8],
                                          const uint32_t (&xvo)[MB])
{
    // Resources rebased to this step's first hidden row: offsets stay small.
    const int64_t wshift = (int64_t)k0 * ldw;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wbase + wshift, wbytes - wshift * 2);
    const int64_t xshift = XP ? (int64_t)(k0 / kStepK) * (MB * 512) : k0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xbase + xshift, xbytes - xshift * 2);
#pragma unroll
    for (int r = 0; r < 8; ++r)
        f.w[r] = load16w<POL>(rw, wvo[r]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        f.x[mb] = load16(rx, xvo[mb]);
}

template <int MB>
__device__ __forceinline__ void compute_step(Frags<MB> &f, f32x4 (&acc)[MB][8], int k0, int H,
                                             int g)
{
    if (k0 + kStepK > H) {
        // K tail: hidden positions >= H must contribute exactly zero even if
        // the memory past H in a row holds non-finite bits.
        const int h0 = k0 + 8 * g;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t v = f.x[mb][d];
                if (h0 + 2 * d >= H)
                    v &= 0xFFFF0000u;
                if (h0 + 2 * d + 1 >= H)
                    v &= 0x0000FFFFu;
                f.x[mb][d] = v;
            }
        }
    }
    bf16x8 xa[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        xa[mb] = __builtin_bit_cast(bf16x8, f.x[mb]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        // Column c of the lane's 8x8 block: hidden rows 2q (low half) and
        // 2q+1 (high half) of dword c/2, half c%2, for q = 0..3.
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        u32x4 bq;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bq[q] = __builtin_amdgcn_perm(f.w[2 * q + 1][c >> 1], f.w[2 * q][c >> 1], sel);
        const bf16x8 bb = __builtin_bit_cast(bf16x8, bq);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[mb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb], bb, acc[mb][c], 0, 0, 0);
    }
}

// Minimum workgroups per CU handed to the register allocator.  One row block
// is left unconstrained (it fits 128 registers: 4 waves per SIMD); two row
// blocks are held to 3 waves per SIMD (168 registers) and four to 2 (256),
// both without spills.
// Epilogue of one (row, 128-column tile) for the thread that holds the tile's
// 8 columns from `colrel` (lane-relative; `gcol` global) of row b: the logits
// or shard store, and the tile's (max, lowest index) and (tile max, sum-exp)
// pairs, which the combine launch folds after the head kernel.  The 16
// threads of a row are 16 consecutive lanes of one wave.
template <int EPI>
__device__ __forceinline__ void emit_tile_row(const HeadArgs &a, const float (&y)[8], int b,
                                              bool rowok, int lane, int tile, int colrel,
                                              int nvalid, int gcol, int cg)
{
    if (EPI == kEpiShard || EPI == kEpiPairLseOut) {
        float *dst;
        if (EPI == kEpiShard)
            dst = a.lanes.shard[lane] + (int64_t)b * a.lanes.shard_ld[lane] + colrel;
        else
            dst = a.out + (int64_t)b * a.ldo + gcol;
        if (rowok) {
            if (nvalid == 8 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                *reinterpret_cast<f32x4 *>(dst) = f32x4{y[0], y[1], y[2], y[3]};
                *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{y[4], y[5], y[6], y[7]};
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (j < nvalid)
                        dst[j] = y[j];
            }
        }
    }
    if (EPI != kEpiShard) {
        // (max, lowest index) over the thread's columns, ascending, then
        // across the 16 threads of this row (one 16-lane row of the wave)
        float bv;
        int bi;
        tile_best(y[0], y[1], y[2], y[3], y[4], y[5], y[6], y[7], nvalid, gcol, bv, bi);
        float se = 0.f;
        if (EPI != kEpiPair) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < nvalid)
                    se += __expf(y[j] - bv);
            se = row16_sum(se);
        }
        if (cg == 0 && rowok) {
            const int64_t idx = (int64_t)b * a.T + tile;
            a.pair[idx] = make_int2(__float_as_int(bv), bi);
            if (EPI != kEpiPair)
                a.mse[idx] = make_float2(bv, se);
        }
    }
}

// The hidden rows of one row group (MB blocks of 16 rows) packed per 32-deep
// step: unit (s, mb, lane) holds X[16 mb + lane % 16][32 s + 8 (lane / 16)
// .. + 7] (zeros past B rows and past H), so that a wave's fragment load of
// a step reads MB contiguous KB instead of 16 half cache lines per row block.
// Positions past H in a row are never read.
// Zero the call's slice counters: every thread of the grid takes words
// i, i + stride, ... of each range.
__device__ __forceinline__ void clear_ranges(const ZeroRanges &z, int64_t i, int64_t stride)
{
#pragma unroll
    for (int r = 0; r < 3; ++r)
        for (int64_t j = i; j < z.n[r]; j += stride)
            z.p[r][j] = 0u;
}

__global__ __launch_bounds__(kThreads) void clear_kernel(const ZeroRanges z)
{
    clear_ranges(z, (int64_t)blockIdx.x * kThreads + threadIdx.x, (int64_t)gridDim.x * kThreads);
}

// Clear the ranges of `z` on stream s (no launch when all are empty).
hipError_t launch_clear(const ZeroRanges &z, hipStream_t s)
{
    const int64_t words = (int64_t)z.n[0] + z.n[1] + z.n[2];
    if (words <= 0)
        return hipSuccess;
    const int64_t wg = (words + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(clear_kernel, dim3((unsigned)(wg < 64 ? wg : 64)), dim3(kThreads), 0, s, z);
    return hipGetLastError();
}

template <int MB>
__global__ __launch_bounds__(MB * 64) void pack_hidden_kernel(const uint16_t *x, int64_t ldx,
                                                              int B, int H, uint16_t *xp,
                                                              const ZeroRanges z)
{
    clear_ranges(z, (int64_t)blockIdx.x * (MB * 64) + threadIdx.x, (int64_t)gridDim.x * (MB * 64));
    const int s = blockIdx.x;
    const int mb = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int row = kRowBlock * mb + (L & 15);
    const int k0 = kStepK * s + 8 * (L >> 4);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < B) {
        const uint16_t *p = x + (int64_t)row * ldx + k0;
        if (k0 + 8 <= H) {
            v = *reinterpret_cast<const u32x4 *>(p);  // 16-byte aligned: ldx % 8 == 0
        } else if (k0 < H) {
            uint16_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                e[j] = k0 + j < H ? p[j] : (uint16_t)0;
            v = __builtin_bit_cast(u32x4, e);
        }
    }
    reinterpret_cast<u32x4 *>(xp)[(int64_t)s * (MB * 64) + threadIdx.x] = v;
}

template <int MB>
struct Occupancy {
    static constexpr int kBlocksPerCU = MB == 1 ? 1 : (MB == 2 ? 3 : 2);
};

template <int MB, int EPI, int POL, bool XP>
__global__ __launch_bounds__(kThreads, Occupancy<MB>::kBlocksPerCU) void head_gemm_kernel(const HeadArgs a)
{
    __shared__ float red[kWaves][kRowBlock][kTileN + 4];

    // 1-D grid in blocks of 8 tiles x all row groups (or all K slices): the
    // row groups of one weight tile get workgroup ids 8 apart.  Workgroups
    // are handed to the 8 XCDs round-robin, so they share one XCD's L2 and
    // all but the first read the tile from it (a placement hint only;
    // results do not depend on where a workgroup runs).  Ids past the last
    // tile exit at once.  A head split into K slices has one row group.
    const int groups = (a.B + kRowBlock * MB - 1) / (kRowBlock * MB);
    const int per_tile = groups * a.kslices;
    const int q = blockIdx.x >> 3;
    const int tile = (q / per_tile) * 8 + (blockIdx.x & 7);
    const int group = (q - (q / per_tile) * per_tile) % groups;
    const int slice = (q - (q / per_tile) * per_tile) / groups;
    if (tile >= a.lanes.tile0[a.lanes.k])
        return;
    const int lane = find_lane(a.lanes, tile);
    // first column inside the lane (negative in a shifted lane's first tile)
    const int c0 = (tile - a.lanes.tile0[lane]) * kTileN - a.lanes.shift[lane];
    const int cb = max(c0, 0);                              // first column loaded
    const int Vi = a.lanes.off[lane + 1] - a.lanes.off[lane];
    const int gcol0 = a.lanes.off[lane] + c0;               // first global column
    const int m0 = group * (kRowBlock * MB);
    // wave index made provably wave-uniform, so that the per-step buffer
    // resources live in scalar registers (no waterfall loops around loads)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int L = threadIdx.x & 63;
    const int n = L & 15;
    const int g = L >> 4;
    const int H = a.H;

    // Readable extents (bytes) from the first loaded column: through the last
    // valid column of the last hidden row, rounded up to whole 16-byte vectors.
    const uint16_t *wbase = a.lanes.w[lane] + cb;
    const int64_t wcols = ((int64_t)(Vi - cb) + 7) & ~(int64_t)7;
    const int64_t wbytes = H > 0 ? (((int64_t)(H - 1) * a.ldw) + wcols) * 2 : 0;
    const int rows_here = min(a.B - m0, kRowBlock * MB);
    // hidden rows: from X itself, or (XP, one row group) packed per step
    const uint16_t *xbase = XP ? a.xp : a.x + (int64_t)m0 * a.ldx;
    const int64_t xbytes =
        XP ? (int64_t)((H + kStepK - 1) / kStepK) * (MB * 1024)
           : (H > 0 ? (((int64_t)(rows_here - 1) * a.ldx) + ((H + 7) & ~7)) * 2 : 0);

    uint32_t wvo[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        wvo[r] = (uint32_t)(((int64_t)(8 * g + r) * a.ldw + max(c0 + 8 * n - cb, 0)) * 2);
    uint32_t xvo[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        xvo[mb] = XP ? (uint32_t)((64 * mb + L) * 16)
                     : (uint32_t)(((int64_t)(kRowBlock * mb + n) * a.ldx + 8 * g) * 2);

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[mb][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The slice's steps are s_begin .. s_end - 1 (all steps without a split).
    // This wave's steps are s_begin + wave, s_begin + wave + 4, ...: nw of
    // them, taken in pairs (one step loading while the other computes) with
    // a single exit at the end of a pair, so that the accumulators stay in
    // place.
    const int nsteps = (H + kStepK - 1) / kStepK;
    const int s_begin = slice * a.slice_steps;
    const int s_len = min(s_begin + a.slice_steps, nsteps) - s_begin;
    const int nw = s_len > wave ? (s_len - wave + kWaves - 1) / kWaves : 0;
    Frags<MB> fa, fb;
    int k0 = (s_begin + wave) * kStepK;
    if (nw > 0)
        load_step<MB, POL, XP>(fa, wbase, wbytes, xbase, xbytes, k0, a.ldw, wvo, xvo);
    for (int i = 0; i + 2 <= nw; i += 2) {
        load_step<MB, POL, XP>(fb, wbase, wbytes, xbase, xbytes, k0 + kWaves * kStepK, a.ldw, wvo,
                           xvo);
        compute_step<MB>(fa, acc, k0, H, g);
        if (i + 2 < nw)
            load_step<MB, POL, XP>(fa, wbase, wbytes, xbase, xbytes, k0 + 2 * kWaves * kStepK, a.ldw,
                               wvo, xvo);
        compute_step<MB>(fb, acc, k0 + kWaves * kStepK, H, g);
        k0 += 2 * kWaves * kStepK;
    }
    if (nw & 1)
        compute_step<MB>(fa, acc, k0, H, g);

    // ---------------- epilogue, one 16-row block at a time ----------------
    // A K slice's partial tile: kPartBlock floats, one row block after the
    // other, each as two halves of one 16-byte unit per thread.
    constexpr int kPartBlock = kRowBlock * MB * kTileN;
    constexpr int kPartHalf = kRowBlock * kTileN / 2;
    static_assert(kPartHalf == 4 * kThreads, "a half holds 4 floats per thread");
    const int erow = threadIdx.x >> 4;  // 0..15: row inside the block
    const int cg = threadIdx.x & 15;    // 8-column group inside the tile
    const int colrel = c0 + 8 * cg;     // column inside the lane
    const int nvalid = colrel < 0 ? 0 : max(0, min(8, Vi - colrel));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if (m0 + kRowBlock * mb >= a.B)
            break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x4 lo = {acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
            f32x4 hi = {acc[mb][4][r], acc[mb][5][r], acc[mb][6][r], acc[mb][7][r]};
            *reinterpret_cast<f32x4 *>(&red[wave][4 * g + r][8 * n]) = lo;
            *reinterpret_cast<f32x4 *>(&red[wave][4 * g + r][8 * n + 4]) = hi;
        }
        __syncthreads();
        float y[8];
        {
            const f32x4 p0l = *reinterpret_cast<const f32x4 *>(&red[0][erow][8 * cg]);
            const f32x4 p0h = *reinterpret_cast<const f32x4 *>(&red[0][erow][8 * cg + 4]);
            const f32x4 p1l = *reinterpret_cast<const f32x4 *>(&red[1][erow][8 * cg]);
            const f32x4 p1h = *reinterpret_cast<const f32x4 *>(&red[1][erow][8 * cg + 4]);
            const f32x4 p2l = *reinterpret_cast<const f32x4 *>(&red[2][erow][8 * cg]);
            const f32x4 p2h = *reinterpret_cast<const f32x4 *>(&red[2][erow][8 * cg + 4]);
            const f32x4 p3l = *reinterpret_cast<const f32x4 *>(&red[3][erow][8 * cg]);
            const f32x4 p3h = *reinterpret_cast<const f32x4 *>(&red[3][erow][8 * cg + 4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                y[j] = ((p0l[j] + p1l[j]) + p2l[j]) + p3l[j];
                y[j + 4] = ((p0h[j] + p1h[j]) + p2h[j]) + p3h[j];
            }
        }
        __syncthreads();  // LDS free for the next block

        const int b = m0 + kRowBlock * mb + erow;
        const bool rowok = b < a.B;

        if (a.kslices > 1) {
            // This slice's partial tile, written through for the workgroup
            // that folds the tile.  A thread's 8 values of row block mb are
            // two 16-byte units at [mb][half][thread], so each store
            // instruction of a wave writes 1 KB of contiguous memory.
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(a.kpart + ((size_t)tile * a.kslices + slice) * kPartBlock,
                          (int64_t)kPartBlock * sizeof(float));
            const uint32_t vo = (uint32_t)(mb * kRowBlock * kTileN + 4 * threadIdx.x) * 4u;
            store16_through(r, vo, y);
            store16_through(r, vo + kPartHalf * 4u, y + 4);
            continue;
        }
        emit_tile_row<EPI>(a, y, b, rowok, lane, tile, colrel, nvalid, gcol0 + 8 * cg, cg);
    }
    if (a.kslices > 1) {
        // The workgroup that finishes a tile's last slice adds the partial
        // tiles in slice order and runs the epilogue; the others are done.
        __shared__ int s_fold;
        wait_all_memory();
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t old = atomicAdd(a.kctr + tile, 1u);
            s_fold = old == (uint32_t)(a.kslices - 1);
        }
        __syncthreads();
        if (!s_fold)
            return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (m0 + kRowBlock * mb >= a.B)
                break;
            const float *p = a.kpart + (size_t)tile * a.kslices * kPartBlock +
                             mb * kRowBlock * kTileN + 4 * threadIdx.x;
            f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
            f32x4 hi = *reinterpret_cast<const f32x4 *>(p + kPartHalf);
            for (int sl = 1; sl < a.kslices; ++sl) {
                p += kPartBlock;
                lo += *reinterpret_cast<const f32x4 *>(p);
                hi += *reinterpret_cast<const f32x4 *>(p + kPartHalf);
            }
            const float y[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int b = m0 + kRowBlock * mb + erow;
            emit_tile_row<EPI>(a, y, b, b < a.B, lane, tile, colrel, nvalid, gcol0 + 8 * cg, cg);
        }
    }
}

// One workgroup per row folds the per-(row, tile) results.  Wave w takes
// lanes w, w + 4, ...; in a lane, thread j merges tiles t0 + j, t0 + j + 64,
// ... in ascending order (kCombineBatch loads in flight), and the DPP row
// steps plus an in-order merge of the four rows combine the threads.  The
// lane results are then folded in
// ascending lane order: the ID of the first lane holding the row maximum
// (lowest index on ties, since lanes ascend), and
// lse = M + log sum_i S_i exp(M_i - M).  Every order here is fixed by the
// tile grid, so lse is reproduced bit for bit.
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(kThreads) void combine_kernel(const int2 *pair, const float2 *mse,
                                                           const LaneTable lanes, int T,
                                                           int32_t *ids, float *lse,
                                                           float *sel_lp, int32_t *lane_ids,
                                                           float *lane_max)
{
    __shared__ float lv[kMaxLanes], lm[kMaxLanes], ls[kMaxLanes];
    __shared__ int li[kMaxLanes];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = tid & 63, wave = tid >> 6;
    const int2 *prow = pair + (int64_t)b * T;
    const float2 *mrow = mse ? mse + (int64_t)b * T : nullptr;
    for (int lane = wave; lane < lanes.k; lane += kWaves) {
        const int t0 = lanes.tile0[lane], t1 = lanes.tile0[lane + 1];
        float bv = -INFINITY, m = -INFINITY, s = 0.f;
        int bi = INT_MAX;
        for (int t = t0 + L; t < t1; t += 64 * kCombineBatch) {
            int2 p[kCombineBatch];
            float2 q[kCombineBatch];
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                const int tu = t + 64 * u;
                p[u] = tu < t1 ? prow[tu] : make_int2(__float_as_int(-INFINITY), INT_MAX);
                if (mrow)
                    q[u] = tu < t1 ? mrow[tu] : make_float2(-INFINITY, 0.f);
            }
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                const float pv = __int_as_float(p[u].x);
                if (better(pv, p[u].y, bv, bi)) {
                    bv = pv;
                    bi = p[u].y;
                }
                if (mrow)
                    lse_merge(m, s, q[u].x, q[u].y);
            }
        }
        wave_best(bv, bi);
        if (mrow)
            wave_lse(m, s);
        if (L == 0) {
            lv[lane] = bv + 0.f;  // -0 reported as +0
            li[lane] = bi;
            lm[lane] = m;
            ls[lane] = s;
        }
    }
    __syncthreads();
    for (int i = tid; i < lanes.k; i += kThreads) {
        if (lane_ids)
            lane_ids[(int64_t)b * lanes.k + i] = li[i];
        if (lane_max)
            lane_max[(int64_t)b * lanes.k + i] = lv[i];
    }
    if (tid == 0) {
        float rv = -INFINITY, rm = -INFINITY, rs = 0.f;
        int ri = INT_MAX;
        for (int i = 0; i < lanes.k; ++i) {
            // a later lane wins only if strictly larger (its indices are higher)
            if (better(lv[i], li[i], rv, ri)) {
                rv = lv[i];
                ri = li[i];
            }
            lse_merge(rm, rs, lm[i], ls[i]);
        }
        ids[b] = ri;
        if (mse) {
            const float l = rm + __logf(rs);
            if (lse)
                lse[b] = l;
            if (sel_lp)
                sel_lp[b] = rv - l;
        }
    }
}

// Each workgroup covers kNormCols columns of one row: every thread loads
// kNormVec 16-byte vectors (all loads issued before the first store), each
// load instruction of the workgroup reading 4 KB contiguous.  The launch
// reserves kNormLdsBytes of LDS that the kernel never touches, so that at
// most two workgroups share a CU.  This in-place read-and-write stream ran
// fastest with 64 KB of loads in flight per CU: over a 2048 x 151936 buffer,
// 8 vectors per thread took 0.396 ms at two workgroups per CU and 0.41-0.42 ms
// at one or three to eight (4 vectors: 0.399 and 0.41-0.44 ms; 16 or 32
// vectors, or 64 to 1024 threads, no better).  The row is 16-byte aligned
// (the ABI requires it); the row's last workgroup steps through its vectors
// one at a time and does the last V % 4 columns per element.
constexpr int kNormVec = 8;
constexpr int kNormCols = kThreads * 4 * kNormVec;
constexpr int kNormLdsBytes = 72 * 1024;
static_assert(2 * kNormLdsBytes <= 160 * 1024 && 3 * kNormLdsBytes > 160 * 1024,
              "the reservation admits exactly two workgroups per CU");

__global__ __launch_bounds__(kThreads) void normalize_kernel(float *lp, int64_t ld,
                                                             const float *lse, int V)
{
    const int b = blockIdx.y;
    const int c0 = blockIdx.x * kNormCols + 4 * threadIdx.x;
    const float l = lse[b];
    float *row = lp + (int64_t)b * ld;
    if (blockIdx.x * kNormCols + kNormCols <= V) {
        f32x4 v[kNormVec];
#pragma unroll
        for (int j = 0; j < kNormVec; ++j)
            v[j] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(row + c0 + 4 * kThreads * j));
#pragma unroll
        for (int j = 0; j < kNormVec; ++j)
            __builtin_nontemporal_store(v[j] - l,
                                        reinterpret_cast<f32x4 *>(row + c0 + 4 * kThreads * j));
        return;
    }
#pragma unroll 1
    for (int c = c0; c < V; c += 4 * kThreads) {
        if (c + 4 <= V) {
            f32x4 *p = reinterpret_cast<f32x4 *>(row + c);
            __builtin_nontemporal_store(__builtin_nontemporal_load(p) - l, p);
        } else {
            for (int e = c; e < V; ++e)
                row[e] -= l;
        }
    }
}

// One 16-byte vector per thread, non-temporal on both sides: in a sweep of
// 1 to 8 vectors per thread and both cache policies on the prefill shards
// this streamed fastest (0.399 ms against 0.454 ms cached; 8 vectors 0.61 ms).
__global__ __launch_bounds__(kThreads) void reconstruct_kernel(const LaneTable lanes,
                                                               float *logits, int64_t ldl)
{
    const int lane = blockIdx.z;
    const int b = blockIdx.y;
    const int Vi = lanes.off[lane + 1] - lanes.off[lane];
    const int col = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (col >= Vi)
        return;
    // shard rows are 16-byte aligned (row stride a multiple of 4, aligned base)
    const float *src = lanes.shard[lane] + (int64_t)b * lanes.shard_ld[lane] + col;
    float *dst = logits + (int64_t)b * ldl + lanes.off[lane] + col;
    if (col + 4 <= Vi && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src)),
                                    reinterpret_cast<f32x4 *>(dst));
    } else {
        for (int j = 0; j < 4 && col + j < Vi; ++j)
            dst[j] = src[j];
    }
}

// Partial (max, lowest index) over a chunk of kArgmaxChunk columns of a row.
// Each thread takes its columns in ascending order, kArgmaxVec non-temporal
// 16-byte loads at a time: two streamed fastest in a sweep of 1 to 8 with
// both cache policies (0.176 ms over the prefill logits against 0.199 ms
// cached).
constexpr int kArgmaxVec = 2;
constexpr int kArgmaxCols = kThreads * 4 * kArgmaxVec;
static_assert(kArgmaxChunk % kArgmaxCols == 0, "whole batches per chunk");
__global__ __launch_bounds__(kThreads) void row_argmax_kernel(const float *logits, int64_t ldl,
                                                              int V, int nchunks, int2 *partial)
{
    __shared__ float wv[kWaves];
    __shared__ int wi[kWaves];
    const int b = blockIdx.y;
    const int c1 = min(V, (int)blockIdx.x * kArgmaxChunk + kArgmaxChunk);
    const float *row = logits + (int64_t)b * ldl;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int cs = blockIdx.x * kArgmaxChunk; cs < c1; cs += kArgmaxCols) {
        const int c0 = cs + 4 * threadIdx.x;
        f32x4 v[kArgmaxVec];
        if (aligned) {
#pragma unroll
            for (int j = 0; j < kArgmaxVec; ++j) {
                const int c = c0 + 4 * kThreads * j;
                if (c + 4 <= c1)
                    v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + c));
            }
        }
#pragma unroll
        for (int j = 0; j < kArgmaxVec; ++j) {
            const int c = c0 + 4 * kThreads * j;
            if (aligned && c + 4 <= c1) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (better(v[j][e], c + e, bv, bi)) {
                        bv = v[j][e];
                        bi = c + e;
                    }
            } else {
                for (int e = c; e < c1 && e < c + 4; ++e)
                    if (better(row[e], e, bv, bi)) {
                        bv = row[e];
                        bi = e;
                    }
            }
        }
    }
    wave_best(bv, bi);
    const int L = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (L == 0) {
        wv[wave] = bv;
        wi[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kWaves; ++w)
            if (better(wv[w], wi[w], bv, bi)) {
                bv = wv[w];
                bi = wi[w];
            }
        partial[(int64_t)b * nchunks + blockIdx.x] = make_int2(__float_as_int(bv), bi);
    }
}


// ---------------------------------------------------------------------------
// Large-batch head GEMM (more than 64 rows; MFMA-bound at prefill shapes).
//
// One workgroup = 8 waves = a BM-row x 256-column block of one lane (BM =
// 256, or 128 for 65-128 rows), laid out as 4 (rows) x 2 (columns) waves;
// each wave owns BM / 4 rows x one 128-column tile, so the per-(row, tile)
// epilogue results come straight out of one wave.  K advances in BK-row
// stages (64 for 256-row blocks, 32 for 128-row ones) through an LDS ring of
// 2 or 3 stages filled by direct-to-LDS buffer loads (1 KB per instruction),
// one 32-deep MFMA step per 32 rows of a stage:
//   * X stage [BM rows][BK k] bf16, 16-byte units XOR-swizzled by row so
//     that the 16 lanes reading one k-group of 16 rows hit distinct banks;
//   * W stage [BK k][256 columns] bf16, row-major as in HBM; a lane reads an
//     8 x 8 block (rows 8g..8g+7, columns 8n..8n+7) and transposes it in
//     registers with v_perm, as in the decode kernel.
// Each logit is accumulated over ascending K steps in one wave with
// v_mfma_f32_16x16x32_bf16.  The token / log-prob / full-logit surfaces all
// use this mainloop for large batches, so they stay bit-identical.
// ---------------------------------------------------------------------------
constexpr int kLBN = 256;
constexpr int kLWaves = 8, kLThreads = kLWaves * 64;

// Block shape of the large-batch kernel: BM rows (256 or 128) x 256 columns,
// K stages of BK rows (64 or 32) in a ring of ST stages.  Each of the 4 x 2
// waves owns BM / 4 rows (BM / 64 row blocks of 16) of one 128-column tile.
//   * 256 x 64, 2 stages: X and W stages of 32 KB each fill 128 KB of LDS
//     (one workgroup per CU).
//   * 128 x 32, 3 stages: X 8 KB and W 16 KB per stage take 72 KB, so two
//     workgroups share a CU, each with two stages of loads in flight while
//     it computes one.
template <int BM, int BK, int ST>
struct LargeShape {
    static_assert((BM == 256 || BM == 128) && (BK == 64 || BK == 32) && ST >= 2,
                  "256- or 128-row blocks, 64- or 32-deep stages, two or more of them");
    static constexpr int kStages = ST;
    static constexpr int kStageXBytes = BM * BK * 2;
    static constexpr int kStageWBytes = BK * kLBN * 2;
    static constexpr int kLdsBytes = kStages * (kStageXBytes + kStageWBytes);
    static constexpr int kSub = BK / 32;             // 32-deep MFMA steps per stage
    static constexpr int kPieces = BK * 2 / 16;      // 16-byte pieces per X row in a stage
    static constexpr int kRowsPerInst = 64 / kPieces;  // X rows per 1 KB load
    static constexpr int kXInst = BM / kRowsPerInst / kLWaves;  // X loads per wave per stage
    static constexpr int kWInst = BK / 2 / kLWaves;             // W loads per wave per stage
    static constexpr int kWaveRows = BM / 4;
    static constexpr int kRB = kWaveRows / kRowBlock;           // row blocks per wave
    static_assert(kLdsBytes <= 160 * 1024, "LDS rings must fit in 160 KB");
    static_assert((ST - 1) * (kXInst + kWInst) <= 15, "the later stages' loads fit a vmcnt wait");
    static_assert(kXInst >= 1 && kWInst >= 1, "every wave loads part of each stage");
};

// X stage layout: 1 KB load j holds rows j*R .. j*R+R-1 (R = 64 / P rows of
// P 16-byte pieces); the piece q of row r sits in slot q ^ swz(r, j).  The
// swizzle spreads the 16 rows a fragment read touches over distinct LDS banks.
template <int P>
__device__ __forceinline__ int x_swz(int r, int j)
{
    static_assert(P == 4 || P == 8, "X swizzle is defined for 4 or 8 pieces per row");
    return P == 4 ? ((r >> 2) & 3) : (((r >> 1) & 3) | ((j & 1) << 2));
}

// Zero the hidden positions at and past `hrem` (0 < hrem < BK) of an X stage
// of BM rows in LDS.  The last stage of a head whose H is not a multiple of
// BK holds the row padding of X there, which may be any bits (NaN included);
// the weight rows past H arrive as zeros (they lie past the weight buffer's
// extent), so after this every product past H is an exact +0 and the hot
// loop needs no masking.  Only that last stage calls it, after its loads
// have landed and before any wave reads it.
template <int BM, int P>
__device__ __forceinline__ void large_zero_x_tail(uint8_t *xst, int hrem)
{
    constexpr int R = 64 / P;
    for (int idx = threadIdx.x; idx < BM * P; idx += kLThreads) {
        const int row = idx / P, q = idx % P;
        const int e0 = 8 * q;  // the piece's first hidden position in the stage
        if (e0 + 8 <= hrem)
            continue;
        const int j = row / R, r = row % R;
        uint16_t *piece =
            reinterpret_cast<uint16_t *>(xst + j * 1024 + (r * P + (q ^ x_swz<P>(r, j))) * 16);
        for (int e = max(hrem - e0, 0); e < 8; ++e)
            piece[e] = 0;
    }
}

struct LargeGrid {
    int mblocks;  // ceil(B / block rows)
    int sm;       // m-blocks per super-tile (8, 4 or 2), or 0 for the plain order
    int nblocks;  // total 256-column blocks over all lanes
};

// Workgroups per super-tile of the XCD-aware order: as many as an XCD has CUs.
constexpr int kSuperWG = 32;

// Super-tile rows for a batch of `mblocks` 256-row blocks: 8 from 8 m-blocks
// up, 4 or 2 for exactly that many, else 0 (plain order).  Timed with
// bench.py on batches of 1 to 8 m-blocks: the super-tiles gained 2-5 % at 2
// and 4 m-blocks, lost up to 1.5 % at 3, and grouping 3, 5, 6 or 7 m-blocks
// into half-empty groups of 2 or 4 lost 15-28 %.
inline __host__ __device__ int super_rows(int mblocks)
{
    return mblocks >= 8 ? 8 : (mblocks == 4 || mblocks == 2 ? mblocks : 0);
}

// Workgroup id -> (m-block, n-block).  The blocks form super-tiles of sm
// m-blocks x kSuperWG / sm n-blocks (8 x 4 from 8 m-blocks up).  XCD x = id
// % 8 (workgroups are handed to the XCDs round-robin) takes super-tiles x,
// x+8, ..., so the 32 workgroups an XCD runs at a time read each K stage's
// hidden-row and weight slabs through its own L2: with 8 x 4, 384 KB per
// stage from beyond the L2 instead of the 1.06 MB that 32 n-blocks of one
// m-block need.  Without super-tiles the m-blocks of one n-block are
// consecutive.  A placement hint only: any bijection gives the same results.
__device__ __forceinline__ bool large_block(const LargeGrid &g, int id, int &mb, int &nb)
{
    if (g.sm > 0) {
        const int sn = kSuperWG / g.sm;
        const int mgroups = (g.mblocks + g.sm - 1) / g.sm;
        const int xcd = id & 7, local = id >> 3;
        const int st = (local / kSuperWG) * 8 + xcd, w = local % kSuperWG;
        mb = (st % mgroups) * g.sm + w % g.sm;
        nb = (st / mgroups) * sn + w / g.sm;
    } else {
        mb = id % g.mblocks;
        nb = id / g.mblocks;
    }
    return mb < g.mblocks && nb < g.nblocks;
}

__device__ __forceinline__ int nblock_lane(const HeadArgs &a, int nb, int &nb0)
{
    // n-blocks of lane i: ceil((V_i + shift_i) / 256), in lane order
    int lane = 0, first = 0;
    for (;;) {
        const int vi = a.lanes.off[lane + 1] - a.lanes.off[lane];
        const int nbl = (vi + a.lanes.shift[lane] + kLBN - 1) / kLBN;
        if (nb < first + nbl || lane + 1 >= a.lanes.k)
            break;
        first += nbl;
        ++lane;
    }
    nb0 = first;
    return lane;
}

// One K step's direct-to-LDS loads of a large-batch block: this wave's XI
// 1 KB loads of hidden rows (k0 = st * BK on) into xst and its WI loads of
// weight rows into wst, through buffer resources rebased at the step so that
// the 32-bit offsets stay within one stage.
template <int XI, int WI, int BK>
__device__ __forceinline__ void large_stage_loads(uint8_t *xst, uint8_t *wst, const uint16_t *xbase,
                                                  int64_t xbytes, const uint16_t *wbase,
                                                  int64_t wbytes, int st, int64_t ldw,
                                                  const uint32_t *xvo, const uint32_t *wvo,
                                                  int wave)
{
    const int k0 = st * BK;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xbase + k0, xbytes - (int64_t)k0 * 2);
#pragma unroll
    for (int i = 0; i < XI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void *)(xst + (XI * wave + i) * 1024), 16,
            xvo[i], 0, 0, 0);
    const int64_t wshift = (int64_t)st * BK * ldw;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wbase + wshift, wbytes - wshift * 2);
#pragma unroll
    for (int i = 0; i < WI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (__attribute__((address_space(3))) void *)(wst + (WI * wave + i) * 1024), 16,
            wvo[i], 0, 0, 0);
}

template <int EPI, int BM, int BK, int ST>
__global__ __launch_bounds__(kLThreads, 1) void head_gemm_large_kernel(const HeadArgs a,
                                                                       const LargeGrid grid)
{
    // the block shape as local constants (usable in device code as values)
    using Shape = LargeShape<BM, BK, ST>;
    constexpr int kStages = Shape::kStages;
    constexpr int kStageXBytes = Shape::kStageXBytes;
    constexpr int kStageWBytes = Shape::kStageWBytes;
    constexpr int kSub = Shape::kSub;
    constexpr int kPieces = Shape::kPieces;
    constexpr int kRowsPerInst = Shape::kRowsPerInst;
    constexpr int kXInst = Shape::kXInst;
    constexpr int kWInst = Shape::kWInst;
    constexpr int kWaveRows = Shape::kWaveRows;
    constexpr int RB = Shape::kRB;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int mb, nb;
    if (!large_block(grid, blockIdx.x, mb, nb))
        return;
    int nb0;
    const int lane = nblock_lane(a, nb, nb0);
    const int Vi = a.lanes.off[lane + 1] - a.lanes.off[lane];
    // first column of the block inside the lane (negative in a shifted
    // lane's first block) and the first column loaded
    const int c0 = (nb - nb0) * kLBN - a.lanes.shift[lane];
    const int cb = max(c0, 0);
    const int m0 = mb * BM;
    const int H = a.H;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int L = threadIdx.x & 63, n = L & 15, g = L >> 4;
    const int wr = wave >> 1, wc = wave & 1;  // wave row (64 rows), wave column (128 cols)

    // global extents (bytes) from the first loaded column
    const uint16_t *wbase = a.lanes.w[lane] + cb;
    const int64_t wcols = ((int64_t)(Vi - cb) + 7) & ~(int64_t)7;
    const int64_t wbytes = H > 0 ? (((int64_t)(H - 1) * a.ldw) + wcols) * 2 : 0;
    const int rows_here = min(a.B - m0, BM);
    const uint16_t *xbase = a.x + (int64_t)m0 * a.ldx;
    const int64_t xbytes = H > 0 ? (((int64_t)(rows_here - 1) * a.ldx) + ((H + 7) & ~7)) * 2 : 0;

    // this wave's loads per stage: X loads kXInst*wave .. (kRowsPerInst rows
    // each) and W loads kWInst*wave .. (2 rows of 512 B each)
    uint32_t xvo[kXInst], wvo[kWInst];
#pragma unroll
    for (int i = 0; i < kXInst; ++i) {
        const int j = kXInst * wave + i;
        const int r = L / kPieces;
        const int q = (L % kPieces) ^ x_swz<kPieces>(r, j);
        xvo[i] = (uint32_t)((((int64_t)(kRowsPerInst * j + r)) * a.ldx + 8 * q) * 2);
    }
#pragma unroll
    for (int i = 0; i < kWInst; ++i) {
        const int j = kWInst * wave + i;
        const int wrow = 2 * j + (L >> 5);
        wvo[i] = (uint32_t)((((int64_t)wrow) * a.ldw + max(c0 + 8 * (L & 31) - cb, 0)) * 2);
    }
    const int nsteps = (H + BK - 1) / BK;
    uint8_t *const xring = smem;
    uint8_t *const wring = smem + kStages * kStageXBytes;

    f32x4 acc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A ring of kStages stages: the loads of steps st+1 .. st+kStages-1 are
    // in flight while step st is computed.
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p)
        if (p < nsteps)
            large_stage_loads<kXInst, kWInst, BK>(xring + p * kStageXBytes, wring + p * kStageWBytes, xbase,
                                      xbytes, wbase, wbytes, p, a.ldw, xvo, wvo, wave);
    for (int st = 0; st < nsteps; ++st) {
        // This wave's loads of step st are done.  Loads complete in order, so
        // the kXInst + kWInst loads of each of the up to kStages - 2 later
        // steps issued so far may still be in flight.
        constexpr int kLoads = kXInst + kWInst;
        const int later = min(kStages - 2, nsteps - 1 - st);
        if (kStages >= 4 && later >= 2)
            __builtin_amdgcn_s_waitcnt(0x0f70 | (kStages >= 4 ? 2 * kLoads : 0));
        else if (kStages >= 3 && later >= 1)
            __builtin_amdgcn_s_waitcnt(0x0f70 | (kStages >= 3 ? kLoads : 0));
        else
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __builtin_amdgcn_s_barrier();  // every wave's loads of step st are in LDS and
                                       // every wave is done reading step st-1
        if (st + kStages - 1 < nsteps) {
            // refills the slots of step st-1
            const int sn = st + kStages - 1, slot = sn % kStages;
            large_stage_loads<kXInst, kWInst, BK>(xring + slot * kStageXBytes, wring + slot * kStageWBytes,
                                      xbase, xbytes, wbase, wbytes, sn, a.ldw, xvo, wvo, wave);
        }
        if (st * BK + BK > H) {
            // the last stage of a ragged H: zero X past H, then let every wave see it
            large_zero_x_tail<BM, kPieces>(xring + (st % kStages) * kStageXBytes, H - st * BK);
            __syncthreads();
        }
        const uint8_t *stage = xring + (st % kStages) * kStageXBytes;
        const uint8_t *wst = wring + (st % kStages) * kStageWBytes;
        // every fragment of the stage first (both 32-deep steps of a 64-deep
        // stage), so that the second step's reads overlap the first step's MFMAs
        u32x4 af[kSub][RB], wq[kSub][8];
#pragma unroll
        for (int ks = 0; ks < kSub; ++ks) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = wr * kWaveRows + rb * 16 + n;
                const int j = row / kRowsPerInst, r = row % kRowsPerInst;
                const int piece = 4 * ks + g;
                af[ks][rb] = *reinterpret_cast<const u32x4 *>(
                    stage + j * 1024 + (r * kPieces + (piece ^ x_swz<kPieces>(r, j))) * 16);
            }
#pragma unroll
            for (int r = 0; r < 8; ++r)
                wq[ks][r] = *reinterpret_cast<const u32x4 *>(
                    wst + (32 * ks + 8 * g + r) * (kLBN * 2) + (wc * 128 + 8 * n) * 2);
        }
        // keep the reads ahead of the MFMAs (the scheduler would sink them)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < kSub; ++ks) {
            bf16x8 xa[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                xa[rb] = __builtin_bit_cast(bf16x8, af[ks][rb]);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                u32x4 bq;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    bq[q] = __builtin_amdgcn_perm(wq[ks][2 * q + 1][c >> 1], wq[ks][2 * q][c >> 1],
                                                  sel);
                const bf16x8 bb = __builtin_bit_cast(bf16x8, bq);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][c] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[rb], bb, acc[rb][c], 0, 0, 0);
            }
        }
    }

    // ---------------- epilogue: this wave's 64 rows x 128-column tile ----------------
    const int tc0 = c0 + wc * 128;                 // tile's first column inside the lane
    if (tc0 >= Vi)
        return;                                    // past the lane's last tile
    const int tile = a.lanes.tile0[lane] + (tc0 + a.lanes.shift[lane]) / kTileN;
    const int colrel = tc0 + 8 * n;                // this lane's first column inside the lane
    const int nvalid = colrel < 0 ? 0 : max(0, min(8, Vi - colrel));
    const int gcol = a.lanes.off[lane] + colrel;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int b = m0 + wr * kWaveRows + rb * 16 + 4 * g + r;
            const bool rowok = b < a.B;
            float y[8];
#pragma unroll
            for (int c = 0; c < 8; ++c)
                y[c] = acc[rb][c][r];
            if (EPI == kEpiShard || EPI == kEpiPairLseOut) {
                float *dst = EPI == kEpiShard
                                 ? a.lanes.shard[lane] + (int64_t)b * a.lanes.shard_ld[lane] + colrel
                                 : a.out + (int64_t)b * a.ldo + gcol;
                if (rowok) {
                    if (nvalid == 8 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                        __builtin_nontemporal_store(f32x4{y[0], y[1], y[2], y[3]},
                                                    reinterpret_cast<f32x4 *>(dst));
                        __builtin_nontemporal_store(f32x4{y[4], y[5], y[6], y[7]},
                                                    reinterpret_cast<f32x4 *>(dst + 4));
                    } else {
#pragma unroll
                        for (int c = 0; c < 8; ++c)
                            if (c < nvalid)
                                dst[c] = y[c];
                    }
                }
            }
            if (EPI != kEpiShard) {
                float bv;
                int bi;
                tile_best(y[0], y[1], y[2], y[3], y[4], y[5], y[6], y[7], nvalid, gcol, bv, bi);
                float se = 0.f;
                if (EPI != kEpiPair) {
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        if (c < nvalid)
                            se += __expf(y[c] - bv);
                    se = row16_sum(se);
                }
                if (n == 0 && rowok) {
                    const int64_t idx = (int64_t)b * a.T + tile;
                    a.pair[idx] = make_int2(__float_as_int(bv), bi);
                    if (EPI != kEpiPair)
                        a.mse[idx] = make_float2(bv, se);
                }
            }
        }
    }
}

// Workgroups of a large-batch launch over mblocks x nblocks blocks: in the
// super-tile order, whole super tiles, and a multiple of 8 of them.
int64_t large_workgroups(int mblocks, int64_t nblocks)
{
    const int sm = super_rows(mblocks);
    if (sm == 0)
        return (int64_t)mblocks * nblocks;
    const int sn = kSuperWG / sm;
    const int64_t supers = (int64_t)((mblocks + sm - 1) / sm) * ((nblocks + sn - 1) / sn);
    return (supers + 7) / 8 * 8 * kSuperWG;
}

template <int EPI, int BM, int BK, int ST>
hipError_t launch_large_epi(const HeadArgs &a, hipStream_t s)
{
    LargeGrid g;
    g.mblocks = (a.B + BM - 1) / BM;
    g.nblocks = 0;
    for (int i = 0; i < a.lanes.k; ++i)
        g.nblocks += (a.lanes.off[i + 1] - a.lanes.off[i] + a.lanes.shift[i] + kLBN - 1) / kLBN;
    g.sm = super_rows(g.mblocks);
    const int64_t nwg = large_workgroups(g.mblocks, g.nblocks);
    const size_t lds = (size_t)LargeShape<BM, BK, ST>::kLdsBytes;
    static std::atomic<uint64_t> lds_done{0};
    const hipError_t e =
        raise_lds_limit((const void *)head_gemm_large_kernel<EPI, BM, BK, ST>, (int)lds, lds_done);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((head_gemm_large_kernel<EPI, BM, BK, ST>), dim3((unsigned)nwg),
                       dim3(kLThreads), lds, s, a, g);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_large_rows(const HeadArgs &a, hipStream_t s)
{
    return large_block_rows(a.B) == 128
               ? launch_large_epi<EPI, 128, kLargeSmallStepK, kLargeSmallStages>(a, s)
               : launch_large_epi<EPI, 256, kLargeStepK, kLargeStages>(a, s);
}

template <int MB, int POL, bool XP = false>
hipError_t launch_mb(const HeadArgs &a, int epi, hipStream_t s)
{
    const int rpg = kRowBlock * MB;
    const int ntiles = a.lanes.tile0[a.lanes.k];
    dim3 grid(((ntiles + 7) / 8) * 8 * ((a.B + rpg - 1) / rpg) * a.kslices);
    const int nsteps = (a.H + kStepK - 1) / kStepK;
    if (XP && nsteps > 0) {
        // the pack launch also clears the call's slice counters
        hipLaunchKernelGGL(pack_hidden_kernel<MB>, dim3(nsteps), dim3(MB * 64), 0, s, a.x,
                           a.ldx, a.B, a.H, a.xp, a.zero);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    } else {
        const hipError_t e = launch_clear(a.zero, s);
        if (e != hipSuccess)
            return e;
    }
    switch (epi) {
    case kEpiPair:
        hipLaunchKernelGGL((head_gemm_kernel<MB, kEpiPair, POL, XP>), grid, dim3(kThreads), 0, s, a);
        break;
    case kEpiPairLse:
        hipLaunchKernelGGL((head_gemm_kernel<MB, kEpiPairLse, POL, XP>), grid, dim3(kThreads), 0, s, a);
        break;
    case kEpiPairLseOut:
        hipLaunchKernelGGL((head_gemm_kernel<MB, kEpiPairLseOut, POL, XP>), grid, dim3(kThreads), 0, s, a);
        break;
    case kEpiShard:
        hipLaunchKernelGGL((head_gemm_kernel<MB, kEpiShard, POL, XP>), grid, dim3(kThreads), 0, s, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Partial completion (row-parallel partials and a registered reduction).
//
// The output is only N columns wide (N / 128 tiles), so the reduction
// dimension is split as well: one workgroup computes a 128-column tile of
// one kPartChunk-row chunk of one lane for 16*MB rows, with the head kernel's
// mainloop (4 waves, K steps interleaved over the waves, wave-order fold
// through LDS), and stores the chunk partial in fp32.  The reduce kernel then
// sums a lane's chunks in ascending order and folds the lanes with the
// registered operator in ascending order, so every output is computed in an
// order fixed by the shapes alone.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_chunk_lane(const PartialArgs &a, int chunk)
{
    int lane = 0;
    while (lane + 1 < a.k && a.chunk0[lane + 1] <= chunk)
        ++lane;
    return lane;
}

template <int MB, int POL>
__global__ __launch_bounds__(kThreads, Occupancy<MB>::kBlocksPerCU) void partial_gemm_kernel(const PartialArgs a)
{
    __shared__ float red[kWaves][kRowBlock][kTileN + 4];

    // workgroup id -> (chunk, tile, row group), row groups innermost
    const int groups = (a.B + kRowBlock * MB - 1) / (kRowBlock * MB);
    const int group = blockIdx.x % groups;
    const int rest = blockIdx.x / groups;
    const int tile = rest % a.T;
    const int chunk = rest / a.T;
    if (chunk >= a.chunk0[a.k])
        return;
    const int lane = find_chunk_lane(a, chunk);
    const int r0 = (chunk - a.chunk0[lane]) * kPartChunk;  // first reduction row in the lane
    const int Hc = min(kPartChunk, a.K[lane] - r0);        // reduction rows of this chunk
    const int c0 = tile * kTileN;
    const int m0 = group * (kRowBlock * MB);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int L = threadIdx.x & 63;
    const int n = L & 15;
    const int g = L >> 4;

    // readable extents from the chunk's first row and the tile's first
    // column (reads past them return zeros); hidden positions >= Hc are
    // masked in registers
    const uint16_t *wbase = a.w[lane] + (int64_t)r0 * a.ldw + c0;
    const int64_t wcols = ((int64_t)(a.N - c0) + 7) & ~(int64_t)7;
    const int64_t wbytes = (((int64_t)(Hc - 1) * a.ldw) + wcols) * 2;
    const int rows_here = min(a.B - m0, kRowBlock * MB);
    const uint16_t *xbase = a.x[lane] + (int64_t)m0 * a.ldx + r0;
    const int64_t xbytes = (((int64_t)(rows_here - 1) * a.ldx) + ((Hc + 7) & ~7)) * 2;

    uint32_t wvo[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        wvo[r] = (uint32_t)(((int64_t)(8 * g + r) * a.ldw + 8 * n) * 2);
    uint32_t xvo[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        xvo[mb] = (uint32_t)(((int64_t)(kRowBlock * mb + n) * a.ldx + 8 * g) * 2);

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[mb][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this wave's steps wave, wave + 4, ... of the chunk, in pairs
    const int nsteps = (Hc + kStepK - 1) / kStepK;
    const int nw = nsteps > wave ? (nsteps - wave + kWaves - 1) / kWaves : 0;
    constexpr int kStride = kWaves * kStepK;
    Frags<MB> fa, fb;
    if (nw > 0)
        load_step<MB, POL>(fa, wbase, wbytes, xbase, xbytes, wave * kStepK, a.ldw, wvo, xvo);
    int k0 = wave * kStepK;
    for (int i = 0; i + 2 <= nw; i += 2) {
        load_step<MB, POL>(fb, wbase, wbytes, xbase, xbytes, k0 + kStride, a.ldw, wvo, xvo);
        compute_step<MB>(fa, acc, k0, Hc, g);
        if (i + 2 < nw)
            load_step<MB, POL>(fa, wbase, wbytes, xbase, xbytes, k0 + 2 * kStride, a.ldw, wvo,
                               xvo);
        compute_step<MB>(fb, acc, k0 + kStride, Hc, g);
        k0 += 2 * kStride;
    }
    if (nw & 1)
        compute_step<MB>(fa, acc, k0, Hc, g);

    // fold the four wave partials (wave order) and store the chunk partial
    const int erow = threadIdx.x >> 4;
    const int cg = threadIdx.x & 15;
    const int col = c0 + 8 * cg;
    const int nvalid = max(0, min(8, a.N - col));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if (m0 + kRowBlock * mb >= a.B)
            break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f32x4 lo = {acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
            const f32x4 hi = {acc[mb][4][r], acc[mb][5][r], acc[mb][6][r], acc[mb][7][r]};
            *reinterpret_cast<f32x4 *>(&red[wave][4 * g + r][8 * n]) = lo;
            *reinterpret_cast<f32x4 *>(&red[wave][4 * g + r][8 * n + 4]) = hi;
        }
        __syncthreads();
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            y[j] = ((red[0][erow][8 * cg + j] + red[1][erow][8 * cg + j]) +
                    red[2][erow][8 * cg + j]) + red[3][erow][8 * cg + j];
        __syncthreads();
        const int b = m0 + kRowBlock * mb + erow;
        if (b < a.B) {
            float *dst = a.part + ((int64_t)chunk * a.B + b) * a.ldp + col;
            if (nvalid == 8) {
                *reinterpret_cast<f32x4 *>(dst) = f32x4{y[0], y[1], y[2], y[3]};
                *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{y[4], y[5], y[6], y[7]};
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (j < nvalid)
                        dst[j] = y[j];
            }
        }
    }
}

// The registered operator on two partials.  Minimum and maximum propagate
// NaN (IEEE 754-2019 minimum / maximum: v_minimum_f32 / v_maximum_f32), as
// numpy's and torch's do.
__device__ __forceinline__ f32x4 reduce_op(int op, f32x4 a, f32x4 b)
{
    switch (op) {
    case kRedSum:
        return a + b;
    case kRedProd:
        return a * b;
    case kRedMin:
        return __builtin_elementwise_minimum(a, b);
    default:
        return __builtin_elementwise_maximum(a, b);
    }
}

// A workgroup covers kThreads / SPLIT * 4 columns of one row: thread (q, j)
// takes column quad q and, of every lane, the chunks j, j + SPLIT, ...
// (ascending); the SPLIT part sums of a lane are added in the fixed order
// ((s0 + s1) + s2) + ... through LDS, and the lanes are folded with the
// operator in ascending lane order.  ldp is a multiple of 4, so a quad is one
// aligned vector (columns past N are never stored).  SPLIT is 8 for batches
// of up to 32 rows and 4 above (chosen from B alone, so the order is fixed
// by the shapes): the down projection at B = 16 took 36.2-36.4 us with 8
// against 37.6-37.9 us with 4, and at B = 64 55.4-55.9 against 54.0-54.7 us.
template <int SPLIT>
__global__ __launch_bounds__(kThreads) void partial_reduce_kernel(const PartialArgs a, int op,
                                                                  float *out, int64_t ldo)
{
    constexpr int kQuads = kThreads / SPLIT;
    __shared__ f32x4 sums[SPLIT][kQuads];
    const int b = blockIdx.y;
    const int q = threadIdx.x % kQuads;
    const int j = threadIdx.x / kQuads;
    const int col = blockIdx.x * (kQuads * 4) + 4 * q;
    const bool colok = col < a.N;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int lane = 0; lane < a.k; ++lane) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if (colok) {
            const float *p = a.part + ((int64_t)a.chunk0[lane] * a.B + b) * a.ldp + col;
            const int64_t stride = (int64_t)a.B * a.ldp;
            const int nc = a.chunk0[lane + 1] - a.chunk0[lane];
            int c = j;
            // four independent loads in flight, added in ascending chunk order
            for (; c + 3 * SPLIT < nc; c += 4 * SPLIT) {
                const f32x4 v0 = *reinterpret_cast<const f32x4 *>(p + c * stride);
                const f32x4 v1 = *reinterpret_cast<const f32x4 *>(p + (c + SPLIT) * stride);
                const f32x4 v2 = *reinterpret_cast<const f32x4 *>(p + (c + 2 * SPLIT) * stride);
                const f32x4 v3 = *reinterpret_cast<const f32x4 *>(p + (c + 3 * SPLIT) * stride);
                s = (((s + v0) + v1) + v2) + v3;
            }
            for (; c < nc; c += SPLIT)
                s += *reinterpret_cast<const f32x4 *>(p + c * stride);
        }
        sums[j][q] = s;
        __syncthreads();
        if (j == 0) {
            f32x4 t = sums[0][q];
#pragma unroll
            for (int u = 1; u < SPLIT; ++u)
                t += sums[u][q];
            acc = lane == 0 ? t : reduce_op(op, acc, t);
        }
        __syncthreads();
    }
    if (j != 0 || !colok)
        return;
    float *dst = out + (int64_t)b * ldo + col;
    if (col + 4 <= a.N) {
        *reinterpret_cast<f32x4 *>(dst) = acc;
    } else {
        for (int e = 0; e < 4 && col + e < a.N; ++e)
            dst[e] = acc[e];
    }
}

template <int MB, int POL>
hipError_t launch_partial_mb(const PartialArgs &a, hipStream_t s)
{
    const int groups = (a.B + kRowBlock * MB - 1) / (kRowBlock * MB);
    const int64_t nwg = (int64_t)a.chunk0[a.k] * a.T * groups;
    hipLaunchKernelGGL((partial_gemm_kernel<MB, POL>), dim3((unsigned)nwg), dim3(kThreads), 0, s,
                       a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_head_gemm(const HeadArgs &a, int epi, hipStream_t s)
{
    if (a.B <= 0 || a.T <= 0)
        return hipSuccess;
    // one row group: every weight tile is read once, so stream it
    switch (rows_per_group(a.B) / kRowBlock) {
    case 1:
        return launch_mb<1, kPolicyStream>(a, epi, s);
    case 2:
        return launch_mb<2, kPolicyStream>(a, epi, s);
    default:
        // more than one row group is the large-batch kernel's
        if (a.B > kRowBlock * kMaxMB)
            return hipErrorInvalidValue;
        return launch_mb<kMaxMB, kPolicyStream, true>(a, epi, s);
    }
}

hipError_t launch_head_gemm_large(const HeadArgs &a, int epi, hipStream_t s)
{
    if (a.B <= 0 || a.T <= 0)
        return hipSuccess;
    switch (epi) {
    case kEpiPair:
        return launch_large_rows<kEpiPair>(a, s);
    case kEpiPairLse:
        return launch_large_rows<kEpiPairLse>(a, s);
    case kEpiPairLseOut:
        return launch_large_rows<kEpiPairLseOut>(a, s);
    case kEpiShard:
        return launch_large_rows<kEpiShard>(a, s);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_combine(const int2 *pair, const float2 *mse, const LaneTable &lanes,
                          int32_t B, int32_t T, int32_t *ids, float *lse, float *sel_lp,
                          int32_t *lane_ids, float *lane_max, hipStream_t s)
{
    if (B <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(B), dim3(kThreads), 0, s, pair, mse, lanes, T, ids,
                       lse, sel_lp, lane_ids, lane_max);
    return hipGetLastError();
}

hipError_t launch_normalize(float *lp, int64_t ld, const float *lse, int32_t B, int32_t V,
                            hipStream_t s)
{
    if (B <= 0 || V <= 0)
        return hipSuccess;
    static std::atomic<uint64_t> lds_done{0};
    const hipError_t e = raise_lds_limit((const void *)normalize_kernel, kNormLdsBytes, lds_done);
    if (e != hipSuccess)
        return e;
    for (int32_t r0 = 0; r0 < B; r0 += kMaxGridRows) {
        const dim3 grid((V + kNormCols - 1) / kNormCols, min(B - r0, kMaxGridRows));
        hipLaunchKernelGGL(normalize_kernel, grid, dim3(kThreads), kNormLdsBytes, s,
                           lp + (int64_t)r0 * ld, ld, lse + r0, V);
        const hipError_t el = hipGetLastError();
        if (el != hipSuccess)
            return el;
    }
    return hipSuccess;
}

hipError_t launch_reconstruct(const LaneTable &lanes, int32_t B, float *logits, int64_t ldl,
                              hipStream_t s)
{
    if (B <= 0)
        return hipSuccess;
    int maxv = 0;
    for (int i = 0; i < lanes.k; ++i)
        maxv = max(maxv, lanes.off[i + 1] - lanes.off[i]);
    LaneTable part = lanes;
    for (int32_t r0 = 0; r0 < B; r0 += kMaxGridRows) {
        for (int i = 0; i < lanes.k; ++i)
            part.shard[i] = lanes.shard[i] + (int64_t)r0 * lanes.shard_ld[i];
        const dim3 grid((maxv + 4 * kThreads - 1) / (4 * kThreads), min(B - r0, kMaxGridRows),
                        lanes.k);
        hipLaunchKernelGGL(reconstruct_kernel, grid, dim3(kThreads), 0, s, part,
                           logits + (int64_t)r0 * ldl, ldl);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_row_argmax(const float *logits, int64_t ldl, int32_t B, int32_t V,
                             int2 *partial, int32_t *ids, hipStream_t s)
{
    if (B <= 0)
        return hipSuccess;
    const int nchunks = (V + kArgmaxChunk - 1) / kArgmaxChunk;
    for (int32_t r0 = 0; r0 < B; r0 += kMaxGridRows) {
        hipLaunchKernelGGL(row_argmax_kernel, dim3(nchunks, min(B - r0, kMaxGridRows)),
                           dim3(kThreads), 0, s, logits + (int64_t)r0 * ldl, ldl, V, nchunks,
                           partial + (int64_t)r0 * nchunks);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    LaneTable one = {};
    one.k = 1;
    one.off[0] = 0;
    one.off[1] = V;
    one.tile0[0] = 0;
    one.tile0[1] = nchunks;
    return launch_combine(partial, nullptr, one, B, nchunks, ids, nullptr, nullptr, nullptr,
                          nullptr, s);
}

hipError_t launch_partial_gemm(const PartialArgs &a, hipStream_t s)
{
    if (a.B <= 0 || a.chunk0[a.k] <= 0)
        return hipSuccess;
    // one row group: every weight byte is read once, so stream it
    switch (rows_per_group(a.B) / kRowBlock) {
    case 1:
        return launch_partial_mb<1, kPolicyStream>(a, s);
    case 2:
        return launch_partial_mb<2, kPolicyStream>(a, s);
    default:
        if (a.B <= kRowBlock * kMaxMB)
            return launch_partial_mb<kMaxMB, kPolicyStream>(a, s);
        return launch_partial_mb<kMaxMB, kPolicyShared>(a, s);
    }
}

hipError_t launch_partial_reduce(const PartialArgs &a, int op, float *out, int64_t ldo,
                                 hipStream_t s)
{
    if (a.B <= 0)
        return hipSuccess;
    if (op < kRedSum || op > kRedMax)
        return hipErrorInvalidValue;
    if (a.B <= 32) {
        constexpr int cols = kThreads / 8 * 4;
        hipLaunchKernelGGL(partial_reduce_kernel<8>, dim3((a.N + cols - 1) / cols, a.B),
                           dim3(kThreads), 0, s, a, op, out, ldo);
        return hipGetLastError();
    }
    // Slices of kMaxGridRows rows: the kernel finds row b of chunk c at
    // part + (c * a.B + b) * ldp, so moving part and out by r0 rows (a.B
    // unchanged) makes y index b stand for row r0 + b.
    constexpr int cols = kThreads / 4 * 4;
    PartialArgs slice = a;
    for (int32_t r0 = 0; r0 < a.B; r0 += kMaxGridRows) {
        slice.part = a.part + (int64_t)r0 * a.ldp;
        hipLaunchKernelGGL(partial_reduce_kernel<4>,
                           dim3((a.N + cols - 1) / cols, min(a.B - r0, kMaxGridRows)),
                           dim3(kThreads), 0, s, slice, op, out + (int64_t)r0 * ldo, ldo);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

int64_t head_launch_items(int32_t B, int32_t H, int32_t V, const int32_t *lane_off, int32_t k)
{
    if (B <= 0)
        return 0;
    int64_t tiles = 0, nblocks = 0;
    for (int i = 0; i < k; ++i) {
        const int64_t vi = (int64_t)lane_off[i + 1] - lane_off[i];
        tiles += (vi + kMaxShift + kTileN - 1) / kTileN;
        nblocks += (vi + kMaxShift + kLBN - 1) / kLBN;
    }
    // the combine launches: one workgroup per row
    int64_t items = (int64_t)B * kThreads;
    if (B >= kLargeBatch) {
        const int mblocks = (B + large_block_rows(B) - 1) / large_block_rows(B);
        items = std::max<int64_t>(items, large_workgroups(mblocks, nblocks) * kLThreads);
    } else {
        items = std::max<int64_t>(items, (tiles + 7) / 8 * 8 * k_slices(B, H, V) * kThreads);
    }
    return items;
}

int64_t partial_launch_items(int32_t B, int32_t N, int32_t chunks)
{
    if (B <= 0)
        return 0;
    const int64_t T = (N + kTileN - 1) / kTileN;
    const int64_t groups = (B + rows_per_group(B) - 1) / rows_per_group(B);
    return (int64_t)chunks * T * groups * kThreads;
}

// ---------------------------------------------------------------------------
// Static scratch of sb_project_tokens_static.  In host code the array's name
// is only a stand-in for its device address: the address of each device's
// copy comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kScratchDevices = 64;

hipError_t static_scratch(int device, void **ptr)
{
    static std::atomic<void *> addr[kScratchDevices];  // zero-initialised
    const bool cached = device >= 0 && device < kScratchDevices;
    if (cached) {
        void *p = addr[device].load(std::memory_order_acquire);
        if (p) {
            *ptr = p;
            return hipSuccess;
        }
    }
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess)
        return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess)
            e = e2;
    }
    if (e != hipSuccess)
        return e;
    if (!p)
        return hipErrorInvalidSymbol;
    if (cached)
        addr[device].store(p, std::memory_order_release);  // racing first calls store the same
    *ptr = p;
    return hipSuccess;
}

}  // namespace sbk
