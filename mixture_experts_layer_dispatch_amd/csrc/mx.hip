// MXFP8 quantisation kernels: weights along either axis (ahead of time, as the
// pages describe: alphalab.site "Mixture-of-Kittens" section 三, weights are
// quantised outside the timed region), and the activations: x and dy along H
// once per token (the dispatch and the reverse-combine gather these codes on
// load), and the row-block transposes of the weight-gradient operands
// (arex-research.com "Cursor 放出 MoK", design section, closing paragraph:
// activation quantisation is fused into dispatch, the GEMMs and SwiGLU).
#include <type_traits>

#include "launch.h"
#include "mx.h"
#include "profile.h"

namespace moe {

// ------------------------------------------------------------------ rows
// X [R, K] bf16 -> codes [R, K] e4m3, scales e8m0, blocks along K.
// Scales are [R, K/32] (kmaj_rows == 0), or K-step-major per matrix of
// kmaj_rows rows: the four scales of row r's K step j (codes 128j..128j+127)
// form word j * kmaj_rows + r, so one K step of consecutive rows is contiguous.
// A thread owns 8 consecutive elements; four neighbouring threads share a
// block and agree on its maximum through two lane exchanges.
__global__ __launch_bounds__(256) void k_mx_quant_rows(const uint4* __restrict__ x, int64_t n8, int K,
                                                       int kmaj_rows, uint2* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool ok = i < n8;
    float v[8];
    if (ok) {
        const uint4 w = x[i];
        v[0] = lo_bf(w.x); v[1] = hi_bf(w.x); v[2] = lo_bf(w.y); v[3] = hi_bf(w.y);
        v[4] = lo_bf(w.z); v[5] = hi_bf(w.z); v[6] = lo_bf(w.w); v[7] = hi_bf(w.w);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int s = mx_scale_exp(amax);
    if (ok) {
        codes[i] = e4m3_pack8(v, s);
        if ((i & 3) == 0) {
            int64_t at = i >> 2;
            if (kmaj_rows > 0) {
                const int nb = K / 32;
                const int64_t row = at / nb;
                const int b = (int)(at - row * nb);
                const int64_t mat = row / kmaj_rows, r = row - mat * kmaj_rows;
                at = mat * kmaj_rows * nb + ((int64_t)(b >> 2) * kmaj_rows + r) * 4 + (b & 3);
            }
            scales[at] = (uint8_t)(s + 127);
        }
    }
}

// ------------------------------------------------------------------ columns
// W [R, C] bf16 (per matrix of a batch) -> codes [C, R]: blocks of 32
// consecutive rows of one column, written transposed so that the block is
// contiguous; scales K-step-major over the C rows of the transposed matrix
// (the scale of row c, block b at byte ((b / 4) * C + c) * 4 + b % 4).
// A thread owns one column of a 32-row band.
__global__ __launch_bounds__(256) void k_mx_quant_cols(const uint16_t* __restrict__ w, int R, int C,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
    const int64_t mat = blockIdx.z;
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int r0 = blockIdx.y * 32;
    if (c >= C) return;
    const uint16_t* src = w + mat * R * (int64_t)C + (int64_t)r0 * C + c;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
        v[q] = bf2f(src[(int64_t)q * C]);
        amax = fmaxf(amax, fabsf(v[q]));
    }
    const int s = mx_scale_exp(amax);
    uint32_t wds[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) wds[q] = e4m3_pack4(v + 4 * q, s);
    uint4* dst = (uint4*)(codes + mat * R * (int64_t)C + (int64_t)c * R + r0);
    dst[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    dst[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
    const int b = blockIdx.y;
    scales[mat * (int64_t)C * (R / 32) + ((int64_t)(b >> 2) * C + c) * 4 + (b & 3)] = (uint8_t)(s + 127);
}

// ------------------------------------------------------------------ MXFP4 rows
// W [R, K] bf16 -> E2M1 codes [R, K/2] (two per byte, the even element in the
// low nibble) and E8M0 scales, blocks of 32 along K, K-step-major per matrix
// of kmaj_rows rows as the MXFP8 weights ([K/128, rows, 4]).  A thread owns 8
// consecutive elements; four neighbouring threads share a block.
__global__ __launch_bounds__(256) void k_mx4_quant_rows(const uint4* __restrict__ x, int64_t n8, int K,
                                                        int kmaj_rows, uint32_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool ok = i < n8;
    float v[8];
    if (ok) {
        const uint4 w = x[i];
        v[0] = lo_bf(w.x); v[1] = hi_bf(w.x); v[2] = lo_bf(w.y); v[3] = hi_bf(w.y);
        v[4] = lo_bf(w.z); v[5] = hi_bf(w.z); v[6] = lo_bf(w.w); v[7] = hi_bf(w.w);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int s = mx4_scale_exp(amax);
    if (ok) {
        codes[i] = e2m1_pack8(v, s);
        if ((i & 3) == 0) {
            const int nb = K / 32;
            const int64_t blk = i >> 2;
            const int64_t row = blk / nb;
            const int b = (int)(blk - row * nb);
            const int64_t mat = row / kmaj_rows, r = row - mat * kmaj_rows;
            scales[mat * kmaj_rows * nb + ((int64_t)(b >> 2) * kmaj_rows + r) * 4 + (b & 3)] = (uint8_t)(s + 127);
        }
    }
}

// ------------------------------------------------------------------ group transpose
// For the weight gradients, whose reduction runs over an expert's rows: rows of
// each expert group, in 32-row blocks (the last one zero-padded), are quantised
// along the row axis and written transposed, group by group: group e (with
// n_e rows padded to np_e = 32 * ceil(n_e / 32)) owns the contiguous block
// starting at code 32 * blk_off[e] * C, laid out [C][np_e], and its scales
// start at blk_off[e] * C, laid out [C][np_e / 32].
struct PadBlock {
    int r0, nv;                // first local row, valid rows of this 32-row block
    int64_t gcode;             // first code of the group's block
    int np;                    // padded rows of the group
    int bl;                    // block index inside the group
};

__device__ __forceinline__ bool map_pad_block(const PadGroups& g, int C, int b, PadBlock& o) {
    if (!g.blk_off) {
        if (b * 32 >= g.dense_rows) return false;
        o.r0 = b * 32;
        o.nv = min(32, g.dense_rows - o.r0);
        o.gcode = 0;
        o.np = 32 * ((g.dense_rows + 31) / 32);
        o.bl = b;
        return true;
    }
    if (b >= g.blk_off[g.E]) return false;
    int a = 0, z = g.E;
    while (z - a > 1) {
        const int mid = (a + z) >> 1;
        if (g.blk_off[mid] <= b) a = mid;
        else z = mid;
    }
    const int lo = g.off[a], hi = g.off[a + 1];
    if (lo < 0 || hi < lo || hi > g.rows) return false;   // reported by the tile prefix
    o.bl = b - g.blk_off[a];
    o.r0 = lo + o.bl * 32;
    o.nv = min(32, hi - o.r0);
    o.gcode = 32LL * g.blk_off[a] * C;
    o.np = 32 * (g.blk_off[a + 1] - g.blk_off[a]);
    return o.nv > 0;
}

// A block quantises one 32-row block of a group over 256 columns.  Its 32
// source rows are resolved once (threads 0..31 look up their slots and
// weights); the 32 x 256 tile is then read row-wise in 16-byte pieces into
// LDS, and each thread takes one column of it: 32 values, one scale, 32 codes.
constexpr int QT_COLS = 256;

template <bool F32>            // fp32 source rows (src.kind == 1), else bf16
__global__ __launch_bounds__(256) void k_mx_quant_group_t(PadGroups g, QtSrc src, int C,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    using T = typename std::conditional<F32, float, uint16_t>::type;
    constexpr int EPC = 16 / sizeof(T);               // elements per 16-byte piece
    constexpr int PPR = QT_COLS / EPC;                // pieces per row
    __shared__ int64_t roff[32];      // element offset of row q in the source; -1: a zero row
    __shared__ float rwt[32];         // the row's factor (the slot's weight for w * dy, else 1)
    __shared__ __attribute__((aligned(16))) T tile[32 * QT_COLS];
    PadBlock pb;
    if (!map_pad_block(g, C, blockIdx.y, pb)) return;         // the same for the whole block
    if (threadIdx.x < 32) {
        const int q = threadIdx.x, r = pb.r0 + q;
        int64_t off = -1;
        float wt = 1.f;
        if (q < pb.nv) {
            if (src.kind == 1) {
                off = (int64_t)r * src.ld;
            } else if (src.kind == 3) {
                off = (int64_t)(src.row0 + r) * src.ld;
            } else {
                const int slot = src.slot_of_row[src.grow0 + r];
                if ((unsigned)slot >= (unsigned)src.S) {
                    raise_err(g.err, ERR_BAD_SLOT);
                } else {
                    off = (int64_t)(slot / src.k) * src.ld;
                    if (src.kind == 0) wt = src.topk_w[slot];
                }
            }
        }
        roff[q] = off;
        rwt[q] = wt;
    }
    __syncthreads();
    const int c0 = blockIdx.x * QT_COLS;
    const T* base;
    if constexpr (F32) base = src.f32;
    else base = src.b16;
    uint4 piece[32 * PPR / 256];
#pragma unroll
    for (int i = 0; i < 32 * PPR / 256; ++i) {
        const int idx = threadIdx.x + 256 * i, q = idx / PPR, col = c0 + (idx % PPR) * EPC;
        const int64_t o = roff[q];
        piece[i] = (o >= 0 && col < C) ? *(const uint4*)(base + o + col) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 32 * PPR / 256; ++i) {
        const int idx = threadIdx.x + 256 * i;
        *(uint4*)(tile + (idx / PPR) * QT_COLS + (idx % PPR) * EPC) = piece[i];
    }
    __syncthreads();
    const int c = c0 + threadIdx.x;
    if (c >= C) return;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
        float x;
        if constexpr (F32) x = tile[q * QT_COLS + threadIdx.x];
        else x = bf2f(tile[q * QT_COLS + threadIdx.x]) * rwt[q];
        v[q] = x;
        amax = fmaxf(amax, fabsf(x));
    }
    const int s = mx_scale_exp(amax);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = e4m3_pack4(v + 4 * q, s);
    uint4* dst = (uint4*)(codes + pb.gcode + (int64_t)c * pb.np + 32 * pb.bl);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    scales[pb.gcode / 32 + (int64_t)c * (pb.np / 32) + pb.bl] = (uint8_t)(s + 127);
}

// ------------------------------------------------------------------ launchers
int launch_mx_quant_rows(const void* x, int64_t rows, int K, void* codes, void* scales, hipStream_t st,
                         int kmaj_rows) {
    ProfScope prof_(st, "mx_quant_rows");
    const int64_t n8 = rows * (int64_t)K / 8;
    if (n8 <= 0) return 0;
    k_mx_quant_rows<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>((const uint4*)x, n8, K, kmaj_rows,
                                                                 (uint2*)codes, (uint8_t*)scales);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mx4_quant_rows(const void* w, int64_t rows, int K, int kmaj_rows, void* codes, void* scales,
                          hipStream_t st) {
    ProfScope prof_(st, "mx4_quant_rows");
    const int64_t n8 = rows * (int64_t)K / 8;
    if (n8 <= 0) return 0;
    k_mx4_quant_rows<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>((const uint4*)w, n8, K, kmaj_rows,
                                                                  (uint32_t*)codes, (uint8_t*)scales);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mx_quant_cols(const void* w, int batch, int R, int C, void* codes, void* scales,
                         hipStream_t st) {
    ProfScope prof_(st, "mx_quant_cols");
    dim3 grid((C + 255) / 256, R / 32, batch);
    k_mx_quant_cols<<<grid, 256, 0, st>>>((const uint16_t*)w, R, C, (uint8_t*)codes, (uint8_t*)scales);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mx_quant_group_t(const PadGroups& g, const QtSrc& src, int C, void* codes, void* scales,
                            hipStream_t st) {
    static const char* names[4] = {"mx_qt_wdy", "mx_qt_f32", "mx_qt_x", "mx_qt_dense"};
    ProfScope prof_(st, names[src.kind & 3]);
    int nblk;
    if (!g.blk_off) {
        nblk = (g.dense_rows + 31) / 32;
    } else {
        const int64_t bound = ((int64_t)g.rows + 31LL * g.E) / 32;
        nblk = (int)(bound < g.rows ? bound : g.rows);
    }
    if (nblk <= 0) return 0;
    dim3 grid((C + QT_COLS - 1) / QT_COLS, nblk);
    if (src.kind == 1) k_mx_quant_group_t<true><<<grid, 256, 0, st>>>(g, src, C, (uint8_t*)codes, (uint8_t*)scales);
    else k_mx_quant_group_t<false><<<grid, 256, 0, st>>>(g, src, C, (uint8_t*)codes, (uint8_t*)scales);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
