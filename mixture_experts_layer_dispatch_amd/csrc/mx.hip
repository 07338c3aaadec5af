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
// A block owns up to QT_RB consecutive 32-row blocks of one group (a chunk of
// at most 128 rows; the grid row of the chunk's first row block does the
// chunk, the others return) and a segment of `steps` x 256 bytes of every
// row, walked in steps of 256 bytes.  Set-up: the block's group is found by
// every thread testing some groups against the block-count prefix at once
// (one memory round trip; a binary search took ten dependent ones and
// dominated the kernel), then the chunk's source rows are resolved once (a
// thread per row looks up its slot and weight).  Each step stages the
// chunk's rows x 256 bytes in LDS (16-byte loads, the next step's in flight
// while this one is quantised), and each thread then takes 16 rows of one
// column: two neighbouring lanes hold a 32-row block and agree on its scale.
// Consecutive lanes write consecutive 16-byte runs of the transposed output,
// so a group of at most 128 rows comes out as one contiguous run per step.
constexpr int QT_RB = 4;

template <bool F32>            // fp32 source rows (src.kind == 1), else bf16
__global__ __launch_bounds__(256) void k_mx_quant_group_t(PadGroups g, QtSrc src, int C,
                                                          int steps, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    using T = typename std::conditional<F32, float, uint16_t>::type;
    constexpr int EPP = 16 / sizeof(T);               // elements per 16-byte piece
    constexpr int CB = 256 / sizeof(T);               // columns per step
    // LDS: row q at q * CB + (q / 16) * GP elements: rows are 256 bytes (16-byte
    // aligned pieces), and each 16-row group is shifted by 8 banks, so the
    // lanes of a wave, which read the same row offset of different 16-row
    // groups, spread over the banks
    constexpr int GP = 32 / sizeof(T);
    constexpr int RM = 32 * QT_RB;
    __shared__ int64_t roff[RM];      // element offset of row q in the source; -1: a zero row
    __shared__ float rwt[RM];         // the row's factor (the slot's weight for w * dy, else 1)
    __shared__ int grp[4];            // first block, padded rows, first row, end row of the group
    __shared__ __attribute__((aligned(16))) T tile[RM * CB + (RM / 16) * GP];
    auto tix = [](int q, int col) { return q * CB + (q >> 4) * GP + col; };
    const int b = blockIdx.y;
    if (threadIdx.x == 0) grp[0] = -1;
    __syncthreads();
    if (!g.blk_off) {
        if (threadIdx.x == 0 && b * 32 < g.dense_rows) {
            grp[0] = 0;
            grp[1] = 32 * ((g.dense_rows + 31) / 32);
            grp[2] = 0;
            grp[3] = g.dense_rows;
        }
    } else {
        for (int e = threadIdx.x; e < g.E; e += 256) {
            const int a = g.blk_off[e], z = g.blk_off[e + 1];
            if (a <= b && b < z) {                     // exactly one group holds block b
                grp[0] = a;
                grp[1] = 32 * (z - a);
                grp[2] = g.off[e];
                grp[3] = g.off[e + 1];
            }
        }
    }
    __syncthreads();
    const int boff = grp[0], np = grp[1], lo = grp[2], hi = grp[3];
    if (boff < 0) return;
    if (lo < 0 || hi < lo || hi > (g.blk_off ? g.rows : g.dense_rows)) return;   // reported by the tile prefix
    const int bl = b - boff;
    if (bl % QT_RB) return;
    const int nbl = min(QT_RB, np / 32 - bl);
    const int R = 32 * nbl, r0 = lo + 32 * bl, nrest = hi - r0;
    const int64_t gcode = 32LL * boff * C;
    if (threadIdx.x < R) {
        const int q = threadIdx.x, r = r0 + q;
        int64_t off = -1;
        float wt = 1.f;
        if (q < nrest) {
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
    const T* base;
    if constexpr (F32) base = src.f32;
    else base = src.b16;
    // step loads: R rows x 16 pieces, eight per thread (rows past R skipped)
    constexpr int PPT = RM * 16 / 256;
    uint4 pc[PPT];
    auto load = [&](int c0) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = threadIdx.x + 256 * i, q = p >> 4, col = c0 + (p & 15) * EPP;
            const int64_t o = q < R ? roff[q] : -1;
            pc[i] = (o >= 0 && col < C) ? *(const uint4*)(base + o + col) : make_uint4(0, 0, 0, 0);
        }
    };
    const int cs0 = blockIdx.x * steps * CB;
    const int nst = min(steps, (C - cs0 + CB - 1) / CB);
    const int units = CB * (R / 16);                  // (column, 16-row group) pairs per step
    load(cs0);
    for (int st = 0; st < nst; ++st) {
        const int c0 = cs0 + st * CB;
        __syncthreads();                              // the previous step's readers are done
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = threadIdx.x + 256 * i, q = p >> 4;
            if (q < R) *(uint4*)(tile + tix(q, (p & 15) * EPP)) = pc[i];
        }
        __syncthreads();
        if (st + 1 < nst) load(c0 + CB);
        for (int u = threadIdx.x; u < units; u += 256) {   // units is a multiple of 64: whole waves
            const int rg = u % (R / 16), cl = u / (R / 16);
            float v[16];
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = 16 * rg + i;
                float x;
                if constexpr (F32) x = tile[tix(q, cl)];
                else x = bf2f(tile[tix(q, cl)]) * rwt[q];
                v[i] = x;
                amax = fmaxf(amax, fabsf(x));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 1));   // the other half of the 32-row block
            const int s = mx_scale_exp(amax);
            const int c = c0 + cl;
            if (c < C) {
                uint4 w;
                w.x = e4m3_pack4(v, s);
                w.y = e4m3_pack4(v + 4, s);
                w.z = e4m3_pack4(v + 8, s);
                w.w = e4m3_pack4(v + 12, s);
                *(uint4*)(codes + gcode + (int64_t)c * np + 32 * bl + 16 * rg) = w;
                if ((rg & 1) == 0) scales[gcode / 32 + (int64_t)c * (np / 32) + bl + rg / 2] = (uint8_t)(s + 127);
            }
        }
    }
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
    // Steps per block: as many as leave at least 4096 working blocks (16 per
    // CU over the launch; the group search and row look-ups are paid once per block, so
    // longer segments help while there are blocks to spare; measured at
    // 2048 tokens x 512 experts, where a step of 8 was 20 % faster than 1,
    // and at 8 experts x 2560 rows, where the source rows come from HBM
    // and each chunk needs its column segments read side by side: 1 step
    // was 2x faster than 4).  Chunks are estimated from the mean group.
    const int cb = src.kind == 1 ? 64 : 128;               // columns per step
    const int64_t rows = g.blk_off ? g.rows : g.dense_rows;
    const int64_t chunks = (g.blk_off && rows <= 128LL * g.E) ? (rows < g.E ? rows : g.E) : (rows + 127) / 128;
    const int64_t total = chunks * ((C + cb - 1) / cb);
    // Source rows that do not stay in cache (gathered token rows past 64 MB,
    // fp32 rows past 256 MB) come from HBM, where a chunk's column segments
    // must be read side by side: one step per block (the 65 536-token
    // stream's x and w*dy operands, 134 MB per macrobatch: 2.33 ms per layer
    // step with eight steps per block, 1.71 with one).
    const int64_t src_rows = src.kind == 1 ? rows : (src.kind == 3 ? g.dense_rows : rows / src.k);
    const int64_t src_bytes = src_rows * src.ld * (src.kind == 1 ? 4 : 2);
    const bool from_hbm = src_bytes > (src.kind == 1 ? (256LL << 20) : (64LL << 20));
    int steps = 1;
    while (!from_hbm && steps < 8 && total / (2 * steps) >= 4096) steps *= 2;
    dim3 grid((C + steps * cb - 1) / (steps * cb), nblk);
    if (src.kind == 1)
        k_mx_quant_group_t<true><<<grid, 256, 0, st>>>(g, src, C, steps, (uint8_t*)codes, (uint8_t*)scales);
    else
        k_mx_quant_group_t<false><<<grid, 256, 0, st>>>(g, src, C, steps, (uint8_t*)codes, (uint8_t*)scales);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
