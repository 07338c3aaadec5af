// Expert-grouped GEMMs of the SwiGLU FFN, forward and backward, on MFMA.
//
// alphalab.site "Mixture-of-Kittens", section 一: each expert runs a SwiGLU
// FFN on the tokens routed to it (gate/up projection, SiLU(g) * u, down
// projection), and the backward computes the expert gradients;
// arex-research.com "Cursor 放出 MoK", design section: the GEMMs are grouped by
// expert, and the router-weight gradient is fused into the SwiGLU backward
// (closing paragraph).
//
// Two grouping shapes:
//   M-grouped  C_e[rows of e, N] = A[rows of e, K] * B_e[N, K]^T   (forward,
//              input gradients): the row count of each expert is dynamic; the
//              grid covers an upper bound of row tiles and each block finds its
//              (expert, row tile) by binary search over a device-side tile
//              prefix, so no count ever reaches the host.
//   K-grouped  C_e[M, N] = sum over rows r of e of A[r, M] (x) B[r, N]
//              (weight gradients): M and N fixed, the reduction runs over the
//              expert's rows in ascending order.
//
// Tiles: 256 threads = 4 waves in a 2 x 2 grid, each wave (TM/2) x (TN/2).
// Both operands are staged through LDS in a [row][k] layout (unpadded
// 128-byte rows with XOR-swizzled 16-byte chunks, so the 16 rows read by one
// MFMA fragment hit 16 different 16-byte bank groups), double-buffered with
// one barrier per K step.
// Operands whose reduction index is the slow memory axis are copied into LDS
// as they lie ([k][row], KS tiles) and read with gfx950's LDS transpose load,
// which hands each lane four consecutive k of one row.
// The MFMA is issued with the B tile as its first operand, so each lane's four
// accumulators are four consecutive output columns (8-byte stores).
// Each output element is a fixed-order fp32 sum: K steps ascend, and the
// MFMA's internal order is fixed, so results are identical run to run and do
// not depend on which other rows share the tile.
#include "gemm_common.h"
#include "profile.h"

namespace moe {

// ================================================================ forward GEMM 1
// g = X W_gate^T, u = X W_up^T, h = SiLU(g) * u; g, u saved (bf16), h to the
// ring.  Tile: TM rows x (TN/2 gate + TN/2 up columns).
//
// Row tiles (TM): 64 when groups are small (each weight byte is then read by
// one or two tiles and the GEMM streams weights; four-wave blocks, 64 + 64
// columns), 128 when the groups are large enough for the GEMM to be MFMA work
// (eight-wave blocks, 128 + 128 columns, one block per CU, loads two K steps
// ahead).  Each wave computes (TM/2) x 64: 32 gate and the matching 32 up
// columns.
template <int TM> struct GateUpShape;
template <> struct GateUpShape<64> { static constexpr int TN = 128, NTHR = 256; };
template <> struct GateUpShape<128> { static constexpr int TN = 256, NTHR = 512; };

template <int TM>
constexpr int gate_up_lds() {
    return TM == 64 ? lds_two_blocks(2 * Smem<64, 128, false, false>::STAGE) : 2 * SmemW8<128, 256>::STAGE;
}

template <int TM>
__global__ __launch_bounds__(GateUpShape<TM>::NTHR, TM == 64 ? 2 : 1) void k_gemm_gate_up(GemmGateUpArgs a) {
    constexpr int TN = GateUpShape<TM>::TN, NTHR = GateUpShape<TM>::NTHR;
    __shared__ __attribute__((aligned(16))) uint16_t smem[gate_up_lds<TM>()];
    int e, lo, hi, nt;
    if (!map_mtile<TM>(a.g, a.I / (TN / 2), blockIdx.x, e, lo, hi, nt)) return;
    const int i0 = nt * (TN / 2);
    f32x4 acc[TM / 32][4];
    const int nk = a.H / kTK;
    const uint16_t* wg = a.w_gate + (int64_t)e * a.I * a.H;
    const uint16_t* wu = a.w_up + (int64_t)e * a.I * a.H;
    RowsGateUp sb{wg, wu, a.H, i0};
    LoadKC<TN, RowsGateUp, NTHR> lb(sb);
    auto run = [&](auto& la) {
        if constexpr (TM == 64) mainloop<TM, TN, false, false>(la, lb, nk, smem, acc);
        else mainloop_w8<TM, TN>(la, lb, nk, smem, acc);
    };
    if (a.x_gather) {
        RowsGather sa{a.x, a.H, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S, a.g.err};
        LoadKC<TM, RowsGather, NTHR> la(sa);
        run(la);
    } else {
        RowsDirect sa{a.x, a.H, a.xrow0 + lo, hi - lo};
        LoadKC<TM, RowsDirect, NTHR> la(sa);
        run(la);
    }
    AccPos<TM, 128> pos;          // wave tile (TM/2) x 64 at column 64 * (wave >> 1)
    const int wn = threadIdx.x >> 7;
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) {
        const int rl = lo + pos.m(mb);
        if (rl >= hi) continue;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int i = i0 + 32 * wn + nb * 16 + 4 * (lane_id() >> 4);
            float gq[4], uq[4], hq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gq[r] = bf2f(f2bf(acc[mb][nb][r]));
                uq[r] = bf2f(f2bf(acc[mb][nb + 2][r]));
                hq[r] = swiglu_h(gq[r], uq[r]);
            }
            if (a.g_out) {                  // null: g, u are not kept (recomputed later)
                const int64_t srow = (int64_t)(a.save_row0 + rl) * a.I + i;
                *(uint2*)(a.g_out + srow) = pack4(gq[0], gq[1], gq[2], gq[3]);
                *(uint2*)(a.u_out + srow) = pack4(uq[0], uq[1], uq[2], uq[3]);
            }
            *(uint2*)(a.h_out + (int64_t)rl * a.I + i) = pack4(hq[0], hq[1], hq[2], hq[3]);
        }
    }
}

// The groups of at least kBigRows rows in 256 x 256 tiles (mainloop_big):
// 256 rows x (128 gate + 128 up columns); wave w holds gate columns
// i0 + 32 (w >> 1) + 0..31 in acc[.][0..1] and the matching up columns in
// acc[.][2..3] (RowsGateUp's quarters).  Same bits as the 128-row tiles.
__global__ __launch_bounds__(kBigThreads, 1) void k_gemm_gate_up_big(GemmGateUpArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t st0[SmemBig::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st1[SmemBig::STAGE];
    int e, lo, hi, nt;
    if (!map_mtile_big(a.g, a.I / (kBig / 2), blockIdx.x, e, lo, hi, nt)) return;
    const int i0 = nt * (kBig / 2);
    f32x4 acc[8][4];
    {
        const RowsGateUp sb{a.w_gate + (int64_t)e * a.I * a.H, a.w_up + (int64_t)e * a.I * a.H, a.H, i0};
        const DirectKC lb(sb);
        if (a.x_gather) {
            const RowsGather sa{a.x, a.H, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S, a.g.err};
            const DirectKC la(sa);
            mainloop_big(la, lb, a.H / kTK, st0, st1, acc);
        } else {
            const RowsDirect sa{a.x, a.H, a.xrow0 + lo, hi - lo};
            const DirectKC la(sa);
            mainloop_big(la, lb, a.H / kTK, st0, st1, acc);
        }
    }
    const int w = threadIdx.x >> 6, lane = lane_id();
    const int wm0 = (w & 1) * 128, wq = w >> 1;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int rl = lo + wm0 + mb * 16 + (lane & 15);
        if (rl >= hi) continue;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int i = i0 + 32 * wq + nb * 16 + 4 * (lane >> 4);
            float gq[4], uq[4], hq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gq[r] = bf2f(f2bf(acc[mb][nb][r]));
                uq[r] = bf2f(f2bf(acc[mb][nb + 2][r]));
                hq[r] = swiglu_h(gq[r], uq[r]);
            }
            if (a.g_out) {
                const int64_t srow = (int64_t)(a.save_row0 + rl) * a.I + i;
                *(uint2*)(a.g_out + srow) = pack4(gq[0], gq[1], gq[2], gq[3]);
                *(uint2*)(a.u_out + srow) = pack4(uq[0], uq[1], uq[2], uq[3]);
            }
            *(uint2*)(a.h_out + (int64_t)rl * a.I + i) = pack4(hq[0], hq[1], hq[2], hq[3]);
        }
    }
}

// ================================================================ forward GEMM 2
// o = w * (h W_down^T), each row scaled by its slot's router weight in fp32
// before the one rounding to bf16.  alphalab.site "Mixture-of-Kittens" keeps
// the final router-weighted reduction as a step of its own after the combine
// (section 二); applying the weight here leaves that step a plain fixed-order
// sum of a token's rows.  Tile TM rows x 128 columns of H;
// with 128-row tiles a block takes two neighbouring column tiles in one K
// loop (K = I is short).
constexpr int G2_TN = 128;

template <int TM>
__global__ __launch_bounds__(256, 2) void k_gemm_down(GemmDownArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<TM, G2_TN, false, false>::STAGE];
    constexpr int NT = short_k_tiles_per_block<TM>();
    const int ncol = a.H / G2_TN;
    int e, lo, hi, np;
    if (!map_mtile<TM>(a.g, (ncol + NT - 1) / NT, blockIdx.x, e, lo, hi, np)) return;
    const int n0 = NT * np * G2_TN;
    const int ntl = min(NT, ncol - NT * np);
    f32x4 acc[TM / 32][4];
    RowsDirect sa{a.h, a.I, lo, hi - lo};
    LoadKC<TM, RowsDirect> la(sa);
    RowsDirect sb{a.w_down + (int64_t)e * a.H * a.I, a.I, n0, G2_TN};
    LoadKC<G2_TN, RowsDirect> lb(sb);
    AccPos<TM, G2_TN> pos;
    float wr[TM / 32];
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) wr[mb] = lo + pos.m(mb) < hi ? a.rw.at(lo + pos.m(mb)) : 0.f;
    int64_t orow[TM / 32];
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) orow[mb] = lo + pos.m(mb) < hi ? a.dest.row(lo + pos.m(mb), a.g.err) : -1;
    auto epi = [&](int t, const f32x4 (&c)[TM / 32][4]) {
#pragma unroll
        for (int mb = 0; mb < TM / 32; ++mb) {
            if (orow[mb] < 0) continue;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int col = n0 + t * G2_TN + pos.n(nb);
                const f32x4 v = c[mb][nb];
                *(uint2*)(a.o + orow[mb] * a.H + col) =
                    pack4(wr[mb] * v[0], wr[mb] * v[1], wr[mb] * v[2], wr[mb] * v[3]);
            }
        }
    };
    if constexpr (NT == 1) {
        mainloop<TM, G2_TN, false, false>(la, lb, a.I / kTK, smem, acc);
        epi(0, acc);
    } else {
        mainloop_tiles<TM, G2_TN, false, false>(la, lb, a.I / kTK, ntl, (int64_t)G2_TN * a.I, smem, acc, epi);
    }
}

// The groups of at least kBigRows rows in 256 x 256 tiles (mainloop_big):
// the same rows, scaled by their router weights, and the same bits (K steps
// ascend and each MFMA sums in a fixed order, whatever the tile shape).
__global__ __launch_bounds__(kBigThreads, 1) void k_gemm_down_big(GemmDownArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t st0[SmemBig::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st1[SmemBig::STAGE];
    int e, lo, hi, nt;
    if (!map_mtile_big(a.g, a.H / kBig, blockIdx.x, e, lo, hi, nt)) return;
    const int n0 = nt * kBig;
    const int w = threadIdx.x >> 6, lane = lane_id();
    const int wm0 = (w & 1) * 128, wn0 = (w >> 1) * 64;
    // the epilogue's row look-ups (destination row, router weight) go out
    // before the K loop, so that their round trips hide behind it
    int64_t orow[8];
    float wr[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int rl = lo + wm0 + mb * 16 + (lane & 15);
        orow[mb] = -1;
        wr[mb] = 0.f;
        if (rl < hi) {
            orow[mb] = a.dest.row(rl, a.g.err);
            wr[mb] = a.rw.at(rl);
        }
    }
    f32x4 acc[8][4];
    {
        const RowsDirect sa{a.h, a.I, lo, hi - lo};
        const RowsDirect sb{a.w_down + (int64_t)e * a.H * a.I, a.I, n0, kBig};
        const DirectKC la(sa), lb(sb);
        mainloop_big(la, lb, a.I / kTK, st0, st1, acc);
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        if (orow[mb] < 0) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int col = n0 + wn0 + nb * 16 + 4 * (lane >> 4);
            const f32x4 v = acc[mb][nb];
            *(uint2*)(a.o + orow[mb] * a.H + col) =
                pack4(wr[mb] * v[0], wr[mb] * v[1], wr[mb] * v[2], wr[mb] * v[3]);
        }
    }
}

// ================================================================ backward: down dgrad
// a = dY W_down (dY row = dy of the row's token, gathered on load), then the
// SwiGLU backward and the router-weight gradient in the epilogue:
//   h = SiLU(g) * u (recomputed from the saved bf16 g, u exactly as forward)
//   dw partial = sum over this tile's columns of a * h
//   dh = w * a;  du = dh * SiLU(g);  dg = dh * u * s * (1 + g (1 - s))
//   hw = w * h   (the down-projection weight-gradient operand)
// Tile TM rows x 128 columns of I; reduction over H.
constexpr int G3_TN = 128;

template <int TM>
__global__ __launch_bounds__(256, 2) void k_gemm_down_dgrad(GemmDownDgradArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[lds_two_blocks(2 * Smem<TM, G3_TN, false, true>::STAGE)];
    __shared__ float red[2][TM];
    int e, lo, hi, nt;
    if (!map_mtile<TM>(a.g, a.I / G3_TN, blockIdx.x, e, lo, hi, nt)) return;
    const int n0 = nt * G3_TN;
    f32x4 acc[TM / 32][4];
    KRowsDirect sb{a.w_down + (int64_t)e * a.H * a.I, a.I, n0, a.H};
    LoadKS<G3_TN, KRowsDirect> lb(sb);
    if (a.dy_gather) {
        RowsGather sa{a.dy, a.H, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S, a.g.err};
        LoadKC<TM, RowsGather> la(sa);
        mainloop<TM, G3_TN, false, true>(la, lb, a.H / kTK, smem, acc);
    } else {
        RowsDirect sa{a.dy, a.H, a.dyrow0 + lo, hi - lo};
        LoadKC<TM, RowsDirect> la(sa);
        mainloop<TM, G3_TN, false, true>(la, lb, a.H / kTK, smem, acc);
    }
    AccPos<TM, G3_TN> pos;
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6, wm = wv & 1, wn = wv >> 1;
    float dot[TM / 32];
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) dot[mb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) {
        const int rl = lo + pos.m(mb);
        const bool ok = rl < hi;
        float wr = 1.0f;
        if (ok && a.topk_w) {
            const int s = a.slot_of_row[a.grow0 + rl];
            wr = (unsigned)s < (unsigned)a.S ? a.topk_w[s] : 0.f;
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            if (!ok) continue;
            const int i = n0 + pos.n(nb);
            const int64_t srow = (int64_t)(a.save_row0 + rl) * a.I + i;
            const uint2 gb = *(const uint2*)(a.g_saved + srow);
            const uint2 ub = *(const uint2*)(a.u_saved + srow);
            const float gq[4] = {lo_bf(gb.x), hi_bf(gb.x), lo_bf(gb.y), hi_bf(gb.y)};
            const float uq[4] = {lo_bf(ub.x), hi_bf(ub.x), lo_bf(ub.y), hi_bf(ub.y)};
            float dg[4], du[4], hw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float av = acc[mb][nb][r];
                const float h = bf2f(f2bf(swiglu_h(gq[r], uq[r])));
                dot[mb] += av * h;
                const float dh = wr * av;
                const float s = sigmoidf_(gq[r]);
                du[r] = dh * (gq[r] * s);
                dg[r] = dh * uq[r] * s * (1.0f + gq[r] * (1.0f - s));
                hw[r] = wr * h;
            }
            const int64_t drow = (int64_t)rl * (2 * a.I);
            *(uint2*)(a.dgu + drow + i) = pack4(dg[0], dg[1], dg[2], dg[3]);
            *(uint2*)(a.dgu + drow + a.I + i) = pack4(du[0], du[1], du[2], du[3]);
            *(uint2*)(a.hw + (int64_t)rl * a.I + i) = pack4(hw[0], hw[1], hw[2], hw[3]);
        }
    }
    if (!a.dw_part) return;
    // reduce the per-lane dots over the 4 lanes that share a row, then over
    // the two column-halves of the tile (waves wn = 0, 1), in a fixed order
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) {
        dot[mb] += __shfl_xor(dot[mb], 16);
        dot[mb] += __shfl_xor(dot[mb], 32);
    }
    if (lane < 16) {
#pragma unroll
        for (int mb = 0; mb < TM / 32; ++mb) red[wn][wm * (TM / 2) + 16 * mb + lane] = dot[mb];
    }
    __syncthreads();
    if (threadIdx.x < TM) {
        const int m = threadIdx.x;
        const int rl = lo + m;
        if (rl < hi) a.dw_part[(int64_t)rl * a.P + nt] = red[0][m] + red[1][m];
    }
}

// The groups of at least kBigRows rows in 256 x 256 tiles (two of the
// 128-column tiles above; mainloop_big with W_down as a KS operand).  The
// epilogue is the one above, per 128-column tile: each wave's 64 columns are
// one half of one such tile, so the dw partials (lane sums, the two shuffles,
// then half 0 + half 1) and every other output keep their bits.
__global__ __launch_bounds__(kBigThreads, 1) void k_gemm_down_dgrad_big(GemmDownDgradArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t st0[SmemBig::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st1[SmemBig::STAGE];
    __shared__ float red[2][2][kBig];                     // [128-column tile][half][row]
    int e, lo, hi, nt;
    if (!map_mtile_big(a.g, a.I / kBig, blockIdx.x, e, lo, hi, nt)) return;
    const int n0 = nt * kBig;
    f32x4 acc[8][4];
    {
        const StepRows sb{a.w_down + (int64_t)e * a.H * a.I, a.I, n0};
        const DirectKS lb(a.I);
        if (a.dy_gather) {
            const RowsGather sa{a.dy, a.H, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S, a.g.err};
            const DirectKC la(sa);
            mainloop_big(la, lb, sb, a.H / kTK, st0, st1, acc);
        } else {
            const RowsDirect sa{a.dy, a.H, a.dyrow0 + lo, hi - lo};
            const DirectKC la(sa);
            mainloop_big(la, lb, sb, a.H / kTK, st0, st1, acc);
        }
    }
    const int w = threadIdx.x >> 6, lane = lane_id();
    const int wm0 = (w & 1) * 128, wq = w >> 1;           // columns n0 + 64 wq: tile wq / 2, half wq % 2
    float dot[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) dot[mb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int rl = lo + wm0 + mb * 16 + (lane & 15);
        const bool ok = rl < hi;
        float wr = 1.0f;
        if (ok && a.topk_w) {
            const int s = a.slot_of_row[a.grow0 + rl];
            wr = (unsigned)s < (unsigned)a.S ? a.topk_w[s] : 0.f;
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            if (!ok) continue;
            const int i = n0 + 64 * wq + nb * 16 + 4 * (lane >> 4);
            const int64_t srow = (int64_t)(a.save_row0 + rl) * a.I + i;
            const uint2 gb = *(const uint2*)(a.g_saved + srow);
            const uint2 ub = *(const uint2*)(a.u_saved + srow);
            const float gq[4] = {lo_bf(gb.x), hi_bf(gb.x), lo_bf(gb.y), hi_bf(gb.y)};
            const float uq[4] = {lo_bf(ub.x), hi_bf(ub.x), lo_bf(ub.y), hi_bf(ub.y)};
            float dg[4], du[4], hw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float av = acc[mb][nb][r];
                const float h = bf2f(f2bf(swiglu_h(gq[r], uq[r])));
                dot[mb] += av * h;
                const float dh = wr * av;
                const float s = sigmoidf_(gq[r]);
                du[r] = dh * (gq[r] * s);
                dg[r] = dh * uq[r] * s * (1.0f + gq[r] * (1.0f - s));
                hw[r] = wr * h;
            }
            const int64_t drow = (int64_t)rl * (2 * a.I);
            *(uint2*)(a.dgu + drow + i) = pack4(dg[0], dg[1], dg[2], dg[3]);
            *(uint2*)(a.dgu + drow + a.I + i) = pack4(du[0], du[1], du[2], du[3]);
            *(uint2*)(a.hw + (int64_t)rl * a.I + i) = pack4(hw[0], hw[1], hw[2], hw[3]);
        }
    }
    if (!a.dw_part) return;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        dot[mb] += __shfl_xor(dot[mb], 16);
        dot[mb] += __shfl_xor(dot[mb], 32);
    }
    if (lane < 16) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) red[wq >> 1][wq & 1][wm0 + 16 * mb + lane] = dot[mb];
    }
    __syncthreads();
    {
        const int t = threadIdx.x >> 8, m = threadIdx.x & 255;        // 512 threads: 2 tiles x 256 rows
        const int rl = lo + m;
        if (rl < hi) a.dw_part[(int64_t)rl * a.P + 2 * nt + t] = red[t][0][m] + red[t][1][m];
    }
}

// ================================================================ backward: gate/up dgrad
// dX = dg W_gate + du W_up: A = [dg | du] rows (K = 2I), B = [W_gate; W_up]
// read with k as the memory row.  Tile TM rows x 128 columns of H; with
// 128-row tiles a block takes two neighbouring column tiles in one K loop.
constexpr int G4_TN = 128;

template <int TM>
__global__ __launch_bounds__(256, 2) void k_gemm_gu_dgrad(GemmGuDgradArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<TM, G4_TN, false, true>::STAGE];
    constexpr int NT = short_k_tiles_per_block<TM>();
    const int ncol = a.H / G4_TN;
    int e, lo, hi, np;
    if (!map_mtile<TM>(a.g, (ncol + NT - 1) / NT, blockIdx.x, e, lo, hi, np)) return;
    const int n0 = NT * np * G4_TN;
    const int ntl = min(NT, ncol - NT * np);
    f32x4 acc[TM / 32][4];
    RowsDirect sa{a.dgu, 2 * a.I, lo, hi - lo};
    LoadKC<TM, RowsDirect> la(sa);
    KRowsGateUp sb{a.w_gate + (int64_t)e * a.I * a.H, a.w_up + (int64_t)e * a.I * a.H, a.H, n0, a.I};
    LoadKS<G4_TN, KRowsGateUp> lb(sb);
    AccPos<TM, G4_TN> pos;
    int64_t orow[TM / 32];
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) orow[mb] = lo + pos.m(mb) < hi ? a.dest.row(lo + pos.m(mb), a.g.err) : -1;
    auto epi = [&](int t, const f32x4 (&c)[TM / 32][4]) {
#pragma unroll
        for (int mb = 0; mb < TM / 32; ++mb) {
            if (orow[mb] < 0) continue;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int col = n0 + t * G4_TN + pos.n(nb);
                const f32x4 v = c[mb][nb];
                *(uint2*)(a.dx + orow[mb] * a.H + col) = pack4(v[0], v[1], v[2], v[3]);
            }
        }
    };
    if constexpr (NT == 1) {
        mainloop<TM, G4_TN, false, true>(la, lb, 2 * a.I / kTK, smem, acc);
        epi(0, acc);
    } else {
        mainloop_tiles<TM, G4_TN, false, true>(la, lb, 2 * a.I / kTK, ntl, G4_TN, smem, acc, epi);
    }
}

// The groups of at least kBigRows rows in 256 x 256 tiles (mainloop_big with
// [W_gate; W_up] as a KS operand); same bits as the 128-row tiles.
__global__ __launch_bounds__(kBigThreads, 1) void k_gemm_gu_dgrad_big(GemmGuDgradArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t st0[SmemBig::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st1[SmemBig::STAGE];
    int e, lo, hi, nt;
    if (!map_mtile_big(a.g, a.H / kBig, blockIdx.x, e, lo, hi, nt)) return;
    const int n0 = nt * kBig;
    const int w = threadIdx.x >> 6, lane = lane_id();
    const int wm0 = (w & 1) * 128, wn0 = (w >> 1) * 64;
    int64_t orow[8];                    // destination rows, looked up before the K loop
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int rl = lo + wm0 + mb * 16 + (lane & 15);
        orow[mb] = rl < hi ? a.dest.row(rl, a.g.err) : -1;
    }
    f32x4 acc[8][4];
    {
        const RowsDirect sa{a.dgu, 2 * a.I, lo, hi - lo};
        const DirectKC la(sa);
        const StepGateUp sb{a.w_gate + (int64_t)e * a.I * a.H, a.w_up + (int64_t)e * a.I * a.H, a.H, n0, a.I};
        const DirectKS lb(a.H);
        mainloop_big(la, lb, sb, 2 * a.I / kTK, st0, st1, acc);
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        if (orow[mb] < 0) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int col = n0 + wn0 + nb * 16 + 4 * (lane >> 4);
            const f32x4 v = acc[mb][nb];
            *(uint2*)(a.dx + orow[mb] * a.H + col) = pack4(v[0], v[1], v[2], v[3]);
        }
    }
}

// ================================================================ weight gradients
// K-grouped: C_e[M, N] = sum over e's rows (ascending) of A[r, M] (x) B[r, N];
// both operands are KS tiles.  A block owns one expert's 128-row slab of C and
// its 64-column tiles g, g + ng, ... (dealt round robin over ng blocks, so
// each block writes one contiguous region).  When the expert has at most kTK
// rows (one K step, the common case for small token counts) the A tile stays
// in LDS for all of them and the next B tile is fetched while the current one
// is multiplied; otherwise each column tile runs the K loop.
template <bool BF16_ONLY, bool STREAM, class SA, class SB>
__device__ __forceinline__ void wgrad_tiles_(LoadKS<W_TM, SA>& la, LoadKS<W_TN, SB>& lb, int nk,
                                             int nt0, int ntn, int nstride, uint16_t* smem,
                                             const WgradEpi& epi) {
    uint16_t* sA = smem;
    uint16_t* sB = smem + Tile<W_TM, true>::SIZE;
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * (W_TM / 2), wn0 = (w >> 1) * (W_TN / 2);
    f32x4 acc[W_TM / 32][W_TN / 32];
    if (nk <= 1) {
        if (nk == 1) {
            la.load(0);
            lb.src.col0 = 0;
            lb.cache_rows(0);
            lb.load_cached(nt0 * W_TN);
            la.store(sA);
        }
        for (int i = 0; i < ntn; ++i) {
            zero_acc<W_TM, W_TN>(acc);
            if (nk == 1) {
                if (i > 0) __syncthreads();          // the staged tile has been written out
                lb.store(sB);
                __syncthreads();
                if (i + 1 < ntn) lb.load_cached((nt0 + (i + 1) * nstride) * W_TN);
                mma_tile<W_TM, W_TN, true, true>(sA, sB, wm0, wn0, acc);
                __syncthreads();
            }
            epi.template store<BF16_ONLY, STREAM>(nt0 + i * nstride, acc, sB);
        }
        return;
    }
    for (int i = 0; i < ntn; ++i) {
        lb.src.col0 = (nt0 + i * nstride) * W_TN;
        zero_acc<W_TM, W_TN>(acc);
        for (int kt = 0; kt < nk; ++kt) {
            la.load(kt);
            lb.load(kt);
            la.store(sA);
            lb.store(sB);
            __syncthreads();
            mma_tile<W_TM, W_TN, true, true>(sA, sB, wm0, wn0, acc);
            __syncthreads();
        }
        epi.template store<BF16_ONLY, STREAM>(nt0 + i * nstride, acc, sB);
        __syncthreads();
    }
}

template <class SA, class SB>
__device__ __forceinline__ void wgrad_tiles(LoadKS<W_TM, SA>& la, LoadKS<W_TN, SB>& lb, int nk,
                                            int ntiles, int g, int ng, uint16_t* smem,
                                            const WgradEpi& epi) {
    const int ntn = wgrad_group_tiles(ntiles, ng, g);
    if (epi.out.mode != 0) wgrad_tiles_<false, false>(la, lb, nk, g, ntn, ng, smem, epi);
    else if (ng > 1) wgrad_tiles_<true, true>(la, lb, nk, g, ntn, ng, smem, epi);
    else wgrad_tiles_<true, false>(la, lb, nk, g, ntn, ng, smem, epi);
}

// The slab kernels' two grids.  One block per (expert, 128-row slab, column
// group) of every expert (one macrobatch, or the dense group); or, LISTED (a
// walk over several macrobatches, modes chosen per expert), a persistent grid
// over the items of the experts that have work (block_list), three blocks per
// CU.
__device__ __forceinline__ int slab_list(const GroupRows& g, const WgradOut& o, int16_t* list) {
    return block_list(g.E, [&](int e) {
        const int a = g.offsets[e], z = g.offsets[e + 1];
        if (a < 0 || z < a || z > g.rows) {
            raise_err(g.err, ERR_BAD_OFFSETS);
            return false;
        }
        const int n = z - a;
        return (g.deep_thr <= 0 || n <= g.deep_thr) && wgrad_mode(o, e, n) >= 0;
    }, list);
}
template <bool LISTED, class Item>
__device__ __forceinline__ void slab_blocks(const GroupRows& g, const WgradOut& o, int nMt, int nng,
                                            const Item& item_fn) {
    if constexpr (LISTED) {
        __shared__ int16_t list[1024];
        const int per = nMt * nng, total = slab_list(g, o, list) * per;
        for (int r = 0;; ++r) {
            const int item = r * (int)gridDim.x + xcd_remap(blockIdx.x, gridDim.x);
            if (item >= total) break;
            if (r) __syncthreads();                 // the previous item's staged tile has been read
            const int d = item / per, rem = item - d * per;
            const int e = list[d];
            const int lo = g.offsets[e];
            item_fn(e, rem / nng, rem % nng, lo, g.offsets[e + 1] - lo);    // validated by the list
        }
    } else {
        int e, mt, ng, lo, n;
        if (!map_ktile(g, nMt, nng, blockIdx.x, e, mt, ng, lo, n)) return;
        item_fn(e, mt, ng, lo, n);
    }
}
constexpr int SLAB_LISTED_PER_CU = 3;
// the listed form: a walk over several macrobatches of routed groups
static inline bool slab_listed(const GroupRows& g, const WgradOut& o) { return g.offsets && o.counts; }
static inline int slab_grid(const GroupRows& g, const WgradOut& o, int nMt, int nng) {
    const int all = (g.offsets ? g.E : 1) * nMt * nng;
    return slab_listed(g, o) ? std::min(all, SLAB_LISTED_PER_CU * 256) : all;
}

// dW_down[e][h, i] = sum over e's rows r of dy[tok(r), h] * hw[r, i].
template <bool LISTED>
__global__ __launch_bounds__(256, LISTED ? SLAB_LISTED_PER_CU : 4) void k_wgrad_down(WgradDownArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[W_SMEM];
    const int ntiles = a.I / W_TN, nng = wgrad_groups(ntiles);
    slab_blocks<LISTED>(a.g, a.out, a.H / W_TM, nng, [&](int e, int mt, int ng, int lo, int n) {
        if (a.g.deep_thr > 0 && n > a.g.deep_thr) return;          // the deep kernel's group
        const int m0 = mt * W_TM;
        const int nk = (n + kTK - 1) / kTK;
        KRowsGroup sb{a.hw, a.I, lo, n, 0};
        LoadKS<W_TN, KRowsGroup> lb(sb);
        WgradOut o = a.out;
        if (wgrad_bind(o, e, n, (int64_t)a.H * a.I) < 0) return;   // nothing to add for this expert
        WgradEpi epi{o, (int64_t)e * a.H * a.I, a.I, m0};
        if (a.dy_gather) {
            KRowsGroupGather sa{a.dy, a.H, a.slot_of_row, a.grow0 + lo, n, m0, a.k, a.S, a.g.err};
            LoadKS<W_TM, KRowsGroupGather> la(sa);
            wgrad_tiles(la, lb, nk, ntiles, ng, nng, smem, epi);
        } else {
            KRowsGroup sa{a.dy, a.H, a.dyrow0 + lo, n, m0};
            LoadKS<W_TM, KRowsGroup> la(sa);
            wgrad_tiles(la, lb, nk, ntiles, ng, nng, smem, epi);
        }
    });
}

// dW_gate[e][i, h] = sum_r dg[r, i] x[tok(r), h]; dW_up likewise with du.
// M runs over the 2I columns of [dg | du].
template <bool LISTED>
__global__ __launch_bounds__(256, 3) void k_wgrad_gate_up(WgradGateUpArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[W_SMEM];
    const int ntiles = a.H / W_TN, nng = wgrad_groups(ntiles);
    slab_blocks<LISTED>(a.g, a.out_gate, 2 * a.I / W_TM, nng, [&](int e, int mt, int ng, int lo, int n) {
        if (a.g.deep_thr > 0 && n > a.g.deep_thr) return;          // the deep kernel's group
        const int m0 = mt * W_TM;
        const int nk = (n + kTK - 1) / kTK;
        const bool up = m0 >= a.I;
        KRowsGroup sa{a.dgu, 2 * a.I, lo, n, m0};
        LoadKS<W_TM, KRowsGroup> la(sa);
        WgradOut o = up ? a.out_up : a.out_gate;
        if (wgrad_bind(o, e, n, (int64_t)a.I * a.H) < 0) return;   // nothing to add for this expert
        WgradEpi epi{o, (int64_t)e * a.I * a.H, a.H, up ? m0 - a.I : m0};
        if (a.x_gather) {
            KRowsGroupGather sb{a.x, a.H, a.slot_of_row, a.grow0 + lo, n, 0, a.k, a.S, a.g.err};
            LoadKS<W_TN, KRowsGroupGather> lb(sb);
            wgrad_tiles(la, lb, nk, ntiles, ng, nng, smem, epi);
        } else {
            KRowsGroup sb{a.x, a.H, a.xrow0 + lo, n, 0};
            LoadKS<W_TN, KRowsGroup> lb(sb);
            wgrad_tiles(la, lb, nk, ntiles, ng, nng, smem, epi);
        }
    });
}

// ---------------------------------------------------------------- deep groups
// Groups with more than kTK rows (hot experts, the dense shared expert of a
// large macrobatch) are GEMMs with a real K: 128 x 128 output tiles, the
// double-buffered K loop, run by a persistent grid over the items (deep group,
// tile) so that a hot expert's tiles spread over the whole chip.
constexpr int D_TM = 128, D_TN = 128, D_GRID = 512;

__device__ __forceinline__ bool dense_wgrad_big(const GroupRows& g) {
    return g.big_thr > 0 && g.dense_rows >= g.big_thr;
}

__device__ __forceinline__ int deep_count(const GroupRows& g) {
    if (g.deep_thr <= 0) return 0;
    if (g.offsets) return g.deep[0];
    return g.dense_rows > g.deep_thr && !dense_wgrad_big(g) ? 1 : 0;
}

// group d of the deep list -> (expert, first row, rows)
__device__ __forceinline__ void deep_group(const GroupRows& g, int d, int& e, int& lo, int& n) {
    if (!g.offsets) {
        e = 0;
        lo = 0;
        n = g.dense_rows;
        return;
    }
    e = g.deep[1 + d];
    lo = g.offsets[e];
    n = g.offsets[e + 1] - lo;          // validated when the list was built
}

__global__ __launch_bounds__(256, 2) void k_wgrad_down_deep(WgradDownArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<D_TM, D_TN, true, true>::STAGE];
    const int nNt = a.I / D_TN, per = (a.H / D_TM) * nNt;
    const int total = deep_count(a.g) * per;
    for (int r = 0, item = deep_item(0); item < total; item = deep_item(++r)) {
        const int d = item / per, tile = item - d * per;
        int e, lo, n;
        deep_group(a.g, d, e, lo, n);
        int mt, nt;
        band_tile(tile, per / nNt, nNt, mt, nt);
        const int m0 = mt * D_TM, n0 = nt * D_TN;
        const int nk = (n + kTK - 1) / kTK;
        KRowsGroup sb{a.hw, a.I, lo, n, n0};
        LoadKS<D_TN, KRowsGroup> lb(sb);
        f32x4 acc[D_TM / 32][D_TN / 32];
        if (a.dy_gather) {
            KRowsGroupGather sa{a.dy, a.H, a.slot_of_row, a.grow0 + lo, n, m0, a.k, a.S, a.g.err};
            LoadKS<D_TM, KRowsGroupGather> la(sa);
            mainloop_ks_pipe<D_TM, D_TN>(la, lb, nk, smem, acc);
        } else {
            KRowsGroup sa{a.dy, a.H, a.dyrow0 + lo, n, m0};
            LoadKS<D_TM, KRowsGroup> la(sa);
            mainloop_ks_pipe<D_TM, D_TN>(la, lb, nk, smem, acc);
        }
        WgradOut o = a.out;
        if (wgrad_bind(o, e, n, (int64_t)a.H * a.I) >= 0)
            staged_tile_store(o, (int64_t)e * a.H * a.I, a.I, m0, n0, acc, (float*)smem);
    }
}

__global__ __launch_bounds__(256, 2) void k_wgrad_gate_up_deep(WgradGateUpArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<D_TM, D_TN, true, true>::STAGE];
    const int nNt = a.H / D_TN, per = (2 * a.I / D_TM) * nNt;
    const int total = deep_count(a.g) * per;
    for (int r = 0, item = deep_item(0); item < total; item = deep_item(++r)) {
        const int d = item / per, tile = item - d * per;
        int e, lo, n;
        deep_group(a.g, d, e, lo, n);
        int mt, nt;
        band_tile(tile, per / nNt, nNt, mt, nt);
        const int m0 = mt * D_TM, n0 = nt * D_TN;
        const int nk = (n + kTK - 1) / kTK;
        const bool up = m0 >= a.I;
        KRowsGroup sa{a.dgu, 2 * a.I, lo, n, m0};
        LoadKS<D_TM, KRowsGroup> la(sa);
        f32x4 acc[D_TM / 32][D_TN / 32];
        if (a.x_gather) {
            KRowsGroupGather sb{a.x, a.H, a.slot_of_row, a.grow0 + lo, n, n0, a.k, a.S, a.g.err};
            LoadKS<D_TN, KRowsGroupGather> lb(sb);
            mainloop_ks_pipe<D_TM, D_TN>(la, lb, nk, smem, acc);
        } else {
            KRowsGroup sb{a.x, a.H, a.xrow0 + lo, n, n0};
            LoadKS<D_TN, KRowsGroup> lb(sb);
            mainloop_ks_pipe<D_TM, D_TN>(la, lb, nk, smem, acc);
        }
        WgradOut o = up ? a.out_up : a.out_gate;
        if (wgrad_bind(o, e, n, (int64_t)a.I * a.H) >= 0)
            staged_tile_store(o, (int64_t)e * a.I * a.H, a.H, up ? m0 - a.I : m0, n0, acc, (float*)smem);
    }
}

// ---------------------------------------------------------------- large groups
// Groups of at least big_thr rows (the GEMM is then MFMA work: each output
// element sums hundreds of products): 256 x 256 output tiles (eight waves,
// operands copied straight into LDS as swizzled K-major tiles), a persistent
// grid over the items (big group, tile); consecutive items of a round go to
// the blocks of one XCD, so the tiles that share an operand strip share its L2.
constexpr int B_GRID = 256;

__device__ __forceinline__ int big_count(const GroupRows& g) {
    if (g.big_thr <= 0) return 0;
    if (g.offsets) return g.deep_big[0];
    return dense_wgrad_big(g) ? 1 : 0;
}

__device__ __forceinline__ void big_group(const GroupRows& g, int d, int& e, int& lo, int& n) {
    if (!g.offsets) {
        e = 0;
        lo = 0;
        n = g.dense_rows;
        return;
    }
    e = g.deep_big[1 + d];
    lo = g.offsets[e];
    n = g.offsets[e + 1] - lo;          // validated when the list was built
}

// A 256 x 256 tile (mainloop_big_kk's layout) stored through LDS 64 rows at a
// time, the rounds alternating the two stage arrays (64 rows x 256 floats,
// 64 KB, 16-byte chunks XOR-swizzled by row so that 16 rows of one chunk, or
// 16 chunks of one row, hit 16 bank groups): every global access is a whole
// 1 KB (fp32) or 512-byte (bf16) row piece.  Ends with a barrier (the stage
// arrays are free for the next item's copies).
__device__ __forceinline__ void big_wgrad_store(const WgradOut& out, int64_t ebase, int64_t ld, int r0, int n0,
                                                const f32x4 (&acc)[8][4], float* b0, float* b1) {
    const int w = threadIdx.x >> 6, lane = lane_id();
    const int wn0 = (w >> 1) * 64;
    // readout: chunk q of a round is row 8 q + threadIdx.x / 64 of the round's
    // 64, column chunk threadIdx.x % 64
    const int rr = threadIdx.x >> 6, cc = threadIdx.x & 63;
#pragma unroll
    for (int rd = 0; rd < 4; ++rd) {                 // rows 64 rd .. 64 rd + 63 of the tile
        float* buf = (rd & 1) ? b1 : b0;
        const int64_t base = ebase + (int64_t)(r0 + 64 * rd + rr) * ld + n0 + 4 * cc;
        if ((w & 1) == (rd >> 1)) {
#pragma unroll
            for (int mbl = 0; mbl < 4; ++mbl) {
                const int rl = mbl * 16 + (lane & 15);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int ch = (wn0 + nb * 16) / 4 + (lane >> 4);
                    *(f32x4*)(buf + rl * 256 + 4 * (ch ^ (rl & 15))) = acc[(rd & 1) * 4 + mbl][nb];
                }
            }
        }
        // the old sums in two batches of four (eight at once spill)
        f32x4 old[4];
        if (out.mode >= 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q) old[q] = wgrad_old(out, base + 8 * q * ld);
        }
        __syncthreads();
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            if (hb && out.mode >= 2) {
#pragma unroll
                for (int q = 0; q < 4; ++q) old[q] = wgrad_old(out, base + 8 * (4 + q) * ld);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = rr + 8 * (4 * hb + q);
                wgrad_put(out, base + 8 * (4 * hb + q) * ld, *(const f32x4*)(buf + r * 256 + 4 * (cc ^ (r & 15))),
                          old[q]);
            }
        }
    }
    __syncthreads();
}

// Items of round r: consecutive ones on the blocks of one XCD; odd rounds
// deal them in reverse, so that a block that took a tile of a larger group
// (the list ascends by expert, a skewed stream's groups mostly shrink along
// it) takes one of a smaller group next.
__device__ __forceinline__ int big_item(int r) {
    const int l = xcd_remap(blockIdx.x, gridDim.x);
    return r * (int)gridDim.x + ((r & 1) ? (int)gridDim.x - 1 - l : l);
}

__global__ __launch_bounds__(kBigThreads, 1) void k_wgrad_down_big(WgradDownArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t st0[SmemBig::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st1[SmemBig::STAGE];
    const int nNt = a.I / kBig, per = (a.H / kBig) * nNt;
    const int total = big_count(a.g) * per;
    for (int r = 0;; ++r) {
        const int item = big_item(r);
        if (item >= total) break;
        const int d = item / per, tile = item - d * per;
        int e, lo, n;
        big_group(a.g, d, e, lo, n);
        int mt, nt;
        band_tile(tile, per / nNt, nNt, mt, nt);
        const int m0 = mt * kBig, n0 = nt * kBig;
        const int nk = (n + kTK - 1) / kTK;
        DirectKSRows<KRowsGroup> lb(KRowsGroup{a.hw, a.I, lo, n, n0}, a.zero);
        f32x4 acc[8][4];
        if (a.dy_gather) {
            DirectKSRows<KRowsGroupGather> la(
                KRowsGroupGather{a.dy, a.H, a.slot_of_row, a.grow0 + lo, n, m0, a.k, a.S, a.g.err}, a.zero);
            mainloop_big_kk(la, lb, nk, st0, st1, acc);
        } else {
            DirectKSRows<KRowsGroup> la(KRowsGroup{a.dy, a.H, a.dyrow0 + lo, n, m0}, a.zero);
            mainloop_big_kk(la, lb, nk, st0, st1, acc);
        }
        WgradOut o = a.out;
        if (wgrad_bind(o, e, n, (int64_t)a.H * a.I) >= 0)
            big_wgrad_store(o, (int64_t)e * a.H * a.I, a.I, m0, n0, acc, (float*)st0, (float*)st1);
    }
}

__global__ __launch_bounds__(kBigThreads, 1) void k_wgrad_gate_up_big(WgradGateUpArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t st0[SmemBig::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st1[SmemBig::STAGE];
    const int nNt = a.H / kBig, per = (2 * a.I / kBig) * nNt;
    const int total = big_count(a.g) * per;
    for (int r = 0;; ++r) {
        const int item = big_item(r);
        if (item >= total) break;
        const int d = item / per, tile = item - d * per;
        int e, lo, n;
        big_group(a.g, d, e, lo, n);
        int mt, nt;
        band_tile(tile, per / nNt, nNt, mt, nt);
        const int m0 = mt * kBig, n0 = nt * kBig;
        const int nk = (n + kTK - 1) / kTK;
        const bool up = m0 >= a.I;
        DirectKSRows<KRowsGroup> la(KRowsGroup{a.dgu, 2 * a.I, lo, n, m0}, a.zero);
        f32x4 acc[8][4];
        if (a.x_gather) {
            DirectKSRows<KRowsGroupGather> lb(
                KRowsGroupGather{a.x, a.H, a.slot_of_row, a.grow0 + lo, n, n0, a.k, a.S, a.g.err}, a.zero);
            mainloop_big_kk(la, lb, nk, st0, st1, acc);
        } else {
            DirectKSRows<KRowsGroup> lb(KRowsGroup{a.x, a.H, a.xrow0 + lo, n, n0}, a.zero);
            mainloop_big_kk(la, lb, nk, st0, st1, acc);
        }
        WgradOut o = up ? a.out_up : a.out_gate;
        if (wgrad_bind(o, e, n, (int64_t)a.I * a.H) >= 0)
            big_wgrad_store(o, (int64_t)e * a.I * a.H, a.H, up ? m0 - a.I : m0, n0, acc, (float*)st0, (float*)st1);
    }
}

// ================================================================ launchers
static inline int mgroup_grid(const GroupRows& g, int TM) {
    if (!g.tile_off) return (g.dense_rows + TM - 1) / TM;
    // sum_e ceil(n_e / TM) <= (rows + E (TM - 1)) / TM, and <= rows
    const int64_t bound = ((int64_t)g.rows + (int64_t)g.E * (TM - 1)) / TM;
    return (int)(bound < g.rows ? bound : g.rows);
}

// row tile of a group description (the tile prefix was built with it)
static inline int row_tile(const GroupRows& g) { return g.tm == 128 ? 128 : 64; }

#define MOE_LAUNCH_TM(KERNEL, NCOLTILES)                                           \
    do {                                                                           \
        const int tm_ = row_tile(a.g);                                             \
        const int grid_ = mgroup_grid(a.g, tm_) * (NCOLTILES);                     \
        if (grid_ <= 0) return 0;                                                  \
        if (tm_ == 128) KERNEL<128><<<grid_, 256, 0, st>>>(a);                     \
        else KERNEL<64><<<grid_, 256, 0, st>>>(a);                                 \
        return hipGetLastError() == hipSuccess ? 0 : -1;                           \
    } while (0)

// the same with the column-tile count depending on the row tile
#define MOE_LAUNCH_TM2(KERNEL, NCOL64, NCOL128)                                    \
    do {                                                                           \
        const int tm_ = row_tile(a.g);                                             \
        const int grid_ = mgroup_grid(a.g, tm_) * (tm_ == 128 ? (NCOL128) : (NCOL64)); \
        if (grid_ <= 0) return 0;                                                  \
        if (tm_ == 128) KERNEL<128><<<grid_, 256, 0, st>>>(a);                     \
        else KERNEL<64><<<grid_, 256, 0, st>>>(a);                                 \
        return hipGetLastError() == hipSuccess ? 0 : -1;                           \
    } while (0)

int launch_gemm_gate_up(const GemmGateUpArgs& a, hipStream_t st) {
    ProfScope prof_(st, "gemm_gate_up");
    const bool dims_ok = a.I % (kBig / 2) == 0 && a.H % kTK == 0;
    const bool dbig = dense_big(a.g, dims_ok);
    if (a.g.tile_big || dbig) {
        if (!dims_ok) return -1;
        const int grid = big_grid(a.g) * (a.I / (kBig / 2));
        if (grid > 0) {
            k_gemm_gate_up_big<<<grid, kBigThreads, 0, st>>>(a);
            if (hipGetLastError() != hipSuccess) return -1;
        }
        if (dbig) return 0;
    }
    const int tm_ = row_tile(a.g);
    const int grid_ = mgroup_grid(a.g, tm_) * (a.I / (tm_ == 128 ? 128 : 64));
    if (grid_ <= 0) return 0;
    if (tm_ == 128) k_gemm_gate_up<128><<<grid_, GateUpShape<128>::NTHR, 0, st>>>(a);
    else k_gemm_gate_up<64><<<grid_, GateUpShape<64>::NTHR, 0, st>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_down(const GemmDownArgs& a, hipStream_t st) {
    ProfScope prof_(st, "gemm_down");
    const bool dims_ok = a.H % kBig == 0 && a.I % kTK == 0;
    const bool dbig = dense_big(a.g, dims_ok);
    if (a.g.tile_big || dbig) {
        if (!dims_ok) return -1;
        const int grid = big_grid(a.g) * (a.H / kBig);
        if (grid > 0) {
            k_gemm_down_big<<<grid, kBigThreads, 0, st>>>(a);
            if (hipGetLastError() != hipSuccess) return -1;
        }
        if (dbig) return 0;
    }
    const int ncol = a.H / G2_TN;
    MOE_LAUNCH_TM2(k_gemm_down, (ncol + short_k_tiles_per_block<64>() - 1) / short_k_tiles_per_block<64>(),
                   (ncol + short_k_tiles_per_block<128>() - 1) / short_k_tiles_per_block<128>());
}

int launch_gemm_down_dgrad(const GemmDownDgradArgs& a, hipStream_t st) {
    ProfScope prof_(st, "gemm_down_dgrad");
    const bool dims_ok = a.I % kBig == 0 && a.H % kTK == 0;
    const bool dbig = dense_big(a.g, dims_ok);
    if (a.g.tile_big || dbig) {
        if (!dims_ok || a.P != a.I / G3_TN) return -1;
        const int grid = big_grid(a.g) * (a.I / kBig);
        if (grid > 0) {
            k_gemm_down_dgrad_big<<<grid, kBigThreads, 0, st>>>(a);
            if (hipGetLastError() != hipSuccess) return -1;
        }
        if (dbig) return 0;
    }
    MOE_LAUNCH_TM(k_gemm_down_dgrad, a.I / G3_TN);
}

int launch_gemm_gu_dgrad(const GemmGuDgradArgs& a, hipStream_t st) {
    ProfScope prof_(st, "gemm_gu_dgrad");
    const bool dims_ok = a.H % kBig == 0 && a.I % kTK == 0;
    const bool dbig = dense_big(a.g, dims_ok);
    if (a.g.tile_big || dbig) {
        if (!dims_ok) return -1;
        const int grid = big_grid(a.g) * (a.H / kBig);
        if (grid > 0) {
            k_gemm_gu_dgrad_big<<<grid, kBigThreads, 0, st>>>(a);
            if (hipGetLastError() != hipSuccess) return -1;
        }
        if (dbig) return 0;
    }
    const int ncol = a.H / G4_TN;
    MOE_LAUNCH_TM2(k_gemm_gu_dgrad, (ncol + short_k_tiles_per_block<64>() - 1) / short_k_tiles_per_block<64>(),
                   (ncol + short_k_tiles_per_block<128>() - 1) / short_k_tiles_per_block<128>());
}

int launch_wgrad_down(const WgradDownArgs& a, hipStream_t st) {
    ProfScope prof_(st, "wgrad_down");
    if (a.g.big_thr > 0) {
        if (a.H % kBig != 0 || a.I % kBig != 0 || !a.zero || a.g.deep_thr <= 0 || a.g.big_thr <= a.g.deep_thr)
            return -1;
        k_wgrad_down_big<<<B_GRID, kBigThreads, 0, st>>>(a);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if (a.g.deep_thr > 0) {
        k_wgrad_down_deep<<<D_GRID, 256, 0, st>>>(a);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if (a.g.offsets && a.g.E > 1024) return -1;               // the block list's bound
    const int grid = slab_grid(a.g, a.out, a.H / W_TM, wgrad_groups(a.I / W_TN));
    if (slab_listed(a.g, a.out)) k_wgrad_down<true><<<grid, 256, 0, st>>>(a);
    else k_wgrad_down<false><<<grid, 256, 0, st>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_wgrad_gate_up(const WgradGateUpArgs& a, hipStream_t st) {
    ProfScope prof_(st, "wgrad_gate_up");
    if (a.g.big_thr > 0) {
        if (a.H % kBig != 0 || a.I % kBig != 0 || !a.zero || a.g.deep_thr <= 0 || a.g.big_thr <= a.g.deep_thr)
            return -1;
        k_wgrad_gate_up_big<<<B_GRID, kBigThreads, 0, st>>>(a);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if (a.g.deep_thr > 0) {
        k_wgrad_gate_up_deep<<<D_GRID, 256, 0, st>>>(a);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if (a.g.offsets && a.g.E > 1024) return -1;               // the block list's bound
    const int grid = slab_grid(a.g, a.out_gate, 2 * a.I / W_TM, wgrad_groups(a.H / W_TN));
    if (slab_listed(a.g, a.out_gate)) k_wgrad_gate_up<true><<<grid, 256, 0, st>>>(a);
    else k_wgrad_gate_up<false><<<grid, 256, 0, st>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// 128-row tiles once the mean group holds at least 192 rows (there the GEMMs
// are MFMA work rather than weight streaming)
int gemm_row_tile(int rows, int E) { return (int64_t)rows >= 192LL * E ? 128 : 64; }
int wgrad_deep_rows() { return kTK; }
// bf16 weight gradients: groups of at least this many rows take the 256 x 256 tiles
int wgrad_big_rows() { return 512; }
int wgrad_big_grid() { return B_GRID; }
int dgrad_col_tiles(int I) { return I / G3_TN; }

}  // namespace moe
