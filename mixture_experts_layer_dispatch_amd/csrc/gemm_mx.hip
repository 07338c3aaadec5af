// MXFP8 expert-grouped GEMMs of the forward (gate/up + SwiGLU + quantisation
// of h, and the down projection) on the scaled fp8 MFMA of gfx950.
//
// arex-research.com "Cursor 放出 MoK", design section, closing paragraph:
// MXFP8 mode, weights pre-quantised, activations quantised inside dispatch, the
// expert GEMM and SwiGLU.  alphalab.site "Mixture-of-Kittens" section 一: the
// expert FFN is a SwiGLU FFN.
//
// Operands are E4M3 codes with one E8M0 scale per 32 codes along K.  A K step
// is 128 codes (one v_mfma_scale_f32_16x16x128_f8f6f4).  Its operand layout:
// lane l (group g = l >> 4) supplies row (l & 15) with the 16 codes at
// K = 16g .. 16g+15 and the 16 at K = 64+16g .. 64+16g+15, and supplies the
// scale of row (l & 15), 32-block g.  Data tiles sit in LDS as [row][128 B]
// with a 144-byte pitch (16 rows read together hit 16 different bank groups),
// scales as one 32-bit word (4 blocks) per row.
#include "gemm_common.h"
#include "mx.h"
#include "profile.h"

namespace moe {

typedef int v8i32 __attribute__((ext_vector_type(8)));

// ================================================================ scale sources
struct ScalesDirect {          // row r -> words of row row0 + r
    const uint32_t* base;
    int64_t ld;                // words per row (K / 128)
    int row0, nvalid;
    __device__ const uint32_t* row(int r) const {
        return r < nvalid ? base + (int64_t)(row0 + r) * ld : nullptr;
    }
};

struct ScalesGateUp {          // same quarter interleave as RowsGateUp
    const uint32_t* wg;
    const uint32_t* wu;
    int64_t ld;
    int i0;
    __device__ const uint32_t* row(int n) const {
        const int q = n >> 5;
        const int i = i0 + ((q >> 1) << 5) + (n & 31);
        return ((q & 1) ? wu : wg) + (int64_t)i * ld;
    }
};

template <int ROWS, class Src>
struct LoadScales {
    const uint32_t* p;
    uint32_t v;
    __device__ explicit LoadScales(const Src& s) {
        p = threadIdx.x < ROWS ? s.row(threadIdx.x) : nullptr;
        v = 0;
    }
    __device__ void load(int kt) { v = p ? p[kt] : 0u; }
    __device__ void store(uint32_t* s) const {
        if (threadIdx.x < ROWS) s[threadIdx.x] = v;
    }
};

// ================================================================ tiles
template <int TM, int TN>
struct SmemMX {
    static constexpr int P = kTK + 8;                 // in uint16: 144 bytes
    static constexpr int A = TM * P;                  // uint16 units
    static constexpr int B = TN * P;
    static constexpr int SA = 2 * TM;                 // TM words
    static constexpr int SB = 2 * TN;
    static constexpr int STAGE = A + B + SA + SB;
};

__device__ __forceinline__ v8i32 frag_mx(const uint16_t* s, int rbase) {
    const int lane = lane_id();
    const uint8_t* p = (const uint8_t*)(s + (rbase + (lane & 15)) * (kTK + 8)) + 16 * (lane >> 4);
    const uint4 a = *(const uint4*)p;
    const uint4 b = *(const uint4*)(p + 64);
    v8i32 v;
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
    v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
    return v;
}

__device__ __forceinline__ int scale_mx(const uint32_t* sc, int rbase) {
    const int lane = lane_id();
    return (int)((sc[rbase + (lane & 15)] >> (8 * (lane >> 4))) & 0xffu);
}

template <int TM, int TN>
__device__ __forceinline__ void mma_tile_mx(const uint16_t* st, int wm0, int wn0,
                                            f32x4 (&acc)[TM / 32][TN / 32]) {
    using SM = SmemMX<TM, TN>;
    constexpr int MB = TM / 32, NB = TN / 32;
    const uint16_t* sA = st;
    const uint16_t* sB = st + SM::A;
    const uint32_t* cA = (const uint32_t*)(st + SM::A + SM::B);
    const uint32_t* cB = cA + TM;
    v8i32 fb[MB], fa[NB];
    int xb[MB], xa[NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        fb[mb] = frag_mx(sA, wm0 + mb * 16);
        xb[mb] = scale_mx(cA, wm0 + mb * 16);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        fa[nb] = frag_mx(sB, wn0 + nb * 16);
        xa[nb] = scale_mx(cB, wn0 + nb * 16);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fa[nb], fb[mb], acc[mb][nb], 0, 0, 0, xa[nb], 0, xb[mb]);
}

// Double-buffered K loop over 128-code steps.
template <int TM, int TN, class LA, class LB, class SA, class SB>
__device__ __forceinline__ void mainloop_mx(LA& la, LB& lb, SA& sa, SB& sb, int nk, uint16_t* smem,
                                            f32x4 (&acc)[TM / 32][TN / 32]) {
    using SM = SmemMX<TM, TN>;
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * (TM / 2), wn0 = (w >> 1) * (TN / 2);
    zero_acc<TM, TN>(acc);
    if (nk <= 0) return;
    auto put = [&](uint16_t* st) {
        la.store(st);
        lb.store(st + SM::A);
        sa.store((uint32_t*)(st + SM::A + SM::B));
        sb.store((uint32_t*)(st + SM::A + SM::B) + TM);
    };
    auto get = [&](int kt) {
        la.load(kt);
        lb.load(kt);
        sa.load(kt);
        sb.load(kt);
    };
    uint16_t* buf0 = smem;
    uint16_t* buf1 = smem + SM::STAGE;
    get(0);
    put(buf0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        uint16_t* cur = (kt & 1) ? buf1 : buf0;
        uint16_t* nxt = (kt & 1) ? buf0 : buf1;
        const bool more = kt + 1 < nk;
        if (more) get(kt + 1);
        mma_tile_mx<TM, TN>(cur, wm0, wn0, acc);
        if (more) put(nxt);
        __syncthreads();
    }
}

// ================================================================ gate/up + SwiGLU
// Like the bf16 kernel; in addition h = SiLU(g) * u, from the fp32
// accumulators, is quantised along I: each wave holds exactly one 32-wide
// block of h per row (lanes l, l^16, l^32, l^48 share it).
constexpr int M1_TM = 64, M1_TN = 128;

__global__ __launch_bounds__(256, 2) void k_gemm_gate_up_mx(GemmGateUpMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SmemMX<M1_TM, M1_TN>::STAGE];
    int e, lo, hi, nt;
    if (!map_mtile<M1_TM>(a.g, a.I / 64, blockIdx.x, e, lo, hi, nt)) return;
    const int i0 = nt * 64;
    const int H = a.H, I = a.I;
    f32x4 acc[2][4];
    const uint16_t* wg = (const uint16_t*)(a.wg_q + (int64_t)e * I * H);
    const uint16_t* wu = (const uint16_t*)(a.wu_q + (int64_t)e * I * H);
    const uint32_t* wgs = (const uint32_t*)(a.wg_s + (int64_t)e * I * (H / 32));
    const uint32_t* wus = (const uint32_t*)(a.wu_s + (int64_t)e * I * (H / 32));
    RowsGateUp db{wg, wu, H / 2, i0};
    ScalesGateUp ds{wgs, wus, H / 128, i0};
    RowsDirect da{(const uint16_t*)a.x_q, H / 2, a.xrow0 + lo, hi - lo};
    ScalesDirect dsa{(const uint32_t*)a.x_s, H / 128, a.xrow0 + lo, hi - lo};
    LoadKC<M1_TM, RowsDirect> la(da);
    LoadKC<M1_TN, RowsGateUp> lb(db);
    LoadScales<M1_TM, ScalesDirect> sa(dsa);
    LoadScales<M1_TN, ScalesGateUp> sb(ds);
    mainloop_mx<M1_TM, M1_TN>(la, lb, sa, sb, H / 128, smem, acc);
    AccPos<M1_TM, M1_TN> pos;
    const int wn = threadIdx.x >> 7, lane = lane_id();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int rl = lo + pos.m(mb);
        float hq[8];
        float amax = 0.f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            float gq[4], uq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gq[r] = bf2f(f2bf(acc[mb][nb][r]));
                uq[r] = bf2f(f2bf(acc[mb][nb + 2][r]));
                // h is quantised from the fp32 accumulators; g and u are kept
                // in bf16 for the backward
                hq[4 * nb + r] = swiglu_h(acc[mb][nb][r], acc[mb][nb + 2][r]);
                amax = fmaxf(amax, fabsf(hq[4 * nb + r]));
            }
            if (rl < hi) {
                const int i = i0 + 32 * wn + nb * 16 + 4 * (lane >> 4);
                const int64_t srow = (int64_t)(a.save_row0 + rl) * I + i;
                *(uint2*)(a.g_out + srow) = pack4(gq[0], gq[1], gq[2], gq[3]);
                *(uint2*)(a.u_out + srow) = pack4(uq[0], uq[1], uq[2], uq[3]);
            }
        }
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int s = mx_scale_exp(amax);
        if (rl < hi) {
            const int ib = i0 + 32 * wn;                     // first column of the block
            uint8_t* hrow = a.h_q + (int64_t)rl * I;
            *(uint32_t*)(hrow + ib + 4 * (lane >> 4)) = e4m3_pack4(hq, s);
            *(uint32_t*)(hrow + ib + 16 + 4 * (lane >> 4)) = e4m3_pack4(hq + 4, s);
            if ((lane >> 4) == 0) a.h_s[(int64_t)rl * (I / 32) + ib / 32] = (uint8_t)(s + 127);
        }
    }
}

// ================================================================ down projection
constexpr int M2_TM = 64, M2_TN = 128;

__global__ __launch_bounds__(256, 2) void k_gemm_down_mx(GemmDownMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SmemMX<M2_TM, M2_TN>::STAGE];
    int e, lo, hi, nt;
    if (!map_mtile<M2_TM>(a.g, a.H / M2_TN, blockIdx.x, e, lo, hi, nt)) return;
    const int n0 = nt * M2_TN;
    const int H = a.H, I = a.I;
    f32x4 acc[2][4];
    RowsDirect da{(const uint16_t*)a.h_q, I / 2, lo, hi - lo};
    ScalesDirect dsa{(const uint32_t*)a.h_s, I / 128, lo, hi - lo};
    RowsDirect db{(const uint16_t*)(a.wd_q + (int64_t)e * H * I), I / 2, n0, M2_TN};
    ScalesDirect dsb{(const uint32_t*)(a.wd_s + (int64_t)e * H * (I / 32)), I / 128, n0, M2_TN};
    LoadKC<M2_TM, RowsDirect> la(da);
    LoadKC<M2_TN, RowsDirect> lb(db);
    LoadScales<M2_TM, ScalesDirect> sa(dsa);
    LoadScales<M2_TN, ScalesDirect> sb(dsb);
    mainloop_mx<M2_TM, M2_TN>(la, lb, sa, sb, I / 128, smem, acc);
    AccPos<M2_TM, M2_TN> pos;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int rl = lo + pos.m(mb);
        if (rl >= hi) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int c = n0 + pos.n(nb);
            const f32x4 v = acc[mb][nb];
            *(uint2*)(a.o + (int64_t)rl * H + c) = pack4(v[0], v[1], v[2], v[3]);
        }
    }
}

// ================================================================ launchers
static inline int mgroup_grid_mx(const GroupRows& g, int TM) {
    if (!g.tile_off) return (g.dense_rows + TM - 1) / TM;
    const int64_t bound = ((int64_t)g.rows + (int64_t)g.E * (TM - 1)) / TM;
    return (int)(bound < g.rows ? bound : g.rows);
}

int launch_gemm_gate_up_mx(const GemmGateUpMXArgs& a, hipStream_t st) {
    ProfScope prof_(st, "gemm_gate_up_mx");
    const int grid = mgroup_grid_mx(a.g, M1_TM) * (a.I / 64);
    if (grid <= 0) return 0;
    k_gemm_gate_up_mx<<<grid, 256, 0, st>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_down_mx(const GemmDownMXArgs& a, hipStream_t st) {
    ProfScope prof_(st, "gemm_down_mx");
    const int grid = mgroup_grid_mx(a.g, M2_TM) * (a.H / M2_TN);
    if (grid <= 0) return 0;
    k_gemm_down_mx<<<grid, 256, 0, st>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
