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
// with XOR-swizzled 16-byte chunks (kc_off: 16 rows read together hit 16
// different bank groups), scales as one 32-bit word (4 blocks) per row.
#include <type_traits>

#include "gemm_common.h"
#include "mx.h"
#include "profile.h"

namespace moe {

typedef int v8i32 __attribute__((ext_vector_type(8)));

// ================================================================ scale sources
// row(r) points at the scale word of row r for K step 0; kstride() is the
// distance in words between K steps.
struct ScalesDirect {          // activations, [rows, K / 128] words
    const uint32_t* base;
    int64_t ld;                // words per row (K / 128)
    int row0, nvalid;
    __device__ const uint32_t* row(int r) const {
        return r < nvalid ? base + (int64_t)(row0 + r) * ld : nullptr;
    }
    __device__ int kstride() const { return 1; }
};

struct ScalesKMajor {          // weights, K-step-major: word (j, r) at j * nrows + r
    const uint32_t* base;
    int nrows;                 // rows of the matrix
    int row0, nvalid;
    __device__ const uint32_t* row(int r) const { return r < nvalid ? base + row0 + r : nullptr; }
    __device__ int kstride() const { return nrows; }
};

struct ScalesGateUp {          // same quarter interleave as RowsGateUp, K-step-major
    const uint32_t* wg;
    const uint32_t* wu;
    int nrows;                 // I
    int i0;
    __device__ const uint32_t* row(int n) const {
        const int q = n >> 5;
        const int i = i0 + ((q >> 1) << 5) + (n & 31);
        return global_select(q & 1, wg, wu) + i;
    }
    __device__ int kstride() const { return nrows; }
};

struct ScalesGather {         // row r = schedule row grow0 + r -> words of its token
    const uint32_t* base;
    int64_t ld;
    const int32_t* slot_of_row;
    int grow0, nvalid, k, S;
    __device__ const uint32_t* row(int r) const {
        if (r >= nvalid) return nullptr;
        const int s = slot_of_row[grow0 + r];
        if ((unsigned)s >= (unsigned)S) return nullptr;
        return base + (int64_t)(s / k) * ld;
    }
    __device__ int kstride() const { return 1; }
};

template <int ROWS, class Src>
struct LoadScales {
    const uint32_t* p;
    uint32_t v;
    int kst;
    __device__ explicit LoadScales(const Src& s) {
        p = threadIdx.x < ROWS ? s.row(threadIdx.x) : nullptr;
        v = 0;
        kst = s.kstride();
    }
    __device__ void load(int kt) { load_off(kt, 0); }
    __device__ void load_off(int kt, int64_t extra) { v = p ? p[extra + (int64_t)kt * kst] : 0u; }
    __device__ void store(uint32_t* s) const {
        if (threadIdx.x < ROWS) s[threadIdx.x] = v;
    }
};

// Rows of two matrices joined along K: K steps [0, nk1) come from the first,
// the rest from the second (the same rows of each).
template <int ROWS>
struct LoadKCCat {
    static constexpr int PER = ROWS * (kTK / 8) / 256;
    const uint16_t* p0[PER];
    const uint16_t* p1[PER];
    int off[PER];
    int nk1;
    uint4 v[PER];
    __device__ LoadKCCat(const RowsDirect& s0, const RowsDirect& s1, int n1) : nk1(n1) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int c = threadIdx.x + 256 * q;
            const int r = c >> 3, kc = c & 7;
            const uint16_t* b0 = s0.row(r);
            const uint16_t* b1 = s1.row(r);
            p0[q] = b0 ? b0 + kc * 8 : nullptr;
            p1[q] = b1 ? b1 + kc * 8 : nullptr;
            off[q] = kc_off(r, kc * 16);
        }
    }
    __device__ void load(int kt) { load_off(kt, 0); }
    // K step kt of the rows `extra` elements further (a later column tile)
    __device__ void load_off(int kt, int64_t extra) {
        const bool second = kt >= nk1;
        const int64_t k = extra + (int64_t)(second ? kt - nk1 : kt) * kTK;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const uint16_t* pb = global_select(second, p0[q], p1[q]);
            v[q] = pb ? *(const uint4*)(pb + k) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ void store(uint16_t* s) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) *(uint4*)(s + off[q]) = v[q];
    }
};

template <int ROWS>
struct LoadScalesCat {         // K-step-major scales of two matrices joined along K
    const uint32_t* p0;
    const uint32_t* p1;
    int kst, nk1;
    uint32_t v;
    __device__ LoadScalesCat(const ScalesKMajor& s0, const ScalesKMajor& s1, int n1)
        : p0(threadIdx.x < ROWS ? s0.row(threadIdx.x) : nullptr),
          p1(threadIdx.x < ROWS ? s1.row(threadIdx.x) : nullptr), kst(s0.kstride()), nk1(n1), v(0) {}
    __device__ void load(int kt) { load_off(kt, 0); }
    __device__ void load_off(int kt, int64_t extra) {
        const bool second = kt >= nk1;
        const uint32_t* pb = global_select(second, p0, p1);
        v = pb ? pb[extra + (int64_t)(second ? kt - nk1 : kt) * kst] : 0u;
    }
    __device__ void store(uint32_t* s) const {
        if (threadIdx.x < ROWS) s[threadIdx.x] = v;
    }
};

// ================================================================ tiles
template <int TM, int TN>
struct SmemMX {
    static constexpr int P = kTK;                     // in uint16: 128-byte swizzled rows (kc_off)
    static constexpr int A = TM * P;                  // uint16 units
    static constexpr int B = TN * P;
    static constexpr int SA = 2 * TM;                 // TM words
    static constexpr int SB = 2 * TN;
    static constexpr int STAGE = A + B + SA + SB;
};

__device__ __forceinline__ v8i32 frag_mx(const uint16_t* s, int rbase) {
    const int lane = lane_id();
    const int row = rbase + (lane & 15);
    const uint4 a = *(const uint4*)(s + kc_off(row, 16 * (lane >> 4)));
    const uint4 b = *(const uint4*)(s + kc_off(row, 64 + 16 * (lane >> 4)));
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
__device__ __forceinline__ void mma_tile_mx_at(const uint16_t* sA, const uint16_t* sB, const uint32_t* cA,
                                               const uint32_t* cB, int wm0, int wn0,
                                               f32x4 (&acc)[TM / 32][TN / 32]) {
    constexpr int MB = TM / 32, NB = TN / 32;
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

// operands in the SmemMX stage layout
template <int TM, int TN>
__device__ __forceinline__ void mma_tile_mx(const uint16_t* st, int wm0, int wn0,
                                            f32x4 (&acc)[TM / 32][TN / 32]) {
    using SM = SmemMX<TM, TN>;
    const uint32_t* cA = (const uint32_t*)(st + SM::A + SM::B);
    mma_tile_mx_at<TM, TN>(st, st + SM::A, cA, cA + TM, wm0, wn0, acc);
}

// The scaled fp8 MFMA started from zero for each 128-code K step, its result
// added to the fp32 accumulator in ascending K order: the MFMA's own
// accumulation then covers one step's 128 products only.
template <int TM, int TN>
__device__ __forceinline__ void mma_tile_mx_stepwise(const uint16_t* st, int wm0, int wn0,
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
        for (int nb = 0; nb < NB; ++nb) {
            const f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fa[nb], fb[mb], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, xa[nb], 0, xb[mb]);
            acc[mb][nb] = f32x4{acc[mb][nb][0] + t[0], acc[mb][nb][1] + t[1], acc[mb][nb][2] + t[2],
                                acc[mb][nb][3] + t[3]};
        }
}

// The same product evaluated on the bf16 MFMA: codes are decoded to bf16 at
// fragment time (an E4M3 value times a power of two has at most 4 significant
// bits, so the decode is exact).  The scaled fp8 MFMA accumulates a 128-product step less
// precisely than fp32 (measured on gfx950: ~5e-5 relative on exactly
// representable operands, vs ~7e-7 for the bf16 MFMA), which flips E4M3 codes
// when its output is quantised again; the GEMMs whose outputs are re-quantised
// (gate/up -> h, down dgrad -> dg, du) use this form.
// Decoding uses the hardware scaled conversion (two E4M3 codes times an fp32
// scale to two bf16); checked on gfx950 against an exact decode of all 256
// codes: exact for power-of-two scales, except that results below 2^-126 are
// flushed to zero (blocks whose largest magnitude is under ~2^-109).
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 frag_mx_bf16(const uint16_t* s, const uint32_t* sc, int rbase, int ks) {
    const int lane = lane_id();
    const int row = rbase + (lane & 15);
    const uint2 c = *(const uint2*)(s + kc_off(row, 32 * ks + 8 * (lane >> 4)));
    const uint32_t e8 = (sc[row] >> (8 * ks)) & 0xffu;
    const float scale = __uint_as_float(e8 ? (e8 << 23) : 0x00400000u);   // 2^(e8 - 127)
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, scale, false));
    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, scale, true));
    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, scale, false));
    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, scale, true));
    return *(const bf16x8*)&v;
}

// MXFP4 (E2M1) operand tiles: 128 codes of a K step are 64 bytes per row,
// stored in the first half of the row's 128-byte LDS slot (four 16-byte
// chunks, swizzled like every KC tile).  Lane group g of a 32-code sub-step
// ks reads the 4 bytes (8 codes) at byte 16 ks + 4 g of its row and decodes
// them exactly with the hardware scaled conversion (checked on gfx950 against
// an exact decode of all 256 byte values: element 2q in the low nibble of
// byte q).
template <int ROWS, class Src, int NTHR = 256>
struct LoadKC4 {
    static constexpr int PER = (ROWS * 4 + NTHR - 1) / NTHR;
    const uint16_t* p[PER];
    int off[PER];
    uint4 v[PER];
    __device__ explicit LoadKC4(const Src& src) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int c = threadIdx.x + NTHR * q;
            const int r = c >> 2, kc = c & 3;
            const uint16_t* b = (c < ROWS * 4) ? src.row(r) : nullptr;
            p[q] = b ? b + kc * 8 : nullptr;
            off[q] = kc_off(r, kc * 16);
        }
    }
    __device__ void load(int kt) { load_off(kt, 0); }
    __device__ void load_off(int kt, int64_t extra) {
#pragma unroll
        for (int q = 0; q < PER; ++q)
            v[q] = p[q] ? *(const uint4*)(p[q] + extra + (int64_t)kt * 32) : make_uint4(0, 0, 0, 0);
    }
    __device__ void store(uint16_t* s) const {
#pragma unroll
        for (int q = 0; q < PER; ++q)
            if (threadIdx.x + NTHR * q < ROWS * 4) *(uint4*)(s + off[q]) = v[q];
    }
};

__device__ __forceinline__ bf16x8 frag_mx4_bf16(const uint16_t* s, const uint32_t* sc, int rbase, int ks) {
    const int lane = lane_id();
    const int row = rbase + (lane & 15);
    const uint32_t c = *(const uint32_t*)(s + kc_off(row, 16 * ks + 4 * (lane >> 4)));
    const uint32_t e8 = (sc[row] >> (8 * ks)) & 0xffu;
    const float scale = __uint_as_float(e8 ? (e8 << 23) : 0x00400000u);   // 2^(e8 - 127)
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0));
    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1));
    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2));
    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3));
    return *(const bf16x8*)&v;
}

template <int TM, int TN, bool B4 = false>
__device__ __forceinline__ void mma_tile_mx_precise(const uint16_t* st, int wm0, int wn0,
                                                    f32x4 (&acc)[TM / 32][TN / 32]) {
    using SM = SmemMX<TM, TN>;
    constexpr int MB = TM / 32, NB = TN / 32;
    const uint16_t* sA = st;
    const uint16_t* sB = st + SM::A;
    const uint32_t* cA = (const uint32_t*)(st + SM::A + SM::B);
    const uint32_t* cB = cA + TM;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        bf16x8 fb[MB], fa[NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) fb[mb] = frag_mx_bf16(sA, cA, wm0 + mb * 16, ks);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (B4) fa[nb] = frag_mx4_bf16(sB, cB, wn0 + nb * 16, ks);
            else fa[nb] = frag_mx_bf16(sB, cB, wn0 + nb * 16, ks);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_16x16x32(fa[nb], fb[mb], acc[mb][nb]);
    }
}

// Double-buffered K loop over 128-code steps.  MODE: how a K step's products
// are formed and summed: MX_ACC, the scaled MFMA accumulating across steps;
// MX_STEPWISE, the scaled MFMA from zero per step, added in fp32; MX_BF16,
// codes decoded exactly to bf16 on the bf16 MFMA (for GEMMs whose outputs
// are quantised again; see the kernels for which each uses).
constexpr int MX_ACC = 0, MX_STEPWISE = 1, MX_BF16 = 2;
constexpr int MX_BF16_B4 = 3;   // as MX_BF16, the B operand in MXFP4 (E2M1 codes)
template <int TM, int TN, int MODE = MX_ACC, class LA, class LB, class SA, class SB>
__device__ __forceinline__ void mainloop_mx(LA& la, LB& lb, SA& sa, SB& sb, int nk, uint16_t* smem,
                                            f32x4 (&acc)[TM / 32][TN / 32], bool keep = false) {
    using SM = SmemMX<TM, TN>;
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * (TM / 2), wn0 = (w >> 1) * (TN / 2);
    if (!keep) zero_acc<TM, TN>(acc);
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
        if constexpr (MODE == MX_BF16) mma_tile_mx_precise<TM, TN>(cur, wm0, wn0, acc);
        else if constexpr (MODE == MX_BF16_B4) mma_tile_mx_precise<TM, TN, true>(cur, wm0, wn0, acc);
        else if constexpr (MODE == MX_STEPWISE) mma_tile_mx_stepwise<TM, TN>(cur, wm0, wn0, acc);
        else mma_tile_mx<TM, TN>(cur, wm0, wn0, acc);
        if (more) put(nxt);
        __syncthreads();
    }
}

// ================================================================ 256 x 256 tiles
// Groups of at least kBigRows rows (see mainloop_big): a 128-code K step is
// 128 bytes per row, the row of a bf16 KC tile, so code tiles are DirectKC
// copies; each row's scale word (four E8M0 scales) is one 4-byte copy, waves
// 0-3 copying A rows 64 (wave & 3) + lane, waves 4-7 the B rows.
// Stage: A codes, B codes, A scale words, B scale words (66 KB).
struct SmemBigMX {
    static constexpr int A = Tile<kBig, false>::SIZE;      // uint16 per code tile
    static constexpr int SC = 2 * kBig;                     // uint16 per kBig scale words
    static constexpr int STAGE = 2 * A + 2 * SC;
};

struct DirectScales {
    const uint32_t* p;             // this lane's row, K step 0
    int kst;                       // words between K steps
    template <class SA, class SB>
    __device__ DirectScales(const SA& sa, const SB& sb, const uint32_t* safe) {
        const int w = threadIdx.x >> 6, r = 64 * (w & 3) + lane_id();
        const uint32_t* b;
        if (w < 4) {
            b = sa.row(r);
            kst = sa.kstride();
        } else {
            b = sb.row(r);
            kst = sb.kstride();
        }
        p = global_select(b == nullptr, b, safe);
    }
    __device__ __forceinline__ void issue(int kt, uint16_t* stage) const {
        const int w = wave_id();
        uint32_t* sc = (uint32_t*)(stage + 2 * SmemBigMX::A) + (w < 4 ? 0 : kBig) + 64 * (w & 3);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(p + (int64_t)kt * kst), (lds_void_t*)sc, 4, 0, 0);
    }
};

// MODE MX_BF16: codes decoded exactly to bf16 (four 32-code sub-steps per K
// step, mma_tile_mx_precise's order); MX_ACC: the scaled fp8 MFMA, one per
// K step (mma_tile_mx_at's).  acc as in mainloop_big.
template <int MODE>
__device__ __forceinline__ void mainloop_big_mx(const DirectKC& la, const DirectKC& lb, const DirectScales& ls,
                                                int nk, uint16_t* st0, uint16_t* st1, f32x4 (&acc)[8][4]) {
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * 128, wn0 = (w >> 1) * 64;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nk <= 0) return;
    la.issue(0, st0);
    lb.issue(0, st0 + SmemBigMX::A);
    ls.issue(0, st0);
    wait_copies();
    __syncthreads();
    // copy slot li of a step (0 .. 8): A codes, B codes, then the scale word
    auto copy = [&](int li, int kt, uint16_t* nxt) {
        if (li < DirectKC::PER) la.issue1(li, kt, nxt);
        else if (li < 2 * DirectKC::PER) lb.issue1(li - DirectKC::PER, kt, nxt + SmemBigMX::A);
        else if (li == 2 * DirectKC::PER) ls.issue(kt, nxt);
    };
    auto step = [&](const uint16_t* cur, uint16_t* nxt, int kt) {
        const bool more = kt + 1 < nk;
        const uint16_t* sA = cur;
        const uint16_t* sB = cur + SmemBigMX::A;
        const uint32_t* cA = (const uint32_t*)(cur + 2 * SmemBigMX::A);
        const uint32_t* cB = cA + kBig;
        if constexpr (MODE == MX_BF16) {
            // row blocks outermost: four B and two A fragments live.  The
            // sub-steps stay a loop (unrolled, the decode of all four is
            // hoisted and spills); the first one, which issues the copies,
            // is peeled so that every copy slot is static.
            auto sub = [&](int ks, bool copies) {
                bf16x8 fa[4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) fa[nb] = frag_mx_bf16(sB, cB, wn0 + nb * 16, ks);
                bf16x8 fb0 = frag_mx_bf16(sA, cA, wm0, ks), fb1;
#pragma unroll
                for (int mb = 0; mb < 8; ++mb) {
                    if (mb + 1 < 8) {
                        if (mb & 1) fb0 = frag_mx_bf16(sA, cA, wm0 + (mb + 1) * 16, ks);
                        else fb1 = frag_mx_bf16(sA, cA, wm0 + (mb + 1) * 16, ks);
                    }
                    if (copies) {
                        copy(mb, kt + 1, nxt);
                        if (mb == 7) copy(8, kt + 1, nxt);
                    }
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[mb][nb] = mfma_16x16x32(fa[nb], (mb & 1) ? fb1 : fb0, acc[mb][nb]);
                }
            };
            sub(0, more);
#pragma unroll 1
            for (int ks = 1; ks < 4; ++ks) sub(ks, false);
        } else {
            v8i32 fa[4];
            int xa[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                fa[nb] = frag_mx(sB, wn0 + nb * 16);
                xa[nb] = scale_mx(cB, wn0 + nb * 16);
            }
            v8i32 fb0 = frag_mx(sA, wm0), fb1;
            int xb0 = scale_mx(cA, wm0), xb1;
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                if (mb + 1 < 8) {
                    if (mb & 1) {
                        fb0 = frag_mx(sA, wm0 + (mb + 1) * 16);
                        xb0 = scale_mx(cA, wm0 + (mb + 1) * 16);
                    } else {
                        fb1 = frag_mx(sA, wm0 + (mb + 1) * 16);
                        xb1 = scale_mx(cA, wm0 + (mb + 1) * 16);
                    }
                }
                if (more) {
                    copy(mb, kt + 1, nxt);
                    if (mb == 7) copy(8, kt + 1, nxt);
                }
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fa[nb], (mb & 1) ? fb1 : fb0, acc[mb][nb], 0, 0, 0, xa[nb], 0, (mb & 1) ? xb1 : xb0);
            }
        }
        wait_copies();
        __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(st0, st1, kt);
        if (kt + 1 < nk) step(st1, st0, kt + 1);
    }
}

// One or two column tiles of one row tile in a single K loop (as
// mainloop_kc_tiles): tile 1's B codes lie bstride uint16 further, its B
// scales bstride_s words further.
template <int TM, int TN, class LA, class LB, class SA, class SB, class EPI>
__device__ __forceinline__ void mainloop_mx_tiles(LA& la, LB& lb, SA& sa, SB& sb, int nk, int ntl,
                                                  int64_t bstride, int64_t bstride_s, uint16_t* smem,
                                                  f32x4 (&acc)[TM / 32][TN / 32], const EPI& epi) {
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
    auto get = [&](int s) {
        const int t = s >= nk ? 1 : 0, kt = s - t * nk;
        la.load(kt);
        lb.load_off(kt, t ? bstride : 0);
        sa.load(kt);
        sb.load_off(kt, t ? bstride_s : 0);
    };
    uint16_t* buf0 = smem;
    uint16_t* buf1 = smem + SM::STAGE;
    get(0);
    put(buf0);
    __syncthreads();
    const int steps = nk * ntl;
    for (int s = 0; s < steps; ++s) {
        uint16_t* cur = (s & 1) ? buf1 : buf0;
        uint16_t* nxt = (s & 1) ? buf0 : buf1;
        const bool more = s + 1 < steps;
        if (more) get(s + 1);
        mma_tile_mx<TM, TN>(cur, wm0, wn0, acc);
        if (more) put(nxt);
        if (s == nk - 1 && more) {
            epi(0, acc);
            zero_acc<TM, TN>(acc);
        }
        __syncthreads();
    }
    epi(ntl - 1, acc);
}

// ================================================================ gate/up + SwiGLU
// Like the bf16 kernel; in addition h = SiLU(g) * u, from the fp32
// accumulators, is quantised along I: each wave holds exactly one 32-wide
// block of h per row (lanes l, l^16, l^32, l^48 share it).
constexpr int M1_TN = 128;     // row tile TM: 64 or 128 (the bf16 GEMMs give the reasons)

template <int TM, bool W4>

__global__ __launch_bounds__(256, 2) void k_gemm_gate_up_mx(GemmGateUpMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SmemMX<TM, M1_TN>::STAGE];
    int e, lo, hi, nt;
    if (!map_mtile<TM>(a.g, a.I / 64, blockIdx.x, e, lo, hi, nt)) return;
    const int i0 = nt * 64;
    const int H = a.H, I = a.I;
    constexpr int WB = W4 ? 2 : 1;              // weight codes per byte
    constexpr int MODE = W4 ? MX_BF16_B4 : MX_BF16;
    f32x4 acc[TM / 32][4];
    const uint16_t* wg = (const uint16_t*)(a.wg_q + (int64_t)e * I * H / WB);
    const uint16_t* wu = (const uint16_t*)(a.wu_q + (int64_t)e * I * H / WB);
    const uint32_t* wgs = (const uint32_t*)(a.wg_s + (int64_t)e * I * (H / 32));
    const uint32_t* wus = (const uint32_t*)(a.wu_s + (int64_t)e * I * (H / 32));
    RowsGateUp db{wg, wu, H / 2 / WB, i0};
    ScalesGateUp ds{wgs, wus, I, i0};
    typename std::conditional<W4, LoadKC4<M1_TN, RowsGateUp>, LoadKC<M1_TN, RowsGateUp>>::type lb(db);
    LoadScales<M1_TN, ScalesGateUp> sb(ds);
    if (a.x_gather) {
        // dispatch fused into the operand loads: a routed row's codes are its
        // token's row of the once-quantised x
        RowsGather da{(const uint16_t*)a.x_q, H / 2, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S,
                      a.g.err};
        ScalesGather dsa{(const uint32_t*)a.x_s, H / 128, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S};
        LoadKC<TM, RowsGather> la(da);
        LoadScales<TM, ScalesGather> sa(dsa);
        mainloop_mx<TM, M1_TN, MODE>(la, lb, sa, sb, H / 128, smem, acc);
    } else {
        RowsDirect da{(const uint16_t*)a.x_q, H / 2, a.xrow0 + lo, hi - lo};
        ScalesDirect dsa{(const uint32_t*)a.x_s, H / 128, a.xrow0 + lo, hi - lo};
        LoadKC<TM, RowsDirect> la(da);
        LoadScales<TM, ScalesDirect> sa(dsa);
        mainloop_mx<TM, M1_TN, MODE>(la, lb, sa, sb, H / 128, smem, acc);
    }
    AccPos<TM, M1_TN> pos;
    const int wn = threadIdx.x >> 7, lane = lane_id();
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) {
        const int rl = lo + pos.m(mb);
        float hq[8];
        float amax = 0.f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // h is quantised from the fp32 accumulators, which are also
                // what the backward reads back (saved g, u are fp32 here)
                hq[4 * nb + r] = swiglu_h(acc[mb][nb][r], acc[mb][nb + 2][r]);
                amax = fmaxf(amax, fabsf(hq[4 * nb + r]));
            }
            if (rl < hi && a.g_out) {       // null: g, u are not kept (recomputed later)
                const int i = i0 + 32 * wn + nb * 16 + 4 * (lane >> 4);
                const int64_t srow = (int64_t)(a.save_row0 + rl) * I + i;
                *(float4*)(a.g_out + srow) = make_float4(acc[mb][nb][0], acc[mb][nb][1],
                                                         acc[mb][nb][2], acc[mb][nb][3]);
                *(float4*)(a.u_out + srow) = make_float4(acc[mb][nb + 2][0], acc[mb][nb + 2][1],
                                                         acc[mb][nb + 2][2], acc[mb][nb + 2][3]);
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

// The groups of at least kBigRows rows in 256 x 256 tiles (MXFP8 weights):
// 256 rows x (128 gate + 128 up columns), each wave's 64 columns the gate and
// up columns of one 32-wide h block, so the epilogue is the one above.
__global__ __launch_bounds__(kBigThreads, 1) void k_gemm_gate_up_mx_big(GemmGateUpMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t st0[SmemBigMX::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st1[SmemBigMX::STAGE];
    int e, lo, hi, nt;
    if (!map_mtile_big(a.g, a.I / (kBig / 2), blockIdx.x, e, lo, hi, nt)) return;
    const int i0 = nt * (kBig / 2);
    const int H = a.H, I = a.I;
    f32x4 acc[8][4];
    {
        const uint16_t* wg = (const uint16_t*)(a.wg_q + (int64_t)e * I * H);
        const uint16_t* wu = (const uint16_t*)(a.wu_q + (int64_t)e * I * H);
        const uint32_t* wgs = (const uint32_t*)(a.wg_s + (int64_t)e * I * (H / 32));
        const uint32_t* wus = (const uint32_t*)(a.wu_s + (int64_t)e * I * (H / 32));
        const RowsGateUp db{wg, wu, H / 2, i0};
        const ScalesGateUp ds{wgs, wus, I, i0};
        const DirectKC lb(db);
        const uint32_t* safe = (const uint32_t*)a.x_s;
        if (a.x_gather) {
            const RowsGather da{(const uint16_t*)a.x_q, H / 2, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S,
                                a.g.err};
            const ScalesGather dsa{(const uint32_t*)a.x_s, H / 128, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S};
            const DirectKC la(da);
            const DirectScales ls(dsa, ds, safe);
            mainloop_big_mx<MX_BF16>(la, lb, ls, H / 128, st0, st1, acc);
        } else {
            const RowsDirect da{(const uint16_t*)a.x_q, H / 2, a.xrow0 + lo, hi - lo};
            const ScalesDirect dsa{(const uint32_t*)a.x_s, H / 128, a.xrow0 + lo, hi - lo};
            const DirectKC la(da);
            const DirectScales ls(dsa, ds, safe);
            mainloop_big_mx<MX_BF16>(la, lb, ls, H / 128, st0, st1, acc);
        }
    }
    const int w = threadIdx.x >> 6, lane = lane_id();
    const int wm0 = (w & 1) * 128, wq = w >> 1;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int rl = lo + wm0 + mb * 16 + (lane & 15);
        float hq[8];
        float amax = 0.f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hq[4 * nb + r] = swiglu_h(acc[mb][nb][r], acc[mb][nb + 2][r]);
                amax = fmaxf(amax, fabsf(hq[4 * nb + r]));
            }
            if (rl < hi && a.g_out) {
                const int i = i0 + 32 * wq + nb * 16 + 4 * (lane >> 4);
                const int64_t srow = (int64_t)(a.save_row0 + rl) * I + i;
                *(float4*)(a.g_out + srow) = make_float4(acc[mb][nb][0], acc[mb][nb][1],
                                                         acc[mb][nb][2], acc[mb][nb][3]);
                *(float4*)(a.u_out + srow) = make_float4(acc[mb][nb + 2][0], acc[mb][nb + 2][1],
                                                         acc[mb][nb + 2][2], acc[mb][nb + 2][3]);
            }
        }
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int s = mx_scale_exp(amax);
        if (rl < hi) {
            const int ib = i0 + 32 * wq;                     // first column of the block
            uint8_t* hrow = a.h_q + (int64_t)rl * I;
            *(uint32_t*)(hrow + ib + 4 * (lane >> 4)) = e4m3_pack4(hq, s);
            *(uint32_t*)(hrow + ib + 16 + 4 * (lane >> 4)) = e4m3_pack4(hq + 4, s);
            if ((lane >> 4) == 0) a.h_s[(int64_t)rl * (I / 32) + ib / 32] = (uint8_t)(s + 127);
        }
    }
}

// ================================================================ down projection
// With 128-row tiles, two neighbouring column tiles per block in one K loop
// (K = I is short).
constexpr int M2_TN = 128;     // row tile TM: 64 or 128 (the bf16 GEMMs give the reasons)

template <int TM, bool W4>

__global__ __launch_bounds__(256, 2) void k_gemm_down_mx(GemmDownMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SmemMX<TM, M2_TN>::STAGE];
    constexpr int NT = W4 ? 1 : short_k_tiles_per_block<TM>();
    const int ncol = a.H / M2_TN;
    int e, lo, hi, np;
    if (!map_mtile<TM>(a.g, (ncol + NT - 1) / NT, blockIdx.x, e, lo, hi, np)) return;
    const int n0 = NT * np * M2_TN;
    const int ntl = min(NT, ncol - NT * np);
    const int H = a.H, I = a.I;
    f32x4 acc[TM / 32][4];
    RowsDirect da{(const uint16_t*)a.h_q, I / 2, lo, hi - lo};
    ScalesDirect dsa{(const uint32_t*)a.h_s, I / 128, lo, hi - lo};
    constexpr int WB = W4 ? 2 : 1;              // weight codes per byte
    RowsDirect db{(const uint16_t*)(a.wd_q + (int64_t)e * H * I / WB), I / 2 / WB, n0, M2_TN};
    ScalesKMajor dsb{(const uint32_t*)(a.wd_s + (int64_t)e * H * (I / 32)), H, n0, M2_TN};
    LoadKC<TM, RowsDirect> la(da);
    typename std::conditional<W4, LoadKC4<M2_TN, RowsDirect>, LoadKC<M2_TN, RowsDirect>>::type lb(db);
    LoadScales<TM, ScalesDirect> sa(dsa);
    LoadScales<M2_TN, ScalesKMajor> sb(dsb);
    AccPos<TM, M2_TN> pos;
    float wr[TM / 32];          // router weight of each row (the combine is a plain sum)
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
                const int col = n0 + t * M2_TN + pos.n(nb);
                const f32x4 v = c[mb][nb];
                *(uint2*)(a.o + orow[mb] * H + col) =
                    pack4(wr[mb] * v[0], wr[mb] * v[1], wr[mb] * v[2], wr[mb] * v[3]);
            }
        }
    };
    if constexpr (W4) {
        // E2M1 weights decoded exactly to bf16 (see frag_mx4_bf16)
        mainloop_mx<TM, M2_TN, MX_BF16_B4>(la, lb, sa, sb, I / 128, smem, acc);
        epi(0, acc);
    } else if constexpr (NT == 1) {
        mainloop_mx<TM, M2_TN>(la, lb, sa, sb, I / 128, smem, acc);
        epi(0, acc);
    } else {
        mainloop_mx_tiles<TM, M2_TN>(la, lb, sa, sb, I / 128, ntl, (int64_t)M2_TN * (I / 2), M2_TN, smem,
                                     acc, epi);
    }
}


// ================================================================ backward: down dgrad
// a = Q(dY) Q(W_down) (reduction over H; dY codes gathered by token, W_down^T
// pre-quantised along H), then in fp32: h = SiLU(g) * u from the saved fp32
// g, u; the dw partial sum of a * h; dh = w a; dg, du.  Writes fp32 h and
// dg | du for the row-wise quantisation of the weight gradients, and dg | du
// quantised along I for the input gradient.  Tile 64 rows x 128 columns of I.
constexpr int M3_TN = 128;     // row tile TM: 64 or 128 (the bf16 GEMMs give the reasons)

template <int TM>

__global__ __launch_bounds__(256, 2) void k_gemm_down_dgrad_mx(GemmDownDgradMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SmemMX<TM, M3_TN>::STAGE];
    __shared__ float red[2][TM];
    int e, lo, hi, nt;
    if (!map_mtile<TM>(a.g, a.I / M3_TN, blockIdx.x, e, lo, hi, nt)) return;
    const int n0 = nt * M3_TN;
    const int H = a.H, I = a.I;
    f32x4 acc[TM / 32][4];
    RowsDirect db{(const uint16_t*)(a.wdt_q + (int64_t)e * I * H), H / 2, n0, M3_TN};
    ScalesKMajor dsb{(const uint32_t*)(a.wdt_s + (int64_t)e * I * (H / 32)), I, n0, M3_TN};
    LoadKC<M3_TN, RowsDirect> lb(db);
    LoadScales<M3_TN, ScalesKMajor> sb(dsb);
    if (a.dy_gather) {
        RowsGather da{(const uint16_t*)a.dy_q, H / 2, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S, a.g.err};
        ScalesGather dsa{(const uint32_t*)a.dy_s, H / 128, a.slot_of_row, a.grow0 + lo, hi - lo, a.k, a.S};
        LoadKC<TM, RowsGather> la(da);
        LoadScales<TM, ScalesGather> sa(dsa);
        mainloop_mx<TM, M3_TN, MX_BF16>(la, lb, sa, sb, H / 128, smem, acc);
    } else {
        RowsDirect da{(const uint16_t*)a.dy_q, H / 2, a.dyrow0 + lo, hi - lo};
        ScalesDirect dsa{(const uint32_t*)a.dy_s, H / 128, a.dyrow0 + lo, hi - lo};
        LoadKC<TM, RowsDirect> la(da);
        LoadScales<TM, ScalesDirect> sa(dsa);
        mainloop_mx<TM, M3_TN, MX_BF16>(la, lb, sa, sb, H / 128, smem, acc);
    }
    AccPos<TM, M3_TN> pos;
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6, wm = wv & 1, wn = wv >> 1;
    float dot[TM / 32], wr[TM / 32];
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) {
        dot[mb] = 0.f;
        wr[mb] = 1.0f;
        const int rl = lo + pos.m(mb);
        if (rl < hi && a.topk_w) {
            const int s = a.slot_of_row[a.grow0 + rl];
            wr[mb] = (unsigned)s < (unsigned)a.S ? a.topk_w[s] : 0.f;
        }
    }
    // The weight gradients' operands h, dg, du are quantised here along the
    // rows of the group (32-row blocks; a tile's rows start on a block of
    // its group) and written transposed, group by group, as
    // launch_mx_quant_group_t lays them out: each quantity in turn is staged
    // in LDS as fp32 (rows past the group as zeros), then each thread takes
    // one column of one 32-row block.
    int gs = 0, np = 32 * ((a.g.dense_rows + 31) / 32);
    int64_t gb = 0;                                  // the group's first 32-row block
    if (a.blk_off) {
        gs = a.g.offsets[e];
        gb = a.blk_off[e];
        np = 32 * (a.blk_off[e + 1] - a.blk_off[e]);
    }
    const int lr0 = lo - gs;                         // the tile's first row in its group
    constexpr int FP = M3_TN + 4;                    // 16 rows of 16 bytes hit 16 bank groups
    static_assert(TM * FP * 4 <= 2 * SmemMX<TM, M3_TN>::STAGE * 2, "the fp32 tile fits the operand stages");
    float* fst = (float*)smem;
    // quantise R staged rows (tile rows rb0 .. rb0 + R - 1) of columns c0 ..
    // c0 + 127 of a matrix of C columns
    auto colquant = [&](const float* src, int R, int rb0, uint8_t* codes, uint8_t* scales, int C, int c0) {
#pragma unroll 1
        for (int u = threadIdx.x; u < M3_TN * (R / 32); u += 256) {
            const int cl = u % M3_TN, b = u / M3_TN;
            const int lr = lr0 + rb0 + 32 * b;       // the block's first row in its group
            if (lr >= np) continue;                  // past the group's padded rows
            const float* col = src + 32 * b * FP + cl;
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(col[j * FP]));
            const int sx = mx_scale_exp(amax);
            const int c = c0 + cl;
            uint8_t* q = codes + 32 * gb * C + (int64_t)c * np + lr;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {             // 16 rows at a time (registers)
                float v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = col[(16 * hb + j) * FP];
                *(uint4*)(q + 16 * hb) = make_uint4(e4m3_pack4(v, sx), e4m3_pack4(v + 4, sx),
                                                    e4m3_pack4(v + 8, sx), e4m3_pack4(v + 12, sx));
            }
            scales[gb * C + (int64_t)c * (np / 32) + lr / 32] = (uint8_t)(sx + 127);
        }
    };
    auto load_gu = [&](int rl, int i, float (&gq)[4], float (&uq)[4]) {
        float4 g4 = make_float4(0.f, 0.f, 0.f, 0.f), u4 = g4;
        if (rl < hi) {
            const int64_t srow = (int64_t)(a.save_row0 + rl) * I + i;
            g4 = *(const float4*)(a.g_saved + srow);
            u4 = *(const float4*)(a.u_saved + srow);
        }
        gq[0] = g4.x; gq[1] = g4.y; gq[2] = g4.z; gq[3] = g4.w;
        uq[0] = u4.x; uq[1] = u4.y; uq[2] = u4.z; uq[3] = u4.w;
    };
    // h (and the router-weight gradient's per-row dots): the whole tile
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) {
        const int rl = lo + pos.m(mb);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            float gq[4], uq[4], hv[4];
            load_gu(rl, n0 + pos.n(nb), gq, uq);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hv[r] = swiglu_h(gq[r], uq[r]);
                dot[mb] += acc[mb][nb][r] * hv[r];
            }
            *(f32x4*)(fst + pos.m(mb) * FP + pos.n(nb)) = f32x4{hv[0], hv[1], hv[2], hv[3]};
        }
    }
    __syncthreads();
    colquant(fst, TM, 0, a.th, a.ths, I, n0);
    // dg and du, the rows of one wave row (TM / 2 rows) at a time (both then
    // fit the LDS); each is also quantised along I for the gate/up input
    // gradient (a 32-column block is 4 lanes x 2 accumulators of one row)
    float* fdg = fst;
    float* fdu = fst + (TM / 2) * FP;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        __syncthreads();                             // the staging area has been read
        if (wm == half) {
#pragma unroll
            for (int mb = 0; mb < TM / 32; ++mb) {
                const int rl = lo + pos.m(mb);
                const int rs = pos.m(mb) - half * (TM / 2);      // row in the staging area
                const bool ok = rl < hi;
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {          // two 32-column blocks of the wave
                    float dgv[8], duv[8];
                    float mg = 0.f, mu = 0.f;
#pragma unroll
                    for (int nbb = 0; nbb < 2; ++nbb) {
                        const int nb = 2 * blk + nbb;
                        float gq[4], uq[4];
                        load_gu(rl, n0 + pos.n(nb), gq, uq);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float dh = wr[mb] * acc[mb][nb][r];
                            const float sg = sigmoidf_(gq[r]);
                            duv[4 * nbb + r] = dh * (gq[r] * sg);
                            dgv[4 * nbb + r] = dh * uq[r] * sg * (1.0f + gq[r] * (1.0f - sg));
                            mg = fmaxf(mg, fabsf(dgv[4 * nbb + r]));
                            mu = fmaxf(mu, fabsf(duv[4 * nbb + r]));
                        }
                        const float z = ok ? 1.f : 0.f;        // rows past the group stage as zeros
                        *(f32x4*)(fdg + rs * FP + pos.n(nb)) =
                            f32x4{z * dgv[4 * nbb], z * dgv[4 * nbb + 1], z * dgv[4 * nbb + 2], z * dgv[4 * nbb + 3]};
                        *(f32x4*)(fdu + rs * FP + pos.n(nb)) =
                            f32x4{z * duv[4 * nbb], z * duv[4 * nbb + 1], z * duv[4 * nbb + 2], z * duv[4 * nbb + 3]};
                    }
                    mg = fmaxf(mg, __shfl_xor(mg, 16));
                    mg = fmaxf(mg, __shfl_xor(mg, 32));
                    mu = fmaxf(mu, __shfl_xor(mu, 16));
                    mu = fmaxf(mu, __shfl_xor(mu, 32));
                    const int sgx = mx_scale_exp(mg), sux = mx_scale_exp(mu);
                    if (ok) {
                        const int ib = n0 + wn * 64 + blk * 32;     // first column of the block
                        uint8_t* qrow = a.dgu_q + (int64_t)rl * (2 * I);
                        *(uint32_t*)(qrow + ib + 4 * (lane >> 4)) = e4m3_pack4(dgv, sgx);
                        *(uint32_t*)(qrow + ib + 16 + 4 * (lane >> 4)) = e4m3_pack4(dgv + 4, sgx);
                        *(uint32_t*)(qrow + I + ib + 4 * (lane >> 4)) = e4m3_pack4(duv, sux);
                        *(uint32_t*)(qrow + I + ib + 16 + 4 * (lane >> 4)) = e4m3_pack4(duv + 4, sux);
                        if ((lane >> 4) == 0) {
                            uint8_t* srow = a.dgu_s + (int64_t)rl * (2 * I / 32);
                            srow[ib / 32] = (uint8_t)(sgx + 127);
                            srow[(I + ib) / 32] = (uint8_t)(sux + 127);
                        }
                    }
                }
            }
        }
        __syncthreads();
        colquant(fdg, TM / 2, half * (TM / 2), a.tdgu, a.tdgus, 2 * I, n0);
        colquant(fdu, TM / 2, half * (TM / 2), a.tdgu, a.tdgus, 2 * I, I + n0);
    }
    if (!a.dw_part) return;
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

// ================================================================ backward: gate/up dgrad
// dX = Q(dg) Q(W_gate) + Q(du) Q(W_up), reductions over I, against the
// transposed pre-quantised weights, in one K loop: the W_gate^T steps, then
// the W_up^T steps; with 128-row tiles a block takes two neighbouring column
// tiles in that loop.
constexpr int M4_TN = 128;     // row tile TM: 64 or 128 (the bf16 GEMMs give the reasons)

template <int TM>

__global__ __launch_bounds__(256, 2) void k_gemm_gu_dgrad_mx(GemmGuDgradMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SmemMX<TM, M4_TN>::STAGE];
    constexpr int NT = short_k_tiles_per_block<TM>();
    const int ncol = a.H / M4_TN;
    int e, lo, hi, np;
    if (!map_mtile<TM>(a.g, (ncol + NT - 1) / NT, blockIdx.x, e, lo, hi, np)) return;
    const int n0 = NT * np * M4_TN;
    const int ntl = min(NT, ncol - NT * np);
    const int H = a.H, I = a.I;
    f32x4 acc[TM / 32][4];
    // one K loop over [dg | du] (2I codes per row) against W_gate^T then W_up^T
    RowsDirect da{(const uint16_t*)a.dgu_q, I, lo, hi - lo};
    ScalesDirect dsa{(const uint32_t*)a.dgu_s, I / 64, lo, hi - lo};
    const int64_t wo = (int64_t)e * H * I;
    RowsDirect dbg{(const uint16_t*)(a.wgt_q + wo), I / 2, n0, M4_TN};
    RowsDirect dbu{(const uint16_t*)(a.wut_q + wo), I / 2, n0, M4_TN};
    ScalesKMajor dsg{(const uint32_t*)(a.wgt_s + wo / 32), H, n0, M4_TN};
    ScalesKMajor dsu{(const uint32_t*)(a.wut_s + wo / 32), H, n0, M4_TN};
    LoadKC<TM, RowsDirect> la(da);
    LoadKCCat<M4_TN> lb(dbg, dbu, I / 128);
    LoadScales<TM, ScalesDirect> sa(dsa);
    LoadScalesCat<M4_TN> sb(dsg, dsu, I / 128);
    AccPos<TM, M4_TN> pos;
    int64_t orow[TM / 32];
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb) orow[mb] = lo + pos.m(mb) < hi ? a.dest.row(lo + pos.m(mb), a.g.err) : -1;
    auto epi = [&](int t, const f32x4 (&c)[TM / 32][4]) {
#pragma unroll
        for (int mb = 0; mb < TM / 32; ++mb) {
            if (orow[mb] < 0) continue;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int col = n0 + t * M4_TN + pos.n(nb);
                const f32x4 v = c[mb][nb];
                *(uint2*)(a.dx + orow[mb] * H + col) = pack4(v[0], v[1], v[2], v[3]);
            }
        }
    };
    if constexpr (NT == 1) {
        mainloop_mx<TM, M4_TN>(la, lb, sa, sb, 2 * I / 128, smem, acc);
        epi(0, acc);
    } else {
        mainloop_mx_tiles<TM, M4_TN>(la, lb, sa, sb, 2 * I / 128, ntl, (int64_t)M4_TN * (I / 2), M4_TN, smem,
                                     acc, epi);
    }
}

// ================================================================ backward: weight gradients
// C_e[m, n] = sum over the expert's padded rows of A^T[m, k] B^T[n, k], both
// operands quantised along rows (32-row blocks) and stored transposed, one
// contiguous [rows][padded K] block per expert, by the group-transpose kernel.  A block owns a 128-row slab of one expert's output
// and walks its 64-column tiles; the A tile stays in LDS when the expert's
// padded rows fit one 128-code K step.
constexpr int X_TM = W_TM, X_TN = W_TN;

struct RowsPadK {              // row r of a transposed operand, from code kb0 on
    const uint8_t* base;
    int64_t ld;                // codes per row
    int row0;
    int64_t kb0;
    __device__ const uint16_t* row(int r) const {
        return (const uint16_t*)(base + (int64_t)(row0 + r) * ld + kb0);
    }
};

template <int ROWS>
struct LoadKCPad {             // K-contiguous fp8 tile; chunks at or past kmax codes read as zero
    static constexpr int PER = ROWS * 8 / 256;
    // thread t, item q: row (t + 256 q) / 8, 16-code chunk t % 8 (the same for
    // every q); addresses are formed at each load to keep few registers live
    RowsPadK src;
    int kmax;
    uint4 v[PER];
    __device__ LoadKCPad(const RowsPadK& s, int kmax_codes) : src(s), kmax(kmax_codes) {}
    __device__ void retarget(int row0) { src.row0 = row0; }   // same K range, other rows
    __device__ void load(int kt) {
        const int kc = threadIdx.x & 7;
        const bool in = kt * 128 + kc * 16 < kmax;
        const uint8_t* b = src.base + src.kb0 + kt * 128 + kc * 16;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int r = (threadIdx.x >> 3) + 32 * q;
            v[q] = in ? *(const uint4*)(b + (int64_t)(src.row0 + r) * src.ld) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ void store(uint16_t* s) const {
        const int kc = threadIdx.x & 7;
#pragma unroll
        for (int q = 0; q < PER; ++q)
            *(uint4*)(s + kc_off((threadIdx.x >> 3) + 32 * q, kc * 16)) = v[q];
    }
};

template <int ROWS>
struct LoadScalesPad {         // scale bytes of blocks at or past nblk read as zero
    const uint8_t* base;
    int64_t ld, b0;
    const uint8_t* p;
    int nblk;
    uint32_t w0, w1, sh, mask;
    __device__ LoadScalesPad(const uint8_t* bs, int64_t l, int row0, int64_t b, int nb)
        : base(bs), ld(l), b0(b), p(nullptr), nblk(nb), w0(0), w1(0), sh(0), mask(0) {
        retarget(row0);
    }
    __device__ void retarget(int row0) {
        p = threadIdx.x < ROWS ? base + (int64_t)(row0 + threadIdx.x) * ld + b0 : nullptr;
    }
    // Four scale bytes from an arbitrary byte address: two aligned words, put
    // together by a byte funnel shift when they are stored, so that neither
    // byte loads nor an early wait hold up the loads issued with them (the
    // words may reach up to 7 bytes past the row; the scale regions keep spare
    // bytes for that).
    __device__ void load(int kt) {
        const int rem = nblk - 4 * kt;
        mask = 0;
        if (!p || rem <= 0) return;
        const uint8_t* q = p + 4 * kt;
        sh = (uint32_t)((uintptr_t)q & 3);
        const uint32_t* w = (const uint32_t*)(q - sh);      // pointer arithmetic keeps it global
        w0 = w[0];
        w1 = w[1];
        mask = rem < 4 ? (1u << (8 * rem)) - 1u : ~0u;
    }
    __device__ void store(uint32_t* s) const {
        if (threadIdx.x < ROWS) s[threadIdx.x] = mask ? __builtin_amdgcn_alignbyte(w1, w0, sh) & mask : 0u;
    }
};

// LDS: the resident A tile and both scale vectors, then one region that holds
// the current B tile and, after its MFMAs, the staged bf16 output tile.
constexpr int X_P = kTK;                                  // uint16 per code row (128 bytes, kc_off)
constexpr int X_CA = X_TM * X_P;                          // A scales: X_TM words
constexpr int X_CB = X_CA + 2 * X_TM;                     // B scales: X_TN words
constexpr int X_REG = X_CB + 2 * X_TN;
constexpr int X_SMEM = X_REG + (X_TM * W_SP > X_TN * X_P ? X_TM * W_SP : X_TN * X_P);
static_assert(X_TM == W_TM && X_TN == W_TN && 64 * W_FP * 2 <= X_TM * W_SP, "WgradEpi's staging fits the region");

// The column-tile walk of one weight-gradient block (A: 128 rows, B: the
// current 64-row column tile).
template <bool BF16_ONLY, bool STREAM>
__device__ __forceinline__ void wgrad_mx_tiles(LoadKCPad<X_TM>& la, LoadScalesPad<X_TM>& sa,
                                               LoadKCPad<X_TN>& lb, LoadScalesPad<X_TN>& sb,
                                               int nk, int nt0, int ntn, int nstride, uint16_t* smem,
                                               const WgradEpi& epi) {
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * (X_TM / 2), wn0 = (w >> 1) * (X_TN / 2);
    uint16_t* region = smem + X_REG;                      // B tile, then the staged output
    uint32_t* cA = (uint32_t*)(smem + X_CA);
    uint32_t* cB = (uint32_t*)(smem + X_CB);
    f32x4 acc[X_TM / 32][X_TN / 32];
    if (nk <= 1) {
        // one K step: A stays in LDS; the next column tile is fetched while the
        // current one is multiplied and written out
        if (nk == 1) {
            la.load(0);
            sa.load(0);
            lb.load(0);
            sb.load(0);
            la.store(smem);
            sa.store(cA);
        }
        for (int i = 0; i < ntn; ++i) {
            zero_acc<X_TM, X_TN>(acc);
            if (nk == 1) {
                if (i > 0) __syncthreads();            // the staged tile i-1 has been written out
                lb.store(region);
                sb.store(cB);
                __syncthreads();
                if (i + 1 < ntn) {
                    lb.retarget((nt0 + (i + 1) * nstride) * X_TN);
                    sb.retarget((nt0 + (i + 1) * nstride) * X_TN);
                    lb.load(0);
                    sb.load(0);
                }
                mma_tile_mx_at<X_TM, X_TN>(smem, region, cA, cB, wm0, wn0, acc);
                __syncthreads();                       // the MFMAs are done with the B tile
            }
            epi.template store<BF16_ONLY, STREAM>(nt0 + i * nstride, acc, region);
        }
        return;
    }
    for (int i = 0; i < ntn; ++i) {
        lb.retarget((nt0 + i * nstride) * X_TN);
        sb.retarget((nt0 + i * nstride) * X_TN);
        zero_acc<X_TM, X_TN>(acc);
        for (int kt = 0; kt < nk; ++kt) {
            la.load(kt);
            sa.load(kt);
            lb.load(kt);
            sb.load(kt);
            __syncthreads();        // the previous step's MFMAs (or staged stores) are done
            la.store(smem);
            sa.store(cA);
            lb.store(region);
            sb.store(cB);
            __syncthreads();
            mma_tile_mx_at<X_TM, X_TN>(smem, region, cA, cB, wm0, wn0, acc);
        }
        __syncthreads();                               // the MFMAs are done with the B tile
        epi.template store<BF16_ONLY, STREAM>(nt0 + i * nstride, acc, region);
    }
}

// STREAM: the slabs' column tiles are dealt over several blocks (streaming
// bf16 stores); a template parameter of the kernel, so that each kernel holds
// two instantiations of the tile walk.  LISTED: the persistent grid of a walk
// over several macrobatches (three blocks per CU) instead of a block per item.
template <bool STREAM, bool LISTED>
__global__ __launch_bounds__(256, LISTED ? 3 : 4) void k_wgrad_mx(WgradMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[X_SMEM];
    const int ntiles = a.N / X_TN, nng = wgrad_groups(ntiles);
    const int nMt = a.M / X_TM;
    const int per = nMt * nng;
    const int64_t mat = (int64_t)(a.msplit == a.M ? a.M : a.msplit) * a.N;   // elements per expert
    // one (expert, slab, column group) item; the group's operands are
    // contiguous [rows][kcodes] blocks (group-major)
    auto item_fn = [&](int e, int mt, int ng) {
        int64_t blk0 = 0;
        int kcodes = 0, rows = 0;
        if (a.g.blk_off) {
            const int lo = a.g.off[e], hi = a.g.off[e + 1];
            if (lo >= 0 && hi >= lo && hi <= a.g.rows) {
                blk0 = a.g.blk_off[e];
                kcodes = 32 * (a.g.blk_off[e + 1] - a.g.blk_off[e]);
                rows = hi - lo;
            }
        } else {
            kcodes = 32 * ((a.g.dense_rows + 31) / 32);
        }
        if (a.g.deep_thr > 0 && kcodes > a.g.deep_thr) return;     // the deep kernel's group
        const int nk = (kcodes + 127) / 128;
        const int m0 = mt * X_TM;
        const bool hi_part = m0 >= a.msplit;
        WgradOut o = hi_part ? a.out_hi : a.out_lo;
        if (wgrad_bind(o, e, rows, mat) < 0) return;               // nothing to add for this expert
        WgradEpi epi{o, (int64_t)e * mat, a.N, hi_part ? m0 - a.msplit : m0};
        const uint8_t* aq = a.at_q + 32 * blk0 * a.M;
        const uint8_t* as_ = a.at_s + blk0 * a.M;
        const uint8_t* bq = a.bt_q + 32 * blk0 * a.N;
        const uint8_t* bs = a.bt_s + blk0 * a.N;
        RowsPadK ra{aq, kcodes, m0, 0};
        LoadKCPad<X_TM> la(ra, kcodes);
        LoadScalesPad<X_TM> sa(as_, kcodes / 32, m0, 0, kcodes / 32);
        const int nt0 = ng, ntn = wgrad_group_tiles(ntiles, nng, ng);
        RowsPadK rb{bq, kcodes, nt0 * X_TN, 0};
        LoadKCPad<X_TN> lb(rb, kcodes);
        LoadScalesPad<X_TN> sb(bs, kcodes / 32, nt0 * X_TN, 0, kcodes / 32);
        if (epi.out.mode == 0) wgrad_mx_tiles<true, STREAM>(la, sa, lb, sb, nk, nt0, ntn, nng, smem, epi);
        else wgrad_mx_tiles<false, false>(la, sa, lb, sb, nk, nt0, ntn, nng, smem, epi);
    };
    if constexpr (LISTED) {
        // a walk over several macrobatches: a persistent grid over the items
        // of the experts with work (block_list; most experts of a skewed
        // stream have no rows in a macrobatch)
        __shared__ int16_t list[1024];
        const int total = per * block_list(a.g.E, [&](int e) {
            const int lo = a.g.off[e], hi = a.g.off[e + 1];
            if (lo < 0 || hi < lo || hi > a.g.rows) return false;
            const int kcodes = 32 * (a.g.blk_off[e + 1] - a.g.blk_off[e]);
            return (a.g.deep_thr <= 0 || kcodes <= a.g.deep_thr) && wgrad_mode(a.out_lo, e, hi - lo) >= 0;
        }, list);
        for (int r = 0;; ++r) {
            const int item = r * (int)gridDim.x + xcd_remap(blockIdx.x, gridDim.x);
            if (item >= total) break;
            if (r) __syncthreads();             // the previous item's staged tile has been read
            const int d = item / per, rem = item - d * per;
            item_fn(list[d], rem / nng, rem % nng);
        }
    } else {
        const int total = (a.g.blk_off ? a.g.E : 1) * per;
        if ((int)blockIdx.x >= total) return;
        const int L = xcd_remap(blockIdx.x, total);
        const int e = L / per, rem = L - e * per;
        item_fn(e, rem / nng, rem % nng);
    }
}

// ---------------------------------------------------------------- deep groups
// Groups past one 128-code K step: 128 x 128 output tiles with the double-
// buffered scaled-MFMA K loop, a persistent grid over (deep group, tile).
constexpr int XD_T = 128, XD_GRID = 512;

__global__ __launch_bounds__(256, 2) void k_wgrad_mx_deep(WgradMXArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SmemMX<XD_T, XD_T>::STAGE];
    const PadGroups& g = a.g;
    const int cnt = g.deep_thr <= 0 ? 0
                  : g.blk_off ? g.deep[0] : (32 * ((g.dense_rows + 31) / 32) > g.deep_thr ? 1 : 0);
    const int nNt = a.N / XD_T, per = (a.M / XD_T) * nNt;
    const int total = cnt * per;
    for (int r = 0, item = deep_item(0); item < total; item = deep_item(++r)) {
        const int d = item / per, tile = item - d * per;
        const int e = g.blk_off ? g.deep[1 + d] : 0;
        int64_t blk0 = 0;
        int kcodes = 32 * ((g.dense_rows + 31) / 32);
        if (g.blk_off) {                                   // offsets validated by the list
            blk0 = g.blk_off[e];
            kcodes = 32 * (g.blk_off[e + 1] - g.blk_off[e]);
        }
        int mt, nt;
        band_tile(tile, per / nNt, nNt, mt, nt);
        const int m0 = mt * XD_T, n0 = nt * XD_T;
        const uint8_t* aq = a.at_q + 32 * blk0 * a.M;
        const uint8_t* as_ = a.at_s + blk0 * a.M;
        const uint8_t* bq = a.bt_q + 32 * blk0 * a.N;
        const uint8_t* bs = a.bt_s + blk0 * a.N;
        RowsPadK ra{aq, kcodes, m0, 0};
        LoadKCPad<XD_T> la(ra, kcodes);
        LoadScalesPad<XD_T> sa(as_, kcodes / 32, m0, 0, kcodes / 32);
        RowsPadK rb{bq, kcodes, n0, 0};
        LoadKCPad<XD_T> lb(rb, kcodes);
        LoadScalesPad<XD_T> sb(bs, kcodes / 32, n0, 0, kcodes / 32);
        f32x4 acc[XD_T / 32][XD_T / 32];
        mainloop_mx<XD_T, XD_T, MX_ACC>(la, lb, sa, sb, (kcodes + 127) / 128, smem, acc);
        const bool hi_part = m0 >= a.msplit;
        WgradOut out = hi_part ? a.out_hi : a.out_lo;
        const int64_t mat = (int64_t)(a.msplit == a.M ? a.M : a.msplit) * a.N;
        if (wgrad_bind(out, e, g.blk_off ? g.off[e + 1] - g.off[e] : g.dense_rows, mat) < 0) continue;
        const int64_t ebase = (int64_t)e * mat;
        const int r0 = hi_part ? m0 - a.msplit : m0;
        static_assert(XD_T == 128 && 128 * W_TFP * 4 <= 2 * SmemMX<XD_T, XD_T>::STAGE * 2, "staging fits");
        staged_tile_store(out, ebase, a.N, r0, n0, acc, (float*)smem);
    }
}

// ================================================================ launchers
static inline int mgroup_grid_mx(const GroupRows& g, int TM) {
    if (!g.tile_off) return (g.dense_rows + TM - 1) / TM;
    const int64_t bound = ((int64_t)g.rows + (int64_t)g.E * (TM - 1)) / TM;
    return (int)(bound < g.rows ? bound : g.rows);
}

#define MOE_LAUNCH_TM_MX(KERNEL, NCOLTILES)                                        \
    do {                                                                           \
        const int tm_ = a.g.tm == 128 ? 128 : 64;                                  \
        const int grid_ = mgroup_grid_mx(a.g, tm_) * (NCOLTILES);                  \
        if (grid_ <= 0) return 0;                                                  \
        if (tm_ == 128) KERNEL<128><<<grid_, 256, 0, st>>>(a);                     \
        else KERNEL<64><<<grid_, 256, 0, st>>>(a);                                 \
        return hipGetLastError() == hipSuccess ? 0 : -1;                           \
    } while (0)

int launch_gemm_gate_up_mx(const GemmGateUpMXArgs& a, hipStream_t st) {
    ProfScope prof_(st, a.w4 ? "gemm_gate_up_mx4" : "gemm_gate_up_mx");
    const bool dims_ok = !a.w4 && a.I % (kBig / 2) == 0 && a.H % 128 == 0;
    const bool dbig = dense_big(a.g, dims_ok);
    if (a.g.tile_big || dbig) {
        if (!dims_ok) return -1;
        const int grid = big_grid(a.g) * (a.I / (kBig / 2));
        if (grid > 0) {
            k_gemm_gate_up_mx_big<<<grid, kBigThreads, 0, st>>>(a);
            if (hipGetLastError() != hipSuccess) return -1;
        }
        if (dbig) return 0;
    }
    const int tm_ = a.g.tm == 128 ? 128 : 64;
    const int grid_ = mgroup_grid_mx(a.g, tm_) * (a.I / 64);
    if (grid_ <= 0) return 0;
    if (a.w4) {
        if (tm_ == 128) k_gemm_gate_up_mx<128, true><<<grid_, 256, 0, st>>>(a);
        else k_gemm_gate_up_mx<64, true><<<grid_, 256, 0, st>>>(a);
    } else {
        if (tm_ == 128) k_gemm_gate_up_mx<128, false><<<grid_, 256, 0, st>>>(a);
        else k_gemm_gate_up_mx<64, false><<<grid_, 256, 0, st>>>(a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_down_mx(const GemmDownMXArgs& a, hipStream_t st) {
    ProfScope prof_(st, a.w4 ? "gemm_down_mx4" : "gemm_down_mx");
    const int ncol = a.H / M2_TN;
    const int tm_ = a.g.tm == 128 ? 128 : 64;
    const int nt_ = a.w4 ? 1 : (tm_ == 128 ? short_k_tiles_per_block<128>() : short_k_tiles_per_block<64>());
    const int grid_ = mgroup_grid_mx(a.g, tm_) * ((ncol + nt_ - 1) / nt_);
    if (grid_ <= 0) return 0;
    if (a.w4) {
        if (tm_ == 128) k_gemm_down_mx<128, true><<<grid_, 256, 0, st>>>(a);
        else k_gemm_down_mx<64, true><<<grid_, 256, 0, st>>>(a);
    } else {
        if (tm_ == 128) k_gemm_down_mx<128, false><<<grid_, 256, 0, st>>>(a);
        else k_gemm_down_mx<64, false><<<grid_, 256, 0, st>>>(a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_down_dgrad_mx(const GemmDownDgradMXArgs& a, hipStream_t st) {
    ProfScope prof_(st, "gemm_down_dgrad_mx");
    MOE_LAUNCH_TM_MX(k_gemm_down_dgrad_mx, a.I / M3_TN);
}

int launch_gemm_gu_dgrad_mx(const GemmGuDgradMXArgs& a, hipStream_t st) {
    ProfScope prof_(st, "gemm_gu_dgrad_mx");
    const int ncol = a.H / M4_TN;
    const int tm_ = a.g.tm == 128 ? 128 : 64;
    const int nt_ = tm_ == 128 ? short_k_tiles_per_block<128>() : short_k_tiles_per_block<64>();
    const int grid_ = mgroup_grid_mx(a.g, tm_) * ((ncol + nt_ - 1) / nt_);
    if (grid_ <= 0) return 0;
    if (tm_ == 128) k_gemm_gu_dgrad_mx<128><<<grid_, 256, 0, st>>>(a);
    else k_gemm_gu_dgrad_mx<64><<<grid_, 256, 0, st>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_wgrad_mx(const WgradMXArgs& a, hipStream_t st) {
    ProfScope prof_(st, a.msplit < a.M ? "wgrad_gate_up_mx" : "wgrad_down_mx");
    if (a.g.deep_thr > 0) {
        k_wgrad_mx_deep<<<XD_GRID, 256, 0, st>>>(a);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    const int ntiles = a.N / X_TN, nng = wgrad_groups(ntiles);
    const bool listed = a.g.blk_off && a.out_lo.counts;        // persistent grid (k_wgrad_mx)
    if (listed && a.g.E > 1024) return -1;                      // the block list's bound
    const int all = (a.g.blk_off ? a.g.E : 1) * (a.M / X_TM) * nng;
    const int grid = listed ? std::min(all, 3 * 256) : all;
    if (grid <= 0) return 0;
    if (nng > 1) {
        if (listed) k_wgrad_mx<true, true><<<grid, 256, 0, st>>>(a);
        else k_wgrad_mx<true, false><<<grid, 256, 0, st>>>(a);
    } else {
        if (listed) k_wgrad_mx<false, true><<<grid, 256, 0, st>>>(a);
        else k_wgrad_mx<false, false><<<grid, 256, 0, st>>>(a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int wgrad_deep_rows_mx() { return 128; }

}  // namespace moe
