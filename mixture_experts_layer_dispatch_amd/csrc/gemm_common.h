// Building blocks of the expert-grouped GEMMs (bf16 and MXFP8): operand
// sources, LDS tiles and loaders, MFMA fragments, the double-buffered K loop,
// and the maps from block id to (expert, tile).  See gemm.hip for the design.
#pragma once

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kTK = 64;

// ================================================================ sources
// Row-major operand whose tile rows are rows of memory (K contiguous).
struct RowsDirect {
    const uint16_t* base;
    int64_t ld;
    int row0, nvalid;
    __device__ const uint16_t* row(int r) const {
        return r < nvalid ? base + (int64_t)(row0 + r) * ld : nullptr;
    }
    __device__ const uint16_t* safe() const { return base; }
};

// Tile row r = schedule row grow0 + r; memory row = token of its slot.
struct RowsGather {
    const uint16_t* base;
    int64_t ld;
    const int32_t* slot_of_row;
    int grow0, nvalid, k, S;
    int32_t* err;
    __device__ const uint16_t* row(int r) const {
        if (r >= nvalid) return nullptr;
        const int s = slot_of_row[grow0 + r];
        if ((unsigned)s >= (unsigned)S) {
            raise_err(err, ERR_BAD_SLOT);
            return nullptr;
        }
        return base + (int64_t)(s / k) * ld;
    }
    __device__ const uint16_t* safe() const { return base; }
};

// Gate/up weight rows interleaved in quarters of 32 so that a wave owns
// matching gate and up columns: tile row n -> quarter q = n / 32,
// q even: W_gate row, q odd: W_up row, both at column i0 + 32*(q/2) + n%32.
struct RowsGateUp {
    const uint16_t* wg;
    const uint16_t* wu;
    int64_t ld;
    int i0;
    __device__ const uint16_t* row(int n) const {
        const int q = n >> 5;
        const int i = i0 + ((q >> 1) << 5) + (n & 31);
        return global_select(q & 1, wg, wu) + (int64_t)i * ld;
    }
    __device__ const uint16_t* safe() const { return wg; }
};

// Operand whose reduction index k is the memory row: krow(k) points at the
// tile's first column in memory row k.
// Every K-row source also splits krow into pre(k) (the loads it needs, issued
// for a whole batch of rows first) and at(k, pre), so that gathered rows cost
// one round trip per batch instead of one per row.
struct KRowsDirect {
    const uint16_t* base;
    int64_t ld;
    int col0, kmax;
    __device__ int pre(int) const { return 0; }
    __device__ const uint16_t* at(int kk, int) const {
        return kk < kmax ? base + (int64_t)kk * ld + col0 : nullptr;
    }
    __device__ const uint16_t* krow(int kk) const { return at(kk, 0); }
};

// k < I: W_gate row k; I <= k < 2I: W_up row k - I.
struct KRowsGateUp {
    const uint16_t* wg;
    const uint16_t* wu;
    int64_t ld;
    int col0, I;
    __device__ int pre(int) const { return 0; }
    __device__ const uint16_t* at(int kk, int) const {
        if (kk < I) return wg + (int64_t)kk * ld + col0;
        if (kk < 2 * I) return wu + (int64_t)(kk - I) * ld + col0;
        return nullptr;
    }
    __device__ const uint16_t* krow(int kk) const { return at(kk, 0); }
};

// k = the k-th row of a group: memory row row0 + k.
struct KRowsGroup {
    const uint16_t* base;
    int64_t ld;
    int row0, n, col0;
    __device__ int pre(int) const { return 0; }
    __device__ const uint16_t* at(int kk, int) const {
        return kk < n ? base + (int64_t)(row0 + kk) * ld + col0 : nullptr;
    }
    __device__ const uint16_t* krow(int kk) const { return at(kk, 0); }
};

// k = the k-th row of a group in schedule rows; memory row = its token.
struct KRowsGroupGather {
    const uint16_t* base;
    int64_t ld;
    const int32_t* slot_of_row;
    int grow0, n, col0, k, S;
    int32_t* err;
    __device__ int pre(int kk) const { return kk < n ? slot_of_row[grow0 + kk] : 0; }
    __device__ const uint16_t* at(int kk, int s) const {
        if (kk >= n) return nullptr;
        if ((unsigned)s >= (unsigned)S) {
            raise_err(err, ERR_BAD_SLOT);
            return nullptr;
        }
        return base + (int64_t)(s / k) * ld + col0;
    }
    __device__ const uint16_t* krow(int kk) const { return at(kk, pre(kk)); }
};

// ================================================================ LDS tiles
// A tile holds ROWS rows (M or N indices) by kTK reduction indices.
//   KC (K contiguous in memory): stored [row][k] in unpadded 128-byte rows
//      (kTK bf16, or 128 fp8 codes); the 16-byte chunk c of row r sits at
//      chunk c ^ ((r >> 1) & 7).  A fragment reads the same chunk of 16 rows:
//      consecutive rows alternate halves of the 64 banks and the swizzle
//      spreads the eight row pairs over the eight chunks, so the 16 reads hit
//      16 different 16-byte bank groups.
//   KS (K is the slow memory axis): stored as it lies in memory, [k][row],
//      pitch ROWS + 16, and read with the LDS transpose load, which hands each
//      lane four consecutive k of one row; the eight k rows read by one
//      32-lane pass land on disjoint 32-byte bank ranges (pitch = 16 mod 32).
template <int ROWS, bool KS>
struct Tile {
    static constexpr int P = KS ? ROWS + 16 : kTK;
    static constexpr int SIZE = KS ? kTK * P : ROWS * P;
};

// LDS (in uint16) that a kernel reserves so that at most two of its blocks
// share a CU: for the weight-streaming GEMMs whose two-block occupancy measured
// faster than three (more concurrent weight streams cost HBM efficiency).
constexpr int kTwoBlocksLds = 160 * 1024 / 3 / 2 + 64;
constexpr int lds_two_blocks(int n) { return n > kTwoBlocksLds ? n : kTwoBlocksLds; }

// uint16 offset in a KC tile of byte `byte` (even) of row r
__device__ __forceinline__ int kc_off(int r, int byte) {
    return r * kTK + (((((byte >> 4) ^ ((r >> 1) & 7)) << 4) | (byte & 15)) >> 1);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Branch-free 16-byte load: a null p reads the always-valid address `safe`
// instead and yields zeros.  Loads guarded by a per-lane branch sit in
// divergent blocks, where the compiler's memory-wait counting falls back to
// waiting for every outstanding load; these never do.  (The zeroing is a
// mask, not a select: a select on a loaded value is turned back into a branch
// around the load.)
__device__ __forceinline__ uint4 ld16_or_zero(const uint16_t* p, const uint16_t* safe) {
    const bool ok = p != nullptr;
    const uint4 x = *(const uint4*)global_select(!ok, p, safe);
    const uint32_t m = 0u - (uint32_t)ok;
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}

// ================================================================ loaders
// KC tile: 16-byte chunks, 8 lanes per 128-byte row segment; NTHR threads
// share the loads.
template <int ROWS, class Src, int NTHR = 256>
struct LoadKC {
    static constexpr int PER = ROWS * (kTK / 8) / NTHR;
    const uint16_t* p[PER];
    int off[PER];
    uint4 v[PER];
    __device__ explicit LoadKC(const Src& src) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int c = threadIdx.x + NTHR * q;
            const int r = c >> 3, kc = c & 7;
            const uint16_t* b = src.row(r);
            p[q] = b ? b + kc * 8 : nullptr;
            off[q] = kc_off(r, kc * 16);
        }
        safe = src.safe();
    }
    const uint16_t* safe;
    __device__ void load(int kt) { load_off(kt, 0); }
    // K step kt of the rows `extra` elements further (a later column tile)
    __device__ void load_off(int kt, int64_t extra) {
#pragma unroll
        for (int q = 0; q < PER; ++q)
            v[q] = p[q] ? *(const uint4*)(p[q] + extra + (int64_t)kt * kTK) : make_uint4(0, 0, 0, 0);
    }
    __device__ void store(uint16_t* s) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) *(uint4*)(s + off[q]) = v[q];
    }
    // Two register stages (R = 0: v, 1: v2) with branch-free loads, for K
    // loops that keep two steps of loads in flight and rely on precise waits.
    uint4 v2[PER];
    template <int R>
    __device__ void load_r(int kt) {
        uint4(&d)[PER] = R ? v2 : v;
#pragma unroll
        for (int q = 0; q < PER; ++q) d[q] = ld16_or_zero(p[q] ? p[q] + (int64_t)kt * kTK : nullptr, safe);
    }
    template <int R>
    __device__ void store_r(uint16_t* s) const {
        const uint4(&d)[PER] = R ? v2 : v;
#pragma unroll
        for (int q = 0; q < PER; ++q) *(uint4*)(s + off[q]) = d[q];
    }
};

// KS tile: copied as it lies in memory, 16 lanes per 256-byte k-row segment.
// src.krow(k) points at the tile's first column in memory row k (or null =
// zeros); src.col0 may be moved between tiles.
template <int ROWS, class Src>
struct LoadKS {
    static constexpr int CPR = ROWS / 8;
    static constexpr int PER = kTK * CPR / 256;
    Src src;
    int kr[PER], cc[PER];
    uint4 v[PER];
    __device__ explicit LoadKS(const Src& s) : src(s) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int c = threadIdx.x + 256 * q;
            kr[q] = c / CPR;
            cc[q] = c % CPR;
        }
    }
    __device__ void load(int kt) { load_off(kt, 0); }
    // K step kt of the columns `extra` elements further (a later column tile)
    __device__ void load_off(int kt, int64_t extra) {
        int pr[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) pr[q] = src.pre(kt * kTK + kr[q]);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const uint16_t* a = src.at(kt * kTK + kr[q], pr[q]);
            v[q] = a ? *(const uint4*)(a + extra + cc[q] * 8) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ void store(uint16_t* s) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) *(uint4*)(s + kr[q] * Tile<ROWS, true>::P + cc[q] * 8) = v[q];
    }
    // Pipelined form for long K loops: load_pipe(kt) uses the row indices the
    // previous call (or prime) fetched and fetches those of step kt + 1, so a
    // gathered source's index load is off the critical path.
    int pn[PER];
    __device__ void prime(int kt) {
#pragma unroll
        for (int q = 0; q < PER; ++q) pn[q] = src.pre(kt * kTK + kr[q]);
    }
    __device__ void load_pipe(int kt) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const uint16_t* a = src.at(kt * kTK + kr[q], pn[q]);
            v[q] = a ? *(const uint4*)(a + cc[q] * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) pn[q] = src.pre((kt + 1) * kTK + kr[q]);
    }
    // Row pointers of K step kt at column 0, kept for loads that only move
    // the column window (src.col0 must be 0 when this is called).
    const uint16_t* rp[PER];
    __device__ void cache_rows(int kt) {
        int pr[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) pr[q] = src.pre(kt * kTK + kr[q]);
#pragma unroll
        for (int q = 0; q < PER; ++q) rp[q] = src.at(kt * kTK + kr[q], pr[q]);
    }
    __device__ void load_cached(int col) {
#pragma unroll
        for (int q = 0; q < PER; ++q)
            v[q] = rp[q] ? *(const uint4*)(rp[q] + col + cc[q] * 8) : make_uint4(0, 0, 0, 0);
    }
};

// ================================================================ fragments
// Natural K order (both operands KC): lane l holds k = ks + 8*(l>>4) + 0..7.
__device__ __forceinline__ bf16x8 frag_kc(const uint16_t* s, int, int rbase, int ks) {
    const int lane = lane_id();
    return *(const bf16x8*)(s + kc_off(rbase + (lane & 15), 2 * (ks + (lane >> 4) * 8)));
}

// Permuted K order, used whenever an operand is KS: lane group g = l>>4 holds
// k = ks + 4g + {0..3} and ks + 16 + 4g + {0..3}.  The MFMA sums over k, so
// the permutation is harmless as long as both operands use it.
__device__ __forceinline__ bf16x8 frag_kc_perm(const uint16_t* s, int, int rbase, int ks) {
    const int lane = lane_id();
    const int row = rbase + (lane & 15);
    const uint2 a = *(const uint2*)(s + kc_off(row, 2 * (ks + 4 * (lane >> 4))));
    const uint2 b = *(const uint2*)(s + kc_off(row, 2 * (ks + 16 + 4 * (lane >> 4))));
    const uint4 v = make_uint4(a.x, a.y, b.x, b.y);
    return *(const bf16x8*)&v;
}

// Transpose load of a 16-lane group: lane i receives element (i % 4) of the
// 8-byte chunk addressed by lane 4r + i/4, for r = 0..3.  Lane j therefore
// addresses k row ks + 4g + j/4 at columns rbase + 4*(j%4), and every lane ends
// up with four consecutive k of row rbase + (lane & 15).
__device__ __forceinline__ bf16x8 frag_ks(const uint16_t* s, int P, int rbase, int ks) {
    const int lane = lane_id();
    const int g = lane >> 4, j = lane & 15;
    const uint16_t* p = s + (ks + 4 * g + (j >> 2)) * P + rbase + 4 * (j & 3);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 16 * P));
    const uint4 v = make_uint4(__builtin_bit_cast(uint2, a).x, __builtin_bit_cast(uint2, a).y,
                               __builtin_bit_cast(uint2, b).x, __builtin_bit_cast(uint2, b).y);
    return *(const bf16x8*)&v;
}

template <bool KS, bool PERM>
__device__ __forceinline__ bf16x8 frag(const uint16_t* s, int P, int rbase, int ks) {
    if constexpr (KS) return frag_ks(s, P, rbase, ks);
    else if constexpr (PERM) return frag_kc_perm(s, P, rbase, ks);
    else return frag_kc(s, P, rbase, ks);
}

// ================================================================ main loop
// sA: TM rows (output rows), sB: TN rows (output columns).  The MFMA takes the
// column operand first, so each lane's four accumulators are four consecutive
// output columns.
template <int TM, int TN, bool AKS, bool BKS>
__device__ __forceinline__ void mma_tile(const uint16_t* sA, const uint16_t* sB, int wm0, int wn0,
                                         f32x4 (&acc)[TM / 32][TN / 32]) {
    constexpr int MB = TM / 32, NB = TN / 32;
    constexpr bool PERM = AKS || BKS;
    constexpr int PA = Tile<TM, AKS>::P, PB = Tile<TN, BKS>::P;
#pragma unroll
    for (int ks = 0; ks < kTK; ks += 32) {
        bf16x8 fb[MB], fa[NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) fb[mb] = frag<AKS, PERM>(sA, PA, wm0 + mb * 16, ks);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) fa[nb] = frag<BKS, PERM>(sB, PB, wn0 + nb * 16, ks);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_16x16x32(fa[nb], fb[mb], acc[mb][nb]);
    }
}

template <int TM, int TN>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[TM / 32][TN / 32]) {
#pragma unroll
    for (int mb = 0; mb < TM / 32; ++mb)
#pragma unroll
        for (int nb = 0; nb < TN / 32; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int TM, int TN, bool AKS, bool BKS>
struct Smem {
    static constexpr int A = Tile<TM, AKS>::SIZE;
    static constexpr int B = Tile<TN, BKS>::SIZE;
    static constexpr int STAGE = A + B;
};

// Double-buffered K loop, one barrier per step.
template <int TM, int TN, bool AKS, bool BKS, class LA, class LB>
__device__ __forceinline__ void mainloop(LA& la, LB& lb, int nk, uint16_t* smem,
                                         f32x4 (&acc)[TM / 32][TN / 32]) {
    using SM = Smem<TM, TN, AKS, BKS>;
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * (TM / 2), wn0 = (w >> 1) * (TN / 2);
    zero_acc<TM, TN>(acc);
    if (nk <= 0) return;
    uint16_t* buf0 = smem;
    uint16_t* buf1 = smem + SM::STAGE;
    la.load(0);
    lb.load(0);
    la.store(buf0);
    lb.store(buf0 + SM::A);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        uint16_t* cur = (kt & 1) ? buf1 : buf0;
        uint16_t* nxt = (kt & 1) ? buf0 : buf1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(kt + 1);
            lb.load(kt + 1);
        }
        mma_tile<TM, TN, AKS, BKS>(cur, cur + SM::A, wm0, wn0, acc);
        if (more) {
            la.store(nxt);
            lb.store(nxt + SM::A);
        }
        __syncthreads();
    }
}

// Eight-wave blocks (512 threads) for GEMMs that are MFMA work: the block
// tile is TM x TNB with both operands KC, the waves form a 2 x 4 grid and
// each computes a (TM/2) x (TNB/4) tile (one wave's share of
// mma_tile<TM, TNB/2>).  A CU holds one such block, so the loads are issued
// two K steps ahead (two register stages, two LDS buffers): with one step in
// flight every barrier waited for the next step's loads.  The loop body issues
// its loads unconditionally (the last steps run in a tail), so each wait
// covers only the older stage.
template <int TM, int TNB>
struct SmemW8 {
    static constexpr int A = Tile<TM, false>::SIZE;
    static constexpr int B = Tile<TNB, false>::SIZE;
    static constexpr int STAGE = A + B;
};

template <int TM, int TNB, class LA, class LB>
__device__ __forceinline__ void mainloop_w8(LA& la, LB& lb, int nk, uint16_t* smem,
                                            f32x4 (&acc)[TM / 32][TNB / 64]) {
    using SM = SmemW8<TM, TNB>;
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * (TM / 2), wn0 = (w >> 1) * (TNB / 4);
    zero_acc<TM, TNB / 2>(acc);
    if (nk <= 0) return;
    uint16_t* buf0 = smem;
    uint16_t* buf1 = smem + SM::STAGE;
    auto mma = [&](const uint16_t* b) { mma_tile<TM, TNB / 2, false, false>(b, b + SM::A, wm0, wn0, acc); };
    la.template load_r<0>(0);
    lb.template load_r<0>(0);
    if (nk > 1) {
        la.template load_r<1>(1);
        lb.template load_r<1>(1);
    }
    la.template store_r<0>(buf0);
    lb.template store_r<0>(buf0 + SM::A);
    __syncthreads();
    int kt = 0;
    // steps kt, kt + 1: buf0 holds kt, stage 1 holds kt + 1, stage 0 is free
    for (; kt + 3 < nk; kt += 2) {
        la.template load_r<0>(kt + 2);
        lb.template load_r<0>(kt + 2);
        mma(buf0);
        la.template store_r<1>(buf1);
        lb.template store_r<1>(buf1 + SM::A);
        __syncthreads();
        la.template load_r<1>(kt + 3);
        lb.template load_r<1>(kt + 3);
        mma(buf1);
        la.template store_r<0>(buf0);
        lb.template store_r<0>(buf0 + SM::A);
        __syncthreads();
    }
    const int rest = nk - kt;              // the last one to three steps
    if (rest == 3) {
        la.template load_r<0>(kt + 2);
        lb.template load_r<0>(kt + 2);
    }
    mma(buf0);
    if (rest == 1) return;
    la.template store_r<1>(buf1);
    lb.template store_r<1>(buf1 + SM::A);
    __syncthreads();
    mma(buf1);
    if (rest == 2) return;
    la.template store_r<0>(buf0);        // buf0 is free since the last barrier
    lb.template store_r<0>(buf0 + SM::A);
    __syncthreads();
    mma(buf0);
}

// Column tiles per block of the GEMMs with a short K loop (down projection,
// gate/up input gradient): two with 128-row tiles (large groups, where the
// GEMM is MFMA work and the pipeline fill of a short K loop shows), one with
// 64-row tiles (small groups stream weights: more blocks in flight measured
// faster).
template <int TM>
constexpr int short_k_tiles_per_block() { return TM == 128 ? 2 : 1; }

// One or two column tiles of one row tile in a single K loop: steps [0, nk)
// for tile 0 and [nk, 2 nk) for tile 1, whose B operand lies bstride elements
// further.  The loads of tile 1's first step are in flight
// while tile 0's epilogue, epi(0, acc), stores its outputs, so a short K loop
// does not pay the pipeline fill once per tile.
template <int TM, int TN, bool AKS, bool BKS, class LA, class LB, class EPI>
__device__ __forceinline__ void mainloop_tiles(LA& la, LB& lb, int nk, int ntl, int64_t bstride,
                                               uint16_t* smem, f32x4 (&acc)[TM / 32][TN / 32],
                                               const EPI& epi) {
    using SM = Smem<TM, TN, AKS, BKS>;
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * (TM / 2), wn0 = (w >> 1) * (TN / 2);
    zero_acc<TM, TN>(acc);
    if (nk <= 0) return;
    uint16_t* buf0 = smem;
    uint16_t* buf1 = smem + SM::STAGE;
    la.load(0);
    lb.load_off(0, 0);
    la.store(buf0);
    lb.store(buf0 + SM::A);
    __syncthreads();
    const int steps = nk * ntl;
    for (int s = 0; s < steps; ++s) {
        uint16_t* cur = (s & 1) ? buf1 : buf0;
        uint16_t* nxt = (s & 1) ? buf0 : buf1;
        const bool more = s + 1 < steps;
        if (more) {
            const int t1 = s + 1 >= nk ? 1 : 0;
            la.load(s + 1 - t1 * nk);
            lb.load_off(s + 1 - t1 * nk, t1 ? bstride : 0);
        }
        mma_tile<TM, TN, AKS, BKS>(cur, cur + SM::A, wm0, wn0, acc);
        if (more) {
            la.store(nxt);
            lb.store(nxt + SM::A);
        }
        if (s == nk - 1 && more) {
            epi(0, acc);
            zero_acc<TM, TN>(acc);
        }
        __syncthreads();
    }
    epi(ntl - 1, acc);
}

// The same K loop for KS operands whose rows may be gathered: index loads run
// one K step ahead of the data loads they feed.
template <int TM, int TN, class LA, class LB>
__device__ __forceinline__ void mainloop_ks_pipe(LA& la, LB& lb, int nk, uint16_t* smem,
                                                 f32x4 (&acc)[TM / 32][TN / 32]) {
    using SM = Smem<TM, TN, true, true>;
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * (TM / 2), wn0 = (w >> 1) * (TN / 2);
    zero_acc<TM, TN>(acc);
    if (nk <= 0) return;
    uint16_t* buf0 = smem;
    uint16_t* buf1 = smem + SM::STAGE;
    la.prime(0);
    lb.prime(0);
    la.load_pipe(0);
    lb.load_pipe(0);
    la.store(buf0);
    lb.store(buf0 + SM::A);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        uint16_t* cur = (kt & 1) ? buf1 : buf0;
        uint16_t* nxt = (kt & 1) ? buf0 : buf1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load_pipe(kt + 1);
            lb.load_pipe(kt + 1);
        }
        mma_tile<TM, TN, true, true>(cur, cur + SM::A, wm0, wn0, acc);
        if (more) {
            la.store(nxt);
            lb.store(nxt + SM::A);
        }
        __syncthreads();
    }
}

// ================================================================ 256 x 256 tiles
// Groups of hundreds of rows or more (each weight tile then feeds hundreds of
// output rows, and the GEMM is MFMA work): 512-thread blocks of 256 x 256
// output, eight waves in a 2 (rows) x 4 (columns) grid, each 128 x 64.  Per
// 64-deep K step a block reads 64 KB of operands for 8.4 MFLOP (128 flop per
// byte from L2, twice the 128 x 128 tile's), and each wave reads 24 KB of
// fragments from LDS for 64 MFMAs.  Operands go from global memory straight
// into LDS (gfx950's global_load_lds, 16 bytes per lane, no register
// staging) in the swizzled KC layout, two stages of 64 KB; the copies of the
// next step go out together after the step's first fragment reads, so they
// fly while the current step computes (spread one per column block, the
// gate/up input gradient took 0.40 instead of 0.37 ms on the expert-parallel
// share).
constexpr int kBigThreads = 512;       // kBig, kBigRows: launch.h

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// KC tile of kBig rows by kTK: the 16-byte chunk g = q * 512 + wave * 64 + lane
// of the tile (row g / 8, slot g % 8) is loaded by lane `lane` of wave `wave`
// in its q-th copy; slot s of row r holds chunk s ^ ((r >> 1) & 7) of the row,
// the layout kc_off describes.  Rows the source does not have read its safe
// row instead (their results are never stored).
struct DirectKC {
    static constexpr int PER = kBig * (kTK / 8) / kBigThreads;
    const uint16_t* p[PER];
    template <class Src>
    __device__ explicit DirectKC(const Src& src) {
        const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int g = q * kBigThreads + w * 64 + lane;
            const int r = g >> 3, c = (g & 7) ^ ((r >> 1) & 7);
            const uint16_t* b = src.row(r);
            p[q] = (b ? b : src.safe()) + c * 8;
        }
    }
    __device__ __forceinline__ void issue1(int q, int kt, uint16_t* tile) const {
        const int w = wave_id();
        __builtin_amdgcn_global_load_lds((glb_void_t*)(p[q] + (int64_t)kt * kTK),
                                         (lds_void_t*)(tile + (q * kBigThreads + w * 64) * 8), 16, 0, 0);
    }
    __device__ __forceinline__ void issue(int kt, uint16_t* tile) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) issue1(q, kt, tile);
    }
};

// KS tile of kTK k-rows by kBig columns, unpadded 512-byte k-rows whose
// 16-byte chunks are XOR-swizzled by k: chunk c of k-row k sits at slot
// c ^ (2 (k & 7)).  The transpose load of a fragment reads 32 bytes (two
// chunks c, c + 1, c even) from each of 8 consecutive k-rows per half-wave;
// the swizzle moves the pair to 8 different 32-byte bank windows.  Chunk
// g = q * 512 + wave * 64 + lane (k-row g / 32, slot g % 32) is copied by that
// lane.  src.step(kt) points at column col0 of k-row kt * kTK; the step's k-rows
// follow at stride src.ld.
struct DirectKS {
    static constexpr int PER = kTK * (kBig / 8) / kBigThreads;
    int off[PER];
    __device__ explicit DirectKS(int64_t ld) {
        const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int g = q * kBigThreads + w * 64 + lane;
            const int k = g >> 5, c = (g & 31) ^ ((k & 7) << 1);
            off[q] = (int)(k * ld) + c * 8;
        }
    }
    __device__ __forceinline__ void issue1(int q, const uint16_t* base, uint16_t* tile) const {
        const int w = wave_id();
        __builtin_amdgcn_global_load_lds((glb_void_t*)(base + off[q]),
                                         (lds_void_t*)(tile + (q * kBigThreads + w * 64) * 8), 16, 0, 0);
    }
};

// element offset of (k-row k, column col) in a DirectKS tile
__device__ __forceinline__ int ks_sw_off(int k, int col) {
    return k * kBig + ((((col >> 3) ^ ((k & 7) << 1))) << 3) + (col & 7);
}

// the B-side fragment of frag_ks from a DirectKS tile (same lanes and k order)
__device__ __forceinline__ bf16x8 frag_ks_sw(const uint16_t* s, int rbase, int ks) {
    const int lane = lane_id();
    const int g = lane >> 4, j = lane & 15;
    const int k1 = ks + 4 * g + (j >> 2), col = rbase + 4 * (j & 3);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(s + ks_sw_off(k1, col)));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(s + ks_sw_off(k1 + 16, col)));
    const uint4 v = make_uint4(__builtin_bit_cast(uint2, a).x, __builtin_bit_cast(uint2, a).y,
                               __builtin_bit_cast(uint2, b).x, __builtin_bit_cast(uint2, b).y);
    return *(const bf16x8*)&v;
}

// K-step bases of a matrix read with k as the memory row, at column col0
struct StepRows {
    const uint16_t* base;
    int64_t ld;
    int col0;
    __device__ const uint16_t* step(int kt) const { return base + (int64_t)kt * kTK * ld + col0; }
};

// K-step bases of [W_gate; W_up] read with k as the memory row (k < I: W_gate
// row k, else W_up row k - I; I a multiple of kTK), at column col0
struct StepGateUp {
    const uint16_t* wg;
    const uint16_t* wu;
    int64_t ld;
    int col0, I;
    __device__ const uint16_t* step(int kt) const {
        const int k = kt * kTK;
        return (k < I ? wg + (int64_t)k * ld : wu + (int64_t)(k - I) * ld) + col0;
    }
};

struct SmemBig {
    static constexpr int A = Tile<kBig, false>::SIZE;     // uint16 per operand tile
    static constexpr int STAGE = 2 * A;                   // A then B; two stages: 128 KB
};

// wait for every copy this thread issued (vmcnt 0; the expcnt and lgkmcnt
// fields left at their maxima would not wait, but lgkmcnt 0 is harmless here)
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0070); }

// acc[mb][nb]: output rows wm0 + 16 mb + (lane & 15), columns wn0 + 16 nb +
// 4 (lane >> 4) + r, with wm0 = 128 (wave & 1), wn0 = 64 (wave >> 1).
// B is a DirectKC tile (LB = DirectKC), or a DirectKS tile over the k-rows
// of src (LB = DirectKS, src.step(kt)); with a KS operand both operands use
// the permuted K order of frag_kc_perm / frag_ks (the 128-row kernels' order,
// so the bits are theirs).
template <class LB, class SrcB>
__device__ __forceinline__ void big_issue_b(const LB& lb, const SrcB& sb, int q, int kt, uint16_t* tile) {
    if constexpr (__is_same(LB, DirectKC)) lb.issue1(q, kt, tile);
    else lb.issue1(q, sb.step(kt), tile);
}

template <class LB, class SrcB>
__device__ __forceinline__ void mainloop_big(const DirectKC& la, const LB& lb, const SrcB& sb, int nk,
                                             uint16_t* st0, uint16_t* st1, f32x4 (&acc)[8][4]) {
    constexpr bool BKS = __is_same(LB, DirectKS);
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * 128, wn0 = (w >> 1) * 64;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nk <= 0) return;
    la.issue(0, st0);
#pragma unroll
    for (int q = 0; q < LB::PER; ++q) big_issue_b(lb, sb, q, 0, st0 + SmemBig::A);
    wait_copies();
    __syncthreads();
    auto fa_of = [&](const uint16_t* sB, int nb, int ks) {
        if constexpr (BKS) return frag_ks_sw(sB, wn0 + nb * 16, ks);
        else return frag_kc(sB, 0, wn0 + nb * 16, ks);
    };
    // one K step on cur while the next step's copies go to nxt; the two
    // stages are separate LDS arrays, so the compiler can tell the copies
    // into one from the reads of the other (it waits for every copy in flight
    // before an LDS read it cannot tell apart from them)
    auto step = [&](const uint16_t* cur, uint16_t* nxt, int kt) {
        const bool more = kt + 1 < nk;
        const uint16_t* sA = cur;
        const uint16_t* sB = cur + SmemBig::A;
        // row blocks outermost: four B fragments and three A fragments live at
        // a time, each A fragment fetched two row blocks ahead (B outermost,
        // with all eight A fragments loaded first, ran the gate/up input
        // gradient 0.343 -> 0.365 ms on the expert-parallel share; one row
        // block ahead, 1-2 % slower than two)
#pragma unroll
        for (int ks = 0; ks < kTK; ks += 32) {
            bf16x8 fa[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) fa[nb] = fa_of(sB, nb, ks);
            auto fbm = [&](int mb) {
                if constexpr (BKS) return frag_kc_perm(sA, 0, wm0 + mb * 16, ks);
                else return frag_kc(sA, 0, wm0 + mb * 16, ks);
            };
            bf16x8 fbr[3];
            fbr[0] = fbm(0);
            fbr[1] = fbm(1);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                if (mb + 2 < 8) fbr[(mb + 2) % 3] = fbm(mb + 2);
                if (more && ks == 0 && mb == 0) {       // the next step's eight copies
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        if (q < DirectKC::PER) la.issue1(q, kt + 1, nxt);
                        else big_issue_b(lb, sb, q - DirectKC::PER, kt + 1, nxt + SmemBig::A);
                    }
                }
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_16x16x32(fa[nb], fbr[mb % 3], acc[mb][nb]);
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

// 256 x 256 tiles: the routed groups of tile_big, or a dense group of at
// least kBigRows rows (then alone)
// (routed groups: the caller builds tile_big only when every GEMM that takes
// it has a 256 x 256 form for its sizes; a launcher that cannot take it fails)
static inline bool dense_big(const GroupRows& g, bool dims_ok) {
    return !g.tile_off && g.tm == 128 && g.dense_rows >= kBigRows && dims_ok;
}

static inline int big_grid(const GroupRows& g) {
    if (!g.tile_off) return (g.dense_rows + kBig - 1) / kBig;
    // groups of n >= kBigRows rows take ceil(n / kBig) <= n / 128 tiles
    const int64_t a = (int64_t)g.rows / 128, b = ((int64_t)g.rows + (int64_t)g.E * (kBig - 1)) / kBig;
    return (int)(a < b ? a : b);
}

// ---------------------------------------------------------------- 256 x 256, K-grouped
// KS tile of kTK k-rows by kBig columns whose k-rows come one by one from a
// K-row source (src.pre / src.at: the k-th row of a group at column col0, or
// null past the group's end or for a bad slot).  Missing rows are copied from
// a zero row, so they add exact zeros, as the zero-filled tiles of the
// 128 x 128 kernels do.  src.pre(k) (a gathered row's slot) is fetched two K
// steps before the copy that needs it: prime(kt) fills pn for step kt,
// ahead(kt) fills pn2, advance() moves pn2 to pn.
template <class Src>
struct DirectKSRows {
    static constexpr int PER = kTK * (kBig / 8) / kBigThreads;
    // copy q of a lane covers k-row k0 + 16 q; its chunk slot (lane & 31) and
    // the k-row's swizzle ((k0 & 7), the same for every q) fix the column
    Src src;
    const uint16_t* zero;             // kBig zero elements
    int k0, co, pn[PER], pn2[PER];
    __device__ DirectKSRows(const Src& s, const uint16_t* z) : src(s), zero(z) {
        const int lane = lane_id(), w = threadIdx.x >> 6;
        k0 = (w * 64 + lane) >> 5;
        co = ((lane & 31) ^ ((k0 & 7) << 1)) * 8;
    }
    __device__ __forceinline__ void prime(int kt) {
#pragma unroll
        for (int q = 0; q < PER; ++q) pn[q] = src.pre(kt * kTK + k0 + 16 * q);
    }
    __device__ __forceinline__ void ahead(int kt) {
#pragma unroll
        for (int q = 0; q < PER; ++q) pn2[q] = src.pre(kt * kTK + k0 + 16 * q);
    }
    __device__ __forceinline__ void advance() {
#pragma unroll
        for (int q = 0; q < PER; ++q) pn[q] = pn2[q];
    }
    __device__ __forceinline__ void issue1(int q, int kt, uint16_t* tile) const {
        const int w = wave_id();
        const uint16_t* r = src.at(kt * kTK + k0 + 16 * q, pn[q]);
        const uint16_t* p = global_select(r == nullptr, r, zero) + co;
        __builtin_amdgcn_global_load_lds((glb_void_t*)p, (lds_void_t*)(tile + (q * kBigThreads + w * 64) * 8),
                                         16, 0, 0);
    }
};

// C[256 x 256] = sum over the group's rows of A[r, m0 + .] (x) B[r, n0 + .],
// both operands DirectKSRows tiles read with the transpose load (the K order
// and the bits of the 128 x 128 kernels).  acc as in mainloop_big.
template <class LA, class LB>
__device__ __forceinline__ void mainloop_big_kk(LA& la, LB& lb, int nk, uint16_t* st0, uint16_t* st1,
                                                f32x4 (&acc)[8][4]) {
    const int w = threadIdx.x >> 6;
    const int wm0 = (w & 1) * 128, wn0 = (w >> 1) * 64;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nk <= 0) return;
    la.prime(0);
    lb.prime(0);
#pragma unroll
    for (int q = 0; q < LA::PER; ++q) la.issue1(q, 0, st0);
#pragma unroll
    for (int q = 0; q < LB::PER; ++q) lb.issue1(q, 0, st0 + SmemBig::A);
    if (nk > 1) {
        la.prime(1);
        lb.prime(1);
    }
    wait_copies();
    __syncthreads();
    auto step = [&](const uint16_t* cur, uint16_t* nxt, int kt) {
        const bool more = kt + 1 < nk, ahead = kt + 2 < nk;
        if (ahead) {
            la.ahead(kt + 2);
            lb.ahead(kt + 2);
        }
        const uint16_t* sA = cur;
        const uint16_t* sB = cur + SmemBig::A;
        // the row blocks outermost: four B fragments and two A fragments live
        // at a time (each accumulator still sees its MFMAs in K order)
#pragma unroll
        for (int ks = 0; ks < kTK; ks += 32) {
            bf16x8 fa[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) fa[nb] = frag_ks_sw(sB, wn0 + nb * 16, ks);
            bf16x8 fb0 = frag_ks_sw(sA, wm0, ks), fb1;
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                if (mb + 1 < 8) {
                    if (mb & 1) fb0 = frag_ks_sw(sA, wm0 + (mb + 1) * 16, ks);
                    else fb1 = frag_ks_sw(sA, wm0 + (mb + 1) * 16, ks);
                }
                if (more && ks == 0 && mb == 0) {      // the next step's copies, together
#pragma unroll
                    for (int q = 0; q < LA::PER + LB::PER; ++q) {
                        if (q < LA::PER) la.issue1(q, kt + 1, nxt);
                        else lb.issue1(q - LA::PER, kt + 1, nxt + SmemBig::A);
                    }
                }
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_16x16x32(fa[nb], (mb & 1) ? fb1 : fb0, acc[mb][nb]);
            }
        }
        if (ahead) {
            la.advance();
            lb.advance();
        }
        wait_copies();
        __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(st0, st1, kt);
        if (kt + 1 < nk) step(st1, st0, kt + 1);
    }
}

// both operands DirectKC
struct NoSrc {};
__device__ __forceinline__ void mainloop_big(const DirectKC& la, const DirectKC& lb, int nk, uint16_t* st0,
                                             uint16_t* st1, f32x4 (&acc)[8][4]) {
    mainloop_big(la, lb, NoSrc{}, nk, st0, st1, acc);
}

// accumulator (mb, nb, r) -> tile coordinates
template <int TM, int TN>
struct AccPos {
    int m_base, n_base;
    __device__ AccPos() {
        const int w = threadIdx.x >> 6, lane = lane_id();
        m_base = (w & 1) * (TM / 2) + (lane & 15);
        n_base = (w >> 1) * (TN / 2) + 4 * (lane >> 4);
    }
    __device__ int m(int mb) const { return m_base + mb * 16; }
    __device__ int n(int nb) const { return n_base + nb * 16; }
};

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack_bf2(a, b), pack_bf2(c, d));
}

// Item of round r of the 128 x 128 weight-gradient kernels' persistent grid:
// a round's consecutive items, the tiles of one row strip that share its
// operand, go to the blocks of one XCD (one L2).
__device__ __forceinline__ int deep_item(int r) {
    return r * (int)gridDim.x + xcd_remap(blockIdx.x, gridDim.x);
}
// Tile t of a group with nNt column tiles, in bands of 8 column tiles (row
// tiles within a band, 8 columns within a row tile), so that 64 consecutive
// items, one XCD's share of a round, are an 8 x 8 square of tiles: 8 row and
// 8 column operand strips (row-major order gave a share of 2 x 32 tiles,
// needing 34 strips in its L2, where the gate/up weight gradient has 32
// column tiles).  nNt not a multiple of 8: row-major.
__device__ __forceinline__ void band_tile(int t, int nMt, int nNt, int& mt, int& nt) {
    if (nNt % 8 != 0) {
        mt = t / nNt;
        nt = t - mt * nNt;
        return;
    }
    const int band = t / (8 * nMt), r = t - band * 8 * nMt;
    mt = r >> 3;
    nt = 8 * band + (r & 7);
}

// ================================================================ tile maps
// M-grouped: find (expert, row range, column tile) of block b.
template <int TM>
__device__ __forceinline__ bool map_mtile(const GroupRows& g, int nNt, int b, int& e, int& lo, int& hi,
                                          int& nt) {
    const int ntiles = g.tile_off ? g.tile_off[g.E] : (g.dense_rows + TM - 1) / TM;
    const int total = ntiles * nNt;
    if (b >= total) return false;
    const int L = xcd_remap(b, total);
    const int mt = L / nNt;
    nt = L - mt * nNt;
    if (!g.tile_off) {
        e = 0;
        lo = mt * TM;
        hi = min(lo + TM, g.dense_rows);
        return true;
    }
    int a = 0, z = g.E;
    while (z - a > 1) {
        const int mid = (a + z) >> 1;
        if (g.tile_off[mid] <= mt) a = mid;
        else z = mid;
    }
    e = a;
    lo = g.offsets[e] + (mt - g.tile_off[e]) * TM;
    hi = min(lo + TM, g.offsets[e + 1]);
    return true;
}

// M-grouped with 256-row tiles: the groups of at least kBigRows rows, over
// their own tile prefix (g.tile_big); a dense group takes them whole.
__device__ __forceinline__ bool map_mtile_big(const GroupRows& g, int nNt, int b, int& e, int& lo, int& hi,
                                              int& nt) {
    const int ntiles = g.tile_off ? g.tile_big[g.E] : (g.dense_rows + kBig - 1) / kBig;
    const int total = ntiles * nNt;
    if (b >= total) return false;
    const int L = xcd_remap(b, total);
    const int mt = L / nNt;
    nt = L - mt * nNt;
    if (!g.tile_off) {
        e = 0;
        lo = mt * kBig;
        hi = min(lo + kBig, g.dense_rows);
        return true;
    }
    int a = 0, z = g.E;
    while (z - a > 1) {
        const int mid = (a + z) >> 1;
        if (g.tile_big[mid] <= mt) a = mid;
        else z = mid;
    }
    e = a;
    lo = g.offsets[e] + (mt - g.tile_big[e]) * kBig;
    hi = min(lo + kBig, g.offsets[e + 1]);
    return true;
}

// K-grouped: block b -> (expert, M tile, N tile) and the expert's rows.
// The experts for which pred(e) holds, ascending, into LDS (list[0 .. count));
// a 256-thread block.  The slab weight-gradient kernels of a macrobatch walk
// build it once per block and run a persistent grid over its items: most
// experts of a skewed stream have no rows in a macrobatch, and a block per
// (expert, slab, column group) of all E experts cost ~0.5 ms per launch in
// dispatching blocks that had nothing to do.
template <class Pred>
__device__ __forceinline__ int block_list(int E, const Pred& pred, int16_t* list) {
    __shared__ int wc[4];
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    int base = 0;
    for (int j = 0; j < E; j += 256) {
        const int e = j + threadIdx.x;
        const bool f = e < E && pred(e);
        const uint64_t m = __ballot(f);
        if (lane == 0) wc[wv] = __popcll(m);
        __syncthreads();
        int pre = base;
        for (int w = 0; w < wv; ++w) pre += wc[w];
        if (f) list[pre + __popcll(m & lanemask_lt())] = (int16_t)e;
        base += wc[0] + wc[1] + wc[2] + wc[3];
        __syncthreads();
    }
    return base;
}

__device__ __forceinline__ bool map_ktile(const GroupRows& g, int nMt, int nNt, int b, int& e, int& mt,
                                          int& nt, int& lo, int& n) {
    const int per = nMt * nNt;
    const int total = (g.offsets ? g.E : 1) * per;
    if (b >= total) return false;
    const int L = xcd_remap(b, total);
    e = L / per;
    const int rem = L - e * per;
    mt = rem / nNt;
    nt = rem - mt * nNt;
    if (!g.offsets) {
        lo = 0;
        n = g.dense_rows;
        return true;
    }
    const int a = g.offsets[e], z = g.offsets[e + 1];
    if (a < 0 || z < a || z > g.rows) {
        raise_err(g.err, ERR_BAD_OFFSETS);
        lo = 0;
        n = 0;
    } else {
        lo = a;
        n = z - a;
    }
    return true;
}

// ================================================================ weight-gradient tiles
// Shared by the bf16 and MXFP8 weight gradients: a block owns one expert's
// 128-row slab of the output and walks its 64-column tiles.
constexpr int W_TM = 128, W_TN = 64;
// The column tiles of a slab are dealt to up to W_G blocks round robin
// (block g: tiles g, g + ng, ...), so that ng neighbouring 128-byte pieces of
// each row are written at about the same time (a plain store kernel of this
// tile shape measured ~5.0 TB/s walking whole rows per block, ~5.7 TB/s dealt
// over 8 blocks).  Slabs of 16 to 63 tiles are dealt over 2 blocks (the down
// projection's 16: 0.87 -> 0.83 ms with streaming stores; over 4 blocks,
// loading the A slab once per block dominates: 1.01 ms); smaller slabs stay
// whole.
constexpr int W_G = 8, W_MIN_TILES = 8;
__host__ __device__ __forceinline__ int wgrad_groups(int ntiles) {
    return ntiles >= W_G * W_MIN_TILES ? W_G : (ntiles >= 16 ? 2 : 1);
}
// tiles of group g out of ng groups over ntiles
__host__ __device__ __forceinline__ int wgrad_group_tiles(int ntiles, int ng, int g) {
    return (ntiles - g + ng - 1) / ng;
}

// LDS of a weight-gradient block: the resident A tile, then a region that
// holds the B tile during the MFMAs and the bf16 output tile afterwards.
constexpr int W_SP = W_TN + 8;                                    // staging pitch
constexpr int W_FP = W_TN + 4;        // fp32 staging pitch: 16 rows of 16 bytes hit 16 bank groups
constexpr int W_REGION = (W_TM * W_SP > Tile<W_TN, true>::SIZE) ? W_TM * W_SP : Tile<W_TN, true>::SIZE;
static_assert(64 * W_FP * 2 <= W_REGION, "half a slab of fp32 sums fits the staging region");
constexpr int W_SMEM = Tile<W_TM, true>::SIZE + W_REGION;

// mode: 0 write bf16; 1 write fp32 partial; 2 add to fp32 partial;
//       3 add to fp32 partial and write bf16 (the last macrobatch of the walk)
// (The partials were once kept as two 16-bit halves, the high half in the
// bf16 output: half the workspace, but the 8-byte accesses to two arrays
// made the 65 536-token stream's weight gradients 15-20 % slower than one
// 16-byte access to an fp32 array.)
__device__ __forceinline__ f32x4 wgrad_old(const WgradOut& o, int64_t idx) {
    return *(const f32x4*)(o.acc + idx);
}
__device__ __forceinline__ void wgrad_put(const WgradOut& o, int64_t idx, const f32x4& v, const f32x4& old) {
    float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
    if (o.mode >= 2) {
        x0 = old[0] + x0; x1 = old[1] + x1; x2 = old[2] + x2; x3 = old[3] + x3;
    }
    if (o.mode == 1 || o.mode == 2) *(float4*)(o.acc + idx) = make_float4(x0, x1, x2, x3);
    else *(uint2*)(o.out + idx) = pack4(x0, x1, x2, x3);
}
// wgrad_old then wgrad_put.  Callers that store several chunks issue the
// wgrad_old loads of all of them first: with one load before each store, each
// store waits for its load's round trip (a thread storing eight chunks paid
// eight in a row; the 65 536-token stream's accumulating weight gradients
// were bound by that latency rather than by HBM).
__device__ __forceinline__ void wgrad_store(const WgradOut& o, int64_t idx, const f32x4& v) {
    f32x4 old = f32x4{0.f, 0.f, 0.f, 0.f};
    if (o.mode >= 2) old = wgrad_old(o, idx);
    wgrad_put(o, idx, v, old);
}

// A 128 x 128 output tile of a four-wave block (AccPos<128, 128> layout)
// stored through LDS, so that every global access is a whole row piece (512
// bytes of fp32 sums, 256 of bf16) rather than each lane's 16 bytes of a
// 64-byte piece.  fst: 128 x W_TFP floats of LDS the block no longer reads
// (the caller has passed a barrier since its last reads); ends with a barrier,
// after which the LDS may be reused.
constexpr int W_TFP = 128 + 4;       // 16 rows of 16 bytes per pass hit 16 bank groups
__device__ __forceinline__ void staged_tile_store(const WgradOut& out, int64_t ebase, int64_t ld, int r0, int n0,
                                                  const f32x4 (&acc)[4][4], float* fst) {
    AccPos<128, 128> pos;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) *(f32x4*)(fst + pos.m(mb) * W_TFP + pos.n(nb)) = acc[mb][nb];
    constexpr int N = 128 * 32 / 256;
    const int r = threadIdx.x >> 5, cc = threadIdx.x & 31;      // chunk q: row r + 8 q, column chunk cc
    const int64_t base = ebase + (int64_t)(r0 + r) * ld + n0 + 4 * cc;
    f32x4 old[N];
    if (out.mode >= 2) {                   // the old sums of all the thread's chunks in one batch
#pragma unroll
        for (int q = 0; q < N; ++q) old[q] = wgrad_old(out, base + 8 * q * ld);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < N; ++q)
        wgrad_put(out, base + 8 * q * ld, *(const f32x4*)(fst + (r + 8 * q) * W_TFP + 4 * cc), old[q]);
    __syncthreads();
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct WgradEpi {
    WgradOut out;
    int64_t ebase;   // first element of the expert's matrix
    int64_t ld;      // row length of the output matrix
    int m0;          // first output row of the slab
    // bf16 output (mode 0) goes through LDS so that every global store writes
    // whole 128-byte row segments; the fp32 accumulation modes store directly.
    // BF16_ONLY: the caller has checked mode == 0, so the stores are
    // unconditional and the compiler can count them in its memory waits.
    // STREAM: streaming (non-temporal) bf16 stores, for slabs whose column
    // tiles are dealt over several blocks: measured faster there (the gradient
    // is not read again by this layer), slower for a slab one block writes
    // alone.
    template <bool BF16_ONLY, bool STREAM = false>
    __device__ __forceinline__ void store(int nt, const f32x4 (&acc)[W_TM / 32][W_TN / 32],
                                          uint16_t* stage) const {
        AccPos<W_TM, W_TN> pos;
        const int n0 = nt * W_TN;
        if (!BF16_ONLY && out.mode != 0) {
            // fp32 running sums: staged in LDS half a slab (64 rows) at a time so
            // that every global access is a whole 256-byte row piece (each
            // lane's own four sums are 16 bytes of a 64-byte piece: the
            // 65 536-token stream's cold experts ran at ~1 TB/s that way); a
            // half's old sums are loaded in one batch (wgrad_store)
            float* fst = (float*)stage;
            const int w = threadIdx.x >> 6;
            constexpr int CPR = W_TN / 4, N = 64 * CPR / 256;
            const int r = threadIdx.x / CPR, cc = threadIdx.x % CPR;    // chunk q: row r + 16 q
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if (half) __syncthreads();                 // the first half is written out
                if ((w & 1) == half) {
#pragma unroll
                    for (int mb = 0; mb < W_TM / 32; ++mb)
#pragma unroll
                        for (int nb = 0; nb < W_TN / 32; ++nb)
                            *(f32x4*)(fst + (pos.m(mb) - 64 * half) * W_FP + pos.n(nb)) = acc[mb][nb];
                }
                const int64_t base = ebase + (int64_t)(m0 + 64 * half + r) * ld + n0 + 4 * cc;
                f32x4 old[N];
                if (out.mode >= 2) {
#pragma unroll
                    for (int q = 0; q < N; ++q) old[q] = wgrad_old(out, base + 256 / CPR * q * ld);
                }
                __syncthreads();
#pragma unroll
                for (int q = 0; q < N; ++q)
                    wgrad_put(out, base + 256 / CPR * q * ld,
                              *(const f32x4*)(fst + (r + 256 / CPR * q) * W_FP + 4 * cc), old[q]);
            }
            return;
        }
#pragma unroll
        for (int mb = 0; mb < W_TM / 32; ++mb)
#pragma unroll
            for (int nb = 0; nb < W_TN / 32; ++nb) {
                const f32x4 v = acc[mb][nb];
                *(uint2*)(stage + pos.m(mb) * W_SP + pos.n(nb)) = pack4(v[0], v[1], v[2], v[3]);
            }
        __syncthreads();
        constexpr int CPR = W_TN / 8;                  // 16-byte chunks per row
        if constexpr (STREAM) {
#pragma unroll
            for (int q = 0; q < W_TM * CPR / 256; ++q) {
                const int c = threadIdx.x + 256 * q;
                const int r = c / CPR, cc = c % CPR;
                __builtin_nontemporal_store(*(const u32x4*)(stage + r * W_SP + cc * 8),
                                            (u32x4*)(out.out + ebase + (int64_t)(m0 + r) * ld + n0 + cc * 8));
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < W_TM * CPR / 256; ++q) {
            const int c = threadIdx.x + 256 * q;
            const int r = c / CPR, cc = c % CPR;
            *(uint4*)(out.out + ebase + (int64_t)(m0 + r) * ld + n0 + cc * 8) =
                *(const uint4*)(stage + r * W_SP + cc * 8);
        }
    }
    __device__ __forceinline__ void operator()(int nt, const f32x4 (&acc)[W_TM / 32][W_TN / 32],
                                               uint16_t* stage) const {
        store<false>(nt, acc, stage);
    }
};

}  // namespace moe
