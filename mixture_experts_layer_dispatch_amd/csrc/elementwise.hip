// Bandwidth-bound steps of the layer: the combine (the final sum of a token's
// weighted expert rows), the reverse-dispatch reduction, the softmax backward,
// and the per-expert tile prefix the grouped GEMMs are launched over.  The
// dispatch itself is fused into the gate/up GEMM's operand loads.
//
// Combine / reverse-dispatch: alphalab.site "Mixture-of-Kittens"
// section 一 (tokens go to their experts and come back) and section 二 (the
// router-weighted reduction; a fixed floating-point accumulation order makes
// the layer bitwise reproducible); arex-research.com "Cursor 放出 MoK", design
// section, first decision (forward dispatch/combine and backward
// reverse-combine/reverse-dispatch all read one schedule table).
//
// Every kernel moves 16-byte chunks (8 bf16) per lane so that a wave reads or
// writes 1 KiB contiguous per instruction; rows are H bf16 long.
#include "common.h"
#include "launch.h"
#include "profile.h"

namespace moe {

// ============================================================== combine
// Lane j < k of the wave holds slot j's ring row and weight; the loops below
// read them with uniform-lane shuffles, so the j order is fixed.
__device__ __forceinline__ void load_slot_rows(const int32_t* __restrict__ row_of_slot,
                                               const float* __restrict__ w, int t, int k,
                                               int ring_row0, int ring_rows, int lane, int& row,
                                               float& wt, int32_t* err) {
    row = -1;
    wt = 0.f;
    if (lane < k) {
        int r = row_of_slot[(size_t)t * k + lane] - ring_row0;
        if ((unsigned)r < (unsigned)ring_rows) row = r;
        else raise_err(err, ERR_BAD_ROW);
        if (w) wt = w[(size_t)t * k + lane];
    }
}

__device__ __forceinline__ void unpack8(const uint4& v, float* a) {
    a[0] = lo_bf(v.x); a[1] = hi_bf(v.x); a[2] = lo_bf(v.y); a[3] = hi_bf(v.y);
    a[4] = lo_bf(v.z); a[5] = hi_bf(v.z); a[6] = lo_bf(v.w); a[7] = hi_bf(v.w);
}

__device__ __forceinline__ uint4 pack8(const float* a) {
    uint4 out;
    out.x = pack_bf2(a[0], a[1]);
    out.y = pack_bf2(a[2], a[3]);
    out.z = pack_bf2(a[4], a[5]);
    out.w = pack_bf2(a[6], a[7]);
    return out;
}

// y_t = [shared_t] + sum_{j=0..k-1} w[t,j] * o[row(t,j)] in fp32, in this
// order, one rounding to bf16 (w == nullptr: unit weights, the
// reverse-dispatch sum of the backward).  With k >= COMBINE_SEG_K slots
// (SEG) a wave takes one 512-column segment of a token and loads up to 8 slot
// rows at once (a wave per token walking its segments one slot row at a time
// left k = 10 latency-bound: 0.064 -> 0.037 ms at T = 2048, H = 4096); with
// fewer slots a wave walks a whole token that way (measured faster for k = 1
// than either batched form).
constexpr int COMBINE_SEG_K = 4;

template <bool SEG>
__global__ __launch_bounds__(256) void k_combine(const uint4* __restrict__ o, int H8,
                                                 const int32_t* __restrict__ row_of_slot,
                                                 const float* __restrict__ w, int t0, int t1,
                                                 int k, int ring_row0, int ring_rows,
                                                 const uint4* __restrict__ shared, int shared_t0,
                                                 uint4* __restrict__ y, int32_t* __restrict__ err) {
    constexpr int NS = 1;                                // segments a wave holds at once
    const int nseg = (H8 + 63) / 64;
    const int64_t L = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = t0 + (int)(SEG ? L / nseg : L);
    if (t >= t1) return;
    const int lane = lane_id();
    int myrow;
    float myw;
    load_slot_rows(row_of_slot, w, t, k, ring_row0, ring_rows, lane, myrow, myw, err);
    for (int sg0 = SEG ? (int)(L % nseg) : 0; sg0 < nseg; sg0 += SEG ? nseg : 1) {
        float acc[NS][8];
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int c = (sg0 + u) * 64 + lane;
            if (shared && c < H8) {
                unpack8(shared[(size_t)(t - shared_t0) * H8 + c], acc[u]);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
            }
        }
        constexpr int JB = SEG ? 8 : 1;                  // slot rows loaded at once
        for (int j0 = 0; j0 < k; j0 += JB) {
            uint4 v[JB][NS];
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
                const int j = j0 + jj;
                const int r = __shfl(myrow, j & 63);
#pragma unroll
                for (int u = 0; u < NS; ++u) {
                    const int c = (sg0 + u) * 64 + lane;
                    v[jj][u] = (j < k && r >= 0 && c < H8) ? o[(size_t)r * H8 + c] : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
                const int j = j0 + jj;
                const int r = __shfl(myrow, j & 63);
                const float wj = w ? __shfl(myw, j & 63) : 1.0f;
                if (j >= k || r < 0) continue;
#pragma unroll
                for (int u = 0; u < NS; ++u) {
                    float x[8];
                    unpack8(v[jj][u], x);
                    if (w) {
#pragma unroll
                        for (int q = 0; q < 8; ++q) acc[u][q] += wj * x[q];
                    } else {
#pragma unroll
                        for (int q = 0; q < 8; ++q) acc[u][q] += x[q];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int c = (sg0 + u) * 64 + lane;
            if (c < H8) y[(size_t)t * H8 + c] = pack8(acc[u]);
        }
    }
}

static int launch_combine_(const void* src, int H, const int32_t* row_of_slot, const float* w, int t0,
                           int t1, int k, int ring_row0, int ring_rows, const void* shared,
                           int shared_t0, void* out, int32_t* err, hipStream_t st) {
    if (t1 <= t0) return 0;
    const int H8 = H / 8, nseg = (H8 + 63) / 64;
    if (k >= COMBINE_SEG_K) {
        const int64_t waves = (int64_t)(t1 - t0) * nseg;
        k_combine<true><<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(
            (const uint4*)src, H8, row_of_slot, w, t0, t1, k, ring_row0, ring_rows,
            (const uint4*)shared, shared_t0, (uint4*)out, err);
    } else {
        k_combine<false><<<(t1 - t0 + 3) / 4, 256, 0, st>>>(
            (const uint4*)src, H8, row_of_slot, w, t0, t1, k, ring_row0, ring_rows,
            (const uint4*)shared, shared_t0, (uint4*)out, err);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ============================================================== softmax backward
// dw[t,j] = sum_p part[row(t,j)][p] (p ascending), then
// d_logit[t, idx[t,j]] = w_j (dw_j - sum_i w_i dw_i), zero for other experts.
// One wave per token.
__global__ __launch_bounds__(256) void k_softmax_bwd(const float* __restrict__ part, int P,
                                                     const int32_t* __restrict__ row_of_slot,
                                                     const int32_t* __restrict__ idx,
                                                     const float* __restrict__ w, int t0, int t1,
                                                     int k, int E, int ring_row0, int ring_rows,
                                                     float* __restrict__ dw,
                                                     float* __restrict__ d_logits,
                                                     int32_t* __restrict__ err) {
    const int t = t0 + blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= t1) return;
    const int lane = lane_id();
    int myrow;
    float wj;
    load_slot_rows(row_of_slot, w, t, k, ring_row0, ring_rows, lane, myrow, wj, err);
    float dwj = 0.f;
    int ej = -1;
    if (lane < k) {
        if (myrow >= 0) {
            const float* pr = part + (size_t)myrow * P;
            for (int p = 0; p < P; ++p) dwj += pr[p];
        }
        ej = idx[(size_t)t * k + lane];
        dw[(size_t)t * k + lane] = dwj;
    }
    float c = 0.f;
    for (int j = 0; j < k; ++j) c += __shfl(wj, j) * __shfl(dwj, j);
    const float dl = wj * (dwj - c);
    if (d_logits) {
        float* out = d_logits + (size_t)t * E;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            float v = 0.f;
            for (int j = 0; j < k; ++j) {
                const int ejj = __shfl(ej, j);
                const float dlj = __shfl(dl, j);
                if (ejj == e) v = dlj;
            }
            if (e < E) out[e] = v;
        }
    }
}

// ============================================================== tile prefix
// tile_off[e] = sum_{e' < e} ceil(count(e') / TM) from one macrobatch's
// offsets; tile_off[E] is the number of row tiles.  With split outputs, also
// the same prefix over the groups below big_rows rows only (small, TM-row
// tiles) and over the others only (big, big_tm-row tiles), for GEMMs that
// take the large groups in a tile form of their own.  One block, E <= 1024.
__device__ __forceinline__ int block_excl_scan(int n, int32_t* wsum, int& total) {
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int wpre = 0;
    for (int q = 0; q < wv; ++q) wpre += wsum[q];
    total = 0;
    for (int q = 0; q < (int)(blockDim.x >> 6); ++q) total += wsum[q];
    __syncthreads();                       // wsum is reused by the next scan
    return wpre + incl - n;
}

__global__ __launch_bounds__(1024) void k_tile_prefix(const int32_t* __restrict__ offsets, int E,
                                                      int rows, int TM, int32_t* __restrict__ tile_off,
                                                      int big_rows, int big_tm, int32_t* __restrict__ small,
                                                      int32_t* __restrict__ big, int32_t* __restrict__ err) {
    __shared__ int32_t wsum[16];
    const int e = threadIdx.x;
    int cnt = 0;
    if (e < E) {
        const int a = offsets[e], b = offsets[e + 1];
        if (a < 0 || b < a || b > rows) raise_err(err, ERR_BAD_OFFSETS);
        else cnt = b - a;
    }
    int total;
    const int n = (cnt + TM - 1) / TM;
    const int pre = block_excl_scan(n, wsum, total);
    if (e < E) tile_off[e] = pre;
    if (e == 0) tile_off[E] = total;
    if (!big) return;
    const bool is_big = cnt >= big_rows;
    const int ns = is_big ? 0 : n;
    const int ps = block_excl_scan(ns, wsum, total);
    if (e < E) small[e] = ps;
    if (e == 0) small[E] = total;
    const int nb = is_big ? (cnt + big_tm - 1) / big_tm : 0;
    const int pb = block_excl_scan(nb, wsum, total);
    if (e < E) big[e] = pb;
    if (e == 0) big[E] = total;
}

// Experts whose group has more than thr rows, in ascending order:
// list[0] = their count, list[1..] = their ids.  Bad offsets count as empty
// (the tile prefix reports them).
__device__ __forceinline__ void flag_list(int f, int e, int32_t* wsum, int32_t* list) {
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const unsigned long long m = __ballot(f);
    const int incl = __popcll(m & ((2ull << lane) - 1ull));
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int wpre = 0;
    for (int q = 0; q < wv; ++q) wpre += wsum[q];
    if (f) list[1 + wpre + incl - 1] = e;
    if (threadIdx.x == 1023) {
        int tot = 0;
        for (int q = 0; q < 16; ++q) tot += wsum[q];
        list[0] = tot;
    }
    __syncthreads();                       // wsum is reused by the next list
}

// With a second list (big), the groups of at least big_thr rows go there
// instead of to list.
__global__ __launch_bounds__(1024) void k_deep_list(const int32_t* __restrict__ offsets, int E,
                                                    int rows, int thr, int32_t* __restrict__ list,
                                                    int big_thr, int32_t* __restrict__ big) {
    __shared__ int32_t wsum[16];
    const int e = threadIdx.x;
    int n = -1;
    if (e < E) {
        const int a = offsets[e], b = offsets[e + 1];
        if (a >= 0 && b >= a && b <= rows) n = b - a;
    }
    const bool is_big = big && n >= big_thr;
    flag_list(n > thr && !is_big ? 1 : 0, e, wsum, list);
    if (big) flag_list(is_big ? 1 : 0, e, wsum, big);
}

// ============================================================== launchers
int launch_combine(const void* o, int H, const int32_t* row_of_slot, const float* w, int t0, int t1,
                   int k, int ring_row0, int ring_rows, const void* shared, int shared_t0, void* y,
                   int32_t* err, hipStream_t st) {
    ProfScope prof_(st, "combine");
    return launch_combine_(o, H, row_of_slot, w, t0, t1, k, ring_row0, ring_rows, shared, shared_t0, y,
                           err, st);
}

int launch_rd_reduce(const void* dxd, int H, const int32_t* row_of_slot, int t0, int t1, int k,
                     int ring_row0, int ring_rows, const void* shared, int shared_t0, void* dx,
                     int32_t* err, hipStream_t st) {
    ProfScope prof_(st, "rd_reduce");
    return launch_combine_(dxd, H, row_of_slot, nullptr, t0, t1, k, ring_row0, ring_rows, shared,
                           shared_t0, dx, err, st);
}

int launch_softmax_bwd(const float* part, int P, const int32_t* row_of_slot, const int32_t* idx,
                       const float* w, int t0, int t1, int k, int E, int ring_row0, int ring_rows,
                       float* dw, float* d_logits, int32_t* err, hipStream_t st) {
    ProfScope prof_(st, "softmax_bwd");
    if (t1 <= t0) return 0;
    k_softmax_bwd<<<(t1 - t0 + 3) / 4, 256, 0, st>>>(part, P, row_of_slot, idx, w, t0, t1, k, E,
                                                     ring_row0, ring_rows, dw, d_logits, err);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_tile_prefix(const int32_t* offsets, int E, int rows, int TM, int32_t* tile_off,
                       int32_t* err, hipStream_t st) {
    return launch_tile_prefix_split(offsets, E, rows, TM, tile_off, 0, 0, nullptr, nullptr, err, st);
}

int launch_tile_prefix_split(const int32_t* offsets, int E, int rows, int TM, int32_t* tile_off,
                             int big_rows, int big_tm, int32_t* small, int32_t* big, int32_t* err,
                             hipStream_t st) {
    ProfScope prof_(st, "tile_prefix");
    if (E > 1024 || (big && (!small || big_rows <= 0 || big_tm <= 0))) return -1;
    k_tile_prefix<<<1, 1024, 0, st>>>(offsets, E, rows, TM, tile_off, big_rows, big_tm, small, big, err);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_deep_list_split(const int32_t* offsets, int E, int rows, int thr, int32_t* list, int big_thr,
                           int32_t* big, hipStream_t st) {
    ProfScope prof_(st, "deep_list");
    if (E > 1024 || !big || big_thr <= thr) return -1;
    k_deep_list<<<1, 1024, 0, st>>>(offsets, E, rows, thr, list, big_thr, big);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_deep_list(const int32_t* offsets, int E, int rows, int thr, int32_t* list, hipStream_t st) {
    ProfScope prof_(st, "deep_list");
    if (E > 1024) return -1;
    k_deep_list<<<1, 1024, 0, st>>>(offsets, E, rows, thr, list, 0, nullptr);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
