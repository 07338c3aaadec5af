// The router projection upstream of the layer, and its backward, on MFMA.
//
// alphalab.site "Mixture-of-Kittens", section 二: the router projection that
// produces the expert logits sits outside the MoE layer (the layer starts
// from the logits); these kernels provide it so that the logit gradient the
// layer's backward returns reaches the router weights and the tokens:
//   logits    = x W_r^T                      [T, E] fp32
//   dx       += d_logits W_r                 [T, H] (added to the layer's dx)
//   dW_r      = d_logits^T x                 [E, H]
// d_logits is rounded to bf16 once (the MFMA operand precision) into a
// zero-padded [T, Ep] copy, Ep = E rounded up to 64; every product
// accumulates in fp32 in a fixed K order (no split K), so results are
// identical run to run.  Tiles: 64 x 128, four waves, the double-buffered K
// loop of the expert GEMMs.
#include "gemm_common.h"
#include "profile.h"

namespace moe {

constexpr int R_TM = 64, R_TN = 128;

__global__ __launch_bounds__(256, 2) void k_router_logits(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          float* __restrict__ logits, int T, int H, int E) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<R_TM, R_TN, false, false>::STAGE];
    const int nN = (E + R_TN - 1) / R_TN;
    const int mt = blockIdx.x / nN, nt = blockIdx.x % nN;
    const int m0 = mt * R_TM, n0 = nt * R_TN;
    f32x4 acc[R_TM / 32][R_TN / 32];
    RowsDirect sa{x, H, m0, T - m0};
    LoadKC<R_TM, RowsDirect> la(sa);
    RowsDirect sb{wr, H, n0, E - n0};
    LoadKC<R_TN, RowsDirect> lb(sb);
    mainloop<R_TM, R_TN, false, false>(la, lb, H / kTK, smem, acc);
    AccPos<R_TM, R_TN> pos;
#pragma unroll
    for (int mb = 0; mb < R_TM / 32; ++mb) {
        const int row = m0 + pos.m(mb);
        if (row >= T) continue;
#pragma unroll
        for (int nb = 0; nb < R_TN / 32; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = n0 + pos.n(nb) + r;
                if (col < E) logits[(int64_t)row * E + col] = acc[mb][nb][r];
            }
    }
}

// d_logits fp32 [T, E] -> bf16 [T, Ep], columns E..Ep-1 zero
__global__ __launch_bounds__(256) void k_router_dl16(const float* __restrict__ dl, int64_t n, int E, int Ep,
                                                     uint16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t t = i / Ep;
    const int e = (int)(i - t * Ep);
    out[i] = e < E ? (uint16_t)f2bf(dl[t * E + e]) : (uint16_t)0;
}

// dx[T, H] += dl16 [T, Ep] W_r [E, H]: W_r read with k (the expert) as the
// memory row; the sum with the stored dx is taken in fp32, rounded once
__global__ __launch_bounds__(256, 2) void k_router_dx(const uint16_t* __restrict__ dl16,
                                                      const uint16_t* __restrict__ wr,
                                                      uint16_t* __restrict__ dx, int T, int H, int E, int Ep) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<R_TM, R_TN, false, true>::STAGE];
    const int nN = H / R_TN;
    const int mt = blockIdx.x / nN, nt = blockIdx.x % nN;
    const int m0 = mt * R_TM, n0 = nt * R_TN;
    f32x4 acc[R_TM / 32][R_TN / 32];
    RowsDirect sa{dl16, Ep, m0, T - m0};
    LoadKC<R_TM, RowsDirect> la(sa);
    KRowsDirect sb{wr, H, n0, E};
    LoadKS<R_TN, KRowsDirect> lb(sb);
    mainloop<R_TM, R_TN, false, true>(la, lb, Ep / kTK, smem, acc);
    AccPos<R_TM, R_TN> pos;
#pragma unroll
    for (int mb = 0; mb < R_TM / 32; ++mb) {
        const int row = m0 + pos.m(mb);
        if (row >= T) continue;
#pragma unroll
        for (int nb = 0; nb < R_TN / 32; ++nb) {
            uint2* p = (uint2*)(dx + (int64_t)row * H + n0 + pos.n(nb));
            const uint2 old = *p;
            const f32x4 v = acc[mb][nb];
            *p = pack4(lo_bf(old.x) + v[0], hi_bf(old.x) + v[1], lo_bf(old.y) + v[2], hi_bf(old.y) + v[3]);
        }
    }
}

// dW_r [E, H] = dl16^T x: both operands read with k (the token) as the memory
// row; the K loop runs over all T tokens in ascending order
__global__ __launch_bounds__(256, 2) void k_router_dw(const uint16_t* __restrict__ dl16,
                                                      const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ dwr, int T, int H, int E, int Ep) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<R_TM, R_TN, true, true>::STAGE];
    const int nN = H / R_TN;
    const int mt = blockIdx.x / nN, nt = blockIdx.x % nN;
    const int m0 = mt * R_TM, n0 = nt * R_TN;
    f32x4 acc[R_TM / 32][R_TN / 32];
    KRowsDirect sa{dl16, Ep, m0, T};
    LoadKS<R_TM, KRowsDirect> la(sa);
    KRowsDirect sb{x, H, n0, T};
    LoadKS<R_TN, KRowsDirect> lb(sb);
    mainloop<R_TM, R_TN, true, true>(la, lb, (T + kTK - 1) / kTK, smem, acc);
    AccPos<R_TM, R_TN> pos;
#pragma unroll
    for (int mb = 0; mb < R_TM / 32; ++mb) {
        const int row = m0 + pos.m(mb);
        if (row >= E) continue;
#pragma unroll
        for (int nb = 0; nb < R_TN / 32; ++nb) {
            const f32x4 v = acc[mb][nb];
            *(uint2*)(dwr + (int64_t)row * H + n0 + pos.n(nb)) = pack4(v[0], v[1], v[2], v[3]);
        }
    }
}

int router_padded_experts(int E) { return (E + kTK - 1) / kTK * kTK; }

int launch_router_logits(const void* x, const void* wr, float* logits, int T, int H, int E, hipStream_t st) {
    ProfScope prof_(st, "router_logits");
    const int grid = ((T + R_TM - 1) / R_TM) * ((E + R_TN - 1) / R_TN);
    k_router_logits<<<grid, 256, 0, st>>>((const uint16_t*)x, (const uint16_t*)wr, logits, T, H, E);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_router_backward(const void* x, const void* wr, const float* d_logits, void* dx, void* dwr,
                           void* dl16, int T, int H, int E, hipStream_t st) {
    const int Ep = router_padded_experts(E);
    {
        ProfScope prof_(st, "router_dl16");
        const int64_t n = (int64_t)T * Ep;
        k_router_dl16<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(d_logits, n, E, Ep, (uint16_t*)dl16);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    {
        ProfScope prof_(st, "router_dx");
        const int grid = ((T + R_TM - 1) / R_TM) * (H / R_TN);
        k_router_dx<<<grid, 256, 0, st>>>((const uint16_t*)dl16, (const uint16_t*)wr, (uint16_t*)dx, T, H, E, Ep);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    {
        ProfScope prof_(st, "router_dw");
        const int grid = (Ep / R_TM) * (H / R_TN);
        k_router_dw<<<grid, 256, 0, st>>>((const uint16_t*)dl16, (const uint16_t*)x, (uint16_t*)dwr, T, H, E, Ep);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

}  // namespace moe
