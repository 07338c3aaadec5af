// Top-k routing and the schedule (counts, exclusive scan, stable permutation).
//
// Routing: alphalab.site "Mixture-of-Kittens" sections 一 and 四 (a router
// keeps the top-k experts of each token; the benchmark feeds Gaussian logits).
// Schedule: arex-research.com "Cursor 放出 MoK", design section, first and
// second decisions (one schedule table drives all four data movements; tokens
// stream through a ring buffer per macrobatch, filled per minibatch).
//
// Layout of a macrobatch: slots [m*Sm, (m+1)*Sm), Sm = M*k; each minibatch i
// covers Smb = mb*k consecutive slots, cut into blocks of kBlockSlots slots.
// The per-block expert histograms turn into per-block row bases (expert-major
// exclusive scan), and a single-wave pass per block assigns stable in-block
// ranks with bit-serial ballot matching.  All of it is integer work, so the
// result is exact and identical run to run.
#include "common.h"
#include "launch.h"
#include "profile.h"

namespace moe {

// ============================================================== routing
// One wave per token; lane l holds logits e = l + 64*j.  k rounds of a wave
// argmax with (value desc, index asc) order, then the softmax of the k kept
// logits in fp32, largest first.
template <int EPL>
__global__ __launch_bounds__(256) void k_topk_route(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out) {
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + (size_t)t * E;
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        int e = lane + 64 * j;
        v[j] = e < E ? row[e] : -INFINITY;
    }
    uint32_t taken = 0;
    float sel_v = 0.f;   // lane r keeps the r-th kept logit (r < k <= 64)
    int sel_e = 0;
    float first = 0.f;
    for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            int e = lane + 64 * j;
            bool ok = e < E && !((taken >> j) & 1u);
            if (ok && (v[j] > bv || (v[j] == bv && e < be))) { bv = v[j]; be = e; }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float ov = __shfl_xor(bv, off);
            int oe = __shfl_xor(be, off);
            if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        // every lane now holds the winner
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == r) { sel_v = bv; sel_e = be; }
        if (r == 0) first = bv;
    }
    // softmax over the kept logits, summed in the fixed order r = 0..k-1
    float ez = lane < k ? expf(sel_v - first) : 0.f;
    float s = 0.f;
    for (int r = 0; r < k; ++r) s += __shfl(ez, r);
    if (lane < k) {
        idx_out[(size_t)t * k + lane] = sel_e;
        w_out[(size_t)t * k + lane] = ez / s;
    }
}

// ============================================================== histogram
struct SchedGeom {
    int k, E;
    int Sm;       // slots per macrobatch
    int Smb;      // slots per minibatch
    int nbpm;     // blocks per minibatch
    int nb;       // blocks per macrobatch
};

__device__ __forceinline__ void block_range(const SchedGeom& g, int blk, int& m, int& lo, int& hi) {
    m = blk / g.nb;
    int b = blk % g.nb;
    int mi = b / g.nbpm, bb = b % g.nbpm;
    lo = m * g.Sm + mi * g.Smb + bb * kBlockSlots;
    hi = min(lo + kBlockSlots, m * g.Sm + (mi + 1) * g.Smb);
}

__global__ __launch_bounds__(256) void k_sched_hist(const int32_t* __restrict__ idx, SchedGeom g,
                                                    int32_t* __restrict__ hist,
                                                    int32_t* __restrict__ err) {
    __shared__ int32_t h[kMaxExperts];
    for (int e = threadIdx.x; e < g.E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    int m, lo, hi;
    block_range(g, blockIdx.x, m, lo, hi);
    for (int s = lo + threadIdx.x; s < hi; s += blockDim.x) {
        int e = idx[s];
        if ((unsigned)e < (unsigned)g.E) atomicAdd(&h[e], 1);   // integer: order-free
        else raise_err(err, ERR_BAD_EXPERT);
    }
    __syncthreads();
    int32_t* out = hist + (size_t)blockIdx.x * g.E;
    for (int e = threadIdx.x; e < g.E; e += blockDim.x) out[e] = h[e];
}

// ============================================================== scan
// One block per macrobatch.  For each expert, a running count over blocks
// (block order = slot order) gives each block's offset inside the expert's
// group (written to `base`); the expert totals are scanned into offsets.  The
// scatter adds the expert's offset to its block base.
__global__ __launch_bounds__(1024) void k_sched_scan(SchedGeom g, int n_mini,
                                                     const int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ base,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ mini_counts) {
    __shared__ int32_t wsum[16];
    const int m = blockIdx.x;
    const int32_t* hm = hist + (size_t)m * g.nb * g.E;
    int32_t* bm = base + (size_t)m * g.nb * g.E;
    const int e = threadIdx.x;
    int run = 0;
    if (e < g.E) {
        for (int mi = 0; mi < n_mini; ++mi) {
            int mrun = 0;
            for (int b0 = 0; b0 < g.nbpm; b0 += 8) {
                int c[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int b = mi * g.nbpm + b0 + q;
                    c[q] = (b0 + q < g.nbpm) ? hm[(size_t)b * g.E + e] : 0;
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int b = mi * g.nbpm + b0 + q;
                    if (b0 + q < g.nbpm) bm[(size_t)b * g.E + e] = run;
                    run += c[q];
                    mrun += c[q];
                }
            }
            mini_counts[((size_t)m * g.E + e) * n_mini + mi] = mrun;
        }
        counts[(size_t)m * g.E + e] = run;
    }
    // exclusive scan of the expert totals, one expert per thread (E <= 1024)
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int wpre = 0;
    for (int q = 0; q < wv; ++q) wpre += wsum[q];
    const int excl = wpre + incl - run;
    if (e < g.E) offsets[(size_t)m * (g.E + 1) + e] = excl;
    if (e == g.E - 1) offsets[(size_t)m * (g.E + 1) + g.E] = excl + run;
}

// ============================================================== scatter
// One wave per block.  cnt[e] starts at the block's first row for expert e and
// walks the block's slots 64 at a time; lanes holding the same expert are
// matched by ballots over the bits of the expert id, ranked by lane order
// (= slot order), and the highest lane of each group advances cnt[e].
__global__ __launch_bounds__(64) void k_sched_scatter(const int32_t* __restrict__ idx, SchedGeom g,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ row_of_slot,
                                                      int32_t* __restrict__ slot_of_row) {
    __shared__ int32_t cnt[kMaxExperts];
    const int lane = lane_id();
    int m, lo, hi;
    block_range(g, blockIdx.x, m, lo, hi);
    const int32_t* bb = base + (size_t)blockIdx.x * g.E;
    const int32_t* off = offsets + (size_t)m * (g.E + 1);
    for (int e = lane; e < g.E; e += 64) cnt[e] = off[e] + bb[e];
    __syncthreads();
    const int nbits = 32 - __clz(max(g.E - 1, 1));
    const uint64_t lt = lanemask_lt();
    for (int s0 = lo; s0 < hi; s0 += 64) {
        const int s = s0 + lane;
        const int e = s < hi ? idx[s] : -1;
        const bool valid = (unsigned)e < (unsigned)g.E;
        uint64_t match = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t ones = __ballot(bit);
            match &= bit ? ones : ~ones;
        }
        if (!valid) match = 0;
        const int rank = __popcll(match & lt);
        int row = 0;
        if (valid) row = cnt[e] + rank;
        __syncthreads();
        const bool leader = valid && (match >> lane) == 1ull;   // highest lane of its group
        if (leader) cnt[e] = row + 1;
        __syncthreads();
        if (valid) {
            const int grow = m * g.Sm + row;
            row_of_slot[s] = grow;
            slot_of_row[grow] = s;
        }
    }
}

// Accumulator slots for a stream of several macrobatches: the routed experts
// with rows in at least two macrobatches (the only ones whose weight
// gradients keep a running sum across the reverse walk) get slots 0, 1, ...
// in expert order, the others -1; past `cap` slots the expert gets -1 and
// ERR_ACC_CAPACITY is raised.  One block of kMaxExperts threads, one expert
// each, and a block-wide scan.
__global__ __launch_bounds__(kMaxExperts) void k_acc_slots(const int32_t* __restrict__ counts, int n_macro,
                                                         int E, int cap, int32_t* __restrict__ slot,
                                                         int32_t* err) {
    __shared__ int32_t sc[kMaxExperts];
    const int e = threadIdx.x;
    int spans = 0;
    if (e < E)
        for (int m = 0; m < n_macro; ++m) spans += counts[(int64_t)m * E + e] > 0;
    const int need = spans >= 2 ? 1 : 0;
    sc[e] = need;
    __syncthreads();
    for (int d = 1; d < kMaxExperts; d <<= 1) {          // inclusive scan
        const int v = e >= d ? sc[e - d] : 0;
        __syncthreads();
        sc[e] += v;
        __syncthreads();
    }
    if (e < E) {
        int sl = need ? sc[e] - 1 : -1;
        if (sl >= cap) {
            raise_err(err, ERR_ACC_CAPACITY);
            sl = -1;
        }
        slot[e] = sl;
    }
}

// ============================================================== host launchers
int launch_acc_slots(const int32_t* counts, int n_macro, int E, int cap, int32_t* slot, int32_t* err,
                     hipStream_t st) {
    ProfScope prof_(st, "acc_slots");
    k_acc_slots<<<1, kMaxExperts, 0, st>>>(counts, n_macro, E, cap, slot, err);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_topk_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                      hipStream_t st) {
    ProfScope prof_(st, "topk_route");
    dim3 grid((T + 3) / 4), block(256);
    const int epl = (E + 63) / 64;
    if (epl <= 1) k_topk_route<1><<<grid, block, 0, st>>>(logits, T, E, k, idx, w);
    else if (epl <= 2) k_topk_route<2><<<grid, block, 0, st>>>(logits, T, E, k, idx, w);
    else if (epl <= 4) k_topk_route<4><<<grid, block, 0, st>>>(logits, T, E, k, idx, w);
    else if (epl <= 8) k_topk_route<8><<<grid, block, 0, st>>>(logits, T, E, k, idx, w);
    else k_topk_route<16><<<grid, block, 0, st>>>(logits, T, E, k, idx, w);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_schedule(const int32_t* idx, int T, int E, int k, int M, int mb, int32_t* hist,
                    int32_t* base, int32_t* counts, int32_t* offsets, int32_t* mini_counts, int32_t* row_of_slot,
                    int32_t* slot_of_row, int32_t* err, hipStream_t st) {
    SchedGeom g;
    g.k = k;
    g.E = E;
    g.Sm = M * k;
    g.Smb = mb * k;
    g.nbpm = (g.Smb + kBlockSlots - 1) / kBlockSlots;
    const int n_mini = M / mb, n_macro = T / M;
    g.nb = g.nbpm * n_mini;
    const int nblk = g.nb * n_macro;
    {
        ProfScope prof_(st, "sched_hist");
        k_sched_hist<<<nblk, 256, 0, st>>>(idx, g, hist, err);
    }
    {
        ProfScope prof_(st, "sched_scan");
        k_sched_scan<<<n_macro, 1024, 0, st>>>(g, n_mini, hist, base, counts, offsets, mini_counts);
    }
    {
        ProfScope prof_(st, "sched_scatter");
        k_sched_scatter<<<nblk, 64, 0, st>>>(idx, g, base, offsets, row_of_slot, slot_of_row);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

size_t schedule_hist_ints(int T, int E, int k, int M, int mb) {
    const int Smb = mb * k;
    const int nbpm = (Smb + kBlockSlots - 1) / kBlockSlots;
    return (size_t)nbpm * (M / mb) * (T / M) * E;
}

}  // namespace moe
