// Internal interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kBlockSlots = 512;   // slots per schedule block

// Row groups of one macrobatch.  offsets == nullptr: a single dense group of
// dense_rows rows (the shared expert).
// 256 x 256 output tiles (eight-wave blocks) for the groups of at least
// kBigRows rows, in the GEMMs that have that form
constexpr int kBig = 256;
constexpr int kBigRows = 256;
constexpr int kBigDgradTiles = 512;   // down dgrad: least macrobatch rows / 256 x I / 256 for that form

struct GroupRows {
    const int32_t* offsets;   // [E+1] macrobatch-local row offsets
    const int32_t* tile_off;  // [E+1] prefix of row tiles (M-grouped GEMMs)
    int E;
    int rows;                 // rows in the macrobatch (bounds check of offsets)
    int dense_rows;
    int32_t* err;
    // weight gradients: groups of more than deep_thr rows (deep_thr > 0) are
    // left to the deep kernels; deep = [count, expert ids...] of those groups
    // (routed groups; a dense group is deep when dense_rows > deep_thr)
    const int32_t* deep;
    int deep_thr;
    int tm;                   // M-grouped GEMMs: row tile of tile_off (64 or 128; 0 = 64)
    // [E+1] prefix of 256-row tiles over the groups of at least kBigRows rows
    // (GEMMs with a 256 x 256 tile form; null: none).  tile_off then counts
    // only the other groups.
    const int32_t* tile_big;
    // weight gradients: groups of at least big_thr rows (big_thr > 0) go to
    // the 256 x 256 kernels instead, deep_big = [count, expert ids...] (a
    // dense group when dense_rows >= big_thr); deep then lists the others
    const int32_t* deep_big;
    int big_thr;
};

struct GemmGateUpArgs {
    GroupRows g;
    const uint16_t* x;        // routed: token rows gathered through slot_of_row; dense: rows xrow0+
    int x_gather;
    int xrow0;
    const int32_t* slot_of_row;
    int grow0;                // global row of the macrobatch's first row
    int k, S;
    const uint16_t* w_gate;   // [E, I, H]
    const uint16_t* w_up;
    int H, I;
    uint16_t* g_out;          // saved g, row (save_row0 + local row); nullptr: not kept
    uint16_t* u_out;
    int save_row0;
    uint16_t* h_out;          // ring h, local rows
};

// Router weight of each output row, for GEMMs whose epilogue scales their rows
// (the down projection writes w * o so that the combine is a plain sum):
// row r of a macrobatch has weight w[slot_of_row[grow0 + r]]; w == nullptr:
// weight 1 (the shared expert).
struct RowWeights {
    const float* w;
    const int32_t* slot_of_row;
    int grow0, S;
    __device__ float at(int r) const {
        if (!w) return 1.0f;
        const int s = slot_of_row[grow0 + r];
        return (unsigned)s < (unsigned)S ? w[s] : 0.0f;
    }
};

// Where an output row of a routed GEMM goes: its ring row (slot_of_row null),
// or, with one expert per token and no shared expert (top-1 routing), its
// token's row of the caller's output, which then needs no combine or
// reverse-dispatch pass: the row is the token's whole sum.  -1: a bad slot
// (raised, nothing written).
struct RowDest {
    const int32_t* slot_of_row;
    int grow0, k, S;
    __device__ int64_t row(int rl, int32_t* err) const {
        if (!slot_of_row) return rl;
        const int s = slot_of_row[grow0 + rl];
        if ((unsigned)s >= (unsigned)S) {
            raise_err(err, ERR_BAD_SLOT);
            return -1;
        }
        return s / k;
    }
};

struct GemmDownArgs {
    GroupRows g;
    const uint16_t* h;        // ring h [rows, I]
    const uint16_t* w_down;   // [E, H, I]
    int H, I;
    uint16_t* o;              // ring o [rows, H]: w * (h W_down^T) per row
    RowWeights rw;
    RowDest dest;             // null slot_of_row: row rl of o; else the token's row
};

struct GemmDownDgradArgs {
    GroupRows g;
    const uint16_t* dy;
    int dy_gather;
    int dyrow0;
    const int32_t* slot_of_row;
    int grow0, k, S;
    const float* topk_w;      // nullptr: weight 1 (shared expert)
    const uint16_t* w_down;
    int H, I;
    const uint16_t* g_saved;
    const uint16_t* u_saved;
    int save_row0;
    uint16_t* dgu;            // ring [rows, 2I]: dg | du
    uint16_t* hw;             // ring [rows, I]: w * h
    float* dw_part;           // ring [rows, P] or nullptr
    int P;
};

struct GemmGuDgradArgs {
    GroupRows g;
    const uint16_t* dgu;
    const uint16_t* w_gate;
    const uint16_t* w_up;
    int H, I;
    uint16_t* dx;             // ring [rows, H]
    RowDest dest;             // as in GemmDownArgs
};

struct WgradOut {
    uint16_t* out;            // bf16 result
    float* acc;               // fp32 running sums across macrobatches (the expert's slot)
    int mode;                 // 0 bf16; 1 write fp32; 2 add fp32; 3 add fp32 and write bf16
    // routed groups over several macrobatches: the mode is chosen per expert
    // from the schedule's counts [n_macro, E] (see wgrad_mode); nullptr: mode
    const int32_t* counts;
    int m, n_macro, E;
    // routed groups over several macrobatches: each expert's accumulator slot
    // (k_acc_slots; -1: none); nullptr: acc holds one matrix per expert
    // index (or the one dense matrix)
    const int32_t* slot;
};

// Weight-gradient mode of expert e with n rows in macrobatch m, the backward
// walking m = n_macro - 1 .. 0: the fp32 sum is only used by experts with
// rows in several macrobatches; an expert's bf16 result is written once, by
// the last macrobatch of the walk that has its rows (or as zeros at m = 0
// when it has none).  -1: nothing to do.
__host__ __device__ inline int wgrad_mode(const WgradOut& o, int e, int n) {
    if (!o.counts) return o.mode;
    bool earlier = false, later = false;          // rows in macrobatches walked before / after m
    for (int q = o.m + 1; q < o.n_macro; ++q) earlier |= o.counts[(int64_t)q * o.E + e] > 0;
    for (int q = 0; q < o.m; ++q) later |= o.counts[(int64_t)q * o.E + e] > 0;
    if (n == 0) return (o.m == 0 && !earlier) ? 0 : -1;
    if (!earlier) return later ? 1 : 0;
    return later ? 2 : 3;
}

// The mode of expert e's gradient, with o.acc moved to the expert's
// accumulator slot (slot[e] matrices of mat elements from the start instead
// of e), so that acc + the element's index in the output addresses its
// running sum.  An expert that needs a slot and has none (more spanning
// experts than the workspace holds, reported by k_acc_slots) gets -1.
__device__ inline int wgrad_bind(WgradOut& o, int e, int n, int64_t mat) {
    o.mode = wgrad_mode(o, e, n);
    if (o.mode >= 1 && o.slot) {
        const int sl = o.slot[e];
        if (sl < 0) o.mode = -1;
        else o.acc += ((int64_t)sl - e) * mat;
    }
    return o.mode;
}

struct WgradDownArgs {
    GroupRows g;
    const uint16_t* dy;
    int dy_gather, dyrow0;
    const int32_t* slot_of_row;
    int grow0, k, S;
    const uint16_t* hw;
    int H, I;
    WgradOut out;
    const uint16_t* zero;     // kBig zero bf16 values (groups in 256 x 256 tiles)
};

struct WgradGateUpArgs {
    GroupRows g;
    const uint16_t* dgu;
    const uint16_t* x;
    int x_gather, xrow0;
    const int32_t* slot_of_row;
    int grow0, k, S;
    int H, I;
    WgradOut out_gate, out_up;
    const uint16_t* zero;     // kBig zero bf16 values (groups in 256 x 256 tiles)
};

struct GemmGateUpMXArgs {
    GroupRows g;
    int w4;                   // weights in MXFP4: wg_q / wu_q hold E2M1 codes [E, I, H/2]
    const uint8_t* x_q;       // codes [tokens, H]: routed rows gathered by token through
    const uint8_t* x_s;       // slot_of_row (x_gather), dense rows xrow0 + local row; scales [tokens, H/32]
    int xrow0;
    int x_gather;
    const int32_t* slot_of_row;
    int grow0, k, S;
    const uint8_t* wg_q;
    const uint8_t* wg_s;
    const uint8_t* wu_q;
    const uint8_t* wu_s;
    int H, I;
    float* g_out;             // saved g, u in fp32; nullptr: not kept
    float* u_out;
    int save_row0;
    uint8_t* h_q;             // ring codes [rows, I]
    uint8_t* h_s;             // ring scales [rows, I/32]
};

struct GemmDownMXArgs {
    GroupRows g;
    int w4;                   // weights in MXFP4: wd_q holds E2M1 codes [E, H, I/2]
    const uint8_t* h_q;
    const uint8_t* h_s;
    const uint8_t* wd_q;      // [E, H, I]
    const uint8_t* wd_s;      // [E, H, I/32]
    int H, I;
    uint16_t* o;              // w * (Q(h) Q(W_down)^T) per row
    RowWeights rw;
    RowDest dest;             // as in GemmDownArgs
};

// Expert groups padded to whole 32-row blocks (the MXFP8 weight gradients
// quantise along rows).  blk_off == nullptr: one dense group of dense_rows.
struct PadGroups {
    const int32_t* off;       // [E+1] macrobatch-local row offsets
    const int32_t* blk_off;   // [E+1] prefix of ceil(n_e / 32)
    int E, rows, dense_rows;
    int32_t* err;
    const int32_t* deep;      // as in GroupRows
    int deep_thr;
};

// Source rows of a quantise-transpose: value(r, c) for local row r.
struct QtSrc {
    int kind;                 // 0: bf16 rows gathered by token, times the row's weight (w * dy)
                              // 1: fp32 rows [rows, ld]; 2: bf16 rows gathered by token (x)
                              // 3: bf16 rows row0 + r (dense; w = 1)
    const uint16_t* b16;
    const float* f32;
    int64_t ld;
    const int32_t* slot_of_row;
    const float* topk_w;
    int grow0, row0, k, S;
};

struct GemmDownDgradMXArgs {
    GroupRows g;
    const uint8_t* dy_q;      // [T, H] codes of dy (quantised along H)
    const uint8_t* dy_s;
    int dy_gather, dyrow0;
    const int32_t* slot_of_row;
    int grow0, k, S;
    const float* topk_w;      // nullptr: weight 1
    const uint8_t* wdt_q;     // [E, I, H] W_down^T codes
    const uint8_t* wdt_s;
    int H, I;
    const float* g_saved;     // fp32
    const float* u_saved;
    int save_row0;
    // h and [dg | du], quantised along the rows of each group and written
    // transposed, group by group (launch_mx_quant_group_t's layout)
    const int32_t* blk_off;   // [E+1] prefix of each group's 32-row blocks (null: one dense group)
    uint8_t* th;
    uint8_t* ths;
    uint8_t* tdgu;
    uint8_t* tdgus;
    uint8_t* dgu_q;           // ring [rows, 2I] codes along I
    uint8_t* dgu_s;           // ring [rows, 2I/32]
    float* dw_part;
    int P;
};

struct GemmGuDgradMXArgs {
    GroupRows g;
    const uint8_t* dgu_q;
    const uint8_t* dgu_s;
    const uint8_t* wgt_q;     // [E, H, I] W_gate^T codes
    const uint8_t* wgt_s;
    const uint8_t* wut_q;
    const uint8_t* wut_s;
    int H, I;
    uint16_t* dx;             // ring [rows, H] bf16
    RowDest dest;             // as in GemmDownArgs
};

struct WgradMXArgs {
    PadGroups g;
    const uint8_t* at_q;      // per group: [M, np_e] codes, K = the group's padded rows
    const uint8_t* at_s;      // per group: [M, np_e / 32]
    const uint8_t* bt_q;      // per group: [N, np_e]
    const uint8_t* bt_s;
    int M, N;
    int msplit;               // rows m >= msplit go to out_hi (row m - msplit)
    WgradOut out_lo, out_hi;
};

// route_sched.hip
int launch_acc_slots(const int32_t* counts, int n_macro, int E, int cap, int32_t* slot, int32_t* err,
                     hipStream_t st);
int launch_topk_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                      hipStream_t st);
int launch_schedule(const int32_t* idx, int T, int E, int k, int M, int mb, int32_t* hist,
                    int32_t* base, int32_t* counts, int32_t* offsets, int32_t* mini_counts,
                    int32_t* row_of_slot, int32_t* slot_of_row, int32_t* err, hipStream_t st);
size_t schedule_hist_ints(int T, int E, int k, int M, int mb);

// elementwise.hip
int launch_combine(const void* o, int H, const int32_t* row_of_slot, const float* w, int t0, int t1,
                   int k, int ring_row0, int ring_rows, const void* shared, int shared_t0, void* y,
                   int32_t* err, hipStream_t st);
int launch_rd_reduce(const void* dxd, int H, const int32_t* row_of_slot, int t0, int t1, int k,
                     int ring_row0, int ring_rows, const void* shared, int shared_t0, void* dx,
                     int32_t* err, hipStream_t st);
int launch_softmax_bwd(const float* part, int P, const int32_t* row_of_slot, const int32_t* idx,
                       const float* w, int t0, int t1, int k, int E, int ring_row0, int ring_rows,
                       float* dw, float* d_logits, int32_t* err, hipStream_t st);
int launch_tile_prefix(const int32_t* offsets, int E, int rows, int TM, int32_t* tile_off,
                       int32_t* err, hipStream_t st);
// the same, plus the prefixes over the groups below big_rows rows (TM-row
// tiles) and over the rest (big_tm-row tiles)
int launch_tile_prefix_split(const int32_t* offsets, int E, int rows, int TM, int32_t* tile_off,
                             int big_rows, int big_tm, int32_t* small, int32_t* big, int32_t* err,
                             hipStream_t st);
int launch_deep_list(const int32_t* offsets, int E, int rows, int thr, int32_t* list, hipStream_t st);
// the same, with the groups of at least big_thr rows in a list of their own
int launch_deep_list_split(const int32_t* offsets, int E, int rows, int thr, int32_t* list, int big_thr,
                           int32_t* big, hipStream_t st);

// mx.hip
int launch_mx_quant_rows(const void* x, int64_t rows, int K, void* codes, void* scales, hipStream_t st,
                         int kmaj_rows = 0);
int launch_mx_quant_cols(const void* w, int batch, int R, int C, void* codes, void* scales,
                         hipStream_t st);
int launch_mx4_quant_rows(const void* w, int64_t rows, int K, int kmaj_rows, void* codes, void* scales,
                          hipStream_t st);

int launch_mx_quant_group_t(const PadGroups& g, const QtSrc& src, int C, void* codes, void* scales,
                            hipStream_t st);

// gemm_mx.hip
int launch_gemm_down_dgrad_mx(const GemmDownDgradMXArgs& a, hipStream_t st);
int launch_gemm_gu_dgrad_mx(const GemmGuDgradMXArgs& a, hipStream_t st);
int launch_wgrad_mx(const WgradMXArgs& a, hipStream_t st);
int launch_gemm_gate_up_mx(const GemmGateUpMXArgs& a, hipStream_t st);
int launch_gemm_down_mx(const GemmDownMXArgs& a, hipStream_t st);

// router.hip
int router_padded_experts(int E);
int launch_router_logits(const void* x, const void* wr, float* logits, int T, int H, int E, hipStream_t st);
int launch_router_backward(const void* x, const void* wr, const float* d_logits, void* dx, void* dwr,
                           void* dl16, int T, int H, int E, hipStream_t st);

// gemm.hip
int launch_gemm_gate_up(const GemmGateUpArgs& a, hipStream_t st);
int launch_gemm_down(const GemmDownArgs& a, hipStream_t st);
int launch_gemm_down_dgrad(const GemmDownDgradArgs& a, hipStream_t st);
int launch_gemm_gu_dgrad(const GemmGuDgradArgs& a, hipStream_t st);
int launch_wgrad_down(const WgradDownArgs& a, hipStream_t st);
int launch_wgrad_gate_up(const WgradGateUpArgs& a, hipStream_t st);
int gemm_row_tile(int rows, int E);   // M-grouped row tile for a macrobatch of rows over E groups
int dgrad_col_tiles(int I);
int wgrad_deep_rows();        // bf16 weight gradients: groups above this go to the deep kernels
int wgrad_big_rows();         // ... and groups of at least this many rows to the 256 x 256 kernels
// blocks of the 256 x 256 weight-gradient kernels' persistent grid
int wgrad_big_grid();
int wgrad_deep_rows_mx();     // MXFP8 weight gradients: the same, in rows

}  // namespace moe
