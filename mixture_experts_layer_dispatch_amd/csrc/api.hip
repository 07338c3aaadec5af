// C ABI of the MoE layer: argument validation, workspace layout, and the
// launch sequence of each call.  Host code only (plus two one-thread kernels
// that read and clear the device error word).
//
// The order of work follows the pages: routing, then one schedule table
// (arex-research.com "Cursor 放出 MoK", design section, first decision);
// the forward walks macrobatches in order through a ring buffer filled per
// minibatch, and the backward walks them in reverse (second decision);
// alphalab.site "Mixture-of-Kittens" section 二: the router-weighted
// reduction closes the forward.
#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "common.h"
#include "launch.h"

using namespace moe;

namespace {

struct Geom {
    int T, H, I, E, k, M, mb, n_macro, n_mini, Sm, Smb, S, P;
    int64_t ring_rows;
    int halves;
    bool shared, mx, w4, recompute;
    int acc_cap;              // experts with fp32 running sums across macrobatches
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
    size_t err, hist, base, tile_off, tile_split, deep, deep_big, zero, ring, ring_half, sh, wacc, total;
    // offsets inside one ring half (bytes)
    size_t f_h, f_o;                  // forward
    size_t f_hs;                      // MXFP8 forward: h scales after the codes (codes at f_h)
    size_t b_dgu, b_hw, b_dx, b_part; // backward
    // offsets inside the shared-expert region
    size_t s_h, s_o, s_dgu, s_hw, s_dx;
    size_t s_hq, s_hs;                // MXFP8 shared expert
    size_t xq, xs;                    // MXFP8 forward: x codes / scales [T, H] (quantised once)
    // MXFP8 backward
    size_t dyq, dys;                  // dy codes / scales [T, H]
    size_t x_dguq, x_dgus, x_dx, x_part;                    // inside a ring half
    size_t tr, tr_wdy, tr_wdys, tr_h, tr_hs, tr_dgu, tr_dgus, tr_x, tr_xs, blk_off;
    size_t tr_sh, tr_shs, tr_sdgu, tr_sdgus;               // the shared expert's h, dg | du
    int64_t kcap;
    size_t s_dguq, s_dgus, s_dxm;                          // shared expert
    size_t wacc_g, wacc_u, wacc_d, wacc_sg, wacc_su, wacc_sd;
    size_t acc_slot;                  // int32 [E]: each routed expert's accumulator slot
    size_t rc_g, rc_u, rc_sg, rc_su;  // recompute mode: one macrobatch's g, u (and the shared expert's)
    size_t dl16;                      // router backward: bf16 d_logits [T, Ep]
};

moe_status make_geom(const moe_config* c, Geom& g) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->T < 1 || c->H < 128 || c->H % 128 || c->I < 128 || c->I % 128) return MOE_ERR_INVALID_ARG;
    if (c->E < 1 || c->E > kMaxExperts || c->k < 1 || c->k > c->E || c->k > kMaxTopK)
        return MOE_ERR_INVALID_ARG;
    if (c->n_shared != 0 && c->n_shared != 1) return MOE_ERR_INVALID_ARG;
    if (c->precision != MOE_PREC_BF16 && c->precision != MOE_PREC_MXFP8 && c->precision != MOE_PREC_MXFP4)
        return MOE_ERR_INVALID_ARG;
    if ((c->flags & ~MOE_FLAG_RECOMPUTE) != 0 || c->macrobatch < 0 || c->minibatch < 0 ||
        c->capacity_rows < 0 || c->acc_experts < 0)
        return MOE_ERR_INVALID_ARG;
    if (c->H > (1 << 16) || c->I > (1 << 16)) return MOE_ERR_INVALID_ARG;
    const int64_t S = (int64_t)c->T * c->k;
    if (S >= (1LL << 30)) return MOE_ERR_INVALID_ARG;
    g.T = c->T; g.H = c->H; g.I = c->I; g.E = c->E; g.k = c->k;
    g.M = c->macrobatch ? c->macrobatch : c->T;
    if (g.M > g.T || g.T % g.M) return MOE_ERR_INVALID_ARG;
    g.mb = c->minibatch ? c->minibatch : g.M;
    if (g.mb > g.M || g.M % g.mb) return MOE_ERR_INVALID_ARG;
    g.n_macro = g.T / g.M;
    g.n_mini = g.M / g.mb;
    g.Sm = g.M * g.k;
    g.Smb = g.mb * g.k;
    g.S = (int)S;
    g.P = dgrad_col_tiles(g.I);
    g.shared = c->n_shared == 1;
    g.mx = c->precision != MOE_PREC_BF16;           // MXFP8 activations in both MX modes
    g.w4 = c->precision == MOE_PREC_MXFP4;
    g.recompute = (c->flags & MOE_FLAG_RECOMPUTE) != 0;
    g.acc_cap = c->acc_experts > 0 && c->acc_experts < c->E ? c->acc_experts : c->E;
    if (c->capacity_rows) {
        if (c->capacity_rows < g.Sm) return MOE_ERR_CAPACITY;
        g.ring_rows = c->capacity_rows;
    } else {
        g.ring_rows = g.n_macro > 1 ? 2LL * g.Sm : g.Sm;
    }
    g.halves = (int)(g.ring_rows / g.Sm);
    if (g.halves > g.n_macro) g.halves = g.n_macro;
    return MOE_OK;
}

Layout make_layout(const Geom& g) {
    Layout L{};
    size_t at = 0;
    auto take = [&](size_t bytes) {
        size_t here = at;
        at = align_up(at + bytes, 256);
        return here;
    };
    L.err = take(256);
    const size_t hist_ints = schedule_hist_ints(g.T, g.E, g.k, g.M, g.mb);
    L.hist = take(hist_ints * 4);
    L.base = take(hist_ints * 4);
    L.tile_off = take((size_t)g.n_macro * (g.E + 1) * 4);
    // per macrobatch: the tile prefixes of the groups below kBigRows rows and
    // of the others (256-row tiles), for the down GEMM's two tile forms
    L.tile_split = take((size_t)g.n_macro * 2 * (g.E + 1) * 4);
    L.deep = take((size_t)(g.E + 1) * 4);        // deep weight-gradient groups of one macrobatch
    L.deep_big = take((size_t)(g.E + 1) * 4);    // ... and those in 256 x 256 tiles
    L.zero = take(1024);                         // zeros the 256 x 256 weight gradients read past a group
    const size_t Sm = (size_t)g.Sm, H = g.H, I = g.I;
    // the forward's ring rows: h and the weighted o of the macrobatch (the
    // dispatched x rows are gathered by the gate/up GEMM's loads, never stored)
    L.f_h = 0;
    L.f_o = align_up(L.f_h + Sm * I * 2, 256);
    const size_t fwd_end = align_up(L.f_o + Sm * H * 2, 256);
    // MXFP8 codes take one byte, so codes + scales fit in the bf16 slot
    L.f_hs = align_up(L.f_h + Sm * I, 256);
    L.b_dgu = 0;
    L.b_hw = align_up(L.b_dgu + Sm * 2 * I * 2, 256);
    L.b_dx = align_up(L.b_hw + Sm * I * 2, 256);
    L.b_part = align_up(L.b_dx + Sm * H * 2, 256);
    const size_t bwd_end = align_up(L.b_part + Sm * g.P * 4, 256);
    L.ring_half = fwd_end > bwd_end ? fwd_end : bwd_end;
    if (g.mx) {
        L.x_dguq = 0;
        L.x_dgus = align_up(L.x_dguq + Sm * 2 * I, 256);
        L.x_dx = align_up(L.x_dgus + Sm * 2 * I / 32, 256);
        L.x_part = align_up(L.x_dx + Sm * H * 2, 256);
        const size_t mx_end = align_up(L.x_part + Sm * g.P * 4, 256);
        if (mx_end > L.ring_half) L.ring_half = mx_end;
    }
    L.ring = take(L.ring_half * g.halves);
    if (g.mx) {
        L.xq = take((size_t)g.T * H);
        L.xs = take((size_t)g.T * H / 32);
        L.dyq = take((size_t)g.T * H);
        L.dys = take((size_t)g.T * H / 32);
        // transposed, row-quantised operands of the weight gradients (one macrobatch,
        // group-major); kcap bounds the macrobatch's rows padded group by group to 32.
        // Scale regions keep 16 spare bytes: their reader loads aligned words.
        L.kcap = (int64_t)align_up(Sm + 32 * (size_t)g.E, 128);
        const size_t kc = (size_t)L.kcap;
        L.tr_wdy = take(H * kc);
        L.tr_wdys = take(H * kc / 32 + 16);
        L.tr_h = take(I * kc);
        L.tr_hs = take(I * kc / 32 + 16);
        L.tr_dgu = take(2 * I * kc);
        L.tr_dgus = take(2 * I * kc / 32 + 16);
        L.tr_x = take(H * kc);
        L.tr_xs = take(H * kc / 32 + 16);
        L.blk_off = take((size_t)(g.E + 1) * 4);
    }
    const size_t M = (size_t)g.M;
    if (g.shared) {
        L.s_h = 0;
        L.s_o = align_up(M * I * 2, 256);
        L.s_hq = align_up(L.s_o + M * H * 2, 256);
        L.s_hs = align_up(L.s_hq + M * I, 256);
        const size_t fe = align_up(L.s_hs + M * I / 32, 256);
        L.s_dgu = 0;
        L.s_hw = align_up(M * 2 * I * 2, 256);
        L.s_dx = align_up(L.s_hw + M * I * 2, 256);
        size_t be = align_up(L.s_dx + M * H * 2, 256);
        if (g.mx) {
            L.s_dguq = 0;
            L.s_dgus = align_up(L.s_dguq + M * 2 * I, 256);
            L.s_dxm = align_up(L.s_dgus + M * 2 * I / 32, 256);
            const size_t me = align_up(L.s_dxm + M * H * 2, 256);
            if (me > be) be = me;
        }
        L.sh = take(fe > be ? fe : be);
        if (g.mx) {                  // its transposed h and dg | du (one dense group of M rows)
            const size_t kcs = align_up(M, 128);
            L.tr_sh = take(I * kcs);
            L.tr_shs = take(I * kcs / 32 + 16);
            L.tr_sdgu = take(2 * I * kcs);
            L.tr_sdgus = take(2 * I * kcs / 32 + 16);
        }
    }
    L.dl16 = take((size_t)g.T * router_padded_experts(g.E) * 2);
    if (g.recompute) {
        const size_t es = g.mx ? 4 : 2;                 // fp32 in MXFP8 mode, as the saved ones
        L.rc_g = take(Sm * I * es);
        L.rc_u = take(Sm * I * es);
        if (g.shared) {
            L.rc_sg = take(M * I * es);
            L.rc_su = take(M * I * es);
        }
    }
    if (g.n_macro > 1) {
        // fp32 running sums for the acc_cap experts that may take rows from
        // several macrobatches (slots assigned on the device, k_acc_slots)
        const size_t per = (size_t)g.acc_cap * I * H * 4;
        L.wacc_g = 0;
        L.wacc_u = per;
        L.wacc_d = 2 * per;
        size_t end = 3 * per;
        if (g.shared) {
            L.wacc_sg = end;
            L.wacc_su = end + I * H * 4;
            L.wacc_sd = end + 2 * I * H * 4;
            end += 3 * I * H * 4;
        }
        L.wacc = take(end);
        L.acc_slot = take((size_t)g.E * 4);
    }
    L.total = at;
    return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

std::atomic<int> g_dev_ok[64];   // 0 unknown, 1 gfx950, 2 other

bool device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return false;
    }
    if (dev < 64) {
        const int v = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (v) return v == 1;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok;
}

__global__ void k_clear_word(int32_t* p) { *p = 0; }
__global__ void k_clear_words(int32_t* p) { p[threadIdx.x] = 0; }

moe_status common_checks(const moe_config* cfg, Geom& g, Layout& L, void* ws, size_t ws_bytes) {
    moe_status s = make_geom(cfg, g);
    if (s != MOE_OK) return s;
    L = make_layout(g);
    if (!ws || !aligned(ws, 256) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

bool sched_ok(const moe_sched* s) {
    return s && s->topk_idx && s->topk_w && s->counts && s->offsets && s->mini_counts &&
           s->row_of_slot && s->slot_of_row && aligned(s->topk_idx, 4) && aligned(s->topk_w, 4) &&
           aligned(s->counts, 4) && aligned(s->offsets, 4) && aligned(s->mini_counts, 4) &&
           aligned(s->row_of_slot, 4) && aligned(s->slot_of_row, 4);
}

bool bf16_ok(const void* p) { return p && aligned(p, 16); }

// the saved activations: not used in recompute mode (saved may then be null)
bool saved_ok(const Geom& g, const moe_saved* s) {
    if (g.recompute) return true;
    if (!s || !bf16_ok(s->g) || !bf16_ok(s->u)) return false;
    return !g.shared || (bf16_ok(s->sg) && bf16_ok(s->su));
}

struct Ptrs {
    char* ws;
    const Layout* L;
    int32_t* err() const { return (int32_t*)(ws + L->err); }
    char* half(int m, int halves) const { return ws + L->ring + (size_t)(m % halves) * L->ring_half; }
    char* sh() const { return ws + L->sh; }
    float* wacc(size_t off) const { return (float*)(ws + L->wacc + off); }
    int32_t* acc_slot() const { return (int32_t*)(ws + L->acc_slot); }
};

// Top-1 routing without a shared expert: a token's layer output (and input
// gradient) is its one routed row, so the down GEMM (and the gate/up input
// gradient) write it straight to the token's row of y (dx) and the combine
// (reverse-dispatch) pass is skipped.  The single fp32 term rounds once
// either way, so the bits are those of the combine.
bool top1_direct(const Geom& g) { return g.k == 1 && !g.shared; }

RowDest token_rows(const Geom& g, const moe_sched* s, int grow0) {
    return top1_direct(g) ? RowDest{s->slot_of_row, grow0, g.k, g.S} : RowDest{nullptr, 0, 1, 0};
}

// Where macrobatch m's gate and up projections are kept for the backward:
// the caller's saved arrays (rows of the whole batch), or in recompute mode
// the workspace's one-macrobatch buffers (local rows), which the forward
// fills for the last macrobatch only and the backward refills for the others.
struct GU {
    void* g;
    void* u;
    int row0;
};

GU gu_routed(const Geom& g, const Layout& L, const Ptrs& P, const moe_saved* saved, int m, bool fwd) {
    if (!g.recompute) return {saved->g, saved->u, m * g.Sm};
    if (fwd && m != g.n_macro - 1) return {nullptr, nullptr, 0};
    return {P.ws + L.rc_g, P.ws + L.rc_u, 0};
}

GU gu_shared(const Geom& g, const Layout& L, const Ptrs& P, const moe_saved* saved, int m, bool fwd) {
    if (!g.recompute) return {saved->sg, saved->su, m * g.M};
    if (fwd && m != g.n_macro - 1) return {nullptr, nullptr, 0};
    return {P.ws + L.rc_sg, P.ws + L.rc_su, 0};
}


// MXFP8 forward: x is quantised along H once per token; the gate/up GEMM
// gathers each routed row's codes by token on load (dispatch fused into the
// operand loads) and quantises h along I in its epilogue; the down GEMM
// writes each row scaled by its router weight; the combine sums a token's
// rows in a fixed order.
moe_status forward_mx(const Geom& g, const Layout& L, const Ptrs& P, const moe_sched* sched,
                      const void* x, const moe_weights* w, void* y, const moe_saved* saved,
                      hipStream_t st) {
    // forward weights: MXFP8 codes, or E2M1 codes (two per byte) in MXFP4 mode;
    // the scales have the same layout in both
    struct FwdW {
        const void *gq, *gs, *uq, *us, *dq, *ds, *sgq, *sgs, *suq, *sus, *sdq, *sds;
    } fw;
    if (g.w4) {
        const moe_weights_mx4* q = w->mx4;
        fw = {q->w_gate_q, q->w_gate_s, q->w_up_q, q->w_up_s, q->w_down_q, q->w_down_s,
              q->s_gate_q, q->s_gate_s, q->s_up_q, q->s_up_s, q->s_down_q, q->s_down_s};
    } else {
        const moe_weights_mx* q = w->mx;
        fw = {q->w_gate_q, q->w_gate_s, q->w_up_q, q->w_up_s, q->w_down_q, q->w_down_s,
              q->s_gate_q, q->s_gate_s, q->s_up_q, q->s_up_s, q->s_down_q, q->s_down_s};
    }
    const int w4 = g.w4 ? 1 : 0;
    int32_t* err = P.err();
    const int tm = gemm_row_tile(g.Sm, g.E);            // row tile of the M-grouped GEMMs
    uint8_t* xq = (uint8_t*)(P.ws + L.xq);
    uint8_t* xs = (uint8_t*)(P.ws + L.xs);
    if (launch_mx_quant_rows(x, g.T, g.H, xq, xs, st)) return MOE_ERR_HIP;
    for (int m = 0; m < g.n_macro; ++m) {
        char* half = P.half(m, g.halves);
        uint8_t* hq = (uint8_t*)(half + L.f_h);
        uint8_t* hs = (uint8_t*)(half + L.f_hs);
        uint16_t* obuf = (uint16_t*)(half + L.f_o);
        const int grow0 = m * g.Sm, t0 = m * g.M;
        const int32_t* off = sched->offsets + (size_t)m * (g.E + 1);
        int32_t* toff = (int32_t*)(P.ws + L.tile_off) + (size_t)m * (g.E + 1);
        // MXFP8 weights: the gate/up GEMM takes groups of at least kBigRows
        // rows in 256 x 256 tiles when groups are large on average
        const bool big = !g.w4 && tm == 128 && g.I % (kBig / 2) == 0;
        int32_t* tsmall = (int32_t*)(P.ws + L.tile_split) + (size_t)m * 2 * (g.E + 1);
        int32_t* tbig = tsmall + (g.E + 1);
        if (big ? launch_tile_prefix_split(off, g.E, g.Sm, tm, toff, kBigRows, kBig, tsmall, tbig, err, st)
                : launch_tile_prefix(off, g.E, g.Sm, tm, toff, err, st))
            return MOE_ERR_HIP;
        GroupRows grp{off, toff, g.E, g.Sm, 0, err, nullptr, 0, tm};
        GroupRows grp_split = grp;
        if (big) {
            grp_split.tile_off = tsmall;
            grp_split.tile_big = tbig;
        }
        const GU keep = gu_routed(g, L, P, saved, m, true);
        GemmGateUpMXArgs a1{grp_split, w4, xq, xs, 0, 1, sched->slot_of_row, grow0, g.k, g.S,
                            (const uint8_t*)fw.gq, (const uint8_t*)fw.gs, (const uint8_t*)fw.uq,
                            (const uint8_t*)fw.us, g.H, g.I, (float*)keep.g, (float*)keep.u, keep.row0,
                            hq, hs};
        if (launch_gemm_gate_up_mx(a1, st)) return MOE_ERR_HIP;
        GemmDownMXArgs a2{grp, w4, hq, hs, (const uint8_t*)fw.dq, (const uint8_t*)fw.ds, g.H, g.I,
                          top1_direct(g) ? (uint16_t*)y : obuf, {sched->topk_w, sched->slot_of_row, grow0, g.S},
                          token_rows(g, sched, grow0)};
        if (launch_gemm_down_mx(a2, st)) return MOE_ERR_HIP;
        const uint16_t* sh_o = nullptr;
        if (g.shared) {
            char* sh = P.sh();
            uint8_t* shq = (uint8_t*)(sh + L.s_hq);
            uint8_t* shs = (uint8_t*)(sh + L.s_hs);
            uint16_t* so = (uint16_t*)(sh + L.s_o);
            GroupRows dense{nullptr, nullptr, 1, g.M, g.M, err, nullptr, 0, gemm_row_tile(g.M, 1)};
            const GU skeep = gu_shared(g, L, P, saved, m, true);
            GemmGateUpMXArgs s1{dense, w4, xq, xs, t0, 0, nullptr, 0, g.k, g.S,
                                (const uint8_t*)fw.sgq, (const uint8_t*)fw.sgs, (const uint8_t*)fw.suq,
                                (const uint8_t*)fw.sus, g.H, g.I, (float*)skeep.g, (float*)skeep.u,
                                skeep.row0, shq, shs};
            if (launch_gemm_gate_up_mx(s1, st)) return MOE_ERR_HIP;
            GemmDownMXArgs s2{dense, w4, shq, shs, (const uint8_t*)fw.sdq, (const uint8_t*)fw.sds, g.H, g.I,
                              so, {nullptr, nullptr, 0, 0}};
            if (launch_gemm_down_mx(s2, st)) return MOE_ERR_HIP;
            sh_o = so;
        }
        if (!top1_direct(g) && launch_combine(obuf, g.H, sched->row_of_slot, nullptr, t0, t0 + g.M, g.k, grow0,
                                              g.Sm, sh_o, t0, y, err, st))
            return MOE_ERR_HIP;
    }
    return MOE_OK;
}


// MXFP8 backward.  Every GEMM runs on the scaled fp8 MFMA with its operands
// quantised along that GEMM's reduction axis: dy along H; dg | du along I
// (quantised in the down-dgrad epilogue from fp32); and for the weight
// gradients, whose reduction runs over an expert's rows, w*dy, h, dg | du and
// x in 32-row blocks of the expert's group, written transposed.
moe_status backward_mx(const Geom& g, const Layout& L, const Ptrs& P, const moe_sched* sched,
                       const moe_saved* saved, const void* x, const moe_weights* w, const void* dy,
                       void* dx, const moe_grads* gr, float* dw, float* d_logits, hipStream_t st) {
    const moe_weights_mx* wq = w->mx;
    int32_t* err = P.err();
    char* ws = P.ws;
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* dyb = (const uint16_t*)dy;
    uint8_t* dyq = (uint8_t*)(ws + L.dyq);
    uint8_t* dys = (uint8_t*)(ws + L.dys);
    if (launch_mx_quant_rows(dy, g.T, g.H, dyq, dys, st)) return MOE_ERR_HIP;
    uint8_t* xq = (uint8_t*)(ws + L.xq);
    uint8_t* xs = (uint8_t*)(ws + L.xs);
    if (g.recompute && g.n_macro > 1 && launch_mx_quant_rows(x, g.T, g.H, xq, xs, st))
        return MOE_ERR_HIP;                     // the codes the recomputation gathers
    uint8_t* twdy = (uint8_t*)(ws + L.tr_wdy);
    uint8_t* twdys = (uint8_t*)(ws + L.tr_wdys);
    uint8_t* th = (uint8_t*)(ws + L.tr_h);
    uint8_t* ths = (uint8_t*)(ws + L.tr_hs);
    uint8_t* tdgu = (uint8_t*)(ws + L.tr_dgu);
    uint8_t* tdgus = (uint8_t*)(ws + L.tr_dgus);
    uint8_t* tx = (uint8_t*)(ws + L.tr_x);
    uint8_t* txs = (uint8_t*)(ws + L.tr_xs);
    int32_t* blk = (int32_t*)(ws + L.blk_off);
    // counts: the schedule's [n_macro, E] counts for routed groups over several
    // macrobatches (per-expert modes), nullptr otherwise
    auto wgrads = [&](const PadGroups& pg, const uint8_t* ah, const uint8_t* ahs, const uint8_t* adgu,
                      const uint8_t* adgus, int mode, const int32_t* counts, int m, uint16_t* dwd,
                      float* accd, uint16_t* dwg, float* accg, uint16_t* dwu, float* accu) -> bool {
        const int32_t* sl = counts ? P.acc_slot() : nullptr;
        WgradMXArgs d{pg, twdy, twdys, ah, ahs, g.H, g.I, g.H,
                      {dwd, accd, mode, counts, m, g.n_macro, g.E, sl},
                      {dwd, accd, mode, counts, m, g.n_macro, g.E, sl}};
        if (launch_wgrad_mx(d, st)) return false;
        WgradMXArgs gu{pg, adgu, adgus, tx, txs, 2 * g.I, g.H, g.I,
                       {dwg, accg, mode, counts, m, g.n_macro, g.E, sl},
                       {dwu, accu, mode, counts, m, g.n_macro, g.E, sl}};
        return launch_wgrad_mx(gu, st) == 0;
    };
    const int tm = gemm_row_tile(g.Sm, g.E);            // row tile of the M-grouped GEMMs
    for (int m = g.n_macro - 1; m >= 0; --m) {
        int mode = 0;
        if (g.n_macro > 1) mode = (m == g.n_macro - 1) ? 1 : (m == 0 ? 3 : 2);
        char* half = P.half(m, g.halves);
        uint8_t* dguq = (uint8_t*)(half + L.x_dguq);
        uint8_t* dgus = (uint8_t*)(half + L.x_dgus);
        uint16_t* dxd = (uint16_t*)(half + L.x_dx);
        float* part = (float*)(half + L.x_part);
        const int grow0 = m * g.Sm, t0 = m * g.M;
        const int32_t* off = sched->offsets + (size_t)m * (g.E + 1);
        int32_t* toff = (int32_t*)(ws + L.tile_off) + (size_t)m * (g.E + 1);
        if (launch_tile_prefix(off, g.E, g.Sm, tm, toff, err, st)) return MOE_ERR_HIP;
        if (launch_tile_prefix(off, g.E, g.Sm, 32, blk, err, st)) return MOE_ERR_HIP;
        GroupRows grp{off, toff, g.E, g.Sm, 0, err, nullptr, 0, tm};
        const GU gu = gu_routed(g, L, P, saved, m, false);
        if (g.recompute && m != g.n_macro - 1) {
            // recompute this macrobatch's g, u (h codes go to scratch that the
            // dgrad below overwrites)
            GemmGateUpMXArgs r1{grp, 0, xq, xs, 0, 1, sched->slot_of_row, grow0, g.k, g.S,
                                (const uint8_t*)wq->w_gate_q, (const uint8_t*)wq->w_gate_s,
                                (const uint8_t*)wq->w_up_q, (const uint8_t*)wq->w_up_s, g.H, g.I,
                                (float*)gu.g, (float*)gu.u, 0, dguq, dgus};
            if (launch_gemm_gate_up_mx(r1, st)) return MOE_ERR_HIP;
        }
        GemmDownDgradMXArgs b1{grp, dyq, dys, 1, 0, sched->slot_of_row, grow0, g.k, g.S,
                               sched->topk_w, (const uint8_t*)wq->w_down_tq,
                               (const uint8_t*)wq->w_down_ts, g.H, g.I, (const float*)gu.g,
                               (const float*)gu.u, gu.row0, blk, th, ths, tdgu, tdgus, dguq, dgus,
                               part, g.P};
        if (launch_gemm_down_dgrad_mx(b1, st)) return MOE_ERR_HIP;
        GemmGuDgradMXArgs b2{grp, dguq, dgus, (const uint8_t*)wq->w_gate_tq,
                             (const uint8_t*)wq->w_gate_ts, (const uint8_t*)wq->w_up_tq,
                             (const uint8_t*)wq->w_up_ts, g.H, g.I, top1_direct(g) ? (uint16_t*)dx : dxd,
                             token_rows(g, sched, grow0)};
        if (launch_gemm_gu_dgrad_mx(b2, st)) return MOE_ERR_HIP;
        // the shared expert's input gradient, then reverse-dispatch and the
        // softmax backward while dXd is still in cache; the weight gradients
        // (the large writes) come last
        const uint16_t* sh_dx = nullptr;
        char* sh = g.shared ? P.sh() : nullptr;
        GroupRows dense{nullptr, nullptr, 1, g.M, g.M, err, nullptr, 0, gemm_row_tile(g.M, 1)};
        if (g.shared) {
            uint8_t* sdguq = (uint8_t*)(sh + L.s_dguq);
            uint8_t* sdgus = (uint8_t*)(sh + L.s_dgus);
            uint16_t* sdx = (uint16_t*)(sh + L.s_dxm);
            const GU sgu = gu_shared(g, L, P, saved, m, false);
            if (g.recompute && m != g.n_macro - 1) {
                GemmGateUpMXArgs r2{dense, 0, xq, xs, t0, 0, nullptr, 0, g.k, g.S,
                                    (const uint8_t*)wq->s_gate_q, (const uint8_t*)wq->s_gate_s,
                                    (const uint8_t*)wq->s_up_q, (const uint8_t*)wq->s_up_s, g.H, g.I,
                                    (float*)sgu.g, (float*)sgu.u, 0, sdguq, sdgus};
                if (launch_gemm_gate_up_mx(r2, st)) return MOE_ERR_HIP;
            }
            GemmDownDgradMXArgs c1{dense, dyq, dys, 0, t0, nullptr, 0, g.k, g.S, nullptr,
                                   (const uint8_t*)wq->s_down_tq, (const uint8_t*)wq->s_down_ts, g.H,
                                   g.I, (const float*)sgu.g, (const float*)sgu.u, sgu.row0, nullptr,
                                   (uint8_t*)(ws + L.tr_sh), (uint8_t*)(ws + L.tr_shs),
                                   (uint8_t*)(ws + L.tr_sdgu), (uint8_t*)(ws + L.tr_sdgus), sdguq, sdgus,
                                   nullptr, g.P};
            if (launch_gemm_down_dgrad_mx(c1, st)) return MOE_ERR_HIP;
            GemmGuDgradMXArgs c2{dense, sdguq, sdgus, (const uint8_t*)wq->s_gate_tq,
                                 (const uint8_t*)wq->s_gate_ts, (const uint8_t*)wq->s_up_tq,
                                 (const uint8_t*)wq->s_up_ts, g.H, g.I, sdx};
            if (launch_gemm_gu_dgrad_mx(c2, st)) return MOE_ERR_HIP;
            sh_dx = sdx;
        }
        if (!top1_direct(g) && launch_rd_reduce(dxd, g.H, sched->row_of_slot, t0, t0 + g.M, g.k, grow0, g.Sm,
                                                sh_dx, t0, dx, err, st))
            return MOE_ERR_HIP;
        if (launch_softmax_bwd(part, g.P, sched->row_of_slot, sched->topk_idx, sched->topk_w, t0,
                               t0 + g.M, g.k, g.E, grow0, g.Sm, dw, d_logits, err, st))
            return MOE_ERR_HIP;
        int32_t* deep = (int32_t*)(ws + L.deep);
        if (launch_deep_list(off, g.E, g.Sm, wgrad_deep_rows_mx(), deep, st)) return MOE_ERR_HIP;
        PadGroups pg{off, blk, g.E, g.Sm, 0, err, deep, wgrad_deep_rows_mx()};
        // (h and dg | du were quantised and transposed by the down input gradient)
        QtSrc qwdy{0, dyb, nullptr, g.H, sched->slot_of_row, sched->topk_w, grow0, 0, g.k, g.S};
        QtSrc qx{2, xb, nullptr, g.H, sched->slot_of_row, nullptr, grow0, 0, g.k, g.S};
        if (launch_mx_quant_group_t(pg, qwdy, g.H, twdy, twdys, st) ||
            launch_mx_quant_group_t(pg, qx, g.H, tx, txs, st))
            return MOE_ERR_HIP;
        const int32_t* cnts = g.n_macro > 1 ? sched->counts : nullptr;
        if (!wgrads(pg, th, ths, tdgu, tdgus, mode, cnts, m, (uint16_t*)gr->d_w_down, P.wacc(L.wacc_d),
                    (uint16_t*)gr->d_w_gate, P.wacc(L.wacc_g), (uint16_t*)gr->d_w_up, P.wacc(L.wacc_u)))
            return MOE_ERR_HIP;
        if (g.shared) {
            PadGroups pd{nullptr, nullptr, 1, g.M, g.M, err, nullptr, wgrad_deep_rows_mx()};
            QtSrc sdy{3, dyb, nullptr, g.H, nullptr, nullptr, 0, t0, g.k, g.S};
            QtSrc sxx{3, xb, nullptr, g.H, nullptr, nullptr, 0, t0, g.k, g.S};
            if (launch_mx_quant_group_t(pd, sdy, g.H, twdy, twdys, st) ||
                launch_mx_quant_group_t(pd, sxx, g.H, tx, txs, st))
                return MOE_ERR_HIP;
            if (!wgrads(pd, (uint8_t*)(ws + L.tr_sh), (uint8_t*)(ws + L.tr_shs), (uint8_t*)(ws + L.tr_sdgu),
                        (uint8_t*)(ws + L.tr_sdgus), mode, nullptr, m, (uint16_t*)gr->d_s_down, P.wacc(L.wacc_sd),
                        (uint16_t*)gr->d_s_gate, P.wacc(L.wacc_sg), (uint16_t*)gr->d_s_up,
                        P.wacc(L.wacc_su)))
                return MOE_ERR_HIP;
        }
    }
    return MOE_OK;
}

// ---------------------------------------------------------------- no-allocation schedule
// moe_schedule_noalloc keeps the schedule's scratch (the error word, the
// per-block histograms and bases) in this fixed device array instead of a
// caller workspace.  Host code never passes the array's name to a kernel (in
// host code it is only a stand-in); the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratch = 16u << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratch];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// bytes of scratch the schedule of `g` needs: error word, histograms, bases
size_t schedule_scratch_bytes(const Geom& g) {
    const size_t hist = schedule_hist_ints(g.T, g.E, g.k, g.M, g.mb) * 4;
    return 256 + 2 * align_up(hist, 256);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
        case MOE_ERR_CAPACITY: return "ring capacity below one macrobatch";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_HIP: return "HIP error";
        case MOE_ERR_UNSUPPORTED: return "not implemented in this build";
    }
    return "unknown status";
}

moe_status moe_validate_config(const moe_config* cfg) {
    Geom g;
    return make_geom(cfg, g);
}

moe_status moe_ring_rows(const moe_config* cfg, int64_t* rows) {
    Geom g;
    moe_status s = make_geom(cfg, g);
    if (s != MOE_OK) return s;
    if (!rows) return MOE_ERR_INVALID_ARG;
    *rows = g.ring_rows;
    return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
    Geom g;
    moe_status s = make_geom(cfg, g);
    if (s != MOE_OK) return s;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = make_layout(g).total;
    return MOE_OK;
}

int moe_device_supported(void) { return device_ok() ? 1 : 0; }

moe_status moe_workspace_region(const moe_config* cfg, const char* name, size_t* offset,
                                size_t* bytes) {
    Geom g;
    moe_status s = make_geom(cfg, g);
    if (s != MOE_OK) return s;
    if (!name || !offset || !bytes || !g.mx) return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(g);
    const size_t th = (size_t)g.T * g.H;
    const size_t tk = (size_t)g.H * (size_t)L.kcap;
    struct { const char* n; size_t off, len; } regions[] = {
        {"x_codes", L.xq, th}, {"x_scales", L.xs, th / 32},
        {"dy_codes", L.dyq, th}, {"dy_scales", L.dys, th / 32},
        // the dW_gate / dW_up operand x of the last macrobatch the backward
        // processed, quantised in 32-row blocks of each expert's group and
        // stored group-major and transposed, with the prefix of the groups'
        // 32-row block counts that places them
        {"wgrad_x_codes", L.tr_x, tk}, {"wgrad_x_scales", L.tr_xs, tk / 32},
        {"wgrad_block_offsets", L.blk_off, (size_t)(g.E + 1) * 4},
    };
    for (const auto& r : regions) {
        if (std::strcmp(r.n, name) == 0) {
            *offset = r.off;
            *bytes = r.len;
            return MOE_OK;
        }
    }
    return MOE_ERR_INVALID_ARG;
}

moe_status moe_schedule(const moe_config* cfg, const float* logits, const moe_sched* sched,
                        void* workspace, size_t workspace_bytes, void* stream) {
    Geom g;
    Layout L;
    moe_status s = common_checks(cfg, g, L, workspace, workspace_bytes);
    if (s != MOE_OK) return s;
    if (!logits || !aligned(logits, 4) || !sched_ok(sched)) return MOE_ERR_INVALID_ARG;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    int32_t* err = (int32_t*)(ws + L.err);
    k_clear_word<<<1, 1, 0, st>>>(err);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    if (launch_topk_route(logits, g.T, g.E, g.k, sched->topk_idx, sched->topk_w, st)) return MOE_ERR_HIP;
    if (launch_schedule(sched->topk_idx, g.T, g.E, g.k, g.M, g.mb, (int32_t*)(ws + L.hist),
                        (int32_t*)(ws + L.base), sched->counts, sched->offsets, sched->mini_counts,
                        sched->row_of_slot, sched->slot_of_row, err, st))
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_schedule_noalloc(const moe_config* cfg, const float* logits, const moe_sched* sched,
                                void* stream) {
    Geom g;
    moe_status s = make_geom(cfg, g);
    if (s != MOE_OK) return s;
    if (!logits || !aligned(logits, 4) || !sched_ok(sched)) return MOE_ERR_INVALID_ARG;
    if (schedule_scratch_bytes(g) > kNoAllocScratch) return MOE_ERR_WORKSPACE;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    char* base = (char*)scratch_ptr();
    if (!base) return MOE_ERR_HIP;
    hipStream_t st = (hipStream_t)stream;
    const size_t hist = align_up(schedule_hist_ints(g.T, g.E, g.k, g.M, g.mb) * 4, 256);
    int32_t* err = (int32_t*)base;
    int32_t* hh = (int32_t*)(base + 256);
    int32_t* bb = (int32_t*)(base + 256 + hist);
    // the histograms and bases are written in full before they are read; the
    // error word is cleared by a kernel (no memset node if the call is captured)
    k_clear_word<<<1, 1, 0, st>>>(err);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    if (launch_topk_route(logits, g.T, g.E, g.k, sched->topk_idx, sched->topk_w, st)) return MOE_ERR_HIP;
    if (launch_schedule(sched->topk_idx, g.T, g.E, g.k, g.M, g.mb, hh, bb, sched->counts,
                        sched->offsets, sched->mini_counts, sched->row_of_slot, sched->slot_of_row,
                        err, st))
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_router_forward(const moe_config* cfg, const void* x, const void* w_router, float* logits,
                              void* stream) {
    Geom g;
    moe_status s = make_geom(cfg, g);
    if (s != MOE_OK) return s;
    if (!bf16_ok(x) || !bf16_ok(w_router) || !logits || !aligned(logits, 4)) return MOE_ERR_INVALID_ARG;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    if (launch_router_logits(x, w_router, logits, g.T, g.H, g.E, (hipStream_t)stream)) return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_router_backward(const moe_config* cfg, const void* x, const void* w_router,
                               const float* d_logits, void* dx, void* dw_router, void* workspace,
                               size_t workspace_bytes, void* stream) {
    Geom g;
    Layout L;
    moe_status s = common_checks(cfg, g, L, workspace, workspace_bytes);
    if (s != MOE_OK) return s;
    if (!bf16_ok(x) || !bf16_ok(w_router) || !bf16_ok(dx) || !bf16_ok(dw_router) || !d_logits ||
        !aligned(d_logits, 4))
        return MOE_ERR_INVALID_ARG;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    if (launch_router_backward(x, w_router, d_logits, dx, dw_router, (char*)workspace + L.dl16, g.T, g.H,
                               g.E, (hipStream_t)stream))
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, const moe_sched* sched, const void* x,
                       const moe_weights* w, void* y, const moe_saved* saved, void* workspace,
                       size_t workspace_bytes, void* stream) {
    Geom g;
    Layout L;
    moe_status s = common_checks(cfg, g, L, workspace, workspace_bytes);
    if (s != MOE_OK) return s;
    if (!sched_ok(sched) || !bf16_ok(x) || !bf16_ok(y) || !w) return MOE_ERR_INVALID_ARG;
    if (!bf16_ok(w->w_gate) || !bf16_ok(w->w_up) || !bf16_ok(w->w_down)) return MOE_ERR_INVALID_ARG;
    if (!saved_ok(g, saved)) return MOE_ERR_INVALID_ARG;
    if (g.shared && (!bf16_ok(w->s_gate) || !bf16_ok(w->s_up) || !bf16_ok(w->s_down)))
        return MOE_ERR_INVALID_ARG;
    const moe_weights_mx* wq = w->mx;
    if (g.w4) {
        const moe_weights_mx4* q = w->mx4;
        if (!q) return MOE_ERR_INVALID_ARG;
        const void* need[] = {q->w_gate_q, q->w_up_q, q->w_down_q, q->w_gate_s, q->w_up_s, q->w_down_s};
        for (const void* p : need)
            if (!p || !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
        if (g.shared) {
            const void* needs[] = {q->s_gate_q, q->s_up_q, q->s_down_q, q->s_gate_s, q->s_up_s, q->s_down_s};
            for (const void* p : needs)
                if (!p || !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
        }
    } else if (g.mx) {
        if (!wq || !bf16_ok(wq->w_gate_q) || !wq->w_gate_s || !bf16_ok(wq->w_up_q) || !wq->w_up_s ||
            !bf16_ok(wq->w_down_q) || !wq->w_down_s)
            return MOE_ERR_INVALID_ARG;
        if (!aligned(wq->w_gate_s, 4) || !aligned(wq->w_up_s, 4) || !aligned(wq->w_down_s, 4))
            return MOE_ERR_INVALID_ARG;
        if (g.shared && (!bf16_ok(wq->s_gate_q) || !bf16_ok(wq->s_up_q) || !bf16_ok(wq->s_down_q) ||
                         !wq->s_gate_s || !wq->s_up_s || !wq->s_down_s || !aligned(wq->s_gate_s, 4) ||
                         !aligned(wq->s_up_s, 4) || !aligned(wq->s_down_s, 4)))
            return MOE_ERR_INVALID_ARG;
    }
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    Ptrs P{(char*)workspace, &L};
    int32_t* err = P.err();
    const uint16_t* xb = (const uint16_t*)x;
    if (g.mx) return forward_mx(g, L, P, sched, x, w, y, saved, st);
    const int tm = gemm_row_tile(g.Sm, g.E);            // row tile of the M-grouped GEMMs
    for (int m = 0; m < g.n_macro; ++m) {
        char* half = P.half(m, g.halves);
        uint16_t* hbuf = (uint16_t*)(half + L.f_h);
        uint16_t* obuf = (uint16_t*)(half + L.f_o);
        const int grow0 = m * g.Sm, t0 = m * g.M;
        const int32_t* off = sched->offsets + (size_t)m * (g.E + 1);
        int32_t* toff = (int32_t*)((char*)workspace + L.tile_off) + (size_t)m * (g.E + 1);
        // the gate/up and down GEMMs take groups of at least kBigRows rows in
        // 256 x 256 tiles when groups are large on average
        const bool big = tm == 128 && g.H % kBig == 0 && g.I % (kBig / 2) == 0;
        int32_t* tsmall = (int32_t*)((char*)workspace + L.tile_split) + (size_t)m * 2 * (g.E + 1);
        int32_t* tbig = tsmall + (g.E + 1);
        if (big ? launch_tile_prefix_split(off, g.E, g.Sm, tm, toff, kBigRows, kBig, tsmall, tbig, err, st)
                : launch_tile_prefix(off, g.E, g.Sm, tm, toff, err, st))
            return MOE_ERR_HIP;
        // dispatch fused into the gate/up GEMM: its operand loads gather each
        // routed row from the row of its token
        GroupRows grp{off, toff, g.E, g.Sm, 0, err, nullptr, 0, tm};
        if (big) {
            grp.tile_off = tsmall;
            grp.tile_big = tbig;
        }
        const GU keep = gu_routed(g, L, P, saved, m, true);
        GemmGateUpArgs a1{grp, xb, 1, 0, sched->slot_of_row, grow0, g.k, g.S,
                          (const uint16_t*)w->w_gate, (const uint16_t*)w->w_up, g.H, g.I,
                          (uint16_t*)keep.g, (uint16_t*)keep.u, keep.row0, hbuf};
        if (launch_gemm_gate_up(a1, st)) return MOE_ERR_HIP;
        GemmDownArgs a2{grp, hbuf, (const uint16_t*)w->w_down, g.H, g.I, top1_direct(g) ? (uint16_t*)y : obuf,
                        {sched->topk_w, sched->slot_of_row, grow0, g.S}, token_rows(g, sched, grow0)};
        if (launch_gemm_down(a2, st)) return MOE_ERR_HIP;
        const uint16_t* sh_o = nullptr;
        if (g.shared) {
            uint16_t* sh_h = (uint16_t*)(P.sh() + L.s_h);
            uint16_t* so = (uint16_t*)(P.sh() + L.s_o);
            GroupRows dense{nullptr, nullptr, 1, g.M, g.M, err, nullptr, 0, gemm_row_tile(g.M, 1)};
            const GU skeep = gu_shared(g, L, P, saved, m, true);
            GemmGateUpArgs s1{dense, xb, 0, t0, nullptr, 0, g.k, g.S,
                              (const uint16_t*)w->s_gate, (const uint16_t*)w->s_up, g.H, g.I,
                              (uint16_t*)skeep.g, (uint16_t*)skeep.u, skeep.row0, sh_h};
            if (launch_gemm_gate_up(s1, st)) return MOE_ERR_HIP;
            GemmDownArgs s2{dense, sh_h, (const uint16_t*)w->s_down, g.H, g.I, so, {nullptr, nullptr, 0, 0}};
            if (launch_gemm_down(s2, st)) return MOE_ERR_HIP;
            sh_o = so;
        }
        // the router-weighted reduction: y_t = [shared] + sum_j (w o)_(t,j), in
        // that fixed order (the rows already carry their weights)
        if (!top1_direct(g) && launch_combine(obuf, g.H, sched->row_of_slot, nullptr, t0, t0 + g.M, g.k, grow0,
                                              g.Sm, sh_o, t0, y, err, st))
            return MOE_ERR_HIP;
    }
    return MOE_OK;
}

moe_status moe_backward(const moe_config* cfg, const moe_sched* sched, const moe_saved* saved,
                        const void* x, const moe_weights* w, const void* dy, void* dx,
                        const moe_grads* gr, float* dw, float* d_logits, void* workspace,
                        size_t workspace_bytes, void* stream) {
    Geom g;
    Layout L;
    moe_status s = common_checks(cfg, g, L, workspace, workspace_bytes);
    if (s != MOE_OK) return s;
    if (g.w4) return MOE_ERR_UNSUPPORTED;       // the MXFP4-weight variant is forward-only
    if (!sched_ok(sched) || !saved_ok(g, saved) || !w || !gr || !bf16_ok(x) || !bf16_ok(dy) ||
        !bf16_ok(dx))
        return MOE_ERR_INVALID_ARG;
    if (!bf16_ok(w->w_gate) || !bf16_ok(w->w_up) || !bf16_ok(w->w_down)) return MOE_ERR_INVALID_ARG;
    if (!bf16_ok(gr->d_w_gate) || !bf16_ok(gr->d_w_up) || !bf16_ok(gr->d_w_down))
        return MOE_ERR_INVALID_ARG;
    if (!dw || !aligned(dw, 4) || (d_logits && !aligned(d_logits, 4))) return MOE_ERR_INVALID_ARG;
    if (g.shared && (!bf16_ok(w->s_gate) || !bf16_ok(w->s_up) || !bf16_ok(w->s_down) ||
                     !bf16_ok(gr->d_s_gate) || !bf16_ok(gr->d_s_up) || !bf16_ok(gr->d_s_down)))
        return MOE_ERR_INVALID_ARG;
    if (g.mx) {
        const moe_weights_mx* wq = w->mx;
        if (!wq || !bf16_ok(wq->w_gate_tq) || !bf16_ok(wq->w_up_tq) || !bf16_ok(wq->w_down_tq) ||
            !wq->w_gate_ts || !wq->w_up_ts || !wq->w_down_ts || !aligned(wq->w_gate_ts, 4) ||
            !aligned(wq->w_up_ts, 4) || !aligned(wq->w_down_ts, 4))
            return MOE_ERR_INVALID_ARG;
        if (g.shared && (!bf16_ok(wq->s_gate_tq) || !bf16_ok(wq->s_up_tq) || !bf16_ok(wq->s_down_tq) ||
                         !wq->s_gate_ts || !wq->s_up_ts || !wq->s_down_ts ||
                         !aligned(wq->s_gate_ts, 4) || !aligned(wq->s_up_ts, 4) ||
                         !aligned(wq->s_down_ts, 4)))
            return MOE_ERR_INVALID_ARG;
    }
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    Ptrs P{(char*)workspace, &L};
    // the accumulator slots of the experts whose gradients span macrobatches
    if (g.n_macro > 1 &&
        launch_acc_slots(sched->counts, g.n_macro, g.E, g.acc_cap, P.acc_slot(), P.err(), st))
        return MOE_ERR_HIP;
    if (g.mx) return backward_mx(g, L, P, sched, saved, x, w, dy, dx, gr, dw, d_logits, st);
    int32_t* err = P.err();
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* dyb = (const uint16_t*)dy;
    const int tm = gemm_row_tile(g.Sm, g.E);            // row tile of the M-grouped GEMMs
    // weight gradients of groups of at least wgrad_big_rows() rows in 256 x 256
    // tiles; rows past a group's end are read from a zero row
    const bool wbig = g.H % kBig == 0 && g.I % kBig == 0;
    const uint16_t* zero = (const uint16_t*)((char*)workspace + L.zero);
    if (wbig) {
        k_clear_words<<<1, 256, 0, st>>>((int32_t*)((char*)workspace + L.zero));
        if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    }
    for (int m = g.n_macro - 1; m >= 0; --m) {
        // weight-gradient accumulation across the reverse walk
        int mode = 0;
        if (g.n_macro > 1) mode = (m == g.n_macro - 1) ? 1 : (m == 0 ? 3 : 2);
        char* half = P.half(m, g.halves);
        uint16_t* dgu = (uint16_t*)(half + L.b_dgu);
        uint16_t* hw = (uint16_t*)(half + L.b_hw);
        uint16_t* dxd = (uint16_t*)(half + L.b_dx);
        float* part = (float*)(half + L.b_part);
        const int grow0 = m * g.Sm, t0 = m * g.M;
        const int32_t* off = sched->offsets + (size_t)m * (g.E + 1);
        int32_t* toff = (int32_t*)((char*)workspace + L.tile_off) + (size_t)m * (g.E + 1);
        // the M-grouped GEMMs take groups of at least kBigRows rows in 256 x 256
        // tiles when groups are large on average
        const bool big = tm == 128 && g.H % kBig == 0 && g.I % kBig == 0;
        int32_t* tsmall = (int32_t*)((char*)workspace + L.tile_split) + (size_t)m * 2 * (g.E + 1);
        int32_t* tbig = tsmall + (g.E + 1);
        if (big ? launch_tile_prefix_split(off, g.E, g.Sm, tm, toff, kBigRows, kBig, tsmall, tbig, err, st)
                : launch_tile_prefix(off, g.E, g.Sm, tm, toff, err, st))
            return MOE_ERR_HIP;
        GroupRows grp{off, toff, g.E, g.Sm, 0, err, nullptr, 0, tm};
        GroupRows grp_split = grp;
        if (big) {
            grp_split.tile_off = tsmall;
            grp_split.tile_big = tbig;
        }
        const GU gu = gu_routed(g, L, P, saved, m, false);
        if (g.recompute && m != g.n_macro - 1) {
            // recompute this macrobatch's g, u (h goes to the hw rows, which
            // the dgrad below overwrites)
            GemmGateUpArgs r1{grp_split, xb, 1, 0, sched->slot_of_row, grow0, g.k, g.S,
                              (const uint16_t*)w->w_gate, (const uint16_t*)w->w_up, g.H, g.I,
                              (uint16_t*)gu.g, (uint16_t*)gu.u, 0, hw};
            if (launch_gemm_gate_up(r1, st)) return MOE_ERR_HIP;
        }
        // reverse-combine (dy gathered on load) + down dgrad + SwiGLU backward + dw partials
        // the down dgrad has few column tiles (I / 256): its 256 x 256 form
        // needs a macrobatch of at least ~two rounds of such tiles over the chip
        // (the expert-parallel share's 320 tiles ran 0.33 -> 0.37 ms in it)
        const bool big_dd = big && (int64_t)(g.Sm / kBig) * (g.I / kBig) >= kBigDgradTiles;
        GemmDownDgradArgs b1{big_dd ? grp_split : grp, dyb, 1, 0, sched->slot_of_row, grow0, g.k, g.S, sched->topk_w,
                             (const uint16_t*)w->w_down, g.H, g.I, (const uint16_t*)gu.g,
                             (const uint16_t*)gu.u, gu.row0, dgu, hw, part, g.P};
        if (launch_gemm_down_dgrad(b1, st)) return MOE_ERR_HIP;
        GemmGuDgradArgs b2{grp_split, dgu, (const uint16_t*)w->w_gate, (const uint16_t*)w->w_up, g.H, g.I,
                           top1_direct(g) ? (uint16_t*)dx : dxd, token_rows(g, sched, grow0)};
        if (launch_gemm_gu_dgrad(b2, st)) return MOE_ERR_HIP;
        // the shared expert's input gradient, then reverse-dispatch and the
        // softmax backward while dXd is still in cache; the weight gradients
        // (the large writes) come last
        const uint16_t* sh_dx = nullptr;
        GroupRows dense{nullptr, nullptr, 1, g.M, g.M, err, nullptr, wgrad_deep_rows(), gemm_row_tile(g.M, 1)};
        uint16_t* sdgu = g.shared ? (uint16_t*)(P.sh() + L.s_dgu) : nullptr;
        uint16_t* shw = g.shared ? (uint16_t*)(P.sh() + L.s_hw) : nullptr;
        if (g.shared) {
            uint16_t* sdx = (uint16_t*)(P.sh() + L.s_dx);
            const GU sgu = gu_shared(g, L, P, saved, m, false);
            if (g.recompute && m != g.n_macro - 1) {
                GemmGateUpArgs r2{dense, xb, 0, t0, nullptr, 0, g.k, g.S,
                                  (const uint16_t*)w->s_gate, (const uint16_t*)w->s_up, g.H, g.I,
                                  (uint16_t*)sgu.g, (uint16_t*)sgu.u, 0, shw};
                if (launch_gemm_gate_up(r2, st)) return MOE_ERR_HIP;
            }
            GemmDownDgradArgs c1{dense, dyb, 0, t0, nullptr, 0, g.k, g.S, nullptr,
                                 (const uint16_t*)w->s_down, g.H, g.I, (const uint16_t*)sgu.g,
                                 (const uint16_t*)sgu.u, sgu.row0, sdgu, shw, nullptr, g.P};
            if (launch_gemm_down_dgrad(c1, st)) return MOE_ERR_HIP;
            GemmGuDgradArgs c2{dense, sdgu, (const uint16_t*)w->s_gate, (const uint16_t*)w->s_up,
                               g.H, g.I, sdx};
            if (launch_gemm_gu_dgrad(c2, st)) return MOE_ERR_HIP;
            sh_dx = sdx;
        }
        // reverse-dispatch: dx_t = [shared] + sum_j dXd[row(t, j)]
        if (!top1_direct(g) && launch_rd_reduce(dxd, g.H, sched->row_of_slot, t0, t0 + g.M, g.k, grow0, g.Sm,
                                                sh_dx, t0, dx, err, st))
            return MOE_ERR_HIP;
        if (launch_softmax_bwd(part, g.P, sched->row_of_slot, sched->topk_idx, sched->topk_w, t0,
                               t0 + g.M, g.k, g.E, grow0, g.Sm, dw, d_logits, err, st))
            return MOE_ERR_HIP;
        int32_t* deep = (int32_t*)((char*)workspace + L.deep);
        int32_t* deep_big = (int32_t*)((char*)workspace + L.deep_big);
        if (wbig ? launch_deep_list_split(off, g.E, g.Sm, wgrad_deep_rows(), deep, wgrad_big_rows(), deep_big, st)
                 : launch_deep_list(off, g.E, g.Sm, wgrad_deep_rows(), deep, st))
            return MOE_ERR_HIP;
        GroupRows kgrp{off, nullptr, g.E, g.Sm, 0, err, deep, wgrad_deep_rows()};
        // the dense group takes the 256 x 256 form only where its tiles fill
        // the persistent grid (a 16 384-row shared expert's dW_gate | dW_up has
        // 128 such tiles for 256 blocks, its dW_down 64; the 128 x 128 deep
        // kernel then keeps the chip busy)
        GroupRows dense_d = dense, dense_gu = dense;
        if (wbig) {
            kgrp.deep_big = deep_big;
            kgrp.big_thr = wgrad_big_rows();
            if ((g.H / kBig) * (g.I / kBig) >= wgrad_big_grid()) dense_d.big_thr = wgrad_big_rows();
            if ((2 * g.I / kBig) * (g.H / kBig) >= wgrad_big_grid()) dense_gu.big_thr = wgrad_big_rows();
        }
        const int32_t* cnts = g.n_macro > 1 ? sched->counts : nullptr;   // per-expert modes
        const int32_t* sl = g.n_macro > 1 ? P.acc_slot() : nullptr;
        WgradDownArgs b3{kgrp, dyb, 1, 0, sched->slot_of_row, grow0, g.k, g.S, hw, g.H, g.I,
                         {(uint16_t*)gr->d_w_down, P.wacc(L.wacc_d), mode, cnts, m, g.n_macro, g.E, sl}, zero};
        if (launch_wgrad_down(b3, st)) return MOE_ERR_HIP;
        WgradGateUpArgs b4{kgrp, dgu, xb, 1, 0, sched->slot_of_row, grow0, g.k, g.S, g.H, g.I,
                           {(uint16_t*)gr->d_w_gate, P.wacc(L.wacc_g), mode, cnts, m, g.n_macro, g.E, sl},
                           {(uint16_t*)gr->d_w_up, P.wacc(L.wacc_u), mode, cnts, m, g.n_macro, g.E, sl}, zero};
        if (launch_wgrad_gate_up(b4, st)) return MOE_ERR_HIP;
        if (g.shared) {
            WgradDownArgs c3{dense_d, dyb, 0, t0, nullptr, 0, g.k, g.S, shw, g.H, g.I,
                             {(uint16_t*)gr->d_s_down, P.wacc(L.wacc_sd), mode}, zero};
            if (launch_wgrad_down(c3, st)) return MOE_ERR_HIP;
            WgradGateUpArgs c4{dense_gu, sdgu, xb, 0, t0, nullptr, 0, g.k, g.S, g.H, g.I,
                               {(uint16_t*)gr->d_s_gate, P.wacc(L.wacc_sg), mode},
                               {(uint16_t*)gr->d_s_up, P.wacc(L.wacc_su), mode}, zero};
            if (launch_wgrad_gate_up(c4, st)) return MOE_ERR_HIP;
        }
    }
    return MOE_OK;
}

moe_status moe_quantize_weights_mxfp8(const moe_config* cfg, const moe_weights* w,
                                      const moe_weights_mx* o, void* stream) {
    Geom g;
    moe_status s = make_geom(cfg, g);
    if (s != MOE_OK) return s;
    if (!w || !o || !bf16_ok(w->w_gate) || !bf16_ok(w->w_up) || !bf16_ok(w->w_down))
        return MOE_ERR_INVALID_ARG;
    const void* need[] = {o->w_gate_q, o->w_gate_s, o->w_up_q, o->w_up_s, o->w_down_q, o->w_down_s,
                          o->w_gate_tq, o->w_gate_ts, o->w_up_tq, o->w_up_ts, o->w_down_tq,
                          o->w_down_ts};
    for (const void* p : need)
        if (!p || !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    if (g.shared) {
        if (!bf16_ok(w->s_gate) || !bf16_ok(w->s_up) || !bf16_ok(w->s_down)) return MOE_ERR_INVALID_ARG;
        const void* needs[] = {o->s_gate_q, o->s_gate_s, o->s_up_q, o->s_up_s, o->s_down_q,
                               o->s_down_s, o->s_gate_tq, o->s_gate_ts, o->s_up_tq, o->s_up_ts,
                               o->s_down_tq, o->s_down_ts};
        for (const void* p : needs)
            if (!p || !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    }
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    const int E = g.E, H = g.H, I = g.I;
    auto one = [&](const void* wg, const void* wu, const void* wd, int n, const void* gq, const void* gs,
                   const void* uq, const void* us, const void* dq, const void* ds, const void* gtq,
                   const void* gts, const void* utq, const void* uts, const void* dtq,
                   const void* dts) -> bool {
        // forward: rows along their reduction axis
        // (scales K-step-major per matrix, so a GEMM's K step of scales is contiguous)
        if (launch_mx_quant_rows(wg, (int64_t)n * I, H, (void*)gq, (void*)gs, st, I)) return false;
        if (launch_mx_quant_rows(wu, (int64_t)n * I, H, (void*)uq, (void*)us, st, I)) return false;
        if (launch_mx_quant_rows(wd, (int64_t)n * H, I, (void*)dq, (void*)ds, st, H)) return false;
        // backward: transposed copies, blocks along the other axis
        if (launch_mx_quant_cols(wg, n, I, H, (void*)gtq, (void*)gts, st)) return false;
        if (launch_mx_quant_cols(wu, n, I, H, (void*)utq, (void*)uts, st)) return false;
        if (launch_mx_quant_cols(wd, n, H, I, (void*)dtq, (void*)dts, st)) return false;
        return true;
    };
    if (!one(w->w_gate, w->w_up, w->w_down, E, o->w_gate_q, o->w_gate_s, o->w_up_q, o->w_up_s,
             o->w_down_q, o->w_down_s, o->w_gate_tq, o->w_gate_ts, o->w_up_tq, o->w_up_ts,
             o->w_down_tq, o->w_down_ts))
        return MOE_ERR_HIP;
    if (g.shared &&
        !one(w->s_gate, w->s_up, w->s_down, 1, o->s_gate_q, o->s_gate_s, o->s_up_q, o->s_up_s,
             o->s_down_q, o->s_down_s, o->s_gate_tq, o->s_gate_ts, o->s_up_tq, o->s_up_ts,
             o->s_down_tq, o->s_down_ts))
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_quantize_weights_mxfp4(const moe_config* cfg, const moe_weights* w,
                                      const moe_weights_mx4* o, void* stream) {
    Geom g;
    moe_status s = make_geom(cfg, g);
    if (s != MOE_OK) return s;
    if (!w || !o || !bf16_ok(w->w_gate) || !bf16_ok(w->w_up) || !bf16_ok(w->w_down))
        return MOE_ERR_INVALID_ARG;
    const void* need[] = {o->w_gate_q, o->w_gate_s, o->w_up_q, o->w_up_s, o->w_down_q, o->w_down_s};
    for (const void* p : need)
        if (!p || !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    if (g.shared) {
        if (!bf16_ok(w->s_gate) || !bf16_ok(w->s_up) || !bf16_ok(w->s_down)) return MOE_ERR_INVALID_ARG;
        const void* needs[] = {o->s_gate_q, o->s_gate_s, o->s_up_q, o->s_up_s, o->s_down_q, o->s_down_s};
        for (const void* p : needs)
            if (!p || !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    }
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    const int E = g.E, H = g.H, I = g.I;
    auto one = [&](const void* wg, const void* wu, const void* wd, int n, const void* gq, const void* gs,
                   const void* uq, const void* us, const void* dq, const void* ds) -> bool {
        return launch_mx4_quant_rows(wg, (int64_t)n * I, H, I, (void*)gq, (void*)gs, st) == 0 &&
               launch_mx4_quant_rows(wu, (int64_t)n * I, H, I, (void*)uq, (void*)us, st) == 0 &&
               launch_mx4_quant_rows(wd, (int64_t)n * H, I, H, (void*)dq, (void*)ds, st) == 0;
    };
    if (!one(w->w_gate, w->w_up, w->w_down, E, o->w_gate_q, o->w_gate_s, o->w_up_q, o->w_up_s,
             o->w_down_q, o->w_down_s))
        return MOE_ERR_HIP;
    if (g.shared && !one(w->s_gate, w->s_up, w->s_down, 1, o->s_gate_q, o->s_gate_s, o->s_up_q,
                         o->s_up_s, o->s_down_q, o->s_down_s))
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_check_device_error(void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t* flags) {
    if (!workspace || !flags || workspace_bytes < 256 || !aligned(workspace, 256))
        return MOE_ERR_INVALID_ARG;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    int32_t v = 0;
    if (hipMemcpyAsync(&v, workspace, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_HIP;
    k_clear_word<<<1, 1, 0, st>>>((int32_t*)workspace);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    *flags = v;
    return MOE_OK;
}

}  // extern "C"
