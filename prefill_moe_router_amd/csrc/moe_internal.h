// moe_internal.h -- host-side plumbing shared by the library's translation
// units: workspace layout and the kernel launchers each .hip file exports.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_router.h"

namespace moe {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// rows of one m-tile of the grouped GEMM (the grouping emits m-tile offsets for it)
#ifndef MOE_TILE_M
#define MOE_TILE_M 128
#endif
constexpr int kGroupedTileM = MOE_TILE_M;
// the smaller m-tile of the bf16 large-tile GEMMs for medium batches (grouped_tile_rows)
constexpr int kWideSmallTileM = 64;

// largest token count the fused single-kernel decode path takes
constexpr int kFusedMaxTokens = 8;
// largest grid of the fused decode kernel (one work-group per CU)
constexpr int kFusedMaxGroups = 1024;

inline size_t act_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

// expert-weight elements per 16-byte chunk of a row (fp32 4, bf16 8, MXINT8 16, 4-bit 32)
inline int weight_chunk_elems(int dt) {
    return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 8 : dt == MOE_MXINT8 ? 16 : 32;
}

// upper bound of the number of m-tiles of P pairs over E experts, for either tile height:
// sum over experts of ceil(count / tile) <= P / tile + (number of nonempty experts)
inline size_t grouped_tile_bound(size_t P, size_t E) { return P / kWideSmallTileM + (P < E ? P : E); }

// Byte offsets of the regions of one workspace.  Region 0 holds the control
// words: [0] the sticky device error word; [8] the fused decode kernel's 64-bit
// call counter, which only grows (the tag of the words that kernel publishes --
// logits and barrier flags -- is derived from it, so it must never be reset on
// its own).
// tokens per work-group of the MFMA router (and per count row of its grouping output)
constexpr int kRouterRows = 32;

struct WsLayout {
    size_t ctrl, tagged, flags, logits, ids, wts, offsets, sorted, slot_pos, active, mtile, tiles, gcounts, h, o, total;
};

inline WsLayout ws_layout(const moe_shape &s) {
    const size_t T = (size_t)s.num_tokens, E = (size_t)s.num_experts, K = (size_t)s.top_k;
    const size_t H = (size_t)s.hidden, I = (size_t)s.intermediate, P = T * K;
    WsLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    L.ctrl = take(256);
    L.tagged = take((size_t)kFusedMaxTokens * E * 8);   // fused decode: logit | call tag words
    L.flags = take((size_t)kFusedMaxGroups * 8);        // fused decode: per-work-group barrier tags
    L.logits = take(T * E * 4);
    L.ids = take(P * 4);
    L.wts = take(P * 4);
    L.offsets = take((E + 1) * 4);
    L.sorted = take(P * 4);
    L.slot_pos = take(P * 4);
    L.active = take((E + 1) * 4);
    L.mtile = take((E + 1) * 4);
    L.tiles = take(grouped_tile_bound(P, E) * 16);
    L.gcounts = take(std::max<size_t>(P > 0 ? (P + 4095) / 4096 : 1, (T + kRouterRows - 1) / kRouterRows) * E * 4);
    L.h = take(P * I * act_bytes(s.act_dtype));
    L.o = take(P * H * 4);
    L.total = off;
    return L;
}

// ---- launchers (each returns the launch's hipError_t) ----------------------------

// s[t,e] = bias[e] + x[t,:].w_router[e,:]  -> logits [T][E] fp32
hipError_t launch_router_logits(const moe_shape &s, const void *x, const void *wr, const float *bias,
                                float *logits, hipStream_t st);
// router GEMM + top-k in one kernel (bf16, E % 32 == 0, E <= 128, H % 512 == 0): ids / w as
// launch_topk; with slot_rank and counts (both or neither) also each slot's rank inside its
// block of kRouterRows tokens and counts[block][E] for launch_group_from_router
bool router_topk_mfma_supported(const moe_shape &s);
hipError_t launch_router_topk_mfma(const moe_shape &s, const void *x, const void *wr, const float *bias,
                                   int32_t *ids, float *w, int32_t *slot_rank, int32_t *counts, hipStream_t st,
                                   hipEvent_t ev0, hipEvent_t ev1);
// grouping from the router's per-block counts and ranks: same outputs as launch_group2
hipError_t launch_group_from_router(const moe_shape &s, const int32_t *ids, int32_t *counts, int32_t *offsets,
                                    int32_t *sorted, int32_t *slot_pos, int32_t *active, int32_t *mtile_off,
                                    int32_t *tiles, int mtile_rows, hipStream_t st);
// top-k + softmax (+ renorm) over logits rows -> ids [T][k] ascending, w [T][k]
hipError_t launch_topk(const moe_shape &s, const float *logits, int32_t *ids, float *w, hipStream_t st);
// multi-block stable grouping (chunks of 4096 slots): counts [chunks][E] scratch;
// mtile_off (optional) receives the m-tile offsets for tiles of mtile_rows rows, and
// tiles (with mtile_off) one {first row, end row of the expert, expert, 0} int4 per m-tile
int group_chunks(int P);
hipError_t launch_group2(const moe_shape &s, const int32_t *ids, int32_t *offsets, int32_t *sorted, int32_t *slot_pos,
                         int32_t *active, int32_t *counts, int32_t *mtile_off, int32_t *tiles, int mtile_rows,
                         int32_t *err, hipStream_t st);
// active = [count, nonempty experts ascending] from existing offsets
hipError_t launch_active(const moe_shape &s, const int32_t *offsets, int32_t *active, hipStream_t st);
// the streaming expert FFN (decode_ffn.hip) covers the shape
bool stream_ffn_supported(const moe_shape &s);
// h[p][i] = (wts ? wts[slot] : 1) * silu(Wg[e,i].x_t) * (Wu[e,i].x_t), act dtype, sorted order
hipError_t launch_decode_gateup(const moe_shape &s, const void *x, const moe_expert_weights &w,
                                const int32_t *offsets, const int32_t *sorted, const int32_t *active,
                                const float *wts, void *h, hipStream_t st);
// o[p][n] = Wd[e,n,:].h[p,:]  fp32, sorted order
hipError_t launch_decode_down(const moe_shape &s, const moe_expert_weights &w, const int32_t *offsets,
                              const int32_t *active, const void *h, float *o, hipStream_t st);
// y[t][n] = sum_j w[t,j] o[slot_pos[t*k+j]][n]
hipError_t launch_combine(const moe_shape &s, const float *o, const float *w, const int32_t *slot_pos,
                          void *y, hipStream_t st);

// whole layer for T <= 8 in one persistent launch (see decode_fused.hip)
bool decode_fused_supported(const moe_shape &s);
// one work-group of the fused kernel for `s` fits a compute unit of the current device
// (true when no device can be queried: nothing is launched then)
bool decode_fused_coresident(const moe_shape &s);
hipError_t launch_decode_fused(const moe_shape &s, const void *x, const void *wr, const float *bias,
                               const moe_expert_weights &w, void *y, int32_t *ids_out, float *w_out, void *ws,
                               hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);

// MFMA grouped GEMM family (see grouped_gemm.hip)
bool grouped_supported(const moe_shape &s);
bool router_mfma_supported(const moe_shape &s);
hipError_t launch_router_mfma(const moe_shape &s, const void *x, const void *wr, const float *bias, float *logits,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
// m-tile offsets and the tile table (tiles of `rows` rows) from existing expert offsets
hipError_t launch_mtile_offsets(const moe_shape &s, const int32_t *offsets, int32_t *mtile_off, int32_t *tiles,
                                int rows, hipStream_t st);
// h'[p][i] = (wts ? wts[slot] : 1) * silu(g) * u, bf16, sorted order
hipError_t launch_gateup_mfma(const moe_shape &s, const void *x, const moe_expert_weights &w, const int32_t *offsets,
                              const int32_t *sorted, const int32_t *mtile_off, const int32_t *tiles, const float *wts,
                              void *h, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
// f32_sorted: o[p][n] fp32 in sorted order; else o'[slot][n] bf16 in slot (token-major) order
hipError_t launch_down_mfma(const moe_shape &s, const moe_expert_weights &w, const int32_t *offsets,
                            const int32_t *sorted, const int32_t *mtile_off, const int32_t *tiles, const void *h,
                            void *o, bool f32_sorted, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
// large-tile bf16 variants of the two expert GEMMs (see grouped_gemm_wide.hip); the
// launchers above route to them when the shape allows
bool wide_gateup_supported(const moe_shape &s);
bool wide_down_supported(const moe_shape &s);
// m-tile height the grouping must use for the grouped GEMMs of moe_forward on `s` (the bf16
// large-tile kernels take 64 or 128; every other kernel takes 128)
int grouped_tile_rows(const moe_shape &s);
hipError_t launch_gateup_wide(const moe_shape &s, const void *x, const moe_expert_weights &w, const int32_t *sorted,
                              const int32_t *mtile_off, const int32_t *tiles, const float *wts, void *h,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_down_wide(const moe_shape &s, const moe_expert_weights &w, const int32_t *sorted,
                            const int32_t *mtile_off, const int32_t *tiles, const void *h, void *o, hipStream_t st,
                            hipEvent_t ev0, hipEvent_t ev1);
// y[t] = sum_j o'[t*k+j] (bf16 rows)
hipError_t launch_combine_rows(const moe_shape &s, const void *o, void *y, hipStream_t st);

// moe_forward's host-side argument validation alone (launches nothing)
moe_status forward_check(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                         const moe_expert_weights *w, const void *y, const int32_t *topk_ids_out,
                         const float *topk_w_out, const void *ws, size_t ws_bytes);
// the whole layer on a given workspace (moe_forward, moe_forward_timed and the
// scratch-backed entry point share it): validation, then the launch sequence
moe_status forward_impl(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                        const moe_expert_weights *w, void *y, int32_t *topk_ids_out, float *topk_w_out, void *ws,
                        size_t ws_bytes, hipStream_t st, hipEvent_t *events, int n_events);

}  // namespace moe
