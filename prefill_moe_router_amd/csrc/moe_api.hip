// moe_api.hip -- the C ABI (include/moe_router.h): host-side validation,
// workspace layout and the launch sequence of every entry point.  Nothing
// here touches device memory from the host or synchronises, except
// moe_check_device_error.
#include <algorithm>
#include <cmath>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int MAX_E = 1024;
constexpr int MAX_K = 32;
constexpr int MAX_DIM = 8192;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// H and I must be multiples of this: a 16-byte chunk (fp32, bf16) or a 32-element scale
// block (MXFP4, NVFP4 in pairs of 16-element blocks, MXINT8)
int weight_epc(int wdt) { return wdt == MOE_F32 ? 4 : wdt == MOE_BF16 ? 8 : 32; }

// shape checks shared by all calls
moe_status check_shape(const moe_shape *s) {
    if (!s) return MOE_ERR_INVALID_ARG;
    if (s->num_tokens < 0 || s->hidden <= 0 || s->intermediate <= 0 || s->num_experts <= 0) return MOE_ERR_INVALID_ARG;
    if (s->top_k < 1 || s->top_k > s->num_experts) return MOE_ERR_INVALID_ARG;
    if (s->act_dtype != MOE_F32 && s->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (s->weight_dtype != MOE_F32 && s->weight_dtype != MOE_BF16 && s->weight_dtype != MOE_MXFP4 &&
        s->weight_dtype != MOE_NVFP4 && s->weight_dtype != MOE_MXINT8)
        return MOE_ERR_INVALID_ARG;
    if (s->path < MOE_PATH_AUTO || s->path > MOE_PATH_GROUPED) return MOE_ERR_INVALID_ARG;
    const int epc = weight_epc(s->weight_dtype);
    if (s->hidden % 8 || s->intermediate % 8) return MOE_ERR_INVALID_ARG;
    if (s->hidden % epc || s->intermediate % epc) return MOE_ERR_INVALID_ARG;
    // supported element-format pairs
    const bool ok_pair = (s->act_dtype == MOE_F32 && s->weight_dtype == MOE_F32) ||
                         (s->act_dtype == MOE_BF16 && s->weight_dtype != MOE_F32);
    if (!ok_pair) return MOE_ERR_UNSUPPORTED;
    if (s->num_experts > MAX_E || s->top_k > MAX_K) return MOE_ERR_UNSUPPORTED;
    if (s->hidden > MAX_DIM || s->intermediate > MAX_DIM) return MOE_ERR_UNSUPPORTED;
    // fp32 rows: at most 16 chunks per lane
    if (s->weight_dtype == MOE_F32 && (s->hidden > 4096 || s->intermediate > 4096)) return MOE_ERR_UNSUPPORTED;
    if ((size_t)s->num_tokens * (size_t)s->top_k > (size_t)INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_ws(const moe_shape *s, const void *ws, size_t ws_bytes) {
    if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < ws_layout(*s).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

moe_status check_weights(const moe_shape *s, const moe_expert_weights *w) {
    if (!w || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
    if (!aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down)) return MOE_ERR_INVALID_ARG;
    const bool scaled = s->weight_dtype == MOE_MXFP4 || s->weight_dtype == MOE_NVFP4 || s->weight_dtype == MOE_MXINT8;
    if (scaled && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARG;
    // scale arrays: 16-byte aligned like every device pointer (the large-tile MXFP4 GEMM
    // loads a tile's scale rows into LDS 16 bytes at a time)
    if (scaled && (!aligned16(w->s_gate) || !aligned16(w->s_up) || !aligned16(w->s_down)))
        return MOE_ERR_INVALID_ARG;
    if (s->weight_dtype == MOE_NVFP4) {
        if (!std::isfinite(w->ts_gate) || !std::isfinite(w->ts_up) || !std::isfinite(w->ts_down))
            return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

moe_status check_path(const moe_shape *s) {
    // the grouped MFMA family covers bf16 experts; fp32 runs on the decode family
    if (s->path == MOE_PATH_GROUPED && !grouped_supported(*s)) return MOE_ERR_UNSUPPORTED;
    if (!stream_ffn_supported(*s)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// The grouped family's routing: the one-kernel router (router GEMM, top-k and block counts)
// whenever the shape allows it.  Measured on the 8192-token shape's layer, it beats the
// router GEMV + top-k + grouping kernels at every T from 32 up, even when its one
// work-group per 32 tokens leaves most of the chip idle.
bool fused_router(const moe_shape &s) { return router_topk_mfma_supported(s); }

// AUTO: the grouped GEMMs from 2 (token, expert) pairs per expert on average with bf16
// experts, 1.5 with MXFP4, 1.25 with MXINT8 and 4 with NVFP4 (whose streaming kernels read a
// quarter of the bytes); measured crossovers on the decode shapes (streaming / grouped):
// bf16 (k = 8, E = 128) 161 / 160 us at T = 24, 190 / 182 at 32; MXFP4 (k = 8, E = 256)
// 513 / 520 us at T = 40, 564 / 533 at 48, 660 / 546 at 64; MXINT8 (same shape) 842 / 943 us
// at T = 32, 1094 / 952 at 48, 1282 / 958 at 64
bool use_grouped(const moe_shape &s) {
    if (s.path == MOE_PATH_GROUPED) return true;
    const long quarters = s.weight_dtype == MOE_BF16     ? 8L    // pairs per expert x 4
                          : s.weight_dtype == MOE_MXFP4  ? 6L
                          : s.weight_dtype == MOE_MXINT8 ? 5L
                                                         : 16L;
    return s.path == MOE_PATH_AUTO && s.num_tokens > 8 &&
           4L * s.num_tokens * s.top_k >= quarters * s.num_experts && grouped_supported(s);
}

template <class T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<uint8_t *>(ws) + off);
}

#define MOE_TRY(expr)                                \
    do {                                             \
        if ((expr) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

#define MOE_CHECK(expr)                  \
    do {                                 \
        const moe_status _st = (expr);   \
        if (_st != MOE_OK) return _st;   \
    } while (0)

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_shape *shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return ws_layout(*shape).total;
}

moe_status moe_router_topk(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                           int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
    MOE_CHECK(check_shape(shape));
    if (shape->num_tokens == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_ids) || !aligned16(topk_w)) return MOE_ERR_INVALID_ARG;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 3u)) return MOE_ERR_INVALID_ARG;
    MOE_CHECK(check_ws(shape, ws, ws_bytes));
    const WsLayout L = ws_layout(*shape);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (fused_router(*shape)) {
        MOE_TRY(launch_router_topk_mfma(*shape, x, w_router, bias, topk_ids, topk_w, nullptr, nullptr, st, nullptr,
                                        nullptr));
        return MOE_OK;
    }
    MOE_TRY(launch_router_logits(*shape, x, w_router, bias, at<float>(ws, L.logits), st));
    MOE_TRY(launch_topk(*shape, at<float>(ws, L.logits), topk_ids, topk_w, st));
    return MOE_OK;
}

moe_status moe_group_tokens(const moe_shape *shape, const int32_t *topk_ids, int32_t *expert_offsets,
                            int32_t *sorted_slots, int32_t *slot_pos, void *ws, size_t ws_bytes, void *stream) {
    MOE_CHECK(check_shape(shape));
    const bool any = shape->num_tokens > 0;  // slot arrays may be NULL when there are no slots
    if (!expert_offsets || (any && (!topk_ids || !sorted_slots || !slot_pos))) return MOE_ERR_INVALID_ARG;
    if (!aligned16(topk_ids) || !aligned16(expert_offsets) || !aligned16(sorted_slots) || !aligned16(slot_pos))
        return MOE_ERR_INVALID_ARG;
    MOE_CHECK(check_ws(shape, ws, ws_bytes));
    const WsLayout L = ws_layout(*shape);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // T == 0 still defines the offsets (all zero)
    MOE_TRY(launch_group2(*shape, topk_ids, expert_offsets, sorted_slots, slot_pos, at<int32_t>(ws, L.active),
                          at<int32_t>(ws, L.gcounts), nullptr, nullptr, kGroupedTileM, at<int32_t>(ws, L.ctrl), st));
    return MOE_OK;
}

moe_status moe_expert_ffn(const moe_shape *shape, const void *x, const moe_expert_weights *w,
                          const int32_t *expert_offsets, const int32_t *sorted_slots, float *expert_out, void *ws,
                          size_t ws_bytes, void *stream) {
    MOE_CHECK(check_shape(shape));
    MOE_CHECK(check_path(shape));
    if (shape->num_tokens == 0) return MOE_OK;
    MOE_CHECK(check_weights(shape, w));
    if (!x || !expert_offsets || !sorted_slots || !expert_out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(expert_offsets) || !aligned16(sorted_slots) || !aligned16(expert_out))
        return MOE_ERR_INVALID_ARG;
    MOE_CHECK(check_ws(shape, ws, ws_bytes));
    const WsLayout L = ws_layout(*shape);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (use_grouped(*shape)) {
        int32_t *mtile = at<int32_t>(ws, L.mtile);
        int32_t *tiles = at<int32_t>(ws, L.tiles);
        const int rows = grouped_tile_rows(*shape);
        MOE_TRY(launch_mtile_offsets(*shape, expert_offsets, mtile, tiles, rows, st));
        MOE_TRY(launch_gateup_mfma(*shape, x, *w, expert_offsets, sorted_slots, mtile, tiles, nullptr,
                                   at<void>(ws, L.h), st, nullptr, nullptr));
        // the fp32 sorted-order down projection runs on the register-staged kernel (128-row tiles)
        if (rows != kGroupedTileM) MOE_TRY(launch_mtile_offsets(*shape, expert_offsets, mtile, tiles, kGroupedTileM, st));
        MOE_TRY(launch_down_mfma(*shape, *w, expert_offsets, sorted_slots, mtile, tiles, at<void>(ws, L.h),
                                 expert_out, true, st, nullptr, nullptr));
        return MOE_OK;
    }
    int32_t *active = at<int32_t>(ws, L.active);
    MOE_TRY(launch_active(*shape, expert_offsets, active, st));
    MOE_TRY(launch_decode_gateup(*shape, x, *w, expert_offsets, sorted_slots, active, nullptr, at<void>(ws, L.h), st));
    MOE_TRY(launch_decode_down(*shape, *w, expert_offsets, active, at<void>(ws, L.h), expert_out, st));
    return MOE_OK;
}

moe_status moe_combine(const moe_shape *shape, const float *expert_out, const float *topk_w, const int32_t *slot_pos,
                       void *y, void *stream) {
    MOE_CHECK(check_shape(shape));
    if (shape->num_tokens == 0) return MOE_OK;
    if (!expert_out || !topk_w || !slot_pos || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned16(expert_out) || !aligned16(topk_w) || !aligned16(slot_pos) || !aligned16(y))
        return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_combine(*shape, expert_out, topk_w, slot_pos, y, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

}  // extern "C"

namespace {

const char *const kStagesStaged = "router_logits,topk,group,gate_up,down,combine";
const char *const kStagesFused = "decode_fused";
const char *const kStagesGrouped = "router_logits,topk,group,gate_up,down,combine";
const char *const kStagesGroupedFusedRouter = "router_topk,group,gate_up,down,combine";

// The single-launch decode kernel needs a work-group on every compute unit at once; when
// one of its work-groups does not fit a compute unit, the staged decode kernels run.
bool use_fused(const moe_shape &s) {
    return !use_grouped(s) && s.num_tokens <= 8 && decode_fused_supported(s) && decode_fused_coresident(s);
}

// Event pair (start, stop) of launch i, taken from ev[2i], ev[2i+1] when present.
struct StageEvents {
    hipEvent_t *ev;
    int n;
    hipEvent_t start(int i) const { return (ev && 2 * i < n) ? ev[2 * i] : nullptr; }
    hipEvent_t stop(int i) const { return (ev && 2 * i + 1 < n) ? ev[2 * i + 1] : nullptr; }
};

// Records the pair around a launch made by the staged launchers.
template <class Fn>
hipError_t around(const StageEvents &se, int i, hipStream_t st, Fn &&fn) {
    hipError_t r;
    if (se.start(i) && (r = hipEventRecord(se.start(i), st)) != hipSuccess) return r;
    if ((r = fn()) != hipSuccess) return r;
    if (se.stop(i) && (r = hipEventRecord(se.stop(i), st)) != hipSuccess) return r;
    return hipSuccess;
}

}  // namespace

namespace moe {

moe_status forward_check(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                         const moe_expert_weights *w, const void *y, const int32_t *topk_ids_out,
                         const float *topk_w_out, const void *ws, size_t ws_bytes) {
    MOE_CHECK(check_shape(shape));
    MOE_CHECK(check_path(shape));
    if (shape->num_tokens == 0) return MOE_OK;
    MOE_CHECK(check_weights(shape, w));
    if (!x || !w_router || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
    if ((topk_ids_out && !aligned16(topk_ids_out)) || (topk_w_out && !aligned16(topk_w_out)))
        return MOE_ERR_INVALID_ARG;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 3u)) return MOE_ERR_INVALID_ARG;
    return check_ws(shape, ws, ws_bytes);
}

moe_status forward_impl(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                        const moe_expert_weights *w, void *y, int32_t *topk_ids_out, float *topk_w_out, void *ws,
                        size_t ws_bytes, hipStream_t st, hipEvent_t *events, int n_events) {
    MOE_CHECK(forward_check(shape, x, w_router, bias, w, y, topk_ids_out, topk_w_out, ws, ws_bytes));
    if (shape->num_tokens == 0) return MOE_OK;
    const StageEvents se{events, n_events};
    if (use_fused(*shape)) {
        MOE_TRY(launch_decode_fused(*shape, x, w_router, bias, *w, y, topk_ids_out, topk_w_out, ws, st, se.start(0),
                                    se.stop(0)));
        return MOE_OK;
    }
    const WsLayout L = ws_layout(*shape);
    int32_t *ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
    float *wts = topk_w_out ? topk_w_out : at<float>(ws, L.wts);
    int32_t *offsets = at<int32_t>(ws, L.offsets), *sorted = at<int32_t>(ws, L.sorted);
    int32_t *slot_pos = at<int32_t>(ws, L.slot_pos), *active = at<int32_t>(ws, L.active);
    float *logits = at<float>(ws, L.logits), *o = at<float>(ws, L.o);
    void *h = at<void>(ws, L.h);
    int32_t *err = at<int32_t>(ws, L.ctrl);
    if (use_grouped(*shape)) {
        int32_t *mtile = at<int32_t>(ws, L.mtile), *tiles = at<int32_t>(ws, L.tiles);
        int si = 0;   // stage index, in the order moe_forward_stages names them
        if (fused_router(*shape)) {
            // router, top-k and the per-block half of the grouping in one kernel
            int32_t *counts = at<int32_t>(ws, L.gcounts);
            MOE_TRY(launch_router_topk_mfma(*shape, x, w_router, bias, ids, wts, slot_pos, counts, st, se.start(si),
                                            se.stop(si)));
            ++si;
            MOE_TRY(around(se, si++, st, [&] {
                return launch_group_from_router(*shape, ids, counts, offsets, sorted, slot_pos, active, mtile, tiles,
                                                grouped_tile_rows(*shape), st);
            }));
        } else {
            if (router_mfma_supported(*shape)) {
                MOE_TRY(launch_router_mfma(*shape, x, w_router, bias, logits, st, se.start(si), se.stop(si)));
                ++si;
            } else {
                MOE_TRY(around(se, si++, st, [&] { return launch_router_logits(*shape, x, w_router, bias, logits, st); }));
            }
            MOE_TRY(around(se, si++, st, [&] { return launch_topk(*shape, logits, ids, wts, st); }));
            MOE_TRY(around(se, si++, st, [&] {
                return launch_group2(*shape, ids, offsets, sorted, slot_pos, active, at<int32_t>(ws, L.gcounts), mtile,
                                     tiles, grouped_tile_rows(*shape), err, st);
            }));
        }
        MOE_TRY(launch_gateup_mfma(*shape, x, *w, offsets, sorted, mtile, tiles, wts, h, st, se.start(si),
                                   se.stop(si)));
        ++si;
        MOE_TRY(launch_down_mfma(*shape, *w, offsets, sorted, mtile, tiles, h, o, false, st, se.start(si),
                                 se.stop(si)));
        ++si;
        MOE_TRY(around(se, si, st, [&] { return launch_combine_rows(*shape, o, y, st); }));
        return MOE_OK;
    }
    MOE_TRY(around(se, 0, st, [&] { return launch_router_logits(*shape, x, w_router, bias, logits, st); }));
    MOE_TRY(around(se, 1, st, [&] { return launch_topk(*shape, logits, ids, wts, st); }));
    MOE_TRY(around(se, 2, st, [&] {
        return launch_group2(*shape, ids, offsets, sorted, slot_pos, active, at<int32_t>(ws, L.gcounts), nullptr,
                             nullptr, kGroupedTileM, err, st);
    }));
    MOE_TRY(around(se, 3, st, [&] {
        return launch_decode_gateup(*shape, x, *w, offsets, sorted, active, nullptr, h, st);
    }));
    MOE_TRY(around(se, 4, st, [&] { return launch_decode_down(*shape, *w, offsets, active, h, o, st); }));
    MOE_TRY(around(se, 5, st, [&] { return launch_combine(*shape, o, wts, slot_pos, y, st); }));
    return MOE_OK;
}

}  // namespace moe

extern "C" {

moe_status moe_forward(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                       const moe_expert_weights *w, void *y, int32_t *topk_ids_out, float *topk_w_out, void *ws,
                       size_t ws_bytes, void *stream) {
    return forward_impl(shape, x, w_router, bias, w, y, topk_ids_out, topk_w_out, ws, ws_bytes,
                        static_cast<hipStream_t>(stream), nullptr, 0);
}

moe_status moe_forward_timed(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                             const moe_expert_weights *w, void *y, int32_t *topk_ids_out, float *topk_w_out,
                             void *ws, size_t ws_bytes, void *stream, void *const *stage_events,
                             int32_t n_stage_events) {
    if (n_stage_events < 0 || (n_stage_events > 0 && !stage_events)) return MOE_ERR_INVALID_ARG;
    return forward_impl(shape, x, w_router, bias, w, y, topk_ids_out, topk_w_out, ws, ws_bytes,
                        static_cast<hipStream_t>(stream),
                        reinterpret_cast<hipEvent_t *>(const_cast<void **>(stage_events)), n_stage_events);
}

const char *moe_forward_stages(const moe_shape *shape) {
    if (check_shape(shape) != MOE_OK) return "";
    if (use_grouped(*shape)) return fused_router(*shape) ? kStagesGroupedFusedRouter : kStagesGrouped;
    return use_fused(*shape) ? kStagesFused : kStagesStaged;
}

moe_status moe_forward_grouping(const moe_shape *shape, const void *ws, size_t ws_bytes, int32_t *expert_offsets,
                                int32_t *sorted_slots, int32_t *slot_pos, void *stream) {
    MOE_CHECK(check_shape(shape));
    MOE_CHECK(check_path(shape));
    if (use_fused(*shape)) return MOE_ERR_UNSUPPORTED;
    const size_t P = (size_t)shape->num_tokens * (size_t)shape->top_k;
    if (!expert_offsets || (P && (!sorted_slots || !slot_pos))) return MOE_ERR_INVALID_ARG;
    if (!aligned16(expert_offsets) || !aligned16(sorted_slots) || !aligned16(slot_pos)) return MOE_ERR_INVALID_ARG;
    MOE_CHECK(check_ws(shape, ws, ws_bytes));
    const WsLayout L = ws_layout(*shape);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint8_t *b = static_cast<const uint8_t *>(ws);
    const size_t E1 = (size_t)shape->num_experts + 1;
    MOE_TRY(hipMemcpyAsync(expert_offsets, b + L.offsets, E1 * 4, hipMemcpyDeviceToDevice, st));
    if (P) {
        MOE_TRY(hipMemcpyAsync(sorted_slots, b + L.sorted, P * 4, hipMemcpyDeviceToDevice, st));
        MOE_TRY(hipMemcpyAsync(slot_pos, b + L.slot_pos, P * 4, hipMemcpyDeviceToDevice, st));
    }
    return MOE_OK;
}

moe_status moe_check_device_error(void *ws, int32_t *err_bits, void *stream) {
    if (!ws || !aligned16(ws) || !err_bits) return MOE_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t v = 0;
    MOE_TRY(hipStreamSynchronize(st));
    MOE_TRY(hipMemcpy(&v, ws, sizeof v, hipMemcpyDeviceToHost));
    *err_bits = v;
    if (v != 0) {
        const int32_t zero = 0;
        MOE_TRY(hipMemcpy(ws, &zero, sizeof zero, hipMemcpyHostToDevice));
        return MOE_ERR_DEVICE;
    }
    return MOE_OK;
}

const char *moe_status_string(moe_status status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or format combination";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_DEVICE: return "device-side error reported";
        default: return "unknown status";
    }
}

}  // extern "C"
