/*
 * moe_router.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN
 * layer: router top-k softmax, token->expert grouping, grouped SwiGLU expert
 * FFN and weighted combine, for decode batches of a few tokens and prefill
 * chunks of thousands.
 *
 * The staged calls follow the four stages the fused MoE profiling plan times
 * separately -- topk, expert kernel, activation, sum ("Decode 吞吐专项实验分析
 * 报告", section "2026-07-14：解除强制 eager / custom all-reduce 禁用验证",
 * subsection "下一步 profiling 方向").  moe_forward runs all of them on the
 * device with no host round trip on the routing result, the per-layer
 * stream synchronisation that "第 9 章 prefill：最大的瓶颈" §9.9 identifies as
 * the serial point of its prefill path, and it never drops a token-expert
 * entry, unlike the fixed 8-entries-per-group kernels of §9.5 there.
 *
 * Conventions shared by every call
 *   - Pointers are device pointers unless stated otherwise; the caller owns
 *     every buffer, including the workspace.  The library allocates nothing
 *     and keeps no global state.  Calls on different workspaces may run
 *     concurrently, with one exception: the single-launch decode path
 *     (moe_forward_stages == "decode_fused", T <= 8) needs one work-group
 *     resident on every compute unit at once, because its work-groups wait
 *     for one another.  It checks at launch that one of its work-groups fits
 *     a compute unit (and runs the staged decode kernels when it does not),
 *     but it cannot see other kernels: a call that overlaps with other work
 *     holding compute units may let its bounded waits expire, which sets
 *     MOE_DEVERR_TIMEOUT (moe_check_device_error) and leaves y invalid.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call synchronises or reads device memory on the
 *     host, except moe_check_device_error, which says so.
 *   - Arguments are validated on the host before anything is launched; a
 *     call that returns an error has launched nothing.
 *   - Layouts are row-major.  Weights are out-major with the contraction
 *     index contiguous ([N][K]).  MXFP4 stores two E2M1 codes per byte (the
 *     even element in the low nibble) with one E8M0 scale byte per 32
 *     consecutive contraction elements.
 *   - Device pointers must be 16-byte aligned.
 *   - The workspace must be zero-filled before its first use.  Zero-filling
 *     it whole again between calls is allowed; clearing parts of it is not:
 *     the decode path keeps a call counter in its control words across calls
 *     (it only grows), and the words it publishes carry that count.  The
 *     sticky device error word (byte 0) is cleared by moe_check_device_error.
 */
#ifndef MOE_ROUTER_H
#define MOE_ROUTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size, k>E, ... */
    MOE_ERR_UNSUPPORTED = -2,  /* legal but not implemented combination       */
    MOE_ERR_WORKSPACE = -3,    /* workspace smaller than moe_workspace_size   */
    MOE_ERR_HIP = -4,          /* a HIP launch or runtime call failed          */
    MOE_ERR_DEVICE = -5        /* moe_check_device_error found a device error  */
};

/* element formats.  MOE_NVFP4: two E2M1 codes per byte as for MXFP4, one OCP FP8 E4M3
   scale byte (bias 7, the NaN codes 0x7F / 0xFF not allowed) per 16 consecutive
   contraction elements, and one fp32 scale per weight tensor: an element is
   e2m1(code) * e4m3(block scale) * tensor scale.  MOE_MXINT8 (OCP MX INT8): one int8
   two's complement code per byte with an implicit scale of 2^-6, and one E8M0 scale
   byte per 32 consecutive contraction elements: an element is code * 2^(scale - 133)
   (block-int8 experts, the format of the fused int8 MoE path of "第 9 章 prefill：
   最大的瓶颈" §9.9; the kernels stay exact for scale codes 8..254). */
enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2, MOE_NVFP4 = 3, MOE_MXINT8 = 4 };

/* expert-FFN kernel family; AUTO picks DECODE for T <= 8 and while T * top_k < 2 * E (bf16
   experts), < 1.5 * E (MXFP4), < 1.25 * E (MXINT8) or < 4 * E (NVFP4), GROUPED above (bf16,
   MXFP4, NVFP4 and MXINT8 experts with bf16 activations) */
enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_GROUPED = 2 };

/* device error bits reported by moe_check_device_error */
enum { MOE_DEVERR_BAD_EXPERT_ID = 1, MOE_DEVERR_TIMEOUT = 2 };

typedef struct moe_shape {
    int32_t num_tokens;    /* T >= 0; T == 0 is a no-op                       */
    int32_t hidden;        /* H, multiple of 8 (of 32 for MXFP4 / NVFP4 / MXINT8), <= 8192 */
    int32_t num_experts;   /* E, 1..1024                                       */
    int32_t top_k;         /* k, 1..min(E, 32)                                 */
    int32_t intermediate;  /* I, multiple of 8 (of 32 for MXFP4 / NVFP4 / MXINT8), <= 8192 */
    int32_t renormalize;   /* nonzero: kept gate weights rescaled to sum 1     */
    int32_t act_dtype;     /* x, router weight, y: MOE_F32 or MOE_BF16         */
    int32_t weight_dtype;  /* experts: MOE_F32 (with F32 acts), MOE_BF16,
                              MOE_MXFP4, MOE_NVFP4 or MOE_MXINT8 (BF16 acts)   */
    int32_t path;          /* MOE_PATH_*                                        */
} moe_shape;

typedef struct moe_expert_weights {
    const void *w_gate;    /* [E][I][H]   (MXFP4 / NVFP4: [E][I][H/2] bytes;
                              MXINT8: [E][I][H] int8 codes)                    */
    const void *w_up;      /* [E][I][H]                                        */
    const void *w_down;    /* [E][H][I]   (MXFP4 / NVFP4: [E][H][I/2] bytes)   */
    const uint8_t *s_gate; /* MXFP4, MXINT8: E8M0 scales [E][I][H/32];
                              NVFP4: E4M3 scales [E][I][H/16]; else unused    */
    const uint8_t *s_up;   /* [E][I][H/32] or [E][I][H/16]                     */
    const uint8_t *s_down; /* [E][H][I/32] or [E][H][I/16]                     */
    float ts_gate;         /* NVFP4 only: the fp32 tensor scales (host values) */
    float ts_up;
    float ts_down;
} moe_expert_weights;

/* Bytes of workspace every call below needs for `shape` (0 on bad shape). */
size_t moe_workspace_size(const moe_shape *shape);

/*
 * Router gate + top-k ("gate" and "topk" stages of the profiling plan).
 *   s[t,e]  = bias[e] + sum_h x[t,h] * w_router[e,h]          (fp32 accumulate)
 *   kept    = the k largest s[t,.] by (score descending, expert id ascending)
 *   topk_w  = softmax over all E of s[t,.], taken at the kept experts and,
 *             when renormalize is set, divided by their sum
 * x [T][H] and w_router [E][H] in act_dtype; bias [E] fp32 or NULL (zero).
 * Outputs: topk_ids [T][k] int32 in ascending expert id, topk_w [T][k] fp32
 * in the same order.
 */
moe_status moe_router_topk(const moe_shape *shape, const void *x, const void *w_router,
                           const float *bias, int32_t *topk_ids, float *topk_w,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Token->expert grouping on the device ("第 9 章" §9.9: the fused path groups
 * by expert on the GPU instead of returning to the host every layer).
 * Slot t*k+j is token t's j-th kept expert.  Outputs:
 *   expert_offsets [E+1]: exclusive prefix of per-expert slot counts
 *   sorted_slots [T*k]  : slots ordered by expert, ascending slot inside each
 *                         expert (stable)
 *   slot_pos [T*k]      : inverse map, sorted_slots[slot_pos[s]] == s
 * An id outside [0, E) sets MOE_DEVERR_BAD_EXPERT_ID in the workspace error
 * word; the slot is then left out of every group (offsets[E] < T*k) and
 * nothing is written out of bounds.
 */
moe_status moe_group_tokens(const moe_shape *shape, const int32_t *topk_ids,
                            int32_t *expert_offsets, int32_t *sorted_slots, int32_t *slot_pos,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Expert FFN ("expert kernel" and "activation" stages) for every grouped slot:
 *   expert_out[p][n] = sum_i Wd[e][n][i] * a[i],
 *   a[i] = silu(g[i]) * u[i], g = Wg[e] x_t, u = Wu[e] x_t, silu(z) = z/(1+e^-z)
 * for p in [expert_offsets[e], expert_offsets[e+1]) and token t =
 * sorted_slots[p] / k.  expert_out is [T*k][H] fp32 in sorted order.  With
 * bf16/MXFP4 weights a is rounded to bf16 before the down projection.
 */
moe_status moe_expert_ffn(const moe_shape *shape, const void *x, const moe_expert_weights *w,
                          const int32_t *expert_offsets, const int32_t *sorted_slots,
                          float *expert_out, void *ws, size_t ws_bytes, void *stream);

/*
 * Weighted combine ("sum" stage):
 *   y[t][n] = sum_{j ascending} topk_w[t][j] * expert_out[slot_pos[t*k+j]][n]
 * accumulated in fp32 and stored once in act_dtype (round to nearest even).
 */
moe_status moe_combine(const moe_shape *shape, const float *expert_out, const float *topk_w,
                       const int32_t *slot_pos, void *y, void *stream);

/*
 * The whole layer (all stages above) on the device.  y [T][H] in act_dtype.
 * topk_ids_out / topk_w_out may be NULL; when given they receive the
 * routing exactly as moe_router_topk would.
 */
moe_status moe_forward(const moe_shape *shape, const void *x, const void *w_router,
                       const float *bias, const moe_expert_weights *w, void *y,
                       int32_t *topk_ids_out, float *topk_w_out,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * moe_forward with stage timing, for the per-stage profile the fused MoE
 * profiling plan asks for (topk / expert kernel / activation / sum times,
 * "Decode 吞吐专项实验分析报告", subsection "下一步 profiling 方向").
 * stage_events holds n_stage_events hipEvent_t handles created by the caller
 * (NULL entries are skipped): stage_events[2i] and stage_events[2i+1] bracket
 * the i-th kernel launch of the call, as named by moe_forward_stages.  For the
 * fused decode launch they are the kernel's own start and end timestamps
 * (hipExtLaunchKernelGGL); for the staged launches they are recorded on
 * `stream` right before and after the launch.  Results are identical to
 * moe_forward.
 */
moe_status moe_forward_timed(const moe_shape *shape, const void *x, const void *w_router,
                             const float *bias, const moe_expert_weights *w, void *y,
                             int32_t *topk_ids_out, float *topk_w_out, void *ws, size_t ws_bytes,
                             void *stream, void *const *stage_events, int32_t n_stage_events);

/*
 * The token->expert grouping that the last moe_forward (or moe_forward_timed) on
 * this workspace built on the device, copied into the caller's buffers on
 * `stream`: expert_offsets [E+1], sorted_slots [T*k] and slot_pos [T*k], as
 * moe_group_tokens defines them, for the ids that call routed.  It lets a caller
 * check the whole-layer call's own grouping output for output against a
 * reference ("第 9 章 prefill：最大的瓶颈" §9.9: a switch of numeric path is
 * checked against the old path's outputs).  Shapes whose moe_forward groups on
 * chip without storing the grouping (the single-launch decode path,
 * moe_forward_stages == "decode_fused") give MOE_ERR_UNSUPPORTED.  `ws` must be
 * the workspace of that call, with the same shape; nothing is checked about
 * whether a call ran.  Enqueues three device-to-device copies.
 */
moe_status moe_forward_grouping(const moe_shape *shape, const void *ws, size_t ws_bytes,
                                int32_t *expert_offsets, int32_t *sorted_slots, int32_t *slot_pos,
                                void *stream);

/* Comma-separated names of the kernel launches moe_forward makes for `shape`,
 * in order (static string; "" for an invalid shape). */
const char *moe_forward_stages(const moe_shape *shape);

/*
 * Synchronises `stream`, reads the workspace's device error word into
 * *err_bits (host pointer, MOE_DEVERR_* bits), clears it, and returns
 * MOE_ERR_DEVICE when it was nonzero.
 */
moe_status moe_check_device_error(void *ws, int32_t *err_bits, void *stream);

/* Bytes of device memory the library keeps per device for moe_forward_noalloc. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The workspace is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per device,
 * held until the process ends; nothing is allocated, by the library or by the
 * HIP runtime on its behalf.  Shapes whose moe_workspace_size exceeds it get
 * MOE_ERR_WORKSPACE before anything is enqueued: every decode batch of up to 8
 * tokens of every supported shape fits (at most 12.2 MiB), and medium batches of
 * up to ~200 tokens of the H=2048 / E=128 / k=8 / I=768 shape.
 *   - All calls on one device share that device's array, which keeps the last
 *     call's contents: calls that overlap on one device (on different streams
 *     or threads) race and must be serialised by the caller.
 *   - The first call on each device also clears the whole array on `stream`
 *     before its launches; a graph that captures that call clears it at every
 *     replay.
 *   - device_err (optional, 16-byte aligned device int32): receives the call's
 *     MOE_DEVERR_* bits (enqueued after the layer; the word is then cleared),
 *     as moe_check_device_error reports them for a caller-owned workspace.
 * Everything else (arguments, results, errors) is as for moe_forward.
 */
moe_status moe_forward_noalloc(const moe_shape *shape, const void *x, const void *w_router,
                               const float *bias, const moe_expert_weights *w, void *y,
                               int32_t *topk_ids_out, float *topk_w_out, int32_t *device_err,
                               void *stream);

/* Static text for a status code. */
const char *moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTER_H */
