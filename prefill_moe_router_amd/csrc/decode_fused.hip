// decode_fused.hip -- the whole MoE layer for a decode batch (T <= 8 tokens)
// in ONE persistent launch: router gate, top-k softmax, grouping, expert
// gate/up + SwiGLU, down projection and weighted combine.
//
// The decode step of the serving report is starved by small kernels and the
// bubbles between them ("Decode 吞吐专项实验分析报告", 一、结论摘要 and
// 四、瓶颈判断: low GPU utilisation with many small kernels and syncs); one
// launch pays the fixed launch/drain cost once.  The routing never leaves the
// device ("第 9 章 prefill：最大的瓶颈" §9.9) and every token-expert pair is
// computed whatever the batch (no 8-entry group limit, §9.5).
//
// One work-group per CU, all co-resident; gate/up and down are separated by a
// grid barrier on per-work-group flag words: each work-group stores this call's
// tag into its own word (a plain store: no read-modify-write contended by the
// whole grid) and waits until every word carries it.  The tag comes from a
// 64-bit call counter in the workspace that only grows (work-group 0 adds one
// after the barrier, when every work-group has read it), with relaxed atomics
// only.  Data that crosses work-groups (logits, h') is written
// with write-through agent-scope stores and read with agent-scope loads, so
// no cache writeback or invalidation is needed at the barrier.  Every wait is
// bounded and sets MOE_DEVERR_TIMEOUT instead of hanging.
//   0. router: expert rows spread one per wave over the work-groups of the
//      first-started XCDs; each logit goes
//      to the workspace as one self-validating 64-bit word (value | call tag),
//      so no barrier is needed before it is read.
//   1. every work-group redundantly takes the top-k of all T tokens (polling
//      until all words carry this call's tag) and groups the T*k slots by
//      expert in LDS (tiny: T*k <= 256).
//   2. gate/up: one wave per (active expert, row i); the two 16-byte-chunked
//      rows are dotted with the tokens of that expert (x staged in LDS);
//      h'[slot][i] = w_slot * silu(g) * u goes to the workspace.   -- barrier
//      (each wave issues its first down-projection loads before waiting)
//   3. down + combine: a work-group owns a tile of output rows, its waves
//      split the active experts; each wave streams the tile's rows of Wd[e]
//      once and dots them with e's h' rows (staged in LDS), and the tile's
//      y[t][n] = sum over t's slots of Wd[e][n].h'[slot] is summed over the
//      waves in LDS -- the weighted sum over the token's experts needs no
//      second pass.
#include <hip/hip_ext.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int FWPB = 8;                 // waves per work-group
constexpr int FTHREADS = FWPB * WAVE;
constexpr int FMAX_T = kFusedMaxTokens;
constexpr int FMAX_P = 256;             // T * k
constexpr int FMAX_G = kFusedMaxGroups; // work-groups (one per CU)
constexpr int FROUNDS_MAX_K = 12;       // top-k by arg-max rounds up to this k, radix walk above
constexpr int FRANK_MAX_E = 128;        // one token: top-k by counted ranks over all E up to this E
                                        // (measured: 0.7 us faster at E = 128, 0.5 us slower at E = 256)
constexpr int FRANK2_MAX_E = FWPB * 64; // one token above that: ranks in two levels (a wave's 64
constexpr int FRANK2_MAX_K = 8;         // experts, then at most 64 candidates) up to this E and k
constexpr int FMAX_C = 8;               // max 16-byte chunks per lane of one row
constexpr int FMAX_WR = 32;             // output rows of one work-group (its tiles' rows)
constexpr size_t FLDS_MAX = 140 * 1024; // staged x / h' bytes per work-group (static LDS ~16 KB)
constexpr uint64_t SPIN_TICKS = 20000000ull;  // 0.2 s of the 100 MHz real-time clock

struct FusedParams {
    const uint8_t *x, *wr;
    const float *bias;
    const uint8_t *wg, *wu, *wd, *sg, *su, *sd;
    uint8_t *y;
    int32_t *ids_out;
    float *w_out;
    uint64_t *logits; // workspace [FMAX_T][E] words: logit bits | (call tag << 32)
    uint8_t *hbuf;    // workspace [P][I] (activation dtype)
    uint64_t *bar;    // workspace control word: completed calls (only grows)
    uint64_t *flags;  // workspace [nblocks] words: the barrier tag each work-group stored last
    int32_t *err;
    float tsg, tsu, tsd;   // tensor scales of the gate, up and down weights (1 unless NVFP4)
    int T, H, E, K, I, renorm, nblocks;
};

// ---- grid barrier --------------------------------------------------------------------

// The call counter: read by every work-group at kernel start; work-group 0 adds one after
// the barrier, which no work-group passes before all have read it.  So every work-group
// reads the same count, and this call's tag (count + 1) differs from every earlier call's.
__device__ __forceinline__ uint64_t call_count(const uint64_t *bar) {
    return __hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival: every wave's cross-group stores are acknowledged first, then the work-group's
// flag word takes this call's tag.
__device__ __forceinline__ void bar_arrive(uint64_t *flags, uint32_t tag) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(flags + blockIdx.x, (uint64_t)tag << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 polls the G flag words (NJ per lane, G <= 64 * NJ) until all carry the tag.
// ACQ: end with an agent-scope acquire (invalidates this CU's stale cache lines) so that
// plain loads may read what other work-groups wrote before the barrier.
template <int NJ, bool ACQ = false>
__device__ __forceinline__ void bar_wait(const uint64_t *flags, int G, uint32_t tag, int32_t *err) {
    if (threadIdx.x < WAVE) {
        const int lane = threadIdx.x;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            uint64_t wd[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int i = lane + WAVE * j;
                wd[j] = i < G ? __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : ((uint64_t)tag << 32);
            }
            bool ready = true;
#pragma unroll
            for (int j = 0; j < NJ; ++j) ready = ready && (uint32_t)(wd[j] >> 32) == tag;
            if (__ballot(!ready) == 0ull) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
                if (lane == 0) atomicOr(err, MOE_DEVERR_TIMEOUT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (ACQ) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

// ---- small helpers -------------------------------------------------------------------

// C chunks of 16 bytes per lane: chunk lane0 + stride*c of the row (c < C), zero past nch.
// Loaded through buffer resources over the row and its scales: chunks past the row end
// read zero without a memory access and without a branch, so every call issues the same
// loads.  (A load under a branch leaves the compiler unsure how many loads are in flight,
// and it then waits for all of them, the next item's prefetch too, before the first use.)
template <class F, int C>
__device__ __forceinline__ void load_chunks(const uint8_t *row, const uint8_t *srow, int nch, int lane0, int stride,
                                            uint4 (&q)[C], uint32_t (&s)[C]) {
    const rsrc_t rw = make_rsrc(row, (uint32_t)nch * 16);
#pragma unroll
    for (int c = 0; c < C; ++c) q[c] = ld_rsrc16(rw, (uint32_t)(lane0 + stride * c) * 16);
    if constexpr (F::SCALED) {
        const rsrc_t rs = make_rsrc(srow, (uint32_t)scale_row_bytes<F>(nch));
#pragma unroll
        for (int c = 0; c < C; ++c) s[c] = load_scale_r<F>(rs, (uint32_t)(lane0 + stride * c));
    } else {
#pragma unroll
        for (int c = 0; c < C; ++c) s[c] = 0u;
    }
}

template <class F, int C>
__device__ __forceinline__ float row_dot(const uint4 (&q)[C], const uint32_t (&s)[C], const uint8_t *act, int nch,
                                         int lane0, int stride) {
    // 16-byte activation chunks: branch-free (chunks past the row end read chunk 0 and
    // are discarded), so that all LDS reads can be issued before the first dot product.
    // MXFP4 chunks take 64 bytes of activations each; there the reads stay per chunk.
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int ch = lane0 + stride * c;
        const bool ok = ch < nch;
        if constexpr (F::XB == 16) {
            const float v = chunk_dot<F>(q[c], s[c], act + (size_t)(ok ? ch : 0) * F::XB, acc);
            acc = ok ? v : acc;
        } else {
            if (ok) acc = chunk_dot<F>(q[c], s[c], act + (size_t)ch * F::XB, acc);
        }
    }
    return acc;
}

// total of each group of LR consecutive lanes (8, 16, 32 or 64), in the group's last lane
template <int LR>
__device__ __forceinline__ float lane_group_sum(float v) {
    v += dpp_f<0x111>(v, 0.f);   // row_shr:1
    v += dpp_f<0x112>(v, 0.f);   // row_shr:2
    v += dpp_f<0x114>(v, 0.f);   // row_shr:4
    if (LR >= 16) v += dpp_f<0x118>(v, 0.f);          // row_shr:8
    if (LR >= 32) v += dpp_f<0x142, 0xa>(v, 0.f);     // row_bcast:15
    if (LR >= 64) v += dpp_f<0x143, 0xc>(v, 0.f);     // row_bcast:31
    return v;
}

__device__ __forceinline__ void store_act_sc1(uint8_t *base, size_t idx, float v, bool f32) {
    if (f32)
        __hip_atomic_store(reinterpret_cast<float *>(base) + idx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        __hip_atomic_store(reinterpret_cast<uint16_t *>(base) + idx, (uint16_t)f32_to_bf16_rne(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}


// Wait (one wave) until the n logit words [0, n) carry this call's tag, and copy the
// values to lg (LDS).  Up to 1024 words (16 per lane) are loaded per poll round trip,
// all loads issued before any is checked.  All the work-groups' pollers share a few
// memory lines with the router's stores, so the polls back off (up to ~0.4 us apart)
// to leave those lines to the writers.  Bounded: MOE_DEVERR_TIMEOUT on expiry.
__device__ __forceinline__ bool poll_words(const uint64_t *words, int n, uint32_t tag, float *lg, uint64_t t0,
                                           int32_t *err) {
    constexpr int NJ = 16;
    const int lane = threadIdx.x & 63;
    for (int base = 0; base < n; base += NJ * WAVE) {
        uint64_t wd[NJ];
        int nap = 1;
        for (;;) {
            bool ready = true;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int i = base + lane + WAVE * j;
                wd[j] = i < n ? __hip_atomic_load(words + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : ((uint64_t)tag << 32);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) ready = ready && (uint32_t)(wd[j] >> 32) == tag;
            if (__ballot(!ready) == 0ull) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
                if (lane == 0) atomicOr(err, MOE_DEVERR_TIMEOUT);
                return false;
            }
            for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(2);
            nap = nap < 8 ? nap * 2 : 8;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int i = base + lane + WAVE * j;
            if (i < n) lg[i] = __uint_as_float((uint32_t)wd[j]);
        }
    }
    return true;
}

// ---- the kernel ------------------------------------------------------------------------

// F: expert weight format; A: activation / router format (FmtF32 or FmtBF16);
// CG / CR / CD: 16-byte chunks per lane of a gate-up row, a router row and a
// down row (slice).
template <class F, class A, int CG, int CR, int CD>
__global__ __launch_bounds__(FTHREADS) void decode_fused_kernel(FusedParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // staged x, later staged h'
    __shared__ int s_ids[FMAX_P];
    __shared__ float s_w[FMAX_P];
    __shared__ int s_tok[FMAX_P];     // token of each slot, in expert-sorted order
    __shared__ float s_wq[FMAX_P];    // routing weight of each slot, in expert-sorted order
    __shared__ int s_act_e[FMAX_P], s_act_start[FMAX_P], s_act_cnt[FMAX_P];
    __shared__ int s_nact;
    __shared__ float s_part[FWPB * FMAX_T * FMAX_WR];   // down partials [wave][token][work-group row]
    __shared__ uint32_t s_tag;

    const int T = p.T, H = p.H, E = p.E, K = p.K, I = p.I, P = T * K;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int G = p.nblocks;
    const int NW = G * FWPB;
    const int gw = blockIdx.x + G * wave;        // consecutive work items land on different CUs
    const bool f32 = A::EPC == 4;
    const int ab = f32 ? 4 : 2;
    const size_t lg_off = ((size_t)T * H * ab + 15) & ~(size_t)15;   // LDS logits after the staged x
    // after the logits: the per-expert token masks of the top-k, then 64 words per wave
    // that lanes with nothing to store write to
    const size_t sel_off = (lg_off + (size_t)T * E * 4 + 15) & ~(size_t)15;
    uint32_t *s_sel = reinterpret_cast<uint32_t *>(smem + sel_off);
    uint32_t *s_trash = s_sel + ((E + 3) & ~3);
    // then (one token) the experts' packed selection keys (16-byte aligned)
    uint64_t *s_pk = reinterpret_cast<uint64_t *>(s_trash + FWPB * WAVE);

    if (tid == 0) {
        s_tag = (uint32_t)call_count(p.bar) + 1u;
        s_nact = 0;
    }
    for (int i = tid; i < FWPB * FMAX_T * FMAX_WR; i += FTHREADS) s_part[i] = 0.f;
    for (int i = tid; i < E; i += FTHREADS) s_sel[i] = 0u;

    // ---- phase 0: router logits (row loads first, then x staged into LDS) ----------------
    {
        const int nch = H / A::EPC;
        const size_t xrow = (size_t)H * ab;
        // Router rows go to the work-groups of the first two XCDs (blocks b with b % 8 < 2
        // under the round-robin block-to-XCD dispatch): measured, they start about 2 us
        // before those of the other XCDs, so the logits are ready when the rest arrive.
        const bool xcd8 = G % 8 == 0;
        const int nrb = xcd8 ? G / 4 : G;                                  // router work-groups
        const int rb = !xcd8 ? (int)blockIdx.x
                             : ((blockIdx.x & 7) < 2 ? (int)(blockIdx.x >> 3) * 2 + (int)(blockIdx.x & 7) : -1);
        const int NRW = nrb * FWPB;
        const int e = rb >= 0 ? rb + nrb * wave : E;
        uint4 q[CR];
        uint32_t sc[CR];
        if (e < E) load_chunks<A, CR>(p.wr + (size_t)e * nch * 16, nullptr, nch, lane, WAVE, q, sc);
        const int n16 = T * H * ab / 16;
        const uint4 *src = reinterpret_cast<const uint4 *>(p.x);
        uint4 *dst = reinterpret_cast<uint4 *>(smem);
        for (int i = tid; i < n16; i += FTHREADS) dst[i] = src[i];
        __syncthreads();
        for (int ee = e; ee < E; ee += NRW) {
            if (ee != e) load_chunks<A, CR>(p.wr + (size_t)ee * nch * 16, nullptr, nch, lane, WAVE, q, sc);
            const float b = p.bias ? p.bias[ee] : 0.f;
            // every token's logit first (lane t keeps token t's), then one store of all of them:
            // a store between the tokens would make the next token wait for it.  Every row
            // t < FMAX_T is rewritten each call (rows past T with the tag only), so a word this
            // call reads was last written by this call or by the one before it.
            float mine = 0.f;
#pragma unroll
            for (int t = 0; t < FMAX_T; ++t) {
                if (t < T) {
                    const float v = dpp_sum64(row_dot<A, CR>(q, sc, smem + t * xrow, nch, lane, WAVE));
                    const float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
                    mine = lane == t ? r + b : mine;
                }
            }
            if (lane < FMAX_T)
                __hip_atomic_store(p.logits + (size_t)lane * E + ee,
                                   (uint64_t)__float_as_uint(mine) | ((uint64_t)s_tag << 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // ---- phase 1: logits to LDS (wave 0 waits for them), top-k + softmax per token (wave t),
    // then grouping
    float *s_lg = reinterpret_cast<float *>(smem + lg_off);   // [T][E], after the staged x
    if (wave == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        poll_words(p.logits, T * E, s_tag, s_lg, t0, p.err);
    }
    __syncthreads();
    const bool rank1 = T == 1 && E <= FRANK_MAX_E;
    const bool rank2 = T == 1 && !rank1 && E <= FRANK2_MAX_E && K <= FRANK2_MAX_K;
    if (rank1 || rank2) {
        // One token: an expert's rank is the number of experts that beat it (a larger logit
        // key, or the same key and a lower id); ranks 0..K-1 are the kept experts.  The same
        // selection as the per-wave top-k below, in a few dependent steps instead of K
        // rounds in one wave.  One slot per kept expert, in ascending id, is the grouping.
        // The key (order key << 32 | ~e) is unique per expert, and the low word gives e back.
        if (rank1) {
            // the E*E comparisons split over all the work-group's waves
            uint32_t *s_rank = s_sel;   // zeroed at kernel start
            for (int e = tid; e < E; e += FTHREADS)
                s_pk[e] = ((uint64_t)f32_order_key(s_lg[e]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
            __syncthreads();
            const int epad = (E + WAVE - 1) / WAVE * WAVE;
            const int nparts = epad >= FTHREADS ? 1 : FTHREADS / epad;
            const int span = (E + nparts - 1) / nparts;
            for (int i = tid; i < epad * nparts; i += FTHREADS) {
                const int e = i % epad, part = i / epad;   // part is the same in the whole wave
                const int j0 = part * span, j1 = min(E, j0 + span);
                const uint64_t mine = e < E ? s_pk[e] : ~0ull;
                uint32_t r = 0;
#pragma unroll 8
                for (int j = j0; j < j1; ++j) r += s_pk[j] > mine ? 1u : 0u;
                if (e < E) atomicAdd(s_rank + e, r);
            }
            __syncthreads();
            for (int e = tid; e < E; e += FTHREADS) {
                const uint32_t r = s_rank[e];
                if (r < (uint32_t)K) s_ids[r] = e;   // s_ids by rank
            }
            __syncthreads();
        } else {
            // Two levels.  Wave w ranks its 64 experts 64w..64w+63 among themselves and keeps
            // those of local rank < K as candidates (slot w*K + local rank; empty slots hold
            // key 0, below every expert's).  An expert of global rank < K has local rank < K,
            // and every expert that beats it beats it locally too, so its rank among the
            // candidates is its global rank; any other candidate has at least K above it.
            uint64_t *s_cand = reinterpret_cast<uint64_t *>(s_trash);   // [FWPB * K] keys
            const int ng = (E + WAVE - 1) / WAVE;
            if (wave < ng) {
                const int e = wave * WAVE + lane;
                const uint64_t mine =
                    e < E ? ((uint64_t)f32_order_key(s_lg[e]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e) : 0ull;
                if (e < E) s_pk[e] = mine;
                if (lane < K) s_cand[wave * K + lane] = 0ull;
                // the wave reads back its own lanes' keys (a wave's LDS accesses complete in order)
                const int jn = min(WAVE, E - wave * WAVE);
                uint32_t r = 0;
#pragma unroll 8
                for (int j = 0; j < jn; ++j) r += s_pk[wave * WAVE + j] > mine ? 1u : 0u;
                if (e < E && r < (uint32_t)K) s_cand[wave * K + r] = mine;
            }
            __syncthreads();
            if (wave == 0) {
                const int nc = ng * K;   // at most 64
                const uint64_t mine = lane < nc ? s_cand[lane] : 0ull;
                uint32_t r = 0;
                for (int j = 0; j < nc; ++j) r += s_cand[j] > mine ? 1u : 0u;
                if (mine != 0ull && r < (uint32_t)K) s_ids[r] = (int)(0xffffffffu - (uint32_t)mine);
            }
        }
        if (wave == 0) {
            // lane j < K: the expert of rank j, its place in ascending id, its weight
            const bool on = lane < K;
            const int ej = on ? s_ids[lane] : 0;
            const float m = f32_from_order_key((uint32_t)(s_pk[s_ids[0]] >> 32));   // the largest logit
            int pos = 0;
            for (int l = 0; l < K; ++l) pos += s_ids[l] < ej ? 1 : 0;
            const float pe = on ? __expf(s_lg[ej] - m) : 0.f;
            float z;
            if (p.renorm) {
                z = wave_sum_u(pe);
            } else {
                float zs = 0.f;
                for (int e0 = 0; e0 < E; e0 += WAVE) {
                    const int e = e0 + lane;
                    zs += e < E ? __expf(s_lg[e] - m) : 0.f;
                }
                z = wave_sum_u(zs);
            }
            const float wj = pe / z;
            if (on) {
                s_act_e[pos] = ej;
                s_act_start[pos] = pos;
                s_act_cnt[pos] = 1;
                s_tok[pos] = 0;
                s_wq[pos] = wj;
                if (blockIdx.x == 0) {
                    if (p.ids_out) p.ids_out[pos] = ej;
                    if (p.w_out) p.w_out[pos] = wj;
                }
            }
            if (lane == 0) s_nact = K;
        }
    } else {
        // top-k of token t in wave t: K rounds of a wave arg-max for small K, otherwise a radix
        // walk over the logit keys (exact either way, ties to the lower id); bit t of s_sel[e] marks that token t
        // kept expert e, and its gate weight replaces the logit at s_lg[t][e]
        if (wave < T) {
            const float *lg = s_lg + (size_t)wave * E;
            int *ii = s_ids + wave * K;
            float *ww = s_w + wave * K;
            uint32_t *tr = s_trash + wave * WAVE;
            if (K <= FROUNDS_MAX_K) {
                if (E <= 64) wave_topk_multi<1, 1, true>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
                else if (E <= 128) wave_topk_multi<2, 1, true>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
                else if (E <= 256) wave_topk_multi<4, 1, true>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
                else if (E <= 512) wave_topk_multi<8, 1, true>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
                else wave_topk_multi<16, 1, true>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
            } else {
                if (E <= 64) wave_topk_multi<1, 1, false>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
                else if (E <= 128) wave_topk_multi<2, 1, false>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
                else if (E <= 256) wave_topk_multi<4, 1, false>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
                else if (E <= 512) wave_topk_multi<8, 1, false>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
                else wave_topk_multi<16, 1, false>(lg, E, K, p.renorm, 1, ii, ww, s_sel, wave, tr);
            }
            // read back as the 32-bit words the top-k stored (other lanes of this wave wrote
            // them; a wave's LDS accesses complete in order)
            for (int j = lane; j < K; j += WAVE) {
                const int e = (int)reinterpret_cast<const uint32_t *>(ii)[j];
                const float wt = __uint_as_float(reinterpret_cast<const uint32_t *>(ww)[j]);
                s_lg[(size_t)wave * E + e] = wt;
                if (blockIdx.x == 0) {
                    if (p.ids_out) p.ids_out[wave * K + j] = e;
                    if (p.w_out) p.w_out[wave * K + j] = wt;
                }
            }
        }
        __syncthreads();
        // Grouping (wave 0) from the token masks: the active experts are those with a nonzero
        // mask, in ascending id; an expert's slots are its tokens in ascending order (slot
        // t*k+j ascends with t), so its count is the mask's popcount and its start the
        // exclusive prefix of the counts.
        if (wave == 0) {
            const uint64_t lt = lanemask_lt();
            int nact = 0, tot = 0;
            for (int e0 = 0; e0 < E; e0 += WAVE) {
                const int e = e0 + lane;
                const uint32_t m = e < E ? s_sel[e] : 0u;
                const int cnt = __popc(m);
                const uint64_t bal = __ballot(m != 0u);
                // inclusive prefix of the counts over the 64 lanes
                const int inc = (int)wave_incl_sum_u((uint32_t)cnt);
                if (m != 0u) {
                    const int dl = nact + __popcll(bal & lt);
                    const int start = tot + inc - cnt;
                    s_act_e[dl] = e;
                    s_act_start[dl] = start;
                    s_act_cnt[dl] = cnt;
                    uint32_t mm = m;
                    for (int c = 0; mm; ++c) {
                        const int t = __builtin_ctz(mm);
                        mm &= mm - 1;
                        s_tok[start + c] = t;
                        s_wq[start + c] = s_lg[(size_t)t * E + e];
                    }
                }
                nact += __popcll(bal);
                tot += __builtin_amdgcn_readlane(inc, WAVE - 1);
            }
            if (lane == 0) s_nact = nact;
        }
    }
    __syncthreads();
    const int U = s_nact;

    // ---- phase 2: gate/up + SwiGLU -> h' (next item's rows in flight while computing) -----
    // A wave's items are gw, gw + NW, ...  Each item's rows are fetched one item ahead.  The
    // loads are branch-free and the loop leaves before a fetch, never around one, so the
    // compiler's wait before an item's first use leaves the next item's loads in flight (a
    // load under a branch would make it wait for every load).
    {
        const int nch = H / F::EPC;
        const size_t xrow = (size_t)H * ab;
        const int nitems = U * I;
        uint4 gq[CG], uq[CG], gq2[CG], uq2[CG];
        uint32_t gs[CG], us[CG], gs2[CG], us2[CG];
        auto fetch = [&](int q, uint4 (&g)[CG], uint32_t (&gsc)[CG], uint4 (&u)[CG], uint32_t (&usc)[CG]) {
            const int uu = q / I, i = q - uu * I;
            const size_t rsel = (size_t)s_act_e[uu] * I + i;
            load_chunks<F, CG>(p.wg + rsel * nch * 16, F::SCALED ? p.sg + rsel * scale_row_bytes<F>(nch) : nullptr, nch,
                               lane, WAVE, g, gsc);
            load_chunks<F, CG>(p.wu + rsel * nch * 16, F::SCALED ? p.su + rsel * scale_row_bytes<F>(nch) : nullptr, nch,
                               lane, WAVE, u, usc);
        };
        auto consume = [&](int q, const uint4 (&g)[CG], const uint32_t (&gsc)[CG], const uint4 (&u)[CG],
                           const uint32_t (&usc)[CG]) {
            const int uu = q / I, i = q - uu * I;
            const int start = s_act_start[uu], cnt = s_act_cnt[uu];
#pragma unroll
            for (int c = 0; c < FMAX_T; ++c) {
                if (c < cnt) {
                    const uint8_t *xa = smem + (size_t)s_tok[start + c] * xrow;
                    const float gv = dpp_sum64(row_dot<F, CG>(g, gsc, xa, nch, lane, WAVE)) * p.tsg;
                    const float uv = dpp_sum64(row_dot<F, CG>(u, usc, xa, nch, lane, WAVE)) * p.tsu;
                    if (lane == 63)
                        store_act_sc1(p.hbuf, (size_t)(start + c) * I + i, s_wq[start + c] * swiglu(gv, uv), f32);
                }
            }
        };
        int q = gw;
        if (q < nitems) {
            fetch(q, gq, gs, uq, us);
            for (;;) {
                const int q2 = q + NW;
                if (q2 >= nitems) {
                    consume(q, gq, gs, uq, us);
                    break;
                }
                fetch(q2, gq2, gs2, uq2, us2);
                consume(q, gq, gs, uq, us);
                const int q3 = q2 + NW;
                if (q3 >= nitems) {
                    consume(q2, gq2, gs2, uq2, us2);
                    break;
                }
                fetch(q3, gq, gs, uq, us);
                consume(q2, gq2, gs2, uq2, us2);
                q = q3;
            }
        }
    }

    // ---- phase 3 set-up: down projection by (row tile, expert) --------------------------
    // A work-group owns tiles of DR consecutive output rows; its wave w takes the active
    // experts w, w+FWPB, ...  An item (tile, expert) is DR rows x I of Wd[e] (one
    // contiguous block) held in registers: lane group r (LR lanes) takes row r, each lane
    // NC of its 16-byte chunks, so a row's dot product is summed over LR lanes only.
    // Per-wave partial sums go to s_part by token and row, and the work-group adds the
    // FWPB partials in a fixed order at the end of each tile.  Two items are in flight,
    // both issued before the barrier wait.
    constexpr int DR_REG = ((CG >= 8 || F::SCALED) ? 8 : 16) / (CD >= 4 ? 4 : CD);   // register budget
    constexpr int DR = DR_REG > 8 ? 8 : DR_REG;                        // rows per tile
    constexpr int LR = WAVE / DR;                                      // lanes per row
    constexpr int NC = DR * CD;                                        // chunks per lane
    const int nchd = I / F::EPC;
    const int rr = lane / LR, li = lane % LR;
    const int ntile = (H + DR - 1) / DR;
    const int ntw = (int)blockIdx.x < ntile ? (ntile - 1 - (int)blockIdx.x) / G + 1 : 0;
    const int nexp = wave < U ? (U - 1 - wave) / FWPB + 1 : 0;
    const int total = ntw * nexp;
    uint4 dqa[NC], dqb[NC];
    uint32_t dsa[NC], dsb[NC];
    // Item sq of the wave is (tile j = sq / nexp, its k-th expert).  Loads are branch-free
    // (an item past the last reloads the last one; a wave with no items loads a row of the
    // first active expert), so the compiler's waits before an item leave the next one's
    // loads in flight.
    // the item's DR rows of Wd[e] are contiguous; one resource covers the rows below H
    // (lane group rr takes row rr, chunks past a row's end read as out of range)
    auto load_item = [&](int sq, uint4 (&dq)[NC], uint32_t (&ds)[NC]) {
        const bool any = total > 0;
        const int sqc = any ? min(sq, total - 1) : 0;
        const int j = any ? sqc / nexp : 0, k = any ? sqc - j * nexp : 0;
        const int n0 = ((int)blockIdx.x + G * j) * DR;
        const int rows = any ? min(DR, H - n0) : 0;
        const size_t rsel0 = (size_t)s_act_e[any ? wave + FWPB * k : 0] * H + (any ? n0 : 0);
        const rsrc_t rw = make_rsrc(p.wd + rsel0 * nchd * 16, (uint32_t)(rows * nchd * 16));
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int ch = li + LR * c;
            dq[c] = ld_rsrc16(rw, ch < nchd ? (uint32_t)(rr * nchd + ch) * 16 : kOutOfRange);
        }
        if constexpr (F::SCALED) {
            const uint32_t srb = (uint32_t)scale_row_bytes<F>(nchd);
            const rsrc_t rs = make_rsrc(p.sd + rsel0 * srb, (uint32_t)rows * srb);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int ch = li + LR * c;
                // chunk index rr * nchd + ch of the resource: its scale sits at row rr's scales
                ds[c] = load_scale_r<F>(rs, ch < nchd ? (uint32_t)(rr * nchd + ch) : kOutOfRange / 4);
            }
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) ds[c] = 0u;
        }
    };
    bar_arrive(p.flags, s_tag);
    load_item(0, dqa, dsa);
    if (total > 1) load_item(1, dqb, dsb);
    if (G <= 4 * WAVE)
        bar_wait<4>(p.flags, G, s_tag, p.err);
    else
        bar_wait<FMAX_G / WAVE>(p.flags, G, s_tag, p.err);
    if (blockIdx.x == 0 && tid == 0) __hip_atomic_fetch_add(p.bar, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // stage h' (all P slots, sorted order; P*I*ab is a multiple of 16) into LDS with
    // 16-byte loads past the non-coherent caches, eight in flight per thread
    {
        const uint32_t nb = (uint32_t)(P * I * ab);
        const int n16 = (int)(nb / 16);
        const rsrc_t hr = make_rsrc(p.hbuf, nb);
        uint4 *dst = reinterpret_cast<uint4 *>(smem);
        for (int i0 = tid; i0 < n16; i0 += 8 * FTHREADS) {
            uint4 v[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) v[b] = ld_rsrc16_agent(hr, (uint32_t)(i0 + b * FTHREADS) * 16);
            __builtin_amdgcn_sched_barrier(0);   // all eight loads before the first store
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int i = i0 + b * FTHREADS;
                if (i < n16) dst[i] = v[b];
            }
        }
    }
    __syncthreads();

    // ---- phase 3: down projection + weighted combine, by output row tile -------------------
    // Each wave adds its experts' contributions to its own partial sums of all the
    // work-group's rows (s_part[wave][token][row]); the work-group then adds the FWPB
    // partials in wave order and stores y once, after every item.
    {
        const size_t hrow = (size_t)I * ab;
        float *part = s_part + (size_t)wave * FMAX_T * FMAX_WR;
        auto consume = [&](int sq, const uint4 (&dq)[NC], const uint32_t (&ds)[NC]) {
            const int j = sq / nexp, k = sq - j * nexp;
            const int u = wave + FWPB * k;
            const int start = s_act_start[u], cnt = s_act_cnt[u];
            for (int c = 0; c < cnt; ++c) {
                const int q = start + c;
                const int t = s_tok[q];
                const uint8_t *ha = smem + (size_t)q * hrow;
                float d = row_dot<F, NC>(dq, ds, ha, nchd, li, LR);
                d = lane_group_sum<LR>(d) * p.tsd;
                if (li == LR - 1) atomicAdd(part + t * FMAX_WR + j * DR + rr, d);
            }
        };
        int sq = 0;
        for (; sq + 2 < total; sq += 2) {
            consume(sq, dqa, dsa);
            load_item(sq + 2, dqa, dsa);
            consume(sq + 1, dqb, dsb);
            load_item(sq + 3, dqb, dsb);
        }
        if (sq < total) consume(sq, dqa, dsa);
        if (sq + 1 < total) consume(sq + 1, dqb, dsb);
        __syncthreads();
        for (int i = tid; i < T * ntw * DR; i += FTHREADS) {
            const int t = i / (ntw * DR), jr = i - t * (ntw * DR);
            const int j = jr / DR, r = jr - j * DR;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < FWPB; ++w) v += s_part[((size_t)w * FMAX_T + t) * FMAX_WR + jr];
            const int n = ((int)blockIdx.x + G * j) * DR + r;
            if (n < H) {
                if (f32)
                    reinterpret_cast<float *>(p.y)[(size_t)t * H + n] = v;
                else
                    reinterpret_cast<uint16_t *>(p.y)[(size_t)t * H + n] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
    }
}

// dynamic LDS of the fused kernel: the staged x, the logits, the expert token masks, the
// per-wave discard words and the packed selection keys after it (phases 0-2), or the
// staged h' (phase 3)
static size_t fused_lds_bytes(const moe_shape &s) {
    const size_t xb = (size_t)s.num_tokens * s.hidden * act_bytes(s.act_dtype);
    const size_t front = ((xb + 15) & ~(size_t)15) + (((size_t)s.num_tokens * s.num_experts * 4 + 15) & ~(size_t)15) +
                         (size_t)((s.num_experts + 3) & ~3) * 4 + (size_t)FWPB * WAVE * 4 +
                         (size_t)s.num_experts * 8;
    return std::max(front, (size_t)s.num_tokens * s.top_k * s.intermediate * act_bytes(s.act_dtype));
}

// rows of the down projection's tiles that one work-group owns (at most FMAX_WR)
template <class F>
static int fused_wg_rows(const moe_shape &s, int G) {
    const int nchd = s.intermediate / F::EPC;
    const int lpr = nchd >= WAVE ? WAVE : (nchd >= 32 ? 32 : 16);
    const int cd = (nchd + lpr - 1) / lpr;
    const int cdb = cd <= 1 ? 1 : cd <= 2 ? 2 : cd <= 4 ? 4 : 8;
    const int cg = (s.hidden / F::EPC + WAVE - 1) / WAVE;
    const int dr_reg = ((cg > 4 || F::SCALED) ? 8 : 16) / (cdb >= 4 ? 4 : cdb);
    const int dr = dr_reg > 8 ? 8 : dr_reg;
    const int ntile = (s.hidden + dr - 1) / dr;
    return (ntile + G - 1) / G * dr;
}

// the number of work-groups the fused kernel runs on (one per compute unit), or 0
static int fused_grid() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                  hipSuccess)
        return 0;
    return cus;
}

static int fused_rows_for(const moe_shape &s, int G) {
    switch (s.weight_dtype) {
        case MOE_F32: return fused_wg_rows<FmtF32>(s, G);
        case MOE_BF16: return fused_wg_rows<FmtBF16>(s, G);
        case MOE_NVFP4: return fused_wg_rows<FmtNV4>(s, G);
        case MOE_MXINT8: return fused_wg_rows<FmtI8>(s, G);
        default: return fused_wg_rows<FmtMX4>(s, G);
    }
}

// true when the fused kernel covers this shape (otherwise the staged kernels run)
static bool fused_bucket_built(int cg, int cr, int cd);
static int bucket(int chunks_per_lane);

bool decode_fused_supported(const moe_shape &s) {
    const size_t P = (size_t)s.num_tokens * s.top_k;
    if (s.num_tokens < 1 || s.num_tokens > FMAX_T || P > FMAX_P) return false;
    const int epc = weight_chunk_elems(s.weight_dtype);
    const int aepc = s.act_dtype == MOE_F32 ? 4 : 8;
    if ((s.hidden / epc + WAVE - 1) / WAVE > FMAX_C) return false;          // gate/up rows
    if ((s.hidden / aepc + WAVE - 1) / WAVE > FMAX_C) return false;         // router rows
    const int nchd = s.intermediate / epc;
    const int lpr = nchd >= WAVE ? WAVE : (nchd >= 32 ? 32 : 16);
    if (nchd < 16 || (nchd + lpr - 1) / lpr > FMAX_C / 2) return false;    // down rows
    // the gfx950 parts have 256 compute units; the launch re-checks with the device's count
    if (fused_lds_bytes(s) > FLDS_MAX) return false;
    if (fused_rows_for(s, 256) > FMAX_WR) return false;
    if (s.num_experts > 1024) return false;
    return fused_bucket_built(bucket((s.hidden / epc + WAVE - 1) / WAVE), bucket((s.hidden / aepc + WAVE - 1) / WAVE),
                              bucket((nchd + lpr - 1) / lpr));
}

template <class F, class A, int CG, int CR, int CD>
static hipError_t fused_launch(const FusedParams &prm, size_t lds, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    auto kern = decode_fused_kernel<F, A, CG, CR, CD>;
    static bool attr_done = false;  // raising the dynamic-LDS cap is idempotent
    if (!attr_done) {
        hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)FLDS_MAX);
        if (r != hipSuccess) return r;
        attr_done = true;
    }
    if (ev0 || ev1) {
        hipExtLaunchKernelGGL(kern, dim3(prm.nblocks), dim3(FTHREADS), lds, st, ev0, ev1, 0, prm);
    } else {
        hipLaunchKernelGGL(kern, dim3(prm.nblocks), dim3(FTHREADS), lds, st, prm);
    }
    return hipGetLastError();
}

static int bucket(int chunks_per_lane) { return chunks_per_lane <= 1 ? 1 : chunks_per_lane <= 2 ? 2 : chunks_per_lane <= 4 ? 4 : 8; }

template <class F, class A>
static hipError_t fused_dispatch(const moe_shape &s, const FusedParams &prm, size_t lds, hipStream_t st,
                                 hipEvent_t ev0, hipEvent_t ev1) {
    const int cg = bucket((s.hidden / F::EPC + WAVE - 1) / WAVE);
    const int cr = bucket((s.hidden / A::EPC + WAVE - 1) / WAVE);
    const int nchd = s.intermediate / F::EPC;
    const int lpr = nchd >= WAVE ? WAVE : (nchd >= 32 ? 32 : 16);
    const int cd = bucket((nchd + lpr - 1) / lpr);
#define MOE_FL(CG, CR, CD) \
    if (cg == CG && cr == CR && cd == CD) return fused_launch<F, A, CG, CR, CD>(prm, lds, st, ev0, ev1)
    // (gate/up, router, down) chunk buckets of the supported shapes
    MOE_FL(4, 4, 2);   // H 2048 bf16, I 768..1024 bf16
    MOE_FL(4, 4, 1);
    MOE_FL(4, 4, 4);
    MOE_FL(2, 8, 1);   // H 4096 MXFP4 (router bf16), I 1024
    MOE_FL(2, 8, 2);
    MOE_FL(1, 4, 1);   // H 2048 MXFP4
    MOE_FL(1, 1, 1);   // H 256 fp32 / H 512 bf16, small I
    MOE_FL(1, 1, 2);
    MOE_FL(2, 2, 1);   // H 1024 bf16
    MOE_FL(2, 2, 2);
    MOE_FL(8, 8, 2);   // H 4096 bf16
    MOE_FL(8, 8, 4);
    MOE_FL(2, 4, 2);   // H 2048 MXINT8, I 768
    MOE_FL(4, 8, 1);   // H 4096 MXINT8, I 1024
#undef MOE_FL
    return hipErrorInvalidConfiguration;
}

// Every work-group of the fused kernel waits on the others, so all of them must be
// resident at once: one per compute unit.  Checked once per kernel instance at the largest
// LDS it may ask for (a work-group that fits then fits with less).
template <class F, class A, int CG, int CR, int CD>
static bool fused_fits_one() {
    static const bool ok = [] {
        auto kern = decode_fused_kernel<F, A, CG, CR, CD>;
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)FLDS_MAX) != hipSuccess)
            return false;
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, FTHREADS, FLDS_MAX) != hipSuccess) return false;
        return n >= 1;
    }();
    return ok;
}

template <class F, class A>
static bool fused_fits(const moe_shape &s) {
    const int cg = bucket((s.hidden / F::EPC + WAVE - 1) / WAVE);
    const int cr = bucket((s.hidden / A::EPC + WAVE - 1) / WAVE);
    const int nchd = s.intermediate / F::EPC;
    const int lpr = nchd >= WAVE ? WAVE : (nchd >= 32 ? 32 : 16);
    const int cd = bucket((nchd + lpr - 1) / lpr);
#define MOE_FF(CG, CR, CD) \
    if (cg == CG && cr == CR && cd == CD) return fused_fits_one<F, A, CG, CR, CD>()
    MOE_FF(4, 4, 2);
    MOE_FF(4, 4, 1);
    MOE_FF(4, 4, 4);
    MOE_FF(2, 8, 1);
    MOE_FF(2, 8, 2);
    MOE_FF(1, 4, 1);
    MOE_FF(1, 1, 1);
    MOE_FF(1, 1, 2);
    MOE_FF(2, 2, 1);
    MOE_FF(2, 2, 2);
    MOE_FF(8, 8, 2);
    MOE_FF(8, 8, 4);
    MOE_FF(2, 4, 2);
    MOE_FF(4, 8, 1);
#undef MOE_FF
    return false;
}

bool decode_fused_coresident(const moe_shape &s) {
    const int G = fused_grid();
    if (G <= 0) {
        (void)hipGetLastError();
        return true;   // no device: nothing will be launched
    }
    // the barrier's flag words and the output-row budget on this device's grid
    if (G > FMAX_G || fused_rows_for(s, G) > FMAX_WR) return false;
    switch (s.weight_dtype) {
        case MOE_F32: return fused_fits<FmtF32, FmtF32>(s);
        case MOE_BF16: return fused_fits<FmtBF16, FmtBF16>(s);
        case MOE_NVFP4: return fused_fits<FmtNV4, FmtBF16>(s);
        case MOE_MXINT8: return fused_fits<FmtI8, FmtBF16>(s);
        default: return fused_fits<FmtMX4, FmtBF16>(s);
    }
}

// (gate/up, router, down) chunk buckets the fused kernel is built for
static bool fused_bucket_built(int cg, int cr, int cd) {
    static const int combos[][3] = {{4, 4, 2}, {4, 4, 1}, {4, 4, 4}, {2, 8, 1}, {2, 8, 2}, {1, 4, 1},
                                    {1, 1, 1}, {1, 1, 2}, {2, 2, 1}, {2, 2, 2}, {8, 8, 2}, {8, 8, 4},
                                    {2, 4, 2}, {4, 8, 1}};
    for (const auto &c : combos)
        if (c[0] == cg && c[1] == cr && c[2] == cd) return true;
    return false;
}

hipError_t launch_decode_fused(const moe_shape &s, const void *x, const void *wr, const float *bias,
                               const moe_expert_weights &w, void *y, int32_t *ids_out, float *w_out, void *ws,
                               hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const WsLayout L = ws_layout(s);
    const int cus = fused_grid();
    if (cus <= 0) return hipErrorNoDevice;
    if (cus > FMAX_G || fused_rows_for(s, cus) > FMAX_WR) return hipErrorInvalidConfiguration;
    FusedParams prm{};
    prm.x = static_cast<const uint8_t *>(x);
    prm.wr = static_cast<const uint8_t *>(wr);
    prm.bias = bias;
    prm.wg = static_cast<const uint8_t *>(w.w_gate);
    prm.wu = static_cast<const uint8_t *>(w.w_up);
    prm.wd = static_cast<const uint8_t *>(w.w_down);
    prm.sg = w.s_gate;
    prm.su = w.s_up;
    prm.sd = w.s_down;
    const bool nv = s.weight_dtype == MOE_NVFP4;
    prm.tsg = nv ? w.ts_gate : 1.f;
    prm.tsu = nv ? w.ts_up : 1.f;
    prm.tsd = nv ? w.ts_down : 1.f;
    prm.y = static_cast<uint8_t *>(y);
    prm.ids_out = ids_out;
    prm.w_out = w_out;
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    prm.logits = reinterpret_cast<uint64_t *>(wsb + L.tagged);
    prm.hbuf = wsb + L.h;
    prm.bar = reinterpret_cast<uint64_t *>(wsb + L.ctrl + 8);
    prm.flags = reinterpret_cast<uint64_t *>(wsb + L.flags);
    prm.err = reinterpret_cast<int32_t *>(wsb + L.ctrl);
    prm.T = s.num_tokens;
    prm.H = s.hidden;
    prm.E = s.num_experts;
    prm.K = s.top_k;
    prm.I = s.intermediate;
    prm.renorm = s.renormalize ? 1 : 0;
    prm.nblocks = cus;
    const size_t lds = fused_lds_bytes(s);
    switch (s.weight_dtype) {
        case MOE_F32: return fused_dispatch<FmtF32, FmtF32>(s, prm, lds, st, ev0, ev1);
        case MOE_BF16: return fused_dispatch<FmtBF16, FmtBF16>(s, prm, lds, st, ev0, ev1);
        case MOE_NVFP4: return fused_dispatch<FmtNV4, FmtBF16>(s, prm, lds, st, ev0, ev1);
        case MOE_MXINT8: return fused_dispatch<FmtI8, FmtBF16>(s, prm, lds, st, ev0, ev1);
        default: return fused_dispatch<FmtMX4, FmtBF16>(s, prm, lds, st, ev0, ev1);
    }
}

}  // namespace moe
