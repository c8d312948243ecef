// group.hip -- token->expert grouping on the device ("第 9 章 prefill：最大的瓶颈"
// §9.9: the fused expert path groups by expert on the GPU instead of going
// back to the host every layer; §9.5: no entry is ever dropped).
//
// A stable counting sort of the slots t*k+j by expert id: per-expert counts,
// their exclusive prefix (expert_offsets), slots placed in ascending slot
// order inside each expert (sorted_slots) and the inverse map (slot_pos).
// The order comes from ballot ranks and a prefix over waves, never from
// atomics, so it is deterministic.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Block-wide exclusive scan of n (<= a few thousand) LDS ints in place;
// returns the total.  tmp holds blockDim.x ints.
__device__ int block_exclusive_scan(int *data, int n, int *tmp) {
    const int tid = threadIdx.x, nth = blockDim.x;
    const int per = (n + nth - 1) / nth;
    const int b = tid * per, e = min(n, b + per);
    int local = 0;
    for (int i = b; i < e; ++i) local += data[i];
    tmp[tid] = local;
    __syncthreads();
    for (int off = 1; off < nth; off <<= 1) {
        const int v = tid >= off ? tmp[tid - off] : 0;
        __syncthreads();
        tmp[tid] += v;
        __syncthreads();
    }
    const int total = tmp[nth - 1];
    int run = tmp[tid] - local;
    __syncthreads();
    for (int i = b; i < e; ++i) {
        const int c = data[i];
        data[i] = run;
        run += c;
    }
    __syncthreads();
    return total;
}

// Single work-group grouping.  LDS: cnt[E] running counts, wcnt[nw][E]
// per-wave counts of the current round, flags[E], tmp[blockDim].
__global__ __launch_bounds__(1024) void group_kernel(const int32_t *__restrict__ ids, int P, int E,
                                                     int32_t *__restrict__ offsets, int32_t *__restrict__ sorted,
                                                     int32_t *__restrict__ slot_pos, int32_t *__restrict__ active,
                                                     int32_t *__restrict__ err) {
    extern __shared__ int smem[];
    const int nth = blockDim.x, nw = nth / WAVE;
    int *cnt = smem;
    int *wcnt = cnt + E;
    int *flags = wcnt + nw * E;
    int *tmp = flags + E;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int e = tid; e < E; e += nth) cnt[e] = 0;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rounds = (P + nth - 1) / nth;
    for (int r = 0; r < rounds; ++r) {
        for (int i = tid; i < nw * E; i += nth) wcnt[i] = 0;
        __syncthreads();
        const int p = r * nth + tid;
        int id = p < P ? ids[p] : -1;
        const bool valid = p < P;
        const bool ok = valid && id >= 0 && id < E;
        if (valid && !ok) atomicOr(err, MOE_DEVERR_BAD_EXPERT_ID);
        if (!ok) id = 0;
        uint64_t match = __ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t bb = __ballot(ok && ((id >> b) & 1));
            match &= ((id >> b) & 1) ? bb : ~bb;
        }
        const int rank_w = __popcll(match & lt_mask);
        if (ok && rank_w == 0) wcnt[wave * E + id] = __popcll(match);
        __syncthreads();
        if (ok) {
            int pre = cnt[id];
            for (int w2 = 0; w2 < wave; ++w2) pre += wcnt[w2 * E + id];
            slot_pos[p] = pre + rank_w;  // rank inside the expert; made absolute below
        } else if (valid) {
            slot_pos[p] = -1;
        }
        __syncthreads();
        for (int e = tid; e < E; e += nth) {
            int s = 0;
            for (int w2 = 0; w2 < nw; ++w2) s += wcnt[w2 * E + e];
            cnt[e] += s;
        }
        __syncthreads();
    }
    // flags of nonempty experts, then both scans
    for (int e = tid; e < E; e += nth) flags[e] = cnt[e] > 0 ? 1 : 0;
    __syncthreads();
    const int total = block_exclusive_scan(cnt, E, tmp);
    const int nact = block_exclusive_scan(flags, E, tmp);
    for (int e = tid; e < E; e += nth) {
        offsets[e] = cnt[e];
        const int next = (e + 1 < E) ? cnt[e + 1] : total;
        if (next > cnt[e]) active[1 + flags[e]] = e;
    }
    if (tid == 0) {
        offsets[E] = total;
        active[0] = nact;
    }
    for (int r = 0; r < rounds; ++r) {
        const int p = r * nth + tid;
        if (p < P) {
            const int id = ids[p];
            if (id >= 0 && id < E) {
                const int pos = cnt[id] + slot_pos[p];
                sorted[pos] = p;
                slot_pos[p] = pos;
            }
        }
    }
    // positions past the grouped slots (only when ids were rejected)
    for (int q = total + tid; q < P; q += nth) sorted[q] = -1;
}

// active list from existing offsets: [count, nonempty experts ascending]
__global__ __launch_bounds__(1024) void active_kernel(const int32_t *__restrict__ offsets, int E,
                                                      int32_t *__restrict__ active) {
    extern __shared__ int smem[];
    int *flags = smem;
    int *tmp = flags + E;
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int e = tid; e < E; e += nth) flags[e] = offsets[e + 1] > offsets[e] ? 1 : 0;
    __syncthreads();
    const int nact = block_exclusive_scan(flags, E, tmp);
    for (int e = tid; e < E; e += nth)
        if (offsets[e + 1] > offsets[e]) active[1 + flags[e]] = e;
    if (tid == 0) active[0] = nact;
}

hipError_t launch_group(const moe_shape &s, const int32_t *ids, int32_t *offsets, int32_t *sorted,
                        int32_t *slot_pos, int32_t *active, int32_t *err, hipStream_t st) {
    const int E = s.num_experts;
    const int P = s.num_tokens * s.top_k;
    // LDS budget 64 KB: (2 + nw) * E ints + nth ints
    int nw = 16;
    while (nw > 1 && ((size_t)(2 + nw) * E + nw * WAVE) * 4 > 65536) nw >>= 1;
    const int nth = nw * WAVE;
    const size_t lds = ((size_t)(2 + nw) * E + nth) * 4;
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(nth), lds, st, ids, P, E, offsets, sorted, slot_pos, active,
                       err);
    return hipGetLastError();
}

hipError_t launch_active(const moe_shape &s, const int32_t *offsets, int32_t *active, hipStream_t st) {
    const int E = s.num_experts;
    const int nth = 1024;
    hipLaunchKernelGGL(active_kernel, dim3(1), dim3(nth), (size_t)(E + nth) * 4, st, offsets, E, active);
    return hipGetLastError();
}

}  // namespace moe
