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

// Block-wide exclusive scan of n (<= a few thousand) LDS ints in place; returns the
// total.  Each thread sums a run of consecutive entries, the runs are scanned inside
// each wave with DPP row shifts and across the (<= 16) waves by the first wave, and each
// thread then rewrites its run: two work-group barriers in all.  tmp holds blockDim.x
// ints (only the first 32 are used).
__device__ int block_exclusive_scan(int *data, int n, int *tmp) {
    const int tid = threadIdx.x, nth = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nw = (nth + 63) >> 6;
    const int per = (n + nth - 1) / nth;
    const int b = min(n, tid * per), e = min(n, b + per);
    int local = 0;
    for (int i = b; i < e; ++i) local += data[i];
    const int incl = (int)wave_incl_sum_u((uint32_t)local);
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int wt = lane < nw ? tmp[lane] : 0;
        const int wi = (int)wave_incl_sum_u((uint32_t)wt);
        if (lane < nw) tmp[16 + lane] = wi - wt;   // exclusive wave offsets
        if (lane == nw - 1) tmp[32] = wi;          // total
    }
    __syncthreads();
    int run = tmp[16 + wave] + incl - local;
    const int total = tmp[32];
    for (int i = b; i < e; ++i) {
        const int c = data[i];
        data[i] = run;
        run += c;
    }
    __syncthreads();
    return total;
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

// Block-wide tail of the grouping, run by every thread of one block: tot[E] holds the
// exclusive expert offsets, flags[E] marks the nonempty experts (both LDS), total is
// the number of grouped slots.  Writes the offsets, -1 into the unused tail of sorted,
// the list of nonempty experts and, when asked, the m-tile offsets and tile table of
// the grouped GEMM (tiles of mtile_rows rows).
__device__ void finish_grouping(int *tot, int *flags, int *tmp, int total, int E, int P, int32_t *__restrict__ offsets,
                                int32_t *__restrict__ sorted, int32_t *__restrict__ active,
                                int32_t *__restrict__ mtile_off, int4 *__restrict__ tiles, int mtile_rows) {
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int e = tid; e < E; e += nth) offsets[e] = tot[e];
    if (tid == 0) offsets[E] = total;
    for (int q = total + tid; q < P; q += nth) sorted[q] = -1;
    // nonempty experts, ascending
    const int nact = block_exclusive_scan(flags, E, tmp);
    for (int e = tid; e < E; e += nth) {
        const int next = (e + 1 < E) ? tot[e + 1] : total;
        if (next > tot[e]) active[1 + flags[e]] = e;
    }
    if (tid == 0) active[0] = nact;
    if (mtile_off) {
        __syncthreads();
        for (int e = tid; e < E; e += nth) {
            const int next = (e + 1 < E) ? tot[e + 1] : total;
            flags[e] = (next - tot[e] + mtile_rows - 1) / mtile_rows;
        }
        __syncthreads();
        const int nt = block_exclusive_scan(flags, E, tmp);
        for (int e = tid; e < E; e += nth) {
            mtile_off[e] = flags[e];
            if (!tiles) continue;
            const int next = (e + 1 < E) ? tot[e + 1] : total;
            const int t_end = (e + 1 < E) ? flags[e + 1] : nt;
            for (int t = flags[e]; t < t_end; ++t) tiles[t] = make_int4(tot[e] + (t - flags[e]) * mtile_rows, next, e, 0);
        }
        if (tid == 0) mtile_off[E] = nt;
    }
}

// ---- multi-block grouping: per-chunk stable ranks, then a scan and a scatter ---------------

// Block b takes slots [b*chunk, (b+1)*chunk): ballot-matched stable ranks inside the
// chunk (written to slot_pos, made absolute by the scatter) and per-expert counts of
// the chunk (counts[b][E]).
__device__ __forceinline__ void group_count_body(const int32_t *__restrict__ ids, int P, int E, int chunk,
                                                 int32_t *__restrict__ counts, int32_t *__restrict__ slot_pos,
                                                 int32_t *__restrict__ err, int blk, int *smem) {
    const int nth = blockDim.x, nw = nth / WAVE;
    int *cnt = smem;
    int *wcnt = cnt + E;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int e = tid; e < E; e += nth) cnt[e] = 0;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int c0 = blk * chunk, c1 = min(P, c0 + chunk);
    const int rounds = (c1 - c0 + nth - 1) / nth;
    for (int r = 0; r < rounds; ++r) {
        for (int i = tid; i < nw * E; i += nth) wcnt[i] = 0;
        __syncthreads();
        const int p = c0 + r * nth + tid;
        int id = p < c1 ? ids[p] : -1;
        const bool valid = p < c1;
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
            slot_pos[p] = pre + rank_w;
        } else if (valid) {
            slot_pos[p] = -1;
        }
        __syncthreads();
        for (int e = tid; e < E; e += nth) {
            int sum = 0;
            for (int w2 = 0; w2 < nw; ++w2) sum += wcnt[w2 * E + e];
            cnt[e] += sum;
        }
        __syncthreads();
    }
    for (int e = tid; e < E; e += nth) counts[(size_t)blk * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void group_count_kernel(const int32_t *__restrict__ ids, int P, int E, int chunk,
                                                           int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ slot_pos, int32_t *__restrict__ err) {
    extern __shared__ int smem[];
    group_count_body(ids, P, E, chunk, counts, slot_pos, err, blockIdx.x, smem);
}

// Every block rebuilds the expert offsets from the chunk counts (exclusive scan of the
// totals) and its own base per expert (offset + counts of the earlier chunks), then
// places its chunk's slots.  Block 0 also writes the offsets, the list of nonempty
// experts and, when asked, the m-tile offsets of the grouped GEMM (tiles of mtile_rows).
__device__ __forceinline__ void group_scatter_body(const int32_t *__restrict__ ids, int P, int E, int chunk, int nb,
                                                   const int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ sorted, int32_t *__restrict__ slot_pos,
                                                   int32_t *__restrict__ active, int32_t *__restrict__ mtile_off,
                                                   int4 *__restrict__ tiles, int mtile_rows, int blk, int *smem) {
    const int nth = blockDim.x;
    int *tot = smem;            // [E] totals, then exclusive offsets
    int *base = tot + E;        // [E] this block's base
    int *flags = base + E;      // [E]
    int *tmp = flags + E;       // [nth]
    const int tid = threadIdx.x, b = blk;
    for (int e = tid; e < E; e += nth) {
        int t = 0, pre = 0;
        for (int b2 = 0; b2 < nb; ++b2) {
            const int c = counts[(size_t)b2 * E + e];
            t += c;
            pre += b2 < b ? c : 0;
        }
        tot[e] = t;
        base[e] = pre;
        flags[e] = t > 0 ? 1 : 0;
    }
    __syncthreads();
    const int total = block_exclusive_scan(tot, E, tmp);
    for (int e = tid; e < E; e += nth) base[e] += tot[e];
    __syncthreads();
    const int c0 = b * chunk, c1 = min(P, c0 + chunk);
    for (int p = c0 + tid; p < c1; p += nth) {
        const int id = ids[p];
        if (id >= 0 && id < E) {
            const int pos = base[id] + slot_pos[p];
            sorted[pos] = p;
            slot_pos[p] = pos;
        }
    }
    if (b != 0) return;
    finish_grouping(tot, flags, tmp, total, E, P, offsets, sorted, active, mtile_off, tiles, mtile_rows);
}

__global__ __launch_bounds__(1024) void group_scatter_kernel(const int32_t *__restrict__ ids, int P, int E, int chunk,
                                                             int nb, const int32_t *__restrict__ counts,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ sorted,
                                                             int32_t *__restrict__ slot_pos,
                                                             int32_t *__restrict__ active,
                                                             int32_t *__restrict__ mtile_off,
                                                             int4 *__restrict__ tiles, int mtile_rows) {
    extern __shared__ int smem[];
    group_scatter_body(ids, P, E, chunk, nb, counts, offsets, sorted, slot_pos, active, mtile_off, tiles, mtile_rows,
                       blockIdx.x, smem);
}

// All slots in one chunk: the count and the scatter of the two-kernel grouping run in
// one work-group (the chunk's counts pass through global memory inside the work-group).
__global__ __launch_bounds__(1024) void group_single_kernel(const int32_t *__restrict__ ids, int P, int E,
                                                            int32_t *__restrict__ counts,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ sorted,
                                                            int32_t *__restrict__ slot_pos,
                                                            int32_t *__restrict__ active,
                                                            int32_t *__restrict__ mtile_off, int4 *__restrict__ tiles,
                                                            int mtile_rows, int32_t *__restrict__ err) {
    extern __shared__ int smem[];
    group_count_body(ids, P, E, P, counts, slot_pos, err, 0, smem);
    __syncthreads();
    group_scatter_body(ids, P, E, P, 1, counts, offsets, sorted, slot_pos, active, mtile_off, tiles, mtile_rows, 0,
                       smem);
}

// ---- grouping from the router's per-block counts -----------------------------------------

// One block: counts[b][e] (slots of router block b that chose e) become the base of
// router block b inside expert e's group, offsets[e] + sum over b' < b of counts[b'][e];
// then the offsets, active list and tile table as above.  nsub = blockDim.x / E threads
// per expert each take a contiguous range of router blocks.
__global__ __launch_bounds__(1024) void group_scan_kernel(int32_t *__restrict__ counts, int nb, int E, int P,
                                                          int32_t *__restrict__ offsets, int32_t *__restrict__ sorted,
                                                          int32_t *__restrict__ active, int32_t *__restrict__ mtile_off,
                                                          int4 *__restrict__ tiles, int mtile_rows) {
    extern __shared__ int smem[];
    const int nth = blockDim.x, tid = threadIdx.x;
    const int nsub = nth / E;
    int *tot = smem;            // [E]
    int *flags = tot + E;       // [E]
    int *tmp = flags + E;       // [nth]
    int *part = tmp + nth;      // [nsub][E]
    const int sub = tid / E, e = tid % E;
    const bool mine = sub < nsub;
    const int per = (nb + nsub - 1) / nsub;
    const int b0 = min(nb, sub * per), b1 = min(nb, b0 + per);
    // the thread's counts are loaded in batches of SCAN_BATCH independent loads (kept in
    // registers for the second pass when the whole range fits one batch)
    constexpr int SCAN_BATCH = 32;
    int cv[SCAN_BATCH];
    if (mine) {
        int local = 0;
        for (int b = b0; b < b1; b += SCAN_BATCH) {
#pragma unroll
            for (int j = 0; j < SCAN_BATCH; ++j) cv[j] = b + j < b1 ? counts[(size_t)(b + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < SCAN_BATCH; ++j) local += cv[j];
        }
        part[sub * E + e] = local;
    }
    __syncthreads();
    for (int x = tid; x < E; x += nth) {
        int t = 0;
        for (int s2 = 0; s2 < nsub; ++s2) t += part[s2 * E + x];
        tot[x] = t;
        flags[x] = t > 0 ? 1 : 0;
    }
    __syncthreads();
    const int total = block_exclusive_scan(tot, E, tmp);
    if (mine) {
        int base = tot[e];
        for (int s2 = 0; s2 < sub; ++s2) base += part[s2 * E + e];
        for (int b = b0; b < b1; b += SCAN_BATCH) {
            if (b1 - b0 > SCAN_BATCH) {
#pragma unroll
                for (int j = 0; j < SCAN_BATCH; ++j) cv[j] = b + j < b1 ? counts[(size_t)(b + j) * E + e] : 0;
            }
#pragma unroll
            for (int j = 0; j < SCAN_BATCH; ++j) {
                if (b + j < b1) counts[(size_t)(b + j) * E + e] = base;
                base += cv[j];
            }
        }
    }
    finish_grouping(tot, flags, tmp, total, E, P, offsets, sorted, active, mtile_off, tiles, mtile_rows);
}

// Slot p of router block b = (p / k) / rows: position = base[b][e] + rank of p inside
// the block (slot_pos holds the rank on entry and the position on exit).
__global__ __launch_bounds__(256) void group_place_kernel(const int32_t *__restrict__ ids, int P, int k, int rows,
                                                          int E, const int32_t *__restrict__ base,
                                                          int32_t *__restrict__ slot_pos,
                                                          int32_t *__restrict__ sorted) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    const int id = ids[p];
    const int b = (p / k) / rows;
    const int pos = base[(size_t)b * E + id] + slot_pos[p];
    sorted[pos] = p;
    slot_pos[p] = pos;
}

hipError_t launch_group_from_router(const moe_shape &s, const int32_t *ids, int32_t *counts, int32_t *offsets,
                                    int32_t *sorted, int32_t *slot_pos, int32_t *active, int32_t *mtile_off,
                                    int32_t *tiles, int mtile_rows, hipStream_t st) {
    const int E = s.num_experts, P = s.num_tokens * s.top_k;
    const int nb = (s.num_tokens + kRouterRows - 1) / kRouterRows;
    const int nth = 1024;
    const int nsub = nth / E;
    hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(nth), (size_t)(2 * E + nth + nsub * E) * 4, st, counts, nb, E,
                       P, offsets, sorted, active, mtile_off, mtile_off ? reinterpret_cast<int4 *>(tiles) : nullptr,
                       mtile_rows);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL(group_place_kernel, dim3((P + 255) / 256), dim3(256), 0, st, ids, P, s.top_k, kRouterRows, E,
                       counts, slot_pos, sorted);
    return hipGetLastError();
}

constexpr int GROUP_CHUNK = 4096;

int group_chunks(int P) { return P > 0 ? (P + GROUP_CHUNK - 1) / GROUP_CHUNK : 1; }

hipError_t launch_group2(const moe_shape &s, const int32_t *ids, int32_t *offsets, int32_t *sorted, int32_t *slot_pos,
                         int32_t *active, int32_t *counts, int32_t *mtile_off, int32_t *tiles, int mtile_rows,
                         int32_t *err, hipStream_t st) {
    const int E = s.num_experts;
    const int P = s.num_tokens * s.top_k;
    const int nb = group_chunks(P);
    int nw = 16;
    while (nw > 1 && ((size_t)(1 + nw) * E) * 4 > 65536) nw >>= 1;
    if (nb == 1) {
        const size_t lds = std::max((size_t)(1 + nw) * E, (size_t)3 * E + nw * WAVE) * 4;
        hipLaunchKernelGGL(group_single_kernel, dim3(1), dim3(nw * WAVE), lds, st, ids, P, E, counts, offsets, sorted,
                           slot_pos, active, mtile_off, mtile_off ? reinterpret_cast<int4 *>(tiles) : nullptr,
                           mtile_rows, err);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(group_count_kernel, dim3(nb), dim3(nw * WAVE), (size_t)(1 + nw) * E * 4, st, ids, P, E,
                       GROUP_CHUNK, counts, slot_pos, err);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess) return r;
    const int nth = 1024;
    hipLaunchKernelGGL(group_scatter_kernel, dim3(nb), dim3(nth), (size_t)(3 * E + nth) * 4, st, ids, P, E, GROUP_CHUNK,
                       nb, counts, offsets, sorted, slot_pos, active, mtile_off,
                       mtile_off ? reinterpret_cast<int4 *>(tiles) : nullptr, mtile_rows);
    return hipGetLastError();
}

hipError_t launch_active(const moe_shape &s, const int32_t *offsets, int32_t *active, hipStream_t st) {
    const int E = s.num_experts;
    const int nth = 1024;
    hipLaunchKernelGGL(active_kernel, dim3(1), dim3(nth), (size_t)(E + nth) * 4, st, offsets, E, active);
    return hipGetLastError();
}

}  // namespace moe
