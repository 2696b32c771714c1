// step_prep.hip -- one step's attention inputs built on the GPU from a
// persistent per-request state table (Model Runner V2 page, "better
// persistent batch and GPU-native input preparation": each active request
// keeps a stable row of a fixed-size state table, and each step gathers the
// step's inputs in the current request order, on the device, with no
// host-device synchronisation -- the scheduled token counts may themselves be
// a device-side result such as the accepted counts of speculative decoding).
//
// For batch entry i with state row r = idx_mapping[i] and n_i scheduled
// tokens: query_start_loc is the running sum of the n_i (cut at the outputs'
// capacity), seq_lens[i] = num_computed[r] + n_i, block_tables[i] is row r of
// the state's block table, and new token k of entry i sits at position
// num_computed[r] + k, reads its input id from the state's token ids and its
// KV slot from the block table.  Rows past the step's tokens are padding
// (slot -1, which the append skips).
//
// One launch.  Every workgroup loads the batch's (row, count, computed)
// triples into LDS and scans the counts itself, so no workgroup waits for
// another; then the workgroups share out the token rows (each finds its
// entry by binary search over the scan) and the block-table gather.  The
// work is a few KB: launch latency bounds it.
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kPrepThreads = 256;

__device__ __forceinline__ int64_t block_incl_scan(int64_t x, int64_t *warp_tot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        warp_tot[wave] = x;
    __syncthreads();
    int64_t before = 0;
    for (int w = 0; w < wave; ++w)
        before += warp_tot[w];
    __syncthreads();
    return x + before;
}

__global__ __launch_bounds__(kPrepThreads) void step_prep_kernel(StepPrepArgs a)
{
    __shared__ int32_t s_row[kMaxPrepReqs];
    __shared__ int32_t s_comp[kMaxPrepReqs];
    __shared__ int64_t s_qsl[kMaxPrepReqs + 1];   // running sums, cut at capacity
    __shared__ int64_t s_tot[kPrepThreads / 64];
    __shared__ int64_t s_carry;

    const int t = threadIdx.x;
    const int S = a.num_reqs;
    const bool lead = blockIdx.x == 0;

    // entries, validated: a bad entry schedules nothing and gathers no row
    if (t == 0) {
        s_carry = 0;
        s_qsl[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < S; base += kPrepThreads) {
        const int i = base + t;
        int64_t n = 0;
        if (i < S) {
            const int r = a.idx_mapping[i];
            int32_t sched = a.num_scheduled[i];
            bool ok = r >= 0 && r < a.num_rows && sched >= 0;
            const int32_t comp = ok ? a.num_computed[r] : 0;
            ok = ok && comp >= 0;
            if (!ok && lead)
                raise_flag(a.err_flag, PA_DEVERR_STEP);
            s_row[i] = ok ? r : -1;
            s_comp[i] = comp;
            n = ok ? sched : 0;
        }
        const int64_t incl = block_incl_scan(n, s_tot) + s_carry;
        if (i < S)
            s_qsl[i + 1] = min(incl, (int64_t)a.max_tokens);
        __syncthreads();
        if (t == kPrepThreads - 1)
            s_carry = incl;
        __syncthreads();
    }
    const int64_t total = s_qsl[S];
    if (lead && t == 0 && s_carry > a.max_tokens)
        raise_flag(a.err_flag, PA_DEVERR_STEP);

    if (lead) {
        for (int i = t; i <= S; i += kPrepThreads)
            a.query_start_loc[i] = (int32_t)s_qsl[i];
        for (int i = t; i < S; i += kPrepThreads)
            a.seq_lens[i] = s_row[i] < 0 ? 0 : s_comp[i] + (int32_t)(s_qsl[i + 1] - s_qsl[i]);
    }

    // token rows (padding beyond the step's tokens)
    const int64_t stride = (int64_t)gridDim.x * kPrepThreads;
    for (int64_t tok = (int64_t)blockIdx.x * kPrepThreads + t; tok < a.max_tokens; tok += stride) {
        int64_t pos = 0, slot = -1;
        int32_t id = 0;
        if (tok < total) {
            // entry i: the last with s_qsl[i] <= tok (entries without tokens are skipped over)
            int lo = 0, hi = S;                 // s_qsl[lo] <= tok < s_qsl[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_qsl[mid] <= tok)
                    lo = mid;
                else
                    hi = mid;
            }
            const int r = s_row[lo];
            pos = s_comp[lo] + (tok - s_qsl[lo]);
            if (pos < a.max_len)
                id = a.token_ids[(int64_t)r * a.max_len + pos];
            else
                raise_flag(a.err_flag, PA_DEVERR_STEP);
            const int64_t j = pos / a.block_size;
            if (j < a.max_blocks) {
                const int32_t b = a.block_table[(int64_t)r * a.max_blocks + j];
                if (b >= 0 && b < a.num_blocks)
                    slot = (int64_t)b * a.block_size + pos % a.block_size;
                else
                    raise_flag(a.err_flag, PA_DEVERR_BLOCK_ID);
            } else {
                raise_flag(a.err_flag, PA_DEVERR_STEP);
            }
        }
        a.positions[tok] = pos;
        a.input_ids[tok] = id;
        a.slot_mapping[tok] = slot;
    }

    // ordered block tables
    const int64_t cells = (int64_t)S * a.max_blocks;
    for (int64_t e = (int64_t)blockIdx.x * kPrepThreads + t; e < cells; e += stride) {
        const int i = (int)(e / a.max_blocks), j = (int)(e % a.max_blocks);
        const int r = s_row[i];
        a.block_tables[e] = r < 0 ? -1 : a.block_table[(int64_t)r * a.max_blocks + j];
    }
}

}  // namespace

hipError_t launch_step_prep(const StepPrepArgs &a, hipStream_t stream)
{
    if (a.num_reqs > kMaxPrepReqs)
        return hipErrorInvalidValue;
    const int64_t work = a.max_tokens > (int64_t)a.num_reqs * a.max_blocks
                             ? a.max_tokens
                             : (int64_t)a.num_reqs * a.max_blocks;
    int64_t wgs = (work + 4 * kPrepThreads - 1) / (4 * kPrepThreads);
    wgs = wgs < 1 ? 1 : (wgs > 512 ? 512 : wgs);
    hipLaunchKernelGGL(step_prep_kernel, dim3((unsigned)wgs), dim3(kPrepThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
