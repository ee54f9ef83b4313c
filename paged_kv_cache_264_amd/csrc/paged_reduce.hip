// Merge of split-context partial softmax results.
//
// A partition p of a sequence carries its max score m_p (natural-log units),
// l_p = sum exp(s - m_p) and o_p = sum exp(s - m_p) v / l_p.  The exact merge
// is the running-max / running-sum rule of online softmax (caojiahao2.github.io
// section 3.2) applied to whole partitions:
//     M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// One work-group per (sequence, q head); the weights are computed once into
// LDS, then the threads split the partitions' rows between them.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kReduceThreads = 256;
constexpr int kWeightChunk = 1024;  // partitions whose weights sit in LDS at once

template <Elem OE, int D>
__global__ __launch_bounds__(kReduceThreads) void paged_reduce_kernel(ReduceArgs a) {
    __shared__ float s_w[kWeightChunk];
    __shared__ float s_red[kReduceThreads / kWave];

    const int bh = blockIdx.x;
    const int row = bh / a.num_q_heads;
    int b = row;
    if (a.query_start_loc) {  // sequence of query token `row`: binary search
        int lo = 0, hi = a.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.query_start_loc[mid] <= row) lo = mid; else hi = mid - 1;
        }
        b = lo;
    }
    const int tid = threadIdx.x;
    const int P = a.partition_size;
    int n = a.context_lens[b];
    n = n < 0 ? 0 : n;
    int n_parts = partition_count(n - window_base(n, a.window), P);
    n_parts = n_parts > a.num_partitions ? a.num_partitions : n_parts;

    if (a.skip_single && n_parts <= 1) return;  // phase 1 wrote these outputs
    if (n_parts == 0) {
        for (int d = tid; d < D; d += kReduceThreads) store_elem<OE>(a.out, (size_t)bh * D + d, 0.f);
        return;
    }

    const float* mp = a.m_part + (size_t)bh * a.num_partitions;
    const float* lp = a.l_part + (size_t)bh * a.num_partitions;
    const float* op = a.o_part + (size_t)bh * a.num_partitions * D;

    // M = max over partitions (block-wide)
    float M = -3.0e38f;
    for (int p = tid; p < n_parts; p += kReduceThreads) M = fmaxf(M, mp[p]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if ((tid & 63) == 0) s_red[tid >> 6] = M;
    __syncthreads();
    M = s_red[0];
#pragma unroll
    for (int w = 1; w < kReduceThreads / kWave; ++w) M = fmaxf(M, s_red[w]);

    // sum_p w_p o_p over all threads: CPL = D / 4 threads read one partition's
    // row as 16-byte pieces, RP = 256 / CPL rows side by side, four rows in
    // flight per thread; the RP row groups then meet in LDS.
    constexpr int CPL = D / 4;
    constexpr int RP = kReduceThreads / CPL;
    static_assert(CPL * RP == kReduceThreads, "rows must tile the work-group");
    __shared__ float4 s_o[kReduceThreads];
    __shared__ float s_ws[RP];
    const int c4 = tid % CPL, r0 = tid / CPL;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
    auto add_row = [&](float w, const float4& x) {
        acc.x = fmaf(w, x.x, acc.x);
        acc.y = fmaf(w, x.y, acc.y);
        acc.z = fmaf(w, x.z, acc.z);
        acc.w = fmaf(w, x.w, acc.w);
        wsum += w;
    };
    for (int c0 = 0; c0 < n_parts; c0 += kWeightChunk) {
        const int c1 = min(n_parts, c0 + kWeightChunk);
        __syncthreads();
        for (int p = c0 + tid; p < c1; p += kReduceThreads)
            s_w[p - c0] = lp[p] * fast_exp2((mp[p] - M) * kLog2e);
        __syncthreads();
        int p = c0 + r0;
        for (; p + 3 * RP < c1; p += 4 * RP) {
            float4 x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                x[k] = *reinterpret_cast<const float4*>(op + (size_t)(p + k * RP) * D + 4 * c4);
#pragma unroll
            for (int k = 0; k < 4; ++k) add_row(s_w[p + k * RP - c0], x[k]);
        }
        for (; p < c1; p += RP)
            add_row(s_w[p - c0], *reinterpret_cast<const float4*>(op + (size_t)p * D + 4 * c4));
    }
    s_o[tid] = acc;
    if (c4 == 0) s_ws[r0] = wsum;
    __syncthreads();
    if (tid < CPL) {
        float4 o = s_o[tid];
        float W = s_ws[0];
#pragma unroll
        for (int r = 1; r < RP; ++r) {
            const float4 x = s_o[r * CPL + tid];
            o.x += x.x;
            o.y += x.y;
            o.z += x.z;
            o.w += x.w;
            W += s_ws[r];
        }
        const size_t d0 = (size_t)bh * D + 4 * tid;
        store_elem<OE>(a.out, d0 + 0, o.x / W);
        store_elem<OE>(a.out, d0 + 1, o.y / W);
        store_elem<OE>(a.out, d0 + 2, o.z / W);
        store_elem<OE>(a.out, d0 + 3, o.w / W);
    }
}

template <Elem OE>
hipError_t launch_d(const ReduceArgs& a, int d, hipStream_t s) {
    const int64_t n_wg = (int64_t)a.num_rows * a.num_q_heads;
    if (n_wg == 0) return hipSuccess;
    if (n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)n_wg), block(kReduceThreads);
    switch (d) {
    case 64: hipLaunchKernelGGL((paged_reduce_kernel<OE, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((paged_reduce_kernel<OE, 128>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((paged_reduce_kernel<OE, 256>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_reduce(const ReduceArgs& a, int out_dtype, int head_dim,
                               hipStream_t stream) {
    switch (static_cast<Elem>(out_dtype)) {
    case Elem::F32: return launch_d<Elem::F32>(a, head_dim, stream);
    case Elem::F16: return launch_d<Elem::F16>(a, head_dim, stream);
    case Elem::BF16: return launch_d<Elem::BF16>(a, head_dim, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
