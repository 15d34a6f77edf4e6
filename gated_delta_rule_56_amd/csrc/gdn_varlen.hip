// Tables of packed sequences: B sequences laid end to end in one token axis, sequence i
// holding tokens cu_seqlens[i] .. cu_seqlens[i + 1]. Each sequence starts a new chunk, so
// sequence i owns workspace chunks chunk0_i .. chunk0_i + ceil(len_i / C) - 1, where chunk0 is
// the running sum of the chunk counts.
//
// The tables are built on the GPU from the caller's device array, so the host needs no copy
// of the lengths. The entries are made safe for any cu_seqlens: every bound is clamped into
// [0, T] and every length to >= 0, and chunks beyond the workspace's chunk count are cut, so
// that no kernel reading the tables leaves its buffers (valid input is never changed by this).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 1024;

// one workgroup: sequence table {first token, tokens, first chunk, 0} by a block-wide scan of
// the chunk counts, in passes of kThreads sequences
__global__ __launch_bounds__(kThreads) void gdn_varlen_seq_kernel(const int32_t *cu, int32_t nseq, int32_t T,
                                                                  int32_t C, int32_t nchunks, int32_t *seqs) {
    __shared__ int32_t part[kThreads / 64];
    __shared__ int32_t carry;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < nseq; base += kThreads) {
        const int i = base + tid;
        int lo = 0, len = 0, nck = 0;
        if (i < nseq) {
            lo = min(max(cu[i], 0), T);
            const int hi = min(max(cu[i + 1], lo), T);
            len = hi - lo;
            nck = (len + C - 1) / C;
        }
        // inclusive scan of nck over the workgroup
        int x = nck;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) part[w] = x;
        __syncthreads();
        int before = carry;
        for (int j = 0; j < w; ++j) before += part[j];
        const int chunk0 = before + x - nck;
        if (i < nseq) {
            int keep = len;
            if (chunk0 >= nchunks) keep = 0;  // past the workspace: cut (never for valid input)
            else if (chunk0 + nck > nchunks) keep = min(len, (nchunks - chunk0) * C);
            int32_t *e = seqs + 4 * i;
            e[0] = lo;
            e[1] = keep;
            e[2] = min(chunk0, nchunks);
            e[3] = 0;
        }
        __syncthreads();
        if (tid == kThreads - 1) carry = before + x;
        __syncthreads();
    }
}

// chunk table {first token, tokens}: slot c belongs to the last sequence whose first chunk is
// <= c, if c is inside its chunk range; other slots are unused (tokens 0)
__global__ __launch_bounds__(256) void gdn_varlen_chunk_kernel(const int32_t *seqs, int32_t nseq, int32_t C,
                                                               int32_t nchunks, int32_t *chunks) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= nchunks) return;
    int lo = 0, hi = nseq - 1, best = -1;
    while (lo <= hi) {  // chunk0 is non-decreasing in the sequence index
        const int mid = (lo + hi) >> 1;
        if (seqs[4 * mid + 2] <= c) {
            best = mid;
            lo = mid + 1;
        } else {
            hi = mid - 1;
        }
    }
    int t0 = 0, n = 0;
    if (best >= 0) {
        const int32_t *e = seqs + 4 * best;
        const int lc = c - e[2];
        if (lc * C < e[1]) {
            t0 = e[0] + lc * C;
            n = min(C, e[1] - lc * C);
        }
    }
    chunks[2 * c] = t0;
    chunks[2 * c + 1] = n;
}

}  // namespace

hipError_t launch_varlen_tables(const int32_t *cu_seqlens, int32_t nseq, int32_t T, int chunk, int32_t *seqs,
                                int32_t *chunks, int32_t nchunks, hipStream_t stream) {
    if (nseq < 1 || nchunks < 1 || T < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gdn_varlen_seq_kernel, dim3(1), dim3(kThreads), 0, stream, cu_seqlens, nseq, T, chunk,
                       nchunks, seqs);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(gdn_varlen_chunk_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, stream, seqs,
                       nseq, chunk, nchunks, chunks);
    return hipGetLastError();
}

}  // namespace gdn
