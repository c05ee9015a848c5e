// layout.hip -- batched 2-D transposes between the channel-first [B, D, L] and
// channel-last [B, L, D] layouts (and [B, N, L] <-> [B, L, N] for B/C and
// their gradients), for the channel-last backward of rows too long for the
// whole-sample kernel: there the inputs are transposed into the workspace, the
// channel-first chunked (and split-row) backward runs, and its results are
// transposed back.  HBM-bound: one read and one write of every element,
// through 64 x 64 LDS tiles so that both the reads (along the source rows) and
// the writes (along the destination rows) are coalesced; the 65-element LDS
// pitch keeps the column reads free of bank conflicts.
#include "sfm_device.h"
#include "sfm_internal.h"

namespace sfm {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, T* __restrict__ out, long long R,
                                                        long long C, long long tiles_r, long long tiles_c) {
    __shared__ T tile[64][65];
    long long id = blockIdx.x;
    const long long tcol = id % tiles_c;
    id /= tiles_c;
    const long long trow = id % tiles_r;
    const long long b = id / tiles_r;
    const long long r0 = trow * 64, c0 = tcol * 64;
    const T* src = in + b * R * C;
    T* dst = out + b * R * C;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const long long r = r0 + i, c = c0 + tx;
        if (r < R && c < C) tile[i][tx] = src[r * C + c];
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const long long c = c0 + i, r = r0 + tx;
        if (c < C && r < R) dst[c * R + r] = tile[tx][i];
    }
}

template <typename T>
hipError_t transpose_t(const void* in, void* out, int64_t batch, int64_t R, int64_t C, hipStream_t s) {
    const long long tr = (R + 63) / 64, tc = (C + 63) / 64;
    const long long blocks = batch * tr * tc;
    if (blocks <= 0) return hipSuccess;
    if (blocks >= (1LL << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((transpose_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const T*>(in),
                       static_cast<T*>(out), (long long)R, (long long)C, tr, tc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose(const void* in, void* out, int64_t batch, int64_t R, int64_t C, int elem_bytes,
                            hipStream_t stream) {
    if (elem_bytes == 2) return transpose_t<uint16_t>(in, out, batch, R, C, stream);
    if (elem_bytes == 4) return transpose_t<uint32_t>(in, out, batch, R, C, stream);
    return hipErrorInvalidValue;
}

}  // namespace sfm
