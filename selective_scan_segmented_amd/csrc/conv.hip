// conv.hip -- boundary-masked depthwise conv1d over batch-folded rows (gfx950).
//
// The techloop walkthrough ("第二个模块", conv-boundary part) and "Seeing Both
// Ways, Running One Way" 8.1 item 5: once B2 samples are laid end to end in a
// folded row, the block's depthwise conv must not let a tap reach into the
// neighbouring sample.  Here the kernel walks folded coordinates (b1, d, s),
// maps s to (sample b = b1*B2 + s/L, t = s mod L) by index arithmetic, and a tap
// at folded position s + j - P counts only if it stays inside the segment
// [s - t, s - t + L) of the same sample; otherwise it reads zero.
//
// HBM-bound (2 io elements per output); each thread produces kPer consecutive
// outputs of one folded row from a register window, so every input element is
// fetched once per thread and neighbouring threads read neighbouring addresses.
#include "sfm_device.h"
#include "sfm_internal.h"

namespace sfm {

namespace {

constexpr int kPer = 8;

template <typename IO, int KW>
__global__ __launch_bounds__(256) void dwconv_kernel(const IO* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ bias, IO* __restrict__ out,
                                                     int B1, int B2, int D, int L, int K, int P, int act,
                                                     long long n_groups, int groups_per_seg) {
    for (long long g = blockIdx.x * (long long)blockDim.x + threadIdx.x; g < n_groups;
         g += (long long)gridDim.x * blockDim.x) {
        // g -> (b1, d, segment j, group within the segment)
        const long long seg = g / groups_per_seg;
        const int gi = (int)(g - seg * groups_per_seg);
        const long long row = seg / B2;        // folded row index b1 * D + d
        const int j = (int)(seg - row * B2);   // segment (sample) within the folded row
        const int b1 = (int)(row / D);
        const int d = (int)(row - (long long)b1 * D);
        const int b = b1 * B2 + j;             // fold index map
        const int t0 = gi * kPer;
        const IO* xr = x + ((size_t)b * D + d) * L;
        IO* orow = out + ((size_t)b * D + d) * L;
        float wk[KW];
#pragma unroll
        for (int q = 0; q < KW; ++q) wk[q] = q < K ? w[(size_t)d * K + q] : 0.0f;
        const float bv = bias ? bias[d] : 0.0f;
        float win[kPer + KW - 1];
#pragma unroll
        for (int q = 0; q < kPer + KW - 1; ++q) {
            const int tt = t0 - P + q;  // stays inside this sample's segment or reads zero
            win[q] = (tt >= 0 && tt < L) ? to_f32(xr[tt]) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int t = t0 + i;
            if (t < L) {
                float acc = bv;
#pragma unroll
                for (int q = 0; q < KW; ++q) acc = __builtin_fmaf(wk[q], win[i + q], acc);
                if (act == 1) acc = silu(acc);
                orow[t] = from_f32<IO>(acc);
            }
        }
    }
}

template <typename IO, int KW>
hipError_t launch_t(const void* x, const float* w, const float* bias, void* out, int64_t B1, int64_t B2, int64_t D,
                    int64_t L, int K, int P, int act, hipStream_t s) {
    const int gps = (int)((L + kPer - 1) / kPer);
    const long long n_groups = B1 * B2 * D * (long long)gps;
    long long blocks = (n_groups + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((dwconv_kernel<IO, KW>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const IO*>(x), w, bias, static_cast<IO*>(out), (int)B1, (int)B2, (int)D, (int)L,
                       K, P, act, n_groups, gps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dwconv1d(const void* x, const float* w, const float* bias, void* out, int64_t B1, int64_t B2,
                           int64_t D, int64_t L, int K, int pad_left, int act, int io_dtype, hipStream_t stream) {
    if (io_dtype == 0) {
        return K <= 4 ? launch_t<float, 4>(x, w, bias, out, B1, B2, D, L, K, pad_left, act, stream)
                      : launch_t<float, 8>(x, w, bias, out, B1, B2, D, L, K, pad_left, act, stream);
    }
    return K <= 4 ? launch_t<__bf16, 4>(x, w, bias, out, B1, B2, D, L, K, pad_left, act, stream)
                  : launch_t<__bf16, 8>(x, w, bias, out, B1, B2, D, L, K, pad_left, act, stream);
}

}  // namespace sfm
