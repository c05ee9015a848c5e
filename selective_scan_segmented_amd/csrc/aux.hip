// aux.hip -- auxiliary head/tail tokens of SF-Mamba on gfx950.
//
// "Seeing Both Ways, Running One Way" 3.2 and the techloop walkthrough
// ("第一个模块：Auxiliary Patch Swapping"): at a stage's first Mamba layer the
// patch sequence x_1..x_T gets a head and a tail token, both set to the mean
// of the patch tokens (length T -> T+2); between consecutive layers the head
// and tail outputs trade places, so the tail's summary of the whole sequence
// opens the next layer.
//
// PAD: one wave owns 64 consecutive (b, d) rows.  Chunks of the rows are
// staged through LDS with coalesced loads; each lane sums its own row in
// float64 in index order (so the mean is bit-identical to a sequential CPU sum),
// and the chunk is written back shifted by one token with coalesced stores.
// The mean is rounded once to the io type (round-to-odd float32 step, then
// round-to-nearest-even bfloat16, see sfm_device.h).
// SWAP: in place it touches only the two end tokens of every row; out of place
// it is a coalesced copy with the two ends exchanged.
#include "sfm_device.h"
#include "sfm_bwd.h"
#include "sfm_internal.h"

namespace sfm {

namespace {

constexpr int kPadWaves = 2;
// tokens per row staged at a time: 16 KB of LDS per wave
template <typename IO> constexpr int pad_chunk() { return 8192 / (int)sizeof(IO) / 64 * 2; }

template <typename IO>
__global__ __launch_bounds__(kWave * kPadWaves) void pad_kernel(const IO* __restrict__ in, IO* __restrict__ out,
                                                                 long long rows, int T) {
    constexpr int kPadChunk = pad_chunk<IO>();
    __shared__ IO stage[kPadWaves][kWave * kPadChunk];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const long long r0 = ((long long)blockIdx.x * kPadWaves + wave) * kWave;
    if (r0 >= rows) return;  // whole wave leaves together; no block barrier is used
    const int nr = (int)((rows - r0) < kWave ? (rows - r0) : kWave);
    const int L = T + 2;
    IO* st = stage[wave];
    const IO* src = in + r0 * T;
    IO* dst = out + r0 * L;
    double acc = 0.0;
    for (int c0 = 0; c0 < T; c0 += kPadChunk) {
        const int len = min(kPadChunk, T - c0);
        const int n = nr * len;
        const float inv = 1.0f / (float)len;
        if (len == T) {
            for (int e = lane; e < n; e += kWave) st[e] = src[e];
        } else {
            for (int e = lane; e < n; e += kWave) {
                const int c = div_small(e, inv);
                const int i = e - c * len;
                st[e] = src[(size_t)c * T + c0 + i];
            }
        }
        wave_lds_sync();
        if (lane < nr) {
            const IO* row = st + lane * len;
            for (int i = 0; i < len; ++i) acc += (double)to_f32(row[i]);  // index order
        }
        for (int e = lane; e < n; e += kWave) {
            const int c = div_small(e, inv);
            const int i = e - c * len;
            dst[(size_t)c * L + 1 + c0 + i] = st[e];
        }
        wave_lds_sync();
    }
    if (lane < nr) {
        const IO m = Io<IO>::from_f64(acc / (double)T);
        dst[(size_t)lane * L] = m;
        dst[(size_t)lane * L + L - 1] = m;
    }
}

template <typename IO>
__global__ __launch_bounds__(256) void swap_inplace_kernel(IO* __restrict__ p, long long rows, int L) {
    for (long long r = blockIdx.x * (long long)blockDim.x + threadIdx.x; r < rows;
         r += (long long)gridDim.x * blockDim.x) {
        IO* row = p + r * L;
        const IO h = row[0];
        const IO t = row[L - 1];
        row[0] = t;
        row[L - 1] = h;
    }
}

template <typename IO>
__global__ __launch_bounds__(256) void swap_copy_kernel(const IO* __restrict__ in, IO* __restrict__ out,
                                                        long long n, int L) {
    for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n;
         e += (long long)gridDim.x * blockDim.x) {
        const long long r = e / L;
        const int t = (int)(e - r * L);
        const int ts = (t == 0) ? L - 1 : (t == L - 1 ? 0 : t);
        out[e] = in[r * L + ts];
    }
}

// Backward of PAD: the mean feeds both end tokens, so each unpadded token
// receives its own padded gradient plus (g_0 + g_{L-1}) / T (float32, one
// rounding to the io type).  One thread per output element.
template <typename IO>
__global__ void pad_bwd_kernel(const IO* __restrict__ gp, IO* __restrict__ gx, long long n, int T) {
    const int L = T + 2;
    for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n;
         e += (long long)gridDim.x * blockDim.x) {
        const long long r = e / T;
        const int i = (int)(e - r * T);
        const IO* g = gp + r * L;
        const float ends = (to_f32(g[0]) + to_f32(g[L - 1])) / (float)T;
        gx[e] = from_f32<IO>(to_f32(g[1 + i]) + ends);
    }
}

// Channel-last: gx[b, i, d] = gp[b, 1 + i, d] + (gp[b, 0, d] + gp[b, L-1, d]) / T
// (the same float operations, in the same order, as the channel-first kernel).
template <typename IO>
__global__ void pad_bwd_cl_kernel(const IO* __restrict__ gp, IO* __restrict__ gx, long long n, int T, int C) {
    const int L = T + 2;
    for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n;
         e += (long long)gridDim.x * blockDim.x) {
        const long long bi = e / C;  // b * T + i
        const int c = (int)(e - bi * C);
        const long long b = bi / T;
        const int i = (int)(bi - b * T);
        const IO* g = gp + b * L * C + c;
        const float ends = (to_f32(g[0]) + to_f32(g[(size_t)(L - 1) * C])) / (float)T;
        gx[e] = from_f32<IO>(to_f32(g[(size_t)(1 + i) * C]) + ends);
    }
}

unsigned grid_for(long long work, int per_block) {
    long long b = (work + per_block - 1) / per_block;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (unsigned)b;
}

template <typename IO>
hipError_t pad_t(const void* in, void* out, int64_t rows, int64_t T, hipStream_t s) {
    const long long waves = (rows + kWave - 1) / kWave;
    const unsigned blocks = (unsigned)((waves + kPadWaves - 1) / kPadWaves);
    hipLaunchKernelGGL((pad_kernel<IO>), dim3(blocks), dim3(kWave * kPadWaves), 0, s,
                       static_cast<const IO*>(in), static_cast<IO*>(out), (long long)rows, (int)T);
    return hipGetLastError();
}

template <typename IO>
hipError_t swap_t(const void* in, void* out, int64_t rows, int64_t L, hipStream_t s) {
    if (in == out) {
        if (L < 2) return hipSuccess;
        hipLaunchKernelGGL((swap_inplace_kernel<IO>), dim3(grid_for(rows, 256)), dim3(256), 0, s,
                           static_cast<IO*>(out), (long long)rows, (int)L);
    } else {
        const long long n = rows * L;
        hipLaunchKernelGGL((swap_copy_kernel<IO>), dim3(grid_for(n, 256)), dim3(256), 0, s,
                           static_cast<const IO*>(in), static_cast<IO*>(out), n, (int)L);
    }
    return hipGetLastError();
}

template <typename IO>
hipError_t pad_bwd_t(const void* gp, void* gx, int64_t rows, int64_t T, hipStream_t s, int64_t channels) {
    if (channels > 0) {
        const long long n = rows * T * channels;
        hipLaunchKernelGGL((pad_bwd_cl_kernel<IO>), dim3(grid_for(n, 256)), dim3(256), 0, s,
                           static_cast<const IO*>(gp), static_cast<IO*>(gx), n, (int)T, (int)channels);
        return hipGetLastError();
    }
    const long long n = rows * T;
    hipLaunchKernelGGL((pad_bwd_kernel<IO>), dim3(grid_for(n, 256)), dim3(256), 0, s, static_cast<const IO*>(gp),
                       static_cast<IO*>(gx), n, (int)T);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_aux_pad_bwd(const void* gp, void* gx, int64_t rows, int64_t T, int io_dtype, hipStream_t stream,
                              int64_t channels) {
    return io_dtype == 0 ? pad_bwd_t<float>(gp, gx, rows, T, stream, channels)
                         : pad_bwd_t<__bf16>(gp, gx, rows, T, stream, channels);
}

hipError_t launch_aux_pad(const void* in, void* out, int64_t rows, int64_t T, int io_dtype, hipStream_t stream) {
    return io_dtype == 0 ? pad_t<float>(in, out, rows, T, stream) : pad_t<__bf16>(in, out, rows, T, stream);
}

hipError_t launch_aux_swap(const void* in, void* out, int64_t rows, int64_t L, int io_dtype, hipStream_t stream) {
    return io_dtype == 0 ? swap_t<float>(in, out, rows, L, stream) : swap_t<__bf16>(in, out, rows, L, stream);
}

}  // namespace sfm
