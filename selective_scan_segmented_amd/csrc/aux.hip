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

#include <cstdlib>

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

// ----------------------------------------------- flat forms for long rows
// floor(a / b) for 0 <= a < 2^40, 1 <= b < 2^31: the float64 quotient is
// correctly rounded and a true quotient k - r/b (r >= 1) stays more than one
// float64 ulp below k, so its floor is exact.
__device__ __forceinline__ long long floor_div(long long a, long long b) {
    return (long long)__builtin_floor((double)a / (double)b);
}

// PAD, part 1 -- the shifted copy: out[r][t] = in[r][t - 1] for 1 <= t <= L-2,
// i.e. output element o of the flat [rows, L] array takes input element
// o - 2r - 1.  Thread i writes the 16 bytes [16i, 16i + 16) of the output
// (8 bf16 / 4 f32) from the input words around them: for bf16 (L even, so rows
// start on words) each output word is the high half of one input word and the
// low half of the next (v_alignbit), the pair moving back one word past a row
// end.  The end tokens of each row receive a neighbour's value here and the
// row mean in part 2, which runs after this kernel.
template <typename IO>
__global__ __launch_bounds__(256) void pad_shift_kernel(const IO* __restrict__ in, IO* __restrict__ out,
                                                        long long rows, int T) {
    constexpr int EW = 4 / (int)sizeof(IO);  // elements per word
    const int L = T + 2;
    const long long nwi = rows * T / EW, nwo = rows * L / EW;  // input / output words
    const long long k0 = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;  // first output word
    if (k0 >= nwo) return;
    const uint32_t* iw = reinterpret_cast<const uint32_t*>(in);
    const long long r0 = floor_div(k0 * EW, L);
    const long long wrap = (r0 + 1) * L;  // first output element of the next row
    // input words from the first one row r0 + 1 might need
    const long long m0 = EW == 2 ? k0 - r0 - 2 : k0 - 2 * r0 - 3;
    uint32_t W[6];
#pragma unroll
    for (int m = 0; m < 6; ++m) W[m] = (m0 + m >= 0 && m0 + m < nwi) ? iw[m0 + m] : 0u;
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool next = (k0 + j) * EW >= wrap;  // this word lies in row r0 + 1
        if constexpr (EW == 2)
            o[j] = next ? __builtin_amdgcn_alignbit(W[j + 1], W[j], 16) : __builtin_amdgcn_alignbit(W[j + 2], W[j + 1], 16);
        else
            o[j] = next ? W[j] : W[j + 2];
    }
    uint32_t* ow = reinterpret_cast<uint32_t*>(out);
    if (k0 + 4 <= nwo) {
        *reinterpret_cast<uint4*>(ow + k0) = uint4{o[0], o[1], o[2], o[3]};
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (k0 + j < nwo) ow[k0 + j] = o[j];
    }
}

// PAD, part 2 -- the row means: one lane per row sums its T tokens in float64
// in index order (bit-identical to a sequential CPU sum) from direct loads,
// sixteen 16-byte units (or words) in flight, and writes both end tokens.
template <typename IO>
__global__ __launch_bounds__(256) void pad_sum_kernel(const IO* __restrict__ in, IO* __restrict__ out, long long rows,
                                                      int T) {
    const long long r = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const IO* row = in + r * T;
    double acc = 0.0;
    int i = 0;
    constexpr int EU = 16 / (int)sizeof(IO);
    if (((size_t)T * sizeof(IO)) % 16 == 0) {
        for (; i + 16 * EU <= T; i += 16 * EU) {
            uint4 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = reinterpret_cast<const uint4*>(row + i)[k];
            const IO* e = reinterpret_cast<const IO*>(v);
#pragma unroll
            for (int k = 0; k < 16 * EU; ++k) acc += (double)to_f32(e[k]);
        }
    } else if (((size_t)T * sizeof(IO)) % 4 == 0) {
        constexpr int EW = 4 / (int)sizeof(IO);
        for (; i + 32 * EW <= T; i += 32 * EW) {
            uint32_t v[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) v[k] = reinterpret_cast<const uint32_t*>(row + i)[k];
            const IO* e = reinterpret_cast<const IO*>(v);
#pragma unroll
            for (int k = 0; k < 32 * EW; ++k) acc += (double)to_f32(e[k]);
        }
    }
    for (; i + 16 <= T; i += 16) {
        IO v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = row[i + k];
#pragma unroll
        for (int k = 0; k < 16; ++k) acc += (double)to_f32(v[k]);
    }
    for (; i < T; ++i) acc += (double)to_f32(row[i]);
    const IO m = Io<IO>::from_f64(acc / (double)T);
    const int L = T + 2;
    out[r * L] = m;
    out[r * L + L - 1] = m;
}

// SWAP out of place: a 16-byte copy per thread (8 bf16 / 4 f32), the elements
// that are a row's first or last token then replaced by the other end's.
template <typename IO>
__global__ __launch_bounds__(256) void swap_copy_vec_kernel(const IO* __restrict__ in, IO* __restrict__ out,
                                                            long long n, int L) {
    constexpr int E = 16 / (int)sizeof(IO);
    const long long e0 = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * E;
    if (e0 >= n) return;
    IO v[E];
    if (e0 + E <= n) {
        *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(in + e0);
    } else {
#pragma unroll
        for (int i = 0; i < E; ++i) v[i] = e0 + i < n ? in[e0 + i] : Io<IO>::zero();
    }
    const long long r0 = floor_div(e0, L);
    const int t0 = (int)(e0 - r0 * L);
    // the row ends inside [e0, e0 + E): few, and at most one pair unless L < E
    for (int i = 0; i < E; ++i) {
        const long long e = e0 + i;
        if (e >= n) break;
        const long long rr = r0 + (t0 + i) / L;
        const int t = (int)(e - rr * L);
        if (t == 0) v[i] = in[rr * L + L - 1];
        else if (t == L - 1) v[i] = in[rr * L];
    }
    if (e0 + E <= n) {
        *reinterpret_cast<uint4*>(out + e0) = *reinterpret_cast<const uint4*>(v);
    } else {
#pragma unroll
        for (int i = 0; i < E; ++i)
            if (e0 + i < n) out[e0 + i] = v[i];
    }
}

unsigned grid_for(long long work, int per_block) {
    long long b = (work + per_block - 1) / per_block;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (unsigned)b;
}

// SFM_PAD_FLAT (diagnostics): 0 keeps the staged kernel for every row
// length, 1 takes the flat kernels wherever they apply.
int pad_flat_env() {
    static const int v = [] {
        const char* e = std::getenv("SFM_PAD_FLAT");
        return e ? std::atoi(e) : -1;
    }();
    return v;
}

template <typename IO>
hipError_t pad_t(const void* in, void* out, int64_t rows, int64_t T, hipStream_t s) {
    // Rows of 64 or more tokens: the shifted copy runs over the whole flat
    // array and the row sums one lane per row (the staged kernel below gives
    // each wave 64 whole rows, too few waves for long rows); bf16 needs an even
    // row length there, so that rows start on 4-byte words.
    const int env = pad_flat_env();
    const bool words = sizeof(IO) == 4 || (T + 2) % 2 == 0;
    if (words && env != 0 && (T >= 64 || env == 1)) {
        const long long nwo = rows * (T + 2) / (4 / (long long)sizeof(IO));
        const long long threads = (nwo + 3) / 4;
        hipLaunchKernelGGL((pad_shift_kernel<IO>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                           static_cast<const IO*>(in), static_cast<IO*>(out), (long long)rows, (int)T);
        hipLaunchKernelGGL((pad_sum_kernel<IO>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                           static_cast<const IO*>(in), static_cast<IO*>(out), (long long)rows, (int)T);
        return hipGetLastError();
    }
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
        const long long threads = (n + 16 / (long long)sizeof(IO) - 1) / (16 / (long long)sizeof(IO));
        hipLaunchKernelGGL((swap_copy_vec_kernel<IO>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
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
