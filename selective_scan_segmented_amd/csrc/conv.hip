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
// HBM-bound (2 io elements per output).  The channel-first layout makes the
// B*D rows of L elements one contiguous array, and the fold is only index
// arithmetic, so the main kernel walks that flat array: thread i owns the 8
// elements [16i, 16i + 16) -- two 16-byte loads and two 16-byte stores (four of
// each for f32), consecutive lanes on consecutive addresses -- and takes the
// conv halo from its neighbours' registers by DPP wave shifts (lanes 0 and 63
// load theirs).  A tap counts only when its element lies in the output's own
// row, which is the sample boundary mask; with L >= 16 a thread's outputs span
// at most two rows.  Shorter rows take a per-row kernel (each thread a register
// window of 8 outputs of one row).
#include "sfm_device.h"
#include "sfm_internal.h"

#include <cstdlib>

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

// ------------------------------------------------------------- flat kernel
constexpr int kE = 16;  // elements per thread

template <int CTRL>
__device__ __forceinline__ uint32_t wshift(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}

// The kE elements of group e (a multiple of kE) as 32-bit words; zeros past n.
template <typename IO>
__device__ __forceinline__ void load_group(const IO* x, long long e, long long n, uint32_t (&wd)[kE * sizeof(IO) / 4]) {
    constexpr int NW = kE * sizeof(IO) / 4;
    if (e >= 0 && e + kE <= n) {
        const uint4* q = reinterpret_cast<const uint4*>(x + e);
#pragma unroll
        for (int k = 0; k < NW / 4; ++k) {
            const uint4 v = q[k];
            wd[4 * k] = v.x;
            wd[4 * k + 1] = v.y;
            wd[4 * k + 2] = v.z;
            wd[4 * k + 3] = v.w;
        }
    } else {
        IO el[kE];
#pragma unroll
        for (int i = 0; i < kE; ++i) el[i] = (e >= 0 && e + i < n) ? x[e + i] : Io<IO>::zero();
#pragma unroll
        for (int k = 0; k < NW; ++k) wd[k] = reinterpret_cast<const uint32_t*>(el)[k];
    }
}

template <typename IO>
__device__ __forceinline__ float elem(const uint32_t* wd, int i) {
    return to_f32(reinterpret_cast<const IO*>(wd)[i]);
}

// floor(a / b) for 0 <= a < 2^40, 1 <= b < 2^31: the float64 quotient is
// correctly rounded and a true quotient k - r/b (r >= 1) stays more than one
// float64 ulp below k, so its floor is exact.
__device__ __forceinline__ long long floor_div(long long a, long long b) {
    return (long long)__builtin_floor((double)a / (double)b);
}

// Thread i: outputs [16i, 16i + 16) of the flat array.  With L >= 16 they
// belong to row r0 (the first s = L - t0 of them) and possibly row r0 + 1;
// the window elements of each row are zeroed for the other row's outputs, and
// the second row's outputs are computed (with that row's weights) only by
// lanes whose span crosses a row end.
template <typename IO, int KW, int P2>
__global__ __launch_bounds__(256) void dwconv_flat_kernel(const IO* __restrict__ x, const float* __restrict__ w,
                                                          const float* __restrict__ bias, IO* __restrict__ out,
                                                          long long n, int L, int D, int K, int act) {
    constexpr int EW = 4 / (int)sizeof(IO);  // elements per word
    constexpr int NW = kE / EW;
    constexpr int WIN = kE + KW - 1;  // elements e0 - P2 .. e0 + kE - 1 + KW - 1 - P2
    const int lane = threadIdx.x & (kWave - 1);
    const long long e0 = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * kE;
    uint32_t own[NW], prv[NW], nxt[NW];
    load_group(x, e0, n, own);
    // the words of lane l - 1 and l + 1 that the window reaches (every lane
    // takes part, also those past n, whose groups are zeros)
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        prv[k] = (k + 1) * EW > kE - P2 ? wshift<0x138>(own[k]) : 0u;  // wave_shr:1
        nxt[k] = k * EW < KW - 1 - P2 ? wshift<0x130>(own[k]) : 0u;    // wave_shl:1
    }
    if (lane == 0 && P2 > 0) load_group(x, e0 - kE, n, prv);
    if (lane == kWave - 1 && KW - 1 - P2 > 0) load_group(x, e0 + kE, n, nxt);
    if (e0 >= n) return;
    const long long row0 = floor_div(e0, L);
    const int t0 = (int)(e0 - row0 * L);
    const int d0 = (int)(row0 - floor_div(row0, D) * D);
    const int sh = KW - K;  // the first KW - K taps of the window weigh 0
    float v0[WIN];          // window as seen from row r0: zero outside it
#pragma unroll
    for (int m = 0; m < WIN; ++m) {
        const int o = m - P2;
        const float v = o < 0 ? elem<IO>(prv, kE + o) : (o < kE ? elem<IO>(own, o) : elem<IO>(nxt, o - kE));
        const int pos = t0 + o;
        v0[m] = (pos >= 0 && pos < L) ? v : 0.0f;
    }
    float acc[kE];
    {
        float wk[KW];
#pragma unroll
        for (int j = 0; j < KW; ++j) wk[j] = j >= sh ? w[(size_t)d0 * K + j - sh] : 0.0f;
        const float b0 = bias ? bias[d0] : 0.0f;
#pragma unroll
        for (int i = 0; i < kE; ++i) {
            acc[i] = b0;
#pragma unroll
            for (int j = 0; j < KW; ++j)
                if (j >= sh) acc[i] = __builtin_fmaf(wk[j], v0[i + j], acc[i]);
        }
    }
    if (t0 + kE > L) {
        // outputs i >= s = L - t0 belong to the next row (channel d0 + 1)
        const int s = L - t0;
        const int d1 = d0 + 1 == D ? 0 : d0 + 1;
        float wk[KW];
#pragma unroll
        for (int j = 0; j < KW; ++j) wk[j] = j >= sh ? w[(size_t)d1 * K + j - sh] : 0.0f;
        const float b1 = bias ? bias[d1] : 0.0f;
        float v1[WIN];
#pragma unroll
        for (int m = 0; m < WIN; ++m) {
            const int o = m - P2;
            const float v = o < 0 ? elem<IO>(prv, kE + o) : (o < kE ? elem<IO>(own, o) : elem<IO>(nxt, o - kE));
            v1[m] = o >= s ? v : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kE; ++i) {
            float a1 = b1;
#pragma unroll
            for (int j = 0; j < KW; ++j)
                if (j >= sh) a1 = __builtin_fmaf(wk[j], v1[i + j], a1);
            acc[i] = i >= s ? a1 : acc[i];
        }
    }
    IO res[kE];
#pragma unroll
    for (int i = 0; i < kE; ++i) res[i] = from_f32<IO>(act == 1 ? silu(acc[i]) : acc[i]);
    if (e0 + kE <= n) {
        uint4* q = reinterpret_cast<uint4*>(out + e0);
        const uint32_t* rw = reinterpret_cast<const uint32_t*>(res);
#pragma unroll
        for (int k = 0; k < NW / 4; ++k) q[k] = uint4{rw[4 * k], rw[4 * k + 1], rw[4 * k + 2], rw[4 * k + 3]};
    } else {
#pragma unroll
        for (int i = 0; i < kE; ++i)
            if (e0 + i < n) out[e0 + i] = res[i];
    }
}

template <typename IO, int KW, int P2>
hipError_t launch_flat(const void* x, const float* w, const float* bias, void* out, long long n, int L, int D, int K,
                       int act, hipStream_t s) {
    const long long threads = (n + kE - 1) / kE;
    const long long blocks = (threads + 255) / 256;
    hipLaunchKernelGGL((dwconv_flat_kernel<IO, KW, P2>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const IO*>(x), w, bias, static_cast<IO*>(out), n, L, D, K, act);
    return hipGetLastError();
}

template <typename IO, int KW>
hipError_t launch_flat_p(const void* x, const float* w, const float* bias, void* out, long long n, int L, int D,
                         int K, int P, int act, hipStream_t s) {
    switch (P + KW - K) {
        case 0: return launch_flat<IO, KW, 0>(x, w, bias, out, n, L, D, K, act, s);
        case 1: return launch_flat<IO, KW, 1>(x, w, bias, out, n, L, D, K, act, s);
        case 2: return launch_flat<IO, KW, 2>(x, w, bias, out, n, L, D, K, act, s);
        case 3: return launch_flat<IO, KW, 3>(x, w, bias, out, n, L, D, K, act, s);
        default: break;
    }
    if constexpr (KW == 8) {
        switch (P + KW - K) {
            case 4: return launch_flat<IO, KW, 4>(x, w, bias, out, n, L, D, K, act, s);
            case 5: return launch_flat<IO, KW, 5>(x, w, bias, out, n, L, D, K, act, s);
            case 6: return launch_flat<IO, KW, 6>(x, w, bias, out, n, L, D, K, act, s);
            case 7: return launch_flat<IO, KW, 7>(x, w, bias, out, n, L, D, K, act, s);
            default: break;
        }
    }
    return hipErrorInvalidValue;
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
    // SFM_CONV_FLAT=0 (diagnostics) keeps the per-row kernel for every row length
    static const bool flat_off = [] {
        const char* e = std::getenv("SFM_CONV_FLAT");
        return e && e[0] == '0';
    }();
    const long long n = B1 * B2 * D * L;
    if (L >= 16 && !flat_off) {
        if (io_dtype == 0)
            return K <= 4 ? launch_flat_p<float, 4>(x, w, bias, out, n, (int)L, (int)D, K, pad_left, act, stream)
                          : launch_flat_p<float, 8>(x, w, bias, out, n, (int)L, (int)D, K, pad_left, act, stream);
        return K <= 4 ? launch_flat_p<__bf16, 4>(x, w, bias, out, n, (int)L, (int)D, K, pad_left, act, stream)
                      : launch_flat_p<__bf16, 8>(x, w, bias, out, n, (int)L, (int)D, K, pad_left, act, stream);
    }
    if (io_dtype == 0) {
        return K <= 4 ? launch_t<float, 4>(x, w, bias, out, B1, B2, D, L, K, pad_left, act, stream)
                      : launch_t<float, 8>(x, w, bias, out, B1, B2, D, L, K, pad_left, act, stream);
    }
    return K <= 4 ? launch_t<__bf16, 4>(x, w, bias, out, B1, B2, D, L, K, pad_left, act, stream)
                  : launch_t<__bf16, 8>(x, w, bias, out, B1, B2, D, L, K, pad_left, act, stream);
}

}  // namespace sfm
