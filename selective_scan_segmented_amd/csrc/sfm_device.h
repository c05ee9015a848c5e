// sfm_device.h -- device-side helpers shared by the libsfm HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sfm {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- io element types
// io tensors hold float32 or bfloat16; kernels are instantiated for both and do
// all arithmetic in float32 (state, accumulation) or float64 (pad mean).
template <typename T> struct Io;
template <> struct Io<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ float to_f32(float v) { return v; }
    static __device__ __forceinline__ float from_f32(float v) { return v; }
    static __device__ __forceinline__ float from_f64(double v) { return (float)v; }  // RNE
    static __device__ __forceinline__ float zero() { return 0.0f; }
    // raw element bits held in a 32-bit register, and their float32 value
    static __device__ __forceinline__ uint32_t bits(float v) { return __float_as_uint(v); }
    static __device__ __forceinline__ float of_bits(uint32_t b) { return __uint_as_float(b); }
};
template <> struct Io<__bf16> {
    static __device__ __forceinline__ float to_f32(__bf16 v) { return (float)v; }
    static __device__ __forceinline__ __bf16 from_f32(float v) { return (__bf16)v; }  // RNE (v_cvt_pk_bf16_f32)
    // float64 -> bfloat16 in one rounding: round to float32 with round-to-odd
    // (truncate, then set the last bit when inexact), then to bfloat16 with
    // round-to-nearest-even.  24 >= 8 + 2 bits makes the two-step result equal
    // to a direct rounding (Boldo & Melquiond, "Emulation of FMA and correctly
    // rounded sums: proved algorithms using rounding to odd", 2008).
    static __device__ __forceinline__ __bf16 from_f64(double v) {
        float f = (float)v;
        double back = (double)f;
        if (back != v && f == f) {
            uint32_t bits = __float_as_uint(f);
            if (__builtin_fabs(back) > __builtin_fabs(v)) bits -= 1u;  // step toward zero
            bits |= 1u;
            f = __uint_as_float(bits);
        }
        return (__bf16)f;
    }
    static __device__ __forceinline__ __bf16 zero() { return (__bf16)0.0f; }
    static __device__ __forceinline__ uint32_t bits(__bf16 v) { return __builtin_bit_cast(unsigned short, v); }
    static __device__ __forceinline__ float of_bits(uint32_t b) { return __uint_as_float(b << 16); }
};

template <typename T> __device__ __forceinline__ float to_f32(T v) { return Io<T>::to_f32(v); }

// element j of a 16-byte packet of io elements, as float32
template <typename T> __device__ __forceinline__ float unpack(const uint4& v, int j);
template <> __device__ __forceinline__ float unpack<float>(const uint4& v, int j) {
    const uint32_t w = j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
    return __uint_as_float(w);
}
template <> __device__ __forceinline__ float unpack<__bf16>(const uint4& v, int j) {
    const int q = j >> 1;
    const uint32_t w = q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <typename T> __device__ __forceinline__ T from_f32(float v) { return Io<T>::from_f32(v); }

// ---------------------------------------------------------------- math
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// softplus(v) = log(1 + e^v) (PyTorch's beta = 1; its threshold 20 changes the
// float32 result by less than half an ulp, so the identity branch is implied).
// Evaluated as max(v, 0) + log1p(e^{-|v|}): the exponent never overflows, and
// log1p(e) for e in (0, 1] is log(w) + c with w = fl(1 + e) and c = e - (w - 1)
// the exact rounding error of that sum (first-order correction; |c| <= 2^-24,
// and dividing it by w in [1, 2] would change the result by less than 2^-25).
// Returns softplus(v) * log2(e), the form the exp2-based discretization uses.
__device__ __forceinline__ float softplus_log2e(float v) {
    const float e = exp2_fast(-__builtin_fabsf(v) * kLog2e);
    const float w = 1.0f + e;
    const float c = e - (w - 1.0f);
    const float l2 = log2_fast(w) + c * kLog2e;
    return __builtin_fmaf(__builtin_fmaxf(v, 0.0f), kLog2e, l2);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + exp2_fast(-v * kLog2e)); }

// Compiler-level ordering point for LDS traffic between lanes of ONE wave
// (a wavefront's LDS operations execute in issue order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS only: this wave's LDS operations complete,
// then s_barrier.  __syncthreads() also waits for every outstanding global
// access (its fence covers global memory), which would drain direct
// global->LDS transfers that the caller still wants in flight; data that such
// transfers bring in must be waited for with wait_vmem / wait_vmem_at_most
// before this barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------- memory movement
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Wait until every vector-memory operation of this wave, including direct
// global->LDS transfers, has completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most k of this wave's vector-memory operations are
// outstanding (they complete in issue order).  k is wave-uniform; values above
// 15 wait as for 15, which is a stricter, still correct, wait.
__device__ __forceinline__ void wait_vmem_at_most(int k) {
    switch (k < 0 ? 0 : (k > 15 ? 15 : k)) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
        case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
        case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    }
}

// One 64-lane direct global->LDS transfer of SIZE bytes per lane: lane i's
// bytes at global address g land at LDS address l + OFF + i * max(SIZE, 4)
// (a transfer of fewer than 4 bytes still gives every lane a 4-byte slot, the
// data in its low bytes: CDNA3 ISA, global loads to LDS).  OFF is an
// immediate of the instruction (it moves both addresses, so g is passed
// pre-decremented).  Consecutive transfers that differ only in OFF share one
// LDS base register; rewriting that register between transfers serialises
// them (measured on gfx950: about twice the time to land a 13-transfer burst
// with ten waves per CU).
template <int SIZE, int OFF>
__device__ __forceinline__ void dma_at(const void* g, void* l) {
    static_assert((SIZE == 16 && OFF % 1024 == 0 && OFF < 4096) || (SIZE == 4 && OFF % 256 == 0 && OFF < 4096) ||
                      (SIZE == 2 && OFF % 256 == 0 && OFF < 4096),
                  "unsupported transfer size / offset");
    const char* gp = static_cast<const char*>(g) - OFF;
    const lds_void_ptr lp = (lds_void_ptr)l;
    // the builtin takes its size and offset as literals
#define SFM_DMA_AT(S, O) \
    if constexpr (SIZE == S && OFF == O) __builtin_amdgcn_global_load_lds(gp, lp, S, O, 0);
    SFM_DMA_AT(16, 0) SFM_DMA_AT(16, 1024) SFM_DMA_AT(16, 2048) SFM_DMA_AT(16, 3072)
    SFM_DMA_AT(4, 0) SFM_DMA_AT(4, 256) SFM_DMA_AT(4, 512) SFM_DMA_AT(4, 768)
    SFM_DMA_AT(4, 1024) SFM_DMA_AT(4, 1280) SFM_DMA_AT(4, 1536) SFM_DMA_AT(4, 1792)
    SFM_DMA_AT(4, 2048) SFM_DMA_AT(4, 2304) SFM_DMA_AT(4, 2560) SFM_DMA_AT(4, 2816)
    SFM_DMA_AT(4, 3072) SFM_DMA_AT(4, 3328) SFM_DMA_AT(4, 3584) SFM_DMA_AT(4, 3840)
    SFM_DMA_AT(2, 0) SFM_DMA_AT(2, 256) SFM_DMA_AT(2, 512) SFM_DMA_AT(2, 768)
    SFM_DMA_AT(2, 1024) SFM_DMA_AT(2, 1280) SFM_DMA_AT(2, 1536) SFM_DMA_AT(2, 1792)
    SFM_DMA_AT(2, 2048) SFM_DMA_AT(2, 2304) SFM_DMA_AT(2, 2560) SFM_DMA_AT(2, 2816)
    SFM_DMA_AT(2, 3072) SFM_DMA_AT(2, 3328) SFM_DMA_AT(2, 3584) SFM_DMA_AT(2, 3840)
#undef SFM_DMA_AT
}

// Compile-time loop: f(std::integral_constant<int, k>) for k = 0 .. K-1.
template <int K, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (K > 0) {
        static_for<K - 1>(f);
        f(std::integral_constant<int, K - 1>{});
    }
}

// Direct global->LDS copy of two regions into one contiguous LDS range:
// n0 16-byte units from g0, then n1 units from g1, landing at l.  Every
// instruction moves 64 units; a lane's source lies in g0 or g1 by its unit
// index, so an instruction may straddle the two.  Full instructions go four per
// LDS base with no lane mask; only the tail is masked.  `l`, n0 and n1 are
// wave-uniform; g0, g1 and l 16-byte aligned.  Nothing is waited for.
__device__ __forceinline__ void dma2_to_lds(const void* g0, int n0, const void* g1, int n1, void* l, int lane) {
    const int n = n0 + n1;
    const int full = n >> 6;
    const char* a = static_cast<const char*>(g0);
    const char* b = static_cast<const char*>(g1) - (size_t)n0 * 16;
    char* lb = static_cast<char*>(l);
    auto src = [&](int u) __attribute__((always_inline)) { return (u < n0 ? a : b) + (size_t)u * 16; };
    int k = 0;
    for (; k + 4 <= full; k += 4) {
        char* ll = lb + k * 1024;
        const int u = k * 64 + lane;
        dma_at<16, 0>(src(u), ll);
        dma_at<16, 1024>(src(u + 64), ll);
        dma_at<16, 2048>(src(u + 128), ll);
        dma_at<16, 3072>(src(u + 192), ll);
    }
    char* ll = lb + k * 1024;
    const int u = k * 64 + lane;
    const int rem = n - u;  // this lane's units left from instruction k on
    if (rem > 0) dma_at<16, 0>(src(u), ll);
    if (rem > 64) dma_at<16, 1024>(src(u + 64), ll);
    if (rem > 128) dma_at<16, 2048>(src(u + 128), ll);
    if (rem > 192) dma_at<16, 3072>(src(u + 192), ll);
}

// Issue direct global->LDS copies of the first (bytes & ~15) bytes of a region:
// 64 lanes x 16 bytes per instruction, four instructions per LDS base, no
// registers involved, nothing waited for.  `g` and `l` must be 16-byte
// aligned; `l` and `bytes` wave-uniform.
__device__ __forceinline__ void dma_to_lds(const void* g, void* l, int bytes, int lane) {
    const int units = bytes >> 4;
    const char* gb = static_cast<const char*>(g) + lane * 16;
    char* lb = static_cast<char*>(l);
    for (int u0 = 0; u0 < units; u0 += 4 * 64) {
        const char* gg = gb + (size_t)u0 * 16;
        char* ll = lb + u0 * 16;
        const int rem = units - u0 - lane;  // this lane moves unit u0 + 64k + lane while 64k < rem
        if (rem > 0) dma_at<16, 0>(gg, ll);
        if (rem > 64) dma_at<16, 1024>(gg + 1024, ll);
        if (rem > 128) dma_at<16, 2048>(gg + 2048, ll);
        if (rem > 192) dma_at<16, 3072>(gg + 3072, ll);
    }
}

// floor(e / len) for 0 <= e < 2^22 and len >= 1, via a float reciprocal: the
// true quotient (e + 0.5) / len is at least 0.5 / len away from an integer,
// while the float32 error of the product is at most (e / len) * 2^-23.
__device__ __forceinline__ int div_small(int e, float inv_len) {
    return (int)(((float)e + 0.5f) * inv_len);
}

}  // namespace sfm
