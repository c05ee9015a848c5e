// scan_cl.hip -- channel-last forward: the folded, segmented selective scan
// (with the fused boundary-masked conv, aux pad and aux swap) for tensors laid
// out [B, L, D] (u, delta, y) and [B, L, N] (B, C), for gfx950 (wave64).
//
// Method as the channel-first kernel ("Seeing Both Ways, Running One Way"
// 3.1-3.3; techloop walkthrough "第一个模块" and "第二个模块"): per sample and
// channel, h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t u_t with the state
// re-initialised at t = 0, y_t = C_t h_t + D u_t.  The pages choose between a
// channel-first and a channel-last layout per model, whichever runs faster;
// this is the second one.
//
// Work mapping: one wave per (folded row b1, tile of 64 channels), lanes are
// channels, the B2 samples of the row run one after the other.  In this layout
// the 64 channels of one position are one contiguous run of 64 io elements, so
// a chunk of W positions of x (plus the conv halo) and of delta is staged into
// LDS as [position][channel] rows by 16-byte direct transfers, eight or sixteen
// units per row, and lane l reads column l (consecutive addresses, no bank
// conflict).  B and C of the chunk (contiguous [W][N]) are widened to float32
// [W][Np] once and read back as 16-byte broadcasts.  y replaces delta in LDS
// and leaves with 16-byte stores, each row to its (swapped) position.  The
// per-position arithmetic is the channel-first kernel's, in the same order,
// so both layouts give bit-identical results on the same values.
#include <algorithm>
#include <type_traits>

#include "sfm_device.h"
#include "sfm_cl.h"
#include "sfm_internal.h"

namespace sfm {

namespace {

// 16-byte units u in [0, units) land at l + 16 u; src(u) is the global address
// of unit u.  Four transfers share one LDS base; lanes past `units` are masked.
template <typename F>
__device__ __forceinline__ void dma_units(F&& src, int units, char* l, int lane) {
    for (int u0 = 0; u0 < units; u0 += 4 * kWave) {
        char* ll = l + u0 * 16;
        const int u = u0 + lane;
        const int rem = units - u;
        if (rem > 0) dma_at<16, 0>(src(u), ll);
        if (rem > 64) dma_at<16, 1024>(src(u + 64), ll);
        if (rem > 128) dma_at<16, 2048>(src(u + 128), ll);
        if (rem > 192) dma_at<16, 3072>(src(u + 192), ll);
    }
}

template <typename IO, int NS, int KW, bool CONV, bool SP, bool SILU>
__global__ __launch_bounds__(2 * kWave) void scan_cl_kernel(ClParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int EB = (int)sizeof(IO);
    constexpr int KX = CONV ? KW : 1;  // conv taps (x rows beyond a chunk: KX - 1)
    // Staggered start: when the whole grid is resident at once, dispatch round r
    // waits r * stagger_ticks (10 ns ticks) so that early rounds compute while
    // later rounds load, instead of every wave waiting for all of the input.
    if (p.stagger_ticks) {
        const unsigned long long r = blockIdx.x / p.stagger_period;
        if (r) {
            const unsigned long long until = __builtin_amdgcn_s_memrealtime() + r * p.stagger_ticks;
            while (__builtin_amdgcn_s_memrealtime() < until) __builtin_amdgcn_s_sleep(2);
        }
    }
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;  // this wave's channel tile within the workgroup
    // XCD-aware order: workgroups go round-robin over the 8 XCDs; giving each
    // XCD a contiguous run of (row, tile group) items keeps a folded row's B/C
    // in one XCD's L2
    const int G = p.tgroups * p.B1;
    int g = blockIdx.x;
    if ((G & 7) == 0) g = (g & 7) * (G >> 3) + (g >> 3);
    const int b1 = g / p.tgroups;
    const int tile = (g - b1 * p.tgroups) * p.cw + wv;
    const int d0 = tile * kWave;
    const int nrows = max(0, min(kWave, p.D - d0));  // 0: a spare wave of the last group (stores nothing)
    const int d = d0 + lane;
    const bool valid = lane < nrows;
    const int col = valid ? lane : 0;  // lanes past the tile read column 0 and are never stored
    const int L = p.L, XL = p.xrow, N = p.N, D = p.D, W = p.W;
    const int P = CONV ? p.P : 0;
    const int sh = p.pad_in ? 1 : 0;  // padded position q is u row q - sh
    const bool pad = p.pad_in != 0;
    const int upr = nrows * EB / 16;  // 16-byte units per row of the tile (the planner makes this whole)
    const int rs = nrows;             // LDS row stride in elements

    IO* xs = reinterpret_cast<IO*>(smem + p.xs_off + wv * p.wave_bytes);  // [W + KX - 1][rs]: row r = padded position t0 - P + r
    IO* ds = reinterpret_cast<IO*>(smem + p.ds_off + wv * p.wave_bytes);  // [W][rs]: delta, then y
    float* bs = reinterpret_cast<float*>(smem + p.bc_off);  // [W][NS]
    float* cs = bs + W * NS;                                // [W][NS]

    float A[NS], Dk, dbias, cw[KW], cb;
#pragma unroll
    for (int n = 0; n < NS; ++n) A[n] = (valid && n < N) ? p.A[(size_t)d * N + n] : 0.0f;
    Dk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;
    dbias = (valid && p.dbias) ? p.dbias[d] : 0.0f;
#pragma unroll
    for (int j = 0; j < KW; ++j) cw[j] = (CONV && valid && j < p.K) ? p.conv_w[(size_t)d * p.K + j] : 0.0f;
    cb = (CONV && valid && p.conv_b) ? p.conv_b[d] : 0.0f;
    // states n >= N stay zero in the B/C stage (the first chunk's barrier publishes this)
    for (int e = tid; e < W * NS; e += nthr)
        if (e % NS >= N) bs[e] = cs[e] = 0.0f;

    const char* xg = static_cast<const char*>(p.u);
    const char* dg = static_cast<const char*>(p.delta);
    char* yg = static_cast<char*>(p.y);
    const float inv_upr = 1.0f / (float)upr;
    const float inv_N = 1.0f / (float)N;

    for (int j = 0; j < p.B2; ++j) {
        const int b = b1 * p.B2 + j;
        const IO* bgl = static_cast<const IO*>(p.Bm) + (size_t)b * L * N;
        const IO* cgl = static_cast<const IO*>(p.Cm) + (size_t)b * L * N;
        // fused aux pad with more than one chunk: the row mean from global memory
        // (float64, index order, one rounding: as the pad kernel)
        float mean = 0.0f;
        if (pad && p.nchunk > 1 && nrows > 0) {
            const IO* xc = static_cast<const IO*>(p.u) + (size_t)b * XL * D + d0 + col;
            double acc = 0.0;
            for (int r = 0; r < XL; ++r) acc += (double)to_f32(xc[(size_t)r * D]);
            mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
        }
        float h[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = 0.0f;
        for (int c = 0; c < p.nchunk; ++c) {
            const int t0 = c * W;
            const int cnt = min(W, L - t0);
            const int xrows = cnt + KX - 1;
            __syncthreads();  // both waves are done with the previous chunk's B/C stage
            // --- stage: B/C element loads in flight (shared by the group), then this wave's x and delta rows
            const int bcn = cnt * N;
            for (int e0 = 0; e0 < bcn; e0 += 8 * nthr) {
                IO bv[8], cv[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int e = e0 + k * nthr + tid;
                    bv[k] = e < bcn ? bgl[(size_t)t0 * N + e] : Io<IO>::zero();
                    cv[k] = e < bcn ? cgl[(size_t)t0 * N + e] : Io<IO>::zero();
                }
                if (e0 == 0) {
                    dma_units(
                        [&](int u) __attribute__((always_inline)) {
                            const int r = div_small(u, inv_upr);
                            const int q = t0 - P + r;
                            const int xr = (q - sh >= 0 && q - sh < XL) ? q - sh : 0;  // other rows are masked on use
                            return xg + (((size_t)b * XL + xr) * D + d0) * EB + (size_t)(u - r * upr) * 16;
                        },
                        xrows * upr, reinterpret_cast<char*>(xs), lane);
                    dma_units(
                        [&](int u) __attribute__((always_inline)) {
                            const int r = div_small(u, inv_upr);
                            return dg + (((size_t)b * L + t0 + r) * D + d0) * EB + (size_t)(u - r * upr) * 16;
                        },
                        cnt * upr, reinterpret_cast<char*>(ds), lane);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int e = e0 + k * nthr + tid;
                    if (e < bcn) {
                        const int t = div_small(e, inv_N);
                        const int n = e - t * N;
                        bs[t * NS + n] = to_f32(bv[k]);
                        cs[t * NS + n] = to_f32(cv[k]);
                    }
                }
            }
            wait_vmem();
            __syncthreads();  // the group's B/C stage is complete
            if (pad && p.nchunk == 1) {
                // the whole sample is staged: u row r sits at LDS row r + sh + P
                double acc = 0.0;
                for (int r = 0; r < XL; ++r) acc += (double)to_f32(xs[(r + sh + P) * rs + col]);
                mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
            }
            // conv input at LDS row r (padded position t0 - P + r): zero outside
            // the sample, the mean on the fused aux tokens
            auto xmask = [&](int r, float v) __attribute__((always_inline)) {
                const int q = t0 - P + r;
                v = (pad && (q == 0 || q == L - 1)) ? mean : v;
                return (q < 0 || q >= L) ? 0.0f : v;
            };
            float win[KW];
#pragma unroll
            for (int jj = 0; jj < KW; ++jj) win[jj] = 0.0f;
            if constexpr (CONV) {
#pragma unroll
                for (int jj = 1; jj < KW; ++jj) win[jj] = xmask(jj - 1, to_f32(xs[(jj - 1) * rs + col]));
            }
            // one position's inputs as raw LDS bits; the loop fetches position
            // i + 1 before position i computes, so LDS latency overlaps the math
            struct In {
                uint32_t xb, db;
                float4 bq[NS / 4], cq[NS / 4];
            };
            auto fetch = [&](int i, In& in) __attribute__((always_inline)) {
                in.xb = Io<IO>::bits(xs[(i + KX - 1) * rs + col]);
                in.db = Io<IO>::bits(ds[i * rs + col]);
                const float4* b4 = reinterpret_cast<const float4*>(bs + i * NS);
                const float4* c4 = reinterpret_cast<const float4*>(cs + i * NS);
#pragma unroll
                for (int q = 0; q < NS / 4; ++q) {
                    in.bq[q] = b4[q];
                    in.cq[q] = c4[q];
                }
            };
            auto step = [&](int i, In& in, auto firstc, auto checkc) __attribute__((always_inline)) {
                constexpr bool FIRST = decltype(firstc)::value;  // the sample start: the state is re-initialised
                constexpr bool CHECK = decltype(checkc)::value;  // the newest conv tap may be outside or an aux token
                // opaque: keeps this position's arithmetic after the previous one's
                // (the next position's exps are not hoisted into it)
                asm volatile("" : "+v"(in.xb), "+v"(in.db));
#pragma unroll
                for (int q = 0; q < NS / 4; ++q)
                    asm volatile("" ::"v"(in.bq[q].x), "v"(in.bq[q].y), "v"(in.bq[q].z), "v"(in.bq[q].w),
                                 "v"(in.cq[q].x), "v"(in.cq[q].y), "v"(in.cq[q].z), "v"(in.cq[q].w));
                const float xnew = CHECK ? xmask(i + KX - 1, Io<IO>::of_bits(in.xb)) : Io<IO>::of_bits(in.xb);
                const float dl = Io<IO>::of_bits(in.db) + dbias;
                float u;
                if constexpr (CONV) {
#pragma unroll
                    for (int jj = 0; jj < KW - 1; ++jj) win[jj] = win[jj + 1];
                    win[KW - 1] = xnew;
                    float acc = cb;
#pragma unroll
                    for (int jj = 0; jj < KW; ++jj) acc = __builtin_fmaf(cw[jj], win[jj], acc);
                    u = SILU ? silu(acc) : acc;
                } else {
                    u = xnew;
                }
                float d2, dt;  // Delta * log2(e) and Delta
                if constexpr (SP) {
                    d2 = softplus_log2e(dl);
                    dt = d2 * kLn2;
                } else {
                    dt = dl;
                    d2 = dl * kLog2e;
                }
                const float du = dt * u;
                float yv = Dk * u;
#pragma unroll
                for (int q = 0; q < NS / 4; ++q) {
                    const float bv[4] = {in.bq[q].x, in.bq[q].y, in.bq[q].z, in.bq[q].w};
                    const float cv[4] = {in.cq[q].x, in.cq[q].y, in.cq[q].z, in.cq[q].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int n = q * 4 + k;
                        const float bx = du * bv[k];
                        if constexpr (FIRST) {
                            h[n] = bx;
                        } else {
                            const float a = exp2_fast(d2 * A[n]);
                            h[n] = __builtin_fmaf(a, h[n], bx);
                        }
                        yv = __builtin_fmaf(cv[k], h[n], yv);
                    }
                }
                if (valid) ds[i * rs + col] = from_f32<IO>(yv);  // delta of position i is no longer needed
            };
            // positions whose newest conv tap (padded position t + lag) is an
            // ordinary input need no masking: i in [i_lo, i_hi)
            const int lag = KX - 1 - P;
            const int i_lo = min(cnt, max(0, sh - t0 - lag));
            const int i_hi = max(i_lo, min(cnt, L - sh - t0 - lag));
            using T_ = std::true_type;
            using F_ = std::false_type;
            In cur, nxt;
            int i = 0;
            fetch(0, cur);
            // invariant: cur holds position i
            auto one = [&](auto checkc) __attribute__((always_inline)) {
                if (i + 1 < cnt) fetch(i + 1, nxt);
                if (c == 0 && i == 0) step(i, cur, T_{}, T_{});
                else step(i, cur, F_{}, checkc);
                cur = nxt;
                ++i;
            };
            while (i < cnt && (i < i_lo || (c == 0 && i == 0))) one(T_{});
            // the unchecked middle, four positions per trip, two register sets alternating
            for (; i + 4 <= i_hi; i += 4) {
                fetch(i + 1, nxt);
                step(i, cur, F_{}, F_{});
                fetch(i + 2, cur);
                step(i + 1, nxt, F_{}, F_{});
                fetch(i + 3, nxt);
                step(i + 2, cur, F_{}, F_{});
                if (i + 4 < cnt) fetch(i + 4, cur);
                step(i + 3, nxt, F_{}, F_{});
            }
            while (i < i_hi) one(F_{});
            while (i < cnt) one(T_{});
            wave_lds_sync();
            // --- y rows out, each to its position (ends exchanged with the fused swap)
            const uint4* ys4 = reinterpret_cast<const uint4*>(ds);
            for (int u = lane; u < cnt * upr; u += kWave) {
                const int r = div_small(u, inv_upr);
                const int tt = t0 + r;
                const int ts = (p.swap_out && L > 1) ? (tt == 0 ? L - 1 : (tt == L - 1 ? 0 : tt)) : tt;
                *reinterpret_cast<uint4*>(yg + (((size_t)b * L + ts) * D + d0) * EB + (size_t)(u - r * upr) * 16) =
                    ys4[u];
            }
        }
    }
}

template <typename IO, int NS, int KW, bool CONV>
hipError_t launch_csp(const ClParams& p, hipStream_t s) {
    const bool silu = CONV && p.act == 1;
    const dim3 grid((unsigned)(p.B1 * p.tgroups)), block((unsigned)(kWave * p.cw));
    const size_t lds = (size_t)p.lds_bytes;
    if (p.softplus) {
        if (silu) hipLaunchKernelGGL((scan_cl_kernel<IO, NS, KW, CONV, true, CONV>), grid, block, lds, s, p);
        else hipLaunchKernelGGL((scan_cl_kernel<IO, NS, KW, CONV, true, false>), grid, block, lds, s, p);
    } else {
        if (silu) hipLaunchKernelGGL((scan_cl_kernel<IO, NS, KW, CONV, false, CONV>), grid, block, lds, s, p);
        else hipLaunchKernelGGL((scan_cl_kernel<IO, NS, KW, CONV, false, false>), grid, block, lds, s, p);
    }
    return hipGetLastError();
}

template <typename IO, int NS>
hipError_t launch_cns(const ClParams& p, hipStream_t s) {
    if (!p.conv_w) return launch_csp<IO, NS, 4, false>(p, s);
    if (p.K <= 4) return launch_csp<IO, NS, 4, true>(p, s);
    return launch_csp<IO, NS, 8, true>(p, s);
}

template <typename IO>
hipError_t launch_cio(const ClParams& p, hipStream_t s) {
    if (p.ns == 4) return launch_cns<IO, 4>(p, s);
    if (p.ns == 8) return launch_cns<IO, 8>(p, s);
    return launch_cns<IO, 16>(p, s);
}

}  // namespace

bool plan_scan_cl(ClParams& p, int io_bytes, int w_hint) {
    p.ns = p.N <= 4 ? 4 : (p.N <= 8 ? 8 : 16);
    p.tiles = (p.D + kWave - 1) / kWave;
    // every row of D channels, and the last tile's part of it, is whole 16-byte units
    if (((long long)p.D * io_bytes) % 16 != 0) return false;
    // two channel tiles per workgroup share one B/C stage (ten waves per CU fit at stage-4 sizes)
    p.cw = p.tiles >= 2 ? 2 : 1;
    p.tgroups = (p.tiles + p.cw - 1) / p.cw;
    const int kx = p.conv_w ? (p.K <= 4 ? 4 : 8) : 1;
    auto up16 = [](long long v) { return (int)((v + 15) & ~15LL); };
    auto wave = [&](int w) {
        return up16((long long)(w + kx - 1) * kWave * io_bytes) + up16((long long)w * kWave * io_bytes);
    };
    auto lds = [&](int w) { return p.cw * wave(w) + 2 * w * p.ns * 4; };
    int W = p.L;
    if (w_hint > 0 && W > w_hint) W = w_hint;
    while (W > 8 && lds(W) > 40 * 1024) W = (W + 1) / 2;
    p.W = W;
    p.nchunk = (p.L + W - 1) / W;
    p.xs_off = 0;
    p.ds_off = up16((long long)(W + kx - 1) * kWave * io_bytes);
    p.wave_bytes = wave(W);
    p.bc_off = p.cw * p.wave_bytes;
    p.lds_bytes = lds(W);
    // staggered start when the grid is resident all at once (as the channel-first plan)
    p.stagger_period = p.stagger_ticks = 0;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    constexpr int kLdsUnit = 1280;
    const int alloc = (p.lds_bytes + kLdsUnit - 1) / kLdsUnit * kLdsUnit;
    const long long per_cu = std::min(160 * 1024 / alloc, 16 / p.cw);
    const long long grid = (long long)p.tgroups * p.B1;
    if (p.nchunk == 1 && grid > cus && grid <= cus * per_cu) {
        const long long wg_bytes =
            (long long)p.cw * kWave * (p.xrow + p.L) * io_bytes + 2LL * p.N * p.L * io_bytes;
        const long long ticks = std::min<long long>(500, (long long)cus * wg_bytes / 47000);
        if (ticks > 0) {
            p.stagger_period = cus;
            p.stagger_ticks = (int)ticks;
        }
    }
    return true;
}

hipError_t launch_scan_cl(const ClParams& p, int io_dtype, hipStream_t s) {
    if (io_dtype == 0) return launch_cio<float>(p, s);
    return launch_cio<__bf16>(p, s);
}

}  // namespace sfm
