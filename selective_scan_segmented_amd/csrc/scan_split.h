// scan_split.h -- the lane-split selective-scan kernel (included by the
// per-type instantiation units split_<io>_n<N>.hip).
//
// Method ("Seeing Both Ways, Running One Way", sections 3.1 and 3.3; techloop
// walkthrough "第二个模块：Batch Folding with Periodic State Reset"):
//   h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t,  y_t = C_t h_t + D x_t,
// over folded rows of B2 samples with the state re-initialised at every
// sample start (Abar = 0 there), Delta = softplus(delta + bias), x the
// boundary-masked depthwise conv of the (aux-padded) input.
//
// Work mapping (MI355X-first):
//  * The N states of one (sample, channel) recurrence are spread over G
//    adjacent lanes, NPL = NS / G states each, so a wave holds 64 / G
//    channels.  On gfx950 an unpacked fp32 VALU instruction occupies a SIMD
//    for about four cycles and a lone wave issues at most one every five to
//    six, so a SIMD needs several waves to stay busy; splitting the states
//    multiplies the waves of a launch by G while keeping each instruction's
//    64 lanes useful.
//  * The per-token work that does not depend on the state (softplus of
//    delta, the conv taps, Delta*u) is divided over the G lanes of a channel
//    as well: lane g of the group computes it for position t0 + g of a block
//    of G positions, and the G state updates of the block take Delta*log2(e)
//    and Delta*u of position t0 + j from lane j by a DPP broadcast.  Each
//    lane's share of y = C.h is summed over the group by DPP adds; the D*u
//    term enters through the partial of the lane that owns the position.
//  * B and C are widened once per sample into float32 LDS rows laid out
//    [t][g][B_0..B_{NPL-1}, C_0..C_{NPL-1}], so a lane reads its states' B and
//    C of one position with NPL/2 16-byte LDS reads.
//  * Staging: a wave's [64/G x L] delta slab and [64/G x XL] conv-input slab
//    are contiguous in HBM (channel-first layout), so they go to LDS by
//    16-byte direct global->LDS transfers; the raw B/C of the sample likewise
//    (one wave issues them for the workgroup).  y overwrites delta in LDS
//    (each position's delta is read before its y is written) and leaves by
//    16-byte stores.  The B2 samples of a folded row are processed in turn.
//  * The reset is a re-initialisation h <- Bbar x at t = 0, so non-finite
//    values never cross a sample boundary; taps outside the sample read 0.
#pragma once

#include "sfm_device.h"
#include "sfm_internal.h"

namespace sfm {
namespace split_detail {

constexpr int kMaxWpg = 8;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// DPP quad_perm control that gives every lane the value of lane J of its
// group of G adjacent lanes.
template <int G, int J>
constexpr int bcast_ctrl() {
    if constexpr (G == 2) return J | (J << 2) | ((2 + J) << 4) | ((2 + J) << 6);
    else return J * 0x55;
}

template <int G, int J>
__device__ __forceinline__ float bcast(float v) {
    if constexpr (G == 1) return v;
    else return dpp<bcast_ctrl<G, J>()>(v);
}

// Sum over the G adjacent lanes of a group, result in every lane of it
// (quad_perm [1,0,3,2] then [2,3,0,1]).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += dpp<0xB1>(v);
    if constexpr (G >= 4) v += dpp<0x4E>(v);
    return v;
}

template <typename IO, int NS, int G, int KW, bool CONV, bool SP, bool SILU>
struct SplitWave {
    static constexpr int NPL = NS / G;   // states per lane
    static constexpr int CPW = kWave / G;  // channels per wave
    static constexpr int NB = NPL / 2;   // float4 B/C reads per position ([B..., C...] per lane)
    static_assert(NPL >= 2 && NPL % 2 == 0, "two or more states per lane");

    const ScanParams& p;
    const int lane, c, g, d, rows;
    float A2[NPL];     // A of this lane's states (the exp takes Delta*log2(e))
    float Dk, dbias, cb, cw[KW];
    float mean;        // fused aux pad: head/tail value of this channel (io-rounded)

    __device__ __forceinline__ SplitWave(const ScanParams& p_, int lane_, int dw0)
        : p(p_), lane(lane_), c(lane_ / G), g(lane_ % G), d(dw0 + lane_ / G),
          rows(max(0, min(CPW, p_.D - dw0))), mean(0.0f) {}

    __device__ __forceinline__ void load_params() {
        const bool valid = c < rows;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int n = g * NPL + i;
            A2[i] = (valid && n < p.N) ? p.A[(size_t)d * p.N + n] : 0.0f;
        }
        Dk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;
        dbias = (valid && p.dbias) ? p.dbias[d] : 0.0f;
        // a K-tap conv runs as a KW-tap window whose first KW - K taps weigh 0
        const int sh = KW - p.K;
#pragma unroll
        for (int j = 0; j < KW; ++j)
            cw[j] = (CONV && valid && j >= sh) ? p.conv_w[(size_t)d * p.K + j - sh] : 0.0f;
        cb = (CONV && valid && p.conv_b) ? p.conv_b[d] : 0.0f;
    }

    // Conv input at padded position q of this lane's channel, for any q:
    // zero outside the sample, the aux-token value at both ends with the fused
    // pad, else the staged value (xr[i] holds unpadded index i).  The LDS read
    // always hits an in-bounds column.
    __device__ __forceinline__ float xq(const IO* xr, int q) const {
        const int L = p.L;
        const bool pad = p.pad_in != 0;
        const int lo = pad ? 1 : 0;
        const int qc = min(max(q, lo), L - 1 - lo);
        float v = to_f32(xr[qc - lo]);
        v = (pad && (q == 0 || q == L - 1)) ? mean : v;
        return (q < 0 || q >= L) ? 0.0f : v;
    }

    // One block of G positions [t0, t0 + G) (positions >= L are skipped):
    // lane g's per-token work for position t0 + g, then the G state updates.
    // win holds this lane's conv taps for position t0 + g - G on entry and
    // for t0 + g on exit.  FIRST: t0 == 0 (the reset).  CHECK: taps may leave
    // the staged interior.
    template <bool FIRST, bool CHECK>
    __device__ __forceinline__ void block(int t0, const IO* xr, IO* dr, const float* bc, float (&h)[NPL],
                                          float (&win)[KW]) {
        const int L = p.L;
        const int tau = t0 + g;                 // this lane's token
        const int tc = CHECK ? min(tau, L - 1) : tau;
        const int P2 = p.P + KW - p.K;           // pad_left of the KW-tap window
        // conv taps of tau: q = tau - P2 + j; the window moves by G per block
        if constexpr (CONV) {
            constexpr int keep = KW > G ? KW - G : 0;
#pragma unroll
            for (int j = 0; j < keep; ++j) win[j] = win[j + G];
#pragma unroll
            for (int j = keep; j < KW; ++j) {
                const int q = tau - P2 + j;
                win[j] = CHECK ? xq(xr, q) : to_f32(xr[q - (p.pad_in ? 1 : 0)]);
            }
        }
        float u;
        if constexpr (CONV) {
            float acc = cb;
#pragma unroll
            for (int j = 0; j < KW; ++j) acc = __builtin_fmaf(cw[j], win[j], acc);
            u = SILU ? silu(acc) : acc;
        } else {
            u = CHECK ? xq(xr, tc) : to_f32(xr[tc - (p.pad_in ? 1 : 0)]);
        }
        const float dl = to_f32(dr[tc]) + dbias;
        float d2, dt;  // Delta * log2(e) and Delta
        if constexpr (SP) {
            d2 = softplus_log2e(dl);
            dt = d2 * kLn2;
        } else {
            dt = dl;
            d2 = dl * kLog2e;
        }
        const float du = dt * u;
        const float dpu = Dk * u;  // D*u of this lane's own token
        float yown = 0.0f;
        static_for<G>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if (FIRST || CHECK ? t0 + j < L : true) {
                const float d2j = bcast<G, j>(d2);
                const float duj = bcast<G, j>(du);
                const float4* q4 = reinterpret_cast<const float4*>(bc + ((t0 + j) * G + g) * (2 * NPL));
                float bv[NPL], cv[NPL];
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const float4 v = q4[k];
                    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int e = 4 * k + m;  // element of [B_0..B_{NPL-1}, C_0..C_{NPL-1}]
                        if (e < NPL) bv[e] = vv[m];
                        else cv[e - NPL] = vv[m];
                    }
                }
                float yp = 0.0f;
#pragma unroll
                for (int i = 0; i < NPL; ++i) {
                    const float bx = duj * bv[i];
                    if (FIRST && j == 0) {
                        h[i] = bx;  // reset: the state is re-initialised at the sample start
                    } else {
                        const float a = exp2_fast(d2j * A2[i]);
                        h[i] = __builtin_fmaf(a, h[i], bx);
                    }
                    yp = i == 0 ? cv[0] * h[0] : __builtin_fmaf(cv[i], h[i], yp);
                }
                yp = group_sum<G>(yp);
                yown = (g == j) ? yp : yown;
            }
        });
        // (lanes past the tile's last channel work on LDS rows that were not
        // loaded and are not stored)
        yown += dpu;
        if (!CHECK || tau < L) dr[tau] = from_f32<IO>(yown);
    }

    // Whole sample: positions [0, L) from the staged rows; y replaces delta.
    __device__ __forceinline__ void sample(const IO* xr, IO* dr, const float* bc) {
        const int L = p.L;
        float h[NPL];
#pragma unroll
        for (int i = 0; i < NPL; ++i) h[i] = 0.0f;
        float win[KW];
        const int P2 = p.P + KW - p.K;
        // taps of the virtual position g - G (the block loop shifts by G first)
#pragma unroll
        for (int j = 0; j < KW; ++j) win[j] = CONV ? xq(xr, g - G - P2 + j) : 0.0f;
        const int nblk = (L + G - 1) / G;
        // Blocks that need no checks: every position < L and every newly read
        // conv tap inside the staged interior [lo, L-1-lo] of padded positions
        // (the taps kept from the previous block were read there already).
        const int lo = p.pad_in ? 1 : 0;
        constexpr int keep = CONV ? (KW > G ? KW - G : 0) : 0;
        const int first_new = CONV ? keep - P2 : 0;           // tap offset of the oldest new tap
        const int last_new = CONV ? KW - 1 - P2 : 0;          // tap offset of the newest tap
        // k*G + first_new >= lo  and  k*G + G-1 + last_new <= L-1-lo  and  k*G + G-1 <= L-1
        int kA = lo - first_new;
        kA = kA <= 0 ? 1 : max(1, (kA + G - 1) / G);
        const int hiA = min(L - 1 - lo - (G - 1) - last_new, L - G);
        int kB = hiA >= 0 ? hiA / G + 1 : 0;
        if (kB > nblk) kB = nblk;
        if (kB < kA) kB = kA;
        block<true, true>(0, xr, dr, bc, h, win);
        int k = 1;
        for (; k < kA && k < nblk; ++k) block<false, true>(k * G, xr, dr, bc, h, win);
        for (; k + 1 < kB; k += 2) {  // two blocks per trip: LDS offsets become immediates
            block<false, false>(k * G, xr, dr, bc, h, win);
            block<false, false>(k * G + G, xr, dr, bc, h, win);
        }
        for (; k < kB; ++k) block<false, false>(k * G, xr, dr, bc, h, win);
        for (; k < nblk; ++k) block<false, true>(k * G, xr, dr, bc, h, win);
    }
};

template <typename IO, int NS, int G, int KW, bool CONV, bool SP, bool SILU>
__global__ __launch_bounds__(kWave * kMaxWpg) void split_kernel(ScanParams p) {
    using W = SplitWave<IO, NS, G, KW, CONV, SP, SILU>;
    constexpr int NPL = W::NPL;
    constexpr int CPW = W::CPW;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    if (p.stagger_ticks) {
        // Staggered start: with the whole grid resident at once, dispatch
        // round r = blockIdx / stagger_period issues its loads r ticks (10 ns)
        // later, so early rounds compute while later rounds load.
        const unsigned long long r = blockIdx.x / p.stagger_period;
        if (r) {
            const unsigned long long until = __builtin_amdgcn_s_memrealtime() + r * p.stagger_ticks;
            while (__builtin_amdgcn_s_memrealtime() < until) __builtin_amdgcn_s_sleep(2);
        }
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // XCD-aware order: the workgroups of one folded row run on one XCD, so the
    // row's B/C stay in one L2
    const int NGRP = p.stiles * p.B1;
    int gi = blockIdx.x;
    if ((NGRP & 7) == 0) gi = (gi & 7) * (NGRP >> 3) + (gi >> 3);
    const int b1 = gi / p.stiles;
    const int tile = gi - b1 * p.stiles;
    const int dw0 = (tile * p.wpg + wave) * CPW;
    W w(p, lane, dw0);
    const int L = p.L, XL = p.xrow, N = p.N, D = p.D;
    float* bc = reinterpret_cast<float*>(smem + p.bc_off);
    IO* braw = reinterpret_cast<IO*>(smem + p.braw_off);
    float* means = reinterpret_cast<float*>(smem + p.mean_off);  // [wpg * 64/G]
    char* slab = smem + p.slab_off + (size_t)wave * p.slab_bytes;
    IO* xs = reinterpret_cast<IO*>(slab);
    IO* ds = reinterpret_cast<IO*>(slab + p.xs_bytes);
    const int rows = w.rows;
    const int nthr = p.wpg * kWave;
    const int tid = threadIdx.x;

    auto issue = [&](int b) __attribute__((always_inline)) {
        if (rows > 0) {
            const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * D + dw0) * XL;
            const IO* dg = static_cast<const IO*>(p.delta) + ((size_t)b * D + dw0) * L;
            dma_to_lds(xg, xs, rows * XL * (int)sizeof(IO), lane);
            dma_to_lds(dg, ds, rows * L * (int)sizeof(IO), lane);
        }
        if (wave == 0) {
            const int nbc = N * L * (int)sizeof(IO) / 16;
            dma2_to_lds(static_cast<const IO*>(p.Bm) + (size_t)b * N * L, nbc,
                        static_cast<const IO*>(p.Cm) + (size_t)b * N * L, nbc, braw, lane);
        }
    };

    issue(b1 * p.B2);
    w.load_params();
    // states n >= N: B = C = 0 for the whole launch (widening never writes them)
    if (N < NS) {
        for (int e = tid; e < L * NS; e += nthr) {
            const int t = e / NS, n = e - t * NS;
            if (n >= N) {
                float* q = bc + (t * G + n / NPL) * (2 * NPL) + n % NPL;
                q[0] = 0.0f;
                q[NPL] = 0.0f;
            }
        }
    }
    // every lane has a row of its own in the slabs (CPW rows are allocated);
    // the rows of channels past D are never loaded nor stored
    const IO* xr = xs + w.c * XL;
    IO* dr = ds + w.c * L;
    for (int j = 0; j < p.B2; ++j) {
        const int b = b1 * p.B2 + j;
        wait_vmem();
        __syncthreads();  // every wave's transfers (this wave's slabs, wave 0's raw B/C) have landed
        // Set-up of the sample, shared by the group's waves.  With the fused
        // pad the first nmean waves take the row means (one lane per channel of
        // the group, so the float64 sums run on all 64 lanes) while the others
        // widen B/C; without it every wave widens.
        const int gch = p.wpg * CPW;  // channels of the group
        const int nmean = p.pad_in ? min(p.wpg, (gch + kWave - 1) / kWave) : 0;
        if (wave < nmean) {
            const int r = wave * kWave + lane;  // channel row of the group
            const int ow = r / CPW, oc = r - ow * CPW;
            const int orows = max(0, min(CPW, D - (tile * p.wpg + ow) * CPW));
            if (r < gch && oc < orows) {
                // float64, index order, one rounding: bit-identical to the aux pad
                const IO* row = reinterpret_cast<const IO*>(smem + p.slab_off + (size_t)ow * p.slab_bytes) + oc * XL;
                double acc = 0.0;
                for (int t = 0; t < XL; ++t) acc += (double)to_f32(row[t]);
                means[r] = to_f32(Io<IO>::from_f64(acc / (double)XL));
            }
        }
        // (with a single wave per group it does both in turn)
        const int wb = nmean < p.wpg ? nmean : 0;  // first widening wave
        if (wave >= wb) {
            // raw [2][N][L] -> float32 [t][g][B.., C..]
            const float invL = 1.0f / (float)L;
            const int wthr = (p.wpg - wb) * kWave;
            for (int e = tid - wb * kWave; e < N * L; e += wthr) {
                const int n = div_small(e, invL), t = e - n * L;
                float* q = bc + (t * G + n / NPL) * (2 * NPL) + n % NPL;
                q[0] = to_f32(braw[e]);
                q[NPL] = to_f32(braw[N * L + e]);
            }
        }
        __syncthreads();  // B/C and the row means of sample b visible to the group
        if (p.pad_in) w.mean = means[wave * CPW + w.c];
        w.sample(xr, dr, bc);
        wave_lds_sync();
        if (rows > 0) {
            if (p.swap_out && L > 1 && w.g == 0 && w.c < rows) {
                const IO a = dr[0];
                dr[0] = dr[L - 1];
                dr[L - 1] = a;
            }
            wave_lds_sync();
            IO* yg = static_cast<IO*>(p.y) + ((size_t)b * D + dw0) * L;
            const int units = rows * L * (int)sizeof(IO) / 16;
            for (int u = lane; u < units; u += kWave)
                reinterpret_cast<uint4*>(yg)[u] = reinterpret_cast<const uint4*>(ds)[u];
        }
        if (j + 1 < p.B2) {
            // this wave's LDS reads of y have completed before transfers rewrite the slab
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue(b + 1);
        }
    }
    (void)NPL;
}

template <typename IO, int NS, int G, int KW, bool CONV, bool SP, bool SILU>
hipError_t launch_t(const ScanParams& p, hipStream_t stream) {
    auto kern = split_kernel<IO, NS, G, KW, CONV, SP, SILU>;
    static bool attr_set = false;
    if (!attr_set && p.lds_bytes > 64 * 1024) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024) != hipSuccess)
            (void)hipGetLastError();
        attr_set = true;
    }
    const unsigned grid = (unsigned)(p.stiles * p.B1);
    const unsigned block = (unsigned)(kWave * p.wpg);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), (size_t)p.lds_bytes, stream, p);
    return hipGetLastError();
}

template <typename IO, int NS, int G, int KW, bool CONV>
hipError_t launch_sp(const ScanParams& p, hipStream_t s) {
    const bool silu = CONV && p.act == 1;
    if (p.softplus)
        return silu ? launch_t<IO, NS, G, KW, CONV, true, CONV>(p, s) : launch_t<IO, NS, G, KW, CONV, true, false>(p, s);
    return silu ? launch_t<IO, NS, G, KW, CONV, false, CONV>(p, s) : launch_t<IO, NS, G, KW, CONV, false, false>(p, s);
}

template <typename IO, int NS, int G>
hipError_t launch_g(const ScanParams& p, hipStream_t s) {
    if (!p.conv_w) return launch_sp<IO, NS, G, 4, false>(p, s);
    if (p.K <= 4) return launch_sp<IO, NS, G, 4, true>(p, s);
    return launch_sp<IO, NS, G, 8, true>(p, s);
}

}  // namespace split_detail
}  // namespace sfm

// One translation unit per (io type, state count):
// SFM_SPLIT_INSTANCE(__bf16, bf16, 8, 2, 4) defines sfm::launch_split_bf16_n8
// for lane groups of 2 and 4.
#define SFM_SPLIT_INSTANCE(IOT, NAME, NSV, GA, GB)                                             \
    namespace sfm {                                                                           \
    hipError_t launch_split_##NAME##_n##NSV(const ScanParams& p, hipStream_t s) {             \
        if (p.split == GA) return split_detail::launch_g<IOT, NSV, GA>(p, s);                 \
        if (p.split == GB) return split_detail::launch_g<IOT, NSV, GB>(p, s);                 \
        return hipErrorInvalidValue;                                                          \
    }                                                                                         \
    }
