// scan.hip -- folded, segmented selective scan for gfx950 (wave64).
//
// Method ("Seeing Both Ways, Running One Way", sections 3.1 and 3.3; techloop
// walkthrough "第二个模块：Batch Folding with Periodic State Reset"):
//   h_s = Abar_s * h_{s-1} + Bbar_s x_s,  y_s = C_s h_s (+ D x_s)
// over folded rows of B2 samples, Abar_s = 0 where s mod L == 0.
//
// Work mapping (MI355X-first, not the pages' CUDA one):
//  * A workgroup owns one folded row b1 and one tile of 64 channels.  The 64
//    lanes of a wave are 64 channels, so every lane walks the same (sample, t)
//    at the same time: B[b,:,t] and C[b,:,t] are wave-uniform and are staged
//    once per wave in LDS as float32, read back as broadcasts.
//  * The folded row (B2*L positions) is cut into `waves` contiguous pieces, one
//    per wave.  Each lane scans its piece sequentially with the N-state float32
//    recurrence in registers -- no cross-lane scan is needed, because the
//    channel dimension already fills the wave; this is what removes the
//    short-sequence under-fill the pages attribute to per-sequence warp scans.
//  * The reset is a re-initialisation (h <- Bbar x) at every sample start, so
//    non-finite values never cross a sample boundary.
//  * When a piece starts inside a sample, the wave needs the state carried in
//    from the piece before it.  Phase 1: every wave computes the aggregate of
//    its piece's tail segment (from its last sample start, or the whole piece if
//    it holds none): flag "contains a reset", sum of Delta*log2e (so the decay
//    product is exp2(A * sum)) and the end state from zero.  The aggregates meet
//    in LDS; each wave folds its predecessors' aggregates with the segmented
//    operator (a reset cuts the carry) and phase 2 rescans its piece from that
//    carry, writing y.  Phase 1 is skipped when all cuts fall on sample starts.
//  * Folding is index arithmetic only: position s of row b1 is sample
//    b = b1*B2 + s/L at t = s mod L; nothing is copied.
//  * Inputs are staged per chunk through LDS with coalesced loads; y is written
//    back into the same LDS slots as delta and stored coalesced.
//  * The optional depthwise conv is fused: the conv input is staged with its
//    halo and the conv taps that fall outside the sample read zero (the
//    boundary masking of the techloop walkthrough's conv-boundary part).
#include "sfm_device.h"
#include "sfm_internal.h"

namespace sfm {

namespace {

constexpr int kMaxWaves = 16;

template <typename IO, int NS, int KW, bool CONV>
struct ScanWave {
    const ScanParams& p;
    const int lane;
    const int d0;
    const int nrows;  // valid channel rows of this tile (<= 64)
    const int b1;
    // per-lane parameters
    float A[NS];
    float Dk, dbias, cw[KW], cb;
    // LDS
    IO* xs;
    IO* ds;
    float* bs;
    float* cs;
    // chunk geometry
    int xrs, xoff, drs, doff, boff;

    __device__ ScanWave(const ScanParams& p_, int lane_, int d0_, int b1_, char* lds)
        : p(p_), lane(lane_), d0(d0_), nrows(min(kWave, p_.D - d0_)), b1(b1_) {
        const int d = d0 + lane;
        const bool valid = d < p.D;
#pragma unroll
        for (int n = 0; n < NS; ++n) A[n] = (valid && n < p.N) ? p.A[(size_t)d * p.N + n] : 0.0f;
        Dk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;
        dbias = (valid && p.dbias) ? p.dbias[d] : 0.0f;
#pragma unroll
        for (int j = 0; j < KW; ++j) cw[j] = (CONV && valid && j < p.K) ? p.conv_w[(size_t)d * p.K + j] : 0.0f;
        cb = (CONV && valid && p.conv_b) ? p.conv_b[d] : 0.0f;
        char* q = lds;
        xs = reinterpret_cast<IO*>(q);
        q += p.xs_bytes;
        ds = reinterpret_cast<IO*>(q);
        q += p.ds_bytes;
        bs = reinterpret_cast<float*>(q);
        q += p.ch * NS * sizeof(float);
        cs = reinterpret_cast<float*>(q);
        // states n >= N stay zero in B and C for the whole kernel
        for (int e = lane; e < p.ch * NS; e += kWave) {
            bs[e] = 0.0f;
            cs[e] = 0.0f;
        }
        wave_lds_sync();
    }

    // Stage the inputs of sample b for positions [t0, t0 + len) into LDS.
    __device__ void stage(int b, int t0, int len) {
        const int L = p.L, D = p.D, N = p.N;
        const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * D + d0) * L;
        const IO* dg = static_cast<const IO*>(p.delta) + ((size_t)b * D + d0) * L;
        const IO* bg = static_cast<const IO*>(p.Bm) + (size_t)b * N * L;
        const IO* cg = static_cast<const IO*>(p.Cm) + (size_t)b * N * L;
        if (p.flat) {
            // whole sample rows: the [64 x L] slabs are contiguous in memory
            xrs = L; xoff = 0; drs = L; doff = 0; boff = 0;
            const int n = nrows * L;
            for (int e = lane; e < n; e += kWave) {
                xs[e] = xg[e];
                ds[e] = dg[e];
            }
            const float invL = 1.0f / (float)L;
            for (int e = lane; e < N * L; e += kWave) {
                const int nn = div_small(e, invL);
                const int t = e - nn * L;
                bs[t * NS + nn] = to_f32(bg[e]);
                cs[t * NS + nn] = to_f32(cg[e]);
            }
        } else {
            // partial rows with the conv halo; zeros outside the sample
            const int xlen = CONV ? len + KW - 1 : len;
            xrs = p.xrs; drs = p.drs;
            xoff = CONV ? t0 - p.P : t0;
            doff = t0; boff = t0;
            const float invx = 1.0f / (float)xlen;
            for (int e = lane; e < nrows * xlen; e += kWave) {
                const int c = div_small(e, invx);
                const int i = e - c * xlen;
                const int t = xoff + i;
                xs[c * xrs + i] = (t >= 0 && t < L) ? xg[(size_t)c * L + t] : Io<IO>::zero();
            }
            const float invd = 1.0f / (float)len;
            for (int e = lane; e < nrows * len; e += kWave) {
                const int c = div_small(e, invd);
                const int i = e - c * len;
                ds[c * drs + i] = dg[(size_t)c * L + t0 + i];
            }
            for (int e = lane; e < N * len; e += kWave) {
                const int nn = div_small(e, invd);
                const int i = e - nn * len;
                bs[i * NS + nn] = to_f32(bg[(size_t)nn * L + t0 + i]);
                cs[i * NS + nn] = to_f32(cg[(size_t)nn * L + t0 + i]);
            }
        }
        wave_lds_sync();
    }

    // Store y for positions [t0, t0 + len) of sample b (y sits in ds).
    __device__ void store(int b, int t0, int len) {
        const int L = p.L;
        IO* yg = static_cast<IO*>(p.y) + ((size_t)b * p.D + d0) * L;
        if (p.flat && len == L) {
            const int n = nrows * L;
            for (int e = lane; e < n; e += kWave) yg[e] = ds[e];
        } else {
            const float inv = 1.0f / (float)len;
            for (int e = lane; e < nrows * len; e += kWave) {
                const int c = div_small(e, inv);
                const int i = e - c * len;
                yg[(size_t)c * L + t0 + i] = ds[c * drs + (t0 - doff) + i];
            }
        }
        wave_lds_sync();
    }

    __device__ __forceinline__ float xs_at(int t) const { return to_f32(xs[lane * xrs + t - xoff]); }

    // Scan positions [t0, t0 + len) of the staged sample.  OUT: write y into ds.
    // AGG: accumulate sum of Delta*log2e in sd2 (no output).
    template <bool OUT>
    __device__ void scan_chunk(int t0, int len, float (&h)[NS], float& sd2) {
        const int L = p.L;
        float win[KW];
        if constexpr (CONV) {
#pragma unroll
            for (int j = 0; j < KW - 1; ++j) {
                const int q = t0 - p.P + j;
                win[j + 1] = (q >= 0 && q < L) ? xs_at(q) : 0.0f;
            }
        }
        int t = t0;
        const int tend = t0 + len;
        if (t == 0) {
            step<OUT, true>(t, h, sd2, win);
            ++t;
        }
#pragma unroll 2
        for (; t < tend; ++t) step<OUT, false>(t, h, sd2, win);
    }

    template <bool OUT, bool FIRST>
    __device__ __forceinline__ void step(int t, float (&h)[NS], float& sd2, float (&win)[KW]) {
        float u;
        if constexpr (CONV) {
#pragma unroll
            for (int j = 0; j < KW - 1; ++j) win[j] = win[j + 1];
            const int q = t - p.P + KW - 1;
            win[KW - 1] = (q < p.L) ? xs_at(q) : 0.0f;
            float acc = cb;
#pragma unroll
            for (int j = 0; j < KW; ++j) acc = __builtin_fmaf(cw[j], win[j], acc);
            u = (p.act == 1) ? silu(acc) : acc;
        } else {
            u = to_f32(xs[lane * xrs + t - xoff]);
        }
        IO* dslot = &ds[lane * drs + t - doff];
        const float dl = to_f32(*dslot) + dbias;
        float d2, dt;  // Delta * log2(e) and Delta
        if (p.softplus) {
            d2 = softplus_log2e(dl);
            dt = d2 * kLn2;
        } else {
            dt = dl;  // exact, so integer-valued steps stay exact
            d2 = dl * kLog2e;
        }
        const float du = dt * u;
        if constexpr (!OUT) sd2 += d2;
        float yv = Dk * u;
        const float* bt = &bs[(t - boff) * NS];
        const float* ct = &cs[(t - boff) * NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const float bx = du * bt[n];
            if constexpr (FIRST) {
                h[n] = bx;  // reset: state re-initialised at the sample start
            } else {
                const float a = exp2_fast(d2 * A[n]);
                h[n] = __builtin_fmaf(a, h[n], bx);
            }
            if constexpr (OUT) yv = __builtin_fmaf(ct[n], h[n], yv);
        }
        if constexpr (OUT) *dslot = from_f32<IO>(yv);
    }

    // Run folded positions [sa, sb) of row b1, state carried in h.
    template <bool OUT>
    __device__ void run(int sa, int sb, float (&h)[NS], float& sd2) {
        const int L = p.L;
        int s = sa;
        while (s < sb) {
            const int j = s / L;
            const int t0 = s - j * L;
            const int len = min(min(p.ch, L - t0), sb - s);
            const int b = b1 * p.B2 + j;
            stage(b, t0, len);
            scan_chunk<OUT>(t0, len, h, sd2);
            wave_lds_sync();
            if (OUT) store(b, t0, len);
            s += len;
        }
    }
};

template <typename IO, int NS, int KW, bool CONV>
__global__ __launch_bounds__(kWave * kMaxWaves) void scan_kernel(ScanParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
    // giving each XCD a contiguous run of (row, tile) items keeps the B/C of a
    // folded row in one XCD's L2.
    const int G = p.tiles * p.B1;
    int g = blockIdx.x;
    if ((G & 7) == 0) g = (g & 7) * (G >> 3) + (g >> 3);
    const int b1 = g / p.tiles;
    const int tile = g - b1 * p.tiles;
    ScanWave<IO, NS, KW, CONV> w(p, lane, tile * kWave, b1, smem + (size_t)wave * p.stage_bytes);

    const int S = p.B2 * p.L;
    const int p0 = min(wave * p.piece, S);
    const int p1 = min(p0 + p.piece, S);
    float h[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = 0.0f;
    float sd2 = 0.0f;

    if (p.need_carry) {
        // phase 1: aggregate of the tail segment of this piece
        int flag = 1;
        if (p0 < p1) {
            int q = ((p1 - 1) / p.L) * p.L;  // last sample start in the piece
            if (q < p0) {
                q = p0;
                flag = 0;
            }
            w.template run<false>(q, p1, h, sd2);
        }
        char* agg = smem + (size_t)p.waves * p.stage_bytes;
        int* aflag = reinterpret_cast<int*>(agg);
        float* asum = reinterpret_cast<float*>(agg + kMaxWaves * sizeof(int));
        float* ah = asum + (size_t)p.waves * kWave;
        if (lane == 0) aflag[wave] = flag;
        asum[wave * kWave + lane] = sd2;
#pragma unroll
        for (int n = 0; n < NS; ++n) ah[((size_t)wave * NS + n) * kWave + lane] = h[n];
        __syncthreads();
        // carry-in: fold predecessors with the segmented operator
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = 0.0f;
        for (int v = 0; v < wave; ++v) {
            const int f = aflag[v];
            const float sv = asum[v * kWave + lane];
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                const float hv = ah[((size_t)v * NS + n) * kWave + lane];
                h[n] = f ? hv : __builtin_fmaf(exp2_fast(w.A[n] * sv), h[n], hv);
            }
        }
        sd2 = 0.0f;
    }
    // phase 2: scan the piece from the carried state and write y
    if (p0 < p1) w.template run<true>(p0, p1, h, sd2);
}

template <typename IO, int NS, int KW, bool CONV>
hipError_t launch_t(const ScanParams& p, hipStream_t stream) {
    auto kern = scan_kernel<IO, NS, KW, CONV>;
    static bool attr_set = false;
    if (!attr_set && p.lds_bytes > 64 * 1024) {
        // allow dynamic LDS beyond 64 KB (gfx950 has 160 KB per workgroup)
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024) != hipSuccess)
            (void)hipGetLastError();  // do not leave a stale error for the launch check
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(p.tiles * p.B1)), dim3((unsigned)(kWave * p.waves)),
                       (size_t)p.lds_bytes, stream, p);
    return hipGetLastError();
}

template <typename IO, int NS>
hipError_t launch_ns(const ScanParams& p, hipStream_t s) {
    if (!p.conv_w) return launch_t<IO, NS, 4, false>(p, s);
    if (p.K <= 4) return launch_t<IO, NS, 4, true>(p, s);
    return launch_t<IO, NS, 8, true>(p, s);
}

template <typename IO>
hipError_t launch_io(const ScanParams& p, hipStream_t s) {
    if (p.ns == 4) return launch_ns<IO, 4>(p, s);
    if (p.ns == 8) return launch_ns<IO, 8>(p, s);
    return launch_ns<IO, 16>(p, s);
}

// LDS row stride (elements) whose length in 4-byte words is odd, so that the
// 64 lanes reading one column hit distinct banks.
int odd_word_stride(int elems, int elem_bytes) {
    int s = elems;
    while (((s * elem_bytes + 3) / 4) % 2 == 0 || (s * elem_bytes) % 4 != 0) ++s;
    return s;
}

}  // namespace

bool plan_scan(ScanParams& p, int io_bytes, int waves_hint, int ch_hint) {
    const int L = p.L, S = p.B2 * p.L;
    p.ns = p.N <= 4 ? 4 : (p.N <= 8 ? 8 : 16);
    const int kw = p.conv_w ? (p.K <= 4 ? 4 : 8) : 0;
    p.tiles = (p.D + kWave - 1) / kWave;
    const int lds_cap = 160 * 1024;
    const int agg_fixed = kMaxWaves * (int)sizeof(int);
    auto stage_bytes = [&](int ch, bool flat, int& xsb, int& dsb, int& xrs, int& drs) {
        if (flat) {
            xrs = L;
            drs = L;
            xsb = kWave * L * io_bytes;
            dsb = xsb;
        } else {
            xrs = odd_word_stride(ch + (kw ? kw - 1 : 0), io_bytes);
            drs = odd_word_stride(ch, io_bytes);
            xsb = kWave * xrs * io_bytes;
            dsb = kWave * drs * io_bytes;
        }
        xsb = (xsb + 15) & ~15;
        dsb = (dsb + 15) & ~15;
        return xsb + dsb + 2 * ch * p.ns * (int)sizeof(float);
    };
    // chunk length: whole samples when they fit comfortably, else fixed chunks
    int xsb = 0, dsb = 0, xrs = 0, drs = 0;
    bool flat = L <= 256;
    int ch = flat ? L : (ch_hint > 0 ? ch_hint : 32);
    int sb = stage_bytes(ch, flat, xsb, dsb, xrs, drs);
    if (flat && sb > 48 * 1024) {
        flat = false;
        ch = ch_hint > 0 ? ch_hint : 32;
        sb = stage_bytes(ch, flat, xsb, dsb, xrs, drs);
    }
    // waves per row
    int W;
    if (waves_hint > 0) {
        W = waves_hint;
    } else if (S <= 256 || p.B2 > 1) {
        // short rows: one or more whole samples per wave, cuts on sample starts
        W = 1;
        for (int c = 1; c <= 8; ++c)
            if (p.B2 % c == 0) W = c;
    } else {
        // long rows: enough waves to fill 256 CUs x 4 SIMDs a few times over
        const long long items = (long long)p.tiles * p.B1;
        long long want = (2048 + items - 1) / items;
        W = (int)(want < 1 ? 1 : (want > kMaxWaves ? kMaxWaves : want));
    }
    if (W > kMaxWaves) W = kMaxWaves;
    if (W > S) W = S;
    auto total_lds = [&](int w, int stage) {
        const int piece = (S + w - 1) / w;
        bool carry = false;
        for (int i = 1; i < w; ++i) {
            const int s0 = i * piece;
            if (s0 < S && s0 % L) carry = true;
        }
        int agg = carry ? agg_fixed + w * kWave * (int)sizeof(float) * (1 + p.ns) : 0;
        return w * stage + agg;
    };
    while (total_lds(W, sb) > lds_cap) {
        if (!flat && ch > 8) {
            ch /= 2;
            sb = stage_bytes(ch, flat, xsb, dsb, xrs, drs);
        } else if (W > 1) {
            --W;
        } else {
            return false;
        }
    }
    p.waves = W;
    p.piece = (S + W - 1) / W;
    p.need_carry = 0;
    for (int i = 1; i < W; ++i) {
        const int s0 = i * p.piece;
        if (s0 < S && s0 % L) p.need_carry = 1;
    }
    p.ch = ch;
    p.flat = flat ? 1 : 0;
    p.xrs = xrs;
    p.drs = drs;
    p.xs_bytes = xsb;
    p.ds_bytes = dsb;
    p.stage_bytes = sb;
    p.lds_bytes = total_lds(W, sb);
    return true;
}

hipError_t launch_scan(const ScanParams& p, int io_dtype, hipStream_t stream) {
    if (io_dtype == 0) return launch_io<float>(p, stream);
    return launch_io<__bf16>(p, stream);
}

}  // namespace sfm
