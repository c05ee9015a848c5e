// bwd.hip -- backward of the boundary-masked depthwise conv + folded, segmented
// selective scan, for gfx950 (wave64).
//
// The pages give the forward only (the method is trained end to end:
// "Seeing Both Ways, Running One Way" 3.3; techloop walkthrough "第二个模块").
// The gradients here are the chain rule of that forward, run in reverse time
// for each (sample, channel):
//   G_t   = dy_t C_t + a_{t+1} G_{t+1}           (gradient reaching the state h_t)
//   dC_t  = dy_t h_t,  dB_t = G_t Delta_t u_t     (summed over channels)
//   du_t  = D dy_t + sum_n G_t Delta_t B_t
//   dDelta_t = sum_n G_t B_t u_t + [t > 0] sum_n G_t h_{t-1} a_t A
//   dA   += [t > 0] G_t h_{t-1} a_t Delta_t,  dD += dy_t u_t
// then softplus and the conv (with its zero taps outside the sample) backwards.
// The reset at every sample start is a re-initialisation, so no gradient
// crosses from a sample into the one before it in the folded row.
//
// Work mapping: one wave per (folded row b1, tile of 64 channels); lanes are
// channels, the B2 samples of the row run one after the other (the API plans
// the backward unfolded, B2 = 1: one sample per wave).  Per sample:
//  * sweep 1 runs the forward recurrence in chunks of Q = 32/N positions and writes
//    the state entering every chunk (fp32) to a caller-provided workspace;
//  * sweep 2 visits the chunks in reverse: it re-runs the chunk forward from
//    its checkpoint keeping the Q states in registers, then steps backwards.
// Inputs are staged through LDS by direct global->LDS transfers (whole sample
// blocks in bwd_whole_kernel, chunk by chunk in bwd_kernel).  dB and dC (sums
// over channels) are summed over the 64 lanes in registers (lane swaps and a
// DPP butterfly; an LDS transpose in the chunked kernel) and stored as this
// tile's partials; per-channel sums (dA, dD, dbias, dconv) are stored per
// folded row.  bwd_reduce_kernel then adds the partials in a fixed order
// (tiles ascending, folded rows in interleaved strands combined in order), so
// every float32 output is bit-repeatable; nothing uses atomics.  Rows too long
// for enough waves are split along L into segments (a token-sum launch, a carry
// pass, the main pass and a seam launch), see plan_bwd.
#include <stdlib.h>

#include <algorithm>

#include <type_traits>

#include "sfm_device.h"
#include "sfm_bwd.h"
#include "sfm_internal.h"

namespace sfm {

namespace {

#ifndef SFM_BWD_HIST
#define SFM_BWD_HIST 32
#endif
constexpr int kHist = SFM_BWD_HIST;  // states of history per chunk held in registers
constexpr int kFwdQ = 16;            // chunk of the split-row forward (no history kept)
constexpr int kRedStride = 68;  // floats per row of the transpose buffer (16-byte rows, no 16-lane bank clash)

__device__ __forceinline__ float sigmoid_f(float v) { return 1.0f / (1.0f + exp2_fast(-v * kLog2e)); }

// Sums over the 64 lanes of v[0 .. V) (V = 8, 16 or 32), without LDS: a butterfly
// whose exchanges halve the values each lane carries (lanes l and l^32, then
// l^16, by lane swaps; then l^15 and l^7, the mirrors inside 16- and 8-lane
// rows, and l^2 by DPP), followed by plain pairwise sums once one value is
// left.  The exchange masks are independent bits, so every lane's result
// covers all 64 lanes; value j ends in the lanes with lane >> (6 - log2 V) == j.
template <int V>
__device__ __forceinline__ float wave_sum_values(const float (&v)[V], int lane) {
    static_assert(V == 8 || V == 16 || V == 32, "8, 16 or 32 values");
    auto dpp = [](float x, auto ctrlc) __attribute__((always_inline)) {
        constexpr int C = decltype(ctrlc)::value;
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), C, 0xF, 0xF, false));
    };
    using Mirror = std::integral_constant<int, 0x140>;      // lane 15 - i of its 16-lane row
    using HalfMirror = std::integral_constant<int, 0x141>;  // lane 7 - i of its 8-lane half row
    using Xor2 = std::integral_constant<int, 0x4E>;         // quad permute [2, 3, 0, 1]
    using Xor1 = std::integral_constant<int, 0xB1>;         // quad permute [1, 0, 3, 2]
    float a[V / 2];
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
        // lanes 0-31 keep value j, lanes 32-63 value j + V/2
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j + V / 2]), false,
                                                        false);
        a[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    float b[V / 4];
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
        // even 16-lane rows keep value j, odd rows j + V/4
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[j]), __float_as_uint(a[j + V / 4]), false,
                                                        false);
        b[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // a halving step by DPP: lanes with the bit clear keep the lower half
    auto halve = [&](auto& in, auto& out, bool upper, auto ctrlc) __attribute__((always_inline)) {
        constexpr int H = sizeof(out) / sizeof(float);
#pragma unroll
        for (int j = 0; j < H; ++j) {
            const float keep = upper ? in[j + H] : in[j];
            const float send = upper ? in[j] : in[j + H];
            out[j] = keep + dpp(send, ctrlc);
        }
    };
    float x;
    if constexpr (V == 32) {
        float c[4], d[2], e[1];
        halve(b, c, (lane & 8) != 0, Mirror{});
        halve(c, d, (lane & 4) != 0, HalfMirror{});
        halve(d, e, (lane & 2) != 0, Xor2{});
        x = e[0];
    } else if constexpr (V == 16) {
        float c[2], d[1];
        halve(b, c, (lane & 8) != 0, Mirror{});
        halve(c, d, (lane & 4) != 0, HalfMirror{});
        x = d[0];
        x += dpp(x, Xor2{});
    } else {
        float c[1];
        halve(b, c, (lane & 8) != 0, Mirror{});
        x = c[0];
        x += dpp(x, HalfMirror{});
        x += dpp(x, Xor2{});
    }
    return x + dpp(x, Xor1{});
}

// MODE 0: whole rows; 1: rows split into segments (after the carry pass); 2: the carry
// pass; 3: the forward output of split rows (after the carry pass's forward half).
template <typename IO, int NS, int KW, bool CONV, bool SP, bool SILU, int Q, int MODE>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kernel(BwdParams p) {
    constexpr bool SPLIT = MODE != 0;
    constexpr bool CARRY = MODE == 2;
    constexpr bool FWD = MODE == 3;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int XW = Q + KW - 1;  // x window columns of a chunk
    constexpr int R = Q < 32 / NS ? Q : 32 / NS;  // positions per dB/dC transpose round (2*NS*R <= 64 rows)
    static_assert(Q % R == 0, "chunk must hold whole transpose rounds");
    const int lane = threadIdx.x;
    // wave g = ((b1 * tiles) + tile) * seg + s: segment s of the sample row b1 in channel tile `tile`
    const int S = SPLIT ? p.seg : 1;
    const int g = blockIdx.x;
    const int s = g % S;
    const int rt = g / S;
    const int b1 = rt / p.tiles;
    const int tile = rt - b1 * p.tiles;
    const int cbeg = s * p.cps;                  // the segment's chunks [cbeg, cend)
    const int cend = SPLIT ? min(p.nchk, cbeg + p.cps) : p.nchk;
    const int d0 = tile * kWave;
    const int nrows = min(kWave, p.D - d0);
    const int d = d0 + lane;
    const bool valid = lane < nrows;
    const int L = p.L, XL = p.xrow, N = p.N;
    const int P = CONV ? p.P : 0;
    const int sh = p.pad_in ? 1 : 0;  // padded position q reads u row index q - sh

    // staged io elements sit in 4-byte slots (raw bits in the low bytes; see dma_at).
    // Two staging buffers, p.stage_bytes apart; xs, dls, dys, braw, hinl point
    // into the one the current chunk uses (set by use_buf).
    uint32_t* xs;    // [64][XW]: column c = position t0 - P + c
    uint32_t* dls;   // [64][Q]   delta, then ddelta as float32
    uint32_t* dys;   // [64][Q]   dy
    uint32_t* braw;  // [64] raw B then C of the chunk
    float* hinl;     // [NS][64] state entering the chunk (reverse sweep)
    auto buf = [&](int off, int i) __attribute__((always_inline)) { return smem + off + i * p.stage_bytes; };
    auto use_buf = [&](int i) __attribute__((always_inline)) {
        xs = reinterpret_cast<uint32_t*>(buf(p.xs_off, i));
        dls = reinterpret_cast<uint32_t*>(buf(p.ds_off, i));
        dys = reinterpret_cast<uint32_t*>(buf(p.dys_off, i));
        braw = reinterpret_cast<uint32_t*>(buf(p.braw_off, i));
        hinl = reinterpret_cast<float*>(buf(p.hin_off, i));
    };
    use_buf(0);
    float* bs = reinterpret_cast<float*>(smem + p.bc_off);  // [Q][NS]
    float* cs = bs + Q * NS;                               // [Q][NS]
    float* red = reinterpret_cast<float*>(smem + p.red_off);  // [64][kRedStride]
    float* dxs = reinterpret_cast<float*>(smem + p.mean_off);  // [64][XW] fp32 dx of the chunk's window

    // per-channel parameters
    float A[NS], Dk, db, cw[KW], cb;
#pragma unroll
    for (int n = 0; n < NS; ++n) A[n] = (valid && n < N) ? p.A[(size_t)d * N + n] : 0.0f;
    Dk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;
    db = (valid && p.dbias) ? p.dbias[d] : 0.0f;
#pragma unroll
    for (int j = 0; j < KW; ++j) cw[j] = (CONV && valid && j < p.K) ? p.conv_w[(size_t)d * p.K + j] : 0.0f;
    cb = (CONV && valid && p.conv_b) ? p.conv_b[d] : 0.0f;
    float gA[NS], gD = 0.0f, gb = 0.0f, gw[KW], gcb = 0.0f;
#pragma unroll
    for (int n = 0; n < NS; ++n) gA[n] = 0.0f;
#pragma unroll
    for (int j = 0; j < KW; ++j) gw[j] = 0.0f;
    // states n >= N stay zero in the B/C stage
    for (int e = lane; e < Q * NS; e += kWave) {
        bs[e] = 0.0f;
        cs[e] = 0.0f;
    }
    float* ws = p.ws + (size_t)g * (SPLIT ? p.cps : p.nchk) * NS * kWave;  // checkpoints, chunk c at c - cbeg
    // carries of the segment waves of this row and tile: [seg][2 NS + 2][64]
    float* car = p.ws + p.car_off + (size_t)rt * S * (2 * NS + 2) * kWave + lane;
    auto carv = [&](int sg, int k) __attribute__((always_inline)) -> float& {
        return car[((size_t)sg * (2 * NS + 2) + k) * kWave];
    };

    for (int j = 0; j < p.B2; ++j) {
        const int b = b1 * p.B2 + j;
        const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * p.D + d0) * XL;
        const IO* dg = static_cast<const IO*>(p.delta) + ((size_t)b * p.D + d0) * L;
        const IO* yg = static_cast<const IO*>(p.dy) + ((size_t)b * p.D + d0) * L;
        const IO* bgl = static_cast<const IO*>(p.Bm) + (size_t)b * N * L;
        const IO* cgl = static_cast<const IO*>(p.Cm) + (size_t)b * N * L;
        IO* dug = static_cast<IO*>(p.du) + ((size_t)b * p.D + d0) * L;
        IO* ddg = static_cast<IO*>(p.ddelta) + ((size_t)b * p.D + d0) * L;

        // --- staging of one chunk by direct global->LDS transfers of single io elements
        // (consecutive lanes take consecutive positions of a row, so the reads coalesce).
        // Element e of a tile lands in slot tile[e]; elements outside the rows or the sample read
        // a valid dummy element instead and are never used (xv and the widening mask them).
        // Tiles: the x window (padded positions [t0 - P, t0 - P + XW)), delta and dy of
        // positions [t0, t0 + cnt) (dy with its ends exchanged when swap_dy), raw B then C.
        constexpr int EB = (int)sizeof(IO);
        constexpr int kPer = 4096 / (kWave * 4);  // transfers per LDS base (4-byte slots)
        auto dma_tile = [&](auto colsc, uint32_t* tile, int ln, auto addr) __attribute__((always_inline)) {
            constexpr int COLS = decltype(colsc)::value;
            static_for<COLS>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                const int e = k * kWave + ln;
                const int r = e / COLS;
                dma_at<EB, (k % kPer) * kWave * 4>(addr(r, e - r * COLS), tile + (k / kPer) * kPer * kWave);
            });
        };
        // Transfers of chunk (t0, cnt) into staging buffer i; with ck >= 0 also the
        // state entering the segment's chunk ck (its checkpoint, [NS][64] floats
        // contiguous in the workspace, one 4-byte transfer per state).  Nothing is waited for;
        // the buffer was last read by LDS instructions of this wave, which have
        // completed before a transfer can write it.
        auto issue = [&](int t0, int cnt, bool with_dy, bool with_c, int ck, int i) __attribute__((always_inline)) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // An opaque copy of the lane index: the per-lane transfer addresses are
            // recomputed here instead of being hoisted out of the chunk loop, where
            // they would be spilled and their reloads would wait for every transfer
            // in flight.
            int ln = lane;
            asm volatile("" : "+v"(ln));
            uint32_t* xb = reinterpret_cast<uint32_t*>(buf(p.xs_off, i));
            uint32_t* db_ = reinterpret_cast<uint32_t*>(buf(p.ds_off, i));
            uint32_t* yb = reinterpret_cast<uint32_t*>(buf(p.dys_off, i));
            uint32_t* rb = reinterpret_cast<uint32_t*>(buf(p.braw_off, i));
            const IO* dummy = xg;
            dma_tile(std::integral_constant<int, XW>{}, xb, ln, [&](int r, int c) {
                const int q = t0 - P + c - sh;
                return (r < nrows && q >= 0 && q < XL) ? xg + (size_t)r * XL + q : dummy;
            });
            dma_tile(std::integral_constant<int, Q>{}, db_, ln, [&](int r, int c) {
                return (r < nrows && c < cnt) ? dg + (size_t)r * L + t0 + c : dummy;
            });
            if (with_dy) {
                dma_tile(std::integral_constant<int, Q>{}, yb, ln, [&](int r, int c) {
                    const int t = t0 + c;
                    const int ts = (p.swap_dy && L > 1) ? (t == 0 ? L - 1 : (t == L - 1 ? 0 : t)) : t;
                    return (r < nrows && c < cnt) ? yg + (size_t)r * L + ts : dummy;
                });
            }
            {
                // raw B then C: element e < N*Q is B[n = e / Q][t0 + e % Q], the next N*Q are C
                // (one 64-element transfer while 2 NS Q <= 64, as with the register history)
                const int half = N * Q;
                static_for<(2 * NS * Q + kWave - 1) / kWave>([&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    const int e = k * kWave + ln;
                    const int e2 = e < half ? e : e - half;
                    const int n = e2 / Q;
                    const int c = e2 - n * Q;
                    const IO* src = (e < 2 * half && c < cnt && (e < half || with_c))
                                        ? (e < half ? bgl : cgl) + (size_t)n * L + t0 + c
                                        : dummy;
                    dma_at<EB, (k % kPer) * kWave * 4>(src, rb + (k / kPer) * kPer * kWave);
                });
            }
            if (ck >= (SPLIT ? 0 : 1)) {  // (a whole row starts from zero: no checkpoint 0)
                const float* hsrc = ws + (size_t)ck * NS * kWave + ln;
                char* hb = buf(p.hin_off, i);
                static_for<NS>([&](auto nc) {
                    constexpr int n = decltype(nc)::value;
                    dma_at<4, n * kWave * 4>(hsrc + n * kWave, hb);
                });
            }
        };
        // After the chunk in the current buffer has landed: widen B/C to float32
        // [c][n]; states n >= N and positions past the sample are zero.
        auto widen = [&](int cnt, bool with_c) __attribute__((always_inline)) {
            for (int e = lane; e < Q * NS; e += kWave) {
                const int c = e / NS;
                const int n = e - c * NS;
                const bool in = n < N && c < cnt;
                bs[e] = in ? Io<IO>::of_bits(braw[n * Q + c]) : 0.0f;
                cs[e] = (in && with_c) ? Io<IO>::of_bits(braw[N * Q + n * Q + c]) : 0.0f;
            }
        };

        // --- fused aux pad: this row's mean, float64 in index order (as the forward).
        // Split rows: a first kernel adds each segment's tokens in float64 and the
        // partials are added here in segment order (the same value whenever the
        // float64 sums are exact, as for bfloat16 rows of moderate range); the
        // carry pass needs it in the first segment only.
        const double* xpart = reinterpret_cast<const double*>(p.ws + p.meanw_off) + (size_t)rt * S * kWave + lane;
        float mean = 0.0f;
        if (p.pad_in && SPLIT && (!CARRY || s == 0)) {
            double acc = 0.0;
            for (int sg = 0; sg < S; ++sg) acc += xpart[(size_t)sg * kWave];
            mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
        } else if (p.pad_in && !CARRY) {
            // windows of MW tokens of all 64 rows (4-byte slots, rows MW slots apart,
            // MW odd for conflict-free row reads) fill both staging buffers: one
            // direct transfer per row, lanes = tokens, then one wait per window
            const int MW = (min(kWave, 2 * p.stage_bytes / (kWave * 4)) - 1) | 1;
            uint32_t* mwin = reinterpret_cast<uint32_t*>(smem + p.xs_off);
            double acc = 0.0;
            for (int c0 = 0; c0 < XL; c0 += MW) {
                const int cnt = min(MW, XL - c0);
                wave_lds_sync();  // the previous window's reads are done
                if (lane < cnt)
                    for (int r = 0; r < nrows; ++r) dma_at<EB, 0>(xg + (size_t)r * XL + c0 + lane, mwin + r * MW);
                wait_vmem();
                wave_lds_sync();
                for (int c = 0; c < cnt; ++c) acc += (double)Io<IO>::of_bits(mwin[lane * MW + c]);
            }
            mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
        }
        // conv/scan input at padded position q = t0 - P + c (column c of the staged window)
        // An interior chunk (full tile, all Q positions, the x window clear of
        // the sample ends and of the aux tokens, past the sample start) needs
        // none of the per-position checks; FAST variants drop them.
        auto xv = [&](auto fastc, int t0, int c) __attribute__((always_inline)) {
            constexpr bool FAST = decltype(fastc)::value;
            const int q = t0 - P + c;
            float v = Io<IO>::of_bits(xs[lane * XW + c]);
            if constexpr (FAST) return v;
            if (p.pad_in && (q == 0 || q == L - 1)) v = mean;
            return (valid && q >= 0 && q < L) ? v : 0.0f;  // zero taps outside the sample
        };
        // z (pre-activation), u, v (pre-softplus) and Delta*log2e at position t0 + i
        auto pre = [&](auto fastc, int t0, int i, float& z, float& u, float& v, float& dt)
                       __attribute__((always_inline)) {
            constexpr bool FAST = decltype(fastc)::value;
            if constexpr (CONV) {
                float acc = cb;
#pragma unroll
                for (int jj = 0; jj < KW; ++jj) acc = __builtin_fmaf(cw[jj], xv(fastc, t0, i + jj), acc);
                z = acc;
                u = SILU ? silu(acc) : acc;
            } else {
                z = xv(fastc, t0, i + P);
                u = z;
            }
            v = ((FAST || valid) ? Io<IO>::of_bits(dls[lane * Q + i]) : 0.0f) + db;
            dt = SP ? softplus_log2e(v) * kLn2 : v;
        };
        // With 16 states the second copy of a chunk body costs more in spills than
        // it saves, so only the narrower state widths take the interior path.
        constexpr bool kInteriorPath = NS <= 8;
        auto interior = [&](int t0, int cnt) __attribute__((always_inline)) {
            const int edge = p.pad_in ? 1 : 0;
            return nrows == kWave && cnt == Q && t0 > 0 && t0 - P >= edge && t0 - P + XW - 1 <= L - 1 - edge;
        };

        // --- sweep 1: forward, checkpoint the state entering each chunk.  The
        // transfers of chunk c+1 go out (into the other buffer) once chunk c has
        // landed, so they are in flight while chunk c runs.
        float h[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = 0.0f;
        if constexpr (!CARRY) {
            // the state entering the segment: the earlier segments' carries composed
            // in order, each the state its segment reaches from zero plus the product
            // of its decays, exp2(A * sum of Delta*log2e), times the state before it
            for (int sg = 0; sg < s; ++sg) {
                const float sd = carv(sg, 2 * NS);
#pragma unroll
                for (int n = 0; n < NS; ++n) h[n] = __builtin_fmaf(exp2_fast(sd * A[n]), h[n], carv(sg, n));
            }
        }
        float sdt = 0.0f;  // carry pass: sum of Delta*log2e over the segment
        int bi = 0;
        // (the carry pass needs the forward for every segment but the row's last)
        const int cstop = (!CARRY || s < S - 1) ? cend : cbeg;
        wave_lds_sync();
        if (cbeg < cstop) issue(cbeg * Q, min(Q, L - cbeg * Q), false, FWD, -1, 0);
        for (int c = cbeg; c < cstop; ++c) {
            const int t0 = c * Q;
            const int cnt = min(Q, L - t0);
            wait_vmem();
            wave_lds_sync();
            // widen before the next transfers go out: any wait on vector memory
            // the compiler puts here then covers nothing in flight
            use_buf(bi);
            widen(cnt, FWD);
            if (!CARRY && !FWD && (SPLIT || c > 0)) {
#pragma unroll
                for (int n = 0; n < NS; ++n) ws[((size_t)(c - cbeg) * NS + n) * kWave + lane] = h[n];
            }
            if (c + 1 < cend) issue(t0 + Q, min(Q, L - t0 - Q), false, FWD, -1, bi ^ 1);
            wave_lds_sync();
            auto fwd = [&](auto fastc) __attribute__((always_inline)) {
                constexpr bool FAST = decltype(fastc)::value;
                for (int i = 0; i < (FAST ? Q : cnt); ++i) {
                    float z, u, v, dt;
                    pre(fastc, t0, i, z, u, v, dt);
                    if constexpr (CARRY) sdt += dt * kLog2e;
                    const float du_ = dt * u;
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        const float bx = du_ * bs[i * NS + n];
                        h[n] = (!FAST && t0 + i == 0) ? bx : __builtin_fmaf(exp2_fast(dt * kLog2e * A[n]), h[n], bx);
                    }
                    if constexpr (FWD) {
                        // y = C.h + D u, in place of this position's delta (already read)
                        float yv = Dk * u;
#pragma unroll
                        for (int n = 0; n < NS; ++n) yv = __builtin_fmaf(cs[i * NS + n], h[n], yv);
                        dls[lane * Q + i] = __float_as_uint(yv);
                    }
                }
            };
            if constexpr (kInteriorPath) {
                if (interior(t0, cnt)) fwd(std::true_type{});
                else fwd(std::false_type{});
            } else {
                fwd(std::false_type{});
            }
            if constexpr (FWD) {
                // this chunk's y, coalesced (the fused swap exchanges the sample's ends)
                wave_lds_sync();
                IO* yo = static_cast<IO*>(p.y) + ((size_t)b * p.D + d0) * L;
                for (int e = lane; e < kWave * Q; e += kWave) {
                    const int r = e / Q;
                    const int cc = e - r * Q;
                    if (r < nrows && cc < cnt) {
                        int t = t0 + cc;
                        if (p.swap_out && L > 1) t = t == 0 ? L - 1 : (t == L - 1 ? 0 : t);
                        yo[(size_t)r * L + t] = from_f32<IO>(__uint_as_float(dls[r * Q + cc]));
                    }
                }
            }
            bi ^= 1;
        }
        if constexpr (CARRY) {
            if (s < S - 1) {
#pragma unroll
                for (int n = 0; n < NS; ++n) carv(s, n) = h[n];
                carv(s, 2 * NS) = sdt;
            }
        }

        // --- carry pass: the carried output gradient the segment passes to its
        // start, reached from zero at its end (no states needed: only the decays
        // and C*dy), and the sum of Delta*log2e, for every segment but the row's first
        if constexpr (CARRY) {
            if (s > 0 && !p.fwd) {
                float Gc[NS];
#pragma unroll
                for (int n = 0; n < NS; ++n) Gc[n] = 0.0f;
                float sdr = 0.0f;
                wait_vmem();
                wave_lds_sync();
                bi = 0;
                issue((cend - 1) * Q, min(Q, L - (cend - 1) * Q), true, true, -1, 0);
                for (int c = cend - 1; c >= cbeg; --c) {
                    const int t0 = c * Q;
                    const int cnt = min(Q, L - t0);
                    wait_vmem();
                    wave_lds_sync();
                    use_buf(bi);
                    widen(cnt, true);
                    if (c > cbeg) issue(t0 - Q, Q, true, true, -1, bi ^ 1);
                    wave_lds_sync();
                    for (int i = cnt - 1; i >= 0; --i) {
                        float z, u, v, dt;
                        pre(std::false_type{}, t0, i, z, u, v, dt);
                        const float dtl = dt * kLog2e;
                        sdr += dtl;
                        const float gy = valid ? Io<IO>::of_bits(dys[lane * Q + i]) : 0.0f;
#pragma unroll
                        for (int n = 0; n < NS; ++n)
                            Gc[n] = exp2_fast(dtl * A[n]) * __builtin_fmaf(gy, cs[i * NS + n], Gc[n]);
                    }
                    bi ^= 1;
                }
#pragma unroll
                for (int n = 0; n < NS; ++n) carv(s, NS + n) = Gc[n];
                carv(s, 2 * NS + 1) = sdr;
            }
        } else if constexpr (!FWD) {

        // --- sweep 2: chunks in reverse.  Chunk c-1's transfers (with its
        // entering state) go out once chunk c has landed; chunk c's ddelta (in
        // its buffer) and finished dx (dxs) leave one chunk later, after that
        // wait, so no wait covers those stores.
        auto write_out = [&](int c) __attribute__((always_inline)) {
            const int t0 = c * Q;
            const int cnt = min(Q, L - t0);
            // write this chunk's ddelta and the completed dx positions (coalesced)
            for (int e = lane; e < kWave * Q; e += kWave) {
                const int r = e / Q;
                const int cc = e - r * Q;
                if (r < nrows && cc < cnt) ddg[(size_t)r * L + t0 + cc] = from_f32<IO>(__uint_as_float(dls[r * Q + cc]));
            }
            // dx columns finished in this chunk: padded positions [lo, hi)
            const int lag = CONV ? KW - 1 - P : 0;
            const int lo = CONV ? (c == cbeg ? max(0, t0 - P) : t0 + lag) : t0;
            const int hi = CONV ? min(L, t0 + cnt + lag) : t0 + cnt;
            // split rows: the kw - 1 positions around a segment boundary take
            // contributions from both segments; each writes its partial to the
            // workspace ([leading | trailing][kw - 1][64]) for the seam kernel
            const int s0 = cbeg * Q, s1 = cend * Q;
            float* seam = p.ws + p.seam_off + (size_t)g * 2 * (KW - 1) * kWave;
            for (int e = lane; e < kWave * XW; e += kWave) {
                const int r = e / XW;
                const int cc = e - r * XW;
                const int q = t0 - P + cc;
                if (r < nrows && q >= lo && q < hi) {
                    const float v = dxs[r * XW + cc];
                    if (CONV && SPLIT && s > 0 && q < s0 + lag)
                        seam[(size_t)(q - s0 + P) * kWave + r] = v;
                    else if (CONV && SPLIT && s < S - 1 && q >= s1 - P)
                        seam[(size_t)(KW - 1 + q - s1 + P) * kWave + r] = v;
                    else
                        dug[(size_t)r * L + q] = from_f32<IO>(v);
                }
            }
        };
        float G[NS];  // a_{t+1} G_{t+1} carried to position t
#pragma unroll
        for (int n = 0; n < NS; ++n) G[n] = 0.0f;
        // entering the segment's end: the later segments' carries composed from the row's end
        for (int sg = S - 1; sg > s; --sg) {
            const float sd = carv(sg, 2 * NS + 1);
#pragma unroll
            for (int n = 0; n < NS; ++n) G[n] = __builtin_fmaf(exp2_fast(sd * A[n]), G[n], carv(sg, NS + n));
        }
        float wdx[KW];  // dx of padded positions t - P + jj, still collecting contributions
#pragma unroll
        for (int jj = 0; jj < KW; ++jj) wdx[jj] = 0.0f;
        wait_vmem();  // the checkpoints stored above have landed before they are read back
        wave_lds_sync();
        bi = 0;
        issue((cend - 1) * Q, min(Q, L - (cend - 1) * Q), true, true, cend - 1 - cbeg, 0);
        int pend = -1;  // chunk whose outputs wait in buffer bi ^ 1 and dxs
        for (int c = cend - 1; c >= cbeg; --c) {
            const int t0 = c * Q;
            const int cnt = min(Q, L - t0);
            wait_vmem();
            wave_lds_sync();
            use_buf(bi);
            widen(cnt, true);  // before any transfer goes out (as in the forward sweep)
            if (pend >= 0) {
                use_buf(bi ^ 1);
                write_out(pend);
            }
            if (c > cbeg) issue(t0 - Q, Q, true, true, c - 1 - cbeg, bi ^ 1);
            use_buf(bi);
            for (int e = lane; e < kWave * XW; e += kWave) dxs[e] = 0.0f;
            float hin[NS];
#pragma unroll
            for (int n = 0; n < NS; ++n) hin[n] = (SPLIT || c > 0) ? hinl[n * kWave + lane] : 0.0f;
            wave_lds_sync();
            auto chunk = [&](auto fastc) __attribute__((always_inline)) {
                constexpr bool FAST = decltype(fastc)::value;
                // re-run the chunk forward, keeping every state
                float hs[Q][NS];
                float zs[Q], us[Q], vs[Q], dts[Q];
#pragma unroll
                for (int i = 0; i < Q; ++i) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (FAST || i < cnt) {
                        pre(fastc, t0, i, zs[i], us[i], vs[i], dts[i]);
                        const float du_ = dts[i] * us[i];
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            const float hp = i > 0 ? hs[i - 1][n] : hin[n];
                            const float bx = du_ * bs[i * NS + n];
                            hs[i][n] = (!FAST && t0 + i == 0) ? bx : __builtin_fmaf(exp2_fast(dts[i] * kLog2e * A[n]), hp, bx);
                        }
                    }
                }
                // backwards through the chunk, R positions per dB/dC transpose round
#pragma unroll
                for (int r0 = Q - R; r0 >= 0; r0 -= R) {
#pragma unroll
                    for (int ii = R - 1; ii >= 0; --ii) {
                        const int i = r0 + ii;
                        // one position at a time: keeps the schedule (and register use) to one step
                        __builtin_amdgcn_sched_barrier(0);
                        float dBv[NS], dCv[NS];
#pragma unroll
                        for (int n = 0; n < NS; ++n) dBv[n] = dCv[n] = 0.0f;
                        if (FAST || i < cnt) {
                            const int t = t0 + i;
                            const float gy = (FAST || valid) ? Io<IO>::of_bits(dys[lane * Q + i]) : 0.0f;
                            const float u = us[i], dt = dts[i];
                            float du_ = Dk * gy;
                            float ddt = 0.0f;
                            gD = __builtin_fmaf(gy, u, gD);
#pragma unroll
                            for (int n = 0; n < NS; ++n) {
                                const float Bv = bs[i * NS + n], Cv = cs[i * NS + n];
                                const float Gn = __builtin_fmaf(gy, Cv, G[n]);
                                dCv[n] = gy * hs[i][n];
                                dBv[n] = Gn * dt * u;
                                du_ = __builtin_fmaf(Gn * dt, Bv, du_);
                                ddt = __builtin_fmaf(Gn * Bv, u, ddt);
                                if (FAST || t > 0) {
                                    const float hp = i > 0 ? hs[i - 1][n] : hin[n];
                                    const float a = exp2_fast(dt * kLog2e * A[n]);
                                    const float w = a * Gn;    // carried to position t - 1
                                    const float dat = w * hp;  // dLoss/da_t times a_t
                                    ddt = __builtin_fmaf(dat, A[n], ddt);
                                    gA[n] = __builtin_fmaf(dat, dt, gA[n]);
                                    G[n] = w;
                                } else {
                                    G[n] = 0.0f;  // reset: nothing reaches the previous sample
                                }
                            }
                            float dv = ddt;
                            if constexpr (SP) dv = vs[i] > 20.0f ? ddt : ddt * sigmoid_f(vs[i]);
                            dls[lane * Q + i] = __float_as_uint(dv);
                            gb += dv;
                            float dz = du_;
                            if constexpr (CONV && SILU) {
                                const float s = sigmoid_f(zs[i]);
                                dz = du_ * (s + zs[i] * s * (1.0f - s));
                            }
                            if constexpr (CONV) {
                                gcb += dz;
#pragma unroll
                                for (int jj = 0; jj < KW; ++jj) {
                                    gw[jj] = __builtin_fmaf(dz, xv(fastc, t0, i + jj), gw[jj]);
                                    wdx[jj] = __builtin_fmaf(dz, cw[jj], wdx[jj]);
                                }
                                // padded position t + lag is complete: it gets no later contribution
                                dxs[lane * XW + i + KW - 1] = wdx[KW - 1];
#pragma unroll
                                for (int jj = KW - 1; jj > 0; --jj) wdx[jj] = wdx[jj - 1];
                                wdx[0] = 0.0f;
                            } else {
                                dxs[lane * XW + i + P] = dz;
                            }
                        }
                        // transpose buffer: row (ii, k), column lane
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            red[(ii * 2 * NS + n) * kRedStride + lane] = dBv[n];
                            red[(ii * 2 * NS + NS + n) * kRedStride + lane] = dCv[n];
                        }
                    }
                    wave_lds_sync();
                    {
                        // lane l sums row l: position r0 + l / (2NS), state l % NS, B or C
                        const int ii = lane / (2 * NS);
                        const int k = lane - ii * 2 * NS;
                        const int n = k % NS;
                        const int t = t0 + r0 + ii;
                        const float4* row = reinterpret_cast<const float4*>(red + lane * kRedStride);
                        float s = 0.0f;
#pragma unroll
                        for (int m = 0; m < kWave / 4; ++m) {
                            const float4 v4 = row[m];
                            s += (v4.x + v4.y) + (v4.z + v4.w);
                        }
                        if (lane < 2 * NS * R && r0 + ii < cnt)
                            p.ws[p.pbc_off + (((size_t)tile * p.B1 * p.B2 + b) * L + t) * 2 * NS + k] = s;
                    }
                    wave_lds_sync();
                }
            };
            if constexpr (kInteriorPath) {
                if (interior(t0, cnt)) chunk(std::true_type{});
                else chunk(std::false_type{});
            } else {
                chunk(std::false_type{});
            }
            if constexpr (CONV) {
                // positions t0 - P .. t0 + lag - 1 are complete once the sample (or
                // segment: a partial) start is passed
                if (c == cbeg) {
                    // after the last shift wdx[m] holds padded position m - 1 - P,
                    // i.e. window column m - 1
#pragma unroll
                    for (int jj = 0; jj < KW - 1; ++jj) dxs[lane * XW + jj] = wdx[jj + 1];
                }
            }
            pend = c;
            bi ^= 1;
        }
        wave_lds_sync();
        use_buf(bi ^ 1);
        write_out(pend);
        wave_lds_sync();
        }  // sweep 2
    }
    if (!CARRY && !FWD && valid) {
        // this row segment's per-channel sums (rows dA[0..N), dD, dbias, dconv_b, dconv_w[0..K))
        float* pc = p.ws + p.pch_off + ((size_t)b1 * S + s) * p.kc * p.D + d;
#pragma unroll
        for (int n = 0; n < NS; ++n)
            if (n < N) pc[(size_t)n * p.D] = gA[n];
        pc[(size_t)N * p.D] = gD;
        pc[(size_t)(N + 1) * p.D] = gb;
        if constexpr (CONV) {
            pc[(size_t)(N + 2) * p.D] = gcb;
#pragma unroll
            for (int jj = 0; jj < KW; ++jj)
                if (jj < p.K) pc[(size_t)(N + 3 + jj) * p.D] = gw[jj];
        }
    }
}

// Whole-sample variant.  The x, delta and dy blocks of one sample and channel
// tile are each one contiguous range of memory ([rows][length], rows = the
// tile's channels), so they are staged once per sample with 16-byte direct
// transfers and serve both sweeps.  ddelta replaces delta in place (position t
// is overwritten after its last read) and the conv-input gradient replaces dy
// (position q is complete only after dy at q was read; the two dy values at the
// sample ends are read up front because swap_dy moves them).  Both blocks leave
// with 16-byte stores once the sample is done.  B and C of the sample are
// widened to float32 once.  dB/dC of each position are summed over the
// channels in registers (wave_sum_values), so the kernel's LDS is the three
// blocks and B/C only: seven workgroups fit a compute unit at stage-4 sizes.
// Channel-last staging: `rows` position rows of this tile (units_per_row 16-byte
// units each, rows `stride` elements apart from `base`) into LDS back to back,
// unit u at l + 16 u.  Four transfers share one LDS base; nothing is waited for.
template <typename IO>
__device__ __forceinline__ void dma_rows(const IO* base, int rows, int stride, int units_per_row, float inv_upr,
                                         IO* l, int lane) {
    const int units = rows * units_per_row;
    const char* g = reinterpret_cast<const char*>(base);
    auto src = [&](int u) __attribute__((always_inline)) {
        const int r = div_small(u, inv_upr);
        return g + (size_t)r * stride * sizeof(IO) + (size_t)(u - r * units_per_row) * 16;
    };
    char* lb = reinterpret_cast<char*>(l);
    for (int u0 = 0; u0 < units; u0 += 4 * kWave) {
        char* ll = lb + u0 * 16;
        const int u = u0 + lane;
        const int rem = units - u;
        if (rem > 0) dma_at<16, 0>(src(u), ll);
        if (rem > 64) dma_at<16, 1024>(src(u + 64), ll);
        if (rem > 128) dma_at<16, 2048>(src(u + 128), ll);
        if (rem > 192) dma_at<16, 3072>(src(u + 192), ll);
    }
}

template <typename IO, int NS, int KW, bool CONV, bool SP, bool SILU, int Q, bool CL>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2))) void bwd_whole_kernel(BwdParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int R = 16 / NS;  // positions per round of the reverse walk
    static_assert(Q % R == 0, "chunk must hold whole transpose rounds");
    constexpr int EB = (int)sizeof(IO);
    const int lane = threadIdx.x;
    const int g = blockIdx.x;
    const int b1 = g / p.tiles;
    const int tile = g - b1 * p.tiles;
    const int d0 = tile * kWave;
    const int nrows = min(kWave, p.D - d0);
    const int d = d0 + lane;
    const bool valid = lane < nrows;
    const int L = p.L, XL = p.xrow, N = p.N;
    const int P = CONV ? p.P : 0;
    const int sh = p.pad_in ? 1 : 0;  // padded position q reads u row index q - sh
    const int lag = CONV ? KW - 1 - P : 0;  // dx of position t + lag is complete after step t

    // channel-first: [rows][XL] x, [rows][L] delta/ddelta and dy/dx (one row per channel);
    // channel-last (CL): the same blocks as [XL][rows] and [L][rows] (one row per position)
    IO* xs = reinterpret_cast<IO*>(smem + p.xs_off);
    IO* ds = reinterpret_cast<IO*>(smem + p.ds_off);        // delta, then ddelta
    IO* ys = reinterpret_cast<IO*>(smem + p.dys_off);       // dy, then dx
    float* bs = reinterpret_cast<float*>(smem + p.bc_off);  // [L][NS]
    float* cs = bs + L * NS;                                // [L][NS]
    const int col = valid ? lane : 0;  // lanes past the tile read channel 0 and mask the value
    const int xrow = col * XL;
    const int row = col * L;
    // LDS element of this lane's channel at x position q / at position t
    auto xi = [&](int q) __attribute__((always_inline)) { return CL ? q * nrows + col : xrow + q; };
    auto ti = [&](int t) __attribute__((always_inline)) { return CL ? t * nrows + col : row + t; };
    const int upr = nrows * EB / 16;  // channel-last: 16-byte units per position row (whole, by the plan)
    const float inv_upr = 1.0f / (float)upr;
    // one position's NS float32 values of B (or C) as whole 16-byte reads
    auto bc_row = [&](const float* base, int t, float (&v)[NS]) __attribute__((always_inline)) {
        const float4* r = reinterpret_cast<const float4*>(base + t * NS);
#pragma unroll
        for (int k = 0; k < NS / 4; ++k) {
            const float4 w = r[k];
            v[4 * k] = w.x;
            v[4 * k + 1] = w.y;
            v[4 * k + 2] = w.z;
            v[4 * k + 3] = w.w;
        }
    };

    float A[NS], Dk, db, cw[KW], cb;
#pragma unroll
    for (int n = 0; n < NS; ++n) A[n] = (valid && n < N) ? p.A[(size_t)d * N + n] : 0.0f;
    Dk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;
    db = (valid && p.dbias) ? p.dbias[d] : 0.0f;
#pragma unroll
    for (int j = 0; j < KW; ++j) cw[j] = (CONV && valid && j < p.K) ? p.conv_w[(size_t)d * p.K + j] : 0.0f;
    cb = (CONV && valid && p.conv_b) ? p.conv_b[d] : 0.0f;
    float gA[NS], gD = 0.0f, gb = 0.0f, gw[KW], gcb = 0.0f;
#pragma unroll
    for (int n = 0; n < NS; ++n) gA[n] = 0.0f;
#pragma unroll
    for (int j = 0; j < KW; ++j) gw[j] = 0.0f;
    // states n >= N stay zero in the B/C stage
    for (int e = lane; e < L * NS; e += kWave)
        if (e % NS >= N) bs[e] = cs[e] = 0.0f;
    float* ws = p.ws + (size_t)g * p.nchk * NS * kWave + lane;
    const int NL = N * L;
    const float inv_L = 1.0f / (float)L;
    const float inv_N = 1.0f / (float)N;

    for (int j = 0; j < p.B2; ++j) {
        const int b = b1 * p.B2 + j;
        const size_t xoff = CL ? (size_t)b * XL * p.D + d0 : ((size_t)b * p.D + d0) * XL;
        const size_t toff = CL ? (size_t)b * L * p.D + d0 : ((size_t)b * p.D + d0) * L;
        const IO* bgl = static_cast<const IO*>(p.Bm) + (size_t)b * NL;
        const IO* cgl = static_cast<const IO*>(p.Cm) + (size_t)b * NL;
        wave_lds_sync();  // the previous sample's LDS reads are done
        // --- staging: B/C element loads (8 per lane in flight), then the three blocks
        for (int e0 = 0; e0 < NL; e0 += 8 * kWave) {
            IO bv[8], cv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = e0 + k * kWave + lane;
                bv[k] = e < NL ? bgl[e] : Io<IO>::zero();
                cv[k] = e < NL ? cgl[e] : Io<IO>::zero();
            }
            if (e0 == 0) {
                if constexpr (CL) {
                    dma_rows(static_cast<const IO*>(p.u) + xoff, XL, p.D, upr, inv_upr, xs, lane);
                    dma_rows(static_cast<const IO*>(p.delta) + toff, L, p.D, upr, inv_upr, ds, lane);
                    dma_rows(static_cast<const IO*>(p.dy) + toff, L, p.D, upr, inv_upr, ys, lane);
                } else {
                    dma_to_lds(static_cast<const IO*>(p.u) + xoff, xs, nrows * XL * EB, lane);
                    dma_to_lds(static_cast<const IO*>(p.delta) + toff, ds, nrows * L * EB, lane);
                    dma_to_lds(static_cast<const IO*>(p.dy) + toff, ys, nrows * L * EB, lane);
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = e0 + k * kWave + lane;
                if (e < NL) {
                    // B, C of the sample: [N][L] channel-first, [L][N] channel-last
                    int n, t;
                    if constexpr (CL) {
                        t = div_small(e, inv_N);
                        n = e - t * N;
                    } else {
                        n = div_small(e, inv_L);
                        t = e - n * L;
                    }
                    bs[t * NS + n] = to_f32(bv[k]);
                    cs[t * NS + n] = to_f32(cv[k]);
                }
            }
        }
        wait_vmem();
        wave_lds_sync();

        // --- fused aux pad: this row's mean, float64 in index order (as the forward)
        float mean = 0.0f;
        if (p.pad_in) {
            double acc = 0.0;
            for (int c = 0; c < XL; ++c) acc += (double)to_f32(xs[xi(c)]);
            mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
        }
        // conv/scan input at padded position q (zero outside the sample)
        auto xv = [&](int q) __attribute__((always_inline)) {
            const int qc = min(max(q - sh, 0), XL - 1);
            float v = to_f32(xs[xi(qc)]);
            if (p.pad_in && (q == 0 || q == L - 1)) v = mean;
            return (valid && q >= 0 && q < L) ? v : 0.0f;
        };
        constexpr int XW = Q + KW - 1;  // conv input window of a chunk
        // window of the chunk at t0: xw[c] = input at padded position t0 - P + c
        auto window = [&](int t0, float (&xw)[XW]) __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < XW; ++c) xw[c] = xv(t0 - P + c);
        };
        // z (pre-activation), u, v (pre-softplus), Delta and Delta*log2e at position t = t0 + i
        auto pre = [&](const float (&xw)[XW], int t, int i, float& z, float& u, float& v, float& dt, float& dtl)
            __attribute__((always_inline)) {
            if constexpr (CONV) {
                float acc = cb;
#pragma unroll
                for (int jj = 0; jj < KW; ++jj) acc = __builtin_fmaf(cw[jj], xw[i + jj], acc);
                z = acc;
                u = SILU ? silu(acc) : acc;
            } else {
                z = xw[i];
                u = z;
            }
            v = (valid ? to_f32(ds[ti(t)]) : 0.0f) + db;
            if constexpr (SP) {
                dtl = softplus_log2e(v);
                dt = dtl * kLn2;
            } else {
                dt = v;
                dtl = v * kLog2e;
            }
        };
        // dy at the two sample ends, before the dx written in place can cover them
        const int ce0 = (p.swap_dy && L > 1) ? L - 1 : 0;
        const float gy_first = valid ? to_f32(ys[ti(ce0)]) : 0.0f;
        const float gy_last = valid ? to_f32(ys[ti(L - 1 - ce0)]) : 0.0f;

        // --- sweep 1: forward, checkpoint the state entering each chunk
        {
            float h[NS];
#pragma unroll
            for (int n = 0; n < NS; ++n) h[n] = 0.0f;
            for (int c = 0; c < p.nchk; ++c) {
                const int t0 = c * Q;
                const int cnt = min(Q, L - t0);
                if (c > 0) {
#pragma unroll
                    for (int n = 0; n < NS; ++n) ws[((size_t)c * NS + n) * kWave] = h[n];
                }
                float xw[XW];
                window(t0, xw);
                // the chunk's per-position inputs first (independent), then the state chain
                float dus[Q], dtls[Q];
#pragma unroll
                for (int i = 0; i < Q; ++i) {
                    float z, u, v, dt;
                    pre(xw, t0 + min(i, cnt - 1), i, z, u, v, dt, dtls[i]);
                    dus[i] = dt * u;
                }
#pragma unroll
                for (int i = 0; i < Q; ++i) {
                    if (i < cnt) {
                        float Bv[NS];
                        bc_row(bs, t0 + i, Bv);
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            const float bx = dus[i] * Bv[n];
                            h[n] = (c == 0 && i == 0) ? bx : __builtin_fmaf(exp2_fast(dtls[i] * A[n]), h[n], bx);
                        }
                    }
                }
            }
        }

        // --- sweep 2: chunks in reverse
        float G[NS];  // a_{t+1} G_{t+1} carried to position t
#pragma unroll
        for (int n = 0; n < NS; ++n) G[n] = 0.0f;
        float wdx[KW];  // dx of padded positions t - P + jj, still collecting contributions
#pragma unroll
        for (int jj = 0; jj < KW; ++jj) wdx[jj] = 0.0f;
        float hnext[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) hnext[n] = p.nchk > 1 ? ws[((size_t)(p.nchk - 1) * NS + n) * kWave] : 0.0f;
        for (int c = p.nchk - 1; c >= 0; --c) {
            const int t0 = c * Q;
            const int cnt = min(Q, L - t0);
            float hin[NS];
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                hin[n] = c > 0 ? hnext[n] : 0.0f;
                // the next chunk's checkpoint, in flight while this chunk runs
                if (c > 1) hnext[n] = ws[((size_t)(c - 1) * NS + n) * kWave];
            }
            // re-run the chunk forward, keeping every state
            float hs[Q][NS];
            float zs[Q], us[Q], vs[Q], dts[Q], dtls[Q];
            float xw[XW];
            window(t0, xw);
            // the chunk's per-position inputs first (independent), then the state chain
            float gys[Q];
#pragma unroll
            for (int i = 0; i < Q; ++i) {
                const int t = t0 + min(i, cnt - 1);
                pre(xw, t, i, zs[i], us[i], vs[i], dts[i], dtls[i]);
                gys[i] = t == 0 ? gy_first : (t == L - 1 ? gy_last : (valid ? to_f32(ys[ti(t)]) : 0.0f));
            }
#pragma unroll
            for (int i = 0; i < Q; ++i) {
                if (i < cnt) {
                    const float du_ = dts[i] * us[i];
                    float Bv[NS];
                    bc_row(bs, t0 + i, Bv);
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        const float hp = i > 0 ? hs[i - 1][n] : hin[n];
                        const float bx = du_ * Bv[n];
                        hs[i][n] = (c == 0 && i == 0) ? bx : __builtin_fmaf(exp2_fast(dtls[i] * A[n]), hp, bx);
                    }
                }
            }
            // backwards through the chunk, R positions per dB/dC transpose round
#pragma unroll
            for (int r0 = Q - R; r0 >= 0; r0 -= R) {
#pragma unroll
                for (int ii = R - 1; ii >= 0; --ii) {
                    const int i = r0 + ii;
                    // one position at a time: keeps the schedule (and register use) to one step
                    __builtin_amdgcn_sched_barrier(0);
                    float dBv[NS], dCv[NS];
#pragma unroll
                    for (int n = 0; n < NS; ++n) dBv[n] = dCv[n] = 0.0f;
                    if (i < cnt) {
                        const int t = t0 + i;
                        const float gy = gys[i];
                        const float u = us[i], dt = dts[i], dtu = dt * u;
                        float sb = 0.0f;  // sum_n G_n B_n
                        float sa = 0.0f;  // sum_n G_n h_{t-1,n} a_n A_n
                        gD = __builtin_fmaf(gy, u, gD);
                        float Bt[NS], Ct[NS];
                        bc_row(bs, t, Bt);
                        bc_row(cs, t, Ct);
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            const float Bv = Bt[n], Cv = Ct[n];
                            const float Gn = __builtin_fmaf(gy, Cv, G[n]);
                            dCv[n] = gy * hs[i][n];
                            dBv[n] = Gn * dtu;
                            sb = __builtin_fmaf(Gn, Bv, sb);
                            if (c > 0 || i > 0) {
                                const float hp = i > 0 ? hs[i - 1][n] : hin[n];
                                const float a = exp2_fast(dtls[i] * A[n]);
                                const float w = a * Gn;    // carried to position t - 1
                                const float dat = w * hp;  // dLoss/da_t times a_t
                                sa = __builtin_fmaf(dat, A[n], sa);
                                gA[n] = __builtin_fmaf(dat, dt, gA[n]);
                                G[n] = w;
                            } else {
                                G[n] = 0.0f;  // reset: nothing reaches the previous sample
                            }
                        }
                        const float ddt = __builtin_fmaf(sb, u, sa);
                        float dv = ddt;
                        if constexpr (SP) dv = vs[i] > 20.0f ? ddt : ddt * sigmoid_f(vs[i]);
                        if (valid) ds[ti(t)] = from_f32<IO>(dv);
                        gb += dv;
                        const float du_ = __builtin_fmaf(dt, sb, Dk * gy);
                        float dz = du_;
                        if constexpr (CONV && SILU) {
                            const float s = sigmoid_f(zs[i]);
                            dz = du_ * (s + zs[i] * s * (1.0f - s));
                        }
                        if constexpr (CONV) {
                            gcb += dz;
#pragma unroll
                            for (int jj = 0; jj < KW; ++jj) {
                                gw[jj] = __builtin_fmaf(dz, xw[i + jj], gw[jj]);
                                wdx[jj] = __builtin_fmaf(dz, cw[jj], wdx[jj]);
                            }
                            // padded position t + lag gets no later contribution
                            if (valid && t + lag < L) ys[ti(t + lag)] = from_f32<IO>(wdx[KW - 1]);
#pragma unroll
                            for (int jj = KW - 1; jj > 0; --jj) wdx[jj] = wdx[jj - 1];
                            wdx[0] = 0.0f;
                        } else {
                            if (valid) ys[ti(t)] = from_f32<IO>(dz);
                        }
                    }
                    // dB/dC of this position summed over the channels (lanes) in registers:
                    // value k (dB_n for k = n, dC_n for k = NS + n) in lanes k * 64 / (2 NS) ..
                    float dv2[2 * NS];
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        dv2[n] = dBv[n];
                        dv2[NS + n] = dCv[n];
                    }
                    const float sum = wave_sum_values<2 * NS>(dv2, lane);
                    constexpr int kShift = NS == 16 ? 1 : (NS == 8 ? 2 : 3);
                    if ((lane & ((1 << kShift) - 1)) == 0 && i < cnt)
                        p.ws[p.pbc_off + (((size_t)tile * p.B1 * p.B2 + b) * L + t0 + i) * 2 * NS + (lane >> kShift)] =
                            sum;
                }
            }
        }
        if constexpr (CONV) {
            // after the step at t = 0 and its shift, wdx[m] holds padded position m - 1 - P
#pragma unroll
            for (int m = 1; m < KW; ++m) {
                const int q = m - 1 - P;
                if (valid && q >= 0 && q < L) ys[ti(q)] = from_f32<IO>(wdx[m]);
            }
        }
        wave_lds_sync();
        // --- ddelta and dx leave as whole blocks
        {
            const int units = nrows * L * EB / 16;
            const uint4* sd = reinterpret_cast<const uint4*>(ds);
            const uint4* sy = reinterpret_cast<const uint4*>(ys);
            char* gd = reinterpret_cast<char*>(static_cast<IO*>(p.ddelta) + toff);
            char* gu = reinterpret_cast<char*>(static_cast<IO*>(p.du) + toff);
            for (int u = lane; u < units; u += kWave) {
                size_t off = (size_t)u * 16;  // channel-first: one contiguous block
                if constexpr (CL) {
                    // channel-last: unit u is part u % upr of position row u / upr
                    const int r = div_small(u, inv_upr);
                    off = (size_t)r * p.D * EB + (size_t)(u - r * upr) * 16;
                }
                *reinterpret_cast<uint4*>(gd + off) = sd[u];
                *reinterpret_cast<uint4*>(gu + off) = sy[u];
            }
        }
    }
    if (valid) {
        // this folded row's per-channel sums (rows dA[0..N), dD, dbias, dconv_b, dconv_w[0..K))
        float* pc = p.ws + p.pch_off + (size_t)b1 * p.kc * p.D + d;
#pragma unroll
        for (int n = 0; n < NS; ++n)
            if (n < N) pc[(size_t)n * p.D] = gA[n];
        pc[(size_t)N * p.D] = gD;
        pc[(size_t)(N + 1) * p.D] = gb;
        if constexpr (CONV) {
            pc[(size_t)(N + 2) * p.D] = gcb;
#pragma unroll
            for (int jj = 0; jj < KW; ++jj)
                if (jj < p.K) pc[(size_t)(N + 3 + jj) * p.D] = gw[jj];
        }
    }
}

// The float32 sums from the partials, each added in a fixed order.  Blocks
// [0, nb_bc): dB/dC[b, n, t] over the channel tiles (ascending).  Blocks from
// nb_bc on: the per-channel sums over the folded rows, 16 outputs per block,
// each split over 16 threads (thread k adds rows b1 = k, k + 16, ... in order)
// whose results are then added k = 0 .. 15.  Every output element is written.
constexpr int kRedOut = 16;  // per-channel outputs per block (and threads per output)

__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p, int nb_bc) {
    const int ns = p.ns, L = p.L, N = p.N, D = p.D;
    const size_t B = (size_t)p.B1 * p.B2;
    if ((int)blockIdx.x < nb_bc) {
        const size_t nbc = B * L * 2 * ns;  // partial dB/dC values per channel tile
        const float* pbc = p.ws + p.pbc_off;
        for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < nbc;
             idx += (size_t)nb_bc * blockDim.x) {
            const int n = (int)(idx % ns);
            size_t r = idx / ns;
            const int c = (int)(r % 2);
            r /= 2;
            const int t = (int)(r % L);
            const size_t b = r / L;
            if (n >= N) continue;
            float s = 0.0f;
            for (int tl = 0; tl < p.tiles; ++tl) s += pbc[(size_t)tl * nbc + idx];
            (c ? p.dCm : p.dBm)[p.cl ? (b * L + t) * N + n : (b * N + n) * L + t] = s;
        }
        return;
    }
    __shared__ float part[kRedOut][kRedOut + 1];
    const float* pch = p.ws + p.pch_off;
    const int oo = threadIdx.x % kRedOut;
    const int k = threadIdx.x / kRedOut;
    const long long o = (long long)((int)blockIdx.x - nb_bc) * kRedOut + oo;  // output: row * D + d
    const bool live = o < (long long)p.kc * D;
    const int row = live ? (int)(o / D) : 0;
    const int d = live ? (int)(o % D) : 0;
    float s = 0.0f;
    if (live)  // rows: folded row b1 and segment s at b1 * seg + s
        for (int b1 = k; b1 < p.B1 * p.seg; b1 += kRedOut) s += pch[((size_t)b1 * p.kc + row) * D + d];
    part[k][oo] = s;
    __syncthreads();
    if (k == 0 && live) {
        float t = 0.0f;
        for (int m = 0; m < kRedOut; ++m) t += part[m][oo];
        if (row < N) p.dA[(size_t)d * N + row] = t;
        else if (row == N) { if (p.dDskip) p.dDskip[d] = t; }
        else if (row == N + 1) { if (p.ddbias) p.ddbias[d] = t; }
        else if (row == N + 2) { if (p.dconv_b) p.dconv_b[d] = t; }
        else p.dconv_w[(size_t)d * p.K + (row - N - 3)] = t;  // rows past N + 1 exist only with the conv
    }
}

// Split rows with the fused pad: each segment's tokens of the unpadded row
// (padded positions 1 .. L-2 inside the segment) added in float64 in index
// order, per channel, for the row mean.
template <typename IO>
__global__ __launch_bounds__(kWave) void bwd_tokens_kernel(BwdParams p) {
    const int lane = threadIdx.x;
    const int S = p.seg, g = blockIdx.x, s = g % S, rt = g / S;
    const int b = rt / p.tiles, tile = rt - b * p.tiles;
    const int d0 = tile * kWave, nrows = min(kWave, p.D - d0);
    const int L = p.L, XL = p.xrow;
    const int s0 = s * p.cps * p.q, s1 = min(L, s0 + p.cps * p.q);
    const int lo = max(s0, 1) - 1, hi = min(s1, L - 1) - 1;  // tokens [lo, hi)
    double acc = 0.0;
    if (lane < nrows) {
        const IO* x = static_cast<const IO*>(p.u) + ((size_t)b * p.D + d0 + lane) * XL;
        int k = lo;
        for (; k + 8 <= hi; k += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = to_f32(x[k + j]);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += (double)v[j];
        }
        for (; k < hi; ++k) acc += (double)to_f32(x[k]);
    }
    reinterpret_cast<double*>(p.ws + p.meanw_off)[(size_t)g * kWave + lane] = acc;
}

// Split rows: the conv-input gradient at the kw - 1 positions around each
// segment boundary, the trailing partial of the segment before it plus the
// leading partial of the segment after it (in that order).
template <typename IO>
__global__ __launch_bounds__(256) void bwd_seam_kernel(BwdParams p) {
    const int km = p.kw - 1, S = p.seg, D = p.D;
    const size_t total = (size_t)p.B1 * (S - 1) * km * D;
    const float* seam = p.ws + p.seam_off;
    for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
        const int d = (int)(idx % D);
        size_t r = idx / D;
        const int j = (int)(r % km);
        r /= km;
        const int s = 1 + (int)(r % (S - 1));
        const size_t b = r / (S - 1);
        const int tile = d / kWave, lane = d - tile * kWave;
        const size_t g = (b * p.tiles + tile) * S + s;  // the segment after the boundary; g - 1 before it
        const float v = seam[((g - 1) * 2 + 1) * km * kWave + (size_t)j * kWave + lane] +
                        seam[(g * 2) * km * kWave + (size_t)j * kWave + lane];
        const int q = s * p.cps * p.q - p.P + j;
        static_cast<IO*>(p.du)[(b * D + d) * p.L + q] = from_f32<IO>(v);
    }
}

template <typename IO, int NS, int KW, bool CONV, bool SP, bool SILU>
hipError_t launch_bt(const BwdParams& p, hipStream_t s) {
    constexpr int Q = kHist / NS;  // kHist states of history in registers
    if (p.whole && p.cl)
        hipLaunchKernelGGL((bwd_whole_kernel<IO, NS, KW, CONV, SP, SILU, Q, true>), dim3((unsigned)(p.B1 * p.tiles)),
                           dim3(kWave), (size_t)p.lds_bytes, s, p);
    else if (p.whole)
        hipLaunchKernelGGL((bwd_whole_kernel<IO, NS, KW, CONV, SP, SILU, Q, false>), dim3((unsigned)(p.B1 * p.tiles)),
                           dim3(kWave), (size_t)p.lds_bytes, s, p);
    else if (p.fwd) {  // split-row forward: token sums, the carry pass's forward half, the output pass
        const unsigned grid = (unsigned)(p.B1 * p.tiles * p.seg);
        if (p.pad_in) hipLaunchKernelGGL(bwd_tokens_kernel<IO>, dim3(grid), dim3(kWave), 0, s, p);
        hipLaunchKernelGGL((bwd_kernel<IO, NS, KW, CONV, SP, SILU, kFwdQ, 2>), dim3(grid), dim3(kWave),
                           (size_t)p.lds_bytes, s, p);
        hipLaunchKernelGGL((bwd_kernel<IO, NS, KW, CONV, SP, SILU, kFwdQ, 3>), dim3(grid), dim3(kWave),
                           (size_t)p.lds_bytes, s, p);
    } else {
        const unsigned grid = (unsigned)(p.B1 * p.tiles * p.seg);
        if (p.seg > 1) {
            if (p.pad_in) hipLaunchKernelGGL(bwd_tokens_kernel<IO>, dim3(grid), dim3(kWave), 0, s, p);
            hipLaunchKernelGGL((bwd_kernel<IO, NS, KW, CONV, SP, SILU, Q, 2>), dim3(grid), dim3(kWave),
                               (size_t)p.lds_bytes, s, p);
            hipLaunchKernelGGL((bwd_kernel<IO, NS, KW, CONV, SP, SILU, Q, 1>), dim3(grid), dim3(kWave),
                               (size_t)p.lds_bytes, s, p);
        } else {
            hipLaunchKernelGGL((bwd_kernel<IO, NS, KW, CONV, SP, SILU, Q, 0>), dim3(grid), dim3(kWave),
                               (size_t)p.lds_bytes, s, p);
        }
        if (CONV && p.seg > 1 && p.kw > 1) {
            const size_t total = (size_t)p.B1 * (p.seg - 1) * (p.kw - 1) * p.D;
            hipLaunchKernelGGL(bwd_seam_kernel<IO>, dim3((unsigned)std::min<size_t>(1024, (total + 255) / 256)),
                               dim3(256), 0, s, p);
        }
    }
    return hipGetLastError();
}

template <typename IO, int NS, int KW, bool CONV>
hipError_t launch_bsp(const BwdParams& p, hipStream_t s) {
    const bool silu = CONV && p.act == 1;
    if (p.softplus)
        return silu ? launch_bt<IO, NS, KW, CONV, true, CONV>(p, s) : launch_bt<IO, NS, KW, CONV, true, false>(p, s);
    return silu ? launch_bt<IO, NS, KW, CONV, false, CONV>(p, s) : launch_bt<IO, NS, KW, CONV, false, false>(p, s);
}

template <typename IO, int NS>
hipError_t launch_bns(const BwdParams& p, hipStream_t s) {
    if (!p.conv_w) return launch_bsp<IO, NS, 4, false>(p, s);
    if (p.K <= 4) return launch_bsp<IO, NS, 4, true>(p, s);
    return launch_bsp<IO, NS, 8, true>(p, s);
}

template <typename IO>
hipError_t launch_bio(const BwdParams& p, hipStream_t s) {
    if (p.ns == 4) return launch_bns<IO, 4>(p, s);
    if (p.ns == 8) return launch_bns<IO, 8>(p, s);
    return launch_bns<IO, 16>(p, s);
}

}  // namespace

bool plan_bwd(BwdParams& p, int io_bytes, size_t* ws_bytes) {
    p.ns = p.N <= 4 ? 4 : (p.N <= 8 ? 8 : 16);
    p.tiles = (p.D + kWave - 1) / kWave;
    p.q = p.fwd ? kFwdQ : kHist / p.ns;
    p.nchk = (p.L + p.q - 1) / p.q;
    p.kc = p.N + 2 + (p.conv_w ? 1 + p.K : 0);  // rows dA (N), dD, dbias [, dconv_b, dconv_w (K)]
    auto up64 = [](long long v) { return (v + 63) & ~63LL; };  // 256-byte aligned regions
    p.seg = 1;
    p.cps = p.nchk;
    p.kw = p.conv_w ? (p.K <= 4 ? 4 : 8) : 1;
    // workspace regions, each on 256 bytes: checkpoints [B1 * tiles * seg][cps][ns][64],
    // dB/dC partials, per-channel partials [B1 * seg][kc][D]; split rows add the
    // carries [B1 * tiles * seg][2 ns + 2][64], float64 token sums [B1 * tiles * seg][64] and the
    // boundary partials [B1 * tiles * seg][2][kw - 1][64]
    auto layout = [&]() {
        const long long waves = (long long)p.B1 * p.tiles * p.seg;
        const long long ck = p.fwd ? 0 : waves * p.cps * p.ns * kWave;  // (the forward keeps only the carries)
        const long long pbc = p.fwd ? 0 : (long long)p.tiles * p.B1 * p.B2 * p.L * 2 * p.ns;
        const long long pch = p.fwd ? 0 : (long long)p.B1 * p.seg * p.kc * p.D;
        const bool split = p.seg > 1;
        p.pbc_off = up64(ck);
        p.pch_off = p.pbc_off + up64(pbc);
        p.car_off = p.pch_off + up64(pch);
        p.meanw_off = p.car_off + (split ? up64(waves * (2 * p.ns + 2) * kWave) : 0);
        p.seam_off = p.meanw_off + (split ? up64(waves * kWave * 2) : 0);  // one float64 per lane
        *ws_bytes = (size_t)(p.seam_off + (split && !p.fwd ? up64(waves * 2 * (p.kw - 1) * kWave) : 0)) * sizeof(float);
    };
    layout();
    auto up16 = [](long long v) { return (int)((v + 15) & ~15LL); };
    // Whole-sample staging: every [rows][length] block (x, delta, dy, ddelta, du)
    // of every sample and tile must start on 16 bytes and span whole 16-byte
    // units (rows = 64, or D mod 64 for the last tile), and everything must
    // leave room for at least two workgroups per compute unit.
    {
        const long long XL = p.xrow, L = p.L, eb = io_bytes;
        const int last = p.D - (p.tiles - 1) * kWave;
        bool ok = (p.D * XL * eb) % 16 == 0 && (p.D * L * eb) % 16 == 0 && (kWave * XL * eb) % 16 == 0 &&
                  (kWave * L * eb) % 16 == 0 && (last * XL * eb) % 16 == 0 && (last * L * eb) % 16 == 0;
        if (p.cl) ok = (p.D * eb) % 16 == 0;  // position rows of D channels in whole 16-byte units
        int off = 0;
        p.xs_off = off;
        off += up16(kWave * XL * eb);
        p.ds_off = off;
        off += up16(kWave * L * eb);
        p.dys_off = off;
        off += up16(kWave * L * eb);
        p.bc_off = off;
        off += up16(2 * L * p.ns * 4);
        p.red_off = off;  // (the dB/dC sums over channels stay in registers)
        const char* force = getenv("SFM_BWD_CHUNKED");  // diagnostics: force the chunked kernel
        if (!p.fwd && ok && L <= 4096 && off <= 64 * 1024 && (p.cl || !(force && atoi(force) > 0))) {
            p.whole = 1;
            p.mean_off = p.braw_off = p.hin_off = p.stage_bytes = 0;
            p.lds_bytes = off;
            return true;
        }
    }
    p.whole = 0;
    if (p.cl) return false;  // channel-last runs only the whole-sample kernel
    const int q = p.q;
    const int kw = p.conv_w ? (p.K <= 4 ? 4 : 8) : 4;
    const int xw = q + kw - 1;
    // two staging buffers (the next chunk's transfers land while this chunk
    // runs), each: x window, delta (then ddelta), dy, raw B/C, entering state
    int off = 0;
    p.xs_off = off;
    off += up16(kWave * xw * 4);  // staged io elements take 4-byte slots
    // (the split-row forward stages no dy or entering state and needs no
    // transpose or dx window)
    const bool bw = !p.fwd;
    p.ds_off = off;
    off += up16(kWave * q * 4);
    p.dys_off = off;
    off += bw ? up16(kWave * q * 4) : 0;
    p.braw_off = off;  // raw B/C of a chunk: 64-element transfers
    off += ((2 * p.ns * q + kWave - 1) / kWave) * kWave * 4;
    p.hin_off = off;
    off += bw ? p.ns * kWave * 4 : 0;
    p.stage_bytes = off;
    off *= 2;
    p.bc_off = off;
    off += up16(2 * q * p.ns * 4);
    p.red_off = off;
    off += bw ? kWave * kRedStride * 4 : 0;
    p.mean_off = off;  // fp32 dx window
    off += bw ? up16(kWave * xw * 4) : 0;
    p.lds_bytes = off;
    // Split rows along L when the rows and tiles alone give fewer waves than
    // the GPU has SIMDs (about eight waves per SIMD wanted): segments of at least
    // 64 positions (kw at least, also the last one) cost a carry pass over the
    // row and a composition of the carries per wave.  SFM_BWD_SEGMENTS=n asks
    // for n segments (tests; the length floor is then kw).
    {
        const long long waves = (long long)p.B1 * p.tiles;
        const char* fs = getenv("SFM_BWD_SEGMENTS");
        const bool forced = fs && atoi(fs) > 0;
        long long want = forced ? atoi(fs) : (waves < 1024 ? (8192 + waves - 1) / waves : 1);
        if (p.fwd && !forced && waves < 1024) {
            // the forward's segments are cheap: as many as the GPU holds at once, one
            // round of resident waves (several rounds measured slower on the long rows)
            const int per_cu = std::max(1, std::min(8, 160 * 1024 / std::max(1, p.lds_bytes)));
            want = std::max(1LL, (long long)device_cus() * per_cu / waves);
        }
        want = std::min<long long>(want, 64);
        if (want > 1) {
            const int floor_pos = forced ? kw : std::max(kw, 64);
            int cps = std::max((int)((p.nchk + want - 1) / want), (floor_pos + q - 1) / q);
            // the last segment gets kw positions at least
            while (cps < p.nchk && p.L - ((p.nchk + cps - 1) / cps - 1) * cps * q < kw) ++cps;
            const int S = (p.nchk + cps - 1) / cps;
            if (S > 1) {
                p.seg = S;
                p.cps = cps;
            }
        }
    }
    layout();
    return p.lds_bytes <= 64 * 1024;
}

hipError_t launch_fwd_split(const BwdParams& p, int io_dtype, hipStream_t s) {
    return io_dtype == 0 ? launch_bio<float>(p, s) : launch_bio<__bf16>(p, s);
}

hipError_t launch_bwd(const BwdParams& p, int io_dtype, hipStream_t s) {
    hipError_t e = io_dtype == 0 ? launch_bio<float>(p, s) : launch_bio<__bf16>(p, s);
    if (e != hipSuccess) return e;
    const size_t nbc = (size_t)p.B1 * p.B2 * p.L * 2 * p.ns;
    const int nb_bc = (int)std::min<size_t>(2048, (nbc + 255) / 256);
    const size_t nb_ch = ((size_t)p.kc * p.D + kRedOut - 1) / kRedOut;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)(nb_bc + nb_ch)), dim3(256), 0, s, p, nb_bc);
    return hipGetLastError();
}

}  // namespace sfm
