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

#include <algorithm>
#include <atomic>

#include "sfm_device.h"
#include "sfm_internal.h"

namespace sfm {
namespace split_detail {

constexpr int kMaxWpg = 8;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// DPP control that gives every lane the value of lane J of its group of G
// adjacent lanes: quad_perm for groups of 2 and 4, row_newbcast:J (lane J of
// each 16-lane row) for groups of 16.
template <int G, int J>
constexpr int bcast_ctrl() {
    if constexpr (G == 2) return J | (J << 2) | ((2 + J) << 4) | ((2 + J) << 6);
    else if constexpr (G == 4) return J * 0x55;
    else return 0x150 + J;
}

template <int G, int J>
__device__ __forceinline__ float bcast(float v) {
    if constexpr (G == 1) return v;
    else return dpp<bcast_ctrl<G, J>()>(v);
}

// bcast for a float64 value (its two halves by two DPP moves)
template <int G, int J>
__device__ __forceinline__ double bcast_f64(double v) {
    const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)b, bcast_ctrl<G, J>(), 0xf, 0xf, true);
    const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), bcast_ctrl<G, J>(), 0xf, 0xf, true);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Sum over the G adjacent lanes of a group, result in every lane of it
// (quad_perm [1,0,3,2] then [2,3,0,1]; for 16-lane groups then row_half_mirror,
// which pairs the two quads of each half-row, and row_mirror, which pairs the
// two halves).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 16, "lane groups of 1, 2, 4 or 16");
    if constexpr (G >= 2) v += dpp<0xB1>(v);
    if constexpr (G >= 4) v += dpp<0x4E>(v);
    if constexpr (G >= 16) {
        v += dpp<0x141>(v);
        v += dpp<0x140>(v);
    }
    return v;
}

// Reduce-scatter over each 16-lane row: p[j] holds this lane's term of sum j;
// lane i of the row returns the sum over the row's 16 lanes of p[i].  Four
// butterfly steps whose partners differ in lane bits 0-3, 0-2, 0-1 and 0
// (row_mirror, row_half_mirror, quad_perm [3,2,1,0] and [1,0,3,2]); at each
// step a lane keeps the half of its values whose index bit matches its own
// lane bit and sends the other half, so 8 + 4 + 2 + 1 DPP adds cover all 16
// sums (against 4 per sum for an all-reduce).  The masks are lane-constant.
__device__ __forceinline__ float row_reduce_scatter16(const float (&p)[16], int lane) {
    const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
    float q8[8], q4[4], q2[2];
#pragma unroll
    for (int m = 0; m < 8; ++m) q8[m] = (b3 ? p[m + 8] : p[m]) + dpp<0x140>(b3 ? p[m] : p[m + 8]);
#pragma unroll
    for (int m = 0; m < 4; ++m) q4[m] = (b2 ? q8[m + 4] : q8[m]) + dpp<0x141>(b2 ? q8[m] : q8[m + 4]);
#pragma unroll
    for (int m = 0; m < 2; ++m) q2[m] = (b1 ? q4[m + 2] : q4[m]) + dpp<0x1B>(b1 ? q4[m] : q4[m + 2]);
    return (b0 ? q2[1] : q2[0]) + dpp<0xB1>(b0 ? q2[0] : q2[1]);
}

// Reduce-scatter over each quad: p[j] holds this lane's term of sum j; lane
// i of the quad returns the sum over the quad's four lanes of p[i & 3].  Two
// butterfly steps (partners differ in lane bit 0, then bit 1), each keeping the
// values whose index bit matches the lane's bit: 3 DPP adds and 6 selects,
// against 8 DPP adds and 4 selects for four all-reduces.
__device__ __forceinline__ float quad_reduce_scatter(const float (&p)[4], int lane) {
    const bool b1 = lane & 2, b0 = lane & 1;
    float q[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) q[m] = (b0 ? p[2 * m + 1] : p[2 * m]) + dpp<0xB1>(b0 ? p[2 * m] : p[2 * m + 1]);
    return (b1 ? q[1] : q[0]) + dpp<0x4E>(b1 ? q[0] : q[1]);
}

// 4-byte direct global->LDS transfers of a tile: words [0, nw) of rows
// [0, rows) of a region whose rows start rowb bytes apart at g, into LDS rows of
// pw words at l.  LDS word e = 64 k + lane of instruction k holds word e % pw of
// row e / pw; a slot past the valid rows or words re-reads the last valid word
// (in bounds, never read back).  Instructions k0, k0 + kstep, ... of ninst (so
// the waves of a group can share a tile), four per LDS base where four remain.
__device__ __forceinline__ void dma_tile4(const char* g, uint32_t rowb, int rows, int nw, int pw, char* l, int lane,
                                          int ninst, int k0 = 0, int kstep = 1) {
    if (rows <= 0 || nw <= 0) return;
    const float inv = 1.0f / (float)pw;
    const uint32_t maxoff = (uint32_t)(rows - 1) * rowb + (uint32_t)(nw - 1) * 4u;
    auto off_of = [&](int k) __attribute__((always_inline)) {
        const int e = k * kWave + lane;
        const int r = div_small(e, inv);
        const int w = e - r * pw;
        return min((uint32_t)r * rowb + (uint32_t)min(w, nw - 1) * 4u, maxoff);
    };
    int k = k0;
    if (kstep == 1) {
        for (; k + 4 <= ninst; k += 4) {
            char* lk = l + k * 256;
            dma_at<4, 0>(g + off_of(k), lk);
            dma_at<4, 256>(g + off_of(k + 1), lk);
            dma_at<4, 512>(g + off_of(k + 2), lk);
            dma_at<4, 768>(g + off_of(k + 3), lk);
        }
    }
    for (; k < ninst; k += kstep) dma_at<4, 0>(g + off_of(k), l + k * 256);
}

// Float64 sum of r[0 .. n) in index order (bit-identical to a sequential CPU
// sum); the LDS reads go out eight at a time, so the additions wait on one
// read latency per eight elements, not per element.
template <typename IO>
__device__ __forceinline__ double row_sum_f64(const IO* r, int n) {
    double acc = 0.0;
    int i = 0;
    for (; i + 8 <= n; i += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = to_f32(r[i + k]);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += (double)v[k];
    }
    for (; i < n; ++i) acc += (double)to_f32(r[i]);
    return acc;
}

template <typename IO, int NS, int G, int KW, bool CONV, bool SP, bool SILU>
struct SplitWave {
    static constexpr int NPL = NS / G;   // states per lane
    static constexpr int CPW = kWave / G;  // channels per wave
    static constexpr int NB = NPL / 2;   // float4 B/C reads per position ([B..., C...] per lane)
    static_assert(NPL == 1 || NPL % 2 == 0, "one or an even number of states per lane");

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

    // The LDS values of an unchecked block, read one block ahead so that their
    // latency hides behind the previous block's arithmetic (with few waves per
    // SIMD nothing else hides it): the B/C of the G positions, the conv taps
    // the block reads new (the others shift in from the previous block) or the
    // input itself without conv, and delta of this lane's position.
    static constexpr int kKeep = CONV ? (KW > G ? KW - G : 0) : 0;
    struct Ahead {
        float2 bcv[NPL == 1 ? G : 1];       // one state per lane: (B, C) of t0 .. t0 + G - 1
        float4 bq[NPL == 1 ? 1 : G * NB];   // several: [B.., C..] of each position
        IO tap[KW];
        IO dl;
    };

    __device__ __forceinline__ void fetch(int t0, const IO* xr, const IO* dr, const float* bc, Ahead& a) const {
        const int tau = t0 + g;
        const int lo = p.pad_in ? 1 : 0;
        const int P2 = p.P + KW - p.K;
        if constexpr (CONV) {
#pragma unroll
            for (int j = kKeep; j < KW; ++j) a.tap[j] = xr[tau - P2 + j - lo];
        } else {
            a.tap[0] = xr[tau - lo];
        }
        a.dl = dr[tau];
        if constexpr (NPL == 1) {
#pragma unroll
            for (int j = 0; j < G; ++j) a.bcv[j] = *reinterpret_cast<const float2*>(bc + ((t0 + j) * G + g) * 2);
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float4* q4 = reinterpret_cast<const float4*>(bc + ((t0 + j) * G + g) * (2 * NPL));
#pragma unroll
                for (int k = 0; k < NB; ++k) a.bq[j * NB + k] = q4[k];
            }
        }
    }

    // LDS byte addresses of an unchecked block's reads (its first new conv
    // tap, delta, and the lane's B/C of its first position) for the
    // software-pipelined loop, which advances them by a constant per trip.
    // They are held as plain 32-bit LDS addresses and re-pinned every trip
    // (an empty asm), so the compiler keeps one register per stream and
    // addresses the second block of a trip by instruction offsets instead of
    // re-adding the LDS base of the array to a running offset.
    struct Cursor {
        uint32_t x, d, b;
    };
    static constexpr uint32_t kStepX = G * sizeof(IO);             // one block of taps / delta
    static constexpr uint32_t kStepB = G * G * 2 * NPL * 4;        // one block of B/C
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    template <typename T>
    static __device__ __forceinline__ T lds_ld(uint32_t a) {
        return *(const __attribute__((address_space(3))) T*)(size_t)a;
    }
    static __device__ __forceinline__ __attribute__((address_space(3))) IO* lds_yp(uint32_t a) {
        return (__attribute__((address_space(3))) IO*)(size_t)a;
    }
    static __device__ __forceinline__ uint32_t lds_addr(const void* q) {
        return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)q;
    }
    __device__ __forceinline__ Cursor cursor(int t0, const IO* xr, const IO* dr, const float* bc) const {
        const int lo = p.pad_in ? 1 : 0;
        const int P2 = p.P + KW - p.K;
        const int tau = t0 + g;
        Cursor c;
        c.x = CONV ? lds_addr(xr + (tau - P2 + kKeep - lo)) : lds_addr(xr + (tau - lo));
        c.d = lds_addr(dr + tau);
        c.b = lds_addr(bc + (t0 * G + g) * (NPL == 1 ? 2 : 2 * NPL));
        return c;
    }
    static __device__ __forceinline__ void pin(Cursor& c) { asm volatile("" : "+v"(c.x), "+v"(c.d), "+v"(c.b)); }
    // fetch() of the block BLK blocks after the cursor's
    template <int BLK>
    __device__ __forceinline__ void fetch_at(const Cursor& c, Ahead& a) const {
        const uint32_t ox = c.x + BLK * kStepX, od = c.d + BLK * kStepX, ob = c.b + BLK * kStepB;
        if constexpr (CONV) {
#pragma unroll
            for (int j = kKeep; j < KW; ++j) a.tap[j] = lds_ld<IO>(ox + (j - kKeep) * (uint32_t)sizeof(IO));
        } else {
            a.tap[0] = lds_ld<IO>(ox);
        }
        a.dl = lds_ld<IO>(od);
        if constexpr (NPL == 1) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const f32x2 v = lds_ld<f32x2>(ob + j * G * 2 * 4);
                a.bcv[j] = make_float2(v.x, v.y);
            }
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j) {
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const f32x4 v = lds_ld<f32x4>(ob + (j * G * 2 * NPL + 4 * k) * 4);
                    a.bq[j * NB + k] = make_float4(v.x, v.y, v.z, v.w);
                }
            }
        }
    }

    // The unchecked block of positions [t0, t0 + G) from fetched values.
    __device__ __forceinline__ void block_ahead(int t0, IO* dr, const Ahead& a, float (&h)[NPL], float (&win)[KW]) {
        block_ahead_y(dr + t0 + g, a, h, win);
    }
    // block_ahead with y of this lane's position stored at yout
    template <typename YP>
    __device__ __forceinline__ void block_ahead_y(YP yout, const Ahead& a, float (&h)[NPL], float (&win)[KW]) {
        float tn[KW];
        if constexpr (CONV) {
#pragma unroll
            for (int j = kKeep; j < KW; ++j) tn[j] = to_f32(a.tap[j]);
        } else {
            tn[0] = to_f32(a.tap[0]);
        }
        compute<false>(yout, true, tn, to_f32(a.dl), a, h, win);
    }

    // An edge block: the first block of a sample, or one whose new conv taps
    // or positions leave the staged interior.  The taps come through xq (zero
    // outside the sample, the aux value at its ends); delta and B/C of a
    // position >= L are read at L - 1 (in bounds) and its results discarded: y
    // is stored for positions < L only, and the state after the sample's last
    // position is never used.  Then the arithmetic of the pipelined blocks.
    template <bool FIRST>
    __device__ __forceinline__ void block_edge(int t0, const IO* xr, IO* dr, const float* bc, float (&h)[NPL],
                                               float (&win)[KW]) {
        const int L = p.L;
        const int tau = t0 + g;
        const int tc = min(tau, L - 1);
        const int P2 = p.P + KW - p.K;
        float tn[KW];
        if constexpr (CONV) {
#pragma unroll
            for (int j = kKeep; j < KW; ++j) tn[j] = xq(xr, tau - P2 + j);
        } else {
            tn[0] = xq(xr, tc);
        }
        Ahead a;
        if constexpr (NPL == 1) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                a.bcv[j] = *reinterpret_cast<const float2*>(bc + (min(t0 + j, L - 1) * G + g) * 2);
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float4* q4 = reinterpret_cast<const float4*>(bc + (min(t0 + j, L - 1) * G + g) * (2 * NPL));
#pragma unroll
                for (int k = 0; k < NB; ++k) a.bq[j * NB + k] = q4[k];
            }
        }
        compute<FIRST>(dr + tc, tau < L, tn, to_f32(dr[tc]), a, h, win);
    }

    // The arithmetic of a block of G positions [t0, t0 + G): lane g's
    // per-token work for position t0 + g (new conv taps tn[kKeep..KW), or the
    // input itself in tn[0] without conv; raw delta dl0), then the G state
    // updates with the B/C of the positions in a; y of this lane's position
    // goes to yout when store is set.  win holds this lane's conv taps for
    // position t0 + g - G on entry and for t0 + g on exit.  FIRST: the block
    // starts the sample (the state is re-initialised at its first position).
    template <bool FIRST, typename YP>
    __device__ __forceinline__ void compute(YP yout, bool store, const float (&tn)[KW], float dl0, const Ahead& a,
                                            float (&h)[NPL], float (&win)[KW]) {
        float u;
        if constexpr (CONV) {
#pragma unroll
            for (int j = 0; j < kKeep; ++j) win[j] = win[j + G];
#pragma unroll
            for (int j = kKeep; j < KW; ++j) win[j] = tn[j];
            float acc = cb;
#pragma unroll
            for (int j = 0; j < KW; ++j) acc = __builtin_fmaf(cw[j], win[j], acc);
            u = SILU ? silu(acc) : acc;
        } else {
            u = tn[0];
        }
        const float dl = dl0 + dbias;
        float d2, dt;
        if constexpr (SP) {
            d2 = softplus_log2e(dl);
            dt = d2 * kLn2;
        } else {
            dt = dl;
            d2 = dl * kLog2e;
        }
        const float du = dt * u;
        const float dpu = Dk * u;
        if constexpr (NPL == 1) {
            float pj[G];
            static_for<G>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const float d2j = bcast<G, j>(d2);
                const float duj = bcast<G, j>(du);
                const float bx = duj * a.bcv[j].x;
                if (FIRST && j == 0) {
                    h[0] = bx;  // reset: the state is re-initialised at the sample start
                } else {
                    const float e = exp2_fast(d2j * A2[0]);
                    h[0] = __builtin_fmaf(e, h[0], bx);
                }
                pj[j] = a.bcv[j].y * h[0];
            });
            const float yv = row_reduce_scatter16(pj, lane) + dpu;
            if (store) *yout = from_f32<IO>(yv);
        } else {
            float yown = 0.0f;
            float pj[G];  // this lane's C.h term of each position (groups of 4: summed after the block)
            static_for<G>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const float d2j = bcast<G, j>(d2);
                const float duj = bcast<G, j>(du);
                float bv[NPL], cv[NPL];
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const float4 v = a.bq[j * NB + k];
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
                        const float e = exp2_fast(d2j * A2[i]);
                        h[i] = __builtin_fmaf(e, h[i], bx);
                    }
                    yp = i == 0 ? cv[0] * h[0] : __builtin_fmaf(cv[i], h[i], yp);
                }
                if constexpr (G == 4) {
                    pj[j] = yp;
                } else {
                    yp = group_sum<G>(yp);
                    yown = (g == j) ? yp : yown;
                }
            });
            if constexpr (G == 4) yown = quad_reduce_scatter(pj, lane);
            if (store) *yout = from_f32<IO>(yown + dpu);
        }
    }

    // Blocks of a sample that need no checks, [kA, kB): every position < L and
    // every newly read conv tap inside the interior [lo, L-1-lo] of padded
    // positions (the taps kept from the previous block were read there already).
    __device__ __forceinline__ void bounds(int& kA, int& kB, int& nblk) const {
        const int L = p.L;
        const int P2 = p.P + KW - p.K;
        nblk = (L + G - 1) / G;
        const int lo = p.pad_in ? 1 : 0;
        constexpr int keep = CONV ? (KW > G ? KW - G : 0) : 0;
        const int first_new = CONV ? keep - P2 : 0;   // tap offset of the oldest new tap
        const int last_new = CONV ? KW - 1 - P2 : 0;  // tap offset of the newest tap
        // k*G + first_new >= lo  and  k*G + G-1 + last_new <= L-1-lo  and  k*G + G-1 <= L-1
        kA = lo - first_new;
        kA = kA <= 0 ? 1 : max(1, (kA + G - 1) / G);
        const int hiA = min(L - 1 - lo - (G - 1) - last_new, L - G);
        kB = hiA >= 0 ? hiA / G + 1 : 0;
        if (kB > nblk) kB = nblk;
        if (kB < kA) kB = kA;
    }

    // State and conv window at the sample start: taps of the virtual position
    // g - G (the block loop shifts the window by G first).
    __device__ __forceinline__ void start(const IO* xr, float (&h)[NPL], float (&win)[KW]) const {
#pragma unroll
        for (int i = 0; i < NPL; ++i) h[i] = 0.0f;
        const int P2 = p.P + KW - p.K;
#pragma unroll
        for (int j = 0; j < KW; ++j) win[j] = CONV ? xq(xr, g - G - P2 + j) : 0.0f;
    }

    // Blocks [k0, k1) of the sample.  xr, dr and bc are addressed by absolute
    // position (they may point before a staged chunk).
    __device__ __forceinline__ void blocks(int k0, int k1, int kA, int kB, const IO* xr, IO* dr, const float* bc,
                                           float (&h)[NPL], float (&win)[KW]) {
        int k = k0;
        if (k == 0 && k < k1) {
            block_edge<true>(0, xr, dr, bc, h, win);
            k = 1;
        }
        for (; k < kA && k < k1; ++k) block_edge<false>(k * G, xr, dr, bc, h, win);
        const int ke = min(kB, k1);
        if (k < ke) {
            // software-pipelined: block k + 1's LDS reads go out before block k
            // computes.  Every trip of the loop reads two blocks ahead of the
            // previous one at a fixed stride (the next trip's first block always
            // exists), so the compiler keeps one running address per stream;
            // the last one or two blocks are peeled.
            Ahead a0, a1;
            Cursor cur = cursor(k * G, xr, dr, bc);
            pin(cur);
            fetch_at<0>(cur, a0);
            for (; k + 2 < ke; k += 2) {
                fetch_at<1>(cur, a1);
                __builtin_amdgcn_sched_barrier(0);
                block_ahead_y(lds_yp(cur.d), a0, h, win);
                fetch_at<2>(cur, a0);
                __builtin_amdgcn_sched_barrier(0);
                block_ahead_y(lds_yp(cur.d + kStepX), a1, h, win);
                cur.x += 2 * kStepX;
                cur.d += 2 * kStepX;
                cur.b += 2 * kStepB;
                pin(cur);
            }
            if (k + 1 < ke) {
                fetch((k + 1) * G, xr, dr, bc, a1);
                __builtin_amdgcn_sched_barrier(0);
                block_ahead(k * G, dr, a0, h, win);
                __builtin_amdgcn_sched_barrier(0);
                block_ahead((k + 1) * G, dr, a1, h, win);
                k += 2;
            } else {
                block_ahead(k * G, dr, a0, h, win);
                ++k;
            }
        }
        for (; k < k1; ++k) block_edge<false>(k * G, xr, dr, bc, h, win);
    }

    // Whole sample: positions [0, L) from the staged rows; y replaces delta.
    __device__ __forceinline__ void sample(const IO* xr, IO* dr, const float* bc) {
        float h[NPL];
        float win[KW];
        int kA, kB, nblk;
        bounds(kA, kB, nblk);
        start(xr, h, win);
        blocks(0, nblk, kA, kB, xr, dr, bc, h, win);
    }
};

template <typename IO, int NS, int G, int KW, bool CONV, bool SP, bool SILU>
__global__ __launch_bounds__(kWave * kMaxWpg) __attribute__((amdgpu_waves_per_eu(NS <= 8 && KW <= 4 ? 4 : 1))) void split_kernel(ScanParams p) {
    using W = SplitWave<IO, NS, G, KW, CONV, SP, SILU>;
    constexpr int NPL = W::NPL;
    constexpr int CPW = W::CPW;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    if (p.stagger_ticks) {
        // Staggered start: dispatch round r = blockIdx / stagger_period issues
        // its loads r ticks (10 ns) later, so early rounds compute while later
        // rounds load.  Rounds that were not resident at launch start late
        // anyway and take no delay.
        const unsigned long long r = blockIdx.x / p.stagger_period;
        if (r && r < (unsigned long long)p.stagger_rounds) {
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
    char* slab = smem + p.slab_off + (size_t)wave * p.slab_bytes;
    IO* xs = reinterpret_cast<IO*>(slab);
    IO* ds = reinterpret_cast<IO*>(slab + p.xs_bytes);
    const int rows = w.rows;
    const int nthr = p.wpg * kWave;
    const int tid = threadIdx.x;

    // Transfers in the order the set-up needs them: the raw B/C (wave 0) and
    // the x slab, then the delta slab last, so the row means and the B/C
    // widening run while delta is still landing.  nd = the delta slab's
    // transfer instructions (the last ones a wave issues).
    const int nd = rows > 0 ? (rows * L * (int)sizeof(IO) / 16 + kWave - 1) / kWave : 0;
    auto issue = [&](int b) __attribute__((always_inline)) {
        if (wave == 0) {
            const int nbc = N * L * (int)sizeof(IO) / 16;
            dma2_to_lds(static_cast<const IO*>(p.Bm) + (size_t)b * N * L, nbc,
                        static_cast<const IO*>(p.Cm) + (size_t)b * N * L, nbc, braw, lane);
        }
        if (rows > 0) {
            const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * D + dw0) * XL;
            dma_to_lds(xg, xs, rows * XL * (int)sizeof(IO), lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (rows > 0) {
            const IO* dg = static_cast<const IO*>(p.delta) + ((size_t)b * D + dw0) * L;
            dma_to_lds(dg, ds, rows * L * (int)sizeof(IO), lane);
        }
    };

    // the parameters' loads go out first, so that the last nd vector-memory
    // operations of a wave are its delta transfers
    w.load_params();
    __builtin_amdgcn_sched_barrier(0);
    issue(b1 * p.B2);
    // states n >= N: B = C = 0 for the whole launch (widening never writes them)
    // every lane has a row of its own in the slabs (CPW rows are allocated);
    // the rows of channels past D are never loaded nor stored
    const IO* xr = xs + w.c * XL;
    IO* dr = ds + w.c * L;
    // One sample of the folded row.  The first sample runs outside the loop:
    // a loop that issues transfers and uses registers loaded before it makes
    // the compiler wait for every outstanding transfer in its preheader, which
    // would undo the early start of the set-up.
    auto run_sample = [&](int j) __attribute__((always_inline)) {
        const int b = b1 * p.B2 + j;
        // at most the delta transfers outstanding (they complete in issue
        // order): this wave's x slab and wave 0's raw B/C have landed
        wait_vmem_at_most(nd);
        lds_barrier();  // every wave's x slab and the raw B/C are visible to the group
        // Set-up of the sample.  With the fused pad every wave takes the row
        // means of its own channels: lane g of a channel sums piece g of the
        // row (ceil(XL / G) tokens) in float64 in index order, and every lane
        // of the group adds the G piece sums in piece order and rounds once --
        // the index-order sum of the aux pad whenever the float64 partial sums
        // are exact.  Then all waves widen B/C.
        if (p.pad_in) {
            const int qp = (XL + G - 1) / G;
            const int i0 = min(w.g * qp, XL), i1 = min(i0 + qp, XL);
            const double part = row_sum_f64(xr + i0, i1 - i0);
            double s = 0.0;
            static_for<G>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                s += bcast_f64<G, j>(part);
            });
            w.mean = to_f32(Io<IO>::from_f64(s / (double)XL));
        }
        // raw [2][N][L] -> float32 [t][g][B.., C..] (states n >= N get B = C = 0).
        // Four-lane groups (the planner's choice for long rows such as stage-3's):
        // thread t widens position t, whose 2 NS floats are contiguous, by
        // 16-byte stores (stage-3: 56.1 -> 54.9 us).  Two-lane groups spread the
        // elements over every thread: at stage-4's 51 positions the per-position
        // form leaves the work to one wave and its registers push the kernel's
        // count from 110 to 125 (26.3 -> 27.3 us); both forms in one instance
        // spill.
        if constexpr (G == 4) {
            for (int t = tid; t < L; t += nthr) {
                float v[2 * NS];
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    const int o = (n / NPL) * (2 * NPL) + n % NPL;
                    v[o] = n < N ? to_f32(braw[n * L + t]) : 0.0f;
                    v[o + NPL] = n < N ? to_f32(braw[(N + n) * L + t]) : 0.0f;
                }
                float4* q = reinterpret_cast<float4*>(bc + t * (2 * NS));
#pragma unroll
                for (int k = 0; k < NS / 2; ++k) q[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
            }
        } else {
            const float invL = 1.0f / (float)L;
            for (int e = tid; e < NS * L; e += nthr) {
                const int n = div_small(e, invL), t = e - n * L;
                float* q = bc + (t * G + n / NPL) * (2 * NPL) + n % NPL;
                q[0] = n < N ? to_f32(braw[e]) : 0.0f;
                q[NPL] = n < N ? to_f32(braw[N * L + e]) : 0.0f;
            }
        }
        __syncthreads();  // B/C of sample b visible to the group
        wait_vmem();      // this wave's delta slab has landed
        w.sample(xr, dr, bc);
        wave_lds_sync();
        if (rows > 0) {
            if (p.swap_out && L > 1 && w.g == 0 && w.c < rows) {
                const IO a = dr[0];
                dr[0] = dr[L - 1];
                dr[L - 1] = a;
            }
            wave_lds_sync();
            // y leaves by 16-byte stores, two LDS reads in flight per lane
            IO* yg = static_cast<IO*>(p.y) + ((size_t)b * D + dw0) * L;
            const int units = rows * L * (int)sizeof(IO) / 16;
            const uint4* ys = reinterpret_cast<const uint4*>(ds);
            uint4* yo = reinterpret_cast<uint4*>(yg);
            for (int u0 = lane; u0 < units; u0 += 2 * kWave) {
                const uint4 v0 = ys[u0];
                const bool two = u0 + kWave < units;
                uint4 v1;
                if (two) v1 = ys[u0 + kWave];
                yo[u0] = v0;
                if (two) yo[u0 + kWave] = v1;
            }
        }
        if (j + 1 < p.B2) {
            // this wave's LDS reads of y have completed before transfers rewrite the slab
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue(b + 1);
        }
    };
    run_sample(0);
    for (int j = 1; j < p.B2; ++j) run_sample(j);
    (void)NPL;
}

// Chunked variant for rows too long to stage delta whole: the conv input x
// stays whole rows in LDS (it feeds the conv windows and the fused pad's row
// mean), while delta/y and the raw B/C move sq positions at a time by 4-byte
// transfers into odd-pitch LDS rows (conflict-free column reads), so about
// five workgroups of four waves fit a CU at stage-3 row lengths.  Per chunk:
// wait, workgroup barrier, B/C widened by all waves, barrier, the blocks of the
// chunk (y over delta in the tile), y stored by 4-byte stores (with the fused
// swap, the end tokens leave one by one), then the next chunk's transfers; the
// next chunk's raw B/C go out as soon as the current one is widened.
template <typename IO, int NS, int G, int KW, bool CONV, bool SP, bool SILU>
__global__ __launch_bounds__(kWave * kMaxWpg) void split_chunk_kernel(ScanParams p) {
    using W = SplitWave<IO, NS, G, KW, CONV, SP, SILU>;
    constexpr int NPL = W::NPL;
    constexpr int CPW = W::CPW;
    constexpr int ew = 4 / (int)sizeof(IO);  // elements per 4-byte word
    extern __shared__ __attribute__((aligned(16))) char smem[];
    if (p.stagger_ticks) {
        const unsigned long long r = blockIdx.x / p.stagger_period;
        if (r && r < (unsigned long long)p.stagger_rounds) {
            const unsigned long long until = __builtin_amdgcn_s_memrealtime() + r * p.stagger_ticks;
            while (__builtin_amdgcn_s_memrealtime() < until) __builtin_amdgcn_s_sleep(2);
        }
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int NGRP = p.stiles * p.B1;
    int gi = blockIdx.x;
    if ((NGRP & 7) == 0) gi = (gi & 7) * (NGRP >> 3) + (gi >> 3);
    const int b1 = gi / p.stiles;
    const int tile = gi - b1 * p.stiles;
    const int dw0 = (tile * p.wpg + wave) * CPW;
    W w(p, lane, dw0);
    const int L = p.L, XL = p.xrow, N = p.N, D = p.D, Q = p.sq;
    const uint32_t rowb = (uint32_t)L * sizeof(IO);
    float* bc = reinterpret_cast<float*>(smem + p.bc_off);        // [Q][G][B.., C..] float32
    char* btile = smem + p.braw_off;                              // raw B rows [N][bpw words]
    char* ctile = btile + p.btile_insts * 256;                    // raw C rows
    char* slab = smem + p.slab_off + (size_t)wave * p.slab_bytes;
    IO* xs = reinterpret_cast<IO*>(slab);                         // [CPW][XL] whole rows
    char* dtile = slab + p.xs_bytes;                              // [CPW][dpw words]
    const int rows = w.rows;
    const int tid = threadIdx.x;

    auto issue_bc = [&](int b, int t0, int len) __attribute__((always_inline)) {
        const int nw = (len + ew - 1) / ew;
        const char* bg = reinterpret_cast<const char*>(static_cast<const IO*>(p.Bm) + ((size_t)b * N) * L + t0);
        const char* cg = reinterpret_cast<const char*>(static_cast<const IO*>(p.Cm) + ((size_t)b * N) * L + t0);
        dma_tile4(bg, rowb, N, nw, p.bpw, btile, lane, p.btile_insts, wave, p.wpg);
        dma_tile4(cg, rowb, N, nw, p.bpw, ctile, lane, p.btile_insts, p.wpg - 1 - wave, p.wpg);
    };
    auto issue_d = [&](int b, int t0, int len) __attribute__((always_inline)) {
        const int nw = (len + ew - 1) / ew;
        const char* dg = reinterpret_cast<const char*>(static_cast<const IO*>(p.delta) + ((size_t)b * D + dw0) * L + t0);
        dma_tile4(dg, rowb, rows, nw, p.dpw, dtile, lane, p.dtile_insts);
    };
    // raw B/C tiles -> float32 [q][g][B.., C..]: work item (q, g) widens the
    // NPL states of lane-group member g at chunk position q, 2 NPL contiguous
    // floats stored by 16-byte writes (states n >= N get B = C = 0)
    auto widen = [&](int len, int first_wave) __attribute__((always_inline)) {
        const int wthr = (p.wpg - first_wave) * kWave;
        const IO* bt = reinterpret_cast<const IO*>(btile);
        const IO* ct = reinterpret_cast<const IO*>(ctile);
        for (int e = tid - first_wave * kWave; e < len * G; e += wthr) {
            const int q = e / G, gg = e - q * G;
            float v[2 * NPL];
#pragma unroll
            for (int i = 0; i < NPL; ++i) {
                const int n = gg * NPL + i;
                v[i] = n < N ? to_f32(bt[n * p.bpw * ew + q]) : 0.0f;
                v[NPL + i] = n < N ? to_f32(ct[n * p.bpw * ew + q]) : 0.0f;
            }
            float4* o = reinterpret_cast<float4*>(bc + e * (2 * NPL));
#pragma unroll
            for (int k = 0; k < NPL / 2; ++k) o[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
        }
    };

    w.load_params();
    const IO* xr = xs + w.c * XL;
    IO* drow = reinterpret_cast<IO*>(dtile) + w.c * p.dpw * ew;  // this lane's delta/y tile row
    const int nch = (L + Q - 1) / Q;
    int kA, kB, nblk;
    w.bounds(kA, kB, nblk);
    for (int j = 0; j < p.B2; ++j) {
        const int b = b1 * p.B2 + j;
        const int len0 = min(Q, L);
        if (rows > 0) {
            const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * D + dw0) * XL;
            dma_to_lds(xg, xs, rows * XL * (int)sizeof(IO), lane);
        }
        issue_bc(b, 0, len0);
        if (rows > 0) issue_d(b, 0, len0);
        IO* yg = static_cast<IO*>(p.y) + ((size_t)b * D + dw0) * L;
        float h[NPL];
        float win[KW];
        IO y0 = Io<IO>::zero();  // fused swap: y at t = 0 of this lane's row, written last
        for (int c = 0; c < nch; ++c) {
            const int t0 = c * Q, len = min(Q, L - t0);
            wait_vmem();
            __syncthreads();  // this chunk's delta and raw B/C (and at c = 0 the x rows) have landed
            if (c == 0 && p.pad_in) {
                // the row means of this wave's channels, as the whole-row kernel
                // takes them: lane g of a channel sums piece g of the row in
                // float64 in index order, the G piece sums are added in piece
                // order and rounded once (it replaced one lane per channel summing
                // whole rows on the first waves while the others widened: base
                // stage-3 275.3 -> 274.3 us)
                const int qp = (XL + G - 1) / G;
                const int i0 = min(w.g * qp, XL), i1 = min(i0 + qp, XL);
                const double part = row_sum_f64(xr + i0, i1 - i0);
                double s2 = 0.0;
                static_for<G>([&](auto jc) {
                    constexpr int jj = decltype(jc)::value;
                    s2 += bcast_f64<G, jj>(part);
                });
                w.mean = to_f32(Io<IO>::from_f64(s2 / (double)XL));
            }
            widen(len, 0);
            __syncthreads();  // B/C of the chunk visible to the group
            if (c + 1 < nch) issue_bc(b, t0 + Q, min(Q, L - t0 - Q));  // the raw B/C tiles are free again
            if (c == 0) w.start(xr, h, win);
            const int k0 = t0 / G;
            const int k1 = c + 1 == nch ? nblk : (t0 + len) / G;
            w.blocks(k0, k1, kA, kB, xr, drow - t0, bc - t0 * G * (2 * NPL), h, win);
            wave_lds_sync();
            if (rows > 0) {
                // y of positions [t0, t0 + len) from the tile, 4-byte words; with the
                // fused swap the words holding positions 0 and L-1 leave element-wise
                const bool sw = p.swap_out && L > 1;
                const int nw = (len + ew - 1) / ew;
                const int wlo = (sw && t0 == 0) ? 1 : 0;
                const int whi = (sw && t0 + len == L) ? nw - 1 : nw;
                const float inv = 1.0f / (float)p.dpw;
                const uint32_t* tw = reinterpret_cast<const uint32_t*>(dtile);
                for (int k = 0; k < p.dtile_insts; ++k) {
                    const int e = k * kWave + lane;
                    const int r = div_small(e, inv), wd = e - r * p.dpw;
                    if (r < rows && wd >= wlo && wd < whi)
                        reinterpret_cast<uint32_t*>(yg + (size_t)r * L + t0)[wd] = tw[e];
                }
                if (sw && w.g == 0 && w.c < rows) {
                    IO* yr = yg + (size_t)w.c * L;
                    if (t0 == 0) {
                        y0 = drow[0];
                        for (int q = 1; q < min(ew, len); ++q) yr[q] = drow[q];
                    }
                    if (t0 + len == L) {
                        const int lw = (nw - 1) * ew;  // first position of the last word, relative to t0
                        for (int q = lw; q < len - 1; ++q) yr[t0 + q] = drow[q];
                        yr[0] = drow[L - 1 - t0];
                        yr[L - 1] = y0;
                    }
                }
            }
            if (c + 1 < nch) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile's reads are done
                if (rows > 0) issue_d(b, t0 + Q, min(Q, L - t0 - Q));
            }
        }
        if (j + 1 < p.B2) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();  // every wave is done with this sample's x rows and B/C
        }
    }
    (void)NPL;
}

// Streaming variant for long rows (one state per lane, G = NS = 16): nothing
// is staged whole.  The wave's x rows (with the conv halo), its delta/y rows
// and the sample's raw B/C rows move sq positions at a time by 4-byte
// transfers into odd-pitch LDS tiles, in two stages: chunk i + 1's transfers
// go out as soon as chunk i has landed and been widened, so they fly while
// chunk i computes, and chunk i's y leaves from its tile at the start of chunk
// i + 1 (after that chunk's wait, so no wait ever covers a fresh store).  The
// chunks of the B2 samples of a folded row form one stream.  The interior
// chunks of a sample all have the same tile shapes, so their per-lane transfer
// and store offsets are computed once; the first and last chunk of a sample
// (clamped halo, ragged end, swapped ends) take the general path.  With the
// fused pad the row mean is taken first, straight from HBM: the 16 lanes of a
// channel each add a contiguous piece of the row in float64, in index order,
// and the 16 piece sums are added in piece order (the index-order sum whenever
// the float64 sums are exact, as they are for bf16 rows whose magnitudes span
// less than 2^33).
constexpr int kFastInsts = 8;  // transfers (or y stores) per tile on the precomputed path

template <typename IO, int NS, int G, int KW, bool CONV, bool SP, bool SILU>
__global__ __launch_bounds__(kWave * kMaxWpg) void split_stream_kernel(ScanParams p) {
    using W = SplitWave<IO, NS, G, KW, CONV, SP, SILU>;
    constexpr int NPL = W::NPL;
    constexpr int CPW = W::CPW;
    constexpr int ew = 4 / (int)sizeof(IO);  // elements per 4-byte word
    static_assert(NPL == 1 && G == 16, "one state per lane, 16 lanes per channel");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int NGRP = p.stiles * p.B1;
    int gi = blockIdx.x;
    if ((NGRP & 7) == 0) gi = (gi & 7) * (NGRP >> 3) + (gi >> 3);
    const int b1 = gi / p.stiles;
    const int tile = gi - b1 * p.stiles;
    const int dw0 = (tile * p.wpg + wave) * CPW;
    W w(p, lane, dw0);
    const int L = p.L, XL = p.xrow, N = p.N, D = p.D, Q = p.sq;
    const int lo = p.pad_in ? 1 : 0;
    const int P2 = p.P + KW - p.K;  // pad_left of the KW-tap window
    const uint32_t rowb = (uint32_t)L * sizeof(IO), xrowb = (uint32_t)XL * sizeof(IO);
    float* bc = reinterpret_cast<float*>(smem + p.bc_off);  // [Q][G][B, C] float32
    char* braw = smem + p.braw_off;                          // 2 stages x (B tile, C tile)
    const int btb = p.btile_insts * 256;
    double* part = reinterpret_cast<double*>(smem + p.mean_off) + wave * kWave;  // float64 piece sums
    char* slab = smem + p.slab_off + (size_t)wave * p.slab_bytes;                // 2 stages x (x tile, delta tile)
    const int xtb = p.xtile_insts * 256, dtb = p.dtile_insts * 256;
    const int rows = w.rows;
    const int nthr = p.wpg * kWave;
    const int tid = threadIdx.x;
    const int nch = (L + Q - 1) / Q;
    const int total = p.B2 * nch;
    // the B/C transfers of a chunk, split into contiguous per-wave ranges
    const int bper = (p.btile_insts + p.wpg - 1) / p.wpg;
    const int bk0 = min(p.btile_insts, wave * bper), bk1 = min(p.btile_insts, bk0 + bper);

    // first 4-byte word of x staged for the chunk at t0 (its oldest conv tap)
    auto xw0 = [&](int t0) __attribute__((always_inline)) { return max(0, t0 - P2 - lo) / ew; };
    auto xnw_of = [&](int t0) __attribute__((always_inline)) {
        const int iend = min(XL, t0 + Q - P2 + KW - 1 - lo);  // one past the newest tap (unpadded)
        return (iend + ew - 1) / ew - xw0(t0);
    };
    // Interior chunks (0 < c < nch - 1 whose conv taps do not reach the row
    // end): the same tile shapes every time.
    const bool fast = nch > 2 && p.xtile_insts <= kFastInsts && p.dtile_insts <= kFastInsts && bper <= kFastInsts;
    auto interior = [&](int c) __attribute__((always_inline)) {
        return fast && c > 0 && c + 1 < nch && c * Q + Q - P2 + KW - 1 - lo <= XL;
    };
    uint32_t xo[kFastInsts], dof[kFastInsts], bo[kFastInsts], yo[kFastInsts];
    if (fast) {
        const int xnw = xnw_of(Q), dnw = Q / ew;
        const float ix = 1.0f / (float)p.xpw, id = 1.0f / (float)p.dpw;
        const uint32_t xmax = (uint32_t)(max(rows, 1) - 1) * xrowb + (uint32_t)(xnw - 1) * 4u;
        const uint32_t dmax = (uint32_t)(max(rows, 1) - 1) * rowb + (uint32_t)(dnw - 1) * 4u;
        const uint32_t bmax = (uint32_t)(N - 1) * rowb + (uint32_t)(dnw - 1) * 4u;
#pragma unroll
        for (int k = 0; k < kFastInsts; ++k) {
            const int e = k * kWave + lane;
            int r = div_small(e, ix), wd = e - r * p.xpw;
            xo[k] = min((uint32_t)r * xrowb + (uint32_t)min(wd, xnw - 1) * 4u, xmax);
            r = div_small(e, id);
            wd = e - r * p.dpw;
            dof[k] = min((uint32_t)r * rowb + (uint32_t)min(wd, dnw - 1) * 4u, dmax);
            // y: word wd of tile row r goes to row r of y (0xffffffff: a slot past the rows or the chunk)
            yo[k] = (r < rows && wd < dnw) ? (uint32_t)r * rowb + (uint32_t)wd * 4u : 0xffffffffu;
            const int eb = (bk0 + k) * kWave + lane;
            const int rb = div_small(eb, id), wb = eb - rb * p.dpw;
            bo[k] = min((uint32_t)rb * rowb + (uint32_t)min(wb, dnw - 1) * 4u, bmax);
        }
    }

    auto issue = [&](int idx) __attribute__((always_inline)) {
        const int j = idx / nch, c = idx - j * nch;
        const int b = b1 * p.B2 + j;
        const int t0 = c * Q, len = min(Q, L - t0);
        char* st = slab + (idx & 1) * (xtb + dtb);
        char* bt = braw + (idx & 1) * 2 * btb;
        const char* xg = reinterpret_cast<const char*>(static_cast<const IO*>(p.u) + ((size_t)b * D + dw0) * XL) +
                         (size_t)xw0(t0) * 4;
        const char* dg = reinterpret_cast<const char*>(static_cast<const IO*>(p.delta) + ((size_t)b * D + dw0) * L + t0);
        const char* bg = reinterpret_cast<const char*>(static_cast<const IO*>(p.Bm) + ((size_t)b * N) * L + t0);
        const char* cg = reinterpret_cast<const char*>(static_cast<const IO*>(p.Cm) + ((size_t)b * N) * L + t0);
        if (interior(c)) {
            // one LDS base per tile, the instruction offsets as immediates
            static_for<kFastInsts>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if (rows > 0 && k < p.xtile_insts) dma_at<4, 256 * k>(xg + xo[k], st);
            });
            static_for<kFastInsts>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if (rows > 0 && k < p.dtile_insts) dma_at<4, 256 * k>(dg + dof[k], st + xtb);
            });
            char* bl = bt + bk0 * 256;
            static_for<kFastInsts>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if (k < bk1 - bk0) dma_at<4, 256 * k>(bg + bo[k], bl);
            });
            static_for<kFastInsts>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if (k < bk1 - bk0) dma_at<4, 256 * k>(cg + bo[k], bl + btb);
            });
            return;
        }
        if (rows > 0) {
            dma_tile4(xg, xrowb, rows, xnw_of(t0), p.xpw, st, lane, p.xtile_insts);
            dma_tile4(dg, rowb, rows, (len + ew - 1) / ew, p.dpw, st + xtb, lane, p.dtile_insts);
        }
        const int nw = (len + ew - 1) / ew;
        dma_tile4(bg, rowb, N, nw, p.bpw, bt, lane, p.btile_insts, wave, p.wpg);
        dma_tile4(cg, rowb, N, nw, p.bpw, bt + btb, lane, p.btile_insts, p.wpg - 1 - wave, p.wpg);
    };
    IO y0 = Io<IO>::zero();  // fused swap: y at t = 0 of this lane's row, written with the sample's last chunk
    auto store_y = [&](int idx) __attribute__((always_inline)) {
        if (rows <= 0) return;
        const int j = idx / nch, c = idx - j * nch;
        const int b = b1 * p.B2 + j;
        const int t0 = c * Q, len = min(Q, L - t0);
        const char* dtile = slab + (idx & 1) * (xtb + dtb) + xtb;
        IO* yg = static_cast<IO*>(p.y) + ((size_t)b * D + dw0) * L;
        const uint32_t* tw = reinterpret_cast<const uint32_t*>(dtile);
        if (interior(c)) {
            char* yc = reinterpret_cast<char*>(yg + t0);
            static_for<kFastInsts>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if (k < p.dtile_insts && yo[k] != 0xffffffffu)
                    *reinterpret_cast<uint32_t*>(yc + yo[k]) = tw[k * kWave + lane];
            });
            return;
        }
        const bool sw = p.swap_out && L > 1;
        const int nw = (len + ew - 1) / ew;
        const int wlo = (sw && t0 == 0) ? 1 : 0;
        const int whi = (sw && t0 + len == L) ? nw - 1 : nw;
        const float inv = 1.0f / (float)p.dpw;
        for (int k = 0; k < p.dtile_insts; ++k) {
            const int e = k * kWave + lane;
            const int r = div_small(e, inv), wd = e - r * p.dpw;
            if (r < rows && wd >= wlo && wd < whi) reinterpret_cast<uint32_t*>(yg + (size_t)r * L + t0)[wd] = tw[e];
        }
        if (sw && w.g == 0 && w.c < rows) {
            const IO* drow = reinterpret_cast<const IO*>(dtile) + w.c * p.dpw * ew;
            IO* yr = yg + (size_t)w.c * L;
            if (t0 == 0) {
                y0 = drow[0];
                for (int q = 1; q < min(ew, len); ++q) yr[q] = drow[q];
            }
            if (t0 + len == L) {
                const int lw = (nw - 1) * ew;  // first position of the last word, relative to t0
                for (int q = max(lw, t0 == 0 ? ew : 0); q < len - 1; ++q) yr[t0 + q] = drow[q];
                yr[0] = drow[L - 1 - t0];
                yr[L - 1] = y0;
            }
        }
    };
    // raw B/C words -> float32 [q][n][B, C]; thread -> (state n, word) without divisions
    auto widen = [&](int idx, int len) __attribute__((always_inline)) {
        const char* bt = braw + (idx & 1) * 2 * btb;
        const uint32_t* bb = reinterpret_cast<const uint32_t*>(bt);
        const uint32_t* cc = reinterpret_cast<const uint32_t*>(bt + btb);
        const int nwd = (len + ew - 1) / ew;
        const int n = tid & (G - 1);
        if (n < N) {
            for (int wd = tid / G; wd < nwd; wd += nthr / G) {
                const uint32_t vb = bb[n * p.bpw + wd], vc = cc[n * p.bpw + wd];
                if constexpr (ew == 2) {
                    const int q = 2 * wd;
                    *reinterpret_cast<float2*>(bc + (q * G + n) * 2) =
                        float2{__builtin_bit_cast(float, vb << 16), __builtin_bit_cast(float, vc << 16)};
                    *reinterpret_cast<float2*>(bc + ((q + 1) * G + n) * 2) =
                        float2{__builtin_bit_cast(float, vb & 0xffff0000u), __builtin_bit_cast(float, vc & 0xffff0000u)};
                } else {
                    *reinterpret_cast<float2*>(bc + (wd * G + n) * 2) =
                        float2{__builtin_bit_cast(float, vb), __builtin_bit_cast(float, vc)};
                }
            }
        }
    };
    // Row mean of sample b for this lane's channel (fused pad), see above.
    auto row_mean = [&](int b) __attribute__((always_inline)) {
        double acc = 0.0;
        if (w.c < rows) {
            const int piece = ((XL + G - 1) / G + 7) & ~7;
            const int i0 = min(XL, w.g * piece), i1 = min(XL, i0 + piece);
            const IO* r = static_cast<const IO*>(p.u) + ((size_t)b * D + w.d) * XL;
            int i = i0;
            // rows of whole 16-byte units: sixteen units in flight per batch
            // (a piece starts on a unit: its length is a multiple of 8 elements)
            constexpr int EU = 16 / (int)sizeof(IO);
            if (((size_t)XL * sizeof(IO)) % 16 == 0) {
                for (; i + 16 * EU <= i1; i += 16 * EU) {
                    uint4 v[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k) v[k] = reinterpret_cast<const uint4*>(r + i)[k];
                    const IO* e = reinterpret_cast<const IO*>(v);
#pragma unroll
                    for (int k = 0; k < 16 * EU; ++k) acc += (double)to_f32(e[k]);
                }
                for (; i + EU <= i1; i += EU) {
                    const uint4 v = *reinterpret_cast<const uint4*>(r + i);
                    const IO* e = reinterpret_cast<const IO*>(&v);
#pragma unroll
                    for (int k = 0; k < EU; ++k) acc += (double)to_f32(e[k]);
                }
            }
            for (; i < i1; ++i) acc += (double)to_f32(r[i]);
        }
        part[lane] = acc;
        wave_lds_sync();
        double s = 0.0;
#pragma unroll
        for (int k = 0; k < G; ++k) s += part[w.c * G + k];
        wave_lds_sync();  // the piece sums are read before the next sample's overwrite them
        return w.c < rows ? to_f32(Io<IO>::from_f64(s / (double)XL)) : 0.0f;
    };

    issue(0);
    w.load_params();
    // states n >= N: B = C = 0 for the whole launch (widening never writes them)
    if (N < NS) {
        for (int e = tid; e < Q * NS; e += nthr) {
            const int q = e / NS, n = e - q * NS;
            if (n >= N) *reinterpret_cast<float2*>(bc + (q * G + n) * 2) = float2{0.0f, 0.0f};
        }
    }
    int kA, kB, nblk;
    w.bounds(kA, kB, nblk);
    float h[NPL];
    float win[KW];
    for (int idx = 0; idx < total; ++idx) {
        const int j = idx / nch, c = idx - j * nch;
        const int t0 = c * Q, len = min(Q, L - t0);
        if (c == 0 && p.pad_in) w.mean = row_mean(b1 * p.B2 + j);
        wait_vmem();
        __syncthreads();  // chunk idx has landed for every wave; chunk idx - 1 is done in every wave
        if (idx > 0) store_y(idx - 1);
        widen(idx, len);
        __syncthreads();  // B/C of the chunk visible to the group; its raw tiles free again
        if (idx + 1 < total) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's reads of the other stage are done
            issue(idx + 1);
        }
        const char* st = slab + (idx & 1) * (xtb + dtb);
        const IO* xr = reinterpret_cast<const IO*>(st) + w.c * p.xpw * ew - xw0(t0) * ew;
        IO* dr = reinterpret_cast<IO*>(const_cast<char*>(st) + xtb) + w.c * p.dpw * ew - t0;
        if (c == 0) w.start(xr, h, win);
        const int k0 = t0 / G;
        const int k1 = c + 1 == nch ? nblk : (t0 + len) / G;
        w.blocks(k0, k1, kA, kB, xr, dr, bc - t0 * G * 2, h, win);
    }
    wave_lds_sync();
    store_y(total - 1);
    (void)NPL;
}

template <typename IO, int NS, int G, int KW, bool CONV, bool SP, bool SILU>
hipError_t launch_t(const ScanParams& p, hipStream_t stream) {
    void (*kern)(ScanParams);
    if constexpr (G == NS) kern = split_stream_kernel<IO, NS, G, KW, CONV, SP, SILU>;
    else kern = p.sq > 0 ? split_chunk_kernel<IO, NS, G, KW, CONV, SP, SILU> : split_kernel<IO, NS, G, KW, CONV, SP, SILU>;
    static bool attr_set[2] = {false, false};
    if (!attr_set[p.sq > 0] && p.lds_bytes > 64 * 1024) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024) != hipSuccess)
            (void)hipGetLastError();
        attr_set[p.sq > 0] = true;
    }
    const unsigned grid = (unsigned)(p.stiles * p.B1);
    const unsigned block = (unsigned)(kWave * p.wpg);
    if (!p.stagger_ticks) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(block), (size_t)p.lds_bytes, stream, p);
        return hipGetLastError();
    }
    // The staggered start delays only the dispatch rounds resident at launch:
    // as many as workgroups of this kernel fit one CU (registers and LDS),
    // asked of the runtime once per (LDS size, block size) and kept.
    static std::atomic<unsigned long long> occ_cache{0};
    const unsigned long long key =
        ((unsigned long long)(unsigned)p.lds_bytes << 17) | ((unsigned long long)(p.sq > 0) << 16) | block;
    unsigned long long c = occ_cache.load(std::memory_order_relaxed);
    int occ;
    if (c && (c >> 8) == key) {
        occ = (int)(c & 0xff);
    } else {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(kern), (int)block,
                                                         (size_t)p.lds_bytes) != hipSuccess || nb <= 0) {
            (void)hipGetLastError();
            nb = 255;  // unknown: every round delays
        }
        occ = std::min(nb, 255);
        occ_cache.store((key << 8) | (unsigned long long)occ, std::memory_order_relaxed);
    }
    ScanParams q = p;
    q.stagger_rounds = occ;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), (size_t)q.lds_bytes, stream, q);
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
// for lane groups of 2 and 4; SFM_SPLIT_INSTANCE3 adds a third group size
// (16, the streaming kernel, with 16 states).
#define SFM_SPLIT_INSTANCE(IOT, NAME, NSV, GA, GB)                                             \
    namespace sfm {                                                                           \
    hipError_t launch_split_##NAME##_n##NSV(const ScanParams& p, hipStream_t s) {             \
        if (p.split == GA) return split_detail::launch_g<IOT, NSV, GA>(p, s);                 \
        if (p.split == GB) return split_detail::launch_g<IOT, NSV, GB>(p, s);                 \
        return hipErrorInvalidValue;                                                          \
    }                                                                                         \
    }
#define SFM_SPLIT_INSTANCE3(IOT, NAME, NSV, GA, GB, GC)                                        \
    namespace sfm {                                                                           \
    hipError_t launch_split_##NAME##_n##NSV(const ScanParams& p, hipStream_t s) {             \
        if (p.split == GA) return split_detail::launch_g<IOT, NSV, GA>(p, s);                 \
        if (p.split == GB) return split_detail::launch_g<IOT, NSV, GB>(p, s);                 \
        if (p.split == GC) return split_detail::launch_g<IOT, NSV, GC>(p, s);                 \
        return hipErrorInvalidValue;                                                          \
    }                                                                                         \
    }
