// scan_kernel.h -- the selective-scan kernel template (included by the
// per-type instantiation units scan_<io>_n<N>.hip and by scan.hip).
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
//    once per wave in LDS as float32, read back as 16-byte broadcasts.
//  * The folded row (B2*L positions) is cut into `waves` contiguous pieces, one
//    per wave.  Each lane scans its piece sequentially with the N-state float32
//    recurrence in registers -- no cross-lane scan is needed, because the
//    channel dimension already fills the wave; this removes the short-sequence
//    under-fill the pages attribute to per-sequence warp scans.
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
//  * Staging (per chunk of positions, through LDS):
//      mode 0 -- whole sample rows: the [64 x L] conv-input and delta slabs are
//                contiguous, so they go straight into LDS by 16-byte direct
//                global->LDS transfers, all in flight at once;
//      mode 1 -- tiles of even-length rows: 4-byte direct transfers into LDS
//                rows padded to an odd number of words (no bank conflicts when
//                the 64 lanes read one column), in groups of four or sixteen
//                transfers with no lane masks; with two stages per wave the
//                transfers of chunk k+1 (x, delta and the raw B/C rows) are in
//                flight while chunk k computes, and y of chunk k is stored
//                after chunk k+1 has landed, so no wait covers a store;
//      mode 2 -- element loads (any shape), 16 per lane in flight.
//    B and C become float32 [t][n] in LDS; y overwrites delta in LDS and is
//    stored with wide coalesced stores.
//  * The position loop is software-pipelined: the LDS reads of position t+1
//    are issued before position t computes, so the wave does not wait on LDS
//    latency each step, and at most two positions' inputs are live.
//  * The optional depthwise conv is fused: a register window slides over the
//    staged conv input and taps outside the sample read zero (the boundary
//    masking of the techloop walkthrough's conv-boundary part).
#pragma once

#include "sfm_device.h"
#include "sfm_internal.h"

namespace sfm {
namespace scan_detail {

constexpr int kMaxWaves = 8;

template <typename IO, int NS, int KW, bool CONV, bool SP, bool SILU, int MODE>
struct ScanWave {
    const ScanParams& p;
    const int lane;
    const int d0;
    const int nrows;  // valid channel rows of this tile (<= 64)
    const int b1;
    // per-lane parameters
    float A[NS];
    float Dk, dbias, cw[KW], cb;
    // LDS stages
    IO* xs;
    IO* ds;
    float* bs;
    float* cs;
    IO* braw;  // mode 0 with bc_dma: raw B then C of one sample, [N][L] each
    // mode 1: the two stages of this wave (x tile, delta/y tile, raw B/C rows,
    // stage i at own1 + i * sb1) and the x / delta offsets each was filled with
    // (scalars, not arrays: a run-time index would put an array in scratch)
    char* own1;
    int sb1;
    int xo0, xo1, do0, do1;
    __device__ __forceinline__ IO* xs_of(int i) const { return reinterpret_cast<IO*>(own1 + i * sb1); }
    __device__ __forceinline__ IO* ds_of(int i) const { return reinterpret_cast<IO*>(own1 + i * sb1 + p.xs_bytes); }
    __device__ __forceinline__ IO* rb_of(int i) const {
        return reinterpret_cast<IO*>(own1 + i * sb1 + p.xs_bytes + p.ds_bytes);
    }
    // geometry of the staged chunk: value at position q of this lane's row is
    // xs[lane*xrs + q - xoff], ds[lane*drs + q - doff]; B/C at bs[(q-boff)*NS + n]
    int xrs, xoff, drs, doff, boff;
    const int wc;  // index of this wave among the cw waves sharing the B/C stage
    float mean;    // fused aux pad: this row's head/tail token value (io-rounded)
    IO y0;         // fused swap: y at t = 0 of the current sample, written last

    __device__ __forceinline__ ScanWave(const ScanParams& p_, int lane_, int d0_, int b1_, char* own, float* bshared, int wc_)
        : p(p_), lane(lane_), d0(d0_), nrows(max(0, min(kWave, p_.D - d0_))), b1(b1_), wc(wc_), mean(0.0f),
          y0(Io<IO>::zero()) {
        xs = reinterpret_cast<IO*>(own);
        // whole-row staging packs the delta rows right after this tile's x rows
        // (one contiguous transfer list; the planner keeps it 16-byte aligned)
        ds = MODE == 0 ? xs + nrows * p.xrow : reinterpret_cast<IO*>(own + p.xs_bytes);
        bs = bshared;
        cs = bshared + p.ch * NS;
        braw = reinterpret_cast<IO*>(reinterpret_cast<char*>(bshared) + p.bcr_off);
        if constexpr (MODE == 1) {
            // own area: [x | delta | raw B/C] per stage, then float32 B/C (one wave per group)
            own1 = own;
            sb1 = p.xs_bytes + p.ds_bytes + p.rb_bytes;
            xo0 = xo1 = do0 = do1 = 0;
            bs = reinterpret_cast<float*>(own + p.stages * sb1);
            cs = bs + p.ch * NS;
        }
    }

    // States n >= N stay zero in B and C for the whole kernel (the first
    // stage's barrier publishes this to the other waves of the group).
    __device__ __forceinline__ void zero_unused_states() {
        if (wc == 0 && p.N < NS) {
            for (int e = lane; e < p.ch * NS; e += kWave) {
                if (e % NS >= p.N) {
                    bs[e] = 0.0f;
                    cs[e] = 0.0f;
                }
            }
        }
        wave_lds_sync();
    }

    // Per-channel parameters into registers.  Called once, after the first
    // stage's loads are in flight, so that they do not delay those.
    bool params_loaded = false;
    __device__ __forceinline__ void load_params() {
        const int d = d0 + lane;
        const bool valid = d < p.D;
#pragma unroll
        for (int n = 0; n < NS; ++n) A[n] = (valid && n < p.N) ? p.A[(size_t)d * p.N + n] : 0.0f;
        Dk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;
        dbias = (valid && p.dbias) ? p.dbias[d] : 0.0f;
#pragma unroll
        for (int j = 0; j < KW; ++j) cw[j] = (CONV && valid && j < p.K) ? p.conv_w[(size_t)d * p.K + j] : 0.0f;
        cb = (CONV && valid && p.conv_b) ? p.conv_b[d] : 0.0f;
        params_loaded = true;
    }

    // ------------------------------------------------------------ staging
    // Raw B/C of a whole sample (already in LDS) -> float32 [t][n].
    __device__ __forceinline__ void widen_bc() {
        const int L = p.L, tot = p.N * L;
        const float invL = 1.0f / (float)L;
        for (int e = lane; e < tot; e += kWave) {
            const int n = div_small(e, invL);
            const int t = e - n * L;
            bs[t * NS + n] = to_f32(braw[e]);
            cs[t * NS + n] = to_f32(braw[tot + e]);
        }
    }

    // B/C of sample b, positions [lo, lo + cnt) -> float32 [q - boff][n].
    // wide: 16-byte loads of the whole [N x L] block (lo == 0, cnt == L, aligned)
    __device__ __forceinline__ void stage_bc(const IO* bg, const IO* cg, int lo, int cnt, bool wide) {
        const int L = p.L, N = p.N;
        if (wide) {
            constexpr int per = 16 / (int)sizeof(IO);
            const int total = N * L;
            const int units = total / per;
            const float invL = 1.0f / (float)L;
            for (int u0 = 0; u0 < units; u0 += 4 * kWave) {
                uint4 vb[4], vc[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int u = u0 + k * kWave + lane;
                    if (u < units) {
                        vb[k] = reinterpret_cast<const uint4*>(bg)[u];
                        vc[k] = reinterpret_cast<const uint4*>(cg)[u];
                    }
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int u = u0 + k * kWave + lane;
                    if (u < units) {
                        int n = div_small(u * per, invL);
                        int t = u * per - n * L;
#pragma unroll
                        for (int j = 0; j < per; ++j) {
                            bs[t * NS + n] = unpack<IO>(vb[k], j);
                            cs[t * NS + n] = unpack<IO>(vc[k], j);
                            if (++t == L) {
                                t = 0;
                                ++n;
                            }
                        }
                    }
                }
            }
            for (int e = units * per + lane; e < total; e += kWave) {
                const int n = div_small(e, invL);
                const int t = e - n * L;
                bs[t * NS + n] = to_f32(bg[e]);
                cs[t * NS + n] = to_f32(cg[e]);
            }
        } else {
            const int total = N * cnt;
            const float inv = 1.0f / (float)cnt;
            for (int e0 = 0; e0 < total; e0 += 8 * kWave) {
                IO vb[8], vc[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int e = e0 + k * kWave + lane;
                    if (e < total) {
                        const int n = div_small(e, inv);
                        const int i = e - n * cnt;
                        vb[k] = bg[(size_t)n * L + lo + i];
                        vc[k] = cg[(size_t)n * L + lo + i];
                    }
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int e = e0 + k * kWave + lane;
                    if (e < total) {
                        const int n = div_small(e, inv);
                        const int i = e - n * cnt;
                        bs[(lo + i - boff) * NS + n] = to_f32(vb[k]);
                        cs[(lo + i - boff) * NS + n] = to_f32(vc[k]);
                    }
                }
            }
        }
    }

    // Rows x positions [lo, hi) of a [rows, L] slab (lo, hi multiples of the
    // elements per 4-byte word) by 4-byte direct transfers into LDS rows of
    // `rs` elements: LDS word e = k * 64 + lane of instruction k holds word
    // e mod rsw of row e / rsw.  Every lane of every instruction transfers (no
    // lane masks, so sixteen instructions share one LDS base): a slot past
    // the valid rows or words re-reads an in-bounds word of this tile (its
    // byte offset is clamped to the last valid word), and such slots are never
    // read.  A valid word's offset never exceeds that clamp.  Instructions
    // go in whole groups of four (the planner allocates tiles in 1 KB units),
    // sixteen per LDS base where they fill one.
    __device__ __forceinline__ void dma_tile(const IO* g, IO* l, int rs, int lo, int hi, int L, int rows) {
        constexpr int ew = 4 / (int)sizeof(IO);
        const int rsw = rs / ew;        // words per LDS row
        const int nw = (hi - lo) / ew;  // words to move per row
        if (rows <= 0 || nw <= 0) return;
        const int ninst = ((rows * rsw + kWave - 1) / kWave + 3) & ~3;
        const float inv = 1.0f / (float)rsw;
        const uint32_t rowb = (uint32_t)L * (uint32_t)sizeof(IO);
        const uint32_t maxoff = __umul24((uint32_t)(rows - 1), rowb) + (uint32_t)(nw - 1) * 4u;
        const char* gb = reinterpret_cast<const char*>(g + lo);
        char* lb = reinterpret_cast<char*>(l);
        auto one = [&](int kk, auto kc, char* lk) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            const int e = kk * kWave + lane;
            const int r = div_small(e, inv);
            const int w = e - r * rsw;
            const uint32_t off = min(__umul24((uint32_t)r, rowb) + (uint32_t)w * 4u, maxoff);
            dma_at<4, k * 256>(gb + off, lk);
        };
        int k0 = 0;
        for (; k0 + 16 <= ninst; k0 += 16) {
            char* lk = lb + k0 * 256;
            static_for<16>([&](auto kc) { one(k0 + decltype(kc)::value, kc, lk); });
        }
        for (; k0 < ninst; k0 += 4) {
            char* lk = lb + k0 * 256;
            static_for<4>([&](auto kc) { one(k0 + decltype(kc)::value, kc, lk); });
        }
    }

    // rows x [lo, lo + cnt) of a [rows, L] slab -> LDS rows of stride `rs`;
    // positions outside [0, L) become zero.  16 element loads per lane in flight.
    __device__ __forceinline__ void stage_rows(const IO* g, IO* l, int rs, int lo, int cnt, int L) {
        const int total = nrows * cnt;
        const float inv = 1.0f / (float)cnt;
        for (int e0 = 0; e0 < total; e0 += 16 * kWave) {
            IO v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int e = e0 + k * kWave + lane;
                v[k] = Io<IO>::zero();
                if (e < total) {
                    const int c = div_small(e, inv);
                    const int t = lo + e - c * cnt;
                    if (t >= 0 && t < L) v[k] = g[(size_t)c * L + t];
                }
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int e = e0 + k * kWave + lane;
                if (e < total) {
                    const int c = div_small(e, inv);
                    l[c * rs + e - c * cnt] = v[k];
                }
            }
        }
    }

    // Mode 0: put the direct transfers of sample b's whole rows (and, with
    // bc_dma, its raw B/C) in flight.  The [64 x XL] and [64 x L] slabs are
    // contiguous and 16-byte aligned.
    bool prefetched = false;
    __device__ __forceinline__ void issue0(int b) {
        const int L = p.L, D = p.D, XL = p.xrow;
        const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * D + d0) * XL;
        const IO* dg = static_cast<const IO*>(p.delta) + ((size_t)b * D + d0) * L;
        const int nx = nrows * XL, nd = nrows * L;
        // order: parameters, B/C, x, delta.  (The compiler inserts a full vmcnt
        // wait before the first LDS read after these transfers, so the B/C
        // widening and the row mean start once delta has landed as well.)
        if (!params_loaded) load_params();
        if (p.bc_dma && (p.cw == 1 || wc == 0)) {
            const int nbc = p.N * L * (int)sizeof(IO) / 16;
            dma2_to_lds(static_cast<const IO*>(p.Bm) + (size_t)b * p.N * L, nbc,
                        static_cast<const IO*>(p.Cm) + (size_t)b * p.N * L, nbc, braw, lane);
        }
        // the x and delta rows are adjacent in LDS and whole 16-byte units
        const int n0 = nx * (int)sizeof(IO) / 16, n = n0 + nd * (int)sizeof(IO) / 16;
        dma2_to_lds(xg, n0, dg, n - n0, xs, lane);
        delta_only = (n + 63) / 64 - 1 - (n0 - 1) / 64;  // transfers after the last one holding x
    }
    int delta_only = 0;

    // Stage the inputs of sample b for positions [t0, t0 + len) into LDS.
    // With cw > 1 the waves of a group share one B/C stage, written by wave 0
    // between two workgroup barriers (every wave stages the same chunks).
    __device__ __forceinline__ void stage(int b, int t0, int len, bool first) {
        const int L = p.L, D = p.D, N = p.N;
        const int XL = p.xrow;             // row length of the u tensor
        const int sh = p.pad_in ? 1 : 0;   // padded position q reads u row index q - sh
        const bool shared = p.cw > 1;
        if (shared && !first) __syncthreads();  // the previous chunk's B/C has been consumed
        const bool own_bc = !shared || wc == 0;
        const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * D + d0) * XL;
        const IO* dg = static_cast<const IO*>(p.delta) + ((size_t)b * D + d0) * L;
        const IO* bg = static_cast<const IO*>(p.Bm) + (size_t)b * N * L;
        const IO* cg = static_cast<const IO*>(p.Cm) + (size_t)b * N * L;
        if constexpr (MODE == 2) {
            if (p.pad_in && t0 == 0) row_mean(xg);
        }
        if constexpr (MODE == 0) {
            xrs = XL; xoff = sh; drs = L; doff = 0; boff = 0;
            if (!prefetched) issue0(b);
            prefetched = false;
            if (!p.bc_dma && own_bc) stage_bc(bg, cg, 0, L, p.bc_wide != 0);
            // parameters, B/C and x have landed (delta too, by the compiler's wait before the first LDS read)
            wait_vmem_at_most(delta_only);
            wave_lds_sync();
            if (p.bc_dma && own_bc) widen_bc();
            if (p.pad_in) {
                // float64, index order: bit-identical to the aux pad
                const double acc = lane < nrows ? sum_in_order(xs + lane * XL, XL, 0.0) : 0.0;
                mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
            }
            wait_vmem();
            wave_lds_sync();
        } else if constexpr (MODE == 2) {
            xrs = p.xrs; drs = p.drs;
            const int lo = (CONV ? t0 - p.P : t0) - sh;  // u row index of LDS column 0
            xoff = lo + sh;
            doff = t0; boff = t0;
            if (!params_loaded) load_params();
            stage_rows(xg, xs, xrs, lo, CONV ? len + KW - 1 : len, XL);
            stage_rows(dg, ds, drs, t0, len, L);
            if (own_bc) stage_bc(bg, cg, t0, len, false);
        }
        if (shared) __syncthreads();  // B/C of this chunk visible to the whole group
        wave_lds_sync();
    }

    // acc + r[0] + r[1] + ... + r[n-1] in float64, one addition at a time in
    // index order; the LDS reads are issued eight at a time
    __device__ __forceinline__ double sum_in_order(const IO* r, int n, double acc) const {
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

    // Fused aux pad, element-load staging: float64 index-order sum of this
    // lane's whole unpadded row, streamed through the x stage before the
    // sample's first chunk.
    __device__ __forceinline__ void row_mean(const IO* xg) {
        const int XL = p.xrow;
        const int step = p.ch;
        double acc = 0.0;
        for (int c0 = 0; c0 < XL; c0 += step) {
            const int cl = min(step, XL - c0);
            stage_rows(xg, xs, p.xrs, c0, cl, XL);  // positions [c0, c0 + cl) -> columns [0, cl)
            wave_lds_sync();
            if (lane < nrows) acc = sum_in_order(xs + lane * p.xrs, cl, acc);
            wave_lds_sync();
        }
        mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
    }

    // ------------------------------------------------------------ mode 1 pipeline
    // Put the transfers of chunk (sample b, positions [t0, t0 + len)) into
    // stage i: the x tile with its conv halo, the delta tile and the raw B and
    // C rows, each word-aligned; nothing is waited for.
    __device__ __forceinline__ void issue1(int b, int t0, int len, int i) {
        constexpr int ew = 4 / (int)sizeof(IO);
        const int L = p.L, D = p.D, N = p.N, XL = p.xrow;
        const int sh = p.pad_in ? 1 : 0;  // padded position q reads u row index q - sh
        const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * D + d0) * XL;
        const IO* dg = static_cast<const IO*>(p.delta) + ((size_t)b * D + d0) * L;
        const IO* bg = static_cast<const IO*>(p.Bm) + (size_t)b * N * L;
        const IO* cg = static_cast<const IO*>(p.Cm) + (size_t)b * N * L;
        // padded positions [qa, qb) needed, i.e. u row indices [qa - sh, qb - sh)
        int qa = (CONV ? t0 - p.P : t0) - sh;
        int qb = (CONV ? t0 + len + KW - 1 - p.P : t0 + len) - sh;
        qa = max(qa, 0) / ew * ew;
        qb = (min(qb, XL) + ew - 1) / ew * ew;
        const int da = t0 / ew * ew;
        const int db = (t0 + len + ew - 1) / ew * ew;
        if (i) {
            xo1 = qa + sh;
            do1 = da;
        } else {
            xo0 = qa + sh;
            do0 = da;
        }
        // the stage was last read by LDS instructions of this wave (y stores);
        // they have completed before any transfer can write it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (qb > qa) dma_tile(xg, xs_of(i), p.xrs, qa, qb, XL, nrows);
        dma_tile(dg, ds_of(i), p.drs, da, db, L, nrows);
        IO* rb = rb_of(i);
        dma_tile(bg, rb, p.rb_rs, da, db, L, N);
        dma_tile(cg, rb + p.rb_bytes / 2 / (int)sizeof(IO), p.rb_rs, da, db, L, N);
        if (!params_loaded) load_params();
    }

    // Raw B/C rows of stage i -> float32 [q - t0][n] for q in [t0, t0 + len).
    __device__ __forceinline__ void widen1(int t0, int len, int i) {
        const int N = p.N, rs = p.rb_rs;
        const IO* rb = rb_of(i) + t0 - (i ? do1 : do0);
        const IO* rc = rb + p.rb_bytes / 2 / (int)sizeof(IO);
        const int tot = N * len;
        const float inv = 1.0f / (float)len;
        for (int e = lane; e < tot; e += kWave) {
            const int n = div_small(e, inv);
            const int q = e - n * len;
            bs[q * NS + n] = to_f32(rb[n * rs + q]);
            cs[q * NS + n] = to_f32(rc[n * rs + q]);
        }
    }

    // Point the compute / store geometry at stage i holding positions from t0.
    __device__ __forceinline__ void use1(int i, int t0) {
        xs = xs_of(i);
        ds = ds_of(i);
        xrs = p.xrs;
        drs = p.drs;
        xoff = i ? xo1 : xo0;
        doff = i ? do1 : do0;
        boff = t0;  // B/C rows hold exactly [t0, t0 + len): ch rows are allocated
    }

    // Fused aux pad: float64 index-order sum of this lane's whole unpadded row
    // of sample b, streamed in windows through the two halves of the stage
    // region (every stage's x, delta and raw B/C areas, all free here; each
    // half a whole number of KB, rows an odd number of words apart): the
    // transfer of window k+1 is in flight while window k is summed.
    __device__ __forceinline__ void mean1(int b) {
        constexpr int ew = 4 / (int)sizeof(IO);
        const int XL = p.xrow;
        const IO* xg = static_cast<const IO*>(p.u) + ((size_t)b * p.D + d0) * XL;
        const int half = (p.stages * sb1 / 2) & ~1023;
        const int rs = (((half / (kWave * 4)) - 1) | 1) * ew;  // row pitch, elements
        const int step = rs - 2 * (ew - 1);                    // window, with room for word alignment
        auto area = [&](int i) __attribute__((always_inline)) { return reinterpret_cast<IO*>(own1 + i * half); };
        auto stride = [&](int) __attribute__((always_inline)) { return rs; };
        auto issue = [&](int c0, int i) __attribute__((always_inline)) {
            const int lo = c0 / ew * ew;
            const int hi = min((c0 + min(step, XL - c0) + ew - 1) / ew * ew, XL);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            dma_tile(xg, area(i), stride(i), lo, hi, XL, nrows);
        };
        double acc = 0.0;
        int i = 0;
        issue(0, 0);
        for (int c0 = 0; c0 < XL; c0 += step, i ^= 1) {
            wait_vmem();
            wave_lds_sync();
            if (c0 + step < XL) issue(c0 + step, i ^ 1);
            const int cl = min(step, XL - c0);
            if (lane < nrows) acc = sum_in_order(area(i) + lane * stride(i) + c0 - c0 / ew * ew, cl, acc);
        }
        wave_lds_sync();
        mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
    }

    // Folded positions [sa, sb) of row b1 through the stages.  Two stages, per
    // chunk: wait for its transfers, store the previous chunk's y (from the
    // other stage), refill the other stage with the next chunk, widen B/C,
    // compute.  A chunk that starts a sample with the fused pad is not
    // prefetched: the row mean needs both stages first.  One stage: wait,
    // widen, compute, store, then fetch the next chunk.
    __device__ __forceinline__ void run1(bool out, int sa, int sb, float (&h)[NS], float& sd2) {
        if (sa >= sb) return;
        const int L = p.L;
        const bool two = p.stages == 2;
        // chunk cursor: sample j of the folded row, positions [t0, t0 + len)
        int s = sa;
        int j = s / L;
        int t0 = s - j * L;
        auto len_at = [&](int ss, int tt) __attribute__((always_inline)) { return min(min(p.ch, L - tt), sb - ss); };
        int len = len_at(s, t0);
        const int bb = b1 * p.B2;
        int i = 0;
        // with the fused pad, the aux tokens at positions 0 and L-1 are the row
        // mean: a piece's segment of a sample needs it when its conv inputs
        // reach either end (a new sample inside the piece starts at 0)
        if (p.pad_in) {
            const int seg_end = min(sb - (s - t0), L);  // end of this piece's part of sample j
            const int first_x = CONV ? t0 - p.P : t0;
            const int last_x = CONV ? seg_end - 1 + KW - 1 - p.P : seg_end - 1;
            if (first_x <= 0 || last_x >= L - 1) mean1(bb + j);
        }
        issue1(bb + j, t0, len, i);
        int pb = -1, pt0 = 0, plen = 0;  // chunk whose y waits in stage i ^ 1
        while (true) {
            wait_vmem();  // this chunk has landed; so have the stores issued before its transfers
            wave_lds_sync();
            if (pb >= 0) {
                use1(i ^ 1, pt0);
                store(pb, pt0, plen);
                pb = -1;
            }
            const int sn = s + len;
            const bool more = sn < sb;
            int nj = j, nt0 = t0 + len;
            if (nt0 == L) {
                nt0 = 0;
                ++nj;
            }
            const int nlen = more ? len_at(sn, nt0) : 0;
            const bool pre = two && more && !(p.pad_in && nt0 == 0);
            if (pre) issue1(bb + nj, nt0, nlen, i ^ 1);
            widen1(t0, len, i);
            wave_lds_sync();
            use1(i, t0);
            if (out) chunk<true>(t0, len, h, sd2);
            else chunk<false>(t0, len, h, sd2);
            wave_lds_sync();
            if (out) {
                if (two) {
                    pb = bb + j;
                    pt0 = t0;
                    plen = len;
                } else {
                    store(bb + j, t0, len);
                }
            }
            if (!more) break;
            s = sn;
            j = nj;
            t0 = nt0;
            len = nlen;
            if (two) i ^= 1;
            if (!pre) {
                // not prefetched: store the pending y, take the row mean when
                // the chunk starts a sample with the fused pad, then fetch it
                if (pb >= 0) {
                    use1(i ^ 1, pt0);
                    store(pb, pt0, plen);
                    pb = -1;
                }
                if (p.pad_in && t0 == 0) {
                    wait_vmem();
                    mean1(bb + j);
                }
                issue1(bb + j, t0, len, i);
            }
        }
        if (pb >= 0) {
            use1(i, pt0);
            store(pb, pt0, plen);
        }
    }

    // Store y for positions [t0, t0 + len) of sample b (y sits in ds).  With
    // the fused swap, position 0 is written at column L-1 and vice versa.
    __device__ __forceinline__ void store(int b, int t0, int len) {
        const int L = p.L;
        IO* yg = static_cast<IO*>(p.y) + ((size_t)b * p.D + d0) * L;
        const bool sw = p.swap_out && L > 1;
        if constexpr (MODE == 0) {  // whole rows: len == L
            if (sw && lane < nrows) {  // exchange the two end tokens of this lane's row in LDS
                const IO a = ds[lane * L];
                ds[lane * L] = ds[lane * L + L - 1];
                ds[lane * L + L - 1] = a;
            }
            wave_lds_sync();
            const int units = nrows * L * (int)sizeof(IO) / 16;  // whole units (planner)
            for (int u = lane; u < units; u += kWave)
                reinterpret_cast<uint4*>(yg)[u] = reinterpret_cast<const uint4*>(ds)[u];
            wave_lds_sync();
        } else {
        // positions written here; the ends go out last when swapping
        const int lo = (sw && t0 == 0) ? 1 : t0;
        const int hi = (sw && t0 + len == L) ? L - 1 : t0 + len;
        // mode 1 writes each swapped end as soon as it is computed (pieces of a
        // sample may sit in different waves; y never overlaps an input), mode 2
        // holds y at t = 0 until the sample's last chunk
        if (sw && t0 == 0 && lane < nrows) {
            if constexpr (MODE == 1) yg[(size_t)lane * L + L - 1] = ds[lane * drs + 0 - doff];
            else y0 = ds[lane * drs + 0 - doff];
        }
        if constexpr (MODE == 1) {
            // whole 4-byte words inside [lo, hi), single elements at the
            // edges; each lane writes its own row (immediate offsets, no
            // per-word index arithmetic)
            constexpr int ew = 4 / (int)sizeof(IO);
            const int ta = (lo + ew - 1) / ew * ew;
            const int tb = max(ta, hi / ew * ew);
            if (lane < nrows) {
                const int nw = (tb - ta) / ew;
                const uint32_t* src = reinterpret_cast<const uint32_t*>(ds + lane * drs + ta - doff);
                uint32_t* dst = reinterpret_cast<uint32_t*>(yg + (size_t)lane * L + ta);
                int w = 0;
                for (; w + 4 <= nw; w += 4) {
                    const uint32_t v0 = src[w], v1 = src[w + 1], v2 = src[w + 2], v3 = src[w + 3];
                    dst[w] = v0;
                    dst[w + 1] = v1;
                    dst[w + 2] = v2;
                    dst[w + 3] = v3;
                }
                for (; w < nw; ++w) dst[w] = src[w];
                for (int t = lo; t < min(ta, hi); ++t) yg[(size_t)lane * L + t] = ds[lane * drs + t - doff];
                for (int t = tb; t < hi; ++t) yg[(size_t)lane * L + t] = ds[lane * drs + t - doff];
            }
        } else if (hi > lo) {
            const int cnt = hi - lo;
            const float inv = 1.0f / (float)cnt;
            for (int e = lane; e < nrows * cnt; e += kWave) {
                const int c = div_small(e, inv);
                const int i = e - c * cnt;
                yg[(size_t)c * L + lo + i] = ds[c * drs + (lo - doff) + i];
            }
        }
        if (sw && t0 + len == L && lane < nrows) {
            yg[(size_t)lane * L] = ds[lane * drs + (L - 1) - doff];
            if constexpr (MODE != 1) yg[(size_t)lane * L + L - 1] = y0;
        }
        wave_lds_sync();
        }
    }

    // ------------------------------------------------------------ compute
    // Conv/scan input at padded position q (wave-uniform): zero outside the
    // sample, the aux-token value at both ends when the pad is fused, else the
    // staged value.  Branch-free: the LDS read always hits a valid column.
    __device__ __forceinline__ float xat(const IO* xr, int q, int L, bool pad) const {
        const int lo = pad ? 1 : 0;
        const int qc = min(max(q, lo), L - 1 - lo);
        float v = to_f32(xr[qc]);
        v = (pad && (q == 0 || q == L - 1)) ? mean : v;
        return (q < 0 || q >= L) ? 0.0f : v;
    }

    // B[t, :] and C[t, :] of one position from LDS (16-byte broadcast reads)
    __device__ __forceinline__ void load_bc(const float* br, const float* cr, int t, float4 (&bq)[NS / 4],
                                            float4 (&cq)[NS / 4]) {
        const float4* b4 = reinterpret_cast<const float4*>(br + t * NS);
        const float4* c4 = reinterpret_cast<const float4*>(cr + t * NS);
#pragma unroll
        for (int q = 0; q < NS / 4; ++q) {
            bq[q] = b4[q];
            cq[q] = c4[q];
        }
    }

    // Makes all of one position's B/C values live at once, so the reads that
    // produced them are waited for with a single counter wait.
    __device__ __forceinline__ static void pin_bc(const float4 (&bq)[NS / 4], const float4 (&cq)[NS / 4]) {
#pragma unroll
        for (int q = 0; q < NS / 4; q += 2) {
            if constexpr (NS >= 8) {
                asm volatile("" ::"v"(bq[q].x), "v"(bq[q].y), "v"(bq[q].z), "v"(bq[q].w), "v"(bq[q + 1].x),
                             "v"(bq[q + 1].y), "v"(bq[q + 1].z), "v"(bq[q + 1].w), "v"(cq[q].x), "v"(cq[q].y),
                             "v"(cq[q].z), "v"(cq[q].w), "v"(cq[q + 1].x), "v"(cq[q + 1].y), "v"(cq[q + 1].z),
                             "v"(cq[q + 1].w));
            } else {
                asm volatile("" ::"v"(bq[q].x), "v"(bq[q].y), "v"(bq[q].z), "v"(bq[q].w), "v"(cq[q].x),
                             "v"(cq[q].y), "v"(cq[q].z), "v"(cq[q].w));
            }
        }
    }

    // One position: conv tap in, Delta, N-state update, readout.  The inputs
    // arrive as raw LDS bits (xb as float32 bits when XF32, else io bits; db
    // always io bits) and are widened here, after the pin, so that the reads
    // issued for the next position stay in flight while this one computes.
    template <bool OUT, bool FIRST, bool XF32>
    __device__ __forceinline__ float core(uint32_t xb, uint32_t db, float (&h)[NS], float (&win)[KW], float& sd2,
                                          const float4 (&bq)[NS / 4], const float4 (&cq)[NS / 4]) {
        // Opaque to the compiler: pins this position's work after the previous
        // position's, so the exp work of later positions is not hoisted (it
        // would cost ~N registers per position and spill).
        asm volatile("" : "+v"(xb), "+v"(db));
        pin_bc(bq, cq);
        const float xnew = XF32 ? __uint_as_float(xb) : Io<IO>::of_bits(xb);
        const float dl = Io<IO>::of_bits(db) + dbias;
        float u;
        if constexpr (CONV) {
#pragma unroll
            for (int j = 0; j < KW - 1; ++j) win[j] = win[j + 1];
            win[KW - 1] = xnew;
            float acc = cb;
#pragma unroll
            for (int j = 0; j < KW; ++j) acc = __builtin_fmaf(cw[j], win[j], acc);
            u = SILU ? silu(acc) : acc;
        } else {
            u = xnew;
        }
        float d2, dt;  // Delta * log2(e) and Delta
        if constexpr (SP) {
            d2 = softplus_log2e(dl);
            dt = d2 * kLn2;
        } else {
            dt = dl;  // exact, so integer-valued steps stay exact
            d2 = dl * kLog2e;
        }
        const float du = dt * u;
        if constexpr (!OUT) sd2 += d2;
        float yv = Dk * u;
#pragma unroll
        for (int q = 0; q < NS / 4; ++q) {
            const float bv[4] = {bq[q].x, bq[q].y, bq[q].z, bq[q].w};
            const float cv[4] = {cq[q].x, cq[q].y, cq[q].z, cq[q].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int n = q * 4 + k;
                const float bx = du * bv[k];
                if constexpr (FIRST) {
                    h[n] = bx;  // reset: state re-initialised at the sample start
                } else {
                    const float a = exp2_fast(d2 * A[n]);
                    h[n] = __builtin_fmaf(a, h[n], bx);
                }
                if constexpr (OUT) yv = __builtin_fmaf(cv[k], h[n], yv);
            }
        }
        return yv;
    }

    // Positions [t, tend) (none of them a sample start), software-pipelined:
    // two register sets are used alternately, position t computing from one
    // while position t+1's LDS reads land in the other, so nothing is copied.
    // CHECK: the newest conv tap may fall outside the sample or on a fused aux
    // token, so it goes through xat; otherwise it is read from LDS directly.
    template <bool OUT, bool CHECK>
    __device__ __forceinline__ void steps(int t, int tend, const IO* xr, IO* dr, const float* br, const float* cr,
                                          int lag, float (&h)[NS], float (&win)[KW], float& sd2) {
        if (t >= tend) return;
        const int L = p.L;
        const bool pad = p.pad_in != 0;
        auto fetch = [&](int tt, uint32_t& xv, uint32_t& dv, float4 (&bb)[NS / 4], float4 (&cc)[NS / 4])
                         __attribute__((always_inline)) {
            if constexpr (CHECK) xv = __float_as_uint(xat(xr, tt + lag, L, pad));
            else xv = Io<IO>::bits(xr[tt + lag]);
            dv = Io<IO>::bits(dr[tt]);
            load_bc(br, cr, tt, bb, cc);
        };
        uint32_t x0, d0, x1, d1;
        float4 bq0[NS / 4], cq0[NS / 4], bq1[NS / 4], cq1[NS / 4];
        auto step = [&](int tt, uint32_t xv, uint32_t dv, const float4 (&bb)[NS / 4], const float4 (&cc)[NS / 4])
                        __attribute__((always_inline)) {
            const float yv = core<OUT, false, CHECK>(xv, dv, h, win, sd2, bb, cc);
            if constexpr (OUT) dr[tt] = from_f32<IO>(yv);
        };
        fetch(t, x0, d0, bq0, cq0);
        if constexpr (!CHECK) {
            // four positions per trip (with a four-tap conv window the window
            // registers return to their roles after one trip: nothing is copied)
            for (; t + 4 < tend; t += 4) {
                fetch(t + 1, x1, d1, bq1, cq1);
                step(t, x0, d0, bq0, cq0);
                fetch(t + 2, x0, d0, bq0, cq0);
                step(t + 1, x1, d1, bq1, cq1);
                fetch(t + 3, x1, d1, bq1, cq1);
                step(t + 2, x0, d0, bq0, cq0);
                fetch(t + 4, x0, d0, bq0, cq0);
                step(t + 3, x1, d1, bq1, cq1);
            }
        } else {
            for (; t + 2 < tend; t += 2) {
                fetch(t + 1, x1, d1, bq1, cq1);
                step(t, x0, d0, bq0, cq0);
                fetch(t + 2, x0, d0, bq0, cq0);
                step(t + 1, x1, d1, bq1, cq1);
            }
        }
        // the last one to four positions; set 0 holds position t
        const int r = tend - t;
        if (r >= 2) fetch(t + 1, x1, d1, bq1, cq1);
        step(t, x0, d0, bq0, cq0);
        if (r >= 2) {
            if (r >= 3) fetch(t + 2, x0, d0, bq0, cq0);
            step(t + 1, x1, d1, bq1, cq1);
            if (r >= 3) {
                if (r >= 4) fetch(t + 3, x1, d1, bq1, cq1);
                step(t + 2, x0, d0, bq0, cq0);
                if (r >= 4) step(t + 3, x1, d1, bq1, cq1);
            }
        }
    }

    // Scan positions [t0, t0 + len) of the staged sample.  OUT: write y into ds.
    // AGG (OUT = false): accumulate the sum of Delta*log2e in sd2, no output.
    template <bool OUT>
    __device__ __forceinline__ void chunk(int t0, int len, float (&h)[NS], float& sd2) {
        const int L = p.L;
        const int P = CONV ? p.P : 0;
        const IO* xr = xs + lane * xrs - xoff;
        IO* dr = ds + lane * drs - doff;
        const float* br = bs - boff * NS;
        const float* cr = cs - boff * NS;
        const bool pad = p.pad_in != 0;
        float win[KW];
#pragma unroll
        for (int j = 0; j < KW; ++j) win[j] = 0.0f;
        if constexpr (CONV) {
#pragma unroll
            for (int j = 0; j < KW - 1; ++j) win[j + 1] = xat(xr, t0 - P + j, L, pad);
        }
        const int lag = CONV ? KW - 1 - P : 0;  // newest conv tap is x[t + lag]; P < K <= KW
        int t = t0;
        const int tend = t0 + len;
        if (t == 0) {
            float4 bq[NS / 4], cq[NS / 4];
            load_bc(br, cr, 0, bq, cq);
            const float y0 = core<OUT, true, true>(__float_as_uint(xat(xr, lag, L, pad)),
                                                             Io<IO>::bits(dr[0]), h, win, sd2, bq, cq);
            if constexpr (OUT) dr[0] = from_f32<IO>(y0);
            ++t;
        }
        // From t >= 1 on the tap t + lag >= 1 is inside the sample and past a
        // fused head token; it stays before the tail token while t < tf.
        const int tf = max(t, min(tend, L - (pad ? 1 : 0) - lag));
        steps<OUT, false>(t, tf, xr, dr, br, cr, lag, h, win, sd2);
        steps<OUT, true>(tf, tend, xr, dr, br, cr, lag, h, win, sd2);
    }

    // Run folded positions [sa, sb) of row b1, state carried in h.
    // out: write y (phase 2); else accumulate the aggregate (phase 1).  One
    // call site, so the staging code is inlined once.
    __device__ __forceinline__ void run(bool out, int sa, int sb, float (&h)[NS], float& sd2) {
        if constexpr (MODE == 1) {
            run1(out, sa, sb, h, sd2);
        } else {
            const int L = p.L;
            int s = sa;
            bool first = true;
            while (s < sb) {
                const int j = s / L;
                const int t0 = s - j * L;
                const int len = min(min(p.ch, L - t0), sb - s);
                const int b = b1 * p.B2 + j;
                stage(b, t0, len, first);
                first = false;
                if (out) chunk<true>(t0, len, h, sd2);
                else chunk<false>(t0, len, h, sd2);
                wave_lds_sync();
                if (out) store(b, t0, len);
                s += len;
            }
        }
    }
};

template <typename IO, int NS, int KW, bool CONV, bool SP, bool SILU, int MODE>
__global__ __launch_bounds__(kWave * kMaxWaves) __attribute__((amdgpu_waves_per_eu(NS <= 8 ? 3 : 2)))
void scan_kernel(ScanParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    if (p.stagger_ticks) {
        const unsigned long long r = blockIdx.x / p.stagger_period;
        if (r) {
            const unsigned long long until = __builtin_amdgcn_s_memrealtime() + r * p.stagger_ticks;
            while (__builtin_amdgcn_s_memrealtime() < until) __builtin_amdgcn_s_sleep(2);
        }
    }
    const int lane = threadIdx.x & (kWave - 1);
    // the wave index is the same for all 64 lanes; saying so keeps every
    // position/piece index derived from it in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
    // giving each XCD a contiguous run of (row, tile) items keeps the B/C of a
    // folded row in one XCD's L2.
    // With wsplit every piece of a folded row is a workgroup of its own
    // (pieces on sample starts need no exchange), consecutive in this order.
    const int G = p.tgroups * p.B1 * (p.wsplit ? p.waves : 1);
    int g = blockIdx.x;
    if ((G & 7) == 0) g = (g & 7) * (G >> 3) + (g >> 3);
    int wp = 0;
    if (p.wsplit) {
        wp = g % p.waves;
        g /= p.waves;
    }
    const int b1 = g / p.tgroups;
    const int tg = g - b1 * p.tgroups;
    if (!p.wsplit) wp = wave / p.cw;    // piece of the folded row
    const int wc = wave - (p.wsplit ? 0 : wp) * p.cw;  // channel tile within the group
    char* grp = smem + (size_t)(p.wsplit ? 0 : wp) * p.group_bytes;
    ScanWave<IO, NS, KW, CONV, SP, SILU, MODE> w(p, lane, (tg * p.cw + wc) * kWave, b1,
                                 grp + p.bc_bytes + (size_t)wc * (p.xs_bytes + p.ds_bytes),
                                 reinterpret_cast<float*>(grp), wc);

    const int S = p.B2 * p.L;
    const int p0 = min(wp * p.piece, S);
    const int p1 = min(p0 + p.piece, S);
    // whole-row staging without carries: the first sample's transfers go out
    // before anything else, so they overlap the rest of the set-up
    if (MODE == 0 && !p.need_carry && p0 < p1) {
        w.issue0(b1 * p.B2 + p0 / p.L);
        w.prefetched = true;
    }
    w.zero_unused_states();
    float h[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = 0.0f;
    float sd2 = 0.0f;

    // phase 1 (only with carries): aggregate of the tail segment of this
    // piece; phase 2: scan the piece from the carried state and write y
    // (whole-row staging never has carries: the planner keeps mode 0 for
    // pieces that start on sample boundaries)
    const bool carry = MODE != 0 && p.need_carry;
    for (int phase = carry ? 1 : 2; phase <= 2; ++phase) {
        int sa = p0, flag = 1;
        if (phase == 1 && p0 < p1) {
            sa = ((p1 - 1) / p.L) * p.L;  // last sample start in the piece
            if (sa < p0) {
                sa = p0;
                flag = 0;
            }
        }
        if (sa < p1) w.run(phase == 2, sa, p1, h, sd2);
        if (MODE == 0 || phase == 2) break;
        char* agg = smem + (size_t)p.waves * p.group_bytes;  // cw == 1 here: wave == piece
        int* aflag = reinterpret_cast<int*>(agg);
        float* asum = reinterpret_cast<float*>(agg + kMaxWaves * sizeof(int));
        float* ah = asum + (size_t)p.waves * kWave;
        if (lane == 0) aflag[wave] = flag;
        asum[wave * kWave + lane] = sd2;
#pragma unroll
        for (int n = 0; n < NS; ++n) ah[((size_t)wave * NS + n) * kWave + lane] = h[n];
        __syncthreads();
        // carry-in: fold predecessors with the segmented operator
        if (!w.params_loaded) w.load_params();
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
}

template <typename IO, int NS, int KW, bool CONV, bool SP, bool SILU, int MODE>
hipError_t launch_t(const ScanParams& p, hipStream_t stream) {
    auto kern = scan_kernel<IO, NS, KW, CONV, SP, SILU, MODE>;
    static bool attr_set = false;
    if (!attr_set && p.lds_bytes > 64 * 1024) {
        // allow dynamic LDS beyond 64 KB (gfx950 has 160 KB per workgroup)
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024) != hipSuccess)
            (void)hipGetLastError();  // do not leave a stale error for the launch check
        attr_set = true;
    }
    const unsigned grid = (unsigned)(p.tgroups * p.B1 * (p.wsplit ? p.waves : 1));
    const unsigned block = (unsigned)(kWave * p.cw * (p.wsplit ? 1 : p.waves));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), (size_t)p.lds_bytes, stream, p);
    return hipGetLastError();
}

// The staging mode, softplus on/off and the conv activation select separate
// kernels, so each kernel holds only the staging path and position loop it
// runs (a runtime choice would let the compiler keep every path's set-up live).
template <typename IO, int NS, int KW, bool CONV, bool SP, bool SILU>
hipError_t launch_mode(const ScanParams& p, hipStream_t s) {
    if (p.mode == 0) return launch_t<IO, NS, KW, CONV, SP, SILU, 0>(p, s);
    if (p.mode == 1) return launch_t<IO, NS, KW, CONV, SP, SILU, 1>(p, s);
    return launch_t<IO, NS, KW, CONV, SP, SILU, 2>(p, s);
}

template <typename IO, int NS, int KW, bool CONV>
hipError_t launch_sp(const ScanParams& p, hipStream_t s) {
    const bool silu = CONV && p.act == 1;
    if (p.softplus)
        return silu ? launch_mode<IO, NS, KW, CONV, true, CONV>(p, s) : launch_mode<IO, NS, KW, CONV, true, false>(p, s);
    return silu ? launch_mode<IO, NS, KW, CONV, false, CONV>(p, s) : launch_mode<IO, NS, KW, CONV, false, false>(p, s);
}

template <typename IO, int NS>
hipError_t launch_ns(const ScanParams& p, hipStream_t s) {
    if (!p.conv_w) return launch_sp<IO, NS, 4, false>(p, s);
    if (p.K <= 4) return launch_sp<IO, NS, 4, true>(p, s);
    return launch_sp<IO, NS, 8, true>(p, s);
}

}  // namespace scan_detail
}  // namespace sfm

// One translation unit per (io type, state count) instantiates the kernels:
// SFM_SCAN_INSTANCE(float, f32, 8) defines sfm::launch_scan_f32_n8.
#define SFM_SCAN_INSTANCE(IOT, NAME, NSV)                                                     \
    namespace sfm {                                                                          \
    hipError_t launch_scan_##NAME##_n##NSV(const ScanParams& p, hipStream_t s) {             \
        return scan_detail::launch_ns<IOT, NSV>(p, s);                                        \
    }                                                                                         \
    }
