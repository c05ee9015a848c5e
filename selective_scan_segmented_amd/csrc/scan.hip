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
//                the 64 lanes read one column);
//      mode 2 -- element loads (any shape), 16 per lane in flight.
//    B and C become float32 [t][n] in LDS; y overwrites delta in LDS and is
//    stored with wide coalesced stores.
//  * The position loop is software-pipelined: the LDS reads of position t+1
//    are issued before position t computes, so the wave does not wait on LDS
//    latency each step, and at most two positions' inputs are live.
//  * The optional depthwise conv is fused: a register window slides over the
//    staged conv input and taps outside the sample read zero (the boundary
//    masking of the techloop walkthrough's conv-boundary part).
#include "sfm_device.h"
#include "sfm_internal.h"

namespace sfm {

namespace {

constexpr int kMaxWaves = 8;

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
    // LDS stages
    IO* xs;
    IO* ds;
    float* bs;
    float* cs;
    // geometry of the staged chunk: value at position q of this lane's row is
    // xs[lane*xrs + q - xoff], ds[lane*drs + q - doff]; B/C at bs[(q-boff)*NS + n]
    int xrs, xoff, drs, doff, boff;
    const int wc;  // index of this wave among the cw waves sharing the B/C stage
    float mean;    // fused aux pad: this row's head/tail token value (io-rounded)
    IO y0;         // fused swap: y at t = 0 of the current sample, written last

    __device__ ScanWave(const ScanParams& p_, int lane_, int d0_, int b1_, char* own, float* bshared, int wc_)
        : p(p_), lane(lane_), d0(d0_), nrows(max(0, min(kWave, p_.D - d0_))), b1(b1_), wc(wc_), mean(0.0f),
          y0(Io<IO>::zero()) {
        const int d = d0 + lane;
        const bool valid = d < p.D;
#pragma unroll
        for (int n = 0; n < NS; ++n) A[n] = (valid && n < p.N) ? p.A[(size_t)d * p.N + n] : 0.0f;
        Dk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;
        dbias = (valid && p.dbias) ? p.dbias[d] : 0.0f;
#pragma unroll
        for (int j = 0; j < KW; ++j) cw[j] = (CONV && valid && j < p.K) ? p.conv_w[(size_t)d * p.K + j] : 0.0f;
        cb = (CONV && valid && p.conv_b) ? p.conv_b[d] : 0.0f;
        xs = reinterpret_cast<IO*>(own);
        ds = reinterpret_cast<IO*>(own + p.xs_bytes);
        bs = bshared;
        cs = bshared + p.ch * NS;
        // states n >= N stay zero in B and C for the whole kernel (the first
        // stage's barrier publishes this to the other waves of the group)
        if (wc == 0) {
            for (int e = lane; e < p.ch * NS; e += kWave) {
                bs[e] = 0.0f;
                cs[e] = 0.0f;
            }
        }
        wave_lds_sync();
    }

    // ------------------------------------------------------------ staging
    // B/C of sample b, positions [lo, lo + cnt) -> float32 [q - boff][n].
    // wide: 16-byte loads of the whole [N x L] block (lo == 0, cnt == L, aligned)
    __device__ void stage_bc(const IO* bg, const IO* cg, int lo, int cnt, bool wide) {
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

    // mode 1: rows x positions [lo, hi) (lo, hi multiples of the elements per
    // 4-byte word) by 4-byte direct transfers into LDS rows of `rs` elements.
    // Lane-contiguous LDS words, per-lane global addresses; words outside the
    // valid rows are not transferred (never read).
    __device__ void dma_tile(const IO* g, IO* l, int rs, int lo, int hi, int L) {
        constexpr int ew = 4 / (int)sizeof(IO);
        const int rsw = rs / ew;        // words per LDS row (odd)
        const int nw = (hi - lo) / ew;  // words to move per row
        const float inv = 1.0f / (float)rsw;
        char* lb = reinterpret_cast<char*>(l);
        for (int k = 0; k < rsw; ++k) {  // 64 words per instruction, rsw instructions per tile
            const int e = k * kWave + lane;
            const int r = div_small(e, inv);
            const int w = e - r * rsw;
            if (r < nrows && w < nw)
                __builtin_amdgcn_global_load_lds(g + (size_t)r * L + lo + w * ew, (lds_void_ptr)(lb + k * 256), 4, 0,
                                                 0);
        }
    }

    // rows x [lo, lo + cnt) of a [rows, L] slab -> LDS rows of stride `rs`;
    // positions outside [0, L) become zero.  16 element loads per lane in flight.
    __device__ void stage_rows(const IO* g, IO* l, int rs, int lo, int cnt, int L) {
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

    // Stage the inputs of sample b for positions [t0, t0 + len) into LDS.
    // With cw > 1 the waves of a group share one B/C stage, written by wave 0
    // between two workgroup barriers (every wave stages the same chunks).
    __device__ void stage(int b, int t0, int len, bool first) {
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
        if (p.pad_in && p.mode != 0 && t0 == 0) row_mean(xg);
        if (p.mode == 0) {
            // whole sample rows: the [64 x XL] and [64 x L] slabs are contiguous
            // and 16-byte aligned; copy them straight into LDS, all in flight
            xrs = XL; xoff = sh; drs = L; doff = 0; boff = 0;
            const int nx = nrows * XL, nd = nrows * L;
            dma_to_lds(xg, xs, nx * (int)sizeof(IO), lane);
            dma_to_lds(dg, ds, nd * (int)sizeof(IO), lane);
            const int donex = (nx * (int)sizeof(IO) & ~15) / (int)sizeof(IO);
            const int doned = (nd * (int)sizeof(IO) & ~15) / (int)sizeof(IO);
            if (lane < nx - donex) xs[donex + lane] = xg[donex + lane];
            if (lane < nd - doned) ds[doned + lane] = dg[doned + lane];
            if (own_bc) stage_bc(bg, cg, 0, L, p.bc_wide != 0);
            wait_vmem();
            if (p.pad_in) {
                wave_lds_sync();
                double acc = 0.0;  // float64, index order: bit-identical to the aux pad
                if (lane < nrows)
                    for (int i = 0; i < XL; ++i) acc += (double)to_f32(xs[lane * XL + i]);
                mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
            }
        } else if (p.mode == 1) {
            constexpr int ew = 4 / (int)sizeof(IO);
            xrs = p.xrs; drs = p.drs;
            // padded positions [qa, qb) needed, i.e. u row indices [qa - sh, qb - sh)
            int qa = (CONV ? t0 - p.P : t0) - sh;
            int qb = (CONV ? t0 + len + KW - 1 - p.P : t0 + len) - sh;
            qa = max(qa, 0) / ew * ew;
            qb = (min(qb, XL) + ew - 1) / ew * ew;
            xoff = qa + sh;
            const int da = t0 / ew * ew;
            const int db = (t0 + len + ew - 1) / ew * ew;
            doff = da;
            boff = t0;  // B/C rows hold exactly [t0, t0 + len): ch rows are allocated
            if (qb > qa) dma_tile(xg, xs, xrs, qa, qb, XL);
            dma_tile(dg, ds, drs, da, db, L);
            if (own_bc) stage_bc(bg, cg, t0, len, false);
            wait_vmem();
        } else {
            xrs = p.xrs; drs = p.drs;
            const int lo = (CONV ? t0 - p.P : t0) - sh;  // u row index of LDS column 0
            xoff = lo + sh;
            doff = t0; boff = t0;
            stage_rows(xg, xs, xrs, lo, CONV ? len + KW - 1 : len, XL);
            stage_rows(dg, ds, drs, t0, len, L);
            if (own_bc) stage_bc(bg, cg, t0, len, false);
        }
        if (shared) __syncthreads();  // B/C of this chunk visible to the whole group
        wave_lds_sync();
    }

    // Fused aux pad, chunked rows: float64 index-order sum of this lane's whole
    // unpadded row, streamed through the x stage before the sample's first chunk.
    __device__ void row_mean(const IO* xg) {
        constexpr int ew = 4 / (int)sizeof(IO);
        const int XL = p.xrow;
        const int step = p.ch;
        double acc = 0.0;
        for (int c0 = 0; c0 < XL; c0 += step) {
            const int cl = min(step, XL - c0);
            int lo = c0;
            if (p.mode == 1) {
                lo = c0 / ew * ew;
                const int hi = (c0 + cl + ew - 1) / ew * ew;
                dma_tile(xg, xs, p.xrs, lo, min(hi, XL), XL);
                wait_vmem();
            } else {
                stage_rows(xg, xs, p.xrs, c0, cl, XL);
            }
            wave_lds_sync();
            if (lane < nrows)
                for (int i = c0; i < c0 + cl; ++i) acc += (double)to_f32(xs[lane * p.xrs + i - lo]);
            wave_lds_sync();
        }
        mean = to_f32(Io<IO>::from_f64(acc / (double)XL));
    }

    // Store y for positions [t0, t0 + len) of sample b (y sits in ds).  With
    // the fused swap, position 0 is written at column L-1 and vice versa.
    __device__ void store(int b, int t0, int len) {
        const int L = p.L;
        IO* yg = static_cast<IO*>(p.y) + ((size_t)b * p.D + d0) * L;
        const bool sw = p.swap_out && L > 1;
        if (p.mode == 0 && len == L) {
            if (sw && lane < nrows) {  // exchange the two end tokens of this lane's row in LDS
                const IO a = ds[lane * L];
                ds[lane * L] = ds[lane * L + L - 1];
                ds[lane * L + L - 1] = a;
            }
            wave_lds_sync();
            const int n = nrows * L;
            const int units = n * (int)sizeof(IO) / 16;
            for (int u = lane; u < units; u += kWave)
                reinterpret_cast<uint4*>(yg)[u] = reinterpret_cast<const uint4*>(ds)[u];
            const int done = units * 16 / (int)sizeof(IO);
            if (lane < n - done) yg[done + lane] = ds[done + lane];
            wave_lds_sync();
            return;
        }
        // positions written here; the ends go out last when swapping
        const int lo = (sw && t0 == 0) ? 1 : t0;
        const int hi = (sw && t0 + len == L) ? L - 1 : t0 + len;
        if (sw && t0 == 0 && lane < nrows) y0 = ds[lane * drs + 0 - doff];
        if (p.mode == 1) {
            // whole 4-byte words inside [lo, hi), single elements at the edges
            constexpr int ew = 4 / (int)sizeof(IO);
            const int ta = (lo + ew - 1) / ew * ew;
            const int tb = max(ta, hi / ew * ew);
            if (tb > ta) {
                const int nw = (tb - ta) / ew;
                const int total = nrows * nw;
                const float inv = 1.0f / (float)nw;
                for (int e = lane; e < total; e += kWave) {
                    const int r = div_small(e, inv);
                    const int w = e - r * nw;
                    const uint32_t v = *reinterpret_cast<const uint32_t*>(&ds[r * drs + ta - doff + w * ew]);
                    *reinterpret_cast<uint32_t*>(&yg[(size_t)r * L + ta + w * ew]) = v;
                }
            }
            if (lane < nrows) {
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
            yg[(size_t)lane * L + L - 1] = y0;
        }
        wave_lds_sync();
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

    // One position: conv tap in, Delta, N-state update, readout.
    template <bool OUT, bool SP, bool SILU, bool FIRST>
    __device__ __forceinline__ float core(float xnew, float dl, float (&h)[NS], float (&win)[KW], float& sd2,
                                          const float4 (&bq)[NS / 4], const float4 (&cq)[NS / 4]) {
        // Opaque to the compiler: pins this position's work after the previous
        // position's, so the exp work of later positions is not hoisted (it
        // would cost ~N registers per position and spill).
        asm volatile("" : "+v"(xnew), "+v"(dl));
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

    // Scan positions [t0, t0 + len) of the staged sample.  OUT: write y into ds.
    // AGG (OUT = false): accumulate the sum of Delta*log2e in sd2, no output.
    template <bool OUT, bool SP, bool SILU>
    __device__ void chunk_t(int t0, int len, float (&h)[NS], float& sd2) {
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
        const int lag = CONV ? KW - 1 - P : 0;  // newest conv tap is x[t + lag]
        int t = t0;
        const int tend = t0 + len;
        // inputs of one position, read from LDS one position ahead of use
        float xc, dc;
        float4 bq[NS / 4], cq[NS / 4];
        auto fetch = [&](int tt, float& xv, float& dv, float4 (&bb)[NS / 4], float4 (&cc)[NS / 4]) {
            xv = xat(xr, tt + lag, L, pad);
            dv = to_f32(dr[tt]);
            load_bc(br, cr, tt, bb, cc);
        };
        if (t == 0) {
            fetch(0, xc, dc, bq, cq);
            const float y0 = core<OUT, SP, SILU, true>(xc, dc + dbias, h, win, sd2, bq, cq);
            if constexpr (OUT) dr[0] = from_f32<IO>(y0);
            ++t;
        }
        // two register sets used alternately: position t computes from one set
        // while position t+1's reads land in the other, so nothing is copied
        float x1, d1;
        float4 bq1[NS / 4], cq1[NS / 4];
        if (t < tend) fetch(t, xc, dc, bq, cq);
        for (; t + 2 <= tend; t += 2) {
            fetch(t + 1, x1, d1, bq1, cq1);
            const float ya = core<OUT, SP, SILU, false>(xc, dc + dbias, h, win, sd2, bq, cq);
            if constexpr (OUT) dr[t] = from_f32<IO>(ya);
            fetch(min(t + 2, tend - 1), xc, dc, bq, cq);  // the last fetch repeats a valid position
            const float yb = core<OUT, SP, SILU, false>(x1, d1 + dbias, h, win, sd2, bq1, cq1);
            if constexpr (OUT) dr[t + 1] = from_f32<IO>(yb);
        }
        if (t < tend) {
            const float ya = core<OUT, SP, SILU, false>(xc, dc + dbias, h, win, sd2, bq, cq);
            if constexpr (OUT) dr[t] = from_f32<IO>(ya);
        }
    }

    template <bool OUT>
    __device__ void chunk(int t0, int len, float (&h)[NS], float& sd2) {
        if (p.softplus) {
            if (CONV && p.act == 1) chunk_t<OUT, true, true>(t0, len, h, sd2);
            else chunk_t<OUT, true, false>(t0, len, h, sd2);
        } else {
            if (CONV && p.act == 1) chunk_t<OUT, false, true>(t0, len, h, sd2);
            else chunk_t<OUT, false, false>(t0, len, h, sd2);
        }
    }

    // Run folded positions [sa, sb) of row b1, state carried in h.
    template <bool OUT>
    __device__ void run(int sa, int sb, float (&h)[NS], float& sd2) {
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
            chunk<OUT>(t0, len, h, sd2);
            wave_lds_sync();
            if (OUT) store(b, t0, len);
            s += len;
        }
    }
};

template <typename IO, int NS, int KW, bool CONV>
__global__ __launch_bounds__(kWave * kMaxWaves) __attribute__((amdgpu_waves_per_eu(NS <= 8 ? 3 : 2)))
void scan_kernel(ScanParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & (kWave - 1);
    // the wave index is the same for all 64 lanes; saying so keeps every
    // position/piece index derived from it in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
    // giving each XCD a contiguous run of (row, tile) items keeps the B/C of a
    // folded row in one XCD's L2.
    const int G = p.tgroups * p.B1;
    int g = blockIdx.x;
    if ((G & 7) == 0) g = (g & 7) * (G >> 3) + (g >> 3);
    const int b1 = g / p.tgroups;
    const int tg = g - b1 * p.tgroups;
    const int wp = wave / p.cw;         // piece of the folded row
    const int wc = wave - wp * p.cw;    // channel tile within the group
    char* grp = smem + (size_t)wp * p.group_bytes;
    ScanWave<IO, NS, KW, CONV> w(p, lane, (tg * p.cw + wc) * kWave, b1,
                                 grp + p.bc_bytes + (size_t)wc * (p.xs_bytes + p.ds_bytes),
                                 reinterpret_cast<float*>(grp), wc);

    const int S = p.B2 * p.L;
    const int p0 = min(wp * p.piece, S);
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
    hipLaunchKernelGGL(kern, dim3((unsigned)(p.tgroups * p.B1)), dim3((unsigned)(kWave * p.cw * p.waves)),
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

// smallest row stride >= elems whose length in 4-byte words is odd (and whole),
// so that the 64 lanes reading one column hit distinct banks
int odd_word_stride(int elems, int elem_bytes) {
    int s = elems;
    while ((s * elem_bytes) % 4 != 0 || ((s * elem_bytes) / 4) % 2 == 0) ++s;
    return s;
}

}  // namespace

bool plan_scan(ScanParams& p, int io_bytes, int waves_hint, int ch_hint) {
    const int L = p.L, S = p.B2 * p.L;
    if (p.xrow <= 0) p.xrow = p.pad_in ? L - 2 : L;
    const int XL = p.xrow;
    const bool fused = p.pad_in || p.swap_out;  // these keep each sample inside one wave
    p.ns = p.N <= 4 ? 4 : (p.N <= 8 ? 8 : 16);
    const int kw = p.conv_w ? (p.K <= 4 ? 4 : 8) : 0;
    p.tiles = (p.D + kWave - 1) / kWave;
    p.bc_wide = ((long long)p.N * L * io_bytes) % 16 == 0 ? 1 : 0;
    constexpr int kLdsCap = 160 * 1024;
    constexpr int kLdsUnit = 1280;  // LDS is handed out to workgroups in units of this size
    const int agg_fixed = kMaxWaves * (int)sizeof(int);
    const int ew = 4 / io_bytes;
    // per-wave x / delta stages
    auto xd_bytes = [&](int ch, int mode, int& xsb, int& dsb, int& xrs, int& drs) {
        if (mode == 0) {
            xrs = XL;
            drs = L;
            xsb = kWave * XL * io_bytes;
            dsb = kWave * L * io_bytes;
        } else {
            // mode 1 rows hold the chunk plus word alignment at both ends
            const int extra = mode == 1 ? 2 * (ew - 1) : 0;
            xrs = odd_word_stride(ch + (kw ? kw - 1 : 0) + extra, io_bytes);
            drs = odd_word_stride(ch + extra, io_bytes);
            xsb = kWave * xrs * io_bytes;
            dsb = kWave * drs * io_bytes;
        }
        xsb = (xsb + 15) & ~15;
        dsb = (dsb + 15) & ~15;
        return xsb + dsb;
    };
    auto bc_bytes = [&](int ch) { return 2 * ch * p.ns * (int)sizeof(float); };
    int xsb = 0, dsb = 0, xrs = 0, drs = 0;
    // mode 0 (whole rows) when the [64 x L] slabs are 16-byte aligned and small
    int mode = 2;
    int ch = ch_hint > 0 ? ch_hint : 32;
    if (L <= 256 && ((long long)p.D * L * io_bytes) % 16 == 0 && ((long long)p.D * XL * io_bytes) % 16 == 0 &&
        ch_hint <= 0 && xd_bytes(L, 0, xsb, dsb, xrs, drs) + bc_bytes(L) <= 20 * 1024) {
        mode = 0;
        ch = L;
    }
    if (mode != 0) {
        mode = ((long long)L * io_bytes) % 4 == 0 && ((long long)XL * io_bytes) % 4 == 0 ? 1 : 2;
        if (ch > L) ch = L;
    }
    // pieces per folded row
    int W;
    if (waves_hint > 0 && !fused) {
        W = waves_hint;
    } else if (S <= 256 || p.B2 > 1 || fused) {
        // short rows: one or more whole samples per wave, cuts on sample starts
        W = 1;
        for (int c = 1; c <= kMaxWaves; ++c)
            if (p.B2 % c == 0) W = c;
    } else {
        // long rows: enough waves to fill 256 CUs x 4 SIMDs a few times over
        const long long items = (long long)p.tiles * p.B1;
        long long want = (2048 + items - 1) / items;
        W = (int)(want < 1 ? 1 : (want > kMaxWaves ? kMaxWaves : want));
    }
    if (W > kMaxWaves) W = kMaxWaves;
    if (W > S) W = S;
    const int piece = (S + W - 1) / W;
    int carry = 0;
    for (int i = 1; i < W; ++i) {
        const int s0 = i * piece;
        if (s0 < S && s0 % L) carry = 1;
    }
    auto lds_total = [&](int cw, int chv, int& grp) {
        grp = bc_bytes(chv) + cw * xd_bytes(chv, mode, xsb, dsb, xrs, drs);
        const int agg = carry ? agg_fixed + W * kWave * (int)sizeof(float) * (1 + p.ns) : 0;
        return W * grp + agg;
    };
    // shrink the chunk until one workgroup of cw = 1 fits
    int grp = 0;
    while (lds_total(1, ch, grp) > kLdsCap) {
        if (mode != 0 && ch > 8) ch /= 2;
        else return false;
    }
    // channel tiles per workgroup sharing one B/C stage: the choice that needs
    // the fewest rounds of resident waves (all pieces must then stage the same
    // chunk sequence, so only without carries and with equal pieces)
    const int vgpr_waves_per_cu = p.ns <= 8 ? 12 : 8;
    int best_cw = 1;
    long long best_rounds = -1;
    for (int cw = 1; cw <= 4; cw *= 2) {
        if (cw > 1 && (carry || S % W || cw * W > kMaxWaves || p.tiles < cw)) break;
        const int tot = lds_total(cw, ch, grp);
        if (tot > kLdsCap) break;
        const int alloc = (tot + kLdsUnit - 1) / kLdsUnit * kLdsUnit;
        int per_cu = kLdsCap / alloc * cw * W;
        const int lim = vgpr_waves_per_cu / (cw * W) * (cw * W);
        if (per_cu > lim) per_cu = lim;
        if (per_cu < cw * W) per_cu = cw * W;
        const long long tgroups = (p.tiles + cw - 1) / cw;
        const long long waves = tgroups * p.B1 * cw * W;
        const long long slots = 256LL * per_cu;
        const long long rounds = (waves + slots - 1) / slots;
        if (best_rounds < 0 || rounds < best_rounds) {
            best_rounds = rounds;
            best_cw = cw;
        }
    }
    p.cw = best_cw;
    p.tgroups = (p.tiles + p.cw - 1) / p.cw;
    p.waves = W;
    p.piece = piece;
    p.need_carry = carry;
    p.ch = ch;
    p.mode = mode;
    p.lds_bytes = lds_total(p.cw, ch, grp);
    p.group_bytes = grp;
    p.bc_bytes = bc_bytes(ch);
    xd_bytes(ch, mode, xsb, dsb, xrs, drs);
    p.xrs = xrs;
    p.drs = drs;
    p.xs_bytes = xsb;
    p.ds_bytes = dsb;
    return true;
}

hipError_t launch_scan(const ScanParams& p, int io_dtype, hipStream_t stream) {
    if (io_dtype == 0) return launch_io<float>(p, stream);
    return launch_io<__bf16>(p, stream);
}

}  // namespace sfm
