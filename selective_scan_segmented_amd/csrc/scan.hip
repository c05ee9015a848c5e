// scan.hip -- launch planning for the folded, segmented selective scan
// (kernel: scan_kernel.h; instantiations: scan_<io>_n<N>.hip).
#include "scan_kernel.h"

#include <algorithm>

namespace sfm {

using scan_detail::kMaxWaves;

namespace {

// smallest row stride >= elems whose length in 4-byte words is odd (and whole),
// so that the 64 lanes reading one column hit distinct banks
int odd_word_stride(int elems, int elem_bytes) {
    int s = elems;
    while ((s * elem_bytes) % 4 != 0 || ((s * elem_bytes) / 4) % 2 == 0) ++s;
    return s;
}

// smallest odd number of 4-byte words >= w (rows that far apart in LDS put the
// 64 lanes reading one column into distinct banks)
int odd_words(int w) { return w | 1; }

// Lane-split plan (scan_split.h), G lanes per channel.  G is the smallest
// group that gives every SIMD of the device about four waves (a lone wave
// issues a VALU instruction at most every five to six cycles, a SIMD with
// four or more every four), else the largest; split_hint > 0 forces G.
// Staging: whole sample rows (x, delta and raw B/C by 16-byte transfers), or,
// when that leaves fewer waves resident per CU than the grid could use,
// chunked (x whole rows; delta/y and raw B/C sq positions at a time by 4-byte
// transfers).  chunk_hint: < 0 automatic, 0 whole rows only, > 0 forces sq.
// Returns false when the shape does not fit (alignment, LDS), leaving the
// classic kernel to plan it.
bool plan_split(ScanParams& p, int io_bytes, int split_hint, int stagger_hint, int chunk_hint, int cus) {
    const int L = p.L, XL = p.xrow, N = p.N, D = p.D;
    const int ns = p.N <= 4 ? 4 : (p.N <= 8 ? 8 : 16);
    const int ew = 4 / io_bytes;
    if (((long long)D * XL * io_bytes) % 16) return false;  // x whole rows by 16-byte transfers
    const bool whole_ok = ((long long)D * L * io_bytes) % 16 == 0 && ((long long)N * L * io_bytes) % 16 == 0 &&
                          L <= 1024 && chunk_hint <= 0;
    const bool chunk_ok = ((long long)L * io_bytes) % 4 == 0 && XL <= 2048 && chunk_hint != 0;
    if (!whole_ok && !chunk_ok) return false;
    int cands[2] = {2, 4};
    int nc = ns == 4 ? 1 : 2;
    if (split_hint > 0) {
        if (split_hint != 2 && split_hint != 4) return false;
        if (ns == 4 && split_hint != 2) return false;
        cands[0] = split_hint;
        nc = 1;
    }
    constexpr int kLdsCap = 160 * 1024;
    constexpr int kLdsUnit = 1280;
    constexpr int kRegWavesPerCu = 20;  // five waves per SIMD by registers
    auto units = [&](int b) { return (b + kLdsUnit - 1) / kLdsUnit * kLdsUnit; };
    int G = 0;
    for (int ci = 0; ci < nc; ++ci) {
        const int g = cands[ci];
        const int cpw = kWave / g;
        if (((long long)cpw * XL * io_bytes) % 16) continue;
        if (whole_ok && !chunk_ok && ((long long)cpw * L * io_bytes) % 16) continue;
        G = g;
        // about four waves per SIMD, a wave of a folded row counting once per
        // sample it walks (stage-4 at B2 = 2: two lanes 32.8 us, four 34.0 us;
        // stage-3 at B2 = 2: four lanes 69.6 us, two 104.6 us)
        const long long waves = (long long)p.B1 * ((D + cpw - 1) / cpw);
        if (waves * p.B2 >= 4LL * 4 * cus) break;
    }
    if (!G) return false;
    const int cpw = kWave / G;
    const int tiles = (D + cpw - 1) / cpw;
    const int wpg = tiles >= 4 ? 4 : (tiles >= 2 ? 2 : 1);
    const int gch = wpg * cpw;
    const int mean_bytes = (gch * (int)sizeof(float) + 15) & ~15;
    const int xsb = (cpw * XL * io_bytes + 15) & ~15;
    const long long grid = (long long)((tiles + wpg - 1) / wpg) * p.B1;
    auto resident = [&](int lds) { return std::min(kRegWavesPerCu, kLdsCap / units(lds) * wpg); };
    // whole rows
    int w_lds = 0, w_res = 0;
    const int bc_w = L * 2 * ns * (int)sizeof(float);
    const int braw_w = (2 * N * L * io_bytes + 15) & ~15;
    const int dsb_w = (cpw * L * io_bytes + 15) & ~15;
    if (whole_ok && ((long long)cpw * L * io_bytes) % 16 == 0) {
        w_lds = bc_w + braw_w + mean_bytes + wpg * (xsb + dsb_w);
        if (w_lds <= kLdsCap) w_res = resident(w_lds);
    }
    // chunked: the largest chunk with the most resident waves
    int c_q = 0, c_lds = 0, c_res = 0, c_dpw = 0, c_di = 0, c_bi = 0;
    if (chunk_ok) {
        const int step = std::max(G, ew);
        for (int q : {64, 48, 32, 24, 16}) {
            if (chunk_hint > 0 && q != chunk_hint) continue;
            if (q % step || q < 2 * step) continue;
            const int qq = std::min(q, (L + step - 1) / step * step);
            const int pw = odd_words((qq + ew - 1) / ew);
            const int di = (cpw * pw + kWave - 1) / kWave;  // transfers of one delta tile
            const int bi = (N * pw + kWave - 1) / kWave;    // of one raw B or C tile
            const int lds = qq * 2 * ns * (int)sizeof(float) + 2 * bi * 256 + mean_bytes + wpg * (xsb + di * 256);
            if (lds > kLdsCap) continue;
            const int r = resident(lds);
            if (r > c_res) {
                c_q = qq;
                c_lds = lds;
                c_res = r;
                c_dpw = pw;
                c_di = di;
                c_bi = bi;
            }
            if (qq >= L) break;
        }
        if (chunk_hint > 0 && !c_q) return false;
    }
    // Whole rows whenever they keep two or more waves per SIMD resident: the
    // chunked staging's per-chunk waits, barriers and B/C widening cost more
    // than its extra residency gains (measured at stage-3 shapes: whole rows,
    // 2 waves per SIMD, 76 us; 24-position chunks, 5 per SIMD, 81-83 us).
    bool chunk;
    if (chunk_hint > 0) chunk = true;
    else if (w_res >= 8 || (w_res > 0 && w_res >= c_res)) chunk = false;
    else chunk = c_res > 0;
    const int res = chunk ? c_res : w_res;
    if (res == 0) return false;
    // fewer than two resident waves per SIMD leaves the classic kernel ahead
    if (split_hint <= 0 && res < 8) return false;
    p.split = G;
    p.wpg = wpg;
    p.stiles = (tiles + wpg - 1) / wpg;
    p.ns = ns;
    p.tiles = tiles;
    p.mode = 0;
    p.ch = L;
    p.waves = 1;
    p.piece = p.B2 * L;
    p.need_carry = 0;
    p.cw = wpg;
    p.tgroups = p.stiles;
    p.xs_bytes = xsb;
    if (chunk) {
        p.sq = c_q;
        p.dpw = c_dpw;
        p.bpw = c_dpw;
        p.dtile_insts = c_di;
        p.btile_insts = c_bi;
        p.bc_off = 0;
        p.braw_off = c_q * 2 * ns * (int)sizeof(float);
        p.mean_off = p.braw_off + 2 * c_bi * 256;
        p.slab_off = p.mean_off + mean_bytes;
        p.ds_bytes = c_di * 256;
        p.lds_bytes = c_lds;
    } else {
        p.sq = 0;
        p.bc_off = 0;
        p.braw_off = bc_w;
        p.mean_off = bc_w + braw_w;
        p.slab_off = bc_w + braw_w + mean_bytes;
        p.ds_bytes = dsb_w;
        p.lds_bytes = w_lds;
    }
    p.slab_bytes = p.xs_bytes + p.ds_bytes;
    // Staggered start (whole rows): dispatch round r (one workgroup per CU)
    // of the rounds resident at launch delays its loads by r times the time
    // HBM needs for one round's inputs at about 6.5 TB/s (65000 bytes per 10 ns
    // tick); workgroups that start later, when a slot frees, take no delay (the
    // launcher counts the resident rounds).  Stage-3 rows (two resident rounds
    // of 2.5): 56.7 -> 56.2 us.
    p.stagger_period = 0;
    p.stagger_ticks = 0;
    if (!chunk && stagger_hint != 0 && grid > cus) {
        const long long wg_bytes = (long long)wpg * cpw * (XL + L) * io_bytes + 2LL * N * L * io_bytes;
        long long ticks = stagger_hint > 0 ? stagger_hint : (long long)cus * wg_bytes / 65000;
        if (ticks > 500) ticks = 500;
        if (ticks > 0) {
            p.stagger_period = cus;
            p.stagger_ticks = (int)ticks;
        }
    }
    return true;
}

// Streaming lane-split plan (split_stream_kernel): one state per lane, 16
// lanes per channel, four channels per wave, for 9 to 16 states.  Every
// (sample, channel) row stays on one wave -- no carries -- and nothing is
// staged whole: x, delta/y and raw B/C move sq positions at a time,
// double-buffered, so the LDS a workgroup needs does not grow with L.  Each
// chunk costs a fixed ~2 us (two workgroup barriers, the wait, widening,
// stores: measured on the long rows as the slope of step time over chunk
// count), so the chunk is the longest that keeps every workgroup resident in
// one round and the kernel's precomputed-transfer path (at most 8 transfers
// per tile and wave); wpg = 4 or 8 waves share one B/C stage.  chunk_hint > 0
// forces a chunk length (a multiple of 16 up to 256); SFM_SCAN_SPLIT_WPG
// (diagnostics) forces the waves per workgroup.  Needs rows of whole 4-byte
// words.
bool plan_stream(ScanParams& p, int io_bytes, int chunk_hint, int cus) {
    if (p.N <= 8) return false;
    const int L = p.L, XL = p.xrow, N = p.N, D = p.D;
    const int ew = 4 / io_bytes;
    if (((long long)L * io_bytes) % 4 || ((long long)XL * io_bytes) % 4) return false;
    if (chunk_hint > 0 && (chunk_hint % 16 || chunk_hint > 256)) return false;
    constexpr int G = 16, cpw = kWave / G;
    constexpr int kLdsCap = 160 * 1024, kLdsUnit = 1280, kWavesPerCu = 8;  // two waves per SIMD by registers
    constexpr int kFast = 8;                                                // see split_stream_kernel
    const int kw = p.conv_w ? (p.K <= 4 ? 4 : 8) : 4;  // compiled conv window
    const int tiles = (D + cpw - 1) / cpw;
    int wpg_hint = 0;
    if (const char* e = std::getenv("SFM_SCAN_SPLIT_WPG")) wpg_hint = std::atoi(e);
    struct Cand { int q, wpg, lds, xi, di, bi, xpw, dpw; };
    auto layout = [&](int q, int wpg, Cand& c) {
        c.q = q;
        c.wpg = wpg;
        c.xpw = odd_words((q + kw - 1) / ew + 2);  // the chunk's taps plus word alignment
        c.dpw = odd_words((q + ew - 1) / ew);
        c.xi = (cpw * c.xpw + kWave - 1) / kWave;
        c.di = (cpw * c.dpw + kWave - 1) / kWave;
        c.bi = (N * c.dpw + kWave - 1) / kWave;
        c.lds = q * G * 2 * (int)sizeof(float) + 2 * 2 * c.bi * 256 + wpg * kWave * (int)sizeof(double) +
                wpg * 2 * (c.xi + c.di) * 256;
    };
    Cand best{};
    long long best_score = -1;
    const int qmax = (L + G - 1) / G * G;
    for (int wpg : {4, 8}) {
        if (wpg_hint > 0 && wpg != wpg_hint) continue;
        const int w = tiles >= wpg ? wpg : (tiles >= 4 ? 4 : (tiles >= 2 ? 2 : 1));
        const long long grid = (long long)((tiles + w - 1) / w) * p.B1;
        for (int q = 256; q >= G; q -= G) {
            if (chunk_hint > 0 && q != chunk_hint) continue;
            Cand c;
            layout(std::min(q, qmax), w, c);
            if (c.lds > kLdsCap) continue;
            const int per_cu = std::min(kLdsCap / ((c.lds + kLdsUnit - 1) / kLdsUnit * kLdsUnit), kWavesPerCu / w);
            if (per_cu < 1) continue;
            const long long rounds = (grid + (long long)cus * per_cu - 1) / ((long long)cus * per_cu);
            const bool fast = c.xi <= kFast && c.di <= kFast && (c.bi + w - 1) / w <= kFast;
            // fewest rounds, then the precomputed path, then the longest chunk, then fewer waves per group
            const long long score = (1000 - std::min(rounds, 999LL)) * 1000000LL + (fast ? 100000 : 0) + c.q * 10 +
                                    (w == 4 ? 1 : 0);
            if (score > best_score) {
                best_score = score;
                best = c;
            }
        }
    }
    if (best_score < 0) return false;
    p.split = G;
    p.wpg = best.wpg;
    p.stiles = (tiles + best.wpg - 1) / best.wpg;
    p.ns = 16;
    p.tiles = tiles;
    p.mode = 0;
    p.ch = best.q;
    p.waves = 1;
    p.piece = p.B2 * L;
    p.need_carry = 0;
    p.cw = best.wpg;
    p.tgroups = p.stiles;
    p.sq = best.q;
    p.xpw = best.xpw;
    p.dpw = best.dpw;
    p.bpw = best.dpw;
    p.xtile_insts = best.xi;
    p.dtile_insts = best.di;
    p.btile_insts = best.bi;
    p.bc_off = 0;
    p.braw_off = best.q * G * 2 * (int)sizeof(float);
    p.mean_off = p.braw_off + 2 * 2 * best.bi * 256;
    p.slab_off = p.mean_off + best.wpg * kWave * (int)sizeof(double);
    p.slab_bytes = 2 * (best.xi + best.di) * 256;
    p.xs_bytes = best.xi * 256;
    p.ds_bytes = best.di * 256;
    p.lds_bytes = best.lds;
    p.stagger_period = 0;
    p.stagger_ticks = 0;
    return true;
}

}  // namespace


// Compute units of the current device (256 when no device can be queried).
int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    return cus;
}

bool plan_scan(ScanParams& p, int io_bytes, int waves_hint, int ch_hint, int stagger_hint, int stages_hint,
               int split_hint, int split_chunk_hint) {
    const int L = p.L, S = p.B2 * p.L;
    if (p.xrow <= 0) p.xrow = p.pad_in ? L - 2 : L;
    p.split = 0;
    // The lane-split kernel when asked for; when one wave per (sample,
    // 64-channel tile) would give the SIMDs fewer than two waves each; and, on
    // rows of at most two samples, up to four each.  Measured on MI355X
    // (same-process A/B): stage-3 shapes, 1.25 one-lane waves per SIMD: 67-71
    // vs 101-102 us; stage-4, 2.5 per SIMD, where the one-lane kernel leaves
    // half the SIMDs with three waves: 29.8-32.7 vs 31.3-33.5 us with two lanes
    // per channel (five balanced waves per SIMD); the base model's stage-3, 4
    // per SIMD: 312 vs 355 us.  Folded rows take their samples in turn on one
    // lane-split wave but as separate pieces on the one-lane kernel: at B2 = 2
    // the lane-split kernel wins (stage-4 32.8 vs 38.5 us, base stage-3 280.8
    // vs 313.6 us), at B2 = 4 it loses (stage-4 40.9 vs 34.6 us).
    const int cus = device_cus();
    const long long lane_waves = (long long)p.B1 * p.B2 * ((p.D + kWave - 1) / kWave);
    const bool want_split = split_hint > 0 ||
                            (split_hint < 0 && (lane_waves < 2LL * 4 * cus || (lane_waves <= 4LL * 4 * cus && p.B2 <= 2)));
    if (want_split && waves_hint <= 0 && ch_hint <= 0) {
        // G = 2 or 4 first (fewer instructions per token); the streaming
        // kernel where those cannot stage the rows (long rows) or when asked for
        if (split_hint != 16 && plan_split(p, io_bytes, split_hint, stagger_hint, split_chunk_hint, cus)) return true;
        if ((split_hint < 0 || split_hint == 16) && plan_stream(p, io_bytes, split_chunk_hint, cus)) return true;
    }
    const int XL = p.xrow;
    // The fused pad/swap keep each sample inside one wave, except with tile
    // staging (even row lengths), whose pieces take the row mean and write the
    // swapped ends themselves
    const bool tile_rows = ((long long)L * io_bytes) % 4 == 0 && ((long long)XL * io_bytes) % 4 == 0;
    const bool fused = (p.pad_in || p.swap_out) && !tile_rows;
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
        // mode 1 transfers go in groups of four 256-byte instructions
        const int unit = mode == 1 ? 1024 : 16;
        xsb = (xsb + unit - 1) / unit * unit;
        dsb = (dsb + unit - 1) / unit * unit;
        return xsb + dsb;
    };
    // B/C stage: float32 [ch][ns] for B and C, plus (mode 0, aligned blocks) the
    // raw [2][N][L] io area they are transferred into
    const int bcr_bytes = ((2 * p.N * L * io_bytes) + 15) & ~15;
    auto bc_bytes = [&](int ch, int m) {
        return 2 * ch * p.ns * (int)sizeof(float) + (m == 0 && p.bc_wide ? bcr_bytes : 0);
    };
    // mode 1 raw B/C rows of one stage: a chunk plus word alignment at both ends
    auto rb_rs_of = [&](int ch) { return (ch + 2 * (ew - 1) + ew - 1) / ew * ew; };
    auto rb_bytes_of = [&](int ch) { return 2 * ((p.N * rb_rs_of(ch) * io_bytes + 1023) / 1024 * 1024); };
    int xsb = 0, dsb = 0, xrs = 0, drs = 0;
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
    // mode 0 (whole rows) when the [64 x L] slabs are 16-byte aligned and
    // small and no piece starts inside a sample (its kernels hold no carry path)
    int mode = 2;
    int ch = ch_hint > 0 ? ch_hint : 32;
    const int part = p.D % kWave;  // rows of a partial last channel tile
    if (!carry && L <= 256 && ((long long)p.D * L * io_bytes) % 16 == 0 &&
        ((long long)p.D * XL * io_bytes) % 16 == 0 && (part * XL * io_bytes) % 16 == 0 &&
        (part * L * io_bytes) % 16 == 0 && ch_hint <= 0 &&
        xd_bytes(L, 0, xsb, dsb, xrs, drs) + bc_bytes(L, 0) <= 20 * 1024) {
        mode = 0;
        ch = L;
    }
    if (mode != 0) {
        mode = ((long long)L * io_bytes) % 4 == 0 && ((long long)XL * io_bytes) % 4 == 0 ? 1 : 2;
        if (ch > L) ch = L;
    }
    // mode 1: pieces that start on sample boundaries need no exchange, so each
    // is a workgroup of its own (one wave), which packs LDS per wave, not per row
    const int wsplit = mode == 1 && !carry ? 1 : 0;
    const int per_wg = wsplit ? 1 : W;
    int stages = stages_hint == 2 ? 2 : 1;
    auto lds_total = [&](int cw, int chv, int& grp) {
        if (mode == 1)  // one wave per group: stages of x, delta and raw B/C, one float32 B/C area
            grp = stages * (xd_bytes(chv, mode, xsb, dsb, xrs, drs) + rb_bytes_of(chv)) + bc_bytes(chv, mode);
        else
            grp = bc_bytes(chv, mode) + cw * xd_bytes(chv, mode, xsb, dsb, xrs, drs);
        const int agg = carry ? agg_fixed + W * kWave * (int)sizeof(float) * (1 + p.ns) : 0;
        return per_wg * grp + agg;
    };
    const int vgpr_waves_per_cu = p.ns <= 8 ? 12 : 8;
    int grp = 0;
    if (mode == 1 && ch_hint <= 0) {
        // Chunk length: every chunk costs a fixed set-up (waits, conv window,
        // loop entry and exit), so long chunks come first; the first that lets
        // as many waves share a CU as the grid (or the register file) can use
        // wins, else the one with the most waves per CU.  One LDS stage per
        // wave unless two are asked for: measured on MI355X, the waves sharing
        // a SIMD hide each other's transfers, and a second stage (which halves
        // the chunk that fits) was slower on every workload but the longest
        // rows (stage-3: 102.5 vs 110.8 us; base stage-3: 319 vs 370 us).
        const long long total_waves = (long long)p.tiles * p.B1 * W;
        const long long need = (total_waves + cus - 1) / cus;
        const int target = (int)(need < vgpr_waves_per_cu ? need : vgpr_waves_per_cu);
        const int cap_ch = (L + ew - 1) / ew * ew;
        static const int cand[][2] = {{1, 64}, {1, 32}, {1, 16}, {1, 8}, {2, 64}, {2, 32}, {2, 16}, {2, 8}};
        int best = -1, best_st = 2, best_per_cu = -1;
        for (const auto& c : cand) {
            if (stages_hint == 1 || stages_hint == 2) {
                if (c[0] != stages_hint) continue;
            }
            stages = c[0];
            const int cc = c[1] < cap_ch ? c[1] : cap_ch;
            const int tot = lds_total(1, cc, grp);
            if (tot > kLdsCap) continue;
            const int per_cu = kLdsCap / ((tot + kLdsUnit - 1) / kLdsUnit * kLdsUnit) * per_wg;
            if (per_cu >= target) {
                best = cc;
                best_st = c[0];
                break;
            }
            if (per_cu > best_per_cu) {
                best_per_cu = per_cu;
                best = cc;
                best_st = c[0];
            }
        }
        if (best < 0) return false;
        ch = best;
        stages = best_st;
    }
    // shrink the chunk until one workgroup of cw = 1 fits
    while (lds_total(1, ch, grp) > kLdsCap) {
        if (mode != 0 && ch > 8) ch /= 2;
        else return false;
    }
    // channel tiles per workgroup sharing one B/C stage: the choice that needs
    // the fewest rounds of resident waves (all pieces must then stage the same
    // chunk sequence, so only without carries and with equal pieces)
    int best_cw = 1, best_per_cu = 1;
    long long best_rounds = -1;
    for (int cw = 1; cw <= 4; cw *= 2) {
        if (cw > 1 && (mode == 1 || carry || S % W || cw * W > kMaxWaves || p.tiles < cw)) break;
        const int tot = lds_total(cw, ch, grp);
        if (tot > kLdsCap) break;
        const int alloc = (tot + kLdsUnit - 1) / kLdsUnit * kLdsUnit;
        int per_cu = kLdsCap / alloc * cw * W;
        const int lim = vgpr_waves_per_cu / (cw * W) * (cw * W);
        if (per_cu > lim) per_cu = lim;
        if (per_cu < cw * W) per_cu = cw * W;
        const long long tgroups = (p.tiles + cw - 1) / cw;
        const long long waves = tgroups * p.B1 * cw * W;
        const long long slots = (long long)cus * per_cu;
        const long long rounds = (waves + slots - 1) / slots;
        if (best_rounds < 0 || rounds < best_rounds) {
            best_rounds = rounds;
            best_cw = cw;
            best_per_cu = per_cu / (cw * W);
        }
    }
    p.cw = best_cw;
    p.stages = mode == 1 ? stages : 1;
    p.wsplit = wsplit;
    p.tgroups = (p.tiles + p.cw - 1) / p.cw;
    p.waves = W;
    p.piece = piece;
    p.need_carry = carry;
    p.ch = ch;
    p.mode = mode;
    p.lds_bytes = lds_total(p.cw, ch, grp);
    p.group_bytes = grp;
    p.bc_bytes = mode == 1 ? 0 : bc_bytes(ch, mode);  // mode 1: inside each wave's own area
    p.bc_dma = mode == 0 && p.bc_wide ? 1 : 0;
    p.bcr_off = 2 * ch * p.ns * (int)sizeof(float);
    xd_bytes(ch, mode, xsb, dsb, xrs, drs);
    p.xrs = xrs;
    p.drs = drs;
    p.xs_bytes = xsb;
    p.ds_bytes = dsb;
    p.rb_rs = mode == 1 ? rb_rs_of(ch) : 0;
    p.rb_bytes = mode == 1 ? rb_bytes_of(ch) : 0;
    // Staggered start.  Whole-row staging loads everything up front; when the
    // whole grid is resident at once, every wave would otherwise wait for the
    // entire input to arrive before its first step.  Delaying dispatch round r
    // by about the time HBM needs for one round's inputs (measured best near
    // 6.5 TB/s worth of a round on MI355X) lets early rounds compute while
    // later rounds load.
    p.stagger_period = 0;
    p.stagger_ticks = 0;
    const long long grid = (long long)p.tgroups * p.B1;
    if (mode == 0 && !carry && grid > cus && grid <= (long long)cus * best_per_cu && stagger_hint != 0) {
        const long long wg_bytes = (long long)p.cw * kWave * (XL + L) * io_bytes + 2LL * p.N * L * io_bytes;
        long long ticks = stagger_hint > 0 ? stagger_hint : (long long)cus * wg_bytes / 65000;
        if (ticks > 500) ticks = 500;
        if (ticks > 0) {
            p.stagger_period = cus;
            p.stagger_ticks = (int)ticks;
        }
    }
    return true;
}

hipError_t launch_scan(const ScanParams& p, int io_dtype, hipStream_t stream) {
    if (p.split) {
        if (io_dtype == 0) {
            if (p.ns == 4) return launch_split_f32_n4(p, stream);
            if (p.ns == 8) return launch_split_f32_n8(p, stream);
            return launch_split_f32_n16(p, stream);
        }
        if (p.ns == 4) return launch_split_bf16_n4(p, stream);
        if (p.ns == 8) return launch_split_bf16_n8(p, stream);
        return launch_split_bf16_n16(p, stream);
    }
    if (io_dtype == 0) {
        if (p.ns == 4) return launch_scan_f32_n4(p, stream);
        if (p.ns == 8) return launch_scan_f32_n8(p, stream);
        return launch_scan_f32_n16(p, stream);
    }
    if (p.ns == 4) return launch_scan_bf16_n4(p, stream);
    if (p.ns == 8) return launch_scan_bf16_n8(p, stream);
    return launch_scan_bf16_n16(p, stream);
}

}  // namespace sfm
