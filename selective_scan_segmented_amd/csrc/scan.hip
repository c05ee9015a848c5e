// scan.hip -- launch planning for the folded, segmented selective scan
// (kernel: scan_kernel.h; instantiations: scan_<io>_n<N>.hip).
#include "scan_kernel.h"

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

bool plan_scan(ScanParams& p, int io_bytes, int waves_hint, int ch_hint, int stagger_hint, int stages_hint) {
    const int L = p.L, S = p.B2 * p.L;
    if (p.xrow <= 0) p.xrow = p.pad_in ? L - 2 : L;
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
    const int cus = device_cus();
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
