// sfm_api.cpp -- the C ABI of libsfm (declared in include/sfm.h): argument
// validation, dispatch to the HIP kernels, error reporting and the adaptive-B1
// lookup table.  Nothing here allocates device memory or synchronises.
#include "sfm.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "sfm_bwd.h"
#include "sfm_cl.h"
#include "sfm_internal.h"

namespace {

thread_local std::string g_last_error;

sfm_status fail(sfm_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

sfm_status ok() {
    g_last_error.clear();
    return SFM_OK;
}

sfm_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(SFM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int io_bytes(int io_dtype) { return io_dtype == SFM_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    const char* name;
    uintptr_t lo, hi;
};

Range rng(const char* name, const void* p, int64_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// products of positive sizes that must stay well inside int32 indexing of one
// (sample, channel) row and int64 element counts overall
bool sane(int64_t v, int64_t hi) { return v >= 1 && v <= hi; }

}  // namespace

extern "C" {

const char* sfm_status_string(sfm_status s) {
    switch (s) {
        case SFM_OK: return "ok";
        case SFM_ERR_NULL: return "null pointer";
        case SFM_ERR_SHAPE: return "invalid shape";
        case SFM_ERR_DTYPE: return "invalid dtype";
        case SFM_ERR_UNSUPPORTED: return "unsupported";
        case SFM_ERR_HIP: return "HIP runtime error";
        case SFM_ERR_ALIAS: return "output overlaps an input";
        case SFM_ERR_ALIGN: return "io pointer not 16-byte aligned";
    }
    return "unknown status";
}

const char* sfm_last_error(void) { return g_last_error.c_str(); }

int sfm_version(void) { return 100; }

sfm_status sfm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* Bm,
                                  const void* Cm, const float* Dskip, const float* delta_bias,
                                  int delta_softplus, const float* conv_w, const float* conv_b, int conv_k,
                                  int conv_pad_left, int conv_act, void* y, int64_t B1, int64_t B2, int64_t D,
                                  int64_t N, int64_t L, int io_dtype, void* stream) {
    return sfm_selective_scan_fwd_ex(u, delta, A, Bm, Cm, Dskip, delta_bias, delta_softplus, conv_w, conv_b, conv_k,
                                     conv_pad_left, conv_act, y, B1, B2, D, N, L, io_dtype, 0, stream);
}

// Argument checks shared by the forward entry points (nothing launched on failure).
static sfm_status fwd_check(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                            int delta_softplus, const float* conv_w, int conv_k, int conv_pad_left, int conv_act,
                            void* y, int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L, int io_dtype,
                            int flags) {
    if (!u || !delta || !A || !Bm || !Cm || !y)
        return fail(SFM_ERR_NULL, "sfm_selective_scan_fwd: u, delta, A, Bm, Cm and y are required");
    if (flags & ~(SFM_FUSE_PAD | SFM_FUSE_SWAP | SFM_LAYOUT_BLD))
        return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd_ex: unknown flags 0x%x", flags);
    const bool pad_in = (flags & SFM_FUSE_PAD) != 0;
    if (pad_in && L < 3)
        return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd_ex: SFM_FUSE_PAD needs L >= 3, got %lld", (long long)L);
    if (io_dtype != SFM_F32 && io_dtype != SFM_BF16)
        return fail(SFM_ERR_DTYPE, "sfm_selective_scan_fwd: io_dtype %d", io_dtype);
    if (!sane(B1, 1 << 24) || !sane(B2, 1 << 16) || !sane(D, 1 << 20) || !sane(L, 1 << 24))
        return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd: B1=%lld B2=%lld D=%lld L=%lld out of range",
                    (long long)B1, (long long)B2, (long long)D, (long long)L);
    if (N < 1 || N > SFM_MAX_N)
        return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd: N=%lld not in [1, %d]", (long long)N, SFM_MAX_N);
    if (B2 * L > (1LL << 30))
        return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd: folded row B2*L=%lld too long", (long long)(B2 * L));
    if (B1 * B2 * D * L > (1LL << 40))
        return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd: tensor too large");
    if (delta_softplus != 0 && delta_softplus != 1)
        return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd: delta_softplus must be 0 or 1");
    if (conv_w) {
        if (conv_k < 1 || conv_k > SFM_MAX_K)
            return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd: conv_k=%d not in [1, %d]", conv_k, SFM_MAX_K);
        if (conv_pad_left < 0 || conv_pad_left >= conv_k)
            return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd: conv_pad_left=%d not in [0, %d)", conv_pad_left,
                        conv_k);
        if (conv_act != SFM_ACT_NONE && conv_act != SFM_ACT_SILU)
            return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd: conv_act=%d", conv_act);
    }
    if (!aligned16(u) || !aligned16(delta) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(y))
        return fail(SFM_ERR_ALIGN, "sfm_selective_scan_fwd: io base pointers must be 16-byte aligned");
    const int64_t B = B1 * B2;
    const int eb = io_bytes(io_dtype);
    const Range ry = rng("y", y, B * D * L * eb);
    const int64_t XL = pad_in ? L - 2 : L;
    const Range ins[] = {rng("u", u, B * D * XL * eb), rng("delta", delta, B * D * L * eb),
                         rng("Bm", Bm, B * N * L * eb), rng("Cm", Cm, B * N * L * eb),
                         rng("A", A, D * N * 4)};
    for (const Range& r : ins)
        if (overlap(ry, r)) return fail(SFM_ERR_ALIAS, "sfm_selective_scan_fwd: y overlaps %s", r.name);

    return SFM_OK;
}

// SFM_SCAN_SPLIT (diagnostics): 0 keeps the one-lane-per-channel kernel, 2 or
// 4 asks for that many lanes per channel, 16 for the streaming kernel (one
// state per lane), unset lets the planner choose.
static int split_hint_env() {
    if (const char* e = std::getenv("SFM_SCAN_SPLIT")) return std::atoi(e);
    return -1;
}
// SFM_SCAN_SPLIT_CHUNK (diagnostics): 0 keeps the lane-split kernel's whole-row
// staging, q > 0 asks for its chunked staging with q positions per chunk (for
// the streaming kernel: its chunk length, a multiple of 16 up to 256).
static int split_chunk_hint_env() {
    if (const char* e = std::getenv("SFM_SCAN_SPLIT_CHUNK")) return std::atoi(e);
    return -1;
}

sfm_status sfm_selective_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* Bm,
                                     const void* Cm, const float* Dskip, const float* delta_bias,
                                     int delta_softplus, const float* conv_w, const float* conv_b, int conv_k,
                                     int conv_pad_left, int conv_act, void* y, int64_t B1, int64_t B2, int64_t D,
                                     int64_t N, int64_t L, int io_dtype, int flags, void* stream) {
    const sfm_status st = fwd_check(u, delta, A, Bm, Cm, delta_softplus, conv_w, conv_k, conv_pad_left, conv_act, y,
                                    B1, B2, D, N, L, io_dtype, flags);
    if (st != SFM_OK) return st;
    const bool pad_in = (flags & SFM_FUSE_PAD) != 0;
    const int eb = io_bytes(io_dtype);
    const int64_t XL = pad_in ? L - 2 : L;

    if (flags & SFM_LAYOUT_BLD) {
        sfm::ClParams c{};
        c.u = u;
        c.delta = delta;
        c.A = A;
        c.Bm = Bm;
        c.Cm = Cm;
        c.Dskip = Dskip;
        c.dbias = delta_bias;
        c.conv_w = conv_w;
        c.conv_b = conv_w ? conv_b : nullptr;
        c.y = y;
        c.B1 = (int)B1;
        c.B2 = (int)B2;
        c.D = (int)D;
        c.N = (int)N;
        c.L = (int)L;
        c.K = conv_w ? conv_k : 1;
        c.P = conv_w ? conv_pad_left : 0;
        c.act = conv_w ? conv_act : 0;
        c.softplus = delta_softplus;
        c.pad_in = pad_in ? 1 : 0;
        c.swap_out = (flags & SFM_FUSE_SWAP) ? 1 : 0;
        c.xrow = (int)XL;
        int w_hint = 0;
        if (const char* e = std::getenv("SFM_CL_CHUNK")) w_hint = std::atoi(e);
        if (!sfm::plan_scan_cl(c, eb, w_hint))
            return fail(SFM_ERR_SHAPE, "sfm_selective_scan_fwd_ex: channel-last rows of D=%lld channels must be whole "
                                       "16-byte units", (long long)D);
        return hip_status(sfm::launch_scan_cl(c, io_dtype, static_cast<hipStream_t>(stream)),
                          "sfm_selective_scan_fwd_ex");
    }
    sfm::ScanParams p{};
    p.u = u;
    p.delta = delta;
    p.A = A;
    p.Bm = Bm;
    p.Cm = Cm;
    p.Dskip = Dskip;
    p.dbias = delta_bias;
    p.conv_w = conv_w;
    p.conv_b = conv_w ? conv_b : nullptr;
    p.y = y;
    p.B1 = (int)B1;
    p.B2 = (int)B2;
    p.D = (int)D;
    p.N = (int)N;
    p.L = (int)L;
    p.K = conv_w ? conv_k : 1;
    p.P = conv_w ? conv_pad_left : 0;
    p.act = conv_w ? conv_act : 0;
    p.softplus = delta_softplus;
    p.pad_in = pad_in ? 1 : 0;
    p.swap_out = (flags & SFM_FUSE_SWAP) ? 1 : 0;
    p.xrow = (int)XL;
    int waves_hint = 0, ch_hint = 0;
    if (const char* e = std::getenv("SFM_SCAN_WAVES")) waves_hint = std::atoi(e);
    if (const char* e = std::getenv("SFM_SCAN_CHUNK")) ch_hint = std::atoi(e);
    int stagger_hint = -1, stages_hint = 0;
    if (const char* e = std::getenv("SFM_SCAN_STAGGER")) stagger_hint = std::atoi(e);
    if (const char* e = std::getenv("SFM_SCAN_STAGES")) stages_hint = std::atoi(e);
    if (!sfm::plan_scan(p, eb, waves_hint, ch_hint, stagger_hint, stages_hint, split_hint_env(), split_chunk_hint_env()))
        return fail(SFM_ERR_UNSUPPORTED, "sfm_selective_scan_fwd: no launch plan fits LDS for this shape");
    return hip_status(sfm::launch_scan(p, io_dtype, static_cast<hipStream_t>(stream)), "sfm_selective_scan_fwd");
}

sfm_status sfm_scan_plan_string(int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L, int conv_k, int io_dtype,
                                int flags, char* buf, int64_t cap) {
    if (!buf || cap < 1) return fail(SFM_ERR_NULL, "sfm_scan_plan_string: buf is required");
    if (io_dtype != SFM_F32 && io_dtype != SFM_BF16) return fail(SFM_ERR_DTYPE, "sfm_scan_plan_string: io_dtype");
    if (!sane(B1, 1 << 24) || !sane(B2, 1 << 16) || !sane(D, 1 << 20) || !sane(L, 1 << 24) || N < 1 ||
        N > SFM_MAX_N || conv_k < 0 || conv_k > SFM_MAX_K)
        return fail(SFM_ERR_SHAPE, "sfm_scan_plan_string: sizes out of range");
    static const float dummy = 0.0f;
    if (flags & SFM_LAYOUT_BLD) {
        if ((flags & ~(SFM_FUSE_PAD | SFM_FUSE_SWAP | SFM_LAYOUT_BLD)) || ((flags & SFM_FUSE_PAD) && L < 3))
            return fail(SFM_ERR_SHAPE, "sfm_scan_plan_string: bad flags for these sizes");
        sfm::ClParams c{};
        c.conv_w = conv_k ? &dummy : nullptr;
        c.B1 = (int)B1;
        c.B2 = (int)B2;
        c.D = (int)D;
        c.N = (int)N;
        c.L = (int)L;
        c.K = conv_k ? conv_k : 1;
        c.pad_in = (flags & SFM_FUSE_PAD) ? 1 : 0;
        c.swap_out = (flags & SFM_FUSE_SWAP) ? 1 : 0;
        c.xrow = c.pad_in ? (int)L - 2 : (int)L;
        int w_hint = 0;
        if (const char* e = std::getenv("SFM_CL_CHUNK")) w_hint = std::atoi(e);
        if (!sfm::plan_scan_cl(c, io_bytes(io_dtype), w_hint))
            return fail(SFM_ERR_SHAPE, "sfm_scan_plan_string: channel-last rows must be whole 16-byte units");
        snprintf(buf, (size_t)cap, "layout=bld chunk=%d chunks=%d ns=%d cw=%d lds=%d grid=%d block=%d stagger=%d/%d",
                 c.W, c.nchunk, c.ns, c.cw, c.lds_bytes, c.B1 * c.tgroups, 64 * c.cw, c.stagger_ticks,
                 c.stagger_period);
        return ok();
    }
    sfm::ScanParams p{};
    p.conv_w = conv_k ? &dummy : nullptr;
    p.B1 = (int)B1;
    p.B2 = (int)B2;
    p.D = (int)D;
    p.N = (int)N;
    p.L = (int)L;
    p.K = conv_k ? conv_k : 1;
    if ((flags & ~(SFM_FUSE_PAD | SFM_FUSE_SWAP)) || ((flags & SFM_FUSE_PAD) && L < 3))
        return fail(SFM_ERR_SHAPE, "sfm_scan_plan_string: bad flags for these sizes");
    p.pad_in = (flags & SFM_FUSE_PAD) ? 1 : 0;
    p.swap_out = (flags & SFM_FUSE_SWAP) ? 1 : 0;
    p.xrow = p.pad_in ? (int)L - 2 : (int)L;
    int waves_hint = 0, ch_hint = 0;
    if (const char* e = std::getenv("SFM_SCAN_WAVES")) waves_hint = std::atoi(e);
    if (const char* e = std::getenv("SFM_SCAN_CHUNK")) ch_hint = std::atoi(e);
    int stagger_hint = -1, stages_hint = 0;
    if (const char* e = std::getenv("SFM_SCAN_STAGGER")) stagger_hint = std::atoi(e);
    if (const char* e = std::getenv("SFM_SCAN_STAGES")) stages_hint = std::atoi(e);
    if (!sfm::plan_scan(p, io_bytes(io_dtype), waves_hint, ch_hint, stagger_hint, stages_hint, split_hint_env(), split_chunk_hint_env()))
        return fail(SFM_ERR_UNSUPPORTED, "sfm_scan_plan_string: no launch plan fits LDS");
    if (p.split) {
        snprintf(buf, (size_t)cap, "split=%d chunk=%d ns=%d wpg=%d lds=%d grid=%lld block=%d stagger=%d/%d", p.split,
                 p.sq, p.ns, p.wpg, p.lds_bytes, (long long)p.stiles * p.B1, 64 * p.wpg, p.stagger_ticks,
                 p.stagger_period);
        return ok();
    }
    snprintf(buf, (size_t)cap,
             "mode=%d ch=%d pieces=%d piece=%d carry=%d cw=%d ns=%d lds=%d grid=%lld block=%d stagger=%d/%d "
             "stages=%d",
             p.mode, p.ch, p.waves, p.piece, p.need_carry, p.cw, p.ns, p.lds_bytes,
             (long long)p.tgroups * p.B1 * (p.wsplit ? p.waves : 1), 64 * p.cw * (p.wsplit ? 1 : p.waves),
             p.stagger_ticks, p.stagger_period, p.stages);
    return ok();
}

sfm_status sfm_dwconv1d_fold(const void* x, const float* w, const float* bias, void* out, int64_t B1, int64_t B2,
                             int64_t D, int64_t L, int K, int pad_left, int act, int io_dtype, void* stream) {
    if (!x || !w || !out) return fail(SFM_ERR_NULL, "sfm_dwconv1d_fold: x, w and out are required");
    if (io_dtype != SFM_F32 && io_dtype != SFM_BF16)
        return fail(SFM_ERR_DTYPE, "sfm_dwconv1d_fold: io_dtype %d", io_dtype);
    if (!sane(B1, 1 << 24) || !sane(B2, 1 << 16) || !sane(D, 1 << 20) || !sane(L, 1 << 24) ||
        B1 * B2 * D * L > (1LL << 40))
        return fail(SFM_ERR_SHAPE, "sfm_dwconv1d_fold: B1=%lld B2=%lld D=%lld L=%lld out of range",
                    (long long)B1, (long long)B2, (long long)D, (long long)L);
    if (K < 1 || K > SFM_MAX_K) return fail(SFM_ERR_SHAPE, "sfm_dwconv1d_fold: K=%d not in [1, %d]", K, SFM_MAX_K);
    if (pad_left < 0 || pad_left >= K)
        return fail(SFM_ERR_SHAPE, "sfm_dwconv1d_fold: pad_left=%d not in [0, %d)", pad_left, K);
    if (act != SFM_ACT_NONE && act != SFM_ACT_SILU) return fail(SFM_ERR_SHAPE, "sfm_dwconv1d_fold: act=%d", act);
    if (!aligned16(x) || !aligned16(out))
        return fail(SFM_ERR_ALIGN, "sfm_dwconv1d_fold: io base pointers must be 16-byte aligned");
    const int64_t bytes = B1 * B2 * D * L * io_bytes(io_dtype);
    if (overlap(rng("out", out, bytes), rng("x", x, bytes)))
        return fail(SFM_ERR_ALIAS, "sfm_dwconv1d_fold: out overlaps x");
    return hip_status(sfm::launch_dwconv1d(x, w, bias, out, B1, B2, D, L, K, pad_left, act, io_dtype,
                                           static_cast<hipStream_t>(stream)),
                      "sfm_dwconv1d_fold");
}

sfm_status sfm_aux_pad_swap(const void* in, void* out, int64_t B, int64_t D, int64_t T, int mode, int io_dtype,
                            void* stream) {
    if (!in || !out) return fail(SFM_ERR_NULL, "sfm_aux_pad_swap: in and out are required");
    if (io_dtype != SFM_F32 && io_dtype != SFM_BF16)
        return fail(SFM_ERR_DTYPE, "sfm_aux_pad_swap: io_dtype %d", io_dtype);
    if (mode != SFM_AUX_PAD && mode != SFM_AUX_SWAP) return fail(SFM_ERR_SHAPE, "sfm_aux_pad_swap: mode %d", mode);
    if (!sane(B, 1 << 24) || !sane(D, 1 << 20))
        return fail(SFM_ERR_SHAPE, "sfm_aux_pad_swap: B=%lld D=%lld out of range", (long long)B, (long long)D);
    if (mode == SFM_AUX_PAD ? (T < 1 || T > (1 << 24)) : (T < -1 || T > (1 << 24)))
        return fail(SFM_ERR_SHAPE, "sfm_aux_pad_swap: T=%lld out of range for mode %d", (long long)T, mode);
    if (B * D * (T + 2) > (1LL << 40)) return fail(SFM_ERR_SHAPE, "sfm_aux_pad_swap: tensor too large");
    if (!aligned16(in) || !aligned16(out))
        return fail(SFM_ERR_ALIGN, "sfm_aux_pad_swap: io base pointers must be 16-byte aligned");
    const int eb = io_bytes(io_dtype);
    const int64_t L = T + 2;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mode == SFM_AUX_PAD) {
        if (overlap(rng("out", out, B * D * L * eb), rng("in", in, B * D * T * eb)))
            return fail(SFM_ERR_ALIAS, "sfm_aux_pad_swap: PAD output overlaps its input");
        return hip_status(sfm::launch_aux_pad(in, out, B * D, T, io_dtype, s), "sfm_aux_pad_swap(PAD)");
    }
    if (in != out && overlap(rng("out", out, B * D * L * eb), rng("in", in, B * D * L * eb)))
        return fail(SFM_ERR_ALIAS, "sfm_aux_pad_swap: SWAP output partially overlaps its input");
    return hip_status(sfm::launch_aux_swap(in, out, B * D, L, io_dtype, s), "sfm_aux_pad_swap(SWAP)");
}

}  // extern "C"

// ------------------------------------------------------------------ adaptive B1
namespace {

struct B1Entry {
    int64_t B, L, D, N, B2;
};

#include "b1_table.inc"

std::vector<B1Entry> load_env_table() {
    std::vector<B1Entry> v;
    const char* path = std::getenv("SFM_B1_TABLE");
    if (!path || !*path) return v;
    FILE* f = std::fopen(path, "r");
    if (!f) return v;
    char line[256];
    while (std::fgets(line, sizeof(line), f)) {
        long long b, l, d, n, b2;
        if (line[0] == '#') continue;
        if (std::sscanf(line, "%lld %lld %lld %lld %lld", &b, &l, &d, &n, &b2) == 5 && b2 >= 1)
            v.push_back(B1Entry{b, l, d, n, b2});
    }
    std::fclose(f);
    return v;
}

double key_distance(const B1Entry& e, int64_t B, int64_t L, int64_t D, int64_t N) {
    auto lg = [](double v) { return std::log2(v); };
    const double db = lg((double)e.B) - lg((double)B);
    const double dl = lg((double)e.L) - lg((double)L);
    const double dd = lg((double)e.D) - lg((double)D);
    const double dn = ((double)e.N - (double)N) / 4.0;
    return db * db + dl * dl + dd * dd + dn * dn;
}

}  // namespace

extern "C" sfm_status sfm_pick_b1(int64_t B, int64_t L, int64_t D, int64_t N, int64_t* B1_out) {
    if (!B1_out) return fail(SFM_ERR_NULL, "sfm_pick_b1: B1_out is required");
    if (!sane(B, 1 << 24) || !sane(L, 1 << 24) || !sane(D, 1 << 20) || N < 1 || N > SFM_MAX_N)
        return fail(SFM_ERR_SHAPE, "sfm_pick_b1: B=%lld L=%lld D=%lld N=%lld out of range", (long long)B,
                    (long long)L, (long long)D, (long long)N);
    std::vector<B1Entry> table = load_env_table();
    for (const B1Entry& e : kB1Table) table.push_back(e);
    int64_t want_b2 = 1;
    double best = 1e300;
    for (const B1Entry& e : table) {  // first entry wins ties: the env file precedes the built-in table
        const double dist = key_distance(e, B, L, D, N);
        if (dist < best) {
            best = dist;
            want_b2 = e.B2;
        }
    }
    int64_t b2 = 1;
    for (int64_t c = 1; c <= want_b2 && c <= B; ++c)
        if (B % c == 0) b2 = c;
    *B1_out = B / b2;
    return ok();
}

// ---------------------------------------------------------------- backward
namespace {

sfm_status bwd_common(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                      const void* dy, const float* conv_w, int conv_k, int conv_pad_left, int conv_act,
                      int delta_softplus, int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L, int io_dtype,
                      int flags, const char* who) {
    if (!u || !delta || !A || !Bm || !Cm || !dy) return fail(SFM_ERR_NULL, "%s: u, delta, A, Bm, Cm, dy are required", who);
    if (flags & ~(SFM_FUSE_PAD | SFM_FUSE_SWAP | SFM_LAYOUT_BLD))
        return fail(SFM_ERR_SHAPE, "%s: unknown flags 0x%x", who, flags);
    if ((flags & SFM_FUSE_PAD) && L < 3) return fail(SFM_ERR_SHAPE, "%s: SFM_FUSE_PAD needs L >= 3", who);
    if (io_dtype != SFM_F32 && io_dtype != SFM_BF16) return fail(SFM_ERR_DTYPE, "%s: io_dtype %d", who, io_dtype);
    if (!sane(B1, 1 << 24) || !sane(B2, 1 << 16) || !sane(D, 1 << 20) || !sane(L, 1 << 24))
        return fail(SFM_ERR_SHAPE, "%s: B1=%lld B2=%lld D=%lld L=%lld out of range", who, (long long)B1,
                    (long long)B2, (long long)D, (long long)L);
    if (N < 1 || N > SFM_MAX_N) return fail(SFM_ERR_SHAPE, "%s: N=%lld not in [1, %d]", who, (long long)N, SFM_MAX_N);
    if (B1 * B2 * D * L > (1LL << 40)) return fail(SFM_ERR_SHAPE, "%s: tensor too large", who);
    if (delta_softplus != 0 && delta_softplus != 1) return fail(SFM_ERR_SHAPE, "%s: delta_softplus must be 0 or 1", who);
    if ((flags & SFM_LAYOUT_BLD) && (D * io_bytes(io_dtype)) % 16 != 0)
        return fail(SFM_ERR_SHAPE, "%s: channel-last rows of D=%lld channels must be whole 16-byte units", who,
                    (long long)D);
    if (conv_w) {
        if (conv_k < 1 || conv_k > SFM_MAX_K) return fail(SFM_ERR_SHAPE, "%s: conv_k=%d not in [1, %d]", who, conv_k, SFM_MAX_K);
        if (conv_pad_left < 0 || conv_pad_left >= conv_k)
            return fail(SFM_ERR_SHAPE, "%s: conv_pad_left=%d not in [0, %d)", who, conv_pad_left, conv_k);
        if (conv_act != SFM_ACT_NONE && conv_act != SFM_ACT_SILU) return fail(SFM_ERR_SHAPE, "%s: conv_act=%d", who, conv_act);
    }
    return ok();
}

void fill_bwd(sfm::BwdParams& p, int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L, const float* conv_w,
              int conv_k, int conv_pad_left, int conv_act, int delta_softplus, int flags) {
    // The backward runs unfolded: every sample starts from a reset, so a folded
    // row's samples are independent work, and one wave per (sample, tile)
    // gives the GPU B2 times the waves of one per (folded row, tile).
    p.B1 = (int)(B1 * B2);
    p.B2 = 1;
    p.D = (int)D;
    p.N = (int)N;
    p.L = (int)L;
    p.conv_w = conv_w;
    p.K = conv_w ? conv_k : 1;
    p.P = conv_w ? conv_pad_left : 0;
    p.act = conv_w ? conv_act : 0;
    p.softplus = delta_softplus;
    p.pad_in = (flags & SFM_FUSE_PAD) ? 1 : 0;
    p.swap_dy = (flags & SFM_FUSE_SWAP) ? 1 : 0;
    p.cl = (flags & SFM_LAYOUT_BLD) ? 1 : 0;
    p.xrow = p.pad_in ? (int)L - 2 : (int)L;
}

// Channel-last rows that the whole-sample kernel cannot stage (too long for
// its LDS): the backward runs channel-first on transposed copies.  The
// workspace holds the channel-first plan's own workspace, then x, delta, dy, B
// and C transposed to [B, D, *] / [B, N, L], then du, ddelta (io) and dB, dC
// (float32) in the channel-first layout, which are transposed back into the
// caller's tensors.  Offsets in bytes, each region on 256 bytes.
struct ClAdapter {
    size_t xT, dT, dyT, bT, cT, duT, ddT, dbT, dcT, total;
};

bool plan_cl_adapter(sfm::BwdParams& q, int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L,
                     const float* conv_w, int conv_k, int conv_pad_left, int conv_act, int delta_softplus, int flags,
                     int eb, ClAdapter& a) {
    fill_bwd(q, B1, B2, D, N, L, conv_w, conv_k, conv_pad_left, conv_act, delta_softplus, flags & ~SFM_LAYOUT_BLD);
    size_t ws = 0;
    if (!sfm::plan_bwd(q, eb, &ws)) return false;
    const size_t B = (size_t)(B1 * B2), XL = (flags & SFM_FUSE_PAD) ? (size_t)L - 2 : (size_t)L;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    size_t off = up(ws);
    a.xT = off;
    off += up(B * D * XL * eb);
    a.dT = off;
    off += up(B * D * L * eb);
    a.dyT = off;
    off += up(B * D * L * eb);
    a.bT = off;
    off += up(B * N * L * eb);
    a.cT = off;
    off += up(B * N * L * eb);
    a.duT = off;
    off += up(B * D * L * eb);
    a.ddT = off;
    off += up(B * D * L * eb);
    a.dbT = off;
    off += up(B * N * L * 4);
    a.dcT = off;
    off += up(B * N * L * 4);
    a.total = off;
    return true;
}

}  // namespace

extern "C" sfm_status sfm_selective_scan_bwd_workspace_size(int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L,
                                                             int conv_k, int io_dtype, int flags, int64_t* bytes) {
    if (!bytes) return fail(SFM_ERR_NULL, "sfm_selective_scan_bwd_workspace_size: bytes is required");
    static const float dummy = 0.0f;
    static const char dummy_io[16] = {0};
    sfm_status st = bwd_common(dummy_io, dummy_io, &dummy, dummy_io, dummy_io, dummy_io, conv_k ? &dummy : nullptr,
                               conv_k ? conv_k : 1, 0, 0, 1, B1, B2, D, N, L, io_dtype, flags,
                               "sfm_selective_scan_bwd_workspace_size");
    if (st != SFM_OK) return st;
    sfm::BwdParams p{};
    fill_bwd(p, B1, B2, D, N, L, conv_k ? &dummy : nullptr, conv_k ? conv_k : 1, 0, 0, 1, flags);
    size_t ws = 0;
    if (!sfm::plan_bwd(p, io_bytes(io_dtype), &ws)) {
        sfm::BwdParams q{};
        ClAdapter a{};
        if (!p.cl || !plan_cl_adapter(q, B1, B2, D, N, L, conv_k ? &dummy : nullptr, conv_k ? conv_k : 1, 0, 0, 1,
                                      flags, io_bytes(io_dtype), a))
            return fail(SFM_ERR_UNSUPPORTED, "sfm_selective_scan_bwd_workspace_size: no plan fits LDS");
        ws = a.total;
    }
    *bytes = (int64_t)ws;
    return ok();
}

extern "C" sfm_status sfm_selective_scan_bwd(
    const void* u, const void* delta, const float* A, const void* Bm, const void* Cm, const float* Dskip,
    const float* delta_bias, int delta_softplus, const float* conv_w, const float* conv_b, int conv_k,
    int conv_pad_left, int conv_act, const void* dy, void* du, void* ddelta, float* dA, float* dBm, float* dCm,
    float* dDskip, float* ddelta_bias, float* dconv_w, float* dconv_b, int64_t B1, int64_t B2, int64_t D, int64_t N,
    int64_t L, int io_dtype, int flags, void* workspace, int64_t workspace_bytes, void* stream) {
    const char* who = "sfm_selective_scan_bwd";
    sfm_status st = bwd_common(u, delta, A, Bm, Cm, dy, conv_w, conv_k, conv_pad_left, conv_act, delta_softplus, B1,
                               B2, D, N, L, io_dtype, flags, who);
    if (st != SFM_OK) return st;
    if (!du || !ddelta || !dA || !dBm || !dCm) return fail(SFM_ERR_NULL, "%s: du, ddelta, dA, dBm, dCm are required", who);
    if (conv_w && !dconv_w) return fail(SFM_ERR_NULL, "%s: dconv_w is required with conv_w", who);
    if (!aligned16(u) || !aligned16(delta) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(dy) || !aligned16(du) ||
        !aligned16(ddelta))
        return fail(SFM_ERR_ALIGN, "%s: io base pointers must be 16-byte aligned", who);
    const int64_t B = B1 * B2;
    const int eb = io_bytes(io_dtype);
    const int64_t XL = (flags & SFM_FUSE_PAD) ? L - 2 : L;
    const int64_t K = conv_w ? conv_k : 0;
    const Range ins[] = {rng("u", u, B * D * XL * eb), rng("delta", delta, B * D * L * eb),
                         rng("Bm", Bm, B * N * L * eb), rng("Cm", Cm, B * N * L * eb), rng("dy", dy, B * D * L * eb),
                         rng("A", A, D * N * 4), rng("Dskip", Dskip, D * 4), rng("delta_bias", delta_bias, D * 4),
                         rng("conv_w", conv_w, D * K * 4), rng("conv_b", conv_b, conv_w ? D * 4 : 0)};
    const Range outs[] = {rng("du", du, B * D * L * eb), rng("ddelta", ddelta, B * D * L * eb),
                          rng("dA", dA, D * N * 4), rng("dBm", dBm, B * N * L * 4), rng("dCm", dCm, B * N * L * 4),
                          rng("dDskip", dDskip, D * 4), rng("ddelta_bias", ddelta_bias, D * 4),
                          rng("dconv_w", dconv_w, D * K * 4), rng("dconv_b", dconv_b, conv_w ? D * 4 : 0),
                          rng("workspace", workspace, workspace_bytes)};
    for (const Range& o : outs)
        for (const Range& i : ins)
            if (o.lo && i.lo && overlap(o, i)) return fail(SFM_ERR_ALIAS, "%s: %s overlaps %s", who, o.name, i.name);
    for (size_t a = 0; a < sizeof(outs) / sizeof(outs[0]); ++a)
        for (size_t c = a + 1; c < sizeof(outs) / sizeof(outs[0]); ++c)
            if (outs[a].lo && outs[c].lo && overlap(outs[a], outs[c]))
                return fail(SFM_ERR_ALIAS, "%s: %s overlaps %s", who, outs[a].name, outs[c].name);
    sfm::BwdParams p{};
    fill_bwd(p, B1, B2, D, N, L, conv_w, conv_k, conv_pad_left, conv_act, delta_softplus, flags);
    size_t need = 0;
    if (!sfm::plan_bwd(p, eb, &need)) {
        sfm::BwdParams q{};
        ClAdapter a{};
        if (!p.cl || !plan_cl_adapter(q, B1, B2, D, N, L, conv_w, conv_k, conv_pad_left, conv_act, delta_softplus,
                                      flags, eb, a))
            return fail(SFM_ERR_UNSUPPORTED, "%s: no plan fits LDS", who);
        if (!workspace || workspace_bytes < (int64_t)a.total)
            return fail(SFM_ERR_SHAPE, "%s: workspace of %lld bytes needed (see sfm_selective_scan_bwd_workspace_size)",
                        who, (long long)a.total);
        const hipStream_t s = static_cast<hipStream_t>(stream);
        char* w = static_cast<char*>(workspace);
        // channel-last -> channel-first: u [B, XL, D], delta/dy [B, L, D], B/C [B, L, N]
        hipError_t e = sfm::launch_transpose(u, w + a.xT, B, XL, D, eb, s);
        if (e == hipSuccess) e = sfm::launch_transpose(delta, w + a.dT, B, L, D, eb, s);
        if (e == hipSuccess) e = sfm::launch_transpose(dy, w + a.dyT, B, L, D, eb, s);
        if (e == hipSuccess) e = sfm::launch_transpose(Bm, w + a.bT, B, L, N, eb, s);
        if (e == hipSuccess) e = sfm::launch_transpose(Cm, w + a.cT, B, L, N, eb, s);
        if (e != hipSuccess) return hip_status(e, who);
        q.u = w + a.xT;
        q.delta = w + a.dT;
        q.A = A;
        q.Bm = w + a.bT;
        q.Cm = w + a.cT;
        q.Dskip = Dskip;
        q.dbias = delta_bias;
        q.conv_b = conv_b;
        q.dy = w + a.dyT;
        q.du = w + a.duT;
        q.ddelta = w + a.ddT;
        q.dA = dA;
        q.dBm = reinterpret_cast<float*>(w + a.dbT);
        q.dCm = reinterpret_cast<float*>(w + a.dcT);
        q.dDskip = dDskip;
        q.ddbias = ddelta_bias;
        q.dconv_w = dconv_w;
        q.dconv_b = dconv_b;
        q.ws = reinterpret_cast<float*>(w);
        e = sfm::launch_bwd(q, io_dtype, s);
        // channel-first -> channel-last: du, ddelta [B, D, L] -> [B, L, D]; dB, dC [B, N, L] -> [B, L, N]
        if (e == hipSuccess) e = sfm::launch_transpose(w + a.duT, du, B, D, L, eb, s);
        if (e == hipSuccess) e = sfm::launch_transpose(w + a.ddT, ddelta, B, D, L, eb, s);
        if (e == hipSuccess) e = sfm::launch_transpose(w + a.dbT, dBm, B, N, L, 4, s);
        if (e == hipSuccess) e = sfm::launch_transpose(w + a.dcT, dCm, B, N, L, 4, s);
        return hip_status(e, who);
    }
    if (!workspace || workspace_bytes < (int64_t)need)
        return fail(SFM_ERR_SHAPE, "%s: workspace of %lld bytes needed (see sfm_selective_scan_bwd_workspace_size)",
                    who, (long long)need);
    p.u = u;
    p.delta = delta;
    p.A = A;
    p.Bm = Bm;
    p.Cm = Cm;
    p.Dskip = Dskip;
    p.dbias = delta_bias;
    p.conv_b = conv_b;
    p.dy = dy;
    p.du = du;
    p.ddelta = ddelta;
    p.dA = dA;
    p.dBm = dBm;
    p.dCm = dCm;
    p.dDskip = dDskip;
    p.ddbias = ddelta_bias;
    p.dconv_w = dconv_w;
    p.dconv_b = dconv_b;
    p.ws = static_cast<float*>(workspace);
    return hip_status(sfm::launch_bwd(p, io_dtype, static_cast<hipStream_t>(stream)), who);
}

// True when the regular forward plans these rows for the streaming lane-split
// kernel (long rows of 9 to 16 states), which runs them faster than the
// split-row scheme and needs no workspace (the long rows: 236 vs 500 us).
static bool regular_plan_streams(int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L, int conv_k, int eb,
                                 int flags) {
    static const float dummy = 0.0f;
    sfm::ScanParams p{};
    p.conv_w = conv_k ? &dummy : nullptr;
    p.B1 = (int)B1;
    p.B2 = (int)B2;
    p.D = (int)D;
    p.N = (int)N;
    p.L = (int)L;
    p.K = conv_k ? conv_k : 1;
    p.pad_in = (flags & SFM_FUSE_PAD) ? 1 : 0;
    p.swap_out = (flags & SFM_FUSE_SWAP) ? 1 : 0;
    p.xrow = p.pad_in ? (int)L - 2 : (int)L;
    int waves_hint = 0, ch_hint = 0;
    if (const char* e = std::getenv("SFM_SCAN_WAVES")) waves_hint = std::atoi(e);
    if (const char* e = std::getenv("SFM_SCAN_CHUNK")) ch_hint = std::atoi(e);
    return sfm::plan_scan(p, eb, waves_hint, ch_hint, -1, 0, split_hint_env(), split_chunk_hint_env()) &&
           p.split == 16;
}

// Split-row forward plan (p.seg > 1) or none: channel-last rows, rows that the
// chunked planner does not split, rows the regular forward streams (unless
// SFM_BWD_SEGMENTS forces a split, for diagnostics), or no plan -> the regular
// forward.
static bool fwd_split_plan(sfm::BwdParams& p, int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L,
                           const float* conv_w, int conv_k, int conv_pad_left, int conv_act, int delta_softplus,
                           int flags, int eb, size_t* need) {
    if (flags & SFM_LAYOUT_BLD) return false;
    if (!std::getenv("SFM_BWD_SEGMENTS") && regular_plan_streams(B1, B2, D, N, L, conv_w ? conv_k : 0, eb, flags))
        return false;
    fill_bwd(p, B1, B2, D, N, L, conv_w, conv_k, conv_pad_left, conv_act, delta_softplus, flags);
    p.fwd = 1;
    p.swap_out = (flags & SFM_FUSE_SWAP) ? 1 : 0;
    *need = 0;
    return sfm::plan_bwd(p, eb, need) && p.seg > 1;
}

extern "C" sfm_status sfm_selective_scan_fwd_ws_size(int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L,
                                                     int conv_k, int io_dtype, int flags, int64_t* bytes) {
    const char* who = "sfm_selective_scan_fwd_ws_size";
    if (!bytes) return fail(SFM_ERR_NULL, "%s: bytes is required", who);
    if (io_dtype != SFM_F32 && io_dtype != SFM_BF16) return fail(SFM_ERR_DTYPE, "%s: io_dtype %d", who, io_dtype);
    if (flags & ~(SFM_FUSE_PAD | SFM_FUSE_SWAP | SFM_LAYOUT_BLD))
        return fail(SFM_ERR_SHAPE, "%s: unknown flags 0x%x", who, flags);
    if (!sane(B1, 1 << 24) || !sane(B2, 1 << 16) || !sane(D, 1 << 20) || !sane(L, 1 << 24) || N < 1 ||
        N > SFM_MAX_N || ((flags & SFM_FUSE_PAD) && L < 3) || conv_k < 0 || conv_k > SFM_MAX_K)
        return fail(SFM_ERR_SHAPE, "%s: B1=%lld B2=%lld D=%lld N=%lld L=%lld conv_k=%d out of range", who,
                    (long long)B1, (long long)B2, (long long)D, (long long)N, (long long)L, conv_k);
    static const float dummy = 0.0f;
    sfm::BwdParams p{};
    size_t need = 0;
    *bytes = fwd_split_plan(p, B1, B2, D, N, L, conv_k ? &dummy : nullptr, conv_k ? conv_k : 1, 0, 0, 1, flags,
                            io_bytes(io_dtype), &need)
                 ? (int64_t)need
                 : 0;
    return ok();
}

extern "C" sfm_status sfm_selective_scan_fwd_ws(const void* u, const void* delta, const float* A, const void* Bm,
                                                const void* Cm, const float* Dskip, const float* delta_bias,
                                                int delta_softplus, const float* conv_w, const float* conv_b,
                                                int conv_k, int conv_pad_left, int conv_act, void* y, int64_t B1,
                                                int64_t B2, int64_t D, int64_t N, int64_t L, int io_dtype, int flags,
                                                void* workspace, int64_t workspace_bytes, void* stream) {
    const char* who = "sfm_selective_scan_fwd_ws";
    const sfm_status st = fwd_check(u, delta, A, Bm, Cm, delta_softplus, conv_w, conv_k, conv_pad_left, conv_act, y,
                                    B1, B2, D, N, L, io_dtype, flags);
    if (st != SFM_OK) return st;
    const int eb = io_bytes(io_dtype);
    sfm::BwdParams p{};
    size_t need = 0;
    if (!fwd_split_plan(p, B1, B2, D, N, L, conv_w, conv_k, conv_pad_left, conv_act, delta_softplus, flags, eb,
                        &need))
        return sfm_selective_scan_fwd_ex(u, delta, A, Bm, Cm, Dskip, delta_bias, delta_softplus, conv_w, conv_b,
                                         conv_k, conv_pad_left, conv_act, y, B1, B2, D, N, L, io_dtype, flags,
                                         stream);
    if (!workspace || workspace_bytes < (int64_t)need)
        return fail(SFM_ERR_SHAPE, "%s: workspace of %lld bytes needed (see sfm_selective_scan_fwd_ws_size)", who,
                    (long long)need);
    const int64_t B = B1 * B2, XL = (flags & SFM_FUSE_PAD) ? L - 2 : L;
    const Range rw = rng("workspace", workspace, workspace_bytes);
    // the kernels read every input after the workspace has been written
    const Range others[] = {rng("u", u, B * D * XL * eb), rng("delta", delta, B * D * L * eb),
                            rng("Bm", Bm, B * N * L * eb), rng("Cm", Cm, B * N * L * eb), rng("A", A, D * N * 4),
                            rng("y", y, B * D * L * eb), rng("Dskip", Dskip, Dskip ? D * 4 : 0),
                            rng("delta_bias", delta_bias, delta_bias ? D * 4 : 0),
                            rng("conv_w", conv_w, conv_w ? D * conv_k * 4 : 0),
                            rng("conv_b", conv_b, conv_w && conv_b ? D * 4 : 0)};
    for (const Range& r : others)
        if (overlap(rw, r)) return fail(SFM_ERR_ALIAS, "%s: workspace overlaps %s", who, r.name);
    p.u = u;
    p.delta = delta;
    p.A = A;
    p.Bm = Bm;
    p.Cm = Cm;
    p.Dskip = Dskip;
    p.dbias = delta_bias;
    p.conv_b = conv_w ? conv_b : nullptr;
    p.y = y;
    p.ws = static_cast<float*>(workspace);
    return hip_status(sfm::launch_fwd_split(p, io_dtype, static_cast<hipStream_t>(stream)), who);
}

// ------------------------------------------------------------ no allocation
// Scratch of sfm_selective_scan_fwd_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address comes from hipGetSymbolAddress, resolved once per device (with that
// device current) and kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[SFM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
sfm_status scratch_of_current_device(const char* who, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SFM_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(SFM_ERR_UNSUPPORTED, "%s: device %d out of range", who, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(SFM_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
        }
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return SFM_OK;
}
}  // namespace

extern "C" sfm_status sfm_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* Bm,
                                                     const void* Cm, const float* Dskip, const float* delta_bias,
                                                     int delta_softplus, const float* conv_w, const float* conv_b,
                                                     int conv_k, int conv_pad_left, int conv_act, void* y,
                                                     int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L,
                                                     int io_dtype, int flags, void* stream) {
    const char* who = "sfm_selective_scan_fwd_noalloc";
    const sfm_status st = fwd_check(u, delta, A, Bm, Cm, delta_softplus, conv_w, conv_k, conv_pad_left, conv_act, y,
                                    B1, B2, D, N, L, io_dtype, flags);
    if (st != SFM_OK) return st;
    sfm::BwdParams p{};
    size_t need = 0;
    if (!fwd_split_plan(p, B1, B2, D, N, L, conv_w, conv_k, conv_pad_left, conv_act, delta_softplus, flags,
                        io_bytes(io_dtype), &need))
        // rows the plan does not split: the regular forward, which uses no scratch
        return sfm_selective_scan_fwd_ex(u, delta, A, Bm, Cm, Dskip, delta_bias, delta_softplus, conv_w, conv_b,
                                         conv_k, conv_pad_left, conv_act, y, B1, B2, D, N, L, io_dtype, flags,
                                         stream);
    if ((long long)need > SFM_NOALLOC_SCRATCH_BYTES)
        return fail(SFM_ERR_UNSUPPORTED, "%s: these rows need %lld bytes of scratch, the static array holds %lld",
                    who, (long long)need, (long long)SFM_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    const sfm_status sst = scratch_of_current_device(who, &ws);
    if (sst != SFM_OK) return sst;
    p.u = u;
    p.delta = delta;
    p.A = A;
    p.Bm = Bm;
    p.Cm = Cm;
    p.Dskip = Dskip;
    p.dbias = delta_bias;
    p.conv_b = conv_w ? conv_b : nullptr;
    p.y = y;
    // every word of the scratch the kernels read is written earlier in the same
    // call (token sums, then carries), so nothing needs clearing between calls
    p.ws = static_cast<float*>(ws);
    return hip_status(sfm::launch_fwd_split(p, io_dtype, static_cast<hipStream_t>(stream)), who);
}

extern "C" sfm_status sfm_aux_pad_bwd_ex(const void* gpad, void* gx, int64_t B, int64_t D, int64_t T, int io_dtype,
                                         int flags, void* stream) {
    const char* who = "sfm_aux_pad_bwd";
    if (!gpad || !gx) return fail(SFM_ERR_NULL, "%s: gpad and gx are required", who);
    if (flags & ~SFM_LAYOUT_BLD) return fail(SFM_ERR_SHAPE, "%s: unknown flags 0x%x", who, flags);
    if (io_dtype != SFM_F32 && io_dtype != SFM_BF16) return fail(SFM_ERR_DTYPE, "%s: io_dtype %d", who, io_dtype);
    if (!sane(B, 1 << 24) || !sane(D, 1 << 20) || !sane(T, 1 << 24))
        return fail(SFM_ERR_SHAPE, "%s: B=%lld D=%lld T=%lld out of range", who, (long long)B, (long long)D,
                    (long long)T);
    if (B * D * (T + 2) > (1LL << 40)) return fail(SFM_ERR_SHAPE, "%s: tensor too large", who);
    if (!aligned16(gpad) || !aligned16(gx)) return fail(SFM_ERR_ALIGN, "%s: io base pointers must be 16-byte aligned", who);
    const int eb = io_bytes(io_dtype);
    if (overlap(rng("gx", gx, B * D * T * eb), rng("gpad", gpad, B * D * (T + 2) * eb)))
        return fail(SFM_ERR_ALIAS, "%s: gx overlaps gpad", who);
    const bool cl = (flags & SFM_LAYOUT_BLD) != 0;
    return hip_status(sfm::launch_aux_pad_bwd(gpad, gx, cl ? B : B * D, T, io_dtype, static_cast<hipStream_t>(stream),
                                              cl ? D : 0),
                      who);
}

extern "C" sfm_status sfm_aux_pad_bwd(const void* gpad, void* gx, int64_t B, int64_t D, int64_t T, int io_dtype,
                                      void* stream) {
    return sfm_aux_pad_bwd_ex(gpad, gx, B, D, T, io_dtype, 0, stream);
}
