// sfm_internal.h -- host/device contract between the C-ABI layer (sfm_api.cpp)
// and the HIP kernels of libsfm.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfm {

// Launch description of one selective-scan call (see scan.hip for the mapping).
struct ScanParams {
    const void* u;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const float* dbias;
    const float* conv_w;
    const float* conv_b;
    void* y;
    int B1, B2, D, N, L;
    int K, P, act, softplus;
    int pad_in;      // u holds unpadded rows of L-2 tokens; the aux pad is fused
    int swap_out;    // y is written with positions 0 and L-1 exchanged
    int xrow;        // row length of the u tensor (L, or L-2 with pad_in)
    // plan (filled by plan_scan)
    int ns;          // compiled state count (4, 8 or 16) >= N
    int tiles;       // ceil(D / 64)
    int cw;          // channel tiles per workgroup sharing one B/C stage (waves per piece)
    int tgroups;     // ceil(tiles / cw)
    int waves;       // pieces per folded row (the workgroup has cw * waves waves)
    int piece;       // folded positions per wave
    int need_carry;  // 1 when some piece starts inside a sample
    int ch;          // positions per LDS chunk
    int mode;        // staging: 0 whole rows (16-byte DMA), 1 tiles (4-byte DMA), 2 element loads
    int xrs, drs;    // LDS row strides (elements) of the x and delta/y stages
    int bc_wide;     // B/C blocks of whole samples are 16-byte aligned
    int bc_dma;      // mode 0: B/C of a sample arrive by direct transfer into a raw area, then widen in LDS
    int bcr_off;     // byte offset of that raw [2][N][L] io area inside the group's B/C region
    int xs_bytes, ds_bytes, bc_bytes, group_bytes, lds_bytes;
    // Staggered start (0 = off): when the whole grid is resident at once, the
    // workgroups of dispatch round r = blockIdx / stagger_period issue their
    // loads r * stagger_ticks (10 ns ticks) after they start.
    int stagger_period, stagger_ticks;
};

// Launch description of one backward call (see bwd.hip).
struct BwdParams {
    const void* u;        // conv input x (unpadded with pad_in), or the scan input without conv
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const float* dbias;
    const float* conv_w;
    const float* conv_b;
    const void* dy;
    void* du;             // gradient of the (padded) conv input, [B, D, L] io
    void* ddelta;         // [B, D, L] io
    float* dA;            // [D, N]
    float* dBm;           // [B, N, L]
    float* dCm;           // [B, N, L]
    float* dDskip;        // [D] or null
    float* ddbias;        // [D] or null
    float* dconv_w;       // [D, K] or null
    float* dconv_b;       // [D] or null
    float* ws;            // workspace: checkpoints [B1 * tiles][nchk][ns][64], then the partial sums below
    int B1, B2, D, N, L;
    int K, P, act, softplus;
    int pad_in;           // u holds unpadded rows of L-2 tokens
    int swap_dy;          // dy is the gradient of the output with positions 0 and L-1 exchanged
    int xrow;             // row length of u
    // plan
    int ns, tiles, q, nchk;
    int whole;            // 1: whole-sample slabs staged once per sample; 0: chunk by chunk
    // partial sums in the workspace (offsets in floats), added up in a fixed order
    // by a second kernel: dB/dC per channel tile [tiles][B][L][2][ns] and the
    // per-channel sums per folded row [B1][kc][D], rows dA (N), dD, dbias [, dconv_b, dconv_w (K)]
    long long pbc_off, pch_off;
    int kc;
    int xs_off, ds_off, dys_off, bc_off, red_off, mean_off, braw_off, lds_bytes;
};

// Launch description of the channel-last forward (see scan_cl.hip): u, delta
// and y are [B, L, D] (u [B, L-2, D] with pad_in), B and C [B, L, N].
struct ClParams {
    const void* u;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const float* dbias;
    const float* conv_w;
    const float* conv_b;
    void* y;
    int B1, B2, D, N, L;
    int K, P, act, softplus;
    int pad_in, swap_out, xrow;
    // plan
    int ns, tiles, W, nchunk;  // positions per LDS chunk and chunks per sample
    int cw, tgroups;           // channel tiles (waves) per workgroup sharing the B/C stage; workgroups per row
    int xs_off, ds_off, wave_bytes, bc_off, lds_bytes;  // x and delta stages of wave w at + w * wave_bytes
    int stagger_period, stagger_ticks;  // staggered start by dispatch round, as ScanParams
};

// Channel-last planning (w_hint > 0 caps the chunk length); false when D rows
// are not whole 16-byte units.
bool plan_scan_cl(ClParams& p, int io_bytes, int w_hint);
hipError_t launch_scan_cl(const ClParams& p, int io_dtype, hipStream_t stream);

// Backward planning; returns false when no plan fits.  ws_bytes: workspace size.
bool plan_bwd(BwdParams& p, int io_bytes, size_t* ws_bytes);
hipError_t launch_bwd(const BwdParams& p, int io_dtype, hipStream_t stream);

// Fills the plan fields; waves_hint / ch_hint <= 0 select automatically,
// stagger_hint < 0 selects automatically, 0 turns the staggered start off and
// > 0 sets the delay per dispatch round in 10 ns ticks.
bool plan_scan(ScanParams& p, int io_bytes, int waves_hint, int ch_hint, int stagger_hint = -1);
hipError_t launch_scan(const ScanParams& p, int io_dtype, hipStream_t stream);
// per-(io type, state count) kernel sets, one translation unit each
hipError_t launch_scan_f32_n4(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_f32_n8(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_f32_n16(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_bf16_n4(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_bf16_n8(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_bf16_n16(const ScanParams& p, hipStream_t s);

hipError_t launch_dwconv1d(const void* x, const float* w, const float* bias, void* out, int64_t B1, int64_t B2,
                           int64_t D, int64_t L, int K, int pad_left, int act, int io_dtype, hipStream_t stream);

hipError_t launch_aux_pad(const void* in, void* out, int64_t rows, int64_t T, int io_dtype, hipStream_t stream);
hipError_t launch_aux_swap(const void* in, void* out, int64_t rows, int64_t L, int io_dtype, hipStream_t stream);
hipError_t launch_aux_pad_bwd(const void* gp, void* gx, int64_t rows, int64_t T, int io_dtype, hipStream_t stream);

}  // namespace sfm
