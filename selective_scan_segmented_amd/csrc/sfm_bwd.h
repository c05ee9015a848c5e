// sfm_bwd.h -- host/device contract of the backward kernels (bwd.hip, and the
// aux-pad gradient in aux.hip) and the C-ABI layer.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfm {

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
    int cl;               // channel-last tensors: u, delta, dy, du, ddelta [B, L, D]; B, C, dB, dC [B, L, N]
    // partial sums in the workspace (offsets in floats), added up in a fixed order
    // by a second kernel: dB/dC per channel tile [tiles][B][L][2][ns] and the
    // per-channel sums per folded row and segment [B1][seg][kc][D], rows dA (N), dD, dbias [, dconv_b, dconv_w (K)]
    long long pbc_off, pch_off;
    // chunked kernel split along L: each sample row is cut into `seg` segments of
    // `cps` chunks, one wave each.  A carry pass writes per segment wave (car_off)
    // the state reached from zero at its end [ns], the carried output gradient
    // reached from zero at its start [ns], and the two step sums (forward,
    // reverse) [2], each over 64 lanes; the fused pad's float64 token sums per
    // segment wave [64] (meanw_off); the conv-input gradient at the kw - 1 positions around each
    // segment boundary comes as two partials per segment wave [2][kw - 1][64]
    // (seam_off: the segment's leading and trailing ones) added by a seam kernel.
    int seg, cps, kw;
    long long car_off, meanw_off, seam_off;
    // forward through the split-row machinery (sfm_selective_scan_fwd_ws): the
    // carry pass's forward half, then a pass that writes y [B, D, L] io (ends
    // exchanged with swap_out); fwd = 1 drops the backward's outputs and regions
    int fwd;
    void* y;
    int swap_out;
    int kc;
    int xs_off, ds_off, dys_off, bc_off, red_off, mean_off, braw_off, lds_bytes;
    int hin_off;          // chunked kernel: a chunk's entering state [ns][64] f32, staged with the chunk
    int stage_bytes;      // chunked kernel: bytes of one staging buffer (x, delta, dy, raw B/C, state); two follow each other
};

// Backward planning; returns false when no plan fits.  ws_bytes: workspace size.
bool plan_bwd(BwdParams& p, int io_bytes, size_t* ws_bytes);
hipError_t launch_bwd(const BwdParams& p, int io_dtype, hipStream_t stream);
// The split-row forward (p.fwd = 1, planned with p.seg > 1): y only, no reduce.
hipError_t launch_fwd_split(const BwdParams& p, int io_dtype, hipStream_t stream);

// Gradient of the aux pad: channel-first rows [rows][T+2] -> [rows][T], or
// channel-last (channels > 0) [B][T+2][channels] -> [B][T][channels] with rows = B.
hipError_t launch_aux_pad_bwd(const void* gp, void* gx, int64_t rows, int64_t T, int io_dtype, hipStream_t stream,
                              int64_t channels = 0);

}  // namespace sfm
