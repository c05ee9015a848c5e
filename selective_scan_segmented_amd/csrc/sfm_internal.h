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
    int mode;        // staging: 0 whole rows (16-byte DMA), 1 double-buffered tiles (4-byte DMA), 2 element loads
    int xrs, drs;    // LDS row strides (elements) of the x and delta/y stages
    int stages;      // mode 1: LDS stages per wave (2: the next chunk's transfers overlap this chunk)
    int wsplit;      // 1: each piece of a folded row is a workgroup of its own (no carries)
    int rb_rs;       // mode 1: row stride (elements) of a stage's raw B/C rows
    int rb_bytes;    // mode 1: bytes of one stage's raw B/C area (B rows, then C rows at rb_bytes / 2)
    int bc_wide;     // B/C blocks of whole samples are 16-byte aligned
    int bc_dma;      // mode 0: B/C of a sample arrive by direct transfer into a raw area, then widen in LDS
    int bcr_off;     // byte offset of that raw [2][N][L] io area inside the group's B/C region
    int xs_bytes, ds_bytes, bc_bytes, group_bytes, lds_bytes;
    // Staggered start (0 = off): when the whole grid is resident at once, the
    // workgroups of dispatch round r = blockIdx / stagger_period issue their
    // loads r * stagger_ticks (10 ns ticks) after they start.
    int stagger_period, stagger_ticks;
    // Lane-split kernels: only rounds r < stagger_rounds delay (the rounds
    // resident at launch); set by the launcher from the kernel's occupancy.
    int stagger_rounds;
    // Lane-split kernel (scan_split.h): split = G lanes per channel (0 = the
    // kernel above), wpg waves of 64/G channels per workgroup sharing one B/C
    // stage, stiles workgroups per folded row; LDS offsets of the float32
    // B/C rows, the raw B/C area and the first wave's x/delta slabs.
    int split, wpg, stiles;
    int bc_off, braw_off, mean_off, slab_off, slab_bytes;
    // Chunked lane-split kernel (sq > 0): x stays whole rows, delta/y and the
    // raw B/C of sq positions at a time by 4-byte transfers into LDS rows of
    // dpw / bpw words (odd pitches), dtile_insts / btile_insts transfers each.
    int sq, dpw, bpw, dtile_insts, btile_insts;
    // Streaming lane-split kernel (split = 16, one state per lane): x tiles too,
    // xpw words per row, xtile_insts transfers, every tile in two stages.
    int xpw, xtile_insts;
};

// Fills the plan fields; waves_hint / ch_hint <= 0 select automatically,
// stagger_hint < 0 selects automatically, 0 turns the staggered start off and
// > 0 sets the delay per dispatch round in 10 ns ticks.
// stages_hint (mode 1): 1 or 2 forces the LDS stages per wave, else automatic.
bool plan_scan(ScanParams& p, int io_bytes, int waves_hint, int ch_hint, int stagger_hint = -1, int stages_hint = 0,
               int split_hint = -1, int split_chunk_hint = -1);
// Compute units of the current device (256 when no device can be queried).
int device_cus();
hipError_t launch_scan(const ScanParams& p, int io_dtype, hipStream_t stream);
// per-(io type, state count) kernel sets, one translation unit each
hipError_t launch_scan_f32_n4(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_f32_n8(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_f32_n16(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_bf16_n4(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_bf16_n8(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_bf16_n16(const ScanParams& p, hipStream_t s);
// lane-split kernel sets (p.split = G), one translation unit each
hipError_t launch_split_f32_n4(const ScanParams& p, hipStream_t s);
hipError_t launch_split_f32_n8(const ScanParams& p, hipStream_t s);
hipError_t launch_split_f32_n16(const ScanParams& p, hipStream_t s);
hipError_t launch_split_bf16_n4(const ScanParams& p, hipStream_t s);
hipError_t launch_split_bf16_n8(const ScanParams& p, hipStream_t s);
hipError_t launch_split_bf16_n16(const ScanParams& p, hipStream_t s);

hipError_t launch_dwconv1d(const void* x, const float* w, const float* bias, void* out, int64_t B1, int64_t B2,
                           int64_t D, int64_t L, int K, int pad_left, int act, int io_dtype, hipStream_t stream);

hipError_t launch_aux_pad(const void* in, void* out, int64_t rows, int64_t T, int io_dtype, hipStream_t stream);
// [batch][R][C] -> [batch][C][R] for 2- or 4-byte elements (layout.hip)
hipError_t launch_transpose(const void* in, void* out, int64_t batch, int64_t R, int64_t C, int elem_bytes,
                            hipStream_t stream);
hipError_t launch_aux_swap(const void* in, void* out, int64_t rows, int64_t L, int io_dtype, hipStream_t stream);

}  // namespace sfm
