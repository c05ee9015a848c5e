// sfm_cl.h -- host/device contract of the channel-last forward (scan_cl.hip) and
// the C-ABI layer.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfm {

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

}  // namespace sfm
