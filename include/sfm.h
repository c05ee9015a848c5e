/*
 * sfm.h -- C ABI of libsfm: the folded, segmented selective scan of SF-Mamba
 * and its companions, as hand-written HIP kernels for AMD Instinct MI355X
 * (gfx950).
 *
 * Plain C: extern "C", only pointers, integers and enums; no C++ exception and
 * no torch type crosses it.  Device pointers point to memory the CALLER owns:
 * the library never allocates, frees or keeps a reference to device memory.
 * The backward and the split-row forward (sfm_selective_scan_bwd,
 * sfm_selective_scan_fwd_ws) take a caller-owned workspace;
 * sfm_selective_scan_fwd_noalloc uses the library's static per-GPU scratch
 * array instead; every other entry point needs no device memory beyond its
 * inputs and outputs.  Every entry point that touches the GPU only
 * enqueues work on `stream` (a hipStream_t; NULL = the null stream) and
 * returns without synchronising: device faults surface at the caller's next
 * synchronisation.  Arguments are validated BEFORE any launch; a violation
 * returns a non-zero status, launches nothing, and leaves a description for
 * sfm_last_error() (thread-local).
 *
 * Page citations (the method has no published code; these web pages describe it):
 *  [SBW] "Seeing Both Ways, Running One Way" (sungsoo.github.io), section 3.1
 *        (selective SSM recurrence), 3.2 (aux head/tail tokens and their swap),
 *        3.3 (batch folding and the periodic state reset), 8.1 (method list).
 *  [TL]  "SF-Mamba：重新思考视觉 Mamba 的信息流与并行效率" (techloop.online),
 *        sections "第一个模块：Auxiliary Patch Swapping", "第二个模块：Batch
 *        Folding with Periodic State Reset" (incl. its conv-boundary part) and
 *        "还有一个工程补充：Adaptive B1".
 *  [GS]  "SF-Mamba: Rethinking State Space Model for Vision" (gist.science),
 *        Technische Zusammenfassung 2.B.
 *
 * Layout conventions (channel-first, as the pages write the tensors):
 *  - io tensors are C-contiguous; `io_dtype` says whether they hold float32 or
 *    bfloat16 (raw IEEE bfloat16 bits).  Base pointers of io tensors must be
 *    16-byte aligned (any tensor from a PyTorch allocation is).
 *  - parameter tensors (A, D, biases, conv weights) are float32, C-contiguous.
 *  - sample b of a batch of B = B1*B2 samples is the j-th segment of folded row
 *    b1 when b = b1*B2 + j ([SBW] 3.3 leaves the order open; any fixed order
 *    gives the same per-sample result).  The fold is never materialised.
 */
#ifndef SFM_H
#define SFM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SFM_OK = 0,
    SFM_ERR_NULL = 1,         /* a required pointer is NULL                        */
    SFM_ERR_SHAPE = 2,        /* a size is out of range or inconsistent            */
    SFM_ERR_DTYPE = 3,        /* io_dtype not one of sfm_dtype                     */
    SFM_ERR_UNSUPPORTED = 4,  /* valid request the library does not implement     */
    SFM_ERR_HIP = 5,          /* the HIP runtime reported an error at launch       */
    SFM_ERR_ALIAS = 6,        /* an output overlaps an input it must not overlap   */
    SFM_ERR_ALIGN = 7         /* an io base pointer is not 16-byte aligned         */
} sfm_status;

typedef enum { SFM_F32 = 0, SFM_BF16 = 1 } sfm_dtype;
typedef enum { SFM_ACT_NONE = 0, SFM_ACT_SILU = 1 } sfm_act;
typedef enum { SFM_AUX_PAD = 0, SFM_AUX_SWAP = 1 } sfm_aux_mode;

/* Largest state size and conv width the kernels are built for. */
#define SFM_MAX_N 16
#define SFM_MAX_K 8

/*
 * sfm_selective_scan_fwd -- selective scan over batch-folded rows with the
 * periodic state reset.  [SBW] 3.1: h_t = Abar_t h_{t-1} + Bbar_t x_t,
 * y_t = C_t h_t; [SBW] 3.3 / [TL] "第二个模块": the batch is folded into
 * B1 rows of length B2*L and Abar is zero at every sample start (t mod L == 0),
 * which keeps the samples independent ([GS] 2.B).  Discretization (zero-order
 * hold of Mamba): Abar = exp(Delta*A[d,n]), Bbar*x = Delta*B[b,n,t]*u[b,d,t];
 * Delta = softplus(delta + delta_bias[d]) (beta 1, threshold 20) when
 * delta_softplus != 0, else delta + delta_bias[d]; y += Dskip[d]*u.
 * The reset is applied as a state re-initialisation, so non-finite values in
 * one sample never reach another.
 *
 * Optional fused conv ([TL] conv-boundary part, [SBW] 8.1 item 5): when
 * conv_w != NULL, `u` holds the conv INPUT x and the scan uses
 *   u[b,d,t] = act(conv_b[d] + sum_{j<conv_k} conv_w[d,j] * x[b,d,t+j-conv_pad_left])
 * with taps outside the sample ([0, L)) reading zero; u stays in fp32 registers.
 *
 * Arguments (device pointers unless noted):
 *   u          [B1*B2, D, L] io   scan input, or the conv input if conv_w != NULL
 *   delta      [B1*B2, D, L] io   raw step input (before bias and softplus)
 *   A          [D, N] f32         state matrix diagonal (normally negative)
 *   Bm, Cm     [B1*B2, N, L] io   input and output projections, shared by all D
 *   Dskip      [D] f32 or NULL    skip weight (NULL = 0)
 *   delta_bias [D] f32 or NULL    (NULL = 0)
 *   delta_softplus                0 or 1
 *   conv_w     [D, conv_k] f32 or NULL (NULL = no fused conv)
 *   conv_b     [D] f32 or NULL
 *   conv_k     1..SFM_MAX_K (ignored without conv); conv_pad_left in [0, conv_k)
 *   conv_act   sfm_act
 *   y          [B1*B2, D, L] io   output; must not overlap any input
 *   B1, B2     folded rows and samples per row (B = B1*B2), >= 1
 *   D          channels >= 1;  N  state size 1..SFM_MAX_N;  L  per-sample length (T+2) >= 1
 *   io_dtype   sfm_dtype of u, delta, Bm, Cm and y
 *   stream     hipStream_t or NULL
 * Returns SFM_OK, or NULL/SHAPE/DTYPE/ALIAS/ALIGN (nothing launched) or HIP.
 *
 * Launch-plan overrides (environment, read on every call; for tuning and
 * tests, results do not depend on them beyond float32 summation order):
 *   SFM_SCAN_WAVES=w    pieces per folded row (carried state between pieces)
 *   SFM_SCAN_CHUNK=c    positions per LDS chunk (tiled staging)
 *   SFM_SCAN_STAGES=2   tiled staging double-buffered per wave (default one stage)
 *   SFM_SCAN_STAGGER=t  delay per dispatch round in 10 ns ticks (0 = off) for
 *                       grids that are resident all at once
 */
sfm_status sfm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* Bm,
                                  const void* Cm, const float* Dskip, const float* delta_bias,
                                  int delta_softplus, const float* conv_w, const float* conv_b,
                                  int conv_k, int conv_pad_left, int conv_act, void* y, int64_t B1,
                                  int64_t B2, int64_t D, int64_t N, int64_t L, int io_dtype, void* stream);

/*
 * sfm_selective_scan_fwd_ex -- sfm_selective_scan_fwd with the stage's aux-token
 * steps fused into the same launch ("Seeing Both Ways, Running One Way" 3.2;
 * techloop walkthrough "第一个模块"):
 *   flags & SFM_FUSE_PAD:  `u` is the UNPADDED [B1*B2, D, L-2] input of a stage's
 *       first Mamba layer; each row is extended in the kernel to
 *       [mean, x_1 .. x_T, mean] exactly as sfm_aux_pad_swap(PAD) would
 *       (float64 index-order mean, one rounding to the io type) before the conv
 *       and the scan read it.  L >= 3.
 *   flags & SFM_FUSE_SWAP: y is written with positions 0 and L-1 exchanged, as
 *       sfm_aux_pad_swap(SWAP) would leave it for the next layer.
 * Results are bit-identical to the unfused sequence pad -> scan -> swap.  With
 * either flag the launch keeps every sample inside one wave (no carried state),
 * so very long single-sample rows run with less parallelism.
 *   flags & SFM_LAYOUT_BLD: channel-last layout ("SF-Mamba" README and the
 *       pages' per-model choice of the faster of channel-first and channel-last):
 *       u, delta, y are [B1*B2, L, D] (u [B1*B2, L-2, D] with SFM_FUSE_PAD),
 *       Bm, Cm [B1*B2, L, N]; every element has the same value as in the
 *       channel-first call on the transposed tensors, bit for bit.  D times the
 *       io element size must be a multiple of 16 bytes (else SFM_ERR_SHAPE).
 *       Override (diagnostics): SFM_CL_CHUNK=w caps the positions staged at once.
 * Other arguments as sfm_selective_scan_fwd; flags = 0 is that function.
 */
#define SFM_FUSE_PAD 1
#define SFM_FUSE_SWAP 2
#define SFM_LAYOUT_BLD 4
sfm_status sfm_selective_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* Bm,
                                     const void* Cm, const float* Dskip, const float* delta_bias,
                                     int delta_softplus, const float* conv_w, const float* conv_b,
                                     int conv_k, int conv_pad_left, int conv_act, void* y, int64_t B1,
                                     int64_t B2, int64_t D, int64_t N, int64_t L, int io_dtype, int flags,
                                     void* stream);

/*
 * sfm_selective_scan_fwd_ws -- sfm_selective_scan_fwd_ex (same arguments, flags
 * and results within the parity tolerance) with a caller-owned device
 * workspace, for rows too long for the in-LDS carries: when samples times
 * 64-channel tiles give fewer than 1024 waves (channel-first only) and the
 * regular forward does not stream the rows (its streaming kernel takes long
 * rows of 9 to 16 states, faster and without a workspace), each sample
 * row is split along L into segments of at least 64 positions, one wave each,
 * in three launches -- the fused pad's float64 token sums per segment, a carry
 * pass (each segment's state reached from zero and the sum of its steps), and
 * the output pass (each segment composes the earlier segments' carries, the
 * recurrence being linear in its entering state with the segment's decay
 * product taken as exp2(A * summed steps), then writes its y).  Every other
 * shape, and any call whose workspace size below is 0, runs
 * sfm_selective_scan_fwd_ex itself (workspace unused, may be NULL).
 * workspace: device memory of at least sfm_selective_scan_fwd_ws_size() bytes
 *   (same sizes, conv_k -- 0 without conv --, io_dtype, flags), owned by the
 *   caller, not overlapping any tensor; it holds the carries [rows x tiles x
 *   segments][2 Np + 2][64] f32 and the token sums for the call's duration.
 * SFM_BWD_SEGMENTS=n (diagnostics) asks for n segments here too.
 * Returns SFM_OK, or NULL/SHAPE/DTYPE/ALIAS/ALIGN/UNSUPPORTED (nothing
 * launched), HIP.
 */
sfm_status sfm_selective_scan_fwd_ws(const void* u, const void* delta, const float* A, const void* Bm,
                                     const void* Cm, const float* Dskip, const float* delta_bias,
                                     int delta_softplus, const float* conv_w, const float* conv_b,
                                     int conv_k, int conv_pad_left, int conv_act, void* y, int64_t B1,
                                     int64_t B2, int64_t D, int64_t N, int64_t L, int io_dtype, int flags,
                                     void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes sfm_selective_scan_fwd_ws needs for these sizes (host only;
 * conv_k = 0 for no conv); 0 when the call runs the regular forward.
 * Returns SFM_OK or NULL/SHAPE/DTYPE. */
sfm_status sfm_selective_scan_fwd_ws_size(int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L,
                                          int conv_k, int io_dtype, int flags, int64_t* bytes);

/*
 * sfm_selective_scan_fwd_noalloc -- sfm_selective_scan_fwd_ws (same arguments
 * without the workspace, same kernels, bit-identical results) for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Where the split-row plan needs a
 * workspace, the call uses a static device array of SFM_NOALLOC_SCRATCH_BYTES
 * instead (one copy per GPU, held until the process ends); it calls no
 * allocator.  Rows that need more (sfm_selective_scan_fwd_ws_size above the
 * limit; 16 x 320 rows of 4002 positions and 8 states need 8.2 MiB) return
 * SFM_ERR_UNSUPPORTED with nothing launched.  Every call on one GPU shares that
 * GPU's array: calls that may overlap in time on one GPU (different streams)
 * race and must be serialised by the caller; nothing in it needs clearing
 * between calls (each call writes what it reads).  The first call on a device
 * resolves the array's device address (the runtime may load the library's
 * code object then): make one call before capturing a graph.
 * Returns as sfm_selective_scan_fwd_ws.
 */
#define SFM_NOALLOC_SCRATCH_BYTES (32LL << 20)
sfm_status sfm_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* Bm,
                                          const void* Cm, const float* Dskip, const float* delta_bias,
                                          int delta_softplus, const float* conv_w, const float* conv_b,
                                          int conv_k, int conv_pad_left, int conv_act, void* y, int64_t B1,
                                          int64_t B2, int64_t D, int64_t N, int64_t L, int io_dtype, int flags,
                                          void* stream);

/*
 * sfm_dwconv1d_fold -- boundary-masked depthwise conv1d over folded rows
 * ([TL] "第二个模块", conv-boundary part; [SBW] 8.1 item 5):
 *   out[b,d,t] = act(bias[d] + sum_{j<K} w[d,j] * x[b,d,t+j-pad_left]),
 * a tap counting only when it stays inside the same sample's segment of the
 * folded row (t+j-pad_left in [0, L)); otherwise it reads zero.
 *   x, out [B1*B2, D, L] io (out must not overlap x);  w [D, K] f32;
 *   bias [D] f32 or NULL;  K 1..SFM_MAX_K;  pad_left in [0, K);  act sfm_act.
 */
sfm_status sfm_dwconv1d_fold(const void* x, const float* w, const float* bias, void* out, int64_t B1,
                             int64_t B2, int64_t D, int64_t L, int K, int pad_left, int act, int io_dtype,
                             void* stream);

/*
 * sfm_selective_scan_bwd -- gradients of sfm_selective_scan_fwd_ex (same
 * arguments and flags) for an upstream gradient dy of its output.  The pages
 * give the forward only ([SBW] 3.3 and [TL] "第二个模块": the model is trained
 * end to end); this is the chain rule of that forward in reverse time, with the
 * reset cutting every gradient path between the samples of a folded row and
 * PyTorch's softplus threshold (derivative 1 above 20).
 *
 * Inputs as the forward (u is the conv input; unpadded [B, D, L-2] with
 * SFM_FUSE_PAD); dy [B1*B2, D, L] io is the gradient of the forward output y
 * (of the swapped y with SFM_FUSE_SWAP).  Outputs (device, overwritten):
 *   du          [B1*B2, D, L] io  gradient of the conv input in the PADDED layout
 *               (positions 0 and L-1 are the aux tokens with SFM_FUSE_PAD; pass
 *               it to sfm_aux_pad_bwd for the unpadded input's gradient)
 *   ddelta      [B1*B2, D, L] io
 *   dA          [D, N] f32;   dBm, dCm [B1*B2, N, L] f32 (summed over channels)
 *   dDskip, ddelta_bias [D] f32 or NULL (not computed)
 *   dconv_w     [D, conv_k] f32 (required with conv_w);  dconv_b [D] f32 or NULL
 * workspace: device memory of at least sfm_selective_scan_bwd_workspace_size()
 *   bytes (same B1, B2, D, N, L, conv_k -- 0 without conv -- io_dtype, flags),
 *   owned by the caller, not overlapping anything else; it holds float32 state
 *   checkpoints (every 32/Np positions, Np = N rounded up to 4, 8 or 16) and
 *   the partial sums of the f32 outputs for the duration of the call; its size
 *   depends on B1 and B2 only through B1*B2 (the backward runs one wave per
 *   sample and channel tile, whatever the fold).  The
 *   library allocates nothing.  The f32 sums are added in a fixed order by a
 *   second kernel (no atomics), so repeated calls give identical bits.
 * flags & SFM_LAYOUT_BLD: channel-last, as the forward: u, delta, dy, du,
 *   ddelta [B1*B2, L, D] (u [B1*B2, L-2, D] with SFM_FUSE_PAD), Bm, Cm, dBm, dCm
 *   [B1*B2, L, N]; D times the io element size must be a multiple of 16 bytes
 *   (else SHAPE).  Samples that fit the whole-sample kernel's LDS run it in the
 *   channel-last layout; longer ones run the channel-first chunked backward on
 *   transposed copies that the workspace then also holds (x, delta, dy, B, C
 *   in, du, ddelta, dB, dC out), with the results transposed back -- the same
 *   bits as a channel-first call on the transposed tensors.
 * Two kernels: when every [rows][length] block of a sample and 64-channel tile
 * is a whole number of 16-byte units on 16-byte boundaries and fits in LDS,
 * each sample is staged once; otherwise chunk by chunk.
 * The chunked kernel splits rows along L when samples times tiles give fewer
 * than 1024 waves: segments of at least 64 positions, one wave each, after a
 * carry pass (per segment: the state reached from zero, the output gradient
 * carried back from zero, the sum of the steps); each wave composes the carries
 * of the other segments of its row (the exact linear composition, its decay
 * product taken as exp2(A * summed steps)), and the conv-input gradient at the
 * positions around a segment boundary that the conv windows of both segments
 * reach is the sum of the two segments' partials.  The workspace then also
 * holds the carries, float64 token sums per segment (the row mean of
 * SFM_FUSE_PAD, added in segment order) and those partials.
 * Environment overrides (diagnostics): SFM_BWD_CHUNKED=1 forces the chunked
 * kernel for channel-first tensors; SFM_BWD_SEGMENTS=n asks the chunked kernel
 * for n segments per row (at most 64; at least the conv window per segment).
 * Both change the workspace size: query it with the same environment.
 * Returns SFM_OK, or NULL/SHAPE/DTYPE/ALIAS/ALIGN/UNSUPPORTED (nothing
 * launched), HIP.
 */
sfm_status sfm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* Bm,
                                  const void* Cm, const float* Dskip, const float* delta_bias,
                                  int delta_softplus, const float* conv_w, const float* conv_b,
                                  int conv_k, int conv_pad_left, int conv_act, const void* dy,
                                  void* du, void* ddelta, float* dA, float* dBm, float* dCm,
                                  float* dDskip, float* ddelta_bias, float* dconv_w, float* dconv_b,
                                  int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L, int io_dtype,
                                  int flags, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes sfm_selective_scan_bwd needs for these sizes (host only;
 * conv_k = 0 for no conv).  Returns SFM_OK or SHAPE/DTYPE/UNSUPPORTED. */
sfm_status sfm_selective_scan_bwd_workspace_size(int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L,
                                                 int conv_k, int io_dtype, int flags, int64_t* bytes);

/*
 * sfm_aux_pad_bwd -- gradient of the aux pad ([SBW] 3.2, [TL] "第一个模块"):
 * both end tokens are the row mean, so gx[b,d,i] = gpad[b,d,1+i] +
 * (gpad[b,d,0] + gpad[b,d,T+1]) / T.  gpad [B, D, T+2] io in, gx [B, D, T] io
 * out (must not overlap); float32 arithmetic, one rounding to io.
 */
sfm_status sfm_aux_pad_bwd(const void* gpad, void* gx, int64_t B, int64_t D, int64_t T, int io_dtype,
                           void* stream);

/* sfm_aux_pad_bwd with flags: SFM_LAYOUT_BLD takes gpad [B, T+2, D] and writes
 * gx [B, T, D] (the same arithmetic per element); flags = 0 is sfm_aux_pad_bwd. */
sfm_status sfm_aux_pad_bwd_ex(const void* gpad, void* gx, int64_t B, int64_t D, int64_t T, int io_dtype,
                              int flags, void* stream);

/*
 * sfm_aux_pad_swap -- the auxiliary head/tail tokens ([SBW] 3.2, [TL]
 * "第一个模块").
 *  mode SFM_AUX_PAD:  in [B, D, T] -> out [B, D, T+2]; out[..,0] = out[..,T+1] =
 *      mean over the T patch tokens (float64 sum in index order, divided by T,
 *      rounded once to the io type, ties to even); out[..,1+t] = in[..,t].
 *      out must not overlap in.  T >= 1.
 *  mode SFM_AUX_SWAP: in, out [B, D, T+2] with T here meaning L-2 (T >= -1 so
 *      L = T+2 >= 1): out = in with positions 0 and L-1 exchanged (the next
 *      layer's head is this layer's tail output and vice versa).  out == in
 *      performs the two-element exchange in place; otherwise out must not
 *      overlap in.
 * Bit-exact in both modes.
 */
sfm_status sfm_aux_pad_swap(const void* in, void* out, int64_t B, int64_t D, int64_t T, int mode,
                            int io_dtype, void* stream);

/*
 * sfm_pick_b1 -- adaptive fold ratio ([TL] "还有一个工程补充：Adaptive B1";
 * [SBW] 8.1 item 6): an offline lookup table keyed by batch size, sequence
 * length, channels and state size, here built by timing the scan on MI355X.
 * Host only (no device call).  Writes B1 (a divisor of B) to *B1_out.
 * Lookup: exact key, else the nearest key in (log2 B, log2 L, log2 D, N); the
 * table's B2 is then reduced to the largest divisor of B not above it.
 * The environment variable SFM_B1_TABLE may name a text file of lines
 * "B L D N B2" that is consulted before the built-in table.
 */
sfm_status sfm_pick_b1(int64_t B, int64_t L, int64_t D, int64_t N, int64_t* B1_out);

/*
 * sfm_scan_plan_string -- host-only diagnostic: writes (NUL-terminated,
 * truncated to `cap` bytes) the launch plan sfm_selective_scan_fwd would use
 * for these sizes -- staging mode, chunk length, pieces per folded row, channel
 * tiles per workgroup, LDS bytes, grid.  conv_k = 0 means no fused conv;
 * flags as for sfm_selective_scan_fwd_ex.
 * Returns SFM_ERR_SHAPE / SFM_ERR_UNSUPPORTED like the scan would.
 */
sfm_status sfm_scan_plan_string(int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L, int conv_k,
                                int io_dtype, int flags, char* buf, int64_t cap);

/* Static text for a status code. */
const char* sfm_status_string(sfm_status s);

/* Thread-local description of the last failure in this thread ("" if none). */
const char* sfm_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int sfm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SFM_H */
