/*
 * sparseconv.h -- C ABI of the MI355X (gfx950) sparse direct convolution library.
 *
 * What it computes.  Direct convolution of dense NCHW fp32 feature maps with an
 * unstructured-sparse filter bank, without lowering (no im2col) and without a dense
 * fallback.  For an image n, output channel m and output position (e, f):
 *
 *     Y[n,m,e,f] = sum over stored non-zeros (c, r, s, v) of row m of  v * X[n, c, iy, ix]
 *                  with iy = e*stride - pad + r, ix = f*stride - pad + s,
 *                  terms with (iy, ix) outside [0,H) x [0,W) omitted,
 *     E = (H + 2*pad - R) / stride + 1,  F = (W + 2*pad - S) / stride + 1.
 *
 * This is the multi-channel convolution of Tuteja et al., "Theoretical and Empirical
 * Analysis of Sparse Convolution", Sec. 3 Eq. (1)-(3) (sum clipped to the image, sparse
 * form over the non-zeros N(oc,h,w), output size Eq. (2)), read with a stride in both
 * axes.  There is no bias and no activation.  The filter bank is the M x (C*R*S) matrix
 * of "Escoin: Efficient Sparse Convolutional Neural Network Inference on GPUs" (lowering
 * section), column index col = c*R*S + r*S + s, stored row by row in CSR form
 * (value / colidx / rowptr, CSR section of the same page).  Packing turns every column
 * index into the input offset of the layout function f(c,r,s) = (c*H + r)*W + s of the
 * UNPADDED input ("weight stretching", same page) and keeps each row's entries contiguous
 * as {offset, value} pairs, so that one load returns everything a non-zero needs (the
 * packed-weight idea of Tuteja et al., Sec. 5.3).
 *
 * Conventions.
 *  - Plain C: fixed-width integers, pointers and sizes.  No exception crosses this ABI.
 *  - "host" pointers are read only during the call and never retained.
 *  - "device" pointers are HIP device allocations on the current device.
 *  - Every entry point returns sc_status; sparseconv_last_error() describes the last
 *    failure of the calling thread.
 *  - All argument checks happen before any device work: on error nothing is written.
 */
#ifndef SPARSECONV_H
#define SPARSECONV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sc_handle sc_handle; /* opaque packed filter bank, immutable after pack */

typedef enum {
  SC_OK = 0,
  SC_EINVAL = 1,       /* null pointer, malformed CSR, overlapping buffers, bad flag */
  SC_ESHAPE = 2,       /* a dimension is <= 0, E or F <= 0, or forward dims differ from the handle */
  SC_ENOMEM = 3,       /* host or device allocation failed */
  SC_EDEVICE = 4,      /* a HIP runtime call or kernel launch failed (incl. no device) */
  SC_EUNSUPPORTED = 5  /* size outside the documented limits below */
} sc_status;

typedef enum {
  SC_WEIGHTS_DENSE = 0, /* values: M*C*R*S fp32, (m,c,r,s) row-major; optional mask */
  SC_WEIGHTS_CSR = 1    /* values/colidx: nnz entries; rowptr: M+1 entries */
} sc_weights_format;

/* Pack flags. */
#define SC_PACK_HOST_ONLY 1u /* build the packed form on the host only: query and export
                                work, forward returns SC_EINVAL.  Needs no GPU. */
#define SC_PACK_ALL_TAPS 2u  /* DENSE weights only: store every filter position, zeros
                                included (mask ignored).  A forward on such a handle is the
                                dense direct convolution with the same kernel: the on-GPU
                                baseline, counterpart of Tuteja et al., Sec. 4 Eq. (5)/(6). */
#define SC_PACK_FP16_WORD 4u /* store each non-zero in the 32-bit packed word of Tuteja et al.,
                                Sec. 5.3 and Fig. 4: the weight rounded to fp16 (to nearest,
                                ties to even) in bits 31-16, the input channel in bits 15-8,
                                the filter column s (px) in bits 7-4 and the filter row r (py)
                                in bits 3-0 (sparseconv_export_words returns them).  The kernel
                                stream then takes 4 bytes per non-zero instead of 8; the fp16
                                weight is widened to fp32 and accumulated in fp32, so the
                                result is the convolution with the fp16-rounded weights.
                                Limits: C <= 256, R <= 16, S <= 16 (SC_EUNSUPPORTED); a finite
                                weight of magnitude >= 65520 (which rounds to infinity) is
                                SC_EINVAL. */
#define SC_PACK_ESCOIN_MAP 8u /* second mapping, for comparison: the dataflow of "Escoin:
                                Efficient Sparse Convolutional Neural Network Inference on
                                GPUs" (dataflow and data-placement sections).  A pad_in
                                kernel writes the zero-padded input to a caller-provided
                                workspace; then one workgroup per output channel (and tile of
                                output positions and image) keeps its CSR row, stretched
                                against the padded pitch ((c*(H+2pad) + r)*(W+2pad) + s), in
                                LDS and reads the padded input through the caches, one output
                                position per thread at a time.  Same result bar as the default
                                mapping.  Such a handle runs only through
                                sparseconv_forward_workspace (or sparseconv_forward_noalloc,
                                within its static workspace).  Not combinable with
                                SC_PACK_FP16_WORD (SC_EINVAL).  Limit: C*(H+2pad)*(W+2pad) <
                                2^30 (SC_EUNSUPPORTED). */

#define SC_PACK_LDS_TILE 16u  /* use the LDS-tile kernel for fp32 weights instead of the default
                                weights-in-code kernel (below).  Not combinable with
                                SC_PACK_ESCOIN_MAP (SC_EINVAL). */
/*
 * Default mapping for fp32 weights (no SC_PACK_LDS_TILE, SC_PACK_ESCOIN_MAP, SC_PACK_FP16_WORD
 * or SC_PACK_ALL_TAPS): the weights-in-code kernel.  Pack writes the layer's non-zeros into
 * the instruction stream of a gfx950 kernel generated for this layer (one FMA with the weight
 * as a 32-bit literal per non-zero; the output channel's accumulator register and the filter
 * tap's input register fixed in the instruction), assembles it in-process (amd_comgr) and
 * loads it on the current device (hipModuleLoadData).  A wavefront holds the accumulators of
 * all output channels of one group for 64 - (S-1)/stride consecutive output positions and
 * reads each input row vector once for all of them (Tuteja et al., Sec. 5.1: one input region,
 * reused by every output channel).  The stretched offsets of "Escoin" (weight stretching)
 * appear as the channel's scalar offset c*H*W plus the row vector's lane offset r*W + s.
 * sc_info.mapping is 2 for such handles and bake_* describe the kernel;
 * sparseconv_export_kernel_source returns its assembly.  If the layer does not fit the
 * mapping (too many output channels per group for the registers), pack uses the LDS-tile
 * kernel; a batch whose input or output exceeds 2^31 bytes runs on the LDS-tile kernel too.
 */

typedef struct {
  int32_t format;          /* sc_weights_format */
  const float* values;     /* host.  DENSE: M*C*R*S values.  CSR: nnz values (row order) */
  const int32_t* colidx;   /* host.  CSR only: nnz column indices, 0 <= col < C*R*S,
                              no duplicate within a row (any order within a row) */
  const int32_t* rowptr;   /* host.  CSR only: M+1 entries, rowptr[0] = 0, non-decreasing,
                              rowptr[M] = nnz */
  const uint8_t* mask;     /* host.  DENSE only, optional M*C*R*S bytes: a position is a
                              stored non-zero iff mask != 0 (explicit zero values kept).
                              NULL: a position is stored iff its value != 0.0f
                              (so -0.0 is dropped and NaN kept). */
} sc_weights;

typedef struct {
  int32_t M, C, R, S, H, W, stride, pad, E, F;
  int64_t nnz;
  int64_t packed_bytes;  /* (2*nnz + M + 1) * 4: canonical {offset, value} entries + rowptr,
                            the CSR size of "Escoin", CSR section; (nnz + M + 1) * 4 with
                            SC_PACK_FP16_WORD (one 32-bit word per non-zero + rowptr) */
  int64_t device_bytes;  /* bytes this handle holds on the device (kernel stream + tables) */
  int32_t tile_pixels;   /* launch plan: extended output positions per workgroup */
  int32_t rows_per_wave; /* launch plan: output-channel slots per wavefront */
  int32_t row_groups;    /* launch plan: workgroups sharing one tile (output-channel groups) */
  int32_t chunk_channels;/* launch plan: input channels staged in LDS at a time */
  int32_t lds_bytes;     /* launch plan: dynamic LDS per workgroup */
  int32_t max_wave_nnz;  /* largest non-zero count given to one wavefront */
  int32_t waves_per_group;  /* launch plan: computing wavefronts per workgroup (one more
                               wavefront copies the input into LDS) */
  int32_t pipeline_depth;   /* launch plan: LDS ring slots (up to depth-1 chunks staged
                               ahead of the one being computed) */
  int32_t step_balance_permille; /* 1000 * (sum over chunks of the busiest wavefront's
                                    non-zero entries) / (sum of the means): the cost of
                                    synchronising the wavefronts once per chunk (>= 1000) */
  int32_t split_pieces;  /* rows longer than a wavefront's fair share are split into pieces
                            held by different wavefronts and summed in a fixed order at the
                            end of a work unit: the number of pieces beyond the first */
  int32_t plan_variants; /* launch plans the handle holds.  The fields above describe the
                            default one (most positions per workgroup); the others have fewer
                            positions per workgroup or fewer rows per wavefront, i.e. more
                            work units, or (8-byte entries only) hold four consecutive
                            positions per lane read with 16-byte LDS reads (504 positions per
                            workgroup), and the forward pass takes the one estimated fastest
                            for its N (small batches and small images use more, smaller
                            units so that every CU has work; denser filters the quad plan) */
  int32_t entry_bytes;   /* bytes per non-zero in the kernel stream: 8 ({LDS offset, fp32
                            weight}), or 4 ({LDS offset, fp16 weight}) with SC_PACK_FP16_WORD */
  int32_t mapping;       /* 0: LDS-tile kernel (the plan fields above); 1: SC_PACK_ESCOIN_MAP
                            (tile_pixels = output positions per workgroup, lds_bytes = its
                            row buffer, max_wave_nnz = the longest row); 2: weights-in-code
                            kernel (the bake_* fields; the plan fields above then describe
                            the handle's LDS-tile plans, used only for batches too large for
                            the weights-in-code kernel) */
  /* weights-in-code kernels (mapping 2): the handle holds a base kernel (described here)
     and variants that give small batches more wavefronts; sparseconv_launch_info tells
     which one a forward of N images launches */
  int32_t bake_groups;      /* output-channel groups; a wavefront holds one group's accumulators */
  int32_t bake_splits;      /* channel splits: wavefronts sharing a unit's input channels, whose
                               partial sums are added in LDS in split order */
  int32_t bake_units_per_wg;/* units (wavefront tile x group) per workgroup */
  int32_t bake_valid_lanes; /* output positions per wavefront, 64 - (S-1)/stride */
  int32_t bake_pitch;       /* extended row pitch F + (S-1)/stride */
  int32_t bake_depth;       /* filter-row steps of input loads in flight */
  int32_t bake_vgprs;       /* VGPRs per lane */
  int32_t bake_lds_bytes;   /* LDS per workgroup (partial sums of the channel splits) */
  int32_t bake_variants;    /* weights-in-code kernels the handle holds */
  int32_t bake_stage;       /* 1: the base kernel stages input rows in LDS (chunks of
                               bake_chunk_channels channels, bake_buffers chunk buffers, the
                               copy running bake_buffers - 1 chunks ahead); 0: it loads them
                               into registers */
  int32_t bake_chunk_channels;
  int32_t bake_buffers;
  int32_t bake_sequential;  /* 1: each workgroup runs every group in turn (the stores of one
                               group overlap the next group's work); 0: one group per workgroup */
  int32_t bake_shared_window; /* 1: a workgroup holds every group's wavefronts for its tiles,
                                 which stage one input window together */
  int64_t bake_code_bytes;  /* bytes of generated code of the base kernel */
} sc_info;

/* The kernel a forward of N images launches (filled by sparseconv_launch_info). */
typedef struct {
  int32_t mapping;       /* 0 LDS-tile kernel, 1 "Escoin" mapping, 2 weights-in-code kernel */
  int32_t variant;       /* index of the plan among the handle's plans of that mapping */
  int64_t grid;          /* workgroups of the (main) launch */
  int64_t waves;         /* wavefronts of the (main) launch */
  int64_t pre_grid;      /* "Escoin" mapping: workgroups of its pad_in launch (else 0) */
  int32_t block;         /* threads per workgroup */
  int32_t lds_bytes;     /* LDS per workgroup */
  int32_t vgprs;         /* weights-in-code: VGPRs per lane */
  int32_t groups;        /* weights-in-code: output-channel groups; LDS-tile: row groups */
  int32_t splits;        /* weights-in-code: channel splits */
  int32_t units_per_wg;  /* weights-in-code: units per workgroup */
  int32_t depth;         /* weights-in-code: load steps in flight */
  int32_t valid_lanes;   /* weights-in-code: output positions per wavefront */
  int32_t tile_pixels;   /* LDS-tile and staged weights-in-code: positions per work unit */
  int32_t rows_per_wave; /* LDS-tile: output-channel slots per wavefront */
  int32_t chunk_channels;/* LDS-tile and staged weights-in-code: input channels per staged chunk */
  int32_t quad;          /* LDS-tile: 1 for a quad plan (16-byte LDS reads) */
  int32_t stage;         /* weights-in-code: 1 when the kernel stages input windows in LDS */
} sc_launch;

/*
 * Pack a filter bank for one layer geometry (once per layer; weights then stay resident).
 *   w          host description of the weights (see sc_weights).
 *   M,C,R,S    output channels, input channels, filter rows, filter columns (all >= 1).
 *   H,W        unpadded input height and width the layer will be applied to (>= 1).
 *   stride>=1, pad>=0; E and F from the formula above must be >= 1.
 *   flags      0, or any of SC_PACK_HOST_ONLY, SC_PACK_ALL_TAPS, SC_PACK_FP16_WORD,
 *              SC_PACK_ESCOIN_MAP (see each flag for the combinations it rejects).
 *   out        receives the new handle (set to NULL on failure).
 * Steps: validate -> CSR (columns sorted within each row, values moved with them) ->
 * stretched offsets -> wavefront schedule balanced by non-zero count -> upload.
 * Limits (SC_EUNSUPPORTED): C*H*W < 2^32 (offsets are u32), M*C*R*S < 2^31,
 * nnz < 2^31.  Errors: SC_EINVAL (null w/out/arrays, malformed CSR, unknown format/flag),
 * SC_ESHAPE, SC_ENOMEM, SC_EDEVICE.
 * The handle owns its device buffers (hipMalloc on the device current at pack time).
 */
sc_status sparseconv_pack(const sc_weights* w, int32_t M, int32_t C, int32_t R, int32_t S,
                          int32_t H, int32_t W, int32_t stride, int32_t pad, uint32_t flags,
                          sc_handle** out);

/*
 * Forward pass: output = conv(input, packed filters), overwriting the whole output.
 *   h         handle from sparseconv_pack (device-resident, not SC_PACK_HOST_ONLY).
 *   input     device, N*C*H*W fp32, NCHW contiguous, 4-byte aligned.
 *   output    device, N*M*E*F fp32, NCHW contiguous; must not overlap input.
 *   N >= 0 (0 is a no-op); C,H,W,M,R,S,stride,pad must equal the handle's.
 *   hip_stream  hipStream_t to launch on (NULL: the default stream).
 * Asynchronous: returns after the launch; nothing is synchronised.  The handle is never
 * written, so forwards on several streams may run at once.  Limits (SC_EUNSUPPORTED):
 * N*C*H*W < 2^31 and N*M*E*F < 2^31 elements.  Errors: SC_EINVAL (null handle or
 * pointers, host-only handle, overlap, a handle packed with SC_PACK_ESCOIN_MAP), SC_ESHAPE
 * (dims differ from the handle), SC_EDEVICE (launch failure).
 */
sc_status sparseconv_forward(const sc_handle* h, const float* input, float* output, int32_t N,
                             int32_t C, int32_t H, int32_t W, int32_t M, int32_t R, int32_t S,
                             int32_t stride, int32_t pad, void* hip_stream);

/*
 * Device workspace a forward of N images needs, in bytes (*bytes; 0 if none).  Handles
 * packed with SC_PACK_ESCOIN_MAP need N*C*(H+2pad)*(W+2pad)*4 bytes (rounded up to 256) for
 * the padded input; all others need none.  SC_EINVAL on a NULL handle or bytes, SC_ESHAPE
 * for N < 0.
 */
sc_status sparseconv_workspace_size(const sc_handle* h, int32_t N, int64_t* bytes);

/*
 * Forward pass with a caller-owned device workspace (the same contract as sparseconv_forward
 * otherwise).  workspace: device, at least sparseconv_workspace_size(h, N) bytes, 4-byte
 * aligned, overlapping neither input nor output (it may be NULL when that size is 0);
 * its contents are scratch, overwritten by the call, and two calls that share a workspace
 * must not run at the same time.  Required for SC_PACK_ESCOIN_MAP handles; for others the
 * workspace is not touched.  Errors as sparseconv_forward, plus SC_EINVAL for a missing,
 * small, misaligned or overlapping workspace.  Limits (SC_EUNSUPPORTED) as
 * sparseconv_forward, plus N*C*ceil((H+2pad)*(W+2pad)/256) and N*M*ceil(E*F/1024) below 2^31.
 */
sc_status sparseconv_forward_workspace(const sc_handle* h, const float* input, float* output,
                                       int32_t N, int32_t C, int32_t H, int32_t W, int32_t M,
                                       int32_t R, int32_t S, int32_t stride, int32_t pad,
                                       void* workspace, int64_t workspace_bytes, void* hip_stream);

/*
 * Forward pass that allocates nothing, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The contract
 * of sparseconv_forward_workspace, with the workspace taken from a static device array of the
 * library instead of the caller (SC_NOALLOC_SCRATCH_BYTES, 256-byte aligned, one copy per GPU,
 * held from the library's first use of that GPU until the process ends).  Handles packed with
 * SC_PACK_ESCOIN_MAP keep the padded input there; a batch that needs more than
 * SC_NOALLOC_SCRATCH_BYTES (sparseconv_workspace_size) is rejected with SC_EUNSUPPORTED before
 * anything is launched (use sparseconv_forward_workspace for it).  Other handles need no
 * workspace and behave exactly as with sparseconv_forward.  The array's address on a device is
 * resolved once (hipGetSymbolAddress) when an SC_PACK_ESCOIN_MAP handle is packed there, or
 * else at the first call on that device.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (each call rewrites all of the array it reads): two calls
 * that overlap in time on one GPU (several streams, or host threads without ordering) race
 * and may give wrong outputs; keep them on one stream.  Errors as sparseconv_forward_workspace,
 * plus SC_EUNSUPPORTED for a batch beyond the array and SC_EDEVICE if its address cannot be
 * resolved.
 */
#define SC_NOALLOC_SCRATCH_BYTES (32LL * 1024 * 1024)
sc_status sparseconv_forward_noalloc(const sc_handle* h, const float* input, float* output, int32_t N,
                                     int32_t C, int32_t H, int32_t W, int32_t M, int32_t R, int32_t S,
                                     int32_t stride, int32_t pad, void* hip_stream);

/* Fill *info with the handle's geometry, sizes and launch plan.  SC_EINVAL on NULL. */
sc_status sparseconv_query(const sc_handle* h, sc_info* info);

/*
 * Copy out the canonical packed form (host buffers owned by the caller):
 *   rowptr  M+1 entries; offsets, values  nnz entries each.
 * Canonical order: rows m ascending; within a row, columns c*R*S + r*S + s ascending.
 * offsets[j] = c*H*W + r*W + s of entry j; values[j] its fp32 weight, bit for bit (with
 * SC_PACK_FP16_WORD: the fp16-rounded weight the kernel uses, widened to fp32 exactly).
 * Any of the three pointers may be NULL to skip it.  SC_EINVAL on a NULL handle.
 */
sc_status sparseconv_export_packed(const sc_handle* h, int32_t* rowptr, uint32_t* offsets,
                                   float* values);

/*
 * Copy out the 32-bit packed words of a handle packed with SC_PACK_FP16_WORD (Tuteja et
 * al., Sec. 5.3 and Fig. 4), in the canonical order above (host buffers owned by the
 * caller): rowptr  M+1 entries (the per-output-channel start/end array of that section);
 * words  nnz entries, words[j] = fp16(v) << 16 | c << 8 | s << 4 | r.  Either pointer may
 * be NULL.  SC_EINVAL on a NULL handle or one packed without SC_PACK_FP16_WORD.
 */
sc_status sparseconv_export_words(const sc_handle* h, int32_t* rowptr, uint32_t* words);

/*
 * Read the handle's device status word into *status (host), and with clear != 0 reset it to
 * 0.  Bit 0 set: in some launch of the LDS-tile kernel on this handle since the last clear, a
 * wavefront's bounded wait on a counter in LDS gave up (after about 2^22 sleeps, far beyond
 * any real wait): that launch's output may be wrong.  The kernel never hangs on such a
 * failure; this word is how it is reported.  The weights-in-code and "Escoin" kernels have no
 * such waits.  Reads device memory with a blocking copy: synchronise the streams that ran
 * forwards on this handle first.  SC_EINVAL on a NULL handle or status, or a host-only
 * handle; SC_EDEVICE if the copy fails.
 */
sc_status sparseconv_device_status(const sc_handle* h, uint32_t* status, int32_t clear);

/*
 * Choose, by measurement, the kernel later forwards of N >= 1 images launch on this handle (as a
 * library's "find" step does): every kernel the handle holds for such a batch (the
 * weights-in-code kernels of its plans, or its LDS-tile plans) runs reps + 1 times on the
 * caller's input and output on hip_stream, the fastest average over the last reps wins and is
 * recorded for N, and *chosen (may be NULL) receives its index (sc_launch.variant).  Arguments as
 * sparseconv_forward, plus 1 <= reps <= 1000.  Blocking: synchronises hip_stream; not for use
 * under stream capture.  The output holds the chosen kernel's result afterwards.  Handles
 * packed with SC_PACK_ESCOIN_MAP hold a single kernel: the call only sets *chosen = 0.  A forward running at the same time on another
 * thread launches the previous or the new choice; either computes the same convolution.
 * Errors as sparseconv_forward, plus SC_EINVAL for reps out of range and SC_EDEVICE if timing
 * fails.
 */
sc_status sparseconv_tune(sc_handle* h, const float* input, float* output, int32_t N, int32_t C, int32_t H,
                          int32_t W, int32_t M, int32_t R, int32_t S, int32_t stride, int32_t pad, int32_t reps,
                          void* hip_stream, int32_t* chosen);

/*
 * Describe the launch a forward of N >= 1 images would make on this handle (the kernel
 * sparseconv_tune chose for N, else the one the forward's cost estimate picks), without
 * launching anything.  SC_EINVAL on a NULL
 * handle or out, SC_ESHAPE for N < 1.
 */
sc_status sparseconv_launch_info(const sc_handle* h, int32_t N, sc_launch* out);

/*
 * Copy out the assembly of the handle's (base) weights-in-code kernel (for inspection and the CPU
 * checks of the generated code): *len receives its length plus one; up to cap - 1 bytes and
 * a terminating NUL are written to buf (host, owned by the caller; may be NULL to query the
 * length).  SC_EINVAL on a NULL handle or len, or a handle without such a kernel (the message
 * says why the layer was not baked).
 */
sc_status sparseconv_export_kernel_source(const sc_handle* h, char* buf, int64_t cap, int64_t* len);

/*
 * Dense direct convolution baseline: the same output as a handle holding every tap, computed
 * from a dense weight tensor already on the device, with no packing and no handle.  Every
 * term of the sum above is evaluated, zero weights included: the dense work and traffic of
 * Tuteja et al., Sec. 4 Eq. (5)/(6) (2*N*E*F*M*C*R*S flops), the baseline their Sec. 6.1 /
 * Fig. 5 compare the sparse kernel with, here on the same GPU.
 *   w_dense_dev  device, M*C*R*S fp32, (m, c, r, s) row-major, 4-byte aligned; read only.
 *   input        device, N*C*H*W fp32, NCHW contiguous, 4-byte aligned.
 *   output       device, N*M*E*F fp32, NCHW contiguous, overwritten; must overlap neither
 *                input nor w_dense_dev.
 *   N >= 0 (0 is a no-op); M,C,R,S,H,W >= 1, stride >= 1, pad >= 0, E and F >= 1.
 *   hip_stream   hipStream_t to launch on (NULL: the default stream), on the current device.
 * Asynchronous, like sparseconv_forward.  Summation order per output: filter rows, then input
 * channels, then filter columns (it differs from the sparse kernels' order, so results agree
 * to rounding, not bit for bit).  Limits (SC_EUNSUPPORTED): N*C*H*W*4 and N*M*E*F*4 below
 * 2^31 bytes, M*C*R*S < 2^31.  Errors: SC_EINVAL (null or misaligned pointers, overlap),
 * SC_ESHAPE (a dimension out of range, E or F < 1), SC_EDEVICE (launch failure).
 */
sc_status sparseconv_dense_forward(const float* w_dense_dev, const float* input, float* output, int32_t N,
                                   int32_t C, int32_t H, int32_t W, int32_t M, int32_t R, int32_t S,
                                   int32_t stride, int32_t pad, void* hip_stream);

/* Free the handle and its device buffers.  NULL, or a pointer that is not a live handle
 * (already destroyed, or never returned by sparseconv_pack), is ignored: the library keeps a
 * registry of live handles, and every entry point reports SC_EINVAL ("invalid or destroyed
 * handle") for a pointer not in it.  Must not race a forward still running on the device that
 * reads this handle (synchronise the stream first). */
void sparseconv_destroy(sc_handle* h);

/* Message of the calling thread's last failure ("" if none).  Valid until that thread's
 * next call into the library. */
const char* sparseconv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSECONV_H */
