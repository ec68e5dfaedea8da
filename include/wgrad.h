/*
 * wgrad.h -- C ABI of the MI355X (gfx950) grouped convolution
 * backward-weight library (libwgrad.so).
 *
 * Operation (Composable Kernel page "grouped_convolution_backward_weight_
 * kernel.hpp": the 1D NWGC/GKXC/NWGK, 2D NHWGC/GKYXC/NHWGK and 3D
 * NDHWGC/GKZYXC/NDHWGK argument constructors, their group strides, and the
 * comment in operator() that the kernel forms the weight gradient from the
 * output gradient and the input), written here for 3D:
 *
 *   dW[g,k,z,y,x,c] = sum_{n,do,ho,wo} [0<=di<Di, 0<=hi<Hi, 0<=wi<Wi]
 *                       dY[n,do,ho,wo,g,k] * X[n,di,hi,wi,g,c]
 *   di = do*stride_d - pad_lo_d + z*dilation_d   (likewise hi with y, wi with x)
 *
 * 2D drops the d axis (Di = Do = Z = 1), 1D the h axis as well. Computed as
 * a batched-over-groups implicit GEMM with M = K/G, N = (C/G)*Z*Y*X and a
 * reduction of length N*Do*Ho*Wo. The pad_hi values only size the output:
 * Ho = floor((Hi + pad_lo + pad_hi - dilation*(Y-1) - 1)/stride) + 1, and so on.
 *
 * Layouts (all dense, row-major, innermost index last):
 *   X  : [N][Di][Hi][Wi][C]    (2D: [N][Hi][Wi][C], 1D: [N][Wi][C])   C = G*(C/G), group-major
 *   dY : [N][Do][Ho][Wo][K]    (2D: [N][Ho][Wo][K], 1D: [N][Wo][K])   K = G*(K/G), group-major
 *   dW : [K][Z][Y][X][C/G]     (2D: [K][Y][X][C/G], 1D: [K][X][C/G])  i.e. GKZYXC
 * X and dY share one 16-bit element type (bf16 or fp16); dW is that type or
 * fp32. A torch tensor [N,C,H,W] (or [N,C,D,H,W]) in channels_last memory
 * order is exactly X; a grouped conv weight [K, C/G, (Z,) Y, X] in
 * channels_last is exactly dW.
 *
 * Ownership: the caller owns every device buffer and the stream. The library
 * allocates no device memory; a plan owns only host memory.
 *
 * Errors: every entry point returns a wgrad_status. WGRAD_OK is 0. On error
 * nothing is enqueued and wgrad_last_error() returns a reason string for the
 * calling thread. No C++ exception crosses this boundary.
 */
#ifndef WGRAD_H
#define WGRAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WGRAD_BF16 = 0,
    WGRAD_FP16 = 1,
    WGRAD_FP32 = 2  /* output only */
} wgrad_dtype;

typedef enum {
    WGRAD_OK = 0,
    WGRAD_ERR_INVALID_ARG = 1, /* bad shape, pointer, alignment or size */
    WGRAD_ERR_UNSUPPORTED = 2, /* valid problem, but an override asks for something the kernels cannot do */
    WGRAD_ERR_HIP = 3          /* a HIP runtime call or launch failed; the reason names it */
} wgrad_status;

/* The problem. C and K are totals over all G groups and must be multiples
 * of G. Each array holds the problem's ndim axes outermost first: ndim 3
 * uses [0] = d, [1] = h, [2] = w; ndim 2 uses [0] = h, [1] = w; ndim 1 uses
 * [0] = w; unused entries are ignored. Lengths, strides and dilations are
 * >= 1, pads >= 0. N may be 0 (dW is then all zeros). */
typedef struct {
    int32_t ndim;       /* 1, 2 or 3 */
    int32_t in_dtype;   /* wgrad_dtype of X and dY: BF16 or FP16 */
    int32_t out_dtype;  /* wgrad_dtype of dW: in_dtype or FP32 */
    int32_t reserved;   /* must be 0 */
    int64_t G, N, C, K;
    int64_t in_len[3];
    int64_t filt_len[3];
    int64_t stride[3];
    int64_t dilation[3];
    int64_t pad_lo[3];
    int64_t pad_hi[3];
} wgrad_problem;

/* Kernel families a plan can use. */
typedef enum {
    WGRAD_VARIANT_AUTO = 0,
    WGRAD_VARIANT_MFMA = 1,      /* MFMA implicit GEMM over flat K tiles, any shape, optional group merge */
    WGRAD_VARIANT_DEPTHWISE = 2, /* C/G = K/G = 1: channel-vector direct kernel */
    WGRAD_VARIANT_ROWSLAB = 3,   /* MFMA implicit GEMM over slabs of output rows, X staged once per
                                    row (channel runs multiple of 32), optional group merge. Two forms:
                                    one filter row per workgroup (filter width 1, 3 or 5, w-dilation
                                    1), or, for 2D 3x3 filters with dilation 1, h-stride <= 3,
                                    w-stride <= 2 and output rows up to 62 wide, every filter row per
                                    workgroup with input rows kept in an LDS ring */
    WGRAD_VARIANT_DGRAD = 4      /* backward data (wgrad_dgrad_plan only): MFMA implicit GEMM over
                                    input positions, reduction over (tap, K/G) */
} wgrad_variant;

/* Overrides for tests and benchmarks; 0 in a field means "the plan decides".
 * Production callers pass NULL. */
typedef struct {
    int32_t split_k;      /* reduction slices S >= 1 */
    int32_t group_merge;  /* Gm: power of two dividing G (MFMA variant) */
    int32_t variant;      /* wgrad_variant */
    int32_t tile;         /* MFMA variant: tile id (see wgrad_plan_info.tile). DEPTHWISE variant:
                             kernel form, 1 = generic filter, 2 = windowed (filter width 3,
                             w-stride 1, w-dilation 1), 3 = strip (3x3, stride 1, dilation 1),
                             4 = tile (3x3, stride 1, dilation 1, C a multiple of 256).
                             ROWSLAB variant: form, 1 = one filter row per workgroup, 2 = every
                             filter row per workgroup (input-row ring). 0 = auto */
} wgrad_overrides;

/* What a plan decided, for logging and tests. */
typedef struct {
    int64_t out_len[3];      /* output lengths, ordered like in_len: (Do, Ho, Wo), (Ho, Wo) or (Wo) */
    int64_t gemm_m;          /* K/G */
    int64_t gemm_n;          /* (C/G)*Z*Y*X */
    int64_t gemm_k;          /* N*Do*Ho*Wo */
    int32_t variant;         /* wgrad_variant actually used */
    int32_t tile;            /* MFMA tile id, depthwise kernel form (1 generic, 2 windowed, 3 strip, 4 tile),
                                2 for the row-slab ring form, or 0 (row-slab, one filter row) */
    int32_t tile_m, tile_n, tile_k;
    int32_t split_k;         /* S */
    int32_t group_merge;     /* Gm */
    int32_t vector_width;    /* elements per global load */
    int64_t grid_main;       /* workgroups of the main kernel */
    int64_t grid_reduce;     /* workgroups of the reduce kernel (0 if none) */
    int64_t workspace_bytes; /* as wgrad_workspace_bytes */
    int32_t num_cus;         /* compute units the plan was sized for */
    int32_t reserved;
} wgrad_plan_info;

typedef struct wgrad_plan_s wgrad_plan_t;

/*
 * Validate a problem and choose kernels, split-K degree S and merge degree
 * Gm (host only, no device work).
 * Source: the support check is the Composable Kernel page's
 * IsSupportedArgument (a yes/no answer with a logged reason for each
 * unsupported case), here a status code with a reason string; the choice of
 * S and Gm follows rocm-libraries PR 12359 ("rocke/wgrad: add group merging
 * (Gm) for depthwise grouped conv"): its commit list sizes split-K from the
 * grid including groups, in waves, clamps it to the grid limit and then
 * snaps it to a multiple of the XCD count; its merge-degree follow-up
 * ("What changed") takes the largest admissible Gm.
 * hip_device >= 0 sizes the plan for that
 * device (it must be gfx950); -1 sizes it for an MI355X (256 CUs, 8 XCDs)
 * without touching the HIP runtime, for host-side tests.
 * Returns WGRAD_ERR_INVALID_ARG for: C or K not a multiple of G, a
 * non-positive length/stride/dilation, a negative pad, an empty output
 * (an output length < 1), ndim not 1, 2 or 3, an unsupported dtype pair, or sizes whose
 * element offsets do not fit in 31 bits. WGRAD_ERR_UNSUPPORTED for an
 * override the kernels cannot honour (e.g. Gm not a power of two dividing G).
 * On success *out owns host memory; free it with wgrad_plan_destroy.
 */
int wgrad_plan(const wgrad_problem* problem, const wgrad_overrides* overrides,
               int hip_device, wgrad_plan_t** out);

/* Bytes of device workspace wgrad_run needs: 0 when S = 1, otherwise
 * S * K * Y * X * (C/G) * 4 (fp32 partials of the unmerged dW, so the size
 * does not depend on Gm).
 * Source: rocm-libraries PR 12359's merge-degree follow-up, "What changed":
 * the two-stage workspace is sized for the unmerged dW, since merging
 * changes how many workgroups write dW and not how large dW is.
 * Host only; a NULL plan gives 0. */
size_t wgrad_workspace_bytes(const wgrad_plan_t* plan);

/*
 * Enqueue dW = wgrad(X, dY) on stream (a hipStream_t; NULL = the null
 * stream) and return without synchronising.
 * Source: the deterministic two-stage split-K epilogue that rocm-libraries
 * PR 11602 leaves the output type to ("Technical Details") and that PR
 * 12359 routes merged groups through (its commit list: merging and split-K
 * compose only via the two-stage workspace store, where the off-diagonal
 * group pairs are masked; packed atomics stay rejected). dW is overwritten (no
 * accumulation, no pre-zeroing needed). With S > 1 it runs two kernels: fp32
 * partials into ws, then a reduce/convert kernel that sums the S slices in
 * one fixed order and rounds to the out dtype (round to nearest even); no
 * atomics, so the same plan on the same inputs gives the same bits.
 * x, dy, dw are device pointers aligned to 16 bytes; ws is a device pointer
 * of at least wgrad_workspace_bytes(plan) bytes (may be NULL when that is 0).
 * A plan may be shared by runs on several streams and host threads at once;
 * runs that may overlap in time must each have a workspace (and dW) of
 * their own.
 * Errors: WGRAD_ERR_INVALID_ARG (NULL or misaligned pointer, ws too small),
 * WGRAD_ERR_HIP (launch failure).
 */
int wgrad_run(const wgrad_plan_t* plan, const void* x, const void* dy, void* dw,
              void* ws, size_t ws_bytes, void* stream);

/*
 * The two launches of wgrad_run, enqueued one at a time (the two stages of
 * the split-K epilogue cited at wgrad_run): stage 1 is the main
 * kernel (with S > 1 it writes the fp32 partials into ws), stage 2 the
 * reduce/convert kernel (a no-op when S = 1). Running stage 1 then stage 2
 * on one stream equals wgrad_run; a caller may enqueue other work between
 * them (for example the next layer's main kernel) or time them separately.
 * Arguments, checks and errors as in wgrad_run; stage not 1 or 2 is
 * WGRAD_ERR_INVALID_ARG. Stage 2 reads the workspace stage 1 wrote, so
 * both must see the same ws and be ordered (same stream or an event).
 */
int wgrad_run_stage(const wgrad_plan_t* plan, int stage, const void* x, const void* dy, void* dw,
                    void* ws, size_t ws_bytes, void* stream);

/* Size of the library-owned split-K scratch that wgrad_run_noalloc uses on
 * each GPU (16 MiB). */
#define WGRAD_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * wgrad_run without a caller workspace and without any device allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * The split-K partials go to a scratch array the library holds on each GPU
 * it runs on, WGRAD_NOALLOC_SCRATCH_BYTES in size, from the first use until
 * the process ends. Plans whose wgrad_workspace_bytes exceeds that size are
 * rejected with WGRAD_ERR_INVALID_ARG before anything is enqueued (plan with
 * a smaller split_k override, or use wgrad_run). The scratch needs no
 * clearing: the main kernel writes every partial the reduce kernel reads.
 * The first call on a GPU looks up the array's device address (no
 * allocation); make one call before capturing a graph.
 * The GPU is the stream's (the current device for the NULL stream). Every
 * call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (different streams, or graphs
 * replayed concurrently) race and give wrong results. Arguments, results
 * and the other errors are those of wgrad_run; plans with S = 1 never touch
 * the array.
 */
int wgrad_run_noalloc(const wgrad_plan_t* plan, const void* x, const void* dy, void* dw, void* stream);

/*
 * Backward data of the same convolution (rocm-libraries PR 11602, "add
 * transpose load for bwd weight and bwd data": its dgrad part, which reads
 * the weight tile K-outer; the direction itself is the adjoint of the forward
 * convolution that the backward-weight pages define):
 *
 *   dX[n,di,hi,wi,g,c] = sum_{k,z,y,x} dY[n,do,ho,wo,g,k] * W[g,k,z,y,x,c]
 *   over the (do, ho, wo) with do*stride_d - pad_lo_d + z*dilation_d = di
 *   (likewise ho with y, wo with x) and 0 <= do < Do, 0 <= ho < Ho, 0 <= wo < Wo.
 *
 * Same wgrad_problem; in_dtype is the type of dY and W, out_dtype the type
 * of dX (in_dtype or FP32). Layouts: dY [N][Do][Ho][Wo][K] (NDHWGK), W
 * [K][Z][Y][X][C/G] (GKZYXC), dX [N][Di][Hi][Wi][C] (NDHWGC); 2D and 1D drop
 * the leading axes as for wgrad. Computed as one GEMM per group with
 * M = N*Di*Hi*Wi input positions, N = C/G and a reduction of length
 * (K/G)*Z*Y*X; every dX element is written exactly once (positions no tap
 * reaches get 0), so there is no workspace and no split of the reduction.
 *
 * Small groups are merged Gm at a time into one block-diagonal GEMM (N =
 * Gm*C/G, reduction (Gm*K/G)*Z*Y*X, zero weight blocks between different
 * groups); wgrad_plan_query reports Gm in group_merge.
 *
 * wgrad_dgrad_plan: validation and errors as wgrad_plan. Overrides: split_k
 * must be 0 or 1, group_merge 0 (auto) or a power of two dividing G (the
 * MFMA kernel), variant AUTO or DGRAD, tile 0 (auto) or a
 * dgrad kernel id: 1, 2, 3 = the MFMA kernel with 128x32, 128x64, 128x128
 * (positions x channels) tiles; 4 = the depthwise direct kernel (C/G = K/G
 * = 1, C % 8 == 0, at most 2048 taps), which auto picks for such shapes, in
 * its row-walking form for 2D 3x3 filters with unit stride and dilation; 5 =
 * the depthwise kernel's per-tap form for any depthwise shape; 7 = the
 * depthwise tile kernel (2D 3x3 filter, unit stride and dilation, C/G = K/G
 * = 1 and C a multiple of 256), which auto picks ahead of 4 where it
 * applies; 6 = the
 * row-ring MFMA kernel (2D 3x3 filter, unit stride and dilation, h pads at
 * most 2 in all, input rows of at most 64 positions, C/G, C and K multiples
 * of 8, Gm*K/G of 32 or 64 and Gm*C/G a multiple of 32), which keeps a group
 * block's weights in LDS and stages each dY row once per workgroup; auto
 * picks it wherever it applies. Anything else is WGRAD_ERR_UNSUPPORTED. wgrad_plan_query reports
 * variant DGRAD, gemm_m/n/k as above and workspace_bytes 0.
 * The plan is released with wgrad_plan_destroy; wgrad_run and
 * wgrad_run_stage reject it (and wgrad_dgrad_run rejects backward-weight
 * plans) with WGRAD_ERR_INVALID_ARG.
 */
int wgrad_dgrad_plan(const wgrad_problem* problem, const wgrad_overrides* overrides,
                     int hip_device, wgrad_plan_t** out);

/*
 * Enqueue dX = dgrad(dY, W) on stream (NULL = the null stream) and return
 * without synchronising. dy, w, dx are device pointers aligned to 16 bytes
 * (dy and w may be NULL only when N = 0); dX is overwritten. One kernel, no
 * atomics: the same plan on the same inputs gives the same bits.
 * Errors: WGRAD_ERR_INVALID_ARG (NULL or misaligned pointer, wrong plan
 * kind), WGRAD_ERR_HIP (launch failure).
 */
int wgrad_dgrad_run(const wgrad_plan_t* plan, const void* dy, const void* w, void* dx, void* stream);

/* Fill *info with the plan's decisions (host only): the kernel family, tile,
 * S and Gm chosen as described at wgrad_plan. Errors: WGRAD_ERR_INVALID_ARG
 * for a NULL plan or info. */
int wgrad_plan_query(const wgrad_plan_t* plan, wgrad_plan_info* info);

/* Kernel name with its flags (tile, atom, "kouter", "spk<S>", "gm<Gm>"),
 * valid until the plan is destroyed; "" for a NULL plan. The flags follow
 * the pages' kernel names: rocm-libraries PR 11602, "Technical Details"
 * (the "kouter" flag for the K-outer LDS tile, before "spk*"), and PR 12359,
 * "Technical Details" (the gm{N} tag, so that merge degrees never share a
 * name). The string is owned by the plan. */
const char* wgrad_plan_describe(const wgrad_plan_t* plan);

/* Release a plan (NULL is allowed). A plan is immutable after creation and
 * may be used from several threads at once. Host memory only. */
void wgrad_plan_destroy(wgrad_plan_t* plan);

/* Reason for the calling thread's last failed call ("" if none), in the
 * manner of the rocke validators in rocm-libraries PR 11602 (its commit
 * list: a bad spec returns a reason string instead of being skipped
 * silently). Owned by the library, valid until the thread's next call. */
const char* wgrad_last_error(void);

/* Library version, "major.minor.patch" (plumbing; no page defines it). */
const char* wgrad_version(void);

/*
 * Self-test of the hardware lane map of the CDNA4 transposed LDS read
 * (ds_read_b64_tr_b16) that every MFMA kernel here builds its operand
 * fragments with (rocm-libraries PR 11602, "Technical Details": the K-outer
 * tile read with ds_read_tr16_b64; its gfx1250 follow-up notes that a
 * per-lane hardware probe settles such a map in one run). One wave fills a
 * 16 x 64 tile of 16-bit codes (row << 8 | column) in LDS and reads one
 * 32x32x16 operand fragment the way the kernels do; out (a device buffer of
 * 512 uint16, 16-byte aligned) receives lane l's eight values at
 * [8*l, 8*l + 8). The map the kernels assume: value e of lane l is the code
 * of row 8*(l/32) + e, column l % 32. Enqueued on stream; no synchronisation.
 * Errors: WGRAD_ERR_INVALID_ARG (NULL or misaligned out), WGRAD_ERR_HIP.
 */
int wgrad_probe_transpose_read(void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WGRAD_H */
