/*
 * cbd.h -- 2-D convolution backward-data (dX = conv_bwd_data(dY, W)) on
 * AMD Instinct MI355X (gfx950), computed as an implicit GEMM with one
 * sub-GEMM per stride-residue class, all classes in a single launch.
 *
 * Plain C ABI: no C++ types, no exceptions, no torch types.  Every call
 * returns a status code; nothing aborts.
 *
 * The operation.  For the forward convolution
 *   y[n, g*K/G+k, ho, wo] = sum_{c, r, s} x[n, g*C/G+c, ho*Sh + r*Dh - Ph,
 *                                            wo*Sw + s*Dw - Pw] * W[g*K/G+k, c, r, s]
 * (zero padding), backward-data is its adjoint in x:
 *   dX[n, g*C/G+c, hi, wi] = sum over k and over the taps (r, s) with
 *   hi + Ph - r*Dh = ho*Sh, wi + Pw - s*Dw = wo*Sw, 0 <= ho < Ho, 0 <= wo < Wo
 *   of dY[n, g*K/G+k, ho, wo] * W[g*K/G+k, c, r, s].
 * dX positions that no tap reaches are written as +0.
 *   - Problem fields and the gkcyx / ngchw / ngkhw layouts: rocMLIR PR #246
 *     "Backward data", the driver command lines at the end of the thread
 *     (batchsize, in/out channels, in_h/in_w, fil_h/fil_w, padding, stride,
 *     dilation, groupsize).
 *   - NHWC / KYXC layouts, bf16 operands with f32 accumulation and a bf16
 *     result, the caller-provided output that is overwritten: fusilli issue
 *     #101 "Non-unit stride input backward different input and dispatches
 *     between BOO and Fusilli" (BOO listing; torch-IR listing's
 *     convolution_backward call with output_mask [true, false, false]).
 *   - One sub-GEMM per stride residue ("multi-kernels", consecutive gemm
 *     ids, arguments reconstructed by the library rather than passed a
 *     kernel id by the client): rocMLIR PR #246; the v4r1 backward-data
 *     strategy named in MIOpen PR #272 "[igemm_dynamic] v4r1 bwd dynamic
 *     kernel".  Here the classes share one launch.
 *   - Plan first, then run (problem -> find solution -> load -> run): the
 *     MIOpen workflow described in the debian-ai thread "MIOpen package LFS
 *     files".
 */
#ifndef CBD_H
#define CBD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CBD_OK = 0,
  CBD_ERR_INVALID_ARG = 1, /* inconsistent problem, NULL pointer, bad index */
  CBD_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels accept
                              (sizes beyond 32-bit buffer addressing, stride
                              product > 64, misaligned pointers)           */
  CBD_ERR_HIP = 3,         /* HIP runtime / launch error; see cbd_last_error */
  CBD_ERR_NO_MEMORY = 4    /* host allocation failed                        */
} cbd_status;

typedef enum { CBD_F32 = 0, CBD_BF16 = 1 } cbd_dtype; /* dY, W and dX share it;
                                                          accumulation is f32 */

typedef enum {
  /* dX [N][G*C/G][Hi][Wi], dY [N][G*K/G][Ho][Wo], W [G*K/G][C/G][Y][X]
     (ngchw / ngkhw / gkcyx; identical to NCHW / KCYX) */
  CBD_LAYOUT_NCHW = 0,
  /* dX [N][Hi][Wi][G*C/G], dY [N][Ho][Wo][G*K/G], W [G*K/G][Y][X][C/G]
     (NHWC / KYXC) */
  CBD_LAYOUT_NHWC = 1
} cbd_layout;

/* The problem.  c and k are TOTAL channel counts; g divides both.  Channel
 * numbering is group-major (channel = g*(C/G) + c, filter row = g*(K/G) + k).
 * Hi and Wi are given (never inferred from Ho/Wo); Ho and Wo follow as
 * floor((Hi + 2*Ph - Dh*(Y-1) - 1) / Sh) + 1 and likewise for W. */
typedef struct {
  int64_t n, g, c, k, hi, wi, y, x;
  int32_t stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
  int32_t layout; /* cbd_layout */
  int32_t dtype;  /* cbd_dtype  */
} cbd_problem;

typedef struct cbd_plan_s cbd_plan_t; /* opaque; immutable once created */

/* Kernel families a plan may use for its main (GEMM) launch. */
typedef enum {
  CBD_KERNEL_AUTO = -1,
  CBD_KERNEL_GENERIC = 0,   /* any layout / dtype: gathered 64x64 tiles, f32 MFMA */
  CBD_KERNEL_NHWC_BF16 = 1, /* NHWC bf16, K/G % 32 == 0, K/G <= 131072,
                               C/G % 8 == 0, at most 16 taps per class:
                               256x256x32 tiles, bf16 MFMA, 4-stage LDS */
  CBD_KERNEL_GROUPED = 2,   /* NHWC, C/G == K/G, at most 9 taps per class.
                               Either C/G in {1,2,4,8} with G dividing 256:
                               per-group accumulation, filter in registers, dY
                               rows streamed through an LDS ring when C/G <= 4,
                               a pixel is a multiple of 16 bytes and a class's
                               taps are one dY row apart; or bf16 with C/G in
                               {8,16,32} and G a multiple of 16, 8 or 4
                               respectively (groups in 256-byte pixel slices,
                               any number of slices, G > 256 included), taps
                               one dY row apart: 16x16x16 MFMA.  The planner
                               prefers the latter for bf16 C/G = 8 whenever it
                               applies. */
  CBD_KERNEL_NCHW_ROWS = 3  /* NCHW / KCYX, f32 or bf16, residue split (no
                               no_split, per_class or ksplit): a workgroup owns
                               whole dX rows of 16 channels of one image and
                               group, stages the dY rows and all W taps it
                               needs in LDS and computes every class from
                               there (16x16x4 f32 MFMA); unreached positions
                               are written in the same rows (no zero-fill
                               launch).  Needs the staged tiles to fit LDS;
                               used only when forced (slower than the
                               generic family on the NCHW problems
                               measured). */
} cbd_kernel;

typedef struct {
  int32_t force_kernel; /* cbd_kernel; CBD_KERNEL_AUTO lets the planner choose */
  int32_t no_split;     /* 1: the zero-insertion form instead of the residue
                           split, as a comparison baseline (the BOO listing
                           of fusilli issue #101 convolves a zero-inserted
                           dY): one GEMM over every dX position and all Y*X
                           taps, where a term whose dY index is not a
                           multiple of the stride (an inserted zero) reads 0.
                           Executes up to S_h*S_w times the MACs; generic and
                           NHWC bf16 families only (grouped: UNSUPPORTED). */
  int32_t rows_per_wg;  /* grouped family, pipelined row kernel: output rows
                           per workgroup (0: the planner's choice; larger than
                           a class's rows: clamped); -1: never the pipelined
                           kernels (row or direct kernel instead; UNSUPPORTED
                           for 16 or 32 channels per group).  Other families
                           ignore it. */
  int32_t grouped_dot;  /* grouped family: 1 keeps the pipelined kernel on
                           dot-product instructions where it would use the
                           4x4x4 MFMA (a comparison switch); 0 or 1 */
  int32_t cols_per_wg;  /* grouped family, MFMA pipelined kernels: positions of
                           a row per workgroup, rounded up to a multiple of 4
                           (4x4x4 kernel) or 16 (16x16x16 kernel) (0: the
                           planner's choice) */
  int32_t ksplit;       /* large-tile (NHWC bf16) and generic kernels: split
                           each tile's K loop over this many workgroups (at
                           most 64; clamped to the k tiles of the shortest
                           class).  Partial tiles go to a caller workspace
                           as f32 and a second kernel sums them in split
                           order and writes dX: such a plan runs only
                           through cbd_run_ws.  For grids too small to fill
                           the GPU (e.g. one GPU's batch shard).
                           0: the planner's choice -- for the large-tile
                           kernel below 64 tiles the plan also holds a
                           split configuration
                           (cbd_plan_info: auto_ksplit), which cbd_run_ws
                           runs when given a workspace of at least
                           auto_workspace_bytes; cbd_run, or a smaller
                           workspace, runs the unsplit one.  1: never
                           split. */
  int32_t per_class;    /* 1: one main launch per residue class instead of one
                           for all (an ablation of the single launch; not
                           with ksplit); 0 or 1 */
  int32_t static_shape; /* shape-specialised instances, which compute the
                           same bits as the descriptor-driven kernel.
                           Large-tile kernel, level 1: k tiles per tap and
                           taps per class fixed at compile time (K/G =
                           2048, one tap per class); level 2: the whole
                           geometry fixed (G = 1, C = K = 2048, Hi = 1, a
                           1x2 filter at stride 2 along W, no padding, even
                           Wi; any N and Wi; not with per_class).  Generic
                           and grouped 4x4x4-MFMA kernels: level 2, the
                           whole plan of one of the listed workload
                           problems (not with per_class or ksplit).  0: the
                           most specialised one that matches; 1: required
                           (UNSUPPORTED if none matches); -1: never (the
                           descriptor-driven kernel, for comparison) */
  int32_t merge_phases; /* grouped 4x4x4-MFMA kernel at stride 2 x 2 with
                           every phase a class (taps one dY row and column
                           apart, at most 4 taps per class): 1 runs one
                           workgroup per block of class rows for all four
                           phases, writing whole dX rows (a comparison
                           form, measured slower; UNSUPPORTED where it does
                           not apply); 0 or -1: one class per workgroup */
  int32_t reserved[3];  /* must be zero */
} cbd_plan_options;

/* Build a plan (host-only work; needs no GPU).  On success *out_plan owns a
 * heap object that the caller frees with cbd_plan_destroy.  Errors:
 * INVALID_ARG for NULL arguments, non-positive sizes, G not dividing C or K,
 * negative padding, Ho or Wo < 1, unknown layout or dtype; UNSUPPORTED for
 * tensors of 2^31 bytes or more, stride_h*stride_w > 64, dilation > 64. */
cbd_status cbd_plan(const cbd_problem* problem, cbd_plan_t** out_plan);

/* As cbd_plan, with options (options may be NULL).  A forced kernel that
 * cannot run the problem gives UNSUPPORTED.
 * With the environment variable CBD_LOG set (to anything but "" or "0"),
 * every plan built is described on stderr: the problem, the kernel chosen
 * and its launch shape, the sub-GEMMs and the zero regions. */
cbd_status cbd_plan_ex(const cbd_problem* problem, const cbd_plan_options* options,
                       cbd_plan_t** out_plan);

/* Run a plan.  dy, w and dx are DEVICE pointers to dense tensors in the
 * plan's layout and dtype, owned by the caller; dy and w are read only, dx
 * is fully overwritten and must not overlap dy or w.  stream is a
 * hipStream_t (NULL = the default stream).  Asynchronous and stream-ordered:
 * no host synchronisation, no allocation, no copies; safe to call from
 * several threads on distinct streams.  Errors: INVALID_ARG for NULL plan or
 * pointers; UNSUPPORTED for a pointer not aligned as the plan requires
 * (cbd_plan_info: align_dy / align_w / align_dx -- the element size for the
 * generic family, 16 bytes otherwise); HIP when a launch fails (detail in
 * cbd_last_error()). */
cbd_status cbd_run(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                   void* stream);

/* As cbd_run, with a workspace.  Plans with options.ksplit >= 2 need one
 * (cbd_plan_info: workspace_bytes); a plan that holds the planner's split
 * configuration (auto_ksplit > 1) runs it when workspace_bytes is at least
 * auto_workspace_bytes, and its unsplit configuration otherwise (also for a
 * NULL workspace); other plans ignore the workspace.  workspace is a DEVICE
 * buffer, 256-byte aligned, owned by the caller, not overlapping dy, w or
 * dx; its contents are scratch (no initialisation needed, overwritten).  The
 * plan's calls on one stream may share a workspace; concurrent calls on
 * different streams need one each.  Errors: as cbd_run, plus INVALID_ARG for
 * a missing, small or overlapping workspace where one is used, and
 * UNSUPPORTED for a misaligned one. */
cbd_status cbd_run_ws(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                      void* workspace, uint64_t workspace_bytes, void* stream);

/* Bytes of device workspace for this plan's fastest configuration: what
 * cbd_run_ws needs for a plan with options.ksplit >= 2 (cbd_run on such a
 * plan fails with INVALID_ARG), else what enables the planner's split
 * configuration (optional); 0: the plan uses none. */
cbd_status cbd_plan_workspace_size(const cbd_plan_t* plan, uint64_t* bytes);

/* Bytes of the workspace that cbd_run_noalloc holds on each GPU. */
#define CBD_NOALLOC_SCRATCH_BYTES (32u << 20)

/* As cbd_run_ws, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the workspace is a device array of CBD_NOALLOC_SCRATCH_BYTES
 * (32 MiB) inside the library, one copy per GPU, held until the process
 * ends; its device address is looked up on the first call on each device,
 * which must be the current device of the calling thread and the device of
 * stream.  A plan with options.ksplit >= 2 runs with it as its workspace; a
 * plan holding the planner's split configuration runs that configuration
 * when its workspace fits (the large-tile kernel's batch shards: at most 32
 * MiB); other plans run as with cbd_run.  No call allocates or frees memory.
 * The array keeps the last call's contents and nothing in it needs to start
 * at zero (split-K partial tiles are written before they are read).  Calls
 * that overlap in time on one GPU (different streams, or threads) share the
 * array and race: serialise them, or use cbd_run_ws with a workspace each.
 * Errors: as cbd_run_ws, plus UNSUPPORTED for a plan whose workspace
 * exceeds CBD_NOALLOC_SCRATCH_BYTES (nothing is launched) and HIP if the
 * array's address cannot be looked up. */
cbd_status cbd_run_noalloc(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                           void* stream);

/* Free a plan.  NULL is allowed. */
void cbd_plan_destroy(cbd_plan_t* plan);

/* Static description of a status code. */
const char* cbd_status_string(cbd_status s);

/* Detail of the last error on the calling thread ("" if none). */
const char* cbd_last_error(void);

/* ---- read-only introspection (tests, bench) ---- */

typedef struct {
  int64_t ho, wo;
  int32_t num_subgemms;     /* stride-residue classes with taps and positions */
  int32_t num_zero_regions; /* dX phase lattices that no tap reaches */
  int32_t kernel;           /* cbd_kernel of the main launch */
  int32_t tile_m, tile_n, tile_k;
  int32_t threads_main;     /* workgroup size of the main launch */
  int32_t launches;         /* kernels per cbd_run (1 to 3) */
  int64_t grid_main;        /* workgroups of the main launch (generic family:
                               includes the zero-fill workgroups folded into it) */
  int64_t grid_zero;        /* workgroups of a separate zero-fill launch (0 if
                               none or folded into the main launch) */
  int64_t useful_flops;     /* 2*N*C*(K/G)*Ho*Wo*Y*X */
  int64_t executed_macs;    /* sum over sub-GEMMs of G*M*N*K (valid-tap MACs
                               plus those of taps falling off dY's edge) */
  int64_t zero_elems;       /* dX elements written by the zero-fill launch */
  int64_t lds_dynamic;      /* dynamic LDS bytes per workgroup of the main
                               launch (grouped family: 0 for the direct kernel) */
  int64_t rows_per_wg;      /* grouped family: output rows per workgroup of the
                               pipelined row kernels; row-block family: dX rows
                               per workgroup (0: another kernel) */
  int64_t cols_per_wg;      /* grouped family, MFMA pipelined kernels: positions
                               per column block of a row (0: other kernels) */
  int64_t ksplit;           /* workgroups per tile of a split-K plan (1: none) */
  int64_t static_shape;     /* main launch: 0 descriptor-driven kernel, 1 or 2
                               the shape-specialised instance of that level */
  int64_t workspace_bytes;  /* device workspace cbd_run_ws needs (0: none) */
  int64_t variant;          /* kernel within the family; grouped: 0 direct,
                               1 one row per workgroup, 2 pipelined rows on
                               dot-product instructions, 3 pipelined rows on
                               4x4x4 MFMA (bf16, C/G = 4, G = 32 or 64),
                               4 pipelined rows on 16x16x16 MFMA (bf16, C/G
                               = 16 or 32), 5 as 3 with the four phases of a
                               2 x 2 stride in one workgroup (merge_phases
                               = 1); other families: 0 */
  int32_t align_dy, align_w, align_dx; /* byte alignment cbd_run requires of
                               each pointer: the element size for the generic
                               family (16 for dx when a zero-fill writes
                               16-byte chunks), 16 for the other families */
  int64_t auto_ksplit;      /* workgroups per tile of the planner's split
                               configuration, which cbd_run_ws runs given
                               auto_workspace_bytes (1: none) */
  int64_t auto_workspace_bytes; /* workspace that enables it (0: none) */
  int32_t zero_in_epilogue; /* 1: the main kernel writes the unreached dX
                               positions itself (generic family: one class
                               at phase (0,0) covering every stride block,
                               written whole; row-block family), so there
                               is no zero-fill work */
  int32_t reserved_;
} cbd_plan_info_t;

typedef struct {
  int32_t id;               /* 0 .. num_subgemms-1, consecutive */
  int32_t class_h, class_w; /* tap class i: taps i, i+T, i+2T, ... */
  int32_t phase_h, phase_w; /* dX positions phase + S*t */
  int32_t beta_h, beta_w;   /* dY row of tap j at position t: t + beta - delta*j */
  int32_t taps_h, taps_w;   /* taps in the class */
  int32_t tstep_h, tstep_w; /* T = S / gcd(S, D) */
  int32_t delta_h, delta_w; /* delta = D / gcd(S, D) */
  int64_t pos_h, pos_w;     /* positions per axis: ceil((Hi - phase) / S) */
  int64_t m, n, k;          /* per-group GEMM: M = C/G, N = N*pos_h*pos_w,
                               K = (K/G)*taps_h*taps_w */
  int64_t tile_begin, tiles;/* this class's workgroups in the main launch (row-
                               block family: 0, 0 -- every workgroup serves
                               every class in its rows) */
} cbd_subgemm_t;

typedef struct {
  int32_t phase_h, phase_w; /* lattice phase + S*t that no tap reaches */
  int64_t pos_h, pos_w;
} cbd_zero_region_t;

cbd_status cbd_plan_info(const cbd_plan_t* plan, cbd_plan_info_t* out);
cbd_status cbd_plan_subgemm(const cbd_plan_t* plan, int32_t i, cbd_subgemm_t* out);
cbd_status cbd_plan_zero_region(const cbd_plan_t* plan, int32_t i, cbd_zero_region_t* out);

#ifdef __cplusplus
}
#endif

#endif /* CBD_H */
