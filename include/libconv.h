/*
 * libconv.h -- forward 2-D / 3-D convolution on AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI: no C++ types, no HIP headers needed by callers.
 *
 * What every convolution entry point computes (the definition):
 *   y[n][co][o] = act( b[co] + sum_{ci < C_in} sum_{k in taps} xz[n][ci][o*s - p + k] * w[co][ci][k] )
 * where o, k, s, p are per-axis (h, w) or (t, h, w) indices, xz is x inside the
 * input and 0 outside (zero padding), there is no kernel flip, and act is the
 * identity or ReLU (max(v, 0)), applied after the bias.  This is the
 * gather-form direct convolution of the page "PP-OCR on Vulkan compute
 * shaders" (lpnh.cn/news/2745477), section 2.2 (output coordinate -> input
 * coordinate, out-of-range taps skipped, bias added per output channel),
 * with the ReLU fused into the write-back as in section 4.4 of that page, and
 * with one more spatial axis (frames) for the Convolution3D layer of the page
 * "SeedVR2 NCNN Vulkan" (Tencent/ncnn discussion 7001), section 3.2.
 *
 * Output extent per axis: out = floor((in + 2*pad - k) / stride) + 1; a
 * geometry whose window does not fit (in + 2*pad < k) is rejected.
 *
 * Conventions shared by every entry point:
 *   Ownership   x, w, bias and y are DEVICE pointers owned by the caller, in
 *               dense row-major layout (x NCHW / NCDHW, w OIHW / OIDHW,
 *               y NCHW / NCDHW), aligned at least to their element size.
 *               libconv keeps no pointer after the call returns, copies
 *               nothing between host and device and never synchronises the
 *               host.
 *   Memory      no call allocates device memory, and none keeps any
 *               between calls (the page "PP-OCR on Vulkan compute shaders",
 *               section 5.2, lists small per-operation allocations among the
 *               costs to remove).  Device memory beyond the operands comes
 *               from the caller, as a workspace (the *_ws calls and
 *               libconv_forward_ex): a plan may pack OIHW weights into it
 *               once per call, for the kernels that copy packed weights
 *               straight into on-chip memory, and keep the fp32 partial sums
 *               of a split reduction (split-K) there.  Without a workspace
 *               (NULL, or the calls without one) a plan does neither.
 *               libconv_workspace_size gives the bytes the best plan uses.
 *   Stream      work is enqueued on `stream` (a hipStream_t; NULL means the
 *               null stream) and the call returns as soon as it is enqueued.
 *               Inputs must stay valid until the stream reaches the kernel.
 *               The calls make no host sync, so they may be recorded into a
 *               HIP graph, and the plan depends only on the shape, the
 *               weight form and the workspace size: a captured call runs the
 *               same kernels as the same call made eagerly (grid, block and
 *               addresses fixed at capture, the rule of capture and replay
 *               in "SDXL UNet under CUDA Graph", sections 2.2-2.3).
 *   Dtypes      x, w, bias and y share one storage dtype (libconv_dtype).
 *               Products and sums are formed in fp32 (fp16/bf16 products are
 *               exact in fp32) and y is rounded once, to nearest even.
 *   Errors      argument errors are returned before anything is enqueued;
 *               a failed launch returns LIBCONV_ERR_LAUNCH.  Nothing aborts or
 *               prints.  A shape no kernel supports returns
 *               LIBCONV_ERR_UNSUPPORTED; there is no silent fallback to
 *               another device or to the host.
 *   Limits      every tensor (and the packed weights) must span fewer than
 *               2^31 bytes; all sizes must be >= 1 except N, which may be 0
 *               (nothing is enqueued).
 *   Threads     calls from several host threads are safe; the only shared
 *               state is a per-device property cache filled once.
 */
#ifndef LIBCONV_H
#define LIBCONV_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LIBCONV_F32 = 0,   /* IEEE binary32 */
  LIBCONV_F16 = 1,   /* IEEE binary16 */
  LIBCONV_BF16 = 2   /* bfloat16 (upper half of binary32) */
} libconv_dtype;

typedef enum {
  LIBCONV_ACT_NONE = 0,
  LIBCONV_ACT_RELU = 1
} libconv_act;

/* Kernel families the dispatcher chooses between. */
typedef enum {
  LIBCONV_ALGO_AUTO = 0,    /* shape-driven choice (the default) */
  LIBCONV_ALGO_DIRECT = 1,  /* LDS halo-tiled direct kernel on the vector ALUs */
  LIBCONV_ALGO_IGEMM = 2    /* implicit GEMM on the matrix cores (MFMA) */
} libconv_algo;

typedef enum {
  LIBCONV_OK = 0,
  LIBCONV_ERR_NULL_POINTER = 1,   /* x, w or y is NULL */
  LIBCONV_ERR_BAD_SHAPE = 2,      /* a size < 1 (N < 0), stride < 1, pad < 0,
                                     channel mismatch, or the window does not fit */
  LIBCONV_ERR_BAD_DTYPE = 3,      /* dtype is not a libconv_dtype */
  LIBCONV_ERR_BAD_ACTIVATION = 4, /* act is not a libconv_act */
  LIBCONV_ERR_ALIAS = 5,          /* y overlaps x, w or bias */
  LIBCONV_ERR_UNSUPPORTED = 6,    /* the requested algorithm cannot run this shape */
  LIBCONV_ERR_NO_DEVICE = 7,      /* no HIP device, or the current device is not gfx950 */
  LIBCONV_ERR_LAUNCH = 8,         /* the kernel launch failed */
  LIBCONV_ERR_BAD_ALGO = 9,       /* algo is not a libconv_algo */
  LIBCONV_ERR_TOO_LARGE = 10,     /* a tensor (or the packed weights) spans 2^31 bytes or more */
  LIBCONV_ERR_OUT_OF_MEMORY = 11, /* not returned by this version (no call allocates) */
  LIBCONV_ERR_MISALIGNED = 12,    /* a workspace is not 256-byte aligned */
  LIBCONV_ERR_SCRATCH_TOO_SMALL = 13 /* conv3d_forward_noalloc: the plan needs more than the
                                        library's scratch array holds */
} libconv_status;

/*
 * 2-D convolution.
 *   x    [N][C_in][H][W]          device, read only
 *   w    [C_out][C_in][KH][KW]    device, read only
 *   bias [C_out] or NULL          device, read only; NULL means no bias
 *   y    [N][C_out][OH][OW]       device, written (every element exactly once)
 *   pad_*    zero padding added on both sides of the axis (>= 0)
 *   stride_* step of the window (>= 1)
 *   dtype    libconv_dtype of x, w, bias and y
 *   act      libconv_act applied after the bias
 *   stream   hipStream_t or NULL
 * Definition: page "PP-OCR on Vulkan compute shaders", section 2.2 (batch
 * added as an outer loop; per-axis pad and stride).
 */
libconv_status conv2d_forward(const void* x, const void* w, const void* bias, void* y,
                              int N, int C_in, int H, int W, int C_out, int KH, int KW,
                              int pad_h, int pad_w, int stride_h, int stride_w,
                              int dtype, int act, void* stream);

/*
 * 3-D convolution over frames.
 *   x    [N][C_in][T][H][W]          y [N][C_out][OT][OH][OW]
 *   w    [C_out][C_in][KT][KH][KW]   bias [C_out] or NULL
 * Other arguments as for conv2d_forward.
 * Definition: the Convolution3D layer of the page "SeedVR2 NCNN Vulkan",
 * section 3.2: the 2-D rule with the frame axis added (zero padding in time
 * as in space).
 */
libconv_status conv3d_forward(const void* x, const void* w, const void* bias, void* y,
                              int N, int C_in, int T, int H, int W,
                              int C_out, int KT, int KH, int KW,
                              int pad_t, int pad_h, int pad_w,
                              int stride_t, int stride_h, int stride_w,
                              int dtype, int act, void* stream);

/*
 * conv2d_forward / conv3d_forward with a caller-owned device workspace
 * (`workspace`, 256-byte aligned, `workspace_bytes` long; NULL means none).
 * With room enough the dispatcher may pack the OIHW / OIDHW weights into the
 * workspace on this call (for the kernels that read packed weights) and
 * split the reduction over several workgroups, keeping their fp32 partial
 * sums there; libconv_workspace_size says how much the best plan takes, and
 * with less the dispatcher picks the best plan that fits.  The workspace
 * must not overlap x, w, bias or y; its contents on entry do not matter and
 * are undefined after the call.  Calls that share a workspace must be
 * ordered (one stream, or events).  Errors as conv2d_forward, plus
 * LIBCONV_ERR_MISALIGNED and LIBCONV_ERR_ALIAS for the workspace.
 */
libconv_status conv2d_forward_ws(const void* x, const void* w, const void* bias, void* y,
                                 int N, int C_in, int H, int W, int C_out, int KH, int KW,
                                 int pad_h, int pad_w, int stride_h, int stride_w,
                                 int dtype, int act, void* workspace, long long workspace_bytes,
                                 void* stream);
libconv_status conv3d_forward_ws(const void* x, const void* w, const void* bias, void* y,
                                 int N, int C_in, int T, int H, int W,
                                 int C_out, int KT, int KH, int KW,
                                 int pad_t, int pad_h, int pad_w,
                                 int stride_t, int stride_h, int stride_w,
                                 int dtype, int act, void* workspace, long long workspace_bytes,
                                 void* stream);

/*
 * conv3d_forward_ws without a caller workspace and without any allocation:
 * for callers that cannot allocate device memory at all (code recorded under
 * HIP graph capture that must not take memory, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is the library's own
 * device array of 64 MiB (LIBCONV_SCRATCH_BYTES), one per GPU, held until the
 * process ends; a plan needing more (libconv_workspace_size above it) returns
 * LIBCONV_ERR_SCRATCH_TOO_SMALL before anything is enqueued.  Same result as
 * conv3d_forward_ws given the workspace libconv_workspace_size names (the
 * same plan).  Every call on one GPU shares that array, so calls that may
 * overlap on one GPU (other streams, other host threads) race: order them.
 * The array's contents carry over between calls; no plan reads any of it
 * before writing it.  2-D: T = KT = 1, pad_t = 0, stride_t = 1.
 */
#define LIBCONV_SCRATCH_BYTES (64LL << 20)
libconv_status conv3d_forward_noalloc(const void* x, const void* w, const void* bias, void* y,
                                      int N, int C_in, int T, int H, int W,
                                      int C_out, int KT, int KH, int KW,
                                      int pad_t, int pad_h, int pad_w,
                                      int stride_t, int stride_h, int stride_w,
                                      int dtype, int act, void* stream);

/* Flags of libconv_forward_ex, libconv_workspace_size and libconv_query_plan. */
enum {
  LIBCONV_PLAN_CAPTURING = 1,  /* accepted and ignored: plans do not depend on graph capture */
  LIBCONV_PLAN_POOL2 = 2,      /* conv2d_forward_pool: 2x2 max pooling fused after the activation */
  LIBCONV_PLAN_CPACK = 4,      /* channel-packed activations (conv3d_forward_cpack) */
  LIBCONV_PLAN_PACKED_W = 8    /* (queries only) the call passes packed weights */
};

/*
 * Every convolution this library computes, with every option: exactly one
 * of w (OIHW / OIDHW) and packed_w (libconv_pack_weights; then only the
 * MFMA kernels run); the frame axis padded by pad_t_front zero frames before
 * the first frame and pad_t_back after the last (as conv3d_forward_tpad);
 * flags LIBCONV_PLAN_POOL2 (as conv2d_forward_pool; 2-D only) or
 * LIBCONV_PLAN_CPACK (channel-packed x and y, as conv3d_forward_cpack);
 * algo a libconv_algo; a workspace as conv3d_forward_ws.  The other calls
 * are this one with some arguments fixed.  2-D: T = KT = 1, time pads 0,
 * stride_t = 1.
 */
libconv_status libconv_forward_ex(const void* x, const void* w, const void* packed_w,
                                  const void* bias, void* y,
                                  int N, int C_in, int T, int H, int W,
                                  int C_out, int KT, int KH, int KW,
                                  int pad_t_front, int pad_t_back, int pad_h, int pad_w,
                                  int stride_t, int stride_h, int stride_w,
                                  int dtype, int act, int algo, int flags,
                                  void* workspace, long long workspace_bytes, void* stream);

/*
 * Workspace bytes the best plan for libconv_forward_ex with these
 * arguments uses (0 when it uses none; flags as libconv_forward_ex, plus
 * LIBCONV_PLAN_PACKED_W for a call given packed weights), or -1 for
 * arguments the call would reject.  Pure host arithmetic: works without a
 * GPU.  The answer is fixed for a shape, so it can be allocated once per
 * layer.
 */
long long libconv_workspace_size(int N, int C_in, int T, int H, int W,
                                 int C_out, int KT, int KH, int KW,
                                 int pad_t_front, int pad_t_back, int pad_h, int pad_w,
                                 int stride_t, int stride_h, int stride_w,
                                 int dtype, int act, int algo, int flags);

/*
 * 3-D convolution with an explicit kernel family (libconv_algo).  With
 * LIBCONV_ALGO_AUTO this is conv3d_forward.  A 2-D convolution is the case
 * T = KT = 1, pad_t = 0, stride_t = 1.  Returns LIBCONV_ERR_UNSUPPORTED if
 * the requested family cannot run the shape.  Meant for tests and for the
 * evidence behind the dispatcher's choice.
 */
libconv_status libconv_forward_algo(const void* x, const void* w, const void* bias, void* y,
                                    int N, int C_in, int T, int H, int W,
                                    int C_out, int KT, int KH, int KW,
                                    int pad_t, int pad_h, int pad_w,
                                    int stride_t, int stride_h, int stride_w,
                                    int dtype, int act, int algo, void* stream);

/*
 * Packed weights: the weights reordered once into the layout the implicit-GEMM
 * kernels stage from, so that a call copies them into on-chip memory without
 * rearranging them (the per-layer weight packing of the Convolution3D backend
 * in "SeedVR2 NCNN Vulkan", section 3.2, does the same at model load).
 * Layout: [round_up(C_out, 128) / 64][ceil(C_in/g)][KT*KH*KW][64][g] entries
 * of g consecutive input channels (16 bytes), g = 8 for 16-bit dtypes and 4
 * for fp32: blocks of 64 output channels, each contiguous; channels beyond
 * C_in / C_out are zero.
 *
 * libconv_packed_weight_bytes: size of that buffer, or -1 if the arguments are
 * out of range, the kernel size has no packed kernels (supported: 1x1x1,
 * 1x3x3 and 3x3x3 taps) or the buffer would span 2^31 bytes or more.
 */
long long libconv_packed_weight_bytes(int C_in, int C_out, int KT, int KH, int KW, int dtype);

/*
 * Pack OIHW / OIDHW weights w (device, read only) into `packed` (device,
 * written; caller-owned, packed_bytes >= libconv_packed_weight_bytes(..)).
 * Enqueued on `stream`; allocates nothing.  The buffers must not overlap.
 */
libconv_status libconv_pack_weights(const void* w, void* packed, long long packed_bytes,
                                    int C_in, int C_out, int KT, int KH, int KW,
                                    int dtype, void* stream);

/*
 * conv3d_forward with packed weights (from libconv_pack_weights) in place of
 * w; always an implicit GEMM on the matrix cores; no workspace (no split).  Returns
 * LIBCONV_ERR_UNSUPPORTED when no packed kernel fits the shape.  A 2-D
 * convolution is the case T = KT = 1, pad_t = 0, stride_t = 1.
 */
libconv_status libconv_forward_packed(const void* x, const void* packed_w, const void* bias,
                                      void* y, int N, int C_in, int T, int H, int W,
                                      int C_out, int KT, int KH, int KW,
                                      int pad_t, int pad_h, int pad_w,
                                      int stride_t, int stride_h, int stride_w,
                                      int dtype, int act, void* stream);

/*
 * conv2d_forward followed by 2x2 max pooling with stride 2, fused into the
 * convolution's epilogue (the conv + activation + pool fusion of the
 * detector in "PP-OCR on Vulkan compute shaders", section 4.4, which halves
 * the dispatches):  y[n][co][i][j] = max over a, b in {0, 1} of
 * act(conv(x, w) + bias)[n][co][2i+a][2j+b], y [N][C_out][OH/2][OW/2]
 * (floor: an odd last row or column of the conv output is dropped).  The
 * max is taken before the one rounding to the storage dtype, which gives
 * the same value as rounding every conv output and pooling them.  Runs on
 * the MFMA kernels only: LIBCONV_ERR_UNSUPPORTED for shapes they do not take
 * (e.g. C_in * KH * KW below one MFMA k-step's channels, 1x1 layers);
 * LIBCONV_ERR_BAD_SHAPE when OH or OW is below 2.
 */
libconv_status conv2d_forward_pool(const void* x, const void* w, const void* bias, void* y,
                                   int N, int C_in, int H, int W, int C_out, int KH, int KW,
                                   int pad_h, int pad_w, int stride_h, int stride_w,
                                   int dtype, int act, void* stream);

/*
 * conv3d_forward with the frame axis padded by pad_t_front zero frames
 * before the first frame and pad_t_back after the last; they may differ.
 * The causal 3-D convolution of the spatio-temporal VAE in "SeedVR2 NCNN
 * Vulkan", section 7.2 (built there from Concat/Crop around a plain
 * Convolution3D) is pad_t_front = KT - 1, pad_t_back = 0: output frame t then
 * reads input frames t-KT+1 .. t only (stride 1).  Output frames:
 * floor((T + pad_t_front + pad_t_back - KT) / stride_t) + 1.
 * Weights: exactly one of w (OIDHW, as conv3d_forward; the dispatcher picks
 * the kernel) and packed_w (from libconv_pack_weights, as
 * libconv_forward_packed: MFMA kernels only); the other is NULL, else
 * LIBCONV_ERR_NULL_POINTER.  No workspace (libconv_forward_ex takes one).
 * Pads must be >= 0.
 */
libconv_status conv3d_forward_tpad(const void* x, const void* w, const void* packed_w,
                                   const void* bias, void* y,
                                   int N, int C_in, int T, int H, int W,
                                   int C_out, int KT, int KH, int KW,
                                   int pad_t_front, int pad_t_back, int pad_h, int pad_w,
                                   int stride_t, int stride_h, int stride_w,
                                   int dtype, int act, void* stream);

/*
 * Channel-packed activations.  The page "PP-OCR on Vulkan compute shaders"
 * (section 2.3) moved its tensors to a channels-together layout for
 * contiguous reads of the channels of a pixel, converting once at the edges
 * rather than in the hot path; the page "SeedVR2 NCNN Vulkan" (section 9)
 * plans to keep its channel packing (pack4) through the whole network so
 * that layers stop packing and unpacking between each other.  Here a group
 * is one 16-byte vector of channels, g = 8 for 16-bit dtypes and 4 for fp32:
 *   x_packed [N][ceil(C/g)][T][H][W][g],  element (n, c, t, h, w) at
 *   [n][c / g][t][h][w][c % g];  channels past C in the last group are 0.
 * (2-D tensors: T = 1.)  In this layout a halo row of one channel group is
 * contiguous memory, which the implicit-GEMM kernels copy straight into
 * on-chip memory, and an output group leaves as one vector store.
 *
 * libconv_cpack_bytes: bytes of such a tensor, or -1 for invalid arguments
 * or 2^31 bytes or more.
 * libconv_pack_activations / libconv_unpack_activations: conversion from
 * and to the plain [N][C][T][H][W] layout, on the device (both pointers
 * device, caller-owned, not overlapping), enqueued on `stream`; unpacking
 * drops the channels past C.  Errors as the convolution calls.
 */
long long libconv_cpack_bytes(int N, int C, int T, int H, int W, int dtype);
libconv_status libconv_pack_activations(const void* x, void* x_packed, int N, int C, int T,
                                        int H, int W, int dtype, void* stream);
libconv_status libconv_unpack_activations(const void* x_packed, void* x, int N, int C, int T,
                                          int H, int W, int dtype, void* stream);

/*
 * conv3d_forward_tpad on channel-packed activations: x is x_packed over
 * C_in channels, y (written) is packed over C_out channels, including the
 * zeros past C_out.  The channels past C_in in x must be finite (they meet
 * zero weights; pack_activations and this call write zeros there).  Both
 * must be 16-byte aligned.  Weights and bias as conv3d_forward_tpad (exactly
 * one of w and packed_w; with packed_w only the MFMA kernels run).  2-D:
 * T = KT = 1, time pads 0.  The MFMA kernels for this layout read packed
 * weights and cover 3x3x3 and 3x3 (stride 1), 3x3 stride 2 and 1x1; with
 * OIDHW weights they run only when libconv_forward_ex (flag
 * LIBCONV_PLAN_CPACK) is given a workspace to pack them into, else the
 * vector-ALU kernel runs.  Without an MFMA kernel for the shape, packed_w is
 * LIBCONV_ERR_UNSUPPORTED.
 */
libconv_status conv3d_forward_cpack(const void* x, const void* w, const void* packed_w,
                                    const void* bias, void* y,
                                    int N, int C_in, int T, int H, int W,
                                    int C_out, int KT, int KH, int KW,
                                    int pad_t_front, int pad_t_back, int pad_h, int pad_w,
                                    int stride_t, int stride_h, int stride_w,
                                    int dtype, int act, void* stream);

/*
 * Frame windows of a long video.  A 3-D convolution can be computed a few
 * output frames at a time, each piece from only the input frames it reads;
 * consecutive pieces share the frames their taps overlap on (KT - stride_t
 * frames).  This is how a video too long to hold whole goes through the
 * network: the long-video plan of "SeedVR2 NCNN Vulkan", section 9, cuts it
 * into chunks of 17 frames that overlap by 5.  Per convolution the pieces
 * compute the whole-video result: each output element is the same sum,
 * rounded once (the kernel chosen for a piece may differ from the
 * whole-video one, and with it the order of the fp32 sums).
 *
 * libconv_frame_window: the input frames [*in_frame0, *in_frame0 +
 * *in_frames) that output frames [out_frame0, out_frame0 + out_frames) of a
 * convolution over T frames read (time padding as conv3d_forward_tpad).
 * Pure host arithmetic.  LIBCONV_ERR_BAD_SHAPE when the output range is
 * empty or beyond the output frames, or reads padding only;
 * LIBCONV_ERR_NULL_POINTER for NULL outputs.
 */
libconv_status libconv_frame_window(int T, int KT, int pad_t_front, int pad_t_back,
                                    int stride_t, int out_frame0, int out_frames,
                                    int* in_frame0, int* in_frames);

/*
 * Output frames [out_frame0, out_frame0 + out_frames) of the convolution
 * conv3d_forward_tpad computes over a T-frame video, from a buffer holding
 * only the input frames libconv_frame_window names for that range.
 * x [N][C_in][in_frames][H][W] (device), y [N][C_out][out_frames][OH][OW]
 * (device), both contiguous; the other arguments describe the whole video
 * and are those of conv3d_forward_tpad (exactly one of w and packed_w).
 * Same errors as conv3d_forward_tpad, and LIBCONV_ERR_BAD_SHAPE for an
 * output range libconv_frame_window rejects.
 */
libconv_status conv3d_forward_frames(const void* x, const void* w, const void* packed_w,
                                     const void* bias, void* y,
                                     int N, int C_in, int T, int H, int W,
                                     int C_out, int KT, int KH, int KW,
                                     int pad_t_front, int pad_t_back, int pad_h, int pad_w,
                                     int stride_t, int stride_h, int stride_w,
                                     int out_frame0, int out_frames,
                                     int dtype, int act, void* stream);

/*
 * Device workspace conv3d_forward_chunked needs: two input-window and two
 * output-chunk buffers, and room for the weights packed once.  -1 if the
 * arguments are invalid for it.
 */
long long libconv_chunked_workspace_bytes(int N, int C_in, int T, int H, int W,
                                          int C_out, int KT, int KH, int KW,
                                          int pad_t_front, int pad_t_back,
                                          int pad_h, int pad_w,
                                          int stride_t, int stride_h, int stride_w,
                                          int chunk_frames, int dtype);

/*
 * The whole-video convolution of conv3d_forward_tpad, streamed in chunks of
 * chunk_frames output frames: x [N][C_in][T][H][W] and y
 * [N][C_out][OT][OH][OW] may be host memory (pinned memory lets the copies
 * run asynchronously; pageable memory works, with copies that block the
 * host) or device memory, and may be larger than the 2^31-byte limit of the
 * other calls; only one chunk's window and output are on the device at a
 * time, in `workspace` (device, caller-owned, at least
 * libconv_chunked_workspace_bytes).  Chunk c + 1's window is copied in on
 * copy_in_stream and chunk c - 1's output copied out on copy_out_stream
 * while chunk c computes on `stream` (the two copy streams let the two
 * directions of the host link run at once).  Each input frame is copied
 * from x once: the frames consecutive windows share (the time halo) move
 * from one window buffer to the other on the device.  The copies start after the
 * work already on `stream`, and `stream` waits for the last of them.
 * copy_out_stream NULL: outputs are copied on copy_in_stream; both NULL:
 * everything runs in order on `stream`.  Weights and bias are on the device;
 * exactly one of w and packed_w (OIDHW weights of a kernel size the packed
 * kernels take are packed once, into the workspace, before the first
 * chunk).  Requires
 * pad_t_front < KT and pad_t_back < KT (every output frame reads an input
 * frame).  LIBCONV_ERR_UNSUPPORTED while either stream is being captured
 * into a graph; a too-small workspace is LIBCONV_ERR_BAD_SHAPE.  The call
 * returns once everything is enqueued: the caller synchronises `stream`
 * before reading y or reusing x or the workspace.
 */
libconv_status conv3d_forward_chunked(const void* x, const void* w, const void* packed_w,
                                      const void* bias, void* y,
                                      int N, int C_in, int T, int H, int W,
                                      int C_out, int KT, int KH, int KW,
                                      int pad_t_front, int pad_t_back, int pad_h, int pad_w,
                                      int stride_t, int stride_h, int stride_w,
                                      int chunk_frames, void* workspace,
                                      long long workspace_bytes, int dtype, int act,
                                      void* stream, void* copy_in_stream,
                                      void* copy_out_stream);

/*
 * Which kernel the dispatcher would launch for this shape, without launching
 * (the per-layer "generic implementation or not?" check of "OpenCL-101
 * issue 52").
 * Arguments as for libconv_forward_algo (algo may force a family).  On
 * LIBCONV_OK: *algo_out is LIBCONV_ALGO_DIRECT or LIBCONV_ALGO_IGEMM,
 * *tile_out the tile configuration id (see libconv_tile_name) and
 * *grid_out the number of workgroups.  Pure host arithmetic: works without a
 * GPU.  Output pointers may not be NULL.
 */
libconv_status libconv_query_algo(int N, int C_in, int T, int H, int W,
                                  int C_out, int KT, int KH, int KW,
                                  int pad_t, int pad_h, int pad_w,
                                  int stride_t, int stride_h, int stride_w,
                                  int dtype, int act, int algo,
                                  int* algo_out, int* tile_out, long long* grid_out);

/*
 * libconv_query_algo with more facts about the plan: *ksplit_out, the
 * number of workgroups that share one output tile's reduction (split-K; 1 =
 * none), for a call given a workspace of workspace_bytes (0: none);
 * `flags` as libconv_forward_ex (LIBCONV_PLAN_POOL2: conv2d_forward_pool;
 * LIBCONV_PLAN_CPACK: channel-packed activations), plus
 * LIBCONV_PLAN_PACKED_W for a call given packed weights (MFMA tiles that
 * read them).  LIBCONV_PLAN_CAPTURING changes nothing: a call plans the same
 * way whether or not its stream is being captured.  Pure host arithmetic:
 * works without a GPU.  Output pointers may not be NULL.
 */
libconv_status libconv_query_plan(int N, int C_in, int T, int H, int W,
                                  int C_out, int KT, int KH, int KW,
                                  int pad_t, int pad_h, int pad_w,
                                  int stride_t, int stride_h, int stride_w,
                                  int dtype, int act, int algo, int flags,
                                  long long workspace_bytes,
                                  int* algo_out, int* tile_out, long long* grid_out,
                                  int* ksplit_out);

/*
 * Batch normalisation folded into the convolution before it, once, on the
 * host, at model load (the detector of "PP-OCR on Vulkan compute shaders"
 * folds each BN layer into the preceding conv's weights and bias on the CPU,
 * so that the GPU runs the fused conv only):
 *   s[co]       = gamma[co] / sqrt(var[co] + eps)
 *   w_out[co][k] = w[co][k] * s[co]                (k < k_per_out = C_in*KT*KH*KW)
 *   b_out[co]   = (b[co] - mean[co]) * s[co] + beta[co]      (b NULL: b = 0)
 * HOST pointers, fp32 in and out, each value computed in fp64 and rounded
 * once.  w_out / b_out may be w / b (in place).  The caller converts the
 * folded weights to the layer's storage dtype and copies them to the device.
 * LIBCONV_ERR_NULL_POINTER for a NULL argument other than b;
 * LIBCONV_ERR_BAD_SHAPE for C_out < 1, k_per_out < 1, or var[co] + eps <= 0
 * (nothing written then).
 */
libconv_status libconv_fold_batchnorm(const float* w, const float* b, const float* gamma,
                                      const float* beta, const float* mean, const float* var,
                                      float eps, int C_out, int k_per_out,
                                      float* w_out, float* b_out);

/* Human-readable name of a tile configuration id; "?" if unknown.  With
 * libconv_query_algo this answers the question the per-operator profiler of
 * "OpenCL-101 issue 52" asks of every layer: which implementation (a tuned
 * kernel or a generic one) a Conv actually runs. */
const char* libconv_tile_name(int tile_id);

/* Workgroups one compute unit holds at once for an MFMA tile configuration
 * and dtype (the per-operator, per-device workgroup sizing that "PP-OCR on
 * Vulkan compute shaders", section 4.4, tunes by hand; here a property of
 * each built tile): with measured = 0, the figure the dispatcher's cost model uses
 * (pure host, works without a GPU); with measured != 0, the HIP runtime's
 * occupancy query for the built kernel on the current device.  -1 for an
 * unknown tile id, a dtype the tile does not run, or (measured) no gfx950
 * device. */
int libconv_tile_occupancy(int tile_id, int dtype, int measured);

/* floor((in + 2*pad - k) / stride) + 1, or -1 if an argument is out of range
 * (in < 1, k < 1, pad < 0, stride < 1) or the window does not fit.  The
 * conv shader of "PP-OCR on Vulkan compute shaders", section 2.2, takes the
 * output extents as inputs without a formula; this is the only rule that
 * gives that page's detector's 640 -> 320 -> 160 at kernel 3, pad 1,
 * stride 2. */
int libconv_out_size(int in, int k, int pad, int stride);

/* The same with pad_lo before and pad_hi after the input (the frame axis of
 * conv3d_forward_tpad): floor((in + pad_lo + pad_hi - k) / stride) + 1, or -1. */
int libconv_out_size2(int in, int k, int pad_lo, int pad_hi, int stride);

/* Static description of a status code; never NULL.  Failures are reported,
 * never turned into an abort (the fault-tolerant backend bring-up of
 * "OpenCL-101 issue 52"). */
const char* libconv_status_string(int status);

/* LIBCONV_OK if `device` exists and is a gfx950 GPU, else LIBCONV_ERR_NO_DEVICE.
 * Never aborts; safe on a host without any GPU: the "is this backend
 * usable" query that "OpenCL-101 issue 52" adds so that a caller can pick
 * another path instead of crashing during initialisation. */
libconv_status libconv_device_supported(int device);

/* Library version as 10000*major + 100*minor + patch, so that a caller can
 * check that the library it loaded is the one it was built against (the
 * build and output-contract checks "SeedVR2 NCNN Vulkan", section 3.6,
 * adds after a layer silently ran elsewhere). */
int libconv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBCONV_H */
