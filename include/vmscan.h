/*
 * vmscan: Vision Mamba bidirectional selective scan and VMamba SS2D cross-scan for MI355X
 * (gfx950).  C ABI: plain pointers and sizes; no C++ or framework types cross this boundary.
 *
 * Pages cited (short keys):
 *   [P1] "状态空间模型如何重塑视觉序列处理 Vision Mamba的技术突破与应用价值" (sumeiyu.com/news/203653),
 *        section "选择性扫描机制的计算效率优势": h_t = A h_{t-1} + B x_t, y_t = C h_t + D x_t.
 *   [P3] "Vision Mamba的双向SSM 计算机视觉模型架构的下一代突破" (aitangshan.cn/news/1404048),
 *        §2.1 (A/A_b, v1/v2 parameter sets), §2.2 (reverse, scan, reverse back; average fusion),
 *        §4.3 (v2 fast path: (out + out_b.flip) / 2).
 *   [P4] "VMamba的SS2D模块 状态空间模型在视觉领域的革新设计" (lpnh.cn/news/670717),
 *        §2.1 (y * act(z) after the core), §2.2 (four cross-scan orders), §3.1 (Δ = softplus of a
 *        projection; per-direction projections), §3.2 (A = -exp(A_log)).
 *   [P5] "Vision Mamba实战 双向SSM Encoder核心代码解析与实现" (lpnh.cn/news/710454),
 *        §1 table (A/A_b [d_inner, d_state], B/C [batch, d_state, seq_len], D/D_b [d_inner]),
 *        §2.2 (bidirectional scan = forward scan + reversed scan of the reversed input),
 *        §4 (delta = softplus(.)).
 *
 * Per direction and per (batch b, channel d) both entry points compute, in fp32:
 *   Δ_t   = softplus(Δ_raw[t] + delta_bias[d])                     [P4] §3.1, [P5] §4
 *   a_t,n = exp(Δ_t A_n),  A_n = -exp(A_log[d, n])                  [P4] §3.2 (zero-order hold)
 *   h_t,n = a_t,n h_{t-1},n + Δ_t B_t,n u_t,  h_{-1} = 0           [P1]
 *   y_t   = Σ_n C_t,n h_t,n + D[d] u_t                              [P1]
 *
 * Conventions shared by every entry point:
 *   - Ownership: every pointer is caller-owned DEVICE memory (except `stream`).  The library never
 *     allocates or frees memory.  Its only state is a thread-local last HIP error and, for
 *     vmscan_fwd_bidir_noalloc, the address of its fixed device scratch buffer on each device.
 *   - Layout: all tensors are dense, row-major, with the shapes stated per argument.  Every
 *     pointer must be 16-byte aligned (else VMSCAN_ERR_ALIGN).  `out` must not alias an input.
 *   - Activation dtype: VMSCAN_F32 (float) or VMSCAN_BF16 (bfloat16 bit patterns, 2 bytes) for
 *     u/x, delta_raw, z, B, C and out.  A_log, D and delta_bias are always float32.  The state
 *     and all arithmetic are float32; bf16 outputs are rounded to nearest even once, at the store.
 *   - d_state: every scan entry point, forward and backward, takes 16 or 32 (else
 *     VMSCAN_ERR_UNSUPPORTED; the workspace and chunk-length queries return 0).  The pages use
 *     16 and suggest a larger state for high-resolution inputs ([P3] §4.1; [P4] §4.2 gives the
 *     16-32 range).  The workspace size depends on d_state.
 *   - Errors: arguments are validated synchronously and a status is returned before anything is
 *     enqueued; on success the kernels are enqueued on `stream` (NULL = the default stream) and the
 *     call returns without waiting.  A failed launch returns VMSCAN_ERR_HIP and the hipError_t
 *     is kept for vmscan_last_hip_error().  No entry point throws or aborts.
 *   - Workspace: caller-provided device scratch of at least the queried size.  When the query
 *     returns 0 none is needed and `workspace` may be NULL (if given, it must still be 16-byte
 *     aligned).  Its contents on entry are ignored.
 *   - Wait status: the waves that hold different state parts of one direction wait for each other
 *     through LDS counters.  Every such wait ends by construction; it is also bounded, and a wait
 *     that runs out of its bound stores 1 into the first int32 of the workspace (the call's status
 *     word, which the call's first kernel sets to 0).  So after the call's kernels have finished,
 *     that word reads 0 unless the results are unspecified.  A library built with
 *     -DVMSCAN_CHECK_WAITS checks the word itself: each scan entry point then waits for its kernels
 *     and returns VMSCAN_ERR_WAIT if it is set.  (A stage-2-only call leaves the word of its stage 1.)
 */
#ifndef VMSCAN_H
#define VMSCAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VMSCAN_OK = 0,
  VMSCAN_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  VMSCAN_ERR_SHAPE = 2,       /* a size is < 1, or too large for the index types               */
  VMSCAN_ERR_UNSUPPORTED = 3, /* d_state or dtype not supported                                */
  VMSCAN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                              */
  VMSCAN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the queried size               */
  VMSCAN_ERR_HIP = 6,         /* a HIP call failed; see vmscan_last_hip_error()                */
  VMSCAN_ERR_SCRATCH = 7,     /* the call needs more than VMSCAN_SCRATCH_BYTES (no-alloc entry) */
  VMSCAN_ERR_WAIT = 8         /* a bounded wait gave up (builds with VMSCAN_CHECK_WAITS only)   */
} vmscan_status;

typedef enum { VMSCAN_F32 = 0, VMSCAN_BF16 = 1 } vmscan_dtype;

/* Human-readable name of a status (static string, never NULL). */
const char *vmscan_status_string(vmscan_status s);

/* hipError_t (as int) behind the last VMSCAN_ERR_HIP returned on the calling thread; 0 if none. */
int vmscan_last_hip_error(void);

/* Chunk length (tokens) the library uses for a bidirectional scan of this shape when
 * chunk_len = 0 is passed to the _ex entry points; a value >= seqlen means one chunk. */
/* chunk_len = VMSCAN_CHUNK_LANE_SCAN selects, for seqlen <= 8192, the scan that spreads each
 * sequence over the lanes instead of splitting it into chunks: one workgroup per (batch, channel),
 * a run of 16 positions per lane, and the state carried between lanes by an associative scan of
 * (decay, state) pairs within each 1024-position wave segment ([P4] §3.2, the parallel cumulative
 * form; [P3] §3, the selective-scan kernel's block scan), so no chunk end state is recomputed.
 * Same results as the other paths up to rounding order; its workspace is the status word only.
 * Longer sequences return VMSCAN_ERR_UNSUPPORTED. */
#define VMSCAN_CHUNK_LANE_SCAN (-1)
int64_t vmscan_fwd_bidir_chunk_len(int64_t batch, int64_t dim, int64_t seqlen, int d_state);

/* Workspace bytes for vmscan_fwd_bidir / vmscan_fwd_bidir_ex (chunk_len 0 = library choice).
 * Returns 0 for invalid arguments. */
size_t vmscan_fwd_bidir_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                        vmscan_dtype dtype);
size_t vmscan_fwd_bidir_workspace_bytes_ex(int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                           vmscan_dtype dtype, int64_t chunk_len);

/*
 * Vision Mamba bidirectional (v2 scan inputs) selective scan, fused with the SiLU gate.
 *   out = ( y_f + flip(y_b') ) / 2 * silu(z)                       [P3] §2.2, §4.3; [P5] §2.2
 * where y_f is the scan above over t = 0..L-1 with (A_log, B, C, D) and y_b' is the same scan of
 * the reversed sequence (reversed u, Δ_raw) with (A_b_log, reversed B_b, reversed C_b, D_b).
 * The backward direction shares u, delta_raw, z and delta_bias with the forward one; B_b and C_b
 * are given in ORIGINAL token order.  No reversed copy is materialised.  The v1 variant of [P3]
 * §2.1 is obtained by passing B_b = B, C_b = C and D_b = D.
 *
 *   u, delta_raw, z : [batch, dim, seqlen]     activation dtype
 *   A_log, A_b_log  : [dim, d_state]           float32
 *   B, C, B_b, C_b  : [batch, d_state, seqlen] activation dtype, original token order
 *   D, D_b          : [dim]                    float32
 *   delta_bias      : [dim]                    float32 (shared by both directions)
 *   out             : [batch, dim, seqlen]     activation dtype
 * Long sequences are split into chunks whose boundary states are carried across workgroups
 * (chunk_len 0 = library choice; otherwise the given length, clamped to [1, min(seqlen, 206)]).
 * The workspace (size from vmscan_fwd_bidir_workspace_bytes[_ex]) holds a float32 copy of
 * B/C/B_b/C_b in position-major order and, for split sequences, the chunk end states.
 */
vmscan_status vmscan_fwd_bidir(const void *u, const void *delta_raw, const void *z,
                               const float *A_log, const float *A_b_log,
                               const void *B, const void *C, const void *B_b, const void *C_b,
                               const float *D, const float *D_b, const float *delta_bias,
                               void *out, int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                               vmscan_dtype dtype, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);
vmscan_status vmscan_fwd_bidir_ex(const void *u, const void *delta_raw, const void *z,
                                  const float *A_log, const float *A_b_log,
                                  const void *B, const void *C, const void *B_b, const void *C_b,
                                  const float *D, const float *D_b, const float *delta_bias,
                                  void *out, int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                  vmscan_dtype dtype, void *workspace, size_t workspace_bytes,
                                  int64_t chunk_len, hipStream_t stream);

/*
 * vmscan_fwd_bidir for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same computation, kernels and
 * results as vmscan_fwd_bidir (bit for bit), with the workspace taken from a fixed scratch
 * buffer of VMSCAN_SCRATCH_BYTES that the library holds in device memory (a file-scope device
 * array, one per GPU, loaded with the library's code object and kept until the process ends)
 * instead of a caller's workspace.  The caller still passes every input and the output, with
 * the layouts, validation and error codes of vmscan_fwd_bidir.  The call allocates nothing
 * (no hipMalloc/hipFree or allocating library routine); on its first call on a device it looks
 * up that device's copy of the buffer (hipGetSymbolAddress, with that device current).
 * A shape whose workspace (vmscan_fwd_bidir_workspace_bytes) exceeds VMSCAN_SCRATCH_BYTES
 * returns VMSCAN_ERR_SCRATCH before anything is enqueued; the other entry points take such shapes.
 * Every call on one GPU uses that GPU's one buffer: calls that overlap on one GPU (on different
 * streams or from different threads) race and give unspecified results; calls ordered on one
 * stream are safe.  The buffer keeps the last call's contents; the forward scan needs none of
 * them cleared.
 */
#define VMSCAN_SCRATCH_BYTES ((size_t)64 << 20)
vmscan_status vmscan_fwd_bidir_noalloc(const void *u, const void *delta_raw, const void *z,
                                       const float *A_log, const float *A_b_log,
                                       const void *B, const void *C, const void *B_b, const void *C_b,
                                       const float *D, const float *D_b, const float *delta_bias,
                                       void *out, int64_t batch, int64_t dim, int64_t seqlen,
                                       int d_state, vmscan_dtype dtype, hipStream_t stream);

/*
 * The two stages of vmscan_fwd_bidir_ex, for callers that time or overlap them separately:
 *   stage 1: preparation: the float32 position-major copy of B/C/B_b/C_b and, for a split
 *            sequence, each chunk's end state (scanned from zero) and Δ sum, in the workspace;
 *   stage 2: the fused bidirectional scan, which reads that copy and folds the carries into
 *            each chunk's initial state; it requires a completed stage 1 with the same inputs,
 *            shapes, chunk_len and workspace, else the output is unspecified;
 *   stage 3: both (= vmscan_fwd_bidir_ex).
 * Other stage values return VMSCAN_ERR_UNSUPPORTED.  Arguments as for vmscan_fwd_bidir_ex.
 */
vmscan_status vmscan_fwd_bidir_stage(const void *u, const void *delta_raw, const void *z,
                                     const float *A_log, const float *A_b_log,
                                     const void *B, const void *C, const void *B_b, const void *C_b,
                                     const float *D, const float *D_b, const float *delta_bias,
                                     void *out, int64_t batch, int64_t dim, int64_t seqlen,
                                     int d_state, vmscan_dtype dtype, void *workspace,
                                     size_t workspace_bytes, int64_t chunk_len, int stage,
                                     hipStream_t stream);

/*
 * The same bidirectional scan with a separate backward branch: in Vim's v2 parameter sets the
 * backward branch has its own convolution, input projection and Δ projection ([P3] §2.1), so
 * its scan input u_b, Δ input delta_raw_b and Δ bias delta_bias_b differ from the forward
 * branch's.  With y_f the scan of (u, delta_raw, delta_bias; A_log, B, C, D) and y_b' that of
 * the reversed (u_b, delta_raw_b; A_b_log, B_b, C_b, D_b) with delta_bias_b:
 *   out = ( y_f + flip(y_b') ) / 2 * silu(z)                       [P3] §2.2, §4.3
 *   u_b, delta_raw_b : [batch, dim, seqlen] activation dtype, ORIGINAL token order (the library
 *                      walks them backwards; no flipped copy is made)
 *   delta_bias_b     : [dim] float32
 * Any of u_b, delta_raw_b, delta_bias_b may alias the forward branch's tensor;
 * vmscan_fwd_bidir_stage(...) equals vmscan_fwd_bidir_v2_stage with u_b = u,
 * delta_raw_b = delta_raw and delta_bias_b = delta_bias.  All other arguments, the workspace
 * (same size query as vmscan_fwd_bidir_workspace_bytes[_ex]), chunk_len, stage, validation and
 * error codes are as for vmscan_fwd_bidir_ex / vmscan_fwd_bidir_stage; out must not alias any
 * input.
 */
vmscan_status vmscan_fwd_bidir_v2(const void *u, const void *delta_raw, const float *delta_bias,
                                  const void *u_b, const void *delta_raw_b, const float *delta_bias_b,
                                  const void *z, const float *A_log, const float *A_b_log,
                                  const void *B, const void *C, const void *B_b, const void *C_b,
                                  const float *D, const float *D_b, void *out,
                                  int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                  vmscan_dtype dtype, void *workspace, size_t workspace_bytes,
                                  int64_t chunk_len, hipStream_t stream);
vmscan_status vmscan_fwd_bidir_v2_stage(const void *u, const void *delta_raw, const float *delta_bias,
                                        const void *u_b, const void *delta_raw_b,
                                        const float *delta_bias_b, const void *z,
                                        const float *A_log, const float *A_b_log,
                                        const void *B, const void *C, const void *B_b, const void *C_b,
                                        const float *D, const float *D_b, void *out,
                                        int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                        vmscan_dtype dtype, void *workspace, size_t workspace_bytes,
                                        int64_t chunk_len, int stage, hipStream_t stream);

/*
 * Gradients of vmscan_fwd_bidir_v2 (the backward pass, for training).  The pages define the
 * forward and check its gradient numerically ([P5] §4 gradcheck); these are its exact
 * derivatives.  Given the forward's inputs and dout = dL/dout [batch, dim, seqlen]:
 *   du, ddelta_raw, du_b, ddelta_raw_b, dz   : [batch, dim, seqlen]  activation dtype
 *   dB, dC, dB_b, dC_b                       : [batch, 16, seqlen]   activation dtype
 *   dA_log, dA_b_log                         : [dim, 16]             float32
 *   dD, dD_b, ddelta_bias, ddelta_bias_b     : [dim]                 float32
 * Every gradient is written (not accumulated), summed over batch where the tensor has no batch
 * dimension, in float32 and rounded once.  du_b, ddelta_raw_b and ddelta_bias_b may each be
 * NULL: the backward branch's gradient for that input is then ADDED to the forward branch's
 * output (du, ddelta_raw, ddelta_bias), which is the gradient of vmscan_fwd_bidir, whose two
 * branches share u, delta_raw and delta_bias (pass the same tensor as u_b etc. then).
 * The library recomputes the forward: it runs the forward scan, which turns the un-gated sum into
 * dz and the scan's output gradient at once (the sum itself is not stored), and it stores the
 * state at window boundaries (in that scan when the sequence is not split, else in a second
 * forward pass per direction), then walks backwards over the sequence with the adjoint
 * recurrence, window by window from those states.  A long sequence with few (batch, channel-group) tiles
 * is split into chunks, the adjoint carry between them coming from a reverse carry pass; the
 * result does not depend on the split beyond float32 rounding order.  Workspace:
 * vmscan_bwd_bidir_v2_workspace_bytes.
 * Gradient outputs must not alias each other or any input.  Validation and error codes as for
 * vmscan_fwd_bidir_v2 (all pointers but the three optional ones are required, all 16-byte
 * aligned); launches are asynchronous on `stream`.  d_state 16 or 32 (B, C, dB, dC are then
 * [batch, d_state, seqlen]; A_log, dA_log [dim, d_state]).
 */
size_t vmscan_bwd_bidir_v2_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                           vmscan_dtype dtype);
vmscan_status vmscan_bwd_bidir_v2(const void *u, const void *delta_raw, const float *delta_bias,
                                  const void *u_b, const void *delta_raw_b, const float *delta_bias_b,
                                  const void *z, const float *A_log, const float *A_b_log,
                                  const void *B, const void *C, const void *B_b, const void *C_b,
                                  const float *D, const float *D_b, const void *dout,
                                  void *du, void *ddelta_raw, float *ddelta_bias,
                                  void *du_b, void *ddelta_raw_b, float *ddelta_bias_b,
                                  void *dz, float *dA_log, float *dA_b_log,
                                  void *dB, void *dC, void *dB_b, void *dC_b, float *dD, float *dD_b,
                                  int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                  vmscan_dtype dtype, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * Gradients of ss2d_cross_scan_fwd (the SS2D backward pass).  Given the forward's inputs and
 * dout = dL/dout [batch, dim, H, W]:
 *   dx                 : [batch, dim, H, W]          activation dtype
 *   ddelta_raw         : [batch, 4, dim, H*W]        activation dtype, each direction's scan order
 *   dB, dC             : [batch, 4, N, H*W]          activation dtype, each direction's scan order
 *   dA_log             : [4, dim, N]                 float32  (N = d_state, 16 or 32)
 *   dD, ddelta_bias    : [4, dim]                    float32
 *   dz                 : [batch, dim, H, W]          activation dtype; NULL exactly when z is NULL
 * Every gradient is written (not accumulated), batch-summed where the tensor has no batch
 * dimension, in float32 and rounded once.  The gradient reaching direction k is dout silu(z)
 * (or dout) in that direction's scan order; each direction's adjoint is walked as in
 * vmscan_bwd_bidir_v2 and its du is mapped back to pixels and summed into dx.  With a gate the
 * library first recomputes the un-gated forward sum for dz.  Workspace:
 * ss2d_cross_scan_bwd_workspace_bytes.  Outputs must not alias each other or any input.
 * Validation and error codes as for ss2d_cross_scan_fwd (z and dz must both be given or both be
 * NULL, else VMSCAN_ERR_NULL); launches are asynchronous on `stream`.  d_state 16 or 32.
 */
size_t ss2d_cross_scan_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                           vmscan_dtype dtype);
vmscan_status ss2d_cross_scan_bwd(const void *x, const void *delta_raw, const float *A_log,
                                  const void *B, const void *C, const float *D, const float *delta_bias,
                                  const void *z, const void *dout, void *dx, void *ddelta_raw,
                                  float *dA_log, void *dB, void *dC, float *dD, float *ddelta_bias,
                                  void *dz, int64_t batch, int64_t dim, int64_t H, int64_t W,
                                  int d_state, vmscan_dtype dtype, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for ss2d_cross_scan_fwd / _ex (chunk_len 0 = library choice); 0 if invalid. */
size_t ss2d_cross_scan_workspace_bytes(int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                       vmscan_dtype dtype);
size_t ss2d_cross_scan_workspace_bytes_ex(int64_t batch, int64_t dim, int64_t H, int64_t W,
                                          int d_state, vmscan_dtype dtype, int64_t chunk_len);

/*
 * VMamba SS2D cross-scan and cross-merge ([P4] §2.2, §3.1).  Direction k scans x in order
 *   k=0 row-major, k=1 column-major, k=2 reversed row-major, k=3 reversed column-major,
 * each with its own delta_raw[:,k], B[:,k], C[:,k] (stored in THAT direction's scan order),
 * A_log[k], D[k] and delta_bias[k], without a gate.  The four outputs are mapped back to
 * row-major pixels and summed in fp32:  out = Σ_k y_k  (times silu(z) when z is not NULL).
 *
 *   x          : [batch, dim, H, W]          activation dtype
 *   delta_raw  : [batch, 4, dim, H*W]        activation dtype, scan order of each direction
 *   A_log      : [4, dim, d_state]           float32
 *   B, C       : [batch, 4, d_state, H*W]    activation dtype, scan order of each direction
 *   D          : [4, dim]                    float32
 *   delta_bias : [4, dim]                    float32
 *   z          : [batch, dim, H, W] or NULL  activation dtype
 *   out        : [batch, dim, H, W]          activation dtype
 * H*W must be < 2^31.  Sequences are either cut into chunks of at most 206 positions (an LDS row),
 * whose entering states come from a chunk pass and a carry prefix, or walked whole, each pair's
 * two directions meeting in float32 rows in the workspace that a merge kernel then sums per
 * pixel.  The library walks whole when H*W > 206 and batch * ceil(dim / 64) >= 256 (enough
 * (batch, channel-group) tiles to fill the GPU without chunks); chunk_len >= H*W asks for the
 * whole walk, 0 < chunk_len < H*W for chunks of that length (at most 206).
 */
vmscan_status ss2d_cross_scan_fwd(const void *x, const void *delta_raw, const float *A_log,
                                  const void *B, const void *C, const float *D,
                                  const float *delta_bias, const void *z, void *out,
                                  int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                  vmscan_dtype dtype, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);
vmscan_status ss2d_cross_scan_fwd_ex(const void *x, const void *delta_raw, const float *A_log,
                                     const void *B, const void *C, const float *D,
                                     const float *delta_bias, const void *z, void *out,
                                     int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                     vmscan_dtype dtype, void *workspace, size_t workspace_bytes,
                                     int64_t chunk_len, hipStream_t stream);

/*
 * ss2d_cross_scan_fwd_ex with x's transposed copy supplied by the caller (for instance the xT_out
 * of ss2d_conv2d_silu_fwd): xT [batch, dim, W, H], activation dtype, must equal x transposed in
 * its last two dimensions; the column-major scans read it instead of a copy made here.  xT NULL
 * gives VMSCAN_ERR_NULL; the rest (arguments, workspace query, errors) as ss2d_cross_scan_fwd_ex.
 */
vmscan_status ss2d_cross_scan_fwd_xt(const void *x, const void *xT, const void *delta_raw,
                                     const float *A_log, const void *B, const void *C, const float *D,
                                     const float *delta_bias, const void *z, void *out,
                                     int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                     vmscan_dtype dtype, void *workspace, size_t workspace_bytes,
                                     int64_t chunk_len, hipStream_t stream);

/*
 * Front of the Vim scan: the depthwise convolution + SiLU that produces the scan input u
 * ([P3] §2.1: each branch's Conv1d of width d_conv over the d_inner channels, v2's conv1d_b for
 * the backward branch; §2.2: the backward branch works on the flipped sequence).  Per
 * (batch b, channel d, position t), with K = d_conv:
 *   u[b,d,t]   = silu(conv_b[d]   + Σ_k conv_w[d,k]   x[b,d,t-(K-1)+k])      (causal)
 *   u_b[b,d,t] = silu(conv_b_b[d] + Σ_k conv_w_b[d,k] x[b,d,t+(K-1)-k])      (the flipped branch's
 *                causal convolution, stored in original token order as vmscan_fwd_bidir_v2's u_b)
 * with x = 0 outside [0, seqlen).  v1 (shared convolution): pass conv_w and conv_b again as
 * conv_w_b and conv_b_b.
 *   x, u, u_b            : [batch, dim, seqlen]   activation dtype
 *   conv_w, conv_w_b     : [dim, d_conv]          float32, d_conv in 1..4
 *   conv_b, conv_b_b     : [dim]                  float32
 * conv_w_b, conv_b_b and u_b are all NULL (forward branch only) or all set (else
 * VMSCAN_ERR_NULL).  x is read once; u and u_b are written once, rounded once.  Outputs must not
 * alias x.  No workspace.  Errors as for the other entry points.
 */
vmscan_status vmscan_conv1d_silu_fwd(const void *x, const float *conv_w, const float *conv_b,
                                     const float *conv_w_b, const float *conv_b_b, void *u, void *u_b,
                                     int64_t batch, int64_t dim, int64_t seqlen, int d_conv,
                                     vmscan_dtype dtype, hipStream_t stream);

/*
 * Front of SS2D: the depthwise 3 x 3 convolution ([P4] §2.1, d_conv = 3 in its table), optionally
 * followed by SiLU, written in the two layouts the cross-scan reads:
 *   pre[b,d,i,j] = conv_b[d] + Σ_{a,c} conv_w[d,a,c] x[b,d,i-1+a,j-1+c]   (zero padding)
 *   x_out[b,d,i,j] = xT_out[b,d,j,i] = act ? silu(pre) : pre
 *   x, x_out             : [batch, dim, H, W]     activation dtype
 *   xT_out               : [batch, dim, W, H]     activation dtype, or NULL (row-major only)
 *   conv_w               : [dim, 3, 3]            float32
 *   conv_b               : [dim]                  float32
 * d_conv must be 3 and act 0 or 1 (else VMSCAN_ERR_UNSUPPORTED).  x is read once, each output
 * written once; both hold the same rounded values.  Outputs must not alias x.  No workspace.
 */
vmscan_status ss2d_conv2d_silu_fwd(const void *x, const float *conv_w, const float *conv_b, int act,
                                   void *x_out, void *xT_out, int64_t batch, int64_t dim, int64_t H,
                                   int64_t W, int d_conv, vmscan_dtype dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VMSCAN_H */
