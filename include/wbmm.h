/*
 * wbmm.h — C ABI of libwbmm: WBMM (Windowed Batch Matrix Multiplication) on AMD MI355X (gfx950).
 *
 * WBMM cuts a feature map into non-overlapping w x w windows (d = w*w pixels), builds for every
 * channel c a d x d matrix M_c from a compact (2w-1) x (2w-1) relative-position table T_c, and
 * mixes every window of every image with one shared matmul out = M_c . x, with no softmax
 * [gecl.asia reading notes, "Core Idea"; arxivdaily abstract; pith page, Fig. 1 caption].
 *
 * Conventions shared by every entry point:
 *   - Index orientation: M_c[i][j] = T_c[(y_i - y_j) + w - 1][(x_i - x_j) + w - 1], in-window
 *     position i = y_i * w + x_i (row-major); the table's first axis is vertical.
 *   - Every pointer argument named as device memory must be a device (HBM) address on the current
 *     HIP device, aligned to its element size (workspaces: see each call).
 *   - The caller owns every buffer. The library never allocates or frees device memory and never
 *     synchronizes: all work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream) and runs asynchronously.
 *   - Arguments are validated on the host before anything is enqueued. On any status other than
 *     WBMM_OK nothing has been enqueued (except WBMM_E_HIP, which reports a failed launch) and
 *     wbmm_last_error() returns a message for the calling thread.
 *   - Outputs are overwritten, never accumulated into.
 *   - Tensor layouts: feature maps are (B, C, H, W) in WBMM_NCHW or (B, H, W, C) in WBMM_NHWC,
 *     dense, no strides. Tables are (C, 2w-1, 2w-1), matrices (C, d, d), mix weights (C, 3, 3),
 *     all dense row-major.
 *   - H and W need not be multiples of w: the map is treated as zero-padded at the bottom and
 *     right to the next multiple of w, and outputs are cropped back to H x W.
 */
#ifndef WBMM_H
#define WBMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WBMM_ABI_VERSION 1

typedef enum wbmm_status {
  WBMM_OK = 0,
  WBMM_E_INVALID = 1,      /* a size, pointer or combination of arguments is invalid          */
  WBMM_E_UNSUPPORTED = 2,  /* valid request this build does not provide (e.g. misalignment)   */
  WBMM_E_WORKSPACE = 3,    /* workspace missing or smaller than the matching *_bytes query    */
  WBMM_E_HIP = 4           /* a HIP launch failed; wbmm_last_error() carries HIP's message    */
} wbmm_status;

typedef enum wbmm_dtype { WBMM_F32 = 0, WBMM_BF16 = 1 } wbmm_dtype;
typedef enum wbmm_layout { WBMM_NCHW = 0, WBMM_NHWC = 1 } wbmm_layout;

/* ABI version this library was built with (WBMM_ABI_VERSION). */
int wbmm_abi_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if none). The pointer
 * stays valid until the next wbmm_* call on the same thread. */
const char* wbmm_last_error(void);

/*
 * wbmm_build_index — relative-position index of one window.
 * Defines: the table lookup that turns an in-window pair (i, j) into a table entry
 *          [gecl.asia reading notes, "Core Idea" and "Method" point 2].
 *   idx[i*d + j] = ((y_i - y_j) + w - 1) * (2w - 1) + ((x_i - x_j) + w - 1)   (int32, d x d)
 * w:   window side, 1 <= w <= 32.
 * idx: device, int32 [d*d], written.
 * Bit-exact. Errors: WBMM_E_INVALID for w out of range or idx == NULL.
 */
wbmm_status wbmm_build_index(int w, int32_t* idx, void* stream);

/*
 * wbmm_build_matrix — materialize M_c from the table (the pages' inference caching of the
 * constructed weights) [gecl.asia reading notes, "Core Idea"; "Method", last sentence].
 *   M[c][i][j] = T[c][idx[i][j]]   (an exact copy in the table's dtype)
 * T: device [C][2w-1][2w-1], dtype `dtype` (WBMM_F32 or WBMM_BF16).
 * M: device [C][d][d], same dtype, written. Must not overlap T.
 * Bit-exact. Errors: WBMM_E_INVALID for C < 1, w out of range, NULL pointers, bad dtype.
 */
wbmm_status wbmm_build_matrix(const void* T, int C, int w, int dtype, void* M, void* stream);

/*
 * wbmm_fold_hier — fold an s x s sub-window table into a w x w window matrix (hierarchical
 * window reparameterization, zero inference cost) [gecl.asia reading notes, "Method" point 4;
 * arxivdaily abstract].
 *   For pairs (i, j) in the same s x s sub-window (sub-windows tile the window from its origin):
 *     M_out[c][i][j] = M_in[c][i][j] + T_sub[c][idx_s(i, j)]   (one add in `dtype`, RNE)
 *   otherwise M_out[c][i][j] = M_in[c][i][j]; idx_s is wbmm_build_index's formula with s for w
 *   applied to the in-sub-window coordinates (y mod s, x mod s).
 * M_in:  device [C][d][d]; T_sub: device [C][2s-1][2s-1]; M_out: device [C][d][d], written;
 *        M_out may equal M_in (in place) but must not partially overlap it.
 * s must divide w and 1 <= s < w. dtype WBMM_F32 or WBMM_BF16 (bf16 adds round to bf16, RNE).
 * Bit-exact. Errors: WBMM_E_INVALID for bad sizes, s not dividing w, NULL pointers.
 */
wbmm_status wbmm_fold_hier(const void* M_in, const void* T_sub, int C, int w, int s, int dtype,
                           void* M_out, void* stream);

/*
 * wbmm_forward_workspace_bytes — device workspace wbmm_forward needs for these arguments
 * (0 when none), the largest need over fp32 and bf16 inputs and outputs (a bf16 z_save with the
 * mix in window mode takes the fp32 pre-mix map through the workspace; bf16 maps with the mix
 * on the fast bf16 shapes keep z there when no z_save is given). Returns 0 for invalid
 * arguments as well; wbmm_forward reports those.
 */
size_t wbmm_forward_workspace_bytes(int B, int C, int H, int W, int w, int layout, int has_mix,
                                    int has_z_save);

/*
 * wbmm_forward — the WBMM layer forward [gecl.asia reading notes, "Core Idea", "Method";
 * pith page, "Core claim"; arxivdaily abstract].
 *   z = crop(reverse(M_c . partition(pad(x))))   for every channel c, window and image;
 *   y = mix3x3(z, mix_w) if mix_w != NULL, else y = z.
 * mix3x3 is the inter-block 3x3 depthwise cross-correlation, zero padding 1, stride 1, no bias:
 *   y[b,c,h,v] = sum_{u,t in 0..2} mix_w[c,u,t] * z[b,c,h+u-1,v+t-1]  (z = 0 outside the map)
 *   [gecl.asia reading notes, "Method" point 3].
 * Sizes: B, C, H, W >= 1; 1 <= w <= 32.
 * layout:    WBMM_NCHW or WBMM_NHWC (x, y and z_save share it).
 * in_dtype:  WBMM_F32 or WBMM_BF16 for x and for T/M. Products accumulate in fp32.
 * out_dtype: WBMM_F32 or WBMM_BF16 for y and z_save (bf16 outputs are rounded RNE from fp32).
 * x:      device map, in_dtype.
 * T, M:   exactly one non-NULL. T: device [C][2w-1][2w-1] — M_c is formed on chip from T_c.
 *         M: device [C][d][d] — the cached (possibly folded) matrices are read from memory.
 * mix_w:  device fp32 [C][3][3] or NULL. The mix runs in fp32 on the fp32 pre-mix map; with
 *         bf16 output, y and z_save are rounded from it (RNE).
 * z_save: device map in out_dtype receiving the pre-mix output z (for the backward), or NULL.
 * y:      device map in out_dtype, written; must not overlap x, T, M, mix_w or z_save.
 * workspace / workspace_bytes: device scratch of at least wbmm_forward_workspace_bytes(...)
 *         bytes (may be NULL when that is 0).
 * Errors: WBMM_E_INVALID (sizes, pointers, both or neither of T/M, overlap of y with x),
 *         WBMM_E_UNSUPPORTED (misaligned pointer), WBMM_E_WORKSPACE, WBMM_E_HIP.
 */
wbmm_status wbmm_forward(int B, int C, int H, int W, int w, int layout, int in_dtype,
                         int out_dtype, const void* x, const void* T, const void* M,
                         const float* mix_w, void* z_save, void* y, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * wbmm_backward_workspace_bytes — device workspace wbmm_backward needs (per-workgroup fp64
 * partial tables, and a dz buffer when the mix cannot be fused). Returns 0 for invalid arguments.
 */
size_t wbmm_backward_workspace_bytes(int B, int C, int H, int W, int w, int layout, int has_mix);

/*
 * wbmm_backward — gradients of wbmm_forward (fp32). The pages train with the operator but do not
 * write out its backward; it follows from the forward by the chain rule:
 *   dz    = mix3x3 adjoint of dy (correlation with the 180-degree rotated mix_w), or dy if no mix;
 *   dmix_w[c,u,t] = sum_{b,h,v} dy[b,c,h,v] * z[b,c,h+u-1,v+t-1];
 *   G_c   = partition(pad(dz));  dx = crop(reverse(M_c^T . G_c));
 *   dT[c][k] = sum over pairs (i,j) with idx[i][j] = k of (G_c . X_c^T)[i][j].
 * x, dy:   device fp32 maps in `layout`.
 * T, M:    exactly one non-NULL (as in wbmm_forward; with M, dT is the gradient with respect to
 *          the table that M was gathered from).
 * mix_w:   device fp32 [C][3][3] or NULL; z_saved (the forward's z_save) is required iff mix_w.
 * dx:      device fp32 map, written, or NULL to skip.
 * dT:      device fp32 [C][2w-1][2w-1], written, or NULL to skip.
 * dmix_w:  device fp32 [C][3][3], written, or NULL to skip (ignored without mix_w).
 * workspace / workspace_bytes: device scratch of at least wbmm_backward_workspace_bytes(...)
 *          bytes, 256-byte aligned; no initial contents are required. Calls that share a
 *          workspace must be ordered on one stream.
 * dT and dmix_w are reduced in a fixed order (fp64 per-workgroup partials summed by a second,
 * small kernel; no floating-point atomics): results are bitwise reproducible run to run.
 * Windows 1 <= w <= 32 (16 < w <= 32: dx through the forward contraction with the table
 * rotated by 180 degrees or the matrix transposed, whose matrix is M^T; dT from row-pair tiles
 * of 32 x 32, with the windows as the sum dimension).
 * Errors: WBMM_E_INVALID, WBMM_E_UNSUPPORTED (misaligned pointer), WBMM_E_WORKSPACE,
 *         WBMM_E_HIP.
 */
wbmm_status wbmm_backward(int B, int C, int H, int W, int w, int layout, const float* x,
                          const float* T, const float* M, const float* mix_w,
                          const float* z_saved, const float* dy, float* dx, float* dT,
                          float* dmix_w, void* workspace, size_t workspace_bytes, void* stream);

/*
 * wbmm_backward_noalloc — wbmm_backward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving or training loops, harnesses that forbid hipMalloc):
 * the same gradients, arguments and errors, minus the workspace. The scratch that the backward
 * needs (per-workgroup fp64 partials, a dz map) is a fixed device array inside the library, one
 * copy per GPU, held until the process ends: WBMM_NOALLOC_SCRATCH_BYTES bytes. A problem whose
 * wbmm_backward_workspace_bytes(...) exceeds that is rejected with WBMM_E_UNSUPPORTED. The call
 * allocates and frees nothing and needs no initial contents in the scratch. Every call on one
 * GPU shares that GPU's scratch: calls that may overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller; calls on one stream are ordered.
 */
#define WBMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
wbmm_status wbmm_backward_noalloc(int B, int C, int H, int W, int w, int layout, const float* x,
                                  const float* T, const float* M, const float* mix_w,
                                  const float* z_saved, const float* dy, float* dx, float* dT,
                                  float* dmix_w, void* stream);

/*
 * wbmm_forward_hier_workspace_bytes — device workspace wbmm_forward_hier needs (0 when none, and
 * 0 for invalid arguments, which wbmm_forward_hier reports).
 */
size_t wbmm_forward_hier_workspace_bytes(int B, int C, int H, int W, int w, int s, int layout,
                                         int has_mix, int has_z_save);

/*
 * wbmm_forward_hier — the layer forward with the hierarchical reparameterization folded on chip
 * [gecl.asia reading notes, "Method" point 4: a sub-window table overlays 7x7 structure in a
 * 14x14 window at no inference cost]. The matrix is
 *   M'_c[i][j] = M_c[i][j] + T_sub[c][idx_s(i, j)]   for pairs i, j in one s x s sub-window,
 *   M'_c[i][j] = M_c[i][j]                           otherwise,
 * each sum one fp32 add (RNE): exactly what wbmm_fold_hier stores. Then z and y as in
 * wbmm_forward. fp32 only; s divides w and s < w. For w = 2s (the sub-windows are the window's
 * quadrants) the fold happens on chip and M' is never formed in memory; for other s, M' is
 * built and folded in the workspace (C w^4 floats) and read as a cached matrix.
 * x, y, z_save: device fp32 maps in `layout`; T: device fp32 [C][2w-1][2w-1];
 * T_sub: device fp32 [C][2s-1][2s-1]; mix_w, z_save, workspace as in wbmm_forward
 * (workspace size from wbmm_forward_hier_workspace_bytes).
 * Errors: WBMM_E_INVALID (sizes, s not dividing w or not below it, NULL or overlapping
 *         pointers), WBMM_E_UNSUPPORTED (no launch shape, misaligned pointer), WBMM_E_WORKSPACE,
 *         WBMM_E_HIP.
 */
wbmm_status wbmm_forward_hier(int B, int C, int H, int W, int w, int s, int layout, const float* x,
                              const float* T, const float* T_sub, const float* mix_w,
                              float* z_save, float* y, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * wbmm_backward_hier_workspace_bytes — device workspace wbmm_backward_hier needs (0 for invalid
 * arguments).
 */
size_t wbmm_backward_hier_workspace_bytes(int B, int C, int H, int W, int w, int s, int layout,
                                          int has_mix);

/*
 * wbmm_backward_hier — gradients of wbmm_forward_hier (fp32). As wbmm_backward with M' in place
 * of M, and in addition the sub-table's gradient:
 *   dx = crop(reverse(M'_c^T . G_c));   dT[c][k] = sum over pairs (i,j) with idx[i][j] = k of
 *   (G_c . X_c^T)[i][j];   dT_sub[c][k'] = the same sum over the pairs inside one s x s
 *   sub-window with idx_s[i][j] = k'.
 * T, T_sub: as in wbmm_forward_hier. dx, dT, dT_sub, dmix_w: written, or NULL to skip
 * (dT_sub: device fp32 [C][2s-1][2s-1]). mix_w, z_saved, dy, workspace as in wbmm_backward.
 * dT, dT_sub and dmix_w are reduced in a fixed order: bitwise reproducible run to run.
 * Any s dividing w with s < w, 1 <= w <= 32: for w = 2s on chip; for other s with M' built in
 * the workspace, dX and dT from the cached-matrix backward, and dT_sub as the table gradient of
 * an s-window layer on the same G and x (a pair of one sub-window is a pair of one window of
 * the s-grid, which the w-grid subdivides).
 * Errors: WBMM_E_INVALID (as wbmm_forward_hier), WBMM_E_UNSUPPORTED (no launch shape,
 *         misaligned pointer), WBMM_E_WORKSPACE, WBMM_E_HIP.
 */
wbmm_status wbmm_backward_hier(int B, int C, int H, int W, int w, int s, int layout,
                               const float* x, const float* T, const float* T_sub,
                               const float* mix_w, const float* z_saved, const float* dy,
                               float* dx, float* dT, float* dT_sub, float* dmix_w,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * wbmm_forward_shifted_workspace_bytes / wbmm_forward_shifted — wbmm_forward on a window grid
 * offset by (oy, ox), 0 <= oy, ox < w: the interleaved grid that alternate layers can use so
 * that information crosses window borders [gecl.asia reading notes, "Limitations": interleaving
 * windows between layers]. Window (wy, wx) covers map rows wy*w - oy .. wy*w - oy + w - 1 and
 * columns wx*w - ox .. wx*w - ox + w - 1; the pixels of a border window that lie outside the map
 * are zeros (no cyclic roll), and only positions inside the map are written. (0, 0) is exactly
 * wbmm_forward. Every other argument, layout, dtype and error as in wbmm_forward; an offset
 * outside [0, w) is WBMM_E_INVALID.
 */
size_t wbmm_forward_shifted_workspace_bytes(int B, int C, int H, int W, int w, int oy, int ox,
                                            int layout, int has_mix, int has_z_save);
wbmm_status wbmm_forward_shifted(int B, int C, int H, int W, int w, int oy, int ox, int layout,
                                 int in_dtype, int out_dtype, const void* x, const void* T,
                                 const void* M, const float* mix_w, void* z_save, void* y,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * wbmm_backward_shifted_workspace_bytes / wbmm_backward_shifted — the gradients of
 * wbmm_forward_shifted (dx, dT, dmix_w), with the arguments, outputs and errors of wbmm_backward
 * plus the grid offset (oy, ox) of the forward. The padding pixels are constants: dT sums the
 * pair products of the map's own pixels only.
 */
size_t wbmm_backward_shifted_workspace_bytes(int B, int C, int H, int W, int w, int oy, int ox,
                                             int layout, int has_mix);
wbmm_status wbmm_backward_shifted(int B, int C, int H, int W, int w, int oy, int ox, int layout,
                                  const float* x, const float* T, const float* M,
                                  const float* mix_w, const float* z_saved, const float* dy,
                                  float* dx, float* dT, float* dmix_w, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * wbmm_dwconv_forward — the standard k x k depthwise convolution (DW-Std) that the pages time
 * WBMM against: every output gathers the k*k neighbours around its own position in its own
 * channel [pith page, Fig. 1 and Fig. 2 captions; operator benchmark, Fig. 3 caption]. Not part of
 * a WBMM layer; provided so the comparison runs on the same hardware.
 *   y[b,c,h,v] = sum_{u,t in 0..k-1} w_dw[c,u,t] * x[b,c,h+u-p,v+t-p],  p = k / 2,
 *   x taken as 0 outside the map (cross-correlation, stride 1, no bias: the frameworks' form).
 * Sizes: B, C, H, W >= 1; k odd, 3 <= k <= 13 (WBMM_E_UNSUPPORTED otherwise, and for rows too
 *         long for one workgroup's staging buffer, about 600 pixels).
 * x:    device fp32 NCHW [B][C][H][W].
 * w_dw: device fp32 [C][k][k].
 * y:    device fp32 NCHW [B][C][H][W], written; must not overlap x or w_dw.
 * Accumulates in fp32 (one fma per tap, taps in row-major order). Enqueued on `stream`; no
 * workspace. Errors: WBMM_E_INVALID (sizes, even k, NULL, overlap), WBMM_E_UNSUPPORTED (k or
 * row length out of range, misaligned pointers), WBMM_E_HIP (launch failure).
 */
wbmm_status wbmm_dwconv_forward(int B, int C, int H, int W, int k, const float* x,
                                const float* w_dw, float* y, void* stream);

/*
 * wbmm_backward_bf16_workspace_bytes / wbmm_backward_bf16 — the layer backward with bf16 maps
 * (mixed-precision training): x, dy, z_saved and dx in bf16, T in bf16 (the forward's table),
 * dT and dmix_w in fp32. Same gradients as wbmm_backward (derived by the chain rule; the pages
 * train with the operator [arxivdaily abstract]):
 *   G = mix adjoint of dy (kept as a bf16 map, RNE), or dy itself without a mix;
 *   dx = M_c^T G per window (bf16 matrix cores, fp32 accumulation, RNE to bf16);
 *   dT_c[k] = sum over pairs with idx = k of (G X^T)[i][j] (bf16 products, fp32 sums over a
 *   group of windows, fp64 across groups in a fixed order); dmix_w as in wbmm_backward.
 * Any 1 <= w <= 32, NCHW or NHWC (`layout`), any map size; w = 14 on NCHW 28x28 or 56x56 maps
 * runs the bf16 matrix-core kernels, other shapes the fp32 kernels on the bf16 values (widened
 * exactly), with dx rounded to bf16 (RNE).
 * mix_w / z_saved: both or neither. dx, dT, dmix_w may each be NULL (skipped). bf16 maps and T
 * must be 16-byte aligned. workspace: at least wbmm_backward_bf16_workspace_bytes(...) bytes,
 * 256-byte aligned (never NULL: the dT partials live there). Errors as in wbmm_backward.
 */
size_t wbmm_backward_bf16_workspace_bytes(int B, int C, int H, int W, int w, int layout,
                                          int has_mix);
wbmm_status wbmm_backward_bf16(int B, int C, int H, int W, int w, int layout, const void* x,
                               const void* T, const float* mix_w, const void* z_saved,
                               const void* dy, void* dx, float* dT, float* dmix_w,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * wbmm_probe_mfma — measurement aid, not part of the method: a matrix-core peak probe. Launches
 * `blocks` workgroups of 4 waves; every wave runs `iters` rounds of 8 independent MFMA
 * accumulation chains on register operands (dtype WBMM_F32: v_mfma_f32_16x16x4f32, WBMM_BF16:
 * v_mfma_f32_16x16x32_bf16) and writes one float per lane to out (device, blocks * 256 floats),
 * so the sustained matrix rate on this part and clock can be set beside the datasheet peak.
 * wbmm_probe_mfma_flops returns the flops of such a launch (0 for invalid arguments).
 * wbmm_set_launch_events attaches to it like to the main kernel of the other calls.
 * Errors: WBMM_E_INVALID (dtype, blocks or iters < 1, NULL or misaligned out), WBMM_E_HIP.
 */
double wbmm_probe_mfma_flops(int dtype, int blocks, int iters);
wbmm_status wbmm_probe_mfma(int dtype, int blocks, int iters, float* out, void* stream);

/*
 * wbmm_set_launch_events — measurement aid, not part of the method. The next wbmm_forward,
 * wbmm_backward (or their _hier, _shifted and _bf16 forms), wbmm_dwconv_forward or wbmm_probe_mfma
 * call made on the calling thread
 * attaches `before` and `after` (hipEvent_t
 * handles passed as void*) to the dispatch of its main contraction kernel (hipExtLaunchKernel's
 * start and stop events), so their elapsed time is that kernel's execution; the pair is then
 * cleared. Both NULL clears a pending pair. The caller owns the events. Errors: WBMM_E_INVALID
 * when exactly one of the two is NULL.
 */
wbmm_status wbmm_set_launch_events(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* WBMM_H */
