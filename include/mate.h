/*
 * mate.h -- C ABI of the MI355X (gfx950) forward core of LinGen's MATE block.
 *
 * The MATE block replaces DiT self-attention with two branches (QbitAI article
 * on LinGen, section "方法"; arXiv-daily abstract of "LinGen: Towards
 * High-Resolution Minute-Length Text-to-Video Generation with Linear
 * Computational Complexity"):
 *   - the MA branch: Rotary Major Scan (RMS) of the T x H x W latent tokens,
 *     average-pooled review tokens put in front, and a bidirectional Mamba2
 *     (SSD) scan over the sequence and its flip;
 *   - the TE branch: TESA, attention inside 3D windows Tw x Sw x Sw whose
 *     partition shifts on alternate layers.
 * This library computes that token-mixing core, and (mate_layer) one whole
 * MATE layer with the projections around it.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA storage).
 *     The caller owns every buffer; the library never allocates or frees
 *     device memory for them and creates no streams (the HIP events of the
 *     timing diagnostics below aside). The device memory it holds is the fixed
 *     scratch array of mate_bissd_scan_noalloc, loaded with the library, and
 *     what hipBLASLt keeps for the handle mate_layer creates on first use.
 *   - Token tensors are channels-last: [batch][T][H][W][...], so the canonical
 *     token index is n = (t*H + h)*W + w and a token's channels are contiguous.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *     call enqueues its kernels asynchronously on it and returns; nothing
 *     synchronises. Calls are thread-safe; buffers used by calls in flight on
 *     different streams must not overlap.
 *   - Arguments are validated on the host before anything is launched. A call
 *     that returns a status other than MATE_OK has launched nothing and written
 *     nothing; mate_last_error() then describes why (thread-local string).
 *   - Token tensors (x, b, c, y, q, k, v, o) must be 16-byte aligned (torch
 *     and hipMalloc allocations are); otherwise MATE_ERR_UNSUPPORTED.
 *   - bf16 means bfloat16 (1 sign, 8 exponent, 7 mantissa bits); arithmetic is
 *     fp32 inside, results are rounded to nearest-even on store.
 */
#ifndef MATE_H
#define MATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MATE_ABI_VERSION 1
#define MATE_ORDER_ZIGZAG 4

typedef enum {
    MATE_OK = 0,
    MATE_ERR_NULL = 1,        /* a required pointer is NULL */
    MATE_ERR_SHAPE = 2,       /* an extent <= 0, order not in 0..4, window/pool not dividing
                                 the grid, shift outside [0, window), heads not divisible by
                                 groups, chunk < 1 */
    MATE_ERR_UNSUPPORTED = 3, /* legal for the method but not built (e.g. a head size the
                                 kernels are not instantiated for; a batch, head count or
                                 review-token count above 65535, the launch grids' y and z
                                 extents; more than 2^22 scan chunks per sequence or window
                                 regions, or 2^26 Mamba channels) */
    MATE_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than the *_workspace_size result */
    MATE_ERR_DEVICE = 5       /* a HIP call or kernel launch failed */
} mate_status;

typedef enum { MATE_F32 = 0, MATE_BF16 = 1 } mate_dtype;

/* Kernel family. AUTO picks the MFMA kernels when the shape has them and the
 * portable kernels otherwise; the other values force one family (FAST returns
 * MATE_ERR_UNSUPPORTED when the shape has no MFMA kernel). Both compute the
 * same result up to rounding order, within the input range that
 * mate_bissd_scan states for its MFMA kernels. */
typedef enum { MATE_ALGO_AUTO = 0, MATE_ALGO_PORTABLE = 1, MATE_ALGO_FAST = 2 } mate_algo;

typedef struct {
    int64_t batch, T, H, W;
} mate_grid;

/* ------------------------------------------------------------------------ */
/* Rotary Major Scan                                                         */
/* ------------------------------------------------------------------------ */
/* Unrolls the T x H x W token tensor into one of four 1D orders that differ in
 * which axis is unrolled first (QbitAI article, section "方法", RMS paragraphs;
 * xllm-io review of the LinGen paper, section 三 "MA-Branch" item 2, which
 * names the four orders and the flipped sequence). Scan position i maps to the
 * canonical token perm(i), with the loops written outermost first:
 *   order 0 spatial-row major      for t, for h, for w   (canonical order)
 *   order 1 spatial-column major   for t, for w, for h
 *   order 2 temporal-row major     for h, for w, for t
 *   order 3 temporal-column major  for w, for h, for t
 * Order 4 (MATE_ORDER_ZIGZAG) is the zigzag scan that the pages compare RMS
 * against (QbitAI article, section "方法"; xllm-io review, section 三 and
 * Table 2, row "Zigzag"). The pages do not define it; it is the snake path:
 * frame t visits rows h = 0..H-1 on even t and H-1..0 on odd t, and the k-th
 * row of the path (k = t*H + its position in the frame) runs w = 0..W-1 on
 * even k and W-1..0 on odd k, so consecutive tokens are grid neighbours. Every
 * entry point that takes an order accepts it.
 * flip != 0 reverses the sequence: perm'(i) = perm(N-1-i), N = T*H*W.
 *
 * Copies whole token rows of `row_bytes` bytes:
 *   inverse == 0:  dst[b][i]       = src[b][perm(i)]   (canonical -> scan order)
 *   inverse != 0:  dst[b][perm(i)] = src[b][i]         (scan order -> canonical)
 * src and dst are [batch][N][row_bytes] and must not overlap. The copy is
 * bit-exact for any row content. row_bytes may be any positive value; rows
 * whose size and addresses are multiples of 16 bytes take the vector path. */
mate_status mate_rms_reorder(const void *src, void *dst, mate_grid g, int64_t row_bytes, int order,
                             int flip, int inverse, void *stream);

/* ------------------------------------------------------------------------ */
/* Bidirectional Mamba2 (SSD) scan with review tokens                         */
/* ------------------------------------------------------------------------ */
/* For every head h (group g = h / (nheads / ngroups)) and for each direction
 * the recurrence
 *     h_u = exp(dt_u * A_h) h_{u-1} + dt_u x_u B_u^T,   y_u = h_u C_u + D_h x_u,
 * runs from h = 0 over the sequence in RMS order `order` (forward) and over
 * the flipped sequence (backward); y = y_forward + y_backward, written back in
 * canonical order (xllm-io review, section 三 "MA-Branch" item 1: Mamba2 gives
 * the lower-triangular map, the bidirectional form the full one).
 *
 * Review tokens (xllm-io review, section 三 item 3; QbitAI article, review-token
 * paragraph): when pool_t, pool_h, pool_w are not all zero, x, B, C and dt are
 * average-pooled over disjoint pool_t x pool_h x pool_w blocks, the pooled grid
 * is unrolled in the same order and put in front of the forward sequence, and
 * its reversal in front of the flipped sequence. Their outputs are dropped;
 * they only prime the state. The pool extents must divide T, H, W.
 *
 * Layouts: x, y [batch][T][H][W][nheads][headdim]          (dtype)
 *          b, c [batch][T][H][W][ngroups][d_state]          (dtype)
 *          dt   [batch][T][H][W][nheads]   fp32, already positive (post-softplus)
 *          a, d [nheads]                   fp32, a < 0 expected
 * `chunk` is the chunk length of the chunked (SSD) evaluation; it does not
 * change the result beyond rounding. */
typedef struct {
    int32_t nheads, headdim, d_state, ngroups, chunk;
    int32_t pool_t, pool_h, pool_w; /* all 0: no review tokens */
    mate_dtype dtype;               /* of x, b, c, y */
    mate_algo algo;
} mate_ssd_desc;

typedef struct {
    const void *x, *b, *c;
    const float *dt, *a, *d;
    void *y;
} mate_ssd_tensors;

/* Bytes of device workspace mate_bissd_scan needs (0 on invalid arguments). */
size_t mate_bissd_workspace_size(mate_grid g, const mate_ssd_desc *d);

/* Supported: headdim and d_state in 8..128 for the portable kernels (the
 * product headdim*d_state <= 16384), chunk in 1..128; bf16 with headdim 64,
 * d_state 64 or 128 and chunk 64 or 128 also has MFMA kernels. The workspace
 * (device memory, at least mate_bissd_workspace_size bytes, 256-byte aligned)
 * is scratch for the call; its contents on entry do not matter.
 *
 * Input range of the MFMA kernels (MATE_ALGO_AUTO picks them for bf16 with the
 * sizes above). Their intra-chunk products and state updates run on fp16 MFMA:
 * x and B are converted to fp16, and C_t . B_u, the decay-weighted products
 * dt_u C_t . B_u, dt_u x_u and dt_u B_u are held in fp16 (accumulation stays
 * fp32; the states are carried in fp32 and staged as bf16). The result is
 * therefore correct to bf16 accuracy when, for every pair of tokens t, u of
 * one chunk,
 *     |x_u| * max(1, dt_u) < 2^15,   |B_u| * max(1, dt_u) < 2^15 (element-wise),
 *     2 |C_t . B_u| * max(1, dt_u) + 2 |D| < 2^15;
 * larger values overflow to inf, and elements of x and B below 2^-14 in
 * magnitude keep fewer significant bits (fp16 subnormals), which matters only
 * when such elements dominate the output. Outside this range, MATE_ALGO_PORTABLE
 * computes in fp32 throughout and has no such limit beyond fp32's own. */
mate_status mate_bissd_scan(const mate_ssd_tensors *t, mate_grid g, int order, const mate_ssd_desc *d,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Backward of mate_bissd_scan for an upstream gradient dy of its output y (the
 * MA half of training the MATE block; the xllm-io review, section 三, "训练配方",
 * trains LinGen end to end). For each direction, with a_u = exp(dt_u A), the
 * adjoint of the recurrence runs from the end of that direction's sequence to
 * its start, G_u = dy_u C_u^T + a_{u+1} G_{u+1}, and the chain rule through each
 * step gives
 *     dx_u  += dt_u G_u B_u + D dy_u,        dB_u += dt_u G_u^T x_u,
 *     dC_u  += h_u^T dy_u,                   ddt_u += x_u^T G_u B_u + A a_u <h_{u-1}, G_u>,
 *     dA    += dt_u a_u <h_{u-1}, G_u>,      dD   += x_u . dy_u;
 * both directions add into the same gradients, dy is 0 at review positions
 * (their outputs are dropped) and the review tokens' dx, dB and ddt flow back
 * through the average pooling to the tokens of their pool blocks. dB and dC are
 * summed over the heads of each group, dA and dD over the batch.
 * Layouts: x, dy, dx [batch][T][H][W][nheads][headdim]   (desc dtype)
 *          b, c, db, dc [batch][T][H][W][ngroups][d_state] (desc dtype)
 *          dt, ddt [batch][T][H][W][nheads] fp32;  a, d, da, dd [nheads] fp32
 * Every output is written whole; outputs must not overlap the inputs. The
 * evaluation is chunked with chunks of its own (64 tokens, 32 for the widest
 * states), whatever the descriptor's chunk. bf16 tensors with headdim 64 and
 * d_state 64 or 128 run on bf16 MFMA with fp32 accumulation (chunk states
 * stored as bf16 and carried across chunks in fp32; the intra-chunk matrices
 * enter as bf16 pairs); other shapes, and fp32 tensors, compute in fp32.
 * Supported: headdim 16, 32 or 64, d_state a multiple of 8 up to 128, and
 * ceil(R / 16) * batch * nheads < 2^24 for R review tokens
 * (MATE_ERR_UNSUPPORTED otherwise); the descriptor's algo is ignored. The
 * workspace (at least mate_bissd_backward_workspace_size bytes, 256-byte
 * aligned) is scratch for the call: it holds four states per chunk and head
 * (bf16 on the MFMA path, fp32 otherwise). Other errors as mate_bissd_scan. */
typedef struct {
    const void *x, *b, *c;
    const float *dt, *a, *d;
    const void *dy;
    void *dx, *db, *dc;
    float *ddt, *da, *dd;
} mate_ssd_grad_tensors;

size_t mate_bissd_backward_workspace_size(mate_grid g, const mate_ssd_desc *d);
mate_status mate_bissd_backward(const mate_ssd_grad_tensors *t, mate_grid g, int order, const mate_ssd_desc *d,
                                void *workspace, size_t workspace_bytes, void *stream);

/* The same scan for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Instead of a caller-provided workspace it uses a scratch array of
 * MATE_STATIC_SCRATCH_BYTES that the library holds in device memory on every
 * GPU it runs on (from the first call on that GPU until the process ends); the
 * call itself allocates and frees nothing. The caller still passes every input
 * and output. Problems whose workspace (mate_bissd_workspace_size) exceeds the
 * array are rejected with MATE_ERR_WORKSPACE before anything is launched; the
 * array holds the scan of the 8x16x16 (16 heads of 64, d_state 64) and smaller
 * workloads. Every call on one GPU shares that GPU's array and leaves its
 * contents behind (the scan needs none of them on entry): calls that overlap on
 * one GPU (different streams, or threads) race and must be serialised by the
 * caller. Other arguments, results and errors as mate_bissd_scan. */
#define MATE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
mate_status mate_bissd_scan_noalloc(const mate_ssd_tensors *t, mate_grid g, int order, const mate_ssd_desc *d,
                                    void *stream);

/* ------------------------------------------------------------------------ */
/* Bidirectional Mamba (selective scan), the ablation's MA-branch variant     */
/* ------------------------------------------------------------------------ */
/* The ablation of the xllm-io review (Table 2, row "Mamba", and the Mamba2
 * bullet under it) builds the MA branch on Mamba instead of Mamba2. Mamba's
 * selective scan gives every channel c (c < channels) its own d_state states
 * and decay rates. For each direction, over the sequences of mate_bissd_scan
 * (review tokens first, order `order`, reversed for the backward direction),
 * from h = 0:
 *     h_u[c][s] = exp(dt_u[c] * A[c][s]) h_{u-1}[c][s] + dt_u[c] x_u[c] B_u[s]
 *     y_u[c]    = sum_s C_u[s] h_u[c][s] + D[c] x_u[c]
 * and y = y_forward + y_backward at the main tokens, in canonical order.
 * Review tokens average x, B and dt over the pool blocks as in
 * mate_bissd_scan. The tensors are a mate_ssd_tensors with these layouts:
 *   x, y [batch][T][H][W][channels] (dtype)   b, c [batch][T][H][W][d_state] (dtype)
 *   dt [batch][T][H][W][channels] fp32 (> 0)  a [channels][d_state] fp32 (< 0)
 *   d [channels] fp32
 * x, b, c, y 16-byte aligned; dt, a, d 4-byte aligned. */
typedef struct {
    int32_t channels, d_state;
    int32_t pool_t, pool_h, pool_w; /* all 0: no review tokens */
    mate_dtype dtype;
} mate_mamba_desc;

size_t mate_bimamba_workspace_size(mate_grid g, const mate_mamba_desc *d);

/* Supported: d_state 8, 16 or 32, any channel count (MATE_ERR_UNSUPPORTED for
 * another d_state). The workspace (at least mate_bimamba_workspace_size bytes,
 * 256-byte aligned) is scratch for the call. Other errors as mate_bissd_scan. */
mate_status mate_bimamba_scan(const mate_ssd_tensors *t, mate_grid g, int order, const mate_mamba_desc *d,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* TESA: attention inside shifted 3D windows                                  */
/* ------------------------------------------------------------------------ */
/* The grid is cut into windows win_t x win_h x win_w (Tw x Sw x Sw) and every
 * token attends only to the tokens of its own window (xllm-io review, section
 * 三 "TE-Branch"); on shifted layers the partition moves (nav.superapi
 * summary, "TE-branch" bullet: windows shift alternately between layers).
 * Along an axis of extent D with window w and shift s (0 <= s < w) the window
 * id of coordinate c is (c + w - s) div w: the interior windows have size w,
 * the first has size s and the last w - s (when s > 0); nothing wraps around.
 * For every head and window:  O_i = sum_j softmax_j(scale * q_i . k_j) v_j.
 * Layouts: q, k, v, o [batch][T][H][W][nheads][headdim] (dtype). The windows
 * must divide the grid. scale <= 0 selects 1/sqrt(headdim). */
typedef struct {
    int32_t nheads, headdim;
    int32_t win_t, win_h, win_w;
    int32_t shift_t, shift_h, shift_w; /* 0 on unshifted layers */
    float scale;
    mate_dtype dtype;
    mate_algo algo;
} mate_tesa_desc;

typedef struct {
    const void *q, *k, *v;
    void *o;
} mate_tesa_tensors;

/* Supported: headdim 8..128 (multiple of 8) and windows of at most 1024 tokens
 * for the portable kernel; bf16 with headdim 64 or 128 also has MFMA kernels,
 * for windows of at most 4096 tokens and for one unshifted window spanning the
 * whole grid (full attention over all T*H*W tokens, any size). */
mate_status mate_tesa(const mate_tesa_tensors *t, mate_grid g, const mate_tesa_desc *d, void *stream);

/* Backward of mate_tesa for an upstream gradient dout of its output o. Inside
 * each window, with S = scale q k^T, P = softmax of each row of S and o = P v:
 *   dv = P^T dout,  dP = dout v^T,  dS_ij = P_ij (dP_ij - sum_l P_il dP_il),
 *   dq = scale dS k,  dk = scale dS^T q
 * (the chain rule through TESA, the attention half of training the MATE block;
 * the xllm-io review, section 三, "训练配方", trains LinGen end to end). P and
 * sum_l P_il dP_il are recomputed from q, k, v and dout, so the forward's output
 * is not an input. All seven tensors are [batch][T][H][W][nheads][headdim] in
 * the descriptor's dtype, 16-byte aligned; dq, dk, dv are written whole and
 * must not overlap the inputs. */
typedef struct {
    const void *q, *k, *v, *dout;
    void *dq, *dk, *dv;
} mate_tesa_grad_tensors;

/* Bytes of workspace (256-byte aligned device memory, scratch for the call):
 * two floats per token and head. 0 when the descriptor is invalid or not built. */
size_t mate_tesa_backward_workspace_size(mate_grid g, const mate_tesa_desc *d);

/* Supported: bf16, headdim 64 or 128, windows of at most 4096 tokens
 * (MATE_ERR_UNSUPPORTED otherwise). Other errors as mate_tesa. */
mate_status mate_tesa_backward(const mate_tesa_grad_tensors *t, mate_grid g, const mate_tesa_desc *d,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* One MATE core forward                                                     */
/* ------------------------------------------------------------------------ */
/* One layer's token mixing. The MATE block replaces a DiT layer's
 * self-attention with two branches whose outputs it combines: the MA branch
 * (RMS reorder of the layer, review tokens, bidirectional Mamba2) and the TE
 * branch (TESA), with the RMS order and the window shift alternating from
 * layer to layer (QbitAI article on LinGen, section "方法": MATE = MA-branch +
 * TE-branch; xllm-io review, section 三 "MA-Branch" item 2 for the alternating
 * orders and "TE-Branch" for the alternating shift). Here the MA branch is
 * mate_bissd_scan in RMS order `order` and the TE branch mate_tesa with the
 * descriptor's shift, on the same grid. The two branch outputs are returned
 * separately (s->y and a->o): their widths differ, and the pages leave their
 * combination to the layer's projections. Both run on `stream`, one after the
 * other; the result equals the two calls made one after the other. The
 * workspace is mate_forward_workspace_size bytes (the scan's). */
size_t mate_forward_workspace_size(mate_grid g, const mate_ssd_desc *sd, const mate_tesa_desc *td);
mate_status mate_forward(const mate_ssd_tensors *s, const mate_ssd_desc *sd, const mate_tesa_tensors *a,
                         const mate_tesa_desc *td, mate_grid g, int order, void *workspace,
                         size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* One MATE layer                                                            */
/* ------------------------------------------------------------------------ */
/* A whole MATE block in place of a DiT layer's self-attention: the MA and TE
 * branches with their projections, summed (QbitAI article on LinGen, section
 * "方法": MATE, made of the MA and TE branches, replaces self-attention and the
 * rest of the DiT stays as it is; the xllm-io review, section 5.1 and its model
 * table, for the LinGen-4B widths: 2560-wide rows, 20 attention heads, and
 * Table 2 for the two branches' shares of a layer's time). For token rows h:
 *   MA:  x = h Wx, z = h Wz, B = h Wb, C = h Wc, dt = softplus(h Wdt + dt_bias),
 *        y = mate_bissd_scan(x, B, C, dt, A, D) in RMS order `order`,
 *        g = y * silu(z), normalised per group of nheads*headdim/ngroups
 *            channels: g / sqrt(mean(g^2) + eps) * norm_w,
 *   TE:  q = h Wq, k = h Wk, v = h Wv, o = mate_tesa(q, k, v),
 *   out = g Wma_out + o Wte_out.
 * The pages give neither the projections nor the MA branch's per-token steps.
 * They follow the Mamba2 block that the MA branch is built from: dt through a
 * bias and softplus, a gate silu(z), and an RMS norm after the gate before the
 * out-projection. Mamba2's short causal convolution is left out: it mixes
 * neighbouring tokens along the scan, so it is not a per-token step, and the
 * pages say nothing about it.
 * Precision: the GEMMs take bf16 operands with fp32 accumulation (hipBLASLt);
 * x, z, B, C, q, k, v, y, o and g are rounded to bf16 between the steps, dt
 * and the norm's sums stay fp32, out is bf16.
 *
 * Layouts: h, out [batch][T][H][W][d_model] bf16 (16-byte aligned, not
 *          overlapping). Weights are row-major [in][out] bf16:
 *   w_x, w_z [d_model][nheads*headdim]   w_b, w_c [d_model][ngroups*d_state]
 *   w_dt [d_model][nheads]               w_ma_out [nheads*headdim][d_model]
 *   w_q, w_k, w_v [d_model][tesa nheads*headdim]
 *   w_te_out [tesa nheads*headdim][d_model]
 *   dt_bias, a, d [nheads] fp32;  norm_w [nheads*headdim] fp32.
 * sd and td describe the two branches as for mate_bissd_scan and mate_tesa
 * (both dtype bf16; td's shift is the layer's); their tensors live in the
 * workspace. */
typedef struct {
    const void *w_x, *w_z, *w_b, *w_c, *w_dt, *w_ma_out;
    const float *dt_bias, *a, *d, *norm_w;
    const void *w_q, *w_k, *w_v, *w_te_out;
} mate_layer_weights;

typedef struct {
    int32_t d_model; /* width of the rows of h and out, a multiple of 8 */
    float norm_eps;  /* eps of the gated RMS norm, >= 0 */
} mate_layer_desc;

/* Bytes of workspace mate_layer needs: the intermediates of both branches, a
 * copy of w_b, w_c and w_dt side by side (B, C and dt come from one GEMM), the
 * scan's workspace and 64 MiB for the GEMMs (0 on invalid arguments). */
size_t mate_layer_workspace_size(mate_grid g, const mate_layer_desc *ld, const mate_ssd_desc *sd,
                                 const mate_tesa_desc *td);

/* Supported: what mate_bissd_scan and mate_tesa support in bf16, with
 * nheads*headdim/ngroups a multiple of 8 and ngroups <= 64. The first call on
 * a device creates the library's hipBLASLt handle for it, and each new GEMM
 * shape its hipBLASLt descriptors (kept for the process). Errors: as the two
 * calls; MATE_ERR_DEVICE also when hipBLASLt has no algorithm for a shape. */
mate_status mate_layer(const void *h, void *out, const mate_layer_weights *w, const mate_layer_desc *ld,
                       const mate_ssd_desc *sd, const mate_tesa_desc *td, mate_grid g, int order, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                               */
/* ------------------------------------------------------------------------ */
const char *mate_status_string(mate_status s);
const char *mate_last_error(void); /* detail of the last non-OK status on this thread */
int mate_abi_version(void);

/* Per-kernel timing with HIP events, for measuring one kernel of the path
 * inside a running workload.
 * mate_timing_begin(kernel) arms the named kernel: from then on, every launch
 * of it (by any call, any stream) is bracketed by a pair of HIP events
 * recorded on the stream it is launched on. Other kernels are untouched.
 * Names: "rms_reorder", "ssd_pool", "ssd_prep", "ssd_cb", "ssd_states",
 * "ssd_seg_pass", "ssd_out", "tesa", "mamba_scan", "tesa_backward",
 * "ssd_backward" (the whole backward of the scan) (unknown name:
 * MATE_ERR_SHAPE; a timing
 * already armed: MATE_ERR_SHAPE).
 * mate_timing_end waits for the recorded events (a host synchronisation on
 * them), stores the number of timed launches and their summed duration in
 * milliseconds, and disarms. NULL outputs: MATE_ERR_NULL (timing stays armed).
 * Events are created on first use and reused; they stay owned by the library.
 * One timing at a time per process. */
mate_status mate_timing_begin(const char *kernel);
mate_status mate_timing_end(int64_t *launches, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* MATE_H */
