/*
 * mmdit.h -- C ABI of the packed NR-MMDiT block and rectified-flow library
 * (libmmdit.so, HIP for AMD gfx950 / MI355X).
 *
 * The library computes the forward pass of a dual-stream joint text+image
 * diffusion-transformer block over a native-resolution packed batch, and the
 * rectified-flow wrapper around it: noising and loss for training, CFG
 * combine and Euler update for sampling.
 *
 * Pages cited (by title and section):
 *   [hyper]  hyper.ai summary of arXiv 2607.19064 "Mage-Flow", sections
 *            方法 (method) and 实验 (experiments).
 *   [blog]   Obsidian-blog close reading of "Mage-Flow: An Efficient
 *            Native-Resolution Foundation Model for Image Generation and
 *            Editing", sections 2.2 (mechanism) and 5 (concepts).
 *
 * Conventions for every call:
 *   - Memory.  All tensor arguments are DEVICE pointers owned by the caller;
 *     the library allocates no device memory and keeps no pointer after a
 *     call returns.  Host pointers are marked "host".  Tensors are dense
 *     row-major; pointers must be 16-byte aligned.
 *   - Types.  MMDIT_BF16 tensors are bfloat16, MMDIT_F32 tensors float32.
 *     Accumulation, norm statistics and softmax are always float32.
 *   - Weights are [out, in] row-major (y = x W^T); no biases.
 *   - Streams.  `stream` is a hipStream_t (NULL = default stream).  Calls are
 *     asynchronous on that stream; only mmdit_pack_plan is host-synchronous.
 *     No call synchronises the device unless the environment variable
 *     MMDIT_SYNC=1 is set (then every launch is followed by a stream sync so a
 *     device fault is attributed to its kernel).
 *   - Errors.  Arguments are validated on the host before the first launch.
 *     A failing call returns a negative mmdit_status, launches nothing (or, for
 *     MMDIT_E_HIP, stops at the failing launch) and leaves a message for
 *     mmdit_last_error() in the calling thread.  The library never aborts.
 *   - Determinism.  No call uses floating-point atomics; results are
 *     bitwise reproducible for the same inputs and pack.
 */
#ifndef MMDIT_H_
#define MMDIT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MMDIT_OK = 0,
  MMDIT_E_INVALID = -1,     /* bad argument (null, negative size, inconsistent pack) */
  MMDIT_E_BUDGET = -2,      /* a sample alone exceeds the token budget */
  MMDIT_E_UNSUPPORTED = -3, /* shape outside the supported set (see mmdit_dims) */
  MMDIT_E_WORKSPACE = -4,   /* workspace missing or smaller than required */
  MMDIT_E_HIP = -5          /* a HIP runtime call or kernel launch failed */
} mmdit_status;

typedef enum { MMDIT_F32 = 0, MMDIT_BF16 = 1 } mmdit_dtype;

typedef void* mmdit_stream; /* hipStream_t */

/* Message of the last failing call on this thread ("" if none). */
const char* mmdit_last_error(void);
/* Library version string. */
const char* mmdit_version(void);

/* ------------------------------------------------------------------ pack */

#define MMDIT_MAX_SAMPLES 256

/* One sample in latent-grid units.  frames = 1 for generation; frames = 2 for
 * editing (target grid followed by the clean source grid, [blog] 2.2(2)). */
typedef struct {
  int32_t h, w, frames, txt_len;
} mmdit_sample;

/* A pack ([hyper] 方法: grids flattened to variable-length token sequences and
 * packed under a token budget, text packed by the same principle; [blog]
 * 2.2(2): cumulative offsets, attention confined to each sample, own 2D RoPE
 * per sample, frame axis for editing).
 *
 * Storage is modality-major: image rows of all samples in one buffer, text
 * rows in another.  Sample b owns image rows [cu_img[b], cu_img[b+1]) and text
 * rows [cu_txt[b], cu_txt[b+1]); its joint sequence is [text; target image;
 * source image] of length cu_joint[b+1]-cu_joint[b].  Image row
 * cu_img[b] + k*h*w + r*w + c carries position (k, r, c): k = 0 target,
 * k = 1 source, row-major raster.  Text rows carry position (0, 0, 0).
 *
 * The caller allocates the device arrays (sizes from mmdit_pack_plan) and sets
 * the pointers; mmdit_pack fills them and the host mirror. */
typedef struct {
  int32_t B;          /* samples */
  int32_t max_joint;  /* longest joint sequence */
  int64_t n_img, n_txt, n_tgt;
  /* device arrays (int32) */
  int32_t* cu_txt;   /* [B+1] */
  int32_t* cu_img;   /* [B+1] */
  int32_t* cu_joint; /* [B+1] */
  int32_t* cu_tgt;   /* [B+1] target rows: sample b owns [cu_tgt[b], cu_tgt[b+1]) */
  int32_t* tgt_len;  /* [B]   h*w */
  int32_t* seg_img;  /* [n_img] sample of every image row */
  int32_t* seg_txt;  /* [n_txt] sample of every text row */
  int32_t* pos_img;  /* [n_img*3] (frame, row, col) of every image row */
  int32_t* tgt_row;  /* [n_tgt] image row of every target row */
  /* host mirror, filled by mmdit_pack */
  int32_t h_cu_txt[MMDIT_MAX_SAMPLES + 1];
  int32_t h_cu_img[MMDIT_MAX_SAMPLES + 1];
  int32_t h_cu_tgt[MMDIT_MAX_SAMPLES + 1];
  int32_t h_frames[MMDIT_MAX_SAMPLES];
} mmdit_pack_t;

/* Next-fit plan ([hyper] 方法, fixed token budget).  host only.  Takes samples
 * in input order while the image tokens sum(frames*h*w) stay <= img_budget
 * and, if joint_budget > 0, image + text tokens stay <= joint_budget.  Returns
 * the number taken and the pack totals.  A first sample that alone exceeds a
 * budget gives MMDIT_E_BUDGET (samples are never truncated); n_taken < n
 * means the caller starts the next pack at sample n_taken.  At most
 * MMDIT_MAX_SAMPLES are taken.  Any output pointer may be NULL. */
mmdit_status mmdit_pack_plan(const mmdit_sample* samples /* host [n] */, int32_t n,
                             int64_t img_budget, int64_t joint_budget, int32_t* n_taken,
                             int64_t* n_img, int64_t* n_txt, int32_t* max_joint);

/* Build the pack of samples[0..n): fills the host mirror and the scalar
 * fields of *io, and writes every device array of *io on `stream`.  The
 * caller must have set the device pointers of *io to buffers of the sizes
 * listed above (B = n, totals from mmdit_pack_plan).  n <= MMDIT_MAX_SAMPLES. */
mmdit_status mmdit_pack(const mmdit_sample* samples /* host [n] */, int32_t n, mmdit_pack_t* io,
                        mmdit_stream stream);

/* Gather per-sample tensors into a packed buffer ([hyper] 方法: each
 * sample's latent grid is flattened into a variable-length token sequence
 * and the samples are concatenated into one packed sequence; [blog] 2.2(2):
 * addressed by cumulative offsets).  src[b] (host array of
 * device pointers) is sample b's [rows_b, width] tensor, where rows_b is the
 * sample's image rows (which = 0), text rows (which = 1) or target rows
 * (which = 2); dst is the packed [n_rows, width] buffer.  width % 8 == 0. */
mmdit_status mmdit_pack_gather(const mmdit_pack_t* pack, int32_t which,
                               const void* const* src /* host [B] */, int32_t width,
                               mmdit_dtype dtype, void* dst, mmdit_stream stream);

/* ------------------------------------------------------------ model dims */

/* Supported: head_dim in {64, 128}; hidden = heads*head_dim; hidden, mlp,
 * c_lat, d_txt multiples of 64; t_dim a multiple of 16; eps > 0.
 * rope_dims: widths of the RoPE bands of the (frame, row, col) axes inside
 * each head ([hyper] 方法 and [blog] 2.2(2): 2D RoPE per sample, a frame axis
 * for editing), in that order from dimension 0; each even (0 allowed: that
 * axis is not rotated) and summing to head_dim, else MMDIT_E_UNSUPPORTED.
 * Pair j of a band of width w turns by pos * rope_theta^(-2j/w).  The
 * workloads here use (head_dim/4, 3*head_dim/8, 3*head_dim/8). */
typedef struct {
  int32_t hidden, heads, head_dim, mlp, c_lat, d_txt, t_dim;
  int32_t rope_dims[3];
  float rope_theta, eps;
  mmdit_dtype dtype;
} mmdit_dims;

/* One stream's block weights ([blog] 5 "MMDiT": text and image tokens keep
 * their own projections and norms).  Shapes [out, in]:
 *   w_mod [6H, H]  adaLN (shift1, scale1, gate1, shift2, scale2, gate2)
 *   w_qkv [3H, H]  columns [Q | K | V], each head-contiguous
 *   g_q, g_k [head_dim] float32 QK-RMSNorm gains (always float32)
 *   w_o [H, H], w_up [mlp, H], w_down [H, mlp]                         */
typedef struct {
  const void *w_mod, *w_qkv;
  const float *g_q, *g_k;
  const void *w_o, *w_up, *w_down;
} mmdit_stream_w;
typedef struct {
  mmdit_stream_w img, txt;
} mmdit_block_w;

/* Workspace bytes needed by mmdit_block_fwd, mmdit_final, rf_loss and
 * rf_final_loss for this pack (0 on invalid arguments). */
size_t mmdit_workspace_size(const mmdit_dims* dims, const mmdit_pack_t* pack);

/* Byte offsets of the block's intermediates inside the workspace after
 * mmdit_block_fwd: out[0] mod_img (float32 [B, 6H]), out[1] mod_txt, out[2]
 * h (dtype [n_img + n_txt, H], image rows first; holds the pre-MLP
 * modulated norm after the call), out[3] qkv ([n_img + n_txt, 3H]; q and k
 * after QK-norm and RoPE), out[4] o (attention output [n_img + n_txt, H]),
 * out[5] u (GELU output [n_img + n_txt, mlp]).  Returns 6. */
int32_t mmdit_workspace_layout(const mmdit_dims* dims, const mmdit_pack_t* pack, size_t* out);

/* ----------------------------------------------------- conditioning, embed */

/* Timestep conditioning c [B, H] (dtype) = W_t2 SiLU(W_t1 emb(t)), emb(t) =
 * [cos(1000 t f_k), sin(1000 t f_k)], f_k = 10000^(-k/(t_dim/2)).
 * w_t1 [H, t_dim], w_t2 [H, H]; t [B] float32 device.  ws: at least
 * B*(t_dim + H)*4 bytes.  (The pages name flow matching in t but no embedding;
 * this is the standard sinusoidal MLP.) */
mmdit_status mmdit_cond(const mmdit_dims* dims, const void* w_t1, const void* w_t2, const float* t,
                        int32_t B, void* c, void* ws, size_t ws_bytes, mmdit_stream stream);

/* adaLN vectors mod [B, chunks*H] (float32) = W SiLU(c), W [chunks*H, H]. */
mmdit_status mmdit_modulation(const mmdit_dims* dims, const void* w, int32_t chunks, int32_t B,
                              const void* c, float* mod, mmdit_stream stream);

/* Token embedding ([blog] 2.2(2): the 128-channel latent is flattened into
 * visual tokens and the frozen text encoder supplies the condition tau; the
 * pages give no input projection, so the reading taken is one bias-free
 * linear map per modality into the hidden width):
 * x_img = zt W_in^T (zt [n_img, c_lat], W_in [H, c_lat]) and
 * x_txt = tau W_txt^T (tau [n_txt, d_txt], W_txt [H, d_txt]). */
mmdit_status mmdit_embed(const mmdit_dims* dims, const void* w_in, const void* w_txt,
                         const mmdit_pack_t* pack, const void* zt, const void* tau, void* x_img,
                         void* x_txt, mmdit_stream stream);

/* ------------------------------------------------------------- the block */

/* One dual-stream block ([blog] 5 "MMDiT", 2.2(2), 2.2(3)), updating the
 * residual streams x_img [n_img, H] and x_txt [n_txt, H] in place:
 *   h = rms(x)(1+scale1)+shift1;  q,k,v = h W_qkv^T;
 *   q,k <- RoPE(g * rms(q,k)) per head (image rows at their (f, r, c), text at 0);
 *   o = softmax(q k^T/sqrt(d)) v within each sample's [text; image] tokens;
 *   x += gate1 * (o W_o^T);  x += gate2 * (GELU(rms(x)(1+scale2)+shift2) W_up^T) W_down^T
 * with the adaLN vectors of sample seg[row] from c [B, H].  ws: at least
 * mmdit_workspace_size bytes; its intermediates are described by
 * mmdit_workspace_layout. */
mmdit_status mmdit_block_fwd(const mmdit_dims* dims, const mmdit_block_w* w,
                             const mmdit_pack_t* pack, const void* c, void* x_img, void* x_txt,
                             void* ws, size_t ws_bytes, mmdit_stream stream);

/* The block's adaLN vectors alone ([blog] 5 "MMDiT": the conditioning only
 * enters through them): mod float32 [2][B][6H], mod[0] the image stream's
 * W_mod SiLU(c) and mod[1] the text stream's, one grouped launch.  They depend
 * on c and the weights only, so a caller may compute them on another stream
 * while the embeddings run. */
mmdit_status mmdit_block_modulation(const mmdit_dims* dims, const mmdit_block_w* w, int32_t B,
                                    const void* c, float* mod, mmdit_stream stream);

/* mmdit_block_fwd with the adaLN vectors from mmdit_block_modulation (mod, as
 * above, for the pack's B samples, read only) instead of c; the same launches
 * otherwise, and bit for bit the same result. */
mmdit_status mmdit_block_fwd_mod(const mmdit_dims* dims, const mmdit_block_w* w,
                                 const mmdit_pack_t* pack, const float* mod, void* x_img,
                                 void* x_txt, void* ws, size_t ws_bytes, mmdit_stream stream);

/* ------------------------------------------------------------- training */

/* The block's training forward and its backward.  The pages train the
 * backbone with the flow-matching objective on packed native-resolution
 * samples ([hyper] 方法; [blog] 2.2(2)) and report the whole training step as
 * their systems figure ([blog] 证据二, Table 4); the gradients here are those
 * of the block's own definition (mmdit_block_fwd) by the chain rule. */

/* Bytes of the buffer that mmdit_block_fwd_train fills and mmdit_block_bwd
 * reads for this pack (0 on invalid arguments): per stream the block input,
 * both modulated norms, q/k before and after their norm, v, the attention
 * output and its log-sum-exp, both branch outputs, the residual after the
 * attention branch and the MLP pre-activation, plus the adaLN vectors. */
size_t mmdit_block_saved_size(const mmdit_dims* dims, const mmdit_pack_t* pack);

/* Same result as mmdit_block_fwd (x_img, x_txt updated in place, the same
 * arithmetic), and every intermediate the backward needs is kept in saved
 * (caller-owned, >= mmdit_block_saved_size bytes, 16-byte aligned; read by
 * mmdit_block_bwd of the same pack, weights and c).  ws as for
 * mmdit_block_fwd. */
mmdit_status mmdit_block_fwd_train(const mmdit_dims* dims, const mmdit_block_w* w,
                                   const mmdit_pack_t* pack, const void* c, void* x_img,
                                   void* x_txt, void* saved, size_t saved_bytes, void* ws,
                                   size_t ws_bytes, mmdit_stream stream);

/* Weight gradients of one stream, float32, each the shape of its weight. */
typedef struct {
  float *w_mod, *w_qkv, *g_q, *g_k, *w_o, *w_up, *w_down;
} mmdit_stream_grad;
typedef struct {
  mmdit_stream_grad img, txt;
} mmdit_block_grad;

/* Workspace bytes of mmdit_block_bwd for this pack (0 on invalid arguments). */
size_t mmdit_block_bwd_workspace_size(const mmdit_dims* dims, const mmdit_pack_t* pack);

/* Backward of one block.  In: dx_img [n_img, H], dx_txt [n_txt, H] (dtype)
 * hold dL/dx_out; out: they hold dL/dx_in (in place).  Every gradient in g
 * is overwritten (float32; a stream without rows gets zeros); dc [B, H]
 * float32 is accumulated (+=), as c feeds every block: zero it before the
 * first block.  The two streams' gradients stay separate even when their
 * weights are the same arrays (single-stream blocks: add them).  saved: as
 * filled by mmdit_block_fwd_train; ws >= mmdit_block_bwd_workspace_size.
 * Deterministic: every sum runs in a fixed order (no atomics). */
mmdit_status mmdit_block_bwd(const mmdit_dims* dims, const mmdit_block_w* w,
                             const mmdit_pack_t* pack, const void* c, const void* saved,
                             size_t saved_bytes, void* dx_img, void* dx_txt,
                             const mmdit_block_grad* g, float* dc, void* ws, size_t ws_bytes,
                             mmdit_stream stream);

/* mmdit_block_bwd with the weight gradients (their transposed operands and
 * GEMMs) on a second stream stream_w: each group waits on stream for the
 * kernel that produces its input, and stream waits for all of them before the
 * call's last launch returns, so completion on stream means the whole
 * backward is done, as with mmdit_block_bwd.  The two chains overlap (the
 * transposes are HBM-bound, the input-gradient chain MFMA-bound).  Bit for
 * bit the same results; stream_w NULL or equal to stream is mmdit_block_bwd.
 * Uses a few events per device that the library creates once; one call at a
 * time per device. */
mmdit_status mmdit_block_bwd2(const mmdit_dims* dims, const mmdit_block_w* w,
                              const mmdit_pack_t* pack, const void* c, const void* saved,
                              size_t saved_bytes, void* dx_img, void* dx_txt,
                              const mmdit_block_grad* g, float* dc, void* ws, size_t ws_bytes,
                              mmdit_stream stream, mmdit_stream stream_w);

/* The rest of the training step's backward.  Loss ([hyper] 方法 objective;
 * [blog] 2.2(2), target latent only):  loss = mean_b SSE_b / (tgt_len_b C). */

/* dv [n_tgt, C] (dtype) = dL/dv = 2 (v - (z - eps)) / (B tgt_len_b C) on the
 * target rows; v as rf_loss. */
mmdit_status rf_loss_grad(const mmdit_pack_t* pack, mmdit_dtype dtype, int32_t C, const void* v,
                          const void* z, const void* eps, void* dv, mmdit_stream stream);

/* Workspace bytes of mmdit_final_bwd and mmdit_embed_bwd for this pack. */
size_t mmdit_wrap_bwd_workspace_size(const mmdit_dims* dims, const mmdit_pack_t* pack);

/* Backward of mmdit_final: from dv [n_tgt, C], writes dx_img [n_img, H]
 * (dtype; zero on rows that are not targets), dw_fmod [2H, H] and dw_out
 * [c_lat, H] (float32, overwritten) and adds the conditioning gradient to dc
 * [B, H] (float32).  x_img: the last block's output. */
mmdit_status mmdit_final_bwd(const mmdit_dims* dims, const void* w_fmod, const void* w_out,
                             const mmdit_pack_t* pack, const void* c, const void* x_img,
                             const void* dv, void* dx_img, float* dw_fmod, float* dw_out, float* dc,
                             void* ws, size_t ws_bytes, mmdit_stream stream);

/* Backward of mmdit_embed: dw_in [H, c_lat] = dx_img^T zt and dw_txt
 * [H, d_txt] = dx_txt^T tau (float32, overwritten; zero for a stream without
 * rows).  dx_img, dx_txt: the gradients reaching the first block's input. */
mmdit_status mmdit_embed_bwd(const mmdit_dims* dims, const mmdit_pack_t* pack, const void* zt,
                             const void* tau, const void* dx_img, const void* dx_txt, float* dw_in,
                             float* dw_txt, void* ws, size_t ws_bytes, mmdit_stream stream);

/* Workspace bytes of mmdit_cond_bwd for B samples. */
size_t mmdit_cond_bwd_workspace_size(const mmdit_dims* dims, int32_t B);

/* Backward of mmdit_cond from dc [B, H] (float32, the sum over the final
 * layer and every block): dw_t1 [H, t_dim], dw_t2 [H, H] (float32,
 * overwritten).  t [B] float32 device, as in the forward. */
mmdit_status mmdit_cond_bwd(const mmdit_dims* dims, const void* w_t1, const void* w_t2, const float* t,
                            int32_t B, const float* dc, float* dw_t1, float* dw_t2, void* ws,
                            size_t ws_bytes, mmdit_stream stream);

/* Sub-steps of the block, exposed so every intermediate can be checked. */

/* y = rms(x[row_map[i]]) * (1 + scale[s]) + shift[s], s = seg[row_map[i]]
 * (row_map NULL = identity); shift = mod + shift_off, scale = mod + scale_off,
 * row stride of mod = mod_stride floats.  x [*, H] -> y [n_rows, H]. */
mmdit_status mmdit_rms_modulate(const mmdit_dims* dims, int64_t n_rows, const void* x,
                                const int32_t* row_map, const int32_t* seg, const float* mod,
                                int64_t mod_stride, int64_t shift_off, int64_t scale_off, void* y,
                                mmdit_stream stream);

/* In place on qkv [n_rows, 3H]: q and k of every head become
 * RoPE(g * q / sqrt(mean(q^2) + eps)) ([hyper] 方法 and [blog] 2.2(2) for
 * RoPE and its frame axis).  pos [n_rows*3] (NULL: all positions 0, i.e. text
 * rows, no rotation).  v is left unchanged. */
mmdit_status mmdit_qk_norm_rope(const mmdit_dims* dims, int64_t n_rows, void* qkv,
                                const int32_t* pos, const float* g_q, const float* g_k,
                                mmdit_stream stream);

/* Block-diagonal joint attention ([blog] 2.2(2): attention confined to each
 * sample of the pack; [blog] 5 "MMDiT": joint over text and image).  Reads
 * q, k, v from qkv_txt [n_txt, 3H] and qkv_img [n_img, 3H]; writes
 * o_txt [n_txt, H] and o_img [n_img, H].  The bfloat16 path stages V
 * transposed per head in ws (at least mmdit_attention_workspace_size bytes;
 * the float32 path needs none and ws may be NULL). */
size_t mmdit_attention_workspace_size(const mmdit_dims* dims, const mmdit_pack_t* pack);
mmdit_status mmdit_attention(const mmdit_dims* dims, const mmdit_pack_t* pack,
                             const void* qkv_img, const void* qkv_txt, void* o_img, void* o_txt,
                             void* ws, size_t ws_bytes, mmdit_stream stream);

typedef enum {
  MMDIT_EPI_STORE = 0,        /* Y = A W^T in the model dtype */
  MMDIT_EPI_STORE_F32 = 1,    /* Y = A W^T as float32 */
  MMDIT_EPI_GELU = 2,         /* Y = GELU(A W^T) (exact erf form) */
  MMDIT_EPI_GATED_RES = 3     /* Y += gate[seg[m], :] * (A W^T)   (Y is in/out) */
} mmdit_epilogue;

/* Dense linear Y [M, N] = A [M, K] W^T, W [N, K], float32 accumulation, with
 * the fused epilogue.  For MMDIT_EPI_GATED_RES, gate is float32 with row
 * stride gate_stride (>= N, a multiple of 4, else MMDIT_E_INVALID /
 * MMDIT_E_UNSUPPORTED) and seg [M] int32.  a_silu != 0 applies SiLU to A.
 * K (the row stride of A and W) must stay below 2^22 (the tiles address
 * their operands with 32-bit offsets), else MMDIT_E_UNSUPPORTED. */
mmdit_status mmdit_linear(mmdit_dtype dtype, int64_t M, int32_t N, int32_t K, const void* A,
                          const void* W, void* Y, int32_t epilogue, const float* gate,
                          int64_t gate_stride, const int32_t* seg, int32_t a_silu,
                          mmdit_stream stream);

/* Final layer on target rows ([blog] 2.2(2): the loss is on the target latent
 * only): v [n_tgt, c_lat] = (rms(x)(1+scale)+shift) W_out^T with (shift,
 * scale) = W_fmod SiLU(c), W_fmod [2H, H], W_out [c_lat, H]. */
mmdit_status mmdit_final(const mmdit_dims* dims, const void* w_fmod, const void* w_out,
                         const mmdit_pack_t* pack, const void* c, const void* x_img, void* v,
                         void* ws, size_t ws_bytes, mmdit_stream stream);

/* mmdit_final with its adaLN vectors computed beforehand: modf float32 [B][2H]
 * = mmdit_modulation(w_fmod, chunks 2, c) (shift, then scale), read only.
 * Same workspace and bit for bit the same v. */
mmdit_status mmdit_final_mod(const mmdit_dims* dims, const void* w_out, const mmdit_pack_t* pack,
                             const float* modf, const void* x_img, void* v, void* ws, size_t ws_bytes,
                             mmdit_stream stream);

/* ------------------------------------------------------- rectified flow */

/* Noising z_t = (1 - t_b) z + t_b eps on target rows ([hyper] 方法, the line
 * under the objective; [blog] 2.2(2)); source rows (frame 1) copy z.
 * z, eps, zt [n_img, C] in dtype; t [B] float32. */
mmdit_status rf_make_xt(const mmdit_pack_t* pack, mmdit_dtype dtype, int32_t C, const void* z,
                        const void* eps, const float* t, void* zt, mmdit_stream stream);

/* The embedding with the noising folded into it (the stack-level fusion of
 * [blog] 2.2(3) and [hyper] 方法): x_txt = tau W_txt^T as in mmdit_embed and
 * x_img = z_t W_in^T with z_t the rf_make_xt noising of z, eps (t [B] float32)
 * formed while the GEMM stages its A operand; zt [n_img, C] receives z_t (the
 * embedding backward reads it).  Bit for bit rf_make_xt then mmdit_embed
 * (bfloat16 with C % 64 == 0 and H % 128 == 0 fuse; otherwise the two run in
 * sequence).  NULL pointers -> MMDIT_E_INVALID. */
mmdit_status rf_embed(const mmdit_dims* dims, const void* w_in, const void* w_txt, const mmdit_pack_t* pack,
                      const void* z, const void* eps, const float* t, const void* tau, void* x_img,
                      void* x_txt, void* zt, mmdit_stream stream);

/* The final layer after its modulation and the flow-matching loss in one call
 * ([blog] 2.2(2) and 2.2(3)): v as mmdit_final_mod (modf float32 [B][2H]),
 * then sse and loss as rf_loss, the per-row sums of squared residuals taken
 * inside the final GEMM's split-K reduction (when the product runs split-K;
 * otherwise by the loss's row-sum kernel).  Bit for bit mmdit_final_mod then
 * rf_loss.  ws: mmdit_workspace_size bytes (the final layer's workspace
 * followed by the row sums); too small -> MMDIT_E_WORKSPACE. */
mmdit_status rf_final_loss(const mmdit_dims* dims, const void* w_out, const mmdit_pack_t* pack,
                           const float* modf, const void* x_img, const void* z, const void* eps, void* v,
                           float* sse, float* loss, void* ws, size_t ws_bytes, mmdit_stream stream);

/* Flow-matching loss ([hyper] 方法 objective; [blog] 2.2(2), target latent
 * only): sse[b] = sum over sample b's target rows of (v - (z - eps))^2 and
 * loss[0] = mean_b sse[b] / (tgt_len_b * C), float32.  v [n_tgt, C]; z, eps
 * [n_img, C].  Deterministic fixed-order reduction; ws (16-byte aligned) >=
 * n_tgt*4 + 4 bytes (per-row sums; never empty). */
mmdit_status rf_loss(const mmdit_pack_t* pack, mmdit_dtype dtype, int32_t C, const void* v,
                     const void* z, const void* eps, float* sse, float* loss, void* ws,
                     size_t ws_bytes, mmdit_stream stream);

/* rf_loss for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels, arguments, result bits and
 * errors as rf_loss, with the per-row sums in a scratch array that the
 * library holds in device memory (16 MiB + 16 B per device, until the process
 * ends) instead of ws.  At most 4,194,304 target rows (n_tgt), else
 * MMDIT_E_UNSUPPORTED.  Allocates nothing (no hipMalloc / hipFree).  Every
 * call on one device shares that device's scratch: calls that overlap on one
 * GPU (concurrent streams or threads) race and must be serialised by the
 * caller. */
mmdit_status rf_loss_noalloc(const mmdit_pack_t* pack, mmdit_dtype dtype, int32_t C, const void* v,
                             const void* z, const void* eps, float* sse, float* loss, mmdit_stream stream);

/* Negative-aware flow-matching loss of the post-training stage ([blog]
 * 2.2(4), the Diffusion-NFT objective: a per-sample reward r in [0, 1]
 * weighs the squared error of a positive-policy velocity, 1 - r that of a
 * negative-policy velocity, both against the target velocity):
 *   sse[b] = r[b] ||v_pos - (z - eps)||^2 + (1 - r[b]) ||v_neg - (z - eps)||^2
 * over sample b's target rows, loss[0] = mean_b sse[b] / (tgt_len_b * C).
 * The target velocity is the base objective's z - eps (same straight path);
 * how v_pos and v_neg are formed from the model is the caller's (the pages
 * do not define it).  v_pos, v_neg [n_tgt, C] and z, eps [n_img, C] in dtype;
 * r [B] float32 device.  Same workspace, reduction order and errors as
 * rf_loss; r[b] = 1 for every b gives rf_loss(v_pos) bit for bit. */
mmdit_status rf_nft_loss(const mmdit_pack_t* pack, mmdit_dtype dtype, int32_t C, const void* v_pos,
                         const void* v_neg, const void* z, const void* eps, const float* r, float* sse,
                         float* loss, void* ws, size_t ws_bytes, mmdit_stream stream);

/* Packed-CFG combine + Euler step ([hyper] 实验 and [blog] 2.2(3): cond and
 * uncond in one packed forward; [blog] 5: integrate the velocity ODE from
 * noise to data).  With v [n_tgt, C] from one forward over the pack,
 *   vhat = v_u + g (v_c - v_u)   (uncond_b < 0: vhat = v_c)
 *   z   += (t_cur - t_next) vhat (z float32 [tgt_len[cond_b], C], in place)
 * where v_c, v_u are the target rows of samples cond_b, uncond_b.  If zt_next
 * is not NULL, the updated z is also written (in dtype) into the target rows
 * of samples cond_b and uncond_b of zt_next [n_img, C], ready for the next
 * forward. */
mmdit_status rf_euler_step(const mmdit_pack_t* pack, mmdit_dtype dtype, int32_t C, const void* v,
                           int32_t cond_b, int32_t uncond_b, float guidance, float t_cur,
                           float t_next, float* z, void* zt_next, mmdit_stream stream);

/* Write z (float32 [tgt_len[b0], C]) into the target rows of samples b0 and
 * b1 (b1 < 0: only b0) of zt [n_img, C] in dtype. */
mmdit_status rf_pack_latent(const mmdit_pack_t* pack, mmdit_dtype dtype, int32_t C, const float* z,
                            int32_t b0, int32_t b1, void* zt, mmdit_stream stream);

/* ------------------------------------------------------------- profiling */

/* Kernel timing for benchmarks.  on != 0 clears the record and brackets
 * every subsequent kernel launch of the library with a pair of hipEvents on
 * the launch's stream; on == 0 stops recording.  Not for use while a stream
 * is being captured into a graph; single-threaded use. */
mmdit_status mmdit_timing_enable(int32_t on);

/* Synchronises the device and reports, per kernel name in first-launch
 * order, the summed event-to-event time in ms and the number of launches
 * since timing was enabled.  names receives max_entries rows of 64 chars
 * (NUL-terminated); any output may be NULL.  Returns the number of entries
 * written, or -1 on a HIP error. */
int32_t mmdit_timing_report(int32_t max_entries, char* names, double* total_ms, int64_t* count);

#ifdef __cplusplus
}
#endif
#endif /* MMDIT_H_ */
