/*
 * mf.h -- C ABI of the packed varlen RoPE joint-attention forward (libmf.so).
 *
 * The method: a native-resolution multimodal diffusion transformer packs the
 * text tokens and the flattened image-latent tokens of several samples into
 * one buffer, delimits the samples by cumulative offsets and runs joint
 * self-attention that never crosses samples; rotary position embeddings are
 * per sample (2D, or 3D with a frame axis for editing), and adaptive
 * normalisation, rotary embedding and the gated residual are fused kernels.
 * Sources: picx.dev summary of Mage-Flow, Methodology > Native-Resolution
 * MMDiT (packing under a token budget, per-sample cumulative offsets, packed
 * CFG, frame coordinate of the 3D rotary embedding) and Methodology >
 * Training Infrastructure (fused adaptive normalisation / RoPE / gating);
 * gist.science "Resumo Tecnico: Mage-Flow", Metodologia > 2. NR-MMDiT
 * (variable-length attention kernels with per-sample 2D rotary embeddings)
 * and > 3. Otimizacao de Nivel de Sistema (fused kernels).
 *
 * Conventions for every call below.
 *  - Plain C: no C++ exceptions cross this boundary, no torch or HIP types.
 *    A stream argument is a hipStream_t passed as void* (NULL = the null
 *    stream of the current device).
 *  - Ownership: the caller allocates and frees every buffer, device or host,
 *    including the attention workspace (size from the query call).  The
 *    library allocates no device memory.
 *  - Device calls validate their scalar arguments and pointer alignment on
 *    the host before any HIP call; on failure they return a negative status
 *    and enqueue nothing.  On success the work is enqueued on `stream` and
 *    the call returns without synchronising.  A launch error reported by
 *    the runtime is returned as MF_ERR_HIP.  T == 0 is a successful no-op.
 *  - Contents of device tables (cu_seqlens, pos, mod_row) are the caller's
 *    contract and are not read on the host, except when the environment
 *    variable MF_DEBUG=1 is set: then each device call copies its tables to
 *    the host, checks them (MF_ERR_TABLE) and synchronises after launching.
 *  - bf16 tensors are row-major with the last dimension contiguous; their
 *    pointers must be 16-byte aligned and their row strides multiples of 8
 *    elements.  int32 tables must be 4-byte aligned.
 *  - Calls are re-entrant; concurrent calls on different streams are safe.
 */
#ifndef MF_H
#define MF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mf_status;

enum {
    MF_OK = 0,
    MF_ERR_NULL = -1,        /* a required pointer is NULL                     */
    MF_ERR_SHAPE = -2,       /* sizes, strides or rope dims out of range       */
    MF_ERR_ALIGN = -3,       /* pointer or stride misaligned                   */
    MF_ERR_UNSUPPORTED = -4, /* head dim or configuration not implemented      */
    MF_ERR_WORKSPACE = -5,   /* workspace missing or smaller than the query    */
    MF_ERR_TABLE = -6,       /* table contents invalid (checked on the host)   */
    MF_ERR_HIP = -7          /* the HIP runtime reported an error              */
};

#define MF_ABI_VERSION 2

/* Human-readable name of a status code; static storage, never NULL. */
const char* mf_status_string(mf_status s);

/* MF_ABI_VERSION of the built library. */
int32_t mf_abi_version(void);

/* ------------------------------------------------------------------------
 * Host-side integer pack tables (CPU only; no device needed).
 *
 * One descriptor per packed sample: text_len text tokens followed by
 * n_frames frames of a grid_h x grid_w latent grid (frame 0 is the generation
 * target or the edit source, frame 1 the edit target).  A 1024x1024 image at
 * 16x downsampling is a 64x64 grid.  mod_row_text / mod_row_image select the
 * adaLN table row used by that sample's text / image tokens.
 * Pages: picx.dev summary of Mage-Flow, Methodology > Native-Resolution MMDiT
 * (packing under a token budget, cumulative offsets, frame axis); gist.science
 * "Resumo Tecnico: Mage-Flow", Metodologia > 2. NR-MMDiT (per-sample 2D
 * positions).
 * ---------------------------------------------------------------------- */
typedef struct mf_sample_desc {
    int32_t text_len;
    int32_t n_frames;
    int32_t grid_h;
    int32_t grid_w;
    int32_t mod_row_text;
    int32_t mod_row_image;
} mf_sample_desc;

/* Total packed tokens T = sum_s (text_len + n_frames * grid_h * grid_w).
 * Errors: MF_ERR_NULL (descs NULL with n > 0, or total NULL), MF_ERR_SHAPE
 * (n < 0, a negative field, or T > INT32_MAX). */
mf_status mf_pack_count(const mf_sample_desc* descs, int32_t n, int64_t* total_tokens);

/* Fill caller-allocated host arrays:
 *   cu_seqlens[n+1]: cu[0] = 0, cu[s+1] = cu[s] + L_s (per-sample cumulative
 *                    offsets that delimit the block-diagonal attention);
 *   pos[T][3]      : (frame, row, col) of every token; text tokens (0,0,0);
 *                    image token i of a sample (0-based, after its text) at
 *                    (i / (h*w), (i % (h*w)) / w, i % w);
 *   seq_id[T]      : sample index of every token (may be NULL);
 *   mod_row[T]     : adaLN row of every token (may be NULL).
 * Per-sample positions restart at every sample, as the per-sample 2D/3D
 * rotary embedding requires.  Errors as mf_pack_count, plus MF_ERR_NULL if
 * cu_seqlens is NULL, or pos is NULL while T > 0. */
mf_status mf_pack_tables(const mf_sample_desc* descs, int32_t n, int32_t* cu_seqlens,
                         int32_t* pos, int32_t* seq_id, int32_t* mod_row);

/* ------------------------------------------------------------------------
 * Fused adaLN modulation + multi-axis rotary embedding of q and k.
 * Pages: picx.dev summary, Methodology > Training Infrastructure (adaptive
 * normalisation and RoPE as one fused kernel); gist.science "Resumo Tecnico",
 * Metodologia > 2. NR-MMDiT (per-sample 2D rotary embedding); picx.dev,
 * Methodology > Native-Resolution MMDiT (frame coordinate for editing).
 *
 * For X in {q, k} and every token t (row of C = H*D channels, c = h*D + e):
 *   if shift != NULL:  u = LN(X[t]) * (1 + scale[m(t)]) + shift[m(t)]
 *                      (LayerNorm without affine, population variance, fp32
 *                      statistics, m(t) = mod_row[t]);
 *   else               u = X[t];
 *   then in every head the dims are split in contiguous blocks of rope_f
 *   (frame), rope_r (row) and rope_c (col) dims; pair j of an axis block
 *   (dims o+2j, o+2j+1) is rotated counter-clockwise by
 *   pos[t][axis] * rope_base^(-2j / D_axis).
 * Output is rounded to bf16 (round-to-nearest-even).
 *
 * q_in, k_in, q_out, k_out: bf16 [T][H][D] with token strides ld_in / ld_out
 *   (elements, >= H*D, multiple of 8).  q_out may equal q_in and k_out may
 *   equal k_in (in place); other overlaps are undefined.
 * shift, scale: bf16 [n_rows][H*D], both NULL (RoPE only) or both set;
 *   when set, n_rows >= 1 (>= 0 when T = 0) and n_rows*H*D <= 2^31.
 * mod_row: int32 [T], every entry in [0, n_rows); required when shift/scale
 *   are set, ignored otherwise (n_rows too).  An entry outside [0, n_rows)
 *   reads no table memory: that token is modulated with zero shift and
 *   scale (MF_ERR_TABLE under MF_DEBUG).
 * pos: int32 [T][3] (frame, row, col).
 * rope_f + rope_r + rope_c == D, each a multiple of 8.  D in {64, 128},
 * H*D <= 8192.
 * eps > 0 when modulating.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_UNSUPPORTED,
 * MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
mf_status mf_modulate_rope(void* stream,
                           const void* q_in, const void* k_in, void* q_out, void* k_out,
                           int64_t T, int32_t H, int32_t D, int64_t ld_in, int64_t ld_out,
                           const void* shift, const void* scale, const int32_t* mod_row,
                           int32_t n_rows, const int32_t* pos, int32_t rope_f, int32_t rope_r,
                           int32_t rope_c, float rope_base, float eps);

/* ------------------------------------------------------------------------
 * Block-diagonal (varlen) joint softmax attention forward.
 * Pages: gist.science "Resumo Tecnico", Metodologia > 2. NR-MMDiT
 * (variable-length attention kernels over packed samples); picx.dev summary,
 * Methodology > Native-Resolution MMDiT (joint text + image attention kept
 * inside each sample by the cumulative offsets).
 *
 * For every packed sequence s (tokens cu_seqlens[s] .. cu_seqlens[s+1]-1)
 * and head h, with Q, K, V that sequence's L_s x D slices:
 *   O = softmax(softmax_scale * Q K^T) V, row-wise, no mask inside the
 *   sequence (joint text + image attention) and nothing across sequences;
 *   lse[h][t] = natural-log sum-exp of row t of softmax_scale * Q K^T.
 * bf16 MFMA products with fp32 accumulation; fp32 online softmax; O rounded
 * to bf16.
 *
 * q, k, v: bf16 [T][H][D], token stride ld_qkv (elements, >= H*D,
 *   multiple of 8), so q/k/v may be slices of one fused [T][3][H][D] buffer.
 * o: bf16 [T][H][D], token stride ld_o; must not overlap q, k or v.
 * lse: NULL or fp32 [H][T].
 * cu_seqlens: device int32 [n_seq+1], cu[0] = 0, non-decreasing,
 *   cu[n_seq] = T.  Empty sequences are allowed.
 * max_seqlen: an upper bound of the sequence lengths (0 < max_seqlen <= T
 *   when T > 0); it sizes the work decomposition.  A value below the true
 *   maximum is a contract violation (MF_ERR_TABLE under MF_DEBUG).
 * softmax_scale: > 0, normally 1/sqrt(D).
 * workspace: device memory of at least mf_varlen_attn_workspace_bytes(...)
 *   bytes, 256-byte aligned; it holds the work-tile schedule built on the
 *   device at the start of every call, so concurrent calls need distinct
 *   workspaces.
 * D in {64, 128}.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_UNSUPPORTED,
 * MF_ERR_WORKSPACE, MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
size_t mf_varlen_attn_workspace_bytes(int32_t n_seq, int64_t T, int32_t H, int32_t D);

mf_status mf_varlen_attn_fwd(void* stream,
                             const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens, int32_t n_seq, int32_t max_seqlen,
                             int64_t T, int32_t H, int32_t D, int64_t ld_qkv, int64_t ld_o,
                             float softmax_scale, void* workspace, size_t workspace_bytes);

/* Allocation-free mf_varlen_attn_fwd, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same computation, arguments and errors as
 * mf_varlen_attn_fwd without the workspace: the workspace is an 80 MiB scratch
 * array inside the library, one per GPU, held until the process ends (its
 * device address is looked up once per device, on the first call there; the
 * call allocates nothing).  Every call on a GPU uses that GPU's array, which
 * keeps the last call's contents: calls that overlap on one GPU (several
 * streams or host threads) race, and the caller must serialise them.  A call
 * whose workspace would exceed 80 MiB (mf_varlen_attn_workspace_bytes above
 * 83886080: D = 128 with a persistent grid above 315 workgroups, or more than
 * about 780 000 sequences at D = 128 on 256 CUs) returns MF_ERR_UNSUPPORTED
 * and enqueues nothing. */
mf_status mf_varlen_attn_fwd_noalloc(void* stream,
                                     const void* q, const void* k, const void* v, void* o, float* lse,
                                     const int32_t* cu_seqlens, int32_t n_seq, int32_t max_seqlen,
                                     int64_t T, int32_t H, int32_t D, int64_t ld_qkv, int64_t ld_o,
                                     float softmax_scale);

/* Test hook: the persistent grid of mf_varlen_attn_fwd.
 * g > 0 runs the attention forward on g persistent workgroups instead of one
 * per compute unit, which moves the cut points of its stream-K work split
 * (tests use it to show that results do not depend on them); g = 0 restores
 * the default.  The setting is process-wide and also changes
 * mf_varlen_attn_workspace_bytes, so set it before sizing a workspace and
 * not while attention calls are in flight.
 * Errors: MF_ERR_SHAPE for g < 0 or g > 65536. */
mf_status mf_set_attn_fwd_grid(int32_t g);

/* ------------------------------------------------------------------------
 * Backward of the block-diagonal attention (training).
 *
 * Gradients of O = softmax(softmax_scale * Q K^T) V per packed sequence and
 * head, given dO = dout and the forward's lse:
 *   P = exp(softmax_scale * Q K^T - lse) (row-wise, recomputed),
 *   D_i = sum_e dO[i,e] O[i,e]  (from the bf16 o),
 *   dV = P^T dO,  dS = P * (dO V^T - D),
 *   dQ = softmax_scale * dS K,  dK = softmax_scale * dS^T Q.
 * The pages train this model with the same fused kernels as the forward
 * (picx.dev summary of Mage-Flow, Methodology > Training Infrastructure);
 * these are the chain-rule gradients of the forward above.  bf16 MFMA
 * products with fp32 accumulation; P and dS are rounded to bf16 as MFMA
 * operands; outputs rounded to bf16.  Deterministic (no atomics).
 *
 * q, k, v: the forward's bf16 [T][H][D] inputs, token stride ld_qkv.
 * o, dout: bf16 [T][H][D], token stride ld_o (the forward's output and its
 *   gradient).
 * lse: fp32 [H][T], the forward's natural-log row sums.
 * dq, dk, dv: bf16 [T][H][D], token stride ld_dqkv; fully written (every
 *   row of every head); they must not overlap any input.
 * cu_seqlens, n_seq, max_seqlen, softmax_scale: as for the forward.
 * workspace: device memory of at least mf_varlen_attn_bwd_workspace_bytes
 *   bytes, 256-byte aligned (it holds D and the work-unit tables; concurrent
 *   calls need distinct workspaces).
 * D in {64, 128}; strides multiples of 8 elements.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_UNSUPPORTED,
 * MF_ERR_WORKSPACE, MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
size_t mf_varlen_attn_bwd_workspace_bytes(int32_t n_seq, int64_t T, int32_t H, int32_t D);

mf_status mf_varlen_attn_bwd(void* stream,
                             const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             const int32_t* cu_seqlens, int32_t n_seq, int32_t max_seqlen,
                             int64_t T, int32_t H, int32_t D, int64_t ld_qkv, int64_t ld_o,
                             int64_t ld_dqkv, float softmax_scale, void* workspace,
                             size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * Backward of the fused adaLN modulation + RoPE (training).
 *
 * Gradients of mf_modulate_rope for q and for k, given the gradients
 * dq_out, dk_out of its outputs:
 *   RoPE: each pair's gradient is turned back by -angle (the rotation's
 *   transpose);
 *   modulation (scale != NULL): with xh = (x - mu) / sigma of the input row
 *   (fp32 statistics, population variance) and du the RoPE-back gradient,
 *     gx = du * (1 + scale[m(t)]),
 *     dx = (gx - mean(gx) - xh * mean(gx * xh)) / sigma,
 *     dshift[r] = sum over tokens t with m(t) = r of (du_q[t] + du_k[t]),
 *     dscale[r] = sum of (du_q[t] * xh_q[t] + du_k[t] * xh_k[t])
 *   (the adaLN rows are shared by q and k); without modulation dx = du.
 * Sources as for mf_modulate_rope; the pages train the model with these
 * fused kernels (picx.dev summary, Methodology > Training Infrastructure).
 *
 * q_in, k_in: the forward's bf16 inputs [T][H][D], token stride ld_in.
 * dq_out, dk_out: bf16 [T][H][D], token stride ld_gout.
 * dq_in, dk_in: bf16 [T][H][D] outputs, token stride ld_gin; they may equal
 *   dq_out / dk_out (in place), other overlaps are undefined.
 * scale: bf16 [n_rows][H*D] or NULL (RoPE only; then mod_row, dshift and
 *   dscale are ignored).  shift is not needed.
 * dshift, dscale: fp32 [n_rows][H*D], overwritten.  Each row sum is added in
 *   one fixed order (segments of equal row in runs of tokens, then groups of
 *   them, in token order; no atomics), so the row sums are bitwise
 *   reproducible from call to call; a row no token maps to is zero.
 * mod_row, pos, rope dims, rope_base, eps: as for mf_modulate_rope;
 *   0 <= mod_row[t] < n_rows.
 * workspace: device memory of at least mf_modulate_rope_bwd_workspace_bytes
 *   bytes, 256-byte aligned, when modulating: the per-token statistics and
 *   the partial row sums, room for 2 fp32 values per token and channel (a
 *   run whose adaLN row changes at every token needs one partial per token;
 *   in a pack about one per 128 tokens is written); unused (may be NULL) for
 *   RoPE only.  Concurrent calls need distinct workspaces.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_UNSUPPORTED,
 * MF_ERR_WORKSPACE, MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
size_t mf_modulate_rope_bwd_workspace_bytes(int64_t T, int32_t H, int32_t D);

mf_status mf_modulate_rope_bwd(void* stream,
                               const void* q_in, const void* k_in, int64_t ld_in,
                               const void* dq_out, const void* dk_out, int64_t ld_gout,
                               void* dq_in, void* dk_in, int64_t ld_gin,
                               int64_t T, int32_t H, int32_t D,
                               const void* scale, const int32_t* mod_row, int32_t n_rows,
                               float* dshift, float* dscale, const int32_t* pos,
                               int32_t rope_f, int32_t rope_r, int32_t rope_c,
                               float rope_base, float eps, void* workspace,
                               size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * Backward of the gated residual and its fused next adaLN (training).
 *
 * With y = x + gate[m(t)] * o and z = LN(y) (1 + scale2[m(t)]) + shift2[m(t)]
 * (recomputed in fp32 from the bf16 inputs), given dy and dz:
 *   dyt = dy + (LN backward of dz * (1 + scale2[m(t)])),
 *   dx = dyt, dout = gate[m(t)] * dyt,
 *   dgate[r] = sum over tokens with m(t) = r of dyt * o,
 *   dshift2[r] = sum of dz, dscale2[r] = sum of dz * yh.
 * Without the fused adaLN (scale2, dz, dshift2, dscale2 all NULL) dyt = dy.
 *
 * x, o: the forward's bf16 [T][C] inputs (o = attention output as [T][H*D]).
 * gate, scale2: bf16 [n_rows][C]; mod_row: int32 [T], 0 <= m < n_rows.
 * dy: bf16 [T][C] or NULL (zero); dz: bf16 [T][C] (fused) or NULL.
 * dx, dout: bf16 [T][C] outputs; dx may equal dy; no other overlap.
 * dgate, dshift2, dscale2: fp32 [n_rows][C], overwritten (row sums as
 *   above, each added in one fixed order as for mf_modulate_rope_bwd:
 *   bitwise reproducible).
 * C a multiple of 64 and at most 8192; eps > 0 when fused.
 * workspace: device memory of at least mf_gated_residual_bwd_workspace_bytes
 *   bytes, 256-byte aligned: the per-token statistics and the partial row
 *   sums (room for 3 fp32 values per token and channel, as for
 *   mf_modulate_rope_bwd); concurrent calls need distinct workspaces.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_WORKSPACE,
 * MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
size_t mf_gated_residual_bwd_workspace_bytes(int64_t T, int32_t C);

mf_status mf_gated_residual_bwd(void* stream,
                                const void* x, const void* o, const void* gate,
                                const int32_t* mod_row, int32_t n_rows,
                                const void* dy, const void* scale2, const void* dz,
                                void* dx, void* dout,
                                float* dgate, float* dshift2, float* dscale2,
                                int64_t T, int32_t C, float eps, void* workspace,
                                size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * Gated residual, optionally fused with the next sub-layer's adaLN.
 * Pages: picx.dev summary, Methodology > Training Infrastructure (fused
 * gating / residual chains); gist.science "Resumo Tecnico", Metodologia > 3.
 * Otimizacao de Nivel de Sistema > Kernels Fundidos.
 *
 *   y[t] = x[t] + gate[m(t)] * o[t]                        (fp32, then bf16)
 *   z[t] = LN(y[t]) * (1 + scale2[m(t)]) + shift2[m(t)]    (from fp32 y)
 * x, o, y, z: bf16 [T][C], contiguous rows (o is the attention output viewed
 *   as [T][H*D]).  y may equal x (in place); z must not overlap x, o or y.
 * gate, shift2, scale2: bf16 [n_rows][C], n_rows >= 1 (>= 0 when T = 0),
 *   n_rows*C <= 2^31.
 * mod_row: int32 [T], every entry in [0, n_rows).  An entry outside reads no
 *   table memory: that token takes zero gate, shift2 and scale2
 *   (MF_ERR_TABLE under MF_DEBUG).
 * shift2, scale2 and z are all NULL (no fused adaLN) or all set.
 * C a multiple of 64 and at most 8192; eps > 0 when z is produced.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_TABLE (MF_DEBUG
 * only), MF_ERR_HIP. */
mf_status mf_gated_residual(void* stream,
                            const void* x, const void* o, void* y,
                            const void* gate, const int32_t* mod_row, int32_t n_rows,
                            const void* shift2, const void* scale2, void* z,
                            int64_t T, int32_t C, float eps);

/* ------------------------------------------------------------------------
 * Block projections around the attention (the pages fuse the adaptive
 * normalisation, rotary embedding and gating / residual chains with the
 * operators around them: picx.dev summary of Mage-Flow, Methodology >
 * Training Infrastructure; gist.science "Resumo Tecnico: Mage-Flow",
 * Metodologia > 3. Otimizacao de Nivel de Sistema > Kernels Fundidos; in an
 * NR-MMDiT block, picx.dev Methodology > Native-Resolution MMDiT, those
 * operators are the projections into and out of the joint attention).
 *
 * mf_block_qkv: QKV projection of the adaLN-modulated residual stream with
 * the rotary embedding of q and k:
 *   u[t]   = LN(x[t]) * (1 + scale[m(t)]) + shift[m(t)]   (fp32, then bf16)
 *   qkv[t] = u[t] W_qkv^T   (fp32 accumulation of bf16 products)
 *   q' = RoPE(qkv[t][0:C]), k' = RoPE(qkv[t][C:2C]), v = qkv[t][2C:3C]
 * with RoPE as in mf_modulate_rope (pairs of adjacent dims of each head,
 * axes frame / row / col in contiguous blocks).
 * x: bf16 [T][C] (C = H*D), token stride ld_x >= C, a multiple of 8.
 * w_qkv: bf16 [3C][C] contiguous (output x input, no bias).
 * qkv: bf16 [T][3C] output (q', k', v side by side), token stride
 *   ld_qkv >= 3C, a multiple of 8; must not overlap x or w_qkv.
 * shift, scale: bf16 [n_rows][C], both NULL (no modulation: u = x; mod_row
 *   and n_rows ignored) or both set with mod_row int32 [T] and n_rows as for
 *   mf_modulate_rope (a row outside [0, n_rows) modulates with zeros);
 *   pos: int32 [T][3]; rope dims as for mf_modulate_rope; eps > 0 when
 *   modulating.
 * workspace: device memory of at least mf_block_qkv_workspace_bytes(T, H,
 *   D) bytes, 256-byte aligned: the modulated rows (bf16 [T][C]), then the
 *   rotation table (fp32 [T][D/2][2], cos and sin of every head pair of
 *   every token).  Owned by the caller, used between calls on one stream
 *   only.
 * Limits: D in {64, 128}, C <= 8192, T * ld_x * 2 and 3C * C * 2 below 2^32.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_UNSUPPORTED,
 * MF_ERR_WORKSPACE, MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
size_t mf_block_qkv_workspace_bytes(int64_t T, int32_t H, int32_t D);

mf_status mf_block_qkv(void* stream,
                       const void* x, int64_t ld_x, const void* w_qkv,
                       void* qkv, int64_t ld_qkv,
                       const void* shift, const void* scale, const int32_t* mod_row,
                       int32_t n_rows, const int32_t* pos, int64_t T, int32_t H, int32_t D,
                       int32_t rope_f, int32_t rope_r, int32_t rope_c,
                       float rope_base, float eps, void* workspace, size_t workspace_bytes);

/* mf_block_out: out projection with the gated residual:
 *   y[t] = x[t] + gate[m(t)] * (o[t] W_o^T)        (fp32, then bf16)
 * o: bf16 [T][C] (the attention output viewed as [T][H*D]), token stride
 *   ld_o >= C, a multiple of 8.  w_o: bf16 [C][C] contiguous (output x
 *   input, no bias).  x, y: bf16 [T][C] contiguous; y must not overlap o,
 *   w_o or x.  gate: bf16 [n_rows][C], n_rows >= 1 (>= 0 when T = 0),
 *   n_rows*C <= 2^31;
 *   mod_row: int32 [T], entries in [0, n_rows) (a row outside gates with
 *   zeros, so y = x there; MF_ERR_TABLE under MF_DEBUG).
 * Limits: C a multiple of 64, at most 8192; T * ld_o * 2 below 2^32.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_UNSUPPORTED,
 * MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
mf_status mf_block_out(void* stream,
                       const void* o, int64_t ld_o, const void* w_o,
                       const void* x, const void* gate, const int32_t* mod_row,
                       int32_t n_rows, void* y, int64_t T, int32_t C);

/* ------------------------------------------------------------------------
 * Packed classifier-free guidance + Euler sampler step after the last block.
 *
 * The backbone predicts a velocity for the straight interpolation
 * z_t = (1 - t) z + t eps between data and noise (gist.science "Resumo
 * Tecnico: Mage-Flow", Metodologia; picx.dev summary, Introduction and
 * Theoretical Foundation); the conditional and unconditional branches of
 * classifier-free guidance run packed in one forward (picx.dev, Methodology
 * > Native-Resolution MMDiT), and the Turbo variants sample in 4 steps.
 *
 * Host (no device): prompt p owns the conditional sample cond[p] and the
 * unconditional sample uncond[p] of the pack described by descs (same
 * latent grid h x w, n_frames >= 1).  Its evolving latents are the last
 * frame's h*w tokens (generation: the only frame; editing: the target
 * frame), in raster order.  mf_cfg_pair_count returns N = sum of h*w;
 * mf_cfg_pair_rows fills the caller-allocated host array rows[N][2] with
 * the packed rows (as in mf_pack_tables) of the conditional and the
 * unconditional copy of each such token, prompts in order.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE (bad sample index, cond == uncond,
 * differing grids, no frame, or any mf_pack_count error). */
mf_status mf_cfg_pair_count(const mf_sample_desc* descs, int32_t n, const int32_t* cond,
                            const int32_t* uncond, int32_t n_prompts, int64_t* n_tokens);
mf_status mf_cfg_pair_rows(const mf_sample_desc* descs, int32_t n, const int32_t* cond,
                           const int32_t* uncond, int32_t n_prompts, int32_t* rows);

/* Device: for every evolving token k (rows[k] = (rc, ru), device int32
 * [N][2]) and latent channel c:
 *   g          = v[ru][c] + guidance * (v[rc][c] - v[ru][c])   (fp32)
 *   z_out[k][c] = z[k][c] + (t - t_next) * g                     (fp32)
 *   x_next[rc][c] = x_next[ru][c] = bf16(z_out[k][c])   (when x_next != NULL)
 * i.e. one Euler step from t to t_next along the guided velocity.
 * v: bf16 velocities of the packed batch [T][Cl], token stride ld_v >= Cl.
 * z, z_out: fp32 [N][Cl] contiguous (z_out may equal z).
 * x_next: NULL or bf16 [T][Cl] with token stride ld_x >= Cl (the next
 *   forward's input rows; rows not in the table are left untouched); must
 *   not overlap v.
 * Cl a multiple of 8, at most 4096; strides multiples of 8; guidance, t and
 * t_next finite.  N = 0 is a no-op.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_TABLE (MF_DEBUG
 * only), MF_ERR_HIP. */
mf_status mf_cfg_euler_step(void* stream, const void* v, int64_t ld_v, const int32_t* rows,
                            const float* z, float* z_out, void* x_next, int64_t ld_x,
                            int64_t n_tokens, int32_t Cl, float guidance, float t, float t_next);

/* ------------------------------------------------------------------------
 * Text-encoder variant: the pages fuse the normalisation and rotary
 * embedding chains inside the frozen Qwen3-VL text encoder's blocks as in the
 * backbone (picx.dev summary of Mage-Flow, Methodology > Training
 * Infrastructure; gist.science "Resumo Tecnico: Mage-Flow", Metodologia > 3
 * > Kernels Fundidos); its prompts are packed like the backbone's samples.
 *
 * mf_qk_norm_rope: per-head RMS normalisation + 1D rotary embedding:
 *   q'[t][h] = RoPE_pos[t](q[t][h] / sqrt(mean_e q[t][h][e]^2 + eps) * wq)
 *   k'[t][h] = RoPE_pos[t](k[t][h] / sqrt(mean_e k[t][h][e]^2 + eps) * wk)
 * RoPE turns pair (2j, 2j+1) of every head counter-clockwise by
 * pos[t] * rope_base^(-2j/D); pos[t] is the token's index inside its prompt.
 * q_in / q_out: bf16 [T][Hq][D] (token strides ld_q / ld_qo); k_in / k_out:
 *   bf16 [T][Hkv][D] (ld_k / ld_ko); strides multiples of 8, outputs may
 *   equal inputs.  wq, wk: bf16 [D]; pos: int32 [T] >= 0.
 * D in {64, 128}; Hq * D and Hkv * D at most 8192; rope_base, eps > 0.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_UNSUPPORTED,
 * MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
mf_status mf_qk_norm_rope(void* stream,
                          const void* q_in, int64_t ld_q, const void* k_in, int64_t ld_k,
                          void* q_out, int64_t ld_qo, void* k_out, int64_t ld_ko,
                          const void* wq, const void* wk, const int32_t* pos,
                          int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                          float rope_base, float eps);

/* Host (no device): cumulative offsets cu_seqlens[n+1] and per-token
 * positions pos[T] (index inside its prompt) of n packed prompts of lengths
 * lens[n] (caller-allocated host arrays, T = sum of lens).
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE (n < 0, a negative length, T > INT32_MAX). */
mf_status mf_prompt_tables(const int32_t* lens, int32_t n, int32_t* cu_seqlens, int32_t* pos);

/* mf_varlen_attn_causal_fwd: causal attention inside each packed prompt,
 * query head h reading key/value head h / (Hq / Hkv):
 *   O[i][h] = sum_{j<=i} softmax_j(softmax_scale * q[i][h] . k[j][h']) v[j][h']
 *   lse[h][i] = natural-log sum-exp of the scaled scores (when lse != NULL)
 * with i, j inside one prompt (cu_seqlens as for mf_varlen_attn_fwd).
 * q, o: bf16 [T][Hq][D] (token strides ld_q, ld_o); k, v: bf16
 *   [T][Hkv][D] sharing token stride ld_kv; strides multiples of 8; o must
 *   not overlap q, k or v.  lse: NULL or fp32 [Hq][T].
 * workspace: >= mf_varlen_attn_causal_workspace_bytes(n_seq, T) bytes
 *   (16 * (T / 32 + n_seq + 1): one work descriptor per slab of queries),
 *   16-byte aligned, caller-owned, one call at a time per workspace.
 * Hq a multiple of Hkv; D in {64, 128}; T * ld_q * 2 and T * ld_kv * 2
 * below 2^32.  T = 0 or n_seq = 0 is a no-op.
 * Errors: MF_ERR_NULL, MF_ERR_SHAPE, MF_ERR_ALIGN, MF_ERR_UNSUPPORTED,
 * MF_ERR_WORKSPACE, MF_ERR_TABLE (MF_DEBUG only), MF_ERR_HIP. */
size_t mf_varlen_attn_causal_workspace_bytes(int32_t n_seq, int64_t T);

mf_status mf_varlen_attn_causal_fwd(void* stream,
                                    const void* q, int64_t ld_q, const void* k, const void* v,
                                    int64_t ld_kv, void* o, int64_t ld_o, float* lse,
                                    const int32_t* cu_seqlens, int32_t n_seq, int64_t T,
                                    int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                    void* workspace, size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MF_H */
