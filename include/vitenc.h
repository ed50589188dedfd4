/*
 * vitenc: the shared pre-LN ViT encoder forward on MI355X (gfx950).
 *
 * The operation is the encoder graph of jepa.cpp "Architecture", section
 * "The shared ViT graph":
 *
 *   tokens = patch_embed(rearranged pixels) [+ pos] [+ cls] [+ modality vec]
 *   per block:  x += ls1 * attn(ln1(x));  x += ls2 * ffn(ln2(x))
 *   out = norm(x)
 *
 * with the hyperparameters and tensor layout of jepa.cpp "GGUF schema (v1)",
 * sections "Encoder (jepa.enc.*)" and "Encoder tensors", the 3-D RoPE and
 * block-causal mask of jepa.cpp "Architecture", sections "3-D RoPE" and
 * "Block-causal attention", and the token order of "GGUF schema (v1)",
 * section "Token order".
 *
 * Conventions for every entry point below:
 *  - Every buffer pointer is DEVICE memory owned by the caller.  The library
 *    never allocates, frees or synchronises device memory; work is enqueued
 *    on the caller's stream (a hipStream_t passed as void*, NULL = the null
 *    stream) and the call returns before it completes.
 *  - Matrices are row-major (PyTorch layout); "[a, b]" means a rows of b
 *    contiguous elements.  Matrices are in the model dtype; norms, biases,
 *    layer scales, position tables and token vectors are always fp32 (the
 *    schema page keeps every add/mul operand f32).
 *  - Failures are refused, never clamped: a refusal returns a non-zero
 *    vitenc_status before any device work is enqueued and sets a
 *    thread-local message readable with vitenc_error_text().
 *  - A model is immutable after creation; concurrent vitenc_encode calls on
 *    one model are allowed when each uses its own workspace and outputs.
 */
#ifndef VITENC_H
#define VITENC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VITENC_ABI_VERSION 5

typedef enum {
    VITENC_OK = 0,
    VITENC_EINVAL = 1,       /* hyperparameter out of range or inconsistent */
    VITENC_ESHAPE = 2,       /* an input shape this model cannot encode */
    VITENC_ENULL = 3,        /* a required pointer is NULL */
    VITENC_EWORKSPACE = 4,   /* workspace smaller than vitenc_workspace_size() */
    VITENC_EDEVICE = 5,      /* the HIP runtime reported an error */
    VITENC_EUNSUPPORTED = 6  /* well-formed but outside what the kernels implement */
} vitenc_status;

enum { VITENC_F32 = 0, VITENC_BF16 = 1, VITENC_F16 = 2 };             /* dtype */
enum { VITENC_POS_NONE = 0, VITENC_POS_TABLE = 1 };                   /* pos_type */
#define VITENC_MAX_HIER 8  /* hierarchical outputs at most */

enum { VITENC_POS_INTERP_NONE = 0, VITENC_POS_INTERP_BICUBIC = 1,
       VITENC_POS_INTERP_TRILINEAR = 2 };                               /* pos_interp */
enum { VITENC_ROPE_NONE = 0, VITENC_ROPE_3D = 1 };                    /* rope */
enum { VITENC_ROPE_TILED = 0, VITENC_ROPE_INTERLEAVED = 1 };          /* rope_layout */
enum { VITENC_ATTN_FULL = 0, VITENC_ATTN_BLOCK_CAUSAL = 1 };          /* attn_mode */
enum { VITENC_WEIGHTS_PLAIN = 0, VITENC_WEIGHTS_MXFP8 = 1 };          /* weight_format */

/* Encoder hyperparameters (jepa.cpp "GGUF schema (v1)", "Encoder (jepa.enc.*)").
 *  embed_dim D, n_layer L, n_head H (head_dim = D / H), ffn_dim F,
 *  patch_size P, tubelet_size t, in_chans C, ln_eps (1e-6 for every family),
 *  rope_theta (10000).
 *  pos_type TABLE: pos_embed has pos_rows rows [CLS?; patches].  With
 *    pos_interp NONE the encoded token count must equal pos_rows.  With
 *    pos_interp BICUBIC or TRILINEAR the table was built for the token grid
 *    pos_grid_t x pos_grid_h x pos_grid_w (pos_rows = prefix + t*h*w) and is
 *    resampled to the input's grid when they differ ("GGUF schema (v1)",
 *    "Encoder tensors": bicubic / trilinear interpolation for other grids):
 *    sample centres aligned, cubic a = -0.75, indices clamped, prefix rows
 *    kept; BICUBIC needs a one-frame table and a one-frame token grid.
 *  rope ROPE_3D: 3-D RoPE on q and k of the patch tokens, d = 2*((hd/3)/2)
 *    rotated dims per axis (t, h, w), rope_layout TILED or INTERLEAVED;
 *    rope_interpolate rescales h and w by (rope_ref_grid - 1)/(grid - 1).
 *  cls_token: a prepended CLS (no pos row unless the table has one, no RoPE).
 *  modality_embed: mod_embed is added to every token.
 *  layer_scale: ls1/ls2 multiply the attention and FFN branches.
 *  attn_mode BLOCK_CAUSAL: key j visible to query i iff frame(i) >= frame(j);
 *    the CLS row sees every key, no patch query sees the CLS key.
 *  dtype: F32 (true fp32 arithmetic throughout), BF16 or F16 (matrices and
 *    activations in that type, fp32 accumulation, fp32 residual stream).
 *  image_patch_embed: the model also has a one-frame tokenizer (V-JEPA 2.1,
 *    "GGUF schema (v1)", enc.patch_embed_img): a one-frame input (T == 1) goes
 *    through it (tubelet 1, token grid 1 x H/P x W/P) and gets the image
 *    modality vector instead of the video one.
 *  n_hier, hier_layers: hierarchical outputs ("GGUF schema (v1)",
 *    jepa.enc.hier_layers / enc.hier_norm.{k}): output k is the residual
 *    stream after block hier_layers[k] through its own norm k; the layer ids
 *    strictly increase within [0, n_layer); at most VITENC_MAX_HIER.
 *  weight_format MXFP8: the four block matrices (qkv, out, up, down) are
 *    stored in 8 bits ("GGUF schema (v1)", "Quantization rules": the
 *    attention and FFN matrices are the quantised ones, everything else keeps
 *    its type): every 32 consecutive weights of a row share a power-of-two
 *    scale and each weight is an E4M3 code; see vitenc_quantize_mxfp8 for
 *    the exact format.  Needs dtype BF16 and embed_dim, ffn_dim multiples of
 *    64; the GEMMs expand the codes to bf16 exactly and run as in BF16. */
typedef struct {
    int32_t embed_dim, n_layer, n_head, ffn_dim;
    int32_t patch_size, tubelet_size, in_chans;
    float ln_eps, rope_theta;
    int32_t pos_type, pos_rows;
    int32_t rope, rope_layout, rope_interpolate, rope_ref_grid;
    int32_t cls_token, modality_embed, layer_scale, attn_mode;
    int32_t dtype;
    int32_t pos_interp, pos_grid_t, pos_grid_h, pos_grid_w;
    int32_t image_patch_embed;
    int32_t n_hier, hier_layers[VITENC_MAX_HIER];
    int32_t weight_format;
} vitenc_hparams;

/* One encoder block ("GGUF schema (v1)", "Encoder tensors", enc.blk.{i}.*).
 * Matrices in the model dtype: qkv_w [3D, D] with rows [q; k; v] and head h
 * at rows [h*hd, (h+1)*hd) of each block; out_w [D, D]; up_w [F, D];
 * down_w [D, F].  fp32 vectors: ln1_w/b, ln2_w/b [D], qkv_b [3D], out_b [D],
 * up_b [F], down_b [D]; ls1/ls2 [D] required iff layer_scale, else ignored.
 * With weight_format MXFP8 the four matrices hold E4M3 codes (one byte per
 * weight, same shapes, 16-byte aligned) and qkv_s, out_s, up_s, down_s their
 * block scales as written by vitenc_quantize_mxfp8; otherwise the *_s
 * pointers are ignored (and the predictor and head never read them). */
typedef struct {
    const float *ln1_w, *ln1_b;
    const void *qkv_w;   const float *qkv_b;
    const void *out_w;   const float *out_b;
    const float *ln2_w, *ln2_b;
    const void *up_w;    const float *up_b;
    const void *down_w;  const float *down_b;
    const float *ls1, *ls2;
    const uint8_t *qkv_s, *out_s, *up_s, *down_s;
} vitenc_block_weights;

/* Encoder weights.  patch_w [D, C*t*P*P] (the strided convolution flattened in
 * C-T-H-W order) in the model dtype; patch_b [D] fp32; pos_embed [pos_rows, D]
 * fp32 iff pos_type TABLE; cls_token [D] fp32 iff cls_token; mod_embed [D]
 * fp32 iff modality_embed; blocks: HOST array of n_layer entries (copied by
 * vitenc_model_create; the device pointers inside are borrowed);
 * norm_w/norm_b [D] fp32 (the final LayerNorm).  With image_patch_embed:
 * patch_img_w [D, C*P*P] (model dtype) and patch_img_b [D], and mod_embed_img
 * [D] iff modality_embed (mod_embed is then the video vector).  hier_norm_w/b
 * [k] [D] fp32 for k < n_hier. */
typedef struct {
    const void *patch_w;  const float *patch_b;
    const float *pos_embed, *cls_token, *mod_embed;
    const vitenc_block_weights *blocks;
    const float *norm_w, *norm_b;
    const void *patch_img_w;  const float *patch_img_b;
    const float *mod_embed_img;
    const float *hier_norm_w[VITENC_MAX_HIER], *hier_norm_b[VITENC_MAX_HIER];
} vitenc_weights;

typedef struct vitenc_model vitenc_model;

/* Validates the hyperparameters and that every required pointer is set, then
 * creates a model that borrows the device weights until vitenc_model_destroy.
 * Refusals: EINVAL (ranges: embed_dim 1..65536, n_layer 1..1024, n_head
 * 1..1024, ffn_dim 1..2^20, patch/tubelet/in_chans 1..1024, ln_eps in [0,1],
 * rope_theta > 0 and finite; embed_dim % n_head; an odd head_dim with RoPE;
 * rope_interpolate without rope_ref_grid; block_causal without RoPE; unknown
 * enum values), ENULL (a required weight), EUNSUPPORTED (head_dim other than
 * 64 or 32 is refused by the attention kernel; embed_dim above 4096). */
vitenc_status vitenc_model_create(const vitenc_hparams *hp, const vitenc_weights *w,
                                  vitenc_model **out);
void vitenc_model_destroy(vitenc_model *m);

/* Bytes of device workspace vitenc_encode needs for a [B, C, T, H, W] input.
 * Refusals: ESHAPE (non-positive sizes, T % tubelet, H % P, W % P, more than
 * 2^22 tokens per item, a pos table whose rows differ from the token count,
 * block_causal with a single-frame grid is accepted). */
vitenc_status vitenc_workspace_size(const vitenc_model *m, int32_t B, int32_t T, int32_t H,
                                    int32_t W, size_t *bytes);

/* Encodes B items.  pixels: fp32 [B, C, T, H, W] (NCTHW, already
 * normalised).  out_tokens: fp32 [B, N, D], N = (CLS ? 1 : 0) + (T/t)(H/P)(W/P),
 * the final-LayerNorm output.  out_pooled: NULL or fp32 [B, D]: the CLS row
 * when the model has a CLS, else the mean of the patch rows.  workspace:
 * ws_bytes >= vitenc_workspace_size() bytes, 256-byte aligned, contents
 * undefined on entry and exit.  Asynchronous on `stream`; errors of the
 * launches themselves are reported as EDEVICE. */
vitenc_status vitenc_encode(const vitenc_model *m, const float *pixels, int32_t B, int32_t T,
                            int32_t H, int32_t W, void *workspace, size_t ws_bytes,
                            float *out_tokens, float *out_pooled, void *stream);

/* ---------------------------------------------------------------------------
 * Masked-latent predictor (SkyVision.cpp README, V-JEPA 2 backend notes,
 * "masked-latent predictor"; hyperparameters and tensors of jepa.cpp "GGUF
 * schema (v1)", section "Predictor (jepa.pred.*)"):
 *
 *   x_ctx = embed(enc_tokens[ctx_ids])                    (enc_dim -> embed_dim)
 *   x_tgt = mask_tokens[mask_index] at every target id
 *   x     = [x_ctx; x_tgt] (+ modality vector) put in increasing token-id order
 *   per block (the encoder's block, full attention, no prefix token, 3-D RoPE
 *   at each token's (t, h, w) on the grid, no interpolation):
 *         x += attn(ln1(x));  x += ffn(ln2(x))
 *   y     = norm(x)
 *   out   = y at the target ids, in the order of tgt_ids, proj_w^T + proj_b
 *   out_ctx = y at the context ids, in the order of ctx_ids, proj_ctx_w^T + proj_ctx_b
 *
 * embed is one linear map (V-JEPA 2; 2.1 after a ViT-B/L encoder) or, with
 * n_hier_in > 1 (V-JEPA 2.1 after a ViT-g/G encoder: pred.embed.0 / .2), the
 * 2-layer MLP embed2(GELU_erf(embed(f))) over the concatenation f of the
 * token's n_hier_in hierarchical encoder features, in level order.  The
 * V-JEPA 2.1 modality vector (pred.mod_embed_img for a one-frame grid,
 * pred.mod_embed_video otherwise) is added to every token, context and mask
 * tokens alike.  proj and proj_context (2.1) map to out_dim, the teacher's
 * width in 2.1 (enc_dim in V-JEPA 2).
 * ------------------------------------------------------------------------- */

/* embed_dim D (1..4096), enc_dim De (1..65536), n_layer, n_head (head_dim
 * D/n_head must be 32 or 64), ffn_dim F, n_mask_tokens (>= 1), ln_eps,
 * rope_theta (> 0), rope_layout TILED or INTERLEAVED, the token grid
 * grid_t x grid_h x grid_w (1..1023 each) on which ids are numbered in the
 * encoder's token order (id = (t*grid_h + h)*grid_w + w), dtype as the encoder.
 * V-JEPA 2.1 options (all 0 = V-JEPA 2): out_dim (0: enc_dim; else 1..65536),
 * n_hier_in (0 or 1: one level; up to VITENC_MAX_HIER), embed_hidden (the
 * embed MLP's hidden width, 1..65536, when n_hier_in > 1), modality_embed and
 * context_proj (0 / 1: the modality vectors / the context projection are
 * present). */
typedef struct {
    int32_t embed_dim, enc_dim, n_layer, n_head, ffn_dim, n_mask_tokens;
    float ln_eps, rope_theta;
    int32_t rope_layout, grid_t, grid_h, grid_w;
    int32_t dtype;
    int32_t out_dim, n_hier_in, embed_hidden, modality_embed, context_proj;
} vitenc_pred_hparams;

/* embed_w [D, De] (with n_hier_in > 1: embed.0 [embed_hidden, n_hier_in*De])
 * and proj_w [out_dim, D] in the model dtype; embed_b [D] (embed_hidden),
 * mask_tokens [n_mask_tokens, D], norm_w/norm_b [D], proj_b [out_dim] fp32;
 * blocks: HOST array of n_layer vitenc_block_weights with the predictor's
 * widths (D, F; layer scales ignored), copied at creation.  V-JEPA 2.1
 * (NULL when the option is off): embed2_w [D, embed_hidden] (model dtype)
 * and embed2_b [D] when n_hier_in > 1; mod_embed_img / mod_embed_video [D]
 * with modality_embed; proj_ctx_w [out_dim, D] (model dtype) and proj_ctx_b
 * [out_dim] with context_proj. */
typedef struct {
    const void *embed_w;  const float *embed_b;
    const float *mask_tokens;
    const vitenc_block_weights *blocks;
    const float *norm_w, *norm_b;
    const void *proj_w;   const float *proj_b;
    const void *embed2_w; const float *embed2_b;
    const float *mod_embed_img, *mod_embed_video;
    const void *proj_ctx_w; const float *proj_ctx_b;
} vitenc_pred_weights;

typedef struct vitenc_predictor vitenc_predictor;

/* Refusals as vitenc_model_create: EINVAL for ranges and enum values, ENULL
 * for a missing weight (an option's tensors included), EUNSUPPORTED for
 * head_dim other than 32 or 64 or embed_dim above 4096. */
vitenc_status vitenc_predictor_create(const vitenc_pred_hparams *hp, const vitenc_pred_weights *w,
                                      vitenc_predictor **out);
void vitenc_predictor_destroy(vitenc_predictor *p);

/* Bytes of device workspace vitenc_predict / vitenc_predict_all need for B
 * items of n_ctx context and n_tgt target ids.  Refusals: ESHAPE (B, n_ctx or
 * n_tgt below 1, n_ctx + n_tgt above the grid's token count). */
vitenc_status vitenc_predict_workspace_size(const vitenc_predictor *p, int32_t B, int32_t n_ctx,
                                            int32_t n_tgt, size_t *bytes);

/* Predicts the teacher features of the target tokens of B items.
 * enc_tokens: fp32 [n_hier_in, B, n_enc, De] (one level: [B, n_enc, De]),
 * the encoder's patch-token features in token order (n_enc must equal
 * grid_t*grid_h*grid_w); ctx_ids int32 [B, n_ctx] and tgt_ids int32
 * [B, n_tgt]: per item, each list strictly increasing, both within
 * [0, n_enc) and disjoint.  The ids are device data and are NOT checked here
 * (the check would need a synchronisation): ids that break the contract give
 * unspecified values in out, but every access stays within the buffers.
 * mask_index: the mask token that fills the targets, in [0, n_mask_tokens).
 * out: fp32 [B, n_tgt, out_dim].  workspace as vitenc_encode's, of
 * vitenc_predict_workspace_size() bytes.  Refusals: those of the workspace
 * size, ENULL, ESHAPE (n_enc), EINVAL (mask_index), EWORKSPACE. */
vitenc_status vitenc_predict(const vitenc_predictor *p, const float *enc_tokens, int32_t B, int32_t n_enc,
                             const int32_t *ctx_ids, int32_t n_ctx, const int32_t *tgt_ids, int32_t n_tgt,
                             int32_t mask_index, void *workspace, size_t ws_bytes, float *out, void *stream);

/* vitenc_predict that also returns the context rows (V-JEPA 2.1 "return all
 * tokens"): out_ctx fp32 [B, n_ctx, out_dim] = the final norm's output at the
 * context ids, in the order of ctx_ids, through proj_context.  out_ctx may be
 * NULL (then this is vitenc_predict); a non-NULL out_ctx on a predictor
 * without context_proj is refused with EINVAL. */
vitenc_status vitenc_predict_all(const vitenc_predictor *p, const float *enc_tokens, int32_t B, int32_t n_enc,
                                 const int32_t *ctx_ids, int32_t n_ctx, const int32_t *tgt_ids, int32_t n_tgt,
                                 int32_t mask_index, void *workspace, size_t ws_bytes, float *out,
                                 float *out_ctx, void *stream);

/* ---------------------------------------------------------------------------
 * Attentive-pool head and classifier (jepa.cpp "GGUF schema (v1)", "Head
 * (jepa.head.*)", kind attentive_pool; SkyVision.cpp README, V-JEPA 2 backend
 * notes, the pooler and classifier heads), on the encoder's output tokens:
 *
 *   x = tokens;  per pooler block (the encoder's block, no RoPE, no mask):
 *         x += attn(ln1(x));  x += ffn(ln2(x))
 *   kv = ln_kv(x);  q = query Wq^T + bq   (the query is not normalised)
 *   a  = per head softmax(q_h k_h^T / sqrt(hd)) v_h, k = kv Wk^T + bk,
 *        v = kv Wv^T + bv, heads concatenated, NO output projection
 *   y  = query + a;  pooled = y + fc2(gelu(fc1(ln2(y))))
 *   logits = pooled cls_w^T + cls_b          (no final norm)
 * ------------------------------------------------------------------------- */

/* embed_dim D (1..4096, a multiple of 4), n_head (D % n_head == 0; with
 * pooler blocks the head width D/n_head must be 32 or 64), ffn_dim F of the
 * blocks and of the head's MLP, n_pool_layers (0..1024), n_classes (0: no
 * classifier), ln_eps, dtype as the encoder. */
typedef struct {
    int32_t embed_dim, n_head, ffn_dim, n_pool_layers, n_classes;
    float ln_eps;
    int32_t dtype;
} vitenc_head_hparams;

/* blocks: HOST array of n_pool_layers vitenc_block_weights (layer scales
 * ignored), copied at creation.  query [D], ln_kv_w/b [D], ln2_w/b [D] fp32,
 * 16-byte aligned; q_w, k_w, v_w [D, D], up_w [F, D], down_w [D, F],
 * cls_w [n_classes, D] in the model dtype; biases fp32 (q_b, k_b, v_b, down_b
 * [D], up_b [F], cls_b [n_classes]).  cls_w / cls_b are required iff
 * n_classes > 0. */
typedef struct {
    const vitenc_block_weights *blocks;
    const float *query;
    const float *ln_kv_w, *ln_kv_b;
    const void *q_w;      const float *q_b;
    const void *k_w;      const float *k_b;
    const void *v_w;      const float *v_b;
    const float *ln2_w, *ln2_b;
    const void *up_w;     const float *up_b;
    const void *down_w;   const float *down_b;
    const void *cls_w;    const float *cls_b;
} vitenc_head_weights;

typedef struct vitenc_head vitenc_head;

/* Refusals: EINVAL (ranges, enum values, a misaligned fp32 vector), ENULL (a
 * missing weight), EUNSUPPORTED (D above 4096 or not a multiple of 4; pooler
 * blocks with a head width other than 32 or 64). */
vitenc_status vitenc_head_create(const vitenc_head_hparams *hp, const vitenc_head_weights *w,
                                 vitenc_head **out);
void vitenc_head_destroy(vitenc_head *h);

/* Bytes of device workspace vitenc_head_forward needs for B items of N
 * tokens.  Refusals: ESHAPE (B or N below 1, N above 2^22, B*N above 2^30). */
vitenc_status vitenc_head_workspace_size(const vitenc_head *h, int32_t B, int32_t N, size_t *bytes);

/* tokens: fp32 [B, N, D], 16-byte aligned (the encoder's out_tokens).
 * pooled: fp32 [B, D], required.  logits: fp32 [B, n_classes] or NULL (no
 * classifier run).  workspace as vitenc_encode's.  Refusals: those of the
 * workspace size, ENULL, EINVAL (misaligned tokens), EWORKSPACE. */
vitenc_status vitenc_head_forward(const vitenc_head *h, const float *tokens, int32_t B, int32_t N,
                                  void *workspace, size_t ws_bytes, float *pooled, float *logits,
                                  void *stream);

/* vitenc_encode that also writes the hierarchical outputs: out_hier NULL
 * or fp32 [n_hier, B, N, D] (output k at offset k*B*N*D). */
vitenc_status vitenc_encode_hier(const vitenc_model *m, const float *pixels, int32_t B, int32_t T,
                                 int32_t H, int32_t W, void *workspace, size_t ws_bytes,
                                 float *out_tokens, float *out_pooled, float *out_hier, void *stream);

/* The 8-bit block weight format of weight_format MXFP8 (the quantised
 * matrices of "GGUF schema (v1)", "Quantization rules", whose q8_0 blocks are
 * 32 consecutive weights of a row sharing one scale).  w: fp32 [rows, cols]
 * (finite values), cols % 64 == 0.  For the block j of row r (weights
 * [32j, 32j+32)) with largest magnitude amax the scale is 2^e, e the smallest
 * integer with amax <= 448 * 2^e, clamped to [-117, 117] (an all-zero block:
 * -117), and each weight becomes the E4M3 code (sign, 4 exponent bits of bias
 * 7, 3 mantissa bits; exponent field 0: subnormals m/8 * 2^-6; largest 448)
 * nearest to w / 2^e, ties to the even mantissa, sign bit = sign of w.  The
 * weight the GEMMs use is code * 2^e, exact in bf16.
 * codes: uint8 [rows, cols]; scales: uint8 [cols/64][rows][2], the byte
 * e + 127 of block j of row r at ((j/2)*rows + r)*2 + j%2 (rows*cols/32
 * bytes).  w and codes 16-byte aligned.  Refusals: ENULL, ESHAPE (sizes),
 * EINVAL (alignment). */
vitenc_status vitenc_quantize_mxfp8(const float *w, int32_t rows, int32_t cols, uint8_t *codes,
                                    uint8_t *scales, void *stream);

/* Thread-local text of the last refusal on this thread ("" if none). */
const char *vitenc_error_text(void);
int32_t vitenc_abi_version(void);

/* ---------------------------------------------------------------------------
 * Step entry points: each runs one step of the encoder graph with the same
 * kernels vitenc_encode uses, on caller buffers.  They exist so that every
 * step can be checked on its own.  dtype is VITENC_F32/BF16/F16 and types
 * every "T" buffer; the layouts named here are those of the encode path.
 * ------------------------------------------------------------------------- */

/* a1-a3 (jepa.cpp "Architecture", "The shared ViT graph": rearrange plus one
 * matmul; "GGUF schema (v1)", "Token order"): pixels fp32 [B,C,T,H,W] ->
 * Z fp32 [B, N, D] = [cls?; patches(pixels) W^T + b] (+ pos) (+ mod).
 * scratch: T, at least B*Np*2*round_up(C*t*P*P, 8) elements (for 16-bit
 * types with C*t*P*P a multiple of 64 each pixel is held as a hi and a lo
 * part, which takes the factor 2).  pos (fp32 [N, D]), cls, mod may be NULL
 * (not applied). */
vitenc_status vitenc_op_embed(int32_t dtype, const float *pixels, int32_t B, int32_t C,
                              int32_t T, int32_t H, int32_t W, int32_t tubelet, int32_t patch,
                              const void *patch_w, const float *patch_b, const float *pos,
                              const float *cls, const float *mod, int32_t D, void *scratch,
                              float *Z, void *stream);

/* a4 LayerNorm ("GGUF schema (v1)", jepa.enc.ln_eps; centred two-pass
 * variance, population, eps inside the root): x fp32 [M, D] -> y [M, D] of
 * type out_dtype (VITENC_F32 for the final norm). */
vitenc_status vitenc_op_layernorm(int32_t out_dtype, const float *x, const float *w,
                                  const float *b, float eps, int32_t M, int32_t D, void *y,
                                  void *stream);

/* a6 tables ("Architecture", "3-D RoPE"; SkyVision.cpp README, V-JEPA 2
 * backend notes): fills rope_table (fp32, vitenc_rope_table_floats(...)
 * floats, device) with the (cos, signed sin) pairs of every position of every
 * axis -- d = 2*((head_dim/3)/2) pairs per position, in the tiled or
 * interleaved frequency order, h and w positions rescaled by
 * (rope_ref_grid - 1)/(g - 1) when rope_interpolate is set -- followed by
 * the packed (t, h, w) grid position of each patch token.  head_dim even;
 * grid axes 1..1023. */
vitenc_status vitenc_op_rope_table(int32_t head_dim, int32_t rope_layout, int32_t rope_interpolate,
                                   int32_t rope_ref_grid, float rope_theta, int32_t gt, int32_t gh,
                                   int32_t gw, float *rope_table, void *stream);

/* a5+a6 fused QKV projection with bias and 3-D RoPE ("Architecture", "3-D
 * RoPE"): Y T [B*N, D] times qkv_w [3D, D]^T + qkv_b, split into heads and
 * written as Q, K: T [B, H, N, hd] (RoPE applied to the patch rows, prefix
 * rows unrotated) and Vt: T [B, H, hd, ldv] (V transposed per head, ldv =
 * round_up(N, 64)).  rope = 0 disables the rotation; grid = (gt, gh, gw) and
 * n_prefix give the token geometry.  rope_table: as filled by
 * vitenc_op_rope_table for this head width and grid (read only; NULL when
 * rope = 0). */
vitenc_status vitenc_op_qkv_rope(int32_t dtype, const void *Y, const void *qkv_w,
                                 const float *qkv_b, int32_t B, int32_t N, int32_t D,
                                 int32_t n_head, int32_t rope, int32_t gt, int32_t gh, int32_t gw,
                                 int32_t n_prefix, const float *rope_table, void *Q, void *K,
                                 void *Vt, void *stream);
int64_t vitenc_rope_table_floats(int32_t head_dim, int32_t gt, int32_t gh, int32_t gw);

/* a7 attention ("Architecture", "Block-causal attention"): per item and head,
 * O = softmax(Q K^T / sqrt(hd) + mask) V with Q, K, Vt in the layouts of
 * vitenc_op_qkv_rope; O: T [B, N, H*hd] (heads concatenated).  attn_mode
 * FULL or BLOCK_CAUSAL with frames of `tokens_per_frame` patch tokens after
 * n_prefix prefix tokens (0 <= n_prefix < N).  scratch: fp32 device memory,
 * 16-byte aligned, of vitenc_attention_scratch_floats() floats for the
 * partial results of rows or query tiles computed split over their keys, NULL
 * when that is 0; contents undefined on entry and exit.  Errors: EINVAL for
 * an unknown dtype or attn_mode or a misaligned scratch, ENULL for a missing
 * pointer (scratch included when it is needed), ESHAPE for inconsistent
 * sizes, EUNSUPPORTED for a head width other than 32 or 64. */
vitenc_status vitenc_op_attention(int32_t dtype, const void *Q, const void *K, const void *Vt,
                                  int32_t B, int32_t N, int32_t n_head, int32_t head_dim,
                                  int32_t attn_mode, int32_t n_prefix,
                                  int32_t tokens_per_frame, float *scratch, void *O, void *stream);

/* Floats of scratch vitenc_op_attention needs for the same arguments: for
 * the prefix rows (split over runs of 256 keys); in fp32, for every row when
 * the query tiles of 128 would make fewer than 16 workgroups (a full-attention
 * call then computes all rows that way); in 16-bit types with the block-causal
 * mask, for the late query tiles computed as two halves of their keys when
 * the grid is small (at most 1024 workgroups).  0 when none applies, -1 for
 * invalid arguments. */
int64_t vitenc_attention_scratch_floats(int32_t dtype, int32_t B, int32_t N, int32_t n_head,
                                        int32_t head_dim, int32_t attn_mode, int32_t n_prefix,
                                        int32_t tokens_per_frame);

/* vitenc_op_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and kernels without the scratch argument.
 * The partial results vitenc_op_attention keeps in the caller's scratch go
 * to a fixed device array of the library instead (the one exception to the
 * rule above that the library holds no device memory), of
 * VITENC_NOALLOC_SCRATCH_FLOATS floats (64 MiB) per device, held until the
 * process ends.  That covers every shape of the five encoder workloads (the
 * largest need is 47 MiB, two 4097-token block-causal clips at 16 heads); a
 * call that needs more (vitenc_attention_scratch_floats of the same
 * arguments above the limit, e.g. prefix rows over millions of keys) is
 * refused with EUNSUPPORTED before any device work.  Every call on one
 * device shares that device's array and each call writes every partial it
 * reads (nothing needs to start at zero), so calls whose executions overlap
 * on one device (different streams or threads) race on it: order them (one
 * stream, or events).  The first call on a device looks the array's address
 * up with that device current.  Other errors as vitenc_op_attention. */
#define VITENC_NOALLOC_SCRATCH_FLOATS (16 << 20)
vitenc_status vitenc_op_attention_noalloc(int32_t dtype, const void *Q, const void *K, const void *Vt,
                                          int32_t B, int32_t N, int32_t n_head, int32_t head_dim,
                                          int32_t attn_mode, int32_t n_prefix,
                                          int32_t tokens_per_frame, void *O, void *stream);

/* a8/a10 projection with bias, layer scale and residual: Z[M, Nout] (fp32)
 * += ls * (A[M, K] W[Nout, K]^T + b); ls may be NULL (= 1). */
vitenc_status vitenc_op_linear_residual(int32_t dtype, const void *A, const void *W,
                                        const float *b, const float *ls, int32_t M,
                                        int32_t Nout, int32_t K, float *Z, void *stream);

/* a9 U[M, Nout] (T) = GELU_erf(A[M, K] W[Nout, K]^T + b). */
vitenc_status vitenc_op_linear_gelu(int32_t dtype, const void *A, const void *W, const float *b,
                                    int32_t M, int32_t Nout, int32_t K, void *U, void *stream);

/* a8-a10 with 8-bit weights: the projections of vitenc_op_linear_residual
 * (epi 0: Z fp32 [M, Nout] += ls * (A W^T + b)) and vitenc_op_linear_gelu
 * (epi 1: U bf16 [M, Nout] = GELU_erf(A W^T + b)) with A bf16 [M, K] and W
 * given as codes [Nout, K] and scales in the format of vitenc_quantize_mxfp8
 * (K % 64 == 0, Nout % 8 == 0, A and codes 16-byte aligned); out is Z or U. */
vitenc_status vitenc_op_linear_mxfp8(int32_t epi, const void *A, const uint8_t *codes,
                                     const uint8_t *scales, const float *b, const float *ls,
                                     int32_t M, int32_t Nout, int32_t K, void *out, void *stream);

/* Position table resampling (the step encode runs for an off-grid input):
 * out [prefix + dt*dh*dw, D] = pos [prefix + st*sh*sw, D] resampled from grid
 * (st, sh, sw) to (dt, dh, dw) with mode VITENC_POS_INTERP_BICUBIC (st = dt =
 * 1) or VITENC_POS_INTERP_TRILINEAR; fp32, prefix rows copied. */
vitenc_status vitenc_op_pos_resample(const float *pos, int32_t prefix, int32_t D, int32_t st, int32_t sh,
                                     int32_t sw, int32_t dt, int32_t dh, int32_t dw, int32_t mode, float *out,
                                     void *stream);

/* a11 pooled feature: pooled[b] = X[b, 0] when cls, else the mean of rows
 * [n_prefix, N) of X[b]; X fp32 [B, N, D]. */
vitenc_status vitenc_op_pool(const float *X, int32_t B, int32_t N, int32_t D, int32_t cls,
                             int32_t n_prefix, float *pooled, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* VITENC_H */
