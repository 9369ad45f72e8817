/*
 * mhe.h -- C ABI of libmhe, the MI355X (gfx950) prefill of the Qwen3-VL text
 * decoder that the MiniMax H3 text/vision encoder truncates at layer 50.
 *
 * Source of the computation: the vllm-omni page
 * "vllm_omni/diffusion/models/minimax_h3/encoder.py" (MiniMax H3 Qwen3-VL
 * layer-50 text/vision encoder), referred to below as the H3 encoder page,
 * and its rendered API documentation page.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense row-major device buffers. "bf16" means IEEE bfloat16
 *    stored as uint16; the library rounds to nearest-even wherever it
 *    produces bf16. Linear weights follow y = x W^T with W stored [out, in].
 *  - Every tensor starts on a 16-byte boundary (the kernels move 16-byte
 *    vectors; PyTorch allocations are 256-byte aligned). The layer, encode and
 *    fused-attention entry points reject misaligned weights and activations
 *    with MHE_ERR_SHAPE; scales and the device position / mask arrays only
 *    need their element alignment.
 *  - The caller owns every device buffer, the workspace and the stream. The
 *    library allocates and frees nothing; host pointer arrays (layer weight
 *    tables, DeepStack feature tables) are read only during the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls enqueue work and return without synchronising the host; results
 *    are valid once the caller synchronises the stream.
 *  - Return value: MHE_OK (0) or an mhe_status code. All argument checks run
 *    on the host before anything is enqueued, so a failed call has launched
 *    nothing. MHE_ERR_HIP reports a launch error returned by the HIP runtime
 *    (work enqueued earlier in the same call may then have run).
 *    mhe_last_error() returns a message for the calling thread's last failure.
 *  - Entry points keep no state between calls; concurrent calls are safe when
 *    each has its own workspace and output buffers.
 */
#ifndef MHE_H
#define MHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHE_ABI_VERSION 1

typedef enum mhe_status {
  MHE_OK = 0,
  MHE_ERR_NULL = 1,        /* a required pointer is NULL */
  MHE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  MHE_ERR_MISMATCH = 3,    /* token ids and patch grids disagree (mhe_rope_index), or grids and
                              n_patches (vision entry points); the visual-mask popcount is the
                              caller's to check (mhe_count_visual) */
  MHE_ERR_UNSUPPORTED = 4, /* valid but not built for (head_dim, K multiple, group size) */
  MHE_ERR_WORKSPACE = 5,   /* workspace too small or misaligned */
  MHE_ERR_HIP = 6          /* the HIP runtime reported an error */
} mhe_status;

/*
 * Model constants. H3 encoder page: hidden size 5120 and 50 retained layers
 * are module constants; head counts, head_dim, intermediate size, rms eps,
 * rope theta and the multimodal rotary section come from the Qwen3-VL config
 * (MiniMaxH3Qwen3VLTextAttention, MiniMaxH3Qwen3VLTextMLP,
 * MiniMaxH3Qwen3VLTextRotaryEmbedding; section default [24, 20, 20]).
 * Supported: head_dim 64 or 128; n_heads a multiple of n_kv_heads with 1, 2, 4 or 8 query heads per key/value head; hidden, n_heads*head_dim and
 * intermediate multiples of 64; hidden <= 8192; seq <= 131072.
 */
typedef struct mhe_config {
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;
  float rms_eps;
  float rope_theta;
  int32_t mrope_section[3];
} mhe_config;

/*
 * One decoder layer's weights, all bf16 device pointers (H3 encoder page,
 * MiniMaxH3Qwen3VLTextDecoderLayer and its attention/MLP):
 *   ln_in  [hidden]                input_layernorm gain
 *   w_q    [n_heads*head_dim, hidden]   rows 0.. of the fused qkv weight
 *   w_k    [n_kv_heads*head_dim, hidden]
 *   w_v    [n_kv_heads*head_dim, hidden]
 *   q_norm [head_dim], k_norm [head_dim]  per-head RMSNorm gains
 *   w_o    [hidden, n_heads*head_dim]
 *   ln_post[hidden]                post_attention_layernorm gain
 *   w_gate [intermediate, hidden], w_up [intermediate, hidden]
 *                                  the two halves of the fused gate_up weight
 *   w_down [hidden, intermediate]
 */
typedef struct mhe_layer_weights {
  const void* ln_in;
  const void* w_q;
  const void* w_k;
  const void* w_v;
  const void* q_norm;
  const void* k_norm;
  const void* w_o;
  const void* ln_post;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
} mhe_layer_weights;

int32_t mhe_abi_version(void);
const char* mhe_status_string(int32_t status);
/* Message for the calling thread's last failed call ("" if none). */
const char* mhe_last_error(void);

/*
 * Bytes of device workspace that mhe_layer_forward / mhe_encode need for
 * `seq` tokens (256-byte aligned base required). Returns 0 for an invalid
 * config or seq <= 0 (mhe_last_error says why).
 */
size_t mhe_workspace_bytes(const mhe_config* cfg, int32_t seq);

/*
 * One decoder layer in place: hidden [seq, hidden] bf16 is read and
 * overwritten with the layer output. H3 encoder page,
 * MiniMaxH3Qwen3VLTextDecoderLayer.forward: residual + attention(RMSNorm(x)),
 * then residual + MLP(RMSNorm(x)); attention is per-head q/k RMSNorm,
 * multimodal rotary from `positions`, causal GQA attention with scale
 * 1/sqrt(head_dim) and the O projection (MiniMaxH3Qwen3VLTextAttention.forward);
 * the MLP is down(silu(gate(x)) * up(x)) (MiniMaxH3Qwen3VLTextMLP.forward).
 * positions: device int32 [3, seq], rows (T, H, W) (the page's [3, 1, seq]
 * int64 position ids, narrowed). The rotary angles are recomputed per call.
 * Errors: NULL pointers, seq <= 0, unsupported config, workspace too small.
 */
int32_t mhe_layer_forward(const mhe_config* cfg, const mhe_layer_weights* w, void* hidden,
                          const int32_t* positions, int32_t seq, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * DeepStack injection in place (H3 encoder page,
 * MiniMaxH3Qwen3VLTextModel._deepstack_process): for r < n_vis,
 * hidden[t_r, :] += feature[r, :] where t_r is the r-th token (ascending)
 * whose visual_mask byte is non-zero; the sum is rounded to bf16 once.
 * hidden [seq, hidden_dim] bf16, visual_mask device uint8 [seq], feature
 * [n_vis, hidden_dim] bf16. n_vis == 0 is a no-op. If the mask has fewer set
 * bytes than n_vis the extra feature rows are ignored; if it has more, only
 * the first n_vis visual tokens are updated (never out of bounds).
 * workspace: at least seq*4 + 256 bytes.
 */
int32_t mhe_deepstack_inject(void* hidden, int32_t seq, int32_t hidden_dim,
                             const uint8_t* visual_mask, int32_t n_vis, const void* feature,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * mhe_deepstack_inject without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same operation, arguments and errors as
 * mhe_deepstack_inject; the visual index list lives in a fixed scratch array
 * inside the library (512 KiB + 256 bytes per GPU, held until the process
 * ends), so seq is limited to 131072 (larger: MHE_ERR_SHAPE). The call itself
 * allocates nothing; the first call on a device looks up that device's copy
 * of the array. Calls that overlap in time on one GPU (different streams or
 * host threads) share that array and race: serialise them.
 */
int32_t mhe_deepstack_inject_noalloc(void* hidden, int32_t seq, int32_t hidden_dim,
                                     const uint8_t* visual_mask, int32_t n_vis, const void* feature,
                                     void* stream);

/*
 * The whole prefill (H3 encoder page, MiniMaxH3Qwen3VLTextModel.forward):
 * out = hidden state after n_layers decoder layers, unnormalised, bf16
 * [seq, hidden]. inputs_embeds [seq, hidden] bf16 is not written (it is
 * copied to `out`, which is then updated in place). layers: host array of
 * n_layers weight tables. After layer l, for l < min(n_ds, n_layers),
 * DeepStack level l (deepstack[l], device bf16 [n_vis, hidden]) is added to
 * the visual rows as in mhe_deepstack_inject; levels beyond n_layers are
 * unused. visual_mask/deepstack may be NULL only when n_ds == 0 or
 * n_vis == 0. `out` must not overlap inputs_embeds or the workspace.
 */
int32_t mhe_encode(const mhe_config* cfg, const mhe_layer_weights* layers, int32_t n_layers,
                   const void* inputs_embeds, const int32_t* positions,
                   const uint8_t* visual_mask, int32_t n_vis, const void* const* deepstack,
                   int32_t n_ds, int32_t seq, void* out, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Count the non-zero bytes of visual_mask [seq] into *count_host (host
 * int32). Synchronises `stream`. For callers that want the pages' feature /
 * token count check (H3 encoder page, _get_placeholder_mask) before
 * mhe_encode; workspace needs seq*4 + 256 bytes.
 */
int32_t mhe_count_visual(const uint8_t* visual_mask, int32_t seq, int32_t* count_host,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- optional launch timing -------------------------------------------------- */

/* Steps of one decoder layer (plus the DeepStack add), as trace bit positions. */
enum {
  MHE_STEP_INPUT_NORM = 0, /* input RMSNorm */
  MHE_STEP_QKV = 1,        /* q | k | v projections */
  MHE_STEP_QK_ROPE = 2,    /* q/k RMSNorm + rotary + K/V relayout */
  MHE_STEP_ATTENTION = 3,  /* causal GQA attention */
  MHE_STEP_O_PROJ = 4,     /* O projection + residual */
  MHE_STEP_POST_NORM = 5,  /* post-attention RMSNorm */
  MHE_STEP_GATE_UP = 6,    /* gate/up projections + SiLU*mul */
  MHE_STEP_DOWN = 7,       /* down projection + residual */
  MHE_STEP_DEEPSTACK = 8,  /* DeepStack scatter-add */
  MHE_STEP_QUANTIZE = 9,   /* FP8 layers: per-tensor quantisation of a GEMM input */
  MHE_STEP_COUNT = 10
};

/*
 * Process-wide, opt-in launch timing (the one piece of library state). With
 * bit s of `step_mask` set, every later launch of step s made by
 * mhe_layer_forward / mhe_encode is bracketed by a pair of HIP events on the
 * call's stream; mask 0 turns recording off (the default). mhe_trace_read
 * waits for the recorded events of `step`, writes the summed kernel time in
 * milliseconds and the number of launches, and clears that step's record.
 * Calls that overlap on several host threads share one record.
 */
int32_t mhe_trace_enable(uint32_t step_mask);
int32_t mhe_trace_read(int32_t step, double* total_ms, int64_t* launches);

/* ---- single steps of the layer, each one kernel (used for per-step checks) ---- */

/*
 * y[r, :] = gamma * x[r, :] / sqrt(mean(x[r, :]^2) + eps), fp32 reduction,
 * one bf16 rounding (H3 encoder page, MiniMaxH3Qwen3VLRMSNorm). x, y
 * [rows, dim] bf16 (may alias), gamma [dim] bf16. dim % 8 == 0, dim <= 8192.
 */
int32_t mhe_rms_norm(const void* x, const void* gamma, void* y, int32_t rows, int32_t dim,
                     float eps, void* stream);

/*
 * Bytes of fp32 scratch with which mhe_linear / mhe_linear_swiglu can balance
 * their last wave of output tiles (split along k, partials summed in a fixed
 * order). Independent of the shape.
 */
size_t mhe_linear_workspace_bytes(void);

/*
 * c[m, n] = sum_k a[m, k] w[n, k] (+ residual[m, n]) with fp32 accumulation
 * and one bf16 rounding (the F.linear calls of the H3 encoder page; the
 * residual form is the decoder layer's residual add fused into the O and
 * down projections). a [m, k], w [n, k], c and residual [m, n] bf16;
 * residual may be NULL or equal to c (in-place), c must not overlap a or w.
 * k % 64 == 0, n % 32 == 0. workspace (256-byte aligned, may be NULL):
 * scratch for the k-split of the last wave of tiles; with NULL or fewer than
 * mhe_linear_workspace_bytes() bytes fewer (or no) tiles are split. The
 * result does not depend on whether a tile is split beyond fp32 summation
 * order.
 */
int32_t mhe_linear(const void* a, const void* w, void* c, const void* residual, int32_t m,
                   int32_t n, int32_t k, void* workspace, size_t workspace_bytes, void* stream);

/*
 * c[m, j] = silu(sum_k a[m,k] w_gate[j,k]) * sum_k a[m,k] w_up[j,k] in fp32,
 * one bf16 rounding (H3 encoder page, MiniMaxH3Qwen3VLTextMLP.forward up to
 * the down projection). a [m, k], w_gate and w_up [n, k], c [m, n].
 * k % 64 == 0, n % 32 == 0. workspace as for mhe_linear.
 */
int32_t mhe_linear_swiglu(const void* a, const void* w_gate, const void* w_up, void* c,
                          int32_t m, int32_t n, int32_t k, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Per-head q/k RMSNorm and multimodal rotary (H3 encoder page,
 * MiniMaxH3Qwen3VLTextAttention.forward up to SDPA, with
 * MiniMaxH3Qwen3VLTextRotaryEmbedding and _apply_interleaved_mrope).
 * qkv [seq, (n_heads + 2 n_kv_heads) head_dim] bf16 holds q | k | v
 * projections per token; q_norm, k_norm [head_dim] bf16 are the per-head
 * gains; positions device int32 [3, seq]. Outputs, in the layouts the attention step reads:
 *   q_out [seq, n_heads, head_dim]
 *   k_out [n_kv_heads, seq_pad, head_dim]
 *   vt_out[n_kv_heads, head_dim, seq_pad]: V transposed, and within each
 *         aligned group of 16 tokens stored in the order
 *         0 1 2 3 8 9 10 11 4 5 6 7 12 13 14 15
 * with seq_pad = seq rounded up to 128; rows/columns past seq are zero.
 */
int32_t mhe_qk_norm_rope(const mhe_config* cfg, const void* qkv, const void* q_norm,
                         const void* k_norm, const int32_t* positions, int32_t seq, void* q_out,
                         void* k_out, void* vt_out, void* stream);

/*
 * Causal GQA attention (H3 encoder page, MiniMaxH3Qwen3VLTextAttention.forward:
 * query head h uses key/value head h / (n_heads / n_kv_heads), key j visible
 * to query i iff j <= i, scale 1/sqrt(head_dim), softmax in fp32).
 * q, k, vt in the layouts mhe_qk_norm_rope writes; o [seq, n_heads*head_dim]
 * bf16 with column h*head_dim + d.
 */
int32_t mhe_attention(const void* q, const void* k, const void* vt, void* o, int32_t seq,
                      int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, void* stream);

/*
 * The attention step as the decoder layer runs it (H3 encoder page,
 * MiniMaxH3Qwen3VLTextAttention.forward from the q/k/v split to SDPA): the
 * query heads are read raw from the q/k/v projection output and RMS-normalised
 * (gain q_norm) and rotated as they are loaded, i.e. the q half of
 * mhe_qk_norm_rope fused into mhe_attention, with the same arithmetic (fp32,
 * one bf16 rounding of q) and the same outputs up to that rounding.
 * qkv, q_norm, positions as for mhe_qk_norm_rope (only the q columns of qkv
 * are read); k, vt in the layouts mhe_qk_norm_rope writes; o as for
 * mhe_attention. workspace: mhe_qnorm_attention_workspace_bytes(cfg, seq)
 * bytes, 256-byte aligned (the rotary cos/sin of every token and slot).
 * Errors: MHE_ERR_NULL, MHE_ERR_SHAPE (config or seq), MHE_ERR_UNSUPPORTED
 * (head_dim other than 64 / 128, or other than 1, 2, 4, 8 query heads per kv
 * head), MHE_ERR_WORKSPACE; nothing is launched then.
 */
size_t mhe_qnorm_attention_workspace_bytes(const mhe_config* cfg, int32_t seq);
int32_t mhe_qnorm_attention(const mhe_config* cfg, const void* qkv, const void* q_norm,
                            const int32_t* positions, const void* k, const void* vt, void* o,
                            int32_t seq, void* workspace, size_t workspace_bytes, void* stream);

/* ---- FP8 linears (online quantisation) ---------------------------------------
 *
 * H3 encoder page: the encoder accepts an FP8 quantisation config only for a
 * checkpoint that is not FP8-serialised (_validate_encoder_quant_config), so
 * the weights are quantised when loaded and every linear layer, among them
 * the fused qkv and gate_up layers (_is_quantized_linear), runs through the
 * quantised method. The page does not print that method; the one built here
 * is per-tensor E4M3 (OCP "fn": bias 7, no infinities, largest finite 448):
 *   s = max|x| / 448, q = E4M3_rne(clamp(x * (448 / max|x|), -448, 448)),
 *   the factor and the product in fp32; an all-zero tensor gives zero codes
 *   and s = 1;
 *   y = (q_x q_w^T) * s_x * s_w accumulated in fp32, then the layer's
 *   epilogue (residual, SiLU * up) as in the bf16 forms.
 * A fused layer is one tensor with one scale: q | k | v rows stacked, gate
 * rows then up rows. Weights are quantised once (mhe_quantize_fp8), the GEMM
 * inputs on every call, inside the FP8 layer. E4M3 tensors are byte arrays;
 * scales are device floats.
 */

/* Workspace bytes of mhe_quantize_fp8 (partial maxima). */
size_t mhe_quantize_fp8_workspace_bytes(void);

/*
 * Quantise one bf16 tensor, stored as n_parts (1..8) row blocks parts[i]
 * [part_rows[i], cols] (host array of device pointers; a fused weight's
 * pieces), into q [sum part_rows, cols] E4M3 (the blocks stacked in order)
 * with one scale written to scale[0] (device float). cols % 8 == 0.
 * workspace: mhe_quantize_fp8_workspace_bytes() bytes, 256-byte aligned.
 */
int32_t mhe_quantize_fp8(const void* const* parts, const int32_t* part_rows, int32_t n_parts,
                         int32_t cols, void* q, float* scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * c[m, n] = scale_a[0] * scale_w[0] * sum_k a[m, k] w[n, k] (+ residual[m, n]),
 * a [m, k] and w [n, k] E4M3, c and residual bf16 (one rounding); residual
 * may be NULL or equal to c. k % 128 == 0, n % 32 == 0. workspace as for
 * mhe_linear.
 */
int32_t mhe_linear_fp8(const void* a, const float* scale_a, const void* w, const float* scale_w,
                       void* c, const void* residual, int32_t m, int32_t n, int32_t k,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * c[m, j] = silu(g) * u with g = sa sw sum_k a[m,k] w[j,k] and
 * u = sa sw sum_k a[m,k] w[n + j, k] (sa = scale_a[0], sw = scale_w[0]):
 * w_gate_up [2n, k] E4M3 is the fused gate_up weight (gate rows, then up
 * rows). k % 128 == 0, n % 32 == 0. workspace as for mhe_linear.
 */
int32_t mhe_linear_swiglu_fp8(const void* a, const float* scale_a, const void* w_gate_up,
                              const float* scale_w, void* c, int32_t m, int32_t n, int32_t k,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decoder layer's weights for the FP8 layer: norms bf16 as in
 * mhe_layer_weights, the four linears E4M3 with their scales (device float):
 *   w_qkv     [(n_heads + 2 n_kv_heads) head_dim, hidden]  q | k | v rows
 *   w_o       [hidden, n_heads head_dim]
 *   w_gate_up [2 intermediate, hidden]  gate rows, then up rows
 *   w_down    [hidden, intermediate]
 */
typedef struct mhe_layer_weights_fp8 {
  const void* ln_in;
  const void* w_qkv;
  const float* s_qkv;
  const void* q_norm;
  const void* k_norm;
  const void* w_o;
  const float* s_o;
  const void* ln_post;
  const void* w_gate_up;
  const float* s_gate_up;
  const void* w_down;
  const float* s_down;
} mhe_layer_weights_fp8;

/*
 * Workspace bytes of mhe_layer_forward_fp8 / mhe_encode_fp8 (0 for an
 * invalid config or seq). The FP8 forms need hidden, n_heads*head_dim and
 * intermediate to be multiples of 128.
 */
size_t mhe_workspace_bytes_fp8(const mhe_config* cfg, int32_t seq);

/*
 * mhe_layer_forward / mhe_encode with the four linears of every layer in FP8:
 * before each GEMM its bf16 input (the normed hidden state, the attention
 * output, the SiLU*up product) is quantised with its own per-tensor scale,
 * taken over all seq rows. Everything else, arguments and errors as in the
 * bf16 forms.
 */
int32_t mhe_layer_forward_fp8(const mhe_config* cfg, const mhe_layer_weights_fp8* w, void* hidden,
                              const int32_t* positions, int32_t seq, void* workspace,
                              size_t workspace_bytes, void* stream);
int32_t mhe_encode_fp8(const mhe_config* cfg, const mhe_layer_weights_fp8* layers, int32_t n_layers,
                       const void* inputs_embeds, const int32_t* positions,
                       const uint8_t* visual_mask, int32_t n_vis, const void* const* deepstack,
                       int32_t n_ds, int32_t seq, void* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---- token-level front end (from token ids to mhe_encode's inputs) ---------- */

/*
 * Multimodal rotary position ids from token ids (H3 encoder page,
 * _get_rope_index with _get_vision_position_ids, and the token types that
 * _encode assigns). HOST function: every pointer is host memory, nothing is
 * enqueued and no GPU is needed.
 *   ids [seq] int32. A token equal to image_token_id is an image placeholder,
 *   equal to video_token_id a video placeholder, anything else text.
 *   image_grid_thw [n_images, 3], video_grid_thw [n_videos, 3]: int32 (t, h, w)
 *   patch grids as the vision tower reports them; spatial_merge is its merge
 *   size (2 for Qwen3-VL). A video of t frames counts as t one-frame grids.
 * The tokens are cut into runs of one type. A text run of n tokens takes
 * positions cur .. cur+n-1 on all three axes and advances cur by n; a visual
 * run takes the next grid of its type and must hold its t * (h/m) * (w/m)
 * tokens; its token at frame f, row r, column c gets (cur+f, cur+r, cur+c) and
 * cur advances by max(h, w)/m.
 * Outputs: positions [3, seq] int32 (rows T, H, W), the layout mhe_encode
 * takes; optional (may be NULL) image_mask, video_mask, visual_mask [seq]
 * uint8 (1 on image / video / either placeholder tokens) and *delta = max
 * position + 1 - seq (the page's rope delta).
 * Errors: NULL ids/positions or grid arrays, seq out of range, equal token
 * ids, a non-positive grid or h, w not multiples of spatial_merge
 * (MHE_ERR_SHAPE); a visual run with no grid left or of another length than
 * its grid (MHE_ERR_MISMATCH; the page's processor brackets every image and
 * video frame with text). Grids left over are ignored, as on the page. On
 * error the outputs are partly written.
 */
int32_t mhe_rope_index(const int32_t* ids, int32_t seq, int32_t image_token_id,
                       int32_t video_token_id, const int32_t* image_grid_thw, int32_t n_images,
                       const int32_t* video_grid_thw, int32_t n_videos, int32_t spatial_merge,
                       int32_t* positions, uint8_t* image_mask, uint8_t* video_mask,
                       uint8_t* visual_mask, int32_t* delta);

/*
 * Token embedding gather (H3 encoder page, _encode: text_model.embed_tokens;
 * the vocab-parallel embedding of the same page for a table shard):
 * out[s, :] = table[ids[s] - row_begin, :] when row_begin <= ids[s] <
 * row_begin + rows, else a zero row, which is also added to *n_outside
 * (device int32, may be NULL; the caller zeroes it). ids device int32 [seq],
 * table device bf16 [rows, hidden_dim], out [seq, hidden_dim] bf16.
 * hidden_dim % 8 == 0.
 */
int32_t mhe_embed_tokens(const int32_t* ids, int32_t seq, const void* table, int32_t row_begin,
                         int32_t rows, int32_t hidden_dim, void* out, int32_t* n_outside,
                         void* stream);

/*
 * Visual placeholder scatter in place (H3 encoder page, _encode:
 * inputs_embeds.masked_scatter(mask, embeds)): for r < n, hidden[t_r, :] =
 * feature[r, :] where t_r is the r-th token (ascending) whose mask byte is
 * set. Same shapes, bounds behaviour and workspace (seq*4 + 256 bytes) as
 * mhe_deepstack_inject; the page's count check is mhe_count_visual.
 */
int32_t mhe_scatter_visual(void* hidden, int32_t seq, int32_t hidden_dim, const uint8_t* mask,
                           int32_t n, const void* feature, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Workspace bytes of mhe_join_visual for `seq` tokens (0 if seq is out of range). */
size_t mhe_join_visual_workspace_bytes(int32_t seq);

/*
 * One DeepStack level for a prompt with both images and videos (H3 encoder
 * page, _aggregate_deepstack): joint[r, :] is the feature row of the r-th
 * visual token (ascending over tokens set in image_mask or video_mask):
 * image_feature[i] if it is the i-th image token, else video_feature[v] if it
 * is the v-th video token. image_mask, video_mask device uint8 [seq]
 * (disjoint); image_feature [n_image, hidden_dim], video_feature [n_video,
 * hidden_dim], joint [n_image + n_video, hidden_dim], bf16. Rows with no
 * matching feature (masks with fewer set bytes than n_image / n_video) are
 * zero, as in the page's zero-initialised joint array. Pass joint with
 * visual_mask = image_mask | video_mask (mhe_rope_index writes it) to
 * mhe_encode.
 */
int32_t mhe_join_visual(const uint8_t* image_mask, const uint8_t* video_mask, int32_t seq,
                        int32_t hidden_dim, const void* image_feature, int32_t n_image,
                        const void* video_feature, int32_t n_video, void* joint, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---- Qwen3-VL vision tower (produces the visual rows and DeepStack levels) -- */

/*
 * Vision tower sizes (H3 encoder page, MiniMaxH3Qwen3VLVisionModel; the values
 * come from the checkpoint's vision config, which the page does not print).
 * Qwen3-VL: hidden 1152, 16 heads (head_dim 72), MLP width 4304 stored padded
 * with zero rows / columns to a multiple of 64 (4352: a zero fc1 row with a
 * zero bias gives gelu(0) = 0, which a zero fc2 column ignores), depth 27,
 * patch_dim = in_channels 3 * temporal patch 2 * 16 * 16 = 1536, spatial
 * merge 2, out_hidden 5120 (the text hidden size), pos_side 48 (2304 learned
 * position embeddings), DeepStack after blocks 8, 16 and 24.
 * Supported: hidden, intermediate and merge^2 * hidden multiples of 64;
 * out_hidden a multiple of 32; head_dim = hidden / n_heads a multiple of 4
 * and <= 128; patch_dim a multiple of 64; merge^2 * hidden <= 8192;
 * n_deepstack <= 8.
 */
typedef struct mhe_vision_config {
  int32_t hidden;
  int32_t n_heads;
  int32_t intermediate;
  int32_t depth;
  int32_t patch_dim;
  int32_t merge;
  int32_t out_hidden;
  int32_t pos_side;
  int32_t n_deepstack;
  int32_t deepstack_index[8];
} mhe_vision_config;

/* One vision block (MiniMaxH3Qwen3VLVisionBlock), bf16 device pointers:
 * norm1/norm2 LayerNorm weight and bias [hidden]; qkv_w [3 hidden, hidden],
 * qkv_b [3 hidden] (q | k | v, head-major inside each); proj_w [hidden, hidden],
 * proj_b; fc1_w [intermediate, hidden], fc1_b; fc2_w [hidden, intermediate], fc2_b. */
typedef struct mhe_vision_block_weights {
  const void *norm1_w, *norm1_b, *qkv_w, *qkv_b, *proj_w, *proj_b;
  const void *norm2_w, *norm2_b, *fc1_w, *fc1_b, *fc2_w, *fc2_b;
} mhe_vision_block_weights;

/* A patch merger (MiniMaxH3Qwen3VLVisionPatchMerger): norm over hidden (main
 * merger) or over merge^2 * hidden (DeepStack mergers); fc1 [M, M] with
 * M = merge^2 * hidden; fc2 [out_hidden, M]; biases likewise. */
typedef struct mhe_vision_merger_weights {
  const void *norm_w, *norm_b, *fc1_w, *fc1_b, *fc2_w, *fc2_b;
} mhe_vision_merger_weights;

/* patch_w [hidden, patch_dim]: the Conv3d kernel [hidden, C, T, P, P]
 * flattened; patch_b [hidden]; pos_table [pos_side^2, hidden]; blocks: host
 * array [depth]; deepstack: host array [n_deepstack]. */
typedef struct mhe_vision_weights {
  const void* patch_w;
  const void* patch_b;
  const void* pos_table;
  const mhe_vision_block_weights* blocks;
  mhe_vision_merger_weights merger;
  const mhe_vision_merger_weights* deepstack;
} mhe_vision_weights;

/* Workspace bytes of the vision entry points for n_patches patches (0 on a
 * bad config or size). */
size_t mhe_vision_workspace_bytes(const mhe_vision_config* cfg, int32_t n_patches);

/*
 * The whole tower (H3 encoder page, MiniMaxH3Qwen3VLVisionModel.forward):
 * pixels [n_patches, patch_dim] bf16 (the processor's flattened patches, in
 * its order: images in turn, frames, then merge x merge blocks), grid_thw
 * HOST int32 [n_grids, 3] (t, h, w in patches; h, w multiples of merge;
 * n_grids <= 64), n_patches = sum t*h*w. Writes merged [n_patches / merge^2,
 * out_hidden] (the image / video embeddings mhe_scatter_visual places) and,
 * for each DeepStack level l, deepstack[l] (host array of device pointers)
 * [n_patches / merge^2, out_hidden]. Each kernel accumulates in fp32 and
 * rounds its output to bf16 once.
 */
int32_t mhe_vision_forward(const mhe_vision_config* cfg, const mhe_vision_weights* w,
                           const void* pixels, const int32_t* grid_thw, int32_t n_grids,
                           void* merged, void* const* deepstack, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Steps of the tower, for per-step checks. hidden [n_patches, hidden] bf16.
 * mhe_vision_embed: hidden = patch embedding + interpolated position table.
 * mhe_vision_blocks: blocks [first, first + count) of w->blocks in place.
 * mhe_vision_merge: one merger on hidden -> out [n_patches / merge^2,
 * out_hidden]; postshuffle 0 for the main merger, 1 for a DeepStack merger. */
int32_t mhe_vision_embed(const mhe_vision_config* cfg, const mhe_vision_weights* w,
                         const void* pixels, const int32_t* grid_thw, int32_t n_grids,
                         void* hidden, void* workspace, size_t workspace_bytes, void* stream);
int32_t mhe_vision_blocks(const mhe_vision_config* cfg, const mhe_vision_weights* w,
                          int32_t first, int32_t count, void* hidden, const int32_t* grid_thw,
                          int32_t n_grids, void* workspace, size_t workspace_bytes, void* stream);
int32_t mhe_vision_merge(const mhe_vision_config* cfg, const mhe_vision_merger_weights* m,
                         int32_t postshuffle, const void* hidden, int32_t n_patches, void* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * The tower's per-frame attention on its own (H3 encoder page,
 * MiniMaxH3Qwen3VLVisionAttention.forward: non-causal softmax(q k^T /
 * sqrt(head_dim)) v within each frame, the page's cu_seqlens), for per-step
 * checks. q [n_patches, n_heads, 128], k [n_heads, seq_pad, 128] and vt
 * [n_heads, 128, seq_pad] in the layouts of mhe_qk_norm_rope (head dims past
 * head_dim zero; seq_pad = n_patches rounded up to 128; V^T token-permuted in
 * groups of 16); o [n_patches, n_heads * head_dim] bf16. The frames are those
 * of grid_thw (HOST int32 [n_grids, 3], patch grids as for
 * mhe_vision_forward, merge their spatial merge size). head_dim % 4 == 0,
 * <= 128. workspace: mhe_vision_attention_workspace_bytes(n_patches) bytes,
 * 256-byte aligned (per-patch frame ranges).
 */
size_t mhe_vision_attention_workspace_bytes(int32_t n_patches);
int32_t mhe_vision_attention(const void* q, const void* k, const void* vt, void* o,
                             int32_t n_patches, int32_t n_heads, int32_t head_dim,
                             const int32_t* grid_thw, int32_t n_grids, int32_t merge,
                             void* workspace, size_t workspace_bytes, void* stream);

/* y = LayerNorm(x) * w + b over rows of dim (biased variance, fp32), one
 * bf16 rounding (nn.LayerNorm of the vision blocks). dim % 8 == 0, <= 8192;
 * x and y may alias. */
int32_t mhe_layer_norm(const void* x, const void* w, const void* b, void* y, int32_t rows,
                       int32_t dim, float eps, void* stream);

/* c = act(a w^T + bias) (+ residual when act == 0), fp32 accumulation, one
 * bf16 rounding: the biased linears of the vision tower. act: 0 none, 1 GELU
 * tanh form, 2 GELU erf form. Shapes and workspace as mhe_linear. */
int32_t mhe_linear_bias(const void* a, const void* w, const void* bias, void* c,
                        const void* residual, int32_t m, int32_t n, int32_t k, int32_t act,
                        void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MHE_H */
