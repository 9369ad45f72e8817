// Launchers of the libmhe kernels (host side, called by api.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <stdint.h>

namespace mhe {

typedef uint16_t bf16_t;

// rmsnorm.hip
bool rmsnorm_supported(int dim);
// y rows are ldy elements apart (>= dim, multiple of 8); x is dense.
hipError_t launch_rmsnorm(const bf16_t* x, const bf16_t* gamma, bf16_t* y, int ldy, int rows,
                          int dim, float eps, hipStream_t stream);
// LayerNorm with weight and bias; x rows ldx apart, y rows ldy apart (x and y
// may alias with ldx == ldy).
hipError_t launch_layernorm(const bf16_t* x, int ldx, const bf16_t* w, const bf16_t* b, bf16_t* y,
                            int ldy, int rows, int dim, float eps, hipStream_t stream);

// gemm.hip: C[m, n] = A[m, :] . B[n, :] with one of these epilogues:
//   kStore C = AB^T, kResidual C = R + AB^T, kSwiGLU C = silu(AB_g^T) * AB_u^T,
//   kBias C = AB^T + b, kBiasResidual C = R + (AB^T + b),
//   kBiasGeluTanh / kBiasGeluErf C = gelu(AB^T + b) (tanh / erf form).
enum class Epilogue {
  kStore = 0, kResidual = 1, kSwiGLU = 2, kBias = 3, kBiasResidual = 4, kBiasGeluTanh = 5,
  kBiasGeluErf = 6
};

// Up to three row segments that together form the B operand (e.g. w_q | w_k | w_v).
struct BSegments {
  const bf16_t* ptr[3];
  int rows[3];
  int count;
};

bool gemm_supported(int n, int k);
// Rows of one load block; each segment of a multi-segment B must be a multiple.
int gemm_segment_rows();
// kStore / kResidual: B is the concatenation of the segments (n = total rows).
// kSwiGLU: seg 0 = gate, seg 1 = up, each n rows; C has n columns.
// `partial` (may be NULL) is fp32 scratch for split-K units of the last wave;
// gemm_partial_bytes() is enough for every shape.
size_t gemm_partial_bytes();
// lda / ldb: row strides in elements (>= k, multiples of 8) of A and of B;
// ldc: row stride of C and of the residual (>= n, multiple of 4).
// bias [n] bf16 for the kBias* epilogues (ignored otherwise).
hipError_t launch_gemm(Epilogue epi, const bf16_t* a, int lda, const BSegments& b, int ldb,
                       bf16_t* c, int ldc, const bf16_t* residual, int m, int n, int k,
                       float* partial, size_t partial_bytes, hipStream_t stream,
                       const bf16_t* bias = nullptr);

// FP8 (E4M3) operands with per-tensor scales: C = epilogue(scale_a * scale_b
// * A B^T), scale pointers device floats. kStore, kResidual and kSwiGLU only;
// k % 128 == 0; lda / ldb in bytes, multiples of 16. Segments as BSegments,
// each with its own scale.
struct F8Segments {
  const uint8_t* ptr[3];
  int rows[3];
  const float* scale[3];
  int count;
};
bool gemm_fp8_supported(int n, int k);
// amax (kSwiGLU only, may be NULL): partial maxima of |C| as stored, one per
// workgroup that writes outputs, gemm_amax_parts(m, n) floats at most; the
// count written goes to *amax_count.
int gemm_amax_parts(int m, int n);
hipError_t launch_gemm_fp8(Epilogue epi, const uint8_t* a, int lda, const float* scale_a,
                           const F8Segments& b, int ldb, bf16_t* c, int ldc,
                           const bf16_t* residual, int m, int n, int k, float* partial,
                           size_t partial_bytes, hipStream_t stream, float* amax = nullptr,
                           int* amax_count = nullptr);

// quant.hip: per-tensor E4M3 quantisation. launch_amax writes nparts
// (<= kAmaxParts; amax_parts(rows) is the usual count) partial maxima of |x|;
// launch_amax_finalize reduces nparts partials (of one tensor, possibly from
// several launches) into scale[0] = max|x| / 448 (1 for an all-zero tensor)
// and factor[0] = 448 / max|x|; launch_quantize_fp8 writes the codes
// q [rows, ldq] of x times factor[0]. cols, ldx, ldq multiples of 8.
constexpr int kAmaxParts = 1024;
int amax_parts(int rows);
hipError_t launch_amax(const bf16_t* x, int ldx, int rows, int cols, float* partial, int nparts,
                       hipStream_t stream);
hipError_t launch_amax_finalize(const float* partial, int nparts, float* scale, float* factor,
                                hipStream_t stream);
hipError_t launch_quantize_fp8(const bf16_t* x, int ldx, int rows, int cols, const float* factor,
                               uint8_t* q, int ldq, hipStream_t stream);
// rmsnorm.hip: the RMSNorm of x quantised to E4M3 without writing it in bf16
// (the codes of exactly the bf16 rows launch_rmsnorm would write): partial
// maxima (rmsnorm_fp8_parts(rows) floats), finalize, quantize.
int rmsnorm_fp8_parts(int rows);
hipError_t launch_rmsnorm_fp8(const bf16_t* x, const bf16_t* gamma, int rows, int dim, float eps,
                              float* partial, float* scale, float* factor, uint8_t* q, int ldq,
                              hipStream_t stream);

// qk_norm_rope.hip
struct RopeParams {
  int n_heads, n_kv_heads, head_dim;
  float eps, theta;
  int section[3];
};
// tokens of the K / V^T layouts: seq rounded up to a multiple of 128
__host__ __device__ inline int seq_pad(int seq) { return (seq + 127) / 128 * 128; }
// table (may be NULL): the rotary cos/sin of every (token, slot), [seq][D/2]
// float pairs from launch_rope_table; without it each workgroup forms its
// tokens' values itself (identical results).
hipError_t launch_rope_table(const RopeParams& p, const int32_t* positions, int seq, float2* table,
                             hipStream_t stream);
hipError_t launch_qk_norm_rope(const RopeParams& p, const bf16_t* qkv, const bf16_t* q_norm,
                               const bf16_t* k_norm, const int32_t* positions, int seq,
                               bf16_t* q_out, bf16_t* k_out, bf16_t* vt_out, hipStream_t stream,
                               const float2* table = nullptr);
// The k heads and the V relayout only (the decoder layer: q is normalised and
// rotated by launch_attention_qnorm); k_out and vt_out as above.
hipError_t launch_k_norm_rope(const RopeParams& p, const bf16_t* qkv, const bf16_t* k_norm,
                              const int32_t* positions, int seq, bf16_t* k_out, bf16_t* vt_out,
                              hipStream_t stream, const float2* table);

// attention.hip
bool attention_supported(int n_heads, int n_kv_heads, int head_dim);
// o rows are ldo elements apart (>= n_heads * head_dim, multiple of 4).
// amax (may be NULL): max |o| as stored of each workgroup, at
// amax[0, attention_amax_parts(seq, n_kv_heads)) (the FP8 layer's input
// maxima for the O projection).
int attention_amax_parts(int seq, int n_kv_heads);
hipError_t launch_attention(const bf16_t* q, const bf16_t* k, const bf16_t* vt, bf16_t* o,
                            int ldo, int seq, int n_heads, int n_kv_heads, int head_dim,
                            hipStream_t stream, float* amax = nullptr);
// The same attention with q taken raw from the q/k/v projection output
// (q_raw rows ldq elements apart, q heads first) and normalised (gain q_gain
// [head_dim], eps) and rotated (cos/sin table rope from launch_rope_table) as
// it is loaded: the q half of launch_qk_norm_rope fused into the attention.
hipError_t launch_attention_qnorm(const bf16_t* q_raw, int ldq, const bf16_t* q_gain, const float2* rope,
                                  float eps, const bf16_t* k, const bf16_t* vt, bf16_t* o, int ldo, int seq,
                                  int n_heads, int n_kv_heads, int head_dim, hipStream_t stream,
                                  float* amax = nullptr);

// deepstack.hip
// Ascending list idx[0, n_vis) of the tokens whose byte in mask is set;
// entries past the popcount are -1; *count = popcount.
hipError_t launch_visual_index(const uint8_t* mask, int seq, int n_vis, int32_t* idx,
                               int32_t* count, hipStream_t stream);
// The library's own device scratch for the visual index list of callers that
// cannot allocate: kStaticIndexRows entries and a count, one copy per device
// (its address looked up on the first call on that device). Calls that
// overlap on one device share it and race.
constexpr int kStaticIndexRows = 1 << 17;
hipError_t static_index_scratch(int32_t** idx, int32_t** count);
// hidden[idx[r]] += feature[r] (fp32 add, one bf16 rounding), r < n_vis
hipError_t launch_deepstack_add(bf16_t* hidden, int hidden_dim, const int32_t* idx, int n_vis,
                                const bf16_t* feature, hipStream_t stream);
// hidden[idx[r]] = feature[r], r < n
hipError_t launch_row_scatter(bf16_t* hidden, int hidden_dim, const int32_t* idx, int n,
                              const bf16_t* feature, hipStream_t stream);

// vision.hip
// Per patch, in the tower's block order: row and column in its image, the
// image's patch grid (h, w) and the token range of its frame.
struct PatchInfo {
  int row, col, h, w, seg_lo, seg_hi, pad0, pad1;
};
constexpr int kMaxVisionGrids = 64;
// Patch grids (t, h, w) of the images / videos of one call, by value.
struct VisionGrids {
  int count, merge;
  int t[kMaxVisionGrids], h[kMaxVisionGrids], w[kMaxVisionGrids];
};
hipError_t launch_patch_info(const VisionGrids& grids, int n, PatchInfo* info, hipStream_t stream);
// hidden[s] += bilinear(table [side*side, dim]) at patch s
hipError_t launch_pos_embed(bf16_t* hidden, int ld, int n, int dim, const bf16_t* table, int side,
                            const PatchInfo* info, hipStream_t stream);
// qkv [n, 3 heads head_dim] (row stride ldq) -> rotated q [n, heads, 128],
// k [heads, seq_pad(n), 128], permuted V^T [heads, 128, seq_pad(n)], zero padded
hipError_t launch_vision_rope_table(const PatchInfo* info, int n, int head_dim, float2* table,
                                    hipStream_t stream);
hipError_t launch_vision_rope(const bf16_t* qkv, int ldq, int n, int heads, int head_dim,
                              const float2* table, bf16_t* q_out, bf16_t* k_out, bf16_t* vt_out,
                              hipStream_t stream);
// Non-causal attention within each frame (info[s].seg_lo .. seg_hi) on the
// layouts above: heads of head_dim (<= 128, stored padded to 128), scale
// 1/sqrt(head_dim); o [n, heads * head_dim] with row stride ldo.
hipError_t launch_segment_attention(const bf16_t* q, const bf16_t* k, const bf16_t* vt, bf16_t* o,
                                    int ldo, int n, int heads, int head_dim,
                                    const PatchInfo* info, hipStream_t stream);

// frontend.hip
// Multimodal rotary positions [3, seq] (host) and optional host masks from
// token ids; returns an mhe_status, with a message in *err on failure.
int rope_index_host(const int32_t* ids, int seq, int image_token_id, int video_token_id,
                    const int32_t* image_grid, int n_images, const int32_t* video_grid,
                    int n_videos, int merge, int32_t* positions, uint8_t* image_mask,
                    uint8_t* video_mask, uint8_t* visual_mask, int32_t* delta,
                    std::string* err);
// out[s] = table[ids[s] - row_begin] for ids in [row_begin, row_begin + rows),
// else a zero row (counted into *n_outside when not NULL)
hipError_t launch_embed_gather(const int32_t* ids, int seq, const bf16_t* table, int row_begin,
                               int rows, int dim, bf16_t* out, int32_t* n_outside,
                               hipStream_t stream);
// joint[r] = the feature row of the r-th visual token (image or video); src:
// n_image + n_video ints of scratch
hipError_t launch_join_visual(const uint8_t* image_mask, const uint8_t* video_mask, int seq,
                              int n_image, const bf16_t* image_feature, int n_video,
                              const bf16_t* video_feature, int dim, int32_t* src, bf16_t* joint,
                              hipStream_t stream);

}  // namespace mhe
