// Per-head q/k RMSNorm and interleaved multimodal rotary, plus the V relayout.
//
// H3 encoder page, MiniMaxH3Qwen3VLTextAttention.forward up to the attention
// call: q and k are viewed as heads of head_dim, each head row is RMS-
// normalised with the q_norm / k_norm gain, then rotated with
// rotate-half RoPE whose angle for frequency slot j is
// pos[axis(j)] * theta^(-2j/D) (MiniMaxH3Qwen3VLTextRotaryEmbedding and
// _apply_interleaved_mrope: axis H for j % 3 == 1, j < 3*section[1]; axis W
// for j % 3 == 2, j < 3*section[2]; axis T otherwise). Angles are formed in
// fp32 (inverse frequency and position product as on the page) and cos/sin
// are kept in fp32; each output is rounded to bf16 once.
//
// The kernel also writes K as [kv_head][seq_pad][D] and V transposed as
// [kv_head][D][seq_pad] with tokens permuted inside every aligned group of 16
// (0 1 2 3 8 9 10 11 4 5 6 7 12 13 14 15), which is the order in which one
// 32x32x16 MFMA step of the attention kernel consumes probabilities, so the
// attention kernel reads both K and V with plain 16-byte LDS loads. seq_pad
// is seq rounded up to 128 (the attention key tile); padding tokens
// (seq <= s < seq_pad) are written as zeros.
//
// HBM-bound: per token it reads and writes (n_heads + 2 n_kv_heads) * D bf16.
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int kTok = 16;          // tokens per workgroup
constexpr int kHeadsPerBlock = 8; // q/k heads per workgroup (grid.y chunks)
constexpr int kThreads = 256;

__device__ __forceinline__ int perm16(int p) {
  // physical slot p of a 16-token group holds token perm16(p)
  return (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1);
}

template <int D>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ q_gain,
    const bf16_t* __restrict__ k_gain, const int32_t* __restrict__ pos, int seq, int seq_pad,
    int n_heads, int n_kv_heads, float eps, float theta, int sec1, int sec2,
    bf16_t* __restrict__ q_out, bf16_t* __restrict__ k_out, bf16_t* __restrict__ vt_out) {
  constexpr int HALF = D / 2;
  const int s0 = blockIdx.x * kTok;
  const int width = (n_heads + 2 * n_kv_heads) * D;
  const int n_chunks = (n_heads + n_kv_heads + kHeadsPerBlock - 1) / kHeadsPerBlock;

  if (static_cast<int>(blockIdx.y) == n_chunks) {
    // ---- V: [seq, kv*D] -> [kv][D][seq_pad], permuted within 16-token groups ----
    const int vbase = (n_heads + n_kv_heads) * D;
    for (int pair = threadIdx.x; pair < n_kv_heads * D; pair += kThreads) {
      const int g = pair / D, d = pair % D;
      float v[kTok];
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        const int s = s0 + t;
        v[t] = s < seq ? bf16_to_f32(qkv[static_cast<size_t>(s) * width + vbase + pair]) : 0.f;
      }
      u32x4 lo, hi;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        lo[p] = pack_bf16x2(v[perm16(2 * p)], v[perm16(2 * p + 1)]);
        hi[p] = pack_bf16x2(v[perm16(8 + 2 * p)], v[perm16(8 + 2 * p + 1)]);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(vt_out + (static_cast<size_t>(g) * D + d) * seq_pad + s0);
      dst[0] = lo;
      dst[1] = hi;
    }
    return;
  }

  // ---- rotary table for the block's tokens: slot j's angle in fp32 ----
  __shared__ float cs[kTok][HALF][2];
  for (int e = threadIdx.x; e < kTok * HALF; e += kThreads) {
    const int t = e / HALF, j = e % HALF;
    const int s = min(s0 + t, seq - 1);
    int axis = 0;
    if (j % 3 == 1 && j < 3 * sec1) axis = 1;
    else if (j % 3 == 2 && j < 3 * sec2) axis = 2;
    const float inv_freq = 1.0f / powf(theta, static_cast<float>(2 * j) / static_cast<float>(D));
    const float ang = static_cast<float>(pos[axis * seq + s]) * inv_freq;
    float sn, cn;
    sincosf(ang, &sn, &cn);
    cs[t][j][0] = cn;
    cs[t][j][1] = sn;
  }
  __syncthreads();

  // ---- q / k head rows: D/8 lanes per row, 8 consecutive elements per lane;
  //      element d pairs with d +- D/2, which sits D/16 lanes away ----
  constexpr int LPR = D / 8;           // lanes per head row
  constexpr int ROWS_PER_PASS = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / LPR;
  const int chunk = lane % LPR;
  const bool first_half = chunk < LPR / 2;
  const int j0 = (chunk % (LPR / 2)) * 8;   // rotary slot of this lane's first element
  const int h_first = blockIdx.y * kHeadsPerBlock;
  const int h_count = min(kHeadsPerBlock, n_heads + n_kv_heads - h_first);
  const int rows = kTok * h_count;
  for (int r0 = wave * ROWS_PER_PASS; r0 < rows; r0 += 4 * ROWS_PER_PASS) {
    const int r = r0 + sub;
    const bool active = r < rows;
    const int t = active ? r / h_count : 0;
    const int h = h_first + (active ? r % h_count : 0);
    const int s = s0 + t;
    const bool is_q = h < n_heads;
    float x[8];
    if (active && s < seq) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qkv + static_cast<size_t>(s) * width + h * D + chunk * 8);
      unpack8(v, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
    ss = group_sum<LPR>(ss);
    const float rinv = rsqrtf(ss / static_cast<float>(D) + eps);
    float gn[8];
    unpack8(*reinterpret_cast<const u32x4*>((is_q ? q_gain : k_gain) + chunk * 8), gn);
    float y[8], o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * rinv * gn[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float partner = __shfl_xor(y[i], LPR / 2, 64);
      const float c = cs[t][j0 + i][0], sn = cs[t][j0 + i][1];
      // first half: x cos - x_partner sin; second half: x cos + x_partner sin
      o[i] = first_half ? y[i] * c - partner * sn : y[i] * c + partner * sn;
    }
    if (!active) continue;
    if (is_q) {
      if (s < seq)
        *reinterpret_cast<u32x4*>(q_out + (static_cast<size_t>(s) * n_heads + h) * D + chunk * 8) = pack8(o);
    } else if (s < seq_pad) {
      const int g = h - n_heads;
      u32x4 v = pack8(o);
      if (s >= seq) v = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(k_out + (static_cast<size_t>(g) * seq_pad + s) * D + chunk * 8) = v;
    }
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(const RopeParams& p, const bf16_t* qkv, const bf16_t* q_norm,
                               const bf16_t* k_norm, const int32_t* positions, int seq,
                               bf16_t* q_out, bf16_t* k_out, bf16_t* vt_out, hipStream_t stream) {
  if (seq <= 0) return hipSuccess;
  const int sp = seq_pad(seq);
  const int n_chunks = (p.n_heads + p.n_kv_heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  dim3 grid(sp / kTok, n_chunks + 1);
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(qk_norm_rope_kernel<128>, grid, dim3(kThreads), 0, stream, qkv, q_norm,
                       k_norm, positions, seq, sp, p.n_heads, p.n_kv_heads, p.eps, p.theta,
                       p.section[1], p.section[2], q_out, k_out, vt_out);
  } else if (p.head_dim == 64) {
    hipLaunchKernelGGL(qk_norm_rope_kernel<64>, grid, dim3(kThreads), 0, stream, qkv, q_norm,
                       k_norm, positions, seq, sp, p.n_heads, p.n_kv_heads, p.eps, p.theta,
                       p.section[1], p.section[2], q_out, k_out, vt_out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mhe
