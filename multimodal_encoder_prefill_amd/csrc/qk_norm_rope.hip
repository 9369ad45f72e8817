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
// The cos/sin of every (token, slot) depend only on the positions, so an
// encode computes them once (rope_table_kernel, [seq][D/2] float pairs) and
// every layer reads them; the single-step entry point without a table builds
// its tokens' angles in LDS instead (same operations, same values).
//
// HBM-bound: per token it reads and writes (n_heads + 2 n_kv_heads) * D bf16.
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int kTok = 16;          // tokens per workgroup
constexpr int kHeadsPerBlock = 8; // q/k heads per workgroup (grid.y chunks)
constexpr int kThreads = 256;

// cos and sin of rotary slot j (< D/2) of token s
__device__ __forceinline__ float2 rope_angle(const int32_t* __restrict__ pos, int seq, int s, int j, int D,
                                             float theta, int sec1, int sec2) {
  int axis = 0;
  if (j % 3 == 1 && j < 3 * sec1) axis = 1;
  else if (j % 3 == 2 && j < 3 * sec2) axis = 2;
  const float inv_freq = 1.0f / powf(theta, static_cast<float>(2 * j) / static_cast<float>(D));
  const float ang = static_cast<float>(pos[axis * seq + s]) * inv_freq;
  float sn, cn;
  sincosf(ang, &sn, &cn);
  return make_float2(cn, sn);
}

__global__ __launch_bounds__(kThreads) void rope_table_kernel(const int32_t* __restrict__ pos, int seq, int D,
                                                             float theta, int sec1, int sec2,
                                                             float2* __restrict__ table) {
  const int half = D / 2;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= seq * half) return;
  table[e] = rope_angle(pos, seq, e / half, e % half, D, theta, sec1, sec2);
}

// q / k head rows handled per wavefront per batch (4 rows per pass)
constexpr int kPasses = 4;

template <int D, bool TABLE>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ q_gain,
    const bf16_t* __restrict__ k_gain, const int32_t* __restrict__ pos,
    const float2* __restrict__ table, int seq, int seq_pad, int n_heads, int n_kv_heads, float eps,
    float theta, int sec1, int sec2, bf16_t* __restrict__ q_out, bf16_t* __restrict__ k_out,
    bf16_t* __restrict__ vt_out) {
  constexpr int HALF = D / 2;
  const int s0 = blockIdx.x * kTok;
  const int width = (n_heads + 2 * n_kv_heads) * D;

  if (blockIdx.y == 0) {
    // ---- V: [seq, kv*D] -> [kv][D][seq_pad], permuted within 16-token groups.
    //      Thread pair (2c, 2c+1) takes the 8 consecutive (head, d) columns of
    //      chunk c; each thread loads them for 8 tokens (16-byte loads) and
    //      stores, per column, its two 4-token pieces of the permuted group:
    //      tokens 0-3 / 4-7 go to slots 0-3 / 8-11, tokens 8-11 / 12-15 to
    //      slots 4-7 / 12-15 (perm16). ----
    const int vbase = (n_heads + n_kv_heads) * D;
    const int half = threadIdx.x & 1;
    for (int g16 = s0; g16 < s0 + kTok; g16 += 16)
    for (int c = threadIdx.x >> 1; c < n_kv_heads * D / 8; c += kThreads / 2) {
      u32x4 v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int s = g16 + 8 * half + t;
        v[t] = s < seq ? *reinterpret_cast<const u32x4*>(qkv + static_cast<size_t>(s) * width + vbase + c * 8)
                       : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int col = c * 8 + i;               // = g * D + d
        const int sh = 16 * (i & 1);
        uint32_t e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (v[t][i >> 1] >> sh) & 0xffffu;
        u32x2 a, b2;
        a[0] = e[0] | (e[1] << 16);
        a[1] = e[2] | (e[3] << 16);
        b2[0] = e[4] | (e[5] << 16);
        b2[1] = e[6] | (e[7] << 16);
        bf16_t* row = vt_out + static_cast<size_t>(col) * seq_pad + g16;
        *reinterpret_cast<u32x2*>(row + 4 * half) = a;
        *reinterpret_cast<u32x2*>(row + 8 + 4 * half) = b2;
      }
    }
    return;
  }

  // ---- rotary cos/sin of the block's tokens into LDS: copied from the
  //      encode's table, or formed here (every head row of a token reads them).
  //      A lane of chunk c uses the slots 8c' .. 8c'+7 (c' = c mod CH) as four
  //      float4 (two (cos, sin) pairs each); token t's float4 number i of
  //      chunk c' is stored at t * HALF/2 + i * CH + c', so that one read
  //      instruction of the CH lanes of a row takes consecutive 16-byte words
  //      (stored chunk-major, those reads were 64 bytes apart and collided
  //      in the LDS banks). ----
  constexpr int CH = HALF / 8;  // slot chunks of 8 per token
  auto cs_index = [](int t, int j) {  // float4 holding slot pair (j, j+1), j even
    return t * (HALF / 2) + ((j % 8) / 2) * CH + j / 8;
  };
  __shared__ __attribute__((aligned(16))) float2 cs[kTok * HALF];
  if constexpr (TABLE) {
    const int n4 = kTok * HALF / 2;  // float4 = two (cos, sin) pairs
    const int valid = (min(s0 + kTok, seq) - min(s0, seq)) * HALF / 2;
    const float4* src = reinterpret_cast<const float4*>(table + static_cast<size_t>(min(s0, seq)) * HALF);
    for (int e = threadIdx.x; e < n4; e += kThreads)
      reinterpret_cast<float4*>(cs)[cs_index(e / (HALF / 2), 2 * (e % (HALF / 2)))] =
          e < valid ? src[e] : make_float4(1.f, 0.f, 1.f, 0.f);
  } else {
    for (int e = threadIdx.x; e < kTok * HALF; e += kThreads) {
      const int t = e / HALF, j = e % HALF;
      cs[2 * cs_index(t, j & ~1) + (j & 1)] =
          rope_angle(pos, seq, min(s0 + t, seq - 1), j, D, theta, sec1, sec2);
    }
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
  const int h_first = (blockIdx.y - 1) * kHeadsPerBlock;
  const int h_count = min(kHeadsPerBlock, n_heads + n_kv_heads - h_first);
  const int rows = kTok * h_count;
  // kPasses row groups per batch: all their loads go out before any math
  for (int rb = wave * ROWS_PER_PASS; rb < rows; rb += 4 * ROWS_PER_PASS * kPasses) {
    float x[kPasses][8];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int r = rb + p * 4 * ROWS_PER_PASS + sub;
      const int t = r < rows ? r / h_count : 0;
      const int h = h_first + (r < rows ? r % h_count : 0);
      const int s = s0 + t;
      if (r < rows && s < seq) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qkv + static_cast<size_t>(s) * width + h * D + chunk * 8);
        unpack8(v, x[p]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[p][i] = 0.f;
      }
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int r = rb + p * 4 * ROWS_PER_PASS + sub;
      const bool active = r < rows;
      const int t = active ? r / h_count : 0;
      const int h = h_first + (active ? r % h_count : 0);
      const int s = s0 + t;
      const bool is_q = h < n_heads;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x[p][i] * x[p][i];
      ss = group_sum<LPR>(ss);
      const float rinv = rsqrtf(ss / static_cast<float>(D) + eps);
      float gn[8];
      unpack8(*reinterpret_cast<const u32x4*>((is_q ? q_gain : k_gain) + chunk * 8), gn);
      float2 cs8[8];
      const float4* tr = reinterpret_cast<const float4*>(cs) + cs_index(t, j0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = tr[i * CH];
        cs8[2 * i] = make_float2(v.x, v.y);
        cs8[2 * i + 1] = make_float2(v.z, v.w);
      }
      float y[8], o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[p][i] * rinv * gn[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float partner = __shfl_xor(y[i], LPR / 2, 64);
        const float c = cs8[i].x, sn = cs8[i].y;
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
}

}  // namespace

hipError_t launch_rope_table(const RopeParams& p, const int32_t* positions, int seq, float2* table,
                             hipStream_t stream) {
  if (seq <= 0) return hipSuccess;
  const int n = seq * (p.head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                     positions, seq, p.head_dim, p.theta, p.section[1], p.section[2], table);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const RopeParams& p, const bf16_t* qkv, const bf16_t* q_norm,
                               const bf16_t* k_norm, const int32_t* positions, int seq,
                               bf16_t* q_out, bf16_t* k_out, bf16_t* vt_out, hipStream_t stream,
                               const float2* table) {
  if (seq <= 0) return hipSuccess;
  const int sp = seq_pad(seq);
  const int n_chunks = (p.n_heads + p.n_kv_heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  dim3 grid(sp / kTok, n_chunks + 1);
#define MHE_QK_LAUNCH(DD, TT)                                                                        \
  hipLaunchKernelGGL((qk_norm_rope_kernel<DD, TT>), grid, dim3(kThreads), 0, stream, qkv, q_norm,   \
                     k_norm, positions, table, seq, sp, p.n_heads, p.n_kv_heads, p.eps, p.theta,   \
                     p.section[1], p.section[2], q_out, k_out, vt_out)
  if (p.head_dim == 128) {
    if (table) MHE_QK_LAUNCH(128, true);
    else MHE_QK_LAUNCH(128, false);
  } else if (p.head_dim == 64) {
    if (table) MHE_QK_LAUNCH(64, true);
    else MHE_QK_LAUNCH(64, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef MHE_QK_LAUNCH
  return hipGetLastError();
}

}  // namespace mhe
