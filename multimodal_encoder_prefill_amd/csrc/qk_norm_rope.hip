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
// A launch covers the q and k heads, or (in the decoder layer, where the
// attention kernel normalises and rotates q as it loads it) the k heads only.
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
// every layer reads them; the single-step entry point without a table forms
// each lane's angles in registers instead (same operations, same values).
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

// Value of the lane N places further along its aligned row of 16 lanes (a DPP
// row rotation: a plain VALU move, no LDS traffic unlike a lane permute).
template <int N>
__device__ __forceinline__ float row_rotate(float x) {
  static_assert(N >= 1 && N <= 15, "row rotation by 1..15 lanes");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

// Sum over an aligned group of LPR lanes, the same bits in every lane of the
// group. For 16-lane groups the rotations by 8, 4, 2, 1 pair the same values
// as the xor butterfly (each step's two addends are equal across the lanes
// that meet), through DPP instead of LDS permutes.
template <int LPR>
__device__ __forceinline__ float head_row_sum(float x) {
  if constexpr (LPR == 16) {
    x += row_rotate<8>(x);
    x += row_rotate<4>(x);
    x += row_rotate<2>(x);
    x += row_rotate<1>(x);
    return x;
  } else {
    return group_sum<LPR>(x);
  }
}

// The element D/2 away in the same head row: LPR/2 lanes away, i.e. the lane
// xor LPR/2 (for 16-lane rows the rotation by 8).
template <int LPR>
__device__ __forceinline__ float rotary_partner(float y) {
  if constexpr (LPR == 16) return row_rotate<8>(y);
  else return __shfl_xor(y, LPR / 2, 64);
}

template <int D, bool TABLE>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ q_gain,
    const bf16_t* __restrict__ k_gain, const int32_t* __restrict__ pos,
    const float2* __restrict__ table, int seq, int seq_pad, int n_heads, int n_kv_heads, float eps,
    float theta, int sec1, int sec2, int first_head, bf16_t* __restrict__ q_out,
    bf16_t* __restrict__ k_out, bf16_t* __restrict__ vt_out) {
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

  // ---- q / k head rows: D/8 lanes per row (a row group), 8 consecutive
  //      elements per lane; element d pairs with d +- D/2, which sits D/16
  //      lanes away. A row group keeps one token and walks its heads, so the
  //      lane's rotary cos/sin (8 slots) are read or formed once, in
  //      registers: no LDS stage and no barrier, and every head row of the
  //      group is loaded before any math. ----
  constexpr int LPR = D / 8;              // lanes per head row
  constexpr int RG = kThreads / LPR;      // row groups per workgroup
  constexpr int SPLIT = RG / kTok;        // row groups per token
  constexpr int HPR = kHeadsPerBlock / SPLIT;  // heads per row group
  static_assert(RG % kTok == 0 && kHeadsPerBlock % SPLIT == 0, "row groups must tile the block");
  const int rg = threadIdx.x / LPR;
  const int chunk = threadIdx.x % LPR;
  const bool first_half = chunk < LPR / 2;
  const int j0 = (chunk % (LPR / 2)) * 8;   // rotary slot of this lane's first element
  const int s = s0 + rg / SPLIT;
  const int hp = (rg % SPLIT) * HPR;        // first head of the group, within the block
  const int h_first = first_head + (blockIdx.y - 1) * kHeadsPerBlock;
  const int h_count = min(kHeadsPerBlock, n_heads + n_kv_heads - h_first);
  u32x4 raw[HPR];
#pragma unroll
  for (int i = 0; i < HPR; ++i)
    raw[i] = (s < seq && hp + i < h_count)
                 ? *reinterpret_cast<const u32x4*>(qkv + static_cast<size_t>(s) * width +
                                                   (h_first + hp + i) * D + chunk * 8)
                 : u32x4{0, 0, 0, 0};
  // cos/sin of slots j0 .. j0+7 of the token (the last real token stands in
  // for padding tokens, whose outputs are zeros or not stored)
  const int sc = min(s, seq - 1);
  float2 cs8[8];
  if constexpr (TABLE) {
    const float4* tr = reinterpret_cast<const float4*>(table + static_cast<size_t>(sc) * HALF + j0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = tr[i];
      cs8[2 * i] = make_float2(v.x, v.y);
      cs8[2 * i + 1] = make_float2(v.z, v.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) cs8[i] = rope_angle(pos, seq, sc, j0 + i, D, theta, sec1, sec2);
  }
  const u32x4 gq = *reinterpret_cast<const u32x4*>(q_gain + chunk * 8);
  const u32x4 gk = *reinterpret_cast<const u32x4*>(k_gain + chunk * 8);

#pragma unroll
  for (int i = 0; i < HPR; ++i) {
    const int h = h_first + hp + i;
    const bool is_q = h < n_heads;
    float x[8], gn[8];
    unpack8(raw[i], x);
    unpack8(is_q ? gq : gk, gn);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    ss = head_row_sum<LPR>(ss);
    const float rinv = rsqrtf(ss / static_cast<float>(D) + eps);
    float y[8], o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e] * rinv * gn[e];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float partner = rotary_partner<LPR>(y[e]);
      const float c = cs8[e].x, sn = cs8[e].y;
      // first half: x cos - x_partner sin; second half: x cos + x_partner sin
      o[e] = first_half ? y[e] * c - partner * sn : y[e] * c + partner * sn;
    }
    if (hp + i >= h_count) continue;
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

hipError_t launch_rope_table(const RopeParams& p, const int32_t* positions, int seq, float2* table,
                             hipStream_t stream) {
  if (seq <= 0) return hipSuccess;
  const int n = seq * (p.head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                     positions, seq, p.head_dim, p.theta, p.section[1], p.section[2], table);
  return hipGetLastError();
}

namespace {

// Heads [first_head, n_heads + n_kv_heads) of every token plus the V relayout.
hipError_t launch_heads(const RopeParams& p, const bf16_t* qkv, const bf16_t* q_norm,
                        const bf16_t* k_norm, const int32_t* positions, int seq, int first_head,
                        bf16_t* q_out, bf16_t* k_out, bf16_t* vt_out, hipStream_t stream,
                        const float2* table) {
  if (seq <= 0) return hipSuccess;
  const int sp = seq_pad(seq);
  const int n_chunks = (p.n_heads + p.n_kv_heads - first_head + kHeadsPerBlock - 1) / kHeadsPerBlock;
  dim3 grid(sp / kTok, n_chunks + 1);
#define MHE_QK_LAUNCH(DD, TT)                                                                        \
  hipLaunchKernelGGL((qk_norm_rope_kernel<DD, TT>), grid, dim3(kThreads), 0, stream, qkv, q_norm,   \
                     k_norm, positions, table, seq, sp, p.n_heads, p.n_kv_heads, p.eps, p.theta,   \
                     p.section[1], p.section[2], first_head, q_out, k_out, vt_out)
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

}  // namespace

hipError_t launch_qk_norm_rope(const RopeParams& p, const bf16_t* qkv, const bf16_t* q_norm,
                               const bf16_t* k_norm, const int32_t* positions, int seq,
                               bf16_t* q_out, bf16_t* k_out, bf16_t* vt_out, hipStream_t stream,
                               const float2* table) {
  return launch_heads(p, qkv, q_norm, k_norm, positions, seq, 0, q_out, k_out, vt_out, stream, table);
}

hipError_t launch_k_norm_rope(const RopeParams& p, const bf16_t* qkv, const bf16_t* k_norm,
                              const int32_t* positions, int seq, bf16_t* k_out, bf16_t* vt_out,
                              hipStream_t stream, const float2* table) {
  // no q head is visited, so q_norm and q_out are never read or written
  return launch_heads(p, qkv, k_norm, k_norm, positions, seq, p.n_heads, nullptr, k_out, vt_out, stream,
                      table);
}

}  // namespace mhe
