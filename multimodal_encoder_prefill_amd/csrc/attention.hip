// Causal grouped-query flash attention on gfx950 MFMA.
//
// H3 encoder page, MiniMaxH3Qwen3VLTextAttention.forward: query head h uses
// key/value head h / (n_heads / n_kv_heads) (the page expands K/V with
// repeat_interleave; here the expansion is an index map and K/V are read once
// per group), key j is visible to query i iff j <= i (is_causal with an
// all-ones padding mask), the scale is 1/sqrt(D) (the SDPA default). Softmax is
// computed online in fp32 (running max and sum, exp2 with a log2(e) pre-scale)
// and the output is rounded to bf16 once.
//
// One workgroup = one key/value head g and 32 query rows; its G wavefronts are
// the G query heads of the group, so every K/V tile staged in LDS serves all G
// heads. Each wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (keys are the MFMA rows, queries the columns), so a lane holds 16 scores of
// a single query per 32-key block and the row max needs only one exchange
// with lane^32; the row sum stays lane-local until the end. O^T = V^T P^T is
// accumulated the same way; V arrives pre-transposed and token-permuted
// (qk_norm_rope.hip) so the probabilities produced by the first product are
// directly the second product's B operand.
//
// Workgroups are numbered so that the key/value head is blockIdx % n_kv_heads:
// with 8 key/value heads, each XCD serves one head and keeps its K/V in its
// own L2. Query blocks are issued longest-first (causal work grows with the
// block index).
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int QB = 32;   // query rows per workgroup
constexpr int KT = 64;   // keys per tile

__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int D, int G>
__global__ __launch_bounds__(64 * G) void attention_kernel(const bf16_t* __restrict__ q,
                                                          const bf16_t* __restrict__ k,
                                                          const bf16_t* __restrict__ vt,
                                                          bf16_t* __restrict__ o, int ldo,
                                                          int seq, int n_heads, int n_kv_heads,
                                                          float scale_log2) {
  constexpr int KCH = D / 8;         // 16-byte chunks per K row
  constexpr int NTH = 64 * G;
  constexpr int K_CHUNKS = KT * KCH;  // per tile
  constexpr int V_CHUNKS = D * (KT / 8);
  constexpr int K_PER_T = (K_CHUNKS + NTH - 1) / NTH;
  constexpr int V_PER_T = (V_CHUNKS + NTH - 1) / NTH;
  constexpr int DS = D / 16;         // MFMA k-steps over head_dim
  constexpr int DB = D / 32;         // 32-row blocks of O^T

  __shared__ __attribute__((aligned(16))) bf16_t k_lds[2][KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[2][D * KT];

  const int sp = (seq + 63) / 64 * 64;
  const int n_qb = (seq + QB - 1) / QB;
  const int g = blockIdx.x % n_kv_heads;
  const int qb = n_qb - 1 - static_cast<int>(blockIdx.x / n_kv_heads);
  const int q0 = qb * QB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = g * G + wave;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;

  // ---- Q rows as the MFMA B operand, kept in registers ----
  bf16x8 qreg[DS];
  {
    const int qi = q0 + lrow;
    const bf16_t* src = q + (static_cast<size_t>(min(qi, seq - 1)) * n_heads + h) * D + lhalf * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(src + s * 16);
      if (qi >= seq) v = u32x4{0, 0, 0, 0};
      qreg[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const bf16_t* kg = k + static_cast<size_t>(g) * sp * D;
  const bf16_t* vg = vt + static_cast<size_t>(g) * D * sp;
  const int last_key = min(q0 + QB - 1, seq - 1);
  const int n_tiles = last_key / KT + 1;

  u32x4 kst[K_PER_T], vst[V_PER_T];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NTH;
      if (c < K_CHUNKS) kst[i] = *reinterpret_cast<const u32x4*>(kg + static_cast<size_t>(t * KT) * D + c * 8);
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int c = tid + i * NTH;
      if (c < V_CHUNKS) {
        const int d = c / (KT / 8), ch = c % (KT / 8);
        vst[i] = *reinterpret_cast<const u32x4*>(vg + static_cast<size_t>(d) * sp + t * KT + ch * 8);
      }
    }
  };
  auto store_tile = [&](int stage) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NTH;
      if (c < K_CHUNKS) {
        const int row = c / KCH, ch = c % KCH;
        const int phys = (KCH == 16) ? (ch ^ (row & 15)) : (ch ^ swz8(row));
        *reinterpret_cast<u32x4*>(&k_lds[stage][row * D + phys * 8]) = kst[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int c = tid + i * NTH;
      if (c < V_CHUNKS) {
        const int d = c / (KT / 8), ch = c % (KT / 8);
        *reinterpret_cast<u32x4*>(&v_lds[stage][d * KT + ((ch ^ swz8(d)) * 8)]) = vst[i];
      }
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[b][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const int qi = q0 + lrow;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const bf16_t* kl = k_lds[cur];
    const bf16_t* vl = v_lds[cur];

    // ---- S^T for 64 keys: two 32-key blocks ----
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
      const int row = kb * 32 + lrow;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const int ch = 2 * s + lhalf;
        const int phys = (KCH == 16) ? (ch ^ (row & 15)) : (ch ^ swz8(row));
        const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kl + row * D + phys * 8));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[s], sacc[kb], 0, 0, 0);
      }
    }

    // ---- online softmax (log2 domain); lane's query is qi, keys per register ----
    const bool diag = (t * KT + KT - 1) > q0;  // tile may hold keys past some query
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = sacc[kb][e] * scale_log2;
        if (diag) {
          const int key = t * KT + kb * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
          if (key > qi) x = -INFINITY;
        }
        sacc[kb][e] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);   // 0 on the first tile (m_run = -inf)
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pop[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = exp2f(sacc[kb][hh * 8 + e] - m_new);
          psum += pv[e];
        }
        pop[kb * 2 + hh] = __builtin_bit_cast(bf16x8, pack8(pv));
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[b][e] *= alpha;

    // ---- O^T += V^T P^T: 4 steps of 16 keys ----
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const int d = b * 32 + lrow;
#pragma unroll
      for (int s = 0; s < KT / 16; ++s) {
        const int ch = 2 * s + lhalf;
        const bf16x8 vop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vl + d * KT + ((ch ^ swz8(d)) * 8)));
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[s], oacc[b], 0, 0, 0);
      }
    }

    if (t + 1 < n_tiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds query lrow, d = 32b + 8(e/4) + 4 lhalf + e%4 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qi < seq) {
    const float inv = 1.f / l_tot;
    bf16_t* dst = o + static_cast<size_t>(qi) * ldo + h * D + lhalf * 4;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 pk;
        pk[0] = pack_bf16x2(oacc[b][gq * 4 + 0] * inv, oacc[b][gq * 4 + 1] * inv);
        pk[1] = pack_bf16x2(oacc[b][gq * 4 + 2] * inv, oacc[b][gq * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + b * 32 + gq * 8) = pk;
      }
  }
}

template <int D>
hipError_t launch_d(const bf16_t* q, const bf16_t* k, const bf16_t* vt, bf16_t* o, int ldo,
                    int seq, int n_heads, int n_kv_heads, hipStream_t stream) {
  const int G = n_heads / n_kv_heads;
  const int n_qb = (seq + QB - 1) / QB;
  const dim3 grid(n_qb * n_kv_heads);
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  switch (G) {
#define MHE_ATTN_CASE(GG)                                                                      \
  case GG:                                                                                     \
    hipLaunchKernelGGL((attention_kernel<D, GG>), grid, dim3(64 * GG), 0, stream, q, k, vt, o, \
                       ldo, seq, n_heads, n_kv_heads, scale_log2);                             \
    break;
    MHE_ATTN_CASE(1)
    MHE_ATTN_CASE(2)
    MHE_ATTN_CASE(4)
    MHE_ATTN_CASE(8)
#undef MHE_ATTN_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool attention_supported(int n_heads, int n_kv_heads, int head_dim) {
  if (n_kv_heads <= 0 || n_heads % n_kv_heads != 0) return false;
  const int g = n_heads / n_kv_heads;
  return (head_dim == 64 || head_dim == 128) && (g == 1 || g == 2 || g == 4 || g == 8);
}

hipError_t launch_attention(const bf16_t* q, const bf16_t* k, const bf16_t* vt, bf16_t* o,
                            int ldo, int seq, int n_heads, int n_kv_heads, int head_dim,
                            hipStream_t stream) {
  if (seq <= 0) return hipSuccess;
  if (ldo < n_heads * head_dim || ldo % 4 != 0) return hipErrorInvalidValue;
  if (head_dim == 128) return launch_d<128>(q, k, vt, o, ldo, seq, n_heads, n_kv_heads, stream);
  if (head_dim == 64) return launch_d<64>(q, k, vt, o, ldo, seq, n_heads, n_kv_heads, stream);
  return hipErrorInvalidValue;
}

}  // namespace mhe
