// Causal grouped-query flash attention on gfx950 MFMA.
//
// H3 encoder page, MiniMaxH3Qwen3VLTextAttention.forward: query head h uses
// key/value head h / (n_heads / n_kv_heads) (the page expands K/V with
// repeat_interleave; here the expansion is an index map and K/V are read once
// per group), key j is visible to query i iff j <= i (is_causal with an
// all-ones padding mask), the scale is 1/sqrt(D) (the SDPA default). Softmax is
// computed online in fp32 (running max and sum, exp2 with a log2(e) pre-scale,
// the max raised lazily) and the output is rounded to bf16 once.
//
// One workgroup = one key/value head g and 32 query rows; its wavefronts each
// take HPW query heads of the group (the decoder: one, so a workgroup of 8
// wavefronts puts two on every SIMD), so every K/V tile staged in LDS serves
// all G heads and every K or V operand read from LDS feeds the MFMAs of HPW
// heads. Each wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (keys are the MFMA rows, queries the columns), so a lane holds 16 scores of
// a single query per 32-key block and the row max needs only one exchange
// with lane^32; the row sum stays lane-local until the end. O^T = V^T P^T is
// accumulated the same way; V arrives pre-transposed and token-permuted
// (qk_norm_rope.hip) so the probabilities produced by the first product are
// directly the second product's B operand. Both products keep eight 16-byte
// LDS operand reads in flight ahead of the MFMA that consumes them (the score
// MFMAs step the head dims outermost, so four independent accumulators take
// turns), and the lane ^ 32 exchanges are v_permlane32_swap, not LDS permutes.
//
// Workgroups are numbered so that the key/value head is blockIdx % n_kv_heads:
// with 8 key/value heads, each XCD serves one head and keeps its K/V in its
// own L2. Query blocks are issued longest-first (causal work grows with the
// block index).
//
// In the decoder layer (QN) the query rows come straight from the q/k/v
// projection's output and the kernel applies the per-head q RMSNorm and the
// multimodal rotary itself as it loads them (the same arithmetic as
// qk_norm_rope.hip: fp32, one bf16 rounding), so q never makes a round trip
// through HBM between the two steps; K and V^T still come from that kernel.
//
// The same kernel serves the vision tower's attention (H3 encoder page,
// MiniMaxH3Qwen3VLVisionAttention.forward): SEG replaces the causal mask by
// "key in the query's frame" (a [seg_lo, seg_hi) token range per query), the
// head_dim of 72 is stored zero-padded to 128 (zero q/k columns add nothing to
// the scores, zero V rows give output columns that are not stored; the score
// MFMAs stop at 80 dims, the PV MFMAs at 96), and with one query head per
// key/value head a workgroup
// takes QW = 8 query blocks of one head so that its 8 wavefronts share every
// K/V tile.
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int QB = 32;   // query rows per workgroup
constexpr int KT = 128;  // keys per tile (the K / V^T layouts are padded to a multiple)

__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// max of three floats as one v_max3_f32. Written out because the compiler
// otherwise precedes every max of MFMA results with a NaN-quieting copy of
// each input; scores here are finite or -inf, never NaN.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// x combined with its value in lane ^ 32 (v_permlane32_swap: a VALU lane
// exchange, no LDS round trip as with a lane permute); both orders give the
// same bits, so every lane holds the same result
__device__ __forceinline__ float max_lane32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_lane32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s + x.lo + x.hi for a pair of bf16 (v_dot2_f32_bf16 against (1, 1))
__device__ __forceinline__ float add_pair(uint32_t x, float s) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                         s, false);
}

// 32-bit LDS address of a pointer into the workgroup's LDS
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<size_t>((__attribute__((address_space(3))) const void*)p));
}

// global_load_lds_dwordx4 in its scalar-base form: lane L copies the 16
// bytes at base + off (base wave-uniform, off the lane's) to LDS address
// lds + 16 L. Written as inline assembly so that the compiler, which does not
// see it as a memory operation, places no wait for it before later LDS reads
// of other stages (the builtin made every tile wait for the next tile's K
// loads before its first score); the kernel waits for it explicitly. M0
// carries the LDS address (one wait state before the load); nothing else in
// this file's device code reads M0, so clang's warning about reserving it is
// silenced.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void global_load_lds16(const char* base, unsigned off, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// DU: head dims actually used by the PV product (a multiple of 32, <= D),
// DK: by the scores (a multiple of 16, <= DU); the layouts keep the padded D,
// the MFMAs skip the columns past DU / DK (all zero).
// QN: q holds the raw projection rows (row stride ldq), normalised with
// q_gain [D] and eps and rotated with the cos/sin table rope [seq][D/2] here;
// otherwise q is already normalised and rotated ([seq][n_heads][D], ldq =
// n_heads * D) and q_gain / rope are unused.
template <int D, int G, int HPW, int QW, bool SEG, bool QN, int DU = D, int DK = DU>
__global__ __launch_bounds__(64 * (G / HPW) * QW) void attention_kernel(
    const bf16_t* q, int ldq, const bf16_t* q_gain, const float2* rope, float eps,
    const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ vt, bf16_t* __restrict__ o, int ldo, int seq, int n_heads,
    int n_kv_heads, float scale_log2, int dout, const PatchInfo* __restrict__ info,
    float* __restrict__ amax) {
  constexpr int HW = G / HPW;        // wavefronts per query block (heads of the group)
  constexpr int WAVES = HW * QW;
  constexpr int KCH = D / 8;          // 16-byte chunks per K row
  static_assert(DU % 32 == 0 && DU <= D && DK % 16 == 0 && DK <= DU, "used head dims");
  constexpr int DS = DK / 16;         // MFMA k-steps of the scores over the used head dims
  constexpr int DB = DU / 32;         // 32-row blocks of O^T
  constexpr int KB = KT / 32;         // 32-key blocks of S^T per tile
  constexpr int PS = KT / 16;         // 16-key MFMA steps of O^T += V^T P^T
  constexpr int VCH = KT / 8;         // 16-byte chunks per V^T row

  __shared__ __attribute__((aligned(16))) bf16_t k_lds[2][KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[2][D * KT];
  // QN: the cos/sin rows of the workgroup's QB queries ([QB][D/2] float2,
  // the 16-byte chunks of row r XOR-swizzled by r % 16, so the 32 rows of a
  // read spread over the banks) and the q gain, one copy for all wavefronts
  constexpr int CS_CH = D / 4;   // 16-byte chunks per cos/sin row
  __shared__ __attribute__((aligned(16))) float cs_lds[QN ? QB * D : 4];
  __shared__ __attribute__((aligned(16))) bf16_t g_lds[QN ? D : 8];

  const int sp = seq_pad(seq);
  const int n_qb = (seq + QB * QW - 1) / (QB * QW);
  const int g = blockIdx.x % n_kv_heads;
  const int qb = n_qb - 1 - static_cast<int>(blockIdx.x / n_kv_heads);
  const int q0 = qb * QB * QW;         // first query row of the workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h0 = g * G + (wave % HW) * HPW;   // this wavefront's first query head
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int qi = q0 + (wave / HW) * QB + lrow;

  // ---- Q rows of the wavefront's heads as MFMA B operands, kept in registers:
  //      lane (lrow, lhalf) holds dims 16 s + 8 lhalf + [0, 8) of query qi for
  //      k-step s (queries past seq: zeros, set once the first K/V tile is
  //      on its way) ----
  bf16x8 qreg[HPW][DS];
  const int qs = min(qi, seq - 1);
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const bf16_t* src = q + static_cast<size_t>(qs) * ldq + (h0 + hh) * D + lhalf * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) qreg[hh][s] = *reinterpret_cast<const bf16x8*>(src + s * 16);
  }
  const bf16_t* kg = k + static_cast<size_t>(g) * sp * D;
  const bf16_t* vg = vt + static_cast<size_t>(g) * D * sp;
  // key range of the workgroup: [0, last query] (causal) or the union of its
  // queries' frames (SEG); per-query limits are applied as masks
  int key_lo = 0, key_hi = min(q0 + QB * QW, seq);
  int my_lo = 0, my_hi = qi + 1;
  // SEG: keys in [in_lo, in_hi) lie in the frame of every query of the
  // workgroup, so tiles inside that range need no mask
  int in_lo = 0, in_hi = 0;
  if constexpr (SEG) {
    __shared__ int range[4];
    if (tid == 0) {
      const int last = min(q0 + QB * QW, seq) - 1;
      range[0] = info[q0].seg_lo;
      range[1] = info[last].seg_hi;
      range[2] = info[last].seg_lo;
      range[3] = info[q0].seg_hi;
    }
    if (qi < seq) {
      my_lo = info[qi].seg_lo;
      my_hi = info[qi].seg_hi;
    }
    __syncthreads();
    key_lo = range[0];     // frames are contiguous and ascending
    key_hi = range[1];
    in_lo = range[2];
    in_hi = range[3];
  }
  const int t_first = key_lo / KT;
  const int n_tiles = (key_hi - 1) / KT + 1 - t_first;

  // ---- K / V^T tiles go straight to LDS (global_load_lds_dwordx4). In
  //      load instruction i, lane L of wavefront w fills the 16 LDS bytes at
  //      offset ((i*WAVES + w)*64 + L)*16 of the tile, i.e. some row and
  //      physical chunk, and fetches the logical chunk the swizzle puts there.
  //      seq_pad is a multiple of the tile and tiles start below key_hi <=
  //      seq, so every address lies inside the K [sp, D] and V^T [D, sp]
  //      blocks of head g. ----
  constexpr int K_ROW_BYTES = D * 2;
  constexpr int V_ROW_BYTES = KT * 2;
  constexpr int K_INSTR = KT * K_ROW_BYTES / (WAVES * 1024);
  constexpr int V_INSTR = D * V_ROW_BYTES / (WAVES * 1024);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  unsigned k_src[K_INSTR], v_src[V_INSTR];  // the lane's byte offsets from the tile's first row
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int off = ((i * WAVES + wave) * 64 + lane) * 16;
    const int row = off / K_ROW_BYTES, phys = (off % K_ROW_BYTES) / 16;
    const int ch = (KCH == 16) ? (phys ^ (row & 15)) : (phys ^ swz8(row));
    k_src[i] = row * K_ROW_BYTES + ch * 16;
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int off = ((i * WAVES + wave) * 64 + lane) * 16;
    const int row = off / V_ROW_BYTES, phys = (off % V_ROW_BYTES) / 16;
    const int ch = (VCH == 16) ? (phys ^ (row & 15)) : (phys ^ swz8(row));
    v_src[i] = row * sp * 2 + ch * 16;
  }
  auto issue_tile = [&](int t, int stage) {
    const char* kb = reinterpret_cast<const char*>(kg) + static_cast<size_t>(t) * KT * K_ROW_BYTES;
    const char* vb = reinterpret_cast<const char*>(vg) + static_cast<size_t>(t) * KT * 2;
#pragma unroll
    for (int i = 0; i < K_INSTR; ++i)
      global_load_lds16(kb, k_src[i], lds_addr(&k_lds[stage][0] + (i * WAVES + wave_u) * 512));
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i)
      global_load_lds16(vb, v_src[i], lds_addr(&v_lds[stage][0] + (i * WAVES + wave_u) * 512));
  };

  f32x16 oacc[HPW][DB];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[hh][b][e] = 0.f;
  float m_run[HPW], l_run[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    // finite, so a lane whose keys all lie in later tiles computes exp2(-inf) = 0, never NaN
    m_run[hh] = -1e30f;
    l_run[hh] = 0.f;
  }

  // ---- the three phases of one key tile, for this wavefront's heads ----
  // LDS byte offsets of this lane's operand reads: row lrow of a 32-row
  // block, logical chunk 2s + lhalf for MFMA k-step s, through the swizzle.
  // A block of 32 rows changes none of the row bits the swizzle uses, so the
  // block enters as an immediate offset.
  uint32_t k_off[DS], v_off[KT / 16];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    const int ch = 2 * s + lhalf;
    k_off[s] = lrow * K_ROW_BYTES + ((KCH == 16) ? (ch ^ (lrow & 15)) : (ch ^ swz8(lrow))) * 16;
  }
#pragma unroll
  for (int s = 0; s < KT / 16; ++s) {
    const int ch = 2 * s + lhalf;
    v_off[s] = lrow * V_ROW_BYTES + ((VCH == 16) ? (ch ^ (lrow & 15)) : (ch ^ swz8(lrow))) * 16;
  }
  // scores: S^T for the tile's 128 keys (four 32-key blocks), every K operand
  // used by all heads
  auto scores = [&](const bf16_t* kl, f32x16 (&sacc)[HPW][KB]) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[hh][kb][e] = 0.f;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(kl) + kb * 32 * K_ROW_BYTES + k_off[s]));
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
          sacc[hh][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[hh][s], sacc[hh][kb], 0, 0, 0);
      }
    }
    if constexpr (HPW == 1) {
      // keep eight K reads in flight ahead of the score MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < KB * DS - 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
  };
  // softmax: online softmax of tile t per head. Scores stay raw; the running
  // max m is kept in the scaled log2 domain and p = exp2(s * scale_log2 - m)
  // is one FMA plus one exp. m is only raised when a tile's max exceeds it by
  // more than 8 (p <= 2^8 meanwhile, exact once divided by the sum), so the O
  // rescale is skipped for the whole wavefront on most tiles.
  auto softmax = [&](int t, f32x16 (&sacc)[HPW][KB], bf16x8 (&pop)[HPW][PS]) {
    // tile may hold keys past some query (causal) or outside some frame (SEG)
    const bool edge = SEG ? (t * KT < in_lo || t * KT + KT > in_hi) : (t * KT + KT - 1) > q0;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = t * KT + kb * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
            if (key < my_lo || key >= my_hi) sacc[hh][kb][e] = -INFINITY;
          }
      }
      // The compiler does not see the max3 assembly as a reader of MFMA
      // results and so keeps no wait states for it; the last block's scores
      // (the only ones whose MFMAs may still be in flight) pass through nops
      // tied to them first (more than the 8-pass MFMA's 11 wait states).
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(sacc[hh][KB - 1]));
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
          m0 = max3(m0, sacc[hh][kb][e], sacc[hh][kb][e + 1]);
          m1 = max3(m1, sacc[hh][kb][e + 2], sacc[hh][kb][e + 3]);
        }
      float tmax = fmaxf(m0, m1);
      tmax = max_lane32(tmax) * scale_log2;
      float alpha = 1.f;
      if (tmax > m_run[hh] + 8.f) {
        alpha = __builtin_amdgcn_exp2f(m_run[hh] - tmax);  // 0 on the first tile
        m_run[hh] = tmax;
      }
      const float neg_m = -m_run[hh];
      // the row sum is taken over the bf16 probabilities the PV product uses
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[hh][kb][half * 8 + e], scale_log2, neg_m));
          const u32x4 pk = pack8(pv);
          ps0 = add_pair(pk[1], add_pair(pk[0], ps0));
          ps1 = add_pair(pk[3], add_pair(pk[2], ps1));
          pop[hh][kb * 2 + half] = __builtin_bit_cast(bf16x8, pk);
        }
      l_run[hh] = l_run[hh] * alpha + (ps0 + ps1);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[hh][b][e] *= alpha;
      }
    }
  };
  // pv: O^T += V^T P^T in 16-key steps, every V operand used by all heads
  auto pv = [&](const bf16_t* vl, bf16x8 (&pop)[HPW][PS]) {
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int s = 0; s < KT / 16; ++s) {
        const bf16x8 vop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(vl) + b * 32 * V_ROW_BYTES + v_off[s]));
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
          oacc[hh][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[hh][s], oacc[hh][b], 0, 0, 0);
      }
    }
    if constexpr (HPW == 1) {
      // eight V reads in flight ahead of the PV MFMAs as well (the
      // exponentials are left to the compiler's placement)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < DB * PS - 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
  };

  f32x16 sacc[HPW][KB];
  bf16x8 pop[HPW][PS];
  if constexpr (QN) {
    // the queries' cos/sin rows and the q gain, by LDS-DMA beside the first
    // tile: lane L of load instruction n fills 16-byte chunk L % CS_CH of
    // row (n WAVES + w) * (64 / CS_CH) + L / CS_CH with the logical chunk
    // the swizzle puts there
    static_assert(QW == 1 && DK == D && DS == D / 16, "the fused q norm: one query block, every head dim");
    constexpr int ROWS_PER_INSTR = 64 / CS_CH;
    constexpr int CS_INSTR = QB / ROWS_PER_INSTR;
#pragma unroll
    for (int n = 0; n * WAVES < CS_INSTR; ++n) {
      const int ins = n * WAVES + wave_u;
      if (ins < CS_INSTR) {
        const int r = ins * ROWS_PER_INSTR + lane / CS_CH, ph = lane % CS_CH;
        const int tok = min(q0 + r, seq - 1);
        global_load_lds16(reinterpret_cast<const char*>(rope),
                          static_cast<unsigned>(tok * (D / 2) * 8 + (ph ^ (r & 15)) * 16),
                          lds_addr(&cs_lds[0] + ins * 256));
      }
    }
    if (wave_u == WAVES - 1 && lane < D / 8)
      global_load_lds16(reinterpret_cast<const char*>(q_gain), 0u + lane * 16, lds_addr(&g_lds[0]));
  }
  issue_tile(t_first, 0);
  // The q values pass through empty assembly here, after the tiles' load
  // instructions, so that no arithmetic on them (and no wait for them) is
  // scheduled ahead of those instructions.
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int s = 0; s < DS; ++s) asm volatile("" : "+v"(qreg[hh][s]));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (QN) {
    // Per-head RMSNorm (gain q_gain, mean over the D dims: this lane's half
    // plus lane ^ 32's) and rotate-half rotary: dims d and d + D/2 are k-steps
    // s and s + DS/2 of the same lane, and their rotary slot j = d is the
    // table entry 16 s + 8 lhalf + e of the query's row.
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        float x[8];
        unpack8(__builtin_bit_cast(u32x4, qreg[hh][s]), x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      }
      ss = sum_lane32(ss);
      const float rinv = rsqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
      for (int s = 0; s < DS / 2; ++s) {
        float xl[8], xh[8], gl[8], gh[8], ol[8], oh[8];
        unpack8(__builtin_bit_cast(u32x4, qreg[hh][s]), xl);
        unpack8(__builtin_bit_cast(u32x4, qreg[hh][s + DS / 2]), xh);
        unpack8(*reinterpret_cast<const u32x4*>(&g_lds[s * 16 + lhalf * 8]), gl);
        unpack8(*reinterpret_cast<const u32x4*>(&g_lds[(s + DS / 2) * 16 + lhalf * 8]), gh);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // (cos, sin) of slots e = 2i, 2i + 1: logical chunk 8 s + 4 lhalf + i of row lrow
          const f32x4 cs = *reinterpret_cast<const f32x4*>(
              &cs_lds[lrow * D + ((8 * s + 4 * lhalf + i) ^ (lrow & 15)) * 4]);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 2 * i + u;
            const float c = cs[2 * u], sn = cs[2 * u + 1];
            const float yl = xl[e] * rinv * gl[e], yh = xh[e] * rinv * gh[e];
            // first half: y cos - y_partner sin; second half: y cos + y_partner sin
            ol[e] = yl * c - yh * sn;
            oh[e] = yh * c + yl * sn;
          }
        }
        qreg[hh][s] = __builtin_bit_cast(bf16x8, pack8(ol));
        qreg[hh][s + DS / 2] = __builtin_bit_cast(bf16x8, pack8(oh));
      }
    }
  }
  if (qi >= seq) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int s = 0; s < DS; ++s) qreg[hh][s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }

  for (int ti = 0; ti < n_tiles; ++ti) {
    const int t = t_first + ti;
    const int cur = ti & 1;
    if (ti + 1 < n_tiles) issue_tile(t + 1, cur ^ 1);
    scores(k_lds[cur], sacc);
    softmax(t, sacc, pop);
    pv(v_lds[cur], pop);
    // the next tile has landed, and every wavefront is done with this one
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- normalise and store: lane holds query lrow, d = 32b + 8(e/4) + 4 lhalf + e%4 ----
  float amx = 0.f;  // max |o| as stored (amax != NULL: FP8 quantisation of o)
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float l_tot = sum_lane32(l_run[hh]);
    if (qi < seq) {
      const float inv = 1.f / l_tot;
      bf16_t* dst = o + static_cast<size_t>(qi) * ldo + (h0 + hh) * dout + lhalf * 4;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          if (D != 128 || b * 32 + gq * 8 + lhalf * 4 < dout) {
            u32x2 pk;
            pk[0] = pack_bf16x2(oacc[hh][b][gq * 4 + 0] * inv, oacc[hh][b][gq * 4 + 1] * inv);
            pk[1] = pack_bf16x2(oacc[hh][b][gq * 4 + 2] * inv, oacc[hh][b][gq * 4 + 3] * inv);
            *reinterpret_cast<u32x2*>(dst + b * 32 + gq * 8) = pk;
            amx = fmaxf(amx, fmaxf(fmaxf(__uint_as_float((pk[0] << 16) & 0x7fffffffu),
                                         __uint_as_float(pk[0] & 0x7fff0000u)),
                                   fmaxf(__uint_as_float((pk[1] << 16) & 0x7fffffffu),
                                         __uint_as_float(pk[1] & 0x7fff0000u))));
          }
        }
    }
  }
  if (amax) {  // uniform; one partial maximum per workgroup
    // the K stages are free after the loop's last barrier
    float* red = reinterpret_cast<float*>(&k_lds[0][0]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amx = fmaxf(amx, __shfl_xor(amx, off, 64));
    if (lane == 0) red[wave] = amx;
    __syncthreads();
    if (tid == 0) {
      float m = red[0];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) m = fmaxf(m, red[w]);
      amax[blockIdx.x] = m;
    }
  }
}

template <int D, bool QN>
hipError_t launch_d(const bf16_t* q, int ldq, const bf16_t* q_gain, const float2* rope, float eps,
                    const bf16_t* k, const bf16_t* vt, bf16_t* o, int ldo, int seq, int n_heads,
                    int n_kv_heads, hipStream_t stream, float* amax) {
  const int G = n_heads / n_kv_heads;
  const int n_qb = (seq + QB - 1) / QB;
  const dim3 grid(n_qb * n_kv_heads);
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  switch (G) {
#define MHE_ATTN_CASE(GG, HH)                                                                      \
  case GG:                                                                                         \
    hipLaunchKernelGGL((attention_kernel<D, GG, HH, 1, false, QN, D>), grid, dim3(64 * (GG / HH)), \
                       0, stream, q, ldq, q_gain, rope, eps, k, vt, o, ldo, seq, n_heads,          \
                       n_kv_heads, scale_log2, D, nullptr, amax);                                  \
    break;
    MHE_ATTN_CASE(1, 1)
    MHE_ATTN_CASE(2, 1)
    MHE_ATTN_CASE(4, 1)
    MHE_ATTN_CASE(8, 1)
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

hipError_t launch_segment_attention(const bf16_t* q, const bf16_t* k, const bf16_t* vt, bf16_t* o,
                                    int ldo, int n, int heads, int head_dim,
                                    const PatchInfo* info, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (head_dim > 128 || head_dim % 4 != 0 || ldo < heads * head_dim || ldo % 4 != 0)
    return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(head_dim));
  if (head_dim <= 80) {
    // 8 query blocks (two wavefronts per SIMD), score MFMAs over 80 dims, PV
    // over 96
    const int n_qb = (n + QB * 8 - 1) / (QB * 8);
    hipLaunchKernelGGL((attention_kernel<128, 1, 1, 8, true, false, 96, 80>), dim3(n_qb * heads), dim3(64 * 8), 0,
                       stream, q, heads * 128, nullptr, nullptr, 0.f, k, vt, o, ldo, n, heads, heads, scale_log2,
                       head_dim, info, nullptr);
  } else if (head_dim <= 96) {
    // 8 query blocks (two wavefronts per SIMD), MFMAs over 96 dims
    const int n_qb = (n + QB * 8 - 1) / (QB * 8);
    hipLaunchKernelGGL((attention_kernel<128, 1, 1, 8, true, false, 96>), dim3(n_qb * heads), dim3(64 * 8), 0,
                       stream, q, heads * 128, nullptr, nullptr, 0.f, k, vt, o, ldo, n, heads, heads, scale_log2,
                       head_dim, info, nullptr);
  } else {
    // all 128 dims need more registers than two wavefronts per SIMD leave
    const int n_qb = (n + QB * 4 - 1) / (QB * 4);
    hipLaunchKernelGGL((attention_kernel<128, 1, 1, 4, true, false, 128>), dim3(n_qb * heads), dim3(64 * 4), 0,
                       stream, q, heads * 128, nullptr, nullptr, 0.f, k, vt, o, ldo, n, heads, heads, scale_log2,
                       head_dim, info, nullptr);
  }
  return hipGetLastError();
}

int attention_amax_parts(int seq, int n_kv_heads) { return (seq + QB - 1) / QB * n_kv_heads; }

hipError_t launch_attention(const bf16_t* q, const bf16_t* k, const bf16_t* vt, bf16_t* o,
                            int ldo, int seq, int n_heads, int n_kv_heads, int head_dim,
                            hipStream_t stream, float* amax) {
  if (seq <= 0) return hipSuccess;
  if (ldo < n_heads * head_dim || ldo % 4 != 0) return hipErrorInvalidValue;
  const int ldq = n_heads * head_dim;
  if (head_dim == 128)
    return launch_d<128, false>(q, ldq, nullptr, nullptr, 0.f, k, vt, o, ldo, seq, n_heads, n_kv_heads, stream, amax);
  if (head_dim == 64)
    return launch_d<64, false>(q, ldq, nullptr, nullptr, 0.f, k, vt, o, ldo, seq, n_heads, n_kv_heads, stream, amax);
  return hipErrorInvalidValue;
}

hipError_t launch_attention_qnorm(const bf16_t* q_raw, int ldq, const bf16_t* q_gain, const float2* rope,
                                  float eps, const bf16_t* k, const bf16_t* vt, bf16_t* o, int ldo, int seq,
                                  int n_heads, int n_kv_heads, int head_dim, hipStream_t stream, float* amax) {
  if (seq <= 0) return hipSuccess;
  if (ldo < n_heads * head_dim || ldo % 4 != 0 || ldq < n_heads * head_dim || ldq % 8 != 0)
    return hipErrorInvalidValue;
  if (head_dim == 128)
    return launch_d<128, true>(q_raw, ldq, q_gain, rope, eps, k, vt, o, ldo, seq, n_heads, n_kv_heads, stream, amax);
  if (head_dim == 64)
    return launch_d<64, true>(q_raw, ldq, q_gain, rope, eps, k, vt, o, ldo, seq, n_heads, n_kv_heads, stream, amax);
  return hipErrorInvalidValue;
}

}  // namespace mhe
