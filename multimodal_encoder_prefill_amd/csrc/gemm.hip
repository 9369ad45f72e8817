// BF16 GEMM family on gfx950 MFMA: C[m, n] = sum_k A[m, k] * B[n, k].
//
// Every linear layer of the decoder is of this form (the F.linear calls of the
// H3 encoder page: q/k/v, o, gate/up and down projections, y = x W^T with W
// stored [out, in]), so both operands are K-contiguous. Accumulation is fp32
// and the result is rounded to bf16 once, after the epilogue:
//   kStore    C = A B^T                       (q | k | v projections)
//   kResidual C = R + A B^T                   (o and down projections plus the
//                                              decoder layer's residual add)
//   kSwiGLU   C = silu(A Bg^T) * (A Bu^T)     (gate/up projections and the
//                                              MLP activation, MiniMaxH3Qwen3VLTextMLP)
//   kBias, kBiasResidual, kBiasGeluTanh, kBiasGeluErf
//             C = A B^T + bias, then + R or GELU (the biased linears of the
//             vision tower: MiniMaxH3Qwen3VLVisionAttention / VisionMLP /
//             VisionPatchMerger; the MLP's GELU is the tanh form, the
//             merger's the erf form)
//
// Tiling: a 256 (m) x 64 NB (n) output tile per workgroup of 4 wavefronts.
// bf16 (gemm16_kernel): 16x16x32 MFMAs; NB = 5 (256 x 320) for the decoder
// linears where whole waves of tiles fill the chip, NB = 4 (256 x 256, with
// partial n-tiles and k-splits) otherwise. The 320-wide tile reads 10% fewer
// LDS bytes per MFMA and makes 4096 x 5120, 4096 x 10240 and 4096 x 2 x 25600
// outputs exact multiples of 256 tiles. FP8 (gemm_f8w_kernel): the same two
// widths on 32x32x64 MFMAs. The weight rows are the MFMA "A" operand and the
// activation rows the "B" operand, so every lane ends up with 4 consecutive
// output columns.
//
// K advances 128 row bytes at a time (64 bf16 or 128 FP8 elements) through
// two LDS stages of (256 + 64 NB) rows of 128 bytes (64 or 72 KB each), the
// 16-byte chunks of each row XOR-swizzled so that the ds_read_b128 operand
// fetches hit distinct banks. Tiles go straight from global memory into LDS
// (global_load_lds_dwordx4, a wave-uniform base per 32-row block and one
// 32-bit offset per lane); lanes past the last row of M or N load that row
// again. One workgroup barrier per k-step, placed where the MFMAs still to
// come have their operands in registers, so that they hide the barrier and
// the first operand reads of the next k-step. The LDS reads of operands go
// out one at a time between the MFMAs (a burst of all of them, from all
// four wavefronts at once, left the MFMAs waiting on the LDS).
//
// Workgroups are remapped so that each XCD (workgroups are dealt round-robin
// over the 8 XCDs) receives a contiguous run of tiles, ordered in groups of m
// tiles so tiles running together on one XCD share A and B panels in its L2.
//
// The epilogue has no per-row branch: C and the residual are addressed
// through buffer resources that end at row M, so the hardware drops stores
// to (and reads zeros from) rows past it; k-split units are a separate
// instantiation that only writes fp32 partials. (Branches there made the
// compiler copy every accumulator out of the AGPRs up front and spill them.)
// Outputs pass through LDS, which is free once the pipeline ends, and leave
// as whole row segments in 16-byte chunks instead of 8 bytes per row and
// lane.
#include <atomic>
#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;  // n extent of the NB = 4 tile (and of the FP8 kernels)
constexpr int kThreads = 256;
constexpr int kGroupM = 8;  // m tiles per ordering group
constexpr int kXcds = 8;

constexpr int BK = 64;  // bf16 k elements per pipeline step (one 128-byte row piece)

typedef __attribute__((ext_vector_type(8))) int i32x8;

struct GemmArgs {
  const void* a;        // bf16 or (FP8 kernels) E4M3 bytes
  const void* bptr[3];
  int brows[3];
  // FP8 kernels: per-tensor scales (device; element 0 of each is the scale)
  // of A and of the B segments, applied to the fp32 sums before the epilogue
  const float* scale_a;
  const float* scale_b[3];
  bf16_t* c;
  const bf16_t* r;
  const bf16_t* bias;
  int m, n, k;
  int lda, ldb;  // row strides (elements) of A and of every B segment
  int ldc;       // row stride of C and of the residual
  int tiles_m, tiles_n;
  // work units of this launch: tiles [tile_begin, tile_begin + units / ksplit),
  // each split into ksplit k-ranges of kt_per_split k-steps. With ksplit > 1 the
  // raw fp32 accumulators go to partial[unit] ([256][256] floats per unit).
  int tile_begin, units, ksplit, kt_per_split;
  float* partial;
  // FP8 kSwiGLU, optional: max |C| (as stored) of each workgroup's outputs, at
  // amax[unit] (whole tiles) or amax[split tile * 64 + row group] (the
  // split-K reduction)
  float* amax;
};

// max |v| over the four bf16 values of a packed pair of words
__device__ __forceinline__ float abs_max4(const u32x2& pk) {
  return fmaxf(fmaxf(__uint_as_float((pk[0] << 16) & 0x7fffffffu), __uint_as_float(pk[0] & 0x7fff0000u)),
               fmaxf(__uint_as_float((pk[1] << 16) & 0x7fffffffu), __uint_as_float(pk[1] & 0x7fff0000u)));
}

// Maximum over a workgroup of 256 threads (red: 4 floats of LDS, not in use).
__device__ __forceinline__ float workgroup_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Output tile (m, n) of logical tile t: groups of kGroupM m-tiles, n-major
// inside a group, so consecutive tiles share B panels and A panels.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group_size = kGroupM * tiles_n;
  const int group = t / group_size;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = t - group * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Chunk swizzle of a 128-byte LDS operand row (8 chunks of 16 bytes): rows
// r..r+7 and r..r+15 map one logical chunk to distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Wait until at most N vector-memory operations of this wavefront are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// f(std::integral_constant<int, i>()) for i = B .. E-1, in order: loop
// indices that select registers (accumulator blocks, operand slots) are
// constants from the start, not only after unrolling.
template <int B, class F, int... I>
__device__ __forceinline__ void static_for_seq(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, B + I>()), ...);
}
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq<B>(f, std::make_integer_sequence<int, E - B>());
}
// c += W X^T on v_mfma_f32_16x16x32_bf16, the accumulator in AGPRs or VGPRs
template <bool AGPR>
__device__ __forceinline__ void mfma16(f32x4& c, const bf16x8& w, const bf16x8& x) {
  if constexpr (AGPR)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(w), "v"(x));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(w), "v"(x));
}
// Wait states between the MFMA writes of eight accumulator blocks (AGPRs or
// VGPRs) and their first VALU read: LONG covers a 4-pass MFMA issued just
// before, the short form follows a long one.
template <bool AGPR, bool LONG>
__device__ __forceinline__ void mfma_result_wait(f32x4 (&c)[8]) {
  if constexpr (AGPR && LONG)
    asm volatile("s_nop 7\n\ts_nop 7" : "+a"(c[0]), "+a"(c[1]), "+a"(c[2]), "+a"(c[3]), "+a"(c[4]), "+a"(c[5]),
                 "+a"(c[6]), "+a"(c[7]));
  else if constexpr (AGPR)
    asm volatile("s_nop 1" : "+a"(c[0]), "+a"(c[1]), "+a"(c[2]), "+a"(c[3]), "+a"(c[4]), "+a"(c[5]), "+a"(c[6]),
                 "+a"(c[7]));
  else if constexpr (LONG)
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(c[4]), "+v"(c[5]),
                 "+v"(c[6]), "+v"(c[7]));
  else
    asm volatile("s_nop 1" : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(c[4]), "+v"(c[5]), "+v"(c[6]),
                 "+v"(c[7]));
}

// accumulator block (IB, JB) of gemm16_kernel: weight blocks 0-7 in a, 8-9 in v
template <int IB, int JB, int V>
__device__ __forceinline__ f32x4& acc16(f32x4 (&a)[8][8], f32x4 (&v)[V][8]) {
  if constexpr (IB < 8)
    return a[IB][JB];
  else
    return v[IB - 8][JB];
}

// c += W X^T on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, both block
// scales `scale`), the accumulator in AGPRs or VGPRs
template <bool AGPR>
__device__ __forceinline__ void mfma_f8(f32x16& c, const i32x8& w, const i32x8& x, int scale) {
  if constexpr (AGPR)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+a"(c) : "v"(w), "v"(x), "v"(scale));
  else
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+v"(c) : "v"(w), "v"(x), "v"(scale));
}
// accumulator block (IB, JB) of gemm_f8w_kernel: weight blocks 0-3 in a, 4 in v
template <int IB, int JB>
__device__ __forceinline__ f32x16& acc_f8(f32x16 (&a)[4][4], f32x16 (&v)[4]) {
  if constexpr (IB < 4)
    return a[IB][JB];
  else
    return v[JB];
}

// 32-bit LDS address of a pointer into the workgroup's LDS
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<size_t>((__attribute__((address_space(3))) const void*)p));
}

// global_load_lds_dwordx4 in its scalar-base form: lane L copies the 16
// bytes at base + off (base wave-uniform, off the lane's) to LDS address
// lds + 16 L. (The compiler builtin always forms a 64-bit address per lane.)
// M0 carries the LDS address and needs one wait state before the load. The
// load counts in vmcnt like any other; callers wait for it explicitly.
// clang warns that M0 is a reserved register it may not preserve across the
// statement: nothing in this file's device code reads M0 except these loads
// (the generated code holds no other M0 access), so the warning is silenced.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void global_load_lds16(const char* base, unsigned off, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier that orders LDS traffic only: it waits for this
// wavefront's LDS operations but leaves global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr bool epi_bias(int e) { return e >= static_cast<int>(Epilogue::kBias); }

constexpr bool epi_residual(int e) {
  return e == static_cast<int>(Epilogue::kResidual) || e == static_cast<int>(Epilogue::kBiasResidual);
}

// silu(g) * u = g / (1 + e^-g) * u, the quotient through the hardware
// reciprocal (v_rcp_f32, 1 ulp) instead of the IEEE division sequence: the
// result is rounded to bf16 anyway, and the epilogue runs once per tile.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// GELU, tanh form: x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), with
// tanh(y) = 1 - 2 / (1 + e^(2y)) (saturates correctly at both ends).
__device__ __forceinline__ float gelu_tanh(float x) {
  const float y = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  return 0.5f * x * (2.f - 2.f * __builtin_amdgcn_rcpf(1.f + __expf(2.f * y)));
}
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.f + erff(x * 0.7071067811865476f));
}

// FP8 scale of the products in output column n: scale_a times the scale of
// the weight segment that holds row n (segments are multiples of 32 rows, so
// four consecutive columns share it).
__device__ __forceinline__ float f8_scale(const GemmArgs& args, int n) {
  const float sb = n < args.brows[0] ? args.scale_b[0][0]
                   : n < args.brows[0] + args.brows[1] ? args.scale_b[1][0]
                                                       : args.scale_b[2][0];
  return args.scale_a[0] * sb;
}

// Non-SwiGLU epilogue of four consecutive outputs (bv, rv: their bias and
// residual, loaded by the caller), rounded to bf16 once.
template <int EPI>
__device__ __forceinline__ u32x2 finish4(float* o, u32x2 bv, u32x2 rv) {
  if constexpr (epi_bias(EPI)) {
    o[0] += __uint_as_float(bv[0] << 16);
    o[1] += __uint_as_float(bv[0] & 0xffff0000u);
    o[2] += __uint_as_float(bv[1] << 16);
    o[3] += __uint_as_float(bv[1] & 0xffff0000u);
  }
  if constexpr (epi_residual(EPI)) {
    o[0] += __uint_as_float(rv[0] << 16);
    o[1] += __uint_as_float(rv[0] & 0xffff0000u);
    o[2] += __uint_as_float(rv[1] << 16);
    o[3] += __uint_as_float(rv[1] & 0xffff0000u);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (EPI == static_cast<int>(Epilogue::kBiasGeluTanh)) o[e] = gelu_tanh(o[e]);
    if constexpr (EPI == static_cast<int>(Epilogue::kBiasGeluErf)) o[e] = gelu_erf(o[e]);
  }
  u32x2 pk;
  pk[0] = pack_bf16x2(o[0], o[1]);
  pk[1] = pack_bf16x2(o[2], o[3]);
  return pk;
}
// the same for columns n..n+3, loading their bias
template <int EPI>
__device__ __forceinline__ u32x2 finish4(float* o, const GemmArgs& args, int n, u32x2 rv) {
  const u32x2 bv = epi_bias(EPI) ? *reinterpret_cast<const u32x2*>(args.bias + n) : u32x2{0, 0};
  return finish4<EPI>(o, bv, rv);
}

// The FP8 GEMMs: operands are E4M3 bytes in the same 128-byte LDS rows as
// the bf16 kernels', a pipeline step covers 128 k in two substeps of 64 k on
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales), and the sums are
// multiplied by scale_a * scale_b before the epilogue. NB = 5 (256 x 320)
// for the decoder linears where whole waves of such tiles fill the chip (as
// for bf16), NB = 4 (256 x 256, partial n-tiles and k-splits) otherwise:
// each wavefront owns 128 tokens x 32 NB weight rows as 4 x NB blocks of
// 32 x 32, 4 NB MFMAs per substep (16 blocks in the 256 AGPRs, the fifth
// weight block's 4 in VGPRs). The operands do not fit double-buffered (32
// bytes per lane each), so they stream as in gemm16_kernel: a substep's
// four activation operands stay in registers through it, the weight
// operands pass through a ring of NB, each read two blocks (8 MFMAs) ahead,
// and the one barrier per k-step sits 8 MFMAs before its end, after the
// last read of the stage. (The 16x16x128 FP8 form would save nothing: with
// 32-byte operands per lane it moves as many register bytes per flop as
// 32x32x64.)
//
// A lane reads 32 bytes of its row (row 32 blk + (lane & 31)): chunks
// 4 s + 2 (lane >> 5) and the next one of substep s (any assignment of k to
// the operand bytes gives the same sum as long as both operands use it).
// Accumulator block (ib, jb): weight rows 32 ib + 8 g + 4 (lane >> 5) + e,
// token 32 jb + (lane & 31), for e < 4 and the four groups g. SwiGLU: the 8-row
// groups of each 32-row weight block alternate gate and up rows of the same 8
// output columns, so groups g and g + 1 of a lane are the two factors of the
// same outputs.
//
// SPLIT: the unit is one k-range of a split tile; the raw fp32 sums (before
// the scales) go to args.partial, [m_local][virtual n], for
// splitk_reduce_kernel. (A separate instantiation, so that each kernel has
// one epilogue: with both in one kernel the compiler read every accumulator
// out ahead of the branch and spilled them.)
template <int EPI, int NB, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void gemm_f8w_kernel(const GemmArgs args) {
  constexpr bool kSwi = EPI == static_cast<int>(Epilogue::kSwiGLU);
  static_assert(EPI <= static_cast<int>(Epilogue::kSwiGLU), "FP8 epilogues: store, residual, SwiGLU");
  static_assert(NB == 4 || NB == 5, "tile width");
  constexpr int BNT = 64 * NB;
  constexpr int kATile = BM * BK, kBTile = BNT * BK;  // one stage, in bf16 units of the byte rows
  constexpr int kRowBytes = BK * 2, kChunks = BK / 8;
  constexpr int kRowsPerBlk = 4096 / kRowBytes;
  constexpr int kBlksA = BM / kRowsPerBlk, kBlksB = BNT / kRowsPerBlk;
  constexpr int kLoads = kBlksA + kBlksB;  // 16 or 18
  constexpr int kSub = 4 * NB;             // MFMAs per substep
  constexpr int kSlots = 2 * kSub;         // MFMAs per k-step
  constexpr int kBar = kSlots - 8;         // the barrier's slot
  // loads [0, kLC) of k-step kt + 2 go out after the barrier of kt, the rest
  // over the first MFMAs of kt + 1, one per 2 MFMAs
  constexpr int kLC = 8;
  constexpr int kWarm = 4;
  static_assert(BK == 64 && 2 * (kLoads - kLC) <= kSub, "pipeline shape");

  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  bf16_t* As = smem;
  bf16_t* Bs = smem + 2 * kATile;

  const int M = args.m, N = args.n, K = args.k;
  const int lda = args.lda, ldb = args.ldb;  // in bytes (one byte per element)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  const int total = args.units;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int q = total / kXcds, rmd = total % kXcds;
  const int unit = xcd * q + min(xcd, rmd) + bid / kXcds;
  int tile_m, tile_n;
  // (whole-tile launches have ksplit 1: constants, not divisions)
  const int ksplit = SPLIT ? args.ksplit : 1;
  tile_coords(args.tile_begin + unit / ksplit, args.tiles_m, args.tiles_n, tile_m, tile_n);
  const int m0 = tile_m * BM;
  const int kt_begin = SPLIT ? (unit % ksplit) * args.kt_per_split : 0;
  const int nk = SPLIT ? min(kt_begin + args.kt_per_split, K / 128) - kt_begin : K / 128;  // k-steps

  auto b_block_base = [&](int i, int& avail) -> const char* {
    const void* base;
    int v;
    if constexpr (kSwi) {
      // block i: wave half i / NB, block i % NB of it; the 8-row group of
      // wavefront w is gate rows for even w, up rows for odd w, output
      // columns j .. j+7
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      const int j = tile_n * (BNT / 2) + (i / NB) * (16 * NB) + (i % NB) * 16 + (w >> 1) * 8;
      base = (w & 1) ? args.bptr[1] : args.bptr[0];
      v = min(j, N - 1);
      avail = N - j;
    } else {
      const int row = tile_n * BNT + kRowsPerBlk * i;
      const int rr = min(row, N - 1);
      if (rr < args.brows[0]) {
        base = args.bptr[0];
        v = rr;
        avail = args.brows[0] - row;
      } else if (rr < args.brows[0] + args.brows[1]) {
        base = args.bptr[1];
        v = rr - args.brows[0];
        avail = args.brows[0] + args.brows[1] - row;
      } else {
        base = args.bptr[2];
        v = rr - args.brows[0] - args.brows[1];
        avail = N - row;
      }
    }
    return static_cast<const char*>(base) + static_cast<size_t>(v) * ldb;
  };

  const int dma_row = wave * (1024 / kRowBytes) + lane / kChunks;
  const int dma_chunk = ((lane % kChunks) ^ swz(dma_row)) * 16;
  const int b_lane_row = kSwi ? lane / kChunks : dma_row;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  bf16_t* const warm_dst = smem + 2 * kATile + 2 * kBTile + wave_u * 512;
  const char* a_ptr[kBlksA];
  const char* b_ptr[kBlksB];
  unsigned a_off[kBlksA], b_off[kBlksB];
#pragma unroll
  for (int i = 0; i < kBlksA; ++i) {
    const int r = m0 + kRowsPerBlk * i;
    a_ptr[i] = static_cast<const char*>(args.a) + static_cast<size_t>(min(r, M - 1)) * lda;
    a_off[i] = min(dma_row, max(M - r, 1) - 1) * lda + dma_chunk;
  }
#pragma unroll
  for (int i = 0; i < kBlksB; ++i) {
    int avail;
    b_ptr[i] = b_block_base(i, avail);
    b_off[i] = min(b_lane_row, max(avail, 1) - 1) * ldb + dma_chunk;
  }
  int warm_avail;
  const char* const warm_ptr = b_block_base((tile_m & 7) * (32 / kRowsPerBlk), warm_avail);
  const unsigned warm_off = min(b_lane_row, max(warm_avail, 1) - 1) * ldb + (lane % kChunks) * 16;

  auto koff = [&](int kt) { return static_cast<size_t>(kt_begin + min(kt, nk - 1)) * kRowBytes; };
  auto issue_load = [&](int kt, int stage, int l) {
    const bool isb = l >= 2 * kBlksA || (l & 1);
    const int i = l >= 2 * kBlksA ? l - kBlksA : l >> 1;
    bf16_t* dst = (isb ? Bs + stage * kBTile : As + stage * kATile) + wave_u * 512 + i * kRowsPerBlk * BK;
    global_load_lds16((isb ? b_ptr[i] : a_ptr[i]) + koff(kt), isb ? b_off[i] : a_off[i], lds_addr(dst));
  };
  auto issue_warm = [&](int kt) { global_load_lds16(warm_ptr + koff(kt), warm_off, lds_addr(warm_dst)); };

  // ---- LDS -> registers: 32 bytes of row 32 blk + lrow per operand ----
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int lswz = swz(lrow);
  const int x_base = (wm * 128 + lrow) * BK;
  const int w_base = (wn * (BNT / 2) + lrow) * BK;
  const int c8[2][2] = {{((2 * lhalf) ^ lswz) * 8, ((2 * lhalf + 1) ^ lswz) * 8},
                        {((4 + 2 * lhalf) ^ lswz) * 8, ((4 + 2 * lhalf + 1) ^ lswz) * 8}};
  auto rd = [&](const bf16_t* p, int s) {
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(p + c8[s][0]);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(p + c8[s][1]);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto rd_x = [&](int stage, int s, int jb) { return rd(As + stage * kATile + x_base + jb * 32 * BK, s); };
  auto rd_w = [&](int stage, int s, int ib) { return rd(Bs + stage * kBTile + w_base + ib * 32 * BK, s); };

  f32x16 acc[4][4];  // weight blocks 0-3 (AGPRs)
  f32x16 accv[4];    // weight block 4 (VGPRs; NB = 5)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    if constexpr (NB == 5)
#pragma unroll
      for (int e = 0; e < 16; ++e) accv[i][e] = 0.f;
  }
  // the zeroing writes, then the first MFMA reads of the same registers
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("s_nop 4" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));
  if constexpr (NB == 5) asm volatile("s_nop 4" : "+v"(accv[0]), "+v"(accv[1]), "+v"(accv[2]), "+v"(accv[3]));
  const int unit_scale = 127;  // E8M0 block scale 2^0, in every lane
  i32x8 xo[2][4];  // activation operands of substeps 0 and 1
  i32x8 wo[NB];    // weight operands: the 2 NB of a k-step (NB s + ib) in a ring of NB
  using Live = std::true_type;
  using Dead = std::false_type;

  auto step = [&](int kt, auto LIVE1, auto LIVE2) {
    const int st = kt & 1;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, kBar>([&](auto G) {
      constexpr int g = decltype(G)::value;
      constexpr int s = g / kSub, ib = (g % kSub) / 4, jb = g % 4;
      mfma_f8<(ib < 4)>(acc_f8<ib, jb>(acc, accv), wo[ib], xo[s][jb], unit_scale);
      // weight operand NB s' + i (i >= 2 of substep 0, all of substep 1)
      // after slot 4 (NB s' + i) - 7, two blocks before its first use
      if constexpr (g % 4 == 1) {
        constexpr int idx = (g + 7) / 4;
        if constexpr (idx < 2 * NB) wo[idx % NB] = rd_w(st, idx / NB, idx % NB);
      }
      // substep 1's activation operands after slots 8, 10, 12, 14
      if constexpr (g >= 8 && g < 16 && g % 2 == 0) xo[1][(g - 8) / 2] = rd_x(st, 1, (g - 8) / 2);
      // loads [kLC, 18) of k-step kt+1 after slots 0, 2, 4, ..
      if constexpr (decltype(LIVE1)::value && g % 2 == 0 && g / 2 < kLoads - kLC)
        issue_load(kt + 1, st ^ 1, kLC + g / 2);
      if constexpr (g == kSub) issue_warm(kt + kWarm);
      __builtin_amdgcn_sched_barrier(0);
    });
    // k-step kt+1 is complete in LDS (only the warm-up load may still be in
    // flight) and no wavefront reads stage st any more
    wait_vmcnt<1>();
    lds_barrier();
    static_for<kBar, kSlots>([&](auto G) {
      constexpr int g = decltype(G)::value;
      constexpr int ib = (g - kSub) / 4, jb = g % 4;
      mfma_f8<(ib < 4)>(acc_f8<ib, jb>(acc, accv), wo[ib], xo[1][jb], unit_scale);
      // the first operands of k-step kt+1 (activations 0-3, weights 0 and 1
      // of its substep 0) and loads [0, kLC) of k-step kt+2
      constexpr int r = g - kBar;
      if constexpr (r == 0 || r == 2 || r == 3 || r == 4) xo[0][r == 0 ? 0 : r - 1] = rd_x(st ^ 1, 0, r == 0 ? 0 : r - 1);
      if constexpr (r == 1) wo[0] = rd_w(st ^ 1, 0, 0);
      if constexpr (r == 5) wo[1] = rd_w(st ^ 1, 0, 1);
      if constexpr (decltype(LIVE2)::value && r < kLC) issue_load(kt + 2, st, r);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  if (nk > 0) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) issue_load(0, 0, l);
#pragma unroll
    for (int l = 0; l < kLC; ++l) issue_load(1, 1, l);
#pragma unroll
    for (int kt = 1; kt < kWarm; ++kt) issue_warm(kt);
    wait_vmcnt<kLC + kWarm - 1>();
    lds_barrier();
    xo[0][0] = rd_x(0, 0, 0);
    wo[0] = rd_w(0, 0, 0);
#pragma unroll
    for (int j = 1; j < 4; ++j) xo[0][j] = rd_x(0, 0, j);
    wo[1] = rd_w(0, 0, 1);
    int kt = 0;
    for (; kt < nk - 2; ++kt) step(kt, Live(), Live());
    if (kt < nk - 1) step(kt++, Live(), Dead());
    step(kt, Dead(), Dead());
    wait_vmcnt<0>();
    lds_barrier();
  }

  // MFMA writes, then VALU reads: 32 wait states before the blocks written
  // last (the last weight block), more before the rest
  if constexpr (NB == 5)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(accv[0]), "+v"(accv[1]), "+v"(accv[2]), "+v"(accv[3]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("s_nop 1" : "+a"(acc[3 - i][0]), "+a"(acc[3 - i][1]), "+a"(acc[3 - i][2]), "+a"(acc[3 - i][3]));

  // ---- split-K unit: raw accumulators to the unit's partial tile ----
  if constexpr (SPLIT) {
    float* dst = args.partial + static_cast<size_t>(unit) * BM * BNT;
    static_for<0, 4 * NB>([&](auto Q) {
      constexpr int jb = decltype(Q)::value / NB, ib = decltype(Q)::value % NB;
      const f32x16& a = acc_f8<ib, jb>(acc, accv);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a[4 * gq + e];
        *reinterpret_cast<f32x4*>(dst + (wm * 128 + jb * 32 + lrow) * BNT + wn * (BNT / 2) + ib * 32 + 8 * gq +
                                  4 * lhalf) = v;
      }
    });
    return;
  }

  // ---- epilogue, through a per-wavefront LDS region (as gemm16_kernel) ----
  const size_t rbytes = static_cast<size_t>(M - m0) * args.ldc * sizeof(bf16_t);
  const int nbytes = static_cast<int>(rbytes < 0x7fffffffu ? rbytes : 0x7fffffffu);
  const size_t first = static_cast<size_t>(m0) * args.ldc;
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(args.c + first, (short)0, nbytes, 0x00020000);
  const int ldc_b = args.ldc * static_cast<int>(sizeof(bf16_t));
  // Weight blocks past N (a partial n-tile of the 256-wide form; N is a
  // multiple of 32) are skipped by wave-uniform tests, their 16-byte chunks
  // by a lane test in the stores.
  if constexpr (kSwi) {
    // 128 x 16 NB outputs per wavefront in two halves of 64 tokens; staging
    // rows of 16 NB + 8 bf16 (144 or 176 bytes)
    constexpr int kCols = 16 * NB, kStg = kCols + 8, kRowChunks = kCols / 8;
    bf16_t* const stg = smem + wave_u * 64 * kStg;
    const int col0 = tile_n * (BNT / 2) + wn * kCols;
    const float sg = args.scale_a[0] * args.scale_b[0][0];
    const float su = args.scale_a[0] * args.scale_b[1][0];
    float amx = 0.f;  // max |C| as stored
    static_for<0, 2>([&](auto H) {
      constexpr int h = decltype(H)::value;
      static_for<0, 2 * NB>([&](auto Q) {
        constexpr int jj = decltype(Q)::value / NB, ib = decltype(Q)::value % NB;
        if (NB == 5 || col0 + ib * 16 < N) {
          const f32x16& a = acc_f8<ib, 2 * h + jj>(acc, accv);
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = silu_mul(a[8 * gp + e] * sg, a[8 * gp + 4 + e] * su);
            u32x2 pk;
            pk[0] = pack_bf16x2(o[0], o[1]);
            pk[1] = pack_bf16x2(o[2], o[3]);
            amx = fmaxf(amx, abs_max4(pk));
            *reinterpret_cast<u32x2*>(stg + (jj * 32 + lrow) * kStg + ib * 16 + gp * 8 + 4 * lhalf) = pk;
          }
        }
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < kRowChunks; ++it) {
        const int c = it * 64 + lane, r = c / kRowChunks, qq = c - r * kRowChunks;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * kStg + qq * 8);
        if (NB == 5 || col0 + qq * 8 < N)
          __builtin_amdgcn_raw_buffer_store_b128(v, c_rsrc, (wm * 128 + h * 64 + r) * ldc_b + (col0 + qq * 8) * 2, 0,
                                                 0);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    });
    if (args.amax) {  // uniform; past the four staging regions
      const float v = workgroup_max(amx, reinterpret_cast<float*>(smem + 4 * 64 * kStg));
      if (tid == 0) args.amax[unit] = v;
    }
  } else {
    // 128 x 32 NB outputs per wavefront in two halves of 64 tokens; staging
    // rows of 32 NB + 8 bf16 (272 or 336 bytes); a half's residual values
    // loaded in the accumulator layout, all before its first add (a load past
    // N reads other columns of the buffer, or zeros past its end, for an
    // output that is not stored)
    constexpr int kCols = 32 * NB, kStg = kCols + 8, kRowChunks = kCols / 8;
    bf16_t* const stg = smem + wave_u * 64 * kStg;
    const int col0 = tile_n * BNT + wn * (BNT / 2);
    const __amdgpu_buffer_rsrc_t r_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        epi_residual(EPI) ? const_cast<bf16_t*>(args.r) + first : args.c + first, (short)0, nbytes, 0x00020000);
    float sc[NB];  // FP8 scale of each weight block's columns (segments are multiples of 32 rows)
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) sc[ib] = NB == 5 || col0 + ib * 32 < N ? f8_scale(args, col0 + ib * 32) : 0.f;
    static_for<0, 2>([&](auto H) {
      constexpr int h = decltype(H)::value;
      u32x2 rv[2][NB][4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            rv[jj][ib][gq] = epi_residual(EPI)
                                 ? __builtin_amdgcn_raw_buffer_load_b64(
                                       r_rsrc,
                                       (wm * 128 + (2 * h + jj) * 32 + lrow) * ldc_b +
                                           (col0 + ib * 32 + 8 * gq + 4 * lhalf) * 2,
                                       0, 0)
                                 : u32x2{0, 0};
      static_for<0, 2 * NB>([&](auto Q) {
        constexpr int jj = decltype(Q)::value / NB, ib = decltype(Q)::value % NB;
        if (NB == 5 || col0 + ib * 32 < N) {
          const f32x16& a = acc_f8<ib, 2 * h + jj>(acc, accv);
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = a[4 * gq + e] * sc[ib];
            *reinterpret_cast<u32x2*>(stg + (jj * 32 + lrow) * kStg + ib * 32 + 8 * gq + 4 * lhalf) =
                finish4<EPI>(o, u32x2{0, 0}, rv[jj][ib][gq]);
          }
        }
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < kRowChunks; ++it) {
        const int c = it * 64 + lane, r = c / kRowChunks, qq = c - r * kRowChunks;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * kStg + qq * 8);
        if (NB == 5 || col0 + qq * 8 < N)
          __builtin_amdgcn_raw_buffer_store_b128(v, c_rsrc, (wm * 128 + h * 64 + r) * ldc_b + (col0 + qq * 8) * 2, 0,
                                                 0);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    });
  }
}

// The bf16 GEMMs on v_mfma_f32_16x16x32_bf16: the 256 x 320 tile (NB = 5)
// and the 256 x 256 one (NB = 4). Same LDS ring, LDS-DMA loads, swizzle,
// warm-up and tile order as gemm_f8w_kernel; each wavefront owns 128 tokens x
// 32 NB weight rows as 8 x WB blocks of 16 x 16 (WB = 2 NB). Per MFMA the
// 16x16x32 form reads and writes a quarter of the accumulator registers of
// the 32x32x16 form for half the products, so the register file moves 20%
// fewer bytes per flop; under the chip's power limit a register-only loop of
// it runs ~10% faster.
//
// A k-step (64 k) is two substeps of 32 k, 8 WB MFMAs each: block (ib, jb)
// multiplies weight rows 16 ib.. by tokens 16 jb.. . A lane holds the weight
// operand of row 16 ib + (lane & 15), 8 k of the substep's 32, and the
// activation operand of token 16 jb + (lane & 15) at the same k, and ends
// with outputs
// (weight row 16 ib + 4 (lane >> 4) + e, token 16 jb + (lane & 15)), e < 4:
// four consecutive output columns of one token. The eight activation
// operands of a substep stay in registers through it; the weight operands
// stream through a ring of four registers, each read two blocks (16 MFMAs)
// before its first use. The one barrier per k-step sits 16 MFMAs before its
// end, after the last read of the stage: those MFMAs (the last two weight
// blocks) cover the barrier and the reads of the next k-step's first
// operands.
//
// All MFMAs are inline assembly: blocks 0-7 accumulate in the 256 AGPRs,
// blocks 8-9 (NB = 5) in VGPRs. (Through the builtin the compiler permuted
// the 64 AGPR accumulators between loop iterations with register moves.)
// The compiler does not see these statements as MFMAs, so the VALU/MFMA
// hazards on the accumulators are covered by explicit waits after zeroing
// them and before the epilogue reads them.
//
// SwiGLU: each 32-row weight block holds 16 gate rows and then the 16 up
// rows of the same output columns, so weight blocks 2p and 2p + 1 of a lane
// are the two factors of the same outputs.
//
// SPLIT: the unit is one k-range of a split tile; the raw fp32 sums go to
// args.partial (laid out [m_local][virtual n], 4 consecutive n per 16-byte
// store) for splitk_reduce_kernel, which applies the epilogue. Partial
// n-tiles (N a multiple of 32, not of the tile): weight blocks past N are
// loaded as copies of row N-1 and their outputs not stored.
template <int EPI, int NB, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void gemm16_kernel(const GemmArgs args) {
  constexpr bool kSwi = EPI == static_cast<int>(Epilogue::kSwiGLU);
  static_assert(NB == 4 || NB == 5, "tile width");
  constexpr int BNT = 64 * NB;                   // weight rows of the tile
  constexpr int WB = 2 * NB;                     // 16-row weight blocks per wavefront
  constexpr int kSub = 8 * WB;                   // MFMAs per substep
  constexpr int kSlots = 2 * kSub;               // MFMAs per k-step
  constexpr int kBar = kSlots - 16;              // the barrier's slot
  constexpr int kATile = BM * BK, kBTile = BNT * BK;
  constexpr int kRowBytes = BK * 2, kChunks = BK / 8;
  constexpr int kRowsPerBlk = 4096 / kRowBytes;  // rows one load instruction of the 4 waves covers
  constexpr int kBlksA = BM / kRowsPerBlk, kBlksB = BNT / kRowsPerBlk;
  constexpr int kLoads = kBlksA + kBlksB;        // 16 or 18 loads per k-step
  // loads [0, kLC) of k-step kt + 2 go out after the barrier of kt, the rest
  // over the first 80 MFMAs of kt + 1, one per 8 MFMAs (one per 4, or more
  // of them after the barrier, measured slower: down +5%)
  constexpr int kLC = 8;
  constexpr int kWarm = 4;  // warm-up distance in k-steps
  static_assert(BK == 64 && kLoads - kLC <= kSub / 8 && (2 * WB) % 4 == 0, "pipeline shape");

  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  bf16_t* As = smem;              // [2][BM][BK]
  bf16_t* Bs = smem + 2 * kATile; // [2][BNT][BK], then 4 KB of warm-up scratch

  const int M = args.m, N = args.n, K = args.k;
  const int lda = args.lda, ldb = args.ldb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  // ---- work unit: contiguous per XCD, then tile and k-range ----
  const int total = args.units;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int q = total / kXcds, rmd = total % kXcds;
  const int unit = xcd * q + min(xcd, rmd) + bid / kXcds;
  int tile_m, tile_n;
  // (whole-tile launches have ksplit 1: constants, not divisions)
  const int ksplit = SPLIT ? args.ksplit : 1;
  tile_coords(args.tile_begin + unit / ksplit, args.tiles_m, args.tiles_n, tile_m, tile_n);
  const int m0 = tile_m * BM;
  const int kt_begin = SPLIT ? (unit % ksplit) * args.kt_per_split : 0;
  const int nk = SPLIT ? min(kt_begin + args.kt_per_split, K / BK) - kt_begin : K / BK;  // k-steps of this unit

  // B row block i (32 rows) of the tile: address of its first row, or for
  // SwiGLU of this wavefront's 8 rows, and the rows of its segment from there
  // on (<= 0: past N).
  auto b_block_base = [&](int i, int& avail) -> const char* {
    const void* base;
    int v;
    if constexpr (kSwi) {
      // block i: wave half i / NB, column group p = i % NB of it (16 output
      // columns); wavefronts 0, 1 load its gate rows, 2, 3 its up rows, 8
      // columns each
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      const int j = tile_n * (BNT / 2) + (i / NB) * (16 * NB) + (i % NB) * 16 + (w & 1) * 8;
      base = (w >> 1) ? args.bptr[1] : args.bptr[0];
      v = min(j, N - 1);
      avail = N - j;
    } else {
      const int row = tile_n * BNT + kRowsPerBlk * i;
      const int rr = min(row, N - 1);
      if (rr < args.brows[0]) {
        base = args.bptr[0];
        v = rr;
        avail = args.brows[0] - row;
      } else if (rr < args.brows[0] + args.brows[1]) {
        base = args.bptr[1];
        v = rr - args.brows[0];
        avail = args.brows[0] + args.brows[1] - row;
      } else {
        base = args.bptr[2];
        v = rr - args.brows[0] - args.brows[1];
        avail = N - row;
      }
    }
    return static_cast<const char*>(base) + static_cast<size_t>(v) * ldb * 2;
  };

  // ---- global -> LDS, as in gemm_f8w_kernel ----
  const int dma_row = wave * (1024 / kRowBytes) + lane / kChunks;
  const int dma_chunk = ((lane % kChunks) ^ swz(dma_row)) * 16;
  const int b_lane_row = kSwi ? lane / kChunks : dma_row;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  bf16_t* const warm_dst = smem + 2 * kATile + 2 * kBTile + wave_u * 512;
  const char* a_ptr[kBlksA];
  const char* b_ptr[kBlksB];
  unsigned a_off[kBlksA], b_off[kBlksB];
#pragma unroll
  for (int i = 0; i < kBlksA; ++i) {
    const int r = m0 + kRowsPerBlk * i;
    a_ptr[i] = static_cast<const char*>(args.a) + static_cast<size_t>(min(r, M - 1)) * lda * 2;
    a_off[i] = min(dma_row, max(M - r, 1) - 1) * lda * 2 + dma_chunk;
  }
#pragma unroll
  for (int i = 0; i < kBlksB; ++i) {
    int avail;
    b_ptr[i] = b_block_base(i, avail);
    b_off[i] = min(b_lane_row, max(avail, 1) - 1) * ldb * 2 + dma_chunk;
  }
  int warm_avail;
  const char* const warm_ptr = b_block_base((tile_m & 7) * (32 / kRowsPerBlk), warm_avail);
  const unsigned warm_off = min(b_lane_row, max(warm_avail, 1) - 1) * ldb * 2 + (lane % kChunks) * 16;

  auto koff = [&](int kt) { return static_cast<size_t>(kt_begin + min(kt, nk - 1)) * kRowBytes; };
  auto issue_load = [&](int kt, int stage, int l) {
    const bool isb = l >= 2 * kBlksA || (l & 1);
    const int i = l >= 2 * kBlksA ? l - kBlksA : l >> 1;
    bf16_t* dst = (isb ? Bs + stage * kBTile : As + stage * kATile) + wave_u * 512 + i * kRowsPerBlk * BK;
    global_load_lds16((isb ? b_ptr[i] : a_ptr[i]) + koff(kt), isb ? b_off[i] : a_off[i], lds_addr(dst));
  };
  auto issue_warm = [&](int kt) { global_load_lds16(warm_ptr + koff(kt), warm_off, lds_addr(warm_dst)); };

  // ---- LDS -> registers: row 16 blk + (lane & 15), chunk 4 s + kc of
  //      substep s through the swizzle (blocks start at multiples of 16 rows,
  //      so the swizzle depends on lane & 15 only). The MFMA takes k group
  //      lane >> 4 from each lane; which 8-k chunk feeds which k group does
  //      not change the sum as long as both operands agree, and kc = 0, 2,
  //      1, 3 for lane >> 4 = 0, 1, 2, 3 has lanes L and L + 32, which the
  //      LDS serves together, read chunks of opposite parity: with the
  //      swizzle that puts their 16-byte reads in distinct banks (chunks kc
  //      and kc + 2 of the same rows collide). ----
  const int r16 = lane & 15, g16 = lane >> 4;
  const int kc = ((g16 & 1) << 1) | (g16 >> 1);
  const int x_base = (wm * 128 + r16) * BK;
  const int w_base = (wn * (BNT / 2) + r16) * BK;
  const int c16[2] = {(kc ^ swz(r16)) * 8, ((4 + kc) ^ swz(r16)) * 8};
  auto rd_x = [&](int stage, int s, int jb) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As + stage * kATile + x_base + jb * 16 * BK +
                                                                        c16[s]));
  };
  auto rd_w = [&](int stage, int s, int ib) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Bs + stage * kBTile + w_base + ib * 16 * BK +
                                                                        c16[s]));
  };

  constexpr int kVB = WB - 8;  // weight blocks accumulating in VGPRs (0 or 2)
  f32x4 acc[8][8];                    // weight blocks 0-7 (AGPRs)
  f32x4 accv[kVB > 0 ? kVB : 1][8];   // weight blocks 8-9 (VGPRs)
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kVB; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) accv[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the zeroing writes, then the first MFMA reads of the same registers
#pragma unroll
  for (int i = 0; i < 8; ++i)
    asm volatile("s_nop 4" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                 "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
#pragma unroll
  for (int i = 0; i < kVB; ++i)
    asm volatile("s_nop 4" : "+v"(accv[i][0]), "+v"(accv[i][1]), "+v"(accv[i][2]), "+v"(accv[i][3]),
                 "+v"(accv[i][4]), "+v"(accv[i][5]), "+v"(accv[i][6]), "+v"(accv[i][7]));

  bf16x8 xo[2][8];  // activation operands of substeps 0 and 1
  bf16x8 wo[4];     // weight operands: the 2 WB of a k-step (WB s + ib) in a ring of four
  using Live = std::true_type;
  using Dead = std::false_type;

  // ---- one k-step: MFMA slot g = 80 s + 8 ib + jb, and after it the reads
  //      and loads placed there. LIVE1 / LIVE2: k-step kt+1 / kt+2 exists
  //      and is loaded. ----
  auto step = [&](int kt, auto LIVE1, auto LIVE2) {
    const int st = kt & 1;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, kBar>([&](auto G) {
      constexpr int g = decltype(G)::value;
      constexpr int s = g / kSub, ib = (g % kSub) / 8, jb = g % 8;
      mfma16<(ib < 8)>(acc16<ib, jb>(acc, accv), wo[(WB * s + ib) & 3], xo[s][jb]);
      // weight operand WB s' + i (i >= 2 of substep 0, all of substep 1)
      // after slot 8 (WB s' + i) - 12, two blocks before its first use
      if constexpr (g % 8 == 4) {
        constexpr int idx = (g + 12) / 8;
        wo[idx & 3] = rd_w(st, idx / WB, idx % WB);
      }
      // substep 1's activation operands, one per 4 slots, 12 or more slots
      // before their first use
      constexpr int x0 = kSub - 40;
      if constexpr (g >= x0 && g < x0 + 32 && g % 4 == 0) xo[1][(g - x0) / 4] = rd_x(st, 1, (g - x0) / 4);
      // loads [kLC, kLoads) of k-step kt+1 after slots 0, 8, 16, ..
      if constexpr (decltype(LIVE1)::value && g % 8 == 0 && g / 8 < kLoads - kLC)
        issue_load(kt + 1, st ^ 1, kLC + g / 8);
      if constexpr (g == kSub) issue_warm(kt + kWarm);
      __builtin_amdgcn_sched_barrier(0);
    });
    // k-step kt+1 is complete in LDS (only the warm-up load may still be in
    // flight) and no wavefront reads stage st any more
    wait_vmcnt<1>();
    lds_barrier();
    static_for<kBar, kSlots>([&](auto G) {
      constexpr int g = decltype(G)::value;
      constexpr int ib = (g - kSub) / 8, jb = g % 8;
      mfma16<(ib < 8)>(acc16<ib, jb>(acc, accv), wo[(WB + ib) & 3], xo[1][jb]);
      // the first operands of k-step kt+1: activations 0-7 and weights 0, 1
      // of its substep 0, in the order they are used
      constexpr int r = g - kBar;
      if constexpr (r == 1)
        wo[0] = rd_w(st ^ 1, 0, 0);
      else if constexpr (r == 9)
        wo[1] = rd_w(st ^ 1, 0, 1);
      else if constexpr (r < 9)
        xo[0][r == 0 ? 0 : r - 1] = rd_x(st ^ 1, 0, r == 0 ? 0 : r - 1);
      // loads [0, kLC) of k-step kt+2 into the stage just read
      if constexpr (decltype(LIVE2)::value && r % 2 == 0) issue_load(kt + 2, st, r / 2);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  if (nk > 0) {
    // k-step 0, the first loads of k-step 1 (k-step 0 again if there is no
    // k-step 1: into a stage that is not read) and the warm-up of k-steps
    // 1 .. kWarm-1 before the wait
#pragma unroll
    for (int l = 0; l < kLoads; ++l) issue_load(0, 0, l);
#pragma unroll
    for (int l = 0; l < kLC; ++l) issue_load(1, 1, l);
#pragma unroll
    for (int kt = 1; kt < kWarm; ++kt) issue_warm(kt);
    wait_vmcnt<kLC + kWarm - 1>();
    lds_barrier();
    xo[0][0] = rd_x(0, 0, 0);
    wo[0] = rd_w(0, 0, 0);
#pragma unroll
    for (int j = 1; j < 8; ++j) xo[0][j] = rd_x(0, 0, j);
    wo[1] = rd_w(0, 0, 1);
    // the last two k-steps are peeled off so that no load runs past the k-range
    int kt = 0;
    for (; kt < nk - 2; ++kt) step(kt, Live(), Live());
    if (kt < nk - 1) step(kt++, Live(), Dead());
    step(kt, Dead(), Dead());
    // the trailing loads and reads have completed
    wait_vmcnt<0>();
    lds_barrier();
  }

  // MFMA writes of the accumulators, then VALU reads: 16 wait states (more
  // than the 4-pass MFMA needs) before the group written last, more before
  // the rest
  static_for<0, kVB>([&](auto I) { mfma_result_wait<false, true>(accv[kVB - 1 - decltype(I)::value]); });
  static_for<0, 8>([&](auto I) {
    constexpr int i = 7 - decltype(I)::value;
    mfma_result_wait<true, kVB == 0 && i == 7>(acc[i]);
  });

  // ---- split-K unit: raw sums to the unit's partial tile, [m_local][virtual
  //      n] with virtual n = the tile's weight row (wave half wn, block ib) ----
  if constexpr (SPLIT) {
    float* dst = args.partial + static_cast<size_t>(unit) * BM * BNT;
    static_for<0, 8 * WB>([&](auto Q) {
      constexpr int jb = decltype(Q)::value / WB, ib = decltype(Q)::value % WB;
      *reinterpret_cast<f32x4*>(dst + (wm * 128 + jb * 16 + r16) * BNT + wn * (BNT / 2) + ib * 16 + 4 * g16) =
          acc16<ib, jb>(acc, accv);
    });
    return;
  }

  // ---- epilogue: outputs leave through a per-wavefront LDS region in two
  //      halves of 64 tokens, as 16-byte chunks along the rows. Rows past M:
  //      buffer resources that end at row M drop the stores and read zeros
  //      (see gemm_f8w_kernel). Weight blocks past N (a partial n-tile of the
  //      256-wide form; N is a multiple of 32, so a 16-row block is wholly
  //      in or out) are skipped by wave-uniform tests, their 16-byte chunks by
  //      a lane test in the stores. ----
  const size_t rbytes = static_cast<size_t>(M - m0) * args.ldc * sizeof(bf16_t);
  const int nbytes = static_cast<int>(rbytes < 0x7fffffffu ? rbytes : 0x7fffffffu);
  const size_t first = static_cast<size_t>(m0) * args.ldc;
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(args.c + first, (short)0, nbytes, 0x00020000);
  const int ldc_b = args.ldc * static_cast<int>(sizeof(bf16_t));
  if constexpr (kSwi) {
    // 128 x 16 NB outputs per wavefront (NB pairs of gate and up blocks);
    // staging rows of 16 NB + 8 bf16 (144 or 176 bytes: a write
    // instruction's 16 rows x 4 column groups hit every bank twice)
    constexpr int kCols = 16 * NB, kStg = kCols + 8, kRowChunks = kCols / 8;
    bf16_t* const stg = smem + wave_u * 64 * kStg;
    const int col0 = tile_n * (BNT / 2) + wn * kCols;
    static_for<0, 2>([&](auto H) {
      constexpr int h = decltype(H)::value;
      static_for<0, 4 * NB>([&](auto Q) {
        constexpr int jj = decltype(Q)::value / NB, p = decltype(Q)::value % NB;
        if (NB == 5 || col0 + 16 * p < N) {
          const f32x4& gt = acc16<2 * p, 4 * h + jj>(acc, accv);
          const f32x4& up = acc16<2 * p + 1, 4 * h + jj>(acc, accv);
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = silu_mul(gt[e], up[e]);
          u32x2 pk;
          pk[0] = pack_bf16x2(o[0], o[1]);
          pk[1] = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<u32x2*>(stg + (jj * 16 + r16) * kStg + p * 16 + 4 * g16) = pk;
        }
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < kRowChunks; ++it) {
        const int c = it * 64 + lane, r = c / kRowChunks, qq = c - r * kRowChunks;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * kStg + qq * 8);
        if (NB == 5 || col0 + qq * 8 < N)
          __builtin_amdgcn_raw_buffer_store_b128(v, c_rsrc, (wm * 128 + h * 64 + r) * ldc_b + (col0 + qq * 8) * 2, 0,
                                                 0);
      }
      // the reads above have returned before the next half overwrites the region
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    });
  } else {
    // Store, residual and bias forms: 128 x 16 WB outputs per wavefront;
    // staging rows of 16 WB + 8 bf16 (272 or 336 bytes, each bank takes two
    // rows of a write instruction). The lane's bias values (one per weight
    // block) are loaded together first, and a half's residual values in the
    // accumulator layout, all before its first add (a load past N reads
    // other columns of the buffer, or zeros past its end, for an output that
    // is not stored).
    constexpr int kCols = 16 * WB, kStg = kCols + 8, kRowChunks = kCols / 8;
    bf16_t* const stg = smem + wave_u * 64 * kStg;
    const int col0 = tile_n * BNT + wn * (BNT / 2);
    u32x2 bv[WB];
#pragma unroll
    for (int ib = 0; ib < WB; ++ib)
      bv[ib] = epi_bias(EPI) && col0 + ib * 16 < N
                   ? *reinterpret_cast<const u32x2*>(args.bias + col0 + ib * 16 + 4 * g16)
                   : u32x2{0, 0};
    const __amdgpu_buffer_rsrc_t r_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        epi_residual(EPI) ? const_cast<bf16_t*>(args.r) + first : args.c + first, (short)0, nbytes, 0x00020000);
    static_for<0, 2>([&](auto H) {
      constexpr int h = decltype(H)::value;
      u32x2 rv[4][WB];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int ib = 0; ib < WB; ++ib)
          rv[jj][ib] = epi_residual(EPI)
                           ? __builtin_amdgcn_raw_buffer_load_b64(
                                 r_rsrc, (wm * 128 + (4 * h + jj) * 16 + r16) * ldc_b + (col0 + ib * 16 + 4 * g16) * 2,
                                 0, 0)
                           : u32x2{0, 0};
      static_for<0, 4 * WB>([&](auto Q) {
        constexpr int jj = decltype(Q)::value / WB, ib = decltype(Q)::value % WB;
        if (NB == 5 || col0 + 16 * ib < N) {
          const f32x4& a = acc16<ib, 4 * h + jj>(acc, accv);
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = a[e];
          *reinterpret_cast<u32x2*>(stg + (jj * 16 + r16) * kStg + ib * 16 + 4 * g16) =
              finish4<EPI>(o, bv[ib], rv[jj][ib]);
        }
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < kRowChunks; ++it) {
        const int c = it * 64 + lane, r = c / kRowChunks, qq = c - r * kRowChunks;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * kStg + qq * 8);
        if (NB == 5 || col0 + qq * 8 < N)
          __builtin_amdgcn_raw_buffer_store_b128(v, c_rsrc, (wm * 128 + h * 64 + r) * ldc_b + (col0 + qq * 8) * 2, 0,
                                                 0);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    });
  }
}

// Sums the ksplit partial tiles of each split tile in a fixed order and
// applies the epilogue. Block (t, y) of 64 NB threads handles rows 4y..4y+3
// of split tile t; each thread 4 consecutive virtual columns. The SwiGLU
// virtual columns follow the kernel that wrote them: gemm16_kernel (bf16)
// pairs 16 gate and 16 up rows per 32-row block, gemm_f8w_kernel (FP8)
// alternates 8 gate and 8 up rows.
template <int EPI, bool F8, int NB>
__global__ __launch_bounds__(64 * NB) void splitk_reduce_kernel(const GemmArgs args) {
  constexpr int BNT = 64 * NB;
  constexpr int kRowThreads = BNT / 4;
  const int t = blockIdx.x;
  const int ml = blockIdx.y * 4 + threadIdx.x / kRowThreads;
  const int vn = (threadIdx.x % kRowThreads) * 4;
  int tile_m, tile_n;
  tile_coords(args.tile_begin + t, args.tiles_m, args.tiles_n, tile_m, tile_n);
  const int m = tile_m * BM + ml;
  bool live = m < args.m;  // every thread stays to the end (workgroup maximum)
  const float* src = args.partial + static_cast<size_t>(t) * args.ksplit * BM * BNT + ml * BNT + vn;
  f32x4 sum = *reinterpret_cast<const f32x4*>(src);
  for (int sidx = 1; sidx < args.ksplit; ++sidx)
    sum += *reinterpret_cast<const f32x4*>(src + static_cast<size_t>(sidx) * BM * BNT);
  const int N = args.n;
  float o[4];
  int n;
  if (EPI == static_cast<int>(Epilogue::kSwiGLU) && !F8) {
    // virtual column vn: wave half vn / (BNT/2), 16-row block (vn % (BNT/2))
    // / 16; even blocks are gate columns whose up partner sits 16 later
    const int r = vn % (BNT / 2), blk = r >> 4;
    live = live && (blk & 1) == 0;
    const int uo = (blk & 1) == 0 ? 16 : 0;
    f32x4 upsum = *reinterpret_cast<const f32x4*>(src + uo);
    for (int sidx = 1; sidx < args.ksplit; ++sidx)
      upsum += *reinterpret_cast<const f32x4*>(src + uo + static_cast<size_t>(sidx) * BM * BNT);
    n = tile_n * (BNT / 2) + (vn / (BNT / 2)) * (BNT / 4) + (blk >> 1) * 16 + (r & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = silu_mul(sum[e], upsum[e]);
  } else if (EPI == static_cast<int>(Epilogue::kSwiGLU)) {
    // virtual column vn: 32-row block vn / 32 (16 outputs each), 8-row group
    // (vn % 32) / 8; even groups are gate columns whose up partner sits 8
    // later
    const int blk = vn >> 5, grp = (vn & 31) >> 3;
    live = live && (grp & 1) == 0;
    const int uo = (grp & 1) == 0 ? 8 : 0;
    f32x4 upsum = *reinterpret_cast<const f32x4*>(src + uo);
    for (int sidx = 1; sidx < args.ksplit; ++sidx)
      upsum += *reinterpret_cast<const f32x4*>(src + uo + static_cast<size_t>(sidx) * BM * BNT);
    n = tile_n * (BNT / 2) + blk * 16 + (grp >> 1) * 8 + (vn & 7);
    sum *= args.scale_a[0] * args.scale_b[0][0];
    upsum *= args.scale_a[0] * args.scale_b[1][0];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = silu_mul(sum[e], upsum[e]);
  } else {
    n = tile_n * BNT + vn;
    if constexpr (F8) {
      if (n < N) sum *= f8_scale(args, n);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = sum[e];
  }
  live = live && n < N;
  const size_t off = static_cast<size_t>(m) * args.ldc + n;
  if constexpr (EPI == static_cast<int>(Epilogue::kSwiGLU)) {
    u32x2 pk;
    pk[0] = pack_bf16x2(o[0], o[1]);
    pk[1] = pack_bf16x2(o[2], o[3]);
    if (live) *reinterpret_cast<u32x2*>(args.c + off) = pk;
    if (F8 && args.amax) {
      __shared__ float red[4];
      const float v = workgroup_max(live ? abs_max4(pk) : 0.f, red);
      if (threadIdx.x == 0) args.amax[t * (BM / 4) + blockIdx.y] = v;
    }
  } else if (live) {
    const u32x2 rv = epi_residual(EPI) ? *reinterpret_cast<const u32x2*>(args.r + off) : u32x2{0, 0};
    *reinterpret_cast<u32x2*>(args.c + off) = finish4<EPI>(o, args, n, rv);
  }
}

template <int EPI, bool F8, int NB, bool SPLIT>
hipError_t launch_epi(const GemmArgs& args, int grid, hipStream_t stream) {
  // two stages of both operands, then the warm-up scratch (4 KB)
  constexpr size_t smem = static_cast<size_t>(2) * (BM + 64 * NB) * BK * sizeof(bf16_t) + 4096;
  // bf16: gemm16_kernel (16x16x32 MFMAs); FP8: gemm_f8w_kernel (32x32x64)
  const void* kernel;
  if constexpr (F8)
    kernel = reinterpret_cast<const void*>(&gemm_f8w_kernel<EPI, NB, SPLIT>);
  else
    kernel = reinterpret_cast<const void*>(&gemm16_kernel<EPI, NB, SPLIT>);
  // the dynamic-LDS limit is raised once per device (bit d: done on device d)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (!bit || !(attr_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  if constexpr (F8)
    hipLaunchKernelGGL((gemm_f8w_kernel<EPI, NB, SPLIT>), dim3(grid), dim3(kThreads), smem, stream, args);
  else
    hipLaunchKernelGGL((gemm16_kernel<EPI, NB, SPLIT>), dim3(grid), dim3(kThreads), smem, stream, args);
  return hipGetLastError();
}

}  // namespace

int gemm_segment_rows() { return 4096 / (BK * 2); }

bool gemm_supported(int n, int k) { return n > 0 && k > 0 && n % 32 == 0 && k % BK == 0; }

int gemm_amax_parts(int m, int n) {
  // whole tiles (SwiGLU: 128 output columns each) plus 64 row groups of each
  // split tile, fewer than one per CU
  return ((m + BM - 1) / BM) * ((n + BN / 2 - 1) / (BN / 2)) + (BM / 4) * 256;
}

bool gemm_fp8_supported(int n, int k) { return n > 0 && k > 0 && n % 32 == 0 && k % (2 * BK) == 0; }

namespace {

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

template <int EPI, bool F8, int NB>
hipError_t run(GemmArgs args, float* partial, size_t partial_bytes, hipStream_t stream, int* amax_count) {
  // One workgroup fills a CU (128 or 144 KB of LDS), so a launch of T tiles
  // runs in ceil(T / CUs) waves. Full waves run whole tiles; when the last
  // wave would leave at least half the CUs idle and is a sizeable part of the
  // launch (at most 4 full waves before it), its R tiles are cut into ksplit
  // k-ranges (ksplit * R <= CUs) whose fp32 partials are summed by a small
  // reduction.
  constexpr int BNT = 64 * NB;
  const int tn = EPI == static_cast<int>(Epilogue::kSwiGLU) ? BNT / 2 : BNT;  // output columns per tile
  args.tiles_n = (args.n + tn - 1) / tn;
  const int tiles = args.tiles_m * args.tiles_n;
  const int nk = args.k / (F8 ? 2 * BK : BK);  // k-steps (128 row bytes each)
  static const int cus = device_cus();
  const int rem = tiles % cus;
  int ksplit = 1;
  // (with amax output, the row groups of the split tiles must fit gemm_amax_parts)
  const bool amax_fits = !args.amax || (tiles + rem * (BM / 4) <= gemm_amax_parts(args.m, args.n));
  if (NB == 4 && partial && rem > 0 && rem <= cus / 2 && tiles / cus <= 4 && amax_fits) {
    ksplit = min(cus / rem, 16);
    ksplit = min(ksplit, nk / 4);
    const size_t cap = partial_bytes / (static_cast<size_t>(BM) * BNT * sizeof(float));
    while (ksplit > 1 && static_cast<size_t>(ksplit) * rem > cap) --ksplit;
  }
  const int full = ksplit > 1 ? tiles - rem : tiles;
  hipError_t e;
  if (full > 0) {
    GemmArgs a = args;
    a.tile_begin = 0;
    a.units = full;
    a.ksplit = 1;
    a.kt_per_split = nk;
    a.partial = nullptr;
    if ((e = launch_epi<EPI, F8, NB, false>(a, full, stream)) != hipSuccess) return e;
  }
  if (amax_count) *amax_count = full + (ksplit > 1 ? rem * (BM / 4) : 0);
  if constexpr (NB == 4) {  // (the 320-wide tile is only taken for whole waves)
    if (ksplit > 1) {
      GemmArgs a = args;
      a.tile_begin = full;
      a.units = rem * ksplit;
      a.ksplit = ksplit;
      a.kt_per_split = (nk + ksplit - 1) / ksplit;
      a.partial = partial;
      a.amax = args.amax ? args.amax + full : nullptr;
      if ((e = launch_epi<EPI, F8, NB, true>(a, a.units, stream)) != hipSuccess) return e;
      hipLaunchKernelGGL((splitk_reduce_kernel<EPI, F8, NB>), dim3(rem, BM / 4), dim3(BNT), 0, stream, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

size_t gemm_partial_bytes() { return static_cast<size_t>(320) * BM * BN * sizeof(float); }

namespace {

// Shared set-up of the bf16 and FP8 launches; es = bytes per operand element.
hipError_t launch_common(Epilogue epi, bool f8, const void* a, int lda, const float* scale_a,
                         const void* const* bptr, const int* brows, const float* const* bscale,
                         int count, int ldb, bf16_t* c, int ldc, const bf16_t* residual, int m,
                         int n, int k, float* partial, size_t partial_bytes, hipStream_t stream,
                         const bf16_t* bias, float* amax, int* amax_count) {
  const int es = f8 ? 1 : 2;
  if (lda < k || ldb < k || ldc < n || (lda * es) % 16 != 0 || (ldb * es) % 16 != 0 || ldc % 4 != 0)
    return hipErrorInvalidValue;
  if (count < 1 || count > 3) return hipErrorInvalidValue;
  if (m <= 0) return hipSuccess;
  // a load block never straddles two weight segments
  if (epi != Epilogue::kSwiGLU && count > 1)
    for (int i = 0; i < count; ++i)
      if (brows[i] % gemm_segment_rows() != 0) return hipErrorInvalidValue;
  GemmArgs args{};
  args.a = a;
  args.scale_a = scale_a;
  for (int i = 0; i < 3; ++i) {
    args.bptr[i] = i < count ? bptr[i] : bptr[0];
    args.brows[i] = i < count ? brows[i] : 0;
    args.scale_b[i] = f8 ? (i < count ? bscale[i] : bscale[0]) : nullptr;
  }
  args.c = c;
  args.r = residual;
  args.bias = bias;
  if (amax && (epi != Epilogue::kSwiGLU || !f8)) return hipErrorInvalidValue;
  args.amax = amax;
  if (amax_count) *amax_count = 0;
  if (static_cast<int>(epi) >= static_cast<int>(Epilogue::kBias) && !bias) return hipErrorInvalidValue;
  args.m = m;
  args.n = n;
  args.k = k;
  args.lda = lda;
  args.ldb = ldb;
  args.ldc = ldc;
  args.tiles_m = (m + BM - 1) / BM;
  // the decoder's linears take 320-wide tiles where those fill whole waves
  // of the chip exactly
  static const int cus = device_cus();
  const int wide_cols = epi == Epilogue::kSwiGLU ? 160 : 320;  // output columns of a 320-wide tile
  const bool wide = n % wide_cols == 0 && (args.tiles_m * (n / wide_cols)) % cus == 0;
  if (f8) {
    switch (epi) {
      case Epilogue::kStore:
        return wide ? run<0, true, 5>(args, partial, partial_bytes, stream, amax_count)
                    : run<0, true, 4>(args, partial, partial_bytes, stream, amax_count);
      case Epilogue::kResidual:
        return wide ? run<1, true, 5>(args, partial, partial_bytes, stream, amax_count)
                    : run<1, true, 4>(args, partial, partial_bytes, stream, amax_count);
      case Epilogue::kSwiGLU:
        return wide ? run<2, true, 5>(args, partial, partial_bytes, stream, amax_count)
                    : run<2, true, 4>(args, partial, partial_bytes, stream, amax_count);
      default: return hipErrorInvalidValue;  // the biased forms are bf16 only
    }
  }
  switch (epi) {
    case Epilogue::kStore:
      return wide ? run<0, false, 5>(args, partial, partial_bytes, stream, amax_count)
                  : run<0, false, 4>(args, partial, partial_bytes, stream, amax_count);
    case Epilogue::kResidual:
      return wide ? run<1, false, 5>(args, partial, partial_bytes, stream, amax_count)
                  : run<1, false, 4>(args, partial, partial_bytes, stream, amax_count);
    case Epilogue::kSwiGLU:
      return wide ? run<2, false, 5>(args, partial, partial_bytes, stream, amax_count)
                  : run<2, false, 4>(args, partial, partial_bytes, stream, amax_count);
    case Epilogue::kBias: return run<3, false, 4>(args, partial, partial_bytes, stream, amax_count);
    case Epilogue::kBiasResidual: return run<4, false, 4>(args, partial, partial_bytes, stream, amax_count);
    case Epilogue::kBiasGeluTanh: return run<5, false, 4>(args, partial, partial_bytes, stream, amax_count);
    case Epilogue::kBiasGeluErf: return run<6, false, 4>(args, partial, partial_bytes, stream, amax_count);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(Epilogue epi, const bf16_t* a, int lda, const BSegments& b, int ldb,
                       bf16_t* c, int ldc, const bf16_t* residual, int m, int n, int k,
                       float* partial, size_t partial_bytes, hipStream_t stream,
                       const bf16_t* bias) {
  const void* bptr[3] = {b.ptr[0], b.ptr[1], b.ptr[2]};
  return launch_common(epi, false, a, lda, nullptr, bptr, b.rows, nullptr, b.count, ldb, c, ldc,
                       residual, m, n, k, partial, partial_bytes, stream, bias, nullptr, nullptr);
}

hipError_t launch_gemm_fp8(Epilogue epi, const uint8_t* a, int lda, const float* scale_a,
                           const F8Segments& b, int ldb, bf16_t* c, int ldc,
                           const bf16_t* residual, int m, int n, int k, float* partial,
                           size_t partial_bytes, hipStream_t stream, float* amax, int* amax_count) {
  if (!scale_a) return hipErrorInvalidValue;
  for (int i = 0; i < b.count && i < 3; ++i)
    if (!b.scale[i]) return hipErrorInvalidValue;
  const void* bptr[3] = {b.ptr[0], b.ptr[1], b.ptr[2]};
  return launch_common(epi, true, a, lda, scale_a, bptr, b.rows, b.scale, b.count, ldb, c, ldc,
                       residual, m, n, k, partial, partial_bytes, stream, nullptr, amax, amax_count);
}

}  // namespace mhe
