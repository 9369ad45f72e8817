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
//
// Tiling: a 256 (m) x 256 (n) output tile per workgroup of 4 wavefronts, each
// wavefront owning 128 x 128 as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16. The
// weight rows are the MFMA "A" operand and the activation rows the "B"
// operand, so every lane ends up with 4 consecutive output columns (8-byte
// stores). K advances 64 at a time through an LDS double buffer (2 x 64 KB);
// rows are 128 bytes and their 16-byte chunks are XOR-swizzled so the
// ds_read_b128 operand fetches of 8 or 16 consecutive lanes hit distinct banks.
// Workgroups are remapped so that each XCD (workgroups are dealt round-robin
// over the 8 XCDs) receives a contiguous run of tiles, ordered in groups of m
// tiles so tiles running together on one XCD share A and B panels in its L2.
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kTileElems = BM * BK;  // per operand per stage (BM == BN)
constexpr int kGroupM = 4;           // m tiles per ordering group
constexpr int kXcds = 8;

struct GemmArgs {
  const bf16_t* a;
  const bf16_t* bptr[3];
  int brows[3];
  bf16_t* c;
  const bf16_t* r;
  int m, n, k;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Buffer resource over [p, p + bytes); the pointer and size are wave-uniform
// and are pinned to scalar registers so loads need no per-lane descriptor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scalar_rsrc(const bf16_t* p, int bytes) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  const uint64_t s = (static_cast<uint64_t>(hi) << 32) | lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(s), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmArgs args) {
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  bf16_t* As = smem;                   // [2][BM][BK]
  bf16_t* Bs = smem + 2 * kTileElems;  // [2][BN][BK]

  const int M = args.m, N = args.n, K = args.k;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  // ---- tile id: contiguous per XCD, then grouped-m ordering ----
  const int total = args.tiles_m * args.tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int q = total / kXcds, rmd = total % kXcds;
  const int logical = xcd * q + min(xcd, rmd) + bid / kXcds;
  const int group_size = kGroupM * args.tiles_n;
  const int group = logical / group_size;
  const int first_m = group * kGroupM;
  const int gm = min(args.tiles_m - first_m, kGroupM);
  const int in_group = logical - group * group_size;
  const int tile_m = first_m + in_group % gm;
  const int tile_n = in_group / gm;
  const int m0 = tile_m * BM;

  // ---- global -> LDS: each operand tile is 8 blocks of 32 rows; block i of
  //      A is rows m0+32i.., block i of B a 32-row slice of one weight
  //      segment. Every block gets its own buffer resource (scalar), bounded
  //      to the rows that exist, so rows past M read as zero. The loads go
  //      straight to LDS (buffer_load_dwordx4 ... lds): lane L of wave w fills
  //      16 bytes at LDS row w*8 + L/8 of the block, physical chunk L%8, so it
  //      fetches the logical chunk that the swizzle puts there.
  const int fill_row = wave * 8 + (lane >> 3);
  const int fill_chunk = (lane & 7) ^ swz(fill_row);
  const int voff = fill_row * K * 2 + fill_chunk * 16;

  __amdgpu_buffer_rsrc_t a_rsrc[8], b_rsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row0 = m0 + 32 * i;
    const int nrows = max(0, min(32, M - row0));
    a_rsrc[i] = scalar_rsrc(args.a + static_cast<size_t>(min(row0, M - 1)) * K, nrows * K * 2);
    const bf16_t* base;
    int v;
    bool ok;
    if (EPI == static_cast<int>(Epilogue::kSwiGLU)) {
      // block i: wave half i/4, slot i%4; slots 0,1 gate rows, 2,3 up rows
      const int j = tile_n * (BN / 2) + (i >> 2) * 64 + (i & 1) * 32;
      ok = j < N;
      base = ((i & 3) < 2) ? args.bptr[0] : args.bptr[1];
      v = ok ? j : 0;
    } else {
      const int row = tile_n * BN + 32 * i;
      ok = row < N;
      const int rr = ok ? row : 0;
      if (rr < args.brows[0]) {
        base = args.bptr[0];
        v = rr;
      } else if (rr < args.brows[0] + args.brows[1]) {
        base = args.bptr[1];
        v = rr - args.brows[0];
      } else {
        base = args.bptr[2];
        v = rr - args.brows[0] - args.brows[1];
      }
    }
    b_rsrc[i] = scalar_rsrc(base + static_cast<size_t>(v) * K, ok ? 32 * K * 2 : 0);
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue_tile = [&](int kt, int stage) {
    const int soff = kt * BK * 2;
    bf16_t* as = As + stage * kTileElems + wave_u * 8 * BK;
    bf16_t* bs = Bs + stage * kTileElems + wave_u * 8 * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc[i], (__attribute__((address_space(3))) void*)(as + i * 32 * BK), 16, voff, soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          b_rsrc[i], (__attribute__((address_space(3))) void*)(bs + i * 32 * BK), 16, voff, soff, 0, 0);
    }
  };

  // operand fetch offsets inside a stage
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int lswz = swz(lrow);
  const int a_base = (wm * 128 + lrow) * BK;  // activation rows (MFMA B operand)
  const int b_base = (wn * 128 + lrow) * BK;  // weight rows (MFMA A operand)

  const int nk = K / BK;
  issue_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue_tile(kt + 1, cur ^ 1);
    const bf16_t* as = As + cur * kTileElems;
    const bf16_t* bs = Bs + cur * kTileElems;
    // operands of substep s+1 are fetched while substep s's 16 MFMAs run
    bf16x8 wop[2][4], xop[2][4];
    auto fetch = [&](int s, int slot) {
      const int chunk = ((2 * s + lhalf) ^ lswz) << 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wop[slot][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bs + b_base + i * 32 * BK + chunk));
        xop[slot][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(as + a_base + i * 32 * BK + chunk));
      }
    };
    fetch(0, 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < BK / 16) fetch(s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop[s & 1][i], xop[s & 1][j], acc[i][j], 0, 0, 0);
      if (s + 1 < BK / 16) {
        // spread the 8 operand reads between the 16 MFMAs
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next stage's loads have landed in LDS, and every wave is done
    // reading this stage before it is refilled
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: lane holds column m = lrow of each 32x32 block and rows
  //      n = 8 g + 4 lhalf + e (e < 4) for the four groups g ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + j * 32 + lrow;
    if (m >= M) continue;
    if (EPI == static_cast<int>(Epilogue::kSwiGLU)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int jb = tile_n * (BN / 2) + wn * 64 + i * 32;
        if (jb >= N) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gt = acc[i][j][4 * g + e];
            const float up = acc[i + 2][j][4 * g + e];
            o[e] = gt / (1.f + __expf(-gt)) * up;
          }
          u32x2 pk;
          pk[0] = pack_bf16x2(o[0], o[1]);
          pk[1] = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<u32x2*>(args.c + static_cast<size_t>(m) * N + jb + 8 * g + 4 * lhalf) = pk;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nb = tile_n * BN + wn * 128 + i * 32;
        if (nb >= N) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const size_t off = static_cast<size_t>(m) * N + nb + 8 * g + 4 * lhalf;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * g + e];
          if (EPI == static_cast<int>(Epilogue::kResidual)) {
            const u32x2 rv = *reinterpret_cast<const u32x2*>(args.r + off);
            o[0] += __uint_as_float(rv[0] << 16);
            o[1] += __uint_as_float(rv[0] & 0xffff0000u);
            o[2] += __uint_as_float(rv[1] << 16);
            o[3] += __uint_as_float(rv[1] & 0xffff0000u);
          }
          u32x2 pk;
          pk[0] = pack_bf16x2(o[0], o[1]);
          pk[1] = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<u32x2*>(args.c + off) = pk;
        }
      }
    }
  }
}

constexpr size_t kSmemBytes = 4 * kTileElems * sizeof(bf16_t);  // 128 KB

template <int EPI>
hipError_t launch_epi(const GemmArgs& args, int grid, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(kSmemBytes));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(gemm_kernel<EPI>, dim3(grid), dim3(kThreads), kSmemBytes, stream, args);
  return hipGetLastError();
}

}  // namespace

bool gemm_supported(int n, int k) { return n > 0 && k > 0 && n % 32 == 0 && k % BK == 0; }

hipError_t launch_gemm(Epilogue epi, const bf16_t* a, const BSegments& b, bf16_t* c,
                       const bf16_t* residual, int m, int n, int k, hipStream_t stream) {
  if (m <= 0) return hipSuccess;
  GemmArgs args{};
  args.a = a;
  for (int i = 0; i < 3; ++i) {
    args.bptr[i] = i < b.count ? b.ptr[i] : b.ptr[0];
    args.brows[i] = i < b.count ? b.rows[i] : 0;
  }
  args.c = c;
  args.r = residual;
  args.m = m;
  args.n = n;
  args.k = k;
  args.tiles_m = (m + BM - 1) / BM;
  args.tiles_n = epi == Epilogue::kSwiGLU ? (n + BN / 2 - 1) / (BN / 2) : (n + BN - 1) / BN;
  const int grid = args.tiles_m * args.tiles_n;
  switch (epi) {
    case Epilogue::kStore: return launch_epi<0>(args, grid, stream);
    case Epilogue::kResidual: return launch_epi<1>(args, grid, stream);
    case Epilogue::kSwiGLU: return launch_epi<2>(args, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mhe
