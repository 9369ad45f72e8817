// Row RMSNorm, one wavefront per row (H3 encoder page, MiniMaxH3Qwen3VLRMSNorm):
// y = gamma * x * rsqrt(mean(x^2) + eps), reduction and scaling in fp32, one
// bf16 rounding. HBM-bound: reads 2*dim bytes and writes 2*dim bytes per row.
//
// Row LayerNorm the same way (the nn.LayerNorm of the page's vision blocks
// and mergers): y = (x - mean) * rsqrt(var + eps) * w + b with the biased
// variance, both moments from the row held in registers.
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int kRowsPerBlock = 4;   // 4 waves, one row each
constexpr int kMaxChunks = 16;     // 16-byte chunks per lane -> dim <= 64*8*16 = 8192

enum NormMode { kWrite = 0, kAmax = 1, kQuantize = 2 };

// MODE kWrite: y = the normed rows in bf16 (x and y may alias with
// ldy == dim: every lane loads its whole row slice before any store).
// MODE kAmax: no output rows; partial[block] = max |y| over the block's rows,
// y as kWrite would store it. MODE kQuantize: the E4M3 codes of those bf16 y
// values times factor[0] (per-tensor quantisation, quant.hip) into q.
// All three compute y with the same operations, so the FP8 forms quantise
// exactly the tensor kWrite writes.
template <int MODE>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const bf16_t* x,
                                                      const bf16_t* __restrict__ gamma,
                                                      bf16_t* y, int ldy, int rows, int dim,
                                                      float eps, float* __restrict__ partial,
                                                      const float* __restrict__ factor,
                                                      uint8_t* __restrict__ q) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const bool live = row < rows;
  if (MODE != kAmax && !live) return;
  const int nchunks = live ? dim >> 3 : 0;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(row) * dim);
  u32x4 v[kMaxChunks];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      v[i] = xr[c];
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
    }
  }
  ss = wave_sum(ss);
  const float r = rsqrtf(ss / static_cast<float>(dim) + eps);
  const float fq = MODE == kQuantize ? factor[0] : 0.f;
  const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      float f[8], g[8];
      unpack8(v[i], f);
      unpack8(gr[c], g);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = g[j] * (f[j] * r);
      const u32x4 yb = pack8(f);
      if constexpr (MODE == kWrite) {
        reinterpret_cast<u32x4*>(y + static_cast<size_t>(row) * ldy)[c] = yb;
      } else {
        unpack8(yb, f);
        if constexpr (MODE == kAmax) {
#pragma unroll
          for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
        } else {
          reinterpret_cast<u32x2*>(q + static_cast<size_t>(row) * ldy)[c] = e4m3x8(f, fq);
        }
      }
    }
  }
  if constexpr (MODE == kAmax) {
    __shared__ float red[kRowsPerBlock];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
}

__global__ __launch_bounds__(256) void layernorm_kernel(const bf16_t* x, int ldx,
                                                        const bf16_t* __restrict__ w,
                                                        const bf16_t* __restrict__ bias,
                                                        bf16_t* y, int ldy, int rows, int dim,
                                                        float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nchunks = dim >> 3;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(row) * ldx);
  u32x4 v[kMaxChunks];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) v[i] = xr[c];
  }
  // mean and variance in one pass over the row, on data shifted by its first
  // element (the shifted-data form of the sums: the shift keeps the squares
  // near the variance's scale, so no cancellation against a large mean),
  // and one wavefront reduction carrying both sums
  const float shift = __uint_as_float(__builtin_amdgcn_readfirstlane(v[0][0] << 16));  // x[row][0] (lane 0)
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float z = f[j] - shift;
        s1 += z;
        s2 += z * z;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    s1 += __shfl_xor(s1, off, 64);
    s2 += __shfl_xor(s2, off, 64);
  }
  const float inv_n = 1.f / static_cast<float>(dim);
  const float zmean = s1 * inv_n;
  const float mean = shift + zmean;
  const float r = rsqrtf(fmaxf(s2 * inv_n - zmean * zmean, 0.f) + eps);
  const u32x4* wr = reinterpret_cast<const u32x4*>(w);
  const u32x4* br = reinterpret_cast<const u32x4*>(bias);
  u32x4* yr = reinterpret_cast<u32x4*>(y + static_cast<size_t>(row) * ldy);
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      float f[8], g[8], bb[8];
      unpack8(v[i], f);
      unpack8(wr[c], g);
      unpack8(br[c], bb);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = (f[j] - mean) * r * g[j] + bb[j];
      yr[c] = pack8(f);
    }
  }
}

}  // namespace

hipError_t launch_layernorm(const bf16_t* x, int ldx, const bf16_t* w, const bf16_t* b, bf16_t* y,
                            int ldy, int rows, int dim, float eps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (ldy < dim || ldy % 8 != 0 || ldx < dim || ldx % 8 != 0) return hipErrorInvalidValue;
  dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(layernorm_kernel, grid, dim3(256), 0, stream, x, ldx, w, b, y, ldy, rows, dim,
                     eps);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const bf16_t* x, const bf16_t* gamma, bf16_t* y, int ldy, int rows,
                          int dim, float eps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (ldy < dim || ldy % 8 != 0) return hipErrorInvalidValue;
  dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(rmsnorm_kernel<kWrite>, grid, dim3(256), 0, stream, x, gamma, y, ldy, rows, dim, eps,
                     nullptr, nullptr, nullptr);
  return hipGetLastError();
}

int rmsnorm_fp8_parts(int rows) { return (rows + kRowsPerBlock - 1) / kRowsPerBlock; }

hipError_t launch_rmsnorm_fp8(const bf16_t* x, const bf16_t* gamma, int rows, int dim, float eps,
                              float* partial, float* scale, float* factor, uint8_t* q, int ldq,
                              hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (ldq < dim || ldq % 8 != 0) return hipErrorInvalidValue;
  const int blocks = rmsnorm_fp8_parts(rows);
  hipLaunchKernelGGL(rmsnorm_kernel<kAmax>, dim3(blocks), dim3(256), 0, stream, x, gamma, nullptr, 0, rows,
                     dim, eps, partial, nullptr, nullptr);
  hipError_t e = launch_amax_finalize(partial, blocks, scale, factor, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rmsnorm_kernel<kQuantize>, dim3(blocks), dim3(256), 0, stream, x, gamma, nullptr, ldq,
                     rows, dim, eps, nullptr, factor, q);
  return hipGetLastError();
}

bool rmsnorm_supported(int dim) { return dim > 0 && dim % 8 == 0 && dim <= 64 * 8 * kMaxChunks; }

}  // namespace mhe
