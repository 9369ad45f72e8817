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

// x and y may alias (with ldy == dim): every lane loads its whole row slice
// before any store.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const bf16_t* x,
                                                      const bf16_t* __restrict__ gamma,
                                                      bf16_t* y, int ldy, int rows, int dim,
                                                      float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nchunks = dim >> 3;
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
  const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);
  u32x4* yr = reinterpret_cast<u32x4*>(y + static_cast<size_t>(row) * ldy);
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      float f[8], g[8];
      unpack8(v[i], f);
      unpack8(gr[c], g);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = g[j] * (f[j] * r);
      yr[c] = pack8(f);
    }
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
  float s1 = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      v[i] = xr[c];
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) s1 += f[j];
    }
  }
  const float mean = wave_sum(s1) / static_cast<float>(dim);
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) s2 += (f[j] - mean) * (f[j] - mean);
    }
  }
  const float r = rsqrtf(wave_sum(s2) / static_cast<float>(dim) + eps);
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
  hipLaunchKernelGGL(rmsnorm_kernel, grid, dim3(256), 0, stream, x, gamma, y, ldy, rows, dim, eps);
  return hipGetLastError();
}

bool rmsnorm_supported(int dim) { return dim > 0 && dim % 8 == 0 && dim <= 64 * 8 * kMaxChunks; }

}  // namespace mhe
