// Per-tensor FP8 (E4M3) quantisation of bf16 tensors, the input side of the
// FP8 linears (H3 encoder page: an FP8 quantisation config on a checkpoint
// that is not FP8-serialised, so weights are quantised when loaded and
// activations on every call; the page does not print the method, and the
// plain per-tensor form is taken):
//
//   s = max|x| / 448,  q = E4M3_rne(clamp(x * (448 / max|x|), -448, 448))
//
// with the factor and the product in fp32 (IEEE division and multiply, no
// fusion) and all-zero tensors giving zero codes and s = 1. E4M3 is the OCP
// "fn" format (bias 7, no infinities, largest finite 448); the gfx950
// conversion v_cvt_pk_fp8_f32 rounds to nearest even and turns values beyond
// the range into NaN, hence the clamp.
//
// The scale needs the whole tensor, so quantisation is three launches:
// partial maxima of |x| (amax_kernel, or fused into the kernel that produces
// x: the RMSNorm pass in rmsnorm.hip, the gate/up GEMM's epilogue),
// amax_finalize_kernel (one workgroup: the scale and the factor 448 / amax),
// and quantize_kernel. The two sweeps are HBM-bound: 2 bytes per element read
// by each, 1 byte per element written by the second.
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte chunks in flight per lane

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// partial[b] = max |x| over rows b*4 + wave, stepping by gridDim.x*4
__global__ __launch_bounds__(kThreads) void amax_kernel(const bf16_t* __restrict__ x, int ldx, int rows,
                                                       int cols, float* __restrict__ partial) {
  __shared__ float red[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = cols / 8;
  float m = 0.f;
  for (int r = blockIdx.x * 4 + wave; r < rows; r += gridDim.x * 4) {
    const u32x4* row = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(r) * ldx);
    for (int c0 = lane; c0 < nch; c0 += 64 * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = c0 + 64 * u < nch ? row[c0 + 64 * u] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          m = fmaxf(m, __uint_as_float((v[u][i] << 16) & 0x7fffffffu));
          m = fmaxf(m, __uint_as_float(v[u][i] & 0x7fff0000u));
        }
    }
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void amax_finalize_kernel(const float* __restrict__ partial, int nparts,
                                                                float* __restrict__ scale,
                                                                float* __restrict__ factor) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < nparts; i += kThreads) m = fmaxf(m, partial[i]);
  const float amax = block_max(m, red);
  if (threadIdx.x == 0) {
    scale[0] = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
    factor[0] = amax > 0.f ? __fdiv_rn(448.f, amax) : 0.f;
  }
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(const bf16_t* __restrict__ x, int ldx, int rows,
                                                           int cols, const float* __restrict__ factor,
                                                           uint8_t* __restrict__ q, int ldq) {
  const float f = factor[0];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = cols / 8;
  for (int r = blockIdx.x * 4 + wave; r < rows; r += gridDim.x * 4) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(r) * ldx);
    u32x2* dst = reinterpret_cast<u32x2*>(q + static_cast<size_t>(r) * ldq);
    for (int c0 = lane; c0 < nch; c0 += 64 * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = c0 + 64 * u < nch ? src[c0 + 64 * u] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (c0 + 64 * u < nch) dst[c0 + 64 * u] = e4m3x8(v[u], f);
    }
  }
}

int sweep_grid(int rows) { return min((rows + 3) / 4, kAmaxParts); }

}  // namespace

int amax_parts(int rows) { return rows > 0 ? sweep_grid(rows) : 0; }

hipError_t launch_amax(const bf16_t* x, int ldx, int rows, int cols, float* partial, int nparts,
                       hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (cols % 8 != 0 || ldx % 8 != 0 || ldx < cols || nparts < 1 || nparts > kAmaxParts)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(amax_kernel, dim3(nparts), dim3(kThreads), 0, stream, x, ldx, rows, cols, partial);
  return hipGetLastError();
}

hipError_t launch_amax_finalize(const float* partial, int nparts, float* scale, float* factor,
                                hipStream_t stream) {
  if (nparts < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kThreads), 0, stream, partial, nparts, scale,
                     factor);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const bf16_t* x, int ldx, int rows, int cols, const float* factor,
                               uint8_t* q, int ldq, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (cols % 8 != 0 || ldx % 8 != 0 || ldq % 8 != 0 || ldx < cols || ldq < cols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_kernel, dim3(sweep_grid(rows)), dim3(kThreads), 0, stream, x, ldx, rows,
                     cols, factor, q, ldq);
  return hipGetLastError();
}

}  // namespace mhe
