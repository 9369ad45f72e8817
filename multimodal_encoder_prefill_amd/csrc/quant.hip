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
// Two launches, because the scale needs the whole tensor: amax_kernel writes
// one partial maximum per workgroup, quantize_kernel reduces the partials
// (every workgroup redoes this small reduction, so no third launch and no
// atomics) and converts. Both are HBM-bound row sweeps: 2 bytes per element
// read by each, 1 byte per element written by the second.
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red may still be read from a previous call
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// partial[b] = max |x| over rows b, b + gridDim.x, ...
__global__ __launch_bounds__(kThreads) void amax_kernel(const bf16_t* __restrict__ x, int ldx, int rows,
                                                       int cols, float* __restrict__ partial) {
  __shared__ float red[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float m = 0.f;
  for (int r = blockIdx.x * 4 + wave; r < rows; r += gridDim.x * 4) {
    const u32x4* row = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(r) * ldx);
    for (int c = lane; c < cols / 8; c += 64) {
      const u32x4 v = row[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, __uint_as_float((v[i] << 16) & 0x7fffffffu));
        m = fmaxf(m, __uint_as_float(v[i] & 0x7fff0000u));
      }
    }
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Two floats to two E4M3 codes in the low 16 bits.
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(const bf16_t* __restrict__ x, int ldx, int rows,
                                                           int cols, const float* __restrict__ partial,
                                                           int nparts, uint8_t* __restrict__ q, int ldq,
                                                           float* __restrict__ scale) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < nparts; i += kThreads) m = fmaxf(m, partial[i]);
  const float amax = block_max(m, red);
  const float factor = amax > 0.f ? __fdiv_rn(448.f, amax) : 0.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int r = blockIdx.x * 4 + wave; r < rows; r += gridDim.x * 4) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(r) * ldx);
    u32x2* dst = reinterpret_cast<u32x2*>(q + static_cast<size_t>(r) * ldq);
    for (int c = lane; c < cols / 8; c += 64) {
      float f[8];
      unpack8(src[c], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fminf(fmaxf(__fmul_rn(f[i], factor), -448.f), 448.f);
      u32x2 o;
      o[0] = cvt2(f[0], f[1]) | (cvt2(f[2], f[3]) << 16);
      o[1] = cvt2(f[4], f[5]) | (cvt2(f[6], f[7]) << 16);
      dst[c] = o;
    }
  }
}

int amax_grid(int rows) { return min((rows + 3) / 4, kAmaxParts); }

}  // namespace

int amax_parts(int rows) { return rows > 0 ? amax_grid(rows) : 0; }

hipError_t launch_amax(const bf16_t* x, int ldx, int rows, int cols, float* partial, int nparts,
                       hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (cols % 8 != 0 || ldx % 8 != 0 || ldx < cols || nparts < 1 || nparts > kAmaxParts)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(amax_kernel, dim3(nparts), dim3(kThreads), 0, stream, x, ldx, rows, cols, partial);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const bf16_t* x, int ldx, int rows, int cols, const float* partial,
                               int nparts, uint8_t* q, int ldq, float* scale, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (cols % 8 != 0 || ldx % 8 != 0 || ldq % 8 != 0 || ldx < cols || ldq < cols || nparts < 1 ||
      nparts > kAmaxParts)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_kernel, dim3(amax_grid(rows)), dim3(kThreads), 0, stream, x, ldx, rows,
                     cols, partial, nparts, q, ldq, scale);
  return hipGetLastError();
}

}  // namespace mhe
