// DeepStack injection (H3 encoder page, MiniMaxH3Qwen3VLTextModel._deepstack_process):
// hidden[t_r] += feature[r] for the r-th visual token t_r in ascending token
// order, summed in fp32 and rounded to bf16 once. The same row kernel without
// the add is the placeholder scatter of _encode (masked_scatter).
//
// visual_index_kernel turns the uint8 mask into the ascending list of visual
// token indices with one workgroup-wide scan (run once per encode); entries
// past the mask's popcount are -1 so a short mask never sends a feature row
// out of bounds, and the popcount is written for the optional count check.
// deepstack_add_kernel is then a row gather/scatter: one wavefront per visual
// row, 16-byte coalesced loads and stores. HBM-bound: 3 * hidden * 2 bytes
// per visual row (read hidden, read feature, write hidden).
#include <mutex>
#include <vector>

#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void visual_index_kernel(const uint8_t* __restrict__ mask,
                                                                   int seq, int n_vis,
                                                                   int32_t* __restrict__ idx,
                                                                   int32_t* __restrict__ count) {
  __shared__ int warp_tot[kScanThreads / 64];
  const int tid = threadIdx.x;
  const int per = (seq + kScanThreads - 1) / kScanThreads;
  const int beg = min(tid * per, seq), end = min(beg + per, seq);
  int local = 0;
  auto set = [&](int s) { return mask[s] != 0; };
  for (int s = beg; s < end; ++s) local += set(s);
  // inclusive scan over the workgroup: within wavefronts, then across them
  const int lane = tid & 63, wave = tid >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) warp_tot[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += warp_tot[w];
  int rank = before + incl - local;  // exclusive prefix
  for (int s = beg; s < end; ++s) {
    if (set(s)) {
      if (rank < n_vis) idx[rank] = s;
      ++rank;
    }
  }
  int total = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) total += warp_tot[w];
  for (int r = total + tid; r < n_vis; r += kScanThreads) idx[r] = -1;
  if (tid == 0) *count = total;
}

// ADD: hidden[t_r] += feature[r] (fp32 sum, one bf16 rounding); otherwise
// hidden[t_r] = feature[r] (a plain copy, the placeholder scatter).
template <bool ADD>
__global__ __launch_bounds__(256) void deepstack_add_kernel(bf16_t* __restrict__ hidden, int dim,
                                                            const int32_t* __restrict__ idx,
                                                            int n_vis,
                                                            const bf16_t* __restrict__ feature) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n_vis) return;
  const int t = idx[r];
  if (t < 0) return;
  u32x4* h = reinterpret_cast<u32x4*>(hidden + static_cast<size_t>(t) * dim);
  const u32x4* f = reinterpret_cast<const u32x4*>(feature + static_cast<size_t>(r) * dim);
  for (int c = lane; c < dim / 8; c += 64) {
    if (!ADD) {
      h[c] = f[c];
      continue;
    }
    float a[8], b[8];
    unpack8(h[c], a);
    unpack8(f[c], b);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += b[j];
    h[c] = pack8(a);
  }
}

}  // namespace

// Scratch of the allocation-free DeepStack entry point: the visual index list
// (kStaticIndexRows entries) and its count, 512 KiB + 256 bytes on every GPU
// the library runs on, held until the process ends. In host code `scratch`
// names a host-side stand-in, never the device memory: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is handed to kernels.
static __device__ __align__(256) int32_t scratch[kStaticIndexRows + 64];

hipError_t static_index_scratch(int32_t** idx, int32_t** count) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<int32_t*> per_device;
  std::lock_guard<std::mutex> lk(mu);
  if (dev < 0) return hipErrorInvalidDevice;
  if (static_cast<size_t>(dev) >= per_device.size()) per_device.resize(dev + 1, nullptr);
  if (!per_device[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = static_cast<int32_t*>(p);
  }
  *idx = per_device[dev];
  *count = per_device[dev] + kStaticIndexRows;
  return hipSuccess;
}

hipError_t launch_visual_index(const uint8_t* mask, int seq, int n_vis, int32_t* idx,
                               int32_t* count, hipStream_t stream) {
  hipLaunchKernelGGL(visual_index_kernel, dim3(1), dim3(kScanThreads), 0, stream, mask, seq, n_vis,
                     idx, count);
  return hipGetLastError();
}

hipError_t launch_deepstack_add(bf16_t* hidden, int hidden_dim, const int32_t* idx, int n_vis,
                                const bf16_t* feature, hipStream_t stream) {
  if (n_vis <= 0) return hipSuccess;
  hipLaunchKernelGGL(deepstack_add_kernel<true>, dim3((n_vis + 3) / 4), dim3(256), 0, stream,
                     hidden, hidden_dim, idx, n_vis, feature);
  return hipGetLastError();
}

hipError_t launch_row_scatter(bf16_t* hidden, int hidden_dim, const int32_t* idx, int n,
                              const bf16_t* feature, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(deepstack_add_kernel<false>, dim3((n + 3) / 4), dim3(256), 0, stream, hidden,
                     hidden_dim, idx, n, feature);
  return hipGetLastError();
}

}  // namespace mhe
