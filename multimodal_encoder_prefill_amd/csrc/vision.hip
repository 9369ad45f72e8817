// Vision-tower specific kernels (H3 encoder page, MiniMaxH3Qwen3VLVisionModel):
//
//  * patch_info_kernel: for every patch, in the order the tower keeps them
//    (frames, then merge x merge blocks row-major, then rows and columns
//    inside a block), its row and column in its image, the image's patch grid
//    and the [start, end) token range of its frame (the page's cu_seqlens).
//  * pos_embed_kernel: hidden += the learned position table bilinearly
//    interpolated at the patch (fast_pos_embed_interpolate; sample row
//    r (side-1)/(h-1), neighbours floor and floor+1 clipped), fp32, one
//    bf16 rounding.
//  * vision_rope_kernel: splits the biased qkv projection into q, k, v,
//    applies the 2-D rotary to q and k (cos/sin from vision_rope_table_kernel,
//    formed once per call; rot_pos_emb and
//    _apply_rotary_pos_emb_vision: angle of slot j < D/4 is row * f_j, of slot
//    D/4 + j col * f_j, f_j = 10000^(-4j/D), the D/2 angles used twice,
//    rotate-half) and writes the attention layouts with head_dim padded to
//    128 by zeros: q [n, heads, 128], k [heads, n_pad, 128] and V transposed
//    [heads, 128, n_pad] with tokens permuted inside groups of 16 as for the
//    decoder (0 1 2 3 8 9 10 11 4 5 6 7 12 13 14 15); n_pad = n rounded up to
//    128, padding tokens zero.
//
// All three are HBM- or latency-bound and small next to the tower's GEMMs.
#include "common.h"
#include "internal.h"

namespace mhe {

namespace {

__device__ __forceinline__ int perm16v(int p) {
  return (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1);
}

__global__ __launch_bounds__(256) void patch_info_kernel(VisionGrids grids, int n,
                                                         PatchInfo* __restrict__ info) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= n) return;
  const int m = grids.merge;
  int base = 0, g = 0;
  for (; g < grids.count; ++g) {
    const int cnt = grids.t[g] * grids.h[g] * grids.w[g];
    if (s < base + cnt) break;
    base += cnt;
  }
  PatchInfo pi{0, 0, 1, 1, s, s + 1, 0, 0};
  if (g < grids.count) {
    const int h = grids.h[g], w = grids.w[g], hw = h * w;
    const int li = s - base;
    const int f = li / hw, p = li % hw;
    const int blk = p / (m * m), inner = p % (m * m);
    const int br = blk / (w / m), bc = blk % (w / m);
    pi.row = br * m + inner / m;
    pi.col = bc * m + inner % m;
    pi.h = h;
    pi.w = w;
    pi.seg_lo = base + f * hw;
    pi.seg_hi = pi.seg_lo + hw;
  }
  info[s] = pi;
}

__global__ __launch_bounds__(256) void pos_embed_kernel(bf16_t* __restrict__ hidden, int ld, int n,
                                                        int dim, const bf16_t* __restrict__ table,
                                                        int side, const PatchInfo* __restrict__ info) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= n) return;
  const PatchInfo pi = info[s];
  const float y = pi.h > 1 ? static_cast<float>(pi.row) * (static_cast<float>(side - 1) / static_cast<float>(pi.h - 1)) : 0.f;
  const float x = pi.w > 1 ? static_cast<float>(pi.col) * (static_cast<float>(side - 1) / static_cast<float>(pi.w - 1)) : 0.f;
  const int y0 = static_cast<int>(y), x0 = static_cast<int>(x);
  const int y1 = min(y0 + 1, side - 1), x1 = min(x0 + 1, side - 1);
  const float dy = y - static_cast<float>(y0), dx = x - static_cast<float>(x0);
  const float w00 = (1.f - dy) * (1.f - dx), w01 = (1.f - dy) * dx, w10 = dy * (1.f - dx), w11 = dy * dx;
  const u32x4* t00 = reinterpret_cast<const u32x4*>(table + static_cast<size_t>(y0 * side + x0) * dim);
  const u32x4* t01 = reinterpret_cast<const u32x4*>(table + static_cast<size_t>(y0 * side + x1) * dim);
  const u32x4* t10 = reinterpret_cast<const u32x4*>(table + static_cast<size_t>(y1 * side + x0) * dim);
  const u32x4* t11 = reinterpret_cast<const u32x4*>(table + static_cast<size_t>(y1 * side + x1) * dim);
  u32x4* h = reinterpret_cast<u32x4*>(hidden + static_cast<size_t>(s) * ld);
  for (int c = lane; c < dim / 8; c += 64) {
    float a[8], b[8];
    unpack8(h[c], a);
    unpack8(t00[c], b);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += w00 * b[j];
    unpack8(t01[c], b);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += w01 * b[j];
    unpack8(t10[c], b);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += w10 * b[j];
    unpack8(t11[c], b);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += w11 * b[j];
    h[c] = pack8(a);
  }
}

constexpr int kVT = 16;    // tokens per workgroup
constexpr int kVD = 128;   // padded head dim of the attention layouts

// cos and sin of rotary slot j (< dh/2) of every patch, formed once per call
// (the positions are the same in every block): angle row * f_j for
// j < dh/4, col * f_(j - dh/4) above, f_i = 10000^(-2i / (dh/2))
__global__ __launch_bounds__(256) void vision_rope_table_kernel(const PatchInfo* __restrict__ info, int n,
                                                               int dh, float2* __restrict__ table) {
  const int half = dh / 2, quarter = dh / 4;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n * half) return;
  const int s = e / half, j = e % half;
  const float inv = powf(10000.f, -static_cast<float>(2 * (j % quarter)) / static_cast<float>(half));
  const PatchInfo pi = info[s];
  const float ang = static_cast<float>(j < quarter ? pi.row : pi.col) * inv;
  float sn, cs;
  sincosf(ang, &sn, &cs);
  table[e] = make_float2(cs, sn);
}

// grid (n_pad / 16, heads); one wavefront, lane l = padded head dims 2l and
// 2l + 1 (the rotate-half partner of an even dim is even: dh % 4 == 0), so
// every load and store moves a pair and the pair's two cos/sin come as one
// 16-byte table read
__global__ __launch_bounds__(64) void vision_rope_kernel(const bf16_t* __restrict__ qkv, int ldq,
                                                         int n, int n_pad, int heads, int dh,
                                                         const float2* __restrict__ table,
                                                         bf16_t* __restrict__ q_out,
                                                         bf16_t* __restrict__ k_out,
                                                         bf16_t* __restrict__ vt_out) {
  const int s0 = blockIdx.x * kVT;
  const int h = blockIdx.y;
  const int d = 2 * threadIdx.x;
  const int half = dh / 2;
  const int hid = heads * dh;
  const bool used = d < dh;
  // slot j of the D/2 angles (the angle of d and d + D/2), and the partner dim
  const int j = used ? d % half : 0;
  const int pd = d < half ? d + half : d - half;
  const float sign = d < half ? -1.f : 1.f;
  auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
  // loads from in-range addresses for every lane and token (the last patch
  // and dim 0 stand in for padding), so all of them can go out together;
  // results outside the patches or the head dims are zeroed afterwards
  const int du = used ? d : 0, pu = used ? pd : 0;
  f32x4 cs[kVT];
  uint32_t w[kVT][5];
#pragma unroll
  for (int t = 0; t < kVT; ++t) {
    const int su = min(s0 + t, n - 1);
    const bf16_t* row = qkv + static_cast<size_t>(su) * ldq + h * dh;
    cs[t] = *reinterpret_cast<const f32x4*>(table + static_cast<size_t>(su) * half + j);
    w[t][0] = *reinterpret_cast<const uint32_t*>(row + du);
    w[t][1] = *reinterpret_cast<const uint32_t*>(row + pu);
    w[t][2] = *reinterpret_cast<const uint32_t*>(row + hid + du);
    w[t][3] = *reinterpret_cast<const uint32_t*>(row + hid + pu);
    w[t][4] = *reinterpret_cast<const uint32_t*>(row + 2 * hid + du);
  }
  float va[kVT], vb[kVT];
#pragma unroll
  for (int t = 0; t < kVT; ++t) {
    const int s = s0 + t;
    const bool real = s < n && used;
    const f32x4 c4 = cs[t];
    const uint32_t qx = w[t][0], qp = w[t][1], kx = w[t][2], kp = w[t][3], vx = w[t][4];
    uint32_t qo = pack_bf16x2(lo(qx) * c4[0] + sign * lo(qp) * c4[1], hi(qx) * c4[2] + sign * hi(qp) * c4[3]);
    uint32_t ko = pack_bf16x2(lo(kx) * c4[0] + sign * lo(kp) * c4[1], hi(kx) * c4[2] + sign * hi(kp) * c4[3]);
    qo = real ? qo : 0u;
    ko = real ? ko : 0u;
    va[t] = real ? lo(vx) : 0.f;
    vb[t] = real ? hi(vx) : 0.f;
    if (s < n) *reinterpret_cast<uint32_t*>(q_out + (static_cast<size_t>(s) * heads + h) * kVD + d) = qo;
    *reinterpret_cast<uint32_t*>(k_out + (static_cast<size_t>(h) * n_pad + s) * kVD + d) = ko;
  }
  // V^T rows d and d + 1: the 16 tokens in the permuted order
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const float* vv = r ? vb : va;
    u32x4 w0, w1;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      w0[p] = pack_bf16x2(vv[perm16v(2 * p)], vv[perm16v(2 * p + 1)]);
      w1[p] = pack_bf16x2(vv[perm16v(8 + 2 * p)], vv[perm16v(8 + 2 * p + 1)]);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(vt_out + (static_cast<size_t>(h) * kVD + d + r) * n_pad + s0);
    dst[0] = w0;
    dst[1] = w1;
  }
}

}  // namespace

hipError_t launch_patch_info(const VisionGrids& grids, int n, PatchInfo* info, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(patch_info_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, grids, n, info);
  return hipGetLastError();
}

hipError_t launch_pos_embed(bf16_t* hidden, int ld, int n, int dim, const bf16_t* table, int side,
                            const PatchInfo* info, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(pos_embed_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, hidden, ld, n, dim,
                     table, side, info);
  return hipGetLastError();
}

hipError_t launch_vision_rope_table(const PatchInfo* info, int n, int head_dim, float2* table,
                                    hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (head_dim > kVD || head_dim % 4 != 0) return hipErrorInvalidValue;
  const int e = n * (head_dim / 2);
  hipLaunchKernelGGL(vision_rope_table_kernel, dim3((e + 255) / 256), dim3(256), 0, stream, info, n,
                     head_dim, table);
  return hipGetLastError();
}

hipError_t launch_vision_rope(const bf16_t* qkv, int ldq, int n, int heads, int head_dim,
                              const float2* table, bf16_t* q_out, bf16_t* k_out, bf16_t* vt_out,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (head_dim > kVD || head_dim % 4 != 0) return hipErrorInvalidValue;
  const int n_pad = seq_pad(n);
  if (ldq % 2 != 0) return hipErrorInvalidValue;  // pairs of bf16 are read as one word
  hipLaunchKernelGGL(vision_rope_kernel, dim3(n_pad / kVT, heads), dim3(kVD / 2), 0, stream, qkv, ldq,
                     n, n_pad, heads, head_dim, table, q_out, k_out, vt_out);
  return hipGetLastError();
}

}  // namespace mhe
