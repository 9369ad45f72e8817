// Token-level front end of the encoder (H3 encoder page, _encode and the
// helpers it calls):
//
//  * rope_index_host: the multimodal rotary position ids of _get_rope_index /
//    _get_vision_position_ids, computed on the host from token ids and the
//    image / video patch grids, together with the per-token image, video and
//    visual masks. Host code only: the ids are a host array the caller has
//    anyway (the page reads them with .tolist()).
//  * embed_gather_kernel: embed_tokens, a row gather from the embedding table.
//    Ids outside the table's row range give zero rows, which is what the
//    page's vocab-parallel embedding does for ids outside a rank's shard.
//  * join_index_kernel + join_kernel: _aggregate_deepstack for a prompt with
//    images and videos: the DeepStack rows of both modalities interleaved in
//    token order (one scan gives every joint row its source row).
//
// The gather and the join are HBM-bound row copies: 2 * hidden * 2 bytes per
// row (read one row, write one row), 16-byte loads and stores, one wavefront
// per row.
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/mhe.h"
#include "common.h"
#include "internal.h"

namespace mhe {

int rope_index_host(const int32_t* ids, int seq, int image_token_id, int video_token_id,
                    const int32_t* image_grid, int n_images, const int32_t* video_grid,
                    int n_videos, int merge, int32_t* positions, uint8_t* image_mask,
                    uint8_t* video_mask, uint8_t* visual_mask, int32_t* delta,
                    std::string* err) {
  auto error = [&](int code, const std::string& m) {
    if (err) *err = m;
    return code;
  };
  // grids in the order runs consume them; a video of t frames is t grids of
  // one frame each
  struct Grid { int t, h, w; };
  std::vector<Grid> grids[3];
  for (int i = 0; i < n_images; ++i)
    grids[1].push_back({image_grid[3 * i], image_grid[3 * i + 1], image_grid[3 * i + 2]});
  for (int i = 0; i < n_videos; ++i)
    for (int f = 0; f < video_grid[3 * i]; ++f)
      grids[2].push_back({1, video_grid[3 * i + 1], video_grid[3 * i + 2]});
  for (int kind = 1; kind <= 2; ++kind)
    for (const Grid& g : grids[kind])
      if (g.t <= 0 || g.h <= 0 || g.w <= 0 || g.h % merge != 0 || g.w % merge != 0)
        return error(MHE_ERR_SHAPE, "grid (" + std::to_string(g.t) + ", " + std::to_string(g.h) + ", " +
                            std::to_string(g.w) + ") must be positive with h, w multiples of " +
                            std::to_string(merge));
  size_t next[3] = {0, 0, 0};
  auto type_of = [&](int s) {
    return ids[s] == image_token_id ? 1 : ids[s] == video_token_id ? 2 : 0;
  };
  int32_t* pt = positions;
  int32_t* ph = positions + seq;
  int32_t* pw = positions + 2 * static_cast<size_t>(seq);
  int64_t cur = 0, max_pos = -1;
  int s = 0;
  while (s < seq) {
    const int kind = type_of(s);
    int e = s;
    while (e < seq && type_of(e) == kind) ++e;
    const int n = e - s;
    if (kind == 0) {
      for (int i = 0; i < n; ++i) pt[s + i] = ph[s + i] = pw[s + i] = static_cast<int32_t>(cur + i);
      cur += n;
    } else {
      if (next[kind] >= grids[kind].size())
        return error(MHE_ERR_MISMATCH, std::string(kind == 1 ? "image" : "video") + " run at token " +
                                           std::to_string(s) + " has no grid left");
      const Grid g = grids[kind][next[kind]++];
      const int lh = g.h / merge, lw = g.w / merge;
      if (static_cast<int64_t>(g.t) * lh * lw != n)
        return error(MHE_ERR_MISMATCH, std::string(kind == 1 ? "image" : "video") + " run at token " +
                            std::to_string(s) + " has " + std::to_string(n) +
                            " tokens, its grid " + std::to_string(static_cast<int64_t>(g.t) * lh * lw));
      int i = s;
      for (int f = 0; f < g.t; ++f)
        for (int r = 0; r < lh; ++r)
          for (int c = 0; c < lw; ++c, ++i) {
            pt[i] = static_cast<int32_t>(cur + f);
            ph[i] = static_cast<int32_t>(cur + r);
            pw[i] = static_cast<int32_t>(cur + c);
          }
      cur += (g.h > g.w ? g.h : g.w) / merge;
    }
    for (int i = s; i < e; ++i) {
      if (image_mask) image_mask[i] = kind == 1;
      if (video_mask) video_mask[i] = kind == 2;
      if (visual_mask) visual_mask[i] = kind != 0;
      const int64_t m = pt[i] > ph[i] ? (pt[i] > pw[i] ? pt[i] : pw[i]) : (ph[i] > pw[i] ? ph[i] : pw[i]);
      if (m > max_pos) max_pos = m;
    }
    s = e;
  }
  if (delta) *delta = static_cast<int32_t>(max_pos + 1 - seq);
  return MHE_OK;
}

namespace {

__global__ __launch_bounds__(256) void embed_gather_kernel(const int32_t* __restrict__ ids, int seq,
                                                           const bf16_t* __restrict__ table,
                                                           int row_begin, int rows, int dim,
                                                           bf16_t* __restrict__ out,
                                                           int32_t* __restrict__ n_outside) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= seq) return;
  const int r = ids[s] - row_begin;
  const bool inside = r >= 0 && r < rows;
  u32x4* dst = reinterpret_cast<u32x4*>(out + static_cast<size_t>(s) * dim);
  if (inside) {
    const u32x4* src = reinterpret_cast<const u32x4*>(table + static_cast<size_t>(r) * dim);
    for (int c = lane; c < dim / 8; c += 64) dst[c] = src[c];
  } else {
    for (int c = lane; c < dim / 8; c += 64) dst[c] = u32x4{0, 0, 0, 0};
    if (lane == 0 && n_outside) atomicAdd(n_outside, 1);
  }
}

// Source row of every joint row, by one workgroup-wide scan over the tokens:
// the r-th visual token (image or video byte set) is the i-th image token or
// the v-th video token, so src[r] = i, or n_image + v, or -1 when that
// feature row does not exist (a mask with more set bytes than features).
// Rows r past the visual-token count are -1 too.
constexpr int kJoinThreads = 1024;

__device__ __forceinline__ int block_exclusive_scan(int x, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kJoinThreads / 64; ++w) {
    if (w < wave) before += wave_tot[w];
    all += wave_tot[w];
  }
  __syncthreads();  // wave_tot is reused by the next scan
  *total = all;
  return before + incl - x;
}

__global__ __launch_bounds__(kJoinThreads) void join_index_kernel(const uint8_t* __restrict__ image_mask,
                                                                 const uint8_t* __restrict__ video_mask,
                                                                 int seq, int n_total, int n_image,
                                                                 int n_video, int32_t* __restrict__ src) {
  __shared__ int wave_tot[kJoinThreads / 64];
  const int tid = threadIdx.x;
  const int per = (seq + kJoinThreads - 1) / kJoinThreads;
  const int beg = min(tid * per, seq), end = min(beg + per, seq);
  int li = 0, lv = 0;
  for (int s = beg; s < end; ++s) {
    if (image_mask[s]) ++li;
    else if (video_mask[s]) ++lv;
  }
  int ti, tv;
  int i = block_exclusive_scan(li, wave_tot, &ti);
  int v = block_exclusive_scan(lv, wave_tot, &tv);
  for (int s = beg; s < end; ++s) {
    const bool img = image_mask[s] != 0, vid = !img && video_mask[s] != 0;
    if (!img && !vid) continue;
    const int r = i + v;
    if (r < n_total) src[r] = img ? (i < n_image ? i : -1) : (v < n_video ? n_image + v : -1);
    if (img) ++i;
    else ++v;
  }
  for (int r = ti + tv + tid; r < n_total; r += kJoinThreads) src[r] = -1;
}

__global__ __launch_bounds__(256) void join_kernel(const int32_t* __restrict__ src, int n_total, int n_image,
                                                   const bf16_t* __restrict__ image_feature,
                                                   const bf16_t* __restrict__ video_feature, int dim,
                                                   bf16_t* __restrict__ joint) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n_total) return;
  const int k = src[r];
  const bf16_t* from = k < 0 ? nullptr
                       : k < n_image ? image_feature + static_cast<size_t>(k) * dim
                                     : video_feature + static_cast<size_t>(k - n_image) * dim;
  u32x4* dst = reinterpret_cast<u32x4*>(joint + static_cast<size_t>(r) * dim);
  for (int c = lane; c < dim / 8; c += 64)
    dst[c] = from ? reinterpret_cast<const u32x4*>(from)[c] : u32x4{0, 0, 0, 0};
}

}  // namespace

hipError_t launch_embed_gather(const int32_t* ids, int seq, const bf16_t* table, int row_begin,
                               int rows, int dim, bf16_t* out, int32_t* n_outside,
                               hipStream_t stream) {
  if (seq <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_gather_kernel, dim3((seq + 3) / 4), dim3(256), 0, stream, ids, seq,
                     table, row_begin, rows, dim, out, n_outside);
  return hipGetLastError();
}

hipError_t launch_join_visual(const uint8_t* image_mask, const uint8_t* video_mask, int seq,
                              int n_image, const bf16_t* image_feature, int n_video,
                              const bf16_t* video_feature, int dim, int32_t* src, bf16_t* joint,
                              hipStream_t stream) {
  const int n_total = n_image + n_video;
  if (n_total <= 0) return hipSuccess;
  hipLaunchKernelGGL(join_index_kernel, dim3(1), dim3(kJoinThreads), 0, stream, image_mask, video_mask, seq,
                     n_total, n_image, n_video, src);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(join_kernel, dim3((n_total + 3) / 4), dim3(256), 0, stream, src, n_total, n_image,
                     image_feature, video_feature, dim, joint);
  return hipGetLastError();
}

}  // namespace mhe
