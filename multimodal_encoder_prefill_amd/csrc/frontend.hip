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
//  * join_kernel: _aggregate_deepstack for a prompt with images and videos:
//    the DeepStack rows of both modalities interleaved in token order.
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

// Position of token t in the ascending index list idx[0, n) (entries past
// the mask's popcount are -1 and compare as larger than every token), or -1.
__device__ __forceinline__ int rank_of(const int32_t* __restrict__ idx, int n, int t) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int v = idx[mid];
    if (v < 0 || v >= t) hi = mid;
    else lo = mid + 1;
  }
  return (lo < n && idx[lo] == t) ? lo : -1;
}

__global__ __launch_bounds__(256) void join_kernel(const int32_t* __restrict__ vis_idx, int n_total,
                                                   const uint8_t* __restrict__ image_mask,
                                                   const int32_t* __restrict__ img_idx, int n_image,
                                                   const bf16_t* __restrict__ image_feature,
                                                   const int32_t* __restrict__ vid_idx, int n_video,
                                                   const bf16_t* __restrict__ video_feature, int dim,
                                                   bf16_t* __restrict__ joint) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n_total) return;
  const int t = vis_idx[r];
  const bf16_t* src = nullptr;
  if (t >= 0) {
    if (image_mask[t]) {
      const int i = rank_of(img_idx, n_image, t);
      if (i >= 0) src = image_feature + static_cast<size_t>(i) * dim;
    } else {
      const int v = rank_of(vid_idx, n_video, t);
      if (v >= 0) src = video_feature + static_cast<size_t>(v) * dim;
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(joint + static_cast<size_t>(r) * dim);
  for (int c = lane; c < dim / 8; c += 64)
    dst[c] = src ? reinterpret_cast<const u32x4*>(src)[c] : u32x4{0, 0, 0, 0};
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

hipError_t launch_join_visual(const int32_t* vis_idx, int n_total, const uint8_t* image_mask,
                              const int32_t* img_idx, int n_image, const bf16_t* image_feature,
                              const int32_t* vid_idx, int n_video, const bf16_t* video_feature,
                              int dim, bf16_t* joint, hipStream_t stream) {
  if (n_total <= 0) return hipSuccess;
  hipLaunchKernelGGL(join_kernel, dim3((n_total + 3) / 4), dim3(256), 0, stream, vis_idx, n_total,
                     image_mask, img_idx, n_image, image_feature, vid_idx, n_video, video_feature,
                     dim, joint);
  return hipGetLastError();
}

}  // namespace mhe
