// Image pseudo-tokens into the text embedding stream (DeepSeek-V4 model page,
// DeepseekV4Model.merge_image_embeddings): IMAGE positions take the aligned
// image tokens in position order; START / NEWLINE / END positions take the
// image_start / image_newline / image_end embeddings; every other position
// keeps its text embedding.  Type codes are those of vit_aligner_layout
// (START 0, IMAGE 1, NEWLINE 2, END 3; anything else is text).
//
// Three launches, deterministic, no atomics:
//   count  block g (kGroup positions): IMAGE positions in the group;
//   scan   one block: exclusive prefix of the group counts, in place, and the
//          total (optionally copied out for the caller);
//   copy   one block per position (grid-stride): the rank of an IMAGE position
//          is the group prefix plus the IMAGE positions before it inside its
//          group (one type load per thread, a block-wide count), then the row
//          is copied in 16-byte chunks.  Text rows exit after one type load.
// HBM-bound: every replaced row is read once from its source and written once.
#include "common.h"

namespace {

constexpr int kGroup = 256;  // positions per count group = threads of count/copy blocks
constexpr int kScanThreads = 1024;
constexpr int kImage = 1;
constexpr int64_t kMaxCopyBlocks = 1 << 20;

VIT_DEV int sentinel_row(int type) {  // row of the [start, newline, end] table, or -1
  return type == 0 ? 0 : type == 2 ? 1 : type == 3 ? 2 : -1;
}

__global__ __launch_bounds__(kGroup) void merge_count_kernel(const int32_t* __restrict__ types,
                                                             int64_t positions,
                                                             int32_t* __restrict__ counts) {
  const int64_t pos = (int64_t)blockIdx.x * kGroup + threadIdx.x;
  const bool img = pos < positions && types[pos] == kImage;
  const int n = __syncthreads_count(img);
  if (threadIdx.x == 0) counts[blockIdx.x] = n;
}

__global__ __launch_bounds__(kScanThreads) void merge_scan_kernel(int32_t* __restrict__ counts,
                                                                  int64_t groups,
                                                                  int32_t* __restrict__ total) {
  __shared__ int s_wave[kScanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int carry = 0;
  for (int64_t base = 0; base < groups; base += kScanThreads) {
    const int64_t i = base + threadIdx.x;
    const int v = i < groups ? counts[i] : 0;
    int x = v;  // inclusive scan inside the wave
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = 0, tile = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int c = s_wave[w];
      before += w < wave ? c : 0;
      tile += c;
    }
    if (i < groups) counts[i] = carry + before + x - v;
    carry += tile;
    __syncthreads();  // s_wave is rewritten by the next tile
  }
  if (total && threadIdx.x == 0) total[0] = carry;
}

__global__ __launch_bounds__(kGroup) void merge_copy_kernel(
    char* __restrict__ embeds, int64_t positions, int64_t row_bytes,
    const int32_t* __restrict__ types, const int32_t* __restrict__ prefix, int64_t n_tokens,
    const char* __restrict__ tokens, const char* __restrict__ sentinels) {
  for (int64_t pos = blockIdx.x; pos < positions; pos += gridDim.x) {
    const int type = types[pos];  // the same for every thread of the block
    const char* from;
    if (type == kImage) {
      const int64_t q = (pos & ~(int64_t)(kGroup - 1)) + threadIdx.x;
      const int before = __syncthreads_count(q < pos && types[q] == kImage);
      const int64_t t = (int64_t)prefix[pos / kGroup] + before;
      if (t >= n_tokens) continue;  // more IMAGE slots than tokens: left as they are
      from = tokens + t * row_bytes;
    } else {
      const int k = sentinel_row(type);
      if (k < 0) continue;
      from = sentinels + k * row_bytes;
    }
    char* to = embeds + pos * row_bytes;
    int64_t c = (int64_t)threadIdx.x * 16;
    for (; c + kGroup * 16 < row_bytes; c += 2 * kGroup * 16) {
      const u32x4 a = ld16(from + c), b = ld16(from + c + kGroup * 16);
      st16(to + c, a);
      st16(to + c + kGroup * 16, b);
    }
    if (c < row_bytes) st16(to + c, ld16(from + c));
  }
}

int64_t groups_of(int64_t positions) { return (positions + kGroup - 1) / kGroup; }

}  // namespace

size_t merge_workspace_bytes(int64_t positions) {
  const int64_t bytes = (groups_of(positions) * (int64_t)sizeof(int32_t) + 255) / 256 * 256;
  return (size_t)(bytes > 0 ? bytes : 256);
}

hipError_t launch_merge_rank(const int32_t* types, int64_t positions, int32_t* n_image, void* ws,
                             hipStream_t s) {
  const int64_t groups = groups_of(positions);
  int32_t* counts = (int32_t*)ws;
  if (groups > 0)
    merge_count_kernel<<<dim3((unsigned)groups), kGroup, 0, s>>>(types, positions, counts);
  merge_scan_kernel<<<1, kScanThreads, 0, s>>>(counts, groups, n_image);
  return hipGetLastError();
}

hipError_t launch_merge_copy(void* embeds, int64_t positions, int64_t row_bytes,
                             const int32_t* types, const void* tokens, int64_t n_tokens,
                             const void* sentinels, const void* ws, hipStream_t s) {
  if (positions == 0) return hipSuccess;
  const int64_t blocks = positions < kMaxCopyBlocks ? positions : kMaxCopyBlocks;
  merge_copy_kernel<<<dim3((unsigned)blocks), kGroup, 0, s>>>(
      (char*)embeds, positions, row_bytes, types, (const int32_t*)ws, n_tokens,
      (const char*)tokens, (const char*)sentinels);
  return hipGetLastError();
}
