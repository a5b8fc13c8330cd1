// Padding removal and rebuild (Kuaishou "如何让Transformer在GPU上跑得更快", Figs. 9-10):
// whole rows move between the padded [B*S][W] layout and the packed [T][W] layout.
// Bandwidth-bound copies: every thread moves 16-byte vectors, consecutive threads cover
// consecutive bytes of a row, so each wavefront reads and writes 1 KiB contiguous runs.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace tel {

constexpr int PAD_THREADS = 256;

__global__ __launch_bounds__(PAD_THREADS) void remove_padding_kernel(
    const u32x4* __restrict__ x_pad, u32x4* __restrict__ x_packed,
    const int32_t* __restrict__ po, int total_tokens, int vec_per_row) {
  const size_t n = (size_t)total_tokens * vec_per_row;
  for (size_t i = (size_t)blockIdx.x * PAD_THREADS + threadIdx.x; i < n;
       i += (size_t)gridDim.x * PAD_THREADS) {
    const int t = (int)(i / vec_per_row), v = (int)(i - (size_t)t * vec_per_row);
    const size_t src_row = (size_t)t + po[t];
    x_packed[i] = __builtin_nontemporal_load(&x_pad[src_row * vec_per_row + v]);
  }
}

__global__ __launch_bounds__(PAD_THREADS) void rebuild_padding_kernel(
    const u32x4* __restrict__ x_packed, u32x4* __restrict__ x_pad,
    const int32_t* __restrict__ cu, int max_seq, int batch, int vec_per_row) {
  const size_t n = (size_t)batch * max_seq * vec_per_row;
  for (size_t i = (size_t)blockIdx.x * PAD_THREADS + threadIdx.x; i < n;
       i += (size_t)gridDim.x * PAD_THREADS) {
    const size_t r = i / vec_per_row;
    const int v = (int)(i - r * vec_per_row);
    const int b = (int)(r / max_seq), p = (int)(r - (size_t)b * max_seq);
    const int32_t start = cu[b], len = cu[b + 1] - start;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (p < len) val = x_packed[(size_t)(start + p) * vec_per_row + v];
    __builtin_nontemporal_store(val, &x_pad[i]);
  }
}

// Offsets and padding removal in one launch (the start of a forward): every workgroup
// scans the lengths itself into LDS (a few dozen integers, read from L2), workgroup 0 also
// writes cu_seqlens, and each 16-byte vector of a packed row finds its sequence by binary
// search in the scanned offsets. padding_offset is not materialised: nothing after this
// kernel needs it.
constexpr int FUSED_MAX_BATCH = 1024;

__global__ __launch_bounds__(PAD_THREADS) void offsets_remove_padding_kernel(
    const int32_t* __restrict__ lens, int batch, int max_seq, int32_t* __restrict__ cu,
    const u32x4* __restrict__ x_pad, u32x4* __restrict__ x_packed, int total_tokens,
    int vec_per_row) {
  __shared__ int32_t s_cu[FUSED_MAX_BATCH + 1];
  __shared__ int32_t wave_tot[PAD_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // exclusive scan: each thread sums a contiguous chunk, chunk sums are scanned in the
  // wavefront (shuffles) and across the 4 wavefronts (LDS), then written as running sums
  const int chunk = (batch + PAD_THREADS - 1) / PAD_THREADS;
  const int b0 = min(tid * chunk, batch), b1 = min(b0 + chunk, batch);
  int32_t sum = 0;
  for (int b = b0; b < b1; ++b) sum += lens[b];
  int32_t inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int32_t run = inc - sum;
  for (int w = 0; w < wave; ++w) run += wave_tot[w];
  if (tid == 0) s_cu[0] = 0;
  for (int b = b0; b < b1; ++b) {
    run += lens[b];
    s_cu[b + 1] = run;
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int b = tid; b <= batch; b += PAD_THREADS) cu[b] = s_cu[b];
  const size_t n = (size_t)total_tokens * vec_per_row;
  for (size_t i = (size_t)blockIdx.x * PAD_THREADS + tid; i < n;
       i += (size_t)gridDim.x * PAD_THREADS) {
    const int t = (int)(i / vec_per_row), v = (int)(i - (size_t)t * vec_per_row);
    int lo = 0, hi = batch;                 // largest b with s_cu[b] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_cu[mid] <= t) lo = mid;
      else hi = mid;
    }
    const size_t src_row = (size_t)lo * max_seq + (t - s_cu[lo]);
    x_packed[i] = __builtin_nontemporal_load(&x_pad[src_row * vec_per_row + v]);
  }
}

// Rebuild for any offsets (the mask form, holes allowed): rows the mask marks invalid
// are zeroed, then every packed row t is written to padded row t + padding_offset[t].
__global__ __launch_bounds__(PAD_THREADS) void zero_masked_rows_kernel(
    const uint8_t* __restrict__ mask, u32x4* __restrict__ x_pad, size_t rows, int vec_per_row) {
  const size_t n = rows * vec_per_row;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * PAD_THREADS + threadIdx.x; i < n;
       i += (size_t)gridDim.x * PAD_THREADS)
    if (mask[i / vec_per_row] == 0) __builtin_nontemporal_store(zero, &x_pad[i]);
}

__global__ __launch_bounds__(PAD_THREADS) void scatter_rows_kernel(
    const u32x4* __restrict__ x_packed, u32x4* __restrict__ x_pad,
    const int32_t* __restrict__ po, int total_tokens, int vec_per_row) {
  const size_t n = (size_t)total_tokens * vec_per_row;
  for (size_t i = (size_t)blockIdx.x * PAD_THREADS + threadIdx.x; i < n;
       i += (size_t)gridDim.x * PAD_THREADS) {
    const int t = (int)(i / vec_per_row), v = (int)(i - (size_t)t * vec_per_row);
    const size_t dst_row = (size_t)t + po[t];
    __builtin_nontemporal_store(x_packed[i], &x_pad[dst_row * vec_per_row + v]);
  }
}

static int grid_for(size_t n) {
  size_t blocks = (n + PAD_THREADS - 1) / PAD_THREADS;
  const size_t cap = 256 * 32;   // enough waves to fill 256 CUs; the loop covers the rest
  if (blocks > cap) blocks = cap;
  return (int)(blocks == 0 ? 1 : blocks);
}

hipError_t launch_remove_padding(const void* x_pad, void* x_packed, const int32_t* po,
                                 int total_tokens, int row_bytes, hipStream_t stream) {
  const int vpr = row_bytes / 16;
  const size_t n = (size_t)total_tokens * vpr;
  if (n == 0) return hipSuccess;
  remove_padding_kernel<<<grid_for(n), PAD_THREADS, 0, stream>>>(
      (const u32x4*)x_pad, (u32x4*)x_packed, po, total_tokens, vpr);
  return hipGetLastError();
}

hipError_t launch_rebuild_padding(const void* x_packed, void* x_pad, const int32_t* cu, int batch,
                                  int max_seq, int row_bytes, hipStream_t stream) {
  const int vpr = row_bytes / 16;
  const size_t n = (size_t)batch * max_seq * vpr;
  if (n == 0) return hipSuccess;
  rebuild_padding_kernel<<<grid_for(n), PAD_THREADS, 0, stream>>>(
      (const u32x4*)x_packed, (u32x4*)x_pad, cu, max_seq, batch, vpr);
  return hipGetLastError();
}

hipError_t launch_rebuild_padding_mask(const void* x_packed, void* x_pad, const uint8_t* mask,
                                       const int32_t* po, int total_tokens, int batch,
                                       int max_seq, int row_bytes, hipStream_t stream) {
  const int vpr = row_bytes / 16;
  const size_t rows = (size_t)batch * max_seq, nz = rows * vpr;
  if (nz == 0) return hipSuccess;
  zero_masked_rows_kernel<<<grid_for(nz), PAD_THREADS, 0, stream>>>(mask, (u32x4*)x_pad, rows,
                                                                     vpr);
  const size_t ns = (size_t)total_tokens * vpr;
  if (ns > 0)
    scatter_rows_kernel<<<grid_for(ns), PAD_THREADS, 0, stream>>>(
        (const u32x4*)x_packed, (u32x4*)x_pad, po, total_tokens, vpr);
  return hipGetLastError();
}

hipError_t launch_offsets_remove_padding(const int32_t* lens, int batch, int max_seq,
                                        int32_t* cu, const void* x_pad, void* x_packed,
                                        int total_tokens, int row_bytes, hipStream_t stream) {
  if (batch <= 0 || batch > FUSED_MAX_BATCH) return hipErrorInvalidValue;
  const int vpr = row_bytes / 16;
  const size_t n = (size_t)total_tokens * vpr;
  const int grid = std::min(grid_for(n), 1024);   // at least one workgroup: it writes cu
  offsets_remove_padding_kernel<<<grid, PAD_THREADS, 0, stream>>>(
      lens, batch, max_seq, cu, (const u32x4*)x_pad, (u32x4*)x_packed, total_tokens, vpr);
  return hipGetLastError();
}

}  // namespace tel
