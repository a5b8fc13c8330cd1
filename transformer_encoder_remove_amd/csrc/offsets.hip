// Offset mask of padding removal (Kuaishou "如何让Transformer在GPU上跑得更快", Fig. 9):
// an exclusive prefix sum of the valid lengths (cu_seqlens) and, per packed token, the
// distance to its row in the padded layout (padding_offset[t] = b * max_seq - cu[b]).
#include "device.h"
#include "launch.h"

namespace tel {

constexpr int SCAN_THREADS = 1024;

// One workgroup scans any batch size: each thread sums a contiguous chunk, the chunk
// sums are scanned across the workgroup (wavefront shuffles, then the 16 wave totals),
// and each thread rewrites its chunk as running sums.
__global__ __launch_bounds__(SCAN_THREADS) void scan_lengths(const int32_t* __restrict__ lens,
                                                             int batch, int32_t* __restrict__ cu) {
  __shared__ int32_t wave_tot[SCAN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = (batch + SCAN_THREADS - 1) / SCAN_THREADS;
  const int b0 = min(tid * chunk, batch), b1 = min(b0 + chunk, batch);
  int32_t s = 0;
  for (int b = b0; b < b1; ++b) s += lens[b];
  // inclusive scan inside the wavefront
  int32_t inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int32_t v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  int32_t run = before + inc - s;   // exclusive prefix of this thread's chunk
  if (tid == 0) cu[0] = 0;
  for (int b = b0; b < b1; ++b) {
    run += lens[b];
    cu[b + 1] = run;
  }
}

// One workgroup per sequence writes the offsets of its tokens.
__global__ __launch_bounds__(256) void fill_padding_offset(const int32_t* __restrict__ cu, int max_seq,
                                                           int32_t* __restrict__ po) {
  const int b = blockIdx.x;
  const int32_t start = cu[b], len = cu[b + 1] - start;
  const int32_t off = b * max_seq - start;
  for (int i = threadIdx.x; i < len; i += blockDim.x) po[start + i] = off;
}

hipError_t launch_offsets(const int32_t* lens, int batch, int max_seq, int32_t* cu,
                          int32_t* padding_offset, hipStream_t stream) {
  scan_lengths<<<1, SCAN_THREADS, 0, stream>>>(lens, batch, cu);
  fill_padding_offset<<<batch, 256, 0, stream>>>(cu, max_seq, padding_offset);
  return hipGetLastError();
}

}  // namespace tel
