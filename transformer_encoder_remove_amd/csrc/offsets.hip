// Offset mask of padding removal (Kuaishou "如何让Transformer在GPU上跑得更快", Fig. 9):
// an exclusive prefix sum of the valid lengths (cu_seqlens) and, per packed token, the
// distance to its row in the padded layout (padding_offset[t] = b * max_seq - cu[b]).
#include "device.h"
#include "launch.h"

namespace tel {

constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_VEC = 4;                              // consecutive lengths per thread
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_VEC;      // lengths per tile
constexpr int SCAN_AHEAD = 4;                            // tiles loaded before any is scanned

// One workgroup scans any batch size, tile by tile: thread tid owns the SCAN_VEC
// consecutive lengths tid * SCAN_VEC .. of each tile (neighbouring threads read
// neighbouring 16-byte spans), SCAN_AHEAD tiles are requested together so the memory
// latency is paid once per SCAN_AHEAD * SCAN_TILE lengths, and each tile is scanned in
// registers (thread-local sums, wavefront shuffle scan, the 16 wave totals in LDS) on top
// of the running total of the tiles before it.
__global__ __launch_bounds__(SCAN_THREADS) void scan_lengths(const int32_t* __restrict__ lens,
                                                             int batch, int32_t* __restrict__ cu) {
  __shared__ int32_t wave_tot[SCAN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = (batch + SCAN_TILE - 1) / SCAN_TILE;
  if (tid == 0) cu[0] = 0;
  int32_t carry = 0;                                     // sum of all earlier tiles
  for (int t0 = 0; t0 < ntiles; t0 += SCAN_AHEAD) {
    int32_t v[SCAN_AHEAD][SCAN_VEC];
#pragma unroll
    for (int a = 0; a < SCAN_AHEAD; ++a)
#pragma unroll
      for (int e = 0; e < SCAN_VEC; ++e) {
        const long long i = (long long)(t0 + a) * SCAN_TILE + tid * SCAN_VEC + e;
        v[a][e] = i < batch ? lens[i] : 0;
      }
#pragma unroll
    for (int a = 0; a < SCAN_AHEAD; ++a) {
      if (t0 + a >= ntiles) break;                       // uniform across the workgroup
      int32_t inc_local[SCAN_VEC];
      int32_t run = 0;
#pragma unroll
      for (int e = 0; e < SCAN_VEC; ++e) {
        run += v[a][e];
        inc_local[e] = run;
      }
      int32_t inc = run;                                 // inclusive scan inside the wavefront
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
      }
      if (lane == 63) wave_tot[wave] = inc;
      __syncthreads();
      int32_t before = 0, tile_total = 0;
#pragma unroll
      for (int w = 0; w < SCAN_THREADS / 64; ++w) {
        const int32_t t = wave_tot[w];
        before += w < wave ? t : 0;
        tile_total += t;
      }
      const int32_t excl = carry + before + inc - run;   // lengths before this thread's first
      const long long i0 = (long long)(t0 + a) * SCAN_TILE + tid * SCAN_VEC;
#pragma unroll
      for (int e = 0; e < SCAN_VEC; ++e)
        if (i0 + e < batch) cu[i0 + e + 1] = excl + inc_local[e];
      carry += tile_total;
      __syncthreads();                                   // wave_tot is rewritten next tile
    }
  }
}

// One wavefront per sequence writes the offsets of its tokens (four sequences per
// workgroup, so a batch of many short sequences is not bound by workgroup dispatch).
constexpr int FILL_WAVES = 4;
__global__ __launch_bounds__(64 * FILL_WAVES) void fill_padding_offset(
    const int32_t* __restrict__ cu, int batch, int max_seq, int32_t* __restrict__ po) {
  const int b = blockIdx.x * FILL_WAVES + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= batch) return;
  const int32_t start = cu[b], len = cu[b + 1] - start;
  const int32_t off = b * max_seq - start;
  for (int i = lane; i < len; i += 64) po[start + i] = off;
}

// The offset mask in its general form: valid positions anywhere in a sequence (holes
// allowed), packed sequence by sequence with positions increasing. One wavefront per
// sequence (four per workgroup, so many short sequences are not bound by workgroup
// dispatch) counts its valid positions 64 at a time with a ballot; the counts are scanned
// as lengths; then one wavefront per sequence gives each valid position its packed index
// t = cu[b] + (valid positions before it) from the same ballots and writes
// padding_offset[t] = b*S + s - t.
constexpr int MASK_WAVES = 4;

// Mask bytes of one lane: W4 reads 4 consecutive positions as one 32-bit word (rows whose
// length is a multiple of 4), else one byte. nonzero_bytes marks the nonzero bytes of a word
// in their top bits (x & 0x7f7f7f7f plus 0x7f7f7f7f carries into bit 7 exactly when one of
// bits 0-6 is set; bit 7 itself is or-ed in).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
  return (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
}

template <bool W4>
__global__ __launch_bounds__(64 * MASK_WAVES) void count_mask_kernel(
    const uint8_t* __restrict__ mask, int batch, int max_seq, int32_t* __restrict__ counts) {
  const int b = blockIdx.x * MASK_WAVES + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= batch) return;
  const uint8_t* row = mask + (size_t)b * max_seq;
  int32_t c = 0;
  if constexpr (W4) {
    const uint32_t* row4 = reinterpret_cast<const uint32_t*>(row);
    for (int w0 = 0; w0 < max_seq / 4; w0 += 64) {
      const int w = w0 + lane;
      if (w < max_seq / 4) c += __popc(nonzero_bytes(row4[w]));
    }
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  } else {
    for (int s0 = 0; s0 < max_seq; s0 += 64) {
      const int s = s0 + lane;
      c += __popcll(__ballot(s < max_seq && row[s] != 0));
    }
  }
  if (lane == 0) counts[b] = c;
}

template <bool W4>
__global__ __launch_bounds__(64 * MASK_WAVES) void compact_mask_kernel(
    const uint8_t* __restrict__ mask, int batch, int max_seq, const int32_t* __restrict__ cu,
    int32_t* __restrict__ po) {
  const int b = blockIdx.x * MASK_WAVES + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= batch) return;
  const uint8_t* row = mask + (size_t)b * max_seq;
  int32_t base = cu[b];
  if constexpr (W4) {
    // each lane: 4 positions; its valid count scanned across the wavefront (shuffles)
    const uint32_t* row4 = reinterpret_cast<const uint32_t*>(row);
    for (int w0 = 0; w0 < max_seq / 4; w0 += 64) {
      const int w = w0 + lane;
      const uint32_t nz = w < max_seq / 4 ? nonzero_bytes(row4[w]) : 0u;
      const int32_t c = __popc(nz);
      int32_t inc = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
      }
      int32_t t = base + inc - c;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (nz & (0x80u << (8 * k))) {
          po[t] = b * max_seq + 4 * w + k - t;
          ++t;
        }
      base += __shfl(inc, 63, 64);
    }
  } else {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int s0 = 0; s0 < max_seq; s0 += 64) {
      const int s = s0 + lane;
      const bool valid = s < max_seq && row[s] != 0;
      const unsigned long long ballot = __ballot(valid);
      if (valid) {
        const int32_t t = base + __popcll(ballot & below);
        po[t] = b * max_seq + s - t;
      }
      base += __popcll(ballot);
    }
  }
}

hipError_t launch_offsets_mask(const uint8_t* mask, int batch, int max_seq, int32_t* cu,
                               int32_t* padding_offset, hipStream_t stream) {
  // the counts go to padding_offset[0, batch) (capacity batch * max_seq), which the
  // compaction overwrites only after the scan has read them
  const int grid = (batch + MASK_WAVES - 1) / MASK_WAVES;
  const bool w4 = max_seq % 4 == 0 && reinterpret_cast<uintptr_t>(mask) % 4 == 0;
  if (w4)
    count_mask_kernel<true><<<grid, 64 * MASK_WAVES, 0, stream>>>(mask, batch, max_seq,
                                                                   padding_offset);
  else
    count_mask_kernel<false><<<grid, 64 * MASK_WAVES, 0, stream>>>(mask, batch, max_seq,
                                                                    padding_offset);
  scan_lengths<<<1, SCAN_THREADS, 0, stream>>>(padding_offset, batch, cu);
  if (w4)
    compact_mask_kernel<true><<<grid, 64 * MASK_WAVES, 0, stream>>>(mask, batch, max_seq, cu,
                                                                     padding_offset);
  else
    compact_mask_kernel<false><<<grid, 64 * MASK_WAVES, 0, stream>>>(mask, batch, max_seq, cu,
                                                                      padding_offset);
  return hipGetLastError();
}

hipError_t launch_offsets(const int32_t* lens, int batch, int max_seq, int32_t* cu,
                          int32_t* padding_offset, hipStream_t stream) {
  scan_lengths<<<1, SCAN_THREADS, 0, stream>>>(lens, batch, cu);
  fill_padding_offset<<<(batch + FILL_WAVES - 1) / FILL_WAVES, 64 * FILL_WAVES, 0, stream>>>(
      cu, batch, max_seq, padding_offset);
  return hipGetLastError();
}

}  // namespace tel

namespace tel {

// Debug check of a forward's lengths before anything reads the padded batch: every length
// in [0, max_seq], their sum equal to total_tokens and their maximum at most max_len. One
// workgroup; out[0] receives the failed conditions as bits (0 = all hold).
__global__ __launch_bounds__(1024) void check_lengths_kernel(const int32_t* __restrict__ lens,
                                                             int batch, int max_seq,
                                                             long long total, int max_len,
                                                             int32_t* __restrict__ out) {
  __shared__ long long wsum[16];
  __shared__ int wmax[16], wbad[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long s = 0;
  int mx = 0, bad = 0;
  for (int b = tid; b < batch; b += 1024) {
    const int l = lens[b];
    bad |= (l < 0 || l > max_seq) ? 1 : 0;
    s += l;
    mx = max(mx, l);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o, 64);
    mx = max(mx, __shfl_xor(mx, o, 64));
    bad |= __shfl_xor(bad, o, 64);
  }
  if (lane == 0) {
    wsum[wave] = s;
    wmax[wave] = mx;
    wbad[wave] = bad;
  }
  __syncthreads();
  if (tid == 0) {
    long long ts = 0;
    int tm = 0, tb = 0;
    for (int w = 0; w < 16; ++w) {
      ts += wsum[w];
      tm = max(tm, wmax[w]);
      tb |= wbad[w];
    }
    out[0] = tb | (ts != total ? 2 : 0) | (tm > max_len ? 4 : 0);
  }
}

hipError_t launch_check_lengths(const int32_t* lens, int batch, int max_seq, long long total,
                                int max_len, int32_t* out, hipStream_t stream) {
  check_lengths_kernel<<<1, 1024, 0, stream>>>(lens, batch, max_seq, total, max_len, out);
  return hipGetLastError();
}

}  // namespace tel
