// Chunk segmentation on the GPU: uniform chunks of P tokens with a cyclic per-layer offset
// (pith.science review of "Attamba: Attending To Multi-Token States", "What carries the
// argument": cyclic chunking shifts the chunk offset by layer index), and the per-token chunk
// map for any chunk offsets (variable-length chunks as cu_seqlens, "If this is right").
#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

constexpr int kScanThreads = 1024;

// Chunks of one sequence of `len` tokens: starts at 0 and at every t = o (mod P), t < len.
__device__ __forceinline__ int chunks_of(int len, int P, int o) {
  if (len <= 0) return 0;
  if (o == 0) return ceil_div(len, P);
  if (len <= o) return 1;
  return 1 + ceil_div(len - o, P);
}

// Local start position of chunk k of a sequence.
__device__ __forceinline__ int chunk_start_local(int k, int P, int o) {
  if (k == 0) return 0;
  return o == 0 ? k * P : o + (k - 1) * P;
}

// One workgroup walks the sequences 1024 at a time: per-sequence chunk counts, a block-wide
// exclusive scan gives each sequence's first chunk index, then the whole workgroup writes the
// block's chunk starts as one flat range (each thread finds its sequence by binary search in
// LDS), so long sequences are written by all threads, not by one.
__global__ __launch_bounds__(kScanThreads) void uniform_chunk_cu_kernel(
    const int32_t* __restrict__ seq_cu, int S, int T, int P, int o, int n_chunks,
    int32_t* __restrict__ chunk_cu) {
  __shared__ int32_t s_first[kScanThreads + 1];  // first chunk index of each sequence
  __shared__ int32_t s_start[kScanThreads];      // first token of each sequence
  __shared__ int32_t s_wave[kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wid = tid / kWave;
  int carry = 0;
  for (int sb = 0; sb < S; sb += kScanThreads) {
    const int s = sb + tid;
    int cnt = 0, start = 0;
    if (s < S) {
      start = seq_cu[s];
      cnt = chunks_of(seq_cu[s + 1] - start, P, o);
    }
    // inclusive scan inside the wave, then across the 16 wave totals
    int incl = cnt;
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += v;
    }
    if (lane == kWave - 1) s_wave[wid] = incl;
    __syncthreads();
    if (wid == 0) {
      int wv = lane < kScanThreads / kWave ? s_wave[lane] : 0;
      for (int off = 1; off < kScanThreads / kWave; off <<= 1) {
        const int v = __shfl_up(wv, off, kWave);
        if (lane >= off) wv += v;
      }
      if (lane < kScanThreads / kWave) s_wave[lane] = wv;
    }
    __syncthreads();
    const int before = (wid > 0 ? s_wave[wid - 1] : 0) + incl - cnt;
    const int total = s_wave[kScanThreads / kWave - 1];
    s_first[tid] = carry + before;
    s_start[tid] = start;
    const int nseq = min(kScanThreads, S - sb);
    if (tid == 0) s_first[nseq] = carry + total;
    __syncthreads();
    for (int f = tid; f < total; f += kScanThreads) {
      const int g = carry + f;
      int lo = 0, hi = nseq;  // find j with s_first[j] <= g < s_first[j + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_first[mid] <= g) lo = mid; else hi = mid;
      }
      if (g < n_chunks) chunk_cu[g] = s_start[lo] + chunk_start_local(g - s_first[lo], P, o);
    }
    carry += total;
    __syncthreads();
  }
  for (int g = carry + tid; g <= n_chunks; g += kScanThreads) chunk_cu[g] = T;
}

// token_chunk[t] = the chunk q with chunk_cu[q] <= t < chunk_cu[q + 1];
// is_end[t] = 1 iff t is the last token of its chunk.
__global__ __launch_bounds__(256) void chunk_index_kernel(const int32_t* __restrict__ chunk_cu,
                                                          int n_chunks, int T,
                                                          int32_t* __restrict__ token_chunk,
                                                          uint8_t* __restrict__ is_end) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = n_chunks;  // invariant: chunk_cu[lo] <= t < chunk_cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_cu[mid] <= t) lo = mid; else hi = mid;
  }
  if (token_chunk) token_chunk[t] = lo;
  if (is_end) is_end[t] = (chunk_cu[lo + 1] == t + 1) ? 1 : 0;
}

// Local position tl (0 <= tl < len) starts a chunk.
__device__ __forceinline__ bool starts_chunk(int tl, int P, int o) {
  return tl == 0 || (tl >= o && (tl - o) % P == 0);
}

// Chunk of local position tl within its sequence.
__device__ __forceinline__ int chunk_of_local(int tl, int P, int o) {
  if (o == 0) return tl / P;
  return tl < o ? 0 : 1 + (tl - o) / P;
}

// The whole uniform layout in one launch, for batches of up to kFusedMaxSeq sequences: every
// workgroup scans the per-sequence chunk counts into LDS (cheap next to a launch), then
// handles kFusedTokens tokens: token -> sequence by binary search in LDS, its chunk index in
// closed form, is_end, and chunk_cu[q] = t for the tokens that start a chunk. Workgroup 0 also
// fills the entries past the last chunk with T. One token per thread: the launch is latency
// bound, so more workgroups finish sooner (16 for 16 384 tokens).
constexpr int kFusedThreads = 1024;
constexpr int kFusedTokens = 1024;
constexpr int kFusedMaxSeq = 4096;

__global__ __launch_bounds__(kFusedThreads) void uniform_layout_kernel(
    const int32_t* __restrict__ seq_cu, int S, int T, int P, int o, int n_chunks,
    int32_t* __restrict__ chunk_cu, int32_t* __restrict__ token_chunk,
    uint8_t* __restrict__ is_end) {
  __shared__ int32_t s_cu[kFusedMaxSeq + 1];      // sequence offsets
  __shared__ int32_t s_first[kFusedMaxSeq + 1];   // first chunk index of each sequence
  __shared__ int32_t s_wave[kFusedThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wid = tid / kWave;
  int carry = 0;
  for (int sb = 0; sb < S; sb += kFusedThreads) {
    const int sq = sb + tid;
    int cnt = 0;
    if (sq < S) {
      const int a = seq_cu[sq], b = seq_cu[sq + 1];
      s_cu[sq] = a;
      cnt = chunks_of(b - a, P, o);
    }
    int incl = cnt;
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += v;
    }
    if (lane == kWave - 1) s_wave[wid] = incl;
    __syncthreads();
    if (wid == 0) {
      int wv = lane < kFusedThreads / kWave ? s_wave[lane] : 0;
      for (int off = 1; off < kFusedThreads / kWave; off <<= 1) {
        const int v = __shfl_up(wv, off, kWave);
        if (lane >= off) wv += v;
      }
      if (lane < kFusedThreads / kWave) s_wave[lane] = wv;
    }
    __syncthreads();
    if (sq < S) s_first[sq] = carry + (wid > 0 ? s_wave[wid - 1] : 0) + incl - cnt;
    carry += s_wave[kFusedThreads / kWave - 1];
    __syncthreads();
  }
  if (tid == 0) {
    s_cu[S] = seq_cu[S];
    s_first[S] = carry;
  }
  __syncthreads();
  const int t0 = blockIdx.x * kFusedTokens;
  for (int t = t0 + tid; t < min(t0 + kFusedTokens, T); t += kFusedThreads) {
    int lo = 0, hi = S;  // the sequence lo whose range s_cu[lo] <= t < s_cu[lo + 1] holds t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_cu[mid] <= t) lo = mid; else hi = mid;
    }
    const int tl = t - s_cu[lo];
    const int q = s_first[lo] + chunk_of_local(tl, P, o);
    if (token_chunk) token_chunk[t] = q;
    if (is_end) is_end[t] = (t + 1 == s_cu[lo + 1] || starts_chunk(tl + 1, P, o)) ? 1 : 0;
    if (starts_chunk(tl, P, o) && q >= 0 && q < n_chunks) chunk_cu[q] = t;
  }
  if (blockIdx.x == 0)
    for (int q = carry + tid; q <= n_chunks; q += kFusedThreads) chunk_cu[q] = T;
}

}  // namespace

hipError_t launch_chunk_index(const int32_t* chunk_cu, int n_chunks, int T,
                              int32_t* token_chunk, uint8_t* is_end, hipStream_t stream) {
  if (T == 0 || n_chunks == 0 || (!token_chunk && !is_end)) return hipSuccess;
  hipLaunchKernelGGL(chunk_index_kernel, dim3(ceil_div(T, 256)), dim3(256), 0, stream, chunk_cu,
                     n_chunks, T, token_chunk, is_end);
  return hipGetLastError();
}

hipError_t launch_uniform_boundaries(const int32_t* seq_cu, int S, int T, int P, int o,
                                     int n_chunks, int32_t* chunk_cu, int32_t* token_chunk,
                                     uint8_t* is_end, hipStream_t stream) {
  if (S <= kFusedMaxSeq) {
    const int blocks = T > 0 ? ceil_div(T, kFusedTokens) : 1;
    hipLaunchKernelGGL(uniform_layout_kernel, dim3(blocks), dim3(kFusedThreads), 0, stream, seq_cu,
                       S, T, P, o, n_chunks, chunk_cu, token_chunk, is_end);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(uniform_chunk_cu_kernel, dim3(1), dim3(kScanThreads), 0, stream, seq_cu, S,
                     T, P, o, n_chunks, chunk_cu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_chunk_index(chunk_cu, n_chunks, T, token_chunk, is_end, stream);
}

}  // namespace attamba
