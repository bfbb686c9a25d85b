// KV-SSM: the two selective scans SSM_K and SSM_V that replace the key and value projections
// and compress each chunk into one boundary state (pith.science review of "Attamba: Attending
// To Multi-Token States", "Core claim"; the selective SSM is the paper's Eq. 3, cited in
// "Assumptions & free parameters").
//
// Mapping on gfx950: a wave runs ONE of the two SSMs over 64 consecutive channels and a group
// of whole chunks (chunks are independent because the state restarts at every chunk start).
// The K and V waves of the same channels and chunks are launched next to each other on the
// same XCD, so the input x that both read comes from HBM once. One lane owns one channel and
// keeps its N state values and N decay rates (A * log2 e) in VGPRs. All lanes of a wave sit on
// the same token, so the per-token rows bm/cm (shared by all channels) are wave-uniform: they
// are read through the constant address space as scalar loads, widened to float32 on the
// scalar unit and enter the VALU instructions as SGPR operands. Per state and token the work
// is one multiply for the exponent, one v_exp_f32, one multiply for the input term, one FMA
// for the state and one FMA for the output; this instruction stream, not HBM, bounds the
// kernel.
// One SSM per wave (rather than both) halves the scalar registers a token's rows need, which
// leaves room to request the next token's rows before the current token's arithmetic, and
// halves the vector registers per lane (72: 7 waves per SIMD to hide latency).
// Chunks of the common length PU are processed fully unrolled: all x/dt loads of the chunk are
// issued at its start, and no state value is carried across a loop back-edge (it restarts at
// the next chunk anyway), so no register copies are needed. Other chunk lengths (random
// chunking, a partial first or last chunk) run in blocks of up to PU tokens with the same
// loads up front and the same one-token row prefetch.
// The Mamba-block variant (BLK) adds, per lane, a causal depthwise convolution of up to 4 taps
// with SiLU on the scan's input and a SiLU gate on its output. The convolution restarts at every
// chunk start like the state, so it needs no tokens from before the chunk: each lane keeps the
// last three inputs of its channel as a window that restarts at zero with every chunk.
#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

// Waves the chip holds at once at this kernel's occupancy (256 CUs x 4 SIMDs x 7 waves). A wave
// walks two chunks (CPW = 2) when the grid then still spans at least 9 such rounds; otherwise
// one, so that smaller grids end with a shorter last round.
constexpr int kResidentWaves = 256 * 4 * 7;
constexpr int kRoundsForTwoChunks = 9;

struct ScanShape {
  int T, d, n_chunks, S;
  int groups;          // chunk groups = ceil(n_chunks / chunks per wave)
  int ctiles;          // channel tiles = d / 64
};

// The operands of one SSM.
template <typename T>
struct SideArgs {
  const T* x;          // input (SSM_V may read its own)
  const T* dt;
  const T* bm;
  const T* cm;
  const float* A;
  const float* D;
  const float* bias;
  T* y;
  T* b;                // boundary outputs or null
  float* h_last;       // hand-off states or null
  // Mamba-block pieces (read only by the BLK instances)
  int conv_width;      // 0: no convolution
  const float* conv_w; // [d, conv_width]
  const float* conv_b; // [d]
  const T* z;          // [T, d] gate input or null
};

// The convolution taps of one lane, right-aligned in 4 slots (w4[3] weighs the current token,
// slots before the first tap are zero), and its bias.
struct ConvLane {
  float w4[4];
  float b;
  __device__ __forceinline__ void load(const float* __restrict__ w, const float* __restrict__ bias,
                                       int K, int c) {
#pragma unroll
    for (int k = 0; k < 4; ++k) w4[k] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < K) w4[4 - K + k] = w[c * K + k];
    b = bias[c];
  }
  // silu of the convolution at the current token xr, whose three predecessors in the chunk are
  // win[0..2] (win[0] the oldest; zero before the chunk start); then xr joins the window
  __device__ __forceinline__ float next(float (&win)[3], float xr) const {
    float acc = fmaf(w4[0], win[0], b);
    acc = fmaf(w4[1], win[1], acc);
    acc = fmaf(w4[2], win[2], acc);
    acc = fmaf(w4[3], xr, acc);
    win[0] = win[1];
    win[1] = win[2];
    win[2] = xr;
    return silu_f32(acc);
  }
};

// Workgroup id -> (SSM, chunk group, channel tile). Workgroups are dispatched round-robin over
// the 8 XCDs (id mod 8), each with its own L2; every channel tile and both SSMs of one chunk
// group are placed on the same XCD, so the group's x and bm/cm rows are fetched from HBM once
// per XCD, and the K and V waves of one tile are consecutive on that XCD.
__device__ __forceinline__ bool map_block(const ScanShape& sh, int& side, int& group,
                                          int& ctile) {
  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  side = slot & 1;
  const int tile = slot >> 1;
  group = (tile / sh.ctiles) * 8 + xcd;
  ctile = tile % sh.ctiles;
  return group < sh.groups;
}

template <typename T, int N>
struct SsmLane {
  float A2[N];   // A[c, n] * log2(e)
  float h[N];
  float D, bias;

  __device__ __forceinline__ void load_params(const float* __restrict__ A,
                                              const float* __restrict__ Dp,
                                              const float* __restrict__ bp, int c) {
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = A[c * N + n] * kLog2e;
    D = Dp[c];
    bias = bp[c];
  }

  // The raw 32-bit words of one token's bm and cm rows (bf16 pairs or float32 values).
  static constexpr int W = sizeof(T) == 2 ? N / 2 : N;
  struct Rows {
    uint32_t b[W], c[W];
  };

  // Wave-uniform rows, read as 32-bit words through the constant address space: the rows are
  // never written while the kernel runs, and uniform constant loads become scalar loads.
  static __device__ __forceinline__ void load_rows(const T* bm, const T* cm, Rows& r) {
    using cptr = const __attribute__((address_space(4))) uint32_t*;
    const cptr wb = (cptr)(bm);
    const cptr wc = (cptr)(cm);
#pragma unroll
    for (int i = 0; i < W; ++i) {
      r.b[i] = wb[i];
      r.c[i] = wc[i];
    }
  }

  // state n of a row as float32 (bf16 pairs are split with shifts on the scalar unit)
  static __device__ __forceinline__ float widen(const uint32_t (&w)[W], int n) {
    if constexpr (sizeof(T) == 2)
      return __uint_as_float((n & 1) ? (w[n >> 1] & 0xffff0000u) : (w[n >> 1] << 16));
    else
      return __uint_as_float(w[n]);
  }

  // One token. FIRST: the state restarts (no decay term). The output sum runs in two halves
  // to shorten its dependency chain.
  template <bool FIRST>
  __device__ __forceinline__ float step(float x, float dt, const Rows& r) {
    const float delta = softplus_f32(dt + bias);
    const float u = delta * x;
    float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float inj = u * widen(r.b, n);
      if (FIRST) {
        h[n] = inj;
      } else {
        h[n] = fmaf(hw_exp2(delta * A2[n]), h[n], inj);
      }
      if (n & 1) y1 = fmaf(h[n], widen(r.c, n), y1);
      else y0 = fmaf(h[n], widen(r.c, n), y0);
    }
    return fmaf(D, x, y0 + y1);
  }
};

// Keeps the scalar loads of the next token's rows above the current token's arithmetic (the
// scheduler would otherwise sink them to their first use and expose their latency).
__device__ __forceinline__ void order_point() { __builtin_amdgcn_sched_barrier(0); }

// Waits for the current token's rows before the next token's are requested: scalar loads
// return out of order, so any later wait for them would also wait for the newer requests.
__device__ __forceinline__ void rows_ready(uint32_t b0, uint32_t c0) {
  asm volatile("" ::"s"(b0), "s"(c0));
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T, int N, int PU, int CPW, bool BLK>
// bf16 with N = 16 (the common case) is held to 7 waves per SIMD (65 VGPRs; 8 waves at 64 VGPRs
// measured the same), and its Mamba-block instance to 5 (96 VGPRs and a 52-byte spill instead of
// 124 VGPRs at 4 waves: 315 us against 340 us at the prefill shape); the other instances are
// left unconstrained.
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(N == 16 && sizeof(T) == 2 ? (BLK ? 5 : 7) : 1))) void kvssm_scan_kernel(
    ScanShape sh, const int32_t* __restrict__ chunk_cu, const int32_t* __restrict__ seq_cu,
    SideArgs<T> ka, SideArgs<T> va) {
  int side, group, ctile;
  if (!map_block(sh, side, group, ctile)) return;
  const SideArgs<T> a = side ? va : ka;
  const T* __restrict__ bm = a.bm;
  const T* __restrict__ cm = a.cm;
  // bf16 x, dt, y through buffer resources (174 against 177 us at the prefill shape); the
  // Mamba-block instance keeps plain pointers (375 against 305-322 us with buffer accesses)
  constexpr bool kBuf = sizeof(T) == 2 && !BLK;
  Column<T, kBuf> x, dt, y, z;
  x.init(a.x, sh.T, sh.d);
  dt.init(a.dt, sh.T, sh.d);
  y.init(a.y, sh.T, sh.d);
  if (BLK && a.z) z.init(a.z, sh.T, sh.d);
  const int lane = threadIdx.x;
  const int c = ctile * kWave + lane;
  const int d = sh.d;
  const int q0 = group * CPW;
  const int q1 = min(q0 + CPW, sh.n_chunks);

  SsmLane<T, N> s;
  s.load_params(a.A, a.D, a.bias, c);
  ConvLane cv{};
  const bool conv = BLK && a.conv_width > 0;
  const bool gated = BLK && a.z != nullptr;
  if (conv) cv.load(a.conv_w, a.conv_b, a.conv_width, c);

  // end of chunk q: boundary state and, for the last chunk of a sequence, the hand-off state
  auto chunk_end = [&](int q, int cs, int ce, float out) {
    if (a.b) a.b[q * d + c] = from_f32<T>(out);
    if (a.h_last) {
      int lo = 0, hi = sh.S;        // sequence s with seq_cu[s] <= cs < seq_cu[s + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seq_cu[mid] <= cs) lo = mid; else hi = mid;
      }
      if (seq_cu[lo + 1] == ce) {
        float* hp = a.h_last + (static_cast<size_t>(lo) * d + c) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) hp[n] = s.h[n];
      }
    }
  };

  int cs = chunk_cu[q0];
  for (int q = q0; q < q1; ++q) {
    const int ce = chunk_cu[q + 1];
    float out = 0.f;
    if (ce - cs == PU) {
      float xs[PU], dts[PU], zs[PU];
#pragma unroll
      for (int j = 0; j < PU; ++j) {
        const int rd = (cs + j) * d;
        xs[j] = x.load(rd, c);
        dts[j] = dt.load(rd, c);
        if (gated) zs[j] = z.load(rd, c);
      }
      float win[3] = {0.f, 0.f, 0.f};   // the chunk starts here: nothing before it counts
      typename SsmLane<T, N>::Rows rn, rc;
      SsmLane<T, N>::load_rows(bm + cs * N, cm + cs * N, rn);
#pragma unroll
      for (int j = 0; j < PU; ++j) {
        const int t = cs + j;
        rc = rn;
        rows_ready(rc.b[0], rc.c[0]);
        if (j + 1 < PU) SsmLane<T, N>::load_rows(bm + (t + 1) * N, cm + (t + 1) * N, rn);
        order_point();
        const float xin = conv ? cv.next(win, xs[j]) : xs[j];
        if (j == 0) out = s.template step<true>(xin, dts[j], rc);
        else out = s.template step<false>(xin, dts[j], rc);
        if (gated) out *= silu_f32(zs[j]);
        y.store(out, t * d, c);
      }
    } else {
      // any other length: blocks of up to PU tokens, each with its x/dt loads issued up front
      // (the state runs on across the blocks of a chunk)
      float win[3] = {0.f, 0.f, 0.f};   // the last three inputs (chunk start: 0)
      for (int bs = cs; bs < ce; bs += PU) {
        const int nb = min(PU, ce - bs);
        float xs[PU], dts[PU], zs[PU];
#pragma unroll
        for (int j = 0; j < PU; ++j) {   // past the block's end: its last token again (unused)
          const int rd = (bs + min(j, nb - 1)) * d;
          xs[j] = x.load(rd, c);
          dts[j] = dt.load(rd, c);
          if (gated) zs[j] = z.load(rd, c);
        }
        // two row sets used in turn (token j reads set j & 1 and requests the next token's
        // rows into the other): with the per-token guards, copying one set into the other
        // would cost 16 scalar moves per token
        typename SsmLane<T, N>::Rows rr[2];
        SsmLane<T, N>::load_rows(bm + bs * N, cm + bs * N, rr[0]);
#pragma unroll
        for (int j = 0; j < PU; ++j) {
          if (j < nb) {
            const int t = bs + j;
            const typename SsmLane<T, N>::Rows& rc = rr[j & 1];
            rows_ready(rc.b[0], rc.c[0]);
            if (j + 1 < nb) SsmLane<T, N>::load_rows(bm + (t + 1) * N, cm + (t + 1) * N, rr[(j + 1) & 1]);
            order_point();
            const float xin = conv ? cv.next(win, xs[j]) : xs[j];
            if (j == 0 && bs == cs) out = s.template step<true>(xin, dts[j], rc);
            else out = s.template step<false>(xin, dts[j], rc);
            if (gated) out *= silu_f32(zs[j]);
            y.store(out, t * d, c);
          }
        }
      }
    }
    chunk_end(q, cs, ce, out);
    cs = ce;
  }
}

template <typename T, int N, bool BLK>
hipError_t launch_typed(const attamba_scan_args& a, const ScanShape& sh, int cpw,
                        hipStream_t stream) {
  const int blocks = ceil_div(sh.groups, 8) * 8 * sh.ctiles * 2;
  const attamba_ssm_block_args* bl = a.block;
  SideArgs<T> k{static_cast<const T*>(a.x), static_cast<const T*>(a.dt_k),
                static_cast<const T*>(a.bm_k), static_cast<const T*>(a.cm_k), a.A_k, a.D_k,
                a.bias_k, static_cast<T*>(a.y_k), static_cast<T*>(a.kb), a.h_last_k,
                bl ? bl->conv_width : 0, bl ? bl->conv_w_k : nullptr, bl ? bl->conv_b_k : nullptr,
                bl ? static_cast<const T*>(bl->z_k) : nullptr};
  SideArgs<T> v{static_cast<const T*>(a.x_v ? a.x_v : a.x), static_cast<const T*>(a.dt_v),
                static_cast<const T*>(a.bm_v), static_cast<const T*>(a.cm_v), a.A_v, a.D_v,
                a.bias_v, static_cast<T*>(a.y_v), static_cast<T*>(a.vb), a.h_last_v,
                bl ? bl->conv_width : 0, bl ? bl->conv_w_v : nullptr, bl ? bl->conv_b_v : nullptr,
                bl ? static_cast<const T*>(bl->z_v) : nullptr};
  if (cpw == 2)
    hipLaunchKernelGGL((kvssm_scan_kernel<T, N, 8, 2, BLK>), dim3(blocks), dim3(kWave), 0, stream, sh,
                       a.chunk_cu, a.seq_cu, k, v);
  else
    hipLaunchKernelGGL((kvssm_scan_kernel<T, N, 8, 1, BLK>), dim3(blocks), dim3(kWave), 0, stream, sh,
                       a.chunk_cu, a.seq_cu, k, v);
  return hipGetLastError();
}

template <typename T, int N>
hipError_t launch_blk(const attamba_scan_args& a, const ScanShape& sh, int cpw, hipStream_t stream) {
  const bool blk = a.block && (a.block->conv_width > 0 || a.block->z_k);
  return blk ? launch_typed<T, N, true>(a, sh, cpw, stream) : launch_typed<T, N, false>(a, sh, cpw, stream);
}

}  // namespace

hipError_t launch_kvssm_scan(const attamba_scan_args& a, hipStream_t stream) {
  if (a.n_chunks == 0 || a.T == 0) return hipSuccess;
  ScanShape sh;
  sh.T = a.T; sh.d = a.d; sh.n_chunks = a.n_chunks; sh.S = a.S;
  sh.ctiles = a.d / kWave;
  const long waves2 = static_cast<long>(ceil_div(ceil_div(a.n_chunks, 2), 8)) * 8 * sh.ctiles * 2;
  const int cpw = waves2 >= static_cast<long>(kRoundsForTwoChunks) * kResidentWaves ? 2 : 1;
  sh.groups = ceil_div(a.n_chunks, cpw);
  if (a.dtype == ATTAMBA_BF16)
    return a.N == 16 ? launch_blk<__bf16, 16>(a, sh, cpw, stream) : launch_blk<__bf16, 32>(a, sh, cpw, stream);
  return a.N == 16 ? launch_blk<float, 16>(a, sh, cpw, stream) : launch_blk<float, 32>(a, sh, cpw, stream);
}

}  // namespace attamba
