// KV-SSM: the two selective scans SSM_K and SSM_V that replace the key and value projections
// and compress each chunk into one boundary state (pith.science review of "Attamba: Attending
// To Multi-Token States", "Core claim"; the selective SSM is the paper's Eq. 3, cited in
// "Assumptions & free parameters").
//
// SSM_V may read its own input (the variant that keeps explicit key and value projections in
// front of the SSMs); by default both SSMs read x, loaded once.
//
// Mapping on gfx950: one lane owns one channel c of both SSMs and keeps the 2*N state values
// and the 2*N decay rates (A * log2 e) in VGPRs; a wave owns 64 consecutive channels and walks
// a group of whole chunks token by token (chunks are independent because the state restarts
// at every chunk start). All lanes of a wave sit on the same token, so the per-token rows
// bm/cm (shared by all channels) are wave-uniform: the pointers are restrict-qualified kernel
// arguments, so they are fetched with scalar loads, widened to float32 on the scalar unit and
// enter the VALU instructions as SGPR operands. Per state and token the work is one multiply
// for the exponent, one v_exp_f32, one multiply for the input term, one FMA for the state and
// one FMA for the output; this instruction stream, not HBM, bounds the kernel.
// Chunks of the common length PU are processed fully unrolled: all x/dt loads of the chunk are
// issued at its start, and no state value is carried across a loop back-edge (it restarts at
// the next chunk anyway), so no register copies are needed. Other chunk lengths (random
// chunking, a partial first or last chunk) take a token loop.
#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

constexpr int kChunksPerWave = 8;

struct ScanShape {
  int T, d, n_chunks, S;
  int groups;          // chunk groups = ceil(n_chunks / kChunksPerWave)
  int ctiles;          // channel tiles = d / 64
};

// Workgroup id -> (chunk group, channel tile). Workgroups are dispatched round-robin over
// the 8 XCDs (id mod 8), each with its own L2; every channel tile of one chunk group is
// placed on the same XCD so the group's bm/cm rows are fetched from HBM once per XCD.
__device__ __forceinline__ bool map_block(const ScanShape& sh, int& group, int& ctile) {
  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  group = (slot / sh.ctiles) * 8 + xcd;
  ctile = slot % sh.ctiles;
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

  // One token. FIRST: the state restarts (no decay term). bm/cm point at the token's rows.
  // The output sum runs in two halves to shorten its dependency chain.
  template <bool FIRST>
  __device__ __forceinline__ float step(float x, float dt, const T* __restrict__ bm,
                                        const T* __restrict__ cm) {
    float b[N], cc[N];
    load_row(bm, b);
    load_row(cm, cc);
    const float delta = softplus_f32(dt + bias);
    const float u = delta * x;
    float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float inj = u * b[n];
      if (FIRST) {
        h[n] = inj;
      } else {
        h[n] = fmaf(hw_exp2(delta * A2[n]), h[n], inj);
      }
      if (n & 1) y1 = fmaf(h[n], cc[n], y1);
      else y0 = fmaf(h[n], cc[n], y0);
    }
    return fmaf(D, x, y0 + y1);
  }

  // A wave-uniform row of N values, read as 32-bit words so that the compiler issues scalar
  // loads (bf16 pairs are split with shifts on the scalar unit).
  static __device__ __forceinline__ void load_row(const T* __restrict__ row, float (&v)[N]) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(row);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int n = 0; n < N / 2; ++n) {
        const uint32_t p = w[n];
        v[2 * n] = __uint_as_float(p << 16);
        v[2 * n + 1] = __uint_as_float(p & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) v[n] = __uint_as_float(w[n]);
    }
  }
};

// SEPX: SSM_V reads its own input xv (explicit key/value projections in front of the SSMs).
template <typename T, int N, int PU, bool SEPX>
__global__ __launch_bounds__(kWave) void kvssm_scan_kernel(
    ScanShape sh, const int32_t* __restrict__ chunk_cu, const T* __restrict__ x,
    const T* __restrict__ xv,
    const T* __restrict__ dtk, const T* __restrict__ dtv, const T* __restrict__ bmk,
    const T* __restrict__ cmk, const T* __restrict__ bmv, const T* __restrict__ cmv,
    const float* __restrict__ A_k, const float* __restrict__ A_v, const float* __restrict__ D_k,
    const float* __restrict__ D_v, const float* __restrict__ bias_k,
    const float* __restrict__ bias_v, T* __restrict__ yk, T* __restrict__ yv,
    T* __restrict__ kb, T* __restrict__ vb, const int32_t* __restrict__ seq_cu,
    float* __restrict__ h_last_k, float* __restrict__ h_last_v) {
  int group, ctile;
  if (!map_block(sh, group, ctile)) return;
  const int lane = threadIdx.x;
  const int c = ctile * kWave + lane;
  const int d = sh.d;
  const int q0 = group * kChunksPerWave;
  const int q1 = min(q0 + kChunksPerWave, sh.n_chunks);

  SsmLane<T, N> sk, sv;
  sk.load_params(A_k, D_k, bias_k, c);
  sv.load_params(A_v, D_v, bias_v, c);

  // end of chunk q: boundary state and, for the last chunk of a sequence, the hand-off state
  auto chunk_end = [&](int q, int cs, int ce, float ok, float ov) {
    if (kb) {
      kb[q * d + c] = from_f32<T>(ok);
      vb[q * d + c] = from_f32<T>(ov);
    }
    if (h_last_k) {
      int lo = 0, hi = sh.S;        // sequence s with seq_cu[s] <= cs < seq_cu[s + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seq_cu[mid] <= cs) lo = mid; else hi = mid;
      }
      if (seq_cu[lo + 1] == ce) {
        float* hk = h_last_k + (static_cast<size_t>(lo) * d + c) * N;
        float* hv = h_last_v + (static_cast<size_t>(lo) * d + c) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) { hk[n] = sk.h[n]; hv[n] = sv.h[n]; }
      }
    }
  };

  int cs = chunk_cu[q0];
  for (int q = q0; q < q1; ++q) {
    const int ce = chunk_cu[q + 1];
    float ok = 0.f, ov = 0.f;
    if (ce - cs == PU) {
      float xs[PU], xvs[PU], dks[PU], dvs[PU];
#pragma unroll
      for (int j = 0; j < PU; ++j) {
        const int o = (cs + j) * d + c;
        xs[j] = to_f32(x[o]); dks[j] = to_f32(dtk[o]); dvs[j] = to_f32(dtv[o]);
        xvs[j] = SEPX ? to_f32(xv[o]) : xs[j];
      }
#pragma unroll
      for (int j = 0; j < PU; ++j) {
        const int t = cs + j;
        if (j == 0) {
          ok = sk.template step<true>(xs[j], dks[j], bmk + t * N, cmk + t * N);
          ov = sv.template step<true>(xvs[j], dvs[j], bmv + t * N, cmv + t * N);
        } else {
          ok = sk.template step<false>(xs[j], dks[j], bmk + t * N, cmk + t * N);
          ov = sv.template step<false>(xvs[j], dvs[j], bmv + t * N, cmv + t * N);
        }
        yk[t * d + c] = from_f32<T>(ok);
        yv[t * d + c] = from_f32<T>(ov);
      }
    } else {
      float nx = to_f32(x[cs * d + c]), ndk = to_f32(dtk[cs * d + c]), ndv = to_f32(dtv[cs * d + c]);
      float nxv = SEPX ? to_f32(xv[cs * d + c]) : nx;
      for (int t = cs; t < ce; ++t) {
        const float xk_t = nx, xv_t = nxv, dk = ndk, dv = ndv;
        if (t + 1 < ce) {
          const int o = (t + 1) * d + c;
          nx = to_f32(x[o]); ndk = to_f32(dtk[o]); ndv = to_f32(dtv[o]);
          nxv = SEPX ? to_f32(xv[o]) : nx;
        }
        if (t == cs) {
          ok = sk.template step<true>(xk_t, dk, bmk + t * N, cmk + t * N);
          ov = sv.template step<true>(xv_t, dv, bmv + t * N, cmv + t * N);
        } else {
          ok = sk.template step<false>(xk_t, dk, bmk + t * N, cmk + t * N);
          ov = sv.template step<false>(xv_t, dv, bmv + t * N, cmv + t * N);
        }
        yk[t * d + c] = from_f32<T>(ok);
        yv[t * d + c] = from_f32<T>(ov);
      }
    }
    chunk_end(q, cs, ce, ok, ov);
    cs = ce;
  }
}

template <typename T, int N, bool SEPX>
hipError_t launch_typed(const attamba_scan_args& a, const ScanShape& sh, hipStream_t stream) {
  const int blocks = ceil_div(sh.groups, 8) * 8 * sh.ctiles;
  hipLaunchKernelGGL((kvssm_scan_kernel<T, N, 8, SEPX>), dim3(blocks), dim3(kWave), 0, stream, sh,
                     a.chunk_cu, static_cast<const T*>(a.x), static_cast<const T*>(a.x_v),
                     static_cast<const T*>(a.dt_k),
                     static_cast<const T*>(a.dt_v), static_cast<const T*>(a.bm_k),
                     static_cast<const T*>(a.cm_k), static_cast<const T*>(a.bm_v),
                     static_cast<const T*>(a.cm_v), a.A_k, a.A_v, a.D_k, a.D_v, a.bias_k,
                     a.bias_v, static_cast<T*>(a.y_k), static_cast<T*>(a.y_v),
                     static_cast<T*>(a.kb), static_cast<T*>(a.vb), a.seq_cu, a.h_last_k,
                     a.h_last_v);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kvssm_scan(const attamba_scan_args& a, hipStream_t stream) {
  if (a.n_chunks == 0 || a.T == 0) return hipSuccess;
  ScanShape sh;
  sh.T = a.T; sh.d = a.d; sh.n_chunks = a.n_chunks; sh.S = a.S;
  sh.groups = ceil_div(a.n_chunks, kChunksPerWave);
  sh.ctiles = a.d / kWave;
  const bool sep = a.x_v != nullptr && a.x_v != a.x;
  if (a.dtype == ATTAMBA_BF16) {
    if (sep) return a.N == 16 ? launch_typed<__bf16, 16, true>(a, sh, stream) : launch_typed<__bf16, 32, true>(a, sh, stream);
    return a.N == 16 ? launch_typed<__bf16, 16, false>(a, sh, stream) : launch_typed<__bf16, 32, false>(a, sh, stream);
  }
  if (sep) return a.N == 16 ? launch_typed<float, 16, true>(a, sh, stream) : launch_typed<float, 32, true>(a, sh, stream);
  return a.N == 16 ? launch_typed<float, 16, false>(a, sh, stream) : launch_typed<float, 32, false>(a, sh, stream);
}

}  // namespace attamba
