// KV-SSM: the two selective scans SSM_K and SSM_V that replace the key and value projections
// and compress each chunk into one boundary state (pith.science review of "Attamba: Attending
// To Multi-Token States", "Core claim"; the selective SSM is the paper's Eq. 3, cited in
// "Assumptions & free parameters").
//
// Mapping on gfx950: one lane owns one channel c of both SSMs and keeps the 2*N state values
// and the 2*N decay rates (A * log2 e) in VGPRs; a wave owns 64 consecutive channels and walks
// a group of whole chunks token by token (chunks are independent because the state restarts
// at every chunk start). All lanes of a wave sit on the same token, so the per-token rows
// bm/cm (shared by all channels) are wave-uniform: they are fetched with scalar loads and
// enter the VALU instructions as SGPR operands. Per state and token the work is one multiply
// for the exponent, one v_exp_f32, one multiply for the input term, one FMA for the state
// and one FMA for the output; this instruction stream, not HBM, bounds the kernel. x and the
// two step-size rows are read once per token for both SSMs (128-byte rows per wave at bf16),
// the next token's row is prefetched while the current one is computed.
#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

constexpr int kChunksPerWave = 8;

struct ScanParams {
  int T, d, n_chunks, S;
  const int32_t* chunk_cu;
  const void *x, *dt_k, *dt_v, *bm_k, *cm_k, *bm_v, *cm_v;
  const float *A_k, *A_v, *D_k, *D_v, *bias_k, *bias_v;
  void *y_k, *y_v, *kb, *vb;
  const int32_t* seq_cu;
  float *h_last_k, *h_last_v;
  int groups;          // chunk groups = ceil(n_chunks / kChunksPerWave)
  int ctiles;          // channel tiles = d / 64
  int group_rows;      // ceil(groups / 8)
};

// Workgroup id -> (chunk group, channel tile). Workgroups are dispatched round-robin over
// the 8 XCDs (id mod 8), each with its own L2; every channel tile of one chunk group is
// placed on the same XCD so the group's bm/cm rows are fetched from HBM once per XCD.
__device__ __forceinline__ bool map_block(const ScanParams& p, int& group, int& ctile) {
  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  group = (slot / p.ctiles) * 8 + xcd;
  ctile = slot % p.ctiles;
  return group < p.groups;
}

template <typename T, int N>
struct SsmLane {
  float A2[N];   // A[c, n] * log2(e)
  float h[N];
  float D, bias;

  __device__ __forceinline__ void load_params(const float* A, const float* Dp, const float* bp,
                                              int c) {
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = A[c * N + n] * kLog2e;
    D = Dp[c];
    bias = bp[c];
  }

  // One token. FIRST: the state restarts (no decay term).
  template <bool FIRST>
  __device__ __forceinline__ float step(float x, float dt, const T* __restrict__ bm,
                                        const T* __restrict__ cm) {
    const float delta = softplus_f32(dt + bias);
    const float u = delta * x;
    float y = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float inj = u * to_f32(bm[n]);
      if (FIRST) {
        h[n] = inj;
      } else {
        h[n] = fmaf(hw_exp2(delta * A2[n]), h[n], inj);
      }
      y = fmaf(h[n], to_f32(cm[n]), y);
    }
    return fmaf(D, x, y);
  }
};

template <typename T, int N>
__global__ __launch_bounds__(kWave) void kvssm_scan_kernel(ScanParams p) {
  int group, ctile;
  if (!map_block(p, group, ctile)) return;
  const int lane = threadIdx.x;
  const int c = ctile * kWave + lane;
  const int d = p.d;
  const int q0 = group * kChunksPerWave;
  const int q1 = min(q0 + kChunksPerWave, p.n_chunks);

  const T* __restrict__ x = static_cast<const T*>(p.x);
  const T* __restrict__ dtk = static_cast<const T*>(p.dt_k);
  const T* __restrict__ dtv = static_cast<const T*>(p.dt_v);
  const T* __restrict__ bmk = static_cast<const T*>(p.bm_k);
  const T* __restrict__ cmk = static_cast<const T*>(p.cm_k);
  const T* __restrict__ bmv = static_cast<const T*>(p.bm_v);
  const T* __restrict__ cmv = static_cast<const T*>(p.cm_v);
  T* __restrict__ yk = static_cast<T*>(p.y_k);
  T* __restrict__ yv = static_cast<T*>(p.y_v);
  T* __restrict__ kb = static_cast<T*>(p.kb);
  T* __restrict__ vb = static_cast<T*>(p.vb);

  SsmLane<T, N> sk, sv;
  sk.load_params(p.A_k, p.D_k, p.bias_k, c);
  sv.load_params(p.A_v, p.D_v, p.bias_v, c);

  const int tb = p.chunk_cu[q0];
  const int te = p.chunk_cu[q1];
  int q = q0;
  int cs = tb;                      // start of chunk q
  int ce = p.chunk_cu[q0 + 1];      // end (exclusive) of chunk q

  float nx = 0.f, ndk = 0.f, ndv = 0.f;
  if (tb < te) {
    const size_t o = static_cast<size_t>(tb) * d + c;
    nx = to_f32(x[o]); ndk = to_f32(dtk[o]); ndv = to_f32(dtv[o]);
  }
  for (int t = tb; t < te; ++t) {
    const float xv = nx, dk = ndk, dv = ndv;
    if (t + 1 < te) {
      const size_t o = static_cast<size_t>(t + 1) * d + c;
      nx = to_f32(x[o]); ndk = to_f32(dtk[o]); ndv = to_f32(dtv[o]);
    }
    const size_t rN = static_cast<size_t>(t) * N;
    float ok, ov;
    if (t == cs) {
      ok = sk.template step<true>(xv, dk, bmk + rN, cmk + rN);
      ov = sv.template step<true>(xv, dv, bmv + rN, cmv + rN);
    } else {
      ok = sk.template step<false>(xv, dk, bmk + rN, cmk + rN);
      ov = sv.template step<false>(xv, dv, bmv + rN, cmv + rN);
    }
    const size_t o = static_cast<size_t>(t) * d + c;
    yk[o] = from_f32<T>(ok);
    yv[o] = from_f32<T>(ov);
    if (t == ce - 1) {              // last token of chunk q: boundary state and hand-off
      if (kb) kb[static_cast<size_t>(q) * d + c] = from_f32<T>(ok);
      if (vb) vb[static_cast<size_t>(q) * d + c] = from_f32<T>(ov);
      if (p.h_last_k) {
        int lo = 0, hi = p.S;       // sequence s with seq_cu[s] <= cs < seq_cu[s + 1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (p.seq_cu[mid] <= cs) lo = mid; else hi = mid;
        }
        if (p.seq_cu[lo + 1] == ce) {
          float* hk = p.h_last_k + (static_cast<size_t>(lo) * d + c) * N;
          float* hv = p.h_last_v + (static_cast<size_t>(lo) * d + c) * N;
#pragma unroll
          for (int n = 0; n < N; ++n) { hk[n] = sk.h[n]; hv[n] = sv.h[n]; }
        }
      }
      ++q;
      cs = ce;
      if (q < q1) ce = p.chunk_cu[q + 1];
    }
  }
}

template <typename T, int N>
hipError_t launch_typed(const ScanParams& p, hipStream_t stream) {
  const int blocks = p.group_rows * 8 * p.ctiles;
  hipLaunchKernelGGL((kvssm_scan_kernel<T, N>), dim3(blocks), dim3(kWave), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kvssm_scan(const attamba_scan_args& a, hipStream_t stream) {
  if (a.n_chunks == 0 || a.T == 0) return hipSuccess;
  ScanParams p;
  p.T = a.T; p.d = a.d; p.n_chunks = a.n_chunks; p.S = a.S;
  p.chunk_cu = a.chunk_cu;
  p.x = a.x; p.dt_k = a.dt_k; p.dt_v = a.dt_v;
  p.bm_k = a.bm_k; p.cm_k = a.cm_k; p.bm_v = a.bm_v; p.cm_v = a.cm_v;
  p.A_k = a.A_k; p.A_v = a.A_v; p.D_k = a.D_k; p.D_v = a.D_v;
  p.bias_k = a.bias_k; p.bias_v = a.bias_v;
  p.y_k = a.y_k; p.y_v = a.y_v; p.kb = a.kb; p.vb = a.vb;
  p.seq_cu = a.seq_cu;
  p.h_last_k = a.h_last_k; p.h_last_v = a.h_last_v;
  p.groups = ceil_div(a.n_chunks, kChunksPerWave);
  p.ctiles = a.d / kWave;
  p.group_rows = ceil_div(p.groups, 8);
  if (a.dtype == ATTAMBA_BF16) {
    return a.N == 16 ? launch_typed<__bf16, 16>(p, stream) : launch_typed<__bf16, 32>(p, stream);
  }
  return a.N == 16 ? launch_typed<float, 16>(p, stream) : launch_typed<float, 32>(p, stream);
}

}  // namespace attamba
