// Backward of the chunk-aware causal attention (pith.science review of "Attamba: Attending To
// Multi-Token States", "What carries the argument": M_train Eq. 5, M_test Eq. 7, window Eq. 8;
// the pages' models are trained with M_train).
//
// With P = softmax over the visible keys (recomputed from the forward's LSE), D_i = dO_i . O_i:
//   dS_ij = P_ij (dO_i . v_j - D_i),  dq_i = scale sum_j dS_ij k_j,
//   dk_j = scale sum_i dS_ij q_i,     dv_j = sum_i P_ij dO_i.
// A key position is read either as a boundary state (kb/vb, by rows whose band starts after it)
// or as a per-token key (k/v, by rows whose band contains it); the gradients follow the same
// split: dkb/dvb collect the first use, dk/dv the second (the KV-SSM backward adds them at the
// chunk's last token).
//
// Kernels: a row-sum kernel for D; a query-centric kernel for dq (one lane per query, the keys of
// its two ranges in order); a key-centric kernel for dk/dv and dkb/dvb (one lane per key; the
// rows that see a key form one contiguous range, because w_i and E_i grow with i, found by
// binary search; the lanes of a wave walk the union of their ranges in step, so every row is
// read once per wave as a broadcast). bf16 with head dims 64 and 128 goes to the matrix-core
// kernels (attn_mfma_bwd.hip, whose dQ kernel computes D itself); these generic kernels cover
// float32 and head dim 32.
#include "attn_geom.h"
#include "common.h"

namespace attamba {
namespace {

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(AttnBwdParams p) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.f.T * p.f.H) return;
  const int i = idx / p.f.H, h = idx % p.f.H;
  const T* o = static_cast<const T*>(p.f.out) + static_cast<size_t>(idx) * HD;
  const T* g = static_cast<const T*>(p.dout) + static_cast<size_t>(idx) * HD;
  float acc = 0.f;
#pragma unroll 8
  for (int e = 0; e < HD; ++e) acc = fmaf(to_f32(o[e]), to_f32(g[e]), acc);
  p.delta[static_cast<size_t>(h) * p.f.T + i] = acc;
}

template <typename T, int HD>
__global__ __launch_bounds__(64) void attn_bwd_dq_kernel(AttnBwdParams bp) {
  const AttnParams& p = bp.f;
  const int s = blockIdx.z, h = blockIdx.y;
  const int s0 = p.seq_cu[s], s1 = p.seq_cu[s + 1];
  const int i = s0 + blockIdx.x * 64 + threadIdx.x;
  if (i >= s1) return;
  const int c0 = p.token_chunk[s0];
  const RowGeom ri = row_geom(p, i, s0, s1, c0);
  const size_t rs = static_cast<size_t>(p.H) * HD;
  const float lse = p.lse[static_cast<size_t>(h) * p.T + i];
  T* dq = static_cast<T*>(bp.dq) + i * rs + h * HD;
  float acc[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) acc[e] = 0.f;
  if (lse != -INFINITY) {
    const float lse2 = lse * kLog2e;
    const float Di = bp.delta[static_cast<size_t>(h) * p.T + i];
    const T* q = static_cast<const T*>(p.q) + i * rs + h * HD;
    const T* go = static_cast<const T*>(bp.dout) + i * rs + h * HD;
    float qs[HD], gs[HD];
    const float c = p.scale * kLog2e;
#pragma unroll
    for (int e = 0; e < HD; ++e) { qs[e] = to_f32(q[e]) * c; gs[e] = to_f32(go[e]); }
    auto visit = [&](const T* kr, const T* vr) {
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) {
        sc = fmaf(qs[e], to_f32(kr[e]), sc);
        dp = fmaf(gs[e], to_f32(vr[e]), dp);
      }
      const float ds = hw_exp2(sc - lse2) * (dp - Di);
#pragma unroll
      for (int e = 0; e < HD; ++e) acc[e] = fmaf(ds, to_f32(kr[e]), acc[e]);
    };
    const T* kb = static_cast<const T*>(p.kb) + h * HD;
    const T* vb = static_cast<const T*>(p.vb) + h * HD;
    for (int k = 0; k < ri.E; ++k) {
      const size_t o = static_cast<size_t>(c0 + k) * rs;
      visit(kb + o, vb + o);
    }
    const T* kt = static_cast<const T*>(p.k) + h * HD;
    const T* vt = static_cast<const T*>(p.v) + h * HD;
    for (int j = ri.w; j <= i; ++j) {
      const size_t o = static_cast<size_t>(j) * rs;
      visit(kt + o, vt + o);
    }
  }
#pragma unroll
  for (int e = 0; e < HD; ++e) dq[e] = from_f32<T>(acc[e] * p.scale);
}

// Key-centric dk/dv. BOUNDARY: lane = boundary state of chunk c0 + x (seen by rows i with
// w_i > its end position); otherwise lane = per-token key at position s0 + x (seen by rows
// i >= j with w_i <= j).
template <typename T, int HD, bool BOUNDARY>
__global__ __launch_bounds__(64) void attn_bwd_dkv_kernel(AttnBwdParams bp) {
  const AttnParams& p = bp.f;
  const int s = blockIdx.z, h = blockIdx.y;
  const int s0 = p.seq_cu[s], s1 = p.seq_cu[s + 1];
  if (s1 <= s0) return;
  const int c0 = p.token_chunk[s0];
  const int nkeys = BOUNDARY ? p.token_chunk[s1 - 1] + 1 - c0 : s1 - s0;
  const int x = blockIdx.x * 64 + threadIdx.x;
  const bool valid = x < nkeys;
  const int kx = valid ? x : nkeys - 1;
  if (blockIdx.x * 64 >= nkeys) return;
  // this lane's rows [ia, ib]
  int ia, ib;
  if (BOUNDARY) {
    const int e = p.chunk_cu[c0 + kx + 1] - 1;   // the chunk's last token
    int lo = e, hi = s1;                          // first i in [e, s1) with w_i > e, else s1
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (row_geom(p, mid, s0, s1, c0).w > e) hi = mid; else lo = mid + 1;
    }
    ia = lo;
    ib = s1 - 1;
  } else {
    const int j = s0 + kx;
    ia = j;
    if (row_geom(p, j, s0, s1, c0).w > j) {
      ib = j - 1;                                 // no row sees this key through its band
    } else {
      int lo = j, hi = s1 - 1;                    // last i in [j, s1) with w_i <= j
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (row_geom(p, mid, s0, s1, c0).w <= j) lo = mid; else hi = mid - 1;
      }
      ib = lo;
    }
  }
  if (!valid) { ia = s1; ib = s0 - 1; }     // empty, and outside every valid lane's range
  const size_t rs = static_cast<size_t>(p.H) * HD;
  const size_t ko = static_cast<size_t>(BOUNDARY ? c0 + kx : s0 + kx) * rs + h * HD;
  const T* kr = static_cast<const T*>(BOUNDARY ? p.kb : p.k) + ko;
  const T* vr = static_cast<const T*>(BOUNDARY ? p.vb : p.v) + ko;
  float ks[HD], vs[HD], dk[HD], dv[HD];
  const float c = p.scale * kLog2e;
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    ks[e] = to_f32(kr[e]) * c;
    vs[e] = to_f32(vr[e]);
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  // walk the union of the wave's row ranges
  int wa = ia, wb = ib;
  for (int off = 32; off >= 1; off >>= 1) {
    wa = min(wa, __shfl_xor(wa, off));
    wb = max(wb, __shfl_xor(wb, off));
  }
  const T* qt = static_cast<const T*>(p.q) + h * HD;
  const T* gt = static_cast<const T*>(bp.dout) + h * HD;
  for (int i = wa; i <= wb; ++i) {
    if (i < ia || i > ib) continue;
    const float lse2 = p.lse[static_cast<size_t>(h) * p.T + i] * kLog2e;
    const float Di = bp.delta[static_cast<size_t>(h) * p.T + i];
    const T* qr = qt + i * rs;
    const T* gr = gt + i * rs;
    float sc = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < HD; ++e) {
      sc = fmaf(ks[e], to_f32(qr[e]), sc);
      dp = fmaf(vs[e], to_f32(gr[e]), dp);
    }
    const float pr = hw_exp2(sc - lse2);
    const float ds = pr * (dp - Di);
#pragma unroll
    for (int e = 0; e < HD; ++e) {
      dv[e] = fmaf(pr, to_f32(gr[e]), dv[e]);
      dk[e] = fmaf(ds, to_f32(qr[e]), dk[e]);
    }
  }
  if (!valid) return;
  T* dko = static_cast<T*>(BOUNDARY ? bp.dkb : bp.dk) + ko;
  T* dvo = static_cast<T*>(BOUNDARY ? bp.dvb : bp.dv) + ko;
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    dko[e] = from_f32<T>(dk[e] * p.scale);
    dvo[e] = from_f32<T>(dv[e]);
  }
}

template <typename T, int HD>
hipError_t launch_generic(const AttnBwdParams& p, hipStream_t stream) {
  const AttnParams& f = p.f;
  hipLaunchKernelGGL((attn_bwd_delta_kernel<T, HD>), dim3(ceil_div(f.T * f.H, 256)), dim3(256), 0,
                     stream, p);
  dim3 grid(ceil_div(f.max_seqlen, 64), f.H, f.S);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD>), grid, dim3(64), 0, stream, p);
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, HD, false>), grid, dim3(64), 0, stream, p);
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, HD, true>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attn_bwd(const AttnBwdParams& p, int hd, int dtype, hipStream_t stream) {
  if (p.f.T == 0) return hipSuccess;
  if (dtype == ATTAMBA_BF16 && (hd == 64 || hd == 128)) return launch_attn_bwd_mfma(p, hd, stream);
  if (dtype == ATTAMBA_BF16) {
    if (hd == 32) return launch_generic<__bf16, 32>(p, stream);
    if (hd == 64) return launch_generic<__bf16, 64>(p, stream);
    return launch_generic<__bf16, 128>(p, stream);
  }
  if (hd == 32) return launch_generic<float, 32>(p, stream);
  if (hd == 64) return launch_generic<float, 64>(p, stream);
  return launch_generic<float, 128>(p, stream);
}

}  // namespace attamba
