// Chunk-aware causal attention over boundary states and per-token keys (pith.science review
// of "Attamba: Attending To Multi-Token States", "What carries the argument": M_train (Eq. 5),
// M_test (Eq. 7) and the window of L leading tokens (Eq. 8); causal reading of M_test from
// the Referee Report's second major comment).
//
// Every query row sees two contiguous key ranges (attn_geom.h), so no mask is materialised:
// a boundary phase over compact boundary states kb/vb and a band phase over per-token keys.
#include "common.h"
#include "attn_geom.h"

namespace attamba {
namespace {

// Generic kernel: one lane per query row, keys visited one at a time with an online softmax in
// float32. Used for float32 activations and for head dims without an MFMA kernel.
template <typename T, int HD>
__global__ __launch_bounds__(64) void attn_rowwise_kernel(AttnParams p) {
  const int s = blockIdx.z, h = blockIdx.y;
  const int s0 = p.seq_cu[s], s1 = p.seq_cu[s + 1];
  const int r0 = s0 + blockIdx.x * 64;
  if (r0 >= s1) return;
  const int i = r0 + threadIdx.x;
  if (i >= s1) return;
  const int c0 = p.token_chunk[s0];
  const RowGeom ri = row_geom(p, i, s0, s1, c0);
  const size_t rs = static_cast<size_t>(p.H) * HD;   // row stride of [., H, HD] tensors
  const T* q = static_cast<const T*>(p.q) + i * rs + h * HD;
  float qs[HD], acc[HD];
  const float qscale = p.scale * kLog2e;             // scores in log2 units
#pragma unroll
  for (int e = 0; e < HD; ++e) { qs[e] = to_f32(q[e]) * qscale; acc[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  auto visit = [&](const T* kr, const T* vr) {
    float sc = 0.f;
#pragma unroll
    for (int e = 0; e < HD; ++e) sc = fmaf(qs[e], to_f32(kr[e]), sc);
    const float mn = fmaxf(m, sc);
    const float corr = hw_exp2(m - mn);
    const float pr = hw_exp2(sc - mn);
    l = fmaf(l, corr, pr);
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] = fmaf(acc[e], corr, pr * to_f32(vr[e]));
    m = mn;
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
  T* out = static_cast<T*>(p.out) + i * rs + h * HD;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int e = 0; e < HD; ++e) out[e] = from_f32<T>(acc[e] * inv);
  if (p.lse) p.lse[static_cast<size_t>(h) * p.T + i] = l > 0.f ? (m + hw_log2(l)) * kLn2 : -INFINITY;
}

template <typename T, int HD>
hipError_t launch_rowwise(const AttnParams& p, hipStream_t stream) {
  dim3 grid(ceil_div(p.max_seqlen, 64), p.H, p.S);
  hipLaunchKernelGGL((attn_rowwise_kernel<T, HD>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attn(const attamba_attn_args& a, float scale, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  AttnParams p;
  p.T = a.T; p.H = a.H; p.S = a.S; p.max_seqlen = a.max_seqlen; p.L = a.L;
  p.train = a.mode == ATTAMBA_MASK_TRAIN ? 1 : 0;
  p.scale = scale;
  p.q = a.q; p.k = a.k; p.v = a.v; p.kb = a.kb; p.vb = a.vb;
  p.seq_cu = a.seq_cu; p.chunk_cu = a.chunk_cu; p.token_chunk = a.token_chunk;
  p.out = a.out; p.lse = a.lse;
  if (a.dtype == ATTAMBA_BF16) {
    if (a.hd == 64 || a.hd == 128) return launch_attn_mfma(p, a.hd, stream);
    return launch_rowwise<__bf16, 32>(p, stream);
  }
  if (a.hd == 32) return launch_rowwise<float, 32>(p, stream);
  if (a.hd == 64) return launch_rowwise<float, 64>(p, stream);
  return launch_rowwise<float, 128>(p, stream);
}

}  // namespace attamba
