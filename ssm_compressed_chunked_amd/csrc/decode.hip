// Decode step over a cache of boundary states plus the L most recent tokens (pith.science
// review of "Attamba: Attending To Multi-Token States", "Core claim": at inference only the
// boundary states are cached; "If this is right": the cache shrinks by about P).
//
// Three launches on the caller's stream:
//   1. decode_update: four lanes per (sequence, channel): zero the state at a chunk start, one
//      SSM_K and SSM_V step, write the token's key/value into its window slot and, at a chunk
//      end, append it as the next boundary state;
//   2. decode_attn_split: the key list of each (sequence, head) — boundary states 0..E-1 then
//      window positions w..pos — is cut into splits (256 keys, or 1024 for bf16 when the grid
//      still holds enough workgroups); each workgroup streams one
//      split (16-byte loads, hd/8 lanes per key row, so one wave instruction reads several
//      whole rows) and leaves an unnormalised partial (o, running max, sum) in the workspace;
//   3. decode_combine: merges the partials of every (sequence, head).
// The step is bound by HBM: the boundary cache is read once per step.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

constexpr int kSplit = 256;          // keys per split workgroup (the finest split)
constexpr int kSplitWide = 1024;     // bf16 caches whose grid keeps kWideMinGroups workgroups
// The 1024-key kernel takes 234 VGPRs (2 waves per SIMD), so a CU holds two of its 4-wave
// workgroups and the chip 512. With at least 4 such rounds (2048 workgroups) the longer splits
// win; with fewer the grid runs short of workgroups and the 256-key split is used. Measured at
// 32 heads of 128 and 32 768 tokens of context: 1024-key splits 45 600 / 47 466 / 48 004 tokens/s
// against 45 300 / 45 434 / 45 448 at 8 / 12 / 16 sequences (2 304 / 3 456 / 4 608 workgroups),
// 256-key splits 44 687 / 32 008 against 43 294 / 26 205 at 6 / 1 sequences.
constexpr int kWideMinGroups = 4 * 2 * 256;
constexpr int kSplitThreads = 256;
constexpr int kUpdLanes = 4;         // lanes per (sequence, channel) in the state update

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// VEC consecutive elements of a 16-byte word as float
template <typename T, int VEC>
__device__ __forceinline__ void unpack16(const u32x4& w, float (&f)[VEC]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
}

// One SSM_K and SSM_V step per (sequence, channel); the N states of a channel are spread over
// kUpdLanes consecutive lanes (NQ each), whose partial outputs meet with two lane swaps.
template <typename T, int N>
__global__ __launch_bounds__(256) void decode_update_kernel(attamba_decode_cache c,
                                                            attamba_decode_inputs in,
                                                            DecodeLaunch dl) {
  constexpr int NQ = N / kUpdLanes;
  const int b = blockIdx.y;
  const int ch = blockIdx.x * (256 / kUpdLanes) + threadIdx.x / kUpdLanes;
  const int part = threadIdx.x % kUpdLanes;
  const int d = c.d;
  const size_t bd = static_cast<size_t>(b) * d + ch;
  const float x = to_f32(static_cast<const T*>(in.x)[bd]);
  const int head = ch / c.hd, e = ch % c.hd;
  auto run = [&](const float* A, const float* D, const float* bias, const T* dt, const T* bm,
                 const T* cm, float* hstate) -> float {
    float a[NQ], hp[NQ], bv[NQ], cv[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      a[n] = A[static_cast<size_t>(ch) * N + part * NQ + n];
      hp[n] = hstate[bd * N + part * NQ + n];
      bv[n] = to_f32(bm[static_cast<size_t>(b) * N + part * NQ + n]);
      cv[n] = to_f32(cm[static_cast<size_t>(b) * N + part * NQ + n]);
    }
    const float delta = softplus_f32(to_f32(dt[bd]) + bias[ch]);
    const float u = delta * x;
    float y = 0.f;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const float inj = u * bv[n];
      const float hn = dl.is_start ? inj : fmaf(hw_exp2(delta * a[n] * kLog2e), hp[n], inj);
      hstate[bd * N + part * NQ + n] = hn;
      y = fmaf(hn, cv[n], y);
    }
    y += __shfl_xor(y, 1, kWave);
    y += __shfl_xor(y, 2, kWave);
    return fmaf(D[ch], x, y);
  };
  const float yk = run(c.A_k, c.D_k, c.bias_k, static_cast<const T*>(in.dt_k),
                       static_cast<const T*>(in.bm_k), static_cast<const T*>(in.cm_k), c.h_k);
  const float yv = run(c.A_v, c.D_v, c.bias_v, static_cast<const T*>(in.dt_v),
                       static_cast<const T*>(in.bm_v), static_cast<const T*>(in.cm_v), c.h_v);
  if (part != 0) return;
  const size_t bh = static_cast<size_t>(b) * c.H + head;
  if (c.L > 0) {
    const size_t o = (bh * c.L + dl.slot) * c.hd + e;
    static_cast<T*>(c.kw)[o] = from_f32<T>(yk);
    static_cast<T*>(c.vw)[o] = from_f32<T>(yv);
  }
  if (dl.is_end) {
    const size_t o = (bh * c.cap + dl.n_bound_before) * c.hd + e;
    static_cast<T*>(c.kb)[o] = from_f32<T>(yk);
    static_cast<T*>(c.vb)[o] = from_f32<T>(yv);
  }
}

// Element offset of key k of (b, h): boundary state k < E, else window position
// w + (k - E), held in ring slot (w mod L + k - E) mod L.
__device__ __forceinline__ size_t key_off(const attamba_decode_cache& c, const DecodeLaunch& dl,
                                          size_t bh, int k, bool& in_window) {
  if (k < dl.E) {
    in_window = false;
    return (bh * c.cap + k) * c.hd;
  }
  in_window = true;
  int sl = dl.w_slot + (k - dl.E);
  if (sl >= c.L) sl -= c.L;
  return (bh * c.L + sl) * c.hd;
}

// One split of SPLIT keys of one (sequence, head). A key row is read by LPK lanes with 16-byte
// loads (KPW rows per wave instruction); the loads of NB rows per lane are issued together
// before any is used, for both the K pass (scores) and the V pass (P V). Every cache row is read
// once per step, so the loads are non-temporal (no cache allocation): 6.3 TB/s against 5.9 TB/s
// with ordinary loads at the 4.4 GB per step of a 32 x 32768-token batch. Splits of 1024 keys
// keep four times the bytes per workgroup in flight between its two reductions: 6.7 TB/s there.
template <typename T, int HD, int SPLIT>
__global__ __launch_bounds__(kSplitThreads) void decode_attn_split_kernel(
    attamba_decode_cache c, attamba_decode_inputs in, DecodeLaunch dl, int max_splits) {
  constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte load
  constexpr int LPK = HD / VEC;                // lanes per key row
  constexpr int KPW = kWave / LPK;             // key rows per wave instruction
  constexpr int NW = kSplitThreads / kWave;
  constexpr int KPB = KPW * NW;                // key rows per workgroup iteration
  constexpr int NIT = SPLIT / KPB;             // iterations per split
  // iterations whose loads fly together (16 rows per lane in the 1024-key split: +0.7 %)
  constexpr int NB = NIT < 8 ? NIT : (SPLIT >= 1024 ? 16 : 8);
  __shared__ float s_p[SPLIT];
  __shared__ float s_red[NW];
  __shared__ float s_acc[NW][KPW][HD];

  const int sp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave, wid = tid / kWave;
  const int sub = lane % LPK, grp = lane / LPK;
  const size_t bh = static_cast<size_t>(b) * c.H + h;
  const int n_keys = dl.E + dl.n_window;
  const int k0 = sp * SPLIT;
  const int nk = min(SPLIT, n_keys - k0);
  float* part = static_cast<float*>(c.workspace) + (bh * max_splits + sp) * (HD + 2);
  if (nk <= 0) {   // no key in this split (only when the whole list is empty)
    for (int e = tid; e < HD; e += kSplitThreads) part[e] = 0.f;
    if (tid == 0) { part[HD] = -INFINITY; part[HD + 1] = 0.f; }
    return;
  }

  float qv[VEC];
  {
    const T* q = static_cast<const T*>(in.q) + bh * HD + sub * VEC;
    const float qs = dl.scale * kLog2e;
#pragma unroll
    for (int v = 0; v < VEC; ++v) qv[v] = to_f32(q[v]) * qs;
  }
  const T* kbase = static_cast<const T*>(c.kb);
  const T* kwin = static_cast<const T*>(c.kw);
  const T* vbase = static_cast<const T*>(c.vb);
  const T* vwin = static_cast<const T*>(c.vw);

  // scores (log2 units)
#pragma unroll
  for (int i0 = 0; i0 < NIT; i0 += NB) {
    u32x4 raw[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int kk = min((i0 + u) * KPB + wid * KPW + grp, nk - 1);
      bool win;
      const size_t off = key_off(c, dl, bh, k0 + kk, win);
      raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>((win ? kwin : kbase) + off + sub * VEC));
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int kk = (i0 + u) * KPB + wid * KPW + grp;
      float kf[VEC];
      unpack16<T, VEC>(raw[u], kf);
      float sc = 0.f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) sc = fmaf(qv[v], kf[v], sc);
#pragma unroll
      for (int off = 1; off < LPK; off <<= 1) sc += __shfl_xor(sc, off, kWave);
      if (sub == 0 && kk < nk) s_p[kk] = sc;
    }
  }
  __syncthreads();
  // max over the split
  float mx = -INFINITY;
  for (int k = tid; k < nk; k += kSplitThreads) mx = fmaxf(mx, s_p[k]);
  for (int off = kWave / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
  if (lane == 0) s_red[wid] = mx;
  __syncthreads();
  mx = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_red[w]);
  __syncthreads();
  float sum = 0.f;
  for (int k = tid; k < SPLIT; k += kSplitThreads) {
    const float pr = k < nk ? hw_exp2(s_p[k] - mx) : 0.f;
    s_p[k] = pr;
    sum += pr;
  }
  for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
  if (lane == 0) s_red[wid] = sum;
  __syncthreads();
  // P V (rows past nk re-read the last key with weight 0)
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
#pragma unroll
  for (int i0 = 0; i0 < NIT; i0 += NB) {
    u32x4 raw[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int kk = min((i0 + u) * KPB + wid * KPW + grp, nk - 1);
      bool win;
      const size_t off = key_off(c, dl, bh, k0 + kk, win);
      raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>((win ? vwin : vbase) + off + sub * VEC));
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float pr = s_p[(i0 + u) * KPB + wid * KPW + grp];
      float vf[VEC];
      unpack16<T, VEC>(raw[u], vf);
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = fmaf(pr, vf[v], acc[v]);
    }
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) s_acc[wid][grp][sub * VEC + v] = acc[v];
  __syncthreads();
  for (int e = tid; e < HD; e += kSplitThreads) {
    float o = 0.f;
    for (int w = 0; w < NW; ++w)
      for (int g = 0; g < KPW; ++g) o += s_acc[w][g][e];
    part[e] = o;
  }
  if (tid == 0) {
    float l = 0.f;
    for (int w = 0; w < NW; ++w) l += s_red[w];
    part[HD] = mx;
    part[HD + 1] = l;
  }
}

// Merges the split partials of one (sequence, head): thread e owns output element e.
template <typename T, int HD>
__global__ __launch_bounds__(HD) void decode_combine_kernel(attamba_decode_cache c,
                                                            attamba_decode_inputs in,
                                                            DecodeLaunch dl, int max_splits) {
  constexpr int NWC = (HD + kWave - 1) / kWave;
  __shared__ float s_red[NWC];
  const int h = blockIdx.x, b = blockIdx.y, e = threadIdx.x;
  const size_t bh = static_cast<size_t>(b) * c.H + h;
  const float* part = static_cast<const float*>(c.workspace) + bh * max_splits * (HD + 2);
  const int ns = dl.n_splits;
  float mx = -INFINITY;
  for (int s = e; s < ns; s += HD) mx = fmaxf(mx, part[s * (HD + 2) + HD]);
  for (int off = (HD < kWave ? HD : kWave) / 2; off > 0; off >>= 1)
    mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
  if (e % kWave == 0) s_red[e / kWave] = mx;
  __syncthreads();
  mx = s_red[0];
#pragma unroll
  for (int w = 1; w < NWC; ++w) mx = fmaxf(mx, s_red[w]);
  float o = 0.f, l = 0.f;
  if (mx > -INFINITY) {
#pragma unroll 8
    for (int s = 0; s < ns; ++s) {
      const float* ps = part + s * (HD + 2);
      const float wgt = hw_exp2(ps[HD] - mx);
      o = fmaf(ps[e], wgt, o);
      l = fmaf(ps[HD + 1], wgt, l);
    }
  }
  static_cast<T*>(in.out)[bh * HD + e] = from_f32<T>(l > 0.f ? o / l : 0.f);
}

template <typename T, int N, int HD>
hipError_t launch_typed(const attamba_decode_cache& c, const attamba_decode_inputs& in,
                        const DecodeLaunch& dl_in, hipStream_t stream) {
  // the workspace holds max_splits partials per (sequence, head), counted at the finest split
  const int max_splits = decode_max_splits(c.cap, c.L);
  const int n_keys = dl_in.E + dl_in.n_window;
  const bool wide = sizeof(T) == 2 &&
                    static_cast<long long>(c.B) * c.H * ceil_div(n_keys, kSplitWide) >= kWideMinGroups;
  DecodeLaunch dl = dl_in;
  dl.n_splits = max(1, ceil_div(n_keys, wide ? kSplitWide : kSplit));
  hipLaunchKernelGGL((decode_update_kernel<T, N>), dim3(c.d * kUpdLanes / 256, c.B), dim3(256), 0,
                     stream, c, in, dl);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  bool launched = false;
  if constexpr (sizeof(T) == 2) {
    if (wide) {
      hipLaunchKernelGGL((decode_attn_split_kernel<T, HD, kSplitWide>), dim3(dl.n_splits, c.H, c.B),
                         dim3(kSplitThreads), 0, stream, c, in, dl, max_splits);
      launched = true;
    }
  }
  if (!launched) {
    hipLaunchKernelGGL((decode_attn_split_kernel<T, HD, kSplit>), dim3(dl.n_splits, c.H, c.B),
                       dim3(kSplitThreads), 0, stream, c, in, dl, max_splits);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_combine_kernel<T, HD>), dim3(c.H, c.B), dim3(HD), 0, stream, c, in,
                     dl, max_splits);
  return hipGetLastError();
}

template <typename T, int N>
hipError_t launch_hd(const attamba_decode_cache& c, const attamba_decode_inputs& in,
                     const DecodeLaunch& dl, hipStream_t stream) {
  if (c.hd == 128) return launch_typed<T, N, 128>(c, in, dl, stream);
  if (c.hd == 64) return launch_typed<T, N, 64>(c, in, dl, stream);
  return launch_typed<T, N, 32>(c, in, dl, stream);
}

// Prefill -> decode hand-off: block (b, h) copies the n_bound completed boundary states of
// sequence b (its chunks c_b .. c_b + n_bound - 1 of the prefill) and the per-token keys/values
// of the window positions w0 .. n0 - 1 into the head-major cache rows.
template <typename T>
__global__ __launch_bounds__(256) void decode_load_prefix_kernel(attamba_decode_cache c,
                                                                 attamba_decode_prefix pf,
                                                                 int n_bound, int w0) {
  const int bh = blockIdx.x;
  const int b = bh / c.H, h = bh % c.H;
  const int hd = c.hd, d = c.d;
  const int s0 = pf.seq_cu[b];
  const int cb = pf.token_chunk[s0];
  const int rows = n_bound + (pf.n0 - w0);
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e >= rows * hd) return;
  const int r = e / hd, k = e % hd;
  const size_t head = static_cast<size_t>(b) * c.H + h;
  const T* sk;
  const T* sv;
  T* dk;
  T* dv;
  size_t so, dof;
  if (r < n_bound) {
    so = static_cast<size_t>(cb + r) * d + h * hd + k;
    dof = (head * c.cap + r) * hd + k;
    sk = static_cast<const T*>(pf.kb); sv = static_cast<const T*>(pf.vb);
    dk = static_cast<T*>(c.kb); dv = static_cast<T*>(c.vb);
  } else {
    const int pos = w0 + (r - n_bound);
    so = static_cast<size_t>(s0 + pos) * d + h * hd + k;
    dof = (head * c.L + pos % c.L) * hd + k;
    sk = static_cast<const T*>(pf.y_k); sv = static_cast<const T*>(pf.y_v);
    dk = static_cast<T*>(c.kw); dv = static_cast<T*>(c.vw);
  }
  dk[dof] = sk[so];
  dv[dof] = sv[so];
}

__global__ __launch_bounds__(256) void copy_f32_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                       size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256)
    dst[i] = src[i];
}

}  // namespace

hipError_t launch_decode_load_prefix(const attamba_decode_cache& c, const attamba_decode_prefix& pf,
                                     int n_bound, int w0, hipStream_t stream) {
  const int rows = n_bound + (pf.n0 - w0);
  if (rows > 0) {
    const dim3 grid(c.B * c.H, ceil_div(rows * c.hd, 256));
    if (c.dtype == ATTAMBA_BF16)
      hipLaunchKernelGGL(decode_load_prefix_kernel<__bf16>, grid, dim3(256), 0, stream, c, pf, n_bound, w0);
    else
      hipLaunchKernelGGL(decode_load_prefix_kernel<float>, grid, dim3(256), 0, stream, c, pf, n_bound, w0);
  }
  const size_t n = static_cast<size_t>(c.B) * c.d * c.N;
  hipLaunchKernelGGL(copy_f32_kernel, dim3(1024), dim3(256), 0, stream, c.h_k, pf.h_last_k, n);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(1024), dim3(256), 0, stream, c.h_v, pf.h_last_v, n);
  return hipGetLastError();
}

int decode_max_splits(int cap, int L) { return ceil_div(cap + L, kSplit) + 1; }

// Scratch of the decode step variant that allocates nothing: the split partials live in this
// file-scope device array instead of a caller workspace. Every GPU the library runs on holds its
// own copy until the process ends. In host code `scratch` names a host-side stand-in, not device
// memory, so its device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever passed to kernels.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(int B, int H, int hd, int cap, int L) {
  return static_cast<size_t>(B) * H * decode_max_splits(cap, L) * (hd + 2) * sizeof(float);
}

hipError_t launch_decode_step(const attamba_decode_cache& c, const attamba_decode_inputs& in,
                              const DecodeLaunch& dl_in, hipStream_t stream) {
  if (c.dtype == ATTAMBA_BF16) {
    return c.N == 16 ? launch_hd<__bf16, 16>(c, in, dl_in, stream) : launch_hd<__bf16, 32>(c, in, dl_in, stream);
  }
  return c.N == 16 ? launch_hd<float, 16>(c, in, dl_in, stream) : launch_hd<float, 32>(c, in, dl_in, stream);
}

}  // namespace attamba
