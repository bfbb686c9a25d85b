// Backward of the KV-SSM scan: reverse-mode gradients of the two selective scans SSM_K and
// SSM_V (pith.science review of "Attamba: Attending To Multi-Token States", "Core claim" for
// the SSMs in place of the key and value projections; the recurrence is the paper's Eq. 3, cited
// in "Assumptions & free parameters"; the pages' results are models trained with M_train, Eq. 5).
//
// Per SSM, channel c and token t of a chunk (the state restarts at the chunk start, so no
// gradient crosses it), with g_t the gradient of y_t (plus that of the boundary state at the
// chunk's last token) and dh the gradient of the state h_t:
//   dh      = g_t Cm_t + e_{t+1} dh_{t+1}              e_t = exp(delta_t A), u_t = delta_t x_t
//   dCm_t  += g_t h_t          dBm_t += u_t dh         (summed over channels)
//   du      = dh . Bm_t        dx_t = D g_t + delta_t du
//   ddelta  = x_t du + sum_n dh h_{t-1} e_t A          dA += dh h_{t-1} e_t delta_t
//   ddt_t   = ddelta sigmoid(dt_t + bias)              dbias += ddt_t, dD += g_t x_t
//
// Mapping on gfx950: two lanes own one channel of ONE SSM, lane l holding states
// n = NL (l / 32) .. NL (l / 32) + NL - 1 (NL = N / 2) of channel l mod 32; a wave = 32 channels
// of SSM_K or of SSM_V; a workgroup = 4 waves = 128 channels of one SSM over one group of whole
// chunks. A chunk is walked backwards in blocks of PB tokens: the block's states are recomputed
// forward from the chunk start and kept in VGPRs, then the block is walked in reverse. The two
// halves of a channel meet with one cross-lane swap for the sums over n (dh . Bm and the decay
// term of ddelta). The channel sums dBm/dCm are reduced across the 32 lanes of each half with
// cross-lane swaps and DPP moves (every lane ends with one summed quantity), across the
// workgroup's waves in LDS, and added to the [T, N] outputs with one float atomic per
// (token, n) per workgroup; the per-channel parameter gradients are accumulated in VGPRs over
// the chunk group and added with float atomics at its end, so results carry float
// reassociation, not bit-for-bit repeatability.
#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kChannels = kWaves * 32;    // channels per workgroup (two lanes per channel)
constexpr int kChunksPerGroup = 16;

template <int N> struct BlockLen;         // tokens per backward block (state values in VGPRs)
template <> struct BlockLen<16> { static constexpr int value = 8; };
template <> struct BlockLen<32> { static constexpr int value = 4; };

__device__ __forceinline__ float swap16_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum of x over lanes l and l ^ 32 (the two halves of one channel)
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// One butterfly step inside a row of 16 lanes: the lane pairs given by the DPP pattern CTRL
// split the S slots in two; the lane with `up` set keeps the upper half.
template <int CTRL, int S, int M>
__device__ __forceinline__ void dpp_step(float (&v)[M], bool up) {
#pragma unroll
  for (int k = 0; k < S / 2; ++k) {
    const float keep = up ? v[S / 2 + k] : v[k];
    const float send = up ? v[k] : v[S / 2 + k];
    v[k] = keep + dpp<CTRL>(send);
  }
}

constexpr int kRowMirror = 0x140;      // lane i <- lane 15 - i within each row of 16
constexpr int kHalfMirror = 0x141;     // lane i <- lane 7 - i within each group of 8
constexpr int kQuad3210 = 0x1B;        // quad_perm [3, 2, 1, 0]
constexpr int kQuad1032 = 0xB1;        // quad_perm [1, 0, 3, 2]

// Sum each of Q = 16 or 32 per-lane values over the 32 lanes of each half of the wave.
// Afterwards v[0] of lane l holds the half's sum of quantity (l >> 1) mod 16 (Q = 16; lanes 2k
// and 2k + 1 agree) or l mod 32 (Q = 32).
template <int Q>
__device__ __forceinline__ void half_reduce_scatter(float (&v)[Q], int lane) {
#pragma unroll
  for (int k = 0; k < Q / 2; ++k) v[k] = swap16_add(v[k], v[Q / 2 + k]);
  dpp_step<kRowMirror, Q / 2>(v, lane & 8);
  dpp_step<kHalfMirror, Q / 4>(v, lane & 4);
  dpp_step<kQuad3210, Q / 8>(v, lane & 2);
  if constexpr (Q == 32) dpp_step<kQuad1032, 2>(v, lane & 1);
  else v[0] += dpp<kQuad1032>(v[0]);
}

// NL values of a token's row (this lane's half of the N states), converted to float32.
template <typename T, int NL>
__device__ __forceinline__ void load_half_row(const T* __restrict__ row, float (&v)[NL]) {
  if constexpr (sizeof(T) == 2) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int k = 0; k < NL / 8; ++k) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + 8 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * k + 2 * e] = __uint_as_float(w[e] << 16);
        v[8 * k + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < NL / 4; ++k) {
      const float4 w = *reinterpret_cast<const float4*>(row + 4 * k);
      v[4 * k] = w.x; v[4 * k + 1] = w.y; v[4 * k + 2] = w.z; v[4 * k + 3] = w.w;
    }
  }
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void kvssm_scan_bwd_kernel(ScanBwdParams p) {
  constexpr int NL = N / 2;              // states per lane
  constexpr int PB = BlockLen<N>::value;
  constexpr int Q = 2 * NL;              // reduced quantities per lane and token: dCm, dBm
  __shared__ float red[PB][2 * N];       // per-block channel sums: dCm[n] at n, dBm[n] at N + n

  // Workgroups go round-robin to the 8 XCDs (id mod 8); all workgroups of one chunk group
  // (both SSMs, every channel tile) sit on one XCD so its Bm/Cm rows are read once per L2.
  const int wgc = ceil_div(p.d, kChannels);
  const int per_group = 2 * wgc;
  const int id = blockIdx.x, slot = id >> 3;
  const int group = (slot / per_group) * 8 + (id & 7);
  const int n_groups = ceil_div(p.n_chunks, kChunksPerGroup);
  if (group >= n_groups) return;
  const int sub = slot % per_group;
  const ScanBwdSide& sd = p.side[sub / wgc];
  const int tid = threadIdx.x, lane = tid & 63;
  const int half = lane >> 5;
  const int c_raw = (sub % wgc) * kChannels + (tid >> 6) * 32 + (lane & 31);
  const bool active = c_raw < p.d;      // wave-uniform (d is a multiple of 64)
  const int c = active ? c_raw : p.d - 1;
  const int d = p.d;
  const int n0 = half * NL;              // this lane's first state
  const T* __restrict__ X = static_cast<const T*>(sd.x);
  const T* __restrict__ DT = static_cast<const T*>(sd.dt);
  const T* __restrict__ BM = static_cast<const T*>(sd.bm) + n0;
  const T* __restrict__ CM = static_cast<const T*>(sd.cm) + n0;
  const T* __restrict__ GY = static_cast<const T*>(sd.gy);
  const T* __restrict__ GB = static_cast<const T*>(sd.gb);

  for (int k = tid; k < PB * 2 * N; k += kThreads) (&red[0][0])[k] = 0.f;

  float A2[NL], dA[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) { A2[n] = sd.A[c * N + n0 + n] * kLog2e; dA[n] = 0.f; }
  const float Dc = sd.D[c], bias = sd.bias[c];
  float dD = 0.f, dbias = 0.f;
  // LDS slot of this lane's summed quantity after the reduction
  const int qi = Q == 32 ? (lane & 31) : ((lane >> 1) & 15);
  const int red_slot = qi < NL ? n0 + qi : N + n0 + (qi - NL);
  const bool red_writer = Q == 32 || (lane & 1) == 0;

  const int q0 = group * kChunksPerGroup;
  const int q1 = min(q0 + kChunksPerGroup, p.n_chunks);
  for (int q = q0; q < q1; ++q) {
    const int cs = p.chunk_cu[q], ce = p.chunk_cu[q + 1];
    float dh[NL];
#pragma unroll
    for (int n = 0; n < NL; ++n) dh[n] = 0.f;
    for (int bs = cs + ((ce - cs - 1) / PB) * PB; bs >= cs; bs -= PB) {
      const int nb = min(PB, ce - bs);
      // state before the block, recomputed from the chunk start
      float h0[NL];
#pragma unroll
      for (int n = 0; n < NL; ++n) h0[n] = 0.f;
      for (int t = cs; t < bs; ++t) {
        const int o = t * d + c;
        const float delta = softplus_f32(to_f32(DT[o]) + bias);
        const float u = delta * to_f32(X[o]);
        float b[NL];
        load_half_row<T, NL>(BM + t * N, b);
#pragma unroll
        for (int n = 0; n < NL; ++n) h0[n] = fmaf(hw_exp2(delta * A2[n]), h0[n], u * b[n]);
      }
      // the block's states
      float hb[PB][NL];
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        if (j < nb) {
          const int t = bs + j;
          const int o = t * d + c;
          const float delta = softplus_f32(to_f32(DT[o]) + bias);
          const float u = delta * to_f32(X[o]);
          float b[NL];
          load_half_row<T, NL>(BM + t * N, b);
#pragma unroll
          for (int n = 0; n < NL; ++n) {
            const float hp = j == 0 ? h0[n] : hb[j > 0 ? j - 1 : 0][n];
            hb[j][n] = fmaf(hw_exp2(delta * A2[n]), hp, u * b[n]);
          }
        }
      }
      // reverse through the block
#pragma unroll
      for (int j = PB - 1; j >= 0; --j) {
        if (j < nb) {
          const int t = bs + j;
          const int o = t * d + c;
          float g = to_f32(GY[o]);
          if (GB && t == ce - 1) g += to_f32(GB[q * d + c]);
          const float xv = to_f32(X[o]);
          const float z = to_f32(DT[o]) + bias;
          const float delta = softplus_f32(z);
          const float u = delta * xv;
          float b[NL], cc[NL];
          load_half_row<T, NL>(BM + t * N, b);
          load_half_row<T, NL>(CM + t * N, cc);
          float du = 0.f, dd = 0.f;
          float part[Q];
#pragma unroll
          for (int n = 0; n < NL; ++n) {
            dh[n] = fmaf(g, cc[n], dh[n]);
            part[n] = g * hb[j][n];
            part[NL + n] = dh[n] * u;
            du = fmaf(dh[n], b[n], du);
            const float e = hw_exp2(delta * A2[n]);
            const float hp = j == 0 ? h0[n] : hb[j > 0 ? j - 1 : 0][n];
            const float dhe = dh[n] * e;
            const float w = dhe * hp;
            dA[n] = fmaf(w, delta, dA[n]);
            dd = fmaf(w, A2[n], dd);
            dh[n] = dhe;
          }
          du = pair_sum(du);
          dd = pair_sum(dd);
          if (half == 0) {
            const float sig = hw_rcp(1.0f + hw_exp2(-z * kLog2e));
            const float dz = fmaf(dd, kLn2, du * xv) * sig;
            dbias += dz;
            dD = fmaf(g, xv, dD);
            if (active) {
              static_cast<T*>(sd.dx)[o] = from_f32<T>(fmaf(du, delta, g * Dc));
              static_cast<T*>(sd.ddt)[o] = from_f32<T>(dz);
            }
          }
          half_reduce_scatter<Q>(part, lane);
          if (active && red_writer) atomicAdd(&red[j][red_slot], part[0]);
        }
      }
      __syncthreads();
      for (int k = tid; k < PB * 2 * N; k += kThreads) {
        const int j = k / (2 * N), qq = k % (2 * N);
        if (j < nb) {
          float* dst = qq < N ? sd.dcm + (bs + j) * N + qq : sd.dbm + (bs + j) * N + (qq - N);
          atomicAdd(dst, (&red[0][0])[k]);
        }
        (&red[0][0])[k] = 0.f;
      }
      __syncthreads();
    }
  }
  if (active) {
#pragma unroll
    for (int n = 0; n < NL; ++n) atomicAdd(sd.dA + c * N + n0 + n, dA[n]);
    if (half == 0) {
      atomicAdd(sd.dD + c, dD);
      atomicAdd(sd.dbias + c, dbias);
    }
  }
}

// Zero-fill of the outputs the main kernel accumulates into (a plain store kernel, so that the
// launch sequence records no memset node when captured in a graph).
__global__ __launch_bounds__(256) void zero_kernel(ZeroList z) {
  const int i = blockIdx.y;
  float* p = z.ptr[i];
  const int n = z.count[i];
  for (int k = blockIdx.x * 256 + threadIdx.x; k < n; k += gridDim.x * 256) p[k] = 0.f;
}

template <typename T, int N>
hipError_t launch_typed(const ScanBwdParams& p, hipStream_t stream) {
  const int per_group = 2 * ceil_div(p.d, kChannels);
  const int groups = ceil_div(p.n_chunks, kChunksPerGroup);
  const int blocks = ceil_div(groups, 8) * 8 * per_group;
  hipLaunchKernelGGL((kvssm_scan_bwd_kernel<T, N>), dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_zero(const ZeroList& z, int n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(256, n), dim3(256), 0, stream, z);
  return hipGetLastError();
}

hipError_t launch_kvssm_scan_bwd(const ScanBwdParams& p, int N, int dtype, hipStream_t stream) {
  if (p.T == 0 || p.n_chunks == 0) return hipSuccess;
  if (dtype == ATTAMBA_BF16)
    return N == 16 ? launch_typed<__bf16, 16>(p, stream) : launch_typed<__bf16, 32>(p, stream);
  return N == 16 ? launch_typed<float, 16>(p, stream) : launch_typed<float, 32>(p, stream);
}

}  // namespace attamba
