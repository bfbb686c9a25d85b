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
// chunks. A chunk is walked backwards in blocks of PB tokens: the block's Bm/Cm rows (the same
// for every channel) are staged once in LDS, its states are recomputed forward from the chunk
// start and kept in VGPRs, then the block is walked in reverse. The two halves of a channel meet
// with one cross-lane swap for the sums over n (dh . Bm and the decay term of ddelta). The
// channel sums dCm (forward pass) and dBm (reverse pass) are reduced across the 32 lanes of each
// half with cross-lane swaps and DPP moves (every lane ends with one summed quantity), across
// the workgroup's waves in LDS, and added to the [T, N] outputs with one float atomic per
// (token, n) per workgroup; the per-channel parameter gradients are accumulated in VGPRs over
// the chunk group and added with float atomics at its end, so results carry float
// reassociation, not bit-for-bit repeatability.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kChannels = kWaves * 32;    // channels per workgroup (two lanes per channel)
constexpr int kChunksPerGroup = 8;

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

// Sum each of Q = 8 or 16 per-lane values over the 32 lanes of each half of the wave.
// Afterwards v[0] of lane l holds the half's sum of quantity (l >> 2) mod 8 (Q = 8; the four
// lanes of a quad agree) or (l >> 1) mod 16 (Q = 16; lanes 2k and 2k + 1 agree).
template <int Q>
__device__ __forceinline__ void half_reduce_scatter(float (&v)[Q], int lane) {
#pragma unroll
  for (int k = 0; k < Q / 2; ++k) v[k] = swap16_add(v[k], v[Q / 2 + k]);
  dpp_step<kRowMirror, Q / 2>(v, lane & 8);
  dpp_step<kHalfMirror, Q / 4>(v, lane & 4);
  if constexpr (Q == 16) {
    dpp_step<kQuad3210, 2>(v, lane & 2);
  } else {
    v[0] += dpp<kQuad3210>(v[0]);
  }
  v[0] += dpp<kQuad1032>(v[0]);
}
template <int Q>
__device__ __forceinline__ int reduced_index(int lane) { return Q == 16 ? (lane >> 1) & 15 : (lane >> 2) & 7; }
template <int Q>
__device__ __forceinline__ bool reduced_writer(int lane) { return Q == 16 ? (lane & 1) == 0 : (lane & 3) == 0; }

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

// NL consecutive float32 values from LDS (16-byte reads, the same address for a half-wave).
template <int NL>
__device__ __forceinline__ void lds_half_row(const float* row, float (&v)[NL]) {
#pragma unroll
  for (int k = 0; k < NL / 4; ++k) {
    const float4 w = *reinterpret_cast<const float4*>(row + 4 * k);
    v[4 * k] = w.x; v[4 * k + 1] = w.y; v[4 * k + 2] = w.z; v[4 * k + 3] = w.w;
  }
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(N == 16 ? 3 : 2, N == 16 ? 3 : 2))) void kvssm_scan_bwd_kernel(
    ScanBwdParams p) {
  constexpr int NL = N / 2;              // states per lane
  constexpr int PB = BlockLen<N>::value;
  constexpr int Q = NL;                  // reduced quantities per lane and token (dCm, then dBm)
  __shared__ float red[PB][2 * N];       // per-block channel sums: dCm[n] at n, dBm[n] at N + n
  __shared__ float sbc[2][PB][N];        // the block's Bm and Cm rows (shared by every channel)

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
  const T* __restrict__ BM0 = static_cast<const T*>(sd.bm);
  const T* __restrict__ CM0 = static_cast<const T*>(sd.cm);
  const T* __restrict__ GY = static_cast<const T*>(sd.gy);
  const T* __restrict__ GB = static_cast<const T*>(sd.gb);

  for (int k = tid; k < PB * 2 * N; k += kThreads) (&red[0][0])[k] = 0.f;

  float A2[NL], dA[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) { A2[n] = sd.A[c * N + n0 + n] * kLog2e; dA[n] = 0.f; }
  const float Dc = sd.D[c], bias = sd.bias[c];
  float dD = 0.f, dbias = 0.f;
  // LDS slots of this lane's summed quantities after the reductions
  const int red_c = n0 + reduced_index<Q>(lane);        // dCm
  const int red_b = N + red_c;                         // dBm
  const bool red_writer = reduced_writer<Q>(lane);

  // One block of nb tokens starting at bs of chunk q [cs, ce); dh carries the state gradient
  // from the block after it. FULL: nb == PB (the common case of chunks of PB tokens): no guards,
  // every per-token load of the block issued at its start.
  float dh[NL];
  auto block = [&](auto full_tag, int q, int cs, int ce, int bs, int nb) {
    constexpr bool FULL = decltype(full_tag)::value;
    // state before the block, recomputed from the chunk start (zero for a block that starts
    // its chunk, as a full one does)
    float h0[NL];
#pragma unroll
    for (int n = 0; n < NL; ++n) h0[n] = 0.f;
    if constexpr (!FULL) {
      for (int t = cs; t < bs; ++t) {
        const int o = t * d + c;
        const float delta = softplus_f32(to_f32(DT[o]) + bias);
        const float u = delta * to_f32(X[o]);
        float b[NL];
        load_half_row<T, NL>(BM + t * N, b);
#pragma unroll
        for (int n = 0; n < NL; ++n) h0[n] = fmaf(hw_exp2(delta * A2[n]), h0[n], u * b[n]);
      }
    }
    // the block's Bm and Cm rows into LDS (the previous block's readers have passed the
    // barrier that ended it)
    for (int k = tid; k < 2 * PB * N; k += kThreads) {
      const int w = k / (PB * N), j = (k / N) % PB, n = k % N;
      if (j < nb) (&sbc[0][0][0])[k] = to_f32((w ? CM0 : BM0)[(bs + j) * N + n]);
    }
    __syncthreads();
    // per-token inputs of the block
    float xs[PB], zs[PB], gs[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      if (FULL || j < nb) {
        const int o = (bs + j) * d + c;
        xs[j] = to_f32(X[o]);
        zs[j] = to_f32(DT[o]) + bias;
        gs[j] = to_f32(GY[o]);
        if (GB && (FULL ? j == PB - 1 : bs + j == ce - 1)) gs[j] += to_f32(GB[q * d + c]);
      }
    }
    // the block's states; dCm_t = sum over channels of g_t h_t needs no state gradient and is
    // reduced here
    float hb[PB][NL];
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      if (FULL || j < nb) {
        const float delta = softplus_f32(zs[j]);
        const float u = delta * xs[j];
        float b[NL], part[Q];
        lds_half_row<NL>(&sbc[0][j][n0], b);
#pragma unroll
        for (int n = 0; n < NL; ++n) {
          const float hp = j == 0 ? h0[n] : hb[j > 0 ? j - 1 : 0][n];
          hb[j][n] = fmaf(hw_exp2(delta * A2[n]), hp, u * b[n]);
          part[n] = gs[j] * hb[j][n];
        }
        half_reduce_scatter<Q>(part, lane);
        if (active && red_writer) atomicAdd(&red[j][red_c], part[0]);
      }
    }
    // reverse through the block
#pragma unroll
    for (int j = PB - 1; j >= 0; --j) {
      if (FULL || j < nb) {
        const int t = bs + j;
        const int o = t * d + c;
        const float g = gs[j], xv = xs[j];
        // delta and the decays are recomputed, not kept from the forward pass (which would hold
        // PB * (NL + 1) more registers): hide z's identity from common-subexpression elimination
        float z = zs[j];
        asm volatile("" : "+v"(z));
        const float delta = softplus_f32(z);
        const float u = delta * xv;
        float b[NL], cc[NL];
        lds_half_row<NL>(&sbc[0][j][n0], b);
        lds_half_row<NL>(&sbc[1][j][n0], cc);
        float du = 0.f, dd = 0.f;
        float part[Q];
#pragma unroll
        for (int n = 0; n < NL; ++n) {
          dh[n] = fmaf(g, cc[n], dh[n]);
          part[n] = dh[n] * u;
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
        if (active && red_writer) atomicAdd(&red[j][red_b], part[0]);
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
  };

  const int q0 = group * kChunksPerGroup;
  const int q1 = min(q0 + kChunksPerGroup, p.n_chunks);
  for (int q = q0; q < q1; ++q) {
    const int cs = p.chunk_cu[q], ce = p.chunk_cu[q + 1];
#pragma unroll
    for (int n = 0; n < NL; ++n) dh[n] = 0.f;
    if (ce - cs == PB) {
      block(std::true_type{}, q, cs, ce, cs, PB);
    } else {
      for (int bs = cs + ((ce - cs - 1) / PB) * PB; bs >= cs; bs -= PB)
        block(std::false_type{}, q, cs, ce, bs, min(PB, ce - bs));
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
