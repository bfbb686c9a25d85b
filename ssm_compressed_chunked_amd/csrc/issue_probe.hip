// Issue-rate microbenchmark for gfx950: how many shader clocks a SIMD needs per wave64
// instruction of the kinds the KV-SSM scan and the chunk attention are made of. It backs the
// instruction-issue rooflines quoted for those kernels; it is not part of the method.
//
// Every wave runs `iters` iterations of an unrolled block of independent instruction chains
// and reads the shader clock (s_memtime) and the constant 100 MHz clock (s_memrealtime)
// before and after, and where it ran (the hardware ids of its XCD, shader engine, CU and SIMD).
// Launched with W workgroups of 4 waves per CU, most SIMDs hold W waves; for every SIMD the
// host divides the span from the first wave's start to the last wave's end by the instructions
// its waves issued, and uses the SIMDs whose waves all ran side by side. dclk / (dreal /
// 100 MHz) is the shader clock.
//
// Built as its own library (libattamba_probe.so), apart from libattamba.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Op {
  kFmaV = 0,      // v_fma_f32 (64-bit VOP3 encoding), all operands in VGPRs
  kFmaS = 1,      // v_fma_f32 (VOP3) with one wave-uniform (SGPR) operand
  kMulV = 2,      // v_mul_f32 (32-bit VOP2 encoding), VGPR operands
  kExp = 3,       // v_exp_f32 with a negated source (VOP3 encoding)
  kMfma = 4,      // v_mfma_f32_32x32x16_bf16
  kScanUpdate = 5,// one state update of the scan: mul, exp, mul (SGPR), fma, fma (SGPR)
  kFmacV = 6,     // v_fmac_f32 (VOP2: the accumulator is the destination), VGPR operands
  kFmacS = 7,     // v_fmac_f32 (VOP2) with one SGPR operand
  kAddV = 8,      // v_add_f32 (VOP2)
  kExpMul = 9,    // v_exp_f32 (32-bit VOP1 encoding) followed by v_mul_f32 (VOP2, VGPR)
  kFmamk = 10,    // v_fmamk_f32 (VOP2 with a 32-bit literal operand)
  kCvtPk = 11,    // v_cvt_pk_bf16_f32 (two float32 to a bf16 pair)
  kDot2 = 12,     // v_dot2 of a bf16 pair with a bf16 pair, float32 accumulator
  kExpFmac = 13,  // v_exp_f32 chains interleaved with independent v_fmac_f32 chains
  kMfmaFmac = 14, // v_mfma_f32_32x32x16_bf16 chains with 8 independent v_fmac_f32 per MFMA
  kMfmaExp = 15,  // the same with 8 independent v_exp_f32 per MFMA
  kMfmaFma3 = 16, // the same with 8 independent v_fma_f32 (VOP3) per MFMA
  kMulDpp = 17,   // v_mul_f32 whose first operand is lane n of each row of 16 (DPP row_newbcast)
  kFmacDpp = 18,  // v_fmac_f32 with such a broadcast operand
  kScanDpp = 19   // the scan's state update with the rows as broadcast operands of VGPRs
};

constexpr int kChains = 8;      // independent chains per lane (VALU ops)
constexpr int kUnroll = 8;      // chain steps per loop iteration
constexpr int kMfmaChains = 4;  // independent accumulators (MFMA)
constexpr int kStates = 16;     // state size of the scan-update block
constexpr int kTokens = 8;      // tokens per iteration of the scan-update block
constexpr int kOutPerWave = 6;

struct ScanRows {
  float b[kStates], c[kStates];  // wave-uniform rows, passed by value so they sit in SGPRs
};

__device__ __forceinline__ void stamp(uint64_t& clk, uint64_t& rt) {
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_sched_barrier(0);
  clk = __builtin_amdgcn_s_memtime();
  rt = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_sched_barrier(0);
}

// x * (lane n of each 16-lane row of v), and acc + (lane n of each row of v) * x, with the
// broadcast as a DPP operand of the VALU instruction (gfx90a and later)
template <int n>
__device__ __forceinline__ float mul_bcast(float v, float x) {
  float r;
  asm volatile("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "=v"(r) : "v"(v), "v"(x), "i"(n));
  return r;
}
template <int n>
__device__ __forceinline__ void fmac_bcast(float& acc, float v, float x) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "+v"(acc) : "v"(v), "v"(x), "i"(n));
}

// the scan's update for states n .. kStates - 1 with broadcast row operands (bb: lane i of every
// row holds b[i], bc: c[i])
template <int n>
struct DppStates {
  static __device__ __forceinline__ void run(float (&h)[kStates], const float (&a2)[kStates],
                                             float delta, float u, float bb, float bc, float& y0,
                                             float& y1) {
    if constexpr (n < kStates) {
      const float e = __builtin_amdgcn_exp2f(delta * a2[n]);
      const float inj = mul_bcast<n>(bb, u);
      h[n] = fmaf(e, h[n], inj);
      if (n & 1) fmac_bcast<n>(y1, bc, h[n]);
      else fmac_bcast<n>(y0, bc, h[n]);
      DppStates<n + 1>::run(h, a2, delta, u, bb, bc, y0, y1);
    }
  }
};

// out[kOutPerWave * wave + {0 .. 5}] = clock before, clock after, real time before, after, the
// HW_ID register (SIMD, CU, shader array and engine of the wave) and the XCC_ID register;
// sink[thread] keeps the chains live.
template <int OP>
__global__ __launch_bounds__(256) void issue_probe_kernel(int iters, float s, const float* vin,
                                                          ScanRows rows, uint64_t* out,
                                                          float* sink) {
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  const int wave = gt >> 6;
  const float a = vin[threadIdx.x & 63];
  const float b = vin[64 + (threadIdx.x & 63)];
  const float cm = vin[128 + (threadIdx.x & 63)];   // a multiplier below 0.53
  uint64_t c0, r0, c1, r1;
  float acc[kStates];
#pragma unroll
  for (int j = 0; j < kStates; ++j) acc[j] = a + 0.01f * j;
  float result = 0.f;
  if constexpr (OP == kMfma) {
    bf16x8 fa, fb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      fa[e] = static_cast<__bf16>(a * (e + 1));
      fb[e] = static_cast<__bf16>(b * (e + 1));
    }
    f32x16 m[kMfmaChains];
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) m[j][v] = 0.f;
    stamp(c0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < kUnroll / 2; ++u)
#pragma unroll
        for (int j = 0; j < kMfmaChains; ++j)
          m[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, m[j], 0, 0, 0);
    }
    stamp(c1, r1);
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) result += m[j][v];
  } else if constexpr (OP == kMfmaFmac || OP == kMfmaExp || OP == kMfmaFma3) {
    bf16x8 fa, fb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      fa[e] = static_cast<__bf16>(a * (e + 1));
      fb[e] = static_cast<__bf16>(b * (e + 1));
    }
    f32x16 m[kMfmaChains];
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) m[j][v] = 0.f;
    stamp(c0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < kUnroll / 2; ++u)
#pragma unroll
        for (int j = 0; j < kMfmaChains; ++j) {
          m[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, m[j], 0, 0, 0);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            float& r = acc[(j * 8 + k) % kStates];
            if constexpr (OP == kMfmaFmac) r = fmaf(a, b, r);
            else if constexpr (OP == kMfmaExp) r = __builtin_amdgcn_exp2f(-r);
            else r = fmaf(r, a, b);
          }
        }
    }
    stamp(c1, r1);
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) result += m[j][v];
#pragma unroll
    for (int j = 0; j < kStates; ++j) result += acc[j];
  } else if constexpr (OP == kScanDpp) {
    // as kScanUpdate, with the rows held in VGPRs (lane i of every 16-lane row holds b[i] and
    // c[i]) and read as DPP broadcast operands instead of SGPRs
    float a2[kStates];
#pragma unroll
    for (int j = 0; j < kStates; ++j) a2[j] = -(1.0f + 0.5f * j) * (1.0f + 0.001f * a);
    const float bb = 0.5f + 0.01f * (threadIdx.x & 15), bc = 0.25f + 0.02f * (threadIdx.x & 15);
    float delta = 0.05f + 0.01f * b, u = a, ysum = 0.f;
    stamp(c0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int t = 0; t < kTokens; ++t) {
        float y0 = 0.f, y1 = 0.f;
        DppStates<0>::run(acc, a2, delta, u, bb, bc, y0, y1);
        ysum += y0 + y1;
        u = fmaf(u, 0.999f, 1e-4f);
        delta = fmaf(delta, 0.999f, 1e-4f);
      }
    }
    stamp(c1, r1);
    result = ysum;
  } else if constexpr (OP == kScanUpdate) {
    // per token, delta and u change, and every state n does
    //   e = 2^(delta * a2[n]); inj = u * b[n]; h[n] = e h[n] + inj; y += h[n] c[n]
    // (the scan's inner work without its loads, stores and softplus); kTokens tokens per
    // iteration, unrolled as the scan unrolls a chunk
    float a2[kStates];
#pragma unroll
    for (int j = 0; j < kStates; ++j) a2[j] = -(1.0f + 0.5f * j) * (1.0f + 0.001f * a);
    float delta = 0.05f + 0.01f * b, u = a, ysum = 0.f;
    stamp(c0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int t = 0; t < kTokens; ++t) {
        float y0 = 0.f, y1 = 0.f;
#pragma unroll
        for (int n = 0; n < kStates; ++n) {
          const float e = __builtin_amdgcn_exp2f(delta * a2[n]);
          const float inj = u * rows.b[n];
          acc[n] = fmaf(e, acc[n], inj);
          if (n & 1) y1 = fmaf(acc[n], rows.c[n], y1);
          else y0 = fmaf(acc[n], rows.c[n], y0);
        }
        ysum += y0 + y1;
        u = fmaf(u, 0.999f, 1e-4f);
        delta = fmaf(delta, 0.999f, 1e-4f);
      }
    }
    stamp(c1, r1);
    result = ysum;
  } else {
    stamp(c0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kChains; ++j) {
          if constexpr (OP == kFmaV) acc[j] = fmaf(acc[j], a, b);
          else if constexpr (OP == kFmaS) acc[j] = fmaf(acc[j], s, b);
          else if constexpr (OP == kMulV) acc[j] = acc[j] * a;
          else if constexpr (OP == kFmacV) acc[j] = fmaf(a, b, acc[j]);
          else if constexpr (OP == kFmacS) acc[j] = fmaf(s, b, acc[j]);
          else if constexpr (OP == kAddV) acc[j] = acc[j] + a;
          else if constexpr (OP == kExpMul) acc[j] = __builtin_amdgcn_exp2f(acc[j]) * cm;
          else if constexpr (OP == kFmamk) acc[j] = fmaf(acc[j], 0.8273f, b);
          else if constexpr (OP == kCvtPk) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 pp = {static_cast<__bf16>(acc[j]), static_cast<__bf16>(a)};
            acc[j] = __builtin_bit_cast(float, pp);
          } else if constexpr (OP == kDot2) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 pa = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
            const bf16x2 pb = {static_cast<__bf16>(b), static_cast<__bf16>(a)};
            acc[j] = __builtin_amdgcn_fdot2_f32_bf16(pa, pb, acc[j], false);
          } else if constexpr (OP == kExpFmac) {
            if (j & 1) acc[j] = fmaf(a, b, acc[j]);
            else acc[j] = __builtin_amdgcn_exp2f(-acc[j]);
          }
          else if constexpr (OP == kMulDpp) acc[j] = mul_bcast<3>(cm, acc[j]);
          else if constexpr (OP == kFmacDpp) fmac_bcast<5>(acc[j], a, b);
          else acc[j] = __builtin_amdgcn_exp2f(-acc[j]);   // converges; never overflows
        }
    }
    stamp(c1, r1);
#pragma unroll
    for (int j = 0; j < kChains; ++j) result += acc[j];
  }
  sink[gt] = result;
  unsigned hw_id, xcc_id;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw_id));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc_id));
  if ((threadIdx.x & 63) == 0) {
    uint64_t* o = out + kOutPerWave * wave;
    o[0] = c0;
    o[1] = c1;
    o[2] = r0;
    o[3] = r1;
    o[4] = hw_id;
    o[5] = xcc_id;
  }
}

// Streaming read: each step a workgroup reads one contiguous block of kReadUnroll x 256 16-byte
// pieces (thread t takes pieces t, t + 256, ...: eight loads in flight per thread, each load
// instruction covering 1 KB per wave), then moves on by the grid's span; every thread writes one
// value, so no load is dropped. The host times the launch with events; bytes / time is the read
// bandwidth a kernel that only reads can reach.
constexpr int kReadUnroll = 8;
__global__ __launch_bounds__(256) void read_stream_kernel(const uint4* __restrict__ buf, size_t n16,
                                                          float* __restrict__ sink) {
  constexpr size_t kStep = kReadUnroll * 256;
  const size_t span = static_cast<size_t>(gridDim.x) * kStep;
  uint32_t acc = 0;
  size_t base = static_cast<size_t>(blockIdx.x) * kStep;
  for (; base + kStep <= n16; base += span) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) v[k] = buf[base + k * 256 + threadIdx.x];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) acc += v[k].x ^ v[k].w;
  }
  for (size_t i = base + threadIdx.x; i < n16; i += 256) acc += buf[i].x;   // the last partial block
  sink[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = static_cast<float>(acc);
}

}  // namespace

extern "C" {

// Instructions of the probed kind that one wave issues per loop iteration.
int attamba_probe_ops_per_iter(int op) {
  switch (op) {
    case kFmaV: case kFmaS: case kMulV: case kExp: case kFmacV: case kFmacS: case kAddV:
    case kFmamk: case kCvtPk: case kDot2: case kMulDpp: case kFmacDpp: return kChains * kUnroll;
    case kExpMul: return kChains * kUnroll;            // exp + mul pairs
    case kExpFmac: return kChains * kUnroll / 2;       // exp + fmac pairs
    case kMfma: case kMfmaFmac: case kMfmaExp: case kMfmaFma3:
      return kMfmaChains * kUnroll / 2;   // MFMAs (each with 8 VALU instructions beside it)
    case kScanUpdate: case kScanDpp: return kStates * kTokens;   // state updates per iteration
    default: return -1;
  }
}

// Runs the probe `op` with `blocks` workgroups of 256 threads (4 waves). vin: 192 floats on the
// device (operand values; the last 64 below 0.53). out: 6 * 4 * blocks uint64 on the device (per wave: clock before,
// clock after, real time before, after, HW_ID, XCC_ID). sink: blocks * 256 floats on the
// device. Returns 0 or a HIP error code; 1 for an unknown op or bad sizes.
int attamba_probe_issue(int op, int blocks, int iters, float s, const float* vin,
                        const float* rows_host, uint64_t* out, float* sink, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || !vin || !out || !sink || !rows_host) return 1;
  ScanRows rows;
  for (int n = 0; n < kStates; ++n) {
    rows.b[n] = rows_host[n];
    rows.c[n] = rows_host[kStates + n];
  }
  const dim3 grid(blocks), block(256);
  switch (op) {
    case kFmaV: hipLaunchKernelGGL(issue_probe_kernel<kFmaV>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kFmaS: hipLaunchKernelGGL(issue_probe_kernel<kFmaS>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kMulV: hipLaunchKernelGGL(issue_probe_kernel<kMulV>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kExp: hipLaunchKernelGGL(issue_probe_kernel<kExp>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kMfma: hipLaunchKernelGGL(issue_probe_kernel<kMfma>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kScanUpdate: hipLaunchKernelGGL(issue_probe_kernel<kScanUpdate>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kFmacV: hipLaunchKernelGGL(issue_probe_kernel<kFmacV>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kFmacS: hipLaunchKernelGGL(issue_probe_kernel<kFmacS>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kAddV: hipLaunchKernelGGL(issue_probe_kernel<kAddV>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kExpMul: hipLaunchKernelGGL(issue_probe_kernel<kExpMul>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kFmamk: hipLaunchKernelGGL(issue_probe_kernel<kFmamk>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kCvtPk: hipLaunchKernelGGL(issue_probe_kernel<kCvtPk>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kDot2: hipLaunchKernelGGL(issue_probe_kernel<kDot2>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kExpFmac: hipLaunchKernelGGL(issue_probe_kernel<kExpFmac>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kMfmaFmac: hipLaunchKernelGGL(issue_probe_kernel<kMfmaFmac>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kMfmaExp: hipLaunchKernelGGL(issue_probe_kernel<kMfmaExp>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kMfmaFma3: hipLaunchKernelGGL(issue_probe_kernel<kMfmaFma3>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kMulDpp: hipLaunchKernelGGL(issue_probe_kernel<kMulDpp>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kFmacDpp: hipLaunchKernelGGL(issue_probe_kernel<kFmacDpp>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    case kScanDpp: hipLaunchKernelGGL(issue_probe_kernel<kScanDpp>, grid, block, 0, stream, iters, s, vin, rows, out, sink); break;
    default: return 1;
  }
  return static_cast<int>(hipGetLastError());
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) of device memory once with `blocks`
// workgroups of 256 threads; sink: blocks * 256 floats on the device. Returns 0 or a HIP error
// code; 1 for bad arguments.
int attamba_probe_read_stream(const void* buf, size_t bytes, float* sink, int blocks,
                              hipStream_t stream) {
  if (!buf || !sink || blocks < 1 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return 1;
  hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
