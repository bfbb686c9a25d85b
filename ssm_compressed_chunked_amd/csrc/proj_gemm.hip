// Input projections of an Attamba layer: the queries and the per-token inputs of the two
// selective SSMs (step size dt, Bm, Cm for SSM_K and SSM_V) are linear maps of the layer input
// x (pith.science review of "Attamba: Attending To Multi-Token States", "Core claim": the SSMs
// take the place of the key and value projections; the selective SSM's inputs are the paper's
// Eq. 3, cited in "Assumptions & free parameters").
//
// Y = x W^T as one bf16 GEMM on the matrix cores: x [T, d] row-major, W [n_out, d] row-major
// (one row per output feature, the stacked weights of q, dt_K, dt_V, Bm_K, Cm_K, Bm_V, Cm_V),
// fp32 accumulation, bf16 outputs written to one tensor per feature segment.
//
// The product is computed transposed, C^T = W x^T, so that an accumulator lane holds one token
// and four consecutive features per register group: each lane stores 8 contiguous bytes.
// Workgroup = 4 waves, tile 128 features x 128 tokens, K steps of 64; wave (wf, wt) owns the
// 64 x 64 quarter (wf, wt) as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16. Both operands are
// K-contiguous, so every operand is one ds_read_b128 from an LDS tile whose 16-byte segments are
// XOR-swizzled by row (conflict-free for 8 consecutive rows). Tiles come from HBM straight into
// LDS (global_load_lds_dwordx4) into two buffers, one barrier per K step.
#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int TM = 128;     // features per tile
constexpr int TN = 128;     // tokens per tile
constexpr int TK = 64;      // K per step
constexpr int NT = 256;     // threads per workgroup
constexpr int kChunks = TM * TK * 2 / 1024;     // 1 KB chunks per operand tile (16)
constexpr int kChunksPerWave = kChunks / 4;     // 4

// element offset of logical 16-byte segment s of tile row r (8 segments per row)
__device__ __forceinline__ int seg_off(int r, int s) { return r * TK + 8 * (s ^ (r & 7)); }

struct ProjTile {
  __bf16 w[2][TM * TK];
  __bf16 x[2][TN * TK];
};

__global__ __launch_bounds__(NT) void proj_gemm_kernel(ProjParams p) {
  __shared__ ProjTile sm;
  // Workgroups go round-robin to the 8 XCDs (id mod 8), each with its own L2. XCD x takes the
  // feature tiles x, x + 8, x + 16, ... (their weight rows, about n_out / 8 x d, stay in its
  // L2) for every token tile in turn; the token tiles' x rows are shared through L2 by the
  // XCD's workgroups running at the same time.
  const int n_ft = ceil_div(p.n_out, TM);
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int n_fx = (n_ft - xcd + 7) / 8;          // feature tiles of this XCD
  const int n_fmax = (n_ft + 7) / 8;
  if (slot % n_fmax >= n_fx) return;
  const int ft = xcd + 8 * (slot % n_fmax), tt = slot / n_fmax;
  if (tt * TN >= p.T) return;
  const int f0 = ft * TM, t0 = tt * TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wid & 1, wt = wid >> 1;
  const int d = p.d;
  const __bf16* W = static_cast<const __bf16*>(p.w);
  const __bf16* X = static_cast<const __bf16*>(p.x);

  // LDS-direct copies: lane l of chunk ch fills slot ch * 64 + l = (row 8 ch + l / 8, physical
  // segment l % 8), which holds logical segment (l % 8) ^ (row & 7). Rows past the matrix
  // re-read its last row (their results are not stored).
  int woff[kChunksPerWave], xoff[kChunksPerWave];
#pragma unroll
  for (int i = 0; i < kChunksPerWave; ++i) {
    const int ch = wid * kChunksPerWave + i;
    const int r = 8 * ch + lane / 8;
    const int s = (lane % 8) ^ (r & 7);
    woff[i] = min(f0 + r, p.n_out - 1) * d + 8 * s;
    xoff[i] = min(t0 + r, p.T - 1) * d + 8 * s;
  }
  auto issue = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
      const int ch = wid * kChunksPerWave + i;
      __builtin_amdgcn_global_load_lds(W + woff[i] + k0, LDS_PTR(void, sm.w[buf] + ch * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(X + xoff[i] + k0, LDS_PTR(void, sm.x[buf] + ch * 512), 16, 0, 0);
    }
  };

  // operand offsets: block i of this wave's features / block j of its tokens, row l % 32,
  // k segment 2 ks + l / 32
  const int q = lane & 31, hf = lane >> 5;
  int aoff[2][4], boff[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      aoff[i][ks] = seg_off(wf * 64 + 32 * i + q, 2 * ks + hf);
      boff[i][ks] = seg_off(wt * 64 + 32 * i + q, 2 * ks + hf);
    }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = d / TK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue((kt + 1) * TK, buf ^ 1);
    const __bf16* sw = sm.w[buf];
    const __bf16* sx = sm.x[buf];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(sw + aoff[i][ks]);
        b[i] = *reinterpret_cast<const bf16x8*>(sx + boff[i][ks]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of step kt + 1 have landed ...
    __syncthreads();                 // ... and every wave is done with step kt
  }

  // epilogue: block (i, j), register group g: token t0 + 64 wt + 32 j + q, features
  // f0 + 64 wf + 32 i + 8 g + 4 hf .. +3 (all four in one output segment)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + wt * 64 + 32 * j + q;
    if (t >= p.T) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = f0 + wf * 64 + 32 * i + 8 * g + 4 * hf;
        if (f >= p.n_out) continue;
        int sgi = 0;
#pragma unroll
        for (int k = 1; k < kMaxProjSegments; ++k)
          if (k < p.n_seg && f >= p.seg_start[k]) sgi = k;
        const int s0 = p.seg_start[sgi], width = p.seg_start[sgi + 1] - s0;
        bf16x4 vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = static_cast<__bf16>(acc[i][j][4 * g + e]);
        __bf16* dst = static_cast<__bf16*>(p.out[sgi]) + static_cast<size_t>(t) * width + (f - s0);
        *reinterpret_cast<bf16x4*>(dst) = vv;
      }
  }
}

}  // namespace

hipError_t launch_proj_gemm(const ProjParams& p, hipStream_t stream) {
  if (p.T == 0 || p.n_out == 0) return hipSuccess;
  const int grid = 8 * ceil_div(ceil_div(p.n_out, TM), 8) * ceil_div(p.T, TN);
  hipLaunchKernelGGL(proj_gemm_kernel, dim3(grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attamba
