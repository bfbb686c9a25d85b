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
// Workgroup = 8 waves (2 per SIMD), tile 256 features x 256 tokens, K steps of 64; wave
// (wf, wt) owns 64 features x 128 tokens as 2 x 4 blocks of v_mfma_f32_32x32x16_bf16. Both
// operands are K-contiguous, so every operand is one ds_read_b128 from an LDS tile whose 16-byte
// segments are XOR-swizzled by row (conflict-free for 16 consecutive rows). Tiles come from HBM
// straight into LDS (global_load_lds_dwordx4) into two buffers (128 KB, one workgroup per CU),
// one barrier per K step. The large tile halves the bytes each CU pulls from L2 per FLOP
// against 128 x 128 tiles, whose data-return path was busy 83 % of the time.
// Within a K step the operands of k-slice ks + 1 are read from LDS while slice ks's eight
// products run, one read after each of the first six products, in an order fixed by
// scheduling barriers (two register stages, 222 VGPRs, still two waves per SIMD); slice 3's
// products run after the barrier, beside the reads of the next step's slice 0 and the copies
// of the step after it. Without this the wave waited for each slice's reads before its
// products: 910 against 978 TFLOP/s. The epilogue finds each feature group's output segment
// on the scalar unit (a per-lane search had read the output pointers with 64 dependent vector
// loads per wave and tile: 911 against 977 TFLOP/s).
// A last feature tile of at most 64 features (the 4 N rows of Bm/Cm at the prefill shape) goes
// to a separate tail kernel (below) instead of a mostly empty 256 x 256 tile.
#include "common.h"
#include "kernels.h"
#include <type_traits>

namespace attamba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int TM = 256;     // features per tile
constexpr int TN = 256;     // tokens per tile
constexpr int TK = 64;      // K per step
constexpr int NW = 8;       // waves per workgroup
constexpr int NT = NW * 64; // threads per workgroup
constexpr int kChunks = TM * TK * 2 / 1024;     // 1 KB chunks per operand tile (32)
constexpr int kChunksPerWave = kChunks / NW;    // 4

// element offset of logical 16-byte segment s of tile row r (8 segments per row). The LDS
// serves a ds_read_b128 16 lanes at a time from 64 four-byte banks (256 bytes): the 16 lanes
// that read one segment of 16 consecutive rows must hit 16 distinct 16-byte slots of that
// window. Rows of 128 bytes alternate between its two halves, so the swizzle takes row bits
// 1..3 (bits 0..2 put rows r and r + 8 on one slot: 4 conflict cycles on every read).
__device__ __forceinline__ int seg_off(int r, int s) { return r * TK + 8 * (s ^ ((r >> 1) & 7)); }

struct ProjTile {
  __bf16 w[2][TM * TK];
  __bf16 x[2][TN * TK];
};

__global__ __launch_bounds__(NT) void proj_gemm_kernel(ProjParams p) {
  __shared__ ProjTile sm;
  // Workgroups go round-robin to the 8 XCDs (id mod 8), each with its own L2. XCD x owns the
  // token tiles x, x + 8, x + 16, ... and walks, for each feature tile in turn, all of them; the
  // workgroups running at once on an XCD then share a few weight tiles and the XCD's token rows
  // through its L2.
  const int n_ft = ceil_div(p.n_out, TM), n_tt = ceil_div(p.T, TN);
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int n_tx = (n_tt - xcd + 7) / 8;          // token tiles of this XCD
  const int n_tmax = (n_tt + 7) / 8;
  const int m = slot % n_tmax, ft = slot / n_tmax;
  if (m >= n_tx || ft >= n_ft) return;
  const int tt = xcd + 8 * m;
  const int f0 = ft * TM, t0 = tt * TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wid & 3, wt = wid >> 2;          // 64 features x 128 tokens per wave
  const int d = p.d;
  const __bf16* W = static_cast<const __bf16*>(p.w);
  const __bf16* X = static_cast<const __bf16*>(p.x);

  // LDS-direct copies: lane l of chunk ch fills slot ch * 64 + l = (row 8 ch + l / 8, physical
  // segment l % 8), which holds logical segment (l % 8) ^ ((row >> 1) & 7). Rows past the matrix
  // re-read its last row (their results are not stored).
  int woff[kChunksPerWave], xoff[kChunksPerWave];
#pragma unroll
  for (int i = 0; i < kChunksPerWave; ++i) {
    const int ch = wid * kChunksPerWave + i;
    const int r = 8 * ch + lane / 8;
    const int s = (lane % 8) ^ ((r >> 1) & 7);
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
  int aoff[2][4], boff[4][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int i = 0; i < 2; ++i) aoff[i][ks] = seg_off(wf * 64 + 32 * i + q, 2 * ks + hf);
#pragma unroll
    for (int j = 0; j < 4; ++j) boff[j][ks] = seg_off(wt * 128 + 32 * j + q, 2 * ks + hf);
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = d / TK;
  // operands of k-slice ks of LDS buffer buf into register stage st, and the products of stage st
  bf16x8 a[2][2], b[2][4];
  auto rd = [&](int st, int buf, int ks) {
    const __bf16* sw = sm.w[buf];
    const __bf16* sx = sm.x[buf];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[st][i] = *reinterpret_cast<const bf16x8*>(sw + aoff[i][ks]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[st][j] = *reinterpret_cast<const bf16x8*>(sx + boff[j][ks]);
  };
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nk > 1) issue(TK, 1);
  rd(0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  // One K step. The scheduling groups pin the order: a product, then one LDS read of the next
  // slice (0x008 = MFMA, 0x100 = LDS read). ISSUE: copy step kt + 2 into the buffer just freed;
  // RD: read slice 0 of step kt + 1 (both compile-time, so the loop body has no branches).
  // One slice's eight products in a fixed order (each accumulator again 8 products later),
  // with the next slice's six operand reads placed after the first six of them; scheduling
  // barriers keep the order as written.
  auto slice = [&](int st, int buf_next, int ks_next, bool read_next) {
    const int nt = st ^ 1;
    const __bf16* sw = sm.w[buf_next];
    const __bf16* sx = sm.x[buf_next];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = u >> 2, j = u & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st][i], b[st][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (read_next && u < 6) {
        if (u < 2) a[nt][u] = *reinterpret_cast<const bf16x8*>(sw + aoff[u][ks_next]);
        else b[nt][u - 2] = *reinterpret_cast<const bf16x8*>(sx + boff[u - 2][ks_next]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto body = [&](int kt, auto ISSUE, auto RD) {
    const int buf = kt & 1;
    slice(0, buf, 1, true);
    slice(1, buf, 2, true);
    slice(0, buf, 3, true);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's reads of buf and its copies of step kt + 1 are done ...
    __syncthreads();                 // ... and every wave's
    if constexpr (decltype(ISSUE)::value) issue((kt + 2) * TK, buf);
    slice(1, buf ^ 1, 0, decltype(RD)::value);
    __builtin_amdgcn_sched_barrier(0);
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  int kt = 0;
  for (; kt + 2 < nk; ++kt) body(kt, yes{}, yes{});
  if (kt + 1 < nk) {
    body(kt, no{}, yes{});
    ++kt;
  }
  body(kt, no{}, no{});

  // epilogue: block (i, j), register group g: token t0 + 128 wt + 32 j + q, features
  // f0 + 64 wf + 32 i + 8 g + 4 hf .. +3 (all four in one output segment). The wave's groups of
  // 4 features are visited in increasing order, so the segment holding them is found by walking
  // the segment boundaries forward on the scalar unit (one compare per group; constant indices
  // into the parameter block when a boundary is crossed); each lane takes its half's segment.
  int sk = 0;                                          // segment of the current feature
  int s_next = p.n_seg > 1 ? p.seg_start[1] : p.n_out;  // its end
  auto seg_at = [&](int k, __bf16*& out, int& s0, int& end) {
#pragma unroll
    for (int m = 0; m < kMaxProjSegments; ++m)
      if (m == k) {
        out = static_cast<__bf16*>(p.out[m]);
        s0 = p.seg_start[m];
        end = p.seg_start[m + 1];
      }
  };
  __bf16* s_out = static_cast<__bf16*>(p.out[0]);
  int s_s0 = 0;
  auto advance = [&](int f) {
    while (f >= s_next && sk + 1 < p.n_seg) {
      ++sk;
      seg_at(sk, s_out, s_s0, s_next);
    }
  };
  // per-lane destination of each of the 8 feature groups, then the stores token block by
  // token block (the 8 stores of one block complete the wave's 128-byte row pieces together)
  __bf16* gout[2][4];
  int gcol[2][4], gwid[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int fb = f0 + wf * 64 + 32 * i + 8 * g;
      gout[i][g] = nullptr;
      gcol[i][g] = 0;
      gwid[i][g] = 0;
      if (fb >= p.n_out) continue;
      advance(fb);
      __bf16* const out_a = s_out;
      const int col_a = fb - s_s0, w_a = s_next - s_s0;
      advance(fb + 4);
      gout[i][g] = hf ? s_out : out_a;
      gcol[i][g] = hf ? fb + 4 - s_s0 : col_a;
      gwid[i][g] = hf ? s_next - s_s0 : w_a;
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + wt * 128 + 32 * j + q;
    if (t >= p.T) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = f0 + wf * 64 + 32 * i + 8 * g + 4 * hf;
        if (f >= p.n_out) continue;
        bf16x4 vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = static_cast<__bf16>(acc[i][j][4 * g + e]);
        *reinterpret_cast<bf16x4*>(gout[i][g] + static_cast<size_t>(t) * gwid[i][g] + gcol[i][g]) = vv;
      }
  }
}

// Features f_lo .. n_out - 1 when they are the at most kTailMax features of a last, partial
// feature tile. As a tile of their own they would cost a whole tile's products for a quarter
// of its outputs or less, and at the prefill shape (24 full feature tiles x 64 token tiles =
// 6 rounds of one workgroup per CU) a seventh round: 404 us against 370 us for the 24 full
// tiles alone. The tail streams x once more for 64 features, so it is bound by that read.
// A 4-wave workgroup takes 64 features x 64 tokens, each wave one 32 x 32 block of
// v_mfma_f32_32x32x16_bf16; the K steps of 64 come into LDS by LDS-direct copies (the same
// swizzled layout as the large tiles) into a ring of kTailStages buffers, so that the copies of
// the next seven steps are in flight while one step's four products run (with two buffers the
// copy latency was exposed at every step: 23 us; now 15-17 us at the prefill shape).
constexpr int kTailMax = 64;
// s_waitcnt immediate: at most n vector-memory operations of this wave outstanding
constexpr int vmcnt_le(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }
constexpr int kTailTokens = 64;
constexpr int kTailStages = 8;

struct TailTile {
  __bf16 w[kTailStages][kTailMax * TK];
  __bf16 x[kTailStages][kTailTokens * TK];
};

__global__ __launch_bounds__(256) void proj_tail_kernel(ProjParams p, int f_lo) {
  __shared__ TailTile sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 31, hf = lane >> 5;
  const int fb = wid & 1, tb = wid >> 1;           // 32-feature block, 32-token block
  const int t0 = blockIdx.x * kTailTokens;
  const int d = p.d;
  const __bf16* W = static_cast<const __bf16*>(p.w);
  const __bf16* X = static_cast<const __bf16*>(p.x);
  // copies: wave w fills 1 KB chunks w and w + 4 of each 8 KB tile (8 rows of 128 bytes each);
  // lane l holds row 8 ch + l / 8, physical segment l % 8 = logical segment (l % 8) ^ ((row >> 1) & 7)
  int woff[2], xoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = wid + 4 * i;
    const int r = 8 * ch + lane / 8;
    const int sg = (lane % 8) ^ ((r >> 1) & 7);
    woff[i] = min(f_lo + r, p.n_out - 1) * d + 8 * sg;
    xoff[i] = min(t0 + r, p.T - 1) * d + 8 * sg;
  }
  auto issue = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = wid + 4 * i;
      __builtin_amdgcn_global_load_lds(W + woff[i] + k0, LDS_PTR(void, sm.w[buf] + ch * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(X + xoff[i] + k0, LDS_PTR(void, sm.x[buf] + ch * 512), 16, 0, 0);
    }
  };
  const int nk = d / TK;
  constexpr int kLoads = 4;          // copies per wave and step
  f32x16 acc = {};
  for (int s = 0; s < kTailStages - 1; ++s)
    if (s < nk) issue(s * TK, s);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % kTailStages;
    // this wave's copies of step kt have landed (those of the later steps issued so far may
    // still fly) ...
    const int later = min(nk - 1 - kt, kTailStages - 2);
    if (later >= 6) __builtin_amdgcn_s_waitcnt(vmcnt_le(6 * kLoads));
    else if (later == 5) __builtin_amdgcn_s_waitcnt(vmcnt_le(5 * kLoads));
    else if (later == 4) __builtin_amdgcn_s_waitcnt(vmcnt_le(4 * kLoads));
    else if (later == 3) __builtin_amdgcn_s_waitcnt(vmcnt_le(3 * kLoads));
    else if (later == 2) __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * kLoads));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_le(1 * kLoads));
    else __builtin_amdgcn_s_waitcnt(0);
    // ... and every wave's, and every wave is done with step kt - 1's buffer. A bare barrier:
    // the fence of __syncthreads would also wait for the later steps' copies.
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (kt + kTailStages - 1 < nk) issue((kt + kTailStages - 1) * TK, (kt + kTailStages - 1) % kTailStages);
    bf16x8 a[TK / 16], b[TK / 16];   // the step's operands, all read before its products
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      a[ks] = *reinterpret_cast<const bf16x8*>(sm.w[buf] + seg_off(32 * fb + q, 2 * ks + hf));
      b[ks] = *reinterpret_cast<const bf16x8*>(sm.x[buf] + seg_off(32 * tb + q, 2 * ks + hf));
    }
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], b[ks], acc, 0, 0, 0);
  }

  // accumulator register 4 gq + e: feature f_lo + 32 fb + 8 gq + 4 hf + e, token t0 + 32 tb + q;
  // the four features of a group lie in one segment (segments start and end on multiples of 4)
  const int t = t0 + 32 * tb + q;
  if (t >= p.T) return;
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    const int f = f_lo + 32 * fb + 8 * gq + 4 * hf;
    if (f >= p.n_out) continue;
    int sel = 0;
#pragma unroll
    for (int m = 1; m < kMaxProjSegments; ++m)
      if (m < p.n_seg && f >= p.seg_start[m]) sel = m;
    __bf16* out = nullptr;
    int s_lo = 0, width = 0;
#pragma unroll
    for (int m = 0; m < kMaxProjSegments; ++m)
      if (m == sel) {
        out = static_cast<__bf16*>(p.out[m]);
        s_lo = p.seg_start[m];
        width = p.seg_start[m + 1] - s_lo;
      }
    bf16x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = static_cast<__bf16>(acc[4 * gq + e]);
    *reinterpret_cast<bf16x4*>(out + static_cast<size_t>(t) * width + (f - s_lo)) = vv;
  }
}

}  // namespace

hipError_t launch_proj_gemm(const ProjParams& p, hipStream_t stream) {
  if (p.T == 0 || p.n_out == 0) return hipSuccess;
  // a last feature tile with at most kTailMax features goes to the tail kernel
  const int rem = p.n_out % TM;
  const bool tail = rem > 0 && rem <= kTailMax;
  const int n_ft = tail ? p.n_out / TM : ceil_div(p.n_out, TM);
  if (n_ft > 0) {
    const int grid = 8 * n_ft * ceil_div(ceil_div(p.T, TN), 8);
    hipLaunchKernelGGL(proj_gemm_kernel, dim3(grid), dim3(NT), 0, stream, p);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (tail) {
    hipLaunchKernelGGL(proj_tail_kernel, dim3(ceil_div(p.T, kTailTokens)), dim3(256), 0, stream, p,
                       p.n_out - rem);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace attamba
