// Chunk-aware causal attention on the bf16 matrix cores of gfx950 (pith.science review of
// "Attamba: Attending To Multi-Token States", "What carries the argument": M_train Eq. 5,
// M_test Eq. 7, window of L leading tokens Eq. 8).
//
// Workgroup = 4 waves = 128 query rows of one (sequence, head); wave = 32 rows. Keys come in
// tiles of 64, first the compact boundary states kb/vb (chunks that end before the window of
// the workgroup's last row), then the per-token keys of the band [w(first row), last row].
// Each tile is staged in LDS (double-buffered: the next tile's global loads are in flight
// while the current one is computed):
//   K rows as they are in memory ([key][hd], rows padded to 16 B past hd so that the 32 key
//   rows a wave reads with ds_read_b128 fall on distinct banks);
//   V transposed to [hd][key] (rows padded by 8 B) so that the PV operand is two 8-byte reads.
// Per tile and wave:
//   S^T (keys x queries) = K Q^T        v_mfma_f32_32x32x16_bf16, Q held in registers
//   online softmax in float32 per query (one lane per query and key half; the two halves
//   meet with one cross-lane max per tile), masking only in tiles that straddle a row's
//   visible range and skipping tiles no row of the wave can see;
//   O^T (hd x queries) += V^T P^T       v_mfma_f32_32x32x16_bf16.
// S^T puts one query per lane, so the softmax statistics, the rescale of O^T and the final
// division are per-lane operations; the P operand of the second product is the first
// product's accumulator converted to bf16 in place (the keys are taken in the accumulator's
// row order, and V^T is read in the same order).
#include <climits>

#include "common.h"
#include "kernels.h"

namespace attamba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int NT = 256;   // threads per workgroup

struct Geo {
  int w;   // first band position
  int E;   // visible boundary states
};

__device__ __forceinline__ Geo geo(const AttnParams& p, int i, int s0, int s1, int c0) {
  Geo g;
  int w = i - p.L + 1;
  if (w < s0) w = s0;
  if (p.train) {
    const int cs = p.chunk_cu[p.token_chunk[i]];
    if (cs < w) w = cs;
  }
  g.w = w;
  g.E = (w < s1) ? p.token_chunk[w] - c0 : p.token_chunk[s1 - 1] + 1 - c0;
  return g;
}

template <int HD>
struct Smem {
  static constexpr int KST = HD + 8;   // K row stride (elements)
  static constexpr int VST = BN + 4;   // V^T row stride (elements)
  __bf16 k[2][BN * KST];
  __bf16 v[2][HD * VST];
};

template <int HD>
struct TileRegs {
  static constexpr int KU = BN * HD / 8 / NT;        // 16-byte K pieces per thread
  static constexpr int VU = (HD / 8) * (BN / 2) / NT; // (hd group, key pair) units per thread
  uint4 k[KU];
  uint4 v0[VU], v1[VU];
};

// Global -> registers for one tile of keys base .. base + BN - 1. Keys past `top` (the last
// valid key) re-read row `top` instead of branching around the load: every row that could
// see such a key masks it. Offsets are 32-bit (element counts below 2^31, checked at the ABI).
template <int HD>
__device__ __forceinline__ void tile_load(TileRegs<HD>& r, const __bf16* __restrict__ kp,
                                          const __bf16* __restrict__ vp, int base, int top,
                                          int hs, int tid) {
#pragma unroll
  for (int u = 0; u < TileRegs<HD>::KU; ++u) {
    const int piece = tid + u * NT;
    const int key = piece / (HD / 8), seg = piece % (HD / 8);
    const int kk = min(base + key, top);
    r.k[u] = *reinterpret_cast<const uint4*>(kp + (kk * hs + seg * 8));
  }
#pragma unroll
  for (int u = 0; u < TileRegs<HD>::VU; ++u) {
    const int unit = tid + u * NT;
    const int gq = unit % (HD / 8), kp2 = unit / (HD / 8);
    const int k0 = min(base + 2 * kp2, top), k1 = min(base + 2 * kp2 + 1, top);
    r.v0[u] = *reinterpret_cast<const uint4*>(vp + (k0 * hs + gq * 8));
    r.v1[u] = *reinterpret_cast<const uint4*>(vp + (k1 * hs + gq * 8));
  }
}

// Registers -> LDS: K rows as they are; V transposed to [hd][key], two keys per 32-bit word.
template <int HD>
__device__ __forceinline__ void tile_store(const TileRegs<HD>& r, __bf16* sk, __bf16* sv, int tid) {
  constexpr int KST = Smem<HD>::KST, VST = Smem<HD>::VST;
#pragma unroll
  for (int u = 0; u < TileRegs<HD>::KU; ++u) {
    const int piece = tid + u * NT;
    const int key = piece / (HD / 8), seg = piece % (HD / 8);
    *reinterpret_cast<uint4*>(sk + key * KST + seg * 8) = r.k[u];
  }
#pragma unroll
  for (int u = 0; u < TileRegs<HD>::VU; ++u) {
    const int unit = tid + u * NT;
    const int gq = unit % (HD / 8), kp2 = unit / (HD / 8);
    const uint32_t a[4] = {r.v0[u].x, r.v0[u].y, r.v0[u].z, r.v0[u].w};
    const uint32_t b[4] = {r.v1[u].x, r.v1[u].y, r.v1[u].z, r.v1[u].w};
    uint32_t* dst = reinterpret_cast<uint32_t*>(sv + (gq * 8) * VST + 2 * kp2);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      dst[(2 * e2) * (VST / 2)] = (a[e2] & 0xffffu) | (b[e2] << 16);
      dst[(2 * e2 + 1) * (VST / 2)] = (a[e2] >> 16) | (b[e2] & 0xffff0000u);
    }
  }
}

template <int HD>
__global__ __launch_bounds__(NT) void attn_mfma_kernel(AttnParams p) {
  constexpr int KST = Smem<HD>::KST, VST = Smem<HD>::VST;
  constexpr int QS = HD / 16;     // k-steps of S^T (16 hd each)
  constexpr int OB = HD / 32;     // 32-row hd blocks of O^T
  __shared__ Smem<HD> sm;

  // Workgroups go round-robin to the 8 XCDs (id mod 8), each with its own L2. All query tiles
  // of one (sequence, head) are placed on one XCD, consecutively, so that its boundary-state
  // prefix is fetched into that L2 once; within a (sequence, head) the tiles with the most
  // keys (the last rows) are issued first so that light tiles form the tail of the grid.
  const int n_qt = ceil_div(p.max_seqlen, BM);
  const int id = blockIdx.x, slot = id >> 3;
  const int bh = (slot / n_qt) * 8 + (id & 7);
  if (bh >= p.S * p.H) return;
  const int s = bh / p.H, h = bh % p.H;
  const int qt = n_qt - 1 - slot % n_qt;
  const int s0 = p.seq_cu[s], s1 = p.seq_cu[s + 1];
  const int r0 = s0 + qt * BM;
  if (r0 >= s1) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int q = lane & 31, hf = lane >> 5;
  const int last = min(r0 + BM, s1) - 1;
  const int c0 = p.token_chunk[s0];
  const size_t hs = static_cast<size_t>(p.H) * HD;   // row stride of [., H, HD]

  // this lane's row, and the wave's row range (rows past the sequence mimic its last row)
  const int i = r0 + wid * 32 + q;
  const bool valid = i < s1;
  const int ic = valid ? i : last;
  const Geo g = geo(p, ic, s0, s1, c0);
  const int wr0 = min(r0 + wid * 32, last), wr1 = min(r0 + wid * 32 + 31, last);
  const int Ew0 = __shfl(g.E, 0), Ew1 = __shfl(g.E, 31);
  const int ww0 = __shfl(g.w, 0), ww1 = __shfl(g.w, 31);
  // the workgroup's key ranges
  const Geo gl = geo(p, last, s0, s1, c0);
  const Geo gf = geo(p, r0, s0, s1, c0);
  const int nbt = ceil_div(gl.E, BN);
  const int band0 = gf.w;
  const int nbd = last >= band0 ? ceil_div(last - band0 + 1, BN) : 0;
  const int ntiles = nbt + nbd;

  // Q^T operand: lane (q, hf) holds hd 16 st + 8 hf .. +7 of its row
  bf16x8 qf[QS];
  {
    const __bf16* qr = static_cast<const __bf16*>(p.q) + ic * hs + h * HD + 8 * hf;
#pragma unroll
    for (int st = 0; st < QS; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qr + 16 * st);
  }
  f32x16 o[OB];
#pragma unroll
  for (int j = 0; j < OB; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[j][v] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c = p.scale * kLog2e;

  const __bf16* kbp = static_cast<const __bf16*>(p.kb) + h * HD;
  const __bf16* vbp = static_cast<const __bf16*>(p.vb) + h * HD;
  const __bf16* ktp = static_cast<const __bf16*>(p.k) + h * HD;
  const __bf16* vtp = static_cast<const __bf16*>(p.v) + h * HD;

  const int hs32 = p.H * HD;
  const int topb = c0 + gl.E - 1;   // last boundary key of the workgroup
  // tile t: boundary tiles first, then band tiles
  auto src_k = [&](int t) { return t < nbt ? kbp : ktp; };
  auto src_v = [&](int t) { return t < nbt ? vbp : vtp; };
  auto base_of = [&](int t) { return t < nbt ? c0 + t * BN : band0 + (t - nbt) * BN; };
  auto top_of = [&](int t) { return t < nbt ? topb : last; };
  TileRegs<HD> regs;
  if (ntiles > 0) {
    tile_load<HD>(regs, src_k(0), src_v(0), base_of(0), top_of(0), hs32, tid);
    tile_store<HD>(regs, sm.k[0], sm.v[0], tid);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    const int tn = more ? t + 1 : t;
    tile_load<HD>(regs, src_k(tn), src_v(tn), base_of(tn), top_of(tn), hs32, tid);

    // which rows of this wave see which keys of the tile
    const bool bnd = t < nbt;
    const int base = bnd ? c0 + t * BN : band0 + (t - nbt) * BN;
    bool skip, full;
    if (bnd) {
      skip = base >= c0 + Ew1;
      full = base + BN <= c0 + Ew0;
    } else {
      skip = base > wr1 || base + BN - 1 < ww0;
      full = base >= ww1 && base + BN - 1 <= wr0;
    }
    if (!skip) {
      const __bf16* sk = sm.k[buf];
      const __bf16* sv = sm.v[buf];
      bf16x8 ka[2][QS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < QS; ++st)
          ka[kb][st] = *reinterpret_cast<const bf16x8*>(sk + (32 * kb + q) * KST + 16 * st + 8 * hf);
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
        for (int st = 0; st < QS; ++st)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][st], qf[st], sacc[kb], 0, 0, 0);
      }
      // V^T fragments of this tile (read while the products above drain)
      bf16x8 va[OB][4];
#pragma unroll
      for (int j = 0; j < OB; ++j) {
        const __bf16* vrow = sv + (32 * j + q) * VST + 4 * hf;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + 16 * ks);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 16 * ks + 8);
          va[j][ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
      // accumulator row v of block kb is key 32 kb + 8 (v / 4) + 4 hf + v % 4
      float sc[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[16 * kb + v] = sacc[kb][v];
      if (!full) {
        const int lo = bnd ? INT_MIN : g.w;
        const int hi = bnd ? c0 + g.E - 1 : ic;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = base + 32 * kb + 8 * (v >> 2) + 4 * hf + (v & 3);
            sc[16 * kb + v] = (key >= lo && key <= hi) ? sc[16 * kb + v] : -INFINITY;
          }
      }
      float tm = sc[0];
#pragma unroll
      for (int e = 1; e < 32; ++e) tm = fmaxf(tm, sc[e]);
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float mn = fmaxf(m, tm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = hw_exp2((m - mu) * c);
      const float mc = mu * c;
      float ls = 0.f;
      bf16x8 pk[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pr = hw_exp2(fmaf(sc[8 * ks + e], c, -mc));
          ls += pr;
          pk[ks][e] = static_cast<__bf16>(pr);
        }
      l = fmaf(l, alpha, ls);
      m = mn;
      if (__any(alpha != 1.0f)) {     // wave-uniform: after the first tiles the max rarely moves
#pragma unroll
        for (int j = 0; j < OB; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[j][v] *= alpha;
      }
      // O^T += V^T P^T; k-step ks = 2 kb + sub covers keys 32 kb + 16 sub + {4 hf .. +3, 8 + 4 hf .. +3}
#pragma unroll
      for (int j = 0; j < OB; ++j)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j][ks], pk[ks], o[j], 0, 0, 0);
    }
    if (more) tile_store<HD>(regs, sm.k[buf ^ 1], sm.v[buf ^ 1], tid);
    __syncthreads();
  }

  // epilogue: combine the two key halves of every query, normalise, write O and LSE
  const float lt = l + __shfl_xor(l, 32);
  if (valid) {
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    __bf16* orow = static_cast<__bf16*>(p.out) + i * hs + h * HD + 4 * hf;
#pragma unroll
    for (int j = 0; j < OB; ++j)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = static_cast<__bf16>(o[j][4 * gq + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * j + 8 * gq) = vv;
      }
    if (p.lse && hf == 0)
      p.lse[static_cast<size_t>(h) * p.T + i] = lt > 0.f ? (m * c + hw_log2(lt)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, int hd, hipStream_t stream) {
  const int n_bh8 = ceil_div(p.S * p.H, 8) * 8;
  dim3 grid(ceil_div(p.max_seqlen, BM) * n_bh8);
  if (hd == 64) {
    hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(NT), 0, stream, p);
  } else {
    hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace attamba
