// Chunk-aware causal attention on the bf16 matrix cores of gfx950 (pith.science review of
// "Attamba: Attending To Multi-Token States", "What carries the argument": M_train Eq. 5,
// M_test Eq. 7, window of L leading tokens Eq. 8).
//
// Workgroup = 4 waves = 128 query rows of one (sequence, head); wave = 32 rows. Keys come in
// tiles of 64, first the compact boundary states kb/vb (chunks that end before the window of
// the workgroup's last row), then the per-token keys of the band [w(first row), last row].
//
// Tiles go from HBM straight into LDS with global_load_lds_dwordx4 (no VGPR staging): the
// next tile's copy is in flight while the current tile is computed (double buffer, one
// barrier per tile). K and V tiles are stored row-major ([key][hd]) with the 16-byte segments
// of each row permuted by an XOR swizzle of the row index, so that both read patterns below
// hit distinct LDS banks without padding (padding is impossible: a wave's LDS-direct copy
// fills 1 KB contiguously).
// Per tile and wave:
//   S^T (keys x queries) = K Q^T        v_mfma_f32_32x32x16_bf16; Q in registers, the K
//                                        operand is one ds_read_b128 per (key block, k-step);
//   online softmax in float32 per query (one lane per query and key half; the two halves
//   meet with one cross-lane max per tile), masking only in tiles that straddle a row's
//   visible range, skipping tiles no row of the wave can see;
//   O^T (hd x queries) += V^T P^T       v_mfma_f32_32x32x16_bf16; the V^T operand comes from
//                                        the row-major V tile through two ds_read_b64_tr_b16
//                                        (the gfx950 transposing LDS read) per k-step.
// S^T puts one query per lane, so the softmax statistics, the rescale of O^T and the final
// division are per-lane operations; the P operand of the second product is the first
// product's accumulator converted to bf16 in place (keys taken in the accumulator's row order;
// the V^T operand is read in the same order).
#include "common.h"
#include "attn_geom.h"
#include "attn_tiles.h"


namespace attamba {
namespace {

using namespace mfma;

constexpr int NT = 256;   // threads per workgroup

// p = 2^(s c - mu) for the 32 scores of this lane, rounded to bf16 and packed as the P^T
// operand of the second product (k-step ks: keys 16 ks + {4 hf .. +3, 8 + 4 hf .. +3}, in the
// accumulator's row order); returns the lane's sum of the rounded p, kept as two partial sums
// so that the additions form two short dependency chains.
__device__ __forceinline__ float tile_exp(const f32x16 (&sacc)[2], float c, float mu,
                                          bf16x8 (&pk)[4]) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float lt[2] = {0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = hw_exp2(fmaf(sacc[ks >> 1][8 * (ks & 1) + e], c, -mu));
      const float p1 = hw_exp2(fmaf(sacc[ks >> 1][8 * (ks & 1) + e + 1], c, -mu));
      const bf16x2 pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
      lt[ks & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lt[ks & 1], false);
      w[e >> 1] = __builtin_bit_cast(unsigned, pp);
    }
    pk[ks] = __builtin_bit_cast(bf16x8, w);
  }
  return lt[0] + lt[1];
}

constexpr int NBUF = 2;   // tiles in LDS: the current one and the copy in flight

template <int HD>
struct Smem {
  __bf16 k[NBUF][BN * HD];
  __bf16 v[NBUF][BN * HD];
};

template <int HD>
__global__ __launch_bounds__(NT) void attn_mfma_kernel(AttnParams p) {
  constexpr int QS = HD / 16;     // k-steps of S^T (16 hd each)
  constexpr int OB = HD / 32;     // 32-row hd blocks of O^T
  constexpr int BM = 128;         // query rows per workgroup (4 waves x 32)
  __shared__ Smem<HD> sm;

  // Workgroups go round-robin to the 8 XCDs (id mod 8), each with its own L2. Consecutive ids
  // take the same query tile of consecutive (sequence, head) pairs, and the (sequence, head)
  // count is padded to a multiple of 8, so every query tile of one (sequence, head) lands on
  // the same XCD, whose L2 then holds that pair's boundary-state prefix (256 KB per pair at
  // hd 64 and 8 192 tokens, 8 pairs per XCD at a time). The last query tiles, which see the most
  // keys, are issued first over the whole grid, so the tail of the grid is made of light tiles.
  const int n_qt = ceil_div(p.max_seqlen, BM);
  const int n_bh8 = ceil_div(p.S * p.H, 8) * 8;
  const int id = blockIdx.x;
  const int bh = id % n_bh8;
  if (bh >= p.S * p.H) return;
  const int s = bh / p.H, h = bh % p.H;
  const int qt = n_qt - 1 - id / n_bh8;
  const int s0 = p.seq_cu[s], s1 = p.seq_cu[s + 1];
  const int r0 = s0 + qt * BM;
  if (r0 >= s1) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 31, hf = lane >> 5;
  const int last = min(r0 + BM, s1) - 1;
  const int c0 = p.token_chunk[s0];
  const int hs = p.H * HD;   // row stride of [., H, HD]; T * H * HD < 2^31 (checked at the ABI)

  // this lane's row, and the wave's row range (rows past the sequence mimic its last row)
  const int i = r0 + wid * 32 + q;
  const int ic = min(i, last);
  const RowGeom g = row_geom(p, ic, s0, s1, c0);
  const int wr0 = min(r0 + wid * 32, last), wr1 = min(r0 + wid * 32 + 31, last);
  const int Ew0 = __builtin_amdgcn_readfirstlane(__shfl(g.E, 0));
  const int Ew1 = __builtin_amdgcn_readfirstlane(__shfl(g.E, 31));
  const int ww0 = __builtin_amdgcn_readfirstlane(__shfl(g.w, 0));
  const int ww1 = __builtin_amdgcn_readfirstlane(__shfl(g.w, 31));
  // the workgroup's key ranges
  const RowGeom gl = row_geom(p, last, s0, s1, c0);
  const RowGeom gf = row_geom(p, r0, s0, s1, c0);
  const int nbt = ceil_div(gl.E, BN);
  const int band0 = gf.w;
  const int nbd = last >= band0 ? ceil_div(last - band0 + 1, BN) : 0;
  const int ntiles = nbt + nbd;
  const int topb = c0 + gl.E - 1;   // last boundary key of the workgroup

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
  // Softmax state of the row: exponent reference mc (log2 units; -inf until the row has seen
  // a key) and the running sum l of p = 2^(s c - mc) over this lane's keys.
  float mc = -INFINITY, l = 0.f;
  const float c = p.scale * kLog2e;

  const __bf16* kbp = static_cast<const __bf16*>(p.kb) + h * HD;
  const __bf16* vbp = static_cast<const __bf16*>(p.vb) + h * HD;
  const __bf16* ktp = static_cast<const __bf16*>(p.k) + h * HD;
  const __bf16* vtp = static_cast<const __bf16*>(p.v) + h * HD;

  // per-lane LDS element offsets that do not depend on the tile
  int koff[QS];                    // S^T operand: row q, segment 2 st + hf (key block 0)
#pragma unroll
  for (int st = 0; st < QS; ++st) koff[st] = tile_off<HD>(q, 16 * st + 8 * hf);
  int voff[OB][2];                 // V^T operand, k-step 0: rows 4 hf + (lane%16)/4 (+8);
  {                                // k-step ks lies 16 ks rows further
    const int sl = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int j = 0; j < OB; ++j)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        voff[j][half] = tile_off<HD>(8 * half + 4 * hf + (sl >> 2), 32 * j + 16 * g16 + 4 * (sl & 3));
  }

  TileCopy<HD> tc;
  tc.init(wid, lane, hs);
  auto issue = [&](int t) {
    const bool bt = t < nbt;
    const int buf = t % NBUF;
    tc.issue(sm.k[buf], sm.v[buf], bt ? kbp : ktp, bt ? vbp : vtp,
             bt ? c0 + t * BN : band0 + (t - nbt) * BN, bt ? topb : last, hs, wid);
  };
  constexpr int kLoadsPerTile = 2 * TileCopy<HD>::NI;               // per wave
  constexpr int kAhead = NBUF - 1;                                 // tiles in flight
#pragma unroll
  for (int a = 0; a < kAhead; ++a)
    if (a < ntiles) issue(a);
  if (ntiles > kAhead) __builtin_amdgcn_s_waitcnt(vmcnt_at_most((kAhead - 1) * kLoadsPerTile));
  else __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t % NBUF;
    if (t + kAhead < ntiles) issue(t + kAhead);

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
      const int kbase = base + 4 * hf;
      const int lo = g.w - kbase;
      const int hi = bnd ? c0 + g.E - 1 - kbase : ic - kbase;
      f32x16 sacc[2];
      // Softmax with a lazy reference. The exact maximum is taken only while some row of the
      // wave has no reference yet, or when the tile's sum of p exceeds 2^64 (a row's scores grew
      // far past its reference); otherwise p = 2^(s c - mc) is used as is: l and
      // O^T share mc, so the result is exact, and p <= 2^64 keeps every value finite. Values of
      // p far below 1 stay normal floats (bf16 and float32 share the exponent range).
      // The exact path computes the scores again from the tile still in LDS: with one place
      // where scores are made per path, none stay live across the branch, which keeps the kernel
      // at 126 VGPRs (4 waves per SIMD instead of 3 at 160).
      bf16x8 pk[4];
      float lt = 0.f;
      bool exact = __any(mc == -INFINITY);
      if (!exact) {
        tile_scores<HD, QS>(sacc, sk, koff, qf, full, bnd, lo, hi);
        lt = tile_exp(sacc, c, mc, pk);
        exact = __any(!(lt <= 0x1p64f));
      }
      if (exact) {
        tile_scores<HD, QS>(sacc, sk, koff, qf, full, bnd, lo, hi);
        float m4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          m4[u] = fmaxf(fmaxf(fmaxf(sacc[0][4 * u], sacc[0][4 * u + 1]), sacc[0][4 * u + 2]),
                        fmaxf(fmaxf(sacc[0][4 * u + 3], sacc[1][4 * u]),
                              fmaxf(sacc[1][4 * u + 1], fmaxf(sacc[1][4 * u + 2], sacc[1][4 * u + 3]))));
        const float tm = half_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * c;
        const float mn = fmaxf(mc, tm);
        // 0 when mc = -inf (nothing accumulated yet), also for rows that still see no key
        const float alpha = hw_exp2(mc - (mn == -INFINITY ? 0.f : mn));
#pragma unroll
        for (int j = 0; j < OB; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[j][v] *= alpha;
        l *= alpha;
        mc = mn;
        lt = tile_exp(sacc, c, mc == -INFINITY ? 0.f : mc, pk);
      }
      l += lt;
      // O^T += V^T P^T; k-step ks covers keys 16 ks + {4 hf .. +3, 8 + 4 hf .. +3}, and V^T is
      // read in the same key order with the transposing LDS read
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < OB; ++j) {
          const i16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, sv + voff[j][0] + 16 * HD * ks));
          const i16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, sv + voff[j][1] + 16 * HD * ks));
          const i16x4 both[2] = {vlo, vhi};
          o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(both),
                                                         pk[ks], o[j], 0, 0, 0);
        }
    }
    // this wave's copies of tile t + 1 have landed (later tiles may still fly) ...
    if (t + kAhead < ntiles) __builtin_amdgcn_s_waitcnt(vmcnt_at_most((kAhead - 1) * kLoadsPerTile));
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();                  // ... and every wave is done with tile t
  }

  // epilogue: combine the two key halves of every query, normalise, write O and LSE
  const float lsum = half_sum(l);
  if (i < s1) {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
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
      p.lse[static_cast<size_t>(h) * p.T + i] = lsum > 0.f ? (mc + hw_log2(lsum)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, int hd, hipStream_t stream) {
  const int n_bh8 = ceil_div(p.S * p.H, 8) * 8;
  dim3 grid(ceil_div(p.max_seqlen, 128) * n_bh8);
  if (hd == 64) {
    hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(NT), 0, stream, p);
  } else {
    hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace attamba
