// Backward of the chunk-aware causal attention on the bf16 matrix cores of gfx950 (pith.science
// review of "Attamba: Attending To Multi-Token States", "What carries the argument": M_train
// Eq. 5, M_test Eq. 7, window Eq. 8). With P recomputed from the forward's LSE and
// D_i = dO_i . O_i: dS = P (dO V^T - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
//
// dK/dV kernel (key-centric): workgroup = 4 waves = 128 keys of one (sequence, head), either
// boundary states (kb/vb) or per-token keys (k/v); wave = 32 keys, whose K and V rows stay in
// registers as the B operands of
//   S  (queries x keys) = Q K^T        and   dP (queries x keys) = dO V^T,
// with the queries that see the workgroup's keys streamed through LDS in tiles of 64 rows (Q and
// dO copied straight from HBM with global_load_lds_dwordx4, double-buffered). The accumulators
// of S and dP hold one key per lane and 16 query rows per lane, so P and dS, converted to bf16 in
// place, are the B operands (queries taken in the accumulator's row order) of
//   dV^T (hd x keys) += dO^T P         and   dK^T (hd x keys) += Q^T dS,
// whose A operands come from the row-major Q and dO tiles through the transposing LDS read
// ds_read_b64_tr_b16. dK^T and dV^T stay in registers until the last query tile.
// The rows that see a key form one contiguous range (w_i and E_i grow with i): for boundary
// state q the rows with c0 + E_i > q, for a per-token key j the rows i >= j with w_i <= j.
//
// dQ kernel (query-centric): the forward's layout (4 waves x 32 query rows, key tiles of 64:
// boundary states first, then the band), with per tile
//   S^T = K Q^T,  dP^T = V dO^T  (Q and dO in registers),  dS^T = P^T (dP^T - D),
//   dQ^T (hd x queries) += K^T dS^T   (K^T through the transposing LDS read).
// It runs first and also writes D_i = dO_i . O_i and every row's w_i and c0 + E_i (the row
// geometry the dK/dV kernel searches). A third launch finalizes the boundary-state gradients
// when their query rows were split over several dK/dV workgroups.
#include "common.h"
#include "attn_geom.h"
#include "attn_tiles.h"

namespace attamba {
namespace {

using namespace mfma;

constexpr int NT = 256;    // threads per workgroup (4 waves)
constexpr int BM = 64;     // query rows per tile of the dK/dV kernel
constexpr int BK = 128;    // keys per workgroup of the dK/dV kernel

template <int HD>
struct DkvSmem {
  __bf16 q[2][BM * HD];
  __bf16 g[2][BM * HD];
  float lse2[2][BM];       // LSE in log2 units; +inf for rows past the sequence or empty rows
  float dd[2][BM];         // D_i
  int wr[2][BM];           // w_i (first band position)
  int ce[2][BM];           // c0 + E_i (first boundary state not seen)
};

// 16 accumulator values of one 32-row block, rounded to bf16 and packed as the B operands of
// k-steps 2 qb and 2 qb + 1 (rows 16 kk + {4 hf .. +3, 8 + 4 hf .. +3}): out[0] and out[1].
__device__ __forceinline__ void pack2(const float (&v)[16], bf16x8* out) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 pp = {static_cast<__bf16>(v[8 * kk + e]), static_cast<__bf16>(v[8 * kk + e + 1])};
      w[e >> 1] = __builtin_bit_cast(unsigned, pp);
    }
    out[kk] = __builtin_bit_cast(bf16x8, w);
  }
}

template <int HD>
__device__ __forceinline__ bf16x8 tr_read(const __bf16* base, int o0, int o1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, base + o0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, base + o1));
  const i16x4 both[2] = {lo, hi};
  return *reinterpret_cast<const bf16x8*>(both);
}

template <int HD>
__global__ __launch_bounds__(NT) void attn_bwd_dkv_mfma_kernel(AttnBwdParams bp) {
  constexpr int QS = HD / 16;
  constexpr int OB = HD / 32;
  __shared__ DkvSmem<HD> sm;
  const AttnParams& p = bp.f;

  // Workgroups go round-robin to the 8 XCDs. Consecutive ids take the same key tile of
  // consecutive (sequence, head) pairs (the pair count padded to a multiple of 8), so all key
  // tiles of one pair sit on one XCD, and the boundary tiles (seen by the most rows) go first
  // over the whole grid. A boundary tile is seen by every later row of its sequence, so its
  // query rows are split over ns workgroups (parts), each walking a contiguous share of the query
  // tiles; their float32 partial sums are added by a finalize launch. Per-token key tiles are
  // seen by a few hundred rows and are not split.
  const int ns = bp.dkv_split;
  const int n_bh8 = ceil_div(p.S * p.H, 8) * 8;
  const int id = blockIdx.x;
  const int bh = id % n_bh8;
  if (bh >= p.S * p.H) return;
  const int s = bh / p.H, h = bh % p.H;
  const int ks = id / n_bh8;
  const int s0 = p.seq_cu[s], s1 = p.seq_cu[s + 1];
  if (s1 <= s0) return;
  const int c0 = p.token_chunk[s0];
  const int nch = p.token_chunk[s1 - 1] + 1 - c0;
  const int nbt = ceil_div(nch, BK), nbd = ceil_div(s1 - s0, BK);
  if (ks >= nbt * ns + nbd) return;
  const bool bnd = ks < nbt * ns;
  const int kt = bnd ? ks / ns : ks - nbt * ns;
  const int part = bnd ? ks % ns : 0;
  const int kbase = bnd ? c0 + kt * BK : s0 + kt * BK;
  const int ktop = bnd ? c0 + nch - 1 : s1 - 1;
  const int kmax = min(kbase + BK - 1, ktop);
  const int* __restrict__ row_w = bp.row_w;
  const int* __restrict__ row_ce = bp.row_ce;

  // rows [ia, ib] that see some key of the workgroup
  int ia, ib = s1 - 1;
  if (bnd) {
    int lo = p.chunk_cu[kbase + 1] - 1, hi = s1;     // first row with c0 + E_i > kbase
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (row_ce[mid] > kbase) hi = mid; else lo = mid + 1;
    }
    ia = lo;
  } else {
    ia = kbase;
    if (row_w[kbase] > kmax) {
      ib = kbase - 1;
    } else {
      int lo = kbase, hi = s1 - 1;                   // last row with w_i <= kmax
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (row_w[mid] <= kmax) lo = mid; else hi = mid - 1;
      }
      ib = lo;
    }
  }
  const int nq = ib >= ia ? ceil_div(ib - ia + 1, BM) : 0;
  const int nparts = bnd ? ns : 1;
  const int tb = part * nq / nparts, te = (part + 1) * nq / nparts;   // this part's query tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 31, hf = lane >> 5;
  const int hs = p.H * HD;
  const int kw0 = kbase + wid * 32, kw1 = min(kw0 + 31, ktop);
  const bool wave_live = kw0 <= ktop;
  const int kx = kw0 + q;                            // this lane's key
  const int kxc = min(kx, ktop);

  bf16x8 kf[QS], vf[QS];
  {
    const size_t ro = static_cast<size_t>(kxc) * hs + h * HD + 8 * hf;
    const __bf16* kr = static_cast<const __bf16*>(bnd ? p.kb : p.k) + ro;
    const __bf16* vr = static_cast<const __bf16*>(bnd ? p.vb : p.v) + ro;
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      kf[st] = *reinterpret_cast<const bf16x8*>(kr + 16 * st);
      vf[st] = *reinterpret_cast<const bf16x8*>(vr + 16 * st);
    }
  }
  f32x16 dka[OB], dva[OB];
#pragma unroll
  for (int j = 0; j < OB; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) { dka[j][v] = 0.f; dva[j][v] = 0.f; }

  int aoff[QS];                    // A operand of S and dP: tile row q (+32 per block), hd 16 st + 8 hf
#pragma unroll
  for (int st = 0; st < QS; ++st) aoff[st] = tile_off<HD>(q, 16 * st + 8 * hf);
  int toff[OB][2];                 // transposing read, k-step 0 (k-step ks lies 16 ks rows further)
  {
    const int sl = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int j = 0; j < OB; ++j)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        toff[j][half] = tile_off<HD>(8 * half + 4 * hf + (sl >> 2), 32 * j + 16 * g16 + 4 * (sl & 3));
  }

  TileCopy<HD> tc;
  tc.init(wid, lane, hs);
  const __bf16* qp = static_cast<const __bf16*>(p.q) + h * HD;
  const __bf16* gp = static_cast<const __bf16*>(bp.dout) + h * HD;
  auto issue = [&](int t) { tc.issue(sm.q[t & 1], sm.g[t & 1], qp, gp, ia + t * BM, s1 - 1, hs, wid); };
  // per-row data of a query tile, loaded by wave 0 one tile ahead and written to LDS just
  // before the barrier that ends the current tile
  float m_l2 = INFINITY, m_dd = 0.f;
  int m_w = 0x7fffffff, m_ce = -0x7fffffff;
  auto meta_load = [&](int t) {
    const int i = ia + t * BM + lane;
    m_l2 = INFINITY; m_dd = 0.f; m_w = 0x7fffffff; m_ce = -0x7fffffff;
    if (i < s1) {
      const float ls = p.lse[static_cast<size_t>(h) * p.T + i];
      if (ls != -INFINITY) m_l2 = ls * kLog2e;
      m_dd = bp.delta[static_cast<size_t>(h) * p.T + i];
      m_w = row_w[i];
      m_ce = row_ce[i];
    }
  };
  auto meta_store = [&](int t) {
    sm.lse2[t & 1][lane] = m_l2;
    sm.dd[t & 1][lane] = m_dd;
    sm.wr[t & 1][lane] = m_w;
    sm.ce[t & 1][lane] = m_ce;
  };
  if (te > tb) {
    issue(tb);
    if (wid == 0) {
      meta_load(tb);
      meta_store(tb);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const float c = p.scale * kLog2e;

  for (int t = tb; t < te; ++t) {
    const int buf = t & 1;
    if (t + 1 < te) {
      issue(t + 1);
      if (wid == 0) meta_load(t + 1);
    }
    const int r0 = ia + t * BM;
    const int rl = min(r0 + BM - 1, s1 - 1);
    // visibility of the wave's keys from the tile's first and last rows (w_i and E_i grow
    // with i), read from the tile's per-row data in LDS
    bool skip, full;
    if (bnd) {
      skip = sm.ce[buf][rl - r0] <= kw0;
      full = sm.ce[buf][0] > kw1;
    } else {
      skip = rl < kw0 || sm.wr[buf][0] > kw1;
      full = sm.wr[buf][rl - r0] <= kw0 && r0 >= kw1;
    }
    if (wave_live && !skip) {
      const __bf16* sq = sm.q[buf];
      const __bf16* sg = sm.g[buf];
      // S and dP of both 32-row blocks first: four independent accumulation chains
      f32x16 sacc[2] = {}, dpacc[2] = {};
#pragma unroll
      for (int st = 0; st < QS; ++st)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sq + aoff[st] + 32 * HD * qb);
          sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[st], sacc[qb], 0, 0, 0);
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(sg + aoff[st] + 32 * HD * qb);
          dpacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, vf[st], dpacc[qb], 0, 0, 0);
        }
      bf16x8 pk[4], dk8[4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float pv[16], dsv[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int rb = 32 * qb + 8 * g4 + 4 * hf;     // first of this lane's 4 rows
          const float4 l2 = *reinterpret_cast<const float4*>(&sm.lse2[buf][rb]);
          const float4 d4 = *reinterpret_cast<const float4*>(&sm.dd[buf][rb]);
          const float l2a[4] = {l2.x, l2.y, l2.z, l2.w};
          const float dda[4] = {d4.x, d4.y, d4.z, d4.w};
          int wa[4] = {0, 0, 0, 0}, cea[4] = {0, 0, 0, 0};
          if (!full) {
            const int4 w4 = *reinterpret_cast<const int4*>(&sm.wr[buf][rb]);
            const int4 c4 = *reinterpret_cast<const int4*>(&sm.ce[buf][rb]);
            wa[0] = w4.x; wa[1] = w4.y; wa[2] = w4.z; wa[3] = w4.w;
            cea[0] = c4.x; cea[1] = c4.y; cea[2] = c4.z; cea[3] = c4.w;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g4 + e;
            float pr = hw_exp2(fmaf(sacc[qb][v], c, -l2a[e]));
            if (!full) {
              const bool vis = bnd ? (kx < cea[e]) : (wa[e] <= kx && kx <= r0 + rb + e);
              pr = vis ? pr : 0.f;
            }
            pv[v] = pr;
            dsv[v] = pr * (dpacc[qb][v] - dda[e]);
          }
        }
        pack2(pv, pk + 2 * qb);
        pack2(dsv, dk8 + 2 * qb);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < OB; ++j) {
          const bf16x8 ga = tr_read<HD>(sg, toff[j][0] + 16 * HD * ks, toff[j][1] + 16 * HD * ks);
          dva[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, pk[ks], dva[j], 0, 0, 0);
          const bf16x8 qa = tr_read<HD>(sq, toff[j][0] + 16 * HD * ks, toff[j][1] + 16 * HD * ks);
          dka[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dk8[ks], dka[j], 0, 0, 0);
        }
    }
    if (wid == 0 && t + 1 < te) meta_store(t + 1);
    __builtin_amdgcn_s_waitcnt(0);     // this wave's copies of tile t + 1 have landed ...
    __syncthreads();                   // ... and every wave is done with tile t
  }

  // epilogue: lane = key, accumulator rows = hd 32 j + 8 g + 4 hf + e
  if (wave_live && kx <= ktop && bnd && ns > 1) {
    // this part's float32 partial sums (dK unscaled) into its slot [part][chunk][H * hd]
    const size_t ro = (static_cast<size_t>(part) * bp.n_chunks + kx) * hs + h * HD + 4 * hf;
    float* dkp = bp.dkb_part + ro;
    float* dvp = bp.dvb_part + ro;
#pragma unroll
    for (int j = 0; j < OB; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 a = {dka[j][4 * g4], dka[j][4 * g4 + 1], dka[j][4 * g4 + 2], dka[j][4 * g4 + 3]};
        const float4 b = {dva[j][4 * g4], dva[j][4 * g4 + 1], dva[j][4 * g4 + 2], dva[j][4 * g4 + 3]};
        *reinterpret_cast<float4*>(dkp + 32 * j + 8 * g4) = a;
        *reinterpret_cast<float4*>(dvp + 32 * j + 8 * g4) = b;
      }
  } else if (wave_live && kx <= ktop) {
    const size_t ro = static_cast<size_t>(kx) * hs + h * HD + 4 * hf;
    __bf16* dko = static_cast<__bf16*>(bnd ? bp.dkb : bp.dk) + ro;
    __bf16* dvo = static_cast<__bf16*>(bnd ? bp.dvb : bp.dv) + ro;
#pragma unroll
    for (int j = 0; j < OB; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = static_cast<__bf16>(dka[j][4 * g4 + e] * p.scale);
          b[e] = static_cast<__bf16>(dva[j][4 * g4 + e]);
        }
        *reinterpret_cast<bf16x4*>(dko + 32 * j + 8 * g4) = a;
        *reinterpret_cast<bf16x4*>(dvo + 32 * j + 8 * g4) = b;
      }
  }
}

template <int HD>
struct DqSmem {
  __bf16 k[2][BN * HD];
  __bf16 v[2][BN * HD];
};

template <int HD>
__global__ __launch_bounds__(NT) void attn_bwd_dq_mfma_kernel(AttnBwdParams bp) {
  constexpr int QS = HD / 16;
  constexpr int OB = HD / 32;
  constexpr int BQ = 128;         // query rows per workgroup (4 waves x 32)
  __shared__ DqSmem<HD> sm;
  const AttnParams& p = bp.f;

  // grid order as in the forward: the same query tile of consecutive (sequence, head) pairs,
  // the last query tiles (the most keys) first over the whole grid
  const int n_qt = ceil_div(p.max_seqlen, BQ);
  const int n_bh8 = ceil_div(p.S * p.H, 8) * 8;
  const int id = blockIdx.x;
  const int bh = id % n_bh8;
  if (bh >= p.S * p.H) return;
  const int s = bh / p.H, h = bh % p.H;
  const int qt = n_qt - 1 - id / n_bh8;
  const int s0 = p.seq_cu[s], s1 = p.seq_cu[s + 1];
  const int r0 = s0 + qt * BQ;
  if (r0 >= s1) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 31, hf = lane >> 5;
  const int last = min(r0 + BQ, s1) - 1;
  const int c0 = p.token_chunk[s0];
  const int hs = p.H * HD;

  const int i = r0 + wid * 32 + q;
  const int ic = min(i, last);
  const RowGeom g = row_geom(p, ic, s0, s1, c0);
  const int wr0 = min(r0 + wid * 32, last), wr1 = min(r0 + wid * 32 + 31, last);
  const int Ew0 = __builtin_amdgcn_readfirstlane(__shfl(g.E, 0));
  const int Ew1 = __builtin_amdgcn_readfirstlane(__shfl(g.E, 31));
  const int ww0 = __builtin_amdgcn_readfirstlane(__shfl(g.w, 0));
  const int ww1 = __builtin_amdgcn_readfirstlane(__shfl(g.w, 31));
  const RowGeom gl = row_geom(p, last, s0, s1, c0);
  const RowGeom gf = row_geom(p, r0, s0, s1, c0);
  const int nbt = ceil_div(gl.E, BN);
  const int band0 = gf.w;
  const int nbd = last >= band0 ? ceil_div(last - band0 + 1, BN) : 0;
  const int ntiles = nbt + nbd;
  const int topb = c0 + gl.E - 1;

  bf16x8 qf[QS], gf8[QS];
  float Dl;   // D_i = dO_i . O_i (this lane's half of the row, then both halves)
  {
    const size_t ro = static_cast<size_t>(ic) * hs + h * HD + 8 * hf;
    const __bf16* qr = static_cast<const __bf16*>(p.q) + ro;
    const __bf16* gr = static_cast<const __bf16*>(bp.dout) + ro;
    const __bf16* orow = static_cast<const __bf16*>(p.out) + ro;
    float part = 0.f;
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      qf[st] = *reinterpret_cast<const bf16x8*>(qr + 16 * st);
      gf8[st] = *reinterpret_cast<const bf16x8*>(gr + 16 * st);
      const bf16x8 of = *reinterpret_cast<const bf16x8*>(orow + 16 * st);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 a = {of[e], of[e + 1]}, b = {gf8[st][e], gf8[st][e + 1]};
        part = __builtin_amdgcn_fdot2_f32_bf16(a, b, part, false);
      }
    }
    Dl = half_sum(part);
  }
  float lse2 = INFINITY;
  if (i < s1) {
    const float ls = p.lse[static_cast<size_t>(h) * p.T + i];
    if (ls != -INFINITY) lse2 = ls * kLog2e;
    // D_i and the row's mask geometry for the dK/dV kernel, which runs after this one
    if (hf == 0) {
      bp.delta[static_cast<size_t>(h) * p.T + i] = Dl;
      if (h == 0) {
        bp.row_w[i] = g.w;
        bp.row_ce[i] = c0 + g.E;
      }
    }
  }
  f32x16 dqa[OB];
#pragma unroll
  for (int j = 0; j < OB; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) dqa[j][v] = 0.f;
  const float c = p.scale * kLog2e;

  const __bf16* kbp = static_cast<const __bf16*>(p.kb) + h * HD;
  const __bf16* vbp = static_cast<const __bf16*>(p.vb) + h * HD;
  const __bf16* ktp = static_cast<const __bf16*>(p.k) + h * HD;
  const __bf16* vtp = static_cast<const __bf16*>(p.v) + h * HD;

  int koff[QS];
#pragma unroll
  for (int st = 0; st < QS; ++st) koff[st] = tile_off<HD>(q, 16 * st + 8 * hf);
  int toff[OB][2];
  {
    const int sl = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int j = 0; j < OB; ++j)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        toff[j][half] = tile_off<HD>(8 * half + 4 * hf + (sl >> 2), 32 * j + 16 * g16 + 4 * (sl & 3));
  }

  TileCopy<HD> tc;
  tc.init(wid, lane, hs);
  auto issue = [&](int t) {
    const bool bt = t < nbt;
    tc.issue(sm.k[t & 1], sm.v[t & 1], bt ? kbp : ktp, bt ? vbp : vtp,
             bt ? c0 + t * BN : band0 + (t - nbt) * BN, bt ? topb : last, hs, wid);
  };
  if (ntiles > 0) issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) issue(t + 1);
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
      tile_scores<HD, QS>(sacc, sk, koff, qf, full, bnd, lo, hi);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 dpacc = {};
#pragma unroll
        for (int st = 0; st < QS; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sv + koff[st] + 32 * HD * kb);
          dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf8[st], dpacc, 0, 0, 0);
        }
        float dsv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pr = hw_exp2(fmaf(sacc[kb][v], c, -lse2));
          dsv[v] = pr * (dpacc[v] - Dl);
        }
        bf16x8 dk8[2];
        pack2(dsv, dk8);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ks = 2 * kb + kk;
#pragma unroll
          for (int j = 0; j < OB; ++j) {
            const bf16x8 ka = tr_read<HD>(sk, toff[j][0] + 16 * HD * ks, toff[j][1] + 16 * HD * ks);
            dqa[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, dk8[kk], dqa[j], 0, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (i < s1) {
    __bf16* orow = static_cast<__bf16*>(bp.dq) + static_cast<size_t>(i) * hs + h * HD + 4 * hf;
#pragma unroll
    for (int j = 0; j < OB; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = static_cast<__bf16>(dqa[j][4 * g4 + e] * p.scale);
        *reinterpret_cast<bf16x4*>(orow + 32 * j + 8 * g4) = vv;
      }
  }
}

// Explicit instantiations: the host pass does not emit the launch stubs of these templates
// from the launches below alone.
template __global__ void attn_bwd_dkv_mfma_kernel<64>(AttnBwdParams);
template __global__ void attn_bwd_dkv_mfma_kernel<128>(AttnBwdParams);
template __global__ void attn_bwd_dq_mfma_kernel<64>(AttnBwdParams);
template __global__ void attn_bwd_dq_mfma_kernel<128>(AttnBwdParams);

// dkb = scale * (sum of the parts' dK), dvb = sum of the parts' dV, rounded to bf16; four
// consecutive elements of [n_chunks, H * hd] per thread.
__global__ __launch_bounds__(256) void attn_bwd_dkv_finalize_kernel(AttnBwdParams bp, int n) {
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float4 k = {0.f, 0.f, 0.f, 0.f}, v = {0.f, 0.f, 0.f, 0.f};
  for (int part = 0; part < bp.dkv_split; ++part) {
    const float4 a = *reinterpret_cast<const float4*>(bp.dkb_part + static_cast<size_t>(part) * n + i);
    const float4 b = *reinterpret_cast<const float4*>(bp.dvb_part + static_cast<size_t>(part) * n + i);
    k.x += a.x; k.y += a.y; k.z += a.z; k.w += a.w;
    v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
  }
  const float sc = bp.f.scale;
  const bf16x4 ko = {static_cast<__bf16>(k.x * sc), static_cast<__bf16>(k.y * sc),
                     static_cast<__bf16>(k.z * sc), static_cast<__bf16>(k.w * sc)};
  const bf16x4 vo = {static_cast<__bf16>(v.x), static_cast<__bf16>(v.y), static_cast<__bf16>(v.z),
                     static_cast<__bf16>(v.w)};
  *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(bp.dkb) + i) = ko;
  *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(bp.dvb) + i) = vo;
}

}  // namespace

int attn_bwd_dkv_split(int T, int hd, int n_chunks, int dtype) {
  const bool mfma = dtype == ATTAMBA_BF16 && (hd == 64 || hd == 128);
  return mfma && static_cast<long>(n_chunks) * 4 <= T ? kDkvSplit : 1;
}

size_t attn_bwd_workspace_elems(int T, int H, int hd, int n_chunks, int dtype) {
  size_t e = static_cast<size_t>(H + 2) * T;
  const int ns = attn_bwd_dkv_split(T, hd, n_chunks, dtype);
  if (ns > 1) e = (e + 63) / 64 * 64 + 2 * static_cast<size_t>(ns) * n_chunks * H * hd;
  return e;
}

hipError_t launch_attn_bwd_mfma(const AttnBwdParams& p, int hd, hipStream_t stream) {
  const int n_bh8 = ceil_div(p.f.S * p.f.H, 8) * 8;
  const dim3 gkv((p.dkv_split + 1) * ceil_div(p.f.max_seqlen, BK) * n_bh8);
  const dim3 gq(ceil_div(p.f.max_seqlen, 128) * n_bh8);
  // dQ first: it also writes D_i = dO_i . O_i and every row's w_i and c0 + E_i, which dK/dV reads
  if (hd == 64) {
    hipLaunchKernelGGL(attn_bwd_dq_mfma_kernel<64>, gq, dim3(NT), 0, stream, p);
    hipLaunchKernelGGL(attn_bwd_dkv_mfma_kernel<64>, gkv, dim3(NT), 0, stream, p);
  } else {
    hipLaunchKernelGGL(attn_bwd_dq_mfma_kernel<128>, gq, dim3(NT), 0, stream, p);
    hipLaunchKernelGGL(attn_bwd_dkv_mfma_kernel<128>, gkv, dim3(NT), 0, stream, p);
  }
  if (p.dkv_split > 1) {
    const int n = p.n_chunks * p.f.H * hd;
    hipLaunchKernelGGL(attn_bwd_dkv_finalize_kernel, dim3(ceil_div(n / 4, 256)), dim3(256), 0, stream, p, n);
  }
  return hipGetLastError();
}

}  // namespace attamba
