// Tile machinery shared by the matrix-core attention kernels (forward and backward) on gfx950:
// bf16 operand types, the XOR swizzle of 64-row tiles in LDS, the LDS-direct tile copy, and
// the masked score product of one 64-key tile.
#pragma once
#include "common.h"

namespace attamba {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int BN = 64;    // keys per tile

// Row r of a tile keeps its 16-byte segment s at position s ^ swz(r). The LDS has 64 banks of
// 4 bytes (a 256-byte window); a ds_read_b128 is served 16 lanes per pass, a ds_read_b64 32
// lanes per pass. Both reads then touch distinct banks in every pass:
// - the K read: 16 lanes, one segment of 16 consecutive rows;
// - the transposing V read: 32 lanes, the four segments 4j .. 4j + 3 of 4 consecutive rows
//   starting at a multiple of 4 (256 bytes).
// At hd 64 a row is half the window (rows alternate halves): swz must differ between the 8 rows
// of one parity in an aligned group of 16, and its bit 2 between rows r and r + 2 of an aligned
// group of 4. At hd 128 a row fills the window: swz must differ over 16 consecutive rows, and its
// bits 2..3 over an aligned group of 4. (With the earlier swizzle, made for the K read alone, the
// forward kernel took 5.4 M bank-conflict cycles per launch at hd 64; with this one, none.)
template <int HD>
__device__ __forceinline__ int swz(int r) {
  if constexpr (HD == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}

// max of x over lanes q and q + 32 (the two key halves of one query): v_permlane32_swap
// exchanges the upper half of one register with the lower half of another.
__device__ __forceinline__ float half_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// element offset of (row r, element e) in a tile
template <int HD>
__device__ __forceinline__ int tile_off(int r, int e) {
  return r * HD + 8 * ((e >> 3) ^ swz<HD>(r)) + (e & 7);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave are
// outstanding (LDS/scalar and export counters left unconstrained).
__host__ __device__ constexpr int vmcnt_at_most(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14);
}

// The LDS-direct copies of one tile. Each wave copies NI chunks of 1 KB; lane l of chunk ch
// fills 16-byte slot ch * 64 + l of the tile, which holds segment pos of tile row r (slot =
// r * SPR + (pos ^ swz(r))). The per-lane part of the source address, r * hs + 8 * seg, does not
// depend on the tile and is computed once.
template <int HD>
struct TileCopy {
  static constexpr int SPR = HD / 8;                    // 16-byte segments per row
  static constexpr int NI = BN * SPR / kWave / 4;       // 1 KB chunks per wave
  int off[NI];   // element offset of this lane's segment from the tile's first key row
  int row[NI];   // its tile row
  int seg8[NI];  // its element offset within the row

  __device__ __forceinline__ void init(int wid, int lane, int hs) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = (wid * NI + i) * kWave + lane;
      const int r = slot / SPR, pos = slot % SPR;
      row[i] = r;
      seg8[i] = 8 * (pos ^ swz<HD>(r));
      off[i] = r * hs + seg8[i];
    }
  }
  // keys base .. base + BN - 1; keys past `top`, the last valid key, re-read row `top` (every
  // row that could see such a key masks it). base, top and wid are wave-uniform.
  __device__ __forceinline__ void issue(__bf16* sk, __bf16* sv, const __bf16* kp,
                                        const __bf16* vp, int base, int top, int hs,
                                        int wid) const {
    if (base + BN - 1 <= top) {
      const __bf16* kt = kp + static_cast<size_t>(base) * hs;
      const __bf16* vt = vp + static_cast<size_t>(base) * hs;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ch = wid * NI + i;
        __builtin_amdgcn_global_load_lds(kt + off[i], LDS_PTR(void, sk + ch * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + off[i], LDS_PTR(void, sv + ch * 512), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ch = wid * NI + i;
        const int go = min(base + row[i], top) * hs + seg8[i];
        __builtin_amdgcn_global_load_lds(kp + go, LDS_PTR(void, sk + ch * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp + go, LDS_PTR(void, sv + ch * 512), 16, 0, 0);
      }
    }
  }
};

// S^T = K Q^T for one tile (keys on accumulator rows, this lane's query on its column). The mask
// enters as the initial accumulator: 0 for a visible key, -inf for a hidden one (accumulator
// row v of block kb is key base + 4 hf + C(kb, v), C = 32 kb + 8 (v / 4) + v % 4); fully
// visible tiles start from the zero accumulator. Visible: lo <= C <= hi (boundary tiles only
// test hi). koff: this lane's operand offsets for key block 0; block 1 lies 32 rows further
// (the swizzle repeats every 16 rows).
template <int HD, int QS>
__device__ __forceinline__ void tile_scores(f32x16 (&sacc)[2], const __bf16* sk,
                                            const int (&koff)[QS], const bf16x8 (&qf)[QS],
                                            bool full, bool bnd, int lo, int hi) {
  const f32x16 zero16 = {};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x8 ka[QS];
#pragma unroll
    for (int st = 0; st < QS; ++st)
      ka[st] = *reinterpret_cast<const bf16x8*>(sk + koff[st] + 32 * HD * kb);
    if (full) {
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], zero16, 0, 0, 0);
    } else {
      if (bnd) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int C = 32 * kb + 8 * (v >> 2) + (v & 3);
          sacc[kb][v] = C <= hi ? 0.f : -INFINITY;
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int C = 32 * kb + 8 * (v >> 2) + (v & 3);
          sacc[kb][v] = (C >= lo && C <= hi) ? 0.f : -INFINITY;
        }
      }
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], sacc[kb], 0, 0, 0);
    }
#pragma unroll
    for (int st = 1; st < QS; ++st)
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], qf[st], sacc[kb], 0, 0, 0);
  }
}

}  // namespace mfma
}  // namespace attamba
