// Launchers of the HIP kernels; called by the C ABI layer after argument validation.
#pragma once
#include <hip/hip_runtime.h>
#include "../../include/attamba.h"

namespace attamba {

hipError_t launch_uniform_boundaries(const int32_t* seq_cu, int S, int T, int P, int o,
                                     int n_chunks, int32_t* chunk_cu, int32_t* token_chunk,
                                     uint8_t* is_end, hipStream_t stream);
hipError_t launch_chunk_index(const int32_t* chunk_cu, int n_chunks, int T,
                              int32_t* token_chunk, uint8_t* is_end, hipStream_t stream);
// Attention kernel parameters (validated by the ABI layer).
struct AttnParams {
  int T, H, S, max_seqlen, L, train;
  float scale;
  const void *q, *k, *v, *kb, *vb;
  const int32_t *seq_cu, *chunk_cu, *token_chunk;
  void* out;
  float* lse;
};

// bf16 matrix-core attention for hd 64 and 128.
hipError_t launch_attn_mfma(const AttnParams& p, int hd, hipStream_t stream);

hipError_t launch_kvssm_scan(const attamba_scan_args& a, hipStream_t stream);
hipError_t launch_chunk_attn(const attamba_attn_args& a, float scale, hipStream_t stream);

struct DecodeLaunch {
  int64_t pos;
  int is_start, is_end;   // this position starts / ends a chunk
  int slot;               // window slot pos mod L (L > 0)
  int n_bound_before;     // boundary states stored before this step
  int E;                  // boundary states attended (chunk ends before the window)
  int n_window;           // window positions attended (pos - w + 1, or 0 if L = 0)
  int w;                  // first window position
  int w_slot;             // its window slot, w mod L (L > 0)
  int n_splits;
  float scale;
};
// Input projection GEMM (bf16): Y = x W^T split into feature segments.
constexpr int kMaxProjSegments = ATTAMBA_PROJ_MAX_SEGMENTS;
struct ProjParams {
  int T, d, n_out, n_seg;
  const void* x;
  const void* w;
  int seg_start[kMaxProjSegments + 1];
  void* out[kMaxProjSegments];
};
hipError_t launch_proj_gemm(const ProjParams& p, hipStream_t stream);

// Backward of the KV-SSM scan: one side per SSM (index 0 = SSM_K, 1 = SSM_V).
struct ScanBwdSide {
  const void *x, *dt, *bm, *cm;   // forward inputs of this SSM
  const void *gy, *gb;            // gradients of its per-token outputs [T, d] and boundary
                                  // states [n_chunks, d] (gb may be null)
  const float *A, *D, *bias;
  void *dx, *ddt;                 // [T, d] activation dtype
  float *dbm, *dcm;               // [T, N], accumulated (zeroed first)
  float *dA, *dD, *dbias;         // [d, N], [d], [d], accumulated (zeroed first)
};
struct ScanBwdParams {
  int T, d, n_chunks;
  const int32_t* chunk_cu;
  ScanBwdSide side[2];
};
hipError_t launch_kvssm_scan_bwd(const ScanBwdParams& p, int N, int dtype, hipStream_t stream);

// Zero-fill of up to kMaxZero float buffers in one launch.
constexpr int kMaxZero = 10;
struct ZeroList {
  float* ptr[kMaxZero];
  int count[kMaxZero];
};
hipError_t launch_zero(const ZeroList& z, int n, hipStream_t stream);

// Backward of the chunk attention.
struct AttnBwdParams {
  AttnParams f;                   // forward geometry and inputs; f.out and f.lse are read
  const void* dout;
  void *dq, *dk, *dv, *dkb, *dvb;
  float* delta;                   // [H, T] rowsum(dout * out)
  int* row_w;                     // [T] first band position w_i of every row
  int* row_ce;                    // [T] c0 + E_i: first boundary state row i does not see
  int n_chunks;
  // Matrix-core path: the query rows of a boundary-state key tile are split over dkv_split
  // workgroups (1 or kDkvSplit), whose float32 partial dK/dV go to their own slot
  // [dkv_split][n_chunks][H * hd] of dkb_part / dvb_part and are summed by a finalize launch.
  int dkv_split;
  float* dkb_part;
  float* dvb_part;
};
constexpr int kDkvSplit = 4;
// 4-byte workspace elements the attention backward needs: delta, row_w and row_ce, plus the
// partial sums of the split boundary tiles (bf16, hd 64/128, at most one chunk per 4 tokens).
size_t attn_bwd_workspace_elems(int T, int H, int hd, int n_chunks, int dtype);
int attn_bwd_dkv_split(int T, int hd, int n_chunks, int dtype);
hipError_t launch_chunk_attn_bwd(const AttnBwdParams& p, int hd, int dtype, hipStream_t stream);
// bf16 matrix-core backward for hd 64 and 128 (needs delta, row_w and row_ce filled).
hipError_t launch_attn_bwd_mfma(const AttnBwdParams& p, int hd, hipStream_t stream);

int decode_max_splits(int cap, int L);
size_t decode_workspace_bytes(int B, int H, int hd, int cap, int L);
// Size of the decode step's static device scratch (the variant that allocates nothing), and
// its device address on the current device (looked up on first use per device).
constexpr size_t kDecodeScratchBytes = ATTAMBA_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch(void** ptr);
hipError_t launch_decode_step(const attamba_decode_cache& c, const attamba_decode_inputs& in,
                              const DecodeLaunch& dl, hipStream_t stream);
hipError_t launch_decode_load_prefix(const attamba_decode_cache& c, const attamba_decode_prefix& pf,
                                     int n_bound, int w0, hipStream_t stream);

}  // namespace attamba
