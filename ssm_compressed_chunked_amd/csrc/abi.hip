// C ABI of libattamba: host-side argument checks, closed-form chunk counts, and the launches on
// the caller's stream. Nothing here allocates device memory or synchronises with the device.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/attamba.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ATTAMBA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTAMBA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int32_t dt) { return dt == ATTAMBA_FP32 || dt == ATTAMBA_BF16; }

// Chunks of one sequence of n tokens, offset o (uniform chunking with cyclic offset).
int64_t chunks_of(int64_t n, int64_t P, int64_t o) {
  if (n <= 0) return 0;
  if (o == 0) return (n + P - 1) / P;
  if (n <= o) return 1;
  return 1 + (n - o + P - 1) / P;
}

// Chunk ends among positions 0 .. x-1 under the positional rule (j + 1 - o) = 0 (mod P).
int64_t ends_before(int64_t x, int64_t P, int64_t o) {
  if (x <= 0) return 0;
  if (o == 0) return x / P;
  return x >= o ? (x - o) / P + 1 : 0;
}

bool starts_chunk(int64_t pos, int64_t P, int64_t o) {
  return pos == 0 || (((pos - o) % P) + P) % P == 0;
}

// Checks shared by the scan and its backward (sizes, dtype and the forward inputs).
int check_scan(const attamba_scan_args* a, const char* name) {
  if (!dtype_ok(a->dtype)) return fail(ATTAMBA_ERR_BAD_DTYPE, "%s: dtype %d", name, a->dtype);
  if (a->T < 0 || a->n_chunks < 0 || a->n_chunks > a->T || (a->T > 0 && a->n_chunks == 0))
    return fail(ATTAMBA_ERR_BAD_SHAPE, "%s: T=%d n_chunks=%d", name, a->T, a->n_chunks);
  if (a->d <= 0 || a->d % 64 != 0) return fail(ATTAMBA_ERR_BAD_SHAPE, "%s: d=%d not a positive multiple of 64", name, a->d);
  if (a->N != 16 && a->N != 32) return fail(ATTAMBA_ERR_UNSUPPORTED, "%s: N=%d (16 or 32)", name, a->N);
  if (static_cast<int64_t>(a->T) * a->d > INT32_MAX)
    return fail(ATTAMBA_ERR_UNSUPPORTED, "%s: T*d exceeds 2^31 elements", name);
  if (!a->chunk_cu || !a->x || !a->dt_k || !a->dt_v || !a->bm_k || !a->cm_k || !a->bm_v || !a->cm_v ||
      !a->A_k || !a->A_v || !a->D_k || !a->D_v || !a->bias_k || !a->bias_v)
    return fail(ATTAMBA_ERR_NULL_ARG, "%s: a required pointer is null", name);
  return ATTAMBA_OK;
}

// Checks shared by the attention and its backward.
int check_attn(const attamba_attn_args* a, const char* name) {
  if (!dtype_ok(a->dtype)) return fail(ATTAMBA_ERR_BAD_DTYPE, "%s: dtype %d", name, a->dtype);
  if (a->T < 0 || a->H < 1 || a->S < 1 || a->n_chunks < 0 || a->L < 0 ||
      (a->T > 0 && (a->max_seqlen < 1 || a->n_chunks < 1)) ||
      (a->mode != ATTAMBA_MASK_TRAIN && a->mode != ATTAMBA_MASK_TEST) || !(a->scale >= 0.0f))
    return fail(ATTAMBA_ERR_BAD_SHAPE, "%s: T=%d H=%d S=%d max_seqlen=%d n_chunks=%d L=%d mode=%d", name, a->T,
                a->H, a->S, a->max_seqlen, a->n_chunks, a->L, a->mode);
  if (a->hd != 32 && a->hd != 64 && a->hd != 128)
    return fail(ATTAMBA_ERR_UNSUPPORTED, "%s: hd=%d (32, 64 or 128)", name, a->hd);
  if (static_cast<int64_t>(a->T) * a->H * a->hd > INT32_MAX)
    return fail(ATTAMBA_ERR_UNSUPPORTED, "%s: T*H*hd exceeds 2^31 elements", name);
  if (a->T > 0 && (!a->q || !a->k || !a->v || !a->kb || !a->vb || !a->seq_cu || !a->chunk_cu ||
                   !a->token_chunk || !a->out))
    return fail(ATTAMBA_ERR_NULL_ARG, "%s: a required pointer is null", name);
  return ATTAMBA_OK;
}

}  // namespace

extern "C" {

const char* attamba_version(void) { return "attamba-mi355x 0.1.0 (gfx950)"; }

const char* attamba_status_string(int status) {
  switch (status) {
    case ATTAMBA_OK: return "ok";
    case ATTAMBA_ERR_NULL_ARG: return "null argument";
    case ATTAMBA_ERR_BAD_SHAPE: return "bad shape or index data";
    case ATTAMBA_ERR_BAD_DTYPE: return "bad dtype";
    case ATTAMBA_ERR_CAPACITY: return "capacity exceeded";
    case ATTAMBA_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTAMBA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* attamba_last_error(void) { return g_last_error.c_str(); }

int attamba_count_chunks(const int32_t* seq_cu_host, int32_t S, int32_t P, int32_t layer_idx,
                         int32_t* n_chunks_out) {
  if (!seq_cu_host || !n_chunks_out) return fail(ATTAMBA_ERR_NULL_ARG, "count_chunks: null pointer");
  if (S < 0 || P < 1 || layer_idx < 0)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "count_chunks: S=%d P=%d layer_idx=%d", S, P, layer_idx);
  if (seq_cu_host[0] != 0) return fail(ATTAMBA_ERR_BAD_SHAPE, "count_chunks: seq_cu[0] != 0");
  const int64_t o = layer_idx % P;
  int64_t total = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t n = static_cast<int64_t>(seq_cu_host[s + 1]) - seq_cu_host[s];
    if (n < 0) return fail(ATTAMBA_ERR_BAD_SHAPE, "count_chunks: seq_cu decreases at %d", s);
    total += chunks_of(n, P, o);
  }
  if (total > INT32_MAX - 1) return fail(ATTAMBA_ERR_BAD_SHAPE, "count_chunks: too many chunks");
  *n_chunks_out = static_cast<int32_t>(total);
  return ok();
}

int attamba_chunk_cu_from_lengths(const int32_t* seq_cu_host, int32_t S,
                                  const int32_t* chunk_len_host, int32_t n_len,
                                  int32_t* chunk_cu_host_out) {
  if (!seq_cu_host || !chunk_cu_host_out || (n_len > 0 && !chunk_len_host))
    return fail(ATTAMBA_ERR_NULL_ARG, "chunk_cu_from_lengths: null pointer");
  if (S < 0 || n_len < 0) return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_cu_from_lengths: S=%d n_len=%d", S, n_len);
  if (seq_cu_host[0] != 0) return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_cu_from_lengths: seq_cu[0] != 0");
  int32_t k = 0;
  int64_t pos = 0;
  chunk_cu_host_out[0] = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t end = seq_cu_host[s + 1];
    if (end < pos) return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_cu_from_lengths: seq_cu decreases at %d", s);
    while (pos < end) {
      if (k >= n_len) return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_cu_from_lengths: lengths end inside sequence %d", s);
      const int64_t len = chunk_len_host[k];
      if (len < 1 || pos + len > end)
        return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_cu_from_lengths: chunk %d (length %lld) crosses sequence %d", k,
                    static_cast<long long>(len), s);
      pos += len;
      chunk_cu_host_out[++k] = static_cast<int32_t>(pos);
    }
  }
  if (k != n_len) return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_cu_from_lengths: %d lengths left over", n_len - k);
  return ok();
}

int attamba_chunk_boundaries(const int32_t* seq_cu, int32_t S, int32_t T, int32_t P,
                             int32_t layer_idx, int32_t n_chunks, int32_t* chunk_cu,
                             int32_t* token_chunk, uint8_t* is_end, attamba_stream_t stream) {
  if (!seq_cu || !chunk_cu) return fail(ATTAMBA_ERR_NULL_ARG, "chunk_boundaries: seq_cu/chunk_cu null");
  if (S < 1 || T < 0 || P < 1 || layer_idx < 0 || n_chunks < 0 || n_chunks > T)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_boundaries: S=%d T=%d P=%d layer_idx=%d n_chunks=%d", S, T, P,
                layer_idx, n_chunks);
  return hip_status(attamba::launch_uniform_boundaries(seq_cu, S, T, P, layer_idx % P, n_chunks,
                                                       chunk_cu, token_chunk, is_end,
                                                       reinterpret_cast<hipStream_t>(stream)),
                    "chunk_boundaries launch");
}

int attamba_chunk_index(const int32_t* chunk_cu, int32_t n_chunks, int32_t T,
                        int32_t* token_chunk, uint8_t* is_end, attamba_stream_t stream) {
  if (!chunk_cu) return fail(ATTAMBA_ERR_NULL_ARG, "chunk_index: chunk_cu null");
  if (n_chunks < 0 || T < 0 || n_chunks > T || (T > 0 && n_chunks == 0))
    return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_index: n_chunks=%d T=%d", n_chunks, T);
  return hip_status(attamba::launch_chunk_index(chunk_cu, n_chunks, T, token_chunk, is_end,
                                                reinterpret_cast<hipStream_t>(stream)),
                    "chunk_index launch");
}

int attamba_kvssm_scan(const attamba_scan_args* a, attamba_stream_t stream) {
  if (!a) return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan: args null");
  if (const int st = check_scan(a, "kvssm_scan")) return st;
  if (!a->y_k || !a->y_v) return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan: y_k or y_v null");
  if (!a->kb != !a->vb) return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan: kb and vb must both be set or both null");
  if (!a->h_last_k != !a->h_last_v) return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan: h_last_k/h_last_v must match");
  if (a->h_last_k && (!a->seq_cu || a->S < 1))
    return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan: h_last needs seq_cu and S >= 1");
  if (const attamba_ssm_block_args* b = a->block) {
    if (b->conv_width < 0 || b->conv_width > 4)
      return fail(ATTAMBA_ERR_BAD_SHAPE, "kvssm_scan: block conv_width=%d (0..4)", b->conv_width);
    if (b->conv_width > 0 && (!b->conv_w_k || !b->conv_b_k || !b->conv_w_v || !b->conv_b_v))
      return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan: block convolution taps or bias null");
    if (!b->z_k != !b->z_v) return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan: block z_k and z_v must both be set or both null");
  }
  return hip_status(attamba::launch_kvssm_scan(*a, reinterpret_cast<hipStream_t>(stream)), "kvssm_scan launch");
}

int attamba_kvssm_scan_bwd(const attamba_scan_bwd_args* b, attamba_stream_t stream) {
  if (!b) return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan_bwd: args null");
  const attamba_scan_args* a = &b->fwd;
  if (const int st = check_scan(a, "kvssm_scan_bwd")) return st;
  if (a->block) return fail(ATTAMBA_ERR_UNSUPPORTED, "kvssm_scan_bwd: the Mamba-block variant has no backward");
  if (!b->gy_k || !b->gy_v || !b->dx_k || !b->dx_v || !b->ddt_k || !b->ddt_v || !b->dbm_k || !b->dcm_k ||
      !b->dbm_v || !b->dcm_v || !b->dA_k || !b->dA_v || !b->dD_k || !b->dD_v || !b->dbias_k || !b->dbias_v)
    return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan_bwd: a required gradient pointer is null");
  if (!b->gkb != !b->gvb) return fail(ATTAMBA_ERR_NULL_ARG, "kvssm_scan_bwd: gkb and gvb must both be set or both null");
  for (const void* ptr : {a->bm_k, a->cm_k, a->bm_v, a->cm_v})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
      return fail(ATTAMBA_ERR_BAD_SHAPE, "kvssm_scan_bwd: bm/cm pointers must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  attamba::ZeroList z{};
  float* bufs[attamba::kMaxZero] = {b->dbm_k, b->dcm_k, b->dbm_v, b->dcm_v, b->dA_k, b->dA_v,
                                    b->dD_k, b->dD_v, b->dbias_k, b->dbias_v};
  const int counts[attamba::kMaxZero] = {a->T * a->N, a->T * a->N, a->T * a->N, a->T * a->N, a->d * a->N,
                                         a->d * a->N, a->d, a->d, a->d, a->d};
  for (int i = 0; i < attamba::kMaxZero; ++i) { z.ptr[i] = bufs[i]; z.count[i] = counts[i]; }
  if (const int st = hip_status(attamba::launch_zero(z, attamba::kMaxZero, s), "kvssm_scan_bwd zero")) return st;
  attamba::ScanBwdParams p{};
  p.T = a->T; p.d = a->d; p.n_chunks = a->n_chunks; p.chunk_cu = a->chunk_cu;
  const bool sep = a->x_v && a->x_v != a->x;
  p.side[0] = {a->x, a->dt_k, a->bm_k, a->cm_k, b->gy_k, b->gkb, a->A_k, a->D_k, a->bias_k,
               b->dx_k, b->ddt_k, b->dbm_k, b->dcm_k, b->dA_k, b->dD_k, b->dbias_k};
  p.side[1] = {sep ? a->x_v : a->x, a->dt_v, a->bm_v, a->cm_v, b->gy_v, b->gvb, a->A_v, a->D_v, a->bias_v,
               b->dx_v, b->ddt_v, b->dbm_v, b->dcm_v, b->dA_v, b->dD_v, b->dbias_v};
  return hip_status(attamba::launch_kvssm_scan_bwd(p, a->N, a->dtype, s), "kvssm_scan_bwd launch");
}

int attamba_chunk_attn_fwd(const attamba_attn_args* a, attamba_stream_t stream) {
  if (!a) return fail(ATTAMBA_ERR_NULL_ARG, "chunk_attn_fwd: args null");
  if (const int st = check_attn(a, "chunk_attn_fwd")) return st;
  const float scale = a->scale > 0.0f ? a->scale : 1.0f / std::sqrt(static_cast<float>(a->hd));
  return hip_status(attamba::launch_chunk_attn(*a, scale, reinterpret_cast<hipStream_t>(stream)),
                    "chunk_attn_fwd launch");
}

int attamba_chunk_attn_bwd(const attamba_attn_bwd_args* b, attamba_stream_t stream) {
  if (!b) return fail(ATTAMBA_ERR_NULL_ARG, "chunk_attn_bwd: args null");
  const attamba_attn_args* a = &b->fwd;
  if (const int st = check_attn(a, "chunk_attn_bwd")) return st;
  if (a->T > 0 && (!a->lse || !b->dout || !b->dq || !b->dk || !b->dv || !b->dkb || !b->dvb || !b->workspace))
    return fail(ATTAMBA_ERR_NULL_ARG, "chunk_attn_bwd: lse, dout, a gradient or the workspace is null");
  if (a->T > 0 && reinterpret_cast<uintptr_t>(b->workspace) % 16 != 0)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_attn_bwd: the workspace must be 16-byte aligned");
  const size_t need = attamba::attn_bwd_workspace_elems(a->T, a->H, a->hd, a->n_chunks, a->dtype);
  if (b->workspace_elems < need)
    return fail(ATTAMBA_ERR_CAPACITY, "chunk_attn_bwd: workspace of %zu elements, %zu needed",
                b->workspace_elems, need);
  attamba::AttnBwdParams p{};
  attamba::AttnParams& f = p.f;
  f.T = a->T; f.H = a->H; f.S = a->S; f.max_seqlen = a->max_seqlen; f.L = a->L;
  f.train = a->mode == ATTAMBA_MASK_TRAIN ? 1 : 0;
  f.scale = a->scale > 0.0f ? a->scale : 1.0f / std::sqrt(static_cast<float>(a->hd));
  f.q = a->q; f.k = a->k; f.v = a->v; f.kb = a->kb; f.vb = a->vb;
  f.seq_cu = a->seq_cu; f.chunk_cu = a->chunk_cu; f.token_chunk = a->token_chunk;
  f.out = a->out; f.lse = a->lse;
  p.dout = b->dout; p.dq = b->dq; p.dk = b->dk; p.dv = b->dv; p.dkb = b->dkb; p.dvb = b->dvb;
  p.delta = b->workspace;
  p.row_w = reinterpret_cast<int*>(b->workspace + static_cast<size_t>(a->H) * a->T);
  p.row_ce = p.row_w + a->T;
  p.n_chunks = a->n_chunks;
  p.dkv_split = attamba::attn_bwd_dkv_split(a->T, a->hd, a->n_chunks, a->dtype);
  if (p.dkv_split > 1) {
    const size_t part = static_cast<size_t>(p.dkv_split) * a->n_chunks * a->H * a->hd;
    p.dkb_part = b->workspace + (static_cast<size_t>(a->H + 2) * a->T + 63) / 64 * 64;
    p.dvb_part = p.dkb_part + part;
  }
  return hip_status(attamba::launch_chunk_attn_bwd(p, a->hd, a->dtype, reinterpret_cast<hipStream_t>(stream)),
                    "chunk_attn_bwd launch");
}

int attamba_chunk_attn_bwd_workspace_size(const attamba_attn_bwd_args* b, size_t* elems) {
  if (!b || !elems) return fail(ATTAMBA_ERR_NULL_ARG, "chunk_attn_bwd_workspace_size: null pointer");
  const attamba_attn_args* a = &b->fwd;
  if (a->T < 0 || a->H < 1 || a->n_chunks < 0)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "chunk_attn_bwd_workspace_size: T=%d H=%d n_chunks=%d", a->T, a->H,
                a->n_chunks);
  *elems = attamba::attn_bwd_workspace_elems(a->T, a->H, a->hd, a->n_chunks, a->dtype);
  return ATTAMBA_OK;
}

int attamba_input_proj(const attamba_proj_args* a, attamba_stream_t stream) {
  if (!a) return fail(ATTAMBA_ERR_NULL_ARG, "input_proj: args null");
  if (!dtype_ok(a->dtype)) return fail(ATTAMBA_ERR_BAD_DTYPE, "input_proj: dtype %d", a->dtype);
  if (a->dtype != ATTAMBA_BF16) return fail(ATTAMBA_ERR_UNSUPPORTED, "input_proj: only bf16 is built");
  if (a->T < 0 || a->d < 64 || a->d % 64 != 0 || a->n_out < 1 || a->n_seg < 1 ||
      a->n_seg > ATTAMBA_PROJ_MAX_SEGMENTS)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "input_proj: T=%d d=%d n_out=%d n_seg=%d", a->T, a->d, a->n_out, a->n_seg);
  if (a->seg_start[0] != 0 || a->seg_start[a->n_seg] != a->n_out)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "input_proj: segments must cover features 0 .. n_out");
  // every segment start and end a multiple of 4: the kernels store 4 features (8 bytes) at once
  for (int i = 0; i < a->n_seg; ++i)
    if (a->seg_start[i + 1] <= a->seg_start[i] || a->seg_start[i] % 4 != 0 || a->seg_start[i + 1] % 4 != 0)
      return fail(ATTAMBA_ERR_BAD_SHAPE, "input_proj: segment %d (start %d, end %d) empty or not on multiples of 4",
                  i, a->seg_start[i], a->seg_start[i + 1]);
  if (static_cast<int64_t>(a->T) * a->d > INT32_MAX || static_cast<int64_t>(a->n_out) * a->d > INT32_MAX ||
      static_cast<int64_t>(a->T) * a->n_out > INT32_MAX)
    return fail(ATTAMBA_ERR_UNSUPPORTED, "input_proj: T*d, n_out*d or T*n_out exceeds 2^31 elements");
  if (!a->x || !a->w) return fail(ATTAMBA_ERR_NULL_ARG, "input_proj: x or w null");
  for (int i = 0; i < a->n_seg; ++i)
    if (!a->out[i]) return fail(ATTAMBA_ERR_NULL_ARG, "input_proj: out[%d] null", i);
  attamba::ProjParams p{};
  p.T = a->T; p.d = a->d; p.n_out = a->n_out; p.n_seg = a->n_seg;
  p.x = a->x; p.w = a->w;
  for (int i = 0; i <= ATTAMBA_PROJ_MAX_SEGMENTS; ++i)
    p.seg_start[i] = i <= a->n_seg ? a->seg_start[i] : a->n_out;
  for (int i = 0; i < ATTAMBA_PROJ_MAX_SEGMENTS; ++i) p.out[i] = i < a->n_seg ? a->out[i] : nullptr;
  return hip_status(attamba::launch_proj_gemm(p, reinterpret_cast<hipStream_t>(stream)), "input_proj launch");
}

int attamba_decode_workspace_size(const attamba_decode_cache* c, size_t* bytes) {
  if (!c || !bytes) return fail(ATTAMBA_ERR_NULL_ARG, "decode_workspace_size: null pointer");
  if (c->B < 1 || c->H < 1 || c->hd < 1 || c->cap < 0 || c->L < 0)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "decode_workspace_size: B=%d H=%d hd=%d cap=%d L=%d", c->B, c->H, c->hd,
                c->cap, c->L);
  *bytes = attamba::decode_workspace_bytes(c->B, c->H, c->hd, c->cap, c->L);
  return ok();
}

int attamba_decode_load_prefix(attamba_decode_cache* c, const attamba_decode_prefix* pf,
                               attamba_stream_t stream) {
  if (!c || !pf) return fail(ATTAMBA_ERR_NULL_ARG, "decode_load_prefix: null pointer");
  if (!dtype_ok(c->dtype)) return fail(ATTAMBA_ERR_BAD_DTYPE, "decode_load_prefix: dtype %d", c->dtype);
  if (c->B < 1 || c->H < 1 || c->P < 1 || c->L < 0 || c->layer_idx < 0 || c->cap < 0 || c->d != c->H * c->hd)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "decode_load_prefix: B=%d H=%d hd=%d d=%d P=%d L=%d cap=%d", c->B, c->H,
                c->hd, c->d, c->P, c->L, c->cap);
  if (c->hd != 32 && c->hd != 64 && c->hd != 128)
    return fail(ATTAMBA_ERR_UNSUPPORTED, "decode_load_prefix: hd=%d (32, 64 or 128)", c->hd);
  if (c->N != 16 && c->N != 32) return fail(ATTAMBA_ERR_UNSUPPORTED, "decode_load_prefix: N=%d (16 or 32)", c->N);
  if (c->d % 64 != 0) return fail(ATTAMBA_ERR_UNSUPPORTED, "decode_load_prefix: d=%d not a multiple of 64", c->d);
  if (!pf->seq_cu_host || !pf->seq_cu || !pf->token_chunk || !pf->y_k || !pf->y_v || !pf->kb || !pf->vb ||
      !pf->h_last_k || !pf->h_last_v || !c->kb || !c->vb || !c->h_k || !c->h_v || (c->L > 0 && (!c->kw || !c->vw)))
    return fail(ATTAMBA_ERR_NULL_ARG, "decode_load_prefix: a required pointer is null");
  if (pf->S != c->B || pf->n0 < 0)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "decode_load_prefix: S=%d (cache B=%d), n0=%d", pf->S, c->B, pf->n0);
  if (pf->seq_cu_host[0] != 0)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "decode_load_prefix: seq_cu must start at 0");
  for (int s = 0; s < pf->S; ++s)
    if (pf->seq_cu_host[s + 1] - pf->seq_cu_host[s] != pf->n0)
      return fail(ATTAMBA_ERR_BAD_SHAPE, "decode_load_prefix: sequence %d has %d tokens, not n0=%d", s,
                  pf->seq_cu_host[s + 1] - pf->seq_cu_host[s], pf->n0);
  if (static_cast<int64_t>(pf->seq_cu_host[pf->S]) * c->d > INT32_MAX)
    return fail(ATTAMBA_ERR_UNSUPPORTED, "decode_load_prefix: T*d exceeds 2^31 elements");
  const int64_t P = c->P, o = c->layer_idx % c->P;
  const int64_t n_bound = ends_before(pf->n0, P, o);
  if (n_bound > c->cap)
    return fail(ATTAMBA_ERR_CAPACITY, "decode_load_prefix: %lld completed chunks exceed cap=%d",
                static_cast<long long>(n_bound), c->cap);
  const int w0 = c->L > 0 ? (pf->n0 - c->L > 0 ? pf->n0 - c->L : 0) : pf->n0;
  const int st = hip_status(attamba::launch_decode_load_prefix(*c, *pf, static_cast<int>(n_bound), w0,
                                                               reinterpret_cast<hipStream_t>(stream)),
                            "decode_load_prefix launch");
  if (st != ATTAMBA_OK) return st;
  c->pos = pf->n0;
  c->n_bound = static_cast<int32_t>(n_bound);
  return ATTAMBA_OK;
}

// Checks of a decode step and its launch. Scratch: the caller's workspace (attamba_decode_step), or,
// with static_scratch, the library's static device array, whose address is looked up only after
// every check has passed (attamba_decode_step_noalloc).
static int decode_step_impl(attamba_decode_cache* c, const attamba_decode_inputs* in, bool static_scratch,
                            attamba_stream_t stream, const char* name) {
  if (!c || !in) return fail(ATTAMBA_ERR_NULL_ARG, "%s: null pointer", name);
  void* workspace = static_scratch ? nullptr : c->workspace;
  const size_t workspace_bytes = static_scratch ? attamba::kDecodeScratchBytes : c->workspace_bytes;
  if (!dtype_ok(c->dtype)) return fail(ATTAMBA_ERR_BAD_DTYPE, "%s: dtype %d", name, c->dtype);
  if (c->B < 1 || c->H < 1 || c->P < 1 || c->L < 0 || c->layer_idx < 0 || c->cap < 0 || c->pos < 0 ||
      c->n_bound < 0 || c->d != c->H * c->hd)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "%s: B=%d H=%d hd=%d d=%d P=%d L=%d cap=%d pos=%lld", name, c->B, c->H,
                c->hd, c->d, c->P, c->L, c->cap, static_cast<long long>(c->pos));
  if (c->hd != 32 && c->hd != 64 && c->hd != 128)
    return fail(ATTAMBA_ERR_UNSUPPORTED, "%s: hd=%d (32, 64 or 128)", name, c->hd);
  if (c->N != 16 && c->N != 32) return fail(ATTAMBA_ERR_UNSUPPORTED, "%s: N=%d (16 or 32)", name, c->N);
  if (c->d % 64 != 0) return fail(ATTAMBA_ERR_UNSUPPORTED, "%s: d=%d not a multiple of 64", name, c->d);
  if (!c->kb || !c->vb || !c->h_k || !c->h_v || !c->A_k || !c->A_v || !c->D_k || !c->D_v || !c->bias_k ||
      !c->bias_v || (!static_scratch && !workspace) || (c->L > 0 && (!c->kw || !c->vw)) || !in->q || !in->x || !in->dt_k ||
      !in->dt_v || !in->bm_k || !in->cm_k || !in->bm_v || !in->cm_v || !in->out)
    return fail(ATTAMBA_ERR_NULL_ARG, "%s: a required pointer is null", name);
  const int64_t P = c->P, o = c->layer_idx % c->P, pos = c->pos;
  if (ends_before(pos, P, o) != c->n_bound)
    return fail(ATTAMBA_ERR_BAD_SHAPE, "%s: n_bound=%d but %lld chunk ends precede pos=%lld", name, c->n_bound,
                static_cast<long long>(ends_before(pos, P, o)), static_cast<long long>(pos));
  attamba::DecodeLaunch dl{};
  dl.pos = pos;
  dl.is_start = starts_chunk(pos, P, o) ? 1 : 0;
  dl.is_end = starts_chunk(pos + 1, P, o) ? 1 : 0;
  if (dl.is_end && c->n_bound >= c->cap)
    return fail(ATTAMBA_ERR_CAPACITY, "%s: boundary cache full (cap=%d)", name, c->cap);
  const size_t need = attamba::decode_workspace_bytes(c->B, c->H, c->hd, c->cap, c->L);
  if (workspace_bytes < need)
    return fail(ATTAMBA_ERR_CAPACITY, "%s: the step needs %zu bytes of scratch, %zu available", name, need,
                workspace_bytes);
  dl.slot = c->L > 0 ? static_cast<int>(pos % c->L) : 0;
  dl.n_bound_before = c->n_bound;
  const int64_t w = c->L > 0 ? (pos - c->L + 1 > 0 ? pos - c->L + 1 : 0) : pos + 1;
  dl.w = static_cast<int>(w);
  dl.w_slot = c->L > 0 ? static_cast<int>(w % c->L) : 0;
  dl.E = static_cast<int>(ends_before(w, P, o));
  dl.n_window = c->L > 0 ? static_cast<int>(pos - w + 1) : 0;
  dl.scale = 1.0f / std::sqrt(static_cast<float>(c->hd));
  if (pos > INT32_MAX - 2) return fail(ATTAMBA_ERR_BAD_SHAPE, "%s: pos too large", name);
  if (static_scratch) {
    const hipError_t e = attamba::decode_scratch(&workspace);
    if (e != hipSuccess)
      return fail(ATTAMBA_ERR_HIP, "%s: device address of the scratch: %s", name, hipGetErrorString(e));
  }
  attamba_decode_cache cl = *c;
  cl.workspace = workspace;
  cl.workspace_bytes = workspace_bytes;
  const int st = hip_status(attamba::launch_decode_step(cl, *in, dl, reinterpret_cast<hipStream_t>(stream)),
                            name);
  if (st != ATTAMBA_OK) return st;
  c->pos = pos + 1;
  c->n_bound += dl.is_end;
  return ATTAMBA_OK;
}

int attamba_decode_step(attamba_decode_cache* c, const attamba_decode_inputs* in,
                        attamba_stream_t stream) {
  return decode_step_impl(c, in, false, stream, "decode_step");
}

int attamba_decode_step_noalloc(attamba_decode_cache* c, const attamba_decode_inputs* in,
                                attamba_stream_t stream) {
  return decode_step_impl(c, in, true, stream, "decode_step_noalloc");
}

}  // extern "C"
