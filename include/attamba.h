/*
 * attamba.h — C ABI of the Attamba KV-SSM forward on AMD Instinct MI355X (gfx950).
 *
 * The method is Attamba ("Attending To Multi-Token States", arXiv 2411.17685): two selective
 * state-space scans SSM_K and SSM_V take the place of the key and value projections and
 * compress every chunk of P tokens into one boundary state; attention then runs over the
 * boundary states of completed chunks, the current partial chunk (M_train) and the L most
 * recent uncompressed tokens (M_test plus sliding window); decoding keeps a cache of
 * boundary states. Page references: pith.science review of the paper, sections "What carries
 * the argument", "Core claim", "If this is right", "Assumptions & free parameters" and the
 * Referee Report; rohan-paul.com summary, "Solution in this Paper" and "Key Insights".
 *
 * Conventions for every entry point:
 *  - Return value: ATTAMBA_OK (0) or one of the ATTAMBA_ERR_* codes. On error nothing has
 *    been launched, and attamba_last_error() (thread-local) describes the first failing
 *    check. Argument checks are host-side and synchronous; kernels never trap.
 *  - Tensors are caller-owned, contiguous, row-major device pointers unless named *_host.
 *    The library allocates no device memory and keeps no state between calls; work that
 *    needs scratch takes a caller-provided workspace.
 *  - Device index arrays (seq_cu, chunk_cu, token_chunk) must be well formed (offsets
 *    non-decreasing, starting at 0, ending at T; every sequence start is a chunk start);
 *    that is the caller's contract. Kernels bound every write by the sizes passed here.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the default
 *    stream); no call synchronises the host with the device.
 *  - Activations are ATTAMBA_FP32 or ATTAMBA_BF16; SSM parameters (A, D, dt bias) are
 *    always float32. Arithmetic is float32 throughout (state, exponentials, softmax and
 *    accumulation); bf16 outputs are rounded to nearest even.
 */
#ifndef ATTAMBA_H
#define ATTAMBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* attamba_stream_t; /* hipStream_t */

enum {
  ATTAMBA_OK = 0,
  ATTAMBA_ERR_NULL_ARG = 1,    /* a required pointer is NULL */
  ATTAMBA_ERR_BAD_SHAPE = 2,   /* sizes negative, inconsistent, or index data malformed */
  ATTAMBA_ERR_BAD_DTYPE = 3,   /* unknown dtype code */
  ATTAMBA_ERR_CAPACITY = 4,    /* an output buffer is too small for the result */
  ATTAMBA_ERR_UNSUPPORTED = 5, /* valid but not built (state size, head dim, width) */
  ATTAMBA_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
};

enum { ATTAMBA_FP32 = 0, ATTAMBA_BF16 = 1 };

/* M_train (paper Eq. 5): a query sees the boundary state of every completed chunk and the
 * per-token outputs of its own partial chunk. M_test (Eq. 7, causal reading): it sees only
 * boundary states of chunks that ended at or before it. Both add the window of the L most
 * recent tokens (Eq. 8). pith.science "What carries the argument"; the Referee Report's
 * second major comment explains why M_test must not expose the current chunk's final state
 * before the chunk is complete. */
enum { ATTAMBA_MASK_TRAIN = 0, ATTAMBA_MASK_TEST = 1 };

const char* attamba_version(void);
const char* attamba_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
const char* attamba_last_error(void);

/* ------------------------------------------------------------------------------------------
 * Segmentation (pith.science "What carries the argument": cyclic chunking shifts the chunk
 * offset by layer index; "Assumptions & free parameters": offset = layer index; "If this is
 * right": variable-length boundaries via cu_seqlens).
 *
 * Uniform chunking of a sequence of n tokens with o = layer_idx mod P: chunks start at local
 * position 0 and at every t with t = o (mod P); the first chunk has length o when o > 0, a
 * trailing partial chunk is a chunk. Chunks never cross sequences.
 * ---------------------------------------------------------------------------------------- */

/* Host only. Number of chunks of the packed batch (S sequences, offsets seq_cu_host[S+1]):
 * per sequence ceil(n/P) if o = 0, 1 + ceil((n-o)/P) if 0 < o < n, 1 if 0 < n <= o, 0 if
 * n = 0. Errors: NULL_ARG; BAD_SHAPE if S < 0, P < 1, layer_idx < 0, seq_cu not starting at 0
 * or decreasing, or the count exceeds INT32_MAX - 1. */
int attamba_count_chunks(const int32_t* seq_cu_host, int32_t S, int32_t P, int32_t layer_idx,
                         int32_t* n_chunks_out);

/* Host only. Explicit (e.g. randomized) chunking: chunk_len_host[n_len] lists chunk lengths
 * sequence by sequence; each is >= 1 and they tile every sequence exactly. Writes the chunk
 * offsets chunk_cu_host_out[n_len + 1] (prefix sums). Errors: NULL_ARG; BAD_SHAPE if the
 * lengths do not tile the sequences. */
int attamba_chunk_cu_from_lengths(const int32_t* seq_cu_host, int32_t S,
                                  const int32_t* chunk_len_host, int32_t n_len,
                                  int32_t* chunk_cu_host_out);

/* Device. Uniform chunking computed on the GPU from the device copy of seq_cu[S+1] over
 * T tokens (seq_cu[0] = 0, non-decreasing, seq_cu[S] = T). Writes chunk_cu[n_chunks + 1] (chunk start offsets, then T), and, if not NULL,
 * token_chunk[T] (chunk of every token) and is_end[T] (1 at the last token of every chunk,
 * else 0). n_chunks must be the count attamba_count_chunks returns for the same seq_cu; the
 * kernels never write past n_chunks + 1 entries. Errors: NULL_ARG (seq_cu, chunk_cu),
 * BAD_SHAPE (S < 1, T < 0, P < 1, layer_idx < 0, n_chunks < 0), HIP. */
int attamba_chunk_boundaries(const int32_t* seq_cu, int32_t S, int32_t T, int32_t P,
                             int32_t layer_idx, int32_t n_chunks, int32_t* chunk_cu,
                             int32_t* token_chunk, uint8_t* is_end, attamba_stream_t stream);

/* Device. Per-token chunk index and chunk-end flags from device chunk offsets
 * chunk_cu[n_chunks + 1] (any chunking, e.g. from attamba_chunk_cu_from_lengths). Either
 * output may be NULL. Errors: NULL_ARG (chunk_cu), BAD_SHAPE (n_chunks < 0, T < 0), HIP. */
int attamba_chunk_index(const int32_t* chunk_cu, int32_t n_chunks, int32_t T,
                        int32_t* token_chunk, uint8_t* is_end, attamba_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * KV-SSM scan (pith.science "Core claim": K^(p) = SSM_K(X^(p)), V^(p) = SSM_V(X^(p)) per
 * chunk; the selective SSM is the paper's Eq. 3, cited in "Assumptions & free parameters").
 * For each SSM S in {K, V}, channel c and token t, with the state reset to zero at every
 * chunk start:
 *   delta = softplus(dt_S[t,c] + bias_S[c])
 *   h[c,:] = exp(delta * A_S[c,:]) * h[c,:] + delta * x[t,c] * bm_S[t,:]
 *   y_S[t,c] = sum_n cm_S[t,n] * h[c,n] + D_S[c] * x[t,c]
 * The boundary state of chunk q is the output at its last token (the review's K^(p)[-1]).
 * Both SSMs read the layer input x. For the variant that keeps explicit key and value
 * projections in front of the SSMs (pith.science "If this is right": dropping them costs
 * about 1 % perplexity), x_v gives SSM_V its own input (x then feeds SSM_K only).
 * ---------------------------------------------------------------------------------------- */
/* Optional Mamba-block pieces around each SSM (pith.science "Assumptions & free parameters":
 * the selective SSM is the core of a Mamba block, Section 3.2, Eq. 3). With them, SSM S scans
 *   xc = silu(conv_b_S + sum_k conv_w_S[c, k] * xin[t - (K-1) + k])     (causal, depthwise)
 * instead of its input xin (x, or x_v for SSM_V), with the skip term D_S * xc, and its outputs
 * become y * silu(z_S[t, c]); silu(v) = v / (1 + e^-v). The block runs on each chunk alone, so the
 * convolution restarts at every chunk start like the state: positions before the chunk start
 * count as zero. The boundary state of a chunk is the (gated) output at its last token.
 * Forward only: the scan backward and the decode step take the plain SSM. */
typedef struct {
  int32_t conv_width;   /* taps K of the convolution, 1..4; 0: no convolution (xc = xin) */
  const float* conv_w_k;/* [d, K] taps of SSM_K's convolution; tap K-1 weighs the current token */
  const float* conv_b_k;/* [d] */
  const float* conv_w_v;/* [d, K] */
  const float* conv_b_v;/* [d] */
  const void* z_k;      /* [T, d] gate input of SSM_K (activation dtype), or NULL: no gate */
  const void* z_v;      /* [T, d] gate input of SSM_V, or NULL */
} attamba_ssm_block_args;

typedef struct {
  int32_t T;        /* tokens in the packed batch (>= 0) */
  int32_t d;        /* channels = H * hd; multiple of 64 */
  int32_t N;        /* state size per channel: 16 or 32 */
  int32_t dtype;    /* activations: ATTAMBA_FP32 or ATTAMBA_BF16 */
  int32_t n_chunks; /* chunks; chunk_cu has n_chunks + 1 entries */
  const int32_t* chunk_cu;            /* [n_chunks + 1] device */
  const void* x;                      /* [T, d] */
  const void* dt_k;                   /* [T, d] step-size pre-activation (bias not added) */
  const void* dt_v;                   /* [T, d] */
  const void* bm_k;                   /* [T, N] input matrix of SSM_K */
  const void* cm_k;                   /* [T, N] output matrix of SSM_K */
  const void* bm_v;                   /* [T, N] */
  const void* cm_v;                   /* [T, N] */
  const float* A_k;                   /* [d, N] (negative entries) */
  const float* A_v;                   /* [d, N] */
  const float* D_k;                   /* [d] */
  const float* D_v;                   /* [d] */
  const float* bias_k;                /* [d] step-size bias */
  const float* bias_v;                /* [d] */
  void* y_k;                          /* [T, d] out: per-token keys, = [T, H, hd] */
  void* y_v;                          /* [T, d] out: per-token values */
  void* kb;                           /* [n_chunks, d] out or NULL: boundary keys */
  void* vb;                           /* [n_chunks, d] out or NULL: boundary values */
  /* Optional hand-off to decoding: the SSM states after the last token of each sequence. */
  const int32_t* seq_cu;              /* [S + 1] device, or NULL */
  int32_t S;
  float* h_last_k;                    /* [S, d, N] out or NULL */
  float* h_last_v;                    /* [S, d, N] out or NULL */
  const void* x_v;                    /* [T, d] input of SSM_V, or NULL: SSM_V reads x */
  const attamba_ssm_block_args* block;/* Mamba-block convolution and gate, or NULL: plain SSMs */
} attamba_scan_args;

/* Errors: NULL_ARG (also a block whose conv_width > 0 lacks a tap or bias array), BAD_SHAPE
 * (T, n_chunks < 0; d not a positive multiple of 64; block conv_width outside 0..4),
 * BAD_DTYPE, UNSUPPORTED (N not 16 or 32, or T*d of 2^31 elements or more), HIP. */
int attamba_kvssm_scan(const attamba_scan_args* args, attamba_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Chunk-aware causal attention over per-token and boundary keys (pith.science "What carries
 * the argument": M_train Eq. 5, M_test Eq. 7, window Eq. 8; the map shrinks from n x n to
 * about n/P + L keys per query).
 * For query row i of a sequence starting at s0, with w_i = max(s0, i - L + 1) and, under
 * M_train, w_i = min(w_i, start of i's chunk): the visible keys are the boundary states of
 * the chunks that end before w_i plus the per-token keys at positions w_i..i. Each position
 * counts once. O_i = softmax(scale * q_i . k_j) v_j over those keys; LSE_i = log of the
 * softmax denominator (natural log). A row with no visible key gets O = 0, LSE = -inf.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t T;           /* tokens */
  int32_t H;           /* heads (query heads = key/value heads) */
  int32_t hd;          /* head dim: 32, 64 or 128 */
  int32_t dtype;       /* q, k, v, kb, vb and out share this type */
  int32_t S;           /* sequences; seq_cu has S + 1 entries */
  int32_t max_seqlen;  /* upper bound on every sequence length (sizes the grid) */
  int32_t n_chunks;
  int32_t L;           /* leading tokens kept uncompressed (>= 0) */
  int32_t mode;        /* ATTAMBA_MASK_TRAIN or ATTAMBA_MASK_TEST */
  float scale;         /* softmax scale; 0 means 1/sqrt(hd) */
  const void* q;       /* [T, H, hd] */
  const void* k;       /* [T, H, hd] per-token keys (y_k) */
  const void* v;       /* [T, H, hd] per-token values (y_v) */
  const void* kb;      /* [n_chunks, H, hd] boundary keys */
  const void* vb;      /* [n_chunks, H, hd] boundary values */
  const int32_t* seq_cu;      /* [S + 1] device */
  const int32_t* chunk_cu;    /* [n_chunks + 1] device */
  const int32_t* token_chunk; /* [T] device */
  void* out;           /* [T, H, hd] out */
  float* lse;          /* [H, T] out or NULL */
} attamba_attn_args;

/* Errors: NULL_ARG, BAD_SHAPE (negative sizes, S < 1, max_seqlen < 1 with T > 0,
 * L < 0, unknown mode), BAD_DTYPE, UNSUPPORTED (hd not 32/64/128, or T*H*hd of 2^31 elements
 * or more), HIP. */
int attamba_chunk_attn_fwd(const attamba_attn_args* args, attamba_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Decode step over a cache of boundary states (pith.science "Core claim": at inference only
 * the final SSM state of each chunk is cached; "If this is right": the cache shrinks by
 * about P, with L leading tokens kept). Uses M_test with the window. Every sequence of the
 * batch is at the same position `pos`, with o = layer_idx mod P:
 *   1. chunk start (pos = 0 or pos = o mod P): the SSM states are zeroed;
 *   2. one SSM_K and SSM_V step gives the token's key and value (the recurrence above);
 *   3. the key/value go to window slot pos mod L (if L > 0) and, if pos ends a chunk
 *      ((pos + 1 - o) = 0 mod P), are appended as boundary state n_bound;
 *   4. attention over boundary states 0 .. E-1, E = number of chunk ends before
 *      w = max(0, pos - L + 1), plus the window positions w..pos;
 *   5. pos and n_bound (host fields) advance.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t B, H, hd, d, N, P, L, layer_idx;
  int32_t cap;         /* boundary-state capacity per sequence */
  int32_t dtype;       /* cache, q, x, dt, bm/cm and out share this type */
  int64_t pos;         /* host: position of the next token (same for all sequences) */
  int32_t n_bound;     /* host: boundary states stored per sequence */
  void* kb;            /* [B, H, cap, hd] boundary keys */
  void* vb;            /* [B, H, cap, hd] boundary values */
  void* kw;            /* [B, H, L, hd] window keys (slot = position mod L); NULL if L = 0 */
  void* vw;            /* [B, H, L, hd] window values */
  float* h_k;          /* [B, d, N] SSM_K state */
  float* h_v;          /* [B, d, N] SSM_V state */
  const float* A_k;    /* [d, N] */
  const float* A_v;
  const float* D_k;    /* [d] */
  const float* D_v;
  const float* bias_k; /* [d] */
  const float* bias_v;
  void* workspace;     /* device scratch of attamba_decode_workspace_size() bytes */
  size_t workspace_bytes;
} attamba_decode_cache;

typedef struct {
  const void* q;       /* [B, H, hd] */
  const void* x;       /* [B, d] */
  const void* dt_k;    /* [B, d] */
  const void* dt_v;    /* [B, d] */
  const void* bm_k;    /* [B, N] */
  const void* cm_k;    /* [B, N] */
  const void* bm_v;    /* [B, N] */
  const void* cm_v;    /* [B, N] */
  void* out;           /* [B, H, hd] out */
} attamba_decode_inputs;

/* Workspace bytes a decode step needs for this cache geometry (B, H, hd, cap, L); host only.
 * Errors: NULL_ARG, BAD_SHAPE. */
int attamba_decode_workspace_size(const attamba_decode_cache* cache, size_t* bytes);

/* Errors: NULL_ARG; BAD_SHAPE (inconsistent sizes, pos < 0, n_bound not the number of chunk
 * ends before pos); CAPACITY (an append would exceed cap, or the workspace is too small);
 * BAD_DTYPE; UNSUPPORTED (hd not 32/64/128, N not 16/32, d not a multiple of 64); HIP.
 * On success cache->pos and cache->n_bound are advanced. */
int attamba_decode_step(attamba_decode_cache* cache, const attamba_decode_inputs* in,
                        attamba_stream_t stream);

/* The same decode step for callers that cannot allocate device memory or be handed a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). Its
 * scratch (the split partials of the attention) is a static device array of
 * ATTAMBA_DECODE_SCRATCH_BYTES that the library holds on every GPU it runs on until the process
 * ends; cache->workspace and cache->workspace_bytes are ignored. Nothing is allocated and no
 * allocating routine is called: the first call on a device looks up the array's device address
 * once (hipGetSymbolAddress). Nothing in the scratch needs to start at zero: every partial the
 * step reads was written by the same step. All calls on one GPU share the one array, so calls
 * that overlap on a GPU (on different streams, or from several threads without ordering) race
 * and give wrong results; calls ordered on one stream are safe. Arguments, semantics and errors
 * are those of attamba_decode_step, plus CAPACITY when the step needs more scratch than
 * ATTAMBA_DECODE_SCRATCH_BYTES (4 * B * H * (hd + 2) * (ceil((cap + L) / 256) + 1) bytes, the
 * size attamba_decode_workspace_size reports), and HIP if the array's address cannot be found. */
#define ATTAMBA_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int attamba_decode_step_noalloc(attamba_decode_cache* cache, const attamba_decode_inputs* in,
                                attamba_stream_t stream);

/* Prefill -> decode hand-off (pith.science "Core claim": at inference only the boundary states
 * are cached; a model serves a prompt by prefilling it and then decoding). A batch of S = B
 * sequences, each of exactly n0 tokens, was prefilled with uniform chunking of the cache's P
 * and layer_idx (attamba_chunk_boundaries, then attamba_kvssm_scan with h_last). This call
 * copies into the cache, for every sequence: the boundary states of the chunks that end before
 * n0 (the first ends_before(n0) chunks of the sequence; a trailing partial chunk lives on in h),
 * the per-token keys and values of the window positions max(0, n0 - L) .. n0 - 1 (slot
 * position mod L), and the SSM states after the last prefix token; then sets cache->pos = n0
 * and cache->n_bound. The cache keeps its other fields. All tensors are device pointers except
 * seq_cu_host. Errors: NULL_ARG; BAD_SHAPE (S != B, a sequence not n0 tokens long, n0 < 0, or the
 * cache geometry invalid as for attamba_decode_step); CAPACITY (more completed chunks than
 * cap); BAD_DTYPE; UNSUPPORTED (hd, N, d as for attamba_decode_step); HIP. */
typedef struct {
  int32_t S;                    /* sequences (must equal cache->B) */
  int32_t n0;                   /* prefix length of every sequence */
  const int32_t* seq_cu_host;   /* [S + 1] host copy of seq_cu */
  const int32_t* seq_cu;        /* [S + 1] device */
  const int32_t* token_chunk;   /* [T] device: the prefill's chunk of every token */
  const void* y_k;              /* [T, d] prefill per-token keys (cache dtype) */
  const void* y_v;              /* [T, d] */
  const void* kb;               /* [n_chunks, d] prefill boundary keys */
  const void* vb;               /* [n_chunks, d] */
  const float* h_last_k;        /* [S, d, N] SSM_K state after each sequence's last token */
  const float* h_last_v;        /* [S, d, N] */
} attamba_decode_prefix;

int attamba_decode_load_prefix(attamba_decode_cache* cache, const attamba_decode_prefix* prefix,
                               attamba_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Input projections (the step just before the path: the queries and the per-token inputs
 * dt, Bm, Cm of SSM_K and SSM_V are linear maps of the layer input; pith.science "Core claim":
 * the SSMs replace the key and value projections; the selective SSM's inputs are the paper's
 * Eq. 3, cited in "Assumptions & free parameters").
 *
 * Y = x W^T, bf16 inputs, fp32 accumulation, bf16 outputs:
 *   x    [T, d]      row-major, the layer input;
 *   w    [n_out, d]  row-major, one row per output feature (the stacked weights, e.g. q, dt_K,
 *                    dt_V, Bm_K, Cm_K, Bm_V, Cm_V: n_out = 3 d + 4 N);
 *   the n_out features form n_seg consecutive segments: segment i holds features
 *   seg_start[i] .. seg_start[i+1]-1 and is written to out[i] as a row-major
 *   [T, seg_start[i+1] - seg_start[i]] tensor.
 * All pointers are device pointers owned by the caller; nothing is allocated.
 * Errors: NULL_ARG (x, w or a used out[i]); BAD_SHAPE (T < 0, d < 64 or not a multiple of 64,
 * n_out < 1, n_seg outside 1..ATTAMBA_PROJ_MAX_SEGMENTS, seg_start not starting at 0, not
 * increasing, not ending at n_out, or a segment start or end not a multiple of 4, so n_out too
 * must be one); UNSUPPORTED (dtype
 * other than bf16, or T*d, n_out*d or T*n_out at or above 2^31); HIP.
 * ---------------------------------------------------------------------------------------- */
#define ATTAMBA_PROJ_MAX_SEGMENTS 12
typedef struct {
  int32_t T, d, n_out, dtype;              /* dtype: ATTAMBA_BF16 */
  int32_t n_seg;
  const void* x;
  const void* w;
  int32_t seg_start[ATTAMBA_PROJ_MAX_SEGMENTS + 1];
  void* out[ATTAMBA_PROJ_MAX_SEGMENTS];
} attamba_proj_args;

int attamba_input_proj(const attamba_proj_args* args, attamba_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Backward pass (training). The pages' results are models trained end to end (pith.science
 * "Core claim" and the Referee Report's summary: about 60M parameters, 1B or 8B tokens), with
 * the M_train mask at training time ("What carries the argument", Eq. 5). These two calls
 * give the reverse-mode gradients of
 * attamba_chunk_attn_fwd and attamba_kvssm_scan for a given gradient of their outputs.
 * Gradient sums over tokens or channels use float atomics: results are reproducible up to
 * float reassociation, not bit for bit.
 * ---------------------------------------------------------------------------------------- */

/* Attention backward. fwd holds the forward call's arguments unchanged (sizes, inputs q, k, v,
 * kb, vb, index arrays, mask); fwd.out and fwd.lse must hold that call's results (lse is
 * required). With P the softmax weights and D_i = dout_i . out_i:
 *   dq_i = scale sum_j P_ij (dout_i . v_j - D_i) k_j over the keys row i sees, and for each key
 *   dk_j = scale sum_i P_ij (dout_i . v_j - D_i) q_i, dv_j = sum_i P_ij dout_i over the rows
 *   that see it. A key position reached through the compact boundary states (rows whose band
 *   starts after it) contributes to dkb/dvb; reached as a per-token key (rows whose band holds
 *   it), to dk/dv. The total gradient of the per-token SSM output at a chunk's last token is
 *   dk plus that chunk's dkb (attamba_kvssm_scan_bwd adds them when given gkb/gvb).
 * All gradients are written in fwd.dtype; every element of dq, dk, dv, dkb, dvb is written.
 * Errors: as attamba_chunk_attn_fwd, plus NULL_ARG for lse, dout, a gradient or workspace, and
 * CAPACITY when workspace_elems is below attamba_chunk_attn_bwd_workspace_size(). */
typedef struct {
  attamba_attn_args fwd;
  const void* dout;    /* [T, H, hd] gradient of out */
  void* dq;            /* [T, H, hd] out */
  void* dk;            /* [T, H, hd] out: gradient of k */
  void* dv;            /* [T, H, hd] out: gradient of v */
  void* dkb;           /* [n_chunks, H, hd] out: gradient of kb */
  void* dvb;           /* [n_chunks, H, hd] out: gradient of vb */
  float* workspace;    /* device scratch, caller-owned, contents on entry ignored */
  size_t workspace_elems; /* its size in 4-byte elements */
} attamba_attn_bwd_args;

int attamba_chunk_attn_bwd(const attamba_attn_bwd_args* args, attamba_stream_t stream);

/* 4-byte workspace elements attamba_chunk_attn_bwd needs for these arguments (only fwd.T, H,
 * hd, n_chunks and dtype are read): (H + 2) * T; for bf16 with hd 64 or 128 and at least 4
 * tokens per chunk, that rounded up to a multiple of 64, plus 8 * n_chunks * H * hd (float32
 * partial sums of the dK/dV of the boundary states, whose query rows are split over 4
 * workgroups). The workspace must be 16-byte aligned. Errors: NULL_ARG, BAD_SHAPE. */
int attamba_chunk_attn_bwd_workspace_size(const attamba_attn_bwd_args* args, size_t* elems);

/* KV-SSM scan backward. fwd holds the forward call's arguments (only its inputs are read; its
 * outputs may be NULL; fwd.block must be NULL: UNSUPPORTED otherwise). Given the gradients of y_k, y_v (and optionally of kb, vb, added at each
 * chunk's last token), writes per SSM S in {K, V}:
 *   dx_S   gradient of S's input through S (x for SSM_K; x_v, or x when x_v is NULL, for SSM_V):
 *          when both SSMs read x, the gradient of x is dx_k + dx_v;
 *   ddt_S  gradient of the step-size pre-activation dt_S;
 *   dbm_S, dcm_S [T, N], dA_S [d, N], dD_S, dbias_S [d]: float32, summed over channels / tokens.
 * bm_k, cm_k, bm_v, cm_v must be 16-byte aligned (each lane reads half a row as vectors).
 * Errors: as attamba_kvssm_scan, plus NULL_ARG for a missing gradient pointer and BAD_SHAPE
 * for a misaligned bm/cm pointer. */
typedef struct {
  attamba_scan_args fwd;
  const void* gy_k;    /* [T, d] gradient of y_k */
  const void* gy_v;    /* [T, d] gradient of y_v */
  const void* gkb;     /* [n_chunks, d] gradient of kb, or NULL (zero) */
  const void* gvb;     /* [n_chunks, d] gradient of vb, or NULL */
  void* dx_k;          /* [T, d] out */
  void* dx_v;          /* [T, d] out */
  void* ddt_k;         /* [T, d] out */
  void* ddt_v;         /* [T, d] out */
  float* dbm_k;        /* [T, N] out */
  float* dcm_k;        /* [T, N] out */
  float* dbm_v;        /* [T, N] out */
  float* dcm_v;        /* [T, N] out */
  float* dA_k;         /* [d, N] out */
  float* dA_v;         /* [d, N] out */
  float* dD_k;         /* [d] out */
  float* dD_v;         /* [d] out */
  float* dbias_k;      /* [d] out */
  float* dbias_v;      /* [d] out */
} attamba_scan_bwd_args;

int attamba_kvssm_scan_bwd(const attamba_scan_bwd_args* args, attamba_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ATTAMBA_H */
