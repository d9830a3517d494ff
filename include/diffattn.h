/*
 * libdiffattn - causal differential attention (DiffAttn) for AMD MI355X (gfx950).
 *
 * What the library computes (per batch element b and head h):
 *
 *   S1 = Q1 K1^T / sqrt(d),  S2 = Q2 K2^T / sqrt(d)              (d = width of Q1, K1)
 *   A_k = softmax over keys j <= i of row i of S_k                (causal mask M)
 *   O   = (A1 - lambda * A2) V                                    (V and O are 2d wide)
 *   Y   = (1 - lambda_init) * w * O * (mean(O^2) + eps)^(-1/2)    (per-head RMSNorm)
 *   lambda      = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init
 *   lambda_init = 0.8 - 0.6 * exp(-0.3 * (l - 1))                 (l = layer index >= 1)
 *
 * Sources:
 *   DiffAttn equation, lambda and lambda_init: "Differential Transformer: Transformer que
 *     cancela ruido de atencao" (pt.news.hada.io), section "Como a atencao diferencial
 *     funciona"; the same DiffAttn and lambda formulas in "Differential Transformer:
 *     Canceling Context Noise with Differential Attention" (priorstack.com, Attention
 *     Mechanism tag page), section "Cancelling Context Noise Through Attention Map
 *     Subtraction".
 *   Causal mask M (0 where key j <= query i, -inf otherwise, giving probability 0):
 *     "A Simple Principle From Noise-Cancelling Headphones Supercharges Transformers Like
 *     Never Before" (intoai.pub), section "A Deeper Dive Into Attention Calculations".
 *   lambda shared by all heads of a layer; per-head RMSNorm followed by the factor
 *     (1 - lambda_init): same intoai.pub page, section "Differential Attention With
 *     Multiple Heads"; pt.news.hada.io, section "Estrutura multi-head e arquitetura
 *     completa".
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers unless stated otherwise. Layout is contiguous
 *     row-major [B, H, N, feature] (feature = d for Q1/Q2/K1/K2, 2d for V and outputs);
 *     p->out_layout may make Y and dout token-major instead (diffattn_layout).
 *   - Grouped-query attention: with p->kv_heads = Hkv < H, K1, K2 and V (and the decode
 *     caches) hold Hkv heads, [B, Hkv, N, *], and query head h uses K/V head h / (H / Hkv).
 *     Combining DiffAttn with GQA is named as a likely further speed-up
 *     ("The Evolution of Transformer Attention", open-bookmarks-2024.blogspot.com, section
 *     "Implementation and Future Prospects"); for decode the cache is 1 / (H / Hkv) the
 *     size. Forward, decode, cache append and the QKV
 *     projection take it, and so does the backward (dK1, dK2 and dV of a shared head sum
 *     the contributions of its query heads).
 *   - The caller owns every buffer, including the workspace whose size is given by
 *     diffattn_workspace_bytes. The library keeps no state between calls and allocates
 *     no device memory; the one exception is the static scratch that
 *     diffattn_decode_noalloc uses instead of a workspace (below).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *   - A call returns a status and never aborts. Argument checks run on the host before
 *     any HIP call, so they also work on a machine without a GPU. A failed launch returns
 *     DIFFATTN_E_HIP and diffattn_last_hip_error() gives the hipError_t value.
 *   - Outputs must not overlap inputs (DIFFATTN_E_ARG).
 *   - A problem with batch, heads or seqlen equal to 0 is valid and does nothing.
 *   - Supported: DIFFATTN_FP32 forward with d in {16, 32, 64}; DIFFATTN_BF16 forward,
 *     decode and backward with d = 64, seqlen (or cache capacity) <= 2^22.
 *     Accumulation is float32 everywhere. Other combinations return
 *     DIFFATTN_E_UNSUPPORTED.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIFFATTN_OK = 0,
  DIFFATTN_E_ARG = 1,          /* null/misaligned pointer, bad size, overlap, bad layer */
  DIFFATTN_E_UNSUPPORTED = 2,  /* dtype / head_dim / mode combination not implemented */
  DIFFATTN_E_WORKSPACE = 3,    /* workspace NULL or smaller than diffattn_workspace_bytes */
  DIFFATTN_E_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  DIFFATTN_E_SCRATCH = 5       /* the problem needs more than the static scratch of
                                  diffattn_decode_noalloc (DIFFATTN_DECODE_SCRATCH_BYTES) */
} diffattn_status;

/* Size of the static device scratch that diffattn_decode_noalloc uses on each device. */
#define DIFFATTN_DECODE_SCRATCH_BYTES (32u << 20)

typedef enum { DIFFATTN_FP32 = 0, DIFFATTN_BF16 = 1 } diffattn_dtype;

typedef enum { DIFFATTN_OP_FWD = 0, DIFFATTN_OP_DECODE = 1, DIFFATTN_OP_BWD = 2 } diffattn_op;

/* Layout of the attention output Y (and of dout in the backward). BHN: [B, H, N, 2d], head
 * by head. BNH: [B, N, H, 2d] = [B, N, H 2d], the heads of each token concatenated along
 * channels, which is what the output projection W_O consumes (intoai.pub, "Differential
 * Attention With Multiple Heads"). Q/K/V, the saved tensors and every gradient stay
 * [B, H, N, *]. */
typedef enum { DIFFATTN_LAYOUT_BHN = 0, DIFFATTN_LAYOUT_BNH = 1 } diffattn_layout;

typedef struct {
  int64_t batch;      /* B >= 0 */
  int64_t heads;      /* H >= 0 */
  int64_t seqlen;     /* N >= 0 (forward/backward) or cache capacity L (decode) */
  int32_t head_dim;   /* d: width of Q1, Q2, K1, K2; V and outputs are 2d wide */
  int32_t causal;     /* must be 1 */
  float rms_eps;      /* eps of the per-head RMSNorm, >= 0, added inside the square root */
  int32_t dtype;      /* a diffattn_dtype: element type of Q/K/V, outputs and gradients
                         (a plain integer, so that any value a caller stores is checked
                         rather than read as an enumeration it does not belong to) */
  int32_t out_layout;   /* diffattn_layout of Y and dout; 0 (BHN) when zero-initialised */
  int64_t kv_heads;     /* heads of K1, K2, V (grouped-query attention: query head h reads
                           K/V head h / (heads / kv_heads)); must divide heads; 0 = heads */
} diffattn_problem;

/* The per-layer lambda scalar, as written by diffattn_lambda into device memory and read
 * by every kernel. Kernels consume only the float fields. A caller may also write this
 * struct itself (for example lambda = 0 to get plain causal softmax attention). */
typedef struct {
  double lambda;            /* exp(a) - exp(b) + lambda_init, in float64 */
  double lambda_init;       /* 0.8 - 0.6 * exp(-0.3 * (l - 1)), in float64 */
  double exp_a;             /* exp(lq1 . lk1) */
  double exp_b;             /* exp(lq2 . lk2) */
  float lambda_f;           /* lambda rounded once to float32 (nearest even) */
  float lambda_init_f;      /* lambda_init rounded once to float32 */
  float one_minus_init_f;   /* (1 - lambda_init) in float64, rounded once to float32 */
  float pad;
} diffattn_lambda_state;

/* Quantities the forward saves for the backward (training mode). All float32, device
 * memory owned by the caller. lse_k[i] = log(sum over j <= i of exp(S_k[i, j])) in natural
 * log units; o1 = A1 V and o2 = A2 V (before the lambda combine); rstd = the RMSNorm
 * factor (mean(O^2) + eps)^(-1/2) of each row. */
typedef struct {
  float* lse1;  /* [B, H, N] */
  float* lse2;  /* [B, H, N] */
  float* o1;    /* [B, H, N, 2d] */
  float* o2;    /* [B, H, N, 2d] */
  float* rstd;  /* [B, H, N] */
} diffattn_saved;

/* lambda and lambda_init for one layer, computed on the device in float64 (dot products
 * summed in index order) and rounded once to float32.
 * Source: pt.news.hada.io, "Como a atencao diferencial funciona", lambda and lambda_init
 * equations; one scalar per layer shared by all heads (intoai.pub, "Differential Attention
 * With Multiple Heads").
 *   dim        length of each lambda vector (the head width d), 1 <= dim <= 1024
 *   layer_idx  l >= 1
 *   lq1..lk2   device float32 vectors [dim]
 *   state_out  device pointer to one diffattn_lambda_state (8-byte aligned)
 * Errors: E_ARG for a NULL pointer, dim out of range or layer_idx < 1. */
diffattn_status diffattn_lambda(int32_t dim, int32_t layer_idx, const float* lq1,
                                const float* lk1, const float* lq2, const float* lk2,
                                diffattn_lambda_state* state_out, void* stream);

/* lambda for n_layers consecutive layers in one call, optionally with one fixed
 * lambda_init for all of them. Besides the schedule above, the same lambda_init in every
 * layer (0.8 is the example given) was also tried, with results reported as fairly robust
 * to the choice (pt.news.hada.io, "Como a atencao diferencial funciona", the note after
 * the lambda_init equation).
 *   dim           length of each lambda vector, 1 <= dim <= 1024
 *   n_layers      number of layers, 0 <= n_layers <= 65535 (0: nothing to do, OK, and no
 *                 pointer is read)
 *   first_layer   layer index l of the first layer (>= 1); layer k uses l = first_layer + k
 *   fixed_init    0: lambda_init follows the per-layer schedule (lambda_init is ignored);
 *                 1: lambda_init, which must be finite, for every layer (first_layer then
 *                 only labels the layers)
 *   lq1..lk2      device float32 [n_layers, dim], layer k at offset k * dim (4-byte aligned)
 *   states_out    device diffattn_lambda_state [n_layers] (8-byte aligned), written
 * One launch, one workgroup per layer; each state is computed exactly as diffattn_lambda
 * computes it (bitwise equal under the schedule). Errors: E_ARG for NULL or misaligned
 * pointers, values out of range, a non-finite fixed lambda_init, or states overlapping
 * the vectors. */
diffattn_status diffattn_lambda_layers(int32_t dim, int32_t n_layers, int32_t first_layer,
                                       int32_t fixed_init, float lambda_init,
                                       const float* lq1, const float* lk1, const float* lq2,
                                       const float* lk2, diffattn_lambda_state* states_out,
                                       void* stream);

/* Causal DiffAttn forward with the per-head RMSNorm and (1 - lambda_init) scale fused in.
 * Source: the DiffAttn equation (pt.news.hada.io "Como a atencao diferencial funciona";
 * priorstack.com "Cancelling Context Noise Through Attention Map Subtraction"), causal
 * mask (intoai.pub "A Deeper Dive Into Attention Calculations"), RMSNorm and scale
 * (intoai.pub "Differential Attention With Multiple Heads").
 *   q1, q2, k1, k2  [B, H, N, d] of p->dtype;  v [B, H, N, 2d] of p->dtype
 *   lam             device diffattn_lambda_state (from diffattn_lambda)
 *   rms_weight      device float32 [H, 2d] per-channel RMSNorm weight, or NULL for ones
 *   out             [B, H, N, 2d] of p->dtype (output Y)
 *   saved           host pointer to a struct of device pointers, or NULL (inference).
 *                   Non-NULL: every field must be a valid device buffer (bf16 only).
 *   workspace       device buffer of at least diffattn_workspace_bytes(OP_FWD) bytes
 *                   (bf16: 32 bytes per block of 256 query rows, B * H * ceil(N / 256)
 *                   blocks; it holds the fast pass's row flags, which select the rows a
 *                   fixup recomputes; contents are scratch, nothing needs to be cleared). May
 *                   be NULL when that size is 0 (float32). Too small or NULL when needed:
 *                   DIFFATTN_E_WORKSPACE. It must not overlap any other argument.
 * Pointers must be 16-byte aligned. */
diffattn_status diffattn_fwd(const diffattn_problem* p, const void* q1, const void* q2,
                             const void* k1, const void* k2, const void* v,
                             const diffattn_lambda_state* lam, const float* rms_weight,
                             void* out, const diffattn_saved* saved, void* workspace,
                             size_t workspace_bytes, void* stream);

/* One autoregressive decode step: a single new query per (b, h) against its K1/K2/V cache.
 * The cache already holds the new token, so the query sits at position len - 1 and sees
 * cached keys 0 .. len - 1 (the last row of the causal mask). Keys are processed in
 * splits whose partial softmax states are merged exactly (log-sum-exp merge).
 * Source: autoregressive generation (intoai.pub, "Let's First Learn About The
 * Decoder-Only Transformer") over the DiffAttn equation above; the whole cache is read
 * from HBM every step (priorstack.com, "Multi-Head Latent Attention: Scaling LLM Serving
 * Throughput via Low-Rank KV Compression", section "The Memory Wall: Why the KV Cache
 * Constrains LLM Serving").
 *   q1, q2      [B, H, d]
 *   k1c, k2c    [B, H, L, d] (p->seqlen = L);  vc [B, H, L, 2d]
 *   cache_len   device int32 [B] or NULL (= L for every sequence). Values are clamped to
 *               [1, L] on the device.
 *   out         [B, H, 2d]
 *   workspace   device buffer of at least diffattn_workspace_bytes(OP_DECODE, p) bytes
 * bf16 only, d = 64, 16-byte aligned pointers. */
diffattn_status diffattn_decode(const diffattn_problem* p, const void* q1, const void* q2,
                                const void* k1c, const void* k2c, const void* vc,
                                const int32_t* cache_len, const diffattn_lambda_state* lam,
                                const float* rms_weight, void* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* diffattn_decode without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It allocates nothing (no hipMalloc, no hipFree, no allocating library call).
 * The split partials go to a static device array of DIFFATTN_DECODE_SCRATCH_BYTES
 * (32 MiB) that each device holds from this entry point's first call on it until the
 * process ends; its device address is looked up once per device.
 *   Arguments, layouts, ownership and results are those of diffattn_decode (same
 *   kernels, bitwise the same output). The current device must be the one that owns
 *   the pointers and the stream.
 *   Limit: diffattn_workspace_bytes(DIFFATTN_OP_DECODE, p) must not exceed
 *   DIFFATTN_DECODE_SCRATCH_BYTES, else DIFFATTN_E_SCRATCH (checked on the host before
 *   any HIP call). That holds, for example, 64 sequences x 16 heads with a cache of 8192.
 *   Every call on one device shares that device's array and leaves its partials there:
 *   calls that overlap in time on one device (two streams, two host threads) race and
 *   must be serialised by the caller. Each call writes every partial it reads, so
 *   nothing needs clearing between calls. */
diffattn_status diffattn_decode_noalloc(const diffattn_problem* p, const void* q1,
                                        const void* q2, const void* k1c, const void* k2c,
                                        const void* vc, const int32_t* cache_len,
                                        const diffattn_lambda_state* lam,
                                        const float* rms_weight, void* out, void* stream);

/* Appends one generated token per sequence to its K1/K2/V cache, in place: the write half
 * of an autoregressive serving step, before the decode call that reads the cache whole
 * (priorstack.com, "Multi-Head Latent Attention: Scaling LLM Serving Throughput via
 * Low-Rank KV Compression", section "The Memory Wall: Why the KV Cache Constrains LLM
 * Serving": the cache grows by one token per generated token).
 * For every sequence b with n = cache_len[b] (a negative value counts as 0) below L, the
 * rows k1_new[b, h], k2_new[b, h] and v_new[b, h] of every head h are copied to cache row
 * n, and cache_len[b] becomes n + 1 on the device, so a following diffattn_decode sees the
 * new token at position len - 1. A sequence whose cache is full (n >= L) is left unchanged,
 * its length included; the caller detects that from cache_len.
 *   k1_new, k2_new [B, H, d];  v_new [B, H, 2d]           (inputs)
 *   k1c, k2c [B, H, L, d]; vc [B, H, L, 2d] (p->seqlen = L) (updated in place)
 *   cache_len  device int32 [B], required                  (updated in place)
 * bf16 only, d = 64, 16-byte aligned rows and caches, 4-byte aligned cache_len; the new
 * rows must not overlap the caches or cache_len, nor the caches each other (E_ARG).
 * The caller owns every buffer; no workspace. */
diffattn_status diffattn_cache_append(const diffattn_problem* p, const void* k1_new,
                                      const void* k2_new, const void* v_new, void* k1c,
                                      void* k2c, void* vc, int32_t* cache_len, void* stream);

/* The input projection of multi-head DiffAttn: the embeddings X are projected into two
 * queries, two keys and one value per head (intoai.pub, "Moving On To The Differential
 * Transformer": X times W_Q, W_K, W_V, with Q and K split into two groups; "Differential
 * Attention With Multiple Heads": separate projections per head). One bf16 MFMA GEMM,
 * float32 accumulation, outputs rounded once to bf16 (nearest even).
 *   x       [B, N, d_model] (p->batch, p->seqlen)
 *   w_qkv   [(H + 2 Hkv) 2d, d_model], the fused weight in the [out_features, in_features]
 *           layout: rows [0, H 2d) are W_Q, then Hkv 2d rows of W_K, then Hkv 2d of W_V
 *           (Hkv = p->kv_heads, or H). Row h 2d + j d + c of W_Q gives channel c of
 *           Q_(j+1) in head h (j = 0, 1), likewise for W_K; row h 2d + c of W_V gives
 *           channel c of V in head h.
 *   q1, q2 [B, H, N, d]; k1, k2 [B, Hkv, N, d]; v [B, Hkv, N, 2d]   (outputs, the
 *           forward's input layout)
 * bf16 only; d a multiple of 32 (at most 256); d_model a multiple of 64 in [64, 65536];
 * H 2d <= 65536; B N < 2^31. Pointers 16-byte aligned; outputs must not overlap each
 * other or the inputs (E_ARG). No workspace. */
diffattn_status diffattn_qkv_proj(const diffattn_problem* p, int64_t d_model, const void* x,
                                  const void* w_qkv, void* q1, void* q2, void* k1, void* k2,
                                  void* v, void* stream);

/* The output projection: the per-head outputs, concatenated over heads along the channel
 * dimension, times W_O back to the model width (intoai.pub, "Differential Attention With
 * Multiple Heads"; pt.news.hada.io, "Estrutura multi-head e arquitetura completa").
 *   attn    [B, N, H 2d]: diffattn_fwd's output in the token-major layout
 *           (p->out_layout = DIFFATTN_LAYOUT_BNH)
 *   w_o     [d_model, H 2d] ([out_features, in_features])
 *   y       [B, N, d_model] (output)
 * bf16 only, float32 accumulation; the same shape limits as diffattn_qkv_proj. */
diffattn_status diffattn_out_proj(const diffattn_problem* p, int64_t d_model, const void* attn,
                                  const void* w_o, void* y, void* stream);

/* Backward of the forward above for the loss sum(Y * dout), recomputing A1 and A2 from
 * the saved log-sum-exps. The pages print no gradient formulas; these follow from the
 * forward by the chain rule:
 *   G   = dL/dO = r g - O r^3 rowsum(g O) / 2d,  g = (1 - lambda_init) w dout, r = rstd
 *   dV  = (A1 - lambda A2)^T G;   dS1 = A1 (G V^T - D1);   dS2 = -lambda A2 (G V^T - D2)
 *   D_k = rowsum(G * O_k);  dQ_k = dS_k K_k / sqrt(d);  dK_k = dS_k^T Q_k / sqrt(d)
 *   dw_h    = (1 - lambda_init) sum over (b, i) of dout * O r   (RMSNorm weight, per head)
 *   dlambda = -sum over (b, h, i) of D2;  dlq1 = dlambda e^a lk1;  dlk1 = dlambda e^a lq1;
 *   dlq2 = -dlambda e^b lk2;  dlk2 = -dlambda e^b lq2   (lambda_init gets no gradient)
 *   inputs  q1..v, lq1..lk2 (device float32 [d]), lam, rms_weight (or NULL), saved (from
 *           diffattn_fwd in training mode on the same inputs), dout [B, H, N, 2d]
 *   outputs dq1, dq2 [B, H, N, d]; dk1, dk2 [B, Hkv, N, d]; dv [B, Hkv, N, 2d] (all
 *           p->dtype; Hkv = p->kv_heads or H, and k1, k2, v have Hkv heads too);
 *           d_attn [B, H, N, 2d] float32 = G, the gradient at the RMSNorm input;
 *           dlq1, dlk1, dlq2, dlk2 device float32 [d];
 *           d_rms_weight device float32 [H, 2d] (the RMSNorm weight gradient), or NULL to
 *           skip it; computed whether or not rms_weight is NULL (then for w = 1)
 *   dout    in p->out_layout (the layout the forward wrote Y in)
 *   workspace at least diffattn_workspace_bytes(OP_BWD, p) bytes
 * bf16 only, d = 64, 16-byte aligned pointers. */
diffattn_status diffattn_bwd(const diffattn_problem* p, const void* q1, const void* q2,
                             const void* k1, const void* k2, const void* v, const float* lq1,
                             const float* lk1, const float* lq2, const float* lk2,
                             const diffattn_lambda_state* lam, const float* rms_weight,
                             const diffattn_saved* saved, const void* dout, void* dq1,
                             void* dq2, void* dk1, void* dk2, void* dv, float* d_attn,
                             float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                             float* d_rms_weight, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Workspace bytes an operation needs for problem p (0 if none; also 0 for an invalid p). */
size_t diffattn_workspace_bytes(diffattn_op op, const diffattn_problem* p);

/* Static human-readable name of a status code. */
const char* diffattn_status_string(diffattn_status s);

/* hipError_t of the last DIFFATTN_E_HIP returned on the calling thread (0 if none). */
int diffattn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
