/*
 * dex.h - C ABI of the Depth Exploration Decoding (DEX) lattice-step library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is "Depth Exploration for LLM Decoding" (arXiv 2606.29223):
 * a decoder of L layers is cut into N stages at the exploration depths
 * X = {d_0 < ... < d_{N-1} = L} (Section 2.3, Definition 4); each stage is a
 * depth explorer (Section 3.1). One call of dex_step runs one round of
 * Algorithm 1 for every live sequence: every node of the depth-position
 * lattice created in that round runs its stage (expand), every new node is
 * decoded by the shared final norm and LM head with depth-coupled sampling
 * (Section 3.3, Algorithm 2), and a sequence whose anchor path reached the
 * final depth commits exactly the final-depth token and collapses the lattice
 * onto the shallowest matching branch (Section 3.2, "Commit process" and
 * "Finite-state control and collapse").
 *
 * Conventions
 *  - Every function returns DEX_OK (0) or a negative dex_status. No exception
 *    crosses the ABI. dex_last_error gives a message for the last failure.
 *  - Device pointers are HIP device addresses on the current device. Host
 *    pointers are ordinary process memory.
 *  - Weight tensors are row-major [out_features][in_features] in the model's
 *    storage type (float for DEX_DTYPE_F32, bfloat16 bits for
 *    DEX_DTYPE_BF16). The caller owns them; dex_create copies them into its
 *    own packed layout inside the workspace, after which the caller may free
 *    them.
 *  - The workspace (size from dex_workspace_bytes) is a caller-owned device
 *    buffer that the context uses until dex_destroy. It holds the K/V cache:
 *    fp16 values for DEX_DTYPE_BF16 models (2 bytes each), bfloat16
 *    (hi, lo) pairs for DEX_DTYPE_F32 models (4 bytes each).
 *  - A context is bound to one HIP stream (passed as void*, a hipStream_t) and
 *    is not thread-safe. Calls that compute enqueue on that stream; dex_step,
 *    dex_ar_step and dex_prefill synchronise it before returning.
 *  - After DEX_EHIP the context is poisoned: only dex_destroy and
 *    dex_last_error are accepted.
 */
#ifndef DEX_H_
#define DEX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DEX_OK = 0,
  DEX_EINVAL = -1, /* invalid argument: shapes, exploration set, tokens, sizes */
  DEX_ENOSPC = -2, /* workspace or output buffer too small, context too long */
  DEX_ESTATE = -3, /* call not valid in the current state (no prefill, all done, mixed modes) */
  DEX_EHIP = -4    /* a HIP runtime call failed; the context is poisoned */
} dex_status;

typedef enum { DEX_DTYPE_F32 = 0, DEX_DTYPE_BF16 = 1 } dex_dtype;
typedef enum { DEX_GREEDY = 0, DEX_SAMPLE = 1 } dex_mode;

/* Decoder shape: pre-RMSNorm layers with rotary attention (rotate-half pairs
 * (i, i + head_dim/2), angle position * rope_base^(-2i/head_dim)) and a SwiGLU
 * feed-forward block; the same final norm and LM head decode every depth
 * (Section 3.4 and Appendix C.2 of the paper). n_heads must be a multiple of
 * n_kv_heads; head_dim is 64 or 128. */
typedef struct {
  int32_t n_layers;   /* L */
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t d_ffn;
  int32_t vocab;
  float rope_base;
  float rms_eps;
  int32_t tied_head;  /* 1: the LM head is the embedding matrix */
  int32_t dtype;      /* dex_dtype: storage of weights and KV */
  int32_t adapter_hidden; /* m of the inducing adapters at the non-final exploration depths
                             ("Depth Exploration for LLM Decoding", Section 3.4, Appendix C.2);
                             0: no adapters. Multiple of 32 (bf16) or 16 (fp32). */
} dex_model_config;

/* Device pointers, row-major [out][in]. Per-layer entries are host arrays of
 * n_layers device pointers. Norm weights are vectors of d_model. */
typedef struct {
  const void* tok_embed;           /* [vocab][d_model] */
  const void* const* attn_norm;    /* [L] -> [d_model] */
  const void* const* wq;           /* [L] -> [n_heads*head_dim][d_model] */
  const void* const* wk;           /* [L] -> [n_kv_heads*head_dim][d_model] */
  const void* const* wv;           /* [L] -> [n_kv_heads*head_dim][d_model] */
  const void* const* wo;           /* [L] -> [d_model][n_heads*head_dim] */
  const void* const* ffn_norm;     /* [L] -> [d_model] */
  const void* const* w_gate;       /* [L] -> [d_ffn][d_model] */
  const void* const* w_up;         /* [L] -> [d_ffn][d_model] */
  const void* const* w_down;       /* [L] -> [d_model][d_ffn] */
  const void* final_norm;          /* [d_model] */
  const void* lm_head;             /* [vocab][d_model]; ignored when tied_head */
  /* Inducing adapters, read when adapter_hidden > 0: host arrays of N-1 device
   * pointers, one per non-final explorer k, storage dtype. A proposal of
   * explorer k is decoded from h + alpha_k (w2_k SiLU(w1_k (RMSNorm(h) * norm_k)
   * + b1_k) + b2_k); the residual stream and the final explorer are unchanged. */
  const void* const* adapter_w1;    /* [N-1] -> [m][d_model] */
  const void* const* adapter_b1;    /* [N-1] -> [m] */
  const void* const* adapter_w2;    /* [N-1] -> [d_model][m] */
  const void* const* adapter_b2;    /* [N-1] -> [d_model] */
  const void* const* adapter_norm;  /* [N-1] -> [d_model] */
  const float* adapter_alpha;       /* host [N-1] */
} dex_weights;

typedef struct {
  int32_t mode;            /* dex_mode */
  float temperature;       /* sampling: the rule takes argmax(z / temperature + g) */
  int32_t decs;            /* 1: depth-coupled sampling masks shallower candidates of the slot chain */
  int32_t max_batch;       /* sequences per context, 1..64 */
  int32_t max_context;     /* prompt + generated tokens per sequence */
  int32_t max_new_tokens;  /* T: a sequence stops after T commits */
  /* Sampling only: device float32 Gumbel(0,1) rows [max_batch][gumbel_rows][vocab];
   * row (b, j) is the noise for target position prompt_len_b + j, shared by
   * every node predicting that position (one row per slot, shared across
   * depths: Appendix C.1). Needs gumbel_rows >= max_new_tokens + N - 1 and a
   * 16-byte aligned pointer (the exit head reads the rows four floats at a time). */
  const float* gumbel;
  int32_t gumbel_rows;
  int32_t debug;           /* bit 0: keep the final-depth logits of each sequence's last commit;
                              bit 1: launch every round eagerly (no HIP-graph replay). By default a
                              round whose plan (FSM states, commit flags, attention chunk count,
                              explore-chunk slots) was seen before is captured once into a HIP graph
                              and replayed;
                              bit 2: grouped attention blocks always run whole spans of key
                              positions (by default a launch does so only when that still fills
                              the GPU). The results are the same bits either way; the bit lets
                              small inputs exercise the span path. */
  int32_t single_exit;     /* 1: the single-exit ablation ("Depth Exploration for LLM Decoding",
                              Section 4, Figure 4 right-top): only explorers 0 and N-1 exit; the
                              intermediate ones run without proposing, so only explorer-0 nodes
                              spawn position children and a commit keeps branch 0 or N-1. The
                              round at state q has one row per explorer 0..q. 0: full DEX. */
  int32_t branch_cap;      /* Pruned lattice (the sparse lattice the same paper names as future work,
                              Appendix E, "Expansion growth and overhead"; the policy is this
                              library's): only nodes of explorers
                              j < branch_cap spawn position children, so a round creates only the
                              nodes whose root path has no run of branch_cap or more depth moves
                              before a position move. Depth children are never pruned and the
                              commit rule is unchanged, so the output is still the plain model's;
                              a commit with branch b >= branch_cap keeps nothing and the next tree
                              starts fresh. 0 (or N): no pruning. Range 0..N; not combined with
                              single_exit (which already implies the cap-1 node set). */
} dex_options;

/* One committed token (Algorithm 1, validate_and_commit). */
typedef struct {
  int32_t seq;       /* sequence index */
  int32_t position;  /* absolute position of the token */
  int32_t token;     /* y = u_{N-1}, the final-depth reference */
  int32_t branch;    /* b: shallowest anchor branch whose candidate equals y (N-1 if none) */
  int32_t layers;    /* d_b: layers the token consumed on its critical path */
} dex_commit;

typedef struct dex_ctx dex_ctx;

/* Device bytes needed by dex_create for this shape, exploration set and
 * options. Pure: touches no device. X (host, n_x entries, 1 <= n_x <= 10)
 * must be strictly increasing with X[0] >= 1 and X[n_x-1] == cfg->n_layers
 * (Definition 4 of the paper); the stages between consecutive depths may have
 * unequal lengths. Errors: DEX_EINVAL. */
int dex_workspace_bytes(const dex_model_config* cfg, const int32_t* X, int32_t n_x,
                        const dex_options* opt, size_t* out_bytes);

/* Validates the configuration, packs the weights into the workspace and
 * builds the RoPE table. L must equal cfg->n_layers. Enqueues on `stream`
 * and synchronises it. Errors: DEX_EINVAL (bad shapes or X, null pointers),
 * DEX_ENOSPC (ws_bytes too small), DEX_EHIP. On success *out owns a host
 * struct released by dex_destroy. */
int dex_create(const dex_model_config* cfg, const dex_weights* w, const int32_t* X, int32_t n_x,
               int32_t L, const dex_options* opt, void* d_workspace, size_t ws_bytes, void* stream,
               dex_ctx** out);

/* Algorithm 1's initialisation ("Depth Exploration for LLM Decoding",
 * Section 3.1, Algorithm 1, the init step before the exploration loop): resets
 * every sequence and runs the prompts through all layers. Positions 0..len-2
 * of each prompt fill the committed KV cache; the last prompt token becomes
 * the anchor of the first cycle (FSM state 0, Section 3.2, "Finite-state
 * control and collapse"). `tokens` holds the
 * prompts back to back (host int32), `lens` their lengths (host, n_seqs).
 * Errors: DEX_EINVAL (n_seqs outside 1..max_batch, len < 1, token outside
 * [0, vocab)), DEX_ENOSPC (len + max_new_tokens > max_context), DEX_EHIP. */
int dex_prefill(dex_ctx* ctx, int32_t n_seqs, const int32_t* tokens, const int32_t* lens);

/* One lattice round for every live sequence (expand, decode with DECS,
 * commit and collapse where the anchor path reached the final explorer).
 * Writes at most one record per sequence into `out` (host, capacity cap) and
 * their count into *n_out. Errors: DEX_ESTATE (no prefill, every sequence
 * done, or the context was stepped with dex_ar_step), DEX_ENOSPC (cap < live
 * sequences), DEX_EHIP. */
int dex_step(dex_ctx* ctx, dex_commit* out, int32_t cap, int32_t* n_out);

/* Plain autoregressive decoding with the same kernels: one full-depth token
 * per live sequence per call (branch = 0, layers = L). DEX is lossless: every
 * committed token is the final-depth reference, so the committed stream is
 * the plain model's ("Depth Exploration for LLM Decoding", Section 3.2,
 * "Commit process"; for sampling, the shared noise of Appendix C.1). This call
 * computes that plain stream on the same batch-invariant kernels, the
 * reference DEX must reproduce bit for bit. Errors as dex_step (DEX_ESTATE if the context
 * was stepped with dex_step since the last prefill). */
int dex_ar_step(dex_ctx* ctx, dex_commit* out, int32_t cap, int32_t* n_out);

/* dex_step for callers that cannot allocate device memory (tight serving
 * loops, harnesses that forbid hipMalloc): the same round as dex_step, with
 * the same records and the same bits, launched eagerly (no HIP graph is
 * captured or instantiated, no timing events are created) and with the
 * round's scratch (row and attention plans, attention and GEMM partial
 * results, exit-head tile summaries) in a static device array of the library
 * instead of the workspace's scratch regions. The array is 64 MiB per GPU,
 * held until the process ends; contexts on one GPU share it, so calls that
 * overlap on one GPU (from any context or thread) race. Nothing in it carries
 * from one call to the next. Can be mixed with dex_step on the same context.
 * Errors as dex_step, plus DEX_ENOSPC when the context's per-round scratch
 * exceeds 64 MiB (it grows with max_batch * 2^(N-1) rows, the vocabulary and
 * max_context: small models and batches fit). */
int dex_step_noalloc(dex_ctx* ctx, dex_commit* out, int32_t cap, int32_t* n_out);

/* For sequence `seq`'s last commit: the anchor-path candidates u_0..u_{N-1}
 * and their top-1 minus top-2 margins (host arrays of N, either may be NULL),
 * and, when options.debug bit 0 is set, the final-depth logits (host array of
 * vocab floats, may be NULL). For dex_ar_step only u[0] and margins[0] are
 * set. Errors: DEX_EINVAL (seq out of range, logits requested without debug),
 * DEX_ESTATE (no commit yet), DEX_EHIP. */
int dex_debug_anchor(dex_ctx* ctx, int32_t seq, int32_t* u, float* margins, float* logits);

/* Per-step counters of the last dex_step / dex_ar_step: rows run at each
 * explorer (host array of N int32, may be NULL) and the total row count. */
int dex_last_step_rows(const dex_ctx* ctx, int32_t* rows_per_stage, int32_t* total_rows);

/* Kernel classes timed by dex_profile. */
typedef enum {
  DEX_PROF_GEMM = 0,     /* stage-batched layer GEMMs (QKV with RMSNorm, RoPE, K/V write; O with
                            residual; gate/up with RMSNorm and SwiGLU; down with residual) */
  DEX_PROF_ATTN = 1,     /* lattice attention and its split-KV combine */
  DEX_PROF_HEAD = 2,     /* exit head: LM-head GEMM with DECS/Gumbel epilogue, argmax reduce */
  DEX_PROF_ROWOPS = 3,   /* standalone per-row kernels (none at present: RMSNorm, RoPE with the
                            K/V write and the embedding gather run fused in other classes) */
  DEX_PROF_LATTICE = 4,  /* schedule with embedding, commit/collapse, KV promotion */
  DEX_PROF_NCLASS = 5
} dex_prof_class;

typedef struct {
  double ms;        /* summed GPU time between HIP events around the class's launches */
  int64_t launches; /* kernel launches timed */
  double bytes;     /* algorithmic HBM bytes of those launches (each weight matrix, KV entry,
                       activation row read or written once; KV values at their stored size,
                       2 bytes for DEX_DTYPE_BF16 models, 4 for DEX_DTYPE_F32) */
  double flops;     /* algorithmic floating-point operations */
} dex_kernel_stats;

/* Per-class timing of later dex_step / dex_ar_step calls with HIP events on
 * the context's stream. enable = 1 turns it on, 0 off. While it is on, rounds
 * run eagerly (no graph replay): event records inside a replayed graph do not
 * bracket the kernels between them. When out is not NULL
 * the stats gathered since the last call are copied into out[0..n-1]
 * (n <= DEX_PROF_NCLASS) and reset. Errors: DEX_EINVAL (bad n), DEX_EHIP. */
int dex_profile(dex_ctx* ctx, int32_t enable, dex_kernel_stats* out, int32_t n);

void dex_destroy(dex_ctx* ctx);

/* Message for the last failure on ctx (or of the last failed dex_create when
 * ctx is NULL). Owned by the library; valid until the next call. */
const char* dex_last_error(const dex_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* DEX_H_ */
