/*
 * rlt.h — C ABI of librlt.so: Recurrent Looped Transformer (RLT) exact replay on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as printed):
 *   [FI] feinterview: "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer"
 *   [DS] deepsonar:   "技术拆解 009｜RLT：给 Transformer 接一条时间回路，潜变量推理与「无限时间深度」的真面目"
 *   [AL] alphalab:    "Recurrent Looped Transformer：路徑變深，就真的更會推理嗎？（2026）"
 *
 * The library computes one sequence family in three calls that follow the pages'
 * state contract ([FI] decoder-state paragraph; [DS] §2.3, §2.5):
 *   rlt_encoder_forward  causal encoder over known tokens, token-parallel: e_t and
 *                        the key/value memory M_{<=t} ([FI] architecture paragraph).
 *   rlt_decoder_replay   the recurrent decoder, stepping t in order, batched over
 *                        B independent sequences ([FI] model-hardware co-design).
 *   rlt_decoder_step     incremental generation: encode one token per sequence,
 *                        one transition, logits ([DS] §2.5).
 * Exact current-policy replay ([FI] model-RL co-design; [AL] §四) is
 *   rlt_state_reset + rlt_encoder_forward(T) + rlt_decoder_replay(T) + rlt_logits.
 * There is no prompt/response argument anywhere: the split never touches the state
 * (Proposition 3.1 on [FI]; [AL] §一).
 *
 * Conventions
 *  - Every pointer marked "device" is device memory owned by the caller; the
 *    library never allocates or frees device memory.  It keeps small host handles.
 *    Such a pointer must be known to HIP (hipMalloc'd, managed or pinned host memory);
 *    plain pageable host memory is refused with RLT_ERR_INVALID before anything is
 *    enqueued, since a kernel reading it would fault.
 *  - Every call that takes a stream only enqueues work on that stream (a
 *    hipStream_t passed as void*; NULL = the default stream) and returns before the
 *    work runs.  Host-side argument and ordering checks happen before anything is
 *    enqueued, so a non-zero return means nothing was enqueued.
 *  - A model is immutable between rlt_model_update_weights calls and may be shared by
 *    states on several streams; one state must be used by one stream at a time.
 *  - Return value: RLT_OK (0) or a negative RLT_ERR_* code; rlt_last_error() gives a
 *    thread-local message for the last failure.  No C++ exception crosses the ABI.
 *  - Matrices are [out, in] row-major (y = W x).
 */
#ifndef RLT_H
#define RLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RLT_OK 0
#define RLT_ERR_INVALID (-1)       /* bad argument or configuration value            */
#define RLT_ERR_UNSUPPORTED (-2)   /* configuration outside what the kernels support */
#define RLT_ERR_CAPACITY (-3)      /* position would exceed the state's T_max        */
#define RLT_ERR_ORDER (-4)         /* decoder would run ahead of the encoder, etc.   */
#define RLT_ERR_STALE_STATE (-5)   /* state built under another weights version      */
#define RLT_ERR_NO_ENC_CACHE (-6)  /* incremental encoding without an encoder cache  */
#define RLT_ERR_HIP (-7)           /* a HIP runtime call failed                      */

#define RLT_FFN_GELU 0             /* W_2 gelu(W_1 h), exact erf GELU                */
#define RLT_FFN_SWIGLU 1           /* W_down(silu(W_gate h) * W_up h)                */
#define RLT_DTYPE_FP32 0           /* all storage and arithmetic fp32                */
#define RLT_DTYPE_BF16 1           /* bf16 storage of weights, e, M, window caches and
                                      matrix-product operands; fp32 accumulation,
                                      residual stream, s_t, softmax and logits      */

typedef struct rlt_model rlt_model;
typedef struct rlt_state rlt_state;

/* Model shape.  L = n_layers is both L_E and L_D: encoder layer l and decoder layer l
 * share W_Q, W_K, W_V, W_O and the FFN ([FI] tied-configuration paragraph; [DS] §2.1).
 * window W >= 1 counts the current token, so W-1 past entries are cached per decoder
 * layer ([DS] §2.2; [FI] decoder-state paragraph).  mem_groups G is 1 (one memory for
 * all decoder layers) or n_layers (one per layer) ([FI] architecture paragraph); any
 * other value is RLT_ERR_UNSUPPORTED.  Kernel limits (RLT_ERR_UNSUPPORTED otherwise):
 * d_model % 64 == 0, ffn_dim % 64 == 0, head_dim = d_model / n_heads in {16,32,64,128}. */
typedef struct {
  int32_t vocab;
  int32_t d_model;
  int32_t n_heads;
  int32_t n_layers;
  int32_t ffn_dim;
  int32_t ffn_kind;    /* RLT_FFN_*   */
  int32_t window;      /* W >= 1      */
  int32_t mem_groups;  /* 1 or L      */
  int32_t dtype;       /* RLT_DTYPE_* */
  float norm_eps;      /* RMSNorm epsilon, > 0 */
} rlt_config;

/* ---- canonical flat weight layout ------------------------------------------------
 * rlt_model_create reads all parameters from ONE fp32 buffer holding the tensors
 * below back to back, in this order, each row-major (per-layer tensors carry a
 * leading L axis, memory projections a leading G axis):
 *   embed [V,d]; w_out [V,d]; s_star [d]; w_ge, w_gs, w_fb [d,d]; b_g [d];
 *   wq, wk, wv, wo [L,d,d];
 *   GELU:   ffn_w1 [L,F,d]; ffn_w2 [L,d,F]
 *   SwiGLU: ffn_gate [L,F,d]; ffn_up [L,F,d]; ffn_down [L,d,F]
 *   wqx, wox [L,d,d]; wkm, wvm [G,d,d];
 *   g_enc_attn, g_enc_ffn [L,d]; g_enc_final [d];
 *   g_dec_self, g_dec_cross, g_dec_ffn [L,d]; g_dec_final [d].
 * rlt_param_info gives each tensor's name, element offset and element count, so a
 * caller can fill the buffer by name. */
int rlt_param_count(const rlt_config* cfg, int32_t* n_tensors, int64_t* total_numel);
int rlt_param_info(const rlt_config* cfg, int32_t index, const char** name,
                   int64_t* offset, int64_t* numel);

/* ---- model: packed weights ----------------------------------------------------------
 * rlt_model_workspace_bytes: bytes of the device workspace that rlt_model_create packs
 * the weights into (bf16 or fp32 per cfg->dtype, kernel-friendly layout).
 * rlt_model_create: validates cfg, packs the canonical fp32 buffer `weights` (device,
 * read only during the enqueued pack kernels) into `workspace` (device, >= the size
 * above, caller-owned, must outlive the model) on `stream`, and returns a host handle.
 * `version` tags every state built from this model ([FI] serving paragraph: a weight
 * update invalidates old states). */
int rlt_model_workspace_bytes(const rlt_config* cfg, size_t* bytes);
int rlt_model_create(const rlt_config* cfg, const float* weights, uint64_t version,
                     void* workspace, size_t workspace_bytes, void* stream, rlt_model** out);
/* Re-packs new weights into the same workspace and sets a new version (must differ
 * from the current one).  States built under the old version then fail every call
 * with RLT_ERR_STALE_STATE until rlt_state_reset. */
int rlt_model_update_weights(rlt_model* model, const float* weights, uint64_t new_version,
                             void* stream);
int rlt_model_get_config(const rlt_model* model, rlt_config* cfg, uint64_t* version);
void rlt_model_release(rlt_model* model);

/* ---- state H_t = (s_t, C^D_t) plus the encoder side ---------------------------------
 * One device blob holds: s [B,d] fp32; the per-layer window caches (ring buffers of
 * W-1 entries); e [B,T_max,d]; the memory keys K^M [G][B][H][T_max][d_h] and values V^M
 * in blocks of 8 positions stored dimension-major, [G][B][H][ceil(T_max/8)][d_h][8] (zeroed
 * by rlt_state_init); optionally the encoder key/value cache (needed to encode
 * incrementally); scratch; an error flag.  The blob layout is internal: use
 * rlt_state_load/read_encoder_outputs to move encoder outputs in and out.
 * keep_encoder_cache = 0 allows only one rlt_encoder_forward call per reset (the whole
 * known sequence at once), which is what exact replay needs.
 * rlt_state_init sets H_0 = (s*, empty caches), t_enc = t_dec = 0 ([FI] decoder-state
 * paragraph: initialised once before BOS with the learned start state and empty caches). */
int rlt_state_bytes(const rlt_model* model, int32_t batch, int32_t t_max,
                    int32_t keep_encoder_cache, size_t* bytes);
int rlt_state_init(const rlt_model* model, void* buffer, size_t buffer_bytes, int32_t batch,
                   int32_t t_max, int32_t keep_encoder_cache, void* stream, rlt_state** out);
/* Back to H_0 under the model's current weights and version; exact replay always starts
 * here ([FI] model-RL co-design: rebuild everything from the sequence start). */
int rlt_state_reset(const rlt_model* model, rlt_state* state, void* stream);
void rlt_state_release(rlt_state* state);

/* Host-side counters (no device access): positions encoded, positions decoded, version. */
int rlt_state_position(const rlt_state* state, int32_t* t_enc, int32_t* t_dec,
                       uint64_t* version);
/* Reads the device error flag (bit 0: a token id outside [0, V) was seen and replaced
 * by 0).  Synchronises `stream` first.  Writes 0 when no device error occurred. */
int rlt_state_device_error(rlt_state* state, void* stream, int32_t* flags);

/* ---- prefix snapshots ([FI] serving paragraph: a conversation's state after a prefix is kept
 * and later continued; it is only valid under the weights version it was built with) --------
 * A snapshot is a HOST buffer: a header (magic "RLTSNAP1", format 1, the model configuration,
 * the weights version, B, t_enc, t_dec, whether the encoder K/V cache is included, and the
 * window convention: the window counts the current token and the ring of W-1 entries keeps
 * position p in slot p mod (W-1)), followed by the state regions packed to the positions in
 * use: device flags, s [B,d], the window rings, e and the memory keys/values for positions
 * < t_enc, and the encoder K/V cache for them when the state keeps one.
 * rlt_state_snapshot_bytes: size of a snapshot of the state at its current position.
 * rlt_state_save: enqueues the copies into `dst` (host memory, >= that size; pinned memory
 *   makes the copies asynchronous) on `stream`; the caller synchronises before reading it.
 * rlt_state_restore: checks the header against the model and the target state, then resets
 *   the target and enqueues the copies from `src` (host memory that stays valid until the
 *   stream reaches them).  The target needs the same configuration and batch, t_max >= the
 *   snapshot's t_enc (a prefix can be restored into a longer state), and an encoder cache in
 *   the snapshot if it keeps one.  Errors: RLT_ERR_INVALID (bad header, size, configuration or
 *   batch), RLT_ERR_STALE_STATE (weights version differs from the model's), RLT_ERR_CAPACITY,
 *   RLT_ERR_NO_ENC_CACHE; nothing is enqueued on error. */
int rlt_state_snapshot_bytes(const rlt_state* state, size_t* bytes);
int rlt_state_save(const rlt_model* model, const rlt_state* state, void* dst, size_t dst_bytes,
                   void* stream);
int rlt_state_restore(const rlt_model* model, rlt_state* state, const void* src, size_t src_bytes,
                      void* stream);

/* ---- the hot path --------------------------------------------------------------------
 * rlt_encoder_forward: tokens (device int32 [B, n], row stride n) are positions
 * t_enc .. t_enc+n-1 of every sequence.  Runs the causal encoder over them (each new
 * position attends to every earlier one), writes e and the G memory rows, advances
 * t_enc by n.  Errors: RLT_ERR_CAPACITY if t_enc+n > T_max; RLT_ERR_NO_ENC_CACHE if
 * t_enc > 0 and the state keeps no encoder cache; RLT_ERR_INVALID if n < 1. */
int rlt_encoder_forward(const rlt_model* model, rlt_state* state, const int32_t* tokens,
                        int32_t n, void* stream);

/* rlt_decoder_replay: n recurrent transitions at positions t_dec+1 .. t_dec+n for all B
 * sequences, in order, inside the library (no host round trip per step).  Each step:
 * gated merge of e_t with s_{t-1}; L blocks of sliding-window self-attention over the
 * layer's cache plus the current entry, cross-attention to memory entries 1..t, tied
 * FFN; final RMSNorm gives s_t ([FI] decoder-state paragraph; [DS] §2.2, §2.4).
 * s_out (device fp32 [B, n, d], row stride n*d per sequence) receives s_t for every
 * step, or is NULL.  Requires t_dec + n <= t_enc (RLT_ERR_ORDER otherwise).  Advances
 * t_dec by n.  Each position is consumed exactly once; there is no rewind. */
int rlt_decoder_replay(const rlt_model* model, rlt_state* state, int32_t n, float* s_out,
                       void* stream);

/* rlt_decoder_replay_noalloc: rlt_decoder_replay for callers that cannot allocate device
 * memory at call time (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, ordering rules, errors and results as
 * rlt_decoder_replay; it allocates nothing (no hipMalloc, no allocating library call).  The
 * batched decoder's per-step scratch (residual stream, projections, fragment-major product
 * operands, norm partial sums, attention partials and their arrival counters, and the split-K
 * partials of the tiled products) lives in a library-owned static device array of
 * 64 MiB, one per GPU, held until the process ends, instead of the state's scratch region.
 * RLT_ERR_UNSUPPORTED when the batch and t_max need more scratch than that.  Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents: calls that overlap on one
 * GPU (two streams, or two threads) race and must be serialised by the caller.  The arrival
 * counters are cleared by a fill kernel at the start of each call. */
int rlt_decoder_replay_noalloc(const rlt_model* model, rlt_state* state, int32_t n, float* s_out,
                               void* stream);

/* rlt_decoder_step: incremental generation ([DS] §2.5): equals
 * rlt_encoder_forward(n = 1) + rlt_decoder_replay(n = 1) + rlt_logits on s_t.
 * tokens: device int32 [B]; s_out: device fp32 [B, d] or NULL; logits: device fp32
 * [B, V] or NULL.  Needs keep_encoder_cache unless t_enc == 0. */
int rlt_decoder_step(const rlt_model* model, rlt_state* state, const int32_t* tokens,
                     float* s_out, float* logits, void* stream);

/* rlt_logits: logits = W_out s for N state rows (next-token distribution read from s_t,
 * [FI] decoder-state paragraph), token-parallel, off the recurrent loop.
 * s: device fp32 [N, d]; logits: device fp32 [N, V]. */
int rlt_logits(const rlt_model* model, const float* s, int64_t n_rows, float* logits,
               void* stream);

/* rlt_score_actions: scores actions under the current policy for RL ([FI] model-RL co-design
 * paragraph: the trainer rebuilds every state under the current weights, scores each action,
 * and the behaviour log-probability recorded by the sampler is the denominator of the
 * importance ratio):
 *   logp_i  = log softmax(W_out s_i / temperature)[a_i]
 *   ratio_i = exp(logp_i - behaviour_logp_i)
 * computed without writing the [N, V] logits (a running log-sum-exp over vocabulary tiles).
 * s: device fp32 [N, d] (rows of s_t, e.g. the response positions of a replay);
 * actions: device int32 [N], ids in [0, V) (an id outside gives logp = NaN);
 * temperature > 0 (1 = the plain softmax); behaviour_logp: device fp32 [N] or NULL;
 * logp_out: device fp32 [N]; ratio_out: device fp32 [N] or NULL (needs behaviour_logp).
 * Errors: RLT_ERR_INVALID for NULL required pointers, n_rows out of range, temperature <= 0
 * or ratio_out without behaviour_logp. */
/* ---- sampling ([FI] model-RL co-design paragraph: the sampler records the log-probability of
 * the distribution it actually drew from, which the trainer's ratio divides by) ----------
 * Row r with uniform u_r in [0, 1) (the caller's random numbers, so a draw is a deterministic
 * function of its inputs):
 *   z = logits_r / temperature; candidates ranked by larger z, then smaller token id;
 *   top_k > 0 (and < V) keeps the first top_k of that ranking;
 *   top_p < 1 then keeps the shortest prefix of the survivors whose mass, renormalised over
 *   them, reaches top_p;
 *   the kept ids in increasing order split [0, 1) in proportion to exp(z); the first id whose
 *   cumulative share exceeds u_r is drawn (u_r at or past the top edge draws the last kept id);
 *   logp_r = z[drawn] - log sum_kept exp(z).
 * The decisions are taken in fp32.  With top-p and no top-k at 4096 < V (V a multiple of 4)
 * the ranking is by the fp32 probability exp(z - max z), so logits whose probabilities round
 * to the same fp32 value rank as ties, by id; the other settings rank by z itself.
 * temperature > 0; top_k >= 0 (0 = no top-k); 0 < top_p <= 1 (1 = no top-p). */
typedef struct rlt_sampling {
  float temperature;
  int32_t top_k;
  float top_p;
} rlt_sampling;

/* rlt_sample_tokens: one draw per row.  logits: device fp32 [n_rows, vocab], 1 <= vocab <= 32768;
 * uniforms: device fp32 [n_rows]; tokens_out: device int32 [n_rows]; logp_out: device fp32
 * [n_rows].  Errors: RLT_ERR_INVALID for NULL pointers, n_rows < 1 or parameters out of range;
 * RLT_ERR_UNSUPPORTED for vocab > 32768. */
int rlt_sample_tokens(const float* logits, int64_t n_rows, int32_t vocab, const rlt_sampling* params,
                      const float* uniforms, int32_t* tokens_out, float* logp_out, void* stream);

/* rlt_decoder_step_sample: rlt_decoder_step (logits required, device fp32 [B, V]) followed by
 * rlt_sample_tokens on its logits: next_tokens (device int32 [B]) and behaviour_logp (device
 * fp32 [B]) are the draws for position t+1.  All checks of both calls run before anything is
 * enqueued. */
int rlt_decoder_step_sample(const rlt_model* model, rlt_state* state, const int32_t* tokens,
                            const rlt_sampling* params, const float* uniforms, int32_t* next_tokens,
                            float* behaviour_logp, float* s_out, float* logits, void* stream);

int rlt_score_actions(const rlt_model* model, const float* s, const int32_t* actions, int64_t n_rows,
                      float temperature, const float* behaviour_logp, float* logp_out,
                      float* ratio_out, void* stream);

/* ---- full back-propagation through time --------------------------------------------
 * The exact gradient of the next-token loss of a replay from H_0 ([DS] deepsonar
 * "技术拆解 009｜RLT…" §2.5 and the recipe of §六: teacher forcing, every valid next-token
 * prediction supervised, gradient through the whole recurrent trajectory; §2.6, second
 * point: the gradient runs through s_{t-1}, the decoder window keys/values and the encoder
 * memory, and a detach only approximates it).  For each sequence b:
 *   loss[b] = sum_{t=0}^{T-2} mask[b][t] * CE(W_out s_t, tokens[b][t+1])
 * (mask NULL = all ones; SFT passes zeros off the assistant targets while the state still runs
 * over every position).  grads receives d(sum_b loss[b]) / d(every parameter), s* included, in
 * the canonical layout above (total_numel floats, overwritten).
 *   weights   device fp32, the canonical buffer (the backward computes in fp32 from it; a bf16
 *             model's buffer holds its bf16-representable values)
 *   tokens    device int32 [batch][seq_len]; an id outside [0, vocab) makes every loss NaN
 *   mask      device fp32 [batch][seq_len-1] or NULL
 *   detach    0 for the exact gradient, or an OR of RLT_DETACH_* approximations
 *   grads     device fp32 [total_numel]; loss device fp32 [batch]
 *   workspace device memory of rlt_bptt_workspace_bytes bytes, owned by the caller
 * All work is enqueued on `stream`.  Errors: RLT_ERR_INVALID (NULL or host pointers, bad
 * sizes, workspace too small), RLT_ERR_UNSUPPORTED (d_model > 256, head_dim > 64,
 * ffn_dim > 1024, window > 1024, or a sequence too long for the sweep's per-sequence LDS:
 * about 4 (2 H T + 2 H W + 30 d) bytes must fit 160 KB); nothing is enqueued on error. */
#define RLT_DETACH_S 1          /* s_{t-1} is a constant in the merge for t >= 1 (0-based) */
#define RLT_DETACH_KV 2         /* earlier window entries are constants for later steps   */
#define RLT_DETACH_MEMORY 4     /* memory rows are constants for cross-attention          */
int rlt_bptt_workspace_bytes(const rlt_config* cfg, int32_t batch, int32_t seq_len, size_t* bytes);
int rlt_bptt(const rlt_config* cfg, const float* weights, const int32_t* tokens, const float* mask,
             int32_t batch, int32_t seq_len, int32_t detach, float* grads, float* loss,
             void* workspace, size_t workspace_bytes, void* stream);

/* ---- test hooks (decoder in isolation, encoder outputs) -----------------------------
 * rlt_state_load_encoder_outputs writes externally computed e (device fp32 [B, n, d])
 * and memory rows (device fp32 [G, B, n, d] each for keys and values) for positions
 * t_enc .. t_enc+n-1 (converted to the storage dtype) and advances t_enc, so the
 * decoder can be checked on its own.  rlt_state_read_encoder_outputs copies positions
 * t0 .. t0+n-1 (< t_enc) back out as fp32 in the same layouts. */
int rlt_state_load_encoder_outputs(const rlt_model* model, rlt_state* state, const float* e,
                                   const float* mem_k, const float* mem_v, int32_t n,
                                   void* stream);
int rlt_state_read_encoder_outputs(const rlt_model* model, const rlt_state* state, int32_t t0,
                                   int32_t n, float* e, float* mem_k, float* mem_v,
                                   void* stream);

/* Decoder implementations.  RLT_PATH_PERSISTENT: one persistent workgroup per sequence
 * runs all n steps (d_model in {64, 128}, window entries <= 256).  RLT_PATH_BATCHED: each
 * step is a sequence of B-batched device-wide kernels (any supported shape).  Both compute
 * the same function and keep the same state layout, so calls may alternate between them.
 * rlt_model_set_decoder_path selects one (RLT_PATH_AUTO = persistent when supported, else
 * batched); RLT_ERR_UNSUPPORTED if the persistent path cannot run this shape.
 * rlt_decoder_path reports the path rlt_decoder_replay would take for a state of
 * t_max positions. */
#define RLT_PATH_AUTO 0
#define RLT_PATH_PERSISTENT 1
#define RLT_PATH_BATCHED 2
int rlt_model_set_decoder_path(rlt_model* model, int32_t path);
int rlt_decoder_path(const rlt_model* model, int32_t t_max, int32_t* path);

const char* rlt_last_error(void);
const char* rlt_version_string(void);

#ifdef __cplusplus
}
#endif
#endif /* RLT_H */
