// Internal layouts and kernel launchers of librlt (host side; no torch types).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rlt.h"

namespace rlt {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------------------
// Packed model workspace (byte offsets from the workspace base).
// Matrices are stored in the model's storage type (bf16 or fp32), [rows, K]
// row-major with K contiguous, which is the "B^T" operand of every
// A[M,K] x W[N,K]^T product and the row order of every matrix-vector product.
//   wgate  [d, 2d]: row j = [W_ge[j,:], W_gs[j,:]]   (gate pre-activation from [e; s])
//   wfb    [d, d]
//   layer l block: wqkv [3d, d] (rows W_Q; W_K; W_V), wo [d, d], wqx [d, d],
//                  wox [d, d], ffn_in [F or 2F, d], ffn_out [d, F]
//     SwiGLU ffn_in interleaves gate and up rows in blocks of 16:
//     rows 32j..32j+15 = W_gate rows 16j..16j+15, rows 32j+16..32j+31 = W_up rows.
//   wkvm per group [2d, d]: rows W_KM; W_VM
//   gains (fp32): g_enc_attn[L][d], g_enc_ffn[L][d], g_enc_final[d],
//                 g_dec_self[L][d], g_dec_cross[L][d], g_dec_ffn[L][d], g_dec_final[d]
// ---------------------------------------------------------------------------
struct ModelLayout {
  int D, H, DH, L, F, F2, V, W, G, ffn_kind, dtype;
  float eps;
  size_t esz;  // bytes per stored element
  size_t embed, wout, sstar, wgate, wfb, bg;
  size_t layers, layer_stride;
  size_t l_qkv, l_wo, l_wqx, l_wox, l_fin, l_fout;  // relative to the layer block
  size_t wkvm, group_stride;
  size_t gains;  // fp32 region
  size_t g_enc_attn, g_enc_ffn, g_enc_final, g_dec_self, g_dec_cross, g_dec_ffn, g_dec_final;  // byte offsets
  // fragment-major bf16 copy of w_out read by action scoring (present when has_wout_frag):
  // 16-byte chunk ((cb * D/64 + ks) * 2 + h) * 64 + lane holds
  // w_out[16 cb + lane % 16][64 ks + 16 (lane / 16) + 8 h .. + 8], rows past V zero
  int has_wout_frag;
  size_t wout_frag;
  // fragment-major copies of the decoder's in-loop weights for the weight-streaming products
  // (bf16, d >= 256): the same per-layer block layout as `layers` at frag_layers, and the
  // merge matrix [2D][2D] (gate rows [W_ge | W_gs] and feedback rows [0 | W_fb] interleaved in
  // blocks of 16) at frag_merge
  int has_frag;
  size_t frag_layers, frag_merge;
  size_t total;
};

// Heads that get the fragment-major copy (bf16, d a multiple of 256, d <= 2048).
inline bool score_frag_eligible(int dtype, int D) { return dtype == RLT_DTYPE_BF16 && D % 256 == 0 && D <= 2048; }

// ---------------------------------------------------------------------------
// State blob (byte offsets from the state base).
//   flags   int32[64]            device error flags
//   s       fp32 [B][d]          recurrent output s_t
//   ring_k/v  [L][B][H][W-1][dh] window caches (entry of position p in slot p mod (W-1))
//   e         [B][T_max][d]
//   mem_k     [G][B][H][T_max][dh]
//   mem_v     [G][B][H][T8/8][dh][8], T8 = T_max rounded up to a multiple of 8: keys in blocks
//             of 8, each block stored dimension-major (8 consecutive keys of one dim are
//             contiguous), so a lane can take 8 keys of one dim with one 16-byte load
//   enc_k/v   [L][B][H][T_max][dh]  (only with keep_encoder_cache)
//   encoder scratch for a chunk of Nc tokens: x fp32 [Nc][d], h [Nc][d], qkv [Nc][3d],
//                                              attn [Nc][d], act [Nc][F]
//   decoder scratch (batched path): see dec_batched.hip
// ---------------------------------------------------------------------------
struct StateLayout {
  int B, T, T8, keep, Wm1, Nc;
  size_t flags, s, ring_k, ring_v, e, mem_k, mem_v, enc_k, enc_v;
  size_t x, h, qkv, attn, act;
  size_t dec_scratch, dec_scratch_bytes;
  size_t total;
};

bool compute_model_layout(const rlt_config& c, ModelLayout* m);
void compute_state_layout(const ModelLayout& m, int B, int T, int keep, StateLayout* s);

// ---------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files).  All return hipError_t of the launch.
// ---------------------------------------------------------------------------

// dst rows r (< rows) of a [rows, cols] fp32 source go to dst row map(r):
//   mode 0: r + row_off;  mode 1 (SwiGLU interleave): (r/16)*32 + row_off + r%16
// and to columns col_off .. col_off+cols-1 of a destination with row length ld.
hipError_t launch_pack_matrix(const float* src, void* dst, int rows, int cols, int ld, int row_off,
                              int col_off, int mode, int dtype, hipStream_t st);
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t st);
hipError_t launch_broadcast_rows(const float* src, float* dst, int rows, int cols, hipStream_t st);
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t st);

// x[m, :] = E[tok(m)] for chunk rows m = i*n + j (sequence b0+i, position j of the call).
hipError_t launch_embed(const int32_t* tokens, int n, int b0, int rows, const void* embed, int V,
                        int D, int dtype, float* x, int32_t* flags, hipStream_t st);

// out[m,:] = storage(g * x[m,:] / rms(x[m,:])); optionally also e[b, t0+j, :] for m = i*n+j.
hipError_t launch_rmsnorm_rows(const float* x, const float* gain, void* out, int rows, int D,
                               float eps, int dtype, void* e_store, int n, int b0, int t0,
                               int Tmax, hipStream_t st);

enum GemmEpi {
  EPI_STORE = 0,        // out[m, n] = storage(acc)          (storage dtype)
  EPI_STORE_F32 = 1,    // outf[m, n] = acc                    (fp32)
  EPI_RESID_F32 = 2,    // outf[m, n] += acc                   (fp32 residual)
  EPI_GELU = 3,         // out[m, n] = storage(gelu(acc))
  EPI_SWIGLU = 4,       // out[m, n/32*16 + n%16] = storage(silu(gate) * up), interleaved rows
  EPI_SCATTER_HEADS = 5 // columns [c0, c0+2D) scattered to the memory layouts (K half, V half)
};

struct GemmArgs {
  const void* A;      // [M, K] row-major, lda
  const void* W;      // [N, K] row-major, ldw
  void* out;          // epilogue destination
  int M, N, K, lda, ldw, ldo;
  int a_f32;          // A is fp32 (converted to the storage type on load)
  int epi;
  // EPI_STORE with scatter of columns >= scatter_c0 (K/V of QKV into a cache): both halves to
  // [B][H][T][dh].  EPI_SCATTER_HEADS (memory rows): keys to [B][H][T][dh], values to the
  // key-blocked [B][H][T8/8][dh][8] layout.  which = (n - c0) / D in {0 (k), 1 (v)}.
  void* sc_k;
  void* sc_v;
  int sc_c0;          // first scattered column (D for QKV, 0 for memory projections)
  int sc_n, sc_b0, sc_t0, sc_T, sc_H, sc_dh, sc_D, sc_B;  // row m -> (b0 + m/n, t0 + m%n)
  // Optional split-K workspace (fp32, splitk_ws_floats long) for EPI_STORE_F32 / EPI_RESID_F32
  // products with too few output tiles to fill the chip: K is split over blockIdx.z, the
  // partials land in the workspace and a second kernel adds them in a fixed order.
  float* splitk_ws;
  size_t splitk_ws_floats;
  int k_split;        // set by launch_gemm
};
// Workspace floats split-K needs for an M x N product (the most launch_gemm will use).
size_t gemm_splitk_ws_floats(int M, int N);
// Fragment-major copy of a packed bf16 [N][K] matrix (N % 16 == 0, K % 64 == 0).
hipError_t launch_pack_frag(const void* w, void* dst, int N, int K, hipStream_t st);

// Weight-streaming products of the decoder step for M <= 512 rows (bf16, wstream.hip):
// Y[M, N] = X[M, K] W^T with W and X both in fragment-major layout (act_offset), one
// 16-column block (or a pair of blocks) and one group of up to 64 rows per workgroup, K split
// over its waves.  RMSNorm is folded
// in: a residual product also writes xb = bf16(g_next * y) and per-block row sums of squares;
// the next product reads xb and scales its rows by 1 / rms(y).
enum WstEpi { WEPI_F32 = 0, WEPI_RESID = 1, WEPI_GELU = 2, WEPI_SWIGLU = 3, WEPI_MERGE = 4 };
struct WstArgs {
  int epi;
  const uint4* xf;          // X, fragment-major bf16 [Mp][K]: Mp = M rounded up to 64
  const float* ssp;         // WEPI_F32 / GELU / SWIGLU: per-block row sums of squares of y, [nt_in][ld_ss]
  int nt_in;                // D / 16 blocks (<= 128)
  int ld_ss;                // row stride of the sums-of-squares arrays: a multiple of 64, >= M
  float eps;
  const uint16_t* e;        // WEPI_MERGE: e of the state, bf16 [M][T][D], row t
  int T, t, D;
  const uint4* wf;          // fragment-major W [N][K]
  int M, N, K;
  float* outf;              // WEPI_F32 output (row-major), WEPI_RESID / WEPI_MERGE residual y (fp32, ldo)
  uint16_t* outb;           // WEPI_GELU / WEPI_SWIGLU activation, fragment-major bf16 with K = ldo
  int ldo;                  // output columns (N, or N / 2 for the paired epilogues)
  float* ssp_out;           // WEPI_RESID / WEPI_MERGE: [ldo/16][ld_ss] row sums of squares of each 16-column block
  const float* gain_next;   // WEPI_RESID (optional) / WEPI_MERGE: gain of the next norm [D]
  uint16_t* xb_out;         // with gain_next: bf16(gain_next * y), fragment-major with K = ldo
  const float* bias;        // WEPI_MERGE: b_g [D]
};
bool wsn_supported(int M, int N, int K);
hipError_t launch_wsn(const WstArgs& a, hipStream_t st);
// The merge's X = [e_t ; bf16(s)] as a fragment-major bf16 [Mp][2D] matrix (rows M..Mp-1 zero).
hipError_t launch_merge_x(const uint16_t* e, const float* s, void* xf, int M, int Mp, int T, int D, int t,
                          hipStream_t st);
// s = g * y / rms(y) from the per-block sums of squares (nt blocks); also s_out[b][step] when set.
hipError_t launch_final_norm_ssp(const float* y, const float* ssp, int nt, int ld_ss, const float* gain, float* s,
                                 float* s_out, int B, int D, float eps, int step, int n, hipStream_t st);
// Fragment-major bf16 copy of the merge matrix [2D][2D] from the fp32 W_ge, W_gs, W_fb [D][D].
hipError_t launch_pack_merge_frag(const float* wge, const float* wgs, const float* wfb, void* dst, int D,
                                  hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, int dtype, hipStream_t st);

// Action scoring: logp_i = log softmax(W_out s_i / temperature)[a_i] (and the ratio against
// behav when ratio is non-null), without writing the logits.  logp holds the row
// log-sum-exp between the two kernels.
hipError_t launch_score_actions(const float* s, const void* w_out, const void* w_frag, const int32_t* actions,
                                const float* behav, float* logp, float* ratio, int N, int D, int V, float temperature,
                                int dtype, hipStream_t st);
// One sampled token and its behaviour log-probability per row of logits [N][V] (V <= 32768).
hipError_t launch_sample_tokens(const float* logits, const float* uniforms, int32_t* tokens, float* logp, int N,
                                int V, float temperature, int top_k, float top_p, hipStream_t st);
// Writes the fragment-major bf16 copy of the fp32 head w [V][D] (layout in ModelLayout).
hipError_t launch_pack_score_head(const float* w, void* dst, int V, int D, hipStream_t st);

// Causal attention for Bc sequences x H heads, queries at positions t0..t0+n-1
// (q rows from a [Bc*n, ldq] buffer, head h at column h*dh), keys/values at positions
// 0..t0+n-1 read from a [B][H][T][dh] layout (kv_ld_b = stride between sequences,
// kv_ld_h = between heads, kv_ld_t = between positions).  Output [Bc*n, D] storage dtype.
struct AttnArgs {
  const void* q; int ldq;
  const void* k; const void* v;
  long long kv_ld_b, kv_ld_h, kv_ld_t;
  void* out; int ldo;
  int Bc, H, dh, n, t0;
};
hipError_t launch_enc_attention(const AttnArgs& a, int dtype, hipStream_t st);

// Persistent small-d decoder: one workgroup per sequence, steps t0 .. t0+n-1.
struct DecSmallArgs {
  const char* ws;      // packed model workspace
  char* state;         // state blob
  float* s_out;        // [B][n][D] or null
  int B, T, t0, n;
};
bool dec_small_supported(const ModelLayout& m, int T);
size_t dec_small_lds_bytes(const ModelLayout& m, int T);
hipError_t launch_dec_small(const ModelLayout& m, const StateLayout& s, const DecSmallArgs& a,
                            hipStream_t st);

// Test-hook conversions between fp32 [.., n, d] and the stored layouts
// (heads_layout 0: [B][T][d]; 1: [B][H][T][dh]; 2: key-blocked [B][H][T8/8][dh][8]).
hipError_t launch_store_tokens(const float* src, void* dst, int B, int n, int D, int t0, int Tmax,
                               int dtype, int heads_layout, int H, int dh, int to_device_layout,
                               hipStream_t st);

// Batched (large-d) decoder step loop.  `scratch` is the decoder scratch region
// (dec_batched_scratch_bytes long); its arrival counters (dec_batched_counters, relative to the
// region) must be zero when a replay starts, and every replay leaves them zero.
bool dec_batched_supported(const ModelLayout& m);
size_t dec_batched_scratch_bytes(const ModelLayout& m, int B, int T);
void dec_batched_counters(const ModelLayout& m, int B, int T, size_t* offset, size_t* bytes);
hipError_t run_dec_batched(const ModelLayout& m, const StateLayout& s, const char* ws, char* state, char* scratch,
                           float* s_out, int t0, int n, hipStream_t st);

// Full-BPTT backward of the replay (bptt.hip), fp32 arithmetic on the canonical fp32 weights.
// Element offsets of the canonical tensors; f1, f2, f3 = ffn_w1, ffn_w2, - (GELU) or
// ffn_gate, ffn_up, ffn_down (SwiGLU).
struct BpttOffsets {
  int64_t embed, w_out, s_star, w_ge, w_gs, w_fb, b_g, wq, wk, wv, wo, f1, f2, f3, wqx, wox, wkm, wvm;
  int64_t g_enc_attn, g_enc_ffn, g_enc_final, g_dec_self, g_dec_cross, g_dec_ffn, g_dec_final;
};
bool bptt_supported(const rlt_config& c, int B, int T, const char** why);
size_t bptt_workspace_bytes(const rlt_config& c, int B, int T);
// detach: bit 0 cuts s_{t-1} into the merge (t >= 2), bit 1 the earlier window entries, bit 2
// the memory rows.  grads (total_numel floats, canonical layout) are overwritten; loss [B].
hipError_t run_bptt(const rlt_config& c, const BpttOffsets& o, const float* w, const int32_t* tok, const float* mask,
                    int B, int T, int detach, float* grads, float* loss, char* ws, size_t total_numel,
                    hipStream_t st);

}  // namespace rlt
