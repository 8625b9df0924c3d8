// Full back-propagation through time of the replay: the exact gradient of the summed next-token
// loss of B sequences with respect to every parameter, s* included.
//
// Pages: [DS] deepsonar "技术拆解 009｜RLT：给 Transformer 接一条时间回路…" §2.5 and the
// build-your-own recipe of §六 (teacher forcing, every valid next-token prediction supervised,
// gradient through the whole recurrent trajectory); §2.6, second point (the gradient runs through
// the recurrent output, the decoder window keys/values and the encoder memory; any detach is an
// approximation); §2.7 (activation checkpointing: the decoder keeps only each step's layer inputs
// and window entries and recomputes the rest backwards).
//
// Arithmetic is fp32 on the canonical fp32 weights.  The pass:
//  1. encoder forward over all B*T tokens, keeping each layer's residual input and mid point;
//     e and the G memories (rows [K | V]);
//  2. decoder forward, one workgroup per sequence over all T steps, keeping per step the layer
//     inputs y_in, the window key/value of every position and s_{t-1} (the tape);
//  3. logits, loss and dz = mask (softmax - onehot) per row; dS = dz W_out; dW_out = dz^T S;
//  4. reverse sweep, one workgroup per sequence, t = T-1 .. 0: the adjoint of s_t (its logit term
//     plus what the next merge sends back) through the final norm, the layers in reverse (FFN,
//     cross-attention, window attention, each recomputed from the tape) and the merge.  Window
//     key/value adjoints accumulate in a ring of W slots per layer (a slot is final when its own
//     position is reached, then cleared); memory-row adjoints accumulate in [G][B*T][2D].  Each
//     product's (output adjoint, input) pair is written out for step 5;
//  5. weight gradients as products over all B*T rows (no rank-B updates inside the sweep); memory
//     adjoints back onto e;
//  6. encoder backward, token-parallel; embedding gradient per token id in position order.
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int NT = 256;   // threads of the per-sequence workgroups (4 waves)

__host__ __device__ inline size_t a64(size_t n) { return (n + 63) / 64 * 64; }

// ---------------------------------------------------------------------------------------------
// Token-parallel building blocks
// ---------------------------------------------------------------------------------------------

// C[m][n] = beta C[m][n] + sum_k A(m,k) B(k,n) with A(m,k) = A[m sam + k sak] and
// B(k,n) = B[k sbk + n sbn] (any transposition through the strides).  64x64 tiles, K in steps of
// 16 through LDS, 4x4 outputs per thread.  With ksplit > 1 slice z of K writes its partial sums
// to part[z][M][N] and gemm_reduce_k adds the slices in order 0..ksplit-1.
struct GArgs {
  const float* A; const float* Bm; float* C; float* part;
  long long sam, sak, sbk, sbn, ldc;
  int M, N, K, ksplit;
  float beta;
};

__global__ __launch_bounds__(256) void gemm_f32_k(GArgs g) {
  __shared__ float As[16][68];
  __shared__ float Bs[16][68];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int kper = (g.K + g.ksplit - 1) / g.ksplit;
  const int kb = blockIdx.z * kper;
  const int ke = min(g.K, kb + kper);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = kb; k0 < ke; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = threadIdx.x + 256 * u;
      int kk, mm;
      if (g.sam == 1) { mm = i % 64; kk = i / 64; } else { kk = i % 16; mm = i / 16; }
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < g.M && k < ke) ? g.A[m * g.sam + k * g.sak] : 0.f;
      int kb2, nn;
      if (g.sbn == 1) { nn = i % 64; kb2 = i / 64; } else { kb2 = i % 16; nn = i / 16; }
      const int n = n0 + nn, k2 = k0 + kb2;
      Bs[kb2][nn] = (n < g.N && k2 < ke) ? g.Bm[k2 * g.sbk + n * g.sbn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      if (g.ksplit == 1) {
        float* c = g.C + m * g.ldc + n;
        *c = g.beta == 0.f ? acc[i][j] : fmaf(g.beta, *c, acc[i][j]);
      } else {
        g.part[(static_cast<size_t>(blockIdx.z) * g.M + m) * g.N + n] = acc[i][j];
      }
    }
  }
}

__global__ void gemm_reduce_k(const float* part, float* C, long long ldc, int M, int N, int ksplit, float beta) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(M) * N) return;
  const int m = static_cast<int>(i / N), n = static_cast<int>(i % N);
  float s = 0.f;
  for (int z = 0; z < ksplit; ++z) s += part[static_cast<size_t>(z) * M * N + i];
  float* c = C + m * ldc + n;
  *c = beta == 0.f ? s : fmaf(beta, *c, s);
}

// out[r] = g * x[r] / rms(x[r]); one wave per row.
__global__ void rms_rows_k(const float* x, long long ldx, const float* gain, float* out, long long ldo, int R, int D,
                           float eps) {
  const int r = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64, lane = threadIdx.x % 64;
  if (r >= R) return;
  const float* xr = x + r * ldx;
  float ss = 0.f;
  for (int c = lane; c < D; c += 64) ss = fmaf(xr[c], xr[c], ss);
  ss = group_sum<64>(ss);
  const float rr = sqrtf(ss / D + eps);
  for (int c = lane; c < D; c += 64) out[r * ldo + c] = gain[c] * xr[c] / rr;
}

// Adjoint of out = g x / r per row: dx[r] += (dn - n mean(dn n)) / r with n = x / r, dn = dout g;
// gprod[r] = dout n (column sums of gprod give the gain's gradient).  One wave per row.
__global__ void rms_bwd_rows_k(const float* x, long long ldx, const float* gain, const float* dout, long long ldd,
                               float* dx, long long lddx, float* gprod, int R, int D, float eps) {
  const int r = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64, lane = threadIdx.x % 64;
  if (r >= R) return;
  const float* xr = x + r * ldx;
  const float* dr = dout + r * ldd;
  float ss = 0.f;
  for (int c = lane; c < D; c += 64) ss = fmaf(xr[c], xr[c], ss);
  ss = group_sum<64>(ss);
  const float rr = sqrtf(ss / D + eps);
  float dot = 0.f;
  for (int c = lane; c < D; c += 64) dot = fmaf(dr[c] * gain[c], xr[c] / rr, dot);
  dot = group_sum<64>(dot) / D;
  for (int c = lane; c < D; c += 64) {
    const float n = xr[c] / rr;
    dx[r * lddx + c] += (dr[c] * gain[c] - n * dot) / rr;
    gprod[static_cast<size_t>(r) * D + c] = dr[c] * n;
  }
}

// Column sums of rows [R][D] in a fixed order: chunk partials, then their ordered sum.
constexpr int kColChunks = 256;
__global__ void colsum_part_k(const float* rows, int R, int D, float* part) {
  __shared__ float red[4][64];
  const int c = blockIdx.x * 64 + threadIdx.x % 64, sub = threadIdx.x / 64;
  const int per = (R + kColChunks - 1) / kColChunks;
  const int r0 = blockIdx.y * per, r1 = min(R, r0 + per);
  float s = 0.f;
  if (c < D)
    for (int r = r0 + sub; r < r1; r += 4) s += rows[static_cast<size_t>(r) * D + c];
  red[sub][threadIdx.x % 64] = s;
  __syncthreads();
  if (sub == 0 && c < D)
    part[static_cast<size_t>(blockIdx.y) * D + c] = (red[0][threadIdx.x] + red[1][threadIdx.x]) +
                                                   (red[2][threadIdx.x] + red[3][threadIdx.x]);
}
__global__ void colsum_fin_k(const float* part, int D, float* out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= D) return;
  float s = 0.f;
  for (int z = 0; z < kColChunks; ++z) s += part[static_cast<size_t>(z) * D + c];
  out[c] += s;
}

__device__ __forceinline__ float gelu_grad(float x) {
  return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * expf(-0.5f * x * x) * 0.39894228040143268f;
}
__device__ __forceinline__ float silu_grad(float x) {
  const float s = sigmoid_f(x);
  return s * (1.0f + x * (1.0f - s));
}

// FFN activation rows: GELU act = gelu(u); SwiGLU (u = [gate | up]) act = silu(gate) up.
__global__ void act_fwd_k(const float* U, int R, int F, int swiglu, float* act) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(R) * F) return;
  const size_t r = i / F, f = i % F;
  if (swiglu) act[i] = silu_f(U[r * 2 * F + f]) * U[r * 2 * F + F + f];
  else act[i] = gelu_erf(U[i]);
}
__global__ void act_bwd_k(const float* U, const float* dact, int R, int F, int swiglu, float* dU) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(R) * F) return;
  const size_t r = i / F, f = i % F;
  if (swiglu) {
    const float g = U[r * 2 * F + f], u = U[r * 2 * F + F + f];
    dU[r * 2 * F + f] = dact[i] * u * silu_grad(g);
    dU[r * 2 * F + F + f] = dact[i] * silu_f(g);
  } else {
    dU[i] = dact[i] * gelu_grad(U[i]);
  }
}

// x[r] = E[tok r]; an id outside [0, V) is clamped and flagged (the loss then reads NaN).
__global__ void embed_fwd_k(const int32_t* tok, const float* E, int R, int D, int V, float* x, int* err) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(R) * D) return;
  const size_t r = i / D, c = i % D;
  int t = tok[r];
  if (t < 0 || t >= V) {
    if (c == 0) atomicOr(err, 1);
    t = t < 0 ? 0 : V - 1;
  }
  x[i] = E[static_cast<size_t>(t) * D + c];
}

// G_embed[v] += sum of dx over the rows whose token is v, in position order; one wave per id.
__global__ void embed_bwd_k(const int32_t* tok, const float* dx, int R, int D, int V, float* gE) {
  const int v = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64, lane = threadIdx.x % 64;
  if (v >= V) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};   // columns lane, lane+64, lane+128, lane+192 (D <= 256)
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int r = r0 + lane;
    const bool hit = r < R && tok[r] == v;
    uint64_t m = __ballot(hit);
    while (m) {
      const int rr = r0 + __builtin_ctzll(m);
      m &= m - 1;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (lane + 64 * u < D) acc[u] += dx[static_cast<size_t>(rr) * D + lane + 64 * u];
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (lane + 64 * u < D) gE[static_cast<size_t>(v) * D + lane + 64 * u] += acc[u];
}

// Softmax cross-entropy per row r = b T + t (one wave per row), in place: Z[r] becomes
// dz = w (softmax(z) - onehot(tok[r+1])) with w = mask[b][t] (1 without a mask) for t < T-1 and
// 0 for the last position; lossr[r] = w (lse - z[target]).
__global__ void ce_rows_k(float* Z, int V, const int32_t* tok, const float* mask, int B, int T, float* lossr) {
  const int r = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64, lane = threadIdx.x % 64;
  if (r >= B * T) return;
  const int b = r / T, t = r % T;
  float w = 0.f;
  if (t < T - 1) w = mask ? mask[static_cast<size_t>(b) * (T - 1) + t] : 1.f;
  float* z = Z + static_cast<size_t>(r) * V;
  if (w == 0.f) {
    for (int v = lane; v < V; v += 64) z[v] = 0.f;
    if (lane == 0) lossr[r] = 0.f;
    return;
  }
  int tgt = tok[r + 1];
  tgt = tgt < 0 ? 0 : (tgt >= V ? V - 1 : tgt);
  float mx = -INFINITY;
  for (int v = lane; v < V; v += 64) mx = fmaxf(mx, z[v]);
  mx = group_max<64>(mx);
  float s = 0.f;
  for (int v = lane; v < V; v += 64) s += expf(z[v] - mx);
  s = group_sum<64>(s);
  const float lse = mx + logf(s);
  const float zt = z[tgt];
  for (int v = lane; v < V; v += 64) z[v] = w * (expf(z[v] - lse) - (v == tgt ? 1.f : 0.f));
  if (lane == 0) lossr[r] = w * (lse - zt);
}

__global__ void seq_loss_k(const float* lossr, int B, int T, const int* err, float* loss) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  float s = 0.f;
  for (int t = 0; t < T; ++t) s += lossr[static_cast<size_t>(b) * T + t];
  loss[b] = *err ? NAN : s;
}

// dst[k][n] = src[n][k] for a [N][K] matrix.
__global__ void transpose_k(const float* src, float* dst, int N, int K) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(N) * K) return;
  const size_t n = i / K, k = i % K;
  dst[k * N + n] = src[i];
}

// ---------------------------------------------------------------------------------------------
// Encoder causal attention (fp32): forward with the row log-sum-exp, and its adjoint.
// QKV rows [R][3D] (q | k | v), head h at columns h*DH.  One thread per query (or key) row,
// the other side staged through LDS in tiles of 64 rows.
// ---------------------------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(64) void enc_attn_fwd_k(const float* QKV, float* O, float* LSE, int T, int H, int D,
                                                     float scale) {
  __shared__ float Ks[64][DH + 1];
  __shared__ float Vs[64][DH + 1];
  const int b = blockIdx.z, h = blockIdx.y, i = blockIdx.x * 64 + threadIdx.x;
  const size_t rb = static_cast<size_t>(b) * T;
  float q[DH], o[DH];
  const bool live = i < T;
  const float* qr = QKV + (rb + min(i, T - 1)) * 3 * D + h * DH;
#pragma unroll
  for (int c = 0; c < DH; ++c) { q[c] = qr[c] * scale; o[c] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int last = min(T - 1, blockIdx.x * 64 + 63);
  for (int j0 = 0; j0 <= last; j0 += 64) {
    const int j = j0 + threadIdx.x;
    const float* kr = QKV + (rb + min(j, T - 1)) * 3 * D + D + h * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) { Ks[threadIdx.x][c] = kr[c]; Vs[threadIdx.x][c] = kr[D + c]; }
    __syncthreads();
    const int jn = min(64, i - j0 + 1);
    for (int jj = 0; live && jj < jn; ++jj) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) s = fmaf(q[c], Ks[jj][c], s);
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn), p = expf(s - mn);
      l = l * a + p;
#pragma unroll
      for (int c = 0; c < DH; ++c) o[c] = fmaf(o[c], a, p * Vs[jj][c]);
      m = mn;
    }
    __syncthreads();
  }
  if (!live) return;
#pragma unroll
  for (int c = 0; c < DH; ++c) O[(rb + i) * D + h * DH + c] = o[c] / l;
  LSE[(static_cast<size_t>(b) * H + h) * T + i] = m + logf(l);
}

// dq_i = scale sum_{j<=i} p_ij (dp_ij - D_i) k_j with p_ij = exp(scale q_i.k_j - lse_i),
// dp_ij = dO_i.v_j, D_i = dO_i.O_i (also stored for the key side).
template <int DH>
__global__ __launch_bounds__(64) void enc_attn_bwd_q_k(const float* QKV, const float* O, const float* dO,
                                                       const float* LSE, float* Dsum, float* dQKV, int T, int H,
                                                       int D, float scale) {
  __shared__ float Ks[64][DH + 1];
  __shared__ float Vs[64][DH + 1];
  const int b = blockIdx.z, h = blockIdx.y, i = blockIdx.x * 64 + threadIdx.x;
  const size_t rb = static_cast<size_t>(b) * T;
  const bool live = i < T;
  const size_t ri = rb + min(i, T - 1);
  float q[DH], g[DH], dq[DH];
  float Di = 0.f;
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    q[c] = QKV[ri * 3 * D + h * DH + c] * scale;
    g[c] = dO[ri * D + h * DH + c];
    Di = fmaf(g[c], O[ri * D + h * DH + c], Di);
    dq[c] = 0.f;
  }
  const float lse = LSE[(static_cast<size_t>(b) * H + h) * T + min(i, T - 1)];
  const int last = min(T - 1, blockIdx.x * 64 + 63);
  for (int j0 = 0; j0 <= last; j0 += 64) {
    const int j = j0 + threadIdx.x;
    const float* kr = QKV + (rb + min(j, T - 1)) * 3 * D + D + h * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) { Ks[threadIdx.x][c] = kr[c]; Vs[threadIdx.x][c] = kr[D + c]; }
    __syncthreads();
    const int jn = min(64, i - j0 + 1);
    for (int jj = 0; live && jj < jn; ++jj) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) { s = fmaf(q[c], Ks[jj][c], s); dp = fmaf(g[c], Vs[jj][c], dp); }
      const float ds = expf(s - lse) * (dp - Di);
#pragma unroll
      for (int c = 0; c < DH; ++c) dq[c] = fmaf(ds, Ks[jj][c], dq[c]);
    }
    __syncthreads();
  }
  if (!live) return;
  Dsum[(static_cast<size_t>(b) * H + h) * T + i] = Di;
#pragma unroll
  for (int c = 0; c < DH; ++c) dQKV[(rb + i) * 3 * D + h * DH + c] = dq[c] * scale;
}

// Key side of a causal attention's adjoint (queries i attend keys j <= i of the same sequence):
// dk_j = scale sum_{i>=j} p_ij (dp_ij - D_i) q_i;  dv_j = sum_{i>=j} p_ij dO_i, with
// p_ij = exp(scale q_i.k_j - lse_i), dp_ij = dO_i.v_j.  Rows r = b T + t of every operand with
// their own strides; the head's columns start at h DH.  accumulate: dK, dV += (else =).
struct KvArgs {
  const float* Q; long long ldq;
  const float* K; const float* V; long long ldkv;
  const float* dO; long long lddo;
  const float* LSE; const float* Dsum;     // [B][H][T]
  float* dK; float* dV; long long lddkv;
  int T, H, accumulate;
  float scale;
};
template <int DH>
__global__ __launch_bounds__(64) void attn_bwd_kv_k(KvArgs a) {
  __shared__ float Qs[64][DH + 1];
  __shared__ float Gs[64][DH + 1];
  __shared__ float Ls[64], Ds[64];
  const int b = blockIdx.z, h = blockIdx.y, j = blockIdx.x * 64 + threadIdx.x, T = a.T;
  const size_t rb = static_cast<size_t>(b) * T;
  const bool live = j < T;
  const size_t rj = rb + min(j, T - 1);
  float k[DH], v[DH], dk[DH], dv[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    k[c] = a.K[rj * a.ldkv + h * DH + c];
    v[c] = a.V[rj * a.ldkv + h * DH + c];
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  for (int i0 = blockIdx.x * 64; i0 < T; i0 += 64) {
    const int i = i0 + threadIdx.x;
    const size_t ri = rb + min(i, T - 1);
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      Qs[threadIdx.x][c] = a.Q[ri * a.ldq + h * DH + c] * a.scale;
      Gs[threadIdx.x][c] = a.dO[ri * a.lddo + h * DH + c];
    }
    Ls[threadIdx.x] = a.LSE[(static_cast<size_t>(b) * a.H + h) * T + min(i, T - 1)];
    Ds[threadIdx.x] = a.Dsum[(static_cast<size_t>(b) * a.H + h) * T + min(i, T - 1)];
    __syncthreads();
    const int ii0 = max(0, j - i0), in = min(64, T - i0);
    for (int ii = ii0; live && ii < in; ++ii) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) { s = fmaf(Qs[ii][c], k[c], s); dp = fmaf(Gs[ii][c], v[c], dp); }
      const float p = expf(s - Ls[ii]);
      const float ds = p * (dp - Ds[ii]);
#pragma unroll
      for (int c = 0; c < DH; ++c) { dv[c] = fmaf(p, Gs[ii][c], dv[c]); dk[c] = fmaf(ds, Qs[ii][c], dk[c]); }
    }
    __syncthreads();
  }
  if (!live) return;
  // Qs holds q * scale, so dk already carries the scale.
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    float* pk = a.dK + rj * a.lddkv + h * DH + c;
    float* pv = a.dV + rj * a.lddkv + h * DH + c;
    *pk = a.accumulate ? *pk + dk[c] : dk[c];
    *pv = a.accumulate ? *pv + dv[c] : dv[c];
  }
}

// Dsum[b][h][t] = dO_r . O_r over head h's columns (r = b T + t).
__global__ void head_dots_k(const float* dO, const float* O, long long ld, int B, int T, int H, int DH, float* Dsum) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(B) * H * T) return;
  const int t = static_cast<int>(i % T), h = static_cast<int>((i / T) % H), b = static_cast<int>(i / (static_cast<size_t>(T) * H));
  const size_t r = static_cast<size_t>(b) * T + t;
  float s = 0.f;
  for (int c = 0; c < DH; ++c) s = fmaf(dO[r * ld + h * DH + c], O[r * ld + h * DH + c], s);
  Dsum[i] = s;
}

// ---------------------------------------------------------------------------------------------
// Decoder: tape forward and reverse sweep, one workgroup of 256 threads per sequence.
// ---------------------------------------------------------------------------------------------
struct DecArgs {
  const float* P;            // canonical weights
  const float* WT;           // transposed copies (W^T [K][N]) of the decoder's matrices
  BpttOffsets o;             // element offsets of the canonical tensors
  BpttOffsets ot;            // element offsets of the transposed copies in WT
  int B, T, D, H, DH, L, F, F2, G, W, swiglu, detach;
  float eps, scale;
  const float* E;            // [R][D]
  const float* MKV;          // [G][R][2D]
  float* YT;                 // [R][L+1][D]  layer inputs, then the last layer's output
  float* KVT;                // [L][R][2D]   window key | value of every position
  float* S;                  // [R][D]
  float* SPREV;              // [R][D]       s_{t-1} (s* at t = 0)
  const float* DS;           // [R][D]       logit-term adjoint of s_t
  float *DQKV, *H1, *DY1, *O1, *DQX, *H2, *DY2, *O2, *DU, *H3, *DY3, *ACT;   // [L][R][.]
  float *QXS, *DO2S;         // [L][R][D]   cross-attention query and output adjoint per step
  float* CLSE;               // [L][B][H][T] cross-attention row log-sum-exp
  float *DA, *DF, *DE;       // [R][D]
  float* DM;                 // [G][R][2D]
  float* RING;               // [L][B][W][2D]
  float* PART;               // [B][(3L+3) D]
};

// LDS map of the decoder kernels (floats).
struct DecLds {
  int y, h, q, k, v, o, y1, h2, qx, o2, y2, h3, u, act, s, e, f, gate, dy, dh, dq, dk, dv, dvec, dx2, dact, du, ds,
      dsc, pw, pw2, pc, pc2, gacc, red, total;
  __host__ __device__ DecLds(int D, int F, int F2, int H, int W, int T) {
    int p = 0;
    auto take = [&](int n) { const int r = p; p += (n + 3) / 4 * 4; return r; };
    y = take(D); h = take(D); q = take(D); k = take(D); v = take(D); o = take(D); y1 = take(D); h2 = take(D);
    qx = take(D); o2 = take(D); y2 = take(D); h3 = take(D); u = take(F2); act = take(F); s = take(D); e = take(D);
    f = take(D); gate = take(D); dy = take(D); dh = take(D); dq = take(D); dk = take(D); dv = take(D);
    dvec = take(D); dx2 = take(D); dact = take(F); du = take(F2); ds = take(D); dsc = take(D);
    pw = take(H * W); pw2 = take(H * W); pc = take(H * T); pc2 = take(H * T);
    gacc = 0; red = 0;
    total = p;
  }
};

// s_waitcnt vmcnt(0): this wave's global stores have completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = group_sum<64>(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// out[i] (+)= sum_j M[i][j] x[j] for a row-major M [Nout][Kin] (Kin a multiple of 64) and x in
// LDS: G contiguous lanes per row, each over a contiguous share of it with 16-byte loads (all
// issued before the sums), then a lane-group sum in a fixed order.
template <int G>
__device__ __forceinline__ void rowdot_g(const float* __restrict__ M, int Nout, int Kin, const float* x, float* out,
                                         bool accumulate) {
  const int per = Kin / G;
  for (int base = 0; base < Nout * G; base += NT) {
    const int tid = base + static_cast<int>(threadIdx.x);
    const int i = tid / G, gi = tid % G;
    float a = 0.f;
    if (i < Nout) {
      const float4* mr = reinterpret_cast<const float4*>(M + static_cast<size_t>(i) * Kin + gi * per);
      const float* xr = x + gi * per;
#pragma unroll 4
      for (int k = 0; k < per / 4; ++k) {
        const float4 w = mr[k];
        a = fmaf(w.x, xr[4 * k], a);
        a = fmaf(w.y, xr[4 * k + 1], a);
        a = fmaf(w.z, xr[4 * k + 2], a);
        a = fmaf(w.w, xr[4 * k + 3], a);
      }
    }
    a = group_sum<G>(a);
    if (i < Nout && gi == 0) out[i] = accumulate ? out[i] + a : a;
  }
}
__device__ __noinline__ void rowdot(const float* M, int Nout, int Kin, const float* x, float* out,
                                       bool accumulate) {
  if (Nout * 16 <= NT) rowdot_g<16>(M, Nout, Kin, x, out, accumulate);
  else if (Nout * 8 <= NT) rowdot_g<8>(M, Nout, Kin, x, out, accumulate);
  else if (Nout * 4 <= NT) rowdot_g<4>(M, Nout, Kin, x, out, accumulate);
  else if (Nout * 2 <= NT) rowdot_g<2>(M, Nout, Kin, x, out, accumulate);
  else rowdot_g<1>(M, Nout, Kin, x, out, accumulate);
}
// out[n] (+)= sum_k W[n][k] x[k] for W [N][K] (canonical layout).
__device__ __forceinline__ void matvec(const float* W, int N, int K, const float* x, float* out,
                                       bool accumulate = false) {
  rowdot(W, N, K, x, out, accumulate);
}
// out[k] (+)= sum_n W[n][k] x[n], given the transposed copy WT = W^T [K][N].
__device__ __forceinline__ void matvec_t(const float* WT, int N, int K, const float* x, float* out,
                                         bool accumulate = false) {
  rowdot(WT, K, N, x, out, accumulate);
}

// out = g x / rms(x) over an LDS vector.
__device__ __forceinline__ void rms_vec(const float* x, const float* g, float* out, int D, float eps, float* red) {
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += NT) ss = fmaf(x[c], x[c], ss);
  const float rr = sqrtf(block_sum(ss, red) / D + eps);
  for (int c = threadIdx.x; c < D; c += NT) out[c] = g[c] * x[c] / rr;
  __syncthreads();
}
// dx += adjoint of out = g x / rms(x) for dout; gacc += dout * x / rms(x).
__device__ __forceinline__ void rms_vec_bwd(const float* x, const float* g, const float* dout, float* dx, float* gacc,
                                            int D, float eps, float* red) {
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += NT) ss = fmaf(x[c], x[c], ss);
  const float rr = sqrtf(block_sum(ss, red) / D + eps);
  float dt = 0.f;
  for (int c = threadIdx.x; c < D; c += NT) dt = fmaf(dout[c] * g[c], x[c] / rr, dt);
  const float dot = block_sum(dt, red) / D;
  for (int c = threadIdx.x; c < D; c += NT) {
    const float n = x[c] / rr;
    dx[c] += (dout[c] * g[c] - n * dot) / rr;
    gacc[c] += dout[c] * n;
  }
  __syncthreads();
}

// Attention of one query (LDS, D wide) over n rows per head, one wave per head (heads h = wave,
// wave + 4, ...) and one lane per row: row i of head h has its key at krow(i) + h DH and its
// value at krow(i) + voff + h DH (16-byte loads).  The probabilities go to P[h * ldp + i], the
// output to out (LDS), the row log-sum-exp to lse[h * ldl] when lse is given.  Each lane reads
// back only the P entries it wrote; the per-dimension sums over lanes run in a fixed order.
template <int DH, typename RowFn>
__device__ __forceinline__ void attend_heads(const float* q, RowFn krow, int voff, int n, int H, float scale, float* P,
                                             int ldp, float* out, float* lse = nullptr, long long ldl = 0) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int h = wave; h < H; h += 4) {
    float* ph = P + h * ldp;
    float qh[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) qh[c] = q[h * DH + c];
    float mx = -INFINITY;
    for (int i = lane; i < n; i += 64) {
      const float4* kr = reinterpret_cast<const float4*>(krow(i) + h * DH);
      float s = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < DH / 4; ++c4) {
        const float4 k = kr[c4];
        s = fmaf(qh[4 * c4], k.x, s);
        s = fmaf(qh[4 * c4 + 1], k.y, s);
        s = fmaf(qh[4 * c4 + 2], k.z, s);
        s = fmaf(qh[4 * c4 + 3], k.w, s);
      }
      s *= scale;
      ph[i] = s;
      mx = fmaxf(mx, s);
    }
    mx = group_max<64>(mx);
    float sum = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float p = expf(ph[i] - mx);
      ph[i] = p;
      sum += p;
    }
    sum = group_sum<64>(sum);
    if (lse && lane == 0) lse[h * ldl] = mx + logf(sum);
    const float inv = 1.0f / sum;
    float acc[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) acc[c] = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float p = ph[i] * inv;
      ph[i] = p;
      const float4* vr = reinterpret_cast<const float4*>(krow(i) + voff + h * DH);
#pragma unroll
      for (int c4 = 0; c4 < DH / 4; ++c4) {
        const float4 v = vr[c4];
        acc[4 * c4] = fmaf(p, v.x, acc[4 * c4]);
        acc[4 * c4 + 1] = fmaf(p, v.y, acc[4 * c4 + 1]);
        acc[4 * c4 + 2] = fmaf(p, v.z, acc[4 * c4 + 2]);
        acc[4 * c4 + 3] = fmaf(p, v.w, acc[4 * c4 + 3]);
      }
    }
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      const float v = group_sum<64>(acc[c]);
      if (lane == c % 64) out[h * DH + c] = v;
    }
  }
  __syncthreads();
}

// Adjoint of attend_heads for the query side: with P and dout (LDS), per head (one lane per row)
// dz_i = p_i (dout.v_i - sum_j p_j dout.v_j) into Z[h * ldp + i], and dq (LDS) = scale sum_i dz_i k_i.
template <int DH, typename RowFn>
__device__ __forceinline__ void attend_heads_bwd(const float* P, const float* dout, RowFn krow, int voff, int n, int H,
                                                 float scale, float* Z, int ldp, float* dq) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int h = wave; h < H; h += 4) {
    const float* ph = P + h * ldp;
    float* zh = Z + h * ldp;
    float gh[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) gh[c] = dout[h * DH + c];
    float sdp = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float4* vr = reinterpret_cast<const float4*>(krow(i) + voff + h * DH);
      float dp = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < DH / 4; ++c4) {
        const float4 v = vr[c4];
        dp = fmaf(gh[4 * c4], v.x, dp);
        dp = fmaf(gh[4 * c4 + 1], v.y, dp);
        dp = fmaf(gh[4 * c4 + 2], v.z, dp);
        dp = fmaf(gh[4 * c4 + 3], v.w, dp);
      }
      zh[i] = dp;
      sdp = fmaf(ph[i], dp, sdp);
    }
    sdp = group_sum<64>(sdp);
    float acc[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) acc[c] = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float z = ph[i] * (zh[i] - sdp);
      zh[i] = z;
      const float4* kr = reinterpret_cast<const float4*>(krow(i) + h * DH);
#pragma unroll
      for (int c4 = 0; c4 < DH / 4; ++c4) {
        const float4 k = kr[c4];
        acc[4 * c4] = fmaf(z, k.x, acc[4 * c4]);
        acc[4 * c4 + 1] = fmaf(z, k.y, acc[4 * c4 + 1]);
        acc[4 * c4 + 2] = fmaf(z, k.z, acc[4 * c4 + 2]);
        acc[4 * c4 + 3] = fmaf(z, k.w, acc[4 * c4 + 3]);
      }
    }
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      const float v = group_sum<64>(acc[c]);
      if (lane == c % 64) dq[h * DH + c] = v * scale;
    }
  }
  __syncthreads();
}

// The forward of decoder layer l at step t from y (LDS) = the layer input, into the LDS map.
// TAPE: the tape pass (computes k, v and writes them to KVT; reads earlier window rows at agent
// scope); otherwise k, v come from the tape.  Ends with m.y2 and the FFN pre-activation m.u /
// activation m.act computed; the caller adds the FFN output.
template <bool TAPE, int DH>
__device__ void layer_fwd(const DecArgs& a, float* sm, const DecLds& m, int b, int t, int l) {
  const int D = a.D, H = a.H, W = a.W;
  const size_t R = static_cast<size_t>(a.B) * a.T, r = static_cast<size_t>(b) * a.T + t;
  float* red = sm + m.total;
  const float* P = a.P;
  rms_vec(sm + m.y, P + a.o.g_dec_self + l * D, sm + m.h, D, a.eps, red);
  const size_t dd = static_cast<size_t>(D) * D;
  matvec(a.P + a.o.wq + l * dd, D, D, sm + m.h, sm + m.q);
  float* kvt = a.KVT + static_cast<size_t>(l) * R * 2 * D;
  if (TAPE) {
    matvec(a.P + a.o.wk + l * dd, D, D, sm + m.h, sm + m.k);
    matvec(a.P + a.o.wv + l * dd, D, D, sm + m.h, sm + m.v);
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += NT) {
      kvt[r * 2 * D + c] = sm[m.k + c];
      kvt[r * 2 * D + D + c] = sm[m.v + c];
    }
    // The window below reads this row back through other waves with ordinary loads.  That is
    // safe because the row's stores complete before the workgroup barrier (vmcnt(0)) and no
    // wave of this launch has read the row's cache lines before (rows are 256-byte aligned and
    // only positions <= t are read), so no stale line can sit in the CU's cache.
    wait_stores();
  } else {
    for (int c = threadIdx.x; c < D; c += NT) {
      sm[m.k + c] = kvt[r * 2 * D + c];
      sm[m.v + c] = kvt[r * 2 * D + D + c];
    }
  }
  __syncthreads();
  // window: positions j0 .. t, every row (the current one included) from the tape
  const int j0 = max(0, t - W + 1), n = t - j0 + 1;
  auto wrow = [&](int i) -> const float* { return kvt + (static_cast<size_t>(b) * a.T + j0 + i) * 2 * D; };
  attend_heads<DH>(sm + m.q, wrow, D, n, H, a.scale, sm + m.pw, W, sm + m.o);
  matvec(a.P + a.o.wo + l * dd, D, D, sm + m.o, sm + m.y1);
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += NT) sm[m.y1 + c] += sm[m.y + c];
  __syncthreads();
  rms_vec(sm + m.y1, P + a.o.g_dec_cross + l * D, sm + m.h2, D, a.eps, red);
  matvec(a.P + a.o.wqx + l * dd, D, D, sm + m.h2, sm + m.qx);
  __syncthreads();
  const int g = a.G == 1 ? 0 : l;
  const float* mkv = a.MKV + (static_cast<size_t>(g) * R + static_cast<size_t>(b) * a.T) * 2 * D;
  auto mrow = [&](int i) -> const float* { return mkv + static_cast<size_t>(i) * 2 * D; };
  float* clse = TAPE ? nullptr : a.CLSE + ((static_cast<size_t>(l) * a.B + b) * H) * a.T + t;
  attend_heads<DH>(sm + m.qx, mrow, D, t + 1, H, a.scale, sm + m.pc, a.T, sm + m.o2, clse, a.T);
  matvec(a.P + a.o.wox + l * dd, D, D, sm + m.o2, sm + m.y2);
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += NT) sm[m.y2 + c] += sm[m.y1 + c];
  __syncthreads();
  rms_vec(sm + m.y2, P + a.o.g_dec_ffn + l * D, sm + m.h3, D, a.eps, red);
  const size_t fd = static_cast<size_t>(a.F) * D;
  if (a.swiglu) {
    matvec(a.P + a.o.f1 + l * fd, a.F, D, sm + m.h3, sm + m.u);
    matvec(a.P + a.o.f2 + l * fd, a.F, D, sm + m.h3, sm + m.u + a.F);
    __syncthreads();
    for (int f = threadIdx.x; f < a.F; f += NT) sm[m.act + f] = silu_f(sm[m.u + f]) * sm[m.u + a.F + f];
  } else {
    matvec(a.P + a.o.f1 + l * fd, a.F, D, sm + m.h3, sm + m.u);
    __syncthreads();
    for (int f = threadIdx.x; f < a.F; f += NT) sm[m.act + f] = gelu_erf(sm[m.u + f]);
  }
  __syncthreads();
}

__device__ __forceinline__ const float* ffn_out_t(const DecArgs& a, int l) {
  const size_t fd = static_cast<size_t>(a.F) * a.D;
  return a.WT + (a.swiglu ? a.ot.f3 : a.ot.f2) + l * fd;
}
__device__ __forceinline__ const float* ffn_out_w(const DecArgs& a, int l) {
  const size_t fd = static_cast<size_t>(a.F) * a.D;
  return a.P + (a.swiglu ? a.o.f3 : a.o.f2) + l * fd;
}

// gated merge from s (LDS) and e_t: y = g e + (1 - g) f, f = W_fb s, g = sigmoid(W_ge e + W_gs s + b_g)
__device__ void merge_fwd(const DecArgs& a, float* sm, const DecLds& m, size_t r) {
  const int D = a.D;
  for (int c = threadIdx.x; c < D; c += NT) sm[m.e + c] = a.E[r * D + c];
  __syncthreads();
  matvec(a.P + a.o.w_fb, D, D, sm + m.s, sm + m.f);
  matvec(a.P + a.o.w_ge, D, D, sm + m.e, sm + m.gate);
  __syncthreads();
  matvec(a.P + a.o.w_gs, D, D, sm + m.s, sm + m.gate, true);
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += NT) {
    const float gt = sigmoid_f(sm[m.gate + c] + a.P[a.o.b_g + c]);
    sm[m.gate + c] = gt;
    sm[m.y + c] = gt * sm[m.e + c] + (1.0f - gt) * sm[m.f + c];
  }
  __syncthreads();
}

template <int DH>
__global__ __launch_bounds__(NT) void dec_tape_k(DecArgs a) {
  extern __shared__ float sm[];
  const int b = blockIdx.x, D = a.D, L = a.L;
  const DecLds m(D, a.F, a.F2, a.H, a.W, a.T);
  float* red = sm + m.total;
  for (int c = threadIdx.x; c < D; c += NT) sm[m.s + c] = a.P[a.o.s_star + c];
  __syncthreads();
  for (int t = 0; t < a.T; ++t) {
    const size_t r = static_cast<size_t>(b) * a.T + t;
    for (int c = threadIdx.x; c < D; c += NT) a.SPREV[r * D + c] = sm[m.s + c];
    merge_fwd(a, sm, m, r);
    for (int l = 0; l < L; ++l) {
      for (int c = threadIdx.x; c < D; c += NT) a.YT[(r * (L + 1) + l) * D + c] = sm[m.y + c];
      layer_fwd<true, DH>(a, sm, m, b, t, l);
      matvec(ffn_out_w(a, l), D, a.F, sm + m.act, sm + m.y);
      __syncthreads();
      for (int c = threadIdx.x; c < D; c += NT) sm[m.y + c] += sm[m.y2 + c];
      __syncthreads();
    }
    for (int c = threadIdx.x; c < D; c += NT) a.YT[(r * (L + 1) + L) * D + c] = sm[m.y + c];
    rms_vec(sm + m.y, a.P + a.o.g_dec_final, sm + m.s, D, a.eps, red);
    for (int c = threadIdx.x; c < D; c += NT) a.S[r * D + c] = sm[m.s + c];
    // this step's window rows are read by other waves in later steps
    wait_stores();
    __syncthreads();
  }
}

template <int DH>
__global__ __launch_bounds__(NT) void dec_sweep_k(DecArgs a) {
  extern __shared__ float sm[];
  const int b = blockIdx.x, D = a.D, L = a.L, H = a.H, W = a.W;
  const DecLds m(D, a.F, a.F2, a.H, a.W, a.T);
  float* red = sm + m.total;
  float* gacc = red + 8;   // [g_dec_self L D][g_dec_cross L D][g_dec_ffn L D][g_dec_final D][b_g D][s* D]
  const int NP = (3 * L + 3) * D;
  const size_t R = static_cast<size_t>(a.B) * a.T;
  const size_t dd = static_cast<size_t>(D) * D;
  for (int i = threadIdx.x; i < NP; i += NT) gacc[i] = 0.f;
  for (int c = threadIdx.x; c < D; c += NT) sm[m.dsc + c] = 0.f;
  __syncthreads();
  for (int t = a.T - 1; t >= 0; --t) {
    const size_t r = static_cast<size_t>(b) * a.T + t;
    // adjoint of s_t, through the final norm
    for (int c = threadIdx.x; c < D; c += NT) {
      sm[m.ds + c] = a.DS[r * D + c] + sm[m.dsc + c];
      sm[m.y + c] = a.YT[(r * (L + 1) + L) * D + c];
      sm[m.dy + c] = 0.f;
    }
    __syncthreads();
    rms_vec_bwd(sm + m.y, a.P + a.o.g_dec_final, sm + m.ds, sm + m.dy, gacc + 3 * L * D, D, a.eps, red);
    for (int l = L - 1; l >= 0; --l) {
      const size_t rl = static_cast<size_t>(l) * R + r;
      for (int c = threadIdx.x; c < D; c += NT) sm[m.y + c] = a.YT[(r * (L + 1) + l) * D + c];
      __syncthreads();
      layer_fwd<false, DH>(a, sm, m, b, t, l);
      // FFN sub-block: y3 = y2 + W2 act(u), u from h3
      for (int c = threadIdx.x; c < D; c += NT) {
        a.DY3[rl * D + c] = sm[m.dy + c];
        a.H3[rl * D + c] = sm[m.h3 + c];
      }
      for (int f = threadIdx.x; f < a.F; f += NT) a.ACT[rl * a.F + f] = sm[m.act + f];
      matvec_t(ffn_out_t(a, l), D, a.F, sm + m.dy, sm + m.dact);
      __syncthreads();
      const size_t fd = static_cast<size_t>(a.F) * D;
      if (a.swiglu) {
        for (int f = threadIdx.x; f < a.F; f += NT) {
          const float gt = sm[m.u + f], up = sm[m.u + a.F + f], da = sm[m.dact + f];
          sm[m.du + f] = da * up * silu_grad(gt);
          sm[m.du + a.F + f] = da * silu_f(gt);
        }
        __syncthreads();
        matvec_t(a.WT + a.ot.f1 + l * fd, a.F, D, sm + m.du, sm + m.dh);
        __syncthreads();
        matvec_t(a.WT + a.ot.f2 + l * fd, a.F, D, sm + m.du + a.F, sm + m.dh, true);
      } else {
        for (int f = threadIdx.x; f < a.F; f += NT) sm[m.du + f] = sm[m.dact + f] * gelu_grad(sm[m.u + f]);
        __syncthreads();
        matvec_t(a.WT + a.ot.f1 + l * fd, a.F, D, sm + m.du, sm + m.dh);
      }
      for (int f = threadIdx.x; f < a.F2; f += NT) a.DU[rl * a.F2 + f] = sm[m.du + f];
      __syncthreads();
      rms_vec_bwd(sm + m.y2, a.P + a.o.g_dec_ffn + l * D, sm + m.dh, sm + m.dy, gacc + (2 * L + l) * D, D, a.eps,
                  red);
      // cross-attention sub-block: y2 = y1 + W_Ox attn(W_Qx h2 over memory rows 0..t)
      for (int c = threadIdx.x; c < D; c += NT) {
        a.DY2[rl * D + c] = sm[m.dy + c];
        a.O2[rl * D + c] = sm[m.o2 + c];
      }
      matvec_t(a.WT + a.ot.wox + l * dd, D, D, sm + m.dy, sm + m.dvec);
      __syncthreads();
      const int g = a.G == 1 ? 0 : l;
      const float* mkv = a.MKV + (static_cast<size_t>(g) * R + static_cast<size_t>(b) * a.T) * 2 * D;
      auto mrow = [&](int i) -> const float* { return mkv + static_cast<size_t>(i) * 2 * D; };
      attend_heads_bwd<DH>(sm + m.pc, sm + m.dvec, mrow, D, t + 1, H, a.scale, sm + m.pc2, a.T, sm + m.dq);
      // the memory rows' adjoints are formed after the sweep, token-parallel, from q_x, this
      // output adjoint and the row log-sum-exp
      for (int c = threadIdx.x; c < D; c += NT) {
        a.QXS[rl * D + c] = sm[m.qx + c];
        a.DO2S[rl * D + c] = sm[m.dvec + c];
      }
      for (int c = threadIdx.x; c < D; c += NT) {
        a.DQX[rl * D + c] = sm[m.dq + c];
        a.H2[rl * D + c] = sm[m.h2 + c];
      }
      matvec_t(a.WT + a.ot.wqx + l * dd, D, D, sm + m.dq, sm + m.dh);
      __syncthreads();
      rms_vec_bwd(sm + m.y1, a.P + a.o.g_dec_cross + l * D, sm + m.dh, sm + m.dy, gacc + (L + l) * D, D, a.eps, red);
      // window self-attention sub-block: y1 = y + W_O attn(q over window rows j0..t)
      for (int c = threadIdx.x; c < D; c += NT) {
        a.DY1[rl * D + c] = sm[m.dy + c];
        a.O1[rl * D + c] = sm[m.o + c];
      }
      matvec_t(a.WT + a.ot.wo + l * dd, D, D, sm + m.dy, sm + m.dvec);
      __syncthreads();
      const int j0 = max(0, t - W + 1), n = t - j0 + 1;
      const float* kvt = a.KVT + static_cast<size_t>(l) * R * 2 * D;
      auto wrow = [&](int i) -> const float* { return kvt + (static_cast<size_t>(b) * a.T + j0 + i) * 2 * D; };
      attend_heads_bwd<DH>(sm + m.pw, sm + m.dvec, wrow, D, n, H, a.scale, sm + m.pw2, W, sm + m.dq);
      // window key/value adjoints: slot j mod W of this layer's ring; each (slot, column) element
      // is always handled by the same thread, so its read-modify-writes stay in program order
      float* ring = a.RING + (static_cast<size_t>(l) * a.B + b) * W * 2 * D;
      for (int e = threadIdx.x; e < W * D; e += NT) {
        const int slot = e / D, c = e % D, h = c / DH;
        const int j = t - ((t % W) - slot + W) % W;   // the window position held by this slot
        if (j < j0) continue;
        const int i = j - j0;
        const float dk = sm[m.pw2 + h * W + i] * sm[m.q + c] * a.scale;
        const float dv = sm[m.pw + h * W + i] * sm[m.dvec + c];
        float* rk = ring + static_cast<size_t>(slot) * 2 * D;
        if (j == t) {
          sm[m.dk + c] = dk + rk[c];
          sm[m.dv + c] = dv + rk[D + c];
          rk[c] = 0.f;
          rk[D + c] = 0.f;
        } else if (!(a.detach & 2)) {
          rk[c] += dk;
          rk[D + c] += dv;
        }
      }
      __syncthreads();
      for (int c = threadIdx.x; c < D; c += NT) {
        a.DQKV[rl * 3 * D + c] = sm[m.dq + c];
        a.DQKV[rl * 3 * D + D + c] = sm[m.dk + c];
        a.DQKV[rl * 3 * D + 2 * D + c] = sm[m.dv + c];
        a.H1[rl * D + c] = sm[m.h + c];
      }
      matvec_t(a.WT + a.ot.wq + l * dd, D, D, sm + m.dq, sm + m.dh);
      __syncthreads();
      matvec_t(a.WT + a.ot.wk + l * dd, D, D, sm + m.dk, sm + m.dh, true);
      __syncthreads();
      matvec_t(a.WT + a.ot.wv + l * dd, D, D, sm + m.dv, sm + m.dh, true);
      __syncthreads();
      rms_vec_bwd(sm + m.y, a.P + a.o.g_dec_self + l * D, sm + m.dh, sm + m.dy, gacc + l * D, D, a.eps, red);
    }
    // gated merge
    for (int c = threadIdx.x; c < D; c += NT) sm[m.s + c] = a.SPREV[r * D + c];
    __syncthreads();
    merge_fwd(a, sm, m, r);
    for (int c = threadIdx.x; c < D; c += NT) {
      const float gt = sm[m.gate + c], dy = sm[m.dy + c];
      const float da = dy * (sm[m.e + c] - sm[m.f + c]) * gt * (1.0f - gt);
      sm[m.dq + c] = da;                     // da
      sm[m.dk + c] = dy * (1.0f - gt);       // df
      sm[m.dv + c] = dy * gt;                // direct term of de_t
      a.DA[r * D + c] = da;
      a.DF[r * D + c] = sm[m.dk + c];
      gacc[(3 * L + 1) * D + c] += da;
    }
    __syncthreads();
    matvec_t(a.WT + a.ot.w_ge, D, D, sm + m.dq, sm + m.dh);
    matvec_t(a.WT + a.ot.w_fb, D, D, sm + m.dk, sm + m.ds);
    __syncthreads();
    matvec_t(a.WT + a.ot.w_gs, D, D, sm + m.dq, sm + m.ds, true);
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += NT) {
      a.DE[r * D + c] = sm[m.dv + c] + sm[m.dh + c];
      if (t == 0) gacc[(3 * L + 2) * D + c] += sm[m.ds + c];
      sm[m.dsc + c] = (a.detach & 1) ? 0.f : sm[m.ds + c];
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < NP; i += NT) a.PART[static_cast<size_t>(b) * NP + i] = gacc[i];
}

// grads[dst + i] += sum_b part[b][src + i] in order b = 0..B-1.
__global__ void part_reduce_k(const float* part, int B, int NP, int src, int n, float* dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += part[static_cast<size_t>(b) * NP + src + i];
  dst[i] += s;
}

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------
struct BpLayout {
  size_t X, XMID, E, MKV, YT, KVT, S, SPREV, Z, DS, LOSSR, ERR;
  size_t DQKV, H1, DY1, O1, DQX, H2, DY2, O2, DU, H3, DY3, ACT, QXS, DO2S, CLSE, DA, DF, DE, DM, RING, PART;
  size_t DX, HF, U, EACT, DACT, DUE, DHF, HA, QKV, O, LSE, DSUM, DO, DQKVE, DHA, GROWS, COLP, WT, GP;
  size_t gp_floats, total;   // floats
};

constexpr size_t kGemmPartFloats = size_t(16) << 20;

size_t wt_floats(const rlt_config& c) {
  const size_t D = c.d_model, L = c.n_layers, F = c.ffn_dim;
  return a64(3 * D * D) + a64(6 * L * D * D) + a64((c.ffn_kind == RLT_FFN_SWIGLU ? 3 : 2) * L * F * D);
}

BpLayout bp_layout(const rlt_config& c, int B, int T) {
  const size_t D = c.d_model, L = c.n_layers, F = c.ffn_dim, G = c.mem_groups, V = c.vocab, W = c.window;
  const size_t F2 = c.ffn_kind == RLT_FFN_SWIGLU ? 2 * F : F;
  const size_t R = static_cast<size_t>(B) * T, H = c.n_heads;
  BpLayout b{};
  size_t p = 0;
  auto take = [&](size_t n) { const size_t r = p; p += a64(n); return r; };
  b.X = take((L + 1) * R * D); b.XMID = take(L * R * D); b.E = take(R * D); b.MKV = take(G * R * 2 * D);
  b.YT = take(R * (L + 1) * D); b.KVT = take(L * R * 2 * D); b.S = take(R * D); b.SPREV = take(R * D);
  b.Z = take(R * V); b.DS = take(R * D); b.LOSSR = take(R); b.ERR = take(64);
  b.DQKV = take(L * R * 3 * D); b.H1 = take(L * R * D); b.DY1 = take(L * R * D); b.O1 = take(L * R * D);
  b.DQX = take(L * R * D); b.H2 = take(L * R * D); b.DY2 = take(L * R * D); b.O2 = take(L * R * D);
  b.DU = take(L * R * F2); b.H3 = take(L * R * D); b.DY3 = take(L * R * D); b.ACT = take(L * R * F);
  b.QXS = take(L * R * D); b.DO2S = take(L * R * D); b.CLSE = take(L * B * H * T);
  b.DA = take(R * D); b.DF = take(R * D); b.DE = take(R * D); b.DM = take(G * R * 2 * D);
  b.RING = take(L * B * W * 2 * D); b.PART = take(static_cast<size_t>(B) * (3 * L + 3) * D);
  b.DX = take(R * D); b.HF = take(R * D); b.U = take(R * F2); b.EACT = take(R * F); b.DACT = take(R * F);
  b.DUE = take(R * F2); b.DHF = take(R * D); b.HA = take(R * D); b.QKV = take(R * 3 * D); b.O = take(R * D);
  b.LSE = take(B * H * T); b.DSUM = take(B * H * T); b.DO = take(R * D); b.DQKVE = take(R * 3 * D);
  b.DHA = take(R * D); b.GROWS = take(R * D); b.COLP = take(kColChunks * D); b.WT = take(wt_floats(c));
  b.gp_floats = kGemmPartFloats;
  b.GP = take(b.gp_floats);
  b.total = p;
  return b;
}

int dec_lds_floats(const rlt_config& c, int T) {
  const int F2 = c.ffn_kind == RLT_FFN_SWIGLU ? 2 * c.ffn_dim : c.ffn_dim;
  const DecLds m(c.d_model, c.ffn_dim, F2, c.n_heads, c.window, T);
  return m.total + 8 + (3 * c.n_layers + 3) * c.d_model;
}

struct Ctx {
  hipStream_t st;
  float* gp;
  size_t gp_floats;
};

// C[M][N] = beta C + A(m,k) B(k,n) over K, split over K when the tiles alone would not fill the chip.
hipError_t gemm(const Ctx& x, const float* A, long long sam, long long sak, const float* Bm, long long sbk,
                long long sbn, float* C, long long ldc, int M, int N, int K, float beta) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int ks = 1;
  if (tiles < 256 && K >= 512) {
    ks = std::min((256 + tiles - 1) / tiles, K / 256);
    ks = std::max(1, std::min<int>(ks, static_cast<int>(x.gp_floats / (static_cast<size_t>(M) * N))));
  }
  GArgs g{A, Bm, C, x.gp, sam, sak, sbk, sbn, ldc, M, N, K, ks, beta};
  gemm_f32_k<<<dim3((N + 63) / 64, (M + 63) / 64, ks), 256, 0, x.st>>>(g);
  if (ks > 1) {
    const size_t n = static_cast<size_t>(M) * N;
    gemm_reduce_k<<<static_cast<unsigned>((n + 255) / 256), 256, 0, x.st>>>(x.gp, C, ldc, M, N, ks, beta);
  }
  return hipGetLastError();
}
// Y[R][N] (+)= X[R][K] W^T for W [N][K]
hipError_t gemm_xwt(const Ctx& x, const float* X, long long ldx, const float* Wm, int N, int K, float* Y,
                    long long ldy, int R, float beta) {
  return gemm(x, X, ldx, 1, Wm, 1, K, Y, ldy, R, N, K, beta);
}
// Y[R][K] (+)= X[R][N] W for W [N][K]
hipError_t gemm_xw(const Ctx& x, const float* X, long long ldx, const float* Wm, int N, int K, float* Y,
                   long long ldy, int R, float beta) {
  return gemm(x, X, ldx, 1, Wm, K, 1, Y, ldy, R, K, N, beta);
}
// G[N][K] += sum_r dOut[r][n] In[r][k]
hipError_t gemm_wgrad(const Ctx& x, const float* dOut, long long ldo, const float* In, long long ldi, float* Gm,
                      int N, int K, int R) {
  return gemm(x, dOut, 1, ldo, In, ldi, 1, Gm, K, N, K, R, 1.0f);
}

hipError_t rms_rows(const Ctx& x, const float* X, long long ldx, const float* g, float* out, long long ldo, int R,
                    int D, float eps) {
  rms_rows_k<<<(R + 3) / 4, 256, 0, x.st>>>(X, ldx, g, out, ldo, R, D, eps);
  return hipGetLastError();
}
// dX += adjoint; the gain gradient (gG) += column sums of dout * n.
hipError_t rms_rows_bwd(const Ctx& x, const float* X, const float* g, const float* dout, float* dX, float* grows,
                        float* colp, float* gG, int R, int D, float eps) {
  rms_bwd_rows_k<<<(R + 3) / 4, 256, 0, x.st>>>(X, D, g, dout, D, dX, D, grows, R, D, eps);
  colsum_part_k<<<dim3((D + 63) / 64, kColChunks), 256, 0, x.st>>>(grows, R, D, colp);
  colsum_fin_k<<<(D + 255) / 256, 256, 0, x.st>>>(colp, D, gG);
  return hipGetLastError();
}

template <int DH>
void launch_enc_attn(int which, const float* QKV, const float* O, const float* dO, float* LSE, float* Dsum, float* out,
                     int B, int T, int H, int D, float scale, hipStream_t st) {
  const dim3 grid((T + 63) / 64, H, B);
  if (which == 0) enc_attn_fwd_k<DH><<<grid, 64, 0, st>>>(QKV, out, LSE, T, H, D, scale);
  else if (which == 1) enc_attn_bwd_q_k<DH><<<grid, 64, 0, st>>>(QKV, O, dO, LSE, Dsum, out, T, H, D, scale);
  else {
    KvArgs k{QKV, 3LL * D, QKV + D, QKV + 2 * D, 3LL * D, dO, D, LSE, Dsum, out + D, out + 2 * D, 3LL * D, T, H, 0,
             scale};
    attn_bwd_kv_k<DH><<<grid, 64, 0, st>>>(k);
  }
}
hipError_t enc_attn(int which, const float* QKV, const float* O, const float* dO, float* LSE, float* Dsum, float* out,
                    int B, int T, int H, int D, hipStream_t st) {
  const int DH = D / H;
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));
  if (DH == 16) launch_enc_attn<16>(which, QKV, O, dO, LSE, Dsum, out, B, T, H, D, scale, st);
  else if (DH == 32) launch_enc_attn<32>(which, QKV, O, dO, LSE, Dsum, out, B, T, H, D, scale, st);
  else launch_enc_attn<64>(which, QKV, O, dO, LSE, Dsum, out, B, T, H, D, scale, st);
  return hipGetLastError();
}

template <int DH>
hipError_t dec_launch_dh(int which, const DecArgs& a, int B, size_t lds, hipStream_t st) {
  const void* fn = which == 0 ? reinterpret_cast<const void*>(&dec_tape_k<DH>)
                              : reinterpret_cast<const void*>(&dec_sweep_k<DH>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  if (which == 0) dec_tape_k<DH><<<B, NT, lds, st>>>(a);
  else dec_sweep_k<DH><<<B, NT, lds, st>>>(a);
  return hipGetLastError();
}
hipError_t dec_launch(int which, int DH, const DecArgs& a, int B, size_t lds, hipStream_t st) {
  if (DH == 16) return dec_launch_dh<16>(which, a, B, lds, st);
  if (DH == 32) return dec_launch_dh<32>(which, a, B, lds, st);
  return dec_launch_dh<64>(which, a, B, lds, st);
}

hipError_t attn_kv(const KvArgs& k, int B, int DH, hipStream_t st) {
  const dim3 grid((k.T + 63) / 64, k.H, B);
  if (DH == 16) attn_bwd_kv_k<16><<<grid, 64, 0, st>>>(k);
  else if (DH == 32) attn_bwd_kv_k<32><<<grid, 64, 0, st>>>(k);
  else attn_bwd_kv_k<64><<<grid, 64, 0, st>>>(k);
  return hipGetLastError();
}

hipError_t transpose(const float* src, float* dst, int N, int K, hipStream_t st) {
  const size_t n = static_cast<size_t>(N) * K;
  transpose_k<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(src, dst, N, K);
  return hipGetLastError();
}

#define BP_TRY(x)                        \
  do {                                   \
    hipError_t err_ = (x);               \
    if (err_ != hipSuccess) return err_; \
  } while (0)

}  // namespace

bool bptt_supported(const rlt_config& c, int B, int T, const char** why) {
  const int DH = c.d_model / c.n_heads;
  if (c.d_model > 256) { *why = "d_model must be <= 256"; return false; }
  if (DH != 16 && DH != 32 && DH != 64) { *why = "head_dim must be 16, 32 or 64"; return false; }
  if (c.ffn_dim > 1024) { *why = "ffn_dim must be <= 1024"; return false; }
  if (c.window > 1024) { *why = "window must be <= 1024"; return false; }
  if (B < 1 || T < 1) { *why = "batch and seq_len must be >= 1"; return false; }
  if (static_cast<long long>(dec_lds_floats(c, T)) * 4 > 160 * 1024) {
    *why = "the decoder sweep's per-sequence vectors (4 (2 H T + 2 H W + ~30 d) bytes) exceed the 160 KB LDS";
    return false;
  }
  return true;
}

size_t bptt_workspace_bytes(const rlt_config& c, int B, int T) { return bp_layout(c, B, T).total * 4; }

hipError_t run_bptt(const rlt_config& c, const BpttOffsets& o, const float* w, const int32_t* tok, const float* mask,
                    int B, int T, int detach, float* grads, float* loss, char* wsb, size_t total_numel,
                    hipStream_t st) {
  const BpLayout lay = bp_layout(c, B, T);
  float* ws = reinterpret_cast<float*>(wsb);
  const int D = c.d_model, H = c.n_heads, L = c.n_layers, F = c.ffn_dim, G = c.mem_groups, V = c.vocab;
  const int swiglu = c.ffn_kind == RLT_FFN_SWIGLU;
  const int F2 = swiglu ? 2 * F : F;
  const int R = B * T;
  const float eps = c.norm_eps;
  const size_t RD = static_cast<size_t>(R) * D, dd = static_cast<size_t>(D) * D, fd = static_cast<size_t>(F) * D;
  Ctx x{st, ws + lay.GP, lay.gp_floats};
  float* gr = grads;

  BP_TRY(launch_zero(grads, total_numel * 4, st));
  BP_TRY(launch_zero(ws + lay.DM, static_cast<size_t>(G) * RD * 2 * 4, st));
  BP_TRY(launch_zero(ws + lay.RING, static_cast<size_t>(L) * B * c.window * 2 * D * 4, st));
  BP_TRY(launch_zero(ws + lay.ERR, 64 * 4, st));

  // transposed copies of the decoder's matrices
  BpttOffsets ot{};
  {
    float* wt = ws + lay.WT;
    size_t p = 0;
    auto tr = [&](int64_t src, int N, int K, int count, int64_t* dst) -> hipError_t {
      *dst = static_cast<int64_t>(p);
      for (int i = 0; i < count; ++i) {
        BP_TRY(transpose(w + src + static_cast<size_t>(i) * N * K, wt + p, N, K, st));
        p += static_cast<size_t>(N) * K;
      }
      return hipSuccess;
    };
    BP_TRY(tr(o.w_ge, D, D, 1, &ot.w_ge));
    BP_TRY(tr(o.w_gs, D, D, 1, &ot.w_gs));
    BP_TRY(tr(o.w_fb, D, D, 1, &ot.w_fb));
    BP_TRY(tr(o.wq, D, D, L, &ot.wq));
    BP_TRY(tr(o.wk, D, D, L, &ot.wk));
    BP_TRY(tr(o.wv, D, D, L, &ot.wv));
    BP_TRY(tr(o.wo, D, D, L, &ot.wo));
    BP_TRY(tr(o.wqx, D, D, L, &ot.wqx));
    BP_TRY(tr(o.wox, D, D, L, &ot.wox));
    BP_TRY(tr(o.f1, F, D, L, &ot.f1));
    BP_TRY(tr(o.f2, swiglu ? F : D, swiglu ? D : F, L, &ot.f2));
    if (swiglu) BP_TRY(tr(o.f3, D, F, L, &ot.f3));
  }

  // 1. encoder forward with the residual stream kept per layer
  float* X = ws + lay.X;
  float* XMID = ws + lay.XMID;
  {
    const size_t n = RD;
    embed_fwd_k<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(tok, w + o.embed, R, D, V, X,
                                                                         reinterpret_cast<int*>(ws + lay.ERR));
    BP_TRY(hipGetLastError());
  }
  for (int l = 0; l < L; ++l) {
    float* xin = X + l * RD;
    float* xmid = XMID + l * RD;
    float* xout = X + (l + 1) * RD;
    BP_TRY(rms_rows(x, xin, D, w + o.g_enc_attn + l * D, ws + lay.HA, D, R, D, eps));
    BP_TRY(gemm_xwt(x, ws + lay.HA, D, w + o.wq + l * dd, D, D, ws + lay.QKV, 3 * D, R, 0.f));
    BP_TRY(gemm_xwt(x, ws + lay.HA, D, w + o.wk + l * dd, D, D, ws + lay.QKV + D, 3 * D, R, 0.f));
    BP_TRY(gemm_xwt(x, ws + lay.HA, D, w + o.wv + l * dd, D, D, ws + lay.QKV + 2 * D, 3 * D, R, 0.f));
    BP_TRY(enc_attn(0, ws + lay.QKV, nullptr, nullptr, ws + lay.LSE, nullptr, ws + lay.O, B, T, H, D, st));
    BP_TRY(launch_copy_f32(xin, xmid, RD, st));
    BP_TRY(gemm_xwt(x, ws + lay.O, D, w + o.wo + l * dd, D, D, xmid, D, R, 1.f));
    BP_TRY(rms_rows(x, xmid, D, w + o.g_enc_ffn + l * D, ws + lay.HF, D, R, D, eps));
    BP_TRY(gemm_xwt(x, ws + lay.HF, D, w + o.f1 + l * fd, F, D, ws + lay.U, F2, R, 0.f));
    if (swiglu) BP_TRY(gemm_xwt(x, ws + lay.HF, D, w + o.f2 + l * fd, F, D, ws + lay.U + F, F2, R, 0.f));
    {
      const size_t n = static_cast<size_t>(R) * F;
      act_fwd_k<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(ws + lay.U, R, F, swiglu, ws + lay.EACT);
      BP_TRY(hipGetLastError());
    }
    BP_TRY(launch_copy_f32(xmid, xout, RD, st));
    BP_TRY(gemm_xwt(x, ws + lay.EACT, F, w + (swiglu ? o.f3 : o.f2) + l * fd, D, F, xout, D, R, 1.f));
  }
  BP_TRY(rms_rows(x, X + L * RD, D, w + o.g_enc_final, ws + lay.E, D, R, D, eps));
  for (int g = 0; g < G; ++g) {
    float* mkv = ws + lay.MKV + static_cast<size_t>(g) * RD * 2;
    BP_TRY(gemm_xwt(x, ws + lay.E, D, w + o.wkm + g * dd, D, D, mkv, 2 * D, R, 0.f));
    BP_TRY(gemm_xwt(x, ws + lay.E, D, w + o.wvm + g * dd, D, D, mkv + D, 2 * D, R, 0.f));
  }

  // 2. decoder tape
  DecArgs a{};
  a.P = w; a.WT = ws + lay.WT; a.o = o; a.ot = ot;
  a.B = B; a.T = T; a.D = D; a.H = H; a.DH = D / H; a.L = L; a.F = F; a.F2 = F2; a.G = G; a.W = c.window;
  a.swiglu = swiglu; a.detach = detach; a.eps = eps; a.scale = 1.0f / sqrtf(static_cast<float>(D / H));
  a.E = ws + lay.E; a.MKV = ws + lay.MKV; a.YT = ws + lay.YT; a.KVT = ws + lay.KVT; a.S = ws + lay.S;
  a.SPREV = ws + lay.SPREV; a.DS = ws + lay.DS;
  a.DQKV = ws + lay.DQKV; a.H1 = ws + lay.H1; a.DY1 = ws + lay.DY1; a.O1 = ws + lay.O1; a.DQX = ws + lay.DQX;
  a.H2 = ws + lay.H2; a.DY2 = ws + lay.DY2; a.O2 = ws + lay.O2; a.DU = ws + lay.DU; a.H3 = ws + lay.H3;
  a.DY3 = ws + lay.DY3; a.ACT = ws + lay.ACT; a.QXS = ws + lay.QXS; a.DO2S = ws + lay.DO2S; a.CLSE = ws + lay.CLSE;
  a.DA = ws + lay.DA; a.DF = ws + lay.DF; a.DE = ws + lay.DE;
  a.DM = ws + lay.DM; a.RING = ws + lay.RING; a.PART = ws + lay.PART;
  const size_t lds = static_cast<size_t>(dec_lds_floats(c, T)) * 4;
  const int DHd = D / H;
  BP_TRY(dec_launch(0, DHd, a, B, lds, st));
  BP_TRY(hipGetLastError());

  // 3. logits, loss, dS and dW_out
  BP_TRY(gemm_xwt(x, ws + lay.S, D, w + o.w_out, V, D, ws + lay.Z, V, R, 0.f));
  ce_rows_k<<<(R + 3) / 4, 256, 0, st>>>(ws + lay.Z, V, tok, mask, B, T, ws + lay.LOSSR);
  BP_TRY(hipGetLastError());
  seq_loss_k<<<(B + 63) / 64, 64, 0, st>>>(ws + lay.LOSSR, B, T, reinterpret_cast<const int*>(ws + lay.ERR), loss);
  BP_TRY(hipGetLastError());
  BP_TRY(gemm_xw(x, ws + lay.Z, V, w + o.w_out, V, D, ws + lay.DS, D, R, 0.f));
  BP_TRY(gemm_wgrad(x, ws + lay.Z, V, ws + lay.S, D, gr + o.w_out, V, D, R));

  // 4. reverse sweep
  BP_TRY(dec_launch(1, DHd, a, B, lds, st));
  BP_TRY(hipGetLastError());
  {
    const int NP = (3 * L + 3) * D;
    const int ng = (3 * L + 1) * D;
    part_reduce_k<<<(ng + 255) / 256, 256, 0, st>>>(ws + lay.PART, B, NP, 0, ng, gr + o.g_dec_self);
    part_reduce_k<<<(D + 255) / 256, 256, 0, st>>>(ws + lay.PART, B, NP, ng, D, gr + o.b_g);
    part_reduce_k<<<(D + 255) / 256, 256, 0, st>>>(ws + lay.PART, B, NP, ng + D, D, gr + o.s_star);
    BP_TRY(hipGetLastError());
  }

  // memory-row adjoints of every layer's cross-attention, token-parallel (queries t attend rows j <= t)
  if (!(detach & 4)) {
    const int DH = D / H;
    for (int l = 0; l < L; ++l) {
      const size_t rl = static_cast<size_t>(l) * R;
      const int g = G == 1 ? 0 : l;
      const size_t n = static_cast<size_t>(B) * H * T;
      head_dots_k<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(ws + lay.DO2S + rl * D, ws + lay.O2 + rl * D,
                                                                            D, B, T, H, DH, ws + lay.DSUM);
      BP_TRY(hipGetLastError());
      const float* mkv = ws + lay.MKV + static_cast<size_t>(g) * RD * 2;
      float* dm = ws + lay.DM + static_cast<size_t>(g) * RD * 2;
      KvArgs k{ws + lay.QXS + rl * D, D, mkv, mkv + D, 2LL * D, ws + lay.DO2S + rl * D, D,
               ws + lay.CLSE + static_cast<size_t>(l) * B * H * T, ws + lay.DSUM, dm, dm + D, 2LL * D, T, H, 1,
               a.scale};
      BP_TRY(attn_kv(k, B, DH, st));
    }
  }

  // 5. decoder weight gradients over all rows
  for (int l = 0; l < L; ++l) {
    const size_t rl = static_cast<size_t>(l) * R;
    const float* dqkv = ws + lay.DQKV + rl * 3 * D;
    const float* h1 = ws + lay.H1 + rl * D;
    BP_TRY(gemm_wgrad(x, dqkv, 3 * D, h1, D, gr + o.wq + l * dd, D, D, R));
    BP_TRY(gemm_wgrad(x, dqkv + D, 3 * D, h1, D, gr + o.wk + l * dd, D, D, R));
    BP_TRY(gemm_wgrad(x, dqkv + 2 * D, 3 * D, h1, D, gr + o.wv + l * dd, D, D, R));
    BP_TRY(gemm_wgrad(x, ws + lay.DY1 + rl * D, D, ws + lay.O1 + rl * D, D, gr + o.wo + l * dd, D, D, R));
    BP_TRY(gemm_wgrad(x, ws + lay.DQX + rl * D, D, ws + lay.H2 + rl * D, D, gr + o.wqx + l * dd, D, D, R));
    BP_TRY(gemm_wgrad(x, ws + lay.DY2 + rl * D, D, ws + lay.O2 + rl * D, D, gr + o.wox + l * dd, D, D, R));
    const float* du = ws + lay.DU + rl * F2;
    const float* h3 = ws + lay.H3 + rl * D;
    BP_TRY(gemm_wgrad(x, du, F2, h3, D, gr + o.f1 + l * fd, F, D, R));
    if (swiglu) BP_TRY(gemm_wgrad(x, du + F, F2, h3, D, gr + o.f2 + l * fd, F, D, R));
    BP_TRY(gemm_wgrad(x, ws + lay.DY3 + rl * D, D, ws + lay.ACT + rl * F, F, gr + (swiglu ? o.f3 : o.f2) + l * fd, D,
                      F, R));
  }
  BP_TRY(gemm_wgrad(x, ws + lay.DF, D, ws + lay.SPREV, D, gr + o.w_fb, D, D, R));
  BP_TRY(gemm_wgrad(x, ws + lay.DA, D, ws + lay.E, D, gr + o.w_ge, D, D, R));
  BP_TRY(gemm_wgrad(x, ws + lay.DA, D, ws + lay.SPREV, D, gr + o.w_gs, D, D, R));
  // memory adjoints back onto e
  float* dE = ws + lay.DE;
  for (int g = 0; g < G; ++g) {
    const float* dm = ws + lay.DM + static_cast<size_t>(g) * RD * 2;
    BP_TRY(gemm_wgrad(x, dm, 2 * D, ws + lay.E, D, gr + o.wkm + g * dd, D, D, R));
    BP_TRY(gemm_wgrad(x, dm + D, 2 * D, ws + lay.E, D, gr + o.wvm + g * dd, D, D, R));
    BP_TRY(gemm_xw(x, dm, 2 * D, w + o.wkm + g * dd, D, D, dE, D, R, 1.f));
    BP_TRY(gemm_xw(x, dm + D, 2 * D, w + o.wvm + g * dd, D, D, dE, D, R, 1.f));
  }

  // 6. encoder backward
  float* dX = ws + lay.DX;
  BP_TRY(launch_zero(dX, RD * 4, st));
  BP_TRY(rms_rows_bwd(x, X + L * RD, w + o.g_enc_final, dE, dX, ws + lay.GROWS, ws + lay.COLP, gr + o.g_enc_final, R,
                      D, eps));
  for (int l = L - 1; l >= 0; --l) {
    float* xin = X + l * RD;
    float* xmid = XMID + l * RD;
    // FFN
    BP_TRY(rms_rows(x, xmid, D, w + o.g_enc_ffn + l * D, ws + lay.HF, D, R, D, eps));
    BP_TRY(gemm_xwt(x, ws + lay.HF, D, w + o.f1 + l * fd, F, D, ws + lay.U, F2, R, 0.f));
    if (swiglu) BP_TRY(gemm_xwt(x, ws + lay.HF, D, w + o.f2 + l * fd, F, D, ws + lay.U + F, F2, R, 0.f));
    const size_t nf = static_cast<size_t>(R) * F;
    act_fwd_k<<<static_cast<unsigned>((nf + 255) / 256), 256, 0, st>>>(ws + lay.U, R, F, swiglu, ws + lay.EACT);
    BP_TRY(hipGetLastError());
    const float* wout = w + (swiglu ? o.f3 : o.f2) + l * fd;
    BP_TRY(gemm_wgrad(x, dX, D, ws + lay.EACT, F, gr + (swiglu ? o.f3 : o.f2) + l * fd, D, F, R));
    BP_TRY(gemm_xw(x, dX, D, wout, D, F, ws + lay.DACT, F, R, 0.f));
    act_bwd_k<<<static_cast<unsigned>((nf + 255) / 256), 256, 0, st>>>(ws + lay.U, ws + lay.DACT, R, F, swiglu,
                                                                        ws + lay.DUE);
    BP_TRY(hipGetLastError());
    BP_TRY(gemm_wgrad(x, ws + lay.DUE, F2, ws + lay.HF, D, gr + o.f1 + l * fd, F, D, R));
    BP_TRY(gemm_xw(x, ws + lay.DUE, F2, w + o.f1 + l * fd, F, D, ws + lay.DHF, D, R, 0.f));
    if (swiglu) {
      BP_TRY(gemm_wgrad(x, ws + lay.DUE + F, F2, ws + lay.HF, D, gr + o.f2 + l * fd, F, D, R));
      BP_TRY(gemm_xw(x, ws + lay.DUE + F, F2, w + o.f2 + l * fd, F, D, ws + lay.DHF, D, R, 1.f));
    }
    BP_TRY(rms_rows_bwd(x, xmid, w + o.g_enc_ffn + l * D, ws + lay.DHF, dX, ws + lay.GROWS, ws + lay.COLP,
                        gr + o.g_enc_ffn + l * D, R, D, eps));
    // attention
    BP_TRY(rms_rows(x, xin, D, w + o.g_enc_attn + l * D, ws + lay.HA, D, R, D, eps));
    BP_TRY(gemm_xwt(x, ws + lay.HA, D, w + o.wq + l * dd, D, D, ws + lay.QKV, 3 * D, R, 0.f));
    BP_TRY(gemm_xwt(x, ws + lay.HA, D, w + o.wk + l * dd, D, D, ws + lay.QKV + D, 3 * D, R, 0.f));
    BP_TRY(gemm_xwt(x, ws + lay.HA, D, w + o.wv + l * dd, D, D, ws + lay.QKV + 2 * D, 3 * D, R, 0.f));
    BP_TRY(enc_attn(0, ws + lay.QKV, nullptr, nullptr, ws + lay.LSE, nullptr, ws + lay.O, B, T, H, D, st));
    BP_TRY(gemm_wgrad(x, dX, D, ws + lay.O, D, gr + o.wo + l * dd, D, D, R));
    BP_TRY(gemm_xw(x, dX, D, w + o.wo + l * dd, D, D, ws + lay.DO, D, R, 0.f));
    BP_TRY(enc_attn(1, ws + lay.QKV, ws + lay.O, ws + lay.DO, ws + lay.LSE, ws + lay.DSUM, ws + lay.DQKVE, B, T, H, D,
                    st));
    BP_TRY(enc_attn(2, ws + lay.QKV, ws + lay.O, ws + lay.DO, ws + lay.LSE, ws + lay.DSUM, ws + lay.DQKVE, B, T, H, D,
                    st));
    const float* dq = ws + lay.DQKVE;
    BP_TRY(gemm_wgrad(x, dq, 3 * D, ws + lay.HA, D, gr + o.wq + l * dd, D, D, R));
    BP_TRY(gemm_wgrad(x, dq + D, 3 * D, ws + lay.HA, D, gr + o.wk + l * dd, D, D, R));
    BP_TRY(gemm_wgrad(x, dq + 2 * D, 3 * D, ws + lay.HA, D, gr + o.wv + l * dd, D, D, R));
    BP_TRY(gemm_xw(x, dq, 3 * D, w + o.wq + l * dd, D, D, ws + lay.DHA, D, R, 0.f));
    BP_TRY(gemm_xw(x, dq + D, 3 * D, w + o.wk + l * dd, D, D, ws + lay.DHA, D, R, 1.f));
    BP_TRY(gemm_xw(x, dq + 2 * D, 3 * D, w + o.wv + l * dd, D, D, ws + lay.DHA, D, R, 1.f));
    BP_TRY(rms_rows_bwd(x, xin, w + o.g_enc_attn + l * D, ws + lay.DHA, dX, ws + lay.GROWS, ws + lay.COLP,
                        gr + o.g_enc_attn + l * D, R, D, eps));
  }
  embed_bwd_k<<<(V + 3) / 4, 256, 0, st>>>(tok, dX, R, D, V, gr + o.embed);
  return hipGetLastError();
}

}  // namespace rlt
