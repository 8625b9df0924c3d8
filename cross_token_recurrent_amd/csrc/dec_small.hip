// Persistent recurrent decoder for small d_model: one workgroup per sequence runs
// every step t0 .. t0+n-1 of its sequence without returning to the host.
//
// Pages: [FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer"
// (decoder-state paragraph; model-hardware co-design principle: the transition is
// sequential within a sequence, ready updates of independent sequences are batched);
// [DS] deepsonar "技术拆解 009｜RLT…" §2.2 (window of W incl. the current token, W-1
// cached entries; cross-attention from the current position only), §2.4 (gated
// feedback of s_{t-1}, final norm gives s_t).
//
// Why this shape on MI355X: at d_model <= 128 a whole decoder layer is a handful of
// 64..256-wide matrix-vector products, so the step is bound by latency, not by HBM or
// MFMA throughput.  Independent sequences never need to synchronise, so each sequence
// gets a workgroup of 8 waves that keeps its window caches, its running state and all
// small vectors in LDS, streams the tied weights (shared by all workgroups, so they stay
// L2-resident) and its own encoder memory rows, and synchronises only with s_barrier.
//
// Per step (bf16 mode: matrix-product operands are rounded to bf16, accumulation,
// residual stream, softmax and s_t stay fp32):
//   merge:  g = sigmoid(W_ge e_t + W_gs s + b_g), f = W_fb s, y = g*e_t + (1-g)*f
//   per layer: SWA over ring + current entry -> W_O; cross-attention over memory
//              entries 0..t (two passes: scores + max, then exp-weighted values) -> W_Ox;
//              FFN; each sub-block pre-RMSNorm with its own gain, residual add.
//   s_t = RMSNorm(y; g_dec_final).
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int NT = 512;          // threads per workgroup (8 waves)
constexpr int NG = NT / 8;       // 8-lane groups for matrix-vector products

struct DecSmallParams {
  const void* wgate;   // [D, 2D]
  const void* wfb;     // [D, D]
  const float* bg;     // [D]
  const char* layers;  // layer blocks
  size_t layer_stride, l_qkv, l_wo, l_wqx, l_wox, l_fin, l_fout;
  const float* g_self;   // [L][D]
  const float* g_cross;  // [L][D]
  const float* g_ffn;    // [L][D]
  const float* g_final;  // [D]
  float* s;              // [B][D]
  void* ring_k;          // [L][B][H][Wm1][DH]
  void* ring_v;
  const void* e;         // [B][T][D]
  const void* mem_k;     // [G][B][H][T][DH]
  const void* mem_v;
  float* s_out;          // [B][n][D] or null
  int B, T, t0, n, L, F, F2, Wm1, G, ffn_kind;
  float eps;
};

// y[r] <- epi(r, W[r,:] . x) for r in [0, N): 8 lanes per row, each lane a 64-element
// stride of 8-element chunks; x is an fp32 LDS vector of length K (K % 64 == 0).
template <typename WT, typename Epi>
__device__ __forceinline__ void matvec(const WT* __restrict__ W, int N, int K, const float* __restrict__ x,
                                       Epi epi) {
  const int sub = threadIdx.x & 7;
  const int grp = threadIdx.x >> 3;
  for (int r = grp; r < N; r += NG) {
    const WT* row = W + static_cast<size_t>(r) * K;
    float acc = 0.f;
#pragma unroll 4
    for (int k = sub * 8; k < K; k += 64) {
      float w[8];
      load8(row + k, w);
      const float4 x0 = *reinterpret_cast<const float4*>(x + k);
      const float4 x1 = *reinterpret_cast<const float4*>(x + k + 4);
      acc += w[0] * x0.x + w[1] * x0.y + w[2] * x0.z + w[3] * x0.w + w[4] * x1.x + w[5] * x1.y + w[6] * x1.z +
             w[7] * x1.w;
    }
    acc = group_sum<8>(acc);
    if (sub == 0) epi(r, acc);
  }
}

// dst[c] = round_to<WT>(gain[c] * y[c] / rms(y)) for c < D.  Every wave computes the
// statistic itself (D <= 128 values from LDS), so no extra barrier is needed.
template <typename WT, int D>
__device__ __forceinline__ void rmsnorm_to(const float* __restrict__ y, const float* __restrict__ gain,
                                           float* __restrict__ dst, float eps, bool round_operand) {
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int c = lane; c < D; c += 64) ss += y[c] * y[c];
  ss = group_sum<64>(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  for (int c = threadIdx.x; c < D; c += NT) {
    const float v = gain[c] * (y[c] * inv);
    dst[c] = round_operand ? round_to<WT>(v) : v;
  }
}

template <typename WT, int D, int DH>
__global__ __launch_bounds__(NT) void dec_small_k(DecSmallParams p) {
  constexpr int H = D / DH;
  constexpr int LPK = DH / 8;            // lanes per memory row (8 elements each)
  constexpr int PARTS = NT / (H * LPK);  // key slices per head in cross-attention
  static_assert(PARTS >= 8 && PARTS % 8 == 0, "cross-attention partition");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = p.L, Wm1 = p.Wm1, T = p.T, F = p.F, F2 = p.F2;
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));

  // ---- LDS carve-up ----
  WT* ringK = reinterpret_cast<WT*>(smem);                       // [L][H][Wm1][DH]
  const size_t ring_elems = static_cast<size_t>(L) * H * Wm1 * DH;
  WT* ringV = ringK + ring_elems;
  float* fbase = reinterpret_cast<float*>(smem + ((2 * ring_elems * sizeof(WT) + 15) / 16) * 16);
  float* y = fbase;                 // [D]   residual stream
  float* xin = y + D;               // [2D]  operand vector (merge input [e; s], normed input)
  float* s_l = xin + 2 * D;         // [D]   s_{t-1} / s_t
  float* qkv = s_l + D;             // [3D]
  float* attn = qkv + 3 * D;        // [D]
  float* gpre = attn + D;           // [D]
  float* fb = gpre + D;             // [D]
  float* red = fb + D;              // [64]
  float* act = red + 64;            // [F2]  FFN activation (and raw gate/up for SwiGLU)
  float* act2 = act + F2;           // [F]
  float* part_o = act2 + F;         // [H][PARTS][DH]
  float* part_l = part_o + H * PARTS * DH;  // [H][PARTS]
  float* sc = part_l + H * PARTS;   // [H][T] cross-attention scores

  // ---- load the carried state: window caches and s ----
  {
    const WT* gk = static_cast<const WT*>(p.ring_k);
    const WT* gv = static_cast<const WT*>(p.ring_v);
    const size_t per_lb = static_cast<size_t>(H) * Wm1 * DH;
    for (int l = 0; l < L; ++l) {
      const size_t src = (static_cast<size_t>(l) * p.B + b) * per_lb;
      for (size_t i = tid; i < per_lb; i += NT) {
        ringK[l * per_lb + i] = gk[src + i];
        ringV[l * per_lb + i] = gv[src + i];
      }
    }
    for (int c = tid; c < D; c += NT) s_l[c] = p.s[static_cast<size_t>(b) * D + c];
  }
  __syncthreads();

  const WT* e_seq = static_cast<const WT*>(p.e) + static_cast<size_t>(b) * T * D;
  const WT* wgate = static_cast<const WT*>(p.wgate);
  const WT* wfb = static_cast<const WT*>(p.wfb);

  for (int step = 0; step < p.n; ++step) {
    const int t = p.t0 + step;   // 0-based position of this transition

    // ---- gated merge of e_t with s_{t-1} ----
    for (int c = tid; c < D; c += NT) {
      xin[c] = load_as_f32(e_seq + static_cast<size_t>(t) * D + c);
      xin[D + c] = round_to<WT>(s_l[c]);
    }
    __syncthreads();
    matvec<WT>(wgate, D, 2 * D, xin, [&](int r, float v) { gpre[r] = v + p.bg[r]; });
    matvec<WT>(wfb, D, D, xin + D, [&](int r, float v) { fb[r] = v; });
    __syncthreads();
    for (int c = tid; c < D; c += NT) {
      const float g = sigmoid_f(gpre[c]);
      y[c] = g * xin[c] + (1.0f - g) * fb[c];
    }
    __syncthreads();

    for (int l = 0; l < L; ++l) {
      const char* lw = p.layers + l * p.layer_stride;
      const WT* wqkv = reinterpret_cast<const WT*>(lw + p.l_qkv);
      const WT* wo = reinterpret_cast<const WT*>(lw + p.l_wo);
      const WT* wqx = reinterpret_cast<const WT*>(lw + p.l_wqx);
      const WT* wox = reinterpret_cast<const WT*>(lw + p.l_wox);
      const WT* wfin = reinterpret_cast<const WT*>(lw + p.l_fin);
      const WT* wfout = reinterpret_cast<const WT*>(lw + p.l_fout);
      WT* rK = ringK + static_cast<size_t>(l) * H * Wm1 * DH;
      WT* rV = ringV + static_cast<size_t>(l) * H * Wm1 * DH;

      // ---- sliding-window self-attention ----
      rmsnorm_to<WT, D>(y, p.g_self + l * D, xin, p.eps, true);
      __syncthreads();
      matvec<WT>(wqkv, 3 * D, D, xin, [&](int r, float v) { qkv[r] = r < D ? v : round_to<WT>(v); });
      __syncthreads();
      const int npast = min(t, Wm1);        // cached entries in the window
      const int ne = npast + 1;             // plus the current token
      for (int idx = tid; idx < H * ne; idx += NT) {
        const int h = idx / ne, i = idx % ne;
        const float* q = qkv + h * DH;
        float acc = 0.f;
        if (i < npast) {
          const int slot = (t - npast + i) % Wm1;
          const WT* kr = rK + (static_cast<size_t>(h) * Wm1 + slot) * DH;
#pragma unroll
          for (int c = 0; c < DH; ++c) acc += q[c] * load_as_f32(kr + c);
        } else {
          const float* kr = qkv + D + h * DH;
#pragma unroll
          for (int c = 0; c < DH; ++c) acc += q[c] * kr[c];
        }
        sc[h * T + i] = acc * scale;
      }
      __syncthreads();
      for (int idx = tid; idx < D; idx += NT) {
        const int h = idx / DH, c = idx % DH;
        const float* sh = sc + h * T;
        float m = -INFINITY;
        for (int i = 0; i < ne; ++i) m = fmaxf(m, sh[i]);
        float sum = 0.f, o = 0.f;
        for (int i = 0; i < ne; ++i) {
          const float w = expf(sh[i] - m);
          sum += w;
          float v;
          if (i < npast) {
            const int slot = (t - npast + i) % Wm1;
            v = load_as_f32(rV + (static_cast<size_t>(h) * Wm1 + slot) * DH + c);
          } else {
            v = qkv[2 * D + h * DH + c];
          }
          o += w * v;
        }
        attn[idx] = round_to<WT>(o / sum);
      }
      __syncthreads();
      // the current entry replaces the oldest one (position t - (W-1)), after all reads above
      if (Wm1 > 0) {
        const int slot = t % Wm1;
        WT* gk = static_cast<WT*>(p.ring_k) + (static_cast<size_t>(l) * p.B + b) * H * Wm1 * DH;
        WT* gv = static_cast<WT*>(p.ring_v) + (static_cast<size_t>(l) * p.B + b) * H * Wm1 * DH;
        for (int idx = tid; idx < D; idx += NT) {
          const int h = idx / DH, c = idx % DH;
          const size_t o = (static_cast<size_t>(h) * Wm1 + slot) * DH + c;
          WT kq, vq;
          store_from_f32(&kq, qkv[D + idx]);
          store_from_f32(&vq, qkv[2 * D + idx]);
          rK[o] = kq;
          rV[o] = vq;
          gk[o] = kq;
          gv[o] = vq;
        }
      }
      matvec<WT>(wo, D, D, attn, [&](int r, float v) { y[r] += v; });
      __syncthreads();

      // ---- cross-attention to memory entries 0..t ----
      rmsnorm_to<WT, D>(y, p.g_cross + l * D, xin, p.eps, true);
      __syncthreads();
      matvec<WT>(wqx, D, D, xin, [&](int r, float v) { qkv[r] = v * scale; });
      __syncthreads();
      {
        const int g = p.G == 1 ? 0 : l;
        const int h = tid / (PARTS * LPK);
        const int part = (tid / LPK) % PARTS;
        const int sub = tid % LPK;
        const size_t head_off = ((static_cast<size_t>(g) * p.B + b) * H + h) * static_cast<size_t>(T) * DH;
        const WT* mk = static_cast<const WT*>(p.mem_k) + head_off + sub * 8;
        const WT* mv = static_cast<const WT*>(p.mem_v) + head_off + sub * 8;
        float q8[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) q8[c] = qkv[h * DH + sub * 8 + c];
        // pass 1: scores and the per-head maximum
        float mloc = -INFINITY;
        for (int j = part; j <= t; j += PARTS) {
          float kv[8];
          load8(mk + static_cast<size_t>(j) * DH, kv);
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) acc += q8[c] * kv[c];
          acc = group_sum<LPK>(acc);
          if (sub == 0) sc[h * T + j] = acc;
          mloc = fmaxf(mloc, acc);
        }
        mloc = group_max<64>(mloc);   // a wave covers one head (64 | PARTS*LPK)
        if ((tid & 63) == 0) red[tid >> 6] = mloc;
        __syncthreads();
        constexpr int WPH = PARTS * LPK / 64;  // waves per head
        float mh = red[h * WPH];
#pragma unroll
        for (int w = 1; w < WPH; ++w) mh = fmaxf(mh, red[h * WPH + w]);
        // pass 2: exp-weighted values
        float o8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
        for (int j = part; j <= t; j += PARTS) {
          const float w = expf(sc[h * T + j] - mh);
          float vv[8];
          load8(mv + static_cast<size_t>(j) * DH, vv);
          lsum += w;
#pragma unroll
          for (int c = 0; c < 8; ++c) o8[c] += w * vv[c];
        }
        float* po = part_o + (static_cast<size_t>(h) * PARTS + part) * DH + sub * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) po[c] = o8[c];
        if (sub == 0) part_l[h * PARTS + part] = lsum;
      }
      __syncthreads();
      // combine the PARTS partial sums of every (head, dim) in a fixed order
      for (int idx = tid; idx < D * 8; idx += NT) {
        const int k = idx & 7, hc = idx >> 3;
        const int h = hc / DH, c = hc % DH;
        float o = 0.f, l_ = 0.f;
        for (int q = k; q < PARTS; q += 8) {
          o += part_o[(static_cast<size_t>(h) * PARTS + q) * DH + c];
          l_ += part_l[h * PARTS + q];
        }
        o = group_sum<8>(o);
        l_ = group_sum<8>(l_);
        if (k == 0) attn[hc] = round_to<WT>(o / l_);
      }
      __syncthreads();
      matvec<WT>(wox, D, D, attn, [&](int r, float v) { y[r] += v; });
      __syncthreads();

      // ---- FFN (tied with encoder layer l) ----
      rmsnorm_to<WT, D>(y, p.g_ffn + l * D, xin, p.eps, true);
      __syncthreads();
      if (p.ffn_kind == RLT_FFN_GELU) {
        matvec<WT>(wfin, F, D, xin, [&](int r, float v) { act[r] = round_to<WT>(gelu_erf(v)); });
        __syncthreads();
        matvec<WT>(wfout, D, F, act, [&](int r, float v) { y[r] += v; });
      } else {
        matvec<WT>(wfin, F2, D, xin, [&](int r, float v) { act[r] = v; });
        __syncthreads();
        for (int i = tid; i < F; i += NT) {
          const int gr = (i / 16) * 32 + i % 16;
          act2[i] = round_to<WT>(silu_f(act[gr]) * act[gr + 16]);
        }
        __syncthreads();
        matvec<WT>(wfout, D, F, act2, [&](int r, float v) { y[r] += v; });
      }
      __syncthreads();
    }

    // ---- s_t = RMSNorm(y; g_dec_final) ----
    rmsnorm_to<WT, D>(y, p.g_final, s_l, p.eps, false);
    __syncthreads();
    if (p.s_out) {
      float* so = p.s_out + (static_cast<size_t>(b) * p.n + step) * D;
      for (int c = tid; c < D; c += NT) so[c] = s_l[c];
    }
  }
  for (int c = tid; c < D; c += NT) p.s[static_cast<size_t>(b) * D + c] = s_l[c];
}

template <int D, int DH>
constexpr int parts_for() {
  return NT / ((D / DH) * (DH / 8));
}

size_t lds_bytes(const ModelLayout& m, int T) {
  const size_t H = m.H, DH = m.DH, D = m.D;
  const size_t ring = 2 * static_cast<size_t>(m.L) * H * (m.W - 1) * DH * m.esz;
  const size_t parts = NT / (H * (DH / 8));
  const size_t floats = D + 2 * D + D + 3 * D + D + D + D + 64 + m.F2 + m.F + H * parts * DH + H * parts +
                        H * static_cast<size_t>(T);
  return (ring + 15) / 16 * 16 + floats * 4;
}

template <typename WT, int D, int DH>
hipError_t launch_t(const ModelLayout& m, const StateLayout& s, const DecSmallArgs& a, hipStream_t st) {
  DecSmallParams p{};
  p.wgate = a.ws + m.wgate;
  p.wfb = a.ws + m.wfb;
  p.bg = reinterpret_cast<const float*>(a.ws + m.bg);
  p.layers = a.ws + m.layers;
  p.layer_stride = m.layer_stride;
  p.l_qkv = m.l_qkv; p.l_wo = m.l_wo; p.l_wqx = m.l_wqx; p.l_wox = m.l_wox; p.l_fin = m.l_fin; p.l_fout = m.l_fout;
  p.g_self = reinterpret_cast<const float*>(a.ws + m.g_dec_self);
  p.g_cross = reinterpret_cast<const float*>(a.ws + m.g_dec_cross);
  p.g_ffn = reinterpret_cast<const float*>(a.ws + m.g_dec_ffn);
  p.g_final = reinterpret_cast<const float*>(a.ws + m.g_dec_final);
  p.s = reinterpret_cast<float*>(a.state + s.s);
  p.ring_k = a.state + s.ring_k;
  p.ring_v = a.state + s.ring_v;
  p.e = a.state + s.e;
  p.mem_k = a.state + s.mem_k;
  p.mem_v = a.state + s.mem_v;
  p.s_out = a.s_out;
  p.B = a.B; p.T = a.T; p.t0 = a.t0; p.n = a.n; p.L = m.L; p.F = m.F; p.F2 = m.F2; p.Wm1 = m.W - 1; p.G = m.G;
  p.ffn_kind = m.ffn_kind; p.eps = m.eps;
  const size_t lds = lds_bytes(m, a.T);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dec_small_k<WT, D, DH>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  dec_small_k<WT, D, DH><<<a.B, NT, lds, st>>>(p);
  return hipGetLastError();
}

}  // namespace

constexpr size_t kMaxLds = 160 * 1024;

bool dec_small_supported(const ModelLayout& m, int T) {
  const bool shape = (m.D == 64 && (m.DH == 16 || m.DH == 32 || m.DH == 64)) ||
                     (m.D == 128 && (m.DH == 16 || m.DH == 32 || m.DH == 64 || m.DH == 128));
  return shape && m.F2 <= 2048 && lds_bytes(m, T) <= kMaxLds;
}

size_t dec_small_lds_bytes(const ModelLayout& m, int T) { return lds_bytes(m, T); }

hipError_t launch_dec_small(const ModelLayout& m, const StateLayout& s, const DecSmallArgs& a, hipStream_t st) {
  if (!dec_small_supported(m, a.T)) return hipErrorInvalidValue;
  const bool bf = m.dtype == RLT_DTYPE_BF16;
#define RLT_DEC_CASE(D_, DH_)                                                            \
  if (m.D == D_ && m.DH == DH_)                                                          \
    return bf ? launch_t<bf16_t, D_, DH_>(m, s, a, st) : launch_t<float, D_, DH_>(m, s, a, st);
  RLT_DEC_CASE(64, 16)
  RLT_DEC_CASE(64, 32)
  RLT_DEC_CASE(64, 64)
  RLT_DEC_CASE(128, 16)
  RLT_DEC_CASE(128, 32)
  RLT_DEC_CASE(128, 64)
  RLT_DEC_CASE(128, 128)
#undef RLT_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace rlt
