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
// Why this shape on MI355X: at d_model <= 128 a decoder layer is a handful of 64..256-wide
// matrix-vector products and two single-query attentions, so a step is bound by VALU issue
// and latency, not by HBM or MFMA throughput.  Independent sequences never synchronise,
// so each sequence gets one workgroup of 4 waves (one per SIMD) that keeps its window
// caches, running state, gains and small vectors in LDS.  The design keeps the number of
// wave instructions per step low and the latency hidden:
//   * matrix-vector products: 8-lane groups per row, weights for the next product
//     prefetched into registers one phase ahead (s_barrier does not wait for global
//     loads), RMSNorm fused into the product's operand fetch;
//   * both attentions run one head per wave with lanes over keys; partial softmax states
//     are combined inside the wave through LDS (no workgroup barrier);
//   * cross-attention streams memory rows with batched loads requested two batches ahead,
//     the first two batches issued two phases before they are needed.
// bf16 mode: matrix-product operands are packed bf16 in LDS and consumed with
// v_dot2c_f32_bf16 (exact bf16 products, fp32 accumulation); the query is split into
// bf16 hi + lo parts for the score dot products, so attention math keeps ~fp32 accuracy;
// the residual stream, softmax statistics and s_t stay fp32.
#include <algorithm>

#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int NT = 256;          // threads per workgroup (4 waves, one per SIMD)
constexpr int NWAVE = NT / 64;
constexpr int NG = NT / 8;       // 8-lane groups for matrix-vector products
constexpr int CMAX = 8;          // prefetched (row, chunk) pairs per lane and product
constexpr int WCAP = 256;        // largest window (entries held at once) supported

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- storage-type operations on 8-element chunks -----------------------------------
template <typename WT> struct Ops;

template <> struct Ops<bf16_t> {
  struct Chunk { uint4 v; };
  static __device__ __forceinline__ Chunk load(const bf16_t* p) { return {*reinterpret_cast<const uint4*>(p)}; }
  static __device__ __forceinline__ Chunk zero() { return {make_uint4(0u, 0u, 0u, 0u)}; }
  static __device__ __forceinline__ Chunk pack(const float (&f)[8]) {
    return {make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                       pack_bf16x2(f[6], f[7]))};
  }
  static __device__ __forceinline__ float d2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
  }
  static __device__ __forceinline__ float dot(const Chunk& w, const Chunk& x, float acc) {
    acc = d2(w.v.x, x.v.x, acc);
    acc = d2(w.v.y, x.v.y, acc);
    acc = d2(w.v.z, x.v.z, acc);
    return d2(w.v.w, x.v.w, acc);
  }
  static __device__ __forceinline__ void unpack(const Chunk& c, float (&f)[8]) {
    const uint32_t w[4] = {c.v.x, c.v.y, c.v.z, c.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <> struct Ops<float> {
  struct Chunk { float4 a, b; };
  static __device__ __forceinline__ Chunk load(const float* p) {
    return {*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  static __device__ __forceinline__ Chunk zero() {
    return {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  }
  static __device__ __forceinline__ Chunk pack(const float (&f)[8]) {
    return {make_float4(f[0], f[1], f[2], f[3]), make_float4(f[4], f[5], f[6], f[7])};
  }
  static __device__ __forceinline__ float dot(const Chunk& w, const Chunk& x, float acc) {
    acc += w.a.x * x.a.x; acc += w.a.y * x.a.y; acc += w.a.z * x.a.z; acc += w.a.w * x.a.w;
    acc += w.b.x * x.b.x; acc += w.b.y * x.b.y; acc += w.b.z * x.b.z; acc += w.b.w * x.b.w;
    return acc;
  }
  static __device__ __forceinline__ void unpack(const Chunk& c, float (&f)[8]) {
    f[0] = c.a.x; f[1] = c.a.y; f[2] = c.a.z; f[3] = c.a.w;
    f[4] = c.b.x; f[5] = c.b.y; f[6] = c.b.z; f[7] = c.b.w;
  }
};

// A 16-element query slice, prepared for dot products with 16-element key rows.
template <typename WT> struct QSlice;
template <> struct QSlice<bf16_t> {
  uint32_t hi[8], lo[8];   // q = hi + lo, both bf16 pairs (~16 significant bits)
  // qf: fp32 query (unused); qh / ql: bf16 hi and lo halves, 16 elements each
  __device__ __forceinline__ void set(const float* qf, const bf16_t* qh, const bf16_t* ql) {
    (void)qf;
    const uint4 h0 = *reinterpret_cast<const uint4*>(qh), h1 = *reinterpret_cast<const uint4*>(qh + 8);
    const uint4 l0 = *reinterpret_cast<const uint4*>(ql), l1 = *reinterpret_cast<const uint4*>(ql + 8);
    hi[0] = h0.x; hi[1] = h0.y; hi[2] = h0.z; hi[3] = h0.w; hi[4] = h1.x; hi[5] = h1.y; hi[6] = h1.z; hi[7] = h1.w;
    lo[0] = l0.x; lo[1] = l0.y; lo[2] = l0.z; lo[3] = l0.w; lo[4] = l1.x; lo[5] = l1.y; lo[6] = l1.z; lo[7] = l1.w;
  }
  __device__ __forceinline__ float dot(const Ops<bf16_t>::Chunk& k0, const Ops<bf16_t>::Chunk& k1) const {
    const uint32_t kv[8] = {k0.v.x, k0.v.y, k0.v.z, k0.v.w, k1.v.x, k1.v.y, k1.v.z, k1.v.w};
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = Ops<bf16_t>::d2(kv[i], lo[i], a);
#pragma unroll
    for (int i = 0; i < 8; ++i) b = Ops<bf16_t>::d2(kv[i], hi[i], b);
    return a + b;
  }
};
template <> struct QSlice<float> {
  float q[16];
  __device__ __forceinline__ void set(const float* src, const float* qh, const float* ql) {
    (void)qh;
    (void)ql;
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = src[i];
  }
  __device__ __forceinline__ float dot(const Ops<float>::Chunk& k0, const Ops<float>::Chunk& k1) const {
    return q[0] * k0.a.x + q[1] * k0.a.y + q[2] * k0.a.z + q[3] * k0.a.w + q[4] * k0.b.x + q[5] * k0.b.y +
           q[6] * k0.b.z + q[7] * k0.b.w + q[8] * k1.a.x + q[9] * k1.a.y + q[10] * k1.a.z + q[11] * k1.a.w +
           q[12] * k1.b.x + q[13] * k1.b.y + q[14] * k1.b.z + q[15] * k1.b.w;
  }
};

// o[0..16) += w * v (v = two 8-element chunks)
template <typename WT>
__device__ __forceinline__ void axpy16(float (&o)[16], float w, const typename Ops<WT>::Chunk& v0,
                                       const typename Ops<WT>::Chunk& v1) {
  float f[8];
  Ops<WT>::unpack(v0, f);
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] += w * f[c];
  Ops<WT>::unpack(v1, f);
#pragma unroll
  for (int c = 0; c < 8; ++c) o[8 + c] += w * f[c];
}

// ---- matrix-vector products out[r] = W[r,:] . x ----------------------------------------
// Lane (grp, sub) owns rows grp, grp+NG, ... and the 8-element chunks sub*8 + 64*c of each
// row; (row, chunk) pairs are enumerated row-major.  The first CMAX pairs are loaded into
// registers ahead of time (wprefetch); the rest, if any, are loaded when needed.
template <typename WT> struct WBuf { typename Ops<WT>::Chunk c[CMAX]; };

template <typename WT>
__device__ __forceinline__ void wprefetch(WBuf<WT>& buf, const WT* __restrict__ W, int N, int K) {
  const int sub = threadIdx.x & 7, grp = threadIdx.x >> 3;
  const int cpl = K >> 6;
#pragma unroll
  for (int p = 0; p < CMAX; ++p) {
    const int ri = p / cpl, ci = p - ri * cpl;
    const int r = min(grp + ri * NG, N - 1);   // rows past N are loaded but never used
    buf.c[p] = Ops<WT>::load(W + static_cast<size_t>(r) * K + sub * 8 + ci * 64);
  }
}

// K = CPL * 64 with CPL <= CMAX: the lane's operand chunks are computed once (xr) and the
// first CMAX / CPL rows come from the prefetched buffer.
template <int CPL, typename WT, typename XF, typename Epi>
__device__ __forceinline__ void wcompute_c(const WBuf<WT>& buf, const WT* __restrict__ W, int N, XF&& xf,
                                           Epi&& epi) {
  using O = Ops<WT>;
  constexpr int K = CPL * 64;
  constexpr int RB = CMAX / CPL;
  const int sub = threadIdx.x & 7, grp = threadIdx.x >> 3;
  typename O::Chunk xr[CPL];
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) xr[ci] = xf(sub * 8 + ci * 64);
  const int nrows = (N + NG - 1) / NG;
  // every lane of the 8-lane group gets every row total; lane `sub` then runs the epilogue
  // of row `sub`, so each epilogue is executed once per row, not once per group lane
  float mine = 0.f;
#pragma unroll
  for (int ri = 0; ri < RB; ++ri) {
    if (ri < nrows) {
      float acc = 0.f;
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci) acc = O::dot(buf.c[ri * CPL + ci], xr[ci], acc);
      acc = group_sum<8>(acc);
      mine = sub == ri ? acc : mine;
    }
  }
  {
    const int r = grp + sub * NG;
    if (sub < RB && sub < nrows && r < N) epi(r, mine);
  }
  for (int ri = RB; ri < nrows; ++ri) {
    const int r = grp + ri * NG;
    float acc = 0.f;
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
      const typename O::Chunk w = O::load(W + static_cast<size_t>(min(r, N - 1)) * K + sub * 8 + ci * 64);
      acc = O::dot(w, xr[ci], acc);
    }
    acc = group_sum<8>(acc);
    if (sub == 0 && r < N) epi(r, acc);
  }
}

// Any K (multiple of 64): every chunk loaded when needed.
template <typename WT, typename XF, typename Epi>
__device__ __forceinline__ void wcompute_any(const WT* __restrict__ W, int N, int K, XF&& xf, Epi&& epi) {
  using O = Ops<WT>;
  const int sub = threadIdx.x & 7, grp = threadIdx.x >> 3;
  for (int r0 = grp; r0 < ((N + NG - 1) / NG) * NG; r0 += NG) {
    float acc = 0.f;
    for (int k = sub * 8; k < K; k += 64) {
      const typename O::Chunk w = r0 < N ? O::load(W + static_cast<size_t>(r0) * K + k) : O::zero();
      acc = O::dot(w, xf(k), acc);
    }
    acc = group_sum<8>(acc);
    if (sub == 0 && r0 < N) epi(r0, acc);
  }
}

template <typename WT, typename XF, typename Epi>
__device__ __forceinline__ void wcompute(const WBuf<WT>& buf, const WT* __restrict__ W, int N, int K, XF&& xf,
                                         Epi&& epi) {
  switch (K >> 6) {
    case 1: wcompute_c<1>(buf, W, N, xf, epi); break;
    case 2: wcompute_c<2>(buf, W, N, xf, epi); break;
    case 3: wcompute_c<3>(buf, W, N, xf, epi); break;
    case 4: wcompute_c<4>(buf, W, N, xf, epi); break;
    case 8: wcompute_c<8>(buf, W, N, xf, epi); break;
    default: wcompute_any(W, N, K, xf, epi); break;
  }
}

// 1 / rms(y) over D values in LDS, computed by every wave on its own.
template <int D>
__device__ __forceinline__ float wave_rms_inv(const float* __restrict__ y, float eps) {
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int c = lane; c < D; c += 64) ss += y[c] * y[c];
  ss = group_sum<64>(ss);
  return 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
}

// Operand chunk k..k+8 of RMS(y; g) in the storage precision.
template <typename WT>
__device__ __forceinline__ typename Ops<WT>::Chunk norm_chunk(const float* __restrict__ y,
                                                              const float* __restrict__ g, float inv, int k) {
  const float4 y0 = *reinterpret_cast<const float4*>(y + k), y1 = *reinterpret_cast<const float4*>(y + k + 4);
  const float4 g0 = *reinterpret_cast<const float4*>(g + k), g1 = *reinterpret_cast<const float4*>(g + k + 4);
  const float f[8] = {g0.x * (y0.x * inv), g0.y * (y0.y * inv), g0.z * (y0.z * inv), g0.w * (y0.w * inv),
                      g1.x * (y1.x * inv), g1.y * (y1.y * inv), g1.z * (y1.z * inv), g1.w * (y1.w * inv)};
  return Ops<WT>::pack(f);
}

// Inside one wave: lanes hold partial softmax states (m, l, o[16]) for the 16 dims starting
// at dim 16*sub of one head (sub = lane % LPK).  Writes o / l (DH dims) to dst.
// wbuf: this wave's LDS scratch of 64*17 + 64 floats.
template <typename WT, int DH>
__device__ __forceinline__ void wave_combine(float m, float l, float (&o)[16], float* __restrict__ wbuf,
                                             WT* __restrict__ dst) {
  constexpr int LPK = DH / 16;
  constexpr int SLOTS = 64 / LPK;
  const int lane = threadIdx.x & 63;
  const float mw = group_max<64>(m);
  const float f = __expf(m - mw);   // lanes without keys: m = -inf -> 0
  float* ob = wbuf;                 // [64][17]
  float* lb = wbuf + 64 * 17;       // [64]
#pragma unroll
  for (int c = 0; c < 16; ++c) ob[lane * 17 + c] = o[c] * f;
  lb[lane] = l * f;
  wave_sync_lds();
  if constexpr (DH <= 64) {
    constexpr int GS = 64 / DH;     // slot groups per dim
    const int d = lane % DH, g = lane / DH;
    const int sub = d / 16, c = d % 16;
    constexpr int PER = SLOTS / GS;
    float acc = 0.f, lacc = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int s = g + GS * k;
      acc += ob[(s * LPK + sub) * 17 + c];
      lacc += lb[s * LPK];
    }
#pragma unroll
    for (int off = DH; off < 64; off <<= 1) {
      acc += __shfl_xor(acc, off, 64);
      lacc += __shfl_xor(lacc, off, 64);
    }
    if (g == 0) store_from_f32(&dst[d], acc / lacc);
  } else {
#pragma unroll
    for (int d = lane; d < DH; d += 64) {
      const int sub = d / 16, c = d % 16;
      float acc = 0.f, lacc = 0.f;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        acc += ob[(s * LPK + sub) * 17 + c];
        lacc += lb[s * LPK];
      }
      store_from_f32(&dst[d], acc / lacc);
    }
  }
  wave_sync_lds();
}

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

template <typename WT, int D, int DH>
__global__ __launch_bounds__(NT) void dec_small_k(DecSmallParams p) {
  using O = Ops<WT>;
  using Chunk = typename O::Chunk;
  constexpr int H = D / DH;
  constexpr int LPK = DH / 16;            // lanes per key row (16 elements each)
  constexpr int SLOTS = 64 / LPK;         // keys per wave pass
  constexpr int KQ = sizeof(WT) == 2 ? 4 : 2;   // memory rows per lane per load batch
  constexpr int NSC = 16;                        // scores per lane per chunk
  static_assert(DH % 16 == 0 && DH <= 128, "head width");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int slot = lane / LPK, sub = lane % LPK;
  const int L = p.L, Wm1 = p.Wm1, T = p.T, F = p.F, F2 = p.F2, G = p.G;
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));
  const int XOPN = 2 * D > F ? 2 * D : F;

  // ---- LDS carve-up ----
  WT* ringK = reinterpret_cast<WT*>(smem);                       // [L][H][Wm1][DH]
  const size_t ring_elems = static_cast<size_t>(L) * H * Wm1 * DH;
  WT* ringV = ringK + ring_elems;
  unsigned char* cur = smem + ((2 * ring_elems * sizeof(WT) + 15) / 16) * 16;
  WT* xop = reinterpret_cast<WT*>(cur);                 // operand vector [max(2D, F)]
  cur += ((XOPN * sizeof(WT) + 15) / 16) * 16;
  float* y = reinterpret_cast<float*>(cur);             // [D] residual stream
  float* s_l = y + D;                                   // [D] s_t
  float* qkv = s_l + D;                                 // [3D]
  float* gpre = qkv + 3 * D;                            // [D]
  float* fbv = gpre + D;                                // [D]
  float* gains = fbv + D;                               // [(3L+1) D]: self, cross, ffn per layer, final
  float* bgl = gains + (3 * L + 1) * D;                 // [D]
  float* wscr = bgl + D;                                // [NWAVE][64*17 + 64] wave scratch
  float* act_raw = wscr + NWAVE * (64 * 17 + 64);       // [F2] (SwiGLU gate/up pre-activations)
  WT* q_hi = reinterpret_cast<WT*>(act_raw + F2);       // [D] query, storage-precision high part
  WT* q_lo = q_hi + D;                                  // [D] low part (bf16 mode only)
  float* my_scr = wscr + wave * (64 * 17 + 64);

  // ---- carried state, gains ----
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
    for (int i = tid; i < L * D; i += NT) {
      gains[i] = p.g_self[i];
      gains[L * D + i] = p.g_cross[i];
      gains[2 * L * D + i] = p.g_ffn[i];
    }
    for (int c = tid; c < D; c += NT) {
      gains[3 * L * D + c] = p.g_final[c];
      bgl[c] = p.bg[c];
      const float s0 = p.s[static_cast<size_t>(b) * D + c];
      s_l[c] = s0;
      store_from_f32(&xop[D + c], s0);
    }
  }
  const WT* e_seq = static_cast<const WT*>(p.e) + static_cast<size_t>(b) * T * D;
  for (int c = tid * 8; c < D; c += NT * 8)
    *reinterpret_cast<Chunk*>(xop + c) = O::load(e_seq + static_cast<size_t>(p.t0) * D + c);
  const WT* wgate = static_cast<const WT*>(p.wgate);
  const WT* wfb = static_cast<const WT*>(p.wfb);
  auto layer_w = [&](int l, size_t off) {
    return reinterpret_cast<const WT*>(p.layers + static_cast<size_t>(l) * p.layer_stride + off);
  };

  WBuf<WT> wa, wb;
  wprefetch(wa, wgate, D, 2 * D);
  wprefetch(wb, wfb, D, D);
  __syncthreads();

  auto xf_op = [&](const WT* v) { return [=](int k) { return O::load(v + k); }; };
  // query element r (pre-scaled): fp32 copy and, in bf16 mode, its hi/lo split
  auto put_q = [&](int r, float v) {
    qkv[r] = v;
    store_from_f32(&q_hi[r], v);
    store_from_f32(&q_lo[r], v - round_to<WT>(v));
  };

  for (int step = 0; step < p.n; ++step) {
    const int t = p.t0 + step;   // 0-based position of this transition
    Chunk e_next = O::zero();
    const bool has_next = step + 1 < p.n;
    if (has_next && tid * 8 < D) e_next = O::load(e_seq + static_cast<size_t>(t + 1) * D + tid * 8);

    // ---- gated merge: xop = [e_t ; bf16(s_{t-1})] ----
    wcompute(wa, wgate, D, 2 * D, xf_op(xop), [&](int r, float v) { gpre[r] = v + bgl[r]; });
    wcompute(wb, wfb, D, D, xf_op(xop + D), [&](int r, float v) { fbv[r] = v; });
    wprefetch(wa, layer_w(0, p.l_qkv), 3 * D, D);
    wprefetch(wb, layer_w(0, p.l_wo), D, D);
    __syncthreads();
    for (int c = tid; c < D; c += NT) {
      const float g = sigmoid_f(gpre[c]);
      y[c] = g * load_as_f32(xop + c) + (1.0f - g) * fbv[c];
    }
    __syncthreads();

    for (int l = 0; l < L; ++l) {
      const float* g_self = gains + l * D;
      const float* g_cross = gains + (L + l) * D;
      const float* g_ffn = gains + (2 * L + l) * D;
      WT* rK = ringK + static_cast<size_t>(l) * H * Wm1 * DH;
      WT* rV = ringV + static_cast<size_t>(l) * H * Wm1 * DH;

      // ---- P1: q,k,v = W_{Q,K,V} RMS(y; g_self); q pre-scaled by 1/sqrt(d_h) ----
      {
        const float inv = wave_rms_inv<D>(y, p.eps);
        wcompute(wa, layer_w(l, p.l_qkv), 3 * D, D, [&](int k) { return norm_chunk<WT>(y, g_self, inv, k); },
                 [&](int r, float v) {
                   if (r < D) put_q(r, v * scale);
                   else qkv[r] = round_to<WT>(v);
                 });
        wprefetch(wa, layer_w(l, p.l_wqx), D, D);
      }
      __syncthreads();

      // ---- P2: window self-attention, one head per wave, lanes over window entries ----
      const int npast = min(t, Wm1);        // cached entries in the window
      const int ne = npast + 1;             // plus the current token
      const int slot0 = Wm1 > 0 ? (t - npast) % Wm1 : 0;   // ring slot of the oldest entry
      for (int h = wave; h < H; h += NWAVE) {
        QSlice<WT> qs;
        qs.set(qkv + h * DH + sub * 16, q_hi + h * DH + sub * 16, q_lo + h * DH + sub * 16);
        float m = -INFINITY, lsum = 0.f;
        float o[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) o[c] = 0.f;
        for (int i0 = 0; i0 < ne; i0 += SLOTS) {
          const int i = i0 + slot;
          const bool ok = i < ne;
          Chunk k0, k1, v0, v1;
          if (i < npast) {
            int sl = slot0 + i;
            sl = sl >= Wm1 ? sl - Wm1 : sl;
            const WT* kr = rK + (static_cast<size_t>(h) * Wm1 + sl) * DH + sub * 16;
            const WT* vr = rV + (static_cast<size_t>(h) * Wm1 + sl) * DH + sub * 16;
            k0 = O::load(kr); k1 = O::load(kr + 8); v0 = O::load(vr); v1 = O::load(vr + 8);
          } else {
            // the current entry (values already rounded to the storage precision)
            float kf[8], vf[8];
            const float* kq = qkv + D + h * DH + sub * 16;
#pragma unroll
            for (int c = 0; c < 8; ++c) { kf[c] = kq[c]; vf[c] = kq[D + c]; }
            k0 = O::pack(kf); v0 = O::pack(vf);
#pragma unroll
            for (int c = 0; c < 8; ++c) { kf[c] = kq[8 + c]; vf[c] = kq[D + 8 + c]; }
            k1 = O::pack(kf); v1 = O::pack(vf);
          }
          float s = qs.dot(k0, k1);
          if constexpr (LPK > 1) s = group_sum<LPK>(s);
          s = ok ? s : -INFINITY;
          const float mnew = fmaxf(m, s);
          const float corr = m == mnew ? 1.f : __expf(m - mnew);   // m = mnew = -inf: nothing seen yet
          const float w = ok ? __expf(s - mnew) : 0.f;
          lsum = lsum * corr + w;
#pragma unroll
          for (int c = 0; c < 16; ++c) o[c] *= corr;
          axpy16<WT>(o, w, v0, v1);
          m = mnew;
        }
        wave_combine<WT, DH>(m, lsum, o, my_scr, xop + h * DH);
        // the current entry replaces the oldest one (position t - (W-1))
        if (Wm1 > 0) {
          const int sl = t % Wm1;
          const size_t gbase = (static_cast<size_t>(l) * p.B + b) * H * Wm1 * DH;
          for (int c = lane; c < DH; c += 64) {
            const size_t o_ = (static_cast<size_t>(h) * Wm1 + sl) * DH + c;
            WT kq, vq;
            store_from_f32(&kq, qkv[D + h * DH + c]);
            store_from_f32(&vq, qkv[2 * D + h * DH + c]);
            rK[o_] = kq;
            rV[o_] = vq;
            static_cast<WT*>(p.ring_k)[gbase + o_] = kq;
            static_cast<WT*>(p.ring_v)[gbase + o_] = vq;
          }
        }
      }
      __syncthreads();

      // ---- P3: y += W_O attn; the first key batch of this layer's memory is issued here ----
      const int grp_l = G == 1 ? 0 : l;
      const size_t mrow0 = (static_cast<size_t>(grp_l) * p.B + b) * H * static_cast<size_t>(T) * DH * sizeof(WT);
      const char* mkb = static_cast<const char*>(p.mem_k) + mrow0;
      const char* mvb = static_cast<const char*>(p.mem_v) + mrow0;
      // lane byte offset of key row j of head hh: ((hh*T + j)*DH + 16*sub) * sizeof(WT)
      auto row_off = [&](int hh, int j) {
        return static_cast<uint32_t>(((hh * T + j) * DH + sub * 16) * sizeof(WT));
      };
      // rows j = base + SLOTS*i (i < KQ), clamped to t (clamped rows are masked out later)
      auto load_rows = [&](const char* mb, int hh, int base, Chunk (&x)[KQ][2]) {
#pragma unroll
        for (int i = 0; i < KQ; ++i) {
          const uint32_t off = row_off(hh, min(base + SLOTS * i, t));
          x[i][0] = O::load(reinterpret_cast<const WT*>(mb + off));
          x[i][1] = O::load(reinterpret_cast<const WT*>(mb + off) + 8);
        }
      };
      Chunk kq0[KQ][2];
      const int h0 = wave < H ? wave : 0;
      load_rows(mkb, h0, slot, kq0);
      wcompute(wb, layer_w(l, p.l_wo), D, D, xf_op(xop), [&](int r, float v) { y[r] += v; });
      wprefetch(wb, layer_w(l, p.l_wox), D, D);
      __syncthreads();

      // ---- P4: q_x = W_Qx RMS(y; g_cross) (pre-scaled by 1/sqrt(d_h)); first value batch ----
      Chunk vq0[KQ][2];
      load_rows(mvb, h0, slot, vq0);
      {
        const float inv = wave_rms_inv<D>(y, p.eps);
        wcompute(wa, layer_w(l, p.l_wqx), D, D, [&](int k) { return norm_chunk<WT>(y, g_cross, inv, k); },
                 [&](int r, float v) { put_q(r, v * scale); });
        wprefetch(wa, layer_w(l, p.l_fin), F2, D);
      }
      __syncthreads();

      // ---- P5: cross-attention over memory rows 0..t, one head per wave ----
      // Keys are taken in chunks of NSC*SLOTS rows.  Per chunk: pass 1 computes every score of
      // the lane into registers (K rows in batches of KQ, the next batch in flight while the
      // current one is used); pass 2 streams the V rows and accumulates exp(s - m) v.  The
      // running (m, l, o) is rescaled once per chunk.
      for (int h = wave; h < H; h += NWAVE) {
        QSlice<WT> qs;
        qs.set(qkv + h * DH + sub * 16, q_hi + h * DH + sub * 16, q_lo + h * DH + sub * 16);
        float m = -INFINITY, lsum = 0.f;
        float o[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) o[c] = 0.f;
        const bool first_head = h == wave;
        for (int c0 = 0; c0 <= t; c0 += NSC * SLOTS) {
          const int cb = c0 + slot;                 // this lane's first row in the chunk
          float sc[NSC];
          float cmax = -INFINITY;
          // two load buffers used alternately by the unrolled batch sequence (no copies)
          Chunk xa[KQ][2], xb[KQ][2];
          if (first_head && c0 == 0) {
#pragma unroll
            for (int i = 0; i < KQ; ++i) { xa[i][0] = kq0[i][0]; xa[i][1] = kq0[i][1]; }
          } else {
            load_rows(mkb, h, cb, xa);
          }
#pragma unroll
          for (int q0 = 0; q0 < NSC; q0 += KQ) {
            if (c0 + SLOTS * q0 > t) break;         // uniform: no row of this batch exists
            Chunk (&cur)[KQ][2] = ((q0 / KQ) & 1) ? xb : xa;
            Chunk (&nxt)[KQ][2] = ((q0 / KQ) & 1) ? xa : xb;
            if (q0 + KQ < NSC && c0 + SLOTS * (q0 + KQ) <= t) load_rows(mkb, h, cb + SLOTS * (q0 + KQ), nxt);
#pragma unroll
            for (int i = 0; i < KQ; ++i) {
              float a = qs.dot(cur[i][0], cur[i][1]);
              if constexpr (LPK > 1) a = group_sum<LPK>(a);
              a = cb + SLOTS * (q0 + i) <= t ? a : -INFINITY;
              sc[q0 + i] = a;
              cmax = fmaxf(cmax, a);
            }
          }
          const float mnew = fmaxf(m, cmax);
          const float corr = m == mnew ? 1.f : __expf(m - mnew);
          lsum *= corr;
#pragma unroll
          for (int c = 0; c < 16; ++c) o[c] *= corr;
          m = mnew;
          const float mref = m == -INFINITY ? 0.f : m;   // lane without rows: every exp(-inf - 0) = 0
          if (first_head && c0 == 0) {
#pragma unroll
            for (int i = 0; i < KQ; ++i) { xa[i][0] = vq0[i][0]; xa[i][1] = vq0[i][1]; }
          } else {
            load_rows(mvb, h, cb, xa);
          }
#pragma unroll
          for (int q0 = 0; q0 < NSC; q0 += KQ) {
            if (c0 + SLOTS * q0 > t) break;
            Chunk (&cur)[KQ][2] = ((q0 / KQ) & 1) ? xb : xa;
            Chunk (&nxt)[KQ][2] = ((q0 / KQ) & 1) ? xa : xb;
            if (q0 + KQ < NSC && c0 + SLOTS * (q0 + KQ) <= t) load_rows(mvb, h, cb + SLOTS * (q0 + KQ), nxt);
#pragma unroll
            for (int i = 0; i < KQ; ++i) {
              const float w = __expf(sc[q0 + i] - mref);   // masked rows: exp(-inf) = 0
              lsum += w;
              axpy16<WT>(o, w, cur[i][0], cur[i][1]);
            }
          }
        }
        wave_combine<WT, DH>(m, lsum, o, my_scr, xop + h * DH);
      }
      __syncthreads();

      // ---- P7: y += W_Ox attn ----
      wcompute(wb, layer_w(l, p.l_wox), D, D, xf_op(xop), [&](int r, float v) { y[r] += v; });
      wprefetch(wb, layer_w(l, p.l_fout), D, F);
      __syncthreads();

      // ---- P8/P9: FFN (tied with encoder layer l) ----
      const bool last = l + 1 == L;
      {
        const float inv = wave_rms_inv<D>(y, p.eps);
        auto xf = [&](int k) { return norm_chunk<WT>(y, g_ffn, inv, k); };
        if (p.ffn_kind == RLT_FFN_GELU) {
          wcompute(wa, layer_w(l, p.l_fin), F, D, xf,
                   [&](int r, float v) { store_from_f32(&xop[r], gelu_erf(v)); });
        } else {
          wcompute(wa, layer_w(l, p.l_fin), F2, D, xf, [&](int r, float v) { act_raw[r] = v; });
        }
        if (last) wprefetch(wa, wgate, D, 2 * D);
        else wprefetch(wa, layer_w(l + 1, p.l_qkv), 3 * D, D);
      }
      __syncthreads();
      if (p.ffn_kind != RLT_FFN_GELU) {
        for (int i = tid; i < F; i += NT) {
          const int gr = (i / 16) * 32 + i % 16;
          store_from_f32(&xop[i], silu_f(act_raw[gr]) * act_raw[gr + 16]);
        }
        __syncthreads();
      }
      wcompute(wb, layer_w(l, p.l_fout), D, F, xf_op(xop), [&](int r, float v) { y[r] += v; });
      if (last) wprefetch(wb, wfb, D, D);
      else wprefetch(wb, layer_w(l + 1, p.l_wo), D, D);
      __syncthreads();
    }

    // ---- s_t = RMSNorm(y; g_dec_final); next merge operand [e_{t+1}; bf16(s_t)] ----
    {
      const float inv = wave_rms_inv<D>(y, p.eps);
      const float* g_fin = gains + 3 * L * D;
      for (int c = tid; c < D; c += NT) {
        const float v = g_fin[c] * (y[c] * inv);
        s_l[c] = v;
        store_from_f32(&xop[D + c], v);
        if (p.s_out) p.s_out[(static_cast<size_t>(b) * p.n + step) * D + c] = v;
      }
      if (has_next && tid * 8 < D) *reinterpret_cast<Chunk*>(xop + tid * 8) = e_next;
    }
    __syncthreads();
  }
  for (int c = tid; c < D; c += NT) p.s[static_cast<size_t>(b) * D + c] = s_l[c];
}

size_t lds_bytes(const ModelLayout& m) {
  const size_t H = m.H, DH = m.DH, D = m.D, L = m.L;
  const size_t ring = 2 * L * H * (m.W - 1) * DH * m.esz;
  const size_t xopn = 2 * D > static_cast<size_t>(m.F) ? 2 * D : m.F;
  const size_t floats = D + D + 3 * D + D + D + (3 * L + 1) * D + D + NWAVE * (64 * 17 + 64) + m.F2;
  return (ring + 15) / 16 * 16 + (xopn * m.esz + 15) / 16 * 16 + floats * 4 + 2 * D * m.esz;
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
  const size_t lds = lds_bytes(m);
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
  const int entries = std::min(m.W, T);   // window entries ever held at once
  // 32-bit memory-row offsets within one (group, sequence)
  const bool offsets = static_cast<size_t>(T) * m.D * m.esz < (size_t(1) << 31);
  return shape && entries <= WCAP && offsets && m.F2 <= 4096 && lds_bytes(m) <= kMaxLds;
}

size_t dec_small_lds_bytes(const ModelLayout& m, int T) {
  (void)T;
  return lds_bytes(m);
}

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
