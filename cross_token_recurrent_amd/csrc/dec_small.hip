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
// matrix-vector products, so a step is bound by latency (dependent phases, memory round
// trips), not by HBM or MFMA throughput.  Independent sequences never synchronise, so each
// sequence gets one 8-wave workgroup that keeps its window caches, running state, gains
// and small vectors in LDS and synchronises only with s_barrier.  Latency is hidden by:
//   * weight prefetch: the next matrix-vector product's weights are loaded into registers
//     one phase ahead (s_barrier does not wait for outstanding global loads);
//   * RMSNorm fused into the consuming product (each wave recomputes the statistic);
//   * window self-attention done per head inside one wave (no workgroup barrier);
//   * cross-attention as one online-softmax pass over memory rows with batched,
//     pipelined loads whose first batch is issued two phases before it is needed.
// bf16 mode: matrix-product operands are packed bf16 in LDS and consumed with
// v_dot2c_f32_bf16 (exact bf16 products, fp32 accumulation); the residual stream,
// softmax statistics, attention math and s_t stay fp32.
#include <algorithm>

#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int NT = 512;          // threads per workgroup (8 waves)
constexpr int NWAVE = NT / 64;
constexpr int NG = NT / 8;       // 8-lane groups for matrix-vector products
constexpr int CMAX = 4;          // prefetched (row, chunk) pairs per lane and product
constexpr int EMAX = 4;          // window entries per lane (window <= 256)

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// ---- storage-type operations on 8-element chunks -----------------------------------
template <typename WT> struct Ops;

template <> struct Ops<bf16_t> {
  struct Chunk { uint4 v; };
  struct QPack { uint32_t hi[4], lo[4]; };  // query split into bf16 hi + lo parts
  static __device__ __forceinline__ Chunk load(const bf16_t* p) { return {*reinterpret_cast<const uint4*>(p)}; }
  static __device__ __forceinline__ Chunk zero() { return {make_uint4(0u, 0u, 0u, 0u)}; }
  static __device__ __forceinline__ Chunk lds(const bf16_t* p) { return {*reinterpret_cast<const uint4*>(p)}; }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  static __device__ __forceinline__ Chunk pack(const float (&f)[8]) {
    return {make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]))};
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
  static __device__ __forceinline__ QPack qpack(const float (&q)[8]) {
    QPack r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = q[2 * i], b = q[2 * i + 1];
      const float ah = bf16_to_f32(f32_to_bf16(a)), bh = bf16_to_f32(f32_to_bf16(b));
      r.hi[i] = pack2(ah, bh);
      r.lo[i] = pack2(a - ah, b - bh);
    }
    return r;
  }
  static __device__ __forceinline__ float qdot(const Chunk& k, const QPack& q) {
    const uint32_t kv[4] = {k.v.x, k.v.y, k.v.z, k.v.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = d2(kv[i], q.lo[i], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = d2(kv[i], q.hi[i], acc);
    return acc;
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
  struct QPack { float q[8]; };
  static __device__ __forceinline__ Chunk load(const float* p) {
    return {*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  static __device__ __forceinline__ Chunk zero() { return {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)}; }
  static __device__ __forceinline__ Chunk lds(const float* p) { return load(p); }
  static __device__ __forceinline__ Chunk pack(const float (&f)[8]) {
    return {make_float4(f[0], f[1], f[2], f[3]), make_float4(f[4], f[5], f[6], f[7])};
  }
  static __device__ __forceinline__ float dot(const Chunk& w, const Chunk& x, float acc) {
    acc += w.a.x * x.a.x; acc += w.a.y * x.a.y; acc += w.a.z * x.a.z; acc += w.a.w * x.a.w;
    acc += w.b.x * x.b.x; acc += w.b.y * x.b.y; acc += w.b.z * x.b.z; acc += w.b.w * x.b.w;
    return acc;
  }
  static __device__ __forceinline__ QPack qpack(const float (&q)[8]) {
    QPack r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.q[i] = q[i];
    return r;
  }
  static __device__ __forceinline__ float qdot(const Chunk& k, const QPack& q) {
    return q.q[0] * k.a.x + q.q[1] * k.a.y + q.q[2] * k.a.z + q.q[3] * k.a.w + q.q[4] * k.b.x + q.q[5] * k.b.y +
           q.q[6] * k.b.z + q.q[7] * k.b.w;
  }
  static __device__ __forceinline__ void unpack(const Chunk& c, float (&f)[8]) {
    f[0] = c.a.x; f[1] = c.a.y; f[2] = c.a.z; f[3] = c.a.w;
    f[4] = c.b.x; f[5] = c.b.y; f[6] = c.b.z; f[7] = c.b.w;
  }
};

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
    const int r = grp + ri * NG;
    buf.c[p] = r < N ? Ops<WT>::load(W + static_cast<size_t>(r) * K + sub * 8 + ci * 64) : Ops<WT>::zero();
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
#pragma unroll
  for (int ri = 0; ri < RB; ++ri) {
    if (ri < nrows) {
      float acc = 0.f;
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci) acc = O::dot(buf.c[ri * CPL + ci], xr[ci], acc);
      acc = group_sum<8>(acc);
      const int r = grp + ri * NG;
      if (sub == 0 && r < N) epi(r, acc);
    }
  }
  for (int ri = RB; ri < nrows; ++ri) {
    const int r = grp + ri * NG;
    float acc = 0.f;
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
      const typename O::Chunk w = r < N ? O::load(W + static_cast<size_t>(r) * K + sub * 8 + ci * 64) : O::zero();
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
  constexpr int KB = sizeof(WT) == 2 ? 4 : 2;   // memory rows per lane per cross-attention batch
  constexpr int H = D / DH;
  constexpr int LPK = DH / 8;            // lanes per memory row (8 elements each)
  constexpr int PARTS = NT / (H * LPK);  // key slices per head in cross-attention
  static_assert(PARTS >= 8 && PARTS % 8 == 0, "cross-attention partition");
  static_assert(H <= NWAVE, "one wave per head in window attention");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  float* part_m = bgl + D;                              // [H][PARTS]
  float* part_l = part_m + H * PARTS;                   // [H][PARTS]
  float* part_o = part_l + H * PARTS;                   // [H][PARTS][DH]
  float* swa_p = part_o + H * PARTS * DH;               // [H][EMAX*64] window probabilities
  float* act_raw = swa_p + H * EMAX * 64;               // [F2] (SwiGLU gate/up pre-activations)

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
  // e_{t0} -> xop[0, D)
  for (int c = tid * 8; c < D; c += NT * 8) {
    const Chunk ec = O::load(e_seq + static_cast<size_t>(p.t0) * D + c);
    *reinterpret_cast<Chunk*>(xop + c) = ec;
  }
  const WT* wgate = static_cast<const WT*>(p.wgate);
  const WT* wfb = static_cast<const WT*>(p.wfb);
  auto layer_w = [&](int l, size_t off) {
    return reinterpret_cast<const WT*>(p.layers + static_cast<size_t>(l) * p.layer_stride + off);
  };

  WBuf<WT> wa, wb;
  wprefetch(wa, wgate, D, 2 * D);
  wprefetch(wb, wfb, D, D);
  __syncthreads();

  auto xf_op = [&](const WT* v) { return [=](int k) { return O::lds(v + k); }; };

  // cross-attention lane roles
  const int xh = tid / (PARTS * LPK);
  const int xpart = (tid / LPK) % PARTS;
  const int xsub = tid % LPK;

  for (int step = 0; step < p.n; ++step) {
    const int t = p.t0 + step;   // 0-based position of this transition
    // prefetch e_{t+1} for the next step's merge
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

      // ---- P1: q,k,v = W_{Q,K,V} RMS(y; g_self) ----
      {
        const float inv = wave_rms_inv<D>(y, p.eps);
        auto xf = [&](int k) {
          float f[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = g_self[k + i] * (y[k + i] * inv);
          return O::pack(f);
        };
        wcompute(wa, layer_w(l, p.l_qkv), 3 * D, D, xf,
                 [&](int r, float v) { qkv[r] = r < D ? v : round_to<WT>(v); });
        wprefetch(wa, layer_w(l, p.l_wqx), D, D);
      }
      __syncthreads();

      // ---- P2: window self-attention, one wave per head ----
      const int npast = min(t, Wm1);        // cached entries in the window
      const int ne = npast + 1;             // plus the current token
      const int slot0 = Wm1 > 0 ? (t - npast) % Wm1 : 0;   // slot of the oldest cached entry
      auto slot_of = [&](int i) {
        const int sl = slot0 + i;
        return sl >= Wm1 ? sl - Wm1 : sl;
      };
      for (int h = wave; h < H; h += NWAVE) {
        const float* q = qkv + h * DH;
        float sc[EMAX];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < EMAX; ++k) {
          const int i = lane + 64 * k;
          float acc = -INFINITY;
          if (i < ne) {
            acc = 0.f;
            if (i < npast) {
              const WT* kr = rK + (static_cast<size_t>(h) * Wm1 + slot_of(i)) * DH;
#pragma unroll
              for (int c8 = 0; c8 < DH; c8 += 8) {
                float kf[8];
                O::unpack(O::lds(kr + c8), kf);
                const float4 q0 = *reinterpret_cast<const float4*>(q + c8);
                const float4 q1 = *reinterpret_cast<const float4*>(q + c8 + 4);
                acc += q0.x * kf[0] + q0.y * kf[1] + q0.z * kf[2] + q0.w * kf[3] + q1.x * kf[4] + q1.y * kf[5] +
                       q1.z * kf[6] + q1.w * kf[7];
              }
            } else {
              const float* kr = qkv + D + h * DH;
#pragma unroll
              for (int c = 0; c < DH; ++c) acc += q[c] * kr[c];
            }
            acc *= scale;
          }
          sc[k] = acc;
          mx = fmaxf(mx, acc);
        }
        mx = group_max<64>(mx);
        float den = 0.f;
        float* ph = swa_p + h * (EMAX * 64);
#pragma unroll
        for (int k = 0; k < EMAX; ++k) {
          const int i = lane + 64 * k;
          const float w = i < ne ? __expf(sc[k] - mx) : 0.f;
          den += w;
          if (i < ne) ph[i] = w;
        }
        den = group_sum<64>(den);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if constexpr (DH >= 64) {
          // lane owns dims lane, lane+64, ...; all entries
#pragma unroll
          for (int c = lane; c < DH; c += 64) {
            float o = 0.f;
            for (int i = 0; i < ne; ++i) {
              float v;
              if (i < npast) {
                v = load_as_f32(rV + (static_cast<size_t>(h) * Wm1 + slot_of(i)) * DH + c);
              } else {
                v = qkv[2 * D + h * DH + c];
              }
              o += ph[i] * v;
            }
            store_from_f32(&xop[h * DH + c], o / den);
          }
        } else {
          // lane (c, g): dim c, entries i = g, g + 64/DH, ...; then a sum over the groups
          constexpr int GS = 64 / DH;
          constexpr int UN = 8;   // entries per lane issued together
          const int c = lane % DH, g0 = lane / DH;
          float o = 0.f;
          for (int i0 = g0; i0 < ne; i0 += GS * UN) {
            float pv[UN], vv[UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
              const int i = min(i0 + GS * u, ne - 1);
              pv[u] = i0 + GS * u < ne ? ph[i] : 0.f;
              vv[u] = i < npast ? load_as_f32(rV + (static_cast<size_t>(h) * Wm1 + slot_of(i)) * DH + c)
                                : qkv[2 * D + h * DH + c];
            }
#pragma unroll
            for (int u = 0; u < UN; ++u) o += pv[u] * vv[u];
          }
#pragma unroll
          for (int off = DH; off < 64; off <<= 1) o += __shfl_xor(o, off, 64);
          if (g0 == 0) store_from_f32(&xop[h * DH + c], o / den);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // the current entry replaces the oldest one (position t - (W-1)) after the reads above
        if (Wm1 > 0) {
          const int slot = t % Wm1;
          const size_t gbase = (static_cast<size_t>(l) * p.B + b) * H * Wm1 * DH;
          for (int c = lane; c < DH; c += 64) {
            const size_t o_ = (static_cast<size_t>(h) * Wm1 + slot) * DH + c;
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

      // ---- P3: y += W_O attn; first memory batch of this layer issued here ----
      const int grp_l = G == 1 ? 0 : l;
      // memory rows of (group, sequence): uniform base + 32-bit per-lane byte offsets
      const size_t mrow0 = (static_cast<size_t>(grp_l) * p.B + b) * H * static_cast<size_t>(T) * DH * sizeof(WT);
      const char* mkb = static_cast<const char*>(p.mem_k) + mrow0;
      const char* mvb = static_cast<const char*>(p.mem_v) + mrow0;
      const uint32_t lane_off = static_cast<uint32_t>((xh * T * DH + xsub * 8) * sizeof(WT));
      constexpr int STRIDE = PARTS * KB;     // key distance between a lane's consecutive batches
      auto issue = [&](Chunk (&kx)[KB], Chunk (&vx)[KB], int jb) {
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          const int j = jb + PARTS * i;
          const uint32_t off = lane_off + static_cast<uint32_t>(j * DH * sizeof(WT));
          kx[i] = j <= t ? O::load(reinterpret_cast<const WT*>(mkb + off)) : O::zero();
          vx[i] = j <= t ? O::load(reinterpret_cast<const WT*>(mvb + off)) : O::zero();
        }
      };
      Chunk kA[KB], vA[KB], kB_[KB], vB_[KB];
      issue(kA, vA, xpart);
      wcompute(wb, layer_w(l, p.l_wo), D, D, xf_op(xop), [&](int r, float v) { y[r] += v; });
      wprefetch(wb, layer_w(l, p.l_wox), D, D);
      __syncthreads();

      // ---- P4: q_x = W_Qx RMS(y; g_cross) (pre-scaled by 1/sqrt(d_h)) ----
      issue(kB_, vB_, xpart + STRIDE);
      {
        const float inv = wave_rms_inv<D>(y, p.eps);
        auto xf = [&](int k) {
          float f[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = g_cross[k + i] * (y[k + i] * inv);
          return O::pack(f);
        };
        wcompute(wa, layer_w(l, p.l_wqx), D, D, xf, [&](int r, float v) { qkv[r] = v * scale; });
        wprefetch(wa, layer_w(l, p.l_fin), F2, D);
      }
      __syncthreads();

      // ---- P5: cross-attention over memory rows 0..t, online softmax per lane ----
      {
        float q8[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) q8[c] = qkv[xh * DH + xsub * 8 + c];
        const typename O::QPack qp = O::qpack(q8);
        float m = -INFINITY, lsum = 0.f;
        float o8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        auto process = [&](const Chunk (&kx)[KB], const Chunk (&vx)[KB], int jb) {
          float s[KB];
          float bm = -INFINITY;
#pragma unroll
          for (int i = 0; i < KB; ++i) {
            float a = O::qdot(kx[i], qp);
            if constexpr (LPK > 1) a = group_sum<LPK>(a);
            s[i] = (jb + PARTS * i <= t) ? a : -INFINITY;
            bm = fmaxf(bm, s[i]);
          }
          const float mnew = fmaxf(m, bm);
          const float corr = __expf(m - mnew);
          lsum *= corr;
#pragma unroll
          for (int c = 0; c < 8; ++c) o8[c] *= corr;
#pragma unroll
          for (int i = 0; i < KB; ++i) {
            const float w = __expf(s[i] - mnew);
            float vv[8];
            O::unpack(vx[i], vv);
            lsum += w;
#pragma unroll
            for (int c = 0; c < 8; ++c) o8[c] += w * vv[c];
          }
          m = mnew;
        };
        // two rotating buffers: batches 0 and 1 were requested two phases earlier; batch
        // i+2 is requested while batch i is processed
        for (int jb = xpart; jb <= t;) {
          process(kA, vA, jb);
          issue(kA, vA, jb + 2 * STRIDE);
          jb += STRIDE;
          if (jb > t) break;
          process(kB_, vB_, jb);
          issue(kB_, vB_, jb + 2 * STRIDE);
          jb += STRIDE;
        }
        float* po = part_o + (static_cast<size_t>(xh) * PARTS + xpart) * DH + xsub * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) po[c] = o8[c];
        if (xsub == 0) {
          part_m[xh * PARTS + xpart] = m;
          part_l[xh * PARTS + xpart] = lsum;
        }
      }
      __syncthreads();

      // ---- P6: combine the PARTS partial softmax states of every (head, dim), fixed order ----
      for (int idx = tid; idx < D * 8; idx += NT) {
        const int k = idx & 7, hc = idx >> 3;
        const int h = hc / DH, c = hc % DH;
        constexpr int QN = PARTS / 8;
        float pm[QN], pl[QN], pov[QN];
#pragma unroll
        for (int qq = 0; qq < QN; ++qq) {
          const int q = k + 8 * qq;
          pm[qq] = part_m[h * PARTS + q];
          pl[qq] = part_l[h * PARTS + q];
          pov[qq] = part_o[(static_cast<size_t>(h) * PARTS + q) * DH + c];
        }
        float mloc = pm[0];
#pragma unroll
        for (int qq = 1; qq < QN; ++qq) mloc = fmaxf(mloc, pm[qq]);
        const float mh = group_max<8>(mloc);
        float o = 0.f, l_ = 0.f;
#pragma unroll
        for (int qq = 0; qq < QN; ++qq) {
          const float w = __expf(pm[qq] - mh);
          o += w * pov[qq];
          l_ += w * pl[qq];
        }
        o = group_sum<8>(o);
        l_ = group_sum<8>(l_);
        if (k == 0) store_from_f32(&xop[hc], o / l_);
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
        auto xf = [&](int k) {
          float f[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = g_ffn[k + i] * (y[k + i] * inv);
          return O::pack(f);
        };
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
  const size_t parts = NT / (H * (DH / 8));
  const size_t xopn = 2 * D > static_cast<size_t>(m.F) ? 2 * D : m.F;
  const size_t floats = D + D + 3 * D + D + D + (3 * L + 1) * D + D + H * parts + H * parts + H * parts * DH +
                        H * EMAX * 64 + m.F2;
  return (ring + 15) / 16 * 16 + (xopn * m.esz + 15) / 16 * 16 + floats * 4;
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
  return shape && entries <= EMAX * 64 && m.F2 <= 4096 && lds_bytes(m) <= kMaxLds;
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
