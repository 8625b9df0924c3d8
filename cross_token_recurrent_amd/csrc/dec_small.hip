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
// matrix-vector products and two single-query attentions, so a step is a chain of short,
// latency-bound phases, while the memory rows of the cross-attention (a few hundred KB per
// step and sequence) must stream from HBM or the Infinity Cache without stalling that
// chain.  Independent sequences never synchronise, so each sequence gets one workgroup of
// 12 waves (three per SIMD) that keeps its window caches, residual stream, gains, W_O (and at
// d = 64 the merge weights) in LDS and splits the work by role, each role running its own
// loop through the same sequence of workgroup barriers (the gated merge, then seven phases
// per layer: QKV, window attention, Q_x, cross-attention, W_Ox, FFN in, FFN out):
//   * 4 product waves run the gated merge and every matrix-vector product: 8- or 16-lane
//     groups per row, weights in registers, RMSNorm fused into the operand fetch, the gated
//     merge fused into the gate/feedback products and SwiGLU/GELU into the FFN input product.
//     Every weight request is issued in the two phases where these waves would otherwise
//     wait (window and cross attention), each product into its own register buffer;
//   * 8 attention waves hold the memory rows of one layer in registers (each a head and a
//     contiguous share of its rows).  The rows of the next layer are requested one 64-row
//     block at a time in each of the six phases between two cross-attentions, so the
//     requests drain in the background without crowding the product waves' weight requests
//     on the CU's vector-memory path; the product waves request only weights, so their loads
//     never queue behind rows (the vector memory counter of a wave retires in order).
//     Scores use lanes over keys; P.V uses lanes over (dim, 8-key block) on the key-blocked
//     value layout, so a lane's dot products run over keys and the sum over its lanes takes
//     at most two row swaps;
//   * window self-attention runs on one attention wave per head: scores with lanes over
//     the ring slots, P.V with lanes over (dim, 8-slot block) of a key-blocked copy of the
//     value ring, then the head's share of the W_O product.
// bf16 mode: matrix-product operands (activations, q, P) are bf16 and every product
// accumulates in fp32 (v_dot2c_f32_bf16); the residual stream, softmax statistics and s_t
// stay fp32.  Scores are kept in the log2 domain (q pre-scaled by log2(e)/sqrt(d_h)).
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

// Wave roles: waves 0..NA-1 do the attention (they hold the memory rows), waves
// NA..NA+NM-1 do the matrix-vector products (they hold the weights).  Each SIMD runs two
// attention waves and one product wave.
constexpr int NA = 8;
constexpr int NM = 4;
constexpr int NT = 64 * (NA + NM);   // 768 threads
constexpr int NTM = 64 * NM;         // product threads
constexpr int WCAP = 256;            // largest window (entries held at once) supported
constexpr float kLog2e = 1.4426950408889634f;

template <int V> using IC = std::integral_constant<int, V>;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// Hardware reciprocal and reciprocal square root (about 1 ulp each): RMSNorm scales,
// softmax normalisers and the logistic function of the gated merge and SwiGLU.
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float rsq_hw(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float sigmoid_hw(float x) { return rcp_hw(1.0f + fast_exp2(-kLog2e * x)); }
__device__ __forceinline__ float silu_hw(float x) { return x * sigmoid_hw(x); }

// Sum over the lanes that hold the same dimension of a P.V product (lanes d, d + DH, ... for
// DH < 64) without the LDS path: v_permlane16_swap / v_permlane32_swap bring the lower row (pair)
// up, and the total lands in the top DH lanes (lane 64 - DH + d holds dimension d), added in the
// same grouping as a butterfly.  Only the first result of each swap is used.
template <int DH>
__device__ __forceinline__ float sum_to_top_rows(float v) {
  if constexpr (DH <= 16) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_permlane16_swap(u, u, false, false)[0]);   // rows 1, 3 += rows 0, 2
  }
  if constexpr (DH <= 32) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_permlane32_swap(u, u, false, false)[0]);   // rows 2, 3 += rows 0, 1
  }
  return v;
}

// threadIdx.x through an empty asm: lane-dependent offsets derived from it are recomputed
// where they are used instead of being hoisted out of the step loop and held in registers.
__device__ __forceinline__ unsigned tid_here() {
  unsigned t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// base + element offset with 32-bit offset arithmetic (scalar base + vector offset loads)
template <typename WT>
__device__ __forceinline__ const WT* at(const WT* base, uint32_t off) {
  return reinterpret_cast<const WT*>(reinterpret_cast<const char*>(base) + off * static_cast<uint32_t>(sizeof(WT)));
}

// ---- storage-type operations on 8-element chunks -----------------------------------
template <typename WT> struct Ops;

template <> struct Ops<bf16_t> {
  struct Chunk { uint4 v; };
  static __device__ __forceinline__ Chunk load(const bf16_t* p) { return {*reinterpret_cast<const uint4*>(p)}; }
  static __device__ __forceinline__ Chunk zero() { return {make_uint4(0u, 0u, 0u, 0u)}; }
  static __device__ __forceinline__ void store(bf16_t* p, const Chunk& c) { *reinterpret_cast<uint4*>(p) = c.v; }
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
  // acc + sum of the 8 elements
  static __device__ __forceinline__ float sum(const Chunk& c, float acc) {
    constexpr uint32_t ones = 0x3F803F80u;   // bf16 pair (1, 1)
    acc = d2(c.v.x, ones, acc);
    acc = d2(c.v.y, ones, acc);
    acc = d2(c.v.z, ones, acc);
    return d2(c.v.w, ones, acc);
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
  static __device__ __forceinline__ void store(float* p, const Chunk& c) {
    *reinterpret_cast<float4*>(p) = c.a;
    *reinterpret_cast<float4*>(p + 4) = c.b;
  }
  static __device__ __forceinline__ Chunk pack(const float (&f)[8]) {
    return {make_float4(f[0], f[1], f[2], f[3]), make_float4(f[4], f[5], f[6], f[7])};
  }
  static __device__ __forceinline__ float dot(const Chunk& w, const Chunk& x, float acc) {
    acc += w.a.x * x.a.x; acc += w.a.y * x.a.y; acc += w.a.z * x.a.z; acc += w.a.w * x.a.w;
    acc += w.b.x * x.b.x; acc += w.b.y * x.b.y; acc += w.b.z * x.b.z; acc += w.b.w * x.b.w;
    return acc;
  }
  static __device__ __forceinline__ float sum(const Chunk& c, float acc) {
    acc += c.a.x; acc += c.a.y; acc += c.a.z; acc += c.a.w;
    acc += c.b.x; acc += c.b.y; acc += c.b.z; acc += c.b.w;
    return acc;
  }
  static __device__ __forceinline__ void unpack(const Chunk& c, float (&f)[8]) {
    f[0] = c.a.x; f[1] = c.a.y; f[2] = c.a.z; f[3] = c.a.w;
    f[4] = c.b.x; f[5] = c.b.y; f[6] = c.b.z; f[7] = c.b.w;
  }
};

// A 16-element query slice in the storage precision, for dot products with key rows.
template <typename WT> struct QVec;
template <> struct QVec<bf16_t> {
  uint32_t q[8];
  __device__ __forceinline__ void load(const bf16_t* p) {
    const uint4 a = *reinterpret_cast<const uint4*>(p), b = *reinterpret_cast<const uint4*>(p + 8);
    q[0] = a.x; q[1] = a.y; q[2] = a.z; q[3] = a.w; q[4] = b.x; q[5] = b.y; q[6] = b.z; q[7] = b.w;
  }
  __device__ __forceinline__ float dot(const Ops<bf16_t>::Chunk& k0, const Ops<bf16_t>::Chunk& k1) const {
    float a = Ops<bf16_t>::d2(q[0], k0.v.x, 0.f);
    a = Ops<bf16_t>::d2(q[1], k0.v.y, a);
    a = Ops<bf16_t>::d2(q[2], k0.v.z, a);
    a = Ops<bf16_t>::d2(q[3], k0.v.w, a);
    a = Ops<bf16_t>::d2(q[4], k1.v.x, a);
    a = Ops<bf16_t>::d2(q[5], k1.v.y, a);
    a = Ops<bf16_t>::d2(q[6], k1.v.z, a);
    return Ops<bf16_t>::d2(q[7], k1.v.w, a);
  }
};
template <> struct QVec<float> {
  float q[16];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + i);
      q[i] = v.x; q[i + 1] = v.y; q[i + 2] = v.z; q[i + 3] = v.w;
    }
  }
  __device__ __forceinline__ float dot(const Ops<float>::Chunk& k0, const Ops<float>::Chunk& k1) const {
    float a = q[0] * k0.a.x;
    a += q[1] * k0.a.y; a += q[2] * k0.a.z; a += q[3] * k0.a.w;
    a += q[4] * k0.b.x; a += q[5] * k0.b.y; a += q[6] * k0.b.z; a += q[7] * k0.b.w;
    a += q[8] * k1.a.x; a += q[9] * k1.a.y; a += q[10] * k1.a.z; a += q[11] * k1.a.w;
    a += q[12] * k1.b.x; a += q[13] * k1.b.y; a += q[14] * k1.b.z; a += q[15] * k1.b.w;
    return a;
  }
};

// ---- matrix-vector products out[r] = W[r,:] . x -----------------------------------------
// Products run on the NTM threads of the product waves; mt = thread index among them.
// With GL lanes per row, thread mt (grp = mt / GL, sub = mt % GL) owns rows grp, grp + NGR,
// ... (NGR = NTM / GL) and, of each row, the 8-element chunks sub + GL*ci (ci < CPL), so
// K = 8 * GL * CPL.  The first CB (row, chunk) pairs come from a register buffer filled
// ahead of time (wpre); the rest are loaded when needed.  Rows past N are clamped on
// load; a wave whose groups all lie past N skips the row.
__device__ __forceinline__ unsigned mtid_here() { return tid_here() - 64u * NA; }

template <typename WT, int GL, int CPL, int CB>
__device__ __forceinline__ void wpre(typename Ops<WT>::Chunk* buf, const WT* __restrict__ W, int N) {
  constexpr int K = 8 * GL * CPL, NGR = NTM / GL;
  const unsigned mt = mtid_here();
  const int sub = mt % GL, grp = mt / GL;
  const int need = (N + NGR - 1) / NGR * CPL;   // buffer slots the product reads
#pragma unroll
  for (int p = 0; p < CB; ++p) {
    if (p >= need) break;
    const int ri = p / CPL, ci = p % CPL;
    const int r = min(grp + ri * NGR, N - 1);
    buf[p] = Ops<WT>::load(at(W, r * K + (sub + GL * ci) * 8));
  }
}

// Lane sub runs the epilogue of the group's rows base + sub (one per lane and round of
// GL rows), so each epilogue runs once per row.  The operand functor xf(k, ss) returns the
// chunk k..k+8 and, for a normalised operand (NORM), adds the chunk's sum of squares to ss:
// the group sum then covers all K and every row result is scaled by 1/rms before the
// epilogue (RMS(y; g) . w = (g*y . w) / rms(y)), so the norm costs no separate reduction.
template <typename WT, int GL, int CPL, int CB, bool NORM = false, typename XF, typename Epi>
__device__ __forceinline__ void wmv(const typename Ops<WT>::Chunk* buf, const WT* __restrict__ W, int N, XF&& xf,
                                    Epi&& epi, float eps = 0.f) {
  using O = Ops<WT>;
  constexpr int K = 8 * GL * CPL, NGR = NTM / GL;
  constexpr int RBU = (CB + CPL - 1) / CPL;   // rows that take chunks from the buffer
  const unsigned mt = mtid_here();
  const int sub = mt % GL, grp = mt / GL;
  const int grp0 = (mt & ~63u) / GL;            // first group of this wave (uniform)
  // rows with at least one group of this wave; the same for every wave when NGR divides N
  // (grp0 < NGR), which keeps the row loop free of branches for compile-time N
  const int nrows = N % NGR == 0 ? N / NGR : (N - grp0 + NGR - 1) / NGR;
  if (nrows <= 0) return;
  typename O::Chunk xr[CPL];
  float ss = 0.f;
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) xr[ci] = xf((sub + GL * ci) * 8, ss);
  float inv = 1.f;
  if constexpr (NORM) inv = rsq_hw(group_sum<GL>(ss) / static_cast<float>(K) + eps);
  auto epi_s = [&](int r, float v) { epi(r, NORM ? v * inv : v); };
  float mine = 0.f;
  int base = 0;
#pragma unroll
  for (int ri = 0; ri < RBU; ++ri) {
    if (ri < nrows) {
      if (ri - base == GL) {   // every lane of the round holds its row: run the epilogues
        const int r = grp + (base + sub) * NGR;
        if (r < N) epi_s(r, mine);
        base += GL;
      }
      const int r = min(grp + ri * NGR, N - 1);
      float acc = 0.f;
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci) {
        const int p = ri * CPL + ci;
        const typename O::Chunk w = p < CB ? buf[p < CB ? p : 0] : O::load(at(W, r * K + (sub + GL * ci) * 8));
        acc = O::dot(w, xr[ci], acc);
      }
      acc = group_sum<GL>(acc);
      mine = sub == ri - base ? acc : mine;
    }
  }
  for (int ri = RBU; ri < nrows; ++ri) {
    if (ri - base == GL) {
      const int r = grp + (base + sub) * NGR;
      if (r < N) epi_s(r, mine);
      base += GL;
    }
    const int r = min(grp + ri * NGR, N - 1);
    float acc = 0.f;
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) acc = O::dot(O::load(at(W, r * K + (sub + GL * ci) * 8)), xr[ci], acc);
    acc = group_sum<GL>(acc);
    mine = sub == ri - base ? acc : mine;
  }
  {
    const int r = grp + (base + sub) * NGR;
    if (base + sub < nrows && r < N) epi_s(r, mine);
  }
}

// SwiGLU input product: rows come in (gate, up) pairs of the interleaved ffn_in layout
// (activation i: gate row (i/16)*32 + i%16, up row 16 further).  Pair i = grp + k*NGR;
// lane sub stores act = silu(gate) * up of the round's pair base + sub.
__device__ __forceinline__ int swiglu_gate_row(int i) { return (i / 16) * 32 + i % 16; }

template <typename WT, int CPL, int CB>
__device__ __forceinline__ void wpre_swiglu(typename Ops<WT>::Chunk* buf, const WT* __restrict__ W, int F) {
  constexpr int GL = 8, K = 8 * GL * CPL, NGR = NTM / GL;
  const unsigned mt = mtid_here();
  const int sub = mt % GL, grp = mt / GL;
#pragma unroll
  for (int p = 0; p < CB; ++p) {
    const int k = p / (2 * CPL), u = (p / CPL) % 2, ci = p % CPL;   // pair k, gate (u = 0) or up row
    const int gr = swiglu_gate_row(min(grp + k * NGR, F - 1));
    buf[p] = Ops<WT>::load(at(W, (gr + 16 * u) * K + (sub + GL * ci) * 8));
  }
}

template <typename WT, int CPL, int CB, typename XF>
__device__ __forceinline__ void wmv_swiglu(const typename Ops<WT>::Chunk* buf, const WT* __restrict__ W, int F,
                                           XF&& xf, WT* __restrict__ out, float eps) {
  using O = Ops<WT>;
  constexpr int GL = 8, K = 8 * GL * CPL, NGR = NTM / GL;
  constexpr int KBU = (CB + 2 * CPL - 1) / (2 * CPL);   // pairs that take chunks from the buffer
  const unsigned mt = mtid_here();
  const int sub = mt % GL, grp = mt / GL;
  const int grp0 = (mt & ~63u) / GL;
  const int npairs = F % NGR == 0 ? F / NGR : (F - grp0 + NGR - 1) / NGR;
  if (npairs <= 0) return;
  typename O::Chunk xr[CPL];
  float ss = 0.f;
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) xr[ci] = xf((sub + GL * ci) * 8, ss);
  const float inv = rsq_hw(group_sum<GL>(ss) / static_cast<float>(K) + eps);   // normalised operand
  float mine = 0.f;
  int base = 0;
  auto pair = [&](int k, auto from_buf) {
    const int gr = swiglu_gate_row(min(grp + k * NGR, F - 1));
    float a[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci) {
        typename O::Chunk w;
        if constexpr (decltype(from_buf)::value >= 0) {
          constexpr int k0 = decltype(from_buf)::value;
          const int p = (2 * k0 + u) * CPL + ci;
          w = p < CB ? buf[p < CB ? p : 0] : O::load(at(W, (gr + 16 * u) * K + (sub + GL * ci) * 8));
        } else {
          w = O::load(at(W, (gr + 16 * u) * K + (sub + GL * ci) * 8));
        }
        acc = O::dot(w, xr[ci], acc);
      }
      a[u] = group_sum<GL>(acc) * inv;
    }
    return silu_hw(a[0]) * a[1];
  };
  auto flush_if_full = [&](int k) {
    if (k - base == GL) {
      const int i = grp + (base + sub) * NGR;
      if (i < F) store_from_f32(&out[i], mine);
      base += GL;
    }
  };
  if (KBU > 0 && npairs > 0) { flush_if_full(0); const float v = pair(0, IC<0>{}); mine = sub == 0 ? v : mine; }
  if (KBU > 1 && npairs > 1) { flush_if_full(1); const float v = pair(1, IC<1>{}); mine = sub == 1 - base ? v : mine; }
  if (KBU > 2 && npairs > 2) { flush_if_full(2); const float v = pair(2, IC<2>{}); mine = sub == 2 - base ? v : mine; }
  if (KBU > 3 && npairs > 3) { flush_if_full(3); const float v = pair(3, IC<3>{}); mine = sub == 3 - base ? v : mine; }
  for (int k = KBU < 4 ? KBU : 4; k < npairs; ++k) {
    flush_if_full(k);
    const float v = pair(k, IC<-1>{});
    mine = sub == k - base ? v : mine;
  }
  {
    const int i = grp + (base + sub) * NGR;
    if (base + sub < npairs && i < F) store_from_f32(&out[i], mine);
  }
}

// Products with K = F (the FFN output product): 16 lanes per row when a 64-row product
// would leave lanes idle and F allows it, else 8; the common chunk counts are unrolled,
// others loop.
template <typename Fn>
__device__ __forceinline__ void dispatch_ffn_out(int D, int F, Fn&& fn) {
  if (D == 64 && F % 128 == 0) {
    switch (F / 128) {
      case 1: fn(IC<16>{}, IC<1>{}); return;
      case 2: fn(IC<16>{}, IC<2>{}); return;
      case 3: fn(IC<16>{}, IC<3>{}); return;
      case 4: fn(IC<16>{}, IC<4>{}); return;
      default: break;
    }
  }
  switch (F / 64) {
    case 1: fn(IC<8>{}, IC<1>{}); return;
    case 2: fn(IC<8>{}, IC<2>{}); return;
    case 3: fn(IC<8>{}, IC<3>{}); return;
    case 4: fn(IC<8>{}, IC<4>{}); return;
    case 6: fn(IC<8>{}, IC<6>{}); return;
    case 8: fn(IC<8>{}, IC<8>{}); return;
    default: fn(IC<8>{}, IC<0>{}); return;   // generic: every chunk loaded when needed
  }
}

// Generic K (multiple of 64), 8 lanes per row, no prefetch.
template <typename WT, typename XF, typename Epi>
__device__ __forceinline__ void wmv_any(const WT* __restrict__ W, int N, int K, XF&& xf, Epi&& epi) {
  using O = Ops<WT>;
  constexpr int NGR = NTM / 8;
  const unsigned mt = mtid_here();
  const int sub = mt & 7, grp = mt >> 3;
  const int nrows = (N + NGR - 1) / NGR;
  for (int ri = 0; ri < nrows; ++ri) {
    const int r = min(grp + ri * NGR, N - 1);
    float acc = 0.f;
    float ss = 0.f;
    for (int k = sub * 8; k < K; k += 64) acc = O::dot(O::load(W + static_cast<size_t>(r) * K + k), xf(k, ss), acc);
    acc = group_sum<8>(acc);
    if (sub == 0 && grp + ri * NGR < N) epi(grp + ri * NGR, acc);
  }
}

// 1 / rms(y) over D values in LDS, computed by every wave on its own.
template <int D>
__device__ __forceinline__ float wave_rms_inv(const float* __restrict__ y, float eps) {
  const int lane = tid_here() & 63;
  float ss = 0.f;
#pragma unroll
  for (int c = lane; c < D; c += 64) ss += y[c] * y[c];
  ss = group_sum<64>(ss);
  return rsq_hw(ss / static_cast<float>(D) + eps);
}

// Operand chunk k..k+8 of g * y in the storage precision; adds sum(y^2) of the chunk to ss.
template <typename WT>
__device__ __forceinline__ typename Ops<WT>::Chunk gain_chunk(const float* __restrict__ y, const float* __restrict__ g,
                                                              int k, float& ss) {
  const float4 y0 = *reinterpret_cast<const float4*>(y + k), y1 = *reinterpret_cast<const float4*>(y + k + 4);
  const float4 g0 = *reinterpret_cast<const float4*>(g + k), g1 = *reinterpret_cast<const float4*>(g + k + 4);
  ss += y0.x * y0.x; ss += y0.y * y0.y; ss += y0.z * y0.z; ss += y0.w * y0.w;
  ss += y1.x * y1.x; ss += y1.y * y1.y; ss += y1.z * y1.z; ss += y1.w * y1.w;
  const float f[8] = {g0.x * y0.x, g0.y * y0.y, g0.z * y0.z, g0.w * y0.w,
                      g1.x * y1.x, g1.y * y1.y, g1.z * y1.z, g1.w * y1.w};
  return Ops<WT>::pack(f);
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
  const void* mem_v;     // [G][B][H][T8/8][DH][8]
  float* s_out;          // [B][n][D] or null
  int B, T, T8, t0, n, L, F, F2, Wm1, G, ffn_kind;
  float eps;
};

// Memory row blocks (of SLOTS rows) per attention wave and chunk; weight chunks per product
// buffer and for the gated merge (kept resident).  bf16: 4 VGPRs per chunk, fp32: 8.
template <typename WT> constexpr int kq_of() { return sizeof(WT) == 2 ? 7 : 2; }
template <typename WT> constexpr int cbx_of() { return sizeof(WT) == 2 ? 8 : 2; }
template <typename WT> constexpr int cbz_of() { return sizeof(WT) == 2 ? 6 : 3; }
constexpr unsigned al16(unsigned x) { return (x + 15u) / 16u * 16u; }

// LDS plan.  The buffers whose size depends only on (storage type, D, DH) come first at
// compile-time offsets; the gains, the operand vector and the window caches follow.
template <int ESZ, int D, int DH, int KQ>
struct Fixed {
  static constexpr unsigned H = D / DH, SLOTS = 64 / (DH / 16);
  static constexpr unsigned eb = 0;                                 // e_t
  static constexpr unsigned sb = al16(eb + D * ESZ);                 // s_{t0-1} operand of the first step
  static constexpr unsigned y0 = al16(sb + D * ESZ);                 // residual stream, two buffers
  static constexpr unsigned y1 = al16(y0 + D * 4);
  static constexpr unsigned kv = al16(y1 + D * 4);                   // current key, value
  static constexpr unsigned qb = al16(kv + 2 * D * 4);               // query (self or cross)
  static constexpr unsigned kcb = al16(qb + D * ESZ);                // current key, storage precision
  static constexpr unsigned bg = al16(kcb + D * ESZ);
  static constexpr unsigned CPS = DH + 4;                           // partial state: m, l, -, -, o[DH]
  static constexpr unsigned cpart = al16(bg + D * 4);                // cross partial states per attention wave
  static constexpr unsigned pbuf = al16(cpart + NA * CPS * 4);       // cross weights per attention wave
  static constexpr unsigned PSW = WCAP + 8;                         // window entries per head, padded
  static constexpr unsigned sws = al16(pbuf + NA * KQ * SLOTS * ESZ);    // window scores per head (fp32)
  static constexpr unsigned swp = al16(sws + H * PSW * 4);           // window weights per head
  static constexpr unsigned opart = al16(swp + H * PSW * ESZ);      // W_O partials per head [H][D] fp32
  static constexpr unsigned yb = al16(opart + H * D * 4);            // residual after the W_O partials
  // merge weights [D][3D] (W_gate row | W_fb row) in LDS for bf16 at d = 64, so the product
  // waves' registers can hold a separate QKV buffer
  static constexpr bool MLDS = ESZ == 2 && D == 64;
  static constexpr unsigned wm = al16(yb + D * 4);
  static constexpr unsigned end = al16(wm + (MLDS ? 3 * D * D * ESZ : 0));
};
struct SmemTail {
  unsigned gains, xop, wo, ring, total;
};
// Window caches in LDS: keys [L][H][Wm1][DH] (row per ring slot), values key-blocked
// [L][H][NB][DH][8] with NB = ceil(Wm1 / 8) (slots past Wm1 stay zero).
__host__ __device__ inline SmemTail smem_tail(unsigned fixed_end, int D, int DH, int L, int Wm1, int F, int esz) {
  SmemTail p{};
  const unsigned nb = (Wm1 + 7) / 8;
  p.gains = fixed_end;                                               // self, cross, ffn per layer, final
  p.xop = al16(p.gains + (3u * L + 1u) * D * 4u);                    // attention output, FFN activation
  p.wo = al16(p.xop + static_cast<unsigned>(F > D ? F : D) * esz);    // W_O of every layer [L][D][D]
  p.ring = al16(p.wo + static_cast<unsigned>(L) * D * D * esz);
  p.total = al16(p.ring + static_cast<unsigned>(L) * (D / DH) * (Wm1 + 8u * nb) * DH * esz);
  return p;
}

template <typename WT, int D, int DH>
__global__ __launch_bounds__(NT) void dec_small_k(DecSmallParams p) {
  using O = Ops<WT>;
  using Chunk = typename O::Chunk;
  constexpr int H = D / DH;
  constexpr int LPK = DH / 16;            // lanes per key row (16 elements each)
  constexpr int SLOTS = 64 / LPK;         // keys per wave pass
  constexpr int WPH = NA / H;             // attention waves per head
  constexpr int KQ = kq_of<WT>();         // memory row blocks per attention wave and chunk
  constexpr int RW = KQ * SLOTS;          // memory rows per attention wave and chunk
  constexpr int R1 = WPH * RW;            // memory rows per chunk and head
  constexpr int TOP = DH < 64 ? 64 - DH : 0;   // first lane holding a summed P.V dimension
  constexpr int CPD = D / 64;             // chunks per lane of a K = D product (8 lanes per row)
  constexpr int CBX = cbx_of<WT>(), CBZ = cbz_of<WT>();
  constexpr int MGR = NTM / 8;            // 8-lane groups of the product waves
  constexpr int MRG = D / MGR;            // merge rows per group
  using FX = Fixed<sizeof(WT), D, DH, KQ>;
  static_assert(DH % 16 == 0 && DH <= 128 && H <= NA && NA % H == 0, "head shape");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int b = blockIdx.x;
  const int L = p.L, Wm1 = p.Wm1, T = p.T, F = p.F;
  const float qscale = kLog2e / sqrtf(static_cast<float>(DH));
  const SmemTail sp = smem_tail(FX::end, D, DH, L, Wm1, F, sizeof(WT));
  const int rpl = H * Wm1 * DH;            // key ring elements per layer (and per layer in the state)
  const int nbw = (Wm1 + 7) / 8;           // value blocks of the ring
  const int vpl = H * nbw * 8 * DH;        // value ring elements per layer (key-blocked)
  WT* ringK = reinterpret_cast<WT*>(smem + sp.ring);
  WT* ringV = ringK + L * rpl;
  WT* xop = reinterpret_cast<WT*>(smem + sp.xop);
  WT* wol = reinterpret_cast<WT*>(smem + sp.wo);
  float* gains = reinterpret_cast<float*>(smem + sp.gains);
  float* opart = reinterpret_cast<float*>(smem + FX::opart);
  float* yb = reinterpret_cast<float*>(smem + FX::yb);
  WT* wml = reinterpret_cast<WT*>(smem + FX::wm);
  WT* eb = reinterpret_cast<WT*>(smem + FX::eb);
  WT* sb = reinterpret_cast<WT*>(smem + FX::sb);
  float* y0 = reinterpret_cast<float*>(smem + FX::y0);
  float* y1 = reinterpret_cast<float*>(smem + FX::y1);
  float* kv = reinterpret_cast<float*>(smem + FX::kv);
  WT* qb = reinterpret_cast<WT*>(smem + FX::qb);
  WT* kcb = reinterpret_cast<WT*>(smem + FX::kcb);
  float* bgl = reinterpret_cast<float*>(smem + FX::bg);
  float* sws = reinterpret_cast<float*>(smem + FX::sws);
  WT* swp = reinterpret_cast<WT*>(smem + FX::swp);
  WT* pbuf = reinterpret_cast<WT*>(smem + FX::pbuf);
  float* cpart = reinterpret_cast<float*>(smem + FX::cpart);
  const float* g_fin = gains + 3 * L * D;

  // ---- carried state, gains, first e ----
  const WT* e_seq = static_cast<const WT*>(p.e) + static_cast<size_t>(b) * T * D;
  {
    const int tid = threadIdx.x;
    const WT* gk = static_cast<const WT*>(p.ring_k);
    const WT* gv = static_cast<const WT*>(p.ring_v);
    for (int l = 0; l < L; ++l) {
      const size_t src = (static_cast<size_t>(l) * p.B + b) * rpl;
      for (int i = tid; i < rpl; i += NT) ringK[l * rpl + i] = gk[src + i];
      // values: state rows [H][Wm1][DH] -> key-blocked [H][NB][DH][8], padding slots zero
      for (int i = tid; i < vpl; i += NT) {
        const int k8 = i % 8, d = (i / 8) % DH, blk = (i / (8 * DH)) % nbw, h = i / (8 * DH * nbw);
        const int sl = blk * 8 + k8;
        WT v{};
        if (sl < Wm1) v = gv[src + (h * Wm1 + sl) * DH + d];
        ringV[l * vpl + i] = v;
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
      store_from_f32(&sb[c], p.s[static_cast<size_t>(b) * D + c]);
    }
    if (tid * 8 < D) O::store(eb + tid * 8, O::load(e_seq + static_cast<size_t>(p.t0) * D + tid * 8));
  }
  const WT* wgate = static_cast<const WT*>(p.wgate);
  const WT* wfb = static_cast<const WT*>(p.wfb);
  auto layer_w = [&](int l, size_t off) {
    return reinterpret_cast<const WT*>(p.layers + static_cast<size_t>(l) * p.layer_stride + off);
  };
  auto is_attn = [&]() { return __builtin_amdgcn_readfirstlane(tid_here() >> 6) < NA; };
  // W_O of every layer stays in LDS: the window-attention wave of head h multiplies its
  // output by columns h*DH.. of W_O right after computing it
  if constexpr (FX::MLDS) {
    const WT* wg = static_cast<const WT*>(p.wgate);
    const WT* wf = static_cast<const WT*>(p.wfb);
    for (int i = threadIdx.x * 8; i < 3 * D * D; i += NT * 8) {
      const int r = i / (3 * D), c = i % (3 * D);
      O::store(wml + i, O::load(c < 2 * D ? wg + r * 2 * D + c : wf + r * D + c - 2 * D));
    }
  }
  for (int l = 0; l < L; ++l) {
    const WT* src = layer_w(l, p.l_wo);
    for (int i = threadIdx.x * 8; i < D * D; i += NT * 8) O::store(wol + l * D * D + i, O::load(src + i));
  }

  // The two roles run their own step loops; both pass the same sequence of workgroup
  // barriers (one per phase: merge, then P1, P2, P4, P5, P7, P8, P9 per layer), so each
  // role's registers are allocated for its own work only.
  if (is_attn()) {
    // ======== attention waves: memory rows (key rows R[2i + c], value items
    // R[2KQ + 2i + r] of block i), window attention, cross-attention (partial softmax
    // states per wave; the product waves combine them in the W_Ox operand fetch) ========
    Chunk R[4 * KQ];
    // Attention wave w takes head w % H and share w / H of the rows of a chunk: rows
    // c0 + share*RW + i*SLOTS + slot (i < KQ) for the scores, and for the P.V pass the
    // value items (dim, 8-key block) lane + 64r of each block of SLOTS rows.  A wave whose
    // first row lies past the position has nothing to do.
    auto mem_load = [&](int l, int tpos, int c0, auto i0c, auto i1c) {
      constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
      const unsigned tid = tid_here();
      const int lane = tid & 63;
      const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
      const int mh = wave % H, mpart = wave / H;
      const int jw = c0 + mpart * RW;   // first row of the wave (uniform)
      if (jw > tpos) return;
      const int mslot = lane / LPK, msub = lane % LPK;
      const int g = p.G == 1 ? 0 : l;
      const WT* kb = static_cast<const WT*>(p.mem_k) + ((static_cast<size_t>(g) * p.B + b) * H + mh) *
                                                          static_cast<size_t>(T) * DH;
      const WT* vb = static_cast<const WT*>(p.mem_v) + ((static_cast<size_t>(g) * p.B + b) * H + mh) *
                                                          static_cast<size_t>(p.T8) * DH;
      const int nb8 = p.T8 / 8;
#pragma unroll
      for (int i = I0; i < I1; ++i) {
        const int jb = jw + i * SLOTS;
        const int j = min(jb + mslot, tpos);   // rows past the position are loaded but masked
        R[2 * i] = O::load(at(kb, j * DH + msub * 16));
        R[2 * i + 1] = O::load(at(kb, j * DH + msub * 16 + 8));
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int it = lane + 64 * r, d = it % DH, blk = it / DH;
          const int bi = min(jb / 8 + blk, nb8 - 1);
          R[2 * KQ + 2 * i + r] = O::load(at(vb, (bi * DH + d) * 8));
        }
      }
    };
    // rows of the next (layer, position), requested in the phases between two cross-attentions
    // (blocks [I0, I1) at each point) so the requests drain while the other phases run
    auto next_rows = [&](int l, int t, bool has_next, auto i0c, auto i1c) {
      if (l + 1 < L) mem_load(l + 1, t, 0, i0c, i1c);
      else if (has_next) mem_load(0, t + 1, 0, i0c, i1c);
    };
    // The KQ blocks are spread over six request points: P7, P8 and P9 of the previous layer, P1,
    // P2 and P4 of the layer itself; one block each, the remainder from P1 on.  Spreading them
    // keeps the vector-memory path free for the product waves' weight requests (measured: the
    // even spread beats requesting the rows early).
    constexpr auto req = [](int i) { return KQ / 6 + ((i + 3) % 6 < KQ % 6 ? 1 : 0); };
    constexpr int B1 = req(0), B2 = B1 + req(1), B3 = B2 + req(2), B4 = B3 + req(3), B5 = B4 + req(4);
    mem_load(0, p.t0, 0, IC<0>{}, IC<B3>{});
    __syncthreads();
    for (int step = 0; step < p.n; ++step) {
      const int t = p.t0 + step;
      const bool has_next = step + 1 < p.n;
      __syncthreads();   // merge
      for (int l = 0; l < L; ++l) {
        WT* rK = ringK + l * rpl;
        WT* rV = ringV + l * vpl;
        mem_load(l, t, 0, IC<B3>{}, IC<B4>{});
        __syncthreads();   // P1
        mem_load(l, t, 0, IC<B4>{}, IC<B5>{});

        // ---- P2: window self-attention, attention wave h for head h.  Scores with lanes
        //      over entries (ring slots 0..8*NB-1, valid below npast, then the current
        //      entry), weights exp2(s - max), P.V with lanes over (dim, 8-slot block). ----
        {
          const unsigned tid = tid_here();
          const int h = __builtin_amdgcn_readfirstlane(tid >> 6);
          if (h < H) {
            const int lane = tid & 63;
            const int slot = lane / LPK, sub = lane % LPK;
            const int npast = min(t, Wm1);        // cached entries in the window (slots 0..npast-1)
            const int ecur = nbw * 8;             // entry index of the current token
            float* ps = sws + h * FX::PSW;
            WT* pw = swp + h * FX::PSW;
            QVec<WT> q;
            q.load(qb + h * DH + sub * 16);
            auto score = [&](int e) {
              // ring slot e (padding slots: masked) or, for the current entry, its storage-precision copy
              const WT* kr = e < ecur ? rK + (h * Wm1 + min(e, Wm1 - 1)) * DH + sub * 16 : kcb + h * DH + sub * 16;
              const Chunk k0 = O::load(kr), k1 = O::load(kr + 8);
              float sc = q.dot(k0, k1);
              if constexpr (LPK > 1) sc = group_sum<LPK>(sc);
              return (e < npast || e == ecur) ? sc : -INFINITY;
            };
            float ls = 0.f, pcur = 0.f;
            if (ecur < SLOTS) {
              // one pass: every entry's score stays in its lane
              const int e = slot;
              const float sc = score(e);
              const float M = group_max<64>(sc);   // finite: the current entry is always present
              const float pr = round_to<WT>(fast_exp2(sc - M));
              if (sub == 0 && e <= ecur) {
                store_from_f32(&pw[e], pr);
                ls = pr;
              }
              // the current entry's weight, from the lane that computed it
              pcur = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr), ecur * LPK));
            } else {
              float mloc = -INFINITY;
              for (int e0 = 0; e0 <= ecur; e0 += SLOTS) {
                const int e = e0 + slot;
                const float sc = score(e);
                if (sub == 0 && e <= ecur) ps[e] = sc;
                mloc = fmaxf(mloc, sc);
              }
              const float M = group_max<64>(mloc);
              wave_sync_lds();
              for (int e = lane; e <= ecur; e += 64) {
                const float pr = round_to<WT>(fast_exp2(ps[e] - M));
                store_from_f32(&pw[e], pr);
                ls += pr;
              }
            }
            const float rls = rcp_hw(group_sum<64>(ls));
            wave_sync_lds();
            float oa = 0.f, ob = 0.f;
            for (int r = 0; lane + 64 * r < DH * nbw; ++r) {
              const int it = lane + 64 * r, d = it % DH, blk = it / DH;
              const Chunk pp = O::load(pw + blk * 8);
              const Chunk vv = O::load(rV + ((h * nbw + blk) * DH + d) * 8);
              if (DH < 128 || (r & 1) == 0) oa = O::dot(pp, vv, oa);
              else ob = O::dot(pp, vv, ob);
            }
            oa = sum_to_top_rows<DH>(oa);
            const float pc = ecur < SLOTS ? pcur : load_as_f32(pw + ecur);
            if (lane >= TOP) {
              const int d = lane - TOP;
              store_from_f32(&xop[h * DH + d], (oa + pc * kv[D + h * DH + d]) * rls);
            }
            if (DH == 128) store_from_f32(&xop[h * DH + 64 + lane], (ob + pc * kv[D + h * DH + 64 + lane]) * rls);
            wave_sync_lds();
            // W_O partial of this head: opart[h][r] = W_O[r, h*DH:(h+1)*DH] . attn_h, lanes over rows
            {
              const WT* wo = wol + l * D * D + h * DH;
#pragma unroll
              for (int r = lane; r < D; r += 64) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < DH; c += 8) acc = O::dot(O::load(wo + r * D + c), O::load(xop + h * DH + c), acc);
                opart[h * D + r] = acc;
              }
            }
            // the current entry replaces the oldest one (position t - (W-1)); all reads are done
            if (Wm1 > 0) {
              const int sl = t % Wm1;
              for (int c = lane; c < DH; c += 64) {
                store_from_f32(&rK[(h * Wm1 + sl) * DH + c], kv[h * DH + c]);
                store_from_f32(&rV[((h * nbw + sl / 8) * DH + c) * 8 + sl % 8], kv[D + h * DH + c]);
              }
            }
          }
        }
        __syncthreads();   // P2
        mem_load(l, t, 0, IC<B5>{}, IC<KQ>{});
        __syncthreads();   // P4

        // ---- P5: cross-attention over memory rows 0..t ----
        {
          const unsigned tid = tid_here();
          const int lane = tid & 63;
          const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
          const int mh = wave % H, mpart = wave / H;
          const int slot = lane / LPK, sub = lane % LPK;
          float m = -INFINITY, lsum = 0.f, oa = 0.f, ob = 0.f;
          WT* pw = pbuf + wave * KQ * SLOTS;
          if (mpart * RW <= t) {
            QVec<WT> q;
            q.load(qb + mh * DH + sub * 16);
            for (int c0 = 0; c0 <= t; c0 += R1) {
              const int jw = c0 + mpart * RW;
              if (jw > t) break;                   // no row of this wave in the chunk (uniform)
              if (c0 > 0) mem_load(l, t, c0, IC<0>{}, IC<KQ>{});
              float s[KQ];
              float cm = -INFINITY;
#pragma unroll
              for (int i = 0; i < KQ; ++i) {
                const int j = jw + i * SLOTS + slot;
                float a = -INFINITY;
                if (jw + i * SLOTS <= t) {         // uniform: the block has a row
                  a = q.dot(R[2 * i], R[2 * i + 1]);
                  if constexpr (LPK > 1) a = group_sum<LPK>(a);
                  a = j <= t ? a : -INFINITY;
                }
                s[i] = a;
                cm = fmaxf(cm, a);
              }
              cm = group_max<64>(cm);              // finite: row jw <= t is here
              const float mn = fmaxf(m, cm);
              const float corr = fast_exp2(m - mn);  // first chunk: m = -inf -> 0 (o, l are 0)
              lsum *= corr;
              oa *= corr;
              ob *= corr;
              m = mn;
              // blocks past the position are skipped; when every block of the wave has rows
              // the loops run without branches so the LDS reads can be issued together
              const bool full = jw + (KQ - 1) * SLOTS <= t;   // uniform
              auto pv_blocks = [&](auto fullc) {
#pragma unroll
                for (int i = 0; i < KQ; ++i) {
                  if (!decltype(fullc)::value && jw + i * SLOTS > t) break;   // uniform
                  const float pr = round_to<WT>(fast_exp2(s[i] - m));   // masked rows: 0
                  if (sub == 0) {
                    store_from_f32(&pw[i * SLOTS + slot], pr);
                    lsum += pr;
                  }
                }
                wave_sync_lds();
#pragma unroll
                for (int i = 0; i < KQ; ++i) {
                  if (!decltype(fullc)::value && jw + i * SLOTS > t) break;   // uniform
#pragma unroll
                  for (int r = 0; r < 2; ++r) {
                    const int blk = (lane + 64 * r) / DH;
                    const Chunk pp = O::load(pw + i * SLOTS + blk * 8);
                    if (DH < 128 || r == 0) oa = O::dot(pp, R[2 * KQ + 2 * i + r], oa);
                    else ob = O::dot(pp, R[2 * KQ + 2 * i + r], ob);
                  }
                }
                wave_sync_lds();
              };
              if (full) pv_blocks(std::true_type{});
              else pv_blocks(std::false_type{});
            }
            // lanes with the same dim hold different key blocks: sum them
            oa = sum_to_top_rows<DH>(oa);
            lsum = group_sum<64>(lsum);
          }
          float* cp = cpart + wave * FX::CPS;
          if (lane >= TOP) cp[4 + lane - TOP] = oa;
          if (DH == 128) cp[4 + 64 + lane] = ob;
          if (lane == 0) {
            cp[0] = m;
            cp[1] = lsum;
          }
        }
        __syncthreads();   // P5
        next_rows(l, t, has_next, IC<0>{}, IC<B1>{});
        __syncthreads();   // P7
        next_rows(l, t, has_next, IC<B1>{}, IC<B2>{});
        __syncthreads();   // P8
        next_rows(l, t, has_next, IC<B2>{}, IC<B3>{});
        __syncthreads();   // P9
      }
    }
  } else {
    // ======== product waves: the gated merge and every matrix-vector product.  The loop is
    // instantiated per FFN kind and FFN output-product shape (lanes per row, chunks per lane),
    // chosen once here, so every branch inside the step loop is on a compile-time shape and the
    // compiler tracks the outstanding weight requests exactly. ========
    dispatch_ffn_out(D, F, [&](auto glc, auto cplc) {
      auto body = [&](auto swc) {
        constexpr int GL2 = decltype(glc)::value, CPL2 = decltype(cplc)::value;
        constexpr bool SWI = decltype(swc)::value;
        // FFN width: a compile-time constant whenever the output product has a fixed shape
        const int Fw = CPL2 > 0 ? 8 * GL2 * CPL2 : F;
        // weight buffers: X: Qx, FFN in (and QKV unless it has its own); Y: Ox; U: FFN out; Q: QKV
        // when the whole plan fits the register budget; Z: merge (resident unless in LDS)
        constexpr int CBZE = FX::MLDS ? 0 : CBZ;
        constexpr int CBY = CBX < D / 32 * CPD ? CBX : D / 32 * CPD;
        constexpr int CBQ0 = CBX < 3 * D / 32 * CPD ? CBX : 3 * D / 32 * CPD;
        constexpr bool SEPQ = (CBQ0 + CBY + 2 * CBX + CBZE) * static_cast<int>(sizeof(Chunk) / 4) <= 128;
        constexpr int CBQ = SEPQ ? CBQ0 : CBX;
        Chunk X[CBX], Y[CBY], U[CBX], Z[CBZE > 0 ? CBZE : 1], Qs[SEPQ ? CBQ : 1];
        Chunk* Q = SEPQ ? Qs : X;
        auto merge_chunk = [&](int ri, int q) {
          const unsigned mt = mtid_here();
          const int sub = mt & 7, grp = mt >> 3;
          const int r = min(grp + ri * MGR, D - 1);   // rows past D (buffer slots beyond the merge): any row
          if constexpr (FX::MLDS) return O::load(wml + r * 3 * D + (sub + 8 * q) * 8);
          else
            return q < 2 * CPD ? O::load(at(wgate, r * 2 * D + (sub + 8 * q) * 8))
                               : O::load(at(wfb, r * D + (sub + 8 * (q - 2 * CPD)) * 8));
        };
#pragma unroll
        for (int pp = 0; pp < CBZE; ++pp) Z[pp] = merge_chunk(pp / (3 * CPD), pp % (3 * CPD));
        wpre<WT, 8, CPD, CBQ>(Q, layer_w(0, p.l_qkv), 3 * D);
        __syncthreads();
        for (int step = 0; step < p.n; ++step) {
          const int t = p.t0 + step;
          const bool has_next = step + 1 < p.n;
          float* y = (step & 1) ? y0 : y1;
          float* yprev = (step & 1) ? y1 : y0;
          Chunk e_next = O::zero();

          // ---- gated merge: y = g * e_t + (1 - g) * W_fb s_{t-1},
          //      g = sigmoid(W_gate [e_t; s_{t-1}] + b_g), s_{t-1} = RMS(y_prev; g_final) ----
          {
            const unsigned mt = mtid_here();
            if (has_next && mt * 8 < D) e_next = O::load(at(e_seq, (t + 1) * D + mt * 8));
            const int sub = mt & 7, grp = mt >> 3;
            // operand [e_t ; g_final * y_prev] (the s part is scaled by 1/rms(y_prev) after the
            // products, as in wmv); the first step takes s_{t0-1} as given
            Chunk xg[2 * CPD];
            float ss = 0.f;
#pragma unroll
            for (int ci = 0; ci < 2 * CPD; ++ci) {
              const int k = (sub + 8 * ci) * 8;
              xg[ci] = ci < CPD ? O::load(eb + k)
                                : (step > 0 ? gain_chunk<WT>(yprev, g_fin, k - D, ss) : O::load(sb + k - D));
            }
            const float inv = step > 0 ? rsq_hw(group_sum<8>(ss) / static_cast<float>(D) + p.eps) : 1.f;
            if (step > 0 && mt < D && p.s_out)
              p.s_out[(static_cast<size_t>(b) * p.n + step - 1) * D + mt] = g_fin[mt] * (yprev[mt] * inv);
            float mine = 0.f;
#pragma unroll
            for (int ri = 0; ri < MRG; ++ri) {
              float ge = 0.f, gsv = 0.f, fs = 0.f;
#pragma unroll
              for (int q = 0; q < 3 * CPD; ++q) {
                const int pp = ri * 3 * CPD + q;
                const Chunk w = pp < CBZE ? Z[pp < CBZE ? pp : 0] : merge_chunk(ri, q);
                if (q < CPD) ge = O::dot(w, xg[q], ge);
                else if (q < 2 * CPD) gsv = O::dot(w, xg[q], gsv);
                else fs = O::dot(w, xg[CPD + q - 2 * CPD], fs);
              }
              const float gs = group_sum<8>(ge) + group_sum<8>(gsv) * inv;
              fs = group_sum<8>(fs) * inv;
              const int r = grp + ri * MGR;
              const float g = sigmoid_hw(gs + bgl[r]);
              const float v = g * load_as_f32(eb + r) + (1.0f - g) * fs;
              mine = sub == ri ? v : mine;
            }
            if (sub < MRG) y[grp + sub * MGR] = mine;
          }
          __syncthreads();   // merge

          for (int l = 0; l < L; ++l) {
            const float* g_self = gains + l * D;
            const float* g_cross = gains + (L + l) * D;
            const float* g_ffn = gains + (2 * L + l) * D;
            const bool last = l + 1 == L;

            // ---- P1: q, k, v = W_{Q,K,V} RMS(y; g_self); q scaled by log2(e)/sqrt(d_h) ----
            {
              wmv<WT, 8, CPD, CBQ, true>(Q, layer_w(l, p.l_qkv), 3 * D,
                                         [&](int k, float& ss) { return gain_chunk<WT>(y, g_self, k, ss); },
                                         [&](int r, float v) {
                                           if (r < D) store_from_f32(&qb[r], v * qscale);
                                           else {
                                             kv[r - D] = round_to<WT>(v);
                                             if (r < 2 * D) store_from_f32(&kcb[r - D], v);
                                           }
                                         },
                                         p.eps);
              const unsigned mt = mtid_here();
              if (l == 0 && has_next && mt * 8 < D) O::store(eb + mt * 8, e_next);
            }
            __syncthreads();   // P1
            // the window attention runs: request the Q_x and W_Ox weights of this layer
            wpre<WT, 8, CPD, CBX>(X, layer_w(l, p.l_wqx), D);
            wpre<WT, 8, CPD, CBY>(Y, layer_w(l, p.l_wox), D);
            __syncthreads();   // P2

            // ---- P4: y_b = y + sum_h W_O[:, h] attn_h (the per-head partials of the window
            //      attention, added in head order; each product wave writes the whole vector, so
            //      its own reads see its own writes); q_x = W_Qx RMS(y_b; g_cross), scaled like q ----
            {
              const int lane = mtid_here() & 63;
#pragma unroll
              for (int c = lane; c < D; c += 64) {
                float v = y[c];
#pragma unroll
                for (int h = 0; h < H; ++h) v += opart[h * D + c];
                yb[c] = v;
              }
              wave_sync_lds();
              wmv<WT, 8, CPD, CBX, true>(X, layer_w(l, p.l_wqx), D,
                                         [&](int k, float& ss) { return gain_chunk<WT>(yb, g_cross, k, ss); },
                                         [&](int r, float v) { store_from_f32(&qb[r], v * qscale); }, p.eps);
            }
            __syncthreads();   // P4
            // the cross-attention runs: request the FFN weights
            if constexpr (!SWI) wpre<WT, 8, CPD, CBX>(X, layer_w(l, p.l_fin), Fw);
            else wpre_swiglu<WT, CPD, CBX>(X, layer_w(l, p.l_fin), Fw);
            if constexpr (CPL2 > 0) wpre<WT, GL2, CPL2, CBX>(U, layer_w(l, p.l_fout), D);
            if constexpr (SEPQ) wpre<WT, 8, CPD, CBQ>(Q, layer_w(last ? 0 : l + 1, p.l_qkv), 3 * D);
            __syncthreads();   // P5

            // ---- P7: y += W_Ox attn; the operand chunk (8 dims of one head) combines the WPH
            //      partial states of the head in a fixed order ----
            auto cross_out = [&](int k, float&) {
              const int h = k / DH, d0 = k % DH;
              float2 ml[WPH];   // (m, l) of every partial state first, for the common maximum
#pragma unroll
              for (int q = 0; q < WPH; ++q) ml[q] = *reinterpret_cast<const float2*>(cpart + (h + H * q) * FX::CPS);
              float M = -INFINITY;
#pragma unroll
              for (int q = 0; q < WPH; ++q) M = fmaxf(M, ml[q].x);
              float lt = 0.f, o[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
              for (int q = 0; q < WPH; ++q) {
                const float* cp = cpart + (h + H * q) * FX::CPS;
                const float4 a = *reinterpret_cast<const float4*>(cp + 4 + d0);
                const float4 c = *reinterpret_cast<const float4*>(cp + 8 + d0);
                const float w = fast_exp2(ml[q].x - M);   // wave without rows: m = -inf -> 0
                lt += w * ml[q].y;
                o[0] += w * a.x; o[1] += w * a.y; o[2] += w * a.z; o[3] += w * a.w;
                o[4] += w * c.x; o[5] += w * c.y; o[6] += w * c.z; o[7] += w * c.w;
              }
              const float rlt = rcp_hw(lt);
#pragma unroll
              for (int i = 0; i < 8; ++i) o[i] *= rlt;
              return O::pack(o);
            };
            wmv<WT, 8, CPD, CBY>(Y, layer_w(l, p.l_wox), D, cross_out, [&](int r, float v) { y[r] = yb[r] + v; });
            __syncthreads();   // P7

            // ---- P8: FFN input product (tied with encoder layer l), activation into xop ----
            {
              auto xf = [&](int k, float& ss) { return gain_chunk<WT>(y, g_ffn, k, ss); };
              if constexpr (!SWI) {
                wmv<WT, 8, CPD, CBX, true>(X, layer_w(l, p.l_fin), Fw, xf,
                                           [&](int r, float v) { store_from_f32(&xop[r], gelu_erf(v)); }, p.eps);
              } else {
                wmv_swiglu<WT, CPD, CBX>(X, layer_w(l, p.l_fin), Fw, xf, xop, p.eps);
              }
              if constexpr (!SEPQ) wpre<WT, 8, CPD, CBQ>(Q, layer_w(last ? 0 : l + 1, p.l_qkv), 3 * D);
            }
            __syncthreads();   // P8

            // ---- P9: y += W_2 act ----
            {
              auto xf = [&](int k, float&) { return O::load(xop + k); };
              auto epi = [&](int r, float v) { y[r] += v; };
              if constexpr (CPL2 > 0) wmv<WT, GL2, CPL2, CBX>(U, layer_w(l, p.l_fout), D, xf, epi);
              else wmv_any(layer_w(l, p.l_fout), D, F, xf, epi);
            }
            __syncthreads();   // P9
            (void)t;
          }
        }
      };
      if (p.ffn_kind == RLT_FFN_GELU) body(std::false_type{});
      else body(std::true_type{});
    });
  }

  // ---- s of the last step; window caches back to the state ----
  {
    const int tid = threadIdx.x;
    const float* yl = ((p.n - 1) & 1) ? y0 : y1;
    const float inv = wave_rms_inv<D>(yl, p.eps);
    if (tid < D) {
      const float v = g_fin[tid] * (yl[tid] * inv);
      if (p.s_out) p.s_out[(static_cast<size_t>(b) * p.n + p.n - 1) * D + tid] = v;
      p.s[static_cast<size_t>(b) * D + tid] = v;
    }
    WT* gk = static_cast<WT*>(p.ring_k);
    WT* gv = static_cast<WT*>(p.ring_v);
    for (int l = 0; l < L; ++l) {
      const size_t dst = (static_cast<size_t>(l) * p.B + b) * rpl;
      for (int i = tid; i < rpl; i += NT) {
        const int d = i % DH, sl = (i / DH) % Wm1, h = i / (DH * Wm1);
        gk[dst + i] = ringK[l * rpl + i];
        gv[dst + i] = ringV[l * vpl + ((h * nbw + sl / 8) * DH + d) * 8 + sl % 8];
      }
    }
  }
}

template <typename WT, int D, int DH>
size_t lds_bytes_t(const ModelLayout& m) {
  using FX = Fixed<sizeof(WT), D, DH, kq_of<WT>()>;
  return smem_tail(FX::end, D, DH, m.L, m.W - 1, m.F, static_cast<int>(sizeof(WT))).total;
}

size_t lds_bytes(const ModelLayout& m) {
  const bool bf = m.esz == 2;
#define RLT_LDS_CASE(D_, DH_)                                                           \
  if (m.D == D_ && m.DH == DH_) return bf ? lds_bytes_t<bf16_t, D_, DH_>(m) : lds_bytes_t<float, D_, DH_>(m);
  RLT_LDS_CASE(64, 16)
  RLT_LDS_CASE(64, 32)
  RLT_LDS_CASE(64, 64)
  RLT_LDS_CASE(128, 16)
  RLT_LDS_CASE(128, 32)
  RLT_LDS_CASE(128, 64)
  RLT_LDS_CASE(128, 128)
#undef RLT_LDS_CASE
  return ~size_t(0);
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
  p.B = a.B; p.T = a.T; p.T8 = s.T8; p.t0 = a.t0; p.n = a.n; p.L = m.L; p.F = m.F; p.F2 = m.F2; p.Wm1 = m.W - 1;
  p.G = m.G; p.ffn_kind = m.ffn_kind; p.eps = m.eps;
  const size_t lds = lds_bytes(m);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dec_small_k<WT, D, DH>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  dec_small_k<WT, D, DH><<<a.B, NT, lds, st>>>(p);
  return hipGetLastError();
}

}  // namespace

// The kernel's (storage type, d_model, head_dim) instances are spread over four translation
// units: the build compiles this file once per part (RLT_DEC_PART = 0..3), and part 0 also
// holds the host-side dispatch.  Without RLT_DEC_PART one unit holds everything.
#define RLT_DEC_SIG(I)                                                                         \
  __attribute__((visibility("hidden"))) hipError_t dec_small_launch_##I(                       \
      const ModelLayout& m, const StateLayout& s, const DecSmallArgs& a, hipStream_t st)
#define RLT_DEC_DEFINE(I, WT_, D_, DH_) \
  RLT_DEC_SIG(I) { return launch_t<WT_, D_, DH_>(m, s, a, st); }
#define RLT_DEC_DECLARE(I) RLT_DEC_SIG(I);

#if !defined(RLT_DEC_PART) || RLT_DEC_PART == 0
RLT_DEC_DEFINE(0, float, 64, 16)
RLT_DEC_DEFINE(1, bf16_t, 64, 16)
RLT_DEC_DEFINE(2, float, 64, 32)
RLT_DEC_DEFINE(3, bf16_t, 64, 32)
#endif
#if !defined(RLT_DEC_PART) || RLT_DEC_PART == 1
RLT_DEC_DEFINE(4, float, 64, 64)
RLT_DEC_DEFINE(5, bf16_t, 64, 64)
RLT_DEC_DEFINE(6, float, 128, 16)
RLT_DEC_DEFINE(7, bf16_t, 128, 16)
#endif
#if !defined(RLT_DEC_PART) || RLT_DEC_PART == 2
RLT_DEC_DEFINE(8, float, 128, 32)
RLT_DEC_DEFINE(9, bf16_t, 128, 32)
RLT_DEC_DEFINE(10, float, 128, 64)
#endif
#if !defined(RLT_DEC_PART) || RLT_DEC_PART == 3
RLT_DEC_DEFINE(11, bf16_t, 128, 64)
RLT_DEC_DEFINE(12, float, 128, 128)
RLT_DEC_DEFINE(13, bf16_t, 128, 128)
#endif

#if !defined(RLT_DEC_PART) || RLT_DEC_PART == 0
RLT_DEC_DECLARE(4) RLT_DEC_DECLARE(5) RLT_DEC_DECLARE(6) RLT_DEC_DECLARE(7) RLT_DEC_DECLARE(8)
RLT_DEC_DECLARE(9) RLT_DEC_DECLARE(10) RLT_DEC_DECLARE(11) RLT_DEC_DECLARE(12) RLT_DEC_DECLARE(13)

constexpr size_t kMaxLds = 160 * 1024;

bool dec_small_supported(const ModelLayout& m, int T) {
  const bool shape = (m.D == 64 && (m.DH == 16 || m.DH == 32 || m.DH == 64)) ||
                     (m.D == 128 && (m.DH == 16 || m.DH == 32 || m.DH == 64 || m.DH == 128));
  // the window ring (W-1 slots plus the current entry) is scanned whole every step
  // 32-bit memory-row offsets within one (group, sequence), value blocks included
  const size_t t8 = (static_cast<size_t>(T) + 7) / 8 * 8;
  const bool offsets = t8 * m.D * m.esz < (size_t(1) << 31);
  // SwiGLU pairs of 16 rows; FFN widths in whole 64-element chunks
  const bool ffn = m.F % 64 == 0 && (m.ffn_kind == RLT_FFN_GELU || m.F % 16 == 0);
  return shape && m.W <= WCAP && offsets && ffn && m.F2 <= 4096 && lds_bytes(m) <= kMaxLds;
}

size_t dec_small_lds_bytes(const ModelLayout& m, int T) {
  (void)T;
  return lds_bytes(m);
}

hipError_t launch_dec_small(const ModelLayout& m, const StateLayout& s, const DecSmallArgs& a, hipStream_t st) {
  if (!dec_small_supported(m, a.T)) return hipErrorInvalidValue;
  const int bf = m.dtype == RLT_DTYPE_BF16 ? 1 : 0;
  static const int kD[7] = {64, 64, 64, 128, 128, 128, 128};
  static const int kDH[7] = {16, 32, 64, 16, 32, 64, 128};
  using Fn = hipError_t (*)(const ModelLayout&, const StateLayout&, const DecSmallArgs&, hipStream_t);
  static const Fn kFn[14] = {dec_small_launch_0,  dec_small_launch_1,  dec_small_launch_2,  dec_small_launch_3,
                             dec_small_launch_4,  dec_small_launch_5,  dec_small_launch_6,  dec_small_launch_7,
                             dec_small_launch_8,  dec_small_launch_9,  dec_small_launch_10, dec_small_launch_11,
                             dec_small_launch_12, dec_small_launch_13};
  for (int c = 0; c < 7; ++c)
    if (m.D == kD[c] && m.DH == kDH[c]) return kFn[2 * c + bf](m, s, a, st);
  return hipErrorInvalidValue;
}
#endif

}  // namespace rlt
