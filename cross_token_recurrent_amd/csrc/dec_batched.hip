// Batched recurrent decoder for large d_model: every step is a fixed sequence of
// B-batched kernels enqueued on the caller's stream (no host synchronisation).
//
// Pages: [FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer"
// (decoder-state paragraph; model-hardware co-design principle: the transition is
// sequential within a sequence while ready updates of independent sequences share one
// batched kernel); [DS] deepsonar "技术拆解 009｜RLT…" §2.2, §2.4.
//
// At d_model >= 1024 one step streams the tied layer weights (hundreds of MB) and, late in
// the sequence, every sequence's encoder memory (tens of GB), so each phase is a
// device-wide kernel:
//   merge:   gpre = [e_t; s] W_gate^T, f = s W_fb^T (MFMA GEMMs), y = g*e + (1-g)*f
//   layer l: h = RMS(y) -> qkv = h W_{Q,K,V}^T -> window attention (one wave per
//            (sequence, head), ring buffer in HBM) -> y += attn W_O^T
//            h = RMS(y) -> q_x = h W_Qx^T -> cross-attention split over key chunks (one
//            wave per (chunk, head, sequence), partial softmax states) -> fixed-order
//            combine -> y += attn W_Ox^T
//            h = RMS(y) -> FFN GEMMs (GELU or SwiGLU epilogue) -> y += act W_2^T
//   final:   s_t = RMS(y; g_dec_final)
// Decoder scratch layout (inside the state's decoder scratch region):
//   y fp32 [B][D] | h [B][D] | xin [B][2D] | gpre fp32 [B][D] | fb fp32 [B][D] |
//   qkv fp32 [B][3D] | attn [B][D] | act [B][F] | part fp32 [B][H][NSMAX][DH+2]
#include <algorithm>

#include "act_layout.h"
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int KCHUNK = 256;   // memory rows per cross-attention work item
constexpr int kWideCombineSplits = 16;   // splits from which the 256-thread combine is faster
// Whether the step runs on the weight-streaming products (wstream.hip) or the tiled ones.
bool use_wst(const ModelLayout& m, int B) {
  return m.has_frag && m.dtype == RLT_DTYPE_BF16 && B <= 512 && m.D <= 2048 && m.D % 64 == 0 && m.F % 32 == 0;
}

// Rows of the products' fragment-major operands (whole 64-row groups, so that every row-group
// size the products choose stays inside them) and the row stride of their sums-of-squares arrays.
int padded_rows(int B) { return (B + 63) / 64 * 64; }
int ss_stride(int B) { return (B + 63) / 64 * 64; }

struct Scratch {
  size_t y, h, xin, gpre, fb, qkv, attn, act, part, splitk, ssp, cnt, xcnt, total;
  size_t cnt_bytes;
  int nsmax;
};

Scratch scratch_layout(const ModelLayout& m, int B, int T) {
  Scratch s{};
  // activation operands are padded to the row blocks / row groups of the weight-streaming
  // products' fragment-major layout (the padding rows are never read into a stored result)
  const size_t D = m.D, Bz = B, Bp = padded_rows(B), e = m.esz;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  s.nsmax = (T + KCHUNK - 1) / KCHUNK;
  s.y = take(Bz * D * 4);
  s.h = take(Bp * D * e);
  s.xin = take(Bp * 2 * D * e);
  s.gpre = take(Bz * D * 4);
  s.fb = take(Bz * D * 4);
  s.qkv = take(Bz * 3 * D * 4);
  s.attn = take(Bp * D * e);
  s.act = take(Bp * static_cast<size_t>(m.F) * e);
  s.part = take(Bz * m.H * static_cast<size_t>(s.nsmax) * (m.DH + 2) * 4);
  s.splitk = take(use_wst(m, B) ? 0 : gemm_splitk_ws_floats(B, m.D) * 4);   // tiled products only
  // weight-streaming products: per-16-column-block row sums of squares, [D/16][ss_stride(B)]
  s.ssp = take(use_wst(m, B) ? D / 16 * ss_stride(B) * 4 : 0);
  // arrival counters of the cross-attention heads, zeroed by the state's reset
  s.cnt = s.xcnt = off;
  s.cnt_bytes = Bz * m.H * 4;
  take(s.cnt_bytes);
  s.total = off;
  return s;
}

// xin[b] = [e_t[b] ; storage(s[b])]
template <typename WT>
__global__ void merge_prep_k(const WT* __restrict__ e, const float* __restrict__ s, WT* __restrict__ xin, int T,
                             int D, int t) {
  const int b = blockIdx.x;
  const WT* er = e + (static_cast<size_t>(b) * T + t) * D;
  WT* xr = xin + static_cast<size_t>(b) * 2 * D;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    xr[c] = er[c];
    store_from_f32(&xr[D + c], s[static_cast<size_t>(b) * D + c]);
  }
}

// y = g * e + (1 - g) * f with g = sigmoid(gpre + b_g)
template <typename WT>
__global__ void merge_combine_k(const float* __restrict__ gpre, const float* __restrict__ fb,
                                const float* __restrict__ bg, const WT* __restrict__ xin, float* __restrict__ y,
                                int D) {
  const int b = blockIdx.x;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    const size_t i = static_cast<size_t>(b) * D + c;
    const float g = sigmoid_f(gpre[i] + bg[c]);
    y[i] = g * load_as_f32(xin + static_cast<size_t>(b) * 2 * D + c) + (1.0f - g) * fb[i];
  }
}

// s = RMS(y; g) -> state s and s_out[b][step]; one wave per row
__global__ void final_norm_k(const float* __restrict__ y, const float* __restrict__ gain, float* __restrict__ s,
                             float* __restrict__ s_out, int B, int D, float eps, int step, int n) {
  const int row = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= B) return;
  const float* yr = y + static_cast<size_t>(row) * D;
  float ss = 0.f;
  for (int c = lane; c < D; c += 64) ss += yr[c] * yr[c];
  ss = group_sum<64>(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  for (int c = lane; c < D; c += 64) {
    const float v = gain[c] * (yr[c] * inv);
    s[static_cast<size_t>(row) * D + c] = v;
    if (s_out) s_out[(static_cast<size_t>(row) * n + step) * D + c] = v;
  }
}

template <typename WT> struct Row16;   // 16 stored elements of a key/value row as fp32
template <> struct Row16<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float (&f)[16]) {
    float a[8];
    load8(p, a);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = a[i];
    load8(p + 8, a);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[8 + i] = a[i];
  }
};
template <> struct Row16<float> {
  static __device__ __forceinline__ void load(const float* p, float (&f)[16]) {
    float a[8];
    load8(p, a);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = a[i];
    load8(p + 8, a);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[8 + i] = a[i];
  }
};

// Per-lane online softmax state over 16 output dims.
struct SoftState {
  float m = -INFINITY, l = 0.f, o[16];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] = 0.f;
  }
  // score s (already masked to -inf when invalid), value row v
  __device__ __forceinline__ void add(float s, const float (&v)[16]) {
    const float mn = fmaxf(m, s);
    if (mn == -INFINITY) return;   // nothing valid yet (uniform within a key group)
    const float corr = m == mn ? 1.f : __expf(m - mn);
    const float w = __expf(s - mn);
    l = l * corr + w;
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] = o[c] * corr + w * v[c];
    m = mn;
  }
};

// Combine the per-lane states of one wave (lanes = (slot, sub), sub = lane % LPK owns dims
// 16*sub .. 16*sub+15) into (m, l, o[DH]) of the whole wave, written by lanes 0..DH-1 to
// m_out / l_out / o_out (or finished as o / l into out when out != null).
template <int DH>
__device__ __forceinline__ void wave_finish(const SoftState& st, float* __restrict__ lds, float* __restrict__ m_out,
                                            float* __restrict__ l_out, float* __restrict__ o_out,
                                            float* __restrict__ out_f, int lane) {
  constexpr int LPK = DH / 16;
  constexpr int SLOTS = 64 / LPK;
  const float mw = group_max<64>(st.m);
  const float f = mw == -INFINITY ? 0.f : __expf(st.m - mw);
  float* ob = lds;              // [64][17]
  float* lb = lds + 64 * 17;    // [64]
#pragma unroll
  for (int c = 0; c < 16; ++c) ob[lane * 17 + c] = st.o[c] * f;
  lb[lane] = st.l * f;
  __syncthreads();
  for (int d = lane; d < DH; d += 64) {
    const int sub = d / 16, c = d % 16;
    float acc = 0.f, lacc = 0.f;
#pragma unroll 8
    for (int s = 0; s < SLOTS; ++s) {
      acc += ob[(s * LPK + sub) * 17 + c];
      lacc += lb[s * LPK];
    }
    if (out_f) {
      out_f[d] = acc / lacc;
    } else {
      o_out[d] = acc;
      if (d == 0) {
        *m_out = mw;
        *l_out = lacc;
      }
    }
  }
}

// Window self-attention, one workgroup of SWA_WAVES waves per (head, sequence): each wave takes a
// contiguous share of the window entries with its own online softmax, and wave 0 combines the
// waves' (m, l, o) in wave order.  Several waves only pay when (head, sequence) pairs are few.
template <typename WT, int DH, int SWA_WAVES>
__global__ __launch_bounds__(64 * SWA_WAVES) void swa_k(const float* __restrict__ qkv, WT* __restrict__ ring_k,
                                                        WT* __restrict__ ring_v, WT* __restrict__ attn, int B, int H,
                                                        int Wm1, int t, float scale, int xf) {
  constexpr int LPK = DH / 16;
  constexpr int SLOTS = 64 / LPK;
  __shared__ float lds[SWA_WAVES][64 * 17 + 64];
  __shared__ float pm[SWA_WAVES], pl[SWA_WAVES], po[SWA_WAVES][DH];
  const int h = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int slot = lane / LPK, sub = lane % LPK;
  const int D = H * DH;
  const float* qr = qkv + static_cast<size_t>(b) * 3 * D + h * DH + sub * 16;
  float q[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) q[c] = qr[c] * scale;
  const int npast = min(t, Wm1);
  const int ne = npast + 1;
  const int slot0 = Wm1 > 0 ? (t - npast) % Wm1 : 0;
  const size_t rbase = ((static_cast<size_t>(b) * H + h) * Wm1) * DH;   // ring is pre-offset to layer l
  // the current entry (position t), in the storage precision of the ring
  float kc[16], vc[16];
  {
    const float* kr = qkv + static_cast<size_t>(b) * 3 * D + D + h * DH + sub * 16;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      kc[c] = round_to<WT>(kr[c]);
      vc[c] = round_to<WT>(kr[D + c]);
    }
  }
  SoftState st;
  st.init();
  // this wave's entries [e0, e1); i < npast come from the ring, i == npast is the current one;
  // ring slots are clamped so that every load is unconditional, and four rounds are unrolled
  // so their loads are in flight together
  const int share = ((ne + SWA_WAVES - 1) / SWA_WAVES + SLOTS - 1) / SLOTS * SLOTS;
  const int e0 = wave * share, e1 = min(e0 + share, ne);
  for (int i0 = e0; i0 < e1; i0 += 4 * SLOTS) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + r * SLOTS + slot;
      float k[16], v[16];
      if (npast > 0) {
        int sl = slot0 + min(i, npast - 1);
        sl = sl >= Wm1 ? sl - Wm1 : sl;
        Row16<WT>::load(ring_k + rbase + static_cast<size_t>(sl) * DH + sub * 16, k);
        Row16<WT>::load(ring_v + rbase + static_cast<size_t>(sl) * DH + sub * 16, v);
      }
      const bool cur = i >= npast;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        k[c] = cur ? kc[c] : k[c];
        v[c] = cur ? vc[c] : v[c];
      }
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) a += q[c] * k[c];
      a = group_sum<LPK>(a);
      st.add(i < e1 ? a : -INFINITY, v);
    }
  }
  wave_finish<DH>(st, lds[wave], &pm[wave], &pl[wave], po[wave], nullptr, lane);
  __syncthreads();
  if (wave == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < SWA_WAVES; ++w) M = fmaxf(M, pm[w]);
    for (int d = lane; d < DH; d += 64) {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < SWA_WAVES; ++w) {
        const float f = pm[w] == -INFINITY ? 0.f : __expf(pm[w] - M);
        num += po[w][d] * f;
        den += pl[w] * f;
      }
      store_from_f32(&attn[act_offset(b, h * DH + d, D, xf)], num / den);
    }
  }
  // the current entry replaces the oldest one (position t - (W-1)); every read of the ring
  // happened before the barrier above
  if (Wm1 > 0) {
    const int sl = t % Wm1;
    const float* kr = qkv + static_cast<size_t>(b) * 3 * D + D + h * DH;
    for (int d = threadIdx.x; d < DH; d += 64 * SWA_WAVES) {
      store_from_f32(&ring_k[rbase + static_cast<size_t>(sl) * DH + d], kr[d]);
      store_from_f32(&ring_v[rbase + static_cast<size_t>(sl) * DH + d], kr[D + d]);
    }
  }
}

// Window self-attention, two-pass: one workgroup per (head, sequence), wave w takes window
// entries [KW w, KW w + KW).  Every key and value row of the wave's entries is requested at
// once (lanes = (slot, 16-dim part), so one load instruction covers SLOTS whole rows), then
// scores -> workgroup max -> exp(s - M) -> P.V over the same registers; the lanes' partial sums
// are folded over slots with lane exchanges, and the waves' sums in wave order, so the result
// does not depend on timing.  Entries past the window are loaded clamped and masked.
template <typename WT> struct SwaKw { static constexpr int v(int DH) { return DH == 128 ? 32 : 64; } };
template <> struct SwaKw<float> { static constexpr int v(int DH) { return DH >= 64 ? 32 : 64; } };

// 16 stored elements of a row as loaded (two 16-byte pieces for bf16, four for fp32), converted
// to fp32 where they are used, so the registers hold the storage precision.
template <typename WT> struct Raw16 {
  static constexpr int N = 16 * sizeof(WT) / 16;
  uint4 v[N];
  __device__ __forceinline__ void load(const WT* p) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ __forceinline__ float get(int c) const {
    if constexpr (sizeof(WT) == 2) {
      const uint4 q = v[c / 8];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
      const uint32_t x = w[(c % 8) / 2];
      return __uint_as_float(c % 2 ? (x & 0xffff0000u) : (x << 16));
    } else {
      const uint4 q = v[c / 4];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
      return __uint_as_float(w[c % 4]);
    }
  }
};

template <typename WT, int DH>
__global__ __launch_bounds__(512) void swa2_k(const float* __restrict__ qkv, WT* __restrict__ ring_k,
                                               WT* __restrict__ ring_v, WT* __restrict__ attn, int H, int Wm1, int t,
                                               float scale, int xf) {
  constexpr int LPK = DH / 16;              // lanes per key row (16 dims each)
  constexpr int SLOTS = 64 / LPK;           // rows per load instruction
  constexpr int KW = SwaKw<WT>::v(DH);      // entries per wave
  constexpr int KPL = KW / SLOTS;           // entries per lane
  __shared__ float wmax[8], pl[8], po[8][DH];
  const int h = blockIdx.x, b = blockIdx.y;
  const int nw = blockDim.x / 64, wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int slot = lane / LPK, sub = lane % LPK;
  const int D = H * DH;
  const int npast = min(t, Wm1), ne = npast + 1;
  const int slot0 = Wm1 > 0 ? (t - npast) % Wm1 : 0;
  const size_t rbase = ((static_cast<size_t>(b) * H + h) * Wm1) * DH;   // ring is pre-offset to layer l
  const float* cur = qkv + static_cast<size_t>(b) * 3 * D + D + h * DH + sub * 16;
  // 1. all key and value rows of this lane's entries
  Raw16<WT> kr[KPL], vr[KPL];
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int i = wave * KW + u * SLOTS + slot;
    int sl = slot0 + min(i, max(npast - 1, 0));
    sl = sl >= Wm1 ? sl - Wm1 : sl;
    if (npast > 0) {
      kr[u].load(ring_k + rbase + static_cast<size_t>(sl) * DH + sub * 16);
      vr[u].load(ring_v + rbase + static_cast<size_t>(sl) * DH + sub * 16);
    } else {   // an empty ring (first position, or W = 1): only the current entry is read
#pragma unroll
      for (int j = 0; j < Raw16<WT>::N; ++j) kr[u].v[j] = vr[u].v[j] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  float q[16], kc[16], vc[16];
  {
    const float* qr = qkv + static_cast<size_t>(b) * 3 * D + h * DH + sub * 16;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      q[c] = qr[c] * scale;
      kc[c] = round_to<WT>(cur[c]);          // the current entry in the ring's storage precision
      vc[c] = round_to<WT>(cur[D + c]);
    }
  }
  // 2. scores (entry npast is the current one; entries >= ne are masked)
  float sc[KPL];
  float mloc = -INFINITY;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int i = wave * KW + u * SLOTS + slot;
    const bool is_cur = i == npast;
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) a += q[c] * (is_cur ? kc[c] : kr[u].get(c));
    a = group_sum<LPK>(a);
    sc[u] = i < ne ? a : -INFINITY;
    mloc = fmaxf(mloc, sc[u]);
  }
  mloc = group_max<64>(mloc);
  if (lane == 0) wmax[wave] = mloc;
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < nw; ++w) M = fmaxf(M, wmax[w]);   // finite: entry 0 is in wave 0
  // 3. P.V over the lane's entries, then folded over the slots (lanes with the same part)
  float o[16], l = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = 0.f;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int i = wave * KW + u * SLOTS + slot;
    const bool is_cur = i == npast;
    const float p = __expf(sc[u] - M);   // masked entries: exp(-inf) = 0
    l += p;
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] += p * (is_cur ? vc[c] : vr[u].get(c));
  }
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    l += __shfl_xor(l, off, 64);
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] += __shfl_xor(o[c], off, 64);
  }
  if (slot == 0) {
#pragma unroll
    for (int c = 0; c < 16; ++c) po[wave][sub * 16 + c] = o[c];
    if (sub == 0) pl[wave] = l;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < DH; d += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int w = 0; w < nw; ++w) {
      num += po[w][d];
      den += pl[w];
    }
    store_from_f32(&attn[act_offset(b, h * DH + d, D, xf)], num / den);
  }
  // 4. the current entry replaces the oldest one (position t - (W-1)); every read of the ring
  //    happened before the barrier above
  if (Wm1 > 0) {
    const int sl = t % Wm1;
    const float* kr = qkv + static_cast<size_t>(b) * 3 * D + D + h * DH;
    for (int d = threadIdx.x; d < DH; d += blockDim.x) {
      store_from_f32(&ring_k[rbase + static_cast<size_t>(sl) * DH + d], kr[d]);
      store_from_f32(&ring_v[rbase + static_cast<size_t>(sl) * DH + d], kr[D + d]);
    }
  }
}

// Cross-attention partial states: one wave per (key chunk, head, sequence).
// Scores with lanes over keys (LPK lanes per key row), then exp(s - M) for the chunk in
// LDS, then P.V with lanes over (dim, 8-key block) reading the key-blocked value layout.
// With FUSE the chunks' partial states are combined in this launch: one chunk writes the head's
// output directly; several write their partials at agent scope and the last of them to arrive (a
// per-(sequence, head) counter, reset to zero by it) combines them in split order:
// attn[b, h*DH + d] = sum_s e^{m_s - M} o_s[d] / sum_s e^{m_s - M} l_s.
template <typename WT, int DH, bool FUSE>
__global__ __launch_bounds__(64) void cross_part_k(const float* __restrict__ qx, const WT* __restrict__ mem_k,
                                                   const WT* __restrict__ mem_v, float* __restrict__ part,
                                                   WT* __restrict__ attn, int* __restrict__ cnt, int B, int H, int T,
                                                   int t, int nsmax, float scale, int xf) {
  constexpr int LPK = DH / 16;
  constexpr int SLOTS = 64 / LPK;
  constexpr int DL = DH < 64 ? DH : 64;   // lanes per block in the P.V pass
  constexpr int BSTEP = 64 / DL;          // blocks taken at once
  constexpr int ND = DH / DL;             // dims per lane (2 when DH = 128)
  __shared__ float ps[KCHUNK];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int slot = lane / LPK, sub = lane % LPK;
  const int D = H * DH;
  const float* qr = qx + static_cast<size_t>(b) * D + h * DH + sub * 16;
  float q[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) q[c] = qr[c] * scale;
  const size_t T8 = (static_cast<size_t>(T) + 7) / 8 * 8;
  const WT* kb = mem_k + (static_cast<size_t>(b) * H + h) * static_cast<size_t>(T) * DH;   // pre-offset to group
  const WT* vb = mem_v + (static_cast<size_t>(b) * H + h) * T8 * DH;
  const int j0 = split * KCHUNK, j1 = min(j0 + KCHUNK, t + 1);
  float mloc = -INFINITY;
  // compile-time trip counts and clamped rows: every load of the chunk is unconditional, so
  // the loads of all iterations can be in flight together
#pragma unroll
  for (int it = 0; it < KCHUNK / SLOTS; ++it) {
    const int i = slot + it * SLOTS;
    const int j = min(j0 + i, j1 - 1);   // rows past the chunk end are loaded but masked
    float k[16];
    Row16<WT>::load(kb + static_cast<size_t>(j) * DH + sub * 16, k);
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) a += q[c] * k[c];
    a = group_sum<LPK>(a);
    a = j0 + i < j1 ? a : -INFINITY;
    if (sub == 0) ps[i] = a;
    mloc = fmaxf(mloc, a);
  }
  const float M = group_max<64>(mloc);   // finite: key j0 <= t is in the chunk
  __syncthreads();
  float lsum = 0.f;
  for (int i = lane; i < KCHUNK; i += 64) {
    const float pr = __expf(ps[i] - M);   // masked keys: exp(-inf) = 0
    ps[i] = pr;
    lsum += pr;
  }
  lsum = group_sum<64>(lsum);
  __syncthreads();
  const int d0 = lane % DL, bq = lane / DL;
  const int nblk = (j1 - j0 + 7) / 8;
  float o[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) o[nd] = 0.f;
#pragma unroll
  for (int it = 0; it < KCHUNK / 8 / BSTEP; ++it) {
    // blocks past the chunk end hold zero weights (masked keys); their loads are clamped
    const int blk = bq + it * BSTEP;
    const int lb = min(blk, nblk - 1);
    const float4 p0 = *reinterpret_cast<const float4*>(ps + blk * 8);
    const float4 p1 = *reinterpret_cast<const float4*>(ps + blk * 8 + 4);
    const float pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      float v[8];
      load8(vb + ((static_cast<size_t>(j0 / 8 + lb)) * DH + d0 + nd * 64) * 8, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) o[nd] += pw[k] * v[k];
    }
  }
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) {
#pragma unroll
    for (int off = DL; off < 64; off <<= 1) o[nd] += __shfl_xor(o[nd], off, 64);
  }
  const int ns = (t + 1 + KCHUNK - 1) / KCHUNK;
  const int oc = h * DH;   // first output column of the head
  if (FUSE && ns == 1) {
    if (bq == 0) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) store_from_f32(&attn[act_offset(b, oc + d0 + nd * 64, D, xf)], o[nd] / lsum);
    }
    return;
  }
  float* pb = part + (static_cast<size_t>(b) * H + h) * nsmax * (DH + 2);
  float* pr = pb + split * (DH + 2);
  if constexpr (!FUSE) {
    if (bq == 0) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) pr[2 + d0 + nd * 64] = o[nd];
    }
    if (lane == 0) {
      pr[0] = M;
      pr[1] = lsum;
    }
  } else {
    if (bq == 0) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd)
        __hip_atomic_store(pr + 2 + d0 + nd * 64, o[nd], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) {
      __hip_atomic_store(pr, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pr + 1, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's partial has been written
    int last = 0;
    if (lane == 0) {
      int* c = cnt + static_cast<size_t>(b) * H + h;
      last = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ns - 1;
      if (last) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!__builtin_amdgcn_readfirstlane(last)) return;
    // the last chunk: lane s holds chunk s's maximum and normaliser; every dimension's
    // weighted sum runs over the chunks in split order (ns < kWideCombineSplits)
    constexpr int NSF = kWideCombineSplits - 1;
    const float mv = lane < ns ? __hip_atomic_load(pb + lane * (DH + 2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : -INFINITY;
    const float lv = lane < ns ? __hip_atomic_load(pb + lane * (DH + 2) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : 0.f;
    float ov[NSF][ND];
#pragma unroll
    for (int sp = 0; sp < NSF; ++sp)
#pragma unroll
      for (int nd = 0; nd < ND; ++nd)
        ov[sp][nd] = __hip_atomic_load(pb + min(sp, ns - 1) * (DH + 2) + 2 + min(d0, DH - 1) + nd * 64,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float Mx = group_max<64>(mv);
    const float wv = lane < ns ? __expf(mv - Mx) : 0.f;
    float acc[ND], lsum_all = 0.f;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) acc[nd] = 0.f;
#pragma unroll
    for (int sp = 0; sp < NSF; ++sp) {
      if (sp < ns) {   // uniform
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv), sp));
        const float lw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), sp));
        lsum_all += w * lw;
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) acc[nd] += w * ov[sp][nd];
      }
    }
    if (bq == 0) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) store_from_f32(&attn[act_offset(b, oc + d0 + nd * 64, D, xf)], acc[nd] / lsum_all);
    }
  }
}

// The combine for many splits (long memories), as its own launch: 256 threads per (head, sequence).  The
// split maxima and the normaliser are taken across the threads, and the weighted sum of the
// split outputs is divided among 256/DH groups of threads (group g takes splits g, g + G, ...,
// eight loads in flight); the groups' sums and the waves' normaliser sums are folded in a
// fixed order, so the result does not depend on timing.
template <typename WT, int DH>
__global__ __launch_bounds__(256) void cross_combine_wide_k(const float* __restrict__ part, WT* __restrict__ attn,
                                                            int H, int ns, int nsmax, int xf) {
  constexpr int G = 256 / DH;
  constexpr int P = DH + 2;
  __shared__ float red[8];
  __shared__ float po[G][DH];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const float* pr = part + (static_cast<size_t>(b) * H + h) * nsmax * P;
  float m = -INFINITY;
  for (int s = tid; s < ns; s += 256) m = fmaxf(m, pr[s * P]);
  m = group_max<64>(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float l = 0.f;
  for (int s = tid; s < ns; s += 256) l += __expf(pr[s * P] - M) * pr[s * P + 1];
  l = group_sum<64>(l);
  if (lane == 0) red[4 + wave] = l;
  const int g = tid / DH, d = tid % DH;
  float o = 0.f;
  int s = g;
  for (; s + 7 * G < ns; s += 8 * G) {
    float mv[8], v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      mv[u] = pr[(s + u * G) * P];
      v[u] = pr[(s + u * G) * P + 2 + d];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) o += __expf(mv[u] - M) * v[u];
  }
  for (; s < ns; s += G) o += __expf(pr[s * P] - M) * pr[s * P + 2 + d];
  po[g][d] = o;
  __syncthreads();
  if (tid < DH) {
    float acc = po[0][tid];
#pragma unroll
    for (int q = 1; q < G; ++q) acc += po[q][tid];
    const float L = (red[4] + red[5]) + (red[6] + red[7]);
    store_from_f32(&attn[act_offset(b, h * DH + tid, H * DH, xf)], acc / L);
  }
}

template <typename WT, int DH>
hipError_t step_attention_launches(bool self, const ModelLayout& m, const Scratch& sc, char* base, char* state,
                                   const StateLayout& S, int l, int t, int xf, hipStream_t st) {
  const int B = S.B, H = m.H;
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));
  if (self) {
    const size_t lay = static_cast<size_t>(l) * B * H * S.Wm1 * DH;
    const float* q = reinterpret_cast<const float*>(base + sc.qkv);
    WT* rk = reinterpret_cast<WT*>(state + S.ring_k) + lay;
    WT* rv = reinterpret_cast<WT*>(state + S.ring_v) + lay;
    WT* out = reinterpret_cast<WT*>(base + sc.attn);
    constexpr int KW = SwaKw<WT>::v(DH);
    const int nw = (S.Wm1 + 1 + KW - 1) / KW;
    if (nw <= 8)
      swa2_k<WT, DH><<<dim3(H, B), 64 * nw, 0, st>>>(q, rk, rv, out, H, S.Wm1, t, scale, xf);
    else if (B * H >= 2048)
      swa_k<WT, DH, 1><<<dim3(H, B), 64, 0, st>>>(q, rk, rv, out, B, H, S.Wm1, t, scale, xf);
    else
      swa_k<WT, DH, 4><<<dim3(H, B), 256, 0, st>>>(q, rk, rv, out, B, H, S.Wm1, t, scale, xf);
  } else {
    const int g = m.G == 1 ? 0 : l;
    const size_t goff = static_cast<size_t>(g) * B * S.T * m.D;
    const size_t goff_v = static_cast<size_t>(g) * B * S.T8 * m.D;
    const int ns = (t + 1 + KCHUNK - 1) / KCHUNK;
    const float* qx = reinterpret_cast<const float*>(base + sc.qkv);
    const WT* mk = reinterpret_cast<const WT*>(state + S.mem_k) + goff;
    const WT* mv = reinterpret_cast<const WT*>(state + S.mem_v) + goff_v;
    float* part = reinterpret_cast<float*>(base + sc.part);
    WT* out = reinterpret_cast<WT*>(base + sc.attn);
    int* xcnt = reinterpret_cast<int*>(base + sc.xcnt);
    // up to kWideCombineSplits - 1 chunks the combine runs in the same launch; past that, the
    // 256-thread combine kernel folds the partials
    if (ns < kWideCombineSplits) {
      cross_part_k<WT, DH, true><<<dim3(ns, H, B), 64, 0, st>>>(qx, mk, mv, part, out, xcnt, B, H, S.T, t, sc.nsmax,
                                                                 scale, xf);
    } else {
      cross_part_k<WT, DH, false><<<dim3(ns, H, B), 64, 0, st>>>(qx, mk, mv, part, out, xcnt, B, H, S.T, t, sc.nsmax,
                                                                  scale, xf);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      cross_combine_wide_k<WT, DH><<<dim3(H, B), 256, 0, st>>>(part, out, H, ns, sc.nsmax, xf);
    }
  }
  return hipGetLastError();
}

template <typename WT>
hipError_t attention(bool self, const ModelLayout& m, const Scratch& sc, char* base, char* state, const StateLayout& S,
                     int l, int t, int xf, hipStream_t st) {
  switch (m.DH) {
    case 16: return step_attention_launches<WT, 16>(self, m, sc, base, state, S, l, t, xf, st);
    case 32: return step_attention_launches<WT, 32>(self, m, sc, base, state, S, l, t, xf, st);
    case 64: return step_attention_launches<WT, 64>(self, m, sc, base, state, S, l, t, xf, st);
    case 128: return step_attention_launches<WT, 128>(self, m, sc, base, state, S, l, t, xf, st);
    default: return hipErrorInvalidValue;
  }
}

#define RLT_CK(x)                  \
  do {                             \
    hipError_t e_ = (x);           \
    if (e_ != hipSuccess) return e_; \
  } while (0)

// One step on the tiled products (fp32 models, models without fragment-major copies, B > 512).
template <typename WT>
hipError_t step_tiled(const ModelLayout& m, const StateLayout& S, const Scratch& sc, const char* ws, char* state,
                      char* base, float* s_out, int t, int step, int n, hipStream_t st) {
  const int B = S.B, D = m.D, dt = m.dtype;
  float* y = reinterpret_cast<float*>(base + sc.y);
  float* s = reinterpret_cast<float*>(state + S.s);
  const float* gains_self = reinterpret_cast<const float*>(ws + m.g_dec_self);
  const float* gains_cross = reinterpret_cast<const float*>(ws + m.g_dec_cross);
  const float* gains_ffn = reinterpret_cast<const float*>(ws + m.g_dec_ffn);
  auto gemm = [&](const void* A, int lda, const void* W, int N, int K, void* out, int ldo, int epi) {
    GemmArgs g{};
    g.A = A; g.W = W; g.out = out;
    g.M = B; g.N = N; g.K = K; g.lda = lda; g.ldw = K; g.ldo = ldo; g.epi = epi;
    g.splitk_ws = reinterpret_cast<float*>(base + sc.splitk);
    g.splitk_ws_floats = gemm_splitk_ws_floats(B, D);
    return launch_gemm(g, dt, st);
  };
  const int nt = std::min(256, std::max(64, D / 4));
  // gated merge
  merge_prep_k<WT><<<B, nt, 0, st>>>(reinterpret_cast<const WT*>(state + S.e), s,
                                     reinterpret_cast<WT*>(base + sc.xin), S.T, D, t);
  RLT_CK(hipGetLastError());
  RLT_CK(gemm(base + sc.xin, 2 * D, ws + m.wgate, D, 2 * D, base + sc.gpre, D, EPI_STORE_F32));
  RLT_CK(gemm(base + sc.xin + static_cast<size_t>(D) * m.esz, 2 * D, ws + m.wfb, D, D, base + sc.fb, D,
              EPI_STORE_F32));
  merge_combine_k<WT><<<B, nt, 0, st>>>(reinterpret_cast<const float*>(base + sc.gpre),
                                        reinterpret_cast<const float*>(base + sc.fb),
                                        reinterpret_cast<const float*>(ws + m.bg),
                                        reinterpret_cast<const WT*>(base + sc.xin), y, D);
  RLT_CK(hipGetLastError());
  for (int l = 0; l < m.L; ++l) {
    const char* lw = ws + m.layers + l * m.layer_stride;
    // window self-attention
    RLT_CK(launch_rmsnorm_rows(y, gains_self + static_cast<size_t>(l) * D, base + sc.h, B, D, m.eps, dt, nullptr,
                               1, 0, 0, 1, st));
    RLT_CK(gemm(base + sc.h, D, lw + m.l_qkv, 3 * D, D, base + sc.qkv, 3 * D, EPI_STORE_F32));
    RLT_CK(attention<WT>(true, m, sc, base, state, S, l, t, 0, st));
    RLT_CK(gemm(base + sc.attn, D, lw + m.l_wo, D, D, y, D, EPI_RESID_F32));
    // cross-attention to memory entries 0..t
    RLT_CK(launch_rmsnorm_rows(y, gains_cross + static_cast<size_t>(l) * D, base + sc.h, B, D, m.eps, dt, nullptr,
                               1, 0, 0, 1, st));
    RLT_CK(gemm(base + sc.h, D, lw + m.l_wqx, D, D, base + sc.qkv, D, EPI_STORE_F32));
    RLT_CK(attention<WT>(false, m, sc, base, state, S, l, t, 0, st));
    RLT_CK(gemm(base + sc.attn, D, lw + m.l_wox, D, D, y, D, EPI_RESID_F32));
    // FFN
    RLT_CK(launch_rmsnorm_rows(y, gains_ffn + static_cast<size_t>(l) * D, base + sc.h, B, D, m.eps, dt, nullptr, 1,
                               0, 0, 1, st));
    RLT_CK(gemm(base + sc.h, D, lw + m.l_fin, m.F2, D, base + sc.act, m.F,
                m.ffn_kind == RLT_FFN_GELU ? EPI_GELU : EPI_SWIGLU));
    RLT_CK(gemm(base + sc.act, m.F, lw + m.l_fout, D, m.F, y, D, EPI_RESID_F32));
  }
  final_norm_k<<<(B + 3) / 4, 256, 0, st>>>(y, reinterpret_cast<const float*>(ws + m.g_dec_final), s, s_out, B, D,
                                           m.eps, step, n);
  return hipGetLastError();
}

// One step on the weight-streaming products: each norm is folded into the residual product
// before it (bf16(g * y) and per-block sums of squares) and the product after it (rows scaled by
// 1 / rms), every product's input is written in the fragment-major layout by its producer, and the
// merge is one product over [e_t ; s_{t-1}].
hipError_t step_wst(const ModelLayout& m, const StateLayout& S, const Scratch& sc, const char* ws, char* state,
                    char* base, float* s_out, int t, int step, int n, hipStream_t st) {
  const int B = S.B, D = m.D;
  float* y = reinterpret_cast<float*>(base + sc.y);
  float* ssp = reinterpret_cast<float*>(base + sc.ssp);
  uint16_t* xb = reinterpret_cast<uint16_t*>(base + sc.h);
  const uint16_t* e = reinterpret_cast<const uint16_t*>(state + S.e);
  const char* frag = ws + m.frag_layers;
  const int nt = D / 16;   // sums-of-squares blocks of the residual stream
  auto prod = [&](int epi, const void* x, int nt_in, const char* wf, int N, int K, float* outf, uint16_t* outb,
                  int ldo, const float* gain_next) {
    WstArgs a{};
    a.epi = epi;
    a.xf = static_cast<const uint4*>(x);
    a.ssp = ssp; a.nt_in = nt_in; a.ld_ss = ss_stride(B); a.eps = m.eps;
    a.e = e; a.T = S.T; a.t = t; a.D = D;
    a.wf = reinterpret_cast<const uint4*>(wf);
    a.M = B; a.N = N; a.K = K;
    a.outf = outf; a.outb = outb; a.ldo = ldo;
    a.ssp_out = ssp;
    a.gain_next = gain_next;
    a.xb_out = xb;
    a.bias = reinterpret_cast<const float*>(ws + m.bg);
    return launch_wsn(a, st);
  };
  const float* gains_self = reinterpret_cast<const float*>(ws + m.g_dec_self);
  const float* gains_cross = reinterpret_cast<const float*>(ws + m.g_dec_cross);
  const float* gains_ffn = reinterpret_cast<const float*>(ws + m.g_dec_ffn);
  float* qkv = reinterpret_cast<float*>(base + sc.qkv);
  uint16_t* attn = reinterpret_cast<uint16_t*>(base + sc.attn);
  uint16_t* act = reinterpret_cast<uint16_t*>(base + sc.act);
  // gated merge: y, bf16(g_self^0 * y) and the sums of squares of its 16-column blocks
  RLT_CK(launch_merge_x(e, reinterpret_cast<const float*>(state + S.s), base + sc.xin, B, padded_rows(B), S.T, D, t,
                        st));
  RLT_CK(prod(WEPI_MERGE, base + sc.xin, 0, ws + m.frag_merge, 2 * D, 2 * D, y, nullptr, D, gains_self));
  for (int l = 0; l < m.L; ++l) {
    const char* lw = frag + l * m.layer_stride;
    const size_t go = static_cast<size_t>(l) * D;
    const float* next_self = l + 1 < m.L ? gains_self + go + D : nullptr;
    RLT_CK(prod(WEPI_F32, xb, nt, lw + m.l_qkv, 3 * D, D, qkv, nullptr, 3 * D, nullptr));
    RLT_CK(attention<bf16_t>(true, m, sc, base, state, S, l, t, 1, st));
    RLT_CK(prod(WEPI_RESID, attn, 0, lw + m.l_wo, D, D, y, nullptr, D, gains_cross + go));
    RLT_CK(prod(WEPI_F32, xb, nt, lw + m.l_wqx, D, D, qkv, nullptr, D, nullptr));
    RLT_CK(attention<bf16_t>(false, m, sc, base, state, S, l, t, 1, st));
    RLT_CK(prod(WEPI_RESID, attn, 0, lw + m.l_wox, D, D, y, nullptr, D, gains_ffn + go));
    RLT_CK(prod(m.ffn_kind == RLT_FFN_GELU ? WEPI_GELU : WEPI_SWIGLU, xb, nt, lw + m.l_fin, m.F2, D, nullptr, act,
                m.F, nullptr));
    RLT_CK(prod(WEPI_RESID, act, 0, lw + m.l_fout, D, m.F, y, nullptr, D, next_self));
  }
  return launch_final_norm_ssp(y, ssp, nt, ss_stride(B), reinterpret_cast<const float*>(ws + m.g_dec_final),
                               reinterpret_cast<float*>(state + S.s), s_out, B, D, m.eps, step, n, st);
}

template <typename WT>
hipError_t run_t(const ModelLayout& m, const StateLayout& S, const char* ws, char* state, char* base, float* s_out,
                 int t0, int n, hipStream_t st) {
  const Scratch sc = scratch_layout(m, S.B, S.T);
  const bool w = use_wst(m, S.B);
  for (int step = 0; step < n; ++step) {
    const int t = t0 + step;
    if constexpr (sizeof(WT) == 2) {
      if (w) {
        RLT_CK(step_wst(m, S, sc, ws, state, base, s_out, t, step, n, st));
        continue;
      }
    }
    RLT_CK(step_tiled<WT>(m, S, sc, ws, state, base, s_out, t, step, n, st));
  }
  return hipSuccess;
}
#undef RLT_CK

}  // namespace

bool dec_batched_supported(const ModelLayout& m) {
  return (m.DH == 16 || m.DH == 32 || m.DH == 64 || m.DH == 128) && m.D % 64 == 0 && m.F % 64 == 0;
}

size_t dec_batched_scratch_bytes(const ModelLayout& m, int B, int T) { return scratch_layout(m, B, T).total; }

void dec_batched_counters(const ModelLayout& m, int B, int T, size_t* offset, size_t* bytes) {
  const Scratch sc = scratch_layout(m, B, T);
  *offset = sc.cnt;
  *bytes = sc.cnt_bytes;
}

hipError_t run_dec_batched(const ModelLayout& m, const StateLayout& s, const char* ws, char* state, char* scratch,
                           float* s_out, int t0, int n, hipStream_t st) {
  if (!dec_batched_supported(m)) return hipErrorInvalidValue;
  return m.dtype == RLT_DTYPE_BF16 ? run_t<bf16_t>(m, s, ws, state, scratch, s_out, t0, n, st)
                                   : run_t<float>(m, s, ws, state, scratch, s_out, t0, n, st);
}

}  // namespace rlt
