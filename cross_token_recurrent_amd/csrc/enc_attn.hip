// Causal multi-head attention of the encoder over known tokens ([FI] architecture
// paragraph: the encoder runs under a causal mask, token-parallel; [AL] §一: the memory
// never shows future tokens).
//
// Grid (query blocks, heads, sequences).  Each query is owned by LPQ = dh/16 lanes, each
// holding 16 dimensions of the (pre-scaled) query and of the output accumulator.  Key and
// value tiles of 64 positions (32 for dh = 128) are staged through LDS as fp32; scores are processed 16
// keys at a time with an online softmax (running max, rescaled sum and output).
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int NTH = 256;
constexpr int KC = 16;    // keys per online-softmax update

template <typename T, int DH>
__global__ __launch_bounds__(NTH) void enc_attn_k(AttnArgs a) {
  constexpr int LPQ = DH / 16;          // lanes per query
  constexpr int QB = NTH / LPQ;         // queries per block
  constexpr int KT = DH >= 128 ? 32 : 64;  // keys per LDS tile (32 KB of fp32 K and V at most)
  __shared__ __attribute__((aligned(16))) float Ks[KT][DH];
  __shared__ __attribute__((aligned(16))) float Vs[KT][DH];

  const int h = blockIdx.y, b = blockIdx.z;
  const int qi = blockIdx.x * QB + threadIdx.x / LPQ;    // query index within the call
  const int part = threadIdx.x % LPQ;
  const bool active = qi < a.n;
  const int qpos = a.t0 + (active ? qi : a.n - 1);
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));

  float q[16], o[16];
  if (active) {
    const T* qp = static_cast<const T*>(a.q) + static_cast<size_t>(b * a.n + qi) * a.ldq + h * DH + part * 16;
    float t8[8];
    load8(qp, t8);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = t8[i] * scale;
    load8(qp + 8, t8);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[8 + i] = t8[i] * scale;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  const int last_q = min(a.n, (blockIdx.x + 1) * QB) - 1;
  const int kend = a.t0 + last_q + 1;                     // keys visible to the block's last query
  const T* kb = static_cast<const T*>(a.k) + b * a.kv_ld_b + h * a.kv_ld_h;
  const T* vb = static_cast<const T*>(a.v) + b * a.kv_ld_b + h * a.kv_ld_h;

  for (int k0 = 0; k0 < kend; k0 += KT) {
    const int kt = min(KT, kend - k0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < KT * DH / 8; idx += NTH) {
      const int j = idx / (DH / 8), c = (idx % (DH / 8)) * 8;
      float kv[8], vv[8];
      if (j < kt) {
        load8(kb + static_cast<size_t>(k0 + j) * a.kv_ld_t + c, kv);
        load8(vb + static_cast<size_t>(k0 + j) * a.kv_ld_t + c, vv);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kv[i] = vv[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Ks[j][c + i] = kv[i];
        Vs[j][c + i] = vv[i];
      }
    }
    __syncthreads();
    for (int j0 = 0; j0 < kt; j0 += KC) {
      float s[KC];
      float cmax = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < KC; ++jj) {
        const float* kr = &Ks[j0 + jj][part * 16];
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc += q[c] * kr[c];
        if constexpr (LPQ > 1) acc = group_sum<LPQ>(acc);
        const int kpos = k0 + j0 + jj;
        const bool ok = (j0 + jj < kt) && kpos <= qpos;
        s[jj] = ok ? acc : -INFINITY;
        cmax = fmaxf(cmax, s[jj]);
      }
      const float mnew = fmaxf(mrun, cmax);
      if (mnew == -INFINITY) continue;      // nothing visible yet (uniform per query)
      const float corr = expf(mrun - mnew);
      lrun *= corr;
#pragma unroll
      for (int c = 0; c < 16; ++c) o[c] *= corr;
#pragma unroll
      for (int jj = 0; jj < KC; ++jj) {
        const float p = expf(s[jj] - mnew);
        lrun += p;
        const float* vr = &Vs[j0 + jj][part * 16];
#pragma unroll
        for (int c = 0; c < 16; ++c) o[c] += p * vr[c];
      }
      mrun = mnew;
    }
  }
  if (active) {
    T* op = static_cast<T*>(a.out) + static_cast<size_t>(b * a.n + qi) * a.ldo + h * DH + part * 16;
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int c = 0; c < 16; ++c) store_from_f32(op + c, o[c] * inv);
  }
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid(0, a.H, a.Bc);
  switch (a.dh) {
    case 16: grid.x = (a.n + NTH - 1) / NTH; enc_attn_k<T, 16><<<grid, NTH, 0, st>>>(a); break;
    case 32: grid.x = (a.n + NTH / 2 - 1) / (NTH / 2); enc_attn_k<T, 32><<<grid, NTH, 0, st>>>(a); break;
    case 64: grid.x = (a.n + NTH / 4 - 1) / (NTH / 4); enc_attn_k<T, 64><<<grid, NTH, 0, st>>>(a); break;
    case 128: grid.x = (a.n + NTH / 8 - 1) / (NTH / 8); enc_attn_k<T, 128><<<grid, NTH, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_enc_attention(const AttnArgs& a, int dtype, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  return dtype == RLT_DTYPE_BF16 ? launch_t<bf16_t>(a, st) : launch_t<float>(a, st);
}

}  // namespace rlt
