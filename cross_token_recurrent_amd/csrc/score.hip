// Action scoring under the current policy ([FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器
// 状态的循环 Transformer", model-RL co-design paragraph: the trainer rebuilds every state under
// the current weights and scores each action; the recorded behaviour log-probability is the
// denominator of the importance ratio).
//
//   logp_i  = z_i[a_i] - log sum_v exp(z_i[v]),   z_i = (W_out s_i) / temperature
//   ratio_i = exp(logp_i - behaviour_i)
//
// The [N, V] logits are never written.  score_lse_k: a workgroup of four waves owns 128 rows
// and walks the vocabulary in 128-wide tiles on the matrix cores (the same 128x128 tile and
// register-prefetched K stages as the token-parallel GEMM); each lane keeps a running maximum
// and sum for its 16 rows over its own columns, so a tile costs no lane reduction; the lanes
// and the two column waves are combined once at the end.  score_finish_k: one wave per row
// takes the target logit (a d-long dot product on the same operand precision) and forms logp
// and the ratio.
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int NTH = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <typename TW> constexpr int pad_of() { return sizeof(TW) == 2 ? 8 : 4; }
template <typename TW> constexpr int chunks_per_thread() { return (BM * BK * static_cast<int>(sizeof(TW)) / 16) / NTH; }

// One BMxBK tile of rows [row0, row0 + rows_valid) into registers; fp32 rows converted to the
// storage type (the operand precision of the token-parallel products).
template <typename TW, bool SRC_F32>
__device__ __forceinline__ void load_tile(const void* __restrict__ base, int ld, int row0, int rows_valid, int k0,
                                          uint4 (&r)[chunks_per_thread<TW>()]) {
  constexpr int EPC = 16 / sizeof(TW);
  constexpr int CPR = BK / EPC;
#pragma unroll
  for (int i = 0; i < chunks_per_thread<TW>(); ++i) {
    const int c = threadIdx.x + i * NTH;
    const int row = c / CPR, kc = (c % CPR) * EPC;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < rows_valid) {
      if constexpr (SRC_F32 && sizeof(TW) == 2) {
        const float* p = static_cast<const float*>(base) + static_cast<size_t>(row0 + row) * ld + k0 + kc;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
      } else {
        v = *reinterpret_cast<const uint4*>(static_cast<const TW*>(base) + static_cast<size_t>(row0 + row) * ld + k0 + kc);
      }
    }
    r[i] = v;
  }
}

template <typename TW>
__device__ __forceinline__ void store_tile(TW* __restrict__ lds, const uint4 (&r)[chunks_per_thread<TW>()]) {
  constexpr int EPC = 16 / sizeof(TW);
  constexpr int CPR = BK / EPC;
  constexpr int PITCH = BK + pad_of<TW>();
#pragma unroll
  for (int i = 0; i < chunks_per_thread<TW>(); ++i) {
    const int c = threadIdx.x + i * NTH;
    *reinterpret_cast<uint4*>(lds + (c / CPR) * PITCH + (c % CPR) * EPC) = r[i];
  }
}

struct ScoreArgs {
  const float* s;       // [N, d] fp32
  const void* w_out;    // [V, d] storage type
  const int32_t* act;   // [N]
  const float* behav;   // [N] or null
  float* logp;          // [N]: log-sum-exp after the first kernel, logp after the second
  float* ratio;         // [N] or null
  int N, D, V;
  float inv_temp;
};

template <typename TW>
__global__ __launch_bounds__(NTH) void score_lse_k(ScoreArgs a) {
  constexpr int PITCH = BK + pad_of<TW>();
  __shared__ __attribute__((aligned(16))) TW As[BM * PITCH];
  __shared__ __attribute__((aligned(16))) TW Ws[BN * PITCH];
  __shared__ float part[2][BM][2];   // (max, sum) of each column half per row

  const int m0 = blockIdx.x * BM;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wave / 2, wn = wave % 2;
  const int mrows = min(BM, a.N - m0);
  const int col_l = lane % 16, row_q = (lane / 16) * 4;
  const float sc = a.inv_temp * kLog2e;   // log2-domain scale

  // running (max, sum) of the lane's columns for its 16 rows (i, v); max in log2 units
  float mx[4][4], sm[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      mx[i][v] = -INFINITY;
      sm[i][v] = 0.f;
    }

  uint4 ra[chunks_per_thread<TW>()], rw[chunks_per_thread<TW>()];
  for (int n0 = 0; n0 < a.V; n0 += BN) {
    const int nrows = min(BN, a.V - n0);
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    load_tile<TW, true>(a.s, a.D, m0, mrows, 0, ra);
    load_tile<TW, false>(a.w_out, a.D, n0, nrows, 0, rw);
    for (int k0 = 0; k0 < a.D; k0 += BK) {
      __syncthreads();
      store_tile<TW>(As, ra);
      store_tile<TW>(Ws, rw);
      __syncthreads();
      if (k0 + BK < a.D) {
        load_tile<TW, true>(a.s, a.D, m0, mrows, k0 + BK, ra);
        load_tile<TW, false>(a.w_out, a.D, n0, nrows, k0 + BK, rw);
      }
      const int r16 = lane % 16, kq = lane / 16;
      if constexpr (sizeof(TW) == 2) {
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + i * 16 + r16) * PITCH + kq * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(Ws + (wn * 64 + j * 16 + r16) * PITCH + kq * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      } else {
#pragma unroll
        for (int kk = 0; kk < BK / 4; ++kk) {
          float af[4], bfr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) af[i] = As[(wm * 64 + i * 16 + r16) * PITCH + kk * 4 + kq];
#pragma unroll
          for (int j = 0; j < 4; ++j) bfr[j] = Ws[(wn * 64 + j * 16 + r16) * PITCH + kk * 4 + kq];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    // fold this tile's columns into the lane's running (max, sum); columns past V are skipped
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x[4];
        float tm = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + col_l;
          x[j] = n < a.V ? acc[i][j][v] * sc : -INFINITY;
          tm = fmaxf(tm, x[j]);
        }
        const float mn = fmaxf(mx[i][v], tm);
        if (mn != -INFINITY) {   // at least one column so far
          float sum = sm[i][v] * __builtin_amdgcn_exp2f(mx[i][v] - mn);
#pragma unroll
          for (int j = 0; j < 4; ++j) sum += __builtin_amdgcn_exp2f(x[j] - mn);
          sm[i][v] = sum;
          mx[i][v] = mn;
        }
      }
    __syncthreads();   // the tiles are reused by the next vocabulary tile
  }
  // combine the 16 column lanes of each row, then the two column halves (fixed order)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float M = group_max<16>(mx[i][v]);
      float t = mx[i][v] == -INFINITY ? 0.f : sm[i][v] * __builtin_amdgcn_exp2f(mx[i][v] - M);
      t = group_sum<16>(t);
      if (col_l == 0) {
        const int r = wm * 64 + i * 16 + row_q + v;
        part[wn][r][0] = M;
        part[wn][r][1] = t;
      }
    }
  __syncthreads();
  if (threadIdx.x < BM && threadIdx.x < mrows) {
    const int r = threadIdx.x;
    const float m0v = part[0][r][0], m1v = part[1][r][0];
    const float M = fmaxf(m0v, m1v);
    const float L = (m0v == -INFINITY ? 0.f : part[0][r][1] * __builtin_amdgcn_exp2f(m0v - M)) +
                    (m1v == -INFINITY ? 0.f : part[1][r][1] * __builtin_amdgcn_exp2f(m1v - M));
    a.logp[m0 + r] = (M + log2f(L)) / kLog2e;   // natural-log log-sum-exp of z = W_out s / temperature
  }
}

// One wave per row: target logit, logp = z[a] - lse, ratio.
template <typename TW>
__global__ __launch_bounds__(NTH) void score_finish_k(ScoreArgs a) {
  const int row = blockIdx.x * (NTH / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= a.N) return;   // uniform per wave
  const int act = a.act[row];
  const bool ok = act >= 0 && act < a.V;
  const TW* w = static_cast<const TW*>(a.w_out) + static_cast<size_t>(ok ? act : 0) * a.D;
  const float* s = a.s + static_cast<size_t>(row) * a.D;
  float acc = 0.f;
  for (int k = lane; k < a.D; k += 64) acc += round_to<TW>(s[k]) * load_as_f32(w + k);
  acc = group_sum<64>(acc);
  if (lane == 0) {
    const float lp = ok ? acc * a.inv_temp - a.logp[row] : __builtin_nanf("");
    a.logp[row] = lp;
    if (a.ratio) a.ratio[row] = expf(lp - a.behav[row]);
  }
}

template <typename TW>
hipError_t launch_t(const ScoreArgs& a, hipStream_t st) {
  score_lse_k<TW><<<(a.N + BM - 1) / BM, NTH, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  score_finish_k<TW><<<(a.N + NTH / 64 - 1) / (NTH / 64), NTH, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_actions(const float* s, const void* w_out, const int32_t* actions, const float* behav,
                                float* logp, float* ratio, int N, int D, int V, float temperature, int dtype,
                                hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (D % BK != 0 || temperature <= 0.f) return hipErrorInvalidValue;
  ScoreArgs a{s, w_out, actions, behav, logp, ratio, N, D, V, 1.0f / temperature};
  return dtype == RLT_DTYPE_BF16 ? launch_t<bf16_t>(a, st) : launch_t<float>(a, st);
}

}  // namespace rlt
