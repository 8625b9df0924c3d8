// Action scoring under the current policy ([FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器
// 状态的循环 Transformer", model-RL co-design paragraph: the trainer rebuilds every state under
// the current weights and scores each action; the recorded behaviour log-probability is the
// denominator of the importance ratio).
//
//   logp_i  = z_i[a_i] - log sum_v exp(z_i[v]),   z_i = (W_out s_i) / temperature
//   ratio_i = exp(logp_i - behaviour_i)
//
// The [N, V] logits are never written.  Two paths:
//  - score_lse_res_k (bf16 heads, d a multiple of 128 up to 2048): the workgroup's rows stay
//    resident in LDS while the head streams past them from a fragment-major copy; each lane
//    keeps a running maximum and sum for its rows over its own columns, the lane that holds
//    column a of a row records z[a], and logp and the ratio are formed at the end.
//  - otherwise score_lse_k + score_finish_k: a workgroup of four waves owns 128 rows and walks
//    the vocabulary in 128-wide tiles (the same tile and register-prefetched K stages as the
//    token-parallel GEMM), writing the row log-sum-exp; score_finish_k then takes the target
//    logit with one wave per row (a d-long dot product on the same operand precision).
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
  const uint4* w_frag;  // fragment-major bf16 copy of w_out, or null
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

// Resident-rows variant (bf16 head, d a multiple of 64*NS): the workgroup's RB rows of s are
// converted to bf16 once and kept in LDS for the whole vocabulary sweep, so s is read from HBM
// once instead of once per vocabulary tile.  W_out is streamed straight from global memory
// into the matrix-core B operand through a ring of NS register stages (64 k per stage); the
// four waves own disjoint 64-column slices of each 256-column vocabulary step, so no W byte is
// loaded twice in a workgroup.  Inside a stage, lane group g = lane/16 takes k = 16g..16g+15;
// the two 8-element halves feed two 16x16x32 products, and the A fragments read from LDS use
// the same k assignment, so each product contracts the same 32 k values on both operands.
// W comes from the fragment-major copy built when the weights are packed: the 64 lanes' 16-byte
// pieces of one (16-column block, stage, half) are contiguous, so each load instruction reads
// one contiguous kilobyte.  (Read from the row-major head, each lane quad would touch four
// different rows, and the vector memory path, not the bytes, would bound the kernel.)
constexpr int RES_COLS = 64;             // vocabulary columns per wave per step
constexpr int RES_KST = 64;              // k per register stage
constexpr int RES_LDS_ELEMS = 64 * 1032; // bf16 elements of the resident block (64 rows of d=1024 + pad)

template <int RB, int NW, int NS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void score_lse_res_k(ScoreArgs a) {
  constexpr int RI = RB / 16;   // 16-row blocks
  constexpr int NT = NW * 64;
  constexpr int RES_VSTEP = NW * RES_COLS;
  __shared__ __attribute__((aligned(16))) bf16_t As[RES_LDS_ELEMS];
  __shared__ float part[NW][RB][2];
  __shared__ float tgt[RB];   // z[a] of each row, taken from the product itself

  const int D = a.D, pitch = D + 8;
  const int m0 = blockIdx.x * RB;
  const int mrows = min(RB, a.N - m0);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int l16 = lane % 16, grp = lane / 16;
  const float sc = a.inv_temp * kLog2e;

  // resident rows: fp32 -> bf16, 8 elements per thread per pass; rows past N are zero
  for (int c = threadIdx.x; c < RB * (D / 8); c += NT) {
    const int r = c / (D / 8), k = (c % (D / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < mrows) {
      const float* p = a.s + static_cast<size_t>(m0 + r) * D + k;
      const float4 x = *reinterpret_cast<const float4*>(p);
      const float4 y = *reinterpret_cast<const float4*>(p + 4);
      v = make_uint4(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w), pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
    }
    *reinterpret_cast<uint4*>(As + r * pitch + k) = v;
  }

  const int KS = D / RES_KST;                         // stages per vocabulary step
  const int nvs = (a.V + RES_VSTEP - 1) / RES_VSTEP;  // vocabulary steps
  const int total = nvs * KS;
  const int ncb = (a.V + 15) / 16;   // 16-column blocks in the fragment copy
  const uint4* __restrict__ Wf = a.w_frag;

  // W stage g -> registers: column block cb = step*16 + wave*4 + j (clamped into the copy;
  // columns past V are masked in the fold), lane holds column 16*cb + l16,
  // k = kstage*64 + 16*grp + 8*h .. +8 in b[j][h]
  auto wload = [&](int g, uint4 (&b)[4][2]) {
    g = min(g, total - 1);
    const int vs = g / KS, ks = g - vs * KS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cb = min(vs * (RES_VSTEP / 16) + wave * (RES_COLS / 16) + j, ncb - 1);
      const uint4* q = Wf + static_cast<size_t>(cb * KS + ks) * 128 + lane;
      b[j][0] = q[0];
      b[j][1] = q[64];
    }
  };

  float mx[RI][4], sm[RI][4];
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      mx[i][v] = -INFINITY;
      sm[i][v] = 0.f;
    }
  f32x4_t acc[RI][4];
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the action of each of the lane's 16 rows (-1 past N); an action outside [0, V) never
  // matches a column, so its row keeps z[a] = NaN
  int act[RI][4];
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = i * 16 + grp * 4 + v;
      const int av = r < mrows ? a.act[m0 + r] : -1;
      act[i][v] = av >= 0 && av < a.V ? av : -1;   // padding columns past V never match
    }
  if (threadIdx.x < RB) tgt[threadIdx.x] = __builtin_nanf("");

  uint4 wb[NS][4][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) wload(s, wb[s]);
  __syncthreads();   // resident rows and tgt written

  for (int g0 = 0; g0 < total; g0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int g = g0 + s;
      const int ks = g % KS;
      const bf16_t* arow = As + l16 * pitch + ks * RES_KST + 16 * grp;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8_t af[RI];
#pragma unroll
        for (int i = 0; i < RI; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(arow + i * 16 * pitch + 8 * h);
#pragma unroll
        for (int i = 0; i < RI; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], __builtin_bit_cast(bf16x8_t, wb[s][j][h]),
                                                                acc[i][j], 0, 0, 0);
      }
      wload(g + NS, wb[s]);
      if (s == NS - 1 && ks == KS - 1) {
        // end of a vocabulary step: fold its columns into the running (max, sum)
        const int nb = (g / KS) * RES_VSTEP + wave * RES_COLS + l16;
#pragma unroll
        for (int i = 0; i < RI; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float x[4];
            float tm = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              x[j] = nb + j * 16 < a.V ? acc[i][j][v] * sc : -INFINITY;
              tm = fmaxf(tm, x[j]);
              // one lane of the workgroup holds column a of this row: it records z[a]
              if (nb + j * 16 == act[i][v]) tgt[i * 16 + grp * 4 + v] = acc[i][j][v] * a.inv_temp;
            }
            const float mn = fmaxf(mx[i][v], tm);
            if (mn != -INFINITY) {
              float sum = sm[i][v] * __builtin_amdgcn_exp2f(mx[i][v] - mn);
#pragma unroll
              for (int j = 0; j < 4; ++j) sum += __builtin_amdgcn_exp2f(x[j] - mn);
              sm[i][v] = sum;
              mx[i][v] = mn;
            }
          }
#pragma unroll
        for (int i = 0; i < RI; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // combine the 16 column lanes of each row, then the four waves (fixed order)
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float M = group_max<16>(mx[i][v]);
      float t = mx[i][v] == -INFINITY ? 0.f : sm[i][v] * __builtin_amdgcn_exp2f(mx[i][v] - M);
      t = group_sum<16>(t);
      if (l16 == 0) {
        const int r = i * 16 + grp * 4 + v;
        part[wave][r][0] = M;
        part[wave][r][1] = t;
      }
    }
  __syncthreads();
  if (threadIdx.x < mrows) {
    const int r = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, part[w][r][0]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = part[w][r][0];
      L += mw == -INFINITY ? 0.f : part[w][r][1] * __builtin_amdgcn_exp2f(mw - M);
    }
    const float lp = tgt[r] - (M + log2f(L)) / kLog2e;
    a.logp[m0 + r] = lp;
    if (a.ratio) a.ratio[m0 + r] = expf(lp - a.behav[m0 + r]);
  }
}

// Fragment-major copy of the fp32 head (layout in the model layout): one thread per 16-byte piece.
__global__ __launch_bounds__(NTH) void pack_score_head_k(const float* __restrict__ w, uint4* __restrict__ dst, int V,
                                                         int D, size_t n_pieces) {
  const size_t c = static_cast<size_t>(blockIdx.x) * NTH + threadIdx.x;
  if (c >= n_pieces) return;
  const int lane = static_cast<int>(c % 64), h = static_cast<int>((c / 64) % 2);
  const size_t t = c / 128;
  const int KS = D / RES_KST;
  const int ks = static_cast<int>(t % KS), cb = static_cast<int>(t / KS);
  const int row = cb * 16 + lane % 16, k = ks * RES_KST + 16 * (lane / 16) + 8 * h;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < V) {
    const float* p = w + static_cast<size_t>(row) * D + k;
    v = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
  }
  dst[c] = v;
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
  constexpr int NW = 8, NS = 2;
  // the resident-rows kernel forms logp and the ratio itself
  if (sizeof(TW) == 2 && a.w_frag && a.D % (RES_KST * NS) == 0 && a.D <= 1024) {
    score_lse_res_k<64, NW, NS><<<(a.N + 63) / 64, NW * 64, 0, st>>>(a);
    return hipGetLastError();
  }
  if (sizeof(TW) == 2 && a.w_frag && a.D % (RES_KST * NS) == 0 && a.D <= 2048) {
    score_lse_res_k<32, NW, NS><<<(a.N + 31) / 32, NW * 64, 0, st>>>(a);
    return hipGetLastError();
  }
  score_lse_k<TW><<<(a.N + BM - 1) / BM, NTH, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  score_finish_k<TW><<<(a.N + NTH / 64 - 1) / (NTH / 64), NTH, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_actions(const float* s, const void* w_out, const void* w_frag, const int32_t* actions,
                                const float* behav, float* logp, float* ratio, int N, int D, int V, float temperature,
                                int dtype, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (D % BK != 0 || temperature <= 0.f) return hipErrorInvalidValue;
  ScoreArgs a{s, w_out, static_cast<const uint4*>(w_frag), actions, behav, logp, ratio, N, D, V, 1.0f / temperature};
  return dtype == RLT_DTYPE_BF16 ? launch_t<bf16_t>(a, st) : launch_t<float>(a, st);
}

hipError_t launch_pack_score_head(const float* w, void* dst, int V, int D, hipStream_t st) {
  if (D % RES_KST != 0) return hipErrorInvalidValue;
  const size_t n = static_cast<size_t>((V + 15) / 16) * 16 * D / 8;
  pack_score_head_k<<<static_cast<unsigned>((n + NTH - 1) / NTH), NTH, 0, st>>>(w, static_cast<uint4*>(dst), V, D, n);
  return hipGetLastError();
}

}  // namespace rlt
