// Next-token sampling with the behaviour log-probability of the distribution actually drawn
// from ([FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer",
// model-RL co-design paragraph: the ratio the trainer forms divides by the sampler's
// log-probability, so the sampler must report it for the truncated distribution it used).
//
// Row r with uniform u_r in [0, 1):
//   z = logits_r / temperature; candidates ranked by larger z, then smaller id;
//   top-k keeps the first k; top-p keeps the shortest prefix of the survivors whose mass,
//   renormalised over them, reaches p; the kept ids in increasing order split [0, 1) in
//   proportion to exp(z) and the first whose cumulative share exceeds u is drawn;
//   logp = z[drawn] - log sum_kept exp(z).
//
// One workgroup of 512 threads per row.  The row is staged through LDS so that thread t holds
// the C consecutive logits [t*C, t*C + C) in registers (token-id order is then thread order
// for every scan).  Both thresholds are found by a bitwise search over order-preserving
// 32-bit keys: bit by bit from the top, a candidate key stays if the count (top-k) or the
// mass (top-p) of elements at or above it still reaches the target.  Every count, sum and
// scan is a fixed-order block reduction (wave shuffles, then the eight wave totals read in
// wave order), so a row's result does not depend on scheduling.  Ties at a threshold are
// resolved in id order with an exclusive scan of the per-thread tie counts.
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int ST = 512;            // threads per row
constexpr int SW = ST / 64;        // waves
constexpr float kLog2eS = 1.4426950408889634f;

struct SampleArgs {
  const float* logits;   // [N, V] fp32
  const float* u;        // [N]
  int32_t* tok;          // [N]
  float* logp;           // [N]
  int N, V, top_k;
  float inv_temp, top_p;
};

// order-preserving key of a float (larger float -> larger key) and its inverse
__device__ __forceinline__ uint32_t fkey(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float funkey(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ bool is_kept(float e) { return (__builtin_bit_cast(uint32_t, e) >> 31) == 0; }

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// Block reductions: each uses its own slot of a two-deep ring, so one barrier per call is
// enough (a slot is rewritten only after every thread has passed the next call's barrier).
struct Red {
  float* buf;   // [2][SW]
  int k = 0;
  __device__ float sum(float v) {
    v = wave_sum(v);
    float* b = buf + (k & 1) * SW;
    ++k;
    if (threadIdx.x % 64 == 0) b[threadIdx.x / 64] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < SW; ++w) s += b[w];
    return s;
  }
  __device__ float max(float v) {
    v = wave_max(v);
    float* b = buf + (k & 1) * SW;
    ++k;
    if (threadIdx.x % 64 == 0) b[threadIdx.x / 64] = v;
    __syncthreads();
    float s = -INFINITY;
#pragma unroll
    for (int w = 0; w < SW; ++w) s = fmaxf(s, b[w]);
    return s;
  }
  // exclusive prefix of v over threads in order
  __device__ float excl_scan(float v) {
    const int lane = threadIdx.x % 64;
    float inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float o = __shfl_up(inc, d, 64);
      if (lane >= d) inc += o;
    }
    float* b = buf + (k & 1) * SW;
    ++k;
    if (lane == 63) b[threadIdx.x / 64] = inc;
    __syncthreads();
    float pre = 0.f;
    for (int w = 0; w < static_cast<int>(threadIdx.x / 64); ++w) pre += b[w];
    return pre + inc - v;
  }
};

template <int C>
__global__ __launch_bounds__(ST) void sample_k(SampleArgs a) {
  static_assert(C >= 1 && C <= 64, "values per thread");
  constexpr int NE = ST * C;
  __shared__ float stage[NE + NE / 32 + 1];
  __shared__ float rbuf[2 * SW];
  __shared__ int pick_lo, pick_hi;
  Red red{rbuf};

  const int row = blockIdx.x;
  const int V = a.V;
  const float* src = a.logits + static_cast<size_t>(row) * V;
  // coalesced load, one pad slot per 32 values so the per-thread runs read without conflicts
  for (int i = threadIdx.x; i < NE; i += ST) stage[i + (i >> 5)] = i < V ? src[i] + 0.0f : -INFINITY;
  if (threadIdx.x == 0) {
    pick_lo = 0x7fffffff;
    pick_hi = -1;
  }
  __syncthreads();
  const int j0 = threadIdx.x * C;
  // the thread's run as order-preserving keys; a logit is recovered from its key when needed
  uint32_t key[C];
  float lm = -INFINITY;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const float xc = stage[(j0 + c) + ((j0 + c) >> 5)];
    key[c] = fkey(xc);
    lm = fmaxf(lm, xc);
  }
  const float mz = red.max(lm) * a.inv_temp;

  // unnormalised probabilities exp(z - max z); an id that is not (or no longer) kept holds
  // -0.0, which adds nothing to any sum and is told apart from an underflowed +0 by its sign
  float e[C];
#pragma unroll
  for (int c = 0; c < C; ++c)
    e[c] = j0 + c < V ? __builtin_amdgcn_exp2f((funkey(key[c]) * a.inv_temp - mz) * kLog2eS) : -0.0f;

  // ---- top-k: the k-th largest key, then ties at it in id order
  if (a.top_k > 0 && a.top_k < V) {
    const float k = static_cast<float>(a.top_k);
    uint32_t tau = 0;
#pragma nounroll
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      float cnt = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) cnt += key[c] >= cand ? 1.f : 0.f;
      if (red.sum(cnt) >= k) tau = cand;
    }
    float gt = 0.f, eq = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      gt += key[c] > tau ? 1.f : 0.f;
      eq += key[c] == tau ? 1.f : 0.f;
    }
    const float need_eq = k - red.sum(gt);
    float r = red.excl_scan(eq);   // ties before this thread's run
#pragma unroll
    for (int c = 0; c < C; ++c) {
      bool keep = key[c] > tau;
      if (key[c] == tau) {
        keep = r < need_eq;
        r += 1.f;
      }
      if (!keep) e[c] = -0.0f;
    }
  }
  float sk = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) sk += e[c];
  const float Sk = red.sum(sk);

  // ---- top-p over the top-k survivors (e is zero outside them)
  if (a.top_p < 1.0f) {
    const float need = a.top_p * Sk;
    uint32_t tau = 0;
#pragma nounroll
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      float ms = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) ms += key[c] >= cand ? e[c] : 0.f;
      if (red.sum(ms) >= need) tau = cand;
    }
    float gt = 0.f, eq = 0.f, e_eq = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool k1 = is_kept(e[c]);
      gt += key[c] > tau ? e[c] : 0.f;
      if (k1 && key[c] == tau) {
        eq += 1.f;
        e_eq = e[c];
      }
    }
    const float mass_gt = red.sum(gt);
    float r = red.excl_scan(eq);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool k1 = is_kept(e[c]);
      bool keep = k1 && key[c] > tau;
      if (k1 && key[c] == tau) {
        keep = mass_gt + r * e_eq < need;   // the mass ranked before this tie is still short
        r += 1.f;
      }
      if (!keep) e[c] = -0.0f;
    }
  }

  // ---- draw: inverse CDF over the kept ids in increasing order
  float mine = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) mine += e[c];
  const float Sp = red.sum(mine);
  float run = red.excl_scan(mine);
  const float target = a.u[row] * Sp;
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (is_kept(e[c])) {
      run += e[c];
      if (run > target && lo == 0x7fffffff) lo = j0 + c;
      hi = j0 + c;
    }
  }
  if (lo != 0x7fffffff) atomicMin(&pick_lo, lo);
  if (hi >= 0) atomicMax(&pick_hi, hi);
  __syncthreads();
  const int pick = pick_lo != 0x7fffffff ? pick_lo : pick_hi;   // u at the top edge: the last kept id
  if (pick >= j0 && pick < j0 + C) {
    uint32_t kv = 0;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (j0 + c == pick) kv = key[c];
    a.tok[row] = pick;
    a.logp[row] = (funkey(kv) * a.inv_temp - mz) - logf(Sp);
  }
}

template <int C>
hipError_t launch_c(const SampleArgs& a, hipStream_t st) {
  sample_k<C><<<a.N, ST, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sample_tokens(const float* logits, const float* uniforms, int32_t* tokens, float* logp, int N,
                                int V, float temperature, int top_k, float top_p, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (V < 1 || V > ST * 64 || !(temperature > 0.f) || top_k < 0 || !(top_p > 0.f) || top_p > 1.f)
    return hipErrorInvalidValue;
  SampleArgs a{logits, uniforms, tokens, logp, N, V, top_k, 1.0f / temperature, top_p};
  const int need = (V + ST - 1) / ST;
  if (need <= 1) return launch_c<1>(a, st);
  if (need <= 2) return launch_c<2>(a, st);
  if (need <= 4) return launch_c<4>(a, st);
  if (need <= 8) return launch_c<8>(a, st);
  if (need <= 16) return launch_c<16>(a, st);
  if (need <= 32) return launch_c<32>(a, st);
  return launch_c<64>(a, st);
}

}  // namespace rlt
