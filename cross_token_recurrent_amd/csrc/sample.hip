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
constexpr int kListMax = 1024;     // undecided elements one wave finishes a threshold search on
constexpr int kPrefixBits = 12;    // key bits decided over all elements first
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
// Every thread adds the eight wave totals in wave order, so all threads hold the same value.
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
  // the staged row; later the survivor list of the top-p search (keys, e, tau)
  constexpr int SZ = NE + NE / 8 > 2 * kListMax + 4 ? NE + NE / 8 : 2 * kListMax + 4;
  __shared__ __attribute__((aligned(16))) float stage[SZ];
  __shared__ float rbuf[2 * SW];
  __shared__ int pick_lo, pick_hi;
  Red red{rbuf};

  const int row = blockIdx.x;
  const int V = a.V;
  const float urow = a.u[row];   // requested early; used by the draw
  const float* src = a.logits + static_cast<size_t>(row) * V;
  // coalesced load into LDS with four pad slots after every 32 values (16-byte aligned runs,
  // and the per-thread runs read back without bank conflicts); -0 becomes +0 so equal logits
  // have equal keys
  auto slot = [](int i) { return i + (i >> 5) * 4; };
  // Every load is unconditional (the address is clamped into the row and padding is
  // selected afterwards), so all of a thread's loads are in flight before the first wait.
  if (C >= 4 && (V & 3) == 0) {
    constexpr int NQ = C >= 4 ? C / 4 : 1;
    const float4* s4 = reinterpret_cast<const float4*>(src);
    const int qmax = V / 4 - 1;
    float4 v[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) v[i] = s4[min(static_cast<int>(threadIdx.x) + i * ST, qmax)];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = threadIdx.x + i * ST;
      const bool in = 4 * q < V;
      const float4 w = make_float4(in ? v[i].x + 0.0f : -INFINITY, in ? v[i].y + 0.0f : -INFINITY,
                                   in ? v[i].z + 0.0f : -INFINITY, in ? v[i].w + 0.0f : -INFINITY);
      *reinterpret_cast<float4*>(stage + slot(4 * q)) = w;
    }
  } else {
    float v[C];
#pragma unroll
    for (int i = 0; i < C; ++i) v[i] = src[min(static_cast<int>(threadIdx.x) + i * ST, V - 1)];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int q = threadIdx.x + i * ST;
      stage[slot(q)] = q < V ? v[i] + 0.0f : -INFINITY;
    }
  }
  if (threadIdx.x == 0) {
    pick_lo = 0x7fffffff;
    pick_hi = -1;
  }
  __syncthreads();
  const int j0 = threadIdx.x * C;
  // the thread's run as order-preserving keys; a logit is recovered from its key when needed
  uint32_t key[C];
  float lm = -INFINITY;
  if constexpr (C >= 4) {
#pragma unroll
    for (int c = 0; c < C; c += 4) {
      const float4 v = *reinterpret_cast<const float4*>(stage + slot(j0 + c));
      key[c] = fkey(v.x); key[c + 1] = fkey(v.y); key[c + 2] = fkey(v.z); key[c + 3] = fkey(v.w);
      lm = fmaxf(lm, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    }
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float xc = stage[slot(j0 + c)];
      key[c] = fkey(xc);
      lm = fmaxf(lm, xc);
    }
  }
  const float mz = red.max(lm) * a.inv_temp;

  // unnormalised probabilities exp(z - max z); an id that is not (or no longer) kept holds
  // -0.0, which adds nothing to any sum and is told apart from an underflowed +0 by its sign
  float e[C];
#pragma unroll
  for (int c = 0; c < C; ++c)
    e[c] = j0 + c < V ? __builtin_amdgcn_exp2f((funkey(key[c]) * a.inv_temp - mz) * kLog2eS) : -0.0f;

  // Threshold search: the largest key tau whose weight at or above it, W(tau) = sum of w over
  // the elements in use with key >= tau, still reaches `target` (w = 1 and in use = valid for
  // top-k; w = e and in use = kept for top-p).  The first `pb` bits are decided over all
  // elements with block sums.  Then only the elements whose key shares tau's pb-bit prefix are
  // undecided; when at most kListMax remain they are gathered into LDS (id order) and wave 0
  // decides the remaining bits alone, the decided weight above the prefix added to its sums.
  // Otherwise the block search simply goes on.
  auto wt = [&](int c, bool mass) { return mass ? e[c] : (j0 + c < V ? 1.f : 0.f); };
  auto search = [&](bool mass, float target, int pb) -> uint32_t {
    uint32_t tau = 0;
    int bit = 31;
#pragma nounroll
    for (; bit >= 32 - pb; --bit) {
      const uint32_t cand = tau | (1u << bit);
      float n = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) n += key[c] >= cand ? wt(c, mass) : 0.f;
      if (red.sum(n) >= target) tau = cand;
    }
    const uint32_t pmask = pb == 0 ? 0u : ~0u << (32 - pb);
    float nu = 0.f, ab = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool use = mass ? is_kept(e[c]) : j0 + c < V;
      nu += use && (key[c] & pmask) == tau ? 1.f : 0.f;
      ab += use && (key[c] & pmask) > tau ? wt(c, mass) : 0.f;
    }
    const float U = red.sum(nu);   // undecided elements
    if (U <= static_cast<float>(kListMax)) {
      const float above = red.sum(ab);
      uint32_t* lk = reinterpret_cast<uint32_t*>(stage);
      float* lw = stage + kListMax;
      int pos = static_cast<int>(red.excl_scan(nu));
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const bool use = mass ? is_kept(e[c]) : j0 + c < V;
        if (use && (key[c] & pmask) == tau) {
          lk[pos] = key[c];
          lw[pos] = wt(c, mass);
          ++pos;
        }
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        constexpr int PER = kListMax / 64;
        uint32_t wk[PER];
        float ww[PER];
        const int nu_all = static_cast<int>(U);
#pragma unroll
        for (int i = 0; i < PER; ++i) {   // slots past the list hold stale data: weight 0
          const int j = threadIdx.x + 64 * i;
          wk[i] = lk[j];
          ww[i] = j < nu_all ? lw[j] : 0.f;
        }
        const float lim = target - above;
#pragma nounroll
        for (; bit >= 0; --bit) {
          const uint32_t cand = tau | (1u << bit);
          float n = 0.f;
#pragma unroll
          for (int i = 0; i < PER; ++i) n += wk[i] >= cand ? ww[i] : 0.f;
          if (wave_sum(n) >= lim) tau = cand;
        }
      }
      __syncthreads();   // every read of the list is done
      if (threadIdx.x == 0) lk[2 * kListMax] = tau;
      __syncthreads();
      tau = lk[2 * kListMax];
      __syncthreads();   // the slot is free again
    } else {
#pragma nounroll
      for (; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        float n = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) n += key[c] >= cand ? wt(c, mass) : 0.f;
        if (red.sum(n) >= target) tau = cand;
      }
    }
    return tau;
  };

  // ---- top-k: the k-th largest key, then ties at it in id order
  if (a.top_k > 0 && a.top_k < V) {
    const float k = static_cast<float>(a.top_k);
    const uint32_t tau = search(false, k, kPrefixBits);
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
      const bool tie = key[c] == tau;
      const bool keep = key[c] > tau || (tie && r < need_eq);
      r += tie ? 1.f : 0.f;
      e[c] = keep ? e[c] : -0.0f;
    }
  }
  float sk = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) sk += e[c];
  const float Sk = red.sum(sk);

  // ---- top-p over the top-k survivors (e is zero outside them)
  if (a.top_p < 1.0f) {
    const float need = a.top_p * Sk;
    // after a top-k of at most kListMax the survivors are gathered at once
    const bool few = a.top_k > 0 && a.top_k < V && a.top_k <= kListMax;
    const uint32_t tau = search(true, need, few ? 0 : kPrefixBits);
    float gt = 0.f, eq = 0.f, e_eq = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool tie = is_kept(e[c]) && key[c] == tau;
      gt += key[c] > tau ? e[c] : 0.f;
      eq += tie ? 1.f : 0.f;
      e_eq = tie ? e[c] : e_eq;
    }
    const float mass_gt = red.sum(gt);
    float r = red.excl_scan(eq);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool k1 = is_kept(e[c]);
      const bool tie = k1 && key[c] == tau;
      // a tie stays while the mass ranked before it is still short of the target
      const bool keep = (k1 && key[c] > tau) || (tie && mass_gt + r * e_eq < need);
      r += tie ? 1.f : 0.f;
      e[c] = keep ? e[c] : -0.0f;
    }
  }

  // ---- draw: inverse CDF over the kept ids in increasing order
  float mine = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) mine += e[c];
  const float Sp = red.sum(mine);
  float run = red.excl_scan(mine);
  const float target = urow * Sp;
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const bool k1 = is_kept(e[c]);
    run += e[c];   // -0 for ids that are not kept
    lo = (k1 && run > target && lo == 0x7fffffff) ? j0 + c : lo;
    hi = k1 ? j0 + c : hi;
  }
  // one LDS atomic per wave: the wave's minimum candidate and maximum kept id first (ids are
  // below 2^24, exact as floats)
  const float wlo = -wave_max(-static_cast<float>(lo == 0x7fffffff ? (1 << 24) : lo));
  const float whi = wave_max(static_cast<float>(hi));
  if (threadIdx.x % 64 == 0) {
    if (wlo < static_cast<float>(1 << 24)) atomicMin(&pick_lo, static_cast<int>(wlo));
    if (whi >= 0.f) atomicMax(&pick_hi, static_cast<int>(whi));
  }
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
