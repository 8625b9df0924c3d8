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
// Three kernels, one workgroup of 512 threads per row, chosen per call:
//  - sample_topk_k (0 < top-k <= 128, 4096 < V, V a multiple of 4) and sample_full_k (no top-k,
//    same V) load the row straight into registers (at most 128 VGPRs, two rows per CU);
//  - sample_k (every other case) stages the row through LDS so that thread t holds the C
//    consecutive logits [t*C, t*C + C) in registers as order-preserving 32-bit keys (token-id
//    order is then thread order for every scan).  Its two paths:
//
// Top-k (k at most the thread count): the k-th largest of the per-thread maxima bounds the
// k-th largest logit from below (k threads each hold an element at least that large).  The
// elements at or above the bound are gathered into LDS in id order; when they fit one wave's
// list, wave 0 finishes the row alone: the exact top-k threshold and its ties, the
// probabilities of the survivors only, the top-p threshold and its ties, and the draw.  No
// further pass over the whole row is made.
//
// Otherwise (no top-k, a larger k, or a bound that admits too many elements) every thread
// keeps its C probabilities and both thresholds are found by a bitwise search: bit by bit from
// the top, a candidate key stays if the count (top-k) or the mass (top-p) of elements at or
// above it still reaches the target; the first bits are decided over all elements with block
// reductions, the rest by one wave over the elements that share the decided prefix.  Ties at
// a threshold are resolved in id order with an exclusive scan of the per-thread tie counts.
//
// Counts are taken with wave ballots (exact integers); every sum and scan is a fixed-order
// reduction (wave shuffles, then the wave totals read in wave order), so a row's result does
// not depend on scheduling.
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int kListMax = 1024;     // undecided elements one wave finishes a threshold search on
constexpr int kPrefixBits = 12;    // key bits decided over all elements first
constexpr int kBoundBits = 16;     // top bits of the k-th largest thread maximum kept as the bound
constexpr int kLeanK = 128;        // largest top-k the lean kernel takes
constexpr int kLeanList = 256;     // its candidate list (at most four entries per lane of one wave)
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
// lanes of the wave for which p holds (the same value on every lane)
__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }
// the smallest and largest key of the wave (every lane gets both)
__device__ __forceinline__ void wave_min_max(uint32_t& lo, uint32_t& hi) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), d, 64)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), d, 64)));
  }
}
// A bitwise search for the largest key with a property that every key of a set has can start
// below the bits all the keys share: those bits come out as the shared prefix either way.
// Returns the prefix and sets `bit` to the highest bit where the keys differ (-1 if all equal).
__device__ __forceinline__ uint32_t shared_prefix(uint32_t kmin, uint32_t kmax, int& bit) {
  const uint32_t diff = kmin ^ kmax;
  bit = diff ? 31 - __clz(static_cast<int>(diff)) : -1;
  if (bit < 0) return kmin;     // one key: it is the answer
  if (bit == 31) return 0u;     // no shared bit
  return kmin & ~((2u << bit) - 1u);
}

// Block reductions over SW waves: each uses its own slot of a two-deep ring, so one barrier per
// call is enough (a slot is rewritten only after every thread has passed the next call's
// barrier).  Every thread adds the wave totals in wave order, so all threads hold the same value.
template <int SW>
struct Red {
  float* buf;   // [2][SW]
  int k = 0;
  // v already equal on every lane of its wave (a ballot count)
  __device__ float sum_waves(float v) {
    float* b = buf + (k & 1) * SW;
    ++k;
    if (threadIdx.x % 64 == 0) b[threadIdx.x / 64] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < SW; ++w) s += b[w];
    return s;
  }
  __device__ float sum(float v) { return sum_waves(wave_sum(v)); }
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
  // exclusive prefix of v over threads in order; `total` gets the sum over all threads
  __device__ float excl_scan(float v, float& total) {
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
    const int me = static_cast<int>(threadIdx.x / 64);
    float pre = 0.f, tot = 0.f;
#pragma unroll
    for (int w = 0; w < SW; ++w) {
      pre += w < me ? b[w] : 0.f;
      tot += b[w];
    }
    total = tot;
    return pre + inc - v;
  }
};

// Exclusive prefix over the lanes of one wave (lane order); lane 0 gets 0.
__device__ __forceinline__ float wave_excl_scan(float v, float& inclusive) {
  const int lane = threadIdx.x % 64;
  float inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  inclusive = inc;
  const float ex = __shfl_up(inc, 1, 64);
  return lane == 0 ? 0.f : ex;
}

// Wave 0 finishes a row whose top-k candidates (every element at or above a bound that is at
// most the k-th largest key) are listed in id order: keys lk[0..n), ids lid[0..n), n <= 64*P.
// Lane l holds list entries l*P .. l*P + P - 1, so list order is lane order, then slot order.
template <int P>
__device__ void finish_on_list(const SampleArgs& a, int row, const uint32_t* lk, const int* lid, int n, float mz,
                               float urow) {
  const int lane = threadIdx.x;
  uint32_t kk[P];
  int id[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int j = lane * P + i;
    kk[i] = j < n ? lk[j] : 0u;   // past the list: below every candidate key
    id[i] = j < n ? lid[j] : 0;
  }
  // top-k: the largest key whose count at or above it still reaches k (every list entry counts
  // at the list's shared prefix, n >= k)
  const int k = a.top_k;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (lane * P + i < n) {
      kmin = min(kmin, kk[i]);
      kmax = max(kmax, kk[i]);
    }
  wave_min_max(kmin, kmax);
  int bit0;
  uint32_t tk = shared_prefix(kmin, kmax, bit0);
#pragma nounroll
  for (int bit = bit0; bit >= 0; --bit) {
    const uint32_t cand = tk | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) cnt += wave_count(kk[i] >= cand);
    tk = cnt >= k ? cand : tk;
  }
  // ties at it stay in id order while fewer than k ids rank above them
  int gt = 0;
  float ties = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    gt += wave_count(kk[i] > tk);
    ties += kk[i] == tk ? 1.f : 0.f;
  }
  const float need_eq = static_cast<float>(k - gt);
  float tie_all;
  float r = wave_excl_scan(ties, tie_all);
  bool keep[P];
  float e[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const bool tie = kk[i] == tk;
    keep[i] = kk[i] > tk || (tie && r < need_eq);
    r += tie ? 1.f : 0.f;
    const float ev = __builtin_amdgcn_exp2f((funkey(kk[i]) * a.inv_temp - mz) * kLog2eS);
    e[i] = keep[i] ? ev : 0.f;
  }
  // top-p over the survivors
  if (a.top_p < 1.0f) {
    float sk = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) sk += e[i];
    const float need = a.top_p * wave_sum(sk);
    // the survivors' whole mass (the same sums as need's) reaches need at their shared prefix
    uint32_t smin = 0xffffffffu, smax = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (keep[i]) {
        smin = min(smin, kk[i]);
        smax = max(smax, kk[i]);
      }
    wave_min_max(smin, smax);
    int bitp;
    uint32_t tp = shared_prefix(smin, smax, bitp);
#pragma nounroll
    for (int bit = bitp; bit >= 0; --bit) {
      const uint32_t cand = tp | (1u << bit);
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < P; ++i) m += kk[i] >= cand ? e[i] : 0.f;
      tp = wave_sum(m) >= need ? cand : tp;
    }
    float gtm = 0.f, pt = 0.f, e_eq = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const bool tie = keep[i] && kk[i] == tp;
      gtm += keep[i] && kk[i] > tp ? e[i] : 0.f;
      pt += tie ? 1.f : 0.f;
      e_eq = tie ? e[i] : e_eq;
    }
    const float mass_gt = wave_sum(gtm);
    e_eq = wave_max(e_eq);   // every tie has the same key, so the same probability
    float pt_all;
    float rp = wave_excl_scan(pt, pt_all);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const bool tie = keep[i] && kk[i] == tp;
      // a tie stays while the mass ranked before it is still short of the target
      keep[i] = (keep[i] && kk[i] > tp) || (tie && mass_gt + rp * e_eq < need);
      rp += tie ? 1.f : 0.f;
      e[i] = keep[i] ? e[i] : 0.f;
    }
  }
  // draw: inverse CDF over the kept ids in increasing order
  float mine = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) mine += e[i];
  float inc;
  float run = wave_excl_scan(mine, inc);
  const float Sp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inc), 63));
  const float target = urow * Sp;
  int lo = 0x7fffffff, hi = -1;
  uint32_t klo = 0, khi = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    run += e[i];
    const bool first = keep[i] && run > target && lo == 0x7fffffff;
    lo = first ? id[i] : lo;
    klo = first ? kk[i] : klo;
    hi = keep[i] ? id[i] : hi;
    khi = keep[i] ? kk[i] : khi;
  }
  // the first lane with a candidate holds the draw; u at the top edge: the last kept id
  const unsigned long long has_lo = __ballot(lo != 0x7fffffff);
  const unsigned long long has_hi = __ballot(hi >= 0);
  const int src = has_lo ? __ffsll(has_lo) - 1 : 63 - __clzll(has_hi);
  if (lane == src) {
    const int pick = has_lo ? lo : hi;
    const uint32_t kv = has_lo ? klo : khi;
    a.tok[row] = pick;
    a.logp[row] = (funkey(kv) * a.inv_temp - mz) - logf(Sp);
  }
}

// One row of the general path (the workgroup's threads all call it for the same row).
template <int C>
__device__ __forceinline__ void sample_row(const SampleArgs& a, int row, float* stage, uint32_t* tmx, float* rbuf,
                                           uint32_t& bcast, int& pick_lo, int& pick_hi) {
  static_assert(C >= 1 && C <= 64, "values per thread");
  Red<SW> red{rbuf};
  const int V = a.V;
  const int lane = threadIdx.x % 64;
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
  // the thread's run as order-preserving keys; a logit is recovered from its key when needed.
  // Ids past V get key 0, below the key of every float (-inf included), so no count, bound or
  // tie test ever takes them.
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
  uint32_t km = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    key[c] = j0 + c < V ? key[c] : 0u;
    km = key[c] > km ? key[c] : km;
  }
  const bool topk = a.top_k > 0 && a.top_k < V;
  tmx[threadIdx.x] = km;
  const float mz = red.max(lm) * a.inv_temp;   // its barrier also ends every read of the stage

  if (topk && a.top_k <= ST) {
    // bound: the k-th largest per-thread maximum, its low bits cleared, found by wave 0 (its
    // counts are ballots on the CU's one scalar unit) and broadcast
    if (threadIdx.x < 64) {
      uint32_t tv[SW];
#pragma unroll
      for (int i = 0; i < SW; ++i) tv[i] = tmx[lane + 64 * i];
      uint32_t b = 0;
#pragma nounroll
      for (int bit = 31; bit >= 32 - kBoundBits; --bit) {
        const uint32_t cand = b | (1u << bit);
        int n = 0;
#pragma unroll
        for (int i = 0; i < SW; ++i) n += wave_count(tv[i] >= cand);
        b = n >= a.top_k ? cand : b;
      }
      if (threadIdx.x == 0) bcast = b;
    }
    __syncthreads();
    const uint32_t lo = bcast;
    if (lo != 0) {
      float nu = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) nu += key[c] >= lo ? 1.f : 0.f;
      float U;
      int pos = static_cast<int>(red.excl_scan(nu, U));
      if (U <= static_cast<float>(kListMax)) {
        uint32_t* lk = reinterpret_cast<uint32_t*>(stage);
        int* lid = reinterpret_cast<int*>(stage + kListMax);
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (key[c] >= lo) {
            lk[pos] = key[c];
            lid[pos] = j0 + c;
            ++pos;
          }
        __syncthreads();
        if (threadIdx.x < 64) {
          const int n = static_cast<int>(U);
          if (n <= 64) finish_on_list<1>(a, row, lk, lid, n, mz, urow);
          else if (n <= 128) finish_on_list<2>(a, row, lk, lid, n, mz, urow);
          else if (n <= 256) finish_on_list<4>(a, row, lk, lid, n, mz, urow);
          else if (n <= 512) finish_on_list<8>(a, row, lk, lid, n, mz, urow);
          else finish_on_list<16>(a, row, lk, lid, n, mz, urow);
        }
        return;   // the whole workgroup (U is the same on every thread)
      }
    }
  }

  // ---- general path
  // unnormalised probabilities exp(z - max z); an id that is not (or no longer) kept holds
  // -0.0, which adds nothing to any sum and is told apart from an underflowed +0 by its sign
  // (branch-free: the exponential is taken for every id, then ids past V get -0)
  float e[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const bool in = key[c] != 0u;
    const float x = (funkey(key[c]) * a.inv_temp - mz) * kLog2eS;
    const float ev = __builtin_amdgcn_exp2f(in ? x : -INFINITY);
    e[c] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, ev) | (in ? 0u : 0x80000000u));
  }

  auto in_use = [&](int c, bool mass) { return mass ? is_kept(e[c]) : key[c] != 0u; };
  // weight at or above a candidate key over the block: an exact count (ballots) or a
  // fixed-order mass
  auto block_weight = [&](bool mass, uint32_t cand) -> float {
    if (mass) {
      float n = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) n += key[c] >= cand ? e[c] : 0.f;
      return red.sum(n);
    }
    float n = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) n += key[c] >= cand ? 1.f : 0.f;
    return red.sum(n);
  };

  // Threshold search: the largest key tau whose weight at or above it, W(tau) = sum of w over
  // the elements in use with key >= tau, still reaches `target` (w = 1 and in use = valid for
  // top-k; w = e and in use = kept for top-p).  The first `pb` bits are decided over all
  // elements with block sums.  Then only the elements in use whose key shares tau's pb-bit
  // prefix are undecided; when at most kListMax remain they are gathered into LDS (id order)
  // and wave 0 decides the remaining bits alone, the decided weight above the prefix added to
  // its sums.  Otherwise the block search goes on.
  auto search = [&](bool mass, float target, int pb) -> uint32_t {
    uint32_t tau = 0;
    int bit = 31;
#pragma nounroll
    for (; bit >= 32 - pb; --bit) {
      const uint32_t cand = tau | (1u << bit);
      if (block_weight(mass, cand) >= target) tau = cand;
    }
    const uint32_t pmask = pb == 0 ? 0u : ~0u << (32 - pb);
    float nu = 0.f, ab = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool use = in_use(c, mass);
      nu += use && (key[c] & pmask) == tau ? 1.f : 0.f;
      ab += use && (key[c] & pmask) > tau ? (mass ? e[c] : 1.f) : 0.f;
    }
    float U;
    const float pos0 = red.excl_scan(nu, U);   // undecided elements before this thread, and in all
    if (U <= static_cast<float>(kListMax)) {
      const float above = pb == 0 ? 0.f : red.sum(ab);
      uint32_t* lk = reinterpret_cast<uint32_t*>(stage);
      float* lw = stage + kListMax;
      int pos = static_cast<int>(pos0);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (in_use(c, mass) && (key[c] & pmask) == tau) {
          lk[pos] = key[c];
          lw[pos] = mass ? e[c] : 1.f;
          ++pos;
        }
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        // slot i of lane l is list entry l + 64 i; only the slots the list reaches are read
        constexpr int PER = kListMax / 64;
        const int n_all = static_cast<int>(U);
        const int np = (n_all + 63) / 64;
        uint32_t wk[PER];
        float ww[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          wk[i] = 0u;   // past the list: below every candidate key
          ww[i] = 0.f;
          const int j = lane + 64 * i;
          if (i < np && j < n_all) {
            wk[i] = lk[j];
            ww[i] = lw[j];
          }
        }
        const float lim = target - above;
#pragma nounroll
        for (; bit >= 0; --bit) {
          const uint32_t cand = tau | (1u << bit);
          float n;
          if (mass) {
            float sm = 0.f;
#pragma unroll
            for (int i = 0; i < PER; ++i)
              if (i < np) sm += wk[i] >= cand ? ww[i] : 0.f;
            n = wave_sum(sm);
          } else {
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < PER; ++i)
              if (i < np) cnt += wave_count(wk[i] >= cand);
            n = static_cast<float>(cnt);
          }
          if (n >= lim) tau = cand;
        }
        if (threadIdx.x == 0) bcast = tau;
      }
      // the list is read by wave 0 only; the next gather comes after further barriers
      __syncthreads();
      return bcast;
    }
#pragma nounroll
    for (; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      if (block_weight(mass, cand) >= target) tau = cand;
    }
    return tau;
  };

  // ---- top-k: the k-th largest key, then ties at it in id order
  if (topk) {
    const float k = static_cast<float>(a.top_k);
    const uint32_t tau = search(false, k, kPrefixBits);
    float gt = 0.f, eq = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      gt += key[c] > tau ? 1.f : 0.f;
      eq += key[c] == tau ? 1.f : 0.f;
    }
    const float need_eq = k - red.sum(gt);
    float n_eq;
    float r = red.excl_scan(eq, n_eq);   // ties before this thread's run
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
    const bool few = topk && a.top_k <= kListMax;
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
    float n_eq;
    float r = red.excl_scan(eq, n_eq);
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
  float Sp;
  float run = red.excl_scan(mine, Sp);
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
__global__ __launch_bounds__(ST) void sample_k(SampleArgs a) {
  static_assert(C >= 1 && C <= 64, "values per thread");
  constexpr int NE = ST * C;
  // the staged row; later the list of a threshold search (keys and weights or ids)
  constexpr int SZ = NE + NE / 8 > 2 * kListMax ? NE + NE / 8 : 2 * kListMax;
  __shared__ __attribute__((aligned(16))) float stage[SZ];
  __shared__ uint32_t tmx[ST];   // per-thread maximum keys (the top-k bound)
  __shared__ float rbuf[2 * SW];
  __shared__ uint32_t bcast;
  __shared__ int pick_lo, pick_hi;
  sample_row<C>(a, blockIdx.x, stage, tmx, rbuf, bcast, pick_lo, pick_hi);
}

// Lean top-k kernel (0 < k <= kLeanK, 4096 < V, V a multiple of 4): no LDS stage and at most
// 128 VGPRs, so two rows share a CU and each fills the other's waits (a row's single-wave
// finish leaves the rest of its workgroup idle).  Thread t loads the 16-byte pieces t, t + 512,
// ... of the row straight into registers as keys (ids 4q..4q+3 of piece q).  The bound and the
// gather are those of the list path above, with at most kLeanList candidates.  When the bound
// admits more (for example logits that grow with the id), the exact top-k threshold is found by
// block count passes over the row re-read from L2, the ties at it are cut in id order (a
// bitwise search for the need-th smallest tie id, when more tie than are needed), and exactly
// the k survivors are gathered.  The gather's order is thread-major, so wave 0 places every
// entry at its rank by id (ids are distinct) before finishing the row on the list.
template <int NQ>
__global__ __launch_bounds__(ST) __attribute__((amdgpu_waves_per_eu(4)))
void sample_topk_k(SampleArgs a) {
  constexpr int C = 4 * NQ;
  __shared__ uint32_t tmx[ST];
  __shared__ float rbuf[2 * SW];
  __shared__ uint32_t bcast;
  __shared__ uint32_t lk[kLeanList], sk[kLeanList];
  __shared__ int lid[kLeanList], sid[kLeanList];
  Red<SW> red{rbuf};

  const int row = blockIdx.x;
  const int V = a.V;
  const int lane = threadIdx.x % 64;
  const float urow = a.u[row];
  const float4* s4 = reinterpret_cast<const float4*>(a.logits + static_cast<size_t>(row) * V);
  const int qmax = V / 4 - 1;
  float4 v[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) v[i] = s4[min(static_cast<int>(threadIdx.x) + i * ST, qmax)];
  // keys (ids past V: 0, below every float's key); -0 becomes +0 so equal logits have equal keys
  uint32_t key[C];
  float lm = -INFINITY;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const bool in = 4 * (static_cast<int>(threadIdx.x) + i * ST) < V;
    key[4 * i] = in ? fkey(v[i].x + 0.0f) : 0u;
    key[4 * i + 1] = in ? fkey(v[i].y + 0.0f) : 0u;
    key[4 * i + 2] = in ? fkey(v[i].z + 0.0f) : 0u;
    key[4 * i + 3] = in ? fkey(v[i].w + 0.0f) : 0u;
    lm = in ? fmaxf(lm, fmaxf(fmaxf(v[i].x, v[i].y), fmaxf(v[i].z, v[i].w))) : lm;
  }
  uint32_t km = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) km = key[c] > km ? key[c] : km;
  tmx[threadIdx.x] = km;
  const float mz = red.max(lm) * a.inv_temp;
  if (threadIdx.x < 64) {
    uint32_t tv[SW];
#pragma unroll
    for (int i = 0; i < SW; ++i) tv[i] = tmx[lane + 64 * i];
    uint32_t b = 0;
#pragma nounroll
    for (int bit = 31; bit >= 32 - kBoundBits; --bit) {
      const uint32_t cand = b | (1u << bit);
      int n = 0;
#pragma unroll
      for (int i = 0; i < SW; ++i) n += wave_count(tv[i] >= cand);
      b = n >= a.top_k ? cand : b;
    }
    if (threadIdx.x == 0) bcast = b;
  }
  __syncthreads();
  const uint32_t lo = bcast;
  float nu = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) nu += key[c] >= lo ? 1.f : 0.f;
  float U;
  int pos = static_cast<int>(red.excl_scan(nu, U));
  auto id_of = [&](int c) { return 4 * (static_cast<int>(threadIdx.x) + (c / 4) * ST) + c % 4; };
  int n;
  if (lo != 0u && U <= static_cast<float>(kLeanList)) {   // the same on every thread
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (key[c] >= lo) {
        lk[pos] = key[c];
        lid[pos] = id_of(c);
        ++pos;
      }
    n = static_cast<int>(U);
  } else {
    // The exact path re-reads the row (from L2) one 16-byte piece at a time instead of
    // keeping the keys live across it, which would push the kernel past 128 VGPRs.
    // fn(q, c, key) for every id 4q + c of the thread's pieces q = t, t + 512, ... (key 0 past V)
    auto each = [&](auto fn) {
#pragma nounroll
      for (int i = 0; i < NQ; ++i) {
        const int q = static_cast<int>(threadIdx.x) + i * ST;
        const float4 v = s4[min(q, qmax)];
        const bool in = 4 * q < V;
        fn(q, 0, in ? fkey(v.x + 0.0f) : 0u);
        fn(q, 1, in ? fkey(v.y + 0.0f) : 0u);
        fn(q, 2, in ? fkey(v.z + 0.0f) : 0u);
        fn(q, 3, in ? fkey(v.w + 0.0f) : 0u);
      }
    };
    // the exact threshold: the largest key whose count at or above it still reaches k
    const float k = static_cast<float>(a.top_k);
    uint32_t tau = 0;
#pragma nounroll
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      float cnt = 0.f;
      each([&](int, int, uint32_t kc) { cnt += kc >= cand ? 1.f : 0.f; });
      if (red.sum(cnt) >= k) tau = cand;
    }
    float gtc = 0.f, tc = 0.f;
    each([&](int, int, uint32_t kc) {
      gtc += kc > tau ? 1.f : 0.f;
      tc += kc == tau ? 1.f : 0.f;
    });
    const float need_eq = k - red.sum(gtc);
    // ties at it are taken in id order: all of them, or those up to the need_eq-th smallest
    // tie id (the largest id x with fewer than need_eq ties below it; ids are below 2^15)
    int id_cut = 0x7fffffff;
    if (red.sum(tc) > need_eq) {
      int x = 0;
#pragma nounroll
      for (int bit = 14; bit >= 0; --bit) {
        const int cand = x | (1 << bit);
        float below = 0.f;
        each([&](int q, int c, uint32_t kc) { below += kc == tau && 4 * q + c < cand ? 1.f : 0.f; });
        if (red.sum(below) < need_eq) x = cand;
      }
      id_cut = x;
    }
    auto take = [&](int q, int c, uint32_t kc) { return kc > tau || (kc == tau && 4 * q + c <= id_cut); };
    float m = 0.f;
    each([&](int q, int c, uint32_t kc) { m += take(q, c, kc) ? 1.f : 0.f; });
    float total;
    pos = static_cast<int>(red.excl_scan(m, total));   // total = k
    each([&](int q, int c, uint32_t kc) {
      if (take(q, c, kc)) {
        lk[pos] = kc;
        lid[pos] = 4 * q + c;
        ++pos;
      }
    });
    n = static_cast<int>(total);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    for (int j = lane; j < n; j += 64) {
      const int idj = lid[j];
      int r = 0;
      for (int m = 0; m < n; ++m) r += lid[m] < idj ? 1 : 0;
      sk[r] = lk[j];
      sid[r] = idj;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    if (n <= 64) finish_on_list<1>(a, row, sk, sid, n, mz, urow);
    else if (n <= 128) finish_on_list<2>(a, row, sk, sid, n, mz, urow);
    else finish_on_list<4>(a, row, sk, sid, n, mz, urow);
  }
}

// Lean kernels without top-k (4096 < V, V a multiple of 4): the same register layout as the
// top-k kernel (piece row i of the row holds ids 2048i .. 2048i + 2047 in thread order), the
// probabilities computed in place of the loaded logits.
//
// NUCLEUS (top-p < 1): the threshold is searched on the probabilities' bit patterns, which order
// non-negative floats as their values, so only the probabilities stay in registers.  Ranking by
// probability instead of by logit merges logits whose fp32 probabilities are equal; those become
// ties and are resolved by id.  The 12 bits below the two that are always 0 are decided over the
// row with block mass sums; when at most 512 elements share the decided prefix, wave 0 decides the
// rest on a list.
// Ties at the threshold stay in id order while the mass ranked before them is short of the
// target: their number comes from that same comparison (monotone in the rank, so a binary
// search), and when fewer ties are kept than exist, a bitwise search finds the id of the last
// kept one.  Everything not kept gets probability 0.
//
// The draw takes the id-order inverse CDF in two levels: the piece row where the cumulative
// mass first exceeds u*S (from the rows' totals, added in a fixed order), then an exclusive scan
// over the threads of that piece row.  The drawn logit is read again for logp.
template <int NQ, bool NUCLEUS>
__global__ __launch_bounds__(ST) __attribute__((amdgpu_waves_per_eu(4)))
void sample_full_k(SampleArgs a) {
  __shared__ float rbuf[2 * SW];
  __shared__ float rowtot[SW][NQ];   // each wave's mass of every piece row
  // the single-wave list of the nucleus search: 512 entries (8 per lane) keep the kernel within
  // 128 VGPRs beside the 64 probabilities; longer prefixes go on with block passes
  constexpr int kNucList = 512;
  __shared__ uint32_t lk[NUCLEUS ? kNucList : 1];
  __shared__ uint32_t bcast;
  __shared__ int pick_lo, pick_hi;
  Red<SW> red{rbuf};

  const int row = blockIdx.x;
  const int V = a.V;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const float urow = a.u[row];
  const float* zrow = a.logits + static_cast<size_t>(row) * V;
  const float4* s4 = reinterpret_cast<const float4*>(zrow);
  const int qmax = V / 4 - 1;
  float4 v[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) v[i] = s4[min(static_cast<int>(threadIdx.x) + i * ST, qmax)];
  float lm = -INFINITY;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const bool in = 4 * (static_cast<int>(threadIdx.x) + i * ST) < V;
    lm = in ? fmaxf(lm, fmaxf(fmaxf(v[i].x, v[i].y), fmaxf(v[i].z, v[i].w))) : lm;
  }
  if (threadIdx.x == 0) {
    pick_lo = 0x7fffffff;
    pick_hi = -1;
  }
  const float mz = red.max(lm) * a.inv_temp;
  // unnormalised probabilities exp(z - max z) in place (0 past V)
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const bool in = 4 * (static_cast<int>(threadIdx.x) + i * ST) < V;
    auto ex = [&](float z) { return in ? __builtin_amdgcn_exp2f((z * a.inv_temp - mz) * kLog2eS) : 0.f; };
    v[i] = make_float4(ex(v[i].x), ex(v[i].y), ex(v[i].z), ex(v[i].w));
  }
  // fn(i, c, x): every element of the thread, x its probability (id 4(t + 512 i) + c)
  auto each = [&](auto fn) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      fn(i, 0, v[i].x);
      fn(i, 1, v[i].y);
      fn(i, 2, v[i].z);
      fn(i, 3, v[i].w);
    }
  };
  auto id_of = [&](int i, int c) { return 4 * (static_cast<int>(threadIdx.x) + i * ST) + c; };

  if constexpr (NUCLEUS) {
    auto bits = [](float x) { return __builtin_bit_cast(uint32_t, x); };
    float st = 0.f;
    each([&](int, int, float x) { st += x; });
    const float need = a.top_p * red.sum(st);
    auto mass_ge = [&](uint32_t cand) {
      float m = 0.f;
      each([&](int, int, float x) { m += bits(x) >= cand ? x : 0.f; });
      return red.sum(m);
    };
    // the largest bit pattern tau whose mass at or above it still reaches the target
    // probabilities lie in [0, 1] (the largest logit gives exp2(0) = 1 exactly), so bits 31 and 30
    // of every pattern are 0 and the search starts at bit 29
    uint32_t tau = 0;
    int bit = 29;
#pragma nounroll
    for (; bit >= 30 - kPrefixBits; --bit) {
      const uint32_t cand = tau | (1u << bit);
      if (mass_ge(cand) >= need) tau = cand;
    }
    const uint32_t pmask = ~0u << (bit + 1);
    float nu = 0.f, ab = 0.f;
    each([&](int, int, float x) {
      nu += (bits(x) & pmask) == tau ? 1.f : 0.f;
      ab += (bits(x) & pmask) > tau ? x : 0.f;
    });
    float U;
    int pos = static_cast<int>(red.excl_scan(nu, U));
    if (U <= static_cast<float>(kNucList)) {
      const float above = red.sum(ab);
      each([&](int, int, float x) {
        if ((bits(x) & pmask) == tau) lk[pos++] = bits(x);
      });
      __syncthreads();
      if (threadIdx.x < 64) {
        constexpr int PER = kNucList / 64;
        const int n_all = static_cast<int>(U);
        const int np = (n_all + 63) / 64;
        uint32_t wk[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          wk[i] = 0u;   // past the list: probability 0, below every candidate
          const int j = lane + 64 * i;
          if (i < np && j < n_all) wk[i] = lk[j];
        }
        const float lim = need - above;
#pragma nounroll
        for (; bit >= 0; --bit) {
          const uint32_t cand = tau | (1u << bit);
          float sm = 0.f;
#pragma unroll
          for (int i = 0; i < PER; ++i)
            if (i < np) sm += wk[i] >= cand ? __builtin_bit_cast(float, wk[i]) : 0.f;
          if (wave_sum(sm) >= lim) tau = cand;
        }
        if (threadIdx.x == 0) bcast = tau;
      }
      __syncthreads();
      tau = bcast;
    } else {
#pragma nounroll
      for (; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        if (mass_ge(cand) >= need) tau = cand;
      }
    }
    float gt = 0.f, eq = 0.f;
    each([&](int, int, float x) {
      gt += bits(x) > tau ? x : 0.f;
      eq += bits(x) == tau ? 1.f : 0.f;
    });
    const float mass_gt = red.sum(gt);
    const int n_eq = static_cast<int>(red.sum(eq));
    const float e_eq = __builtin_bit_cast(float, tau);
    // ties kept: the ranks r with mass_gt + r * e_eq < need (monotone in r)
    int lo_r = 0, hi_r = n_eq;
    while (lo_r < hi_r) {
      const int mid = (lo_r + hi_r) / 2;
      if (mass_gt + static_cast<float>(mid) * e_eq < need) lo_r = mid + 1;
      else hi_r = mid;
    }
    const int n_keep = lo_r;
    // The search and mass_gt add the same masses in different orders, so mass_gt can round to
    // need or above: then no tie is kept (the mass above the threshold already reaches the
    // target), as the comparison at rank 0 says.
    // Fewer kept than tied: the id of the last kept tie.  Up to 64 ties are gathered and wave 0
    // ranks their ids; more take a bitwise search (the largest id x with fewer than n_keep ties
    // below it; ids are below 2^15).
    int id_cut = 0x7fffffff;
    if (n_keep == 0) {
      id_cut = -1;
    } else if (n_keep < n_eq && n_eq <= 64) {
      float n_all;
      int tp = static_cast<int>(red.excl_scan(eq, n_all));
      int* tid = reinterpret_cast<int*>(lk);   // the list is no longer read
      each([&](int i, int c, float y) {
        if (bits(y) == tau) tid[tp++] = id_of(i, c);
      });
      __syncthreads();
      if (threadIdx.x < 64) {
        const int mine = lane < n_eq ? tid[lane] : 0x7fffffff;
        int rank = 0;
        for (int j = 0; j < n_eq; ++j) rank += tid[j] < mine ? 1 : 0;
        if (lane < n_eq && rank == n_keep - 1) bcast = static_cast<uint32_t>(mine);
      }
      __syncthreads();
      id_cut = static_cast<int>(bcast);
    } else if (n_keep < n_eq) {
      int x = 0;
#pragma nounroll
      for (int b = 14; b >= 0; --b) {
        const int cand = x | (1 << b);
        float below = 0.f;
        each([&](int i, int c, float y) { below += bits(y) == tau && id_of(i, c) < cand ? 1.f : 0.f; });
        if (red.sum(below) < static_cast<float>(n_keep)) x = cand;
      }
      id_cut = x;
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      auto keep = [&](int c, float x) { return bits(x) > tau || (bits(x) == tau && id_of(i, c) <= id_cut) ? x : 0.f; };
      v[i] = make_float4(keep(0, v[i].x), keep(1, v[i].y), keep(2, v[i].z), keep(3, v[i].w));
    }
  }

  // each wave's mass of every piece row
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const float w = wave_sum((v[i].x + v[i].y) + (v[i].z + v[i].w));
    if (lane == 0) rowtot[wave][i] = w;
  }
  __syncthreads();
  // piece-row totals (waves added in order) and the total mass, the same on every thread
  auto row_total = [&](int i) {
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < SW; ++w) r += rowtot[w][i];
    return r;
  };
  float Sp = 0.f;
#pragma unroll
  for (int i = 0; i < NQ; ++i) Sp += row_total(i);
  const float target = urow * Sp;
  // the first piece row whose cumulative mass exceeds the target; failing that (u at the top
  // edge) the last piece row holding a kept id; and the mass of the rows before it
  int istar = (V - 1) / (4 * ST);
  if constexpr (NUCLEUS) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) istar = row_total(i) > 0.f ? i : istar;
  }
  float cum = 0.f, cum_star = 0.f;
  bool found = false;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const float r = row_total(i);
    const bool hit = !found && cum + r > target;
    istar = hit ? i : istar;
    cum_star = hit ? cum : cum_star;
    found = found || hit;
    cum += r;
  }
  if (!found) {
    cum_star = 0.f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) cum_star += i < istar ? row_total(i) : 0.f;
  }
  float4 vi = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < NQ; ++i)
    if (i == istar) vi = v[i];
  const float mi = (vi.x + vi.y) + (vi.z + vi.w);
  float tot;
  float run = cum_star + red.excl_scan(mi, tot);
  const int id0 = 4 * (static_cast<int>(threadIdx.x) + istar * ST);
  int lo = 0x7fffffff, hi = -1;
  const float ev[4] = {vi.x, vi.y, vi.z, vi.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // kept: an id below V (no truncation) or a probability left nonzero (nucleus)
    const bool kept = NUCLEUS ? ev[c] > 0.f : id0 + c < V;
    run += ev[c];
    lo = (kept && run > target && lo == 0x7fffffff) ? id0 + c : lo;
    hi = kept ? id0 + c : hi;
  }
  const float wlo = -wave_max(-static_cast<float>(lo == 0x7fffffff ? (1 << 24) : lo));
  const float whi = wave_max(static_cast<float>(hi));
  if (lane == 0) {
    if (wlo < static_cast<float>(1 << 24)) atomicMin(&pick_lo, static_cast<int>(wlo));
    if (whi >= 0.f) atomicMax(&pick_hi, static_cast<int>(whi));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // no id of the piece row passed the target (rounding at its end): its last kept id
    const int pick = pick_lo != 0x7fffffff ? pick_lo : pick_hi;
    if (pick >= 0) {
      a.tok[row] = pick;
      a.logp[row] = (zrow[pick] * a.inv_temp - mz) - logf(Sp);
    }
  }
}

template <int NQ, bool NUCLEUS>
hipError_t launch_full(const SampleArgs& a, hipStream_t st) {
  sample_full_k<NQ, NUCLEUS><<<a.N, ST, 0, st>>>(a);
  return hipGetLastError();
}

template <int NQ>
hipError_t launch_lean(const SampleArgs& a, hipStream_t st) {
  sample_topk_k<NQ><<<a.N, ST, 0, st>>>(a);
  return hipGetLastError();
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
  if (top_k > 0 && top_k <= kLeanK && top_k < V && V > 8 * ST && V % 4 == 0)
    return V > 32 * ST ? launch_lean<16>(a, st) : V > 16 * ST ? launch_lean<8>(a, st) : launch_lean<4>(a, st);
  if ((top_k == 0 || top_k >= V) && V > 8 * ST && V % 4 == 0) {
    if (top_p >= 1.0f)
      return V > 32 * ST ? launch_full<16, false>(a, st) : V > 16 * ST ? launch_full<8, false>(a, st)
                                                          : launch_full<4, false>(a, st);
    return V > 32 * ST ? launch_full<16, true>(a, st) : V > 16 * ST ? launch_full<8, true>(a, st)
                                                       : launch_full<4, true>(a, st);
  }
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
