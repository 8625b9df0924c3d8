// Causal multi-head attention of the encoder over known tokens ([FI] architecture
// paragraph: the encoder runs under a causal mask, token-parallel; [AL] §一: the memory
// never shows future tokens).
//
// bf16 storage: a flash-attention kernel on the matrix cores (v_mfma_f32_16x16x16_bf16).
// A workgroup of four waves takes 64 queries of one (sequence, head), 16 per wave; key and
// value tiles of 64 positions are staged through LDS (values transposed).  Each wave computes
// the transposed score tile S^T = K Q^T (keys x its 16 queries), so a lane holds four keys of
// one query: the online softmax needs only in-lane work plus a reduction over the four lane
// rows (two lane shuffles), and the bf16 weights P^T are already laid out as the B operand
// of O^T += V^T P^T.  Scores in the log2 domain, fp32 accumulation, weights rounded to bf16
// before the value product (the normaliser sums the rounded weights).
//
// fp32 storage: each query is owned by LPQ = dh/16 lanes, each holding 16 dimensions of the
// (pre-scaled) query and of the output accumulator.  Key and value tiles of 64 positions (32
// for dh = 128) are staged through LDS as fp32; scores are processed 16 keys at a time with an
// online softmax (running max, rescaled sum and output).
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

typedef __attribute__((ext_vector_type(4))) short s4_t;    // four bf16: a 16x16x16 MFMA operand
typedef __attribute__((ext_vector_type(4))) float f4_t;

// D += A B on v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16][8 (l / 16) .. +8] and
// B[8 (l / 16) .. +8][l % 16] as eight bf16 (any fixed order of the 32 contracted indices that the
// two operands share), and D[4 (l / 16) + v][l % 16].
__device__ __forceinline__ f4_t mfma32(const uint4& a, const uint4& b, f4_t c) {
  return __builtin_bit_cast(f4_t, __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                          __builtin_bit_cast(bf16x8_t, b),
                                                                          __builtin_bit_cast(f32x4_t, c), 0, 0, 0));
}

// sum / max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ float rows4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}

template <int DH>
__global__ __launch_bounds__(NTH) void enc_attn_mfma_k(AttnArgs a) {
  constexpr int BQ = 64, BK = 64;
  constexpr int KP = DH + 8;        // K tile row pitch (elements; rows stay 16-byte aligned)
  constexpr int VP = BK + 8;        // V^T tile row pitch
  // V^T row d holds key j at column j ^ vsw(d): the 16 lanes that store one key's 8-dim chunks
  // (dims 8 apart) then land in 8 different banks instead of one, and the groups of four keys
  // the products read stay contiguous (the swizzle only flips key bits 2..4)
  auto vsw = [](int d) { return 4 * ((d >> 3) & 7); };
  constexpr int ND = DH / 16;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[BK * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[DH * VP];

  const int h = blockIdx.y, b = blockIdx.z;
  const int qb = gridDim.x - 1 - blockIdx.x;            // late (longer) query blocks first
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int qi = qb * BQ + wave * 16 + col;              // this lane's query
  const int qc = min(qi, a.n - 1);
  const int qpos = a.t0 + qc;
  const int kend = a.t0 + min(a.n, (qb + 1) * BQ);      // keys the block needs
  const int wave_last = a.t0 + min(a.n - 1, qb * BQ + wave * 16 + 15);
  const float sc = kLog2e / sqrtf(static_cast<float>(DH));

  // Q^T as the B operand of S^T = K Q^T: lane holds q[col][32kc + 8grp .. +8] (d_h >= 32, the
  // 16x16x32 products) or q[col][16kk + 4grp .. +4] (d_h = 16)
  constexpr bool K32 = DH >= 32;
  constexpr int NQ8 = K32 ? DH / 32 : 1, NQ4 = K32 ? 1 : ND;
  uint4 qreg8[NQ8];
  s4_t qreg[NQ4];
  const bf16_t* qp = static_cast<const bf16_t*>(a.q) + static_cast<size_t>(b * a.n + qc) * a.ldq + h * DH;
  if constexpr (K32) {
#pragma unroll
    for (int kc = 0; kc < NQ8; ++kc) qreg8[kc] = *reinterpret_cast<const uint4*>(qp + 32 * kc + 8 * grp);
  } else {
#pragma unroll
    for (int kk = 0; kk < ND; ++kk) qreg[kk] = *reinterpret_cast<const s4_t*>(qp + 16 * kk + 4 * grp);
  }
  f4_t o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lp = 0.f;   // running max (per query); this lane's share of the sum

  const bf16_t* kb = static_cast<const bf16_t*>(a.k) + b * a.kv_ld_b + h * a.kv_ld_h;
  const bf16_t* vb = static_cast<const bf16_t*>(a.v) + b * a.kv_ld_b + h * a.kv_ld_h;
  // the next tile's K and V chunks are requested into registers before this tile's products, so
  // their latency overlaps the matrix work; they go to LDS after the next barrier
  constexpr int NCH = (BK * DH / 8 + NTH - 1) / NTH;   // 16-byte chunks per thread and tile
  uint4 kpre[NCH], vpre[NCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTH;
      const int j = c / (DH / 8), d0 = (c % (DH / 8)) * 8;
      uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
      if (c < BK * DH / 8 && k0 + j < kend) {
        kv = *reinterpret_cast<const uint4*>(kb + static_cast<size_t>(k0 + j) * a.kv_ld_t + d0);
        vv = *reinterpret_cast<const uint4*>(vb + static_cast<size_t>(k0 + j) * a.kv_ld_t + d0);
      }
      kpre[i] = kv;
      vpre[i] = vv;
    }
  };
  gload(0);
  for (int k0 = 0; k0 < kend; k0 += BK) {
    __syncthreads();   // every read of the previous tile is done
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTH;
      if (c >= BK * DH / 8) break;
      const int j = c / (DH / 8), d0 = (c % (DH / 8)) * 8;
      *reinterpret_cast<uint4*>(Ks + j * KP + d0) = kpre[i];
      const uint32_t w[4] = {vpre[i].x, vpre[i].y, vpre[i].z, vpre[i].w};
      const int jc = j ^ vsw(d0);   // the eight dims of a chunk share their 8-block
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Vt[(d0 + 2 * q) * VP + jc] = static_cast<bf16_t>(w[q] & 0xffffu);
        Vt[(d0 + 2 * q + 1) * VP + jc] = static_cast<bf16_t>(w[q] >> 16);
      }
    }
    __syncthreads();
    if (k0 + BK < kend) gload(k0 + BK);
    if (k0 > wave_last) continue;   // uniform: the whole tile lies after this wave's queries

    // S^T sub-tiles of 16 keys: lane holds keys k0 + 16ks + 4grp + v of query col
    float s[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f4_t acc = f4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (K32) {
#pragma unroll
        for (int kc = 0; kc < NQ8; ++kc)
          acc = mfma32(*reinterpret_cast<const uint4*>(Ks + (16 * ks + col) * KP + 32 * kc + 8 * grp), qreg8[kc], acc);
      } else {
#pragma unroll
        for (int kk = 0; kk < ND; ++kk) {
          const s4_t ka = *reinterpret_cast<const s4_t*>(Ks + (16 * ks + col) * KP + 16 * kk + 4 * grp);
          acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, qreg[kk], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = k0 + 16 * ks + 4 * grp + v;
        s[ks][v] = key <= qpos ? acc[v] * sc : -INFINITY;   // causal (key < kend follows)
        mt = fmaxf(mt, s[ks][v]);
      }
    }
    const float mn = fmaxf(m, rows4_max(mt));   // finite: key 0 is visible to every query
    const float corr = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    lp *= corr;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[dt] *= corr;
    s4_t pk[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float pr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pr[v] = round_to<bf16_t>(__builtin_amdgcn_exp2f(s[ks][v] - m));
        lp += pr[v];
      }
      const uint32_t lo = pack_bf16x2(pr[0], pr[1]), hi = pack_bf16x2(pr[2], pr[3]);
      pk[ks] = __builtin_bit_cast(s4_t, make_uint2(lo, hi));
    }
    // O^T[d][q] += V^T[d][keys] P^T[keys][q], 32 keys per product: lane grp contracts keys
    // 32p + 4grp .. +3 (from score tile 2p) and 32p + 16 + 4grp .. +3 (tile 2p + 1) on both operands
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const int row = 16 * dt + col;
      const bf16_t* vr = Vt + row * VP;
      const int sw = vsw(row);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + ((32 * p + 4 * grp) ^ sw));
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + ((32 * p + 16 + 4 * grp) ^ sw));
        const uint2 p0 = __builtin_bit_cast(uint2, pk[2 * p]), p1 = __builtin_bit_cast(uint2, pk[2 * p + 1]);
        o[dt] = mfma32(make_uint4(lo.x, lo.y, hi.x, hi.y), make_uint4(p0.x, p0.y, p1.x, p1.y), o[dt]);
      }
    }
  }
  const float inv = 1.0f / rows4_sum(lp);
  if (qi < a.n) {
    bf16_t* op = static_cast<bf16_t*>(a.out) + static_cast<size_t>(b * a.n + qi) * a.ldo + h * DH;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const uint32_t lo = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv), hi = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * dt + 4 * grp) = make_uint2(lo, hi);
    }
  }
}

template <int DH>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t st) {
  dim3 grid((a.n + 63) / 64, a.H, a.Bc);
  enc_attn_mfma_k<DH><<<grid, NTH, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    switch (a.dh) {
      case 16: return launch_mfma<16>(a, st);
      case 32: return launch_mfma<32>(a, st);
      case 64: return launch_mfma<64>(a, st);
      case 128: return launch_mfma<128>(a, st);
      default: return hipErrorInvalidValue;
    }
  } else {
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
}

}  // namespace

hipError_t launch_enc_attention(const AttnArgs& a, int dtype, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  return dtype == RLT_DTYPE_BF16 ? launch_t<bf16_t>(a, st) : launch_t<float>(a, st);
}

}  // namespace rlt
