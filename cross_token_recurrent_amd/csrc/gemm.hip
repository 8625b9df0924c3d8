// Token-parallel matrix products on the MFMA units: C[M,N] = A[M,K] * W[N,K]^T.
//
// Used for every dense contraction the encoder runs over known tokens (QKV, attention
// output, FFN, memory projections) and for the output head ([FI] model-hardware
// co-design: encoder features and memory projections are token-parallel).
// bf16 mode: v_mfma_f32_16x16x32_bf16 with fp32 accumulation; fp32 mode:
// v_mfma_f32_16x16x4_f32.  A block computes a 128x128 tile with 4 waves (2x2), each
// wave a 64x64 sub-tile of 4x4 MFMA 16x16 tiles; K advances 64 per LDS stage (two MFMA
// k-steps between barriers), with up to two stages of global loads in flight ahead of it.  The epilogue stages
// each wave's results through LDS, 16 rows at a time, so every lane writes whole 16-byte
// chunks of a row (or of a head's slice of it, for the cache scatters).
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NTH = 256;

template <typename TW> struct Tile;
template <> struct Tile<bf16_t> { static constexpr int PAD = 8; };   // row pitch 80 B
template <> struct Tile<float> { static constexpr int PAD = 4; };    // row pitch 144 B

// Number of 16-byte chunks of one BMxBK (or BNxBK) tile, per thread.
template <typename TW> constexpr int chunks_per_thread() { return (BM * BK * sizeof(TW) / 16) / NTH; }

// One tile's chunks as loaded: 16 bytes of the storage type per chunk, or, for an fp32 source
// feeding bf16 storage, the 32 source bytes of the chunk (converted when stored to LDS, so
// a load in flight is not waited on until its stage is consumed).
template <typename TW, bool SRC_F32> struct Raw {
  static constexpr bool CONV = SRC_F32 && sizeof(TW) == 2;
  uint4 v[chunks_per_thread<TW>()][CONV ? 2 : 1];
};

// Load one tile's chunks.  Rows past the operand are clamped to its last row (their products
// land in rows or columns the epilogue never writes), so every load is unconditional.
template <typename TW, bool SRC_F32>
__device__ __forceinline__ void load_tile(const void* __restrict__ base, int ld, int row0, int rows_valid, int k0,
                                          Raw<TW, SRC_F32>& r) {
  constexpr int EPC = 16 / sizeof(TW);     // elements per chunk
  constexpr int CPR = BK / EPC;            // chunks per row
#pragma unroll
  for (int i = 0; i < chunks_per_thread<TW>(); ++i) {
    const int c = threadIdx.x + i * NTH;
    const int row = min(c / CPR, rows_valid - 1), kc = (c % CPR) * EPC;
    if constexpr (Raw<TW, SRC_F32>::CONV) {
      const float* p = static_cast<const float*>(base) + static_cast<size_t>(row0 + row) * ld + k0 + kc;
      r.v[i][0] = *reinterpret_cast<const uint4*>(p);
      r.v[i][1] = *reinterpret_cast<const uint4*>(p + 4);
    } else {
      const TW* p = static_cast<const TW*>(base) + static_cast<size_t>(row0 + row) * ld + k0 + kc;
      r.v[i][0] = *reinterpret_cast<const uint4*>(p);
    }
  }
}

template <typename TW, bool SRC_F32>
__device__ __forceinline__ void store_tile(TW* __restrict__ lds, const Raw<TW, SRC_F32>& r) {
  constexpr int EPC = 16 / sizeof(TW);
  constexpr int CPR = BK / EPC;
  constexpr int PITCH = BK + Tile<TW>::PAD;
#pragma unroll
  for (int i = 0; i < chunks_per_thread<TW>(); ++i) {
    const int c = threadIdx.x + i * NTH;
    const int row = c / CPR, kc = (c % CPR) * EPC;
    uint4 v = r.v[i][0];
    if constexpr (Raw<TW, SRC_F32>::CONV) {
      const float4 a = __builtin_bit_cast(float4, r.v[i][0]);
      const float4 b = __builtin_bit_cast(float4, r.v[i][1]);
      v = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
    }
    *reinterpret_cast<uint4*>(lds + row * PITCH + kc) = v;
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Eight consecutive elements in the storage type: one 16-byte store (two for fp32) when
// vec, else element by element for the first nvalid.
template <typename TW>
__device__ __forceinline__ void store8(TW* p, const float (&f)[8], bool vec, int nvalid) {
  if (vec && nvalid >= 8) {
    if constexpr (sizeof(TW) == 2) {
      *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                                pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    } else {
      *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < nvalid) store_from_f32(p + e, f[e]);
  }
}

// Columns n..n+7 of row m in the storage type (EPI_STORE, EPI_GELU, EPI_SCATTER_HEADS): the
// output itself and/or the scatter of the key/value columns into their cache layouts.
template <typename TW>
__device__ __forceinline__ void store_row8(const GemmArgs& g, int m, int n, const float (&f)[8], bool vec_out) {
  const int nvalid = g.N - n;
  if (g.epi != EPI_SCATTER_HEADS)
    store8(static_cast<TW*>(g.out) + static_cast<size_t>(m) * g.ldo + n, f, vec_out, nvalid);
  if (g.sc_k && n >= g.sc_c0) {
    const int rel = n - g.sc_c0;
    const int which = rel / g.sc_D;
    if (which < 2) {
      // a chunk never straddles a head: dh and the column offsets are multiples of 8
      const int c = rel % g.sc_D, h = c / g.sc_dh, cc = c % g.sc_dh;
      const int b = g.sc_b0 + m / g.sc_n, t = g.sc_t0 + m % g.sc_n;
      const size_t bh = static_cast<size_t>(b) * g.sc_H + h;
      if (which == 1 && g.epi == EPI_SCATTER_HEADS) {
        // memory values: key-blocked [..][T8/8][dh][8]
        TW* base = static_cast<TW*>(g.sc_v) + (bh * ((g.sc_T + 7) / 8) + t / 8) * g.sc_dh * 8 + t % 8;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < nvalid) store_from_f32(base + (cc + e) * 8, f[e]);
      } else {
        TW* dst = static_cast<TW*>(which == 0 ? g.sc_k : g.sc_v) + (bh * g.sc_T + t) * g.sc_dh + cc;
        store8(dst, f, true, nvalid);
      }
    }
  }
}

template <typename TW, bool A_F32, int NS>
__global__ __launch_bounds__(NTH) void gemm_nt_k(GemmArgs g) {
  constexpr int PITCH = BK + Tile<TW>::PAD;
  constexpr int TILE_BYTES = BM * PITCH * static_cast<int>(sizeof(TW));
  constexpr int SP = 64 + 4;                     // staging row pitch (floats)
  constexpr int STAGE_BYTES = 4 * 16 * SP * 4;   // 16 rows per wave
  constexpr int LDS_BYTES = 2 * TILE_BYTES > STAGE_BYTES ? 2 * TILE_BYTES : STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  TW* As = reinterpret_cast<TW*>(lds);
  TW* Ws = reinterpret_cast<TW*>(lds + TILE_BYTES);

  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  // split-K: this block's slice of K, and its partial goes to the workspace as plain fp32
  const int kslice = g.K / g.k_split, kbeg = blockIdx.z * kslice;
  if (g.k_split > 1) {
    g.out = g.splitk_ws + static_cast<size_t>(blockIdx.z) * g.M * g.N;
    g.ldo = g.N;
    g.epi = EPI_STORE_F32;
  }
  const int wm = wave / 2, wn = wave % 2;
  const int mrows = min(BM, g.M - m0), nrows = min(BN, g.N - n0);

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // NS stages of K in flight: stage k is requested NS stages before it is consumed (the
  // requests past the end of K re-read the last stage and are never consumed)
  Raw<TW, A_F32> ra[NS];
  Raw<TW, false> rw[NS];
  const int kend = kbeg + kslice;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int kk = min(kbeg + s * BK, kend - BK);
    load_tile<TW, A_F32>(g.A, g.lda, m0, mrows, kk, ra[s]);
    load_tile<TW, false>(g.W, g.ldw, n0, nrows, kk, rw[s]);
  }

  for (int k00 = kbeg; k00 < kend; k00 += NS * BK)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int k0 = k00 + s * BK;   // the slice is a multiple of NS * BK
    __syncthreads();
    store_tile<TW, A_F32>(As, ra[s]);
    store_tile<TW, false>(Ws, rw[s]);
    __syncthreads();
    {
      const int kk = min(k0 + NS * BK, kend - BK);
      load_tile<TW, A_F32>(g.A, g.lda, m0, mrows, kk, ra[s]);
      load_tile<TW, false>(g.W, g.ldw, n0, nrows, kk, rw[s]);
    }
    const int r16 = lane % 16, kq = lane / 16;
    if constexpr (sizeof(TW) == 2) {
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + i * 16 + r16) * PITCH + ks * 32 + kq * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(Ws + (wn * 64 + j * 16 + r16) * PITCH + ks * 32 + kq * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
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

  // Epilogue.  MFMA 16x16 output: lane holds rows 4*(lane/16)+v, column lane%16.  Per pass
  // the wave stages 16 rows of its 64x64 sub-tile (activation applied) and writes them back
  // as row chunks.
  __syncthreads();   // the operand tiles are dead: their LDS becomes the staging area
  float* st = reinterpret_cast<float*>(lds) + wave * 16 * SP;
  const int col_l = lane % 16, row_q = (lane / 16) * 4;
  const int mw = m0 + wm * 64, nw = n0 + wn * 64;
  const int epi = g.epi;
  const bool f32_out = epi == EPI_STORE_F32 || epi == EPI_RESID_F32;
  const size_t out_esz = f32_out ? 4 : sizeof(TW);
  const bool vec_out = g.out && (reinterpret_cast<uintptr_t>(g.out) % 16 == 0) && ((g.ldo * out_esz) % 16 == 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (epi == EPI_SWIGLU) {
#pragma unroll
      for (int jp = 0; jp < 2; ++jp)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          st[(row_q + v) * SP + jp * 16 + col_l] = silu_f(acc[i][2 * jp][v]) * acc[i][2 * jp + 1][v];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float x = acc[i][j][v];
          st[(row_q + v) * SP + j * 16 + col_l] = epi == EPI_GELU ? gelu_erf(x) : x;
        }
    }
    wave_sync_lds();
    const int mr = mw + 16 * i;
    if (f32_out) {
      // 16 rows x 16 float4 chunks
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = lane + 64 * k, r = c / 16, c4 = (c % 16) * 4;
        const int m = mr + r, n = nw + c4;
        if (m >= g.M || n >= g.N) continue;
        const float4 v = *reinterpret_cast<const float4*>(st + r * SP + c4);
        float* p = static_cast<float*>(g.out) + static_cast<size_t>(m) * g.ldo + n;
        if (vec_out && n + 4 <= g.N) {
          if (epi == EPI_RESID_F32) {
            const float4 o = *reinterpret_cast<const float4*>(p);
            *reinterpret_cast<float4*>(p) = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
          } else {
            *reinterpret_cast<float4*>(p) = v;
          }
        } else {
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e >= g.N) break;
            if (epi == EPI_RESID_F32) p[e] += vv[e];
            else p[e] = vv[e];
          }
        }
      }
    } else if (epi == EPI_SWIGLU) {
      // 16 rows x 32 activation columns (gate/up pairs of the sub-tile), 8 per lane
      const int r = lane / 4, c8 = (lane % 4) * 8;
      const int m = mr + r, oc = nw / 2 + c8;
      if (m < g.M && oc < g.N / 2) {
        float f[8];
        const float4 a = *reinterpret_cast<const float4*>(st + r * SP + c8);
        const float4 b = *reinterpret_cast<const float4*>(st + r * SP + c8 + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        store8(static_cast<TW*>(g.out) + static_cast<size_t>(m) * g.ldo + oc, f, vec_out, g.N / 2 - oc);
      }
    } else {
      // 16 rows x 8 chunks of 8 columns
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = lane + 64 * k, r = c / 8, c8 = (c % 8) * 8;
        const int m = mr + r, n = nw + c8;
        if (m >= g.M || n >= g.N) continue;
        float f[8];
        const float4 a = *reinterpret_cast<const float4*>(st + r * SP + c8);
        const float4 b = *reinterpret_cast<const float4*>(st + r * SP + c8 + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        store_row8<TW>(g, m, n, f, vec_out);
      }
    }
    wave_sync_lds();
  }
}

// Split-K reduction: out = (or +=) the sum of the S partials, added in the order z = 0..S-1.
__global__ __launch_bounds__(256) void splitk_reduce_k(const float* __restrict__ ws, float* __restrict__ out, int M,
                                                       int N, int ldo, int S, int resid) {
  const int n4 = N / 4;
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<size_t>(M) * n4) return;
  const int m = static_cast<int>(i / n4), c = static_cast<int>(i % n4) * 4;
  const size_t plane = static_cast<size_t>(M) * N;
  float4 s = *reinterpret_cast<const float4*>(ws + static_cast<size_t>(m) * N + c);
  for (int z = 1; z < S; ++z) {
    const float4 v = *reinterpret_cast<const float4*>(ws + z * plane + static_cast<size_t>(m) * N + c);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(m) * ldo + c);
  if (resid) {
    const float4 r = *o;
    s.x += r.x; s.y += r.y; s.z += r.z; s.w += r.w;
  }
  *o = s;
}

constexpr int kMaxSplit = 8;
constexpr int kFillBlocks = 256;   // one block per CU

}  // namespace

size_t gemm_splitk_ws_floats(int M, int N) { return static_cast<size_t>(kMaxSplit) * M * N; }

hipError_t launch_gemm(const GemmArgs& g0, int dtype, hipStream_t st) {
  GemmArgs g = g0;
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % BK != 0) return hipErrorInvalidValue;
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM);
  if (grid.y > 65535u) return hipErrorInvalidValue;
  // prefetch depth: two stages when they divide K
  const int nsd = g.K % (2 * BK) == 0 ? 2 : 1;
  // split K when the output tiles leave most CUs idle (fp32-output epilogues only): the
  // largest S <= 8 whose slices stay multiples of the prefetch depth and fit the workspace
  g.k_split = 1;
  const int tiles = static_cast<int>(grid.x * grid.y);
  const bool vec4 = g.N % 4 == 0 && g.ldo % 4 == 0 && reinterpret_cast<uintptr_t>(g.out) % 16 == 0;
  if (g.splitk_ws && vec4 && (g.epi == EPI_STORE_F32 || g.epi == EPI_RESID_F32) && 2 * tiles <= kFillBlocks) {
    int S = 1;
    while (S * 2 <= kMaxSplit && tiles * S * 2 <= kFillBlocks && g.K % (S * 2 * nsd * BK) == 0 &&
           static_cast<size_t>(S) * 2 * g.M * g.N <= g.splitk_ws_floats)
      S *= 2;
    g.k_split = S;
  }
  grid.z = g.k_split;
  const bool k2 = nsd == 2;
  if (dtype == RLT_DTYPE_BF16) {
    if (g.a_f32) {
      if (k2) gemm_nt_k<bf16_t, true, 2><<<grid, NTH, 0, st>>>(g);
      else gemm_nt_k<bf16_t, true, 1><<<grid, NTH, 0, st>>>(g);
    } else {
      if (k2) gemm_nt_k<bf16_t, false, 2><<<grid, NTH, 0, st>>>(g);
      else gemm_nt_k<bf16_t, false, 1><<<grid, NTH, 0, st>>>(g);
    }
  } else {
    if (k2) gemm_nt_k<float, false, 2><<<grid, NTH, 0, st>>>(g);
    else gemm_nt_k<float, false, 1><<<grid, NTH, 0, st>>>(g);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.k_split == 1) return e;
  const size_t n = static_cast<size_t>(g.M) * (g.N / 4);
  splitk_reduce_k<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(
      g.splitk_ws, static_cast<float*>(g.out), g.M, g.N, g.ldo, g.k_split, g.epi == EPI_RESID_F32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace rlt

// ---------------------------------------------------------------------------------------------
// Fragment-major copy of a packed [N][K] bf16 matrix (N % 16 == 0, K % 64 == 0), streamed by the
// decoder step's weight-streaming products: the 16-byte piece ((cb * K/64 + ks) * 2 + h) * 64 + lane
// holds W[16 cb + lane % 16][64 ks + 16 (lane / 16) + 8 h .. +8], so the 64 lanes' pieces of one
// matrix-core B operand are one contiguous kilobyte.
// ---------------------------------------------------------------------------------------------
namespace rlt {
namespace {

__global__ __launch_bounds__(256) void pack_frag_k(const bf16_t* __restrict__ w, uint4* __restrict__ dst, int N, int K,
                                                   size_t n_pieces) {
  const size_t c = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= n_pieces) return;
  const int lane = static_cast<int>(c % 64), h = static_cast<int>((c / 64) % 2);
  const size_t t = c / 128;
  const int KS = K / 64;
  const int ks = static_cast<int>(t % KS), cb = static_cast<int>(t / KS);
  const int row = cb * 16 + lane % 16, k = ks * 64 + 16 * (lane / 16) + 8 * h;
  dst[c] = *reinterpret_cast<const uint4*>(w + static_cast<size_t>(row) * K + k);
}

}  // namespace

hipError_t launch_pack_frag(const void* w, void* dst, int N, int K, hipStream_t st) {
  if (N % 16 != 0 || K % 64 != 0) return hipErrorInvalidValue;
  const size_t n = static_cast<size_t>(N) * K / 8;
  pack_frag_k<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(static_cast<const bf16_t*>(w),
                                                                        static_cast<uint4*>(dst), N, K, n);
  return hipGetLastError();
}

}  // namespace rlt
