// Weight-streaming products of the batched decoder step at decode-sized batches (M <= 64
// sequences, bf16): Y[M, N] = X[M, K] W^T, with every weight byte read from HBM once per step
// and shared by the M sequences ([FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环
// Transformer", model-hardware co-design principle: ready updates of independent sequences
// share one batched kernel; the tied layer weights are streamed once per step).
//
// One workgroup (4 waves) owns a 64-column tile of W, a group of 16*mb rows and a K-slice of KS
// columns.  Each wave streams its 16-column block from the fragment-major copy straight into the
// matrix-core B operand (register stages of 2 KB per wave), while the K-slice of X for the
// group's rows is staged once into LDS as bf16 (every load of the slice in flight at once).  The
// row groups of one tile are consecutive in dispatch order modulo the XCD count, so they share
// the tile's weight stream through one L2:
//   IN_BF16   X is a bf16 [M, K] activation;
//   IN_MERGE  X = [e_t ; bf16(s_{t-1})] for the gated merge.
// RMSNorm is folded in without a launch of its own.  A norm's input is the residual stream y
// after a residual product; that product's epilogue also writes xb = bf16(g * y) (g the gain of
// the next norm) and the tile's per-row sums of squares.  The next product reads xb as its X and
// multiplies its accumulator rows by 1/rms(y), computed from those sums in a fixed order: the
// per-row scale commutes with the product, so this is RMS(y; g) W^T with the operand g*y
// rounded to bf16 once.
// K is split only where the slice would not fit (S = 1 up to K = 2048 at 16 rows).  With S > 1
// each workgroup writes its fp32 partial at agent scope; the last of the S to arrive (a per-tile
// counter) adds the S partials in slice order 0..S-1 and applies the epilogue, so results do not
// depend on timing and no second launch is needed.  Epilogues:
//   EPI_F32     Y / rms stored fp32 (projections for the attentions);
//   EPI_RESID   y += Y, plus xb = bf16(g_next * y) and the tile's row sums of squares of y;
//   EPI_GELU    bf16(gelu(Y / rms));
//   EPI_SWIGLU  bf16(silu(gate / rms) * up / rms), gate and up rows interleaved in blocks of 16;
//   EPI_MERGE   y = g * e_t + (1 - g) * f with g = sigmoid(W_ge e_t + W_gs s + b_g) and
//               f = W_fb s ([DS] deepsonar "技术拆解 009｜RLT…" §2.4), gate and feedback rows
//               interleaved in blocks of 16, plus xb and the sums of squares for the first norm.
// Counters are zero between launches: the last workgroup of a tile resets its counter.
//
// Fragment-major copy of a [N][K] matrix: the 16-byte piece ((cb * K/64 + ks) * 2 + h) * 64 + lane
// holds W[16 cb + lane % 16][64 ks + 16 (lane / 16) + 8 h .. + 8].
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int WNT = 256;           // threads per workgroup (4 waves, one 16-column block each)
constexpr int XPAD = 8;            // LDS row padding of the X slice (bf16 elements)
constexpr int kXsBytes = 16 * 4 * (512 + XPAD) * 2;   // largest X slice: 64 rows x 512 (= 32 x 1024 = 16 x 2048)
constexpr int XJ = 16;             // 8-element X chunks per thread, all requested at once

// Largest K slice: the bf16 slice of 16*MB rows fits kXsBytes (every thread stages XJ chunks).
__host__ __device__ constexpr int ks_max(int MB) { return 2048 / MB; }

// 64-bit loads and stores at agent scope: they bypass the non-coherent cache levels, so a
// partial written by one workgroup is seen by the tile's last workgroup on any XCD.
__device__ __forceinline__ void store_agent(float* p, f32x4_t v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(q, __builtin_bit_cast(uint64_t, float2{v[0], v[1]}), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, __builtin_bit_cast(uint64_t, float2{v[2], v[3]}), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4_t load_agent(const float* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const float2 lo = __builtin_bit_cast(float2, __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const float2 hi = __builtin_bit_cast(float2, __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return f32x4_t{lo.x, lo.y, hi.x, hi.y};
}

// s_waitcnt vmcnt(0): this wave's stores have completed.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

constexpr bool scales_rows(int EPI) { return EPI == WEPI_F32 || EPI == WEPI_GELU || EPI == WEPI_SWIGLU; }

template <int MB, int IN, int EPI, int NS>
__global__ __launch_bounds__(WNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void wst_k(WstArgs a) {
  // row group blockIdx.y: rows 16*MB*y .. of every operand and output (the groups of one tile
  // share the tile's weight stream through the cache)
  {
    const int r0g = blockIdx.y * 16 * MB;
    a.M -= r0g;
    if (IN == WIN_BF16) a.x = static_cast<const bf16_t*>(a.x) + static_cast<size_t>(r0g) * a.ldx;
    if (IN == WIN_MERGE || EPI == WEPI_MERGE) a.e += static_cast<size_t>(r0g) * a.T * a.D;
    if (IN == WIN_MERGE) a.s += static_cast<size_t>(r0g) * a.D;
    if (a.outf) a.outf += static_cast<size_t>(r0g) * a.ldo;
    if (a.outb) a.outb += static_cast<size_t>(r0g) * a.ldo;
    if (a.xb_out) a.xb_out += static_cast<size_t>(r0g) * a.ldo;
    if (a.ssp_out) a.ssp_out += r0g;
    if (a.ssp) a.ssp += r0g;
    const int nt = a.N / 64;
    if (a.part) a.part += static_cast<size_t>(blockIdx.y) * nt * a.S * 4 * MB * 256;
    if (a.cnt) a.cnt += blockIdx.y * nt;
  }
  __shared__ __attribute__((aligned(16))) unsigned char lds[kXsBytes];
  __shared__ float inv[64];
  __shared__ float red[4][64];
  __shared__ int last_flag;
  constexpr int ROWS = 16 * MB;
  constexpr int SRC = IN == WIN_BF16 ? 1 : 2;   // 16-byte loads per 8-element chunk (the s half of the merge is fp32)
  bf16_t* xs = reinterpret_cast<bf16_t*>(lds);
  const int tile = blockIdx.x / a.S, sl = blockIdx.x % a.S;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, l16 = lane % 16, grp = lane / 16;
  const int KS = a.KS, kb = sl * KS, nst = KS / 64, pitch = KS + XPAD;
  // 1. weight stages: the first NS are requested before anything else
  const uint4* wbase = a.wf + (static_cast<size_t>(tile * 4 + wave) * (a.K / 64) + kb / 64) * 128 + lane;
  uint4 wb[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint4* q = wbase + static_cast<size_t>(min(s, nst - 1)) * 128;
    wb[s][0] = q[0];
    wb[s][1] = q[64];
  }
  // 2. this thread's chunks of the X slice, all requested at once: chunk c = tid + 256 j is row
  //    c / cpr, columns 8 (c % cpr) .. +7 of the slice (chunks past the slice re-read the last
  //    one and are not stored; rows past M are loaded clamped and stored as zero)
  const int cpr = KS / 8, nchunk = ROWS * cpr;
  uint4 raw[XJ][SRC];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int c = min(tid + WNT * j, nchunk - 1);
    const int r = min(c / cpr, a.M - 1), kc = (c % cpr) * 8;
    if constexpr (IN == WIN_BF16) {
      raw[j][0] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.x) + static_cast<size_t>(r) * a.ldx + kb + kc);
    } else {   // WIN_MERGE: [e_t ; s]; a chunk lies wholly in one half (D % 8 == 0)
      const int k = kb + kc;
      if (k < a.D) {
        raw[j][0] = *reinterpret_cast<const uint4*>(a.e + (static_cast<size_t>(r) * a.T + a.t) * a.D + k);
      } else {
        const float* p = a.s + static_cast<size_t>(r) * a.D + (k - a.D);
        raw[j][0] = *reinterpret_cast<const uint4*>(p);
        raw[j][1] = *reinterpret_cast<const uint4*>(p + 4);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int c = tid + WNT * j;
    if (c >= nchunk) continue;
    const int r = c / cpr, kc = (c % cpr) * 8;
    uint4 v = raw[j][0];
    if constexpr (IN == WIN_MERGE) {
      if (kb + kc >= a.D) {
        const float4 lo = __builtin_bit_cast(float4, raw[j][0]), hi = __builtin_bit_cast(float4, raw[j][1]);
        v = make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w));
      }
    }
    if (r >= a.M) v = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(xs + r * pitch + kc) = v;
  }
  __syncthreads();
  // 3. the products: two 16x16x32 MFMAs per 64-wide stage and row block
  f32x4_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16_t* arow = xs + l16 * pitch + 16 * grp;
  for (int s0 = 0; s0 < nst; s0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s0 + s < nst) {   // uniform
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < MB; ++i) {
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(arow + i * 16 * pitch + (s0 + s) * 64 + 8 * h);
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8_t, wb[s][h]), acc[i], 0, 0, 0);
          }
        if (s0 + NS < nst) {   // uniform: a ring only when the slice has more than NS stages
          const uint4* q = wbase + static_cast<size_t>(min(s0 + s + NS, nst - 1)) * 128;
          wb[s][0] = q[0];
          wb[s][1] = q[64];
        }
      }
    }
  }
  // 4. split-K: partials in fragment order (one float4 per lane and row block), written at
  //    agent scope; the tile's last workgroup adds them in slice order 0..S-1.  What the
  //    epilogue reads besides the partials (old residual rows, e_t, the norm's sums of squares)
  //    is requested with them.
  const int col = tile * 64 + wave * 16 + l16;
  const float* pp = nullptr;
  if (a.S > 1) {
    float* mine = a.part + (static_cast<size_t>(tile) * a.S * 4 + wave) * MB * 256 + lane * 4;
#pragma unroll
    for (int i = 0; i < MB; ++i) store_agent(mine + static_cast<size_t>(sl) * 4 * MB * 256 + i * 256, acc[i]);
    wait_vm();
    __syncthreads();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(a.cnt + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int is_last = old == a.S - 1;
      if (is_last) __hip_atomic_store(a.cnt + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = is_last;
    }
    __syncthreads();
    if (!last_flag) return;
    pp = mine;
  }
  float yold[MB][4], et[MB][4];
  if constexpr (EPI == WEPI_RESID) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        yold[i][v] = a.outf[static_cast<size_t>(min(16 * i + 4 * grp + v, a.M - 1)) * a.ldo + col];
  }
  if constexpr (EPI == WEPI_MERGE) {
    const int oc = tile * 32 + (wave >> 1) * 16 + l16;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        et[i][v] = bf16_to_f32(a.e[(static_cast<size_t>(min(16 * i + 4 * grp + v, a.M - 1)) * a.T + a.t) * a.D + oc]);
  }
  float ssv[16];
  const int srow = tid % 64, spart = tid / 64;
  if constexpr (scales_rows(EPI)) {
    // thread t sums tiles t/64, t/64 + 4, ... of row t % 64 (nt_in <= 64)
#pragma unroll
    for (int u = 0; u < 16; ++u) ssv[u] = a.ssp[min(spart + 4 * u, a.nt_in - 1) * 64 + min(srow, ROWS - 1)];
  }
  if (pp) {
    constexpr int ZB = 32 / MB;   // slices per batch: 32 float4 in flight per lane
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int z0 = 0; z0 < a.S; z0 += ZB) {
      f32x4_t pv[ZB][MB];
#pragma unroll
      for (int z = 0; z < ZB; ++z)
#pragma unroll
        for (int i = 0; i < MB; ++i)
          pv[z][i] = load_agent(pp + static_cast<size_t>(min(z0 + z, a.S - 1)) * 4 * MB * 256 + i * 256);
#pragma unroll
      for (int z = 0; z < ZB; ++z)
        if (z0 + z < a.S) {
#pragma unroll
          for (int i = 0; i < MB; ++i) acc[i] += pv[z][i];
        }
    }
  }
  if constexpr (scales_rows(EPI)) {
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) ss += spart + 4 * u < a.nt_in ? ssv[u] : 0.f;
    red[spart][srow] = ss;
    __syncthreads();
    if (tid < ROWS) {
      const float tot = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
      inv[tid] = 1.0f / sqrtf(tot / static_cast<float>(a.K) + a.eps);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][v] *= inv[16 * i + 4 * grp + v];
  }
  // 5. epilogue: lane holds rows 16 i + 4 grp + v of column `col`
  if constexpr (EPI == WEPI_F32 || EPI == WEPI_GELU) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * i + 4 * grp + v;
        if (row < a.M) {
          if constexpr (EPI == WEPI_F32) a.outf[static_cast<size_t>(row) * a.ldo + col] = acc[i][v];
          else a.outb[static_cast<size_t>(row) * a.ldo + col] = f32_to_bf16(gelu_erf(acc[i][v]));
        }
      }
  } else if constexpr (EPI == WEPI_RESID) {
    const float gn = a.gain_next ? a.gain_next[col] : 0.f;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * i + 4 * grp + v;
        float sq = 0.f;
        if (row < a.M) {
          const float y = yold[i][v] + acc[i][v];
          a.outf[static_cast<size_t>(row) * a.ldo + col] = y;
          if (a.gain_next) a.xb_out[static_cast<size_t>(row) * a.ldo + col] = f32_to_bf16(gn * y);
          sq = y * y;
        }
        sq = group_sum<16>(sq);
        if (l16 == 0) red[wave][row] = sq;
      }
    __syncthreads();
    if (tid < ROWS) a.ssp_out[tile * 64 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
  } else {   // WEPI_SWIGLU / WEPI_MERGE: waves 1 and 3 hold the second member of each pair
    float* xch = reinterpret_cast<float*>(lds);   // [2][64 rows][16]; the X slice is dead
    const int oc = tile * 32 + (wave >> 1) * 16 + l16;   // output column (waves 0 and 2)
    __syncthreads();
    if (wave & 1) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) xch[((wave >> 1) * 64 + 16 * i + 4 * grp + v) * 16 + l16] = acc[i][v];
    }
    __syncthreads();
    if (!(wave & 1)) {
      const float gn = EPI == WEPI_MERGE ? a.gain_next[oc] : 0.f;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * i + 4 * grp + v;
          const float second = xch[((wave >> 1) * 64 + row) * 16 + l16];
          if constexpr (EPI == WEPI_SWIGLU) {
            if (row < a.M) a.outb[static_cast<size_t>(row) * a.ldo + oc] = f32_to_bf16(silu_f(acc[i][v]) * second);
          } else {
            float sq = 0.f;
            if (row < a.M) {
              const float gt = sigmoid_f(acc[i][v] + a.bias[oc]);
              const float y = gt * et[i][v] + (1.0f - gt) * second;
              a.outf[static_cast<size_t>(row) * a.ldo + oc] = y;
              a.xb_out[static_cast<size_t>(row) * a.ldo + oc] = f32_to_bf16(gn * y);
              sq = y * y;
            }
            sq = group_sum<16>(sq);
            if (l16 == 0) red[wave >> 1][row] = sq;
          }
        }
    }
    if constexpr (EPI == WEPI_MERGE) {
      __syncthreads();
      if (tid < ROWS) a.ssp_out[tile * 64 + tid] = red[0][tid] + red[1][tid];
    }
  }
}

// s = g * y / rms(y) with the row sums of squares from per-tile partials; also s_out[b][step].
__global__ __launch_bounds__(256) void final_norm_ssp_k(const float* __restrict__ y, const float* __restrict__ ssp,
                                                        int nt, const float* __restrict__ gain, float* __restrict__ s,
                                                        float* __restrict__ s_out, int D, float eps, int step, int n) {
  const int b = blockIdx.x;
  __shared__ float inv_s;
  if (threadIdx.x == 0) {
    float ss = 0.f;
    for (int j = 0; j < nt; ++j) ss += ssp[j * 64 + b];
    inv_s = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  }
  __syncthreads();
  const float inv = inv_s;
  for (int c = threadIdx.x * 4; c < D; c += 256 * 4) {
    const float4 v = *reinterpret_cast<const float4*>(y + static_cast<size_t>(b) * D + c);
    const float4 g = *reinterpret_cast<const float4*>(gain + c);
    const float4 o = make_float4(g.x * (v.x * inv), g.y * (v.y * inv), g.z * (v.z * inv), g.w * (v.w * inv));
    *reinterpret_cast<float4*>(s + static_cast<size_t>(b) * D + c) = o;
    if (s_out) *reinterpret_cast<float4*>(s_out + (static_cast<size_t>(b) * n + step) * D + c) = o;
  }
}

// Fragment-major bf16 copy of the merge matrix [2D][2D], built from the fp32 canonical tensors:
// rows 32j .. 32j+15 are [W_ge | W_gs] rows 16j .. 16j+15, rows 32j+16 .. 32j+31 are [0 | W_fb]
// rows 16j .. 16j+15.
__global__ __launch_bounds__(256) void pack_merge_frag_k(const float* __restrict__ wge, const float* __restrict__ wgs,
                                                         const float* __restrict__ wfb, uint4* __restrict__ dst, int D,
                                                         size_t n_pieces) {
  const size_t c = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= n_pieces) return;
  const int K = 2 * D, KS = K / 64;
  const int lane = static_cast<int>(c % 64), h = static_cast<int>((c / 64) % 2);
  const size_t t = c / 128;
  const int ks = static_cast<int>(t % KS), cb = static_cast<int>(t / KS);
  const int row = cb * 16 + lane % 16, k = ks * 64 + 16 * (lane / 16) + 8 * h;
  const int blk = row / 32, within = row % 32, src_row = blk * 16 + within % 16;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int kk = k + j;
    if (within < 16) v[j] = kk < D ? wge[static_cast<size_t>(src_row) * D + kk] : wgs[static_cast<size_t>(src_row) * D + kk - D];
    else v[j] = kk < D ? 0.f : wfb[static_cast<size_t>(src_row) * D + kk - D];
  }
  dst[c] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

template <int MB, int IN, int EPI>
hipError_t launch_ns(const WstArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.N / 64 * a.S), static_cast<unsigned>((a.M + 16 * MB - 1) / (16 * MB)));
  const int nst = a.KS / 64;
  // a 16-stage weight ring for the long bf16 slices (the merge's slice holds fp32 rows too)
  if (IN == WIN_BF16 && nst >= 16) wst_k<MB, IN, EPI, (IN == WIN_BF16 ? 16 : 8)><<<grid, WNT, 0, st>>>(a);
  else if (nst >= 8) wst_k<MB, IN, EPI, 8><<<grid, WNT, 0, st>>>(a);
  else if (nst >= 4) wst_k<MB, IN, EPI, 4><<<grid, WNT, 0, st>>>(a);
  else wst_k<MB, IN, EPI, 2><<<grid, WNT, 0, st>>>(a);
  return hipGetLastError();
}

template <int IN, int EPI>
hipError_t launch_mb(const WstArgs& a, hipStream_t st) {
  switch (a.mb) {
    case 1: return launch_ns<1, IN, EPI>(a, st);
    case 2: return launch_ns<2, IN, EPI>(a, st);
    case 4: return launch_ns<4, IN, EPI>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool wst_supported(int M, int N, int K) { return M >= 1 && M <= 64 && N % 64 == 0 && K % 64 == 0; }

int wst_choose_split(int mb, int K) {
  // the fewest slices whose width is a multiple of 64 and fits the LDS slice: a split costs its
  // workgroups a round trip to the partials and back, more than the parallelism it adds
  for (int S = 1; S <= K / 64; ++S)
    if (K % S == 0 && (K / S) % 64 == 0 && K / S <= ks_max(mb)) return S;
  return K / 64;
}

size_t wst_part_floats(int M, int mb, int N, int S) {
  const int groups = (M + 16 * mb - 1) / (16 * mb);
  return S > 1 ? static_cast<size_t>(N / 64) * S * 4 * mb * 256 * groups : 0;
}

size_t wst_counters(int M, int mb, int N) { return static_cast<size_t>(N / 64) * ((M + 16 * mb - 1) / (16 * mb)); }

hipError_t launch_wst(const WstArgs& a, hipStream_t st) {
  if (!wst_supported(a.M, a.N, a.K) || a.S < 1 || a.K % a.S != 0) return hipErrorInvalidValue;
  if (a.mb != 1 && a.mb != 2 && a.mb != 4) return hipErrorInvalidValue;
  const int KS = a.K / a.S;
  if (KS % 64 != 0 || KS > ks_max(a.mb) || a.KS != KS) return hipErrorInvalidValue;
  if (a.S > 1 && (!a.part || !a.cnt)) return hipErrorInvalidValue;
  const bool scale = a.epi == WEPI_F32 || a.epi == WEPI_GELU || a.epi == WEPI_SWIGLU;
  if ((scale && (!a.ssp || a.nt_in < 1 || a.nt_in > 64)) || (a.epi == WEPI_RESID && (!a.ssp_out || (a.gain_next && !a.xb_out))) ||
      (a.epi == WEPI_MERGE && (!a.ssp_out || !a.bias || !a.e || !a.s || !a.gain_next || !a.xb_out)) ||
      (a.in == WIN_MERGE && (!a.e || !a.s)))
    return hipErrorInvalidValue;
  switch (a.in * 8 + a.epi) {
    case WIN_BF16 * 8 + WEPI_F32: return launch_mb<WIN_BF16, WEPI_F32>(a, st);
    case WIN_BF16 * 8 + WEPI_GELU: return launch_mb<WIN_BF16, WEPI_GELU>(a, st);
    case WIN_BF16 * 8 + WEPI_SWIGLU: return launch_mb<WIN_BF16, WEPI_SWIGLU>(a, st);
    case WIN_BF16 * 8 + WEPI_RESID: return launch_mb<WIN_BF16, WEPI_RESID>(a, st);
    case WIN_MERGE * 8 + WEPI_MERGE: return launch_mb<WIN_MERGE, WEPI_MERGE>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_final_norm_ssp(const float* y, const float* ssp, int nt, const float* gain, float* s, float* s_out,
                                 int B, int D, float eps, int step, int n, hipStream_t st) {
  if (D % 4 != 0 || B > 64) return hipErrorInvalidValue;
  final_norm_ssp_k<<<B, 256, 0, st>>>(y, ssp, nt, gain, s, s_out, D, eps, step, n);
  return hipGetLastError();
}

hipError_t launch_pack_merge_frag(const float* wge, const float* wgs, const float* wfb, void* dst, int D,
                                  hipStream_t st) {
  if (D % 32 != 0) return hipErrorInvalidValue;
  const size_t n = static_cast<size_t>(2 * D) * (2 * D) / 8;
  pack_merge_frag_k<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(wge, wgs, wfb, static_cast<uint4*>(dst), D, n);
  return hipGetLastError();
}

}  // namespace rlt
