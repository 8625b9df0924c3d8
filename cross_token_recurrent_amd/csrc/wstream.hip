// Weight-streaming products of the batched decoder step (M <= 512 sequences, bf16):
// Y[M, N] = X[M, K] W^T, with every weight byte read from HBM once per step and shared by the
// M sequences ([FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环
// Transformer", model-hardware co-design principle: ready updates of independent sequences
// share one batched kernel; the tied layer weights are streamed once per step).
//
// One workgroup of NW waves owns one 16-column block of the output (a gate/up or gate/feedback
// pair of blocks for the paired epilogues) over one group of up to 64 rows and the whole of K
// (past 64 rows, grid y walks the row groups; their reads of a weight block meet in L2).  Its waves split K
// into contiguous runs of 64-wide stages, so every CU streams weight bytes that no other CU
// reads, and no workgroup waits for another.  Both operands come from fragment-major copies, so
// every load instruction of a wave reads one contiguous kilobyte:
//   W  the piece ((cb * K/64 + ks) * 2 + h) * 64 + lane holds W[16 cb + lane % 16][64 ks + 16 (lane / 16) + 8 h .. + 8];
//   X  the piece ((i * K/64 + ks) * 2 + h) * 64 + lane holds X[16 i + lane % 16][64 ks + 16 (lane / 16) + 8 h .. + 8]
//      (act_offset in device_common.h), written in that layout by whatever produces X: the
//      residual epilogues here (the next norm's operand), the FFN activation epilogues, the
//      attention kernels and the merge's input packing.
// Loaded row by row instead, the 16 rows of an A fragment touch 16 cache lines per instruction,
// and at M = 64 those reads (four bytes of X per byte of W) bound the product.  Each wave keeps
// NSR stages of loads in flight; the waves' partial tiles are added through LDS in wave order,
// so results do not depend on timing.
// RMSNorm is folded in without a launch of its own.  A norm's input is the residual stream y
// after a residual product; that product's epilogue also writes xb = bf16(g * y) (g the gain of
// the next norm) and its 16-column block's per-row sums of squares.  The next product reads xb as
// its X and multiplies its accumulator rows by 1/rms(y), computed from those sums in a fixed
// order: the per-row scale commutes with the product, so this is RMS(y; g) W^T with the operand
// g*y rounded to bf16 once.  Epilogues:
//   EPI_F32     Y / rms stored fp32, row-major (projections for the attentions);
//   EPI_RESID   y += Y, plus xb = bf16(g_next * y) and the block's row sums of squares of y;
//   EPI_GELU    bf16(gelu(Y / rms));
//   EPI_SWIGLU  bf16(silu(gate / rms) * up / rms), gate and up rows interleaved in blocks of 16;
//   EPI_MERGE   y = g * e_t + (1 - g) * f with g = sigmoid(W_ge e_t + W_gs s + b_g) and
//               f = W_fb s ([DS] deepsonar "技术拆解 009｜RLT…" §2.4), gate and feedback rows
//               interleaved in blocks of 16, plus xb and the sums of squares for the first norm.
// Rows past M are carried through the products (their fragment pieces are never written) and
// never stored: a matrix-core output row depends only on the same row of A.
#include "act_layout.h"
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int kWsnMaxTiles = 128;  // most 16-column sums of squares per row (D <= 2048)
constexpr int kWsnMaxRows = 512;   // rows of one product: up to 8 row groups of 64

constexpr bool scales_rows(int EPI) { return EPI == WEPI_F32 || EPI == WEPI_GELU || EPI == WEPI_SWIGLU; }

template <int MB, int EPI, int NW, int NSR, int NCB>
__global__ __launch_bounds__(NW * 64) void wsn_k(WstArgs a) {
  // NCB column blocks per workgroup (their waves share each X load through the CU's L1): whole
  // pairs for the paired epilogues (block 2p the gate, 2p+1 its partner), else independent blocks
  constexpr bool PAIRED = EPI == WEPI_SWIGLU || EPI == WEPI_MERGE;
  static_assert(NCB == 1 || NCB == 2 || NCB == 4 || NCB == 8, "column blocks per workgroup");
  static_assert(!PAIRED || NCB >= 2, "paired epilogues take whole pairs");
  constexpr int KW = NW / NCB;                                               // K runs per column block
  constexpr int NT = NW * 64;
  constexpr int ROWS = 16 * MB;
  constexpr int NP = NT / 64;                   // parts per row in the sum-of-squares reduction
  constexpr int UM = kWsnMaxTiles / NP;
  static_assert(NW % NCB == 0 && kWsnMaxTiles % NP == 0, "wave split");
  __shared__ __attribute__((aligned(16))) float red[NW][ROWS * 16];
  __shared__ float rpart[NP][64];
  __shared__ float inv[64];
  const int unit = blockIdx.x;
  const int r0 = blockIdx.y * ROWS;   // first row of this workgroup's group of ROWS rows
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int cbw = wave % NCB, kw = wave / NCB;
  const int cb = unit * NCB + cbw;
  const int nst_all = a.K / 64, base = nst_all / KW, rem = nst_all % KW;
  const int s_lo = kw * base + min(kw, rem), nst = base + (kw < rem ? 1 : 0);
  const uint4* wbase = a.wf + (static_cast<size_t>(cb) * nst_all + s_lo) * 128 + lane;
  const size_t xblk = static_cast<size_t>(nst_all) * 128;   // pieces per 16-row block of X
  const uint4* xbase = a.xf + (r0 / 16) * xblk + static_cast<size_t>(s_lo) * 128 + lane;
  uint4 wb[NSR][2], xr[NSR][MB][2];
  auto load_stage = [&](int r, int s) {
    const uint4* q = wbase + static_cast<size_t>(s) * 128;
    wb[r][0] = q[0];
    wb[r][1] = q[64];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const uint4* p = xbase + i * xblk + static_cast<size_t>(s) * 128;
      xr[r][i][0] = p[0];
      xr[r][i][1] = p[64];
    }
  };
#pragma unroll
  for (int r = 0; r < NSR; ++r)
    if (r < nst) load_stage(r, r);
  // the norm's row sums of squares: thread t adds blocks t / 64, t / 64 + NP, ... of row t % 64
  float ssv[scales_rows(EPI) ? UM : 1];
  const int srow = tid % 64, spart = tid / 64;
  if constexpr (scales_rows(EPI)) {
#pragma unroll
    for (int u = 0; u < UM; ++u)
      ssv[u] = a.ssp[static_cast<size_t>(min(spart + NP * u, a.nt_in - 1)) * a.ld_ss + r0 + min(srow, ROWS - 1)];
  }
  f32x4_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nst; s0 += NSR) {
#pragma unroll
    for (int r = 0; r < NSR; ++r) {
      if (s0 + r < nst) {   // uniform
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < MB; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xr[r][i][h]),
                                                             __builtin_bit_cast(bf16x8_t, wb[r][h]), acc[i], 0, 0, 0);
        if (s0 + r + NSR < nst) load_stage(r, s0 + r + NSR);
      }
    }
  }
  // partial tiles of the K runs into LDS: lane holds rows 16 i + 4 (lane / 16) + v of column lane % 16
  float* mine = red[kw * NCB + cbw];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) mine[(16 * i + 4 * (lane / 16) + v) * 16 + lane % 16] = acc[i][v];
  if constexpr (scales_rows(EPI)) {
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < UM; ++u) ss += spart + NP * u < a.nt_in ? ssv[u] : 0.f;
    rpart[spart][srow] = ss;
  }
  __syncthreads();
  if constexpr (scales_rows(EPI)) {
    if (tid < ROWS) {
      float tot = rpart[0][tid];
#pragma unroll
      for (int p = 1; p < NP; ++p) tot += rpart[p][tid];
      inv[tid] = 1.0f / sqrtf(tot / static_cast<float>(a.K) + a.eps);
    }
    __syncthreads();
  }
  // epilogue: output o = (block b, row, column c of the block); 16 lanes hold the 16 columns of
  // one row.  A pair yields one output block (the pair's index), independent blocks one each.
  constexpr int NOB = PAIRED ? NCB / 2 : NCB;   // output blocks per workgroup
#pragma unroll
  for (int j = 0; j < (NOB * ROWS * 16 + NT - 1) / NT; ++j) {
    const int ob = tid + NT * j;
    if (ob >= NOB * ROWS * 16) break;   // uniform per wave (ROWS * 16 is a multiple of 64)
    const int b = ob / (ROWS * 16), o = ob % (ROWS * 16);
    const int lrow = o / 16, c = o % 16, row = r0 + lrow;
    const int blk = unit * NOB + b, oc = blk * 16 + c;
    const int c0 = PAIRED ? 2 * b : b;   // this output's (first) column block in the workgroup
    float v0 = red[c0][o];
#pragma unroll
    for (int k = 1; k < KW; ++k) v0 += red[k * NCB + c0][o];
    float v1 = 0.f;
    if constexpr (PAIRED) {
      v1 = red[c0 + 1][o];
#pragma unroll
      for (int k = 1; k < KW; ++k) v1 += red[k * NCB + c0 + 1][o];
    }
    const bool ok = row < a.M;
    if constexpr (scales_rows(EPI)) {
      v0 *= inv[lrow];
      v1 *= inv[lrow];
    }
    if constexpr (EPI == WEPI_F32) {
      if (ok) a.outf[static_cast<size_t>(row) * a.ldo + oc] = v0;
    } else if constexpr (EPI == WEPI_GELU) {
      if (ok) a.outb[act_offset(row, oc, a.ldo, 1)] = f32_to_bf16(gelu_erf(v0));
    } else if constexpr (EPI == WEPI_SWIGLU) {
      if (ok) a.outb[act_offset(row, oc, a.ldo, 1)] = f32_to_bf16(silu_f(v0) * v1);
    } else {   // WEPI_RESID / WEPI_MERGE: new residual row, its bf16 norm operand and the block's sums of squares
      float sq = 0.f;
      if (ok) {
        float y;
        if constexpr (EPI == WEPI_RESID) {
          y = a.outf[static_cast<size_t>(row) * a.ldo + oc] + v0;
        } else {
          const float et = bf16_to_f32(a.e[(static_cast<size_t>(row) * a.T + a.t) * a.D + oc]);
          const float gt = sigmoid_f(v0 + a.bias[oc]);
          y = gt * et + (1.0f - gt) * v1;
        }
        a.outf[static_cast<size_t>(row) * a.ldo + oc] = y;
        if (a.gain_next) a.xb_out[act_offset(row, oc, a.ldo, 1)] = f32_to_bf16(a.gain_next[oc] * y);
        sq = y * y;
      }
      sq = group_sum<16>(sq);
      if (c == 0) a.ssp_out[static_cast<size_t>(blk) * a.ld_ss + row] = sq;
    }
  }
}

// The merge's X = [e_t ; bf16(s_{t-1})] ([M][2D]) in the fragment-major layout, one 16-byte piece
// per thread; rows past M (up to the next multiple of 16) are written as zeros.
__global__ __launch_bounds__(256) void merge_x_k(const bf16_t* __restrict__ e, const float* __restrict__ s,
                                                 uint4* __restrict__ xf, int M, int T, int D, int t, int n_pieces) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n_pieces) return;
  const int K = 2 * D, lane = c % 64, h = (c / 64) % 2, q = c / 128, ks = q % (K / 64), i = q / (K / 64);
  const int row = 16 * i + lane % 16, k = 64 * ks + 16 * (lane / 16) + 8 * h;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < M) {
    if (k < D) {
      v = *reinterpret_cast<const uint4*>(e + (static_cast<size_t>(row) * T + t) * D + k);
    } else {
      const float4 lo = *reinterpret_cast<const float4*>(s + static_cast<size_t>(row) * D + (k - D));
      const float4 hi = *reinterpret_cast<const float4*>(s + static_cast<size_t>(row) * D + (k - D) + 4);
      v = make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w));
    }
  }
  xf[c] = v;
}

// s = g * y / rms(y) with the row sums of squares from per-block partials; also s_out[b][step].
__global__ __launch_bounds__(256) void final_norm_ssp_k(const float* __restrict__ y, const float* __restrict__ ssp,
                                                        int nt, int ld_ss, const float* __restrict__ gain, float* __restrict__ s,
                                                        float* __restrict__ s_out, int D, float eps, int step, int n) {
  const int b = blockIdx.x;
  __shared__ float inv_s;
  if (threadIdx.x < 64) {   // lane j adds blocks j, j + 64, ...; the lanes' sums in a fixed order
    float ss = 0.f;
    for (int j = threadIdx.x; j < nt; j += 64) ss += ssp[static_cast<size_t>(j) * ld_ss + b];
    ss = group_sum<64>(ss);
    if (threadIdx.x == 0) inv_s = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
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

// Register ring depth: every stage holds its W pair and MB X pairs (8 + 8 MB VGPRs); at 16 waves
// per workgroup a wave has 128 VGPRs, of which about 40 go to addresses, sums and accumulators.
template <int MB, int NW>
constexpr int wsn_ring() {
  constexpr int per_stage = 8 + MB * 8;
  constexpr int budget = 512 / (NW / 4 > 0 ? NW / 4 : 1) - 40;
  constexpr int r = (budget > 256 ? 256 : budget) / per_stage;
  return r >= 8 ? 8 : r >= 4 ? 4 : r >= 2 ? 2 : 1;
}

template <int MB, int EPI, int NCB>
hipError_t launch_wsn_t(const WstArgs& a, hipStream_t st) {
  constexpr int NW = 16;
  const dim3 grid(static_cast<unsigned>(a.N / (16 * NCB)), static_cast<unsigned>((a.M + 16 * MB - 1) / (16 * MB)));
  wsn_k<MB, EPI, NW, wsn_ring<MB, NW>(), NCB><<<grid, NW * 64, 0, st>>>(a);
  return hipGetLastError();
}

template <int EPI, int NCB>
hipError_t launch_wsn_mb(const WstArgs& a, hipStream_t st) {
  // 16-row blocks per row group: enough for all rows up to 64; a product whose grid would leave
  // half the CUs without a weight stream of their own takes groups of half the rows when the
  // doubled grid still fits one round of the chip (the groups of one column block are adjacent
  // in dispatch order modulo the XCD count when N/(16 NCB) is a multiple of 8, so they share its
  // weight stream through one L2)
  int mb = a.M <= 16 ? 1 : a.M <= 32 ? 2 : 4;
  const int units = a.N / (16 * NCB);
  if (a.M <= 64 && mb > 1 && 2 * units * ((a.M + 16 * mb - 1) / (16 * mb)) <= 256) mb /= 2;
  if (mb == 1) return launch_wsn_t<1, EPI, NCB>(a, st);
  if (mb == 2) return launch_wsn_t<2, EPI, NCB>(a, st);
  return launch_wsn_t<4, EPI, NCB>(a, st);
}

template <int EPI>
hipError_t launch_wsn_nw(const WstArgs& a, hipStream_t st) {
  // 16 waves per workgroup (measured on the step's shapes).  Up to 64 rows: two independent
  // column blocks per workgroup once the single-block grid would take more than one round of the
  // chip's CUs, one or two pairs for the paired epilogues.  Past 64 rows every row group re-reads X per
  // workgroup, so a workgroup takes more columns: two independent blocks, or the most pairs
  // (up to four) that still leave at least 256 workgroups.
  const int groups = (a.M + 63) / 64, nb = a.N / 16;
  if constexpr (EPI == WEPI_SWIGLU || EPI == WEPI_MERGE) {
    if (groups > 1 && nb % 8 == 0 && nb / 8 * groups >= 256) return launch_wsn_mb<EPI, 8>(a, st);
    if (groups > 1 && nb % 4 == 0 && nb / 4 * groups >= 256) return launch_wsn_mb<EPI, 4>(a, st);
    // up to 64 rows: two pairs per workgroup when one pair per workgroup would take more than
    // one round of the CUs and two take at most one (the reference model's FFN input)
    if (groups == 1 && nb % 4 == 0 && nb / 2 > 256 && nb / 4 <= 256) return launch_wsn_mb<EPI, 4>(a, st);
    return launch_wsn_mb<EPI, 2>(a, st);
  } else {
    return nb * groups >= 384 ? launch_wsn_mb<EPI, 2>(a, st) : launch_wsn_mb<EPI, 1>(a, st);
  }
}

}  // namespace

bool wsn_supported(int M, int N, int K) {
  return M >= 1 && M <= kWsnMaxRows && N % 32 == 0 && K % 64 == 0;
}

hipError_t launch_wsn(const WstArgs& a, hipStream_t st) {
  if (!wsn_supported(a.M, a.N, a.K) || !a.wf || !a.xf || a.ld_ss < 64 || a.ld_ss % 64 != 0 ||
      a.ld_ss < (a.M + 63) / 64 * 64)   // (operands are padded to whole 64-row groups)
    return hipErrorInvalidValue;
  const bool scale = scales_rows(a.epi);
  if ((scale && (!a.ssp || a.nt_in < 1 || a.nt_in > kWsnMaxTiles)) ||
      (a.epi == WEPI_F32 && !a.outf) || ((a.epi == WEPI_GELU || a.epi == WEPI_SWIGLU) && !a.outb) ||
      (a.epi == WEPI_RESID && (!a.outf || !a.ssp_out || (a.gain_next && !a.xb_out) || a.N / 16 > kWsnMaxTiles)) ||
      (a.epi == WEPI_MERGE && (!a.outf || !a.ssp_out || !a.bias || !a.e || !a.gain_next || !a.xb_out ||
                               a.N / 32 > kWsnMaxTiles || a.N != 2 * a.D)))
    return hipErrorInvalidValue;
  switch (a.epi) {
    case WEPI_F32: return launch_wsn_nw<WEPI_F32>(a, st);
    case WEPI_GELU: return launch_wsn_nw<WEPI_GELU>(a, st);
    case WEPI_SWIGLU: return launch_wsn_nw<WEPI_SWIGLU>(a, st);
    case WEPI_RESID: return launch_wsn_nw<WEPI_RESID>(a, st);
    case WEPI_MERGE: return launch_wsn_nw<WEPI_MERGE>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge_x(const uint16_t* e, const float* s, void* xf, int M, int Mp, int T, int D, int t,
                          hipStream_t st) {
  if (M < 1 || Mp < M || Mp % 16 != 0 || D % 64 != 0) return hipErrorInvalidValue;
  const int n = Mp / 16 * (2 * D / 64) * 128;
  merge_x_k<<<(n + 255) / 256, 256, 0, st>>>(e, s, static_cast<uint4*>(xf), M, T, D, t, n);
  return hipGetLastError();
}

hipError_t launch_final_norm_ssp(const float* y, const float* ssp, int nt, int ld_ss, const float* gain, float* s,
                                 float* s_out, int B, int D, float eps, int step, int n, hipStream_t st) {
  if (D % 4 != 0 || ld_ss < B) return hipErrorInvalidValue;
  final_norm_ssp_k<<<B, 256, 0, st>>>(y, ssp, nt, ld_ss, gain, s, s_out, D, eps, step, n);
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
