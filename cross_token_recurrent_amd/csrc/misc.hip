// Weight packing, embedding gather, row RMSNorm and layout conversions.
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {
namespace {

constexpr int kThreads = 256;

inline int grid_for(size_t n, int per_block = kThreads, int cap = 65536) {
  size_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > static_cast<size_t>(cap)) g = cap;
  return static_cast<int>(g);
}

template <typename T>
__global__ void pack_matrix_k(const float* __restrict__ src, T* __restrict__ dst, int rows, int cols, int ld,
                              int row_off, int col_off, int mode) {
  const size_t total = static_cast<size_t>(rows) * cols;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int r = static_cast<int>(i / cols), c = static_cast<int>(i % cols);
    const int dr = mode == 0 ? r + row_off : (r / 16) * 32 + row_off + r % 16;
    store_from_f32(&dst[static_cast<size_t>(dr) * ld + col_off + c], src[i]);
  }
}

__global__ void copy_f32_k(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

__global__ void broadcast_rows_k(const float* __restrict__ src, float* __restrict__ dst, int rows, int cols) {
  const size_t total = static_cast<size_t>(rows) * cols;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = src[i % cols];
}

__global__ void zero_k(uint32_t* __restrict__ dst, size_t n_words) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n_words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = 0u;
}

// One wave per row; D is a multiple of 64.
template <typename T>
__global__ void embed_k(const int32_t* __restrict__ tokens, int n, int rows, const T* __restrict__ E, int V,
                        int D, float* __restrict__ x, int32_t* __restrict__ flags) {
  const int row = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= rows) return;
  int tok = tokens[row];  // tokens are [Bc, n] contiguous, same order as rows
  if (tok < 0 || tok >= V) {
    if (lane == 0) atomicOr(flags, 1);
    tok = 0;
  }
  const T* src = E + static_cast<size_t>(tok) * D;
  float* dst = x + static_cast<size_t>(row) * D;
  for (int c = lane; c < D; c += 64) dst[c] = load_as_f32(src + c);
  (void)n;
}

// One wave per row.
template <typename T>
__global__ void rmsnorm_rows_k(const float* __restrict__ x, const float* __restrict__ gain, T* __restrict__ out,
                               int rows, int D, float eps, T* __restrict__ e_store, int n, int b0, int t0,
                               int Tmax) {
  const int row = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= rows) return;
  const float* xr = x + static_cast<size_t>(row) * D;
  float ss = 0.f;
  for (int c = lane; c < D; c += 64) ss += xr[c] * xr[c];
  ss = group_sum<64>(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  T* o = out + static_cast<size_t>(row) * D;
  T* es = nullptr;
  if (e_store) {
    const int b = b0 + row / n, t = t0 + row % n;
    es = e_store + (static_cast<size_t>(b) * Tmax + t) * D;
  }
  for (int c = lane; c < D; c += 64) {
    const float v = gain[c] * (xr[c] * inv);
    store_from_f32(o + c, v);
    if (es) store_from_f32(es + c, v);
  }
}

// The same for D = 256 * NV: each lane keeps its NV float4 of the row in registers (one read
// of x, every load in flight at once) and writes 4 elements per store.
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

template <typename T, int NV>
__global__ __launch_bounds__(256) void rmsnorm_rows_v_k(const float* __restrict__ x, const float* __restrict__ gain,
                                                        T* __restrict__ out, int rows, float eps,
                                                        T* __restrict__ e_store, int n, int b0, int t0, int Tmax) {
  constexpr int D = 256 * NV;
  const int row = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= rows) return;
  const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(row) * D);
  float4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = xr[lane + 64 * i];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  ss = group_sum<64>(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  T* o = out + static_cast<size_t>(row) * D;
  T* es = nullptr;
  if (e_store) {
    const int b = b0 + row / n, t = t0 + row % n;
    es = e_store + (static_cast<size_t>(b) * Tmax + t) * D;
  }
  const float4* g4 = reinterpret_cast<const float4*>(gain);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c4 = lane + 64 * i;
    const float4 g = g4[c4];
    const float a = g.x * (v[i].x * inv), b = g.y * (v[i].y * inv), c = g.z * (v[i].z * inv),
                d = g.w * (v[i].w * inv);
    store4<T>(o + 4 * c4, a, b, c, d);
    if (es) store4<T>(es + 4 * c4, a, b, c, d);
  }
}

// The same for D = 64 and 128: D/4 lanes per row (4 or 2 rows per wave), one float4 each.
// Rows past the end are read clamped so that every lane of a group joins the sum.
template <typename T, int D>
__global__ __launch_bounds__(256) void rmsnorm_rows_s_k(const float* __restrict__ x, const float* __restrict__ gain,
                                                        T* __restrict__ out, int rows, float eps,
                                                        T* __restrict__ e_store, int n, int b0, int t0, int Tmax) {
  constexpr int G = D / 4;
  constexpr int RPW = 64 / G;
  const int row = (blockIdx.x * 4 + static_cast<int>(threadIdx.x) / 64) * RPW + (threadIdx.x % 64) / G;
  const int l = threadIdx.x % G;
  const int r = min(row, rows - 1);
  const float4 v = reinterpret_cast<const float4*>(x + static_cast<size_t>(r) * D)[l];
  float ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  ss = group_sum<G>(ss);
  if (row >= rows) return;
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  const float4 g = reinterpret_cast<const float4*>(gain)[l];
  const float a = g.x * (v.x * inv), b = g.y * (v.y * inv), c = g.z * (v.z * inv), d = g.w * (v.w * inv);
  store4<T>(out + static_cast<size_t>(row) * D + 4 * l, a, b, c, d);
  if (e_store) {
    const int bb = b0 + row / n, t = t0 + row % n;
    store4<T>(e_store + (static_cast<size_t>(bb) * Tmax + t) * D + 4 * l, a, b, c, d);
  }
}

// fp32 [B, n, D] <-> stored layout.  heads_layout 0: [B][T][D]; 1: [B][H][T][dh].
template <typename T>
__global__ void store_tokens_k(float* __restrict__ flat, T* __restrict__ dev, int B, int n, int D, int t0, int Tmax,
                               int heads_layout, int H, int dh, int to_device) {
  const size_t total = static_cast<size_t>(B) * n * D;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int c = static_cast<int>(i % D);
    const size_t bj = i / D;
    const int j = static_cast<int>(bj % n), b = static_cast<int>(bj / n);
    size_t di;
    if (heads_layout == 2) {
      // key-blocked values: [B][H][T8/8][dh][8]
      const int h = c / dh, cc = c % dh, t = t0 + j;
      const size_t nblk = static_cast<size_t>(Tmax + 7) / 8;
      di = (((static_cast<size_t>(b) * H + h) * nblk + t / 8) * dh + cc) * 8 + t % 8;
    } else if (heads_layout == 1) {
      const int h = c / dh, cc = c % dh;
      di = ((static_cast<size_t>(b) * H + h) * Tmax + t0 + j) * dh + cc;
    } else {
      di = (static_cast<size_t>(b) * Tmax + t0 + j) * D + c;
    }
    if (to_device)
      store_from_f32(dev + di, flat[i]);
    else
      flat[i] = load_as_f32(dev + di);
  }
  (void)H;
}

}  // namespace

hipError_t launch_pack_matrix(const float* src, void* dst, int rows, int cols, int ld, int row_off, int col_off,
                              int mode, int dtype, hipStream_t st) {
  const int g = grid_for(static_cast<size_t>(rows) * cols);
  if (dtype == RLT_DTYPE_BF16)
    pack_matrix_k<bf16_t><<<g, kThreads, 0, st>>>(src, static_cast<bf16_t*>(dst), rows, cols, ld, row_off, col_off,
                                                  mode);
  else
    pack_matrix_k<float><<<g, kThreads, 0, st>>>(src, static_cast<float*>(dst), rows, cols, ld, row_off, col_off,
                                                 mode);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t st) {
  copy_f32_k<<<grid_for(n), kThreads, 0, st>>>(src, dst, n);
  return hipGetLastError();
}

hipError_t launch_broadcast_rows(const float* src, float* dst, int rows, int cols, hipStream_t st) {
  broadcast_rows_k<<<grid_for(static_cast<size_t>(rows) * cols), kThreads, 0, st>>>(src, dst, rows, cols);
  return hipGetLastError();
}

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t st) {
  // All regions are 256-byte aligned and sized in whole 4-byte words.
  const size_t words = bytes / 4;
  zero_k<<<grid_for(words), kThreads, 0, st>>>(static_cast<uint32_t*>(dst), words);
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t* tokens, int n, int b0, int rows, const void* embed, int V, int D, int dtype,
                        float* x, int32_t* flags, hipStream_t st) {
  (void)b0;
  const int g = (rows + 3) / 4;
  if (dtype == RLT_DTYPE_BF16)
    embed_k<bf16_t><<<g, 256, 0, st>>>(tokens, n, rows, static_cast<const bf16_t*>(embed), V, D, x, flags);
  else
    embed_k<float><<<g, 256, 0, st>>>(tokens, n, rows, static_cast<const float*>(embed), V, D, x, flags);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rmsnorm_v(const float* x, const float* gain, T* out, int rows, int D, float eps, T* e_store, int n,
                            int b0, int t0, int Tmax, hipStream_t st) {
  const int g = (rows + 3) / 4;
  switch (D / 256) {
    case 1: rmsnorm_rows_v_k<T, 1><<<g, 256, 0, st>>>(x, gain, out, rows, eps, e_store, n, b0, t0, Tmax); break;
    case 2: rmsnorm_rows_v_k<T, 2><<<g, 256, 0, st>>>(x, gain, out, rows, eps, e_store, n, b0, t0, Tmax); break;
    case 4: rmsnorm_rows_v_k<T, 4><<<g, 256, 0, st>>>(x, gain, out, rows, eps, e_store, n, b0, t0, Tmax); break;
    default: rmsnorm_rows_v_k<T, 8><<<g, 256, 0, st>>>(x, gain, out, rows, eps, e_store, n, b0, t0, Tmax); break;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const float* x, const float* gain, void* out, int rows, int D, float eps, int dtype,
                               void* e_store, int n, int b0, int t0, int Tmax, hipStream_t st) {
  if (D == 256 || D == 512 || D == 1024 || D == 2048) {
    if (dtype == RLT_DTYPE_BF16)
      return launch_rmsnorm_v<bf16_t>(x, gain, static_cast<bf16_t*>(out), rows, D, eps, static_cast<bf16_t*>(e_store),
                                      n, b0, t0, Tmax, st);
    return launch_rmsnorm_v<float>(x, gain, static_cast<float*>(out), rows, D, eps, static_cast<float*>(e_store), n,
                                   b0, t0, Tmax, st);
  }
  if (D == 64 || D == 128) {
    const int per_block = 4 * (64 / (D / 4));   // rows per 256-thread block
    const int gs = (rows + per_block - 1) / per_block;
    if (dtype == RLT_DTYPE_BF16) {
      bf16_t* o = static_cast<bf16_t*>(out);
      bf16_t* es = static_cast<bf16_t*>(e_store);
      if (D == 64) rmsnorm_rows_s_k<bf16_t, 64><<<gs, 256, 0, st>>>(x, gain, o, rows, eps, es, n, b0, t0, Tmax);
      else rmsnorm_rows_s_k<bf16_t, 128><<<gs, 256, 0, st>>>(x, gain, o, rows, eps, es, n, b0, t0, Tmax);
    } else {
      float* o = static_cast<float*>(out);
      float* es = static_cast<float*>(e_store);
      if (D == 64) rmsnorm_rows_s_k<float, 64><<<gs, 256, 0, st>>>(x, gain, o, rows, eps, es, n, b0, t0, Tmax);
      else rmsnorm_rows_s_k<float, 128><<<gs, 256, 0, st>>>(x, gain, o, rows, eps, es, n, b0, t0, Tmax);
    }
    return hipGetLastError();
  }
  const int g = (rows + 3) / 4;
  if (dtype == RLT_DTYPE_BF16)
    rmsnorm_rows_k<bf16_t><<<g, 256, 0, st>>>(x, gain, static_cast<bf16_t*>(out), rows, D, eps,
                                              static_cast<bf16_t*>(e_store), n, b0, t0, Tmax);
  else
    rmsnorm_rows_k<float><<<g, 256, 0, st>>>(x, gain, static_cast<float*>(out), rows, D, eps,
                                             static_cast<float*>(e_store), n, b0, t0, Tmax);
  return hipGetLastError();
}

hipError_t launch_store_tokens(const float* src, void* dst, int B, int n, int D, int t0, int Tmax, int dtype,
                               int heads_layout, int H, int dh, int to_device_layout, hipStream_t st) {
  const int g = grid_for(static_cast<size_t>(B) * n * D);
  float* flat = const_cast<float*>(src);
  if (dtype == RLT_DTYPE_BF16)
    store_tokens_k<bf16_t><<<g, kThreads, 0, st>>>(flat, static_cast<bf16_t*>(dst), B, n, D, t0, Tmax, heads_layout,
                                                   H, dh, to_device_layout);
  else
    store_tokens_k<float><<<g, kThreads, 0, st>>>(flat, static_cast<float*>(dst), B, n, D, t0, Tmax, heads_layout, H,
                                                  dh, to_device_layout);
  return hipGetLastError();
}

}  // namespace rlt
