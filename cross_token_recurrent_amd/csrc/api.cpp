// Host runtime of librlt: configuration checks, packed-weight and state layouts,
// state counters and versioning, and the launch sequences of the three hot-path calls.
//
// Pages: [FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer";
//        [DS] deepsonar "技术拆解 009｜RLT：给 Transformer 接一条时间回路…".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "rlt_internal.h"

using namespace rlt;

struct rlt_model {
  rlt_config cfg;
  ModelLayout lay;
  int path;  // RLT_PATH_*
  uint64_t version;
  char* ws;
  size_t ws_bytes;
};

struct rlt_state {
  rlt_config cfg;
  StateLayout lay;
  uint64_t version;
  int t_enc, t_dec;
  char* buf;
  size_t bytes;
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  g_err = std::string(where) + ": " + hipGetErrorString(e);
  return RLT_ERR_HIP;
}

#define RLT_HIP(call, where)                    \
  do {                                          \
    hipError_t _e = (call);                     \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_config(const rlt_config* c) {
  if (!c) return fail(RLT_ERR_INVALID, "config is NULL");
  if (c->vocab < 1 || c->d_model < 1 || c->n_heads < 1 || c->n_layers < 1 || c->ffn_dim < 1)
    return fail(RLT_ERR_INVALID, "vocab, d_model, n_heads, n_layers and ffn_dim must be >= 1");
  if (c->window < 1) return fail(RLT_ERR_INVALID, "window must be >= 1 (it counts the current token)");
  if (c->ffn_kind != RLT_FFN_GELU && c->ffn_kind != RLT_FFN_SWIGLU)
    return fail(RLT_ERR_INVALID, "ffn_kind must be RLT_FFN_GELU or RLT_FFN_SWIGLU");
  if (c->dtype != RLT_DTYPE_FP32 && c->dtype != RLT_DTYPE_BF16)
    return fail(RLT_ERR_INVALID, "dtype must be RLT_DTYPE_FP32 or RLT_DTYPE_BF16");
  if (!(c->norm_eps > 0.0f)) return fail(RLT_ERR_INVALID, "norm_eps must be > 0");
  if (c->d_model % c->n_heads != 0) return fail(RLT_ERR_UNSUPPORTED, "d_model must be a multiple of n_heads");
  if (c->mem_groups != 1 && c->mem_groups != c->n_layers)
    return fail(RLT_ERR_UNSUPPORTED, "mem_groups must be 1 or n_layers");
  const int dh = c->d_model / c->n_heads;
  if (dh != 16 && dh != 32 && dh != 64 && dh != 128)
    return fail(RLT_ERR_UNSUPPORTED, "head_dim must be 16, 32, 64 or 128");
  if (c->d_model % 64 != 0 || c->ffn_dim % 64 != 0)
    return fail(RLT_ERR_UNSUPPORTED, "d_model and ffn_dim must be multiples of 64");
  return RLT_OK;
}

struct ParamDesc {
  const char* name;
  int64_t numel;
};

std::vector<ParamDesc> param_table(const rlt_config& c) {
  const int64_t V = c.vocab, d = c.d_model, L = c.n_layers, F = c.ffn_dim, G = c.mem_groups;
  std::vector<ParamDesc> t = {
      {"embed", V * d}, {"w_out", V * d}, {"s_star", d}, {"w_ge", d * d}, {"w_gs", d * d},
      {"w_fb", d * d},  {"b_g", d},       {"wq", L * d * d}, {"wk", L * d * d}, {"wv", L * d * d},
      {"wo", L * d * d}};
  if (c.ffn_kind == RLT_FFN_GELU) {
    t.push_back({"ffn_w1", L * F * d});
    t.push_back({"ffn_w2", L * d * F});
  } else {
    t.push_back({"ffn_gate", L * F * d});
    t.push_back({"ffn_up", L * F * d});
    t.push_back({"ffn_down", L * d * F});
  }
  const ParamDesc rest[] = {{"wqx", L * d * d},   {"wox", L * d * d},   {"wkm", G * d * d},
                            {"wvm", G * d * d},   {"g_enc_attn", L * d}, {"g_enc_ffn", L * d},
                            {"g_enc_final", d},   {"g_dec_self", L * d}, {"g_dec_cross", L * d},
                            {"g_dec_ffn", L * d}, {"g_dec_final", d}};
  for (const auto& r : rest) t.push_back(r);
  return t;
}

int64_t param_offset(const rlt_config& c, const char* name, int64_t* numel) {
  int64_t off = 0;
  for (const auto& p : param_table(c)) {
    if (std::strcmp(p.name, name) == 0) {
      if (numel) *numel = p.numel;
      return off;
    }
    off += p.numel;
  }
  return -1;
}

// Packs the canonical fp32 buffer into the workspace layout (enqueued on `st`).
int pack_weights(const rlt_model& m, const float* w, hipStream_t st) {
  const rlt_config& c = m.cfg;
  const ModelLayout& L = m.lay;
  const int D = L.D, F = L.F, dt = L.dtype;
  char* ws = m.ws;
  auto src = [&](const char* name) { return w + param_offset(c, name, nullptr); };
  auto mat = [&](const float* s, size_t dst, int rows, int cols, int ld, int row_off, int col_off,
                 int mode) -> int {
    RLT_HIP(launch_pack_matrix(s, ws + dst, rows, cols, ld, row_off, col_off, mode, dt, st), "pack");
    return RLT_OK;
  };
  auto f32 = [&](const float* s, size_t dst, size_t n) -> int {
    RLT_HIP(launch_copy_f32(s, reinterpret_cast<float*>(ws + dst), n, st), "pack gains");
    return RLT_OK;
  };
  int rc;
#define TRY(x) \
  if ((rc = (x)) != RLT_OK) return rc
  TRY(mat(src("embed"), L.embed, L.V, D, D, 0, 0, 0));
  TRY(mat(src("w_out"), L.wout, L.V, D, D, 0, 0, 0));
  TRY(f32(src("s_star"), L.sstar, D));
  TRY(mat(src("w_ge"), L.wgate, D, D, 2 * D, 0, 0, 0));
  TRY(mat(src("w_gs"), L.wgate, D, D, 2 * D, 0, D, 0));
  TRY(mat(src("w_fb"), L.wfb, D, D, D, 0, 0, 0));
  TRY(f32(src("b_g"), L.bg, D));
  const size_t dd = static_cast<size_t>(D) * D, fd = static_cast<size_t>(F) * D;
  for (int l = 0; l < L.L; ++l) {
    const size_t base = L.layers + l * L.layer_stride;
    TRY(mat(src("wq") + l * dd, base + L.l_qkv, D, D, D, 0, 0, 0));
    TRY(mat(src("wk") + l * dd, base + L.l_qkv, D, D, D, D, 0, 0));
    TRY(mat(src("wv") + l * dd, base + L.l_qkv, D, D, D, 2 * D, 0, 0));
    TRY(mat(src("wo") + l * dd, base + L.l_wo, D, D, D, 0, 0, 0));
    TRY(mat(src("wqx") + l * dd, base + L.l_wqx, D, D, D, 0, 0, 0));
    TRY(mat(src("wox") + l * dd, base + L.l_wox, D, D, D, 0, 0, 0));
    if (L.ffn_kind == RLT_FFN_GELU) {
      TRY(mat(src("ffn_w1") + l * fd, base + L.l_fin, F, D, D, 0, 0, 0));
      TRY(mat(src("ffn_w2") + l * fd, base + L.l_fout, D, F, F, 0, 0, 0));
    } else {
      TRY(mat(src("ffn_gate") + l * fd, base + L.l_fin, F, D, D, 0, 0, 1));
      TRY(mat(src("ffn_up") + l * fd, base + L.l_fin, F, D, D, 16, 0, 1));
      TRY(mat(src("ffn_down") + l * fd, base + L.l_fout, D, F, F, 0, 0, 0));
    }
  }
  for (int g = 0; g < L.G; ++g) {
    const size_t base = L.wkvm + g * L.group_stride;
    TRY(mat(src("wkm") + g * dd, base, D, D, D, 0, 0, 0));
    TRY(mat(src("wvm") + g * dd, base, D, D, D, D, 0, 0));
  }
  TRY(f32(src("g_enc_attn"), L.g_enc_attn, static_cast<size_t>(L.L) * D));
  TRY(f32(src("g_enc_ffn"), L.g_enc_ffn, static_cast<size_t>(L.L) * D));
  TRY(f32(src("g_enc_final"), L.g_enc_final, D));
  TRY(f32(src("g_dec_self"), L.g_dec_self, static_cast<size_t>(L.L) * D));
  TRY(f32(src("g_dec_cross"), L.g_dec_cross, static_cast<size_t>(L.L) * D));
  TRY(f32(src("g_dec_ffn"), L.g_dec_ffn, static_cast<size_t>(L.L) * D));
  TRY(f32(src("g_dec_final"), L.g_dec_final, D));
  if (L.has_wout_frag) RLT_HIP(launch_pack_score_head(src("w_out"), ws + L.wout_frag, L.V, D, st), "pack head fragments");
  if (L.has_frag) {
    auto frag = [&](size_t from, size_t to, int N, int K) -> int {
      RLT_HIP(launch_pack_frag(ws + from, ws + to, N, K, st), "pack weight fragments");
      return RLT_OK;
    };
    RLT_HIP(launch_pack_merge_frag(src("w_ge"), src("w_gs"), src("w_fb"), ws + L.frag_merge, D, st),
            "pack merge fragments");
    for (int l = 0; l < L.L; ++l) {
      const size_t src_l = L.layers + l * L.layer_stride, dst_l = L.frag_layers + l * L.layer_stride;
      TRY(frag(src_l + L.l_qkv, dst_l + L.l_qkv, 3 * D, D));
      TRY(frag(src_l + L.l_wo, dst_l + L.l_wo, D, D));
      TRY(frag(src_l + L.l_wqx, dst_l + L.l_wqx, D, D));
      TRY(frag(src_l + L.l_wox, dst_l + L.l_wox, D, D));
      TRY(frag(src_l + L.l_fin, dst_l + L.l_fin, L.F2, D));
      TRY(frag(src_l + L.l_fout, dst_l + L.l_fout, D, F));
    }
  }
#undef TRY
  return RLT_OK;
}

int check_pair(const rlt_model* m, const rlt_state* s) {
  if (!m || !s) return fail(RLT_ERR_INVALID, "model or state is NULL");
  if (std::memcmp(&m->cfg, &s->cfg, sizeof(rlt_config)) != 0)
    return fail(RLT_ERR_INVALID, "state was built for a different model configuration");
  if (m->version != s->version)
    return fail(RLT_ERR_STALE_STATE,
                "state was built under weights version " + std::to_string(s->version) +
                    " but the model is at version " + std::to_string(m->version) +
                    "; reset the state and replay from the sequence start");
  return RLT_OK;
}

int reset_state(const rlt_model* m, rlt_state* s, hipStream_t st) {
  const StateLayout& S = s->lay;
  RLT_HIP(launch_zero(s->buf + S.flags, 256, st), "reset flags");
  RLT_HIP(launch_broadcast_rows(reinterpret_cast<const float*>(m->ws + m->lay.sstar),
                                reinterpret_cast<float*>(s->buf + S.s), S.B, m->lay.D, st),
          "reset s");
  if (S.ring_v > S.ring_k) {
    RLT_HIP(launch_zero(s->buf + S.ring_k, S.e - S.ring_k, st), "reset window caches");
  }
  size_t cnt_off = 0, cnt_bytes = 0;
  dec_batched_counters(m->lay, S.B, S.T, &cnt_off, &cnt_bytes);
  if (cnt_bytes) RLT_HIP(launch_zero(s->buf + S.dec_scratch + cnt_off, cnt_bytes, st), "reset decoder counters");
  s->version = m->version;
  s->t_enc = 0;
  s->t_dec = 0;
  return RLT_OK;
}

}  // namespace

namespace rlt {

bool compute_model_layout(const rlt_config& c, ModelLayout* m) {
  ModelLayout& L = *m;
  L.D = c.d_model;
  L.H = c.n_heads;
  L.DH = c.d_model / c.n_heads;
  L.L = c.n_layers;
  L.F = c.ffn_dim;
  L.F2 = c.ffn_kind == RLT_FFN_SWIGLU ? 2 * c.ffn_dim : c.ffn_dim;
  L.V = c.vocab;
  L.W = c.window;
  L.G = c.mem_groups;
  L.ffn_kind = c.ffn_kind;
  L.dtype = c.dtype;
  L.eps = c.norm_eps;
  L.esz = c.dtype == RLT_DTYPE_BF16 ? 2 : 4;
  const size_t D = L.D, V = L.V, F = L.F, F2 = L.F2, e = L.esz;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.embed = take(V * D * e);
  L.wout = take(V * D * e);
  L.sstar = take(D * 4);
  L.wgate = take(2 * D * D * e);
  L.wfb = take(D * D * e);
  L.bg = take(D * 4);
  size_t rel = 0;
  auto take_rel = [&](size_t bytes) {
    size_t o = rel;
    rel = align_up(rel + bytes);
    return o;
  };
  L.l_qkv = take_rel(3 * D * D * e);
  L.l_wo = take_rel(D * D * e);
  L.l_wqx = take_rel(D * D * e);
  L.l_wox = take_rel(D * D * e);
  L.l_fin = take_rel(F2 * D * e);
  L.l_fout = take_rel(D * F * e);
  L.layer_stride = rel;
  L.layers = take(L.L * L.layer_stride);
  L.group_stride = align_up(2 * D * D * e);
  L.wkvm = take(L.G * L.group_stride);
  L.gains = off;
  L.g_enc_attn = take(L.L * D * 4);
  L.g_enc_ffn = take(L.L * D * 4);
  L.g_enc_final = take(D * 4);
  L.g_dec_self = take(L.L * D * 4);
  L.g_dec_cross = take(L.L * D * 4);
  L.g_dec_ffn = take(L.L * D * 4);
  L.g_dec_final = take(D * 4);
  L.has_frag = L.dtype == RLT_DTYPE_BF16 && L.D >= 256 ? 1 : 0;
  if (L.has_frag) {
    L.frag_layers = take(L.L * L.layer_stride);
    L.frag_merge = take(4 * D * D * e);
  } else {
    L.frag_layers = L.frag_merge = 0;
  }
  L.has_wout_frag = score_frag_eligible(L.dtype, L.D) ? 1 : 0;
  L.wout_frag = L.has_wout_frag ? take((V + 15) / 16 * 16 * D * 2) : 0;
  L.total = off;
  return true;
}

void compute_state_layout(const ModelLayout& m, int B, int T, int keep, StateLayout* s) {
  StateLayout& S = *s;
  S.B = B;
  S.T = T;
  S.T8 = (T + 7) / 8 * 8;
  S.keep = keep;
  S.Wm1 = m.W - 1;
  const size_t D = m.D, e = m.esz, Bz = B, Tz = T, L = m.L, G = m.G, F = m.F;
  const size_t heads_tokens = static_cast<size_t>(m.H) * m.DH;  // = D
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  S.flags = take(256);
  S.s = take(Bz * D * 4);
  S.ring_k = take(L * Bz * S.Wm1 * heads_tokens * e);
  S.ring_v = take(L * Bz * S.Wm1 * heads_tokens * e);
  S.e = take(Bz * Tz * D * e);
  S.mem_k = take(G * Bz * Tz * D * e);
  S.mem_v = take(G * Bz * static_cast<size_t>(S.T8) * D * e);
  if (keep) {
    S.enc_k = take(L * Bz * Tz * D * e);
    S.enc_v = take(L * Bz * Tz * D * e);
  } else {
    S.enc_k = S.enc_v = 0;
  }
  const size_t budget = 65536;
  size_t nc = std::min(Bz * Tz, budget);
  nc = std::max(nc, std::max(Tz, Bz));
  S.Nc = static_cast<int>(nc);
  S.x = take(nc * D * 4);
  S.h = take(nc * D * e);
  S.qkv = take(nc * 3 * D * e);
  S.attn = take(nc * D * e);
  S.act = take(nc * F * e);
  S.dec_scratch_bytes = dec_batched_scratch_bytes(m, B, T);
  S.dec_scratch = take(S.dec_scratch_bytes);
  S.total = off;
}

}  // namespace rlt

namespace {

// Snapshot header (host byte order); the packed regions follow it.
struct SnapHeader {
  char magic[8];
  uint32_t header_bytes, format;
  rlt_config cfg;
  uint64_t version;
  int32_t batch, t_enc, t_dec, keep;
  int32_t window_convention;  // 1: window counts the current token, ring slot = p mod (W-1)
  int32_t reserved;
  uint64_t payload_bytes;
};
constexpr char kSnapMagic[8] = {'R', 'L', 'T', 'S', 'N', 'A', 'P', '1'};

// One packed region: `height` rows of `width` bytes; rows are `pitch` bytes apart in the state
// blob and contiguous in the snapshot.
struct SnapRegion {
  size_t off, width, height, pitch;
};

// The regions of a state with layout S at t positions (t <= S.T); `keep` selects the encoder cache.
std::vector<SnapRegion> snap_regions(const ModelLayout& M, const StateLayout& S, int t, int keep) {
  const size_t e = M.esz, D = M.D, dh = M.DH, B = S.B, L = M.L, G = M.G, H = M.H, T = S.T;
  const size_t ring = L * B * static_cast<size_t>(S.Wm1) * D * e;
  const size_t t8 = (static_cast<size_t>(t) + 7) / 8 * 8;
  std::vector<SnapRegion> r = {
      {S.flags, 256, 1, 256},
      {S.s, B * D * 4, 1, B * D * 4},
      {S.ring_k, ring, ring ? 1u : 0u, ring},
      {S.ring_v, ring, ring ? 1u : 0u, ring},
      {S.e, t * D * e, B, T * D * e},
      {S.mem_k, t * dh * e, G * B * H, T * dh * e},
      {S.mem_v, t8 * dh * e, G * B * H, static_cast<size_t>(S.T8) * dh * e},
  };
  if (keep) {
    r.push_back({S.enc_k, t * dh * e, L * B * H, T * dh * e});
    r.push_back({S.enc_v, t * dh * e, L * B * H, T * dh * e});
  }
  return r;
}

size_t snap_payload(const std::vector<SnapRegion>& r) {
  size_t n = 0;
  for (const auto& x : r) n += x.width * x.height;
  return n;
}

bool is_device_pointer(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // plain pageable host memory is not registered with HIP
    return false;
  }
  return attr.type == hipMemoryTypeDevice;
}

// Memory a kernel will read or write must be known to HIP (device, managed or pinned host
// memory).  Plain pageable host memory is not, and a kernel touching it would fault, so it is
// refused before anything is enqueued.  A NULL pointer passes: required arguments are checked
// for NULL separately.
int need_gpu_memory(const void* p, const char* what) {
  if (!p) return RLT_OK;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(RLT_ERR_INVALID, std::string(what) + " is not memory the GPU can access (plain host memory?)");
  }
  if (attr.type == hipMemoryTypeUnregistered)
    return fail(RLT_ERR_INVALID, std::string(what) + " is not memory the GPU can access (plain host memory?)");
  return RLT_OK;
}

// need_gpu_memory over a list of (pointer, name) pairs; the first failure is returned.
int need_gpu_memory(std::initializer_list<std::pair<const void*, const char*>> args) {
  for (const auto& a : args) {
    int rc = need_gpu_memory(a.first, a.second);
    if (rc) return rc;
  }
  return RLT_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Library-owned decoder scratch for rlt_decoder_replay_noalloc: one array per GPU, allocated
// with the code object when the library loads on that GPU and held until the process ends.  In
// host code the array's name is only a stand-in; its device address on each GPU comes from
// hipGetSymbolAddress with that GPU current, looked up once per device.
// ---------------------------------------------------------------------------------------------
namespace {

constexpr size_t kStaticScratchBytes = size_t(64) << 20;
__device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `device` (looked up once, with that device current).
int static_scratch(int device, char** out) {
  if (device < 0 || device >= kMaxDevices) return fail(RLT_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    RLT_HIP(hipGetDevice(&cur), "current device");
    if (cur != device) RLT_HIP(hipSetDevice(device), "select device");
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != device) RLT_HIP(hipSetDevice(cur), "restore device");
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    g_scratch_ptr[device] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[device]);
  return RLT_OK;
}

}  // namespace

extern "C" {

const char* rlt_last_error(void) { return g_err.c_str(); }
const char* rlt_version_string(void) { return "librlt 0.1 (gfx950)"; }

int rlt_param_count(const rlt_config* cfg, int32_t* n_tensors, int64_t* total_numel) {
  int rc = check_config(cfg);
  if (rc) return rc;
  auto t = param_table(*cfg);
  int64_t tot = 0;
  for (auto& p : t) tot += p.numel;
  if (n_tensors) *n_tensors = static_cast<int32_t>(t.size());
  if (total_numel) *total_numel = tot;
  return RLT_OK;
}

int rlt_param_info(const rlt_config* cfg, int32_t index, const char** name, int64_t* offset,
                   int64_t* numel) {
  int rc = check_config(cfg);
  if (rc) return rc;
  auto t = param_table(*cfg);
  if (index < 0 || index >= static_cast<int32_t>(t.size())) return fail(RLT_ERR_INVALID, "index out of range");
  int64_t off = 0;
  for (int i = 0; i < index; ++i) off += t[i].numel;
  if (name) *name = t[index].name;
  if (offset) *offset = off;
  if (numel) *numel = t[index].numel;
  return RLT_OK;
}

int rlt_model_workspace_bytes(const rlt_config* cfg, size_t* bytes) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(RLT_ERR_INVALID, "bytes is NULL");
  ModelLayout L;
  compute_model_layout(*cfg, &L);
  *bytes = L.total;
  return RLT_OK;
}

int rlt_model_create(const rlt_config* cfg, const float* weights, uint64_t version, void* workspace,
                     size_t workspace_bytes, void* stream, rlt_model** out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!weights || !workspace || !out) return fail(RLT_ERR_INVALID, "weights, workspace and out must be non-NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(RLT_ERR_INVALID, "workspace must be 256-byte aligned");
  ModelLayout L;
  compute_model_layout(*cfg, &L);
  if (workspace_bytes < L.total)
    return fail(RLT_ERR_INVALID, "workspace too small: need " + std::to_string(L.total) + " bytes");
  rc = need_gpu_memory({{weights, "weights"}, {workspace, "workspace"}});
  if (rc) return rc;
  rlt_model* m = new (std::nothrow) rlt_model;
  if (!m) return fail(RLT_ERR_INVALID, "out of host memory");
  m->cfg = *cfg;
  m->lay = L;
  m->path = RLT_PATH_AUTO;
  m->version = version;
  m->ws = static_cast<char*>(workspace);
  m->ws_bytes = workspace_bytes;
  rc = pack_weights(*m, weights, as_stream(stream));
  if (rc) {
    delete m;
    return rc;
  }
  *out = m;
  return RLT_OK;
}

int rlt_model_update_weights(rlt_model* model, const float* weights, uint64_t new_version, void* stream) {
  if (!model || !weights) return fail(RLT_ERR_INVALID, "model and weights must be non-NULL");
  if (new_version == model->version)
    return fail(RLT_ERR_INVALID, "a weight update must carry a new version");
  int rc = need_gpu_memory(weights, "weights");
  if (rc) return rc;
  rc = pack_weights(*model, weights, as_stream(stream));
  if (rc) return rc;
  model->version = new_version;
  return RLT_OK;
}

int rlt_model_get_config(const rlt_model* model, rlt_config* cfg, uint64_t* version) {
  if (!model) return fail(RLT_ERR_INVALID, "model is NULL");
  if (cfg) *cfg = model->cfg;
  if (version) *version = model->version;
  return RLT_OK;
}

void rlt_model_release(rlt_model* model) { delete model; }

int rlt_state_bytes(const rlt_model* model, int32_t batch, int32_t t_max, int32_t keep_encoder_cache,
                    size_t* bytes) {
  if (!model || !bytes) return fail(RLT_ERR_INVALID, "model and bytes must be non-NULL");
  if (batch < 1 || t_max < 1) return fail(RLT_ERR_INVALID, "batch and t_max must be >= 1");
  StateLayout S;
  compute_state_layout(model->lay, batch, t_max, keep_encoder_cache ? 1 : 0, &S);
  *bytes = S.total;
  return RLT_OK;
}

int rlt_state_init(const rlt_model* model, void* buffer, size_t buffer_bytes, int32_t batch, int32_t t_max,
                   int32_t keep_encoder_cache, void* stream, rlt_state** out) {
  if (!model || !buffer || !out) return fail(RLT_ERR_INVALID, "model, buffer and out must be non-NULL");
  if (batch < 1 || t_max < 1) return fail(RLT_ERR_INVALID, "batch and t_max must be >= 1");
  if (reinterpret_cast<uintptr_t>(buffer) % kAlign != 0)
    return fail(RLT_ERR_INVALID, "state buffer must be 256-byte aligned");
  StateLayout S;
  compute_state_layout(model->lay, batch, t_max, keep_encoder_cache ? 1 : 0, &S);
  if (buffer_bytes < S.total)
    return fail(RLT_ERR_INVALID, "state buffer too small: need " + std::to_string(S.total) + " bytes");
  if (int rc0 = need_gpu_memory(buffer, "state buffer")) return rc0;
  rlt_state* s = new (std::nothrow) rlt_state;
  if (!s) return fail(RLT_ERR_INVALID, "out of host memory");
  s->cfg = model->cfg;
  s->lay = S;
  s->buf = static_cast<char*>(buffer);
  s->bytes = buffer_bytes;
  // Memory rows are zeroed once: the decoder reads whole 8-key value blocks, and rows past
  // the current position (multiplied by a zero weight) must hold finite values.
  const ModelLayout& M = model->lay;
  const size_t memv_bytes = static_cast<size_t>(M.G) * S.B * S.T8 * M.D * M.esz;
  hipError_t ze = launch_zero(s->buf + S.mem_k, S.mem_v - S.mem_k, as_stream(stream));
  if (ze == hipSuccess) ze = launch_zero(s->buf + S.mem_v, memv_bytes, as_stream(stream));
  if (ze != hipSuccess) {
    delete s;
    return fail(RLT_ERR_HIP, std::string("zero memory rows: ") + hipGetErrorString(ze));
  }
  int rc = reset_state(model, s, as_stream(stream));
  if (rc) {
    delete s;
    return rc;
  }
  *out = s;
  return RLT_OK;
}

int rlt_state_reset(const rlt_model* model, rlt_state* state, void* stream) {
  if (!model || !state) return fail(RLT_ERR_INVALID, "model and state must be non-NULL");
  if (std::memcmp(&model->cfg, &state->cfg, sizeof(rlt_config)) != 0)
    return fail(RLT_ERR_INVALID, "state was built for a different model configuration");
  return reset_state(model, state, as_stream(stream));
}

void rlt_state_release(rlt_state* state) { delete state; }

int rlt_state_snapshot_bytes(const rlt_state* state, size_t* bytes) {
  if (!state || !bytes) return fail(RLT_ERR_INVALID, "state and bytes must be non-NULL");
  ModelLayout M;
  compute_model_layout(state->cfg, &M);
  *bytes = sizeof(SnapHeader) + snap_payload(snap_regions(M, state->lay, state->t_enc, state->lay.keep));
  return RLT_OK;
}

int rlt_state_save(const rlt_model* model, const rlt_state* state, void* dst, size_t dst_bytes, void* stream) {
  int rc = check_pair(model, state);
  if (rc) return rc;
  if (!dst) return fail(RLT_ERR_INVALID, "dst is NULL");
  if (is_device_pointer(dst)) return fail(RLT_ERR_INVALID, "a snapshot lives in host memory");
  const auto regions = snap_regions(model->lay, state->lay, state->t_enc, state->lay.keep);
  const size_t payload = snap_payload(regions);
  if (dst_bytes < sizeof(SnapHeader) + payload)
    return fail(RLT_ERR_INVALID, "snapshot buffer too small: need " + std::to_string(sizeof(SnapHeader) + payload));
  SnapHeader h{};
  std::memcpy(h.magic, kSnapMagic, sizeof(kSnapMagic));
  h.header_bytes = sizeof(SnapHeader);
  h.format = 1;
  h.cfg = state->cfg;
  h.version = state->version;
  h.batch = state->lay.B;
  h.t_enc = state->t_enc;
  h.t_dec = state->t_dec;
  h.keep = state->lay.keep;
  h.window_convention = 1;
  h.payload_bytes = payload;
  std::memcpy(dst, &h, sizeof(h));
  char* out = static_cast<char*>(dst) + sizeof(SnapHeader);
  for (const auto& r : regions) {
    if (r.width == 0 || r.height == 0) continue;
    RLT_HIP(hipMemcpy2DAsync(out, r.width, state->buf + r.off, r.pitch, r.width, r.height, hipMemcpyDefault,
                             as_stream(stream)),
            "save snapshot");
    out += r.width * r.height;
  }
  return RLT_OK;
}

int rlt_state_restore(const rlt_model* model, rlt_state* state, const void* src, size_t src_bytes, void* stream) {
  if (!model || !state || !src) return fail(RLT_ERR_INVALID, "model, state and src must be non-NULL");
  if (std::memcmp(&model->cfg, &state->cfg, sizeof(rlt_config)) != 0)
    return fail(RLT_ERR_INVALID, "state was built for a different model configuration");
  if (is_device_pointer(src)) return fail(RLT_ERR_INVALID, "a snapshot lives in host memory");
  if (src_bytes < sizeof(SnapHeader)) return fail(RLT_ERR_INVALID, "snapshot shorter than its header");
  SnapHeader h;
  std::memcpy(&h, src, sizeof(h));
  if (std::memcmp(h.magic, kSnapMagic, sizeof(kSnapMagic)) != 0 || h.header_bytes != sizeof(SnapHeader) ||
      h.format != 1 || h.window_convention != 1)
    return fail(RLT_ERR_INVALID, "not a snapshot of this format");
  if (std::memcmp(&h.cfg, &model->cfg, sizeof(rlt_config)) != 0)
    return fail(RLT_ERR_INVALID, "snapshot was taken under a different model configuration");
  if (h.version != model->version)
    return fail(RLT_ERR_STALE_STATE, "snapshot was taken under weights version " + std::to_string(h.version) +
                                         ", the model is at " + std::to_string(model->version));
  if (h.batch != state->lay.B) return fail(RLT_ERR_INVALID, "snapshot batch differs from the state's");
  if (h.t_enc < 0 || h.t_dec < 0 || h.t_dec > h.t_enc) return fail(RLT_ERR_INVALID, "snapshot positions are corrupt");
  if (h.t_enc > state->lay.T) return fail(RLT_ERR_CAPACITY, "snapshot holds more positions than the state's t_max");
  if (state->lay.keep && !h.keep)
    return fail(RLT_ERR_NO_ENC_CACHE, "the state keeps an encoder cache but the snapshot has none");
  StateLayout Ssrc = state->lay;  // the snapshot's packed widths depend only on t, B and the model
  Ssrc.keep = h.keep;
  const auto src_regions = snap_regions(model->lay, Ssrc, h.t_enc, h.keep);
  const size_t payload = snap_payload(src_regions);
  if (h.payload_bytes != payload || src_bytes < sizeof(SnapHeader) + payload)
    return fail(RLT_ERR_INVALID, "snapshot size does not match its header");
  int rc = reset_state(model, state, as_stream(stream));
  if (rc) return rc;
  const auto dst_regions = snap_regions(model->lay, state->lay, h.t_enc, state->lay.keep);
  const char* in = static_cast<const char*>(src) + sizeof(SnapHeader);
  for (size_t i = 0; i < src_regions.size(); ++i) {
    const SnapRegion& r = src_regions[i];
    if (i < dst_regions.size() && r.width && r.height) {
      const SnapRegion& d = dst_regions[i];
      RLT_HIP(hipMemcpy2DAsync(state->buf + d.off, d.pitch, in, r.width, r.width, r.height, hipMemcpyDefault,
                               as_stream(stream)),
              "restore snapshot");
    }
    in += r.width * r.height;
  }
  state->t_enc = h.t_enc;
  state->t_dec = h.t_dec;
  return RLT_OK;
}

int rlt_state_position(const rlt_state* state, int32_t* t_enc, int32_t* t_dec, uint64_t* version) {
  if (!state) return fail(RLT_ERR_INVALID, "state is NULL");
  if (t_enc) *t_enc = state->t_enc;
  if (t_dec) *t_dec = state->t_dec;
  if (version) *version = state->version;
  return RLT_OK;
}

int rlt_state_device_error(rlt_state* state, void* stream, int32_t* flags) {
  if (!state || !flags) return fail(RLT_ERR_INVALID, "state and flags must be non-NULL");
  int32_t v = 0;
  RLT_HIP(hipMemcpyAsync(&v, state->buf + state->lay.flags, sizeof(v), hipMemcpyDeviceToHost,
                         as_stream(stream)),
          "read device flags");
  RLT_HIP(hipStreamSynchronize(as_stream(stream)), "synchronise");
  *flags = v;
  return RLT_OK;
}

int rlt_model_set_decoder_path(rlt_model* model, int32_t path) {
  if (!model) return fail(RLT_ERR_INVALID, "model is NULL");
  if (path != RLT_PATH_AUTO && path != RLT_PATH_PERSISTENT && path != RLT_PATH_BATCHED)
    return fail(RLT_ERR_INVALID, "path must be RLT_PATH_AUTO, RLT_PATH_PERSISTENT or RLT_PATH_BATCHED");
  if (path == RLT_PATH_PERSISTENT && !dec_small_supported(model->lay, 1))
    return fail(RLT_ERR_UNSUPPORTED, "the persistent decoder does not support this model shape");
  if (path == RLT_PATH_BATCHED && !dec_batched_supported(model->lay))
    return fail(RLT_ERR_UNSUPPORTED, "the batched decoder does not support this model shape");
  model->path = path;
  return RLT_OK;
}

static int choose_path(const rlt_model* model, int t_max) {
  if (model->path == RLT_PATH_BATCHED) return RLT_PATH_BATCHED;
  if (dec_small_supported(model->lay, t_max)) return RLT_PATH_PERSISTENT;
  if (model->path == RLT_PATH_PERSISTENT) return -1;
  return dec_batched_supported(model->lay) ? RLT_PATH_BATCHED : -1;
}

int rlt_decoder_path(const rlt_model* model, int32_t t_max, int32_t* path) {
  if (!model || !path) return fail(RLT_ERR_INVALID, "model and path must be non-NULL");
  if (t_max < 1) return fail(RLT_ERR_INVALID, "t_max must be >= 1");
  const int p = choose_path(model, t_max);
  if (p < 0) return fail(RLT_ERR_UNSUPPORTED, "no decoder implementation for this configuration");
  *path = p;
  return RLT_OK;
}

int rlt_encoder_forward(const rlt_model* model, rlt_state* state, const int32_t* tokens, int32_t n,
                        void* stream) {
  int rc = check_pair(model, state);
  if (rc) return rc;
  if (!tokens) return fail(RLT_ERR_INVALID, "tokens is NULL");
  if (n < 1) return fail(RLT_ERR_INVALID, "n must be >= 1");
  rc = need_gpu_memory(tokens, "tokens");
  if (rc) return rc;
  const StateLayout& S = state->lay;
  const ModelLayout& M = model->lay;
  if (static_cast<int64_t>(state->t_enc) + n > S.T)
    return fail(RLT_ERR_CAPACITY, "encoder positions would exceed the state's T_max");
  if (state->t_enc > 0 && !S.keep)
    return fail(RLT_ERR_NO_ENC_CACHE,
                "the state keeps no encoder cache, so the known sequence must be encoded in one call");
  hipStream_t st = as_stream(stream);
  char* sb = state->buf;
  const char* ws = model->ws;
  const int D = M.D, H = M.H, DH = M.DH, dt = M.dtype;
  const int t0 = state->t_enc;
  const int bc_max = std::max(1, std::min(S.B, S.Nc / n));
  float* x = reinterpret_cast<float*>(sb + S.x);
  int32_t* flags = reinterpret_cast<int32_t*>(sb + S.flags);
  for (int b0 = 0; b0 < S.B; b0 += bc_max) {
    const int bc = std::min(bc_max, S.B - b0);
    const int rows = bc * n;
    RLT_HIP(launch_embed(tokens + static_cast<size_t>(b0) * n, n, b0, rows, ws + M.embed, M.V, D, dt, x,
                         flags, st),
            "embed");
    for (int l = 0; l < M.L; ++l) {
      const char* lw = ws + M.layers + l * M.layer_stride;
      RLT_HIP(launch_rmsnorm_rows(x, reinterpret_cast<const float*>(ws + M.g_enc_attn) + l * D, sb + S.h,
                                  rows, D, M.eps, dt, nullptr, n, b0, t0, S.T, st),
              "encoder norm");
      GemmArgs g{};
      g.A = sb + S.h; g.W = lw + M.l_qkv; g.out = sb + S.qkv;
      g.M = rows; g.N = 3 * D; g.K = D; g.lda = D; g.ldw = D; g.ldo = 3 * D;
      g.epi = EPI_STORE;
      const size_t cache_layer = static_cast<size_t>(l) * S.B * S.T * D * M.esz;
      if (S.keep) {
        g.sc_k = sb + S.enc_k + cache_layer;
        g.sc_v = sb + S.enc_v + cache_layer;
        g.sc_c0 = D;
        g.sc_n = n; g.sc_b0 = b0; g.sc_t0 = t0; g.sc_T = S.T; g.sc_H = H; g.sc_dh = DH; g.sc_D = D;
        g.sc_B = S.B;
      }
      RLT_HIP(launch_gemm(g, dt, st), "encoder qkv");
      AttnArgs a{};
      a.q = sb + S.qkv; a.ldq = 3 * D;
      if (S.keep) {
        const size_t bo = static_cast<size_t>(b0) * H * S.T * DH * M.esz;
        a.k = sb + S.enc_k + cache_layer + bo;
        a.v = sb + S.enc_v + cache_layer + bo;
        a.kv_ld_b = static_cast<long long>(H) * S.T * DH;
        a.kv_ld_h = static_cast<long long>(S.T) * DH;
        a.kv_ld_t = DH;
        a.t0 = t0;
      } else {
        a.k = sb + S.qkv + static_cast<size_t>(D) * M.esz;
        a.v = sb + S.qkv + static_cast<size_t>(2 * D) * M.esz;
        a.kv_ld_b = static_cast<long long>(n) * 3 * D;
        a.kv_ld_h = DH;
        a.kv_ld_t = 3 * D;
        a.t0 = 0;
      }
      a.out = sb + S.attn; a.ldo = D;
      a.Bc = bc; a.H = H; a.dh = DH; a.n = n;
      RLT_HIP(launch_enc_attention(a, dt, st), "encoder attention");
      GemmArgs o{};
      o.A = sb + S.attn; o.W = lw + M.l_wo; o.out = x;
      o.M = rows; o.N = D; o.K = D; o.lda = D; o.ldw = D; o.ldo = D; o.epi = EPI_RESID_F32;
      RLT_HIP(launch_gemm(o, dt, st), "encoder attention output");
      RLT_HIP(launch_rmsnorm_rows(x, reinterpret_cast<const float*>(ws + M.g_enc_ffn) + l * D, sb + S.h,
                                  rows, D, M.eps, dt, nullptr, n, b0, t0, S.T, st),
              "encoder norm");
      GemmArgs f{};
      f.A = sb + S.h; f.W = lw + M.l_fin; f.out = sb + S.act;
      f.M = rows; f.N = M.F2; f.K = D; f.lda = D; f.ldw = D; f.ldo = M.F;
      f.epi = M.ffn_kind == RLT_FFN_GELU ? EPI_GELU : EPI_SWIGLU;
      RLT_HIP(launch_gemm(f, dt, st), "encoder ffn in");
      GemmArgs f2{};
      f2.A = sb + S.act; f2.W = lw + M.l_fout; f2.out = x;
      f2.M = rows; f2.N = D; f2.K = M.F; f2.lda = M.F; f2.ldw = M.F; f2.ldo = D; f2.epi = EPI_RESID_F32;
      RLT_HIP(launch_gemm(f2, dt, st), "encoder ffn out");
    }
    RLT_HIP(launch_rmsnorm_rows(x, reinterpret_cast<const float*>(ws + M.g_enc_final), sb + S.h, rows, D,
                                M.eps, dt, sb + S.e, n, b0, t0, S.T, st),
            "encoder final norm");
    for (int gi = 0; gi < M.G; ++gi) {
      const size_t goff = static_cast<size_t>(gi) * S.B * S.T * D * M.esz;
      const size_t goff_v = static_cast<size_t>(gi) * S.B * S.T8 * D * M.esz;
      GemmArgs g{};
      g.A = sb + S.h; g.W = ws + M.wkvm + gi * M.group_stride; g.out = nullptr;
      g.M = rows; g.N = 2 * D; g.K = D; g.lda = D; g.ldw = D; g.ldo = 0;
      g.epi = EPI_SCATTER_HEADS;
      g.sc_k = sb + S.mem_k + goff;
      g.sc_v = sb + S.mem_v + goff_v;
      g.sc_c0 = 0;
      g.sc_n = n; g.sc_b0 = b0; g.sc_t0 = t0; g.sc_T = S.T; g.sc_H = H; g.sc_dh = DH; g.sc_D = D; g.sc_B = S.B;
      RLT_HIP(launch_gemm(g, dt, st), "memory projection");
    }
  }
  state->t_enc += n;
  return RLT_OK;
}

int rlt_decoder_replay(const rlt_model* model, rlt_state* state, int32_t n, float* s_out, void* stream) {
  int rc = check_pair(model, state);
  if (rc) return rc;
  if (n < 1) return fail(RLT_ERR_INVALID, "n must be >= 1");
  if (static_cast<int64_t>(state->t_dec) + n > state->t_enc)
    return fail(RLT_ERR_ORDER, "decoder would run ahead of the encoder (t_dec + n > t_enc)");
  rc = need_gpu_memory(s_out, "s_out");
  if (rc) return rc;
  const ModelLayout& M = model->lay;
  const StateLayout& S = state->lay;
  hipStream_t st = as_stream(stream);
  const int path = choose_path(model, S.T);
  if (path == RLT_PATH_PERSISTENT) {
    DecSmallArgs a{};
    a.ws = model->ws;
    a.state = state->buf;
    a.s_out = s_out;
    a.B = S.B;
    a.T = S.T;
    a.t0 = state->t_dec;
    a.n = n;
    RLT_HIP(launch_dec_small(M, S, a, st), "decoder replay (persistent)");
  } else if (path == RLT_PATH_BATCHED) {
    RLT_HIP(run_dec_batched(M, S, model->ws, state->buf, state->buf + S.dec_scratch, s_out, state->t_dec, n, st),
            "decoder replay (batched)");
  } else {
    return fail(RLT_ERR_UNSUPPORTED, "no decoder implementation for this configuration");
  }
  state->t_dec += n;
  return RLT_OK;
}

int rlt_decoder_replay_noalloc(const rlt_model* model, rlt_state* state, int32_t n, float* s_out, void* stream) {
  int rc = check_pair(model, state);
  if (rc) return rc;
  if (n < 1) return fail(RLT_ERR_INVALID, "n must be >= 1");
  if (static_cast<int64_t>(state->t_dec) + n > state->t_enc)
    return fail(RLT_ERR_ORDER, "decoder would run ahead of the encoder (t_dec + n > t_enc)");
  rc = need_gpu_memory(s_out, "s_out");
  if (rc) return rc;
  const ModelLayout& M = model->lay;
  const StateLayout& S = state->lay;
  hipStream_t st = as_stream(stream);
  const int path = choose_path(model, S.T);
  if (path == RLT_PATH_PERSISTENT) {
    // the persistent decoder keeps everything in LDS and registers: no scratch at all
    DecSmallArgs a{};
    a.ws = model->ws;
    a.state = state->buf;
    a.s_out = s_out;
    a.B = S.B;
    a.T = S.T;
    a.t0 = state->t_dec;
    a.n = n;
    RLT_HIP(launch_dec_small(M, S, a, st), "decoder replay (persistent)");
  } else if (path == RLT_PATH_BATCHED) {
    if (S.dec_scratch_bytes > kStaticScratchBytes)
      return fail(RLT_ERR_UNSUPPORTED, "the batched decoder needs " + std::to_string(S.dec_scratch_bytes) +
                                           " bytes of scratch for this batch and t_max; the library's static scratch holds " +
                                           std::to_string(kStaticScratchBytes));
    hipPointerAttribute_t attr;
    RLT_HIP(hipPointerGetAttributes(&attr, state->buf), "state device");
    char* base = nullptr;
    rc = static_scratch(attr.device, &base);
    if (rc) return rc;
    // the arrival counters of the weight-streaming products start at zero (cleared with a fill
    // kernel, which graph capture records like any launch)
    size_t cnt_off = 0, cnt_bytes = 0;
    dec_batched_counters(M, S.B, S.T, &cnt_off, &cnt_bytes);
    if (cnt_bytes) RLT_HIP(launch_zero(base + cnt_off, cnt_bytes, st), "clear decoder counters");
    RLT_HIP(run_dec_batched(M, S, model->ws, state->buf, base, s_out, state->t_dec, n, st), "decoder replay (batched)");
  } else {
    return fail(RLT_ERR_UNSUPPORTED, "no decoder implementation for this configuration");
  }
  state->t_dec += n;
  return RLT_OK;
}

int rlt_logits(const rlt_model* model, const float* s, int64_t n_rows, float* logits, void* stream) {
  if (!model || !s || !logits) return fail(RLT_ERR_INVALID, "model, s and logits must be non-NULL");
  if (n_rows < 1 || n_rows > 0x7fffffff) return fail(RLT_ERR_INVALID, "n_rows out of range");
  if (int rc = need_gpu_memory({{s, "s"}, {logits, "logits"}})) return rc;
  const ModelLayout& M = model->lay;
  GemmArgs g{};
  g.A = s; g.a_f32 = 1; g.W = model->ws + M.wout; g.out = logits;
  g.M = static_cast<int>(n_rows); g.N = M.V; g.K = M.D; g.lda = M.D; g.ldw = M.D; g.ldo = M.V;
  g.epi = EPI_STORE_F32;
  RLT_HIP(launch_gemm(g, M.dtype, as_stream(stream)), "logits");
  return RLT_OK;
}

int rlt_score_actions(const rlt_model* model, const float* s, const int32_t* actions, int64_t n_rows,
                      float temperature, const float* behaviour_logp, float* logp_out, float* ratio_out,
                      void* stream) {
  if (!model || !s || !actions || !logp_out) return fail(RLT_ERR_INVALID, "model, s, actions and logp_out must be non-NULL");
  if (n_rows < 1 || n_rows > 0x7fffffff) return fail(RLT_ERR_INVALID, "n_rows out of range");
  if (!(temperature > 0.f)) return fail(RLT_ERR_INVALID, "temperature must be > 0");
  if (ratio_out && !behaviour_logp) return fail(RLT_ERR_INVALID, "ratio_out needs behaviour_logp");
  if (int rc = need_gpu_memory({{s, "s"}, {actions, "actions"}, {behaviour_logp, "behaviour_logp"},
                                {logp_out, "logp_out"}, {ratio_out, "ratio_out"}}))
    return rc;
  const ModelLayout& M = model->lay;
  RLT_HIP(launch_score_actions(s, model->ws + M.wout, M.has_wout_frag ? model->ws + M.wout_frag : nullptr, actions,
                               behaviour_logp, logp_out, ratio_out,
                               static_cast<int>(n_rows), M.D, M.V, temperature, M.dtype, as_stream(stream)),
          "score actions");
  return RLT_OK;
}

int rlt_decoder_step(const rlt_model* model, rlt_state* state, const int32_t* tokens, float* s_out,
                     float* logits, void* stream) {
  int rc = check_pair(model, state);
  if (rc) return rc;
  if (state->t_dec != state->t_enc)
    return fail(RLT_ERR_ORDER, "decoder_step needs t_dec == t_enc (every encoded position decoded)");
  if (state->t_enc >= state->lay.T) return fail(RLT_ERR_CAPACITY, "state is full (t == T_max)");
  if (state->t_enc > 0 && !state->lay.keep)
    return fail(RLT_ERR_NO_ENC_CACHE, "incremental generation needs keep_encoder_cache");
  if (!tokens) return fail(RLT_ERR_INVALID, "tokens is NULL");
  // every pointer and the decoder implementation are checked before the first launch, so a
  // failure enqueues nothing and leaves the state's positions as they were
  rc = need_gpu_memory({{tokens, "tokens"}, {s_out, "s_out"}, {logits, "logits"}});
  if (rc) return rc;
  if (choose_path(model, state->lay.T) < 0)
    return fail(RLT_ERR_UNSUPPORTED, "no decoder implementation for this configuration");
  rc = rlt_encoder_forward(model, state, tokens, 1, stream);
  if (rc) return rc;
  rc = rlt_decoder_replay(model, state, 1, s_out, stream);
  if (rc) return rc;
  if (logits) {
    const float* s = reinterpret_cast<const float*>(state->buf + state->lay.s);
    rc = rlt_logits(model, s, state->lay.B, logits, stream);
    if (rc) return rc;
  }
  return RLT_OK;
}

namespace {
constexpr int32_t kMaxSampleVocab = 32768;

int check_sampling(const rlt_sampling* p, int64_t n_rows, int32_t vocab) {
  if (!p) return fail(RLT_ERR_INVALID, "sampling parameters are NULL");
  if (!(p->temperature > 0.f)) return fail(RLT_ERR_INVALID, "temperature must be > 0");
  if (p->top_k < 0) return fail(RLT_ERR_INVALID, "top_k must be >= 0");
  if (!(p->top_p > 0.f) || p->top_p > 1.f) return fail(RLT_ERR_INVALID, "top_p must be in (0, 1]");
  if (n_rows < 1 || n_rows > 0x7fffffff) return fail(RLT_ERR_INVALID, "n_rows out of range");
  if (vocab < 1) return fail(RLT_ERR_INVALID, "vocab must be >= 1");
  if (vocab > kMaxSampleVocab) return fail(RLT_ERR_UNSUPPORTED, "sampling supports vocab <= 32768");
  return RLT_OK;
}
}  // namespace

int rlt_sample_tokens(const float* logits, int64_t n_rows, int32_t vocab, const rlt_sampling* params,
                      const float* uniforms, int32_t* tokens_out, float* logp_out, void* stream) {
  if (!logits || !uniforms || !tokens_out || !logp_out)
    return fail(RLT_ERR_INVALID, "logits, uniforms, tokens_out and logp_out must be non-NULL");
  int rc = check_sampling(params, n_rows, vocab);
  if (rc) return rc;
  rc = need_gpu_memory({{logits, "logits"}, {uniforms, "uniforms"}, {tokens_out, "tokens_out"}, {logp_out, "logp_out"}});
  if (rc) return rc;
  RLT_HIP(launch_sample_tokens(logits, uniforms, tokens_out, logp_out, static_cast<int>(n_rows), vocab,
                               params->temperature, params->top_k, params->top_p, as_stream(stream)),
          "sample tokens");
  return RLT_OK;
}

int rlt_decoder_step_sample(const rlt_model* model, rlt_state* state, const int32_t* tokens,
                            const rlt_sampling* params, const float* uniforms, int32_t* next_tokens,
                            float* behaviour_logp, float* s_out, float* logits, void* stream) {
  int rc = check_pair(model, state);
  if (rc) return rc;
  if (!logits || !uniforms || !next_tokens || !behaviour_logp)
    return fail(RLT_ERR_INVALID, "logits, uniforms, next_tokens and behaviour_logp must be non-NULL");
  rc = check_sampling(params, state->lay.B, model->lay.V);
  if (rc) return rc;
  rc = need_gpu_memory({{uniforms, "uniforms"}, {next_tokens, "next_tokens"}, {behaviour_logp, "behaviour_logp"}});
  if (rc) return rc;
  rc = rlt_decoder_step(model, state, tokens, s_out, logits, stream);
  if (rc) return rc;
  return rlt_sample_tokens(logits, state->lay.B, model->lay.V, params, uniforms, next_tokens, behaviour_logp,
                           stream);
}

int rlt_bptt_workspace_bytes(const rlt_config* cfg, int32_t batch, int32_t seq_len, size_t* bytes) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(RLT_ERR_INVALID, "bytes is NULL");
  const char* why = "";
  if (!bptt_supported(*cfg, batch, seq_len, &why)) return fail(RLT_ERR_UNSUPPORTED, why);
  *bytes = bptt_workspace_bytes(*cfg, batch, seq_len);
  return RLT_OK;
}

int rlt_bptt(const rlt_config* cfg, const float* weights, const int32_t* tokens, const float* mask, int32_t batch,
             int32_t seq_len, int32_t detach, float* grads, float* loss, void* workspace, size_t workspace_bytes,
             void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!weights || !tokens || !grads || !loss || !workspace)
    return fail(RLT_ERR_INVALID, "weights, tokens, grads, loss and workspace must be non-NULL");
  if (detach & ~(RLT_DETACH_S | RLT_DETACH_KV | RLT_DETACH_MEMORY))
    return fail(RLT_ERR_INVALID, "detach holds unknown bits");
  const char* why = "";
  if (!bptt_supported(*cfg, batch, seq_len, &why)) return fail(RLT_ERR_UNSUPPORTED, why);
  if (workspace_bytes < bptt_workspace_bytes(*cfg, batch, seq_len))
    return fail(RLT_ERR_INVALID, "workspace is smaller than rlt_bptt_workspace_bytes");
  rc = need_gpu_memory({{weights, "weights"}, {tokens, "tokens"}, {mask, "mask"}, {grads, "grads"}, {loss, "loss"},
                        {workspace, "workspace"}});
  if (rc) return rc;
  BpttOffsets o{};
  const bool sw = cfg->ffn_kind == RLT_FFN_SWIGLU;
  o.embed = param_offset(*cfg, "embed", nullptr);
  o.w_out = param_offset(*cfg, "w_out", nullptr);
  o.s_star = param_offset(*cfg, "s_star", nullptr);
  o.w_ge = param_offset(*cfg, "w_ge", nullptr);
  o.w_gs = param_offset(*cfg, "w_gs", nullptr);
  o.w_fb = param_offset(*cfg, "w_fb", nullptr);
  o.b_g = param_offset(*cfg, "b_g", nullptr);
  o.wq = param_offset(*cfg, "wq", nullptr);
  o.wk = param_offset(*cfg, "wk", nullptr);
  o.wv = param_offset(*cfg, "wv", nullptr);
  o.wo = param_offset(*cfg, "wo", nullptr);
  o.f1 = param_offset(*cfg, sw ? "ffn_gate" : "ffn_w1", nullptr);
  o.f2 = param_offset(*cfg, sw ? "ffn_up" : "ffn_w2", nullptr);
  o.f3 = sw ? param_offset(*cfg, "ffn_down", nullptr) : -1;
  o.wqx = param_offset(*cfg, "wqx", nullptr);
  o.wox = param_offset(*cfg, "wox", nullptr);
  o.wkm = param_offset(*cfg, "wkm", nullptr);
  o.wvm = param_offset(*cfg, "wvm", nullptr);
  o.g_enc_attn = param_offset(*cfg, "g_enc_attn", nullptr);
  o.g_enc_ffn = param_offset(*cfg, "g_enc_ffn", nullptr);
  o.g_enc_final = param_offset(*cfg, "g_enc_final", nullptr);
  o.g_dec_self = param_offset(*cfg, "g_dec_self", nullptr);
  o.g_dec_cross = param_offset(*cfg, "g_dec_cross", nullptr);
  o.g_dec_ffn = param_offset(*cfg, "g_dec_ffn", nullptr);
  o.g_dec_final = param_offset(*cfg, "g_dec_final", nullptr);
  int32_t nt = 0;
  int64_t total = 0;
  rlt_param_count(cfg, &nt, &total);
  RLT_HIP(run_bptt(*cfg, o, weights, tokens, mask, batch, seq_len, detach, grads, loss,
                   static_cast<char*>(workspace), static_cast<size_t>(total), as_stream(stream)),
          "bptt");
  return RLT_OK;
}

int rlt_state_load_encoder_outputs(const rlt_model* model, rlt_state* state, const float* e,
                                   const float* mem_k, const float* mem_v, int32_t n, void* stream) {
  int rc = check_pair(model, state);
  if (rc) return rc;
  if (!e || !mem_k || !mem_v) return fail(RLT_ERR_INVALID, "e, mem_k and mem_v must be non-NULL");
  if (n < 1) return fail(RLT_ERR_INVALID, "n must be >= 1");
  rc = need_gpu_memory({{e, "e"}, {mem_k, "mem_k"}, {mem_v, "mem_v"}});
  if (rc) return rc;
  const StateLayout& S = state->lay;
  const ModelLayout& M = model->lay;
  if (static_cast<int64_t>(state->t_enc) + n > S.T) return fail(RLT_ERR_CAPACITY, "positions exceed T_max");
  hipStream_t st = as_stream(stream);
  const int t0 = state->t_enc;
  RLT_HIP(launch_store_tokens(e, state->buf + S.e, S.B, n, M.D, t0, S.T, M.dtype, 0, M.H, M.DH, 1, st),
          "load e");
  const size_t gsrc = static_cast<size_t>(S.B) * n * M.D;
  const size_t gdst = static_cast<size_t>(S.B) * S.T * M.D * M.esz;
  const size_t gdst_v = static_cast<size_t>(S.B) * S.T8 * M.D * M.esz;
  for (int g = 0; g < M.G; ++g) {
    RLT_HIP(launch_store_tokens(mem_k + g * gsrc, state->buf + S.mem_k + g * gdst, S.B, n, M.D, t0, S.T,
                                M.dtype, 1, M.H, M.DH, 1, st),
            "load memory keys");
    RLT_HIP(launch_store_tokens(mem_v + g * gsrc, state->buf + S.mem_v + g * gdst_v, S.B, n, M.D, t0, S.T,
                                M.dtype, 2, M.H, M.DH, 1, st),
            "load memory values");
  }
  state->t_enc += n;
  return RLT_OK;
}

int rlt_state_read_encoder_outputs(const rlt_model* model, const rlt_state* state, int32_t t0, int32_t n,
                                   float* e, float* mem_k, float* mem_v, void* stream) {
  if (!model || !state) return fail(RLT_ERR_INVALID, "model and state must be non-NULL");
  if (std::memcmp(&model->cfg, &state->cfg, sizeof(rlt_config)) != 0)
    return fail(RLT_ERR_INVALID, "state was built for a different model configuration");
  if (n < 1 || t0 < 0 || t0 + n > state->t_enc) return fail(RLT_ERR_INVALID, "positions not encoded yet");
  if (int rc = need_gpu_memory({{e, "e"}, {mem_k, "mem_k"}, {mem_v, "mem_v"}})) return rc;
  const StateLayout& S = state->lay;
  const ModelLayout& M = model->lay;
  hipStream_t st = as_stream(stream);
  if (e) {
    RLT_HIP(launch_store_tokens(e, state->buf + S.e, S.B, n, M.D, t0, S.T, M.dtype, 0, M.H, M.DH, 0, st),
            "read e");
  }
  const size_t gsrc = static_cast<size_t>(S.B) * n * M.D;
  const size_t gdst = static_cast<size_t>(S.B) * S.T * M.D * M.esz;
  const size_t gdst_v = static_cast<size_t>(S.B) * S.T8 * M.D * M.esz;
  for (int g = 0; g < M.G; ++g) {
    if (mem_k) {
      RLT_HIP(launch_store_tokens(mem_k + g * gsrc, state->buf + S.mem_k + g * gdst, S.B, n, M.D, t0, S.T,
                                  M.dtype, 1, M.H, M.DH, 0, st),
              "read memory keys");
    }
    if (mem_v) {
      RLT_HIP(launch_store_tokens(mem_v + g * gsrc, state->buf + S.mem_v + g * gdst_v, S.B, n, M.D, t0, S.T,
                                  M.dtype, 2, M.H, M.DH, 0, st),
              "read memory values");
    }
  }
  return RLT_OK;
}

}  // extern "C"
