// C-ABI layer: argument checks, workspace layout, launch geometry.  No device memory is
// allocated or read here; every call only enqueues kernels on the caller's stream.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/dqg.h"
#include "dqg_internal.hpp"

namespace {

using dqg::GemvArgs;
using dqg::MoeArgs;

constexpr int kMaxE = 4096;
constexpr int kMaxK = 32;
constexpr int kMaxTK = 65536;
// Experts (and GEMV calls) with at least this many tokens use the matrix cores: a product of
// two or more token rows with one weight matrix is a real contraction, and the matrix cores
// take its multiply-adds off the vector ALU, which bounds the vector-ALU tiles (measured
// best at 2 against 1, 3, 5, 9 and 16 on the batched Q30 layers and the T = 4 GEMV).
constexpr int kMfmaMinTokens = 2;
// dense GEMV: calls with at most this many tokens run gemv_tok_kernel (one token on its
// vector ALUs, 2 to 4 on its matrix-core body, which decodes each weight once for all
// tokens), more tokens the expert tiles' E = 1 case (16- or 32-row matrix-core tiles)
constexpr int kGemvTokMaxTokens = 4;
constexpr int kMaxSplitDown = 16;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of the multi-launch path.  Its layout depends only on (H, I, E, k) and the
// workspace's capacity t_cap (the largest T whose layout fits the caller's bytes), so calls
// with any T <= t_cap on one workspace find every region at the same place.  The split
// partials are kept zero between calls (their readers clear them).
struct MoePlan {
  int T, H, I, E, k, TK, A;
  int tiles_gu, tiles_dn, S_gu, S_dn;
  int t_cap, sgu_max, sdn_max;
  size_t o_err, o_fx, o_nact, o_rec, o_slots, o_nvalid, o_ids, o_wts, o_h, o_pgu, o_pdn;
  size_t o_rtp, o_rtl, total;  // router partials [splits][t_cap][E] and logits [t_cap][E]
  bool ok;  // partial buffers addressable with 32-bit byte offsets
};

bool moe_sizes_ok(int T, int H, int I, int E, int k) {
  if (T < 1 || H < 1 || I < 1 || E < 1 || k < 1) return false;
  if (E > kMaxE || k > kMaxK || k > E) return false;
  if ((long long)T * k > kMaxTK) return false;
  if (H % 64 || I % 64) return false;
  if ((long long)H * I > (1LL << 31)) return false;
  return true;
}

// Expected number of distinct experts when T tokens each pick k of E uniformly: sizes the
// K splits so that the active tiles fill the GPU (only performance depends on it).
int expected_active(int T, int E, int k) {
  const double miss = std::pow(1.0 - (double)k / E, (double)T);
  return std::max(1, std::min(std::min(E, T * k), (int)std::lround(E * (1.0 - miss))));
}

// K splits of a streaming kernel: `per_wg` blocks (16 byte rows each) per workgroup when
// possible -- a few batches each, so that many workgroups keep bytes in flight while the
// split partials and their finishers stay cheap -- but at most `max_split`, and few enough
// that the fp32 split partials (partial_bytes per split) stay under 15% of the weight bytes
// the kernel streams.
int pick_ex_split(int nblk, int per_wg, int max_split, double weight_bytes,
                  double partial_bytes) {
  int S = (nblk + per_wg - 1) / per_wg;
  const double budget = 0.15 * weight_bytes / std::max(partial_bytes, 1.0);
  S = std::min(S, std::max(1, (int)budget));
  return std::max(1, std::min(S, max_split));
}

// maximum K splits of the two expert kernels for a workspace of capacity t_cap (bounded
// so that the partials stay addressable with 32-bit byte offsets)
int moe_split_max(int nblk, int per_wg, int cap, long long tk_cap, long long row_bytes) {
  const long long fit = ((1LL << 31) - 1) / std::max(1LL, tk_cap * row_bytes);
  return (int)std::max(1LL, std::min<long long>(std::min((nblk + per_wg - 1) / per_wg, cap), fit));
}

// Bytes of a split-partial region: splits x tk_cap x row_bytes with the uncapped number of
// splits, but never more than 2^31 (the capped count keeps offsets below that anyway).  The
// bound grows with t_cap, so the workspace total is monotonic in the capacity and the layout
// a workspace gets depends only on its size (the capped count alone would shrink the region,
// and the total with it, each time the cap drops by one split).
size_t split_region_bytes(int nblk, int per_wg, int cap, long long tk_cap, long long row_bytes) {
  const long long uncapped = std::min((nblk + per_wg - 1) / per_wg, cap);
  return (size_t)std::min<long long>(uncapped * tk_cap * row_bytes, 1LL << 31);
}

void moe_layout(MoePlan& p, int t_cap) {
  const int H = p.H, I = p.I, k = p.k;
  const long long tkc = (long long)t_cap * k;
  const int a_cap = (int)std::min<long long>(p.E, tkc);
  p.t_cap = t_cap;
  p.sgu_max = moe_split_max(H / 32, 4, dqg::ex_max_split(), tkc, 8LL * I);
  p.sdn_max = moe_split_max(I / 32, 8, kMaxSplitDown, tkc, 4LL * H);
  size_t o = 0;
  p.o_err = o;     o += 256;
  // single-launch exchange regions for the token counts this capacity allows
  p.o_fx = o;
  o = up256(o + (dqg::fused_supported(H, I, k) ? dqg::fused_ws_bytes(H, I, p.E, k, t_cap) : 0));
  p.o_nact = o;    o += 256;
  p.o_rec = o;     o = up256(o + 16 * (size_t)a_cap);
  p.o_slots = o;   o = up256(o + sizeof(int) * tkc);
  p.o_nvalid = o;  o = up256(o + sizeof(int) * (size_t)t_cap);
  p.o_ids = o;     o = up256(o + sizeof(int) * tkc);
  p.o_wts = o;     o = up256(o + sizeof(float) * tkc);
  p.o_h = o;       o = up256(o + sizeof(uint16_t) * (size_t)tkc * I);
  p.o_pgu = o;     o = up256(o + split_region_bytes(H / 32, 4, dqg::ex_max_split(), tkc, 8LL * I));
  p.o_pdn = o;     o = up256(o + split_region_bytes(I / 32, 8, kMaxSplitDown, tkc, 4LL * H));
  p.o_rtp = o;     o = up256(o + sizeof(float) * (size_t)dqg::router_splits(H) * t_cap * p.E);
  p.o_rtl = o;     o = up256(o + sizeof(float) * (size_t)t_cap * p.E);
  p.total = o;
}

// Plan of a call with T tokens on a workspace of ws_bytes (0: the size query for T).
MoePlan plan_moe(int T, int H, int I, int E, int k, size_t ws_bytes = 0) {
  MoePlan p{};
  p.T = T; p.H = H; p.I = I; p.E = E; p.k = k;
  p.TK = T * k;
  p.A = std::min(E, p.TK);
  p.tiles_gu = (I + 127) / 128;
  p.tiles_dn = (H + 127) / 128;
  moe_layout(p, T);
  p.ok = true;
  if (ws_bytes > p.total) {  // the largest capacity that fits the caller's workspace
    int lo = T, hi = kMaxTK / k;
    while (lo < hi) {
      const int mid = lo + (hi - lo + 1) / 2;
      MoePlan q = p;
      moe_layout(q, mid);
      if (q.total <= ws_bytes) lo = mid; else hi = mid - 1;
    }
    moe_layout(p, lo);
  }
  const int a_est = expected_active(T, E, k);
  const double gu_bytes = (double)a_est * H * I * 1.125, dn_bytes = gu_bytes / 2;
  // gate_up: no K split when the unsplit grid (active experts x column tiles) already gives
  // every compute unit 1.5 workgroups -- the partials and their finisher then cost more than
  // the parallelism they add; otherwise splits of 16 blocks (32 K indices each).  Down: 32
  // blocks per split (no split at all for I <= 1024).  Measured over T = 4 .. 64 on the
  // 128- and 512-expert shapes, FP4 and FP8 (4, 8, 16, 32 and 64 blocks per split).
  const bool wide_gu = (long long)a_est * p.tiles_gu >= 384;
  p.S_gu = wide_gu ? 1
                   : std::min(pick_ex_split(H / 32, 16, dqg::ex_max_split(), gu_bytes,
                                            8.0 * p.TK * I),
                              p.sgu_max);
  p.S_dn = std::min(pick_ex_split(I / 32, 32, kMaxSplitDown, dn_bytes, 4.0 * p.TK * H), p.sdn_max);
  return p;
}

int check_moe_common(const uint16_t* x, int T, int H, int I, int E, int k, const uint8_t* wgu,
                     const uint16_t* sgu, const uint8_t* wd, const uint16_t* sd, int group,
                     int format, const uint16_t* res, uint16_t* out, void* ws,
                     size_t ws_bytes) {
  if (!x || !wgu || !sgu || !wd || !sd || !out) return DQG_ERR_INVALID_ARG;
  if (T < 1 || H < 1 || I < 1 || E < 1 || k < 1 || k > E) return DQG_ERR_INVALID_ARG;
  const int fmt = format & 0xFF;
  const int flags = format & ~0xFF;
  if (fmt != DQG_FMT_INT4 && fmt != DQG_FMT_FP4_E2M1 && fmt != DQG_FMT_FP8_E4M3)
    return DQG_ERR_UNSUPPORTED;
  if (flags & ~(DQG_PATH_FORCE_GEMV | DQG_PATH_FORCE_MFMA | DQG_PATH_NO_FUSED))
    return DQG_ERR_UNSUPPORTED;
  if ((flags & DQG_PATH_FORCE_GEMV) && (flags & DQG_PATH_FORCE_MFMA)) return DQG_ERR_INVALID_ARG;
  if (group != 32 && group != 128) return DQG_ERR_UNSUPPORTED;
  if (!moe_sizes_ok(T, H, I, E, k)) return DQG_ERR_UNSUPPORTED;
  if (H % group || I % group) return DQG_ERR_UNSUPPORTED;
  // one code per byte: an FP8 expert matrix of 2 H I bytes must fit the kernels' 32-bit offsets
  if (fmt == DQG_FMT_FP8_E4M3 && (long long)H * I > (1LL << 30)) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(wgu) || !aligned16(sgu) || !aligned16(wd) || !aligned16(sd) ||
      !aligned16(out) || (res && !aligned16(res)))
    return DQG_ERR_MISALIGNED;
  if (!ws) return DQG_ERR_WORKSPACE;
  if (!aligned16(ws)) return DQG_ERR_MISALIGNED;
  if (ws_bytes < plan_moe(T, H, I, E, k).total) return DQG_ERR_WORKSPACE;
  return DQG_OK;
}

MoeArgs make_moe_args(const MoePlan& p, const uint16_t* x, const uint8_t* wgu,
                      const uint16_t* sgu, const uint8_t* wd, const uint16_t* sd, int group,
                      int format, const uint16_t* res, uint16_t* out, void* ws) {
  char* b = static_cast<char*>(ws);
  MoeArgs a{};
  a.x = x; a.T = p.T; a.H = p.H; a.I = p.I; a.E = p.E; a.k = p.k; a.group = group;
  a.fmt = format & 0xFF;
  a.wgu = wgu; a.sgu = sgu; a.wd = wd; a.sd = sd; a.res = res; a.out = out;
  a.ws.err = reinterpret_cast<int*>(b + p.o_err);
  a.ws.n_active = reinterpret_cast<int*>(b + p.o_nact);
  a.ws.rec = reinterpret_cast<int4*>(b + p.o_rec);
  a.ws.slot_list = reinterpret_cast<int*>(b + p.o_slots);
  a.ws.nvalid = reinterpret_cast<int*>(b + p.o_nvalid);
  a.ws.ids = reinterpret_cast<int32_t*>(b + p.o_ids);
  a.ws.wts = reinterpret_cast<float*>(b + p.o_wts);
  a.ws.hop = reinterpret_cast<uint16_t*>(b + p.o_h);
  a.ws.part_gu = reinterpret_cast<float*>(b + p.o_pgu);
  a.ws.part_dn = reinterpret_cast<float*>(b + p.o_pdn);
  a.ws.tk_cap = p.t_cap * p.k;
  a.S_gu = p.S_gu;
  a.S_dn = p.S_dn;
  const int flags = format & ~0xFF;
  a.mfma_min = (flags & DQG_PATH_FORCE_GEMV) ? INT_MAX
               : (flags & DQG_PATH_FORCE_MFMA) ? 1
                                               : kMfmaMinTokens;
  return a;
}

// matrix-core tile height of the expert kernels: none when no expert can reach mfma_min
// Matrix-core tiles per pass of a hot expert: one 16-row tile (an expert with more tokens
// takes more passes, whose weight re-reads mostly hit L2); a second tile would raise the
// register count of the combined kernel, and with it lower the occupancy of every expert.
int mfma_tiles(const MoeArgs& a) { return a.mfma_min > a.T ? 0 : 1; }

bool use_fused(int T, int H, int I, int E, int k, int format) {
  return E <= 512 && dqg::fused_supported_t(T, H, I, k, format & 0xFF) &&
         !(format & DQG_PATH_NO_FUSED);
}

// logits == nullptr: the router units compute them from wr (fused_router_supported(E, T))
int run_fused(const MoePlan& p, const uint16_t* x, const float* logits, const uint16_t* wr,
              float* logits_out, const uint8_t* wgu, const uint16_t* sgu, const uint8_t* wd,
              const uint16_t* sd, int group, int format, const uint16_t* res, uint16_t* out,
              int32_t* ids_out, float* w_out, void* ws, hipStream_t st,
              const uint8_t* efmt = nullptr, const uint16_t* cb = nullptr) {
  dqg::FusedArgs f{};
  f.efmt = efmt;
  f.cb = cb;
  f.x = x; f.logits = logits; f.H = p.H; f.I = p.I; f.E = p.E; f.k = p.k; f.group = group;
  f.wr = logits ? nullptr : wr;
  f.logits_out = logits ? nullptr : logits_out;
  f.fmt = format & 0xFF;
  f.wgu = wgu; f.sgu = sgu; f.wd = wd; f.sd = sd; f.res = res; f.out = out;
  f.ids_out = ids_out; f.w_out = w_out;
  char* b = static_cast<char*>(ws);
  f.err = reinterpret_cast<int*>(b + p.o_err);
  dqg::fused_layout(f, b + p.o_fx, p.H, p.I, p.E, p.k, p.T, f.wr != nullptr);
  return dqg::launch_fused_layer(f, st) == hipSuccess ? DQG_OK : DQG_ERR_HIP;
}

int run_moe(MoeArgs& a, const MoePlan& p, const float* logits, hipStream_t st) {
  hipError_t e = dqg::launch_schedule(a, logits, st);
  if (e != hipSuccess) return DQG_ERR_HIP;
  e = dqg::launch_moe_experts(a, p.A, mfma_tiles(a), st);
  if (e != hipSuccess) return DQG_ERR_HIP;
  return DQG_OK;
}

// GEMV workspace: split partials [S_max][t_cap][N], zero between calls (the finishing
// workgroups clear them); t_cap = the largest T whose layout fits the caller's bytes.
struct GemvPlan {
  int tiles, S, mt, t_cap, s_max;
  size_t total;
};

void gemv_layout(GemvPlan& g, int K, int N, int t_cap) {
  g.t_cap = t_cap;
  const long long fit = ((1LL << 31) - 1) / std::max(1LL, 4LL * t_cap * N);
  g.s_max = (int)std::max(1LL, std::min<long long>(
                                   std::min((K / 32 + 7) / 8, dqg::ex_max_split_gemv()), fit));
  // [error word, 256 bytes][partials]
  g.total = g.s_max > 1 ? 256 + up256(sizeof(float) * (size_t)g.s_max * t_cap * N) : 0;
}

GemvPlan plan_gemv(int T, int K, int N, size_t ws_bytes = 0) {
  GemvPlan g{};
  g.tiles = (N + 127) / 128;
  g.mt = (T <= kGemvTokMaxTokens) ? 0 : (T <= 16 ? 1 : 2);
  gemv_layout(g, K, N, T);
  if (ws_bytes > g.total && g.total > 0) {
    int lo = T, hi = 4096;
    while (lo < hi) {
      const int mid = lo + (hi - lo + 1) / 2;
      GemvPlan q = g;
      gemv_layout(q, K, N, mid);
      if (q.total <= ws_bytes) lo = mid; else hi = mid - 1;
    }
    gemv_layout(g, K, N, lo);
  }
  // 16 blocks (two batches) per workgroup: measured best for N = 256 .. 34816, T = 1 and 4
  // (8 or 4 blocks: more partial traffic and finishers; 32 or 64: too few workgroups)
  g.S = std::min(pick_ex_split(K / 32, 16, dqg::ex_max_split_gemv(), (double)K / 2 * N * 1.06,
                               4.0 * T * N),
                 g.s_max);
  return g;
}

bool gemv_sizes_ok(int T, int K, int N, int group) {
  if (T < 1 || K < 2 || N < 1) return false;
  if (group != 32 && group != 128) return false;
  if (K % group || N % 64) return false;
  if (T > 4096 || K > 65536) return false;
  // buffer views: the packed matrix, its scales, x and the split partials must be
  // addressable with 32-bit byte offsets
  if ((long long)(K / 2) * N >= (1LL << 31) || (long long)T * K * 2 >= (1LL << 31)) return false;
  return true;
}

// ---- allocation-free GEMV: library-owned split-partial scratch -----------------------------
// [error word, 256 bytes][split partials], one copy per GPU (a device global: it is zero-filled
// when the code object loads, and every completed call leaves its partials zero again).
constexpr size_t kScratchPartialBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device.
int scratch_address(void** out);

}  // namespace

static __device__ __align__(256) unsigned char scratch[256 + kScratchPartialBytes];

namespace {
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DQG_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DQG_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DQG_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DQG_OK;
}
}  // namespace

extern "C" {

int dqg_abi_version(void) { return DQG_ABI_VERSION; }

const char* dqg_status_string(int status) {
  switch (status) {
    case DQG_OK: return "DQG_OK";
    case DQG_ERR_INVALID_ARG: return "DQG_ERR_INVALID_ARG";
    case DQG_ERR_UNSUPPORTED: return "DQG_ERR_UNSUPPORTED";
    case DQG_ERR_MISALIGNED: return "DQG_ERR_MISALIGNED";
    case DQG_ERR_WORKSPACE: return "DQG_ERR_WORKSPACE";
    case DQG_ERR_HIP: return "DQG_ERR_HIP";
    default: return "DQG_ERR_UNKNOWN";
  }
}

int topk_route(const float* logits, int T, int E, int k, int32_t* ids, float* weights,
               hipStream_t stream) {
  if (!logits || !ids || !weights) return DQG_ERR_INVALID_ARG;
  if (T < 1 || E < 1 || k < 1 || k > E) return DQG_ERR_INVALID_ARG;
  if (E > kMaxE || k > kMaxK) return DQG_ERR_UNSUPPORTED;
  if (((uintptr_t)logits & 3u) || ((uintptr_t)ids & 3u) || ((uintptr_t)weights & 3u))
    return DQG_ERR_MISALIGNED;
  return dqg::launch_topk(logits, T, E, k, ids, weights, stream) == hipSuccess ? DQG_OK
                                                                                : DQG_ERR_HIP;
}

size_t moe_fp4_ffn_workspace_bytes(int T, int H, int I, int E, int k) {
  if (!moe_sizes_ok(T, H, I, E, k)) return 0;
  const MoePlan p = plan_moe(T, H, I, E, k);
  return p.ok ? p.total : 0;
}

int moe_fp4_ffn(const uint16_t* x, int T, int H, int I, int E, int k, const int32_t* ids,
                const float* weights, const uint8_t* w_gate_up, const uint16_t* s_gate_up,
                const uint8_t* w_down, const uint16_t* s_down, int group, int format,
                const uint16_t* residual, uint16_t* out, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  if (!ids || !weights) return DQG_ERR_INVALID_ARG;
  int rc = check_moe_common(x, T, H, I, E, k, w_gate_up, s_gate_up, w_down, s_down, group,
                            format, residual, out, workspace, workspace_bytes);
  if (rc != DQG_OK) return rc;
  if (((uintptr_t)ids & 3u) || ((uintptr_t)weights & 3u)) return DQG_ERR_MISALIGNED;
  const MoePlan p = plan_moe(T, H, I, E, k, workspace_bytes);
  MoeArgs a = make_moe_args(p, x, w_gate_up, s_gate_up, w_down, s_down, group, format, residual,
                            out, workspace);
  a.ids = ids;
  a.wts = weights;
  return run_moe(a, p, nullptr, stream);
}

int moe_fp4_layer(const uint16_t* x, const float* logits, int T, int H, int I, int E, int k,
                  const uint8_t* w_gate_up, const uint16_t* s_gate_up, const uint8_t* w_down,
                  const uint16_t* s_down, int group, int format, const uint16_t* residual,
                  uint16_t* out, int32_t* ids_out, float* weights_out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  if (!logits) return DQG_ERR_INVALID_ARG;
  int rc = check_moe_common(x, T, H, I, E, k, w_gate_up, s_gate_up, w_down, s_down, group,
                            format, residual, out, workspace, workspace_bytes);
  if (rc != DQG_OK) return rc;
  if (((uintptr_t)logits & 3u) || ((uintptr_t)ids_out & 3u) || ((uintptr_t)weights_out & 3u))
    return DQG_ERR_MISALIGNED;
  const MoePlan p = plan_moe(T, H, I, E, k, workspace_bytes);
  if (use_fused(T, H, I, E, k, format))
    return run_fused(p, x, logits, nullptr, nullptr, w_gate_up, s_gate_up, w_down, s_down, group,
                     format, residual, out, ids_out, weights_out, workspace, stream);
  MoeArgs a = make_moe_args(p, x, w_gate_up, s_gate_up, w_down, s_down, group, format, residual,
                            out, workspace);
  a.ids_w = ids_out ? ids_out : a.ws.ids;
  a.wts_w = weights_out ? weights_out : a.ws.wts;
  a.ids = a.ids_w;
  a.wts = a.wts_w;
  return run_moe(a, p, logits, stream);
}

size_t router_logits_workspace_bytes(int T, int H, int E) {
  if (T < 1 || H < 8 || E < 8 || H % 8 || E % 8 || E > kMaxE || T > kMaxTK) return 0;
  return up256(sizeof(float) * (size_t)dqg::router_splits(H) * T * E);
}

int router_logits(const uint16_t* x, int T, int H, int E, const uint16_t* w_router,
                  float* logits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x || !w_router || !logits) return DQG_ERR_INVALID_ARG;
  if (T < 1 || H < 1 || E < 1) return DQG_ERR_INVALID_ARG;
  const size_t need = router_logits_workspace_bytes(T, H, E);
  if (need == 0) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_router) || ((uintptr_t)logits & 3u))
    return DQG_ERR_MISALIGNED;
  if (!workspace || workspace_bytes < need) return DQG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DQG_ERR_MISALIGNED;
  return dqg::launch_router(x, T, H, w_router, E, static_cast<float*>(workspace), logits,
                            stream) == hipSuccess ? DQG_OK : DQG_ERR_HIP;
}

int moe_fp4_layer_from_hidden(const uint16_t* x, const uint16_t* w_router, int T, int H, int I,
                              int E, int k, const uint8_t* w_gate_up, const uint16_t* s_gate_up,
                              const uint8_t* w_down, const uint16_t* s_down, int group,
                              int format, const uint16_t* residual, uint16_t* out,
                              float* logits_out, int32_t* ids_out, float* weights_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!w_router) return DQG_ERR_INVALID_ARG;
  int rc = check_moe_common(x, T, H, I, E, k, w_gate_up, s_gate_up, w_down, s_down, group,
                            format, residual, out, workspace, workspace_bytes);
  if (rc != DQG_OK) return rc;
  if (E % 8) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(w_router)) return DQG_ERR_MISALIGNED;
  if (((uintptr_t)logits_out & 3u) || ((uintptr_t)ids_out & 3u) || ((uintptr_t)weights_out & 3u))
    return DQG_ERR_MISALIGNED;
  const MoePlan p = plan_moe(T, H, I, E, k, workspace_bytes);
  char* b = static_cast<char*>(workspace);
  if (use_fused(T, H, I, E, k, format) && dqg::fused_router_supported(E, T))
    return run_fused(p, x, nullptr, w_router, logits_out, w_gate_up, s_gate_up, w_down, s_down,
                     group, format, residual, out, ids_out, weights_out, workspace, stream);
  // the router call, then the layer on its logits
  float* lg = logits_out ? logits_out : reinterpret_cast<float*>(b + p.o_rtl);
  if (dqg::launch_router(x, T, H, w_router, E, reinterpret_cast<float*>(b + p.o_rtp), lg,
                         stream) != hipSuccess)
    return DQG_ERR_HIP;
  if (use_fused(T, H, I, E, k, format))
    return run_fused(p, x, lg, nullptr, nullptr, w_gate_up, s_gate_up, w_down, s_down, group,
                     format, residual, out, ids_out, weights_out, workspace, stream);
  MoeArgs a = make_moe_args(p, x, w_gate_up, s_gate_up, w_down, s_down, group, format, residual,
                            out, workspace);
  a.ids_w = ids_out ? ids_out : a.ws.ids;
  a.wts_w = weights_out ? weights_out : a.ws.wts;
  a.ids = a.ids_w;
  a.wts = a.wts_w;
  return run_moe(a, p, lg, stream);
}

int moe_fp4_layer_mixed(const uint16_t* x, const float* logits, int T, int H, int I, int E,
                        int k, const uint8_t* w_gate_up, const uint16_t* s_gate_up,
                        const uint8_t* w_down, const uint16_t* s_down,
                        const uint8_t* expert_formats, const uint16_t* codebooks, int group,
                        int format, const uint16_t* residual, uint16_t* out, int32_t* ids_out,
                        float* weights_out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!logits || !expert_formats) return DQG_ERR_INVALID_ARG;
  int rc = check_moe_common(x, T, H, I, E, k, w_gate_up, s_gate_up, w_down, s_down, group,
                            format, residual, out, workspace, workspace_bytes);
  if (rc != DQG_OK) return rc;
  if ((format & 0xFF) != DQG_FMT_FP4_E2M1) return DQG_ERR_UNSUPPORTED;  // FP4 hot experts
  if (E % 4) return DQG_ERR_UNSUPPORTED;                                // table read as words
  if ((uintptr_t)expert_formats & 3u) return DQG_ERR_MISALIGNED;
  if (codebooks && !aligned16(codebooks)) return DQG_ERR_MISALIGNED;
  if (((uintptr_t)logits & 3u) || ((uintptr_t)ids_out & 3u) || ((uintptr_t)weights_out & 3u))
    return DQG_ERR_MISALIGNED;
  const MoePlan p = plan_moe(T, H, I, E, k, workspace_bytes);
  // the single launch stages the codebooks of at most two slots per down unit (256 rows):
  // with FE-XC experts it needs I / 2 >= 256
  if (use_fused(T, H, I, E, k, format) && !(codebooks && I / 2 < 256))
    return run_fused(p, x, logits, nullptr, nullptr, w_gate_up, s_gate_up, w_down, s_down,
                     group, format, residual, out, ids_out, weights_out, workspace, stream,
                     expert_formats, codebooks);
  MoeArgs a = make_moe_args(p, x, w_gate_up, s_gate_up, w_down, s_down, group, format, residual,
                            out, workspace);
  a.efmt = expert_formats;
  a.cb = codebooks;
  a.ids_w = ids_out ? ids_out : a.ws.ids;
  a.wts_w = weights_out ? weights_out : a.ws.wts;
  a.ids = a.ids_w;
  a.wts = a.wts_w;
  return run_moe(a, p, logits, stream);
}

size_t packed_gemv_int4_workspace_bytes(int T, int K, int N, int group) {
  if (!gemv_sizes_ok(T, K, N, group)) return 0;
  return plan_gemv(T, K, N).total;
}

int packed_gemv_int4(const uint16_t* x, int T, int K, int N, const uint8_t* w,
                     const uint16_t* s, int group, uint16_t* y, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  if (!x || !w || !s || !y) return DQG_ERR_INVALID_ARG;
  if (T < 1 || K < 1 || N < 1) return DQG_ERR_INVALID_ARG;
  if (!gemv_sizes_ok(T, K, N, group)) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(y)) return DQG_ERR_MISALIGNED;
  GemvPlan gp = plan_gemv(T, K, N, workspace ? workspace_bytes : 0);
  if (gp.S > 1 && (!workspace || workspace_bytes < gp.total)) {
    if (workspace) return DQG_ERR_WORKSPACE;
    gp.S = 1;  // no workspace: no K split
  }
  if (workspace && !aligned16(workspace)) return DQG_ERR_MISALIGNED;
  GemvArgs g{};
  g.x = x; g.T = T; g.K = K; g.N = N; g.group = group; g.w = w; g.s = s; g.y = y; g.S = gp.S;
  g.t_cap = gp.t_cap;
  if (gp.S > 1) {
    g.err = static_cast<int*>(workspace);
    g.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 256);
  }
  return dqg::launch_gemv_ex(g, gp.mt, stream) == hipSuccess ? DQG_OK : DQG_ERR_HIP;
}

int packed_gemv_int4_noalloc(const uint16_t* x, int T, int K, int N, const uint8_t* w,
                             const uint16_t* s, int group, uint16_t* y, int* status,
                             hipStream_t stream) {
  if (!x || !w || !s || !y) return DQG_ERR_INVALID_ARG;
  if (T < 1 || K < 1 || N < 1) return DQG_ERR_INVALID_ARG;
  if (!gemv_sizes_ok(T, K, N, group)) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(y)) return DQG_ERR_MISALIGNED;
  if ((uintptr_t)status & 3u) return DQG_ERR_MISALIGNED;
  // the layout of a workspace sized exactly for T tokens; its partials must fit the scratch
  const GemvPlan gp = plan_gemv(T, K, N);
  if (gp.S > 1 && gp.total > 256 + kScratchPartialBytes) return DQG_ERR_WORKSPACE;
  if (stream) {  // the scratch address below is the current device's: the stream must be on it
    int sdev = -1, cur = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || hipGetDevice(&cur) != hipSuccess)
      return DQG_ERR_HIP;
    if (sdev != cur) return DQG_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc != DQG_OK) return rc;
  GemvArgs g{};
  g.x = x; g.T = T; g.K = K; g.N = N; g.group = group; g.w = w; g.s = s; g.y = y; g.S = gp.S;
  g.t_cap = gp.t_cap;
  if (gp.S > 1) {
    g.err = status ? status : static_cast<int*>(ws);
    g.part = reinterpret_cast<float*>(static_cast<char*>(ws) + 256);
  }
  return dqg::launch_gemv_ex(g, gp.mt, stream) == hipSuccess ? DQG_OK : DQG_ERR_HIP;
}

int packed_gemv_int4_prepack_sizes(int K, int N, int group, size_t* w_bytes, size_t* s_bytes) {
  if (!w_bytes || !s_bytes) return DQG_ERR_INVALID_ARG;
  if (K < 1 || N < 1) return DQG_ERR_INVALID_ARG;
  if (!gemv_sizes_ok(1, K, N, group)) return DQG_ERR_UNSUPPORTED;
  const size_t tiles = (size_t)(N + 127) / 128;
  *w_bytes = tiles * (size_t)K * 64;
  *s_bytes = tiles * (size_t)(K / group) * 256;
  return DQG_OK;
}

int packed_gemv_int4_prepack(const uint8_t* w, const uint16_t* s, int K, int N, int group,
                             uint8_t* w_tiled, uint16_t* s_tiled, hipStream_t stream) {
  if (!w || !s || !w_tiled || !s_tiled) return DQG_ERR_INVALID_ARG;
  if (K < 1 || N < 1) return DQG_ERR_INVALID_ARG;
  if (!gemv_sizes_ok(1, K, N, group)) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(w) || !aligned16(s) || !aligned16(w_tiled) || !aligned16(s_tiled))
    return DQG_ERR_MISALIGNED;
  return dqg::launch_gemv_prepack(w, s, K, N, group, w_tiled, s_tiled, stream) == hipSuccess
             ? DQG_OK
             : DQG_ERR_HIP;
}

int packed_gemv_int4_tiled(const uint16_t* x, int T, int K, int N, const uint8_t* w_tiled,
                           const uint16_t* s_tiled, int group, uint16_t* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!x || !w_tiled || !s_tiled || !y) return DQG_ERR_INVALID_ARG;
  if (T < 1 || K < 1 || N < 1) return DQG_ERR_INVALID_ARG;
  if (T > 4 || !gemv_sizes_ok(T, K, N, group)) return DQG_ERR_UNSUPPORTED;
  // the prepacked weights are addressed with 32-bit byte offsets
  if ((long long)((N + 127) / 128) * K * 64 >= (1LL << 31)) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_tiled) || !aligned16(s_tiled) || !aligned16(y))
    return DQG_ERR_MISALIGNED;
  // the workspace of packed_gemv_int4 for T tokens (the same split partials and error word)
  GemvPlan gp = plan_gemv(T, K, N, workspace ? workspace_bytes : 0);

  if (gp.S > 1 && (!workspace || workspace_bytes < gp.total)) {
    if (workspace) return DQG_ERR_WORKSPACE;
    gp.S = 1;  // no workspace: no K split
  }
  if (workspace && !aligned16(workspace)) return DQG_ERR_MISALIGNED;
  GemvArgs g{};
  g.x = x; g.T = T; g.K = K; g.N = N; g.group = group; g.w = w_tiled; g.s = s_tiled; g.y = y;
  g.S = gp.S; g.t_cap = gp.t_cap;
  if (gp.S > 1) {
    g.err = static_cast<int*>(workspace);
    g.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 256);
  }
  return dqg::launch_gemv_tiled(g, stream) == hipSuccess ? DQG_OK : DQG_ERR_HIP;
}

int packed_dequant_f32(const uint8_t* w, const uint16_t* s, int K, int N, int group,
                       int format, float* out, hipStream_t stream) {
  if (!w || !s || !out) return DQG_ERR_INVALID_ARG;
  if (K < 2 || N < 1) return DQG_ERR_INVALID_ARG;
  if (format != DQG_FMT_INT4 && format != DQG_FMT_FP4_E2M1 && format != DQG_FMT_FP8_E4M3)
    return DQG_ERR_UNSUPPORTED;
  if (group != 32 && group != 128) return DQG_ERR_UNSUPPORTED;
  if (K % group || N % 16) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(w) || !aligned16(s) || !aligned16(out)) return DQG_ERR_MISALIGNED;
  return dqg::launch_dequant(w, s, K, N, group, format, out, stream) == hipSuccess ? DQG_OK
                                                                                     : DQG_ERR_HIP;
}

int dqg_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!p || !sink || bytes == 0) return DQG_ERR_INVALID_ARG;
  if (bytes % 16 || bytes / 16 / 4096 >= (size_t)1 << 31) return DQG_ERR_UNSUPPORTED;
  if (!aligned16(p) || ((uintptr_t)sink & 3u)) return DQG_ERR_MISALIGNED;
  return dqg::launch_stream_read(p, bytes, sink, stream) == hipSuccess ? DQG_OK : DQG_ERR_HIP;
}

}  // extern "C"
