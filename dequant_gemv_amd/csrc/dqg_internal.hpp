// Internal host/device structures shared by the kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dqg {

// Device-side views into the caller's MoE workspace (laid out by plan_moe).
struct MoeWs {
  int* err;             // [1]  sticky error word (1: an expert id outside [0, E) was seen)
  int* n_active;        // [1]  number of distinct valid experts this call
  int4* rec;            // [A]  per active index: {expert, first slot position, slots, 0}
  int* slot_list;       // [T*k] slots (t*k + j) grouped by expert, ascending within an expert
  int* nvalid;          // [T]  number of valid slots of token t
  int32_t* ids;         // [T*k] routing written by the layer call when the caller passes none
  float* wts;           // [T*k]
  uint16_t* hop;        // [T*k, I] SiLU(gate) * up as 16-bit operands (bf16 / fp16)
  float* part_gu;       // [S_gu_max][tk_cap][2I] gate/up split partials (zero between calls)
  float* part_dn;       // [S_dn_max][tk_cap][H]  down split partials per slot (zero between calls)
  int tk_cap;           // slots of the workspace's capacity: the partials' split stride
};

struct MoeArgs {
  const uint16_t* x;
  int T, H, I, E, k, group, fmt;
  const int32_t* ids;   // routing read by the expert kernels
  const float* wts;
  int32_t* ids_w;       // routing written by the schedule kernel (layer call)
  float* wts_w;
  const uint8_t* wgu;
  const uint16_t* sgu;
  const uint8_t* wd;
  const uint16_t* sd;
  const uint16_t* res;
  uint16_t* out;
  MoeWs ws;
  int S_gu, S_dn;
  int mfma_min;         // experts with at least this many tokens use the MFMA tiles
  int combine;          // this down launch also runs the per-token combine (the last one)
  const uint8_t* efmt;  // per-expert formats [E] of a mixed FP4 layer, or null
  const uint16_t* cb;   // FE-XC codebooks bf16 [E][2 (gate_up, down)][2][256][8], or null
};

struct GemvArgs {
  const uint16_t* x;
  int T, K, N, group;
  const uint8_t* w;
  const uint16_t* s;
  uint16_t* y;
  float* part;          // [S_max, t_cap, N] split partials (S > 1; zero between calls)
  int t_cap;            // tokens of the workspace's capacity: the partials' split stride
  int S;
  int wb;               // blocks (32 K) per K split of the one-token kernel (set by the launcher)
  int* err;             // error word (bit 1: a wait gave up), may be null
};

// Single-launch layer for T <= FX_MAX_T (routing + expert FFN + combine); see dqg_fused.hip.
struct FusedArgs {
  const uint16_t* x;
  const float* logits;  // fp32 [T, E], or null when the router units compute them
  const uint16_t* wr;   // router weight bf16 [H, E] (router units), or null
  float* logits_out;    // optional fp32 [T, E] copy of the router's logits (may be null)
  const uint8_t* efmt;  // per-expert formats [E] of a mixed FP4 layer (FMT_INT2 entries), or null
  const uint16_t* cb;   // FE-XC codebooks bf16 [E][2 (gate_up, down)][2][256][8], or null
  float* rpart;         // [2][rs][T][E] router partial rows, two copies
  int n_r, rs;          // router units (the first n_r workgroups) and row splits
  int H, I, E, k, group, fmt;
  const uint8_t* wgu;
  const uint16_t* sgu;
  const uint8_t* wd;
  const uint16_t* sd;
  const uint16_t* res;
  uint16_t* out;
  int32_t* ids_out;     // optional routing outputs (may be null)
  float* w_out;
  float* gpart;         // [2][k * I/128 * ks][256] gate/up partial rows, two copies
  float* ypart;         // [2][H/128 * n_chunks][128] output partial rows, two copies
  unsigned int* calls;  // call counter: every call adds 2^20 in total (parity source)
  unsigned int* rcalls; // router call counter: calls with router units add 2^20
  int* err;
  int n_a, n_b, n_chunks, ks, n_mt;
  int T, chunks_per_token;  // tokens (1 .. FX_MAX_T) and down chunks per token
  int hold_down;        // down units load their weights only once gate/up results appear
  int dr;               // down byte rows per lane: 8 (256-row chunks) or 4 (128-row chunks)
};
// tokens of the single-launch layer, at most (measured at the 128-expert shape against the
// multi-launch path: T = 5 30 vs 45 us, T = 8 46 vs 55 us, T = 12 65 vs 68 us, T = 16 84 vs 78 us)
constexpr int FX_MAX_T = 8;
bool fused_supported(int H, int I, int k);
bool fused_supported_t(int T, int H, int I, int k, int fmt);
bool fused_router_supported(int E, int T);
// exchange regions for T = 1 .. t_max (one per token count)
size_t fused_ws_bytes(int H, int I, int E, int k, int t_max);
// lays out the call's region; with_router: the first workgroups compute the logits
void fused_layout(FusedArgs& f, void* ws, int H, int I, int E, int k, int T, bool with_router);
hipError_t launch_fused_layer(const FusedArgs& f, hipStream_t st);

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* wts,
                       hipStream_t st);
hipError_t launch_schedule(const MoeArgs& a, const float* logits, hipStream_t st);
// gate_up + down expert kernels, one launch each; mt = 0: vector-ALU tiles only, mt = 1:
// 16-token matrix-core tiles for experts with at least mfma_min tokens and vector-ALU
// passes for the others, in the same launch
hipError_t launch_moe_experts(const MoeArgs& a, int A, int mt, hipStream_t st);
int ex_max_split();
constexpr unsigned EX_SPIN_LIMIT = 1u << 16;  // polling rounds before a wait gives up
// dense INT4 GEMV; mt = 0: vector-ALU tiles (T = 1), 1 or 2: matrix-core tiles
hipError_t launch_gemv_ex(const GemvArgs& g, int mt, hipStream_t st);
// dense INT4 GEMV on the prepacked layout (1 <= T <= 4, vector ALUs), g.S K splits
hipError_t launch_gemv_tiled(const GemvArgs& g, hipStream_t st);
// rearranges a [K/2, N] INT4 matrix and its [K/G, N] scales into the prepacked layout
hipError_t launch_gemv_prepack(const uint8_t* w, const uint16_t* s, int K, int N, int group,
                               uint8_t* wt, uint16_t* st_, hipStream_t st);
int ex_max_split_gemv();
hipError_t launch_dequant(const uint8_t* w, const uint16_t* s, int K, int N, int group, int fmt,
                          float* out, hipStream_t st);
// measurement aid: read `bytes` (a multiple of 16) from p once (see stream_read_kernel)
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t st);
// router logits[T, E] = x W_r through partials [router_splits(H)][T][E] (see router_unit)
int router_splits(int H);
hipError_t launch_router(const uint16_t* x, int T, int H, const uint16_t* wr, int E, float* part,
                         float* logits, hipStream_t st);

}  // namespace dqg
