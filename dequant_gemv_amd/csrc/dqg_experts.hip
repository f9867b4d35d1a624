// Expert kernels of the multi-launch MoE path (any T): gate_up + SiLU*up, and down + the
// top-k combine, over the device-built schedule (active experts, their slot lists).
//
// FireEcho page, "The Goliath Kernel: Why It's Fast": the packed bytes of all experts sit
// in one buffer indexed by expert ids read on the device, and are dequantized in registers
// inside the tile loop; "Speed Optimization History": one multi-expert kernel with a fused
// gate_up projection.
//
// Work unit: a workgroup (4 waves) owns one expert, 128 output columns and a range of
// "blocks" (16 byte rows = 32 K indices, never straddling a scale group).  In every wave,
// lane l reads the 8 columns col + 8 (l % 16) .. +7 of byte rows 16 b + 4 (l / 16) + j
// (j = 0..3) of a block b: 16 lanes cover a full 128-byte row segment, 4 lanes groups of
// 4 rows cover the block.  Each byte becomes the 16-bit pair (W[2r], W[2r+1]) (bf16 for
// FP4 via the gfx950 FP4 convert, fp16 for INT4), so a lane holds, per column, the 8
// weights of K = 32 b + 8 (l / 16) .. +7 -- exactly the K slice that a 16x16x32 MFMA B
// operand lane holds.  The activation operand of a token is the matching 16 bytes of the
// token's row (bf16 x, or h rounded to bf16 / fp16).
//
// Experts with at least `mfma_min` tokens run the matrix-core body: per block and column
// i, one v_mfma_f32_16x16x32 (bf16 or f16) per 16 tokens, the group scale applied to its
// fp32 result.  The others run the vector-ALU body: per token and column, four dot2
// instructions, the operands staged in LDS once per pass.  Both bodies produce the same
// per-(token, column) partial sums, reduced over lane groups and waves in LDS; K splits
// of one tile are summed by the last workgroup to finish (a completion counter), and the
// k slots of a token by the workgroup that completes that token's output tile, in slot
// order, so every result has a fixed summation order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqg_device.hpp"
#include "dqg_internal.hpp"

namespace dqg {

constexpr int EX_THREADS = 256;
constexpr int EX_VT = 4;          // tokens per vector-ALU pass
constexpr int EX_LDS = 8192;      // floats of LDS: the operand window, then the reductions
constexpr int EX_MAX_SPLIT = 64;  // K splits of gate_up, at most
constexpr int EX_MAX_SPLIT_GEMV = 64;  // K splits of the GEMV, at most
constexpr int EX_CPOL_SC1 = 16;   // cache policy: agent-coherent access
// cache policy: non-temporal (the dense GEMV reads each weight once per call; streaming them
// leaves L2 to the partial rows and the code of the split finishers)
constexpr int EX_STREAM = 2;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---- schedule entries, clamped ------------------------------------------------------------
// Whatever the workspace holds, no index derived from it leaves the call's buffers.
__device__ __forceinline__ bool expert_record(const MoeArgs& a, int act, int* beg, int* cnt,
                                              int* e) {
  const int TK = a.T * a.k;
  const int4 r = a.ws.rec[act];
  *e = r.x;
  *beg = min(max(r.y, 0), TK);
  *cnt = min(max(r.z, 0), TK - *beg);
  return r.x >= 0 && r.x < a.E && *cnt > 0;
}
// slot at position i of the slot list, or -1 when it is not a slot of this call
__device__ __forceinline__ int slot_at(const MoeArgs& a, int i) {
  const int s = a.ws.slot_list[i];
  return ((unsigned)s < (unsigned)(a.T * a.k)) ? s : -1;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ex_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7FFFFFFF, 0x00020000);
}
// agent-coherent 16-byte store / load at byte offset `off` of a buffer
__device__ __forceinline__ void st4_sc1(__amdgpu_buffer_rsrc_t r, int off, float4 v) {
  const u32x4_t d = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                     __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, EX_CPOL_SC1);
}
__device__ __forceinline__ float4 ld4_sc1_raw(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, EX_CPOL_SC1);
  return make_float4(__uint_as_float(d.x), __uint_as_float(d.y), __uint_as_float(d.z),
                     __uint_as_float(d.w));
}
// Split partials are published with the bit pattern 0 reserved for "not written yet"
// (+0.0 is stored as -0.0, which sums identically); readers poll until no component is 0,
// and clear the values back to 0 after use.
__device__ __forceinline__ float pub1(float v) {
  return __float_as_uint(v) == 0u ? __uint_as_float(0x80000000u) : v;
}
__device__ __forceinline__ float4 pub4(float4 v) {
  return make_float4(pub1(v.x), pub1(v.y), pub1(v.z), pub1(v.w));
}
__device__ __forceinline__ bool ready4(float4 v) {
  return (__float_as_uint(v.x) != 0u) & (__float_as_uint(v.y) != 0u) &
         (__float_as_uint(v.z) != 0u) & (__float_as_uint(v.w) != 0u);
}
// Waits until the n (<= 16) floats at byte offsets off[i] are all published (bounded:
// returns false when the wait gives up), then clears them.  Every one of the 16 offsets
// must name a published value of this wait: callers fill those past n with repeats of
// earlier ones, so that the loads, checks and clears run without branches (this runs once,
// cold, at the end of a dependency chain, where code size is time).
__device__ __forceinline__ bool take16(__amdgpu_buffer_rsrc_t r, const int (&off)[16], int n,
                                       float (&v)[16]) {
  bool ok = false;
  for (unsigned spin = 0; spin < EX_SPIN_LIMIT; ++spin) {
    asm volatile("" ::: "memory");  // every round reloads the values
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off[i], 0, EX_CPOL_SC1));
    bool all = true;
#pragma unroll
    for (int i = 0; i < 16; ++i) all = all && (__float_as_uint(v[i]) != 0u);
    if (all) {
      ok = true;
      break;
    }
    __builtin_amdgcn_s_sleep(8);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, r, off[i], 0, EX_CPOL_SC1);
  return ok;
}

// One lane of the workgroup polls the published float4 at byte offset `off` (bounded,
// with a backoff) while the others wait at the barrier: waiting workgroups then add almost
// no memory traffic.  The values themselves are read afterwards with take16.
__device__ __forceinline__ void wg_wait_published(__amdgpu_buffer_rsrc_t r, int off) {
  if (threadIdx.x == 0) {
    for (unsigned spin = 0; spin < EX_SPIN_LIMIT; ++spin) {
      if (ready4(ld4_sc1_raw(r, off))) break;
      __builtin_amdgcn_s_sleep(8);
    }
  }
  __syncthreads();
}

__device__ __forceinline__ float4 f4_add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ---- weights of one block for one lane ----------------------------------------------------
struct WBlock {
  uint2 w[4];  // byte rows 16 b + 4 kg + j, 8 columns
  uint4 s;     // the 8 columns' bf16 scales of the block's group
};

// Buffer views of one expert's packed matrix and scales.  Loads go through buffer
// instructions: a uniform descriptor, a 32-bit lane offset, the row stride as a uniform
// offset.  A request marked out of range uses an offset past the descriptor's size, so the
// hardware returns zeros without touching memory; every load is issued unconditionally
// and the compiler can count outstanding loads exactly.
struct ExpertView {
  __amdgpu_buffer_rsrc_t w, s;
  int ld;      // bytes per byte row (= columns)
  int group;
};
constexpr int EX_OOB = 0x7FFFFF00;  // an offset past every descriptor's size

__device__ __forceinline__ __amdgpu_buffer_rsrc_t view_rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

template <int WAUX>
__device__ __forceinline__ void load_wblock(const ExpertView& v, int blk, int kg, int col,
                                            bool ok, WBlock& o) {
  const int wo = ok ? (16 * blk + 4 * kg) * v.ld + col : EX_OOB;
  const int so = ok ? (((32 * blk) / v.group) * v.ld + col) * 2 : EX_OOB;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x2_t d = __builtin_amdgcn_raw_buffer_load_b64(v.w, wo, j * v.ld, WAUX);
    o.w[j] = make_uint2(d.x, d.y);
  }
  const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(v.s, so, 0, WAUX);
  o.s = make_uint4(d.x, d.y, d.z, d.w);
}

// byte B of d -> exact 16-bit pair (W[2r], W[2r+1]): bf16 for FP4, fp16 for INT4
template <int FMT, int B>
__device__ __forceinline__ uint32_t dec_pair(uint32_t d) {
  if constexpr (FMT == FMT_FP4) {
    return __builtin_bit_cast(uint32_t, fp4_pair_bf16<B>(d));
  } else {
    const f16x2_t bias = {(_Float16)(-INT4_F16_BIAS_LO), (_Float16)(-INT4_F16_BIAS_HI)};
    return __builtin_bit_cast(uint32_t, int4_pair_f16_biased<B>(d) + bias);
  }
}

// the lane's 4 pairs of column I (byte rows j = 0..3 of the block)
template <int FMT, int I>
__device__ __forceinline__ u32x4_t decode_col(const WBlock& b) {
  const uint32_t d0 = (I < 4) ? b.w[0].x : b.w[0].y, d1 = (I < 4) ? b.w[1].x : b.w[1].y;
  const uint32_t d2 = (I < 4) ? b.w[2].x : b.w[2].y, d3 = (I < 4) ? b.w[3].x : b.w[3].y;
  return u32x4_t{dec_pair<FMT, I % 4>(d0), dec_pair<FMT, I % 4>(d1), dec_pair<FMT, I % 4>(d2),
                 dec_pair<FMT, I % 4>(d3)};
}

__device__ __forceinline__ void scales8(const uint4& s, float (&sf)[8]) {
  sf[0] = bf16_lo(s.x); sf[1] = bf16_hi(s.x);
  sf[2] = bf16_lo(s.y); sf[3] = bf16_hi(s.y);
  sf[4] = bf16_lo(s.z); sf[5] = bf16_hi(s.z);
  sf[6] = bf16_lo(s.w); sf[7] = bf16_hi(s.w);
}

template <int FMT>
__device__ __forceinline__ float dot2p(uint32_t p, uint32_t x, float c) {
  if constexpr (FMT == FMT_FP4)
    return dot2_bf16(__builtin_bit_cast(bf16x2_t, p), __builtin_bit_cast(bf16x2_t, x), c);
  else
    return dot2_f16(__builtin_bit_cast(f16x2_t, p), __builtin_bit_cast(f16x2_t, x), c);
}

// ---- activation operands: 8 consecutive K values of one token as 16-bit values ------------
__device__ __forceinline__ uint32_t bf16pair_to_f16pair(uint32_t v) {
  const f16x2_t h = {(_Float16)bf16_lo(v), (_Float16)bf16_hi(v)};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t f32pair_to_bf16pair(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
__device__ __forceinline__ uint32_t f32pair_to_f16pair(float lo, float hi) {
  const f16x2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}
// from a bf16 row: the q-th group of 8 values (K = 8 q .. 8 q + 7)
template <int FMT>
__device__ __forceinline__ uint4 op_from_bf16(const uint16_t* row, int q8) {
  uint4 v = reinterpret_cast<const uint4*>(row)[q8];
  if constexpr (FMT == FMT_INT4) {
    v.x = bf16pair_to_f16pair(v.x);
    v.y = bf16pair_to_f16pair(v.y);
    v.z = bf16pair_to_f16pair(v.z);
    v.w = bf16pair_to_f16pair(v.w);
  }
  return v;
}
// from an fp32 row (h): rounded to bf16 (FP4) or fp16 (INT4), nearest even
template <int FMT>
__device__ __forceinline__ uint4 op_from_f32(const float* row, int q8) {
  const float4 a = reinterpret_cast<const float4*>(row)[2 * q8];
  const float4 b = reinterpret_cast<const float4*>(row)[2 * q8 + 1];
  if constexpr (FMT == FMT_FP4)
    return make_uint4(f32pair_to_bf16pair(a.x, a.y), f32pair_to_bf16pair(a.z, a.w),
                      f32pair_to_bf16pair(b.x, b.y), f32pair_to_bf16pair(b.z, b.w));
  else
    return make_uint4(f32pair_to_f16pair(a.x, a.y), f32pair_to_f16pair(a.z, a.w),
                      f32pair_to_f16pair(b.x, b.y), f32pair_to_f16pair(b.z, b.w));
}

template <int FMT>
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint4& a, const u32x4_t& b, f32x4_t c) {
  const u32x4_t av = {a.x, a.y, a.z, a.w};
  if constexpr (FMT == FMT_FP4)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// ---- the pipelined stream over one expert matrix ---------------------------------------------
// Operand source of a phase: gate_up reads bf16 x rows (token = slot / k), down reads the
// 16-bit h operands written by gate_up (by slot); both through a buffer descriptor.
struct OpSrc {
  __amdgpu_buffer_rsrc_t r;
  bool from_x;         // x rows (bf16; converted to fp16 for INT4) or h rows (ready)
  int row_bytes;       // 2 H or 2 I
  int k;
};
template <int FMT>
__device__ __forceinline__ uint4 load_op(const OpSrc& src, int slot, int q8) {
  const int row = src.from_x ? slot / src.k : slot;
  const int off = slot < 0 ? EX_OOB : row * src.row_bytes + 16 * q8;
  const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(src.r, off, 0, 0);
  uint4 v = make_uint4(d.x, d.y, d.z, d.w);
  if constexpr (FMT == FMT_INT4) {
    if (src.from_x) {
      v.x = bf16pair_to_f16pair(v.x);
      v.y = bf16pair_to_f16pair(v.y);
      v.z = bf16pair_to_f16pair(v.z);
      v.w = bf16pair_to_f16pair(v.w);
    }
  }
  return v;
}

constexpr int EX_G = 8;                       // blocks per group (all waves together), at most
constexpr int EX_MAXCH = 32;                  // tokens per pass, at most
constexpr int EX_WROW = EX_G * 4 + 1;         // uint4 per token row of an operand window
constexpr int EX_WIN = EX_MAXCH * EX_WROW;    // uint4 per window
static_assert(EX_WIN * 4 <= EX_LDS, "the operand window fits the LDS buffer");

// LDS floats of a kernel instantiation: the larger of its operand window and its
// reduction buffer (16 partials x min(VT, 4) tokens x 128 columns for the vector-ALU
// tiles, 4 x 16 tokens x 128 columns for the matrix-core tiles)
constexpr int ex_lds_floats(int MT, int VT) {
  return MT > 0 ? EX_LDS : (16 * (VT < 4 ? VT : 4) * 128 > VT * EX_WROW * 4
                                ? 16 * (VT < 4 ? VT : 4) * 128
                                : VT * EX_WROW * 4);
}

enum { BODY_VALU = 0, BODY_MFMA = 1 };

template <int BODY, int MT>
struct Acc;
template <int VT>
struct Acc<BODY_VALU, VT> {  // VALU: up to VT tokens per pass
  float v[VT][8];
};
template <int MT>
struct Acc<BODY_MFMA, MT> {
  f32x4_t v[MT][8];
};

// The lane's weights of one group: RBW blocks (b = g0 + off + step * r); blocks past b1
// (and columns past the tile) load as zero.  WAUX: the loads' cache policy (EX_STREAM for
// weights that are read once per call).
template <int RBW, int WAUX = 0>
__device__ __forceinline__ void load_group(const ExpertView& v, int g0, int off, int step,
                                           int b1, int kg, int col, bool col_ok,
                                           WBlock (&wb)[RBW]) {
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    const int b = g0 + off + step * r;
    load_wblock<WAUX>(v, b, kg, col, col_ok && b < b1, wb[r]);
  }
}

// Operand window of group g0 (GB blocks) for NTOK token rows: the thread's share of the
// global loads, then (after the compute) its LDS stores.  Rows past the pass's tokens
// and blocks past b1 are zero.
template <int FMT, int GB, int NTOK>
struct Window {
  static constexpr int NST = (NTOK * GB * 4 + EX_THREADS - 1) / EX_THREADS;
  uint4 st[NST];
  __device__ __forceinline__ void load(const OpSrc& src, const int* s_slot, int nch, int g0,
                                       int b1) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int i = threadIdx.x + EX_THREADS * u;
      const int t = i / (GB * 4), r = i - t * (GB * 4);
      const int b = g0 + (r >> 2);
      const bool ok = t < nch && b < b1;
      const int slot = ok ? s_slot[min(t, EX_MAXCH - 1)] : -1;
      st[u] = load_op<FMT>(src, slot, 4 * b + (r & 3));
    }
  }
  __device__ __forceinline__ void store(uint4* win) const {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int i = threadIdx.x + EX_THREADS * u;
      const int t = i / (GB * 4), r = i - t * (GB * 4);
      if (t < NTOK) win[t * EX_WROW + r] = st[u];
    }
  }
};

// The vector-ALU tiles keep INT4 pairs biased, (1024 + lo, 64 + hi): the bias
// 1032 x[2r] + 72 x[2r+1] of the lane's rows is removed once per token and block (corr).
template <int FMT, int I>
__device__ __forceinline__ u32x4_t decode_col_valu(const WBlock& b) {
  if constexpr (FMT == FMT_FP4) {
    return decode_col<FMT, I>(b);
  } else {
    const uint32_t d0 = (I < 4) ? b.w[0].x : b.w[0].y, d1 = (I < 4) ? b.w[1].x : b.w[1].y;
    const uint32_t d2 = (I < 4) ? b.w[2].x : b.w[2].y, d3 = (I < 4) ? b.w[3].x : b.w[3].y;
    return u32x4_t{__builtin_bit_cast(uint32_t, int4_pair_f16_biased<I % 4>(d0)),
                   __builtin_bit_cast(uint32_t, int4_pair_f16_biased<I % 4>(d1)),
                   __builtin_bit_cast(uint32_t, int4_pair_f16_biased<I % 4>(d2)),
                   __builtin_bit_cast(uint32_t, int4_pair_f16_biased<I % 4>(d3))};
  }
}

template <int FMT, int NTOK, int VT, int I>
__device__ __forceinline__ void valu_col(const WBlock& b, float sc, const uint4 (&op)[NTOK],
                                         const float (&corr)[NTOK], float (&acc)[VT][8]) {
  const u32x4_t P = decode_col_valu<FMT, I>(b);
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    float d = dot2p<FMT>(P.x, op[t].x, corr[t]);
    d = dot2p<FMT>(P.y, op[t].y, d);
    d = dot2p<FMT>(P.z, op[t].z, d);
    d = dot2p<FMT>(P.w, op[t].w, d);
    acc[t][I] = fmaf(sc, d, acc[t][I]);
  }
}
template <int FMT, int MT, int I>
__device__ __forceinline__ void mfma_col(const WBlock& b, float sc, const uint4 (&A)[MT],
                                         f32x4_t (&acc)[MT][8]) {
  const u32x4_t B = decode_col<FMT, I>(b);
  const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const f32x4_t D = mfma_16x16x32<FMT>(A[m], B, zero);
    acc[m][I] += sc * D;
  }
}

// One block: `wrow` = the window entry of this block and lane group for token row 0.
// VALU: NTOK token rows; MFMA: MT tiles of 16 rows (rows past the pass are zero).
template <int FMT, int BODY, int MT, int NTOK>
__device__ __forceinline__ void compute_block(const WBlock& b, const uint4* wrow,
                                              Acc<BODY, MT>& acc) {
  float sf[8];
  scales8(b.s, sf);
  if constexpr (BODY == BODY_VALU) {
    uint4 op[NTOK];
    float corr[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      op[t] = wrow[t * EX_WROW];
      corr[t] = 0.0f;
      if constexpr (FMT == FMT_INT4) {
        const f16x2_t bias = {(_Float16)(-INT4_F16_BIAS_LO), (_Float16)(-INT4_F16_BIAS_HI)};
        const uint32_t bb = __builtin_bit_cast(uint32_t, bias);
        corr[t] = dot2p<FMT>(bb, op[t].x, corr[t]);
        corr[t] = dot2p<FMT>(bb, op[t].y, corr[t]);
        corr[t] = dot2p<FMT>(bb, op[t].z, corr[t]);
        corr[t] = dot2p<FMT>(bb, op[t].w, corr[t]);
      }
    }
    valu_col<FMT, NTOK, MT, 0>(b, sf[0], op, corr, acc.v);
    valu_col<FMT, NTOK, MT, 1>(b, sf[1], op, corr, acc.v);
    valu_col<FMT, NTOK, MT, 2>(b, sf[2], op, corr, acc.v);
    valu_col<FMT, NTOK, MT, 3>(b, sf[3], op, corr, acc.v);
    valu_col<FMT, NTOK, MT, 4>(b, sf[4], op, corr, acc.v);
    valu_col<FMT, NTOK, MT, 5>(b, sf[5], op, corr, acc.v);
    valu_col<FMT, NTOK, MT, 6>(b, sf[6], op, corr, acc.v);
    valu_col<FMT, NTOK, MT, 7>(b, sf[7], op, corr, acc.v);
  } else {
    const int q = threadIdx.x & 15;
    uint4 A[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) A[m] = wrow[(16 * m + q) * EX_WROW];
    mfma_col<FMT, MT, 0>(b, sf[0], A, acc.v);
    mfma_col<FMT, MT, 1>(b, sf[1], A, acc.v);
    mfma_col<FMT, MT, 2>(b, sf[2], A, acc.v);
    mfma_col<FMT, MT, 3>(b, sf[3], A, acc.v);
    mfma_col<FMT, MT, 4>(b, sf[4], A, acc.v);
    mfma_col<FMT, MT, 5>(b, sf[5], A, acc.v);
    mfma_col<FMT, MT, 6>(b, sf[6], A, acc.v);
    mfma_col<FMT, MT, 7>(b, sf[7], A, acc.v);
  }
}

template <int FMT, int BODY, int MT, int NTOK, int RBW, int STEP>
__device__ __forceinline__ void compute_group(const WBlock (&wb)[RBW], const uint4* win, int off,
                                              Acc<BODY, MT>& acc) {
  const int kg = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int r = 0; r < RBW; ++r)
    compute_block<FMT, BODY, MT, NTOK>(wb[r], win + (off + STEP * r) * 4 + kg, acc);
}

// Streams blocks [b0, b1) of one expert matrix in batches of GB = RBW * STEP blocks: the
// wave takes blocks bb + off + STEP * r (r < RBW) of batch bb.  A batch's weights go to
// registers and its activation operands to an LDS window; the caller has loaded the first
// batch into wa (so that those loads overlap its own set-up).  Splits are sized so that a
// workgroup streams a few batches (many workgroups keep the bytes in flight; fewer splits
// keep the partial traffic low).
// Leaves the LDS free (a barrier follows the last batch).
template <int FMT, int BODY, int MT, int NTOK, int RBW, int STEP, int WAUX = 0>
__device__ __forceinline__ void stream_expert(const ExpertView& v, int col, bool col_ok,
                                              const OpSrc& src, const int* s_slot, int nch,
                                              int b0, int b1, int off, float* lds,
                                              WBlock (&wa)[RBW], Acc<BODY, MT>& acc) {
  constexpr int GB = RBW * STEP;
  const int kg = (threadIdx.x & 63) >> 4;
  uint4* win = reinterpret_cast<uint4*>(lds);
  if constexpr (BODY == BODY_VALU) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc.v[t][i] = 0.0f;
  } else {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc.v[m][i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  for (int bb = b0; bb < b1; bb += GB) {
    if (bb != b0) load_group<RBW, WAUX>(v, bb, off, STEP, b1, kg, col, col_ok, wa);
    Window<FMT, GB, NTOK> wnd;
    wnd.load(src, s_slot, nch, bb, b1);
    if (bb != b0) __syncthreads();  // the previous batch is done with the window
    wnd.store(win);
    __syncthreads();
    compute_group<FMT, BODY, MT, NTOK, RBW, STEP>(wa, win, off, acc);
  }
  __syncthreads();
}

// One pass of a phase: dispatch the token count (VALU: 1, 2, 4 or 8 rows; MFMA: MT tiles)
// to a compile-time width.
template <int FMT, int VT, int RBW, int STEP, int WAUX = 0>
__device__ __forceinline__ void stream_valu(const ExpertView& v, int col, bool col_ok,
                                            const OpSrc& src, const int* s_slot, int nch, int b0,
                                            int b1, int off, float* lds, WBlock (&wa)[RBW],
                                            Acc<BODY_VALU, VT>& acc) {
  if (VT <= 1 || nch <= 1)
    stream_expert<FMT, BODY_VALU, VT, 1, RBW, STEP, WAUX>(v, col, col_ok, src, s_slot, nch, b0,
                                                          b1, off, lds, wa, acc);
  else if (VT <= 2 || nch <= 2)
    stream_expert<FMT, BODY_VALU, VT, (VT < 2 ? VT : 2), RBW, STEP, WAUX>(
        v, col, col_ok, src, s_slot, nch, b0, b1, off, lds, wa, acc);
  else if (VT <= 4 || nch <= 4)
    stream_expert<FMT, BODY_VALU, VT, (VT < 4 ? VT : 4), RBW, STEP, WAUX>(
        v, col, col_ok, src, s_slot, nch, b0, b1, off, lds, wa, acc);
  else
    stream_expert<FMT, BODY_VALU, VT, VT, RBW, STEP, WAUX>(v, col, col_ok, src, s_slot, nch, b0,
                                                           b1, off, lds, wa, acc);
}

// 16-bit h operand pair (bf16 for FP4, fp16 for INT4) of SiLU(g) * u, two columns
template <int FMT>
__device__ __forceinline__ uint32_t h_pair(float g0, float u0, float g1, float u1) {
  const float h0 = silu_mul(g0, u0), h1 = silu_mul(g1, u1);
  if constexpr (FMT == FMT_FP4)
    return f32pair_to_bf16pair(h0, h1);
  else
    return f32pair_to_f16pair(h0, h1);
}
template <int FMT>
__device__ __forceinline__ void store_h4(uint16_t* hop, size_t idx, float4 g, float4 u) {
  *reinterpret_cast<uint2*>(hop + idx) =
      make_uint2(h_pair<FMT>(g.x, u.x, g.y, u.y), h_pair<FMT>(g.z, u.z, g.w, u.w));
}

// Reduce a pass's partial sums over lane groups and waves through LDS and hand each
// (token, 4 columns) total to emit(m, c4, total...).  NP partials per output: the
// thread's (wave, lane group) position p; roles: gate_up has gate / up per wave parity.
// ======================================================================================
// gate_up + SiLU*up.  Grid: x = 128-column h tile, y = K split, z = active-expert index.
// Waves: w & 1 = gate (0) or up (1) columns, w >> 1 = even or odd blocks of each group.
// ======================================================================================
template <int FMT, int MT, int VT>
__global__ void __launch_bounds__(EX_THREADS) gateup_ex_kernel(MoeArgs a) {
  constexpr int TS = VT < 4 ? VT : 4;  // token slots of the vector-ALU reduction
  __shared__ __align__(16) float lds[ex_lds_floats(MT, VT)];
  __shared__ int s_slot[EX_MAXCH];
  const int act = blockIdx.z;
  int beg, cnt, e;
  if (!expert_record(a, act, &beg, &cnt, &e)) return;
  const int H = a.H, I = a.I, k = a.k, TK = a.T * k;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, q = l & 15, kg = l >> 4;
  const int role = wv & 1, khalf = wv >> 1;
  const int nt = blockIdx.x, S = a.S_gu, s = blockIdx.y;  // y == S: the split finisher
  const int TKc = a.ws.tk_cap;
  const int nblk = H / 32;
  const int b0 = (s * nblk) / S, b1 = ((s + 1) * nblk) / S;
  const size_t ld = 2 * (size_t)I;
  const int n0 = 128 * nt;                 // first h column of the tile
  const int ncols = min(128, I - n0);      // valid h columns (64 or 128)
  const bool col_ok = 8 * q < ncols;
  const int col = role * I + n0 + 8 * q;
  const ExpertView v{view_rsrc(a.wgu + (size_t)e * (H / 2) * ld, (size_t)(H / 2) * ld),
                     view_rsrc(a.sgu + (size_t)e * (H / a.group) * ld,
                               (size_t)(H / a.group) * ld * 2),
                     (int)ld, a.group};
  const OpSrc src{view_rsrc(a.x, (size_t)a.T * H * 2), true, 2 * H, k};
  // Experts with at least mfma_min tokens take MT matrix-core tiles of 16 rows (MT > 0),
  // the others VT-token vector-ALU passes, in the same launch.
  const bool use_mfma = MT > 0 && cnt >= a.mfma_min;
  const int CH = use_mfma ? 16 * MT : VT;
  const __amdgpu_buffer_rsrc_t pr = ex_rsrc(a.ws.part_gu);

  auto emit = [&](int slot, int c4, float4 g, float4 u) {
    if (S == 1) {
      store_h4<FMT>(a.ws.hop, (size_t)slot * I + n0 + c4, g, u);
    } else {
      const int base = ((s * TKc + slot) * 2 * I + n0 + c4) * 4;
      st4_sc1(pr, base, pub4(g));
      st4_sc1(pr, base + 4 * I, pub4(u));
    }
  };

  if (s == S) {  // finisher: sum the S split partials in split order, SiLU(g) * u
    const int slot0 = slot_at(a, beg);
    if (slot0 >= 0) wg_wait_published(pr, (((S - 1) * TKc + slot0) * 2 * I + n0) * 4);
    for (int it = tid; it < cnt * 64; it += EX_THREADS) {  // pairs of columns
      const int t = it >> 6, c2 = 2 * (it & 63);
      if (c2 >= ncols) continue;
      const int slot = slot_at(a, beg + t);
      if (slot < 0) continue;
      float g0 = 0.0f, g1 = 0.0f, u0 = 0.0f, u1 = 0.0f;
      for (int p0 = 0; p0 < S; p0 += 4) {
        int off[16];
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int base = (((p0 + i < S ? p0 + i : p0) * TKc + slot) * 2 * I + n0 + c2) * 4;
          off[4 * i] = base;
          off[4 * i + 1] = base + 4;
          off[4 * i + 2] = base + 4 * I;
          off[4 * i + 3] = base + 4 * I + 4;
        }
        if (!take16(pr, off, 4 * min(4, S - p0), v)) atomicOr(a.ws.err, 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (p0 + i < S) {
            g0 += v[4 * i];
            g1 += v[4 * i + 1];
            u0 += v[4 * i + 2];
            u1 += v[4 * i + 3];
          }
      }
      const uint32_t hp = h_pair<FMT>(g0, u0, g1, u1);
      *reinterpret_cast<uint32_t*>(a.ws.hop + (size_t)slot * I + n0 + c2) = hp;
    }
    return;
  }

  for (int m0 = 0; m0 < cnt; m0 += CH) {
    const int nch = min(CH, cnt - m0);
    WBlock wa[2];  // the first group's weights load while the slots are fetched
    load_group<2>(v, b0, khalf, 2, b1, kg, col, col_ok, wa);
    if (tid < nch) s_slot[tid] = slot_at(a, beg + m0 + tid);
    __syncthreads();
    if constexpr (MT > 0) {
      if (use_mfma) {
        Acc<BODY_MFMA, MT> acc;
        stream_expert<FMT, BODY_MFMA, MT, 16 * MT, 2, 2>(v, col, col_ok, src, s_slot, nch, b0,
                                                         b1, khalf, lds, wa, acc);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (16 * m >= nch) break;
          // red[role][khalf][token 0..15][column 0..127]
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              lds[((role * 2 + khalf) * 16 + 4 * kg + r) * 128 + 8 * q + i] = acc.v[m][i][r];
          __syncthreads();
          for (int it = tid; it < 16 * 32; it += EX_THREADS) {
            const int t = it >> 5, c4 = 4 * (it & 31);
            if (16 * m + t >= nch || c4 >= ncols) continue;
            const int slot = s_slot[16 * m + t];
            if (slot < 0) continue;
            const float4* r4 = reinterpret_cast<const float4*>(lds);
            const float4 g = f4_add(r4[((0 * 16 + t) * 128 + c4) / 4], r4[((1 * 16 + t) * 128 + c4) / 4]);
            const float4 u = f4_add(r4[((2 * 16 + t) * 128 + c4) / 4], r4[((3 * 16 + t) * 128 + c4) / 4]);
            emit(slot, c4, g, u);
          }
          __syncthreads();
        }
        continue;
      }
    }
    Acc<BODY_VALU, VT> acc;
    stream_valu<FMT, VT, 2, 2>(v, col, col_ok, src, s_slot, nch, b0, b1, khalf, lds, wa, acc);
    // two halves of 4 tokens: red[role][khalf][kg][token 0..3][column 0..127]
#pragma unroll
    for (int hh = 0; hh < (VT + 3) / 4; ++hh) {
      if (4 * hh >= nch) break;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (4 * hh + t < VT)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            lds[((((role * 2 + khalf) * 4 + kg) * TS + t) * 128) + 8 * q + i] = acc.v[4 * hh + t][i];
      __syncthreads();
      if (tid < TS * 32) {
        const int t = tid >> 5, c4 = 4 * (tid & 31);
        const int slot = (4 * hh + t < nch) ? s_slot[4 * hh + t] : -1;
        if (slot >= 0 && c4 < ncols) {
          const float4* r4 = reinterpret_cast<const float4*>(lds);
          float4 g = make_float4(0.0f, 0.0f, 0.0f, 0.0f), u = g;
#pragma unroll
          for (int p = 0; p < 8; ++p) {  // p = khalf * 4 + kg
            g = f4_add(g, r4[(((0 * 8 + p) * TS + t) * 128 + c4) / 4]);
            u = f4_add(u, r4[(((1 * 8 + p) * TS + t) * 128 + c4) / 4]);
          }
          emit(slot, c4, g, u);
        }
      }
      __syncthreads();
    }
  }
}

// ======================================================================================
// down + top-k combine.  Grid: x = 128-column output tile, y = K split over I, z =
// active-expert index (z >= A: per-token combiners, in the last down launch only).  All 4
// waves share the columns; wave w takes blocks b0 + w + 4 r.
// ======================================================================================
// Combiner: out[t, m .. m+3] = bf16(residual + sum_j w_j * sum_s part[s][t k + j]), j and s
// ascending.  The k * S partial rows of a token are polled 16 at a time (an invalid slot's
// rows were published as zeros by the schedule) and cleared after use.
__device__ __forceinline__ void combine_token(const MoeArgs& a, __amdgpu_buffer_rsrc_t pr, int t,
                                              int m) {
  const int k = a.k, H = a.H, S = a.S_dn, TKc = a.ws.tk_cap;
  const int total = k * S;
  float acc = 0.0f, y = 0.0f;
  for (int u0 = 0; u0 < total; u0 += 16) {
    int off[16];
    float wv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = (u0 + i < total) ? u0 + i : u0;
      const int j = u / S, p = u - j * S, slot = t * k + j;
      off[i] = ((p * TKc + slot) * H + m) * 4;
      const int e = a.ids[slot];
      wv[i] = (e >= 0 && e < a.E) ? a.wts[slot] : 0.0f;
    }
    float v[16];
    if (!take16(pr, off, min(16, total - u0), v)) atomicOr(a.ws.err, 2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (u0 + i < total) {
        y += v[i];
        if ((u0 + i) % S == S - 1) {
          acc = fmaf(wv[i], y, acc);
          y = 0.0f;
        }
      }
    }
  }
  if (a.res) acc += bf16_to_f32(a.res[(size_t)t * H + m]);
  a.out[(size_t)t * H + m] = f32_to_bf16(acc);
}

constexpr int EX_COMBINE_TOKENS = 2;  // tokens per combiner workgroup (x 128 columns)

template <int FMT, int MT, int VT>
__global__ void __launch_bounds__(EX_THREADS) down_ex_kernel(MoeArgs a) {
  constexpr int TS = VT < 4 ? VT : 4;  // token slots of the vector-ALU reduction
  __shared__ __align__(16) float lds[ex_lds_floats(MT, VT)];
  __shared__ int s_slot[EX_MAXCH];
  const int H = a.H, I = a.I, k = a.k;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, q = l & 15, kg = l >> 4;
  const int mt = blockIdx.x, S = a.S_dn, s = blockIdx.y;
  const int TKc = a.ws.tk_cap;
  const int m0c = 128 * mt;
  const int ncols = min(128, H - m0c);
  const __amdgpu_buffer_rsrc_t pr = ex_rsrc(a.ws.part_dn);
  const int A = min(a.E, a.T * k);
  if ((int)blockIdx.z >= A) {  // combiner of tokens [8 zc, 8 zc + 8), this tile
    if (s != 0) return;
    const int t0 = ((int)blockIdx.z - A) * EX_COMBINE_TOKENS;
    if (t0 < a.T)  // the first token's last slot, last split
      wg_wait_published(pr, (((S - 1) * TKc + t0 * k + k - 1) * H + m0c) * 4);
    for (int it = tid; it < EX_COMBINE_TOKENS * 128; it += EX_THREADS) {
      const int t = t0 + (it >> 7), c = it & 127;
      if (t < a.T && c < ncols) combine_token(a, pr, t, m0c + c);
    }
    return;
  }
  const int act = blockIdx.z;
  int beg, cnt, e;
  if (!expert_record(a, act, &beg, &cnt, &e)) return;
  const int nblk = I / 32;
  const int b0 = (s * nblk) / S, b1 = ((s + 1) * nblk) / S;
  const size_t ld = (size_t)H;
  const bool col_ok = 8 * q < ncols;
  const int col = m0c + 8 * q;
  const ExpertView v{view_rsrc(a.wd + (size_t)e * (I / 2) * ld, (size_t)(I / 2) * ld),
                     view_rsrc(a.sd + (size_t)e * (I / a.group) * ld,
                               (size_t)(I / a.group) * ld * 2),
                     (int)ld, a.group};
  const OpSrc src{view_rsrc(a.ws.hop, (size_t)TKc * I * 2), false, 2 * I, k};
  const bool use_mfma = MT > 0 && cnt >= a.mfma_min;  // as in gate_up
  const int CH = use_mfma ? 16 * MT : VT;
  auto emit = [&](int slot, int c4, float4 y) {
    st4_sc1(pr, ((s * TKc + slot) * H + m0c + c4) * 4, pub4(y));
  };

  for (int c0 = 0; c0 < cnt; c0 += CH) {
    const int nch = min(CH, cnt - c0);
    WBlock wa[2];  // the first group's weights load while the slots are fetched
    load_group<2>(v, b0, wv, 4, b1, kg, col, col_ok, wa);
    if (tid < nch) s_slot[tid] = slot_at(a, beg + c0 + tid);
    __syncthreads();
    bool done = false;
    if constexpr (MT > 0) {
      if (use_mfma) {
      done = true;
      Acc<BODY_MFMA, MT> acc;
      stream_expert<FMT, BODY_MFMA, MT, 16 * MT, 2, 4>(v, col, col_ok, src, s_slot, nch, b0, b1,
                                                       wv, lds, wa, acc);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (16 * m >= nch) break;
        // red[wave][token 0..15][column 0..127]
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            lds[(wv * 16 + 4 * kg + r) * 128 + 8 * q + i] = acc.v[m][i][r];
        __syncthreads();
        for (int it = tid; it < 16 * 32; it += EX_THREADS) {
          const int t = it >> 5, c4 = 4 * (it & 31);
          if (16 * m + t >= nch || c4 >= ncols) continue;
          const int slot = s_slot[16 * m + t];
          if (slot < 0) continue;
          const float4* r4 = reinterpret_cast<const float4*>(lds);
          float4 y = r4[((0 * 16 + t) * 128 + c4) / 4];
#pragma unroll
          for (int p = 1; p < 4; ++p) y = f4_add(y, r4[((p * 16 + t) * 128 + c4) / 4]);
          emit(slot, c4, y);
        }
        __syncthreads();
      }
      }
    }
    if (!done) {
      Acc<BODY_VALU, VT> acc;
      stream_valu<FMT, VT, 2, 4>(v, col, col_ok, src, s_slot, nch, b0, b1, wv, lds, wa, acc);
#pragma unroll
      for (int hh = 0; hh < (VT + 3) / 4; ++hh) {
        if (4 * hh >= nch) break;
        // red[wave][kg][token 0..3][column 0..127]
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (4 * hh + t < VT)
#pragma unroll
            for (int i = 0; i < 8; ++i)
              lds[(((wv * 4 + kg) * TS + t) * 128) + 8 * q + i] = acc.v[4 * hh + t][i];
        __syncthreads();
        if (tid < TS * 32) {
          const int t = tid >> 5, c4 = 4 * (tid & 31);
          const int slot = (4 * hh + t < nch) ? s_slot[4 * hh + t] : -1;
          if (slot >= 0 && c4 < ncols) {
            const float4* r4 = reinterpret_cast<const float4*>(lds);
            float4 y = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
            for (int p = 0; p < 16; ++p)  // p = wave * 4 + kg
              y = f4_add(y, r4[((p * TS + t) * 128 + c4) / 4]);
            emit(slot, c4, y);
          }
        }
        __syncthreads();
      }
    }
  }
}

// ======================================================================================
// dense packed INT4 GEMV: y [T, N] = x [T, K] W, the E = 1 case of the expert tiles.
// Grid: x = 128-column tile, y = K split; wave w takes blocks g0 + w + 4 r.  Splits are
// summed by the last workgroup of a tile, in split order, which also resets the counter.
// (FastInfer page, "Specialized matrix-vector result": a single-row matrix-vector product
// over contiguous stored weights with fp32 reductions; here the weights are packed 4-bit
// codes decoded in registers.)
// ======================================================================================
template <int MT, int VT>
__global__ void __launch_bounds__(EX_THREADS) gemv_ex_kernel(GemvArgs g) {
  constexpr int FMT = FMT_INT4;
  constexpr int TS = VT < 4 ? VT : 4;  // token slots of the vector-ALU reduction
  __shared__ __align__(16) float lds[ex_lds_floats(MT, VT)];
  __shared__ int s_slot[EX_MAXCH];
  const int T = g.T, K = g.K, N = g.N;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, q = l & 15, kg = l >> 4;
  const int tile = blockIdx.x, S = g.S, s = blockIdx.y;  // y == S: the split finisher
  const int nblk = K / 32;
  const int b0 = (s * nblk) / S, b1 = ((s + 1) * nblk) / S;
  const int m0c = 128 * tile;
  const int ncols = min(128, N - m0c);
  const int Tc = g.t_cap;
  const bool col_ok = 8 * q < ncols;
  const int col = m0c + 8 * q;
  const ExpertView v{view_rsrc(g.w, (size_t)(K / 2) * N),
                     view_rsrc(g.s, (size_t)(K / g.group) * N * 2), N, g.group};
  const OpSrc src{view_rsrc(g.x, (size_t)T * K * 2), true, 2 * K, 1};
  const int CH = MT > 0 ? 16 * MT : VT;
  const __amdgpu_buffer_rsrc_t pr = ex_rsrc(g.part);
  auto emit = [&](int t, int c4, float4 y) {
    if (S == 1) {
      const uint2 o =
          make_uint2((uint32_t)f32_to_bf16(y.x) | ((uint32_t)f32_to_bf16(y.y) << 16),
                     (uint32_t)f32_to_bf16(y.z) | ((uint32_t)f32_to_bf16(y.w) << 16));
      *reinterpret_cast<uint2*>(g.y + (size_t)t * N + m0c + c4) = o;
    } else {
      st4_sc1(pr, ((s * Tc + t) * N + m0c + c4) * 4, pub4(y));
    }
  };

  if (s == S) {  // finisher: sum the S split partials in split order
    // every thread polls its own partials directly (a one-lane wait on the last split before
    // the gather would add a round trip to the end of the call: 10.4 -> 9.9 us at N = 8192)
    for (int it = tid; it < T * 128; it += EX_THREADS) {
      const int t = it >> 7, c = it & 127;
      if (c >= ncols) continue;
      float y = 0.0f;
      for (int p0 = 0; p0 < S; p0 += 16) {
        int off[16];
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          off[i] = (((p0 + i < S ? p0 + i : p0) * Tc + t) * N + m0c + c) * 4;
        if (!take16(pr, off, min(16, S - p0), v) && g.err) atomicOr(g.err, 2);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (p0 + i < S) y += v[i];
      }
      g.y[(size_t)t * N + m0c + c] = f32_to_bf16(y + 0.0f);  // -0.0 sums become +0.0
    }
    return;
  }

  for (int c0 = 0; c0 < T; c0 += CH) {
    const int nch = min(CH, T - c0);
    WBlock wa[2];  // the first group's weights load while the token list is set up
    load_group<2, EX_STREAM>(v, b0, wv, 4, b1, kg, col, col_ok, wa);
    if (tid < nch) s_slot[tid] = c0 + tid;
    __syncthreads();
    if constexpr (MT > 0) {
      Acc<BODY_MFMA, MT> acc;
      stream_expert<FMT, BODY_MFMA, MT, 16 * MT, 2, 4, EX_STREAM>(v, col, col_ok, src, s_slot, nch, b0, b1,
                                                       wv, lds, wa, acc);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (16 * m >= nch) break;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            lds[(wv * 16 + 4 * kg + r) * 128 + 8 * q + i] = acc.v[m][i][r];
        __syncthreads();
        for (int it = tid; it < 16 * 32; it += EX_THREADS) {
          const int t = it >> 5, c4 = 4 * (it & 31);
          if (16 * m + t >= nch || c4 >= ncols) continue;
          const float4* r4 = reinterpret_cast<const float4*>(lds);
          float4 y = r4[((0 * 16 + t) * 128 + c4) / 4];
#pragma unroll
          for (int p = 1; p < 4; ++p) y = f4_add(y, r4[((p * 16 + t) * 128 + c4) / 4]);
          emit(c0 + 16 * m + t, c4, y);
        }
        __syncthreads();
      }
    } else {
      Acc<BODY_VALU, VT> acc;
      stream_valu<FMT, VT, 2, 4, EX_STREAM>(v, col, col_ok, src, s_slot, nch, b0, b1, wv, lds, wa,
                                       acc);
#pragma unroll
      for (int hh = 0; hh < (VT + 3) / 4; ++hh) {
        if (4 * hh >= nch) break;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (4 * hh + t < VT)
#pragma unroll
            for (int i = 0; i < 8; ++i)
              lds[(((wv * 4 + kg) * TS + t) * 128) + 8 * q + i] = acc.v[4 * hh + t][i];
        __syncthreads();
        if (tid < TS * 32) {
          const int t = tid >> 5, c4 = 4 * (tid & 31);
          if (4 * hh + t < nch && c4 < ncols) {
            const float4* r4 = reinterpret_cast<const float4*>(lds);
            float4 y = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
            for (int p = 0; p < 16; ++p) y = f4_add(y, r4[((p * TS + t) * 128 + c4) / 4]);
            emit(c0 + 4 * hh + t, c4, y);
          }
        }
        __syncthreads();
      }
    }
  }
}

// tokens per vector-ALU pass for calls with T tokens (no expert has more than T)
static int valu_width(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : EX_VT; }

hipError_t launch_gemv_ex(const GemvArgs& g, int mt, hipStream_t st) {
  const dim3 grid((g.N + 127) / 128, g.S + (g.S > 1 ? 1 : 0)), block(EX_THREADS);
  const int vt = valu_width(g.T);
  if (mt == 1)
    hipLaunchKernelGGL((gemv_ex_kernel<1, 1>), grid, block, 0, st, g);
  else if (mt == 2)
    hipLaunchKernelGGL((gemv_ex_kernel<2, 1>), grid, block, 0, st, g);
  else if (vt == 1)
    hipLaunchKernelGGL((gemv_ex_kernel<0, 1>), grid, block, 0, st, g);
  else if (vt == 2)
    hipLaunchKernelGGL((gemv_ex_kernel<0, 2>), grid, block, 0, st, g);
  else if (vt == 4)
    hipLaunchKernelGGL((gemv_ex_kernel<0, 4>), grid, block, 0, st, g);
  else
    hipLaunchKernelGGL((gemv_ex_kernel<0, EX_VT>), grid, block, 0, st, g);
  return hipGetLastError();
}

int ex_max_split_gemv() { return EX_MAX_SPLIT_GEMV; }

// ---- launchers --------------------------------------------------------------------------------
template <int FMT, int MT, int VT>
static hipError_t launch_phase(const MoeArgs& a, int A, bool down, hipStream_t st) {
  if (!down) {
    hipLaunchKernelGGL((gateup_ex_kernel<FMT, MT, VT>),
                       dim3((a.I + 127) / 128, a.S_gu + (a.S_gu > 1 ? 1 : 0), A),
                       dim3(EX_THREADS), 0, st, a);
  } else {
    const int zc = a.combine ? (a.T + EX_COMBINE_TOKENS - 1) / EX_COMBINE_TOKENS : 0;
    hipLaunchKernelGGL((down_ex_kernel<FMT, MT, VT>), dim3((a.H + 127) / 128, a.S_dn, A + zc),
                       dim3(EX_THREADS), 0, st, a);
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_ex_t(const MoeArgs& a0, int A, int mt, hipStream_t st) {
  // one launch per phase: with matrix-core tiles (mt > 0) the kernel serves the experts
  // below the threshold with EX_VT-token vector-ALU passes in the same launch
  const int vt = valu_width(a0.T);
  MoeArgs a = a0;
  for (int down = 0; down < 2; ++down) {
    a.combine = down;  // the down launch also runs the per-token combiners
    hipError_t e;
    if (mt == 1) e = launch_phase<FMT, 1, EX_VT>(a, A, down, st);
    else if (vt == 1) e = launch_phase<FMT, 0, 1>(a, A, down, st);
    else if (vt == 2) e = launch_phase<FMT, 0, 2>(a, A, down, st);
    else e = launch_phase<FMT, 0, EX_VT>(a, A, down, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_moe_experts(const MoeArgs& a, int A, int mt, hipStream_t st) {
  if (mt < 0 || mt > 1) return hipErrorInvalidValue;
  if (a.fmt == FMT_FP4) return launch_ex_t<FMT_FP4>(a, A, mt, st);
  if (a.fmt == FMT_INT4) return launch_ex_t<FMT_INT4>(a, A, mt, st);
  return hipErrorInvalidValue;
}

int ex_max_split() { return EX_MAX_SPLIT; }

}  // namespace dqg
