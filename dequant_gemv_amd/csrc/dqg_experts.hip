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
// cold, at the end of a dependency chain, where code size is time).  SLEEP: the backoff between
// rounds (s_sleep units of 64 clocks).
template <int SLEEP = 8>
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
    __builtin_amdgcn_s_sleep(SLEEP);
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
// A lane's share of one block (32 K indices): the byte rows that hold K = 32 b + 8 kg .. +7 of
// 8 columns -- 4 rows of 4-bit pairs, 8 rows of FP8 codes, or 2 rows of 2-bit codes (INT2:
// four K indices per byte; FE-XC: the two codebook codes of the 8 K indices) -- and the
// columns' scales.
template <int FMT>
struct WBlockT {
  static constexpr int R = FMT == FMT_FP8                        ? 8
                           : (FMT == FMT_INT2 || FMT == FMT_FEXC) ? 2
                                                                  : 4;  // byte rows per lane
  uint2 w[R];  // byte rows 4 R b + R kg + j, 8 columns
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

// Expert e's view of a [K, ld] matrix read in format F, its slabs slab_rows byte rows apart
// (the 2-bit codes of a mixed layer's cold experts fill the first K / 4 rows of a 4-bit slab).
template <int F>
__device__ __forceinline__ ExpertView expert_view(const uint8_t* w, const uint16_t* s, int e,
                                                  int K, int slab_rows, size_t ld, int group) {
  const int rows = F == FMT_FP8 ? K : (F == FMT_INT2 || F == FMT_FEXC) ? K / 4 : K / 2;
  return ExpertView{view_rsrc(w + (size_t)e * slab_rows * ld, (size_t)rows * ld),
                    view_rsrc(s + (size_t)e * (K / group) * ld, (size_t)(K / group) * ld * 2),
                    (int)ld, group};
}

template <int FMT, int WAUX>
__device__ __forceinline__ void load_wblock(const ExpertView& v, int blk, int kg, int col,
                                            bool ok, WBlockT<FMT>& o) {
  constexpr int R = WBlockT<FMT>::R;
  const int wo = ok ? (4 * R * blk + R * kg) * v.ld + col : EX_OOB;
  const int so = ok ? (((32 * blk) / v.group) * v.ld + col) * 2 : EX_OOB;
#pragma unroll
  for (int j = 0; j < R; ++j) {
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

// INT2: lane row j holds K 4 j .. 4 j + 3 of every column byte in bits 0-1, 2-3, 4-5, 6-7
// (code c means c - 2).  The masks move the codes of K 4 j, 4 j + 1 (lo) or 4 j + 2, 4 j + 3
// (hi) of every byte into its two nibbles, which the FP4 conversion reads as c / 2 exactly
// (E2M1 codes 0..3 are 0, 0.5, 1, 1.5): the tiles double the scale and add -sum(x).
__device__ __forceinline__ uint32_t int2_lo_nibbles(uint32_t d) {
  return (d & 0x03030303u) | ((d << 2) & 0x30303030u);
}
__device__ __forceinline__ uint32_t int2_hi_nibbles(uint32_t d) {
  return ((d >> 4) & 0x03030303u) | ((d >> 2) & 0x30303030u);
}
constexpr uint32_t BF16_MINUS_ONE_PAIR = 0xBF80BF80u;

// the lane's 4 pairs of column I: K = 32 b + 8 kg + 2 p, + 1 (p = 0..3) as 16-bit pairs.
// 4-bit formats: byte I % 4 of row p holds the pair; FP8: rows 2 p and 2 p + 1 hold one code
// each, interleaved by one v_perm_b32 so that one conversion yields the bf16 pair (E4M3
// values are exact in bf16).
template <int FMT, int I>
__device__ __forceinline__ u32x4_t decode_col(const WBlockT<FMT>& b) {
  if constexpr (FMT == FMT_FP8) {
    constexpr uint32_t B = I % 4;
    constexpr uint32_t sel = B | ((4u + B) << 8) | (B << 16) | ((4u + B) << 24);
    uint32_t r[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = (I < 4) ? b.w[2 * p].x : b.w[2 * p].y;
      const uint32_t hi = (I < 4) ? b.w[2 * p + 1].x : b.w[2 * p + 1].y;
      r[p] = __builtin_bit_cast(uint32_t, fp8_pair_bf16<0>(__builtin_amdgcn_perm(hi, lo, sel)));
    }
    return u32x4_t{r[0], r[1], r[2], r[3]};
  } else if constexpr (FMT == FMT_INT2) {
    const uint32_t d0 = (I < 4) ? b.w[0].x : b.w[0].y, d1 = (I < 4) ? b.w[1].x : b.w[1].y;
    return u32x4_t{dec_pair<FMT_FP4, I % 4>(int2_lo_nibbles(d0)),
                   dec_pair<FMT_FP4, I % 4>(int2_hi_nibbles(d0)),
                   dec_pair<FMT_FP4, I % 4>(int2_lo_nibbles(d1)),
                   dec_pair<FMT_FP4, I % 4>(int2_hi_nibbles(d1))};
  } else {
    const uint32_t d0 = (I < 4) ? b.w[0].x : b.w[0].y, d1 = (I < 4) ? b.w[1].x : b.w[1].y;
    const uint32_t d2 = (I < 4) ? b.w[2].x : b.w[2].y, d3 = (I < 4) ? b.w[3].x : b.w[3].y;
    return u32x4_t{dec_pair<FMT, I % 4>(d0), dec_pair<FMT, I % 4>(d1), dec_pair<FMT, I % 4>(d2),
                   dec_pair<FMT, I % 4>(d3)};
  }
}

__device__ __forceinline__ void scales8(const uint4& s, float (&sf)[8]) {
  sf[0] = bf16_lo(s.x); sf[1] = bf16_hi(s.x);
  sf[2] = bf16_lo(s.y); sf[3] = bf16_hi(s.y);
  sf[4] = bf16_lo(s.z); sf[5] = bf16_hi(s.z);
  sf[6] = bf16_lo(s.w); sf[7] = bf16_hi(s.w);
}

// 16-bit operands: bf16 for FP4 and FP8 (x stays bf16), fp16 for INT4
template <int FMT>
__device__ __forceinline__ float dot2p(uint32_t p, uint32_t x, float c) {
  if constexpr (FMT != FMT_INT4)
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
// from an fp32 row (h): rounded to bf16 (FP4, FP8) or fp16 (INT4), nearest even
template <int FMT>
__device__ __forceinline__ uint4 op_from_f32(const float* row, int q8) {
  const float4 a = reinterpret_cast<const float4*>(row)[2 * q8];
  const float4 b = reinterpret_cast<const float4*>(row)[2 * q8 + 1];
  if constexpr (FMT != FMT_INT4)
    return make_uint4(f32pair_to_bf16pair(a.x, a.y), f32pair_to_bf16pair(a.z, a.w),
                      f32pair_to_bf16pair(b.x, b.y), f32pair_to_bf16pair(b.z, b.w));
  else
    return make_uint4(f32pair_to_f16pair(a.x, a.y), f32pair_to_f16pair(a.z, a.w),
                      f32pair_to_f16pair(b.x, b.y), f32pair_to_f16pair(b.z, b.w));
}

template <int FMT>
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint4& a, const u32x4_t& b, f32x4_t c) {
  const u32x4_t av = {a.x, a.y, a.z, a.w};
  if constexpr (FMT != FMT_INT4)
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
template <int FMT, int RBW, int WAUX = 0>
__device__ __forceinline__ void load_group(const ExpertView& v, int g0, int off, int step,
                                           int b1, int kg, int col, bool col_ok,
                                           WBlockT<FMT> (&wb)[RBW]) {
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    const int b = g0 + off + step * r;
    load_wblock<FMT, WAUX>(v, b, kg, col, col_ok && b < b1, wb[r]);
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
__device__ __forceinline__ u32x4_t decode_col_valu(const WBlockT<FMT>& b) {
  if constexpr (FMT != FMT_INT4) {
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
__device__ __forceinline__ void valu_col(const WBlockT<FMT>& b, float sc, const uint4 (&op)[NTOK],
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
// c0: the products' initial value (zero; for INT2 the tile's -sum(x) per token row)
template <int FMT, int MT, int I>
__device__ __forceinline__ void mfma_col(const WBlockT<FMT>& b, float sc, const uint4 (&A)[MT],
                                         const f32x4_t (&c0)[MT], f32x4_t (&acc)[MT][8]) {
  const u32x4_t B = decode_col<FMT, I>(b);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const f32x4_t D = mfma_16x16x32<FMT>(A[m], B, c0[m]);
    acc[m][I] += sc * D;
  }
}

// FE-XC: lane row j of a block holds codebook j's code of the lane's 8 K indices for 8
// columns; the weights are C[0][c0] + C[1][c1] (8 bf16 each: one uint4 of the LDS copy cbl,
// [2][256] vectors) times the scale.  A vector's 8 values line up with the token's 8 K
// values as they are, so each codebook gives one dot2 chain (vector ALU) or one product
// into the column's accumulator (matrix cores): the decomposition is exact.
template <int BODY, int MT, int NTOK>
__device__ __forceinline__ void fexc_block(const WBlockT<FMT_FEXC>& b, const uint4* wrow,
                                           const uint4* cbl, const float (&sf)[8],
                                           Acc<BODY, MT>& acc) {
  if constexpr (BODY == BODY_VALU) {
    uint4 op[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) op[t] = wrow[t * EX_WROW];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t d0 = (i < 4) ? b.w[0].x : b.w[0].y, d1 = (i < 4) ? b.w[1].x : b.w[1].y;
      const uint4 v0 = cbl[(d0 >> (8 * (i & 3))) & 0xFFu];
      const uint4 v1 = cbl[256 + ((d1 >> (8 * (i & 3))) & 0xFFu)];
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        float d = dot2p<FMT_FEXC>(v0.x, op[t].x, 0.0f);
        d = dot2p<FMT_FEXC>(v0.y, op[t].y, d);
        d = dot2p<FMT_FEXC>(v0.z, op[t].z, d);
        d = dot2p<FMT_FEXC>(v0.w, op[t].w, d);
        d = dot2p<FMT_FEXC>(v1.x, op[t].x, d);
        d = dot2p<FMT_FEXC>(v1.y, op[t].y, d);
        d = dot2p<FMT_FEXC>(v1.z, op[t].z, d);
        d = dot2p<FMT_FEXC>(v1.w, op[t].w, d);
        acc.v[t][i] = fmaf(sf[i], d, acc.v[t][i]);
      }
    }
  } else {
    const int q = threadIdx.x & 15;
    uint4 A[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) A[m] = wrow[(16 * m + q) * EX_WROW];
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t d0 = (i < 4) ? b.w[0].x : b.w[0].y, d1 = (i < 4) ? b.w[1].x : b.w[1].y;
      const uint4 v0 = cbl[(d0 >> (8 * (i & 3))) & 0xFFu];
      const uint4 v1 = cbl[256 + ((d1 >> (8 * (i & 3))) & 0xFFu)];
      const u32x4_t B0 = {v0.x, v0.y, v0.z, v0.w}, B1 = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const f32x4_t D = mfma_16x16x32<FMT_FEXC>(A[m], B1, mfma_16x16x32<FMT_FEXC>(A[m], B0, zero));
        acc.v[m][i] += sf[i] * D;
      }
    }
  }
}

// One block: `wrow` = the window entry of this block and lane group for token row 0.
// VALU: NTOK token rows; MFMA: MT tiles of 16 rows (rows past the pass are zero).
// FP8 blocks hold twice the bytes of the 4-bit ones; left free, the scheduler decodes every
// column of a block ahead of its products and the matrix-core kernel needs 264 registers
// (one wave per SIMD).  A fence after each column keeps one column's operands live.
template <int FMT>
__device__ __forceinline__ void col_fence() {
  if constexpr (FMT == FMT_FP8) __builtin_amdgcn_sched_barrier(0);
}

template <int FMT, int BODY, int MT, int NTOK>
__device__ __forceinline__ void compute_block(const WBlockT<FMT>& b, const uint4* wrow,
                                              Acc<BODY, MT>& acc, const uint4* cbl) {
  float sf[8];
  scales8(b.s, sf);
  if constexpr (FMT == FMT_INT2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sf[i] *= 2.0f;  // the decoded pairs hold c / 2
  }
  if constexpr (FMT == FMT_FEXC) {
    fexc_block<BODY, MT, NTOK>(b, wrow, cbl, sf, acc);
  } else if constexpr (BODY == BODY_VALU) {
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
      } else if constexpr (FMT == FMT_INT2) {  // -sum(x) of the lane's 8 K indices
        corr[t] = dot2p<FMT>(BF16_MINUS_ONE_PAIR, op[t].x, corr[t]);
        corr[t] = dot2p<FMT>(BF16_MINUS_ONE_PAIR, op[t].y, corr[t]);
        corr[t] = dot2p<FMT>(BF16_MINUS_ONE_PAIR, op[t].z, corr[t]);
        corr[t] = dot2p<FMT>(BF16_MINUS_ONE_PAIR, op[t].w, corr[t]);
      }
    }
    valu_col<FMT, NTOK, MT, 0>(b, sf[0], op, corr, acc.v);
    col_fence<FMT>();
    valu_col<FMT, NTOK, MT, 1>(b, sf[1], op, corr, acc.v);
    col_fence<FMT>();
    valu_col<FMT, NTOK, MT, 2>(b, sf[2], op, corr, acc.v);
    col_fence<FMT>();
    valu_col<FMT, NTOK, MT, 3>(b, sf[3], op, corr, acc.v);
    col_fence<FMT>();
    valu_col<FMT, NTOK, MT, 4>(b, sf[4], op, corr, acc.v);
    col_fence<FMT>();
    valu_col<FMT, NTOK, MT, 5>(b, sf[5], op, corr, acc.v);
    col_fence<FMT>();
    valu_col<FMT, NTOK, MT, 6>(b, sf[6], op, corr, acc.v);
    col_fence<FMT>();
    valu_col<FMT, NTOK, MT, 7>(b, sf[7], op, corr, acc.v);
  } else {
    const int q = threadIdx.x & 15;
    uint4 A[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) A[m] = wrow[(16 * m + q) * EX_WROW];
    f32x4_t c0[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      c0[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (FMT == FMT_INT2) {  // -sum(x) of every token row, in every column
        const u32x4_t mo = {BF16_MINUS_ONE_PAIR, BF16_MINUS_ONE_PAIR, BF16_MINUS_ONE_PAIR,
                            BF16_MINUS_ONE_PAIR};
        c0[m] = mfma_16x16x32<FMT>(A[m], mo, c0[m]);
      }
    }
    mfma_col<FMT, MT, 0>(b, sf[0], A, c0, acc.v);
    col_fence<FMT>();
    mfma_col<FMT, MT, 1>(b, sf[1], A, c0, acc.v);
    col_fence<FMT>();
    mfma_col<FMT, MT, 2>(b, sf[2], A, c0, acc.v);
    col_fence<FMT>();
    mfma_col<FMT, MT, 3>(b, sf[3], A, c0, acc.v);
    col_fence<FMT>();
    mfma_col<FMT, MT, 4>(b, sf[4], A, c0, acc.v);
    col_fence<FMT>();
    mfma_col<FMT, MT, 5>(b, sf[5], A, c0, acc.v);
    col_fence<FMT>();
    mfma_col<FMT, MT, 6>(b, sf[6], A, c0, acc.v);
    col_fence<FMT>();
    mfma_col<FMT, MT, 7>(b, sf[7], A, c0, acc.v);
  }
}

template <int FMT, int BODY, int MT, int NTOK, int RBW, int STEP>
__device__ __forceinline__ void compute_group(const WBlockT<FMT> (&wb)[RBW], const uint4* win, int off,
                                              Acc<BODY, MT>& acc, const uint4* cbl) {
  const int kg = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int r = 0; r < RBW; ++r)
    compute_block<FMT, BODY, MT, NTOK>(wb[r], win + (off + STEP * r) * 4 + kg, acc, cbl);
}

// Streams blocks [b0, b1) of one expert matrix in batches of GB = RBW * STEP blocks: the
// wave takes blocks bb + off + STEP * r (r < RBW) of batch bb.  A batch's weights go to
// registers and its activation operands to an LDS window; the caller has loaded the first
// batch into wa (so that those loads overlap its own set-up).  Splits are sized so that a
// workgroup streams a few batches (many workgroups keep the bytes in flight; fewer splits
// keep the partial traffic low).
// Leaves the LDS free (a barrier follows the last batch).
template <int FMT, int BODY, int MT, int NTOK, int RBW, int STEP, int WAUX = 0, bool PF = false>
__device__ __forceinline__ void stream_expert(const ExpertView& v, int col, bool col_ok,
                                              const OpSrc& src, const int* s_slot, int nch,
                                              int b0, int b1, int off, float* lds,
                                              WBlockT<FMT> (&wa)[RBW], Acc<BODY, MT>& acc,
                                              const uint4* cbl = nullptr) {
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
  if constexpr (!PF) {
    for (int bb = b0; bb < b1; bb += GB) {
      if (bb != b0) load_group<FMT, RBW, WAUX>(v, bb, off, STEP, b1, kg, col, col_ok, wa);
      Window<FMT, GB, NTOK> wnd;
      wnd.load(src, s_slot, nch, bb, b1);
      if (bb != b0) __syncthreads();  // the previous batch is done with the window
      wnd.store(win);
      __syncthreads();
      compute_group<FMT, BODY, MT, NTOK, RBW, STEP>(wa, win, off, acc, cbl);
    }
  } else {
    // Double-buffered: batch g computes from `cur` while the next batch's weights load into
    // `nxt`.  Those loads are issued after batch g's operand-window loads, so the in-order
    // wait for the window leaves them in flight across the compute.
    WBlockT<FMT> wb[RBW];
    for (int bb = b0; bb < b1; bb += GB) {
      Window<FMT, GB, NTOK> wnd;
      wnd.load(src, s_slot, nch, bb, b1);
      load_group<FMT, RBW, WAUX>(v, bb + GB, off, STEP, b1, kg, col, col_ok, wb);
      if (bb != b0) __syncthreads();  // the previous batch is done with the window
      wnd.store(win);
      __syncthreads();
      compute_group<FMT, BODY, MT, NTOK, RBW, STEP>(wa, win, off, acc, cbl);
#pragma unroll
      for (int r = 0; r < RBW; ++r) wa[r] = wb[r];
    }
  }
  __syncthreads();
}

// One pass of a phase: dispatch the token count (VALU: 1, 2, 4 or 8 rows; MFMA: MT tiles)
// to a compile-time width.
template <int FMT, int VT, int RBW, int STEP, int WAUX = 0, bool PF = false>
__device__ __forceinline__ void stream_valu(const ExpertView& v, int col, bool col_ok,
                                            const OpSrc& src, const int* s_slot, int nch, int b0,
                                            int b1, int off, float* lds, WBlockT<FMT> (&wa)[RBW],
                                            Acc<BODY_VALU, VT>& acc, const uint4* cbl = nullptr) {
  if (VT <= 1 || nch <= 1)
    stream_expert<FMT, BODY_VALU, VT, 1, RBW, STEP, WAUX, PF>(v, col, col_ok, src, s_slot, nch,
                                                              b0, b1, off, lds, wa, acc, cbl);
  else if (VT <= 2 || nch <= 2)
    stream_expert<FMT, BODY_VALU, VT, (VT < 2 ? VT : 2), RBW, STEP, WAUX, PF>(
        v, col, col_ok, src, s_slot, nch, b0, b1, off, lds, wa, acc, cbl);
  else if (VT <= 4 || nch <= 4)
    stream_expert<FMT, BODY_VALU, VT, (VT < 4 ? VT : 4), RBW, STEP, WAUX, PF>(
        v, col, col_ok, src, s_slot, nch, b0, b1, off, lds, wa, acc, cbl);
  else
    stream_expert<FMT, BODY_VALU, VT, VT, RBW, STEP, WAUX, PF>(v, col, col_ok, src, s_slot, nch,
                                                               b0, b1, off, lds, wa, acc, cbl);
}

// One pass of a phase in weight format F: the first batch's weights load while the pass's
// slot list is fetched into LDS, then the stream (matrix-core or vector-ALU body).
template <int F, int BODY, int MT, int RBW, int STEP, bool PF>
__device__ __forceinline__ void run_pass(const MoeArgs& a, const ExpertView& v, int col,
                                         bool col_ok, const OpSrc& src, int* s_slot, int first,
                                         int nch, int b0, int b1, int off, float* lds,
                                         const uint4* cbl, Acc<BODY, MT>& acc) {
  const int kg = (threadIdx.x & 63) >> 4;
  WBlockT<F> wa[RBW];
  load_group<F, RBW>(v, b0, off, STEP, b1, kg, col, col_ok, wa);
  if ((int)threadIdx.x < nch) s_slot[threadIdx.x] = slot_at(a, first + threadIdx.x);
  __syncthreads();
  if constexpr (BODY == BODY_MFMA)
    stream_expert<F, BODY_MFMA, MT, 16 * MT, RBW, STEP, 0, PF>(
        v, col, col_ok, src, s_slot, nch, b0, b1, off, lds, wa, acc, cbl);
  else
    stream_valu<F, MT, RBW, STEP, 0, PF>(v, col, col_ok, src, s_slot, nch, b0, b1, off,
                                                  lds, wa, acc, cbl);
}

// The weight format of expert e in a kernel of base format FMT: with a per-expert table
// (MIX), INT2 and FE-XC entries (FE-XC only with codebooks) run the 2-bit tiles, any other
// entry the FP4 ones.
template <int FMT, bool MIX>
__device__ __forceinline__ int expert_format(const MoeArgs& a, int e) {
  if constexpr (!MIX) {
    return FMT;
  } else {
    const int f = a.efmt[e];
    return (f == FMT_INT2 || (f == FMT_FEXC && a.cb != nullptr)) ? f : FMT_FP4;
  }
}

// An FE-XC expert's two codebooks of one projection (m = 0 gate_up, 1 down) into LDS:
// [2][256] uint4 from the bf16 table [E][2][2][256][8].  The caller's next barrier
// publishes them.
__device__ __forceinline__ void stage_codebooks(const MoeArgs& a, int e, int m, uint4* cbl) {
  const uint4* src = reinterpret_cast<const uint4*>(a.cb) + ((size_t)e * 2 + m) * 512;
  for (int i = threadIdx.x; i < 512; i += EX_THREADS) cbl[i] = src[i];
}

// A pass in the expert's format: FMT, or (MIX) the 2-bit formats of a mixed layer.
template <int FMT, bool MIX, int BODY, int MT, int RBW, int STEP, bool PF>
__device__ __forceinline__ void run_pass_fmt(int ef, const MoeArgs& a, const uint8_t* w,
                                             const uint16_t* sc, int e, int K, size_t ld,
                                             int col, bool col_ok, const OpSrc& src,
                                             int* s_slot, int first, int nch, int b0, int b1,
                                             int off, float* lds, const uint4* cbl,
                                             Acc<BODY, MT>& acc) {
  const int slab = K / fmt_kb(FMT);
  if constexpr (MIX) {
    if (ef == FMT_INT2) {
      run_pass<FMT_INT2, BODY, MT, RBW, STEP, PF>(
          a, expert_view<FMT_INT2>(w, sc, e, K, slab, ld, a.group), col, col_ok, src, s_slot,
          first, nch, b0, b1, off, lds, cbl, acc);
      return;
    }
    if (ef == FMT_FEXC) {
      run_pass<FMT_FEXC, BODY, MT, RBW, STEP, PF>(
          a, expert_view<FMT_FEXC>(w, sc, e, K, slab, ld, a.group), col, col_ok, src, s_slot,
          first, nch, b0, b1, off, lds, cbl, acc);
      return;
    }
  }
  run_pass<FMT, BODY, MT, RBW, STEP, PF>(a, expert_view<FMT>(w, sc, e, K, slab, ld, a.group), col,
                                     col_ok, src, s_slot, first, nch, b0, b1, off, lds, cbl, acc);
}

// 16-bit h operand pair (bf16 for FP4 and FP8, fp16 for INT4) of SiLU(g) * u, two columns
template <int FMT>
__device__ __forceinline__ uint32_t h_pair(float g0, float u0, float g1, float u1) {
  const float h0 = silu_mul(g0, u0), h1 = silu_mul(g1, u1);
  if constexpr (FMT != FMT_INT4)
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
// PF: double-buffered weights (for unsplit launches, whose workgroups walk all of K)
template <int FMT, int MT, int VT, bool MIX, bool PF>
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

  const int ef = expert_format<FMT, MIX>(a, e);
  __shared__ uint4 s_cb[MIX ? 512 : 1];
  if constexpr (MIX)
    if (ef == FMT_FEXC) stage_codebooks(a, e, 0, s_cb);

  for (int m0 = 0; m0 < cnt; m0 += CH) {
    const int nch = min(CH, cnt - m0);
    if constexpr (MT > 0) {
      if (use_mfma) {
        Acc<BODY_MFMA, MT> acc;
        run_pass_fmt<FMT, MIX, BODY_MFMA, MT, 2, 2, PF>(ef, a, a.wgu, a.sgu, e, H, ld, col, col_ok,
                                                    src, s_slot, beg + m0, nch, b0, b1, khalf,
                                                    lds, s_cb, acc);
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
    run_pass_fmt<FMT, MIX, BODY_VALU, VT, 2, 2, PF>(ef, a, a.wgu, a.sgu, e, H, ld, col, col_ok, src,
                                                s_slot, beg + m0, nch, b0, b1, khalf, lds, s_cb,
                                                acc);
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

template <int FMT, int MT, int VT, bool MIX>
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
  const OpSrc src{view_rsrc(a.ws.hop, (size_t)TKc * I * 2), false, 2 * I, k};
  const bool use_mfma = MT > 0 && cnt >= a.mfma_min;  // as in gate_up
  const int CH = use_mfma ? 16 * MT : VT;
  auto emit = [&](int slot, int c4, float4 y) {
    st4_sc1(pr, ((s * TKc + slot) * H + m0c + c4) * 4, pub4(y));
  };

  const int ef = expert_format<FMT, MIX>(a, e);
  __shared__ uint4 s_cb[MIX ? 512 : 1];
  if constexpr (MIX)
    if (ef == FMT_FEXC) stage_codebooks(a, e, 1, s_cb);

  for (int c0 = 0; c0 < cnt; c0 += CH) {
    const int nch = min(CH, cnt - c0);
    bool done = false;
    if constexpr (MT > 0) {
      if (use_mfma) {
      done = true;
      Acc<BODY_MFMA, MT> acc;
      run_pass_fmt<FMT, MIX, BODY_MFMA, MT, 2, 4, false>(ef, a, a.wd, a.sd, e, I, ld, col, col_ok, src,
                                                  s_slot, beg + c0, nch, b0, b1, wv, lds, s_cb,
                                                  acc);
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
      run_pass_fmt<FMT, MIX, BODY_VALU, VT, 2, 4, false>(ef, a, a.wd, a.sd, e, I, ld, col, col_ok, src,
                                                  s_slot, beg + c0, nch, b0, b1, wv, lds, s_cb,
                                                  acc);
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
// dense packed INT4 GEMV for three or more tokens: y [T, N] = x [T, K] W on matrix-core tiles,
// the E = 1 case of the expert tiles.  Grid: x = 128-column tile, y = K split (+ one finisher
// row); wave w takes blocks g0 + w + 4 r.  Split partials are summed in split order by the
// finisher row.  (FastInfer page, "Specialized matrix-vector result": a matrix-vector
// product over contiguous stored weights with fp32 reductions; here the weights are packed
// 4-bit codes decoded in registers.)  One or two tokens run gemv_tok_kernel.
// ======================================================================================
template <int MT, int VT>
__global__ void __launch_bounds__(EX_THREADS) gemv_ex_kernel(GemvArgs g) {
  static_assert(MT > 0, "one or two tokens run gemv_tok_kernel");
  constexpr int FMT = FMT_INT4;
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
    WBlockT<FMT> wa[2];  // the first group's weights load while the token list is set up
    load_group<FMT, 2, EX_STREAM>(v, b0, wv, 4, b1, kg, col, col_ok, wa);
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
    }
  }
}

// ======================================================================================
// Dense packed INT4 GEMV for one to four tokens: one on the vector ALUs, two to four on
// matrix cores sharing the same decode, on the [K/2, N] or the prepacked layout (FastInfer page, "Specialized matrix-vector result"; eole page,
// "Packed Marlin projections" for the fused gate/up width and for weights rearranged once
// while the model is prepared for inference).
//
// Grid: 128-column tile fastest, then the K split, then one finisher workgroup per tile.  A
// lane owns 8 columns and, in each block of 16 byte rows, the 4 rows 4 kq .. 4 kq + 3; a wave
// takes 4 consecutive blocks of each round of 16.  Two rows r, r + 1 of one column are
// decoded together: one v_perm_b32 puts byte c of row r in bits 0-7 and byte c of row r + 1
// in bits 16-23, and one and-or per nibble gives the fp16 pairs (1024 + lo_r, 1024 + lo_r+1)
// and (64 + hi_r, 64 + hi_r+1), which meet the activation pairs (x[2r], x[2r+2]) and
// (x[2r+1], x[2r+3]) in v_dot2_f32_f16: 1.5 decode instructions and one dot2 per byte (the
// byte-at-a-time decode takes 3 and one).  The activations of a round are converted once per
// workgroup into that paired fp16 order in LDS, with the bias -(1032 sum x[even] + 72 sum
// x[odd]) of each 8 K values (n - 8 against the 1024- and 64-based magic pairs).  A wave sums
// its 4 blocks before it applies the group scale (G = 128: one per chunk and column; G = 32:
// one per block).  With two tokens each decoded pair meets both tokens' activations.
//
// PRE = true reads the prepacked layout: blocks of 2048 bytes holding exactly the 16-byte
// pieces a wave's lanes take from one block, lane l at 16 l (rows 4 kq, 4 kq + 1) and at
// 1024 + 16 l (rows 4 kq + 2, 4 kq + 3), 8 columns each, the two rows' bytes interleaved per
// column pair so that the decode needs one shift per 4 bytes instead of a byte permute per 2
// (row_pair); blocks ordered by round of 16, then tile.  A workgroup's round is then one contiguous 32 KB stretch right after the previous
// workgroup's, and each load instruction reads 1 KB contiguous (the [K/2, N] layout spreads
// a round over 256 row segments of 128 bytes).  Scales [K/G][tiles x 128].  With one token,
// the same arithmetic in the same order as the [K/2, N] call.
//
// MF = true (2 to 4 tokens, either layout): the same decoded fp16 pairs become the B
// operand of v_mfma_f32_16x16x32_f16 instead of meeting each token in dot2.  Lane (q, kq)
// holds K group kq of its 8 columns 8 q + i, which is the B operand of one 16x16x32 product
// over the 16 columns 8 q' + i (one product per i); the A operand is token q's paired
// activations of group kq (zero rows past the tokens), and the accumulator input is each
// token's bias term summed over the scale group (a lane-group sum at staging), so the
// decode's 1024 / 64 offsets cancel exactly as on the vector ALUs.  The decode is shared by
// every token; what the tokens add is one matrix-core product per column and block.
// ======================================================================================
// Byte c = i of rows r (bits 0-7) and r + 1 (bits 16-23) of the lane's row pair pp in block j,
// ready for the nibble and-or (the other bits are masked off).  [K/2, N] layout: one byte
// permute per column.  Prepacked: the unit already holds rows r and r + 1 of columns 2m, 2m + 1
// as (r, 2m), (r, 2m + 1), (r + 1, 2m), (r + 1, 2m + 1) in dword m, so column 2m is that dword
// and column 2m + 1 the dword shifted by 8: one shift per two columns.
template <bool PRE>
__device__ __forceinline__ uint32_t row_pair(const uint2 (&w)[16], int j, int pp, int i) {
  const uint2 ra = w[4 * j + 2 * pp], rb = w[4 * j + 2 * pp + 1];
  if constexpr (PRE) {
    const int m = i >> 1;
    const uint32_t d = m == 0 ? ra.x : m == 1 ? ra.y : m == 2 ? rb.x : rb.y;
    return (i & 1) ? d >> 8 : d;
  } else {
    const uint32_t sel = (uint32_t)(i & 3) | ((uint32_t)((i & 3) + 4) << 16);
    return __builtin_amdgcn_perm(i < 4 ? rb.x : rb.y, i < 4 ? ra.x : ra.y, sel);
  }
}

constexpr int GV_ROUND = 16;  // blocks per round of a workgroup: 4 waves x 4 blocks
constexpr int GV_MAX_T = 4;   // tokens of this kernel (more take the expert tiles' E = 1 case)
constexpr int GV_PRE_MAX_T = 4;  // tokens of the GEMV on prepacked weights

template <int G, int NT, bool PRE, bool MF = false>
__global__ void __launch_bounds__(EX_THREADS) gemv_tok_kernel(GemvArgs g) {
  // activations of a round, per token and 8 K: (x0,x2),(x1,x3),(x4,x6),(x5,x7) and the bias
  __shared__ __align__(16) uint4 xs[NT][GV_ROUND * 4];
  __shared__ float cs[NT][GV_ROUND * 4];
  // matrix-core body: the bias of each token summed per scale group of the round (G = 128:
  // a wave's 4 blocks; G = 32: one block)
  __shared__ float bs[MF ? NT : 1][GV_ROUND];
  __shared__ __align__(16) float red[4][MF ? 1 : 4][NT][128];  // [wave][row lane][token][column]
  static_assert(NT * GV_ROUND * 4 <= EX_THREADS, "one activation group per thread");
  static_assert(!MF || NT == 4, "the matrix-core body serves 2 to 4 tokens");
  const int K = g.K, N = g.N, S = g.S, Tc = g.t_cap;  // g.T <= NT
  const int tiles = (N + 127) / 128;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, q = l & 15, kq = l >> 4;
  const __amdgpu_buffer_rsrc_t pr = ex_rsrc(g.part);
  const int Wc = tiles * S;
  if ((int)blockIdx.x >= Wc) {
    // finisher of one tile: the S split partials in split order, polled with the shortest
    // backoff (measured against 8 units: N = 8192 7.35 -> 7.18 us, N = 34816 18.6-18.8 ->
    // 18.5 us; the finishers are the last step of the call, and there are few of them)
    const int tile = blockIdx.x - Wc;
    const int ncols = min(128, N - 128 * tile);
    for (int it = tid; it < NT * 128; it += EX_THREADS) {
      const int t = it >> 7, c = it & 127;
      if (t >= g.T || c >= ncols) continue;
      float y = 0.0f;
      for (int p0 = 0; p0 < S; p0 += 16) {
        int off[16];
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          off[i] = ((min(p0 + i, S - 1) * Tc + t) * N + 128 * tile + c) * 4;
        if (!take16<1>(pr, off, min(16, S - p0), v) && g.err) atomicOr(g.err, 2);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (p0 + i < S) y += v[i];
      }
      g.y[(size_t)t * N + 128 * tile + c] = f32_to_bf16(y + 0.0f);  // -0.0 sums become +0.0
    }
    return;
  }
  const int tile = blockIdx.x % tiles, s = blockIdx.x / tiles;
  const int nblk = K / 32;
  const int blk0 = s * g.wb, blk1 = min(blk0 + g.wb, nblk);
  const int ncols = min(128, N - 128 * tile);
  const int col = 128 * tile + 8 * q;
  const bool col_ok = 8 * q < ncols;
  const int ld = PRE ? 128 * tiles : N;  // scale row stride
  const __amdgpu_buffer_rsrc_t wr =
      view_rsrc(g.w, PRE ? (size_t)tiles * K * 64 : (size_t)(K / 2) * N);
  const __amdgpu_buffer_rsrc_t sr = view_rsrc(g.s, (size_t)(K / G) * ld * 2);
  const __amdgpu_buffer_rsrc_t xr = view_rsrc(g.x, (size_t)g.T * K * 2);
  constexpr int NS = G == 128 ? 1 : 4;  // scale loads per chunk
  // staging: thread tid < 64 NT converts the 8 activations of group tid % 64 of token tid / 64
  const int xt = tid / (GV_ROUND * 4), xg = tid - xt * (GV_ROUND * 4);
  // fp16 constants kept in registers so that each nibble takes one v_and_or_b32
  uint32_t M_LO = 0x000F000Fu, M_HI = 0x00F000F0u, F_LO = 0x64006400u, F_HI = 0x54005400u;
  asm volatile("" : "+s"(M_LO), "+s"(M_HI), "+v"(F_LO), "+v"(F_HI));
  float acc[NT][8];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[tt][i] = 0.0f;
  float macc[MF ? 8 : 1][4];  // matrix-core body: [column i][token 4 kq + r]
#pragma unroll
  for (int i = 0; i < (MF ? 8 : 1); ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) macc[i][r] = 0.0f;
  for (int r0 = blk0; r0 < blk1; r0 += GV_ROUND) {
    // The round's activations are loaded before its weights: in-order completion then lets
    // the staging threads convert them while the weights are still in flight.  Groups past
    // the split load as zero.
    const int k0 = 32 * r0 + 8 * xg;
    const int xo = (xt < g.T && k0 < 32 * blk1) ? (xt * K + k0) * 2 : EX_OOB;
    const u32x4_t xv4 = __builtin_amdgcn_raw_buffer_load_b128(xr, xo, 0, 0);
    // the wave's scales and 4 blocks of the round (blocks past blk1 load as zero); the
    // scales go first, so that work the compiler places on them waits for no weight
    uint2 w[16];
    uint4 sc[NS];
    const int cb = r0 + 4 * wv;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int o = (col_ok && cb + j < blk1) ? ((32 * (cb + j) / G) * ld + col) * 2 : EX_OOB;
      const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(sr, o, 0, EX_STREAM);
      sc[j] = make_uint4(d.x, d.y, d.z, d.w);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (PRE) {
        const int b = cb + j, rd = b >> 4;  // block b of round rd
        const int o = (col_ok && b < blk1)
                          ? (16 * rd * tiles + tile * min(16, nblk - 16 * rd) + (b & 15)) * 2048 +
                                16 * l
                          : EX_OOB;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(wr, o, 1024 * h, EX_STREAM);
          w[4 * j + 2 * h] = make_uint2(d.x, d.y);
          w[4 * j + 2 * h + 1] = make_uint2(d.z, d.w);
        }
      } else {
        const int o = (col_ok && cb + j < blk1) ? (16 * (cb + j) + 4 * kq) * N + col : EX_OOB;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const u32x2_t d = __builtin_amdgcn_raw_buffer_load_b64(wr, o, r * N, EX_STREAM);
          w[4 * j + r] = make_uint2(d.x, d.y);
        }
      }
    }
    if (r0 != blk0) __syncthreads();  // the previous round is done with xs / cs
    if (xt < NT) {  // paired fp16 order and the bias term of the 8 values
      const uint32_t h01 = bf16pair_to_f16pair(xv4.x), h23 = bf16pair_to_f16pair(xv4.y);
      const uint32_t h45 = bf16pair_to_f16pair(xv4.z), h67 = bf16pair_to_f16pair(xv4.w);
      const uint32_t e0 = __builtin_amdgcn_perm(h23, h01, 0x05040100u);
      const uint32_t o0 = __builtin_amdgcn_perm(h23, h01, 0x07060302u);
      const uint32_t e1 = __builtin_amdgcn_perm(h67, h45, 0x05040100u);
      const uint32_t o1 = __builtin_amdgcn_perm(h67, h45, 0x07060302u);
      xs[xt][xg] = make_uint4(e0, o0, e1, o1);
      const uint32_t m1032 = 0xE408E408u, m72 = 0xD480D480u;  // fp16 (-1032, -1032), (-72, -72)
      float c = dot2p<FMT_INT4>(e0, m1032, 0.0f);
      c = dot2p<FMT_INT4>(o0, m72, c);
      c = dot2p<FMT_INT4>(e1, m1032, c);
      c = dot2p<FMT_INT4>(o1, m72, c);
      cs[xt][xg] = c;
      if constexpr (MF) {  // sum the group's bias terms over the lanes of one scale group
        constexpr int W = G == 128 ? 16 : 4;  // 8-K groups per scale group
#pragma unroll
        for (int m = 1; m < W; m <<= 1) c += __shfl_xor(c, m, W);
        if ((xg & (W - 1)) == 0) bs[xt][xg / W] = c;
      }
    }
    __syncthreads();
    if constexpr (MF) {
      // lane (q, kq): A = token q's 8 K values of group kq (zero past the tokens), B = the
      // 8 K values of column 8 q + i, one 16x16x32 product per column i: the 16 columns
      // 8 q' + i of a product are the lanes' i-th columns.  D rows 4 kq .. 4 kq + 3 are
      // tokens; the accumulator input carries the tokens' bias term of the scale group.
      f32x4_t D[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gi = (4 * wv + j) * 4 + kq;
        const uint4 av = q < NT ? xs[q][gi] : make_uint4(0u, 0u, 0u, 0u);
        if (G != 128 || j == 0) {
          f32x4_t c0;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            c0[r] = 4 * kq + r < NT ? bs[4 * kq + r][G == 128 ? wv : 4 * wv + j] : 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) D[i] = c0;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t bv[4];
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const uint32_t p = row_pair<PRE>(w, j, pp, i);
            bv[2 * pp] = (p & M_LO) | F_LO;
            bv[2 * pp + 1] = (p & M_HI) | F_HI;
          }
          const u32x4_t B = {bv[0], bv[1], bv[2], bv[3]};
          D[i] = mfma_16x16x32<FMT_INT4>(av, B, D[i]);
        }
        if (G != 128 || j == 3) {
          float sf[8];
          scales8(sc[G == 128 ? 0 : j], sf);
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) macc[i][r] = fmaf(sf[i], D[i][r], macc[i][r]);
        }
      }
      continue;
    }
    float d[NT][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gi = (4 * wv + j) * 4 + kq;  // the lane's 8 K values of its block j
      uint4 xv[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        xv[tt] = xs[tt][gi];
        const float cc = cs[tt][gi];
#pragma unroll
        for (int i = 0; i < 8; ++i) d[tt][i] = (G == 128 && j > 0) ? d[tt][i] + cc : cc;
      }
      // each pair is decoded once and meets every token
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const uint32_t p = row_pair<PRE>(w, j, pp, i);
          const uint32_t lo = (p & M_LO) | F_LO, hi = (p & M_HI) | F_HI;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            d[tt][i] = dot2p<FMT_INT4>(lo, pp == 0 ? xv[tt].x : xv[tt].z, d[tt][i]);
            d[tt][i] = dot2p<FMT_INT4>(hi, pp == 0 ? xv[tt].y : xv[tt].w, d[tt][i]);
          }
        }
      }
      if (G != 128 || j == 3) {
        float sf[8];
        scales8(sc[G == 128 ? 0 : j], sf);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[tt][i] = fmaf(sf[i], d[tt][i], acc[tt][i]);
      }
    }
  }
  if constexpr (MF) {
    if (kq == 0)  // tokens 0 .. 3
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wv][0][r][8 * q + i] = macc[i][r];
  } else {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wv][kq][tt][8 * q + i] = acc[tt][i];
  }
  __syncthreads();
  for (int it = tid; it < NT * 128; it += EX_THREADS) {
    const int t = it >> 7, c = it & 127;
    if (t >= g.T || c >= ncols) continue;
    float v = 0.0f;
    if constexpr (MF) {
#pragma unroll
      for (int p = 0; p < 4; ++p) v += red[p][0][t][c];
    } else {
#pragma unroll
      for (int p = 0; p < 16; ++p) v += red[p >> 2][p & 3][t][c];
    }
    if (S == 1)
      g.y[(size_t)t * N + 128 * tile + c] = f32_to_bf16(v + 0.0f);
    else
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pub1(v)), pr,
                                            ((s * Tc + t) * N + 128 * tile + c) * 4, 0,
                                            EX_CPOL_SC1);
  }
}

// tokens per vector-ALU pass for calls with T tokens (no expert has more than T)
static int valu_width(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : EX_VT; }

hipError_t launch_gemv_ex(const GemvArgs& g, int mt, hipStream_t st) {
  if (mt == 0) {
    // gemv_tok_kernel: one token on the vector ALUs, 2 to 4 on its matrix-core body; whole
    // rounds of GV_ROUND blocks per split, at most the plan's S splits
    if (g.T < 1 || g.T > GV_MAX_T) return hipErrorInvalidValue;
    GemvArgs h = g;
    const int nblk = g.K / 32, tiles = (g.N + 127) / 128;
    const int per = (nblk + g.S - 1) / g.S;
    h.wb = GV_ROUND * ((per + GV_ROUND - 1) / GV_ROUND);
    h.S = (nblk + h.wb - 1) / h.wb;
    const dim3 grid1(tiles * h.S + (h.S > 1 ? tiles : 0));
    if (g.group == 128) {
      if (g.T == 1) hipLaunchKernelGGL((gemv_tok_kernel<128, 1, false>), grid1, dim3(EX_THREADS), 0, st, h);
      else hipLaunchKernelGGL((gemv_tok_kernel<128, 4, false, true>), grid1, dim3(EX_THREADS), 0, st, h);
    } else {
      if (g.T == 1) hipLaunchKernelGGL((gemv_tok_kernel<32, 1, false>), grid1, dim3(EX_THREADS), 0, st, h);
      else hipLaunchKernelGGL((gemv_tok_kernel<32, 4, false, true>), grid1, dim3(EX_THREADS), 0, st, h);
    }
    return hipGetLastError();
  }
  const dim3 grid((g.N + 127) / 128, g.S + (g.S > 1 ? 1 : 0)), block(EX_THREADS);
  // more tokens: matrix-core tiles of 16 (mt = 1) or 32 (mt = 2) rows per pass
  if (mt == 1)
    hipLaunchKernelGGL((gemv_ex_kernel<1, 1>), grid, block, 0, st, g);
  else if (mt == 2)
    hipLaunchKernelGGL((gemv_ex_kernel<2, 1>), grid, block, 0, st, g);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int ex_max_split_gemv() { return EX_MAX_SPLIT_GEMV; }

// the GEMV on the prepacked layout: one token on the vector ALUs, 2 to 4 tokens on the
// matrix-core body of the same kernel; whole rounds per split as launch_gemv_ex
hipError_t launch_gemv_tiled(const GemvArgs& g, hipStream_t st) {
  if (g.T < 1 || g.T > GV_PRE_MAX_T) return hipErrorInvalidValue;
  GemvArgs h = g;
  const int nblk = g.K / 32, tiles = (g.N + 127) / 128;
  const int per = (nblk + g.S - 1) / g.S;
  h.wb = GV_ROUND * ((per + GV_ROUND - 1) / GV_ROUND);
  h.S = (nblk + h.wb - 1) / h.wb;
  const dim3 grid(tiles * h.S + (h.S > 1 ? tiles : 0)), block(EX_THREADS);
  // one token: the vector-ALU body; 2 to 4 tokens: the matrix-core body (measured at
  // N = 34816: 2 tokens 20.6-21.4 vs 22.3-22.6 us, 4 tokens 22.3 vs 30.0 us; one token
  // 20.0 vs 18.9 us, the products of three zero rows do not pay for the saved dot2 work);
  // the same instances as launch_gemv_ex on the [K/2, N] layout, so both calls agree bitwise
  // The one-token instance on this layout needs 78 registers and would run 6 waves per SIMD;
  // it is held at 4 workgroups per compute unit (the occupancy of the [K/2, N] instance) by
  // reserving unused LDS up to 39 KB per workgroup: with more workgroups in flight the call
  // is slower (measured: 6 waves per SIMD 18.85 vs 18.51 us at N = 34816).
  constexpr size_t kT1Lds = 39 * 1024 - 9472;  // 9472 bytes: the instance's own LDS
#define DQG_GT_LAUNCH(GG, NN, MM, LDS) \
  hipLaunchKernelGGL((gemv_tok_kernel<GG, NN, true, MM>), grid, block, LDS, st, h)
  if (g.group == 128) {
    if (g.T == 1) DQG_GT_LAUNCH(128, 1, false, kT1Lds);
    else DQG_GT_LAUNCH(128, 4, true, 0);
  } else {
    if (g.T == 1) DQG_GT_LAUNCH(32, 1, false, kT1Lds);
    else DQG_GT_LAUNCH(32, 4, true, 0);
  }
#undef DQG_GT_LAUNCH
  return hipGetLastError();
}

// Rearranges w [K/2, N] and s [K/G, N] into the prepacked layout that gemv_tok_kernel<.., true>
// reads: one thread per 16-byte unit, a grid-stride loop over the weight units, then the
// scale units.
__global__ void __launch_bounds__(256) gemv_prepack_kernel(const uint8_t* __restrict__ w,
                                                           const uint16_t* __restrict__ s,
                                                           int K, int N, int G,
                                                           uint8_t* __restrict__ wt,
                                                           uint16_t* __restrict__ st) {
  const int nb = K / 32, ng = K / G, tiles = (N + 127) / 128;
  const long long nw = (long long)tiles * nb * 128, ns = (long long)tiles * ng * 16;
  for (long long u = blockIdx.x * 256LL + threadIdx.x; u < nw + ns; u += (long long)gridDim.x * 256) {
    if (u < nw) {
      // unit u of the output: round st, tile t, block b of the tile (nbi blocks per tile
      // in this round)
      const int l = (int)(u & 63), h = (int)((u >> 6) & 1);
      const long long ob = u >> 7;  // output block
      const int st = (int)(ob / (16LL * tiles));
      const int nbi = min(16, nb - 16 * st);
      const int rem = (int)(ob - 16LL * tiles * st);
      const int t = rem / nbi, b = 16 * st + rem % nbi;
      const int r = 16 * b + 4 * (l >> 4) + 2 * h, c = 128 * t + 8 * (l & 15);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (c < N) {
        const uint2 a = *reinterpret_cast<const uint2*>(w + (size_t)r * N + c);
        const uint2 b2 = *reinterpret_cast<const uint2*>(w + (size_t)(r + 1) * N + c);
        // dword m: (r, 2m), (r, 2m + 1), (r + 1, 2m), (r + 1, 2m + 1) of the 8 columns
        v = make_uint4((a.x & 0xFFFFu) | (b2.x << 16), (a.x >> 16) | (b2.x & 0xFFFF0000u),
                       (a.y & 0xFFFFu) | (b2.y << 16), (a.y >> 16) | (b2.y & 0xFFFF0000u));
      }
      reinterpret_cast<uint4*>(wt)[u] = v;
    } else {
      const long long v_ = u - nw;  // 8 scales of row gr, columns c .. c + 7
      const int gr = (int)(v_ / (16LL * tiles)), c = 8 * (int)(v_ % (16LL * tiles));
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (c < N) v = *reinterpret_cast<const uint4*>(s + (size_t)gr * N + c);
      reinterpret_cast<uint4*>(st)[v_] = v;
    }
  }
}

hipError_t launch_gemv_prepack(const uint8_t* w, const uint16_t* s, int K, int N, int group,
                               uint8_t* wt, uint16_t* st_, hipStream_t st) {
  const long long tiles = (N + 127) / 128;
  const long long units = tiles * (K / 32) * 128 + tiles * (K / group) * 16;
  const long long want = (units + 255) / 256, grid = want < 65536 ? want : 65536;
  hipLaunchKernelGGL(gemv_prepack_kernel, dim3((unsigned)grid), dim3(256), 0, st, w, s, K, N,
                     group, wt, st_);
  return hipGetLastError();
}

// ---- launchers --------------------------------------------------------------------------------
template <int FMT, int MT, int VT, bool MIX>
static hipError_t launch_phase(const MoeArgs& a, int A, bool down, hipStream_t st) {
  if (!down) {
    // unsplit gate_up workgroups stream all of K: they prefetch each next batch's weights
    // (measured faster there, slower for the short streams of split launches)
    const dim3 grid((a.I + 127) / 128, a.S_gu + (a.S_gu > 1 ? 1 : 0), A);
    if (a.S_gu == 1)
      hipLaunchKernelGGL((gateup_ex_kernel<FMT, MT, VT, MIX, true>), grid, dim3(EX_THREADS), 0,
                         st, a);
    else
      hipLaunchKernelGGL((gateup_ex_kernel<FMT, MT, VT, MIX, false>), grid, dim3(EX_THREADS), 0,
                         st, a);
  } else {
    const int zc = a.combine ? (a.T + EX_COMBINE_TOKENS - 1) / EX_COMBINE_TOKENS : 0;
    hipLaunchKernelGGL((down_ex_kernel<FMT, MT, VT, MIX>), dim3((a.H + 127) / 128, a.S_dn, A + zc),
                       dim3(EX_THREADS), 0, st, a);
  }
  return hipGetLastError();
}

template <int FMT, bool MIX = false>
static hipError_t launch_ex_t(const MoeArgs& a0, int A, int mt, hipStream_t st) {
  // one launch per phase: with matrix-core tiles (mt > 0) the kernel serves the experts
  // below the threshold with EX_VT-token vector-ALU passes in the same launch
  const int vt = valu_width(a0.T);
  MoeArgs a = a0;
  for (int down = 0; down < 2; ++down) {
    a.combine = down;  // the down launch also runs the per-token combiners
    hipError_t e;
    if (mt == 1) e = launch_phase<FMT, 1, EX_VT, MIX>(a, A, down, st);
    else if (vt == 1) e = launch_phase<FMT, 0, 1, MIX>(a, A, down, st);
    else if (vt == 2) e = launch_phase<FMT, 0, 2, MIX>(a, A, down, st);
    else e = launch_phase<FMT, 0, EX_VT, MIX>(a, A, down, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_moe_experts(const MoeArgs& a, int A, int mt, hipStream_t st) {
  if (mt < 0 || mt > 1) return hipErrorInvalidValue;
  if (a.efmt) {  // a mixed layer: FP4 experts with 2-bit cold ones
    if (a.fmt != FMT_FP4) return hipErrorInvalidValue;
    return launch_ex_t<FMT_FP4, true>(a, A, mt, st);
  }
  if (a.fmt == FMT_FP4) return launch_ex_t<FMT_FP4>(a, A, mt, st);
  if (a.fmt == FMT_INT4) return launch_ex_t<FMT_INT4>(a, A, mt, st);
  if (a.fmt == FMT_FP8) return launch_ex_t<FMT_FP8>(a, A, mt, st);
  return hipErrorInvalidValue;
}

int ex_max_split() { return EX_MAX_SPLIT; }

}  // namespace dqg
