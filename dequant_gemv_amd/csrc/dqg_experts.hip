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
constexpr int EX_RB = 4;          // blocks in flight per wave
constexpr int EX_VT = 4;          // tokens per vector-ALU pass
constexpr int EX_LDS = 8192;      // floats of LDS: operand staging, then the reductions
constexpr int EX_MAX_SPLIT = 8;   // gate_up K splits summed by the finalizer
constexpr int EX_CPOL_SC1 = 16;   // cache policy: agent-coherent access

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---- schedule entries, clamped ------------------------------------------------------------
// Whatever the workspace holds, no index derived from it leaves the call's buffers.
__device__ __forceinline__ bool expert_range(const MoeArgs& a, int act, int* beg, int* cnt,
                                             int* e) {
  const int TK = a.T * a.k;
  const int b = min(max(a.ws.act_off[act], 0), TK);
  const int en = min(max(a.ws.act_off[act + 1], b), TK);
  *beg = b;
  *cnt = en - b;
  *e = a.ws.act_expert[act];
  return *e >= 0 && *e < a.E;
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
__device__ __forceinline__ float4 ld4_sc1(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, EX_CPOL_SC1);
  return make_float4(__uint_as_float(d.x), __uint_as_float(d.y), __uint_as_float(d.z),
                     __uint_as_float(d.w));
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

__device__ __forceinline__ void load_wblock(const uint8_t* w, const uint16_t* s, size_t ld,
                                            int group, int blk, int kg, int col, bool ok,
                                            WBlock& o) {
  if (!ok) {
    o.w[0] = o.w[1] = o.w[2] = o.w[3] = make_uint2(0u, 0u);
    o.s = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const uint8_t* p = w + (size_t)(16 * blk + 4 * kg) * ld + col;
#pragma unroll
  for (int j = 0; j < 4; ++j) o.w[j] = *reinterpret_cast<const uint2*>(p + (size_t)j * ld);
  o.s = *reinterpret_cast<const uint4*>(s + (size_t)((32 * blk) / group) * ld + col);
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

// ---- the two compute bodies -----------------------------------------------------------------
// Operand source of a phase: gate_up reads bf16 x rows (token = slot / k), down reads fp32
// h rows (by slot).
struct OpSrc {
  const uint16_t* x;  // gate_up
  const float* h;     // down
  int row_elems;      // H (x) or I (h)
  int k;
};
template <int FMT>
__device__ __forceinline__ uint4 load_op(const OpSrc& src, int slot, int q8) {
  if (slot < 0) return make_uint4(0u, 0u, 0u, 0u);
  if (src.x) return op_from_bf16<FMT>(src.x + (size_t)(slot / src.k) * src.row_elems, q8);
  return op_from_f32<FMT>(src.h + (size_t)slot * src.row_elems, q8);
}

template <int FMT, int I>
__device__ __forceinline__ void valu_col(const WBlock& b, float sc, const uint4 (&op)[EX_VT],
                                         int nch, float (&acc)[EX_VT][8]) {
  const u32x4_t P = decode_col<FMT, I>(b);
#pragma unroll
  for (int t = 0; t < EX_VT; ++t) {
    if (t < nch) {
      float d = dot2p<FMT>(P.x, op[t].x, 0.0f);
      d = dot2p<FMT>(P.y, op[t].y, d);
      d = dot2p<FMT>(P.z, op[t].z, d);
      d = dot2p<FMT>(P.w, op[t].w, d);
      acc[t][I] = fmaf(sc, d, acc[t][I]);
    }
  }
}
template <int FMT>
__device__ __forceinline__ void valu_cols(const WBlock& b, const float (&sf)[8],
                                          const uint4 (&op)[EX_VT], int nch,
                                          float (&acc)[EX_VT][8]) {
  valu_col<FMT, 0>(b, sf[0], op, nch, acc);
  valu_col<FMT, 1>(b, sf[1], op, nch, acc);
  valu_col<FMT, 2>(b, sf[2], op, nch, acc);
  valu_col<FMT, 3>(b, sf[3], op, nch, acc);
  valu_col<FMT, 4>(b, sf[4], op, nch, acc);
  valu_col<FMT, 5>(b, sf[5], op, nch, acc);
  valu_col<FMT, 6>(b, sf[6], op, nch, acc);
  valu_col<FMT, 7>(b, sf[7], op, nch, acc);
}

// Vector-ALU pass over up to EX_VT tokens (s_slot[0 .. nch)), blocks b = first, first +
// step, ... < b1.  The tokens' operands for blocks [b0, b1) are staged in LDS first.
// acc[t][i]: token t, column col + i, summed over this lane's rows.
template <int FMT>
__device__ __forceinline__ void valu_pass(const uint8_t* w, const uint16_t* s, size_t ld,
                                          int group, int col, bool col_ok, const OpSrc& src,
                                          const int* s_slot, int nch, int b0, int b1,
                                          int first, int step, float* lds,
                                          float (&acc)[EX_VT][8]) {
  const int tid = threadIdx.x, kg = (tid & 63) >> 4;
  const int nb = b1 - b0;
  uint4* ops = reinterpret_cast<uint4*>(lds);  // [t][block - b0][kg]
  for (int i = tid; i < nch * nb * 4; i += EX_THREADS) {
    const int t = i / (nb * 4), r = i - t * (nb * 4);
    ops[i] = load_op<FMT>(src, s_slot[t], 4 * b0 + r);
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < EX_VT; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = 0.0f;
  for (int bb = first; bb < b1; bb += step * EX_RB) {
    WBlock wb[EX_RB];
#pragma unroll
    for (int r = 0; r < EX_RB; ++r)
      if (bb + step * r < b1) load_wblock(w, s, ld, group, bb + step * r, kg, col, col_ok, wb[r]);
#pragma unroll
    for (int r = 0; r < EX_RB; ++r) {
      const int b = bb + step * r;
      if (b < b1) {
        float sf[8];
        scales8(wb[r].s, sf);
        uint4 op[EX_VT];
#pragma unroll
        for (int t = 0; t < EX_VT; ++t)
          if (t < nch) op[t] = ops[(t * nb + (b - b0)) * 4 + kg];
        valu_cols<FMT>(wb[r], sf, op, nch, acc);
      }
    }
  }
  __syncthreads();  // the staged operands are dead; the LDS is reused by the reductions
}

template <int FMT, int MT, int I>
__device__ __forceinline__ void mfma_col(const WBlock& b, float sc, const uint4 (&A)[MT],
                                         int nmt, f32x4_t (&acc)[MT][8]) {
  const u32x4_t B = decode_col<FMT, I>(b);
  const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < nmt) {
      const f32x4_t D = mfma_16x16x32<FMT>(A[m], B, zero);
      acc[m][I] += sc * D;
    }
  }
}

// Matrix-core pass over up to 16 MT tokens: M-tile m covers tokens 16 m .. 16 m + 15 of
// s_slot.  acc[m][i][r]: token 16 m + 4 kg + r, column col + i (D layout of the MFMA).
template <int FMT, int MT>
__device__ __forceinline__ void mfma_pass(const uint8_t* w, const uint16_t* s, size_t ld,
                                          int group, int col, bool col_ok, const OpSrc& src,
                                          const int* s_slot, int nch, int b1, int first,
                                          int step, f32x4_t (&acc)[MT][8]) {
  const int l = threadIdx.x & 63, q = l & 15, kg = l >> 4;
  const int nmt = (nch + 15) >> 4;
  int slot[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) slot[m] = (16 * m + q < nch) ? s_slot[16 * m + q] : -1;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[m][i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int bb = first; bb < b1; bb += step * EX_RB) {
    WBlock wb[EX_RB];
    uint4 A[EX_RB][MT];
#pragma unroll
    for (int r = 0; r < EX_RB; ++r) {
      const int b = bb + step * r;
      if (b < b1) {
        load_wblock(w, s, ld, group, b, kg, col, col_ok, wb[r]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          A[r][m] = (m < nmt) ? load_op<FMT>(src, slot[m], 4 * b + kg) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int r = 0; r < EX_RB; ++r) {
      if (bb + step * r < b1) {
        float sf[8];
        scales8(wb[r].s, sf);
        mfma_col<FMT, MT, 0>(wb[r], sf[0], A[r], nmt, acc);
        mfma_col<FMT, MT, 1>(wb[r], sf[1], A[r], nmt, acc);
        mfma_col<FMT, MT, 2>(wb[r], sf[2], A[r], nmt, acc);
        mfma_col<FMT, MT, 3>(wb[r], sf[3], A[r], nmt, acc);
        mfma_col<FMT, MT, 4>(wb[r], sf[4], A[r], nmt, acc);
        mfma_col<FMT, MT, 5>(wb[r], sf[5], A[r], nmt, acc);
        mfma_col<FMT, MT, 6>(wb[r], sf[6], A[r], nmt, acc);
        mfma_col<FMT, MT, 7>(wb[r], sf[7], A[r], nmt, acc);
      }
    }
  }
}

// ======================================================================================
// gate_up + SiLU*up.  Grid: x = 128-column h tile, y = K split, z = active-expert index.
// Waves: w & 1 = gate (0) or up (1) columns, w >> 1 = even or odd blocks of the split.
// ======================================================================================
template <int FMT, int MT>
__global__ void __launch_bounds__(EX_THREADS) gateup_ex_kernel(MoeArgs a) {
  __shared__ __align__(16) float lds[EX_LDS];
  __shared__ int s_slot[64];
  __shared__ int s_flag;
  const int act = blockIdx.z;
  if (act >= *a.ws.n_active) return;
  int beg, cnt, e;
  if (!expert_range(a, act, &beg, &cnt, &e) || cnt == 0) return;
  const int H = a.H, I = a.I, k = a.k, TK = a.T * k;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, q = l & 15, kg = l >> 4;
  const int role = wv & 1, khalf = wv >> 1;
  const int nt = blockIdx.x, S = gridDim.y, s = blockIdx.y;
  const int nblk = H / 32;
  const int b0 = (s * nblk) / S, b1 = ((s + 1) * nblk) / S;
  const size_t ld = 2 * (size_t)I;
  const int n0 = 128 * nt;                 // first h column of the tile
  const int ncols = min(128, I - n0);      // valid h columns (64 or 128)
  const bool col_ok = 8 * q < ncols;
  const int col = role * I + n0 + 8 * q;
  const uint8_t* w = a.wgu + (size_t)e * (H / 2) * ld;
  const uint16_t* sc = a.sgu + (size_t)e * (H / a.group) * ld;
  const OpSrc src{a.x, nullptr, H, k};
  const bool use_mfma = MT > 0 && cnt >= a.mfma_min;
  const int vt = min(EX_VT, EX_LDS / (16 * (b1 - b0)));
  const int CH = use_mfma ? 16 * (MT > 0 ? MT : 1) : vt;
  const __amdgpu_buffer_rsrc_t pr = ex_rsrc(a.ws.part_gu);

  // emit the totals of (token m of the pass, 4 columns c4 .. c4+3) of the tile
  auto emit = [&](int slot, int c4, float4 g, float4 u) {
    if (S == 1) {
      *reinterpret_cast<float4*>(a.ws.h + (size_t)slot * I + n0 + c4) =
          make_float4(silu_mul(g.x, u.x), silu_mul(g.y, u.y), silu_mul(g.z, u.z),
                      silu_mul(g.w, u.w));
    } else {
      const int base = ((s * TK + slot) * 2 * I + n0 + c4) * 4;
      st4_sc1(pr, base, g);
      st4_sc1(pr, base + 4 * I, u);
    }
  };

  for (int m0 = 0; m0 < cnt; m0 += CH) {
    const int nch = min(CH, cnt - m0);
    __syncthreads();
    if (tid < nch) s_slot[tid] = slot_at(a, beg + m0 + tid);
    __syncthreads();
    if constexpr (MT > 0) {
      if (use_mfma) {
        f32x4_t acc[MT][8];
        mfma_pass<FMT, MT>(w, sc, ld, a.group, col, col_ok, src, s_slot, nch, b1, b0 + khalf,
                           2, acc);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (16 * m >= nch) break;
          __syncthreads();
          // red[role][khalf][token 0..15][column 0..127]
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              lds[((role * 2 + khalf) * 16 + 4 * kg + r) * 128 + 8 * q + i] = acc[m][i][r];
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
        }
        continue;
      }
    }
    float acc[EX_VT][8];
    valu_pass<FMT>(w, sc, ld, a.group, col, col_ok, src, s_slot, nch, b0, b1, b0 + khalf, 2,
                   lds, acc);
    // two halves of 4 tokens: red[role][khalf][kg][token 0..3][column 0..127]
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (4 * hh >= nch) break;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          lds[((((role * 2 + khalf) * 4 + kg) * 4 + t) * 128) + 8 * q + i] = acc[4 * hh + t][i];
      __syncthreads();
      if (tid < 4 * 32) {
        const int t = tid >> 5, c4 = 4 * (tid & 31);
        const int slot = (4 * hh + t < nch) ? s_slot[4 * hh + t] : -1;
        if (slot >= 0 && c4 < ncols) {
          const float4* r4 = reinterpret_cast<const float4*>(lds);
          float4 g = make_float4(0.0f, 0.0f, 0.0f, 0.0f), u = g;
#pragma unroll
          for (int p = 0; p < 8; ++p) {  // p = khalf * 4 + kg
            g = f4_add(g, r4[(((0 * 8 + p) * 4 + t) * 128 + c4) / 4]);
            u = f4_add(u, r4[(((1 * 8 + p) * 4 + t) * 128 + c4) / 4]);
          }
          emit(slot, c4, g, u);
        }
      }
      __syncthreads();
    }
  }
  if (S == 1) return;

  // the last K split of this (expert, tile) sums the partials in split order
  unsigned* counter = a.ws.cnt_gu + (size_t)act * gridDim.x + nt;
  if (!last_arriver(counter, (unsigned)S, &s_flag)) return;
  for (int it = tid; it < cnt * 32; it += EX_THREADS) {
    const int t = it >> 5, c4 = 4 * (it & 31);
    if (c4 >= ncols) continue;
    const int slot = slot_at(a, beg + t);
    if (slot < 0) continue;
    float4 gv[EX_MAX_SPLIT], uv[EX_MAX_SPLIT];
#pragma unroll
    for (int p = 0; p < EX_MAX_SPLIT; ++p) {
      if (p >= S) break;
      const int base = ((p * TK + slot) * 2 * I + n0 + c4) * 4;
      gv[p] = ld4_sc1(pr, base);
      uv[p] = ld4_sc1(pr, base + 4 * I);
    }
    float4 g = gv[0], u = uv[0];
#pragma unroll
    for (int p = 1; p < EX_MAX_SPLIT; ++p) {
      if (p >= S) break;
      g = f4_add(g, gv[p]);
      u = f4_add(u, uv[p]);
    }
    *reinterpret_cast<float4*>(a.ws.h + (size_t)slot * I + n0 + c4) =
        make_float4(silu_mul(g.x, u.x), silu_mul(g.y, u.y), silu_mul(g.z, u.z),
                    silu_mul(g.w, u.w));
  }
}

// ======================================================================================
// down + top-k combine.  Grid: x = 128-column output tile, y = K split over I, z =
// active-expert index.  All 4 waves share the columns; wave w takes blocks b0 + w + 4 i.
// ======================================================================================
// out[t, tile] = bf16(residual + sum_j w_j * sum_s part[s][t k + j]) in ascending j, s
template <int NB>
__device__ __forceinline__ void combine4(const MoeArgs& a, __amdgpu_buffer_rsrc_t pr, int t,
                                         int m, int S) {
  const int k = a.k, TK = a.T * k, H = a.H;
  const int JB = max(1, NB / S);
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j0 = 0; j0 < k; j0 += JB) {
    float4 v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int j = j0 + u / S, p = u % S;
      v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (u < JB * S && j < k) {
        const int slot = t * k + j;
        const int e = a.ids[slot];
        if (e >= 0 && e < a.E) v[u] = ld4_sc1(pr, ((p * TK + slot) * H + m) * 4);
      }
    }
    float4 y = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int j = j0 + u / S, p = u % S;
      y = f4_add(y, v[u]);  // zero beyond the batch
      if (u < JB * S && j < k && p == S - 1) {
        const int slot = t * k + j;
        const int e = a.ids[slot];
        const float wj = (e >= 0 && e < a.E) ? a.wts[slot] : 0.0f;
        acc.x = fmaf(wj, y.x, acc.x);
        acc.y = fmaf(wj, y.y, acc.y);
        acc.z = fmaf(wj, y.z, acc.z);
        acc.w = fmaf(wj, y.w, acc.w);
        y = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
  }
  if (a.res) {
    const uint2 r = *reinterpret_cast<const uint2*>(a.res + (size_t)t * H + m);
    acc.x += bf16_lo(r.x);
    acc.y += bf16_hi(r.x);
    acc.z += bf16_lo(r.y);
    acc.w += bf16_hi(r.y);
  }
  const uint2 o = make_uint2((uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16),
                             (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16));
  *reinterpret_cast<uint2*>(a.out + (size_t)t * H + m) = o;
}

template <int FMT, int MT>
__global__ void __launch_bounds__(EX_THREADS) down_ex_kernel(MoeArgs a) {
  __shared__ __align__(16) float lds[EX_LDS];
  __shared__ int s_slot[64];
  __shared__ int s_list[EX_THREADS];
  __shared__ int s_nlist;
  const int act = blockIdx.z;
  if (act >= *a.ws.n_active) return;
  int beg, cnt, e;
  if (!expert_range(a, act, &beg, &cnt, &e) || cnt == 0) return;
  const int H = a.H, I = a.I, k = a.k, TK = a.T * k;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, q = l & 15, kg = l >> 4;
  const int mt = blockIdx.x, S = gridDim.y, s = blockIdx.y;
  const int nblk = I / 32;
  const int b0 = (s * nblk) / S, b1 = ((s + 1) * nblk) / S;
  const size_t ld = (size_t)H;
  const int m0c = 128 * mt;
  const int ncols = min(128, H - m0c);
  const bool col_ok = 8 * q < ncols;
  const int col = m0c + 8 * q;
  const uint8_t* w = a.wd + (size_t)e * (I / 2) * ld;
  const uint16_t* sc = a.sd + (size_t)e * (I / a.group) * ld;
  const OpSrc src{nullptr, a.ws.h, I, k};
  const bool use_mfma = MT > 0 && cnt >= a.mfma_min;
  const int vt = min(EX_VT, EX_LDS / (16 * (b1 - b0)));
  const int CH = use_mfma ? 16 * (MT > 0 ? MT : 1) : vt;
  const __amdgpu_buffer_rsrc_t pr = ex_rsrc(a.ws.part_dn);
  auto emit = [&](int slot, int c4, float4 y) {
    st4_sc1(pr, ((s * TK + slot) * H + m0c + c4) * 4, y);
  };

  for (int c0 = 0; c0 < cnt; c0 += CH) {
    const int nch = min(CH, cnt - c0);
    __syncthreads();
    if (tid < nch) s_slot[tid] = slot_at(a, beg + c0 + tid);
    __syncthreads();
    if constexpr (MT > 0) {
      if (use_mfma) {
        f32x4_t acc[MT][8];
        mfma_pass<FMT, MT>(w, sc, ld, a.group, col, col_ok, src, s_slot, nch, b1, b0 + wv, 4,
                           acc);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (16 * m >= nch) break;
          __syncthreads();
          // red[wave][token 0..15][column 0..127]
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              lds[(wv * 16 + 4 * kg + r) * 128 + 8 * q + i] = acc[m][i][r];
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
        }
        continue;
      }
    }
    float acc[EX_VT][8];
    valu_pass<FMT>(w, sc, ld, a.group, col, col_ok, src, s_slot, nch, b0, b1, b0 + wv, 4, lds,
                   acc);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (4 * hh >= nch) break;
      // red[wave][kg][token 0..3][column 0..127]
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          lds[(((wv * 4 + kg) * 4 + t) * 128) + 8 * q + i] = acc[4 * hh + t][i];
      __syncthreads();
      if (tid < 4 * 32) {
        const int t = tid >> 5, c4 = 4 * (tid & 31);
        const int slot = (4 * hh + t < nch) ? s_slot[4 * hh + t] : -1;
        if (slot >= 0 && c4 < ncols) {
          const float4* r4 = reinterpret_cast<const float4*>(lds);
          float4 y = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
          for (int p = 0; p < 16; ++p)  // p = wave * 4 + kg
            y = f4_add(y, r4[((p * 4 + t) * 128 + c4) / 4]);
          emit(slot, c4, y);
        }
      }
      __syncthreads();
    }
  }

  // count this workgroup's (token, tile) contributions; the workgroup completing a
  // token's tile combines its k slots
  wait_mem();
  __syncthreads();
  const int ntile = gridDim.x;
  for (int base = 0; base < cnt; base += EX_THREADS) {
    if (tid == 0) s_nlist = 0;
    __syncthreads();
    const int i = base + tid;
    if (i < cnt) {
      const int slot = slot_at(a, beg + i);
      if (slot >= 0) {
        const int t = slot / k;
        const unsigned expected = (unsigned)(a.ws.nvalid[t] * S);
        if (add_cnt(a.ws.cnt_dn + (size_t)t * ntile + mt, 1u) + 1u == expected)
          s_list[atomicAdd(&s_nlist, 1)] = t;
      }
    }
    __syncthreads();
    const int nl = s_nlist;
    for (int it = tid; it < nl * 32; it += EX_THREADS) {
      const int c4 = 4 * (it & 31);
      if (c4 < ncols) combine4<16>(a, pr, s_list[it >> 5], m0c + c4, S);
    }
    __syncthreads();
  }
}

// ---- launchers --------------------------------------------------------------------------------
template <int FMT, int MT>
static hipError_t launch_ex_t(const MoeArgs& a, int A, hipStream_t st) {
  const int ntile_gu = (a.I + 127) / 128, ntile_dn = (a.H + 127) / 128;
  hipLaunchKernelGGL((gateup_ex_kernel<FMT, MT>), dim3(ntile_gu, a.S_gu, A), dim3(EX_THREADS), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((down_ex_kernel<FMT, MT>), dim3(ntile_dn, a.S_dn, A), dim3(EX_THREADS), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_moe_experts(const MoeArgs& a, int A, int mt, hipStream_t st) {
#define DQG_EX_CASE(F, M) \
  if (a.fmt == F && mt == M) return launch_ex_t<F, M>(a, A, st);
  DQG_EX_CASE(FMT_FP4, 0)
  DQG_EX_CASE(FMT_FP4, 1)
  DQG_EX_CASE(FMT_FP4, 2)
  DQG_EX_CASE(FMT_INT4, 0)
  DQG_EX_CASE(FMT_INT4, 1)
  DQG_EX_CASE(FMT_INT4, 2)
#undef DQG_EX_CASE
  return hipErrorInvalidValue;
}

int ex_max_split() { return EX_MAX_SPLIT; }

}  // namespace dqg
