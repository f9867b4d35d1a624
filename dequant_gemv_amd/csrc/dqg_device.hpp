// Device-side building blocks for the packed 4-bit kernels (gfx950 only).
//
// A packed matrix is [K/2 byte rows][N bytes]: byte (r, n) holds K index 2r in its low
// nibble and 2r+1 in its high nibble; one bf16 scale per G consecutive K and column
// (FireEcho page, "The Goliath Kernel: Why It's Fast": packed bytes are split into low
// and high nibble and dequantized with a scale in registers inside the tile loop).
//
// Work unit of every vector-ALU tile: one lane owns 16 consecutive columns (one 16-byte
// load per byte row) and walks "blocks" of 16 byte rows (= 32 K indices).  A block never
// straddles a scale group (G is 32 or 128), so the group scale is applied once per block
// and column to the fp32 block sum instead of once per weight.
//
// Decode paths (exact: a code has at most 3 significant bits, so the products below are
// exact and only the fp32 sums round):
//   FP4 (E2M1), activations bf16  -> v_cvt_scalef32_pk_bf16_fp4 (unit scale) turns one
//       byte into the bf16 pair (W[2r], W[2r+1]); v_dot2_f32_bf16 multiplies it with the
//       bf16 pair (x[2r], x[2r+1]) and accumulates in fp32.  2 instructions / 2 weights.
//   FP4, activations fp32         -> v_cvt_scalef32_pk_f32_fp4 + two fp32 FMAs.
//   INT4, activations fp16        -> one v_perm_b32 puts the byte in both halves, one
//       and/or forms the fp16 pair (1024 + lo, 64 + hi) (the nibble lands in the mantissa
//       under a fixed exponent), v_dot2_f32_f16 accumulates; the bias
//       1032*x[2r] + 72*x[2r+1] (1024 + 8 and 64 + 8) is removed once per block.
//   INT4, activations fp32        -> nibbles to bytes, v_cvt_f32_ubyte*, FMAs; the -8 is
//       removed once per block as -8 * sum(x).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dqg {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum { FMT_INT4 = 0, FMT_FP4 = 1, FMT_FP8 = 2, FMT_INT2 = 3, FMT_FEXC = 4 };
enum { X_BF16 = 0, X_F16 = 1, X_F32 = 2 };

constexpr int BLK_ROWS = 16;  // byte rows per block (32 K indices)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- element decode -----------------------------------------------------------------
template <int B>
__device__ __forceinline__ bf16x2_t fp4_pair_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
}
template <int B>
__device__ __forceinline__ f32x2_t fp4_pair_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}
// FP8 E4M3 (OCP) bytes 2W and 2W+1 of w -> bf16 / f32 pair (exact: 4 significant bits)
template <int W>
__device__ __forceinline__ bf16x2_t fp8_pair_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, W);
}
template <int W>
__device__ __forceinline__ f32x2_t fp8_pair_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, W);
}
// K indices per stored byte
__host__ __device__ constexpr int fmt_kb(int fmt) { return fmt == FMT_FP8 ? 1 : 2; }
// byte B of w -> fp16 pair (1024 + low nibble, 64 + high nibble)
template <int B>
__device__ __forceinline__ f16x2_t int4_pair_f16_biased(uint32_t w) {
  constexpr uint32_t sel = (uint32_t)B | (0x0Cu << 8) | ((uint32_t)B << 16) | (0x0Cu << 24);
  const uint32_t p = __builtin_amdgcn_perm(w, w, sel);
  return __builtin_bit_cast(f16x2_t, (p & 0x00F0000Fu) | 0x54006400u);
}
constexpr float INT4_F16_BIAS_LO = 1032.0f;  // 1024 magic + 8 symmetric offset
constexpr float INT4_F16_BIAS_HI = 72.0f;    // 64 magic + 8 symmetric offset

__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
__device__ __forceinline__ float dot2_f16(f16x2_t a, f16x2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// ---- one block (16 byte rows x 16 columns) for NT tokens --------------------------------
// wv[r]   : the lane's 16 bytes of byte row r of the block
// xl      : LDS activations, token t row r at xl[t * xs + r] (already offset to the block)
//           X_BF16 / X_F16: uint32 pairs; X_F32: float2 pairs
// accb    : per-token per-column block sums (in/out, start at zero)
template <int FMT, int XM, int NT>
__device__ __forceinline__ void block_dot(const uint4 (&wv)[BLK_ROWS], const void* xl, int xs,
                                          float (&accb)[NT][16]) {
#pragma unroll
  for (int r = 0; r < BLK_ROWS; ++r) {
    const uint32_t d[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
    if constexpr (XM == X_BF16) {
      static_assert(FMT == FMT_FP4, "bf16 activations pair with the FP4 decode");
      bf16x2_t xp[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        xp[t] = __builtin_bit_cast(bf16x2_t, static_cast<const uint32_t*>(xl)[t * xs + r]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2_t p0 = fp4_pair_bf16<0>(d[q]);
        const bf16x2_t p1 = fp4_pair_bf16<1>(d[q]);
        const bf16x2_t p2 = fp4_pair_bf16<2>(d[q]);
        const bf16x2_t p3 = fp4_pair_bf16<3>(d[q]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          accb[t][4 * q + 0] = dot2_bf16(p0, xp[t], accb[t][4 * q + 0]);
          accb[t][4 * q + 1] = dot2_bf16(p1, xp[t], accb[t][4 * q + 1]);
          accb[t][4 * q + 2] = dot2_bf16(p2, xp[t], accb[t][4 * q + 2]);
          accb[t][4 * q + 3] = dot2_bf16(p3, xp[t], accb[t][4 * q + 3]);
        }
      }
    } else if constexpr (XM == X_F16) {
      static_assert(FMT == FMT_INT4, "fp16 activations pair with the INT4 decode");
      f16x2_t xp[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        xp[t] = __builtin_bit_cast(f16x2_t, static_cast<const uint32_t*>(xl)[t * xs + r]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x2_t p0 = int4_pair_f16_biased<0>(d[q]);
        const f16x2_t p1 = int4_pair_f16_biased<1>(d[q]);
        const f16x2_t p2 = int4_pair_f16_biased<2>(d[q]);
        const f16x2_t p3 = int4_pair_f16_biased<3>(d[q]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          accb[t][4 * q + 0] = dot2_f16(p0, xp[t], accb[t][4 * q + 0]);
          accb[t][4 * q + 1] = dot2_f16(p1, xp[t], accb[t][4 * q + 1]);
          accb[t][4 * q + 2] = dot2_f16(p2, xp[t], accb[t][4 * q + 2]);
          accb[t][4 * q + 3] = dot2_f16(p3, xp[t], accb[t][4 * q + 3]);
        }
      }
    } else {  // X_F32
      float2 xv[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) xv[t] = static_cast<const float2*>(xl)[t * xs + r];
      if constexpr (FMT == FMT_FP4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x2_t f[4];
          f[0] = fp4_pair_f32<0>(d[q]);
          f[1] = fp4_pair_f32<1>(d[q]);
          f[2] = fp4_pair_f32<2>(d[q]);
          f[3] = fp4_pair_f32<3>(d[q]);
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int b = 0; b < 4; ++b)
              accb[t][4 * q + b] =
                  fmaf(f[b].y, xv[t].y, fmaf(f[b].x, xv[t].x, accb[t][4 * q + b]));
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = d[q] & 0x0F0F0F0Fu;
          const uint32_t hi = (d[q] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float fl = (float)((lo >> (8 * b)) & 0xFFu);
            const float fh = (float)((hi >> (8 * b)) & 0xFFu);
#pragma unroll
            for (int t = 0; t < NT; ++t)
              accb[t][4 * q + b] = fmaf(fh, xv[t].y, fmaf(fl, xv[t].x, accb[t][4 * q + b]));
          }
        }
      }
    }
  }
}

// Apply the block's scales (16 bf16 at sp) and per-token correction to the block sums and
// add them into acc.
template <int FMT, int XM, int NT>
__device__ __forceinline__ void block_scale_add(const uint4& s0, const uint4& s1,
                                                const float* corr, int cs,
                                                const float (&accb)[NT][16],
                                                float (&acc)[NT][16]) {
  const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  float sf[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sf[2 * i] = bf16_lo(sw[i]);
    sf[2 * i + 1] = bf16_hi(sw[i]);
  }
  constexpr bool has_corr = (FMT == FMT_INT4);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float c = has_corr ? corr[t * cs] : 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[t][j] = fmaf(sf[j], accb[t][j] + c, acc[t][j]);
  }
}

// Walk blocks [blk_begin, blk_end) with stride blk_step for the lane's 16 columns at
// byte column col0 of a packed matrix (row stride ld bytes; scales row stride ld).
template <int FMT, int XM, int NT>
__device__ __forceinline__ void tile_rows(const uint8_t* __restrict__ w,
                                          const uint16_t* __restrict__ s, int ld, int group,
                                          int col0, int blk_begin, int blk_end, int blk_step,
                                          const void* xl, int xs, const float* corr, int cs,
                                          float (&acc)[NT][16]) {
  for (int blk = blk_begin; blk < blk_end; blk += blk_step) {
    const uint8_t* wp = w + (size_t)blk * BLK_ROWS * ld + col0;
    uint4 wv[BLK_ROWS];
#pragma unroll
    for (int r = 0; r < BLK_ROWS; ++r)
      wv[r] = *reinterpret_cast<const uint4*>(wp + (size_t)r * ld);
    const uint16_t* sp = s + (size_t)((blk * 2 * BLK_ROWS) / group) * ld + col0;
    const uint4 s0 = *reinterpret_cast<const uint4*>(sp);
    const uint4 s1 = *reinterpret_cast<const uint4*>(sp + 8);
    float accb[NT][16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) accb[t][j] = 0.0f;
    const void* xb;
    if constexpr (XM == X_F32)
      xb = static_cast<const float2*>(xl) + blk * BLK_ROWS;
    else
      xb = static_cast<const uint32_t*>(xl) + blk * BLK_ROWS;
    block_dot<FMT, XM, NT>(wv, xb, xs, accb);
    block_scale_add<FMT, XM, NT>(s0, s1, corr + blk, cs, accb, acc);
  }
}

// ---- activation staging into LDS ----------------------------------------------------------
// Row pairs of NT tokens (missing tokens are zero).  Kp = K/2 byte rows.
// X_BF16: copy bf16 pairs.  X_F16: bf16 -> fp16 pairs + per-block bias correction.
// X_F32 from fp32 source: copy float2 pairs (+ per-block -8*sum for INT4).
template <int XM, int FMT, int NT>
__device__ __forceinline__ void stage_bf16_rows(const uint16_t* const (&src)[NT], int Kp,
                                                uint32_t* xl, float* corr, int nthreads,
                                                int tid) {
  for (int i = tid; i < NT * Kp; i += nthreads) {
    const int t = i / Kp, r = i - t * Kp;
    uint32_t v = 0;
    if (src[t]) v = reinterpret_cast<const uint32_t*>(src[t])[r];
    if constexpr (XM == X_F16) {
      const f16x2_t h = {(_Float16)bf16_lo(v), (_Float16)bf16_hi(v)};
      v = __builtin_bit_cast(uint32_t, h);
    }
    xl[t * Kp + r] = v;
  }
  if constexpr (XM == X_F16) {
    __syncthreads();
    const int nb = Kp / BLK_ROWS;
    for (int i = tid; i < NT * nb; i += nthreads) {
      const int t = i / nb, b = i - t * nb;
      float c = 0.0f;
      for (int r = 0; r < BLK_ROWS; ++r) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, xl[t * Kp + b * BLK_ROWS + r]);
        c = fmaf(-INT4_F16_BIAS_LO, (float)h.x, c);
        c = fmaf(-INT4_F16_BIAS_HI, (float)h.y, c);
      }
      corr[t * nb + b] = c;
    }
  }
}

template <int FMT, int NT>
__device__ __forceinline__ void stage_f32_rows(const float* const (&src)[NT], int Kp, float2* xl,
                                               float* corr, int nthreads, int tid) {
  for (int i = tid; i < NT * Kp; i += nthreads) {
    const int t = i / Kp, r = i - t * Kp;
    float2 v = make_float2(0.0f, 0.0f);
    if (src[t]) v = reinterpret_cast<const float2*>(src[t])[r];
    xl[t * Kp + r] = v;
  }
  if constexpr (FMT == FMT_INT4) {
    __syncthreads();
    const int nb = Kp / BLK_ROWS;
    for (int i = tid; i < NT * nb; i += nthreads) {
      const int t = i / nb, b = i - t * nb;
      float c = 0.0f;
      for (int r = 0; r < BLK_ROWS; ++r) {
        const float2 v = xl[t * Kp + b * BLK_ROWS + r];
        c += v.x + v.y;
      }
      corr[t * nb + b] = -8.0f * c;
    }
  }
}

// ---- top-k routing: one wavefront per token ---------------------------------------------
// Order-preserving integer key of a logit: larger float -> larger int; -0.0 and +0.0 get the
// same key (so they tie and the lower expert index ranks first).  The map is an involution
// on the bits, so key_to_float undoes it (returning +0.0 for either zero).
__device__ __forceinline__ int logit_key(float v) {
  const int b = __float_as_int(v + 0.0f);  // -0.0 + 0.0 = +0.0
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_to_float(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}
// Maximum over the wavefront, uniform result: DPP within each row of 16 lanes (xor 1, xor 2,
// rotate 4, rotate 8), then the four row maxima through readlane.
__device__ __forceinline__ int wave_max_key(int v) {
  v = max(v, __builtin_amdgcn_update_dpp((int)0x80000000, v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp((int)0x80000000, v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp((int)0x80000000, v, 0x124, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp((int)0x80000000, v, 0x128, 0xF, 0xF, false));
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a + b) + (c + d);
}

// Top-k of one row of E logits (E <= 64 * MAXV) by one wavefront; lane j < k returns the
// j-th selection (rank order) in *sel_e / *sel_w, with w = softmax over the k selected
// logits (top logit subtracted).  Each round takes the wave maximum of the not-yet-taken
// keys, then the lowest expert index holding that key (ballot over expert = lane + 64 i,
// i ascending), so ties go to the lower index.  Logits must not be NaN.
template <int MAXV>
__device__ __forceinline__ void wave_route(const float* __restrict__ row, int E, int k, int lane,
                                           int* sel_e, float* sel_w) {
  // all loads issued together (clamped index, result replaced afterwards)
  float lv[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) lv[i] = row[min(lane + 64 * i, E - 1)];
  int key[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    key[i] = (lane + 64 * i < E) ? logit_key(lv[i]) : (int)0x80000000;
  unsigned long long taken = 0;
  int my_key = 0, my_e = -1, top = 0;
  for (int j = 0; j < k; ++j) {
    int m = (int)0x80000000;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (!((taken >> i) & 1ull) && lane + 64 * i < E) m = max(m, key[i]);
    m = wave_max_key(m);
    int win = -1;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const unsigned long long bal =
          __ballot(!((taken >> i) & 1ull) && lane + 64 * i < E && key[i] == m);
      if (bal) {
        const int l = __ffsll((long long)bal) - 1;
        win = l + 64 * i;
        if (lane == l) taken |= 1ull << i;
        break;
      }
    }
    if (j == 0) top = m;
    if (lane == j) {
      my_key = m;
      my_e = win;
    }
  }
  const float ex = (lane < k) ? expf(key_to_float(my_key) - key_to_float(top)) : 0.0f;
  const float s = wave_sum_f32(ex);
  *sel_e = my_e;
  *sel_w = ex / s;
}

// Same selection for E > 512: keys are re-read from memory (L1/L2) every round instead of
// being held in registers; `taken` covers up to 64 entries per lane (E <= 4096).
__device__ __forceinline__ void wave_route_mem(const float* __restrict__ row, int E, int k,
                                               int lane, int* sel_e, float* sel_w) {
  unsigned long long taken = 0;
  int my_key = 0, my_e = -1, top = 0;
  const int nv = (E + 63) / 64;
  for (int j = 0; j < k; ++j) {
    int m = (int)0x80000000;
    for (int i = 0; i < nv; ++i)
      if (!((taken >> i) & 1ull) && lane + 64 * i < E) m = max(m, logit_key(row[lane + 64 * i]));
    m = wave_max_key(m);
    int win = -1;
    for (int i = 0; i < nv; ++i) {
      const bool mine = !((taken >> i) & 1ull) && lane + 64 * i < E &&
                        logit_key(row[lane + 64 * i]) == m;
      const unsigned long long bal = __ballot(mine);
      if (bal) {
        const int l = __ffsll((long long)bal) - 1;
        win = l + 64 * i;
        if (lane == l) taken |= 1ull << i;
        break;
      }
    }
    if (j == 0) top = m;
    if (lane == j) {
      my_key = m;
      my_e = win;
    }
  }
  const float ex = (lane < k) ? expf(key_to_float(my_key) - key_to_float(top)) : 0.0f;
  const float s = wave_sum_f32(ex);
  *sel_e = my_e;
  *sel_w = ex / s;
}

// MAXE: the largest E the caller supports (E <= 512 keeps the keys in registers).
template <int MAXE = 4096>
__device__ __forceinline__ void route_row(const float* __restrict__ row, int E, int k, int lane,
                                          int* sel_e, float* sel_w) {
  if (E <= 128)
    wave_route<2>(row, E, k, lane, sel_e, sel_w);
  else if (MAXE <= 512 || E <= 512)
    wave_route<8>(row, E, k, lane, sel_e, sel_w);
  else
    wave_route_mem(row, E, k, lane, sel_e, sel_w);
}

__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int lane, int32_t* ids, float* wts) {
  int e;
  float w;
  route_row<4096>(logits + (size_t)t * E, E, k, lane, &e, &w);
  if (lane < k) {
    ids[(size_t)t * k + lane] = e;
    wts[(size_t)t * k + lane] = w;
  }
}

// ---- top-k routing with a short dependency chain: one wavefront per row ------------------
// The same selection and weights as wave_route for E <= 64 * MAXV, without k serial
// wave-wide rounds (each of which passes values between vector and scalar units):
//  1. lane l holds the keys of elements l, l + 64, ...; groups of L = 64 / G adjacent lanes
//     take their maximum, G = max(4, the smallest power of two >= k) <= 32 groups;
//  2. theta = the k-th largest group maximum (the smallest one when G == k).  k distinct
//     elements have keys >= theta, so all of the top k have keys >= theta (if fewer than k
//     groups hold elements, theta is the smallest key and every element qualifies);
//  3. the C >= k elements with keys >= theta are compacted into LDS (ballot prefix counts) as
//     64-bit composites key << 32 | ~index, which are distinct and order the elements like
//     the keys with ties to the lower index;
//  4. candidate p's rank is the number of candidates with a larger composite; every element
//     that beats a top-k element is a candidate, so ranks 0..k-1 are exactly the selection.
// wave_topk_select writes the selection to LDS, ids[r] and keys[r] for rank r < k (visible
// to the calling wavefront on return); wave_topk_weights turns it into lane j < k's id and
// weight (softmax over the k selected logits, top logit subtracted); wave_topk does both,
// through its scratch.  `cand` is the calling wavefront's own LDS scratch of 64 * MAXV + 68
// eight-byte entries, 16-byte aligned.  Needs 1 <= k <= 32.
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, __builtin_amdgcn_update_dpp((int)0x7FFFFFFF, v, 0xB1, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp((int)0x7FFFFFFF, v, 0x4E, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp((int)0x7FFFFFFF, v, 0x124, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp((int)0x7FFFFFFF, v, 0x128, 0xF, 0xF, false));
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// wave_topk_select_keys takes the keys already in registers: key[v] of element lane + 64 v
// (any value for elements >= E).
template <int MAXV>
__device__ __forceinline__ void wave_topk_select_keys(const int (&key)[MAXV], int E, int k,
                                                      int lane, long long* cand, int* ids,
                                                      int* keys) {
  int m = (int)0x80000000;
#pragma unroll
  for (int v = 0; v < MAXV; ++v)
    if (lane + 64 * v < E) m = max(m, key[v]);
  // group maxima over L lanes (L = 16, 8, 4 or 2 for G = 4, 8, 16, 32)
  const int G = k <= 4 ? 4 : (k <= 8 ? 8 : (k <= 16 ? 16 : 32));
  m = max(m, __builtin_amdgcn_update_dpp((int)0x80000000, m, 0xB1, 0xF, 0xF, false));
  if (G <= 16) m = max(m, __builtin_amdgcn_update_dpp((int)0x80000000, m, 0x4E, 0xF, 0xF, false));
  if (G <= 8) m = max(m, __builtin_amdgcn_update_dpp((int)0x80000000, m, 0x141, 0xF, 0xF, false));
  if (G <= 4) m = max(m, __builtin_amdgcn_update_dpp((int)0x80000000, m, 0x140, 0xF, 0xF, false));
  int* sel = reinterpret_cast<int*>(cand + 64 * MAXV + 4);  // scratch for the group ranks
  int theta;
  if (G == k) {
    theta = wave_min_i32(m);
  } else {
    // rank the G group maxima (lane g < G takes group g's) and keep the k-th largest
    const int L = 64 / G;
    if (lane % L == 0) sel[lane / L] = m;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const int mine = (lane < G) ? sel[lane] : (int)0x7FFFFFFF;
    int gt0 = 0, gt1 = 0;
    for (int h = 0; h < G; h += 4) {
      const int4 q = *reinterpret_cast<const int4*>(sel + h);
      gt0 += (q.x > mine) + (q.y > mine);
      gt1 += (q.z > mine) + (q.w > mine);
    }
    theta = wave_min_i32((lane < G && gt0 + gt1 < k) ? mine : (int)0x7FFFFFFF);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  // compaction of the candidates, in element order
  int C = 0;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int e = lane + 64 * v;
    const bool c = e < E && key[v] >= theta;
    const unsigned long long b = __ballot(c);
    if (c) {
      const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(b >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((unsigned)b, 0u));
      cand[pos] = (long long)(((unsigned long long)(unsigned)key[v] << 32) |
                              (unsigned long long)(0xFFFFFFFFu - (unsigned)e));
    }
    C += __popcll(b);
  }
  // composites that no candidate is below fill the list to 32 entries and 4 past its end, so
  // that the rank loops read whole groups
  const long long below = (long long)0x8000000000000000ll;
  if (lane < 4) cand[C + lane] = below;
  if (lane >= C && lane < 32) cand[lane] = below;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (C <= 32) {
    // the usual case: every lane reads the 32 entries at once and compares them unrolled
    const long long me = cand[lane < 32 ? lane : 31];
    long long cv[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const longlong2 u = reinterpret_cast<const longlong2*>(cand)[i];
      cv[2 * i] = u.x;
      cv[2 * i + 1] = u.y;
    }
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
#pragma unroll
    for (int h = 0; h < 32; h += 4) {
      r0 += (cv[h] > me);
      r1 += (cv[h + 1] > me);
      r2 += (cv[h + 2] > me);
      r3 += (cv[h + 3] > me);
    }
    const int r = (r0 + r1) + (r2 + r3);
    if (lane < C && r < k) {
      ids[r] = (int)(0xFFFFFFFFu - (unsigned)(unsigned long long)me);
      keys[r] = (int)(me >> 32);
    }
  } else {
    for (int p0 = 0; p0 < C; p0 += 64) {
      const int p = p0 + lane;
      if (p < C) {
        const long long me = cand[p];
        int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
        for (int h = 0; h < C; h += 4) {
          const longlong2 u = *reinterpret_cast<const longlong2*>(cand + h);
          const longlong2 w = *reinterpret_cast<const longlong2*>(cand + h + 2);
          r0 += (u.x > me);
          r1 += (u.y > me);
          r2 += (w.x > me);
          r3 += (w.y > me);
        }
        const int r = (r0 + r1) + (r2 + r3);
        if (r < k) {
          ids[r] = (int)(0xFFFFFFFFu - (unsigned)(unsigned long long)me);
          keys[r] = (int)(me >> 32);
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

template <int MAXV>
__device__ __forceinline__ void wave_topk_select(const float* __restrict__ row, int E, int k,
                                                 int lane, long long* cand, int* ids,
                                                 int* keys) {
  int key[MAXV];
#pragma unroll
  for (int v = 0; v < MAXV; ++v) key[v] = logit_key(row[min(lane + 64 * v, E - 1)]);
  wave_topk_select_keys<MAXV>(key, E, k, lane, cand, ids, keys);
}

__device__ __forceinline__ void wave_topk_weights(const int* ids, const int* keys, int k,
                                                  int lane, int* sel_e, float* sel_w) {
  const int my_e = (lane < k) ? ids[lane] : -1;
  const int my_key = (lane < k) ? keys[lane] : 0;
  const float ex = (lane < k) ? expf(key_to_float(my_key) - key_to_float(keys[0])) : 0.0f;
  const float s = wave_sum_f32(ex);
  *sel_e = my_e;
  *sel_w = ex / s;
}

template <int MAXV>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int lane,
                                          long long* cand, int* sel_e, float* sel_w) {
  int* sel = reinterpret_cast<int*>(cand + 64 * MAXV + 4);  // ids [0, 32), keys [64, 96)
  wave_topk_select<MAXV>(row, E, k, lane, cand, sel, sel + 64);
  wave_topk_weights(sel, sel + 64, k, lane, sel_e, sel_w);
}

// ---- workgroup column sums ----------------------------------------------------------------
// Lane tid owns columns chunk*16 .. chunk*16+15 of row-lane tid / CPR (chunk = tid % CPR).
// Sum the 16 partials over all row-lanes: one LDS transpose (4 x b128 writes per lane, a
// barrier, then thread c < CPR*16 reads its column from every row-lane with all reads in
// flight).  Summation order is fixed (row-lane ascending).  `red` holds THREADS*16 floats;
// the caller must not overwrite it before a following barrier.
template <int CPR, int THREADS>
__device__ __forceinline__ float wg_colsum(const float (&acc)[16], float* red, int tid) {
  constexpr int RL = THREADS / CPR, COLS = CPR * 16;
  const int rl = tid / CPR, ch = tid % CPR;
  float4* dst = reinterpret_cast<float4*>(red + rl * COLS + ch * 16);
  dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  dst[2] = make_float4(acc[8], acc[9], acc[10], acc[11]);
  dst[3] = make_float4(acc[12], acc[13], acc[14], acc[15]);
  __syncthreads();
  float s = 0.0f;
  if (tid < COLS) {
    float v[RL];
#pragma unroll
    for (int r = 0; r < RL; ++r) v[r] = red[r * COLS + tid];
#pragma unroll
    for (int r = 0; r < RL; ++r) s += v[r];
  }
  return s;
}

// ---- router logits: one unit of the router GEMV --------------------------------------------
// logits[t, e] = sum_c x[t, c] W_r[c, e] (W_r bf16 [H, E], fp32 accumulation) is split into
// units of RT_ROWS rows of W_r and 128 columns.  A unit runs on 256 threads, 16 row-lanes x
// 16 column-lanes; a lane owns 8 consecutive rows and 8 consecutive columns (one 16-byte load
// per row).  Fixed order: fma over the lane's rows ascending, then the 16 row-lanes summed
// ascending through LDS.  The full logit is the sum of the units' partials over the row
// splits in ascending order, starting from +0.0 -- the same on every path that uses it, so
// the logits (and with them the routing) are bitwise identical between the single-launch
// layer and the separate router call.
constexpr int RT_ROWS = 128;
constexpr int RT_MAX_T = 4;  // tokens per unit
// Partial of rows [RT_ROWS rs, +RT_ROWS) and columns [128 ct, +128) for tokens t0 .. t0+nt-1
// (nt <= RT_MAX_T): on return thread c < 128 holds column 128 ct + c of token t0 + t in
// part[t] (0 for columns >= E).  red: 16 * 128 floats of LDS.  Needs H % 8 == 0, E % 8 == 0,
// 16-byte aligned x and W_r.  Every thread of the workgroup must call it.
__device__ __forceinline__ void router_unit(const uint16_t* __restrict__ x, int H,
                                            const uint16_t* __restrict__ wr, int E, int rs,
                                            int ct, int t0, int nt, float* red, int tid,
                                            float (&part)[RT_MAX_T]) {
  const int rl = tid >> 4, ch = tid & 15;
  const int r0 = RT_ROWS * rs + 8 * rl, c0 = 128 * ct + 8 * ch;
  const bool on = r0 < H && c0 < E;
  uint4 w[8];
  uint4 xv[RT_MAX_T];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = on ? *reinterpret_cast<const uint4*>(wr + (size_t)(r0 + i) * E + c0)
              : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < RT_MAX_T; ++t)
    xv[t] = (on && t < nt) ? *reinterpret_cast<const uint4*>(x + (size_t)(t0 + t) * H + r0)
                           : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < RT_MAX_T; ++t) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    const uint32_t xw[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xi = (i & 1) ? bf16_hi(xw[i >> 1]) : bf16_lo(xw[i >> 1]);
      const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = fmaf(xi, (j & 1) ? bf16_hi(ww[j >> 1]) : bf16_lo(ww[j >> 1]), acc[j]);
    }
    if (t < nt) {  // uniform
      float4* dst = reinterpret_cast<float4*>(red + rl * 128 + ch * 8);
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      __syncthreads();
      float s = 0.0f;
      if (tid < 128) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = red[r * 128 + tid];
#pragma unroll
        for (int r = 0; r < 16; ++r) s += v[r];
      }
      part[t] = s;
      __syncthreads();
    } else {
      part[t] = 0.0f;
    }
  }
}

// ---- cross-workgroup exchange ----------------------------------------------------------
// Data that another workgroup reads within the same launch moves with agent-coherent
// (sc1) loads and stores: relaxed agent-scope atomic accesses, which need no cache
// writeback or invalidate.  (An agent-scope fence writes back and invalidates the L2 and
// costs tens of microseconds when hundreds of workgroups issue it.)  Ordering: each thread
// waits until its own stores are acknowledged, the workgroup meets at a barrier, then one
// thread increments the counter.
__device__ __forceinline__ void st_sc1(float* base, size_t idx, float v) {
  __hip_atomic_store(base + idx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_sc1(const float* base, size_t idx) {
  return __hip_atomic_load(base + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_cnt(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_cnt(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_cnt(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait for this thread's outstanding memory operations (stores acknowledged)
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Every thread has stored its partial results with st_sc1; returns true (in all threads)
// for exactly one workgroup -- the one whose increment completes `expected`.  That
// workgroup reads the others' partials with ld_sc1 and resets the counter.
__device__ __forceinline__ bool last_arriver(unsigned* counter, unsigned expected, int* s_flag) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = add_cnt(counter, 1u);
    *s_flag = (prev + 1u == expected) ? 1 : 0;
  }
  __syncthreads();
  return *s_flag != 0;
}

}  // namespace dqg
