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

enum { FMT_INT4 = 0, FMT_FP4 = 1 };
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

// ---- cross-workgroup "last arriver" -----------------------------------------------------
// Every thread has stored its partial results; returns true (in all threads) for exactly
// one workgroup -- the one whose increment completes `expected`.  That workgroup then
// reads the others' partials (after the acquire fence) and resets the counter.
__device__ __forceinline__ bool last_arriver(unsigned* counter, unsigned expected, int* s_flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(counter, 1u);
    *s_flag = (prev + 1u == expected) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *s_flag != 0;
  if (last) __threadfence();
  return last;
}

}  // namespace dqg
