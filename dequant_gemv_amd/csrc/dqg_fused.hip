// Single-launch packed-MoE layer for up to FX_MAX_T = 8 tokens: routing, fused gate_up,
// SiLU*up, down projection and the top-k combine in one kernel.
//
// FireEcho page, "The Goliath Kernel: Why It's Fast": one launch reads the expert ids from
// device memory and indexes the contiguous packed buffer, with the dequant in registers
// inside the tile loop.  Measured on MI355X: a launch costs about 1.6 us even inside a
// graph, every dependent memory round trip about 1 us, and a workgroup that reads a matrix
// in 128-byte row segments streams about 2.5x faster than one reading 32-byte segments.
// A whole T=1 layer moves only ~21 MB, so it is one launch whose workgroups read full
// 128-byte lines and exchange data with as few round trips as possible.
//
// Slots s = t k + j (token t, rank j).  Every workgroup first routes its token itself (one
// wavefront, threshold + compaction + rank selection; no other workgroup is waited for) --
// from the logits, or from the partial logits of the router units, which then come first in
// the grid (the router GEMV x W_r, 128 rows of W_r each).  A byte row holds KB = 2 K indices
// (4-bit formats) or 1 (FP8).
// Workgroups (256 threads, 4 waves), every lane owning 16 columns x a few byte rows:
//   gate_up units (s, nt, ks): slot s, h columns [128 nt, 128 nt + 128) -- 128 bytes of
//     gate and 128 bytes of up per byte row (16 lanes) -- over 16 GUR byte rows from
//     16 GUR ks on (16 row-lanes x GUR rows; GUR = 8 for one token with 4-bit weights, 16
//     otherwise).  Each publishes its partial gate/up row and exits; gate_up units never
//     wait.  (A slot is one unit set: an expert chosen by two tokens is read twice, mostly
//     from cache the second time.)
//   down units (mt, c): output columns [128 mt, 128 mt + 128) (8 lanes) over byte rows
//     [256 c, 256 c + 256) of the concatenated per-slot down matrices (32 row-lanes x 8
//     rows); for T > 1 a token's rows fill whole chunks.  On layers with >= 16 MiB of gate_up
//     weights per token, their weight loads wait for the first gate/up partial of their
//     range (the gate_up loads, which are on the critical path, get the bandwidth first);
//     then the threads gather the KS partial gate/up pairs of the unit's 256 KB h values
//     (ascending ks), form h = SiLU(g)*u into LDS, and every lane scales its sum by its slot
//     weight.  A token's chunks publish partial output rows, except its last chunk of each
//     column tile, which gathers them in ascending c, adds its own and the residual, and
//     writes the token's bf16 output.
// Publication protocol: exchange buffers hold the bit pattern 0 when empty and producers
// never store 0 (+0.0 is stored as -0.0, which computes identically); consumers poll the
// data itself with agent-coherent (sc1) loads, all of a gather's loads in flight at once.
// Each buffer exists twice: a call uses copy p = bit 20 of a 32-bit call counter, to which
// the T x n_mt finishing down units add shares summing to exactly 2^20 (so bit 20 flips once
// per call, also across wrap-around, and no unit of a call can see it flipped before every
// unit has read it, since each finishing unit waits on all others of its token, and those
// on every gate_up unit of the token); producers clear their slots of copy 1-p, which the
// previous call used and the next call will use.  Each token count T has its own counter
// and buffers in the workspace, so that calls with different T never leave data in each
// other's slots (likewise each format class: the 4-bit formats and FP8).  The router's
// partial rows follow the same scheme with a counter of their
// own that only calls with router units advance, so that calls without them (which leave
// those rows alone) cannot put a later router call on a copy that still holds old rows.
// A unit only waits on units with lower block ids, so in-order dispatch
// cannot deadlock; waits are bounded and set bit 1 of the error word on timeout instead of
// hanging.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqg_device.hpp"
#include "dqg_internal.hpp"

namespace dqg {

constexpr int FX_THREADS = 256;
constexpr unsigned FX_SPIN_LIMIT = 1u << 20;
constexpr int CPOL_SC1 = 16;       // cache-policy operand: agent-coherent access

// published value: never the empty pattern 0 (+0.0 becomes -0.0)
__device__ __forceinline__ float pub(float v) {
  return __float_as_uint(v) == 0u ? __uint_as_float(0x80000000u) : v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7FFFFFFF, 0x00020000);
}

// A gate_up unit covers 16 row-lanes x GUR byte rows; GUR = 8 for one token and 16 for
// several, where there are T times more slots and fewer, larger units keep all of them
// resident (measured at the 128-expert shape: T = 4 is 12 % faster with 16, T = 1 the same).
// A down unit covers 32 row-lanes x DR byte rows: DR = 8 (256-row chunks) in general, DR = 4
// (128-row chunks) for one token where that spreads the layer's bytes more evenly over the
// compute units (fx_down_rows).
constexpr int FX_DR_MAX = 8;
constexpr int fx_krows(int gur) { return 16 * gur; }
constexpr int fx_max_ks(int gur) { return 2048 / 2 / fx_krows(gur); }  // H <= 2048
static inline int fx_gu_rows(int H, int T) { return (T > 1 && (H / 2) % fx_krows(16) == 0) ? 16 : 8; }

template <int FMT, int ROWS>
__device__ __forceinline__ void rows_dot_x(const uint4 (&wv)[ROWS], const uint32_t (&xr)[ROWS],
                                           float (&acc)[16]) {
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const uint32_t d[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
    if constexpr (FMT == FMT_FP4) {
      const bf16x2_t xp = __builtin_bit_cast(bf16x2_t, xr[r]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[4 * q + 0] = dot2_bf16(fp4_pair_bf16<0>(d[q]), xp, acc[4 * q + 0]);
        acc[4 * q + 1] = dot2_bf16(fp4_pair_bf16<1>(d[q]), xp, acc[4 * q + 1]);
        acc[4 * q + 2] = dot2_bf16(fp4_pair_bf16<2>(d[q]), xp, acc[4 * q + 2]);
        acc[4 * q + 3] = dot2_bf16(fp4_pair_bf16<3>(d[q]), xp, acc[4 * q + 3]);
      }
    } else {
      const f16x2_t xp = __builtin_bit_cast(f16x2_t, xr[r]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[4 * q + 0] = dot2_f16(int4_pair_f16_biased<0>(d[q]), xp, acc[4 * q + 0]);
        acc[4 * q + 1] = dot2_f16(int4_pair_f16_biased<1>(d[q]), xp, acc[4 * q + 1]);
        acc[4 * q + 2] = dot2_f16(int4_pair_f16_biased<2>(d[q]), xp, acc[4 * q + 2]);
        acc[4 * q + 3] = dot2_f16(int4_pair_f16_biased<3>(d[q]), xp, acc[4 * q + 3]);
      }
    }
  }
}

// INT2 (cold experts of a mixed FP4 layer): byte row q holds K indices 4q .. 4q+3 of one
// column in bits 0-1, 2-3, 4-5, 6-7; code c means c - 2.  d & 0x33333333 leaves in every
// byte the codes of K 4q and 4q+2 in the low bits of its two nibbles, (d >> 2) & 0x33333333
// those of 4q+1 and 4q+3; the FP4 (E2M1) conversion reads a nibble 0..3 as c / 2 exactly
// (0, 0.5, 1, 1.5), so one and + one conversion give the pair (c_a / 2, c_b / 2).  The sum
// is doubled and 2 sum(x) removed once per lane (returned as corr, both exact in fp32).
template <int ROWS>
__device__ __forceinline__ float rows_dot_x_int2(const uint4 (&wv)[ROWS / 2],
                                                 const uint32_t (&xr)[ROWS], float (&acc)[16]) {
#pragma unroll
  for (int i = 0; i < ROWS / 2; ++i) {
    const uint32_t d[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
    // x pairs (x[4i], x[4i+2]) and (x[4i+1], x[4i+3]) of the lane's K range
    const bf16x2_t x02 = __builtin_bit_cast(bf16x2_t,
                                            __builtin_amdgcn_perm(xr[2 * i + 1], xr[2 * i], 0x05040100u));
    const bf16x2_t x13 = __builtin_bit_cast(bf16x2_t,
                                            __builtin_amdgcn_perm(xr[2 * i + 1], xr[2 * i], 0x07060302u));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t m0 = d[q] & 0x33333333u, m1 = (d[q] >> 2) & 0x33333333u;
      acc[4 * q + 0] = dot2_bf16(fp4_pair_bf16<0>(m0), x02, acc[4 * q + 0]);
      acc[4 * q + 1] = dot2_bf16(fp4_pair_bf16<1>(m0), x02, acc[4 * q + 1]);
      acc[4 * q + 2] = dot2_bf16(fp4_pair_bf16<2>(m0), x02, acc[4 * q + 2]);
      acc[4 * q + 3] = dot2_bf16(fp4_pair_bf16<3>(m0), x02, acc[4 * q + 3]);
      acc[4 * q + 0] = dot2_bf16(fp4_pair_bf16<0>(m1), x13, acc[4 * q + 0]);
      acc[4 * q + 1] = dot2_bf16(fp4_pair_bf16<1>(m1), x13, acc[4 * q + 1]);
      acc[4 * q + 2] = dot2_bf16(fp4_pair_bf16<2>(m1), x13, acc[4 * q + 2]);
      acc[4 * q + 3] = dot2_bf16(fp4_pair_bf16<3>(m1), x13, acc[4 * q + 3]);
    }
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] *= 2.0f;
  float sx = 0.0f;
  const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
#pragma unroll
  for (int p = 0; p < ROWS; ++p) sx = dot2_bf16(one, __builtin_bit_cast(bf16x2_t, xr[p]), sx);
  return -2.0f * sx;
}

// down: ROWS / 2 INT2 byte rows times the lane's 2 ROWS h values (K 4i + m <-> hf[4i + m]);
// same decode in f32; returns -2 sum(h) for the code offset
template <int ROWS>
__device__ __forceinline__ float rows_dot_f32_int2(const uint4 (&wv)[ROWS / 2],
                                                   const float (&hf)[2 * ROWS], float (&acc)[16]) {
#pragma unroll
  for (int i = 0; i < ROWS / 2; ++i) {
    const uint32_t d[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
    const float h0 = hf[4 * i], h1 = hf[4 * i + 1], h2 = hf[4 * i + 2], h3 = hf[4 * i + 3];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t m0 = d[q] & 0x33333333u, m1 = (d[q] >> 2) & 0x33333333u;
      f32x2_t a[4], b[4];
      a[0] = fp4_pair_f32<0>(m0); a[1] = fp4_pair_f32<1>(m0);
      a[2] = fp4_pair_f32<2>(m0); a[3] = fp4_pair_f32<3>(m0);
      b[0] = fp4_pair_f32<0>(m1); b[1] = fp4_pair_f32<1>(m1);
      b[2] = fp4_pair_f32<2>(m1); b[3] = fp4_pair_f32<3>(m1);
#pragma unroll
      for (int J = 0; J < 4; ++J)
        acc[4 * q + J] = fmaf(b[J].y, h3, fmaf(a[J].y, h2, fmaf(b[J].x, h1,
                              fmaf(a[J].x, h0, acc[4 * q + J]))));
    }
  }
  float sh = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] *= 2.0f;
#pragma unroll
  for (int i = 0; i < 2 * ROWS; ++i) sh += hf[i];
  return -2.0f * sh;
}

// FE-XC (codebook experts of a mixed FP4 layer): code row 2g + m holds codebook m's 8-bit
// code of group g (8 consecutive K indices) for 16 columns; the group's weights are
// C[0][c0] + C[1][c1], 8 bf16 each (one uint4 of the LDS copy `cb`, [2][256] vectors).
// gate_up: ROWS 4-bit-row equivalents = ROWS / 4 groups; x pairs xr[4g + p] hold K 8g + 2p
// and 8g + 2p + 1 of the lane's range, which meet the vectors' pairs in v_dot2_f32_bf16.
__device__ __forceinline__ uint32_t byte_of(const uint4& w, int j) {
  const uint32_t d = (j < 4) ? w.x : (j < 8) ? w.y : (j < 12) ? w.z : w.w;
  return (d >> (8 * (j & 3))) & 0xFFu;
}
// 16 bytes per lane from global memory straight into LDS, through no registers: the wave's
// lanes land in consecutive 16-byte slots from dst_wave, which must be the same in every lane
__device__ __forceinline__ void copy_to_lds16(const uint4* src, uint4* dst_wave) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                   (__attribute__((address_space(3))) void*)dst_wave, 16, 0, 0);
}

template <int ROWS>
__device__ __forceinline__ void rows_dot_x_fexc(const uint4 (&wv)[ROWS / 2],
                                                const uint32_t (&xr)[ROWS], const uint4* cb,
                                                float (&acc)[16]) {
#pragma unroll
  for (int g = 0; g < ROWS / 4; ++g) {
    bf16x2_t xp[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) xp[p] = __builtin_bit_cast(bf16x2_t, xr[4 * g + p]);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 v0 = cb[byte_of(wv[2 * g], j)], v1 = cb[256 + byte_of(wv[2 * g + 1], j)];
      float s = acc[j];
      s = dot2_bf16(__builtin_bit_cast(bf16x2_t, v0.x), xp[0], s);
      s = dot2_bf16(__builtin_bit_cast(bf16x2_t, v0.y), xp[1], s);
      s = dot2_bf16(__builtin_bit_cast(bf16x2_t, v0.z), xp[2], s);
      s = dot2_bf16(__builtin_bit_cast(bf16x2_t, v0.w), xp[3], s);
      s = dot2_bf16(__builtin_bit_cast(bf16x2_t, v1.x), xp[0], s);
      s = dot2_bf16(__builtin_bit_cast(bf16x2_t, v1.y), xp[1], s);
      s = dot2_bf16(__builtin_bit_cast(bf16x2_t, v1.z), xp[2], s);
      s = dot2_bf16(__builtin_bit_cast(bf16x2_t, v1.w), xp[3], s);
      acc[j] = s;
    }
  }
}

// down: the lane's 2 ROWS fp32 h values split into bf16 hi + lo pairs (hi = the top 16 bits,
// lo = the exact remainder rounded to bf16: about 16 significant bits of h in all)
template <int ROWS>
__device__ __forceinline__ void rows_dot_f32_fexc(const uint4 (&wv)[ROWS / 2],
                                                  const float (&hf)[2 * ROWS], const uint4* cb,
                                                  float (&acc)[16]) {
#pragma unroll
  for (int g = 0; g < ROWS / 4; ++g) {
    bf16x2_t hh[4], hl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = hf[8 * g + 2 * p], b = hf[8 * g + 2 * p + 1];
      const uint32_t ah = __float_as_uint(a) & 0xFFFF0000u, bh = __float_as_uint(b) & 0xFFFF0000u;
      hh[p] = __builtin_bit_cast(bf16x2_t, (ah >> 16) | bh);
      const uint32_t al = f32_to_bf16(a - __uint_as_float(ah));
      const uint32_t bl = f32_to_bf16(b - __uint_as_float(bh));
      hl[p] = __builtin_bit_cast(bf16x2_t, al | (bl << 16));
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 v0 = cb[byte_of(wv[2 * g], j)], v1 = cb[256 + byte_of(wv[2 * g + 1], j)];
      const uint32_t vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float s = acc[j];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        s = dot2_bf16(__builtin_bit_cast(bf16x2_t, vv[q]), hh[q & 3], s);
        s = dot2_bf16(__builtin_bit_cast(bf16x2_t, vv[q]), hl[q & 3], s);
      }
      acc[j] = s;
    }
  }
}

// FP8 gate_up rows: rows 2i and 2i+1 meet the x pair xr[i]; their bytes are interleaved per
// column (v_perm_b32) so that one conversion gives the bf16 pair (w[2i][c], w[2i+1][c]).
template <int ROWS>
__device__ __forceinline__ void rows_dot_x_fp8(const uint4 (&wv)[ROWS], const uint32_t (&xr)[ROWS],
                                               float (&acc)[16]) {
#pragma unroll
  for (int i = 0; i < ROWS / 2; ++i) {
    const uint32_t a[4] = {wv[2 * i].x, wv[2 * i].y, wv[2 * i].z, wv[2 * i].w};
    const uint32_t b[4] = {wv[2 * i + 1].x, wv[2 * i + 1].y, wv[2 * i + 1].z, wv[2 * i + 1].w};
    const bf16x2_t xp = __builtin_bit_cast(bf16x2_t, xr[i]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = __builtin_amdgcn_perm(b[q], a[q], 0x05010400u);  // a0 b0 a1 b1
      const uint32_t hi = __builtin_amdgcn_perm(b[q], a[q], 0x07030602u);  // a2 b2 a3 b3
      acc[4 * q + 0] = dot2_bf16(fp8_pair_bf16<0>(lo), xp, acc[4 * q + 0]);
      acc[4 * q + 1] = dot2_bf16(fp8_pair_bf16<1>(lo), xp, acc[4 * q + 1]);
      acc[4 * q + 2] = dot2_bf16(fp8_pair_bf16<0>(hi), xp, acc[4 * q + 2]);
      acc[4 * q + 3] = dot2_bf16(fp8_pair_bf16<1>(hi), xp, acc[4 * q + 3]);
    }
  }
}

// FP8 down rows: row r (one h value) times its 16 bytes, decoded to f32 pairs
template <int ROWS>
__device__ __forceinline__ void rows_dot_f32_fp8(const uint4 (&wv)[ROWS], const float (&hf)[ROWS],
                                                 float (&acc)[16]) {
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const uint32_t d[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x2_t f0 = fp8_pair_f32<0>(d[q]), f1 = fp8_pair_f32<1>(d[q]);
      acc[4 * q + 0] = fmaf(f0.x, hf[r], acc[4 * q + 0]);
      acc[4 * q + 1] = fmaf(f0.y, hf[r], acc[4 * q + 1]);
      acc[4 * q + 2] = fmaf(f1.x, hf[r], acc[4 * q + 2]);
      acc[4 * q + 3] = fmaf(f1.y, hf[r], acc[4 * q + 3]);
    }
  }
}

template <int FMT, int ROWS>
__device__ __forceinline__ void rows_dot_f32(const uint4 (&wv)[ROWS], const float (&hf)[2 * ROWS],
                                             float (&acc)[16]) {
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const uint32_t d[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
    const float x0 = hf[2 * r], x1 = hf[2 * r + 1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (FMT == FMT_FP4) {
        f32x2_t f[4];
        f[0] = fp4_pair_f32<0>(d[q]);
        f[1] = fp4_pair_f32<1>(d[q]);
        f[2] = fp4_pair_f32<2>(d[q]);
        f[3] = fp4_pair_f32<3>(d[q]);
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[4 * q + b] = fmaf(f[b].y, x1, fmaf(f[b].x, x0, acc[4 * q + b]));
      } else {
        const uint32_t lo = d[q] & 0x0F0F0F0Fu;
        const uint32_t hi = (d[q] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float fl = (float)((lo >> (8 * b)) & 0xFFu);
          const float fh = (float)((hi >> (8 * b)) & 0xFFu);
          acc[4 * q + b] = fmaf(fh, x1, fmaf(fl, x0, acc[4 * q + b]));
        }
      }
    }
  }
}

// With one token the k experts are distinct and their weights and scales are read once per
// call: non-temporal loads (`nt`, uniform), so that streaming them does not evict from L2 the
// exchange rows and the code that the end of the chain runs.  With several tokens an expert
// chosen twice is streamed once per slot and its repeats are meant to hit L2: plain loads.
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_nt t = __builtin_nontemporal_load(static_cast<const u32x4_nt*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <int ROWS>
__device__ __forceinline__ void load_rows(const uint8_t* wp, size_t ld, uint4 (&wv)[ROWS],
                                          bool nt) {
  if (nt) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) wv[r] = ld_stream16(wp + (size_t)r * ld);
  } else {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) wv[r] = *reinterpret_cast<const uint4*>(wp + (size_t)r * ld);
  }
}

__device__ __forceinline__ void scales16(const uint16_t* sp, float (&sf)[16], bool nt) {
  uint4 s0, s1;
  if (nt) {
    s0 = ld_stream16(sp);
    s1 = ld_stream16(sp + 8);
  } else {
    s0 = *reinterpret_cast<const uint4*>(sp);
    s1 = *reinterpret_cast<const uint4*>(sp + 8);
  }
  const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sf[2 * i] = bf16_lo(sw[i]);
    sf[2 * i + 1] = bf16_hi(sw[i]);
  }
}

// x pairs of byte rows r0 .. r0+ROWS-1 (+ the INT4 bias correction of those rows)
template <int FMT, int ROWS>
__device__ __forceinline__ float load_x_rows(const uint16_t* x, int r0, uint32_t (&xr)[ROWS]) {
  static_assert(ROWS % 4 == 0, "x pairs are loaded 4 at a time");
  const uint4* xp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint32_t*>(x) + r0);
#pragma unroll
  for (int i = 0; i < ROWS / 4; ++i) {
    const uint4 v = xp[i];
    xr[4 * i] = v.x; xr[4 * i + 1] = v.y; xr[4 * i + 2] = v.z; xr[4 * i + 3] = v.w;
  }
  float corr = 0.0f;
  if constexpr (FMT == FMT_INT4) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const f16x2_t h = {(_Float16)bf16_lo(xr[r]), (_Float16)bf16_hi(xr[r])};
      xr[r] = __builtin_bit_cast(uint32_t, h);
      corr = fmaf(-INT4_F16_BIAS_LO, (float)h.x, corr);
      corr = fmaf(-INT4_F16_BIAS_HI, (float)h.y, corr);
    }
  }
  return corr;
}

// Poll n (1 <= n <= NG) published floats p[i * stride] until none is the empty pattern; all
// loads of one round are in flight together.  Every round issues NG loads (those past n repeat
// the last one), so that the code has no branches: the units that run it do so once per
// launch, at the end of the layer's dependency chain, from an instruction cache that the
// weight stream has left cold, and code size is time there.  `tight`: no sleep between
// rounds (one token: few units poll, and each round trip is on the critical path; measured
// 0.08 us faster at the 128-expert shape, while with 8 tokens the extra polling traffic of
// many more units slowed the layer).  Returns false on timeout.
constexpr int FX_GATHER = 16;
template <int NG>
__device__ __forceinline__ bool gather_sc1(const float* p, size_t stride, int n, float* v,
                                           bool tight) {
  for (unsigned spins = 0; spins < FX_SPIN_LIMIT; ++spins) {
    bool ready = true;
#pragma unroll
    for (int i = 0; i < NG; ++i) v[i] = ld_sc1(p, (size_t)(i < n ? i : n - 1) * stride);
#pragma unroll
    for (int i = 0; i < NG; ++i) ready = ready && (__float_as_uint(v[i]) != 0u);
    if (ready) return true;
    if (!tight) __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// EXT: the call uses router units or router partial rows, a per-expert format table,
// codebooks or the logits output.  Without them (EXT false) those paths are compiled out:
// the plain layer's code is then shorter and denser, which the cold instruction fetches on
// its dependency chain repay (Q30 T = 1 12.3 -> 11.6 us, T = 4 24.7 -> 22.9 us).
template <int FMT, int GUR, int DR, bool EXT>
__global__ void __launch_bounds__(FX_THREADS) fused_layer_kernel(FusedArgs a) {
  constexpr int KB = fmt_kb(FMT);                  // K indices per stored byte
  constexpr int KROWS = fx_krows(GUR);             // gate_up byte rows per unit
  constexpr int MAX_KS = 2048 / KB / KROWS;        // gate_up K splits (H <= 2048)
  constexpr int DROWS = 32 * DR;                   // down byte rows per unit
  constexpr int NH = KB * DROWS;                   // h values of a down unit
  constexpr int NPL = KB * DR;                     // h values of a down lane
  // the final units gather a token's chunk rows in rounds of FXG loads (128-row chunks: up
  // to 33 chunks per token in one round)
  constexpr int FXG = DR == 4 ? 32 : FX_GATHER;
  __shared__ int s_ids[32];
  __shared__ int s_key[32];
  __shared__ float s_w[32];
  __shared__ __align__(16) float s_red[FX_THREADS * 16];
  __shared__ __align__(16) long long s_route[64 * 8 + 68];
  __shared__ __align__(4) unsigned char s_fmt[FMT == FMT_FP4 ? 512 : 4];  // per-expert formats
  __shared__ uint4 s_cb[FMT == FMT_FP4 ? 2 * 512 : 1];  // FE-XC codebooks: 2 sets of [2][256]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if constexpr (!EXT) {
    a.efmt = nullptr;
    a.cb = nullptr;
    a.wr = nullptr;
    a.n_r = 0;
    a.logits_out = nullptr;
  }
  const int H = a.H, I = a.I, k = a.k;
  const bool nt = a.T == 1;  // weights streamed once: non-temporal loads; polls back to back
  const int NT = I / 128, KS = a.ks, NC = a.n_chunks;
  const size_t rsz = (size_t)a.rs * a.T * a.E;       // one copy of the router partial rows

  if ((int)blockIdx.x < a.n_r) {
    // ================= router unit: rows [128 rs, 128 rs + 128) of W_r, all T tokens =====
    const unsigned c0 = ld_cnt(a.rcalls);
    float pv[RT_MAX_T];
    router_unit(a.x, H, a.wr, a.E, blockIdx.x, 0, 0, a.T, s_red, tid, pv);
    const int par = (int)((__builtin_amdgcn_readfirstlane(c0) >> 20) & 1u);
    if (tid < a.E) {
      for (int t = 0; t < a.T; ++t) {
        const size_t o = ((size_t)blockIdx.x * a.T + t) * a.E + tid;
        st_sc1(a.rpart + par * rsz, o, pub(pv[t]));
        st_sc1(a.rpart + (1 - par) * rsz, o, 0.0f);
      }
    }
    return;
  }
  const int bid = blockIdx.x - a.n_r;
  // the token this workgroup works for: a gate_up unit's slot's, a down unit's chunk's
  // (chunks never span tokens when T > 1)
  const int tok = (a.T == 1) ? 0
                  : (bid < a.n_a) ? (bid / KS / NT) / k
                                  : ((bid - a.n_a) % NC) / a.chunks_per_token;

  // ---- routing of that token by one wavefront per workgroup (E <= 512); which one varies
  // with the block id, so that the routing waves of the workgroups sharing a compute unit
  // tend to land on different SIMDs.  Only the down units need the weights; a gate_up unit
  // only needs its slot's id. ----
  if (wv == (int)(blockIdx.x & 3)) {
    // mixed layer: the expert formats (4 per lane-word, E % 4 == 0) are loaded here and
    // stored to LDS after the selection, so that their loads are in flight together with the
    // routing's own
    uint32_t fw[2] = {0u, 0u};
    if constexpr (FMT == FMT_FP4) {
      if (a.efmt) {
        const uint32_t* ef = reinterpret_cast<const uint32_t*>(a.efmt);
        if (4 * lane < a.E) fw[0] = ef[lane];
        if (4 * (lane + 64) < a.E) fw[1] = ef[lane + 64];
      }
    }
    float lg[2] = {0.0f, 0.0f};  // router mode: this lane's logits (elements lane, lane + 64)
    if (a.wr) {
      // gather the token's logits from the router units' partial rows (E <= 128), summed
      // over the row splits in ascending order from +0.0
      const unsigned c0 = ld_cnt(a.rcalls);
      const int par = (int)((__builtin_amdgcn_readfirstlane(c0) >> 20) & 1u);
      const float* rp = a.rpart + par * rsz + (size_t)tok * a.E;
      const size_t st = (size_t)a.T * a.E;
      // branch-free rounds: splits past rs repeat the last one and lanes past E read
      // element E - 1 (their values are polled but never summed into a kept logit)
      const int e0 = min(lane, a.E - 1), e1 = min(lane + 64, a.E - 1);
      bool ok = false;
      for (unsigned spins = 0; spins < FX_SPIN_LIMIT; ++spins) {
        float v0[16], v1[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const size_t qo = (size_t)(q < a.rs ? q : a.rs - 1) * st;
          v0[q] = ld_sc1(rp, qo + e0);
          v1[q] = ld_sc1(rp, qo + e1);
        }
        bool ready = true;
#pragma unroll
        for (int q = 0; q < 16; ++q)
          ready = ready && __float_as_uint(v0[q]) != 0u && __float_as_uint(v1[q]) != 0u;
        if (__all(ready)) {
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (q < a.rs) {
              lg[0] += v0[q];
              lg[1] += v1[q];
            }
          ok = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!ok && lane == 0) atomicOr(a.err, 2);
      const int key[2] = {logit_key(lg[0]), logit_key(lg[1])};
      wave_topk_select_keys<2>(key, a.E, k, lane, s_route, s_ids, s_key);
    } else {
      const float* row = a.logits + (size_t)tok * a.E;
      if (a.E <= 128)
        wave_topk_select<2>(row, a.E, k, lane, s_route, s_ids, s_key);
      else
        wave_topk_select<8>(row, a.E, k, lane, s_route, s_ids, s_key);
    }
    if constexpr (FMT == FMT_FP4) {
      if (a.efmt) {
        uint32_t* sf32 = reinterpret_cast<uint32_t*>(s_fmt);
        if (4 * lane < a.E) sf32[lane] = fw[0];
        if (4 * (lane + 64) < a.E) sf32[lane + 64] = fw[1];
      }
    }
    if (bid >= a.n_a) {
      int sel_e;
      float sel_w;
      wave_topk_weights(s_ids, s_key, k, lane, &sel_e, &sel_w);
      const int ub = bid - a.n_a;
      // the token's last chunk of column tile 0 writes the optional routing outputs
      const bool report = ub / NC == 0 && ub % NC == (tok + 1) * a.chunks_per_token - 1;
      if (lane < k) {
        s_w[lane] = sel_w;
        if (report && a.ids_out) a.ids_out[tok * k + lane] = sel_e;  // each output optional
        if (report && a.w_out) a.w_out[tok * k + lane] = sel_w;
      }
      if (report && a.logits_out) {
        if (lane < a.E) a.logits_out[(size_t)tok * a.E + lane] = lg[0];
        if (lane + 64 < a.E) a.logits_out[(size_t)tok * a.E + lane + 64] = lg[1];
      }
    }
  }
  __syncthreads();
  // The buffer parity is first needed when results are published or gathered: the counter
  // load is issued here, after routing, and its value is taken only at that point (the empty
  // asm keeps the compiler from waiting for it earlier), so that its latency overlaps the
  // weight loads instead of delaying them.
  unsigned calls = __hip_atomic_load(a.calls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int S = a.T * k;                             // slots of the call
  const size_t gsz = (size_t)S * NT * KS * 256;      // one copy of the gate/up partial rows
  const size_t psz = (size_t)a.n_mt * NC * 128;

  if (bid < a.n_a) {
    // ================= gate_up unit (slot s = tok k + j, nt, ks) =================
    const int ks = bid % KS, grp = bid / KS;
    const int s = grp / NT, nt = grp - s * NT;
    const int e = s_ids[s - tok * k];
    const int rl = tid >> 4, ch = tid & 15;
    const size_t ld = 2 * (size_t)I;
    const int col0 = (ch < 8) ? (128 * nt + 16 * ch) : (I + 128 * nt + 16 * (ch - 8));
    const int r0 = ks * KROWS + GUR * rl;                // byte row; K index KB r0
    const uint8_t* w = a.wgu + (size_t)e * (H / KB) * ld;
    bool i2 = false;  // an INT2 or FE-XC expert of a mixed layer: the K range in half the rows
    bool fx = false;  // FE-XC (codebooks staged in LDS)
    if constexpr (FMT == FMT_FP4) {
      if (a.efmt != nullptr) {
        const int f = s_fmt[e];
        fx = f == FMT_FEXC && a.cb != nullptr;
        i2 = f == FMT_INT2 || fx;
      }
    }
    if constexpr (FMT == FMT_FP4) {
      if (fx) {  // the expert's gate_up codebooks, copied into LDS ahead of its codes
        const uint4* src = reinterpret_cast<const uint4*>(a.cb) + (size_t)e * 1024;
        const int wb = 64 * __builtin_amdgcn_readfirstlane(tid >> 6);
        copy_to_lds16(src + tid, s_cb + wb);
        copy_to_lds16(src + 256 + tid, s_cb + 256 + wb);
      }
    }
    uint4 wvv[GUR];
    if (i2)
      load_rows(w + (size_t)(r0 / 2) * ld + col0, ld, reinterpret_cast<uint4(&)[GUR / 2]>(wvv),
                nt);
    else
      load_rows(w + (size_t)r0 * ld + col0, ld, wvv, nt);
    float sf[16];
    scales16(a.sgu + (size_t)e * (H / a.group) * ld + (size_t)((KB * r0) / a.group) * ld + col0,
             sf, nt);
    uint32_t xr[GUR];
    float corr = 0.0f;
    if constexpr (FMT == FMT_FP8)  // x pairs of K indices r0 .. r0 + GUR - 1
      load_x_rows<FMT_FP4, GUR / 2>(a.x + (size_t)tok * H, r0 / 2,
                                    reinterpret_cast<uint32_t(&)[GUR / 2]>(xr));
    else
      corr = load_x_rows<FMT, GUR>(a.x + (size_t)tok * H, r0, xr);
    // all loads above are issued before the first use (the scheduler would otherwise sink
    // some of them to their uses, which serializes memory round trips)
    __builtin_amdgcn_sched_barrier(0);
    float accb[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) accb[c] = 0.0f;
    if constexpr (FMT == FMT_FP8) {
      rows_dot_x_fp8<GUR>(wvv, xr, accb);
    } else {
      if (fx) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's codebook copies have landed
        __syncthreads();
        rows_dot_x_fexc<GUR>(reinterpret_cast<const uint4(&)[GUR / 2]>(wvv), xr, s_cb, accb);
      } else if (i2) {
        corr = rows_dot_x_int2<GUR>(reinterpret_cast<const uint4(&)[GUR / 2]>(wvv), xr, accb);
      } else {
        rows_dot_x<FMT, GUR>(wvv, xr, accb);
      }
    }
    // reduce the 16 row-lanes; thread i then owns partial column i (i < 128 gate, else up)
#pragma unroll
    for (int c = 0; c < 16; ++c) accb[c] = sf[c] * (accb[c] + corr);
    const float mine = wg_colsum<16, FX_THREADS>(accb, s_red, tid);
    const size_t slot = (size_t)grp * KS + ks;
    asm volatile("" : "+v"(calls));
    const int par = (int)((__builtin_amdgcn_readfirstlane(calls) >> 20) & 1u);  // uniform
    st_sc1(a.gpart + par * gsz, slot * 256 + tid, pub(mine));
    st_sc1(a.gpart + (1 - par) * gsz, slot * 256 + tid, 0.0f);
    return;
  }

  // ================= down unit (mt, c) =================
  asm volatile("" : "+v"(calls));
  // uniform, so that the exchange buffers' descriptors stay in scalar registers
  const int par = (int)((__builtin_amdgcn_readfirstlane(calls) >> 20) & 1u);
  const float* gpart = a.gpart + par * gsz;
  float* pbuf = a.ypart + par * psz;
  float* pold = a.ypart + (1 - par) * psz;
  const int ub = bid - a.n_a;
  const int mt = ub / NC, c = ub - mt * NC;
  const int rl = tid >> 3, ch = tid & 7;
  const int col0 = 128 * mt + 16 * ch;
  const int R = c * DROWS + DR * rl;   // row in the concatenated slot list
  const int rows_per_slot = I / KB;
  const bool active = R < S * rows_per_slot;
  const int sl = active ? R / rows_per_slot : tok * k;  // slot of the row
  const int j = sl - tok * k;                           // its rank within the token
  const int r0 = active ? R - sl * rows_per_slot : 0;
  // The down weights are needed only once h is complete: on layers whose gate_up weights
  // take long enough to stream to matter (hold_down), hold their loads until the first
  // gate/up partial of this unit's range is published, so that the gate_up units, which are
  // on the critical path, have the memory bandwidth to themselves until then.
  if (a.hold_down) {
    const int f0 = NH * c;
    if (tid == 0 && f0 < S * I) {
      const int jj = f0 / I, n = f0 - jj * I;
      const float* p = gpart + ((size_t)((jj * NT + (n >> 7)) * KS + KS - 1)) * 256 + (n & 127);
      for (unsigned spins = 0; spins < FX_SPIN_LIMIT; ++spins) {
        if (__float_as_uint(ld_sc1(p, 0)) != 0u) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
  }
  uint4 wvv[DR];
  float sf[16];
  bool i2 = false;  // an INT2 or FE-XC expert of a mixed layer
  bool fx = false;  // FE-XC: codebook set `cset` (the chunk's first or second slot)
  int cset = 0;
  // FE-XC codebooks of the chunk's first two slots (a chunk spans at most two when
  // I / 2 >= 256, which the host requires with codebooks), copied into LDS by the whole
  // workgroup once the weight loads are issued, so that they land during the h gather
  int stage_e[2] = {-1, -1};
  const int sl_a = (c * DROWS) / rows_per_slot;
  if constexpr (FMT == FMT_FP4) {
    if (a.efmt != nullptr && a.cb != nullptr) {
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const int slz = sl_a + z;
        if (slz < S && slz * rows_per_slot < (c + 1) * DROWS) {
          const int ez = s_ids[slz - tok * k];
          if (s_fmt[ez] == FMT_FEXC) stage_e[z] = ez;
        }
      }
    }
  }
  if (active) {
    const int e = s_ids[j];
    if constexpr (FMT == FMT_FP4) {
      if (a.efmt != nullptr) {
        const int f = s_fmt[e];
        fx = f == FMT_FEXC && a.cb != nullptr;
        i2 = f == FMT_INT2 || fx;
        cset = sl - sl_a;
      }
    }
    const uint8_t* wd = a.wd + (size_t)e * rows_per_slot * H;
    if (i2)
      load_rows(wd + (size_t)(r0 / 2) * H + col0, H,
                reinterpret_cast<uint4(&)[DR / 2]>(wvv), nt);
    else
      load_rows(wd + (size_t)r0 * H + col0, H, wvv, nt);
    scales16(a.sd + (size_t)e * (I / a.group) * H + (size_t)((KB * r0) / a.group) * H + col0,
             sf, nt);
  }
  const bool staged = stage_e[0] >= 0 || stage_e[1] >= 0;  // uniform
  if constexpr (FMT == FMT_FP4) {
    if (staged) {
      const int wb = 64 * __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
      for (int z = 0; z < 2; ++z)
        if (stage_e[z] >= 0) {
          const uint4* src = reinterpret_cast<const uint4*>(a.cb) + (size_t)stage_e[z] * 1024 + 512;
          copy_to_lds16(src + tid, s_cb + 512 * z + wb);
          copy_to_lds16(src + 256 + tid, s_cb + 512 * z + 256 + wb);
        }
    }
  }
  // gather h for this unit's rows: flat h index f = KB R covers the NH values from NH c on;
  // thread t < NH / 2 owns f = NH c + 2t, +1 (two columns of one slot); the KS partial gate
  // and up pairs are polled together and summed in ascending ks
  float* hl = s_red;  // NH floats, reused as the reduction buffer afterwards
  if (tid < NH / 2) {
    const int f = NH * c + 2 * tid;
    float2 h2 = make_float2(0.0f, 0.0f);
    if (f < S * I) {
      const int jj = f / I, n = f - jj * I, nt = n >> 7, nc = n & 127;
      const __amdgpu_buffer_rsrc_t gr = rsrc(gpart);
      const int base = (((jj * NT + nt) * KS) * 256 + nc) * 4;
      f32x2_t g2 = {0.0f, 0.0f}, u2 = {0.0f, 0.0f};
      bool ok = false;
      for (unsigned spins = 0; spins < FX_SPIN_LIMIT; ++spins) {
        f32x2_t gv[MAX_KS], uv[MAX_KS];
        // every round reloads the partials (the compiler must not keep an earlier round's
        // values) and issues MAX_KS loads of each (those past KS repeat the last: no branches)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < MAX_KS; ++q) {
          const int qq = q < KS ? q : KS - 1;
          gv[q] = __builtin_amdgcn_raw_buffer_load_b64(gr, base + qq * 1024, 0, CPOL_SC1);
          uv[q] = __builtin_amdgcn_raw_buffer_load_b64(gr, base + qq * 1024 + 512, 0, CPOL_SC1);
        }
        bool ready = true;
#pragma unroll
        for (int q = 0; q < MAX_KS; ++q)
          ready = ready && __float_as_uint(gv[q].x) && __float_as_uint(gv[q].y) &&
                  __float_as_uint(uv[q].x) && __float_as_uint(uv[q].y);
        if (ready) {
          g2 = gv[0];
          u2 = uv[0];
#pragma unroll
          for (int q = 1; q < MAX_KS; ++q)
            if (q < KS) {
              g2 += gv[q];
              u2 += uv[q];
            }
          ok = true;
          break;
        }
        if (!nt) __builtin_amdgcn_s_sleep(4);
      }
      if (!ok) atomicOr(a.err, 2);
      // __expf (v_exp_f32 on x log2(e)): a short sequence on the chain's cold tail
      h2 = make_float2(g2.x / (1.0f + __expf(-g2.x)) * u2.x,
                       g2.y / (1.0f + __expf(-g2.y)) * u2.y);
    }
    reinterpret_cast<float2*>(hl)[tid] = h2;
  }
  if constexpr (FMT == FMT_FP4)
    if (staged) __builtin_amdgcn_s_waitcnt(0);  // this wave's codebook copies have landed
  __syncthreads();
  float acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
  if (active) {
    float hf[2 * DR];  // the lane's NPL h values
#pragma unroll
    for (int i = 0; i < NPL / 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(hl)[(NPL / 4) * rl + i];
      hf[4 * i + 0] = v.x;
      hf[4 * i + 1] = v.y;
      hf[4 * i + 2] = v.z;
      hf[4 * i + 3] = v.w;
    }
    float corr = 0.0f;
    if constexpr (FMT == FMT_INT4) {
#pragma unroll
      for (int i = 0; i < 2 * DR; ++i) corr += hf[i];
      corr *= -8.0f;
    }
    float accb[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) accb[q] = 0.0f;
    if constexpr (FMT == FMT_FP8) {
      rows_dot_f32_fp8<DR>(wvv, reinterpret_cast<const float(&)[DR]>(hf), accb);
    } else {
      if (fx)
        rows_dot_f32_fexc<DR>(reinterpret_cast<const uint4(&)[DR / 2]>(wvv), hf,
                                     s_cb + 512 * cset, accb);
      else if (i2)
        corr = rows_dot_f32_int2<DR>(reinterpret_cast<const uint4(&)[DR / 2]>(wvv),
                                            hf, accb);
      else
        rows_dot_f32<FMT, DR>(wvv, hf, accb);
    }
    const float wj = s_w[j];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = wj * (sf[q] * (accb[q] + corr));
  }
  __syncthreads();  // hl is reused by the reduction below
  // reduce the 32 row-lanes; thread i < 128 then owns output column 128 mt + i
  const float mine = wg_colsum<8, FX_THREADS>(acc, s_red, tid);
  if (tid >= 128) return;
  const int m = 128 * mt + tid;
  const int NCt = a.chunks_per_token, c_first = tok * NCt;
  const size_t row0 = (size_t)mt * NC;
  if (c != c_first + NCt - 1) {
    st_sc1(pbuf, (row0 + c) * 128 + tid, pub(mine));
    st_sc1(pold, (row0 + c) * 128 + tid, 0.0f);
    return;
  }
  // the token's last chunk of the tile: gather its earlier chunks' rows (all in flight),
  // ascending c
  float y = 0.0f;
  for (int c0 = 0; c0 < NCt - 1; c0 += FXG) {
    const int n = min(FXG, NCt - 1 - c0);
    float pv[FXG];
    if (!gather_sc1<FXG>(pbuf + (row0 + c_first + c0) * 128 + tid, 128, n, pv, nt))
      atomicOr(a.err, 2);
#pragma unroll
    for (int i = 0; i < FXG; ++i)
      if (i < n) y += pv[i];
  }
  y += mine;
  const size_t o = (size_t)tok * H + m;
  if (a.res) y += bf16_to_f32(a.res[o]);
  a.out[o] = f32_to_bf16(y);
  if (tid == 0) {  // the T x n_mt finishing units add shares summing to 2^20
    const unsigned nf = (unsigned)(a.T * a.n_mt), fi = (unsigned)(tok * a.n_mt + mt);
    const unsigned share = (1u << 20) / nf;
    const unsigned add = (fi + 1 < nf) ? share : (1u << 20) - (nf - 1) * share;
    __hip_atomic_fetch_add(a.calls, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.wr) __hip_atomic_fetch_add(a.rcalls, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// router units in the launch: E <= 128 (two logits per lane of the routing wavefront) and
// at most RT_MAX_T tokens (one router unit covers every token of the call)
bool fused_router_supported(int E, int T) { return E <= 128 && E % 8 == 0 && T <= RT_MAX_T; }

bool fused_supported(int H, int I, int k) {
  return H % 256 == 0 && H <= 2048 && I % 128 == 0 && k <= 32;
}

// T > 1: a token's down rows must fill whole chunks, so that no chunk spans two tokens
bool fused_supported_t(int T, int H, int I, int k, int fmt) {
  return fused_supported(H, I, k) && T >= 1 && T <= FX_MAX_T &&
         (T == 1 || (k * (I / fmt_kb(fmt))) % (32 * FX_DR_MAX) == 0);
}

// gate_up rows per lane: FP8 always 16 (one byte per K index: H / 256 splits at most 8)
static inline int fx_gur(int H, int T, int fmt) { return fmt == FMT_FP8 ? 16 : fx_gu_rows(H, T); }

// Weight bytes of the most loaded compute unit when the gate_up units (n_a of ga bytes) come
// first and the down units (n_b of db bytes) after them.  Measured on MI355X: the dispatcher
// puts workgroup b on XCD b mod 8 and hands each XCD's workgroups to its 32 compute units in
// turn (local index i on unit i mod 32); with every unit's loads in flight at once, a compute
// unit receives its bytes at a roughly fixed share of the bandwidth, so the most loaded one
// ends the weight stream.
static long long fx_max_cu_bytes(int n_a, long long ga, int n_b, long long db) {
  constexpr int XCD = 8, CU = 32;
  long long load[XCD * CU] = {};
  for (int b = 0; b < n_a + n_b; ++b)
    load[(b % XCD) * CU + (b / XCD) % CU] += b < n_a ? ga : db;
  long long m = 0;
  for (long long v : load) m = v > m ? v : m;
  return m;
}

// Down byte rows per lane (DR): 8, or 4 for one token when the smaller down units spread the
// layer's bytes more evenly (the 128-expert shape: 384 gate_up units + 192 down units put
// three 36 KB units on a quarter of the compute units; 384 + 384 smaller ones put at most
// 90 KB on any).  Router units are left out, so that the choice, and with it the workspace
// layout, does not depend on them.
static int fx_down_rows(int H, int I, int k, int T, int fmt) {
  if (T != 1) return FX_DR_MAX;
  const int kb = fmt_kb(fmt);
  const long long rows = (long long)k * (I / kb);                  // down byte rows
  const int ks = H / kb / fx_krows(fx_gur(H, T, fmt));
  const int n_a = k * (I / 128) * ks;
  const long long ga = (long long)fx_krows(fx_gur(H, T, fmt)) * 256;
  const int n_mt = H / 128;
  const int n8 = n_mt * (int)((rows + 255) / 256), n4 = n_mt * (int)((rows + 127) / 128);
  return fx_max_cu_bytes(n_a, ga, n4, 128 * 128) < fx_max_cu_bytes(n_a, ga, n8, 256 * 128)
             ? 4 : FX_DR_MAX;
}

// Sizes of one call's exchange buffers (T tokens, format class of fmt)
struct FxSizes {
  int ks, n_chunks, n_mt, dr;
  size_t gpart, ypart, rpart, total;
};
static FxSizes fx_sizes(int H, int I, int E, int k, int T, int fmt) {
  FxSizes z{};
  const int kb = fmt_kb(fmt);
  z.ks = H / kb / fx_krows(fx_gur(H, T, fmt));
  z.n_mt = H / 128;
  z.dr = fx_down_rows(H, I, k, T, fmt);
  z.n_chunks = (T * k * (I / kb) + 32 * z.dr - 1) / (32 * z.dr);
  z.gpart = 2 * (size_t)T * k * (I / 128) * z.ks * 256 * 4;   // gate/up partial rows
  z.ypart = 2 * (size_t)z.n_mt * z.n_chunks * 128 * 4;        // output partial rows
  z.rpart = fused_router_supported(E, T) ? 2 * (size_t)router_splits(H) * T * E * 4 : 0;
  z.total = (256 + z.gpart + z.ypart + z.rpart + 255) & ~(size_t)255;  // + call counters
  return z;
}

// Workspace of the single-launch layer: per token count T (1 .. FX_MAX_T) one region for the
// 4-bit formats and one for FP8, each with its call counters and its two copies of the
// exchange buffers.  Calls with a different T or format class use different slots, so they
// never meet buffers that another layout left non-empty.
static size_t fused_pair_bytes(int H, int I, int E, int k, int T) {
  return fx_sizes(H, I, E, k, T, FMT_FP4).total + fx_sizes(H, I, E, k, T, FMT_FP8).total;
}

size_t fused_ws_bytes(int H, int I, int E, int k, int t_max) {
  size_t o = 0;
  for (int T = 1; T <= t_max && T <= FX_MAX_T; ++T) o += fused_pair_bytes(H, I, E, k, T);
  return o;
}

// f.fmt must be set
void fused_layout(FusedArgs& f, void* ws, int H, int I, int E, int k, int T, bool with_router) {
  char* p = static_cast<char*>(ws);
  for (int t = 1; t < T; ++t) p += fused_pair_bytes(H, I, E, k, t);
  if (f.fmt == FMT_FP8) p += fx_sizes(H, I, E, k, T, FMT_FP4).total;
  const FxSizes z = fx_sizes(H, I, E, k, T, f.fmt);
  const int kb = fmt_kb(f.fmt);
  f.T = T;
  f.rs = router_splits(H);
  f.n_r = with_router ? f.rs : 0;
  f.ks = z.ks;
  f.n_mt = z.n_mt;
  f.n_chunks = z.n_chunks;
  f.dr = z.dr;
  f.chunks_per_token = f.n_chunks / T;
  f.n_a = T * k * (I / 128) * f.ks;
  f.n_b = f.n_mt * f.n_chunks;
  f.hold_down = (size_t)k * (H / kb) * (2 * (size_t)I) >= ((size_t)1 << 24);
  f.calls = reinterpret_cast<unsigned int*>(p);
  f.rcalls = reinterpret_cast<unsigned int*>(p + 64);  // the router's own parity counter
  f.gpart = reinterpret_cast<float*>(p + 256);
  f.ypart = reinterpret_cast<float*>(p + 256 + z.gpart);
  f.rpart = z.rpart ? reinterpret_cast<float*>(p + 256 + z.gpart + z.ypart) : nullptr;
}

template <bool EXT>
static void launch_fused_ext(const FusedArgs& f, hipStream_t st) {
  const int grid = f.n_r + f.n_a + f.n_b;
  const bool big = fx_gur(f.H, f.T, f.fmt) == 16;
  const dim3 g(grid), b(FX_THREADS);
  // 128-row down chunks (dr 4) are only chosen for one token, where gate_up has 8 rows per
  // lane (16 for FP8)
  const bool d4 = f.dr == 4;
  if (f.fmt == FMT_FP8) {
    if (d4)
      hipLaunchKernelGGL((fused_layer_kernel<FMT_FP8, 16, 4, EXT>), g, b, 0, st, f);
    else
      hipLaunchKernelGGL((fused_layer_kernel<FMT_FP8, 16, 8, EXT>), g, b, 0, st, f);
  } else if (f.fmt == FMT_FP4) {
    if (big)
      hipLaunchKernelGGL((fused_layer_kernel<FMT_FP4, 16, 8, EXT>), g, b, 0, st, f);
    else if (d4)
      hipLaunchKernelGGL((fused_layer_kernel<FMT_FP4, 8, 4, EXT>), g, b, 0, st, f);
    else
      hipLaunchKernelGGL((fused_layer_kernel<FMT_FP4, 8, 8, EXT>), g, b, 0, st, f);
  } else {
    if (big)
      hipLaunchKernelGGL((fused_layer_kernel<FMT_INT4, 16, 8, EXT>), g, b, 0, st, f);
    else if (d4)
      hipLaunchKernelGGL((fused_layer_kernel<FMT_INT4, 8, 4, EXT>), g, b, 0, st, f);
    else
      hipLaunchKernelGGL((fused_layer_kernel<FMT_INT4, 8, 8, EXT>), g, b, 0, st, f);
  }
}

hipError_t launch_fused_layer(const FusedArgs& f, hipStream_t st) {
  const bool ext = f.n_r > 0 || f.wr || f.efmt || f.cb || f.logits_out;
  if (ext)
    launch_fused_ext<true>(f, st);
  else
    launch_fused_ext<false>(f, st);
  return hipGetLastError();
}

}  // namespace dqg
