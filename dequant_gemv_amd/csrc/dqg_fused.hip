// Single-launch packed-MoE layer for one token (T = 1): routing, fused gate_up, SiLU*up,
// down projection and the top-k combine in one kernel.
//
// FireEcho page, "The Goliath Kernel: Why It's Fast": one launch reads the expert ids from
// device memory and indexes the contiguous packed buffer, with the dequant in registers
// inside the tile loop.  On MI355X a launch costs about 1.6 us even inside a graph, a whole
// T=1 layer moves only ~21 MB, and every dependent memory round trip costs about 1 us, so
// the layer is one launch and its workgroups exchange data with as few round trips as
// possible: consumers poll the data itself instead of a separate counter.
//
// Workgroups (256 threads, 4 waves) play one of two roles, decided by blockIdx.x:
//   gate_up (the first n_a = k * I/32 workgroups): slot j, h columns [32t, 32t+32).  64
//     row-lanes x 4 lanes (2 x 16 B of gate, 2 x 16 B of up per byte row) walk all H/32
//     K blocks; the K reduction stays in registers, wave shuffles and LDS.  SiLU(g)*u is
//     stored to the h buffer with agent-coherent (sc1) stores.
//   down + combine (the rest): output columns [64m, 64m+64) for one chunk of 64 K blocks
//     of the concatenated (slot, K block) list.  The weights are loaded first; then each
//     lane polls the 32 h values of its block until they are all published, scales its
//     block sum by its slot weight, and the workgroup reduces in LDS.  The last chunk of a
//     column tile polls the other chunks' partial rows, sums all chunks in ascending order,
//     adds the residual and writes bf16 out (deterministic).
// Publication protocol: the h and partial buffers hold the bit pattern 0 when empty, and a
// producer never stores 0 (+0.0 is stored as -0.0, which computes identically).  Each
// buffer exists twice; a call uses copy p = (completed calls) & 1, read from a 64-bit call
// counter that the last chunk of every column tile increments without waiting, and its
// producers clear their slots of copy 1-p, which the previous call used and which the next
// call will use.  Polls are bounded and report a timeout in the error word (bit 1) instead
// of hanging.  Down workgroups only wait on workgroups with lower block ids (gate_up, and
// the earlier chunks of their tile), so in-order dispatch cannot deadlock.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqg_device.hpp"
#include "dqg_internal.hpp"

namespace dqg {

constexpr int FX_THREADS = 256;
constexpr int FX_RL = 64;          // row-lanes per workgroup (4 lanes per byte row)
constexpr unsigned FX_SPIN_LIMIT = 1u << 20;
constexpr int CPOL_SC1 = 16;       // cache-policy operand: agent-coherent access

// published value: never the empty pattern 0 (+0.0 becomes -0.0)
__device__ __forceinline__ float pub(float v) {
  return __float_as_uint(v) == 0u ? __uint_as_float(0x80000000u) : v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7FFFFFFF, 0x00020000);
}

// sum over the 16 row-lanes of a wave that share (lane % 4)
__device__ __forceinline__ float wave_sum_rl4(float v) {
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// One K block (16 byte rows) of a lane's 16 columns against activations held in
// registers: xr[r] is the pair for byte row r (bf16 for FP4, fp16 for INT4 in the gate_up
// role); for the fp32 role xf[2r], xf[2r+1].
template <int FMT>
__device__ __forceinline__ void block_dot_x16(const uint4 (&wv)[BLK_ROWS],
                                              const uint32_t (&xr)[BLK_ROWS], float (&acc)[16]) {
#pragma unroll
  for (int r = 0; r < BLK_ROWS; ++r) {
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

template <int FMT>
__device__ __forceinline__ void block_dot_f32(const uint4 (&wv)[BLK_ROWS],
                                              const float (&xf)[2 * BLK_ROWS], float (&acc)[16]) {
#pragma unroll
  for (int r = 0; r < BLK_ROWS; ++r) {
    const uint32_t d[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
    const float x0 = xf[2 * r], x1 = xf[2 * r + 1];
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

__device__ __forceinline__ void load_block(const uint8_t* wp, size_t ld, uint4 (&wv)[BLK_ROWS]) {
#pragma unroll
  for (int r = 0; r < BLK_ROWS; ++r) wv[r] = *reinterpret_cast<const uint4*>(wp + (size_t)r * ld);
}

__device__ __forceinline__ void scales16(const uint16_t* sp, float (&sf)[16]) {
  const uint4 s0 = *reinterpret_cast<const uint4*>(sp);
  const uint4 s1 = *reinterpret_cast<const uint4*>(sp + 8);
  const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sf[2 * i] = bf16_lo(sw[i]);
    sf[2 * i + 1] = bf16_hi(sw[i]);
  }
}

// block b of the gate_up role: x pairs for byte rows 16b..16b+15 (+ INT4 bias correction)
template <int FMT>
__device__ __forceinline__ float load_x_block(const uint16_t* x, int b, uint32_t (&xr)[BLK_ROWS]) {
  const uint4* xp = reinterpret_cast<const uint4*>(x) + b * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = xp[i];
    xr[4 * i + 0] = v.x;
    xr[4 * i + 1] = v.y;
    xr[4 * i + 2] = v.z;
    xr[4 * i + 3] = v.w;
  }
  float corr = 0.0f;
  if constexpr (FMT == FMT_INT4) {
#pragma unroll
    for (int r = 0; r < BLK_ROWS; ++r) {
      const f16x2_t h = {(_Float16)bf16_lo(xr[r]), (_Float16)bf16_hi(xr[r])};
      xr[r] = __builtin_bit_cast(uint32_t, h);
      corr = fmaf(-INT4_F16_BIAS_LO, (float)h.x, corr);
      corr = fmaf(-INT4_F16_BIAS_HI, (float)h.y, corr);
    }
  }
  return corr;
}

template <int FMT>
__global__ void __launch_bounds__(FX_THREADS) fused_t1_kernel(FusedArgs a) {
  __shared__ int s_ids[32];
  __shared__ float s_w[32];
  __shared__ float s_red[4][64];
  __shared__ int s_par;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I, k = a.k;
  const int rl = tid >> 2, ch = tid & 3;
  const int n_mt = H / 64;

  // ---- routing (wave 0 of every workgroup) and the buffer parity (wave 1) ----
  if (wv == 0) {
    int e;
    float w;
    route_row<512>(a.logits, a.E, k, lane, &e, &w);
    if (lane < k) {
      s_ids[lane] = e;
      s_w[lane] = w;
      if (blockIdx.x == 0 && a.ids_out) {
        a.ids_out[lane] = e;
        a.w_out[lane] = w;
      }
    }
  } else if (tid == 64) {
    const unsigned long long calls =
        __hip_atomic_load(a.calls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_par = (int)((calls / (unsigned long long)n_mt) & 1ull);
  }
  __syncthreads();
  const int par = s_par;
  float* hbuf = a.h + (size_t)par * k * I;
  float* hold = a.h + (size_t)(1 - par) * k * I;
  float* pbuf = a.ypart + (size_t)par * a.n_chunks * H;
  float* pold = a.ypart + (size_t)(1 - par) * a.n_chunks * H;

  const int bid = blockIdx.x;
  const int tiles_a = I / 32;
  if (bid < a.n_a) {
    // ================= gate_up role =================
    int u = bid;
    if ((a.n_a & 31) == 0) {  // keep the 4 tiles that share 128-byte lines on one XCD
      const int xcd = bid & 7, slot = bid >> 3;
      u = (slot >> 2) * 32 + xcd * 4 + (slot & 3);
    }
    const int j = u / tiles_a, t = u - j * tiles_a;
    const int e = s_ids[j];
    const size_t ld = 2 * (size_t)I;
    const uint8_t* w = a.wgu + (size_t)e * (H / 2) * ld;
    const uint16_t* sc = a.sgu + (size_t)e * (H / a.group) * ld;
    const int col0 = (ch < 2) ? (32 * t + 16 * ch) : (I + 32 * t + 16 * (ch - 2));
    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.0f;
    const int nblk = H / 32;
    for (int b = rl; b < nblk; b += FX_RL) {
      uint4 wvv[BLK_ROWS];
      load_block(w + (size_t)b * BLK_ROWS * ld + col0, ld, wvv);
      float sf[16];
      scales16(sc + (size_t)((b * 32) / a.group) * ld + col0, sf);
      uint32_t xr[BLK_ROWS];
      const float corr = load_x_block<FMT>(a.x, b, xr);
      float accb[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) accb[c] = 0.0f;
      block_dot_x16<FMT>(wvv, xr, accb);
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = fmaf(sf[c], accb[c] + corr, acc[c]);
    }
    // reduce over row-lanes: 16 per wave, then 4 waves
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float v = wave_sum_rl4(acc[c]);
      if (lane < 4) s_red[wv][lane * 16 + c] = v;
    }
    __syncthreads();
    if (tid < 32) {
      // column n of the tile: gate sum in s_red[.][n], up sum in s_red[.][32 + n]
      float g = 0.0f, uu = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        g += s_red[q][tid];
        uu += s_red[q][32 + tid];
      }
      const int idx = j * I + 32 * t + tid;
      st_sc1(hbuf, idx, pub(g / (1.0f + expf(-g)) * uu));
      st_sc1(hold, idx, 0.0f);
    }
    return;
  }

  // ================= down + combine role =================
  const int nblkI = I / 32;
  int ub = bid - a.n_a;
  if ((a.n_b & 15) == 0) {  // adjacent 64-column tiles (one 128-byte line) on one XCD
    const int xcd = ub & 7, slot = ub >> 3;
    ub = (slot >> 1) * 16 + xcd * 2 + (slot & 1);
  }
  const int chunk = ub / n_mt, mt = ub - chunk * n_mt;
  const int q = chunk * FX_RL + rl;  // this row-lane's (slot, K block)
  const bool active = q < k * nblkI;
  const int j = active ? q / nblkI : 0;
  const int b = active ? q - j * nblkI : 0;
  const int col0 = 64 * mt + 16 * ch;
  float acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = 0.0f;
  if (active) {
    uint4 wvv[BLK_ROWS];
    float sf[16];
    const int e = s_ids[j];
    const uint8_t* w = a.wd + (size_t)e * (I / 2) * H;
    const uint16_t* sc = a.sd + (size_t)e * (I / a.group) * H;
    load_block(w + (size_t)b * BLK_ROWS * H + col0, H, wvv);
    scales16(sc + (size_t)((b * 32) / a.group) * H + col0, sf);
    // poll the 32 h values of this block until all are published
    float hf[2 * BLK_ROWS];
    const __amdgpu_buffer_rsrc_t hr = rsrc(hbuf);
    const int hoff = (j * I + 32 * b) * 4;
    unsigned spins = 0;
    while (true) {
      bool ready = true;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(hr, hoff + 16 * i, 0, CPOL_SC1);
        hf[4 * i + 0] = v.x;
        hf[4 * i + 1] = v.y;
        hf[4 * i + 2] = v.z;
        hf[4 * i + 3] = v.w;
        ready = ready && __float_as_uint(v.x) && __float_as_uint(v.y) && __float_as_uint(v.z) &&
                __float_as_uint(v.w);
      }
      if (ready) break;
      if (++spins > FX_SPIN_LIMIT) {
        atomicOr(a.err, 2);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    float corr = 0.0f;
    if constexpr (FMT == FMT_INT4) {
#pragma unroll
      for (int i = 0; i < 2 * BLK_ROWS; ++i) corr += hf[i];
      corr *= -8.0f;
    }
    float accb[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) accb[c] = 0.0f;
    block_dot_f32<FMT>(wvv, hf, accb);
    const float wj = s_w[j];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = wj * (sf[c] * (accb[c] + corr));
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const float v = wave_sum_rl4(acc[c]);
    if (lane < 4) s_red[wv][lane * 16 + c] = v;
  }
  __syncthreads();
  if (tid >= 64) return;
  const float mine = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
  const int m = 64 * mt + tid;
  if (chunk != a.n_chunks - 1) {
    st_sc1(pbuf, (size_t)chunk * H + m, pub(mine));
    st_sc1(pold, (size_t)chunk * H + m, 0.0f);
    return;
  }
  // last chunk of the tile: gather the earlier chunks' partial rows in order
  float y = 0.0f;
  for (int c = 0; c < a.n_chunks - 1; ++c) {
    float v;
    unsigned spins = 0;
    while (__float_as_uint(v = ld_sc1(pbuf, (size_t)c * H + m)) == 0u) {
      if (++spins > FX_SPIN_LIMIT) {
        atomicOr(a.err, 2);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    y += v;
  }
  y += mine;
  if (a.res) y += bf16_to_f32(a.res[m]);
  a.out[m] = f32_to_bf16(y);
  if (tid == 0) __hip_atomic_fetch_add(a.calls, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

size_t fused_ws_bytes(int H, int I, int k) {
  const int n_chunks = (k * (I / 32) + FX_RL - 1) / FX_RL;
  size_t o = 256;                               // call counter
  o += 2 * (size_t)k * I * 4;                   // h, two copies
  o = (o + 255) & ~(size_t)255;
  o += 2 * (size_t)n_chunks * H * 4;            // partial rows, two copies
  return (o + 255) & ~(size_t)255;
}

void fused_layout(FusedArgs& f, void* ws, int H, int I, int k) {
  char* p = static_cast<char*>(ws);
  f.n_chunks = (k * (I / 32) + FX_RL - 1) / FX_RL;
  f.n_a = k * (I / 32);
  f.n_b = f.n_chunks * (H / 64);
  f.calls = reinterpret_cast<unsigned long long*>(p);
  size_t o = 256;
  f.h = reinterpret_cast<float*>(p + o);
  o += 2 * (size_t)k * I * 4;
  o = (o + 255) & ~(size_t)255;
  f.ypart = reinterpret_cast<float*>(p + o);
}

hipError_t launch_fused_t1(const FusedArgs& f, hipStream_t st) {
  const int grid = f.n_a + f.n_b;
  if (f.fmt == FMT_FP4)
    hipLaunchKernelGGL(fused_t1_kernel<FMT_FP4>, dim3(grid), dim3(FX_THREADS), 0, st, f);
  else
    hipLaunchKernelGGL(fused_t1_kernel<FMT_INT4>, dim3(grid), dim3(FX_THREADS), 0, st, f);
  return hipGetLastError();
}

}  // namespace dqg
