// HIP kernels for gfx950: top-k routing, the device-built expert schedule and the dense
// packed INT4 GEMV.  The expert kernels of the multi-launch MoE path are in
// dqg_experts.hip, the single-launch T = 1 layer in dqg_fused.hip.  Host launchers at the
// bottom; the C ABI lives in dqg_api.cpp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqg_device.hpp"
#include "dqg_internal.hpp"

namespace dqg {

// =====================================================================================
// top-k routing: one wavefront per token
// =====================================================================================
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token(logits, t, E, k, lane, ids, wts);
}

// =====================================================================================
// schedule: (optional routing) + per-expert slot lists, one workgroup
// =====================================================================================
constexpr int SCHED_THREADS = 1024;

// exclusive scan of n (<= 4 * SCHED_THREADS) ints in LDS, in place; returns the total
__device__ int block_exclusive_scan(int* a, int n, int* tmp) {
  const int tid = threadIdx.x;
  const int per = (n + SCHED_THREADS - 1) / SCHED_THREADS;
  const int b = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < n) local += a[b + i];
  tmp[tid] = local;
  __syncthreads();
  // Hillis-Steele over SCHED_THREADS partials
  for (int off = 1; off < SCHED_THREADS; off <<= 1) {
    const int v = (tid >= off) ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += v;
    __syncthreads();
  }
  int run = (tid > 0) ? tmp[tid - 1] : 0;
  const int total = tmp[SCHED_THREADS - 1];
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      const int v = a[b + i];
      a[b + i] = run;
      run += v;
    }
  __syncthreads();
  return total;
}

__global__ void __launch_bounds__(SCHED_THREADS) schedule_kernel(MoeArgs a, const float* logits) {
  extern __shared__ int sm[];
  const int E = a.E, T = a.T, k = a.k, TK = T * k;
  int* cnt = sm;                         // [E] slots per expert
  int* aidx = cnt + E;                   // [E] active index of each expert
  int* base = aidx + E;                  // [E] first slot position of each expert
  int* tmp = base + E;                   // [SCHED_THREADS]
  int* chunk_ids = tmp + SCHED_THREADS;  // [SCHED_THREADS]
  int* s_flag = chunk_ids + SCHED_THREADS;
  const int tid = threadIdx.x;

  if (logits) {  // routing from logits, one wave per token
    const int lane = tid & 63, wv = tid >> 6;
    for (int t = wv; t < T; t += SCHED_THREADS / 64)
      route_token(logits, t, E, k, lane, a.ids_w, a.wts_w);
    __threadfence_block();
    __syncthreads();
  }
  const int32_t* ids = a.ids;
  // reset the cross-workgroup counters used by the expert kernels of this call
  for (int i = tid; i < a.ws.n_cnt; i += SCHED_THREADS) a.ws.cnt[i] = 0u;
  for (int i = tid; i < E; i += SCHED_THREADS) cnt[i] = 0;
  if (tid == 0) *s_flag = 0;
  __syncthreads();
  for (int i = tid; i < TK; i += SCHED_THREADS) {
    const int e = ids[i];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else
      *s_flag = 1;
  }
  for (int t = tid; t < T; t += SCHED_THREADS) {
    int nv = 0;
    for (int j = 0; j < k; ++j) {
      const int e = ids[t * k + j];
      nv += (e >= 0 && e < E);
    }
    a.ws.nvalid[t] = nv;
  }
  __syncthreads();
  if (tid == 0 && *s_flag) atomicOr(a.ws.err, 1);
  // active experts in ascending id order; slot offsets per expert
  for (int i = tid; i < E; i += SCHED_THREADS) {
    aidx[i] = cnt[i] > 0 ? 1 : 0;
    base[i] = cnt[i];
  }
  __syncthreads();
  const int n_active = block_exclusive_scan(aidx, E, tmp);
  const int total = block_exclusive_scan(base, E, tmp);
  for (int i = tid; i < E; i += SCHED_THREADS)
    if (cnt[i] > 0) {
      a.ws.act_expert[aidx[i]] = i;
      a.ws.act_off[aidx[i]] = base[i];
    }
  if (tid == 0) {
    *a.ws.n_active = n_active;
    a.ws.act_off[n_active] = total;
  }
  __syncthreads();
  // stable placement: slots of one expert keep ascending slot order
  for (int c0 = 0; c0 < TK; c0 += SCHED_THREADS) {
    const int i = c0 + tid;
    const int e = (i < TK) ? ids[i] : -1;
    chunk_ids[tid] = e;
    __syncthreads();
    if (e >= 0 && e < E) {
      int rank = 0;
      for (int q = 0; q < tid; ++q) rank += (chunk_ids[q] == e);
      a.ws.slot_list[base[e] + rank] = i;
    }
    __syncthreads();
    if (e >= 0 && e < E) atomicAdd(&base[e], 1);
    __syncthreads();
  }
  // tokens with no valid slot: out = residual (or zero)
  for (int t = 0; t < T; ++t) {
    if (a.ws.nvalid[t] != 0) continue;
    for (int m = tid; m < a.H; m += SCHED_THREADS)
      a.out[(size_t)t * a.H + m] = a.res ? a.res[(size_t)t * a.H + m] : (uint16_t)0;
  }
}

// Column totals of acc[NT][16] over the workgroup's row-lanes, token by token, through one
// LDS transpose each (wg_colsum); tot[t * COLS + c] receives token t's total of column c.
template <int CPR, int THREADS, int NT>
__device__ __forceinline__ void colsum_tokens(const float (&acc)[NT][16], float* red, float* tot,
                                              int tid) {
  constexpr int COLS = CPR * 16;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float v = wg_colsum<CPR, THREADS>(acc[t], red, tid);
    if (tid < COLS) tot[t * COLS + tid] = v;
    __syncthreads();
  }
}

// =====================================================================================
// dense packed INT4 GEMV
// =====================================================================================
constexpr int GV_THREADS = 256, GV_CPR = 4, GV_RL = GV_THREADS / GV_CPR, GV_WAVES = 4;

template <int NT>
__global__ void __launch_bounds__(GV_THREADS) gemv_kernel(GemvArgs g) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = g.K, N = g.N, T = g.T;
  const int Kp = K / 2, nblk = K / 32;
  const int tid = threadIdx.x, rl = tid / GV_CPR, ch = tid % GV_CPR;
  const int tile = blockIdx.x;
  const int col0 = tile * 64 + 16 * ch;
  const int S = gridDim.y, s = blockIdx.y;
  const int b0 = (s * nblk) / S, b1 = ((s + 1) * nblk) / S;
  uint32_t* xl = reinterpret_cast<uint32_t*>(smem);
  float* corr = reinterpret_cast<float*>(xl + NT * Kp);
  float* red = corr + NT * nblk;                                      // [GV_THREADS * 16]
  float* tot = red + GV_THREADS * 16;                                 // [NT][64]
  __shared__ int s_flag;

  for (int c0 = 0; c0 < T; c0 += NT) {
    const uint16_t* src[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) src[t] = (c0 + t < T) ? g.x + (size_t)(c0 + t) * K : nullptr;
    __syncthreads();
    stage_bf16_rows<X_F16, FMT_INT4, NT>(src, Kp, xl, corr, GV_THREADS, tid);
    __syncthreads();
    float acc[NT][16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[t][j] = 0.0f;
    tile_rows<FMT_INT4, X_F16, NT>(g.w, g.s, N, g.group, col0, b0 + rl, b1, GV_RL, xl, Kp, corr,
                                   nblk, acc);
    colsum_tokens<GV_CPR, GV_THREADS, NT>(acc, red, tot, tid);
    for (int i = tid; i < NT * 64; i += GV_THREADS) {
      const int t = i / 64, c = i % 64;
      if (c0 + t >= T) continue;
      const float v = tot[t * 64 + c];
      const int n = tile * 64 + c;
      if (S == 1)
        g.y[(size_t)(c0 + t) * N + n] = f32_to_bf16(v);
      else
        st_sc1(g.part, ((size_t)s * T + c0 + t) * N + n, v);
    }
  }
  if (S == 1) return;
  unsigned* counter = g.cnt + tile;
  if (!last_arriver(counter, (unsigned)S, &s_flag)) return;
  for (int i = tid; i < T * 64; i += GV_THREADS) {
    const int t = i / 64, n = tile * 64 + i % 64;
    float v = 0.0f;
    for (int q = 0; q < S; ++q) v += ld_sc1(g.part, ((size_t)q * T + t) * N + n);
    g.y[(size_t)t * N + n] = f32_to_bf16(v);
  }
  if (tid == 0) st_cnt(counter, 0u);
}

// =====================================================================================
// test aid: dequantize with the compute kernels' decode
// =====================================================================================
template <int FMT>
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ w,
                                                      const uint16_t* __restrict__ s, int K, int N,
                                                      int group, float* __restrict__ out) {
  // one thread per 4 bytes of one byte row
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nq = (size_t)(K / 2) * (N / 4);
  if (idx >= nq) return;
  const int r = (int)(idx / (N / 4));
  const int n = (int)(idx % (N / 4)) * 4;
  const uint32_t d = *reinterpret_cast<const uint32_t*>(w + (size_t)r * N + n);
  float lo[4], hi[4];
  if constexpr (FMT == FMT_FP4) {
    const bf16x2_t p[4] = {fp4_pair_bf16<0>(d), fp4_pair_bf16<1>(d), fp4_pair_bf16<2>(d),
                           fp4_pair_bf16<3>(d)};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t u = __builtin_bit_cast(uint32_t, p[b]);
      lo[b] = bf16_lo(u);
      hi[b] = bf16_hi(u);
    }
  } else {
    const f16x2_t p[4] = {int4_pair_f16_biased<0>(d), int4_pair_f16_biased<1>(d),
                          int4_pair_f16_biased<2>(d), int4_pair_f16_biased<3>(d)};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      lo[b] = (float)p[b].x - (INT4_F16_BIAS_LO - 8.0f) - 8.0f;
      hi[b] = (float)p[b].y - (INT4_F16_BIAS_HI - 8.0f) - 8.0f;
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float sc_lo = bf16_to_f32(s[(size_t)((2 * r) / group) * N + n + b]);
    const float sc_hi = bf16_to_f32(s[(size_t)((2 * r + 1) / group) * N + n + b]);
    out[(size_t)(2 * r) * N + n + b] = lo[b] * sc_lo;
    out[(size_t)(2 * r + 1) * N + n + b] = hi[b] * sc_hi;
  }
}

// =====================================================================================
// host launchers
// =====================================================================================
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* wts,
                       hipStream_t st) {
  const int grid = (T + 3) / 4;
  hipLaunchKernelGGL(topk_kernel, dim3(grid), dim3(256), 0, st, logits, T, E, k, ids, wts);
  return hipGetLastError();
}

hipError_t launch_schedule(const MoeArgs& a, const float* logits, hipStream_t st) {
  const size_t sm = (size_t)(3 * a.E + 2 * SCHED_THREADS + 4) * sizeof(int);
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(SCHED_THREADS), sm, st, a, logits);
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_gemv_t(const GemvArgs& g, hipStream_t st) {
  const int Kp = g.K / 2, nblk = g.K / 32;
  const size_t sm = (size_t)NT * Kp * 4 + (size_t)NT * nblk * 4 + (size_t)GV_THREADS * 16 * 4 +
                    (size_t)NT * 64 * 4;
  hipLaunchKernelGGL(gemv_kernel<NT>, dim3(g.N / 64, g.S), dim3(GV_THREADS), sm, st, g);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs& g, int nt, hipStream_t st) {
  if (nt == 1) return launch_gemv_t<1>(g, st);
  if (nt == 2) return launch_gemv_t<2>(g, st);
  return launch_gemv_t<4>(g, st);
}

hipError_t launch_dequant(const uint8_t* w, const uint16_t* s, int K, int N, int group, int fmt,
                          float* out, hipStream_t st) {
  const size_t nq = (size_t)(K / 2) * (N / 4);
  const int grid = (int)((nq + 255) / 256);
  if (fmt == FMT_FP4)
    hipLaunchKernelGGL(dequant_kernel<FMT_FP4>, dim3(grid), dim3(256), 0, st, w, s, K, N, group,
                       out);
  else
    hipLaunchKernelGGL(dequant_kernel<FMT_INT4>, dim3(grid), dim3(256), 0, st, w, s, K, N, group,
                       out);
  return hipGetLastError();
}

}  // namespace dqg
