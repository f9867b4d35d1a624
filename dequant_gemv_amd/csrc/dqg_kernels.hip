// HIP kernels for gfx950: top-k routing, the device-built expert schedule and the
// dequantize test aid.  The expert kernels of the multi-launch MoE path and the dense GEMV
// are in dqg_experts.hip, the single-launch layer in dqg_fused.hip; also the router GEMV.  Host launchers at the
// bottom; the C ABI lives in dqg_api.cpp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqg_device.hpp"
#include "dqg_internal.hpp"

namespace dqg {

// =====================================================================================
// top-k routing: one wavefront per token
// =====================================================================================
// LDS scratch entries (8 bytes) of one routing wavefront: wave_topk over E <= 64 * v
constexpr int route_scratch(int v) { return 64 * v + 68; }

__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ wts) {
  __shared__ __align__(16) long long scratch[4][route_scratch(8)];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  if (E > 512) {
    route_token(logits, t, E, k, lane, ids, wts);
    return;
  }
  int e;
  float w;
  if (E <= 128)
    wave_topk<2>(logits + (size_t)t * E, E, k, lane, scratch[wv], &e, &w);
  else
    wave_topk<8>(logits + (size_t)t * E, E, k, lane, scratch[wv], &e, &w);
  if (lane < k) {
    ids[(size_t)t * k + lane] = e;
    wts[(size_t)t * k + lane] = w;
  }
}

// =====================================================================================
// schedule: (optional routing) + per-expert slot lists, one workgroup
// =====================================================================================
// Active experts in ascending id order get records {expert, first slot position, slot
// count, 0} (records past the active count: all zero); the slot list holds, per active
// expert, its slots t*k + j in ascending slot order.
constexpr int SCHED_THREADS = 1024;

constexpr int SCHED_LDS_IDS = 2048;  // slots whose ids are kept in LDS

// Routing wavefronts of the schedule kernel and their LDS scratch (after the int arrays,
// 16-byte aligned): E <= 128 uses all 16 waves, E <= 512 the first 8 (larger scratch each),
// E > 512 the register-free selection with no scratch.
__host__ __device__ constexpr int sched_route_waves(int E) { return E <= 128 ? 16 : (E <= 512 ? 8 : 0); }
__host__ __device__ constexpr int sched_int_words(int E) {
  return (3 * E + 4 + SCHED_THREADS + SCHED_LDS_IDS + 3) & ~3;
}
__host__ __device__ constexpr int sched_scratch_entries(int E) {
  return E <= 128 ? route_scratch(2) : route_scratch(8);
}

// Inclusive prefix sum over the 64 lanes with DPP: shifts by 1, 2, 4, 8 within each row of 16
// lanes (lanes shifted in from outside the row add 0), then the last lane of row 0 into row 1
// and of row 2 into row 3 (row_bcast:15), then lane 31 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// exclusive prefix sums over experts of cnt (-> pos) by wave 0 (lane l takes experts
// [l * per, l * per + per)); with `records`, active experts also get their records.
// Returns the number of active experts in lane 63's s_nact.
__device__ __forceinline__ void sched_scan(const MoeArgs& a, const int* cnt, int* pos, int E,
                                           bool records, int* s_nact) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64, e0 = lane * per;
  int c = 0, n = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      c += cnt[e];
      n += cnt[e] > 0;
    }
  }
  const int ci = wave_incl_sum(c), ni = wave_incl_sum(n);
  int cx = ci - c, nx = ni - n;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int ce = cnt[e];
      pos[e] = cx;
      if (records && ce > 0) a.ws.rec[nx] = make_int4(e, cx, ce, 0);
      cx += ce;
      nx += ce > 0;
    }
  }
  if (lane == 63) *s_nact = ni;
}

__global__ void __launch_bounds__(SCHED_THREADS) schedule_kernel(MoeArgs a, const float* logits) {
  extern __shared__ int sm[];
  const int E = a.E, T = a.T, k = a.k, TK = T * k;
  int* cnt = sm;                                   // [E] slots per expert
  unsigned* mask = reinterpret_cast<unsigned*>(cnt + E);  // [E] token masks of a round
  int* pos = cnt + 2 * E;                          // [E] next slot position
  int* s_misc = pos + E;                           // invalid, n_active, duplicate, empty token
  int* chunk_ids = s_misc + 4;                     // [SCHED_THREADS]
  int* lids = chunk_ids + SCHED_THREADS;           // [SCHED_LDS_IDS] ids when TK fits
  const bool in_lds = TK <= SCHED_LDS_IDS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < E; i += SCHED_THREADS) cnt[i] = 0;
  if (tid < 4) s_misc[tid] = 0;
  // Routing from logits: the routing waves count their tokens' experts (always k distinct,
  // in-range ids) as they select them, so no separate counting pass follows.
  if (logits) __syncthreads();

  if (logits) {  // routing from logits, one wave per token
    const int RW = sched_route_waves(E);
    long long* scratch = reinterpret_cast<long long*>(sm + sched_int_words(E)) +
                         (size_t)wv * sched_scratch_entries(E);
    const int stride = RW ? RW : SCHED_THREADS / 64;
    if (E <= 128) {
      // the logits of the wave's next 4 tokens are loaded together, then selected one after
      // another (rows shift through registers): one memory round trip per 4 tokens
      int* sel = reinterpret_cast<int*>(scratch + 64 * 2 + 4);
      for (int t0 = wv; t0 < T && wv < RW; t0 += 4 * stride) {
        int key[4][2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float* row = logits + (size_t)min(t0 + r * stride, T - 1) * E;
#pragma unroll
          for (int v = 0; v < 2; ++v) key[r][v] = logit_key(row[min(lane + 64 * v, E - 1)]);
        }
#pragma unroll 1
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + r * stride;
          if (t >= T) break;
          int e;
          float w;
          wave_topk_select_keys<2>(key[0], E, k, lane, scratch, sel, sel + 64);
          wave_topk_weights(sel, sel + 64, k, lane, &e, &w);
          if (lane < k) {
            a.ids_w[(size_t)t * k + lane] = e;
            a.wts_w[(size_t)t * k + lane] = w;
            if (in_lds) lids[t * k + lane] = e;
            atomicAdd(&cnt[e], 1);
          }
          if (lane == 0) a.ws.nvalid[t] = k;
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            key[q][0] = key[q + 1][0];
            key[q][1] = key[q + 1][1];
          }
        }
      }
    } else
    for (int t = wv; t < T && (RW == 0 || wv < RW); t += stride) {
      int e;
      float w;
      const float* row = logits + (size_t)t * E;
      if (E <= 128)
        wave_topk<2>(row, E, k, lane, scratch, &e, &w);
      else if (E <= 512)
        wave_topk<8>(row, E, k, lane, scratch, &e, &w);
      else
        route_row<4096>(row, E, k, lane, &e, &w);
      if (lane < k) {
        a.ids_w[(size_t)t * k + lane] = e;
        a.wts_w[(size_t)t * k + lane] = w;
        if (in_lds) lids[t * k + lane] = e;
        atomicAdd(&cnt[e], 1);
      }
      if (lane == 0) a.ws.nvalid[t] = k;
    }
  } else if (in_lds) {
    for (int i = tid; i < TK; i += SCHED_THREADS) lids[i] = a.ids[i];
  }
  if (!in_lds) __threadfence_block();  // routing results are read back from memory
  __syncthreads();
  const int32_t* ids = in_lds ? lids : a.ids;
  if (!logits) {  // given ids: count the valid ones, flag invalid ids and empty tokens
    for (int i = tid; i < TK; i += SCHED_THREADS) {
      const int e = ids[i];
      if (e >= 0 && e < E)
        atomicAdd(&cnt[e], 1);
      else
        s_misc[0] = 1;
    }
    for (int t = tid; t < T; t += SCHED_THREADS) {
      int nv = 0;
      for (int j = 0; j < k; ++j) {
        const int e = ids[t * k + j];
        nv += (e >= 0 && e < E);
      }
      a.ws.nvalid[t] = nv;
      if (nv == 0) s_misc[3] = 1;
    }
    __syncthreads();
  }
  if (tid == 0 && s_misc[0]) atomicOr(a.ws.err, 1);
  if (wv == 0) sched_scan(a, cnt, pos, E, true, &s_misc[1]);
  __syncthreads();
  const int n_active = s_misc[1];
  const int A = min(E, TK);
  if (tid == 0) *a.ws.n_active = n_active;
  for (int i = n_active + tid; i < A; i += SCHED_THREADS) a.ws.rec[i] = make_int4(0, 0, 0, 0);
  // stable placement, 32 tokens per round: a slot's rank within its expert is the number
  // of the round's earlier tokens in the expert's token mask; pos[e] advances per round.
  // A token that lists an expert twice shows up as a mask bit that is already set: then
  // the placement is redone in chunks of SCHED_THREADS slots, rank = earlier equal ids.
  for (int t0 = 0; t0 < T; t0 += 32) {
    for (int e = tid; e < E; e += SCHED_THREADS) mask[e] = 0u;
    __syncthreads();
    const int n_r = min(32, T - t0) * k;  // <= SCHED_THREADS
    const int i = tid;
    const int e = (i < n_r) ? ids[t0 * k + i] : -1;
    const bool ok = e >= 0 && e < E;
    if (ok && (atomicOr(&mask[e], 1u << (i / k)) & (1u << (i / k)))) s_misc[2] = 1;
    __syncthreads();
    if (ok) {
      const int rank = __popc(mask[e] & ((1u << (i / k)) - 1u));
      a.ws.slot_list[pos[e] + rank] = t0 * k + i;
    }
    __syncthreads();
    for (int x = tid; x < E; x += SCHED_THREADS) pos[x] += __popc(mask[x]);
    __syncthreads();
    if (s_misc[2]) break;
  }
  if (s_misc[2]) {
    if (wv == 0) sched_scan(a, cnt, pos, E, false, &s_misc[1]);
    __syncthreads();
    for (int c0 = 0; c0 < TK; c0 += SCHED_THREADS) {
      const int i = c0 + tid;
      const int e = (i < TK) ? ids[i] : -1;
      chunk_ids[tid] = e;
      __syncthreads();
      if (e >= 0 && e < E) {
        int rank = 0;
        for (int q = 0; q < tid; ++q) rank += (chunk_ids[q] == e);
        a.ws.slot_list[pos[e] + rank] = i;
      }
      __syncthreads();
      if (e >= 0 && e < E) atomicAdd(&pos[e], 1);
      __syncthreads();
    }
  }
  // an invalid slot has no expert: its down partial rows are published as zeros, so that
  // the combiners (which read every slot of a token) find them
  if (s_misc[0]) {
    const long long n = (long long)a.S_dn * TK * a.H;
    for (long long idx = tid; idx < n; idx += SCHED_THREADS) {
      const int m = (int)(idx % a.H);
      const long long rest = idx / a.H;
      const int slot = (int)(rest % TK), sp = (int)(rest / TK);
      const int e = ids[slot];
      if (e < 0 || e >= E)
        a.ws.part_dn[((size_t)sp * a.ws.tk_cap + slot) * a.H + m] = __uint_as_float(0x80000000u);
    }
  }
  // tokens with no valid slot: out = residual (or zero)
  if (s_misc[3]) {
    for (int t = 0; t < T; ++t) {
      if (a.ws.nvalid[t] != 0) continue;
      for (int m = tid; m < a.H; m += SCHED_THREADS)
        a.out[(size_t)t * a.H + m] = a.res ? a.res[(size_t)t * a.H + m] : (uint16_t)0;
    }
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
// router logits from the hidden state (FireEcho page, "Architecture": the MoE FFN with
// fused dispatch, read as the plain linear router x W_r): one workgroup per router unit
// (row split rs, 128-column tile ct, group of up to 4 tokens) writes its partials
// part[(rs T + t) E + e]; the reduction adds them in ascending rs from +0.0.  Same
// arithmetic as the router units of the single-launch layer (router_unit).
// =====================================================================================
__global__ void __launch_bounds__(256) router_partial_kernel(const uint16_t* __restrict__ x,
                                                             int T, int H,
                                                             const uint16_t* __restrict__ wr,
                                                             int E, float* __restrict__ part) {
  __shared__ __align__(16) float red[16 * 128];
  const int rs = blockIdx.x, ct = blockIdx.y, t0 = RT_MAX_T * blockIdx.z;
  const int nt = min(RT_MAX_T, T - t0);
  float pv[RT_MAX_T];
  router_unit(x, H, wr, E, rs, ct, t0, nt, red, threadIdx.x, pv);
  const int e = 128 * ct + threadIdx.x;
  if (threadIdx.x < 128 && e < E) {
#pragma unroll
    for (int t = 0; t < RT_MAX_T; ++t)
      if (t < nt) part[((size_t)rs * T + t0 + t) * E + e] = pv[t];
  }
}

__global__ void __launch_bounds__(256) router_reduce_kernel(const float* __restrict__ part,
                                                            int RS, int T, int E,
                                                            float* __restrict__ logits) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n = (size_t)T * E;
  if (i >= n) return;
  // all loads of a group of 16 splits in flight together; sums in ascending split order
  float s = 0.0f;
  for (int r0 = 0; r0 < RS; r0 += 16) {
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = (r0 + q < RS) ? part[(size_t)(r0 + q) * n + i] : 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (r0 + q < RS) s += v[q];
  }
  logits[i] = s;
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
  const size_t nq = (size_t)(K / fmt_kb(FMT)) * (N / 4);
  if (idx >= nq) return;
  const int r = (int)(idx / (N / 4));
  const int n = (int)(idx % (N / 4)) * 4;
  const uint32_t d = *reinterpret_cast<const uint32_t*>(w + (size_t)r * N + n);
  float lo[4], hi[4];
  if constexpr (FMT == FMT_FP8) {  // one code per byte: row r is K index r
    const f32x2_t p0 = fp8_pair_f32<0>(d), p1 = fp8_pair_f32<1>(d);
    const float v[4] = {p0.x, p0.y, p1.x, p1.y};
#pragma unroll
    for (int b = 0; b < 4; ++b)
      out[(size_t)r * N + n + b] = v[b] * bf16_to_f32(s[(size_t)(r / group) * N + n + b]);
    return;
  } else if constexpr (FMT == FMT_FP4) {
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
// =====================================================================================
// measurement aid: a plain streaming read (achievable HBM read bandwidth).  Each workgroup
// reads one contiguous 64 KiB chunk with 16-byte non-temporal loads, 8 in flight per thread
// (measured on MI355X: 6.1-6.2 TB/s over 2 GiB; grid-strided reads of the same bytes were
// 5-10 % slower).  The loaded words are folded with xor and written to sink only when the
// result equals `key`, so no load can be dropped.
// =====================================================================================
constexpr int SR_THREADS = 256;
constexpr int SR_CHUNK16 = 4096;  // 16-byte words per workgroup (64 KiB)
constexpr int SR_UNROLL = 8;
__global__ void __launch_bounds__(SR_THREADS) stream_read_kernel(const uint4* __restrict__ p,
                                                                 size_t n16, uint32_t key,
                                                                 uint32_t* sink) {
  const size_t b = (size_t)blockIdx.x * SR_CHUNK16;
  uint32_t acc = 0;
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  for (int i = threadIdx.x; i < SR_CHUNK16; i += SR_THREADS * SR_UNROLL) {
    u4 v[SR_UNROLL];
#pragma unroll
    for (int j = 0; j < SR_UNROLL; ++j) {
      const size_t idx = b + i + (size_t)j * SR_THREADS;
      v[j] = idx < n16 ? __builtin_nontemporal_load(reinterpret_cast<const u4*>(p + idx))
                       : u4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < SR_UNROLL; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == key) sink[0] = acc;
}

hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)((n16 + SR_CHUNK16 - 1) / SR_CHUNK16);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(SR_THREADS), 0, st,
                     static_cast<const uint4*>(p), n16, 0x9E3779B9u, sink);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* wts,
                       hipStream_t st) {
  const int grid = (T + 3) / 4;
  hipLaunchKernelGGL(topk_kernel, dim3(grid), dim3(256), 0, st, logits, T, E, k, ids, wts);
  return hipGetLastError();
}

// Calls with at least this many tokens route in topk_kernel (one wavefront per token across
// the GPU) before the schedule kernel, which then takes the ids as given: the schedule's 16
// routing waves on one compute unit take about 0.09 us per token (1.9 us at T = 16, 6.1 us at
// T = 64), the extra launch about 1.3 us more than that at T = 16 (measured: Q30 T = 64
// 104.0 -> 101.1 us, T = 16 60.7 -> 62.0 us with the split).
constexpr int SCHED_SPLIT_ROUTE_T = 32;

hipError_t launch_schedule(const MoeArgs& a, const float* logits, hipStream_t st) {
  if (logits && a.T >= SCHED_SPLIT_ROUTE_T) {  // the layer call routes into ids_w / wts_w
    hipError_t e = launch_topk(logits, a.T, a.E, a.k, a.ids_w, a.wts_w, st);
    if (e != hipSuccess) return e;
    logits = nullptr;  // a.ids is a.ids_w on this path
  }
  const size_t sm = (size_t)sched_int_words(a.E) * sizeof(int) +
                    (size_t)sched_route_waves(a.E) * sched_scratch_entries(a.E) * 8;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(SCHED_THREADS), sm, st, a, logits);
  return hipGetLastError();
}

int router_splits(int H) { return (H + RT_ROWS - 1) / RT_ROWS; }

hipError_t launch_router(const uint16_t* x, int T, int H, const uint16_t* wr, int E, float* part,
                         float* logits, hipStream_t st) {
  const int RS = router_splits(H);
  const dim3 grid(RS, (E + 127) / 128, (T + RT_MAX_T - 1) / RT_MAX_T);
  hipLaunchKernelGGL(router_partial_kernel, grid, dim3(256), 0, st, x, T, H, wr, E, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = (size_t)T * E;
  hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     part, RS, T, E, logits);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* w, const uint16_t* s, int K, int N, int group, int fmt,
                          float* out, hipStream_t st) {
  const size_t nq = (size_t)(K / fmt_kb(fmt)) * (N / 4);
  const int grid = (int)((nq + 255) / 256);
  if (fmt == FMT_FP8)
    hipLaunchKernelGGL(dequant_kernel<FMT_FP8>, dim3(grid), dim3(256), 0, st, w, s, K, N, group,
                       out);
  else if (fmt == FMT_FP4)
    hipLaunchKernelGGL(dequant_kernel<FMT_FP4>, dim3(grid), dim3(256), 0, st, w, s, K, N, group,
                       out);
  else
    hipLaunchKernelGGL(dequant_kernel<FMT_INT4>, dim3(grid), dim3(256), 0, st, w, s, K, N, group,
                       out);
  return hipGetLastError();
}

}  // namespace dqg
