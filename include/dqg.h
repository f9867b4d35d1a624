/*
 * dqg.h -- packed 4-bit dequant-in-register MoE FFN and dense GEMV for decode on
 * AMD Instinct MI355X (gfx950).  C linkage, plain pointers and sizes.
 *
 * Every pointer argument is a caller-owned DEVICE pointer unless stated otherwise.
 * bf16 values travel as uint16_t bit patterns.  All compute calls are asynchronous on
 * `stream`: they never synchronize, never allocate and never read device memory from
 * the host, so they can be captured into a hipGraph.  The caller keeps every buffer
 * alive until the stream work has completed.  The library owns no device memory and
 * keeps no state between calls (reentrant), except that concurrent calls must not
 * share one workspace -- and except the one allocation-free entry point,
 * packed_gemv_int4_noalloc, whose scratch array the library holds per GPU.
 *
 * Argument checks happen on the host before any launch; a failed check returns a
 * negative status and launches nothing.  A launch failure is reported as DQG_ERR_HIP
 * (read with hipGetLastError, no synchronization).
 *
 * Storage formats (FireEcho page, section "The Goliath Kernel: Why It's Fast": all
 * experts of a layer in one contiguous [E, K//2, N] buffer whose bytes are split into
 * a low nibble, taken first, and a high nibble, each dequantized with a scale inside
 * the matmul loop):
 *   packed weights  uint8 [E, K/2, N]: byte [e, r, n] holds K index 2r in bits 0-3 and
 *                   K index 2r+1 in bits 4-7; N is the contiguous axis.
 *   group scales    bf16  [E, K/G, N]: one scale per G consecutive K and per column.
 *   element value   DQG_FMT_INT4:     nibble - 8            (symmetric INT4)
 *                   DQG_FMT_FP4_E2M1: OCP MX E2M1 (sign bit, 2-bit exponent with bias 1,
 *                                     1-bit mantissa: magnitudes 0 .5 1 1.5 2 3 4 6)
 *   weight          W[k, n] = value(nibble) * scale[k / G, n]   (exact in fp32)
 * Shapes: K even, K % G == 0, N % 16 == 0, G in {32, 128}; base pointers of packed
 * weights, scales, x, residual and out 16-byte aligned.  Anything else returns
 * DQG_ERR_UNSUPPORTED or DQG_ERR_MISALIGNED so that the caller can keep another path.
 */
#ifndef DQG_H
#define DQG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DQG_ABI_VERSION 2

typedef enum dqg_status {
  DQG_OK = 0,
  DQG_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, k > E, ...        */
  DQG_ERR_UNSUPPORTED = -2, /* shape/format outside what the kernels implement     */
  DQG_ERR_MISALIGNED = -3,  /* a base pointer is not 16-byte aligned               */
  DQG_ERR_WORKSPACE = -4,   /* workspace null or smaller than the query returns    */
  DQG_ERR_HIP = -5          /* a kernel launch failed                              */
} dqg_status;

typedef enum dqg_format {
  DQG_FMT_INT4 = 0,     /* value = nibble - 8                                           */
  DQG_FMT_FP4_E2M1 = 1, /* value = E2M1(nibble)                                         */
  DQG_FMT_FP8_E4M3 = 2, /* value = E4M3(byte), one byte per weight: packed matrices are
                           [K, N] instead of [K/2, N]; the MoE layer calls only
                           (see moe_fp4_layer)                                           */
  DQG_FMT_INT2 = 3,     /* value = code - 2, four codes per byte: only as an entry of the
                           per-expert table of moe_fp4_layer_mixed                       */
  DQG_FMT_FEXC = 4      /* FE-XC 2x8 codebook codes: only as an entry of that table       */
} dqg_format;

/* Path flags, OR-ed into the `format` argument of the MoE calls (testing aid; the
 * default, 0, picks the path from the shapes).  FORCE_GEMV runs every expert on the
 * vector-ALU tiles, FORCE_MFMA runs every expert with at least one token on the bf16
 * matrix-core tiles, NO_FUSED disables the single-launch layer (T <= 8). */
#define DQG_PATH_FORCE_GEMV 0x100
#define DQG_PATH_FORCE_MFMA 0x200
#define DQG_PATH_NO_FUSED 0x400

/* Version of this ABI (DQG_ABI_VERSION).  Host only. */
int dqg_abi_version(void);

/* Human-readable name of a status code.  Host only; never fails. */
const char* dqg_status_string(int status);

/*
 * topk_route -- expert selection for T tokens (FireEcho page, "The Goliath Kernel":
 * expert IDs live in a GPU tensor and are read by the expert kernel with no host
 * synchronization).
 *   logits  fp32 [T, E], finite values (NaN/inf give unspecified ids)
 *   ids     int32 [T, k] out: the k largest logits of each row in rank order; equal
 *           logits (including -0.0 vs +0.0) rank the lower expert index first
 *   weights fp32 [T, k] out: softmax over the k selected logits (the top logit is
 *           subtracted before exponentiation), in the same order as ids
 * Requires 1 <= k <= E, 1 <= E <= 4096, k <= 32, T >= 1.
 */
int topk_route(const float* logits, int T, int E, int k, int32_t* ids, float* weights,
               hipStream_t stream);

/*
 * Bytes of device workspace that moe_fp4_ffn / moe_fp4_layer / moe_fp4_layer_from_hidden
 * need for T tokens with these sizes.  Host only.  Returns 0 for invalid sizes.
 * The workspace holds a sticky int32 error word at byte 0 (bit 0: an expert id outside
 * [0, E) was seen -- the slot then contributes zero; bit 1: a wait between workgroups gave
 * up -- the output of that call is not valid), the device-built expert schedule, and
 * exchange buffers that must hold zeros between calls.  Zero-fill a workspace once before
 * its first use; every completed call leaves it ready for the next -- except a call that set
 * bit 1: a late producer may then leave a published value behind, so zero-fill the whole
 * workspace again before reusing it.  Its layout depends only on (H, I, E, k) and its size
 * (the size grows with T), so one workspace serves calls with any T up to the T it was sized
 * for.  Calls that may run at the same time must not share a workspace.  Only the caller
 * clears the error word.
 */
size_t moe_fp4_ffn_workspace_bytes(int T, int H, int I, int E, int k);

/*
 * moe_fp4_ffn -- packed-MoE expert FFN with the top-k weighted combine, for a given
 * routing (FireEcho page: "The Goliath Kernel" -- dequant of both nibbles times the
 * scale in registers inside the tile loop; "Speed Optimization History" -- fused
 * gate_up projection, one multi-expert kernel over a contiguous packed buffer;
 * FastInfer page, "Confirmed elementwise SwiGLU scheduling" -- SiLU(gate) * up).
 *
 *   x          bf16 [T, H] tokens
 *   ids        int32 [T, k] expert of each slot (device, read by the kernels)
 *   weights    fp32 [T, k] combine weight of each slot
 *   w_gate_up  uint8 [E, H/2, 2I], s_gate_up bf16 [E, H/G, 2I]; columns [0, I) are the
 *              gate projection, [I, 2I) the up projection
 *   w_down     uint8 [E, I/2, H],  s_down    bf16 [E, I/G, H]
 *              (DQG_FMT_FP8_E4M3: [E, H, 2I] and [E, I, H], one code per byte)
 *   group      G (32 or 128), format DQG_FMT_INT4, DQG_FMT_FP4_E2M1 or DQG_FMT_FP8_E4M3,
 *              optionally OR-ed with DQG_PATH_* flags
 *   residual   bf16 [T, H] or NULL
 *   out        bf16 [T, H]:
 *     out[t] = bf16_rne( residual[t] + sum_{j<k} weights[t,j] * y_{t,j} ), j ascending,
 *     y_{t,j} = (SiLU(g) * u) W_down[e],  [g | u] = x[t] W_gate_up[e],  e = ids[t,j],
 *   accumulated in fp32.
 * Each expert's weights are streamed once per call for up to 16 of its tokens (the
 * matrix-core tiles) or 4 (the vector-ALU tiles); experts with >= 2 tokens run on bf16
 * (FP4, FP8) or fp16 (INT4) MFMA tiles, single-token experts on vector-ALU dot2 tiles, in
 * one launch per projection.  h = SiLU(g) * u enters the down projection as a 16-bit operand, bf16
 * (FP4, FP8) or fp16 (INT4), on the multi-launch path, and in fp32 on the single-launch layer
 * (moe_fp4_layer, T <= 8).
 * Results are deterministic (fixed reduction order, no floating-point atomics).
 * Requires H % 64 == 0, I % 64 == 0, H and I multiples of G, 1 <= k <= min(E, 32),
 * E <= 4096, T*k <= 65536.  out may not alias x or residual.  With DQG_FMT_INT4 the
 * activations must satisfy |x| < 65504 (INT4 tiles multiply in fp16, accumulate in fp32;
 * bf16 values convert to fp16 exactly above 2^-14 and within 2^-25 below), and on the
 * multi-launch path (T > 8, or DQG_PATH_NO_FUSED) h = SiLU(g) * u enters the down
 * projection as fp16, so |h| must stay below 65504 too (larger values become inf).
 */
int moe_fp4_ffn(const uint16_t* x, int T, int H, int I, int E, int k, const int32_t* ids,
                const float* weights, const uint8_t* w_gate_up, const uint16_t* s_gate_up,
                const uint8_t* w_down, const uint16_t* s_down, int group, int format,
                const uint16_t* residual, uint16_t* out, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * moe_fp4_layer -- topk_route followed by moe_fp4_ffn in one call (routing computed on
 * the device from `logits` fp32 [T, E]; same rules as topk_route).  For T <= 8 the
 * whole layer runs as a single kernel launch when E <= 512, H % 256 == 0, H <= 2048,
 * I % 128 == 0 and (for T > 1) k * I / 2 is a multiple of 256; every slot then streams its
 * expert itself (an expert chosen by several tokens is read once per token).  Other calls
 * route inside the schedule of the multi-launch path.  ids_out (int32 [T, k]) and
 * weights_out (fp32 [T, k]) are optional outputs of the routing (NULL to skip).
 * DQG_FMT_FP8_E4M3 (FireEcho page, "Quantization Formats": an 8-bit FP format; read as OCP
 * E4M3) takes w_gate_up uint8 [E, H, 2I] and w_down uint8 [E, I, H], one code per byte, with
 * the same scales, on both paths and in moe_fp4_ffn and moe_fp4_layer_from_hidden alike
 * (H * I at most 2^30, else DQG_ERR_UNSUPPORTED).  E4M3 codes S.1111.111 (NaN) give
 * unspecified results.
 */
int moe_fp4_layer(const uint16_t* x, const float* logits, int T, int H, int I, int E, int k,
                  const uint8_t* w_gate_up, const uint16_t* s_gate_up, const uint8_t* w_down,
                  const uint16_t* s_down, int group, int format, const uint16_t* residual,
                  uint16_t* out, int32_t* ids_out, float* weights_out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/*
 * moe_fp4_layer_mixed -- moe_fp4_layer for a layer whose experts mix FP4 (hot), FE-XC and
 * INT2 (cold) weights (FireEcho page, "Quantization Formats": FP4 for hot experts, the 2-bit
 * FE-XC codebook format and a scalar 2-bit INT2 format for the cold ones).
 *   expert_formats  uint8 [E] on the device, 4-byte aligned, E % 4 == 0: DQG_FMT_INT2 marks
 *                   an INT2 expert, DQG_FMT_FEXC an FE-XC expert; any other value means FP4
 *                   (format must be DQG_FMT_FP4_E2M1)
 *   codebooks       bf16 [E, 2, 2, 256, 8] (16-byte aligned) or NULL: per expert, for gate_up
 *                   then down, two codebooks of 256 vectors of 8.  An FE-XC expert's codes fill the
 *                   first quarter-K rows of its slab as [K/8, 2, N] bytes (codebook m's code of
 *                   the group of K indices 8g .. 8g+7 in byte row 2g + m); its weights are
 *                   (C[0][c0] + C[1][c1])[i] * scale.  Without codebooks an FE-XC entry reads
 *                   its slab as FP4.
 *   w_gate_up, w_down  as for FP4, every expert at its FP4 slab offset; an INT2 expert's codes
 *                   fill the first quarter-K rows of its slab: [H/4, 2I] and [I/4, H] bytes,
 *                   K index 4r + i in bits 2i .. 2i+1 of byte row r (code c means c - 2); the
 *                   scales keep their layout.  INT2 experts stream half the bytes.
 * Runs as one launch where moe_fp4_layer would (with codebooks also I >= 512: a down unit's
 * 256 rows then span at most two experts, whose codebooks it stages), otherwise on the
 * multi-launch kernels, where INT2 and FE-XC experts take 2-bit tiles of their own: INT2
 * codes decode to c / 2 (the scale doubled, -sum(x) per block added), FE-XC vectors meet
 * the operands as they are, one product per codebook; both on the vector-ALU or the
 * matrix-core body by token count, as FP4 experts (DQG_PATH_* flags apply).  Other
 * arguments and rules as moe_fp4_layer.
 */
int moe_fp4_layer_mixed(const uint16_t* x, const float* logits, int T, int H, int I, int E,
                        int k, const uint8_t* w_gate_up, const uint16_t* s_gate_up,
                        const uint8_t* w_down, const uint16_t* s_down,
                        const uint8_t* expert_formats, const uint16_t* codebooks, int group,
                        int format, const uint16_t* residual, uint16_t* out, int32_t* ids_out,
                        float* weights_out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Bytes of device workspace router_logits needs (the router's fp32 partial rows, 4 bytes x
 * ceil(H / 128) x T x E).  Host only.  Returns 0 for unsupported sizes (H or E not a
 * multiple of 8, E > 4096).
 */
size_t router_logits_workspace_bytes(int T, int H, int E);

/*
 * router_logits -- the MoE router on the hidden state (FireEcho page, "Architecture": the
 * packed MoE FFN dispatches from the hidden state; read as the plain linear router, no bias).
 *   x        bf16 [T, H];  w_router bf16 [H, E] (E contiguous)
 *   logits   fp32 [T, E] out: logits[t, e] = sum_c x[t, c] * w_router[c, e]
 * fp32 accumulation in a fixed order: 128-row partials (each an ordered fma chain over 8
 * rows per lane, then 16 lanes summed in order) added in ascending row order from +0.0 --
 * the same arithmetic as the router inside moe_fp4_layer_from_hidden, so both give
 * bitwise-identical logits.  Needs H % 8 == 0, E % 8 == 0, E <= 4096, x and w_router
 * 16-byte aligned, and a workspace of router_logits_workspace_bytes (scratch, no state
 * kept between calls).  Two launches on `stream`.  Deterministic.
 */
int router_logits(const uint16_t* x, int T, int H, int E, const uint16_t* w_router,
                  float* logits, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_fp4_layer_from_hidden -- router_logits followed by moe_fp4_layer, the routing taken
 * from the hidden state x itself.  Same arguments and rules as moe_fp4_layer, with
 * w_router bf16 [H, E] in place of logits (E % 8 == 0), the same workspace (size query
 * moe_fp4_ffn_workspace_bytes), and logits_out (fp32 [T, E], nullable) an optional copy of
 * the router's logits.  When the single-launch layer applies (see moe_fp4_layer) and
 * E <= 128 and T <= 4, the router runs inside that launch: its first ceil(H / 128) workgroups compute
 * 128-row partials of the logits and every other workgroup adds them up before its
 * top-k, so the layer stays one launch.  Otherwise the router call runs first.  The
 * logits, and so the routing, are bitwise identical on both paths.
 */
int moe_fp4_layer_from_hidden(const uint16_t* x, const uint16_t* w_router, int T, int H, int I,
                              int E, int k, const uint8_t* w_gate_up, const uint16_t* s_gate_up,
                              const uint8_t* w_down, const uint16_t* s_down, int group,
                              int format, const uint16_t* residual, uint16_t* out,
                              float* logits_out, int32_t* ids_out, float* weights_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace packed_gemv_int4 needs for T tokens (0: the call never splits
 * K and needs none).  Host only.  Returns 0 also for invalid sizes.
 */
size_t packed_gemv_int4_workspace_bytes(int T, int K, int N, int group);

/*
 * packed_gemv_int4 -- dense packed INT4 GEMV (FastInfer page, "Specialized
 * matrix-vector result": a token vector times a stored weight, FP32 products and
 * reductions; eole page, "Packed Marlin projections": gate and up packed into one
 * projection for 1-token and 4-token decode).
 *   x  bf16 [T, K];  w uint8 [K/2, N];  s bf16 [K/G, N];  y bf16 [T, N] out
 *   y[t, n] = bf16_rne( sum_k x[t,k] * (nibble[k,n] - 8) * s[k/G, n] ), fp32 accumulation.
 * x must satisfy |x| < 65504 (the INT4 tiles multiply in fp16 with fp32 accumulation;
 * bf16 values convert to fp16 exactly above 2^-14 and within 2^-25 below).  T = 1 runs on
 * vector-ALU dot2 tiles, T >= 2 on fp16 MFMA tiles (T <= 4: each weight decoded once for
 * all tokens).  When the query returns a non-zero size the call splits K
 * across workgroups: pass a workspace of at least that many bytes, zero-filled before its
 * first use; every completed call leaves it zero-filled again, and one workspace serves
 * calls with any T up to the T it was sized for.  Its first int32 is an error word (bit 1:
 * a wait between workgroups gave up; the output is then not valid and a late producer may
 * leave a partial behind: zero-fill the workspace again before reusing it).  With a NULL
 * workspace the call runs without the K
 * split (correct, fewer workgroups).  Deterministic.  Calls that may run at the same time
 * must not share a workspace.
 */
int packed_gemv_int4(const uint16_t* x, int T, int K, int N, const uint8_t* w,
                     const uint16_t* s, int group, uint16_t* y, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * packed_gemv_int4_noalloc -- packed_gemv_int4 for callers that cannot allocate device memory
 * or pass a workspace (code under hipGraph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, arithmetic, kernels and results as packed_gemv_int4 with a
 * workspace sized for T (bitwise identical outputs), except that the K-split partials live in
 * a library-owned device array of 16 MiB + 256 bytes per GPU, held until the process ends.
 * The call allocates nothing.  status: NULL, or a device int32 into which a call ORs bit 1
 * when a wait between workgroups gave up (the output is then not valid; the caller clears
 * it).  Calls whose partials (K splits x T x N x 4 bytes) exceed 16 MiB return
 * DQG_ERR_WORKSPACE before any launch.  Calls that may overlap on one GPU (different
 * streams, or another thread) race on that array and must not; stream must belong to the
 * current device.  Every completed call leaves the array's partials zero; after a status bit
 * 1 that no longer holds for the rest of the process.
 */
int packed_gemv_int4_noalloc(const uint16_t* x, int T, int K, int N, const uint8_t* w,
                             const uint16_t* s, int group, uint16_t* y, int* status,
                             hipStream_t stream);

/*
 * Prepacked dense GEMV (eole page, "Packed Marlin projections": projection weights are
 * rearranged once while the model is prepared for inference, ahead of the decode kernels
 * that read them).  The same INT4 weights and scales as packed_gemv_int4, stored so that
 * every workgroup of the GEMV streams one contiguous stretch of memory:
 *   w_tiled uint8: blocks of 2048 bytes, block (t, b) = byte rows 16 b .. 16 b + 15 (32 K)
 *     of column tile t (columns 128 t .. 128 t + 127; the last tile padded with zero bytes).
 *     Inside a block, 128 units of 16 bytes, unit u = 64 h + l (h = 0, 1; l = 0 .. 63,
 *     q = l % 16, kq = l / 16) hold byte rows r = 16 b + 4 kq + 2 h and r + 1 of columns
 *     c = 128 t + 8 q .. +7: bytes 4 m .. 4 m + 3 (m = 0 .. 3) are (r, c + 2 m),
 *     (r, c + 2 m + 1), (r + 1, c + 2 m), (r + 1, c + 2 m + 1).  Blocks are ordered by step
 *     i = b / 16, then tile, then b: with n_i = min(16, K/32 - 16 i) blocks in step i, block
 *     (t, b) starts at byte 2048 (16 i tiles + t n_i + b - 16 i).  tiles = ceil(N / 128);
 *     K * 64 bytes per tile in all.
 *   s_tiled bf16 [K/G][tiles * 128]: s_tiled[g][c] = s[g][c] (0 for c >= N).
 * The rearrangement is a permutation plus zero padding: the GEMV reads exactly the bytes of
 * the [K/2, N] layout (plus the padding of a ragged last tile).
 */

/* Host only: bytes of the prepacked weights and scales for a [K/2, N] INT4 matrix with group
 * G.  Sizes as for packed_gemv_int4 (T = 1); DQG_ERR_UNSUPPORTED otherwise. */
int packed_gemv_int4_prepack_sizes(int K, int N, int group, size_t* w_bytes, size_t* s_bytes);

/*
 * packed_gemv_int4_prepack -- rearranges w uint8 [K/2, N] and s bf16 [K/G, N] into w_tiled
 * and s_tiled (sizes from packed_gemv_int4_prepack_sizes; every byte of both is written).
 * Asynchronous on `stream`; the inputs are only read.  All four pointers 16-byte aligned.
 */
int packed_gemv_int4_prepack(const uint8_t* w, const uint16_t* s, int K, int N, int group,
                             uint8_t* w_tiled, uint16_t* s_tiled, hipStream_t stream);

/*
 * packed_gemv_int4_tiled -- the dense packed INT4 GEMV of packed_gemv_int4 (same
 * y[t, n] = bf16_rne( sum_k x[t,k] * (nibble[k,n] - 8) * s[k/G, n] ), fp32 accumulation,
 * same bounds on x) on the prepacked weights, for 1 <= T <= 4 tokens: one token on
 * vector-ALU dot2 tiles, 2 to 4 on fp16 matrix-core tiles with fp32 accumulation (more return
 * DQG_ERR_UNSUPPORTED; so do prepacked weights of 2 GiB or more, ceil(N/128) K 64 bytes, which
 * the kernel addresses with 32-bit offsets).  x bf16 [T, K], y bf16 [T, N].  All pointers
 * 16-byte aligned.  The workspace is that of packed_gemv_int4 for T tokens (size from
 * packed_gemv_int4_workspace_bytes, the same contract: zero-filled before first use, left
 * zero-filled by every completed call, error word bit 1 when a wait between workgroups gave
 * up, NULL for no K split); one workspace may serve both calls.  Deterministic, and the arithmetic and summation order
 * are those of packed_gemv_int4 for the same T: the two calls give bitwise identical results.
 * Calls that may run at the same time must not share a workspace.
 */
int packed_gemv_int4_tiled(const uint16_t* x, int T, int K, int N, const uint8_t* w_tiled,
                           const uint16_t* s_tiled, int group, uint16_t* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * packed_dequant_f32 -- TEST AID: dequantize one packed matrix with the same in-register
 * decode the compute kernels use.  w uint8 [K/2, N] (FP8: [K, N]), s bf16 [K/G, N] -> out
 * fp32 [K, N], out[k, n] = value(code[k, n]) * s[k/G, n], exact.
 */
int packed_dequant_f32(const uint8_t* w, const uint16_t* s, int K, int N, int group,
                       int format, float* out, hipStream_t stream);

/*
 * dqg_stream_read -- MEASUREMENT AID: read `bytes` (a multiple of 16) at p (16-byte aligned)
 * once with 16-byte non-temporal loads, one contiguous 64 KiB chunk per workgroup, to
 * calibrate the achievable HBM read bandwidth against which the compute kernels are judged.
 * sink: a device uint32 that the kernel may write (the xor of the data is stored only when it
 * equals a fixed key, so that no load can be optimized away).
 */
int dqg_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DQG_H */
