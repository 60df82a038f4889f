/*
 * rf.h -- C ABI of a small MI355X (gfx950) library that computes chains of
 * dependent reductions ("cascaded reductions") in one pass with a running,
 * rescaled state.
 *
 * The operations follow the statement of the problem on the source pages:
 *   - attention: scores Q K^T, safe softmax, product with V, computed with a
 *     running max m, a running denominator l and an accumulator rescaled by
 *     exp(m_old - m_new), divided by l once at the end
 *     ("RedFuser episode transcript", cues 9, 15, 17 and 19);
 *   - split-KV decode: the key sequence is split into segments whose partial
 *     states (m, l, acc) are merged by rescaling to a common max
 *     (transcript cues 21 and 39; "RedFuser episode visual explainer",
 *     widgets "Merging partial states across blocks (FlashDecoding-style)"
 *     and "Single-Segment vs Multi-Segment");
 *   - the same split over a shared latent cache (multi-latent attention,
 *     transcript cues 41 and 55);
 *   - MoE routing: softmax followed by top-k (transcript cue 11;
 *     "Online normalizer calculation for softmax", abstract);
 *   - safe softmax alone, fused at the thread, wave or workgroup level of the
 *     reduction tree (transcript cue 47);
 *   - variance and moment of inertia: a centre, then the centred second
 *     moment, at the same fusion levels (transcript cue 47);
 *   - FP8: per-token abs-max, scale, e4m3 cast, then GEMM (transcript cue 33).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers on the current HIP device, row-major
 *     and contiguous, 16-byte aligned unless stated otherwise. The caller
 *     allocates and owns every buffer (including workspaces); the library
 *     allocates nothing. The only state kept between calls is a per-device
 *     cache of the compute-unit count (read once, used to pick a launch
 *     shape).
 *   - Outputs must not alias inputs.
 *   - Calls only enqueue work on `stream` (0 = the null stream) and return.
 *     All arguments are validated before anything is enqueued, so a call that
 *     returns RF_ERR_INVALID_ARG or RF_ERR_UNSUPPORTED has launched nothing.
 *     RF_ERR_LAUNCH means the HIP runtime refused a launch; the calls that
 *     enqueue more than one kernel (rf_absmax_quant_gemm_fp8: quantiser,
 *     then GEMM; rf_softmax level 0: three row passes) stop at the refused
 *     one, and the kernels enqueued before it stay enqueued. Kernel faults
 *     surface at the caller's next synchronisation, as with any HIP launch.
 *   - A call whose output is empty (a zero batch or row count) returns RF_OK
 *     and enqueues nothing; null pointers are accepted only then.
 *   - Calls are re-entrant; rf_last_error() is per host thread.
 *   - A call enqueues kernels only (no allocation, memset, copy or host
 *     synchronisation), so it can be recorded into a HIP graph by stream
 *     capture and replayed; a replay reads the buffers' contents at that time.
 *   - Inputs are expected finite; a NaN propagates to the rows it touches.
 */
#ifndef RF_H_
#define RF_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RF_ABI_VERSION 8

typedef enum {
  RF_OK = 0,
  RF_ERR_INVALID_ARG = 1, /* null pointer, misalignment, negative size, inconsistent shape */
  RF_ERR_UNSUPPORTED = 2, /* valid request this build has no kernel for (dtype, head size, k, K) */
  RF_ERR_LAUNCH = 3,      /* the HIP runtime refused a launch; detail in rf_last_error() */
  RF_STATUS_MAX_ENUM_ = 0x7fffffff /* not a status: makes every non-negative int a valid value */
} rf_status;

/* Element type. Any non-negative int may be passed; others than the two named
 * here are rejected with RF_ERR_INVALID_ARG. */
typedef enum { RF_F32 = 0, RF_BF16 = 1, RF_DTYPE_MAX_ENUM_ = 0x7fffffff } rf_dtype;

/*
 * rf_attn_fwd -- O = softmax(scale * Q K^T [+ causal mask]) V, one pass over
 * K/V tiles with running (m, l, acc) per query row (transcript cues 15-19).
 *
 *   dt     RF_BF16: q, k, v, o are bf16, math in fp32 (MFMA for both
 *          contractions), d in {64, 128} and one head's K (or V) under
 *          2 GiB (Lk * d * 2 < 2^31, else RF_ERR_UNSUPPORTED); RF_F32: all
 *          fp32 (FMA), d in {64, 128}.
 *   q      [B, Hq, Lq, d]      k, v  [B, Hkv, Lk, d]     o  [B, Hq, Lq, d] (dt)
 *   lse    [B, Hq, Lq] fp32 or NULL: m + ln(l) of the scaled scores.
 *   Hq % Hkv == 0; query head h reads key/value head h / (Hq / Hkv).
 *   causal != 0 masks key j for query i when j > i and needs Lq == Lk.
 *   Lk >= 1 whenever the output is non-empty. scale is explicit (no default)
 *   and may be any finite value, zero and negative included (a zero scale
 *   weights every unmasked key equally); a NaN or infinite scale returns
 *   RF_ERR_INVALID_ARG. The same holds for every scale argument below.
 */
rf_status rf_attn_fwd(rf_dtype dt, const void* q, const void* k, const void* v, void* o,
                      float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
                      int causal, hipStream_t stream);

/*
 * rf_attn_decode_split -- first half of split-KV decode (one query row per
 * head). Keys are split into S segments of ceil(Lk / S) keys (the last ones
 * may be shorter or empty); for every (b, query head, segment) it writes the
 * unnormalised partial state over that segment's keys:
 *   part_m   [B, Hq, S]     max of the scaled scores (-inf for an empty segment)
 *   part_l   [B, Hq, S]     sum of exp(score - part_m)          (0 if empty)
 *   part_acc [B, Hq, S, d]  sum of exp(score - part_m) * v      (0 if empty)
 * all fp32 (transcript cue 39: Multi-Segment; cue 21: the states merge).
 *
 *   dt     RF_BF16: q [B, Hq, d], k, v [B, Hkv, Lk, d] bf16, scores and
 *          P V on MFMA with fp32 accumulation; RF_F32: q, k, v fp32, all
 *          arithmetic fp32 (fp32 MFMA v_mfma_f32_16x16x4_f32: fp32 products
 *          and sums).
 *   d in {64, 128}; Hq % Hkv == 0 and Hq / Hkv <= 16; S >= 1; Lk >= 1; one
 *   head's K (or V) under 2 GiB (Lk * d * sizeof(element) < 2^31, else
 *   RF_ERR_UNSUPPORTED).
 */
rf_status rf_attn_decode_split(rf_dtype dt, const void* q, const void* k, const void* v,
                               float* part_m, float* part_l, float* part_acc, int B, int Hq,
                               int Hkv, int Lk, int d, int S, float scale, hipStream_t stream);

/*
 * rf_merge_states -- second half of split-KV decode: for each of `rows` rows,
 * merge S partial states by rescaling each to the common max m* and adding
 * (transcript cue 21): w_s = exp(m_s - m*) (0 for m_s = -inf),
 * l = sum w_s l_s, o = sum w_s acc_s / l, lse = m* + ln(l).
 * A row whose states are all empty gets o = 0 and lse = -inf.
 *
 *   part_m, part_l [rows, S] fp32; part_acc [rows, S, d] fp32;
 *   o [rows, d] in out_dt (RF_BF16 or RF_F32); lse [rows] fp32 or NULL.
 *   1 <= d <= 1024, d % 4 == 0.
 */
rf_status rf_merge_states(const float* part_m, const float* part_l, const float* part_acc,
                          int rows, int S, int d, rf_dtype out_dt, void* o, float* lse,
                          hipStream_t stream);

/*
 * rf_mla_decode_split -- split-KV decode over a shared latent cache
 * (multi-latent attention: transcript cues 41 and 55 name the multi-latent
 * decode workload; the split and the partial states are those of
 * rf_attn_decode_split, cues 21 and 39). Every key is one latent row; the
 * score of query head h is scale * q_h . row over all Dqk columns, its value
 * is the row's first Dv columns, and all H heads of a sequence share the rows.
 * Writes the same unnormalised partial states as rf_attn_decode_split, to be
 * merged by rf_merge_states with d = Dv.
 *
 *   q        [B, H, Dqk] bf16
 *   kv       [B, Lk, Dqk] bf16 (latent rows)
 *   part_m, part_l [B, H, S] fp32;  part_acc [B, H, S, Dv] fp32 (16-byte aligned)
 *   Dqk == 576 and Dv == 512 (else RF_ERR_UNSUPPORTED); H a multiple of 16, at
 *   most 128 (each group of 16 heads streams the cache once); segments of
 *   ceil(Lk / S) keys, empty ones written as the identity (-inf, 0, 0).
 */
rf_status rf_mla_decode_split(const void* q, const void* kv, float* part_m, float* part_l,
                              float* part_acc, int B, int H, int Lk, int Dqk, int Dv, int S,
                              float scale, hipStream_t stream);

/*
 * rf_mla_decode -- rf_mla_decode_split and the merge of its S partial states
 * (the rule of rf_merge_states, transcript cue 21) in one launch: each
 * workgroup writes its partial state as rf_mla_decode_split does, makes it
 * visible device-wide and counts itself in on its (sequence, head group)'s
 * counter; the workgroup that completes the count merges that group's S
 * states, writes O and lse, and sets the counter back to 0.
 *
 *   q, kv, part_m, part_l, part_acc, B, H, Lk, Dqk, Dv, S, scale: as for
 *           rf_mla_decode_split (the partial states are written too).
 *   counters [B * H / 16] int32, caller-owned, 4-byte aligned: all 0 before
 *           the first call; every call that returns RF_OK and runs to
 *           completion leaves them 0. Calls that share a counters array must
 *           not run at the same time.
 *   o       [B, H, 512] in out_dt (RF_BF16 or RF_F32), 16-byte aligned;
 *   lse     [B, H] fp32 (natural log) or NULL.
 * Publishing a state across the 8 XCDs costs an L2 write-back per workgroup,
 * so on MI355X this measured slower than the two launches for S = 8 .. 32.
 */
rf_status rf_mla_decode(const void* q, const void* kv, float* part_m, float* part_l, float* part_acc,
                        int32_t* counters, rf_dtype out_dt, void* o, float* lse, int B, int H, int Lk,
                        int Dqk, int Dv, int S, float scale, hipStream_t stream);

/*
 * rf_softmax_topk -- MoE routing: per row of logits, softmax then top-k
 * (transcript cue 11; "Online normalizer calculation for softmax", abstract),
 * fused into one pass over the row.
 *
 *   logits  [T, E] fp32;  weights [T, k] fp32;  indices [T, k] int32.
 *   Experts are ranked by logit descending, equal logits by index ascending,
 *   and returned in that order. weights are the softmax probabilities of the
 *   selected experts, divided by their own sum when renormalize != 0.
 *   1 <= k <= min(E, 32); E <= 1024; E % 4 == 0.
 */
rf_status rf_softmax_topk(const float* logits, int T, int E, int k, int renormalize,
                          float* weights, int32_t* indices, hipStream_t stream);

/* Where rf_softmax, rf_row_variance and rf_row_inertia update their running
 * state in the reduction tree. */
enum {
  RF_FUSE_NONE = 0,   /* unfused cascade: max kernel, sum kernel, divide kernel */
  RF_FUSE_THREAD = 1, /* per value, in each thread; thread states merged after */
  RF_FUSE_WAVE = 2,   /* per 256-value wave segment; wave states merged after */
  RF_FUSE_BLOCK = 3   /* per 1024-value workgroup tile */
};

/*
 * rf_softmax -- safe softmax of each row, y_ij = exp(x_ij - m_i) / l_i with
 * m_i = max_j x_ij and l_i = sum_j exp(x_ij - m_i), with the max -> sum
 * cascade fused at the chosen level of the reduction tree (transcript cue 47:
 * fusion levels on safe softmax of 1K to 8K values; cue 17: the running state
 * rescaled by exp(m_old - m_new) when the max grows). Every fused level reads
 * x once; RF_FUSE_NONE reads it three times and keeps m and l in `work`.
 *
 *   x [T, E] fp32;  y [T, E] fp32;  4 <= E <= 8192, E % 4 == 0.
 *   work  [2 * T] fp32 caller-owned scratch, 4-byte aligned, used (and
 *         overwritten) only by RF_FUSE_NONE; may be NULL otherwise.
 *   Rows are expected to hold at least one finite value.
 */
rf_status rf_softmax(const float* x, int T, int E, int level, float* work, float* y,
                     hipStream_t stream);

/*
 * rf_row_variance -- per row, the mean mu_i = (1/E) sum_j x_ij and the
 * population variance (1/E) sum_j (x_ij - mu_i)^2 (transcript cue 47 names
 * the variance cascade: a mean, then the centred second moment). `level`
 * (RF_FUSE_*) is where the running state (count, mean, centred sum) is
 * updated; each step moves the mean and corrects the centred sum of the
 * earlier values by count * (mean_old - mean_new)^2 (cue 17: correct for the
 * changed earlier result, then add the tile's term). Fused levels read x once;
 * RF_FUSE_NONE runs a mean pass and a centred pass. Positions are summed
 * relative to each row's first value, so rows with a mean far above their
 * spread keep their digits.
 *
 *   x [T, E] fp32 (16-byte aligned);  mean [T], var [T] fp32.
 *   4 <= E <= 8192, E % 4 == 0. No workspace.
 */
rf_status rf_row_variance(const float* x, int T, int E, int level, float* mean, float* var,
                          hipStream_t stream);

/*
 * rf_row_inertia -- per row of point masses w_ij >= 0 at positions x_ij on a
 * line, the centre of mass c_i = sum_j w_ij x_ij / sum_j w_ij and the moment
 * of inertia about it, I_i = sum_j w_ij (x_ij - c_i)^2 (transcript cue 47
 * names the moment-of-inertia cascade). Fusion levels and the incremental step
 * as in rf_row_variance, with masses in place of counts. A row whose masses
 * sum to 0 gets centre NaN and inertia 0.
 *
 *   x, w [T, E] fp32 (16-byte aligned);  centre [T], inertia [T] fp32.
 *   4 <= E <= 8192, E % 4 == 0. No workspace.
 */
rf_status rf_row_inertia(const float* x, const float* w, int T, int E, int level, float* centre,
                         float* inertia, hipStream_t stream);

/*
 * rf_absmax_quant_fp8 -- per-row abs-max, scale and e4m3 cast (transcript
 * cue 33, first reduction): a_i = max_k |x_ik|, s_i = fp32(a_i / 448),
 * q_ik = e4m3(fp32(x_ik / s_i)), divisions correctly rounded, e4m3 = OCP
 * E4M3 (no infinities, largest 448) with round-to-nearest-even after clamping
 * the magnitude to 448. A row with a_i = 0 gets s_i = 0 and all codes 0.
 *
 *   x [rows, cols] bf16;  q [rows, cols] uint8 (e4m3 codes);  scale [rows] fp32.
 *   cols % 8 == 0 and cols <= 8192; q needs only 8-byte alignment.
 */
rf_status rf_absmax_quant_fp8(const void* x, int rows, int cols, uint8_t* q, float* scale,
                              hipStream_t stream);

/*
 * rf_absmax_quant_gemm_fp8 -- the FP8 cascade: quantise A per row exactly as
 * rf_absmax_quant_fp8 does, then C_ij = bf16(s_i * t_j * sum_k A_q[i,k] B_q[j,k])
 * with fp32 accumulation (transcript cue 33: abs-max, then the GEMM over the
 * scaled values).
 *
 *   a       [M, K] bf16
 *   b       [N, K] uint8 e4m3 codes (K contiguous; the K x N operand stored
 *           column by column), b_scale [N] fp32 (per output column)
 *   a_q     [M, K] uint8 workspace, written (caller-owned, 16-byte aligned)
 *   a_scale [M] fp32, written
 *   c       [M, N] bf16
 *   K % 128 == 0 and K <= 8192; M, N >= 0.
 */
rf_status rf_absmax_quant_gemm_fp8(const void* a, const uint8_t* b, const float* b_scale, int M,
                                   int N, int K, uint8_t* a_q, float* a_scale, void* c,
                                   hipStream_t stream);

/*
 * rf_absmax_quant_gemm_fp8_noalloc -- rf_absmax_quant_gemm_fp8 for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, hosts that forbid hipMalloc): the same two kernels, with the
 * quantised A held in a library-owned device array of RF_NOALLOC_SCRATCH_BYTES
 * (one copy per GPU, kept until the process ends) instead of a caller
 * workspace. The call allocates nothing; its first call on a device looks up
 * that device's copy of the array.
 *
 *   a, b, b_scale, a_scale, c, M, N, K as for rf_absmax_quant_gemm_fp8.
 *   M * K <= RF_NOALLOC_SCRATCH_BYTES, else RF_ERR_UNSUPPORTED.
 *   Every call on one GPU uses the same array: calls that can overlap on one
 *   GPU (other streams, other host threads) race and must be serialised by the
 *   caller. Each call writes every scratch byte it reads, so nothing has to be
 *   cleared between calls.
 */
#define RF_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
rf_status rf_absmax_quant_gemm_fp8_noalloc(const void* a, const uint8_t* b, const float* b_scale,
                                           int M, int N, int K, float* a_scale, void* c,
                                           hipStream_t stream);

/*
 * rf_absmax_quant_gemm_fp8_running -- the FP8 cascade as one pass with a running
 * per-row scale (transcript cue 33, the loop as stated there): no abs-max pass
 * over A first. K is walked in tiles of 64 columns; for tile t, row i's
 * running abs-max a_i rises to include the tile, s_i = fp32(a_i / 448), the
 * tile is quantised with that s_i exactly like rf_absmax_quant_fp8 quantises a
 * row (correctly rounded fp32 x / s_i, round-to-nearest-even e4m3; codes 0
 * while a_i = 0), and when s_i grew the running fp32 accumulator row is first
 * multiplied by s_old / s_new. At the end C_ij = bf16(s_i * t_j * acc_ij).
 * Early tiles are quantised with a smaller scale than the row's final one, so
 * C differs from rf_absmax_quant_gemm_fp8 by the quantisation of those tiles.
 *
 *   a       [M, K] bf16
 *   b       [N, K] uint8 e4m3 codes (K contiguous), b_scale [N] fp32
 *   a_scale [M] fp32, written: the final scale (equal to rf_absmax_quant_fp8's)
 *   c       [M, N] bf16
 *   K % 128 == 0 and K <= 8192; M, N >= 0. No workspace.
 */
rf_status rf_absmax_quant_gemm_fp8_running(const void* a, const uint8_t* b, const float* b_scale,
                                           int M, int N, int K, float* a_scale, void* c,
                                           hipStream_t stream);

/*
 * Measurement support (not a step of the path): the matrix-core rate this GPU
 * sustains and the shader clock it runs at, against which the MFMA-bound
 * kernels above are compared. The clock depends on the operand data (the
 * board's power limit lowers it as more bits switch), so the loop multiplies
 * data the caller supplies.
 *
 * rf_peak_mfma -- `blocks` workgroups of 4 waves; each lane loads 8 operand
 * vectors, then runs `iters` iterations of 8 MFMAs (operands j and (j+3) % 8)
 * onto 4 independent accumulators, with no memory traffic in the loop.
 *   kind RF_PEAK_BF16: v_mfma_f32_32x32x16_bf16, 32768 flops per wave-MFMA
 *   kind RF_PEAK_FP8:  v_mfma_f32_32x32x64_f8f6f4 on e4m3, 131072 flops
 *   flops per call = blocks * 4 * iters * 8 * (flops per wave-MFMA)
 *   src   [blocks * 256][256] bytes, 32-byte aligned: lane t of workgroup b
 *         reads row 256 b + t; operand j is at byte 32 j (bf16: 8 values in
 *         its first 16 bytes; fp8: 32 e4m3 codes)
 *   out   [blocks * 4] fp32, written: per wave, the sum of all its
 *         accumulator elements (a checksum of the products)
 *   clock [blocks * 2] uint64 or NULL: per workgroup, shader-clock cycles and
 *         constant-rate ticks from its start to its end (rf_wall_clock_khz
 *         gives the tick rate; cycles / ticks * rate = shader clock)
 *   1 <= blocks <= 65536, 1 <= iters <= 2^20.
 */
typedef enum { RF_PEAK_BF16 = 0, RF_PEAK_FP8 = 1 } rf_peak_kind;
rf_status rf_peak_mfma(int kind, const void* src, int blocks, int iters, float* out,
                       unsigned long long* clock, hipStream_t stream);

/*
 * rf_peak_read -- HBM read stream: `blocks` workgroups of 256 threads read
 * `bytes` of `src` once in 16-byte loads, workgroup b its own contiguous share,
 * eight independent loads in flight per thread. out[b] = XOR of the 32-bit
 * words workgroup b read, so the XOR over out is the XOR of every word of src
 * whatever the order.
 *   src 16-byte aligned, bytes % 16 == 0;  out [blocks] uint32;
 *   1 <= blocks <= 65536.
 */
rf_status rf_peak_read(const void* src, long long bytes, int blocks, uint32_t* out,
                       hipStream_t stream);

/* Rate of the constant-rate counter of the current device, in kHz. */
rf_status rf_wall_clock_khz(int* khz);

/* Human-readable name of a status code (static storage). */
const char* rf_status_string(rf_status s);

/* Detail of the last non-OK return on this host thread ("" if none). */
const char* rf_last_error(void);

/* RF_ABI_VERSION of the built library. */
int rf_abi_version(void);

/* Identity of the sources the library was built from: a hex digest of every
 * kernel source and header, this header and the compiler flags, fixed at build
 * time. A loader compares it with the digest of the sources it was shipped
 * with and refuses a library built from others. */
const char* rf_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* RF_H_ */
