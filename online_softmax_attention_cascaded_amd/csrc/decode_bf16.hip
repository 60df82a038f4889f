// Split-KV decode (Multi-Segment) and the merge of partial states.
//
// First kernel: one workgroup per (batch, key/value head, segment). It streams
// the segment's K and V rows once for the whole GQA group of query heads and
// keeps, per query head, a running max m, a running denominator l and an
// unnormalised accumulator, rescaled by exp(m_old - m_new) when the max grows
// ("RedFuser episode transcript", cues 19 and 39). The four waves take
// interleaved 32-key steps of the segment and their states are merged at the
// end the same way partial states are merged across segments (cue 21); the
// merged, still unnormalised state (m, l, acc) is written to memory.
//
// Second kernel: per query row, rescale the S partial states to the common max,
// add, divide by l once (cue 21; "RedFuser episode visual explainer", widget
// "Merging partial states across blocks (FlashDecoding-style)").
//
// Decode is bound by HBM bandwidth: every K/V byte is read exactly once per
// GQA group, and throughput is set by how many bytes each CU keeps in flight.
// Both contractions use v_mfma_f32_16x16x32_bf16 with the group's query heads
// in the N (or M) dimension, so bf16 K/V never need a VALU widening.
//  - K rows go straight from global memory into the A operand of S^T = K Q^T
//    (16-byte loads), two steps ahead of their use, in three register sets
//    whose roles rotate with a 3-way unrolled loop (no register copies, so no
//    wait on the newest loads).
//  - V rows are loaded one step ahead straight into a two-slot LDS ring per
//    wave (buffer loads to LDS, no registers), in their natural row-major
//    layout; the B operand of O = P V is read back transposed with
//    ds_read_b64_tr_b16, four keys of one column per lane per read.
//  - Both are read with the streaming (non-temporal) cache policy: every byte
//    is used once, and the hint took the kernel from 6.0 to 7.0 TB/s.
#include "rf_device.hpp"
#include "rf_launch.hpp"

#include <type_traits>

namespace rf {
namespace {

constexpr int STEP = 32;                  // keys per wave step
constexpr int NW = 4;                     // waves per workgroup
constexpr int kMaxVSlot = STEP * 128 * 2; // one step of V rows at head size 128, 8 KB
constexpr int kSmem = NW * 2 * kMaxVSlot; // two slots per wave, 64 KB

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

// ds_read_b64_tr_b16 through inline asm. The compiler cannot tell whether a
// read from LDS overlaps a pending buffer-to-LDS load, so for the builtin it
// drains every outstanding load first (including the prefetches of later
// steps). The asm form is invisible to that analysis; its results become
// usable only through tr_wait(), which waits for the LDS reads explicitly.
__device__ __forceinline__ u32x2 tr_read(uint32_t lds_addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// V slot layout: row r (a key) holds 2 D bytes = D / 8 chunks of 16 bytes;
// logical chunk c sits at physical chunk c ^ vswz(r). vswz is even, so the
// chunk pairs {2n, 2n + 1} (one 16-column block) stay together; at head size
// 128 the transposed reads of 32 consecutive lanes (rows 8g + 0..3 and
// 8g + 8 + 0..3 of a slot, one 32-byte pair each) land on distinct banks.
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return D == 128 ? 2 * (row & 3) + 8 * ((row >> 3) & 1) : 2 * (row & 3);
}

template <int V>
using ic = std::integral_constant<int, V>;

struct KRegs {
  u32x4 k[2][4];  // A operand of S^T = K Q^T: [key block][d step] (D / 32 d steps used)
};

// Arrays the lambdas below capture are sized for head size 128 (a size that
// depends on the template argument keeps the host pass from emitting the
// kernel); head size 64 uses their leading elements.
template <int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ part_m, float* __restrict__ part_l,
    float* __restrict__ part_acc, int Hq, int Hkv, int Lk, int S, int seg_len, float scale) {
  constexpr int kRow = 2 * D;              // bytes per K/V row
  constexpr int kVSlot = STEP * kRow;      // one step of V rows
  constexpr int NDS = D / 32;              // k-steps of the 16x16x32 score product
  constexpr int NKL = 2 * NDS;             // K loads per step (per lane)
  constexpr int NVL = kVSlot / 1024;       // 1 KB V loads per step
  constexpr int NB = D / 16;               // 16-column blocks of the output
  constexpr int kChunks = D / 8;           // 16-byte chunks per row
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];

  const int s = blockIdx.x % S;
  const int bhk = blockIdx.x / S;  // b * Hkv + hk
  const int b = bhk / Hkv, hk = bhk - b * Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to M0
  const int g = lane >> 4, lq = lane & 15;

  const int t0 = min(s * seg_len, Lk), t1 = min(t0 + seg_len, Lk);
  const int nsteps = (t1 - t0 + STEP - 1) / STEP;

  const uint16_t* kp = k + (size_t)bhk * Lk * D;
  const uint16_t* vp = v + (size_t)bhk * Lk * D;

  // Q^T as the B operand: lane holds query head hk*G + lq (zero if lq >= G), d = 32*ds + 8*g.
  bf16x8 qf[4];
  {
    const uint16_t* qrow = q + ((size_t)b * Hq + hk * G + lq) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (lq < G) w = *reinterpret_cast<const u32x4*>(qrow + 32 * ds + 8 * g);
      qf[ds] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Every load below is issued unconditionally; a step past the segment gets
  // the scalar offset kv_end, the byte size of one head's K (or V), so its
  // loads read zeros without touching memory. That keeps the number of loads
  // in flight, and so every wait count, fixed.
  const int kv_end = Lk * D * 2;
  auto soff_of = [&](int step) {
    return __builtin_amdgcn_readfirstlane(step < nsteps ? (t0 + step * STEP) * kRow : kv_end);
  };

  // K row loaded by this lane for key block kb: row i = lq of the block holds key
  // 8*(lq/4) + 4*kb + lq%4, so lane group g ends up with keys 8g..8g+7 of the step.
  // Buffer loads: 32-bit offsets, and rows past Lk read as zero (masked below).
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)kv_end);
  int kvo[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) kvo[kb] = (8 * (lq >> 2) + (lq & 3) + 4 * kb) * kRow + 16 * g;
  auto load_k = [&](int step, KRegs& r) {
    const int soff = soff_of(step);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
        r.k[kb][ds] = buf_load16_stream(krs, kvo[kb] + 64 * ds, soff);
  };

  // V step -> LDS slot: NVL 1 KB loads, load i covers rows (1024 / kRow) i ..
  // of the step; lane l writes physical chunk l % kChunks of its row, so it
  // fetches the logical chunk (l % kChunks) ^ vswz(row). Rows past Lk read as
  // zero (their scores are masked anyway); rows past the segment are real keys
  // whose weights are 0.
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (uint32_t)kv_end);
  int vvo[8];
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int row = (1024 / kRow) * i + lane / kChunks;
    vvo[i] = row * kRow + (((lane % kChunks) ^ vswz<D>(row)) << 4);
  }
  char* vslots = smem + wave * 2 * kVSlot;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_char*)vslots;  // LDS byte address
  auto issue_v = [&](int step, int slot) {
    char* dst = vslots + __builtin_amdgcn_readfirstlane(slot * kVSlot);
    const int soff = soff_of(step);
#pragma unroll
    for (int i = 0; i < NVL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + i * 1024), 16, vvo[i], soff, 0,
                                               kStreamPolicy);
  };
  // Transposed read of d block nb: lane (g, lq) points at row 8g + lq/4 (+4 for
  // the second read), columns 16 nb + 4 (lq % 4) .. + 3; the LDS returns to lane
  // lq the four keys of column 16 nb + lq.
  int vto[8];
  {
    const int row = 8 * g + (lq >> 2);
    const int sw = vswz<D>(row) >> 1;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) vto[nb] = row * kRow + ((nb ^ sw) << 5) + 8 * (lq & 3);
  }

  float m_run = kNegInf, l_run = 0.f;  // statistics of query head lq
  f32x4 oacc[8];                       // O[q = 4g + r][d = 16*nb + lq]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{};

  KRegs ks[3];
  // Prologue, in the order the waits below assume: K(0), V(0), K(1).
  load_k(wave, ks[0]);
  issue_v(wave, 0);
  load_k(wave + NW, ks[1]);

  // Iteration j handles step wave + NW j with K set j % 3 and V slot j % 2. It
  // first issues V(j + 1) and K(j + 2), so inside the unrolled loop exactly
  // 2 NKL + NVL loads are issued after V(j): K(j + 1), V(j + 1), K(j + 2). In
  // the tail iterations after the loop some of those K loads feed nothing and
  // the compiler drops them, so the tail waits for all loads instead.
  auto body = [&](auto cset, auto tail_c, int j) {
    constexpr int C = decltype(cset)::value;
    constexpr bool TAIL = decltype(tail_c)::value != 0;
    const int step = wave + NW * j;
    issue_v(step + NW, (j + 1) & 1);
    load_k(step + 2 * NW, ks[(C + 2) % 3]);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetches ahead of the math
    const int kbase = t0 + step * STEP;
    // ---- S^T = K Q^T: sacc[kb][r] is the score of key kbase + 8g + 4kb + r, head lq.
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 a = f32x4{};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) a = mfma16(__builtin_bit_cast(bf16x8, ks[C].k[kb][ds]), qf[ds], a);
      sacc[kb] = a;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float sc = sacc[kb][r] * scale;
        if (kbase + 8 * g + 4 * kb + r >= t1) sc = kNegInf;
        sacc[kb][r] = sc;
        mx = fmaxf(mx, sc);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float ms = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - ms) * kLog2e);
    // P enters the second product as a sum of two bf16 terms (p = hi + lo), so
    // the weights keep about 16 significant bits; the extra MFMAs are free in a
    // kernel bound by HBM.
    float rs = 0.f;
    bf16x8 pa, pa_lo;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2((sacc[kb][r] - ms) * kLog2e);
        rs += p;
        const __bf16 hi = (__bf16)p;
        pa[4 * kb + r] = hi;
        pa_lo[4 * kb + r] = (__bf16)(p - (float)hi);
      }
    rs += __shfl_xor(rs, 16, kWave);
    rs += __shfl_xor(rs, 32, kWave);
    l_run = alpha * l_run + rs;
    m_run = m_new;
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r, kWave);
    // ---- wait for V(j) to land in its slot (tied to l_run so that the wait
    // stays behind the softmax instead of being hoisted into the products).
    if constexpr (TAIL)
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(l_run) : : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%1)" : "+v"(l_run) : "i"(2 * NKL + NVL) : "memory");
    // ---- O += P V: B operands of the eight d blocks (keys 8g..8g+3, then
    // 8g+4..8g+7, of column 16 nb + lq), read transposed from the slot.
    const uint32_t vs = lds_base + (uint32_t)((j & 1) * kVSlot);
    u32x2 vt[8][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      vt[nb][0] = tr_read(vs + vto[nb]);
      vt[nb][1] = tr_read(vs + vto[nb] + 4 * kRow);
    }
    if constexpr (NB == 8)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(vt[0][0]), "+v"(vt[0][1]), "+v"(vt[1][0]), "+v"(vt[1][1]),
                     "+v"(vt[2][0]), "+v"(vt[2][1]), "+v"(vt[3][0]), "+v"(vt[3][1]),
                     "+v"(vt[4][0]), "+v"(vt[4][1]), "+v"(vt[5][0]), "+v"(vt[5][1]),
                     "+v"(vt[6][0]), "+v"(vt[6][1]), "+v"(vt[7][0]), "+v"(vt[7][1]));
    else
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(vt[0][0]), "+v"(vt[0][1]), "+v"(vt[1][0]), "+v"(vt[1][1]),
                     "+v"(vt[2][0]), "+v"(vt[2][1]), "+v"(vt[3][0]), "+v"(vt[3][1]));
    // rescale O rows 4g + r by their head's alpha, then accumulate.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 vb = __builtin_bit_cast(
          bf16x8, u32x4{vt[nb][0][0], vt[nb][0][1], vt[nb][1][0], vt[nb][1][1]});
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[nb][r] *= ar[r];
      oacc[nb] = mfma16(pa, vb, oacc[nb]);
      oacc[nb] = mfma16(pa_lo, vb, oacc[nb]);
    }
  };

  // This wave's steps: wave, wave + NW, ... below nsteps.
  const int niter = (nsteps - wave + NW - 1) / NW;
  int j = 0;
  for (; j + 3 <= niter; j += 3) {
    body(ic<0>{}, ic<0>{}, j);
    body(ic<1>{}, ic<0>{}, j + 1);
    body(ic<2>{}, ic<0>{}, j + 2);
  }
  if (j < niter) body(ic<0>{}, ic<1>{}, j);
  if (j + 1 < niter) body(ic<1>{}, ic<1>{}, j + 1);

  // ---- merge the four waves' states (same rule as the merge across segments).
  // The loads issued past the end still write their (zero) rows into the V
  // slots: drain them before the slots are reused.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  float* sm_m = reinterpret_cast<float*>(smem);      // [NW][16]
  float* sm_l = sm_m + NW * 16;                       // [NW][16]
  float* sm_acc = sm_l + NW * 16;                     // [NW][16][D]
  if (g == 0) {
    sm_m[wave * 16 + lq] = m_run;
    sm_l[wave * 16 + lq] = l_run;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qh = 4 * g + r;
      if (qh < G) sm_acc[(wave * 16 + qh) * D + 16 * nb + lq] = oacc[nb][r];
    }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int qh = idx / D, d = idx - qh * D;
    float mw[NW], ms = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = sm_m[w * 16 + qh];
      ms = fmaxf(ms, mw[w]);
    }
    // No shortcut for ms = -inf: every weight is then 0, and 0 * l keeps a NaN
    // that reached l (scores that are all NaN leave the max at -inf).
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = (mw[w] == kNegInf) ? 0.f : fast_exp2((mw[w] - ms) * kLog2e);
      l += wt * sm_l[w * 16 + qh];
      acc += wt * sm_acc[(w * 16 + qh) * D + d];
    }
    const size_t row = ((size_t)b * Hq + hk * G + qh) * S + s;
    part_acc[row * D + d] = acc;
    if (d == 0) {
      part_m[row] = ms;
      part_l[row] = l;
    }
  }
}

// Fold one partial state (ms, ls, as) into a running (m, l, acc): both sides
// are rescaled to the larger max; a side with max -inf is empty and has weight 0.
__device__ __forceinline__ void fold_state(float& m, float& l, f32x4& acc, float ms, float ls,
                                           const f32x4& as) {
  const float mn = fmaxf(m, ms);
  const float a = (m == kNegInf) ? 0.f : fast_exp2((m - mn) * kLog2e);
  const float b = (ms == kNegInf) ? 0.f : fast_exp2((ms - mn) * kLog2e);
  l = l * a + ls * b;
  acc = acc * a + as * b;
  m = mn;
}

// One wave per row, no LDS. Lane (h, c) covers columns 4c..4c+3 of a
// 128-column block and folds the states s = h, h + 2, ... with the rescale-
// and-add rule (cue 21), loading kChunk states at a time so their loads are
// in flight together; the two half-waves then merge their states and lanes of
// the first half write the row. Each 128-column block of a row is its own
// wave (grid y), so wide rows do not serialise their blocks.
constexpr int kChunk = 8;

__global__ __launch_bounds__(64) void merge_states_kernel(const float* __restrict__ part_m,
                                                          const float* __restrict__ part_l,
                                                          const float* __restrict__ part_acc,
                                                          int S, int d, int out_bf16,
                                                          void* __restrict__ o,
                                                          float* __restrict__ lse) {
  const size_t row = blockIdx.x;
  const int lane = threadIdx.x, h = lane >> 5, c = lane & 31;
  const float* mrow = part_m + row * S;
  const float* lrow = part_l + row * S;
  const float* arow = part_acc + row * S * d;
  {
    const int c0 = 128 * blockIdx.y;
    const int col = c0 + 4 * c;
    const bool act = col < d;
    float m = kNegInf, l = 0.f;
    f32x4 acc = f32x4{};
    for (int s0 = 0; s0 < S; s0 += 2 * kChunk) {
      float ms[kChunk], ls[kChunk];
      f32x4 as[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        const int s = s0 + h + 2 * i;
        const int sc = min(s, S - 1);  // loads stay unconditional; out-of-range states are empty
        ms[i] = mrow[sc];
        ls[i] = lrow[sc];
        as[i] = act ? *reinterpret_cast<const f32x4*>(arow + (size_t)sc * d + col) : f32x4{};
        if (s >= S) ms[i] = kNegInf;
      }
#pragma unroll
      for (int i = 0; i < kChunk; ++i) fold_state(m, l, acc, ms[i], ls[i], as[i]);
    }
    // Merge the other half-wave's state (lane c + 32 holds the same columns).
    const float m2 = __shfl_xor(m, 32, kWave), l2 = __shfl_xor(l, 32, kWave);
    f32x4 a2;
#pragma unroll
    for (int e = 0; e < 4; ++e) a2[e] = __shfl_xor(acc[e], 32, kWave);
    fold_state(m, l, acc, m2, l2, a2);
    if (h == 0 && act) {
      const float inv = (l > 0.f) ? 1.f / l : (l == 0.f ? 0.f : l);  // a NaN in l stays NaN
      acc *= inv;
      if (out_bf16) {
        const u32x2 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + row * d + col) = w;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(o) + row * d + col) = acc;
      }
    }
    if (lse && lane == 0 && c0 == 0) lse[row] = (m == kNegInf && l == 0.f) ? kNegInf : m + logf(l);
  }
}

}  // namespace

hipError_t launch_decode_split_bf16(const void* q, const void* k, const void* v, float* part_m,
                                    float* part_l, float* part_acc, int B, int Hq, int Hkv, int Lk,
                                    int d, int S, float scale, hipStream_t stream) {
  const int seg_len = (Lk + S - 1) / S;
  dim3 grid(B * Hkv * S);
  if (d == 64)
    hipLaunchKernelGGL((decode_split_kernel<64>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), part_m, part_l, part_acc, Hq, Hkv, Lk, S,
                       seg_len, scale);
  else
    hipLaunchKernelGGL((decode_split_kernel<128>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), part_m, part_l, part_acc, Hq, Hkv, Lk, S,
                       seg_len, scale);
  return hipGetLastError();
}

hipError_t launch_merge_states(const float* part_m, const float* part_l, const float* part_acc,
                               int rows, int S, int d, int out_bf16, void* o, float* lse,
                               hipStream_t stream) {
  hipLaunchKernelGGL(merge_states_kernel, dim3(rows, (d + 127) / 128), dim3(64), 0, stream, part_m,
                     part_l, part_acc, S, d, out_bf16, o, lse);
  return hipGetLastError();
}

}  // namespace rf
