// Split-KV decode partial states for fp32 K/V (Multi-Segment).
//
// The same states as the bf16 kernel: per (batch, query head, segment) the
// max m of the segment's scaled scores, l = sum exp(score - m) and the
// unnormalised acc = sum exp(score - m) v, built in one pass with the running
// (m, l, acc) rescaled by exp(m_old - m_new) when the max grows ("RedFuser
// episode transcript", cues 19, 21 and 39). All arithmetic is fp32: both
// contractions run on v_mfma_f32_16x16x4_f32 (fp32 products, fp32 sums), the
// exponentials and the statistics on the VALU.
//
// One workgroup of 4 waves per (batch, key/value head, segment) streams the
// segment's K and V rows once for the whole GQA group (up to 16 query heads
// in the MFMA's N dimension). The waves take interleaved 16-key steps:
//  - K rows go straight from memory into the A operand of S^T = K Q^T, two
//    steps ahead, in three register sets whose roles rotate with a 3-way
//    unrolled loop. Lane (key i, slot g) loads the key's values
//    16 c + 4 g .. + 3 with load c, so the four slots of a key read 64
//    contiguous bytes per load (a layout with each slot reading its own
//    quarter of the row touched four times as many cache lines per load and
//    ran at 3.8 instead of 7.0 TB/s).
//  - V rows go one step ahead into a two-slot LDS ring per wave (buffer loads
//    to LDS, contiguous); lane (column i, slot g) reads row 4 g + r, columns
//    64 a + 4 i .. + 3 with one 16-byte read that feeds four column blocks
//    of O^T = V^T P^T, whose B operand is the lane's own probability.
//  - Every load uses the streaming cache policy (bytes read once).
// The four waves' states are merged at the end by the rule that merges
// segments.
#include "rf_device.hpp"
#include "rf_launch.hpp"

#include <type_traits>

namespace rf {
namespace {

constexpr int STEP = 16;                   // keys per wave step
constexpr int NW = 4;                      // waves per workgroup
constexpr int kMaxVSlot = STEP * 128 * 4;  // one step of V rows at head size 128, 8 KB
constexpr int kSmem = NW * 2 * kMaxVSlot;  // two slots per wave, 64 KB

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int V>
using ic = std::integral_constant<int, V>;

struct KRegs {
  u32x4 k[8];  // this lane's D / 4 consecutive K values of its key (D / 16 loads used)
};

template <int D>
__global__ __launch_bounds__(256, 2) void decode_split_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ part_acc, int Hq,
    int Hkv, int Lk, int S, int seg_len, float scale) {
  constexpr int kRow = 4 * D;             // bytes per K/V row
  constexpr int kVSlot = STEP * kRow;     // one step of V rows
  constexpr int NKL = D / 16;             // 16-byte K loads per lane per step
  constexpr int NVL = kVSlot / 1024;      // 1 KB V loads per step
  constexpr int NA = D / 64;              // 64-column groups of the output
  constexpr int NDB = D / 16;             // 16-column blocks of the output
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];

  const int s = blockIdx.x % S;
  const int bhk = blockIdx.x / S;  // b * Hkv + hk
  const int b = bhk / Hkv, hk = bhk - b * Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;

  const int t0 = min(s * seg_len, Lk), t1 = min(t0 + seg_len, Lk);
  const int nsteps = (t1 - t0 + STEP - 1) / STEP;

  // Q^T, the B operand of S^T = K Q^T: lane (head i16, k slot g) holds
  // q[head][16 c + 4 g + e] for MFMA 4 c + e (0 for heads past the group).
  float qf[32];
  {
    const float* qrow = q + ((size_t)b * Hq + hk * G + i16) * D + 4 * g;
#pragma unroll
    for (int c = 0; c < NKL; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (i16 < G) w = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * c + e] = __uint_as_float(w[e]);
    }
  }

  // Every load is issued unconditionally; a step past the segment takes the
  // scalar offset kv_end (the byte size of one head's K or V), so it reads
  // zeros without touching memory and every wait count below stays fixed.
  const int kv_end = Lk * kRow;
  auto soff_of = [&](int step) {
    return __builtin_amdgcn_readfirstlane(step < nsteps ? (t0 + step * STEP) * kRow : kv_end);
  };
  // K, the A operand: lane (key i16 of the step, k slot g) loads its key's
  // values 16 c + 4 g .. + 3 with load c (MFMA 4 c + e takes value e), so the
  // four slots of a key read 64 contiguous bytes per load.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (size_t)bhk * Lk * D, (uint32_t)kv_end);
  const int kvo = i16 * kRow + 16 * g;
  auto load_k = [&](int step, KRegs& r) {
    const int soff = soff_of(step);
#pragma unroll
    for (int c = 0; c < NKL; ++c) r.k[c] = buf_load16_stream(krs, kvo + 64 * c, soff);
  };
  // V rows of a step: NVL contiguous 1 KB loads into the wave's slot.
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + (size_t)bhk * Lk * D, (uint32_t)kv_end);
  char* vslots = smem + wave * 2 * kVSlot;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_char*)vslots;
  auto issue_v = [&](int step, int slot) {
    char* dst = vslots + __builtin_amdgcn_readfirstlane(slot * kVSlot);
    const int soff = soff_of(step);
#pragma unroll
    for (int n = 0; n < NVL; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + n * 1024), 16, 1024 * n + 16 * lane,
                                               soff, 0, kStreamPolicy);
  };

  float m_run = kNegInf, l_run = 0.f;  // statistics of query head i16
  // O^T: oacc[4 a + e][r'] is column d = 64 a + 16 g + 4 r' + e of head i16.
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};

  KRegs ks[3];
  // Prologue, in the order the waits below assume: K(0), V(0), K(1).
  load_k(wave, ks[0]);
  issue_v(wave, 0);
  load_k(wave + NW, ks[1]);

  // Iteration j handles step wave + NW j with K set j % 3 and V slot j % 2. It
  // first issues V(j + 1) and K(j + 2), so inside the unrolled loop exactly
  // 2 NKL + NVL loads are issued after V(j). In the tail iterations after the
  // loop some of those K loads feed nothing and the compiler drops them, so
  // the tail waits for all loads instead.
  auto body = [&](auto cset, auto tail_c, int j) __attribute__((always_inline)) {
    constexpr int C = decltype(cset)::value;
    constexpr bool TAIL = decltype(tail_c)::value != 0;
    const int step = wave + NW * j;
    issue_v(step + NW, (j + 1) & 1);
    load_k(step + 2 * NW, ks[(C + 2) % 3]);
    __builtin_amdgcn_sched_barrier(0);
    const int kbase = t0 + step * STEP;
    // ---- S^T = K Q^T: sacc[r] is the score of key kbase + 4 g + r, head i16.
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int c = 0; c < NKL; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc = mfma4(__uint_as_float(ks[C].k[c][e]), qf[4 * c + e], sacc);
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sc = sacc[r] * scale;
      if (kbase + 4 * g + r >= t1) sc = kNegInf;
      sacc[r] = sc;
      mx = fmaxf(mx, sc);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float ms = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - ms) * kLog2e);
    float p[4], rs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2((sacc[r] - ms) * kLog2e);
      rs += p[r];
    }
    rs += __shfl_xor(rs, 16, kWave);
    rs += __shfl_xor(rs, 32, kWave);
    l_run = alpha * l_run + rs;
    m_run = m_new;
    // ---- wait for V(j) in its slot (tied to l_run so it stays behind the softmax)
    if constexpr (TAIL)
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(l_run) : : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%1)" : "+v"(l_run) : "i"(2 * NKL + NVL) : "memory");
    // ---- O^T += V^T P^T: k-step r covers keys 4 g + r; lane (d row i16, slot g)
    // reads row 4 g + r, columns 64 a + 4 i16 .. + 3: one 16-byte read feeds
    // the four blocks 4 a + e.
    const uint32_t vrow = lds_base + (uint32_t)((j & 1) * kVSlot) + (uint32_t)(4 * g * kRow + 16 * i16);
    u32x4 vt[4][2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      vt[r][0] = lds_read16<0>(vrow + r * kRow);
      if constexpr (NA == 2) vt[r][1] = lds_read16<256>(vrow + r * kRow);
    }
    if constexpr (NA == 2)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(vt[0][0]), "+v"(vt[0][1]), "+v"(vt[1][0]), "+v"(vt[1][1]),
                     "+v"(vt[2][0]), "+v"(vt[2][1]), "+v"(vt[3][0]), "+v"(vt[3][1]));
    else
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(vt[0][0]), "+v"(vt[1][0]), "+v"(vt[2][0]), "+v"(vt[3][0]));
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          oacc[4 * a + e] = mfma4(__uint_as_float(vt[r][a][e]), p[r], oacc[4 * a + e]);
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

  // ---- merge the four waves' states (the rule that merges segments). The
  // loads issued past the end still write their (zero) rows into the V slots:
  // drain them before the slots are reused.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  float* sm_m = reinterpret_cast<float*>(smem);      // [NW][16]
  float* sm_l = sm_m + NW * 16;                       // [NW][16]
  float* sm_acc = sm_l + NW * 16;                     // [NW][16][D]
  if (g == 0) {
    sm_m[wave * 16 + i16] = m_run;
    sm_l[wave * 16 + i16] = l_run;
  }
  if (i16 < G) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm_acc[(wave * 16 + i16) * D + 64 * a + 16 * g + 4 * r + e] = oacc[4 * a + e][r];
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
    // that reached l.
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

}  // namespace

hipError_t launch_decode_split_f32(const float* q, const float* k, const float* v, float* part_m,
                                   float* part_l, float* part_acc, int B, int Hq, int Hkv, int Lk,
                                   int d, int S, float scale, hipStream_t stream) {
  const int seg_len = (Lk + S - 1) / S;
  dim3 grid(B * Hkv * S);
  if (d == 64)
    hipLaunchKernelGGL((decode_split_f32_kernel<64>), grid, dim3(256), 0, stream, q, k, v, part_m,
                       part_l, part_acc, Hq, Hkv, Lk, S, seg_len, scale);
  else
    hipLaunchKernelGGL((decode_split_f32_kernel<128>), grid, dim3(256), 0, stream, q, k, v, part_m,
                       part_l, part_acc, Hq, Hkv, Lk, S, seg_len, scale);
  return hipGetLastError();
}

}  // namespace rf

