// Split-KV decode over a shared latent cache (multi-latent attention): every
// key is one latent row of 576 bf16 values (512 latent + 64 positional); the
// score of query head h is q_h . row, the value is the row's first 512
// columns. The cascade and its split are the ones of split-KV decode ("RedFuser
// episode transcript", cues 19, 21 and 39; cues 41 and 55 place the
// multi-latent decode kernel among the method's workloads): per segment a
// running max, denominator and unnormalised accumulator per head, written out
// as a partial state and merged by rf_merge_states.
//
// One workgroup (8 waves) per (batch, segment, group of 16 heads). The rows of
// a 32-key step (36 KB) go from HBM into LDS once, in a ring of stages filled
// by buffer loads with the LDS flag, each instruction one contiguous 1 KB.
//  * Scores: S[key][head] over 576 columns on v_mfma_f32_16x16x32_bf16 with
//    the 16 heads in N; wave (kt, dq) computes the 16 keys kt of the step over
//    its quarter of the columns, the eight partial tiles are summed through
//    LDS in a fixed order, so every wave holds the same scores and updates
//    the same running (m, l).
//  * Values: wave w accumulates O^T for columns 64 w .. 64 w + 63; the V^T
//    operand is read from the same LDS rows with the transposing read
//    ds_read_b64_tr_b16. P enters as a bf16 hi + lo pair (the matrix cores
//    have time to spare here), so the weights keep about 16 bits.
//  * Latent rows are stored with their 16-byte chunks XOR-swizzled by
//    f(r) = 2 (r & 7) | ((r >> 3) & 1): sixteen rows read at one column (score
//    operand) and four rows by two column chunks (transposing reads) both
//    fall on distinct banks. Positional parts: swizzle (r >> 1) & 7.
//  * Rows are loaded with the streaming (non-temporal) cache policy, since
//    each is read once (about 10 % faster than the default policy here).
#include "rf_device.hpp"
#include "rf_launch.hpp"

#include <atomic>

namespace rf {
namespace {

constexpr int DL = 512;                       // latent columns = value columns
constexpr int DR = 64;                        // positional columns
constexpr int DQK = DL + DR;                  // 576
constexpr int kRowBytes = DQK * 2;            // 1152 bytes per key
constexpr int STEP = 32;                      // keys per step
constexpr int kLatBytes = STEP * DL * 2;      // 32 KB
constexpr int kStageBytes = kLatBytes + STEP * DR * 2;  // + 4 KB
constexpr int NWAVE = 8;
constexpr int kPartBytes = NWAVE * 64 * 16;   // partial score tiles
// LDS stages (NST, a template parameter of the split kernel): 4 stages loaded
// three steps ahead fit one workgroup per CU; 2 stages loaded one step ahead
// take 80 KB, so two workgroups share a CU and one streams while the other
// fills or drains its pipeline. The launcher takes the second form when the
// grid has more workgroups than the GPU has CUs (measured: 10 % faster split
// from 16 segments of 8192 rows up, slower at 8, where the grid is one
// workgroup per CU).
template <int NST>
constexpr int smem_bytes() { return NST * kStageBytes + kPartBytes; }
constexpr float kTau = 8.f;

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lat_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ f32x4 mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fused merge. Every workgroup of a (sequence, head group) makes its partial
// state visible device-wide and counts itself in; the one that completes the
// count merges the group's S states with the rescale-and-add rule (each state
// moved to the common max, weight 0 for an empty one), writes O = acc / l and
// lse = m + ln l, and returns the counter to zero for the next call.
__device__ __forceinline__ void merge_if_last(int* __restrict__ counters, int* s_last, int cidx, int S,
                                              int H, int b, int hg, const float* __restrict__ part_m,
                                              const float* __restrict__ part_l,
                                              const float* __restrict__ part_acc, void* __restrict__ o,
                                              float* __restrict__ lse, int out_bf16) {
  // One wave publishes for the workgroup. Every wave first waits until the L2
  // has acknowledged its own stores of the state (the barrier alone does not
  // wait for them); thread 0's agent-scope release, an L2 write-back costly
  // enough to issue once per workgroup rather than once per wave, then covers
  // them all, and only the last workgroup pays the acquire (an L2 invalidate)
  // before reading the states.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const bool last =
        __hip_atomic_fetch_add(counters + cidx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_last = last;
  }
  __syncthreads();
  if (!*s_last) return;
  // 16 heads x 512 columns: thread t takes head t / 32, columns 16 (t % 32) .. + 15.
  const int t = threadIdx.x, head = hg * 16 + (t >> 5), c0 = 16 * (t & 31);
  const size_t r0 = ((size_t)b * H + head) * S;
  float m = kNegInf, l = 0.f;
  f32x4 acc[4] = {};
#pragma unroll 4
  for (int si = 0; si < S; ++si) {
    const float ms = part_m[r0 + si], ls = part_l[r0 + si];
    const f32x4* as = reinterpret_cast<const f32x4*>(part_acc + (r0 + si) * DL + c0);
    const float mn = fmaxf(m, ms);
    const float wa = (m == kNegInf) ? 0.f : fast_exp2((m - mn) * kLog2e);
    const float wb = (ms == kNegInf) ? 0.f : fast_exp2((ms - mn) * kLog2e);
    l = l * wa + ls * wb;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = acc[i] * wa + as[i] * wb;
    m = mn;
  }
  const float inv = (l > 0.f) ? 1.f / l : (l == 0.f ? 0.f : l);  // a NaN in l stays NaN
  const size_t orow = ((size_t)b * H + head) * DL + c0;
  if (out_bf16) {
    u32x4 w[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = acc[i] * inv;
      w[i >> 1][2 * (i & 1)] = pack_bf16x2(v[0], v[1]);
      w[i >> 1][2 * (i & 1) + 1] = pack_bf16x2(v[2], v[3]);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(o) + orow);
    dst[0] = w[0];
    dst[1] = w[1];
  } else {
    f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(o) + orow);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = acc[i] * inv;
  }
  if (lse && (t & 31) == 0) lse[(size_t)b * H + head] = (m == kNegInf && l == 0.f) ? kNegInf : m + logf(l);
  if (t == 0) counters[cidx] = 0;
}

// MERGE: the single-launch form (the workgroup that completes its group's
// count folds the group's states); a separate instantiation, so the split-only
// form carries none of that code and the two are told apart in a profile.
template <int NST, bool MERGE>
__global__ __launch_bounds__(512, NST == 2 ? 2 : 1) void mla_decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, float* __restrict__ part_m,
    float* __restrict__ part_l, float* __restrict__ part_acc, int H, int Lk, int S, int seg_len,
    float c, uint32_t q_and, uint32_t q_xor, int* __restrict__ counters, void* __restrict__ o,
    float* __restrict__ lse, int out_bf16) {
  __shared__ __attribute__((aligned(1024))) char smem[smem_bytes<NST>()];
  // Flag of the fused merge, in the stage memory: written only after the last
  // stage has been consumed. (A second LDS object would make the compiler
  // wait for every pending buffer-to-LDS load before each LDS read.)
  int* const s_last = reinterpret_cast<int*>(smem);
  const int ngroups = H >> 4;
  const int hg = blockIdx.x % ngroups;
  const int s = (blockIdx.x / ngroups) % S;
  const int b = blockIdx.x / (ngroups * S);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int k0 = min(s * seg_len, Lk), k1 = min(k0 + seg_len, Lk);
  const int head = hg * 16 + l16;

  // ---- partial-state outputs: row (b, head, s)
  const size_t prow = ((size_t)b * H + head) * S + s;
  if (k0 >= k1) {  // empty segment: the identity state
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      *reinterpret_cast<f32x4*>(part_acc + prow * DL + 64 * wave + 16 * mt + 4 * g4) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave == 0 && g4 == 0) {
      part_m[prow] = kNegInf;
      part_l[prow] = 0.f;
    }
    if constexpr (MERGE)
      merge_if_last(counters, s_last, b * ngroups + hg, S, H, b, hg, part_m, part_l, part_acc, o, lse,
                    out_bf16);
    return;
  }
  const int nsteps = (k1 - k0 + STEP - 1) / STEP;

  // ---- scores: wave (kt, dq) = (wave & 1, wave >> 1): keys 16 kt .. +15 of
  // the step; k-steps (32 columns each) 4 dq .. 4 dq + 3 of the latent part,
  // and for dq = 3 also the two positional k-steps.
  const int kt = wave & 1, dq = wave >> 1;
  const int nks = (dq == 3) ? 6 : 4;
  bf16x8_t qf[6];
  {
    const uint16_t* qr = q + ((size_t)b * H + head) * DQK;
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int ks = (j < 4) ? 4 * dq + j : 16 + (j - 4);  // global k-step (16, 17 = positional)
      u32x4 w = {0u, 0u, 0u, 0u};
      if (j < nks) w = *reinterpret_cast<const u32x4*>(qr + 32 * ks + 8 * g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (w[e] & q_and) ^ q_xor;  // sign / zero of the scale
      qf[j] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  const int srow = 16 * kt + l16;  // key row this lane reads for the score operand
  int sofs[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    if (j < 4) {
      const int ch = 4 * (4 * dq + j) + g4;  // 16-byte chunk of the latent row
      sofs[j] = srow * 1024 + 16 * (ch ^ lat_swz(srow));
    } else {
      const int ch = 4 * (j - 4) + g4;       // chunk of the positional part
      sofs[j] = kLatBytes + srow * 128 + 16 * (ch ^ rope_swz(srow));
    }
  }

  // ---- values: wave w owns columns 64 w .. +63 (four 16-column tiles). For
  // the transposing read, lane j of a 16-lane group points at row r0 + j / 4,
  // columns c0 + 4 (j % 4) .. +3; r0 = 4 g4 (slots 0..3) and 16 + 4 g4 (4..7).
  int vofs[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 16 * hh + 4 * g4 + (l16 >> 2);
      const int col = 64 * wave + 16 * mt + 4 * (l16 & 3);
      vofs[mt][hh] = row * 1024 + 16 * ((col >> 3) ^ lat_swz(row)) + 2 * (col & 7);
    }

  // ---- HBM -> LDS: latent rows 4 w .. 4 w + 3 of the step (one 1 KB load
  // each: lane l writes physical chunk l, fetching logical chunk l ^ f(row)),
  // and for waves 0..3 positional rows 8 w .. 8 w + 7 (lane l: row 8 w + l / 8,
  // physical chunk l % 8).
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(kv + (size_t)b * Lk * DQK, (uint32_t)Lk * kRowBytes);
  int lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * wave + i;
    lo[i] = row * kRowBytes + 16 * (lane ^ lat_swz(row));
  }
  const int rrow = 8 * wave + (lane >> 3);
  const int ro = rrow * kRowBytes + DL * 2 + 16 * ((lane & 7) ^ rope_swz(rrow & 31));
  auto issue = [&](int t) {
    char* st = smem + (t % NST) * kStageBytes;
    // steps past the segment point past the cache: zeros, no memory traffic
    const int soff = __builtin_amdgcn_readfirstlane((t < nsteps ? k0 + STEP * t : Lk) * kRowBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + (4 * wave + i) * 1024), 16, lo[i],
                                               soff, 0, kStreamPolicy);
    if (wave < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + kLatBytes + wave * 1024), 16, ro,
                                               soff, 0, kStreamPolicy);
  };

  float* const spart = reinterpret_cast<float*>(smem + NST * kStageBytes);
  f32x4 oacc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_c = kNegInf, l_run = 0.f;  // reference max (exp2 units) and denominator
  float m_true = kNegInf;             // the segment's true max, exp2 units

  // Keys of the last step that lie past the segment are still loaded (rows
  // of the next segment, or zeros past the cache) and masked; steps past the
  // segment load zeros from past the cache, which keeps every wave's load
  // count per step constant.
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) issue(t);
  for (int t = 0; t < nsteps; ++t) {
    // This wave's loads of step t have landed (those of the next NST - 2
    // steps may stay in flight); after the barrier every wave's have, and
    // every wave is done with step t-1, whose stage then takes step
    // t + NST - 1.
    if constexpr (NST == 4) {
      if (wave < 4)
        asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
      static_assert(NST == 2, "two or four stages");
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();
    issue(t + NST - 1);
    const char* st = smem + (t % NST) * kStageBytes;

    // partial scores of keys 16 kt .. +15, in two independent accumulation
    // chains (even and odd k-steps)
    f32x4 sp0 = {0.f, 0.f, 0.f, 0.f}, sp1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 6; j += 2) {
      if (j < nks) sp0 = mfma16(*reinterpret_cast<const bf16x8_t*>(st + sofs[j]), qf[j], sp0);
      if (j < nks) sp1 = mfma16(*reinterpret_cast<const bf16x8_t*>(st + sofs[j + 1]), qf[j + 1], sp1);
    }
    *reinterpret_cast<f32x4*>(spart + (wave * 64 + lane) * 4) = sp0 + sp1;
    lds_barrier();
    // full scores: lane holds keys 4 g4 + i (tile 0) and 16 + 4 g4 + i (tile 1)
    f32x4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 a = *reinterpret_cast<const f32x4*>(spart + ((0 * 2 + tt) * 64 + lane) * 4);
#pragma unroll
      for (int d = 1; d < 4; ++d) a += *reinterpret_cast<const f32x4*>(spart + ((d * 2 + tt) * 64 + lane) * 4);
      sc[tt] = a;
    }
    const int kb = k0 + STEP * t;
    if (kb + STEP > k1) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * tt + 4 * g4 + i >= k1) sc[tt][i] = kNegInf;
    }
    // online statistics of head l16 (its 32 keys sit in lanes l16 + 16 g4)
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, sc[tt][i]);
    mx = half_swap_max(row_swap_max(mx)) * c;
    m_true = __builtin_fmaxf(m_true, mx);
    if (t == 0) {
      m_c = mx;  // the first step of a segment holds at least one key
    } else if (__any(mx > m_c + kTau)) {
      float alpha = 1.f;
      if (mx > m_c + kTau) {
        alpha = fast_exp2(m_c - mx);
        m_c = mx;
      }
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) oacc[mt] *= alpha;
    }
    float p[8], rsum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * tt + i] = fast_exp2(fmaf(sc[tt][i], c, -m_c));
        rsum += p[4 * tt + i];
      }
    l_run += half_swap_sum(row_swap_sum(rsum));
    // P^T operand: slot j of lane group g4 <-> key (j < 4 ? 4 g4 + j : 16 + 4 g4 + j - 4)
    u32x4 phi, plo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = p[2 * j], a1 = p[2 * j + 1];
      const uint32_t hi = pack_bf16x2(a0, a1);
      phi[j] = hi;
      plo[j] = pack_bf16x2(a0 - bf16_lo(hi), a1 - bf16_hi(hi));
    }
    // O^T[c][head] += V^T[c][key] P^T[key][head]
    // all eight transposing reads first, then each tile waits for its own two
    const uint32_t sa = lds_addr(st);
    u32x4 va[4];
    static_for<4>([&](auto mc) {
      constexpr int mt = decltype(mc)::value;
      const u32x2 r0 = lds_read_tr16<0>(sa + vofs[mt][0]);
      const u32x2 r1 = lds_read_tr16<0>(sa + vofs[mt][1]);
      va[mt] = u32x4{r0[0], r0[1], r1[0], r1[1]};
    });
    static_for<4>([&](auto mc) {
      constexpr int mt = decltype(mc)::value;
      lds_wait_for<2 * (3 - mt)>(va[mt]);
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, va[mt]);
      oacc[mt] = mfma16(a, __builtin_bit_cast(bf16x8_t, phi), oacc[mt]);
      oacc[mt] = mfma16(a, __builtin_bit_cast(bf16x8_t, plo), oacc[mt]);
    });
  }
  // drain the loads issued for steps past the end before the workgroup exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- partial state: m = the segment's max scaled score; l and acc are
  // moved from the reference (at most kTau below it) to that max.
  const float f = fast_exp2(m_c - m_true);
  l_run *= f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) oacc[mt] *= f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    *reinterpret_cast<f32x4*>(part_acc + prow * DL + 64 * wave + 16 * mt + 4 * g4) = oacc[mt];
  if (wave == 0 && g4 == 0) {
    part_m[prow] = m_true * kLn2;
    part_l[prow] = l_run;
  }
  if constexpr (MERGE)
    merge_if_last(counters, s_last, b * ngroups + hg, S, H, b, hg, part_m, part_l, part_acc, o, lse,
                  out_bf16);
}

}  // namespace

hipError_t launch_mla_decode_split(const void* q, const void* kv, float* part_m, float* part_l,
                                   float* part_acc, int B, int H, int Lk, int S, float scale,
                                   int* counters, void* o, float* lse, int out_bf16,
                                   hipStream_t stream) {
  const int seg_len = (Lk + S - 1) / S;
  const dim3 grid(B * S * (H / 16));
  // CU count of the current device, queried once per device
  static std::atomic<int> cu_count[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = (dev >= 0 && dev < 64) ? cu_count[dev].load(std::memory_order_relaxed) : 0;
  if (cus == 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  const ScoreScale sc = score_scale(scale);
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(kv);
#define RF_MLA_LAUNCH(NST_, MERGE_)                                                                  \
  hipLaunchKernelGGL((mla_decode_split_kernel<NST_, MERGE_>), grid, dim3(512), 0, stream, qq, kk,     \
                     part_m, part_l, part_acc, H, Lk, S, seg_len, sc.c, sc.q_and, sc.q_xor, counters, \
                     o, lse, out_bf16)
  const bool two_stage = (long long)grid.x > cus;
  if (counters) {
    if (two_stage) RF_MLA_LAUNCH(2, true); else RF_MLA_LAUNCH(4, true);
  } else {
    if (two_stage) RF_MLA_LAUNCH(2, false); else RF_MLA_LAUNCH(4, false);
  }
#undef RF_MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace rf
