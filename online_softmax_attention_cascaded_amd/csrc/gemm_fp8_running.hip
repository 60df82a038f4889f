// Single-pass quantise-then-GEMM with a running per-row scale: the literal
// loop of the FP8 cascade ("RedFuser episode transcript", cue 33). There is no
// separate abs-max pass over A. For each K tile of 64 columns, every row of A
// raises its running abs-max with the tile's values, the tile is quantised to
// e4m3 with the current scale s = fp32(absmax / 448), and when the scale grew
// the accumulator row is first multiplied by s_old / s_new, so it always holds
// the sum in units of the current scale. At the end C = s_final * t * acc.
// Early K tiles are therefore quantised with a smaller scale than the row's
// final one (finer steps, different codes from the final-scale path).
//
// Workgroup tile 128 x 512: every A tile is quantised by N / 512 workgroups
// (the price of having no pre-pass), half as often as with square 256 tiles.
// Eight waves of 64 x 128 (two per SIMD, 128 accumulator registers each) on
// v_mfma_f32_32x32x64_f8f6f4 taking A first: a lane holds one column of C and,
// in each group of four registers, rows 8 g + 0..3 of a 32-row block (+ 4 in
// the upper half of the wave), so a rescale touches only the register groups
// whose rows moved.
//
// Pipeline, one K tile (step) t per barrier: the MFMAs of step t read the code
// tile of step t and the B stage, while the same waves quantise step t + 1
// from registers into the other code tile, so the quantiser's VALU work and
// the matrix cores overlap. B goes HBM -> LDS by buffer loads straight into
// LDS, 128 K columns (two steps) per stage, two stages; each lane's share of
// A (4 lanes per row, 16 values per step) is loaded into registers a stage
// ahead. The quantiser: abs-max on the bf16 magnitude bits (packed 16-bit
// max), combined over the row's 4 lanes by DPP; on growth the new scale, the
// ratio s_old / s_new (published in LDS for the step's MFMA waves) and 1 / s;
// codes as the correctly rounded x / s (one Markstein correction of
// x * RN(1/s), exact for s >= 2^-90; smaller nonzero scales divide) through
// the hardware round-to-nearest-even e4m3 convert.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int BM = 128, BN = 512, BK = 64;  // BK: K columns per step of the running scale
constexpr int LK = 128;                      // K columns per B stage (two steps)
constexpr int kBStage = BN * LK;             // 64 KB of e4m3 B per stage
constexpr int kCodes = BM * BK;              // 8 KB of e4m3 A codes per step
constexpr int kOffCodes = 2 * kBStage;
constexpr int kOffRatio = kOffCodes + 2 * kCodes;
constexpr int kOffScale = kOffRatio + 2 * BM * 4;
constexpr int kSmem = kOffScale + BM * 4;    // 145.5 KB
constexpr int kGroupM = 8;                   // tile rows per band of the tile order
// Smallest scale of the one-correction division: below it x - s q can
// underflow and the correction is no longer exact.
constexpr float kMinFastScale = 0x1p-90f;

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// B stage: 128-byte rows, 16-byte chunks XOR (row >> 1) & 7, so the operand
// reads of 16 consecutive rows (one LDS pass of ds_read_b128) use all 64 banks.
__device__ __forceinline__ int b_off(int row, int chunk) {
  return row * LK + ((chunk ^ ((row >> 1) & 7)) << 4);
}
// Code tile: 64-byte rows, chunks XOR (row >> 2) & 3 (the same property).
__device__ __forceinline__ int c_off(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Tile order: workgroups are dealt to the 8 XCDs round-robin, so workgroup b is
// renumbered to give each XCD a contiguous run of tile ids, which then walk
// bands of kGroupM tile rows column by column (at 32 x 8 tiles each XCD gets a
// block of 8 tile rows x 4 tile columns).
__device__ __forceinline__ void tile_of(int b, int ntm, int ntn, int& tm, int& tn) {
  const int T = ntm * ntn;
  const int t = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  const int first = (t / (kGroupM * ntn)) * kGroupM;
  const int rows = min(kGroupM, ntm - first);
  const int r = t - first * ntn;
  tm = first + r % rows;
  tn = r / rows;
}

__global__ __launch_bounds__(512, 1) void gemm_fp8_running_kernel(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ bq, const float* __restrict__ sb,
    int M, int N, int K, float* __restrict__ a_scale, uint16_t* __restrict__ c, int vec) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  float* const ratio_s = reinterpret_cast<float*>(smem + kOffRatio);
  float* const scale_s = reinterpret_cast<float*>(smem + kOffScale);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;  // 64-row half, 128-column quarter
  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const __amdgpu_buffer_rsrc_t ars =
      make_rsrc(a + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K * 2));
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(bq + (size_t)n0 * K, (uint32_t)(min(BN, N - n0) * K));

  // ---- B: wave w fills rows 64 w .. 64 w + 63 of a stage, eight 1 KB blocks
  // of 8 rows; lane l writes physical chunk l % 8 of row 8 i + l / 8. Rows past
  // N read as 0 (the row offset is in the per-lane offset, which the buffer
  // range checks).
  const int brow = 64 * wave + (lane >> 3);
  auto issue_b = [&](int g) {
    char* st = smem + (g & 1) * kBStage;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = brow + 8 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void*)(st + (8 * wave + i) * 1024), 16,
                                               row * K + 16 * ((lane & 7) ^ ((row >> 1) & 7)),
                                               g * LK, 0, 0);
    }
  };

  // ---- A: lanes 4 r' .. 4 r' + 3 of wave w share row qr = 16 w + r'; lane
  // quarter q holds chunks (8 bf16) q and q + 4 of each step, so each load
  // instruction reads 64 contiguous bytes of 16 rows. Rows past M read as 0.
  const int qr = tid >> 2, q = lane & 3;
  const int avoff = qr * K * 2 + 16 * q;
  auto issue_a = [&](int t, u32x4 (&dst)[2]) {
    dst[0] = buf_load16(ars, avoff, t * BK * 2);
    dst[1] = buf_load16(ars, avoff + 64, t * BK * 2);
  };

  // ---- quantiser state of row qr (identical in its 4 lanes).
  uint32_t amax_bits = 0;  // running abs-max as bf16 magnitude bits
  float s_run = 0.f, rcp = 0.f;

  // Step t's codes of row qr from its 16 values (chunks q and q + 4 of the
  // step), the row's ratio for step t.
  auto quant = [&](int t, const u32x4& x0, const u32x4& x1) {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, x0[e] & 0x7fff7fffu));
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, x1[e] & 0x7fff7fffu));
    }
    uint32_t m = max((uint32_t)m2[0], (uint32_t)m2[1]);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kDppQuadXor1, 0xF, 0xF, true));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kDppQuadXor2, 0xF, 0xF, true));
    float ratio = 1.f;
    if (m > amax_bits) {
      // The accumulator row holds the sum in units of s_run; it moves to s_new.
      const float s_new = __uint_as_float(m << 16) / 448.f;
      if (amax_bits != 0) ratio = s_run / s_new;
      amax_bits = m;
      s_run = s_new;
      rcp = 1.f / s_new;
    }
    if (q == 0) ratio_s[(t & 1) * BM + qr] = ratio;
    char* const codes = smem + kOffCodes + (t & 1) * kCodes;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32x4 xv = k ? x1 : x0;
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[2 * e] = bf16_lo(xv[e]);
        y[2 * e + 1] = bf16_hi(xv[e]);
      }
      if (!(s_run > 0.f && s_run < kMinFastScale)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float q0 = y[j] * rcp;
          y[j] = fmaf(fmaf(-s_run, q0, y[j]), rcp, q0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = y[j] / s_run;
      }
      uint32_t lo = 0u, hi = 0u;
      if (s_run > 0.f) {
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo, true);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)hi, true);
      }
      // bf16 chunk q (k = 0) or q + 4 (k = 1) -> code bytes 8 q (+ 32) of the row
      *reinterpret_cast<u32x2*>(codes + c_off(qr, 2 * k + (q >> 1)) + 8 * (q & 1)) = u32x2{lo, hi};
    }
  };

  // ---- MFMA operands. A code fragment i: rows wm*64 + 32 i + li; B fragment
  // j: rows wn*128 + 32 j + li; each lane takes 32 bytes of the step's 64.
  const int half = lane >> 5, li = lane & 31;
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  auto rd = [](const char* p) { return *reinterpret_cast<const u32x4*>(p); };
  auto frag = [](const u32x4& lo, const u32x4& hi) {
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto mfma_step = [&](int t) {
    const char* const codes = smem + kOffCodes + (t & 1) * kCodes;
    const char* const st = smem + ((t >> 1) & 1) * kBStage;
    const int ks = 4 * (t & 1);  // first 16-byte chunk of the step in a B row
    // Move the accumulator rows whose scale grew to this step's scale. Lane l
    // reads the ratio of row wm*64 + l; the ballot tells every lane which rows
    // moved. Register e of block i holds row 8 (e / 4) + e % 4 (lanes 0-31)
    // or that + 4 (lanes 32-63) of the block, so a group of four registers
    // covers 8 rows and is multiplied only when one of them moved, each lane by
    // the ratios of its own rows (exactly 1 for rows that did not move).
    const float rl = ratio_s[(t & 1) * BM + wm * 64 + lane];
    const uint64_t moved = __ballot(rl != 1.f);
    if (moved) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          // registers 4 gq .. 4 gq + 3 of block i: rows 8 gq + 0..3 (+ 4 for
          // lanes 32-63) of the block; rows that did not move have ratio 1
          if ((moved >> (32 * i + 8 * gq)) & 0xffull) {
            const f32x4 rt = *reinterpret_cast<const f32x4*>(
                ratio_s + (t & 1) * BM + wm * 64 + 32 * i + 8 * gq + 4 * half);
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[i][j][4 * gq + k] *= rt[k];
          }
        }
      }
    }
    i32x8 fa[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + 32 * i + li;
      fa[i] = frag(rd(codes + c_off(row, 2 * half)), rd(codes + c_off(row, 2 * half + 1)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + 32 * j + li;
      const i32x8 fb = frag(rd(st + b_off(row, ks + 2 * half)), rd(st + b_off(row, ks + 2 * half + 1)));
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i][j] = mfma_fp8(fa[i], fb, acc[i][j]);
    }
  };

  // Issue order: step t issues A(t + 2) (2 loads per lane), then at even t
  // B stage t / 2 + 1 (8 loads per lane). At the start of step t the B stage
  // of t must have landed: at even t it was issued at step t - 2, followed
  // only by A(t + 1); at odd t it has already been waited for. The A
  // registers are waited for where the quantiser first reads them.
  const int nt = K / BK, ng = K / LK;  // K is a multiple of 128
  u32x4 A0[2], A1[2];
  issue_a(0, A0);
  issue_b(0);
  issue_a(1, A1);
  quant(0, A0[0], A0[1]);
  for (int t = 0; t < nt; t += 2) {
    // step t (even)
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    lds_barrier();
    if (t + 2 < nt) issue_a(t + 2, A0);
    if ((t >> 1) + 1 < ng) issue_b((t >> 1) + 1);
    mfma_step(t);
    quant(t + 1, A1[0], A1[1]);
    // step t + 1 (odd)
    lds_barrier();
    if (t + 3 < nt) issue_a(t + 3, A1);
    mfma_step(t + 1);
    if (t + 2 < nt) quant(t + 2, A0[0], A0[1]);
  }

  // ---- final scales: s_final of each row (and A's scale output, written once
  // per row by the workgroups of the first column tile).
  if (q == 0) {
    scale_s[qr] = s_run;
    if (tn == 0 && m0 + qr < M) a_scale[m0 + qr] = s_run;
  }
  lds_barrier();

  // Epilogue: lane holds C column n0 + wn*128 + 32 j + li and, in register e
  // of block i, row m0 + wm*64 + 32 i + 8 (e / 4) + 4 half + e % 4. Lanes 2p and
  // 2p + 1 trade one value of each register pair (e, e + 1), so the even lane
  // stores columns (n, n + 1) of the pair's first row and the odd lane those
  // of its second row, 4 bytes each.
  const bool odd = lane & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 128 + 32 * j + li;
    const float tj = col < N ? sb[col] : 0.f;
    const int pcol = col & ~1;  // first column of the lane pair
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int lrow = wm * 64 + 32 * i + 8 * (e >> 2) + 4 * half + (e & 3);
        const float v0 = acc[i][j][e] * scale_s[lrow] * tj;          // row lrow
        const float v1 = acc[i][j][e + 1] * scale_s[lrow + 1] * tj;  // row lrow + 1
        const float send = odd ? v0 : v1;
        const float got = __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(send), kDppQuadXor1, 0xF, 0xF, true));
        const int row = m0 + lrow + (odd ? 1 : 0);
        const float lo = odd ? got : v0, hi = odd ? v1 : got;
        if (row < M) {
          uint16_t* dst = c + (size_t)row * N + pcol;
          if (vec && pcol + 1 < N) {
            *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(lo, hi);
          } else {
            if (pcol < N) dst[0] = __builtin_bit_cast(uint16_t, (__bf16)lo);
            if (pcol + 1 < N) dst[1] = __builtin_bit_cast(uint16_t, (__bf16)hi);
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp8_running(const void* a, const uint8_t* b_q, const float* b_scale, int M,
                                   int N, int K, float* a_scale, void* c, hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int vec = (N % 2 == 0) && (reinterpret_cast<uintptr_t>(c) % 4 == 0);
  hipLaunchKernelGGL(gemm_fp8_running_kernel, dim3(tiles), dim3(512), 0, stream,
                     static_cast<const uint16_t*>(a), b_q, b_scale, M, N, K, a_scale,
                     static_cast<uint16_t*>(c), vec);
  return hipGetLastError();
}

}  // namespace rf
