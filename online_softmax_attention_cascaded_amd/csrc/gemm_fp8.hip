// FP8 GEMM with per-row and per-column scales, the second reduction of the
// quantise-then-GEMM cascade ("RedFuser episode transcript", cue 33):
//   C[i][j] = bf16( s_i * t_j * sum_k Aq[i][k] * Bq[j][k] ),
// e4m3 operands, fp32 accumulation on v_mfma_f32_32x32x64_f8f6f4.
//
// Both operands are K-contiguous (A is [M, K], B is [N, K]), which is exactly
// the per-lane layout of the MFMA operands. Workgroup tile 256 x 256, four
// waves of 128 x 128 (16 accumulator blocks of 32 x 32 each). K is staged 64
// bytes at a time through a ring of four LDS stages filled by buffer loads
// straight into LDS (no staging registers; rows past M or N read as 0), three
// stages ahead of the MFMAs so HBM/L2 latency is covered. The 16-byte chunks of
// each 64-byte LDS row are XOR-swizzled by the row so the operand reads of
// consecutive lanes use distinct banks. The scales are applied once, in the
// epilogue.
#include "rf_device.hpp"
#include "rf_launch.hpp"

#include <type_traits>

namespace rf {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kStages = 4;
constexpr int kTileBytes = BM * BK;          // 16 KB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;  // A + B
constexpr int kGroupM = 4;                   // tile rows per band of the tile order

typedef __attribute__((address_space(3))) void lds_void;

// ds_read_b128 serves 16 lanes per LDS cycle (64 banks of 4 bytes). The operand
// read of 16 consecutive lanes touches 16 consecutive rows: rows r and r + 4
// share banks unless their chunks differ, which the XOR with (row >> 2) & 3
// guarantees over any 16 aligned rows.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // Operand formats 0 / 0 = e4m3 for A and B; no block scaling.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Tile order. Workgroups are dealt to the 8 XCDs round-robin, so workgroup b is
// first renumbered to give each XCD a contiguous run of tile ids; the ids then
// walk bands of kGroupM tile rows column by column. A run of 32 ids on a
// 16 x 16 tile grid is a 4 x 8 block of C, whose operand rows (4 + 8 tiles)
// are what that XCD's L2 has to hold per K step.
__device__ __forceinline__ void tile_of(int b, int ntm, int ntn, int& tm, int& tn) {
  const int T = ntm * ntn;
  const int t = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  const int first = (t / (kGroupM * ntn)) * kGroupM;
  const int rows = min(kGroupM, ntm - first);
  const int r = t - first * ntn;
  tm = first + r % rows;
  tn = r / rows;
}

template <int V>
using ic = std::integral_constant<int, V>;

__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(const uint8_t* __restrict__ aq,
                                                          const float* __restrict__ sa,
                                                          const uint8_t* __restrict__ bq,
                                                          const float* __restrict__ sb, int M,
                                                          int N, int K,
                                                          uint16_t* __restrict__ c, int vec) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- HBM -> LDS: per stage and operand, wave w fills four 1 KB blocks
  // (16 rows of 64 B); lane l writes row 16 (4 w + i) + l / 4, physical chunk
  // l % 4, so it fetches logical chunk (l % 4) ^ swz(row).
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(aq + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K));
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(bq + (size_t)n0 * K, (uint32_t)(min(BN, N - n0) * K));
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * (4 * wave + i) + (lane >> 2);
    const int chunk = (lane & 3) ^ swz(row);
    voff[i] = row * K + 16 * chunk;
  }
  auto issue = [&](int kt) {
    char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void*)(st + (4 * wave + i) * 1024), 16,
                                               voff[i], kt * BK, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void*)(st + kTileBytes + (4 * wave + i) * 1024),
                                               16, voff[i], kt * BK, 0, 0);
    }
  };
  // Wait until this wave's loads of a stage have landed while `newer` later
  // stages (8 loads each) may stay in flight.
  auto wait_stage = [](int newer) {
    if (newer >= 3)
      asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (newer == 2)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (newer == 1)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // ---- LDS -> registers. Fragment f of a step: f < 4 is B rows wn*128 + 32 f + li,
  // f >= 4 is A rows wm*128 + 32 (f - 4) + li; each is 32 bytes of K (logical
  // chunks 2 half and 2 half + 1), read as two 16-byte halves.
  const int half = lane >> 5, li = lane & 31;
  int fo[8][2];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      fo[f][h] = (f < 4) ? kTileBytes + lds_off(wn * 128 + 32 * f + li, 2 * half + h)
                         : lds_off(wm * 128 + 32 * (f - 4) + li, 2 * half + h);
  u32x4 fr[2][8][2];  // two fragment sets: the step being multiplied and the next
  auto read_half = [&](u32x4 (&set)[8][2], const char* st, int t) {
    set[t >> 1][t & 1] = *reinterpret_cast<const u32x4*>(st + fo[t >> 1][t & 1]);
  };
  auto frag = [](const u32x4 (&p)[2]) {
    return i32x8{(int)p[0][0], (int)p[0][1], (int)p[0][2], (int)p[0][3],
                 (int)p[1][0], (int)p[1][1], (int)p[1][2], (int)p[1][3]};
  };

  // acc[i][j] holds the 32 x 32 block (A rows 32 i, B rows 32 j) transposed:
  // the MFMA takes B as its first operand, so a lane holds one row of C
  // (A row li) and 16 of its columns, four consecutive ones per group of four
  // registers, which makes the epilogue's stores 8 bytes wide.
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  // One K step: 16 MFMAs on fragment set CUR; when READ, the 16 halves of the
  // next step's fragments are read into set 1 - CUR, one after each MFMA, from
  // the stage the loads made visible at the barrier above them.
  auto step = [&](auto cur_c, auto read_c, int kt) {
    constexpr int CUR = decltype(cur_c)::value;
    constexpr bool READ = decltype(read_c)::value != 0;
    const char* nst = smem + ((kt + 1) % kStages) * kStageBytes;
    if constexpr (READ) {
      wait_stage(min(2, nk - 2 - kt));
      lds_barrier();
      if (kt + 4 < nk) issue(kt + 4);  // refills the stage step kt - 1 read
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = t >> 2, j = t & 3;
      acc[i][j] = mfma_fp8(frag(fr[CUR][j]), frag(fr[CUR][4 + i]), acc[i][j]);
      if constexpr (READ) read_half(fr[1 - CUR], nst, t);
    }
    if constexpr (READ) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
    }
  };

  for (int s = 0; s < 4 && s < nk; ++s) issue(s);
  wait_stage(min(3, nk - 1));
  lds_barrier();
#pragma unroll
  for (int t = 0; t < 16; ++t) read_half(fr[0], smem, t);

  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    step(ic<0>{}, ic<1>{}, kt);
    step(ic<1>{}, ic<1>{}, kt + 1);
  }
  if (kt + 1 < nk) {
    step(ic<0>{}, ic<1>{}, kt);
    step(ic<1>{}, ic<0>{}, kt + 1);
  } else {
    step(ic<0>{}, ic<0>{}, kt);
  }

  // Epilogue: lane holds C row m0 + wm*128 + 32 i + li, columns
  // n0 + wn*128 + 32 j + 8 g + 4 half + (0..3) in registers 4 g .. 4 g + 3.
  // vec: N % 4 == 0, c 8-byte and the column scales 16-byte aligned.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + 32 * i + li;
    if (row >= M) continue;
    const float si = sa[row];
    uint16_t* crow = c + (size_t)row * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * 128 + 32 * j + 8 * g + 4 * half;
        if (vec && col + 3 < N) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(sb + col);
          const uint32_t lo = pack_bf16x2(acc[i][j][4 * g] * si * t[0], acc[i][j][4 * g + 1] * si * t[1]);
          const uint32_t hi = pack_bf16x2(acc[i][j][4 * g + 2] * si * t[2], acc[i][j][4 * g + 3] * si * t[3]);
          *reinterpret_cast<u32x2*>(crow + col) = u32x2{lo, hi};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < N)
              crow[col + e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i][j][4 * g + e] * si * sb[col + e]));
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp8_scaled(const uint8_t* a_q, const float* a_scale, const uint8_t* b_q,
                                  const float* b_scale, int M, int N, int K, void* c,
                                  hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int vec = (N % 4 == 0) && (reinterpret_cast<uintptr_t>(c) % 8 == 0) &&
                  (reinterpret_cast<uintptr_t>(b_scale) % 16 == 0);
  hipLaunchKernelGGL(gemm_fp8_kernel, dim3(tiles), dim3(256), 0, stream, a_q, a_scale, b_q,
                     b_scale, M, N, K, static_cast<uint16_t*>(c), vec);
  return hipGetLastError();
}

}  // namespace rf
