// FP8 GEMM with per-row and per-column scales, the second reduction of the
// quantise-then-GEMM cascade ("RedFuser episode transcript", cue 33):
//   C[i][j] = bf16( s_i * t_j * sum_k Aq[i][k] * Bq[j][k] ),
// e4m3 operands, fp32 accumulation on v_mfma_f32_32x32x64_f8f6f4.
//
// Both operands are K-contiguous (A is [M, K], B is [N, K]), which is exactly
// the per-lane layout of the MFMA operands. Workgroup tile 256 x 256 (one per
// CU at 4096^2), sixteen waves of 64 x 64, four per SIMD, so one wave's wait
// on an LDS read or a barrier is covered by the MFMAs of the others. K is
// staged 128 bytes at a time through two LDS stages filled by buffer loads
// straight into LDS (no staging registers; rows past M or N read as 0): while
// the MFMAs of one stage run, the loads of the next fill the other, with one
// barrier per 128 bytes of K. A step reads its fragments from its own stage,
// in two k-substeps of 64 bytes. The 16-byte chunks of each 128-byte LDS row
// are XOR-swizzled by the row so the operand reads of consecutive lanes use
// distinct banks. The scales are applied once, in the epilogue, which stages
// the bf16 tile in LDS so that every row of C is written as whole 512-byte
// segments.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kStages = 2;
constexpr int kTileBytes = BM * BK;          // 32 KB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;  // A + B
constexpr int kGroupM = 4;                   // tile rows per band of the tile order
constexpr int kThreads = 1024;               // 16 waves

typedef __attribute__((address_space(3))) void lds_void;

// ds_read_b128 serves 16 lanes per LDS cycle (64 banks of 4 bytes). The operand
// read of 16 consecutive lanes touches 16 consecutive rows at one logical
// chunk. A 128-byte row spans half the banks, so rows r and r + 1 sit in
// different halves; the XOR with (row >> 1) & 7 gives the 8 row pairs of any
// 16 aligned rows 8 different chunks, i.e. distinct 4-bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
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

__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(const uint8_t* __restrict__ aq,
                                                          const float* __restrict__ sa,
                                                          const uint8_t* __restrict__ bq,
                                                          const float* __restrict__ sb, int M,
                                                          int N, int K,
                                                          uint16_t* __restrict__ c, int vec8) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;   // 16 waves
  const int wm = wave >> 2, wn = wave & 3;                          // 4 x 4 waves of 64 x 64
  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // HBM -> LDS: per stage and operand, wave w fills two 1 KB blocks (8 rows of
  // 128 B each); lane l writes row 8 b + l / 8 of block b at physical chunk
  // l % 8, so it fetches the logical chunk that the swizzle puts there.
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(aq + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K));
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(bq + (size_t)n0 * K, (uint32_t)(min(BN, N - n0) * K));
  int voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (2 * wave + i) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    voff[i] = row * K + 16 * chunk;
  }
  auto issue = [&](int kt) {
    char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void*)(st + (2 * wave + i) * 1024), 16, voff[i],
                                               kt * BK, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void*)(st + kTileBytes + (2 * wave + i) * 1024), 16,
                                               voff[i], kt * BK, 0, 0);
    }
  };
  // Wait until this wave's loads of a stage have landed while `newer` later
  // stages (4 loads each) may stay in flight.
  auto wait_stage = [](int newer) {
    if (newer >= 1)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // Fragments of a step, read from that step's stage: B blocks j (rows
  // wn*64 + 32 j + li) and A blocks i (rows wm*64 + 32 i + li); in k-substep q
  // each is 32 bytes of K (logical chunks 4 q + 2 half and 4 q + 2 half + 1)
  // read as two 16-byte halves.
  const int half = lane >> 5, li = lane & 31;
  int bo[2][2][2], ao[2][2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < 2; ++j) bo[q][j][h] = kTileBytes + lds_off(wn * 64 + 32 * j + li, 4 * q + 2 * half + h);
#pragma unroll
    for (int i = 0; i < 2; ++i) ao[q][i][h] = lds_off(wm * 64 + 32 * i + li, 4 * q + 2 * half + h);
  }
  auto rd = [](const char* st, int off) { return *reinterpret_cast<const u32x4*>(st + off); };
  auto frag = [](const u32x4& p0, const u32x4& p1) {
    return i32x8{(int)p0[0], (int)p0[1], (int)p0[2], (int)p0[3],
                 (int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3]};
  };

  // acc[i][j] holds the 32 x 32 block (A rows 32 i, B rows 32 j) transposed:
  // the MFMA takes B as its first operand, so a lane holds one row of C (A row
  // li) and 16 of its columns, four consecutive ones per group of four registers.
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    // This wave's loads of stage kt have landed; after the barrier everyone's
    // have, and everyone is done with stage kt-1, whose slot takes stage kt+1.
    wait_stage(0);
    lds_barrier();
    const char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 b0[2], b1[2], a[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        b0[h] = rd(st, bo[q][0][h]);
        a[0][h] = rd(st, ao[q][0][h]);
        b1[h] = rd(st, bo[q][1][h]);
        a[1][h] = rd(st, ao[q][1][h]);
      }
      // the next stage's loads go out behind the first fragment reads, so
      // those reads do not queue behind them (1 % in A/B, identical output)
      if (q == 0) {
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) issue(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        acc[i][0] = mfma_fp8(frag(b0[0], b0[1]), frag(a[i][0], a[i][1]), acc[i][0]);
        acc[i][1] = mfma_fp8(frag(b1[0], b1[1]), frag(a[i][0], a[i][1]), acc[i][1]);
      }
    }
  }

  // Epilogue through LDS: the scaled bf16 tile (256 x 256, 512 B per row, the
  // 16-byte chunks of row r XOR-swizzled by r & 31) replaces the stage ring,
  // then every wave stores 16 whole rows, 32 lanes x 16 B per row.
  lds_barrier();   // everyone is done with the last stage
  char* const ct = smem;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tr = wm * 64 + 32 * i + li;     // tile row
    const int row = m0 + tr;
    const float si = row < M ? sa[row] : 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int tc = wn * 64 + 32 * j + 8 * g + 4 * half;   // tile column
        const int col = n0 + tc;
        float t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (col + e < N) ? sb[col + e] : 0.f;
        const uint32_t lo = pack_bf16x2(acc[i][j][4 * g] * si * t[0], acc[i][j][4 * g + 1] * si * t[1]);
        const uint32_t hi = pack_bf16x2(acc[i][j][4 * g + 2] * si * t[2], acc[i][j][4 * g + 3] * si * t[3]);
        const int chunk = (tc >> 3) ^ (tr & 31);
        *reinterpret_cast<u32x2*>(ct + tr * 512 + chunk * 16 + (tc & 7) * 2) = u32x2{lo, hi};
      }
    }
  }
  lds_barrier();
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int tr = 16 * wave + 2 * r + (lane >> 5);
    const int row = m0 + tr;
    const int tc = 8 * (lane & 31);
    const int col = n0 + tc;
    if (row >= M) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ct + tr * 512 + (((tc >> 3) ^ (tr & 31)) * 16));
    uint16_t* dst = c + (size_t)row * N + col;
    if (vec8 && col + 7 < N) {
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp8_scaled(const uint8_t* a_q, const float* a_scale, const uint8_t* b_q,
                                  const float* b_scale, int M, int N, int K, void* c,
                                  hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int vec8 = (N % 8 == 0) && (reinterpret_cast<uintptr_t>(c) % 16 == 0);
  hipLaunchKernelGGL(gemm_fp8_kernel, dim3(tiles), dim3(kThreads), 0, stream, a_q, a_scale, b_q,
                     b_scale, M, N, K, static_cast<uint16_t*>(c), vec8);
  return hipGetLastError();
}

}  // namespace rf

