// FP8 GEMM with per-row and per-column scales, the second reduction of the
// quantise-then-GEMM cascade ("RedFuser episode transcript", cue 33):
//   C[i][j] = bf16( s_i * t_j * sum_k Aq[i][k] * Bq[j][k] ),
// e4m3 operands, fp32 accumulation on v_mfma_f32_32x32x64_f8f6f4.
//
// Both operands are K-contiguous (A is [M, K], B is [N, K]), which is exactly
// the per-lane layout of the MFMA operands, so tiles go from HBM to LDS with
// 16-byte loads and from LDS to registers with 16-byte reads and no shuffles.
// Workgroup tile 256 x 256, four waves of 128 x 128 (16 accumulator blocks of
// 32 x 32 each), K staged 64 bytes at a time through two LDS buffers; the
// 16-byte chunks of each 64-byte LDS row are XOR-swizzled by the row so the
// operand reads of consecutive lanes use distinct banks. The scales are applied
// once, in the epilogue.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kTileBytes = BM * BK;           // 16 KB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;   // A + B

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 3)) << 4);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // Operand formats 0 / 0 = e4m3 for A and B; no block scaling.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(const uint8_t* __restrict__ aq,
                                                          const float* __restrict__ sa,
                                                          const uint8_t* __restrict__ bq,
                                                          const float* __restrict__ sb, int M,
                                                          int N, int K,
                                                          uint16_t* __restrict__ c) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / ntn) * BM, n0 = (blockIdx.x % ntn) * BN;

  // Global -> LDS staging: thread owns chunk (tid & 3) of rows (tid >> 2) + 64 i.
  const int lc = tid & 3, lr = tid >> 2;
  u32x4 ra[4], rb[4];
  auto load = [&](int kt) {
    const int k0 = kt * BK + 16 * lc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ar = min(m0 + lr + 64 * i, M - 1), br = min(n0 + lr + 64 * i, N - 1);
      ra[i] = *reinterpret_cast<const u32x4*>(aq + (size_t)ar * K + k0);
      rb[i] = *reinterpret_cast<const u32x4*>(bq + (size_t)br * K + k0);
    }
  };
  auto store = [&](int buf) {
    char* as = smem + buf * kStageBytes;
    char* bs = as + kTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(as + lds_off(lr + 64 * i, lc)) = ra[i];
      *reinterpret_cast<u32x4*>(bs + lds_off(lr + 64 * i, lc)) = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  const int half = lane >> 5, li = lane & 31;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    const char* as = smem + (kt & 1) * kStageBytes;
    const char* bs = as + kTileBytes;
    i32x8 af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + 32 * i + li;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(as + lds_off(row, 2 * half));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(as + lds_off(row, 2 * half + 1));
      af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + 32 * j + li;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(bs + lds_off(row, 2 * half));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(bs + lds_off(row, 2 * half + 1));
      bf[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_fp8(af[i], bf[j], acc[i][j]);
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: lane holds column li of each 32 x 32 block, rows 8*(r/4) + 4*half + r%4.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 128 + 32 * j + li;
    if (col >= N) continue;
    const float tj = sb[col];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < M) {
          const float val = acc[i][j][r] * sa[row] * tj;
          c[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, (__bf16)val);
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
  hipLaunchKernelGGL(gemm_fp8_kernel, dim3(tiles), dim3(256), 0, stream, a_q, a_scale, b_q,
                     b_scale, M, N, K, static_cast<uint16_t*>(c));
  return hipGetLastError();
}

}  // namespace rf
