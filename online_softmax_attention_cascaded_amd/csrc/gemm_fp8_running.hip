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
// Workgroup tile 256 x 256, eight waves of 128 x 64 (two per SIMD: 128
// accumulator registers each, leaving room for the VALU rescale), with
// v_mfma_f32_32x32x64_f8f6f4 taking B first (a lane holds one row of C and four
// consecutive columns per register group). Per K step, the bf16 A tile (256
// rows x 128 bytes) and the e4m3 B tile (256 rows x 64 bytes) go HBM -> LDS by
// buffer loads to LDS, one step ahead. Then two lanes share each A row (32
// values each): abs-max (integer max on the bf16 magnitude bits, combined
// across the pair by v_permlane32_swap), the new scale, the rescale ratio
// (published in LDS), the codes (correctly rounded x / s by one Markstein
// correction of x * RN(1/s), hardware round-to-nearest-even e4m3 convert),
// written into an LDS code tile in the MFMA operand layout. After a barrier
// each wave rescales its accumulator rows if any ratio differs from 1 and
// runs the step's 8 MFMAs.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kABytes = BM * BK * 2;           // bf16 A tile, 32 KB
constexpr int kBBytes = BN * BK;               // e4m3 B tile, 16 KB
constexpr int kStageBytes = kABytes + kBBytes;  // 48 KB, two stages
constexpr int kCodeBytes = BM * BK;            // e4m3 A codes of the step, 16 KB

typedef __attribute__((address_space(3))) void lds_void;

// Operand tiles (64-byte rows, 16-byte chunks XOR (row >> 2) & 3): conflict-free
// for the 16-lane passes of ds_read_b128 (same layout as the final-scale GEMM).
__device__ __forceinline__ int op_off(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 2) & 3)) << 4);
}
// bf16 A tile (128-byte rows, 8 chunks): chunk XOR (row & 7), so one lane per
// row reading chunk c touches at most two rows per bank group.
__device__ __forceinline__ int a_off(int row, int chunk) {
  return row * (2 * BK) + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__global__ __launch_bounds__(512, 2) void gemm_fp8_running_kernel(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ bq, const float* __restrict__ sb,
    int M, int N, int K, float* __restrict__ a_scale, uint16_t* __restrict__ c, int vec) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageBytes + kCodeBytes];
  __shared__ float ratio_s[BM];
  __shared__ float scale_s[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;  // 128-row half, 64-column quarter
  const int ntn = (N + BN - 1) / BN;
  const int tm = blockIdx.x / ntn, tn = blockIdx.x % ntn;
  const int m0 = tm * BM, n0 = tn * BN;
  char* const codes = smem + 2 * kStageBytes;

  // ---- HBM -> LDS. A: wave w fills rows 32 w .. 32 w + 31, four 1 KB blocks of
  // 8 rows; lane l writes physical chunk l % 8 of row 8 i + l / 8. B: wave w
  // fills two 1 KB blocks of 16 rows (physical chunk l % 4 of row 16 i + l / 4).
  const __amdgpu_buffer_rsrc_t ars =
      make_rsrc(a + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K * 2));
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(bq + (size_t)n0 * K, (uint32_t)(min(BN, N - n0) * K));
  // Per-lane parts of the load offsets; the per-block parts are immediates.
  const int arow0 = 32 * wave + (lane >> 3), brow0 = 32 * wave + (lane >> 2);
  auto issue = [&](int kt) {
    char* st = smem + (kt & 1) * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = arow0 + 8 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void*)(st + (4 * wave + i) * 1024), 16,
                                               row * K * 2 + 16 * ((lane & 7) ^ (row & 7)),
                                               kt * BK * 2, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = brow0 + 16 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void*)(st + kABytes + (2 * wave + i) * 1024),
                                               16, row * K + 16 * ((lane & 3) ^ ((row >> 2) & 3)),
                                               kt * BK, 0, 0);
    }
  };

  // ---- quantiser state: lanes l and l + 32 of wave w share A row qr of the
  // tile; lane half qh takes columns 32 qh .. 32 qh + 31 (chunks 4 qh .. 4 qh + 3).
  const int qr = 32 * wave + (lane & 31), qh = lane >> 5;
  uint32_t amax_bits = 0;  // running abs-max as bf16 magnitude bits
  float s_run = 0.f;

  // ---- MFMA operands: fragment f < 4 is B rows wn*128 + 32 f + li, f >= 4 is
  // A code rows wm*128 + 32 (f - 4) + li; 32 bytes of K each.
  const int half = lane >> 5, li = lane & 31;
  // Fragment f, half h: f < 2 is B row wn*64 + 32 f + li in the stage, f >= 2
  // is A code row wm*128 + 32 (f - 2) + li in the code tile.
  auto fo = [&](int f, int h) {
    return (f < 2) ? kABytes + op_off(wn * 64 + 32 * f + li, 2 * half + h)
                   : 2 * kStageBytes + op_off(wm * 128 + 32 * (f - 2) + li, 2 * half + h);
  };
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // stage kt visible; every wave is done with the previous codes
    if (kt + 1 < nk) issue(kt + 1);
    const char* st = smem + (kt & 1) * kStageBytes;

    // ---- running abs-max, scale and codes of row qr for this K tile: one pass
    // over the row's 64 values for the abs-max, a second to quantise them (LDS
    // reads are cheap; keeping all 64 in registers would not fit beside the
    // accumulators).
    uint32_t tmax = 0;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(st + a_off(qr, 4 * qh + ch));
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = max(tmax, max(xv[e] & 0x7fffu, (xv[e] >> 16) & 0x7fffu));
    }
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(tmax, tmax, false, false);
      tmax = max((uint32_t)pr[0], (uint32_t)pr[1]);  // both lanes of the pair
    }
    const uint32_t anew_bits = max(amax_bits, tmax);
    const float s_new = __uint_as_float(anew_bits << 16) / 448.f;
    // The accumulator row holds the sum in units of s_run; it moves to s_new.
    if (qh == 0) ratio_s[qr] = (anew_bits > amax_bits && amax_bits != 0) ? s_run / s_new : 1.f;
    amax_bits = anew_bits;
    s_run = s_new;
    const float rcp = (s_new > 0.f) ? 1.f / s_new : 0.f;
#pragma unroll 1
    for (int cc = 2 * qh; cc < 2 * qh + 2; ++cc) {  // 16 values -> one 16-byte chunk of codes
      uint32_t w[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(st + a_off(qr, 2 * cc + hh));
        float y[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[2 * e] = bf16_lo(xv[e]);
          y[2 * e + 1] = bf16_hi(xv[e]);
        }
        if (rcp <= 3.4e38f) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float q0 = y[j] * rcp;
            const float r = fmaf(-s_new, q0, y[j]);
            y[j] = __builtin_copysignf(fmaf(r, rcp, q0), y[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = y[j] / s_new;
        }
        uint32_t lo = 0u, hi = 0u;
        if (s_new > 0.f) {
          lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo, true);
          hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
          hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)hi, true);
        }
        w[2 * hh] = lo;
        w[2 * hh + 1] = hi;
      }
      *reinterpret_cast<u32x4*>(codes + op_off(qr, cc)) = u32x4{w[0], w[1], w[2], w[3]};
    }
    lds_barrier();  // codes and ratios visible

    // ---- move the accumulator rows of this wave to the new scales.
    float rt[4];
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rt[i] = ratio_s[wm * 128 + 32 * i + li];
      grow |= rt[i] != 1.f;
    }
    if (__any(grow)) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] *= rt[i];
    }

    // ---- 8 MFMAs on the step's codes and B tile: the two B fragments once,
    // each A fragment just before its two MFMAs.
    auto frag = [&](const char* base, int f) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(base + fo(f, 0));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(base + fo(f, 1));
      return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    i32x8 fb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = frag(st, j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x8 fa = frag(smem, 2 + i);
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_fp8(fb[j], fa, acc[i][j]);
    }
  }

  // ---- final scales: s_final of each row (and A's scale output, written once
  // per row by the workgroups of the first column tile).
  if (qh == 0) {
    scale_s[qr] = s_run;
    if (tn == 0 && m0 + qr < M) a_scale[m0 + qr] = s_run;
  }
  lds_barrier();

  // Epilogue: lane holds C row m0 + wm*128 + 32 i + li, columns
  // n0 + wn*64 + 32 j + 8 g + 4 half + (0..3) in registers 4 g .. 4 g + 3.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lrow = wm * 128 + 32 * i + li;
    const int row = m0 + lrow;
    if (row >= M) continue;
    const float si = scale_s[lrow];
    uint16_t* crow = c + (size_t)row * N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * 64 + 32 * j + 8 * g + 4 * half;
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

hipError_t launch_gemm_fp8_running(const void* a, const uint8_t* b_q, const float* b_scale, int M,
                                   int N, int K, float* a_scale, void* c, hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int vec = (N % 4 == 0) && (reinterpret_cast<uintptr_t>(c) % 8 == 0) &&
                  (reinterpret_cast<uintptr_t>(b_scale) % 16 == 0);
  hipLaunchKernelGGL(gemm_fp8_running_kernel, dim3(tiles), dim3(512), 0, stream,
                     static_cast<const uint16_t*>(a), b_q, b_scale, M, N, K, a_scale,
                     static_cast<uint16_t*>(c), vec);
  return hipGetLastError();
}

}  // namespace rf
