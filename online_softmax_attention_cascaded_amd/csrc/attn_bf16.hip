// bf16 attention forward for head size 128 on gfx950 MFMA.
//
// One pass over 64-key tiles of K and V per block of 128 query rows, with a
// running max m, running denominator l and an fp32 accumulator per row; when a
// tile raises the max the state is rescaled by exp(m_old - m_new), and the
// accumulator is divided by l once at the end ("RedFuser episode transcript",
// cues 15-19). Both contractions run on v_mfma_f32_32x32x16_bf16.
//
// Layout choices (CDNA4, wave64):
//  * Scores are computed transposed, S^T = K Q^T, so each lane owns ONE query
//    row (lane & 31) and 32 of the tile's keys; the softmax statistics and the
//    rescale of the output are then lane-local, and the probabilities already
//    sit in the B-operand layout of the second product O^T = V^T P^T.
//  * The second product needs V with keys contiguous per lane, so V tiles are
//    written into LDS transposed (Vt[d][key]). Keys are stored in the order the
//    MFMA k-slots expect (bits 2 and 3 of the key index swapped), so each lane
//    reads its 8 keys with one 16-byte LDS read.
//  * K tiles stay row-major in LDS with the 16-byte chunk index XOR-swizzled by
//    the row, and Vt rows are swizzled the same way, so the 16-byte operand
//    reads of consecutive lanes fall in distinct banks.
//  * Tiles are double-buffered in LDS: the global loads of tile t+1 are issued
//    before tile t is computed and written to the other buffer afterwards.
//  * Workgroups of one (batch, head) are placed on the same XCD (workgroups are
//    dealt round-robin to the 8 XCDs), so its K/V stream is shared in one L2.
//    Causal blocks are issued longest first.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int D = 128;
constexpr int BM = 128;  // query rows per workgroup, 32 per wave
constexpr int BN = 64;   // keys per tile
constexpr int kKBytes = BN * D * 2;
constexpr int kStage = 2 * kKBytes;  // K tile + transposed V tile

__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}
__device__ __forceinline__ int vt_off(int d, int pos) {
  const int swz = (d ^ (d >> 3)) & 7;
  return d * 128 + (((pos >> 3) ^ swz) << 4) + ((pos >> 2) & 1) * 8;
}
// Position of key k (0..63) inside a transposed V row: bits 2 and 3 swapped.
__device__ __forceinline__ int key_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int BH,
    int Hq, int Hkv, int Lq, int Lk, float c, int nqb) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  // Workgroup -> (batch*head, query block).
  const int id = blockIdx.x;
  int bh, qb;
  if ((BH & 7) == 0) {
    const int x = id & 7, j = id >> 3;
    bh = (j / nqb) * 8 + x;
    qb = j % nqb;
  } else {
    bh = id / nqb;
    qb = id % nqb;
  }
  if (CAUSAL) qb = nqb - 1 - qb;
  const int b = bh / Hq, h = bh - b * Hq, hk = h / (Hq / Hkv);
  const int q0 = qb * BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, li = lane & 31;
  const int qrow = q0 + wave * 32 + li;
  const int wave_last_row = q0 + wave * 32 + 31;

  const uint16_t* qp = q + (size_t)bh * Lq * D;
  const uint16_t* kp = k + (size_t)(b * Hkv + hk) * Lk * D;
  const uint16_t* vp = v + (size_t)(b * Hkv + hk) * Lk * D;

  // Q^T as the B operand of S^T = K Q^T: lane holds q row `li`, d = 16*ds + 8*g + [0, 8).
  bf16x8 qf[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < Lq) w = *reinterpret_cast<const u32x4*>(qp + (size_t)qrow * D + 16 * ds + 8 * g);
    qf[ds] = __builtin_bit_cast(bf16x8, w);
  }

  const int kend = CAUSAL ? min(Lk, q0 + BM) : Lk;
  const int ntiles = (kend + BN - 1) / BN;

  // Global -> register staging of one tile.
  const int lc = tid & 15;    // 16-byte chunk of a 256-byte row
  const int lr = tid >> 4;    // K: row lr + 16*i ; V: keys 4*lr + j
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
    const int t0 = t * BN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(t0 + lr + 16 * i, Lk - 1);
      kreg[i] = *reinterpret_cast<const u32x4*>(kp + (size_t)key * D + 8 * lc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(t0 + 4 * lr + j, Lk - 1);
      vreg[j] = *reinterpret_cast<const u32x4*>(vp + (size_t)key * D + 8 * lc);
    }
  };
  auto store_tile = [&](int buf) {
    char* kb = smem + buf * kStage;
    char* vb = kb + kKBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(kb + k_off(lr + 16 * i, lc)) = kreg[i];
    const int pos = key_pos(4 * lr);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a0 = vreg[0][e], a1 = vreg[1][e], a2 = vreg[2][e], a3 = vreg[3][e];
      const int d = 8 * lc + 2 * e;
      u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
      u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
      *reinterpret_cast<u32x2*>(vb + vt_off(d, pos)) = lo;
      *reinterpret_cast<u32x2*>(vb + vt_off(d + 1, pos)) = hi;
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf;  // running max of the raw dot products of row qrow
  float l_run = 0.f;      // running denominator relative to m_run * c (log2 units)

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) load_tile(t + 1);
    const int t0 = t * BN;
    const bool active = !CAUSAL || t0 <= wave_last_row;
    if (active) {
      const char* kb = smem + (t & 1) * kStage;
      const char* vb = kb + kKBytes;
      // ---- S^T = K Q^T for the tile's two 32-key blocks.
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kb + k_off(li, 2 * ds + g));
        const bf16x8 kb1 = *reinterpret_cast<const bf16x8*>(kb + k_off(32 + li, 2 * ds + g));
        s0 = mfma_bf16(ka, qf[ds], s0);
        s1 = mfma_bf16(kb1, qf[ds], s1);
      }
      // ---- mask: keys past Lk, and keys after the row when causal.
      const bool need_mask = (t0 + BN > Lk) || (CAUSAL && t0 + BN - 1 > q0 + wave * 32);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key0 = t0 + 8 * (r >> 2) + 4 * g + (r & 3);
          const int key1 = key0 + 32;
          if (key0 >= Lk || (CAUSAL && key0 > qrow)) s0[r] = kNegInf;
          if (key1 >= Lk || (CAUSAL && key1 > qrow)) s1[r] = kNegInf;
        }
      }
      // ---- online statistics of row qrow (its 64 scores are split over lanes li, li+32).
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run, mx);
      const float mc = (m_new == kNegInf) ? 0.f : m_new * c;
      const float alpha = fast_exp2(m_run * c - mc);  // 0 while m_run = -inf
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = fast_exp2(fmaf(s0[r], c, -mc));
        s1[r] = fast_exp2(fmaf(s1[r], c, -mc));
        rs += s0[r] + s1[r];
      }
      rs += __shfl_xor(rs, 32, kWave);
      l_run = alpha * l_run + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      // ---- P^T (bf16) in the B-operand layout: k-step ks uses registers 8*(ks&1) .. +7.
      bf16x8 pf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x16& src = (ks < 2) ? s0 : s1;
        const int base = 8 * (ks & 1);
        bf16x8 p;
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = (__bf16)src[base + j];
        pf[ks] = p;
      }
      // ---- O^T += V^T P^T.
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 va =
              *reinterpret_cast<const bf16x8*>(vb + vt_off(32 * db + li, 16 * ks + 8 * g));
          oacc[db] = mfma_bf16(va, pf[ks], oacc[db]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (bf16), lse = m + ln l.
  if (qrow < Lq) {
    const float inv = 1.f / l_run;
    uint16_t* orow = o + ((size_t)bh * Lq + qrow) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int d0 = 32 * db + 8 * mm + 4 * g;
        u32x2 w = {pack_bf16x2(oacc[db][4 * mm] * inv, oacc[db][4 * mm + 1] * inv),
                   pack_bf16x2(oacc[db][4 * mm + 2] * inv, oacc[db][4 * mm + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    }
    if (lse && g == 0) lse[(size_t)bh * Lq + qrow] = (m_run * c + __log2f(l_run)) * kLn2;
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
                                int causal, hipStream_t stream) {
  (void)d;
  const int nqb = (Lq + BM - 1) / BM;
  const int BH = B * Hq;
  const float c = scale * kLog2e;
  dim3 grid(BH * nqb);
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(o);
  if (causal)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<true>, grid, dim3(256), 0, stream, qq, kk, vv, oo, lse,
                       BH, Hq, Hkv, Lq, Lk, c, nqb);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<false>, grid, dim3(256), 0, stream, qq, kk, vv, oo,
                       lse, BH, Hq, Hkv, Lq, Lk, c, nqb);
  return hipGetLastError();
}

}  // namespace rf
