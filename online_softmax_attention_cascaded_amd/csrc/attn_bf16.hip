// bf16 attention forward for head size 128 on gfx950 MFMA.
//
// One pass over 64-key tiles of K and V per block of 128 query rows, with a
// running reference max m, running denominator l and an fp32 accumulator per
// row; when the reference moves the state is rescaled by exp(m_old - m_new),
// and the accumulator is divided by l once at the end ("RedFuser episode
// transcript", cues 15-19). Both contractions run on v_mfma_f32_32x32x16_bf16.
//
// Layout choices (CDNA4, wave64):
//  * Scores are computed transposed, S^T = K Q^T, so each lane owns ONE query
//    row (lane & 31) and 32 of the tile's keys; the softmax statistics and the
//    rescale of the output are then lane-local, and the probabilities already
//    sit in the B-operand layout of the second product O^T = V^T P^T.
//  * The second product needs V with keys contiguous per lane, so V tiles are
//    written into LDS transposed (Vt[d][key]); keys are stored in the order the
//    MFMA k-slots expect (bits 2 and 3 of the key index swapped), so each lane
//    reads its 8 keys with one 16-byte LDS read.
//  * LDS rows are XOR-swizzled (K: chunk ^ (row & 15) on 256-byte rows; Vt:
//    chunk ^ ((d ^ d >> 3) & 7) on 128-byte rows), so the 16-byte operand reads
//    of consecutive lanes, and the transposing 8-byte writes, spread over the
//    banks. All LDS addresses are loop-invariant registers plus immediate
//    offsets; the loop is unrolled by two so the double-buffer offset is an
//    immediate too.
//  * The reference max is moved only when a score exceeds it by more than 2^8
//    (in exp2 units), which is rare after the first tile; l and the accumulator
//    always share the same reference, so O = acc / l and lse = m + ln l are
//    exact whatever the reference.
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
constexpr float kTau = 8.f;          // lazy-rescale threshold, exp2 units

// Position of key k (0..63) inside a transposed V row: bits 2 and 3 swapped.
__device__ __forceinline__ int key_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
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

  // ---- global -> register staging of one tile (thread: 16-byte chunk lc of
  // K rows lr + 16 i, and of V keys 4 lr + j). Buffer loads: rows past Lk read 0
  // (they are masked out of the scores).
  const int lc = tid & 15, lr = tid >> 4;
  const uint32_t kv_bytes = (uint32_t)Lk * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, kv_bytes);
  const int kvo = (lr * D + 8 * lc) * 2;
  const int vvo = (4 * lr * D + 8 * lc) * 2;
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
    const int tb = t * BN * D * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) kreg[i] = buf_load16(krs, kvo, tb + i * 16 * D * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) vreg[j] = buf_load16(vrs, vvo, tb + j * D * 2);
  };

  // ---- lane-constant LDS offsets.
  // K write: row lr + 16 i, chunk lc ^ (row & 15) = lc ^ lr.
  const int kw = lr * 256 + ((lc ^ lr) << 4);
  // Vt write: rows d = 8 lc + jj (jj = 2e + hh), position key_pos(4 lr); the
  // chunk is swizzled by vt_swz(d) = (d ^ (d >> 3)) & 7, which differs across
  // the 8 values of lc that write the same jj together.
  const int vpos = key_pos(4 * lr);
  const int vch = vpos >> 3;
  const int vw = kKBytes + 8 * lc * 128 + ((vpos >> 2) & 1) * 8;
  int vwj[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) vwj[jj] = vw + jj * 128 + ((vch ^ ((jj ^ lc) & 7)) << 4);
  // K read (A operand): row li (+32 kb), chunk (2 ds + g) ^ (li & 15).
  int kr[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) kr[ds] = li * 256 + (((2 * ds + g) ^ (li & 15)) << 4);
  // Vt read (A operand of O^T = V^T P^T): row d = 32 db + li, chunk (2 ks + g) ^ vt_swz(d).
  int vr[4][4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = 32 * db + li, swz = (d ^ (d >> 3)) & 7;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) vr[db][ks] = kKBytes + d * 128 + (((2 * ks + g) ^ swz) << 4);
  }

  auto store_tile = [&](char* buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(buf + kw + i * 16 * 256) = kreg[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a0 = vreg[0][e], a1 = vreg[1][e], a2 = vreg[2][e], a3 = vreg[3][e];
      u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
      u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
      *reinterpret_cast<u32x2*>(buf + vwj[2 * e]) = lo;
      *reinterpret_cast<u32x2*>(buf + vwj[2 * e + 1]) = hi;
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_c = kNegInf;  // reference max of row qrow, in exp2 units (score * c)
  float l_run = 0.f;    // running denominator relative to m_c

  auto compute = [&](const char* buf, int t) {
    const int t0 = t * BN;
    // ---- S^T = K Q^T for the tile's two 32-key blocks.
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(buf + kr[ds]);
      const bf16x8 kb1 = *reinterpret_cast<const bf16x8*>(buf + kr[ds] + 32 * 256);
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
    // ---- tile max of row qrow (its 64 scores are split over lanes li, li+32).
    float mx = __builtin_fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = max3(mx, s0[r], s1[r]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mxc = mx * c;
    if (t == 0) {
      m_c = mxc;  // every row sees key 0, so this is finite
    } else if (__any(mxc > m_c + kTau)) {
      float alpha = 1.f;
      if (mxc > m_c + kTau) {
        alpha = fast_exp2(m_c - mxc);
        m_c = mxc;
      }
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
    }
    // ---- P^T (bf16) in the B-operand layout: k-step ks uses registers 8*(ks&1) .. +7
    // of s0 (ks < 2) or s1; the row sum stays in fp32 so lse keeps fp32 accuracy.
    bf16x8 pf[4];
    float rs = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x16& src = (ks < 2) ? s0 : s1;
      const int base = 8 * (ks & 1);
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(fmaf(src[base + 2 * j], c, -m_c));
        const float p1 = fast_exp2(fmaf(src[base + 2 * j + 1], c, -m_c));
        rs += p0 + p1;
        w[j] = pack_bf16x2(p0, p1);
      }
      pf[ks] = __builtin_bit_cast(bf16x8, w);
    }
    rs += __shfl_xor(rs, 32, kWave);
    l_run += rs;
    // ---- O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(buf + vr[db][ks]);
        oacc[db] = mfma_bf16(va, pf[ks], oacc[db]);
      }
    }
  };

  auto step = [&](char* cur, char* nxt, int t) {
    if (t + 1 < ntiles) load_tile(t + 1);
    if (!CAUSAL || t * BN <= wave_last_row) compute(cur, t);
    if (t + 1 < ntiles) store_tile(nxt);
    __syncthreads();
  };

  load_tile(0);
  store_tile(smem);
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(smem, smem + kStage, t);
    if (t + 1 < ntiles) step(smem + kStage, smem, t + 1);
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
    if (lse && g == 0) lse[(size_t)bh * Lq + qrow] = (m_c + __log2f(l_run)) * kLn2;
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
