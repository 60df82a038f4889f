// Split-KV decode partial states for fp32 K/V (Multi-Segment).
//
// The same states as the bf16 kernel: per (batch, query head, segment) the
// max m of the segment's scaled scores, l = sum exp(score - m) and the
// unnormalised acc = sum exp(score - m) v, built in one pass with the running
// (m, l, acc) rescaled by exp(m_old - m_new) when the max grows ("RedFuser
// episode transcript", cues 19, 21 and 39). Plain fp32 arithmetic (FMA):
// this path serves fp32 caches, where the contract is fp32 accuracy.
//
// One workgroup of 4 waves per (batch, key/value head, segment) streams the
// segment's K and V rows once for the whole GQA group; the kernel is compiled
// per group size rounded up to a power of two (GP), so its loops over heads
// are exact. The waves take interleaved 64-key chunks; in a chunk lane j owns
// key j for the scores (its K row in 16-byte loads, all issued before the
// FMAs that use them; the query rows are wave-uniform), the chunk's max and
// sum per head are wave reductions, and the probabilities go through LDS to
// the product with V, where each lane owns D / 64 columns of V rows read
// eight keys ahead (four probabilities per LDS read). The four waves' states
// are merged at the end by the same rule that merges segments.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int NW = 4;        // waves per workgroup
constexpr int CH = 64;       // keys per chunk (one per lane)
constexpr int MAXG = 16;     // query heads per key/value head

template <int D, int GP>
__global__ __launch_bounds__(256) void decode_split_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ part_acc, int Hq,
    int Hkv, int Lk, int S, int seg_len, float scale) {
  constexpr int NC = D / 64;  // output columns per lane
  __shared__ float qs[MAXG][D];  // used for 8 or 16 heads only
  __shared__ float ps[NW][MAXG][CH];
  __shared__ float sm_m[NW][MAXG], sm_l[NW][MAXG];
  __shared__ float sm_acc[NW][MAXG][D];

  const int s = blockIdx.x % S;
  const int bhk = blockIdx.x / S;  // b * Hkv + hk
  const int b = bhk / Hkv, hk = bhk - b * Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const int t0 = min(s * seg_len, Lk), t1 = min(t0 + seg_len, Lk);
  const int nchunks = (t1 - t0 + CH - 1) / CH;


  // The group's query rows: read straight from memory at wave-uniform
  // addresses (scalar loads, FMA operands from SGPRs) for up to 4 heads; from
  // LDS for 8 or 16 heads, whose rows do not fit the scalar registers.
  const float* const qg = q + ((size_t)b * Hq + hk * G) * D;
  if constexpr (GP >= 8) {
    for (int i = tid; i < GP * D; i += 256) {
      const int h = i / D, d = i - h * D;
      qs[h][d] = (h < G) ? qg[h * D + d] : 0.f;
    }
    __syncthreads();
  }
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (size_t)bhk * Lk * D, (uint32_t)Lk * D * 4);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + (size_t)bhk * Lk * D, (uint32_t)Lk * D * 4);
  constexpr int PVU = 8;

  float m_run[GP], l_run[GP], acc[GP][NC];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) acc[h][cc] = 0.f;
  }

  for (int ch = wave; ch < nchunks; ch += NW) {
    const int kbase = t0 + ch * CH;
    const int key = kbase + lane;
    const bool valid = key < t1;
    // ---- scores of key `key` against the group's query rows
    float sc[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) sc[h] = 0.f;
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const u32x4 w = buf_load16(krs, (int)((uint32_t)key * (D * 4) + 16 * d4), 0);
      const f32x4 kv = __builtin_bit_cast(f32x4, w);
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (h < G) {
          const f32x4 qv = (GP >= 8) ? *reinterpret_cast<const f32x4*>(&qs[h][4 * d4])
                                     : *reinterpret_cast<const f32x4*>(qg + h * D + 4 * d4);
          sc[h] = fmaf(qv[0], kv[0], sc[h]);
          sc[h] = fmaf(qv[1], kv[1], sc[h]);
          sc[h] = fmaf(qv[2], kv[2], sc[h]);
          sc[h] = fmaf(qv[3], kv[3], sc[h]);
        }
      }
    }
    // ---- online update per head
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h < G) {
        const float x = valid ? sc[h] * scale : kNegInf;
        const float m_new = fmaxf(m_run[h], wave_max(x));
        const float mr = (m_new == kNegInf) ? 0.f : m_new;  // all scores -inf so far: every p is 0
        const float alpha = (m_run[h] == kNegInf) ? 0.f : fast_exp2((m_run[h] - mr) * kLog2e);
        const float p = fast_exp2((x - mr) * kLog2e);  // 0 for a masked key
        l_run[h] = alpha * l_run[h] + wave_sum(p);
        m_run[h] = m_new;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) acc[h][cc] *= alpha;
        ps[wave][h][lane] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();  // the wave's own p row is read back by every lane
    // ---- acc += P V: lane owns columns cc * 64 + lane
    const int nk = min(CH, t1 - kbase);
    // eight keys' V values in flight at a time; keys past the segment are
    // skipped (their weight is 0, and 0 * v must not touch v)
    for (int j0 = 0; j0 < nk; j0 += PVU) {
      float vv[PVU][NC];
#pragma unroll
      for (int u = 0; u < PVU; ++u)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
          vv[u][cc] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
              vrs, (int)(((uint32_t)(kbase + j0 + u) * D + cc * 64 + lane) * 4u), 0, 0));
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (h < G) {
#pragma unroll
          for (int u4 = 0; u4 < PVU / 4; ++u4) {
            const f32x4 p4 = *reinterpret_cast<const f32x4*>(&ps[wave][h][j0 + 4 * u4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int u = 4 * u4 + e;
              if (j0 + u < nk) {
#pragma unroll
                for (int cc = 0; cc < NC; ++cc) acc[h][cc] = fmaf(p4[e], vv[u][cc], acc[h][cc]);
              }
            }
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();  // reads of p finish before the next chunk rewrites it
  }

  // ---- merge the four waves' states (the rule that merges segments)
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    if (h < G) {
      if (lane == 0) {
        sm_m[wave][h] = m_run[h];
        sm_l[wave][h] = l_run[h];
      }
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) sm_acc[wave][h][cc * 64 + lane] = acc[h][cc];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx - h * D;
    float mw[NW], ms = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = sm_m[w][h];
      ms = fmaxf(ms, mw[w]);
    }
    // No shortcut for ms = -inf: every weight is then 0, and 0 * l keeps a NaN
    // that reached l.
    float l = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = (mw[w] == kNegInf) ? 0.f : fast_exp2((mw[w] - ms) * kLog2e);
      l += wt * sm_l[w][h];
      a += wt * sm_acc[w][h][d];
    }
    const size_t row = ((size_t)b * Hq + hk * G + h) * S + s;
    part_acc[row * D + d] = a;
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
  const int G = Hq / Hkv;
#define RF_DEC32(D_, GP_)                                                                           \
  hipLaunchKernelGGL((decode_split_f32_kernel<D_, GP_>), grid, dim3(256), 0, stream, q, k, v, part_m, \
                     part_l, part_acc, Hq, Hkv, Lk, S, seg_len, scale)
#define RF_DEC32_G(D_)                    \
  if (G <= 1) RF_DEC32(D_, 1);            \
  else if (G <= 2) RF_DEC32(D_, 2);       \
  else if (G <= 4) RF_DEC32(D_, 4);       \
  else if (G <= 8) RF_DEC32(D_, 8);       \
  else RF_DEC32(D_, 16)
  if (d == 64) {
    RF_DEC32_G(64);
  } else {
    RF_DEC32_G(128);
  }
#undef RF_DEC32_G
#undef RF_DEC32
  return hipGetLastError();
}

}  // namespace rf

