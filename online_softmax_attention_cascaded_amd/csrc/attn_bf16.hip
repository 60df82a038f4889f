// bf16 attention forward for head sizes 64 and 128 on gfx950 MFMA.
//
// One pass over 64-key tiles of K and V per block of 128 query rows, with a
// running reference max m, running denominator l and an fp32 accumulator per
// row; when the reference moves the state is rescaled by exp(m_old - m_new),
// and the accumulator is divided by l once at the end ("RedFuser episode
// transcript", cues 15-19). Both contractions run on v_mfma_f32_32x32x16_bf16.
//
// Layout and schedule (CDNA4, wave64):
//  * Scores are computed transposed, S^T = K Q^T, so each lane owns ONE query
//    row (lane & 31) and 32 of the tile's keys; the softmax statistics and the
//    rescale of the output are lane-local, and the probabilities already sit
//    in the B-operand layout of the second product O^T = V^T P^T.
//  * K and V tiles go from HBM straight into LDS (buffer loads with the LDS
//    flag: no staging registers, rows past the end read as 0), row-major with
//    the 16-byte chunks XOR-swizzled by the row so operand reads spread over the
//    banks. V^T operands are read with the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16), four keys of one column per lane per read.
//  * K runs one tile ahead of V: while the softmax of tile t runs on the VALU,
//    the scores of tile t+1 are already being computed on the matrix cores.
//    Two LDS buffers per operand; one barrier per tile.
//  * The reference max is moved only when a score exceeds it by more than 8 (in
//    exp2 units: a probability above 2^8), which is rare after the first tile;
//    l and the accumulator always share the same reference, so O = acc / l and
//    lse = m + ln l are exact whatever the reference. The per-tile row max is
//    only taken when a lane's probability sum shows that the bound may have
//    been crossed.
//  * Workgroups of one (batch, head) are placed on the same XCD (workgroups are
//    dealt round-robin to the 8 XCDs), so its K/V stream is shared in one L2.
//    A causal workgroup takes query blocks u and nqb-1-u one after the other,
//    so all causal workgroups have the same number of key tiles.
#include "rf_device.hpp"
#include "rf_launch.hpp"

#include <type_traits>

namespace rf {
namespace {

constexpr int BM = 128;                 // query rows per workgroup, 32 per wave
constexpr int BN = 64;                  // keys per tile
constexpr int kMaxTileBytes = BN * 128 * 2;  // 16 KB per operand tile at head size 128
constexpr float kTau = 8.f;             // lazy-rescale threshold, exp2 units
constexpr float kPmax = 256.f;          // 2^kTau: largest probability against the reference
constexpr int KA = 3;                   // K fragment reads run this many MFMAs ahead
constexpr int VA = 4;                   // V^T fragment reads run this many MFMAs ahead

typedef __attribute__((address_space(3))) void lds_void;

struct Scores {
  f32x16 s0, s1;  // keys 0..31 and 32..63 of the tile (accumulator layout)
};

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Geometry of one head size: rows of K and V are 2 D bytes, D / 8 chunks of
// 16 bytes. K's swizzle spreads the 16 consecutive rows that one operand read
// touches over all 256 bytes of the bank space; V's is even, so each 32-byte
// pair of chunks stays together for the transposing reads, and rows 8 and 16
// apart share it.
template <int D>
struct Geo {
  static constexpr int kRow = 2 * D;
  static constexpr int kTileBytes = BN * kRow;
  static constexpr int kChunks = D / 8;
  static constexpr int kRowsPerKB = 1024 / kRow;
  static constexpr int kLoads = kTileBytes / 1024 / 4;  // 1 KB loads per wave per tile
  static constexpr int ND = D / 16;                     // k-steps of the score product
  static constexpr int NDB = D / 32;                    // 32-column blocks of the output
  static constexpr int NSM = 2 * ND;                    // score MFMAs per tile
  static constexpr int NPV = 4 * NDB;                   // P V MFMAs per tile
  static __device__ __forceinline__ int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  static __device__ __forceinline__ int vswz(int row) { return D == 128 ? 2 * (row & 7) : 2 * (row & 3); }
};

// QX: the query bits go through (w & q_and) ^ q_xor (a scale <= 0); the
// positive-scale instances leave them as they are.
template <int D, bool CAUSAL, bool QX>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int BH,
    int Hq, int Hkv, int Lq, int Lk, float c, uint32_t q_and, uint32_t q_xor, int nqb) {
  using Gm = Geo<D>;
  constexpr int kRow = Gm::kRow, kTileBytes = Gm::kTileBytes, ND = Gm::ND, NDB = Gm::NDB;
  constexpr int NSM = Gm::NSM, NPV = Gm::NPV;
  // [K0 | K1 | V0 | V1], one tile each, sized for head size 128 (a size that
  // depends on the template argument keeps the host pass from emitting the
  // kernel). Arrays the lambdas below capture are sized for head size 128 for
  // the same reason; head size 64 uses their leading elements.
  __shared__ __attribute__((aligned(1024))) char smem[4 * kMaxTileBytes];

  // Workgroup -> (batch*head, work unit). A unit is one query block, or for
  // causal attention the pair of blocks u and nqb-1-u, so every unit has the
  // same number of key tiles. The longer block goes first, so the workgroups
  // of one head start on the same key tiles together and share them in L2
  // (the shorter block second re-reads its tiles: about 360 MB per launch
  // against 270 MB of operands; the other order fetched 477 MB).
  const int nunits = CAUSAL ? (nqb + 1) / 2 : nqb;
  const int id = blockIdx.x;
  int bh, unit;
  if ((BH & 7) == 0) {
    const int x = id & 7, j = id >> 3;
    bh = (j / nunits) * 8 + x;
    unit = j % nunits;
  } else {
    bh = id / nunits;
    unit = id % nunits;
  }
  const int b = bh / Hq, h = bh - b * Hq, hk = h / (Hq / Hkv);
  const int npass = (CAUSAL && 2 * unit + 1 != nqb) ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
  const int qb = !CAUSAL ? unit : (pass == 0 ? nqb - 1 - unit : unit);
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
  for (int ds = 0; ds < ND; ++ds) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < Lq) w = *reinterpret_cast<const u32x4*>(qp + (size_t)qrow * D + 16 * ds + 8 * g);
    if constexpr (QX) {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (w[e] & q_and) ^ q_xor;  // sign / zero of the scale
    }
    qf[ds] = __builtin_bit_cast(bf16x8, w);
  }

  const int kend = CAUSAL ? min(Lk, q0 + BM) : Lk;
  const int ntiles = (kend + BN - 1) / BN;

  // ---- HBM -> LDS. Each wave fills kLoads 1 KB blocks per tile; lane l writes
  // 16 bytes at block + 16 l, i.e. row blk * kRowsPerKB + l / kChunks, physical
  // chunk l % kChunks, so it fetches the logical chunk that the swizzle puts
  // there.
  const uint32_t kv_bytes = (uint32_t)Lk * kRow;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, kv_bytes);
  int kso[4], vso[4];
#pragma unroll
  for (int i = 0; i < Gm::kLoads; ++i) {
    const int row = (Gm::kLoads * wave + i) * Gm::kRowsPerKB + lane / Gm::kChunks;
    const int pc = lane % Gm::kChunks;
    kso[i] = row * kRow + ((pc ^ Gm::kswz(row)) << 4);
    vso[i] = row * kRow + ((pc ^ Gm::vswz(row)) << 4);
  }
  auto load_k = [&](int t, char* buf) {
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(buf + (Gm::kLoads * wave + i) * 1024),
                                               16, kso[i], t * kTileBytes, 0, 0);
  };
  auto load_v = [&](int t, char* buf) {
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(buf + (Gm::kLoads * wave + i) * 1024),
                                               16, vso[i], t * kTileBytes, 0, 0);
  };

  // ---- LDS -> registers.
  // K (A operand of S^T): row li (+32 kb), logical chunk 2 ds + g.
  int kr[8];
#pragma unroll
  for (int ds = 0; ds < ND; ++ds) kr[ds] = li * kRow + (((2 * ds + g) ^ Gm::kswz(li)) << 4);
  // V^T (A operand of O^T, lane = head-size column 32 db + li, k-slots 8 g..8 g+7).
  // The MFMA k-slots of k-step ks are, for lane half g, the keys
  // 16 ks + 4 g + {0..3} (slots 0..3) and 16 ks + 8 + 4 g + {0..3} (slots 4..7):
  // the layout of the score accumulator rows. One transposing read gives lane
  // i of a 16-lane group the four keys k0..k0+3 of column d0 + i, when lane j
  // of the group points at row k0 + j/4, columns d0 + 4 (j%4) .. +3.
  int vr[4];
  {
    const int j = lane & 15, G = (lane >> 4) & 1;
    const int row = 4 * g + (j >> 2);       // + 16 ks + 8 hh (immediates)
    const int x = Gm::vswz(row);            // swizzle of every row this lane reads
    const int cl = 2 * G + ((j >> 1) & 1);  // chunk within the 32-column block
#pragma unroll
    for (int db = 0; db < NDB; ++db) vr[db] = row * kRow + (((4 * db + cl) ^ x) << 4) + 8 * (j & 1);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_c = kNegInf;  // reference max of row qrow, in exp2 units (score * c)
  float l_run = 0.f;    // running denominator relative to m_c

  char* const K0 = smem;
  char* const K1 = smem + kTileBytes;
  char* const V0 = smem + 2 * kTileBytes;
  char* const V1 = smem + 3 * kTileBytes;
  auto active = [&](int t) { return !CAUSAL || t * BN <= wave_last_row; };

  // Scores of one tile: ND k-steps on two independent accumulators.
  auto scores = [&](const char* kb, Scores& s) {
    s.s0 = f32x16{};
    s.s1 = f32x16{};
#pragma unroll
    for (int ds = 0; ds < ND; ++ds) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kb + kr[ds]);
      const bf16x8 kb1 = *reinterpret_cast<const bf16x8*>(kb + kr[ds] + 32 * kRow);
      s.s0 = mfma_bf16(ka, qf[ds], s.s0);
      s.s1 = mfma_bf16(kb1, qf[ds], s.s1);
    }
  };

  // One tile: softmax of tile t (scores `cur`) and O += V(t) P(t), with the
  // scores of tile t+1 computed into `nxt` in the same instruction stream so
  // the matrix cores work while the exponentials run on the VALU (NEXT; a
  // causal wave's last tile leaves them out).
  auto tile = [&](auto next_c, int t, Scores& cur, Scores& nxt, const char* knext, const char* vb) {
    constexpr bool NEXT = decltype(next_c)::value;
    const int t0 = t * BN;
    const bool need_mask = (t0 + BN > Lk) || (CAUSAL && t0 + BN - 1 > q0 + wave * 32);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key0 = t0 + 8 * (r >> 2) + 4 * g + (r & 3);
        const int key1 = key0 + 32;
        if (key0 >= Lk || (CAUSAL && key0 > qrow)) cur.s0[r] = kNegInf;
        if (key1 >= Lk || (CAUSAL && key1 > qrow)) cur.s1[r] = kNegInf;
      }
    }
    // Row max (four independent max3 chains, then the two halves of the wave),
    // in exp2 units, and the move of the reference when some row's max exceeds
    // it by more than kTau: l and the accumulator are rescaled with it.
    auto row_max_c = [&]() {
      float m4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) m4[j] = __builtin_fmaxf(cur.s0[j], cur.s1[j]);
#pragma unroll
      for (int r = 4; r < 16; ++r) m4[r & 3] = max3(m4[r & 3], cur.s0[r], cur.s1[r]);
      return half_swap_max(__builtin_fmaxf(__builtin_fmaxf(m4[0], m4[1]), __builtin_fmaxf(m4[2], m4[3]))) * c;
    };
    auto move_reference = [&](float mxc) {
      if (!__any(mxc > m_c + kTau)) return false;
      float alpha = 1.f;
      if (mxc > m_c + kTau) {
        alpha = fast_exp2(m_c - mxc);
        m_c = mxc;
      }
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      return true;
    };
    // Tile 0 sets the reference (every row sees key 0, so it is finite). Later
    // tiles compute their probabilities against the current reference first,
    // without a max: a lane's probabilities are each at most their sum, so
    // while no lane's sum exceeds 2^kTau no score rose above the reference by
    // more than kTau and nothing has to move. Otherwise the max is taken, the
    // reference moved if needed and the probabilities recomputed (rare after
    // the first tiles).
    if (t == 0) m_c = row_max_c();
    // ---- one basic block: the NSM score MFMAs of tile t+1, each K fragment read
    // KA MFMAs ahead (the fences keep every read next to its MFMA), and the
    // probabilities of tile t (2 fma, 2 exp2, 1 bf16 pack, 2 adds per pair). The
    // compiler issues the exponentials after the score MFMAs; they overlap with
    // the other wave on the SIMD (steering them between the MFMAs measured no
    // faster). Then the 16 P V MFMAs, each with its two transposing V reads
    // issued VA MFMAs ahead.
    // The two waves on a SIMD belong to different workgroups and run the same
    // loop out of step. While one is in this block (score MFMAs interleaved
    // with the exponentials, the VALU-heavy part) it takes issue priority over
    // one in the P V block below, whose MFMAs then fill the gaps: 3 % faster
    // than equal priority (the reverse, or priority only for the VALU
    // instructions inside this block, measured slower).
    __builtin_amdgcn_s_setprio(1);
    if constexpr (NEXT) {
      nxt.s0 = f32x16{};
      nxt.s1 = f32x16{};
    }
    bf16x8 kf[KA + 1];
    auto kread = [&](int i) {
      return *reinterpret_cast<const bf16x8*>(knext + kr[i >> 1] + (i & 1) * 32 * kRow);
    };
#pragma unroll
    for (int i = 0; i < KA; ++i)
      if constexpr (NEXT) kf[i] = kread(i);
    u32x4 pw[4];
    float rs = 0.f;
    constexpr int EV = 16 / NSM;  // probability pairs per score MFMA
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (NEXT && i % EV == 0) {
        const int m = i / EV;
        if (m + KA < NSM) kf[(m + KA) % (KA + 1)] = kread(m + KA);
        if (m & 1)
          nxt.s1 = mfma_bf16(kf[m % (KA + 1)], qf[m >> 1], nxt.s1);
        else
          nxt.s0 = mfma_bf16(kf[m % (KA + 1)], qf[m >> 1], nxt.s0);
      }
      // probabilities 2i, 2i+1: k-step ks = i/4, pair jj = i%4 of P^T's B operand
      const int ks = i >> 2, jj = i & 3;
      const f32x16& src = (ks < 2) ? cur.s0 : cur.s1;
      const int e = 8 * (ks & 1) + 2 * jj;
      const float p0 = fast_exp2(fmaf(src[e], c, -m_c));
      const float p1 = fast_exp2(fmaf(src[e + 1], c, -m_c));
      rs += p0 + p1;
      pw[ks][jj] = pack_bf16x2(p0, p1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (t > 0 && __any(rs > kPmax) && move_reference(row_max_c())) {
      rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ks = i >> 2, jj = i & 3;
        const f32x16& src = (ks < 2) ? cur.s0 : cur.s1;
        const int e = 8 * (ks & 1) + 2 * jj;
        const float p0 = fast_exp2(fmaf(src[e], c, -m_c));
        const float p1 = fast_exp2(fmaf(src[e + 1], c, -m_c));
        rs += p0 + p1;
        pw[ks][jj] = pack_bf16x2(p0, p1);
      }
    }
    l_run += half_swap_sum(rs);
    // O^T += V^T P^T; consecutive MFMAs update different accumulators. MFMA i
    // (k-step i / NDB, d block i % NDB) takes its V^T operand from two
    // transposing reads issued VA MFMAs ahead; each MFMA waits for exactly its
    // own reads.
    const uint32_t va = lds_addr(vb);
    u32x4 vf[VA + 1];
    auto vread = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint32_t a = va + vr[i % NDB];
      const u32x2 lo = lds_read_tr16<(i / NDB) * 16 * kRow>(a);
      const u32x2 hi = lds_read_tr16<(i / NDB) * 16 * kRow + 8 * kRow>(a);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    __builtin_amdgcn_s_setprio(0);
    static_for<VA>([&](auto ic) { vf[decltype(ic)::value] = vread(ic); });
    static_for<NPV>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + VA < NPV) vf[(i + VA) % (VA + 1)] = vread(std::integral_constant<int, i + VA>{});
      // reads issued after MFMA i's own: two per later MFMA already in flight
      constexpr int later = (NPV - 1 - i) < VA ? (NPV - 1 - i) : VA;
      lds_wait_for<2 * later>(vf[i % (VA + 1)]);
      oacc[i % NDB] = mfma_bf16(__builtin_bit_cast(bf16x8, vf[i % (VA + 1)]),
                                __builtin_bit_cast(bf16x8, pw[i / NDB]), oacc[i % NDB]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Prologue: K(0), V(0), K(1) in LDS; scores of tile 0.
  load_k(0, K0);
  load_v(0, V0);
  if (ntiles > 1) load_k(1, K1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  Scores sa, sb;
  scores(K0, sa);
  lds_barrier();  // K0 is refilled below

  // Iteration t: LDS holds K(t+1) and V(t); it loads K(t+2) and V(t+1) into the
  // buffers that held K(t) and V(t-1), both consumed before the last barrier.
  // At the last tile the scores of the (absent) next tile are computed from
  // stale LDS data and never used, except in causal attention, where a wave
  // leaves out the scores of a tile it will not process (its last tile of
  // each query block: 1-2 % of the causal time, identical output; for the
  // non-causal kernel the second form raised register use into spills).
  auto iter = [&](int t, Scores& cur, Scores& nxt, char* kcur, char* knext, char* vcur,
                  char* vnext) {
    if (t + 2 < ntiles) load_k(t + 2, kcur);
    if (t + 1 < ntiles) load_v(t + 1, vnext);
    if (active(t)) {
      if constexpr (!CAUSAL) {
        tile(std::true_type{}, t, cur, nxt, knext, vcur);
      } else {
        if (t + 1 < ntiles && active(t + 1))
          tile(std::true_type{}, t, cur, nxt, knext, vcur);
        else
          tile(std::false_type{}, t, cur, nxt, knext, vcur);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
  };
  for (int t = 0; t < ntiles; t += 2) {
    iter(t, sa, sb, K0, K1, V0, V1);
    if (t + 1 < ntiles) iter(t + 1, sb, sa, K1, K0, V1, V0);
  }

  // ---- epilogue: O = acc / l (bf16), lse = m + ln l.
  if (qrow < Lq) {
    const float inv = 1.f / l_run;
    uint16_t* orow = o + ((size_t)bh * Lq + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
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
  }  // pass
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
                                int causal, hipStream_t stream) {
  const int nqb = (Lq + BM - 1) / BM;
  const int BH = B * Hq;
  const ScoreScale sc = score_scale(scale);
  dim3 grid(BH * (causal ? (nqb + 1) / 2 : nqb));
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(o);
  const bool qx = sc.q_and != ~0u || sc.q_xor != 0u;
#define RF_ATTN_LAUNCH(D_, C_)                                                                     \
  do {                                                                                            \
    if (qx)                                                                                       \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<D_, C_, true>), grid, dim3(256), 0, stream, qq, kk, \
                         vv, oo, lse, BH, Hq, Hkv, Lq, Lk, sc.c, sc.q_and, sc.q_xor, nqb);         \
    else                                                                                          \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<D_, C_, false>), grid, dim3(256), 0, stream, qq,  \
                         kk, vv, oo, lse, BH, Hq, Hkv, Lq, Lk, sc.c, sc.q_and, sc.q_xor, nqb);     \
  } while (0)
  if (d == 64) {
    if (causal) RF_ATTN_LAUNCH(64, true); else RF_ATTN_LAUNCH(64, false);
  } else {
    if (causal) RF_ATTN_LAUNCH(128, true); else RF_ATTN_LAUNCH(128, false);
  }
#undef RF_ATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace rf
