// Variance and moment of inertia of rows of 4 .. 8192 fp32 values: the cascade
// "centre (mean, or centre of mass) -> centred second moment", fused into one
// pass at the thread, wave or workgroup level of the reduction tree, beside the
// unfused two-pass cascade ("RedFuser episode transcript", cue 47 names these
// cascades; cue 17 states the incremental form: correct the running state for
// the changed earlier result, then add the tile's term).
//
// State of a set of points (w_i, x_i): total mass W, centre c and
// I = sum w_i (x_i - c)^2. When a tile (mass W_t, first moment S_t) arrives,
// the centre moves to c' = c + (S_t - W_t c) / (W + W_t); the state's I is
// corrected by W (c - c')^2 (the earlier points' squared distances are now
// taken about c'), and the tile's own sum of w (x - c')^2 is added. Two states
// merge the same way, the shift term being W_a W_b / (W_a + W_b) (c_b - c_a)^2.
// Variance is the case w = 1 (var = I / n).
//
// Positions enter shifted by the row's first value x_0 (y = x - x_0, exact
// when x is within a factor 2 of x_0): the sums then stay of the order of the
// spread, not of the offset, and the centre is x_0 + c at the end. All forms,
// the unfused one included, work on the shifted positions.
//
// Mappings. Thread and wave level: one wave per row (4 rows per workgroup);
// lane l holds the 16-byte chunks l + 64 j of its row. Block level: one
// workgroup per row, thread t holds chunks t + 256 j. The fused forms load the
// whole row once through buffer loads with the streaming cache policy (chunks
// past the row read as 0 with no memory traffic and carry no mass). Unfused: one kernel for the centre, a
// second one for the centred sum, each reading the row.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

struct Moments {
  float W, c, I;
};

__device__ __forceinline__ float rcp_or_zero(float w) { return w > 0.f ? __builtin_amdgcn_rcpf(w) : 0.f; }

// Merge state (W2, c2, I2) into s.
__device__ __forceinline__ void merge_into(Moments& s, float W2, float c2, float I2) {
  const float W = s.W + W2;
  const float f = W2 * rcp_or_zero(W);
  const float d = c2 - s.c;
  s.I = (s.I + I2) + d * d * s.W * f;
  s.c = s.c + d * f;
  s.W = W;
}

// Incremental step with a tile of mass Wt and first moment St: moves the
// centre, adds the correction of the earlier points, returns the new centre
// (the caller adds the tile's centred term about it).
__device__ __forceinline__ float advance(Moments& s, float Wt, float St) {
  const float Wn = s.W + Wt;
  const float cn = s.c + (St - Wt * s.c) * rcp_or_zero(Wn);
  const float d = s.c - cn;
  s.I += s.W * d * d;
  s.W = Wn;
  s.c = cn;
  return cn;
}

__device__ __forceinline__ float mass(f32x4 w) { return (w[0] + w[1]) + (w[2] + w[3]); }
__device__ __forceinline__ float first(f32x4 y, f32x4 w) {
  return (w[0] * y[0] + w[1] * y[1]) + (w[2] * y[2] + w[3] * y[3]);
}
__device__ __forceinline__ float centred(f32x4 y, f32x4 w, float c) {
  const float d0 = y[0] - c, d1 = y[1] - c, d2 = y[2] - c, d3 = y[3] - c;
  return (w[0] * d0 * d0 + w[1] * d1 * d1) + (w[2] * d2 * d2 + w[3] * d3 * d3);
}

__device__ __forceinline__ f32x4 load_chunk(__amdgpu_buffer_rsrc_t r, int chunk) {
  return __builtin_bit_cast(f32x4, buf_load16_stream(r, chunk * 16, 0));
}

// Positions (shifted) and masses of one chunk; unit masses when !WEIGHTED,
// zero mass past the row.
template <bool WEIGHTED>
struct ChunkReader {
  __amdgpu_buffer_rsrc_t rx, rw;
  int nch;
  float x0;
  __device__ __forceinline__ void read(int chunk, f32x4& y, f32x4& w) const {
    const f32x4 x = load_chunk(rx, chunk);
    y = f32x4{x[0] - x0, x[1] - x0, x[2] - x0, x[3] - x0};
    if constexpr (WEIGHTED) {
      w = load_chunk(rw, chunk);
    } else {
      const float one = chunk < nch ? 1.f : 0.f;
      w = f32x4{one, one, one, one};
    }
  }
};

template <bool WEIGHTED>
__device__ __forceinline__ void write_result(const Moments& s, float x0, float* out_c, float* out_i,
                                             size_t row) {
  if constexpr (WEIGHTED) {
    out_c[row] = s.W > 0.f ? x0 + s.c : __builtin_nanf("");
    out_i[row] = s.I;
  } else {
    out_c[row] = x0 + s.c;
    out_i[row] = s.I / s.W;
  }
}

__device__ __forceinline__ float block_sum(float v, float* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  const float r = (sm[0] + sm[1]) + (sm[2] + sm[3]);
  __syncthreads();
  return r;
}

// LEVEL 1 (thread) and 2 (wave): one wave per row; NJ chunks per lane, taken
// in groups of G = min(NJ, 8) chunks: the loads of group g + 1 are issued
// before group g is folded in, so at most two groups are in registers.
template <int NJ, int LEVEL, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void moments_wave_row_kernel(const float* __restrict__ x,
                                                                    const float* __restrict__ w,
                                                                    int T, int E,
                                                                    float* __restrict__ out_c,
                                                                    float* __restrict__ out_i) {
  constexpr int G = NJ < 8 ? NJ : 8;
  constexpr int NG = NJ / G;
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (size_t)T) return;
  ChunkReader<WEIGHTED> rd;
  rd.rx = make_rsrc(x + row * E, (uint32_t)E * 4u);
  rd.rw = WEIGHTED ? make_rsrc(w + row * E, (uint32_t)E * 4u) : rd.rx;
  rd.nch = E >> 2;
  rd.x0 = x[row * E];

  f32x4 y[2][G], m[2][G];
  Moments s{0.f, 0.f, 0.f};
  static_for<G>([&](auto j) { rd.read(lane + kWave * j, y[0][j], m[0][j]); });
  static_for<NG>([&](auto g) {
    constexpr int b = g % 2;
    if constexpr (g + 1 < NG)
      static_for<G>([&](auto j) { rd.read(lane + kWave * ((g + 1) * G + j), y[1 - b][j], m[1 - b][j]); });
    static_for<G>([&](auto j) {
      if constexpr (LEVEL == 1) {
        const float cn = advance(s, mass(m[b][j]), first(y[b][j], m[b][j]));
        s.I += centred(y[b][j], m[b][j], cn);
      } else {
        if (kWave * 4 * (g * G + j) < E) {  // segment inside the row (uniform)
          const float cn = advance(s, wave_sum(mass(m[b][j])), wave_sum(first(y[b][j], m[b][j])));
          s.I += wave_sum(centred(y[b][j], m[b][j], cn));
        }
      }
    });
  });
  if constexpr (LEVEL == 1) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
      merge_into(s, __shfl_xor(s.W, o, kWave), __shfl_xor(s.c, o, kWave), __shfl_xor(s.I, o, kWave));
  }
  if (lane == 0) write_result<WEIGHTED>(s, rd.x0, out_c, out_i, row);
}

// LEVEL 3 (block): one workgroup per row; NJ chunks per thread, one 1024-value
// tile per j.
template <int NJ, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void moments_block_row_kernel(const float* __restrict__ x,
                                                                     const float* __restrict__ w,
                                                                     int E, float* __restrict__ out_c,
                                                                     float* __restrict__ out_i) {
  __shared__ float sm[kWaves];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  ChunkReader<WEIGHTED> rd;
  rd.rx = make_rsrc(x + row * E, (uint32_t)E * 4u);
  rd.rw = WEIGHTED ? make_rsrc(w + row * E, (uint32_t)E * 4u) : rd.rx;
  rd.nch = E >> 2;
  rd.x0 = x[row * E];
  f32x4 y[NJ], m[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) rd.read(tid + kThreads * j, y[j], m[j]);

  Moments s{0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (kThreads * j * 4 >= E) continue;  // tile past the row (uniform)
    const float Wt = block_sum(mass(m[j]), sm);
    const float St = block_sum(first(y[j], m[j]), sm);
    const float cn = advance(s, Wt, St);
    s.I += block_sum(centred(y[j], m[j], cn), sm);
  }
  if (tid == 0) write_result<WEIGHTED>(s, rd.x0, out_c, out_i, row);
}

// Unfused cascade, pass 1: centre of each row. Writes the centre to out_c and
// the shifted centre c (x_0 + c = centre, kept unrounded by x_0) to out_i,
// which pass 2 reads and then overwrites with the second moment.
template <bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void centre_pass_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w, int E,
                                                               float* __restrict__ out_c,
                                                               float* __restrict__ out_i) {
  __shared__ float sm[kWaves];
  const size_t row = blockIdx.x;
  ChunkReader<WEIGHTED> rd;
  rd.rx = make_rsrc(x + row * E, (uint32_t)E * 4u);
  rd.rw = WEIGHTED ? make_rsrc(w + row * E, (uint32_t)E * 4u) : rd.rx;
  rd.nch = E >> 2;
  rd.x0 = x[row * E];
  float Wt = 0.f, St = 0.f;
  for (int c = threadIdx.x; c < rd.nch; c += kThreads) {
    f32x4 y, m;
    rd.read(c, y, m);
    Wt += mass(m);
    St += first(y, m);
  }
  Wt = block_sum(Wt, sm);
  St = block_sum(St, sm);
  if (threadIdx.x == 0) {
    const float c = St / Wt;
    out_c[row] = (!WEIGHTED || Wt > 0.f) ? rd.x0 + c : __builtin_nanf("");
    out_i[row] = Wt > 0.f ? c : 0.f;
  }
}

// Pass 2: sum of w (y - c)^2 about the centre from pass 1 (read from out_i,
// then replaced by the result: every thread reads it before the block sum's
// barriers, thread 0 writes after them).
template <bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void centred_pass_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ w, int E,
                                                                float* out_i) {
  __shared__ float sm[kWaves];
  const size_t row = blockIdx.x;
  ChunkReader<WEIGHTED> rd;
  rd.rx = make_rsrc(x + row * E, (uint32_t)E * 4u);
  rd.rw = WEIGHTED ? make_rsrc(w + row * E, (uint32_t)E * 4u) : rd.rx;
  rd.nch = E >> 2;
  rd.x0 = x[row * E];
  const float c = out_i[row];
  float acc = 0.f;
  for (int k = threadIdx.x; k < rd.nch; k += kThreads) {
    f32x4 y, m;
    rd.read(k, y, m);
    acc += centred(y, m, c);
  }
  acc = block_sum(acc, sm);
  if (threadIdx.x == 0) out_i[row] = WEIGHTED ? acc : acc / (float)E;
}

template <int LEVEL, bool WEIGHTED>
void launch_wave_rows(const float* x, const float* w, int T, int E, float* oc, float* oi,
                      hipStream_t stream) {
  const dim3 grid((T + kWaves - 1) / kWaves), block(kThreads);
  if (E <= 1024)
    hipLaunchKernelGGL((moments_wave_row_kernel<4, LEVEL, WEIGHTED>), grid, block, 0, stream, x, w, T, E, oc, oi);
  else if (E <= 2048)
    hipLaunchKernelGGL((moments_wave_row_kernel<8, LEVEL, WEIGHTED>), grid, block, 0, stream, x, w, T, E, oc, oi);
  else if (E <= 4096)
    hipLaunchKernelGGL((moments_wave_row_kernel<16, LEVEL, WEIGHTED>), grid, block, 0, stream, x, w, T, E, oc, oi);
  else
    hipLaunchKernelGGL((moments_wave_row_kernel<32, LEVEL, WEIGHTED>), grid, block, 0, stream, x, w, T, E, oc, oi);
}

template <bool WEIGHTED>
void launch_block_rows(const float* x, const float* w, int T, int E, float* oc, float* oi,
                       hipStream_t stream) {
  const dim3 grid(T), block(kThreads);
  if (E <= 1024)
    hipLaunchKernelGGL((moments_block_row_kernel<1, WEIGHTED>), grid, block, 0, stream, x, w, E, oc, oi);
  else if (E <= 2048)
    hipLaunchKernelGGL((moments_block_row_kernel<2, WEIGHTED>), grid, block, 0, stream, x, w, E, oc, oi);
  else if (E <= 4096)
    hipLaunchKernelGGL((moments_block_row_kernel<4, WEIGHTED>), grid, block, 0, stream, x, w, E, oc, oi);
  else
    hipLaunchKernelGGL((moments_block_row_kernel<8, WEIGHTED>), grid, block, 0, stream, x, w, E, oc, oi);
}

template <bool WEIGHTED>
hipError_t launch_moments(const float* x, const float* w, int T, int E, int level, float* oc,
                          float* oi, hipStream_t stream) {
  switch (level) {
    case 1: launch_wave_rows<1, WEIGHTED>(x, w, T, E, oc, oi, stream); break;
    case 2: launch_wave_rows<2, WEIGHTED>(x, w, T, E, oc, oi, stream); break;
    case 3: launch_block_rows<WEIGHTED>(x, w, T, E, oc, oi, stream); break;
    default: {
      const dim3 grid(T), block(kThreads);
      hipLaunchKernelGGL((centre_pass_kernel<WEIGHTED>), grid, block, 0, stream, x, w, E, oc, oi);
      hipLaunchKernelGGL((centred_pass_kernel<WEIGHTED>), grid, block, 0, stream, x, w, E, oi);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_row_variance(const float* x, int T, int E, int level, float* mean, float* var,
                               hipStream_t stream) {
  return launch_moments<false>(x, nullptr, T, E, level, mean, var, stream);
}

hipError_t launch_row_inertia(const float* x, const float* w, int T, int E, int level,
                              float* centre, float* inertia, hipStream_t stream) {
  return launch_moments<true>(x, w, T, E, level, centre, inertia, stream);
}

}  // namespace rf
