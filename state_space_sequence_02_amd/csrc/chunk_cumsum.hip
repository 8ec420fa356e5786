// chunk_cumsum: in-chunk cumulative sum of the log-decay A*dt, in log2 units
// (devotd.net news item on the Mamba-2 CUDA Tile forward-pass kernels,
// section 2 and its chunk_cumsum code figure: zero-padded dt tile, float cast,
// inclusive cumsum along the chunk, times LOG2E; section 3: the cumsum and dt
// stored so later stages read them contiguously).
//
// One workgroup per (chunk, head tile, batch); thread i owns time step i of
// the chunk and reads its head tile's dt values with 16-byte loads (they are
// contiguous in [B, L, H]).  The sum is a tree: a log-depth scan inside each
// 64-lane wavefront on the VALU's cross-lane (DPP) paths, then the wave
// totals added through LDS.  Every partial sum is of same-sign terms
// (A <= 0, dt >= 0), so its relative error grows with the tree depth (at most
// 9 roundings for Q = 256) rather than with Q.
//
// Outputs are time-contiguous [B, H, nc, Q] float32: dA_cs (log2 units) and
// dt_T (dt transposed, 0 past the end of the sequence).
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

constexpr int kHeadTile = 8;  // heads per workgroup: one 16-byte bf16 dt load per thread

template <typename T>
__device__ __forceinline__ float load_f32(const T* p);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_f32<bf16>(const bf16* p) { return bf2f(*p); }

template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
  typedef bf16x8 type;
  static constexpr int n = 8;
};
template <>
struct Vec16<float> {
  typedef f32x4 type;
  static constexpr int n = 4;
};

// v + (v of the lane selected by the DPP control), 0 where no lane is selected.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false);
  return v + __builtin_bit_cast(float, s);
}

// Inclusive scan over a wavefront's 64 lanes: Hillis-Steele inside each
// 16-lane row (row_shr 1, 2, 4, 8), then each row total carried into the rows
// above it (row_bcast 15 into rows 1 and 3, row_bcast 31 into rows 2 and 3).
__device__ __forceinline__ float wave_scan(float v) {
  v = dpp_add<0x111, 0xf>(v);
  v = dpp_add<0x112, 0xf>(v);
  v = dpp_add<0x114, 0xf>(v);
  v = dpp_add<0x118, 0xf>(v);
  v = dpp_add<0x142, 0xa>(v);
  v = dpp_add<0x143, 0xc>(v);
  return v;
}

template <typename T>
__global__ void __launch_bounds__(256) chunk_cumsum_kernel(const T* __restrict__ dt,
                                                           const float* __restrict__ A,
                                                           float* __restrict__ dA_cs,
                                                           float* __restrict__ dt_T, int L, int H,
                                                           int Q, int nc) {
  __shared__ float wave_tot[kHeadTile][4];
  const int c = blockIdx.x;
  const int h0 = blockIdx.y * kHeadTile;
  const int b = blockIdx.z;
  const int i = threadIdx.x;  // time step in the chunk
  const int lane = lane_id();
  const int w = wave_id();
  const int nwaves = (blockDim.x + 63) >> 6;
  const int t = c * Q + i;
  const int nh = min(kHeadTile, H - h0);

  float v[kHeadTile];
  float dtv[kHeadTile];
#pragma unroll
  for (int k = 0; k < kHeadTile; ++k) dtv[k] = 0.f;
  if (i < Q && t < L) {
    const T* src = dt + ((int64_t)b * L + t) * H + h0;
    constexpr int VE = Vec16<T>::n;
    if (H % VE == 0) {  // h0 is a multiple of the head tile (8), so of VE: every vector is aligned
#pragma unroll
      for (int k0 = 0; k0 < kHeadTile; k0 += VE) {
        if (k0 < nh) {
          const typename Vec16<T>::type u = *(const typename Vec16<T>::type*)(src + k0);
#pragma unroll
          for (int e = 0; e < VE; ++e) dtv[k0 + e] = (float)u[e];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kHeadTile; ++k)
        if (k < nh) dtv[k] = load_f32(src + k);
    }
  }
#pragma unroll
  for (int k = 0; k < kHeadTile; ++k) v[k] = (k < nh) ? wave_scan(A[h0 + k] * dtv[k]) : 0.f;
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < kHeadTile; ++k) wave_tot[k][w] = v[k];
  }
  __syncthreads();
  if (w > 0) {
#pragma unroll
    for (int k = 0; k < kHeadTile; ++k) {
      float pre = wave_tot[k][0];
      for (int u = 1; u < w; ++u) pre += wave_tot[k][u];
      v[k] += pre;
    }
  }
  (void)nwaves;
  if (i < Q) {
#pragma unroll
    for (int k = 0; k < kHeadTile; ++k) {
      if (k < nh) {
        const int64_t o = (((int64_t)b * H + h0 + k) * nc + c) * Q + i;
        dA_cs[o] = v[k] * kLog2e;
        dt_T[o] = dtv[k];
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_cumsum(const Dims& d, const void* dt, const float* A, float* dA_cs,
                               float* dt_T, hipStream_t s) {
  const int threads = (int)((d.Q + 63) / 64 * 64);
  dim3 grid((unsigned)d.nc, (unsigned)((d.H + kHeadTile - 1) / kHeadTile), (unsigned)d.B);
  if (d.bf16)
    chunk_cumsum_kernel<bf16><<<grid, threads, 0, s>>>((const bf16*)dt, A, dA_cs, dt_T, (int)d.L,
                                                       (int)d.H, (int)d.Q, (int)d.nc);
  else
    chunk_cumsum_kernel<float><<<grid, threads, 0, s>>>((const float*)dt, A, dA_cs, dt_T,
                                                        (int)d.L, (int)d.H, (int)d.Q, (int)d.nc);
  return hipGetLastError();
}

}  // namespace m2
