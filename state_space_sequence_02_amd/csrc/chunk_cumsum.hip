// chunk_cumsum: in-chunk cumulative sum of the log-decay A*dt, in log2 units
// (devotd.net news item on the Mamba-2 CUDA Tile forward-pass kernels,
// section 2 and its chunk_cumsum code figure: zero-padded dt tile, float cast,
// inclusive cumsum along the chunk, times LOG2E; section 3: the cumsum and dt
// stored so later stages read them contiguously).
//
// One wavefront per (chunk, head tile, batch); lane l owns time steps
// 4 l .. 4 l + 3 of the chunk and reads its head tile's dt values with 16-byte
// loads (they are contiguous in [B, L, H]).  The sum is a tree: the lane's
// four steps in order, then a log-depth scan of the lane totals across the
// wavefront on the VALU's cross-lane (DPP) paths.  Every partial sum is of
// same-sign terms (A <= 0, dt >= 0), so its relative error grows with the
// tree depth (at most 10 roundings for Q = 256) rather than with Q.
//
// Outputs are time-contiguous [B, H, nc, Q] float32: dA_cs (log2 units) and
// dt_T (dt transposed, 0 past the end of the sequence).
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

constexpr int kHeadTile = 8;  // heads per wavefront: one 16-byte bf16 dt load per time step

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

// One wavefront per (chunk, head tile, batch), four per workgroup; lane l
// owns time steps 4 l .. 4 l + 3 of the chunk (Q <= 256) for the tile's
// heads.  Per head: the lane's four steps summed in order, the lane totals
// scanned across the wavefront, and the lane's exclusive prefix (the
// inclusive scan of the lane below, moved up one lane) added to its four
// partial sums; outputs leave as one 16-byte store per head and array.
template <typename T>
__global__ void __launch_bounds__(256) chunk_cumsum_kernel(const T* __restrict__ dt,
                                                           const float* __restrict__ A,
                                                           float* __restrict__ dA_cs,
                                                           float* __restrict__ dt_T, int L, int H,
                                                           int Q, int nc, int ntile) {
  const int c = blockIdx.x;
  const int tile = blockIdx.y * 4 + wave_id();
  const int b = blockIdx.z;
  if (tile >= ntile) return;  // whole wavefront
  const int h0 = tile * kHeadTile;
  const int nh = min(kHeadTile, H - h0);
  const int lane = lane_id();
  const int i0 = 4 * lane;  // this lane's first step in the chunk

  float dtv[4][kHeadTile];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int k = 0; k < kHeadTile; ++k) dtv[s][k] = 0.f;
  constexpr int VE = Vec16<T>::n;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t t = (int64_t)c * Q + i0 + s;
    if (i0 + s < Q && t < L) {
      const T* src = dt + ((int64_t)b * L + t) * H + h0;
      if (H % VE == 0) {  // h0 is a multiple of the head tile (8), so of VE: every vector is aligned
#pragma unroll
        for (int k0 = 0; k0 < kHeadTile; k0 += VE) {
          if (k0 < nh) {
            const typename Vec16<T>::type u = *(const typename Vec16<T>::type*)(src + k0);
#pragma unroll
            for (int e = 0; e < VE; ++e) dtv[s][k0 + e] = (float)u[e];
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < kHeadTile; ++k)
          if (k < nh) dtv[s][k] = load_f32(src + k);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kHeadTile; ++k) {
    if (k < nh) {
      const float a = A[h0 + k];
      f32x4 v;
      v[0] = a * dtv[0][k];
      v[1] = v[0] + a * dtv[1][k];
      v[2] = v[1] + a * dtv[2][k];
      v[3] = v[2] + a * dtv[3][k];
      const float incl = wave_scan(v[3]);
      const float pre = __builtin_bit_cast(
          float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, incl), 0x138, 0xf, 0xf, false));
      if (i0 < Q) {
        const int64_t o = (((int64_t)b * H + h0 + k) * nc + c) * Q + i0;
        f32x4 cs, d;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          cs[s] = (pre + v[s]) * kLog2e;
          d[s] = dtv[s][k];
        }
        *(f32x4*)(dA_cs + o) = cs;
        *(f32x4*)(dt_T + o) = d;
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_cumsum(const Dims& d, const void* dt, const float* A, float* dA_cs,
                               float* dt_T, hipStream_t s) {
  // one wavefront covers a chunk (4 steps per lane), and the 16-byte stores
  // need Q % 4 == 0: every supported chunk size (16 .. 256) qualifies
  if (d.Q > 256 || d.Q % 4 != 0) return hipErrorInvalidValue;
  const int ntile = (int)((d.H + kHeadTile - 1) / kHeadTile);
  dim3 grid((unsigned)d.nc, (unsigned)((ntile + 3) / 4), (unsigned)d.B);
  if (d.bf16)
    chunk_cumsum_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)dt, A, dA_cs, dt_T, (int)d.L,
                                                   (int)d.H, (int)d.Q, (int)d.nc, ntile);
  else
    chunk_cumsum_kernel<float><<<grid, 256, 0, s>>>((const float*)dt, A, dA_cs, dt_T, (int)d.L,
                                                    (int)d.H, (int)d.Q, (int)d.nc, ntile);
  return hipGetLastError();
}

}  // namespace m2
