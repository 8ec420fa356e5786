// decode_step: the recurrence advanced by one token per (batch, head), in
// place on the float32 state - the constant-memory inference mode of the same
// model (devotd.net news item on the Mamba-2 CUDA Tile forward-pass kernels,
// section 1: a fixed-size hidden state updated as tokens are processed;
// disconfirmai.com "Jane Street ML Engineers Map Mamba-2 Recurrent State
// Computation to Tensor Cores with cuTile", abstract: the recurrent state).
//
//     state[p, n] = exp(dt A) state[p, n] + dt x[p] B[n]
//     y[p]        = sum_n state[p, n] C[n] + D x[p]
//
// One wavefront per state row (b, h, p); lane l owns n = l, l + 64, ...
// (64 consecutive floats per access, so every load and store is a full
// 256-byte line).  The state is read once and written once: the step is
// bound by HBM bandwidth on it.  y[p] is the wavefront sum of the lanes'
// partial dot products.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

constexpr int kRowsPerBlock = 4;  // wavefronts (state rows) per workgroup

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld<bf16>(const bf16* p) { return bf2f(*p); }

template <typename T>
__device__ __forceinline__ void st(T* p, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st<bf16>(bf16* p, float v) { *p = f2bf(v); }

// Sum over the 64 lanes (butterfly; every lane ends with the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename T, int NV>
__global__ void __launch_bounds__(64 * kRowsPerBlock) decode_step_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ D,
    float* __restrict__ state, T* __restrict__ y, int64_t rows, int H, int P, int N, int G) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wavefront leaves together
  const int lane = threadIdx.x & 63;
  const int p = (int)(row % P);
  const int64_t bh = row / P;  // b * H + h
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  const int g = h / (H / G);

  const float dtv = ld(dt + bh);
  const float decay = fast_exp2(dtv * A[h] * kLog2e);
  const float xv = ld(x + bh * P + p);
  const float u = dtv * xv;
  const T* Bg = Bm + (b * G + g) * N;
  const T* Cg = Cm + (b * G + g) * N;
  float* s = state + row * N;

  float part = 0.f;
  if constexpr (NV > 0) {  // N is exactly 64 * NV: every lane busy, no bounds checks
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int n = lane + 64 * e;
      const float v = decay * s[n] + u * ld(Bg + n);
      s[n] = v;
      part += v * ld(Cg + n);
    }
  } else {
    for (int n = lane; n < N; n += 64) {
      const float v = decay * s[n] + u * ld(Bg + n);
      s[n] = v;
      part += v * ld(Cg + n);
    }
  }
  const float yv = wave_sum(part) + (D ? D[h] : 0.f) * xv;
  if (lane == 0) st(y + bh * P + p, yv);
}

template <typename T>
hipError_t launch_t(const Dims& d, const void* x, const void* dt, const float* A, const void* B,
                    const void* C, const float* D, float* state, void* y, hipStream_t s) {
  const int64_t rows = d.B * d.H * d.P;
  const unsigned grid = (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const int threads = 64 * kRowsPerBlock;
#define M2_DECODE(NV)                                                                          \
  decode_step_kernel<T, NV><<<grid, threads, 0, s>>>(                                         \
      (const T*)x, (const T*)dt, A, (const T*)B, (const T*)C, D, state, (T*)y, rows, (int)d.H, \
      (int)d.P, (int)d.N, (int)d.G)
  switch (d.N) {
    case 64: M2_DECODE(1); break;
    case 128: M2_DECODE(2); break;
    case 256: M2_DECODE(4); break;
    case 512: M2_DECODE(8); break;
    default: M2_DECODE(0); break;
  }
#undef M2_DECODE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step(const Dims& d, const void* x, const void* dt, const float* A,
                              const void* B, const void* C, const float* D, float* state,
                              void* y, hipStream_t s) {
  return d.bf16 ? launch_t<bf16>(d, x, dt, A, B, C, D, state, y, s)
                : launch_t<float>(d, x, dt, A, B, C, D, state, y, s);
}

}  // namespace m2
