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
// The state is read once and written once: the step is bound by HBM
// bandwidth on it.  State sizes 64 .. 512 take 16-byte accesses (below);
// other sizes run one wavefront per state row (b, h, p), lane l owning
// n = l, l + 64, ... (64 consecutive floats per access, every load and store
// a full 256-byte line).  y[p] is the sum of the row's lanes' partial dot
// products.
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

__device__ __forceinline__ float bf2f_any(float v) { return v; }
__device__ __forceinline__ float bf2f_any(bf16 v) { return bf2f(v); }

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

// State sizes 64, 128, 256 and 512: 16-byte accesses.  Lane l of a row's
// LPR lanes owns columns 4 l .. 4 l + 3 (+ 256 k); a wavefront covers 64 /
// LPR rows per pass and makes PASSES passes, all of its state loads issued
// before the first update.  y[p] is the sum over the row's lanes.  Four
// passes measured best up to about half a million state rows (B = 128 at
// H = 32, P = 64, N = 256: 110 -> 100 us against one row per wavefront and
// 4-byte accesses), two from a million rows on (B = 512: 410 us with four,
// 401 with two).

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  typedef f32x4 type;
  static __device__ __forceinline__ float at(const type& v, int e) { return v[e]; }
};
template <>
struct Vec4<bf16> {
  typedef bf16x4 type;
  static __device__ __forceinline__ float at(const type& v, int e) { return bf2f(v[e]); }
};

template <typename T, int N, int PASSES>
__global__ void __launch_bounds__(64 * kRowsPerBlock) decode_step_vec_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ D,
    float* __restrict__ state, T* __restrict__ y, int64_t rows, int H, int P, int G) {
  constexpr int VPL = N >= 256 ? N / 256 : 1;  // 16-byte state vectors per lane and row
  constexpr int LPR = N >= 256 ? 64 : N / 4;   // lanes per row
  constexpr int RPP = 64 / LPR;                // rows per pass
  typedef typename Vec4<T>::type V4;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int sub = lane / LPR, cl = lane % LPR;
  const int64_t row0 = wave * (RPP * PASSES) + sub;

  f32x4 sv[PASSES][VPL];
#pragma unroll
  for (int it = 0; it < PASSES; ++it) {
    const int64_t row = row0 + it * RPP;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      sv[it][k] = row < rows ? *(const f32x4*)(state + row * N + 4 * cl + 256 * k)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int it = 0; it < PASSES; ++it) {
    const int64_t row = row0 + it * RPP;
    const bool live = row < rows;
    const int64_t rr = live ? row : 0;
    const int p = (int)(rr % P);
    const int64_t bh = rr / P;  // b * H + h
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const float dtv = bf2f_any(dt[bh]);
    const float decay = fast_exp2(dtv * A[h] * kLog2e);
    const float xv = bf2f_any(x[bh * P + p]);
    const float u = dtv * xv;
    const T* Bg = Bm + (b * G + g) * N;
    const T* Cg = Cm + (b * G + g) * N;
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int n = 4 * cl + 256 * k;
      const V4 bv = *(const V4*)(Bg + n);
      const V4 cv = *(const V4*)(Cg + n);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = decay * sv[it][k][e] + u * Vec4<T>::at(bv, e);
        part += v[e] * Vec4<T>::at(cv, e);
      }
      if (live) *(f32x4*)(state + row * N + n) = v;
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) part += __shfl_xor(part, off, 64);
    if (live && cl == 0) st(y + bh * P + p, part + (D ? D[h] : 0.f) * xv);
  }
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
#define M2_DECODE_VP(NN, PP)                                                                   \
  {                                                                                            \
    constexpr int RPW = (NN >= 256 ? 1 : 256 / NN) * PP; /* rows per wavefront */               \
    const int64_t waves = (rows + RPW - 1) / RPW;                                              \
    decode_step_vec_kernel<T, NN, PP><<<(unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock), \
                                        threads, 0, s>>>(                                      \
        (const T*)x, (const T*)dt, A, (const T*)B, (const T*)C, D, state, (T*)y, rows,         \
        (int)d.H, (int)d.P, (int)d.G);                                                         \
  }
#define M2_DECODE_VEC(NN)          \
  if (rows >= (int64_t(1) << 20))  \
    M2_DECODE_VP(NN, 2)            \
  else                             \
    M2_DECODE_VP(NN, 4)
  switch (d.N) {
    case 64: M2_DECODE_VEC(64); break;
    case 128: M2_DECODE_VEC(128); break;
    case 256: M2_DECODE_VEC(256); break;
    case 512: M2_DECODE_VEC(512); break;
    default: M2_DECODE(0); break;
  }
#undef M2_DECODE_VEC
#undef M2_DECODE_VP
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
