// state_passing: the decayed jump that carries the state across chunks in
// chunk order (devotd.net news item on the Mamba-2 CUDA Tile forward-pass
// kernels, section 2: fwd_pass_state yields the state at every chunk start
// and after the last chunk, walking chunks in order while independent parts
// of the state run in parallel; disconfirmai.com "Jane Street ML Engineers
// Map Mamba-2 Recurrent State Computation to Tensor Cores with cuTile",
// body: jump formula with the decay as a log-space sum).
//
// Work split: one thread per 4 consecutive (p, n) state entries of one
// (batch, head); every thread walks all chunks in order.  Memory bound: each
// chunk's state is read once and overwritten once, in place.  Loads run
// kDepth chunks ahead of use so that enough bytes are in flight per CU.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

constexpr int kDepth = 16;
constexpr int kThreads = 256;

// V is float4 when P*N is a multiple of 4 (every bfloat16 size), else float.
// With `hst` non-null (float4 only) the chunk-start states go there as
// bfloat16 (round to nearest even) and `states` is only read; otherwise they
// overwrite `states` in place.
template <typename V>
__global__ void __launch_bounds__(kThreads) state_passing_kernel(
    float* __restrict__ states, const float* __restrict__ dA_cs, const float* __restrict__ init,
    float* __restrict__ final_state, bf16* __restrict__ hst, int64_t H, int64_t PNv,
    int64_t blocks_per_head, int nc, int Q) {
  const int64_t bh = (int64_t)blockIdx.x / blocks_per_head;  // b * H + h
  const int64_t gid = ((int64_t)blockIdx.x % blocks_per_head) * kThreads + threadIdx.x;
  if (gid >= PNv) return;
  const int64_t b = bh / H, h = bh % H;
  const int64_t chunk_stride = H * PNv;  // V units between consecutive chunks
  V* base = (V*)states + (b * nc * H + h) * PNv + gid;
  const float* cs_last = dA_cs + bh * (int64_t)nc * Q + (Q - 1);

  V run = V{};
  if (init) run = ((const V*)init)[bh * PNv + gid];

  V buf[kDepth];
#pragma unroll
  for (int k = 0; k < kDepth; ++k)
    if (k < nc) buf[k] = __builtin_nontemporal_load(base + (int64_t)k * chunk_stride);

  for (int c0 = 0; c0 < nc; c0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int c = c0 + k;
      if (c < nc) {
        const V cur = buf[k];
        if (c + kDepth < nc)
          buf[k] = __builtin_nontemporal_load(base + (int64_t)(c + kDepth) * chunk_stride);
        const float decay = exp2f(cs_last[(int64_t)c * Q]);
        if constexpr (sizeof(V) == 16) {
          if (hst) {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = f2bf(run[e]);
            *((bf16x4*)hst + (b * nc * H + h) * PNv + gid + (int64_t)c * chunk_stride) = o;
          } else {
            __builtin_nontemporal_store(run, base + (int64_t)c * chunk_stride);
          }
        } else {
          __builtin_nontemporal_store(run, base + (int64_t)c * chunk_stride);
        }
        run = decay * run + cur;
      }
    }
  }
  if (final_state) ((V*)final_state)[bh * PNv + gid] = run;
}

// v + (v of the lane the DPP control selects), 0 where no lane is selected.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false);
  return v + __builtin_bit_cast(float, s);
}

// Sum over the wavefront's 64 lanes, complete in lane 63: a scan inside each
// 16-lane row (row_shr 1, 2, 4, 8), then the row totals carried upwards
// (row_bcast 15, 31) - cross-lane VALU paths instead of LDS permutes.
__device__ __forceinline__ float wave_total_in_lane63(float v) {
  v = dpp_add<0x111, 0xf>(v);
  v = dpp_add<0x112, 0xf>(v);
  v = dpp_add<0x114, 0xf>(v);
  v = dpp_add<0x118, 0xf>(v);
  v = dpp_add<0x142, 0xa>(v);
  return dpp_add<0x143, 0xc>(v);
}

// Backward pass: the same jump run in reverse chunk order on the adjoint.
// With r_c the gradient of the loss with respect to the start state of
// chunk c, r_nc = dfinal and r_c = 2^cs_last(c) r_{c+1} + E_c, where E_c is
// chunk c's adjoint chunk state.  Writes g_c = r_{c+1} (the gradient reaching
// chunk c's end state) as bfloat16, dh0 = r_0 in float32, and for every chunk
// the per-wavefront parts of 2^cs_last(c) <g_c, h_c>: the end-of-chunk
// gradient times the decayed start state, the part of the derivative with
// respect to the chunk's log decays that flows through the carried state.
// h_c is the forward pass's bfloat16 start state of chunk c.
__global__ void __launch_bounds__(kThreads) state_passing_reverse_kernel(
    const f32x4* __restrict__ E, const float* __restrict__ dA_cs,
    const f32x4* __restrict__ dfinal, const bf16x4* __restrict__ hst, bf16x4* __restrict__ gst,
    f32x4* __restrict__ dh0, float* __restrict__ dots, int64_t H, int64_t PNv,
    int64_t blocks_per_head, int nc, int Q) {
  const int64_t bh = (int64_t)blockIdx.x / blocks_per_head;  // b * H + h
  const int64_t blk = (int64_t)blockIdx.x % blocks_per_head;
  const int64_t gid = blk * kThreads + threadIdx.x;
  const bool live = gid < PNv;  // dead lanes still take part in the wave sums
  const int64_t g = live ? gid : 0;
  const int64_t b = bh / H, h = bh % H;
  const int64_t chunk_stride = H * PNv;
  const int64_t base = (b * nc * H + h) * PNv + g;
  const float* cs_last = dA_cs + bh * (int64_t)nc * Q + (Q - 1);
  const int64_t wph = blocks_per_head * (kThreads / 64);
  float* dot_out = dots + bh * (int64_t)nc * wph + blk * (kThreads / 64) + (threadIdx.x >> 6);

  f32x4 run = f32x4{0.f, 0.f, 0.f, 0.f};
  if (dfinal && live) run = dfinal[bh * PNv + g];

  // slot k of a ring holds chunk nc-1-(c0+k): its E, its start state and its
  // total log decay.  Every slot is reloaded unconditionally (chunks past the
  // first clamped to chunk 0, loaded and never used), so no value in the ring
  // is a merge of a fresh load with an old one: the compiler then never has
  // to wait for the load it just issued, which would also wait for every
  // older load of the ring.
  f32x4 eb[kDepth];
  bf16x4 hb[kDepth];
  float lb[kDepth];
#pragma unroll
  for (int k = 0; k < kDepth; ++k) {
    const int c = max(nc - 1 - k, 0);
    eb[k] = __builtin_nontemporal_load(E + base + (int64_t)c * chunk_stride);
    hb[k] = hst[base + (int64_t)c * chunk_stride];
    lb[k] = cs_last[(int64_t)c * Q];
  }
  for (int c0 = 0; c0 < nc; c0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int c = nc - 1 - (c0 + k);
      const f32x4 cur = eb[k];
      const bf16x4 hcur = hb[k];
      const float lc = lb[k];
      const int cn = max(c - kDepth, 0);  // chunk this slot holds next
      eb[k] = __builtin_nontemporal_load(E + base + (int64_t)cn * chunk_stride);
      hb[k] = hst[base + (int64_t)cn * chunk_stride];
      lb[k] = cs_last[(int64_t)cn * Q];
      if (c >= 0) {
        f32x4 hc;
#pragma unroll
        for (int e = 0; e < 4; ++e) hc[e] = bf2f(hcur[e]);
        if (live) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = f2bf(run[e]);
          gst[base + (int64_t)c * chunk_stride] = o;
        }
        const float decay = exp2f(lc);
        float part = live ? run[0] * hc[0] + run[1] * hc[1] + run[2] * hc[2] + run[3] * hc[3] : 0.f;
        part = wave_total_in_lane63(part);
        if ((threadIdx.x & 63) == 63) dot_out[(int64_t)c * wph] = decay * part;
        run = decay * run + cur;
      }
    }
  }
  if (dh0 && live) dh0[bh * PNv + g] = run;
}

}  // namespace

int64_t state_reverse_waves_per_head(const Dims& d) {
  const int64_t PNv = d.P * d.N / 4;
  return (PNv + kThreads - 1) / kThreads * (kThreads / 64);
}

hipError_t launch_state_passing_reverse(const Dims& d, const float* E, const float* dA_cs,
                                        const float* dfinal, const void* hst, void* gst,
                                        float* dh0, float* dots, hipStream_t s) {
  const int64_t PN = d.P * d.N;
  if (PN % 4 != 0) return hipErrorInvalidValue;
  const int64_t PNv = PN / 4, bph = (PNv + kThreads - 1) / kThreads;
  state_passing_reverse_kernel<<<(unsigned)(d.B * d.H * bph), kThreads, 0, s>>>(
      (const f32x4*)E, dA_cs, (const f32x4*)dfinal, (const bf16x4*)hst, (bf16x4*)gst,
      (f32x4*)dh0, dots, d.H, PNv, bph, (int)d.nc, (int)d.Q);
  return hipGetLastError();
}

hipError_t launch_state_passing(const Dims& d, float* states, const float* dA_cs,
                                const float* init, float* final_state, hipStream_t s) {
  const int64_t PN = d.P * d.N;
  if (PN % 4 == 0) {
    const int64_t PNv = PN / 4, bph = (PNv + kThreads - 1) / kThreads;
    state_passing_kernel<f32x4><<<(unsigned)(d.B * d.H * bph), kThreads, 0, s>>>(
        states, dA_cs, init, final_state, nullptr, d.H, PNv, bph, (int)d.nc, (int)d.Q);
  } else {
    const int64_t bph = (PN + kThreads - 1) / kThreads;
    state_passing_kernel<float><<<(unsigned)(d.B * d.H * bph), kThreads, 0, s>>>(
        states, dA_cs, init, final_state, nullptr, d.H, PN, bph, (int)d.nc, (int)d.Q);
  }
  return hipGetLastError();
}

hipError_t launch_state_passing_bf16(const Dims& d, const float* states, const float* dA_cs,
                                     const float* init, void* hst, float* final_state,
                                     hipStream_t s) {
  const int64_t PN = d.P * d.N;
  if (PN % 4 != 0) return hipErrorInvalidValue;
  const int64_t PNv = PN / 4, bph = (PNv + kThreads - 1) / kThreads;
  state_passing_kernel<f32x4><<<(unsigned)(d.B * d.H * bph), kThreads, 0, s>>>(
      const_cast<float*>(states), dA_cs, init, final_state, (bf16*)hst, d.H, PNv, bph,
      (int)d.nc, (int)d.Q);
  return hipGetLastError();
}

}  // namespace m2
