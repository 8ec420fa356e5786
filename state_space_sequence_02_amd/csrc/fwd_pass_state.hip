// fwd_pass_state as one kernel (the pages' own second kernel; the library's
// default forward runs it over spans of chunks at large sizes and as
// chunk_state + state_passing below them, both faster on this chip): the
// per-chunk B X^T contraction and the
// decayed jump that carries the state across chunks, walking the chunks in
// order with the running state held in MFMA accumulators (devotd.net news
// item on the Mamba-2 CUDA Tile forward-pass kernels, section 2: the second
// kernel yields the state at every chunk start and after the last chunk,
// keeping chunk order while independent parts of the state run in parallel;
// disconfirmai.com "Jane Street ML Engineers Map Mamba-2 Recurrent State
// Computation to Tensor Cores with cuTile", body: the jump formula with the
// rows of X pre-scaled by exponentials of the log-space cumulative sum).
//
// For head h, chunk c in order, with cs the chunk's cumulative sum (log2
// units) and w_j = 2^(cs[Q-1] - cs[j]) dt_j:
//     h_start[c] = run                                 (stored as bf16)
//     run = 2^(cs[Q-1]) run + sum_j (w_j x_j) (outer) B_j
// and the final state (float32) after the last chunk.  The per-chunk states
// never reach memory and the running state never leaves float32.
//
// Work split: one workgroup per (batch, head, 32 rows of P, 64 columns of N):
// 4 waves, wave w owning p-tile (w & 1) and the 32 columns 32 (w >> 1) .. of
// the slice, as two MFMA tiles D[n, p] += B^T[n, j] (w x)[j, p], tile nt
// covering n = 32 (w >> 1) + 16 nt + m for MFMA row m.
//
// Per chunk the slice's x rows (Q x 32), B rows (Q x 64), cumulative sums and
// weights w_j (precomputed with the cumulative sums) arrive by direct-to-LDS
// loads into one of three LDS buffers, two chunks ahead of use, so about two
// chunks of loads are in flight per CU (one workgroup per CU).  A wave issues
// its share of chunk c + 2's loads spread over chunk c's MFMAs: issued in one
// burst they would queue behind the CU's address unit and hold back the wave.
// The x operand is scaled by w_j as it is read (the MFMA's K runs along j),
// so a chunk needs one barrier.  Workgroup ids place every tile of a head on
// one XCD (id % 8), so a head's x rows are fetched into that XCD's L2 once.
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

template <int Q, int N>
struct FCfg {
  static constexpr int P = 64, PS = 32, NS = 64, NT = 256, NW = 4;
  static constexpr int TPH = (P / PS) * (N / NS);  // workgroups per (batch, head)
  static constexpr int XS_BYTES = Q * PS * 2;      // x rows, 64 bytes each
  static constexpr int BS_BYTES = Q * NS * 2;      // B rows, 128 bytes each
  static constexpr int CS_BYTES = Q * 4;           // cumulative sums, then weights
  static constexpr int BUF = XS_BYTES + BS_BYTES + 2 * CS_BYTES;
  static constexpr int NBUF = 3;
  static constexpr int LDS = NBUF * BUF;
  static constexpr int KS = Q / 32;
  static constexpr int XI = XS_BYTES / 1024 / NW;  // direct-to-LDS loads per wave per chunk
  static constexpr int BI = BS_BYTES / 1024 / NW;
  static constexpr int LOADS = XI + BI;            // (+1 in waves 0 and 1: sums, weights)
  static constexpr int PPK = (LOADS + 1 + KS - 1) / KS;  // loads issued per K step
  static_assert(XI >= 1 && BI >= 1, "chunk too short for the tile");
  static_assert(LDS <= 160 * 1024, "three buffers must fit in LDS");
};

// 16-byte chunk positions inside an LDS row (involutions).  Transpose reads
// of one instruction touch rows 8g + a (a = 0..3, g = 0..3), 32 contiguous
// bytes per row; these XORs spread each instruction over all eight 16-byte
// bank groups of a 128-byte bank period, four rows on each.
//   x rows (64 bytes = 4 chunks, two rows per period): (a >> 1) flips the
//   32-byte half.
//   B rows (128 bytes = 8 chunks): a picks one of four 32-byte slots.
__device__ __forceinline__ int xswz(int r, int c) { return c ^ (((r >> 1) & 1) << 1); }
__device__ __forceinline__ int bswz(int r, int c) { return c ^ ((r & 3) << 1); }

// Load `i` of chunk c into buffer `buf` (an LDS byte address): K::XI x loads,
// then K::BI B loads, then the cumulative sums (wave 0) or weights (wave 1);
// waves 2 and 3 issue nothing for the last.  Rows past L are clamped to L-1:
// their weight is 0.
template <int Q, int N>
__device__ __forceinline__ void load_piece(int i, uint32_t buf, const bf16* __restrict__ x,
                                           const bf16* __restrict__ Bm,
                                           const float* __restrict__ dA_cs,
                                           const float* __restrict__ w_T, int b, int c, int h,
                                           int g, int p0, int n0, int L, int H, int G, int nc) {
  using K = FCfg<Q, N>;
  const int lane = lane_id();
  const int w = wave_id();
  const int64_t tok0 = (int64_t)c * Q;
  if (i < K::XI) {
    const int k = w + K::NW * i;
    const int s = k * 64 + lane;
    const int r = s >> 2, pos = s & 3;
    int64_t t = tok0 + r;
    if (t > L - 1) t = L - 1;
    dma16(x + (((int64_t)b * L + t) * H + h) * K::P + p0 + 8 * xswz(r, pos), buf + k * 1024);
  } else if (i < K::LOADS) {
    const int k = w + K::NW * (i - K::XI);
    const int s = k * 64 + lane;
    const int r = s >> 3, pos = s & 7;
    int64_t t = tok0 + r;
    if (t > L - 1) t = L - 1;
    dma16(Bm + (((int64_t)b * L + t) * G + g) * N + n0 + 8 * bswz(r, pos),
          buf + K::XS_BYTES + k * 1024);
  } else if (i == K::LOADS) {
    if (w < 2 && lane < Q / 4) {
      const int64_t cb = (((int64_t)b * H + h) * nc + c) * Q;
      dma16((w == 0 ? dA_cs : w_T) + cb + 4 * lane,
            buf + K::XS_BYTES + K::BS_BYTES + w * K::CS_BYTES);
    }
  }
}

// Waits until every memory operation of this wave except the `NEWER` most
// recent ones has completed (vector memory operations retire in issue order).
template <int NEWER>
__device__ __forceinline__ void wait_older() {
  static_assert(NEWER < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | (NEWER & 15) | ((NEWER >> 4) << 14));  // lgkmcnt(0)
}

template <int Q, int N>
__global__ void __launch_bounds__(256, 1) fwd_pass_state_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ dA_cs,
    const float* __restrict__ w_T, const float* __restrict__ init, bf16* __restrict__ hst,
    float* __restrict__ final_state, int L, int H, int G, int nc, int BH) {
  using K = FCfg<Q, N>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  // Every tile of a head on one XCD: id = 8 r + xcd, head u = 8 (r / TPH) + xcd.
  const int xcd = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int u = (r / K::TPH) * 8 + xcd;
  if (u >= BH) return;
  const int tile = r % K::TPH;
  const int b = u / H, h = u % H, g = h / (H / G);
  const int p0 = (tile & 1) * K::PS, n0 = (tile >> 1) * K::NS;

  const int lane = lane_id();
  const int w = wave_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int pw = w & 1, nq = w >> 1;

  // Running state: acc[nt][r] = run[p = p0 + 16 pw + L16][n = n0 + 32 nq + 16 nt + 4 grp + r].
  const int prow = p0 + 16 * pw + L16;
  const int ncol = n0 + 32 * nq + 4 * grp;
  f32x4 acc[2];
  if (init) {
    const float* src = init + ((int64_t)u * K::P + prow) * N + ncol;
    acc[0] = *(const f32x4*)src;
    acc[1] = *(const f32x4*)(src + 16);
  } else {
    acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint32_t sbase = lds_addr(smem);
#pragma unroll
  for (int i = 0; i <= K::LOADS; ++i)
    load_piece<Q, N>(i, sbase, x, Bm, dA_cs, w_T, b, 0, h, g, p0, n0, L, H, G, nc);
  const int c1 = min(1, nc - 1);
#pragma unroll
  for (int i = 0; i <= K::LOADS; ++i)
    load_piece<Q, N>(i, sbase + K::BUF, x, Bm, dA_cs, w_T, b, c1, h, g, p0, n0, L, H, G, nc);
  if (w < 2) wait_older<K::LOADS + 1>(); else wait_older<K::LOADS>();
  lds_barrier();

  const int64_t hrow = ((int64_t)b * nc * H + h) * K::P + prow;  // h_start row of chunk 0
  const int xo = (L16 & 1) * 8;  // lane L points at 8-byte block L % 4 of a 32-byte block
  for (int c = 0; c < nc; ++c) {
    const int cur = c % 3;
    const uint32_t nbuf = sbase + ((c + 2) % 3) * K::BUF;
    const int cn = min(c + 2, nc - 1);  // past the end: re-load the last chunk, never used
    const unsigned char* xs = smem + cur * K::BUF;
    const unsigned char* bs = xs + K::XS_BYTES;
    const float* css = (const float*)(bs + K::BS_BYTES);
    const float* wts = css + Q;
    {  // h_start[c] = run: 4 consecutive n per lane and tile (issued before the loads)
      bf16* dst = hst + (hrow + (int64_t)c * H * K::P) * N + ncol;
      bf16x4 o0, o1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o0[e] = f2bf(acc[0][e]);
        o1[e] = f2bf(acc[1][e]);
      }
      *(bf16x4*)dst = o0;
      *(bf16x4*)(dst + 16) = o1;
    }
    const float decay = fast_exp2(css[Q - 1]);
    acc[0] *= decay;
    acc[1] *= decay;
    // All of the chunk's operand reads first (one LDS latency per chunk), then
    // the scaling and MFMAs with chunk c + 2's loads spread among them.
    bf16x8 xr[K::KS], br[K::KS][2];
    f32x4 wa[K::KS], wb[K::KS];
#pragma unroll
    for (int ks = 0; ks < K::KS; ++ks) {
      const int k0 = 32 * ks + 8 * grp;
      const int ra = k0 + (L16 >> 2), rb = ra + 4;
      // x operand: column p = 16 pw + L16, K rows k0 .. k0 + 7
      const int xc = 2 * pw + ((L16 & 3) >> 1);
      xr[ks] = cat(lds_read_tr((const bf16*)(xs + ra * 64 + xswz(ra, xc) * 16 + xo)),
                   lds_read_tr((const bf16*)(xs + rb * 64 + xswz(rb, xc) * 16 + xo)));
      wa[ks] = *(const f32x4*)(wts + k0);
      wb[ks] = *(const f32x4*)(wts + k0 + 4);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int bc = 4 * nq + 2 * nt + ((L16 & 3) >> 1);
        br[ks][nt] = cat(lds_read_tr((const bf16*)(bs + ra * 128 + bswz(ra, bc) * 16 + xo)),
                         lds_read_tr((const bf16*)(bs + rb * 128 + bswz(rb, bc) * 16 + xo)));
      }
    }
#pragma unroll
    for (int ks = 0; ks < K::KS; ++ks) {
#pragma unroll
      for (int q = 0; q < K::PPK; ++q)
        load_piece<Q, N>(ks * K::PPK + q, nbuf, x, Bm, dA_cs, w_T, b, cn, h, g, p0, n0, L, H, G, nc);
      bf16x8 xop;  // scaled by w_j
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xop[e] = f2bf(bf2f(xr[ks][e]) * wa[ks][e]);
        xop[4 + e] = f2bf(bf2f(xr[ks][4 + e]) * wb[ks][e]);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt] = mfma16x16x32(br[ks][nt], xop, acc[nt]);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads spread as written
    }
    // Chunk c + 1 (loaded during the previous chunk) has landed once only this
    // chunk's two h_start stores and chunk c + 2's loads are newer.
    if (w < 2) wait_older<2 + K::LOADS + 1>(); else wait_older<2 + K::LOADS>();
    lds_barrier();
  }

  float* dst = final_state + ((int64_t)u * K::P + prow) * N + ncol;
  *(f32x4*)dst = acc[0];
  *(f32x4*)(dst + 16) = acc[1];
}

template <int Q, int N>
hipError_t launch_fused(const Dims& d, const void* x, const void* B, const float* dA_cs,
                        const float* w_T, const float* init, void* hst, float* final_state,
                        hipStream_t s) {
  using K = FCfg<Q, N>;
  auto kern = fwd_pass_state_kernel<Q, N>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS);
  if (attr != hipSuccess) return attr;
  const int64_t BH = d.B * d.H;
  const int64_t grid = (BH + 7) / 8 * 8 * K::TPH;
  kern<<<(unsigned)grid, K::NT, K::LDS, s>>>((const bf16*)x, (const bf16*)B, dA_cs, w_T, init,
                                           (bf16*)hst, final_state, (int)d.L, (int)d.H,
                                           (int)d.G, (int)d.nc, (int)BH);
  return hipGetLastError();
}

template <int Q>
hipError_t launch_fused_n(const Dims& d, const void* x, const void* B, const float* dA_cs,
                          const float* w_T, const float* init, void* hst, float* final_state,
                          hipStream_t s) {
  switch (d.N) {
    case 64: return launch_fused<Q, 64>(d, x, B, dA_cs, w_T, init, hst, final_state, s);
    case 128: return launch_fused<Q, 128>(d, x, B, dA_cs, w_T, init, hst, final_state, s);
    case 256: return launch_fused<Q, 256>(d, x, B, dA_cs, w_T, init, hst, final_state, s);
    default: return hipErrorInvalidValue;
  }
}

// w_T = 2^(cs[Q-1] - cs[j]) dt_j per (batch, head, chunk), the weights of the
// jump formula's B X^T contraction, computed once for every state tile.
__global__ void __launch_bounds__(256) chunk_weights_kernel(const float* __restrict__ dA_cs,
                                                            const float* __restrict__ dt_T,
                                                            float* __restrict__ w_T, int64_t n,
                                                            int Q) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t last = i - i % Q + (Q - 1);
  w_T[i] = fast_exp2(dA_cs[last] - dA_cs[i]) * dt_T[i];
}

}  // namespace

hipError_t launch_chunk_weights(const Dims& d, const float* dA_cs, const float* dt_T, float* w_T,
                                hipStream_t s) {
  const int64_t n = d.B * d.H * d.nc * d.Q;
  chunk_weights_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dA_cs, dt_T, w_T, n, (int)d.Q);
  return hipGetLastError();
}

bool fused_state_supported(const Dims& d) {
  return d.bf16 && d.P == 64 && (d.N == 64 || d.N == 128 || d.N == 256) &&
         (d.Q == 64 || d.Q == 128 || d.Q == 256);
}

hipError_t launch_fwd_pass_state(const Dims& d, const void* x, const void* B, const float* dA_cs,
                                 const float* w_T, const float* init, void* hst,
                                 float* final_state, hipStream_t s) {
  switch (d.Q) {
    case 64: return launch_fused_n<64>(d, x, B, dA_cs, w_T, init, hst, final_state, s);
    case 128: return launch_fused_n<128>(d, x, B, dA_cs, w_T, init, hst, final_state, s);
    case 256: return launch_fused_n<256>(d, x, B, dA_cs, w_T, init, hst, final_state, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m2
