// Backward pass of the chunked SSD: the in-chunk gradient kernels.  The pages
// give only the forward pass and note that a backward pass is still to be
// published (disconfirmai.com "Jane Street ML Engineers Map Mamba-2 Recurrent
// State Computation to Tensor Cores with cuTile", lead paragraph); what is
// computed here is the exact derivative of the forward's chunked form
// (devotd.net news item on the Mamba-2 CUDA Tile forward-pass kernels,
// section 2) written as matrix products.
//
// Per (batch, chunk, head), with cs the in-chunk cumulative log decay,
// M[i, j] = 2^(cs_i - cs_j) for i >= j (else 0), CB = C B^T of the head's
// group, dY and X the chunk's rows, h the chunk's start state, g the gradient
// reaching its end state (both [P, N]) and y~ the forward output without the
// D skip:
//     dU  = (M o CB)^T dY + diag(2^(cs_last - cs)) B g^T         [Q, P]
//     dx  = dt o dU + D dY
//     dC += (M o W) B + diag(2^cs) dY h,   W = dY (dt o X)^T       (summed over
//     dB += (M o W)^T C + diag(2^(cs_last - cs) dt) X g^T           the group's heads)
//     d(A dt)_k = sum_{i >= k > j} T_ij + sum_{i >= k} T^h_i + sum_{j < k} T^S_j
//                 + 2^cs_last <g, h>
//     ddt_k = x_k . dU_k + A d(A dt)_k,   dA = sum_k dt_k d(A dt)_k,  dD = sum dy . x
// with T_ij = (M o CB)_ij dt_j (dy_i . x_j) for i > j, T^h_i = 2^cs_i
// dy_i . (h C_i) and T^S_j = dt_j x_j . dU^state_j: each sum collects terms
// of single interactions whose decay spans position k, the form that does not
// cancel (the equivalent suffix sum of dy . y~ - dt x . dU subtracts nearly
// equal totals and loses the result to rounding).  <g, h> comes from the
// reverse state pass, T^h from chunk_bwd_dbdc.
//
// Four kernels share the work.  chunk_bwd_wsum: one workgroup per (batch,
// chunk, group); per head W is formed, masked and accumulated over the
// group's heads in float32 registers (the group sum is taken before the
// products with B and C, so those run once per group rather than once per
// head), with the rectangle sums of T.  chunk_bwd_dbdc: one workgroup per
// (batch, chunk, group, 64 state columns); per head the state terms (and
// their T^h parts) accumulate in registers; the products of the summed W
// with B and C follow once, from LDS.  chunk_bwd_dx: one workgroup per
// (batch, chunk, group, run of heads); C B^T of the group is formed once
// and kept in float32 accumulators; per head the masked, decayed tiles feed
// dU^T = dY^T (M o CB) + ... as MFMA operands straight from registers; the
// epilogue forms dx, the row dot products, ddt and the per-chunk parts of
// dA, dD.  Above state size 256, chunk_bwd_dus first forms dx's state term
// B g^T, which dx then reads.
//
// All use bfloat16 MFMA with float32 accumulation.  chunk_bwd_dx runs Q/32
// waves; wave w owns the output column tiles w and Q/16-1-w (equal causal
// work per wave) and the lower-triangle tiles of the Q x Q interaction
// matrix in the column strips of those two tiles (Q/16 + 1).
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

template <int Q>
struct BwdCfg {
  static constexpr int P = 64, QT = Q / 16, NW = Q / 32, NT = 64 * NW;
  static constexpr int NTILE = QT * (QT + 1) / 2;  // lower-triangle 16x16 tiles
  static constexpr int SLOTS = QT + 1;             // of them per wave
  static_assert(NTILE == NW * SLOTS, "triangle tiles split evenly over the waves");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The value, hidden from the optimiser: addresses computed from it inside a
// loop stay inside the loop instead of being hoisted out of it and held in
// registers for its whole length.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Triangle tile (ti >= tj) -> its index in the packed tile array.
__device__ __forceinline__ int tix_of(int ti, int tj) { return ti * (ti + 1) / 2 + tj; }

// Slot k of wave w: the row strips of tiles w and QT-1-w, (w, 0..w) then
// (QT-1-w, 0..QT-1-w): QT+1 tiles for every wave.
template <int QT>
__device__ __forceinline__ int slot_ti(int w, int k) { return k <= w ? w : QT - 1 - w; }
template <int QT>
__device__ __forceinline__ int slot_tj(int w, int k) { return k <= w ? k : k - w - 1; }

// LDS tiles are stored with their 16-byte chunks permuted per row so that
// the 16 rows an MFMA operand read touches fall on distinct banks.
// Element (r, col) of a [rows][64] tile (128-byte rows, 8 chunks):
__device__ __forceinline__ int t64(int r, int col) {
  return r * 64 + ((((col >> 3) ^ (r >> 1)) & 7) << 3) + (col & 7);
}
// The same for tiles read only by transposed 8-byte reads of 16 rows
// 8 g + q (g, q < 4) x 4 column pieces.  Such a read is served half a wave
// (g = 0, 1 or g = 2, 3) at a time; the chunk permutation follows bit 0 of
// g and bit 1 of q, so within each half the 32 lanes' pieces fall on all 64
// banks once.
__device__ __forceinline__ int swz_g(int r) { return 2 * (((r >> 3) & 1) | (((r >> 1) & 1) << 1)); }
__device__ __forceinline__ int t64g(int r, int col) {
  return r * 64 + ((((col >> 3) ^ swz_g(r)) & 7) << 3) + (col & 7);
}
// Element (r, col) of a [64][N] tile (N/8 chunks per row).
template <int N>
__device__ __forceinline__ int tN(int r, int col) {
  if constexpr (N >= 128)
    return r * N + (((col >> 3) ^ (r & 15)) << 3) + (col & 7);
  else
    return t64(r, col);
}

// rows [ROWS][64] of bfloat16 in registers on their way into an LDS tile;
// row r comes from src + r * stride (in elements), rows at or past `valid`
// are zero.  load() issues every 16-byte load of the thread before store()
// writes the first one, so a tile costs one memory latency rather than one
// per piece, and a caller can keep the next tile's loads in flight while it
// works on the current one.
template <int ROWS, int NT>
struct RowSlab {
  static constexpr int IT = (ROWS * 8 + NT - 1) / NT;
  bf16x8 v[IT];
  __device__ __forceinline__ void load(const bf16* __restrict__ src, int64_t stride,
                                       int64_t valid) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int s = threadIdx.x + it * NT;
      const int r = s >> 3, ch = s & 7;
      v[it] = zero8();
      if (s < ROWS * 8 && r < valid) v[it] = *(const bf16x8*)(src + (int64_t)r * stride + ch * 8);
    }
  }
  template <bool TG = false>
  __device__ __forceinline__ void store(bf16* dst) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int s = threadIdx.x + it * NT;
      if (s < ROWS * 8)
        *(bf16x8*)(dst + (TG ? t64g(s >> 3, (s & 7) * 8) : t64(s >> 3, (s & 7) * 8))) = v[it];
    }
  }
};

template <int ROWS, int NT, bool TG = false>
__device__ __forceinline__ void load_rows64(bf16* dst, const bf16* __restrict__ src,
                                            int64_t stride, int64_t valid) {
  RowSlab<ROWS, NT> slab;
  slab.load(src, stride, valid);
  slab.template store<TG>(dst);
}

// ---------------------------------------------------------------------------
// chunk_bwd_dx
// ---------------------------------------------------------------------------
// v + (v of the lane CTRL selects inside its 16-lane row), 0 where none.
template <int CTRL>
__device__ __forceinline__ float row_shr_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false);
  return v + __builtin_bit_cast(float, s);
}
// Inclusive prefix sum over the 16 lanes of each row (lane order).
__device__ __forceinline__ float row_scan16(float v) {
  v = row_shr_add<0x111>(v);
  v = row_shr_add<0x112>(v);
  v = row_shr_add<0x114>(v);
  return row_shr_add<0x118>(v);
}
typedef short s16x4v __attribute__((ext_vector_type(4)));

// D(16x16, f32) += A(16x16, bf16) * B(16x16, bf16): lane l holds A row (l & 15)
// and B column (l & 15) at K = 4 (l >> 4) .. +3, the accumulator as for the
// 16x16x32 form.  Its K layout is the accumulator's row layout, so a float32
// tile feeds it as a B operand straight from registers.
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4v, a),
                                                   __builtin_bit_cast(s16x4v, b), c, 0, 0, 0);
}

// v summed over the four 16-lane groups, in every lane: the lanes hold a
// 4 x 16 matrix (group k, lane j of the group), which is the B operand of a
// 16x16x4 float32 MFMA; against an A of ones every output row is the
// matrix's column sums.  One matrix-core instruction instead of two lane
// permutes through LDS, each waited for.
__device__ __forceinline__ float group_sum4(float v) {
  const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, v, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  return d[0];
}

// Slot k of wave w in chunk_bwd_dx: the column strips of tiles w and
// QT-1-w, (w..QT-1, w) then (QT-1-w..QT-1, QT-1-w): QT+1 tiles for every wave.
template <int QT>
__device__ __forceinline__ int cslot_strip(int w, int k) { return k < QT - w ? 0 : 1; }
template <int QT>
__device__ __forceinline__ int cslot_ti(int w, int k) {
  return k < QT - w ? w + k : (QT - 1 - w) + (k - (QT - w));
}
template <int QT>
__device__ __forceinline__ int cslot_tj(int w, int k) { return k < QT - w ? w : QT - 1 - w; }

template <int Q, int N>
struct DxLds {
  using K = BwdCfg<Q>;
  static constexpr int nT = N / 64;
  // the state term comes precomputed (chunk_bwd_dus) above N = 256
  static constexpr bool EXT = N > 256;
  // one head's buffer: g [64][N] (tN order; none with EXT), dY [Q][64] (t64
  // order), cs, dt, T^h parts [nT][Q], rectangle sums R [Q], boundary dot
  // parts [64]
  static constexpr int GS = 0, YS = EXT ? 0 : 64 * N * 2, CS = YS + Q * 128, DT = CS + Q * 4;
  static constexpr int TH = DT + Q * 4, RS = TH + nT * Q * 4, DOT = RS + Q * 4;
  // the reverse pass's boundary dot parts: one per wave of a head there
  // (256-thread blocks over P N / 4 entries), at least 64 slots
  static constexpr int NDOT = (64 * N / 4 + 255) / 256 * 4;
  static constexpr int BUF = DOT + (NDOT > 64 ? NDOT : 64) * 4;
  static constexpr int SM = 2 * BUF;                  // x.dU, T^S [Q] each
  static constexpr int RED = SM + 2 * Q * 4;          // per-wave dy.x parts
  static constexpr int BYTES = RED + 64;
  static_assert(2 * Q * 128 <= 2 * BUF, "setup slices of C and B fit in the head buffers");
};

// Issues the direct-to-LDS loads of one head's buffer.
template <int Q, int N>
__device__ __forceinline__ void issue_dx_loads(uint32_t buf, const bf16* __restrict__ gsrc,
                                               const bf16* __restrict__ dyr, int64_t stride,
                                               int64_t valid, const float* __restrict__ cs,
                                               const float* __restrict__ dt,
                                               const float* __restrict__ thp,
                                               const float* __restrict__ rs,
                                               const float* __restrict__ dp, int wph) {
  using S = DxLds<Q, N>;
  constexpr int TH4 = S::nT * Q / 4;  // 16-byte pieces of the T^h parts
  constexpr int NW = BwdCfg<Q>::NW, KG = S::EXT ? 0 : N / 8, KY = Q / 8, KTH = (TH4 + 63) / 64;
  constexpr int KTOT = KG + KY + KTH + 4;
  const int lane = lane_id();
  for (int k = wave_id(); k < KTOT; k += NW) {
    if (k < KG) {  // g rows: N/8 chunks each
      const int s = k * 64 + lane;
      const int r = s / (N / 8), pos = s % (N / 8);
      const int ch = (N >= 128) ? (pos ^ (r & 15)) : (pos ^ ((r >> 1) & 7));
      dma16(gsrc + (int64_t)r * N + ch * 8, buf + S::GS + k * 1024);
    } else if (k < KG + KY) {  // dY rows (past the sequence end: the last row again)
      const int s = (k - KG) * 64 + lane;
      int r = s >> 3;
      const int ch = (s & 7) ^ ((r >> 1) & 7);
      if (r > valid - 1) r = (int)(valid - 1);
      dma16(dyr + (int64_t)r * stride + ch * 8, buf + S::YS + (k - KG) * 1024);
    } else if (k < KG + KY + KTH) {
      const int kk = k - KG - KY;
      if (kk * 64 + lane < TH4) dma16(thp + (kk * 64 + lane) * 4, buf + S::TH + kk * 1024);
    } else {
      const int kk = k - KG - KY - KTH;  // 0: cs, 1: dt, 2: R, 3: dot parts
      const int n4 = kk == 3 ? wph / 4 : Q / 4;
      const float* src = kk == 0 ? cs : kk == 1 ? dt : kk == 2 ? rs : dp;
      const int off = kk == 0 ? S::CS : kk == 1 ? S::DT : kk == 2 ? S::RS : S::DOT;
      if (lane < n4) dma16(src + lane * 4, buf + off + lane * 16);
    }
  }
}

// ---------------------------------------------------------------------------
// chunk_bwd_dus (state size 512)
// ---------------------------------------------------------------------------
// The state term of dU before its row decay, dUs[j, p] = sum_n B[j, n] g[p, n]
// (g: the gradient reaching the chunk's end, bf16 [P, N]), for a state size
// whose B operands do not fit beside chunk_bwd_dx's other registers; dx
// then reads it instead of forming it.  One workgroup per (batch, chunk,
// group, run of heads), 8 waves, Q = 256: wave w owns the chunk's row tiles
// w and w + 8, whose B rows stay in registers as MFMA operands for every
// head of the run.  Each head's g arrives by direct-to-LDS loads into a
// double buffer, each row's 16-byte chunks permuted by the row's low four
// bits, so the 16 rows of an operand read fall on distinct banks.  Output
// float32 [B, L, H, P], in the layout of dx's accumulators: lane (L16, grp)
// of p tile pt holds rows j = 16 t + L16, columns 16 pt + 4 grp .. + 3.
template <int N>
struct DusCfg {
  static constexpr int Q = 256, P = 64, NW = 8, NT = 512, KB = N / 32;
  static constexpr int RCH = N / 8;      // 16-byte chunks per g row
  static constexpr int BUF = P * N * 2;  // one head's g
  static constexpr int LDS = 2 * BUF;
  static_assert(RCH % 16 == 0, "row permutation stays inside the row");
};

__device__ __forceinline__ int gswz(int r, int ch) { return ch ^ (r & 15); }

template <int N>
__global__ void __launch_bounds__(512, 1) chunk_bwd_dus_kernel(
    const bf16* __restrict__ Bm, const bf16* __restrict__ gst, float* __restrict__ dus, int L,
    int H, int G, int nc, int hpw, int slices) {
  using K = DusCfg<N>;
  constexpr int P = K::P, Q = K::Q, KB = K::KB;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  int bid = blockIdx.x;
  const int slice = bid % slices;
  bid /= slices;
  const int g = bid % G;
  bid /= G;
  const int c = bid % nc;
  const int b = bid / nc;
  const int HG = H / G;
  const int h0 = g * HG + slice * hpw;
  const int nh = min(hpw, HG - slice * hpw);
  if (nh <= 0) return;  // whole workgroup

  const int lane = lane_id();
  const int w = wave_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int64_t tok0 = (int64_t)c * Q;
  const int64_t valid = (int64_t)L - tok0;
  const uint32_t base = lds_addr(smem);

  // head h's g into buffer `buf`: P * N / 512 wave-loads of 1 KB
  auto issue = [&](int h, int buf) {
    const bf16* src = gst + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
    for (int k = w; k < P * N / 512; k += K::NW) {
      const int s = k * 64 + lane;
      const int r = s / K::RCH, pos = s % K::RCH;
      dma16(src + (int64_t)r * N + gswz(r, pos) * 8, base + buf * K::BUF + k * 1024);
    }
  };
  const int rot = c % nh;
  const auto head_at = [&](int k) { return h0 + (k + rot < nh ? k + rot : k + rot - nh); };
  issue(head_at(0), 0);

  // B operands of this wave's two row tiles (zero past the sequence end)
  bf16x8 bop[2][KB];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = (w + 8 * s) * 16 + L16;
    const bf16* src = Bm + (((int64_t)b * L + tok0 + i) * G + g) * N + 8 * grp;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bop[s][kb] = zero8();
      if (i < valid) bop[s][kb] = *(const bf16x8*)(src + 32 * kb);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int k = 0; k < nh; ++k) {
    const int h = head_at(k);
    if (k + 1 < nh) issue(head_at(k + 1), (k + 1) & 1);
    const bf16* gs = (const bf16*)(smem + (k & 1) * K::BUF);
    f32x4 acc[2][4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[0][pt] = acc[1][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int r = pt * 16 + L16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = *(const bf16x8*)(gs + r * N + gswz(r, 4 * kb + grp) * 8);
        acc[0][pt] = mfma16x16x32(a, bop[0][kb], acc[0][pt]);
        acc[1][pt] = mfma16x16x32(a, bop[1][kb], acc[1][pt]);
      }
    }
    // the next head's g has landed (and this wave's older stores drained):
    // then this head's stores, which the next such wait covers a head later
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int i = (w + 8 * s) * 16 + L16;
      if (i < valid) {
        float* dst = dus + (((int64_t)b * L + tok0 + i) * H + h) * P + 4 * grp;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) *(f32x4*)(dst + 16 * pt) = acc[s][pt];
      }
    }
    lds_barrier();  // every wave's g landed; the buffer just read is free
  }
}

// The log-decay gradient is formed without cancellation: for position k,
//   d(A dt)_k = R_k + sum_{i >= k} T^h_i + sum_{j < k} T^S_j + 2^cs_last <g, h_start>,
// R_k = sum_{i >= k > j} (M o CB)_ij dt_j (dy_i . x_j) (from the summed-W
// kernel), T^h_i = 2^cs_i dy_i . (h_start C_i) (from the dB/dC kernel) and
// T^S_j = dt_j x_j . dU^state_j (here).  Every sum is of terms of single
// interactions, so no large opposite contributions cancel.
template <int Q, int N>
__global__ void __launch_bounds__(BwdCfg<Q>::NT, 1) chunk_bwd_dx_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ dy, const bf16* __restrict__ Bm,
    const bf16* __restrict__ Cm, const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    const bf16* __restrict__ gst, const float* __restrict__ dots, const float* __restrict__ th,
    const float* __restrict__ rsum, const float* __restrict__ A, const float* __restrict__ D,
    bf16* __restrict__ dx, bf16* __restrict__ ddt, float* __restrict__ dA_part,
    float* __restrict__ dD_part, const float* __restrict__ dus, int L, int H, int G, int nc,
    int hpw, int slices, int wph) {
  using K = BwdCfg<Q>;
  using S = DxLds<Q, N>;
  // EXT: the state term B g^T arrives from chunk_bwd_dus (float32 [B, L, H,
  // P], before its row decay) instead of being formed here from resident B
  // operands, which would not fit in the registers at this state size
  constexpr bool EXT = S::EXT;
  constexpr int P = 64, QT = K::QT, NW = K::NW, NT = K::NT, SLOTS = K::SLOTS;
  constexpr int KN = EXT ? 1 : N / 32;
  constexpr int nT = S::nT;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  int bid = blockIdx.x;
  const int slice = bid % slices;
  bid /= slices;
  const int g = bid % G;
  bid /= G;
  const int c = bid % nc;
  const int b = bid / nc;
  const int HG = H / G;
  const int h0 = g * HG + slice * hpw;
  const int nh = min(hpw, HG - slice * hpw);
  if (nh <= 0) return;  // whole workgroup

  const int lane = lane_id();
  const int w = wave_id();
  const int64_t tok0 = (int64_t)c * Q;
  const int64_t valid = (int64_t)L - tok0;  // rows of this chunk inside the sequence
  const int J[2] = {w, QT - 1 - w};
  const uint32_t base = lds_addr(smem);

  // ---- C B^T of the group (float32, this wave's column strips) and the
  // B operands of this wave's output columns for the state term.
  f32x4 cb[SLOTS];
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) cb[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 Bop[2][KN];
  {
    const int L16 = lane & 15, grp = lane >> 4;
    bf16* Cs = (bf16*)smem;
    bf16* Bs = Cs + Q * 64;
    const int64_t row0 = ((int64_t)b * L + tok0) * G + g;
    // 64-column slices of C and B.  Above N = 256 (eight slices) the next
    // slice's loads fly while the current one's MFMAs run (at N = 256 that
    // measured 5 us slower, so there each slice is loaded, then used).
    RowSlab<Q, NT> sc, sb;
    if constexpr (EXT) {
      sc.load(Cm + row0 * N, (int64_t)G * N, valid);
      sb.load(Bm + row0 * N, (int64_t)G * N, valid);
    }
#pragma unroll
    for (int ns = 0; ns < N / 64; ++ns) {
      if constexpr (EXT) {
        lds_barrier();  // every wave is done with the previous slice
        sc.store(Cs);
        sb.store(Bs);
        if (ns + 1 < N / 64) {
          sc.load(Cm + row0 * N + (ns + 1) * 64, (int64_t)G * N, valid);
          sb.load(Bm + row0 * N + (ns + 1) * 64, (int64_t)G * N, valid);
        }
        lds_barrier();  // this slice visible to every wave
      } else {
        __syncthreads();
        load_rows64<Q, NT>(Cs, Cm + row0 * N + ns * 64, (int64_t)G * N, valid);
        load_rows64<Q, NT>(Bs, Bm + row0 * N + ns * 64, (int64_t)G * N, valid);
        __syncthreads();
      }
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const int ti = cslot_ti<QT>(w, k), tj = cslot_tj<QT>(w, k);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 a = *(const bf16x8*)(Cs + t64(ti * 16 + L16, 32 * kk + 8 * grp));
          const bf16x8 bb = *(const bf16x8*)(Bs + t64(tj * 16 + L16, 32 * kk + 8 * grp));
          cb[k] = mfma16x16x32(a, bb, cb[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!EXT) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            Bop[s][2 * ns + kk] = *(const bf16x8*)(Bs + t64(J[s] * 16 + L16, 32 * kk + 8 * grp));
      }
    }
    __syncthreads();  // slices consumed before the head buffers take their space
  }

  auto issue = [&](int h, int slot) {
    const int64_t xrow0 = (((int64_t)b * L + tok0) * H + h) * P;
    const int64_t cb0 = (((int64_t)b * H + h) * nc + c) * Q;
    issue_dx_loads<Q, N>(base + slot * S::BUF,
                         gst + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N, dy + xrow0,
                         (int64_t)H * P, valid, dA_cs + cb0, dt_T + cb0,
                         th + (((int64_t)b * nc + c) * H + h) * nT * Q, rsum + cb0,
                         dots + (((int64_t)b * H + h) * nc + c) * wph, wph);
  };

  float* exs = (float*)(smem + S::SM);
  float* tsv = exs + Q;
  float* red = (float*)(smem + S::RED);

  // this lane's x values of head h in the accumulator layout (zero past the
  // end); loaded one head ahead, so that no wait inside a head's work would
  // also wait for the next head's direct-to-LDS loads
  bf16x4 xr[2][4];
  f32x4 dsr[2][EXT ? 4 : 1];  // EXT: the precomputed state term, same layout
  // (strip s's values as soon as that strip of the previous head is done)
  auto load_x = [&](int h, int s) {
    const int L16 = opaque(lane & 15), grp = opaque(lane >> 4);
    const int64_t xrow0 = (((int64_t)b * L + tok0) * H + h) * P;
    const int j = J[s] * 16 + L16;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      xr[s][pt] = __builtin_bit_cast(bf16x4, (short __attribute__((ext_vector_type(4)))){0, 0, 0, 0});
      if (j < valid)
        xr[s][pt] = *(const bf16x4*)(x + xrow0 + (int64_t)j * H * P + pt * 16 + 4 * grp);
      if constexpr (EXT) {
        dsr[s][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < valid) dsr[s][pt] = *(const f32x4*)(dus + xrow0 + (int64_t)j * H * P + pt * 16 + 4 * grp);
      }
    }
  };

  // each workgroup walks its heads from a different one, so the workgroups
  // in flight touch different heads' slices of the token rows
  const int rot = c % nh;
  const auto head_at = [&](int k) { return h0 + (k + rot < nh ? k + rot : k + rot - nh); };
  issue(head_at(0), 0);
  load_x(head_at(0), 0);
  load_x(head_at(0), 1);
  for (int hh = 0; hh < nh; ++hh) {
    const int h = head_at(hh);
    __builtin_amdgcn_s_waitcnt(0);  // this head's buffer and x values landed
    __syncthreads();                // ... for every wave; the other buffer is free
    if (hh + 1 < nh) issue(head_at(hh + 1), (hh + 1) & 1);
    const unsigned char* cur = smem + (hh & 1) * S::BUF;
    const bf16* Gs = (const bf16*)(cur + S::GS);
    const bf16* Ys = (const bf16*)(cur + S::YS);
    const float* css = (const float*)(cur + S::CS);
    const float* dts = (const float*)(cur + S::DT);
    const int L16 = opaque(lane & 15), grp = opaque(lane >> 4);
    const int64_t xrow0 = (((int64_t)b * L + tok0) * H + h) * P;

    // One pass per output column tile s (tiles w and QT-1-w): the state
    // term of dU^T[p][j], scaled per column by 2^(cs_last - cs_j), T^S_j,
    // the causal part sum_{i >= j} dY^T[p][i] (M o CB)[i][j] with the masked,
    // decayed C B^T tile of each slot of the strip used as the B operand from
    // registers (16x16x16: its K rows are the accumulator's rows), and the
    // epilogue.  acc[pt][r] = dU[j = 16 J[s] + L16][p = 16 pt + 4 grp + r].
    const float csL = css[Q - 1];
    const float Dh = D ? D[h] : 0.f;
    float dd = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int j = J[s] * 16 + L16;
      f32x4 acc[4];
      if constexpr (EXT) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = dsr[s][pt];
      } else {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KN; ++ks) {
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            const bf16x8 a = *(const bf16x8*)(Gs + tN<N>(pt * 16 + L16, 32 * ks + 8 * grp));
            acc[pt] = mfma16x16x32(a, Bop[s][ks], acc[pt]);
          }
        }
      }
      const float sc = fast_exp2(csL - css[j]);
      float ts = 0.f;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[pt][r] *= sc;
          ts += bf2f(xr[s][pt][r]) * acc[pt][r];
        }
      ts = group_sum4(ts);
      if (grp == 0) tsv[j] = dts[j] * ts;  // T^S_j

      const float csj = css[j];
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        if (cslot_strip<QT>(w, k) == s) {
          // the slot's dY^T operands and row cs, all read before any is used
          const int ti = cslot_ti<QT>(w, k);
          const int yr = ti * 16 + 4 * grp + (L16 >> 2);
          bf16x4 ya[4];
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) ya[pt] = lds_read_tr(Ys + t64(yr, pt * 16 + 4 * (L16 & 3)));
          const f32x4 yc = *(const f32x4*)(css + ti * 16 + 4 * grp);
          bf16x4 bop;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = ti * 16 + 4 * grp + r;
            const float e = fast_exp2(fminf(yc[r] - csj, 0.f)) * cb[k][r];
            bop[r] = f2bf(i >= j ? e : 0.f);
          }
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) acc[pt] = mfma16x16x16(ya[pt], bop, acc[pt]);
        }
      }

      float ex = 0.f;
      if (j < valid) {
        const float dtj = dts[j];
        const int64_t off = xrow0 + (int64_t)j * H * P;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const int p0 = pt * 16 + 4 * grp;
          const bf16x4 dv = *(const bf16x4*)(Ys + t64(j, p0));
          bf16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float du = acc[pt][r], xf = bf2f(xr[s][pt][r]), df = bf2f(dv[r]);
            o[r] = f2bf(dtj * du + Dh * df);
            ex += xf * du;
            dd += df * xf;
          }
          *(bf16x4*)(dx + off + p0) = o;
        }
      }
      ex = group_sum4(ex);
      if (grp == 0) exs[j] = ex;
      if (hh + 1 < nh) load_x(head_at(hh + 1), s);
    }
    const float Ah = A[h];
    dd = wave_sum(dd);
    if (lane == 0) red[w] = dd;
    lds_barrier();  // LDS only: the loads in flight keep flying

    // ---- d(A dt)_k, ddt, and the dA and dD parts (one wave)
    if (w == 0) {
      constexpr int E = Q / 64;
      const float* rsv = (const float*)(cur + S::RS);
      const float* thv = (const float*)(cur + S::TH);
      const float* dpv = (const float*)(cur + S::DOT);
      float dp = 0.f;
      for (int i = lane; i < wph; i += 64) dp += dpv[i];
      const float dc = wave_sum(dp);
      float rk[E], ps[E], sh[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int k = lane * E + e;
        rk[e] = rsv[k];
        ps[e] = tsv[k];
        float t = 0.f;
#pragma unroll
        for (int nt = 0; nt < nT; ++nt) t += thv[nt * Q + k];
        sh[e] = t;
      }
      // suffix sums of T^h (over i >= k) and exclusive prefix sums of T^S
      // (over j < k): inside the lane, then across lanes
#pragma unroll
      for (int e = E - 2; e >= 0; --e) sh[e] += sh[e + 1];
      float run = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float v = ps[e];
        ps[e] = run;
        run += v;
      }
      float suf = sh[0], pre = run;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float a = __shfl_down(suf, off, 64);
        const float bq = __shfl_up(pre, off, 64);
        if (lane + off < 64) suf += a;
        if (lane >= off) pre += bq;
      }
      float suf_after = __shfl_down(suf, 1, 64);
      if (lane == 63) suf_after = 0.f;
      float pre_before = __shfl_up(pre, 1, 64);
      if (lane == 0) pre_before = 0.f;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int k = lane * E + e;
        const float da = rk[e] + sh[e] + suf_after + ps[e] + pre_before + dc;
        if (k < valid) ddt[((int64_t)b * L + tok0 + k) * H + h] = f2bf(exs[k] + Ah * da);
        part += dts[k] * da;
      }
      part = wave_sum(part);
      if (lane == 0) {
        float sd = 0.f;
        for (int i = 0; i < NW; ++i) sd += red[i];
        dA_part[((int64_t)b * nc + c) * H + h] = part;
        dD_part[((int64_t)b * nc + c) * H + h] = sd;
      }
    }
  }
}

// Issues the direct-to-LDS loads of one head's dY and x rows of the chunk
// ([Q][64] each, t64 chunk order; rows past the sequence end repeat its last
// row and must be masked by the consumer) and its cs and dt rows.
template <int Q>
__device__ __forceinline__ void issue_rows_loads(uint32_t buf, const bf16* __restrict__ dyr,
                                                 const bf16* __restrict__ xr, int64_t stride,
                                                 int64_t valid, const float* __restrict__ cs,
                                                 const float* __restrict__ dt) {
  constexpr int NW = BwdCfg<Q>::NW, KT = Q / 8;  // wave-loads (1 KB) per tile
  const int lane = lane_id();
  for (int k = wave_id(); k < 2 * KT + 2; k += NW) {
    if (k < 2 * KT) {
      const int s = (k % KT) * 64 + lane;
      int r = s >> 3;
      const int ch = (s & 7) ^ ((r >> 1) & 7);
      if (r > valid - 1) r = (int)(valid - 1);
      dma16((k < KT ? dyr : xr) + (int64_t)r * stride + ch * 8, buf + k * 1024);
    } else if (lane < Q / 4) {
      dma16((k == 2 * KT ? cs : dt) + lane * 4, buf + 2 * Q * 128 + (k - 2 * KT) * Q * 4);
    }
  }
}

template <int Q>
struct WsLds {
  static constexpr int BUF = 2 * Q * 128 + 2 * Q * 4;  // dY, x rows; cs, dt
  static constexpr int RP = 2 * BUF;                    // column-sum parts, 2 x [NW][Q]
  static constexpr int RS = RP + 2 * BwdCfg<Q>::NW * Q * 4;  // row sums, 2 x [Q]
  static constexpr int BYTES = RS + 2 * Q * 4;
  static_assert(2 * Q * 128 <= 2 * BUF, "setup slices of C and B fit in the head buffers");
  static_assert(Q <= 256, "one wave forms the prefix over the chunk");
};

// Inclusive prefix sum over the 64 lanes of a wave: inside each 16-lane row,
// then each row total carried into the rows above it (row_bcast 15 into rows
// 1 and 3, row_bcast 31 into rows 2 and 3).
__device__ __forceinline__ float wave_scan64(float v) {
  v = row_scan16(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
  return v;
}

// Per head also the rectangle sums of the log-decay gradient,
//     R_k = sum_{i >= k > j} T_ij,   T_ij = (M o CB)_ij dt_j (dy_i . x_j),
// from the same W tiles.  Going from k to k + 1 the rectangle gains column
// k below the diagonal and loses row k left of it, so
//     R_k = sum_{m < k} (colsum_m - rowsum_m),
//     colsum_m = sum_{i > m} T_im,   rowsum_m = sum_{j < m} T_mj.
// Per tile each lane adds its T values into running row sums (one per row
// it holds, over the strip) and a column sum (over its rows, then across the
// four lane groups); after the head the row sums are reduced across their 16
// lanes, and one wave forms the prefix over the chunk from the per-wave
// column parts and the row sums.
template <int Q>
__global__ void __launch_bounds__(BwdCfg<Q>::NT, 1) chunk_bwd_wsum_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ dy, const bf16* __restrict__ Bm,
    const bf16* __restrict__ Cm, const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    bf16* __restrict__ wsum, float* __restrict__ rsum, int L, int H, int G, int nc, int N) {
  using K = BwdCfg<Q>;
  using S = WsLds<Q>;
  constexpr int P = 64, QT = K::QT, NW = K::NW, NT = K::NT, SLOTS = K::SLOTS;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  int bid = blockIdx.x;
  const int g = bid % G;
  bid /= G;
  const int c = bid % nc;
  const int b = bid / nc;
  const int HG = H / G;
  const int lane = lane_id();
  const int w = wave_id();
  const int64_t tok0 = (int64_t)c * Q;
  const int64_t valid = (int64_t)L - tok0;
  const uint32_t base = lds_addr(smem);
  float* rp = (float*)(smem + S::RP);
  float* rs = (float*)(smem + S::RS);

  // ---- C B^T of the group on this wave's triangle tiles (float32)
  f32x4 cb[SLOTS];
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) cb[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const int L16 = lane & 15, grp = lane >> 4;
    bf16* Cs = (bf16*)smem;
    bf16* Bs = Cs + Q * 64;
    const int64_t row0 = ((int64_t)b * L + tok0) * G + g;
    // 64-column slices of C and B, the next slice's loads in flight while
    // the current one's MFMAs run
    RowSlab<Q, NT> sc, sb;
    sc.load(Cm + row0 * N, (int64_t)G * N, valid);
    sb.load(Bm + row0 * N, (int64_t)G * N, valid);
    for (int ns = 0; ns < N / 64; ++ns) {
      lds_barrier();  // every wave is done with the previous slice
      sc.store(Cs);
      sb.store(Bs);
      if (ns + 1 < N / 64) {
        sc.load(Cm + row0 * N + (ns + 1) * 64, (int64_t)G * N, valid);
        sb.load(Bm + row0 * N + (ns + 1) * 64, (int64_t)G * N, valid);
      }
      lds_barrier();  // this slice visible to every wave
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const int ti = slot_ti<QT>(w, k), tj = slot_tj<QT>(w, k);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 a = *(const bf16x8*)(Cs + t64(ti * 16 + L16, 32 * kk + 8 * grp));
          const bf16x8 bb = *(const bf16x8*)(Bs + t64(tj * 16 + L16, 32 * kk + 8 * grp));
          cb[k] = mfma16x16x32(a, bb, cb[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    for (int i = threadIdx.x; i < 2 * NW * Q; i += NT) rp[i] = 0.f;
    __syncthreads();  // slices consumed before the head buffers take their space
  }

  auto issue = [&](int h, int slot) {
    const int64_t xrow0 = (((int64_t)b * L + tok0) * H + h) * P;
    const int64_t cb0 = (((int64_t)b * H + h) * nc + c) * Q;
    issue_rows_loads<Q>(base + slot * S::BUF, dy + xrow0, x + xrow0, (int64_t)H * P, valid,
                        dA_cs + cb0, dt_T + cb0);
  };
  // R of head h from the column parts in rp[buf] (zeroed for reuse) and the
  // row sums in rs[buf], by wave `fw`: lane l takes m = 4 l .. 4 l + 3
  auto finish_rect = [&](int h, int buf, int fw) {
    if (w != fw) return;
    float* part = rp + buf * NW * Q;
    const float* rows = rs + buf * Q;
    float d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * lane + e;
      float v = 0.f;
      if (m < Q) {
        for (int i = 0; i < NW; ++i) {
          v += part[i * Q + m];
          part[i * Q + m] = 0.f;
        }
        v -= rows[m];
      }
      d[e] = v;
    }
    const float tot = ((d[0] + d[1]) + d[2]) + d[3];
    const float pre = wave_scan64(tot) - tot;  // sum over the lanes below
    float* out = rsum + (((int64_t)b * H + h) * nc + c) * Q;
    if (4 * lane < Q) {
      const float r1 = pre + d[0], r2 = r1 + d[1], r3 = r2 + d[2];
      *(f32x4*)(out + 4 * lane) = f32x4{pre, r1, r2, r3};
    }
  };

  f32x4 ws[SLOTS];
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) ws[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(g * HG, 0);
  for (int hh = 0; hh < HG; ++hh) {
    __builtin_amdgcn_s_waitcnt(0);  // this head's rows landed
    __syncthreads();                // ... for every wave; the other buffer is free
    // (before the next head's loads are issued: anything the compiler waits
    // for here would otherwise wait for them too)
    if (hh > 0) finish_rect(g * HG + hh - 1, (hh - 1) & 1, (hh - 1) % NW);
    if (hh + 1 < HG) issue(g * HG + hh + 1, (hh + 1) & 1);
    const unsigned char* cur = smem + (hh & 1) * S::BUF;
    const bf16* Ys = (const bf16*)cur;
    const bf16* Xs = (const bf16*)(cur + Q * 128);
    const float* css = (const float*)(cur + 2 * Q * 128);
    const float* dts = css + Q;
    float* part = rp + (hh & 1) * NW * Q + w * Q;
    const int L16 = opaque(lane & 15), grp = opaque(lane >> 4);
    float* rows = rs + (hh & 1) * Q;
    // running row sums of the current strip: at its end, across the 16 lanes
    // of each row into rows[]
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
    auto flush_rows = [&](int ti) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float t = row_scan16(rsum[r]);
        if (L16 == 15) rows[ti * 16 + 4 * grp + r] = t;
        rsum[r] = 0.f;
      }
    };
    // cs of this lane's rows in its two strips (rows past the sequence end
    // hold a repeated row: masked through vq)
    const int vq = valid < Q ? (int)valid : Q;
    float ci[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ci[0][r] = css[w * 16 + 4 * grp + r];
      ci[1][r] = css[(QT - 1 - w) * 16 + 4 * grp + r];
    }
    // Software pipeline over the wave's tiles: while tile k's elementwise
    // work runs, the MFMAs of tile k + 1 (operands read during tile k - 1)
    // and the LDS reads of tile k + 2 are in flight.
    // dY operands of the wave's two row strips, read once per head (every
    // tile of a strip shares them); the x operands per tile
    bf16x8 ya[2][2], ob[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      ya[0][kk] = *(const bf16x8*)(Ys + t64(w * 16 + L16, 32 * kk + 8 * grp));
      ya[1][kk] = *(const bf16x8*)(Ys + t64((QT - 1 - w) * 16 + L16, 32 * kk + 8 * grp));
    }
    float ocs[2], odt[2];  // column cs and dt of tiles k + 1 (even/odd slot)
    auto read_tile = [&](int k) {
      const int tj = slot_tj<QT>(w, k);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) ob[kk] = *(const bf16x8*)(Xs + t64(tj * 16 + L16, 32 * kk + 8 * grp));
      ocs[k & 1] = css[tj * 16 + L16];
      odt[k & 1] = dts[tj * 16 + L16];
    };
    auto tile_mma = [&](int k) {
      f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k <= w) {  // wave-uniform: the strip of row tile w
        a4 = mfma16x16x32(ya[0][0], ob[0], a4);
        a4 = mfma16x16x32(ya[0][1], ob[1], a4);
      } else {
        a4 = mfma16x16x32(ya[1][0], ob[0], a4);
        a4 = mfma16x16x32(ya[1][1], ob[1], a4);
      }
      return a4;
    };
    read_tile(0);
    f32x4 an = tile_mma(0);
    read_tile(1);
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
      const int ti = slot_ti<QT>(w, k), tj = slot_tj<QT>(w, k);
      const f32x4 a4 = an;
      const float csj = ocs[k & 1], dtj = odt[k & 1];
      if (k + 1 < SLOTS) an = tile_mma(k + 1);
      if (k + 2 < SLOTS) read_tile(k + 2);
      const int j = tj * 16 + L16;
      const bool first = k <= w;  // wave-uniform: tile of the strip of row tile w
      float col = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ti * 16 + 4 * grp + r;
        const float d = fminf((first ? ci[0][r] : ci[1][r]) - csj, 0.f);
        const float ev = fast_exp2(d) * dtj;
        const float e = (i >= j && i < vq) ? ev : 0.f;
        const float wm = e * a4[r];
        ws[k][r] += wm;
        const float t = (i > j) ? cb[k][r] * wm : 0.f;
        rsum[r] += t;
        col += t;
      }
      // column j's total over the four lane groups, added into its LDS part
      // by the first group (an add without return: nothing waits for it)
      col = group_sum4(col);
      if (grp == 0) __hip_atomic_fetch_add(part + j, col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (k == w) flush_rows(w);  // end of the first strip (wave-uniform)
      __builtin_amdgcn_sched_barrier(0);
    }
    flush_rows(QT - 1 - w);
  }
  __syncthreads();
  finish_rect(g * HG + HG - 1, (HG - 1) & 1, (HG - 1) % NW);

  const int L16 = lane & 15, grp = lane >> 4;
  bf16* out = wsum + (((int64_t)b * nc + c) * G + g) * (int64_t)(K::NTILE * 256);
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    bf16* dst = out + tix_of(slot_ti<QT>(w, k), slot_tj<QT>(w, k)) * 256 + 4 * grp * 16 + L16;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r * 16] = f2bf(ws[k][r]);
  }
}

// ---------------------------------------------------------------------------
// chunk_bwd_dbdc
// ---------------------------------------------------------------------------
// Q/32 waves: wave w owns output row tiles w and Q/16-1-w of dB and dC (row
// tile t has t+1 causal tiles for dC and Q/16-t for dB: Q/16+1 per pair, so
// every wave has the same work).  Per head the wave's own rows of dY and x go
// straight to registers in MFMA operand order, loaded one head ahead, and the
// shared h and g column tiles, cs and dt arrive by direct-to-LDS loads into a
// double buffer: the next head's bytes are in flight while this head computes.
template <int Q>
struct BcCfg {
  static constexpr int QT = Q / 16, NW = Q / 32, NT = 64 * NW;
};

template <int Q>
struct BcLds {
  static constexpr int BS = 0;                 // B columns [Q][64]
  static constexpr int CS = BS + Q * 128;      // C columns [Q][64]
  static constexpr int BUF = 2 * 8192 + 2 * Q * 4;  // h, g columns [64][64]; cs, dt
  static constexpr int HEAD = CS + Q * 128;    // two head buffers, later the summed W
  static constexpr int WT = BwdCfg<Q>::NTILE * 512;
  static constexpr int BYTES = HEAD + (WT > 2 * BUF ? WT : 2 * BUF);
};

// Issues the direct-to-LDS loads of one head's h and g column tiles (64 rows
// x 64 columns, stored with the t64g chunk order) and its cs and dt rows.
template <int Q>
__device__ __forceinline__ void issue_head_loads(uint32_t buf, const bf16* __restrict__ hsrc,
                                                 const bf16* __restrict__ gsrc, int N,
                                                 const float* __restrict__ cs,
                                                 const float* __restrict__ dt) {
  constexpr int NW = BcCfg<Q>::NW;
  const int lane = lane_id();
  for (int k = wave_id(); k < 18; k += NW) {
    if (k < 16) {
      const int s = (k & 7) * 64 + lane;  // chunk at LDS position s of the tile
      const int r = s >> 3, ch = (s & 7) ^ swz_g(r);
      dma16((k < 8 ? hsrc : gsrc) + (int64_t)r * N + ch * 8, buf + (k >> 3) * 8192 + (k & 7) * 1024);
    } else if (lane < Q / 4) {
      dma16((k == 16 ? cs : dt) + lane * 4, buf + 16384 + (k - 16) * Q * 4);
    }
  }
}

template <int Q>
__global__ void __launch_bounds__(BcCfg<Q>::NT, 1) chunk_bwd_dbdc_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ dy, const bf16* __restrict__ Bm,
    const bf16* __restrict__ Cm, const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    const bf16* __restrict__ hst, const bf16* __restrict__ gst, const bf16* __restrict__ wsum,
    bf16* __restrict__ dB, bf16* __restrict__ dC, float* __restrict__ th, int L, int H, int G,
    int nc, int N, int64_t M, int nT) {
  using K = BcCfg<Q>;
  using S = BcLds<Q>;
  constexpr int P = 64, QT = K::QT, NT = K::NT;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  // The nT column tiles of one (batch, chunk, group) sit on one XCD
  // (workgroup id mod 8) and share its L2 for the per-head rows.
  const int64_t q = blockIdx.x;
  const int64_t blk = q / (8 * nT), rem = q % (8 * nT);
  const int nt = (int)(rem / 8);
  const int64_t m = blk * 8 + rem % 8;
  if (m >= M) return;  // whole workgroup
  const int g = (int)(m % G);
  const int64_t bc = m / G;
  const int c = (int)(bc % nc);
  const int b = (int)(bc / nc);
  const int HG = H / G;

  const int lane = lane_id();
  const int w = wave_id();
  const int64_t tok0 = (int64_t)c * Q;
  const int64_t valid = (int64_t)L - tok0;
  const int R[2] = {w, QT - 1 - w};  // output row tiles

  bf16* Bs = (bf16*)(smem + S::BS);
  bf16* Cs = (bf16*)(smem + S::CS);
  const uint32_t head_lds = lds_addr(smem + S::HEAD);

  auto st_of = [&](int h) {
    return (((int64_t)b * nc + c) * H + h) * (int64_t)P * N + nt * 64;
  };
  auto cs_of = [&](int h) { return (((int64_t)b * H + h) * nc + c) * (int64_t)Q; };
  // this lane's dY and x operand pieces of head h (zero past the sequence end)
  bf16x8 nY[2][2], nX[2][2];
  auto load_rows = [&](int h) {
    const int L16 = opaque(lane & 15), grp = opaque(lane >> 4);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int row = R[s] * 16 + L16;
      const int64_t off = (((int64_t)b * L + tok0 + row) * H + h) * P + 8 * grp;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        nY[s][kk] = zero8();
        nX[s][kk] = zero8();
        if (row < valid) {
          nY[s][kk] = *(const bf16x8*)(dy + off + 32 * kk);
          nX[s][kk] = *(const bf16x8*)(x + off + 32 * kk);
        }
      }
    }
  };

  const int h0 = g * HG;
  issue_head_loads<Q>(head_lds, hst + st_of(h0), gst + st_of(h0), N, dA_cs + cs_of(h0),
                      dt_T + cs_of(h0));
  load_rows(h0);
  {
    const int64_t row0 = ((int64_t)b * L + tok0) * G + g;
    RowSlab<Q, NT> sb, sc;  // both tiles' loads in flight together
    sb.load(Bm + row0 * N + nt * 64, (int64_t)G * N, valid);
    sc.load(Cm + row0 * N + nt * 64, (int64_t)G * N, valid);
    sb.template store<true>(Bs);
    sc.template store<true>(Cs);
  }

  f32x4 accC[2][4], accB[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      accC[s][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      accB[s][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // this lane's C values of the T^h parts (the same for every head)
  __syncthreads();
  bf16x4 cth[2][4];
  {
    const int L16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) cth[s][ct][r] = Cs[t64g(R[s] * 16 + 4 * grp + r, ct * 16 + L16)];
  }

  // The T^h parts of a head leave one head later, before the next head's
  // loads: a store issued after those loads would hold up the wait for them
  // (the vector memory counter retires in issue order) by a store's round
  // trip at the end of every head.
  f32x4 thv[2];
  auto store_th = [&](int hs) {
    if ((lane & 15) == 15) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
        *(f32x4*)(th + ((((int64_t)b * nc + c) * H + hs) * nT + nt) * Q + R[s] * 16 + 4 * (lane >> 4)) =
            thv[s];
    }
  };
  for (int hh = 0; hh < HG; ++hh) {
    const int h = h0 + hh;
    // this head's buffer and rows have landed (and every wave is done with
    // the other buffer)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (hh > 0) store_th(h - 1);
    const unsigned char* cur = smem + S::HEAD + (hh & 1) * S::BUF;
    const bf16* Hs = (const bf16*)cur;
    const bf16* Gs = (const bf16*)(cur + 8192);
    const float* css = (const float*)(cur + 16384);
    const float* dts = css + Q;
    bf16x8 aY[2][2], aX[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        aY[s][kk] = nY[s][kk];
        aX[s][kk] = nX[s][kk];
      }
    if (hh + 1 < HG) {
      issue_head_loads<Q>(head_lds + ((hh + 1) & 1) * S::BUF, hst + st_of(h + 1),
                          gst + st_of(h + 1), N, dA_cs + cs_of(h + 1), dt_T + cs_of(h + 1));
      load_rows(h + 1);
    }

    // state terms of this wave's rows: 2^cs_i (dY h)[i, n] into dC and
    // 2^(cs_last - cs_j) dt_j (X g)[j, n] into dB; T^h_i parts
    const int L16 = opaque(lane & 15), grp = opaque(lane >> 4);
    const float csL = css[Q - 1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float eC[4], eB[4], thr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = R[s] * 16 + 4 * grp + r;
        eC[r] = fast_exp2(css[i]);
        eB[r] = fast_exp2(csL - css[i]) * dts[i];
        thr[r] = 0.f;
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        f32x4 tc = f32x4{0.f, 0.f, 0.f, 0.f}, tb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int r0 = 32 * kk + 8 * grp + (L16 >> 2), c0 = ct * 16 + 4 * (L16 & 3);
          const int oa = t64g(r0, c0), ob = t64g(r0 + 4, c0);
          const bf16x8 hb = cat(lds_read_tr(Hs + oa), lds_read_tr(Hs + ob));
          const bf16x8 gb = cat(lds_read_tr(Gs + oa), lds_read_tr(Gs + ob));
          tc = mfma16x16x32(aY[s][kk], hb, tc);
          tb = mfma16x16x32(aX[s][kk], gb, tb);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float vc = eC[r] * tc[r];
          accC[s][ct][r] += vc;
          accB[s][ct][r] += eB[r] * tb[r];
          thr[r] += vc * bf2f(cth[s][ct][r]);
        }
      }
      // T^h parts of this column tile: 2^cs_i dy_i . (h C_i) over its 64
      // columns (each row's total in the last lane of its 16)
#pragma unroll
      for (int r = 0; r < 4; ++r) thv[s][r] = row_scan16(thr[r]);
    }
  }
  store_th(h0 + HG - 1);

  // the group's summed W (bfloat16 triangle tiles) into LDS, then the
  // products with B and C
  __syncthreads();
  const int L16 = lane & 15, grp = lane >> 4;
  bf16* Wt = (bf16*)(smem + S::HEAD);
  {
    // every 16-byte load issued before the first LDS write: one memory
    // latency, not one per piece
    constexpr int NP = BwdCfg<Q>::NTILE * 32, WI = (NP + NT - 1) / NT;
    const bf16* src = wsum + m * (int64_t)(BwdCfg<Q>::NTILE * 256);
    bf16x8 wv[WI];
#pragma unroll
    for (int it = 0; it < WI; ++it) {
      const int i = threadIdx.x + it * NT;
      if (i < NP) wv[it] = *(const bf16x8*)(src + i * 8);
    }
#pragma unroll
    for (int it = 0; it < WI; ++it) {
      const int i = threadIdx.x + it * NT;
      if (i < NP) *(bf16x8*)(Wt + i * 8) = wv[it];
    }
  }
  __syncthreads();

#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int ti = R[s];  // dC rows: sum over j <= i
    for (int kp = 0; kp <= (ti >> 1); ++kp) {
      const int tj = 2 * kp + (grp >> 1);
      const bool live = tj <= ti;
      const int tjc = live ? tj : ti;
      bf16x8 a = *(const bf16x8*)(Wt + tix_of(ti, tjc) * 256 + L16 * 16 + 8 * (grp & 1));
      if (!live) a = zero8();
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int br = 32 * kp + 8 * grp + (L16 >> 2), bcol = ct * 16 + 4 * (L16 & 3);
        const bf16x8 bb = cat(lds_read_tr(Bs + t64g(br, bcol)), lds_read_tr(Bs + t64g(br + 4, bcol)));
        accC[s][ct] = mfma16x16x32(a, bb, accC[s][ct]);
      }
    }
    const int tj = R[s];  // dB rows: sum over i >= j
    for (int kp = tj >> 1; kp < QT / 2; ++kp) {
      const int tii = 2 * kp + (grp >> 1);
      const bool live = tii >= tj;
      const int tic = live ? tii : tj;
      const bf16* wp = Wt + tix_of(tic, tj) * 256 + (8 * (grp & 1) + (L16 >> 2)) * 16 + 4 * (L16 & 3);
      bf16x8 a = cat(lds_read_tr(wp), lds_read_tr(wp + 64));
      if (!live) a = zero8();
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int cr = 32 * kp + 8 * grp + (L16 >> 2), ccol = ct * 16 + 4 * (L16 & 3);
        const bf16x8 cc = cat(lds_read_tr(Cs + t64g(cr, ccol)), lds_read_tr(Cs + t64g(cr + 4, ccol)));
        accB[s][ct] = mfma16x16x32(a, cc, accB[s][ct]);
      }
    }
  }

#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = R[s] * 16 + 4 * grp + r;
      if (i < valid) {
        const int64_t o = (((int64_t)b * L + tok0 + i) * G + g) * N + nt * 64 + L16;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          dC[o + ct * 16] = f2bf(accC[s][ct][r]);
          dB[o + ct * 16] = f2bf(accB[s][ct][r]);
        }
      }
    }
}

// dA[h] and dD[h]: sums of the per-(batch, chunk) parts, one wave per head,
// in a fixed order.
__global__ void __launch_bounds__(64) bwd_param_sums_kernel(const float* __restrict__ dA_part,
                                                            const float* __restrict__ dD_part,
                                                            float* __restrict__ dA,
                                                            float* __restrict__ dD, int64_t BC,
                                                            int H) {
  const int h = blockIdx.x;
  float a = 0.f, d = 0.f;
  for (int64_t u = threadIdx.x; u < BC; u += 64) {
    a += dA_part[u * H + h];
    d += dD_part[u * H + h];
  }
  a = wave_sum(a);
  d = wave_sum(d);
  if (threadIdx.x == 0) {
    dA[h] = a;
    if (dD) dD[h] = d;
  }
}

int cu_count_bwd() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

template <int Q, int N>
hipError_t launch_dx(const Dims& d, const void* x, const void* dy, const void* B, const void* C,
                     const float* dA_cs, const float* dt_T, const void* gst, const float* dots,
                     int wph, const float* th, const float* rsum, const float* A, const float* D,
                     void* dx, void* ddt, float* dA_part, float* dD_part, const float* dus,
                     hipStream_t s) {
  if (DxLds<Q, N>::EXT && dus == nullptr) return hipErrorInvalidValue;
  auto kern = chunk_bwd_dx_kernel<Q, N>;
  constexpr int lds = DxLds<Q, N>::BYTES;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int64_t HG = d.H / d.G;
  int64_t hpw = (d.B * d.nc * d.H) / cu_count_bwd();
  if (hpw < 1) hpw = 1;
  if (hpw > HG) hpw = HG;
  const int64_t slices = (HG + hpw - 1) / hpw;
  hpw = (HG + slices - 1) / slices;
  const int64_t grid = d.B * d.nc * d.G * slices;
  kern<<<(unsigned)grid, BwdCfg<Q>::NT, lds, s>>>(
      (const bf16*)x, (const bf16*)dy, (const bf16*)B, (const bf16*)C, dA_cs, dt_T,
      (const bf16*)gst, dots, th, rsum, A, D, (bf16*)dx, (bf16*)ddt, dA_part, dD_part, dus,
      (int)d.L, (int)d.H, (int)d.G, (int)d.nc, (int)hpw, (int)slices, wph);
  return hipGetLastError();
}

template <int N>
hipError_t launch_dus(const Dims& d, const void* B, const void* gst, float* dus, hipStream_t s) {
  using K = DusCfg<N>;
  auto kern = chunk_bwd_dus_kernel<N>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS);
  if (attr != hipSuccess) return attr;
  const int64_t HG = d.H / d.G;
  int64_t hpw = (d.B * d.nc * d.H) / cu_count_bwd();
  if (hpw < 1) hpw = 1;
  if (hpw > HG) hpw = HG;
  const int64_t slices = (HG + hpw - 1) / hpw;
  hpw = (HG + slices - 1) / slices;
  const int64_t grid = d.B * d.nc * d.G * slices;
  kern<<<(unsigned)grid, K::NT, K::LDS, s>>>((const bf16*)B, (const bf16*)gst, dus, (int)d.L,
                                             (int)d.H, (int)d.G, (int)d.nc, (int)hpw,
                                             (int)slices);
  return hipGetLastError();
}

template <int Q>
hipError_t launch_dbdc(const Dims& d, const void* x, const void* dy, const void* B, const void* C,
                       const float* dA_cs, const float* dt_T, const void* hst, const void* gst,
                       void* wsum, float* rsum, void* dB, void* dC, float* th, hipStream_t s) {
  auto wk = chunk_bwd_wsum_kernel<Q>;
  constexpr int wlds = WsLds<Q>::BYTES;
  static const hipError_t wattr =
      hipFuncSetAttribute((const void*)wk, hipFuncAttributeMaxDynamicSharedMemorySize, wlds);
  if (wattr != hipSuccess) return wattr;
  wk<<<(unsigned)(d.B * d.nc * d.G), BwdCfg<Q>::NT, wlds, s>>>(
      (const bf16*)x, (const bf16*)dy, (const bf16*)B, (const bf16*)C, dA_cs, dt_T, (bf16*)wsum,
      rsum, (int)d.L, (int)d.H, (int)d.G, (int)d.nc, (int)d.N);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto kern = chunk_bwd_dbdc_kernel<Q>;
  constexpr int lds = BcLds<Q>::BYTES;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int64_t M = d.B * d.nc * d.G;
  const int nT = (int)(d.N / 64);
  const int64_t grid = (M + 7) / 8 * 8 * nT;
  kern<<<(unsigned)grid, BcCfg<Q>::NT, lds, s>>>(
      (const bf16*)x, (const bf16*)dy, (const bf16*)B, (const bf16*)C, dA_cs, dt_T,
      (const bf16*)hst, (const bf16*)gst, (const bf16*)wsum, (bf16*)dB, (bf16*)dC, th, (int)d.L,
      (int)d.H, (int)d.G, (int)d.nc, (int)d.N, M, nT);
  return hipGetLastError();
}

}  // namespace

bool backward_supported(const Dims& d) {
  return d.bf16 && d.P == 64 &&
         (((d.N == 64 || d.N == 128 || d.N == 256) && (d.Q == 64 || d.Q == 128 || d.Q == 256)) ||
          (d.N == 512 && d.Q == 256));
}

bool backward_state_term_separate(const Dims& d) { return d.N > 256; }

hipError_t launch_chunk_bwd_dus(const Dims& d, const void* B, const void* gst, float* dus,
                                hipStream_t s) {
  if (d.N == 512 && d.Q == 256 && d.P == 64 && d.bf16) return launch_dus<512>(d, B, gst, dus, s);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_bwd_dx(const Dims& d, const void* x, const void* dy, const void* B,
                               const void* C, const float* dA_cs, const float* dt_T,
                               const void* gst, const float* dots, int wph, const float* th,
                               const float* rsum, const float* A, const float* D, void* dx,
                               void* ddt, float* dA_part, float* dD_part, const float* dus,
                               hipStream_t s) {
#define M2_DX(QQ, NN)                                                                         \
  if (d.Q == QQ && d.N == NN)                                                                 \
    return launch_dx<QQ, NN>(d, x, dy, B, C, dA_cs, dt_T, gst, dots, wph, th, rsum, A, D, dx, \
                             ddt, dA_part, dD_part, dus, s);
  M2_DX(64, 64) M2_DX(64, 128) M2_DX(64, 256)
  M2_DX(128, 64) M2_DX(128, 128) M2_DX(128, 256)
  M2_DX(256, 64) M2_DX(256, 128) M2_DX(256, 256) M2_DX(256, 512)
#undef M2_DX
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_bwd_dbdc(const Dims& d, const void* x, const void* dy, const void* B,
                                 const void* C, const float* dA_cs, const float* dt_T,
                                 const void* hst, const void* gst, void* wsum, float* rsum,
                                 void* dB, void* dC, float* th, hipStream_t s) {
  switch (d.Q) {
    case 64:
      return launch_dbdc<64>(d, x, dy, B, C, dA_cs, dt_T, hst, gst, wsum, rsum, dB, dC, th, s);
    case 128:
      return launch_dbdc<128>(d, x, dy, B, C, dA_cs, dt_T, hst, gst, wsum, rsum, dB, dC, th, s);
    case 256:
      return launch_dbdc<256>(d, x, dy, B, C, dA_cs, dt_T, hst, gst, wsum, rsum, dB, dC, th, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_param_sums(const Dims& d, const float* dA_part, const float* dD_part,
                                 float* dA, float* dD, hipStream_t s) {
  bwd_param_sums_kernel<<<(unsigned)d.H, 64, 0, s>>>(dA_part, dD_part, dA, dD, d.B * d.nc,
                                                     (int)d.H);
  return hipGetLastError();
}

}  // namespace m2
