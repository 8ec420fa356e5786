// chunk_scan (compute_out), grouped variant used by the fused forward pass:
// one workgroup serves one (batch, chunk, B/C group) and a run of that
// group's heads.  The pages fuse the output stage so the chunk x chunk matrix
// never reaches memory (devotd.net news item on the Mamba-2 CUDA Tile
// forward-pass kernels, section 2); here it additionally never gets recomputed
// per head: G^T = B C^T depends only on the group, so it is formed once per
// workgroup, kept in fp32 accumulators, and reused by every head of the run,
// each head applying its own decay mask (disconfirmai.com "Jane Street ML
// Engineers Map Mamba-2 Recurrent State Computation to Tensor Cores with
// cuTile", body: exponential row scaling keeps the matrix-product form).
// The C operand of the carried-state contraction is likewise loaded once and
// kept in registers for all heads.
//
// Per head the kernel streams only what is head-specific: the chunk-start
// state (bfloat16, P x N) and the chunk's x rows (Q x P), plus the head's
// cumulative sums.  They arrive through gfx950 direct-to-LDS loads into a
// double buffer: while the waves compute head k from one buffer, head k+1's
// bytes land in the other, so HBM stays busy with one workgroup per CU.
// Both LDS tiles are XOR-swizzled in 16-byte units so the MFMA operand reads
// (row reads of the state, transpose reads of x) spread over the LDS banks.
//
// Math, MFMA layouts, the transposed Y^T formulation and the row and K
// permutations are those of the per-head chunk_scan kernel: Y^T[p, i] with
// MFMA row m of p-tile pt standing for p = 16 (m/4) + 4 pt + m%4 (P = 64),
// and the in-chunk product's K element e of lane group q standing for
// j = 32 jp + 4q + e (e < 4) or 32 jp + 16 + 4q + (e - 4).
#include "common.h"
#include "launch.h"

namespace m2 {

namespace {

constexpr int kHopAhead = 3;  // state-operand reads in flight ahead of the MFMAs

enum ScanMode { kWhole = 0, kFirstHalf = 1, kSecondHalf = 2 };

template <int P, int Q, int N>
struct GCfg {
  static constexpr int QT = Q / 16, NW = Q / 32, PT = P / 16, NBLK = N / 64;
  static constexpr int HS_BYTES = P * N * 2;     // state tile, bf16
  static constexpr int XS_BYTES = Q * P * 2;     // x tile, bf16
  static constexpr int CS_BYTES = Q * 4;         // cumulative sums (and dt), fp32
  static constexpr int BUF = HS_BYTES + XS_BYTES + 2 * CS_BYTES;
  static constexpr int SROW = 64 + 8;            // staging row stride (elements)
  static constexpr int STG = 2 * Q * SROW * 2;   // B and C staging for G
  static constexpr int LDS = BUF + (BUF > STG ? BUF : STG);
  static constexpr int RLH = N / 8;              // 16-byte chunks per state row
  static_assert(P == 64, "grouped chunk_scan is specialised for headdim 64");
  static_assert(N == 64 || N == 128 || N == 256, "state size must be 64, 128 or 256");
};

// Chunk position of 16-byte chunk c of state row r (row length RLH chunks).
template <int RLH>
__device__ __forceinline__ int hswz(int r, int c) {
  return c ^ (((r & 3) | (((r >> 4) & 3) << 2)) & (RLH - 1));
}
// Chunk position of 16-byte chunk c of x row r (8 chunks per row).  A
// transpose read touches 16 rows 4g + e (+ 32 jp) and, per row, four chunks
// of the same parity; xor-ing with (r >> 1) alternates that parity between
// neighbouring even (and odd) rows so two rows share each bank group, the
// least 16-byte chunks allow.
__device__ __forceinline__ int xswz(int r, int c) { return c ^ ((r >> 1) & 7); }

// Issues the direct-to-LDS loads of one head into buffer `buf`:
// state rows (P x N bf16), x rows (Q x P bf16, rows past L clamped to L-1,
// whose values are never used with a nonzero weight), cumulative sums, dt.
// In the second half pass only the state columns and the sums are needed.
// The state rows are `ldn` elements long; this pass reads columns n0 .. n0 + N - 1.
template <int P, int Q, int N, int MODE>
__device__ __forceinline__ void load_head(uint32_t buf, const bf16* __restrict__ hst,
                                          const bf16* __restrict__ x,
                                          const float* __restrict__ dA_cs,
                                          const float* __restrict__ dt_T, int b, int c, int h,
                                          int L, int H, int nc, int ldn, int n0) {
  using K = GCfg<P, Q, N>;
  const int lane = lane_id();
  const int w = wave_id();
  // state: P*N/512 wave-loads of 64 chunks
  const bf16* hsrc = hst + (((int64_t)b * nc + c) * H + h) * (int64_t)P * ldn + n0;
  constexpr int HI = P * N / 512 / K::NW;
#pragma unroll
  for (int i = 0; i < HI; ++i) {
    const int k = w + K::NW * i;
    const int s = k * 64 + lane;
    const int r = s / K::RLH, pos = s % K::RLH;
    const int cc = hswz<K::RLH>(r, pos);  // involution: position <-> chunk
    dma16(hsrc + (int64_t)r * ldn + cc * 8, buf + k * 1024);
  }
  const uint32_t cs = buf + K::HS_BYTES + K::XS_BYTES;
  const int64_t cb = (((int64_t)b * H + h) * nc + c) * Q;
  if (MODE == kSecondHalf) {  // cumulative sums only (wave 0)
    if (w == 0 && lane < Q / 4) dma16(dA_cs + cb + lane * 4, cs);
    return;
  }
  // x rows: Q/8 wave-loads of 8 rows
  const uint32_t xs = buf + K::HS_BYTES;
  constexpr int XI = Q / 8 / K::NW;
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int k = w + K::NW * i;
    const int s = k * 64 + lane;
    const int r = s >> 3, pos = s & 7;
    int64_t t = (int64_t)c * Q + r;
    if (t > L - 1) t = L - 1;
    dma16(x + (((int64_t)b * L + t) * H + h) * P + xswz(r, pos) * 8, xs + k * 1024);
  }
  // cumulative sums (wave 0) and dt (wave 1): Q/4 chunks each
  if (w < 2 && lane < Q / 4) {
    const float* src = (w == 0 ? dA_cs : dt_T) + cb + lane * 4;
    dma16(src, cs + w * K::CS_BYTES);
  }
}


// Two floats to two bfloat16 (round to nearest even) in one conversion.
typedef float cs_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 cs_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ cs_bf16x2 pk2(float a, float b) {
  return __builtin_convertvector((cs_f32x2){a, b}, cs_bf16x2);
}
__device__ __forceinline__ bf16x4 pk4(float a, float b, float c, float d) {
  return __builtin_shufflevector(pk2(a, b), pk2(c, d), 0, 1, 2, 3);
}

// Four elements (rows j = j0 + r) of the masked, decayed in-chunk weights of
// column i: G^T * 2^(cs_i - cs_j) * dt_j, with lw_j = cs_j - log2(dt_j)
// (dt_j = 0 gives +inf and weight 0).  Tiles strictly below the diagonal need
// no mask; the diagonal tile is masked causally and carries the skip term D
// on j == i, where the decay is 1.
__device__ __forceinline__ bf16x4 weights4(const f32x4 gt, const f32x4 lw, float csi, bool diag,
                                           int j0, int i, float Dh) {
  float v[4];
  if (!diag) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = gt[r] * fast_exp2(csi - lw[r]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + r;
      float gv = (j <= i) ? gt[r] * fast_exp2(csi - lw[r]) : 0.f;
      if (j == i) gv += Dh;
      v[r] = gv;
    }
  }
  return pk4(v[0], v[1], v[2], v[3]);
}

// In-chunk contribution for both of a wave's i-tiles (t0 < t1): scales the
// carried-state parts by 2^cs_i, then walks the j-tile pairs once, reading
// each pair's x operand and weight exponents a single time and applying them
// to every i-tile at or below the pair.  G^T tile (jt, t0) sits in slot jt,
// (jt, t1) in slot QT - jt.
// L16 and grp (the lane's position in its 16-lane row and its row) come from
// the caller, hidden from the optimiser per head: otherwise it hoists every
// diagonal-tile comparison out of the head loop as a 64-bit lane mask, runs
// out of scalar registers and reloads the masks from spill lanes at each use.
template <int QT, int P>
__device__ __forceinline__ void in_chunk(const f32x4 (&Gs)[QT + 1], f32x4 (&Y0)[P / 16],
                                         f32x4 (&Y1)[P / 16], int t0, int t1, const float* css,
                                         const float* lws, const unsigned char* Xs, float Dh,
                                         int L16, int grp) {
  constexpr int PT = P / 16;
  const int i0 = 16 * t0 + L16, i1 = 16 * t1 + L16;
  const float cs0 = css[i0], cs1 = css[i1];
  const float sc0 = fast_exp2(cs0), sc1 = fast_exp2(cs1);
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    Y0[pt] *= sc0;
    Y1[pt] *= sc1;
  }
  // Byte offsets of the lane's transposed x reads inside a 32-row block: the
  // swizzle of row 32 jp + r equals that of row r (it uses bits 1..3 of the
  // row), so block jp is these offsets plus a constant jp * 32 rows.
  const unsigned char* xa[PT][2];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    const int ra = 4 * grp + (L16 >> 2), rb = ra + 16;
    const int p0 = 4 * PT * (L16 & 3) + 4 * pt;
    const int ch = p0 >> 3, off = (p0 & 7) * 2;
    xa[pt][0] = Xs + ra * (P * 2) + (xswz(ra, ch) << 4) + off;
    xa[pt][1] = Xs + rb * (P * 2) + (xswz(rb, ch) << 4) + off;
  }
#pragma unroll
  for (int jp = 0; jp < QT / 2; ++jp) {
    if (2 * jp > t1) break;
    const int ja = 2 * jp, jb = 2 * jp + 1;
    bf16x8 xop[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const bf16* pa = (const bf16*)(xa[pt][0] + jp * 32 * (P * 2));
      const bf16* pb = (const bf16*)(xa[pt][1] + jp * 32 * (P * 2));
      xop[pt] = cat(lds_read_tr(pa), lds_read_tr(pb));
    }
    const f32x4 lwa = *(const f32x4*)(lws + 16 * ja + 4 * grp);
    const f32x4 lwb = *(const f32x4*)(lws + 16 * jb + 4 * grp);
    const bf16x4 zero4 = pk4(0.f, 0.f, 0.f, 0.f);
    {  // tile t1 (2 jp <= t1 here)
      const bf16x4 lo = weights4(Gs[QT - ja], lwa, cs1, ja == t1, 16 * ja + 4 * grp, i1, Dh);
      const bf16x4 hi = jb <= t1
          ? weights4(Gs[QT - jb], lwb, cs1, jb == t1, 16 * jb + 4 * grp, i1, Dh) : zero4;
      const bf16x8 gm = cat(lo, hi);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) Y1[pt] = mfma16x16x32(xop[pt], gm, Y1[pt]);
    }
    if (ja < QT / 2 && ja <= t0) {  // tile t0
      const bf16x4 lo = weights4(Gs[ja < QT / 2 ? ja : 0], lwa, cs0, ja == t0,
                                 16 * ja + 4 * grp, i0, Dh);
      const bf16x4 hi = (jb < QT / 2 && jb <= t0)
          ? weights4(Gs[jb < QT / 2 ? jb : 0], lwb, cs0, jb == t0, 16 * jb + 4 * grp, i0, Dh)
          : zero4;
      const bf16x8 gm = cat(lo, hi);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) Y0[pt] = mfma16x16x32(xop[pt], gm, Y0[pt]);
    }
  }
}

// Stores one i-tile of Y^T: lane (i, group q) holds p = 4 PT q .. 4 PT q + 4 PT - 1.
template <int P>
__device__ __forceinline__ void store_tile(const f32x4 (&Yt)[P / 16], int t, bf16* __restrict__ y,
                                           int64_t ybase, int H, int64_t valid) {
  constexpr int PT = P / 16;
  const int lane = lane_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int i = 16 * t + L16;
  if (i < valid) {
    bf16* dst = y + (ybase + (int64_t)i * H) * P + 4 * PT * grp;
#pragma unroll
    for (int pt = 0; pt < PT; pt += 2) {
      const bf16x8 o = cat(pk4(Yt[pt][0], Yt[pt][1], Yt[pt][2], Yt[pt][3]),
                           pk4(Yt[pt + 1][0], Yt[pt + 1][1], Yt[pt + 1][2], Yt[pt + 1][3]));
      *(bf16x8*)(dst + 4 * pt) = o;
    }
  }
}

// The first half pass's y, rounded to bfloat16 for the second pass (at
// state size 512 y = first half + second half's carried-state term; a
// float32 hand-over would move 8 bytes per output element through HBM, this
// moves 4): the same lane layout as store_tile, 4 PT consecutive p of one
// token per lane, in a [B, L, H, P] bfloat16 buffer.
template <int P>
__device__ __forceinline__ void store_part(const f32x4 (&Yt)[P / 16], int t,
                                           bf16* __restrict__ part, int64_t ybase, int H,
                                           int64_t valid) {
  store_tile<P>(Yt, t, part, ybase, H, valid);
}

// Adds the first half pass's y to one i-tile (rows past the sequence end are
// neither read nor stored).
template <int P>
__device__ __forceinline__ void add_part(f32x4 (&Yt)[P / 16], int t,
                                         const bf16* __restrict__ part, int64_t ybase, int H,
                                         int64_t valid) {
  constexpr int PT = P / 16;
  const int lane = lane_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int i = 16 * t + L16;
  if (i < valid) {
    const bf16* src = part + (ybase + (int64_t)i * H) * P + 4 * PT * grp;
#pragma unroll
    for (int pt = 0; pt < PT; pt += 2) {
      const bf16x8 v = *(const bf16x8*)(src + 4 * pt);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Yt[pt][e] += bf2f(v[e]);
        Yt[pt + 1][e] += bf2f(v[4 + e]);
      }
    }
  }
}

template <int P, int Q, int N, int MODE>
__global__ void __launch_bounds__(Q * 2) chunk_scan_grouped_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const bf16* __restrict__ Cm,
    const float* __restrict__ dA_cs, const float* __restrict__ dt_T,
    const bf16* __restrict__ hst, const float* __restrict__ Dv, bf16* __restrict__ y,
    bf16* __restrict__ part, int L, int H, int G, int nc, int hpw, int slices, int n0) {
  using K = GCfg<P, Q, N>;
  constexpr int QT = K::QT, PT = K::PT, NBLK = K::NBLK, SROW = K::SROW;
  // rows of B, C and the start states hold ldn columns; G^T runs over all of
  // them (GBLK blocks of 64), the carried-state term over N from n0
  constexpr int ldn = MODE == kWhole ? N : 2 * N;
  constexpr int GBLK = MODE == kSecondHalf ? 0 : ldn / 64;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  bf16* Cs = (bf16*)(smem + K::BUF);  // phase-A staging aliases buffer 1
  bf16* Bs = Cs + Q * SROW;

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

  const int tid = threadIdx.x;
  constexpr int nthr = Q * 2;
  const int lane = lane_id();
  const int w = wave_id();
  const int L16 = lane & 15, grp = lane >> 4;
  const int t0 = w, t1 = QT - 1 - w;
  const int64_t tok0 = (int64_t)c * Q;

  // Head 0's bytes start flowing while G is formed.
  const uint32_t sbase = lds_addr(smem);
  // each workgroup walks its heads from a different one, so the workgroups
  // in flight touch different heads' slices of the token rows; the c / 8
  // term spreads the start heads of one XCD's chunks (c = XCD mod 8) too
  const int rot = nh > 0 ? (c + (c >> 3)) % nh : 0;
  load_head<P, Q, N, MODE>(sbase, hst, x, dA_cs, dt_T, b, c, h0 + rot, L, H, nc, ldn, n0);

  // ---- Phase A: G^T tiles of this wave's two i-tiles, and its C operands.
  // G^T tiles: j-tile jt of i-tile t0 in slot jt (jt <= t0), of i-tile t1 in
  // slot QT - jt (jt <= t1); together exactly QT + 1 slots.
  f32x4 Gs[QT + 1];
#pragma unroll
  for (int a = 0; a <= QT; ++a) Gs[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 C0[NBLK][2], C1[NBLK][2];
  constexpr int ABLK = GBLK > NBLK ? GBLK : NBLK;  // 64-column blocks staged
  // Each block's C and B rows pass through registers on their way to LDS;
  // block nb + 1's loads are issued before block nb's MFMAs, so their
  // latency hides behind them.
  constexpr int SIT = Q * 8 / nthr;  // 16-byte pieces per thread and block
  static_assert(Q * 8 % nthr == 0, "staging pieces per thread");
  bf16x8 sc[SIT], sbv[SIT];
  auto stage_load = [&](int nb) {
#pragma unroll
    for (int it = 0; it < SIT; ++it) {
      const int idx = tid + it * nthr;
      const int r = idx >> 3, c8 = (idx & 7) * 8;
      const int64_t t = tok0 + r;
      if (t < L) {
        const int64_t off = (((int64_t)b * L + t) * G + g) * ldn + n0 + nb * 64 + c8;
        sc[it] = *(const bf16x8*)(Cm + off);
        if (nb < GBLK) sbv[it] = *(const bf16x8*)(Bm + off);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[it][e] = sbv[it][e] = f2bf(0.f);
      }
    }
  };
  stage_load(0);
#pragma unroll
  for (int nb = 0; nb < ABLK; ++nb) {
    lds_barrier();
#pragma unroll
    for (int it = 0; it < SIT; ++it) {
      const int idx = tid + it * nthr;
      const int r = idx >> 3, c8 = (idx & 7) * 8;
      *(bf16x8*)(Cs + r * SROW + c8) = sc[it];
      if (nb < GBLK) *(bf16x8*)(Bs + r * SROW + c8) = sbv[it];
    }
    if (nb + 1 < ABLK) stage_load(nb + 1);
    lds_barrier();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int koff = kk * 32 + grp * 8;
      const bf16x8 c0 = *(const bf16x8*)(Cs + (16 * t0 + L16) * SROW + koff);
      const bf16x8 c1 = *(const bf16x8*)(Cs + (16 * t1 + L16) * SROW + koff);
      if (nb < NBLK) {
        C0[nb][kk] = c0;
        C1[nb][kk] = c1;
      }
      if (nb < GBLK) {
#pragma unroll
        for (int jt = 0; jt < QT; ++jt) {
          if (jt <= t1) {
            const bf16x8 bop = *(const bf16x8*)(Bs + (16 * jt + L16) * SROW + koff);
            if (jt < QT / 2 && jt <= t0) Gs[jt] = mfma16x16x32(bop, c0, Gs[jt]);
            Gs[QT - jt] = mfma16x16x32(bop, c1, Gs[QT - jt]);
          }
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();

  // ---- Phase B: heads.
  for (int k = 0; k < nh; ++k) {
    const int kr = k + rot < nh ? k + rot : k + rot - nh;
    const int h = h0 + kr;
    unsigned char* cur = smem + (k & 1) * K::BUF;
    if (k + 1 < nh)
      load_head<P, Q, N, MODE>(sbase + ((k + 1) & 1) * K::BUF, hst, x, dA_cs, dt_T, b, c,
                               h0 + (kr + 1 < nh ? kr + 1 : kr + 1 - nh), L, H, nc, ldn, n0);
    const unsigned char* Hs = cur;
    const unsigned char* Xs = cur + K::HS_BYTES;
    const float* css = (const float*)(Xs + K::XS_BYTES);
    const float* dts = css + Q;

    f32x4 Y[2][PT];
#pragma unroll
    for (int a = 0; a < PT; ++a) Y[0][a] = Y[1][a] = f32x4{0.f, 0.f, 0.f, 0.f};
    // carried-state term: Y^T[p, i] = sum_n h[p, n] C[i, n].  The state
    // operands are read kHopAhead MFMA pairs ahead of use (a small register
    // ring), so several LDS reads are in flight while the MFMAs run.
    {
      constexpr int NIT = NBLK * 2 * PT;
      auto hop_at = [&](int it) {
        const int nb = it / (2 * PT), kk = (it / PT) % 2, pt = it % PT;
        const int r = 16 * (L16 >> 2) + 4 * pt + (L16 & 3);
        const int cc = nb * 8 + kk * 4 + grp;
        return *(const bf16x8*)(Hs + r * (N * 2) + (hswz<K::RLH>(r, cc) << 4));
      };
      bf16x8 ring[kHopAhead];
#pragma unroll
      for (int a = 0; a < kHopAhead; ++a) ring[a] = hop_at(a);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int nb = it / (2 * PT), kk = (it / PT) % 2, pt = it % PT;
        const bf16x8 hop = ring[it % kHopAhead];
        if (it + kHopAhead < NIT) ring[it % kHopAhead] = hop_at(it + kHopAhead);
        Y[0][pt] = mfma16x16x32(hop, C0[nb][kk], Y[0][pt]);
        Y[1][pt] = mfma16x16x32(hop, C1[nb][kk], Y[1][pt]);
        // keep each read where it is: the scheduler would otherwise sink it
        // next to its MFMAs to shorten live ranges, one read in flight
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int64_t valid = L - tok0;
    const int64_t ybase = ((int64_t)b * L + tok0) * H + h;
    if (MODE == kSecondHalf) {
      // carried-state term of the second half, scaled by 2^cs_i, plus the
      // first pass's float32 y
      const float sc0 = fast_exp2(css[16 * t0 + L16]), sc1 = fast_exp2(css[16 * t1 + L16]);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        Y[0][pt] *= sc0;
        Y[1][pt] *= sc1;
      }
      add_part<P>(Y[0], t0, part, ybase, H, valid);
      add_part<P>(Y[1], t1, part, ybase, H, valid);
      __builtin_amdgcn_s_waitcnt(0);  // next head's bytes have landed
      store_tile<P>(Y[0], t0, y, ybase, H, valid);
      store_tile<P>(Y[1], t1, y, ybase, H, valid);
      lds_barrier();
      continue;
    }
    // dt_j -> cs_j - log2(dt_j), in place (the in-chunk weights' exponent offset)
    if (tid < Q) {
      float* lw = (float*)dts;
      lw[tid] = css[tid] - __builtin_amdgcn_logf(lw[tid]);
    }
    lds_barrier();  // weights visible; next head's loads stay in flight
    const float Dh = Dv ? Dv[h] : 0.f;
    int l16 = L16, lgrp = grp;
    asm volatile("" : "+v"(l16), "+v"(lgrp));
    in_chunk<QT, P>(Gs, Y[0], Y[1], t0, t1, css, dts, Xs, Dh, l16, lgrp);

    __builtin_amdgcn_s_waitcnt(0);  // next head's bytes have landed (and older stores drained)
    if (MODE == kFirstHalf) {
      store_part<P>(Y[0], t0, part, ybase, H, valid);
      store_part<P>(Y[1], t1, part, ybase, H, valid);
    } else {
      store_tile<P>(Y[0], t0, y, ybase, H, valid);
      store_tile<P>(Y[1], t1, y, ybase, H, valid);
    }
    lds_barrier();
  }
}

int cu_count() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

template <int P, int Q, int N, int MODE>
hipError_t launch_grouped(const Dims& d, const void* x, const void* B, const void* C,
                          const float* dA_cs, const float* dt_T, const void* hst, const float* D,
                          void* y, void* part, int n0, hipStream_t s) {
  using K = GCfg<P, Q, N>;
  auto kern = chunk_scan_grouped_kernel<P, Q, N, MODE>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS);
  if (attr != hipSuccess) return attr;
  // Heads per workgroup: enough workgroups to cover every CU once, as many
  // heads per workgroup as that allows (G^T is formed once per workgroup).
  const int64_t HG = d.H / d.G;
  int64_t hpw = (d.B * d.nc * d.H) / cu_count();
  if (hpw < 1) hpw = 1;
  if (hpw > HG) hpw = HG;
  const int64_t slices = (HG + hpw - 1) / hpw;
  hpw = (HG + slices - 1) / slices;  // balance the slices
  const int64_t grid = d.B * d.nc * d.G * slices;
  kern<<<(unsigned)grid, Q * 2, K::LDS, s>>>(
      (const bf16*)x, (const bf16*)B, (const bf16*)C, dA_cs, dt_T, (const bf16*)hst, D,
      (bf16*)y, (bf16*)part, (int)d.L, (int)d.H, (int)d.G, (int)d.nc, (int)hpw, (int)slices, n0);
  return hipGetLastError();
}

template <int Q>
hipError_t launch_grouped_n(const Dims& d, const void* x, const void* B, const void* C,
                            const float* dA_cs, const float* dt_T, const void* hst,
                            const float* D, void* y, void* part, hipStream_t s) {
  switch (d.N) {
    case 64: return launch_grouped<64, Q, 64, kWhole>(d, x, B, C, dA_cs, dt_T, hst, D, y, nullptr, 0, s);
    case 128: return launch_grouped<64, Q, 128, kWhole>(d, x, B, C, dA_cs, dt_T, hst, D, y, nullptr, 0, s);
    case 256: return launch_grouped<64, Q, 256, kWhole>(d, x, B, C, dA_cs, dt_T, hst, D, y, nullptr, 0, s);
    case 512: {
      if (!part) return hipErrorInvalidValue;
      const hipError_t e = launch_grouped<64, Q, 256, kFirstHalf>(d, x, B, C, dA_cs, dt_T, hst,
                                                                   D, y, part, 0, s);
      if (e != hipSuccess) return e;
      return launch_grouped<64, Q, 256, kSecondHalf>(d, x, B, C, dA_cs, dt_T, hst, D, y, part,
                                                     256, s);
    }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool grouped_scan_supported(const Dims& d) {
  return d.bf16 && d.P == 64 && (d.N == 64 || d.N == 128 || d.N == 256 || d.N == 512) &&
         (d.Q == 64 || d.Q == 128 || d.Q == 256);
}

size_t grouped_scan_part_bytes(const Dims& d) {
  return d.N == 512 ? (size_t)(d.B * d.L * d.H * d.P) * 2 : 0;
}

hipError_t launch_chunk_scan_grouped(const Dims& d, const void* x, const void* B, const void* C,
                                     const float* dA_cs, const float* dt_T, const void* hst,
                                     const float* D, void* y, void* part, hipStream_t s) {
  switch (d.Q) {
    case 64: return launch_grouped_n<64>(d, x, B, C, dA_cs, dt_T, hst, D, y, part, s);
    case 128: return launch_grouped_n<128>(d, x, B, C, dA_cs, dt_T, hst, D, y, part, s);
    case 256: return launch_grouped_n<256>(d, x, B, C, dA_cs, dt_T, hst, D, y, part, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m2
