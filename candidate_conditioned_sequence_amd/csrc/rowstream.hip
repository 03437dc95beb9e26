// Weight-stationary row-streaming GEMMs for the projections whose weight is
// small and whose rows are many: the query projection over the C*n_q query
// rows and the key/value projections over the history stream, forward
// (a1, a2) and backward (the dX half of a7).
//
// What they compute is the same as the tiled GEMM path (pith.science verdict
// record, pith_extraction.key_machinery: Q from the normalised Wukong output,
// K and V from the normalised HSTU output; gist.science Technical Summary
// section 2.1: pre-norm projections):
//   forward   Y = Norm(H) W^T, also writing Norm(H) and the row statistics;
//   backward  dX = Norm backward(dY W^T) + R, with the per-row sums of the
//             norm backward and column partials of dgamma / dbeta.
//
// Design.  With K, N <= 512 the weight is at most 256 KB, while the rows
// number in the millions.  A tiled GEMM re-streams the weight tile for every
// row tile, and on this shape that traffic (and its LDS round trip and
// barrier per K step) bounds it far below the HBM rate.  Here each wave owns
// 32 output columns and keeps their K-deep weight slice in registers for the
// whole launch (K/4 VGPRs); blocks of 32 rows stream through LDS, moved by
// direct global-to-LDS transfers so they occupy no registers, one or two
// blocks ahead.  One v_mfma_f32_32x32x16_bf16 per 16-deep K step gives the
// transposed tile D[n][m]: lane l holds row m = l % 32 and 16 of the wave's
// columns, 4 consecutive ones per register group, so the epilogues store
// 8-byte pieces of a row straight from registers.  Rows past M read row M-1
// and are never stored.  One workgroup per CU, persistent over the blocks.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kRB = 32;   // rows per block: the column dimension of one 32x32 MFMA tile

// LDS blocks hold unpadded rows; the 16-byte chunk c of block row r sits at
// chunk position c ^ (r & 7), so one fragment read (one chunk of 32
// consecutive rows) touches every bank group, and a transfer instruction
// (64 consecutive positions) still covers whole rows.
WHALE_DEV int swz(int c, int r) { return c ^ (r & 7); }

// Direct global -> LDS transfers: lane i writes the i-th slot (16 or 4 bytes)
// after the wave-uniform LDS byte address, reading a wave-uniform base (in
// SGPRs) plus a 32-bit per-lane byte offset.  They are issued from inline
// asm so the compiler does not treat them as pending writes to every LDS
// buffer (which would make each LDS read wait for them); every wave waits
// for its own transfers with an explicit vmcnt before the barrier that
// publishes them.  No register receives data.
WHALE_DEV void dma16(const void* base, uint32_t voff, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base)
                   : "memory", "m0");
}
WHALE_DEV void dma4(const void* base, uint32_t voff, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base)
                   : "memory", "m0");
}
// A panel is 32 rows x 256 columns (512-byte rows) of one source array.  One
// instruction moves rows r, r+1 of it (r even): lane l takes chunk position
// l % 32 of row r + l / 32, i.e. source chunk (l % 32) ^ (row & 7).  Source
// rows are src + min(m0 + row, M - 1) * ld; m0, r and the pointers are
// wave-uniform.
WHALE_DEV void dma_rows(const bf16* src, int64_t ld, int64_t m0, int r, int64_t M, int lane, uint32_t lds) {
  const int64_t mr = m0 + r;
  const bf16* base = src + (mr < M - 1 ? mr : M - 1) * ld;
  const int hl = lane >> 5;
  const uint32_t row2 = (hl && mr + 1 < M) ? (uint32_t)(2 * ld) : 0u;
  dma16(base, row2 + 16u * (uint32_t)((lane & 31) ^ ((r + hl) & 7)), lds);
}
constexpr int kPanel = kRB * 512;   // bytes of one panel
// s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15) as a builtin the compiler tracks.
constexpr int kVmcnt0 = 0x0F70;
template <int N> WHALE_DEV void wait_vm() { __asm__ volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory"); }

// acc += W slice x (32 rows of the block at xrow)^T over K: fragment reads
// run four K steps ahead of the MFMAs (all K/16 at once would not fit in
// registers next to the resident weight slice).
// The block is K/256 panels; K step ks reads chunk 2 (ks % 16) + hh of row
// l32 of panel ks / 16.  The swizzle changes only the low three bits of the
// chunk index, so that is at 16384 (ks / 16) + 128 ((ks % 16) / 4) +
// 16 ((2 (ks % 4) + hh) ^ (l32 & 7)): four per-lane offsets, the rest an
// immediate.
template <int K>
WHALE_DEV void block_mfma(f32x16& acc, const bf16x8 (&wf)[K / 16], uint32_t xbuf, int l32, int hh) {
  constexpr int KS = K / 16, AHEAD = 4;
  uint32_t xa[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) xa[kk] = xbuf + 512 * l32 + 16 * ((2 * kk + hh) ^ (l32 & 7));
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 xf = lds_ld8(xa[ks & 3] + kPanel * (ks >> 4) + 128 * ((ks & 15) >> 2));
    mma32(acc, wf[ks], xf);
  }
  __builtin_amdgcn_sched_group_barrier(0x0100, AHEAD, 0);
#pragma unroll
  for (int ks = 0; ks < KS - AHEAD; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x0008, AHEAD, 0);
}

// Output staging.  A block of 32 rows x N columns (bf16) sits in LDS with
// the 16-byte chunk c of row r at position c ^ (r & 7).  Each wave writes
// its 4-column pieces (row l32, columns n0 + 8 g + 4 hh) from registers;
// after a barrier, whole rows leave as 16 bytes per lane (N/8 lanes a row),
// so every store instruction writes complete 128-byte lines.
template <int N>
WHALE_DEV void stage_piece(uint32_t ob, int l32, int hh, int n0, int g, const bf16x4& v) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int c = (n0 >> 3) + g;
  *(lds_bf16x4*)(uintptr_t)(ob + l32 * (N * 2) + 16 * (c ^ (l32 & 7)) + 8 * hh) = v;
}
// Rows of the staged block: instruction j covers rows j * (64 / (N/8)) ...;
// wave w takes j = w + NW t.  emit(m, n, v) writes the 8 values v of row m
// from column n on.  Rows past M store again row M-1's values (their inputs
// are copies of row M-1, so the values are the same bits), so the stores
// need no branch.
template <int N, int NW, typename Emit>
WHALE_DEV void store_rows(uint32_t ob, int w, int lane, int64_t m0, int64_t M, Emit emit) {
  constexpr int RC = N / 8, RPI = 64 / RC, NIW = kRB / RPI / NW;
  static_assert(NIW >= 1 && (kRB / RPI) % NW == 0, "rows per wave");
#pragma unroll
  for (int t = 0; t < NIW; ++t) {
    const int j = w + NW * t;
    const int r = j * RPI + lane / RC, c = lane % RC;
    const bf16x8 v = lds_ld8(ob + r * (N * 2) + 16 * (c ^ (r & 7)));
    emit(min(m0 + r, M - 1), 8 * c, v);
  }
}
// vmcnt(IPW * k) for k = 0, 1, 2 newer blocks of transfers in flight.
template <int IPW> WHALE_DEV void wait_newer(int k) {
  if (k >= 2) wait_vm<2 * IPW>();
  else if (k == 1) wait_vm<IPW>();
  else wait_vm<0>();
}

WHALE_DEV bf16x4 lds_ld4(uint32_t a) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return *(const lds_bf16x4*)(uintptr_t)a;
}
WHALE_DEV f32x2 lds_ldf2(uint32_t a) {
  typedef __attribute__((address_space(3))) f32x2 lds_f32x2;
  return *(const lds_f32x2*)(uintptr_t)a;
}
WHALE_DEV f32x4 lds_ldf4(uint32_t a) {
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  return *(const lds_f32x4*)(uintptr_t)a;
}

// ------------------------------------------------------------------ forward
// Y = Norm(H) W^T.  Waves with n0 < nsplit use W and write Y, the others W2
// and Y2 (the K and V projections in one pass over the history rows).  With
// the tied gate (gate = 1) the ngroups * N weight rows are split into
// column groups of N, one per workgroup; the staged block holds Z = the
// product (bf16) and the stores write Z (when kept) and U = SiLU(Z) Z.  Each
// wave moves and normalises the rows of its own transfers (2 rows per
// instruction at K = 256), so one barrier per block publishes both the
// normalised next block and this block's staged output.  Four input
// buffers keep three blocks of transfers in flight (HBM latency at one
// workgroup per CU needs that much); two output tiles alternate.
// EPI: 0 plain stores (Y / Y2 split at nsplit), 1 the tied gate, 2 the tied
// gate's backward (no norm): the staged product P = dY W_D^T is scaled by
// SiLU'(u) u + SiLU(u) with u = Z, read two lines ahead of the stores;
// 3 the fusion MLP's backward (no norm): the rows H = dF and Z arrive
// together, each wave forms dZ = dF SiLU'(Z) for its rows (in LDS and to
// Xn), the MFMAs read dZ, and columns >= nsplit add the residual dF.  The
// second input stream leaves room for two buffers only;
// 4 the fusion MLP (K = 512, no norm): the rows are [H | H2] (two panels),
// Y = H2 + SiLU(P) with the residual read from the second panel in LDS, and
// Z = P (when kept) from a second staged tile.
template <int K, int N, int EPI>
__global__ __launch_bounds__(N / 32 * 64) void rs_fwd_kernel(RsFwdArgs a) {
  constexpr int NW = N / 32, NT = NW * 64;
  constexpr int CPR = K / 8;                       // 16-byte chunks per row
  constexpr int BLK = kRB * K * 2;                 // bytes per block
  constexpr int NI = BLK / 1024;                   // transfer instructions per block
  constexpr int IPW = NI / NW;                     // ... per wave
  constexpr int NBUF = (EPI == 3 || EPI == 4) ? 2 : (K == 512 ? 3 : 4);
  static_assert(NI % NW == 0 && IPW >= 1 && (K == 256 || (K == 512 && N == 256 && (EPI == 0 || EPI == 4))),
                "panels, whole instructions");
  __shared__ __attribute__((aligned(1024))) char xs[NBUF][BLK];
  __shared__ __attribute__((aligned(1024))) char zb[EPI == 3 ? NBUF : 1][EPI == 3 ? BLK : 16];
  __shared__ __attribute__((aligned(1024))) char ob[2][kRB * N * 2];
  __shared__ __attribute__((aligned(1024))) char ob2[EPI == 4 ? 2 : 1][EPI == 4 ? kRB * N * 2 : 16];
  __shared__ __attribute__((aligned(16))) float gb[2][K];

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            hh = lane >> 5;
  const int64_t M = a.M;
  const int64_t nblk = (M + kRB - 1) / kRB;
  // Workgroup id 8 q + x (x = XCD): column group q % ngroups, row-block
  // walker 8 (q / ngroups) + x, so the groups of one row block share an XCD.
  const int ng = a.ngroups;
  const int grp = (blockIdx.x >> 3) % ng;
  const int G = gridDim.x / ng, b0 = ((blockIdx.x >> 3) / ng) * 8 + (blockIdx.x & 7);
  const int nmine = b0 < nblk ? (int)((nblk - 1 - b0) / G + 1) : 0;
  const bool nrm = EPI != 2 && a.kind != 2;

  const int n0 = 32 * w;
  // This wave's 32 output columns in the whole product (column group grp):
  // W and Y below nsplit, W2 and Y2 from it on.  The gate and its backward
  // (EPI 1, 2) take every group's rows from W (nsplit = N there).
  const int gc0 = grp * N + n0;
  const bool second = (EPI == 1 || EPI == 2) ? false : gc0 >= a.nsplit;
  const bf16* Wr = second ? a.W2 + (int64_t)(gc0 - a.nsplit + l32) * K : a.W + (int64_t)(gc0 + l32) * K;
  bf16x8 wf[K / 16];
#pragma unroll
  for (int ks = 0; ks < K / 16; ++ks) wf[ks] = ld8<bf16>(Wr + 16 * ks + 8 * hh);
  for (int k = tid; k < K; k += NT) {
    gb[0][k] = nrm ? a.gamma[k] : 1.f;
    gb[1][k] = nrm && a.kind == 0 ? a.beta[k] : 0.f;
  }
  // The weight slice is resident from here on: a wait the compiler sees, so
  // that it places no wait for these loads inside the loop.
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  auto emit = [&](int64_t m, int n, const bf16x8& v) {
    if (EPI == 1) {
      const int col = grp * N + n;
      if (a.Z) st8<bf16>(a.Z + m * a.ldz + col, v);
      if (a.Y) {
        bf16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float z = to_f(v[e]); u[e] = from_f<bf16>(siluf_(z) * z); }
        st8<bf16>(a.Y + m * a.ldy + col, u);
      }
    } else {
      const int col = grp * N + n;
      st8<bf16>(col < a.nsplit ? a.Y + m * a.ldy + col : a.Y2 + m * a.ldy + (col - a.nsplit), v);
    }
  };

  // Transfers of block b into buffer p: instruction j of the block covers
  // chunk positions [64 j, 64 j + 64); this wave issues j = w + NW t.
  auto issue = [&](int b, int p) {
    const int64_t m0 = (int64_t)b * kRB;
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
      const int j = w + NW * t, panel = j >> 4;
      dma_rows(panel ? a.H2 : a.H, panel ? a.ldh2 : a.ldh, m0, 2 * (j & 15), M, lane,
               lds_addr(&xs[p][panel * kPanel + 1024 * (j & 15)]));
      if constexpr (EPI == 3) dma_rows(a.Z, a.ldz, m0, 2 * j, M, lane, lds_addr(&zb[p][1024 * j]));
    }
  };
  // Normalise this wave's rows of block b in buffer p (after its transfers
  // landed): statistics over the row's CPR lanes (two passes, as the norm
  // kernels), the normalised row written back in place, to Xn and the
  // statistics to stats.
  auto normalise = [&](int b, int p) {
    if constexpr (EPI == 3) {
      // dZ = dF SiLU'(Z) over this wave's rows, into the Z buffer and to Xn.
      const int64_t m0 = (int64_t)b * kRB;
#pragma unroll
      for (int t = 0; t < IPW; ++t) {
        const int j = w + NW * t;
        const int q = 64 * j + lane, r = q / CPR, c = swz(q % CPR, r);
        const bf16x8 df = lds_ld8(lds_addr(&xs[p][16 * q]));
        const uint32_t za = lds_addr(&zb[p][16 * q]);
        const bf16x8 z = lds_ld8(za);
        bf16x8 dz;
#pragma unroll
        for (int u = 0; u < 8; ++u) dz[u] = from_f<bf16>(to_f(df[u]) * dsiluf_(to_f(z[u])));
        *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)za = dz;
        st8<bf16>(a.Xn + min(m0 + r, M - 1) * K + 8 * c, dz);   // (rows past M: row M-1 again)
      }
      return;
    }
    if (!nrm) return;
    const int64_t m0 = (int64_t)b * kRB;
    if constexpr (K == 512) {
      // A block is two panels of 256 columns; instruction j holds half-rows
      // 2 (j % 16) and 2 (j % 16) + 1 of panel j / 16.  This wave's
      // instructions j0 = w + NW t (t = 0, 1) and j0 + 16 are the two halves
      // of the same rows (NW = 8), so a row's statistics reduce over the 32
      // lanes of its lane half, across the wave's two instructions.
#pragma unroll
      for (int t = 0; t < IPW / 2; ++t) {
        const int j0 = w + NW * t;
        const int r = 2 * j0 + hh, pos = l32, c = swz(pos, r);
        const uint32_t la0 = lds_addr(&xs[p][1024 * j0 + 16 * lane]);
        const uint32_t la1 = la0 + kPanel;
        const bf16x8 raw0 = lds_ld8(la0), raw1 = lds_ld8(la1);
        float v[16];
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) { v[u] = to_f(raw0[u]); v[u + 8] = to_f(raw1[u]); }
#pragma unroll
        for (int u = 0; u < 16; ++u) s += v[u];
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) s += __shfl_xor(s, o);
        const float mean = a.kind == 0 ? s / K : 0.f;
        float qs = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) { const float dl = v[u] - mean; qs += dl * dl; }
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) qs += __shfl_xor(qs, o);
        const float rstd = 1.f / sqrtf(qs / K + a.eps);
        const int64_t m = min(m0 + r, M - 1);   // (rows past M: row M-1 again, same values)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int col = 256 * half + 8 * c;
          const f32x4 g0 = lds_ldf4(lds_addr(&gb[0][col])), g1 = lds_ldf4(lds_addr(&gb[0][col + 4]));
          const f32x4 e0 = lds_ldf4(lds_addr(&gb[1][col])), e1 = lds_ldf4(lds_addr(&gb[1][col + 4]));
          bf16x8 y;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            y[u] = from_f<bf16>((v[8 * half + u] - mean) * rstd * g0[u] + e0[u]);
            y[u + 4] = from_f<bf16>((v[8 * half + u + 4] - mean) * rstd * g1[u] + e1[u]);
          }
          *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(half ? la1 : la0) = y;
          if (a.Xn && grp == 0) st8<bf16>(a.Xn + m * K + col, y);
        }
        if (a.stats && pos == 0 && grp == 0) *reinterpret_cast<f32x2*>(a.stats + 2 * m) = f32x2{mean, rstd};
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
      const int j = w + NW * t;
      const int q = 64 * j + lane, r = q / CPR, pos = q % CPR;
      const int c = swz(pos, r);
      const uint32_t la = lds_addr(&xs[p][16 * q]);
      const bf16x8 raw = lds_ld8(la);
      float v[8];
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) { v[u] = to_f(raw[u]); s += v[u]; }
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) s += __shfl_xor(s, o);
      const float mean = a.kind == 0 ? s / K : 0.f;
      float qs = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) { const float dl = v[u] - mean; qs += dl * dl; }
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) qs += __shfl_xor(qs, o);
      const float rstd = 1.f / sqrtf(qs / K + a.eps);
      const f32x4 g0 = lds_ldf4(lds_addr(&gb[0][8 * c])), g1 = lds_ldf4(lds_addr(&gb[0][8 * c + 4]));
      const f32x4 e0 = lds_ldf4(lds_addr(&gb[1][8 * c])), e1 = lds_ldf4(lds_addr(&gb[1][8 * c + 4]));
      bf16x8 y;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        y[u] = from_f<bf16>((v[u] - mean) * rstd * g0[u] + e0[u]);
        y[u + 4] = from_f<bf16>((v[u + 4] - mean) * rstd * g1[u] + e1[u]);
      }
      *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)la = y;
      const int64_t m = min(m0 + r, M - 1);   // (rows past M: row M-1 again, same values)
      if (a.Xn && grp == 0) st8<bf16>(a.Xn + m * K + 8 * c, y);
      if (a.stats && pos == 0 && grp == 0) *reinterpret_cast<f32x2*>(a.stats + 2 * m) = f32x2{mean, rstd};
    }
  };

  for (int k = 0; k < NBUF - 1 && k < nmine; ++k) issue(b0 + k * G, k);
  wait_newer<IPW>(min(NBUF - 2, nmine - 1));        // block 0 landed
  __syncthreads();                                   // gamma / beta
  if (nmine > 0) normalise(b0, 0);
  __syncthreads();

  for (int i = 0; i < nmine; ++i) {
    const int p = i % NBUF;
    const int64_t m0 = (int64_t)(b0 + i * G) * kRB;
    // Buffer (i+3) % 4 was last read by block i-1, before the last barrier.
    if (i + NBUF - 1 < nmine) issue(b0 + (i + NBUF - 1) * G, (i + NBUF - 1) % NBUF);
    // The gate input of the rows this wave stores for block i (see
    // store_rows), in flight during the MFMAs.
    constexpr int RC = N / 8, RPI = 64 / RC, NIW = kRB / RPI / NW;
    bf16x8 zin[EPI == 2 ? NIW : 1];
    if constexpr (EPI == 2) {
#pragma unroll
      for (int t = 0; t < NIW; ++t) {
        const int r = (w + NW * t) * RPI + lane / RC;
        const int64_t m = min(m0 + r, M - 1);
        zin[t] = ld8<bf16>(a.Z + m * a.ldz + grp * N + 8 * (lane % RC));
      }
    }
    f32x16 acc = zero16();
    block_mfma<K>(acc, wf, lds_addr(EPI == 3 ? &zb[p][0] : &xs[p][0]), l32, hh);
    // Output tile i & 1 was last read by the stores of block i-2, before
    // the last barrier.
    const uint32_t obp = lds_addr(&ob[i & 1][0]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 o;
      if constexpr (EPI == 4) {
        // residual H2 of row l32, columns n0 + 8 g + 4 hh + u (second panel)
        const int c = (n0 >> 3) + g;
        const bf16x4 rv = lds_ld4(lds_addr(&xs[p][kPanel]) + 512 * l32 + 16 * (c ^ (l32 & 7)) + 8 * hh);
        bf16x4 zo;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float z = acc[4 * g + u];
          o[u] = from_f<bf16>(to_f(rv[u]) + siluf_(z));
          zo[u] = from_f<bf16>(z);
        }
        stage_piece<N>(lds_addr(&ob2[i & 1][0]), l32, hh, n0, g, zo);
      } else if (EPI == 3 && second) {
        // residual dF of row l32, columns n0 - nsplit + 8 g + 4 hh + u
        const int c = ((n0 - a.nsplit) >> 3) + g;
        const bf16x4 rv = lds_ld4(lds_addr(&xs[p][0]) + 512 * l32 + 16 * (c ^ (l32 & 7)) + 8 * hh);
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = from_f<bf16>(acc[4 * g + u] + to_f(rv[u]));
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = from_f<bf16>(acc[4 * g + u]);
      }
      stage_piece<N>(obp, l32, hh, n0, g, o);
    }
    // This wave's transfers of block i+1 have landed once at most the newer
    // blocks' ones are outstanding (loads complete in order; the stores
    // issued between are waited for too, which measured no slower than
    // counting them).
    if (i + 1 < nmine) {
      wait_newer<IPW>(min(NBUF - 2, nmine - i - 2));
      normalise(b0 + (i + 1) * G, (i + 1) % NBUF);
    }
    __syncthreads();
    if constexpr (EPI == 2) {
#pragma unroll
      for (int t = 0; t < NIW; ++t) {
        const int r = (w + NW * t) * RPI + lane / RC, c = lane % RC;
        const bf16x8 v = lds_ld8(obp + r * (N * 2) + 16 * (c ^ (r & 7)));
        const int64_t m = min(m0 + r, M - 1);   // (rows past M: row M-1 again, same values)
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float u = to_f(zin[t][e]);
          o[e] = from_f<bf16>(to_f(v[e]) * (dsiluf_(u) * u + siluf_(u)));
        }
        st8<bf16>(a.Y + m * a.ldy + grp * N + 8 * c, o);
      }
    } else {
      store_rows<N, NW>(obp, w, lane, m0, M, emit);
      if constexpr (EPI == 4) {
        if (a.Z)
          store_rows<N, NW>(lds_addr(&ob2[i & 1][0]), w, lane, m0, M,
                            [&](int64_t m, int n, const bf16x8& v) { st8<bf16>(a.Z + m * a.ldz + n, v); });
      }
    }
  }
}

// ----------------------------------------------------------------- backward
// dX = Norm backward(dY W^T) + R with dY = [X | X2] split at ksplit along K.
// Per block: MFMAs, then this wave's partial row sums of the norm backward
// (over its 32 columns) go to LDS; one barrier publishes them and the next
// block's transfers; then the transfers of block i+2 start, the previous
// block's staged output rows are stored, and every wave forms the full row
// sums in a fixed order and stages its columns.  Two input buffers are all
// that fit next to the output tiles (x, R and the K-deep dY rows per block).
// dgamma / dbeta column partials accumulate in registers over all rows a
// lane handles and are reduced across lanes once, at the end:
// part [gridDim.x, 2, N].  HASR: R is read (K = 256 only, for LDS space).
template <int K, int N, bool HASR>
__global__ __launch_bounds__(N / 32 * 64) void rs_bwd_kernel(RsBwdArgs a) {
  constexpr int NW = N / 32, NT = NW * 64;
  constexpr int XB = kRB * K * 2, NB = kRB * N * 2;
  constexpr int XI = XB / 1024 / NW, NI = NB / 1024 / NW;   // transfer instructions per wave
  static_assert(XB % (1024 * NW) == 0 && NB % (1024 * NW) == 0 && XI >= 1 && NI >= 1, "block / wave split");
  static_assert((K == 256 || K == 512) && N == 256, "panels of 256 columns");
  __shared__ __attribute__((aligned(1024))) char xs[2][XB];
  __shared__ __attribute__((aligned(1024))) char ns[2][NB];
  __shared__ __attribute__((aligned(1024))) char rsb[HASR ? 2 : 1][HASR ? NB : 16];
  __shared__ __attribute__((aligned(1024))) char ob[2][NB];
  __shared__ __attribute__((aligned(256))) float ss[2][64];
  __shared__ __attribute__((aligned(16))) float red[2][NW][kRB][2];
  __shared__ __attribute__((aligned(16))) float gm[N];

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            hh = lane >> 5;
  const int64_t M = a.M;
  const int64_t nblk = (M + kRB - 1) / kRB;
  const int G = gridDim.x, b0 = blockIdx.x;
  const int nmine = b0 < nblk ? (int)((nblk - 1 - b0) / G + 1) : 0;
  const int kind = a.kind;
  const bool nrm = kind != 2, hasR = HASR && a.R != nullptr;

  const int n0 = 32 * w;
  bf16x8 wf[K / 16];
  {
    const bf16* Wr = a.W + (int64_t)(n0 + l32) * K;
#pragma unroll
    for (int ks = 0; ks < K / 16; ++ks) wf[ks] = ld8<bf16>(Wr + 16 * ks + 8 * hh);
  }
  for (int n = tid; n < N; n += NT) gm[n] = nrm ? a.gamma[n] : 1.f;
  __builtin_amdgcn_s_waitcnt(kVmcnt0);   // weight slice resident (see the forward kernel)

  auto issue = [&](int b, int p) {
    const int64_t m0 = (int64_t)b * kRB;
#pragma unroll
    for (int t = 0; t < XI; ++t) {
      const int j = w + NW * t, panel = j >> 4;
      dma_rows(panel ? a.X2 : a.X, panel ? a.ldx2 : a.ldx, m0, 2 * (j & 15), M, lane,
               lds_addr(&xs[p][panel * kPanel + 1024 * (j & 15)]));
    }
    if (nrm) {
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        const int j = w + NW * t;
        dma_rows(a.nx, N, m0, 2 * j, M, lane, lds_addr(&ns[p][1024 * j]));
      }
      if (w == NW - 1) {
        const int64_t last = M - 1 - m0;
        const int row = (lane >> 1) < last ? (lane >> 1) : (int)last;
        dma4(a.stats + 2 * m0, (uint32_t)(8 * row + 4 * (lane & 1)), lds_addr(&ss[p][0]));
      }
    }
    if (hasR) {
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        const int j = w + NW * t;
        dma_rows(a.R, N, m0, 2 * j, M, lane, lds_addr(&rsb[HASR ? p : 0][1024 * j]));
      }
    }
  };

  auto ydst = [&](int64_t m, int n, const bf16x8& v) { st8<bf16>(a.Y + m * N + n, v); };
  float pg[16], pb[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) { pg[u] = 0.f; pb[u] = 0.f; }
  const float invn = 1.f / N;

  if (nmine > 0) issue(b0, 0);
  wait_vm<0>();
  __syncthreads();
  if (nmine > 1) issue(b0 + G, 1);

  for (int i = 0; i < nmine; ++i) {
    const int p = i & 1;
    const int64_t m0 = (int64_t)(b0 + i * G) * kRB;
    f32x16 acc = zero16();
    block_mfma<K>(acc, wf, lds_addr(&xs[p][0]), l32, hh);
    // acc[4 g + u] = dY W^T at row m0 + l32, column n0 + 8 g + 4 hh + u.
    // x and R of those columns are read now (the buffer is refilled after
    // the barrier) and kept as bf16.
    bf16x4 xv[4], r4[4];
    float mean = 0.f, rstd = 1.f;
    if (nrm) {
      const f32x2 st = lds_ldf2(lds_addr(&ss[p][2 * l32]));
      mean = st[0];
      rstd = st[1];
    }
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = swz((n0 >> 3) + g, l32);
      const uint32_t off = l32 * (N * 2) + 16 * c + 8 * hh;
      if (nrm) xv[g] = lds_ld4(lds_addr(&ns[p][0]) + off);
      if (hasR) r4[g] = lds_ld4(lds_addr(&rsb[HASR ? p : 0][0]) + off);
      const f32x4 gg = lds_ldf4(lds_addr(&gm[n0 + 8 * g + 4 * hh]));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float xh = nrm ? (to_f(xv[g][u]) - mean) * rstd : 0.f;
        const float gd = acc[4 * g + u] * gg[u];
        s1 += gd;
        s2 += gd * xh;
      }
    }
    if (nrm) {
      s1 = half_sum(s1);
      s2 = half_sum(s2);
      if (hh == 0) *(__attribute__((address_space(3))) f32x2*)(uintptr_t)lds_addr(&red[p][w][l32][0]) = f32x2{s1, s2};
    }
    // This wave's transfers of block i+1 (and its older stores) are done.
    wait_vm<0>();
    __syncthreads();
    // Buffer p is free since the barrier; block i+2 goes there.
    if (i + 2 < nmine) issue(b0 + (i + 2) * G, p);
    // The previous block's output (staged before the barrier).
    if (i > 0) store_rows<N, NW>(lds_addr(&ob[(i - 1) & 1][0]), w, lane, m0 - (int64_t)G * kRB, M, ydst);

    float c1 = 0.f, c2 = 0.f;
    if (nrm) {
      float t1 = 0.f, t2 = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const f32x2 e = lds_ldf2(lds_addr(&red[p][v][l32][0]));
        t1 += e[0];
        t2 += e[1];
      }
      c1 = kind == 0 ? t1 * invn : 0.f;
      c2 = t2 * invn;
    }
    // Output tile i & 1 was last read by the stores of block i-2, before
    // this block's barrier.
    const uint32_t obp = lds_addr(&ob[i & 1][0]);
    const bool valid = m0 + l32 < M;
    {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 gg = lds_ldf4(lds_addr(&gm[n0 + 8 * g + 4 * hh]));
        bf16x4 o;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = 4 * g + u;
          const float dxn = acc[e];
          const float xh = nrm ? (to_f(xv[g][u]) - mean) * rstd : 0.f;
          const float rv = hasR ? to_f(r4[g][u]) : 0.f;
          o[u] = from_f<bf16>(rv + (nrm ? rstd * (dxn * gg[u] - c1 - xh * c2) : dxn));
          if (valid) {
            pg[e] += dxn * xh;
            pb[e] += dxn;
          }
        }
        stage_piece<N>(obp, l32, hh, n0, g, o);
      }
    }
  }
  if (nmine > 0) {
    __syncthreads();
    store_rows<N, NW>(lds_addr(&ob[(nmine - 1) & 1][0]), w, lane, (int64_t)(b0 + (nmine - 1) * G) * kRB, M, ydst);
  }

  if (nrm) {
    // Column partials: lanes with the same hh hold the same 16 columns.
#pragma unroll
    for (int o = 1; o < 32; o <<= 1)
#pragma unroll
      for (int e = 0; e < 16; ++e) { pg[e] += __shfl_xor(pg[e], o); pb[e] += __shfl_xor(pb[e], o); }
    if (l32 == 0) {
      float* pr = a.part + (int64_t)blockIdx.x * 2 * N;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int n = n0 + 8 * g + 4 * hh + u;
          pr[n] = pg[4 * g + u];
          pr[N + n] = pb[4 * g + u];
        }
    }
  }
}

constexpr int kCUsRS = 256;

}  // namespace

bool rs_fwd_ok(int K, int N) { return (K == 256 && (N == 256 || N == 512)) || (K == 512 && N == 256); }
// Plain projection K -> ngroups * N by column groups at K = 512.
bool rs_fwd_groups_ok(int K, int Ntot) { return K == 512 && Ntot % 256 == 0 && kCUsRS % (8 * (Ntot / 256)) == 0; }
bool rs_bwd_ok(int K, int N) { return (K == 256 || K == 512) && N == 256; }
int64_t rs_bwd_grid(int64_t M) {
  const int64_t g = (M + 63) / 64;
  return g < kCUsRS ? g : kCUsRS;
}

hipError_t launch_rs_fwd(const RsFwdArgs& a, int K, int N, hipStream_t st) {
  if (!rs_fwd_ok(K, N) || a.M < 0 || a.nsplit % 32 != 0 || a.nsplit <= 0) return hipErrorInvalidValue;
  // Column groups: the gated forms (nsplit = N), or the plain projection at
  // K = 512 (N = 256 per group; nsplit anywhere on the 256-column grid).
  if (a.ngroups < 1 || kCUsRS % (8 * a.ngroups) != 0 ||
      (a.ngroups > 1 && !(a.gate != 0 && a.nsplit == N) && !(a.gate == 0 && K == 512 && a.nsplit % N == 0)))
    return hipErrorInvalidValue;
  if (a.M == 0) return hipSuccess;
  // Row-block walkers per column group: a multiple of 8 (one set per XCD).
  const int64_t nblk = (a.M + kRB - 1) / kRB;
  const int64_t per = kCUsRS / a.ngroups;
  const int64_t gg = ((nblk < per ? nblk : per) + 7) / 8 * 8;
  const int g = (int)(gg * a.ngroups);
  if (K == 256 && N == 256 && a.gate == 0)
    hipLaunchKernelGGL((rs_fwd_kernel<256, 256, 0>), dim3(g), dim3(512), 0, st, a);
  else if (K == 256 && N == 512 && a.gate == 0)
    hipLaunchKernelGGL((rs_fwd_kernel<256, 512, 0>), dim3(g), dim3(1024), 0, st, a);
  else if (K == 256 && N == 512 && a.gate == 1)
    hipLaunchKernelGGL((rs_fwd_kernel<256, 512, 1>), dim3(g), dim3(1024), 0, st, a);
  else if (K == 256 && N == 512 && a.gate == 2 && a.Z != nullptr)
    hipLaunchKernelGGL((rs_fwd_kernel<256, 512, 2>), dim3(g), dim3(1024), 0, st, a);
  else if (K == 256 && N == 512 && a.gate == 3 && a.Z != nullptr && a.Xn != nullptr && a.ngroups == 1)
    hipLaunchKernelGGL((rs_fwd_kernel<256, 512, 3>), dim3(g), dim3(1024), 0, st, a);
  else if (a.gate == 4 && K == 512 && N == 256 && a.H2 != nullptr && a.ngroups == 1)
    hipLaunchKernelGGL((rs_fwd_kernel<512, 256, 4>), dim3(g), dim3(512), 0, st, a);
  else if (a.gate == 0 && K == 512 && N == 256) {
    // The two 256-column panels of a row come from H itself.
    RsFwdArgs b = a;
    b.H2 = a.H + 256; b.ldh2 = a.ldh;
    hipLaunchKernelGGL((rs_fwd_kernel<512, 256, 0>), dim3(g), dim3(512), 0, st, b);
  }
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_rs_bwd(const RsBwdArgs& a, int K, int N, hipStream_t st) {
  // Columns [0, 256) of dY come from X, [256, 512) from X2.
  // (At K = 512 the LDS holds no R tiles: R must be null there.)
  if (!rs_bwd_ok(K, N) || a.M < 0 || a.ksplit != 256 || (K == 512 && (a.X2 == nullptr || a.R != nullptr)))
    return hipErrorInvalidValue;
  if (a.M == 0) return hipSuccess;
  const int g = (int)rs_bwd_grid(a.M);
  if (K == 256)
    hipLaunchKernelGGL((rs_bwd_kernel<256, 256, true>), dim3(g), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((rs_bwd_kernel<512, 256, false>), dim3(g), dim3(512), 0, st, a);
  return hipGetLastError();
}
