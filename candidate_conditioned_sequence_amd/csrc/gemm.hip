// Projection, fusion-MLP and FFN GEMMs (gfx950 MFMA, fp32 accumulation).
//
//  * gemm_nt: Y[M,N] = op(X)[M,K] W[N,K]^T.  Both operands are
//    K-contiguous, so the 32x32x16 MFMA operands are 16-byte rows of the LDS
//    tiles.  The X tile loader can apply the row norm (stats + gamma/beta),
//    read the concatenation [X | X2], or form dZ = dF * SiLU'(Z) on the fly.
//    W rows may come from two matrices (K and V projections in one pass over
//    H_s; gate and up halves of a separate-gate SwiGLU side by side).
//    The accumulators are staged through LDS so that the epilogue reads its
//    other operands and writes its outputs in 16-byte coalesced chunks; the
//    epilogue fuses the residual, SiLU, the shared-gate SwiGLU product
//    G = SiLU(U) U (gist.science Technical Summary §2.2; paper-daily.com deep
//    reading §2), the gate derivatives, and -- for tiles that span whole rows
//    -- the norm backward, so dX never goes to memory.
//  * wgrad: dW[N,K] = sum_m G[m,n] X[m,k].  The contraction runs over the
//    rows of both operands.  Each thread loads an 8x8 block, transposes it in
//    registers and writes eight 16-byte rows of the transposed LDS tile.  M is
//    split into fixed chunks whose fp32 partials a second kernel sums in a
//    fixed order: deterministic, no atomics.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

template <typename T>
WHALE_DEV x8_t<T> norm8(const x8_t<T>& v, float mean, float rstd, const float* g, const float* bt, int kind) {
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(g), g1 = *reinterpret_cast<const f32x4*>(g + 4);
  f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
  if (kind == 0) { b0 = *reinterpret_cast<const f32x4*>(bt); b1 = *reinterpret_cast<const f32x4*>(bt + 4); }
  x8_t<T> o;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    o[u] = from_f<T>((to_f(v[u]) - mean) * rstd * g0[u] + b0[u]);
    o[u + 4] = from_f<T>((to_f(v[u + 4]) - mean) * rstd * g1[u] + b1[u]);
  }
  return o;
}

template <typename T>
WHALE_DEV x8_t<T> dact8(const x8_t<T>& g, const x8_t<T>& z) {
  x8_t<T> o;
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = from_f<T>(to_f(g[u]) * dsiluf_(to_f(z[u])));
  return o;
}

template <typename T> WHALE_DEV void ld8f(const T* p, float* f) {
  const x8_t<T> v = ld8<T>(p);
#pragma unroll
  for (int u = 0; u < 8; ++u) f[u] = to_f(v[u]);
}
template <typename T> WHALE_DEV void st8f(T* p, const float* f) {
  x8_t<T> v;
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = from_f<T>(f[u]);
  st8<T>(p, v);
}

// ------------------------------------------------------------------ gemm_nt
// Persistent kernel: each workgroup walks a strided list of BM x BN output
// tiles inside its XCD's contiguous tile range (so the column tiles of one row
// block meet in one L2), BK-deep K steps double-buffered in LDS, one wave per
// 64x64 sub-tile.  The first K step of the next tile is loaded into registers
// before the epilogue of the current one, so its latency hides behind the
// epilogue.  The fp32 accumulators are staged through LDS, SROWS rows at a
// time, for coalesced 16-byte epilogue accesses.
template <typename T, int PRO, int EPI, bool YF32, int BM, int BN, int BK>
__global__ __launch_bounds__((BM / 64) * (BN / 64) * 64, 2) void gemm_nt_kernel(GemmArgs a, int tiles_n, int ntiles) {
  constexpr int NWN = BN / 64, NWM = BM / 64, NT = NWM * NWN * 64;
  constexpr int LDT = BK + 8;                 // LDS tile row stride (elements)
  constexpr int SLD = BN + 4;                 // staging row stride (floats)
  constexpr int CPR = BK / 8;                 // 8-element chunks per tile row
  constexpr int ACH = (BM * CPR + NT - 1) / NT, BCH = (BN * CPR + NT - 1) / NT;   // chunks per thread
  static_assert((BM * CPR) % 64 == 0 && (BN * CPR) % NT == 0, "tile/threads");
  // The epilogue stages 64 rows per pass (row-complete for the norm backward).
  constexpr int SROWS = 64;
  constexpr int TILE_BYTES = 2 * (BM + BN) * LDT * (int)sizeof(T);
  constexpr int STG_BYTES = SROWS * SLD * 4;
  __shared__ __attribute__((aligned(32))) char smem[TILE_BYTES > STG_BYTES ? TILE_BYTES : STG_BYTES];
  T* As = reinterpret_cast<T*>(smem);                    // [2][BM*LDT]
  T* Bs = As + 2 * BM * LDT;                             // [2][BN*LDT]
  float* stg = reinterpret_cast<float*>(smem);           // [SROWS][SLD], between K loops
  typedef typename std::conditional<YF32, float, T>::type YT;
  // Norm prologue: gamma / beta of the K columns (K = d <= 512) held in LDS.
  __shared__ __attribute__((aligned(16))) float sgb[PRO == PRO_NORM ? 2 * 512 : 4];
  if (PRO == PRO_NORM) {
    for (int k = threadIdx.x; k < a.K && k < 512; k += blockDim.x) {
      sgb[k] = a.norm_kind != 2 ? a.gamma[k] : 1.f;
      sgb[512 + k] = a.norm_kind == 0 ? a.beta[k] : 0.f;
    }
    __syncthreads();
  }

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wm = w / NWN, wn = w % NWN;
  const int64_t M = a.M;
  const int N = a.N, K = a.K;
  const T* X = (const T*)a.X;
  const T* X2 = (const T*)a.X2;
  const T* W = (const T*)a.W;
  const T* W2 = (const T*)a.W2;
  const int Hs = N / 2;   // EPI_GATE_SEP: number of gate rows
  YT* Y = (YT*)a.Y;
  const T* R = (const T*)a.R;
  T* Z = (T*)a.Z;

  // This workgroup's tiles: XCD x = blockIdx % 8 owns [x n / 8, (x+1) n / 8).
  const int G = gridDim.x, xcd = blockIdx.x & 7, rnk = blockIdx.x >> 3;
  const int gx = (G - xcd + 7) >> 3;
  const int t_lo = (int)((int64_t)xcd * ntiles / 8), t_hi = (int)((int64_t)(xcd + 1) * ntiles / 8);

  float amean[ACH], arstd[ACH];
  const T* aptr[ACH];
  const T* aptr2[ACH];
  const T* bptr[BCH];
  // PIPE K steps in flight in registers (slot = K step mod PIPE).
  constexpr int PIPE = 2;
  x8_t<T> ar[PIPE][ACH], br[PIPE][BCH];

  auto setup = [&](int tile) {
    const int tn = tile % tiles_n, tm = tile / tiles_n;
    const int64_t m0 = (int64_t)tm * BM;
    const int n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int ch = tid + NT * i;
      // Rows past M (and chunks past the tile) read row M-1: their products
      // land in output rows or columns the epilogues never write, and the
      // loads stay unmasked.
      const int64_t m = min(m0 + ch / CPR, M - 1);
      amean[i] = 0.f;
      arstd[i] = 1.f;
      if (PRO == PRO_NORM && a.norm_kind != 2) { amean[i] = a.stats[2 * m]; arstd[i] = a.stats[2 * m + 1]; }
      aptr[i] = X + m * a.ldx + 8 * (ch % CPR);
      aptr2[i] = X2 ? X2 + m * a.ldx2 + 8 * (ch % CPR) : aptr[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int ch = tid + NT * i;
      const int tr = ch / CPR;
      const T* p;
      if (EPI == EPI_GATE_SEP) {
        // tile rows [64 v, 64 v + 32) gate rows, [64 v + 32, 64 v + 64) up rows, same output columns
        const int n = min(n0 / 2 + (tr >> 6) * 32 + (tr & 31), Hs - 1);
        p = W + (int64_t)(((tr >> 5) & 1) ? Hs + n : n) * a.ldw;
      } else {
        const int n = min(n0 + tr, N - 1);
        p = (W2 != nullptr && n >= a.nsplit) ? W2 + (int64_t)(n - a.nsplit) * a.ldw : W + (int64_t)n * a.ldw;
      }
      bptr[i] = p + 8 * (ch % CPR);
    }
  };
  // Raw loads of one K step into a slot; the prologue math (norm, dZ) is
  // applied when the slot is written to LDS, so the loads stay in flight.
  auto load = [&](int slot, int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const bool second = PRO == PRO_CONCAT && k0 >= a.ksplit;
      ar[slot][i] = ld8<T>(second ? aptr2[i] + (k0 - a.ksplit) : aptr[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) br[slot][i] = ld8<T>(bptr[i] + k0);
  };
  auto store = [&](int slot, int buf, int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int ch = tid + NT * i;
      if (ch >= BM * CPR) continue;
      x8_t<T> v = ar[slot][i];
      if (PRO == PRO_GATE) {
#pragma unroll
        for (int u = 0; u < 8; ++u) { const float z = to_f(v[u]); v[u] = from_f<T>(siluf_(z) * z); }
      } else if (PRO == PRO_DACT) {
        v = dact8<T>(v, ld8<T>(aptr2[i] + k0));
      } else if (PRO == PRO_NORM && a.norm_kind != 2) {
        const int k = k0 + 8 * (ch % CPR);
        v = norm8<T>(v, amean[i], arstd[i], &sgb[k], &sgb[512 + k], 0);
      }
      st8<T>(&As[buf * BM * LDT + (ch / CPR) * LDT + 8 * (ch % CPR)], v);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int ch = tid + NT * i;
      st8<T>(&Bs[buf * BN * LDT + (ch / CPR) * LDT + 8 * (ch % CPR)], br[slot][i]);
    }
  };
  // (With a single K step the second slot refetches it; it is never read.)
  auto prefetch_tile = [&](int t) {
    setup(t);
#pragma unroll
    for (int u = 0; u < PIPE; ++u) load(u, min(u * BK, a.K - BK));
  };

  const int nk = K / BK;
  int tile = t_lo + rnk;
  if (tile < t_hi) prefetch_tile(tile);

  for (; tile < t_hi; tile += gx) {
    const int tn = tile % tiles_n, tm = tile / tiles_n;
    const int64_t m0 = (int64_t)tm * BM;
    const int n0 = tn * BN;
    store(0, 0, 0);
    __syncthreads();

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) acc[i][jj] = zero16();
    for (int kt0 = 0; kt0 < nk; kt0 += PIPE) {
#pragma unroll
      for (int u = 0; u < PIPE; ++u) {
        const int kt = kt0 + u;
        if (kt < nk) {
          const int buf = kt & 1;
          const T* At = As + buf * BM * LDT;
          const T* Bt = Bs + buf * BN * LDT;
          __builtin_amdgcn_s_setprio(1);
          // slot u (K step kt) is in LDS now: refill it with K step kt + PIPE
          // (the last steps reload the last K step)
          load(u, min(kt + PIPE, nk - 1) * BK);
#pragma unroll
          for (int ks = 0; ks < BK / 16; ++ks) {
            x8_t<T> af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) af[i] = ld8<T>(&At[(wm * 64 + 32 * i + l32) * LDT + 16 * ks + 8 * hh]);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) bf[jj] = ld8<T>(&Bt[(wn * 64 + 32 * jj + l32) * LDT + 16 * ks + 8 * hh]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int jj = 0; jj < 2; ++jj) mma32(acc[i][jj], af[i], bf[jj]);
          }
          if constexpr (sizeof(T) == 2) {
            constexpr int NV = ACH + BCH;
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
              __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
                if (4 * ks + m < NV) __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);
              }
            }
          }
          __builtin_amdgcn_s_setprio(0);
          store((u + 1) % PIPE, buf ^ 1, min(kt + 1, nk - 1) * BK);
          __syncthreads();
        }
      }
    }
    // Epilogue inputs (residual R, saved pre-activation Z) of every pass are
    // loaded now, from clamped rows and columns (unused where out of range),
    // ahead of the next tile's operand loads: waiting for them later does not
    // wait for those.
    constexpr int OUTC = (EPI == EPI_GATE_SEP) ? BN / 2 : BN;   // output columns per tile
    constexpr int CH = SROWS * OUTC / 8;                         // 8-column chunks per pass
    constexpr int CPT = (CH + NT - 1) / NT;
    constexpr int NP = BM / SROWS;
    // (The separate-gate backward needs two inputs per chunk; preloading both
    // would not fit in registers, so it loads them where they are used.)
    constexpr int NL = (EPI == EPI_RESID || EPI == EPI_SILU_RESID || EPI == EPI_DUAL_RESID2 || EPI == EPI_DGATE_TIED) ? 1 : 0;
    x8_t<T> pre[NP][CPT][1];
    if constexpr (NL > 0 && EPI != EPI_NORM_BWD) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          const int c = min(tid + i * NT, CH - 1);
          const int row = c / (OUTC / 8), col = 8 * (c % (OUTC / 8));
          const int64_t m = min(m0 + p * SROWS + row, M - 1);
          const int n = min(n0 + col, N - 1);
          if (EPI == EPI_DUAL_RESID2) {
            pre[p][i][0] = ld8<T>(R + m * a.ldr + max(n - a.nsplit, 0));
          } else if (EPI == EPI_DGATE_TIED) {
            pre[p][i][0] = ld8<T>(Z + m * a.ldz + n);
          } else {
            pre[p][i][0] = ld8<T>(R + m * a.ldr + n);
          }
        }
    }

    // The next tile's first K steps go in flight during this epilogue (the
    // last tile refetches its own, unused: an unconditional prefetch lets the
    // waits above count exactly).
    prefetch_tile(tile + gx < t_hi ? tile + gx : tile);

#pragma unroll
    for (int pass = 0; pass < BM / SROWS; ++pass) {
      // Stage rows [pass*SROWS, (pass+1)*SROWS) of the tile (fp32).
      if (SROWS == BM || wm == pass) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              stg[(wm * 64 - pass * SROWS + 32 * i + acc_row(r, hh)) * SLD + wn * 64 + 32 * jj + l32] = acc[i][jj][r];
      }
      __syncthreads();
      const int64_t r0 = m0 + pass * SROWS;

      if (EPI == EPI_NORM_BWD) {
        // The tile spans whole rows (N == BN).  A group of BN/8 lanes owns a
        // row; each thread handles NIT rows of the pass, NB at a time.  The
        // inputs of a batch (x, R, the row statistics) are loaded first, the
        // row sums of its NB rows advance together, then a second sweep
        // writes the outputs.
        constexpr int LPR = BN / 8;                 // lanes per row (power of two, <= 64)
        constexpr int RPP = 64 / LPR;               // rows per wave pass
        constexpr int NIT = SROWS / ((NT / 64) * RPP);
        constexpr int NB = NIT < (BN >= 256 ? 4 : 2) ? NIT : (BN >= 256 ? 4 : 2);   // registers
        const int rpp = RPP;
        const int sub = lane / LPR, cl = lane % LPR;
        const int c0 = 8 * cl;
        float pg[8], pb[8], gmm[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) { pg[u] = 0.f; pb[u] = 0.f; gmm[u] = a.norm_kind == 2 ? 1.f : a.gamma[c0 + u]; }
        const float invn = 1.f / N;
#pragma unroll
        for (int i0 = 0; i0 < NIT; i0 += NB) {
          x8_t<T> xin[NB], rin[NB];
          float mean[NB], rstd[NB], s1[NB], s2[NB];
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int row = (w + (i0 + j) * (NT / 64)) * RPP + sub;
            const int64_t m = min(r0 + row, M - 1);
            xin[j] = ld8<T>((const T*)a.nx + m * N + c0);
            rin[j] = R ? ld8<T>(R + m * a.ldr + c0) : zero8<T>();
            mean[j] = 0.f;
            rstd[j] = 1.f;
            if (a.norm_kind != 2) { mean[j] = a.stats[2 * m]; rstd[j] = a.stats[2 * m + 1]; }
          }
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int row = (w + (i0 + j) * (NT / 64)) * RPP + sub;
            const bool ok = r0 + row < M;
            s1[j] = 0.f;
            s2[j] = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const float xh = (to_f(xin[j][u]) - mean[j]) * rstd[j];
              const float gd = ok ? stg[row * SLD + c0 + u] * gmm[u] : 0.f;
              s1[j] += gd;
              s2[j] += gd * xh;
            }
          }
#pragma unroll
          for (int o = 1; o < LPR; o <<= 1)
#pragma unroll
            for (int j = 0; j < NB; ++j) { s1[j] += __shfl_xor(s1[j], o); s2[j] += __shfl_xor(s2[j], o); }
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int row = (w + (i0 + j) * (NT / 64)) * RPP + sub;
            const int64_t m = r0 + row;
            if (m >= M) continue;
            const float c1 = a.norm_kind != 0 ? 0.f : s1[j] * invn, c2 = s2[j] * invn;
            float o8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const float dxn = stg[row * SLD + c0 + u];
              const float xh = (to_f(xin[j][u]) - mean[j]) * rstd[j];
              pg[u] += dxn * xh;
              pb[u] += dxn;
              o8[u] = to_f(rin[j][u]) + (a.norm_kind == 2 ? dxn : rstd[j] * (dxn * gmm[u] - c1 - xh * c2));
            }
            st8f<YT>(Y + m * a.ldy + c0, o8);
          }
        }
        // Column partials of dgamma / dbeta over this tile's rows, fixed order.
        __syncthreads();
        float* red = stg;   // [NT/64 * rpp][2][N]
        const int slot = w * rpp + sub;
#pragma unroll
        for (int u = 0; u < 8; ++u) { red[(slot * 2 + 0) * N + c0 + u] = pg[u]; red[(slot * 2 + 1) * N + c0 + u] = pb[u]; }
        __syncthreads();
        // One partial row per 64-row pass (a pass wholly past M writes none).
        const int nslots = (NT / 64) * rpp;
        if (r0 < M) {
          for (int c = tid; c < 2 * N; c += NT) {
            const int which = c / N, col = c % N;
            float sacc = 0.f;
            for (int q = 0; q < nslots; ++q) sacc += red[(q * 2 + which) * N + col];
            a.part[((int64_t)tm * NP + pass) * 2 * N + c] = sacc;
          }
        }
      } else {
        // Generic epilogue: 8-column chunks, coalesced 16-byte accesses.
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          const int c = tid + i * NT;
          if (c >= CH) continue;
          const int row = c / (OUTC / 8), col = 8 * (c % (OUTC / 8));
          const int64_t m = r0 + row;
          if (m >= M) continue;
          float v[8];
          if (EPI == EPI_GATE_SEP) {
            const int n = n0 / 2 + col;
            if (n >= Hs) continue;
            const int sc = (col / 32) * 64 + (col % 32);
            float u8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) { v[u] = stg[row * SLD + sc + u]; u8[u] = stg[row * SLD + sc + 32 + u]; }
            float g8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) g8[u] = siluf_(v[u]) * u8[u];
            st8f<YT>(Y + m * a.ldy + n, g8);
            if (Z) { st8f<T>(Z + m * a.ldz + n, v); st8f<T>(Z + m * a.ldz + Hs + n, u8); }
            continue;
          }
          const int n = n0 + col;
          if (n >= N) continue;
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = stg[row * SLD + col + u];
          float p8[8];
          if constexpr (NL > 0) {
#pragma unroll
            for (int u = 0; u < 8; ++u) p8[u] = to_f(pre[pass][i][0][u]);
          }
          if (EPI == EPI_STORE) {
            if (a.Y2 != nullptr && n >= a.nsplit) st8f<YT>((YT*)a.Y2 + m * a.ldy + (n - a.nsplit), v);
            else st8f<YT>(Y + m * a.ldy + n, v);
          } else if (EPI == EPI_RESID) {
            for (int u = 0; u < 8; ++u) p8[u] += v[u];
            st8f<YT>(Y + m * a.ldy + n, p8);
          } else if (EPI == EPI_DUAL_RESID2) {
            if (n < a.nsplit) {
              st8f<YT>(Y + m * a.ldy + n, v);
            } else {
              for (int u = 0; u < 8; ++u) p8[u] += v[u];
              st8f<YT>((YT*)a.Y2 + m * a.ldy + (n - a.nsplit), p8);
            }
          } else if (EPI == EPI_SILU_RESID) {
            for (int u = 0; u < 8; ++u) p8[u] += siluf_(v[u]);
            st8f<YT>(Y + m * a.ldy + n, p8);
            if (Z) st8f<T>(Z + m * a.ldz + n, v);
          } else if (EPI == EPI_GATE_TIED) {
            float g8[8];
            for (int u = 0; u < 8; ++u) g8[u] = siluf_(v[u]) * v[u];
            st8f<YT>(Y + m * a.ldy + n, g8);
            if (Z) st8f<T>(Z + m * a.ldz + n, v);
          } else if (EPI == EPI_DGATE_TIED) {
            for (int u = 0; u < 8; ++u) v[u] *= dsiluf_(p8[u]) * p8[u] + siluf_(p8[u]);
            st8f<YT>(Y + m * a.ldy + n, v);
          } else if (EPI == EPI_DGATE_SEP) {
            float ug[8], uu[8], o1[8], o2[8];
            ld8f<T>(Z + m * a.ldz + n, ug);
            ld8f<T>(Z + m * a.ldz + N + n, uu);
            for (int u = 0; u < 8; ++u) { o1[u] = v[u] * uu[u] * dsiluf_(ug[u]); o2[u] = v[u] * siluf_(ug[u]); }
            st8f<YT>(Y + m * a.ldy + n, o1);
            st8f<YT>(Y + m * a.ldy + N + n, o2);
          }
        }
      }
      __syncthreads();
    }
  }
}

// Resident workgroups per CU for the persistent launch (bounded by LDS and registers).
constexpr int kCUs = 256;

template <typename T, int PRO, int EPI, int BM, int BN, int BK>
hipError_t gemm_go(const GemmArgs& a, hipStream_t st) {
  const int tiles_n = (a.N + BN - 1) / BN;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t nt = tiles_m * tiles_n;
  if (nt == 0) return hipSuccess;
  if (nt > (int64_t)1 << 30) return hipErrorInvalidValue;
  constexpr int NT = (BM / 64) * (BN / 64) * 64;
  constexpr int LDT = BK + 8, SLD = BN + 4;
  constexpr int SROWS = 64;
  constexpr int lds = (2 * (BM + BN) * LDT * (int)sizeof(T) > SROWS * SLD * 4) ? 2 * (BM + BN) * LDT * (int)sizeof(T)
                                                                               : SROWS * SLD * 4;
  constexpr int per_cu_lds = 160 * 1024 / lds;
  constexpr int per_cu_thr = 2048 / NT;
  constexpr int per_cu = per_cu_lds < per_cu_thr ? (per_cu_lds < 3 ? per_cu_lds : 3) : (per_cu_thr < 3 ? per_cu_thr : 3);
  int64_t g = (int64_t)kCUs * (per_cu > 0 ? per_cu : 1);
  if (g > nt) g = nt;
  g = (g + 7) / 8 * 8;                       // every XCD gets workgroups
  if (a.y_f32)
    hipLaunchKernelGGL((gemm_nt_kernel<T, PRO, EPI, true, BM, BN, BK>), dim3((unsigned)g), dim3(NT), 0, st, a,
                       tiles_n, (int)nt);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<T, PRO, EPI, false, BM, BN, BK>), dim3((unsigned)g), dim3(NT), 0, st, a,
                       tiles_n, (int)nt);
  return hipGetLastError();
}

template <typename T, int PRO>
hipError_t gemm_epi(const GemmArgs& a, hipStream_t st) {
  switch (a.epi) {
    case EPI_STORE: return gemm_go<T, PRO, EPI_STORE, 128, sizeof(T) == 2 ? 256 : 128, 64>(a, st);
    case EPI_RESID: return gemm_go<T, PRO, EPI_RESID, 128, sizeof(T) == 2 ? 256 : 128, 64>(a, st);
    case EPI_SILU_RESID: return gemm_go<T, PRO, EPI_SILU_RESID, 128, sizeof(T) == 2 ? 256 : 128, 64>(a, st);
    case EPI_GATE_TIED: return gemm_go<T, PRO, EPI_GATE_TIED, 128, 128, 64>(a, st);
    case EPI_GATE_SEP: return gemm_go<T, PRO, EPI_GATE_SEP, 128, 128, 64>(a, st);
    case EPI_DGATE_TIED: return gemm_go<T, PRO, EPI_DGATE_TIED, 128, 128, 32>(a, st);
    case EPI_DGATE_SEP: return gemm_go<T, PRO, EPI_DGATE_SEP, 128, 128, 32>(a, st);
    case EPI_DUAL_RESID2: return gemm_go<T, PRO, EPI_DUAL_RESID2, 128, sizeof(T) == 2 ? 256 : 128, 32>(a, st);
    case EPI_NORM_BWD:
      // Row-complete tiles (BN == N); the K step shrinks with the tile so
      // that the double-buffered tiles fit in LDS.
      if (a.N != 64 && a.N != 128 && a.N != 256 && a.N != 512) return hipErrorInvalidValue;
      if (a.N <= 64) return gemm_go<T, PRO, EPI_NORM_BWD, 64, 64, 32>(a, st);
      if (a.N <= 128) return gemm_go<T, PRO, EPI_NORM_BWD, 64, 128, 32>(a, st);
      // bf16 with a plain prologue: 128-row tiles (eight waves), the epilogue
      // staged 64 rows per pass, so each weight tile serves twice the rows.
      if (a.N <= 256) {
        if constexpr (sizeof(T) == 2 && PRO == PRO_PLAIN) return gemm_go<T, PRO, EPI_NORM_BWD, 128, 256, 32>(a, st);
        return gemm_go<T, PRO, EPI_NORM_BWD, 64, 256, 32>(a, st);
      }
      return gemm_go<T, PRO, EPI_NORM_BWD, 64, 512, sizeof(T) == 2 ? 32 : 16>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t gemm_pro(const GemmArgs& a, hipStream_t st) {
  switch (a.pro) {
    case PRO_PLAIN: return gemm_epi<T, PRO_PLAIN>(a, st);
    case PRO_NORM: return gemm_epi<T, PRO_NORM>(a, st);
    case PRO_CONCAT: return gemm_epi<T, PRO_CONCAT>(a, st);
    case PRO_DACT: return gemm_epi<T, PRO_DACT>(a, st);
    case PRO_GATE:
      if (a.epi != EPI_RESID) return hipErrorInvalidValue;
      return gemm_go<T, PRO_GATE, EPI_RESID, 128, sizeof(T) == 2 ? 256 : 128, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ wgrad

constexpr int WM = 64, LDW = WM + 8;

// Output tile TW x TW (TW = 128: 4 waves of 64 x 64; TW = 256, bf16: 8 waves
// of 128 x 64, which reads every row of G and X half as often).
template <int TW> struct WgTile {
  static constexpr int NW = TW / 32;                       // waves
  static constexpr int WTN = TW == 256 ? 128 : 64, WTK = 64;   // per-wave tile
  static constexpr int NWK = TW / WTK;                      // waves along K
};

template <typename T, int PRO, int GPRO, int TW>
__global__ __launch_bounds__(TW / 32 * 64) void wgrad_kernel(WgradArgs a, int tiles_k, int ntiles, int64_t chunk) {
  using Tl = WgTile<TW>;
  constexpr int WN = TW, WK = TW, NI = Tl::WTN / 32, NJ = Tl::WTK / 32;
  __shared__ __attribute__((aligned(32))) T Gt[2][WN * LDW];   // [n][m]
  __shared__ __attribute__((aligned(32))) T Xt[2][WK * LDW];   // [k][m]
  // One logical id per (slice, tile); consecutive ids share an XCD, so the
  // tiles of one slice, which read the same rows of G and X, meet in its L2.
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int split = lid / ntiles, tl = lid % ntiles;
  const int tk = tl % tiles_k, tnn = tl / tiles_k;
  const int n0 = tnn * WN, k0 = tk * WK;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wm = w / Tl::NWK, wn = w % Tl::NWK;   // this wave's n and k sub-tile
  const int N = a.N, K = a.K;
  const int64_t mb = (int64_t)split * chunk;
  const int64_t me = min(a.M, mb + chunk);
  const T* G = (const T*)a.G;
  const T* G2 = (const T*)a.G2;
  const T* Gz = (const T*)a.Gz;
  const T* X = (const T*)a.X;
  const T* X2 = (const T*)a.X2;

  // Every thread moves half of one 8x8 block of G and half of the matching
  // block of X (4 rows of 8 columns each), so the prologue work on X (norm,
  // gate) and on G (activation derivative) is spread over all four waves.
  // Block bk: rows 8 (bk % 8) .. +8 of the m-step, columns 8 (bk / 8) .. +8 of
  // the tile; this thread takes rows 4*half .. +4 of it.
  const int bk = tid >> 1, half = tid & 1;
  const int rb = 8 * (bk & 7) + 4 * half, cb = 8 * (bk >> 3);
  // Columns past N / K read the last 8-column group (their sums are never
  // written); rows past the chunk read its last row and are zeroed when
  // stored, so every load is unmasked and all of them are in flight at once.
  const int gcol = min(n0 + cb, N - 8), xcol = min(k0 + cb, K - 8);
  const T* gsrc = (G2 != nullptr && gcol >= a.nsplit) ? G2 + (gcol - a.nsplit) : G + gcol;
  const T* gsrcz = GPRO == 1 ? Gz + gcol : gsrc;   // activation input for the G prologue
  const T* xsrc;                                   // column base of this thread's 8 X columns
  const T* xsrcz = nullptr;                        // second operand of the X prologue
  int xld = a.ldx;
  if (PRO == WPRO_CONCAT && xcol >= a.ksplit) { xsrc = X2 + (xcol - a.ksplit); xld = a.ldx2; }
  else {
    xsrc = X + xcol;
    if (PRO == WPRO_GATE_SEP) xsrcz = X + a.gate_H + xcol;
  }
  float gm[8], bt[8];
  if (PRO == WPRO_NORM) {
#pragma unroll
    for (int u = 0; u < 8; ++u) { gm[u] = a.gamma[xcol + u]; bt[u] = a.norm_kind == 0 ? a.beta[xcol + u] : 0.f; }
  }

  // Raw loads of one m-step into a register stage; the prologues run when
  // the stage is stored.
  struct Stage {
    x8_t<T> gr[4], gz[4], xr[4], xz[4];
    float mn[4], rs[4];
    int64_t mrow0;
  };
  auto load = [&](Stage& S, int64_t mbase) {
    S.mrow0 = mbase;
    int64_t mr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mr[i] = mbase + rb + i;
    if (mbase + WM > me) {   // only a chunk's last step can run past it
#pragma unroll
      for (int i = 0; i < 4; ++i) mr[i] = min(mr[i], me - 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mr[i];
      S.gr[i] = ld8<T>(gsrc + m * a.ldg);
      if (GPRO == 1) S.gz[i] = ld8<T>(gsrcz + m * a.ldg);
      S.xr[i] = ld8<T>(xsrc + m * xld);
      if (PRO == WPRO_GATE_SEP) S.xz[i] = ld8<T>(xsrcz + m * xld);
      if (PRO == WPRO_NORM && a.norm_kind != 2) { S.mn[i] = a.stats[2 * m]; S.rs[i] = a.stats[2 * m + 1]; }
    }
  };
  // Prologues, zeros for rows past the chunk, then transposed into
  // [column][m]: 4 consecutive m of one column per write.
  auto store = [&](Stage& S, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x8_t<T> g = GPRO == 1 ? dact8<T>(S.gr[i], S.gz[i]) : S.gr[i];
      x8_t<T> x = S.xr[i];
      if (PRO == WPRO_GATE_TIED) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float uf = to_f(x[e]); x[e] = from_f<T>(siluf_(uf) * uf); }
      } else if (PRO == WPRO_GATE_SEP) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = from_f<T>(siluf_(to_f(x[e])) * to_f(S.xz[i][e]));
      } else if (PRO == WPRO_NORM && a.norm_kind != 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = from_f<T>((to_f(x[e]) - S.mn[i]) * S.rs[i] * gm[e] + bt[e]);
      }
      S.gr[i] = g;
      S.xr[i] = x;
    }
    if (S.mrow0 + WM > me) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (S.mrow0 + rb + i >= me) { S.gr[i] = zero8<T>(); S.xr[i] = zero8<T>(); }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x4_t<T> tg, tx;
#pragma unroll
      for (int i = 0; i < 4; ++i) { tg[i] = S.gr[i][e]; tx[i] = S.xr[i][e]; }
      st4<T>(&Gt[buf][(cb + e) * LDW + rb], tg);
      st4<T>(&Xt[buf][(cb + e) * LDW + rb], tx);
    }
  };

  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) acc[i][jj] = zero16();

  const int64_t nsteps = me > mb ? (me - mb + WM - 1) / WM : 0;
  // MFMAs of one step on LDS buffer buf, with the loads of step `next` into
  // stage L issued between them (the last steps reload the last step).
  auto step = [&](int buf, Stage& L, int64_t next) {
    __builtin_amdgcn_s_setprio(1);
    load(L, mb + min(next, nsteps - 1) * WM);
#pragma unroll
    for (int ks = 0; ks < WM / 16; ++ks) {
      x8_t<T> af[NI], bf[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        af[i] = ld8<T>(&Gt[buf][(wm * Tl::WTN + 32 * i + l32) * LDW + 16 * ks + 8 * hh]);
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
        bf[jj] = ld8<T>(&Xt[buf][(wn * Tl::WTK + 32 * jj + l32) * LDW + 16 * ks + 8 * hh]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) mma32(acc[i][jj], af[i], bf[jj]);
    }
    if constexpr (sizeof(T) == 2) {
      constexpr int NV = 4 * (2 + (GPRO == 1) + (PRO == WPRO_GATE_SEP));
      constexpr int NMQ = NI * NJ;
#pragma unroll
      for (int ks = 0; ks < WM / 16; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x0100, NI + NJ, 0);
#pragma unroll
        for (int mq = 0; mq < NMQ; ++mq) {
          __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
          if (NMQ * ks + mq < NV) __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Two register stages: step s + 2 is loaded while step s is multiplied and
  // step s + 1 stored.  Whole pairs of steps run as one straight block (the
  // last pair's second store writes a buffer that is not read again), then
  // an odd last step.
  Stage S0, S1;
  if (nsteps > 0) {
    load(S0, mb);
    store(S0, 0);
    load(S1, mb + min((int64_t)1, nsteps - 1) * WM);
  }
  __syncthreads();
  int64_t s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(0, S0, s + 2);
    store(S1, 1);
    __syncthreads();
    step(1, S1, s + 3);
    store(S0, 0);
    __syncthreads();
  }
  if (s < nsteps) step(0, S0, s + 2);

  // A dual output (dW | dW2) always goes through the partial buffer; the
  // reduction pass splits the rows.
  float* out = (a.splits > 1 || a.dW2 != nullptr) ? a.partial + (int64_t)split * N * K : a.dW;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = n0 + wm * Tl::WTN + 32 * i + acc_row(r, hh);
        const int k = k0 + wn * Tl::WTK + 32 * jj + l32;
        if (n < N && k < K) out[(int64_t)n * K + k] = acc[i][jj][r];
      }
}

__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                           float* __restrict__ out, float* __restrict__ out2,
                                                           int64_t nsplit_elems) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // Eight partial sums (slice k goes to sum k % 8), eight loads in flight,
  // combined in a fixed tree: deterministic.
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  int k = 0;
  for (; k + 8 <= splits; k += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(k + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += v[u];
  }
  for (; k < splits; ++k) acc[k & 7] += part[(int64_t)k * n + i];
  const float s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  if (out2 != nullptr && i >= nsplit_elems) out2[i - nsplit_elems] = s;
  else out[i] = s;
}

// The 256-wide tile needs N, K >= 256 (and bf16, for its LDS).
bool wgrad_big_tile(int N, int K) { return N >= 256 && K >= 256; }

// Prologues with extra operands (activation input, norm statistics, separate
// gate) keep the 128-wide tile: the 256-wide one would spill.
template <typename T, int PRO, int GPRO>
constexpr bool wgrad_big_ok() { return sizeof(T) == 2 && GPRO == 0 && PRO != WPRO_NORM && PRO != WPRO_GATE_SEP; }

template <typename T, int PRO, int GPRO>
void wgrad_launch(const WgradArgs& a, dim3 grid, int tiles_k, int nt, int64_t chunk, bool big, hipStream_t st) {
  if constexpr (wgrad_big_ok<T, PRO, GPRO>()) {
    if (big) {
      hipLaunchKernelGGL((wgrad_kernel<T, PRO, GPRO, 256>), grid, dim3(512), 0, st, a, tiles_k, nt, chunk);
      return;
    }
  }
  hipLaunchKernelGGL((wgrad_kernel<T, PRO, GPRO, 128>), grid, dim3(256), 0, st, a, tiles_k, nt, chunk);
}

template <typename T>
hipError_t wgrad_t(const WgradArgs& a, hipStream_t st) {
  const bool gz = a.Gz != nullptr;
  const bool big = sizeof(T) == 2 && wgrad_big_tile(a.N, a.K) && !gz && a.pro != WPRO_NORM && a.pro != WPRO_GATE_SEP;
  const int TWv = big ? 256 : 128;
  const int tiles_k = (a.K + TWv - 1) / TWv, tiles_n = (a.N + TWv - 1) / TWv;
  const int nt = tiles_k * tiles_n;
  int64_t chunk = (a.M + a.splits - 1) / a.splits;
  chunk = (chunk + WM - 1) / WM * WM;
  dim3 grid((unsigned)(nt * a.splits));
  switch (a.pro) {
    case WPRO_PLAIN: gz ? wgrad_launch<T, WPRO_PLAIN, 1>(a, grid, tiles_k, nt, chunk, big, st)
                        : wgrad_launch<T, WPRO_PLAIN, 0>(a, grid, tiles_k, nt, chunk, big, st); break;
    case WPRO_NORM: wgrad_launch<T, WPRO_NORM, 0>(a, grid, tiles_k, nt, chunk, big, st); break;
    case WPRO_CONCAT: gz ? wgrad_launch<T, WPRO_CONCAT, 1>(a, grid, tiles_k, nt, chunk, big, st)
                         : wgrad_launch<T, WPRO_CONCAT, 0>(a, grid, tiles_k, nt, chunk, big, st); break;
    case WPRO_GATE_TIED: wgrad_launch<T, WPRO_GATE_TIED, 0>(a, grid, tiles_k, nt, chunk, big, st); break;
    case WPRO_GATE_SEP: wgrad_launch<T, WPRO_GATE_SEP, 0>(a, grid, tiles_k, nt, chunk, big, st); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)a.N * a.K;
  if (a.splits == 1 && a.dW2 == nullptr) return hipSuccess;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.partial, a.splits, n,
                     a.dW, a.dW2, (int64_t)a.nsplit * a.K);
  return hipGetLastError();
}

// ------------------------------------------------------------------ misc

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int rows, int cols, T* __restrict__ dst,
                                                        int ldd, int col0) {
  __shared__ T tile[32][33];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int yy = ty; yy < 32; yy += 8) {
    const int r = by + yy, c = bx + tx;
    if (r < rows && c < cols) tile[yy][tx] = src[(int64_t)r * cols + c];
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int c = bx + yy, r = by + tx;
    if (r < rows && c < cols) dst[(int64_t)c * ldd + col0 + r] = tile[tx][yy];
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

}  // namespace

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, n);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const GemmArgs& a, bool bf16_data, hipStream_t st) {
  if (a.K % 64 != 0) return hipErrorInvalidValue;
  return bf16_data ? gemm_pro<bf16>(a, st) : gemm_pro<float>(a, st);
}

int wgrad_splits(int64_t M, int N, int K) {
  // About 256 workgroups of the 256-wide tile (one per CU), else 1024 of the
  // 128-wide one.  (fp32 runs the 128-wide tile with the same count.)
  const bool big = wgrad_big_tile(N, K);
  const int TWv = big ? 256 : 128;
  const int tiles = ((N + TWv - 1) / TWv) * ((K + TWv - 1) / TWv);
  const int target = big ? 256 : 1024;
  int64_t s = (target + tiles - 1) / tiles;
  const int64_t maxs = (M + 511) / 512;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_wgrad(const WgradArgs& a, bool bf16_data, hipStream_t st) {
  if (a.N < 8 || a.K < 8 || a.N % 8 != 0 || a.K % 8 != 0) return hipErrorInvalidValue;   // whole 8-column groups
  return bf16_data ? wgrad_t<bf16>(a, st) : wgrad_t<float>(a, st);
}

hipError_t launch_transpose(const void* src, int rows, int cols, void* dst, int ldd, int col0, bool bf16_data,
                            hipStream_t st) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  if (bf16_data)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)src, rows, cols, (bf16*)dst, ldd, col0);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, st, (const float*)src, rows, cols, (float*)dst, ldd, col0);
  return hipGetLastError();
}
