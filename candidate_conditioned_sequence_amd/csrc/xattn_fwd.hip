// Jagged softmax cross-attention, forward (Eq. (4) of the WHALE paper as
// described by the pith.science verdict record, pith_extraction.key_machinery,
// and the paper-daily.com deep reading, §2): every query token of every
// candidate of request b attends over request b's whole history, K/V shared
// by all C candidates (M-FALCON, Footnote 1 in the pith.science referee
// report).
//
// Design (gfx950):
//  * One workgroup = 4 waves = one (request b, head j, block of 4*QPW
//    queries).  Its K/V tiles of BN = 64 history rows are staged in LDS once
//    and read by all of its queries; the query blocks of one (b, j) are
//    adjacent logical ids placed on one XCD, so they stream the same K/V
//    through that XCD's L2 at about the same time.
//  * Each wave owns QPW queries.  It computes S^T = K Q^T with 32x32x16 MFMA
//    (A = K rows from LDS, B = its Q fragments held in registers for the
//    whole history).  In the S^T accumulator layout a lane holds one query
//    column and 16 history rows, so the softmax max/sum reduce inside the
//    lane plus one exchange between the two lane halves, and the
//    probabilities P^T are already laid out as the B operand of the next
//    product O^T += V^T P^T: no data movement between the two products.
//    V stays row-major in LDS; the A operand of that product (V^T rows, 8
//    history rows per lane) comes from two transposing LDS reads.
//  * Online softmax in base 2 with the scale folded in.  Lazy rescaling:
//    the running reference max is only moved when a tile's max exceeds it by
//    more than kTau (probabilities then stay below 2^kTau, harmless in fp32
//    accumulation and bf16 operands); the result O / l is independent of the
//    reference, and lse = ref + log2(l) is exact.
//  * The ragged tail is masked (scores of rows past L_b set to -inf): no
//    padding of the history, and nothing past it is read.
#include "common.h"
#include "kernels.h"

namespace {

// exp2 argument s*c - ref.  The fp32 path rounds s*c first so that the row
// holding the maximum gets exactly exp2(0) = 1 (a single-row history then
// returns its value row bit for bit); bf16 rounds that difference away, so
// the bf16 path uses one fused multiply-add.
template <typename T>
WHALE_DEV float scaled_arg(float s, float c, float ref) {
  if constexpr (sizeof(T) == 4) {
#pragma clang fp contract(off)
    const float sc = s * c;     // rounded on its own: no fused multiply-add here
    return sc - ref;
  } else {
    return fmaf(s, c, -ref);
  }
}

constexpr int kBN = 64;           // history rows per tile
constexpr float kTau = 8.0f;      // lazy-rescale threshold (log2 units)

template <typename T, int DH, int kNW>
struct FwdTile {
  static constexpr int KLD = DH + 8;          // K and V tile row stride (elements)
  static constexpr int CPR = DH / 8;          // 8-element chunks per row
  static constexpr int NCH = kBN * CPR / (kNW * 64);   // chunks per thread per tensor
  static_assert(NCH >= 1 && kBN * CPR % (kNW * 64) == 0, "tile/threads mismatch");
};

// kNW waves per workgroup, QPW queries per wave.
//
// Scores live in the log2 domain relative to a per-column reference ref:
// t = c*s - ref with c = scale * log2(e), p = exp2(t).  For bf16 the factor
// c is folded into the Q fragments once (Q*c rounded to bf16: a relative
// error near 2^-9, below that of the bf16 probabilities) and -ref is the
// accumulator input of the score MFMA, so the common path spends no VALU
// instruction between the MFMA output and the exponential.  fp32 keeps Q
// exact and forms t with a separate multiply and subtract.
// d_h = 128 keeps one workgroup per CU (its operands and accumulators need
// more than the 256 registers two workgroups would leave each wave).
template <typename T, int DH, int QPW, int kNW>
__global__ __launch_bounds__(kNW * 64, DH >= 128 ? 1 : 2) void xattn_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int64_t* __restrict__ offsets, T* __restrict__ A, float* __restrict__ lse,
    int d, int h, int QR, int nqb, float c, int nblocks, const int64_t* __restrict__ coffs, int n_q,
    const int32_t* __restrict__ guard) {
  if (guard != nullptr && *guard != 0) return;   // debug mode: offsets failed validation (uniform)
  using TT = FwdTile<T, DH, kNW>;
  constexpr int NQ = QPW / 32, KS = DH / 16, NE = DH / 32, QB = kNW * QPW;
  constexpr int KBR = DH >= 128 ? 1 : 2;       // key blocks whose K operands are read at once
  constexpr int KLD = TT::KLD, CPR = TT::CPR, NCH = TT::NCH;
  constexpr bool kFold = sizeof(T) == 2;
  __shared__ __attribute__((aligned(32))) T Ks[2][kBN * KLD];
  __shared__ __attribute__((aligned(32))) T Vs[2][kBN * KLD];

  const int lid = pair_xcd_order(blockIdx.x, nqb, nblocks / nqb);
  const int qbi = lid % nqb;
  const int bj = lid / nqb;
  const int j = bj % h, b = bj / h;
  const int64_t lo = offsets[b];
  const int L = (int)(offsets[b + 1] - lo);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  // Query rows of request b: C*n_q of them, or n_q per candidate from the
  // candidate offsets when requests carry different numbers of candidates.
  const int64_t c0 = coffs ? coffs[b] : 0;
  const int64_t qrow0 = coffs ? c0 * n_q : (int64_t)b * QR;
  const int QRb = coffs ? (int)((coffs[b + 1] - c0) * n_q) : QR;
  if (qbi * QB >= QRb) return;                 // the whole block is past them (uniform)
  const int qbase = qbi * QB + w * QPW;

  // Q fragments: B operand of S^T = K Q^T, lane = query column.
  x8_t<T> qf[NQ][KS];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const int q = qbase + 32 * qb + l32;
    const T* src = Q + (qrow0 + q) * d + j * DH + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks] = (q < QRb) ? ld8<T>(src + 16 * ks) : zero8<T>();
      if (kFold) {
#pragma unroll
        for (int u = 0; u < 8; ++u) qf[qb][ks][u] = from_f<T>(to_f(qf[qb][ks][u]) * c);
      }
    }
  }

  f32x16 oacc[NE][NQ], bias[NQ];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    bias[qb] = zero16();
#pragma unroll
    for (int e = 0; e < NE; ++e) oacc[e][qb] = zero16();
  }
  // Row sums in four partial chains per query block; chain v takes the v-th
  // pair of every 8-value group, in the same order as the ping-pong kernel,
  // so the two kernels give the same bits.
  float mref[NQ], lsum[NQ][4];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) { mref[qb] = 0.f; for (int v = 0; v < 4; ++v) lsum[qb][v] = 0.f; }

  const int ntiles = (L + kBN - 1) / kBN;
  const T* Kh = K + lo * d + j * DH;
  const T* Vh = V + lo * d + j * DH;

  // Rows past the history are loaded as copies of its last row (unmasked
  // loads: no EXEC writes between MFMAs): their scores are set to -inf, so
  // their probabilities are exactly 0 and they add nothing.
  x8_t<T> kr[NCH], vr[NCH];
  auto load_tile = [&](int t) {
    const int nvalid = min(kBN, L - t * kBN);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + i * kNW * 64;
      const int row = min(ch / CPR, nvalid - 1), e0 = 8 * (ch % CPR);
      const int64_t off = (int64_t)(t * kBN + row) * d + e0;
      kr[i] = ld8<T>(Kh + off);
      vr[i] = ld8<T>(Vh + off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + i * kNW * 64;
      const int row = ch / CPR, e0 = 8 * (ch % CPR);
      st8<T>(&Ks[buf][row * KLD + e0], kr[i]);
      st8<T>(&Vs[buf][row * KLD + e0], vr[i]);
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int nvalid = min(kBN, L - t * kBN);

    // Scores of two 32-row key blocks, accumulated onto -ref (bf16) or 0.
    // All K operands are read first (one LDS wait), then the 16 MFMAs are
    // issued at raised wave priority, so the other wave's softmax fills in.
    // (d_h = 128 reads and multiplies one key block at a time, which halves
    // the live K operands.)
    __builtin_amdgcn_s_setprio(1);
    f32x16 s[2][NQ];
#pragma unroll
    for (int kb0 = 0; kb0 < 2; kb0 += KBR) {
      x8_t<T> ka[KBR][KS];
#pragma unroll
      for (int i = 0; i < KBR; ++i)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[i][ks] = ld8<T>(&Ks[buf][(32 * (kb0 + i) + l32) * KLD + 16 * ks + 8 * hh]);
#pragma unroll
      for (int i = 0; i < KBR; ++i) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int qb = 0; qb < NQ; ++qb) {
            if (ks == 0) s[kb0 + i][qb] = bias[qb];
            mma32(s[kb0 + i][qb], ka[i][ks], qf[qb][ks]);
          }
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x0100, KBR * KS, 0);
      __builtin_amdgcn_sched_group_barrier(0x0008, KBR * KS * NQ, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (!kFold) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] = scaled_arg<T>(s[kb][qb][r], c, mref[qb]);
    }
    if (nvalid < kBN) {
      // row 32 kb + acc_row(r, hh) >= nvalid, as 4 hh against a uniform
      // bound; h4 is opaque, so the 32 row indices are not hoisted out of
      // the loop into registers of their own
      int h4 = 4 * hh;
      __asm__ volatile("" : "+v"(h4));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (h4 >= nvalid - (32 * kb + acc_row(r, 0))) s[kb][qb][r] = -INFINITY;
    }

    // Tile max of t per query column (both lane halves).  The first tile
    // always sets the reference; later ones move it only by more than kTau.
    float tmax[NQ];
    bool need = t == 0;
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      tmax[qb] = half_max(mx);
      need |= tmax[qb] > kTau;
    }
    if (__ballot(need)) {
      // Move the reference by the tile max: shift this tile's t, rescale O
      // and the sums (alpha = 0 on the first tile, where both are zero).
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) {
        const float sh = (t == 0 || tmax[qb] > kTau) ? tmax[qb] : 0.f;
        const float alpha = t == 0 ? 0.f : fast_exp2(-sh);
        mref[qb] += sh;
#pragma unroll
        for (int v = 0; v < 4; ++v) lsum[qb][v] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] -= sh;
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[e][qb][r] *= alpha;
        if (kFold) {
#pragma unroll
          for (int r = 0; r < 16; ++r) bias[qb][r] = -mref[qb];
        }
      }
    }

    // P^T = exp2(t), packed pairwise into the B operands; per-lane-half row
    // sums of the fp32 values with plain adds (a v_dot2 on the packed pairs
    // would share the matrix core with the other wave's MFMAs).
    x8_t<T> pf[2][NQ][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          if constexpr (sizeof(T) == 2) {
            u32x4 words;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int r = 8 * mm + 2 * v;
              f32x2 pp = {fast_exp2(s[kb][qb][r]), fast_exp2(s[kb][qb][r + 1])};
              const bf16x2 pk = __builtin_convertvector(pp, bf16x2);
              lsum[qb][v] += pp[0];
              lsum[qb][v] += pp[1];
              words[v] = __builtin_bit_cast(unsigned, pk);
            }
            pf[kb][qb][mm] = __builtin_bit_cast(bf16x8, words);
          } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const float p = fast_exp2(s[kb][qb][8 * mm + u]);
              lsum[qb][u >> 1] += p;
              pf[kb][qb][mm][u] = from_f<T>(p);
            }
          }
        }

    // O^T[e][q] += V^T[e][key] P^T[key][q].  Operand element u of lane half
    // hh is history row 4*hh + u (u < 4) or 8 + 4*hh + (u - 4) of the
    // 16-row step, matching the accumulator rows of P^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const x8_t<T> a = lds_colA<T>(&Vs[buf][0], KLD, 32 * kb + 16 * mm, 32 * e, lane);
#pragma unroll
          for (int qb = 0; qb < NQ; ++qb) mma32(oacc[e][qb], a, pf[kb][qb][mm]);
        }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: combine the two lane halves' sums, normalise, store A and lse.
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const int q = qbase + 32 * qb + l32;
    const float ltot = half_sum((lsum[qb][0] + lsum[qb][1]) + (lsum[qb][2] + lsum[qb][3]));
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (q < QRb) {
      T* dst = A + (qrow0 + q) * d + j * DH + 4 * hh;
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          x4_t<T> o;
#pragma unroll
          for (int u = 0; u < 4; ++u) o[u] = from_f<T>(oacc[e][qb][4 * g + u] * inv);
          st4<T>(dst + 32 * e + 8 * g, o);
        }
      if (lse != nullptr && hh == 0)
        lse[(qrow0 + q) * h + j] = ltot > 0.f ? (mref[qb] + log2f(ltot)) * kLn2 : -INFINITY;
    }
  }
}

// ------------------------------------------------------------ ping-pong
// bf16 kernel for many queries per request.  A workgroup of 8 waves serves
// 512 queries of one (request, head): waves 0-3 form group A and 4-7 group B,
// so every SIMD holds one wave of each.  Every wave runs the same loop:
//   MFMA(u): scores of tile u and the PV product of tile u-1 (32 MFMAs and the
//            LDS reads feeding them), barrier,
//   VALU(u): tile traffic, max, rare rescale, exponentials, packing and row
//            sums of tile u, barrier,
// and group B starts one barrier late (A ends one barrier later), so between
// two barriers one wave of each SIMD feeds the matrix core while the other
// does the softmax.  Row sums use plain fp32 adds: a packed bf16 dot
// instruction would occupy the matrix core the other wave is using.
//
// Tiles of 64 history rows rotate through 3 LDS buffers.  In its VALU(v)
// phase group A stores K of tile v+1 and starts loading K of tile v+2; group
// B does the same for V (its VALU(v) is one phase later, and V of a tile is
// first read one tile later than K).  Each buffer is reused only after both
// groups' last read of it, with barriers in between.  The phase barrier waits
// only for this wave's LDS traffic (lgkmcnt), so the global loads stay in
// flight across it.
constexpr int kNBUF = 3;               // LDS tiles resident at once
constexpr int kPPQ = 64;              // queries per wave
constexpr int kPPW = 8;               // waves per workgroup
constexpr int kPPQB = kPPQ * kPPW;    // queries per workgroup

WHALE_DEV void phase_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0); vmcnt and expcnt untouched
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <int DH>
__global__ __launch_bounds__(kPPW * 64, 1) void xattn_fwd_pp_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const int64_t* __restrict__ offsets, bf16* __restrict__ A, float* __restrict__ lse,
    int d, int h, int QR, int nqb, float c, int nblocks, const int64_t* __restrict__ coffs, int n_q,
    const int32_t* __restrict__ guard, int rank) {
  if (guard != nullptr && *guard != 0) return;   // debug mode: offsets failed validation (uniform)
  constexpr int NQ = kPPQ / 32, KS = DH / 16, NE = DH / 32;
  constexpr int KLD = DH + 8, CPR = DH / 8;
  constexpr int NCH = kBN * CPR / (4 * 64);      // chunks per thread of one tensor (4 waves per tensor)
  static_assert(NCH >= 1 && kBN * CPR % (4 * 64) == 0, "tile/threads mismatch");
  // V rows are 192 bytes apart: the four rows that 32 lanes of a transposing
  // read touch then fall in four different 16-bank groups.
  constexpr int VLD = DH + 32;
  constexpr uint32_t kBufBytes = kBN * KLD * 2, kVBufBytes = kBN * VLD * 2;
  __shared__ __attribute__((aligned(32))) bf16 Ks[kNBUF][kBN * KLD];
  __shared__ __attribute__((aligned(32))) bf16 Vs[kNBUF][kBN * VLD];

  __shared__ __attribute__((aligned(16))) int rk_len[kRankMaxB], rk_perm[kRankMaxB];
  const int lid = pair_xcd_order(blockIdx.x, nqb, nblocks / nqb);
  const int qbi = lid % nqb;
  const int bj = lid / nqb;
  const int j = bj % h, nreq = nblocks / nqb / h;
  int b = bj / h;
  if (rank != 0 && nreq <= kRankMaxB) {   // uniform: longest history first
    rank_requests(offsets, nreq, rk_len, rk_perm);
    b = rk_perm[b];
  }
  const int64_t lo = offsets[b];
  const int L = (int)(offsets[b + 1] - lo);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv >> 2;                                // 0 = A, 1 = B
  const int gtid = tid & 255;                             // thread index within the group
  // Query rows of request b (see xattn_fwd_kernel).
  const int64_t c0 = coffs ? coffs[b] : 0;
  const int64_t qrow0 = coffs ? c0 * n_q : (int64_t)b * QR;
  const int QRb = coffs ? (int)((coffs[b + 1] - c0) * n_q) : QR;
  if (qbi * kPPQB >= QRb) return;              // the whole block is past them (uniform)
  const int qbase = qbi * kPPQB + wv * kPPQ;

  bf16x8 qf[NQ][KS];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const int q = qbase + 32 * qb + l32;
    const bf16* src = Q + (qrow0 + q) * d + j * DH + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks] = (q < QRb) ? ld8<bf16>(src + 16 * ks) : zero8<bf16>();
#pragma unroll
      for (int u = 0; u < 8; ++u) qf[qb][ks][u] = (bf16)((float)qf[qb][ks][u] * c);
    }
  }

  f32x16 oacc[NE][NQ], s[2][NQ];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
    for (int e = 0; e < NE; ++e) oacc[e][qb] = zero16();
  // Row sums in four partial chains per query block (summed after the loop).
  float mref[NQ], lsum[NQ][4];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) { mref[qb] = 0.f; for (int v = 0; v < 4; ++v) lsum[qb][v] = 0.f; }
  bf16x8 pf[2][NQ][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) { pf[kb][qb][0] = zero8<bf16>(); pf[kb][qb][1] = zero8<bf16>(); }

  const int ntiles = (L + kBN - 1) / kBN;
  // LDS byte addresses: per-lane part + uniform buffer offset + constants.
  const uint32_t kbase = lds_addr(&Ks[0][0]) + 2 * (l32 * KLD + 8 * hh);
  const uint32_t vbase = lds_addr(&Vs[0][0]) + 2 * lds_colA_lane<bf16>(VLD, lane);

  // Group A moves K tiles, group B V tiles.  Rows past the history are copies
  // of its last row (unmasked loads); their scores are set to -inf.
  const bf16* Gsrc = (grp == 0 ? K : V) + lo * d + j * DH;
  bf16* Gdst = grp == 0 ? &Ks[0][0] : &Vs[0][0];
  const int gld = grp == 0 ? KLD : VLD;
  // Two register stages: tile t is staged in xr[t & 1].  It is loaded by this
  // group's MFMA step t-2, between its score MFMAs (loads issued there cost
  // the matrix cores less than a burst of loads at the start of a VALU
  // step), and written to LDS by VALU step t-1.
  bf16x8 xr[2][NCH];
  auto load_tile = [&](int t, bf16x8 (&xs)[NCH]) {
    const int last = L - 1 - t * kBN;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = gtid + i * 256;
      const int row = min(ch / CPR, last), e0 = 8 * (ch % CPR);
      xs[i] = ld8<bf16>(Gsrc + (int64_t)(t * kBN + row) * d + e0);
    }
  };
  auto store_tile = [&](int buf, const bf16x8 (&xs)[NCH]) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = gtid + i * 256;
      const int row = ch / CPR, e0 = 8 * (ch % CPR);
      st8<bf16>(Gdst + buf * (kBN * gld) + row * gld + e0, xs[i]);
    }
  };

  // MFMA step u: scores of tile u onto -ref, and O += V P of tile u-1.  For
  // u = ntiles the scores read a resident buffer and are never used; for
  // u = 0 the product is skipped.
  auto mfma_step = [&](int u, bf16x8 (&xl)[NCH]) {
    __builtin_amdgcn_s_setprio(1);
    // This group's share of tile u+2 goes out between the score MFMAs (the
    // last two steps reload the last tile, which is never stored).
    load_tile(min(u + 2, ntiles - 1), xl);
    // (the buffer bases are opaque to the compiler, so every read below uses
    // one base register and an immediate offset)
    uint32_t kaddr = kbase + (uint32_t)(u % kNBUF) * kBufBytes;
    __asm__("" : "+v"(kaddr));
    // Four independent score chains (kb, qb) interleaved: each accumulator
    // recurs every fourth MFMA.
    bf16x8 ka[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[kb][ks] = lds_ld8(kaddr + 2 * (32 * kb * KLD + 16 * ks));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = -mref[qb];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) mma32(s[kb][qb], ka[kb][ks], qf[qb][ks]);
    __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 8, 0);
    if (u >= 1) {
      uint32_t vaddr = vbase + (uint32_t)((u + kNBUF - 1) % kNBUF) * kVBufBytes;
      __asm__("" : "+v"(vaddr));
      // Four independent output chains (e, qb) interleaved.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          bf16x8 a[NE];
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const uint32_t o = vaddr + 2 * ((32 * kb + 16 * mm) * VLD + 32 * e);
            a[e] = cat44<bf16>(lds_tr4_at(o), lds_tr4_at(o + 2 * 8 * VLD));
          }
#pragma unroll
          for (int e = 0; e < NE; ++e)
#pragma unroll
            for (int qb = 0; qb < NQ; ++qb) mma32(oacc[e][qb], a[e], pf[kb][qb][mm]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // VALU step u: tile u+1 into LDS, then the softmax of tile u's scores into
  // pf (row sums into lsum).
  auto valu_step = [&](int u, bf16x8 (&xs)[NCH]) {
    if (u + 1 < ntiles) store_tile((u + 1) % kNBUF, xs);
    const int nvalid = min(kBN, L - u * kBN);
    if (nvalid < kBN) {
      // row 32 kb + acc_row(r, hh) >= nvalid, as 4 hh against a uniform
      // bound; h4 is opaque, so the 32 row indices are not hoisted out of
      // the loop into registers of their own
      int h4 = 4 * hh;
      __asm__ volatile("" : "+v"(h4));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (h4 >= nvalid - (32 * kb + acc_row(r, 0))) s[kb][qb][r] = -INFINITY;
    }
    // Does any score of this lane pass kTau?  A balanced three-input max
    // tree over the lane's 64 values (32 instructions), no exchange between
    // lanes.  Only then (or on the first tile) are the column maxima formed
    // and the reference moved: the same decisions as comparing every column
    // maximum with kTau.
    float lv[22];
#pragma unroll
    for (int i = 0; i < 21; ++i) {
      const int a = 3 * i;
      lv[i] = max3f(s[a >> 5][(a >> 4) & 1][a & 15], s[(a + 1) >> 5][((a + 1) >> 4) & 1][(a + 1) & 15],
                    s[(a + 2) >> 5][((a + 2) >> 4) & 1][(a + 2) & 15]);
    }
    lv[21] = s[1][1][15];
    float l2[8];
#pragma unroll
    for (int i = 0; i < 7; ++i) l2[i] = max3f(lv[3 * i], lv[3 * i + 1], lv[3 * i + 2]);
    l2[7] = lv[21];
    const float lmax = fmaxf(max3f(l2[0], l2[1], l2[2]), max3f(max3f(l2[3], l2[4], l2[5]), l2[6], l2[7]));
    if (__ballot(u == 0 || lmax > kTau)) {
      float tmax[NQ];
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) {
        // four independent max chains, then combined
        float m4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) m4[v] = s[v >> 1][qb][8 * (v & 1)];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int r = 1; r < 8; ++r) m4[v] = fmaxf(m4[v], s[v >> 1][qb][8 * (v & 1) + r]);
        tmax[qb] = half_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      }
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) {
        const float sh = (u == 0 || tmax[qb] > kTau) ? tmax[qb] : 0.f;
        const float alpha = u == 0 ? 0.f : fast_exp2(-sh);
        mref[qb] += sh;
#pragma unroll
        for (int v = 0; v < 4; ++v) lsum[qb][v] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] -= sh;
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[e][qb][r] *= alpha;
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          u32x4 words;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = 8 * mm + 2 * v;
            const f32x2 pp = {fast_exp2(s[kb][qb][r]), fast_exp2(s[kb][qb][r + 1])};
            lsum[qb][v] += pp[0];
            lsum[qb][v] += pp[1];
            words[v] = __builtin_bit_cast(unsigned, __builtin_convertvector(pp, bf16x2));
          }
          pf[kb][qb][mm] = __builtin_bit_cast(bf16x8, words);
        }
  };

  // Prologue: tile 0 of both tensors into buffer 0 (each group its tensor),
  // tile 1 of this group's tensor into registers.
  if (ntiles > 0) { load_tile(0, xr[0]); store_tile(0, xr[0]); }
  if (ntiles > 1) load_tile(1, xr[1]);

  phase_barrier();

  if (grp == 1) phase_barrier();
  if (ntiles > 0)
  for (int u = 0; u <= ntiles; u += 2) {
    mfma_step(u, xr[0]);
    phase_barrier();
    if (u < ntiles) valu_step(u, xr[1]);
    phase_barrier();
    if (u + 1 <= ntiles) {
      mfma_step(u + 1, xr[1]);
      phase_barrier();
      if (u + 1 < ntiles) valu_step(u + 1, xr[0]);
      phase_barrier();
    }
  }
  if (grp == 0) phase_barrier();

#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const int q = qbase + 32 * qb + l32;
    const float ltot = half_sum((lsum[qb][0] + lsum[qb][1]) + (lsum[qb][2] + lsum[qb][3]));
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (q < QRb) {
      bf16* dst = A + (qrow0 + q) * d + j * DH + 4 * hh;
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o;
#pragma unroll
          for (int u = 0; u < 4; ++u) o[u] = (bf16)(oacc[e][qb][4 * g + u] * inv);
          st4<bf16>(dst + 32 * e + 8 * g, o);
        }
      if (lse != nullptr && hh == 0)
        lse[(qrow0 + q) * h + j] = ltot > 0.f ? (mref[qb] + log2f(ltot)) * kLn2 : -INFINITY;
    }
  }
}

template <int DH>
hipError_t launch_fwd_pp(const XattnArgs& a, hipStream_t st) {
  const int nqb = (a.QR + kPPQB - 1) / kPPQB;
  const int64_t nblk = (int64_t)a.B * a.h * nqb;
  if (nblk == 0) return hipSuccess;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((xattn_fwd_pp_kernel<DH>), dim3((unsigned)nblk), dim3(kPPW * 64), 0, st,
                     (const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.V, a.offsets, (bf16*)a.A, a.lse,
                     a.d, a.h, a.QR, nqb, c, (int)nblk, a.cand_offsets, a.n_q, a.guard, (int)a.rank_order);
  return hipGetLastError();
}

template <typename T, int DH, int QPW, int kNW>
hipError_t launch_fwd_t(const XattnArgs& a, hipStream_t st) {
  constexpr int QB = kNW * QPW;
  const int nqb = (a.QR + QB - 1) / QB;
  const int64_t nblk = (int64_t)a.B * a.h * nqb;
  if (nblk == 0) return hipSuccess;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((xattn_fwd_kernel<T, DH, QPW, kNW>), dim3((unsigned)nblk), dim3(kNW * 64), 0, st,
                     (const T*)a.Q, (const T*)a.K, (const T*)a.V, a.offsets, (T*)a.A, a.lse,
                     a.d, a.h, a.QR, nqb, c, (int)nblk, a.cand_offsets, a.n_q, a.guard);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fwd_dh(const XattnArgs& a, hipStream_t st) {
  const bool wide = a.QR >= 1024;
  if constexpr (sizeof(T) == 2) {
    if (wide && a.dh == 64) return launch_fwd_pp<64>(a, st);
  }
  switch (a.dh) {
    case 32: return wide ? launch_fwd_t<T, 32, 64, 4>(a, st) : launch_fwd_t<T, 32, 32, 4>(a, st);
    case 64: return wide ? launch_fwd_t<T, 64, 64, 4>(a, st) : launch_fwd_t<T, 64, 32, 4>(a, st);
    case 128: return launch_fwd_t<T, 128, 32, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_xattn_fwd(const XattnArgs& a, bool bf16_data, hipStream_t st) {
  return bf16_data ? launch_fwd_dh<bf16>(a, st) : launch_fwd_dh<float>(a, st);
}
