// Jagged softmax cross-attention, backward.
//
// The pages describe the backward as split along the query dimension, with
// Q-parallel and KV-parallel schedules chosen by shape (paper-daily.com deep
// reading §2; gist.science Technical Summary §2.2, "Asymmetric Backward
// Variants"; pith.science verdict record, referee_report.summary).  Here:
//  * a Q-parallel kernel: each workgroup owns a block of queries of one
//    (request, head); it first forms D[m, j] = <dA[m, j], A[m, j]> for its
//    queries (from the dA rows it holds anyway) and writes it for the
//    KV-parallel kernel, then walks the request's history, recomputing
//    P = exp2(s*c - lse2), dP = dA V^T, dS = P (dP - D), and accumulates
//    dQ^T += K^T dS^T in registers: no reduction at all;
//  * a KV-parallel kernel: each workgroup owns 128 history rows of one
//    (request, head) and walks the request's queries (or one of S query
//    splits of them), accumulating dV^T += dA^T P and dK^T += Q^T dS in
//    registers.  dK/dV sum over every query of every candidate of the
//    request: the gradient of the K/V shared across candidates.  With S > 1
//    the fp32 partials are summed in a fixed order by a second kernel.
// Both kernels use the same register trick as the forward: the MFMA
// accumulator of the score-like product is reused directly as the B operand
// of the next product, with the A operand read column-wise from the same
// row-major LDS tile (transposing LDS reads) in the matching row order.
// Deterministic: no atomics.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kNW = 4;

// Probabilities and dS of one 32x32 score block, packed pairwise into two
// B operands (bf16: v_cvt_pk; the pair order is the accumulator row order).
template <typename T>
WHALE_DEV void p_ds_pack(const f32x16& s, const f32x16& dp, x8_t<T> (&pf)[2], x8_t<T> (&dsf)[2]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      u32x4 pw, dw;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 8 * mm + 2 * v;
        const f32x2 pp = {fast_exp2(s[r]), fast_exp2(s[r + 1])};
        const f32x2 dd = {pp[0] * dp[r], pp[1] * dp[r + 1]};
        pw[v] = __builtin_bit_cast(unsigned, __builtin_convertvector(pp, bf16x2));
        dw[v] = __builtin_bit_cast(unsigned, __builtin_convertvector(dd, bf16x2));
      }
      pf[mm] = __builtin_bit_cast(bf16x8, pw);
      dsf[mm] = __builtin_bit_cast(bf16x8, dw);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(s[r]);
      pf[r >> 3][r & 7] = p;
      dsf[r >> 3][r & 7] = p * dp[r];
    }
  }
}

// ----------------------------------------------------------------- dQ
// Scores in the log2 domain: t = c*s - lse2 with c = scale*log2(e).  For bf16
// c is folded into the Q fragments once (rounded to bf16, as in the forward)
// and -lse2 (one value per lane: this query) is the accumulator input of the
// score MFMA; -D likewise starts the dP MFMA, so P = exp2(acc) and
// dS = P * acc' need no other VALU work.  fp32 keeps Q exact and forms t with
// one fused multiply-add.
// (d_h = 128: one workgroup per CU, for the register room; likewise below.)
template <typename T, int DH, int NWQ>
__global__ __launch_bounds__(NWQ * 64, DH >= 128 ? 1 : 2) void bwd_dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int64_t* __restrict__ offsets, const T* __restrict__ dA, const T* __restrict__ A,
    const float* __restrict__ lse, float* __restrict__ Dbuf, T* __restrict__ dQ, int d, int h, int QR, int nqb,
    float c, float scale, int nblocks, const int32_t* __restrict__ guard) {
  if (guard != nullptr && *guard != 0) return;   // debug mode: offsets failed validation (uniform)
  constexpr int BN = 64, KS = DH / 16, NE = DH / 32, QB = NWQ * 32;
  constexpr int KLD = DH + 8, CPR = DH / 8, NCH = BN * CPR / (NWQ * 64);
  static_assert(NCH >= 1 && BN * CPR % (NWQ * 64) == 0, "tile/threads mismatch");
  constexpr bool kFold = sizeof(T) == 2;
  __shared__ __attribute__((aligned(32))) T Ks[2][BN * KLD];
  __shared__ __attribute__((aligned(32))) T Vs[2][BN * KLD];

  const int lid = xcd_remap(blockIdx.x, nblocks);
  const int qbi = lid % nqb;
  const int bj = lid / nqb;
  const int j = bj % h, b = bj / h;
  const int64_t lo = offsets[b];
  const int L = (int)(offsets[b + 1] - lo);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int64_t qrow0 = (int64_t)b * QR;
  const int q = qbi * QB + w * 32 + l32;
  const bool qok = q < QR;

  x8_t<T> qf[KS], gf[KS];
  // D = <dA, A> of this lane's query: each lane holds half of the row (the
  // chunks of hh), the two halves meet across l and l ^ 32.
  float dpart = 0.f;
  {
    const int64_t off = (qrow0 + q) * d + j * DH + 8 * hh;
    x8_t<T> af[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = qok ? ld8<T>(Q + off + 16 * ks) : zero8<T>();
      gf[ks] = qok ? ld8<T>(dA + off + 16 * ks) : zero8<T>();
      af[ks] = qok ? ld8<T>(A + off + 16 * ks) : zero8<T>();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int u = 0; u < 8; ++u) dpart = fmaf(to_f(af[ks][u]), to_f(gf[ks][u]), dpart);
      if (kFold) {
#pragma unroll
        for (int u = 0; u < 8; ++u) qf[ks][u] = from_f<T>(to_f(qf[ks][u]) * c);
      }
    }
  }
  const float lse2 = qok ? lse[(qrow0 + q) * h + j] * kLog2e : INFINITY;
  const float Dq = half_sum(dpart);
  if (qok && hh == 0) Dbuf[(qrow0 + q) * h + j] = Dq;

  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = zero16();

  const int ntiles = (L + BN - 1) / BN;
  const T* Kh = K + lo * d + j * DH;
  const T* Vh = V + lo * d + j * DH;
  // Rows past the history are loaded as copies of its last row (no masked
  // loads in the loop); their probabilities are set to 0 below.
  x8_t<T> kr[NCH], vr[NCH];
  auto load_tile = [&](int t) {
    const int last = L - 1 - t * BN;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + i * NWQ * 64;
      const int row = min(ch / CPR, last), e0 = 8 * (ch % CPR);
      const int64_t off = (int64_t)(t * BN + row) * d + e0;
      kr[i] = ld8<T>(Kh + off);
      vr[i] = ld8<T>(Vh + off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + i * NWQ * 64;
      const int row = ch / CPR, e0 = 8 * (ch % CPR);
      st8<T>(&Ks[buf][row * KLD + e0], kr[i]);
      st8<T>(&Vs[buf][row * KLD + e0], vr[i]);
    }
  };

  if (ntiles > 0) { load_tile(0); store_tile(0); }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    // The next tile's loads go out between the first score MFMAs; the last
    // step reloads its own tile and stores it into the idle buffer.
    const int tnext = min(t + 1, ntiles - 1);
    const int nvalid = min(BN, L - t * BN);
    x8_t<T> dsf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = kFold ? -lse2 : 0.f; dp[r] = -Dq; }
      // all operand reads of this key block first (one LDS wait), then the
      // MFMAs at raised priority
      x8_t<T> ka[KS], va[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        ka[ks] = ld8<T>(&Ks[buf][(32 * kb + l32) * KLD + 16 * ks + 8 * hh]);
        va[ks] = ld8<T>(&Vs[buf][(32 * kb + l32) * KLD + 16 * ks + 8 * hh]);
      }
      __builtin_amdgcn_s_setprio(1);
      if (kb == 0) load_tile(tnext);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        mma32(s, ka[ks], qf[ks]);
        mma32(dp, va[ks], gf[ks]);
      }
      __builtin_amdgcn_sched_group_barrier(0x0100, 2 * KS, 0);
      if (kb == 0) {
#pragma unroll
        for (int i = 0; i < 2 * NCH; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x0008, 2 * KS - 2 * NCH, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x0008, 2 * KS, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      if (!kFold) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = fmaf(s[r], c, -lse2);
      }
      if (nvalid < BN) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + acc_row(r, hh) >= nvalid) s[r] = -INFINITY;
      }
      x8_t<T> pf_unused[2];
      p_ds_pack<T>(s, dp, pf_unused, dsf[kb]);   // P itself is not needed here
    }
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
          mma32(acc[e], lds_colA<T>(&Ks[buf][0], KLD, 32 * kb + 16 * mm, 32 * e, lane), dsf[kb][mm]);
    store_tile(buf ^ 1);
    __syncthreads();
  }

  if (qok) {
    T* dst = dQ + (qrow0 + q) * d + j * DH + 4 * hh;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        x4_t<T> o;
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = from_f<T>(acc[e][4 * g + u] * scale);
        st4<T>(dst + 32 * e + 8 * g, o);
      }
  }
}

// ----------------------------------------------------------------- dK, dV
// Lanes are keys and accumulator rows are queries, so -lse2 and -D vary with
// the row: each query tile stores them negated in LDS and the 4-row groups a
// lane needs are read straight into the score / dP accumulators as their
// starting values.  bf16 folds c into the K fragments.  Query rows past the
// split are loaded as copies of its last row with -lse2 = -inf, so P = 0 and
// dS = 0 for them.
template <typename T, int DH, int NWK>
__global__ __launch_bounds__(NWK * 64, DH >= 128 ? 1 : 2) void bwd_dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int64_t* __restrict__ offsets, const T* __restrict__ dA, const float* __restrict__ lse,
    const float* __restrict__ Dbuf, T* __restrict__ dK, T* __restrict__ dV, float* __restrict__ part,
    int d, int h, int QR, int nkt, int qchunk, float c, float scale, int64_t T_rows, int nblocks,
    const int32_t* __restrict__ guard) {
  if (guard != nullptr && *guard != 0) return;   // debug mode: offsets failed validation (uniform)
  constexpr int QT = 64, KS = DH / 16, NE = DH / 32;
  constexpr int KLD = DH + 8, CPR = DH / 8, NCH = QT * CPR / (NWK * 64);
  constexpr int KB = NWK * 32;   // history rows per workgroup
  static_assert(NCH >= 1 && QT * CPR % (NWK * 64) == 0, "tile/threads mismatch");
  constexpr bool kFold = sizeof(T) == 2;
  __shared__ __attribute__((aligned(32))) T Qs[2][QT * KLD];
  __shared__ __attribute__((aligned(32))) T Gs[2][QT * KLD];
  __shared__ __attribute__((aligned(16))) float nl_s[2][QT];   // -lse2 (bf16) or lse2 (fp32)
  __shared__ __attribute__((aligned(16))) float nd_s[2][QT];   // -D

  const int split = blockIdx.y;
  const int lid = xcd_remap(blockIdx.x, nblocks);
  const int kt = lid % nkt;
  const int bj = lid / nkt;
  const int j = bj % h, b = bj / h;
  const int64_t lo = offsets[b];
  const int L = (int)(offsets[b + 1] - lo);
  if (kt * KB >= L) return;                        // workgroup-uniform
  const int q_begin = split * qchunk;
  const int q_end = min(QR, q_begin + qchunk);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);   // wave index as a scalar
  const int key = kt * KB + w * 32 + l32;
  const bool kok = key < L;
  const int64_t qrow0 = (int64_t)b * QR;

  x8_t<T> kf[KS], vf[KS];
  {
    const int64_t off = (lo + key) * d + j * DH + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = kok ? ld8<T>(K + off + 16 * ks) : zero8<T>();
      vf[ks] = kok ? ld8<T>(V + off + 16 * ks) : zero8<T>();
      if (kFold) {
#pragma unroll
        for (int u = 0; u < 8; ++u) kf[ks][u] = from_f<T>(to_f(kf[ks][u]) * c);
      }
    }
  }
  f32x16 dk[NE], dv[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) { dk[e] = zero16(); dv[e] = zero16(); }

  const int ntiles = q_end > q_begin ? (q_end - q_begin + QT - 1) / QT : 0;
  x8_t<T> qr[NCH], gr[NCH];
  float lraw = 0.f, draw = 0.f;   // raw lse and D of query lane
  int lq = 0;
  // Raw loads only: the arithmetic on the loaded values waits until the
  // values are stored, so no wait on the loads sits at the top of a step.
  auto load_tile = [&](int t) {
    const int qt0 = q_begin + t * QT;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + i * NWK * 64;
      const int row = ch / CPR, e0 = 8 * (ch % CPR);
      const int qq = min(qt0 + row, q_end - 1);
      const int64_t off = (qrow0 + qq) * d + j * DH + e0;
      qr[i] = ld8<T>(Q + off);
      gr[i] = ld8<T>(dA + off);
    }
    // lane i of every wave fetches query i's lse and D
    lq = qt0 + lane;
    const int qc = min(lq, q_end - 1);
    lraw = lse[(qrow0 + qc) * h + j];
    draw = Dbuf[(qrow0 + qc) * h + j];
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + i * NWK * 64;
      const int row = ch / CPR, e0 = 8 * (ch % CPR);
      st8<T>(&Qs[buf][row * KLD + e0], qr[i]);
      st8<T>(&Gs[buf][row * KLD + e0], gr[i]);
    }
    // Every wave writes the same 64 values (no branch for the loads to sink
    // into).
    {
      const float l2 = lraw * kLog2e;
      const bool ok = lq < q_end;
      nl_s[buf][lane] = kFold ? (ok ? -l2 : -INFINITY) : (ok ? l2 : INFINITY);
      nd_s[buf][lane] = ok ? -draw : 0.f;
    }
  };

  if (ntiles > 0) { load_tile(0); store_tile(0); }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    // The next tile's loads go out between the first score MFMAs.  The last
    // step reloads its own tile and stores it into the idle buffer, which is
    // never read again: the loads, MFMAs and stores stay one straight block.
    const int tnext = min(t + 1, ntiles - 1);
    x8_t<T> pf[2][2], dsf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s, dp, l2blk;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&nl_s[buf][32 * qb + 8 * g + 4 * hh]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&nd_s[buf][32 * qb + 8 * g + 4 * hh]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          dp[4 * g + u] = d4[u];
          if (kFold) {
            s[4 * g + u] = l4[u];
          } else {
            s[4 * g + u] = 0.f;
            l2blk[4 * g + u] = l4[u];
          }
        }
      }
      x8_t<T> qa[KS], ga[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[ks] = ld8<T>(&Qs[buf][(32 * qb + l32) * KLD + 16 * ks + 8 * hh]);
        ga[ks] = ld8<T>(&Gs[buf][(32 * qb + l32) * KLD + 16 * ks + 8 * hh]);
      }
      __builtin_amdgcn_s_setprio(1);
      if (qb == 0) load_tile(tnext);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        mma32(s, qa[ks], kf[ks]);
        mma32(dp, ga[ks], vf[ks]);
      }
      __builtin_amdgcn_sched_group_barrier(0x0100, 2 * KS, 0);
      if (qb == 0) {
#pragma unroll
        for (int i = 0; i < 2 * NCH + 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x0008, 2 * KS - (2 * NCH + 2), 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x0008, 2 * KS, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      if (!kFold) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = fmaf(s[r], c, -l2blk[r]);
      }
      p_ds_pack<T>(s, dp, pf[qb], dsf[qb]);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          mma32(dv[e], lds_colA<T>(&Gs[buf][0], KLD, 32 * qb + 16 * mm, 32 * e, lane), pf[qb][mm]);
          mma32(dk[e], lds_colA<T>(&Qs[buf][0], KLD, 32 * qb + 16 * mm, 32 * e, lane), dsf[qb][mm]);
        }
    store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!kok) return;
  // dV == nullptr: shared key-value form (V is K), one gradient dK + dV.
  const bool tied = dV == nullptr;
  if (part == nullptr) {
    T* dkp = dK + (lo + key) * d + j * DH;
    if (tied) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkp[32 * e + acc_row(r, hh)] = from_f<T>(fmaf(dk[e][r], scale, dv[e][r]));
      return;
    }
    T* dvp = dV + (lo + key) * d + j * DH;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ee = 32 * e + acc_row(r, hh);
        dkp[ee] = from_f<T>(dk[e][r] * scale);
        dvp[ee] = from_f<T>(dv[e][r]);
      }
  } else {
    float* pk = part + ((int64_t)split * 2 * T_rows + lo + key) * d + j * DH;
    if (tied) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) pk[32 * e + acc_row(r, hh)] = fmaf(dk[e][r], scale, dv[e][r]);
      return;
    }
    float* pv = pk + T_rows * d;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ee = 32 * e + acc_row(r, hh);
        pk[ee] = dk[e][r] * scale;
        pv[ee] = dv[e][r];
      }
  }
}

// Partials are [S][2][n] (dK then dV); with dV == nullptr (shared key-value
// form) only the first half of each split holds data, already dK + dV.
template <typename T>
__global__ __launch_bounds__(256) void kv_split_reduce_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                              T* __restrict__ dK, T* __restrict__ dV,
                                                              const int32_t* __restrict__ guard) {
  if (guard != nullptr && *guard != 0) return;   // debug mode: offsets failed validation (uniform)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (dV ? 2 * n : n)) return;
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += part[(int64_t)k * 2 * n + i];
  if (i < n) dK[i] = from_f<T>(s);
  else dV[i - n] = from_f<T>(s);
}

template <typename T, int DH>
hipError_t bwd_t(const XattnBwdArgs& a, hipStream_t st) {
  const float c = a.scale * kLog2e;
  hipError_t e;
  {
    // The dQ kernel also forms D = <dA, A> and writes it to Dbuf, which the
    // dK/dV kernel reads after it (same stream).
    // Eight waves (256 queries) per workgroup where the request has enough
    // queries: one K/V tile load then serves twice the queries of a CU.
    auto go = [&](auto nwq) {
      constexpr int NWQ = decltype(nwq)::value;
      const int nqb = (a.QR + NWQ * 32 - 1) / (NWQ * 32);
      const int64_t nblk = (int64_t)a.B * a.h * nqb;
      hipLaunchKernelGGL((bwd_dq_kernel<T, DH, NWQ>), dim3((unsigned)nblk), dim3(NWQ * 64), 0, st, (const T*)a.Q,
                         (const T*)a.K, (const T*)a.V, a.offsets, (const T*)a.dA, (const T*)a.A, a.lse, a.Dbuf,
                         (T*)a.dQ, a.d, a.h, a.QR, nqb, c, a.scale, (int)nblk, a.guard);
    };
    bool done = false;
    if constexpr (DH == 64) {
      if (a.QR >= 512) { go(std::integral_constant<int, 8>()); done = true; }
    }
    if (!done) go(std::integral_constant<int, kNW>());
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.T == 0 || a.max_L == 0) return hipSuccess;
  {
    int qchunk = (a.QR + a.splits - 1) / a.splits;
    qchunk = (qchunk + 63) / 64 * 64;
    float* part = a.splits > 1 ? a.partial : nullptr;
    // Eight waves (256 history rows) per workgroup when there is no query
    // split: one Q / dA tile load then serves twice the rows of a CU.
    auto go = [&](auto nwk) {
      constexpr int NWK = decltype(nwk)::value;
      const int nkt = (a.max_L + NWK * 32 - 1) / (NWK * 32);
      const int64_t nblk = (int64_t)a.B * a.h * nkt;
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, DH, NWK>), dim3((unsigned)nblk, a.splits), dim3(NWK * 64), 0, st,
                         (const T*)a.Q, (const T*)a.K, (const T*)a.V, a.offsets, (const T*)a.dA, a.lse, a.Dbuf,
                         (T*)a.dK, (T*)a.dV, part, a.d, a.h, a.QR, nkt, qchunk, c, a.scale, a.T, (int)nblk,
                         a.guard);
    };
    bool done = false;
    if constexpr (DH == 64) {
      if (a.splits == 1) { go(std::integral_constant<int, 8>()); done = true; }
    }
    if (!done) go(std::integral_constant<int, kNW>());
    e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    const int64_t n = a.T * a.d;
    const int64_t nr = a.dV ? 2 * n : n;
    hipLaunchKernelGGL(kv_split_reduce_kernel<T>, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, st, a.partial,
                       a.splits, n, (T*)a.dK, (T*)a.dV, a.guard);
    return hipGetLastError();
  }
}

template <typename T>
hipError_t bwd_dh(const XattnBwdArgs& a, hipStream_t st) {
  switch (a.dh) {
    case 32: return bwd_t<T, 32>(a, st);
    case 64: return bwd_t<T, 64>(a, st);
    case 128: return bwd_t<T, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int xattn_bwd_splits(int B, int h, int QR, int max_L, int dh) {
  (void)dh;
  const int64_t nwg = (int64_t)B * h * ((max_L + 127) / 128);
  const int maxs = (QR + 63) / 64;
  if (nwg >= 512 || nwg == 0) return 1;
  int64_t s = (512 + nwg - 1) / nwg;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_xattn_bwd(const XattnBwdArgs& a, bool bf16_data, hipStream_t st) {
  return bf16_data ? bwd_dh<bf16>(a, st) : bwd_dh<float>(a, st);
}
