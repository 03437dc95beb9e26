// HSTU jagged self-attention with relative position and time bias, forward.
//
// The pages describe the HSTU module, which produces the history states H_s
// the fusion attention reads, as sequential attention with relative
// position-and-time biases (pith.science verdict record,
// pith_extraction.key_machinery; gist.science Technical Summary §2.1), and
// leave rab(p, t) undefined (pith.science review page, referee minor comment
// on Eq. (2), pointing to the HSTU paper, reference [34]).  The reading
// computed here: per request b and head, for history rows i, j < L_b,
//   A_i = (1 / L_b) * sum_{j <= i} SiLU(scale <q_i, k_j> + rab(i, j)) v_j,
//   rab(i, j) = w_pos[min(i - j, NP - 1)] + w_time[min(floor(log2(max(dt, 1))), NT - 1)],
// dt = tau_i - tau_j, tables shared by all heads.
//
// Design (gfx950):
//  * One workgroup = 4 waves = one (request, head, block of 128 queries);
//    each wave owns 32 queries.  A block walks the key tiles (64 history
//    rows) up to its last query; K/V tiles are staged in LDS with the tile's
//    timestamps.  The work of a block grows with its index within the
//    request, and the work of a request with the square of its length, so
//    workgroups are issued level by level: every request's last query block
//    first, then every request's second-to-last, and so on (longest first).
//    Workgroups go to the XCDs round-robin, so the (request, head) order is
//    rotated by one per level: a pair lands on a different XCD at each
//    level, and no XCD collects the long requests.
//  * S^T = K Q^T with 32x32x16 MFMA (lane = query column, 16 key rows per
//    lane and 32-row block), with -log2(e) scale folded into Q and the
//    position bias as the accumulators' start, then per element: the time
//    bias by an LDS gather at the leading-bit position of the saturated time
//    difference (the time table is stored in that order, so no log and no
//    clip), one add and SiLU.  Each wave classifies each key tile once,
//    before its MFMAs: far (every pair at least NP - 1 rows apart: the
//    table's last entry, folded into a second time table), interior (every
//    i - j in [0, NP - 1]: a gather at immediate offsets from one base, no
//    mask) or edge (clamped gather and the causal mask).  The packed
//    probabilities feed O^T += V^T P^T with V read column-wise by
//    transposing LDS reads, as in the fusion attention.
//  * Timestamps are kept as 32-bit tau - tau_first + 2^30, so the time
//    difference of any pair is exact and below 2^31 when every timestamp of
//    a request differs from its first by less than 2^30 (the caller's
//    contract); a time table of at most 32 entries then covers every bucket.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kHQB = 128;       // queries per workgroup
constexpr int kHBN = 64;        // history rows per key tile
constexpr int kMaxPos = 4096;   // largest position table

// Leading-zero count of x, -1 for x == 0, in one instruction (the compiler's
// clz of a possibly-zero value adds a compare and a select).
__device__ __forceinline__ int leading_zeros_or_m1(uint32_t x) {
  int r;
  __asm__("v_ffbh_u32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

template <typename T, int DH>
__global__ __launch_bounds__(256, (DH >= 128 || sizeof(T) == 4) ? 1 : 3) void hstu_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ ts, const float* __restrict__ w_pos,
    int n_pos, const float* __restrict__ w_time, int n_time, T* __restrict__ A, int d, int h, int nqb,
    float scale, int nbh, const int32_t* __restrict__ guard) {
  if (guard != nullptr && *guard != 0) return;   // debug mode: offsets failed validation (uniform)
  constexpr int KS = DH / 16, NE = DH / 32, KLD = DH + 8, CPR = DH / 8;
  constexpr int NCH = kHBN * CPR / 256;
  constexpr int KBR = DH >= 128 ? 1 : 2;         // key blocks whose K operands are read at once
  static_assert(NCH >= 1 && kHBN * CPR % 256 == 0, "tile/threads mismatch");
  // K tiles and their timestamps are double buffered, V tiles single
  // buffered (V is read only by the last product of a tile): 44,676 bytes of
  // LDS at d_h = 64 in bf16, below the largest size of which the hardware
  // keeps three workgroups on a CU (measured between 52,000 and 53,892).
  __shared__ __attribute__((aligned(32))) T Ks[2][kHBN * KLD];
  __shared__ __attribute__((aligned(32))) T Vs[kHBN * KLD];
  __shared__ __attribute__((aligned(16))) uint32_t Ts[2][kHBN];
  // Both tables are stored times -log2(e) (see the SiLU below).
  __shared__ float Wp[kMaxPos];
  // Wt[1 + c] = w_time[min(31 - c, NT - 1)] for a time difference with c
  // leading zeros; Wt[0] (difference 0, leading-bit search -1) = w_time[0].
  // Wf is the same plus the last position entry (far tiles).
  __shared__ float Wt[33];
  __shared__ float Wf[33];

  const int level = blockIdx.x / nbh;           // nbh = B * h blocks per level
  const int qbi = nqb - 1 - level;
  const int bj = (int)((blockIdx.x % nbh + qbi) % nbh);
  const int j = bj % h, b = bj / h;
  const int64_t lo = offsets[b];
  const int L = (int)(offsets[b + 1] - lo);
  if (qbi * kHQB >= L) return;                   // workgroup-uniform
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Timestamps are kept as tau - tau_first + 2^30, positive in 31 bits under
  // the caller's contract, so an unsigned saturating difference is
  // max(tau_i - tau_j, 0) exactly.
  const int64_t t0 = ts[lo] - (int64_t{1} << 30);
  constexpr float kNegLog2e = -1.4426950408889634f;

  for (int k = tid; k < n_pos; k += 256) Wp[k] = kNegLog2e * w_pos[k];
  if (tid < 33) {
    Wt[tid] = kNegLog2e * w_time[tid == 0 ? 0 : min(32 - tid, n_time - 1)];
    Wf[tid] = Wt[tid] + kNegLog2e * w_pos[n_pos - 1];
  }

  const int qw = qbi * kHQB + w * 32;            // first query of this wave
  const int i = qw + l32;                        // this lane's query (row within the request)
  const bool iok = i < L;
  // Q fragments times sc = -log2(e) scale (for bf16 rounded once, a
  // relative error near 2^-9, as in the fusion attention): the score MFMA
  // then yields -log2(e) (scale <q, k> + position bias) directly, its
  // accumulators starting from the position bias.
  const float sc = kNegLog2e * scale;
  x8_t<T> qf[KS];
  {
    const T* src = Q + (lo + i) * d + j * DH + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = iok ? ld8<T>(src + 16 * ks) : zero8<T>();
#pragma unroll
      for (int u = 0; u < 8; ++u) qf[ks][u] = from_f<T>(to_f(qf[ks][u]) * sc);
    }
  }
  const uint32_t ti = iok ? (uint32_t)(ts[lo + i] - t0) : 0u;
  f32x16 oacc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) oacc[e] = zero16();

  const int qend = min(L, qbi * kHQB + kHQB);
  const int ntiles = (qend + kHBN - 1) / kHBN;
  const T* Kh = K + lo * d + j * DH;
  const T* Vh = V + lo * d + j * DH;
  // Rows past the history are copies of its last row; every key they stand
  // for is past every valid query, so the causal mask removes them.
  x8_t<T> kr[NCH], vr[NCH];
  uint32_t tr = 0;
  auto load_tile = [&](int t) {
    const int last = L - 1 - t * kHBN;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * 256;
      const int row = min(ch / CPR, last), e0 = 8 * (ch % CPR);
      const int64_t off = (int64_t)(t * kHBN + row) * d + e0;
      kr[c] = ld8<T>(Kh + off);
      vr[c] = ld8<T>(Vh + off);
    }
    if (tid < kHBN) tr = (uint32_t)(ts[lo + t * kHBN + min(tid, last)] - t0);
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * 256;
      const int row = ch / CPR, e0 = 8 * (ch % CPR);
      st8<T>(&Ks[buf][row * KLD + e0], kr[c]);
    }
    if (tid < kHBN) Ts[buf][tid] = tr;
  };
  auto store_v = [&]() {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * 256;
      const int row = ch / CPR, e0 = 8 * (ch % CPR);
      st8<T>(&Vs[row * KLD + e0], vr[c]);
    }
  };

  load_tile(0);
  store_k(0);
  store_v();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int j0 = t * kHBN;
    // Tile-uniform cases for this wave: far (every pair at least NP - 1 rows
    // apart: the last position entry, folded into the time table Wf; no
    // mask), interior (every i - j in [0, NP - 1]: no clamp, no mask), else
    // edge (clamp and causal mask).
    const bool far = qw - (j0 + kHBN - 1) >= n_pos - 1;
    const bool interior = !far && j0 + kHBN - 1 <= qw && qw + 31 - j0 <= n_pos - 1;
    // With y = -log2(e) x, SiLU(x) = -ln(2) y / (1 + 2^y): the factor -ln(2)
    // is applied once to the output, so each element costs an add (the time
    // bias), an exp2, an add, a reciprocal and a multiply.  Interior tiles
    // read the position table at one base address (row offsets become
    // immediates).  The mode is uniform over the tile, so one branch covers
    // all 32 elements of the lane and they can be interleaved.
    x8_t<T> pf[2][2];
    auto tile = [&](auto modec) {
      constexpr int kMode = decltype(modec)::value;   // 0 edge, 1 interior, 2 far
      f32x16 s[2];
      // position bias (times -log2(e)) as the accumulator start, row
      // j0 + 32 kb + acc_row(r, hh) of the lane's query i
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if constexpr (kMode == 2) {
          s[kb] = zero16();
        } else if constexpr (kMode == 1) {
          const float* wrow = &Wp[i - j0 - 32 * kb - 4 * hh - 27];
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = wrow[27 - 8 * (r >> 2) - (r & 3)];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = Wp[min(max(i - (j0 + 32 * kb + acc_row(r, hh)), 0), n_pos - 1)];
        }
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb0 = 0; kb0 < 2; kb0 += KBR) {
        x8_t<T> ka[KBR][KS];
#pragma unroll
        for (int u = 0; u < KBR; ++u)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            ka[u][ks] = ld8<T>(&Ks[buf][(32 * (kb0 + u) + l32) * KLD + 16 * ks + 8 * hh]);
#pragma unroll
        for (int u = 0; u < KBR; ++u)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) mma32(s[kb0 + u], ka[u][ks], qf[ks]);
      }
      __builtin_amdgcn_s_setprio(0);
      const float* wt1 = (kMode == 2 ? Wf : Wt) + 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uint32_t tj[16];   // timestamps of this lane's 16 rows (4-row groups)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint4 v4 = *reinterpret_cast<const uint4*>(&Ts[buf][32 * kb + 8 * g + 4 * hh]);
          tj[4 * g + 0] = v4.x;
          tj[4 * g + 1] = v4.y;
          tj[4 * g + 2] = v4.z;
          tj[4 * g + 3] = v4.w;
        }
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = j0 + 32 * kb + acc_row(r, hh);
          const uint32_t dt = __builtin_elementwise_sub_sat(ti, tj[r]);
          const int lz = leading_zeros_or_m1(dt);
          const float y = s[kb][r] + wt1[lz];
          const float pr = y * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(y));
          p[r] = (kMode != 0 || jj <= i) ? pr : 0.f;
        }
        // packed pairwise into the B operands, in accumulator row order
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int u = 0; u < 8; ++u) pf[kb][mm][u] = from_f<T>(p[8 * mm + u]);
      }
    };
    if (far) tile(std::integral_constant<int, 2>());
    else if (interior) tile(std::integral_constant<int, 1>());
    else tile(std::integral_constant<int, 0>());
    // V of tile t, stored after the previous tile's last barrier, is visible
    // to every wave from here on.
    __syncthreads();
    // O^T[e][q] += V^T[e][key] P^T[key][q]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
          mma32(oacc[e], lds_colA<T>(&Vs[0], KLD, 32 * kb + 16 * mm, 32 * e, lane), pf[kb][mm]);
    if (t + 1 < ntiles) store_k(buf ^ 1);
    // Every wave is done with V of tile t (and K of tile t + 1 is visible).
    __syncthreads();
    if (t + 1 < ntiles) store_v();
  }

  if (iok) {
    const float inv = -0.6931471805599453f / (float)L;   // -ln(2) / L_b
    T* dst = A + (lo + i) * d + j * DH + 4 * hh;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        x4_t<T> o;
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = from_f<T>(oacc[e][4 * g + u] * inv);
        st4<T>(dst + 32 * e + 8 * g, o);
      }
  }
}

template <typename T, int DH>
hipError_t launch_hstu_t(const HstuArgs& a, hipStream_t st) {
  const int nqb = (a.max_L + kHQB - 1) / kHQB;
  const int64_t nblk = (int64_t)a.B * a.h * nqb;
  if (nblk == 0) return hipSuccess;
  if (nblk * 256 >= (int64_t{1} << 32)) return hipErrorInvalidValue;   // work-item count of one launch
  hipLaunchKernelGGL((hstu_fwd_kernel<T, DH>), dim3((unsigned)nblk), dim3(256), 0, st, (const T*)a.Q,
                     (const T*)a.K, (const T*)a.V, a.offsets, a.timestamps, a.w_pos, a.n_pos, a.w_time, a.n_time,
                     (T*)a.A, a.d, a.h, nqb, a.scale, a.B * a.h, a.guard);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_hstu_dh(const HstuArgs& a, hipStream_t st) {
  switch (a.dh) {
    case 32: return launch_hstu_t<T, 32>(a, st);
    case 64: return launch_hstu_t<T, 64>(a, st);
    case 128: return launch_hstu_t<T, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int hstu_max_pos() { return kMaxPos; }

hipError_t launch_hstu_fwd(const HstuArgs& a, bool bf16_data, hipStream_t st) {
  return bf16_data ? launch_hstu_dh<bf16>(a, st) : launch_hstu_dh<float>(a, st);
}
