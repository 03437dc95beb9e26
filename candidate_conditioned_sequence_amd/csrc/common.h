// Shared device helpers for the libwhalefuse kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <climits>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define WHALE_DEV __device__ __forceinline__

// --------------------------------------------------------------- element types
// Every MFMA operand chunk holds 8 elements per lane.  For bf16 this is one
// v_mfma_f32_32x32x16_bf16 operand.  For fp32 it is fed to eight
// v_mfma_f32_32x32x2_f32 issues, element i of every lane going to issue i;
// the contraction index each (lane half, element) pair stands for is then a
// bijection onto the 16 k values of the step, the same for A and B, so the
// sum is the full contraction either way.
template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 x8; typedef bf16x4 x4; };
template <> struct Vec<float> { typedef f32x8 x8; typedef f32x4 x4; };

template <typename T> using x8_t = typename Vec<T>::x8;
template <typename T> using x4_t = typename Vec<T>::x4;

WHALE_DEV float to_f(bf16 x) { return (float)x; }
WHALE_DEV float to_f(float x) { return x; }
template <typename T> WHALE_DEV T from_f(float x);
template <> WHALE_DEV bf16 from_f<bf16>(float x) { return (bf16)x; }   // v_cvt_pk_bf16_f32: nearest even
template <> WHALE_DEV float from_f<float>(float x) { return x; }

template <typename T> WHALE_DEV x8_t<T> zero8() { x8_t<T> v; for (int i = 0; i < 8; ++i) v[i] = from_f<T>(0.f); return v; }

template <typename T> WHALE_DEV x8_t<T> ld8(const T* p) { return *reinterpret_cast<const x8_t<T>*>(p); }
template <typename T> WHALE_DEV void st8(T* p, const x8_t<T>& v) { *reinterpret_cast<x8_t<T>*>(p) = v; }
template <typename T> WHALE_DEV x4_t<T> ld4(const T* p) { return *reinterpret_cast<const x4_t<T>*>(p); }
template <typename T> WHALE_DEV void st4(T* p, const x4_t<T>& v) { *reinterpret_cast<x4_t<T>*>(p) = v; }

// Two 4-element runs -> one 8-element operand.
template <typename T> WHALE_DEV x8_t<T> cat44(const x4_t<T>& a, const x4_t<T>& b) {
  x8_t<T> v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

// --------------------------------------------------------------- MFMA
// D[32x32] += A[32x16] * B[16x32].  Lane l supplies row (A) / column (B)
// l % 32 and eight contraction values for half l / 32.  The accumulator
// register r of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l % 32].
WHALE_DEV void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
WHALE_DEV void mma32(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], acc, 0, 0, 0);
}

// Row of accumulator register r for lane half hh (column is lane % 32).
WHALE_DEV constexpr int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

WHALE_DEV f32x16 zero16() { f32x16 v; for (int i = 0; i < 16; ++i) v[i] = 0.f; return v; }

// --------------------------------------------------------------- transposed operands
// A operand of a 32x32x16 step taken column-wise from a row-major LDS tile
// X[row][col] (row stride ld elements): lane l gets column c0 + l % 32 and, for
// lane half hh = l / 32, the rows r0 + 4 hh + u (u < 4) and r0 + 8 + 4 hh + (u - 4)
// (u >= 4) -- the row order of a 32x32 accumulator's column, so an accumulator
// can be fed back as the matching B operand.
//
// bf16 uses the gfx950 transposing LDS read ds_read_b64_tr_b16: within each
// 16-lane group, lane i supplies a pointer p_i to four consecutive 16-bit
// elements and lane j receives p_{4k + j/4}[j % 4] for k = 0..3.  Lane i of
// group g therefore points at row r0 + 4 (g / 2) + i / 4, column
// c0 + 16 (g % 2) + 4 (i % 4); the second read is 8 rows further down.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

WHALE_DEV bf16x4 lds_tr4(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) bf16*)(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// LDS reads from a 32-bit LDS byte address (one base register plus an
// immediate offset per read).
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
WHALE_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
WHALE_DEV bf16x8 lds_ld8(uint32_t a) { return *(const lds_bf16x8*)(uintptr_t)a; }
WHALE_DEV bf16x4 lds_tr4_at(uint32_t a) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
  return __builtin_bit_cast(bf16x4, v);
}

template <typename T> WHALE_DEV x8_t<T> lds_colA(const T* X, int ld, int r0, int c0, int lane);

template <> WHALE_DEV bf16x8 lds_colA<bf16>(const bf16* X, int ld, int r0, int c0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const bf16* p = X + (r0 + 4 * (g >> 1) + (i >> 2)) * ld + c0 + 16 * (g & 1) + 4 * (i & 3);
  return cat44<bf16>(lds_tr4(p), lds_tr4(p + 8 * ld));
}

// The same reads split into a per-lane element offset (computed once) and a
// tile-uniform base X + r0*ld + c0.
template <typename T> WHALE_DEV int lds_colA_lane(int ld, int lane);
template <> WHALE_DEV int lds_colA_lane<bf16>(int ld, int lane) {
  const int g = lane >> 4, i = lane & 15;
  return (4 * (g >> 1) + (i >> 2)) * ld + 16 * (g & 1) + 4 * (i & 3);
}
template <> WHALE_DEV int lds_colA_lane<float>(int ld, int lane) {
  return 4 * (lane >> 5) * ld + (lane & 31);
}
template <typename T> WHALE_DEV x8_t<T> lds_colA_at(const T* base, int ld, int off);
template <> WHALE_DEV bf16x8 lds_colA_at<bf16>(const bf16* base, int ld, int off) {
  return cat44<bf16>(lds_tr4(base + off), lds_tr4(base + off + 8 * ld));
}
template <> WHALE_DEV f32x8 lds_colA_at<float>(const float* base, int ld, int off) {
  f32x8 v;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v[u] = base[off + u * ld];
    v[u + 4] = base[off + (8 + u) * ld];
  }
  return v;
}

template <> WHALE_DEV f32x8 lds_colA<float>(const float* X, int ld, int r0, int c0, int lane) {
  const int hh = lane >> 5, c = c0 + (lane & 31);
  f32x8 v;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v[u] = X[(r0 + 4 * hh + u) * ld + c];
    v[u + 4] = X[(r0 + 8 + 4 * hh + u) * ld + c];
  }
  return v;
}

// --------------------------------------------------------------- misc
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  This
// gives each XCD one contiguous range of logical ids so that workgroups
// that read the same data (one request's K/V, one weight tile) share that
// XCD's L2.  A bijection on [0, n).
WHALE_DEV int xcd_remap(int id, int n) {
  const int nx = 8;
  const int per = n / nx, rem = n % nx;
  const int x = id % nx, i = id / nx;
  return x * per + (x < rem ? x : rem) + i;
}

// Order for grids whose logical id is pair * nb + k, a pair being one
// (request, head) whose nb blocks read the same rows and whose work grows
// with the request's length.  With contiguous ranges (xcd_remap) each XCD
// would take one eighth of the batch, and the lengths of a few neighbouring
// requests can differ widely; here XCD x takes pairs x, x + 8, x + 16, ...
// whole and in that order, so a pair's blocks still share one L2 while each
// XCD sees a spread of the batch.  Pairs past the last full group of eight
// keep the plain order.  A bijection on [0, npairs * nb).
WHALE_DEV int pair_xcd_order(int id, int nb, int npairs) {
  const int full = (npairs / 8) * 8 * nb;   // blocks of complete groups of 8 pairs
  if (id >= full) return id;
  const int x = id % 8, i = id / 8;
  return ((i / nb) * 8 + x) * nb + i % nb;
}

// Longest-first order of the B requests of a batch (ties by index), so
// that the (request, head) pairs dealt to the XCDs come longest first and
// the shortest run last (list scheduling): perm[rank] = request, in LDS.
// Every thread of the workgroup calls it (two barriers); lens holds B
// rounded up to 4 entries, and each thread ranks its requests against all
// B lengths, four per LDS read.  Each output element is still produced by
// one workgroup with the same arithmetic, so the order changes no result.
WHALE_DEV void rank_requests(const int64_t* __restrict__ offsets, int B, int* lens, int* perm) {
  const int B4 = (B + 3) & ~3;
  for (int b = threadIdx.x; b < B4; b += blockDim.x)
    lens[b] = b < B ? (int)(offsets[b + 1] - offsets[b]) : INT_MIN;
  __syncthreads();
  const int4* l4 = reinterpret_cast<const int4*>(lens);
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int Lb = lens[b];
    int rank = 0;
#pragma unroll 4
    for (int c4 = 0; c4 < B4 / 4; ++c4) {
      const int4 v = l4[c4];
      const int c = 4 * c4;
      rank += (v.x > Lb) | ((v.x == Lb) & (c < b));
      rank += (v.y > Lb) | ((v.y == Lb) & (c + 1 < b));
      rank += (v.z > Lb) | ((v.z == Lb) & (c + 2 < b));
      rank += (v.w > Lb) | ((v.w == Lb) & (c + 3 < b));
    }
    perm[rank] = b;
  }
  __syncthreads();
}

WHALE_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// max of three (one v_max3_f32: the inner max has no other use)
WHALE_DEV float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
// Logistic sigmoid with the hardware reciprocal (about 1 ulp): the IEEE
// division sequence would cost ten instructions per element in the gate and
// activation prologues / epilogues.  1 + e^-z = inf gives 0, as it should.
WHALE_DEV float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }
WHALE_DEV float siluf_(float z) { return z * sigmoidf_(z); }
WHALE_DEV float dsiluf_(float z) { float s = sigmoidf_(z); return s * (1.f + z * (1.f - s)); }

// Combine a value across the two lane halves (lanes l and l ^ 32) with one
// v_permlane32_swap: both halves get the same result, formed in the same
// order (low half's value first).
WHALE_DEV f32x2 half_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  return f32x2{__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}
// med3(a, b, +inf) = max(a, b) without the quieting moves fmaxf adds.
WHALE_DEV float half_max(float v) {
  const f32x2 p = half_pair(v);
  return __builtin_amdgcn_fmed3f(p[0], p[1], INFINITY);
}
WHALE_DEV float half_sum(float v) { const f32x2 p = half_pair(v); return p[0] + p[1]; }

WHALE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
