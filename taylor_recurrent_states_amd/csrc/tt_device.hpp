// Device-side building blocks shared by the kernels of libtaylor_states.so:
// the packed symmetric feature-row tables, bf16 helpers and MFMA wrappers
// for gfx950 (CDNA4).
//
// Feature rows ("Expanding Attention: A Taylor-Series Route to Linear-Time
// Transformers with a Fixed Number of Recurrent States", abstract): the m-th
// Taylor term (q.k)^m / m! is an inner product of symmetric tensor powers,
// stored packed as the C(d+m-1, m) non-decreasing index tuples t.  Row t of
// the key side is the monomial mu_t(x) = prod_l x[t_l]; the query side
// carries the multinomial weight, phi_t(x) = mu_t(x) / alpha(t)!.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tt {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Compile-time row tables.  One table per supported key width holds the rows
// of the largest supported order; smaller orders use a prefix (blocks are in
// ascending m).  Entry: code = idx0 | idx1 << B | idx2 << 2B | ... | m << 24
// | w << 27, with B = index_bits(dk) bits per index (enough for dk - 1), m
// the order and w indexing 1/alpha(t)! in {1, 1/2, 1/4, 1/6, 1/12, 1/24,
// 1/120}; weight = 1/alpha(t)! rounded to fp32.
// ---------------------------------------------------------------------------

constexpr int binom(int a, int b) {
  if (b < 0 || b > a) return 0;
  long long r = 1;
  for (int i = 1; i <= b; ++i) r = r * (a - b + i) / i;
  return (int)r;
}

constexpr int rows_for(int dk, int n) { return binom(dk + n - 1, n - 1); }

// bits per index in a row code, and the number of Taylor terms compiled for
// each key width (the largest order is max_terms - 1)
constexpr int index_bits(int dk) { return dk <= 8 ? 3 : dk <= 16 ? 4 : dk <= 32 ? 5 : 6; }
constexpr int max_terms(int dk) { return dk <= 8 ? 6 : dk <= 16 ? 5 : 3; }
// Terms compiled for each key width, counting the widest shapes (dk = 32 and
// 64 with four or five terms: 6,545 to 814,385 rows), whose row codes live in
// a table built once per device at run time instead of a compile-time table.
constexpr int max_terms_all(int dk) { return dk <= 8 ? 6 : 5; }
template <int DK, int NT>
constexpr bool runtime_rows() { return NT > max_terms(DK); }
static_assert(index_bits(8) * 5 <= 24 && index_bits(16) * 4 <= 24 && index_bits(64) * 4 <= 24, "code fields");

constexpr uint32_t weight_index(int denom) {
  return denom == 1 ? 0u : denom == 2 ? 1u : denom == 4 ? 2u : denom == 6 ? 3u : denom == 12 ? 4u : denom == 24 ? 5u : 6u;
}

// Row codes of all feature rows of orders 0 .. nmax-1 for key width dk, in
// feature order: m-blocks ascending, inside a block the non-decreasing index
// tuples in lexicographic order.  A code holds the order m (bits 24-26), the
// m indices (ib bits each from bit 0) and the weight index of 1/alpha(t)!
// (bits 27-29); `weight` (may be null) receives 1/alpha(t)!.  Used at compile
// time for the tables below and on the host for the run-time tables of the
// widest shapes.  Returns the number of rows written.
constexpr int enumerate_rows(int dk, int nmax, int ib, uint32_t* code, float* weight) {
  int r = 0;
  for (int m = 0; m < nmax; ++m) {
    int t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    bool more = true;
    while (more) {
      uint32_t c = (uint32_t)m << 24;
      for (int l = 0; l < m; ++l) c |= (uint32_t)t[l] << (ib * l);
      // 1 / prod over runs of equal indices of (run length)!
      int denom = 1, run = 1;
      for (int l = 1; l <= m; ++l) {
        if (l < m && t[l] == t[l - 1]) {
          ++run;
        } else {
          for (int f = 2; f <= run; ++f) denom *= f;
          run = 1;
        }
      }
      code[r] = c | (weight_index(denom) << 27);
      if (weight != nullptr) weight[r] = 1.0f / (float)denom;
      ++r;
      // next non-decreasing tuple in lexicographic order
      int i = m - 1;
      while (i >= 0 && t[i] == dk - 1) --i;
      if (i < 0) {
        more = false;
      } else {
        ++t[i];
        for (int j = i + 1; j < m; ++j) t[j] = t[i];
      }
    }
  }
  return r;
}

template <int DK, int NMAX>
struct RowTable {
  static constexpr int W = rows_for(DK, NMAX);
  static constexpr int IB = index_bits(DK);
  uint32_t code[W];
  float weight[W];
  constexpr RowTable() : code(), weight() { enumerate_rows(DK, NMAX, IB, code, weight); }
};

static_assert(rows_for(16, 3) == 153, "W(16,3)");
static_assert(rows_for(16, 5) == 4845, "W(16,5)");
static_assert(rows_for(64, 3) == 2145, "W(64,3)");
static_assert(rows_for(8, 6) == 1287, "W(8,6)");

// Device copies, constant-initialised in each code object (read-only).
static __device__ const RowTable<8, 6> kRows8 = RowTable<8, 6>();
static __device__ const RowTable<16, 5> kRows16 = RowTable<16, 5>();
static __device__ const RowTable<32, 3> kRows32 = RowTable<32, 3>();
static __device__ const RowTable<64, 3> kRows64 = RowTable<64, 3>();

template <int DK> struct RowsOf;
template <> struct RowsOf<8> { static __device__ const RowTable<8, 6>& get() { return kRows8; } };
template <> struct RowsOf<16> { static __device__ const RowTable<16, 5>& get() { return kRows16; } };
template <> struct RowsOf<32> { static __device__ const RowTable<32, 3>& get() { return kRows32; } };
template <> struct RowsOf<64> { static __device__ const RowTable<64, 3>& get() { return kRows64; } };

// Row codes and weights of a (DK, NT) shape: the compile-time table, or for
// the widest shapes the run-time table `big` (weights from the codes).
template <int DK, int NT>
struct RowSrc {
  const uint32_t* big;
  __device__ uint32_t code(int r) const {
    if constexpr (runtime_rows<DK, NT>()) return big[r];
    else return RowsOf<DK>::get().code[r];
  }
  __device__ float weight(int r) const;
};

__host__ __device__ constexpr int row_order(uint32_t code) { return (int)((code >> 24) & 7u); }
// index l of a row code of key width DK
template <int DK>
__host__ __device__ constexpr int row_index_c(uint32_t code, int l) {
  return (int)((code >> (index_bits(DK) * l)) & ((1u << index_bits(DK)) - 1u));
}
// 1/alpha(t)! from the weight index of a row code
__host__ __device__ constexpr float row_weight(uint32_t code) {
  const uint32_t w = (code >> 27) & 7u;
  return w == 0 ? 1.0f : w == 1 ? 0.5f : w == 2 ? 0.25f : w == 3 ? 1.0f / 6.0f : w == 4 ? 1.0f / 12.0f
       : w == 5 ? 1.0f / 24.0f : 1.0f / 120.0f;
}
// code of a padding row (order 7: contributes nothing)
constexpr uint32_t kPadRow = 7u << 24;
template <int DK>
__device__ inline int row_index(uint32_t code, int l) { return row_index_c<DK>(code, l); }

template <int DK, int NT>
__device__ inline float RowSrc<DK, NT>::weight(int r) const {
  if constexpr (runtime_rows<DK, NT>()) return row_weight(big[r]);
  else return RowsOf<DK>::get().weight[r];
}

// mu_t(x) for a row code of key width DK, reading coordinates through `get(i)`.
template <int DK, typename Get>
__device__ inline float monomial(uint32_t code, Get get) {
  const int m = row_order(code);
  float p = 1.0f;
  for (int l = 0; l < m; ++l) p *= get(row_index<DK>(code, l));
  return p;
}

// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename TIn> __device__ inline float load_f32(const TIn* p, size_t i);
template <> __device__ inline float load_f32<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float load_f32<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ inline uint16_t f32_to_bf16(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// Two fp32 -> packed bf16x2 (lo in bits 0..15).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): 16 significant bits.
__device__ inline void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// split_bf16 of two values at once, packed (a in bits 0..15): the same bits,
// with one conversion per plane instead of one per value.
__device__ inline void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// Stores of results no kernel of the same call reads back (outputs, updated
// states): non-temporal, so they stream to memory without taking cache
// lines that the loads still need.  On the decode step at steady state from
// HBM this measured 37.5 -> 27.9 us per step.
__device__ inline void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ inline void store_nt(float* p, f32x4_t v) { __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p)); }

// a.lo * b.lo + a.hi * b.hi + c for packed bf16 pairs a and b (products
// exact, one fp32 rounding), in the three-operand encoding: the builtin is
// compiled to the two-operand form, which accumulates in place and so costs a
// register copy whenever c must survive.
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// 1/x by the hardware reciprocal (v_rcp_f32: within 1 ulp for normal x).
__device__ inline float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------------------
// L2 normalisation of one q or k row ("Expanding Attention", abstract: unit
// q and k keep q.k inside the series' convergence radius; a temperature is
// folded into the queries as `scale`).  x <- r(scale * x / ||x||_2), where r
// rounds once to the nearest value of the input dtype (ties to even).  The
// quotient is evaluated in fp64: squares of the fp32 coordinates (exact in
// fp64) summed in groups of 8 consecutive coordinates (group_sumsq), the
// group sums added as a balanced pairwise tree, neighbours first
// (((g0+g1)+(g2+g3))+..., which a shfl_xor butterfly over lane offsets 1, 2,
// 4 gives when each lane holds one group), then f = scale / sqrt(sum) and
// x_i * f (unit_coord), each an IEEE fp64 operation.  That value lies within
// about 10 fp64 ulps of the exact unit coordinate, so r gives the correctly
// rounded unit row except where the exact value lies that close to a
// rounding boundary.  The operation order is fixed, so every kernel gives the
// same bits.  A zero row gives NaN.
// ---------------------------------------------------------------------------

// Sum of squares of the 8 coordinates get(8g) .. get(8g+7), in index order,
// in fp64 (each square of an fp32 value is exact).
template <typename Get>
__device__ inline double group_sumsq(Get get, int g) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double xi = (double)get(8 * g + e);
    s = s + xi * xi;
  }
  return s;
}

// fp64 -> bf16 rounded once to nearest even.  The fp64 value is first
// rounded to fp32 by rounding to odd (toward zero, then the last bit set if
// the conversion was inexact): that keeps the information the second
// rounding needs, so fp32 -> bf16 to nearest even then gives the correctly
// rounded bf16 of the fp64 value.  (Rounding to nearest fp32 first could
// land exactly on a bf16 midpoint and round a second time.)  The bit
// operations also keep the compiler from folding the two conversions.
__device__ inline float round_bf16_from_f64(double y) {
  float t = (float)y;
  const double back = (double)t;
  if (back != y) {
    uint32_t b = __float_as_uint(t);
    if (fabs(back) > fabs(y)) b -= 1u;  // one fp32 step toward zero
    t = __uint_as_float(b | 1u);
  }
  return bf16_to_f32(f32_to_bf16(t));
}

// One unit coordinate: r(x * f) with x * f in fp64, rounded once to the
// input dtype (nearest even).
template <typename TIn>
__device__ inline float unit_coord(float x, double f) {
  const double y = (double)x * f;
  if constexpr (std::is_same<TIn, uint16_t>::value)
    return round_bf16_from_f64(y);
  else
    return (float)y;
}

// ---------------------------------------------------------------------------
// MFMA wrappers (16x16 output tiles).  Lane l = 16*g + i  (i = l%16, g = l/16).
//   bf16 16x16x32: A lane holds A[i][8g .. 8g+7]; B lane holds B[8g .. 8g+7][i];
//   f32  16x16x4 : A lane holds A[i][g];          B lane holds B[g][i];
//   D (both)     : lane holds D[4g + s][i], s = 0..3.
// ---------------------------------------------------------------------------

typedef f32x4_t f32x4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// split_bf16x2 of eight values (x0.xyzw, then x1.xyzw) into packed hi and lo
// planes of four dwords each (the same bits as eight split_bf16 calls).
__device__ inline void split_bf16x8(f32x4 x0, f32x4 x1, u32x4& hi, u32x4& lo) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split_bf16x2(x0.x, x0.y, h0, l0);
  split_bf16x2(x0.z, x0.w, h1, l1);
  split_bf16x2(x1.x, x1.y, h2, l2);
  split_bf16x2(x1.z, x1.w, h3, l3);
  hi = u32x4{h0, h1, h2, h3};
  lo = u32x4{l0, l1, l2, l3};
}

// Workgroup barrier ordering LDS only: each wave waits for its own LDS
// operations, not for its global loads and stores in flight (a plain
// __syncthreads() also drains outstanding global stores).  For kernels whose
// waves never read global memory written by another wave of the workgroup.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Transposing LDS read of 16-bit data (gfx950 ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane l receives element l%4 of the 8-byte pieces
// addressed by lanes 4s + l/4, s = 0..3 (probed on gfx950).  Consequence used
// by the kernels: if lane j of group g addresses row 8g + 4h + j/4 and column
// c(j%4) of a row-major bf16 tile X[k][col], lane (i, g) receives
// X[8g + 4h + s][c(i/4) + i%4] for s = 0..3; two reads (h = 0, 1) give the
// bf16 16x16x32 MFMA fragment whose K index runs over the tile's rows.
__device__ inline uint2 lds_tr16(const void* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// static_for<B, E>(f): f(integral_constant<int, i>) for i in [B, E)
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Calls fn(integral_constant<DK>, integral_constant<N>) for a supported
// (dk, n); hipErrorInvalidValue otherwise.
template <typename Fn>
inline hipError_t with_dkn(int dk, int n, Fn&& fn) {
  using std::integral_constant;
#define TT_CASE(D, NN) \
  if (dk == D && n == NN) return fn(integral_constant<int, D>{}, integral_constant<int, NN>{});
  TT_CASE(8, 1) TT_CASE(8, 2) TT_CASE(8, 3) TT_CASE(8, 4) TT_CASE(8, 5) TT_CASE(8, 6)
  TT_CASE(16, 1) TT_CASE(16, 2) TT_CASE(16, 3) TT_CASE(16, 4) TT_CASE(16, 5)
  TT_CASE(32, 1) TT_CASE(32, 2) TT_CASE(32, 3) TT_CASE(32, 4) TT_CASE(32, 5)
  TT_CASE(64, 1) TT_CASE(64, 2) TT_CASE(64, 3) TT_CASE(64, 4) TT_CASE(64, 5)
#undef TT_CASE
  return hipErrorInvalidValue;
}

}  // namespace tt
