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

// ---------------------------------------------------------------------------
// Compile-time row tables.  One table per supported key width holds the rows
// of the largest supported order; smaller orders use a prefix (blocks are in
// ascending m).  Entry: code = idx0 | idx1<<6 | idx2<<12 | idx3<<18 | m<<24
// | w<<27, where w indexes 1/alpha(t)! in {1, 1/2, 1/4, 1/6, 1/24}; weight =
// 1/alpha(t)! rounded to fp32.
// ---------------------------------------------------------------------------

constexpr int binom(int a, int b) {
  if (b < 0 || b > a) return 0;
  long long r = 1;
  for (int i = 1; i <= b; ++i) r = r * (a - b + i) / i;
  return (int)r;
}

constexpr int rows_for(int dk, int n) { return binom(dk + n - 1, n - 1); }

template <int DK, int NMAX>
struct RowTable {
  static constexpr int W = rows_for(DK, NMAX);
  uint32_t code[W];
  float weight[W];
  constexpr RowTable() : code(), weight() {
    int r = 0;
    for (int m = 0; m < NMAX; ++m) {
      int t[4] = {0, 0, 0, 0};
      bool more = true;
      while (more) {
        uint32_t c = (uint32_t)m << 24;
        for (int l = 0; l < m; ++l) c |= (uint32_t)t[l] << (6 * l);
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
        const uint32_t widx = denom == 1 ? 0u : denom == 2 ? 1u : denom == 4 ? 2u : denom == 6 ? 3u : 4u;
        code[r] = c | (widx << 27);
        weight[r] = 1.0f / (float)denom;
        ++r;
        // next non-decreasing tuple in lexicographic order
        int i = m - 1;
        while (i >= 0 && t[i] == DK - 1) --i;
        if (i < 0) {
          more = false;
        } else {
          ++t[i];
          for (int j = i + 1; j < m; ++j) t[j] = t[i];
        }
      }
    }
  }
};

static_assert(rows_for(16, 3) == 153, "W(16,3)");
static_assert(rows_for(16, 5) == 4845, "W(16,5)");
static_assert(rows_for(64, 3) == 2145, "W(64,3)");

// Device copies, constant-initialised in each code object (read-only).
static __device__ const RowTable<16, 5> kRows16 = RowTable<16, 5>();
static __device__ const RowTable<32, 3> kRows32 = RowTable<32, 3>();
static __device__ const RowTable<64, 3> kRows64 = RowTable<64, 3>();

template <int DK> struct RowsOf;
template <> struct RowsOf<16> { static __device__ const RowTable<16, 5>& get() { return kRows16; } };
template <> struct RowsOf<32> { static __device__ const RowTable<32, 3>& get() { return kRows32; } };
template <> struct RowsOf<64> { static __device__ const RowTable<64, 3>& get() { return kRows64; } };

__host__ __device__ constexpr int row_order(uint32_t code) { return (int)((code >> 24) & 7u); }
__host__ __device__ constexpr int row_index_c(uint32_t code, int l) { return (int)((code >> (6 * l)) & 63u); }
// 1/alpha(t)! from the weight index of a row code
__host__ __device__ constexpr float row_weight(uint32_t code) {
  const uint32_t w = (code >> 27) & 7u;
  return w == 0 ? 1.0f : w == 1 ? 0.5f : w == 2 ? 0.25f : w == 3 ? 1.0f / 6.0f : 1.0f / 24.0f;
}
// code of a padding row (order 7: contributes nothing)
constexpr uint32_t kPadRow = 7u << 24;
__device__ inline int row_index(uint32_t code, int l) { return (int)((code >> (6 * l)) & 63u); }

// mu_t(x) for a row code, reading coordinates through `get(i)`.
template <typename Get>
__device__ inline float monomial(uint32_t code, Get get) {
  const int m = row_order(code);
  float p = 1.0f;
  for (int l = 0; l < m; ++l) p *= get(row_index(code, l));
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

// 1/x by the hardware reciprocal (v_rcp_f32: within 1 ulp for normal x).
__device__ inline float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------------------
// L2 normalisation of one q or k row ("Expanding Attention", abstract: unit
// q and k keep q.k inside the series' convergence radius; a temperature is
// folded into the queries as `scale`).  x <- r(scale * x / ||x||_2), where r
// rounds to the input dtype (bf16: nearest even; fp32: identity).  Every
// operation is one IEEE fp32 operation rounded to nearest even, in a fixed
// order (row_norm_factor: squares summed in groups of 8, group sums by a
// pairwise tree, no fused multiply-add; then the square root, scale / root,
// and x_i * that factor).  The result is a fixed function of the input bits,
// the same in every kernel, and a host can reproduce it exactly.  A zero row
// gives NaN.
// ---------------------------------------------------------------------------

// Sum of squares of the 8 coordinates get(8g) .. get(8g+7), in index order.
template <typename Get>
__device__ inline float group_sumsq(Get get, int g) {
#pragma clang fp contract(off)
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xi = get(8 * g + e);
    const float sq = xi * xi;
    s = s + sq;
  }
  return s;
}

// The factor scale / ||x||_2 of a row whose coordinates get(0) .. get(D-1)
// are fp32 values.  Squares are summed in groups of 8 consecutive
// coordinates (group_sumsq); the group sums are added as a balanced pairwise
// tree, neighbours first (((g0+g1)+(g2+g3))+...).  A kernel that spreads a
// row over D/8 lanes reaches the same bits with a shfl_xor butterfly over
// lane offsets 1, 2, 4 (IEEE addition commutes).
template <int D, typename Get>
__device__ inline float row_norm_factor(Get get, float scale) {
#pragma clang fp contract(off)
  constexpr int G = D / 8;
  static_assert(D % 8 == 0 && (G & (G - 1)) == 0, "groups of 8, a power-of-two count");
  float g[G];
#pragma unroll
  for (int j = 0; j < G; ++j) g[j] = group_sumsq(get, j);
#pragma unroll
  for (int w = 1; w < G; w *= 2)
#pragma unroll
    for (int j = 0; j + w < G; j += 2 * w) g[j] = g[j] + g[j + w];
  return scale / sqrtf(g[0]);
}

// One unit coordinate: r(x * f), rounded to the input dtype.
template <typename TIn>
__device__ inline float unit_coord(float x, float f) {
#pragma clang fp contract(off)
  const float y = x * f;
  if constexpr (std::is_same<TIn, uint16_t>::value)
    return bf16_to_f32(f32_to_bf16(y));
  else
    return y;
}

template <typename TIn, int D>
__device__ inline void normalize_row(float (&x)[D], float scale) {
  const float f = row_norm_factor<D>([&](int i) { return x[i]; }, scale);
#pragma unroll
  for (int i = 0; i < D; ++i) x[i] = unit_coord<TIn>(x[i], f);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (16x16 output tiles).  Lane l = 16*g + i  (i = l%16, g = l/16).
//   bf16 16x16x32: A lane holds A[i][8g .. 8g+7]; B lane holds B[8g .. 8g+7][i];
//   f32  16x16x4 : A lane holds A[i][g];          B lane holds B[g][i];
//   D (both)     : lane holds D[4g + s][i], s = 0..3.
// ---------------------------------------------------------------------------

typedef float f32x4 __attribute__((ext_vector_type(4)));
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
  TT_CASE(16, 1) TT_CASE(16, 2) TT_CASE(16, 3) TT_CASE(16, 4) TT_CASE(16, 5)
  TT_CASE(32, 1) TT_CASE(32, 2) TT_CASE(32, 3)
  TT_CASE(64, 1) TT_CASE(64, 2) TT_CASE(64, 3)
#undef TT_CASE
  return hipErrorInvalidValue;
}

}  // namespace tt
