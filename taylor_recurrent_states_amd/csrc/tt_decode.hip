// Decode step, state merge and the feature-map test hook.
//
// Decode ("Expanding Attention: A Taylor-Series Route to Linear-Time
// Transformers with a Fixed Number of Recurrent States", abstract: one
// rank-one outer-product update per state per token, constant work in the
// context length):  S += mu(k) (x) [v, 1];  o = phi(q).S[:, :dv] / phi(q).S[:, dv].
//
// The step is HBM-bound: every float of the state is read once and written
// once.  One workgroup per head; a wavefront's 64 lanes are the 64 value
// columns, so each state row (256 B) is one coalesced load and one
// coalesced store.  mu(k) and phi(q) are computed once per head into LDS.
// The updated state is written with non-temporal stores: at steady state the
// states of all heads do not fit the memory-side cache, and stores that take
// cache lines there slow the step's loads down.
#include "tt_device.hpp"
#include "tt_internal.hpp"

namespace tt {

namespace {

constexpr int kDV = 64;
constexpr int kDecodeThreads = 256;

// NORM: q and k arrive raw; wave 0 turns q into r(qscale q/|q|) and wave 1
// k into r(k/|k|) in LDS, dk/8 lanes per row with the arithmetic of
// normalize_kernel (the prefill's normalisation pass): group sums of squares
// in fp64, a butterfly over the groups, then unit_coord.
//
// Small states (at most 48 rows per wave, e.g. 153 rows at dk = 16, n = 3):
// every wave issues the loads of all its state rows (and each thread its
// normaliser row) before anything else, so the whole step's reads are in
// flight while q, k and the feature rows are prepared.  Larger states
// stream their rows eight at a time.  Partial sums are reduced with wave
// shuffles and one workgroup barrier; the order is fixed, so results are
// bitwise reproducible.
//
// States of more than kDecodeLdsRows rows (dk = 32 and 64 with four or five
// terms) do not fit mu and phi in LDS: the step then walks the rows in
// chunks of kDecodeChunkRows, forming the chunk's features in LDS and
// updating and reading out its rows before the next chunk.
constexpr int kDecodeLdsRows = 8192;
constexpr int kDecodeChunkRows = 4096;

template <int DK, int N, typename TIn, bool NORM>
__global__ __launch_bounds__(kDecodeThreads, 8) void decode_kernel(const TIn* __restrict__ q,
                                                                const TIn* __restrict__ k,
                                                                const TIn* __restrict__ v,
                                                                float* __restrict__ num_plane,
                                                                float* __restrict__ den_plane,
                                                                float* __restrict__ o, float qscale,
                                                                const uint32_t* __restrict__ big_rows) {
  constexpr int W = rows_for(DK, N);
  constexpr bool CHUNKED = W > kDecodeLdsRows;
  constexpr int LW = CHUNKED ? kDecodeChunkRows : W;  // feature rows held in LDS at a time
  constexpr int per = (W + 3) / 4;       // rows of the value plane per wave
  constexpr bool RES = per <= 48;        // all of a wave's rows held in registers
  __shared__ float s_q[DK], s_k[DK];
  __shared__ float s_mu[LW], s_phi[LW];
  __shared__ float s_red[4][kDV];
  __shared__ float s_den[4];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const RowSrc<DK, N> tab{big_rows};
  float* __restrict__ S = num_plane + (size_t)bh * W * kDV;
  float* __restrict__ D = den_plane + (size_t)bh * W;
  const int r0 = wave * per;
  const int r1 = min(W, r0 + per);

  // state reads first (small states): they overlap everything up to the
  // update. With NORM they follow the normalisation of q and k, so that the
  // resident rows do not share registers with it (at 8 waves per SIMD they
  // would spill); the other resident workgroups cover the later start.
  float sv[RES ? per : 1];
  float dv = 0.f;
  auto load_state = [&]() {
    if constexpr (RES) {
#pragma unroll
      for (int u = 0; u < per; ++u)
        if (r0 + u < r1) sv[u] = S[(size_t)(r0 + u) * kDV + lane];
      if (tid < W) dv = D[tid];
    }
  };
  if constexpr (!NORM) load_state();
  const float vc = load_f32(v, (size_t)bh * kDV + lane);

  if (tid < DK) {
    s_q[tid] = load_f32(q, (size_t)bh * DK + tid);
    s_k[tid] = load_f32(k, (size_t)bh * DK + tid);
  }
  if constexpr (NORM) {  // in place in LDS: wave 0 normalises q, wave 1 k
    __syncthreads();
    constexpr int G = DK / 8;  // lanes per row, one group of 8 coordinates each
    if (wave < 2 && lane < G) {
      float* row = wave == 0 ? s_q : s_k;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = row[8 * lane + e];
      double ss = group_sumsq([&](int i) { return x[i & 7]; }, lane);
#pragma unroll
      for (int off = 1; off < G; off *= 2) ss = ss + __shfl_xor(ss, off);
      const double f = (double)(wave == 0 ? qscale : 1.0f) / sqrt(ss);
#pragma unroll
      for (int e = 0; e < 8; ++e) row[8 * lane + e] = unit_coord<TIn>(x[e], f);
    }
    load_state();
  }
  float acc = 0.f, accd = 0.f;
  if constexpr (CHUNKED) {
    // chunk c covers rows [c0, c0 + cn); wave w updates its quarter of the
    // chunk's value rows, thread tid the normaliser rows tid (mod 256)
    for (int c0 = 0; c0 < W; c0 += LW) {
      const int cn = min(LW, W - c0);
      __syncthreads();  // q and k ready; the previous chunk's features read
      for (int r = tid; r < cn; r += kDecodeThreads) {
        const uint32_t code = tab.code(c0 + r);
        s_mu[r] = monomial<DK>(code, [&](int i) { return s_k[i]; });
        s_phi[r] = row_weight(code) * monomial<DK>(code, [&](int i) { return s_q[i]; });
      }
      __syncthreads();
      // the readout of a chunk is summed on its own and then added, so that
      // no fp32 accumulation chain runs over all rows
      const int a0 = wave * (LW / 4), a1 = min(cn, a0 + LW / 4);
      float accc = 0.f, accdc = 0.f;
      int r = a0;
      for (; r + 8 <= a1; r += 8) {
        float sv8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) sv8[u] = S[(size_t)(c0 + r + u) * kDV + lane];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          sv8[u] = fmaf(s_mu[r + u], vc, sv8[u]);
          store_nt(&S[(size_t)(c0 + r + u) * kDV + lane], sv8[u]);
          accc = fmaf(s_phi[r + u], sv8[u], accc);
        }
      }
      for (; r < a1; ++r) {
        float x = S[(size_t)(c0 + r) * kDV + lane];
        x = fmaf(s_mu[r], vc, x);
        store_nt(&S[(size_t)(c0 + r) * kDV + lane], x);
        accc = fmaf(s_phi[r], x, accc);
      }
      for (int rr = tid; rr < cn; rr += kDecodeThreads) {
        const float d = D[c0 + rr] + s_mu[rr];
        store_nt(&D[c0 + rr], d);
        accdc = fmaf(s_phi[rr], d, accdc);
      }
      acc += accc;
      accd += accdc;
    }
  } else {
  __syncthreads();
  for (int r = tid; r < W; r += kDecodeThreads) {
    const uint32_t code = tab.code(r);
    s_mu[r] = monomial<DK>(code, [&](int i) { return s_k[i]; });
    s_phi[r] = tab.weight(r) * monomial<DK>(code, [&](int i) { return s_q[i]; });
  }
  __syncthreads();

  // value plane: wave w updates rows [r0, r1) and reads them out
  if constexpr (RES) {
#pragma unroll
    for (int u = 0; u < per; ++u)
      if (r0 + u < r1) {
        const float s = fmaf(s_mu[r0 + u], vc, sv[u]);
        store_nt(&S[(size_t)(r0 + u) * kDV + lane], s);
        acc = fmaf(s_phi[r0 + u], s, acc);
      }
  } else {
    int r = r0;
    for (; r + 8 <= r1; r += 8) {
      float s[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) s[u] = S[(size_t)(r + u) * kDV + lane];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s[u] = fmaf(s_mu[r + u], vc, s[u]);
        store_nt(&S[(size_t)(r + u) * kDV + lane], s[u]);
        acc = fmaf(s_phi[r + u], s[u], acc);
      }
    }
    for (; r < r1; ++r) {
      float s = S[(size_t)r * kDV + lane];
      s = fmaf(s_mu[r], vc, s);
      store_nt(&S[(size_t)r * kDV + lane], s);
      acc = fmaf(s_phi[r], s, acc);
    }
  }

  // normaliser plane
  if constexpr (RES) {
    if (tid < W) {
      const float d = dv + s_mu[tid];
      store_nt(&D[tid], d);
      accd = s_phi[tid] * d;
    }
  } else {
    for (int rr = tid; rr < W; rr += kDecodeThreads) {
      const float d = D[rr] + s_mu[rr];
      store_nt(&D[rr], d);
      accd = fmaf(s_phi[rr], d, accd);
    }
  }
  }  // CHUNKED
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) accd += __shfl_xor(accd, off);
  s_red[wave][lane] = acc;
  if (lane == 0) s_den[wave] = accd;
  __syncthreads();
  if (wave == 0) {
    const float num = (s_red[0][lane] + s_red[1][lane]) + (s_red[2][lane] + s_red[3][lane]);
    const float den = (s_den[0] + s_den[1]) + (s_den[2] + s_den[3]);
    o[(size_t)bh * kDV + lane] = num / den;
  }
}

// NT: the number of terms of the row table (the compile-time table of DK,
// or the run-time table `big_rows` for more terms than it holds).
template <int DK, int NT, typename TIn>
__global__ void feature_map_kernel(const TIn* __restrict__ x, size_t rows, int W, int weighted,
                                   float* __restrict__ out, const uint32_t* __restrict__ big_rows) {
  const RowSrc<DK, NT> tab{big_rows};
  const size_t total = rows * (size_t)W;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t row = e / W;
    const int t = (int)(e - row * W);
    const uint32_t code = tab.code(t);
    float val = monomial<DK>(code, [&](int i) { return load_f32(x, row * DK + i); });
    if (weighted) val *= tab.weight(t);
    out[e] = val;
  }
}

// Rows [0, rows0) of x0 -> out0 with scale s0, then rows [0, rows1) of x1 ->
// out1 with scale s1.  A row is spread over D/8 consecutive lanes, one group
// of 8 coordinates each (a 16-byte bf16 or two 16-byte fp32 accesses), so a
// wave reads and writes contiguous memory.  Each lane sums the squares of its
// group (group_sumsq), a shfl_xor butterfly over the row's lanes adds the
// group sums as a pairwise tree, and each lane scales its own coordinates
// (unit_coord); the decode kernel's normalisation does the same, so both
// give the same bits.  out may be x (every
// coordinate is read before it is written, by the same lane).
template <int D, typename TIn>
__global__ __launch_bounds__(256) void normalize_kernel(const TIn* x0, TIn* out0, float s0, size_t rows0,
                                                        const TIn* x1, TIn* out1, float s1, size_t rows1) {
  constexpr int G = D / 8;                      // lanes per row
  constexpr int NV = 8 * sizeof(TIn) / 16;      // 16-byte pieces per group
  const size_t total = (rows0 + rows1) * G;     // one item per (row, group)
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  // every lane of a wave runs the same number of iterations (the butterfly
  // needs the whole row's lanes): items past the end are computed on row 0
  // of x0 and not stored
  const size_t iters = (total + stride - 1) / stride;
  for (size_t it = 0; it < iters; ++it) {
    const size_t item = it * stride + (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = item < total;
    const size_t r = live ? item / G : 0;
    const int g = (int)(item % G);
    const bool first = r < rows0;
    const size_t row = first ? r : r - rows0;
    const u32x4* src = reinterpret_cast<const u32x4*>((first ? x0 : x1) + row * D + 8 * g);
    u32x4 seg[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) seg[i] = src[i];
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (sizeof(TIn) == 2)
        x[e] = bf16_to_f32((uint16_t)((seg[0][e >> 1] >> (16 * (e & 1))) & 0xFFFFu));
      else
        x[e] = __uint_as_float(seg[e >> 2][e & 3]);
    }
    double ss = group_sumsq([&](int i) { return x[i & 7]; }, g);
#pragma unroll
    for (int o = 1; o < G; o *= 2) ss = ss + __shfl_xor(ss, o);
    const double f = (double)(first ? s0 : s1) / sqrt(ss);
    if (live) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = unit_coord<TIn>(x[e], f);
      if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          seg[0][e] = (uint32_t)f32_to_bf16(x[2 * e]) | ((uint32_t)f32_to_bf16(x[2 * e + 1]) << 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) seg[e >> 2][e & 3] = __float_as_uint(x[e]);
      }
      u32x4* dst = reinterpret_cast<u32x4*>((first ? out0 : out1) + row * D + 8 * g);
#pragma unroll
      for (int i = 0; i < NV; ++i) dst[i] = seg[i];
    }
  }
}

__global__ void merge_kernel_vec(float4* dst, const float4* a,
                                 const float4* b, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x) {
    const float4 x = a[i], y = b[i];
    dst[i] = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
  }
}

__global__ void merge_kernel_scalar(float* dst, const float* a,
                                    const float* b, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = a[i] + b[i];
}

unsigned grid_for(size_t work, unsigned block) {
  size_t g = (work + block - 1) / block;
  if (g > 8192) g = 8192;  // grid-stride beyond ~32 workgroups per CU
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, tt_dtype dt, int BH, int dk, int n,
                         float* states, float* o, bool normed, float qscale, hipStream_t s) {
  const int W = rows_for(dk, n);
  float* num = states;
  float* den = states + (size_t)BH * W * kDV;
  const uint32_t* big = nullptr;
  const hipError_t eb = big_row_codes(dk, n, &big);
  if (eb != hipSuccess) return eb;
  return with_dkn(dk, n, [&](auto DKc, auto Nc) {
    constexpr int DK = decltype(DKc)::value, N = decltype(Nc)::value;
    auto go = [&](auto Tc, auto NORMc) {
      using T = decltype(Tc);
      hipLaunchKernelGGL((decode_kernel<DK, N, T, decltype(NORMc)::value>), dim3(BH), dim3(kDecodeThreads), 0, s,
                         (const T*)q, (const T*)k, (const T*)v, num, den, o, qscale, big);
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    if (dt == TT_F32) {
      if (normed) go(float{}, yes{}); else go(float{}, no{});
    } else {
      if (normed) go(uint16_t{}, yes{}); else go(uint16_t{}, no{});
    }
    return hipGetLastError();
  });
}

hipError_t launch_normalize(tt_dtype dt, int d, const void* x0, void* out0, float s0, size_t rows0,
                            const void* x1, void* out1, float s1, size_t rows1, hipStream_t s) {
  const unsigned block = 256;
  const unsigned grid = grid_for((rows0 + rows1) * (size_t)(d / 8), block);
#define TT_NORM(D, T)                                                                                     \
  hipLaunchKernelGGL((normalize_kernel<D, T>), dim3(grid), dim3(block), 0, s, (const T*)x0, (T*)out0, s0, \
                     rows0, (const T*)x1, (T*)out1, s1, rows1)
  if (dt == TT_F32) {
    if (d == 8) TT_NORM(8, float);
    else if (d == 16) TT_NORM(16, float);
    else if (d == 32) TT_NORM(32, float);
    else TT_NORM(64, float);
  } else {
    if (d == 8) TT_NORM(8, uint16_t);
    else if (d == 16) TT_NORM(16, uint16_t);
    else if (d == 32) TT_NORM(32, uint16_t);
    else TT_NORM(64, uint16_t);
  }
#undef TT_NORM
  return hipGetLastError();
}

hipError_t launch_feature_map(const void* x, tt_dtype dt, size_t rows, int dk, int n, int weighted,
                              float* out, hipStream_t s) {
  const int W = rows_for(dk, n);
  const unsigned block = 256;
  const unsigned grid = grid_for(rows * (size_t)W, block);
  const uint32_t* big = nullptr;
  const hipError_t eb = big_row_codes(dk, n, &big);
  if (eb != hipSuccess) return eb;
#define TT_FEAT(DK, NT, T)                                                                                   \
  hipLaunchKernelGGL((feature_map_kernel<DK, NT, T>), dim3(grid), dim3(block), 0, s, (const T*)x, rows, W, \
                     weighted, out, big)
  // the compile-time table of a key width serves every n up to its terms;
  // dk = 32 and 64 with more terms read the run-time table
  const bool rt = big != nullptr;
  if (dt == TT_F32) {
    if (dk == 8) TT_FEAT(8, 6, float);
    else if (dk == 16) TT_FEAT(16, 5, float);
    else if (dk == 32) { if (rt) TT_FEAT(32, 5, float); else TT_FEAT(32, 3, float); }
    else { if (rt) TT_FEAT(64, 5, float); else TT_FEAT(64, 3, float); }
  } else {
    if (dk == 8) TT_FEAT(8, 6, uint16_t);
    else if (dk == 16) TT_FEAT(16, 5, uint16_t);
    else if (dk == 32) { if (rt) TT_FEAT(32, 5, uint16_t); else TT_FEAT(32, 3, uint16_t); }
    else { if (rt) TT_FEAT(64, 5, uint16_t); else TT_FEAT(64, 3, uint16_t); }
  }
#undef TT_FEAT
  return hipGetLastError();
}

hipError_t launch_merge(float* dst, const float* a, const float* b, size_t n, hipStream_t s) {
  const unsigned block = 256;
  const bool aligned = ((((uintptr_t)dst) | ((uintptr_t)a) | ((uintptr_t)b)) & 15u) == 0;
  if (aligned && n >= 4) {
    const size_t n4 = n / 4;
    hipLaunchKernelGGL(merge_kernel_vec, dim3(grid_for(n4, block)), dim3(block), 0, s, (float4*)dst,
                       (const float4*)a, (const float4*)b, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t done = n4 * 4;
    if (done < n)
      hipLaunchKernelGGL(merge_kernel_scalar, dim3(1), dim3(block), 0, s, dst + done, a + done, b + done,
                         n - done);
  } else {
    hipLaunchKernelGGL(merge_kernel_scalar, dim3(grid_for(n, block)), dim3(block), 0, s, dst, a, b, n);
  }
  return hipGetLastError();
}

}  // namespace tt
