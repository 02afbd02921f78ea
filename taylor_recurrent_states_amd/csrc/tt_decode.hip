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
// coalesced store.  Rows are streamed eight at a time per wave to keep many
// loads in flight.  mu(k) and phi(q) are computed once per head into LDS.
#include "tt_device.hpp"
#include "tt_internal.hpp"

namespace tt {

namespace {

constexpr int kDV = 64;
constexpr int kDecodeThreads = 256;

template <int DK, int N, typename TIn>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const TIn* __restrict__ q,
                                                                const TIn* __restrict__ k,
                                                                const TIn* __restrict__ v,
                                                                float* __restrict__ num_plane,
                                                                float* __restrict__ den_plane,
                                                                float* __restrict__ o) {
  constexpr int W = rows_for(DK, N);
  __shared__ float s_q[DK], s_k[DK];
  __shared__ float s_mu[W], s_phi[W];
  __shared__ float s_red[4][kDV];
  __shared__ float s_den[kDecodeThreads];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const auto& tab = RowsOf<DK>::get();

  if (tid < DK) {
    s_q[tid] = load_f32(q, (size_t)bh * DK + tid);
    s_k[tid] = load_f32(k, (size_t)bh * DK + tid);
  }
  __syncthreads();
  for (int r = tid; r < W; r += kDecodeThreads) {
    const uint32_t code = tab.code[r];
    s_mu[r] = monomial(code, [&](int i) { return s_k[i]; });
    s_phi[r] = tab.weight[r] * monomial(code, [&](int i) { return s_q[i]; });
  }
  __syncthreads();

  // value plane: wave w streams rows [r0, r1)
  const float vc = load_f32(v, (size_t)bh * kDV + lane);
  float* __restrict__ S = num_plane + (size_t)bh * W * kDV;
  constexpr int per = (W + 3) / 4;
  const int r0 = wave * per;
  const int r1 = min(W, r0 + per);
  float acc = 0.f;
  int r = r0;
  for (; r + 8 <= r1; r += 8) {
    float s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] = S[(size_t)(r + u) * kDV + lane];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s[u] = fmaf(s_mu[r + u], vc, s[u]);
      S[(size_t)(r + u) * kDV + lane] = s[u];
      acc = fmaf(s_phi[r + u], s[u], acc);
    }
  }
  for (; r < r1; ++r) {
    float s = S[(size_t)r * kDV + lane];
    s = fmaf(s_mu[r], vc, s);
    S[(size_t)r * kDV + lane] = s;
    acc = fmaf(s_phi[r], s, acc);
  }
  s_red[wave][lane] = acc;

  // normaliser plane
  float* __restrict__ D = den_plane + (size_t)bh * W;
  float accd = 0.f;
  for (int rr = tid; rr < W; rr += kDecodeThreads) {
    const float d = D[rr] + s_mu[rr];
    D[rr] = d;
    accd = fmaf(s_phi[rr], d, accd);
  }
  s_den[tid] = accd;
  __syncthreads();
  for (int w = kDecodeThreads / 2; w > 0; w >>= 1) {
    if (tid < w) s_den[tid] += s_den[tid + w];
    __syncthreads();
  }
  if (wave == 0) {
    const float num = (s_red[0][lane] + s_red[1][lane]) + (s_red[2][lane] + s_red[3][lane]);
    o[(size_t)bh * kDV + lane] = num / s_den[0];
  }
}

template <int DK, typename TIn>
__global__ void feature_map_kernel(const TIn* __restrict__ x, size_t rows, int W, int weighted,
                                   float* __restrict__ out) {
  const auto& tab = RowsOf<DK>::get();
  const size_t total = rows * (size_t)W;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t row = e / W;
    const int t = (int)(e - row * W);
    const uint32_t code = tab.code[t];
    float val = monomial(code, [&](int i) { return load_f32(x, row * DK + i); });
    if (weighted) val *= tab.weight[t];
    out[e] = val;
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
                         float* states, float* o, hipStream_t s) {
  const int W = rows_for(dk, n);
  float* num = states;
  float* den = states + (size_t)BH * W * kDV;
  return with_dkn(dk, n, [&](auto DKc, auto Nc) {
    constexpr int DK = decltype(DKc)::value, N = decltype(Nc)::value;
    if (dt == TT_F32)
      hipLaunchKernelGGL((decode_kernel<DK, N, float>), dim3(BH), dim3(kDecodeThreads), 0, s,
                         (const float*)q, (const float*)k, (const float*)v, num, den, o);
    else
      hipLaunchKernelGGL((decode_kernel<DK, N, uint16_t>), dim3(BH), dim3(kDecodeThreads), 0, s,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, num, den, o);
    return hipGetLastError();
  });
}

hipError_t launch_feature_map(const void* x, tt_dtype dt, size_t rows, int dk, int n, int weighted,
                              float* out, hipStream_t s) {
  const int W = rows_for(dk, n);
  const unsigned block = 256;
  const unsigned grid = grid_for(rows * (size_t)W, block);
#define TT_FEAT(DK, T) \
  hipLaunchKernelGGL((feature_map_kernel<DK, T>), dim3(grid), dim3(block), 0, s, (const T*)x, rows, W, weighted, out)
  if (dt == TT_F32) {
    if (dk == 16) TT_FEAT(16, float);
    else if (dk == 32) TT_FEAT(32, float);
    else TT_FEAT(64, float);
  } else {
    if (dk == 16) TT_FEAT(16, uint16_t);
    else if (dk == 32) TT_FEAT(32, uint16_t);
    else TT_FEAT(64, uint16_t);
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
