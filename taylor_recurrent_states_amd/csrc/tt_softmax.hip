// Exact causal softmax attention, the quantity the truncated Taylor kernel
// approximates ("Expanding Attention: A Taylor-Series Route to Linear-Time
// Transformers with a Fixed Number of Recurrent States", abstract: the
// method is compared with softmax attention in prefill time and in decode
// time per token).  A baseline on the same GPU, no scale inside exp:
//
//     o_i = sum_{j<=i} exp(q_i.k_j) v_j / sum_{j<=i} exp(q_i.k_j)
//
// Prefill (bf16 inputs, fp32 output): one workgroup of 4 waves per (head,
// block of 64 queries); a wave owns 16 queries and all 64 value columns as
// O^T accumulator tiles.  Key blocks of 64 keys are staged in LDS (double
// buffered) and visited from the first to the diagonal one.  Scores are
// formed as S^T = K Q^T by MFMA so that each lane holds 16 scores of one
// query whose fp32 probabilities, packed to bf16, are directly the B
// operand of O^T += V^T P^T.  The running maximum is kept in base 2 (scores
// times log2 e; exp2 on the hardware unit).  The diagonal block feeds P as
// a hi + lo bf16 pair (early queries see few keys, so their weights are not
// averaged over many roundings); earlier blocks feed bf16 P.  The running
// sum uses the same rounded P as the numerator.
//
// Decode: a split-key pass (one workgroup per (head, 2048 keys): scores,
// local maximum, exp, local sum, weighted value sum) and a combine pass that
// rescales the partial sums to the global maximum.  The new token's k and v
// are written into the cache at `pos` by the first split and taken from the
// inputs by the split that covers `pos`, so no workgroup reads a cache row
// written in the same step.
#include "tt_device.hpp"
#include "tt_internal.hpp"

namespace tt {
namespace {

constexpr int kSDV = 64;      // value columns
constexpr int kSQB = 64;      // queries per prefill workgroup
constexpr int kSKB = 64;      // keys per prefill block
constexpr int kSplit = 2048;  // keys per decode split
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline int srho(int tau, int i) { return 8 * (i >> 2) + 4 * tau + (i & 3); }

template <int DK>
struct SCfg {
  static constexpr int PADE = 8;                 // 16-byte row padding (bank spread)
  static constexpr int KS = DK + PADE;           // K tile row stride, bf16 elements
  static constexpr int VS = kSDV + PADE;         // V tile row stride
  static constexpr int B_K = kSKB * KS * 2;      // bytes of one K tile
  static constexpr int B_V = kSKB * VS * 2;      // bytes of one V tile
  static constexpr int LDS = 2 * (B_K + B_V);
  static constexpr int KSEG = kSKB * DK / 8;     // 16-byte segments of a K tile
  static constexpr int VSEG = kSKB * kSDV / 8;   // of a V tile
  static constexpr int NKS = (KSEG + 255) / 256;
  static constexpr int NVS = VSEG / 256;
  static_assert(VSEG % 256 == 0, "V segments per thread");
};

template <int DK>
__global__ __launch_bounds__(256) void softmax_prefill_kernel(const uint16_t* __restrict__ Qg,
                                                              const uint16_t* __restrict__ Kg,
                                                              const uint16_t* __restrict__ Vg, int BH, int N,
                                                              float* __restrict__ Og) {
  using C = SCfg<DK>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS];
  auto sK = [&](int b) { return lds + b * (C::B_K + C::B_V); };
  auto sV = [&](int b) { return lds + b * (C::B_K + C::B_V) + C::B_K; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nqb = (N + kSQB - 1) / kSQB;
  // Block -> (head, query block), heaviest query blocks of a head first.
  // Workgroups are dealt round-robin over the 8 XCDs; with BH a multiple of
  // 8 every block of one head lands on one XCD, whose L2 then serves that
  // head's K and V to all its query blocks.
  int bh, qb;
  {
    const int b = blockIdx.x;
    if (BH % 8 == 0) {
      const int x = b & 7, r = b >> 3;
      bh = x + 8 * (r / nqb);
      qb = nqb - 1 - r % nqb;
    } else {
      bh = b / nqb;
      qb = nqb - 1 - b % nqb;
    }
  }
  const int q0 = qb * kSQB;
  const uint16_t* Qh = Qg + (size_t)bh * N * DK;
  const uint16_t* Kh = Kg + (size_t)bh * N * DK;
  const uint16_t* Vh = Vg + (size_t)bh * N * kSDV;

  // this lane's query and its Q^T fragment (B operand of S^T = K Q^T)
  const int my_q = q0 + 16 * w + li;
  const size_t qrow = (size_t)min(my_q, N - 1);
  constexpr int XD = DK == 16 ? 1 : DK / 32;
  u32x4 qf[XD];
#pragma unroll
  for (int h = 0; h < XD; ++h) {
    if constexpr (DK == 16) {
      const uint2 a = *reinterpret_cast<const uint2*>(Qh + qrow * 16 + 4 * lg);
      qf[h] = u32x4{a.x, a.y, 0u, 0u};
    } else {
      qf[h] = *reinterpret_cast<const u32x4*>(Qh + qrow * DK + 32 * h + 8 * lg);
    }
  }

  // staging of one key block: global -> registers -> LDS (rows past N are
  // clamped to N-1; such keys exceed every valid query and are masked)
  u32x4 rk[C::NKS], rv[C::NVS];
  auto issue = [&](int kb) {
    const int k0 = kb * kSKB;
#pragma unroll
    for (int i = 0; i < C::NKS; ++i) {
      const int seg = tid + 256 * i;
      if (seg < C::KSEG) {
        const int tok = seg / (DK / 8), part = seg % (DK / 8);
        rk[i] = *reinterpret_cast<const u32x4*>(Kh + (size_t)min(k0 + tok, N - 1) * DK + part * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVS; ++i) {
      const int seg = tid + 256 * i;
      const int tok = seg >> 3, part = seg & 7;
      rv[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)min(k0 + tok, N - 1) * kSDV + part * 8);
    }
  };
  auto commit = [&](int b) {
    unsigned char* K = sK(b);
    unsigned char* V = sV(b);
#pragma unroll
    for (int i = 0; i < C::NKS; ++i) {
      const int seg = tid + 256 * i;
      if (seg < C::KSEG) {
        const int tok = seg / (DK / 8), part = seg % (DK / 8);
        *reinterpret_cast<u32x4*>(K + (tok * C::KS + part * 8) * 2) = rk[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVS; ++i) {
      const int seg = tid + 256 * i;
      const int tok = seg >> 3, part = seg & 7;
      *reinterpret_cast<u32x4*>(V + (tok * C::VS + part * 8) * 2) = rv[i];
    }
  };
  // V^T fragment (A operand of O^T += V^T P^T) for keys hb*32 .. hb*32+31 and
  // columns ct*16 .. ct*16+15, by two transposing reads of the token-major tile
  const int trow = 8 * lg + (li >> 2);
  auto load_vt = [&](const unsigned char* V, int hb, int ct) {
    const unsigned char* p = V + ((hb * 32 + trow) * C::VS + ct * 16 + 4 * (li & 3)) * 2;
    const uint2 a = lds_tr16(p), c = lds_tr16(p + 4 * C::VS * 2);
    return u32x4{a.x, a.y, c.x, c.y};
  };

  f32x4 o[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) o[ct] = zero4();
  float m = -__builtin_inff();  // running maximum (base 2), shared by the 4 lanes of a query
  float l = 0.f;                // this lane's part of the running sum

  const int nkb = qb + 1;
  issue(0);
  commit(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int b = kb & 1;
    if (kb + 1 < nkb) issue(kb + 1);
    const unsigned char* K = sK(b);
    const unsigned char* V = sV(b);
    const int k0 = kb * kSKB;
    const bool diag = kb == qb;

    // scores: x[hb][tau][s] = q_my . k_(k0 + hb*32 + 8*lg + 4*tau + s)
    float sc[2][2][4];
    float bmax = -__builtin_inff();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int arow = hb * 32 + srho(tau, li);
        f32x4 x = zero4();
        if constexpr (DK == 16) {
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          const uint2 a = *reinterpret_cast<const uint2*>(K + (arow * C::KS + 4 * lg) * 2);
          const uint2 bq = {qf[0].x, qf[0].y};
          x = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, bq),
                                                        x, 0, 0, 0);
        } else {
#pragma unroll
          for (int h = 0; h < XD; ++h) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(K + (arow * C::KS + 32 * h + 8 * lg) * 2);
            x = mfma_bf16(a, qf[h], x);
          }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int key = k0 + hb * 32 + 8 * lg + 4 * tau + s;
          const float v = (diag && key > my_q) ? -__builtin_inff() : x[s] * kLog2e;
          sc[hb][tau][s] = v;
          bmax = fmaxf(bmax, v);
        }
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m, bmax);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o[ct] *= alpha;

#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float p[8];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int s = 0; s < 4; ++s) p[4 * tau + s] = __builtin_amdgcn_exp2f(sc[hb][tau][s] - m);
      u32x4 ph, pl;
      if (diag) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t h2, l2;
          split_bf16x2(p[2 * e], p[2 * e + 1], h2, l2);
          ph[e] = h2;
          pl[e] = l2;
          l += __uint_as_float(h2 << 16) + __uint_as_float(l2 << 16);
          l += __uint_as_float(h2 & 0xFFFF0000u) + __uint_as_float(l2 & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ph[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
          l += __uint_as_float(ph[e] << 16) + __uint_as_float(ph[e] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const u32x4 a = load_vt(V, hb, ct);
        o[ct] = mfma_bf16(a, ph, o[ct]);
        if (diag) o[ct] = mfma_bf16(a, pl, o[ct]);
      }
    }
    if (kb + 1 < nkb) {
      commit(b ^ 1);
      __syncthreads();
    }
  }

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (my_q < N) {
    const float r = 1.0f / l;
    float* Orow = Og + ((size_t)bh * N + my_q) * kSDV;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x4 v = o[ct] * r;
      *reinterpret_cast<f32x4*>(Orow + ct * 16 + 4 * lg) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------

__device__ inline float block_reduce_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ inline float block_reduce_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// A row of D values (16-byte aligned) as fp32, by 16-byte loads.
template <int D, typename TIn>
__device__ inline void load_row(const TIn* p, float (&x)[D]) {
  constexpr int EPS = 16 / (int)sizeof(TIn);
#pragma unroll
  for (int i = 0; i < D / EPS; ++i) {
    const u32x4 seg = reinterpret_cast<const u32x4*>(p)[i];
#pragma unroll
    for (int e = 0; e < EPS; ++e) {
      if constexpr (sizeof(TIn) == 2)
        x[i * EPS + e] = __uint_as_float(e & 1 ? (seg[e >> 1] & 0xFFFF0000u) : (seg[e >> 1] << 16));
      else
        x[i * EPS + e] = __uint_as_float(seg[e]);
    }
  }
}

// One (head, split): keys [sp*kSplit, min(pos+1, (sp+1)*kSplit)).
// part[(bh*nsplit + sp)*(kSDV+2)] = {max (base 2), sum, acc[kSDV]}.
template <int DK, typename TIn>
__global__ __launch_bounds__(256) void softmax_decode_split(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                            const TIn* __restrict__ v, TIn* Kc, TIn* Vc, int pos,
                                                            int cap, float* __restrict__ part) {
  constexpr int R = kSplit / 256;
  __shared__ float s_q[DK], s_knew[DK];
  __shared__ float s_p[kSplit];
  __shared__ float s_red[4];
  __shared__ float s_acc[4][kSDV];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sp = blockIdx.x, nsplit = gridDim.x, bh = blockIdx.y;
  const int t0 = sp * kSplit;
  const int t1 = min(pos + 1, t0 + kSplit);
  TIn* Kh = Kc + (size_t)bh * cap * DK;
  TIn* Vh = Vc + (size_t)bh * cap * kSDV;
  if (tid < DK) {
    s_q[tid] = load_f32(q, (size_t)bh * DK + tid);
    s_knew[tid] = load_f32(k, (size_t)bh * DK + tid);
    if (sp == 0) Kh[(size_t)pos * DK + tid] = k[(size_t)bh * DK + tid];
  }
  const float vnew = load_f32(v, (size_t)bh * kSDV + lane);
  if (sp == 0 && w == 0) Vh[(size_t)pos * kSDV + lane] = v[(size_t)bh * kSDV + lane];
  __syncthreads();

  float sc[R];
  float mx = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + tid + 256 * r;
    float d = -__builtin_inff();
    if (t < t1) {
      d = 0.f;
      if (t == pos) {
#pragma unroll
        for (int i = 0; i < DK; ++i) d = fmaf(s_q[i], s_knew[i], d);
      } else {
        float kr[DK];
        load_row<DK, TIn>(Kh + (size_t)t * DK, kr);
#pragma unroll
        for (int i = 0; i < DK; ++i) d = fmaf(s_q[i], kr[i], d);
      }
      d *= kLog2e;
    }
    sc[r] = d;
    mx = fmaxf(mx, d);
  }
  mx = block_reduce_max(mx, s_red);
  float ls = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float p = __builtin_amdgcn_exp2f(sc[r] - mx);  // 0 for keys past t1
    s_p[tid + 256 * r] = p;
    ls += p;
  }
  ls = block_reduce_sum(ls, s_red);  // its barriers also publish s_p

  // weighted values: wave w takes keys t0 + w, t0 + w + 4, ...; lane = column
  const int nk = t1 - t0;
  float acc = 0.f;
  int j = w;
  for (; j + 4 * 7 < nk; j += 4 * 8) {
    float vv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + j + 4 * u;
      vv[u] = (t == pos) ? vnew : load_f32(Vh, (size_t)t * kSDV + lane);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = fmaf(s_p[j + 4 * u], vv[u], acc);
  }
  for (; j < nk; j += 4) {
    const int t = t0 + j;
    acc = fmaf(s_p[j], (t == pos) ? vnew : load_f32(Vh, (size_t)t * kSDV + lane), acc);
  }
  s_acc[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    float* dst = part + ((size_t)bh * nsplit + sp) * (kSDV + 2);
    dst[2 + lane] = (s_acc[0][lane] + s_acc[1][lane]) + (s_acc[2][lane] + s_acc[3][lane]);
    if (lane == 0) {
      dst[0] = mx;
      dst[1] = ls;
    }
  }
}

// o = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s; one wave per head.
__global__ __launch_bounds__(64) void softmax_decode_combine(const float* __restrict__ part, int nsplit,
                                                             float* __restrict__ o) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const float* P = part + (size_t)bh * nsplit * (kSDV + 2);
  float M = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, P[(size_t)s * (kSDV + 2)]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float f = __builtin_amdgcn_exp2f(P[(size_t)s * (kSDV + 2)] - M);
    L = fmaf(P[(size_t)s * (kSDV + 2) + 1], f, L);
    acc = fmaf(P[(size_t)s * (kSDV + 2) + 2 + lane], f, acc);
  }
  o[(size_t)bh * kSDV + lane] = acc / L;
}

}  // namespace

size_t softmax_decode_splits(int pos) { return (size_t)pos / kSplit + 1; }

hipError_t launch_softmax_prefill(const void* Q, const void* K, const void* V, int BH, int N, int dk, float* O,
                                  hipStream_t s) {
  const int nqb = (N + kSQB - 1) / kSQB;
  const dim3 grid((unsigned)(BH * nqb));
  if (dk == 16)
    hipLaunchKernelGGL(softmax_prefill_kernel<16>, grid, dim3(256), 0, s, (const uint16_t*)Q, (const uint16_t*)K,
                       (const uint16_t*)V, BH, N, O);
  else if (dk == 32)
    hipLaunchKernelGGL(softmax_prefill_kernel<32>, grid, dim3(256), 0, s, (const uint16_t*)Q, (const uint16_t*)K,
                       (const uint16_t*)V, BH, N, O);
  else
    hipLaunchKernelGGL(softmax_prefill_kernel<64>, grid, dim3(256), 0, s, (const uint16_t*)Q, (const uint16_t*)K,
                       (const uint16_t*)V, BH, N, O);
  return hipGetLastError();
}

hipError_t launch_softmax_decode(const void* q, const void* k, const void* v, tt_dtype dt, int BH, int dk,
                                 void* Kc, void* Vc, int pos, int cap, float* o, float* part, hipStream_t s) {
  const int nsplit = (int)softmax_decode_splits(pos);
  const dim3 grid((unsigned)nsplit, (unsigned)BH);
#define TT_SDEC(D, T)                                                                                          \
  hipLaunchKernelGGL((softmax_decode_split<D, T>), grid, dim3(256), 0, s, (const T*)q, (const T*)k, (const T*)v, \
                     (T*)Kc, (T*)Vc, pos, cap, part)
  if (dt == TT_F32) {
    if (dk == 16) TT_SDEC(16, float);
    else if (dk == 32) TT_SDEC(32, float);
    else TT_SDEC(64, float);
  } else {
    if (dk == 16) TT_SDEC(16, uint16_t);
    else if (dk == 32) TT_SDEC(32, uint16_t);
    else TT_SDEC(64, uint16_t);
  }
#undef TT_SDEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(softmax_decode_combine, dim3((unsigned)BH), dim3(64), 0, s, part, nsplit, o);
  return hipGetLastError();
}

}  // namespace tt
