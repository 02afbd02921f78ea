// Prefill for large feature sets with bf16 inputs (n = 3, dk = 32 and 64:
// 561 and 2,145 rows, octet order inside the library): the output pass reads
// the state instead of carrying it.
//
// "Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
// with a Fixed Number of Recurrent States" (abstract): states of disjoint
// token sets add, so the output of query i in span s splits into the readout
// of the state of all spans before s and the quadratic form over the keys of
// span s up to i (comment thread on the paper, item 46888355: (Q'K)V = Q'(KV)
// for everything but the span's own causal block):
//
//   num/den(i) = phi(q_i).S_prefix(s) + sum_{span start <= j <= i} K_n(q_i.k_j) [v_j, 1]
//
// Three launches:
//   1. stream_totals_kernel: the state of each span of kStL tokens (hi + lo
//      bf16 mu, exact products, fp32 accumulation);
//   2. stream_scan_kernel: exclusive prefix over spans, in place, rewritten
//      as MFMA operand fragments (the prefix shifted by its column means,
//      bf16; normaliser rows hi + lo bf16); the sum over all spans is the
//      final state, written in feature order;
//   3. stream_out_kernel: one workgroup per 128 queries.  Phase A is the
//      in-span causal block, flash-style (S^T = K Q^T and O^T += V^T P^T on
//      MFMA, P = K_n(S) in registers, hi + lo bf16 on the diagonal block);
//      phase B is the readout GEMM phi(Q) S_prefix over all feature rows,
//      with phi generated per 32-row block into LDS and the state fragments
//      streamed from the workspace (L2); the two are added and divided.
// No state update runs in the output pass and no row-group partial outputs
// exist; the workspace holds one state per (head, span).
#pragma once

#include "tt_prefill_kernels.hpp"

namespace tt {
namespace {

constexpr int kStL = 1024;  // tokens per span
constexpr int kStQ = 128;   // queries per output workgroup
constexpr int kStK = 64;    // keys per key block of the in-span causal block
constexpr int kStT = kStL / kStQ;  // output workgroups per span

// x_a * x[b], x_a * x[b+1] for a packed bf16 pair {x[b], x[b+1]}: a bf16
// dot product with one zero term is the exact product (16 significant bits)
// in fp32.  The 3-operand form with an inline zero accumulator; the
// compiler's choice for the builtin is the 2-operand form, which needs a
// zeroed destination register per product.
__device__ inline void prod_pair(uint32_t xa_lo, uint32_t xa_hi, uint32_t pair, float& p0, float& p1) {
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(p0) : "v"(xa_lo), "v"(pair));
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(p1) : "v"(xa_hi), "v"(pair));
}

template <int DK>
struct StCfg {
  static constexpr int W = oct_rows(DK);  // internal rows (octets)
  static constexpr int NO = W / 8;
  static constexpr int NKB = (W + 31) / 32;  // 32-row blocks of the readout
  static constexpr int XD = DK / 32;         // 32-coordinate pieces of a q or k row
  static constexpr int KS = DK + 8;          // K and Q tile row stride (bf16)
  static constexpr int VS = kDV + 8;         // V tile row stride
  static constexpr int PHS = 32 + 8;         // phi tile row stride: one 32-row block
  static constexpr int B_K = kStK * KS * 2, B_V = kStK * VS * 2;
  static constexpr int LDS_A = 2 * (B_K + B_V);             // phase A: K, V double-buffered
  static constexpr int B_Q = kStQ * KS * 2, B_PHI = kStQ * PHS * 2;
  static constexpr int LDS_B = B_Q + 2 * B_PHI;             // phase B: Q tile, phi double-buffered
  static constexpr int OXS = kDV + 4;                       // exchange row stride (floats)
  // exchange: numerators, normalisers, and the hi half of the normaliser readout
  static constexpr int LDS_X = (kStQ * OXS + 2 * kStQ) * 4;
  static constexpr int LDS = LDS_A > LDS_B ? (LDS_A > LDS_X ? LDS_A : LDS_X) : (LDS_B > LDS_X ? LDS_B : LDS_X);
  static constexpr int KSEG = kStK * DK / 8, VSEG = kStK * kDV / 8, QSEG = kStQ * DK / 8;
  static constexpr int NKS = KSEG / 256, NVS = VSEG / 256, NQS = QSEG / 256;
  static_assert(KSEG % 256 == 0 && VSEG % 256 == 0 && QSEG % 256 == 0, "16-byte segments per thread");
};

// ---------------------------------------------------------------------------
// Fragment layout of a prefix state in the workspace.  The span state of
// (head, span) is [WP][64] fp32 values, then [WP] fp32 normalisers (the
// totals pass writes it so).  The scan rewrites the 32 x 16 region of rows
// 32j .. 32j+31 and columns 16ct .. 16ct+15 as the A operand of the readout
// MFMA (S^T: lane (i, g) holds rows 32j + 8g .. 8g+7 of column 16ct + i),
// 16 bytes per lane: lane l's piece sits in row 32j + l/4 at columns
// 16ct + 4(l%4) .. +3 (piece h = 1, rows 32j + 16 .. 31, is unused; row 16
// of block 0 holds the column means of the readout shift, in fp32).
// Normaliser rows 32j .. 32j+31 become eight hi bf16 then eight lo bf16 per
// group g of 8 rows (the same for every lane of the group).
// ---------------------------------------------------------------------------
__device__ inline size_t st_frag_off(int j, int ct, int l, int h) {
  return (size_t)(32 * j + 16 * h + (l >> 2)) * kDV + 16 * ct + 4 * (l & 3);
}
__device__ inline size_t st_den_off(int WP, int j, int g, int h) {
  return (size_t)WP * kDV + 32 * j + 8 * g + 4 * h;
}

// Span totals: one workgroup of 4 waves per (head, span, 128 feature rows);
// wave w owns the 32-row block j = 4*rb + w for all 64 value columns (eight
// accumulator tiles) and its normaliser.  Per 64-token block the waves stage
// K and V in LDS; each wave then builds the mu rows of its own block (lane =
// token, one octet at a time, hi + lo bf16: a product of two bf16 values is
// exact in fp32 and splits exactly into two bf16) into a wave-private tile
// and contracts them with V by MFMA, so no workgroup barrier separates the
// features from their use.  The mu tile is token-major with the chunk
// swizzle and row shift of the pipe kernel (conflict-free transposing reads).
template <int DK>
struct StTot {
  static constexpr int NW = 4;
  static constexpr int KS = DK + 8;                    // K tile row stride (bf16)
  static constexpr int VS = kDV + 8;                   // V tile row stride
  static constexpr int MUS = 32, MUSH = 4;             // mu rows: 32 elements, +4 every 8 tokens
  static constexpr int MUPL = kStK * MUS + 32;         // elements per mu plane (with the shift's slack)
  static constexpr int B_K = kStK * KS * 2, B_V = kStK * VS * 2;
  static constexpr int B_MU = 2 * MUPL * 2;            // hi and lo planes of one wave
  // one K/V buffer (51.6 KB at dk = 64): three workgroups fit a CU's 160 KB,
  // whose other waves cover the second barrier per token block
  static constexpr int LDS = (B_K + B_V) + NW * B_MU;
  static constexpr int KSEG = kStK * DK / 8, VSEG = kStK * kDV / 8;
  static constexpr int NKS = (KSEG + NW * 64 - 1) / (NW * 64), NVS = VSEG / (NW * 64);
  static constexpr int NRB = (StCfg<DK>::NKB + NW - 1) / NW;  // 256-row groups
  static constexpr int WP = NRB * NW * 32;                     // padded rows of a span state
  // first row past the readout's blocks: a copy of row 0 and of its
  // normaliser, which the scan rewrites nowhere (every scan workgroup reads it)
  static constexpr int R0COPY = StCfg<DK>::NKB * 32;
  static_assert(R0COPY < WP, "a spare row for the copy of row 0");
  static_assert(VSEG % (NW * 64) == 0, "V segments per thread");
};

template <int DK>
__global__ __launch_bounds__(256, 3) void stream_totals_kernel(const uint16_t* __restrict__ Kg,
                                                            const uint16_t* __restrict__ Vg, int BH, int N,
                                                            int nspan, float* __restrict__ ws) {
  using C = StTot<DK>;
  constexpr int NKB = StCfg<DK>::NKB, NO = StCfg<DK>::NO;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  // block -> (head, span, row group): the row groups of a span share
  // blockIdx % 8 (one XCD, whose L2 then serves the span's K and V to all)
  const int b = blockIdx.x;
  const int rb = (b >> 3) % C::NRB;
  const int hs = (b / (8 * C::NRB)) * 8 + (b & 7);
  if (hs >= BH * nspan) return;
  const int bh = hs / nspan, s = hs % nspan;
  const int t_begin = s * kStL, t_end = min(N, t_begin + kStL);
  const int ntb = (t_end - t_begin + kStK - 1) / kStK;
  const int j = rb * C::NW + w;       // this wave's 32-row block
  const bool active = j < NKB;        // wave-uniform; blocks past the last octet hold zero rows
  const uint16_t* Kh = Kg + (size_t)bh * N * DK;
  const uint16_t* Vh = Vg + (size_t)bh * N * kDV;
  auto sK = [&](int) { return lds; };
  auto sV = [&](int) { return lds + C::B_K; };
  uint16_t* sMu = reinterpret_cast<uint16_t*>(lds + (C::B_K + C::B_V) + w * C::B_MU);

  u32x4 rk[C::NKS], rv[C::NVS];
  auto issue = [&](int tb) {  // rows past the span end are clamped to its last token (their mu is zero)
    const int k0 = t_begin + tb * kStK;
#pragma unroll
    for (int i = 0; i < C::NKS; ++i) {
      const int seg = tid + C::NW * 64 * i;
      if (seg < C::KSEG) {
        const int tok = seg / (DK / 8), part = seg % (DK / 8);
        rk[i] = *reinterpret_cast<const u32x4*>(Kh + (size_t)min(k0 + tok, t_end - 1) * DK + part * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVS; ++i) {
      const int seg = tid + C::NW * 64 * i, tok = seg >> 3, part = seg & 7;
      rv[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)min(k0 + tok, t_end - 1) * kDV + part * 8);
    }
  };
  // K rows of tokens past the span end are stored as zeros, so their mu rows
  // of order 1 and 2 vanish; the order-0 row is masked where it is built
  auto commit = [&](int buf, int tb) {
    const int k0 = t_begin + tb * kStK;
#pragma unroll
    for (int i = 0; i < C::NKS; ++i) {
      const int seg = tid + C::NW * 64 * i;
      if (seg < C::KSEG) {
        const int tok = seg / (DK / 8), part = seg % (DK / 8);
        *reinterpret_cast<u32x4*>(sK(buf) + (tok * C::KS + part * 8) * 2) =
            k0 + tok < t_end ? rk[i] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVS; ++i) {
      const int seg = tid + C::NW * 64 * i, tok = seg >> 3, part = seg & 7;
      *reinterpret_cast<u32x4*>(sV(buf) + (tok * C::VS + part * 8) * 2) = rv[i];
    }
  };

  f32x4 st[2][4], dn[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    dn[t] = zero4();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) st[t][ct] = zero4();
  }
  const u32x4 ones_bf = (li == 0) ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                                  : u32x4{0u, 0u, 0u, 0u};
  const uint32_t* tab = OctOf<DK>::get().d;
  // this lane's token row in the mu tile; chunk c of it sits at c ^ mswz
  const int mswz = (lane >> 2) & 3;
  uint16_t* muRow = sMu + lane * C::MUS + C::MUSH * (lane >> 3);
  // transposing-read addresses (see the pipe kernel): token 8*lg + li/4 (+4)
  // of a 32-token half, chunks (li & 3) ^ z
  const int trow = 8 * lg + (li >> 2);
  const int cz0 = (li & 3) ^ ((2 * lg) & 3);
  const int cz1 = (li & 3) ^ ((2 * lg + 1) & 3);
  auto load_mu = [&](int pl, int tau, int th) {
    const unsigned char* r0 = reinterpret_cast<const unsigned char*>(sMu) +
                              (pl * C::MUPL + (th * 32 + trow) * C::MUS + C::MUSH * (4 * th + lg) + 4 * tau) * 2;
    const uint2 a = lds_tr16(r0 + cz0 * 16);
    const uint2 c = lds_tr16(r0 + 4 * C::MUS * 2 + cz1 * 16);
    return u32x4{a.x, a.y, c.x, c.y};
  };
  auto load_v = [&](const unsigned char* V, int th, int ct) {
    const unsigned char* p = V + ((th * 32 + trow) * C::VS + ct * 16 + 4 * (li & 3)) * 2;
    const uint2 a = lds_tr16(p), c = lds_tr16(p + 4 * C::VS * 2);
    return u32x4{a.x, a.y, c.x, c.y};
  };

  // the wave's four octet descriptors, decoded once (wave-uniform): when all
  // four are order-2 octets (every wave but the first two), the block loop
  // issues the LDS reads of all four together and builds them without
  // per-octet table loads or branches on the order
  int om[4], oa[4], ob[4];
  uint32_t omask[4][4];  // diagonal octets: the pairs of x[b0 ..] with b < a cleared
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int o = 4 * j + c;
    const uint32_t d = (active && o < NO) ? tab[o] : 0xFFu;
    om[c] = __builtin_amdgcn_readfirstlane((int)(d & 0xFF));
    oa[c] = __builtin_amdgcn_readfirstlane((int)((d >> 8) & 0xFF));
    ob[c] = __builtin_amdgcn_readfirstlane((int)(d >> 16));
#pragma unroll
    for (int e = 0; e < 4; ++e)
      omask[c][e] = (ob[c] + 2 * e >= oa[c] ? 0x0000FFFFu : 0u) | (ob[c] + 2 * e + 1 >= oa[c] ? 0xFFFF0000u : 0u);
  }
  const bool all2 = om[0] == 2 && om[1] == 2 && om[2] == 2 && om[3] == 2;
  // hi and lo planes of one octet's eight products, to this lane's token row
  auto put_octet = [&](int c, const float* mu) {
    uint32_t hb[8], lb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      hb[u] = __float_as_uint(mu[u]) & 0xFFFF0000u;
      lb[u] = __float_as_uint(mu[u] - __uint_as_float(hb[u]));
    }
    uint16_t* dst = muRow + 8 * (c ^ mswz);
    reinterpret_cast<uint2*>(dst)[0] = uint2{__builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u),
                                             __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u)};
    reinterpret_cast<uint2*>(dst)[1] = uint2{__builtin_amdgcn_perm(hb[5], hb[4], 0x07060302u),
                                             __builtin_amdgcn_perm(hb[7], hb[6], 0x07060302u)};
    reinterpret_cast<uint2*>(dst + C::MUPL)[0] = uint2{__builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u),
                                                       __builtin_amdgcn_perm(lb[3], lb[2], 0x07060302u)};
    reinterpret_cast<uint2*>(dst + C::MUPL)[1] = uint2{__builtin_amdgcn_perm(lb[5], lb[4], 0x07060302u),
                                                       __builtin_amdgcn_perm(lb[7], lb[6], 0x07060302u)};
  };

  issue(0);
  commit(0, 0);
  __syncthreads();
  for (int tb = 0; tb < ntb; ++tb) {
    const int buf = tb & 1;
    if (tb + 1 < ntb) issue(tb + 1);
    if (active && all2) {
      const uint16_t* x = reinterpret_cast<const uint16_t*>(sK(buf)) + lane * C::KS;
      uint32_t xa[4];
      u32x4 xb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        xa[c] = x[oa[c]];
        xb[c] = *reinterpret_cast<const u32x4*>(x + ob[c]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (ob[c] <= oa[c]) {  // the octet holding (a, a): rows b < a are zero
#pragma unroll
          for (int e = 0; e < 4; ++e) xb[c][e] &= omask[c][e];
        }
        float mu[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) prod_pair(xa[c], xa[c] << 16, xb[c][e], mu[2 * e], mu[2 * e + 1]);
        put_octet(c, mu);
      }
    } else if (active) {
      const uint16_t* x = reinterpret_cast<const uint16_t*>(sK(buf)) + lane * C::KS;
      const bool kvalid = t_begin + tb * kStK + lane < t_end;  // tokens past the span end: zero rows
      // mu rows of octets 4j .. 4j+3 for this lane's token, hi and lo planes
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int o = 4 * j + c;
        const uint32_t d = o < NO ? tab[o] : 0xFFu;  // wave-uniform
        const int m = d & 0xFF, a = (d >> 8) & 0xFF, b0 = (int)(d >> 16);
        float mu[8];
        if (m == 2) {
          const uint32_t xa = x[a];  // {x_a, 0}; shifted: {0, x_a}
          const u32x4 xb = *reinterpret_cast<const u32x4*>(x + b0);
#pragma unroll
          for (int e = 0; e < 4; ++e) prod_pair(xa, xa << 16, xb[e], mu[2 * e], mu[2 * e + 1]);
          if (b0 <= a) {  // the octet holding (a, a): rows b < a are zero
#pragma unroll
            for (int u = 0; u < 8; ++u) mu[u] = b0 + u >= a ? mu[u] : 0.f;
          }
        } else if (m == 1) {
          const u32x4 xb = *reinterpret_cast<const u32x4*>(x + b0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mu[2 * e] = __uint_as_float(xb[e] << 16);
            mu[2 * e + 1] = __uint_as_float(xb[e] & 0xFFFF0000u);
          }
        } else {  // order 0 (row 0: the token count) or past the last octet
#pragma unroll
          for (int u = 0; u < 8; ++u) mu[u] = (m == 0 && u == 0 && kvalid) ? 1.f : 0.f;
        }
        put_octet(c, mu);
      }
    }
    if (active) {
      // the tile is wave-private: this wave's LDS writes done, then its reads
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const unsigned char* V = sV(buf);
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        u32x4 vf[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) vf[ct] = load_v(V, th, ct);
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int pl = 0; pl < 2; ++pl) {
            const u32x4 af = load_mu(pl, tau, th);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) st[tau][ct] = mfma_bf16(af, vf[ct], st[tau][ct]);
            dn[tau] = mfma_bf16(af, ones_bf, dn[tau]);
          }
      }
    }
    if (tb + 1 < ntb) {
      __syncthreads();  // every wave's reads of the K and V tiles done
      commit(buf ^ 1, tb + 1);
      __syncthreads();
    }
  }
  if (!active) return;
  float* S = ws + (size_t)hs * C::WP * (kDV + 1);
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 32 * j + 8 * lg + 4 * tau + e;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) S[(size_t)row * kDV + 16 * ct + li] = st[tau][ct][e];
      if (li == 0) S[(size_t)C::WP * kDV + row] = dn[tau][e];
      if (row == 0) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) S[(size_t)C::R0COPY * kDV + 16 * ct + li] = st[tau][ct][e];
        if (li == 0) S[(size_t)C::WP * kDV + C::R0COPY] = dn[tau][e];
      }
    }
}

// Exclusive scan over spans, in place, into fragments; final states (feature
// order, plane layout), starting from `init` (plane layout, or null).  One
// workgroup per (head, 32-row block), wave = column tile; lanes li == 0 of
// wave 0 also write the block's normaliser fragments (group lg).
//
// The value fragment of each prefix is the state shifted by the running mean
// of its column: with Z the normaliser rows, Zh their hi bf16 plane and a_c
// the bf16 rounding of S[0][c] / Z[0] (0 when that is not finite), the
// fragment holds S[r][c] - a_c Zh[r] rounded to bf16.  The readout adds
// a_c (phi . Zh) back (the hi half of its normaliser readout), so
//   phi . S = phi . (S - a Zh) + a (phi . Zh)
// holds for any a_c, and rounding the fragment to bf16 moves an output by
// about 2^-9 |v - a| rather than 2^-9 |v|.  a_c Zh[r] is exact in fp32 (two
// bf16 factors), so the difference is one fp32 rounding of the exact value.
// Every workgroup scans row 0 and Z[0] itself, from the copy the totals pass
// leaves in row StTot::R0COPY (the same additions in the same order, so the
// same a_c); block 0's writes a_c into row 16 of the span's region, which
// the hi-only fragments leave free.
// The workgroup reads the elements whose fragments it writes, at other
// addresses of the same region (the normaliser rows by every wave); a
// barrier after the reads of a group of spans orders them before the
// group's writes.
template <int DK>
__global__ __launch_bounds__(256) void stream_scan_kernel(float* ws, int nspan, int WP, int BH, int W,
                                                          const float* init, float* states, int bh0, int BHtot) {
  using C = StCfg<DK>;
  const int bh = blockIdx.x / C::NKB, j = blockIdx.x % C::NKB;
  // init and states hold BHtot heads (plane layout); this launch scans heads
  // bh0 .. bh0 + BH - 1 of them, whose span states the workspace holds
  const size_t gh = (size_t)bh0 + bh;
  const int lane = threadIdx.x & 63, ct = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const bool den_lane = ct == 0 && li == 0;
  const size_t per = (size_t)WP * (kDV + 1);
  float* base = ws + (size_t)bh * nspan * per;
  const int col = 16 * ct + li;
  int ra[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) ra[u] = abi_row<DK>(32 * j + 8 * lg + u);
  const int r0 = abi_row<DK>(0);
  float run[8], runz[8], run0 = 0.f, runz0 = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    run[u] = (init != nullptr && ra[u] >= 0) ? init[(gh * W + ra[u]) * kDV + col] : 0.f;
    runz[u] = (init != nullptr && ra[u] >= 0) ? init[(size_t)BHtot * W * kDV + gh * W + ra[u]] : 0.f;
  }
  if (init != nullptr) {
    run0 = init[(gh * W + r0) * kDV + col];
    runz0 = init[(size_t)BHtot * W * kDV + gh * W + r0];
  }
  constexpr int G = 4;  // spans whose loads are in flight together
  for (int s0 = 0; s0 < nspan; s0 += G) {
    float t[G][8], tz[G][8], t0[G], tz0[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (s0 + g < nspan) {
        const float* p = base + (size_t)(s0 + g) * per;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          t[g][u] = p[(size_t)(32 * j + 8 * lg + u) * kDV + col];
          tz[g][u] = p[(size_t)WP * kDV + 32 * j + 8 * lg + u];
        }
        t0[g] = p[(size_t)StTot<DK>::R0COPY * kDV + col];
        tz0[g] = p[(size_t)WP * kDV + StTot<DK>::R0COPY];
      }
    }
    // every read of these spans, by every wave, has returned before any
    // fragment is written
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (s0 + g < nspan) {
        float* p = base + (size_t)(s0 + g) * per;
        u32x4 zhi, zlo;
        split_bf16x8(f32x4{runz[0], runz[1], runz[2], runz[3]}, f32x4{runz[4], runz[5], runz[6], runz[7]}, zhi, zlo);
        const float rz0 = runz0 > 0.f ? 1.0f / runz0 : 0.f;
        uint32_t abits = pack_bf16x2(run0 * rz0, 0.f) & 0xFFFFu;
        if ((abits & 0x7F80u) == 0x7F80u) abits = 0u;
        const float a = __uint_as_float(abits << 16);
        float sh[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sh[2 * e] = __builtin_fmaf(-a, __uint_as_float(zhi[e] << 16), run[2 * e]);
          sh[2 * e + 1] = __builtin_fmaf(-a, __uint_as_float(zhi[e] & 0xFFFF0000u), run[2 * e + 1]);
        }
        *reinterpret_cast<u32x4*>(p + st_frag_off(j, ct, lane, 0)) =
            u32x4{pack_bf16x2(sh[0], sh[1]), pack_bf16x2(sh[2], sh[3]), pack_bf16x2(sh[4], sh[5]),
                  pack_bf16x2(sh[6], sh[7])};
        if (j == 0 && lg == 0) p[16 * kDV + col] = a;
        if (den_lane) {
          *reinterpret_cast<u32x4*>(p + st_den_off(WP, j, lg, 0)) = zhi;
          *reinterpret_cast<u32x4*>(p + st_den_off(WP, j, lg, 1)) = zlo;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          run[u] += t[g][u];
          runz[u] += tz[g][u];
        }
        run0 += t0[g];
        runz0 += tz0[g];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (ra[u] >= 0) states[(gh * W + ra[u]) * kDV + col] = run[u];
    if (den_lane && ra[u] >= 0) states[(size_t)BHtot * W * kDV + gh * W + ra[u]] = runz[u];
  }
}

// Output pass: one workgroup of 4 waves per 128 queries of a span.
template <int DK, bool UNN>
__global__ __launch_bounds__(256, 3) void stream_out_kernel(const uint16_t* __restrict__ Qg,
                                                         const uint16_t* __restrict__ Kg,
                                                         const uint16_t* __restrict__ Vg, int BH, int N, int nspan,
                                                         int WP, const float* __restrict__ ws, bool has_init,
                                                         float* __restrict__ Og, float* __restrict__ Dg) {
  using C = StCfg<DK>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  // block -> (head, span, tile): the kStT tiles of a span share blockIdx % 8,
  // so they are dealt to one XCD and its L2 serves the span's prefix state to
  // all of them; within a span the tiles with the longest causal block come
  // first
  const int b = blockIdx.x;
  const int sg = (b / (8 * kStT)) * 8 + (b & 7);
  const int tile = kStT - 1 - (b >> 3) % kStT;
  if (sg >= BH * nspan) return;
  const int bh = sg / nspan, s = sg % nspan;
  const int q0 = s * kStL + tile * kStQ;
  if (q0 >= N) return;
  const uint16_t* Qh = Qg + (size_t)bh * N * DK;
  const uint16_t* Kh = Kg + (size_t)bh * N * DK;
  const uint16_t* Vh = Vg + (size_t)bh * N * kDV;

  // ---------------- phase A: the span's causal block ----------------
  // wave w owns queries q0 + 32w .. +31 (two 16-query tiles) and all 64
  // value columns as O^T tiles (columns x queries)
  const int qw0 = q0 + 32 * w;
  u32x4 qf[2][C::XD];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int h = 0; h < C::XD; ++h)
      qf[qt][h] = *reinterpret_cast<const u32x4*>(Qh + (size_t)min(qw0 + 16 * qt + li, N - 1) * DK + 32 * h + 8 * lg);
  f32x4 oA[2][4], dA[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    dA[qt] = zero4();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) oA[qt][ct] = zero4();
  }
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  {
    auto sK = [&](int buf) { return lds + buf * (C::B_K + C::B_V); };
    auto sV = [&](int buf) { return lds + buf * (C::B_K + C::B_V) + C::B_K; };
    const int kbeg = s * kStL;
    const int kend = min(q0 + kStQ, N);
    const int nkb = (kend - kbeg + kStK - 1) / kStK;
    u32x4 rk[C::NKS], rv[C::NVS];
    auto issue = [&](int kb) {  // rows past N are clamped (such keys exceed every valid query: masked)
      const int k0 = kbeg + kb * kStK;
#pragma unroll
      for (int i = 0; i < C::NKS; ++i) {
        const int seg = tid + 256 * i, tok = seg / (DK / 8), part = seg % (DK / 8);
        rk[i] = *reinterpret_cast<const u32x4*>(Kh + (size_t)min(k0 + tok, N - 1) * DK + part * 8);
      }
#pragma unroll
      for (int i = 0; i < C::NVS; ++i) {
        const int seg = tid + 256 * i, tok = seg >> 3, part = seg & 7;
        rv[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)min(k0 + tok, N - 1) * kDV + part * 8);
      }
    };
    auto commit = [&](int buf) {
#pragma unroll
      for (int i = 0; i < C::NKS; ++i) {
        const int seg = tid + 256 * i, tok = seg / (DK / 8), part = seg % (DK / 8);
        *reinterpret_cast<u32x4*>(sK(buf) + (tok * C::KS + part * 8) * 2) = rk[i];
      }
#pragma unroll
      for (int i = 0; i < C::NVS; ++i) {
        const int seg = tid + 256 * i, tok = seg >> 3, part = seg & 7;
        *reinterpret_cast<u32x4*>(sV(buf) + (tok * C::VS + part * 8) * 2) = rv[i];
      }
    };
    // V^T fragment (A operand of O^T += V^T P^T), keys hb*32 .. +31, columns ct*16 .. +15
    const int trow = 8 * lg + (li >> 2);
    auto load_vt = [&](const unsigned char* V, int hb, int ct) {
      const unsigned char* p = V + ((hb * 32 + trow) * C::VS + ct * 16 + 4 * (li & 3)) * 2;
      const uint2 a = lds_tr16(p), c = lds_tr16(p + 4 * C::VS * 2);
      return u32x4{a.x, a.y, c.x, c.y};
    };
    issue(0);
    commit(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
      const int buf = kb & 1;
      if (kb + 1 < nkb) issue(kb + 1);
      const int k0 = kbeg + kb * kStK;
      if (k0 <= qw0 + 31) {  // some key of the block reaches a query of this wave (wave-uniform)
        const bool diag = k0 + kStK - 1 > qw0;  // keys after the wave's first query: mask, hi + lo P
        const unsigned char* K = sK(buf);
        const unsigned char* V = sV(buf);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          // P^T fragments (B operand): lane (query i, g) holds keys hb*32 + 8g .. +7
          u32x4 ph[2], pl[2];
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            float p[8];
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
              const int arow = hb * 32 + rho(tau, li);
              f32x4 x = zero4();
#pragma unroll
              for (int h = 0; h < C::XD; ++h) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(K + (arow * C::KS + 32 * h + 8 * lg) * 2);
                x = mfma_bf16(a, qf[qt][h], x);
              }
              const int query = qw0 + 16 * qt + li;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int key = k0 + hb * 32 + 8 * lg + 4 * tau + e;
                const float v = taylor_poly<3>(x[e]);
                p[4 * tau + e] = (diag && key > query) ? 0.f : v;
              }
            }
            if (diag) {
              uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
              split_bf16x2(p[0], p[1], h0, l0);
              split_bf16x2(p[2], p[3], h1, l1);
              split_bf16x2(p[4], p[5], h2, l2);
              split_bf16x2(p[6], p[7], h3, l3);
              ph[qt] = u32x4{h0, h1, h2, h3};
              pl[qt] = u32x4{l0, l1, l2, l3};
            } else {
              ph[qt] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                             pack_bf16x2(p[6], p[7])};
              pl[qt] = u32x4{0u, 0u, 0u, 0u};
            }
            // normaliser: every row of ones^T P^T is the column sum, the same P as the numerator
            dA[qt] = mfma_bf16(ones, ph[qt], dA[qt]);
            if (diag) dA[qt] = mfma_bf16(ones, pl[qt], dA[qt]);
          }
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const u32x4 a = load_vt(V, hb, ct);
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
              oA[qt][ct] = mfma_bf16(a, ph[qt], oA[qt][ct]);
              if (diag) oA[qt][ct] = mfma_bf16(a, pl[qt], oA[qt][ct]);
            }
          }
        }
      }
      if (kb + 1 < nkb) {
        commit(buf ^ 1);
        __syncthreads();
      }
    }
  }
  __syncthreads();  // phase A's tiles are free

  // ---------------- phase B: readout of the prefix state ----------------
  // wave w owns value columns 16w .. 16w+15 of all 128 queries (eight O^T
  // tiles) and the normalisers of query tiles 2w, 2w+1, from the hi and lo
  // planes of the normaliser rows (dC).  The value fragments are the state
  // shifted by a_c Zh (see stream_scan_kernel); a_c (phi . Zh), with phi . Zh
  // the hi half of dC, is added back in the combine.
  // dC[k]: the normaliser readout of query tile 2w + k, hi plane in rows 0-7
  // of the product (lanes lg < 2) and lo plane in rows 8-15 (lanes lg >= 2):
  // the A operand's rows all repeat the normaliser rows, so rows 8-15 carry
  // the lo plane and one MFMA reads out both planes
  f32x4 nB[8], dC[2];
#pragma unroll
  for (int qt = 0; qt < 8; ++qt) nB[qt] = zero4();
  dC[0] = dC[1] = zero4();
  const bool has_prefix = s > 0 || has_init;
  if (has_prefix) {
    uint16_t* sQ = reinterpret_cast<uint16_t*>(lds);
    auto sPhi = [&](int buf) { return reinterpret_cast<uint16_t*>(lds + C::B_Q + buf * C::B_PHI); };
#pragma unroll
    for (int i = 0; i < C::NQS; ++i) {
      const int seg = tid + 256 * i, tok = seg / (DK / 8), part = seg % (DK / 8);
      *reinterpret_cast<u32x4*>(sQ + tok * C::KS + part * 8) =
          *reinterpret_cast<const u32x4*>(Qh + (size_t)min(q0 + tok, N - 1) * DK + part * 8);
    }
    // phi of 32-row block j: wave w builds octet 4j + w for the 128 tokens
    // (lane = token, two passes); the octet's descriptor is wave-uniform
    const uint32_t* tab = OctOf<DK>::get().d;
    auto gen = [&](int j, uint16_t* P) {
      const int o = 4 * j + w;
      const uint32_t d = o < C::NO ? tab[o] : 0xFFu;
      const int m = d & 0xFF, a = (d >> 8) & 0xFF, b0 = (int)(d >> 16);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok = 64 * h + lane;
        const uint16_t* x = sQ + tok * C::KS;
        float ph[8];
        if (m == 2) {
          const uint32_t xa = x[a];  // {x_a, 0}; shifted: {0, x_a}
          const u32x4 xb = *reinterpret_cast<const u32x4*>(x + b0);
#pragma unroll
          for (int e = 0; e < 4; ++e) prod_pair(xa, xa << 16, xb[e], ph[2 * e], ph[2 * e + 1]);
          if (b0 <= a) {  // the octet holding (a, a): rows b < a are zero, weight 1/2 on b == a
#pragma unroll
            for (int u = 0; u < 8; ++u) ph[u] = b0 + u > a ? ph[u] : (b0 + u == a ? 0.5f * ph[u] : 0.f);
          }
        } else if (m == 1) {
          const u32x4 xb = *reinterpret_cast<const u32x4*>(x + b0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ph[2 * e] = __uint_as_float(xb[e] << 16);
            ph[2 * e + 1] = __uint_as_float(xb[e] & 0xFFFF0000u);
          }
        } else {  // order 0 (row 0, weight 1) or past the last octet
#pragma unroll
          for (int u = 0; u < 8; ++u) ph[u] = (m == 0 && u == 0) ? 1.f : 0.f;
        }
        *reinterpret_cast<u32x4*>(P + tok * C::PHS + 8 * w) =
            u32x4{pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3]), pack_bf16x2(ph[4], ph[5]),
                  pack_bf16x2(ph[6], ph[7])};
      }
    };
    const float* S = ws + ((size_t)bh * nspan + s) * (size_t)WP * (kDV + 1);
    const int dpl = li >= 8 ? 1 : 0;  // A-operand rows 8-15: the lo plane
    auto load_s = [&](int j, u32x4& sf, u32x4& dcb) {
      sf = *reinterpret_cast<const u32x4*>(S + st_frag_off(j, w, lane, 0));
      dcb = *reinterpret_cast<const u32x4*>(S + st_den_off(WP, j, lg, dpl));
    };
    u32x4 sf, dcb;
    load_s(0, sf, dcb);
    __syncthreads();  // Q tile staged
    gen(0, sPhi(0));
    __syncthreads();
    for (int j = 0; j < C::NKB; ++j) {
      const uint16_t* P = sPhi(j & 1);
      // the next block's state fragments first: their latency runs under
      // the generation of its phi rows and this block's MFMAs
      u32x4 nsf, ndcb;
      if (j + 1 < C::NKB) load_s(j + 1, nsf, ndcb);
      if (j + 1 < C::NKB) gen(j + 1, sPhi((j + 1) & 1));
      u32x4 af[8];
#pragma unroll
      for (int qt = 0; qt < 8; ++qt)
        af[qt] = *reinterpret_cast<const u32x4*>(P + (qt * 16 + li) * C::PHS + 8 * lg);
#pragma unroll
      for (int qt = 0; qt < 8; ++qt) nB[qt] = mfma_bf16(sf, af[qt], nB[qt]);
      // normalisers of query tiles 2w, 2w+1 (w is wave-uniform: a scalar branch)
      switch (w) {
        case 0: dC[0] = mfma_bf16(dcb, af[0], dC[0]); dC[1] = mfma_bf16(dcb, af[1], dC[1]); break;
        case 1: dC[0] = mfma_bf16(dcb, af[2], dC[0]); dC[1] = mfma_bf16(dcb, af[3], dC[1]); break;
        case 2: dC[0] = mfma_bf16(dcb, af[4], dC[0]); dC[1] = mfma_bf16(dcb, af[5], dC[1]); break;
        default: dC[0] = mfma_bf16(dcb, af[6], dC[0]); dC[1] = mfma_bf16(dcb, af[7], dC[1]); break;
      }
      if (j + 1 < C::NKB) {
        sf = nsf; dcb = ndcb;
      }
      __syncthreads();
    }
  }

  // ---------------- combine: phase B's tiles to the row split of phase A ----------------
  float* sX = reinterpret_cast<float*>(lds);
  float* sXd = sX + kStQ * C::OXS;
  float* sXh = sXd + kStQ;
#pragma unroll
  for (int qt = 0; qt < 8; ++qt)
    *reinterpret_cast<f32x4*>(sX + (qt * 16 + li) * C::OXS + 16 * w + 4 * lg) = nB[qt];
  // lane (lg = 0, li) holds the hi readout of query li, lane (lg = 2, li) the lo one
  const float dlo0 = __shfl_xor(dC[0].x, 32), dlo1 = __shfl_xor(dC[1].x, 32);
  if (lg == 0) {
    sXd[(2 * w) * 16 + li] = dC[0].x + dlo0;
    sXd[(2 * w + 1) * 16 + li] = dC[1].x + dlo1;
    sXh[(2 * w) * 16 + li] = dC[0].x;
    sXh[(2 * w + 1) * 16 + li] = dC[1].x;
  }
  // column means of the readout shift (0 without a prefix state)
  f32x4 acol[4];
  const float* Sa = ws + ((size_t)bh * nspan + s) * (size_t)WP * (kDV + 1) + 16 * kDV;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
    acol[ct] = has_prefix ? *reinterpret_cast<const f32x4*>(Sa + 16 * ct + 4 * lg) : zero4();
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int ql = 32 * w + 16 * qt + li;
    const int q = q0 + ql;
    if (q >= N) continue;
    const float den = dA[qt].x + sXd[ql];
    const float r = UNN ? 1.0f : 1.0f / den;
    const float dh = sXh[ql];
    float* orow = Og + ((size_t)bh * N + q) * kDV;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x4 num =
          oA[qt][ct] + *reinterpret_cast<const f32x4*>(sX + ql * C::OXS + 16 * ct + 4 * lg) + acol[ct] * dh;
      store_nt(orow + 16 * ct + 4 * lg, num * r);
    }
    if (UNN && lg == 0) Dg[(size_t)bh * N + q] = den;
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs with more than 256 feature rows: the same three launches on
// fp32 MFMA (16x16x4), rows in feature order, no hi/lo splits (fp32
// operands are exact).  The span totals come from stream_totals_f32_kernel
// over spans of kStL tokens.  The prefix state is rewritten per
// 16-row block and 16-column tile as the readout's A operand (lane (i, g)
// holds rows 16j + 4g .. 4g+3 of column 16ct + i: one 16-byte load); the
// normaliser rows are read in place.
// ---------------------------------------------------------------------------
// Four consecutive inputs, and one, as fp32: fp32 as stored, bf16 widened
// (exact), so the fp32 kernels also take bf16 inputs.
__device__ inline f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ inline f32x4 ld4f(const uint16_t* p) {
  const uint2 r = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
               __uint_as_float(r.y & 0xFFFF0000u)};
}
__device__ inline float ld1f(const float* p) { return *p; }
__device__ inline float ld1f(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

template <int DK, int NT>
struct StF {
  static constexpr int W = rows_for(DK, NT);
  static constexpr int NKB = (W + 15) / 16;  // 16-row blocks of the readout
  static constexpr int NKP = (NKB + 1) / 2; // pairs of 16-row blocks: one phi tile and one barrier each
  static constexpr int XS = DK + 1;          // K tile row stride (floats; odd: column reads hit distinct banks)
  // Q tile row stride: the coordinates, then the ones column; odd, so that the
  // 64 lanes (tokens) reading one column of their rows hit distinct banks
  static constexpr int QS = DK + 1;
  static constexpr int VS = kDV + 4;         // V tile row stride
  static constexpr int PHS = 32 + 4;         // phi tile row stride: two 16-row blocks
  static constexpr int B_K = kStK * XS * 4, B_V = kStK * VS * 4;
  static constexpr int LDS_A = 2 * (B_K + B_V);
  static constexpr int B_Q = kStQ * QS * 4, B_PHI = kStQ * PHS * 4;
  static constexpr int LDS_B = B_Q + 2 * B_PHI;
  static constexpr int OXS = kDV + 4;
  static constexpr int LDS_X = (kStQ * OXS + kStQ) * 4;
  static constexpr int LDS = LDS_A > LDS_B ? (LDS_A > LDS_X ? LDS_A : LDS_X) : (LDS_B > LDS_X ? LDS_B : LDS_X);
  static constexpr int KSEG = kStK * DK / 4, VSEG = kStK * kDV / 4, QSEG = kStQ * DK / 4;  // 16-byte segments
  static constexpr int NKS = (KSEG + 255) / 256, NVS = VSEG / 256, NQS = (QSEG + 255) / 256;
  static_assert(VSEG % 256 == 0, "V segments per thread");
};

__device__ inline size_t stf_frag_off(int j, int ct, int l) {
  return (size_t)(16 * j + (l >> 2)) * kDV + 16 * ct + 4 * (l & 3);
}

// Exclusive scan over spans (in place) into fragments, and the final states;
// one workgroup per (head, 16-row block), wave = column tile, wave 0's lanes
// 0-15 also take the block's normaliser rows (in place, natural layout).
template <int DK, int NT>
__global__ __launch_bounds__(256) void stream_scan_f32_kernel(float* ws, int nspan, int WP, int BH,
                                                              const float* init, float* states, int bh0, int BHtot) {
  using C = StF<DK, NT>;
  constexpr int W = C::W;
  const int bh = blockIdx.x / C::NKB, j = blockIdx.x % C::NKB;
  const size_t gh = (size_t)bh0 + bh;  // head in init and states (BHtot heads)
  const int lane = threadIdx.x & 63, ct = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const bool den_lane = ct == 0 && lane < 16;
  const size_t per = (size_t)WP * (kDV + 1);
  float* base = ws + (size_t)bh * nspan * per;
  const int col = 16 * ct + li;
  const int rd = 16 * j + lane;
  float run[4], rund = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 16 * j + 4 * lg + u;
    run[u] = (init != nullptr && r < W) ? init[(gh * W + r) * kDV + col] : 0.f;
  }
  if (init != nullptr && den_lane && rd < W) rund = init[(size_t)BHtot * W * kDV + gh * W + rd];
  constexpr int G = 4;
  for (int s0 = 0; s0 < nspan; s0 += G) {
    float t[G][4], td[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (s0 + g < nspan) {
        const float* p = base + (size_t)(s0 + g) * per;
#pragma unroll
        for (int u = 0; u < 4; ++u) t[g][u] = p[(size_t)(16 * j + 4 * lg + u) * kDV + col];
        if (den_lane) td[g] = p[(size_t)WP * kDV + rd];
      }
    }
    // every read of these spans has returned before any fragment is written
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (s0 + g < nspan) {
        float* p = base + (size_t)(s0 + g) * per;
        *reinterpret_cast<f32x4*>(p + stf_frag_off(j, ct, lane)) = f32x4{run[0], run[1], run[2], run[3]};
#pragma unroll
        for (int u = 0; u < 4; ++u) run[u] += t[g][u];
        if (den_lane) {
          p[(size_t)WP * kDV + rd] = rund;
          rund += td[g];
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 16 * j + 4 * lg + u;
    if (r < W) states[(gh * W + r) * kDV + col] = run[u];
  }
  if (den_lane && rd < W) states[(size_t)BHtot * W * kDV + gh * W + rd] = rund;
}

// Output pass for fp32 inputs: one workgroup of 4 waves per 128 queries of a
// span, 3 workgroups per CU; phase A (the span's causal block) and phase B
// (readout of the prefix state) as in stream_out_kernel, on fp32 MFMA.  Lane layouts of f32
// 16x16x4: A[i][g], B[g][i]; D: lane holds D[4g + s][i].
template <int DK, int NT, bool UNN, class TIn>
__global__ __launch_bounds__(256, 3) void stream_out_f32_kernel(const TIn* __restrict__ Qg,
                                                                const TIn* __restrict__ Kg,
                                                                const TIn* __restrict__ Vg, int BH, int N,
                                                                int nspan, int WP, const float* __restrict__ ws,
                                                                bool has_init, float* __restrict__ Og,
                                                                float* __restrict__ Dg,
                                                                const uint32_t* __restrict__ big_rows) {
  using C = StF<DK, NT>;
  constexpr int W = C::W;
  constexpr int KT = DK / 4;  // K-steps of the scores
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  const int b = blockIdx.x;
  const int sg = (b / (8 * kStT)) * 8 + (b & 7);
  const int tile = kStT - 1 - (b >> 3) % kStT;
  if (sg >= BH * nspan) return;
  const int bh = sg / nspan, s = sg % nspan;
  const int q0 = s * kStL + tile * kStQ;
  if (q0 >= N) return;
  const TIn* Qh = Qg + (size_t)bh * N * DK;
  const TIn* Kh = Kg + (size_t)bh * N * DK;
  const TIn* Vh = Vg + (size_t)bh * N * kDV;

  // Phase B (the prefix readout) runs first: phase A's accumulators are then
  // not live across it, which keeps the kernel within 3 waves per SIMD.
  // Phase B's last barrier orders its LDS reads before phase A's tiles.
  // ---------------- phase B: readout of the prefix state ----------------
  f32x4 nB[8];
  float dp[2] = {0.f, 0.f};  // partial normaliser readouts (rows of this lane's group)
#pragma unroll
  for (int qt = 0; qt < 8; ++qt) nB[qt] = zero4();
  if (s > 0 || has_init) {
    float* sQ = reinterpret_cast<float*>(lds);
    auto sPhi = [&](int buf) { return reinterpret_cast<float*>(lds + C::B_Q + buf * C::B_PHI); };
#pragma unroll
    for (int i = 0; i < C::NQS; ++i) {
      const int seg = tid + 256 * i;
      if (seg < C::QSEG) {
        const int tok = seg / (DK / 4), part = seg % (DK / 4);
        const f32x4 x = ld4f(Qh + (size_t)min(q0 + tok, N - 1) * DK + part * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sQ[tok * C::QS + part * 4 + e] = x[e];  // odd stride: 4-byte stores
      }
    }
    if (tid < kStQ) sQ[tid * C::QS + DK] = 1.f;  // the ones column
    // phi rows 32J + 8w .. +7 (a pair of 16-row blocks) of the 128 tokens
    // (lane = token, two passes); row codes and weights are wave-uniform.
    // Every row takes MAXM factors from the token's row of the Q tile: its
    // coordinates, then the ones column past its order (all of them for the
    // order-0 row and for padding rows, whose weight is 0), so there is no
    // branch or loop per row; the products run left to right from the
    // weight, as one factor at a time would.
    constexpr int MAXM = NT - 1 > 1 ? NT - 1 : 1;
    const RowSrc<DK, NT> tab{big_rows};
    auto gen = [&](int J, float* P) {
      int col[8][MAXM];
      float wt[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = 32 * J + 8 * w + u;
        const uint32_t code = r < W ? tab.code(r) : kPadRow;
        const int m = row_order(code);
        wt[u] = r < W ? tab.weight(r) : 0.f;
#pragma unroll
        for (int l = 0; l < MAXM; ++l) col[u][l] = (m == 7 || l >= m) ? DK : row_index<DK>(code, l);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok = 64 * h + lane;
        const float* xr = sQ + tok * C::QS;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          f32x4 ph;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int u = 4 * g + e;
            float v = wt[u];
#pragma unroll
            for (int l = 0; l < MAXM; ++l) v *= xr[col[u][l]];
            ph[e] = v;
          }
          *reinterpret_cast<f32x4*>(P + tok * C::PHS + 8 * w + 4 * g) = ph;
        }
      }
    };
    const float* S = ws + ((size_t)bh * nspan + s) * (size_t)WP * (kDV + 1);
    auto load_s = [&](int j, f32x4& sa, f32x4& da) {
      sa = *reinterpret_cast<const f32x4*>(S + stf_frag_off(j, w, lane));
      da = *reinterpret_cast<const f32x4*>(S + (size_t)WP * kDV + 16 * j + 4 * lg);
    };
    // block j = 2J + half of the pair; blocks past NKB hold zero phi rows and
    // read the zero-padded state rows of the same span (j < WP / 16)
    // The widest shapes (tens of thousands of rows) sum the readout in
    // segments of kSeg pairs, added into nT and dT, so that no fp32
    // accumulation chain is longer than a segment plus the segment count.
    constexpr bool SEG = runtime_rows<DK, NT>();
    constexpr int kSeg = 128;
    f32x4 nT[SEG ? 8 : 1];
    float dT[2] = {0.f, 0.f};
#pragma unroll
    for (int qt = 0; qt < (SEG ? 8 : 1); ++qt) nT[qt] = zero4();
    f32x4 sa[2], da[2];
    load_s(0, sa[0], da[0]);
    load_s(1, sa[1], da[1]);
    __syncthreads();  // Q tile staged
    gen(0, sPhi(0));
    __syncthreads();
    for (int J = 0; J < C::NKP; ++J) {
      const float* P = sPhi(J & 1);
      if (J + 1 < C::NKP) gen(J + 1, sPhi((J + 1) & 1));
      f32x4 na[2], nd[2];
      if (J + 1 < C::NKP) {
        load_s(2 * J + 2, na[0], nd[0]);
        load_s(2 * J + 3, na[1], nd[1]);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 af[8];
#pragma unroll
        for (int qt = 0; qt < 8; ++qt)
          af[qt] = *reinterpret_cast<const f32x4*>(P + (qt * 16 + li) * C::PHS + 16 * hf + 4 * lg);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int qt = 0; qt < 8; ++qt) nB[qt] = mfma_f32(sa[hf][e], af[qt][e], nB[qt]);
        // normalisers of query tiles 2w, 2w+1: this lane's share (rows
        // 4lg .. 4lg+3 of the block, query li) of phi . Z, on the VALU (an
        // fp32 MFMA against broadcast rows would use one column in 16)
        switch (w) {
          case 0:
#pragma unroll
            for (int e = 0; e < 4; ++e) { dp[0] = __builtin_fmaf(da[hf][e], af[0][e], dp[0]); dp[1] = __builtin_fmaf(da[hf][e], af[1][e], dp[1]); }
            break;
          case 1:
#pragma unroll
            for (int e = 0; e < 4; ++e) { dp[0] = __builtin_fmaf(da[hf][e], af[2][e], dp[0]); dp[1] = __builtin_fmaf(da[hf][e], af[3][e], dp[1]); }
            break;
          case 2:
#pragma unroll
            for (int e = 0; e < 4; ++e) { dp[0] = __builtin_fmaf(da[hf][e], af[4][e], dp[0]); dp[1] = __builtin_fmaf(da[hf][e], af[5][e], dp[1]); }
            break;
          default:
#pragma unroll
            for (int e = 0; e < 4; ++e) { dp[0] = __builtin_fmaf(da[hf][e], af[6][e], dp[0]); dp[1] = __builtin_fmaf(da[hf][e], af[7][e], dp[1]); }
            break;
        }
      }
      if (J + 1 < C::NKP) {
        sa[0] = na[0]; sa[1] = na[1];
        da[0] = nd[0]; da[1] = nd[1];
      }
      if constexpr (SEG) {
        if ((J + 1) % kSeg == 0 || J + 1 == C::NKP) {
#pragma unroll
          for (int qt = 0; qt < 8; ++qt) {
            nT[qt] += nB[qt];
            nB[qt] = zero4();
          }
          dT[0] += dp[0];
          dT[1] += dp[1];
          dp[0] = dp[1] = 0.f;
        }
      }
      __syncthreads();
    }
    if constexpr (SEG) {
#pragma unroll
      for (int qt = 0; qt < 8; ++qt) nB[qt] = nT[qt];
      dp[0] = dT[0];
      dp[1] = dT[1];
    }
  }

  // ---------------- phase A: the span's causal block ----------------
  const int qw0 = q0 + 32 * w;
  float qf[2][KT];  // B operand of S^T = K Q^T: q[query][4t + g]
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int t = 0; t < KT; ++t) qf[qt][t] = ld1f(Qh + (size_t)min(qw0 + 16 * qt + li, N - 1) * DK + 4 * t + lg);
  f32x4 oA[2][4];
  float da0[2];  // this lane's share (keys 4lg .. 4lg+3 of each tile) of P.1 for query li
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    da0[qt] = 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) oA[qt][ct] = zero4();
  }
  {
    auto sK = [&](int buf) { return reinterpret_cast<float*>(lds + buf * (C::B_K + C::B_V)); };
    auto sV = [&](int buf) { return reinterpret_cast<float*>(lds + buf * (C::B_K + C::B_V) + C::B_K); };
    const int kbeg = s * kStL;
    const int kend = min(q0 + kStQ, N);
    const int nkb = (kend - kbeg + kStK - 1) / kStK;
    f32x4 rk[C::NKS], rv[C::NVS];
    auto issue = [&](int kb) {
      const int k0 = kbeg + kb * kStK;
#pragma unroll
      for (int i = 0; i < C::NKS; ++i) {
        const int seg = tid + 256 * i;
        if (seg < C::KSEG) {
          const int tok = seg / (DK / 4), part = seg % (DK / 4);
          rk[i] = ld4f(Kh + (size_t)min(k0 + tok, N - 1) * DK + part * 4);
        }
      }
#pragma unroll
      for (int i = 0; i < C::NVS; ++i) {
        const int seg = tid + 256 * i, tok = seg >> 4, part = seg & 15;
        rv[i] = ld4f(Vh + (size_t)min(k0 + tok, N - 1) * kDV + part * 4);
      }
    };
    auto commit = [&](int buf) {
      float* K = sK(buf);
      float* V = sV(buf);
#pragma unroll
      for (int i = 0; i < C::NKS; ++i) {
        const int seg = tid + 256 * i;
        if (seg < C::KSEG) {
          const int tok = seg / (DK / 4), part = seg % (DK / 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) K[tok * C::XS + part * 4 + e] = rk[i][e];
        }
      }
#pragma unroll
      for (int i = 0; i < C::NVS; ++i) {
        const int seg = tid + 256 * i, tok = seg >> 4, part = seg & 15;
        *reinterpret_cast<f32x4*>(V + tok * C::VS + part * 4) = rv[i];
      }
    };
    issue(0);
    commit(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
      const int buf = kb & 1;
      if (kb + 1 < nkb) issue(kb + 1);
      const int k0 = kbeg + kb * kStK;
      const float* K = sK(buf);
      const float* V = sV(buf);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int kt0 = k0 + 16 * kt;
        if (kt0 > qw0 + 31) continue;             // every key of the tile is after this wave's queries
        const bool diag = kt0 + 15 > qw0;         // keys after the wave's first query: mask
        float p[2][4];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          f32x4 x = zero4();
#pragma unroll
          for (int t = 0; t < KT; ++t) x = mfma_f32(K[(16 * kt + li) * C::XS + 4 * t + lg], qf[qt][t], x);
          const int query = qw0 + 16 * qt + li;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = taylor_poly<NT>(x[e]);
            p[qt][e] = (diag && kt0 + 4 * lg + e > query) ? 0.f : v;
          }
          // normaliser on the VALU (an fp32 MFMA against ones would use one column in 16)
          da0[qt] += (p[qt][0] + p[qt][1]) + (p[qt][2] + p[qt][3]);
        }
        // O^T += V^T P^T: K-slot g of step e is key kt0 + 4g + e
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = V[(16 * kt + 4 * lg + e) * C::VS + 16 * ct + li];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) oA[qt][ct] = mfma_f32(a, p[qt][e], oA[qt][ct]);
          }
      }
      if (kb + 1 < nkb) {
        commit(buf ^ 1);
        __syncthreads();
      }
    }
  }
  __syncthreads();

#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {  // add the four key groups' shares
    da0[qt] += __shfl_xor(da0[qt], 16);
    da0[qt] += __shfl_xor(da0[qt], 32);
  }
  // ---------------- combine ----------------
  float* sX = reinterpret_cast<float*>(lds);
  float* sXd = sX + kStQ * C::OXS;
#pragma unroll
  for (int qt = 0; qt < 8; ++qt)
    *reinterpret_cast<f32x4*>(sX + (qt * 16 + li) * C::OXS + 16 * w + 4 * lg) = nB[qt];
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // add the four row groups' shares
    dp[k] += __shfl_xor(dp[k], 16);
    dp[k] += __shfl_xor(dp[k], 32);
  }
  if (lg == 0) {
    sXd[(2 * w) * 16 + li] = dp[0];
    sXd[(2 * w + 1) * 16 + li] = dp[1];
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int ql = 32 * w + 16 * qt + li;
    const int q = q0 + ql;
    if (q >= N) continue;
    const float den = da0[qt] + sXd[ql];
    const float r = UNN ? 1.0f : 1.0f / den;
    float* orow = Og + ((size_t)bh * N + q) * kDV;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x4 num = oA[qt][ct] + *reinterpret_cast<const f32x4*>(sX + ql * C::OXS + 16 * ct + 4 * lg);
      store_nt(orow + 16 * ct + 4 * lg, num * r);
    }
    if (UNN && lg == 0) Dg[(size_t)bh * N + q] = den;
  }
}

// Span totals for fp32 inputs: one workgroup of 4 waves per (head, span, 128
// feature rows); wave w owns rows 128*rb + 32w .. +31 (two 16-row tiles) for
// all 64 value columns.  Per 64-token block each lane (= token) builds the
// wave's 32 mu rows into a wave-private tile and adds them to its own
// partial normalisers (summed over the lanes once at the end); the values
// are contracted with V on fp32 MFMA (A = mu^T, B = V, 4 tokens per step).
template <int DK, int NT>
struct StFT {
  static constexpr int W = rows_for(DK, NT);
  static constexpr int NRB = (W + 127) / 128;   // 128-row groups
  static constexpr int WP = NRB * 128;          // padded rows of a span state
  static constexpr int KS = DK + 4;             // K tile row stride: coordinates, a ones and a zero column, pad
  static constexpr int ONE = DK, ZERO = DK + 1; // the constant columns of the K tile
  static constexpr int MAXM = NT - 1 > 1 ? NT - 1 : 1;  // factors per row (orders 0 .. NT-1)
  static constexpr int VS = kDV + 16;           // V tile row stride: rows 4 apart hit distinct bank groups
  static constexpr int B_K = kStK * KS * 4, B_V = kStK * VS * 4;
  static constexpr int LDS = B_K + B_V;
  static constexpr int KSEG = kStK * DK / 4, VSEG = kStK * kDV / 4;
  static constexpr int NKS = (KSEG + 255) / 256, NVS = VSEG / 256;
};

// Span totals, fp32: one workgroup of 4 waves per (head, span, 128 feature
// rows); wave w owns rows R0 = 128 rb + 32 w .. +31 as two 16-row tiles for
// all 64 value columns.  The A operand of the 16x16x4 MFMA is built in place:
// lane (i, g) holds row R0 + 16 rt + i of token 4t + g, the product of the
// row's factors read from the staged K tile.  Each row has MAXM factor
// columns: its coordinates, then the ones column (1 for tokens inside the
// span, 0 past its end) for factors past its order; the order-0 row is all
// ones columns and a padding row starts with the zero column.  So every row
// costs MAXM LDS reads and MAXM - 1 multiplies, with no branch, in the same
// left-to-right order as one factor at a time from 1.  The normaliser rows
// are per-lane sums over the lane's tokens, added over the four token
// residues at the end.
template <int DK, int NT, class TIn>
__global__ __launch_bounds__(256, 4) void stream_totals_f32_kernel(const TIn* __restrict__ Kg,
                                                                   const TIn* __restrict__ Vg, int BH, int N,
                                                                   int nspan, float* __restrict__ ws,
                                                                   const uint32_t* __restrict__ big_rows) {
  using C = StFT<DK, NT>;
  constexpr int W = C::W;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int b = blockIdx.x;
  const int rb = (b >> 3) % C::NRB;
  const int hs = (b / (8 * C::NRB)) * 8 + (b & 7);
  if (hs >= BH * nspan) return;
  const int bh = hs / nspan, s = hs % nspan;
  const int t_begin = s * kStL, t_end = min(N, t_begin + kStL);
  const int ntb = (t_end - t_begin + kStK - 1) / kStK;
  const int R0 = 128 * rb + 32 * w;  // this wave's first row
  const bool active = R0 < W;        // wave-uniform
  const TIn* Kh = Kg + (size_t)bh * N * DK;
  const TIn* Vh = Vg + (size_t)bh * N * kDV;
  float* sK = reinterpret_cast<float*>(lds);
  float* sV = reinterpret_cast<float*>(lds + C::B_K);

  f32x4 rk[C::NKS], rv[C::NVS];
  auto issue = [&](int tb) {
    const int k0 = t_begin + tb * kStK;
#pragma unroll
    for (int i = 0; i < C::NKS; ++i) {
      const int seg = tid + 256 * i;
      if (seg < C::KSEG) {
        const int tok = seg / (DK / 4), part = seg % (DK / 4);
        rk[i] = ld4f(Kh + (size_t)min(k0 + tok, t_end - 1) * DK + part * 4);
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVS; ++i) {
      const int seg = tid + 256 * i, tok = seg >> 4, part = seg & 15;
      rv[i] = ld4f(Vh + (size_t)min(k0 + tok, t_end - 1) * kDV + part * 4);
    }
  };
  // K rows of tokens past the span end are stored as zeros, and their ones
  // column as 0 (so every row of such a token is 0)
  auto commit = [&](int tb) {
    const int k0 = t_begin + tb * kStK;
#pragma unroll
    for (int i = 0; i < C::NKS; ++i) {
      const int seg = tid + 256 * i;
      if (seg < C::KSEG) {
        const int tok = seg / (DK / 4), part = seg % (DK / 4);
        *reinterpret_cast<f32x4*>(sK + tok * C::KS + part * 4) = k0 + tok < t_end ? rk[i] : zero4();
      }
    }
    if (tid < kStK) {
      sK[tid * C::KS + C::ONE] = k0 + tid < t_end ? 1.f : 0.f;
      sK[tid * C::KS + C::ZERO] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < C::NVS; ++i) {
      const int seg = tid + 256 * i, tok = seg >> 4, part = seg & 15;
      *reinterpret_cast<f32x4*>(sV + tok * C::VS + part * 4) = rv[i];
    }
  };

  // byte offsets in the K tile of this lane's factor columns, for token g
  // (token 4t + g adds 16 t KS bytes, a compile-time offset)
  const RowSrc<DK, NT> tab{big_rows};
  uint32_t foff[2][C::MAXM];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = R0 + 16 * rt + li;
    const uint32_t code = r < W ? tab.code(r) : kPadRow;
    const int m = row_order(code);
#pragma unroll
    for (int l = 0; l < C::MAXM; ++l) {
      const int col = m == 7 ? (l == 0 ? C::ZERO : C::ONE) : (l < m ? row_index<DK>(code, l) : C::ONE);
      foff[rt][l] = (uint32_t)((lg * C::KS + col) * 4);
    }
  }
  f32x4 st[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) st[rt][ct] = zero4();
  float zacc[2] = {0.f, 0.f};

  issue(0);
  for (int tb = 0; tb < ntb; ++tb) {
    commit(tb);
    __syncthreads();
    if (tb + 1 < ntb) issue(tb + 1);
    if (active) {
      const unsigned char* Kb = reinterpret_cast<const unsigned char*>(sK);
#pragma unroll
      for (int t = 0; t < kStK / 4; ++t) {
        float bv[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) bv[ct] = sV[(4 * t + lg) * C::VS + 16 * ct + li];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          float a = *reinterpret_cast<const float*>(Kb + foff[rt][0] + t * 16 * C::KS);
#pragma unroll
          for (int l = 1; l < C::MAXM; ++l) a *= *reinterpret_cast<const float*>(Kb + foff[rt][l] + t * 16 * C::KS);
          zacc[rt] += a;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) st[rt][ct] = mfma_f32(a, bv[ct], st[rt][ct]);
        }
      }
    }
    __syncthreads();  // the K and V tiles are overwritten next
  }
  if (!active) return;
  float* S = ws + (size_t)hs * C::WP * (kDV + 1);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = R0 + 16 * rt + 4 * lg + e;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) S[(size_t)row * kDV + 16 * ct + li] = st[rt][ct][e];
    }
  // normalisers: the lanes' partial sums over the four token residues
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float z = zacc[rt];
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    if (lg == 0) S[(size_t)C::WP * kDV + R0 + 16 * rt + li] = z;
  }
}

template <int DK, int NT>
constexpr bool use_stream_f32() { return StF<DK, NT>::W > 256; }

// bf16 inputs with four or more terms (dk = 16: 969 or 4,845 rows; dk = 32
// and 64: 6,545 to 814,385 rows) run the same kernels, widening their inputs
// to fp32 as they stage them
template <int DK, int NT>
constexpr bool bf16_uses_stream_f32() { return DK >= 16 && NT >= 4; }

template <int DK, int NT, class TIn>
hipError_t stream_launch_f32(const void* Q, const void* K, const void* V, int BH, int N, const PrefillPlan& p,
                             const float* states_in, float* O, float* den_out, float* states, float* ws,
                             hipStream_t s, int bh0, int BHtot) {
  using T = StFT<DK, NT>;
  const uint32_t* big = nullptr;
  if constexpr (runtime_rows<DK, NT>()) {
    const hipError_t eb = big_row_codes(DK, NT, &big);
    if (eb != hipSuccess) return eb;
  }
  static_assert(StF<DK, NT>::NKP * 32 <= T::WP, "the readout's row blocks (pairs) lie inside the span state");
  const unsigned sgs = (unsigned)((BH * p.nspan + 7) / 8 * 8);  // (head, span) pairs, padded to the 8 XCDs
  hipLaunchKernelGGL((stream_totals_f32_kernel<DK, NT, TIn>), dim3(sgs * T::NRB), dim3(256), 0, s, (const TIn*)K,
                     (const TIn*)V, BH, N, p.nspan, ws, big);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((stream_scan_f32_kernel<DK, NT>), dim3((unsigned)(BH * StF<DK, NT>::NKB)), dim3(256), 0, s, ws,
                     p.nspan, (int)T::WP, BH, states_in, states, bh0, BHtot);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(sgs * kStT);
  if (den_out)
    hipLaunchKernelGGL((stream_out_f32_kernel<DK, NT, true, TIn>), grid, dim3(256), 0, s, (const TIn*)Q,
                       (const TIn*)K, (const TIn*)V, BH, N, p.nspan, (int)T::WP, (const float*)ws,
                       states_in != nullptr, O, den_out, big);
  else
    hipLaunchKernelGGL((stream_out_f32_kernel<DK, NT, false, TIn>), grid, dim3(256), 0, s, (const TIn*)Q,
                       (const TIn*)K, (const TIn*)V, BH, N, p.nspan, (int)T::WP, (const float*)ws,
                       states_in != nullptr, O, den_out, big);
  return hipGetLastError();
}

// The shapes of this path: bf16 inputs with n = 3 and dk = 32 or 64, in
// 64-token chunks (the totals pass).
template <int DK, int NT>
constexpr bool use_stream() { return NT == 3 && (DK == 32 || DK == 64); }

template <int DK>
hipError_t stream_launch(const void* Q, const void* K, const void* V, int BH, int N, const PrefillPlan& p,
                         const float* states_in, float* O, float* den_out, float* states, float* ws, hipStream_t s,
                         int bh0, int BHtot) {
  using T = StTot<DK>;
  static_assert(StCfg<DK>::NKB * 32 <= T::WP, "the readout's row blocks lie inside the span state");
  const unsigned hsg = (unsigned)((BH * p.nspan + 7) / 8 * 8);  // (head, span) pairs, padded to the 8 XCDs
  hipLaunchKernelGGL((stream_totals_kernel<DK>), dim3(hsg * T::NRB), dim3(T::NW * 64), 0, s, (const uint16_t*)K,
                     (const uint16_t*)V, BH, N, p.nspan, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((stream_scan_kernel<DK>), dim3((unsigned)(BH * StCfg<DK>::NKB)), dim3(256), 0, s, ws, p.nspan,
                     (int)T::WP, BH, p.W, states_in, states, bh0, BHtot);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(hsg * kStT);
  if (den_out)
    hipLaunchKernelGGL((stream_out_kernel<DK, true>), grid, dim3(256), 0, s, (const uint16_t*)Q, (const uint16_t*)K,
                       (const uint16_t*)V, BH, N, p.nspan, (int)T::WP, (const float*)ws, states_in != nullptr, O,
                       den_out);
  else
    hipLaunchKernelGGL((stream_out_kernel<DK, false>), grid, dim3(256), 0, s, (const uint16_t*)Q, (const uint16_t*)K,
                       (const uint16_t*)V, BH, N, p.nspan, (int)T::WP, (const float*)ws, states_in != nullptr, O,
                       den_out);
  return hipGetLastError();
}

}  // namespace
}  // namespace tt
