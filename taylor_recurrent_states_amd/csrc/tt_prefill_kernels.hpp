// Chunked causal prefill on MFMA.
//
// "Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
// with a Fixed Number of Recurrent States" (abstract): the causal history of
// a head is the state S[t, :] = sum_j mu_t(k_j) [v_j, 1]; states of disjoint
// token sets add, so prefill is a scan over spans of the sequence.  Inside a
// chunk of 64 tokens the output is the readout of the state before the chunk
// plus the chunk's own causal block of the quadratic form, (Q'K)V = Q'(KV)
// applied to everything but the diagonal block (comment thread on the paper,
// item 46888355, reply on the associativity):
//
//   num/den(i) = phi(q_i).S_prev + sum_{j in chunk, j <= i} K_n(q_i.k_j) [v_j, 1]
//   S_prev    += mu(K_chunk)^T [V_chunk, 1]
//
// Three launches per call:
//   1. totals : one workgroup per (head, span, column group) folds its span
//               into a state from zero and writes it to the workspace.  bf16
//               inputs use a hi+lo bf16 split of mu, which is exact for a
//               product of two bf16 values, so span totals carry fp32
//               accumulation error only.
//   2. scan   : exclusive prefix over spans, in place; the sum over all spans
//               is the final state (written in the library's plane layout).
//   3. sweep  : one workgroup per (head, span, column group) starts from its
//               prefix, keeps the state in MFMA accumulators, and per chunk
//               does the readout, the intra-chunk block and the update.
//
// The state never leaves registers inside a span.  It is held as 16x16 MFMA
// accumulator tiles (rows = feature rows, columns = value columns).  The
// normaliser column ("+1", comment thread reply on the extra column) lives in
// LDS as one fp32 per feature row and is contracted by MFMA against a ones
// column, so it stays in fp32.
//
// Lane layouts (probed on gfx950): lane l = 16g + i.
//   bf16 16x16x32: A[i][8g..8g+7], B[8g..8g+7][i];   f32 16x16x4: A[i][g], B[g][i];
//   D: lane holds D[4g + s][i], s = 0..3.
// For bf16 a 32-row K-block is two accumulator tiles tau = 0, 1 whose M index
// 4g'+s holds row 8g' + 4tau + s.  Read back as an MFMA B operand, lane g's
// k-slots 8g..8g+7 are then rows 8g..8g+7 in natural order, so every LDS
// tile (features, P, V^T) is stored in natural order.
#pragma once

#include "tt_device.hpp"
#include "tt_internal.hpp"

namespace tt {
namespace {

// MODE_OUTPUT_UNN: the output pass with unnormalised outputs (numerators to O,
// normalisers to a separate buffer); the pipe kernel only
enum { MODE_TOTALS = 0, MODE_OUTPUT = 1, MODE_OUTPUT_UNN = 2 };

constexpr int kCH = 64;  // tokens per chunk
constexpr int kDV = 64;  // value columns

// Pick J (K-blocks per wave per slab) <= jmax minimising the padded count.
constexpr int pick_j(int maxkb, int jmax) {
  int best = 1, best_pad = 1 << 30;
  for (int j = (jmax < 1 ? 1 : jmax); j >= 1; --j) {
    int ns = (maxkb + j - 1) / j;
    int pad = ns * j;
    if (pad < best_pad) { best = j; best_pad = pad; }
  }
  return best;
}

// Octet-aligned internal row order for bf16 inputs with n = 3 and dk >= 32.
// Rows come in groups of 8 ("octets") x_a * x[b0 .. b0+7] with b0 a multiple
// of 8: octet 0 holds the order-0 row (then 7 zero rows), then dk/8 octets of
// order 1 (x[b0..b0+7]), then for every a the octets b0 = 8*floor(a/8), ...,
// dk-8 of order 2, whose rows with b < a are zero.  A lane (= token) builds an
// octet from one 16-byte read of its coordinates and one scalar read.  The
// span workspace uses this order; the final states are written in feature
// order through abi_row().
constexpr bool use_oct(bool bf, int dk, int nt) { return bf && nt == 3 && dk >= 32; }
constexpr int oct_rows(int dk) { return 8 + dk + dk * (dk + 8) / 2; }
constexpr int internal_rows(bool bf, int dk, int nt) { return use_oct(bf, dk, nt) ? oct_rows(dk) : rows_for(dk, nt); }

// octet descriptors: m | a << 8 | b0 << 16
template <int DK>
struct OctTable {
  static constexpr int NO = oct_rows(DK) / 8;
  uint32_t d[NO];
  constexpr OctTable() : d() {
    int o = 0;
    d[o++] = 0u;
    for (int b0 = 0; b0 < DK; b0 += 8) d[o++] = 1u | ((uint32_t)b0 << 16);
    for (int a = 0; a < DK; ++a)
      for (int b0 = a / 8 * 8; b0 < DK; b0 += 8) d[o++] = 2u | ((uint32_t)a << 8) | ((uint32_t)b0 << 16);
  }
};
static __device__ const OctTable<32> kOct32 = OctTable<32>();
static __device__ const OctTable<64> kOct64 = OctTable<64>();
template <int DK> struct OctOf;
template <> struct OctOf<32> { static __device__ const OctTable<32>& get() { return kOct32; } };
template <> struct OctOf<64> { static __device__ const OctTable<64>& get() { return kOct64; } };

// feature-order row of internal octet row r, or -1 for a zero (padding) row
template <int DK>
__device__ inline int abi_row(int r) {
  constexpr int NO = OctTable<DK>::NO;
  const int o = r >> 3, u = r & 7;
  if (o >= NO) return -1;
  const uint32_t d = OctOf<DK>::get().d[o];
  const int m = d & 0xFF, a = (d >> 8) & 0xFF, b = (int)(d >> 16) + u;
  if (m == 0) return u == 0 ? 0 : -1;
  if (m == 1) return 1 + b;
  if (b < a) return -1;
  return 1 + DK + a * DK - a * (a - 1) / 2 + (b - a);
}

// feature rows per slab at most: bf16 256, fp32 128 (halved for 128-token
// chunks, whose tiles take twice the LDS per row)
constexpr int srmax(bool bf, int ch) { return (bf ? 256 : 128) / (ch > 64 ? 2 : 1); }

template <typename TIn_, int DK_, int NT_, int NVT_, int NRP_, int NRG_, int MODE_, int CH_ = 64>
struct Cfg {
  using TIn = TIn_;
  static constexpr bool BF = std::is_same<TIn_, uint16_t>::value;
  static constexpr bool OUT = (MODE_ == MODE_OUTPUT);
  static constexpr int DK = DK_, NT = NT_, NVT = NVT_, NRP = NRP_;
  static constexpr int CH = CH_;            // tokens per chunk
  static constexpr int QT = CH / 16;        // 16-query tiles per chunk
  static constexpr int NTS = (CH + 63) / 64;  // token slots per lane (lane = token within 64)
  static constexpr int NRG = NRG_;  // row groups: workgroups that split the feature rows of one span
  static constexpr int NW = NVT * NRP;
  static constexpr int NTHR = NW * 64;
  static constexpr int W = rows_for(DK, NT);             // feature rows
  static constexpr bool OCT = use_oct(BF, DK, NT);       // octet-aligned internal row order
  static constexpr int WI = internal_rows(BF, DK, NT);   // internal rows
  static constexpr int KB = BF ? 32 : 16;  // feature rows (and tokens) per K-block
  static constexpr int TPK = BF ? 2 : 1;   // accumulator tiles per K-block
  static constexpr int NKB = (WI + KB - 1) / KB;
  static constexpr int MAXKB = (NKB + NRP - 1) / NRP;
  static constexpr int SRMAX = srmax(BF, CH);
  static constexpr int J = pick_j(MAXKB, SRMAX / (NRP * KB));
  static constexpr int NSLAB_ALL = (MAXKB + J - 1) / J;  // slabs over all feature rows
  static constexpr int NSLAB = (NSLAB_ALL + NRG - 1) / NRG;  // slabs per row group
  static constexpr int MKB = NSLAB * J;    // K-blocks per wave (padded)
  static constexpr int SR = NRP * J * KB;  // feature rows per slab
  static constexpr int WP = NSLAB_ALL * SR;  // padded feature rows
  static constexpr int RWG = NSLAB * SR;     // feature rows of one row group
  // Totals pass over large feature sets: there is no readout, so each wave
  // takes one K-block of a slab for J column tiles (WPK waves per K-block)
  // instead of J K-blocks for one column tile; mu fragments are then read by
  // fewer waves.  Same accumulator count per wave.
  static constexpr bool TR = !OUT && WP > 256 && NVT == 4 && NW % (NRP * J) == 0 && (NW / (NRP * J)) * J == 4;
  static constexpr int WPK = TR ? NW / (NRP * J) : 1;
  static constexpr int TB = CH / KB;       // token K-blocks per chunk
  static_assert(CH % KB == 0 && CH >= 16 && CH <= 128, "chunk: a multiple of the token block, 16 .. 128");
  static constexpr int GC = 16 * NVT;      // value columns per workgroup
  using Elem = typename std::conditional<BF, uint16_t, float>::type;
  static constexpr int ES = sizeof(Elem);
  static constexpr int PADE = 16 / ES;     // 16-byte row padding
  // Q/K staging rows hold the input dtype: fp32 rows padded to an odd
  // stride (conflict-free scalar reads), bf16 rows padded to 16 bytes
  static constexpr int XS = BF ? DK + 8 : DK + 1;
  // small feature sets of narrow keys are generated by fully unrolled code
  // (lane = token, the token's row held in registers)
  static constexpr bool UNR = WP <= 256 && DK <= 16;
  static constexpr int PHS = SR + PADE;    // phi row stride (elements)
  // mu: [row][token] (mu^T, read with plain vector loads), or token-major
  // [token][row] for the octet generator (read with transposing loads)
  // (token-major stride = 40 mod 128 elements: the fastest measured for the
  // transposing reads, 336 bytes at 128-row slabs)
  static constexpr int MUS = OCT ? (SR + 8 + 87) / 128 * 128 + 40 : CH + PADE;
  static constexpr int VS = CH + PADE;     // V^T row stride
  static constexpr int PS = CH + PADE;     // P row stride
  static constexpr int NMU = (BF && !OUT) ? 2 : 1;  // mu planes (hi, lo) in the totals pass
  static constexpr int NPP = BF ? 2 : 1;            // P planes (hi, lo)
  static constexpr int PPL = CH * PS;               // elements per P plane
  static constexpr int MUPL = OCT ? CH * MUS : SR * MUS;  // elements per mu plane
  // LDS carve-up (bytes, 16-aligned); Q, P and phi exist in the output pass
  // only.  The normaliser is double-buffered across chunks (read the state
  // before the chunk, write the state after it); the phi/mu slab tiles are
  // double-buffered across slabs when the budget allows, so that the next
  // slab is generated while this one is contracted.
  static constexpr int al(int b) { return (b + 15) / 16 * 16; }
  static constexpr int TABB = UNR ? 0 : al((OCT ? WI / 8 : WP) * 4);  // row codes / octet descriptors
  static constexpr int B_PHI = OUT ? al(CH * PHS * ES) : 0;
  static constexpr int B_MU = al(NMU * MUPL * ES);
  // partial num and normaliser tiles of the row parts (none with one row part)
  static constexpr int RED_BYTES = (OUT && NRP > 1) ? NW * QT * 64 * 16 * 2 : 0;
  static constexpr int lds_for(int nbuf) {
    const int fixed = TABB + al(CH * XS * ES) * (OUT ? 2 : 1) + al(GC * VS * ES) + (OUT ? al(NPP * PPL * ES) : 0) +
                      al(2 * RWG * 4) + al(CH * 4);
    const int slabs = nbuf * (B_PHI + B_MU);
    return fixed + (slabs > RED_BYTES ? slabs : RED_BYTES);
  }
  static constexpr int NBUF = lds_for(2) <= 160 * 1024 ? 2 : 1;
  static constexpr int O_TAB = 0;
  static constexpr int O_K = O_TAB + TABB;
  static constexpr int O_Q = O_K + al(CH * XS * ES);
  static constexpr int O_V = O_Q + (OUT ? al(CH * XS * ES) : 0);
  static constexpr int O_P = O_V + al(GC * VS * ES);
  static constexpr int O_DEN = O_P + (OUT ? al(NPP * PPL * ES) : 0);
  static constexpr int O_DENQ = O_DEN + al(2 * RWG * 4);
  static constexpr int O_PHI = O_DENQ + al(CH * 4);
  static constexpr int O_MU = O_PHI + NBUF * B_PHI;
  static constexpr int O_END = O_MU + NBUF * B_MU;
  static constexpr int LDS = (O_END > O_PHI + RED_BYTES ? O_END : O_PHI + RED_BYTES);
  static_assert(LDS == lds_for(NBUF), "LDS carve-up");
  // whether the tiles of this shape and chunk length fit the 160 KB of LDS of
  // a CU (always for 64-token chunks; the plan refuses a chunk length whose
  // tiles do not fit)
  static constexpr bool FITS = LDS <= 160 * 1024;
  static_assert(FITS || CH != 64, "LDS budget");
  // global -> register staging in 16-byte segments
  static constexpr int EPS = 16 / ES;                // elements per segment
  static constexpr int QSEG = CH * DK / EPS;         // segments of a Q or K chunk
  static constexpr int VSEG = CH * GC / EPS;         // segments of a V chunk (group columns)
  static constexpr int NQS = (QSEG + NTHR - 1) / NTHR;
  static constexpr int NVS = (VSEG + NTHR - 1) / NTHR;
};

template <int NT>
__device__ inline float taylor_poly(float x) {
  // K_n(x) = sum_{m<n} x^m/m!  by Horner, coefficients 1/m! in fp32
  constexpr float c[6] = {1.0f, 1.0f, 0.5f, 1.0f / 6.0f, 1.0f / 24.0f, 1.0f / 120.0f};
  float p = c[NT - 1];
#pragma unroll
  for (int m = NT - 2; m >= 0; --m) p = fmaf(p, x, c[m]);
  return p;
}

// (key block, query tile) pairs of the causal intra-chunk block, key blocks
// of KB tokens against 16-query tiles: pair p -> (kb[p], qt[p]), every query
// tile that reaches a key of the block, ordered by key block.
template <int CH, int KB>
struct PairTable {
  static constexpr int count() {
    int n = 0;
    for (int kb = 0; kb < CH / KB; ++kb)
      for (int qt = 0; qt < CH / 16; ++qt) n += (qt * 16 + 15 >= kb * KB) ? 1 : 0;
    return n;
  }
  static constexpr int N = count();
  int kb[N], qt[N];
  constexpr PairTable() : kb(), qt() {
    int n = 0;
    for (int b = 0; b < CH / KB; ++b)
      for (int t = 0; t < CH / 16; ++t)
        if (t * 16 + 15 >= b * KB) {
          kb[n] = b;
          qt[n] = t;
          ++n;
        }
  }
  static __device__ const PairTable& get() {
    static constexpr PairTable t{};
    return t;
  }
};

// bf16 accumulator-tile row for M index i of tile tau: 8*(i/4) + 4*tau + i%4
__device__ inline int rho(int tau, int i) { return 8 * (i >> 2) + 4 * tau + (i & 3); }

__device__ inline u32x4 lds_u32x4(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(base + byte_off);
}
__device__ inline f32x4 lds_f32x4(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const f32x4*>(base + byte_off);
}

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t b) { return bf16_to_f32(b); }

// Feature generation with every row index known at compile time (small W).
// Lane = token; wave w takes the groups of G consecutive rows g == w (mod NW).
// phi rows (query side, weight folded in, row 0 left out) go to the
// row-contiguous tile sPhi[token][row] as one 16-byte store per group; mu rows
// (key side) go to sMu[row][token] (hi and, in the totals pass, lo planes).
template <class C>
__device__ __attribute__((always_inline)) inline void gen_unrolled(int sl, int w, int lane, int nvalid, const typename C::Elem* sQ,
                                    const typename C::Elem* sK, typename C::Elem* sPhi, typename C::Elem* sMu) {
  using Elem = typename C::Elem;
  constexpr bool BF = C::BF;
  constexpr int G = BF ? 8 : 4;  // rows per 16-byte group
  constexpr int NG = C::SR / G;
  constexpr RowTable<C::DK, max_terms(C::DK)> tab{};
  float xk[C::DK], xq[C::DK];
  if constexpr (BF) {
#pragma unroll
    for (int d8 = 0; d8 < C::DK / 8; ++d8) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(sK + lane * C::XS + 8 * d8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xk[8 * d8 + 2 * e] = __uint_as_float(a[e] << 16);
        xk[8 * d8 + 2 * e + 1] = __uint_as_float(a[e] & 0xFFFF0000u);
      }
      if constexpr (C::OUT) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(sQ + lane * C::XS + 8 * d8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xq[8 * d8 + 2 * e] = __uint_as_float(b[e] << 16);
          xq[8 * d8 + 2 * e + 1] = __uint_as_float(b[e] & 0xFFFF0000u);
        }
      }
    }
  } else {
#pragma unroll
    for (int d = 0; d < C::DK; ++d) {
      xk[d] = to_f32(sK[lane * C::XS + d]);
      if constexpr (C::OUT) xq[d] = to_f32(sQ[lane * C::XS + d]);
    }
  }
  // staged K rows past the sequence end are zero, so only the constant m = 0 row needs the mask
  const float kmask = lane < nvalid ? 1.f : 0.f;
  auto mono = [&](const float* x, auto Rc) -> float {
    constexpr int R = decltype(Rc)::value;
    constexpr uint32_t code = R < C::W ? tab.code[R] : kPadRow;
    constexpr int m = row_order(code);
    if constexpr (m == 7) {
      return 0.f;
    } else {
      float p = 1.f;
      static_for<0, m>([&](auto lc) { p *= x[row_index_c<C::DK>(code, decltype(lc)::value)]; });
      return p;
    }
  };
  static_for<0, C::NSLAB>([&](auto slc) {
    constexpr int SL = decltype(slc)::value;
    if (SL != sl) return;
    static_for<0, NG>([&](auto gc) {
      constexpr int GI = decltype(gc)::value;
      if (GI % C::NW != w) return;
      constexpr int RB = SL * C::SR + GI * G;  // first row of the group
      float mu[G];
      static_for<0, G>([&](auto uc) {
        constexpr int U = decltype(uc)::value;
        if constexpr (RB + U == 0) mu[U] = kmask;
        else mu[U] = mono(xk, std::integral_constant<int, RB + U>{});
      });
      if constexpr (C::OUT) {
        float ph[G];
        static_for<0, G>([&](auto uc) {
          constexpr int U = decltype(uc)::value;
          constexpr int R = RB + U;
          constexpr uint32_t code = R < C::W ? tab.code[R] : kPadRow;
          if constexpr (R == 0 || R >= C::W) ph[U] = 0.f;
          else ph[U] = row_weight(code) * mono(xq, std::integral_constant<int, R>{});
        });
        if constexpr (BF) {
          u32x4 pk = {pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3]), pack_bf16x2(ph[4], ph[5]),
                      pack_bf16x2(ph[6], ph[7])};
          *reinterpret_cast<u32x4*>(sPhi + lane * C::PHS + GI * G) = pk;
        } else {
          *reinterpret_cast<f32x4*>(sPhi + lane * C::PHS + GI * G) = f32x4{ph[0], ph[1], ph[2], ph[3]};
        }
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if constexpr (BF) {
          uint16_t hi, lo;
          split_bf16(mu[u], hi, lo);
          sMu[(GI * G + u) * C::MUS + lane] = hi;
          if constexpr (!C::OUT) sMu[C::MUPL + (GI * G + u) * C::MUS + lane] = lo;
        } else {
          sMu[(GI * G + u) * C::MUS + lane] = mu[u];
        }
      }
    });
  });
}


// Octet generator (bf16, octet row order): wave w builds the octets of slab sl
// with index == w (mod NW), lane = token.  phi (row 0 excluded: the order-0
// term is added in fp32; weight 1/2 on b == a) to sPhi[token][row]; mu to the
// token-major sMu[token][row], hi and (totals pass) lo planes split exactly.
template <class C>
__device__ __attribute__((always_inline)) inline void gen_octets(int sl, int w, int lane, int nvalid, const uint32_t* tab, const uint16_t* sQ,
                                  const uint16_t* sK, uint16_t* sPhi, uint16_t* sMu) {
  constexpr int NOS = C::SR / 8;
  constexpr int NO = OctTable<C::DK>::NO;
  const float kmask = lane < nvalid ? 1.f : 0.f;
  auto unpack8 = [](const u32x4 v, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(v[e] << 16);
      x[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
    }
  };
  for (int oi = w; oi < NOS; oi += C::NW) {
    const int o = sl * NOS + oi;
    const uint32_t d = __builtin_amdgcn_readfirstlane(o < NO ? tab[o] : 0xFFu);  // wave-uniform: scalar branches
    const int m = d & 0xFF, a = (d >> 8) & 0xFF, b0 = (int)(d >> 16);
    float mu[8], ph[8];
    if (m == 2) {
      // x_a * x[b0 + u] straight from packed bf16: a bf16 dot product with
      // one zero term is the exact product (16 significant bits) in fp32
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      auto prod8 = [](uint32_t xa_bits, const u32x4 xb, float* out) {
        const bf16x2_t lo = __builtin_bit_cast(bf16x2_t, xa_bits);        // {x_a, 0}
        const bf16x2_t hi = __builtin_bit_cast(bf16x2_t, xa_bits << 16);  // {0, x_a}
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the element goes through a scalar first: bit-casting the vector
          // element expression directly made clang reuse element 0 for all e
          const uint32_t w = xb[e];
          const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
          out[2 * e] = __builtin_amdgcn_fdot2_f32_bf16(lo, v, 0.f, false);
          out[2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(hi, v, 0.f, false);
        }
      };
      prod8((uint32_t)sK[lane * C::XS + a], *reinterpret_cast<const u32x4*>(sK + lane * C::XS + b0), mu);
      if constexpr (C::OUT)
        prod8((uint32_t)sQ[lane * C::XS + a], *reinterpret_cast<const u32x4*>(sQ + lane * C::XS + b0), ph);
      if (b0 <= a) {  // the octet holding the diagonal b == a (wave-uniform): rows b < a are zero,
                      // and the query weight of (a, a) is 1/2
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          mu[u] = b0 + u >= a ? mu[u] : 0.f;
          if constexpr (C::OUT) ph[u] = b0 + u > a ? ph[u] : (b0 + u == a ? 0.5f * ph[u] : 0.f);
        }
      }
    } else if (m == 1) {
      unpack8(*reinterpret_cast<const u32x4*>(sK + lane * C::XS + b0), mu);
      if constexpr (C::OUT) unpack8(*reinterpret_cast<const u32x4*>(sQ + lane * C::XS + b0), ph);
    } else {  // order 0 (row 0 only) or past the last octet
#pragma unroll
      for (int u = 0; u < 8; ++u) { mu[u] = (m == 0 && u == 0) ? kmask : 0.f; ph[u] = 0.f; }
    }
    const int rl = oi * 8;
    if constexpr (C::OUT) {
      *reinterpret_cast<u32x4*>(sPhi + lane * C::PHS + rl) =
          u32x4{pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3]), pack_bf16x2(ph[4], ph[5]), pack_bf16x2(ph[6], ph[7])};
      *reinterpret_cast<u32x4*>(sMu + lane * C::MUS + rl) =
          u32x4{pack_bf16x2(mu[0], mu[1]), pack_bf16x2(mu[2], mu[3]), pack_bf16x2(mu[4], mu[5]), pack_bf16x2(mu[6], mu[7])};
    } else {
      // rows are products of at most two bf16 values: hi = truncation, lo = rest, both exact
      uint32_t hb[8], lb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        hb[u] = __float_as_uint(mu[u]) & 0xFFFF0000u;
        lb[u] = __float_as_uint(mu[u] - __uint_as_float(hb[u]));
      }
      auto pk = [](const uint32_t* x) {
        return u32x4{__builtin_amdgcn_perm(x[1], x[0], 0x07060302u), __builtin_amdgcn_perm(x[3], x[2], 0x07060302u),
                     __builtin_amdgcn_perm(x[5], x[4], 0x07060302u), __builtin_amdgcn_perm(x[7], x[6], 0x07060302u)};
      };
      *reinterpret_cast<u32x4*>(sMu + lane * C::MUS + rl) = pk(hb);
      *reinterpret_cast<u32x4*>(sMu + C::MUPL + lane * C::MUS + rl) = pk(lb);
    }
  }
}

// Run generator (table-driven rows, any order): wave w builds the rows
// [w*RPW, (w+1)*RPW) of slab sl, lane = token.  Consecutive rows of one order
// that share all but their last index form a run; the product over the shared
// indices is kept for the run, so a row costs one coordinate read and one
// multiply per side.  phi rows (query side, weight folded in, row 0 left out)
// go to sPhi[token][row] in 16-byte stores; mu rows to sMu[row][token].
template <class C>
__device__ __attribute__((always_inline)) inline void gen_runs(int sl, int w, int lane, int nvalid, const uint32_t* tab,
                                const typename C::Elem* sQ, const typename C::Elem* sK, typename C::Elem* sPhi,
                                typename C::Elem* sMu) {
  using Elem = typename C::Elem;
  constexpr int RPW = C::SR / C::NW;  // rows per wave
  constexpr int G = C::BF ? 8 : 4;    // rows per 16-byte phi store
  static_assert(RPW % G == 0, "rows per wave must fill whole phi stores");
  const int rb = w * RPW;
  const uint32_t* trow = tab + sl * C::SR + rb;
  const float kmask = lane < nvalid ? 1.f : 0.f;
  const Elem* xq = sQ + lane * C::XS;
  const Elem* xk = sK + lane * C::XS;
  uint32_t pkey = 0xFFFFFFFFu;  // order and leading indices of the run in progress
  float pq = 1.f, pk = 1.f;
  for (int g0 = 0; g0 < RPW; g0 += G) {
    uint32_t codes[G];
#pragma unroll
    for (int c4 = 0; c4 < G / 4; ++c4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(trow + g0 + 4 * c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) codes[4 * c4 + e] = __builtin_amdgcn_readfirstlane(v[e]);
    }
    float ph[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const uint32_t code = codes[u];
      const int m = row_order(code);
      float mu = 0.f, phv = 0.f;
      if (m == 0) {
        mu = kmask;
      } else if (m < 7) {
        const uint32_t key = (code & ((1u << (index_bits(C::DK) * (m - 1))) - 1u)) | ((uint32_t)m << 24);
        if (key != pkey) {
          pkey = key;
          pq = 1.f;
          pk = 1.f;
          for (int l = 0; l < m - 1; ++l) {
            const int ix = row_index<C::DK>(code, l);
            pk *= to_f32(xk[ix]);
            if constexpr (C::OUT) pq *= to_f32(xq[ix]);
          }
        }
        const int il = row_index<C::DK>(code, m - 1);
        mu = pk * to_f32(xk[il]);
        if constexpr (C::OUT) phv = row_weight(code) * pq * to_f32(xq[il]);
      }
      ph[u] = phv;
      const int rl = rb + g0 + u;
      if constexpr (C::BF) {
        uint16_t hi, lo;
        split_bf16(mu, hi, lo);
        sMu[rl * C::MUS + lane] = hi;
        if constexpr (!C::OUT) sMu[C::MUPL + rl * C::MUS + lane] = lo;
      } else {
        sMu[rl * C::MUS + lane] = mu;
      }
    }
    if constexpr (C::OUT) {
      Elem* dst = sPhi + lane * C::PHS + rb + g0;
      if constexpr (C::BF) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3]),
                                               pack_bf16x2(ph[4], ph[5]), pack_bf16x2(ph[6], ph[7])};
      } else {
        *reinterpret_cast<f32x4*>(dst) = f32x4{ph[0], ph[1], ph[2], ph[3]};
      }
    }
  }
}

// Feature generation for the row groups g == part (mod nparts) of all WP rows,
// lane = token; xq/xk hold the token's query and key coordinates.  Both sides
// go to token-major tiles with one 16-byte store per group of 8 rows: phi to
// sPhi[token][row], mu to sMu[token][row] (hi, and lo in the totals pass),
// which the update reads back through transposing LDS reads.
template <class C>
__device__ __attribute__((always_inline)) inline void gen_groups(int part, int nparts, int lane, int nvalid, const float* xq, const float* xk,
                                  typename C::Elem* sPhi, typename C::Elem* sMu) {
  constexpr int G = 8;
  constexpr int NG = C::WP / G;
  constexpr RowTable<C::DK, max_terms(C::DK)> tab{};
  const float kmask = lane < nvalid ? 1.f : 0.f;
  auto mono = [&](const float* x, auto Rc) -> float {
    constexpr int R = decltype(Rc)::value;
    constexpr uint32_t code = R < C::W ? tab.code[R] : kPadRow;
    constexpr int m = row_order(code);
    if constexpr (m == 7) {
      return 0.f;
    } else {
      float p = 1.f;
      static_for<0, m>([&](auto lc) { p *= x[row_index_c<C::DK>(code, decltype(lc)::value)]; });
      return p;
    }
  };
  // chunk swizzle and row shift of the token-major mu tile (PCfg::MUSWZ,
  // PCfg::MUSH): 16-byte chunks go out as two 8-byte halves
  const int mswz = C::MUSWZ ? ((lane >> 2) & 3) : 0;
  typename C::Elem* muRow = sMu + lane * C::MUS + C::MUSH * (lane >> 3);
  auto st_mu = [&](typename C::Elem* dst, u32x4 v) {
    if constexpr (C::MUSWZ) {
      reinterpret_cast<uint2*>(dst)[0] = uint2{v.x, v.y};
      reinterpret_cast<uint2*>(dst)[1] = uint2{v.z, v.w};
    } else {
      *reinterpret_cast<u32x4*>(dst) = v;
    }
  };
  static_for<0, NG>([&](auto gc) {
    constexpr int GI = decltype(gc)::value;
    if (GI % nparts != part) return;
    constexpr int RB = GI * G;
    const int MB = (GI ^ mswz) * G;  // where chunk GI of this token lives
    float mu[G];
    static_for<0, G>([&](auto uc) {
      constexpr int U = decltype(uc)::value;
      if constexpr (RB + U == 0) mu[U] = kmask;
      else mu[U] = mono(xk, std::integral_constant<int, RB + U>{});
    });
    if constexpr (C::OUT) {
      float ph[G];
      static_for<0, G>([&](auto uc) {
        constexpr int U = decltype(uc)::value;
        constexpr int R = RB + U;
        constexpr uint32_t code = R < C::W ? tab.code[R] : kPadRow;
        if constexpr (R == 0 || R >= C::W) ph[U] = 0.f;
        else ph[U] = row_weight(code) * mono(xq, std::integral_constant<int, R>{});
      });
      u32x4 pk = {pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3]), pack_bf16x2(ph[4], ph[5]),
                  pack_bf16x2(ph[6], ph[7])};
      *reinterpret_cast<u32x4*>(sPhi + lane * C::PHS + RB) = pk;
    }
    if constexpr (C::OUT) {
      st_mu(muRow + MB, u32x4{pack_bf16x2(mu[0], mu[1]), pack_bf16x2(mu[2], mu[3]), pack_bf16x2(mu[4], mu[5]),
                              pack_bf16x2(mu[6], mu[7])});
    } else {
      // exact split: rows are products of at most two bf16 values (n <= 3 here),
      // so mu has at most 16 significant bits; hi = mu truncated to bf16 and
      // lo = mu - hi (exact, at most 8 significant bits, so also a bf16)
      static_assert(C::NT <= 3, "two-factor rows only");
      uint32_t hb[G], lb[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        hb[u] = __float_as_uint(mu[u]) & 0xFFFF0000u;
        lb[u] = __float_as_uint(mu[u] - __uint_as_float(hb[u]));
      }
      auto pk = [](const uint32_t* x) {  // upper halves of two words per dword
        return u32x4{__builtin_amdgcn_perm(x[1], x[0], 0x07060302u), __builtin_amdgcn_perm(x[3], x[2], 0x07060302u),
                     __builtin_amdgcn_perm(x[5], x[4], 0x07060302u), __builtin_amdgcn_perm(x[7], x[6], 0x07060302u)};
      };
      st_mu(muRow + MB, pk(hb));
      st_mu(muRow + C::MUPL + MB, pk(lb));
    }
  });
}

template <class C>
__global__ __launch_bounds__(C::NTHR) void sweep_kernel(const typename C::TIn* __restrict__ Qg,
                                                        const typename C::TIn* __restrict__ Kg,
                                                        const typename C::TIn* __restrict__ Vg, int N,
                                                        int span, int nspan, float* __restrict__ ws,
                                                        float* __restrict__ part, float* __restrict__ Og,
                                                        float* __restrict__ Dg) {
  using TIn = typename C::TIn;
  using Elem = typename C::Elem;
  constexpr bool BF = C::BF;
  constexpr bool OUT = C::OUT;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS];

  uint32_t* sTab = reinterpret_cast<uint32_t*>(lds + C::O_TAB);
  Elem* sQ = reinterpret_cast<Elem*>(lds + C::O_Q);
  Elem* sK = reinterpret_cast<Elem*>(lds + C::O_K);
  Elem* sV = reinterpret_cast<Elem*>(lds + C::O_V);
  Elem* sP = reinterpret_cast<Elem*>(lds + C::O_P);
  float* sDen = reinterpret_cast<float*>(lds + C::O_DEN);  // [2][RWG]: state before / after the chunk
  float* sDenQ = reinterpret_cast<float*>(lds + C::O_DENQ);
  auto phi_buf = [&](int b) { return reinterpret_cast<Elem*>(lds + C::O_PHI + b * C::B_PHI); };
  auto mu_buf = [&](int b) { return reinterpret_cast<Elem*>(lds + C::O_MU + b * C::B_MU); };
  float* sRed = reinterpret_cast<float*>(lds + C::O_PHI);  // reused after the slabs

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in an SGPR: branches on it are scalar
  const int li = lane & 15;  // i
  const int lg = lane >> 4;  // g
  const int ct = w % C::NVT;  // value column tile of this wave
  const int rp = w / C::NVT;  // row part of this wave
  const int ngroups = kDV / C::GC;
  const int rg = blockIdx.x % C::NRG;                      // row group
  const int grp = (blockIdx.x / C::NRG) % ngroups;         // column group
  const int s_idx = (blockIdx.x / (C::NRG * ngroups)) % nspan;
  const int bh = blockIdx.x / (C::NRG * ngroups * nspan);
  const int slab0 = rg * C::NSLAB;                         // first slab of the row group
  const int nsl = min(C::NSLAB, C::NSLAB_ALL - slab0);     // its slabs (>= 1)
  const int gcol0 = grp * C::GC;  // first value column of the group
  const int t_begin = s_idx * span;
  const int t_end = min(N, t_begin + span);

  const TIn* Qh = Qg + (size_t)bh * N * C::DK;
  const TIn* Kh = Kg + (size_t)bh * N * C::DK;
  const TIn* Vh = Vg + (size_t)bh * N * kDV;
  const size_t ws_span = (size_t)C::WP * (kDV + 1);
  float* wsS = ws + ((size_t)bh * nspan + s_idx) * ws_span;
  // partial outputs of the row groups: numerators [BH][NRG][N][dv], then normalisers [BH][NRG][N]
  const int nbh = gridDim.x / (C::NRG * ngroups * nspan);
  float* pnum = part + ((size_t)bh * C::NRG + rg) * N * kDV;
  float* pden = part + (size_t)nbh * C::NRG * N * kDV + ((size_t)bh * C::NRG + rg) * N;
  (void)pnum;
  (void)pden;

  // feature-row codes for the table-driven generator; padded rows contribute nothing
  if constexpr (C::OCT) {
    const auto& tab = OctOf<C::DK>::get();
    for (int r = tid; r < C::WI / 8; r += C::NTHR) sTab[r] = tab.d[r];
  } else if constexpr (!C::UNR) {
    const auto& tab = RowsOf<C::DK>::get();
    for (int r = tid; r < C::WP; r += C::NTHR) sTab[r] = (r < C::W) ? tab.code[r] : kPadRow;
  }

  // state registers: st[j][tau], K-block kb = (slab*NRP + rp)*J + j%J
  f32x4 st[C::MKB][C::TPK];
#pragma unroll
  for (int j = 0; j < C::MKB; ++j)
#pragma unroll
    for (int t = 0; t < C::TPK; ++t) st[j][t] = zero4();

  auto kb_of = [&](int j) { return ((slab0 + j / C::J) * C::NRP + rp) * C::J + (j % C::J); };
  // feature row held by lane (col, g) at register s of tile tau of K-block kb
  auto acc_row = [&](int kb, int tau, int s) {
    return BF ? kb * C::KB + 8 * lg + 4 * tau + s : kb * C::KB + 4 * lg + s;
  };

  if constexpr (OUT) {
    // start from the exclusive prefix of this span (the row group's slabs)
#pragma unroll
    for (int j = 0; j < C::MKB; ++j) {
      if (j / C::J >= nsl) continue;
      const int kb = kb_of(j);
#pragma unroll
      for (int t = 0; t < C::TPK; ++t) {
        f32x4 v;
        v.x = wsS[(size_t)acc_row(kb, t, 0) * kDV + gcol0 + ct * 16 + li];
        v.y = wsS[(size_t)acc_row(kb, t, 1) * kDV + gcol0 + ct * 16 + li];
        v.z = wsS[(size_t)acc_row(kb, t, 2) * kDV + gcol0 + ct * 16 + li];
        v.w = wsS[(size_t)acc_row(kb, t, 3) * kDV + gcol0 + ct * 16 + li];
        st[j][t] = v;
      }
    }
    for (int r = tid; r < C::RWG; r += C::NTHR)
      sDen[r] = r < nsl * C::SR ? wsS[(size_t)C::WP * kDV + slab0 * C::SR + r] : 0.f;
  } else {
    for (int r = tid; r < C::RWG; r += C::NTHR) sDen[r] = 0.f;
  }
  __syncthreads();

  const u32x4 ones_bf = (li == 0) ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                                  : u32x4{0u, 0u, 0u, 0u};
  const float ones_f = (li == 0) ? 1.0f : 0.0f;

  // Chunk staging: every thread owns fixed 16-byte segments of the Q, K and V
  // tiles; the next chunk's segments are loaded into registers while the
  // current chunk is computed.
  u32x4 rq[C::NQS], rk[C::NQS], rv[C::NVS];
  auto issue = [&](int c0n) {
#pragma unroll
    for (int i = 0; i < C::NQS; ++i) {
      const int seg = tid + i * C::NTHR;
      const int tok = seg / (C::DK / C::EPS);
      const int part = seg - tok * (C::DK / C::EPS);
      const bool ok = seg < C::QSEG && c0n + tok < t_end;
      const size_t off = (size_t)(c0n + tok) * C::DK + part * C::EPS;
      rk[i] = ok ? *reinterpret_cast<const u32x4*>(Kh + off) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (OUT) rq[i] = ok ? *reinterpret_cast<const u32x4*>(Qh + off) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < C::NVS; ++i) {  // segment = (column group, token): lanes walk tokens
      const int seg = tid + i * C::NTHR;
      const int tok = seg % C::CH;
      const int part = seg / C::CH;
      const bool ok = seg < C::VSEG && c0n + tok < t_end;
      const size_t off = (size_t)(c0n + tok) * kDV + gcol0 + part * C::EPS;
      rv[i] = ok ? *reinterpret_cast<const u32x4*>(Vh + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int i = 0; i < C::NQS; ++i) {
      const int seg = tid + i * C::NTHR;
      if (seg < C::QSEG) {
        const int tok = seg / (C::DK / C::EPS);
        const int part = seg - tok * (C::DK / C::EPS);
        if constexpr (BF) {
          // 16-byte aligned rows: one vector store per segment
          *reinterpret_cast<u32x4*>(sK + tok * C::XS + part * C::EPS) = rk[i];
          if constexpr (OUT) *reinterpret_cast<u32x4*>(sQ + tok * C::XS + part * C::EPS) = rq[i];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sK[tok * C::XS + part * 4 + e] = __uint_as_float(rk[i][e]);
            if constexpr (OUT) sQ[tok * C::XS + part * 4 + e] = __uint_as_float(rq[i][e]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVS; ++i) {
      const int seg = tid + i * C::NTHR;
      if (seg < C::VSEG) {
        const int tok = seg % C::CH;
        const int col0 = (seg / C::CH) * C::EPS;
        if constexpr (BF) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sV[(col0 + e) * C::VS + tok] = (Elem)((rv[i][e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) sV[(col0 + e) * C::VS + tok] = __uint_as_float(rv[i][e]);
        }
      }
    }
  };

  issue(t_begin);
  int db = 0;  // normaliser buffer holding the state before the current chunk
  for (int c0 = t_begin; c0 < t_end; c0 += C::CH) {
    const int nvalid = min(C::CH, t_end - c0);
    const float* Den = sDen + db * C::RWG;  // rows of the row group
    float* DenN = sDen + (db ^ 1) * C::RWG;

    // ---- 1. stage this chunk, start loading the next ----
    commit();
    __syncthreads();
    if (c0 + C::CH < t_end) issue(c0 + C::CH);
    // V^T fragments, once per chunk (bf16): the totals remap's J column tiles, or
    // this wave's column tile in the output pass
    u32x4 vfr[C::TR && BF ? C::J : 1][C::TB];
    if constexpr (OUT && BF) {
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb)
        vfr[0][tb] = lds_u32x4((const unsigned char*)sV, ((ct * 16 + li) * C::VS + tb * 32 + 8 * lg) * 2);
    }
    if constexpr (C::TR && BF) {
#pragma unroll
      for (int c = 0; c < C::J; ++c)
#pragma unroll
        for (int tb = 0; tb < C::TB; ++tb)
          vfr[c][tb] = lds_u32x4((const unsigned char*)sV,
                                 ((((w % C::WPK) * C::J + c) * 16 + li) * C::VS + tb * 32 + 8 * lg) * 2);
    }

    // ---- 2. intra-chunk block P = tril(K_n(Q K^T)) (output pass) ----
    f32x4 num[C::QT];
    f32x4 den[C::QT];
#pragma unroll
    for (int q = 0; q < C::QT; ++q) { num[q] = zero4(); den[q] = zero4(); }
    float m0 = 0.f, den0 = 0.f;
    // the intra-chunk block and the m = 0 row belong to the row group holding row 0
    if constexpr (OUT) if (rg == 0) {
      // (key block, query tile) pairs on or below the diagonal: key blocks
      // of 32 (bf16) meet query tiles qt >= 2 kb, key blocks of 16 (fp32)
      // query tiles qt >= kb; pair p decodes as (kb, qt) in order of kb
      using PT = PairTable<C::CH, C::KB>;
      constexpr int NTILE = PT::N * C::TPK;
      for (int ti = w; ti < NTILE; ti += C::NW) {
        const int pair = ti / C::TPK, tau = ti % C::TPK;
        const int kb = PT::get().kb[pair], qt = PT::get().qt[pair];
        const int key_row = BF ? kb * 32 + rho(tau, li) : kb * 16 + li;  // A operand row (key)
        const int qry_row = qt * 16 + li;                                // B operand column (query)
        f32x4 x = zero4();
        if constexpr (BF) {
          if constexpr (C::DK == 16) {
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            const uint2 a = *reinterpret_cast<const uint2*>(sK + key_row * C::XS + 4 * lg);
            const uint2 b = *reinterpret_cast<const uint2*>(sQ + qry_row * C::XS + 4 * lg);
            x = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                          __builtin_bit_cast(s16x4, b), x, 0, 0, 0);
          } else {
#pragma unroll
            for (int h = 0; h < C::DK / 32; ++h) {
              const u32x4 a = *reinterpret_cast<const u32x4*>(sK + key_row * C::XS + 32 * h + 8 * lg);
              const u32x4 b = *reinterpret_cast<const u32x4*>(sQ + qry_row * C::XS + 32 * h + 8 * lg);
              x = mfma_bf16(a, b, x);
            }
          }
        } else {
#pragma unroll
          for (int jd = 0; jd < C::DK / 4; ++jd)
            x = mfma_f32(sK[key_row * C::XS + 4 * jd + lg], sQ[qry_row * C::XS + 4 * jd + lg], x);
        }
        // lane (query = qt*16 + li, g) holds keys key_of(s)
        const int query = qt * 16 + li;
        float p[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int key = BF ? kb * 32 + 8 * lg + 4 * tau + s : kb * 16 + 4 * lg + s;
          p[s] = (key <= query && key < nvalid) ? taylor_poly<C::NT>(x[s]) : 0.f;
        }
        const int kbase = BF ? kb * 32 + 8 * lg + 4 * tau : kb * 16 + 4 * lg;
        if constexpr (BF) {
          uint2 hi, lo;
          split_bf16x2(p[0], p[1], hi.x, lo.x);
          split_bf16x2(p[2], p[3], hi.y, lo.y);
          *reinterpret_cast<uint2*>(&sP[query * C::PS + kbase]) = hi;
          *reinterpret_cast<uint2*>(&sP[C::PPL + query * C::PS + kbase]) = lo;
        } else {
          *reinterpret_cast<f32x4*>(&sP[query * C::PS + kbase]) = f32x4{p[0], p[1], p[2], p[3]};
        }
      }
      // m = 0 row (exact in fp32): S[0][cols] and the token count S[0][dv]
      m0 = __shfl(st[0][0].x, li);  // lane (col, g = 0) holds row 0 of K-block 0 (rp = 0 only)
      den0 = Den[0];
    }

    // ---- 3. feature slabs: readout (output pass) then update ----
    // phi / mu tiles of slab sl (compile-time) into the given buffers
    // (the generators take one token per lane; a chunk of 128 tokens is two
    // token slots per lane, a chunk shorter than 64 leaves lanes idle)
    auto gen_slab = [&](auto slc, Elem* sPhi, Elem* sMu) {
      constexpr int sl = decltype(slc)::value;
#pragma unroll
      for (int h = 0; h < C::NTS; ++h) {
        const int tok = lane + 64 * h;
        if (tok >= C::CH) break;
        if constexpr (C::UNR) {
          gen_unrolled<C>(sl, w, tok, nvalid, sQ, sK, sPhi, sMu);
        } else if constexpr (C::OCT) {
          gen_octets<C>(slab0 + sl, w, tok, nvalid, sTab, sQ, sK, sPhi, sMu);
        } else {
          gen_runs<C>(slab0 + sl, w, tok, nvalid, sTab, sQ, sK, sPhi, sMu);
        }
      }
    };
    gen_slab(std::integral_constant<int, 0>{}, phi_buf(0), mu_buf(0));
    __syncthreads();
    // slabs unrolled at compile time so that every state register index is static
    static_for<0, C::NSLAB>([&](auto slc) {
      constexpr int sl = decltype(slc)::value;
      if (sl >= nsl) return;  // past the row group's last slab (uniform)
      const int row0 = sl * C::SR;  // first row of the slab within the row group
      Elem* const sPhi = phi_buf(sl % C::NBUF);
      Elem* const sMu = mu_buf(sl % C::NBUF);
      (void)sPhi;
      if constexpr (OUT) {
        // value readout over this wave's K-blocks of the slab; with the same phi
        // fragments, the normaliser readout of the query tiles qt == ct (mod NVT)
        // over these K-blocks (partials over the row parts are added per chunk)
#pragma unroll
        for (int jl = 0; jl < C::J; ++jl) {
          const int j = sl * C::J + jl;
          const int kbl = rp * C::J + jl;  // K-block within the slab
          if constexpr (BF) {
            // the state and the normaliser rows enter the readout as hi + lo
            // bf16 (16 significant bits): rounded to one bf16 each, values and
            // normaliser would round independently and move an output by
            // about 2^-9 |o|
            u32x4 b, bl;
            split_bf16x8(st[j][0], st[j][C::TPK - 1], b, bl);
            u32x4 bd = {0u, 0u, 0u, 0u}, bdl = {0u, 0u, 0u, 0u};  // normaliser rows of the K-block in column 0
            if (li == 0) {
              const f32x4 d0 = *reinterpret_cast<const f32x4*>(Den + row0 + kbl * 32 + 8 * lg);
              const f32x4 d1 = *reinterpret_cast<const f32x4*>(Den + row0 + kbl * 32 + 8 * lg + 4);
              split_bf16x8(d0, d1, bd, bdl);
            }
            // all four fragments are read before the first MFMA: the normaliser
            // MFMAs below sit behind wave-uniform branches, which the compiler
            // does not move loads across
            u32x4 a[C::QT];
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt)
              a[qt] = lds_u32x4((const unsigned char*)sPhi, ((qt * 16 + li) * C::PHS + kbl * 32 + 8 * lg) * 2);
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) num[qt] = mfma_bf16(a[qt], b, num[qt]);
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) num[qt] = mfma_bf16(a[qt], bl, num[qt]);
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt)
              if (qt % C::NVT == ct) {
                den[qt] = mfma_bf16(a[qt], bd, den[qt]);
                den[qt] = mfma_bf16(a[qt], bdl, den[qt]);
              }
          } else {
            const f32x4 d = *reinterpret_cast<const f32x4*>(Den + row0 + kbl * 16 + 4 * lg);
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) {
              const f32x4 a = lds_f32x4((const unsigned char*)sPhi,
                                        ((qt * 16 + li) * C::PHS + kbl * 16 + 4 * lg) * 4);
              num[qt] = mfma_f32(a.x, st[j][0].x, num[qt]);
              num[qt] = mfma_f32(a.y, st[j][0].y, num[qt]);
              num[qt] = mfma_f32(a.z, st[j][0].z, num[qt]);
              num[qt] = mfma_f32(a.w, st[j][0].w, num[qt]);
              if (qt % C::NVT == ct) {
                den[qt] = mfma_f32(a.x, ones_f * d.x, den[qt]);
                den[qt] = mfma_f32(a.y, ones_f * d.y, den[qt]);
                den[qt] = mfma_f32(a.z, ones_f * d.z, den[qt]);
                den[qt] = mfma_f32(a.w, ones_f * d.w, den[qt]);
              }
            }
          }
        }
      }

      // bf16 mu^T fragment (A operand, rows rho(tau, i)) of slab K-block kbl, token block tb, plane pl
      auto mu_frag = [&](int pl, int kbl, int tau, int tb) -> u32x4 {
        if constexpr (C::OCT) {  // token-major tile: two transposing reads
          const unsigned char* p = (const unsigned char*)sMu +
              (pl * C::MUPL + (tb * 32 + 8 * lg + (li >> 2)) * C::MUS + kbl * 32 + 8 * (li & 3) + 4 * tau) * 2;
          const uint2 x = lds_tr16(p), y = lds_tr16(p + 4 * C::MUS * 2);
          return u32x4{x.x, x.y, y.x, y.y};
        } else {
          return lds_u32x4((const unsigned char*)sMu,
                           (pl * C::MUPL + (kbl * 32 + rho(tau, li)) * C::MUS + tb * 32 + 8 * lg) * 2);
        }
      };
      if constexpr (C::TR) {
        // totals remap: K-block kbl of the slab, column tiles ct0 .. ct0+J-1 in st[sl*J + c];
        // the first of the K-block's WPK waves also takes its normaliser rows
        const int kbl = w / C::WPK;
        const int ct0 = (w % C::WPK) * C::J;
        const bool den_own = (w % C::WPK) == 0;
        f32x4 dacc[C::TPK];
#pragma unroll
        for (int t = 0; t < C::TPK; ++t) dacc[t] = zero4();
        // bf16: every hi/lo fragment of the K-block is read before the first
        // MFMA (the normaliser MFMAs sit behind a wave-uniform branch)
        u32x4 mfr[BF ? C::TB : 1][2][2];
        if constexpr (BF) {
#pragma unroll
          for (int tb = 0; tb < C::TB; ++tb)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
              mfr[tb][tau][0] = mu_frag(0, kbl, tau, tb);
              mfr[tb][tau][1] = mu_frag(1, kbl, tau, tb);
            }
        }
#pragma unroll
        for (int tb = 0; tb < C::TB; ++tb) {
          if constexpr (BF) {
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
              for (int c = 0; c < C::J; ++c) {
                st[sl * C::J + c][tau] = mfma_bf16(mfr[tb][tau][0], vfr[c][tb], st[sl * C::J + c][tau]);
                st[sl * C::J + c][tau] = mfma_bf16(mfr[tb][tau][1], vfr[c][tb], st[sl * C::J + c][tau]);
              }
            }
          } else {
            const f32x4 a = lds_f32x4((const unsigned char*)sMu, ((kbl * 16 + li) * C::MUS + tb * 16 + 4 * lg) * 4);
#pragma unroll
            for (int c = 0; c < C::J; ++c) {
              const f32x4 b = lds_f32x4((const unsigned char*)sV, (((ct0 + c) * 16 + li) * C::VS + tb * 16 + 4 * lg) * 4);
              f32x4& s4 = st[sl * C::J + c][0];
              s4 = mfma_f32(a.x, b.x, s4);
              s4 = mfma_f32(a.y, b.y, s4);
              s4 = mfma_f32(a.z, b.z, s4);
              s4 = mfma_f32(a.w, b.w, s4);
            }
            if (den_own) {
              dacc[0] = mfma_f32(a.x, ones_f, dacc[0]);
              dacc[0] = mfma_f32(a.y, ones_f, dacc[0]);
              dacc[0] = mfma_f32(a.z, ones_f, dacc[0]);
              dacc[0] = mfma_f32(a.w, ones_f, dacc[0]);
            }
          }
        }
        if constexpr (BF) {
          if (den_own) {  // normaliser rows of the K-block from the same fragments
            constexpr int NPF = (int)(sizeof(mfr[0][0]) / sizeof(mfr[0][0][0]));
#pragma unroll
            for (int tb = 0; tb < C::TB; ++tb)
#pragma unroll
              for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int pl = 0; pl < NPF; ++pl) dacc[tau] = mfma_bf16(mfr[tb][tau][pl], ones_bf, dacc[tau]);
          }
        }
        if (den_own && li == 0) {  // four consecutive normaliser rows per tile: one 16-byte access each way
#pragma unroll
          for (int tau = 0; tau < C::TPK; ++tau) {
            const int r = row0 + (BF ? kbl * 32 + 8 * lg + 4 * tau : kbl * 16 + 4 * lg);
            *reinterpret_cast<f32x4*>(DenN + r) = *reinterpret_cast<const f32x4*>(Den + r) + dacc[tau];
          }
        }
      } else {
      // value update S[kb] += mu^T V; the wave whose column tile is kbl % NVT
      // also takes the normaliser rows DenN = Den + mu^T 1 of the K-block from
      // the same fragments
#pragma unroll
      for (int jl = 0; jl < C::J; ++jl) {
        const int j = sl * C::J + jl;
        const int kbl = rp * C::J + jl;
        const bool den_own = (kbl % C::NVT) == ct;  // wave-uniform
        f32x4 dacc[C::TPK];
#pragma unroll
        for (int t = 0; t < C::TPK; ++t) dacc[t] = zero4();
        // bf16: the K-block's fragments (and V^T in the totals pass) are read
        // before the first MFMA (the normaliser MFMAs sit behind a branch)
        u32x4 mfr[BF ? C::TB : 1][2][OUT ? 1 : 2];
        u32x4 bvt[BF ? C::TB : 1];
        if constexpr (BF) {
#pragma unroll
          for (int tb = 0; tb < C::TB; ++tb) {
            if constexpr (OUT) bvt[tb] = vfr[0][tb];
            else bvt[tb] = lds_u32x4((const unsigned char*)sV, ((ct * 16 + li) * C::VS + tb * 32 + 8 * lg) * 2);
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
              for (int pl = 0; pl < (OUT ? 1 : 2); ++pl) mfr[tb][tau][pl] = mu_frag(pl, kbl, tau, tb);
          }
        }
#pragma unroll
        for (int tb = 0; tb < C::TB; ++tb) {
          if constexpr (BF) {
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
              for (int pl = 0; pl < (OUT ? 1 : 2); ++pl)
                st[j][tau % C::TPK] = mfma_bf16(mfr[tb][tau][pl], bvt[tb], st[j][tau % C::TPK]);
          } else {
            const f32x4 b = lds_f32x4((const unsigned char*)sV, ((ct * 16 + li) * C::VS + tb * 16 + 4 * lg) * 4);
            const f32x4 a = lds_f32x4((const unsigned char*)sMu, ((kbl * 16 + li) * C::MUS + tb * 16 + 4 * lg) * 4);
            st[j][0] = mfma_f32(a.x, b.x, st[j][0]);
            st[j][0] = mfma_f32(a.y, b.y, st[j][0]);
            st[j][0] = mfma_f32(a.z, b.z, st[j][0]);
            st[j][0] = mfma_f32(a.w, b.w, st[j][0]);
            if (den_own) {
              dacc[0] = mfma_f32(a.x, ones_f, dacc[0]);
              dacc[0] = mfma_f32(a.y, ones_f, dacc[0]);
              dacc[0] = mfma_f32(a.z, ones_f, dacc[0]);
              dacc[0] = mfma_f32(a.w, ones_f, dacc[0]);
            }
          }
        }
        if constexpr (BF) {
          if (den_own) {  // normaliser rows of the K-block from the same fragments
            constexpr int NPF = (int)(sizeof(mfr[0][0]) / sizeof(mfr[0][0][0]));
#pragma unroll
            for (int tb = 0; tb < C::TB; ++tb)
#pragma unroll
              for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int pl = 0; pl < NPF; ++pl) dacc[tau] = mfma_bf16(mfr[tb][tau][pl], ones_bf, dacc[tau]);
          }
        }
        if (den_own && li == 0) {  // four consecutive normaliser rows per tile: one 16-byte access each way
#pragma unroll
          for (int tau = 0; tau < C::TPK; ++tau) {
            const int r = row0 + (BF ? kbl * 32 + 8 * lg + 4 * tau : kbl * 16 + 4 * lg);
            *reinterpret_cast<f32x4*>(DenN + r) = *reinterpret_cast<const f32x4*>(Den + r) + dacc[tau];
          }
        }
      }
      }
      // next slab: into the other buffer while this one may still be read,
      // or (single buffer) after every wave is done with this one
      if constexpr (sl + 1 < C::NSLAB) {
        if (sl + 1 < nsl) {
          if constexpr (C::NBUF == 1) __syncthreads();
          gen_slab(std::integral_constant<int, sl + 1>{}, phi_buf((sl + 1) % C::NBUF), mu_buf((sl + 1) % C::NBUF));
        }
      }
      __syncthreads();
    });
    if constexpr (OUT) {
      // ---- 4. intra-chunk contribution, m = 0 row, reduction, normalise ----
      // (with several row groups: partial num / den of this group's rows to
      // the partial buffers, normalised by combine_kernel)
      if (rp == 0 && rg == 0) {
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt) {
          constexpr int KBW = BF ? 32 : 16;
#pragma unroll
          for (int kb = 0; kb < C::CH / KBW; ++kb) {
            if (kb * KBW > qt * 16 + 15) continue;
            if constexpr (BF) {
              const u32x4 b = lds_u32x4((const unsigned char*)sV, ((ct * 16 + li) * C::VS + kb * 32 + 8 * lg) * 2);
              const u32x4 ah = lds_u32x4((const unsigned char*)sP, ((qt * 16 + li) * C::PS + kb * 32 + 8 * lg) * 2);
              const u32x4 al = lds_u32x4((const unsigned char*)sP,
                                         (C::PPL + (qt * 16 + li) * C::PS + kb * 32 + 8 * lg) * 2);
              num[qt] = mfma_bf16(ah, b, num[qt]);
              num[qt] = mfma_bf16(al, b, num[qt]);
            } else {
              const f32x4 b = lds_f32x4((const unsigned char*)sV, ((ct * 16 + li) * C::VS + kb * 16 + 4 * lg) * 4);
              const f32x4 a = lds_f32x4((const unsigned char*)sP, ((qt * 16 + li) * C::PS + kb * 16 + 4 * lg) * 4);
              num[qt] = mfma_f32(a.x, b.x, num[qt]);
              num[qt] = mfma_f32(a.y, b.y, num[qt]);
              num[qt] = mfma_f32(a.z, b.z, num[qt]);
              num[qt] = mfma_f32(a.w, b.w, num[qt]);
            }
          }
          num[qt] += f32x4{m0, m0, m0, m0};
        }
      }
      // row-part partials (numerators, and the normaliser of the owned query
      // tiles qt == ct mod NVT) of the waves with rp != 0 go through LDS
      float* sRedD = sRed + C::NW * C::QT * 64 * 4;
      if constexpr (C::NRP > 1) {
        if (rp != 0) {
#pragma unroll
          for (int qt = 0; qt < C::QT; ++qt) {
            *reinterpret_cast<f32x4*>(sRed + (((w * C::QT + qt) * 64) + lane) * 4) = num[qt];
            *reinterpret_cast<f32x4*>(sRedD + (((w * C::QT + qt) * 64) + lane) * 4) = den[qt];
          }
        }
      }
      __syncthreads();
      if (rp == 0) {
        if constexpr (C::NRP > 1) {
          for (int r2 = 1; r2 < C::NRP; ++r2) {
            const int w2 = r2 * C::NVT + ct;
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) {
              num[qt] += *reinterpret_cast<const f32x4*>(sRed + (((w2 * C::QT + qt) * 64) + lane) * 4);
              den[qt] += *reinterpret_cast<const f32x4*>(sRedD + (((w2 * C::QT + qt) * 64) + lane) * 4);
            }
          }
        }
        // intra-chunk normaliser (row group 0) of the owned query tiles, then publish per query
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt) {
          if (qt % C::NVT != ct) continue;
          constexpr int KBW = BF ? 32 : 16;
#pragma unroll
          for (int kb = 0; kb < C::CH / KBW; ++kb) {
            if (kb * KBW > qt * 16 + 15 || rg != 0) continue;
            if constexpr (BF) {
              const u32x4 ah = lds_u32x4((const unsigned char*)sP, ((qt * 16 + li) * C::PS + kb * 32 + 8 * lg) * 2);
              const u32x4 al = lds_u32x4((const unsigned char*)sP,
                                         (C::PPL + (qt * 16 + li) * C::PS + kb * 32 + 8 * lg) * 2);
              den[qt] = mfma_bf16(ah, ones_bf, den[qt]);
              den[qt] = mfma_bf16(al, ones_bf, den[qt]);
            } else {
              const f32x4 a = lds_f32x4((const unsigned char*)sP, ((qt * 16 + li) * C::PS + kb * 16 + 4 * lg) * 4);
              den[qt] = mfma_f32(a.x, ones_f, den[qt]);
              den[qt] = mfma_f32(a.y, ones_f, den[qt]);
              den[qt] = mfma_f32(a.z, ones_f, den[qt]);
              den[qt] = mfma_f32(a.w, ones_f, den[qt]);
            }
          }
          if (li == 0) {
            if constexpr (C::NRG == 1) {
              // Dg non-null: outputs stay unnormalised and the normalisers go to Dg
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                const float dq = den[qt][s] + den0;
                sDenQ[qt * 16 + 4 * lg + s] = Dg ? 1.0f : rcp_fast(dq);
                if (Dg && qt * 16 + 4 * lg + s < nvalid) Dg[(size_t)bh * N + c0 + qt * 16 + 4 * lg + s] = dq;
              }
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (qt * 16 + 4 * lg + s < nvalid) pden[c0 + qt * 16 + 4 * lg + s] = den[qt][s] + den0;
            }
          }
        }
      }
      if constexpr (C::NRG == 1) __syncthreads();  // every query's 1/den is published
      if (rp == 0) {
        if constexpr (C::NRG > 1) {
          // partial numerator of this row group; lane (col, g) holds queries 4g+s of each query tile
          float* pb = pnum + (size_t)(c0 + 4 * lg) * kDV + gcol0 + ct * 16 + li;
#pragma unroll
          for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
            for (int s = 0; s < 4; ++s)
              if (qt * 16 + 4 * lg + s < nvalid) pb[(qt * 16 + s) * kDV] = num[qt][s];
        } else {
        // o = num * (1/den); lane (col, g) holds queries 4g+s of each query tile
        float* ob = Og + ((size_t)bh * N + c0 + 4 * lg) * kDV + gcol0 + ct * 16 + li;
        if (nvalid == C::CH) {
#pragma unroll
          for (int qt = 0; qt < C::QT; ++qt) {
            const f32x4 rd = *reinterpret_cast<const f32x4*>(sDenQ + qt * 16 + 4 * lg);
#pragma unroll
            for (int s = 0; s < 4; ++s) store_nt(&ob[(qt * 16 + s) * kDV], num[qt][s] * rd[s]);
          }
        } else {
#pragma unroll
          for (int qt = 0; qt < C::QT; ++qt) {
            const f32x4 rd = *reinterpret_cast<const f32x4*>(sDenQ + qt * 16 + 4 * lg);
#pragma unroll
            for (int s = 0; s < 4; ++s)
              if (qt * 16 + 4 * lg + s < nvalid) store_nt(&ob[(qt * 16 + s) * kDV], num[qt][s] * rd[s]);
          }
        }
        }
      }
      __syncthreads();
    }
    db ^= 1;
  }

  if constexpr (!OUT) {
    // span total of the row group's rows -> workspace
#pragma unroll
    for (int j = 0; j < C::MKB; ++j) {
      if (j / C::J >= nsl) continue;
      int kb, col;
      if constexpr (C::TR) {  // (slab j/J, K-block w/WPK, column tile (w%WPK)*J + j%J)
        kb = (slab0 + j / C::J) * C::NRP * C::J + w / C::WPK;
        col = ((w % C::WPK) * C::J + j % C::J) * 16 + li;
      } else {
        kb = kb_of(j);
        col = gcol0 + ct * 16 + li;
      }
#pragma unroll
      for (int t = 0; t < C::TPK; ++t) {
#pragma unroll
        for (int s = 0; s < 4; ++s) wsS[(size_t)acc_row(kb, t, s) * kDV + col] = st[j][t][s];
      }
    }
    if (grp == 0)
      for (int r = tid; r < nsl * C::SR; r += C::NTHR) wsS[(size_t)C::WP * kDV + slab0 * C::SR + r] = sDen[db * C::RWG + r];
  }
}


// ---------------------------------------------------------------------------
// Warp-specialised sweep for small feature sets with bf16 inputs.
//
// 8 waves: waves 0-3 are producers, waves 4-7 consumers (one per 16-column
// value tile), so every SIMD holds one of each and the producers' VALU work
// (staging, the intra-chunk block P, feature generation) overlaps the
// consumers' MFMA work (readout, P.[V,1], update).  Producers prepare chunk
// c+1 in one half of a double buffer while consumers work on chunk c in the
// other; one workgroup barrier per chunk swaps them (an LDS-only barrier: no
// wave reads global memory another wave wrote, so output stores and input
// loads stay in flight across it).  The normaliser state of K-block j lives in
// the accumulators of consumer j % 4, which publishes it each chunk as bf16
// readout fragments (double-buffered; row 0, the token count, in fp32).
// Outputs are normalised one chunk late, once all four consumers have
// published 1/den.
//
// Every LDS tile is written token-major, 16 bytes per lane and store (V as
// loaded, mu and phi as generated; a shifted mu row goes out as two 8-byte
// halves in one instruction); operands whose contraction index is the token
// (V, mu^T) are read back with transposing LDS reads.  The readout and P.V
// produce O^T tiles (value columns x queries), so each lane ends up with four
// consecutive columns of one query and stores them as one 16-byte write.
// ---------------------------------------------------------------------------

template <int DK_, int NT_, int MODE_>
struct PCfg {
  using TIn = uint16_t;
  using Elem = uint16_t;
  static constexpr bool BF = true;
  static constexpr bool OUT = (MODE_ != MODE_TOTALS);
  static constexpr bool UNN = (MODE_ == MODE_OUTPUT_UNN);
  static constexpr int DK = DK_, NT = NT_;
  static constexpr int NTHR = 512;
  static constexpr int NW = 8;
  static constexpr int W = rows_for(DK, NT);
  static constexpr int KB = 32, TPK = 2;
  static constexpr int NKB = (W + KB - 1) / KB;
  static constexpr int WP = NKB * KB;
  static constexpr int SR = WP;
  static constexpr int NSLAB = 1;
  static constexpr int PADE = 8;  // 16-byte row padding (bank spread)
  static constexpr int PHS = WP + PADE;   // phi[token][row]
  // mu[token][row]: when WP = 32 (mod 64) the rows are unpadded and the
  // 16-byte chunk c of token t is stored at chunk c ^ ((t >> 2) & 3), which
  // spreads each 16-lane group of a transposing read (4 tokens x 4 chunks)
  // over all 16-byte bank groups; other widths keep a 16-byte row padding
  static constexpr bool MUSWZ = WP % 64 == 32;
  static constexpr int MUS = MUSWZ ? WP : WP + PADE;
  // with the swizzle, each block of 8 tokens also starts 8 bytes (MUSH = 4
  // elements) after the end of the previous one: token t's row begins at
  // t * MUS + MUSH * (t >> 3). The 32 lanes of a transposing read (tokens
  // 0-3 and 8-11 of a 16-token group, the same chunks and the same half)
  // then fall on opposite halves of each 16-byte bank group. Rows are stored
  // as 8-byte-aligned pairs; each plane ends with 32 elements of slack.
  static constexpr int MUSH = MUSWZ ? 4 : 0;
  static constexpr int VS = kDV + PADE;   // V[token][col]
  static constexpr int PS = kCH + PADE;   // P[query][key]
  static constexpr int NMU = OUT ? 1 : 2;
  static constexpr int MUPL = kCH * MUS + (MUSWZ ? 32 : 0);
  static_assert(!MUSWZ || MUSH * (kCH / 8 - 1) <= 32 - 4, "row shift slack");
  static constexpr int PPL = kCH * PS;
  static constexpr int al(int b) { return (b + 15) / 16 * 16; }
  // one buffer of each kind; two of each are allocated
  static constexpr int B_V = al(kCH * VS * 2);
  static constexpr int B_PHI = OUT ? al(kCH * PHS * 2) : 0;
  static constexpr int B_MU = al(NMU * MUPL * 2);
  static constexpr int B_P = OUT ? al(2 * PPL * 2) : 0;
  static constexpr int O_V = 0;
  static constexpr int O_PHI = O_V + 2 * B_V;
  static constexpr int O_MU = O_PHI + 2 * B_PHI;
  static constexpr int O_P = O_MU + 2 * B_MU;
  static constexpr int O_DEN = O_P + 2 * B_P;             // bf16 normaliser rows [2][hi, lo][WP]
  static constexpr int O_DEN0 = O_DEN + al(4 * WP * 2);    // fp32 normaliser of row 0 [2]
  static constexpr int O_RDEN = O_DEN0 + 16;               // 1/den per query [2][64]
  // output pass, per query: phi . Zh over rows >= 1 (the normaliser readout
  // from the hi plane), the factor of the state shift's add-back [2][64]
  static constexpr int O_G = O_RDEN + (OUT ? al(2 * kCH * 4) : 0);
  static constexpr int LDS = O_G + (OUT ? al(2 * kCH * 4) : 0);
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static constexpr int QV = DK / 8;  // 16-byte pieces of a q or k row
};

template <class C>
__global__ __launch_bounds__(C::NTHR) void pipe_kernel(const uint16_t* __restrict__ Qg,
                                                       const uint16_t* __restrict__ Kg,
                                                       const uint16_t* __restrict__ Vg, int N, int span,
                                                       int nspan, float* __restrict__ ws,
                                                       float* __restrict__ Og, float* __restrict__ Dg) {
  using Elem = uint16_t;
  constexpr bool OUT = C::OUT;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS];
  auto sV = [&](int b) { return reinterpret_cast<Elem*>(lds + C::O_V + b * C::B_V); };
  auto sPhi = [&](int b) { return reinterpret_cast<Elem*>(lds + C::O_PHI + b * C::B_PHI); };
  auto sMu = [&](int b) { return reinterpret_cast<Elem*>(lds + C::O_MU + b * C::B_MU); };
  auto sP = [&](int b) { return reinterpret_cast<Elem*>(lds + C::O_P + b * C::B_P); };
  uint16_t* sDenB = reinterpret_cast<uint16_t*>(lds + C::O_DEN);  // [2][hi, lo][WP] bf16 normaliser rows
  float* sDen0 = reinterpret_cast<float*>(lds + C::O_DEN0);         // [2] row-0 normaliser (token count)
  float* sRden = reinterpret_cast<float*>(lds + C::O_RDEN);         // [2][query%16][query/16]
  float* sG = reinterpret_cast<float*>(lds + C::O_G);               // [2][query%16][query/16]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in an SGPR: branches on it are scalar
  const bool producer = w < 4;
  const int pw = w & 3;       // producer index / consumer column tile
  const int li = lane & 15, lg = lane >> 4;
  const int s_idx = blockIdx.x % nspan;
  const int bh = blockIdx.x / nspan;
  const int t_begin = s_idx * span;
  const int t_end = min(N, t_begin + span);
  const int nch = (t_end - t_begin + kCH - 1) / kCH;
  const uint16_t* Qh = Qg + (size_t)bh * N * C::DK;
  const uint16_t* Kh = Kg + (size_t)bh * N * C::DK;
  const uint16_t* Vh = Vg + (size_t)bh * N * kDV;
  float* wsS = ws + ((size_t)bh * nspan + s_idx) * (size_t)C::WP * (kDV + 1);

  // ---------------- producer state ----------------
  constexpr int NXT = 6 * 2;  // X^T tiles (key block, query tile, tau) on or below the diagonal
  constexpr int XPP = NXT / 4;  // per producer wave
  constexpr int XD = C::DK == 16 ? 1 : C::DK / 32;
  struct Stage {  // one chunk's inputs in flight, held in registers
    u32x4 pq[C::QV], pk[C::QV], pv[2];
    u32x4 xa[XPP][XD], xb[XPP][XD];
  };
  // Loads are unconditional so that the compiler can count them in flight:
  // token indices are clamped into the span (and the chunk index by the
  // caller); rows past the span end are masked where they are consumed.
  auto p_issue = [&](int ci, Stage& sg) {  // global -> registers for chunk ci (ci < nch)
    auto& pq = sg.pq; auto& pk = sg.pk; auto& pv = sg.pv; auto& xa = sg.xa; auto& xb = sg.xb;
    const int c0 = t_begin + ci * kCH;
    const int tl = t_end - 1;
    const size_t row = (size_t)min(c0 + lane, tl);
    // issued in the order p_build consumes them (loads complete in order):
    // V, the operands of P, then the key and query rows
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // V segments: (column group, token), lanes walk tokens
      const int seg = pw * 64 + lane + i * 256;
      const int tok = seg & 63, grp8 = seg >> 6;
      pv[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)min(c0 + tok, tl) * kDV + grp8 * 8);
    }
    if constexpr (OUT) {
#pragma unroll
      for (int t = 0; t < XPP; ++t) {
        const int ti = pw + 4 * t, pair = ti >> 1, tau = ti & 1;
        const int kb = pair < 4 ? 0 : 1, qt = pair < 4 ? pair : pair - 2;
        const size_t key = (size_t)min(c0 + kb * 32 + rho(tau, li), tl);
        const size_t qry = (size_t)min(c0 + qt * 16 + li, tl);
#pragma unroll
        for (int h = 0; h < XD; ++h) {
          if constexpr (C::DK == 16) {
            const uint2 a = *reinterpret_cast<const uint2*>(Kh + key * 16 + 4 * lg);
            const uint2 bq = *reinterpret_cast<const uint2*>(Qh + qry * 16 + 4 * lg);
            xa[t][h] = u32x4{a.x, a.y, 0u, 0u};
            xb[t][h] = u32x4{bq.x, bq.y, 0u, 0u};
          } else {
            xa[t][h] = *reinterpret_cast<const u32x4*>(Kh + key * C::DK + 32 * h + 8 * lg);
            xb[t][h] = *reinterpret_cast<const u32x4*>(Qh + qry * C::DK + 32 * h + 8 * lg);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::QV; ++i) {
      pk[i] = *reinterpret_cast<const u32x4*>(Kh + row * C::DK + 8 * i);
      if constexpr (OUT) pq[i] = *reinterpret_cast<const u32x4*>(Qh + row * C::DK + 8 * i);
    }
  };
  auto p_build = [&](int ci, const Stage& sg) {  // registers -> LDS buffer (ci & 1): V, P, phi, mu
    const auto& pq = sg.pq; const auto& pk = sg.pk; const auto& pv = sg.pv; const auto& xa = sg.xa;
    const auto& xb = sg.xb;
    const int b = ci & 1;
    const int c0 = t_begin + ci * kCH;
    const int nvalid = min(kCH, t_end - c0);
    Elem* V = sV(b);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = pw * 64 + lane + i * 256;
      const int tok = seg & 63, col0 = (seg >> 6) * 8;
      *reinterpret_cast<u32x4*>(V + tok * C::VS + col0) = pv[i];
    }
    if constexpr (OUT) {
      Elem* P = sP(b);
#pragma unroll
      for (int t = 0; t < XPP; ++t) {
        const int ti = pw + 4 * t, pair = ti >> 1, tau = ti & 1;
        const int kb = pair < 4 ? 0 : 1, qt = pair < 4 ? pair : pair - 2;
        f32x4 x = zero4();
        if constexpr (C::DK == 16) {
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          const uint2 a = {xa[t][0].x, xa[t][0].y}, bq = {xb[t][0].x, xb[t][0].y};
          x = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, bq),
                                                        x, 0, 0, 0);
        } else {
#pragma unroll
          for (int h = 0; h < XD; ++h) x = mfma_bf16(xa[t][h], xb[t][h], x);
        }
        const int query = qt * 16 + li;
        float pr[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int key = kb * 32 + 8 * lg + 4 * tau + s;
          pr[s] = (key <= query && key < nvalid) ? taylor_poly<C::NT>(x[s]) : 0.f;
        }
        const int kbase = kb * 32 + 8 * lg + 4 * tau;
        // the first chunk of a span also gets the lo plane of P (its queries
        // may have few keys in all); later chunks have at least one chunk of
        // keys in the state part of their normaliser and take P as bf16
        if (ci == 0) {
          uint2 hi, lo;
          split_bf16x2(pr[0], pr[1], hi.x, lo.x);
          split_bf16x2(pr[2], pr[3], hi.y, lo.y);
          *reinterpret_cast<uint2*>(&P[query * C::PS + kbase]) = hi;
          *reinterpret_cast<uint2*>(&P[C::PPL + query * C::PS + kbase]) = lo;
        } else {
          *reinterpret_cast<uint2*>(&P[query * C::PS + kbase]) = uint2{pack_bf16x2(pr[0], pr[1]),
                                                                        pack_bf16x2(pr[2], pr[3])};
        }
      }
    }
    // features: lane = token, this producer takes 8-row groups g == pw (mod 4).
    // Keys past the span end are zeroed (their mu rows of order >= 1 vanish;
    // the order-0 row is masked in gen_groups); queries past the end are not
    // stored, and V of those tokens meets only zero weights.
    float xk[C::DK], xq[C::DK];
    const uint32_t kmask = lane < nvalid ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < C::QV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xk[8 * i + 2 * e] = __uint_as_float((pk[i][e] & kmask) << 16);
        xk[8 * i + 2 * e + 1] = __uint_as_float(pk[i][e] & kmask & 0xFFFF0000u);
        if constexpr (OUT) {
          xq[8 * i + 2 * e] = __uint_as_float(pq[i][e] << 16);
          xq[8 * i + 2 * e + 1] = __uint_as_float(pq[i][e] & 0xFFFF0000u);
        }
      }
    gen_groups<C>(pw, 4, lane, nvalid, xq, xk, OUT ? sPhi(b) : nullptr, sMu(b));
  };

  // ---------------- consumer state ----------------
  f32x4 st[C::NKB][2];
#pragma unroll
  for (int j = 0; j < C::NKB; ++j) st[j][0] = st[j][1] = zero4();
  f32x4 nprev[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) nprev[q] = zero4();
  f32x4 mprev = zero4();  // column means of the previous chunk's readout shift
  const int ct = pw;
  // all ones: every column of a product with it holds the row sums
  const u32x4 ones_bf = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

  // Producer and consumer waves run separate loops with the same number of
  // workgroup barriers (one per chunk, plus one after the prologue), so their
  // loop-carried registers never overlap.
  // Both roles run nch2 = nch rounded up to even loop steps with one barrier
  // each (plus one after the prologue); consumers skip the work of a padding
  // step, producers build an all-masked chunk in it.
  const int nch2 = (nch + 1) & ~1;
  if (producer) {
    // two register stages, loop unrolled by two so every stage index is
    // static: chunk c is loaded two steps before it is built
    auto cl = [&](int c) { return c < nch - 1 ? c : nch - 1; };
    Stage sg[2];
    p_issue(cl(0), sg[0]);
    p_issue(cl(1), sg[1]);
    p_build(0, sg[0]);
    p_issue(cl(2), sg[0]);
    lds_barrier();
    for (int ci = 0; ci < nch2; ci += 2) {
      p_build(ci + 1, sg[1]);
      p_issue(cl(ci + 3), sg[1]);
      lds_barrier();
      p_build(ci + 2, sg[0]);
      p_issue(cl(ci + 4), sg[0]);
      lds_barrier();
    }
  } else {
    constexpr int NJD = (C::NKB + 3) / 4;   // normaliser K-blocks of this consumer: j = 4*jd + ct
    // normaliser rows j*32 + 8*lg + 4*tau + s of the owned K-blocks (lanes li == 0 carry them)
    f32x4 dstate[NJD][2];
#pragma unroll
    for (int jd = 0; jd < NJD; ++jd) dstate[jd][0] = dstate[jd][1] = zero4();
    // hi + lo bf16 readout fragments and the fp32 row 0.  The ones operand
    // fills every column, so every lane of group lg holds the group's rows
    // 8lg .. 8lg+7 (dstate[jd][row / 4 % 2][row % 4]); lane li < 8 splits
    // row 8lg + li, one value per lane instead of eight in lane li == 0.
    auto publish_den = [&](int buf) {
      // a select tree on the bits of li (a per-lane index into the
      // registers would go through scratch memory)
      const bool b0 = (li & 1) != 0, b1 = (li & 2) != 0, b2 = (li & 4) != 0;
#pragma unroll
      for (int jd = 0; jd < NJD; ++jd) {
        const int j = 4 * jd + ct;
        if (j < C::NKB) {
          const f32x4 d0 = dstate[jd][0], d1 = dstate[jd][1];
          const float p0 = b0 ? d0.y : d0.x, p1 = b0 ? d0.w : d0.z;
          const float p2 = b0 ? d1.y : d1.x, p3 = b0 ? d1.w : d1.z;
          const float q0 = b1 ? p1 : p0, q1 = b1 ? p3 : p2;
          const float v = b2 ? q1 : q0;
          uint16_t h, l;
          split_bf16(v, h, l);
          if (li < 8) {
            sDenB[2 * buf * C::WP + j * 32 + 8 * lg + li] = h;
            sDenB[(2 * buf + 1) * C::WP + j * 32 + 8 * lg + li] = l;
          }
        }
      }
      if (ct == 0 && lg == 0 && li == 0) sDen0[buf] = dstate[0][0].x;
    };
    if constexpr (OUT) {
#pragma unroll
      for (int j = 0; j < C::NKB; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 v;
#pragma unroll
          for (int s = 0; s < 4; ++s) v[s] = wsS[(size_t)(j * 32 + 8 * lg + 4 * t + s) * kDV + ct * 16 + li];
          st[j][t] = v;
        }
#pragma unroll
      for (int jd = 0; jd < NJD; ++jd) {
        const int j = 4 * jd + ct;
        if (j < C::NKB) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s) dstate[jd][t][s] = wsS[(size_t)C::WP * kDV + j * 32 + 8 * lg + 4 * t + s];
        }
      }
      publish_den(0);
    }
    lds_barrier();
    // transposing-read addresses of this lane: token row 8*lg + li/4 (+4 for
    // the second read) of a 32-token block; V columns ct*16 + 4*(li%4); mu
    // columns 8*(li%4) + 4*tau of a K-block (rows rho(tau, i) of the A tile)
    const int trow = 8 * lg + (li >> 2);
    auto load_v = [&](const unsigned char* V, int tb, int col_tile) {
      const unsigned char* p = V + ((tb * 32 + trow) * C::VS + col_tile * 16 + 4 * (li & 3)) * 2;
      const uint2 a = lds_tr16(p), c = lds_tr16(p + 4 * C::VS * 2);
      return u32x4{a.x, a.y, c.x, c.y};
    };
    // mu chunk swizzle (PCfg::MUSWZ): token 8*lg + li/4 (+4) of a 32-token
    // block has (t >> 2) & 3 = 2*(lg & 1) (+1)
    // (4j + c) ^ z = 4j + (c ^ z) for z < 4: the K-block part of the address
    // stays a compile-time offset
    const int cz0 = (li & 3) ^ (C::MUSWZ ? ((2 * lg) & 3) : 0);
    const int cz1 = (li & 3) ^ (C::MUSWZ ? ((2 * lg + 1) & 3) : 0);
    auto load_mu = [&](const unsigned char* Mu, int pl, int j, int tau, int tb) {
      // token tb * 32 + trow (+4) lies in 8-token block 4 * tb + lg
      const unsigned char* r0 =
          Mu + (pl * C::MUPL + (tb * 32 + trow) * C::MUS + C::MUSH * (4 * tb + lg) + 32 * j + 4 * tau) * 2;
      const uint2 a = lds_tr16(r0 + cz0 * 16);
      const uint2 c = lds_tr16(r0 + 4 * C::MUS * 2 + cz1 * 16);
      return u32x4{a.x, a.y, c.x, c.y};
    };
    constexpr int NPL = C::OUT ? 1 : 2;     // mu planes: hi only in the output pass, hi + lo in the totals pass
    // one chunk step; the LDS buffer index is a compile-time constant (the
    // loop below is unrolled by two), so LDS addresses are immediates
    auto chunk_step = [&](const int ci, auto bc) {
      constexpr int b = decltype(bc)::value;
      if (ci >= nch) {  // padding step
        lds_barrier();
        return;
      }
      const int c0 = t_begin + ci * kCH;
      const unsigned char* V = (const unsigned char*)sV(b);
      const unsigned char* Mu = (const unsigned char*)sMu(b);
      // V^T fragments of this wave's 16 columns for both 32-token blocks:
      // the A operand of P.V (output pass) and the B operand of the update
      u32x4 bvk[2];
      if constexpr (OUT) {
        bvk[0] = load_v(V, 0, ct);
        bvk[1] = load_v(V, 1, ct);
      }
      // update of K-block j from mu fragments mf[tau][tb][pl]: S += mu^T V, and
      // the normaliser (mu^T 1) of the blocks this wave owns from the same fragments
      auto update_block = [&](int j, const u32x4 (*mf)[2][NPL]) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int pl = 0; pl < NPL; ++pl) st[j][tau] = mfma_bf16(mf[tau][tb][pl], bvk[tb], st[j][tau]);
        if (j % 4 == ct) {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
              for (int pl = 0; pl < NPL; ++pl)
                dstate[j / 4][tau] = mfma_bf16(mf[tau][tb][pl], ones_bf, dstate[j / 4][tau]);
        }
      };
      auto fetch_mu = [&](int j, u32x4 (*dst)[2][NPL]) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int pl = 0; pl < NPL; ++pl) dst[tau][tb][pl] = load_mu(Mu, pl, j, tau, tb);
      };
      if constexpr (OUT) {
        // previous chunk: normalise (adding back a (phi . Z_hi), below) and
        // store, 16 bytes per lane and query tile; done first so that its
        // registers are free during the K-block loop
        if (ci > 0) {
          const f32x4 rd = *reinterpret_cast<const f32x4*>(sRden + (b ^ 1) * kCH + li * 4);
          const f32x4 gq = *reinterpret_cast<const f32x4*>(sG + (b ^ 1) * kCH + li * 4);
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) {
            float* ob = Og + ((size_t)bh * N + c0 - kCH + qt * 16 + li) * kDV + ct * 16 + 4 * lg;
            store_nt(ob, (nprev[qt] + mprev * gq[qt]) * rd[qt]);
          }
        }
        const unsigned char* Phi = (const unsigned char*)sPhi(b);
        const unsigned char* P = (const unsigned char*)sP(b);
        // num[qt] is the O^T tile (columns ct*16 + 4*lg + s, query qt*16 + li)
        f32x4 num[4], den = zero4(), denh = zero4();
#pragma unroll
        for (int q = 0; q < 4; ++q) num[q] = zero4();
        // normaliser fragment of K-block j: the same normaliser rows in every
        // column of the B tile, so every column of the product holds the
        // readout (lanes li == 0 use it); fetched one K-block ahead
        auto load_bdn = [&](int j, int pl) {
          return *reinterpret_cast<const u32x4*>(sDenB + (2 * b + pl) * C::WP + j * 32 + 8 * lg);
        };
        u32x4 bdn[2];
        bdn[0] = load_bdn(0, 0);
        const float den0 = sDen0[b];
        // m = 0 row (fp32): S[0][col] for this lane's four columns
        f32x4 m0;
#pragma unroll
        for (int s = 0; s < 4; ++s) m0[s] = __shfl(st[0][0].x, 4 * lg + s);
        // Readout of rows >= 1 from a shifted state.  With a_c the running
        // mean of value column c (S[0][c] over the token count Z[0], rounded
        // to bf16) and Zh the hi bf16 plane of the normaliser rows,
        //   sum_r phi_r S[r][c] = sum_r phi_r (S[r][c] - a_c Zh[r]) + a_c (phi . Zh),
        // an identity for any a_c.  The shifted state goes to the MFMA rounded
        // to bf16 (a_c Zh[r] is exact in fp32, so one bf16 dot product per
        // row forms the difference); phi . Zh over rows >= 1 is the hi half of
        // the normaliser readout (the same bf16 phi), and a_c (phi . Zh) is
        // added in fp32 when the chunk is normalised.  Rounding the state then
        // moves an output by about 2^-9 |v - a| instead of 2^-9 |v|: values
        // offset from zero keep the accuracy of zero-mean ones.  A non-finite
        // mean (non-finite inputs) falls back to no shift.
        const float rz0 = den0 > 0.f ? rcp_fast(den0) : 0.f;
        auto col_mean = [&](float s0) {  // bf16 bits of a_c (0 when not finite in bf16)
          const uint32_t bits = pack_bf16x2(s0 * rz0, 0.f) & 0xFFFFu;
          return (bits & 0x7F80u) != 0x7F80u ? bits : 0u;
        };
        const uint32_t abits = col_mean(__shfl(st[0][0].x, li));  // column ct*16 + li
        const uint32_t nab = abits ^ 0x8000u;  // {-a_c, 0} as a bf16 pair; nab << 16 is {0, -a_c}
        // readout of K-block j, then its update (the readout has taken st[j]
        // into bs first); phi and mu fragments one K-block ahead
        u32x4 af[2][4];
        u32x4 mf[2][2][2][NPL];
        auto load_phi = [&](int j, u32x4* dst) {
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) dst[qt] = lds_u32x4(Phi, ((qt * 16 + li) * C::PHS + j * 32 + 8 * lg) * 2);
        };
        load_phi(0, af[0]);
        fetch_mu(0, mf[0]);
#pragma unroll
        for (int j = 0; j < C::NKB; ++j) {
          // lo plane of the normaliser rows, read before the next K-block's
          // fragments (LDS reads complete in order: read after them, the
          // normaliser MFMA would wait for all of them) and used after the
          // value readout's MFMAs
          const u32x4 bdl = load_bdn(j, 1);
          // keep the scheduler from moving that read behind the prefetch
          __builtin_amdgcn_sched_barrier(0);
          if (j + 1 < C::NKB) {
            load_phi(j + 1, af[(j + 1) & 1]);
            fetch_mu(j + 1, mf[(j + 1) & 1]);
            bdn[(j + 1) & 1] = load_bdn(j + 1, 0);
          }
          // S[rows 8lg..8lg+7 of K-block j][column ct*16 + li] - a Zh[rows]
          // as the A operand (S^T), rounded to bf16; bdn holds Zh of the same
          // rows as bf16 pairs (row 8lg + 2e in the low half of dword e)
          float sh[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = bdn[j & 1][e];  // through a scalar (see prod8)
            const f32x4 sv = st[j][e >> 1];
            sh[2 * e] = dot2_bf16(nab, w, sv[(2 * e) & 3]);
            sh[2 * e + 1] = dot2_bf16(nab << 16, w, sv[(2 * e + 1) & 3]);
          }
          const u32x4 bs = {pack_bf16x2(sh[0], sh[1]), pack_bf16x2(sh[2], sh[3]), pack_bf16x2(sh[4], sh[5]),
                            pack_bf16x2(sh[6], sh[7])};
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) num[qt] = mfma_bf16(bs, af[j & 1][qt], num[qt]);
          // normaliser readout of this wave's query tile (hi plane into denh,
          // lo plane into den): ct is wave-uniform, so this is a scalar branch
          // to one of four MFMA pairs (no operand select)
          switch (ct) {
            case 0: denh = mfma_bf16(af[j & 1][0], bdn[j & 1], denh); den = mfma_bf16(af[j & 1][0], bdl, den); break;
            case 1: denh = mfma_bf16(af[j & 1][1], bdn[j & 1], denh); den = mfma_bf16(af[j & 1][1], bdl, den); break;
            case 2: denh = mfma_bf16(af[j & 1][2], bdn[j & 1], denh); den = mfma_bf16(af[j & 1][2], bdl, den); break;
            default: denh = mfma_bf16(af[j & 1][3], bdn[j & 1], denh); den = mfma_bf16(af[j & 1][3], bdl, den); break;
          }
          update_block(j, mf[j & 1]);
        }
        // phi . Zh over rows >= 1 for queries ct*16 + 4*lg + s (every lane
        // holds it): the add-back factor, read when the chunk is normalised
        if (li == 0) {
#pragma unroll
          for (int s = 0; s < 4; ++s) sG[b * kCH + (4 * lg + s) * 4 + ct] = denh[s];
        }
        // intra-chunk block: O^T += V^T P^T, normaliser P.1 for query tile ct;
        // the lo plane of P only in the first chunk of the span (see p_build)
        auto intra = [&](auto loc) {
          constexpr bool LO = decltype(loc)::value;
          u32x4 ph[4][2], pl[4][2];  // (query tile, key block) on or below the diagonal
#pragma unroll
          for (int qt = 0; qt < 4; ++qt)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              if (kb * 32 <= qt * 16 + 15) {
                ph[qt][kb] = lds_u32x4(P, ((qt * 16 + li) * C::PS + kb * 32 + 8 * lg) * 2);
                if constexpr (LO) pl[qt][kb] = lds_u32x4(P, (C::PPL + (qt * 16 + li) * C::PS + kb * 32 + 8 * lg) * 2);
              }
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              if (kb * 32 <= qt * 16 + 15) {
                num[qt] = mfma_bf16(bvk[kb], ph[qt][kb], num[qt]);
                if constexpr (LO) num[qt] = mfma_bf16(bvk[kb], pl[qt][kb], num[qt]);
                if (qt == ct) {
                  // every column of the product holds P.1 (lanes li == 0 read den)
                  den = mfma_bf16(ph[qt][kb], ones_bf, den);
                  if constexpr (LO) den = mfma_bf16(pl[qt][kb], ones_bf, den);
                }
              }
            }
            num[qt] += m0;
          }
        };
        if (ci == 0)
          intra(std::true_type{});
        else
          intra(std::false_type{});
        if (li == 0) {
          // unnormalised mode: outputs keep their numerators and the
          // normalisers go to Dg
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float dq = denh[s] + den[s] + den0;
            if constexpr (C::UNN) {
              sRden[b * kCH + (4 * lg + s) * 4 + ct] = 1.0f;
              const int t = c0 + ct * 16 + 4 * lg + s;
              if (t < t_end) Dg[(size_t)bh * N + t] = dq;
            } else {
              sRden[b * kCH + (4 * lg + s) * 4 + ct] = rcp_fast(dq);
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) nprev[q] = num[q];
        // a_c of this lane's four output columns, as the shift took them
#pragma unroll
        for (int s = 0; s < 4; ++s) mprev[s] = __uint_as_float(col_mean(m0[s]) << 16);
      }
      if constexpr (!OUT) {
        // totals pass (hi + lo planes), state split by rows: consumer ct owns
        // K-blocks 4q + ct for all four column tiles (st[4q + c'], so each mu
        // fragment is read by one wave only); the last NKB % 4 K-blocks are
        // split by column tile (st[4*FQ + jr], column tile ct)
        constexpr int FQ = C::NKB / 4, R = C::NKB % 4;
        u32x4 bva[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            bva[c][tb] = load_v(V, tb, c);
        u32x4 mf[FQ + R][2][2][NPL];
#pragma unroll
        for (int q = 0; q < FQ; ++q) fetch_mu(4 * q + ct, mf[q]);
#pragma unroll
        for (int jr = 0; jr < R; ++jr) fetch_mu(4 * FQ + jr, mf[FQ + jr]);
#pragma unroll
        for (int q = 0; q < FQ; ++q) {
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl) st[4 * q + c][tau] = mfma_bf16(mf[q][tau][tb][pl], bva[c][tb], st[4 * q + c][tau]);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
              for (int pl = 0; pl < NPL; ++pl) dstate[q][tau] = mfma_bf16(mf[q][tau][tb][pl], ones_bf, dstate[q][tau]);
        }
#pragma unroll
        for (int jr = 0; jr < R; ++jr) {
          const int j = 4 * FQ + jr;
          const u32x4 bv0 = bva[ct][0], bv1 = bva[ct][1];  // this wave's column tile (ct is wave-uniform)
#pragma unroll
          for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int pl = 0; pl < NPL; ++pl) {
              st[j][tau] = mfma_bf16(mf[FQ + jr][tau][0][pl], bv0, st[j][tau]);
              st[j][tau] = mfma_bf16(mf[FQ + jr][tau][1][pl], bv1, st[j][tau]);
            }
          if (j % 4 == ct) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl)
                  dstate[j / 4][tau] = mfma_bf16(mf[FQ + jr][tau][tb][pl], ones_bf, dstate[j / 4][tau]);
          }
        }
      }
      if constexpr (OUT) publish_den(b ^ 1);
      lds_barrier();
    };
    for (int ci = 0; ci < nch2; ci += 2) {
      chunk_step(ci, std::integral_constant<int, 0>{});
      chunk_step(ci + 1, std::integral_constant<int, 1>{});
    }
    if constexpr (OUT) {
      // last chunk: normalise and store
      const int lc0 = t_begin + (nch - 1) * kCH;
      const int nvalid = t_end - lc0;
      const f32x4 rd = *reinterpret_cast<const f32x4*>(sRden + ((nch - 1) & 1) * kCH + li * 4);
      const f32x4 gq = *reinterpret_cast<const f32x4*>(sG + ((nch - 1) & 1) * kCH + li * 4);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        if (qt * 16 + li < nvalid) {
          float* ob = Og + ((size_t)bh * N + lc0 + qt * 16 + li) * kDV + ct * 16 + 4 * lg;
          store_nt(ob, (nprev[qt] + mprev * gq[qt]) * rd[qt]);
        }
      }
    } else {
      // span total: row-split K-blocks (all column tiles), then the column-split ones
      constexpr int FQ = C::NKB / 4;
#pragma unroll
      for (int q = 0; q < FQ; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s)
              wsS[(size_t)((4 * q + ct) * 32 + 8 * lg + 4 * t + s) * kDV + c * 16 + li] = st[4 * q + c][t][s];
#pragma unroll
      for (int j = 4 * FQ; j < C::NKB; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int s = 0; s < 4; ++s) wsS[(size_t)(j * 32 + 8 * lg + 4 * t + s) * kDV + ct * 16 + li] = st[j][t][s];
      if (li == 0) {
#pragma unroll
        for (int jd = 0; jd < NJD; ++jd) {
          const int j = 4 * jd + ct;
          if (j < C::NKB) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int s = 0; s < 4; ++s) wsS[(size_t)C::WP * kDV + j * 32 + 8 * lg + 4 * t + s] = dstate[jd][t][s];
          }
        }
      }
    }
  }
}

// Exclusive scan of span totals over spans (in place) and the final states.
// The workspace rows are internal rows: feature order, or the octet order
// when octdk is 32 or 64 (mapped back with abi_row; padding rows dropped).
// The scan starts from the carried-in states `init` (plane layout; null for
// zero states).  Each state element is read from `init` and written to
// `states` by the same thread, so the two may be the same buffer.
__global__ void scan_kernel(float* ws, int nspan, int WP, int W, int BH, int octdk, const float* init,
                            float* states) {
  const size_t per = (size_t)WP * (kDV + 1);
  const size_t total = (size_t)BH * per;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = e / per;
    const size_t off = e - bh * per;
    const bool val = off < (size_t)WP * kDV;
    const int r = (int)(val ? off / kDV : off - (size_t)WP * kDV);
    const int ra = octdk == 64 ? abi_row<64>(r) : octdk == 32 ? abi_row<32>(r) : (r < W ? r : -1);
    // index of this element in the plane layout (padding rows: none)
    const size_t si = ra < 0 ? 0
                      : val ? (bh * W + ra) * kDV + (off - (size_t)r * kDV)
                            : (size_t)BH * W * kDV + bh * W + ra;
    float* p = ws + bh * nspan * per + off;
    float run = (init != nullptr && ra >= 0) ? init[si] : 0.f;
    int s = 0;
    for (; s + 8 <= nspan; s += 8) {  // eight independent loads in flight
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = p[(size_t)(s + u) * per];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        p[(size_t)(s + u) * per] = run;
        run += t[u];
      }
    }
    for (; s < nspan; ++s) {
      const float t = p[(size_t)s * per];
      p[(size_t)s * per] = run;
      run += t;
    }
    if (ra >= 0) states[si] = run;
  }
}

// Per-shape launch configuration: the smallest row split NRP (waves sharing a
// value-column tile) that keeps the state at <= 160 accumulator floats per
// lane; 4 waves for NRP = 1, else 8 waves with 8/NRP value tiles per group.
constexpr int pick_nrp(int nkb, int fpk, int cap = 160) {
  const int opts[4] = {1, 2, 4, 8};
  for (int i = 0; i < 4; ++i)
    if ((nkb + opts[i] - 1) / opts[i] * fpk <= cap) return opts[i];
  return 8;
}

// Row groups for large feature sets: the fewest groups of whole slabs that
// keep a wave's share of the state at <= 96 accumulator floats per lane,
// with the slabs spread evenly (every group gets at least one).
constexpr int pick_nrg(int nkb, int nrp, int kb, bool bf, int ch = 64, int cap = 96) {
  const int maxkb = (nkb + nrp - 1) / nrp;
  const int j = pick_j(maxkb, srmax(bf, ch) / (nrp * kb));
  const int ns = (maxkb + j - 1) / j;
  const int per = j * (bf ? 2 : 1) * 4;  // accumulator floats per lane per slab
  int rgs = cap / per;
  if (rgs < 1) rgs = 1;
  if (rgs > ns) rgs = ns;
  const int nrg = (ns + rgs - 1) / rgs;
  const int even = (ns + nrg - 1) / nrg;
  return (ns + even - 1) / even;
}

// Small feature sets (<= 256 rows): one workgroup holds the whole state of
// NVT column tiles.  Larger ones: 8 waves over all 64 columns (NVT = 4,
// NRP = 2) and the rows split over NRG row groups, so every feature row is
// generated once per chunk; the output pass then writes per-group partial
// numerators and normalisers that combine_kernel adds and divides.  A wave's
// share of a large state is capped at 96 accumulator floats per lane for
// bf16 (64 with four or more terms, whose slabs hold 32 floats) and 80 for
// fp32 (whose output pass holds more fragments), so that the output pass
// fits the register file without spilling.  Chunks of 128
// tokens hold twice the output tiles per wave, so their state share per
// lane is capped lower (128 / 64 accumulator floats).
template <typename TIn, int DK, int NT, int CH = 64>
struct Shape {
  static constexpr bool BF = std::is_same<TIn, uint16_t>::value;
  static constexpr int W = internal_rows(BF, DK, NT);
  static constexpr int KB = BF ? 32 : 16;
  static constexpr int NKB = (W + KB - 1) / KB;
  static constexpr bool LARGE = NKB * KB > 256;
  static constexpr int CAP_SMALL = CH > 64 ? 128 : 160;
  static constexpr int CAP_LARGE = CH > 64 ? 64 : (BF ? (NT >= 4 ? 64 : 96) : 80);
  static constexpr int NRP = LARGE ? 2 : pick_nrp(NKB, BF ? 8 : 4, CAP_SMALL);
  static constexpr int NVT = LARGE ? 4 : (NRP == 1 ? 4 : 8 / NRP);
  static constexpr int NRG = LARGE ? pick_nrg(NKB, NRP, KB, BF, CH, CAP_LARGE) : 1;
  using Tot = Cfg<TIn, DK, NT, NVT, NRP, NRG, MODE_TOTALS, CH>;
  using Out = Cfg<TIn, DK, NT, NVT, NRP, NRG, MODE_OUTPUT, CH>;
  static_assert(Tot::WP == Out::WP, "modes share the workspace layout");
  static constexpr bool FITS = Tot::FITS && Out::FITS;
  static_assert((NRG - 1) * Out::NSLAB < Out::NSLAB_ALL, "every row group holds a slab");
  static_assert(NRG == 1 || !Out::UNR, "row groups only with the run or octet generators");
};

// O = (sum over row groups of the partial numerators) / (sum of the partial
// normalisers), four columns per thread.
__global__ void combine_kernel(const float* __restrict__ part, int BH, int N, int nrg, float* __restrict__ O,
                               float* __restrict__ Dg) {
  const size_t total = (size_t)BH * N * (kDV / 4);
  const float* pden = part + (size_t)BH * nrg * N * kDV;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const size_t c4 = e % (kDV / 4);
    const size_t t = (e / (kDV / 4)) % N;
    const size_t bh = e / ((size_t)(kDV / 4) * N);
    f32x4 acc = zero4();
    float d = 0.f;
    for (int r = 0; r < nrg; ++r) {
      const size_t row = (bh * nrg + r) * N + t;
      acc += *reinterpret_cast<const f32x4*>(part + row * kDV + 4 * c4);
      d += pden[row];
    }
    if (Dg) {  // unnormalised: the numerator to O, the normaliser to Dg
      store_nt(O + (bh * N + t) * kDV + 4 * c4, acc);
      if (c4 == 0) Dg[bh * N + t] = d;
    } else {
      store_nt(O + (bh * N + t) * kDV + 4 * c4, acc * (1.0f / d));
    }
  }
}


// Exclusive scan over spans of the span totals in the workspace (in place),
// and the final states.
inline hipError_t launch_scan(float* ws, const PrefillPlan& p, int BH, int WP, int octdk, const float* states_in,
                              float* states, hipStream_t s) {
  const size_t total = (size_t)BH * WP * (kDV + 1);
  unsigned g = (unsigned)((total + 255) / 256);
  if (g > 16384) g = 16384;
  hipLaunchKernelGGL(scan_kernel, dim3(g), dim3(256), 0, s, ws, p.nspan, WP, p.W, BH, octdk, states_in, states);
  return hipGetLastError();
}

// bf16 inputs with at most 256 feature rows take the warp-specialised pipe
// kernel when the chunk is 64 tokens
template <int DK, int NT>
constexpr bool use_pipe() { return DK >= 16 && (rows_for(DK, NT) + 31) / 32 * 32 <= 256; }

// The sweep-kernel path for chunks of CH tokens: the plan's padded rows,
// column groups and row groups, and the launches (span totals, span scan,
// output pass, row-group combine).  bf16 needs CH >= 32 (token blocks of
// 32) and dk >= 16.
template <int CH>
hipError_t sweep_shape(int dk, int n, tt_dtype dt, int* wp, int* ngroups, int* nrg) {
  return with_dkn(dk, n, [&](auto DKc, auto Nc) -> hipError_t {
    constexpr int DK = decltype(DKc)::value, NT = decltype(Nc)::value;
    auto fill = [&](auto tag) -> hipError_t {
      using S = Shape<decltype(tag), DK, NT, CH>;
      if constexpr (!S::FITS) {
        return hipErrorInvalidValue;
      } else {
        *wp = S::Out::WP;
        *ngroups = kDV / S::Out::GC;
        *nrg = S::NRG;
        return hipSuccess;
      }
    };
    if constexpr (runtime_rows<DK, NT>()) {
      return hipErrorInvalidValue;  // the widest shapes take the streamed path only
    } else {
      if (dt == TT_BF16) {
        if constexpr (DK < 16 || CH < 32 || (CH == 64 && use_pipe<DK, NT>())) {
          return hipErrorInvalidValue;
        } else {
          return fill(uint16_t{});
        }
      }
      return fill(float{});
    }
  });
}

template <int CH>
hipError_t sweep_launch(const void* Q, const void* K, const void* V, tt_dtype dt, int BH, int N, int dk, int n,
                        const PrefillPlan& p, const float* states_in, float* O, float* den_out, float* states,
                        float* ws, hipStream_t s) {
  return with_dkn(dk, n, [&](auto DKc, auto Nc) -> hipError_t {
    constexpr int DK = decltype(DKc)::value, NT = decltype(Nc)::value;
    auto go = [&](auto tag) -> hipError_t {
      using TIn = decltype(tag);
      using S = Shape<TIn, DK, NT, CH>;
      if constexpr (!S::FITS) {
        return hipErrorInvalidValue;  // refused by the plan
      } else {
        const unsigned nblk = (unsigned)((size_t)BH * p.nspan * p.ngroups * S::NRG);
        float* part = ws + (size_t)BH * p.nspan * S::Out::WP * (kDV + 1);  // row-group partial outputs
        hipLaunchKernelGGL((sweep_kernel<typename S::Tot>), dim3(nblk), dim3(S::Tot::NTHR), 0, s, (const TIn*)Q,
                           (const TIn*)K, (const TIn*)V, N, p.span, p.nspan, ws, part, O, den_out);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_scan(ws, p, BH, (int)S::Out::WP, S::Out::OCT ? DK : 0, states_in, states, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((sweep_kernel<typename S::Out>), dim3(nblk), dim3(S::Out::NTHR), 0, s, (const TIn*)Q,
                           (const TIn*)K, (const TIn*)V, N, p.span, p.nspan, ws, part, O, den_out);
        e = hipGetLastError();
        if (e != hipSuccess || S::NRG == 1) return e;
        const size_t total = (size_t)BH * N * (kDV / 4);
        unsigned g = (unsigned)((total + 255) / 256);
        if (g > 16384) g = 16384;
        hipLaunchKernelGGL(combine_kernel, dim3(g), dim3(256), 0, s, (const float*)part, BH, N, S::NRG, O, den_out);
        return hipGetLastError();
      }
    };
    if constexpr (runtime_rows<DK, NT>()) {
      return hipErrorInvalidValue;  // the widest shapes take the streamed path only
    } else {
      if (dt == TT_BF16) {
        if constexpr (DK < 16 || CH < 32 || (CH == 64 && use_pipe<DK, NT>())) {
          return hipErrorInvalidValue;
        } else {
          return go(uint16_t{});
        }
      }
      return go(float{});
    }
  });
}

}  // namespace
}  // namespace tt
