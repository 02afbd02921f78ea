// Prefill plans and launches.  The kernels live in tt_prefill_kernels.hpp and
// tt_prefill_stream.hpp; this unit compiles the paths for chunks of 64 tokens
// (the warp-specialised pipe kernel for bf16 inputs with at most 256 feature
// rows, the streamed-state output pass for bf16 with n = 3 and dk = 32 or 64
// and for fp32 with more than 256 rows, the sweep kernel for everything
// else), and dispatches other chunk lengths
// to the units that compile the sweep kernel for them (tt_prefill_c16, _c32,
// _c128).
//
// "Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
// with a Fixed Number of Recurrent States" (abstract): the states add across
// token sets, so the chunking is free; the chunk length only moves work
// between the intra-chunk quadratic block and the state readout and update.
#include "tt_prefill_kernels.hpp"
#include "tt_prefill_stream.hpp"

namespace tt {

int plan_prefill(int B, int H, int N, int dk, int dv, int n, int chunk, tt_dtype dt, PrefillPlan* p) {
  (void)dv;
  if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
    return fail(TT_ERR_UNSUPPORTED, "chunk=%d not compiled (16, 32, 64 or 128)", chunk);
  if (dt == TT_BF16 && dk < 16) return fail(TT_ERR_UNSUPPORTED, "dk=%d prefill takes fp32 inputs only", dk);
  if (dt == TT_BF16 && chunk < 32)
    return fail(TT_ERR_UNSUPPORTED, "chunk=%d with bf16 inputs (32, 64 or 128: token blocks of 32)", chunk);
  if (dk >= 32 && n >= 4 && chunk != 64)
    return fail(TT_ERR_UNSUPPORTED, "chunk=%d with dk=%d, n=%d (these shapes run the streamed path: chunk 64)",
                chunk, dk, n);
  int wp = 0, ngroups = 0, nrg = 1, wg_per_cu = 2;
  bool stream = false;
  hipError_t e = hipSuccess;
  if (chunk == 64) {
    e = with_dkn(dk, n, [&](auto DKc, auto Nc) {
      constexpr int DK = decltype(DKc)::value, NT = decltype(Nc)::value;
      if constexpr (use_stream<DK, NT>()) {
        if (dt == TT_BF16) {  // large bf16 feature sets: the streamed-state output pass
          wp = StTot<DK>::WP;
          ngroups = 1;
          nrg = StTot<DK>::NRB;
          stream = true;
          return hipSuccess;
        }
      }
      if constexpr (use_stream_f32<DK, NT>()) {
        // large fp32 feature sets: the same, on fp32 MFMA; bf16 with dk = 16
        // and n >= 4 too (inputs widened to fp32 as they are staged)
        if (dt == TT_F32 || (dt == TT_BF16 && bf16_uses_stream_f32<DK, NT>())) {
          wp = StFT<DK, NT>::WP;
          ngroups = 1;
          nrg = StFT<DK, NT>::NRB;
          stream = true;
          return hipSuccess;
        }
      }
      if constexpr (use_pipe<DK, NT>()) {
        if (dt == TT_BF16) {
          wp = PCfg<DK, NT, MODE_OUTPUT>::WP;
          ngroups = 1;
          wg_per_cu = 1;
          return hipSuccess;
        }
      }
      return sweep_shape<64>(dk, n, dt, &wp, &ngroups, &nrg);
    });
  } else if (chunk == 16) {
    e = sweep_shape_chunk16(dk, n, dt, &wp, &ngroups, &nrg);
  } else if (chunk == 32) {
    e = sweep_shape_chunk32(dk, n, dt, &wp, &ngroups, &nrg);
  } else {
    e = sweep_shape_chunk128(dk, n, dt, &wp, &ngroups, &nrg);
  }
  if (e != hipSuccess) return fail(TT_ERR_UNSUPPORTED, "(dk=%d, n=%d, chunk=%d) not compiled", dk, n, chunk);
  const long long BH = (long long)B * H;
  if (stream) {  // spans of kStL tokens: the output pass's causal block is one span
    p->W = rows_for(dk, n);
    p->Wpad = wp;
    p->chunk = chunk;
    p->span = kStL;
    p->nspan = (N + kStL - 1) / kStL;
    p->ngroups = ngroups;
    p->nrg = nrg;
    p->part_floats = 0;
    p->ws_floats = (size_t)BH * p->nspan * (size_t)wp * (kDV + 1);
    p->streamed = true;
    return TT_OK;
  }
  const int nchunk = (N + chunk - 1) / chunk;
  // enough workgroups to fill the 256 CUs once
  const long long slots = 256LL * wg_per_cu;
  long long want = (slots + BH * ngroups * nrg - 1) / (BH * ngroups * nrg);
  if (want < 1) want = 1;
  if (want > nchunk) want = nchunk;
  const int span = (int)(((nchunk + want - 1) / want) * chunk);
  const int nspan = (N + span - 1) / span;
  p->W = rows_for(dk, n);
  p->Wpad = wp;
  p->chunk = chunk;
  p->span = span;
  p->nspan = nspan;
  p->ngroups = ngroups;
  p->nrg = nrg;
  p->part_floats = nrg > 1 ? (size_t)BH * nrg * (size_t)N * (kDV + 1) : 0;
  p->ws_floats = (size_t)BH * nspan * (size_t)wp * (kDV + 1) + p->part_floats;
  p->streamed = false;
  return TT_OK;
}

hipError_t launch_prefill(const void* Q, const void* K, const void* V, tt_dtype dt, int BH, int N, int dk, int n,
                          const PrefillPlan& p, const float* states_in, float* O, float* den_out, float* states,
                          float* ws, hipStream_t s, int bh0, int BHtot) {
  // head groups (bh0 > 0 or BHtot > BH) exist for the streamed paths only
  if (!p.streamed && (bh0 != 0 || BHtot != BH)) return hipErrorInvalidValue;
  if (p.chunk == 16) return sweep_launch_chunk16(Q, K, V, dt, BH, N, dk, n, p, states_in, O, den_out, states, ws, s);
  if (p.chunk == 32) return sweep_launch_chunk32(Q, K, V, dt, BH, N, dk, n, p, states_in, O, den_out, states, ws, s);
  if (p.chunk == 128)
    return sweep_launch_chunk128(Q, K, V, dt, BH, N, dk, n, p, states_in, O, den_out, states, ws, s);
  return with_dkn(dk, n, [&](auto DKc, auto Nc) -> hipError_t {
    constexpr int DK = decltype(DKc)::value, NT = decltype(Nc)::value;
    if constexpr (use_stream<DK, NT>()) {
      if (dt == TT_BF16)
        return stream_launch<DK>(Q, K, V, BH, N, p, states_in, O, den_out, states, ws, s, bh0, BHtot);
    }
    if constexpr (use_stream_f32<DK, NT>()) {
      if (dt == TT_F32)
        return stream_launch_f32<DK, NT, float>(Q, K, V, BH, N, p, states_in, O, den_out, states, ws, s, bh0,
                                                BHtot);
      if constexpr (bf16_uses_stream_f32<DK, NT>()) {
        if (dt == TT_BF16)
          return stream_launch_f32<DK, NT, uint16_t>(Q, K, V, BH, N, p, states_in, O, den_out, states, ws, s,
                                                     bh0, BHtot);
      }
    }
    if constexpr (use_pipe<DK, NT>()) {
      if (dt == TT_BF16) {
        using PT = PCfg<DK, NT, MODE_TOTALS>;
        using PO = PCfg<DK, NT, MODE_OUTPUT>;
        using PU = PCfg<DK, NT, MODE_OUTPUT_UNN>;
        const unsigned nblk = (unsigned)((size_t)BH * p.nspan);
        hipLaunchKernelGGL((pipe_kernel<PT>), dim3(nblk), dim3(PT::NTHR), 0, s, (const uint16_t*)Q,
                           (const uint16_t*)K, (const uint16_t*)V, N, p.span, p.nspan, ws, O, den_out);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_scan(ws, p, BH, (int)PO::WP, 0, states_in, states, s);
        if (e != hipSuccess) return e;
        if (den_out)
          hipLaunchKernelGGL((pipe_kernel<PU>), dim3(nblk), dim3(PU::NTHR), 0, s, (const uint16_t*)Q,
                             (const uint16_t*)K, (const uint16_t*)V, N, p.span, p.nspan, ws, O, den_out);
        else
          hipLaunchKernelGGL((pipe_kernel<PO>), dim3(nblk), dim3(PO::NTHR), 0, s, (const uint16_t*)Q,
                             (const uint16_t*)K, (const uint16_t*)V, N, p.span, p.nspan, ws, O, den_out);
        return hipGetLastError();
      }
    }
    return sweep_launch<64>(Q, K, V, dt, BH, N, dk, n, p, states_in, O, den_out, states, ws, s);
  });
}

}  // namespace tt
