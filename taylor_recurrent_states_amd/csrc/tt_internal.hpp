// Host-side declarations shared by the translation units of libtaylor_states.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/taylor_states.h"

namespace tt {

// Records a message for tt_last_error() and returns `code`.
int fail(int code, const char* fmt, ...);

// Device address of the run-time row-code table of (dk, n) when n exceeds the
// compile-time tables of dk (dk = 32 or 64 with n = 4 or 5; built on the
// current device on first use), else null.  Every launcher of such a shape
// passes it to its kernels.
hipError_t big_row_codes(int dk, int n, const uint32_t** out);

// Launchers (argument checking is done by the C entry points).
hipError_t launch_feature_map(const void* x, tt_dtype dt, size_t rows, int dk, int n, int weighted,
                              float* out, hipStream_t s);
hipError_t launch_merge(float* dst, const float* a, const float* b, size_t n, hipStream_t s);
// normed: q and k are normalised in the kernel (q scaled by qscale).
hipError_t launch_decode(const void* q, const void* k, const void* v, tt_dtype dt, int BH, int dk, int n,
                         float* states, float* o, bool normed, float qscale, hipStream_t s);
// Row normalisation of two row sets (d in {16, 32, 64}, 16-byte aligned rows):
// out0 = r(s0 x0 / |x0|) for rows0 rows, then the same for x1 with s1.
hipError_t launch_normalize(tt_dtype dt, int d, const void* x0, void* out0, float s0, size_t rows0,
                            const void* x1, void* out1, float s1, size_t rows1, hipStream_t s);

// Softmax baseline: causal prefill (bf16 inputs, dk in {16, 32, 64}, dv = 64)
// and one decode step against a KV cache.  Decode partials: one record of
// dv + 2 floats per (head, split of 2048 keys); softmax_decode_splits(pos)
// splits cover keys 0 .. pos.
hipError_t launch_softmax_prefill(const void* Q, const void* K, const void* V, int BH, int N, int dk, float* O,
                                  hipStream_t s);
size_t softmax_decode_splits(int pos);
hipError_t launch_softmax_decode(const void* q, const void* k, const void* v, tt_dtype dt, int BH, int dk,
                                 void* Kc, void* Vc, int pos, int cap, float* o, float* part, hipStream_t s);

// Prefill plan: how the sequence and the columns are split over workgroups.
struct PrefillPlan {
  int W;          // feature rows
  int Wpad;       // rows rounded up to the row-tile multiple
  int chunk;      // tokens per chunk
  int span;       // tokens per span (multiple of chunk)
  int nspan;      // spans per head
  int ngroups;    // column groups (workgroups per head-span)
  int nrg;        // row groups (workgroups per head-span and column group)
  size_t part_floats;  // row-group partial outputs, floats (0 with one row group)
  size_t ws_floats;    // workspace: span states, then the partial outputs, floats
  bool streamed;       // the streamed-state path: spans of a fixed length, whatever the head count, so the
                       // heads can run in groups with one group's workspace (ws_floats is per head x BH)
};

int plan_prefill(int B, int H, int N, int dk, int dv, int n, int chunk, tt_dtype dt, PrefillPlan* p);
// states_in: carried-in states in the plane layout, or null for zero states.
// den_out: null for normalised outputs; otherwise O receives the numerators
// and den_out [BH][N] the normalisers.  Q, K, V, O and den_out hold the BH
// heads of this launch; states_in and states hold BHtot heads (plane layout)
// of which this launch's are bh0 .. bh0 + BH - 1 (bh0 = 0, BHtot = BH except
// for head groups of a streamed plan).
hipError_t launch_prefill(const void* Q, const void* K, const void* V, tt_dtype dt, int BH, int N, int dk,
                          int n, const PrefillPlan& p, const float* states_in, float* O, float* den_out,
                          float* states, float* ws, hipStream_t s, int bh0, int BHtot);

// The sweep-kernel prefill path for chunks of 16, 32 and 128 tokens (one
// compilation unit each): plan figures and launches, as for 64 tokens.
hipError_t sweep_shape_chunk16(int dk, int n, tt_dtype dt, int* wp, int* ngroups, int* nrg);
hipError_t sweep_shape_chunk32(int dk, int n, tt_dtype dt, int* wp, int* ngroups, int* nrg);
hipError_t sweep_shape_chunk128(int dk, int n, tt_dtype dt, int* wp, int* ngroups, int* nrg);
#define TT_SWEEP_LAUNCH_DECL(NAME)                                                                              \
  hipError_t NAME(const void* Q, const void* K, const void* V, tt_dtype dt, int BH, int N, int dk, int n,         \
                  const PrefillPlan& p, const float* states_in, float* O, float* den_out, float* states, float* ws, \
                  hipStream_t s);
TT_SWEEP_LAUNCH_DECL(sweep_launch_chunk16)
TT_SWEEP_LAUNCH_DECL(sweep_launch_chunk32)
TT_SWEEP_LAUNCH_DECL(sweep_launch_chunk128)
#undef TT_SWEEP_LAUNCH_DECL

}  // namespace tt
