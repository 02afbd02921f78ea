// C entry points of libtaylor_states.so: argument validation, planning and
// launch on the caller's stream.  No allocation, no global state apart from
// the thread-local error message and the fixed device scratch array of the
// no-allocation prefill (below).
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "tt_device.hpp"
#include "tt_internal.hpp"

namespace tt {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

static int ok() {
  g_err[0] = '\0';
  return TT_OK;
}

static int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool shape_supported(int dk, int dv, int n) {
  if (dv != 64 || n < 1) return false;
  if (dk == 8) return n <= 6;
  if (dk == 16) return n <= 5;
  if (dk == 32 || dk == 64) return n <= 5;
  return false;
}

static int check_shape(int dk, int dv, int n) {
  if (dk < 1 || dv < 1 || n < 1) return fail(TT_ERR_INVALID_ARG, "dk=%d dv=%d n=%d must be >= 1", dk, dv, n);
  if (!shape_supported(dk, dv, n))
    return fail(TT_ERR_UNSUPPORTED,
                "(dk=%d, dv=%d, n=%d) not compiled: dv must be 64; dk=8 with n<=6, dk=16, 32 or 64 with n<=5",
                dk, dv, n);
  return TT_OK;
}

static int check_dtype(tt_dtype dt) {
  if (dt != TT_F32 && dt != TT_BF16) return fail(TT_ERR_INVALID_ARG, "in_dtype %d is not TT_F32/TT_BF16", (int)dt);
  return TT_OK;
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool valid_scale(float s) { return s > 0.0f && s <= 3.4028235e38f; }  // finite and positive

// Bytes of one normalised copy of Q (or K) in the workspace of the normalised
// prefill; sized for fp32 so that one query serves both dtypes.
static size_t normed_copy_bytes(int B, int H, int N, int dk) {
  return align256((size_t)B * H * N * dk * sizeof(float));
}

// tt_prefill, tt_prefill_from and tt_prefill_normed: states_in is null for
// zero states; normed: Q and K are first normalised into the workspace tail
// (Q scaled by qscale) and the prefill reads those copies.
static int prefill_impl(const void* Q, const void* K, const void* V, tt_dtype in_dtype, int B, int H, int N,
                        int dk, int dv, int n, int chunk, const float* states_in, float* O, float* den,
                        float* states, void* workspace, size_t workspace_bytes, bool normed, float qscale,
                        void* stream, const char* name) {
  if (!Q || !K || !V || !O || !states) return fail(TT_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (B < 1 || H < 1 || N < 1) return fail(TT_ERR_INVALID_ARG, "B=%d H=%d N=%d must be >= 1", B, H, N);
  int rc = check_dtype(in_dtype);
  if (rc) return rc;
  rc = check_shape(dk, dv, n);
  if (rc) return rc;
  if ((long long)B * H > (1LL << 24)) return fail(TT_ERR_UNSUPPORTED, "B*H=%lld too large", (long long)B * H);
  PrefillPlan p;
  rc = plan_prefill(B, H, N, dk, dv, n, chunk, in_dtype, &p);
  if (rc) return rc;
  const size_t base = p.ws_floats * sizeof(float);
  const size_t copy = normed ? normed_copy_bytes(B, H, N, dk) : 0;
  const size_t need = normed ? align256(base) + 2 * copy : base;
  if (normed && !valid_scale(qscale))
    return fail(TT_ERR_INVALID_ARG, "temperature %g must be finite and positive", (double)qscale);
  // Streamed plans (spans of a fixed length) run the heads in groups when the
  // workspace holds the span states (and, normalised, the copies of Q and K)
  // of fewer than all heads but at least one.
  const int BH = B * H;
  const size_t per_head = base / (size_t)BH;
  auto need_for = [&](size_t g) {
    return normed ? align256(per_head * g) + 2 * normed_copy_bytes(1, (int)g, N, dk) : per_head * g;
  };
  int group = BH;
  size_t used = need;
  if (p.streamed && workspace && need > 0 && workspace_bytes < need) {
    const size_t per_total = need_for(1);
    size_t g = workspace_bytes / per_total;  // within one of the largest fit
    while (g > 0 && need_for(g) > workspace_bytes) --g;
    while (g + 1 < (size_t)BH && need_for(g + 1) <= workspace_bytes) ++g;
    if (g >= 1) {
      // as many groups as g heads each need, with the heads spread evenly
      const size_t ngroups = ((size_t)BH + g - 1) / g;
      group = (int)(((size_t)BH + ngroups - 1) / ngroups);
      used = need_for((size_t)group);
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < used)) {
    if (p.streamed)
      return fail(TT_ERR_WORKSPACE, "workspace of %zu bytes needed (or %zu per head, heads in groups), %zu given",
                  need, need_for(1), workspace ? workspace_bytes : (size_t)0);
    return fail(TT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  }
  if ((((uintptr_t)Q) | ((uintptr_t)K) | ((uintptr_t)V) | ((uintptr_t)O) | ((uintptr_t)workspace)) & 15u)
    return fail(TT_ERR_INVALID_ARG, "Q, K, V, O and workspace must be 16-byte aligned");
  if (den) {
    const size_t db = (size_t)B * H * N * sizeof(float);
    const size_t sb = (size_t)B * H * tt_state_floats(dk, dv, n) * sizeof(float);
    if (((uintptr_t)den) & 3u) return fail(TT_ERR_INVALID_ARG, "den must be 4-byte aligned");
    if (overlap(den, db, O, (size_t)B * H * N * dv * sizeof(float)) || overlap(den, db, states, sb) ||
        (states_in && overlap(den, db, states_in, sb)) || (workspace && overlap(den, db, workspace, used)))
      return fail(TT_ERR_INVALID_ARG, "den overlaps O, the states or the workspace");
  }
  if (states_in) {
    const size_t sb = (size_t)B * H * tt_state_floats(dk, dv, n) * sizeof(float);
    if (states_in != states && overlap(states_in, sb, states, sb))
      return fail(TT_ERR_INVALID_ARG, "states_in and states overlap without being the same buffer");
    if (overlap(states_in, sb, O, (size_t)B * H * N * dv * sizeof(float)) ||
        (workspace && overlap(states_in, sb, workspace, used)))
      return fail(TT_ERR_INVALID_ARG, "states_in overlaps O or the workspace");
  }
  char what[64];
  snprintf(what, sizeof(what), "%s launch", name);
  // head groups (one group of all heads when the workspace holds them), one
  // after another on the stream, each with the workspace from its start
  const size_t esz = in_dtype == TT_BF16 ? 2 : 4;
  PrefillPlan pg = p;
  for (int g0 = 0; g0 < BH; g0 += group) {
    const int gs = group < BH - g0 ? group : BH - g0;
    pg.ws_floats = p.ws_floats / (size_t)BH * (size_t)gs;
    const void* Qg = (const char*)Q + (size_t)g0 * N * dk * esz;
    const void* Kg = (const char*)K + (size_t)g0 * N * dk * esz;
    if (normed) {  // normalised copies of this group's rows after its span states
      unsigned char* qn = (unsigned char*)workspace + align256(pg.ws_floats * sizeof(float));
      unsigned char* kn = qn + normed_copy_bytes(1, gs, N, dk);
      const size_t rows = (size_t)gs * N;
      const hipError_t e =
          launch_normalize(in_dtype, dk, Qg, qn, qscale, rows, Kg, kn, 1.0f, rows, (hipStream_t)stream);
      if (e != hipSuccess) return hip_status(e, what);
      Qg = qn;
      Kg = kn;
    }
    const hipError_t e = launch_prefill(Qg, Kg, (const char*)V + (size_t)g0 * N * dv * esz, in_dtype, gs, N, dk, n,
                                        pg, states_in, O + (size_t)g0 * N * dv, den ? den + (size_t)g0 * N : nullptr,
                                        states, (float*)workspace, (hipStream_t)stream, g0, BH);
    if (e != hipSuccess) return hip_status(e, what);
  }
  return ok();
}

static int decode_impl(const void* q, const void* k, const void* v, tt_dtype in_dtype, int B, int H, int dk,
                       int dv, int n, float* states, float* o, bool normed, float qscale, void* stream,
                       const char* name) {
  if (!q || !k || !v || !states || !o) return fail(TT_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (B < 1 || H < 1) return fail(TT_ERR_INVALID_ARG, "B=%d H=%d must be >= 1", B, H);
  int rc = check_dtype(in_dtype);
  if (rc) return rc;
  rc = check_shape(dk, dv, n);
  if (rc) return rc;
  if (normed && !valid_scale(qscale))
    return fail(TT_ERR_INVALID_ARG, "temperature %g must be finite and positive", (double)qscale);
  if ((long long)B * H > 0x7fffffffLL) return fail(TT_ERR_UNSUPPORTED, "B*H too large");
  char what[64];
  snprintf(what, sizeof(what), "%s launch", name);
  return hip_status(launch_decode(q, k, v, in_dtype, B * H, dk, n, states, o, normed, qscale, (hipStream_t)stream),
                    what);
}

// Device scratch of tt_prefill_noalloc: one array per GPU, loaded with the
// code object and held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress returns for
// the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[TT_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

// Device address of `scratch` on the current device (null on error, with
// the error recorded for tt_last_error()).
static void* scratch_for_current_device(int* rc) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *rc = hip_status(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *rc = fail(TT_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
    *rc = hip_status(g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev] : hipErrorInvalidSymbol,
                     "hipGetSymbolAddress(scratch)");
    return nullptr;
  }
  *rc = TT_OK;
  return g_scratch_ptr[dev];
}

// Row codes of the widest shapes (dk = 32 and 64 with four or five terms:
// up to 58,905 and 814,385 rows, too many for a compile-time table in every
// kernel's code object): one table per key width and GPU, enumerated on the
// host in feature order (enumerate_rows, the generator of the compile-time
// tables), copied once per device on first use (a synchronous copy) and held
// until the process ends.  Kernels get its device address as an argument.
static __device__ uint32_t big_rows32[rows_for(32, 5)];
static __device__ uint32_t big_rows64[rows_for(64, 5)];

namespace {
std::once_flag g_rows_once[2][kMaxDevices];
const uint32_t* g_rows_ptr[2][kMaxDevices];
hipError_t g_rows_err[2][kMaxDevices];
}  // namespace

hipError_t big_row_codes(int dk, int n, const uint32_t** out) {
  *out = nullptr;
  if (n <= max_terms(dk)) return hipSuccess;  // the compile-time tables serve
  if ((dk != 32 && dk != 64) || n > 5) return hipErrorInvalidValue;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  const int w = dk == 32 ? 0 : 1;
  std::call_once(g_rows_once[w][dev], [dk, w, dev] {
    const int W = rows_for(dk, 5);
    uint32_t* codes = new uint32_t[(size_t)W];
    enumerate_rows(dk, 5, index_bits(dk), codes, nullptr);
    void* p = nullptr;
    hipError_t r = dk == 32 ? hipGetSymbolAddress(&p, HIP_SYMBOL(big_rows32))
                            : hipGetSymbolAddress(&p, HIP_SYMBOL(big_rows64));
    if (r == hipSuccess) r = hipMemcpy(p, codes, (size_t)W * sizeof(uint32_t), hipMemcpyHostToDevice);
    delete[] codes;
    g_rows_err[w][dev] = r;
    g_rows_ptr[w][dev] = r == hipSuccess ? static_cast<const uint32_t*>(p) : nullptr;
  });
  if (g_rows_err[w][dev] != hipSuccess) return g_rows_err[w][dev];
  *out = g_rows_ptr[w][dev];
  return *out ? hipSuccess : hipErrorInvalidSymbol;
}

}  // namespace tt

using namespace tt;

extern "C" {

size_t tt_state_rows(int dk, int n) {
  if (dk < 1 || n < 1) return 0;
  // C(dk+n-1, n-1) computed incrementally; exact at each step
  unsigned __int128 r = 1;
  for (int i = 1; i <= n - 1; ++i) {
    r = r * (unsigned __int128)(dk + i) / (unsigned __int128)i;
    if (r > (unsigned __int128)SIZE_MAX) return 0;
  }
  return (size_t)r;
}

size_t tt_state_floats(int dk, int dv, int n) {
  if (dv < 1) return 0;
  const size_t w = tt_state_rows(dk, n);
  if (w == 0) return 0;
  unsigned __int128 f = (unsigned __int128)w * (unsigned __int128)(dv + 1);
  if (f > (unsigned __int128)SIZE_MAX) return 0;
  return (size_t)f;
}

int tt_prefill_workspace_bytes(int B, int H, int N, int dk, int dv, int n, int chunk, size_t* bytes) {
  if (!bytes) return fail(TT_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 1 || H < 1 || N < 1) return fail(TT_ERR_INVALID_ARG, "B=%d H=%d N=%d must be >= 1", B, H, N);
  int rc = check_shape(dk, dv, n);
  if (rc) return rc;
  // the query takes no dtype: report the larger of the fp32 and bf16 plans,
  // over the dtypes this shape and chunk length run with (an error only if
  // neither does)
  PrefillPlan pf, pb;
  const int rf = plan_prefill(B, H, N, dk, dv, n, chunk, TT_F32, &pf);
  const int rb = plan_prefill(B, H, N, dk, dv, n, chunk, TT_BF16, &pb);
  if (rf && rb) return plan_prefill(B, H, N, dk, dv, n, chunk, TT_F32, &pf);  // the fp32 message
  size_t w = 0;
  if (!rf) w = pf.ws_floats;
  if (!rb && pb.ws_floats > w) w = pb.ws_floats;
  *bytes = w * sizeof(float);
  return ok();
}

int tt_prefill_workspace_bytes_dtype(int B, int H, int N, int dk, int dv, int n, int chunk, tt_dtype in_dtype,
                                     size_t* bytes) {
  if (!bytes) return fail(TT_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 1 || H < 1 || N < 1) return fail(TT_ERR_INVALID_ARG, "B=%d H=%d N=%d must be >= 1", B, H, N);
  int rc = check_dtype(in_dtype);
  if (rc) return rc;
  rc = check_shape(dk, dv, n);
  if (rc) return rc;
  PrefillPlan p;
  rc = plan_prefill(B, H, N, dk, dv, n, chunk, in_dtype, &p);
  if (rc) return rc;
  *bytes = p.ws_floats * sizeof(float);
  return ok();
}

int tt_prefill(const void* Q, const void* K, const void* V, tt_dtype in_dtype, int B, int H, int N, int dk,
               int dv, int n, int chunk, float* O, float* states, void* workspace, size_t workspace_bytes,
               void* stream) {
  return prefill_impl(Q, K, V, in_dtype, B, H, N, dk, dv, n, chunk, nullptr, O, nullptr, states, workspace,
                      workspace_bytes, false, 1.0f, stream, "tt_prefill");
}

int tt_prefill_noalloc(const void* Q, const void* K, const void* V, tt_dtype in_dtype, int B, int H, int N, int dk,
                       int dv, int n, int chunk, float* O, float* states, void* stream) {
  if (B < 1 || H < 1 || N < 1) return fail(TT_ERR_INVALID_ARG, "B=%d H=%d N=%d must be >= 1", B, H, N);
  size_t need = 0;
  int rc = tt_prefill_workspace_bytes_dtype(B, H, N, dk, dv, n, chunk, in_dtype, &need);
  if (rc) return rc;
  // a streamed plan runs its heads in groups that fit the scratch
  PrefillPlan p;
  if (plan_prefill(B, H, N, dk, dv, n, chunk, in_dtype, &p) == TT_OK && p.streamed)
    need = p.ws_floats / ((size_t)B * H) * sizeof(float);
  if (need > (size_t)TT_NOALLOC_SCRATCH_BYTES)
    return fail(TT_ERR_WORKSPACE,
                "this shape needs %zu bytes of scratch; tt_prefill_noalloc holds %zu (use tt_prefill with a "
                "workspace)",
                need, (size_t)TT_NOALLOC_SCRATCH_BYTES);
  void* ws = scratch_for_current_device(&rc);
  if (!ws) return rc;
  return prefill_impl(Q, K, V, in_dtype, B, H, N, dk, dv, n, chunk, nullptr, O, nullptr, states, ws,
                      (size_t)TT_NOALLOC_SCRATCH_BYTES, false, 1.0f, stream, "tt_prefill_noalloc");
}

int tt_prefill_from(const void* Q, const void* K, const void* V, tt_dtype in_dtype, int B, int H, int N, int dk,
                    int dv, int n, int chunk, const float* states_in, float* O, float* states, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!states_in) return fail(TT_ERR_INVALID_ARG, "states_in is NULL (use tt_prefill for zero states)");
  return prefill_impl(Q, K, V, in_dtype, B, H, N, dk, dv, n, chunk, states_in, O, nullptr, states, workspace,
                      workspace_bytes, false, 1.0f, stream, "tt_prefill_from");
}

int tt_prefill_from_unnormalized(const void* Q, const void* K, const void* V, tt_dtype in_dtype, int B, int H,
                                 int N, int dk, int dv, int n, int chunk, const float* states_in, float* num,
                                 float* den, float* states, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!den) return fail(TT_ERR_INVALID_ARG, "den is NULL");
  return prefill_impl(Q, K, V, in_dtype, B, H, N, dk, dv, n, chunk, states_in, num, den, states, workspace,
                      workspace_bytes, false, 1.0f, stream, "tt_prefill_from_unnormalized");
}

int tt_prefill_normed_workspace_bytes(int B, int H, int N, int dk, int dv, int n, int chunk, size_t* bytes) {
  int rc = tt_prefill_workspace_bytes(B, H, N, dk, dv, n, chunk, bytes);
  if (rc) return rc;
  *bytes = align256(*bytes) + 2 * normed_copy_bytes(B, H, N, dk);
  return ok();
}

int tt_prefill_normed(const void* Q, const void* K, const void* V, tt_dtype in_dtype, int B, int H, int N, int dk,
                      int dv, int n, int chunk, float temperature, const float* states_in, float* O,
                      float* states, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(Q, K, V, in_dtype, B, H, N, dk, dv, n, chunk, states_in, O, nullptr, states, workspace,
                      workspace_bytes, true, temperature, stream, "tt_prefill_normed");
}

int tt_normalize_rows(const void* x, tt_dtype in_dtype, size_t rows, int d, float scale, void* out, void* stream) {
  if (rows == 0) return ok();
  if (!x || !out) return fail(TT_ERR_INVALID_ARG, "a pointer is NULL");
  int rc = check_dtype(in_dtype);
  if (rc) return rc;
  if (d < 1) return fail(TT_ERR_INVALID_ARG, "d=%d must be >= 1", d);
  if (d != 8 && d != 16 && d != 32 && d != 64)
    return fail(TT_ERR_UNSUPPORTED, "d=%d not compiled (8, 16, 32 or 64)", d);
  if (!valid_scale(scale)) return fail(TT_ERR_INVALID_ARG, "scale %g must be finite and positive", (double)scale);
  if ((((uintptr_t)x) | ((uintptr_t)out)) & 15u) return fail(TT_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  const size_t nb = rows * (size_t)d * (in_dtype == TT_F32 ? 4 : 2);
  if (x != out && overlap(x, nb, out, nb)) return fail(TT_ERR_INVALID_ARG, "x and out overlap without being equal");
  return hip_status(launch_normalize(in_dtype, d, x, out, scale, rows, nullptr, nullptr, 1.0f, 0, (hipStream_t)stream),
                    "tt_normalize_rows launch");
}

int tt_decode_step(const void* q, const void* k, const void* v, tt_dtype in_dtype, int B, int H, int dk, int dv,
                   int n, float* states, float* o, void* stream) {
  return decode_impl(q, k, v, in_dtype, B, H, dk, dv, n, states, o, false, 1.0f, stream, "tt_decode_step");
}

int tt_decode_step_normed(const void* q, const void* k, const void* v, tt_dtype in_dtype, int B, int H, int dk,
                          int dv, int n, float temperature, float* states, float* o, void* stream) {
  return decode_impl(q, k, v, in_dtype, B, H, dk, dv, n, states, o, true, temperature, stream,
                     "tt_decode_step_normed");
}

int tt_state_merge(float* dst, const float* a, const float* b, size_t nfloats, void* stream) {
  if (nfloats == 0) return ok();
  if (!dst || !a || !b) return fail(TT_ERR_INVALID_ARG, "a pointer is NULL");
  return hip_status(launch_merge(dst, a, b, nfloats, (hipStream_t)stream), "tt_state_merge launch");
}

int tt_feature_map(const void* x, tt_dtype in_dtype, size_t rows, int dk, int n, int weighted, float* out,
                   void* stream) {
  if (rows == 0) return ok();
  if (!x || !out) return fail(TT_ERR_INVALID_ARG, "a pointer is NULL");
  if (weighted != 0 && weighted != 1) return fail(TT_ERR_INVALID_ARG, "weighted must be 0 or 1");
  int rc = check_dtype(in_dtype);
  if (rc) return rc;
  if (dk < 1 || n < 1) return fail(TT_ERR_INVALID_ARG, "dk=%d n=%d must be >= 1", dk, n);
  if (!shape_supported(dk, 64, n)) return fail(TT_ERR_UNSUPPORTED, "(dk=%d, n=%d) not compiled", dk, n);
  return hip_status(launch_feature_map(x, in_dtype, rows, dk, n, weighted, out, (hipStream_t)stream),
                    "tt_feature_map launch");
}

int tt_softmax_prefill(const void* Q, const void* K, const void* V, tt_dtype in_dtype, int B, int H, int N, int dk,
                       int dv, float* O, void* stream) {
  if (!Q || !K || !V || !O) return fail(TT_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (B < 1 || H < 1 || N < 1 || dk < 1 || dv < 1)
    return fail(TT_ERR_INVALID_ARG, "B=%d H=%d N=%d dk=%d dv=%d must be >= 1", B, H, N, dk, dv);
  int rc = check_dtype(in_dtype);
  if (rc) return rc;
  if (in_dtype != TT_BF16) return fail(TT_ERR_UNSUPPORTED, "tt_softmax_prefill takes bf16 inputs only");
  if ((dk != 16 && dk != 32 && dk != 64) || dv != 64)
    return fail(TT_ERR_UNSUPPORTED, "(dk=%d, dv=%d) not compiled: dk in {16, 32, 64}, dv = 64", dk, dv);
  if ((long long)B * H * ((N + 63) / 64) > 0x7fffffffLL) return fail(TT_ERR_UNSUPPORTED, "too many query blocks");
  if ((((uintptr_t)Q) | ((uintptr_t)K) | ((uintptr_t)V) | ((uintptr_t)O)) & 15u)
    return fail(TT_ERR_INVALID_ARG, "Q, K, V and O must be 16-byte aligned");
  return hip_status(launch_softmax_prefill(Q, K, V, B * H, N, dk, O, (hipStream_t)stream),
                    "tt_softmax_prefill launch");
}

int tt_softmax_decode_workspace_bytes(int B, int H, int pos, size_t* bytes) {
  if (!bytes) return fail(TT_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 1 || H < 1 || pos < 0) return fail(TT_ERR_INVALID_ARG, "B=%d H=%d must be >= 1, pos=%d >= 0", B, H, pos);
  *bytes = (size_t)B * H * softmax_decode_splits(pos) * (64 + 2) * sizeof(float);
  return ok();
}

int tt_softmax_decode_step(const void* q, const void* k, const void* v, tt_dtype in_dtype, int B, int H, int dk,
                           int dv, void* Kcache, void* Vcache, int pos, int capacity, float* o, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !Kcache || !Vcache || !o) return fail(TT_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (B < 1 || H < 1 || dk < 1 || dv < 1)
    return fail(TT_ERR_INVALID_ARG, "B=%d H=%d dk=%d dv=%d must be >= 1", B, H, dk, dv);
  if (pos < 0 || pos >= capacity)
    return fail(TT_ERR_INVALID_ARG, "pos=%d must lie in [0, capacity=%d)", pos, capacity);
  int rc = check_dtype(in_dtype);
  if (rc) return rc;
  if ((dk != 16 && dk != 32 && dk != 64) || dv != 64)
    return fail(TT_ERR_UNSUPPORTED, "(dk=%d, dv=%d) not compiled: dk in {16, 32, 64}, dv = 64", dk, dv);
  if ((long long)B * H > 65535) return fail(TT_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)B * H);
  if ((((uintptr_t)Kcache) | ((uintptr_t)Vcache)) & 15u)
    return fail(TT_ERR_INVALID_ARG, "Kcache and Vcache must be 16-byte aligned");
  size_t need = 0;
  rc = tt_softmax_decode_workspace_bytes(B, H, pos, &need);
  if (rc) return rc;
  if (!workspace || workspace_bytes < need)
    return fail(TT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  return hip_status(launch_softmax_decode(q, k, v, in_dtype, B * H, dk, Kcache, Vcache, pos, capacity, o,
                                          (float*)workspace, (hipStream_t)stream),
                    "tt_softmax_decode_step launch");
}

const char* tt_last_error(void) { return g_err; }

}  // extern "C"
