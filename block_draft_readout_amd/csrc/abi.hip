// C ABI of libbdr: argument validation, workspace sizing and dispatch to the
// gfx950 kernel launchers.  Every host-checkable argument is validated before
// anything is enqueued; the device architecture is checked once per device.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "bdr_internal.h"

using namespace bdr;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(BDR_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

bool valid_dtype(int dt) { return dt == BDR_F32 || dt == BDR_BF16; }
// calls with a GEMM weight also take the packed bf16 layout
bool valid_gemm_dtype(int dt) { return valid_dtype(dt) || dt == BDR_BF16_PACKED; }

constexpr int64_t kMaxVocab = 0x7FFFFFFELL;
constexpr int64_t kMaxElems = int64_t(1) << 40;  // per tensor; keeps index math in range
constexpr int64_t kMaxBytes = 0x7FFFFFFFLL;      // per buffer resource
constexpr int64_t kMaxMarkovVocab = int64_t(1) << 21;

// 0 unknown, 1 gfx950, 2 other; compute units per device
int g_dev_state[256];
int g_dev_cus[256];
std::mutex g_dev_mu;

// Checks that the current device is gfx950; *cus receives its compute-unit count.
int check_device(int* cus = nullptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 256) return fail(BDR_EUNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_cus[dev] = prop.multiProcessorCount;
    if (g_dev_state[dev] == 2)
      return fail(BDR_EUNSUPPORTED, "device %d is %s; libbdr is built for gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (g_dev_state[dev] != 1)
    return fail(BDR_EUNSUPPORTED, "device %d is not gfx950; libbdr is built for gfx950 only", dev);
  if (cus) *cus = g_dev_cus[dev];
  return BDR_OK;
}

int need_ptr(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(BDR_EINVAL, "%s must not be NULL", name);
  if (!aligned(p, align)) return fail(BDR_EINVAL, "%s must be %zu-byte aligned", name, align);
  return BDR_OK;
}

int need_ws(const void* ws, size_t have, size_t need) {
  if (need == 0) return BDR_OK;
  if (!ws) return fail(BDR_EWORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned(ws, 256)) return fail(BDR_EWORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(BDR_EWORKSPACE, "workspace of %zu bytes required, got %zu", need, have);
  return BDR_OK;
}

#define BDR_TRY(x)               \
  do {                           \
    const int rc_ = (x);         \
    if (rc_ != BDR_OK) return rc_; \
  } while (0)

int fc_shape(int64_t rows, int64_t hidden, int n_taps, int wdt) {
  if (!valid_gemm_dtype(wdt)) return fail(BDR_EINVAL, "unknown dtype %d", wdt);
  const int dt = act_dtype(static_cast<bdr_dtype>(wdt));
  if (n_taps < 1) return fail(BDR_EINVAL, "n_taps must be >= 1, got %d", n_taps);
  if (n_taps > BDR_MAX_TAPS) return fail(BDR_EUNSUPPORTED, "n_taps %d > %d", n_taps, BDR_MAX_TAPS);
  if (rows < 0) return fail(BDR_EINVAL, "rows must be >= 0");
  if (hidden <= 0) return fail(BDR_EINVAL, "hidden must be > 0");
  const int ks = dt == BDR_BF16 ? 32 : 16;
  if (hidden % ks)
    return fail(BDR_EUNSUPPORTED, "hidden %lld must be a multiple of %d for this dtype",
                static_cast<long long>(hidden), ks);
  // each tap [rows, H] and each 64-row slab of fc_w must stay below 2^31 bytes
  const int64_t es = dt == BDR_BF16 ? 2 : 4;
  if (rows > kMaxBytes / (hidden * es) || hidden * n_taps > kMaxBytes / (64 * es))
    return fail(BDR_EUNSUPPORTED, "fc problem too large (per-operand byte limit 2^31)");
  if (wdt == BDR_BF16_PACKED) {
    if (n_taps > 1 && hidden % 128)
      return fail(BDR_EUNSUPPORTED, "a multi-tap fc with packed weights needs hidden %% 128 == 0");
    if (packed_weight_bytes(hidden, hidden * n_taps) == 0)
      return fail(BDR_EUNSUPPORTED, "packed fc_w would reach 2^31 bytes");
  }
  return BDR_OK;
}

int lm_shape(int64_t rows, int64_t hidden, int64_t vocab, int wdt) {
  if (!valid_gemm_dtype(wdt)) return fail(BDR_EINVAL, "unknown dtype %d", wdt);
  const int dt = act_dtype(static_cast<bdr_dtype>(wdt));
  if (rows < 0) return fail(BDR_EINVAL, "rows must be >= 0");
  if (hidden <= 0) return fail(BDR_EINVAL, "hidden must be > 0");
  if (vocab <= 0) return fail(BDR_EINVAL, "vocab must be > 0");
  if (vocab > kMaxVocab) return fail(BDR_EUNSUPPORTED, "vocab must be < 2^31 - 1");
  const int e = dt == BDR_BF16 ? 8 : 4;
  if (hidden % e)
    return fail(BDR_EUNSUPPORTED, "hidden %lld must be a multiple of %d for this dtype",
                static_cast<long long>(hidden), e);
  const int64_t es = dt == BDR_BF16 ? 2 : 4;
  if (rows > kMaxBytes / (hidden * es) || hidden > kMaxBytes / (64 * es) ||
      vocab > kMaxElems / hidden || rows > kMaxElems / vocab)
    return fail(BDR_EUNSUPPORTED, "LM-head problem too large (per-operand byte limit 2^31)");
  if (wdt == BDR_BF16_PACKED) {
    if (packed_weight_bytes(vocab, hidden) == 0)
      return fail(BDR_EUNSUPPORTED, "packed lm_head_w would reach 2^31 bytes");
    // a slab's logits are addressed with 32-bit offsets
    if (std::min<int64_t>(rows, kPackedSlabRows) * vocab * 4 >= (int64_t(1) << 32))
      return fail(BDR_EUNSUPPORTED, "LM head with packed weights: vocab too large");
  }
  return BDR_OK;
}

int block_shape(int64_t batch, int k, int64_t vocab) {
  if (batch < 0) return fail(BDR_EINVAL, "batch must be >= 0");
  if (k < 1) return fail(BDR_EINVAL, "k must be >= 1, got %d", k);
  if (k > BDR_MAX_K) return fail(BDR_EUNSUPPORTED, "k %d > %d", k, BDR_MAX_K);
  if (vocab <= 0) return fail(BDR_EINVAL, "vocab must be > 0");
  if (vocab > kMaxVocab) return fail(BDR_EUNSUPPORTED, "vocab must be < 2^31 - 1");
  if (batch > 0x7FFFFFFFLL / (k + 1)) return fail(BDR_EUNSUPPORTED, "batch too large");
  if (batch * (k + 1) > kMaxElems / vocab) return fail(BDR_EUNSUPPORTED, "block too large");
  return BDR_OK;
}

int markov_shape(int dt, const void* w1, const void* w2, int rank, int64_t vocab, int k) {
  if (!valid_dtype(dt)) return fail(BDR_EINVAL, "unknown dtype %d", dt);
  // logits of 16 rows of one position, and each Markov matrix, under 2^31 bytes
  if (vocab > kMaxMarkovVocab) return fail(BDR_EUNSUPPORTED, "vocab must be <= 2^21 here");
  if (rank < 0) return fail(BDR_EINVAL, "rank must be >= 0");
  if (rank > BDR_MAX_RANK) return fail(BDR_EUNSUPPORTED, "rank %d > %d", rank, BDR_MAX_RANK);
  if ((w1 == nullptr) != (w2 == nullptr))
    return fail(BDR_EINVAL, "markov_w1 and markov_w2 must both be given or both be NULL");
  if (w1 && rank > 0) {
    const int e = dt == BDR_BF16 ? 8 : 4;
    if (rank % e) return fail(BDR_EUNSUPPORTED, "rank %d must be a multiple of %d for this dtype", rank, e);
    BDR_TRY(need_ptr(w1, "markov_w1"));
    BDR_TRY(need_ptr(w2, "markov_w2"));
  }
  return BDR_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------- no-allocation scratch
// The Markov hand-off workspace of dspark_draft_block_noalloc.  Each device the
// library runs on holds its own copy of this array until the process ends (zero
// when the code object is loaded).  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is taken once per device with
// hipGetSymbolAddress (that device current) and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[BDR_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[256];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 256) return fail(BDR_EUNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(BDR_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BDR_OK;
}

// zero-fills n bytes (n % 16 == 0) with vector stores: the hand-off slots and
// counters must start at zero, whatever an earlier call on this device left
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" {

int bdr_abi_version(void) { return 11; }

void bdr_set_markov_poll_timeout_us(double us) { bdr::set_poll_timeout_us(us); }

void bdr_set_markov_forced_time_out(int on) { bdr::set_forced_time_out(on != 0); }

int bdr_set_row_split_override(int ring, int64_t workgroups, int ksplit) {
  if (ring < 0 || workgroups < 0 || ksplit < 0 || workgroups > (int64_t(1) << 20) || ksplit > 256)
    return fail(BDR_EINVAL, "row-split override: ring %d, workgroups %lld, ksplit %d out of range",
                ring, static_cast<long long>(workgroups), ksplit);
  bdr::set_row_split_override(ring, workgroups, ksplit);
  return BDR_OK;
}

const char* bdr_last_error(void) { return g_err; }

// ---------------------------------------------------------------------------- packed weights
size_t bdr_packed_weight_bytes(int64_t rows, int64_t cols) {
  return packed_weight_bytes(rows, cols);
}

int bdr_pack_weight(const void* w, int64_t rows, int64_t cols, void* packed, void* stream) {
  const size_t bytes = packed_weight_bytes(rows, cols);
  if (bytes == 0)
    return fail(BDR_EUNSUPPORTED, "weight [%lld, %lld] cannot be packed (cols %% 8 == 0 and a "
                "packed copy under 2^31 bytes are required)", static_cast<long long>(rows),
                static_cast<long long>(cols));
  BDR_TRY(need_ptr(w, "w"));
  BDR_TRY(need_ptr(packed, "packed"));
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(w), p0 = reinterpret_cast<uintptr_t>(packed);
  const uintptr_t wbytes = static_cast<uintptr_t>(rows) * static_cast<uintptr_t>(cols) * 2;
  if (w0 < p0 + bytes && p0 < w0 + wbytes) return fail(BDR_EINVAL, "packed overlaps w");
  BDR_TRY(check_device());
  const hipError_t e = launch_pack_weight(w, rows, cols, packed, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "bdr_pack_weight launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S1
size_t dflash_fuse_fc_workspace_bytes(int64_t rows, int64_t hidden, int n_taps, bdr_dtype dt) {
  if (fc_shape(rows, hidden, n_taps, dt) != BDR_OK || rows == 0) return 0;
  return plan_gemm(rows, hidden, hidden * n_taps, dt, true, n_taps).workspace;
}

int dflash_fuse_fc(const void* const* taps, int n_taps, int64_t rows, int64_t hidden,
                   bdr_dtype dt, const void* fc_w, void* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  BDR_TRY(fc_shape(rows, hidden, n_taps, dt));
  if (rows == 0) return BDR_OK;
  if (!taps) return fail(BDR_EINVAL, "taps must not be NULL");
  for (int t = 0; t < n_taps; ++t) {
    if (!taps[t]) return fail(BDR_EINVAL, "taps[%d] must not be NULL", t);
    if (!aligned(taps[t], 16)) return fail(BDR_EINVAL, "taps[%d] must be 16-byte aligned", t);
  }
  BDR_TRY(need_ptr(fc_w, "fc_w"));
  BDR_TRY(need_ptr(out, "out"));
  const GemmPlan p = plan_gemm(rows, hidden, hidden * n_taps, dt, true, n_taps);
  BDR_TRY(need_ws(workspace, workspace_bytes, p.workspace));
  BDR_TRY(check_device());
  hipError_t e = launch_gemm(p, dt, taps, n_taps, hidden, rows, hidden, fc_w, out,
                             act_dtype(dt) == BDR_BF16 ? OUT_BF16 : OUT_F32, workspace,
                             as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dflash_fuse_fc launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S1 + S2 in one launch
namespace {
// the pair plan when both GEMMs take it (bf16, row-split shapes), else !ok
PairPlan fc_lm_pair(int64_t rows, int64_t hidden, int n_taps, int64_t lm_rows, int64_t vocab,
                    bdr_dtype dt) {
  if (act_dtype(dt) != BDR_BF16 || rows == 0 || lm_rows == 0) return PairPlan{};
  return plan_gemm_pair(lm_rows, vocab, hidden, rows, hidden, hidden * n_taps, n_taps,
                        dt == BDR_BF16_PACKED);
}
}  // namespace

size_t dflash_fuse_fc_lm_head_workspace_bytes(int64_t rows, int64_t hidden, int n_taps,
                                              int64_t lm_rows, int64_t vocab, bdr_dtype dt) {
  if (fc_shape(rows, hidden, n_taps, dt) != BDR_OK ||
      lm_shape(lm_rows, hidden, vocab, dt) != BDR_OK)
    return 0;
  const PairPlan pp = fc_lm_pair(rows, hidden, n_taps, lm_rows, vocab, dt);
  if (pp.ok) return pp.workspace;
  return rows == 0 ? 0 : plan_gemm(rows, hidden, hidden * n_taps, dt, true, n_taps).workspace;
}

int dflash_fuse_fc_lm_head(const void* const* taps, int n_taps, int64_t rows, int64_t hidden,
                           bdr_dtype dt, const void* fc_w, void* fc_out, const void* lm_hidden,
                           int64_t lm_rows, int64_t vocab, const void* lm_head_w, float* logits,
                           void* workspace, size_t workspace_bytes, void* stream) {
  BDR_TRY(fc_shape(rows, hidden, n_taps, dt));
  BDR_TRY(lm_shape(lm_rows, hidden, vocab, dt));
  if (rows > 0) {
    if (!taps) return fail(BDR_EINVAL, "taps must not be NULL");
    for (int t = 0; t < n_taps; ++t) {
      if (!taps[t]) return fail(BDR_EINVAL, "taps[%d] must not be NULL", t);
      if (!aligned(taps[t], 16)) return fail(BDR_EINVAL, "taps[%d] must be 16-byte aligned", t);
    }
    BDR_TRY(need_ptr(fc_w, "fc_w"));
    BDR_TRY(need_ptr(fc_out, "fc_out"));
  }
  if (lm_rows > 0) {
    BDR_TRY(need_ptr(lm_hidden, "lm_hidden"));
    BDR_TRY(need_ptr(lm_head_w, "lm_head_w"));
    BDR_TRY(need_ptr(logits, "logits"));
  }
  if (rows == 0 && lm_rows == 0) return BDR_OK;
  const PairPlan pp = fc_lm_pair(rows, hidden, n_taps, lm_rows, vocab, dt);
  const GemmPlan pf = rows > 0 && !pp.ok ? plan_gemm(rows, hidden, hidden * n_taps, dt, true, n_taps)
                                         : GemmPlan{};
  BDR_TRY(need_ws(workspace, workspace_bytes, pp.ok ? pp.workspace : pf.workspace));
  BDR_TRY(check_device());
  const hipStream_t st = as_stream(stream);
  hipError_t e;
  if (pp.ok) {
    e = launch_gemm_pair(pp, lm_hidden, lm_head_w, logits, taps, n_taps, hidden, fc_w, fc_out,
                         workspace, dt == BDR_BF16_PACKED, st);
    if (e != hipSuccess) return hip_fail(e, "dflash_fuse_fc_lm_head launch");
    return BDR_OK;
  }
  if (rows > 0) {
    e = launch_gemm(pf, dt, taps, n_taps, hidden, rows, hidden, fc_w, fc_out,
                    act_dtype(dt) == BDR_BF16 ? OUT_BF16 : OUT_F32, workspace, st);
    if (e != hipSuccess) return hip_fail(e, "dflash_fuse_fc_lm_head fc launch");
  }
  if (lm_rows > 0) {
    const GemmPlan pl = plan_gemm(lm_rows, vocab, hidden, dt, false);
    const void* a[1] = {lm_hidden};
    e = launch_gemm(pl, dt, a, 1, hidden, lm_rows, vocab, lm_head_w, logits, OUT_F32, nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "dflash_fuse_fc_lm_head LM-head launch");
  }
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S2
int dspark_lm_head(const void* hidden, int64_t rows, int64_t hidden_size, int64_t vocab,
                   bdr_dtype dt, const void* lm_head_w, float* logits, void* stream) {
  BDR_TRY(lm_shape(rows, hidden_size, vocab, dt));
  if (rows == 0) return BDR_OK;
  BDR_TRY(need_ptr(hidden, "hidden"));
  BDR_TRY(need_ptr(lm_head_w, "lm_head_w"));
  BDR_TRY(need_ptr(logits, "logits"));
  BDR_TRY(check_device());
  const GemmPlan p = plan_gemm(rows, vocab, hidden_size, dt, false);
  const void* a[1] = {hidden};
  hipError_t e = launch_gemm(p, dt, a, 1, hidden_size, rows, vocab, lm_head_w, logits, OUT_F32,
                             nullptr, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dspark_lm_head launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S1 taps: hc average
int dflash_hc_average(const void* const* captured, int n_taps, int hc, int64_t rows,
                      int64_t hidden, int64_t stream_stride, int64_t row_stride, bdr_dtype dt,
                      void* const* taps_out, void* stream) {
  if (!valid_dtype(dt)) return fail(BDR_EINVAL, "unknown dtype %d", dt);
  if (n_taps < 1) return fail(BDR_EINVAL, "n_taps must be >= 1, got %d", n_taps);
  if (n_taps > BDR_MAX_TAPS) return fail(BDR_EUNSUPPORTED, "n_taps %d > %d", n_taps, BDR_MAX_TAPS);
  if (hc < 1) return fail(BDR_EINVAL, "hc must be >= 1, got %d", hc);
  if (hc > BDR_MAX_HC) return fail(BDR_EUNSUPPORTED, "hc %d > %d", hc, BDR_MAX_HC);
  if (rows < 0) return fail(BDR_EINVAL, "rows must be >= 0");
  if (hidden <= 0) return fail(BDR_EINVAL, "hidden must be > 0");
  if (hidden % 8) return fail(BDR_EUNSUPPORTED, "hidden must be a multiple of 8");
  if (stream_stride < 0 || row_stride < hidden || stream_stride % 8 || row_stride % 8)
    return fail(BDR_EINVAL, "strides must be multiples of 8 elements, row_stride >= hidden, "
                "stream_stride >= 0");
  if (rows > kMaxElems / hidden || rows > kMaxElems / row_stride || hc > kMaxElems / (stream_stride + 1))
    return fail(BDR_EUNSUPPORTED, "problem too large");
  if (rows == 0) return BDR_OK;
  if (!captured || !taps_out) return fail(BDR_EINVAL, "captured and taps_out must not be NULL");
  for (int t = 0; t < n_taps; ++t) {
    if (!captured[t] || !taps_out[t]) return fail(BDR_EINVAL, "tap %d pointer is NULL", t);
    if (!aligned(captured[t], 16) || !aligned(taps_out[t], 16))
      return fail(BDR_EINVAL, "tap %d pointers must be 16-byte aligned", t);
  }
  BDR_TRY(check_device());
  hipError_t e = launch_hc_average(captured, taps_out, n_taps, hc, rows, hidden, stream_stride,
                                   row_stride, dt, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dflash_hc_average launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S1/S2, fp8 weights
namespace {

// bf16 activations [rows, H] read against E4M3 weights [N, K] with K = n_seg * H
int fp8_shape(int64_t rows, int64_t hidden, int n_seg, int64_t n_out) {
  if (n_seg < 1) return fail(BDR_EINVAL, "n_taps must be >= 1, got %d", n_seg);
  if (n_seg > BDR_MAX_TAPS) return fail(BDR_EUNSUPPORTED, "n_taps %d > %d", n_seg, BDR_MAX_TAPS);
  if (rows < 0) return fail(BDR_EINVAL, "rows must be >= 0");
  if (hidden <= 0) return fail(BDR_EINVAL, "hidden must be > 0");
  if (n_out <= 0) return fail(BDR_EINVAL, "output width must be > 0");
  if (n_out > kMaxVocab) return fail(BDR_EUNSUPPORTED, "output width must be < 2^31 - 1");
  if (hidden % 64)
    return fail(BDR_EUNSUPPORTED, "hidden %lld must be a multiple of 64 for fp8 weights",
                static_cast<long long>(hidden));
  // each activation tensor, and the W rows one workgroup streams (<= 192 rows), under 2^31 bytes
  if (rows > kMaxBytes / (hidden * 2) || hidden * n_seg > kMaxBytes / 192 ||
      n_out > kMaxElems / (hidden * n_seg) || rows > kMaxElems / n_out)
    return fail(BDR_EUNSUPPORTED, "problem too large (per-operand byte limit 2^31)");
  return BDR_OK;
}

}  // namespace

size_t dflash_fuse_fc_fp8_workspace_bytes(int64_t rows, int64_t hidden, int n_taps) {
  if (fp8_shape(rows, hidden, n_taps, hidden) != BDR_OK || rows == 0) return 0;
  return plan_gemm_fp8(rows, hidden, hidden * n_taps, true, n_taps).workspace;
}

int dflash_fuse_fc_fp8(const void* const* taps, int n_taps, int64_t rows, int64_t hidden,
                       const uint8_t* fc_q, const float* fc_scale, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  BDR_TRY(fp8_shape(rows, hidden, n_taps, hidden));
  if (rows == 0) return BDR_OK;
  if (!taps) return fail(BDR_EINVAL, "taps must not be NULL");
  for (int t = 0; t < n_taps; ++t) {
    if (!taps[t]) return fail(BDR_EINVAL, "taps[%d] must not be NULL", t);
    if (!aligned(taps[t], 16)) return fail(BDR_EINVAL, "taps[%d] must be 16-byte aligned", t);
  }
  BDR_TRY(need_ptr(fc_q, "fc_q"));
  BDR_TRY(need_ptr(fc_scale, "fc_scale", 4));
  BDR_TRY(need_ptr(out, "out"));
  const GemmPlan p = plan_gemm_fp8(rows, hidden, hidden * n_taps, true, n_taps);
  if (!p.stream) return fail(BDR_EUNSUPPORTED, "fc shape not supported with fp8 weights");
  BDR_TRY(need_ws(workspace, workspace_bytes, p.workspace));
  BDR_TRY(check_device());
  hipError_t e = launch_gemm_fp8(p, taps, n_taps, hidden, rows, hidden, fc_q, fc_scale, out,
                                 OUT_BF16, workspace, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dflash_fuse_fc_fp8 launch");
  return BDR_OK;
}

int dspark_lm_head_fp8(const void* hidden, int64_t rows, int64_t hidden_size, int64_t vocab,
                       const uint8_t* lm_head_q, const float* lm_head_scale, float* logits,
                       void* stream) {
  BDR_TRY(fp8_shape(rows, hidden_size, 1, vocab));
  if (rows == 0) return BDR_OK;
  BDR_TRY(need_ptr(hidden, "hidden"));
  BDR_TRY(need_ptr(lm_head_q, "lm_head_q"));
  BDR_TRY(need_ptr(lm_head_scale, "lm_head_scale", 4));
  BDR_TRY(need_ptr(logits, "logits"));
  const GemmPlan p = plan_gemm_fp8(rows, vocab, hidden_size, false);
  if (!p.stream) return fail(BDR_EUNSUPPORTED, "LM-head shape not supported with fp8 weights");
  BDR_TRY(check_device());
  const void* a[1] = {hidden};
  hipError_t e = launch_gemm_fp8(p, a, 1, hidden_size, rows, vocab, lm_head_q, lm_head_scale,
                                 logits, OUT_F32, nullptr, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dspark_lm_head_fp8 launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S3
size_t dspark_markov_workspace_bytes(int64_t batch, int k) {
  if (batch < 0 || k < 1 || k > BDR_MAX_K) return 0;
  return markov_workspace(batch, k);
}

int dspark_markov_argmax(const float* logits, int64_t batch, int k, int64_t vocab,
                         bdr_dtype wdt, const void* markov_w1, const void* markov_w2, int rank,
                         const int32_t* prev_token, int32_t* draft_tokens, int32_t* status,
                         void* workspace, size_t workspace_bytes, void* stream) {
  BDR_TRY(block_shape(batch, k, vocab));
  BDR_TRY(markov_shape(wdt, markov_w1, markov_w2, rank, vocab, k));
  if (batch == 0) return BDR_OK;
  BDR_TRY(need_ptr(logits, "logits"));
  BDR_TRY(need_ptr(prev_token, "prev_token", 4));
  BDR_TRY(need_ptr(draft_tokens, "draft_tokens", 4));
  if (status) BDR_TRY(need_ptr(status, "status", 4));
  BDR_TRY(need_ws(workspace, workspace_bytes, markov_workspace(batch, k)));
  int cus = 0;
  BDR_TRY(check_device(&cus));
  hipError_t e = launch_markov(logits, batch, k, vocab, wdt, markov_w1, markov_w2, rank,
                               prev_token, draft_tokens, status, workspace, cus,
                               as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dspark_markov_argmax launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S2+S3
size_t dspark_draft_workspace_bytes(int64_t batch, int k, int64_t vocab, int logits_in_workspace) {
  if (batch < 0 || k < 1 || k > BDR_MAX_K || vocab <= 0 || vocab > kMaxVocab) return 0;
  size_t n = markov_workspace(batch, k);
  if (logits_in_workspace) n += align256(static_cast<size_t>(batch) * k * vocab * 4);
  return n;
}

int dspark_draft_block(const void* draft_hidden, int64_t batch, int k, int64_t hidden,
                       int64_t vocab, bdr_dtype dt, const void* lm_head_w, const void* markov_w1,
                       const void* markov_w2, int rank, const int32_t* prev_token,
                       int32_t* draft_tokens, float* logits_out, int32_t* status,
                       void* workspace, size_t workspace_bytes, void* stream) {
  BDR_TRY(block_shape(batch, k, vocab));
  BDR_TRY(lm_shape(batch * k, hidden, vocab, dt));
  BDR_TRY(markov_shape(act_dtype(dt), markov_w1, markov_w2, rank, vocab, k));
  if (batch == 0) return BDR_OK;
  BDR_TRY(need_ptr(draft_hidden, "draft_hidden"));
  BDR_TRY(need_ptr(lm_head_w, "lm_head_w"));
  BDR_TRY(need_ptr(prev_token, "prev_token", 4));
  BDR_TRY(need_ptr(draft_tokens, "draft_tokens", 4));
  if (logits_out) BDR_TRY(need_ptr(logits_out, "logits_out"));
  if (status) BDR_TRY(need_ptr(status, "status", 4));
  const size_t need = dspark_draft_workspace_bytes(batch, k, vocab, logits_out == nullptr);
  BDR_TRY(need_ws(workspace, workspace_bytes, need));
  int cus = 0;
  BDR_TRY(check_device(&cus));
  char* ws = static_cast<char*>(workspace);
  float* logits = logits_out;
  if (!logits) {
    logits = reinterpret_cast<float*>(ws);
    ws += align256(static_cast<size_t>(batch) * k * vocab * 4);
  }
  const GemmPlan p = plan_gemm(batch * k, vocab, hidden, dt, false);
  const void* a[1] = {draft_hidden};
  hipError_t e = launch_gemm(p, dt, a, 1, hidden, batch * k, vocab, lm_head_w, logits, OUT_F32,
                             nullptr, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dspark_draft_block LM-head launch");
  e = launch_markov(logits, batch, k, vocab, act_dtype(dt), markov_w1, markov_w2, rank,
                    prev_token, draft_tokens, status, ws, cus, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dspark_draft_block Markov launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S2+S3, no allocation
int dspark_draft_block_noalloc(const void* draft_hidden, int64_t batch, int k, int64_t hidden,
                               int64_t vocab, bdr_dtype dt, const void* lm_head_w,
                               const void* markov_w1, const void* markov_w2, int rank,
                               const int32_t* prev_token, int32_t* draft_tokens,
                               float* logits_out, int32_t* status, void* stream) {
  BDR_TRY(block_shape(batch, k, vocab));
  BDR_TRY(lm_shape(batch * k, hidden, vocab, dt));
  BDR_TRY(markov_shape(act_dtype(dt), markov_w1, markov_w2, rank, vocab, k));
  const size_t need = markov_workspace(batch, k);
  if (need > BDR_NOALLOC_SCRATCH_BYTES)
    return fail(BDR_EUNSUPPORTED,
                "batch %lld x k %d needs %zu bytes of hand-off scratch; the static scratch "
                "holds %d (batch * k <= 256)", static_cast<long long>(batch), k, need,
                BDR_NOALLOC_SCRATCH_BYTES);
  if (batch == 0) return BDR_OK;
  BDR_TRY(need_ptr(draft_hidden, "draft_hidden"));
  BDR_TRY(need_ptr(lm_head_w, "lm_head_w"));
  BDR_TRY(need_ptr(prev_token, "prev_token", 4));
  BDR_TRY(need_ptr(draft_tokens, "draft_tokens", 4));
  BDR_TRY(need_ptr(logits_out, "logits_out"));
  if (status) BDR_TRY(need_ptr(status, "status", 4));
  int cus = 0;
  BDR_TRY(check_device(&cus));
  void* ws = nullptr;
  BDR_TRY(scratch_address(&ws));
  const GemmPlan p = plan_gemm(batch * k, vocab, hidden, dt, false);
  if (p.workspace != 0) return fail(BDR_EUNSUPPORTED, "LM-head plan needs a workspace");
  const hipStream_t st = as_stream(stream);
  const size_t n16 = need / 16;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<unsigned>(std::min<size_t>((n16 + 255) / 256, 1024))),
                     dim3(256), 0, st, static_cast<uint4*>(ws), n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "dspark_draft_block_noalloc scratch clear");
  const void* a[1] = {draft_hidden};
  e = launch_gemm(p, dt, a, 1, hidden, batch * k, vocab, lm_head_w, logits_out, OUT_F32, nullptr,
                  st);
  if (e != hipSuccess) return hip_fail(e, "dspark_draft_block_noalloc LM-head launch");
  e = launch_markov(logits_out, batch, k, vocab, act_dtype(dt), markov_w1, markov_w2, rank,
                    prev_token, draft_tokens, status, ws, cus, st);
  if (e != hipSuccess) return hip_fail(e, "dspark_draft_block_noalloc Markov launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- S4
size_t spec_verify_workspace_bytes(int64_t batch, int k, int64_t vocab) {
  if (batch < 0 || k < 1 || k > BDR_MAX_K || vocab <= 0 || vocab > kMaxVocab) return 0;
  return verify_workspace(batch, k, vocab);
}

int spec_verify_greedy(const void* target_logits, bdr_dtype dt, int64_t batch, int k,
                       int64_t vocab, const int32_t* draft_tokens, const float* confidence,
                       float threshold, int32_t* block_len, int32_t* accepted, int32_t* bonus,
                       int32_t* target_argmax, int64_t* accept_counts, int64_t* proposed_counts,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dt)) return fail(BDR_EINVAL, "unknown dtype %d", dt);
  BDR_TRY(block_shape(batch, k, vocab));
  if (batch == 0) return BDR_OK;
  BDR_TRY(need_ptr(target_logits, "target_logits"));
  BDR_TRY(need_ptr(draft_tokens, "draft_tokens", 4));
  if (confidence) BDR_TRY(need_ptr(confidence, "confidence", 4));
  BDR_TRY(need_ptr(block_len, "block_len", 4));
  BDR_TRY(need_ptr(accepted, "accepted", 4));
  BDR_TRY(need_ptr(bonus, "bonus", 4));
  if (target_argmax) BDR_TRY(need_ptr(target_argmax, "target_argmax", 4));
  if (accept_counts) BDR_TRY(need_ptr(accept_counts, "accept_counts", 8));
  if (proposed_counts) BDR_TRY(need_ptr(proposed_counts, "proposed_counts", 8));
  BDR_TRY(need_ws(workspace, workspace_bytes, verify_workspace(batch, k, vocab)));
  BDR_TRY(check_device());
  hipError_t e = launch_verify(target_logits, dt, batch, k, vocab, draft_tokens, confidence,
                               threshold, block_len, accepted, bonus, target_argmax,
                               accept_counts, proposed_counts, workspace, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_verify_greedy launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- sampling
int dspark_gumbel_noise(int64_t batch, int k, int64_t vocab, uint64_t seed, int stream_id,
                        float* noise, void* stream) {
  BDR_TRY(block_shape(batch, k, vocab));
  if (vocab > kMaxMarkovVocab) return fail(BDR_EUNSUPPORTED, "vocab must be <= 2^21 here");
  if (stream_id < 0) return fail(BDR_EINVAL, "stream_id must be >= 0");
  if (batch == 0) return BDR_OK;
  BDR_TRY(need_ptr(noise, "noise", 4));
  BDR_TRY(check_device());
  hipError_t e = launch_gumbel_noise(noise, batch, k, vocab, seed,
                                     static_cast<uint32_t>(stream_id), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dspark_gumbel_noise launch");
  return BDR_OK;
}

static int need_temperature(float t) {
  if (!(t > 0.f) || !std::isfinite(t)) return fail(BDR_EINVAL, "temperature must be finite and > 0");
  if (!std::isfinite(1.0f / t)) return fail(BDR_EUNSUPPORTED, "temperature too small");
  return BDR_OK;
}

size_t dspark_markov_sample_workspace_bytes(int64_t batch, int k, int64_t vocab) {
  if (batch < 0 || k < 1 || k > BDR_MAX_K || vocab <= 0 || vocab > kMaxMarkovVocab) return 0;
  return markov_sample_workspace(batch, k, vocab);
}

int dspark_markov_sample(const float* logits, int64_t batch, int k, int64_t vocab,
                         bdr_dtype wdt, const void* markov_w1, const void* markov_w2, int rank,
                         const int32_t* prev_token, float temperature, uint64_t seed,
                         int32_t* draft_tokens, float* draft_logits, const float* confidence,
                         float threshold, int32_t* status, void* workspace,
                         size_t workspace_bytes, void* stream) {
  BDR_TRY(block_shape(batch, k, vocab));
  BDR_TRY(markov_shape(wdt, markov_w1, markov_w2, rank, vocab, k));
  BDR_TRY(need_temperature(temperature));
  if (batch == 0) return BDR_OK;
  BDR_TRY(need_ptr(logits, "logits"));
  BDR_TRY(need_ptr(prev_token, "prev_token", 4));
  BDR_TRY(need_ptr(draft_tokens, "draft_tokens", 4));
  BDR_TRY(need_ptr(draft_logits, "draft_logits"));
  if (confidence) BDR_TRY(need_ptr(confidence, "confidence", 4));
  if (status) BDR_TRY(need_ptr(status, "status", 4));
  BDR_TRY(need_ws(workspace, workspace_bytes, markov_sample_workspace(batch, k, vocab)));
  int cus = 0;
  BDR_TRY(check_device(&cus));
  hipError_t e = launch_markov_sample(logits, batch, k, vocab, wdt, markov_w1, markov_w2, rank,
                                      prev_token, 1.0f / temperature, seed, draft_tokens,
                                      draft_logits, confidence, threshold, status, workspace, cus,
                                      as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dspark_markov_sample launch");
  return BDR_OK;
}

size_t spec_verify_sample_workspace_bytes(int64_t batch, int k, int64_t vocab) {
  if (batch < 0 || k < 1 || k > BDR_MAX_K || vocab <= 0 || vocab > kMaxVocab) return 0;
  return sample_verify_workspace(batch, k, vocab);
}

int spec_verify_sample(const void* target_logits, bdr_dtype dt, int64_t batch, int k,
                       int64_t vocab, const int32_t* draft_tokens, const float* draft_logits,
                       const float* confidence, float threshold, float temperature, uint64_t seed,
                       int32_t* block_len, int32_t* accepted, int32_t* bonus,
                       int64_t* accept_counts, int64_t* proposed_counts, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dt)) return fail(BDR_EINVAL, "unknown dtype %d", dt);
  BDR_TRY(block_shape(batch, k, vocab));
  BDR_TRY(need_temperature(temperature));
  if (batch == 0) return BDR_OK;
  BDR_TRY(need_ptr(target_logits, "target_logits"));
  BDR_TRY(need_ptr(draft_tokens, "draft_tokens", 4));
  BDR_TRY(need_ptr(draft_logits, "draft_logits"));
  if (confidence) BDR_TRY(need_ptr(confidence, "confidence", 4));
  BDR_TRY(need_ptr(block_len, "block_len", 4));
  BDR_TRY(need_ptr(accepted, "accepted", 4));
  BDR_TRY(need_ptr(bonus, "bonus", 4));
  if (accept_counts) BDR_TRY(need_ptr(accept_counts, "accept_counts", 8));
  if (proposed_counts) BDR_TRY(need_ptr(proposed_counts, "proposed_counts", 8));
  BDR_TRY(need_ws(workspace, workspace_bytes, sample_verify_workspace(batch, k, vocab)));
  BDR_TRY(check_device());
  hipError_t e = launch_verify_sample(target_logits, dt, batch, k, vocab, draft_tokens,
                                      draft_logits, confidence, threshold, 1.0f / temperature,
                                      seed, block_len, accepted, bonus, accept_counts,
                                      proposed_counts, workspace, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_verify_sample launch");
  return BDR_OK;
}

// ---------------------------------------------------------------------------- loop
int spec_commit(const int32_t* draft_tokens, const int32_t* accepted, const int32_t* bonus,
                const int32_t* block_len, int64_t batch, int k, int32_t* next_prev,
                int32_t* emitted, int32_t* draft_list, int32_t* row_index, int32_t* row_count,
                int32_t* row_offsets, void* stream) {
  if (batch < 0) return fail(BDR_EINVAL, "batch must be >= 0");
  if (k < 1) return fail(BDR_EINVAL, "k must be >= 1, got %d", k);
  if (k > BDR_MAX_K) return fail(BDR_EUNSUPPORTED, "k %d > %d", k, BDR_MAX_K);
  if (batch > 0x7FFFFFFFLL / (k + 1)) return fail(BDR_EUNSUPPORTED, "batch too large");
  if (batch == 0) return BDR_OK;
  BDR_TRY(need_ptr(draft_tokens, "draft_tokens", 4));
  BDR_TRY(need_ptr(accepted, "accepted", 4));
  BDR_TRY(need_ptr(bonus, "bonus", 4));
  if (block_len) BDR_TRY(need_ptr(block_len, "block_len", 4));
  BDR_TRY(need_ptr(next_prev, "next_prev", 4));
  for (const int32_t* p : {static_cast<const int32_t*>(emitted), static_cast<const int32_t*>(draft_list),
                           static_cast<const int32_t*>(row_index), static_cast<const int32_t*>(row_count),
                           static_cast<const int32_t*>(row_offsets)})
    if (p) BDR_TRY(need_ptr(p, "output", 4));
  BDR_TRY(check_device());
  hipError_t e = launch_commit(draft_tokens, accepted, bonus, block_len, batch, k, next_prev,
                               emitted, draft_list, row_index, row_count, row_offsets,
                               as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "spec_commit launch");
  return BDR_OK;
}

size_t dflash_fuse_fc_rows_workspace_bytes(int64_t max_rows, int64_t hidden, int n_taps,
                                           bdr_dtype dt) {
  if (fc_shape(max_rows, hidden, n_taps, dt) != BDR_OK) return 0;
  return fc_rows_workspace(max_rows, hidden, n_taps, dt);
}

int dflash_fuse_fc_rows(const void* const* taps, int n_taps, int64_t rows, int64_t hidden,
                        bdr_dtype dt, const int32_t* row_index, const int32_t* row_count,
                        int64_t max_rows, const void* fc_w, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  BDR_TRY(fc_shape(max_rows, hidden, n_taps, dt));
  BDR_TRY(fc_shape(rows, hidden, n_taps, dt));
  if (max_rows == 0) return BDR_OK;
  if (!taps) return fail(BDR_EINVAL, "taps must not be NULL");
  for (int t = 0; t < n_taps; ++t) {
    if (rows > 0 && !taps[t]) return fail(BDR_EINVAL, "taps[%d] must not be NULL", t);
    if (!aligned(taps[t], 16)) return fail(BDR_EINVAL, "taps[%d] must be 16-byte aligned", t);
  }
  BDR_TRY(need_ptr(row_index, "row_index", 4));
  BDR_TRY(need_ptr(row_count, "row_count", 4));
  BDR_TRY(need_ptr(fc_w, "fc_w"));
  BDR_TRY(need_ptr(out, "out"));
  BDR_TRY(need_ws(workspace, workspace_bytes, fc_rows_workspace(max_rows, hidden, n_taps, dt)));
  BDR_TRY(check_device());
  hipError_t e = launch_fc_rows(taps, n_taps, rows, hidden, dt, row_index, row_count, max_rows,
                                fc_w, out, workspace, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dflash_fuse_fc_rows launch");
  return BDR_OK;
}

size_t dflash_fuse_fc_rows_fp8_workspace_bytes(int64_t max_rows, int64_t hidden, int n_taps) {
  if (fp8_shape(max_rows, hidden, n_taps, hidden) != BDR_OK) return 0;
  return fc_rows_fp8_workspace(max_rows, hidden, n_taps);
}

int dflash_fuse_fc_rows_fp8(const void* const* taps, int n_taps, int64_t rows, int64_t hidden,
                            const int32_t* row_index, const int32_t* row_count, int64_t max_rows,
                            const uint8_t* fc_q, const float* fc_scale, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  BDR_TRY(fp8_shape(max_rows, hidden, n_taps, hidden));
  BDR_TRY(fp8_shape(rows, hidden, n_taps, hidden));
  if (max_rows == 0) return BDR_OK;
  if (!taps) return fail(BDR_EINVAL, "taps must not be NULL");
  for (int t = 0; t < n_taps; ++t) {
    if (rows > 0 && !taps[t]) return fail(BDR_EINVAL, "taps[%d] must not be NULL", t);
    if (!aligned(taps[t], 16)) return fail(BDR_EINVAL, "taps[%d] must be 16-byte aligned", t);
  }
  BDR_TRY(need_ptr(row_index, "row_index", 4));
  BDR_TRY(need_ptr(row_count, "row_count", 4));
  BDR_TRY(need_ptr(fc_q, "fc_q"));
  BDR_TRY(need_ptr(fc_scale, "fc_scale", 4));
  BDR_TRY(need_ptr(out, "out"));
  if (!plan_gemm_fp8(max_rows, hidden, hidden * n_taps, true, n_taps).stream)
    return fail(BDR_EUNSUPPORTED, "fc shape not supported with fp8 weights");
  BDR_TRY(need_ws(workspace, workspace_bytes, fc_rows_fp8_workspace(max_rows, hidden, n_taps)));
  BDR_TRY(check_device());
  hipError_t e = launch_fc_rows_fp8(taps, n_taps, rows, hidden, row_index, row_count, max_rows,
                                    fc_q, fc_scale, out, workspace, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "dflash_fuse_fc_rows_fp8 launch");
  return BDR_OK;
}

}  // extern "C"
