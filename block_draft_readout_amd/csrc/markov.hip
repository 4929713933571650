// Host side of the DSpark Markov-biased semi-autoregressive argmax: workspace
// layout and dispatch to the chain or per-position schedule.

#include <atomic>
#include <cmath>

#include "markov_kernels.h"

namespace bdr {

// How long a poll of the persistent chain waits for the other workgroups before
// giving up (the whole chain normally takes tens of microseconds).
constexpr double kDefaultPollTimeoutUs = 50000.0;
static std::atomic<double> g_poll_timeout_us{kDefaultPollTimeoutUs};

void set_poll_timeout_us(double us) {
  g_poll_timeout_us.store(std::isfinite(us) && us >= 0.0 ? us : kDefaultPollTimeoutUs);
}

// While set, every bounded wait disregards what it reads and gives up when its
// limit passes, so the time-out path runs whatever the workgroups' timing.
static std::atomic<unsigned> g_forced_time_out{0u};

void set_forced_time_out(bool on) { g_forced_time_out.store(on ? 1u : 0u); }

// wall-clock ticks of the current device for the poll limit (the device's
// constant-rate counter; its rate in kHz is a device attribute)
static unsigned long long poll_ticks() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    khz = 100000;   // 100 MHz, the gfx9 real-time counter
  return static_cast<unsigned long long>(g_poll_timeout_us.load() * 1e-3 * khz);
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

// keys | slots | tokens | completion counter | error word
static size_t keys_bytes(int64_t B, int k) {
  return align256(static_cast<size_t>(B) * k * kArriveGroups * 8);
}
static size_t slots_bytes(int64_t B, int k) {
  return align256(static_cast<size_t>(B) * k * kChainSlots * kSlotStride * 8);
}
static size_t tokens_bytes(int64_t B, int k) {
  return align256(static_cast<size_t>(B) * k * kTokenStride * 8);
}

size_t markov_workspace(int64_t B, int k) {
  return keys_bytes(B, k) + slots_bytes(B, k) + tokens_bytes(B, k) + 256 + 256;
}

MarkovArgs markov_args(const float* logits, int64_t B, int k, int64_t V, const void* w1,
                       const void* w2, int rank, const int32_t* prev, int32_t* draft,
                       int32_t* status, void* workspace) {
  MarkovArgs g{};
  g.logits = logits;
  g.B = B;
  g.V = V;
  g.k = k;
  g.r = (w1 && w2) ? rank : 0;
  g.w1 = w1;
  g.w2 = w2;
  g.prev = prev;
  char* ws = static_cast<char*>(workspace);
  size_t off = 0;
  g.keys = reinterpret_cast<unsigned long long*>(ws + off);
  off += keys_bytes(B, k);
  g.slots = reinterpret_cast<unsigned long long*>(ws + off);
  off += slots_bytes(B, k);
  g.tokens = reinterpret_cast<unsigned long long*>(ws + off);
  off += tokens_bytes(B, k);
  g.done = reinterpret_cast<unsigned*>(ws + off);
  off += 256;
  g.err = reinterpret_cast<unsigned*>(ws + off);   // the last 256 bytes
  g.status = status;
  g.poll_ticks = poll_ticks();
  g.forced_time_out = g_forced_time_out.load();
  g.draft = draft;
  g.vtiles = (V + 15) / 16;
  return g;
}

hipError_t launch_markov(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                         const void* w1, const void* w2, int rank, const int32_t* prev,
                         int32_t* draft, int32_t* status, void* workspace, int n_cu,
                         hipStream_t stream) {
  const MarkovArgs g = markov_args(logits, B, k, V, w1, w2, rank, prev, draft, status, workspace);
  return markov_dispatch<false>(g, wdt, n_cu, stream);
}

}  // namespace bdr
