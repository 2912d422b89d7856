// tara_attn_fwd_noalloc: tara_attn_fwd without a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation). The workspace lives in a
// fixed device array of this library, `scratch`, TARA_NOALLOC_SCRATCH_BYTES
// long; each device the library runs on holds its own copy until the process
// ends. The call is split into sub-calls of one batch element and as many
// heads as that array holds, enqueued in order on the caller's stream with the
// same kernels as tara_attn_fwd, so the outputs are the same.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "tara.h"
#include "tara_internal.h"

namespace {

constexpr size_t kScratchBytes = TARA_NOALLOC_SCRATCH_BYTES;

// The workspace of every no-alloc call on a device. In host code this name is
// only a stand-in for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for it (scratch_ptr), never the name itself.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // address of scratch on each device, once looked up

// The address of scratch on the current device (looked up once per device,
// with that device current).
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return tara::set_error(TARA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return tara::set_error(TARA_ERR_HIP, "device index " + std::to_string(dev) + " beyond the library's 64");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return tara::set_error(TARA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TARA_OK;
}

}  // namespace

extern "C" int tara_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int dtype, int B, int H, int N, int D, const int64_t q_str[3],
                                     const int64_t k_str[3], const int64_t v_str[3], const int64_t o_str[3],
                                     const uint8_t* seg_type, const float* token_time, const int16_t* picture_id,
                                     const float* mask_weight, const tara_params_t* p, tara_stream_t stream_) {
  tara::set_error(TARA_OK, "");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  tara::Call c{};
  if (int st = tara::make_call(c, q, k, v, o, lse, dtype, B, H, N, D, q_str, k_str, v_str, o_str, seg_type,
                               token_time, picture_id, mask_weight, p))
    return st;
  if (B == 0 || H == 0 || N == 0) {
    tara::set_empty_info(c);
    return TARA_OK;
  }
  // the largest group of heads whose workspace fits, for a full group and for
  // the last, smaller one (the workspace need not grow with the head count: a
  // fused call's tail split depends on it)
  auto fits = [&](int heads) { return tara::call_workspace(tara::sub_call(c, 0, 0, heads)) <= kScratchBytes; };
  int hc = 0;
  for (int g = H; g >= 1 && hc == 0; --g)
    if (fits(g) && (H % g == 0 || fits(H % g))) hc = g;
  if (hc == 0)
    return tara::set_error(TARA_ERR_WORKSPACE,
                           "the no-alloc entry point holds " + std::to_string(kScratchBytes) +
                               " bytes of workspace; one head of this call needs " +
                               std::to_string(tara::call_workspace(tara::sub_call(c, 0, 0, 1))) +
                               " (use tara_attn_fwd with a caller workspace)");
  void* ws = nullptr;
  if (int st = scratch_ptr(&ws)) return st;
  tara_run_info_t info{}, sub{};
  for (int b = 0; b < B; ++b)
    for (int h0 = 0; h0 < H; h0 += hc) {
      // the first group of a batch element encodes its metadata; the others reuse it
      const tara::Call s = tara::sub_call(c, b, h0, std::min(hc, H - h0));
      if (tara::call_workspace(s) > kScratchBytes)   // guarded by the choice of hc above
        return tara::set_error(TARA_ERR_WORKSPACE, "internal: a group of heads outgrew the no-alloc array");
      if (int st = tara::enqueue_call(s, static_cast<char*>(ws), h0 == 0, false, stream, &sub)) return st;
      const int grid = info.grid + sub.grid, launches = info.launches + sub.launches;
      info = sub;
      info.grid = grid;
      info.launches = launches;
    }
  tara::set_last_info(info);
  return TARA_OK;
}
