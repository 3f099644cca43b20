// Allocation-free variant of the NoPE attention call, for callers that cannot
// allocate (or pass) a workspace: code under graph capture, tight serving
// loops. Its split-K records and counters live in one file-scope device
// array per GPU of kStaticScratchBytes, found once per device with
// hipGetSymbolAddress; every call on a GPU uses that GPU's copy, so calls that
// overlap on one GPU race (order them on one stream).
#include <mutex>

#include "common.h"
#include "internal.h"

namespace beam {

constexpr size_t kStaticScratchBytes = size_t(16) << 20;  // 16 MiB per GPU

// Device memory of this array is reached only through the address that
// hipGetSymbolAddress returns for the current device (static_scratch).
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

// The array's address on the current device, looked up on the first call
// made with that device current.
static int static_scratch(void** out, const char* fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return abi_fail(BEAM_E_NODEV, "%s: no current HIP device", fn);
  if (dev >= kMaxDevices)
    return abi_fail(BEAM_E_UNSUPPORTED, "%s: device index %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return abi_fail(BEAM_E_HIP, "%s: hipGetSymbolAddress of the scratch array: %s", fn,
                      hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BEAM_OK;
}

}  // namespace beam

extern "C" int beam_attn_nope_ssmax_static(const beam_dims* dims, int T, const uint16_t* q,
                                           const int32_t* pos, const int32_t* seq,
                                           const beam_kv* kv, const float* sink, uint16_t* o,
                                           int max_pos, void* stream) {
  using namespace beam;
  if (!dims) return abi_fail(BEAM_E_NULL, "%s: dims is NULL", __func__);
  if (T <= 0) return abi_fail(BEAM_E_SHAPE, "%s: T <= 0", __func__);
  if (max_pos < 0) return abi_fail(BEAM_E_SHAPE, "%s: max_pos < 0", __func__);
  if (kv && kv->npos > kv->Lmax)
    return abi_fail(BEAM_E_UNSUPPORTED, "%s: a ring cache serves sliding-window attention only",
                    __func__);
  const size_t need = beam_workspace_size(dims, BEAM_OP_ATTN_NOPE, T, max_pos + 1);
  if (need == (size_t)-1) return abi_fail(BEAM_E_SHAPE, "%s: invalid dims", __func__);
  if (need > kStaticScratchBytes)
    return abi_fail(BEAM_E_WORKSPACE,
                    "%s: T = %d tokens up to position %d need %zu bytes of scratch, more than "
                    "the %zu of the static array (use beam_attn_nope_ssmax with a workspace)",
                    __func__, T, max_pos, need, kStaticScratchBytes);
  void* ws = nullptr;
  const int rc = static_scratch(&ws, __func__);
  if (rc) return rc;
  return attn_entry(dims, T, q, pos, seq, kv, sink, o, max_pos, ws, kStaticScratchBytes, stream,
                    0, true, __func__);
}
