// Decode attention for callers that cannot allocate device memory: the partial records
// of the split live in a fixed device array of this library instead of a caller's
// workspace.  Same kernels and results as lvq_decode_attn.
#include <atomic>

#include "lvq_internal.h"

namespace {

constexpr size_t kScratchBytes = lvq::kNoAllocScratchBytes;

// The scratch array.  Each device the library runs on holds its own copy (at its own
// address) until the process ends.  In host code this name is not a device address:
// host code only ever uses the address hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[64];

// Device address of the current device's scratch array, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" int lvq_decode_attn_noalloc(const uint16_t* q, const int32_t* page_table,
                                       const uint8_t* index_pages, const uint16_t* bf16_pages,
                                       const int32_t* bf16_table, const uint16_t* codebooks, int t,
                                       const int32_t* pos, const int32_t* seq_len, const int32_t* q_end,
                                       const float* rope_tab, const lvq_attn_shape* shp, float* out,
                                       float* lse, void* stream) {
  // an invalid shape reports 0 bytes here and is refused by lvq_decode_attn's checks
  const size_t need = lvq_decode_attn_workspace_bytes(shp);
  if (need > kScratchBytes)
    return lvq::set_error(LVQ_ENOSPC, "lvq_decode_attn_noalloc: this shape needs %zu bytes of partial "
                                      "records, beyond the library's fixed %zu-byte scratch array",
                          need, kScratchBytes);
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess)
    return lvq::set_error(LVQ_EDEVICE, "lvq_decode_attn_noalloc: scratch address: %s", hipGetErrorString(e));
  return lvq_decode_attn(q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos, seq_len,
                         q_end, rope_tab, shp, out, lse, ws, kScratchBytes, stream);
}
