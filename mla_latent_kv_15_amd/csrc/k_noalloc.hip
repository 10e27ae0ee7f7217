// mla_decode without a caller workspace, for callers that cannot allocate
// device memory: the step's scratch is one fixed device array per GPU.
//
// `scratch` below is a device variable.  In host code its name is only a
// host-side stand-in, never a device address: host code reaches the array
// through the address hipGetSymbolAddress returns for the current device,
// looked up once per device and kept in g_ptr.
#include <mutex>

#include "mla_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` on each GPU

// the array's device address on the current device (looked up on first use)
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLA_ERR_HIP;
  if (dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" int mla_decode_noalloc(const mla_config* cfg, const mla_weights* w, const void* h,
                                  const int32_t* positions, const void* kv_cache, int num_pages,
                                  const int32_t* page_table, int max_pages,
                                  const int32_t* kv_lens, int B, int max_kv_len,
                                  const float* rope_table, int rope_len, int num_splits,
                                  void* out, void* stream) {
  size_t need = 0;
  int r = mla::decode_args_status(cfg, w, h, positions, kv_cache, num_pages, page_table,
                                  max_pages, kv_lens, B, max_kv_len, rope_table, rope_len,
                                  num_splits, out, &need);
  if (r || B == 0) return r;
  if (need > kScratchBytes) return MLA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  r = scratch_on_current_device(&ws);
  if (r) return r;
  return mla_decode(cfg, w, h, positions, kv_cache, num_pages, page_table, max_pages, kv_lens, B,
                    max_kv_len, rope_table, rope_len, num_splits, ws, kScratchBytes, out, stream);
}
