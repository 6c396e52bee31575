// pa_reshape_and_decode_static: the one-call decode step with its split-K
// partials in a library-owned device array instead of a caller workspace,
// for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In host
// code `scratch` names only a host-side stand-in, so its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever passed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pagedattn.h"

namespace {

constexpr size_t kScratchBytes = PA_STATIC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];  // device address of `scratch` on device d (null: lookup failed)

// Device address of the current device's copy of `scratch`.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = e == hipSuccess ? p : nullptr;
  });
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int pa_reshape_and_decode_static(void* out, const void* q, const void* key, const void* value,
                                 void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, float scale, int32_t dtype,
                                 int32_t partition_size, int32_t max_context_len, void* stream) {
  void* ws = scratch_address();
  if (ws == nullptr) return PA_ERR_LAUNCH;
  // The step's checks run before any launch; with a workspace always given,
  // PA_ERR_WORKSPACE can only mean that the partials need more bytes than
  // the array holds.
  const int rc = pa_reshape_and_decode(out, q, key, value, k_cache, v_cache, slot_mapping,
                                       block_tables, context_lens, num_seqs, num_q_heads,
                                       num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                       num_blocks, scale, dtype, partition_size, max_context_len,
                                       ws, kScratchBytes, stream);
  return rc == PA_ERR_WORKSPACE ? PA_ERR_SCRATCH : rc;
}

}  // extern "C"
