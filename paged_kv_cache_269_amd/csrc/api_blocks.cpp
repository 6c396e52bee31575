// C-ABI host layer of the block operations: copy-on-write copies inside the
// pool and swaps between caches.  Declarations and the meaning of every
// argument: include/pagedattn.h.
#include "pagedattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "launch.h"

namespace {

constexpr int kMaxGridYZ = 65535;

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
  }
}

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

// The address a kernel uses for `p`: device memory as is, pinned host
// memory through its device mapping.  Pageable host memory (or anything the
// runtime does not know) has none: nullptr.
const void* device_view(const void* p) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error this query leaves behind
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return p;
  if (attr.type == hipMemoryTypeHost) {
    void* dev = nullptr;  // the mapping of this very address (offsets into the allocation kept)
    if (hipHostGetDevicePointer(&dev, const_cast<void*>(p), 0) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return dev;
  }
  return nullptr;
}

}  // namespace

extern "C" {

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   int32_t dtype, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb || !(block_size == 8 || block_size == 16 || block_size == 32) || !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_pairs > kMaxGridYZ || num_kv_heads <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return PA_ERR_NULL;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * eb;
  hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, block_pairs, num_pairs, block_bytes,
                                        num_blocks, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_swap_blocks(const void* src_cache, void* dst_cache, const int64_t* block_pairs,
                   int32_t num_pairs, int64_t block_bytes, void* stream) {
  if (num_pairs < 0 || block_bytes <= 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!src_cache || !dst_cache || !block_pairs) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_pairs; ++i)
    if (block_pairs[2 * i] < 0 || block_pairs[2 * i + 1] < 0) return PA_ERR_RANGE;
  const char* src = static_cast<const char*>(src_cache);
  char* dst = static_cast<char*>(dst_cache);
  // Runs of pairs whose source and destination blocks both advance by one
  // move as one copy.
  for (int32_t i = 0; i < num_pairs;) {
    int32_t j = i + 1;
    while (j < num_pairs && block_pairs[2 * j] == block_pairs[2 * (j - 1)] + 1 &&
           block_pairs[2 * j + 1] == block_pairs[2 * (j - 1) + 1] + 1)
      ++j;
    const hipError_t e = hipMemcpyAsync(dst + block_pairs[2 * i + 1] * block_bytes,
                                        src + block_pairs[2 * i] * block_bytes,
                                        (size_t)(j - i) * block_bytes, hipMemcpyDefault,
                                        (hipStream_t)stream);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
    i = j;
  }
  return PA_OK;
}

int pa_swap_blocks_mapped(const void* src_cache, void* dst_cache, const int64_t* block_pairs,
                          int32_t num_pairs, int64_t block_bytes, int64_t src_blocks,
                          int64_t dst_blocks, void* stream) {
  if (num_pairs < 0 || num_pairs > kMaxGridYZ || block_bytes <= 0 || block_bytes % 16 ||
      src_blocks <= 0 || dst_blocks <= 0)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!src_cache || !dst_cache || !block_pairs) return PA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src_cache) | reinterpret_cast<uintptr_t>(dst_cache)) % 16)
    return PA_ERR_UNSUPPORTED;
  const void* src = device_view(src_cache);
  void* dst = const_cast<void*>(device_view(dst_cache));
  const int64_t* pairs = static_cast<const int64_t*>(device_view(block_pairs));
  if (!src || !dst || !pairs) return PA_ERR_UNSUPPORTED;  // not reachable from the device
  hipError_t e = pa::launch_swap_blocks(src, dst, pairs, num_pairs, block_bytes, src_blocks,
                                        dst_blocks, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_validate_copy_host(const int32_t* block_pairs, int32_t num_pairs, int64_t num_blocks) {
  if (num_pairs < 0 || num_blocks < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!block_pairs) return PA_ERR_NULL;
  std::vector<int32_t> dst(num_pairs), src(num_pairs);
  for (int32_t i = 0; i < num_pairs; ++i) {
    src[i] = block_pairs[2 * i];
    dst[i] = block_pairs[2 * i + 1];
    if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks)
      return PA_ERR_RANGE;
  }
  std::sort(dst.begin(), dst.end());
  if (std::adjacent_find(dst.begin(), dst.end()) != dst.end()) return PA_ERR_RANGE;
  for (int32_t s : src)
    if (std::binary_search(dst.begin(), dst.end(), s)) return PA_ERR_RANGE;
  return PA_OK;
}

}  // extern "C"
