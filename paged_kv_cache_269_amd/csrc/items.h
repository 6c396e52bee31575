// Decode work items: (head unit, sequence, partition).
#pragma once

#include "common.h"
#include "launch.h"

namespace pa {

// Context length of sequence s, clamped to [0, max_len] like every kernel does.
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int s) {
  const int L = a.context_lens[s];
  return L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
}

// Partitions of a context of L tokens; an empty context still has one item,
// which writes its zero row.
__device__ __forceinline__ int parts_of(int L, int part_blocks) {
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int P = (nb + part_blocks - 1) / part_blocks;
  return P > 0 ? P : 1;
}

// Host: compute units of the current device (cached per device; <= 0 on a
// runtime error).
inline int compute_units() {
  static int per_device[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cacheable = dev >= 0 && dev < 64;
  int cus = cacheable ? __atomic_load_n(&per_device[dev], __ATOMIC_RELAXED) : 0;
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return -1;
    if (cacheable && cus > 0) __atomic_store_n(&per_device[dev], cus, __ATOMIC_RELAXED);
  }
  return cus;
}

// Host: workgroups of `kernel` (block of `threads`) resident on the current
// device at once, cached per device.  Returns <= 0 on a runtime error.
struct ResidentCache {
  int per_device[64] = {};
};

inline int resident_workgroups(const void* kernel, int threads, ResidentCache& c) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cacheable = dev >= 0 && dev < 64;
  int resident = cacheable ? __atomic_load_n(&c.per_device[dev], __ATOMIC_RELAXED) : 0;
  if (resident <= 0) {
    int per_cu = 0;
    const int cus = compute_units();
    if (cus <= 0 ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
      return -1;
    resident = per_cu * cus;
    if (cacheable && resident > 0) __atomic_store_n(&c.per_device[dev], resident, __ATOMIC_RELAXED);
  }
  return resident;
}

}  // namespace pa
