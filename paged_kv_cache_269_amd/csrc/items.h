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

}  // namespace pa
