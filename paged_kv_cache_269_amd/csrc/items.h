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

// Pool blocks of BS-token blocks that hold 16-token tile j of a sequence
// (tokens 16j .. 16j+15; `bt` is its table row of M entries): one block
// (BS 16), half of one (BS 32: rows 16 (j % 2) ..), or two (BS 8: the tile's
// first 8 rows in block bt[2j], the last 8 in bt[2j+1]).  Every kernel works
// on 16-token tiles; only this mapping and the descriptors below see BS.
template <int BS>
struct TileIds {
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static constexpr int H = BS == 8 ? 2 : 1;  // blocks per tile
  int id[H];
};

// A block-table row read through the constant address space: the table does
// not change during a launch, so the compiler may read it with scalar loads
// even in kernels that also store to global memory (which it could
// otherwise not prove free of aliasing with the table).
typedef const __attribute__((address_space(4))) int32_t* TableRow;
__device__ __forceinline__ TableRow table_row(const int32_t* p) { return (TableRow)p; }

template <int BS, typename Ptr>
__device__ __forceinline__ TileIds<BS> tile_ids(Ptr bt, int j, int M) {
  TileIds<BS> t;
  if constexpr (BS == 16) {
    t.id[0] = bt[j];
  } else if constexpr (BS == 32) {
    t.id[0] = bt[j >> 1];
  } else {
    t.id[0] = bt[2 * j];
    t.id[1] = bt[min(2 * j + 1, M - 1)];  // past the context when clamped: masked
  }
  return t;
}

// Buffer descriptors of one 16-token tile of one KV head in both caches,
// one per block it spans; empty (zero records: loads return zeros, touch
// nothing) for a tile past the item's end or a block id outside the pool.
// TB = bytes of a 16-row tile.
template <int BS, int TB>
struct TileDesc {
  static constexpr int H = TileIds<BS>::H;
  static constexpr int HB = TB / H;  // bytes per block part
  Rsrc k[H], v[H];
  // Part and offset of byte `off` of the tile (off known at compile time
  // per load, so the part is too).
  static constexpr int part(int off) { return off / HB; }
};

template <int BS, int TB>
__device__ __forceinline__ TileDesc<BS, TB> tile_desc(const DecodeArgs& a, const TileIds<BS>& ids,
                                                      int j, int kvh, bool ok) {
  TileDesc<BS, TB> d;
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
#pragma unroll
  for (int h = 0; h < TileIds<BS>::H; ++h) {
    const bool okh = ok && (uint32_t)ids.id[h] < (uint32_t)a.num_blocks_i32;
    const int64_t bid = okh ? ids.id[h] : 0;
    int64_t off;
    if constexpr (BS == 32)
      off = (bid * a.num_kv_heads + kvh) * (2 * TB) + (j & 1) * TB;
    else
      off = (bid * a.num_kv_heads + kvh) * TileDesc<BS, TB>::HB;
    d.k[h] = make_rsrc(kc + off, okh ? TileDesc<BS, TB>::HB : 0);
    d.v[h] = make_rsrc(vc + off, okh ? TileDesc<BS, TB>::HB : 0);
  }
  return d;
}

// Tokens of a 16-token tile that count (`left` = context tokens from the
// tile's first on): tokens in a block whose id lies outside the pool do not.
template <int BS>
__device__ __forceinline__ int tile_limit(const DecodeArgs& a, const TileIds<BS>& ids, int left) {
  int n = min(kBlockSize, left);
  if ((uint32_t)ids.id[0] >= (uint32_t)a.num_blocks_i32) return 0;
  if constexpr (BS == 8) {
    if ((uint32_t)ids.id[1] >= (uint32_t)a.num_blocks_i32) n = min(n, 8);
  }
  return n;
}

// Fused KV write: where sequence s's new token goes (slot_mapping[s], the
// rule of [CX] §2.2: block * block_size + offset) and whether it is the last
// position of the context -- then the item holding tile (L-1)/16 uses the
// new row itself, as if the write had come first ([CX] §1.1: o_t attends to
// K_{1:t}, token t included).  `owner`: this item is the one of its
// (sequence, KV head) that stores the row.
struct NewToken {
  bool store;     // store the row (owner, slot inside the pool)
  bool sub;       // tile `tile`, row `row` of the context take the new row
  int tile, row;
  int64_t off;    // byte offset of the slot's row of KV head kvh in either cache
};

template <int BS>
__device__ __forceinline__ NewToken new_token(const DecodeArgs& a, const int32_t* bt, int s,
                                              int kvh, int L, bool owner, int row_bytes) {
  NewToken t{false, false, 0, 0, 0};
  if (a.new_slots == nullptr) return t;
  const int64_t slot = a.new_slots[s];
  if (slot < 0 || slot >= a.num_blocks * BS) return t;
  t.store = owner;
  t.off = ((slot / BS) * a.num_kv_heads + kvh) * (int64_t)(BS * row_bytes) +
          (slot % BS) * (int64_t)row_bytes;
  if (L > 0) {
    const int64_t pos = (int64_t)bt[(L - 1) / BS] * BS + (L - 1) % BS;
    t.sub = pos == slot;
    t.tile = (L - 1) / kBlockSize;
    t.row = (L - 1) % kBlockSize;
  }
  return t;
}

// This lane's 16-byte chunk `c` of sequence s's new row for KV head kvh
// (zeros when there is no fused write: the descriptor is then empty).
__device__ __forceinline__ Rsrc new_row_rsrc(const DecodeArgs& a, const void* base, int s,
                                             int kvh, int row_bytes) {
  const bool on = a.new_slots != nullptr;
  const char* p = on ? static_cast<const char*>(base) +
                           ((int64_t)s * a.num_kv_heads + kvh) * row_bytes
                     : static_cast<const char*>(a.q);
  return make_rsrc(p, on ? row_bytes : 0);
}

// Store `n` bytes (8 or 16) of a new row at byte `off` of a cache.
template <typename T>
__device__ __forceinline__ void store_row_part(const void* cache, int64_t off, const T& v) {
  *reinterpret_cast<T*>(static_cast<char*>(const_cast<void*>(cache)) + off) = v;
}

// Sequence that grid slot `slot` works on.  The hardware dispatcher starts
// workgroups in grid order, so slots take the sequences in decreasing order
// of context length (ties by index): the longest items start first and the
// last to start are the shortest, which keeps the tail of the launch short
// (longest-processing-time-first list scheduling).  Each wave finds its
// sequence by bisection on the length, counting with ballots over the
// lengths held in registers.  Launches with more than kOrderMaxSeqs
// sequences keep the grid order, and so do launches whose items all start at
// once (no more items than compute units: the order cannot matter there, and
// skipping it saves each item the loads it needs).
constexpr int kOrderMaxSeqs = 256;

__device__ __forceinline__ int longest_first(const DecodeArgs& a, int slot) {
  if (a.num_seqs > kOrderMaxSeqs || a.grid_order) return slot;
  const int lane = threadIdx.x & 63;
  constexpr int kChunks = kOrderMaxSeqs / 64;
  int len[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int s = c * 64 + lane;
    len[c] = s < a.num_seqs ? clamp_len(a, s) : -1;
  }
  auto count_ge = [&](int v) {
    int n = 0;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(len[c] >= v));
    return n;
  };
  // largest length v with at least slot + 1 sequences of length >= v
  int lo = 0, hi = a.max_len;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (count_ge(mid) > slot)
      lo = mid;
    else
      hi = mid - 1;
  }
  int r = slot - count_ge(lo + 1);  // rank among the sequences of length lo, by index
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(len[c] == lo);
    const int k = __builtin_popcountll(m);
    if (r < k) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      const uint64_t hit = __builtin_amdgcn_ballot_w64(((m >> lane) & 1) && below == r);
      return c * 64 + __builtin_ctzll(hit);
    }
    r -= k;
  }
  return slot;  // not reached: slot < num_seqs
}

}  // namespace pa
