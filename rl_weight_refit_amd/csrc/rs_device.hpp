// Device-side region tables shared by the planner (which fills them) and the
// HIP kernels (which walk them).  Plain data; no HIP types, so the planner
// compiles as ordinary C++.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace rs {

constexpr int kThreads = 256;         // threads per workgroup (4 wave64s)
// Device pointers passed per launch in the kernel arguments: 500 keeps
// LaunchArgs (24 + 8 * kPool bytes) under the 4 KiB kernel-argument budget.
#ifndef RS_POOL
#define RS_POOL 500
#endif
constexpr int kPool = RS_POOL;
constexpr int kMaxFan = 16;           // destination replicas per region
constexpr uint32_t kThinTile = 16384; // LDS tile of the thin bucket, bytes
constexpr uint32_t kLongRow = 2048;   // bulk rows at least this long are walked row by row
constexpr uint32_t kChunkShift = 8;   // the unit table holds the region of every 256th unit
// Bulk spread groups: kSpread consecutive whole units of a region are copied
// together in pieces of kSpreadPiece bytes dealt round-robin to the group's
// workgroups, so each workgroup's bytes are spread over the group's range
// (kSpread 1: off).  The planner sizes bulk units to whole pieces where it can.
#ifndef RS_SPREAD
#define RS_SPREAD 8
#endif
#ifndef RS_SPREAD_PIECE
#define RS_SPREAD_PIECE 1024
#endif
constexpr uint32_t kSpread = RS_SPREAD;
constexpr uint32_t kSpreadPiece = RS_SPREAD_PIECE;
static_assert(kSpread >= 1 && kSpreadPiece >= 16 && (kSpreadPiece & (kSpreadPiece - 1)) == 0,
              "spread pieces are a power of two of 16-byte vectors");
// MXFP8 work units are staged in LDS, kMxSlots 16-byte slots (8 bf16
// elements each) per workgroup.  A row takes mx_row_pitch(inner) slots
// (normally the power of two at or above its 8-element groups, at least one
// 32-element block), so a unit holds kMxSlots / mx_row_pitch(inner) whole
// rows; rows longer than kMxBatchElems are split at block boundaries first.
#ifndef RS_MX_SLOTS
#define RS_MX_SLOTS 1024
#endif
#ifndef RS_MX_THREADS
#define RS_MX_THREADS 256
#endif
constexpr uint32_t kMxSlots = RS_MX_SLOTS;
constexpr uint32_t kMxThreads = RS_MX_THREADS;   // threads per MXFP8 workgroup
constexpr uint32_t kMxBatchElems = kMxSlots * 8;
static_assert(kMxThreads % 64 == 0 && kMxSlots % (2 * kMxThreads) == 0, "whole slot pairs per lane");

constexpr uint32_t mx_slot_shift(uint32_t inner) {
  uint32_t s = 2;
  while ((1u << s) < (inner + 7) / 8) ++s;
  return s;
}
// Slots per row of a multi-row MXFP8 unit: 2^mx_slot_shift(inner), unless a
// pitch of the row's groups plus two spare slots (for rows staged as aligned
// source lines), rounded up to whole 32-element blocks, fits at least half
// as many rows again into the kMxSlots (rows of 2,368 elements: 3 at 300
// slots, 2 at 512; such rows run in launches of their own, which a smaller
// gain does not pay for).  A pitch that is not a power of two is then never one.
constexpr uint32_t mx_row_pitch(uint32_t inner) {
  const uint32_t lp = 1u << mx_slot_shift(inner);
  const uint32_t p = ((inner + 7) / 8 + 2 + 3) & ~3u;
  return (p <= kMxSlots && 2 * (kMxSlots / p) >= 3 * (kMxSlots / lp)) ? p : lp;
}
constexpr bool mx_pitched(uint32_t inner) { return (mx_row_pitch(inner) & (mx_row_pitch(inner) - 1)) != 0; }
// Most rows a unit at a pitch that is not a power of two holds.
constexpr uint32_t mx_max_pitched_rows() {
  uint32_t m = 0;
  for (uint32_t inner = 1; inner <= kMxBatchElems; ++inner)
    if (mx_pitched(inner) && kMxSlots / mx_row_pitch(inner) > m) m = kMxSlots / mx_row_pitch(inner);
  return m;
}

enum Bucket : uint32_t { kBulk = 0, kThin = 1, kTiny = 2, kMx = 3, kBuckets = 4 };
// Launch kind of thin sibling groups loaded whole (reported as thin regions;
// a kernel of their own, so the thin kernel keeps its register budget).
constexpr uint32_t kThinGroup = kBuckets;
// The same for groups with a member whose LDS reads are 4 bytes or narrower
// (that kernel swizzles its LDS slots).
constexpr uint32_t kThinGroupNarrow = kBuckets + 1;
// MXFP8 regions off the common shapes -- rows at a pitch that is not a power
// of two (mx_row_pitch), and two-piece regions (a block two source shards
// share) -- in launches and a kernel instantiation of their own, so the
// common kernel keeps its registers.
constexpr uint32_t kMxAux = kBuckets + 2;
static_assert(kThinGroup == kBuckets && kThinGroupNarrow == kBuckets + 1 && kMxAux == kBuckets + 2,
              "launch kinds follow the buckets in this order");
// Region bucket of a launch kind.
constexpr uint32_t bucket_of_kind(uint32_t kind) {
  return kind == kThinGroup || kind == kThinGroupNarrow ? uint32_t(kThin) : kind == kMxAux ? uint32_t(kMx) : kind;
}

// Region flags.
enum : uint32_t {
  kFlagOuterMask = 3u,      // number of outer dims (0..3)
  kFlagSrcPacked = 1u << 2, // consecutive rows are contiguous on the source side
  kFlagDstPacked = 1u << 3, // ... on the destination side
  // Thin sibling group loaded whole: the group's units belong to its first
  // member (the others have none); a unit copies rows of the group's column
  // span [min src_off, max src_off + inner) into LDS once and writes every
  // member's (packed) destination rows from there.
  kFlagGroupLoad = 1u << 4,
};
// Largest column span of a sibling group loaded whole, and the LDS tile a
// unit of such a group fills (rows x span bytes).
constexpr uint32_t kGroupSpanMax = 4096;
#ifndef RS_GROUP_TILE
#define RS_GROUP_TILE 16384
#endif
constexpr uint32_t kGroupTile = RS_GROUP_TILE;
static_assert(kGroupTile >= kGroupSpanMax && (kGroupTile & 15u) == 0, "group tile holds whole spans");

// A copy region: rows x inner bytes.  Row r = i0 + e0*(i1 + e1*i2) starts at
// src_off + i0*sstr[0] + i1*sstr[1] + i2*sstr[2] (same on the destination
// side with dstr), relative to the region's buffer pointers.
struct alignas(16) CopyRegion {
  uint64_t src_off;
  uint64_t dst_off;
  uint64_t sstr[3];
  uint64_t dstr[3];
  uint32_t e0, e1;
  uint32_t rows;
  uint32_t inner;
  uint32_t rows_per_unit;
  uint32_t unit_begin;      // first work unit of this region in its launch
  uint32_t flags;           // bits 0-7: kFlag*; bits 8-11: low bits of the OR of
                            // offsets, strides and inner (they bound the vector width);
                            // thin regions, bits 16-23: size of the sibling group the
                            // region belongs to (0: none), bits 24-31: its index there
  uint16_t src_ptr;         // index into the launch's pointer pool
  uint16_t n_dst;
  uint16_t dst_ptr[kMaxFan];
};
static_assert(sizeof(CopyRegion) == 128, "CopyRegion must stay 128 bytes");

// An MXFP8 install region: rows x inner bf16 elements (inner along the
// destination's last dim, starting on a 32-element block boundary), from
// one source or, for a block two source shards share, from two pieces.  Element
// bytes go to dst, block scales to scale (one byte per block,
// sc_inner bytes apart).
struct alignas(16) MxRegion {
  uint64_t src_off;
  uint64_t dst_off;
  uint64_t sc_off;
  uint64_t sstr[3];
  uint64_t dstr[3];
  uint64_t scstr[3];
  uint32_t e0, e1;
  uint32_t rows;
  uint32_t inner;           // elements
  uint32_t rows_per_unit;
  uint32_t unit_begin;
  uint32_t flags;
  uint32_t sc_inner;
  uint16_t src_ptr;
  uint16_t n_dst;
  uint16_t dst_ptr[kMaxFan];
  uint16_t sc_ptr[kMaxFan];
  // Two-piece regions (one block wide, where a source shard boundary falls
  // inside a 32-element block): columns [split, inner) of row r come from
  // src2_ptr at src2_off + row offset by sstr2, column split first.
  // split == inner: one piece.
  uint16_t src2_ptr;
  uint16_t pad0;
  uint32_t split;
  uint64_t src2_off;
  uint64_t sstr2[3];
};
static_assert(sizeof(MxRegion) == 240, "MxRegion must stay 240 bytes");
// The kernels read the 16-bit pool indices as the 32-bit words holding them:
// src_ptr, n_dst, dst_ptr[] (and sc_ptr[]) follow one another from a
// 4-byte-aligned src_ptr.
static_assert(offsetof(CopyRegion, src_ptr) % 4 == 0 && offsetof(CopyRegion, n_dst) == offsetof(CopyRegion, src_ptr) + 2 &&
              offsetof(CopyRegion, dst_ptr) == offsetof(CopyRegion, src_ptr) + 4, "CopyRegion pool index layout");
static_assert(offsetof(MxRegion, src_ptr) % 4 == 0 && offsetof(MxRegion, n_dst) == offsetof(MxRegion, src_ptr) + 2 &&
              offsetof(MxRegion, dst_ptr) == offsetof(MxRegion, src_ptr) + 4 &&
              offsetof(MxRegion, sc_ptr) == offsetof(MxRegion, dst_ptr) + 2 * kMaxFan &&
              offsetof(MxRegion, src2_ptr) == offsetof(MxRegion, sc_ptr) + 2 * kMaxFan,
              "MxRegion pool index layout");

// Kernel arguments of one launch.
struct LaunchArgs {
  const void* regions;          // CopyRegion[] or MxRegion[]
  // Region of unit min(c << kChunkShift, n_units - 1), for c = 0 ..
  // ceil(n_units >> kChunkShift) inclusive (bulk, thin, mx; NULL for tiny).
  const uint32_t* unit_region;
  uint32_t n_regions;
  uint32_t n_units;
  void* ptr[kPool];             // the launch's pointer pool
};
static_assert(sizeof(LaunchArgs) <= 4096, "kernel arguments must fit in 4 KiB");
static_assert(kPool >= 2 + 2 * kMaxFan, "the pool holds every pointer of one region");

// Kernel arguments of a launch whose pointers come from a device table of the
// plan (its regions' pool indices index that table): the same fields, the
// pool replaced by the table's address.
struct TableArgs {
  const void* regions;
  const uint32_t* unit_region;
  uint32_t n_regions;
  uint32_t n_units;
  void* const* ptab;
};

}  // namespace rs
