// HIP kernels of the single-GPU M->N relayout, written for gfx950 (CDNA4,
// wave64).  Every kernel walks the region table built by the planner; a
// region copies rows x inner bytes between strided row sets.  The work is
// bitwise data movement bound by HBM bandwidth, so there is no MFMA here:
// the kernels aim at wide, coalesced global accesses and enough bytes in
// flight per CU.
//
//  bulk  one workgroup per work unit (<= unit_bytes).  16-byte vectors when
//        every address of the region is 16-byte aligned.  Eight consecutive
//        whole units of a region form a spread group: its bytes are cut into
//        1 KiB pieces dealt round-robin to the eight workgroups, so each
//        workgroup's loads and stores spread over the group's range rather
//        than one contiguous run (about 7 % faster on MI355X).  Units outside
//        whole groups: long rows are walked row by row by the whole workgroup;
//        the vectors of short rows are numbered across the unit so every lane
//        loads its share in one batch (sub-wave lane groups per row when rows
//        have several outer dims).  Misaligned regions (source and
//        destination differ modulo 16): rows of 512 bytes or more are staged
//        through a static LDS area (whole source lines by direct-to-LDS
//        loads) and every 16-byte-aligned destination block is rebuilt from
//        two aligned LDS reads joined by byte funnel shifts; shorter rows
//        number their (row, vector) pairs across the unit, each 16-byte
//        store from two aligned source loads joined the same way; the edges
//        of a row go byte by byte, and no load leaves a row.
//        Launched so that at most five workgroups share a CU (see
//        bulk_lds_pad): fewer streams concurrently per CU copy faster.
//  thin  runs shorter than the thin threshold (e.g. the 8-byte rows of a
//        column shard): rows are gathered through an LDS tile so the side
//        that is contiguous across rows is written (or read) with 16-byte
//        vectors.  Sibling regions (same source rows, different columns)
//        whose destinations are packed are loaded whole by a kernel of
//        their own: one workgroup reads a block of the group's source rows
//        once (direct-to-LDS 16-byte loads when the block is contiguous and
//        aligned) and writes every member's rows from LDS with 16-byte
//        stores.  Other siblings take their units member-fastest, in short
//        XCD turns, so the workgroups reading one block of source rows run
//        together on one XCD and share its lines.
//  tiny  regions of at most a few hundred bytes: one lane per region, a
//        wave-level prefix sum of their granule counts, then all 64 lanes
//        share the wave's granules.
//  mx    BF16 -> MXFP8 install.  A work unit (whole rows or one row segment,
//        at most 16 KB of bf16) is loaded straight into LDS with 16-byte
//        direct-to-LDS loads, so the data takes no VGPRs and eight
//        workgroups per CU keep their loads in flight.  Then two lanes per
//        32-element block: integer amax, exact scaled E4M3 conversion, 16
//        code bytes per lane; the block scales are gathered in LDS and
//        written by consecutive lanes at the end.  Units are taken in the
//        same XCD turns as the bulk kernel's (6 % faster than dispatch order).
//        The region's fields and pointers are read once at kernel entry, so
//        no table read (a vector load whose wait would also wait for the
//        stores issued before it) sits between a unit's stores.
//
// Fan-out: a region may name up to 16 destination replicas; the data is read
// once and stored to each (the one-GPU analogue of serving every replica from
// one received copy, "How NCCL M2N Reshard maximizes network bandwidth" in the
// news summary of NVIDIA's Reshard announcement).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "rs_device.hpp"

namespace rs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint64_t row_off(uint32_t r, uint32_t e0, uint32_t e1, uint32_t nouter,
                                            uint64_t s0, uint64_t s1, uint64_t s2) {
  if (nouter <= 1) return uint64_t(r) * s0;
  const uint32_t i0 = r % e0;
  const uint32_t t = r / e0;
  if (nouter == 2) return uint64_t(i0) * s0 + uint64_t(t) * s1;
  const uint32_t i1 = t % e1;
  const uint32_t i2 = t / e1;
  return uint64_t(i0) * s0 + uint64_t(i1) * s1 + uint64_t(i2) * s2;
}

// Tuning knobs (compile-time).  Streaming data is touched once, so loads
// and stores are non-temporal by default.
#ifndef RS_NT_LOAD
#define RS_NT_LOAD 1
#endif
#ifndef RS_NT_STORE
#define RS_NT_STORE 1
#endif
#ifndef RS_UNROLL
#define RS_UNROLL 4   // 16-byte vectors in flight per lane in the bulk kernel
#endif
#ifndef RS_BULK_MIN_WAVES
#define RS_BULK_MIN_WAVES 1  // occupancy floor (waves per SIMD) for the bulk kernel
#endif

__device__ __forceinline__ u32x4 ld16(const void* p) {
#if RS_NT_LOAD
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
#else
  return *static_cast<const u32x4*>(p);
#endif
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
#if RS_NT_STORE
  __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
#else
  *static_cast<u32x4*>(p) = v;
#endif
}

#ifndef RS_XCD_MAP
#define RS_XCD_MAP 1     // bulk kernel: 1 = map workgroups so each XCD walks its own units
#endif
#ifndef RS_XCD_CHUNK
#define RS_XCD_CHUNK 4096   // units per XCD turn (0: one contiguous eighth per XCD)
#endif
#ifndef RS_THIN_GROUP_DMA
#define RS_THIN_GROUP_DMA 1    // group-loaded thin units: aligned blocks go straight into LDS
#endif
#ifndef RS_THIN_LDS_AUX
#define RS_THIN_LDS_AUX 2      // cache policy of those direct-to-LDS loads (2: non-temporal)
#endif
#ifndef RS_MIS_LDS
#define RS_MIS_LDS 1           // bulk kernel: misaligned rows staged through LDS where they fit
#endif
#ifndef RS_MIS_LDS_AUX
#define RS_MIS_LDS_AUX 2       // cache policy of those direct-to-LDS loads (2: non-temporal)
#endif
// Static LDS of the bulk kernel for misaligned rows: a 16 KiB unit of rows of
// at least 512 bytes needs at most 16384 + 31 * 32 bytes (a row slot is
// ceil(row / 16) + 1 lines: at most 31 bytes beyond the row's own).
constexpr uint32_t kMisTile = RS_MIS_LDS ? 17408u : 16u;
#ifndef RS_THIN_SWIZZLE
#define RS_THIN_SWIZZLE 1      // group-loaded thin units with members <= 4 bytes: swizzled LDS slots
#endif
#ifndef RS_THIN_GROUP_BATCH
#define RS_THIN_GROUP_BATCH 1  // group-loaded thin units: a lane's loads all in flight before LDS writes
#endif
#ifndef RS_THIN_XCD_CHUNK
#define RS_THIN_XCD_CHUNK 16  // thin kernel: units per XCD turn (0: dispatch order)
#endif
#ifndef RS_MX_XCD_MAP
#define RS_MX_XCD_MAP 1  // MXFP8 kernel: same choice
#endif
#ifndef RS_MX_XCD_CHUNK
#define RS_MX_XCD_CHUNK RS_XCD_CHUNK
#endif

// Work unit of workgroup b out of n.  Workgroups are dispatched round-robin
// over the 8 XCDs (b -> XCD b % 8), each with its own L2.  Remapped, XCD x
// takes runs of `chunk` consecutive units in turn (or, with chunk 0, one
// contiguous eighth of all units), so neighbouring units stay on one XCD;
// taking turns keeps every XCD's share a mix of the plan's regions, so an
// XCD that drew only the slower regions does not finish last.  Units past
// the last whole round of 8 chunks keep their order.
template <bool kMap>
__device__ __forceinline__ uint32_t unit_of_block(uint32_t b, uint32_t n, uint32_t chunk) {
  if (!kMap) return b;
  const uint32_t x = b & 7u, i = b >> 3;
  if (chunk == 0) {
    const uint32_t per = n >> 3, rem = n & 7u;
    return x * per + min(x, rem) + i;
  }
  const uint32_t full = n / (8u * chunk) * (8u * chunk);
  if (b >= full) return b;
  return ((i / chunk) * 8u + x) * chunk + i % chunk;
}

// Pool indices of a region: the 16-bit fields from src_ptr on (source,
// replica count, destinations, then for MXFP8 regions the scale
// destinations), read as the aligned 32-bit words that hold them, so a
// workgroup-uniform read is a scalar load.  A 16-bit read is a vector load,
// and its wait (vmcnt counts loads and stores together on CDNA) would also
// wait for every store the wave has issued.
template <class Reg>
__device__ __forceinline__ uint32_t pool_field(const Reg* R, uint32_t i) {
  uint32_t w;
  __builtin_memcpy(&w, reinterpret_cast<const char*>(&R->src_ptr) + 4u * (i >> 1), 4);
  return (w >> ((i & 1u) << 4)) & 0xFFFFu;
}
template <class Reg>
__device__ __forceinline__ uint32_t src_pool(const Reg* R) { return pool_field(R, 0); }
template <class Reg>
__device__ __forceinline__ uint32_t n_dst_of(const Reg* R) { return pool_field(R, 1); }
template <class Reg>
__device__ __forceinline__ uint32_t dst_pool(const Reg* R, uint32_t j) { return pool_field(R, 2 + j); }
__device__ __forceinline__ uint32_t sc_pool(const MxRegion* R, uint32_t j) {
  return pool_field(R, 2 + kMaxFan + j);
}

// Pointer pool entry i of a launch.  Every kernel is built twice: with the
// pointers in its arguments (LaunchArgs), and with them in a device table of
// the plan (TableArgs) for launches with more pointers than the arguments
// hold.  The table is read through the constant address space (it does not
// change while the kernel runs), so a uniform index is a scalar load, as for
// the arguments; the pointer is marked global so that the accesses through
// it stay global (not flat) instructions.
typedef __attribute__((address_space(4))) const uint64_t const_u64;
typedef __attribute__((address_space(1))) char global_char;
__device__ __forceinline__ void* pool_ptr(const LaunchArgs& a, uint32_t i) { return a.ptr[i]; }
__device__ __forceinline__ void* pool_ptr(const TableArgs& a, uint32_t i) {
  return (void*)(global_char*)(((const_u64*)(a.ptab))[i]);
}

// Replica j's destination pointer (j uniform), taken from lane j of the
// wave, which read it at the unit's start: a pool index read from the table
// inside a store loop is a vector load, and its wait would also wait for
// the stores of the replicas before it.
__device__ __forceinline__ char* replica(uint64_t dl, uint32_t j) {
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(dl), j);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(dl >> 32), j);
  return (char*)(global_char*)((uint64_t(hi) << 32) | lo);
}

// Region of a work unit: the chunk table brackets it, a short binary search
// over the regions' first units finds it (all loads are uniform).
template <class Reg, class Args>
__device__ __forceinline__ const Reg* find_region(const Args& a, uint32_t unit) {
  const Reg* regs = static_cast<const Reg*>(a.regions);
  const uint32_t c = unit >> kChunkShift;
  uint32_t lo = __builtin_amdgcn_readfirstlane(a.unit_region[c]);
  uint32_t hi = __builtin_amdgcn_readfirstlane(a.unit_region[c + 1]) + 1;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (regs[mid].unit_begin <= unit) lo = mid; else hi = mid;
  }
  return regs + lo;
}

// Copies one granule of g bytes (g in {1,2,4,8,16}; both addresses g-aligned).
__device__ __forceinline__ void copy_granule(char* d, const char* s, uint32_t g) {
  switch (g) {
    case 16: *reinterpret_cast<u32x4*>(d) = *reinterpret_cast<const u32x4*>(s); break;
    case 8: *reinterpret_cast<u32x2*>(d) = *reinterpret_cast<const u32x2*>(s); break;
    case 4: *reinterpret_cast<uint32_t*>(d) = *reinterpret_cast<const uint32_t*>(s); break;
    case 2: *reinterpret_cast<uint16_t*>(d) = *reinterpret_cast<const uint16_t*>(s); break;
    default: *d = *s; break;
  }
}

__device__ __forceinline__ uint32_t low_granule(uint32_t bits) {
  bits |= 16u;
  return bits & (0u - bits);
}

// A whole wave copies n bytes from s to d at the widest granule their
// co-alignment allows, with byte-wise head and tail.
__device__ void wave_copy_span(char* d, const char* s, uint64_t n, uint32_t lane) {
  const uint32_t diff = uint32_t((reinterpret_cast<uintptr_t>(s) ^ reinterpret_cast<uintptr_t>(d)) & 15u);
  const uint32_t g = low_granule(diff);
  uint64_t h = (g - (reinterpret_cast<uintptr_t>(d) & (g - 1))) & (g - 1);
  if (h > n) h = n;
  if (lane < h) d[lane] = s[lane];
  const uint64_t nb = (n - h) / g;
  char* db = d + h;
  const char* sb = s + h;
  switch (g) {
    case 16:
      for (uint64_t k = lane; k < nb; k += 64)
        reinterpret_cast<u32x4*>(db)[k] = reinterpret_cast<const u32x4*>(sb)[k];
      break;
    case 8:
      for (uint64_t k = lane; k < nb; k += 64)
        reinterpret_cast<u32x2*>(db)[k] = reinterpret_cast<const u32x2*>(sb)[k];
      break;
    case 4:
      for (uint64_t k = lane; k < nb; k += 64)
        reinterpret_cast<uint32_t*>(db)[k] = reinterpret_cast<const uint32_t*>(sb)[k];
      break;
    case 2:
      for (uint64_t k = lane; k < nb; k += 64)
        reinterpret_cast<uint16_t*>(db)[k] = reinterpret_cast<const uint16_t*>(sb)[k];
      break;
    default:
      for (uint64_t k = lane; k < nb; k += 64) db[k] = sb[k];
      break;
  }
  const uint64_t done = h + nb * g;
  if (lane < n - done) d[done + lane] = s[done + lane];
}

// Bytes r .. r + 15 of the 32-byte concatenation A | B (r uniform, < 16).
template <int Q>
__device__ __forceinline__ u32x4 funnel_q(u32x4 A, u32x4 B, uint32_t t) {
  const uint32_t c[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
  return u32x4{__builtin_amdgcn_alignbyte(c[Q + 1], c[Q], t), __builtin_amdgcn_alignbyte(c[Q + 2], c[Q + 1], t),
               __builtin_amdgcn_alignbyte(c[Q + 3], c[Q + 2], t), __builtin_amdgcn_alignbyte(c[Q + 4], c[Q + 3], t)};
}
__device__ __forceinline__ u32x4 funnel16(u32x4 A, u32x4 B, uint32_t r) {
  const uint32_t t = r & 3u;
  switch (r >> 2) {
    case 0: return funnel_q<0>(A, B, t);
    case 1: return funnel_q<1>(A, B, t);
    case 2: return funnel_q<2>(A, B, t);
    default: return funnel_q<3>(A, B, t);
  }
}

// The workgroup copies n bytes between two ranges congruent modulo 16.
__device__ __forceinline__ void block_copy_congruent(char* d, const char* s, uint32_t n, uint32_t tid) {
  uint32_t h = uint32_t((16u - (reinterpret_cast<uintptr_t>(d) & 15u)) & 15u);
  if (h > n) h = n;
  if (tid < h) d[tid] = s[tid];
  const uint32_t nv = (n - h) >> 4;
  u32x4* dv = reinterpret_cast<u32x4*>(d + h);
  const u32x4* sv = reinterpret_cast<const u32x4*>(s + h);
  for (uint32_t v = tid; v < nv; v += kThreads) dv[v] = sv[v];
  const uint32_t done = h + (nv << 4);
  if (tid < n - done) d[done + tid] = s[done + tid];
}

__device__ __forceinline__ void block_copy_bytes(char* d, const char* s, uint32_t n, uint32_t tid) {
  for (uint32_t k = tid; k < n; k += kThreads) d[k] = s[k];
}

// ---------------------------------------------------------------------------
// bulk
// ---------------------------------------------------------------------------

// Short aligned rows: lane groups of L lanes per row; each lane holds M
// vectors of each of U rows before storing them.
template <bool kFan1, int M, class Args>
__device__ __forceinline__ void bulk_short_rows(const Args& a, const CopyRegion* R,
                                                const char* sp, char* dp0, uint64_t dst_off,
                                                uint32_t r0, uint32_t r1, uint32_t vpr, uint32_t L,
                                                uint32_t e0, uint32_t e1, uint32_t nouter,
                                                uint64_t s0, uint64_t s1, uint64_t s2,
                                                uint64_t d0, uint64_t d1, uint64_t d2, uint32_t nd, uint64_t dl) {
  constexpr int U = RS_UNROLL / M > 0 ? RS_UNROLL / M : 1;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, wave = tid >> 6;
  const uint32_t sub = lane & (L - 1u);
  const uint32_t G = 64u / L;
  const uint32_t step = 4u * G;
  for (uint32_t rb = r0 + wave * G + lane / L; rb < r1; rb += U * step) {
    u32x4 x[U][M];
    uint64_t dofs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t r = rb + u * step;
      const bool rv = r < r1;
      const uint64_t so = rv ? row_off(r, e0, e1, nouter, s0, s1, s2) : 0;
      dofs[u] = rv ? row_off(r, e0, e1, nouter, d0, d1, d2) : 0;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint32_t v = sub + m * L;
        if (rv && v < vpr) x[u][m] = ld16(sp + so + 16ull * v);
      }
    }
    for (uint32_t j = 0; j < nd; ++j) {
      char* d = kFan1 ? dp0 : replica(dl, j);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t r = rb + u * step;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint32_t v = sub + m * L;
          if (r < r1 && v < vpr) st16(d + dofs[u] + 16ull * v, x[u][m]);
        }
      }
    }
  }
}

// Short aligned rows of a region with at most one outer dim (row r at
// r * stride on each side), numbered flat: vector f = i * vpr + v (row
// r0 + i, vector v of it).  Lane tid takes f = f0 + tid + k * kThreads, so
// every lane loads RS_UNROLL vectors and a unit of up to RS_UNROLL * kThreads
// vectors is one load batch, whatever vpr is.  The row is floor(f / vpr),
// computed as (f * ceil(2^32 / vpr)) >> 32: exact for f < 2^20 and vpr < 2^11
// (the error term f / 2^32 stays below the smallest gap 1 / vpr).
template <bool kFan1, class Args>
__device__ __forceinline__ void bulk_short_flat(const Args& a, const CopyRegion* R,
                                                const char* sp, uint64_t dst_off, uint32_t r0,
                                                uint32_t r1, uint32_t vpr, uint64_t s0, uint64_t d0,
                                                uint32_t nd, uint64_t dl) {
  constexpr int U = RS_UNROLL;
  const uint32_t tid = threadIdx.x;
  const uint64_t magic = ((uint64_t(1) << 32) + vpr - 1) / vpr;
  const uint32_t nvec = (r1 - r0) * vpr;
  for (uint32_t f0 = 0; f0 < nvec; f0 += U * kThreads) {
    u32x4 x[U];
    uint64_t o[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint32_t f = f0 + k * kThreads + tid;
      const uint32_t i = uint32_t((uint64_t(f) * magic) >> 32);
      const uint32_t r = r0 + i;
      const uint32_t v = f - i * vpr;
      o[k] = uint64_t(r) * d0 + 16ull * v;
      if (f < nvec) x[k] = ld16(sp + uint64_t(r) * s0 + 16ull * v);
    }
    for (uint32_t j = 0; j < nd; ++j) {
      char* d = kFan1 ? static_cast<char*>(pool_ptr(a, dst_pool(R, 0))) + dst_off : replica(dl, j);
#pragma unroll
      for (int k = 0; k < U; ++k)
        if (f0 + k * kThreads + tid < nvec) st16(d + o[k], x[k]);
    }
  }
}

// Spread groups (aligned rows).  The kSpread consecutive units of a group
// cover rows g0 .. g0 + kSpread * rpu - 1 of the region, numbered as one run
// of 16-byte vectors cut into pieces of kPieceVec vectors; the group's
// workgroup j takes pieces j, j + kSpread, j + 2 kSpread, ...  It moves one
// unit's worth of bytes, as before, but from kSpread-apart pieces spread
// over the group's range: on MI355X a plain copy that spreads each
// workgroup this way streams about 10 % faster than one that gives each
// workgroup one contiguous run.
constexpr uint32_t kPieceVec = kSpreadPiece / 16;
constexpr uint32_t kWaves = kThreads / 64;

// Rows with at most one outer dim (row r at r * stride): lane by lane, group
// vector f is row f / vpr (magic division, exact while f * vpr < 2^32).
template <bool kFan1, class Args>
__device__ __forceinline__ void bulk_spread_flat(const Args& a, const CopyRegion* R,
                                                 const char* sp, uint64_t dst_off, uint32_t g0,
                                                 uint32_t j, uint32_t nvec, uint32_t vpr,
                                                 uint64_t s0, uint64_t d0, uint32_t nd, uint64_t dl) {
  constexpr int U = RS_UNROLL;
  const uint32_t tid = threadIdx.x;
  const uint64_t magic = ((uint64_t(1) << 32) + vpr - 1) / vpr;
  for (uint32_t t0 = 0; t0 < nvec; t0 += U * kThreads) {
    u32x4 x[U];
    uint64_t o[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint32_t t = t0 + k * kThreads + tid;
      const uint32_t f = ((t / kPieceVec) * kSpread + j) * kPieceVec + t % kPieceVec;
      const uint32_t i = uint32_t((uint64_t(f) * magic) >> 32);
      const uint64_t r = g0 + i;
      const uint32_t v = f - i * vpr;
      o[k] = r * d0 + 16ull * v;
      if (t < nvec) x[k] = ld16(sp + r * s0 + 16ull * v);
    }
    for (uint32_t jd = 0; jd < nd; ++jd) {
      char* d = kFan1 ? static_cast<char*>(pool_ptr(a, dst_pool(R, 0))) + dst_off : replica(dl, jd);
#pragma unroll
      for (int k = 0; k < U; ++k)
        if (t0 + k * kThreads + tid < nvec) st16(d + o[k], x[k]);
    }
  }
}

// Rows of whole 1 KiB pieces (vpr a multiple of 64), any number of outer
// dims: a piece lies in one row and is one wave's 64 vectors, so all row
// arithmetic is uniform.  A wave's pieces are kWaves * kSpread apart in the
// group; it splits its first piece's row into outer indices once and then
// advances piece column and indices by carries, with no division per piece.
template <bool kFan1, class Args>
__device__ __forceinline__ void bulk_spread_rows(const Args& a, const CopyRegion* R,
                                                 const char* sp, uint64_t dst_off, uint32_t g0,
                                                 uint32_t j, uint32_t npu, uint32_t ppr,
                                                 uint32_t e0, uint32_t e1, uint32_t nouter,
                                                 uint64_t s0, uint64_t s1, uint64_t s2,
                                                 uint64_t d0, uint64_t d1, uint64_t d2, uint32_t nd, uint64_t dl) {
  constexpr int U = RS_UNROLL;
  constexpr uint32_t kStep = kWaves * kSpread;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t lo = 16ull * lane;
  const uint32_t di = kStep / ppr, dc = kStep % ppr;
  const uint32_t p0 = wave * kSpread + j;
  uint32_t c = p0 % ppr;
  uint32_t i0 = g0 + p0 / ppr, i1 = 0, i2 = 0;
  if (nouter >= 2) {
    i1 = i0 / e0;
    i0 -= i1 * e0;
    if (nouter == 3) {
      i2 = i1 / e1;
      i1 -= i2 * e1;
    }
  }
  for (uint32_t l0 = 0; l0 < npu; l0 += U * kWaves) {
    u32x4 x[U];
    uint64_t o[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint64_t cb = uint64_t(c) * kSpreadPiece + lo;
      o[k] = i0 * d0 + i1 * d1 + i2 * d2 + cb;
      if (l0 + k * kWaves + wave < npu) x[k] = ld16(sp + (i0 * s0 + i1 * s1 + i2 * s2 + cb));
      // the wave's next piece: kStep pieces on, carried into row and outer indices
      c += dc;
      uint32_t adv = di;
      if (c >= ppr) {
        c -= ppr;
        ++adv;
      }
      i0 += adv;
      if (nouter >= 2) {
        while (i0 >= e0) {
          i0 -= e0;
          if (++i1 == e1 && nouter == 3) {
            i1 = 0;
            ++i2;
          }
        }
      }
    }
    for (uint32_t jd = 0; jd < nd; ++jd) {
      char* d = kFan1 ? static_cast<char*>(pool_ptr(a, dst_pool(R, 0))) + dst_off : replica(dl, jd);
#pragma unroll
      for (int k = 0; k < U; ++k)
        if (l0 + k * kWaves + wave < npu) st16(d + o[k], x[k]);
    }
  }
}

// Rows of a misaligned region (source and destination differ modulo 16)
// into one destination, rows [r0, r1) of n bytes.  Per row, once the
// destination is 16-byte aligned (hd bytes in), output vector v is bytes
// r .. r + 15 of the aligned 16-byte source lines L(v) and L(v) + 16 (r =
// the source's offset in its line, 0 when the row is co-aligned), joined by
// byte funnel shifts; only vectors whose lines lie inside the row are done
// so, so no load leaves the row.  The unit's (row, vector) pairs are
// numbered flat, so every lane has several loads in flight; the row edges
// (under 32 bytes at the head, 48 at the tail) are one byte per item, loaded
// in the same batches, before any store.
struct MisRow {
  const char* s;
  char* d;
  uint32_t hd, r;
  int lo, hi;        // vectors lo .. hi (none when hi < lo)
  uint32_t b0, b1;   // edges: bytes [0, b0) and [b1, n)
};

__device__ __forceinline__ MisRow mis_row(const char* s, char* d, uint32_t n) {
  MisRow m;
  m.s = s;
  m.d = d;
  m.hd = uint32_t((16u - (reinterpret_cast<uintptr_t>(d) & 15u)) & 15u);
  m.r = uint32_t((reinterpret_cast<uintptr_t>(s) + m.hd) & 15u);
  if (m.r == 0) {
    m.lo = 0;
    m.hi = n >= m.hd + 16u ? int((n - m.hd) >> 4) - 1 : -1;
  } else {
    m.lo = m.hd >= m.r ? 0 : 1;
    m.hi = n + m.r >= m.hd + 32u ? int((n + m.r - m.hd - 32u) >> 4) : -1;
  }
  m.b0 = min(n, m.hd + 16u * uint32_t(m.lo));
  m.b1 = m.hi >= m.lo ? m.hd + 16u * uint32_t(m.hi + 1) : m.b0;
  return m;
}

__device__ __forceinline__ void bulk_misaligned_rows(const char* sp, char* dp, uint32_t r0, uint32_t r1,
                                                     uint32_t n, uint32_t e0, uint32_t e1, uint32_t nouter,
                                                     uint64_t s0, uint64_t s1, uint64_t s2,
                                                     uint64_t d0, uint64_t d1, uint64_t d2) {
  constexpr int U = 4;          // vector items per lane per batch
  constexpr int UE = 4;         // edge bytes per lane per batch
  constexpr uint32_t kEdge = 80;  // edge slots per row: head 0-31, tail 32-79
  const uint32_t tid = threadIdx.x;
  const uint32_t nvr = (n + 15u) >> 4;   // vector slots per row
  const uint32_t rows = r1 - r0;
  const uint32_t total = rows * nvr, te = rows * kEdge;
  const uint64_t magic = ((uint64_t(1) << 32) + nvr - 1) / nvr;
  // Batches: a lane's vector loads and edge-byte loads are all issued
  // before its stores.
  const uint32_t nbv = (total + U * kThreads - 1) / (U * kThreads);
  const uint32_t nbe = (te + UE * kThreads - 1) / (UE * kThreads);
  const uint32_t nbat = max(nbv, nbe);
  for (uint32_t bt = 0; bt < nbat; ++bt) {
    u32x4 A[U], B[U];
    char* dv[U];
    uint32_t rr[U];
    bool ok[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint32_t f = (bt * U + k) * kThreads + tid;
      ok[k] = false;
      rr[k] = 0;
      dv[k] = nullptr;
      if (f < total) {
        const uint32_t i = uint32_t((uint64_t(f) * magic) >> 32);
        const int v = int(f - i * nvr);
        const MisRow m = mis_row(sp + row_off(r0 + i, e0, e1, nouter, s0, s1, s2),
                                 dp + row_off(r0 + i, e0, e1, nouter, d0, d1, d2), n);
        if (v >= m.lo && v <= m.hi) {
          const char* line = m.s + m.hd - m.r + 16u * uint32_t(v);
          A[k] = *reinterpret_cast<const u32x4*>(line);
          if (m.r) B[k] = *reinterpret_cast<const u32x4*>(line + 16u);
          ok[k] = true;
          rr[k] = m.r;
          dv[k] = m.d + m.hd + 16u * uint32_t(v);
        }
      }
    }
    char eb[UE];
    char* ed[UE];
#pragma unroll
    for (int k = 0; k < UE; ++k) {
      const uint32_t f = (bt * UE + k) * kThreads + tid;
      ed[k] = nullptr;
      eb[k] = 0;
      if (f < te) {
        const uint32_t i = f / kEdge, e = f - i * kEdge;
        const MisRow m = mis_row(sp + row_off(r0 + i, e0, e1, nouter, s0, s1, s2),
                                 dp + row_off(r0 + i, e0, e1, nouter, d0, d1, d2), n);
        const uint32_t pos = e < 32u ? e : m.b1 + (e - 32u);
        if (e < 32u ? pos < m.b0 : pos < n) {
          eb[k] = m.s[pos];
          ed[k] = m.d + pos;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (ok[k]) st16(dv[k], rr[k] ? funnel16(A[k], B[k], rr[k]) : A[k]);
#pragma unroll
    for (int k = 0; k < UE; ++k)
      if (ed[k]) *ed[k] = eb[k];
  }
}

// Misaligned rows staged through LDS (rows of at least kMisMinRow bytes
// whose unit fits the bulk kernel's kMisTile staging area; replicas at one
// alignment).  Row i of the unit takes LDS slot i (lm 16-byte lines): row
// byte x at slot byte h_i + x, h_i = source address mod 16.  Source lines
// wholly inside a row cover its bytes [f0, f1); the row's 16-byte-aligned
// destination blocks inside that span cover [e0, e1).
//   Phase 1: the whole lines go straight into LDS with direct-to-LDS
//   16-byte loads, and the bytes of the partial first and last lines
//   ([0, f0) and [f1, n), under 16 each) into registers, all before one
//   wait, so no load leaves the row.
//   Phase 2, per destination: each block is two aligned LDS reads joined by
//   a funnel shift and one 16-byte store; the edge bytes [0, e0) and
//   [e1, n) come from the registers or, inside [f0, f1), from LDS.
constexpr uint32_t kMisMinRow = 512;
constexpr int kMisEdge = 4;   // edge bytes per lane and source: 32 per row, rows * 32 <= kMisEdge * kThreads

struct MisSpan {
  uint32_t h, f0, f1, e0, e1;
};
__device__ __forceinline__ MisSpan mis_span(const char* src, const char* dst, uint32_t n) {
  MisSpan m;
  m.h = uint32_t(reinterpret_cast<uintptr_t>(src) & 15u);
  m.f0 = (16u - m.h) & 15u;
  m.f1 = n >= m.f0 + 16u ? m.f0 + ((n - m.f0) & ~15u) : m.f0;
  const uint32_t y0 = (16u - uint32_t(reinterpret_cast<uintptr_t>(dst) & 15u)) & 15u;  // first block start
  m.e0 = m.f0 + ((y0 - m.f0) & 15u);
  m.e1 = m.f1 >= m.e0 + 16u ? m.e0 + ((m.f1 - m.e0) & ~15u) : m.e0;
  return m;
}

template <bool kFan1, class Args>
__device__ __forceinline__ void bulk_misaligned_lds(const Args& a, const CopyRegion* R, const char* sp,
                                                    char* dp0, uint64_t dst_off, uint32_t r0, uint32_t rows,
                                                    uint32_t n, uint32_t lm, uint32_t e0, uint32_t e1,
                                                    uint32_t nouter, uint64_t s0, uint64_t s1, uint64_t s2,
                                                    uint64_t d0, uint64_t d1, uint64_t d2, uint32_t nd,
                                                    char* lds, uint64_t dl) {
  const uint32_t tid = threadIdx.x;
  // Phase 1: partial-line bytes into registers (edge slot e < 16: row byte
  // e; e >= 16: row byte f1 + e - 16), whole lines into LDS.
  char eb[kMisEdge];
#pragma unroll
  for (int k = 0; k < kMisEdge; ++k) {
    const uint32_t f = uint32_t(k) * kThreads + tid;
    eb[k] = 0;
    if (f < rows * 32u) {
      const uint32_t i = f >> 5, e = f & 31u;
      const char* src = sp + row_off(r0 + i, e0, e1, nouter, s0, s1, s2);
      const uint32_t h = uint32_t(reinterpret_cast<uintptr_t>(src) & 15u), f0 = (16u - h) & 15u;
      const uint32_t f1 = n >= f0 + 16u ? f0 + ((n - f0) & ~15u) : f0;
      const uint32_t pos = e < 16u ? e : f1 + (e - 16u);
      if (e < 16u ? pos < f0 : pos < n) eb[k] = src[pos];
    }
  }
  const uint32_t slots = rows * lm;
  const uint64_t mag = ((uint64_t(1) << 32) + lm - 1) / lm;   // exact: slots * lm < 2^32
  for (uint32_t f0 = 0; f0 < slots; f0 += kThreads) {
    const uint32_t f = f0 + tid;
    if (f < slots) {
      const uint32_t i = uint32_t((uint64_t(f) * mag) >> 32), j = f - i * lm;
      const char* src = sp + row_off(r0 + i, e0, e1, nouter, s0, s1, s2);
      const int x0 = int(16u * j) - int(reinterpret_cast<uintptr_t>(src) & 15u);   // row byte at line j
      if (x0 >= 0 && uint32_t(x0) + 16u <= n)
        __builtin_amdgcn_global_load_lds(src + x0, (lds_void*)(lds + 16u * (f0 + (tid & ~63u))), 16, 0,
                                         RS_MIS_LDS_AUX);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Phase 2.
  const uint32_t mb = (n + 15u) / 16u + 1u;   // aligned destination blocks a row can touch
  const uint32_t blocks = rows * mb;
  const uint64_t magb = ((uint64_t(1) << 32) + mb - 1) / mb;
  for (uint32_t jd = 0; jd < nd; ++jd) {
    char* dp = kFan1 ? dp0 : replica(dl, jd);
    for (uint32_t f = tid; f < blocks; f += kThreads) {
      const uint32_t i = uint32_t((uint64_t(f) * magb) >> 32), b = f - i * mb;
      char* dst = dp + row_off(r0 + i, e0, e1, nouter, d0, d1, d2);
      const MisSpan m = mis_span(sp + row_off(r0 + i, e0, e1, nouter, s0, s1, s2), dst, n);
      const uint32_t y = m.e0 + 16u * b;   // row byte at the start of block b
      if (y + 16u > m.e1) continue;
      const uint32_t o = 16u * i * lm + m.h + y, o0 = o & ~15u, sh = o & 15u;
      const u32x4 A = *reinterpret_cast<const u32x4*>(lds + o0);
      st16(dst + y, sh ? funnel16(A, *reinterpret_cast<const u32x4*>(lds + o0 + 16u), sh) : A);
    }
#pragma unroll
    for (int k = 0; k < kMisEdge; ++k) {
      const uint32_t f = uint32_t(k) * kThreads + tid;
      if (f < rows * 32u) {
        const uint32_t i = f >> 5, e = f & 31u;
        char* dst = dp + row_off(r0 + i, e0, e1, nouter, d0, d1, d2);
        const MisSpan m = mis_span(sp + row_off(r0 + i, e0, e1, nouter, s0, s1, s2), dst, n);
        // from the registers: [0, f0) and [f1, n)
        const uint32_t pr = e < 16u ? e : m.f1 + (e - 16u);
        if (e < 16u ? pr < m.f0 : pr < n) dst[pr] = eb[k];
        // from LDS: [f0, e0) and [e1, f1)
        const uint32_t pl = e < 16u ? m.f0 + e : m.e1 + (e - 16u);
        if (e < 16u ? pl < m.e0 : pl < m.f1) dst[pl] = lds[16u * i * lm + m.h + pl];
      }
    }
  }
}

template <bool kFan1, class Args>
__device__ __forceinline__ void bulk_body(const Args& a, const CopyRegion* R, uint32_t unit,
                                          char* mis_tile) {
  const uint32_t tid = threadIdx.x;
  const uint64_t src_off = R->src_off, dst_off = R->dst_off;
  const uint64_t s0 = R->sstr[0], s1 = R->sstr[1], s2 = R->sstr[2];
  const uint64_t d0 = R->dstr[0], d1 = R->dstr[1], d2 = R->dstr[2];
  const uint32_t e0 = R->e0, e1 = R->e1, rows = R->rows, inner = R->inner;
  const uint32_t rpu = R->rows_per_unit, ub = R->unit_begin, flags = R->flags;
  const uint32_t nd = kFan1 ? 1u : n_dst_of(R);
  const uint32_t nouter = flags & kFlagOuterMask;
  const char* sp = static_cast<const char*>(pool_ptr(a, src_pool(R))) + src_off;
  char* dp0 = static_cast<char*>(pool_ptr(a, dst_pool(R, 0))) + dst_off;
  // Several replicas: lane j of each wave holds replica j's pointer.
  uint64_t dl = 0;
  if (!kFan1 && (tid & 63u) < nd)
    dl = reinterpret_cast<uint64_t>(pool_ptr(a, dst_pool(R, tid & 63u))) + dst_off;

  uint32_t al = (flags >> 8) & 15u;
  al |= uint32_t(reinterpret_cast<uintptr_t>(sp) & 15u);
  for (uint32_t j = 0; j < nd; ++j)
    al |= uint32_t((reinterpret_cast<uintptr_t>(pool_ptr(a, dst_pool(R, j))) + dst_off) & 15u);

  const uint32_t r0 = (unit - ub) * rpu;
  const uint32_t r1 = min(r0 + rpu, rows);

  if (kSpread > 1 && al == 0) {
    // A whole group of whole-piece units goes the spread way.
    const uint32_t vpr = inner >> 4;
    const uint64_t nvec = uint64_t(rpu) * vpr;
    const uint32_t ul = unit - ub, j = ul % kSpread;
    const uint64_t g0 = uint64_t(ul - j) * rpu;
    if (g0 + uint64_t(kSpread) * rpu <= rows && nvec % kPieceVec == 0) {
      if (nouter <= 1 && nvec * kSpread * vpr < (uint64_t(1) << 32)) {
        bulk_spread_flat<kFan1>(a, R, sp, dst_off, uint32_t(g0), j, uint32_t(nvec), vpr, s0, d0, nd, dl);
        return;
      }
      if (kPieceVec == 64 && vpr % kPieceVec == 0) {
        bulk_spread_rows<kFan1>(a, R, sp, dst_off, uint32_t(g0), j, uint32_t(nvec / kPieceVec),
                                vpr / kPieceVec, e0, e1, nouter, s0, s1, s2, d0, d1, d2, nd, dl);
        return;
      }
    }
  }

  if (al == 0 && inner >= kLongRow) {
    // Long rows: the workgroup walks one row at a time.
    const uint32_t vpr = inner >> 4;
    for (uint32_t r = r0; r < r1; ++r) {
      const uint64_t so = row_off(r, e0, e1, nouter, s0, s1, s2);
      const uint64_t dof = row_off(r, e0, e1, nouter, d0, d1, d2);
      const char* s = sp + so;
      for (uint32_t v = tid; v < vpr; v += RS_UNROLL * kThreads) {
        u32x4 x[RS_UNROLL];
#pragma unroll
        for (int k = 0; k < RS_UNROLL; ++k)
          if (v + k * kThreads < vpr) x[k] = ld16(s + 16ull * (v + k * kThreads));
        for (uint32_t j = 0; j < nd; ++j) {
          char* d = (kFan1 ? dp0 : replica(dl, j)) + dof;
#pragma unroll
          for (int k = 0; k < RS_UNROLL; ++k)
            if (v + k * kThreads < vpr) st16(d + 16ull * (v + k * kThreads), x[k]);
        }
      }
    }
  } else if (al == 0) {
    // Short rows.  With at most one outer dim the unit's vectors are numbered
    // flat; otherwise L lanes per row (a power of two >= the row's vectors,
    // at most 64), 64 / L rows per wave step, each lane moving one or two
    // vectors of each of several rows per iteration.
    const uint32_t vpr = inner >> 4;
    if (nouter <= 1) {
      bulk_short_flat<kFan1>(a, R, sp, dst_off, r0, r1, vpr, s0, d0, nd, dl);
      return;
    }
    uint32_t L = 1;
    while (L < vpr && L < 64u) L <<= 1;
    if (vpr > L)
      bulk_short_rows<kFan1, 2>(a, R, sp, dp0, dst_off, r0, r1, vpr, L, e0, e1, nouter,
                                s0, s1, s2, d0, d1, d2, nd, dl);
    else
      bulk_short_rows<kFan1, 1>(a, R, sp, dp0, dst_off, r0, r1, vpr, L, e0, e1, nouter,
                                s0, s1, s2, d0, d1, d2, nd, dl);
  } else {
#if RS_MIS_LDS
    // Misaligned rows that fit the staging area, replicas at one alignment:
    // through LDS.
    const uint32_t lm = (inner + 15u) / 16u + 1u;
    bool congruent = true;
    for (uint32_t j = 1; j < nd; ++j)
      congruent &= ((reinterpret_cast<uintptr_t>(pool_ptr(a, dst_pool(R, j))) ^ reinterpret_cast<uintptr_t>(
                        pool_ptr(a, dst_pool(R, 0)))) & 15u) == 0;
    if (congruent && inner >= kMisMinRow && uint64_t(r1 - r0) * lm * 16u <= kMisTile &&
        (r1 - r0) * 32u <= uint32_t(kMisEdge) * kThreads) {
      bulk_misaligned_lds<kFan1>(a, R, sp, dp0, dst_off, r0, r1 - r0, inner, lm, e0, e1, nouter, s0, s1, s2,
                                 d0, d1, d2, nd, mis_tile, dl);
      return;
    }
#endif
    // Misaligned: funnel-shifted 16-byte vectors numbered across the unit,
    // once per destination (each replica may sit at its own alignment).
    for (uint32_t j = 0; j < nd; ++j) {
      char* dp = kFan1 ? dp0 : replica(dl, j);
      bulk_misaligned_rows(sp, dp, r0, r1, inner, e0, e1, nouter, s0, s1, s2, d0, d1, d2);
    }
  }
}

template <class Args>
__global__ __launch_bounds__(kThreads, RS_BULK_MIN_WAVES) void rs_bulk_kernel(Args a) {
  // One workgroup per work unit (looping workgroups measured slower).
  const uint32_t unit = unit_of_block<RS_XCD_MAP != 0>(blockIdx.x, gridDim.x, RS_XCD_CHUNK);
  const CopyRegion* R = find_region<CopyRegion>(a, unit);
  __shared__ __attribute__((aligned(16))) char mis_tile[kMisTile];
  if (n_dst_of(R) == 1)
    bulk_body<true>(a, R, unit, mis_tile);
  else
    bulk_body<false>(a, R, unit, mis_tile);
}

// ---------------------------------------------------------------------------
// thin (LDS-staged)
// ---------------------------------------------------------------------------

// Packed destination rows of one member of a group loaded whole: output
// byte q of the member's rows [r0, r1) is LDS byte row * S + cm + col of
// the staged span (row = q / inner, col = q % inner).  G: the granule the
// LDS side allows (a divisor of inner, cm and S); 16-byte stores where the
// destination is 16-byte aligned, granules for the rest.
// LDS slot swizzle of group-loaded blocks with members that read granules of
// 4 bytes or less: 16-byte slot s is kept at slot s ^ ((s >> 4) & 7), i.e. byte a at
// a ^ (((a >> 8) & 7) << 4).  A member's stores read 4-byte (or narrower)
// granules of rows 4v .. 4v + 3, 32 bytes apart for 32-byte rows: unswizzled,
// a wave's reads fall on two bank groups (32 lanes per bank); swizzled, on
// sixteen.  The map only permutes slots inside aligned groups of eight and
// is its own inverse, so the loads fetch source slot swz(p) into slot p.
template <bool kSw>
__device__ __forceinline__ uint32_t lds_swz8(uint32_t a) {
  return kSw ? a ^ (((a >> 8) & 7u) << 4) : a;
}

template <int G, bool kSw>
__device__ __forceinline__ void group_store(char* D, const char* lds, uint32_t cm, uint32_t S, uint32_t inner,
                                           uint32_t nbytes, uint32_t tid) {
  uint32_t head = 0;
  if ((reinterpret_cast<uintptr_t>(D) & 15u) == 0) {
    const uint32_t nvec = nbytes >> 4;
    for (uint32_t v = tid; v < nvec; v += kThreads) {
      uint32_t row = (16u * v) / inner;
      uint32_t col = 16u * v - row * inner;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 16 / G; ++k) {
        const char* p = lds + lds_swz8<kSw>(row * S + cm + col);
        if (G == 16) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(p);
          w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
        } else if (G == 8) {
          const u32x2 t = *reinterpret_cast<const u32x2*>(p);
          w[2 * k] = t.x;
          w[2 * k + 1] = t.y;
        } else if (G == 4) {
          w[k] = *reinterpret_cast<const uint32_t*>(p);
        } else if (G == 2) {
          w[k >> 1] |= uint32_t(*reinterpret_cast<const uint16_t*>(p)) << (16 * (k & 1));
        } else {
          w[k >> 2] |= uint32_t(*reinterpret_cast<const uint8_t*>(p)) << (8 * (k & 3));
        }
        col += G;
        if (col >= inner) {
          col -= inner;
          ++row;
        }
      }
      st16(D + 16u * v, u32x4{w[0], w[1], w[2], w[3]});
    }
    head = nvec << 4;
  }
  // The rest (a tail, or everything for a misaligned destination) by
  // granules as wide as both sides allow.
  const uint32_t g = low_granule(uint32_t(G) | uint32_t(reinterpret_cast<uintptr_t>(D) & 15u));
  for (uint32_t q = head + tid * g; q < nbytes; q += kThreads * g) {
    const uint32_t row = q / inner, col = q - row * inner;
    copy_granule(D + q, lds + lds_swz8<kSw>(row * S + cm + col), g);
  }
}

// One unit of a sibling group loaded whole (kFlagGroupLoad; R is the
// group's first member, the members follow it in the table): rows
// [r0, r1) of the group's column span go into LDS once -- 16-byte vectors
// when consecutive rows of the span are contiguous in the source -- and
// every member writes its packed destination rows from there.
// kSw: some member reads granules of 4 bytes or less; slots swizzled
// (lds_swz8) where the block goes straight into LDS.
template <bool kSw, class Args>
__device__ __forceinline__ void thin_group_body(const Args& a, const CopyRegion* R, uint32_t ul, char* tile,
                                                uint64_t lo, uint32_t S) {
  const uint32_t tid = threadIdx.x;
  const uint32_t gm = (R->flags >> 16) & 255u;
  const uint32_t rows = R->rows, rpu = R->rows_per_unit;
  const uint32_t e0 = R->e0, e1 = R->e1, nouter = R->flags & kFlagOuterMask;
  const uint64_t s0 = R->sstr[0], s1 = R->sstr[1], s2 = R->sstr[2];
  const char* base = static_cast<const char*>(pool_ptr(a, src_pool(R))) + lo;
  const uint32_t r0 = ul * rpu, r1 = min(r0 + rpu, rows), T = r1 - r0;
  // The members' fields, read before any store, lane m of every wave holding
  // member m's (members past 64 read theirs in the store loop): a table read
  // after a store is a vector load, and its wait would also wait for the
  // stores of the members before it.  Not in the swizzled instantiation,
  // where the extra registers would cost it two workgroups per CU.
  const uint32_t lane = tid & 63u;
  uint32_t m_cm = 0, m_inner = 0, m_nd = 0;
  uint64_t m_dst = 0;
  if (!kSw && lane < gm) {
    const CopyRegion* M = R + lane;
    m_cm = uint32_t(M->src_off - lo);
    m_inner = M->inner;
    m_nd = n_dst_of(M);
    m_dst = reinterpret_cast<uint64_t>(pool_ptr(a, dst_pool(M, 0))) + M->dst_off;
  }
  uint32_t sh = 0;
  bool swz = false;
  if (nouter <= 1 && s0 == S) {
    // One contiguous block: byte head, then 16-byte vectors with all of a
    // lane's loads in flight before any LDS write, then a byte tail.
    const char* src = base + uint64_t(r0) * S;
    sh = uint32_t(reinterpret_cast<uintptr_t>(src) & 15u);
    const uint32_t n = T * S;
#if RS_THIN_GROUP_DMA
    if (sh == 0 && (n & 15u) == 0) {
      // Aligned block: straight into LDS with direct-to-LDS 16-byte loads
      // (no registers; every load of the unit in flight at once).
      constexpr uint32_t kB = (kGroupTile / 16 + kThreads - 1) / kThreads;
      const uint32_t nv = n >> 4;
      swz = kSw && (nv & 7u) == 0;
#pragma unroll
      for (uint32_t k = 0; k < kB; ++k) {
        const uint32_t v = k * kThreads + tid;
        const uint32_t vs = swz ? v ^ ((v >> 4) & 7u) : v;   // below nv: nv is a multiple of 8
        if (v < nv)
          __builtin_amdgcn_global_load_lds(src + 16u * vs,
                                           (lds_void*)(tile + 16u * (k * kThreads + (tid & ~63u))), 16, 0,
                                           RS_THIN_LDS_AUX);
      }
      __builtin_amdgcn_s_waitcnt(0);
    } else
#endif
    {
#if RS_THIN_GROUP_BATCH
    uint32_t h = (16u - sh) & 15u;
    if (h > n) h = n;
    if (tid < h) tile[sh + tid] = src[tid];
    const uint32_t nv = (n - h) >> 4;
    const u32x4* sv = reinterpret_cast<const u32x4*>(src + h);
    u32x4* dv = reinterpret_cast<u32x4*>(tile + sh + h);
    constexpr uint32_t kB = (kGroupTile / 16 + kThreads - 1) / kThreads;
    u32x4 x[kB];
#pragma unroll
    for (uint32_t k = 0; k < kB; ++k)
      if (k * kThreads + tid < nv) x[k] = ld16(sv + k * kThreads + tid);
#pragma unroll
    for (uint32_t k = 0; k < kB; ++k)
      if (k * kThreads + tid < nv) dv[k * kThreads + tid] = x[k];
    const uint32_t done = h + (nv << 4);
    if (tid < n - done) tile[sh + done + tid] = src[done + tid];
#else
    block_copy_congruent(tile + sh, src, n, tid);
#endif
    }
  } else {
    uint32_t al = uint32_t(reinterpret_cast<uintptr_t>(base) & 15u) | S | uint32_t(s0 & 15u);
    if (nouter >= 2) al |= uint32_t(s1 & 15u);
    if (nouter >= 3) al |= uint32_t(s2 & 15u);
    const uint32_t g = low_granule(al), gpr = S / g, total = T * gpr;
    for (uint32_t f = tid; f < total; f += kThreads) {
      const uint32_t row = f / gpr, k = f - row * gpr;
      copy_granule(tile + row * S + k * g, base + row_off(r0 + row, e0, e1, nouter, s0, s1, s2) + k * g, g);
    }
  }
  __syncthreads();
  const char* lds = tile + sh;
  for (uint32_t m = 0; m < gm; ++m) {
    const CopyRegion* M = R + m;
    uint32_t cm, inner, nd;
    uint64_t d0;
    if (!kSw && m < 64u) {
      cm = __builtin_amdgcn_readlane(m_cm, m);
      inner = __builtin_amdgcn_readlane(m_inner, m);
      nd = __builtin_amdgcn_readlane(m_nd, m);
      // readlane returns an int: each half goes through uint32_t, so the
      // low half is not sign-extended into the high one.
      const uint32_t dlo = __builtin_amdgcn_readlane(uint32_t(m_dst), m);
      const uint32_t dhi = __builtin_amdgcn_readlane(uint32_t(m_dst >> 32), m);
      d0 = (uint64_t(dhi) << 32) | dlo;
    } else {
      cm = uint32_t(M->src_off - lo);
      inner = M->inner;
      nd = n_dst_of(M);
      d0 = reinterpret_cast<uint64_t>(pool_ptr(a, dst_pool(M, 0))) + M->dst_off;
    }
    const uint32_t nbytes = T * inner;
    const uint32_t G = low_granule((sh + cm) | S | inner);
    for (uint32_t j = 0; j < nd; ++j) {
      char* D = (j == 0 ? (char*)(global_char*)d0 : static_cast<char*>(pool_ptr(a, dst_pool(M, j))) + M->dst_off) +
                uint64_t(r0) * inner;
      if (kSw && swz) {
        switch (G) {
          case 4: group_store<4, true>(D, lds, cm, S, inner, nbytes, tid); break;
          case 2: group_store<2, true>(D, lds, cm, S, inner, nbytes, tid); break;
          default: group_store<1, true>(D, lds, cm, S, inner, nbytes, tid); break;
        }
      } else {
        switch (G) {
          case 16: group_store<16, false>(D, lds, cm, S, inner, nbytes, tid); break;
          case 8: group_store<8, false>(D, lds, cm, S, inner, nbytes, tid); break;
          case 4: group_store<4, false>(D, lds, cm, S, inner, nbytes, tid); break;
          case 2: group_store<2, false>(D, lds, cm, S, inner, nbytes, tid); break;
          default: group_store<1, false>(D, lds, cm, S, inner, nbytes, tid); break;
        }
      }
    }
  }
}

template <bool kSw, class Args>
__device__ __forceinline__ void thin_group_unit(const Args& a, const CopyRegion* R, uint32_t ul, char* tile) {
  const uint32_t gm = (R->flags >> 16) & 255u;
  uint64_t lo = R->src_off, hi = R->src_off + R->inner;
  for (uint32_t m = 1; m < gm; ++m) {
    lo = min(lo, R[m].src_off);
    hi = max(hi, R[m].src_off + R[m].inner);
  }
  thin_group_body<kSw && RS_THIN_SWIZZLE>(a, R, ul, tile, lo, uint32_t(hi - lo));
}

// Thin sibling groups loaded whole (launches of their own: this path needs
// more registers than the thin kernel's others).  kSw: groups with a member
// whose LDS reads are 4 bytes or narrower (swizzled LDS slots).
template <bool kSw, class Args>
__global__ __launch_bounds__(kThreads) void rs_thin_group_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char tile[kGroupTile + 16];
  const uint32_t unit = unit_of_block<RS_THIN_XCD_CHUNK != 0>(blockIdx.x, gridDim.x, RS_THIN_XCD_CHUNK);
  const CopyRegion* R = find_region<CopyRegion>(a, unit);
  thin_group_unit<kSw>(a, R, unit - R->unit_begin, tile);
}

template <class Args>
__global__ __launch_bounds__(kThreads) void rs_thin_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char tile[kThinTile + 16];
  const uint32_t tid = threadIdx.x;
  const uint32_t unit = unit_of_block<RS_THIN_XCD_CHUNK != 0>(blockIdx.x, gridDim.x, RS_THIN_XCD_CHUNK);
  const CopyRegion* R = find_region<CopyRegion>(a, unit);
  uint32_t ul = unit - R->unit_begin;
  const uint32_t gm = (R->flags >> 16) & 255u;
  if (gm > 1) {
    // Sibling group (same source rows, different columns): its units are
    // taken member-fastest, so the workgroups reading the same source rows
    // run together and share the fetched lines.
    const uint32_t m = R->flags >> 24;
    const uint32_t nu = (R->rows + R->rows_per_unit - 1) / R->rows_per_unit;
    const uint32_t local = ul + m * nu;
    R = R - m + local % gm;
    ul = local / gm;
  }
  const uint64_t src_off = R->src_off, dst_off = R->dst_off;
  const uint64_t s0 = R->sstr[0], s1 = R->sstr[1], s2 = R->sstr[2];
  const uint64_t d0 = R->dstr[0], d1 = R->dstr[1], d2 = R->dstr[2];
  const uint32_t e0 = R->e0, e1 = R->e1, rows = R->rows, inner = R->inner;
  const uint32_t rpu = R->rows_per_unit, flags = R->flags;
  const uint32_t nd = n_dst_of(R);
  const uint32_t nouter = flags & kFlagOuterMask;
  const char* sp = static_cast<const char*>(pool_ptr(a, src_pool(R))) + src_off;

  uint32_t al = (flags >> 8) & 15u;
  al |= uint32_t(reinterpret_cast<uintptr_t>(sp) & 15u);
  for (uint32_t j = 0; j < nd; ++j)
    al |= uint32_t((reinterpret_cast<uintptr_t>(pool_ptr(a, dst_pool(R, j))) + dst_off) & 15u);
  const uint32_t g = low_granule(al);
  const uint32_t gpr = inner / g;

  const uint32_t r0 = ul * rpu;
  const uint32_t r1 = min(r0 + rpu, rows);
  const uint32_t T = r1 - r0;
  const uint32_t nbytes = T * inner;
  const uint32_t total = T * gpr;

  if (flags & kFlagDstPacked) {
    // Gather strided source rows into LDS (congruent with the first
    // destination mod 16), then write the contiguous destination block.
    const char* D0 = static_cast<const char*>(pool_ptr(a, dst_pool(R, 0))) + dst_off + uint64_t(r0) * inner;
    const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(D0) & 15u);
    for (uint32_t f = tid; f < total; f += kThreads) {
      const uint32_t row = f / gpr;
      const uint32_t k = f - row * gpr;
      const uint64_t so = row_off(r0 + row, e0, e1, nouter, s0, s1, s2);
      copy_granule(tile + sh + row * inner + k * g, sp + so + uint64_t(k) * g, g);
    }
    __syncthreads();
    for (uint32_t j = 0; j < nd; ++j) {
      char* Dj = static_cast<char*>(pool_ptr(a, dst_pool(R, j))) + dst_off + uint64_t(r0) * inner;
      if ((reinterpret_cast<uintptr_t>(Dj) & 15u) == sh)
        block_copy_congruent(Dj, tile + sh, nbytes, tid);
      else
        block_copy_bytes(Dj, tile + sh, nbytes, tid);
    }
  } else if (flags & kFlagSrcPacked) {
    // Read the contiguous source block with vectors, scatter rows from LDS.
    const char* S = sp + uint64_t(r0) * inner;
    const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(S) & 15u);
    block_copy_congruent(tile + sh, S, nbytes, tid);
    __syncthreads();
    for (uint32_t f = tid; f < total; f += kThreads) {
      const uint32_t row = f / gpr;
      const uint32_t k = f - row * gpr;
      const uint64_t dof = row_off(r0 + row, e0, e1, nouter, d0, d1, d2);
      for (uint32_t j = 0; j < nd; ++j) {
        char* d = static_cast<char*>(pool_ptr(a, dst_pool(R, j))) + dst_off + dof + uint64_t(k) * g;
        copy_granule(d, tile + sh + row * inner + k * g, g);
      }
    }
  } else {
    // Neither side contiguous across rows: granule by granule.
    for (uint32_t f = tid; f < total; f += kThreads) {
      const uint32_t row = f / gpr;
      const uint32_t k = f - row * gpr;
      const uint64_t so = row_off(r0 + row, e0, e1, nouter, s0, s1, s2);
      const uint64_t dof = row_off(r0 + row, e0, e1, nouter, d0, d1, d2);
      for (uint32_t j = 0; j < nd; ++j) {
        char* d = static_cast<char*>(pool_ptr(a, dst_pool(R, j))) + dst_off + dof + uint64_t(k) * g;
        copy_granule(d, sp + so + uint64_t(k) * g, g);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// tiny (wave prefix sum over many small regions)
// ---------------------------------------------------------------------------

template <class Args>
__device__ __forceinline__ uint32_t region_granule(const Args& a, const CopyRegion* R) {
  uint32_t al = (R->flags >> 8) & 15u;
  al |= uint32_t((reinterpret_cast<uintptr_t>(pool_ptr(a, R->src_ptr)) + R->src_off) & 15u);
  for (uint32_t j = 0; j < R->n_dst; ++j)
    al |= uint32_t((reinterpret_cast<uintptr_t>(pool_ptr(a, R->dst_ptr[j])) + R->dst_off) & 15u);
  return low_granule(al);
}

// One granule of g bytes (g in {1,2,4,8,16}, p g-aligned) into / out of a
// 16-byte register.
__device__ __forceinline__ u32x4 load_granule(const char* p, uint32_t g) {
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  switch (g) {
    case 16: v = *reinterpret_cast<const u32x4*>(p); break;
    case 8: {
      const u32x2 w = *reinterpret_cast<const u32x2*>(p);
      v.x = w.x;
      v.y = w.y;
      break;
    }
    case 4: v.x = *reinterpret_cast<const uint32_t*>(p); break;
    case 2: v.x = *reinterpret_cast<const uint16_t*>(p); break;
    default: v.x = uint8_t(*p); break;
  }
  return v;
}
__device__ __forceinline__ void store_granule(char* p, uint32_t g, u32x4 v) {
  switch (g) {
    case 16: *reinterpret_cast<u32x4*>(p) = v; break;
    case 8: *reinterpret_cast<u32x2*>(p) = u32x2{v.x, v.y}; break;
    case 4: *reinterpret_cast<uint32_t*>(p) = v.x; break;
    case 2: *reinterpret_cast<uint16_t*>(p) = uint16_t(v.x); break;
    default: *p = char(v.x); break;
  }
}

// Each lane owns one region (its granule size and granule count go to LDS);
// a wave-level inclusive scan of the counts numbers the wave's granules, and
// the 64 lanes then walk them together, each finding its granule's region by
// a binary search over the wave's starts, kTinyInFlight granules per lane at
// a time so their loads overlap.
constexpr int kTinyInFlight = 4;

template <class Args>
__global__ __launch_bounds__(kThreads) void rs_tiny_kernel(Args a) {
  __shared__ uint32_t start[kThreads];
  __shared__ uint32_t gpr_of[kThreads];
  __shared__ uint8_t gsize[kThreads];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, wave = tid >> 6;
  const CopyRegion* regs = static_cast<const CopyRegion*>(a.regions);
  const uint32_t ri = blockIdx.x * kThreads + tid;
  uint32_t cnt = 0, g = 1, gpr = 0;
  if (ri < a.n_regions) {
    const CopyRegion* R = regs + ri;
    g = region_granule(a, R);
    gpr = R->inner / g;
    cnt = R->rows * gpr;
  }
  // Inclusive scan of the per-lane granule counts across the wave.
  uint32_t scan = cnt;
  for (uint32_t off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(scan, off, 64);
    if (lane >= off) scan += y;
  }
  const uint32_t total = __shfl(scan, 63, 64);
  start[tid] = scan - cnt;
  gpr_of[tid] = gpr;
  gsize[tid] = uint8_t(g);
  __syncthreads();
  const uint32_t* ws = start + wave * 64;
  const uint32_t base = blockIdx.x * kThreads + wave * 64;
  for (uint32_t f0 = lane; f0 < total; f0 += kTinyInFlight * 64) {
    u32x4 v[kTinyInFlight];
    uint32_t owner[kTinyInFlight];
    uint64_t dofs[kTinyInFlight];
#pragma unroll
    for (int u = 0; u < kTinyInFlight; ++u) {
      const uint32_t f = f0 + u * 64;
      owner[u] = 0;
      dofs[u] = 0;
      if (f < total) {
        // Last lane whose start <= f (empty regions share starts; take the last).
        uint32_t lo = 0, hi = 64;
        while (hi - lo > 1) {
          const uint32_t mid = (lo + hi) >> 1;
          if (ws[mid] <= f) lo = mid; else hi = mid;
        }
        owner[u] = lo;
        const CopyRegion* R = regs + base + lo;
        const uint32_t gl = gsize[wave * 64 + lo], gp = gpr_of[wave * 64 + lo];
        const uint32_t local = f - ws[lo];
        const uint32_t row = local / gp;
        const uint32_t k = local - row * gp;
        const uint32_t nouter = R->flags & kFlagOuterMask;
        const uint64_t so = row_off(row, R->e0, R->e1, nouter, R->sstr[0], R->sstr[1], R->sstr[2]);
        dofs[u] = R->dst_off + row_off(row, R->e0, R->e1, nouter, R->dstr[0], R->dstr[1], R->dstr[2]) +
                  uint64_t(k) * gl;
        v[u] = load_granule(static_cast<const char*>(pool_ptr(a, R->src_ptr)) + R->src_off + so + uint64_t(k) * gl, gl);
      }
    }
#pragma unroll
    for (int u = 0; u < kTinyInFlight; ++u) {
      if (f0 + u * 64 < total) {
        const CopyRegion* R = regs + base + owner[u];
        const uint32_t gl = gsize[wave * 64 + owner[u]];
        for (uint32_t j = 0; j < R->n_dst; ++j)
          store_granule(static_cast<char*>(pool_ptr(a, R->dst_ptr[j])) + dofs[u], gl, v[u]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// mx: BF16 -> MXFP8 (E4M3 elements, E8M0 block scales), quantised on install
// ---------------------------------------------------------------------------

// Shared exponent of a block from the bf16 bits of its largest magnitude:
// X = clamp(floor(log2(amax)) - 8, -127, 127); an all-zero block gives -127.
__device__ __forceinline__ int shared_exp(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  const uint32_t E = amax_bits >> 7;
  const int e = E ? int(E) - 127 : (31 - __builtin_clz(amax_bits & 0x7Fu)) - 133;
  const int X = e - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Four E4M3 codes (one 32-bit word, element i in byte i) of two words of
// packed bf16 (w0, w1) with magnitudes (m0, m1) = w & 0x7FFF7FFF.  The
// magnitude is first clamped to T = 448 * 2^X (bf16 magnitudes order like
// their bit patterns, and T is a bf16 value), so the conversion saturates;
// v_cvt_scalef32_pk_fp8_bf16 then gives round-to-nearest-even of v / 2^X,
// exactly, for every finite bf16 (subnormals included).
__device__ __forceinline__ uint32_t e4m3x4(uint32_t w0, uint32_t w1, uint32_t m0, uint32_t m1,
                                           uint32_t T2, float scale) {
  const uint32_t c0 = (w0 & 0x80008000u) | pk_min_u16(m0, T2);
  const uint32_t c1 = (w1 & 0x80008000u) | pk_min_u16(m1, T2);
  s16x2 r = s16x2{0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, c0), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, c1), scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

#ifndef RS_MX_MIN_WAVES
#define RS_MX_MIN_WAVES 1  // occupancy floor (waves per SIMD) the register allocator must keep
#endif
#ifndef RS_MX_FUNNEL
#define RS_MX_FUNNEL 1     // sources whose rows are not 16-byte aligned: funnel-shifted 16-byte loads
#endif
#ifndef RS_MX_LINES
#define RS_MX_LINES 1      // such sources staged as aligned lines in LDS, groups rebuilt in phase 2
#endif
#ifndef RS_MX_LDS_AUX
#define RS_MX_LDS_AUX 2    // cache policy of the direct-to-LDS loads (2: non-temporal)
#endif


// Block codes of one lane's two adjacent 8-element groups xa, xb (bf16
// pairs, 16 elements, half a block; zeros past the row end).  The two lanes
// of a block call this together: the block's amax is exchanged between them
// with a DPP quad permute.
struct MxCodes {
  u32x4 v;           // E4M3 codes of the 16 elements, element i in byte i
  uint8_t scale;     // E8M0 block scale
};

__device__ __forceinline__ MxCodes mx_encode(u32x4 xa, u32x4 xb) {
  const uint32_t a0 = xa.x & 0x7FFF7FFFu, a1 = xa.y & 0x7FFF7FFFu, a2 = xa.z & 0x7FFF7FFFu,
                 a3 = xa.w & 0x7FFF7FFFu;
  const uint32_t b0 = xb.x & 0x7FFF7FFFu, b1 = xb.y & 0x7FFF7FFFu, b2 = xb.z & 0x7FFF7FFFu,
                 b3 = xb.w & 0x7FFF7FFFu;
  const uint32_t mm = pk_max_u16(pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3)),
                                 pk_max_u16(pk_max_u16(b0, b1), pk_max_u16(b2, b3)));
  uint32_t amax = max(mm & 0xFFFFu, mm >> 16);
  // quad_perm [1,0,3,2]: the partner lane holds the other half of the block
  amax = max(amax, uint32_t(__builtin_amdgcn_update_dpp(0, int(amax), 0xB1, 0xF, 0xF, true)));
  const bool bad = amax >= 0x7F80u;   // a NaN or Inf in the block
  const int X = shared_exp(amax);
  const uint32_t T = (uint32_t(X + 135) << 7) | 0x60u;   // bf16 bits of 448 * 2^X
  const uint32_t T2 = T | (T << 16);
  const float sc = __builtin_amdgcn_ldexpf(1.0f, X);
  MxCodes c;
  c.v.x = e4m3x4(xa.x, xa.y, a0, a1, T2, sc);
  c.v.y = e4m3x4(xa.z, xa.w, a2, a3, T2, sc);
  c.v.z = e4m3x4(xb.x, xb.y, b0, b1, T2, sc);
  c.v.w = e4m3x4(xb.z, xb.w, b2, b3, T2, sc);
  if (bad) c.v = u32x4{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
  c.scale = bad ? uint8_t(0xFF) : uint8_t(X + 127);
  return c;
}

// One work unit of the MXFP8 kernel: nr rows (nr <= kMxSlots / P) of inner
// elements, staged in LDS with row i at slot i * P (one 16-byte slot per
// 8-element group), P = mx_row_pitch(inner).  kOneRow: the unit is a single
// row, whose addresses are uniform across the workgroup.  kPitch: P is not a
// power of two, so slot s belongs to row s / P (a multiply by a reciprocal
// that is exact for every slot index) instead of s >> log2(P).
// The fields of an MXFP8 region a work unit needs, read from the table once
// at kernel entry, before any branch or store: a table read after a store is
// a vector load (the compiler cannot rule out that the store changed the
// table), and its wait would also wait for the stores already issued.
struct MxFields {
  uint64_t src_off, dst_off, sc_off;
  uint64_t s0, s1, s2, d0, d1, d2, c0, c1, c2;
  uint32_t e0, e1, inner, nouter, sc_inner, nd, split;
  const char* sp;       // source buffer + src_off
  char* dk;             // first destination's element and scale buffers
  char* sk;
  const char* sp2;      // two-piece regions: second source + src2_off, and its strides
  uint64_t t0, t1, t2;
};

template <class Args>
__device__ __forceinline__ MxFields mx_fields(const Args& a, const MxRegion* R) {
  MxFields f;
  f.src_off = R->src_off;
  f.dst_off = R->dst_off;
  f.sc_off = R->sc_off;
  f.s0 = R->sstr[0]; f.s1 = R->sstr[1]; f.s2 = R->sstr[2];
  f.d0 = R->dstr[0]; f.d1 = R->dstr[1]; f.d2 = R->dstr[2];
  f.c0 = R->scstr[0]; f.c1 = R->scstr[1]; f.c2 = R->scstr[2];
  f.e0 = R->e0;
  f.e1 = R->e1;
  f.inner = R->inner;
  f.nouter = R->flags & kFlagOuterMask;
  f.sc_inner = R->sc_inner;
  f.nd = n_dst_of(R);
  f.sp = static_cast<const char*>(pool_ptr(a, src_pool(R))) + f.src_off;
  f.dk = static_cast<char*>(pool_ptr(a, dst_pool(R, 0)));
  f.sk = static_cast<char*>(pool_ptr(a, sc_pool(R, 0)));
  f.split = R->split;
  f.sp2 = nullptr;
  f.t0 = f.t1 = f.t2 = 0;
  if (f.split < f.inner) {
    f.sp2 = static_cast<const char*>(pool_ptr(a, pool_field(R, 2 + 2 * kMaxFan))) + R->src2_off;
    f.t0 = R->sstr2[0];
    f.t1 = R->sstr2[1];
    f.t2 = R->sstr2[2];
  }
  return f;
}

// Eight bf16 elements as a 16-byte group: the first n of v, the rest zero.
__device__ __forceinline__ u32x4 pack8(const uint16_t* v, uint32_t n) {
  uint32_t w[4];
#pragma unroll
  for (uint32_t i = 0; i < 4; ++i)
    w[i] = (2 * i < n ? uint32_t(v[2 * i]) : 0u) | (2 * i + 1 < n ? uint32_t(v[2 * i + 1]) << 16 : 0u);
  return u32x4{w[0], w[1], w[2], w[3]};
}

// The n (1..8) elements at q as a zero-filled group.  Every load reads one
// of the n (element min(i, n - 1)), so all eight are issued before the first
// wait instead of one after another.
__device__ __forceinline__ u32x4 gather8(const uint16_t* q, uint32_t n) {
  uint16_t v[8];
#pragma unroll
  for (uint32_t i = 0; i < 8; ++i) v[i] = q[min(i, n - 1u)];
  return pack8(v, n);
}

// The first n (clamped to 0..8) of the eight bf16 elements of x, the rest zero.
__device__ __forceinline__ u32x4 keep_elems(u32x4 x, int n) {
  auto keep = [&](uint32_t w, int i) -> uint32_t {   // dword i holds elements 2i, 2i + 1
    return n >= 2 * i + 2 ? w : (n == 2 * i + 1 ? (w & 0xFFFFu) : 0u);
  };
  return u32x4{keep(x.x, 0), keep(x.y, 1), keep(x.z, 2), keep(x.w, 3)};
}

// Rows of a pitched unit whose offsets the second MXFP8 kernel keeps in LDS.
constexpr uint32_t kMxRowTab = 64;
static_assert(mx_max_pitched_rows() <= kMxRowTab, "a pitched unit's rows fit the row table");

template <bool kOneRow, bool kFan1, bool kTwo = false, bool kPitch = false, class Args>
__device__ __forceinline__ void mx_unit(const Args& a, const MxRegion* R, const MxFields& f, uint32_t r0,
                                        uint32_t nr, u32x4* stage, uint8_t* sc_stage, uint64_t* rt = nullptr) {
  constexpr uint32_t K = kMxSlots / kMxThreads;
  const uint32_t tid = threadIdx.x;
  const uint64_t s0 = f.s0, s1 = f.s1, s2 = f.s2;
  const uint64_t d0 = f.d0, d1 = f.d1, d2 = f.d2;
  const uint64_t c0 = f.c0, c1 = f.c1, c2 = f.c2;
  const uint32_t e0 = f.e0, e1 = f.e1, inner = f.inner;
  const uint32_t nouter = f.nouter;
  const uint32_t sc_inner = f.sc_inner, nd = f.nd;
  const uint64_t dst_off_r = f.dst_off, sc_off_r = f.sc_off;
  const char* sp = f.sp;
  char* const dk = f.dk;
  char* const sk = f.sk;
  const uint64_t so1 = kOneRow ? row_off(r0, e0, e1, nouter, s0, s1, s2) : 0;
  const uint64_t do1 = kOneRow ? row_off(r0, e0, e1, nouter, d0, d1, d2) : 0;
  const uint32_t lg = mx_slot_shift(inner), Lp = kPitch ? mx_row_pitch(inner) : 1u << lg;
  const uint32_t ng = (inner + 7u) >> 3;
  // Row and slot-in-row of slot s (and of scale byte t, 4 per 4 slots):
  // ceil(2^32 / P) times s, high word, is s / P for s < kMxSlots and
  // P <= kMxSlots (likewise for P / 4 and t < kMxSlots / 4).
  const uint32_t mrow = kPitch ? 0xFFFFFFFFu / Lp + 1u : 0u;
  const uint32_t msc = kPitch ? 0xFFFFFFFFu / (Lp >> 2) + 1u : 0u;
  auto row_of = [&](uint32_t s) -> uint32_t { return kPitch ? __umulhi(s, mrow) : s >> lg; };
  auto col_of = [&](uint32_t s, uint32_t rl) -> uint32_t { return kPitch ? s - rl * Lp : s & (Lp - 1u); };
  // Byte offsets of row rl of the unit (source from sp; destination and
  // scale including the region's offsets).  kPitch: computed once per row,
  // by one lane each, into the LDS row table rt, and read from there (no
  // division per slot).
  if (kPitch) {
    if (tid < nr) {
      rt[tid] = row_off(r0 + tid, e0, e1, nouter, s0, s1, s2);
      rt[kMxRowTab + tid] = dst_off_r + row_off(r0 + tid, e0, e1, nouter, d0, d1, d2);
      rt[2 * kMxRowTab + tid] = sc_off_r + row_off(r0 + tid, e0, e1, nouter, c0, c1, c2);
    }
    __syncthreads();
  }
  auto src_row = [&](uint32_t rl) -> uint64_t {
    return kPitch ? rt[rl] : kOneRow ? so1 : row_off(r0 + rl, e0, e1, nouter, s0, s1, s2);
  };
  auto dst_row = [&](uint32_t rl) -> uint64_t {
    return kPitch ? rt[kMxRowTab + rl] : dst_off_r + (kOneRow ? do1 : row_off(r0 + rl, e0, e1, nouter, d0, d1, d2));
  };
  auto sc_row = [&](uint32_t rl) -> uint64_t {
    return kPitch ? rt[2 * kMxRowTab + rl] : sc_off_r + row_off(r0 + rl, e0, e1, nouter, c0, c1, c2);
  };

  // Phase 1: every group of the unit into its LDS slot.  Whole, 16-byte
  // aligned groups load straight into LDS; a partial or misaligned group is
  // gathered element by element (zero-filled) and written by its lane.
  // Source rows not 16-byte aligned (a source shard boundary off the 8-
  // element grid): each group is two aligned 16-byte loads joined by a
  // funnel shift, half the unit at a time, so all of a lane's loads of a
  // half are in flight together; groups whose lines would reach past the
  // row (its first and last) are gathered element by element.
  const bool mis_rows =
      !kTwo && RS_MX_FUNNEL &&
      ((reinterpret_cast<uintptr_t>(sp) | (kOneRow ? so1 : (s0 | (nouter >= 2 ? s1 : 0) | (nouter >= 3 ? s2 : 0)))) &
       15u) != 0;
  // Line layout (such rows when a row's slots hold its lines with two to
  // spare and every row's two partial lines have a lane): slot j of row i
  // holds the row's aligned source line j (row byte x at slot byte
  // h_i + x, h_i = row address mod 16), whole lines by direct-to-LDS loads
  // and the in-row elements of the partial first and last lines by their
  // lanes after the wait; phase 2 rebuilds each group with funnel shifts.
  const bool lines = RS_MX_LINES && mis_rows && ng + 2u <= Lp && 2u * nr <= kMxThreads;
  if (lines) {
    uint16_t pe[7];
    uint32_t pb = 0, pn = 0;   // LDS byte of the first element, element count
    if (tid < 2u * nr) {
      const uint32_t rl = tid >> 1, side = tid & 1u;
      const char* rs = sp + src_row(rl);
      const uint32_t h = uint32_t(reinterpret_cast<uintptr_t>(rs) & 15u), nb = 2u * inner;
      const uint32_t jl = (h + nb - 1u) >> 4;   // last line
      uint32_t b0 = 0, b1 = 0;                  // row bytes [b0, b1) of this partial line
      if (side == 0) {
        if (h != 0 || nb < 16u) b1 = min(16u - h, nb);  // a partial first line
      } else if (jl > 0 && ((h + nb) & 15u) != 0) {
        b0 = 16u * jl - h;                               // a partial last line
        b1 = nb;
      }
      pn = (b1 - b0) >> 1;
      pb = (kPitch ? rl * Lp : rl << lg) * 16u + h + b0;
      const uint16_t* q = reinterpret_cast<const uint16_t*>(rs + b0);
#pragma unroll
      for (uint32_t e = 0; e < 7; ++e) pe[e] = e < pn ? q[e] : uint16_t(0);
    }
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) {
      const uint32_t s = k * kMxThreads + tid;
      const uint32_t rl = row_of(s), j = col_of(s, rl);
      if (rl < nr) {
        const char* rs = sp + src_row(rl);
        const int x0 = int(16u * j) - int(reinterpret_cast<uintptr_t>(rs) & 15u);   // row byte at line j
        if (x0 >= 0 && uint32_t(x0) + 16u <= 2u * inner)
          __builtin_amdgcn_global_load_lds(rs + x0, (lds_void*)(stage + k * kMxThreads + (tid & ~63u)), 16, 0,
                                           RS_MX_LDS_AUX);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    uint16_t* st16p = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(stage) + pb);
#pragma unroll
    for (uint32_t e = 0; e < 7; ++e)
      if (e < pn) st16p[e] = pe[e];
  } else if (mis_rows) {
#pragma unroll
    for (uint32_t half = 0; half < 2; ++half) {
      u32x4 A[K / 2], B[K / 2];
      uint32_t sh[K / 2];
      bool fun[K / 2];
#pragma unroll
      for (uint32_t kk = 0; kk < K / 2; ++kk) {
        const uint32_t k = half * (K / 2) + kk;
        const uint32_t s = k * kMxThreads + tid;
        const uint32_t rl = row_of(s), g = col_of(s, rl);
        fun[kk] = false;
        sh[kk] = 0;
        if (rl < nr && g < ng) {
          const char* rs = sp + src_row(rl);
          const char* p = rs + uint64_t(g) * 16u;
          const uint32_t r = uint32_t(reinterpret_cast<uintptr_t>(p) & 15u);
          const char* L = p - r;
          if (g * 8u + 8u <= inner && L >= rs && L + (r ? 32u : 16u) <= rs + 2u * inner) {
            A[kk] = *reinterpret_cast<const u32x4*>(L);
            if (r) B[kk] = *reinterpret_cast<const u32x4*>(L + 16u);
            fun[kk] = true;
            sh[kk] = r;
          }
        }
      }
#pragma unroll
      for (uint32_t kk = 0; kk < K / 2; ++kk) {
        const uint32_t k = half * (K / 2) + kk;
        const uint32_t s = k * kMxThreads + tid;
        const uint32_t rl = row_of(s), g = col_of(s, rl);
        if (fun[kk]) {
          stage[s] = sh[kk] ? funnel16(A[kk], B[kk], sh[kk]) : A[kk];
        } else if (rl < nr && g < ng) {
          stage[s] = gather8(reinterpret_cast<const uint16_t*>(
                                 sp + src_row(rl) +
                                 uint64_t(g) * 16u),
                             min(inner - g * 8u, 8u));
        }
      }
    }
  } else
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) {
    const uint32_t s = k * kMxThreads + tid;
    const uint32_t rl = row_of(s), g = col_of(s, rl);
    if (kTwo && rl < nr && g < ng) {
      // Two pieces: each element from the piece that holds its column (the
      // column clamped to the row, so all eight loads are issued at once).
      const char* p1 = sp + row_off(r0 + rl, e0, e1, nouter, s0, s1, s2);
      const char* p2 = f.sp2 + row_off(r0 + rl, e0, e1, nouter, f.t0, f.t1, f.t2);
      uint16_t v[8];
#pragma unroll
      for (uint32_t i = 0; i < 8; ++i) {
        const uint32_t c = min(g * 8u + i, inner - 1u);
        v[i] = *reinterpret_cast<const uint16_t*>(c < f.split ? p1 + 2u * c : p2 + 2u * (c - f.split));
      }
      stage[s] = pack8(v, min(inner - g * 8u, 8u));
    } else if (rl < nr && g < ng) {
      const char* p = sp + src_row(rl) +
                      uint64_t(g) * 16u;
      if (g * 8u + 8u <= inner && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
        __builtin_amdgcn_global_load_lds(p, (lds_void*)(stage + k * kMxThreads + (tid & ~63u)), 16, 0,
                                         RS_MX_LDS_AUX);
      } else {
        stage[s] = gather8(reinterpret_cast<const uint16_t*>(p), min(inner - g * 8u, 8u));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Phase 2: each lane quantises two adjacent slots (a pair of lanes per
  // block) and stores their 16 code bytes to every replica.
#pragma unroll
  for (uint32_t k = 0; k < K / 2; ++k) {
    const uint32_t s = 2 * (k * kMxThreads + tid);
    const uint32_t rl = row_of(s), g = col_of(s, rl);
    const uint32_t col = g * 8u;
    const int nvalid = rl < nr ? int(min(inner, col + 16u)) - int(min(inner, col)) : 0;
    u32x4 xa = nvalid > 0 ? stage[s] : u32x4{0u, 0u, 0u, 0u};
    u32x4 xb = nvalid > 8 ? stage[s + 1] : u32x4{0u, 0u, 0u, 0u};
    if (kPitch && lines && nvalid > 0) {
      // Groups g, g + 1 of the row read straight from bytes h .. h + 31 of
      // its lines g .. g + 2 (unaligned LDS reads), elements past the row's
      // end zeroed.
      const uint32_t h = uint32_t((reinterpret_cast<uintptr_t>(sp) + src_row(rl)) & 15u);
      const char* lb = reinterpret_cast<const char*>(stage) + 16u * s + h;
      __builtin_memcpy(&xa, lb, 16);
      if (nvalid > 8) __builtin_memcpy(&xb, lb + 16, 16);
      xa = keep_elems(xa, nvalid);
      xb = keep_elems(xb, nvalid - 8);
    } else if (lines && nvalid > 0) {
      // Groups g, g + 1 of the row: bytes h .. h + 31 of lines g .. g + 2,
      // elements past the row's end zeroed.
      const char* rs = sp + src_row(rl);
      const uint32_t h = uint32_t(reinterpret_cast<uintptr_t>(rs) & 15u);
      if (h) {
        const u32x4 L2 = nvalid > 8 ? stage[s + 2] : u32x4{0u, 0u, 0u, 0u};
        const u32x4 L0 = xa, L1 = stage[s + 1];
        xa = funnel16(L0, L1, h);
        xb = nvalid > 8 ? funnel16(L1, L2, h) : u32x4{0u, 0u, 0u, 0u};
      }
      xa = keep_elems(xa, nvalid);
      xb = keep_elems(xb, nvalid - 8);
    }
    const MxCodes c = mx_encode(xa, xb);
    if (nvalid > 0) {
      const uint64_t doff = dst_row(rl) + col;
      for (uint32_t j = 0; j < (kFan1 ? 1u : nd); ++j) {
        char* d = (kFan1 ? dk : static_cast<char*>(pool_ptr(a, dst_pool(R, j)))) + doff;
        if (nvalid == 16 && (reinterpret_cast<uintptr_t>(d) & 15u) == 0) {
          __builtin_nontemporal_store(c.v, reinterpret_cast<u32x4*>(d));
        } else {
          const uint32_t w[4] = {c.v.x, c.v.y, c.v.z, c.v.w};
          for (int i = 0; i < 16; ++i)
            if (i < nvalid) d[i] = char((w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        }
      }
      if ((g & 3u) == 0) sc_stage[s >> 2] = c.scale;
    }
  }
  // Phase 3: the unit's block scales, block b of row i at LDS byte
  // i * P / 4 + b, written by consecutive lanes.
  __syncthreads();
  const uint32_t nb = (inner + 31u) >> 5;
  for (uint32_t t = tid; t < kMxSlots / 4; t += kMxThreads) {
    const uint32_t rl = kPitch ? __umulhi(t, msc) : t >> (lg - 2);
    const uint32_t b = kPitch ? t - rl * (Lp >> 2) : t & ((Lp >> 2) - 1u);
    if (rl < nr && b < nb) {
      const uint64_t so = sc_row(rl) + uint64_t(b) * sc_inner;
      const char v = char(sc_stage[t]);
      for (uint32_t j = 0; j < (kFan1 ? 1u : nd); ++j)
        __builtin_nontemporal_store(v, (kFan1 ? sk : static_cast<char*>(pool_ptr(a, sc_pool(R, j)))) + so);
    }
  }
}

template <bool kOneRow, class Args>
__device__ __forceinline__ void mx_unit_fan(const Args& a, const MxRegion* R, const MxFields& f,
                                            uint32_t r0, uint32_t nr, u32x4* stage, uint8_t* sc_stage) {
  if (f.nd == 1)
    mx_unit<kOneRow, true>(a, R, f, r0, nr, stage, sc_stage);
  else
    mx_unit<kOneRow, false>(a, R, f, r0, nr, stage, sc_stage);
}

// kAux: launches of the two-piece regions and of those whose rows take a
// pitch that is not a power of two (mx_row_pitch; a two-piece region, one
// block wide, never does); every unit, one row or several, on the multi-row
// path.
template <bool kAux, class Args>
__global__ __launch_bounds__(kMxThreads, RS_MX_MIN_WAVES) void rs_mx_kernel(Args a) {
  __shared__ u32x4 stage[kMxSlots];
  __shared__ __attribute__((aligned(16))) uint8_t sc_stage[kMxSlots / 4];
  const uint32_t unit = unit_of_block<RS_MX_XCD_MAP != 0>(blockIdx.x, gridDim.x, RS_MX_XCD_CHUNK);
  const MxRegion* R = find_region<MxRegion>(a, unit);
  const uint32_t r0 = (unit - R->unit_begin) * R->rows_per_unit;
  const uint32_t nr = min(R->rows_per_unit, R->rows - r0);
  const MxFields f = mx_fields(a, R);
  if (kAux) {
    __shared__ uint64_t rt[3 * kMxRowTab];
    if (f.split < f.inner)
      mx_unit<false, false, true>(a, R, f, r0, nr, stage, sc_stage);
    else if (f.nd == 1)
      mx_unit<false, true, false, true>(a, R, f, r0, nr, stage, sc_stage, rt);
    else
      mx_unit<false, false, false, true>(a, R, f, r0, nr, stage, sc_stage, rt);
  } else if (nr == 1) {
    mx_unit_fan<true>(a, R, f, r0, nr, stage, sc_stage);
  } else {
    mx_unit_fan<false>(a, R, f, r0, nr, stage, sc_stage);
  }
}

}  // namespace

// Bulk workgroups resident per CU.  The copy streams best with fewer than
// the register file would allow (on MI355X, with spread groups, 4 to 6 per CU
// tie, 8 is about 1 % slower and 3 about 14 % slower), so each bulk launch
// asks for enough dynamic LDS, which the kernel never touches, to leave room
// for only this many.  0 = no cap.
#ifndef RS_BULK_RESIDENT
#define RS_BULK_RESIDENT 5
#endif
constexpr int kMaxDevices = 64;

// Dynamic LDS bytes per bulk workgroup on device `dev` (cached).
size_t bulk_lds_pad(int dev) {
  static std::atomic<int> cache[kMaxDevices];   // 0: not yet known; else pad + 1
  if (RS_BULK_RESIDENT <= 0) return 0;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return size_t(c - 1);
  }
  int per_cu = 0, per_wg = 0;
  if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
      hipDeviceGetAttribute(&per_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      per_cu <= 0 || per_wg <= 0)
    return 0;
  // The kernel's own static LDS (kMisTile) counts toward the per-workgroup share.
  int pad = ((per_cu / RS_BULK_RESIDENT) & ~511) - int(kMisTile);
  if (pad < 0) pad = 0;
  if (pad + int(kMisTile) > per_wg) pad = per_wg - int(kMisTile);
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(pad + 1, std::memory_order_relaxed);
  return size_t(pad);
}

// Static table area of reshard_execute_no_alloc: a plan's region and chunk
// tables are copied here on every such call instead of into an allocation
// the plan owns.  Each device holds its own copy of the array from the
// library's load until the process ends.  `scratch` is a host-side stand-in
// in host code: its device address comes from hipGetSymbolAddress, looked
// up once per device with that device current, and only that address is
// handed to copies and kernels.
extern const uint64_t kTableAreaBytes = uint64_t(4) << 20;
__device__ __align__(256) char scratch[uint64_t(4) << 20];

hipError_t table_area(int dev, char** out) {
  static std::atomic<char*> addr[kMaxDevices];
  static std::mutex mu;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  char* p = addr[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(mu);
  p = addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    p = static_cast<char*>(a);
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

template <class Args>
hipError_t launch_kind(uint32_t bucket, uint32_t grid, const Args& args, hipStream_t stream, int dev) {
  if (grid == 0) return hipSuccess;
  switch (bucket) {
    case kBulk:
      hipLaunchKernelGGL(rs_bulk_kernel<Args>, dim3(grid), dim3(kThreads), bulk_lds_pad(dev), stream, args);
      break;
    case kThin: hipLaunchKernelGGL(rs_thin_kernel<Args>, dim3(grid), dim3(kThreads), 0, stream, args); break;
    case kThinGroup:
      hipLaunchKernelGGL((rs_thin_group_kernel<false, Args>), dim3(grid), dim3(kThreads), 0, stream, args);
      break;
    case kThinGroupNarrow:
      hipLaunchKernelGGL((rs_thin_group_kernel<true, Args>), dim3(grid), dim3(kThreads), 0, stream, args);
      break;
    case kTiny: hipLaunchKernelGGL(rs_tiny_kernel<Args>, dim3(grid), dim3(kThreads), 0, stream, args); break;
    case kMx:
      hipLaunchKernelGGL((rs_mx_kernel<false, Args>), dim3(grid), dim3(kMxThreads), 0, stream, args);
      break;
    case kMxAux:
      hipLaunchKernelGGL((rs_mx_kernel<true, Args>), dim3(grid), dim3(kMxThreads), 0, stream, args);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch(uint32_t bucket, uint32_t grid, const LaunchArgs& args, hipStream_t stream, int dev) {
  return launch_kind(bucket, grid, args, stream, dev);
}

hipError_t launch(uint32_t bucket, uint32_t grid, const TableArgs& args, hipStream_t stream, int dev) {
  return launch_kind(bucket, grid, args, stream, dev);
}

}  // namespace rs
