// HIP kernels of the single-GPU M->N relayout, written for gfx950 (CDNA4,
// wave64).  Every kernel walks the region table built by the planner; a
// region copies rows x inner bytes between strided row sets.  The work is
// bitwise data movement bound by HBM bandwidth, so there is no MFMA here:
// the kernels aim at wide, coalesced global accesses and enough bytes in
// flight per CU.
//
//  bulk  one workgroup per work unit (<= unit_bytes).  16-byte vectors when
//        every address of the region is 16-byte aligned: long rows are walked
//        row by row by the whole workgroup (row address math is uniform, so it
//        runs on the scalar unit), short rows are split among sub-wave lane
//        groups.  Otherwise each wave copies one row at the widest granule the
//        source/destination co-alignment allows, with byte head and tail.
//  thin  runs shorter than the thin threshold (e.g. the 8-byte rows of a
//        column shard): rows are gathered through an LDS tile so the side
//        that is contiguous across rows is written (or read) with 16-byte
//        vectors.
//  tiny  regions of at most a few hundred bytes: one lane per region, a
//        wave-level prefix sum of their granule counts, then all 64 lanes
//        share the wave's granules.
//  mx    BF16 -> MXFP8 install: four lanes per 32-element block (8 bf16 = 16
//        bytes each), integer amax, integer round-to-nearest-even E4M3
//        encoding, 8 code bytes per lane and one scale byte per block.
//
// Fan-out: a region may name up to 16 destination replicas; the data is read
// once and stored to each (the one-GPU analogue of serving every replica from
// one received copy, "How NCCL M2N Reshard maximizes network bandwidth" in the
// news summary of NVIDIA's Reshard announcement).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "rs_device.hpp"

namespace rs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
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

template <bool kFan1>
__device__ __forceinline__ void bulk_body(const LaunchArgs& a, const CopyRegion* R, uint32_t unit) {
  const uint32_t tid = threadIdx.x;
  const uint64_t src_off = R->src_off, dst_off = R->dst_off;
  const uint64_t s0 = R->sstr[0], s1 = R->sstr[1], s2 = R->sstr[2];
  const uint64_t d0 = R->dstr[0], d1 = R->dstr[1], d2 = R->dstr[2];
  const uint32_t e0 = R->e0, e1 = R->e1, rows = R->rows, inner = R->inner;
  const uint32_t rpu = R->rows_per_unit, ub = R->unit_begin, flags = R->flags;
  const uint32_t nd = kFan1 ? 1u : R->n_dst;
  const uint32_t nouter = flags & kFlagOuterMask;
  const char* sp = static_cast<const char*>(a.ptr[R->src_ptr]) + src_off;
  char* dp0 = static_cast<char*>(a.ptr[R->dst_ptr[0]]) + dst_off;

  uint32_t al = (flags >> 8) & 15u;
  al |= uint32_t(reinterpret_cast<uintptr_t>(sp) & 15u);
  for (uint32_t j = 0; j < nd; ++j)
    al |= uint32_t((reinterpret_cast<uintptr_t>(a.ptr[R->dst_ptr[j]]) + dst_off) & 15u);

  const uint32_t r0 = (unit - ub) * rpu;
  const uint32_t r1 = min(r0 + rpu, rows);

  if (al == 0 && inner >= kLongRow) {
    // Long rows: the workgroup walks one row at a time.
    const uint32_t vpr = inner >> 4;
    for (uint32_t r = r0; r < r1; ++r) {
      const uint64_t so = row_off(r, e0, e1, nouter, s0, s1, s2);
      const uint64_t dof = row_off(r, e0, e1, nouter, d0, d1, d2);
      const char* s = sp + so;
      for (uint32_t v = tid; v < vpr; v += 4 * kThreads) {
        const bool b1 = v + kThreads < vpr, b2 = v + 2 * kThreads < vpr, b3 = v + 3 * kThreads < vpr;
        u32x4 x0 = ld16(s + 16ull * v), x1{}, x2{}, x3{};
        if (b1) x1 = ld16(s + 16ull * (v + kThreads));
        if (b2) x2 = ld16(s + 16ull * (v + 2 * kThreads));
        if (b3) x3 = ld16(s + 16ull * (v + 3 * kThreads));
        for (uint32_t j = 0; j < nd; ++j) {
          char* d = (kFan1 ? dp0 : static_cast<char*>(a.ptr[R->dst_ptr[j]]) + dst_off) + dof;
          st16(d + 16ull * v, x0);
          if (b1) st16(d + 16ull * (v + kThreads), x1);
          if (b2) st16(d + 16ull * (v + 2 * kThreads), x2);
          if (b3) st16(d + 16ull * (v + 3 * kThreads), x3);
        }
      }
    }
  } else if (al == 0) {
    // Short rows: L lanes per row (a power of two >= the row's vectors, at
    // most 64), 64 / L rows per wave step; each lane moves <= 2 vectors of a
    // row and two rows per iteration.
    const uint32_t vpr = inner >> 4;
    uint32_t L = 1;
    while (L < vpr && L < 64u) L <<= 1;
    const uint32_t lane = tid & 63u, wave = tid >> 6;
    const uint32_t sub = lane & (L - 1u);
    const uint32_t G = 64u / L;
    const uint32_t step = 4u * G;
    for (uint32_t rb = r0 + wave * G + lane / L; rb < r1; rb += 2u * step) {
      const uint32_t ra = rb, rc = rb + step;
      const bool hc = rc < r1;
      const uint64_t soa = row_off(ra, e0, e1, nouter, s0, s1, s2);
      const uint64_t doa = row_off(ra, e0, e1, nouter, d0, d1, d2);
      const uint64_t soc = hc ? row_off(rc, e0, e1, nouter, s0, s1, s2) : 0;
      const uint64_t doc = hc ? row_off(rc, e0, e1, nouter, d0, d1, d2) : 0;
      const uint32_t v0 = sub, v1 = sub + L;
      const bool a0 = v0 < vpr, a1 = v1 < vpr;
      u32x4 xa0{}, xa1{}, xc0{}, xc1{};
      if (a0) xa0 = ld16(sp + soa + 16ull * v0);
      if (a1) xa1 = ld16(sp + soa + 16ull * v1);
      if (hc && a0) xc0 = ld16(sp + soc + 16ull * v0);
      if (hc && a1) xc1 = ld16(sp + soc + 16ull * v1);
      for (uint32_t j = 0; j < nd; ++j) {
        char* d = kFan1 ? dp0 : static_cast<char*>(a.ptr[R->dst_ptr[j]]) + dst_off;
        if (a0) st16(d + doa + 16ull * v0, xa0);
        if (a1) st16(d + doa + 16ull * v1, xa1);
        if (hc && a0) st16(d + doc + 16ull * v0, xc0);
        if (hc && a1) st16(d + doc + 16ull * v1, xc1);
      }
    }
  } else {
    // Misaligned: one row per wave at the co-alignment granule.
    const uint32_t lane = tid & 63u, wave = tid >> 6;
    for (uint32_t r = r0 + wave; r < r1; r += 4) {
      const uint64_t so = row_off(r, e0, e1, nouter, s0, s1, s2);
      const uint64_t dof = row_off(r, e0, e1, nouter, d0, d1, d2);
      for (uint32_t j = 0; j < nd; ++j) {
        char* d = static_cast<char*>(a.ptr[R->dst_ptr[j]]) + dst_off + dof;
        wave_copy_span(d, sp + so, inner, lane);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void rs_bulk_kernel(LaunchArgs a) {
  const uint32_t unit = blockIdx.x;
  const uint32_t ri = __builtin_amdgcn_readfirstlane(a.unit_region[unit]);
  const CopyRegion* R = static_cast<const CopyRegion*>(a.regions) + ri;
  if (R->n_dst == 1)
    bulk_body<true>(a, R, unit);
  else
    bulk_body<false>(a, R, unit);
}

// ---------------------------------------------------------------------------
// thin (LDS-staged)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void rs_thin_kernel(LaunchArgs a) {
  __shared__ __attribute__((aligned(16))) char tile[kThinTile + 16];
  const uint32_t tid = threadIdx.x;
  const uint32_t unit = blockIdx.x;
  const uint32_t ri = __builtin_amdgcn_readfirstlane(a.unit_region[unit]);
  const CopyRegion* R = static_cast<const CopyRegion*>(a.regions) + ri;
  const uint64_t src_off = R->src_off, dst_off = R->dst_off;
  const uint64_t s0 = R->sstr[0], s1 = R->sstr[1], s2 = R->sstr[2];
  const uint64_t d0 = R->dstr[0], d1 = R->dstr[1], d2 = R->dstr[2];
  const uint32_t e0 = R->e0, e1 = R->e1, rows = R->rows, inner = R->inner;
  const uint32_t rpu = R->rows_per_unit, ub = R->unit_begin, flags = R->flags;
  const uint32_t nd = R->n_dst;
  const uint32_t nouter = flags & kFlagOuterMask;
  const char* sp = static_cast<const char*>(a.ptr[R->src_ptr]) + src_off;

  uint32_t al = (flags >> 8) & 15u;
  al |= uint32_t(reinterpret_cast<uintptr_t>(sp) & 15u);
  for (uint32_t j = 0; j < nd; ++j)
    al |= uint32_t((reinterpret_cast<uintptr_t>(a.ptr[R->dst_ptr[j]]) + dst_off) & 15u);
  const uint32_t g = low_granule(al);
  const uint32_t gpr = inner / g;

  const uint32_t r0 = (unit - ub) * rpu;
  const uint32_t r1 = min(r0 + rpu, rows);
  const uint32_t T = r1 - r0;
  const uint32_t nbytes = T * inner;
  const uint32_t total = T * gpr;

  if (flags & kFlagDstPacked) {
    // Gather strided source rows into LDS (congruent with the first
    // destination mod 16), then write the contiguous destination block.
    const char* D0 = static_cast<const char*>(a.ptr[R->dst_ptr[0]]) + dst_off + uint64_t(r0) * inner;
    const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(D0) & 15u);
    for (uint32_t f = tid; f < total; f += kThreads) {
      const uint32_t row = f / gpr;
      const uint32_t k = f - row * gpr;
      const uint64_t so = row_off(r0 + row, e0, e1, nouter, s0, s1, s2);
      copy_granule(tile + sh + row * inner + k * g, sp + so + uint64_t(k) * g, g);
    }
    __syncthreads();
    for (uint32_t j = 0; j < nd; ++j) {
      char* Dj = static_cast<char*>(a.ptr[R->dst_ptr[j]]) + dst_off + uint64_t(r0) * inner;
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
        char* d = static_cast<char*>(a.ptr[R->dst_ptr[j]]) + dst_off + dof + uint64_t(k) * g;
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
        char* d = static_cast<char*>(a.ptr[R->dst_ptr[j]]) + dst_off + dof + uint64_t(k) * g;
        copy_granule(d, sp + so + uint64_t(k) * g, g);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// tiny (wave prefix sum over many small regions)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t region_granule(const LaunchArgs& a, const CopyRegion* R) {
  uint32_t al = (R->flags >> 8) & 15u;
  al |= uint32_t((reinterpret_cast<uintptr_t>(a.ptr[R->src_ptr]) + R->src_off) & 15u);
  for (uint32_t j = 0; j < R->n_dst; ++j)
    al |= uint32_t((reinterpret_cast<uintptr_t>(a.ptr[R->dst_ptr[j]]) + R->dst_off) & 15u);
  return low_granule(al);
}

__global__ __launch_bounds__(kThreads) void rs_tiny_kernel(LaunchArgs a) {
  __shared__ uint32_t start[kThreads];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, wave = tid >> 6;
  const CopyRegion* regs = static_cast<const CopyRegion*>(a.regions);
  const uint32_t ri = blockIdx.x * kThreads + tid;
  uint32_t cnt = 0;
  if (ri < a.n_regions) {
    const CopyRegion* R = regs + ri;
    cnt = R->rows * (R->inner / region_granule(a, R));
  }
  // Inclusive scan of the per-lane granule counts across the wave.
  uint32_t scan = cnt;
  for (uint32_t off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(scan, off, 64);
    if (lane >= off) scan += y;
  }
  const uint32_t total = __shfl(scan, 63, 64);
  start[tid] = scan - cnt;
  __syncthreads();
  const uint32_t* ws = start + wave * 64;
  const uint32_t base = blockIdx.x * kThreads + wave * 64;
  for (uint32_t f = lane; f < total; f += 64) {
    // Last lane whose start <= f (empty regions share starts; take the last).
    uint32_t lo = 0, hi = 64;
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (ws[mid] <= f) lo = mid; else hi = mid;
    }
    const CopyRegion* R = regs + base + lo;
    const uint32_t g = region_granule(a, R);
    const uint32_t gpr = R->inner / g;
    const uint32_t local = f - ws[lo];
    const uint32_t row = local / gpr;
    const uint32_t k = local - row * gpr;
    const uint32_t nouter = R->flags & kFlagOuterMask;
    const uint64_t so = row_off(row, R->e0, R->e1, nouter, R->sstr[0], R->sstr[1], R->sstr[2]);
    const uint64_t dof = row_off(row, R->e0, R->e1, nouter, R->dstr[0], R->dstr[1], R->dstr[2]);
    const char* s = static_cast<const char*>(a.ptr[R->src_ptr]) + R->src_off + so + uint64_t(k) * g;
    for (uint32_t j = 0; j < R->n_dst; ++j) {
      char* d = static_cast<char*>(a.ptr[R->dst_ptr[j]]) + R->dst_off + dof + uint64_t(k) * g;
      copy_granule(d, s, g);
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

// E4M3 code of v * 2^-X for a bf16 bit pattern b: round to nearest even,
// saturating at 448, sign of zero kept.  |v| = M * 2^k with an 8-bit integer
// M; the result's binade exponent is ee = max(floor(log2|q|), -6) and its grid
// step 2^(ee-3), so the code is (ee + 6) * 8 + RNE(M * 2^(k - X - ee + 3)).
__device__ __forceinline__ uint32_t e4m3(uint32_t b, int X) {
  const uint32_t sign = (b >> 8) & 0x80u;
  const uint32_t E = (b >> 7) & 0xFFu;
  const uint32_t M = E ? (0x80u | (b & 0x7Fu)) : (b & 0x7Fu);
  if (M == 0) return sign;
  const int k = E ? int(E) - 134 : -133;
  const int msb = 31 - __builtin_clz(M);
  const int fl = msb + k - X;
  if (fl >= 9) return sign | 0x7Eu;
  const int ee = fl < -6 ? -6 : fl;
  const int sh = ee - 3 - (k - X);
  uint32_t n;
  if (sh <= 0) {
    n = M << (-sh);
  } else if (sh > 30) {
    n = 0;
  } else {
    n = M >> sh;
    const uint32_t rem = M & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    n += (rem > half || (rem == half && (n & 1u))) ? 1u : 0u;
  }
  uint32_t code = uint32_t((ee + 6) * 8) + n;
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

__global__ __launch_bounds__(kThreads) void rs_mx_kernel(LaunchArgs a) {
  const uint32_t tid = threadIdx.x;
  const uint32_t unit = blockIdx.x;
  const uint32_t ri = __builtin_amdgcn_readfirstlane(a.unit_region[unit]);
  const MxRegion* R = static_cast<const MxRegion*>(a.regions) + ri;
  const uint64_t src_off = R->src_off, dst_off = R->dst_off, sc_off = R->sc_off;
  const uint64_t s0 = R->sstr[0], s1 = R->sstr[1], s2 = R->sstr[2];
  const uint64_t d0 = R->dstr[0], d1 = R->dstr[1], d2 = R->dstr[2];
  const uint64_t c0 = R->scstr[0], c1 = R->scstr[1], c2 = R->scstr[2];
  const uint32_t e0 = R->e0, e1 = R->e1, rows = R->rows, inner = R->inner;
  const uint32_t rpu = R->rows_per_unit, ub = R->unit_begin, flags = R->flags;
  const uint32_t sc_inner = R->sc_inner;
  const uint32_t nd = R->n_dst;
  const uint32_t nouter = flags & kFlagOuterMask;
  const char* sp = static_cast<const char*>(a.ptr[R->src_ptr]) + src_off;

  const uint32_t r0 = (unit - ub) * rpu;
  const uint32_t r1 = min(r0 + rpu, rows);
  const uint32_t nb = (inner + 31u) >> 5;
  const uint32_t total = (r1 - r0) * nb;
  const uint32_t quad = tid >> 2, sub = tid & 3u;

  for (uint32_t fb = quad; fb < total; fb += kThreads / 4) {
    const uint32_t rr = fb / nb;
    const uint32_t b = fb - rr * nb;
    const uint32_t row = r0 + rr;
    const uint64_t so = row_off(row, e0, e1, nouter, s0, s1, s2);
    const uint64_t dof = row_off(row, e0, e1, nouter, d0, d1, d2);
    const uint64_t sco = row_off(row, e0, e1, nouter, c0, c1, c2);
    const uint32_t col = b * 32u + sub * 8u;
    const int nvalid = int(min(inner, col + 8u)) - int(min(inner, col));
    const uint16_t* s = reinterpret_cast<const uint16_t*>(sp + so) + col;
    uint32_t w[4] = {0, 0, 0, 0};
    if (nvalid == 8 && (reinterpret_cast<uintptr_t>(s) & 15u) == 0) {
      const u32x4 x = ld16(s);
      w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    } else {
      for (int i = 0; i < 8; ++i)
        if (i < nvalid) w[i >> 1] |= uint32_t(s[i]) << (16 * (i & 1));
    }
    uint32_t amax = 0;
    for (int i = 0; i < 4; ++i) {
      amax = max(amax, w[i] & 0x7FFFu);
      amax = max(amax, (w[i] >> 16) & 0x7FFFu);
    }
    amax = max(amax, uint32_t(__shfl_xor(int(amax), 1, 64)));
    amax = max(amax, uint32_t(__shfl_xor(int(amax), 2, 64)));
    const bool bad = amax >= 0x7F80u;
    const int X = shared_exp(amax);
    uint32_t lo = 0, hi = 0;
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = bad ? 0x7Fu : e4m3(w[i >> 1] >> (16 * (i & 1)) & 0xFFFFu, X);
      lo |= c << (8 * i);
    }
    for (int i = 4; i < 8; ++i) {
      const uint32_t c = bad ? 0x7Fu : e4m3(w[i >> 1] >> (16 * (i & 1)) & 0xFFFFu, X);
      hi |= c << (8 * (i - 4));
    }
    const uint8_t scale = bad ? uint8_t(0xFF) : uint8_t(X + 127);
    for (uint32_t j = 0; j < nd; ++j) {
      char* d = static_cast<char*>(a.ptr[R->dst_ptr[j]]) + dst_off + dof + col;
      if (nvalid == 8 && (reinterpret_cast<uintptr_t>(d) & 7u) == 0) {
        u32x2 v;
        v.x = lo;
        v.y = hi;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(d));
      } else {
        for (int i = 0; i < 8; ++i)
          if (i < nvalid) d[i] = char(((i < 4 ? lo : hi) >> (8 * (i & 3))) & 0xFFu);
      }
      if (sub == 0) {
        char* sc = static_cast<char*>(a.ptr[R->sc_ptr[j]]) + sc_off + sco + uint64_t(b) * sc_inner;
        *sc = char(scale);
      }
    }
  }
}

}  // namespace

hipError_t launch(uint32_t bucket, uint32_t grid, const LaunchArgs& args, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  switch (bucket) {
    case kBulk: hipLaunchKernelGGL(rs_bulk_kernel, dim3(grid), dim3(kThreads), 0, stream, args); break;
    case kThin: hipLaunchKernelGGL(rs_thin_kernel, dim3(grid), dim3(kThreads), 0, stream, args); break;
    case kTiny: hipLaunchKernelGGL(rs_tiny_kernel, dim3(grid), dim3(kThreads), 0, stream, args); break;
    case kMx: hipLaunchKernelGGL(rs_mx_kernel, dim3(grid), dim3(kThreads), 0, stream, args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rs
