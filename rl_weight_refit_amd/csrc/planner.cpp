// CPU planner of the single-GPU M->N relayout.
//
// Steps (all integer arithmetic):
//  1. Layout resolution: every slot's global box.  Shard(d) cuts dim d like
//     torch.chunk (chunk = ceil(len/parts), trailing chunks short or empty);
//     mesh dims sharding the same tensor dim nest in mesh-dim order.  The
//     pages describe a layout as global shape + device mesh + placements
//     (news summary of NVIDIA's Reshard announcement, "Recasting refit as a
//     DTensor-to-DTensor transfer").
//  2. Intersection: per tensor dim, a linear sweep over the sorted source and
//     destination intervals gives the overlapping pieces; their Cartesian
//     product gives the exact overlap boxes ("NCCL Reshard Refit
//     (Experimental)", "xferdtensor Transports": the Python transport
//     computes the exact shard overlaps and moves each destination region
//     once).  One source replica is read per box (replicas hold the same
//     bytes; cf. the geometry-based replica deduplication of the ModelExpress
//     PR #3632) and destination replicas with equal views share that read.
//  3. Views: a destination may be a slice of a fused buffer (gate/up in one
//     w13 buffer, "Execution Flow: Setup Time"), so region addresses go
//     through per-slot (base, strides) views and land in place.
//  4. Coalescing, chunking and bucketing: element size folds into the
//     innermost run, runs merge while both sides stay contiguous, outer dims
//     merge when both sides allow it, long runs split into work units; each
//     region goes to one of four kernels (bulk, LDS-staged thin, batched
//     tiny, MXFP8).  All regions of a bucket run in one launch, which is the
//     one-launch-per-batch idea of the coalesced collective in "NeMo-RL:
//     Optimizing Non-Colocated Refit for Asynchronous RL", "Optimization #2".
#include "planner.hpp"

#include <algorithm>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <numeric>
#include <sstream>
#include <utility>

namespace rs {
namespace {

constexpr int64_t kMaxSlots = 65536;
constexpr uint64_t kMaxRows = (1ull << 31) - 1;
constexpr uint32_t kMaxUnitsPerLaunch = 1u << 23;
// Destination siblings (see build_plan) are interleaved in chunks of this
// many units (0: off).  On MI355X, a TP3 -> TP2 split of a 2,049-wide bf16
// dim: 0.288 ms without, 0.270 / 0.261 / 0.259 / 0.260 ms with chunks of
// 16 / 32 / 64 / 256 units (0.391 ms with 1).
#ifndef RS_DST_CHUNK
#define RS_DST_CHUNK 64
#endif
constexpr uint32_t kMaxTinyBytes = 1u << 16;   // largest opts.tiny_bytes
constexpr int kMxBlock = 32;

int esize_of(int32_t dt) {
  switch (dt) {
    case RS_U8: case RS_I8: return 1;
    case RS_U16: case RS_I16: case RS_BF16: case RS_F16: return 2;
    case RS_U32: case RS_I32: case RS_F32: return 4;
    case RS_U64: case RS_I64: case RS_F64: return 8;
    default: return 0;
  }
}

struct Errors {
  std::ostringstream text;
  int invalid = 0, mismatch = 0, unsupported = 0;
  template <class... A>
  void add(int* counter, A&&... parts) {
    ++*counter;
    (text << ... << parts);
    text << "\n";
  }
  rs_status status() const {
    if (invalid) return RS_ERR_INVALID;
    if (mismatch) return RS_ERR_MISMATCH;
    if (unsupported) return RS_ERR_UNSUPPORTED;
    return RS_OK;
  }
};

struct Interval {
  int64_t start, len;
};

// A validated layout (one side of one tensor).
struct Layout {
  int ndim = 0, esize = 0, dtype = 0, quant = 0;
  int64_t shape[RS_MAX_DIMS] = {};
  int mesh_ndim = 0;
  int64_t mesh[RS_MAX_MESH] = {};
  int pl[RS_MAX_MESH] = {};
  int64_t nslots = 0;
  std::vector<int32_t> coord_to_slot;  // linear mesh coord -> slot
  std::vector<int32_t> slot_to_coord;  // slot -> linear mesh coord
  std::vector<int> shard_md[RS_MAX_DIMS];   // mesh dims sharding tensor dim d, in order
  std::vector<Interval> iv[RS_MAX_DIMS];    // interval index -> interval
  std::vector<int> rep_md;                  // Replicate mesh dims, in order
  int64_t nrep = 1;
  bool split = false;                       // one buffer per local dim-0 index
  std::vector<int64_t> ptr_base;            // slot -> first pointer index of the side
  int64_t nptrs = 0;                        // pointers the side takes
  std::vector<rs_view> views;               // resolved per slot
  std::vector<rs_view> scale_views;         // MXFP8 destinations
  std::vector<Interval> box;                // slot * ndim + d

  int64_t coord_of(int64_t lin, int md) const {
    int64_t div = 1;
    for (int i = md + 1; i < mesh_ndim; ++i) div *= mesh[i];
    return (lin / div) % mesh[md];
  }
  const Interval* slot_box(int64_t slot) const { return &box[slot * ndim]; }
};

void chunk(int64_t len, int64_t parts, int64_t idx, int64_t* start, int64_t* n) {
  const int64_t cs = len > 0 ? (len + parts - 1) / parts : 0;
  const int64_t a = std::min(idx * cs, len);
  const int64_t b = std::min((idx + 1) * cs, len);
  *start = a;
  *n = b - a;
}

void dense_view(const Interval* box, int ndim, int64_t last_div, rs_view* v) {
  std::memset(v, 0, sizeof(*v));
  int64_t acc = 1;
  for (int d = ndim - 1; d >= 0; --d) {
    v->strides[d] = acc;
    int64_t n = box[d].len;
    if (d == ndim - 1 && last_div > 1) n = (n + last_div - 1) / last_div;
    acc *= n;
  }
}

// Every byte count and byte offset of a plan stays below 2^62, so sums and
// products of them cannot overflow 64-bit arithmetic.
constexpr int64_t kMaxBytes = int64_t(1) << 62;
constexpr int64_t kMaxPtrs = int64_t(1) << 31;   // buffer pointers per side of a tensor

// True when prod(shape) * esize < 2^62 (zero extents ignored, so the dense
// strides of any box of the tensor stay below the bound too).
bool fits_bytes(const int64_t* shape, int ndim, int64_t esize) {
  int64_t v = esize;
  for (int i = 0; i < ndim; ++i) {
    if (shape[i] == 0) continue;
    if (v >= kMaxBytes / shape[i]) return false;
    v *= shape[i];
  }
  return v < kMaxBytes;
}

// True when the highest byte the view addresses for a box (last extent
// divided by last_div, rounded up; dim 0 skipped for split parts) is below
// 2^62.  Negative fields are reported separately and pass here.
bool view_fits(const rs_view& v, const Interval* box, int ndim, bool split, int64_t last_div,
               int64_t esize) {
  unsigned __int128 hi = v.base > 0 ? uint64_t(v.base) : 0;
  for (int i = split ? 1 : 0; i < ndim; ++i) {
    int64_t n = box[i].len;
    if (i == ndim - 1 && last_div > 1) n = (n + last_div - 1) / last_div;
    if (n == 0) return true;   // an empty box addresses nothing
    if (v.strides[i] > 0) hi += (unsigned __int128)(n - 1) * uint64_t(v.strides[i]);
  }
  return (hi + 1) * uint64_t(esize) < (unsigned __int128)kMaxBytes;
}

bool parse_layout(const rs_tensor_desc* d, const char* side, int t, bool is_dst, Layout& L,
                  Errors& E) {
  const int before = E.invalid;
  if (!d) {
    E.add(&E.invalid, "tensor ", t, " ", side, ": description is NULL");
    return false;
  }
  if (d->ndim < 1 || d->ndim > RS_MAX_DIMS) {
    E.add(&E.invalid, "tensor ", t, " ", side, ": ndim ", d->ndim, " not in [1, ", RS_MAX_DIMS, "]");
    return false;
  }
  L.ndim = d->ndim;
  L.dtype = d->dtype;
  L.esize = esize_of(d->dtype);
  if (!L.esize) E.add(&E.invalid, "tensor ", t, " ", side, ": unknown dtype ", d->dtype);
  bool shape_ok = true;
  for (int i = 0; i < L.ndim; ++i) {
    L.shape[i] = d->global_shape[i];
    if (L.shape[i] < 0) {
      E.add(&E.invalid, "tensor ", t, " ", side, ": global_shape[", i, "] = ", L.shape[i], " < 0");
      shape_ok = false;
    }
  }
  if (shape_ok && !fits_bytes(L.shape, L.ndim, L.esize ? L.esize : 1)) {
    E.add(&E.invalid, "tensor ", t, " ", side, ": the global tensor holds 2^62 bytes or more");
    shape_ok = false;
  }
  if (d->mesh_ndim < 1 || d->mesh_ndim > RS_MAX_MESH) {
    E.add(&E.invalid, "tensor ", t, " ", side, ": mesh_ndim ", d->mesh_ndim, " not in [1, ",
          RS_MAX_MESH, "]");
    return false;
  }
  L.mesh_ndim = d->mesh_ndim;
  L.nslots = 1;
  bool mesh_ok = true;
  for (int i = 0; i < L.mesh_ndim; ++i) {
    L.mesh[i] = d->mesh_shape[i];
    L.pl[i] = d->placements[i];
    if (L.mesh[i] < 1) {
      E.add(&E.invalid, "tensor ", t, " ", side, ": mesh_shape[", i, "] = ", L.mesh[i], " < 1");
      mesh_ok = false;
    } else if (L.nslots <= kMaxSlots) {
      L.nslots = L.mesh[i] > kMaxSlots ? kMaxSlots + 1 : L.nslots * L.mesh[i];
    }
    if (L.pl[i] != RS_REPLICATE && (L.pl[i] < 0 || L.pl[i] >= L.ndim))
      E.add(&E.invalid, "tensor ", t, " ", side, ": placements[", i, "] = ", L.pl[i],
            " is neither Replicate (-1) nor a tensor dim < ", L.ndim);
  }
  if (mesh_ok && L.nslots > kMaxSlots) {
    E.add(&E.invalid, "tensor ", t, " ", side, ": mesh has more than ", kMaxSlots, " slots");
    mesh_ok = false;
  }
  if (d->quant != RS_Q_NONE && d->quant != RS_Q_MXFP8_E4M3)
    E.add(&E.invalid, "tensor ", t, " ", side, ": unknown quant mode ", d->quant);
  if (!is_dst && d->quant != RS_Q_NONE)
    E.add(&E.invalid, "tensor ", t, " ", side, ": quant is a destination setting");
  L.quant = is_dst ? d->quant : RS_Q_NONE;
  if (!mesh_ok || E.invalid != before) return false;

  L.coord_to_slot.resize(L.nslots);
  L.slot_to_coord.assign(L.nslots, -1);
  for (int64_t c = 0; c < L.nslots; ++c) {
    const int64_t s = d->slot_of_coord ? d->slot_of_coord[c] : c;
    if (s < 0 || s >= L.nslots || L.slot_to_coord[s] != -1) {
      E.add(&E.invalid, "tensor ", t, " ", side, ": slot_of_coord is not a permutation of 0..",
            L.nslots - 1, " (entry ", c, " = ", s, ")");
      return false;
    }
    L.coord_to_slot[c] = static_cast<int32_t>(s);
    L.slot_to_coord[s] = static_cast<int32_t>(c);
  }

  if (!shape_ok) return false;
  for (int i = 0; i < L.mesh_ndim; ++i) {
    if (L.pl[i] == RS_REPLICATE) {
      L.rep_md.push_back(i);
      L.nrep *= L.mesh[i];
    } else {
      L.shard_md[L.pl[i]].push_back(i);
    }
  }
  for (int dd = 0; dd < L.ndim; ++dd) {
    std::vector<Interval> cur{{0, L.shape[dd]}};
    for (int md : L.shard_md[dd]) {
      std::vector<Interval> next;
      next.reserve(cur.size() * L.mesh[md]);
      for (const Interval& p : cur)
        for (int64_t c = 0; c < L.mesh[md]; ++c) {
          int64_t a, n;
          chunk(p.len, L.mesh[md], c, &a, &n);
          next.push_back({p.start + a, n});
        }
      cur.swap(next);
    }
    L.iv[dd] = std::move(cur);
  }
  L.box.resize(L.nslots * L.ndim);
  for (int64_t s = 0; s < L.nslots; ++s) {
    const int64_t lin = L.slot_to_coord[s];
    for (int dd = 0; dd < L.ndim; ++dd) {
      int64_t idx = 0;
      for (int md : L.shard_md[dd]) idx = idx * L.mesh[md] + L.coord_of(lin, md);
      L.box[s * L.ndim + dd] = L.iv[dd][idx];
    }
  }

  if (d->split_dim0 != 0 && d->split_dim0 != 1)
    E.add(&E.invalid, "tensor ", t, " ", side, ": split_dim0 = ", d->split_dim0, " is not 0 or 1");
  L.split = d->split_dim0 == 1;
  if (L.split && L.quant == RS_Q_MXFP8_E4M3 && L.ndim < 2)
    E.add(&E.unsupported, "tensor ", t, " ", side,
          ": a split MXFP8 destination needs at least 2 dims (blocks run along the last dim)");
  L.ptr_base.resize(L.nslots);
  L.nptrs = 0;
  for (int64_t s = 0; s < L.nslots; ++s) {
    L.ptr_base[s] = L.nptrs;
    L.nptrs += L.split ? L.slot_box(s)[0].len : 1;
    if (L.nptrs > kMaxPtrs) {
      E.add(&E.invalid, "tensor ", t, " ", side, ": more than ", kMaxPtrs, " buffer pointers");
      return false;
    }
  }
  L.views.resize(L.nslots);
  for (int64_t s = 0; s < L.nslots; ++s) {
    if (d->views) {
      L.views[s] = d->views[s];
      if (L.views[s].base < 0)
        E.add(&E.invalid, "tensor ", t, " ", side, ": views[", s, "].base < 0");
      for (int i = 0; i < L.ndim; ++i)
        if (L.views[s].strides[i] < 0)
          E.add(&E.invalid, "tensor ", t, " ", side, ": views[", s, "].strides[", i, "] < 0");
      if (!view_fits(L.views[s], L.slot_box(s), L.ndim, L.split, 1, L.esize ? L.esize : 1))
        E.add(&E.invalid, "tensor ", t, " ", side, ": views[", s, "] reaches 2^62 bytes or more");
    } else {
      dense_view(L.slot_box(s), L.ndim, 1, &L.views[s]);
    }
  }
  if (L.quant == RS_Q_MXFP8_E4M3) {
    L.scale_views.resize(L.nslots);
    for (int64_t s = 0; s < L.nslots; ++s) {
      if (d->scale_views) {
        L.scale_views[s] = d->scale_views[s];
        if (L.scale_views[s].base < 0)
          E.add(&E.invalid, "tensor ", t, " ", side, ": scale_views[", s, "].base < 0");
        for (int i = 0; i < L.ndim; ++i)
          if (L.scale_views[s].strides[i] < 0)
            E.add(&E.invalid, "tensor ", t, " ", side, ": scale_views[", s, "].strides[", i, "] < 0");
        if (!view_fits(L.scale_views[s], L.slot_box(s), L.ndim, L.split, kMxBlock, 1))
          E.add(&E.invalid, "tensor ", t, " ", side, ": scale_views[", s, "] reaches 2^62 bytes or more");
      } else {
        dense_view(L.slot_box(s), L.ndim, kMxBlock, &L.scale_views[s]);
      }
    }
  }
  return E.invalid == before;
}

// Overlapping pieces of two partitions of one tensor dim.
struct Piece {
  int64_t si, di, start, len;
};

std::vector<Piece> sweep(const std::vector<Interval>& a, const std::vector<Interval>& b) {
  std::vector<Piece> out;
  size_t i = 0, j = 0;
  auto skip = [](const std::vector<Interval>& v, size_t k) {
    while (k < v.size() && v[k].len == 0) ++k;
    return k;
  };
  i = skip(a, i);
  j = skip(b, j);
  while (i < a.size() && j < b.size()) {
    const int64_t lo = std::max(a[i].start, b[j].start);
    const int64_t ea = a[i].start + a[i].len, eb = b[j].start + b[j].len;
    const int64_t hi = std::min(ea, eb);
    if (hi > lo) out.push_back({int64_t(i), int64_t(j), lo, hi - lo});
    if (ea <= eb) i = skip(a, i + 1);
    if (eb <= ea) j = skip(b, j + 1);
  }
  return out;
}

// Linear mesh coordinate from per-dim interval indices and replicate coords.
int64_t compose_coord(const Layout& L, const int64_t* ividx, int64_t rep_ordinal) {
  int64_t coord[RS_MAX_MESH] = {};
  for (int dd = 0; dd < L.ndim; ++dd) {
    int64_t idx = ividx[dd];
    for (int k = int(L.shard_md[dd].size()) - 1; k >= 0; --k) {
      const int md = L.shard_md[dd][k];
      coord[md] = idx % L.mesh[md];
      idx /= L.mesh[md];
    }
  }
  for (int k = int(L.rep_md.size()) - 1; k >= 0; --k) {
    const int md = L.rep_md[k];
    coord[md] = rep_ordinal % L.mesh[md];
    rep_ordinal /= L.mesh[md];
  }
  int64_t lin = 0;
  for (int md = 0; md < L.mesh_ndim; ++md) lin = lin * L.mesh[md] + coord[md];
  return lin;
}

// Ordinal of a destination class: mixed radix over its sharding coords.
int64_t class_ordinal(const Layout& L, const int64_t* ividx) {
  int64_t ord = 0;
  for (int dd = 0; dd < L.ndim; ++dd) ord = ord * int64_t(L.iv[dd].size()) + ividx[dd];
  return ord;
}

bool same_view(const rs_view& a, const rs_view& b, int ndim) {
  if (a.base != b.base) return false;
  for (int i = 0; i < ndim; ++i)
    if (a.strides[i] != b.strides[i]) return false;
  return true;
}

// A region before it is split to fit the kernels.
struct Dim {
  uint64_t ext, ss, ds, sc;  // extent; byte strides on src, dst, scale sides
  uint64_t ss2;              // source stride of a two-piece MXFP8 region's second piece (0: none)
};

// Outer dims, outermost first.  A region keeps at most 3 outer dims plus
// one that finalize adds while cutting long rows (regions are peeled to that
// when they are built); WideDims holds the up to rank + 1 dims of a region
// being built.
template <int Cap>
struct DimsT {
  Dim d[Cap];
  int n = 0;
  DimsT() {}  // entries past n stay unset
  void push_back(const Dim& x) {
    if (n == Cap) std::abort();  // unreachable: regions are peeled before they grow past Cap
    d[n++] = x;
  }
  void pop_back() { --n; }
  Dim& back() { return d[n - 1]; }
  Dim& front() { return d[0]; }
  bool empty() const { return n == 0; }
  size_t size() const { return size_t(n); }
  const Dim* begin() const { return d; }
  const Dim* end() const { return d + n; }
};
using Dims = DimsT<4>;
using WideDims = DimsT<RS_MAX_DIMS + 1>;

struct Raw {
  // Fields without initializers are set where a region is built; a Raw is
  // a few hundred bytes, so value-initializing each one would cost more
  // than the planning it takes part in.
  Raw() {}
  uint32_t tensor;
  bool mx;
  uint32_t src_index;
  uint32_t n_dst;
  uint32_t dst_index[kMaxFan], sc_index[kMaxFan];
  uint64_t src_off, dst_off, sc_off;
  uint64_t inner;                 // bytes (copy) or elements (mx)
  uint64_t sc_inner;
  Dims outer;
  // MXFP8 only.  A block that two source shards share is installed by a
  // region with two pieces: columns [0, split) come from the first source
  // (src_index, src_off, outer ss), columns [split, inner) from the second
  // (src2_index, src2_off, outer ss2).  split == inner: one piece.
  uint64_t split = 0;
  uint32_t src2_index = 0;
  uint64_t src2_off = 0;
  // While planning: destination-local first column and the offsets of
  // column 0 of these rows (elements, scale bytes), to group the pieces of
  // one row box before cutting them into regions.
  uint64_t c0 = 0, kloc = 0, drow = 0, srow = 0;
};

uint64_t rows_of(const Dims& o) {
  uint64_t r = 1;
  for (const Dim& d : o) r *= d.ext;
  return r;
}

// Merge mergeable adjacent outer dims; drop extent-1 dims.
template <int Cap>
void merge_outer(DimsT<Cap>& o, bool with_scale) {
  DimsT<Cap> m;
  for (const Dim& d : o) {
    if (d.ext == 1) continue;
    if (!m.empty()) {
      Dim& p = m.back();  // p outer, d inner
      if (p.ss == d.ext * d.ss && p.ds == d.ext * d.ds && (!with_scale || p.sc == d.ext * d.sc) &&
          p.ss2 == d.ext * d.ss2) {
        p.ext *= d.ext;
        p.ss = d.ss;
        p.ds = d.ds;
        p.sc = d.sc;
        p.ss2 = d.ss2;
        continue;
      }
    }
    m.push_back(d);
  }
  o = m;
}

#ifndef RS_THIN_SIBLINGS
#define RS_THIN_SIBLINGS 1   // group thin regions that read the same source rows
#endif
#ifndef RS_FANOUT_UNIT_SHIFT
#define RS_FANOUT_UNIT_SHIFT 0  // bulk units of regions with several destinations: unit_bytes >> this
#endif
#ifndef RS_THIN_GROUP_LOAD
#define RS_THIN_GROUP_LOAD 1 // load short-span sibling groups whole (one workgroup per row block)
#endif

struct Opts {
  bool fanout = true;
  uint64_t unit = 16384;
  uint64_t tiny = 256;
  uint64_t thin = 128;
};

// Same destinations and rows (the pieces of one MXFP8 row box).
bool same_row_box(const Raw& a, const Raw& b) {
  if (a.tensor != b.tensor || a.n_dst != b.n_dst || a.drow != b.drow || a.srow != b.srow ||
      a.outer.n != b.outer.n || a.kloc != b.kloc)
    return false;
  for (uint32_t j = 0; j < a.n_dst; ++j)
    if (a.dst_index[j] != b.dst_index[j] || a.sc_index[j] != b.sc_index[j]) return false;
  for (int i = 0; i < a.outer.n; ++i)
    if (a.outer.d[i].ext != b.outer.d[i].ext || a.outer.d[i].ds != b.outer.d[i].ds ||
        a.outer.d[i].sc != b.outer.d[i].sc)
      return false;
  return true;
}

// Columns [c, c + n) of piece p as a one-source region (c block-aligned,
// n whole blocks or up to the row end).
Raw mx_part(const Raw& p, uint64_t c, uint64_t n) {
  Raw r = p;
  r.src_off = p.src_off + (c - p.c0) * 2;
  r.dst_off = p.drow + c;
  r.sc_off = p.srow + (c / kMxBlock) * p.sc_inner;
  r.inner = n;
  r.split = n;
  merge_outer(r.outer, true);
  return r;
}

void cut_mx_pieces(std::vector<Raw>& raws, Errors& E) {
  std::vector<size_t> mx;
  for (size_t i = 0; i < raws.size(); ++i)
    if (raws[i].mx) mx.push_back(i);
  if (mx.empty()) return;
  // Pieces of one row box are created consecutively (columns innermost),
  // but sort to be independent of that order.
  std::stable_sort(mx.begin(), mx.end(), [&](size_t x, size_t y) {
    const Raw& a = raws[x];
    const Raw& b = raws[y];
    if (a.tensor != b.tensor) return a.tensor < b.tensor;
    if (a.dst_index[0] != b.dst_index[0]) return a.dst_index[0] < b.dst_index[0];
    if (a.drow != b.drow) return a.drow < b.drow;
    if (a.srow != b.srow) return a.srow < b.srow;
    return a.c0 < b.c0;
  });
  std::vector<Raw> out;
  out.reserve(raws.size());
  for (size_t i = 0; i < raws.size(); ++i)
    if (!raws[i].mx) out.push_back(std::move(raws[i]));
  size_t g = 0;
  while (g < mx.size()) {
    size_t e = g + 1;
    while (e < mx.size() && same_row_box(raws[mx[g]], raws[mx[e]])) ++e;
    const uint64_t K = raws[mx[g]].kloc;
    for (size_t i = g; i < e; ++i) {
      const Raw& p = raws[mx[i]];
      const uint64_t a = p.c0, b = p.c0 + p.inner;
      if (i > g && a % kMxBlock != 0) {
        // The block holding column a starts in the previous piece.
        const Raw& q = raws[mx[i - 1]];
        const uint64_t B = a - a % kMxBlock, Eb = std::min<uint64_t>(B + kMxBlock, K);
        if (q.c0 > B || b < Eb || q.c0 + q.inner != a) {
          E.add(&E.unsupported, "tensor ", p.tensor, ": MXFP8 block at columns ", B, "..", Eb,
                " of a destination shard takes values from more than two source shards "
                "(source shards narrower than a 32-element block along the last dim)");
          continue;
        }
        Raw r = q;
        r.src_off = q.src_off + (B - q.c0) * 2;
        r.src2_index = p.src_index;
        r.src2_off = p.src_off;
        r.split = a - B;
        r.inner = Eb - B;
        r.dst_off = q.drow + B;
        r.sc_off = q.srow + (B / kMxBlock) * q.sc_inner;
        for (int k = 0; k < r.outer.n; ++k) r.outer.d[k].ss2 = p.outer.d[k].ss;
        merge_outer(r.outer, true);
        out.push_back(std::move(r));
      }
      // Whole blocks of this piece alone (the last block may be short).
      const uint64_t lo = (a + kMxBlock - 1) / kMxBlock * kMxBlock;
      const uint64_t hi = b == K ? b : b - b % kMxBlock;
      if (hi > lo) out.push_back(mx_part(p, lo, hi - lo));
    }
    if (raws[mx[g]].c0 != 0 || raws[mx[e - 1]].c0 + raws[mx[e - 1]].inner != K)
      E.add(&E.invalid, "internal: MXFP8 pieces of tensor ", raws[mx[g]].tensor,
            " do not tile the destination row");
    g = e;
  }
  raws.swap(out);
}

// Splits a raw region until the kernels can take it: at most 3 outer dims,
// rows < 2^31, every extent < 2^32, and (copy) inner <= unit bytes.
void finalize(Raw r, const Opts& o, std::vector<Raw>& out) {  // r by value: it is modified
  if (r.mx && r.inner > kMxBatchElems) {
    // Split long MXFP8 rows into block-aligned segments of one batch each.
    const uint64_t C = kMxBatchElems;
    const uint64_t q = r.inner / C, rem = r.inner % C;
    const uint64_t sc_step = (C / kMxBlock) * r.sc_inner;
    if (rem) {
      Raw tail = r;
      tail.inner = rem;
      tail.split = rem;   // one piece (two-piece regions are one block wide)
      tail.src_off += q * C * 2;
      tail.dst_off += q * C;
      tail.sc_off += q * sc_step;
      finalize(tail, o, out);
    }
    r.inner = C;
    r.split = C;
    r.outer.push_back({q, 2 * C, C, sc_step});
    merge_outer(r.outer, true);
  }
  const uint64_t unit = r.n_dst > 1 ? o.unit >> RS_FANOUT_UNIT_SHIFT : o.unit;
  if (!r.mx && r.inner > unit) {
    const uint64_t q = r.inner / unit, rem = r.inner % unit;
    if (rem) {
      Raw tail = r;
      tail.inner = rem;
      tail.src_off += q * unit;
      tail.dst_off += q * unit;
      finalize(std::move(tail), o, out);
    }
    r.inner = unit;
    r.outer.push_back({q, unit, unit, 0});
    merge_outer(r.outer, false);
  }
  const uint64_t rows = rows_of(r.outer);
  if (rows == 0 || r.inner == 0) return;
  bool ext_big = false;
  for (const Dim& d : r.outer) ext_big |= d.ext > 0xFFFFFFFFull;
  if (r.outer.size() > 3 || rows > kMaxRows || ext_big) {
    // Peel the outermost dim: either one index at a time (too many dims) or
    // in halves (too many rows).
    const Dim top = r.outer.front();
    Dims rest;
    for (int i = 1; i < r.outer.n; ++i) rest.push_back(r.outer.d[i]);
    if (r.outer.size() > 3) {
      for (uint64_t i = 0; i < top.ext; ++i) {
        Raw s = r;
        s.outer = rest;
        s.src_off += i * top.ss;
        s.src2_off += i * top.ss2;
        s.dst_off += i * top.ds;
        s.sc_off += i * top.sc;
        finalize(std::move(s), o, out);
      }
    } else {
      const uint64_t h = top.ext / 2;
      for (int part = 0; part < 2; ++part) {
        Raw s = r;
        const uint64_t n = part ? top.ext - h : h;
        const uint64_t first = part ? h : 0;
        s.outer.n = 0;
        s.outer.push_back(Dim{n, top.ss, top.ds, top.sc, top.ss2});
        for (const Dim& x : rest) s.outer.push_back(x);
        s.src_off += first * top.ss;
        s.src2_off += first * top.ss2;
        s.dst_off += first * top.ds;
        s.sc_off += first * top.sc;
        finalize(std::move(s), o, out);
      }
    }
    return;
  }
  out.push_back(std::move(r));
}

// True when finalize would keep r exactly as it is (the common case), so
// the caller can use it in place instead of copying it.
bool final_as_is(const Raw& r, const Opts& o) {
  if (r.mx && r.inner > kMxBatchElems) return false;
  if (!r.mx && r.inner > (r.n_dst > 1 ? o.unit >> RS_FANOUT_UNIT_SHIFT : o.unit)) return false;
  const uint64_t rows = rows_of(r.outer);
  if (rows == 0 || r.inner == 0 || rows > kMaxRows || r.outer.size() > 3) return false;
  for (const Dim& d : r.outer)
    if (d.ext > 0xFFFFFFFFull) return false;
  return true;
}

// finalize without copying r where that is possible: returns true when r
// itself (possibly cut to unit-sized rows in place) is final and comes
// after the pieces appended to out; false when out holds all of r's pieces.
bool finalize_at(Raw& r, const Opts& o, std::vector<Raw>& out) {
  if (final_as_is(r, o)) return true;
  const uint64_t unit = r.n_dst > 1 ? o.unit >> RS_FANOUT_UNIT_SHIFT : o.unit;
  if (!r.mx && r.inner > unit && r.outer.size() < 3) {
    const uint64_t q = r.inner / unit, rem = r.inner % unit;
    if (rem) {
      Raw tail = r;
      tail.inner = rem;
      tail.src_off += q * unit;
      tail.dst_off += q * unit;
      finalize(std::move(tail), o, out);
    }
    r.inner = unit;
    r.outer.push_back({q, unit, unit, 0});
    merge_outer(r.outer, false);
    if (final_as_is(r, o)) return true;
    finalize(r, o, out);
    return false;
  }
  finalize(r, o, out);
  return false;
}

struct Final {
  const Raw* rp;
  uint32_t bucket;
  uint32_t flags;
  uint64_t rows;
  uint32_t rows_per_unit;
  uint32_t units;
};

// Fills the fields shared by the public and device views.
void outer_fields(const Dims& o, uint64_t ext[3], uint64_t ss[3], uint64_t ds[3],
                  uint64_t sc[3], uint64_t* ss2 = nullptr) {
  // Device convention: index 0 is the innermost outer dim.
  for (int k = 0; k < 3; ++k) {
    ext[k] = 1;
    ss[k] = ds[k] = sc[k] = 0;
    if (ss2) ss2[k] = 0;
  }
  const int n = int(o.size());
  for (int k = 0; k < n; ++k) {
    const Dim& d = o.d[n - 1 - k];
    ext[k] = d.ext;
    ss[k] = d.ss;
    ds[k] = d.ds;
    sc[k] = d.sc;
    if (ss2) ss2[k] = d.ss2;
  }
}

bool packed(const uint64_t ext[3], const uint64_t st[3], int nouter, uint64_t inner) {
  uint64_t want = inner;
  for (int k = 0; k < nouter; ++k) {
    if (st[k] != want) return false;
    want *= ext[k];
  }
  return true;
}

void align_up(std::vector<uint8_t>& img, size_t a) {
  img.resize((img.size() + a - 1) / a * a, 0);
}

}  // namespace

rs_status shard_box(const rs_tensor_desc* d, int64_t slot, int64_t* off, int64_t* len,
                    std::string& err) {
  Errors E;
  Layout L;
  if (!parse_layout(d, "desc", 0, d && d->quant != RS_Q_NONE, L, E)) {
    err = E.text.str();
    return E.status() == RS_OK ? RS_ERR_INVALID : E.status();
  }
  if (slot < 0 || slot >= L.nslots || !off || !len) {
    err = "slot out of range or NULL output\n";
    return RS_ERR_INVALID;
  }
  const Interval* b = L.slot_box(slot);
  for (int i = 0; i < L.ndim; ++i) {
    off[i] = b[i].start;
    len[i] = b[i].len;
  }
  return RS_OK;
}

// Gives the region just built (raws.back()) the outer dims w.  A region
// with more than 3 is replaced by one region per index of its outermost
// dims (as finalize would peel it), so a Raw never holds more than 3 dims
// from here on.
void peel_into(std::vector<Raw>& raws, const Raw& proto, const WideDims& w, int k) {
  if (w.n - k <= 3) {
    Raw& r = raws.emplace_back(proto);
    r.outer.n = 0;
    for (int i = k; i < w.n; ++i) r.outer.push_back(w.d[i]);
    return;
  }
  const Dim& top = w.d[k];
  for (uint64_t i = 0; i < top.ext; ++i) {
    Raw s = proto;
    s.src_off += i * top.ss;
    s.dst_off += i * top.ds;
    if (s.mx) {  // MXFP8 pieces: row offsets on the element and scale sides
      s.drow += i * top.ds;
      s.srow += i * top.sc;
    } else {
      s.sc_off += i * top.sc;
    }
    peel_into(raws, s, w, k + 1);
  }
}
void set_outer(std::vector<Raw>& raws, const WideDims& w) {
  Raw& r = raws.back();
  if (w.n <= 3) {
    r.outer.n = 0;
    for (int i = 0; i < w.n; ++i) r.outer.push_back(w.d[i]);
    return;
  }
  const Raw proto = r;
  raws.pop_back();
  peel_into(raws, proto, w, 0);
}

rs_status build_plan(const rs_tensor_desc* src, const rs_tensor_desc* dst, int32_t n,
                     const rs_plan_opts* popts, PlanData& out, std::string& err) {
  const auto t0 = std::chrono::steady_clock::now();
  Errors E;
  Opts o;
  if (n < 0) E.add(&E.invalid, "n_tensors = ", n, " < 0");
  if (n > 0 && (!src || !dst)) E.add(&E.invalid, "src or dst description array is NULL");
  if (popts) {
    if (popts->struct_size != sizeof(rs_plan_opts))
      E.add(&E.invalid, "opts.struct_size = ", popts->struct_size, ", expected ",
            sizeof(rs_plan_opts));
    const uint64_t u = popts->unit_bytes ? popts->unit_bytes : o.unit;
    if (u < 4096 || u > (1u << 24) || (u & (u - 1)))
      E.add(&E.invalid, "opts.unit_bytes = ", u, " is not a power of two in [4096, 2^24]");
    for (int i = 0; i < 4; ++i)
      if (popts->reserved[i]) E.add(&E.invalid, "opts.reserved[", i, "] must be 0");
    // The thin kernel stages a unit of whole rows in its kThinTile LDS tile,
    // so no thin row may be longer than the tile; the tiny kernel numbers a
    // wave's granules (up to 64 regions of tiny_bytes) with 32-bit counters.
    if (popts->thin_bytes > kThinTile)
      E.add(&E.invalid, "opts.thin_bytes = ", popts->thin_bytes, " exceeds the ", kThinTile,
            "-byte LDS tile of the thin kernel");
    if (popts->tiny_bytes > kMaxTinyBytes)
      E.add(&E.invalid, "opts.tiny_bytes = ", popts->tiny_bytes, " exceeds ", kMaxTinyBytes);
    o.fanout = popts->fanout != 0;
    o.unit = u;
    o.tiny = popts->tiny_bytes;
    o.thin = popts->thin_bytes ? popts->thin_bytes : o.thin;
  }
  if (E.status() != RS_OK) {
    err = E.text.str();
    return E.status();
  }

  std::vector<Layout> S(n), D(n);
  uint64_t n_src_ptrs = 0, n_dst_ptrs = 0;
  std::vector<uint64_t> src_base(n), dst_base(n), sc_base(n);
  for (int t = 0; t < n; ++t) {
    const bool okS = parse_layout(&src[t], "src", t, false, S[t], E);
    const bool okD = parse_layout(&dst[t], "dst", t, true, D[t], E);
    if (!okS || !okD) continue;
    if (S[t].ndim != D[t].ndim) {
      E.add(&E.mismatch, "tensor ", t, ": src ndim ", S[t].ndim, " != dst ndim ", D[t].ndim);
      continue;
    }
    for (int i = 0; i < S[t].ndim; ++i)
      if (S[t].shape[i] != D[t].shape[i])
        E.add(&E.mismatch, "tensor ", t, ": global_shape[", i, "] src ", S[t].shape[i], " != dst ",
              D[t].shape[i]);
    if (D[t].quant == RS_Q_MXFP8_E4M3) {
      if (S[t].dtype != RS_BF16)
        E.add(&E.mismatch, "tensor ", t, ": MXFP8 install needs a bf16 source (dtype ",
              S[t].dtype, ")");
      if (D[t].dtype != RS_U8)
        E.add(&E.mismatch, "tensor ", t, ": MXFP8 destination dtype must be RS_U8 (dtype ",
              D[t].dtype, ")");
    } else if (S[t].dtype != D[t].dtype) {
      E.add(&E.mismatch, "tensor ", t, ": src dtype ", S[t].dtype, " != dst dtype ", D[t].dtype);
    }
  }
  for (int t = 0; t < n; ++t) {
    src_base[t] = n_src_ptrs;
    n_src_ptrs += S[t].nptrs;
    dst_base[t] = n_dst_ptrs;
    n_dst_ptrs += D[t].nptrs;
    sc_base[t] = n_dst_ptrs;
    if (D[t].quant == RS_Q_MXFP8_E4M3) n_dst_ptrs += D[t].nptrs;
  }
  // Blockwise-scaled weights: the scale tensor must follow the weight's
  // layouts block for block.
  for (int t = 0; t < n && E.status() == RS_OK; ++t) {
    const int32_t so = src[t].scale_of;
    if (dst[t].scale_of != 0 && dst[t].scale_of != so)
      E.add(&E.invalid, "tensor ", t, ": dst scale_of ", dst[t].scale_of, " differs from src ", so);
    if (so == 0) continue;
    const int w = so - 1;
    if (w < 0 || w >= n || w == t || src[w].scale_of != 0) {
      E.add(&E.invalid, "tensor ", t, ": scale_of ", so, " does not name another, unscaled tensor");
      continue;
    }
    const int nd = S[t].ndim;
    if (S[w].ndim != nd) {
      E.add(&E.mismatch, "tensor ", t, ": scales have ", nd, " dims, weight tensor ", w, " has ",
            S[w].ndim);
      continue;
    }
    int64_t blk[RS_MAX_DIMS];
    bool ok = true;
    for (int d = 0; d < nd; ++d) {
      blk[d] = src[t].scale_block[d];
      if (blk[d] < 1) {
        E.add(&E.invalid, "tensor ", t, ": scale_block[", d, "] = ", blk[d], " < 1");
        ok = false;
      } else if (S[t].shape[d] != (S[w].shape[d] + blk[d] - 1) / blk[d]) {
        E.add(&E.mismatch, "tensor ", t, ": scale extent ", S[t].shape[d], " along dim ", d,
              " is not ceil(", S[w].shape[d], " / ", blk[d], ")");
        ok = false;
      }
    }
    if (!ok) continue;
    const Layout* pairs[2][2] = {{&S[w], &S[t]}, {&D[w], &D[t]}};
    const char* names[2] = {"src", "dst"};
    for (int sd = 0; sd < 2; ++sd) {
      const Layout& W = *pairs[sd][0];
      const Layout& C = *pairs[sd][1];
      bool same = W.mesh_ndim == C.mesh_ndim;
      for (int i = 0; same && i < W.mesh_ndim; ++i)
        same = W.mesh[i] == C.mesh[i] && W.pl[i] == C.pl[i];
      if (!same) {
        E.add(&E.mismatch, "tensor ", t, ": ", names[sd], " mesh/placements differ from weight tensor ", w);
        continue;
      }
      for (int64_t sl = 0; sl < W.nslots; ++sl) {
        const Interval* wb = W.slot_box(sl);
        const Interval* cb = C.slot_box(sl);
        for (int d = 0; d < nd; ++d) {
          const int64_t ws = wb[d].start, we = ws + wb[d].len;
          const int64_t cs = cb[d].start, ce = cs + cb[d].len;
          const bool match = wb[d].len == 0 ? cb[d].len == 0
                                            : (ws == cs * blk[d] && we == std::min(ce * blk[d], W.shape[d]));
          if (!match) {
            E.add(&E.unsupported, "tensor ", t, ": ", names[sd], " slot ", sl, " holds weight [", ws,
                  ", ", we, ") but scales [", cs, ", ", ce, ") along dim ", d, " (block ", blk[d],
                  "): a shard boundary falls inside a scale block");
            break;
          }
        }
      }
    }
  }
  if (E.status() != RS_OK) {
    err = E.text.str();
    return E.status();
  }

  out.src_used.assign(n_src_ptrs, 0);
  out.dst_used.assign(n_dst_ptrs, 0);
  out.src_align.assign(n_src_ptrs, 1);
  out.src_span.assign(n_src_ptrs, 0);
  out.dst_span.assign(n_dst_ptrs, 0);

  // ---- steps 2 and 3: overlap boxes -> byte regions -------------------------
  // Scratch reused across calls on this thread (plans are often rebuilt
  // for the same layouts; keeping capacity avoids fresh allocations).
  struct Target {
    int64_t dslot, sslot;
  };
  struct Scratch {
    std::vector<Target> targets;
    std::vector<uint8_t> done;
    std::vector<size_t> grp;
    std::vector<Raw> raws, split;
    std::vector<uint32_t> cut;
  };
  thread_local Scratch scratch;
  std::vector<Target>& targets = scratch.targets;
  std::vector<uint8_t>& done = scratch.done;
  std::vector<size_t>& grp = scratch.grp;
  std::vector<Raw>& raws = scratch.raws;
  raws.clear();
  for (int t = 0; t < n; ++t) {
    const Layout& A = S[t];
    const Layout& B = D[t];
    const int nd = A.ndim;
    const bool mx = B.quant == RS_Q_MXFP8_E4M3;
    std::vector<Piece> pieces[RS_MAX_DIMS];
    bool empty = false;
    for (int dd = 0; dd < nd; ++dd) {
      pieces[dd] = sweep(A.iv[dd], B.iv[dd]);
      empty |= pieces[dd].empty();
    }
    if (empty) continue;
    if (mx) {
      for (int64_t s = 0; s < A.nptrs; ++s) out.src_align[src_base[t] + s] = 2;
    }
    size_t odo[RS_MAX_DIMS] = {};
    while (true) {
      int64_t si[RS_MAX_DIMS], di[RS_MAX_DIMS], start[RS_MAX_DIMS], len[RS_MAX_DIMS];
      for (int dd = 0; dd < nd; ++dd) {
        const Piece& p = pieces[dd][odo[dd]];
        si[dd] = p.si;
        di[dd] = p.di;
        start[dd] = p.start;
        len[dd] = p.len;
      }
      const int64_t cls = class_ordinal(B, di);
      // Destination slots of this class, each with its source replica.
      targets.clear();
      for (int64_t rep = 0; rep < B.nrep; ++rep) {
        const int64_t dlin = compose_coord(B, di, rep);
        const int64_t dslot = B.coord_to_slot[dlin];
        const int64_t choice = (o.fanout ? cls : dlin) % A.nrep;
        const int64_t slin = compose_coord(A, si, choice);
        targets.push_back({dslot, A.coord_to_slot[slin]});
      }
      // Group destination replicas that read the same source through the same
      // views; each group becomes one region (one read, n_dst writes).
      done.assign(targets.size(), 0);
      for (size_t a = 0; a < targets.size(); ++a) {
        if (done[a]) continue;
        grp.clear();
        grp.push_back(a);
        done[a] = 1;
        if (o.fanout) {
          for (size_t b = a + 1; b < targets.size() && grp.size() < size_t(kMaxFan); ++b) {
            if (done[b] || targets[b].sslot != targets[a].sslot) continue;
            if (!same_view(B.views[targets[b].dslot], B.views[targets[a].dslot], nd)) continue;
            if (mx && !same_view(B.scale_views[targets[b].dslot],
                                 B.scale_views[targets[a].dslot], nd))
              continue;
            grp.push_back(b);
            done[b] = 1;
          }
        }
        const int64_t ss = targets[a].sslot, ds0 = targets[a].dslot;
        const Interval* sb = A.slot_box(ss);
        const Interval* db = B.slot_box(ds0);
        const rs_view& sv = A.views[ss];
        const rs_view& dv = B.views[ds0];
        // A side held as one buffer per dim-0 index takes one region per
        // index of the box along dim 0 (the dim-0 offset picks the buffer).
        const bool split = A.split || B.split;
        const int64_t nparts = split ? len[0] : 1;
        for (int64_t p0 = 0; p0 < nparts; ++p0) {
          int64_t st[RS_MAX_DIMS], ln[RS_MAX_DIMS];
          for (int dd = 0; dd < nd; ++dd) {
            st[dd] = start[dd];
            ln[dd] = len[dd];
          }
          if (split) {
            st[0] = start[0] + p0;
            ln[0] = 1;
          }
          const int64_t s0 = st[0] - sb[0].start, d0 = st[0] - db[0].start;
          Raw& r = raws.emplace_back();  // built in place: a Raw is a few hundred bytes
          r.tensor = t;
          r.mx = mx;
          r.src_index = uint32_t(src_base[t] + (A.split ? A.ptr_base[ss] + s0 : ss));
          r.n_dst = 0;
          for (size_t g : grp) {
            const int64_t dk = targets[g].dslot;
            const int64_t part = B.split ? B.ptr_base[dk] + d0 : dk;
            r.dst_index[r.n_dst] = uint32_t(dst_base[t] + part);
            r.sc_index[r.n_dst] = mx ? uint32_t(sc_base[t] + part) : 0;
            ++r.n_dst;
          }
          int64_t so = sv.base, dof = dv.base, sco = 0;
          for (int dd = A.split ? 1 : 0; dd < nd; ++dd) so += (st[dd] - sb[dd].start) * sv.strides[dd];
          for (int dd = B.split ? 1 : 0; dd < nd; ++dd) dof += (st[dd] - db[dd].start) * dv.strides[dd];
          if (!mx) {
            const uint64_t es = A.esize;
            r.src_off = uint64_t(so) * es;
            r.dst_off = uint64_t(dof) * es;
            r.sc_off = 0;
            r.sc_inner = 0;
            // Element size folds into the innermost run; runs grow while both
            // sides stay contiguous.
            WideDims keep;
            for (int dd = 0; dd < nd; ++dd)
              if (ln[dd] != 1)
                keep.push_back({uint64_t(ln[dd]), uint64_t(sv.strides[dd]) * es,
                                uint64_t(dv.strides[dd]) * es, 0});
            uint64_t run = es;
            while (!keep.empty() && keep.back().ss == run && keep.back().ds == run) {
              run *= keep.back().ext;
              keep.pop_back();
            }
            r.inner = run;
            merge_outer(keep, false);
            set_outer(raws, keep);
          } else {
            const rs_view& cv = B.scale_views[ds0];
            const int last = nd - 1;
            const int64_t c0 = st[last] - db[last].start;
            if ((sv.strides[last] != 1 && ln[last] > 1) || (dv.strides[last] != 1 && ln[last] > 1))
              E.add(&E.unsupported, "tensor ", t,
                    ": MXFP8 install needs a contiguous last dim on both sides");
            for (int dd = B.split ? 1 : 0; dd < last; ++dd)
              sco += (st[dd] - db[dd].start) * cv.strides[dd];
            sco += cv.base;
            // One piece of a destination row box: columns [c0, c0 + inner)
            // from one source shard.  Pieces are cut into regions below,
            // once all pieces of the row box are known.
            r.src_off = uint64_t(so) * 2;
            r.dst_off = uint64_t(dof);
            r.sc_off = 0;
            r.inner = uint64_t(ln[last]);
            r.split = r.inner;
            r.sc_inner = uint64_t(cv.strides[last]);
            r.c0 = uint64_t(c0);
            r.kloc = uint64_t(db[last].len);
            r.drow = uint64_t(dof - c0);
            r.srow = uint64_t(sco);
            // Extent-1 dims dropped, nothing merged: the pieces of one row
            // box (same rows, other sources) must keep the same dims.
            WideDims w;
            for (int dd = 0; dd < last; ++dd)
              if (ln[dd] != 1)
                w.push_back({uint64_t(ln[dd]), uint64_t(sv.strides[dd]) * 2,
                             uint64_t(dv.strides[dd]), uint64_t(cv.strides[dd])});
            set_outer(raws, w);
          }
        }
      }
      int dd = nd - 1;
      while (dd >= 0 && ++odo[dd] == pieces[dd].size()) odo[dd--] = 0;
      if (dd < 0) break;
    }
  }
  if (E.status() != RS_OK) {
    err = E.text.str();
    return E.status();
  }

  // ---- MXFP8 row boxes: pieces -> regions ----------------------------------
  // The pieces of one destination row box (same tensor, destinations,
  // rows) tile its columns [0, kloc) in source-shard order.  Blocks inside
  // one piece become one-source regions; a block that two pieces share (a
  // source shard boundary off the 32-column grid) becomes a two-piece
  // region one block wide, whose kernel work unit gathers the block's
  // values from both sources before taking its amax.
  cut_mx_pieces(raws, E);
  if (E.status() != RS_OK) {
    err = E.text.str();
    return E.status();
  }

  // ---- step 4: split, bucket, size work units ------------------------------
  std::vector<Raw>& split = scratch.split;
  std::vector<uint32_t>& cut = scratch.cut;
  split.clear();
  cut.resize(raws.size());
  // Regions the kernels take as they are (or once cut to unit-sized rows)
  // stay in raws; the pieces of the others go to `split`.  cut[i]: end of
  // raw i's pieces in split, top bit set when raws[i] itself follows them.
  for (size_t i = 0; i < raws.size(); ++i) {
    const bool kept = finalize_at(raws[i], o, split);
    cut[i] = uint32_t(split.size()) | (kept ? 0x80000000u : 0u);
  }

  thread_local std::vector<Final> fin;
  fin.clear();
  fin.reserve(raws.size() + split.size());
  uint64_t bytes_read = 0, bytes_written = 0, bytes_nofan = 0;
  auto add_final = [&](const Raw& r) {
    Final f;
    f.rp = &r;
    f.rows = rows_of(r.outer);
    const int nouter = int(r.outer.size());
    uint64_t ext[3], ss[3], ds[3], sc[3];
    outer_fields(r.outer, ext, ss, ds, sc);
    f.flags = uint32_t(nouter);
    const uint64_t nd = r.n_dst;
    if (r.mx) {
      f.bucket = kMx;
      const uint64_t row_bytes = r.inner * 2;
      // Whole rows per LDS-staged work unit (a long row is one segment).
      const uint64_t rpu = kMxSlots / mx_row_pitch(uint32_t(r.inner));
      f.rows_per_unit = uint32_t(std::min<uint64_t>(rpu, f.rows));
      const uint64_t nb = (r.inner + kMxBlock - 1) / kMxBlock;
      bytes_read += f.rows * row_bytes;
      bytes_written += nd * f.rows * (r.inner + nb);
      bytes_nofan += nd * f.rows * row_bytes;
    } else {
      const uint64_t total = f.rows * r.inner;
      if (packed(ext, ss, nouter, r.inner)) f.flags |= kFlagSrcPacked;
      if (packed(ext, ds, nouter, r.inner)) f.flags |= kFlagDstPacked;
      uint64_t rpu;
      if (total <= o.tiny) {
        f.bucket = kTiny;
        rpu = f.rows;
      } else if (r.inner < o.thin) {
        f.bucket = kThin;
        rpu = std::max<uint64_t>(1, kThinTile / r.inner);
      } else {
        f.bucket = kBulk;
        rpu = std::max<uint64_t>(1, (nd > 1 ? o.unit >> RS_FANOUT_UNIT_SHIFT : o.unit) / r.inner);
        // Whole spread pieces per unit, where that keeps at least half of it.
        const uint64_t m = kSpreadPiece / std::gcd<uint64_t>(r.inner, kSpreadPiece);
        if (kSpread > 1 && rpu >= m) rpu -= rpu % m;
      }
      f.rows_per_unit = uint32_t(std::min<uint64_t>(rpu, f.rows));
      bytes_read += total;
      bytes_written += nd * total;
      bytes_nofan += nd * total;
    }
    f.units = uint32_t((f.rows + f.rows_per_unit - 1) / f.rows_per_unit);
    // Bookkeeping for execute-time checks.
    {
      uint64_t span_s = r.src_off, span_d = r.dst_off, span_c = r.sc_off;
      const uint64_t ib = r.mx ? r.inner * 2 : r.inner;
      const uint64_t ob = r.mx ? r.inner : r.inner;
      for (int k = 0; k < 3; ++k) {
        span_s += (ext[k] - 1) * ss[k];
        span_d += (ext[k] - 1) * ds[k];
        span_c += (ext[k] - 1) * sc[k];
      }
      span_s += ib;
      span_d += ob;
      span_c += r.mx ? ((r.inner + kMxBlock - 1) / kMxBlock - 1) * r.sc_inner + 1 : 0;
      out.src_used[r.src_index] = 1;
      out.src_span[r.src_index] = std::max(out.src_span[r.src_index], span_s);
      for (uint32_t j = 0; j < r.n_dst; ++j) {
        const uint32_t di = r.dst_index[j];
        out.dst_used[di] = 1;
        out.dst_span[di] = std::max(out.dst_span[di], span_d);
        if (r.mx) {
          const uint32_t ci = r.sc_index[j];
          out.dst_used[ci] = 1;
          out.dst_span[ci] = std::max(out.dst_span[ci], span_c);
        }
      }
    }
    fin.push_back(f);
  };
  for (size_t i = 0, sp = 0; i < raws.size(); ++i) {
    for (; sp < (cut[i] & 0x7FFFFFFFu); ++sp) add_final(split[sp]);
    if (cut[i] >> 31) add_final(raws[i]);
  }

  // Copy regions that write the same destination rows side by side (one
  // outer dim, one replica, same destination buffer, rows and row stride,
  // first rows in one destination row: the pieces a source shard boundary
  // cuts a row into) and split them off 128-byte boundaries are cut into
  // chunks of RS_DST_CHUNK units' rows and their chunks interleaved, so the
  // two writes of a 64-byte line that two pieces share land close together
  // in time and meet in the caches instead of reaching HBM as two partial
  // writes.
  thread_local std::deque<Raw> chunk_raws;
  chunk_raws.clear();
  if (RS_DST_CHUNK > 0) {
    auto key_of = [](const Final& f, uint64_t k[4]) -> bool {
      const Raw& r = *f.rp;
      if (f.bucket != kBulk || r.n_dst != 1 || r.outer.size() != 1 || f.rows < 2) return false;
      const Dim& d = r.outer.d[0];
      k[0] = r.dst_index[0];
      k[1] = d.ds;
      k[2] = d.ext;
      k[3] = d.ds ? r.dst_off / d.ds : r.dst_off;
      // Only pieces whose destination rows do not split at 128-byte
      // boundaries: elsewhere no line is written by two pieces.
      return d.ds > r.inner && ((r.dst_off | r.inner | d.ds) & 127u) != 0;
    };
    // Group the candidates by key (sorted, so planning stays n log n), each
    // group led by its first member in plan order.
    struct Cand {
      uint64_t k[4];
      size_t i;
    };
    std::vector<Cand> cand;
    for (size_t i = 0; i < fin.size(); ++i) {
      Cand c;
      if (key_of(fin[i], c.k)) {
        c.i = i;
        cand.push_back(c);
      }
    }
    std::sort(cand.begin(), cand.end(), [](const Cand& x, const Cand& y) {
      for (int q = 0; q < 4; ++q)
        if (x.k[q] != y.k[q]) return x.k[q] < y.k[q];
      return x.i < y.i;
    });
    std::vector<int32_t> group_of_fin(fin.size(), -1);   // group number, -1: none
    std::vector<std::vector<size_t>> groups;
    for (size_t a0 = 0; a0 < cand.size();) {
      size_t a1 = a0 + 1;
      while (a1 < cand.size() && std::equal(cand[a1].k, cand[a1].k + 4, cand[a0].k)) ++a1;
      if (a1 - a0 >= 2) {
        std::vector<size_t> g;
        for (size_t q = a0; q < a1; ++q) {
          g.push_back(cand[q].i);
          group_of_fin[cand[q].i] = int32_t(groups.size());
        }
        groups.push_back(std::move(g));
      }
      a0 = a1;
    }
    std::vector<Final> out_fin;
    out_fin.reserve(fin.size());
    for (size_t i = 0; i < fin.size(); ++i) {
      const int32_t gi = group_of_fin[i];
      if (gi < 0) {
        out_fin.push_back(fin[i]);
        continue;
      }
      const std::vector<size_t>& grp = groups[size_t(gi)];
      if (grp[0] != i) continue;   // emitted with its group's first member
      uint64_t rpu = 1;
      for (size_t q : grp) rpu = std::max<uint64_t>(rpu, fin[q].rows_per_unit);
      const uint64_t C = uint64_t(RS_DST_CHUNK) * rpu, rows = fin[i].rows;
      for (uint64_t c0 = 0; c0 < rows; c0 += C) {
        const uint64_t n = std::min(C, rows - c0);
        for (size_t q : grp) {
          const Final& f = fin[q];
          Raw& r = chunk_raws.emplace_back(*f.rp);
          r.src_off += c0 * r.outer.d[0].ss;
          r.dst_off += c0 * r.outer.d[0].ds;
          r.outer.d[0].ext = n;
          Final g = f;
          g.rp = &r;
          g.rows = n;
          g.rows_per_unit = uint32_t(std::min<uint64_t>(f.rows_per_unit, n));
          g.units = uint32_t((n + g.rows_per_unit - 1) / g.rows_per_unit);
          out_fin.push_back(g);
        }
      }
    }
    fin.swap(out_fin);
  }

  // ---- device image: per bucket, launch groups bounded by the pointer pool --
  out.image.clear();
  out.launches.clear();
  out.region_tensor.clear();
  out.region_tensor.reserve(fin.size());
  out.image.reserve(fin.size() * sizeof(MxRegion) + 8 * 256 + 4 * (fin.size() + 8) +
                    4 * ((bytes_read / o.unit) >> kChunkShift) + 4096);
  uint64_t nreg_bucket[kBuckets] = {}, nunit_bucket[kBuckets] = {};
  std::vector<int32_t> pool_src(n_src_ptrs, -1), pool_dst(n_dst_ptrs, -1);
  // Thin sibling groups (consecutive thin regions reading the same source
  // rows at different columns) and which of them are loaded whole: every
  // member writes packed rows and the group's column span is short.  Those
  // run in launches of their own, with a kernel of their own.
  // Thin regions reading the same source rows (same buffer, row count and
  // outer dims, column offsets within one source row).  Loaded whole, their
  // widths may differ; taking units member-fastest, they must also have
  // equal units.
  auto same_src_rows = [](const Final& x, const Final& y) {
    if (x.rp->src_index != y.rp->src_index || x.rows != y.rows ||
        x.rp->outer.size() != y.rp->outer.size() || x.rp->outer.size() == 0)
      return false;
    uint64_t xe[3], xs[3], xd[3], xc[3], ye[3], ys[3], yd[3], yc[3];
    outer_fields(x.rp->outer, xe, xs, xd, xc);
    outer_fields(y.rp->outer, ye, ys, yd, yc);
    for (int q = 0; q < 3; ++q)
      if (xe[q] != ye[q] || xs[q] != ys[q]) return false;
    const uint64_t a = x.rp->src_off, b = y.rp->src_off;
    return (a > b ? a - b : b - a) < xs[0];
  };
  auto same_units = [](const Final& x, const Final& y) {
    return x.units == y.units && x.rows_per_unit == y.rows_per_unit;
  };
  std::vector<uint32_t> group_of(fin.size(), 0);  // 1 + group number, 0: none
  std::vector<uint8_t> whole(fin.size(), 0);   // 1: loaded whole; 2: loaded whole, narrow members
  if (RS_THIN_SIBLINGS) {
    std::vector<size_t> thin;
    for (size_t q = 0; q < fin.size(); ++q)
      if (fin[q].bucket == kThin) thin.push_back(q);
    uint32_t ng = 0;
    // Members [k, e) become group ng; loaded whole when every member writes
    // packed rows and their column span fits the group tile.
    auto make_group = [&](size_t k, size_t e, bool allow_whole) -> bool {
      bool packed_all = true;
      uint64_t lo = ~uint64_t(0), hi = 0;
      for (size_t q = k; q < e; ++q) {
        const Final& f = fin[thin[q]];
        packed_all &= (f.flags & kFlagDstPacked) != 0;
        lo = std::min(lo, f.rp->src_off);
        hi = std::max(hi, f.rp->src_off + f.rp->inner);
      }
      const bool w = RS_THIN_GROUP_LOAD && packed_all && hi - lo <= kGroupSpanMax;
      if (!w && !allow_whole) return false;
      // Members reading granules of 4 bytes or less from LDS.
      uint64_t wb = hi - lo;
      for (size_t q = k; q < e; ++q) wb |= fin[thin[q]].rp->inner | (fin[thin[q]].rp->src_off - lo);
      ++ng;
      for (size_t q = k; q < e; ++q) {
        group_of[thin[q]] = ng;
        whole[thin[q]] = w ? ((wb & 7u) ? 2 : 1) : 0;
      }
      return true;
    };
    size_t k = 0;
    while (k < thin.size()) {
      size_t e = k + 1;
      while (e < thin.size() && e - k < 255 && same_src_rows(fin[thin[k]], fin[thin[e]])) ++e;
      // The whole run as one group loaded whole, or else runs of members
      // with equal units (loaded whole where they qualify, member-fastest
      // otherwise).
      if (e - k < 2 || !make_group(k, e, false)) {
        size_t q = k;
        while (q < e) {
          size_t r = q + 1;
          while (r < e && same_units(fin[thin[q]], fin[thin[r]])) ++r;
          if (r - q >= 2) make_group(q, r, true);
          q = r;
        }
      }
      k = e;
    }
  }

  // Launch passes: one per bucket, then the thin groups loaded whole (with
  // and without narrow members), then the MXFP8 regions of the second MXFP8
  // kernel (two-piece, or rows at a pitch that is not a power of two).
  // Pooled form (table == false): each launch
  // takes regions in order while their pointers fit the kernel-argument pool
  // of kPool entries (pool_cut tells whether that split any pass).  Table
  // form: no pool limit; pool indices are indices into the caller's
  // pointers, source pointers first, then destination pointers (the device
  // table reshard_execute fills).  record: this form's regions and counts
  // go into the plan summary.
  auto mx_aux = [](const Raw& r) { return r.split < r.inner || mx_pitched(uint32_t(r.inner)); };
  bool pool_cut = false;
  auto emit = [&](bool table, std::vector<uint8_t>& image, std::vector<Launch>& launches, bool record) {
    for (uint32_t pass = 0; pass <= kBuckets + 2; ++pass) {
      const uint32_t kernel = pass;   // launch kind: the buckets, kThinGroup, kThinGroupNarrow, kMxAux
      const uint32_t bucket = bucket_of_kind(kernel);
      const uint8_t want_whole = kernel == kThinGroup ? 1 : kernel == kThinGroupNarrow ? 2 : 0;
      std::vector<const Final*> list;
      list.reserve(fin.size());
      for (size_t q = 0; q < fin.size(); ++q)
        if (fin[q].bucket == bucket && (bucket != kThin || whole[q] == want_whole) &&
            (bucket != kMx || mx_aux(*fin[q].rp) == (kernel == kMxAux)))
          list.push_back(&fin[q]);
      size_t i = 0;
      while (i < list.size()) {
        // Greedy group: regions in order while their pointers fit the pool.
        std::vector<uint32_t> members;    // pool slot -> caller pointer index (| kDstBit)
        std::vector<const Final*> batch;
        if (!table) members.reserve(kPool);
        batch.reserve(list.size() - i);
        uint64_t units = 0;
        while (i < list.size()) {
          const Final* f = list[i];
          if (table) {
            if (!batch.empty() && units + f->units > kMaxUnitsPerLaunch) break;
            batch.push_back(f);
            units += f->units;
            ++i;
            continue;
          }
          uint32_t need[2 + 2 * kMaxFan];
          int nneed = 0;
          need[nneed++] = f->rp->src_index;
          if (f->rp->mx && f->rp->split < f->rp->inner) need[nneed++] = f->rp->src2_index;
          for (uint32_t j = 0; j < f->rp->n_dst; ++j) {
            need[nneed++] = f->rp->dst_index[j] | kDstBit;
            if (f->rp->mx) need[nneed++] = f->rp->sc_index[j] | kDstBit;
          }
          size_t add = 0;
          for (int q = 0; q < nneed; ++q) {
            const uint32_t k = need[q];
            const int32_t at = (k & kDstBit) ? pool_dst[k & ~kDstBit] : pool_src[k];
            if (at < 0) {
              bool dup = false;
              for (int q2 = 0; q2 < q; ++q2) dup |= need[q2] == k;
              add += dup ? 0 : 1;
            }
          }
          if (!batch.empty() && (members.size() + add > size_t(kPool) ||
                               units + f->units > kMaxUnitsPerLaunch)) {
            pool_cut |= members.size() + add > size_t(kPool);
            break;
          }
          for (int q = 0; q < nneed; ++q) {
            const uint32_t k = need[q];
            int32_t& at = (k & kDstBit) ? pool_dst[k & ~kDstBit] : pool_src[k];
            if (at < 0) {
              at = int32_t(members.size());
              members.push_back(k);
            }
          }
          batch.push_back(f);
          units += f->units;
          ++i;
        }
        auto pool = [&](uint32_t k) -> uint16_t {
          if (table) return uint16_t((k & kDstBit) ? n_src_ptrs + (k & ~kDstBit) : k);
          return uint16_t((k & kDstBit) ? pool_dst[k & ~kDstBit] : pool_src[k]);
        };
        Launch L;
        L.bucket = kernel;
        L.n_regions = uint32_t(batch.size());
        L.pool = members;
        L.table = table;
        align_up(image, 256);
        L.regions_off = image.size();
        const size_t rsz = bucket == kMx ? sizeof(MxRegion) : sizeof(CopyRegion);
        image.resize(image.size() + rsz * batch.size(), 0);
        uint32_t ub = 0;
        std::vector<uint32_t> unit_region;
        unit_region.reserve(2 + (units >> kChunkShift));
        // Thin sibling groups: consecutive thin regions that read the same
        // source rows (same source buffer, outer dims and row count, column
        // offsets within one source row) take their units interleaved in the
        // kernel, so the workgroups reading the same rows run together and
        // share the fetched lines.  Flags bits 16-23 hold the group size,
        // bits 24-31 the member index.
        std::vector<uint32_t> sib(batch.size(), 0);
        std::vector<uint32_t> units_k(batch.size()), rpu_k(batch.size());
        for (size_t k = 0; k < batch.size(); ++k) {
          units_k[k] = batch[k]->units;
          rpu_k[k] = batch[k]->rows_per_unit;
        }
        if (bucket == kThin) {
          // Sibling groups of this launch: consecutive members of one group
          // (a group cut by the pointer pool continues in the next launch as
          // a group of its own).  Flags bits 16-23 hold the group size, bits
          // 24-31 the member index.
          size_t k = 0;
          while (k < batch.size()) {
            const uint32_t gid = group_of[size_t(batch[k] - fin.data())];
            size_t e = k + 1;
            while (gid && e < batch.size() && group_of[size_t(batch[e] - fin.data())] == gid) ++e;
            if (e - k >= 2) {
              for (size_t q = k; q < e; ++q) sib[q] = (uint32_t(e - k) << 16) | (uint32_t(q - k) << 24);
              if (kernel == kThinGroup || kernel == kThinGroupNarrow) {
                // The group's units belong to its first member: each unit
                // moves rows_per_unit rows of every member.
                uint64_t lo = ~uint64_t(0), hi = 0;
                for (size_t q = k; q < e; ++q) {
                  lo = std::min(lo, batch[q]->rp->src_off);
                  hi = std::max(hi, batch[q]->rp->src_off + batch[q]->rp->inner);
                }
                const uint64_t rows = batch[k]->rows;
                // Whole 128-byte slot groups per unit where that keeps most of
                // the tile: a contiguous, aligned block then goes straight into
                // LDS (and can be swizzled) whatever the span.
                uint64_t rpu = std::max<uint64_t>(1, kGroupTile / (hi - lo));
                const uint64_t m = 128 / std::gcd<uint64_t>(hi - lo, 128);
                if (rpu >= 2 * m) rpu -= rpu % m;
                rpu = std::min<uint64_t>(rpu, rows);
                for (size_t q = k; q < e; ++q) {
                  sib[q] |= kFlagGroupLoad;
                  rpu_k[q] = uint32_t(rpu);
                  units_k[q] = q == k ? uint32_t((rows + rpu - 1) / rpu) : 0;
                }
              }
            } else if (kernel == kThinGroup || kernel == kThinGroupNarrow) {
              // A lone member left by a pool cut: a group of one.
              sib[k] = kFlagGroupLoad | (1u << 16);
              const uint64_t rows = batch[k]->rows, w = batch[k]->rp->inner;
              uint64_t rpu = std::max<uint64_t>(1, kGroupTile / w);
              const uint64_t m = 128 / std::gcd<uint64_t>(w, 128);
              if (rpu >= 2 * m) rpu -= rpu % m;
              rpu = std::min<uint64_t>(rpu, rows);
              rpu_k[k] = uint32_t(rpu);
              units_k[k] = uint32_t((rows + rpu - 1) / rpu);
            }
            k = e;
          }
        }
        for (size_t k = 0; k < batch.size(); ++k) {
          const Final& f = *batch[k];
          const Raw& r = *f.rp;
          uint64_t ext[3], ss[3], ds[3], sc[3], ss2[3];
          outer_fields(r.outer, ext, ss, ds, sc, ss2);
          uint8_t* dstp = image.data() + L.regions_off + rsz * k;
          if (bucket == kMx) {
            MxRegion m;
            std::memset(&m, 0, sizeof(m));
            m.src_off = r.src_off;
            m.dst_off = r.dst_off;
            m.sc_off = r.sc_off;
            for (int q = 0; q < 3; ++q) {
              m.sstr[q] = ss[q];
              m.dstr[q] = ds[q];
              m.scstr[q] = sc[q];
            }
            m.split = uint32_t(r.split);
            if (r.split < r.inner) {
              m.src2_ptr = pool(r.src2_index);
              m.src2_off = r.src2_off;
              for (int q = 0; q < 3; ++q) m.sstr2[q] = ss2[q];
            }
            m.e0 = uint32_t(ext[0]);
            m.e1 = uint32_t(ext[1]);
            m.rows = uint32_t(f.rows);
            m.inner = uint32_t(r.inner);
            m.rows_per_unit = f.rows_per_unit;
            m.unit_begin = ub;
            m.flags = f.flags;
            m.sc_inner = uint32_t(r.sc_inner);
            m.src_ptr = pool(r.src_index);
            m.n_dst = uint16_t(r.n_dst);
            for (uint32_t j = 0; j < r.n_dst; ++j) {
              m.dst_ptr[j] = pool(r.dst_index[j] | kDstBit);
              m.sc_ptr[j] = pool(r.sc_index[j] | kDstBit);
            }
            std::memcpy(dstp, &m, sizeof(m));
          } else {
            CopyRegion c;
            std::memset(&c, 0, sizeof(c));
            c.src_off = r.src_off;
            c.dst_off = r.dst_off;
            uint64_t al = r.src_off | r.dst_off | r.inner;
            for (int q = 0; q < 3; ++q) {
              c.sstr[q] = ss[q];
              c.dstr[q] = ds[q];
              if (ext[q] > 1) al |= ss[q] | ds[q];
            }
            c.e0 = uint32_t(ext[0]);
            c.e1 = uint32_t(ext[1]);
            c.rows = uint32_t(f.rows);
            c.inner = uint32_t(r.inner);
            c.rows_per_unit = rpu_k[k];
            c.unit_begin = ub;
            c.flags = f.flags | (uint32_t(al & 15) << 8) | sib[k];
            c.src_ptr = pool(r.src_index);
            c.n_dst = uint16_t(r.n_dst);
            for (uint32_t j = 0; j < r.n_dst; ++j) c.dst_ptr[j] = pool(r.dst_index[j] | kDstBit);
            std::memcpy(dstp, &c, sizeof(c));
          }
          if (bucket != kTiny) {
            // Chunk table: the region of every (1 << kChunkShift)-th unit.
            const uint64_t first = (uint64_t(ub) + (1u << kChunkShift) - 1) >> kChunkShift;
            for (uint64_t c = first; (c << kChunkShift) < uint64_t(ub) + units_k[k]; ++c)
              unit_region.push_back(uint32_t(k));
          }
          ub += units_k[k];

          if (record) out.region_tensor.push_back(r.tensor);
        }
        if (bucket == kTiny) {
          L.n_units = uint32_t((batch.size() + kThreads - 1) / kThreads);
          L.units_off = 0;
        } else {
          L.n_units = ub;
          unit_region.push_back(uint32_t(batch.size() - 1));  // entry for unit n_units - 1
          align_up(image, 256);
          L.units_off = image.size();
          image.resize(image.size() + 4 * unit_region.size());
          std::memcpy(image.data() + L.units_off, unit_region.data(), 4 * unit_region.size());
        }
        for (uint32_t k : members) ((k & kDstBit) ? pool_dst[k & ~kDstBit] : pool_src[k]) = -1;
        if (record) {
          nreg_bucket[bucket] += batch.size();
          nunit_bucket[bucket] += L.n_units;
        }
        launches.push_back(std::move(L));
      }
    }
    align_up(image, 256);
  };
  emit(false, out.image, out.launches, true);
  // A plan whose pointers the pool cut into more launches also gets the
  // table form (one launch per pass), which reshard_execute runs once the
  // plan holds a device table of the call's pointers.  Pool indices are 16
  // bits wide, so the caller's pointers must number at most 65,536.
  out.table_image.clear();
  out.table_launches.clear();
  if (pool_cut && n_src_ptrs + n_dst_ptrs <= 65536) {
    out.table_image.reserve(out.image.size());
    emit(true, out.table_image, out.table_launches, false);
  }

  rs_plan_info& I = out.info;
  std::memset(&I, 0, sizeof(I));
  I.n_tensors = uint64_t(n);
  I.n_src_ptrs = n_src_ptrs;
  I.n_dst_ptrs = n_dst_ptrs;
  I.n_regions = out.region_tensor.size();
  for (uint32_t b = 0; b < kBuckets; ++b) {
    I.n_regions_bucket[b] = nreg_bucket[b];
    I.n_units_bucket[b] = nunit_bucket[b];
  }
  I.n_launches = out.table_launches.empty() ? out.launches.size() : out.table_launches.size();
  I.n_launches_pooled = out.launches.size();
  I.bytes_read = bytes_read;
  I.bytes_written = bytes_written;
  I.bytes_read_no_fanout = bytes_nofan;
  I.plan_ns = uint64_t(std::chrono::duration_cast<std::chrono::nanoseconds>(
                           std::chrono::steady_clock::now() - t0)
                           .count());
  return RS_OK;
}

rs_status region_info(const PlanData& d, uint64_t index, rs_region* out) {
  if (index >= d.region_tensor.size()) return RS_ERR_INVALID;
  uint64_t base = 0;
  for (const Launch& L : d.launches) {
    if (index >= base + L.n_regions) {
      base += L.n_regions;
      continue;
    }
    const uint64_t k = index - base;
    std::memset(out, 0, sizeof(*out));
    out->tensor = d.region_tensor[index];
    out->bucket = bucket_of_kind(L.bucket);
    auto user = [&](uint16_t slot) { return L.pool[slot] & ~kDstBit; };
    if (out->bucket == kMx) {
      MxRegion m;
      std::memcpy(&m, d.image.data() + L.regions_off + k * sizeof(MxRegion), sizeof(m));
      out->src_index = user(m.src_ptr);
      out->n_dst = m.n_dst;
      for (uint32_t j = 0; j < m.n_dst; ++j) {
        out->dst_index[j] = user(m.dst_ptr[j]);
        out->scale_index[j] = user(m.sc_ptr[j]);
      }
      out->src_off = m.src_off;
      out->dst_off = m.dst_off;
      out->scale_off = m.sc_off;
      out->inner = m.inner;
      const uint32_t nouter = m.flags & kFlagOuterMask;
      const uint64_t e2 = (nouter >= 3) ? uint64_t(m.rows) / (uint64_t(m.e0) * m.e1) : 1;
      const uint64_t ext[3] = {nouter >= 1 ? m.e0 : 1u, nouter >= 2 ? m.e1 : 1u, e2};
      for (int q = 0; q < 3; ++q) {
        out->ext[q] = ext[q];
        out->src_stride[q] = m.sstr[q];
        out->dst_stride[q] = m.dstr[q];
        out->scale_stride[q] = m.scstr[q];
      }
      out->scale_inner_stride = m.sc_inner;
      out->split = m.split;
      if (m.split < m.inner) {
        out->src2_index = user(m.src2_ptr);
        out->src2_off = m.src2_off;
        for (int q = 0; q < 3; ++q) out->src2_stride[q] = m.sstr2[q];
      }
    } else {
      CopyRegion c;
      std::memcpy(&c, d.image.data() + L.regions_off + k * sizeof(CopyRegion), sizeof(c));
      out->src_index = user(c.src_ptr);
      out->n_dst = c.n_dst;
      for (uint32_t j = 0; j < c.n_dst; ++j) out->dst_index[j] = user(c.dst_ptr[j]);
      out->src_off = c.src_off;
      out->dst_off = c.dst_off;
      out->inner = c.inner;
      out->split = c.inner;
      const uint32_t nouter = c.flags & kFlagOuterMask;
      const uint64_t e2 = (nouter >= 3) ? uint64_t(c.rows) / (uint64_t(c.e0) * c.e1) : 1;
      const uint64_t ext[3] = {nouter >= 1 ? c.e0 : 1u, nouter >= 2 ? c.e1 : 1u, e2};
      for (int q = 0; q < 3; ++q) {
        out->ext[q] = ext[q];
        out->src_stride[q] = c.sstr[q];
        out->dst_stride[q] = c.dstr[q];
      }
    }
    return RS_OK;
  }
  return RS_ERR_INVALID;
}

}  // namespace rs
