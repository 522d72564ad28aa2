// Host-side fuzz of the relayout planner (test infrastructure; no GPU).
//
// Built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_planner_sanitized.py.  For random layouts it
//   1. builds a plan with rs::build_plan,
//   2. replays every region (rs::region_info) on host buffers of exactly the
//      size each slot's view needs, so a region reaching outside its buffer
//      is an AddressSanitizer report (and an explicit check here),
//   3. checks that every destination byte inside a view is written exactly
//      once and every byte outside the views not at all, and that every
//      copied element holds its own global linear index (the sources are
//      filled that way, so replicas hold equal bytes),
// and for corrupted descriptors (bad ranks, placements, permutations, views,
// sizes near the int64 range ...) that the planner returns an error without
// any sanitizer report.
//
// Usage: planner_fuzz <cases> <seed>
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "planner.hpp"

namespace {

uint64_t g_bucket_regions[4] = {};   // regions replayed, per bucket
uint64_t g_valid_rejected = 0;       // uncorrupted cases the planner declined (e.g. MXFP8 blocks across sources)
uint64_t g_sibling_groups = 0;       // thin sibling groups checked
uint64_t g_two_piece = 0;            // MXFP8 regions with two source pieces replayed
uint64_t g_group_loads = 0;          // thin sibling groups loaded whole
uint64_t g_table_forms = 0;          // plans with a table form (pointers from a device table) checked

struct Rng {
  uint64_t s;
  uint64_t next() {  // splitmix64
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int64_t uni(int64_t lo, int64_t hi) { return lo + int64_t(next() % uint64_t(hi - lo + 1)); }
  bool coin(int pct) { return int(next() % 100) < pct; }
};

int esize(int dtype) {
  switch (dtype) {
    case RS_U8: case RS_I8: return 1;
    case RS_U16: case RS_I16: case RS_BF16: case RS_F16: return 2;
    case RS_U32: case RS_I32: case RS_F32: return 4;
    default: return 8;
  }
}

[[noreturn]] void die(const char* what, uint64_t c) {
  std::fprintf(stderr, "case %" PRIu64 ": %s\n", c, what);
  std::exit(1);
}

// One side of one tensor with the storage its pointers refer to.
struct Side {
  rs_tensor_desc d{};
  std::vector<int32_t> perm;
  std::vector<rs_view> views, scale_views;
};

int64_t slots_of(const rs_tensor_desc& d) {
  int64_t n = 1;
  for (int i = 0; i < d.mesh_ndim; ++i) n *= d.mesh_shape[i];
  return n;
}

// Random layout of a tensor of the given global shape.
Side random_side(Rng& g, int ndim, const int64_t* shape, int dtype, bool mx) {
  Side S;
  rs_tensor_desc& d = S.d;
  d.ndim = ndim;
  d.dtype = mx ? RS_U8 : dtype;
  for (int i = 0; i < ndim; ++i) d.global_shape[i] = shape[i];
  d.mesh_ndim = int32_t(g.uni(1, 3));
  for (int i = 0; i < d.mesh_ndim; ++i) {
    d.mesh_shape[i] = g.uni(1, i == 0 ? 4 : 3);
    d.placements[i] = g.coin(30) ? RS_REPLICATE : int32_t(g.uni(0, ndim - 1));
  }
  const int64_t ns = slots_of(d);
  if (g.coin(30)) {
    S.perm.resize(ns);
    for (int64_t i = 0; i < ns; ++i) S.perm[i] = int32_t(i);
    for (int64_t i = ns - 1; i > 0; --i) std::swap(S.perm[i], S.perm[g.uni(0, i)]);
    d.slot_of_coord = S.perm.data();
  }
  d.split_dim0 = g.coin(15) ? 1 : 0;
  d.quant = mx ? RS_Q_MXFP8_E4M3 : RS_Q_NONE;
  std::string err;
  auto padded = [&](std::vector<rs_view>& vs, bool scales) {
    vs.resize(ns);
    for (int64_t s = 0; s < ns; ++s) {
      int64_t off[RS_MAX_DIMS], len[RS_MAX_DIMS];
      if (rs::shard_box(&d, s, off, len, err) != RS_OK) return false;
      if (scales) len[ndim - 1] = (len[ndim - 1] + 31) / 32;
      rs_view& v = vs[s];
      std::memset(&v, 0, sizeof(v));
      v.base = g.uni(0, 5);
      int64_t acc = 1;
      for (int i = ndim - 1; i >= 0; --i) {
        v.strides[i] = acc;
        acc *= len[i] + (i == ndim - 1 && mx && !scales ? 0 : g.uni(0, 2));
      }
    }
    return true;
  };
  // MXFP8 element views keep the last dim contiguous (the planner requires it).
  if (g.coin(25) && padded(S.views, false)) d.views = S.views.data();
  if (mx && g.coin(25) && padded(S.scale_views, true)) d.scale_views = S.scale_views.data();
  return S;
}

// Elements a view spans for a box (0 for an empty box); split parts skip dim 0.
uint64_t span_elems(const rs_view* v, const int64_t* len, int ndim, bool part) {
  uint64_t vol = 1;
  for (int i = 0; i < ndim; ++i) vol *= uint64_t(len[i]);
  if (vol == 0) return 0;
  if (!v) return part ? vol / uint64_t(len[0]) : vol;
  uint64_t hi = uint64_t(v->base);
  for (int i = part ? 1 : 0; i < ndim; ++i) hi += uint64_t(len[i] - 1) * uint64_t(v->strides[i]);
  return hi + 1;
}

struct Buf {
  std::vector<uint8_t> bytes;
  std::vector<uint8_t> writes;  // destination: times each byte was written
};

// One destination buffer and the elements it must receive.
struct DstInfo {
  int tensor, slot, part;  // part -1: whole slot
  bool scale;
};

void put_index(uint8_t* p, uint64_t v, int es) {
  for (int b = 0; b < es; ++b) p[b] = uint8_t(v >> (8 * b));
}

bool run_case(Rng& g, uint64_t c, bool corrupt) {
  const int nt = int(g.uni(1, 3));
  std::vector<Side> src(nt), dst(nt);
  std::vector<int> dtypes(nt);
  std::vector<bool> mx(nt);
  for (int t = 0; t < nt; ++t) {
    // Ranks 1-3 mostly; ranks 4-7 (small extents) give regions with more
    // than three outer dims, which the planner peels.
    const int ndim = g.coin(80) ? int(g.uni(1, 3)) : int(g.uni(4, 7));
    int64_t shape[RS_MAX_DIMS] = {};
    for (int i = 0; i < ndim; ++i)
      shape[i] = g.coin(5) ? 0 : g.uni(1, i == ndim - 1 ? 80 : (ndim > 3 ? 4 : 12));
    mx[t] = ndim >= 2 && g.coin(25);
    static const int kTypes[] = {RS_U8, RS_BF16, RS_I32, RS_F64};
    dtypes[t] = mx[t] ? RS_BF16 : kTypes[g.uni(0, 3)];
    src[t] = random_side(g, ndim, shape, dtypes[t], false);
    dst[t] = random_side(g, ndim, shape, dtypes[t], mx[t]);
  }
  rs_plan_opts opts{};
  opts.struct_size = sizeof(opts);
  opts.fanout = g.coin(80) ? 1 : 0;
  opts.unit_bytes = g.coin(70) ? 0 : (4096u << g.uni(0, 4));
  opts.tiny_bytes = g.coin(50) ? 1024 : (g.coin(50) ? 0 : (g.coin(90) ? uint32_t(g.uni(0, 4096)) : 65536u));
  opts.thin_bytes = g.coin(70) ? 128 : (g.coin(80) ? uint32_t(g.uni(1, 4096)) : uint32_t(g.uni(4096, 16384)));

  std::vector<rs_tensor_desc> S(nt), D(nt);
  for (int t = 0; t < nt; ++t) {
    S[t] = src[t].d;
    D[t] = dst[t].d;
  }
  std::vector<int32_t> bad_perm;
  std::vector<rs_view> bad_views;
  if (corrupt) {
    const int t = int(g.uni(0, nt - 1));
    rs_tensor_desc& x = g.coin(50) ? S[t] : D[t];
    const int64_t huge[] = {int64_t(1) << 31, int64_t(1) << 40, int64_t(1) << 62, INT64_MAX};
    switch (g.uni(0, 13)) {
      case 0: x.ndim = g.coin(50) ? 0 : RS_MAX_DIMS + 1; break;
      case 1: x.dtype = 99; break;
      case 2: x.global_shape[g.uni(0, x.ndim - 1)] = -g.uni(1, 5); break;
      case 3: x.global_shape[g.uni(0, x.ndim - 1)] = huge[g.uni(0, 3)]; break;
      case 4: x.mesh_ndim = g.coin(50) ? 0 : RS_MAX_MESH + 1; break;
      case 5: x.mesh_shape[g.uni(0, x.mesh_ndim - 1)] = g.coin(50) ? -g.uni(0, 3) : huge[g.uni(0, 3)]; break;
      case 6: x.placements[g.uni(0, x.mesh_ndim - 1)] = int32_t(g.uni(x.ndim, RS_MAX_DIMS + 3)); break;
      case 7: {
        const int64_t ns = slots_of(x);
        bad_perm.assign(ns, 0);  // not a permutation unless a single slot
        if (ns == 1) bad_perm[0] = 1;
        x.slot_of_coord = bad_perm.data();
        break;
      }
      case 8: case 9: {
        const int64_t ns = slots_of(x);
        bad_views.assign(ns, rs_view{});
        for (auto& v : bad_views) {
          v.base = 0;
          for (int i = 0; i < RS_MAX_DIMS; ++i) v.strides[i] = 1;
        }
        rs_view& v = bad_views[g.uni(0, ns - 1)];
        if (g.coin(30)) v.base = -1;
        else if (g.coin(50)) v.strides[g.uni(0, x.ndim - 1)] = -g.uni(1, 3);
        else v.strides[g.uni(0, x.ndim - 1)] = huge[g.uni(1, 3)];
        x.views = bad_views.data();
        break;
      }
      case 10: x.quant = 5; break;
      case 11: x.split_dim0 = 2; break;
      case 12: x.scale_of = int32_t(g.uni(nt + 1, nt + 4)); break;
      default: opts.unit_bytes = 3000; break;
    }
  }

  rs::PlanData P;
  std::string err;
  const rs_status st = rs::build_plan(S.data(), D.data(), nt, &opts, P, err);
  if (st != RS_OK) {
    if (err.empty()) die("error status without a message", c);
    if (!corrupt) {
      if (st != RS_ERR_UNSUPPORTED) {
        std::fprintf(stderr, "%s", err.c_str());
        die("a well-formed random layout was rejected as malformed", c);
      }
      ++g_valid_rejected;
    }
    return false;
  }
  // Some corruptions describe valid if unusual layouts (a huge view stride,
  // an enormous extent): the plan is accepted but not replayed on the host.
  if (corrupt) return true;

  // Buffers, in the pointer order of reshard_execute.
  std::vector<Buf> sbuf, dbuf;
  std::vector<DstInfo> dinfo;
  for (int t = 0; t < nt; ++t) {
    const rs_tensor_desc& d = S[t];
    const int es = esize(d.dtype);
    int64_t strides[RS_MAX_DIMS];
    int64_t acc = 1;
    for (int i = d.ndim - 1; i >= 0; --i) {
      strides[i] = acc;
      acc *= d.global_shape[i];
    }
    for (int64_t s = 0; s < slots_of(d); ++s) {
      int64_t off[RS_MAX_DIMS], len[RS_MAX_DIMS];
      if (rs::shard_box(&d, s, off, len, err) != RS_OK) die("shard_box failed on a planned layout", c);
      const rs_view* v = d.views ? &d.views[s] : nullptr;
      const int nparts = d.split_dim0 ? int(len[0]) : 1;
      for (int p = 0; p < nparts; ++p) {
        Buf b;
        b.bytes.assign(span_elems(v, len, d.ndim, d.split_dim0 != 0) * uint64_t(es), 0);
        // fill: every element holds its global linear index
        int64_t idx[RS_MAX_DIMS] = {};
        int64_t vol = 1;
        for (int i = 0; i < d.ndim; ++i) vol *= len[i];
        for (int64_t e = 0; e < vol; ++e) {
          int64_t r = e;
          for (int i = d.ndim - 1; i >= 0; --i) {
            idx[i] = r % len[i];
            r /= len[i];
          }
          if (d.split_dim0 && idx[0] != p) continue;
          uint64_t gl = 0, lo = v ? uint64_t(v->base) : 0;
          for (int i = 0; i < d.ndim; ++i) gl += uint64_t(off[i] + idx[i]) * uint64_t(strides[i]);
          if (v) {
            for (int i = d.split_dim0 ? 1 : 0; i < d.ndim; ++i) lo += uint64_t(idx[i]) * uint64_t(v->strides[i]);
          } else {
            uint64_t a2 = 1;
            for (int i = d.ndim - 1; i >= (d.split_dim0 ? 1 : 0); --i) {
              lo += uint64_t(idx[i]) * a2;
              a2 *= uint64_t(len[i]);
            }
          }
          put_index(&b.bytes[lo * es], gl, es);
        }
        sbuf.push_back(std::move(b));
      }
    }
  }
  for (int t = 0; t < nt; ++t) {
    const rs_tensor_desc& d = D[t];
    const int es = mx[t] ? 1 : esize(d.dtype);
    for (int pass = 0; pass < (mx[t] ? 2 : 1); ++pass) {
      const bool scale = pass == 1;
      for (int64_t s = 0; s < slots_of(d); ++s) {
        int64_t off[RS_MAX_DIMS], len[RS_MAX_DIMS];
        if (rs::shard_box(&d, s, off, len, err) != RS_OK) die("shard_box failed on a planned layout", c);
        const int nparts = d.split_dim0 ? int(len[0]) : 1;
        if (scale) len[d.ndim - 1] = (len[d.ndim - 1] + 31) / 32;
        const rs_view* v = scale ? (d.scale_views ? &d.scale_views[s] : nullptr)
                                 : (d.views ? &d.views[s] : nullptr);
        for (int p = 0; p < nparts; ++p) {
          Buf b;
          const uint64_t n = span_elems(v, len, d.ndim, d.split_dim0 != 0) * uint64_t(es);
          b.bytes.assign(n, 0xA5);
          b.writes.assign(n, 0);
          dbuf.push_back(std::move(b));
          dinfo.push_back({t, int(s), d.split_dim0 ? p : -1, scale});
        }
      }
    }
  }
  if (sbuf.size() != P.info.n_src_ptrs || dbuf.size() != P.info.n_dst_ptrs)
    die("pointer counts differ from the documented order", c);

  // Work units as the copy kernels take them: every launch's units cover
  // each of its regions' units exactly once.  Thin sibling groups (flags
  // bits 16-31) must be consecutive regions with equal unit counts, which
  // the thin kernel relies on when it takes their units member-fastest.
  auto walk_units = [&](const std::vector<rs::Launch>& launches, const std::vector<uint8_t>& image) {
  for (const rs::Launch& L : launches) {
    if (L.bucket == rs::kTiny || rs::bucket_of_kind(L.bucket) == rs::kMx) {
      if (L.bucket == rs::kMx || L.bucket == rs::kMxAux) {
        // MXFP8 launches: the second kind holds exactly the two-piece
        // regions and those whose rows take a pitch that is not a power of
        // two (a two-piece region, one block wide, never does).
        const rs::MxRegion* mr = reinterpret_cast<const rs::MxRegion*>(image.data() + L.regions_off);
        for (uint32_t k = 0; k < L.n_regions; ++k) {
          const bool two = mr[k].split < mr[k].inner, pitched = rs::mx_pitched(mr[k].inner);
          if ((two || pitched) != (L.bucket == rs::kMxAux)) die("MXFP8 region in the wrong launch kind", c);
          if (two && pitched) die("two-piece region at a pitch", c);
          if (mr[k].rows_per_unit != std::min<uint32_t>(mr[k].rows, rs::kMxSlots / rs::mx_row_pitch(mr[k].inner)))
            die("MXFP8 rows per unit", c);
        }
      }
      continue;
    }
    const rs::CopyRegion* regs = reinterpret_cast<const rs::CopyRegion*>(image.data() + L.regions_off);
    std::vector<std::vector<uint8_t>> seen(L.n_regions);
    for (uint32_t k = 0; k < L.n_regions; ++k) {
      const uint32_t nu = (regs[k].rows + regs[k].rows_per_unit - 1) / regs[k].rows_per_unit;
      const uint32_t gm = (regs[k].flags >> 16) & 255u, m = regs[k].flags >> 24;
      const bool whole = (regs[k].flags & rs::kFlagGroupLoad) != 0;
      // A group loaded whole: its first member takes all of the group's
      // units (rows_per_unit rows of every member each), the others none.
      seen[k].assign(whole && m ? 0 : nu, 0);
      const bool group_launch = L.bucket == rs::kThinGroup || L.bucket == rs::kThinGroupNarrow;
      if (L.bucket != rs::kThin && !group_launch && gm) die("sibling group outside the thin bucket", c);
      if ((gm == 1 && !whole) || (gm && m >= gm) || (!gm && m)) die("bad sibling group fields", c);
      if (whole != group_launch) die("group-load flag outside its launch kind", c);
      if (whole && !gm) die("group-load flag outside a sibling group", c);
      if (gm && (k < m || k - m + gm > L.n_regions)) die("sibling group leaves its launch", c);
      if (gm && m == 0) ++g_sibling_groups;
      if (whole && m == 0) ++g_group_loads;
      if (gm) {
        const rs::CopyRegion& h = regs[k - m];
        const uint32_t want_ub = whole ? h.unit_begin + (m ? nu : 0) : h.unit_begin + m * nu;
        if (((h.flags >> 16) & 255u) != gm || (h.flags >> 24) != 0 || h.rows != regs[k].rows ||
            h.rows_per_unit != regs[k].rows_per_unit || want_ub != regs[k].unit_begin ||
            ((h.flags ^ regs[k].flags) & rs::kFlagGroupLoad))
          die("sibling group members differ", c);
        if (whole) {
          // The group's column span fits the thin kernel's LDS tile.
          uint64_t lo = ~uint64_t(0), hi = 0;
          for (uint32_t q = 0; q < gm; ++q) {
            lo = std::min<uint64_t>(lo, regs[k - m + q].src_off);
            hi = std::max<uint64_t>(hi, regs[k - m + q].src_off + regs[k - m + q].inner);
            if (!(regs[k - m + q].flags & rs::kFlagDstPacked)) die("group-load member not packed", c);
          }
          if (hi - lo > rs::kGroupSpanMax || uint64_t(h.rows_per_unit) * (hi - lo) > rs::kGroupTile)
            die("group-load span exceeds the LDS tile", c);
        }
      }
    }
    for (uint32_t u = 0; u < L.n_units; ++u) {
      uint32_t k = 0;
      while (k + 1 < L.n_regions && regs[k + 1].unit_begin <= u) ++k;
      uint32_t ul = u - regs[k].unit_begin;
      const uint32_t gm = (regs[k].flags >> 16) & 255u;
      if (gm > 1 && !(regs[k].flags & rs::kFlagGroupLoad)) {
        const uint32_t m = regs[k].flags >> 24;
        const uint32_t nu = (regs[k].rows + regs[k].rows_per_unit - 1) / regs[k].rows_per_unit;
        const uint32_t local = ul + m * nu;
        k = k - m + local % gm;
        ul = local / gm;
      }
      if (ul >= seen[k].size() || seen[k][ul]++) die("a work unit is missed or taken twice", c);
    }
    for (const auto& v : seen)
      for (uint8_t x : v)
        if (x != 1) die("a work unit is not taken", c);
  }
  };
  walk_units(P.launches, P.image);
  // Table form (a plan whose pointers the kernel-argument pool cut into
  // several launches of one kind): the same regions in the same order, one
  // launch per kind, every pool index the caller's pointer index (sources
  // first) that the pooled form's pool slot names.  Sibling-group fields and
  // units may differ where the pool cut a group.
  if (!P.table_launches.empty()) {
    ++g_table_forms;
    if (P.info.n_launches != P.table_launches.size() || P.info.n_launches_pooled != P.launches.size() ||
        P.table_launches.size() >= P.launches.size())
      die("table form launch counts", c);
    walk_units(P.table_launches, P.table_image);
    const uint64_t ns = P.info.n_src_ptrs;
    auto caller = [&](const rs::Launch& L, uint16_t slot) -> uint64_t {
      if (slot >= L.pool.size()) die("pool slot out of range", c);
      const uint32_t e = L.pool[slot];
      return (e & rs::kDstBit) ? ns + (e & ~rs::kDstBit) : e;
    };
    size_t ti = 0, tk = 0;
    for (const rs::Launch& L : P.launches) {
      if (L.table) die("pooled launch marked as table form", c);
      for (uint32_t k = 0; k < L.n_regions; ++k, ++tk) {
        while (ti < P.table_launches.size() && tk >= P.table_launches[ti].n_regions) {
          tk = 0;
          ++ti;
        }
        if (ti >= P.table_launches.size()) die("table form has fewer regions", c);
        const rs::Launch& T = P.table_launches[ti];
        if (!T.table || !T.pool.empty() || T.bucket != L.bucket) die("table launch fields", c);
        if (rs::bucket_of_kind(L.bucket) == rs::kMx) {
          rs::MxRegion a, b;
          std::memcpy(&a, P.image.data() + L.regions_off + k * sizeof(a), sizeof(a));
          std::memcpy(&b, P.table_image.data() + T.regions_off + tk * sizeof(b), sizeof(b));
          bool same = a.src_off == b.src_off && a.dst_off == b.dst_off && a.sc_off == b.sc_off &&
                      a.e0 == b.e0 && a.e1 == b.e1 && a.rows == b.rows && a.inner == b.inner &&
                      a.rows_per_unit == b.rows_per_unit && a.flags == b.flags && a.sc_inner == b.sc_inner &&
                      a.n_dst == b.n_dst && a.split == b.split && caller(L, a.src_ptr) == b.src_ptr;
          for (int q = 0; q < 3; ++q)
            same &= a.sstr[q] == b.sstr[q] && a.dstr[q] == b.dstr[q] && a.scstr[q] == b.scstr[q];
          for (uint32_t j = 0; j < a.n_dst; ++j)
            same &= caller(L, a.dst_ptr[j]) == b.dst_ptr[j] && caller(L, a.sc_ptr[j]) == b.sc_ptr[j];
          if (a.split < a.inner) {
            same &= caller(L, a.src2_ptr) == b.src2_ptr && a.src2_off == b.src2_off;
            for (int q = 0; q < 3; ++q) same &= a.sstr2[q] == b.sstr2[q];
          }
          if (!same) die("table form MXFP8 region differs", c);
        } else {
          rs::CopyRegion a, b;
          std::memcpy(&a, P.image.data() + L.regions_off + k * sizeof(a), sizeof(a));
          std::memcpy(&b, P.table_image.data() + T.regions_off + tk * sizeof(b), sizeof(b));
          bool same = a.src_off == b.src_off && a.dst_off == b.dst_off && a.e0 == b.e0 && a.e1 == b.e1 &&
                      a.rows == b.rows && a.inner == b.inner && (a.flags & 0xFFFu) == (b.flags & 0xFFFu) &&
                      a.n_dst == b.n_dst && caller(L, a.src_ptr) == b.src_ptr;
          if (L.bucket != rs::kThin && L.bucket != rs::kThinGroup && L.bucket != rs::kThinGroupNarrow)
            same &= a.rows_per_unit == b.rows_per_unit && a.flags == b.flags;
          for (int q = 0; q < 3; ++q) same &= a.sstr[q] == b.sstr[q] && a.dstr[q] == b.dstr[q];
          for (uint32_t j = 0; j < a.n_dst; ++j) same &= caller(L, a.dst_ptr[j]) == b.dst_ptr[j];
          if (!same) die("table form region differs", c);
        }
      }
    }
    if (ti + 1 != P.table_launches.size() || tk != P.table_launches.back().n_regions)
      die("table form has more regions", c);
  } else if (P.info.n_launches != P.launches.size() || P.info.n_launches_pooled != P.launches.size()) {
    die("launch counts", c);
  }

  // Replay every region.
  for (uint64_t k = 0; k < P.info.n_regions; ++k) {
    rs_region R;
    if (rs::region_info(P, k, &R) != RS_OK) die("region_info failed", c);
    if (R.src_index >= sbuf.size() || R.n_dst < 1 || R.n_dst > RS_MAX_FANOUT || R.bucket > 3)
      die("bad region fields", c);
    ++g_bucket_regions[R.bucket];
    const bool isq = R.bucket == 3;
    const uint64_t rows = R.ext[0] * R.ext[1] * R.ext[2];
    const bool two = isq && R.split < R.inner;
    if (R.split > R.inner || (!isq && R.split != R.inner)) die("bad split", c);
    if (two && (R.inner > 32 || R.src2_index >= sbuf.size())) die("bad two-piece region", c);
    if (two) ++g_two_piece;
    const uint64_t rd = isq ? 2 * R.split : R.inner;
    const uint64_t nb = isq ? (R.inner + 31) / 32 : 0;
    for (uint64_t r = 0; r < rows; ++r) {
      const uint64_t i0 = r % R.ext[0], i1 = (r / R.ext[0]) % R.ext[1], i2 = r / (R.ext[0] * R.ext[1]);
      const uint64_t so = R.src_off + i0 * R.src_stride[0] + i1 * R.src_stride[1] + i2 * R.src_stride[2];
      const Buf& sb = sbuf[R.src_index];
      if (so + rd > sb.bytes.size()) die("region reads past its source buffer", c);
      if (two) {
        const uint64_t so2 = R.src2_off + i0 * R.src2_stride[0] + i1 * R.src2_stride[1] +
                             i2 * R.src2_stride[2];
        if (so2 + 2 * (R.inner - R.split) > sbuf[R.src2_index].bytes.size())
          die("region reads past its second source buffer", c);
      }
      for (uint32_t j = 0; j < R.n_dst; ++j) {
        if (R.dst_index[j] >= dbuf.size()) die("bad destination index", c);
        Buf& db = dbuf[R.dst_index[j]];
        const uint64_t o = R.dst_off + i0 * R.dst_stride[0] + i1 * R.dst_stride[1] + i2 * R.dst_stride[2];
        if (o + R.inner > db.bytes.size()) die("region writes past its destination buffer", c);
        if (!isq) std::memcpy(&db.bytes[o], &sb.bytes[so], R.inner);
        for (uint64_t b = 0; b < R.inner; ++b) ++db.writes[o + b];
        if (isq) {
          if (R.scale_index[j] >= dbuf.size()) die("bad scale index", c);
          Buf& cb = dbuf[R.scale_index[j]];
          const uint64_t co = R.scale_off + i0 * R.scale_stride[0] + i1 * R.scale_stride[1] +
                              i2 * R.scale_stride[2];
          for (uint64_t b = 0; b < nb; ++b) {
            const uint64_t q = co + b * R.scale_inner_stride;
            if (q >= cb.bytes.size()) die("region writes past its scale buffer", c);
            ++cb.writes[q];
          }
        }
      }
    }
  }

  // Every destination element written exactly once, nothing else; copies
  // hold their global index.
  for (size_t bi = 0; bi < dbuf.size(); ++bi) {
    const DstInfo& di = dinfo[bi];
    const rs_tensor_desc& d = D[di.tensor];
    const int es = mx[di.tensor] ? 1 : esize(d.dtype);
    int64_t off[RS_MAX_DIMS], len[RS_MAX_DIMS];
    rs::shard_box(&d, di.slot, off, len, err);
    if (di.scale) len[d.ndim - 1] = (len[d.ndim - 1] + 31) / 32;
    const rs_view* v = di.scale ? (d.scale_views ? &d.scale_views[di.slot] : nullptr)
                                : (d.views ? &d.views[di.slot] : nullptr);
    int64_t gstr[RS_MAX_DIMS];
    int64_t acc = 1;
    for (int i = d.ndim - 1; i >= 0; --i) {
      gstr[i] = acc;
      acc *= d.global_shape[i];
    }
    std::vector<uint8_t> expect_writes(dbuf[bi].bytes.size(), 0);
    int64_t vol = 1;
    for (int i = 0; i < d.ndim; ++i) vol *= len[i];
    for (int64_t e = 0; e < vol; ++e) {
      int64_t idx[RS_MAX_DIMS], r = e;
      for (int i = d.ndim - 1; i >= 0; --i) {
        idx[i] = r % len[i];
        r /= len[i];
      }
      if (di.part >= 0 && idx[0] != di.part) continue;
      uint64_t lo = v ? uint64_t(v->base) : 0;
      if (v) {
        for (int i = di.part >= 0 ? 1 : 0; i < d.ndim; ++i) lo += uint64_t(idx[i]) * uint64_t(v->strides[i]);
      } else {
        uint64_t a2 = 1;
        for (int i = d.ndim - 1; i >= (di.part >= 0 ? 1 : 0); --i) {
          lo += uint64_t(idx[i]) * a2;
          a2 *= uint64_t(len[i]);
        }
      }
      for (int b = 0; b < es; ++b) expect_writes[lo * es + b] = 1;
      if (!mx[di.tensor]) {
        uint64_t gl = 0;
        for (int i = 0; i < d.ndim; ++i) gl += uint64_t(off[i] + idx[i]) * uint64_t(gstr[i]);
        uint8_t want[8];
        put_index(want, gl, es);
        if (std::memcmp(&dbuf[bi].bytes[lo * es], want, es) != 0) die("wrong value in a destination", c);
      }
    }
    if (expect_writes != dbuf[bi].writes) die("a destination byte is written other than once", c);
  }
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t cases = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1000;
  const uint64_t seed = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1;
  uint64_t planned = 0, rejected = 0, corrupt_ok = 0;
  for (uint64_t c = 0; c < cases; ++c) {
    Rng g{seed * 0x100000001B3ull + c};
    const bool corrupt = g.coin(35);
    const bool ok = run_case(g, c, corrupt);
    if (ok && !corrupt) ++planned;
    else if (ok) ++corrupt_ok;
    else ++rejected;
  }
  std::printf("cases %" PRIu64 ": planned and replayed %" PRIu64 ", rejected %" PRIu64
              " (%" PRIu64 " of them uncorrupted, unsupported), corrupted but accepted %" PRIu64
              "; regions replayed: bulk %" PRIu64 ", thin %" PRIu64 ", tiny %" PRIu64 ", mxfp8 %" PRIu64
              "; thin sibling groups %" PRIu64 " (loaded whole %" PRIu64 "); two-piece MXFP8 regions %" PRIu64
              "; table forms %" PRIu64 "\n",
              cases, planned, rejected, g_valid_rejected, corrupt_ok, g_bucket_regions[0],
              g_bucket_regions[1], g_bucket_regions[2], g_bucket_regions[3], g_sibling_groups, g_group_loads, g_two_piece,
              g_table_forms);
  return 0;
}
