// C ABI of the relayout library: plan objects, argument checks, device table
// upload and kernel launches.  See include/reshard.h for the contract.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <sstream>
#include <string>
#include <vector>

#include "planner.hpp"
#include "reshard.h"
#include "rs_device.hpp"

namespace rs {
// Enqueues one launch of a bucket's kernel on `stream`, whose device is `dev`
// (pointers in the arguments, or in a device table).
hipError_t launch(uint32_t bucket, uint32_t grid, const LaunchArgs& args, hipStream_t stream, int dev);
hipError_t launch(uint32_t bucket, uint32_t grid, const TableArgs& args, hipStream_t stream, int dev);
// Device address of the library's static table area on device `dev` (see
// kernels.hip); looked up once per device.
hipError_t table_area(int dev, char** out);
extern const uint64_t kTableAreaBytes;
}

struct rs_plan {
  rs::PlanData d;
  mutable std::mutex mu;
  struct DevTable {
    int device;
    void* ptr;
  };
  mutable std::vector<DevTable> tables;  // one upload of d.image (+ d.table_image) per device
  // Device tables of the caller's pointers for the table form of the
  // launches: one per pointer set a device has seen, immutable once
  // uploaded, at most kMaxPointerSets per device.
  struct PtrTable {
    int device;
    std::vector<void*> ptrs;  // sources then destinations; NULL where no region reads it
    void* ptr;
  };
  mutable std::vector<PtrTable> ptr_tables;
  static constexpr int kMaxPointerSets = 8;
};

namespace {

thread_local std::string g_error;

rs_status fail(rs_status s, const std::string& msg) {
  g_error = msg;
  return s;
}

bool debug_checks() {
  const char* e = std::getenv("RESHARD_DEBUG_CHECKS");
  return e && e[0] == '1';
}

}  // namespace

extern "C" {

rs_status reshard_plan(const rs_tensor_desc* src, const rs_tensor_desc* dst, int32_t n_tensors,
                       const rs_plan_opts* opts, rs_plan** out) {
  g_error.clear();
  if (!out) return fail(RS_ERR_INVALID, "out is NULL\n");
  *out = nullptr;
  rs_plan* p = new (std::nothrow) rs_plan();
  if (!p) return fail(RS_ERR_ALLOC, "cannot allocate a plan\n");
  std::string err;
  rs_status st;
  try {
    st = rs::build_plan(src, dst, n_tensors, opts, p->d, err);
  } catch (const std::bad_alloc&) {
    st = RS_ERR_ALLOC;
    err = "host allocation failed while planning\n";
  }
  if (st != RS_OK) {
    delete p;
    return fail(st, err);
  }
  *out = p;
  return RS_OK;
}

}  // extern "C"

namespace {

// Device tables of a plan on `dev`, uploaded on first use (blocking).
rs_status plan_tables(const rs_plan* plan, int dev, char** base) {
  std::lock_guard<std::mutex> lock(plan->mu);
  for (const auto& t : plan->tables)
    if (t.device == dev) {
      *base = static_cast<char*>(t.ptr);
      return RS_OK;
    }
  int cur = 0;
  hipError_t he = hipGetDevice(&cur);
  if (he != hipSuccess) return fail(RS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(he) + "\n");
  if (cur != dev && (he = hipSetDevice(dev)) != hipSuccess)
    return fail(RS_ERR_HIP, std::string("hipSetDevice: ") + hipGetErrorString(he) + "\n");
  // The table form's regions follow the pooled form's (whose image ends on
  // a 256-byte boundary).
  const std::vector<uint8_t>& img = plan->d.image;
  const std::vector<uint8_t>& timg = plan->d.table_image;
  void* p = nullptr;
  rs_status st = RS_OK;
  std::string msg;
  he = hipMalloc(&p, img.size() + timg.size());
  if (he != hipSuccess) {
    st = RS_ERR_ALLOC;
    msg = std::string("hipMalloc of the plan tables: ") + hipGetErrorString(he) + "\n";
  } else if ((he = hipMemcpy(p, img.data(), img.size(), hipMemcpyHostToDevice)) != hipSuccess ||
             (!timg.empty() && (he = hipMemcpy(static_cast<char*>(p) + img.size(), timg.data(), timg.size(),
                                               hipMemcpyHostToDevice)) != hipSuccess)) {
    (void)hipFree(p);
    st = RS_ERR_HIP;
    msg = std::string("upload of the plan tables: ") + hipGetErrorString(he) + "\n";
  } else {
    plan->tables.push_back({dev, p});
    *base = static_cast<char*>(p);
  }
  if (cur != dev) (void)hipSetDevice(cur);
  return st == RS_OK ? RS_OK : fail(st, msg);
}

// Device table of this call's pointers for the table form of the launches,
// or NULL to run the pooled form: found among the tables of the pointer
// sets the plan has seen on device `dev`, else uploaded (a blocking
// allocation and copy) while the device holds fewer than kMaxPointerSets
// and `stream` is not capturing a graph.  An allocation or copy that fails
// leaves the pooled form to run; it is not an error.
void* pointer_table(const rs_plan* plan, int dev, void* const* src_ptrs, void* const* dst_ptrs,
                    hipStream_t stream) {
  const rs::PlanData& d = plan->d;
  const size_t ns = d.src_used.size(), nd = d.dst_used.size();
  std::vector<void*> want(ns + nd, nullptr);
  for (size_t i = 0; i < ns; ++i)
    if (d.src_used[i]) want[i] = src_ptrs[i];
  for (size_t i = 0; i < nd; ++i)
    if (d.dst_used[i]) want[ns + i] = dst_ptrs[i];
  std::lock_guard<std::mutex> lock(plan->mu);
  int seen = 0;
  for (const auto& t : plan->ptr_tables) {
    if (t.device != dev) continue;
    ++seen;
    if (t.ptrs == want) return t.ptr;
  }
  if (seen >= rs_plan::kMaxPointerSets) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return nullptr;
  }
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess || (cur != dev && hipSetDevice(dev) != hipSuccess)) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = nullptr;
  const size_t bytes = want.size() * sizeof(void*);
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    p = nullptr;
  } else if (hipMemcpy(p, want.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p);
    p = nullptr;
  }
  if (cur != dev) (void)hipSetDevice(cur);
  if (p) plan->ptr_tables.push_back({dev, std::move(want), p});
  return p;
}

// Where execute() finds the plan's device tables.
enum class Tables {
  kPlanOwned,   // uploaded once per device into an allocation the plan owns
  kStaticArea,  // copied on every call into the library's static area (no allocation)
};

rs_status execute(const rs_plan* plan, void* const* src_ptrs, void* const* dst_ptrs, void* stream,
                  Tables where) {
  if (!plan) return fail(RS_ERR_INVALID, "plan is NULL\n");
  const rs::PlanData& d = plan->d;
  std::ostringstream err;
  int nerr = 0;
  if (d.info.n_src_ptrs && !src_ptrs) {
    err << "src_ptrs is NULL but the plan has " << d.info.n_src_ptrs << " source slots\n";
    ++nerr;
  }
  if (d.info.n_dst_ptrs && !dst_ptrs) {
    err << "dst_ptrs is NULL but the plan has " << d.info.n_dst_ptrs << " destination slots\n";
    ++nerr;
  }
  if (nerr) return fail(RS_ERR_INVALID, err.str());
  for (size_t i = 0; i < d.src_used.size(); ++i) {
    if (d.src_used[i] && !src_ptrs[i]) {
      err << "src_ptrs[" << i << "] is NULL but that source slot is read\n";
      ++nerr;
    } else if (src_ptrs[i] && reinterpret_cast<uintptr_t>(src_ptrs[i]) % d.src_align[i]) {
      err << "src_ptrs[" << i << "] is not aligned to its element size " << int(d.src_align[i])
          << "\n";
      ++nerr;
    }
  }
  for (size_t i = 0; i < d.dst_used.size(); ++i)
    if (d.dst_used[i] && !dst_ptrs[i]) {
      err << "dst_ptrs[" << i << "] is NULL but that destination slot is written\n";
      ++nerr;
    }
  if (!nerr && debug_checks()) {
    // Sources and destinations must not overlap (byte ranges each pointer's
    // regions reach).
    for (size_t i = 0; i < d.src_used.size(); ++i) {
      if (!d.src_used[i]) continue;
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(src_ptrs[i]), a1 = a0 + d.src_span[i];
      for (size_t j = 0; j < d.dst_used.size(); ++j) {
        if (!d.dst_used[j]) continue;
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(dst_ptrs[j]), b1 = b0 + d.dst_span[j];
        if (a0 < b1 && b0 < a1) {
          err << "src_ptrs[" << i << "] and dst_ptrs[" << j << "] overlap\n";
          ++nerr;
        }
      }
    }
  }
  if (nerr) return fail(RS_ERR_INVALID, err.str());
  if (where == Tables::kStaticArea && d.image.size() > rs::kTableAreaBytes) {
    err << "the plan's device tables take " << d.image.size() << " bytes, more than the "
        << rs::kTableAreaBytes << "-byte static table area of reshard_execute_no_alloc "
        << "(use reshard_execute)\n";
    return fail(RS_ERR_UNSUPPORTED, err.str());
  }
  if (d.launches.empty()) return RS_OK;

  // The kernels run on the stream's device, so the tables must live there.
  int dev = 0;
  hipError_t he = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (he != hipSuccess)
    return fail(RS_ERR_HIP, std::string("device of the stream: ") + hipGetErrorString(he) + "\n");
  if (debug_checks()) {
    // Every pointer is device memory of the stream's device, with room for
    // every byte its regions reach (a short buffer would fault the GPU).
    auto check = [&](const char* side, size_t i, void* p, uint64_t span) {
      hipDeviceptr_t base = nullptr;
      size_t size = 0;
      hipPointerAttribute_t attr;
      hipError_t e = hipMemGetAddressRange(&base, &size, p);
      if (e == hipSuccess) e = hipPointerGetAttributes(&attr, p);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        err << side << "[" << i << "] is not device memory (" << hipGetErrorString(e) << ")\n";
        ++nerr;
        return;
      }
      const uintptr_t end = reinterpret_cast<uintptr_t>(base) + size, at = reinterpret_cast<uintptr_t>(p);
      if (at + span > end) {
        err << side << "[" << i << "] needs " << span << " bytes but its allocation ends " << (end - at)
            << " bytes after it\n";
        ++nerr;
      }
      if (attr.type == hipMemoryTypeDevice && attr.device != dev) {
        err << side << "[" << i << "] is memory of device " << attr.device << ", the stream runs on device "
            << dev << "\n";
        ++nerr;
      }
    };
    for (size_t i = 0; i < d.src_used.size(); ++i)
      if (d.src_used[i]) check("src_ptrs", i, src_ptrs[i], d.src_span[i]);
    for (size_t i = 0; i < d.dst_used.size(); ++i)
      if (d.dst_used[i]) check("dst_ptrs", i, dst_ptrs[i], d.dst_span[i]);
    if (nerr) return fail(RS_ERR_INVALID, err.str());
  }
  char* base = nullptr;
  void* ptab = nullptr;
  if (where == Tables::kPlanOwned) {
    const rs_status ts = plan_tables(plan, dev, &base);
    if (ts != RS_OK) return ts;
    if (!d.table_launches.empty())
      ptab = pointer_table(plan, dev, src_ptrs, dst_ptrs, static_cast<hipStream_t>(stream));
  } else {
    he = rs::table_area(dev, &base);
    if (he != hipSuccess)
      return fail(RS_ERR_HIP, std::string("address of the static table area: ") + hipGetErrorString(he) + "\n");
    // Stream-ordered: earlier work on this stream (a previous call's
    // kernels) has finished reading the area before the copy lands.
    he = hipMemcpyAsync(base, d.image.data(), d.image.size(), hipMemcpyHostToDevice,
                        static_cast<hipStream_t>(stream));
    if (he != hipSuccess)
      return fail(RS_ERR_HIP, std::string("copy of the plan tables: ") + hipGetErrorString(he) + "\n");
  }
  // The table form: its regions after the pooled form's, every pointer
  // from the device table.
  const std::vector<rs::Launch>& launches = ptab ? d.table_launches : d.launches;
  char* const lbase = ptab ? base + d.image.size() : base;
  for (size_t li = 0; li < launches.size(); ++li) {
    const rs::Launch& L = launches[li];
    const void* regions = lbase + L.regions_off;
    const uint32_t* unit_region = L.units_off ? reinterpret_cast<const uint32_t*>(lbase + L.units_off) : nullptr;
    if (L.table) {
      const rs::TableArgs args{regions, unit_region, L.n_regions, L.n_units, static_cast<void* const*>(ptab)};
      he = rs::launch(L.bucket, L.n_units, args, static_cast<hipStream_t>(stream), dev);
    } else {
      rs::LaunchArgs args;
      std::memset(&args, 0, sizeof(args));
      args.regions = regions;
      args.unit_region = unit_region;
      args.n_regions = L.n_regions;
      args.n_units = L.n_units;
      for (size_t k = 0; k < L.pool.size(); ++k) {
        const uint32_t e = L.pool[k];
        args.ptr[k] = (e & rs::kDstBit) ? dst_ptrs[e & ~rs::kDstBit] : src_ptrs[e];
      }
      he = rs::launch(L.bucket, L.n_units, args, static_cast<hipStream_t>(stream), dev);
    }
    if (he != hipSuccess) {
      std::ostringstream m;
      m << "kernel launch " << li << " of " << launches.size() << ": " << hipGetErrorString(he)
        << (li ? " (the earlier launches stay enqueued)" : "") << "\n";
      return fail(RS_ERR_HIP, m.str());
    }
  }
  return RS_OK;
}

}  // namespace

extern "C" {

rs_status reshard_execute(const rs_plan* plan, void* const* src_ptrs, void* const* dst_ptrs,
                          void* stream) {
  g_error.clear();
  try {
    return execute(plan, src_ptrs, dst_ptrs, stream, Tables::kPlanOwned);
  } catch (const std::bad_alloc&) {
    return fail(RS_ERR_ALLOC, "host allocation failed\n");
  }
}

rs_status reshard_execute_no_alloc(const rs_plan* plan, void* const* src_ptrs, void* const* dst_ptrs,
                                   void* stream) {
  g_error.clear();
  try {
    return execute(plan, src_ptrs, dst_ptrs, stream, Tables::kStaticArea);
  } catch (const std::bad_alloc&) {
    return fail(RS_ERR_ALLOC, "host allocation failed\n");
  }
}

rs_status reshard_plan_info(const rs_plan* plan, rs_plan_info* info) {
  g_error.clear();
  if (!plan || !info) return fail(RS_ERR_INVALID, "plan or info is NULL\n");
  *info = plan->d.info;
  return RS_OK;
}

rs_status reshard_plan_region(const rs_plan* plan, uint64_t index, rs_region* out) {
  g_error.clear();
  if (!plan || !out) return fail(RS_ERR_INVALID, "plan or out is NULL\n");
  if (rs::region_info(plan->d, index, out) != RS_OK)
    return fail(RS_ERR_INVALID, "region index out of range\n");
  return RS_OK;
}

rs_status reshard_shard_box(const rs_tensor_desc* desc, int64_t slot, int64_t* offsets,
                            int64_t* lengths) {
  g_error.clear();
  try {
    std::string err;
    const rs_status st = rs::shard_box(desc, slot, offsets, lengths, err);
    if (st != RS_OK) return fail(st, err);
    return RS_OK;
  } catch (const std::bad_alloc&) {
    return fail(RS_ERR_ALLOC, "host allocation failed\n");
  }
}

void reshard_plan_destroy(rs_plan* plan) {
  if (!plan) return;
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (const auto& t : plan->tables) {
    if (hipSetDevice(t.device) == hipSuccess) (void)hipFree(t.ptr);
  }
  for (const auto& t : plan->ptr_tables) {
    if (hipSetDevice(t.device) == hipSuccess) (void)hipFree(t.ptr);
  }
  if (have_cur && !plan->tables.empty()) (void)hipSetDevice(cur);
  delete plan;
}

const char* reshard_last_error(void) { return g_error.c_str(); }

}  // extern "C"
