// CPU planner of the M->N relayout: descriptors -> flat region tables.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "reshard.h"
#include "rs_device.hpp"

namespace rs {

constexpr uint32_t kDstBit = 0x80000000u;  // pool entry refers to dst_ptrs (else src_ptrs)

// One kernel launch of a plan: a contiguous slice of the device image.
struct Launch {
  uint32_t bucket = 0;
  uint32_t n_regions = 0;
  uint32_t n_units = 0;        // workgroups to launch
  uint64_t regions_off = 0;    // byte offset of the region array in the image
  uint64_t units_off = 0;      // byte offset of the unit -> region table (0 if none)
  std::vector<uint32_t> pool;  // pool slot -> caller pointer index (| kDstBit for dst_ptrs)
  bool table = false;          // table form: pool index = caller pointer index, sources
                               // first (the pointers come from a device table)
};

struct PlanData {
  std::vector<uint32_t> region_tensor;  // tensor of each region, in image order
  std::vector<uint8_t> image;      // device tables, uploaded once per device
  std::vector<Launch> launches;
  // Table form of the launches (empty unless the pointer pool cut a pass of
  // the pooled form into several launches): regions in the same order, in
  // an image of their own, uploaded after `image`.
  std::vector<uint8_t> table_image;
  std::vector<Launch> table_launches;
  std::vector<uint8_t> src_used;   // pointer index -> referenced by some region
  std::vector<uint8_t> dst_used;
  std::vector<uint8_t> src_align;  // required pointer alignment (bytes)
  std::vector<uint64_t> src_span;  // bytes touched past each pointer (for overlap checks)
  std::vector<uint64_t> dst_span;
  rs_plan_info info{};
};

// Builds a plan.  On failure returns the most severe status and appends one
// line per violation to `err`.
rs_status build_plan(const rs_tensor_desc* src, const rs_tensor_desc* dst, int32_t n,
                     const rs_plan_opts* opts, PlanData& out, std::string& err);

// Public view of region `index` (image order), rebuilt from the device image.
rs_status region_info(const PlanData& d, uint64_t index, rs_region* out);

// Global box of one slot of a layout.
rs_status shard_box(const rs_tensor_desc* d, int64_t slot, int64_t* off, int64_t* len,
                    std::string& err);

}  // namespace rs
