/*
 * reshard.h -- C ABI of the single-GPU DTensor-to-DTensor M->N relayout.
 *
 * What it computes.  The Reshard collective moves the logical values of a
 * tensor from one DTensor distribution to another; a distribution is a global
 * shape, a device mesh and one Shard/Replicate placement per mesh dimension
 * (news summary of NVIDIA's Reshard announcement, "Recasting refit as a
 * DTensor-to-DTensor transfer" and "The Reshard collective").  Every
 * destination shard is assembled from exactly the overlapping regions of the
 * source shards, and each destination region is moved once ("NCCL Reshard
 * Refit (Experimental)", "xferdtensor Transports", the Python transport).
 * The result equals the golden transport of that section: the full tensor,
 * sliced per destination.
 *
 * Here all M source shards and all N destination shards are separate buffers
 * in one GPU's memory, so the transfer is a device-local gather/scatter:
 *   reshard_plan     (CPU)  descriptors -> one flat, coalesced, bucketed
 *                           region table (plan once, execute many; cf. the
 *                           descriptor caching of the ModelExpress PR
 *                           "feat(refit): add ModelExpress Megatron-to-vLLM
 *                           reshard path - #3632", "Performance measured on
 *                           real model tensors");
 *   reshard_execute  (GPU)  one batched HIP launch per region bucket on the
 *                           caller's stream.
 *
 * Placement semantics.  Shard(d) cuts tensor dim d like torch.chunk (chunk
 * size ceil(len/parts); trailing shards may be short or empty, as PyTorch
 * DTensor does).  Several mesh dims sharding one tensor dim nest in mesh-dim
 * order, the lower mesh dim outermost.  Replicate mesh dims hold copies; each
 * destination replica receives the whole shard, and any one source replica
 * may be read (they must hold equal bytes).
 *
 * Threading: every function is thread-safe; a plan is immutable after
 * reshard_plan and may be executed concurrently on several streams as long as
 * those executions write disjoint destinations.
 */
#ifndef RESHARD_H
#define RESHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RS_MAX_DIMS 8      /* tensor rank limit */
#define RS_MAX_MESH 4      /* mesh rank limit */
#define RS_REPLICATE (-1)  /* placements[i] == RS_REPLICATE: Replicate; d >= 0: Shard(d) */
#define RS_MAX_FANOUT 16   /* destination replicas served by one read (plan detail) */

typedef enum rs_status {
  RS_OK = 0,
  RS_ERR_INVALID = 1,     /* malformed argument (bad rank, placement, view, null pointer ...) */
  RS_ERR_MISMATCH = 2,    /* source and destination describe different tensors */
  RS_ERR_UNSUPPORTED = 3, /* well-formed but outside what this library implements */
  RS_ERR_ALLOC = 4,       /* host or device allocation failed */
  RS_ERR_HIP = 5          /* a HIP runtime call failed */
} rs_status;

/* Element types.  The relayout is bitwise, so only the element size matters,
 * except that MXFP8 installation needs a bf16 source. */
typedef enum rs_dtype {
  RS_U8 = 1, RS_I8 = 2, RS_U16 = 3, RS_I16 = 4, RS_BF16 = 5, RS_F16 = 6,
  RS_U32 = 7, RS_I32 = 8, RS_F32 = 9, RS_U64 = 10, RS_I64 = 11, RS_F64 = 12
} rs_dtype;

/* Destination installation modes. */
typedef enum rs_quant {
  RS_Q_NONE = 0,
  /* BF16 source -> MXFP8 destination, quantised on install ("NCCL Reshard
   * Refit (Experimental)", "Enabling It": the generation side quantises each
   * received BF16 shard before installing it).  Rule (OCP Microscaling
   * Formats v1.0, MXFP8 E4M3): blocks of 32 consecutive elements along the
   * destination shard's last dim, from local column 0 (a short last block
   * uses its valid elements); shared exponent X = floor(log2(amax)) - 8,
   * clamped to [-127, 127], X = -127 for an all-zero block; scale byte
   * (E8M0) = X + 127; element byte = E4M3 of v * 2^-X, round to nearest
   * even, saturating to +-448; the sign of zero is kept; a block holding a
   * NaN or an infinity gets scale 0xFF and elements 0x7F.  Element buffers
   * hold one byte per element; scale buffers one byte per block. */
  RS_Q_MXFP8_E4M3 = 1
} rs_quant;

/* Where a shard lives inside the buffer the caller passes for its slot:
 * element (i_0, ..., i_{n-1}) of the shard's local box is at element offset
 * base + sum_d i_d * strides[d] from the buffer pointer (in elements of the
 * tensor's dtype; for MXFP8 element buffers in bytes).  Views let a
 * destination be a slice of a fused buffer (gate and up projections in one
 * w13 / gate_up_proj buffer, "NCCL Reshard Refit (Experimental)", "Execution
 * Flow: Setup Time": the slice-of-a-fused-tensor case), written in place
 * with no staging buffer.  base >= 0, strides >= 0. */
typedef struct rs_view {
  int64_t base;
  int64_t strides[RS_MAX_DIMS];
} rs_view;

/* One side (source or destination) of one tensor.  The fields mirror the
 * per-parameter record of "NCCL Reshard Refit (Experimental)", "Execution
 * Flow: Setup Time" (global_shape, dtype, mesh info and placements). */
typedef struct rs_tensor_desc {
  int32_t ndim;                          /* 1..RS_MAX_DIMS */
  int32_t dtype;                         /* rs_dtype; destination of an MXFP8 install: RS_U8 */
  int64_t global_shape[RS_MAX_DIMS];     /* >= 0 */
  int32_t mesh_ndim;                     /* 1..RS_MAX_MESH */
  int32_t placements[RS_MAX_MESH];       /* RS_REPLICATE or a tensor dim */
  int64_t mesh_shape[RS_MAX_MESH];       /* >= 1 each; slots = product (<= 65536) */
  /* Optional rank grid: prod(mesh_shape) entries, row-major mesh coordinate
   * -> buffer slot (a permutation).  NULL = identity.  Borrowed during
   * reshard_plan only. */
  const int32_t* slot_of_coord;
  /* Optional per-slot views (prod(mesh_shape) entries).  NULL = every slot is
   * a dense row-major array of its local box at offset 0.  Borrowed during
   * reshard_plan only. */
  const rs_view* views;
  int32_t quant;                         /* rs_quant; destination only */
  /* MXFP8 destinations: per-slot views of the scale buffers, over the local
   * shape with the last extent replaced by ceil(last / 32).  NULL = dense. */
  const rs_view* scale_views;
  /* 0: each slot is one buffer.  1: each slot's shard is held as separate
   * buffers, one per local index along tensor dim 0 (for example one buffer
   * per expert of a grouped [E, ...] weight, as a training side holds them
   * before stacking; "NCCL Reshard Refit (Experimental)", "Execution Flow:
   * Setup Time", the grouped-expert pre hook).  The slot then takes one
   * pointer per local dim-0 index, in order, in the pointer array, and its
   * view describes each part (strides[0] is ignored; base applies to every
   * part).  An MXFP8 destination splits its scale buffers the same way. */
  int32_t split_dim0;
  /* Blockwise-scaled weights (read from the source description; the
   * destination's must be 0 or equal).  0: an ordinary tensor.  w + 1: this
   * tensor holds the scales of tensor w of the same plan, one per block of
   * scale_block[d] weight elements along each dim d (1 = unblocked), so its
   * global shape is ceil(weight shape / block) and it uses the weight's
   * meshes and placements.  Blockwise-FP8 weights move as bytes next to
   * their scale siblings ("NCCL Reshard Refit (Experimental)", "Enabling It"
   * and "Design Overview": FP8 weights with their _scale_inv tensors); the
   * planner checks that every shard boundary of both sides falls on a block
   * boundary, so each destination receives exactly the scales of its weight
   * blocks, and reports RS_ERR_UNSUPPORTED naming the slot otherwise. */
  int32_t scale_of;
  int32_t scale_block[RS_MAX_DIMS];
} rs_tensor_desc;

/* Planning options.  Pass NULL for the defaults. */
typedef struct rs_plan_opts {
  uint32_t struct_size;   /* sizeof(rs_plan_opts) */
  uint32_t fanout;        /* 1 (default): destination replicas with equal views share one read */
  uint64_t unit_bytes;    /* bulk work-unit size, power of two in [4096, 2^24]; default 16384.
                             A unit holds whole rows (rows longer than a unit are cut into
                             unit-sized parts); its row count is trimmed to make the unit a whole
                             number of KiB wherever that keeps at least half of it */
  uint32_t tiny_bytes;    /* regions of at most this many bytes are batched 64 per wave (0: none);
                             default 256 (larger regions copy faster one workgroup each);
                             at most 65536, else RS_ERR_INVALID */
  uint32_t thin_bytes;    /* contiguous runs shorter than this are staged through LDS; default 128
                             (0: default); at most 16384 (the LDS tile a thin work unit fills),
                             else RS_ERR_INVALID */
  uint32_t reserved[4];   /* must be zero */
} rs_plan_opts;

typedef struct rs_plan rs_plan;

/* Summary of a plan.  Byte counts are algorithmic: bytes_read counts every
 * source byte the plan reads once (fan-out reads once for all replicas);
 * bytes_written counts every destination byte (and scale byte) written. */
typedef struct rs_plan_info {
  uint64_t n_tensors;
  uint64_t n_src_ptrs;           /* entries reshard_execute expects in src_ptrs */
  uint64_t n_dst_ptrs;           /* entries reshard_execute expects in dst_ptrs */
  uint64_t n_regions;            /* regions after coalescing and splitting */
  uint64_t n_regions_bucket[4];  /* bulk, thin (LDS), tiny, mxfp8 */
  uint64_t n_units_bucket[4];    /* work units (grid size) per bucket */
  uint64_t n_launches;           /* kernel launches per reshard_execute (see n_launches_pooled) */
  uint64_t bytes_read;
  uint64_t bytes_written;
  uint64_t bytes_read_no_fanout; /* source bytes if every replica read its own copy */
  uint64_t plan_ns;              /* wall time reshard_plan spent building this plan (CPU) */
  uint64_t n_launches_pooled;    /* kernel launches when the pointers travel in the kernel
                                    arguments: reshard_execute_no_alloc, and reshard_execute
                                    without a device pointer table (equal to n_launches
                                    unless the plan has more pointers than one launch's
                                    arguments hold; see reshard_execute) */
} rs_plan_info;

/* One region of a plan, for inspection (tests, tools).  A region copies
 * rows x inner (bytes; for MXFP8 regions: bf16 elements read, bytes
 * written) from src_ptrs[src_index] + src_off to every
 * dst_ptrs[dst_index[j]] + dst_off, j < n_dst.  Row r (0 <= r <
 * ext[0]*ext[1]*ext[2]) is decomposed as r = i0 + ext[0]*(i1 + ext[1]*i2)
 * and starts at + sum_k ik * stride[k] (bytes) on each side. */
typedef struct rs_region {
  uint32_t tensor;
  uint32_t bucket;               /* 0 bulk, 1 thin (LDS), 2 tiny, 3 mxfp8 */
  uint32_t src_index;
  uint32_t n_dst;
  uint32_t dst_index[RS_MAX_FANOUT];
  uint32_t scale_index[RS_MAX_FANOUT]; /* MXFP8 only: indices into dst_ptrs */
  uint64_t src_off, dst_off, scale_off;
  uint64_t inner;
  uint64_t ext[3];
  uint64_t src_stride[3], dst_stride[3], scale_stride[3];
  uint64_t scale_inner_stride;   /* MXFP8 only: bytes between consecutive block scales */
  /* Second source piece (MXFP8 only).  A 32-element block whose values two
   * source shards hold (their boundary falls inside the block) is installed
   * by a region one block wide: columns [0, split) of each row come from
   * src_index as above, columns [split, inner) from src2_index at src2_off
   * + sum_k ik * src2_stride[k], column split first.  split == inner for
   * every one-source region. */
  uint64_t split;
  uint32_t src2_index;
  uint32_t reserved0;
  uint64_t src2_off;
  uint64_t src2_stride[3];
} rs_region;

/* Plan n_tensors tensor pairs (for example gate, up and down of one layer)
 * into ONE region table.  Pure CPU work; nothing touches a GPU.  src[t] and
 * dst[t] describe the two sides of tensor t and must agree on ndim and
 * global_shape; dtypes must be equal, or src bf16 and dst RS_U8 with
 * quant = RS_Q_MXFP8_E4M3.  On success *out receives the plan.  On failure
 * *out = NULL and reshard_last_error() lists every violation found, not only
 * the first (cf. the single error listing every violation of
 * "NCCL Reshard Refit (Experimental)", "Enabling It").
 * Errors: RS_ERR_INVALID, RS_ERR_MISMATCH, RS_ERR_UNSUPPORTED (for example an
 * MXFP8 block whose 32 values come from more than two source shards, i.e.
 * source shards narrower than a block along the last dim, or a
 * non-contiguous last dim on an MXFP8 tensor), RS_ERR_ALLOC. */
rs_status reshard_plan(const rs_tensor_desc* src, const rs_tensor_desc* dst, int32_t n_tensors,
                       const rs_plan_opts* opts, rs_plan** out);

/* Run a plan on `stream` (a hipStream_t; NULL = the default stream).
 * src_ptrs: device pointers of the source buffers, tensor by tensor, slot by
 *   slot (tensor 0 slots 0..M0-1, then tensor 1, ...); a split_dim0 side has
 *   one pointer per local dim-0 index of each slot instead (slot by slot).
 * dst_ptrs: device pointers of the destination buffers, tensor by tensor:
 *   the element buffers in slot order (per part for split_dim0), and for
 *   MXFP8 tensors as many scale buffers right after them.  Fused
 *   destinations pass the same pointer for several tensors (their views
 *   differ).  rs_plan_info gives the expected counts.
 * Both arrays are host arrays, read before the call returns; the buffers
 * are owned by the caller and must stay alive until the work on `stream`
 * completes.  Sources and destinations must not overlap.
 * Asynchronous: returns once the launches are enqueued.  Every argument is
 * checked before anything is launched (a NULL pointer for a non-empty slot
 * fails the whole call with RS_ERR_INVALID and nothing written).  With the
 * environment variable RESHARD_DEBUG_CHECKS=1 it also checks that sources
 * and destinations do not overlap and that every pointer is device memory of
 * the stream's device with room for every byte its regions reach (a few
 * microseconds per pointer).  The first
 * call on a device uploads the plan's tables there (a blocking allocation
 * and copy); later calls allocate nothing and only enqueue kernels, so they
 * may be captured into a HIP graph.
 * Pointer tables: one launch's kernel arguments hold 500 pointers.  So that
 * a batch of many small tensors still moves in one launch per kernel (the
 * one coalesced call of "NeMo-RL: Optimizing Non-Colocated Refit for
 * Asynchronous RL", "Optimization #2"), a plan
 * with more (rs_plan_info.n_launches < n_launches_pooled) keeps on each
 * device a table of the pointers of every call with a pointer set it has
 * not seen, up to 8 sets per device, each uploaded by that call (a blocking
 * allocation and copy; never while `stream` is capturing a graph) and freed
 * with the plan; a call whose pointers have a table runs n_launches
 * launches that read them from it, any other call the n_launches_pooled
 * launches that carry them in their arguments.  The results are the same.
 * Errors: RS_ERR_INVALID, RS_ERR_ALLOC, RS_ERR_HIP (launch or upload
 * failure).  Faults during execution surface on the stream like any HIP
 * error. */
rs_status reshard_execute(const rs_plan* plan, void* const* src_ptrs, void* const* dst_ptrs,
                          void* stream);
/* Partial failure: a plan runs as one launch per kernel kind it uses, and
 * the pooled form of a plan with more pointers than one launch's arguments
 * hold as more (rs_plan_info.n_launches, n_launches_pooled).  All argument
 * checks come before the first launch; if the HIP runtime then refuses launch k,
 * launches 0..k-1 stay enqueued and write their regions, the call returns
 * RS_ERR_HIP naming launch k, and the destinations are only partly
 * installed (execute again once the cause is fixed). */

/* reshard_execute for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, launches and results as
 * reshard_execute (in n_launches_pooled launches: no pointer tables), but
 * the plan's region tables are not uploaded into an
 * allocation of the plan: every call copies them (hipMemcpyAsync on
 * `stream`, from the plan's host image) into a static device array of the
 * library, RESHARD_TABLE_AREA_BYTES long, which each GPU holds from the
 * library's load until the process ends.  The call allocates no device
 * memory (no hipMalloc, no hipFree).
 * Sharing: every call on a GPU uses that GPU's one area, which keeps the
 * last call's tables.  Calls on one stream are ordered and safe; calls that
 * overlap on one GPU (other streams, other threads, other plans) race for
 * the area and may read each other's tables -- serialise them.
 * Errors: those of reshard_execute, and RS_ERR_UNSUPPORTED, before anything
 * is copied or launched, for a plan whose tables exceed the area
 * (rs_plan_info gives n_regions; a region takes 128 bytes, an MXFP8 region
 * 240, plus 4 bytes per 256 work units). */
#define RESHARD_TABLE_AREA_BYTES (4u << 20)
rs_status reshard_execute_no_alloc(const rs_plan* plan, void* const* src_ptrs,
                                   void* const* dst_ptrs, void* stream);

/* Fill *info: the plan's pointer counts, region and work-unit counts per
 * kernel, launches per execute, algorithmic bytes and planning time.  The
 * per-receiver descriptor count and the bytes a refit moves are the figures
 * the ModelExpress PR reports for its plans ("feat(refit): add ModelExpress
 * Megatron-to-vLLM reshard path - #3632", "Performance measured on real model
 * tensors": descriptors per receiver, wire bytes against engine bytes).
 * Errors: RS_ERR_INVALID for NULL arguments. */
rs_status reshard_plan_info(const rs_plan* plan, rs_plan_info* info);

/* Copy region `index` (0 <= index < n_regions) into *out.
 * Errors: RS_ERR_INVALID for NULL arguments or an index out of range. */
rs_status reshard_plan_region(const rs_plan* plan, uint64_t index, rs_region* out);

/* Global box of one slot of a layout: offsets[d] and lengths[d] for
 * d < desc->ndim (torch.chunk rule above).  Lets a caller size its buffers.
 * Errors: RS_ERR_INVALID for a malformed description or slot out of range. */
rs_status reshard_shard_box(const rs_tensor_desc* desc, int64_t slot, int64_t* offsets,
                            int64_t* lengths);

/* Free a plan and its device tables.  A plan is built once and reused for
 * every refit of the same layouts: the descriptor caching that the
 * ModelExpress PR lists among its transport changes ("feat(refit): add
 * ModelExpress Megatron-to-vLLM reshard path - #3632", "Performance measured
 * on real model tensors"); destroy ends that reuse.  Every stream that
 * executed the plan must have been synchronised.  NULL is ignored. */
void reshard_plan_destroy(rs_plan* plan);

/* Message of the last failing call on this thread ("" if none): one line
 * per violation found, all of them, as the validation of "NCCL Reshard Refit
 * (Experimental)", "Enabling It" reports every problem of a configuration in
 * one error rather than the first only.  The string stays valid until the
 * next call on this thread. */
const char* reshard_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RESHARD_H */
