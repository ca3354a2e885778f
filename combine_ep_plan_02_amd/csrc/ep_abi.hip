// ep_abi.hip -- host side of libep_mi355x.so: argument checks, workspace
// layout, launch configuration.  The C ABI is declared in include/ep_mi355x.h.
//
// Checks run on the host before anything is enqueued and mirror the
// validation contract of ROCm/aiter PR #6960 (contiguous 16-byte aligned
// rows, row length a multiple of the vector width, no output aliasing an
// input, early return on empty input) and the status classes of the CANN
// "aclnnMoeDistributeDispatchV2" return codes.
#include "ep_mi355x.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <type_traits>
#include <string>
#include <unordered_map>

#include "ep_common.h"
#include "ep_plan_kernels.h"
#include "ep_row_kernels.h"

#define EP_EXPORT extern "C" __attribute__((visibility("default")))

// Cache policy of each row stream (true: non-temporal), chosen by measurement
// on MI355X in the plan -> dispatch -> combine sequence: streaming stores for
// every row written (expandX, the combined rows, the all-to-all receive
// buffer), so no dirty lines are left in the 256 MB Infinity Cache for the
// next kernel to write back; streaming loads for the combine's gathered rows
// (~7.1 TB/s for streaming reads against ~6.4 TB/s for default reads);
// default loads for x and the all-to-all input, which measured faster next
// to streaming stores.
constexpr bool kDispatchNtLoad = false, kDispatchNtStore = true;
constexpr bool kCombineNtLoad = true, kCombineNtStore = true;
constexpr bool kQuantNtLoad = false, kQuantNtStore = true;
constexpr bool kCopyNtLoad = false, kCopyNtStore = true;
// Vectors per lane of one (token, column chunk) work item.
constexpr int kDispatchUnroll = 2;
constexpr int kCombineUnroll = 1;
// Waves (work items) per workgroup of the combine gathers.  bf16 rows: 2
// measured ~3% faster than 4 or 8 at T=8192, H=7168, K=8 (1 and 16 in
// between).  Code rows: 4 (2 was no faster at H=7168 and 3% slower at
// T=4096, H=4096).
constexpr int kCombineWaves = 2;
constexpr int kCombineQuantWaves = 4;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return EP_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range_ {
  const void* p;
  size_t n;
};

// [a, a+na) and [b, b+nb) share a byte.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Rows of a [cap_rows][...] buffer that a kernel can reach: positions are
// int32, so rows at or past 2^31 are never read or written.  Byte ranges for
// the overlap checks are taken over these rows, which keeps them from
// overflowing for any cap_rows.
size_t reachable_rows(int64_t cap_rows) {
  const int64_t lim = (int64_t)1 << 31;
  return (size_t)(cap_rows < lim ? cap_rows : lim);
}

// W * R * stride_bytes (the bytes of the all-to-all's in and out buffers)
// fits in int64.
bool splits_bytes_fit(int32_t W, int64_t R, int64_t stride_bytes) {
  return R == 0 || R <= INT64_MAX / W / stride_bytes;
}

// Tokens one launch of a row kernel covers.  A launch holds at most
// 2^32 - 1 work-items per grid dimension; the row kernels' grids grow with
// the token count, so the host launches them over slices of at most 2^31
// work-items, offsetting the per-token pointers (x, pos, weights, out, ...)
// by the slice's first token.  Rows addressed through pos are global and
// need no offset.  Every workload of practical size is one slice.
int64_t slice_tokens(int64_t work_items_per_token) {
  const int64_t n = ((int64_t)1 << 31) / work_items_per_token;
  return n > 0 ? n : 1;
}

int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(EP_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

int check_dims(int32_t T, int32_t K, int32_t E, int32_t W) {
  if (T < 0) return fail(EP_ERR_INVALID, "T must be >= 0 (got %d)", T);
  if (K < 1 || K > EP_MAX_K) return fail(EP_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)", EP_MAX_K, K);
  if (E < 1 || E > EP_MAX_E) return fail(EP_ERR_UNSUPPORTED, "E must be in [1, %d] (got %d)", EP_MAX_E, E);
  if (W < 1) return fail(EP_ERR_UNSUPPORTED, "W must be >= 1 (got %d)", W);
  if (E % W) return fail(EP_ERR_UNSUPPORTED, "E (%d) must be a multiple of W (%d)", E, W);
  if (T % W) return fail(EP_ERR_UNSUPPORTED, "T (%d) must be a multiple of W (%d)", T, W);
  if ((int64_t)T * K >= (int64_t)1 << 31) return fail(EP_ERR_UNSUPPORTED, "T*K must be < 2^31");
  return EP_OK;
}

int check_rows(int32_t H, int32_t dtype) {
  if (dtype != EP_BF16 && dtype != EP_FP8_E4M3FN && dtype != EP_INT8)
    return fail(EP_ERR_INVALID, "unknown row dtype %d", dtype);
  if (H < 1 || H > EP_MAX_H) return fail(EP_ERR_UNSUPPORTED, "H must be in [1, %d] (got %d)", EP_MAX_H, H);
  const int vec = dtype == EP_BF16 ? 8 : 16;
  if (H % vec) return fail(EP_ERR_UNSUPPORTED, "H (%d) must be a multiple of %d for this row dtype", H, vec);
  return EP_OK;
}

struct PlanGeometry {
  int Tw, tile_tokens, tiles_per_rank, ntiles;
};

PlanGeometry plan_geometry(int32_t T, int32_t K, int32_t W) {
  PlanGeometry g{};
  g.Tw = T / W;
  if (g.Tw == 0) return g;
  g.tile_tokens = ep::plan_tile_tokens(K, g.Tw);
  g.tiles_per_rank = (g.Tw + g.tile_tokens - 1) / g.tile_tokens;
  g.ntiles = g.tiles_per_rank * W;
  return g;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace: [header (256 B): ticket, epoch, done] [flags: ntiles u32] [aggregates: ntiles x E i32]
//            [inclusive: ntiles x E i32] [descriptors: ntiles x E u64], each
// region 256-byte aligned.  The look-back path uses ticket, flags,
// aggregates and inclusive; the fused path only the descriptors.
struct WorkspaceLayout {
  size_t flags, aggregates, inclusive, descriptors, total;
};

WorkspaceLayout workspace_layout(int ntiles, int E) {
  WorkspaceLayout l{};
  l.flags = 256;
  l.aggregates = l.flags + round256((size_t)ntiles * 4);
  l.inclusive = l.aggregates + round256((size_t)ntiles * E * 4);
  l.descriptors = l.inclusive + round256((size_t)ntiles * E * 4);
  l.total = l.descriptors + round256((size_t)ntiles * E * 8);
  return l;
}

size_t fused_lds_bytes(int E) { return (size_t)(ep::kPlanWaves + 6) * E * sizeof(int32_t); }

// Tiles of the fused plan kernel that fit on the current device at once
// (workgroups per CU by occupancy times the CU count).  The fused kernel's
// tiles wait for each other, so it is only used when its whole grid fits; its
// waits are bounded, so a grid that cannot become resident (the device held
// by other work for longer than the bound) ends with EP_DEVERR_PLAN_STALL
// instead of hanging.
int fused_capacity(int E) {
  static std::mutex mu;
  static std::unordered_map<long long, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const long long key = ((long long)dev << 32) | (unsigned)E;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  int cap = 0;
  const size_t lds = fused_lds_bytes(E);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ep::plan_fused_kernel, ep::kPlanThreads, lds) ==
          hipSuccess)
    cap = per_cu * cus;
  (void)hipGetLastError();
  cache[key] = cap;
  return cap;
}

int id_bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// Clears the given bits of the device error word, keeping any other bit a
// kernel on another stream raised since they were read.
__global__ void clear_error_bits_kernel(unsigned int bits) {
  __hip_atomic_fetch_and(&ep::g_device_error, ~bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

EP_EXPORT int ep_supported(int32_t T, int32_t K, int32_t E, int32_t W, int32_t H, int32_t out_dtype) {
  const std::string saved = g_last_error;
  const bool yes = check_dims(T, K, E, W) == EP_OK && check_rows(H, out_dtype) == EP_OK;
  g_last_error = saved;
  return yes ? 1 : 0;
}

EP_EXPORT size_t ep_workspace_size(int32_t T, int32_t K, int32_t E, int32_t W) {
  const std::string saved = g_last_error;
  const bool good = check_dims(T, K, E, W) == EP_OK;
  g_last_error = saved;
  if (!good) return 0;
  return workspace_layout(plan_geometry(T, K, W).ntiles, E).total;
}

EP_EXPORT int ep_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace) return fail(EP_ERR_NULLPTR, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(EP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes % 4) return fail(EP_ERR_WORKSPACE, "workspace size must be a multiple of 4");
  const size_t n = ws_bytes / 4;
  if (n == 0) return ok();
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)workspace, n);
  return launch_status("ep_workspace_init");
}

EP_EXPORT int64_t ep_expand_rows_bound(int32_t T, int32_t K, int32_t E, int32_t major_align,
                                       int32_t pad_empty_experts) {
  if (T < 0 || K < 1 || E < 1 || major_align > EP_MAX_ALIGN) return -1;
  const int64_t a = major_align < 1 ? 1 : major_align;
  return (int64_t)T * K + (int64_t)E * (pad_empty_experts ? a : a - 1);
}

namespace {

// Where the plan kernels keep their state: the ticket, epoch and done
// counter (header), the look-back flags, aggregates and inclusive prefixes,
// and the one-launch path's count descriptors.
struct PlanState {
  uint32_t* header;
  uint32_t* flags;
  int32_t* aggregates;
  int32_t* inclusive;
  uint64_t* desc;
};

// Tiles and descriptors the one-launch plan may use.  The kernel is taken
// only when its whole grid fits on the device at once with room to spare:
// half of what fits (workgroups per CU by occupancy times the CU count), so
// that a second plan, or another kernel, on another stream still leaves it
// resident.  Its waits are bounded (a tile gives up after one spin budget),
// so a grid kept from becoming resident ends with EP_DEVERR_PLAN_STALL
// instead of hanging.
bool fused_fits(int ntiles, int E) {
  return ntiles > 0 && (int64_t)ntiles * E <= ep::kFusedMaxDescriptorsPerTile &&
         2 * ntiles <= fused_capacity(E);
}

int check_plan_args(int32_t T, int32_t K, int32_t E, int32_t W, const int32_t* topk_ids,
                    const uint8_t* active, const ep_plan_opts_t* opts, const ep_plan_t* plan,
                    ep_plan_opts_t& o) {
  int rc = check_dims(T, K, E, W);
  if (rc) return rc;
  o = ep_plan_opts_t{};
  if (opts) o = *opts;
  if (o.major_align < 1) o.major_align = 1;
  if (o.major_align > EP_MAX_ALIGN)
    return fail(EP_ERR_UNSUPPORTED, "major_align must be <= %d (got %d)", EP_MAX_ALIGN, o.major_align);
  if (o.expert_token_nums_type != 0 && o.expert_token_nums_type != 1)
    return fail(EP_ERR_INVALID, "expert_token_nums_type must be 0 or 1 (got %d)", o.expert_token_nums_type);
  if ((uint32_t)o.flags & ~(uint32_t)(EP_PLAN_LOOKBACK | EP_PLAN_TEST_STALL))
    return fail(EP_ERR_INVALID, "unknown plan flags 0x%x", (unsigned)o.flags);
  if (ep_expand_rows_bound(T, K, E, o.major_align, o.pad_empty_experts) >= (int64_t)1 << 31)
    return fail(EP_ERR_UNSUPPORTED, "T*K plus the expert padding must be < 2^31");
  if (!plan) return fail(EP_ERR_NULLPTR, "plan is NULL");
  if (!plan->in_splits || !plan->src_offsets || !plan->out_splits || !plan->dst_offsets ||
      !plan->expert_counts || !plan->expert_offsets || !plan->rank_offsets)
    return fail(EP_ERR_NULLPTR, "a required plan output is NULL");
  const int64_t ncopies = (int64_t)T * K;
  if (ncopies > 0 && (!topk_ids || !plan->pos)) return fail(EP_ERR_NULLPTR, "topk_ids or pos is NULL");
  const int64_t* outs64[] = {plan->in_splits, plan->src_offsets, plan->out_splits, plan->dst_offsets,
                             plan->expert_counts, plan->expert_offsets, plan->rank_offsets};
  for (int i = 0; i < 7; ++i)
    if (!aligned(outs64[i], 8)) return fail(EP_ERR_INVALID, "plan int64 outputs must be 8-byte aligned");
  if (!aligned(topk_ids, 4) || !aligned(plan->pos, 4) || !aligned(plan->occ, 4))
    return fail(EP_ERR_INVALID, "topk_ids, pos and occ must be 4-byte aligned");
  if (!aligned(o.expert_token_nums, 8))
    return fail(EP_ERR_INVALID, "expert_token_nums must be 8-byte aligned");
  return EP_OK;
}

// No output may overlap an input or another output (the workspace, when the
// caller brings one, counts as both).
int check_plan_overlaps(int32_t T, int32_t K, int32_t E, int32_t W, const int32_t* topk_ids,
                        const uint8_t* active, const ep_plan_opts_t& o, const ep_plan_t* plan,
                        const void* workspace, size_t ws_bytes) {
  const int64_t ncopies = (int64_t)T * K;
  const size_t we = (size_t)W * E * 8;
  struct Range { const void* p; size_t n; const char* name; };
  const Range ranges[] = {
      {topk_ids, (size_t)ncopies * 4, "topk_ids"}, {active, active ? (size_t)T : 0, "active"},
      {o.active_copies, o.active_copies ? (size_t)ncopies : 0, "active_copies"},
      {workspace, workspace ? ws_bytes : 0, "workspace"}, {plan->pos, (size_t)ncopies * 4, "pos"},
      {o.expert_token_nums, o.expert_token_nums ? (size_t)E * 8 : 0, "expert_token_nums"},
      {plan->occ, plan->occ ? (size_t)ncopies * 4 : 0, "occ"},
      {plan->in_splits, we, "in_splits"}, {plan->src_offsets, we, "src_offsets"},
      {plan->out_splits, we, "out_splits"}, {plan->dst_offsets, we, "dst_offsets"},
      {plan->expert_counts, (size_t)E * 8, "expert_counts"},
      {plan->expert_offsets, (size_t)E * 8, "expert_offsets"},
      {plan->rank_offsets, (size_t)(W + 1) * 8, "rank_offsets"}};
  const int nr = sizeof ranges / sizeof ranges[0];
  for (int i = 0; i < nr; ++i)
    for (int j = (i < 3 ? 3 : i + 1); j < nr; ++j)
      if (overlap(ranges[i].p, ranges[i].n, ranges[j].p, ranges[j].n))
        return fail(EP_ERR_INVALID, "%s overlaps %s", ranges[i].name, ranges[j].name);
  return EP_OK;
}

int launch_plan(int32_t T, int32_t K, int32_t E, int32_t W, const int32_t* topk_ids, const uint8_t* active,
                const ep_plan_opts_t& o, const ep_plan_t* plan, const PlanState& st, bool fused,
                hipStream_t s) {
  const PlanGeometry g = plan_geometry(T, K, W);
  const int64_t ncopies = (int64_t)T * K;
  if (fused) {
    // Single pass: every tile resident at once, counts exchanged through
    // self-validating descriptors.  The test hook withholds the last tile's
    // counts and shortens the spin budget, so every tile gives up quickly.
    const bool test_stall = (o.flags & EP_PLAN_TEST_STALL) != 0;
    const size_t lds = fused_lds_bytes(E);
    hipLaunchKernelGGL(ep::plan_fused_kernel, dim3(g.ntiles), dim3(ep::kPlanThreads), lds, s, topk_ids, active,
                       o.active_copies, K, E, W, g.Tw, g.tile_tokens, g.tiles_per_rank, g.ntiles, id_bits_for(E),
                       o.major_align, o.pad_empty_experts ? 1 : 0, o.expert_token_nums_type,
                       o.expert_token_nums, st.header, st.desc, plan->pos, plan->occ, plan->in_splits,
                       plan->src_offsets, plan->out_splits, plan->dst_offsets, plan->expert_counts,
                       plan->expert_offsets, plan->rank_offsets, test_stall ? ep::kTestSpinLimit : ep::kSpinLimit,
                       test_stall ? g.ntiles - 1 : -1);
    return launch_status("ep_plan (fused kernel)");
  }
  uint32_t* ticket = st.header + ep::kHeaderTicket;
  if (g.ntiles > 0) {
    const size_t lds = (size_t)(ep::kPlanWaves + 2) * E * sizeof(int32_t);
    hipLaunchKernelGGL(ep::plan_tile_kernel, dim3(g.ntiles), dim3(ep::kPlanThreads), lds, s, topk_ids,
                       active, o.active_copies, K, E, g.Tw, g.tile_tokens, g.tiles_per_rank, g.ntiles, id_bits_for(E),
                       plan->pos, ticket, st.flags, st.aggregates, st.inclusive);
    const int rc = launch_status("ep_plan (tile kernel)");
    if (rc) return rc;
  }
  const int64_t per_block = (int64_t)ep::kFinalizeThreads * ep::kFinalizeCopiesPerThread;
  int64_t blocks = (ncopies + per_block - 1) / per_block;
  if (blocks < W) blocks = W;
  hipLaunchKernelGGL(ep::plan_finalize_kernel, dim3((unsigned)blocks), dim3(ep::kFinalizeThreads), 0, s,
                     topk_ids, ncopies, K, E, W, g.Tw > 0 ? g.Tw : 1, g.tiles_per_rank, g.ntiles,
                     o.major_align, o.pad_empty_experts ? 1 : 0, o.expert_token_nums_type,
                     o.expert_token_nums, st.aggregates, st.inclusive, st.flags, ticket, plan->pos, plan->occ,
                     plan->in_splits, plan->src_offsets, plan->out_splits, plan->dst_offsets,
                     plan->expert_counts, plan->expert_offsets, plan->rank_offsets);
  return launch_status("ep_plan (finalize kernel)");
}

}  // namespace

EP_EXPORT int ep_plan(int32_t T, int32_t K, int32_t E, int32_t W, const int32_t* topk_ids,
                      const uint8_t* active, const ep_plan_opts_t* opts, const ep_plan_t* plan,
                      void* workspace, size_t ws_bytes, void* stream) {
  ep_plan_opts_t o;
  int rc = check_plan_args(T, K, E, W, topk_ids, active, opts, plan, o);
  if (rc) return rc;
  if (!workspace) return fail(EP_ERR_NULLPTR, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(EP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const PlanGeometry g = plan_geometry(T, K, W);
  const WorkspaceLayout l = workspace_layout(g.ntiles, E);
  if (ws_bytes < l.total)
    return fail(EP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, l.total);
  rc = check_plan_overlaps(T, K, E, W, topk_ids, active, o, plan, workspace, l.total);
  if (rc) return rc;
  uint8_t* ws = (uint8_t*)workspace;
  const PlanState st{(uint32_t*)ws, (uint32_t*)(ws + l.flags), (int32_t*)(ws + l.aggregates),
                     (int32_t*)(ws + l.inclusive), (uint64_t*)(ws + l.descriptors)};
  const bool fused = !(o.flags & EP_PLAN_LOOKBACK) && fused_fits(g.ntiles, E);
  return launch_plan(T, K, E, W, topk_ids, active, o, plan, st, fused, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// The plan without a caller workspace (ep_plan_noalloc): its state lives in
// `scratch`, one static array per device, laid out at fixed offsets that do
// not depend on the dimensions, so calls of any size may follow each other:
//   [0, 256)            header: ticket, epoch, done counter
//   [256, +16 KiB)      look-back flags, up to kScratchTiles tiles
//   then 512 KiB        one-launch descriptors (its limit of 65536)
//   then 1.5 MiB each   look-back aggregates and inclusive prefixes
// The array starts as zeros (static storage), which is the initial state;
// every plan returns the flags, ticket and done counter to zero, and the
// descriptors carry the epoch of the call that wrote them (the epoch only
// grows), so no call needs the array cleared.  Calls that overlap on one
// device share the array and race, as two plans on one workspace do.
// ---------------------------------------------------------------------------
constexpr size_t kScratchHeader = 256;
constexpr int kScratchTiles = 4096;
constexpr size_t kScratchFlags = kScratchHeader;
constexpr size_t kScratchDesc = kScratchFlags + (size_t)kScratchTiles * 4;
constexpr size_t kScratchAgg = kScratchDesc + (size_t)ep::kFusedMaxDescriptorsPerTile * 8;
constexpr size_t kScratchPartBytes = (size_t)3 << 19;  // 1.5 MiB
constexpr size_t kScratchIncl = kScratchAgg + kScratchPartBytes;
constexpr size_t kScratchBytes = kScratchIncl + kScratchPartBytes;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU holds its own copy); only this
// address is ever handed to a kernel.
int scratch_address(uint8_t** out) {
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EP_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(EP_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(EP_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    addr[dev] = (uint8_t*)p;
  }
  *out = addr[dev];
  return EP_OK;
}

}  // namespace

EP_EXPORT int ep_plan_noalloc(int32_t T, int32_t K, int32_t E, int32_t W, const int32_t* topk_ids,
                              const uint8_t* active, const ep_plan_opts_t* opts, const ep_plan_t* plan,
                              void* stream) {
  ep_plan_opts_t o;
  int rc = check_plan_args(T, K, E, W, topk_ids, active, opts, plan, o);
  if (rc) return rc;
  const PlanGeometry g = plan_geometry(T, K, W);
  const bool fused = !(o.flags & EP_PLAN_LOOKBACK) && fused_fits(g.ntiles, E);
  if (!fused && (g.ntiles > kScratchTiles || (size_t)g.ntiles * E * 4 > kScratchPartBytes))
    return fail(EP_ERR_UNSUPPORTED,
                "the plan needs %d tiles x %d experts of look-back state; the static scratch holds %d tiles "
                "and %zu tile-experts (use ep_plan with a workspace)",
                g.ntiles, E, kScratchTiles, kScratchPartBytes / 4);
  rc = check_plan_overlaps(T, K, E, W, topk_ids, active, o, plan, nullptr, 0);
  if (rc) return rc;
  uint8_t* base = nullptr;
  rc = scratch_address(&base);
  if (rc) return rc;
  const PlanState st{(uint32_t*)base, (uint32_t*)(base + kScratchFlags), (int32_t*)(base + kScratchAgg),
                     (int32_t*)(base + kScratchIncl), (uint64_t*)(base + kScratchDesc)};
  return launch_plan(T, K, E, W, topk_ids, active, o, plan, st, fused, (hipStream_t)stream);
}

EP_EXPORT int ep_dispatch(int32_t T, int32_t K, int32_t H, const uint16_t* x, const int32_t* pos,
                          int32_t out_dtype, void* expand_x, float* expand_scales, const float* weights,
                          float* expand_weights, int64_t cap_rows, void* stream) {
  if (T < 0) return fail(EP_ERR_INVALID, "T must be >= 0 (got %d)", T);
  if (K < 1 || K > EP_MAX_K) return fail(EP_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)", EP_MAX_K, K);
  int rc = check_rows(H, out_dtype);
  if (rc) return rc;
  if ((int64_t)T * K >= (int64_t)1 << 31) return fail(EP_ERR_UNSUPPORTED, "T*K must be < 2^31");
  if (cap_rows < (int64_t)T * K)
    return fail(EP_ERR_INVALID, "cap_rows (%lld) must be >= T*K (%lld)", (long long)cap_rows,
                (long long)T * K);
  if (T == 0) return ok();
  if (!x || !pos || !expand_x) return fail(EP_ERR_NULLPTR, "x, pos and expand_x are required");
  const bool quant = out_dtype != EP_BF16;  // fp8 or int8 codes + one scale per row
  if (quant && !expand_scales) return fail(EP_ERR_NULLPTR, "expand_scales is required for quantised rows");
  if (!aligned(x, 16) || !aligned(expand_x, 16))
    return fail(EP_ERR_INVALID, "x and expand_x must be 16-byte aligned");
  if (!aligned(pos, 4) || (quant && !aligned(expand_scales, 4)))
    return fail(EP_ERR_INVALID, "pos and expand_scales must be 4-byte aligned");
  if ((weights == nullptr) != (expand_weights == nullptr))
    return fail(EP_ERR_NULLPTR, "weights and expand_weights go together");
  if (!aligned(weights, 4) || !aligned(expand_weights, 4))
    return fail(EP_ERR_INVALID, "weights and expand_weights must be 4-byte aligned");
  const size_t xb = (size_t)T * H * 2, pb = (size_t)T * K * 4;
  const size_t cap = reachable_rows(cap_rows);
  const size_t eb = cap * H * (quant ? 1 : 2);
  const size_t sb = quant ? cap * 4 : 0;
  const size_t wtb = weights ? pb : 0;  // weights [T][K] fp32, as large as pos
  if (overlap(expand_x, eb, x, xb) || overlap(expand_x, eb, pos, pb) || overlap(expand_x, eb, weights, wtb))
    return fail(EP_ERR_INVALID, "expand_x overlaps an input");
  if (quant && (overlap(expand_scales, sb, x, xb) || overlap(expand_scales, sb, pos, pb) ||
              overlap(expand_scales, sb, weights, wtb) || overlap(expand_scales, sb, expand_x, eb)))
    return fail(EP_ERR_INVALID, "expand_scales overlaps another buffer");
  const size_t wb = expand_weights ? cap * 4 : 0;
  if (expand_weights &&
      (overlap(expand_weights, wb, x, xb) || overlap(expand_weights, wb, pos, pb) ||
       overlap(expand_weights, wb, expand_x, eb) || overlap(expand_weights, wb, weights, pb) ||
       (quant && overlap(expand_weights, wb, expand_scales, sb))))
    return fail(EP_ERR_INVALID, "expand_weights overlaps another buffer");

  hipStream_t s = (hipStream_t)stream;
  const dim3 block(ep::kRowThreads);
  if (!quant) {
    const int V = H / 8;
    const int chunks = (V + ep::kWave * kDispatchUnroll - 1) / (ep::kWave * kDispatchUnroll);
    const int64_t Ts = slice_tokens((int64_t)chunks * ep::kWave);
    for (int64_t t0 = 0; t0 < T; t0 += Ts) {
      const int Tn = (int)(T - t0 < Ts ? T - t0 : Ts);
      const int64_t items = (int64_t)Tn * chunks;
      const dim3 cgrid((unsigned)((items + ep::kTokensPerBlock - 1) / ep::kTokensPerBlock));
      hipLaunchKernelGGL((ep::dispatch_bf16_kernel<kDispatchUnroll, kDispatchNtLoad, kDispatchNtStore>), cgrid,
                         block, 0, s, (const ep::u32x4*)x + t0 * V, pos + t0 * K, (ep::u32x4*)expand_x,
                         weights ? weights + t0 * K : nullptr, expand_weights, Tn, K, V, chunks, cap_rows);
      rc = launch_status("ep_dispatch (bf16)");
      if (rc) return rc;
    }
    return ok();
  }
  const int NG = H / 16;
  ep::u32x4* qv = (ep::u32x4*)expand_x;
  const int per_thread = (NG + ep::kRowThreads - 1) / ep::kRowThreads;
  const int64_t Ts = slice_tokens(ep::kRowThreads);  // one workgroup per token
  for (int64_t t0 = 0; t0 < T; t0 += Ts) {
    const int Tn = (int)(T - t0 < Ts ? T - t0 : Ts);
    const dim3 tgrid((unsigned)Tn);
    const ep::u32x4* xv = (const ep::u32x4*)x + t0 * NG * 2;
    const int32_t* pn = pos + t0 * K;
    const float* wn = weights ? weights + t0 * K : nullptr;
    auto launch = [&](auto qt) {
      constexpr int QT = decltype(qt)::value;
#define EP_QDISP(G)                                                                                          \
  hipLaunchKernelGGL((ep::dispatch_quant_kernel<QT, G, kQuantNtLoad, kQuantNtStore>), tgrid, block, 0, s, xv, pn, qv, \
                     expand_scales, wn, expand_weights, Tn, K, NG, cap_rows)
      if (per_thread <= 1) EP_QDISP(1);
      else if (per_thread <= 2) EP_QDISP(2);
      else if (per_thread <= 4) EP_QDISP(4);
      else EP_QDISP(8);
#undef EP_QDISP
    };
    if (out_dtype == EP_FP8_E4M3FN) launch(std::integral_constant<int, ep::kQFp8>{});
    else launch(std::integral_constant<int, ep::kQInt8>{});
    rc = launch_status("ep_dispatch (quantised rows)");
    if (rc) return rc;
  }
  return ok();
}

EP_EXPORT int ep_combine(int32_t T, int32_t K, int32_t H, const uint16_t* y, int64_t cap_rows,
                         const int32_t* pos, const float* weights, uint16_t* out, void* stream) {
  if (T < 0) return fail(EP_ERR_INVALID, "T must be >= 0 (got %d)", T);
  if (K < 1 || K > EP_MAX_K) return fail(EP_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)", EP_MAX_K, K);
  int rc = check_rows(H, EP_BF16);
  if (rc) return rc;
  if ((int64_t)T * K >= (int64_t)1 << 31) return fail(EP_ERR_UNSUPPORTED, "T*K must be < 2^31");
  if (cap_rows < 0) return fail(EP_ERR_INVALID, "cap_rows must be >= 0");
  if (T == 0) return ok();
  if (!y || !pos || !weights || !out) return fail(EP_ERR_NULLPTR, "y, pos, weights and out are required");
  if (!aligned(y, 16) || !aligned(out, 16)) return fail(EP_ERR_INVALID, "y and out must be 16-byte aligned");
  if (!aligned(pos, 4) || !aligned(weights, 4)) return fail(EP_ERR_INVALID, "pos and weights must be 4-byte aligned");
  const size_t ob = (size_t)T * H * 2;
  if (overlap(out, ob, y, reachable_rows(cap_rows) * H * 2) || overlap(out, ob, pos, (size_t)T * K * 4) ||
      overlap(out, ob, weights, (size_t)T * K * 4))
    return fail(EP_ERR_INVALID, "out overlaps an input");

  hipStream_t s = (hipStream_t)stream;
  const dim3 block(kCombineWaves * ep::kWave);
  const int V = H / 8;
  const int chunks = (V + ep::kWave * kCombineUnroll - 1) / (ep::kWave * kCombineUnroll);
  const ep::u32x4* yv = (const ep::u32x4*)y;
  const int64_t Ts = slice_tokens((int64_t)chunks * ep::kWave);
  for (int64_t t0 = 0; t0 < T; t0 += Ts) {
    const int Tn = (int)(T - t0 < Ts ? T - t0 : Ts);
    const int64_t items = (int64_t)Tn * chunks;
    const dim3 cgrid((unsigned)((items + kCombineWaves - 1) / kCombineWaves));
    const int32_t* pn = pos + t0 * K;
    const float* wn = weights + t0 * K;
    ep::u32x4* ov = (ep::u32x4*)out + t0 * V;
    if (K <= 4)
      hipLaunchKernelGGL((ep::combine_kernel<4, kCombineUnroll, kCombineWaves, kCombineNtLoad, kCombineNtStore>),
                         cgrid, block, 0, s, yv, pn, wn, ov, Tn, K, V, chunks, cap_rows);
    else if (K <= 8)
      hipLaunchKernelGGL((ep::combine_kernel<8, kCombineUnroll, kCombineWaves, kCombineNtLoad, kCombineNtStore>),
                         cgrid, block, 0, s, yv, pn, wn, ov, Tn, K, V, chunks, cap_rows);
    else
      hipLaunchKernelGGL((ep::combine_kernel<16, kCombineUnroll, kCombineWaves, kCombineNtLoad, kCombineNtStore>),
                         cgrid, block, 0, s, yv, pn, wn, ov, Tn, K, V, chunks, cap_rows);
    rc = launch_status("ep_combine");
    if (rc) return rc;
  }
  return ok();
}

constexpr int kSmoothMaxH = 16384;  // 4 groups of 16 values per thread stay in VGPRs

EP_EXPORT int ep_dispatch_smooth(int32_t T, int32_t K, int32_t E, int32_t H, const uint16_t* x,
                                 const int32_t* topk_ids, const int32_t* pos, const float* smooth_scales,
                                 int32_t out_dtype, void* expand_x, float* expand_scales, int64_t cap_rows,
                                 void* stream) {
  if (T < 0) return fail(EP_ERR_INVALID, "T must be >= 0 (got %d)", T);
  if (K < 1 || K > EP_MAX_K) return fail(EP_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)", EP_MAX_K, K);
  if (E < 1 || E > EP_MAX_E) return fail(EP_ERR_UNSUPPORTED, "E must be in [1, %d] (got %d)", EP_MAX_E, E);
  if (out_dtype != EP_FP8_E4M3FN && out_dtype != EP_INT8)
    return fail(EP_ERR_INVALID, "smoothing quantises to fp8 or int8 rows (got dtype %d)", out_dtype);
  int rc = check_rows(H, out_dtype);
  if (rc) return rc;
  if (H > kSmoothMaxH) return fail(EP_ERR_UNSUPPORTED, "H must be <= %d with smoothing (got %d)", kSmoothMaxH, H);
  if ((int64_t)T * K >= (int64_t)1 << 31) return fail(EP_ERR_UNSUPPORTED, "T*K must be < 2^31");
  if (cap_rows < (int64_t)T * K)
    return fail(EP_ERR_INVALID, "cap_rows (%lld) must be >= T*K", (long long)cap_rows);
  if (T == 0) return ok();
  if (!x || !topk_ids || !pos || !smooth_scales || !expand_x || !expand_scales)
    return fail(EP_ERR_NULLPTR, "x, topk_ids, pos, smooth_scales, expand_x and expand_scales are required");
  if (!aligned(x, 16) || !aligned(expand_x, 16) || !aligned(smooth_scales, 16))
    return fail(EP_ERR_INVALID, "x, expand_x and smooth_scales must be 16-byte aligned");
  if (!aligned(topk_ids, 4) || !aligned(pos, 4) || !aligned(expand_scales, 4))
    return fail(EP_ERR_INVALID, "topk_ids, pos and expand_scales must be 4-byte aligned");
  const size_t eb = reachable_rows(cap_rows) * H, sb = reachable_rows(cap_rows) * 4;
  const Range_ ins[] = {{x, (size_t)T * H * 2}, {topk_ids, (size_t)T * K * 4}, {pos, (size_t)T * K * 4},
                        {smooth_scales, (size_t)E * H * 4}};
  for (const auto& r : ins)
    if (overlap(expand_x, eb, r.p, r.n) || overlap(expand_scales, sb, r.p, r.n))
      return fail(EP_ERR_INVALID, "an output overlaps an input");
  if (overlap(expand_x, eb, expand_scales, sb)) return fail(EP_ERR_INVALID, "expand_x overlaps expand_scales");
  const int NG = H / 16;
  const int per_thread = (NG + ep::kRowThreads - 1) / ep::kRowThreads;
  hipStream_t s = (hipStream_t)stream;
  const float4* sm = (const float4*)smooth_scales;
  ep::u32x4* qv = (ep::u32x4*)expand_x;
  const int64_t Ts = slice_tokens(ep::kRowThreads);  // one workgroup per token
  for (int64_t t0 = 0; t0 < T; t0 += Ts) {
    const int Tn = (int)(T - t0 < Ts ? T - t0 : Ts);
    const ep::u32x4* xv = (const ep::u32x4*)x + t0 * NG * 2;
    const int32_t* idn = topk_ids + t0 * K;
    const int32_t* pn = pos + t0 * K;
    auto launch = [&](auto qt) {
      constexpr int QT = decltype(qt)::value;
#define EP_SMOOTH(G)                                                                                      \
  hipLaunchKernelGGL((ep::dispatch_smooth_kernel<QT, G, kQuantNtStore>), dim3((unsigned)Tn), dim3(ep::kRowThreads), \
                     0, s, xv, idn, pn, sm, qv, expand_scales, Tn, K, E, NG, cap_rows)
      if (per_thread <= 1) EP_SMOOTH(1);
      else if (per_thread <= 2) EP_SMOOTH(2);
      else EP_SMOOTH(4);
#undef EP_SMOOTH
    };
    if (out_dtype == EP_FP8_E4M3FN) launch(std::integral_constant<int, ep::kQFp8>{});
    else launch(std::integral_constant<int, ep::kQInt8>{});
    rc = launch_status("ep_dispatch_smooth");
    if (rc) return rc;
  }
  return ok();
}

EP_EXPORT int ep_combine_quant(int32_t T, int32_t K, int32_t H, const void* codes, int32_t code_dtype,
                               const float* row_scales, int64_t cap_rows, const int32_t* pos,
                               const float* weights, uint16_t* out, void* stream) {
  if (T < 0) return fail(EP_ERR_INVALID, "T must be >= 0 (got %d)", T);
  if (K < 1 || K > EP_MAX_K) return fail(EP_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)", EP_MAX_K, K);
  if (code_dtype != EP_FP8_E4M3FN && code_dtype != EP_INT8)
    return fail(EP_ERR_INVALID, "codes must be fp8 or int8 (got dtype %d)", code_dtype);
  int rc = check_rows(H, code_dtype);
  if (rc) return rc;
  if ((int64_t)T * K >= (int64_t)1 << 31) return fail(EP_ERR_UNSUPPORTED, "T*K must be < 2^31");
  if (cap_rows < 0) return fail(EP_ERR_INVALID, "cap_rows must be >= 0");
  if (T == 0) return ok();
  if (!codes || !row_scales || !pos || !weights || !out)
    return fail(EP_ERR_NULLPTR, "codes, row_scales, pos, weights and out are required");
  if (!aligned(codes, 16) || !aligned(out, 16)) return fail(EP_ERR_INVALID, "codes and out must be 16-byte aligned");
  if (!aligned(row_scales, 4) || !aligned(pos, 4) || !aligned(weights, 4))
    return fail(EP_ERR_INVALID, "row_scales, pos and weights must be 4-byte aligned");
  const size_t ob = (size_t)T * H * 2;
  if (overlap(out, ob, codes, reachable_rows(cap_rows) * H) ||
      overlap(out, ob, row_scales, reachable_rows(cap_rows) * 4) ||
      overlap(out, ob, pos, (size_t)T * K * 4) || overlap(out, ob, weights, (size_t)T * K * 4))
    return fail(EP_ERR_INVALID, "out overlaps an input");
  const int NG = H / 16;
  const int chunks = (NG + ep::kWave - 1) / ep::kWave;
  const dim3 block(kCombineQuantWaves * ep::kWave);
  hipStream_t s = (hipStream_t)stream;
  const ep::u32x4* cv = (const ep::u32x4*)codes;
  const int64_t Ts = slice_tokens((int64_t)chunks * ep::kWave);
  for (int64_t t0 = 0; t0 < T; t0 += Ts) {
    const int Tn = (int)(T - t0 < Ts ? T - t0 : Ts);
    const int64_t items = (int64_t)Tn * chunks;
    const dim3 grid((unsigned)((items + kCombineQuantWaves - 1) / kCombineQuantWaves));
    const int32_t* pn = pos + t0 * K;
    const float* wn = weights + t0 * K;
    ep::u32x4* ov = (ep::u32x4*)out + t0 * NG * 2;
    auto launch = [&](auto qt) {
      constexpr int QT = decltype(qt)::value;
      if (K <= 4)
        hipLaunchKernelGGL((ep::combine_quant_kernel<QT, 4, kCombineQuantWaves, kCombineNtLoad, kCombineNtStore>),
                           grid, block, 0, s, cv, row_scales, pn, wn, ov, Tn, K, NG, chunks, cap_rows);
      else if (K <= 8)
        hipLaunchKernelGGL((ep::combine_quant_kernel<QT, 8, kCombineQuantWaves, kCombineNtLoad, kCombineNtStore>),
                           grid, block, 0, s, cv, row_scales, pn, wn, ov, Tn, K, NG, chunks, cap_rows);
      else
        hipLaunchKernelGGL((ep::combine_quant_kernel<QT, 16, kCombineQuantWaves, kCombineNtLoad, kCombineNtStore>),
                           grid, block, 0, s, cv, row_scales, pn, wn, ov, Tn, K, NG, chunks, cap_rows);
    };
    if (code_dtype == EP_FP8_E4M3FN) launch(std::integral_constant<int, ep::kQFp8>{});
    else launch(std::integral_constant<int, ep::kQInt8>{});
    rc = launch_status("ep_combine_quant");
    if (rc) return rc;
  }
  return ok();
}

namespace {

constexpr int kTailMaxH = 16384;  // two vectors per thread of a 1024-thread workgroup

int check_tail(int32_t T, int32_t H, const void* residual, const void* gamma, float eps,
               const void* residual_out, const void* norm_out) {
  if (T < 0) return fail(EP_ERR_INVALID, "T must be >= 0 (got %d)", T);
  if (H < 8 || H % 8 || H > kTailMaxH)
    return fail(EP_ERR_UNSUPPORTED, "H must be a multiple of 8 in [8, %d] (got %d)", kTailMaxH, H);
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(EP_ERR_INVALID, "eps must be finite and >= 0");
  if (T == 0) return EP_OK;
  if (!residual || !gamma || !residual_out || !norm_out)
    return fail(EP_ERR_NULLPTR, "residual, gamma, residual_out and norm_out are required");
  if (!aligned(residual, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) || !aligned(norm_out, 16))
    return fail(EP_ERR_INVALID, "residual, gamma, residual_out and norm_out must be 16-byte aligned");
  const size_t rb = (size_t)T * H * 2;
  if (overlap(residual_out, rb, residual, rb) || overlap(residual_out, rb, gamma, (size_t)H * 2) ||
      overlap(norm_out, rb, residual, rb) || overlap(norm_out, rb, gamma, (size_t)H * 2) ||
      overlap(norm_out, rb, residual_out, rb))
    return fail(EP_ERR_INVALID, "residual_out and norm_out must not overlap each other or an input");
  return EP_OK;
}

// One workgroup per token, sized by the row: 256 threads up to 256 vectors
// (H <= 2048), then 512, then 1024, so that a thread holds at most two
// vectors (H <= 16384).  Larger workgroups measured 3-5% faster at H = 7168
// (fewer sequential load rounds per thread).  The fused tail and the tail
// alone pick the same size for the same H, so their sums of squares run in
// the same order and their outputs are bit-identical.
int tail_threads(int V) { return V <= 256 ? 256 : V <= 512 ? 512 : 1024; }

// One workgroup per token, launched over token slices (slice_tokens); x and
// pos / w are NULL for the tail alone and for no combine input respectively.
template <int KMAX>
int launch_tail(const char* what, int V, hipStream_t s, const ep::u32x4* y, const int32_t* pos,
                const float* w, const ep::u32x4* x, const ep::u32x4* res, const ep::u32x4* gamma, float eps,
                ep::u32x4* ro, ep::u32x4* no, int T, int K, int64_t cap) {
  const int nt = tail_threads(V);
  const int NV = (V + nt - 1) / nt;
  const int64_t Ts = slice_tokens(nt);
  for (int64_t t0 = 0; t0 < T; t0 += Ts) {
    const int Tn = (int)(T - t0 < Ts ? T - t0 : Ts);
    const dim3 grid((unsigned)Tn);
    const int32_t* pn = pos ? pos + t0 * K : nullptr;
    const float* wn = w ? w + t0 * K : nullptr;
    const ep::u32x4* xn = x ? x + t0 * V : nullptr;
    const ep::u32x4* rn = res + t0 * V;
    ep::u32x4* ron = ro + t0 * V;
    ep::u32x4* non = no + t0 * V;
#define EP_TAIL(NT, NVV)                                                                            \
  hipLaunchKernelGGL((ep::combine_add_rmsnorm_kernel<KMAX, NVV, NT, kCombineNtLoad, kCombineNtStore>), \
                     grid, dim3(NT), 0, s, y, pn, wn, xn, rn, gamma, eps, ron, non, Tn, K, V, cap)
    if (nt == 256) {
      EP_TAIL(256, 1);  // V <= 256
    } else if (nt == 512) {
      EP_TAIL(512, 1);  // V <= 512
    } else if (NV <= 1) {
      EP_TAIL(1024, 1);
    } else {
      EP_TAIL(1024, 2);  // V <= 2048 (H <= 16384)
    }
#undef EP_TAIL
    const int rc = launch_status(what);
    if (rc) return rc;
  }
  return ok();
}

}  // namespace

EP_EXPORT int ep_combine_add_rmsnorm(int32_t T, int32_t K, int32_t H, const uint16_t* y, int64_t cap_rows,
                                     const int32_t* pos, const float* weights, const uint16_t* residual,
                                     const uint16_t* gamma, float eps, uint16_t* residual_out,
                                     uint16_t* norm_out, void* stream) {
  if (K < 1 || K > EP_MAX_K) return fail(EP_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)", EP_MAX_K, K);
  int rc = check_tail(T, H, residual, gamma, eps, residual_out, norm_out);
  if (rc) return rc;
  if ((int64_t)T * K >= (int64_t)1 << 31) return fail(EP_ERR_UNSUPPORTED, "T*K must be < 2^31");
  if (cap_rows < 0) return fail(EP_ERR_INVALID, "cap_rows must be >= 0");
  if (T == 0) return ok();
  if (!y || !pos || !weights) return fail(EP_ERR_NULLPTR, "y, pos and weights are required");
  if (!aligned(y, 16)) return fail(EP_ERR_INVALID, "y must be 16-byte aligned");
  if (!aligned(pos, 4) || !aligned(weights, 4)) return fail(EP_ERR_INVALID, "pos and weights must be 4-byte aligned");
  const size_t rb = (size_t)T * H * 2, yb = reachable_rows(cap_rows) * H * 2, pb = (size_t)T * K * 4;
  for (const void* o : {(const void*)residual_out, (const void*)norm_out})
    if (overlap(o, rb, y, yb) || overlap(o, rb, pos, pb) || overlap(o, rb, weights, pb))
      return fail(EP_ERR_INVALID, "an output overlaps an input");
  const int V = H / 8;
  hipStream_t s = (hipStream_t)stream;
  auto args = [&](auto launch) {
    return launch("ep_combine_add_rmsnorm", V, s, (const ep::u32x4*)y, pos, weights,
                  (const ep::u32x4*)nullptr, (const ep::u32x4*)residual, (const ep::u32x4*)gamma, eps,
                  (ep::u32x4*)residual_out, (ep::u32x4*)norm_out, T, K, cap_rows);
  };
  if (K <= 4) return args(launch_tail<4>);
  if (K <= 8) return args(launch_tail<8>);
  return args(launch_tail<16>);
}

EP_EXPORT int ep_add_rmsnorm(int32_t T, int32_t H, const uint16_t* x, const uint16_t* residual,
                             const uint16_t* gamma, float eps, uint16_t* residual_out, uint16_t* norm_out,
                             void* stream) {
  int rc = check_tail(T, H, residual, gamma, eps, residual_out, norm_out);
  if (rc) return rc;
  if (T == 0) return ok();
  if (!x) return fail(EP_ERR_NULLPTR, "x is required");
  if (!aligned(x, 16)) return fail(EP_ERR_INVALID, "x must be 16-byte aligned");
  const size_t rb = (size_t)T * H * 2;
  if (overlap(residual_out, rb, x, rb) || overlap(norm_out, rb, x, rb))
    return fail(EP_ERR_INVALID, "an output overlaps x");
  const int V = H / 8;
  return launch_tail<1>("ep_add_rmsnorm", V, (hipStream_t)stream, nullptr, nullptr, nullptr,
                        (const ep::u32x4*)x, (const ep::u32x4*)residual, (const ep::u32x4*)gamma, eps,
                        (ep::u32x4*)residual_out, (ep::u32x4*)norm_out, T, 1, 0);
}

EP_EXPORT int ep_plan_splits(int32_t W, const int64_t* in_splits, int64_t* src_offsets,
                             int64_t* out_splits, int64_t* dst_offsets, int64_t* rank_offsets,
                             void* stream) {
  if (W < 1 || W > EP_MAX_SPLITS_W)
    return fail(EP_ERR_UNSUPPORTED, "W must be in [1, %d] (got %d)", EP_MAX_SPLITS_W, W);
  if (!in_splits || !src_offsets || !out_splits || !dst_offsets || !rank_offsets)
    return fail(EP_ERR_NULLPTR, "all plan arrays are required");
  const void* ps[] = {in_splits, src_offsets, out_splits, dst_offsets, rank_offsets};
  const size_t ns[] = {(size_t)W * W * 8, (size_t)W * W * 8, (size_t)W * W * 8, (size_t)W * W * 8,
                       (size_t)(W + 1) * 8};
  for (int i = 0; i < 5; ++i) {
    if (!aligned(ps[i], 8)) return fail(EP_ERR_INVALID, "split arrays must be 8-byte aligned");
    for (int j = i + 1; j < 5; ++j)
      if (overlap(ps[i], ns[i], ps[j], ns[j])) return fail(EP_ERR_INVALID, "split arrays overlap");
  }
  hipLaunchKernelGGL(ep::plan_splits_kernel, dim3(1), dim3(ep::kSplitsPlanThreads), 0, (hipStream_t)stream,
                     W, in_splits, src_offsets, out_splits, dst_offsets, rank_offsets);
  return launch_status("ep_plan_splits");
}

EP_EXPORT int ep_dispatch_splits(int32_t W, int64_t R, int64_t stride_bytes, const void* in,
                                 const int64_t* src_offsets, const int64_t* out_splits,
                                 const int64_t* dst_offsets, const int64_t* rank_offsets, void* out,
                                 void* stream) {
  if (W < 1 || W > EP_MAX_SPLITS_W)
    return fail(EP_ERR_UNSUPPORTED, "W must be in [1, %d] (got %d)", EP_MAX_SPLITS_W, W);
  if (R < 0) return fail(EP_ERR_INVALID, "R must be >= 0");
  if (stride_bytes <= 0 || stride_bytes % 16)
    return fail(EP_ERR_UNSUPPORTED, "stride_bytes must be a positive multiple of 16 (got %lld)",
                (long long)stride_bytes);
  if (!splits_bytes_fit(W, R, stride_bytes))
    return fail(EP_ERR_UNSUPPORTED, "W * R * stride_bytes must fit in 63 bits");
  if (R == 0) return ok();
  if (!in || !out || !src_offsets || !out_splits || !dst_offsets || !rank_offsets)
    return fail(EP_ERR_NULLPTR, "all buffers are required");
  if (!aligned(in, 16) || !aligned(out, 16)) return fail(EP_ERR_INVALID, "in and out must be 16-byte aligned");
  const size_t bytes = (size_t)W * R * stride_bytes;
  if (overlap(in, bytes, out, bytes)) return fail(EP_ERR_INVALID, "out overlaps in");
  const int64_t* plan[] = {src_offsets, out_splits, dst_offsets, rank_offsets};
  const size_t plan_bytes[] = {(size_t)W * W * 8, (size_t)W * W * 8, (size_t)W * W * 8,
                               (size_t)(W + 1) * 8};
  for (int i = 0; i < 4; ++i)
    if (overlap(out, bytes, plan[i], plan_bytes[i]))
      return fail(EP_ERR_INVALID, "out overlaps a plan array");
  const int64_t Vr = stride_bytes / 16;
  const int chunks = W * W;
  int bpc = (2048 + chunks - 1) / chunks;
  const int64_t max_rows_per_chunk = R;  // no chunk holds more than its sender's R rows
  const int64_t need = (max_rows_per_chunk + ep::kTokensPerBlock - 1) / ep::kTokensPerBlock;
  if (bpc > need) bpc = (int)need;
  if (bpc < 1) bpc = 1;
  const dim3 grid(chunks, bpc);
  hipStream_t s = (hipStream_t)stream;
  const ep::u32x4* iv = (const ep::u32x4*)in;
  ep::u32x4* ov = (ep::u32x4*)out;
  const int64_t per_lane = (Vr + ep::kWave - 1) / ep::kWave;
  if (per_lane <= 1)
    hipLaunchKernelGGL((ep::copy_splits_kernel<1, kCopyNtLoad, kCopyNtStore>), grid, dim3(ep::kRowThreads), 0, s, iv, ov, src_offsets,
                       out_splits, dst_offsets, rank_offsets, W, R, Vr);
  else if (per_lane <= 2)
    hipLaunchKernelGGL((ep::copy_splits_kernel<2, kCopyNtLoad, kCopyNtStore>), grid, dim3(ep::kRowThreads), 0, s, iv, ov, src_offsets,
                       out_splits, dst_offsets, rank_offsets, W, R, Vr);
  else if (per_lane <= 4)
    hipLaunchKernelGGL((ep::copy_splits_kernel<4, kCopyNtLoad, kCopyNtStore>), grid, dim3(ep::kRowThreads), 0, s, iv, ov, src_offsets,
                       out_splits, dst_offsets, rank_offsets, W, R, Vr);
  else
    hipLaunchKernelGGL((ep::copy_splits_kernel<8, kCopyNtLoad, kCopyNtStore>), grid, dim3(ep::kRowThreads), 0, s, iv, ov, src_offsets,
                       out_splits, dst_offsets, rank_offsets, W, R, Vr);
  return launch_status("ep_dispatch_splits");
}

EP_EXPORT int ep_all_to_all_splits(int32_t W, int64_t R, int64_t stride_bytes, const int64_t* in_splits,
                                   const void* in, void* out, int64_t* src_offsets, int64_t* out_splits,
                                   int64_t* dst_offsets, int64_t* rank_offsets, void* stream) {
  if (W < 1 || W > EP_MAX_SPLITS_W)
    return fail(EP_ERR_UNSUPPORTED, "W must be in [1, %d] (got %d)", EP_MAX_SPLITS_W, W);
  if (R < 0) return fail(EP_ERR_INVALID, "R must be >= 0");
  if (stride_bytes <= 0 || stride_bytes % 16)
    return fail(EP_ERR_UNSUPPORTED, "stride_bytes must be a positive multiple of 16 (got %lld)",
                (long long)stride_bytes);
  if (!splits_bytes_fit(W, R, stride_bytes))
    return fail(EP_ERR_UNSUPPORTED, "W * R * stride_bytes must fit in 63 bits");
  const bool any_plan = src_offsets || out_splits || dst_offsets || rank_offsets;
  if (R == 0 && !any_plan) return ok();
  if (!in_splits) return fail(EP_ERR_NULLPTR, "in_splits is required");
  if (R > 0 && (!in || !out)) return fail(EP_ERR_NULLPTR, "in and out are required");
  if (R > 0 && (!aligned(in, 16) || !aligned(out, 16)))
    return fail(EP_ERR_INVALID, "in and out must be 16-byte aligned");
  const size_t bytes = (size_t)W * R * stride_bytes;
  const size_t mb = (size_t)W * W * 8;
  const void* arrays[] = {in_splits, src_offsets, out_splits, dst_offsets, rank_offsets, in, out};
  const size_t sizes[] = {mb, mb, mb, mb, (size_t)(W + 1) * 8, bytes, bytes};
  for (int i = 0; i < 5; ++i)
    if (arrays[i] && !aligned(arrays[i], 8)) return fail(EP_ERR_INVALID, "split arrays must be 8-byte aligned");
  // outputs (1-4, 6) must not overlap each other or an input (0, 5)
  for (int i = 0; i < 7; ++i)
    for (int j = i + 1; j < 7; ++j) {
      const bool out_i = i != 0 && i != 5, out_j = j != 0 && j != 5;
      if ((out_i || out_j) && arrays[i] && arrays[j] && sizes[i] && sizes[j] &&
          overlap(arrays[i], sizes[i], arrays[j], sizes[j]))
        return fail(EP_ERR_INVALID, "an output of the all-to-all overlaps another buffer");
    }
  // Work split by output rows (at most W*R of them): a wave copies a run of
  // rows of about kA2ARowsPerWaveBytes, a workgroup four runs at a time; at
  // most kA2ABlocks workgroups (four per CU on MI355X), each looping over
  // runs, so every workgroup's setup (staging the send matrix, its receiver
  // bases) serves several runs.  Measured on W=8, R=4096, 4 KB rows against
  // one workgroup per four runs: 41 against 43 us warm, 52 against 56 us
  // with the Infinity Cache flushed.
  const int64_t Vr = stride_bytes / 16;
  int64_t rows_per_wave = ep::kA2ARowsPerWaveBytes / stride_bytes;
  if (rows_per_wave < 1) rows_per_wave = 1;
  const int64_t rows = (int64_t)W * R;
  const int64_t per_block = rows_per_wave * ep::kTokensPerBlock;
  const int64_t n_ranges = (rows + per_block - 1) / per_block;
  int64_t blocks = n_ranges < ep::kA2ABlocks ? n_ranges : ep::kA2ABlocks;
  if (blocks < 1) blocks = 1;
  const size_t lds = ((size_t)W * W + W + 1) * sizeof(int64_t);
  hipStream_t s = (hipStream_t)stream;
  const ep::u32x4* iv = (const ep::u32x4*)in;
  ep::u32x4* ov = (ep::u32x4*)out;
  const int64_t per_lane = (Vr + ep::kWave - 1) / ep::kWave;
#define EP_A2A(U)                                                                                               \
  hipLaunchKernelGGL((ep::all_to_all_splits_kernel<U, kCopyNtLoad, kCopyNtStore>), dim3((unsigned)blocks),        \
                     dim3(ep::kRowThreads), lds, s, iv, ov, in_splits, src_offsets, out_splits, dst_offsets,     \
                     rank_offsets, W, R, Vr, rows_per_wave, n_ranges)
  if (per_lane <= 1) EP_A2A(1);
  else if (per_lane <= 2) EP_A2A(2);
  else if (per_lane <= 4) EP_A2A(4);
  else EP_A2A(8);
#undef EP_A2A
  return launch_status("ep_all_to_all_splits");
}

EP_EXPORT const char* ep_last_error(void) { return g_last_error.c_str(); }

EP_EXPORT int ep_device_error(void* stream, int32_t* code) {
  if (!code) return fail(EP_ERR_NULLPTR, "code is NULL");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(EP_ERR_HIP, "stream synchronize failed: %s", hipGetErrorString(e));
  unsigned int v = 0;
  e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(ep::g_device_error), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(EP_ERR_HIP, "reading the device error word failed: %s", hipGetErrorString(e));
  if (v != 0) {
    // Only the bits just read are cleared (an atomic AND on the device), so
    // a bit raised meanwhile by a kernel on another stream is kept for the
    // next call.
    hipLaunchKernelGGL(clear_error_bits_kernel, dim3(1), dim3(1), 0, (hipStream_t)stream, v);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(EP_ERR_HIP, "clearing the device error word failed: %s", hipGetErrorString(e));
  }
  *code = (int32_t)v;
  return ok();
}
