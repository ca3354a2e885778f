// ep_plan_kernels.h -- exchange plan, stable occurrences and positions.
//
// What is computed (PyTorch compare view "ciflow/h100-symm-mem/166772":
// make2dExchangePlan, get_occurrence_numbers, _allToAllV_2d_index_push_kernel):
// split counts per (source rank, expert), their scans, the transposed
// out_splits, and for every live copy (t,k) its global expandX row
//   pos = expert_offsets[e] + #(earlier live copies of expert e, all ranks)
// which equals rank_offsets[d] + dst_offsets[s][e] + occurrence.
//
// Two paths.  plan_fused_kernel (below) computes everything in one launch
// when all tiles fit on the device at once: tiles exchange their counts as
// self-validating descriptors while running.  Larger grids use two kernels:
//  1. plan_tile_kernel -- one workgroup per tile of tokens of one source rank.
//     Each wave ranks its 64-copy chunks in order with a ballot-based
//     match-any over the expert-id bits (stable, no LDS atomics), keeping a
//     private per-wave histogram in LDS; waves are combined in wave order.
//     The tile's histogram is then scanned across tiles with a decoupled
//     look-back (tile ids from an atomic ticket, so every predecessor is
//     already running): each tile publishes its aggregate, accumulates
//     predecessors' aggregates until it meets an inclusive prefix, then
//     publishes its own inclusive prefix.  It writes, per copy, the number
//     of earlier live copies of the same expert over all tiles (a partial
//     position, into pos).
//  2. plan_finalize_kernel -- every workgroup rescans the E expert totals
//     (the last tile's inclusive prefix) to get expert_offsets; workgroup s<W
//     writes rank s's rows of the W x E plan arrays; all workgroups turn the
//     partial positions into final positions and occurrences.  Workgroup 0
//     returns the look-back flags and ticket to zero for the next call.
#pragma once

#include "ep_common.h"

namespace ep {

constexpr int kPlanThreads = 512;
constexpr int kPlanWaves = kPlanThreads / kWave;           // 8
constexpr int kPlanChunks = 4;                              // 64-copy chunks per wave
constexpr int kPlanTileCopies = kPlanWaves * kWave * kPlanChunks;  // 2048

constexpr uint32_t kFlagAggregate = 1u;
constexpr uint32_t kFlagInclusive = 2u;
constexpr int kSpinLimit = 1 << 20;  // bounded polling: the kernel always exits
constexpr int kTestSpinLimit = 256;  // the stall test's budget (EP_PLAN_TEST_STALL)

constexpr int kFinalizeThreads = 256;
constexpr int kFinalizeCopiesPerThread = 4;

// Rows an expert with `count` rows occupies in expandX: padded up to a
// multiple of `align`, and one unit for an empty expert with pad_empty.
__device__ __forceinline__ int padded_rows(int count, int align, int pad_empty) {
  int p = (count + align - 1) / align * align;
  if (pad_empty && p == 0) p = align;
  return p;
}

// Rank g's expert token numbers: counts (type 1) or their inclusive prefix
// over the rank's local experts (type 0).
__device__ void write_expert_token_nums(const int32_t* cnt, int g, int ne, int type, int64_t* out,
                                        int nthreads) {
  for (int le = threadIdx.x; le < ne; le += nthreads) {
    int64_t v = cnt[g * ne + le];
    if (type == 0) {
      v = 0;
      for (int l2 = 0; l2 <= le; ++l2) v += cnt[g * ne + l2];
    }
    out[(int64_t)g * ne + le] = v;
  }
}

// Tokens per tile: as many as fit kPlanTileCopies copies, never crossing a
// source rank boundary.
inline int plan_tile_tokens(int K, int Tw) {
  int tt = kPlanTileCopies / K;
  if (tt < 1) tt = 1;
  if (tt > Tw) tt = Tw;
  return tt < 1 ? 1 : tt;
}

__global__ __launch_bounds__(kPlanThreads) void plan_tile_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ active,
    const uint8_t* __restrict__ active_copies, int K, int E,
    int Tw, int tile_tokens, int tiles_per_rank, int ntiles, int id_bits,
    int32_t* __restrict__ pos_partial, uint32_t* ticket, uint32_t* flags,
    int32_t* aggregates, int32_t* inclusive) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                          // [kPlanWaves][E]: counts, then wave-exclusive
  int32_t* tile_agg = lds + kPlanWaves * E;     // [E]: this tile's counts
  int32_t* prefix = tile_agg + E;               // [E]: copies of e in earlier tiles
  __shared__ int s_tile;
  __shared__ int s_lo, s_hi, s_incl, s_more;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;

  if (tid == 0) s_tile = (int)__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = tid; i < (kPlanWaves + 2) * E; i += kPlanThreads) lds[i] = 0;
  __syncthreads();
  const int b = s_tile;
  if (b >= ntiles) {  // only possible with a workspace that was never initialised
    if (tid == 0) raise_device_error(kErrPlanStall);
    return;
  }

  const int s = b / tiles_per_rank;
  const int j = b - s * tiles_per_rank;
  const int64_t t0 = (int64_t)s * Tw + (int64_t)j * tile_tokens;
  int64_t t1 = t0 + tile_tokens;
  if (t1 > (int64_t)(s + 1) * Tw) t1 = (int64_t)(s + 1) * Tw;
  const int64_t c0 = t0 * K;
  const int n = (int)((t1 - t0) * K);
  const int seg = (n + kPlanWaves - 1) / kPlanWaves;
  const int cs = wave * seg;                       // wave's first copy, tile-relative
  const int ce = min(cs + seg, n);

  // All of the wave's ids and mask bytes are requested before any is used
  // (the bytes are combined once loaded: a short-circuit test would wait for
  // each byte before issuing the next load).
  int e_reg[kPlanChunks];
  uint32_t a_reg[kPlanChunks], ac_reg[kPlanChunks];
#pragma unroll
  for (int ch = 0; ch < kPlanChunks; ++ch) {
    const int c = cs + ch * kWave + lane;
    e_reg[ch] = -1;
    a_reg[ch] = 0;
    ac_reg[ch] = 1;
    if (c < ce) {
      const int64_t gc = c0 + c;
      e_reg[ch] = ids[gc];
      a_reg[ch] = active ? active[gc / K] : 1u;
      if (active_copies) ac_reg[ch] = active_copies[gc];
    }
  }
  bool act_reg[kPlanChunks];
#pragma unroll
  for (int ch = 0; ch < kPlanChunks; ++ch) act_reg[ch] = a_reg[ch] != 0 && ac_reg[ch] != 0;

  // Stable in-wave ranking, chunk by chunk, in flattened (t,k) order: peers
  // (lanes holding the same expert) come from one ballot per id bit; a lane's
  // rank is its wave's running count for the expert plus the peers below it;
  // the highest peer advances the count.
  int32_t* myhist = hist + wave * E;
  int r_reg[kPlanChunks];
#pragma unroll
  for (int ch = 0; ch < kPlanChunks; ++ch) {
    const int e = e_reg[ch];
    bool live = false;
    if (act_reg[ch]) {
      live = (unsigned)e < (unsigned)E;
      if (!live) raise_device_error(kErrBadExpert);
    }
    uint64_t peers = ballot(live);
    for (int bit = 0; bit < id_bits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t ones = ballot(live && set);
      peers &= set ? ones : ~ones;
    }
    int r = 0;
    if (live) {
      const int below = __popcll(peers & lanemask_lt());
      const int base = myhist[e];
      r = base + below;
      if ((peers >> lane) == 1ull) myhist[e] = base + __popcll(peers);  // highest peer
    }
    e_reg[ch] = live ? e : -1;
    r_reg[ch] = r;
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // Combine waves in wave order: hist[w][e] becomes the wave-exclusive prefix.
  for (int e = tid; e < E; e += kPlanThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      const int v = hist[w * E + e];
      hist[w * E + e] = run;
      run += v;
    }
    tile_agg[e] = run;
  }
  __syncthreads();

  // Decoupled look-back across tiles.
  if (b == 0) {
    for (int e = tid; e < E; e += kPlanThreads) inclusive[e] = tile_agg[e];
    __threadfence();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(&flags[0], kFlagInclusive, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    for (int e = tid; e < E; e += kPlanThreads) aggregates[(int64_t)b * E + e] = tile_agg[e];
    __threadfence();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(&flags[b], kFlagAggregate, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);

    // Wave 0 polls a window of up to 64 predecessors at once (lane l: tile
    // hi - l).  The nearest inclusive prefix in the window ends the walk;
    // otherwise the whole window's aggregates are added and the window moves
    // back.  The window's values are summed by all threads in parallel.
    int hi = b - 1;
    while (true) {
      if (wave == 0) {
        const int p = hi - lane;
        uint32_t st = kFlagInclusive;  // before tile 0: an empty prefix
        if (p >= 0) {
          for (int spin = 0; spin < kSpinLimit; ++spin) {
            st = __hip_atomic_load(&flags[p], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            if (st != 0) break;
            __builtin_amdgcn_s_sleep(1);
          }
        }
        const uint64_t incl = ballot(p >= 0 && st == kFlagInclusive);
        const uint64_t none = ballot(p >= 0 && st == 0);
        if (lane == 0) {
          if (none) {
            raise_device_error(kErrPlanStall);
            s_incl = -1; s_lo = 0; s_hi = -1; s_more = 0;
          } else if (incl) {
            const int jn = hi - __builtin_ctzll(incl);   // nearest inclusive prefix
            s_incl = jn; s_lo = jn + 1; s_hi = hi; s_more = 0;
          } else {
            const int lo = hi - (kWave - 1);
            s_incl = -1; s_lo = lo < 0 ? 0 : lo; s_hi = hi; s_more = lo > 0;
          }
        }
      }
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const int lo = s_lo, top = s_hi, jn = s_incl, more = s_more;
      // Rows lo..top of the aggregates, then row jn of the inclusive prefixes.
      const int rows = top - lo + 1 + (jn >= 0 ? 1 : 0);
      const int total = rows * E;
      for (int base = tid; base < total; base += kPlanThreads * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = base + u * kPlanThreads;
          v[u] = 0;
          if (i < total) {
            const int row = i / E, e = i - row * E;
            const int q = lo + row;
            v[u] = q <= top ? aggregates[(int64_t)q * E + e] : inclusive[(int64_t)jn * E + e];
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = base + u * kPlanThreads;
          if (i < total) atomicAdd(&prefix[i % E], v[u]);
        }
      }
      __syncthreads();  // the window variables are rewritten by the next poll
      if (!more) break;
      hi = lo - 1;
    }
    for (int e = tid; e < E; e += kPlanThreads) inclusive[(int64_t)b * E + e] = prefix[e] + tile_agg[e];
    __threadfence();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(&flags[b], kFlagInclusive, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // Partial position: earlier live copies of the same expert over all tiles.
#pragma unroll
  for (int ch = 0; ch < kPlanChunks; ++ch) {
    const int c = cs + ch * kWave + lane;
    if (c < ce) {
      const int e = e_reg[ch];
      pos_partial[c0 + c] = e >= 0 ? prefix[e] + myhist[e] + r_reg[ch] : -1;
    }
  }
}

// Block-wide exclusive scan of n <= 1024 ints held in LDS `a` (in place);
// returns the total.  256 threads, 4 consecutive values per thread.
__device__ int block_exclusive_scan_1024(int32_t* a, int n, int32_t* wave_sums) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  int v[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid * 4 + i;
    v[i] = idx < n ? a[idx] : 0;
    local += v[i];
  }
  // inclusive scan of `local` across the wave
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  int wave_base = 0;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kFinalizeThreads / kWave; ++w) {
    const int ws = wave_sums[w];
    if (w < wave) wave_base += ws;
    total += ws;
  }
  int run = wave_base + incl - local;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid * 4 + i;
    if (idx < n) a[idx] = run;
    run += v[i];
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kFinalizeThreads) void plan_finalize_kernel(
    const int32_t* __restrict__ ids, int64_t n_copies, int K, int E, int W, int Tw,
    int tiles_per_rank, int ntiles, int major_align, int pad_empty, int token_nums_type,
    int64_t* __restrict__ expert_token_nums, const int32_t* __restrict__ aggregates,
    const int32_t* __restrict__ inclusive, uint32_t* flags, uint32_t* ticket,
    int32_t* __restrict__ pos, int32_t* __restrict__ occ, int64_t* __restrict__ in_splits,
    int64_t* __restrict__ src_offsets, int64_t* __restrict__ out_splits,
    int64_t* __restrict__ dst_offsets, int64_t* __restrict__ expert_counts,
    int64_t* __restrict__ expert_offsets, int64_t* __restrict__ rank_offsets) {
  __shared__ int32_t eoff[1024];
  __shared__ int32_t cnt[1024];
  __shared__ int32_t row[1024];
  __shared__ int32_t wave_sums[kFinalizeThreads / kWave];
  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int ne = E / W;
  const int32_t* totals = ntiles > 0 ? inclusive + (int64_t)(ntiles - 1) * E : nullptr;

  for (int e = tid; e < E; e += kFinalizeThreads) {
    const int c = totals ? totals[e] : 0;
    cnt[e] = c;
    eoff[e] = padded_rows(c, major_align, pad_empty);
  }
  __syncthreads();
  const int n_live = block_exclusive_scan_1024(eoff, E, wave_sums);

  if (g < W && expert_token_nums)
    write_expert_token_nums(cnt, g, ne, token_nums_type, expert_token_nums, kFinalizeThreads);
  if (g == 0) {
    for (int e = tid; e < E; e += kFinalizeThreads) {
      expert_counts[e] = cnt[e];
      expert_offsets[e] = eoff[e];
    }
    for (int d = tid; d <= W; d += kFinalizeThreads)
      rank_offsets[d] = d < W ? eoff[d * ne] : n_live;
  }

  if (g < W) {  // rank s = g's rows of the W x E arrays
    const int s = g;
    const int first = s * tiles_per_rank;
    const int last = first + tiles_per_rank - 1;
    for (int e = tid; e < E; e += kFinalizeThreads) {
      int base = 0, cnt = 0;
      if (ntiles > 0) {
        base = inclusive[(int64_t)first * E + e] - (first > 0 ? aggregates[(int64_t)first * E + e]
                                                              : inclusive[e]);
        cnt = inclusive[(int64_t)last * E + e] - base;
      }
      row[e] = cnt;
      in_splits[(int64_t)s * E + e] = cnt;
      out_splits[(int64_t)e * W + s] = cnt;
      dst_offsets[(int64_t)s * E + e] = base + eoff[e] - eoff[(e / ne) * ne];
    }
    __syncthreads();
    block_exclusive_scan_1024(row, E, wave_sums);
    for (int e = tid; e < E; e += kFinalizeThreads) src_offsets[(int64_t)s * E + e] = row[e];
  }

  // Final positions and occurrences.
  const int64_t per_block = (int64_t)kFinalizeThreads * kFinalizeCopiesPerThread;
  const int64_t cbeg = (int64_t)g * per_block;
  for (int64_t c = cbeg + tid; c < n_copies && c < cbeg + per_block; c += kFinalizeThreads) {
    const int p = pos[c];
    if (p >= 0) {
      const int e = ids[c];
      const int s = (int)((c / K) / Tw);
      const int first = s * tiles_per_rank;
      // copies of e before rank s = exclusive prefix of rank s's first tile
      const int before_rank = first > 0 ? inclusive[(int64_t)first * E + e] - aggregates[(int64_t)first * E + e] : 0;
      pos[c] = eoff[e] + p;
      if (occ) occ[c] = p - before_rank;
    } else if (occ) {
      occ[c] = -1;
    }
  }

  if (g == 0) {
    for (int i = tid; i < ntiles; i += kFinalizeThreads) flags[i] = 0;
    if (tid == 0) *ticket = 0;
  }
}

// ---------------------------------------------------------------------------
// Fused single-pass plan for grids whose tiles all fit on the device at
// once.  Each tile ranks its copies as in plan_tile_kernel, then publishes
// its per-expert counts as 64-bit
// descriptors (call epoch << 32 | count) with relaxed device-scope atomic
// stores: a descriptor carries its own validity, so no cache write-back or
// invalidate is needed between publishing and reading.  Every tile then reads
// all tiles' descriptors (polling each until it carries this call's epoch)
// and derives, per expert, the copies in earlier tiles, the totals, and the
// copies before its source rank; the final positions and occurrences follow
// directly from the ranks still held in registers.  Workgroup s < W also
// writes rank s's rows of the W x E plan arrays.
// ---------------------------------------------------------------------------
constexpr int kFusedMaxDescriptorsPerTile = 1 << 16;  // ntiles * E read by every tile
constexpr int kDescBatch = 16;                         // descriptor loads in flight per thread
// Workspace header words (u32): the look-back ticket, the fused kernel's
// epoch and its count of tiles done reading.
constexpr int kHeaderTicket = 0;
constexpr int kHeaderEpoch = 1;
constexpr int kHeaderDone = 2;

// Polls a descriptor until it carries `epoch`.  The wait is bounded per
// thread, over all of its waits together (`budget` polls), and per tile: the
// first thread that runs out of polls raises EP_DEVERR_PLAN_STALL and sets the
// tile's LDS flag `stalled`, after which every wait of the tile returns at
// once.  A tile therefore gives up within one budget in all, however many
// descriptors are missing; its counts then read as 0 and the plan is invalid.
__device__ __forceinline__ uint64_t wait_descriptor(const uint64_t* d, uint32_t epoch, int& budget,
                                                    int* stalled) {
  uint64_t v = __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while ((uint32_t)(v >> 32) != epoch) {
    if (budget <= 0 || __hip_atomic_load(stalled, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
      if (__hip_atomic_exchange(stalled, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
        raise_device_error(kErrPlanStall);
      return 0;
    }
    --budget;
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return v & 0xffffffffull;
}

// Block-wide exclusive scan of n <= 1024 ints in LDS `a` (in place) for a
// 512-thread block, 2 consecutive values per thread; returns the total.
__device__ int block_exclusive_scan_512(int32_t* a, int n, int32_t* wave_sums) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int i0 = tid * 2;
  const int v0 = i0 < n ? a[i0] : 0;
  const int v1 = i0 + 1 < n ? a[i0 + 1] : 0;
  const int local = v0 + v1;
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int ws = wave_sums[w];
    if (w < wave) base += ws;
    total += ws;
  }
  const int ex = base + incl - local;
  if (i0 < n) a[i0] = ex;
  if (i0 + 1 < n) a[i0 + 1] = ex + v0;
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kPlanThreads) void plan_fused_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ active,
    const uint8_t* __restrict__ active_copies, int K, int E, int W, int Tw, int tile_tokens,
    int tiles_per_rank, int ntiles, int id_bits, int major_align, int pad_empty,
    int token_nums_type, int64_t* __restrict__ expert_token_nums, uint32_t* header,
    uint64_t* desc, int32_t* __restrict__ pos, int32_t* __restrict__ occ,
    int64_t* __restrict__ in_splits, int64_t* __restrict__ src_offsets,
    int64_t* __restrict__ out_splits, int64_t* __restrict__ dst_offsets,
    int64_t* __restrict__ expert_counts, int64_t* __restrict__ expert_offsets,
    int64_t* __restrict__ rank_offsets, int spin_limit, int withhold_tile) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                       // [kPlanWaves][E]
  int32_t* tot = hist + kPlanWaves * E;      // [E] all tiles -> expert offsets
  int32_t* pre = tot + E;                    // [E] tiles before this one
  int32_t* rbase = pre + E;                  // [E] tiles before this tile's rank
  int32_t* rin = rbase + E;                  // [E] tiles of rank blockIdx.x (if < W)
  int32_t* rbg = rin + E;                    // [E] tiles before rank blockIdx.x
  int32_t* cnt = rbg + E;                    // [E] true totals (tot is padded, then scanned)
  __shared__ int32_t wave_sums[kPlanWaves];
  __shared__ int s_stalled;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int b = blockIdx.x;
  if (tid == 0) s_stalled = 0;  // read only after the barrier below
  // This launch's descriptor tag: one more than the launches completed on
  // this workspace (kept in the workspace, so replays of a captured graph
  // get fresh tags too; 0 never tags a descriptor).
  const uint32_t epoch =
      __hip_atomic_load(&header[kHeaderEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  for (int i = tid; i < (kPlanWaves + 6) * E; i += kPlanThreads) lds[i] = 0;

  const int s = b / tiles_per_rank;
  const int j = b - s * tiles_per_rank;
  const int64_t t0 = (int64_t)s * Tw + (int64_t)j * tile_tokens;
  int64_t t1 = t0 + tile_tokens;
  if (t1 > (int64_t)(s + 1) * Tw) t1 = (int64_t)(s + 1) * Tw;
  const int64_t c0 = t0 * K;
  const int n = (int)((t1 - t0) * K);
  const int seg = (n + kPlanWaves - 1) / kPlanWaves;
  const int cs = wave * seg;
  const int ce = min(cs + seg, n);

  // All loads of the tile's ids and mask bytes go out together: the mask
  // bytes are combined after the barrier (a short-circuit test here would
  // wait for each byte before issuing the next load).
  int e_reg[kPlanChunks];
  uint32_t a_reg[kPlanChunks], ac_reg[kPlanChunks];
#pragma unroll
  for (int ch = 0; ch < kPlanChunks; ++ch) {
    const int c = cs + ch * kWave + lane;
    e_reg[ch] = -1;
    a_reg[ch] = 0;
    ac_reg[ch] = 1;
    if (c < ce) {
      const int64_t gc = c0 + c;
      e_reg[ch] = ids[gc];
      a_reg[ch] = active ? active[gc / K] : 1u;
      if (active_copies) ac_reg[ch] = active_copies[gc];
    }
  }
  __syncthreads();  // LDS zeroed
  bool act_reg[kPlanChunks];
#pragma unroll
  for (int ch = 0; ch < kPlanChunks; ++ch) act_reg[ch] = a_reg[ch] != 0 && ac_reg[ch] != 0;

  int32_t* myhist = hist + wave * E;
  int r_reg[kPlanChunks];
#pragma unroll
  for (int ch = 0; ch < kPlanChunks; ++ch) {
    const int e = e_reg[ch];
    bool live = false;
    if (act_reg[ch]) {
      live = (unsigned)e < (unsigned)E;
      if (!live) raise_device_error(kErrBadExpert);
    }
    uint64_t peers = ballot(live);
    for (int bit = 0; bit < id_bits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t ones = ballot(live && set);
      peers &= set ? ones : ~ones;
    }
    int r = 0;
    if (live) {
      const int below = __popcll(peers & lanemask_lt());
      const int base = myhist[e];
      r = base + below;
      if ((peers >> lane) == 1ull) myhist[e] = base + __popcll(peers);
    }
    e_reg[ch] = live ? e : -1;
    r_reg[ch] = r;
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // Wave-exclusive prefixes and this tile's counts, published at once.
  for (int e = tid; e < E; e += kPlanThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      const int v = hist[w * E + e];
      hist[w * E + e] = run;
      run += v;
    }
    if (b != withhold_tile)  // withhold_tile >= 0 only to test the stall path
      __hip_atomic_store(&desc[(int64_t)b * E + e], ((uint64_t)epoch << 32) | (uint32_t)run,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Read every tile's counts.  Thread (e, h) sums tiles p = h, h + tpe, ...
  // for expert e in registers (tpe threads per expert), E > 512 gives a
  // thread two experts.
  const int g = b;  // this workgroup also writes rank g's plan rows when g < W
  const int first_s = s * tiles_per_rank;
  const int first_g = g * tiles_per_rank, last_g = first_g + tiles_per_rank - 1;
  const int tpe = E >= kPlanThreads ? 1 : kPlanThreads / E;
  const int n_exp = E > kPlanThreads ? 2 : 1;
  int budget = spin_limit;
  if (tid < tpe * E || E > kPlanThreads) {
    for (int xe = 0; xe < n_exp; ++xe) {
      const int e = E > kPlanThreads ? tid + xe * kPlanThreads : tid % E;
      const int h = E >= kPlanThreads ? 0 : tid / E;
      if (e >= E) continue;
      int a_tot = 0, a_pre = 0, a_rbase = 0, a_rin = 0, a_rbg = 0;
      for (int p0 = h; p0 < ntiles; p0 += tpe * kDescBatch) {
        uint64_t raw[kDescBatch];
#pragma unroll
        for (int u = 0; u < kDescBatch; ++u) {
          const int p = p0 + u * tpe;
          raw[u] = p < ntiles ? __hip_atomic_load(&desc[(int64_t)p * E + e], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                              : ((uint64_t)epoch << 32);
        }
#pragma unroll
        for (int u = 0; u < kDescBatch; ++u) {
          const int p = p0 + u * tpe;
          if (p >= ntiles) continue;
          int v = (uint32_t)(raw[u] >> 32) == epoch ? (int)(raw[u] & 0xffffffffull)
                                                     : (int)wait_descriptor(&desc[(int64_t)p * E + e], epoch, budget, &s_stalled);
          a_tot += v;
          if (p < b) a_pre += v;
          if (p < first_s) a_rbase += v;
          if (p >= first_g && p <= last_g) a_rin += v;
          if (p < first_g) a_rbg += v;
        }
      }
      if (tpe == 1) {
        tot[e] = a_tot; pre[e] = a_pre; rbase[e] = a_rbase; rin[e] = a_rin; rbg[e] = a_rbg;
      } else {
        atomicAdd(&tot[e], a_tot);
        atomicAdd(&pre[e], a_pre);
        atomicAdd(&rbase[e], a_rbase);
        atomicAdd(&rin[e], a_rin);
        atomicAdd(&rbg[e], a_rbg);
      }
    }
  }
  __syncthreads();
  // The last tile to finish reading advances the workspace's epoch; every
  // tile read it at its start, before any tile could finish reading.  The
  // counter's old value is only looked at when the tile's work is done, so
  // its round trip overlaps the rest of the kernel.
  uint32_t done = 0;
  if (tid == 0)
    done = __hip_atomic_fetch_add(&header[kHeaderDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // Final positions and occurrences of this tile's copies.
  int32_t* eoff = tot;  // padded, then scanned in place; true totals kept in cnt
  for (int e = tid; e < E; e += kPlanThreads) {
    cnt[e] = tot[e];
    tot[e] = padded_rows(tot[e], major_align, pad_empty);
    if (g == 0) expert_counts[e] = cnt[e];
  }
  __syncthreads();
  const int n_live = block_exclusive_scan_512(eoff, E, wave_sums);
  if (g < W && expert_token_nums)
    write_expert_token_nums(cnt, g, E / W, token_nums_type, expert_token_nums, kPlanThreads);
#pragma unroll
  for (int ch = 0; ch < kPlanChunks; ++ch) {
    const int c = cs + ch * kWave + lane;
    if (c < ce) {
      const int e = e_reg[ch];
      int p = -1, o = -1;
      if (e >= 0) {
        const int within = pre[e] + myhist[e] + r_reg[ch];  // earlier copies of e, all tiles
        p = eoff[e] + within;
        o = within - rbase[e];
      }
      pos[c0 + c] = p;
      if (occ) occ[c0 + c] = o;
    }
  }

  if (g == 0) {
    for (int e = tid; e < E; e += kPlanThreads) expert_offsets[e] = eoff[e];
    const int ne = E / W;
    for (int d = tid; d <= W; d += kPlanThreads) rank_offsets[d] = d < W ? eoff[d * ne] : n_live;
  }
  if (g < W) {
    const int ne = E / W;
    for (int e = tid; e < E; e += kPlanThreads) {
      const int cnt = rin[e];
      in_splits[(int64_t)g * E + e] = cnt;
      out_splits[(int64_t)e * W + g] = cnt;
      dst_offsets[(int64_t)g * E + e] = rbg[e] + eoff[e] - eoff[(e / ne) * ne];
    }
    __syncthreads();
    block_exclusive_scan_512(rin, E, wave_sums);
    for (int e = tid; e < E; e += kPlanThreads) src_offsets[(int64_t)g * E + e] = rin[e];
  }
  if (tid == 0 && done == (uint32_t)ntiles - 1u) {
    __hip_atomic_store(&header[kHeaderDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&header[kHeaderEpoch], epoch == 0xffffffffu ? 0u : epoch, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace ep
