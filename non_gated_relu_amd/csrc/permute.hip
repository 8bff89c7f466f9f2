// permute.hip -- stable grouping of routing slots by expert, tile schedules,
// the optional row gather, and the weighted combine.
//
// The experts are applied as one stacked weight tensor per projection indexed
// by the routing result (exo commit "Add support for Nemotron sharding",
// typing stubs SwitchMLP.fc1 / fc2 and SwitchGLU.__call__(x, indices)); the
// GEMMs want the rows of one expert contiguous, so slots s = t*k + j are
// grouped by expert with a histogram, an exclusive scan and a stable
// placement (slot ids ascend inside an expert).  No atomics decide an order:
// LDS integer atomics only count, and ranks inside a wave come from ballots.
#include "select.hpp"

namespace moe {

namespace {

constexpr int PM_THREADS = 256;
constexpr int PM_WAVES = PM_THREADS / WAVE;

// Lanes of this wave holding the same key (keys < 2^9, one extra bit marks
// validity), found with one ballot per key bit.
__device__ __forceinline__ uint64_t match_key(uint32_t key) {
  uint64_t m = ~uint64_t(0);
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    uint64_t bb = ballot((key >> b) & 1u);
    m &= ((key >> b) & 1u) ? bb : ~bb;
  }
  return m;
}

// Copies the expert ids of slots [s0, s0 + n), n <= MAXN, into LDS.  All
// loads are issued before the first store, so the chunk costs one memory
// round trip.  Ids outside [0, E) are clamped so every later write stays
// inside its array.  Ends with a barrier.
template <int MAXN>
__device__ void stage_ids(const int32_t* __restrict__ idx, int64_t s0, int n, int E,
                          int32_t* ids) {
  constexpr int PER = MAXN / PM_THREADS;
  int32_t v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = threadIdx.x + i * PM_THREADS;
    v[i] = q < n ? idx[s0 + q] : 0;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = threadIdx.x + i * PM_THREADS;
    if (q < n) ids[q] = min(max(v[i], 0), E - 1);
  }
  __syncthreads();
}

// Place the slots [s_begin, s_begin + n) in order; ids[i] is the expert of
// slot s_begin + i.  run[e] holds the next free position of expert e and is
// advanced; wc is a zeroed [PM_WAVES][E] scratch.
__device__ void place_chunk(const int32_t* ids, int64_t s_begin, int n, int E, int32_t* run,
                            int32_t* wc, int32_t* __restrict__ sorted_slot,
                            int32_t* __restrict__ slot_pos) {
  const int wave = threadIdx.x / WAVE;
  for (int r0 = 0; r0 < n; r0 += PM_THREADS) {
    const int i = r0 + threadIdx.x;
    const bool valid = i < n;
    const int64_t s = s_begin + i;
    const int e = valid ? ids[i] : 0;
    const uint32_t key = valid ? (uint32_t(e) | 0x200u) : 0u;
    const uint64_t m = match_key(key);
    const int rank = __popcll(m & lanemask_lt());
    if (valid && rank == 0) wc[wave * E + e] = __popcll(m);
    __syncthreads();
    int pos = 0;
    if (valid) {
      pos = run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wc[w * E + e];
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += PM_THREADS) {
      int add = 0;
      for (int w = 0; w < PM_WAVES; ++w) {
        add += wc[w * E + x];
        wc[w * E + x] = 0;
      }
      run[x] += add;
    }
    if (valid) {
      sorted_slot[pos] = static_cast<int32_t>(s);
      slot_pos[s] = pos;
    }
    __syncthreads();
  }
}

// Exclusive scan of n <= PM_THREADS * 4 values held in LDS `v` (in place);
// returns the total.  All threads must call.  Each thread owns 4 consecutive
// entries; a wave scans its threads' sums with shuffles, and the waves'
// totals are added through LDS (two barriers in all).
__device__ int32_t block_exclusive_scan(int32_t* v, int n, int32_t* tmp) {
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / WAVE;
  int32_t loc[4];
  int32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = t * 4 + i;
    loc[i] = j < n ? v[j] : 0;
    sum += loc[i];
  }
  int32_t incl = sum;  // inclusive scan of the sums over the wave's lanes
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const int32_t up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  if (lane == WAVE - 1) tmp[wave] = incl;
  __syncthreads();
  int32_t run = incl - sum;
  int32_t total = 0;
#pragma unroll
  for (int w = 0; w < PM_WAVES; ++w) {
    const int32_t wt = tmp[w];
    if (w < wave) run += wt;
    total += wt;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = t * 4 + i;
    if (j < n) v[j] = run;
    run += loc[i];
  }
  __syncthreads();
  return total;
}

// M-tile schedule of a grouped GEMM (layout in internal.hpp): group g covers
// the rows range(g) = [a, b); tiles of `bm` rows, groups in order, then the
// optional extra group.  All threads must call; tiles/tmp are LDS scratch.
// After the scan of the groups' tile counts, each thread writes whole tiles:
// tile j belongs to the last group whose first tile is at or before j
// (groups without tiles share their successor's first tile), found by a
// binary search, so a group with many tiles costs no thread more than others.
template <typename Range>
__device__ void emit_schedule(Range range, int n_groups, const ScheduleSpec& sp, int32_t* tiles,
                              int32_t* tmp, int32_t* carry) {
  if (threadIdx.x == 0) *carry = 0;
  __syncthreads();
  for (int g0 = 0; g0 < n_groups; g0 += 1024) {
    const int n = min(1024, n_groups - g0);
    for (int i = threadIdx.x; i < n; i += PM_THREADS) {
      int64_t a, b;
      range(g0 + i, a, b);
      tiles[i] = b > a ? static_cast<int32_t>((b - a + sp.bm - 1) / sp.bm) : 0;
    }
    __syncthreads();
    const int32_t total = block_exclusive_scan(tiles, n, tmp);
    const int32_t base = *carry;
    for (int32_t j = threadIdx.x; j < total; j += PM_THREADS) {
      int lo = 0, hi = n - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tiles[mid] <= j)
          lo = mid;
        else
          hi = mid - 1;
      }
      int64_t a, b;
      range(g0 + lo, a, b);
      const int32_t at = base + j;
      if (at < sp.max_tiles) {
        const int64_t m = a + int64_t(j - tiles[lo]) * sp.bm;
        const int32_t rows = static_cast<int32_t>(min<int64_t>(sp.bm, b - m));
        sp.sched[2 + 2 * at] = (g0 + lo) | (rows << 16);
        sp.sched[3 + 2 * at] = static_cast<int32_t>(m);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) *carry += total;
    __syncthreads();
  }
  const int32_t extra =
      sp.extra_rows > 0 ? static_cast<int32_t>((sp.extra_rows + sp.bm - 1) / sp.bm) : 0;
  for (int j = threadIdx.x; j < extra; j += PM_THREADS) {
    const int32_t at = *carry + j;
    if (at < sp.max_tiles) {
      const int32_t rows = static_cast<int32_t>(min<int64_t>(sp.bm, sp.extra_rows - int64_t(j) * sp.bm));
      sp.sched[2 + 2 * at] = n_groups | (rows << 16);
      sp.sched[3 + 2 * at] = j * sp.bm;
    }
  }
  if (threadIdx.x == 0) {
    sp.sched[0] = min(*carry + extra, sp.max_tiles);
    sp.sched[1] = min(*carry, sp.max_tiles);
  }
  __syncthreads();
}

// Small problems (all slots in one workgroup): histogram, scan, schedule,
// placement.
__device__ __forceinline__ void permute_small(const PermuteArgs& p) {
  __shared__ int32_t cnt[1024];
  __shared__ int32_t run[1024];
  __shared__ int32_t tiles[1024];
  __shared__ int32_t wc[PM_WAVES * 256];
  __shared__ int32_t tmp[PM_THREADS];
  __shared__ int32_t carry;
  const int E = p.n_experts;
  __shared__ int32_t ids[PM_SMALL_MAX];
  const int n = static_cast<int>(p.slots);
  for (int e = threadIdx.x; e < E; e += PM_THREADS) cnt[e] = 0;
  for (int i = threadIdx.x; i < PM_WAVES * E; i += PM_THREADS) wc[i] = 0;
  stage_ids<PM_SMALL_MAX>(p.topk_idx, 0, n, E, ids);
  for (int i = threadIdx.x; i < n; i += PM_THREADS) atomicAdd(&cnt[ids[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PM_THREADS) {
    run[e] = cnt[e];
    p.expert_counts[e] = cnt[e];
  }
  __syncthreads();
  block_exclusive_scan(run, E, tmp);
  for (int e = threadIdx.x; e < E; e += PM_THREADS) p.expert_offsets[e] = run[e];
  if (threadIdx.x == 0) p.expert_offsets[E] = n;
  __syncthreads();
  if (p.sched.sched)
    emit_schedule(
        [&](int g, int64_t& a, int64_t& b) {
          a = run[g];
          b = run[g] + cnt[g];
        },
        E, p.sched, tiles, tmp, &carry);
  place_chunk(ids, 0, n, E, run, wc, p.sorted_slot, p.slot_pos);
}

// The same outputs from one wave, for at most 64 slots (one per lane) and
// 256 experts, without a workgroup barrier: a lane's slot finds the slots of
// its expert with ballots (match_key), the first of them scatters the count,
// and the experts' counts, offsets and tile counts are scanned across the
// wave with shuffles, expert x = lane + 64 j in ascending order.
constexpr int PW_MAX_SLOTS = WAVE;
__device__ void permute_wave(const PermuteArgs& p) {
  __shared__ int32_t cnt[RT_MAXE];
  __shared__ int32_t off[RT_MAXE];
  const int lane = lane_id();
  const int E = p.n_experts;
  const int S = static_cast<int>(p.slots);
  const bool valid = lane < S;
  const int e = valid ? min(max(p.topk_idx[lane], 0), E - 1) : 0;
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j)
    if (lane + WAVE * j < E) cnt[lane + WAVE * j] = 0;
  const uint64_t m = match_key(valid ? (uint32_t(e) | 0x200u) : 0u);
  const int rank = __popcll(m & lanemask_lt());
  wave_lds_sync();
  if (valid && rank == 0) cnt[e] = __popcll(m);
  wave_lds_sync();
  // per expert: count, exclusive offset, tile count and first tile
  const ScheduleSpec& sp = p.sched;
  int32_t c[RT_EPL], o[RT_EPL], nt[RT_EPL], t0[RT_EPL];
  int32_t carry = 0, tcarry = 0;
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    const int x = lane + WAVE * j;
    c[j] = x < E ? cnt[x] : 0;
    nt[j] = c[j] > 0 && sp.sched ? (c[j] + sp.bm - 1) / sp.bm : 0;
    int32_t ic = c[j], it = nt[j];  // inclusive scans over the wave's lanes
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
      const int32_t uc = __shfl_up(ic, d), ut = __shfl_up(it, d);
      if (lane >= d) {
        ic += uc;
        it += ut;
      }
    }
    o[j] = carry + ic - c[j];
    t0[j] = tcarry + it - nt[j];
    carry += __shfl(ic, WAVE - 1);
    tcarry += __shfl(it, WAVE - 1);
    if (x < E) {
      p.expert_counts[x] = c[j];
      p.expert_offsets[x] = o[j];
      off[x] = o[j];
    }
  }
  if (lane == 0) p.expert_offsets[E] = S;
  wave_lds_sync();
  if (valid) {
    const int pos = off[e] + rank;
    p.sorted_slot[pos] = lane;
    p.slot_pos[lane] = pos;
  }
  if (!sp.sched) return;
  // the schedule: each expert's tiles, groups in order, then the extra group
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    const int x = lane + WAVE * j;
    for (int q = 0; q < nt[j]; ++q) {
      const int32_t at = t0[j] + q;
      if (at < sp.max_tiles) {
        sp.sched[2 + 2 * at] = x | (min(sp.bm, c[j] - q * sp.bm) << 16);
        sp.sched[3 + 2 * at] = o[j] + q * sp.bm;
      }
    }
  }
  const int32_t extra =
      sp.extra_rows > 0 ? static_cast<int32_t>((sp.extra_rows + sp.bm - 1) / sp.bm) : 0;
  for (int q = lane; q < extra; q += WAVE) {
    const int32_t at = tcarry + q;
    if (at < sp.max_tiles) {
      const int32_t rows = static_cast<int32_t>(min<int64_t>(sp.bm, sp.extra_rows - int64_t(q) * sp.bm));
      sp.sched[2 + 2 * at] = E | (rows << 16);
      sp.sched[3 + 2 * at] = q * sp.bm;
    }
  }
  if (lane == 0) {
    sp.sched[0] = min(tcarry + extra, sp.max_tiles);
    sp.sched[1] = min(tcarry, sp.max_tiles);
  }
}

__global__ __launch_bounds__(PM_THREADS) void permute_small_kernel(PermuteArgs p) {
  permute_small(p);
}

// Decode-sized calls: the grouped top-k of every token from its logits (16
// waves, each taking tokens w, w + 16, ...) and then the permute of their
// slots, in one launch.  The selection is route.hip's, so the routing is the
// same; the barrier makes each wave's topk_idx visible to the permute, which
// runs on the first PM_THREADS threads while the other waves end (a barrier
// waits only for the waves of the workgroup that have not ended).
constexpr int SP_THREADS = 1024;
constexpr int SP_WAVES = SP_THREADS / WAVE;
static_assert(SP_THREADS >= RT_MAXE, "one thread per expert stages the bias");
__global__ __launch_bounds__(SP_THREADS) void select_permute_kernel(RouteArgs r, PermuteArgs p) {
  __shared__ f32x4_t lds_l[SP_MAX_LOGITS / 4];
  __shared__ float lds_b[RT_MAXE];
  __shared__ SelScratch scr[SP_WAVES];
  // every token's logits and the correction bias into LDS, all loads in
  // flight together
  const int n4 = static_cast<int>(r.tokens) * r.n_experts / 4;
  constexpr int PER = SP_MAX_LOGITS / 4 / SP_THREADS;
  f32x4_t v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = u * SP_THREADS + threadIdx.x;
    if (i < n4) v[u] = reinterpret_cast<const f32x4_t*>(r.logits)[i];
  }
  const float bias = threadIdx.x < r.n_experts ? r.e_bias[threadIdx.x] : 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = u * SP_THREADS + threadIdx.x;
    if (i < n4) lds_l[i] = v[u];
  }
  if (threadIdx.x < r.n_experts) lds_b[threadIdx.x] = bias;
  __syncthreads();
  const int wave = threadIdx.x / WAVE;
  const float* logits = reinterpret_cast<const float*>(lds_l);
  for (int64_t t = wave; t < r.tokens; t += SP_WAVES)
    select_one(r, logits + t * r.n_experts, t, scr[wave], lds_b);
  __syncthreads();
  if (p.slots <= PW_MAX_SLOTS) {  // (E <= RT_MAXE here)
    if (threadIdx.x >= WAVE) return;
    permute_wave(p);
    return;
  }
  if (threadIdx.x >= PM_THREADS) return;
  permute_small(p);
}

// Large problems, pass 1: per-chunk expert histogram.
__global__ __launch_bounds__(PM_THREADS) void permute_hist_kernel(PermuteArgs p) {
  __shared__ int32_t cnt[256];
  __shared__ int32_t ids[PM_CHUNK];
  const int E = p.n_experts;
  for (int e = threadIdx.x; e < E; e += PM_THREADS) cnt[e] = 0;
  const int64_t s0 = int64_t(blockIdx.x) * PM_CHUNK;
  const int n = static_cast<int>(min<int64_t>(PM_CHUNK, p.slots - s0));
  stage_ids<PM_CHUNK>(p.topk_idx, s0, n, E, ids);
  for (int i = threadIdx.x; i < n; i += PM_THREADS) atomicAdd(&cnt[ids[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PM_THREADS) p.block_counts[blockIdx.x * E + e] = cnt[e];
}

// Pass 2 (one workgroup): per-expert totals, offsets, each chunk's base, and
// the GEMM schedule.  H = PM_THREADS / E threads share an expert's column of
// chunk counts, each owning a run of consecutive chunks.  When a run fits in
// registers (at most PM_SCAN_REG chunks) a thread issues the loads of its
// whole run before using any (coalesced: the threads of one run index are
// consecutive experts),
// scans it in registers, and writes each chunk's final base once the runs'
// totals and the expert offsets are known.  Otherwise each expert's column
// is walked in global memory.
constexpr int PM_SCAN_REG = 48;  // loads in flight per thread (vmcnt counts to 63)
__global__ __launch_bounds__(PM_THREADS) void permute_scan_kernel(PermuteArgs p) {
  __shared__ int32_t off[1024];
  __shared__ int32_t cnt[1024];
  __shared__ int32_t tiles[1024];
  __shared__ int32_t tmp[PM_THREADS];
  __shared__ int32_t run_total[PM_THREADS];
  __shared__ int32_t carry;
  const int E = p.n_experts;
  const int H = E <= PM_THREADS ? PM_THREADS / E : 1;  // threads per expert column
  const int per = (p.n_chunks + H - 1) / H;            // chunks per run
  const bool in_reg = E <= PM_THREADS && per <= PM_SCAN_REG;
  const int e = threadIdx.x % E;
  const int h = threadIdx.x / E;  // run h of expert e's column (none when h >= H)
  const int b0 = h * per;
  const int nrun = h < H ? max(min(per, p.n_chunks - b0), 0) : 0;  // chunks in this run
  int32_t v[PM_SCAN_REG];
  int32_t before = 0;  // the counts of expert e in chunks before this run
  if (in_reg) {
    // every load is issued (from a clamped, valid chunk) before the first use
    const int last = p.n_chunks - 1;
#pragma unroll
    for (int u = 0; u < PM_SCAN_REG; ++u) v[u] = p.block_counts[min(b0 + u, last) * E + e];
#pragma unroll
    for (int u = 0; u < PM_SCAN_REG; ++u) v[u] = u < nrun ? v[u] : 0;
    int32_t total = 0;
#pragma unroll
    for (int u = 0; u < PM_SCAN_REG; ++u) {
      const int32_t c = v[u];
      v[u] = total;  // the chunk's base inside its run
      total += c;
    }
    if (h < H) run_total[h * E + e] = total;
    __syncthreads();
    if (h < H) {
      for (int j = 0; j < h; ++j) before += run_total[j * E + e];
      if (h == H - 1) {
        const int32_t all = before + total;
        p.expert_counts[e] = all;
        off[e] = all;
        cnt[e] = all;
      }
    }
  } else {
    constexpr int B = 8;  // chunk counts loaded per batch
    for (int x = threadIdx.x; x < E; x += PM_THREADS) {
      int32_t total = 0;
      for (int c0 = 0; c0 < p.n_chunks; c0 += B) {
        int32_t w[B];
#pragma unroll
        for (int u = 0; u < B; ++u)
          w[u] = c0 + u < p.n_chunks ? p.block_counts[(c0 + u) * E + x] : 0;
#pragma unroll
        for (int u = 0; u < B; ++u) {
          if (c0 + u < p.n_chunks) {
            p.block_counts[(c0 + u) * E + x] = total;
            total += w[u];
          }
        }
      }
      p.expert_counts[x] = total;
      off[x] = total;
      cnt[x] = total;
    }
  }
  __syncthreads();
  block_exclusive_scan(off, E, tmp);
  for (int x = threadIdx.x; x < E; x += PM_THREADS) p.expert_offsets[x] = off[x];
  if (in_reg) {
    const int32_t base = before + off[e];
#pragma unroll
    for (int u = 0; u < PM_SCAN_REG; ++u)
      if (u < nrun) p.block_counts[(b0 + u) * E + e] = v[u] + base;
  } else {
    for (int x = threadIdx.x; x < E; x += PM_THREADS)
      for (int b = 0; b < p.n_chunks; ++b) p.block_counts[b * E + x] += off[x];
  }
  if (threadIdx.x == 0) p.expert_offsets[E] = static_cast<int32_t>(p.slots);
  if (p.sched.sched)
    emit_schedule(
        [&](int g, int64_t& a, int64_t& b) {
          a = off[g];
          b = off[g] + cnt[g];
        },
        E, p.sched, tiles, tmp, &carry);
}

// Pass 3: stable placement of each chunk from its base.
__global__ __launch_bounds__(PM_THREADS) void permute_place_kernel(PermuteArgs p) {
  __shared__ int32_t run[256];
  __shared__ int32_t wc[PM_WAVES * 256];
  __shared__ int32_t ids[PM_CHUNK];
  const int E = p.n_experts;
  for (int e = threadIdx.x; e < E; e += PM_THREADS) run[e] = p.block_counts[blockIdx.x * E + e];
  for (int i = threadIdx.x; i < PM_WAVES * E; i += PM_THREADS) wc[i] = 0;
  const int64_t s0 = int64_t(blockIdx.x) * PM_CHUNK;
  const int n = static_cast<int>(min<int64_t>(PM_CHUNK, p.slots - s0));
  stage_ids<PM_CHUNK>(p.topk_idx, s0, n, E, ids);
  place_chunk(ids, s0, n, E, run, wc, p.sorted_slot, p.slot_pos);
}

// x_perm[r] = x[sorted_slot[r] / k], 16 bytes per lane.
__global__ __launch_bounds__(PM_THREADS) void gather_rows_kernel(GatherArgs p) {
  const int chunks = p.row_bytes / 16;
  const int64_t total = p.rows * chunks;
  for (int64_t i = int64_t(blockIdx.x) * PM_THREADS + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * PM_THREADS) {
    const int64_t r = i / chunks;
    const int c = static_cast<int>(i - r * chunks);
    const int64_t src = p.sorted_slot[r] / p.div;
    const i32x4_t v = *reinterpret_cast<const i32x4_t*>(
        static_cast<const char*>(p.src) + src * p.row_bytes + c * 16);
    *reinterpret_cast<i32x4_t*>(static_cast<char*>(p.dst) + r * p.row_bytes + c * 16) = v;
  }
}

// Schedule of a grouped GEMM from group offsets in global memory.
__global__ __launch_bounds__(PM_THREADS) void schedule_kernel(ScheduleArgs p) {
  __shared__ int32_t tiles[1024];
  __shared__ int32_t tmp[PM_THREADS];
  __shared__ int32_t carry;
  emit_schedule(
      [&](int g, int64_t& a, int64_t& b) {
        // no offsets: a single group spans every row
        a = p.offsets ? min<int64_t>(max(p.offsets[g], 0), p.rows) : 0;
        b = p.offsets ? min<int64_t>(max(p.offsets[g + 1], 0), p.rows) : p.rows;
      },
      p.n_groups, p.spec, tiles, tmp, &carry);
}

// y[t] = sum_j w[t,j] * y_perm[slot_pos[t*k+j]] (+ shared[t]) (+ residual[t]),
// fp32, rounded once.  y may alias the residual: a thread reads its own
// elements before writing them.
template <bool BF16_OUT>
__global__ __launch_bounds__(PM_THREADS) void combine_kernel(CombineArgs p) {
  // one float4 of one token per thread, over a flat grid of tokens x columns
  const int d4 = p.hidden / 4;
  const int64_t idx = int64_t(blockIdx.x) * PM_THREADS + threadIdx.x;
  const int64_t t = idx / d4;
  if (t >= p.tokens) return;
  const int c = static_cast<int>(idx - t * d4);
  const int k = p.top_k;
  const int32_t* pos = p.slot_pos + t * k;
  const float* wt = p.topk_w + t * k;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // the (read-once) rows of up to 8 slots are fetched together, then summed
  // in ascending j
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4_t v[8];
    float w[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj < k) {
        w[jj] = wt[j0 + jj];
        v[jj] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t*>(p.y_perm + int64_t(pos[j0 + jj]) * p.hidden) + c);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj < k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(w[jj], v[jj][q], acc[q]);
      }
    }
  }
  if (p.shared) {
    const f32x4_t sv =
        __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p.shared + t * p.hidden) + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = acc[q] + sv[q];
  }
  if (p.residual) {  // the block's residual stream, added before the one rounding
    if (BF16_OUT) {
      const uint2 rv =
          reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.residual) + t * p.hidden)[c];
      acc[0] = acc[0] + __uint_as_float(rv.x << 16);
      acc[1] = acc[1] + __uint_as_float(rv.x & 0xFFFF0000u);
      acc[2] = acc[2] + __uint_as_float(rv.y << 16);
      acc[3] = acc[3] + __uint_as_float(rv.y & 0xFFFF0000u);
    } else {
      const f32x4_t rv =
          reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p.residual) + t * p.hidden)[c];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = acc[q] + rv[q];
    }
  }
  if (BF16_OUT) {
    uint32_t lo = pack_bf16x2(acc[0], acc[1]);
    uint32_t hi = pack_bf16x2(acc[2], acc[3]);
    reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + t * p.hidden)[c] = make_uint2(lo, hi);
  } else {
    reinterpret_cast<f32x4_t*>(static_cast<float*>(p.y) + t * p.hidden)[c] = acc;
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& p, hipStream_t stream, Timing t) {
  if (p.n_chunks <= 1)
    return launch_k(permute_small_kernel, dim3(1), dim3(PM_THREADS), stream, t, p);
  hipError_t e;
  if ((e = launch_k(permute_hist_kernel, dim3(p.n_chunks), dim3(PM_THREADS), stream,
                    Timing{t.start, nullptr}, p)) != hipSuccess)
    return e;
  if ((e = launch_k(permute_scan_kernel, dim3(1), dim3(PM_THREADS), stream, Timing{}, p)) !=
      hipSuccess)
    return e;
  return launch_k(permute_place_kernel, dim3(p.n_chunks), dim3(PM_THREADS), stream,
                  Timing{nullptr, t.stop}, p);
}

hipError_t launch_select_permute(const RouteArgs& r, const PermuteArgs& p, hipStream_t stream,
                                 Timing t) {
  if (p.slots <= 0) return hipSuccess;
  return launch_k(select_permute_kernel, dim3(1), dim3(SP_THREADS), stream, t, r, p);
}

hipError_t launch_gather(const GatherArgs& p, hipStream_t stream) {
  const int64_t total = p.rows * (p.row_bytes / 16);
  int64_t blocks = (total + PM_THREADS - 1) / PM_THREADS;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(PM_THREADS), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_schedule(const ScheduleArgs& p, hipStream_t stream, Timing t) {
  return launch_k(schedule_kernel, dim3(1), dim3(PM_THREADS), stream, t, p);
}

hipError_t launch_combine(const CombineArgs& p, bool bf16_out, hipStream_t stream, Timing t) {
  const int64_t threads = p.tokens * (p.hidden / 4);
  if (threads <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((threads + PM_THREADS - 1) / PM_THREADS));
  if (bf16_out) return launch_k(combine_kernel<true>, grid, dim3(PM_THREADS), stream, t, p);
  return launch_k(combine_kernel<false>, grid, dim3(PM_THREADS), stream, t, p);
}

}  // namespace moe
