// grouped_w8a16.hip — one launch of weight-only int8 GEMMs over routed experts (gfx950).
//
// "Phase 5a: int8 weight-only quantization" (Summary) runs a mixture-of-experts block as a
// single grouped GEMM over expert weights that are stacked into one tensor per projection,
// with per-output-channel int8 codes.  Here the expert-grouped dispatch happens inside the
// kernel: workgroup (tile, slot) covers 16 output channels of one expert.  When there are at
// least as many assignments as experts every expert gets a row of workgroups (slot = expert,
// highest id first).  With fewer, most experts receive no token, so the grid has one row per
// assignment only and a workgroup's expert is the slot-th largest id that occurs: every
// workgroup marks the ids' experts in an LDS bitmap and picks from it, slots past the number
// of distinct experts exit at once, and the picked expert's first batch of weight loads is
// issued before the row scan.  Wavefront 0 scans the ids in order (ballot + prefix popcount,
// so the row list is deterministic) and collects the assignments p = token * topk + slot
// routed to the expert into an LDS list; a workgroup whose list is empty exits.  The listed
// rows are then processed in passes of up to 8: each pass copies its (gathered) activation
// rows into LDS with direct-to-LDS loads, and runs the dense weight-only GEMM's inner loop
// (split-K across the wavefronts, every weight load of a wave in flight at once,
// live-row-only fragment reads, ordered reduction through LDS).  The first row of
// workgroups collects assignments whose id is outside [0, num_experts) and writes zeros for
// them.  When experts can need more than two passes, up to 32 extra rows of workgroups take
// the experts' later passes (numbered from the highest expert down, from the rows per expert
// that every workgroup counts in LDS), and a workgroup walks as many tiles as bring the grid
// within one round of resident workgroups.  One token (every assignment a single row, its
// expert the id itself) and two to four tokens with at most 64 assignments (every id in one
// wavefront) take kernels without the bitmap, the scan and the staged rows: a wavefront per
// output channel streams its row of codes and meets each activation row with v_dot2.  A
// second entry point fuses the SiLU·mul between the gate/up and down projections of the
// mixture-of-experts block: gate and up are one call over weights stacked [2n, k] per
// expert, each workgroup computes 16 gate and the 16 matching up channels and stores
// silu(gate) * up (the block's activation step is a reading: no page spells it out).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant_mma.hpp"
#include "launch.h"
#include "sync.hpp"

namespace i8ql {
namespace {

constexpr int kUnroll = 8;  // steps of k whose weight loads a wavefront keeps in flight
constexpr int kList = 1024;     // assignments held in LDS per scan window
constexpr int kScanBatch = 8;   // 64-id groups whose loads a wavefront keeps in flight together
constexpr int kMaxPassRows = 8;  // activation rows staged in LDS per pass
constexpr size_t kMaxStageBytes = 128 * 1024;  // LDS for the staged rows of one pass
constexpr int kMaxTileSeq = 16;   // 16-channel tiles one workgroup walks, at most
constexpr int64_t kCusPerGpu = 256;  // MI355X compute units (sizes the tiles per workgroup)
constexpr int kMaxExtraRows = 32;     // rows of workgroups that take experts' later passes
constexpr int64_t kHistMaxExperts = 4096;  // experts counted in LDS for that split

template <int WAVES>
constexpr size_t red_bytes() { return static_cast<size_t>(WAVES) * 64 * sizeof(v4f); }

// Dynamic LDS: [WAVES][64] v4f partial tiles, the staged rows of one pass (pass_rows rows,
// see stage_rows), a 16-byte zero block, the expert bitmap (one bit per expert, 16-byte
// multiple) or, when later passes are split over extra workgroups, the rows per expert (one
// int per expert).
__host__ __device__ inline size_t xs_bytes(int pass_rows, int64_t k) {
  return 1024 * static_cast<size_t>(stage_insts(pass_rows, k)) + 16;
}
__host__ __device__ inline size_t bitmap_bytes(int64_t experts) {
  return 16 * static_cast<size_t>((experts + 127) / 128);
}
__host__ __device__ inline size_t hist_bytes(int64_t experts) {
  return 16 * static_cast<size_t>((experts + 3) / 4);
}

// Later passes split over extra workgroups.  An expert with c rows takes ceil(c / pass_rows)
// passes; its own workgroup runs the first, and its later ones (ex = passes - 1 of them) are
// numbered globally from the highest expert id down.  Extra row j runs later pass number j;
// the expert's own workgroup runs the ones numbered xrows and beyond.  From the rows per
// expert in hist[], wavefront-uniformly: for `mine` < 0 (an extra row, j = -mine - 1) the
// expert and its pass index (>= 1), or expert -1 when fewer later passes exist; for an
// expert's own workgroup (mine = e) the global number of its first later pass.
__device__ __forceinline__ void later_pass(const int* hist, int64_t experts, int pass_rows,
                                           int64_t mine, int lane, int64_t& e_out,
                                           int& pass_out, int64_t& first_out) {
  int64_t before = 0;  // later passes of the experts above the current group
  for (int64_t top = experts - 1; top >= 0; top -= 64) {
    const int64_t e = top - lane;  // lane 0 holds the highest expert of this group
    const int c = e >= 0 ? hist[e] : 0;
    const int ex = c > pass_rows ? (c + pass_rows - 1) / pass_rows - 1 : 0;
    int incl = ex;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    if (mine >= 0) {
      if (mine > top - 64) {  // this group holds the expert
        const int src = static_cast<int>(top - mine);
        first_out = before + __shfl(incl - ex, src);
        return;
      }
    } else {
      const int64_t j = -mine - 1;
      const int in_group = __shfl(incl, 63);
      if (j < before + in_group) {
        const uint64_t here = __ballot(before + incl > j && before + incl - ex <= j);
        const int src = __ffsll(static_cast<unsigned long long>(here)) - 1;
        e_out = top - src;
        pass_out = static_cast<int>(j - (before + __shfl(incl - ex, src))) + 1;
        return;
      }
    }
    before += __shfl(incl, 63);
  }
  e_out = -1;
  pass_out = 0;
  first_out = before;
}

// Ids [p, p + 64 * kScanBatch) for this lane, 64 apart: idv[j] = ids[p + 64 j + lane].
// Groups that start past the end are not loaded (-1); lanes past the end of a partial group
// re-read the last id and must be masked by the caller.
__device__ __forceinline__ void load_id_batch(const int32_t* __restrict__ ids, int64_t total,
                                              int64_t p, int lane,
                                              int32_t (&idv)[kScanBatch]) {
#pragma unroll
  for (int j = 0; j < kScanBatch; ++j) {
    idv[j] = -1;
    if (p + 64 * j < total) {
      const int64_t q = p + 64 * j + lane;
      idv[j] = ids[q < total ? q : total - 1];
    }
  }
}

// The slot-th largest set bit of present[0, words) (wavefront-uniform), or -1 when fewer
// bits are set.  Words are taken 64 at a time from the top; a prefix sum of their popcounts
// across the lanes finds the word holding the bit.
__device__ __forceinline__ int nth_present_from_top(const uint32_t* present, int words,
                                                        int slot, int lane) {
  int rem = slot;
  for (int top = words - 1; top >= 0; top -= 64) {
    const int w = top - lane;  // lane 0 holds the highest word of this group
    const uint32_t bits = w >= 0 ? present[w] : 0u;
    const int pc = __popc(bits);
    int incl = pc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    const int in_group = __shfl(incl, 63);
    if (rem < in_group) {
      const uint64_t here = __ballot(incl > rem && incl - pc <= rem);
      const int src = __ffsll(static_cast<unsigned long long>(here)) - 1;
      int pick = -1;
      if (lane == src) {
        uint32_t b = bits;  // drop the set bits above the one wanted
        for (int r = rem - (incl - pc); r > 0; --r) b &= ~(1u << (31 - __clz(static_cast<int>(b))));
        pick = w * 32 + 31 - __clz(static_cast<int>(b));
      }
      return __shfl(pick, src);
    }
    rem -= in_group;
  }
  return -1;
}

// Workgroup: 16 output channels of one expert, split over KS wavefronts along k.  BITMAP:
// the expert is the slot-th largest id present (fewer assignments than experts); otherwise
// every expert has its own row of workgroups.  SILU: each expert's weights are [2n, k], gate
// rows then up rows; the workgroup computes the 16 gate channels with wavefronts [0, KS) and
// the 16 matching up channels with [KS, 2 KS), and stores silu(gate) * up.
// (Three wavefronts per SIMD for the one-row-per-expert form, which the compiler otherwise
// missed by a few registers; the bitmap form needs more than a third of them.)
template <int KS, bool BITMAP, bool SILU, int YT>
__global__ __launch_bounds__(64 * KS * (SILU ? 2 : 1))
__attribute__((amdgpu_waves_per_eu(BITMAP ? 1 : 3))) void grouped_w8a16_kernel(
    const uint16_t* __restrict__ x, int x_per_assignment, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t num_experts, const int32_t* __restrict__ ids,
    int64_t total, int64_t topk, void* __restrict__ y, int64_t n, int64_t k, int pass_rows,
    int tseq, int xrows) {
  constexpr int TILES = SILU ? 2 : 1;
  constexpr int WAVES = KS * TILES;
  constexpr int kEpiWave = WAVES - 1;  // reduces the partial tiles and stores the outputs
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int list[kList];
  __shared__ int s_count;
  __shared__ int64_t s_next;
  __shared__ int64_t s_expert;
  v4f* red = reinterpret_cast<v4f*>(smem);
  char* xs = smem + red_bytes<WAVES>();
  char* xzero = xs + 1024 * stage_insts(pass_rows, k);
  uint32_t* present = reinterpret_cast<uint32_t*>(xzero + 16);
  int* hist = reinterpret_cast<int*>(xzero + 16);  // (the bitmap's place; never both)

  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform: a scalar
  const bool invalid_row = blockIdx.y == 0;
  // tseq consecutive 16-channel tiles, one after the other: the expert choice, the row scan
  // and the staged activation rows serve all of them
  const int64_t nb = static_cast<int64_t>(blockIdx.x) * tseq * 16;
  if (threadIdx.x == 0) *reinterpret_cast<v4u*>(xzero) = v4u{0u, 0u, 0u, 0u};

  // Wavefront 0's first batch of ids, loaded once: the bitmap pass and the first window of
  // the row scan both use it.
  int32_t idv[kScanBatch];
  bool idv_loaded = false;
  int64_t e = num_experts;  // the invalid-id row matches ids outside [0, num_experts)
  // The passes this workgroup runs: pass index gi when gi == pass_a or gi > pass_b (every
  // pass by default).  With later passes split over extra rows (!BITMAP, xrows > 0, all
  // ids in one scan window) an extra row runs its one pass, and an expert's own row its
  // first pass and the later ones that no extra row took.
  int pass_a = 0, pass_b = 0;
  if constexpr (!BITMAP) {
    // every expert has a row of workgroups, highest id first: the always-on shared experts
    // are appended after the routed ones and receive every token, so they start first
    // instead of forming the tail.  The extra rows come before them, for the same reason.
    const int64_t y_row = static_cast<int64_t>(blockIdx.y);
    if (!invalid_row) e = y_row > xrows ? num_experts - (y_row - xrows) : -1;
    if (!invalid_row && xrows > 0) {
      // ---- rows per expert, then this workgroup's passes ------------------------------
      for (int64_t i = threadIdx.x; i < num_experts; i += 64 * WAVES) hist[i] = 0;
      lds_barrier();
      // (every id load in flight at once: total <= kList here)
      constexpr int kPer = (kList + 64 * WAVES - 1) / (64 * WAVES);
      int32_t hv[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int64_t q = threadIdx.x + static_cast<int64_t>(j) * 64 * WAVES;
        hv[j] = q < total ? ids[q] : -1;
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (hv[j] >= 0 && hv[j] < num_experts) atomicAdd(hist + hv[j], 1);
      lds_barrier();
      if (wave == 0) {
        int64_t pe = 0, first = 0;
        int pp = 0;
        later_pass(hist, num_experts, pass_rows, e >= 0 ? e : -y_row, lane, pe, pp, first);
        if (lane == 0) {
          if (e < 0) {
            s_expert = pe;
            s_count = pp;
          } else {
            s_next = first;
          }
        }
      }
      lds_barrier();
      if (e < 0) {
        e = s_expert;
        pass_a = s_count;
        pass_b = 0x7fffffff;
        if (e < 0) return;  // fewer later passes than extra rows (uniform)
      } else {
        // later passes numbered below xrows went to the extra rows
        pass_b = static_cast<int>(max(static_cast<int64_t>(0),
                                      static_cast<int64_t>(xrows) - s_next));
      }
      pass_a = __builtin_amdgcn_readfirstlane(pass_a);
      pass_b = __builtin_amdgcn_readfirstlane(pass_b);
      __syncthreads();  // s_count and s_next are written again by the scan
    }
  } else if (!invalid_row) {
    // ---- the expert of this slot: mark every expert named by an id, then pick ---------
    const int words = static_cast<int>((num_experts + 31) / 32);
    for (int i = threadIdx.x; i < words; i += 64 * WAVES) present[i] = 0u;
    if (wave == 0) {
      load_id_batch(ids, total, 0, lane, idv);
      idv_loaded = true;
    }
    lds_barrier();  // the bitmap is clear
    // 64-id groups: wavefront w marks groups w, w + WAVES, ..., kScanBatch loads in flight
    const int64_t groups = (total + 63) / 64;
    for (int64_t g0 = wave; g0 < groups; g0 += static_cast<int64_t>(WAVES) * kScanBatch) {
      int32_t b[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        const int64_t g = g0 + static_cast<int64_t>(j) * WAVES;
        const int64_t q = g * 64 + lane;
        b[j] = g < groups ? ids[q < total ? q : total - 1] : -1;
      }
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        const int64_t q = (g0 + static_cast<int64_t>(j) * WAVES) * 64 + lane;
        const int32_t id = b[j];
        if (q < total && id >= 0 && id < num_experts)
          atomicOr(present + (id >> 5), 1u << (id & 31));
      }
    }
    lds_barrier();  // the bitmap is complete
    if (wave == 0) {
      // slots in decreasing id order, for the same reason as above
      const int pick =
          nth_present_from_top(present, words, static_cast<int>(blockIdx.y) - 1, lane);
      if (lane == 0) s_expert = pick;
    }
    lds_barrier();
    e = s_expert;
    if (e < 0) return;  // fewer distinct experts than slots (uniform over the workgroup)
  }
  // (uniform; a value read from LDS is not known to be, and the addresses built from it
  // would be computed per lane)
  e = __builtin_amdgcn_readfirstlane(static_cast<int>(e));

  // Weight rows per expert: TILES * n; this wavefront's tile (0: the channels themselves or
  // the gate rows, 1: the up rows) starts at row tile * n of its expert.  Per 16-channel
  // tile at n0: a buffer resource over the tile's weight rows (rows past n read as zeros;
  // their channels are never stored) and (the epilogue's wavefront) the 4 output-channel
  // scales of its lane group.  voff: this lane's row and 32-channel slot within any tile.
  const int tile = wave / KS;
  float sc[TILES][4] = {};
  auto weight_tile = [&](int64_t n0) {
    const int64_t rows = invalid_row ? 0 : min(static_cast<int64_t>(16), n - n0);
    return weight_rsrc(wq + (invalid_row ? 0 : ((e * TILES + tile) * n + n0) * k), rows * k);
  };
  const int voff = (lane % 16) * static_cast<int>(k) + 32 * (lane / 16);
  auto load_scales = [&](int64_t n0) {
    if (wave == kEpiWave) {
      const int64_t nc = n0 + 4 * (lane / 16);
#pragma unroll
      for (int ti = 0; ti < TILES; ++ti)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sc[ti][r] = w_scale[(e * TILES + ti) * n + min(nc + r, n - 1)];
    }
  };
  int sb, se;
  wave_step_range(k, KS, wave % KS, sb, se);
  v4u w[kUnroll][2];
  bool w_loaded = false;
  // The first tile's scales are requested before the scan so that their latency overlaps
  // it; they go to the last wavefront, which runs the epilogue, so that the scan on
  // wavefront 0 never waits for them (with one wavefront it does).  A picked expert has rows
  // for certain, so its first batch of weight loads goes out before the scan too.
  int64_t sc_n0 = nb;  // the tile whose scales sc holds
  if (!invalid_row) load_scales(nb);
  if (!invalid_row && BITMAP) {
    load_weight_batch_rsrc<kUnroll>(weight_tile(nb), voff, sb, w);
    w_loaded = true;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  int64_t p_next = 0;
  while (true) {
    // ---- expert-grouped dispatch: collect the next window of assignments for e --------
    // The ids are read kScanBatch * 64 at a time, every load of a batch in flight at once
    // (one memory round trip per batch instead of one per 64 ids), then matched 64 at a time
    // in order.
    if (wave == 0) {
      int base = 0;
      int64_t p = p_next;
      bool full = false;
      while (p < total && !full) {
        if (!(idv_loaded && p == 0)) load_id_batch(ids, total, p, lane, idv);
        idv_loaded = false;
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
          const int64_t mine = p + lane;
          if (p >= total) break;
          const int32_t id = idv[j];
          const bool match =
              mine < total && (invalid_row ? (id < 0 || id >= num_experts) : (id == e));
          const uint64_t mask = __ballot(match);
          const int cnt = __popcll(mask);
          if (base + cnt > kList) {  // the window is full; resume at p next time
            full = true;
            break;
          }
          if (match) {
            const uint64_t below = lane == 0 ? 0ull : (mask & ((~0ull) >> (64 - lane)));
            list[base + __popcll(below)] = static_cast<int>(mine);
          }
          base += cnt;
          p += 64;
        }
      }
      if (lane == 0) {
        s_count = base;
        s_next = p;
      }
    }
    lds_barrier();
    const int count = s_count;
    p_next = s_next;

    if (invalid_row) {
      const int nt = tseq;
      for (int i = threadIdx.x; i < count * 16 * nt; i += 64 * WAVES) {
        const int64_t row = list[i / (16 * nt)];
        const int64_t c = nb + i % (16 * nt);
        if (c >= n) continue;
        if constexpr (YT == I8QL_F32) {
          static_cast<float*>(y)[row * n + c] = 0.0f;
        } else {
          static_cast<uint16_t*>(y)[row * n + c] = 0;
        }
      }
    } else if (count > 0) {
      const int64_t pitch = 2 * k + 16;
      const int div = x_per_assignment ? 1 : static_cast<int>(topk);
      for (int g = 0; g < count; g += pass_rows) {
        {
          const int gi = g / pass_rows;  // (the whole list is one window when split)
          if (gi != pass_a && gi <= pass_b) continue;  // uniform
        }
        // Activation rows of this pass, then the tiles one after the other.  For each tile
        // (unless its first batch of weight loads is already in flight) its scales and first
        // batch of weight loads (a later pass re-reads the same weights, from cache); on the
        // first tile wait for the rows only (loads issued after them may stay in flight) and
        // publish them to every wavefront.  The compiler barriers keep the weight loads
        // behind the copy, which the wait count relies on.
        const int rows = min(pass_rows, count - g);
        stage_rows<WAVES>(x, list + g, div, rows, k, xs);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const bool live = lane % 16 < rows;
        const char* xrow = xs + (live ? lane % 16 : 0) * pitch;
        v4u xb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) xb[c] = v4u{0u, 0u, 0u, 0u};
        const int nt = tseq;
        for (int ti = 0; ti < nt; ++ti) {
          const int64_t n0 = nb + 16 * ti;
          if (n0 >= n) break;  // uniform
          // The step range, the weight offset and the staged row pass through opaque copies,
          // so that the compiler derives the batch's offsets here, per tile, instead of
          // holding them all in registers across the loops (the staged row as an LDS byte
          // offset: a pointer through the copy would lose its address space and turn the
          // fragment reads into flat loads).
          const __amdgpu_buffer_rsrc_t wt = weight_tile(n0);
          int s0 = sb, s1 = se, vo = voff;
          int xo = static_cast<int>(xrow - smem);
          asm volatile("" : "+s"(s0), "+s"(s1));
          asm volatile("" : "+v"(vo));
          asm volatile("" : "+v"(xo));
          const char* xr = smem + xo;
          if (w_loaded) {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            w_loaded = false;
          } else {
            if (sc_n0 != n0) {
              load_scales(n0);
              sc_n0 = n0;
            }
            load_weight_batch_rsrc<kUnroll>(wt, vo, s0, w);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if (ti == 0) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kUnroll, 0));
          }
          if (ti == 0) bare_barrier();
          v4f acc = {0.f, 0.f, 0.f, 0.f};
          mma_batch_staged<kUnroll>(w, xr, live, xzero, k, s0, s1, xb, acc);
          for (int s = s0 + kUnroll; s < s1; s += kUnroll) {
            load_weight_batch_rsrc<kUnroll>(wt, vo, s, w);
            __builtin_amdgcn_sched_barrier(0);
            mma_batch_staged<kUnroll>(w, xr, live, xzero, k, s, s1, xb, acc);
          }
          red[wave * 64 + lane] = acc;
          lds_barrier();
          if (wave == kEpiWave && lane % 16 < rows) {
            v4f sum[TILES];
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt) {
              sum[tt] = red[tt * KS * 64 + lane];
#pragma unroll
              for (int w2 = 1; w2 < KS; ++w2) sum[tt] += red[(tt * KS + w2) * 64 + lane];
            }
            const int64_t row = list[g + lane % 16];
            const int64_t nc = n0 + 4 * (lane / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int64_t c = nc + r;
              if (c >= n) continue;
              float v = sum[0][r] * sc[0][r];
              if constexpr (SILU) {
                // silu(gate) * up, with silu(v) = v / (1 + exp(-v))
                v = v / (1.0f + expf(-v)) * (sum[1][r] * sc[1][r]);
              }
              if constexpr (YT == I8QL_F32) {
                static_cast<float*>(y)[row * n + c] = v;
              } else {
                static_cast<uint16_t*>(y)[row * n + c] = f32_to_bf16_rne(v);
              }
            }
          }
          lds_barrier();  // red[] (and, after the last tile, the staged rows) are reused
        }
      }
    }
    if (p_next >= total) break;
    __syncthreads();  // the next window overwrites list[]
  }
}

// ---- one token (T = 1) ------------------------------------------------------------------
// With one token every assignment is a product of one activation row with one expert's
// matrix, and its expert is the id itself: no bitmap, no row scan, no staged rows.
// Workgroup (4 channels, assignment p): its wavefronts read the id (one scalar load), then,
// as the dense one-row kernel does, each lane issues every 16-byte code chunk of its
// channel's row (SILU: the gate row and the matching up row) with the chunk's 16 bf16
// activations beside it, expands the codes exactly to bf16, adds bf16 pairs of products
// into a float32 sum with v_dot2_f32_bf16, the lanes' sums meet in a fixed shuffle
// butterfly, and lane 0 applies the channel's scale (SILU: silu(g) * u as the tiled kernel
// computes it) and stores.  Ids outside [0, num_experts) store zeros.  k <= 64 * 16 *
// kRowChunks.
constexpr int kRowChunks = 8;
typedef short v2s __attribute__((ext_vector_type(2)));  // a bf16 pair, as the builtin takes it

// acc + the 16 products of a 16-byte code chunk w with its activations x[0..1] (8 bf16
// each; masked to zero by `in` for a chunk past the row's end): the codes expand exactly to
// bf16 and v_dot2_f32_bf16 adds each bf16 pair of products into the float32 sum, in order.
__device__ __forceinline__ float dot_chunk(const v4u w, const v4u (&x)[2], uint32_t in,
                                           float acc) {
  v8bf a[2];
  i8x16_to_bf16(w, a[0], a[1]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const v4u xm = x[h] & in;
    const v4u av = __builtin_bit_cast(v4u, a[h]);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};  // bf16 pairs of codes
    const uint32_t xw[4] = {xm.x, xm.y, xm.z, xm.w};  // bf16 pairs of activations
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2s, aw[e]),
                                            __builtin_bit_cast(v2s, xw[e]), acc, false);
  }
  return acc;
}

template <int KC, bool SILU, int YT>
__global__ __launch_bounds__(256) void grouped_one_token_kernel(
    const uint16_t* __restrict__ x, int x_per_assignment, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t num_experts, const int32_t* __restrict__ ids,
    int64_t topk, void* __restrict__ y, int64_t n, int64_t k) {
  constexpr int TILES = SILU ? 2 : 1;
  const int lane = threadIdx.x % 64;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (c >= n) return;  // (uniform over the wavefront)
  const int64_t p = blockIdx.y;
  const int32_t id = __builtin_amdgcn_readfirstlane(ids[p]);
  if (id < 0 || id >= num_experts) {
    if (lane == 0) {
      if constexpr (YT == I8QL_F32) {
        static_cast<float*>(y)[p * n + c] = 0.0f;
      } else {
        static_cast<uint16_t*>(y)[p * n + c] = 0;
      }
    }
    return;
  }
  const int64_t chunks = k / 16;
  const v4u* xr = reinterpret_cast<const v4u*>(x + (x_per_assignment ? p : p / topk) * k);
  const v4u* wr[TILES];
#pragma unroll
  for (int ti = 0; ti < TILES; ++ti)
    wr[ti] = reinterpret_cast<const v4u*>(wq + ((id * TILES + ti) * n + c) * k);
  v4u w[TILES][KC], xv[KC][2];
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int64_t ch = lane + 64 * static_cast<int64_t>(i);
    const int64_t cc = ch < chunks ? ch : 0;  // in bounds; multiplied by nothing below
#pragma unroll
    for (int ti = 0; ti < TILES; ++ti) w[ti][i] = wr[ti][cc];
    xv[i][0] = xr[2 * cc];
    xv[i][1] = xr[2 * cc + 1];
  }
  asm volatile("" ::: "memory");  // the loads stay here, in order, ahead of every use
  __builtin_amdgcn_sched_barrier(0);
  float acc[TILES] = {};
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const uint32_t in = lane + 64 * i < chunks ? 0xffffffffu : 0u;
#pragma unroll
    for (int ti = 0; ti < TILES; ++ti) acc[ti] = dot_chunk(w[ti][i], xv[i], in, acc[ti]);
  }
#pragma unroll
  for (int ti = 0; ti < TILES; ++ti)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[ti] += __shfl_xor(acc[ti], off, 64);
  if (lane != 0) return;
  float v = acc[0] * w_scale[(id * TILES) * n + c];
  if constexpr (SILU) {
    // silu(gate) * up, with silu(v) = v / (1 + exp(-v))
    v = v / (1.0f + expf(-v)) * (acc[1] * w_scale[(id * TILES + 1) * n + c]);
  }
  if constexpr (YT == I8QL_F32) {
    static_cast<float*>(y)[p * n + c] = v;
  } else {
    static_cast<uint16_t*>(y)[p * n + c] = f32_to_bf16_rne(v);
  }
}

// Launches the one-token kernel when it applies (t == 1, k within its chunks); false when
// it does not (nothing launched).
template <bool SILU, int YT>
bool launch_one_token(const void* x, int x_per_assignment, const int8_t* wq,
                      const float* w_scale, int64_t num_experts, const int32_t* ids,
                      int64_t t, int64_t topk, void* y, int64_t n, int64_t k,
                      hipStream_t stream, hipError_t* err) {
  const int64_t per_lane = (k / 16 + 63) / 64;
  if (t != 1 || per_lane > kRowChunks) return false;
  const dim3 grid(static_cast<unsigned>((n + 3) / 4), static_cast<unsigned>(t * topk));
  const auto* xx = static_cast<const uint16_t*>(x);
#define I8QL_ONE(KC)                                                                       \
  hipLaunchKernelGGL((grouped_one_token_kernel<KC, SILU, YT>), grid, dim3(256), 0, stream, \
                     xx, x_per_assignment, wq, w_scale, num_experts, ids, topk, y, n, k)
  if (per_lane <= 2) {
    I8QL_ONE(2);
  } else if (per_lane <= 4) {
    I8QL_ONE(4);
  } else {
    I8QL_ONE(8);
  }
#undef I8QL_ONE
  *err = hipGetLastError();
  return true;
}

// ---- a few tokens (SiLU·mul, 2 <= t <= kFewMaxTokens, t * topk <= 64) ------------------
// With at most 64 assignments one wavefront holds every id (one load per lane), so a
// workgroup finds its expert and that expert's rows without a bitmap, a row scan or staged
// rows.  Workgroup (4 channels, assignment p): p's id is the expert; the workgroup runs it
// only when p is the expert's first assignment (the lowest lane of the ballot of equal ids;
// the expert's other workgroups exit).  Each lane issues every code chunk of its channel's
// row (SILU: and of the matching up row) and the channel's scales once, then takes the
// expert's rows in ascending order, one at a time: the chunks' activations, dot_chunk, the
// shuffle butterfly, and lane 0 scales (SILU: silu(g) * u) and stores, as the one-token
// kernel does.  An id outside [0, num_experts) stores zeros for its own assignment.
// (Measured on the 16B MoE and dropped: four rows' activations loaded together whether or
// not the expert has them, 1.5-1.8x slower at 1 and 4 tokens, every wavefront reading rows
// that most experts do not have; four rows together only while four remain, 1.3x slower at
// 4 tokens, the registers they hold costing occupancy.)
constexpr int64_t kFewMaxTokens = 8;
constexpr int kFewAssignments = 64;

template <int KC, bool SILU, int YT>
__global__ __launch_bounds__(256) void grouped_few_kernel(
    const uint16_t* __restrict__ x, int x_per_assignment, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t num_experts, const int32_t* __restrict__ ids,
    int total, int64_t topk, void* __restrict__ y, int64_t n, int64_t k) {
  constexpr int TILES = SILU ? 2 : 1;
  const int lane = threadIdx.x % 64;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (c >= n) return;  // (uniform over the wavefront)
  const int p = static_cast<int>(blockIdx.y);
  const int32_t my_id = lane < total ? ids[lane] : -1;
  const int32_t id = __builtin_amdgcn_readfirstlane(__shfl(my_id, p));
  if (id < 0 || id >= num_experts) {
    if (lane == 0) {
      if constexpr (YT == I8QL_F32) {
        static_cast<float*>(y)[p * n + c] = 0.0f;
      } else {
        static_cast<uint16_t*>(y)[p * n + c] = 0;
      }
    }
    return;
  }
  uint64_t rows = __ballot(lane < total && my_id == id);  // the expert's assignments
  if (__ffsll(static_cast<unsigned long long>(rows)) - 1 != p) return;  // not the first
  const int64_t chunks = k / 16;
  v4u w[TILES][KC];
#pragma unroll
  for (int ti = 0; ti < TILES; ++ti) {
    const v4u* wr = reinterpret_cast<const v4u*>(wq + ((id * TILES + ti) * n + c) * k);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int64_t ch = lane + 64 * static_cast<int64_t>(i);
      w[ti][i] = wr[ch < chunks ? ch : 0];  // in bounds; multiplied by nothing below
    }
  }
  float sc[TILES];  // (loaded with the weights: read at the end, each row waited for them)
#pragma unroll
  for (int ti = 0; ti < TILES; ++ti) sc[ti] = w_scale[(id * TILES + ti) * n + c];
  const int div = x_per_assignment ? 1 : static_cast<int>(topk);
  while (rows != 0) {
    const int r = __ffsll(static_cast<unsigned long long>(rows)) - 1;
    rows &= rows - 1;
    const v4u* xr = reinterpret_cast<const v4u*>(x + static_cast<int64_t>(r / div) * k);
    v4u xv[KC][2];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int64_t ch = lane + 64 * static_cast<int64_t>(i);
      const int64_t cc = ch < chunks ? ch : 0;
      xv[i][0] = xr[2 * cc];
      xv[i][1] = xr[2 * cc + 1];
    }
    asm volatile("" ::: "memory");  // the loads stay here, in order, ahead of every use
    __builtin_amdgcn_sched_barrier(0);
    float acc[TILES] = {};
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const uint32_t in = lane + 64 * i < chunks ? 0xffffffffu : 0u;
#pragma unroll
      for (int ti = 0; ti < TILES; ++ti) acc[ti] = dot_chunk(w[ti][i], xv[i], in, acc[ti]);
    }
#pragma unroll
    for (int ti = 0; ti < TILES; ++ti)
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc[ti] += __shfl_xor(acc[ti], off, 64);
    if (lane != 0) continue;
    float v = acc[0] * sc[0];
    if constexpr (SILU) {
      // silu(gate) * up, with silu(v) = v / (1 + exp(-v))
      v = v / (1.0f + expf(-v)) * (acc[1] * sc[1]);
    }
    if constexpr (YT == I8QL_F32) {
      static_cast<float*>(y)[r * n + c] = v;
    } else {
      static_cast<uint16_t*>(y)[r * n + c] = f32_to_bf16_rne(v);
    }
  }
}

// Launches the few-token kernel when it applies (the SiLU·mul call, 2 <= t <= kFewMaxTokens,
// t * topk <= 64, k within its chunks); false when it does not (nothing launched).  The
// plain call keeps the tiled kernel: at 4 tokens on the 16B MoE the few-token kernel made
// the gate, up and down layer 60.4 -> 62.7 us (each launch alone was faster, with the
// touched weights left in the Infinity Cache between launches), while the SiLU·mul call
// goes 41.4 -> 26.2 us and the block 75.6 -> 60.0 us; the SiLU·mul call at 6 and 8 tokens
// 50.8 -> 36.5 and 68.0 -> 49.3 us.
template <bool SILU, int YT>
bool launch_few(const void* x, int x_per_assignment, const int8_t* wq, const float* w_scale,
                int64_t num_experts, const int32_t* ids, int64_t t, int64_t topk, void* y,
                int64_t n, int64_t k, hipStream_t stream, hipError_t* err) {
  if constexpr (!SILU) return false;
  const int64_t per_lane = (k / 16 + 63) / 64;
  if (t < 2 || t > kFewMaxTokens || t * topk > kFewAssignments || per_lane > kRowChunks)
    return false;
  const dim3 grid(static_cast<unsigned>((n + 3) / 4), static_cast<unsigned>(t * topk));
  const auto* xx = static_cast<const uint16_t*>(x);
  const int total = static_cast<int>(t * topk);
#define I8QL_FEW(KC)                                                                     \
  hipLaunchKernelGGL((grouped_few_kernel<KC, SILU, YT>), grid, dim3(256), 0, stream, xx, \
                     x_per_assignment, wq, w_scale, num_experts, ids, total, topk, y, n, k)
  if (per_lane <= 2) {
    I8QL_FEW(2);
  } else if (per_lane <= 4) {
    I8QL_FEW(4);
  } else {
    I8QL_FEW(8);
  }
#undef I8QL_FEW
  *err = hipGetLastError();
  return true;
}

// Compute units of the current device (cached per device; kCusPerGpu when the query fails).
int device_cus() {
  static std::atomic<int> cached[kMaxDevices];  // static storage: starts at zero
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kCusPerGpu;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();  // (not the next launch's error)
      cus = kCusPerGpu;
    }
    cached[dev].store(cus, std::memory_order_relaxed);  // a race only repeats the query
  }
  return cus;
}

// Workgroups of KERN (`threads` threads, `lds` bytes of dynamic LDS) that one compute unit
// holds at once: the runtime's occupancy query, which counts registers, wavefront slots and
// LDS (its static part included).  Cached per device for the last LDS size asked; 1 when
// the query fails.
template <auto KERN>
int resident_per_cu(int threads, size_t lds) {
  static std::atomic<int64_t> cached[kMaxDevices];  // (lds << 16) | count; 0: none
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  const bool tracked = dev >= 0 && dev < kMaxDevices;
  if (tracked) {
    const int64_t c = cached[dev].load(std::memory_order_relaxed);
    if (c != 0 && static_cast<size_t>(c >> 16) == lds) return static_cast<int>(c & 0xffff);
  }
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void*>(KERN),
                                                   threads, lds) != hipSuccess ||
      blocks < 1) {
    (void)hipGetLastError();
    blocks = 1;
  }
  blocks = blocks > 0xffff ? 0xffff : blocks;
  if (tracked)
    cached[dev].store((static_cast<int64_t>(lds) << 16) | blocks, std::memory_order_relaxed);
  return blocks;
}

template <int KS, bool BITMAP, bool SILU, int YT>
hipError_t launch_mode(const void* x, int x_per_assignment, const int8_t* wq,
                       const float* w_scale, int64_t num_experts, const int32_t* ids,
                       int64_t t, int64_t topk, void* y, int64_t n, int64_t k,
                       hipStream_t stream) {
  constexpr int WAVES = KS * (SILU ? 2 : 1);
  constexpr auto kern = grouped_w8a16_kernel<KS, BITMAP, SILU, YT>;
  // Rows staged per pass: an expert that each token picks at most once receives at most t
  // rows; one that receives more takes more passes (any count is handled).  Long rows stage
  // fewer per pass so that they fit the LDS budget (the caller bounds k so one row does).
  int pass_rows = static_cast<int>(min(static_cast<int64_t>(kMaxPassRows), t));
  while (pass_rows > 1 && xs_bytes(pass_rows, k) > kMaxStageBytes) --pass_rows;
  // Extra rows of workgroups for experts' later passes, when experts can need more than two
  // passes (fewer take the two-tile walk below), every id fits one scan window and the rows
  // per expert fit LDS: at most one per pass that the assignments could fill, and 32.
  int xrows = 0;
  if (!BITMAP && t > 2 * pass_rows && t * topk <= kList && num_experts <= kHistMaxExperts) {
    xrows = static_cast<int>(min(static_cast<int64_t>(kMaxExtraRows),
                                 (t * topk + pass_rows - 1) / pass_rows));
    xrows = static_cast<int>(min(static_cast<int64_t>(xrows), 65535 - 1 - num_experts));
  }
  const size_t lds = red_bytes<WAVES>() + xs_bytes(pass_rows, k) +
                     (xrows > 0 ? hist_bytes(num_experts) : bitmap_bytes(num_experts));
  const hipError_t e = allow_dynamic_lds<kern>(static_cast<int>(lds));
  if (e != hipSuccess) return e;
  // One row of workgroups per slot, after the row that handles invalid ids: one slot per
  // expert, or, with fewer assignments than experts, one per assignment (the most distinct
  // experts there can be).
  const int64_t slots = BITMAP ? t * topk : num_experts;
  // Tiles per workgroup, walked one after the other, so that each workgroup's expert choice,
  // row scan and staged rows serve more output channels.  With fewer assignments than
  // experts (every expert has at most t rows, one pass) as many as keep about four
  // workgroups per compute unit over the grid (at most 16).  Otherwise an expert with many
  // rows takes several passes, and walking tiles multiplies the passes of a workgroup that
  // runs them all: two tiles while no expert can need more than two passes (an expert that
  // each token picks at most once gets at most t rows; at T = 16 on the 16B MoE, 2 tiles
  // made gate and down 12-15 % faster than one).  With later passes on extra rows each
  // workgroup runs about one pass, and the walk is as long as brings the grid within one
  // round of the workgroups that the compute units hold at once (16B MoE at T = 64: gate
  // 80.1 -> 53.7 us, down 87.6 -> 65.1 us; a grid just past one round, or far below it, was
  // up to 1.5x slower).
  const int64_t tiles = (n + 15) / 16;
  int64_t per = BITMAP ? tiles * slots / (4 * kCusPerGpu) : (t <= 2 * pass_rows ? 2 : 1);
  if (xrows > 0) {
    const int64_t fit = static_cast<int64_t>(resident_per_cu<kern>(64 * WAVES, lds)) *
                        device_cus() / (slots + 1 + xrows);  // workgroups per grid row
    per = fit >= 1 ? (tiles + fit - 1) / fit : kMaxTileSeq;
  }
  if (per > kMaxTileSeq) per = kMaxTileSeq;
  const int tseq = per < 1 ? 1 : static_cast<int>(per);
  const dim3 grid(static_cast<unsigned>((tiles + tseq - 1) / tseq),
                  static_cast<unsigned>(slots + 1 + xrows));
  hipLaunchKernelGGL(kern, grid, dim3(64 * WAVES), lds, stream,
                     static_cast<const uint16_t*>(x), x_per_assignment, wq, w_scale,
                     num_experts, ids, t * topk, topk, y, n, k, pass_rows, tseq, xrows);
  return hipGetLastError();
}

template <int KS, bool SILU, int YT>
hipError_t launch_waves(const void* x, int x_per_assignment, const int8_t* wq,
                        const float* w_scale, int64_t num_experts, const int32_t* ids,
                        int64_t t, int64_t topk, void* y, int64_t n, int64_t k,
                        hipStream_t stream) {
  if (t * topk < num_experts)
    return launch_mode<KS, true, SILU, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids,
                                           t, topk, y, n, k, stream);
  return launch_mode<KS, false, SILU, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids,
                                          t, topk, y, n, k, stream);
}

// Wavefronts per tile: the fewest of 1, 2, 4 and 8 with which each streams at most kUnroll
// steps of k (one batch of loads in flight), 8 beyond; at most 4 with SiLU·mul, whose two
// tiles would otherwise make workgroups of 1024 threads (128 registers each: spills).
template <bool SILU, int YT>
hipError_t launch_yt(const void* x, int x_per_assignment, const int8_t* wq,
                     const float* w_scale, int64_t num_experts, const int32_t* ids, int64_t t,
                     int64_t topk, void* y, int64_t n, int64_t k, hipStream_t stream) {
  hipError_t err = hipSuccess;
  if (launch_one_token<SILU, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t, topk,
                                 y, n, k, stream, &err) ||
      launch_few<SILU, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t, topk, y, n,
                           k, stream, &err))
    return err;
  const int64_t steps = (k + kStepK - 1) / kStepK;
  if (steps <= kUnroll)
    return launch_waves<1, SILU, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t,
                                     topk, y, n, k, stream);
  if (steps <= 2 * kUnroll)
    return launch_waves<2, SILU, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t,
                                     topk, y, n, k, stream);
  if (SILU || steps <= 4 * kUnroll)
    return launch_waves<4, SILU, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t,
                                     topk, y, n, k, stream);
  if constexpr (!SILU)
    return launch_waves<8, SILU, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t,
                                     topk, y, n, k, stream);
  return hipErrorInvalidValue;  // not reached
}

}  // namespace

hipError_t launch_grouped_w8a16_gemm(const void* x, int x_per_assignment, const int8_t* wq,
                                     const float* w_scale, int64_t num_experts,
                                     const int32_t* expert_ids, int64_t t, int64_t topk,
                                     void* y, i8ql_dtype y_dtype, int64_t n, int64_t k,
                                     hipStream_t stream) {
  if (y_dtype == I8QL_F32)
    return launch_yt<false, I8QL_F32>(x, x_per_assignment, wq, w_scale, num_experts,
                                      expert_ids, t, topk, y, n, k, stream);
  return launch_yt<false, I8QL_BF16>(x, x_per_assignment, wq, w_scale, num_experts, expert_ids,
                                     t, topk, y, n, k, stream);
}

hipError_t launch_grouped_w8a16_silu_gemm(const void* x, int x_per_assignment,
                                          const int8_t* wq, const float* w_scale,
                                          int64_t num_experts, const int32_t* expert_ids,
                                          int64_t t, int64_t topk, void* h, i8ql_dtype h_dtype,
                                          int64_t n, int64_t k, hipStream_t stream) {
  if (h_dtype == I8QL_F32)
    return launch_yt<true, I8QL_F32>(x, x_per_assignment, wq, w_scale, num_experts,
                                     expert_ids, t, topk, h, n, k, stream);
  return launch_yt<true, I8QL_BF16>(x, x_per_assignment, wq, w_scale, num_experts, expert_ids,
                                    t, topk, h, n, k, stream);
}

}  // namespace i8ql
