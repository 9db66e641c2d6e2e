// w8a8_gemm.hip — int8 x int8 -> int32 GEMM on the gfx950 matrix cores with a fused scale
// epilogue.
//
// W8A8 quantizes both operands to int8 so the product runs on the 8-bit matrix units ("Day
// 6 — Quantize It Yourself", The mechanism, block 5); weights carry one scale per output
// channel and activations one per token, and the output is not quantized
// ("feat(quantization): support compressed-tensors W8A8 and mixed modules", Design and
// Supported Execution Scheme).  Biases follow the output channels (same page, Summary).
//
//   acc[i, j] = sum_c xq[i, c] * wq[j, c]   exact in int32 (k <= 133144)
//   y[i, j]   = ((float)acc * x_scale[i]) * w_scale[j] (+ bias[j]) -> float32 or bf16 (RNE),
//               or acc itself for int32 output.
//
// Data movement.  Both operands are K-contiguous (the nn.Linear [out, in] layout and
// row-major tokens).  A workgroup of 4 or 8 wavefronts (per k-group) owns a BM x BN output
// tile and walks k in steps of BK bytes.  Each step's A and B slices are copied global -> LDS
// by the gfx950 direct-to-LDS loads (global_load_lds_dwordx4: 16 bytes per lane, one wavefront
// instruction fills 1 KiB = 1024 / BK rows), so no VGPRs hold staged data and up to STAGES
// steps are in flight.  Each step waits (s_waitcnt vmcnt) for its own loads, passes one
// barrier, which also retires the reads of the stage about to be refilled, and refills that
// stage with the step STAGES ahead.
//
// LDS layout.  A stage holds BM + BN rows of BK bytes.  The BK / 16 chunks of each row are
// XOR-swizzled (see swizzle()) so that the 16-byte fragment reads of a wavefront are free
// of bank conflicts; the swizzle is applied on the global side (each lane fetches the
// logical chunk that belongs in its fixed LDS slot).
//
// MFMA.  Each wavefront owns a (BM / WM) x (BN / WN) sub-tile of 32 x 32 blocks of
// v_mfma_i32_32x32x32_i8.  Fragment layout: lane l supplies row l % 32 of a 32-row block and
// 16 consecutive k of a 32-k slice at offset 16 * (l / 32); A and B use the same k
// assignment, which is all the sum needs.  Accumulator: lane l, register r holds row
// 8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32 of the block.  The k loop is
// software-pipelined one 32-k slice ahead: the fragments of slice s + 1 are read while the
// MFMAs of slice s run, and the barrier of step t + 1 sits between the last slice's reads
// and its MFMAs.
//
// Tails.  Rows past m or n read a clamped valid row and are never stored.  Chunks past k
// (k % 16 == 0, so chunks are whole) read the row start; once the last step has landed its
// A chunks past k are overwritten with zeros in LDS, so they add nothing.
//
// Configurations (all with 128-byte k steps; see kCandidates): tiles from 64 x 32 to
// 320 x 256, including widths that are not powers of two (160, 192, 320) so that more
// shapes fill the 256 CUs in whole rounds, and, for the fewest tiles, 64 x 32 / 64 x 64 /
// 128 x 64 tiles with 4 or 2 k-groups (in-workgroup split-K: each group walks its share of k
// through its own LDS stages and the partial int32 tiles are summed exactly through LDS).
// The launch picks one per shape by a fitted launch-time model.  With 3 or more stages the
// loads of the stage being refilled are spread over the slices of a step between MFMAs;
// with 2 they follow the barrier, interleaved with the last slice's MFMAs.
//
// Epilogue.  Scales (and bias) are applied in registers; the values then pass through a
// per-wavefront LDS area so that the output is written with 16-byte row-contiguous stores
// (see epilogue_lds).  Stored straight from registers (2 or 4 bytes per lane) the epilogue
// took 10-29% of the kernel time on MI355X; 2048x19456x2560 went from 139 to 107 us.
//
// Tile order.  Consecutive workgroup ids are spread round-robin over the 8 XCDs, each with
// its own L2.  The linear id is remapped so that every XCD receives a contiguous range of
// tiles, walked in groups of GROUP_M tile rows so that neighbouring workgroups share A rows
// and B rows in the XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "launch.h"
#include "sync.hpp"

namespace i8ql {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;
constexpr int64_t kMaxGrid = 2147483647;  // workgroups per launch (x dimension)
constexpr int kGroupM = 8;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Physical 16-byte chunk of logical chunk c in LDS row `row`: c ^ swizzle<BK>(row).
// BK = 64 (4 chunks per row): the reads of one logical chunk by any 8 consecutive rows
// cover a whole 128-byte (32-bank) line, and by any 16 consecutive rows a whole 256-byte
// (64-bank) line.  BK = 128 (8 chunks): the same for 8 rows, and each parity class of 16
// consecutive rows covers all 8 slots of its half.  Both depend on row bits 0..4 only
// (period 32), so a fragment's swizzle is that of its row within the 32-row block.
template <int BK>
__device__ __forceinline__ int swizzle(int row) {
  if constexpr (BK == 64) {
    return ((row >> 1) ^ (row >> 3)) & 3;
  } else {
    return (row & 7) ^ ((row >> 3) & 3);
  }
}

// Linear workgroup id -> (tile row, tile column), XCD-contiguous and grouped.  With k split
// across `splits` workgroups per tile, consecutive units of an XCD's range are the splits of
// one tile (so they run at the same time, on the same XCD).
__device__ __forceinline__ bool tile_of(int64_t tiles_m, int64_t tiles_n, int splits,
                                        int64_t& tm, int64_t& tn, int& split) {
  const int64_t total = tiles_m * tiles_n * splits;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t b = blockIdx.x;
  const int64_t u = (b % kXcds) * per_xcd + b / kXcds;
  if (u >= total) return false;
  const int64_t t = u / splits;
  split = static_cast<int>(u % splits);
  const int64_t group = t / (kGroupM * tiles_n);
  const int64_t first_m = group * kGroupM;
  const int64_t gsize = min(tiles_m - first_m, static_cast<int64_t>(kGroupM));
  const int64_t in_group = t % (kGroupM * tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
  return true;
}

// k split across workgroups.  The workspace starts with kSplitMaxTiles int32 arrival
// counters (one per output tile; a fixed region, so that no call's partial tiles ever lie
// where a later call with more tiles keeps counters), then one partial tile per (tile,
// split): [tiles][splits][WAVES][TM * TN * 16][64 lanes] int32, so that every store and load
// instruction of a wavefront moves 256 contiguous bytes.  Each workgroup stores its partial
// accumulators, waits until they are written and counts itself in; the last of a tile's
// splits to arrive adds the other splits' partials to its own (int32 addition is exact and
// associative, so the sum does not depend on the arrival order), returns the counter to
// zero for the next call and applies the epilogue.  No workgroup waits for another, so the
// kernel needs no co-residency.
//
// Visibility without cache-wide operations: the partial tiles are written and read with
// device-scope (relaxed atomic) accesses, which the 8 XCDs' separate L2 caches keep
// coherent, and each wavefront waits for its stores to complete before the barrier that
// precedes the count.  The reader issues its loads only after it has seen the count.  A
// device-scope fence instead writes back or invalidates a whole L2 per call, and with one
// per workgroup those serialized: 128 x 128 tiles, 2 splits, 512 x 6144 x 2560 took 162 us
// against 18 us without a split.
constexpr int64_t kSplitMaxTiles = 4096;  // split plans have at most this many tiles

template <class C>
__device__ bool splitk_fixup(v16i (&acc)[C::TM][C::TN], int* __restrict__ ws, int64_t tile,
                             int split, int splits, int wave, int lane, int* last_flag) {
  constexpr int TM = C::TM, TN = C::TN;
  constexpr int64_t kSlot = static_cast<int64_t>(C::WAVES) * TM * TN * 16 * 64;  // ints
  int* ctr = ws;
  int* part = ws + kSplitMaxTiles;
  const int64_t wofs = static_cast<int64_t>(wave) * TM * TN * 16 * 64 + lane;
  int* mine = part + (tile * splits + split) * kSlot + wofs;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __hip_atomic_store(mine + ((i * TN + j) * 16 + r) * 64, acc[i][j][r], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wavefront's stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(ctr + tile, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == splits - 1;
    if (last) __hip_atomic_store(ctr + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last_flag = last;
  }
  __syncthreads();
  if (!*last_flag) return false;
  for (int sp = 0; sp < splits; ++sp) {
    if (sp == split) continue;
    const int* other = part + (tile * splits + sp) * kSlot + wofs;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[i][j][r] += __hip_atomic_load(other + ((i * TN + j) * 16 + r) * 64,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

// Wait until at most `pending` of this wavefront's load batches (LOADS instructions each)
// are outstanding and its LDS reads are done, then barrier.  After it every wavefront's
// loads of the awaited step have landed and every read of the stage about to be refilled
// has completed.  The LDS drain is inline asm because the compiler would drop it (it only
// tracks the reads' destination registers, not the reuse of the stage by other wavefronts);
// the vmcnt wait uses the builtin so that the compiler knows the loads have landed.
template <int LOADS>
__device__ __forceinline__ void wait_and_barrier(int pending) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (pending >= 3) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * LOADS, 15));
  } else if (pending == 2) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * LOADS, 15));
  } else if (pending == 1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(LOADS, 15));
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  }
  bare_barrier();
}

// Tile geometry and per-thread addressing shared by the pieces of the kernel.  GS: weight
// scales per group of 128 input channels; each stage then also holds the step's scales, one
// 256-byte slot per wavefront (a dword per lane, loaded with the operand rows).
template <int BM_, int BN_, int BK_, int STAGES_, int KS_, int WM_, int WN_, bool GS_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, KS = KS_;
  static constexpr int WM = WM_, WN = WN_;          // wavefront grid of a k-group
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES * KS;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wavefront sub-tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int CHUNKS = BK / 16;            // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 1024 / BK;   // rows per wavefront load instruction
  static constexpr int LOADS = (BM + BN) / ROWS_PER_LOAD / WAVES;  // per wavefront per step
  static constexpr int SLICES = BK / 32;
  static constexpr bool GS = GS_;
  static constexpr int ROW_BYTES = (BM + BN) * BK;   // operand rows of a stage
  static constexpr int STAGE_BYTES = ROW_BYTES + (GS ? WAVES * 256 : 0);
  static constexpr int VM = LOADS + (GS ? 1 : 0);    // vector-memory loads per wave per step
  static constexpr size_t GROUP_BYTES = static_cast<size_t>(STAGES) * STAGE_BYTES;
  static constexpr size_t RED_BYTES = static_cast<size_t>(KS / 2) * BM * BN * 4;
  static constexpr size_t LDS_BYTES = KS * GROUP_BYTES > RED_BYTES ? KS * GROUP_BYTES : RED_BYTES;
  // the epilogue's parameter table per wavefront of the first k-group: row scales, column
  // scales, bias, each in whole 64-value copies
  static constexpr int PAR_RM = (WTM + 63) / 64 * 64, PAR_RN = (WTN + 63) / 64 * 64;
  static constexpr int PAR_WORDS = PAR_RM + 2 * PAR_RN;
  static constexpr size_t PAR_BYTES = static_cast<size_t>(WAVES) * PAR_WORDS * 4;
  // whether a kernel whose stages take `stage_lds` bytes keeps the table: it must fit in the
  // 160 KiB of LDS, and the tiles whose accumulators take more than 128 registers (their
  // kernels use every register) keep reading the parameters from memory instead
  static constexpr bool params_fit(size_t stage_lds) {
    return stage_lds + PAR_BYTES <= 160 * 1024 && TM * TN <= 8;
  }
  static_assert(KS == 1 || KS == 2 || KS == 4, "k-groups per workgroup");
  static_assert(BK == 64 || BK == 128, "BK is 64 or 128 bytes");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "sub-tile must be whole 32x32 blocks");
  static_assert(LOADS * ROWS_PER_LOAD * WAVES == BM + BN, "loads must split over waves");
  static_assert(STAGES >= 2 && STAGES <= 4, "wait_and_barrier handles up to 3 pending");
  static_assert(VM * (STAGES - 1) <= 63, "vmcnt range");
  static_assert(!GS || (KS == 1 && STAGES >= 3 && BK == 128 && WTN <= 64),
                "group scales: one k-group, spread refills, a step per group, one scale load");
};

// Group-scale state of a lane (GS only): where its column's scales are, this wavefront's
// scale slot in a stage, the scales of the step being computed (one per 32-column block) and
// the float accumulators, to which each step adds its exact int32 partial times its scale.
template <class C>
struct GroupScales {
  const float* src;  // scales of this lane's load column: step g at src[g]
  int slot;          // byte offset of this wavefront's scale slot within a stage
  float cur[C::TN];
  v16f facc[C::TM][C::TN];
};

// The scales of the step held in `stage`, for this lane's columns j * 32 + lane % 32.
template <class C>
__device__ __forceinline__ void gs_read(const int8_t* stage, GroupScales<C>& gs, int lane) {
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
    gs.cur[j] = *reinterpret_cast<const float*>(stage + gs.slot + (j * 32 + lane % 32) * 4);
}

// End of a step: facc += (float)acc * scale (the conversion is exact: a step's partial sum
// is below 128 * 127^2 < 2^24 in magnitude).  The next step's first slice starts from a
// zero C operand instead of a cleared acc.
template <class C>
__device__ __forceinline__ void gs_apply(const v16i (&acc)[C::TM][C::TN], GroupScales<C>& gs) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        gs.facc[i][j][r] = __fmaf_rn(static_cast<float>(acc[i][j][r]), gs.cur[j],
                                     gs.facc[i][j][r]);
}

// Issue this wavefront's direct-to-LDS loads of k step `step` into `stage`.  A chunk past
// the end of the row (k % 16 == 0, so chunks are whole) reads the row start instead, which is
// in bounds; those A chunks are zeroed before use.
template <class C>
__device__ __forceinline__ void issue_step(int8_t* stage, const int8_t* const* src,
                                           const int* col, const int* dst, int step,
                                           int64_t k, const GroupScales<C>& gs) {
  const int64_t k0 = static_cast<int64_t>(step) * C::BK;
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int64_t kk = k0 + col[j];
    const int8_t* g = src[j] + (kk < k ? kk : 0);
    __builtin_amdgcn_global_load_lds(g, stage + dst[j], 16, 0, 0);
  }
  if constexpr (C::GS) __builtin_amdgcn_global_load_lds(gs.src + step, stage + gs.slot, 4, 0, 0);
}

// Loads [J0, J1) of issue_step (for spreading a step's loads over several slices).
template <class C, int J0, int J1>
__device__ __forceinline__ void issue_part(int8_t* stage, const int8_t* const* src,
                                           const int* col, const int* dst, int step,
                                           int64_t k, const GroupScales<C>& gs) {
  const int64_t k0 = static_cast<int64_t>(step) * C::BK;
#pragma unroll
  for (int j = J0; j < J1; ++j) {
    const int64_t kk = k0 + col[j];
    const int8_t* g = src[j] + (kk < k ? kk : 0);
    __builtin_amdgcn_global_load_lds(g, stage + dst[j], 16, 0, 0);
  }
  // (the step's scales go with its first part)
  if constexpr (C::GS && J0 == 0)
    __builtin_amdgcn_global_load_lds(gs.src + step, stage + gs.slot, 4, 0, 0);
}

// Read the fragments of 32-k slice `slice` of a step from an LDS stage.
template <class C>
__device__ __forceinline__ void read_slice(const int8_t* stage, int slice, int a_off,
                                           int b_off, int fx, int lane, v4i (&a)[C::TM],
                                           v4i (&b)[C::TN]) {
  const int pofs = ((2 * slice + lane / 32) ^ fx) * 16;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
    a[i] = *reinterpret_cast<const v4i*>(stage + a_off + i * 32 * C::BK + pofs);
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
    b[j] = *reinterpret_cast<const v4i*>(stage + b_off + j * 32 * C::BK + pofs);
}

// FRESH: the slice starts new sums (C operand zero, an inline constant), so a group-scale
// step needs no clearing of the previous step's accumulators.
template <class C, bool FRESH = false>
__device__ __forceinline__ void mfma_slice(const v4i (&a)[C::TM], const v4i (&b)[C::TN],
                                           v16i (&acc)[C::TM][C::TN]) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], FRESH ? v16i{} : acc[i][j],
                                                        0, 0, 0);
}

// Scheduling hint for the instructions just emitted in this basic block: one MFMA of the
// slice whose fragments are already in registers (its operand wait then only covers reads
// issued a slice earlier), then the next slice's TM + TN fragment reads, then the remaining
// MFMAs, which hide the reads' latency.
template <class C, int ID>
__device__ __forceinline__ void reads_under_mfmas() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);                    // MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, C::TM + C::TN, ID);        // DS reads
  __builtin_amdgcn_sched_group_barrier(0x008, C::TM * C::TN - 1, ID);    // MFMAs
}

// The last step of a k that is not a multiple of BK holds `valid` real chunks per row; its
// other A chunks (loaded from the row start) are overwritten with zeros once the step has
// landed.  Ends with the LDS writes drained and a barrier.  (Only used with one k-group.)
template <class C>
__device__ __forceinline__ void zero_tail(int8_t* stage, int valid) {
  const int dead = C::CHUNKS - valid;
  for (int e = threadIdx.x % (64 * C::WAVES); e < C::BM * dead; e += 64 * C::WAVES) {
    const int row = e / dead;
    const int chunk = valid + e % dead;
    *reinterpret_cast<v4i*>(stage + row * C::BK + (chunk ^ swizzle<C::BK>(row)) * 16) =
        v4i{0, 0, 0, 0};
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  bare_barrier();
}

// Slices 1 .. SLICES-1 of step t: each slice's fragments are read while the previous
// slice's MFMAs run.  On return fragment set (SLICES - 1) % 2 holds the last slice.
template <class C>
__device__ __forceinline__ void step_inner(const int8_t* stage, int a_off, int b_off, int fx,
                                           int lane, v4i (&fa)[2][C::TM], v4i (&fb)[2][C::TN],
                                           v16i (&acc)[C::TM][C::TN]) {
  // slice 0 (with group scales it starts the step's own sums)
  read_slice<C>(stage, 1, a_off, b_off, fx, lane, fa[1], fb[1]);
  mfma_slice<C, C::GS>(fa[0], fb[0], acc);
  reads_under_mfmas<C, 0>();
#pragma unroll
  for (int s = 1; s + 1 < C::SLICES; ++s) {
    read_slice<C>(stage, s + 1, a_off, b_off, fx, lane, fa[(s + 1) % 2], fb[(s + 1) % 2]);
    mfma_slice<C>(fa[s % 2], fb[s % 2], acc);
    reads_under_mfmas<C, 0>();
  }
}

// With 3 or more stages the stage refilled during step t (step t + STAGES - 1, into the
// stage freed by the previous barrier) is not needed for two more steps, so its loads are
// spread over the slices of step t, a few between the MFMAs of each slice, instead of
// queueing all at once behind the barrier.
template <class C>
struct Spread {
  static constexpr int kParts = C::SLICES - 1;
  static constexpr int kPer = (C::LOADS + kParts - 1) / kParts;
  static constexpr int lo(int s) { return s * kPer < C::LOADS ? s * kPer : C::LOADS; }
  static constexpr int hi(int s) { return lo(s + 1); }
};

template <class C, int S>
__device__ __forceinline__ void spread_slice(const int8_t* stage, int8_t* fill,
                                             const int8_t* const* src, const int* col,
                                             const int* dst, int fill_step, int64_t k,
                                             int a_off, int b_off, int fx, int lane,
                                             v4i (&fa)[2][C::TM], v4i (&fb)[2][C::TN],
                                             v16i (&acc)[C::TM][C::TN],
                                             const GroupScales<C>& gs) {
  if constexpr (S + 1 < C::SLICES) {
    using P = Spread<C>;
    read_slice<C>(stage, S + 1, a_off, b_off, fx, lane, fa[(S + 1) % 2], fb[(S + 1) % 2]);
    issue_part<C, P::lo(S), P::hi(S)>(fill, src, col, dst, fill_step, k, gs);
    mfma_slice<C, C::GS && S == 0>(fa[S % 2], fb[S % 2], acc);
    constexpr int kLoads = P::hi(S) - P::lo(S) + (C::GS && S == 0 ? 1 : 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);                       // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, C::TM + C::TN, 2);           // DS reads
    if constexpr (kLoads > 0) __builtin_amdgcn_sched_group_barrier(0x020, kLoads, 2);
    __builtin_amdgcn_sched_group_barrier(0x008, C::TM * C::TN - 1, 2);       // MFMAs
    spread_slice<C, S + 1>(stage, fill, src, col, dst, fill_step, k, a_off, b_off, fx, lane,
                           fa, fb, acc, gs);
  }
}

// Scheduling hint after the barrier of a step that refills a stage: one MFMA of the previous
// step's last slice, the next slice's fragment reads, then the direct-to-LDS loads spread
// between the remaining MFMAs.  Issued in one burst, the loads of all wavefronts queue in
// the address unit (64 bytes per clock) and stall each wavefront for hundreds of cycles with
// the matrix cores idle; spread out, the MFMAs cover that wait.
template <class C, int ID>
__device__ __forceinline__ void loads_under_mfmas() {
  constexpr int kMfma = C::TM * C::TN;
  // loads per remaining MFMA (all of them after the first MFMA when it is the only one)
  constexpr int kPer = kMfma > 1 ? (C::LOADS + kMfma - 2) / (kMfma - 1) : C::LOADS;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);                // MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, C::TM + C::TN, ID);    // DS reads
  if constexpr (kMfma == 1) {
    __builtin_amdgcn_sched_group_barrier(0x020, kPer, ID);           // VMEM (LDS DMA) loads
  } else {
#pragma unroll
    for (int i = 0; i + 1 < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x020, kPer, ID);         // VMEM (LDS DMA) loads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);            // MFMA
    }
  }
}

// One steady-state k step t of this k-group's ksteps steps (t + 1 < ksteps; global step
// base + t).  ISSUE: a stage is refilled, with step t + STAGES - 1 spread over this step's
// slices (3 or more stages) or with step t + STAGES right after this step's barrier (2
// stages).  ZERO: step t + 1 is the partial last step.
template <class C, bool ISSUE, bool ZERO>
__device__ __forceinline__ void k_step(int8_t* lds, const int8_t* const* src, const int* col,
                                       const int* dst, int a_off, int b_off, int fx, int lane,
                                       int base, int t, int ksteps, int64_t k, int tail_valid,
                                       v4i (&fa)[2][C::TM], v4i (&fb)[2][C::TN],
                                       v16i (&acc)[C::TM][C::TN], GroupScales<C>& gs) {
  constexpr bool kSpread = C::STAGES >= 3;
  // (the stage of step t holds its scales until step t + 1 refills it, after this step)
  if constexpr (C::GS) gs_read<C>(lds + (t % C::STAGES) * C::STAGE_BYTES, gs, lane);
  if constexpr (ISSUE && kSpread) {
    const int u = t + C::STAGES - 1;
    spread_slice<C, 0>(lds + (t % C::STAGES) * C::STAGE_BYTES,
                       lds + (u % C::STAGES) * C::STAGE_BYTES, src, col, dst, base + u, k,
                       a_off, b_off, fx, lane, fa, fb, acc, gs);
  } else {
    step_inner<C>(lds + (t % C::STAGES) * C::STAGE_BYTES, a_off, b_off, fx, lane, fa, fb, acc);
  }
  int8_t* next = lds + ((t + 1) % C::STAGES) * C::STAGE_BYTES;
  // Keep this step's MFMAs in front of the LDS drain: they do not touch memory, so nothing
  // else stops the scheduler from sinking them below it and waiting on the fresh reads.
  __builtin_amdgcn_sched_barrier(0);
  wait_and_barrier<C::VM>(min(C::STAGES - 2, ksteps - 2 - t));
  if (ZERO && tail_valid != 0) zero_tail<C>(next, tail_valid);
  constexpr int last = (C::SLICES - 1) % 2;  // SLICES is even, so set 0 is free
  if constexpr (ISSUE && !kSpread) {
    // (the fragment reads come first in program order: the loads write LDS, so the compiler
    // keeps reads that follow them in place)
    read_slice<C>(next, 0, a_off, b_off, fx, lane, fa[0], fb[0]);
    issue_step<C>(lds + (t % C::STAGES) * C::STAGE_BYTES, src, col, dst, base + t + C::STAGES,
                  k, gs);
    mfma_slice<C>(fa[last], fb[last], acc);
    loads_under_mfmas<C, 1>();
  } else {
    read_slice<C>(next, 0, a_off, b_off, fx, lane, fa[0], fb[0]);
    mfma_slice<C>(fa[last], fb[last], acc);
    reads_under_mfmas<C, 1>();
  }
  if constexpr (C::GS) gs_apply<C>(acc, gs);
}

// Epilogue through LDS.  A wavefront's accumulators hold one column per lane (32x32 MFMA
// layout: lane l, register r -> row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32), so
// stored straight from registers every instruction writes 2 or 4 bytes per lane.  Instead,
// each wavefront converts one 32-row block and up to two 32-column blocks of output values at
// a time into a private LDS area (32-bit words, rows padded to 72 words so that the two half
// wavefronts, 4 rows apart, write disjoint banks), then reads them back row-contiguous and
// writes 16 bytes per lane (8 bf16 or 4 float32 / int32 values), eight or four lanes per
// 128-byte row segment.  Needs rows of the output that are whole 16-byte chunks
// (n * element size % 16 == 0) and a 16-byte aligned output.
constexpr int kScrWords = 72;                   // words per scratch row (64 + padding)
constexpr int kScrBytes = 32 * kScrWords * 4;   // scratch per wavefront

// GS: the accumulators hold the float32 bits of the weight-scaled sums (the group scales
// were applied per step), so only the token scale and the bias remain.
template <int YT, bool GS>
__device__ __forceinline__ float epilogue_value(int a, float sx, float sw) {
  if constexpr (GS) return __fmul_rn(__int_as_float(a), sx);
  return __fmul_rn(__fmul_rn(static_cast<float>(a), sx), sw);
}

// Copy the epilogue's row scales (rows r0 .. r0 + WTM), column scales (unless GS) and bias
// (if any) of a wavefront's sub-tile into its table `par` (direct-to-LDS, 64 values per
// instruction, indices clamped).  Issued before the first k step's loads, so every later
// wait for those covers it too; int32 output needs none of it.
template <class C, int YT, bool GS>
__device__ __forceinline__ void epi_params(float* par, int lane, const float* __restrict__ x_scale,
                                           const float* __restrict__ w_scale,
                                           const float* __restrict__ bias, int64_t m, int64_t n,
                                           int64_t r0, int64_t c0) {
  if constexpr (YT == I8QL_I32) return;
#pragma unroll
  for (int h = 0; h < C::PAR_RM / 64; ++h) {
    const int64_t r = r0 + h * 64 + lane;
    __builtin_amdgcn_global_load_lds(x_scale + (r < m ? r : m - 1), par + h * 64, 4, 0, 0);
  }
#pragma unroll
  for (int h = 0; h < C::PAR_RN / 64; ++h) {
    const int64_t c = c0 + h * 64 + lane;
    const int64_t cc = c < n ? c : n - 1;
    if constexpr (!GS)
      __builtin_amdgcn_global_load_lds(w_scale + cc, par + C::PAR_RM + h * 64, 4, 0, 0);
    if (bias)
      __builtin_amdgcn_global_load_lds(bias + cc, par + C::PAR_RM + C::PAR_RN + h * 64, 4, 0, 0);
  }
}

// BIAS: bias is not null (a template flag, so that each output value costs no select).
// PAR: the parameters come from the wavefront's table `par` (epi_params, landed), else from
// global memory here.
template <class C, int YT, bool GS, bool BIAS, bool PAR>
__device__ __forceinline__ void epilogue_lds(const v16i (&acc)[C::TM][C::TN], int* scr,
                                             int lane, const float* __restrict__ x_scale,
                                             const float* __restrict__ w_scale,
                                             const float* __restrict__ bias, void* y,
                                             int64_t m, int64_t n, int64_t r0, int64_t c0,
                                             const float* par) {
  constexpr int TM = C::TM, TN = C::TN;
  constexpr int ES = YT == I8QL_BF16 ? 2 : 4;  // output element bytes
  constexpr int PER = 16 / ES;                  // output elements per 16-byte store
  float sw[TN], bj[TN];
  if constexpr (YT != I8QL_I32) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t c = c0 + j * 32 + lane % 32;
      if constexpr (PAR) {
        sw[j] = GS ? 1.0f : par[C::PAR_RM + j * 32 + lane % 32];
        bj[j] = BIAS ? par[C::PAR_RM + C::PAR_RN + j * 32 + lane % 32] : 0.0f;
      } else {
        sw[j] = GS ? 1.0f : w_scale[c < n ? c : n - 1];
        bj[j] = BIAS ? bias[c < n ? c : n - 1] : 0.0f;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float sx[16];
    if constexpr (YT != I8QL_I32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (PAR) {
          sx[r] = par[i * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4];
        } else {
          const int64_t row = r0 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
          sx[r] = x_scale[row < m ? row : m - 1];
        }
      }
    }
#pragma unroll
    for (int jc = 0; jc < TN; jc += 2) {
      const int nb = TN - jc < 2 ? TN - jc : 2;  // 32-column blocks in this piece
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        if (jj >= nb) break;
        const int j = jc + jj;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r / 4) + 4 * (lane / 32) + r % 4;
          int bits;
          if constexpr (YT == I8QL_I32) {
            bits = acc[i][j][r];
          } else {
            float v = epilogue_value<YT, GS>(acc[i][j][r], sx[r], sw[j]);
            if constexpr (BIAS) v = __fadd_rn(v, bj[j]);
            bits = __float_as_int(v);
          }
          scr[row * kScrWords + jj * 32 + lane % 32] = bits;
        }
      }
      const int cpr = nb * 32 / PER;  // 16-byte output chunks per row of this piece
#pragma unroll
      for (int u = 0; u < 32 * 64 / PER / 64; ++u) {  // up to 32 * cpr chunks, 64 per pass
        const int q = u * 64 + lane;
        if (q >= 32 * cpr) break;
        const int row = q / cpr, cg = q % cpr;
        const int* src = scr + row * kScrWords + cg * PER;
        const int64_t rg = r0 + i * 32 + row;
        const int64_t cgl = c0 + jc * 32 + cg * PER;
        if (rg < m && cgl < n) {
          v4i out;
          if constexpr (ES == 4) {
            out = *reinterpret_cast<const v4i*>(src);
          } else {
            const v4i a = *reinterpret_cast<const v4i*>(src);
            const v4i b = *reinterpret_cast<const v4i*>(src + 4);
            const int w8[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              // round to nearest even, two values per instruction (v_cvt_pk_bf16_f32)
              const v2f pair = {__int_as_float(w8[2 * h]), __int_as_float(w8[2 * h + 1])};
              out[h] = __builtin_bit_cast(int, __builtin_convertvector(pair, v2bf));
            }
          }
          *reinterpret_cast<v4i*>(static_cast<char*>(y) + (rg * n + cgl) * ES) = out;
        }
      }
    }
  }
}

// Epilogue straight from registers, for outputs whose rows are not whole 16-byte chunks (or
// a misaligned output).  Per 32-row block the row scales are loaded up front at clamped
// (valid) indices, so that their loads are issued together and waited for once instead of
// once per output row.  (r0, c0): the wavefront's first output row and column.
template <class C, int YT, bool GS>
__device__ __forceinline__ void epilogue_regs(const v16i (&acc)[C::TM][C::TN], int lane,
                                              const float* __restrict__ x_scale,
                                              const float* __restrict__ w_scale,
                                              const float* __restrict__ bias, void* y,
                                              int64_t m, int64_t n, int64_t r0, int64_t c0) {
  constexpr int TM = C::TM, TN = C::TN;
  const int64_t row_base = r0 + 4 * (lane / 32);
  const int64_t col_base = c0 + lane % 32;
  float sw[TN], bj[TN];
  if constexpr (YT != I8QL_I32) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t c = col_base + j * 32;
      sw[j] = GS ? 1.0f : w_scale[c < n ? c : n - 1];
      bj[j] = bias ? bias[c < n ? c : n - 1] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float sx[16];
    if constexpr (YT != I8QL_I32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row_base + i * 32 + 8 * (r / 4) + r % 4;
        sx[r] = x_scale[row < m ? row : m - 1];
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t c = col_base + j * 32;
      if (c >= n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row_base + i * 32 + 8 * (r / 4) + r % 4;
        if (row >= m) continue;
        const int a = acc[i][j][r];
        if constexpr (YT == I8QL_I32) {
          static_cast<int32_t*>(y)[row * n + c] = a;
        } else {
          float v = epilogue_value<YT, GS>(a, sx[r], sw[j]);
          if (bias) v = __fadd_rn(v, bj[j]);
          if constexpr (YT == I8QL_F32) {
            static_cast<float*>(y)[row * n + c] = v;
          } else {
            static_cast<uint16_t*>(y)[row * n + c] = f32_to_bf16_rne(v);
          }
        }
      }
    }
  }
}

// The fused epilogue of a wavefront's accumulators: through LDS with 16-byte stores when the
// output allows it, else from registers.  `scr` is this wavefront's LDS scratch; the caller
// has made sure no wavefront still reads the LDS it overlaps.
template <class C, int YT, bool GS = false, bool PAR = false>
__device__ __forceinline__ void epilogue(const v16i (&acc)[C::TM][C::TN], int* scr, int lane,
                                         const float* __restrict__ x_scale,
                                         const float* __restrict__ w_scale,
                                         const float* __restrict__ bias, void* y, int64_t m,
                                         int64_t n, int64_t r0, int64_t c0,
                                         const float* par = nullptr) {
  constexpr int kES = YT == I8QL_BF16 ? 2 : 4;
  if (n % (16 / kES) == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0) {
    if (bias)
      epilogue_lds<C, YT, GS, true, PAR>(acc, scr, lane, x_scale, w_scale, bias, y, m, n, r0,
                                         c0, par);
    else
      epilogue_lds<C, YT, GS, false, PAR>(acc, scr, lane, x_scale, w_scale, bias, y, m, n, r0,
                                          c0, par);
  } else {
    epilogue_regs<C, YT, GS>(acc, lane, x_scale, w_scale, bias, y, m, n, r0, c0);
  }
}

// XS (KS == 1 only): `splits` > 1 splits k across that many workgroups per output tile,
// each walking an equal share (within one step) of the k steps; `ws` is the workspace of
// splitk_fixup (zero counters on entry; they are zero again on exit).  Without XS the
// fix-up is not compiled in (it would push the largest tiles past the register file) and
// `splits` must be 1.
//
// GS: w_scale holds one scale per (output channel, group of 128 input channels), [n, k / 128]
// (k % 128 == 0); each k step is one group, and its exact int32 partial is converted and
// multiplied by the step's scale into float32 accumulators (see gs_apply).
template <int BM, int BN, int BK, int STAGES, int KS, int WM, int WN, int YT, bool XS,
          bool GS = false>
__global__ __launch_bounds__(64 * WM * WN * KS) void w8a8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int8_t* __restrict__ wq, const float* __restrict__ w_scale,
    const float* __restrict__ bias, void* __restrict__ y, int64_t m, int64_t n, int64_t k,
    int splits_arg, int* __restrict__ ws) {
  static_assert(!XS || KS == 1, "k split across workgroups needs one k-group");
  static_assert(!(XS && GS), "group scales are not combined with a split");
  using C = Cfg<BM, BN, BK, STAGES, KS, WM, WN, GS>;
  const int splits = XS ? splits_arg : 1;
  constexpr int TM = C::TM, TN = C::TN;
  extern __shared__ __attribute__((aligned(16))) int8_t lds_all[];
  __shared__ int last_flag;  // (only used with XS)

  const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
  int64_t tm, tn;
  int split;
  if (!tile_of(tiles_m, tiles_n, splits, tm, tn, split)) return;
  const int64_t m0 = tm * BM;
  const int64_t n0 = tn * BN;

  const int lane = threadIdx.x % 64;
  // (readfirstlane: wavefront-uniform, so per-wave addressing can live in scalar registers)
  const int group = __builtin_amdgcn_readfirstlane(threadIdx.x / (64 * C::WAVES));
  const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x / 64) % C::WAVES);
  const int wm = wave / WN, wn = wave % WN;
  // This workgroup's share of the k steps (all of them without a split); each k-group walks
  // its own equal share of those (KS > 1 only when it divides evenly) in its own LDS stages;
  // all groups pass the same barriers.
  const int64_t total_steps = (k + BK - 1) / BK;
  const int sbeg = static_cast<int>(total_steps * split / splits);
  const int send = static_cast<int>(total_steps * (split + 1) / splits);
  const int ksteps = (send - sbeg) / KS;
  const int base = sbeg + group * ksteps;
  int8_t* lds = lds_all + group * C::GROUP_BYTES;

  // This lane's part of each of the wavefront's load instructions: instruction j covers
  // rows ROWS_PER_LOAD * (wave + WAVES * j) + [0, ROWS_PER_LOAD) of the stacked [A; B] slice.
  const int8_t* src[C::LOADS];
  int col[C::LOADS];
  int dst[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int blk = wave + C::WAVES * j;
    const int trow = blk * C::ROWS_PER_LOAD + lane / C::CHUNKS;  // row of the stacked tile
    const int pchunk = lane % C::CHUNKS;
    col[j] = (pchunk ^ swizzle<BK>(trow)) * 16;
    if (trow < BM)
      src[j] = xq + min(m0 + trow, m - 1) * k;
    else
      src[j] = wq + min(n0 + (trow - BM), n - 1) * k;
    dst[j] = blk * C::ROWS_PER_LOAD * BK;  // wave-uniform LDS offset of the instruction
  }

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
  GroupScales<C> gs;
  if constexpr (GS) {
    // lane l loads the scale of its wavefront sub-tile's column l % WTN (WTN <= 64), which
    // lands at position l of the wavefront's slot: columns j * 32 + lane % 32 are then read
    // back at that position
    const int64_t groups = k / BK;
    gs.src = w_scale + min(n0 + wn * C::WTN + lane % C::WTN, n - 1) * groups;
    gs.slot = C::ROW_BYTES + wave * 256;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) gs.facc[i][j][r] = 0.0f;
  }

  // the epilogue's parameters, copied to LDS past the stages before any step's loads (where
  // they fit: PARAMS), so that the epilogue does not wait for a memory round trip; the first
  // k-group runs the epilogue
  constexpr bool PARAMS = C::params_fit(C::LDS_BYTES);
  float* const par = PARAMS ? reinterpret_cast<float*>(lds_all + C::LDS_BYTES) + wave * C::PAR_WORDS
                            : nullptr;
  if constexpr (PARAMS) {
    if (group == 0)
      epi_params<C, YT, GS>(par, lane, x_scale, w_scale, bias, m, n, m0 + wm * C::WTM,
                            n0 + wn * C::WTN);
  }

  // steps issued ahead of the first: all stages, but with 3 or more stages the last one is
  // filled during step 0
  constexpr int kAhead = STAGES >= 3 ? STAGES - 1 : STAGES;
#pragma unroll
  for (int s = 0; s < kAhead; ++s)
    if (s < ksteps) issue_step<C>(lds + s * C::STAGE_BYTES, src, col, dst, base + s, k, gs);

  const int frow = lane % 32;
  const int fx = swizzle<BK>(frow);  // swizzle of this lane's fragment rows (period 32)
  const int a_off = (wm * C::WTM + frow) * BK;
  const int b_off = (BM + wn * C::WTN + frow) * BK;
  // (the partial last step of k belongs to the last split)
  const int tail_valid =
      KS == 1 && split == splits - 1 ? static_cast<int>((k % BK) / 16) : 0;  // 0: none

  v4i fa[2][TM], fb[2][TN];
  wait_and_barrier<C::VM>(min(kAhead - 1, ksteps - 1));
  if (tail_valid != 0 && ksteps == 1) zero_tail<C>(lds, tail_valid);
  read_slice<C>(lds, 0, a_off, b_off, fx, lane, fa[0], fb[0]);
  int t = 0;
  for (; t + kAhead < ksteps; ++t)
    k_step<C, true, false>(lds, src, col, dst, a_off, b_off, fx, lane, base, t, ksteps, k,
                           tail_valid, fa, fb, acc, gs);
  for (; t + 2 < ksteps; ++t)
    k_step<C, false, false>(lds, src, col, dst, a_off, b_off, fx, lane, base, t, ksteps, k,
                            tail_valid, fa, fb, acc, gs);
  if (t + 1 < ksteps) {
    k_step<C, false, true>(lds, src, col, dst, a_off, b_off, fx, lane, base, t, ksteps, k,
                           tail_valid, fa, fb, acc, gs);
    ++t;
  }
  if constexpr (GS) gs_read<C>(lds + (t % STAGES) * C::STAGE_BYTES, gs, lane);
  step_inner<C>(lds + (t % STAGES) * C::STAGE_BYTES, a_off, b_off, fx, lane, fa, fb, acc);
  mfma_slice<C>(fa[(C::SLICES - 1) % 2], fb[(C::SLICES - 1) % 2], acc);
  if constexpr (GS) {
    gs_apply<C>(acc, gs);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = __float_as_int(gs.facc[i][j][r]);
  }

  if constexpr (KS > 1) {
    // Sum the k-groups' partial tiles in a fixed tree through LDS (int32, exact): in each
    // round the upper half of the groups stores its accumulators and the lower half adds
    // its partner's.  Each wavefront's registers go to a lane-contiguous block.
    constexpr int kRegs = TM * TN * 16;
    int* red = reinterpret_cast<int*>(lds_all);
#pragma unroll
    for (int h = KS / 2; h >= 1; h /= 2) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      bare_barrier();  // every group is done with its LDS stages / the previous round
      if (group >= h && group < 2 * h) {
        int* out = red + ((group - h) * C::WAVES + wave) * kRegs * 64 + lane;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) out[((i * TN + j) * 16 + r) * 64] = acc[i][j][r];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      bare_barrier();
      if (group < h) {
        const int* in = red + (group * C::WAVES + wave) * kRegs * 64 + lane;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] += in[((i * TN + j) * 16 + r) * 64];
      }
    }
    if (group != 0) return;
  }
  if constexpr (XS) {
    if (splits > 1 &&
        !splitk_fixup<C>(acc, ws, tm * tiles_n + tn, split, splits, wave, lane, &last_flag))
      return;
  }

  // ---- fused epilogue ----------------------------------------------------------------
  static_assert(C::RED_BYTES + C::WAVES * kScrBytes <= C::LDS_BYTES, "epilogue scratch");
  if constexpr (KS == 1) {
    // every wavefront is done reading the stages before any scratch is written
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bare_barrier();
  }
  epilogue<C, YT, GS, PARAMS>(acc,
                              reinterpret_cast<int*>(lds_all + C::RED_BYTES + wave * kScrBytes),
                              lane, x_scale, w_scale, bias, y, m, n, m0 + wm * C::WTM,
                              n0 + wn * C::WTN, par);
}

// ---- persistent variant (two stages of both operands, one k-group) ---------------------
// With 128 KiB of stages a compute unit holds one workgroup, so a kernel that ends with its
// tile idles the matrix cores twice per tile: while the first stage's loads travel (the next
// workgroup starts from empty stages) and while the epilogue converts and writes the output.
// At 16384 x 24576 x 4096 with 256 x 256 tiles that is about 12 us of a 63 us round (time
// against k: 1.59 us per k step plus a fixed 12 us per round of 256 tiles).  Here each
// workgroup walks tiles v, v + G, ... (G workgroups, a multiple of the 8 XCDs, so a workgroup
// stays on its XCD's share of the tile order) and keeps the two-stage pipeline running
// across tiles: during the second-to-last k step the freed stage is refilled with the next
// tile's step 0, and after the last step's fragment reads (and a barrier) the last stage is
// refilled with its step 1, so those loads travel while the epilogue runs.  The epilogue
// therefore cannot use the stages: it goes through a small per-wavefront area after them
// (16 rows x 32 columns of 32-bit values at a time) with the tile's row scales, column scales
// and bias copied there by direct-to-LDS loads when the tile starts.  Its output stores are
// buffer stores: stores of rows past m or columns past n are sent past the buffer's end,
// where the hardware drops them.  The last tile refills from itself (in-bounds loads of no
// use) and the kernel drains every load before it ends.  Needs k > BK (two steps at least), output rows of whole
// 16-byte chunks and a 16-byte aligned output.
constexpr int kPScrWords = 64;                  // words per scratch row (swizzled)
constexpr int kPScrBytes = 8 * kPScrWords * 4;  // 8 rows of output values

// Word of value (row, col) of an 8 x 64 piece in the scratch, by 4-word chunks.  A row's
// 16-byte reads (8 or 16 lanes per row) take chunks 2c, 2c + 1 or c: flipping bit 0 of the
// chunks with bit 3 set puts each read's chunks on distinct banks of 32; rows 2s and 2s + 1
// (read in one pass of 64 banks) differ in bit 0 of the chunk, and rows r and r + 4
// (written by the two halves of one instruction) in bit 3.
__device__ __forceinline__ int pscr_word(int row, int col) {
  int c = col >> 2;
  c ^= (c >> 3) & 1;
  c ^= (row & 1) ^ (((row >> 2) & 1) << 3);
  return row * kPScrWords + c * 4 + (col & 3);
}

template <class C, int YT>
struct Persist {
  static constexpr int ES = YT == I8QL_BF16 ? 2 : 4;  // output element bytes
  static constexpr int PER = 16 / ES;                  // output elements per 16-byte store
  static constexpr int PIECE_STORES = 8 * 64 / PER / 64;   // per 8 x 64 piece and lane
  static constexpr int PARAM_BYTES = (C::WTM + 2 * C::WTN) * 4;    // row scales, col scales, bias
  static constexpr int WAVE_BYTES = kPScrBytes + PARAM_BYTES;
  static constexpr size_t STAGES_BYTES = 2 * static_cast<size_t>(C::STAGE_BYTES);
  static constexpr size_t LDS_BYTES = STAGES_BYTES + static_cast<size_t>(C::WAVES) * WAVE_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS per workgroup");
  static_assert(C::WTM % 64 == 0 && C::WTN % 64 == 0, "parameter copies of 64 values");
};

// Copy this wavefront's row scales, column scales and bias (if any) for the tile at (r0, c0)
// into `par` (direct-to-LDS, 64 values per instruction; indices clamped).  Int32
// output uses none of them (and the scales may then be null): nothing is loaded.
template <class C, int YT>
__device__ __forceinline__ void persist_params(float* par, int lane,
                                               const float* __restrict__ x_scale,
                                               const float* __restrict__ w_scale,
                                               const float* __restrict__ bias, int64_t m,
                                               int64_t n, int64_t r0, int64_t c0) {
  if constexpr (YT == I8QL_I32) return;
#pragma unroll
  for (int h = 0; h < C::WTM / 64; ++h) {
    const int64_t r = r0 + h * 64 + lane;
    __builtin_amdgcn_global_load_lds(x_scale + (r < m ? r : m - 1), par + h * 64, 4, 0, 0);
  }
#pragma unroll
  for (int h = 0; h < C::WTN / 64; ++h) {
    const int64_t c = c0 + h * 64 + lane;
    const int64_t cc = c < n ? c : n - 1;
    __builtin_amdgcn_global_load_lds(w_scale + cc, par + C::WTM + h * 64, 4, 0, 0);
    if (bias) __builtin_amdgcn_global_load_lds(bias + cc, par + C::WTM + C::WTN + h * 64, 4, 0, 0);
  }
}

// The fused epilogue of the persistent kernel: 8 x 64 pieces through `scr` (every store
// instruction writes whole 128-byte lines of bf16 rows), scales and bias from `par`, output
// through the buffer resource `yr` over the tile's rows (rows past m lie past its end).
// (r0, c0): the wavefront's first row and column relative to the tile's first row and in
// the whole output.  The lane's scales and biases are read once.  A piece's reads follow its
// writes, and the next piece's writes its reads, without a wait: the LDS executes one
// wavefront's instructions in issue order.  BIAS: the tile has a bias.
template <class C, int YT, bool BIAS>
__device__ __forceinline__ void persist_epilogue(const v16i (&acc)[C::TM][C::TN],
                                                 int8_t* lds_all, int area, int lane,
                                                 __amdgpu_buffer_rsrc_t yr, int64_t n,
                                                 int r0, int64_t c0) {
  using P = Persist<C, YT>;
  static_assert(C::TN % 2 == 0, "pieces of two 32-column blocks");
  // (the area's offset is opaque, so that the compiler derives the scratch and parameter
  // addresses here instead of holding them in registers across the tile loop)
  asm volatile("" : "+s"(area));
  asm volatile("" : "+v"(lane));
  int* scr = reinterpret_cast<int*>(lds_all + area);
  const float* par = reinterpret_cast<const float*>(lds_all + area + kPScrBytes);
  constexpr int PER = P::PER;
  constexpr int CPR = 64 / PER;  // 16-byte chunks per row of a piece
  // register 4g + q of a 32 x 32 block holds row 8g + 4(lane / 32) + q
  float sx[C::TM][4][4], sw[C::TN], bj[C::TN];
  if constexpr (YT != I8QL_I32) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f t = *reinterpret_cast<const v4f*>(par + i * 32 + 8 * g + 4 * (lane / 32));
#pragma unroll
        for (int q = 0; q < 4; ++q) sx[i][g][q] = t[q];
      }
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      sw[j] = par[C::WTM + j * 32 + lane % 32];
      bj[j] = BIAS ? par[C::WTM + C::WTN + j * 32 + lane % 32] : 0.0f;
    }
  }
  const int nb = static_cast<int>(n) * P::ES;  // bytes per output row
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int jp = 0; jp < C::TN / 2; ++jp) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = 2 * jp + jj;
            const int row = 4 * (lane / 32) + q;  // within the piece
            int bits;
            if constexpr (YT == I8QL_I32) {
              bits = acc[i][j][4 * g + q];
            } else {
              float v = epilogue_value<YT, false>(acc[i][j][4 * g + q], sx[i][g][q], sw[j]);
              if constexpr (BIAS) v = __fadd_rn(v, bj[j]);
              bits = __float_as_int(v);
            }
            scr[pscr_word(row, jj * 32 + lane % 32)] = bits;
          }
#pragma unroll
        for (int u = 0; u < P::PIECE_STORES; ++u) {
          const int qq = u * 64 + lane;
          const int row = qq / CPR, cg = qq % CPR;
          v4i out;
          if constexpr (P::ES == 4) {
            out = *reinterpret_cast<const v4i*>(scr + pscr_word(row, cg * PER));
          } else {
            const v4i a = *reinterpret_cast<const v4i*>(scr + pscr_word(row, cg * PER));
            const v4i b = *reinterpret_cast<const v4i*>(scr + pscr_word(row, cg * PER + 4));
            const int w8[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const v2f pair = {__int_as_float(w8[2 * e]), __int_as_float(w8[2 * e + 1])};
              out[e] = __builtin_bit_cast(int, __builtin_convertvector(pair, v2bf));
            }
          }
          const int64_t col = c0 + jp * 64 + cg * PER;
          // (r0 + BM) * n * ES < 2^31: checked at launch)
          const int off = (r0 + i * 32 + 8 * g + row) * nb + static_cast<int>(col) * P::ES;
          const int voff = col < n ? off : -16;  // (past the end: dropped)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, out), yr, voff, 0, 0);
        }
      }
}

// Operand rows of the persistent kernel, read through buffer resources over xq ([m, k]) and
// wq ([n, k]).  Load j of a wavefront covers stacked rows ROWS_PER_LOAD * (wave + WAVES * j)
// + lrow (lrow = lane / CHUNKS): A rows for the first BM / (WAVES * ROWS_PER_LOAD) loads,
// then B rows.  A multiple of 32 rows apart, they share this lane's swizzled chunk offset
// `colb`, so a lane's offset for load j is its (clamped) row times k plus colb, and step s
// adds s * BK as the scalar offset: no address arithmetic per step.  Chunks past k read the
// next row's codes (or zeros past the buffer's end): the A chunks are zeroed in LDS before
// use, so whatever B holds there adds nothing.
template <class C>
__device__ __forceinline__ void persist_offsets(int (&voff)[C::LOADS], int64_t m0, int64_t n0,
                                                int64_t m, int64_t n, int64_t k, int wave,
                                                int lrow, int colb) {
  constexpr int kRowsPerRound = C::WAVES * C::ROWS_PER_LOAD;
  static_assert(kRowsPerRound % 32 == 0 && C::BM % kRowsPerRound == 0, "load rows");
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int trow = (wave + C::WAVES * j) * C::ROWS_PER_LOAD + lrow;
    const int64_t row = j < C::BM / kRowsPerRound ? min(m0 + trow, m - 1)
                                                   : min(n0 + (trow - C::BM), n - 1);
    voff[j] = static_cast<int>(row * k) + colb;
  }
}

template <class C>
__device__ __forceinline__ void persist_issue(int8_t* stage, __amdgpu_buffer_rsrc_t ra,
                                              __amdgpu_buffer_rsrc_t rb,
                                              const int (&voff)[C::LOADS], int wave, int step) {
  constexpr int kRowsPerRound = C::WAVES * C::ROWS_PER_LOAD;
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    int8_t* d = stage + (wave + C::WAVES * j) * C::ROWS_PER_LOAD * C::BK;
    __attribute__((address_space(3))) void* dl = (__attribute__((address_space(3))) void*)d;
    const __amdgpu_buffer_rsrc_t r = j < C::BM / kRowsPerRound ? ra : rb;
    const int vo = voff[j];
    // (builtin arguments are named values: clang rejects a value-dependent expression
    // written directly into this builtin's argument list)
    const int so = step * C::BK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dl, 16, vo, so, 0, 0);
  }
}

// One steady k step of the persistent kernel: compute the step in `cur`, wait for the step
// in `nxt` and barrier (optionally zero its tail), read its first slice, refill `cur` with
// step `fstep` of the rows at offsets `fvoff`, and finish this step's last slice.
template <class C, bool ZERO>
__device__ __forceinline__ void persist_step(int8_t* cur, int8_t* nxt, __amdgpu_buffer_rsrc_t ra,
                                             __amdgpu_buffer_rsrc_t rb,
                                             const int (&fvoff)[C::LOADS], int wave, int fstep,
                                             int tail_valid, int a_off, int b_off, int fx,
                                             int lane, v4i (&fa)[2][C::TM], v4i (&fb)[2][C::TN],
                                             v16i (&acc)[C::TM][C::TN]) {
  step_inner<C>(cur, a_off, b_off, fx, lane, fa, fb, acc);
  __builtin_amdgcn_sched_barrier(0);
  wait_and_barrier<C::VM>(0);
  if (ZERO && tail_valid != 0) zero_tail<C>(nxt, tail_valid);
  constexpr int last = (C::SLICES - 1) % 2;
  read_slice<C>(nxt, 0, a_off, b_off, fx, lane, fa[0], fb[0]);
  persist_issue<C>(cur, ra, rb, fvoff, wave, fstep);
  mfma_slice<C>(fa[last], fb[last], acc);
  loads_under_mfmas<C, 1>();
}

template <int BM, int BN, int BK, int WM, int WN, int YT>
__global__ __launch_bounds__(64 * WM * WN) void w8a8_kernel_persistent(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int8_t* __restrict__ wq, const float* __restrict__ w_scale,
    const float* __restrict__ bias, void* __restrict__ y, int64_t m, int64_t n, int64_t k) {
  using C = Cfg<BM, BN, BK, 2, 1, WM, WN>;
  using P = Persist<C, YT>;
  constexpr int TM = C::TM, TN = C::TN;
  extern __shared__ __attribute__((aligned(16))) int8_t lds_all[];
  const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
  const int64_t total = tiles_m * tiles_n;
  const int64_t G = gridDim.x;
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int wm = wave / WN, wn = wave % WN;
  const int area = static_cast<int>(P::STAGES_BYTES) + wave * P::WAVE_BYTES;  // scratch, params
  const int ksteps = static_cast<int>((k + BK - 1) / BK);  // >= 2
  const int tail_valid = static_cast<int>((k % BK) / 16);  // 0: none

  // Tile id v in [0, vend): (m0, n0) in the XCD-contiguous grouped order of tile_of, or
  // false for the ids of the per-XCD ranges' padding (total % 8 != 0).  With G a multiple of
  // 8, the ids v, v + G, ... of a workgroup all belong to its XCD.
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t vend = per_xcd * kXcds;
  auto tile_at = [&](int64_t v, int64_t& m0, int64_t& n0) -> bool {
    // (opaque divisors: their division sequences are not hoisted into registers held
    // across the tile loop)
    int64_t pxc = per_xcd, tn_ = tiles_n, tm_ = tiles_m;
    asm volatile("" : "+s"(pxc), "+s"(tn_), "+s"(tm_));
    const int64_t u = (v % kXcds) * pxc + v / kXcds;
    if (u >= total) return false;
    const int64_t grp = u / (kGroupM * tn_);
    const int64_t first_m = grp * kGroupM;
    const int64_t gsize = min(tm_ - first_m, static_cast<int64_t>(kGroupM));
    const int64_t in_group = u % (kGroupM * tn_);
    m0 = (first_m + in_group % gsize) * BM;
    n0 = (in_group / gsize) * BN;
    return true;
  };
  const int lrow = lane / C::CHUNKS;
  const int colb = ((lane % C::CHUNKS) ^ swizzle<BK>(wave * C::ROWS_PER_LOAD + lrow)) * 16;
  // the first tile of this workgroup
  int64_t v = blockIdx.x;
  int64_t m0 = 0, n0 = 0;
  while (v < vend && !tile_at(v, m0, n0)) v += G;
  if (v >= vend) return;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(xq), 0, static_cast<int>(m * k), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(wq), 0, static_cast<int>(n * k), 0x00020000);
  int voff[C::LOADS];
  persist_offsets<C>(voff, m0, n0, m, n, k, wave, lrow, colb);
  int sbase = 0;  // stage of the tile's step 0
  persist_issue<C>(lds_all, ra, rb, voff, wave, 0);
  persist_issue<C>(lds_all + C::STAGE_BYTES, ra, rb, voff, wave, 1);

  const int frow = lane % 32;
  const int fx = swizzle<BK>(frow);
  const int a_off = (wm * C::WTM + frow) * BK;
  const int b_off = (BM + wn * C::WTN + frow) * BK;
  constexpr int last = (C::SLICES - 1) % 2;
  while (true) {
    // the next valid tile (or this one again: its loads are in bounds and never used)
    int64_t vn = v + G, nm0 = m0, nn0 = n0;
    while (vn < vend && !tile_at(vn, nm0, nn0)) vn += G;
    const bool has_next = vn < vend;
    if (!has_next) {
      nm0 = m0;
      nn0 = n0;
    }
    int nvoff[C::LOADS];
    persist_offsets<C>(nvoff, nm0, nn0, m, n, k, wave, lrow, colb);
    auto st = [&](int t) { return lds_all + ((sbase + t) & 1) * C::STAGE_BYTES; };

    // Step 0 has landed once at most VM operations are outstanding: loads complete in issue
    // order, so while step 0's were outstanding step 1's (issued later) would be too.  (The
    // previous epilogue's stores count as well and may complete in any order relative to
    // the loads, so the count cannot leave them out; they are waited for too.)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::VM, 15));
    bare_barrier();
    persist_params<C, YT>(reinterpret_cast<float*>(lds_all + area + kPScrBytes), lane, x_scale,
                      w_scale, bias, m, n, m0 + wm * C::WTM, n0 + wn * C::WTN);
    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    v4i fa[2][TM], fb[2][TN];
    read_slice<C>(st(0), 0, a_off, b_off, fx, lane, fa[0], fb[0]);
    int t = 0;
    for (; t + 2 < ksteps; ++t)
      persist_step<C, false>(st(t), st(t + 1), ra, rb, voff, wave, t + 2, tail_valid, a_off,
                             b_off, fx, lane, fa, fb, acc);
    // second-to-last step: the freed stage takes the next tile's step 0
    persist_step<C, true>(st(t), st(t + 1), ra, rb, nvoff, wave, 0, tail_valid, a_off, b_off,
                          fx, lane, fa, fb, acc);
    ++t;
    // last step: once every wavefront has read its fragments, its stage takes the next
    // tile's step 1
    step_inner<C>(st(t), a_off, b_off, fx, lane, fa, fb, acc);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bare_barrier();
    persist_issue<C>(st(t), ra, rb, nvoff, wave, 1);
    mfma_slice<C>(fa[last], fb[last], acc);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const int64_t rows = min(static_cast<int64_t>(BM), m - m0);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(y) + m0 * n * P::ES, 0, static_cast<int>(rows * n * P::ES),
        0x00020000);
    if (bias)
      persist_epilogue<C, YT, true>(acc, lds_all, area, lane, yr, n, wm * C::WTM,
                                    n0 + wn * C::WTN);
    else
      persist_epilogue<C, YT, false>(acc, lds_all, area, lane, yr, n, wm * C::WTM,
                                     n0 + wn * C::WTN);
    if (!has_next) break;
    v = vn;
    m0 = nm0;
    n0 = nn0;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) voff[j] = nvoff[j];
    sbase = (sbase + ksteps) & 1;
  }
  // the last tile's refills and stores: nothing may land in LDS after the workgroup ends
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
}

// ---- two LDS slots for A, three for B ---------------------------------------------------
// With two stages of both operands only one step of loads is in flight while a step
// computes, and the weight rows (read once from HBM) arrive late.  A third stage of both
// does not fit in LDS for the large tiles, but a third one of B alone does (256x256: 2 x 32 +
// 3 x 32 KiB; 256x192: 136 KiB; 128x320: 152 KiB).  Step t computes from A slot t % 2 and B
// slot t % 3; after the barrier that ends step t the workgroup refills A slot t % 2 with step
// t + 2 and B slot t % 3 with step t + 3, in that order, so the weight loads have two steps
// to land and the activation loads one.  At the end of step u the only loads allowed to be
// outstanding are then B(u + 2)'s.  Measured on MI355X against the same tile with two
// stages of both: 4-20 % faster for 256x192 and 10-25 % for 128x320 over 44 shapes; for
// 256x256 it helps long-k and few-row shapes but costs 2-3 % on large ones, which keep the
// symmetric kernel.
template <class C>
struct SplitStages {
  static constexpr int LA = C::BM / C::ROWS_PER_LOAD / C::WAVES;  // A loads per wave per step
  static constexpr int LB = C::LOADS - LA;                         // B loads per wave per step
  static constexpr int A_BYTES = C::BM * C::BK;
  static constexpr int B_BYTES = C::BN * C::BK;
  static constexpr size_t LDS_BYTES = 2 * static_cast<size_t>(A_BYTES) +
                                      3 * static_cast<size_t>(B_BYTES);
  static_assert(LA * C::ROWS_PER_LOAD * C::WAVES == C::BM, "A rows split evenly over waves");
  static_assert(2 * LB + LA <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS per workgroup");
  static_assert(C::WAVES * kScrBytes <= LDS_BYTES, "epilogue scratch");
};

// Loads [J0, J1) of a step into one operand's slot (dst offsets relative to that slot).
template <class C, int J0, int J1>
__device__ __forceinline__ void issue_rows(int8_t* slot, const int8_t* const* src,
                                           const int* col, const int* dst, int step,
                                           int64_t k) {
  const int64_t k0 = static_cast<int64_t>(step) * C::BK;
#pragma unroll
  for (int j = J0; j < J1; ++j) {
    const int64_t kk = k0 + col[j];
    const int8_t* g = src[j] + (kk < k ? kk : 0);
    __builtin_amdgcn_global_load_lds(g, slot + dst[j], 16, 0, 0);
  }
}

// LDS drain, wait until at most `outstanding` loads of this wavefront are in flight, barrier.
template <int OUTSTANDING>
__device__ __forceinline__ void drain_wait_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(OUTSTANDING, 15));
  bare_barrier();
}

template <int BM, int BN, int BK, int WM, int WN, int YT>
__global__ __launch_bounds__(64 * WM * WN) void w8a8_kernel_split(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int8_t* __restrict__ wq, const float* __restrict__ w_scale,
    const float* __restrict__ bias, void* __restrict__ y, int64_t m, int64_t n, int64_t k) {
  using C = Cfg<BM, BN, BK, 2, 1, WM, WN>;
  using P = SplitStages<C>;
  constexpr int TM = C::TM, TN = C::TN;
  extern __shared__ __attribute__((aligned(16))) int8_t lds_all[];

  int64_t tm, tn;
  int split;
  if (!tile_of((m + BM - 1) / BM, (n + BN - 1) / BN, 1, tm, tn, split)) return;
  const int64_t m0 = tm * BM;
  const int64_t n0 = tn * BN;
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int wm = wave / WN, wn = wave % WN;
  const int ksteps = static_cast<int>((k + BK - 1) / BK);
  int8_t* const aslots = lds_all;
  int8_t* const bslots = lds_all + 2 * P::A_BYTES;

  // Load instruction j covers rows ROWS_PER_LOAD * (wave + WAVES * j) + [0, ROWS_PER_LOAD) of
  // the stacked [A; B] slice; the first LA instructions are A rows, the rest B rows.
  const int8_t* src[C::LOADS];
  int col[C::LOADS];
  int dst[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int blk = wave + C::WAVES * j;
    const int trow = blk * C::ROWS_PER_LOAD + lane / C::CHUNKS;
    col[j] = ((lane % C::CHUNKS) ^ swizzle<BK>(trow)) * 16;
    if (j < P::LA) {
      src[j] = xq + min(m0 + trow, m - 1) * k;
      dst[j] = blk * C::ROWS_PER_LOAD * BK;
    } else {
      src[j] = wq + min(n0 + (trow - BM), n - 1) * k;
      dst[j] = (blk * C::ROWS_PER_LOAD - BM) * BK;
    }
  }

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // prologue: A0 B0, then B1 A1 B2 (B1 before A1, so that A1 landing implies B1 has)
  constexpr bool PARAMS = C::params_fit(P::LDS_BYTES);
  float* const par = PARAMS ? reinterpret_cast<float*>(lds_all + P::LDS_BYTES) + wave * C::PAR_WORDS
                            : nullptr;
  if constexpr (PARAMS)
    epi_params<C, YT, false>(par, lane, x_scale, w_scale, bias, m, n, m0 + wm * C::WTM,
                             n0 + wn * C::WTN);
  issue_rows<C, 0, P::LA>(aslots, src, col, dst, 0, k);
  issue_rows<C, P::LA, C::LOADS>(bslots, src, col, dst, 0, k);
  if (ksteps > 1) {
    issue_rows<C, P::LA, C::LOADS>(bslots + P::B_BYTES, src, col, dst, 1, k);
    issue_rows<C, 0, P::LA>(aslots + P::A_BYTES, src, col, dst, 1, k);
  }
  if (ksteps > 2) issue_rows<C, P::LA, C::LOADS>(bslots + 2 * P::B_BYTES, src, col, dst, 2, k);

  const int frow = lane % 32;
  const int fx = swizzle<BK>(frow);
  const int a_off = (wm * C::WTM + frow) * BK;
  const int b_rel = (wn * C::WTN + frow) * BK;
  const int tail_valid = static_cast<int>((k % BK) / 16);  // 0: none
  // fragment reads address step t's B rows from its A slot
  auto b_off = [&](int t) {
    return static_cast<int>((bslots + (t % 3) * P::B_BYTES) - (aslots + (t % 2) * P::A_BYTES)) +
           b_rel;
  };
  auto a_slot = [&](int t) { return aslots + (t % 2) * P::A_BYTES; };

  if (ksteps > 2) {
    drain_wait_barrier<2 * P::LB + P::LA>();
  } else if (ksteps == 2) {
    drain_wait_barrier<P::LB + P::LA>();
  } else {
    drain_wait_barrier<0>();
  }
  if (tail_valid != 0 && ksteps == 1) zero_tail<C>(aslots, tail_valid);
  v4i fa[2][TM], fb[2][TN];
  read_slice<C>(aslots, 0, a_off, b_off(0), fx, lane, fa[0], fb[0]);
  constexpr int last = (C::SLICES - 1) % 2;  // SLICES is even, so set 0 is free
  int t = 0;
  // steady state: refill A(t + 2) and B(t + 3)
  for (; t + 3 < ksteps; ++t) {
    step_inner<C>(a_slot(t), a_off, b_off(t), fx, lane, fa, fb, acc);
    __builtin_amdgcn_sched_barrier(0);
    drain_wait_barrier<P::LB>();
    read_slice<C>(a_slot(t + 1), 0, a_off, b_off(t + 1), fx, lane, fa[0], fb[0]);
    issue_rows<C, 0, P::LA>(a_slot(t), src, col, dst, t + 2, k);
    issue_rows<C, P::LA, C::LOADS>(bslots + (t % 3) * P::B_BYTES, src, col, dst, t + 3, k);
    mfma_slice<C>(fa[last], fb[last], acc);
    loads_under_mfmas<C, 1>();
  }
  // t = ksteps - 3: refill A only
  if (t + 2 < ksteps) {
    step_inner<C>(a_slot(t), a_off, b_off(t), fx, lane, fa, fb, acc);
    __builtin_amdgcn_sched_barrier(0);
    drain_wait_barrier<P::LB>();
    read_slice<C>(a_slot(t + 1), 0, a_off, b_off(t + 1), fx, lane, fa[0], fb[0]);
    issue_rows<C, 0, P::LA>(a_slot(t), src, col, dst, t + 2, k);
    mfma_slice<C>(fa[last], fb[last], acc);
    reads_under_mfmas<C, 1>();
    ++t;
  }
  // t = ksteps - 2: nothing left to load; the last step may be partial
  if (t + 1 < ksteps) {
    step_inner<C>(a_slot(t), a_off, b_off(t), fx, lane, fa, fb, acc);
    __builtin_amdgcn_sched_barrier(0);
    drain_wait_barrier<0>();
    if (tail_valid != 0) zero_tail<C>(a_slot(t + 1), tail_valid);
    read_slice<C>(a_slot(t + 1), 0, a_off, b_off(t + 1), fx, lane, fa[0], fb[0]);
    mfma_slice<C>(fa[last], fb[last], acc);
    reads_under_mfmas<C, 1>();
    ++t;
  }
  step_inner<C>(a_slot(t), a_off, b_off(t), fx, lane, fa, fb, acc);
  mfma_slice<C>(fa[(C::SLICES - 1) % 2], fb[(C::SLICES - 1) % 2], acc);

  // every wavefront is done reading the slots before any scratch is written
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  bare_barrier();
  epilogue<C, YT, false, PARAMS>(acc, reinterpret_cast<int*>(lds_all + wave * kScrBytes), lane,
                                 x_scale, w_scale, bias, y, m, n, m0 + wm * C::WTM,
                                 n0 + wn * C::WTN, par);
}

template <int BM, int BN, int BK, int YT, int WM, int WN>
hipError_t launch_split(const int8_t* xq, const float* x_scale, const int8_t* wq,
                        const float* w_scale, const float* bias, void* y, int64_t m, int64_t n,
                        int64_t k, hipStream_t stream) {
  using C = Cfg<BM, BN, BK, 2, 1, WM, WN>;
  using P = SplitStages<C>;
  constexpr auto kern = w8a8_kernel_split<BM, BN, BK, WM, WN, YT>;
  constexpr size_t kLds = C::params_fit(P::LDS_BYTES) ? P::LDS_BYTES + C::PAR_BYTES : P::LDS_BYTES;
  const hipError_t e = allow_dynamic_lds<kern>(static_cast<int>(kLds));
  if (e != hipSuccess) return e;
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(C::THREADS), kLds,
                     stream, xq, x_scale, wq, w_scale, bias, y, m, n, k);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int STAGES, int KS, int YT, int WM, int WN, bool XS,
          bool GS = false>
hipError_t launch_cfg(const int8_t* xq, const float* x_scale, const int8_t* wq,
                      const float* w_scale, const float* bias, void* y, int64_t m, int64_t n,
                      int64_t k, int splits, int* ws, hipStream_t stream) {
  using C = Cfg<BM, BN, BK, STAGES, KS, WM, WN, GS>;
  constexpr auto kern = w8a8_kernel<BM, BN, BK, STAGES, KS, WM, WN, YT, XS, GS>;
  // (the parameter table past the stages where it fits, as the kernel decides)
  constexpr size_t kLds = C::params_fit(C::LDS_BYTES) ? C::LDS_BYTES + C::PAR_BYTES : C::LDS_BYTES;
  const hipError_t e = allow_dynamic_lds<kern>(static_cast<int>(kLds));
  if (e != hipSuccess) return e;
  const int64_t units = ((m + BM - 1) / BM) * ((n + BN - 1) / BN) * splits;
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(C::THREADS), kLds,
                     stream, xq, x_scale, wq, w_scale, bias, y, m, n, k, splits, ws);
  return hipGetLastError();
}

// Tile configuration by a cost model.  Every configuration computes the same products; they
// differ in how well one shape fills the 256 CUs and in how many loaded bytes each MFMA
// costs.  Large tiles load fewer bytes per MFMA, but a shape whose tile count is just above a
// multiple of the CU count leaves most CUs idle in its last round, so tile shapes that are not
// powers of two (192, 160 and 320 wide) are candidates too, as are small tiles whose k is split
// between k-groups inside the workgroup (few tiles, long k).  A launch's time is modelled as
//   t = t_step * R * S + t_round * R + t0,   R = ceil(tiles / CUs), S = k steps per k-group,
// one workgroup per CU and round; the coefficients (us) are a least-squares fit (relative
// error) to graph-timed MI355X measurements of every candidate on 44 shapes (M 16..16384,
// N 1024..28672, K 1024..18944, bf16 output).  On those shapes the chosen configurations
// take 0.9% longer in total than the per-shape best, also when each shape is predicted from
// a fit that left it out.  Examples (us): 2048x19456x2560 106 with 256x320 tiles (256x256:
// 2 rounds + 96 tiles, 3 rounds), 2048x6144x2560 37 with 256x192 (256 tiles, one round),
// 2048x2560x9728 56 with 128x160 (256 tiles), 16384x12288x4096 750-765 with 256x256 or
// 320x256.
//
// Configurations with one k-group per workgroup can also split k across P workgroups per
// tile (a plan (configuration, P)); then R counts tiles * P units, S is the steps of one
// split, and the fix-up (partial tiles through the workspace, summed by the last arrival)
// adds t_fix = f0 + f1 * P * BM * BN / 16384, fitted (relative error) to graph-timed MI355X
// sweeps of every plan on 45 shapes (M 128..2048, N 1024..24576, K 2560..12288, weights
// rotating beyond the Infinity Cache): the model's picks take 0.12% longer in total than the
// per-shape best, also with each shape predicted by a fit that left it out.  A split wins on
// the long-k shapes: 512 x 2560 x 9728 27.6 us with 128 x 128 tiles and 3 splits (33.6
// without), 128 x 2560 x 9728 15.1 us with 64 x 64 tiles and 3 splits (18.8).
//
// Group-scale products (w8a8_gemm_g128) run on the configurations marked `gs`: one k-group,
// spread refills (3 or more stages) and wavefront sub-tiles at most 64 columns wide, so that
// one dword load per wavefront carries a step's scales.  They use the same model with each
// step's time scaled by kGsStep (the per-step conversion and fused multiply-add of the int32
// partials).
struct Candidate {
  int bm, bn, ks;                // tile and k-groups
  bool xsplit;                   // k may be split across workgroups
  bool gs;                       // runs group-scale products
  double t_step, t_round, t0;    // cost model (us)
};
constexpr Candidate kCandidates[] = {
    {256, 256, 1, true, false, 1.3616, 21.063, -10.348},   // 0: 2 stages, 8 wavefronts 64x128
    {256, 320, 1, false, false, 1.5576, 27.308, -14.718},  // 1: 2 stages, 8 wavefronts 64x160
    {256, 192, 1, false, false, 1.0216, 17.150, -7.651},   // 2: 2 A + 3 B slots, 8 waves 64x96
    {128, 320, 1, false, false, 0.9822, 13.467, -3.992},   // 3: 2 A + 3 B slots, 8 waves 32x160
    {128, 160, 1, true, false, 0.5742, 7.669, 0.439},      // 4: 3 stages, 4 wavefronts 32x160
    {256, 128, 1, true, true, 0.7426, 12.247, -6.637},     // 5: 3 stages, 8 wavefronts 64x64
    {128, 128, 1, true, true, 0.5263, 5.399, 0.071},       // 6: 3 stages, 8 wavefronts 64x32
    {128, 64, 2, false, false, 0.6945, 4.216, 0.586},      // 7: 3 stages, 2 k-groups of 4 waves
    {64, 64, 2, false, false, 0.4855, 2.353, 2.777},       // 8: 3 stages, 2 k-groups of 4 waves
    {64, 32, 4, false, false, 0.6247, 2.558, 2.713},       // 9: 3 stages, 4 k-groups of 2 waves
    {64, 64, 1, true, true, 0.2183, 0.705, 5.779},         // 10: 4 stages, 4 wavefronts
    {320, 256, 1, false, false, 1.5310, 26.719, -12.773},  // 11: 2 stages, 8 wavefronts 160x64
};
constexpr double kGsStep = 1.0;  // step-time factor of group-scale products
// Configuration 0 with more tiles than one round runs the persistent kernel (see
// launch_persistent), whose time per round of one tile per workgroup is modelled apart:
// 1.63 us per k step plus 8.4 us, from MI355X graph timings at 16384 x 24576 x k (k 128 to
// 4096, 24 rounds); it predicts the 8B prefill GEMMs at 16384 tokens within 3 %.
constexpr double kPersistStep = 1.63, kPersistRound = 8.4;
constexpr int kNumCandidates = static_cast<int>(sizeof(kCandidates) / sizeof(kCandidates[0]));
constexpr double kFix0 = 0.0, kFix1 = 2.1;  // split fix-up cost model (us)

int device_cus();

// The persistent kernel for a two-stage configuration, when it applies (see
// w8a8_kernel_persistent): one split, at least two k steps, more tiles than one round,
// output rows of whole 16-byte chunks on a 16-byte aligned output, and operands and tile
// row blocks that buffer resources can span.  Returns false when it does not apply (nothing launched).
template <int BM, int BN, int BK, int WM, int WN, int YT>
bool launch_persistent(const int8_t* xq, const float* x_scale, const int8_t* wq,
                       const float* w_scale, const float* bias, void* y, int64_t m, int64_t n,
                       int64_t k, int splits, hipStream_t stream, hipError_t* err) {
  using C = Cfg<BM, BN, BK, 2, 1, WM, WN>;
  using P = Persist<C, YT>;
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  const int64_t g = device_cus() / kXcds * kXcds;
  if (splits != 1 || k <= BK || tiles <= g || g < kXcds || (n * P::ES) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(y) % 16 != 0 ||
      static_cast<int64_t>(BM) * n * P::ES >= (1ll << 31) || m * k >= (1ll << 31) ||
      n * k >= (1ll << 31))
    return false;
  constexpr auto kern = w8a8_kernel_persistent<BM, BN, BK, WM, WN, YT>;
  *err = allow_dynamic_lds<kern>(static_cast<int>(P::LDS_BYTES));
  if (*err != hipSuccess) return true;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(g)), dim3(C::THREADS), P::LDS_BYTES,
                     stream, xq, x_scale, wq, w_scale, bias, y, m, n, k);
  *err = hipGetLastError();
  return true;
}

template <int YT>
hipError_t launch_candidate(int c, const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, const float* bias, void* y, int64_t m,
                            int64_t n, int64_t k, int splits, int* ws, hipStream_t stream) {
#define I8QL_W8A8_CFG(...) \
  launch_cfg<__VA_ARGS__>(xq, x_scale, wq, w_scale, bias, y, m, n, k, splits, ws, stream)
#define I8QL_W8A8_SPLIT(...) \
  launch_split<__VA_ARGS__>(xq, x_scale, wq, w_scale, bias, y, m, n, k, stream)
  hipError_t perr = hipSuccess;
  switch (c) {
    case 0:
      if (launch_persistent<256, 256, 128, 4, 2, YT>(xq, x_scale, wq, w_scale, bias, y, m, n, k,
                                                      splits, stream, &perr))
        return perr;
      return I8QL_W8A8_CFG(256, 256, 128, 2, 1, YT, 4, 2, true);
    case 1: return I8QL_W8A8_CFG(256, 320, 128, 2, 1, YT, 4, 2, false);
    case 2: return I8QL_W8A8_SPLIT(256, 192, 128, YT, 4, 2);
    case 3: return I8QL_W8A8_SPLIT(128, 320, 128, YT, 4, 2);
    case 4: return I8QL_W8A8_CFG(128, 160, 128, 3, 1, YT, 4, 1, true);
    case 5: return I8QL_W8A8_CFG(256, 128, 128, 3, 1, YT, 4, 2, true);
    case 6: return I8QL_W8A8_CFG(128, 128, 128, 3, 1, YT, 2, 4, true);
    case 7: return I8QL_W8A8_CFG(128, 64, 128, 3, 2, YT, 2, 2, false);
    case 8: return I8QL_W8A8_CFG(64, 64, 128, 3, 2, YT, 2, 2, false);
    case 9: return I8QL_W8A8_CFG(64, 32, 128, 3, 4, YT, 2, 1, false);
    case 10: return I8QL_W8A8_CFG(64, 64, 128, 4, 1, YT, 2, 2, true);
    default: return I8QL_W8A8_CFG(320, 256, 128, 2, 1, YT, 2, 4, false);
  }
#undef I8QL_W8A8_CFG
#undef I8QL_W8A8_SPLIT
}

template <int YT>
hipError_t launch_candidate_gs(int c, const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, const float* bias, void* y, int64_t m,
                               int64_t n, int64_t k, hipStream_t stream) {
#define I8QL_W8A8_GS(...) \
  launch_cfg<__VA_ARGS__>(xq, x_scale, wq, w_scale, bias, y, m, n, k, 1, nullptr, stream)
  switch (c) {
    case 5: return I8QL_W8A8_GS(256, 128, 128, 3, 1, YT, 4, 2, false, true);
    case 6: return I8QL_W8A8_GS(128, 128, 128, 3, 1, YT, 2, 4, false, true);
    default: return I8QL_W8A8_GS(64, 64, 128, 4, 1, YT, 2, 2, false, true);
  }
#undef I8QL_W8A8_GS
}

// Compute units of the current device (cached per device id).
int device_cus() {
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;  // idempotent; a race only repeats the query
  }
  return cached[dev];
}

int64_t plan_workspace(int c, int splits, int64_t m, int64_t n) {
  if (splits <= 1) return 0;
  const Candidate& d = kCandidates[c];
  const int64_t tiles = ((m + d.bm - 1) / d.bm) * ((n + d.bn - 1) / d.bn);
  return (kSplitMaxTiles + tiles * splits * static_cast<int64_t>(d.bm) * d.bn) * 4;
}

// Modelled time of plan (c, splits); negative when the plan is not valid for the shape.
double plan_time(int c, int splits, int64_t m, int64_t n, int64_t k, int cus) {
  const Candidate& d = kCandidates[c];
  const int64_t ksteps = (k + 127) / 128;
  if (d.ks > 1 && k % (128 * d.ks) != 0) return -1.0;
  if (splits > 1 && (!d.xsplit || splits > ksteps)) return -1.0;
  const int64_t tiles = ((m + d.bm - 1) / d.bm) * ((n + d.bn - 1) / d.bn);
  if (splits > 1 && tiles > kSplitMaxTiles) return -1.0;
  const int64_t units = tiles * splits;
  if (units > kMaxGrid - kXcds) return -1.0;
  const double rounds = static_cast<double>((units + cus - 1) / cus);
  const double steps = static_cast<double>((ksteps / d.ks + splits - 1) / splits);
  const int64_t g = cus / kXcds * kXcds;  // persistent workgroups
  if (c == 0 && splits == 1 && ksteps >= 2 && g >= kXcds && tiles > g && n % 8 == 0 &&
      m * k < (1ll << 31) && n * k < (1ll << 31) && 256 * n * 2 < (1ll << 31)) {
    const double prounds = static_cast<double>((tiles + g - 1) / g);
    return kPersistStep * prounds * steps + kPersistRound * prounds;
  }
  double t = d.t_step * rounds * steps + d.t_round * rounds + d.t0;
  if (splits > 1) t += kFix0 + kFix1 * splits * (d.bm * d.bn / 16384.0);
  return t;
}

// The plan with the lowest modelled time whose workspace fits in ws_bytes (no split needs
// none, so a plan always exists).  Every split count up to I8QL_W8A8_MAX_SPLITS is tried for
// the configurations that allow one.
int choose_plan(int64_t m, int64_t n, int64_t k, int cus, int64_t ws_bytes, int* splits_out) {
  int best = kNumCandidates - 1, best_s = 1;
  double best_t = 0.0;
  bool found = false;
  for (int c = 0; c < kNumCandidates; ++c) {
    for (int sp = 1; sp <= I8QL_W8A8_MAX_SPLITS; ++sp) {
      if (sp > 1 && plan_workspace(c, sp, m, n) > ws_bytes) break;
      const double t = plan_time(c, sp, m, n, k, cus);
      if (t < 0.0) break;  // (more splits are not valid either)
      if (!found || t < best_t) {
        best = c;
        best_s = sp;
        best_t = t;
        found = true;
      }
    }
  }
  *splits_out = best_s;
  return best;
}

// The group-scale configuration with the lowest modelled time.
int choose_gs(int64_t m, int64_t n, int64_t k, int cus) {
  int best = 10;
  double best_t = 0.0;
  bool found = false;
  const int64_t ksteps = (k + 127) / 128;
  for (int c = 0; c < kNumCandidates; ++c) {
    const Candidate& d = kCandidates[c];
    if (!d.gs) continue;
    const int64_t units = ((m + d.bm - 1) / d.bm) * ((n + d.bn - 1) / d.bn);
    if (units > kMaxGrid - kXcds) continue;
    const double rounds = static_cast<double>((units + cus - 1) / cus);
    const double t = kGsStep * d.t_step * rounds * ksteps + d.t_round * rounds + d.t0;
    if (!found || t < best_t) {
      best = c;
      best_t = t;
      found = true;
    }
  }
  return best;
}

template <int YT>
hipError_t launch_yt(const int8_t* xq, const float* x_scale, const int8_t* wq,
                     const float* w_scale, const float* bias, void* y, int64_t m, int64_t n,
                     int64_t k, int config, int splits, void* ws, int64_t ws_bytes,
                     hipStream_t stream) {
  int c = config, sp = splits;
  if (c < 0) c = choose_plan(m, n, k, device_cus(), ws ? ws_bytes : 0, &sp);
  return launch_candidate<YT>(c, xq, x_scale, wq, w_scale, bias, y, m, n, k, sp,
                              static_cast<int*>(ws), stream);
}

// ---- the allocation-free entry point's workspace ----------------------------------------
// For callers that cannot allocate device memory, split plans keep their partial tiles and
// counters in this file-scope array instead of a caller's workspace: one copy per GPU, held
// until the process ends, shared by every such call on that GPU (calls that overlap in time
// race on it).  In host code `scratch` names a host-side stand-in, not device memory: kernels
// get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) int scratch[I8QL_W8A8_SCRATCH_BYTES / 4];

__global__ void zero_ints(int* p, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0;
}

// The device address of `scratch` on the current device, looked up once per device (that
// device current).  The first lookup also clears the counter region with a small kernel on
// `stream` (static storage starts zeroed; every call leaves the counters at zero).
hipError_t scratch_address(void** out, hipStream_t stream) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zero_ints, dim3((kSplitMaxTiles + 255) / 256), dim3(256), 0, stream,
                       static_cast<int*>(p), static_cast<int>(kSplitMaxTiles));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

static_assert(kNumCandidates == I8QL_W8A8_NUM_CONFIGS, "configuration count of the C ABI");
static_assert(I8QL_W8A8_SCRATCH_BYTES % 256 == 0 && I8QL_W8A8_SCRATCH_BYTES > kSplitMaxTiles * 4,
              "scratch holds the counters and at least some partial tiles");

hipError_t launch_w8a8_gemm_noalloc(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                    const float* w_scale, const float* bias, void* y,
                                    i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                    int config, int splits, hipStream_t stream) {
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws, stream);
  if (e != hipSuccess) return e;
  return launch_w8a8_gemm(xq, x_scale, wq, w_scale, bias, y, y_dtype, m, n, k, config, splits,
                          ws, I8QL_W8A8_SCRATCH_BYTES, stream);
}

int w8a8_choose_config(int64_t m, int64_t n, int64_t k, int cus) {
  int sp = 1;
  return choose_plan(m, n, k, cus, 0, &sp);
}

int w8a8_choose_plan(int64_t m, int64_t n, int64_t k, int cus, int64_t ws_bytes,
                     int* splits) {
  return choose_plan(m, n, k, cus, ws_bytes, splits);
}

int64_t w8a8_plan_workspace(int config, int splits, int64_t m, int64_t n) {
  return plan_workspace(config, splits, m, n);
}

bool w8a8_plan_valid(int config, int splits, int64_t m, int64_t n, int64_t k) {
  return plan_time(config, splits, m, n, k, 256) >= 0.0;
}

int w8a8_choose_gs_config(int64_t m, int64_t n, int64_t k, int cus) {
  return choose_gs(m, n, k, cus);
}

void w8a8_config_geometry(int config, int32_t* out5) {
  out5[0] = kCandidates[config].bm;
  out5[1] = kCandidates[config].bn;
  out5[2] = kCandidates[config].ks;
  out5[3] = kCandidates[config].xsplit ? 1 : 0;
  out5[4] = kCandidates[config].gs ? 1 : 0;
}

hipError_t launch_w8a8_gemm_g128(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                 const float* w_scale, const float* bias, void* y,
                                 i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                 int config, hipStream_t stream) {
  const int c = config >= 0 ? config : choose_gs(m, n, k, device_cus());
  if (y_dtype == I8QL_F32)
    return launch_candidate_gs<I8QL_F32>(c, xq, x_scale, wq, w_scale, bias, y, m, n, k, stream);
  return launch_candidate_gs<I8QL_BF16>(c, xq, x_scale, wq, w_scale, bias, y, m, n, k, stream);
}

hipError_t launch_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, const float* bias, void* y,
                            i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k, int config,
                            int splits, void* ws, int64_t ws_bytes, hipStream_t stream) {
  switch (y_dtype) {
    case I8QL_I32:
      return launch_yt<I8QL_I32>(xq, x_scale, wq, w_scale, bias, y, m, n, k, config, splits,
                                 ws, ws_bytes, stream);
    case I8QL_F32:
      return launch_yt<I8QL_F32>(xq, x_scale, wq, w_scale, bias, y, m, n, k, config, splits,
                                 ws, ws_bytes, stream);
    default:
      return launch_yt<I8QL_BF16>(xq, x_scale, wq, w_scale, bias, y, m, n, k, config, splits,
                                  ws, ws_bytes, stream);
  }
}

}  // namespace i8ql
