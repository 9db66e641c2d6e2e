// dequant_mma.hpp — the inner loop shared by the weight-only (W8A16) kernels on gfx950.
//
// Weight-only int8 saves HBM bytes, not arithmetic ("Phase 5a: int8 weight-only
// quantization", Summary): the int8 codes are expanded to bf16 in registers and the product
// runs on the bf16 matrix cores ("Day 6 — Quantize It Yourself", The mechanism, block 5).
// The expansion is exact: every code in [-127, 127] is a bf16 value.
//
// Tile shape: one wavefront owns 16 weight rows (output channels) and up to MT x 16
// activation rows.  v_mfma_f32_16x16x32_bf16 takes the weights as operand A (row i = lane
// % 16) and the activations as operand B (column j = lane % 16); lanes 16g .. 16g+15 carry
// k-slots 8g .. 8g+7.  Only the pairing of A and B slots matters for the sum, so each lane
// feeds both operands from the same 32 consecutive input channels: k0 + 32 * (lane / 16)
// + [0, 32), i.e. one 128-channel step is four MFMAs.  A step reads 16 rows x 128 bytes of
// weights: every lane issues two 16-byte loads and each row's 128-byte line is read whole
// by four lanes.  The accumulator holds D[n][m]: lane l, register r is channel
// 4 * (l / 16) + r of the tile and activation row l % 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8ql {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kStepK = 128;  // input channels per wavefront step

// Four int8 codes -> two dwords holding four bf16 values (exact).  Each code converts to a
// float32 whose low 16 bits are zero (|code| < 256), so its high half is the bf16; one byte
// permute packs the high halves of two floats.
__device__ __forceinline__ uint2 i8x4_to_bf16x4(uint32_t w) {
  const uint32_t f0 = __float_as_uint(static_cast<float>(static_cast<int8_t>(w)));
  const uint32_t f1 = __float_as_uint(static_cast<float>(static_cast<int8_t>(w >> 8)));
  const uint32_t f2 = __float_as_uint(static_cast<float>(static_cast<int8_t>(w >> 16)));
  const uint32_t f3 = __float_as_uint(static_cast<float>(static_cast<int8_t>(w >> 24)));
  // v_perm_b32 selector: bytes 2, 3 of the second operand, then bytes 2, 3 of the first
  return make_uint2(__builtin_amdgcn_perm(f1, f0, 0x07060302u),
                    __builtin_amdgcn_perm(f3, f2, 0x07060302u));
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16 codes -> two 8-wide bf16 MFMA operands.
__device__ __forceinline__ void i8x16_to_bf16(const v4u w, v8bf& a0, v8bf& a1) {
  const uint2 p0 = i8x4_to_bf16x4(w[0]), p1 = i8x4_to_bf16x4(w[1]);
  const uint2 q0 = i8x4_to_bf16x4(w[2]), q1 = i8x4_to_bf16x4(w[3]);
  a0 = __builtin_bit_cast(v8bf, v4u{p0.x, p0.y, p1.x, p1.y});
  a1 = __builtin_bit_cast(v8bf, v4u{q0.x, q0.y, q1.x, q1.y});
}

// 16 bytes at p + (ok ? off : 0), replaced by zeros when !ok.  The address is always in
// bounds and the load unconditional, so it compiles to one 16-byte load and a select (a
// guarded load would become branches around 4-byte loads).
__device__ __forceinline__ v4u load16_or_zero(const void* p, int64_t off, bool ok) {
  const v4u v = *reinterpret_cast<const v4u*>(static_cast<const char*>(p) + (ok ? off : 0));
  return ok ? v : v4u{0u, 0u, 0u, 0u};
}

// Issue the weight loads of steps [s, s + U): two 16-byte loads per lane per step, all
// unconditional so that the compiler keeps them together ahead of their use instead of
// sinking each into a branch.  Loads of steps at or past s_end, or of chunks past k, read
// the row start instead (in bounds); the multiply gives them zero activations, which is
// exact because int8 codes are always finite.  No select on the loaded values here: it
// would make the wave wait for the loads before the batch is even issued.
template <int U>
__device__ __forceinline__ void load_weight_batch(const int8_t* __restrict__ wrow, int64_t k,
                                                  int s, int s_end, v4u (&w)[U][2]) {
  const int sub = 32 * ((threadIdx.x % 64) / 16);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t kk = static_cast<int64_t>(s + u) * kStepK + sub;
    const bool in = (s + u) < s_end;
    w[u][0] = *reinterpret_cast<const v4u*>(wrow + (in && kk < k ? kk : 0));
    w[u][1] = *reinterpret_cast<const v4u*>(wrow + (in && kk + 16 < k ? kk + 16 : 0));
  }
}

// Multiply a loaded batch (steps [s, s + U)) by activation rows staged in LDS: xrow[mt] is
// this lane's row (input channel c at byte 2c), xzero 16 zero bytes.  Every step is
// computed; for steps at or past s_end and for chunks past k the activations are read from
// xzero.  The in-order vmcnt wait before step u covers only that step's two loads, so each
// step is converted and multiplied while the later ones are still in flight.
//
// Only lanes whose activation row exists (live[mt]) read LDS: the others keep whatever xb
// holds, which only reaches output columns that are never stored.  With one decode row
// that is 4 of 64 lanes, so the fragment reads cost a sixteenth of the LDS bandwidth.
//
// GS (one weight scale per step of 128 input channels, "Day 6 — Quantize It Yourself", The
// mechanism, block 1: each run of 128 consecutive input channels of a row has its own scale): each
// step's four MFMAs go into a zeroed partial tile, which is then multiplied by the step's
// scales of the lane's 4 channels (gs: the workgroup's LDS table [step][16 channels]) and
// added to the accumulator; steps past s_end add nothing.
template <int MT, int U, bool GS = false>
__device__ __forceinline__ void mma_batch_lds(const v4u (&w)[U][2], const char* const (&xrow)[MT],
                                              const bool (&live)[MT], const char* xzero,
                                              int64_t k, int s, int s_end, v4u (&xb)[MT][4],
                                              v4f (&acc)[MT], const float* gs = nullptr) {
  const int sub = 32 * ((threadIdx.x % 64) / 16);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t kk = static_cast<int64_t>(s + u) * kStepK + sub;
    const bool in = (s + u) < s_end;
    v8bf a[4];
    i8x16_to_bf16(w[u][0], a[0], a[1]);
    i8x16_to_bf16(w[u][1], a[2], a[3]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (live[mt]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t kc = kk + 8 * c;
          const char* xp = in && kc < k ? xrow[mt] + 2 * kc : xzero;
          xb[mt][c] = *reinterpret_cast<const v4u*>(xp);
        }
      }
      if constexpr (GS) {
        v4f part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a[c], __builtin_bit_cast(v8bf, xb[mt][c]), part, 0, 0, 0);
        if (in) {
          const v4f sc = *reinterpret_cast<const v4f*>(
              gs + (s + u) * 16 + 4 * ((threadIdx.x % 64) / 16));
          acc[mt] += part * sc;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a[c], __builtin_bit_cast(v8bf, xb[mt][c]), acc[mt], 0, 0, 0);
      }
    }
  }
}

// A buffer resource over the `bytes` bytes at `base` (wavefront-uniform; bytes < 2^31):
// loads through it at offsets at or past `bytes` return zeros instead of reading memory.
// Dword 3 is the raw (untyped) format of the CDNA buffer descriptor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const int8_t* base,
                                                              int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(base), 0,
                                           static_cast<int>(bytes), 0x00020000);
}

// load_weight_batch through a buffer resource over one 16-row weight tile: voff is this
// lane's byte offset in the tile (row (lane % 16) * k plus its 32-channel slot), s the first
// step.  Every load of the batch shares the one offset register (steps and halves differ by
// immediate offsets), no bounds select is needed: rows past the tile and bytes past its end
// read as zeros, and chunks past k or steps past the caller's range read other codes of the
// tile, which the caller never multiplies by a nonzero activation (mma_batch_staged skips
// such steps and feeds zeros past k).
template <int U>
__device__ __forceinline__ void load_weight_batch_rsrc(__amdgpu_buffer_rsrc_t rs, int voff,
                                                       int s, v4u (&w)[U][2]) {
  const int soff = s * kStepK;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    w[u][0] = __builtin_bit_cast(
        v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + u * kStepK, soff, 0));
    w[u][1] = __builtin_bit_cast(
        v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + u * kStepK + 16, soff, 0));
  }
}

// mma_batch_lds for one activation tile, with the bounds handled by wavefront-uniform
// branches instead of per-read selects: a step that lies wholly below k reads its four
// fragments at the staged row's base plus immediate offsets, only a step that straddles k (k
// not a multiple of 128) reads xzero for the chunks past k, and a step at or past s_end is
// multiplied by zeros.  Every step of the batch is converted and multiplied, so every load of
// the batch has an unconditional use: the compiler keeps the loads where load_weight_batch_rsrc
// issued them, which the callers' vmcnt arithmetic relies on.  xrow: this lane's staged row
// (input channel c at byte 2c), read only when `live`.
template <int U>
__device__ __forceinline__ void mma_batch_staged(const v4u (&w)[U][2], const char* xrow,
                                                 bool live, const char* xzero, int64_t k, int s,
                                                 int s_end, v4u (&xb)[4], v4f& acc) {
  const int sub = 32 * ((threadIdx.x % 64) / 16);
  const char* xp = xrow + 2 * (static_cast<int64_t>(s) * kStepK + sub);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    v8bf a[4];
    i8x16_to_bf16(w[u][0], a[0], a[1]);
    i8x16_to_bf16(w[u][1], a[2], a[3]);
    if (s + u >= s_end) {  // uniform
#pragma unroll
      for (int c = 0; c < 4; ++c) xb[c] = v4u{0u, 0u, 0u, 0u};
    } else if (live) {
      if (static_cast<int64_t>(s + u + 1) * kStepK <= k) {  // uniform
#pragma unroll
        for (int c = 0; c < 4; ++c)
          xb[c] = *reinterpret_cast<const v4u*>(xp + u * 2 * kStepK + 16 * c);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t kc = static_cast<int64_t>(s + u) * kStepK + sub + 8 * c;
          xb[c] = *reinterpret_cast<const v4u*>(kc < k ? xp + u * 2 * kStepK + 16 * c : xzero);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c], __builtin_bit_cast(v8bf, xb[c]), acc,
                                                    0, 0, 0);
  }
}

// Accumulate the wavefront's partial product over steps [s_begin, s_end), activations read
// from global memory (L2-resident: every workgroup reads the same rows).
//   wrow      : this lane's weight row (row n0 + lane % 16, clamped into the matrix)
//   xrow      : this lane's activation row for each m-tile (lane % 16 within the tile);
//               always a valid row, xok says whether it is a real one (else the MFMA
//               column is fed zeros)
// All loads of a batch of U steps are issued unconditionally (at in-bounds addresses) before
// the first is used; steps past s_end, chunks past k and rows past m get zero activations.
// GS: as in mma_batch_lds, with the step's scales of the lane's 4 channels read from global
// memory with the batch (gsr[r]: the [k / 128] scale row of channel 4 * (lane / 16) + r).
template <int MT, int U, bool GS = false>
__device__ __forceinline__ void dequant_mma_steps(const int8_t* __restrict__ wrow,
                                                  const uint16_t* const (&xrow)[MT],
                                                  const bool (&xok)[MT], int64_t k,
                                                  int s_begin, int s_end, v4f (&acc)[MT],
                                                  const float* const* gsr = nullptr) {
  const int lane = threadIdx.x % 64;
  const int sub = 32 * (lane / 16);  // this lane's 32 channels within a step
  for (int s = s_begin; s < s_end; s += U) {
    v4u w[U][2];
    v4u xr[U][MT][4];
    v4f gsc[GS ? U : 1];
    if constexpr (GS) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int st = min(s + u, s_end - 1);  // past the range: any valid scale (adds 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) gsc[u][r] = gsr[r][st];
      }
    }
    load_weight_batch<U>(wrow, k, s, s_end, w);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kk = static_cast<int64_t>(s + u) * kStepK + sub;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t kc = kk + 8 * c;
          xr[u][mt][c] = *reinterpret_cast<const v4u*>(xrow[mt] + (kc < k ? kc : 0));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kk = static_cast<int64_t>(s + u) * kStepK + sub;
      const bool in = (s + u) < s_end;
      v8bf a[4];
      i8x16_to_bf16(w[u][0], a[0], a[1]);
      i8x16_to_bf16(w[u][1], a[2], a[3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v4f part = {0.f, 0.f, 0.f, 0.f};
        v4f& dst = GS ? part : acc[mt];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool ok = in && xok[mt] && kk + 8 * c < k;
          const v4u xb = ok ? xr[u][mt][c] : v4u{0u, 0u, 0u, 0u};
          dst = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c], __builtin_bit_cast(v8bf, xb), dst,
                                                        0, 0, 0);
        }
        if constexpr (GS) {
          if (in) acc[mt] += part * gsc[u];
        }
      }
    }
  }
}

// Staged activation rows in LDS: row r at r * (2k + 16) bytes (consecutive rows shifted by
// one 16-byte slot, so the row-parallel fragment reads do not collide on banks), i.e. a run
// of 16-byte slots where slot q = r * (k / 8 + 1) + c holds chunk c of row r and the last
// slot of each row is padding.  Copy instructions (1 KiB each) needed for `rows` rows:
__host__ __device__ inline int stage_insts(int rows, int64_t k) {
  return static_cast<int>((rows * (k / 8 + 1) + 63) / 64);
}

// Issue the direct-to-LDS copy of `rows` activation rows into xs (1 KiB-aligned): row r is
// x row r, or, with a gather list, x row list[r] / div.  Each wavefront instruction fills
// one contiguous KiB, lane l its l-th slot; padding slots and slots past the last row load
// the first chunk of the first row, which is in bounds.  The loads count in vmcnt like any
// other: the caller waits for them before a barrier that publishes the rows.
template <int WAVES>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ x, const int* list,
                                           int div, int rows, int64_t k, char* xs) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int per_row = static_cast<int>(k / 8) + 1;
  const int insts = stage_insts(rows, k);
  int r = (wave * 64 + lane) / per_row, c = (wave * 64 + lane) % per_row;
  const int adv_r = (64 * WAVES) / per_row, adv_c = (64 * WAVES) % per_row;
  const int64_t first = list ? list[0] / div : 0;
  for (int i = wave; i < insts; i += WAVES) {
    const bool ok = r < rows && c < per_row - 1;
    const int64_t xr = ok ? (list ? list[r] / div : r) : first;
    const uint16_t* g = x + xr * k + (ok ? 8 * c : 0);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const int8_t*>(g), xs + 1024 * i, 16, 0,
                                     0);
    c += adv_c;
    r += adv_r;
    if (c >= per_row) {
      c -= per_row;
      ++r;
    }
  }
}

// Split the steps of k among the waves of a workgroup: wave w gets [begin, end).
__device__ __forceinline__ void wave_step_range(int64_t k, int waves, int wave, int& begin,
                                                int& end) {
  const int steps = static_cast<int>((k + kStepK - 1) / kStepK);
  const int per = (steps + waves - 1) / waves;
  begin = min(steps, wave * per);
  end = min(steps, begin + per);
}

// Round a float32 to the nearest-even bfloat16 bit pattern (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace i8ql
