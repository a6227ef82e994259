// Device-side building blocks shared by the forward and backward kernels (gfx950 only).
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64), lane l, half
// h = l / 32:
//   A (32 x 16, M x K): lane holds A[m = l % 32][k = 8h .. 8h + 7]
//   B (16 x 32, K x N): lane holds B[k = 8h .. 8h + 7][n = l % 32]
//   C (32 x 32):        register i holds C[m = 8(i/4) + 4h + (i%4)][n = l % 32]
// fp32 variant v_mfma_f32_32x32x2_f32: A lane holds A[l % 32][h], B holds B[h][l % 32],
// C as above.
//
// LDS tiles of bf16 rows (K, V, Q, dO, dS^T) are stored row-major with the 16-byte chunks
// of each row XOR-swizzled: physical chunk = chunk ^ swz<D>(row). The LDS has 64 banks of
// 4 bytes and serves 16 lanes per cycle; the swizzle keeps both access patterns the
// kernels use free of bank conflicts:
//   (a) 16-byte reads of one logical chunk by 16 consecutive rows (MFMA row operands), and
//   (b) transpose reads, where 16 lanes take 4 consecutive rows x 32 bytes.
//   D = 128 (16 chunks / 256-byte row):  swz = ((row & 3) << 2) | ((row >> 2) & 3)
//   D = 64  (8 chunks / 128-byte row, two rows per bank line):
//                                        swz = (((row >> 1) & 1) << 2) | ((row >> 2) & 3)
// swz depends on row & 15 only, so moving by a multiple of 16 rows is a plain offset.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value: branches
// that depend on it stay scalar branches instead of per-lane exec masking.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Raw buffer resource over [base, base + bytes). Loads through it at a byte offset >= bytes
// return zero instead of touching memory (the hardware range check of raw buffers), which
// zero-fills tiles that run past the end of a sequence without any per-lane test.
// Word 3 selects 32-bit data format, as for every gfx9-family raw buffer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
__device__ __forceinline__ int swz(int row) {
  static_assert(D == 32 || D == 64 || D == 128, "tile width");
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else return (row >> 2) & 3;  // 4 chunks / 64-byte row, four rows per bank line
}

// Byte offset of element (row, col) in a swizzled bf16 tile with D columns.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * (D * 2) + (((col >> 3) ^ swz<D>(row)) << 4) + ((col & 7) << 1);
}

// 16-byte LDS read at a precomputed address.
__device__ __forceinline__ bf16x8 lds_ld8(const FA_LDS char* p) { return *reinterpret_cast<const FA_LDS bf16x8*>(p); }

// 16-byte read of 8 consecutive bf16 (col multiple of 8) from a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 lds_read8(const FA_LDS char* tile, int row, int col) {
  return *reinterpret_cast<const FA_LDS bf16x8*>(tile + tile_off<D>(row, col));
}

// Transpose read (ds_read_b64_tr_b16). Within each 16-lane group, lane 4r + c supplies
// the address of row r, columns 4c .. 4c + 3 of a 4 x 16 block of 16-bit elements, and
// lane j of the group receives column j: (row 0, row 1, row 2, row 3).
__device__ __forceinline__ bf16x4 lds_read_tr(const FA_LDS char* addr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)addr);
  return __builtin_bit_cast(bf16x4, r);
}

// MFMA A operand "X^T" (M = column index of X, K = row index of X) for the 32 columns
// [col0, col0 + 32) and the 8 rows {r0 + 4h + 0..3, r0 + 8 + 4h + 0..3} of a swizzled tile
// X: lane l receives X[those rows][col0 + l % 32]. This is the row permutation that the
// accumulator layout of a 32 x 32 MFMA block hands to the next product (registers
// 8t .. 8t + 7 of a C tile cover rows 16t + {4h..4h+3, 8+4h..8+4h+3}).
template <int D>
__device__ __forceinline__ bf16x8 lds_read_tr8(const FA_LDS char* tile, int r0, int col0) {
  const int l = lane_id();
  const int h = l >> 5;
  const int j = l & 15;
  const int rr = j >> 2;                          // row inside the 4-row block
  const int cc = col0 + ((l >> 4) & 1) * 16 + (j & 3) * 4;
  bf16x4 lo = lds_read_tr(tile + tile_off<D>(r0 + 4 * h + rr, cc));
  bf16x4 hi = lds_read_tr(tile + tile_off<D>(r0 + 8 + 4 * h + rr, cc));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The two per-lane addresses of lds_read_tr8<D>(tile, 0, col0), tile-relative. Adding
// 16 t * 2D bytes to both gives the read at r0 = 16 t (swz<D> depends on row & 15 only).
template <int D>
__device__ __forceinline__ void tr8_offsets(int col0, int& lo, int& hi) {
  const int l = lane_id();
  const int h = l >> 5;
  const int j = l & 15;
  const int cc = col0 + ((l >> 4) & 1) * 16 + (j & 3) * 4;
  lo = tile_off<D>(4 * h + (j >> 2), cc);
  hi = tile_off<D>(8 + 4 * h + (j >> 2), cc);
}

__device__ __forceinline__ bf16x8 lds_tr8(const FA_LDS char* lo, const FA_LDS char* hi) {
  return __builtin_shufflevector(lds_read_tr(lo), lds_read_tr(hi), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Pack 8 fp32 accumulator values (registers base .. base + 7) into a bf16 MFMA operand,
// round-to-nearest-even.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int base) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)c[base + i];
  return r;
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32); }

// The value held by the lane 32 positions away (the other half of the wave), through
// v_permlane32_swap: for lanes < 32 the second result is the upper half's value, for
// lanes >= 32 the first result is the lower half's value.
__device__ __forceinline__ float other_half(float x) {
  const int xi = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, lane_id() < 32 ? (int)r[1] : (int)r[0]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The (b, h) slice of a call: its row count, the element offset of its first row and the
// offset of its lse / D rows. Dense [B, H, N, d]: every slice has N rows of stride d.
// Packed sequences [total, H, d] (a.cu != nullptr): sequence b owns tokens cu[b] ..
// cu[b+1] - 1 (clamped into [0, total], so no boundary array can send an access outside
// the tensors), rows are a.rs = H d apart, lse / D are [H, total].
struct HeadSlice {
  int N;
  size_t hoff, loff;
};
template <int D, class Args>
__device__ __forceinline__ HeadSlice head_slice(const Args& a, int bh) {
  if (!a.cu) return HeadSlice{a.N, (size_t)bh * a.N * D, (size_t)bh * a.N};
  const int b = bh / a.H, hh = bh % a.H;
  const int c0 = min(max(a.cu[b], 0), a.total), c1 = min(max(a.cu[b + 1], c0), a.total);
  return HeadSlice{c1 - c0, (size_t)c0 * a.rs + (size_t)hh * D, (size_t)hh * a.total + c0};
}

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): per round the 64-bit products M0 x0 and M1 x2 give the new
// state (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); the key then
// advances by two Weyl increments. It generates the dropout mask from (position, head,
// batch, seed) alone, so the backward regenerates the forward's mask without storing it.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
    // three-input XORs as one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), x1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), x3, k1, 0x96);
    x1 = (uint32_t)p1;
    x3 = (uint32_t)p0;
    x0 = n0;
    x2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{x0, x1, x2, x3};
}

// Dropout keep rule: one generator call per block of 4 keys x 2 queries, counter
// (key / 4, query / 2, head, batch), key (seed_lo, seed_hi); key j of query i takes word
// j % 4, 16-bit half i % 2 (0 = low), and is kept iff that value is >= thr (floor(p 2^16));
// kept probabilities are scaled by 1 / (1 - p). With thr_hi = thr << 16, a high half is
// >= thr iff its word is >= thr_hi, a low half iff the word shifted left by 16 is.

// Keep bits of two packed words: x01 holds the values of items 0 (low) and 1 (high),
// x23 those of items 2 and 3. Bit k = item k kept.
__device__ __forceinline__ uint32_t dropout_keep4(uint32_t x01, uint32_t x23, uint32_t thr_hi) {
  return (uint32_t)((x01 << 16) >= thr_hi) | ((uint32_t)(x01 >= thr_hi) << 1) |
         ((uint32_t)((x23 << 16) >= thr_hi) << 2) | ((uint32_t)(x23 >= thr_hi) << 3);
}

// Query-per-lane layout (forward and dQ kernels): in the 32-key block at kb0, lane (ql, h)
// holds query qi and keys kb0 + 8 g + 4 h + r (g, r = 0..3). Queries 2m and 2m + 1 sit in
// lanes ql and ql ^ 1 of one quad and share each key group's call: for the group pairs
// (0, 1) and (2, 3) the lane makes the call of group 2 gp + (ql & 1), packs the halves of its
// query (v_perm_b32, two values to a word) and swaps the other halves with its neighbour
// (one DPP exchange per packed word). Returns the block's keep bits, bit 4 g + r.
__device__ __forceinline__ uint32_t dropout_bits_qlane(int kb0, int qi, int ql, int h, uint32_t head, uint32_t bat,
                                                       uint32_t seed_lo, uint32_t seed_hi, uint32_t thr) {
  const uint32_t odd = (uint32_t)(ql & 1);
  const uint32_t thr_hi = thr << 16;
  // byte selectors of v_perm_b32(w_hi, w_lo): low halves of both words, or high halves
  const uint32_t sel_own = odd ? 0x07060302u : 0x05040100u;
  const uint32_t sel_other = odd ? 0x05040100u : 0x07060302u;
  uint32_t bits = 0;
#pragma unroll
  for (int gp = 0; gp < 2; ++gp) {
    const int g = 2 * gp + (int)odd;
    const u32x4 w = philox4x32_10((uint32_t)(kb0 + 8 * g + 4 * h) >> 2, (uint32_t)qi >> 1, head, bat, seed_lo,
                                  seed_hi);
    const uint32_t own01 = __builtin_amdgcn_perm(w[1], w[0], sel_own);
    const uint32_t own23 = __builtin_amdgcn_perm(w[3], w[2], sel_own);
    const uint32_t snd01 = __builtin_amdgcn_perm(w[1], w[0], sel_other);
    const uint32_t snd23 = __builtin_amdgcn_perm(w[3], w[2], sel_other);
    // quad_perm [1, 0, 3, 2]: the value of lane ql ^ 1
    const uint32_t rcv01 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)snd01, 0xB1, 0xF, 0xF, false);
    const uint32_t rcv23 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)snd23, 0xB1, 0xF, 0xF, false);
    bits |= (dropout_keep4(own01, own23, thr_hi) << (4 * g)) |
            (dropout_keep4(rcv01, rcv23, thr_hi) << (4 * (g ^ 1)));
  }
  return bits;
}

// Key-per-lane layout (dK/dV kernel): lane (kl, h) holds key `key` and, in query group G,
// queries q_g0 + 8 (G - g0) + e (e = 0..3; q_g0 counts the lane's 4 h offset). The lanes of
// a quad hold keys 4c .. 4c + 3, the keys of one call. For the group pair (g0, g0 + 1) the
// quad needs four calls (two query pairs per group): lane q = key % 4 makes the call of group
// g0 + q / 2, query pair q % 2; a 4 x 4 transpose across the quad (two rounds of DPP
// exchanges) then leaves in lane q word q of every call, which holds its key's values for
// that call's two queries. Returns bit 4 (G - g0) + e = query e of group G kept.
__device__ __forceinline__ uint32_t dropout_bits_klane(int key, int q_g0, uint32_t head, uint32_t bat,
                                                       uint32_t seed_lo, uint32_t seed_hi, uint32_t thr) {
  const uint32_t q = (uint32_t)(key & 3);
  const uint32_t qpair = (uint32_t)(q_g0 + 8 * (int)(q >> 1) + 2 * (int)(q & 1)) >> 1;
  const u32x4 w = philox4x32_10((uint32_t)key >> 2, qpair, head, bat, seed_lo, seed_hi);
  // round 1, lanes q and q ^ 1: swap the words whose index differs from q in bit 0
  const bool o1 = (q & 1u) != 0;
  const uint32_t s0 = o1 ? w[0] : w[1], s1 = o1 ? w[2] : w[3];
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0xB1, 0xF, 0xF, false);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0xB1, 0xF, 0xF, false);
  const uint32_t a0 = o1 ? r0 : w[0], a1 = o1 ? w[1] : r0, a2 = o1 ? r1 : w[2], a3 = o1 ? w[3] : r1;
  // round 2, lanes q and q ^ 2 (quad_perm [2, 3, 0, 1]): the same in bit 1
  const bool o2 = (q & 2u) != 0;
  const uint32_t t0 = o2 ? a0 : a2, t1 = o2 ? a1 : a3;
  const uint32_t u0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t0, 0x4E, 0xF, 0xF, false);
  const uint32_t u1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t1, 0x4E, 0xF, 0xF, false);
  const uint32_t b0 = o2 ? u0 : a0, b1 = o2 ? u1 : a1, b2 = o2 ? a2 : u0, b3 = o2 ? a3 : u1;
  // b_j: word q of lane j's call (group g0 + j / 2, query pair j % 2), halves by query parity
  const uint32_t thr_hi = thr << 16;
  return dropout_keep4(b0, b1, thr_hi) | (dropout_keep4(b2, b3, thr_hi) << 4);
}

// 16-byte global load/store helpers (addresses 16-byte aligned).
__device__ __forceinline__ u32x4 gload16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void lds_store16(FA_LDS char* p, u32x4 v) { *reinterpret_cast<FA_LDS u32x4*>(p) = v; }

}  // namespace fa
