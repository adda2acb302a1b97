// MFMA tile and cross-lane helpers shared by the chunked kernels (the
// forward prefill and its gradients) on gfx950: bf16 packing, the
// v_mfma_f32_32x32x16_bf16 wrapper, the permuted k-order and XOR-swizzled
// LDS tiles, transpose operand reads, and DPP / permlane sums.  Every
// definition sits in an anonymous namespace, so each translation unit
// keeps its own inlined copy.
#pragma once

#include "la_device.h"

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Split a pair into bf16 high parts and bf16 low parts (x - high), so that
// high + low carries x to about 2^-16 relative.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 8 consecutive elements of storage type DT, as fp32.
__device__ __forceinline__ void unpack8(const u32x4& w, float* x, bf16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack8(const u32x4& w, float* x, f16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = float(__builtin_bit_cast(f16_t, uint16_t(w[i] & 0xffffu)));
    x[2 * i + 1] = float(__builtin_bit_cast(f16_t, uint16_t(w[i] >> 16)));
  }
}

// Position of k-index k inside the permuted order: within each 16, quads 1
// and 2 are swapped ([0-3, 8-11, 4-7, 12-15] at positions 0..15).
__device__ __forceinline__ constexpr int perm_pos(int k) {
  const int q = (k >> 2) & 3;
  const int pq = q == 1 ? 2 : (q == 2 ? 1 : q);
  return (k & ~15) | (pq << 2) | (k & 3);
}

// XOR swizzle of the 16-byte blocks of tile row r.  Two read patterns must
// spread over the 64 LDS banks: 16 lanes reading one block of 16
// consecutive rows (row-wise operands), and 32 lanes reading 4 consecutive
// rows x 4 consecutive blocks (transposed operands; rows start at a multiple
// of 4).  D = 128: 16 blocks per row, the swizzle is a bijection on 0..15 for
// any 16 consecutive rows and takes 4 values 4 apart over each aligned group
// of 4 rows.  D = 64: 8 blocks per row (two rows per bank line), the same
// with the row pair's parity taking one bit.
template <int D>
__device__ __forceinline__ int blk_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Byte offset of logical 16-byte block b of row r.
template <int D>
__device__ __forceinline__ int tile_off(int r, int b) {
  return r * (2 * D) + ((b ^ blk_swz<D>(r)) << 4);
}

// Row-wise MFMA operand: the 8 bf16 of logical block b of row r.
template <int D>
__device__ __forceinline__ u32x4 row_operand(const char* tile, int r, int b) {
  return *reinterpret_cast<const u32x4*>(tile + tile_off<D>(r, b));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposed MFMA operand from a token-major tile, by two LDS transpose
// reads (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane s reads
// 8 bytes at row k0 + 8 g + 4 h + s / 4, columns c + 4 (s % 4) .. + 3 of the
// group's 16-column block; the instruction hands lane s back element s % 4 of
// the reads of lanes s / 4 + {0, 4, 8, 12}, i.e. column (s) of the block at 4
// consecutive rows.  Result: lane (n = lane % 32, g = lane / 32) holds rows
// k0 + 8 g .. k0 + 8 g + 7 of column colbase + n, the operand layout of
// v_mfma_f32_32x32x16_bf16 for a k = row operand.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const char* tile, int k0, int colbase, int lane) {
  const int g = lane >> 5, s = lane & 15;
  const int c = colbase + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = k0 + 8 * g + 4 * h + (s >> 2);
    const char* p = tile + tile_off<D>(r, c >> 3) + ((c & 7) << 1);
    const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    const u32x2 y = __builtin_bit_cast(u32x2, x);
    out[2 * h] = y[0];
    out[2 * h + 1] = y[1];
  }
  return out;
}

// v_mfma_f32_16x16x32_bf16: lane (n = lane % 16, q = lane / 16) holds
// k-values 8 q .. 8 q + 7 of row (A) or column (B) n; the result holds rows
// 4 q .. 4 q + 3 of column n.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The transposed operand of v_mfma_f32_16x16x32_bf16 from a token-major
// tile: lane (n, q) holds rows k0 + 8 q .. k0 + 8 q + 7 of column
// colbase + n (the same two LDS transpose reads as tr_operand, with the four
// 16-lane groups taking four 8-row blocks of one 16-column block).
template <int D>
__device__ __forceinline__ u32x4 tr_operand16(const char* tile, int k0, int colbase, int lane) {
  const int q = lane >> 4, s = lane & 15;
  const int c = colbase + 4 * (s & 3);
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = k0 + 8 * q + 4 * h + (s >> 2);
    const char* p = tile + tile_off<D>(r, c >> 3) + ((c & 7) << 1);
    const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    const u32x2 y = __builtin_bit_cast(u32x2, x);
    out[2 * h] = y[0];
    out[2 * h + 1] = y[1];
  }
  return out;
}

// Features 8 fb .. 8 fb + 7 of row r (4 packed bf16 pairs) at their
// perm_pos positions: two 8-byte pieces.
template <int D>
__device__ __forceinline__ void row_write_perm(char* tile, int r, int fb, const u32x4& w) {
  const int p0 = perm_pos(8 * fb), p1 = perm_pos(8 * fb + 4);
  *reinterpret_cast<u32x2*>(tile + tile_off<D>(r, p0 >> 3) + ((p0 & 7) << 1)) = u32x2{w[0], w[1]};
  *reinterpret_cast<u32x2*>(tile + tile_off<D>(r, p1 >> 3) + ((p1 & 7) << 1)) = u32x2{w[2], w[3]};
}

// Features 8 fb .. 8 fb + 7 of row r in natural order: one 16-byte block.
template <int D>
__device__ __forceinline__ void blk_write(char* tile, int r, int fb, const u32x4& w) {
  *reinterpret_cast<u32x4*>(tile + tile_off<D>(r, fb)) = w;
}

__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
               pack_bf16(x[6], x[7])};
}

// bf16 high parts (hi = pack8(x), given) and low parts x - hi.
__device__ __forceinline__ u32x4 low8(const float* x, const u32x4& hi) {
  u32x4 lo;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    lo[i] = pack_bf16(x[2 * i] - __uint_as_float(hi[i] << 16),
                      x[2 * i + 1] - __uint_as_float(hi[i] & 0xffff0000u));
  return lo;
}

// Cross-lane sums without LDS traffic.  row_sum<FB>: sum over each aligned
// group of FB (8 or 16) lanes, in every lane of the group (DPP quad
// permutes and row mirrors).  group_sum<FB>: sum over the lanes that share
// lane % FB (DPP rotate within a row for FB = 8, then the gfx950 row and
// half-wave swaps), in every such lane.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
// The swaps return both registers as a two-element vector.  Its elements are
// read through one 64-bit cast: at -O3 this compiler folds a subscript of the
// second element into the first.
template <class V>
__device__ __forceinline__ float pair_sum(const V& r) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, r);
  return __builtin_bit_cast(float, unsigned(u)) + __builtin_bit_cast(float, unsigned(u >> 32));
}
__device__ __forceinline__ float swap_sum16(float x) {   // x[l] + x[l ^ 16]
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return pair_sum(r);
}
__device__ __forceinline__ float swap_sum32(float x) {   // x[l] + x[l ^ 32]
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return pair_sum(r);
}
template <int FB>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);     // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);     // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);    // row_half_mirror
  if constexpr (FB == 16) x += dpp<0x140>(x);   // row_mirror
  return x;
}
// Exchange lanes 32-63 of a with lanes 0-31 of b (v_permlane32_swap): a
// keeps its lower half and takes b's lower half into its upper lanes, b
// takes a's upper half into its lower lanes and keeps its upper half.
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  const unsigned long long u = __builtin_bit_cast(unsigned long long, r);   // see pair_sum
  a = unsigned(u);
  b = unsigned(u >> 32);
}

// Padded position of feature 8 fb + e in a wave's z increments (see DZS).
__device__ __forceinline__ int dz_index(int fb, int e) { return 8 * fb + e + ((fb >> 3) << 2); }

// x[l] + x[l ^ 32] of a in lanes 0-31 and of b in lanes 32-63 (the swap
// trades lanes 32-63 of its first register with lanes 0-31 of its second).
__device__ __forceinline__ float swap_fold32(float a, float b) {
  return pair_sum(__builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                   __builtin_bit_cast(unsigned, b), false, false));
}
// x[l] + x[l ^ 16] of a in even rows of 16 lanes and of b in odd rows (the
// swap trades the odd rows of its first register with the even rows of its
// second).
__device__ __forceinline__ float swap_fold16(float a, float b) {
  return pair_sum(__builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                   __builtin_bit_cast(unsigned, b), false, false));
}
// Reduce-scatter of 8 per-lane values v[e] (feature 8 fb + e, fb = lane % FB)
// over the lanes of a wave that share fb: on return every lane holds the
// totals of features 8 fb + base + {0, 1} in s0, s1 and the function returns
// base (lanes l and l ^ 8 hold the same pair when FB = 8).
template <int FB>
__device__ __forceinline__ int reduce_scatter8(const float (&v)[8], int lane, float& s0,
                                               float& s1) {
  float t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = swap_fold32(v[i], v[i + 4]);   // feature i + 4 (lane / 32)
  s0 = swap_fold16(t[0], t[2]);   // feature 2 (row & 1) + 4 (lane / 32) + {0, 1}
  s1 = swap_fold16(t[1], t[3]);
  if constexpr (FB == 8) {
    s0 += dpp<0x128>(s0);          // row_ror:8, lanes l and l ^ 8 share fb
    s1 += dpp<0x128>(s1);
  }
  return 4 * (lane >> 5) + 2 * ((lane >> 4) & 1);
}

// Inclusive scans over the lanes of a wave without LDS traffic (gfx9 DPP):
// shifts by 1, 2, 4 and 8 lanes within each row of 16, then each row's last
// lane carried into the next row by row broadcasts.  W = 32 scans lanes 0-31
// and 32-63 separately, W = 64 the whole wave.  A lane whose shifted source
// lies before its row's start, or a row left out of a broadcast, reads the
// identity idn.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_or(float x, float idn) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, idn),
                                                               __builtin_bit_cast(int, x), CTRL,
                                                               ROWS, 0xF, false));
}
struct ScanAdd {
  __device__ float operator()(float a, float b) const { return a + b; }
};
struct ScanMax {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
template <int W, class Op>
__device__ __forceinline__ float wave_scan(float x, float idn, Op op) {
  static_assert(W == 32 || W == 64, "scan width");
  x = op(x, dpp_or<0x111>(x, idn));        // row_shr:1
  x = op(x, dpp_or<0x112>(x, idn));        // row_shr:2
  x = op(x, dpp_or<0x114>(x, idn));        // row_shr:4
  x = op(x, dpp_or<0x118>(x, idn));        // row_shr:8
  x = op(x, dpp_or<0x142, 0xA>(x, idn));   // row_bcast:15 into rows 1 and 3
  if constexpr (W == 64) x = op(x, dpp_or<0x143, 0xC>(x, idn));   // row_bcast:31 into rows 2, 3
  return x;
}
// Lane l's value of x in every lane (v_readlane: a scalar result).
__device__ __forceinline__ float lane_bcast(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

template <int FB>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (FB == 8) x += dpp<0x128>(x);     // row_ror:8
  return swap_sum32(swap_sum16(x));
}

}  // namespace
}  // namespace la
