// Shared device helpers for the gfx950 jagged-attention kernels.
//
// Data layout (all tensors packed, no padding between sequences):
//   q, k, v, out, dout, dq, dk, dv : [T, H, D] row-major, D contiguous
//   lse, delta                     : [T, H] fp32
//   offsets                        : int32 [B+1], prefix sums of lengths
// A sequence b of head h is a strided view: row r lives at
//   base + ((offsets[b] + r) * H + h) * D.
//
// Jagged edges ("Jagged Flash Attention (JFA)", section "Four generations",
// item 1): rows past a sequence's end are read as zeros and never written.
// On gfx950 this is done by a buffer resource whose record count ends at the
// sequence's last row: out-of-range loads return 0 and out-of-range stores are
// dropped by the hardware range check.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jfa {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) char lds_t;

constexpr int kBiasRadius = 128;
constexpr int kBiasLen = 2 * kBiasRadius + 1;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInit = -1.0e30f;  // running-max start value (finite: keeps exp2(m_old - m_new) at 0)
constexpr float kRescaleSlack = 8.0f;  // log2 units: the running max lags the true max by at most this, so P <= 256

// ---------------------------------------------------------------------------
// Buffer views with hardware range checks.
struct View {
  __amdgpu_buffer_rsrc_t r;
};

__device__ __forceinline__ View make_view(const void* base, uint32_t bytes) {
  View v;
  v.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
  return v;
}

// Rows [0, rows) of one (sequence, head) slice: row stride `row_stride` bytes,
// `row_bytes` valid bytes per row.
__device__ __forceinline__ View seq_view(const void* base, int rows, uint32_t row_stride, uint32_t row_bytes) {
  uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * row_stride + row_bytes : 0u;
  return make_view(base, bytes);
}

__device__ __forceinline__ i32x4 ld16(const View& v, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(v.r, off, 0, 0);
}
__device__ __forceinline__ float ld4f(const View& v, uint32_t off) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(v.r, off, 0, 0));
}
__device__ __forceinline__ i32x2 ld8(const View& v, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(v.r, off, 0, 0);
}
__device__ __forceinline__ void st16(const View& v, uint32_t off, i32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, v.r, off, 0, 0);
}
__device__ __forceinline__ void st8(const View& v, uint32_t off, i32x2 x) {
  __builtin_amdgcn_raw_buffer_store_b64(x, v.r, off, 0, 0);
}
__device__ __forceinline__ void st4f(const View& v, uint32_t off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(x), v.r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// MFMA fragments. A fragment is the 8 k-values one lane feeds into a 16-deep
// slice of a 32x32 product: lane l (half g = l / 32) owns k-slots 8g .. 8g+7.
// bf16 uses one v_mfma_f32_32x32x16_bf16; fp32 issues eight
// v_mfma_f32_32x32x2_f32 (k-slot 8g+e goes in step e), same contraction.
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ void mma(f32x16& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[e], b.hi[e], c, 0, 0, 0);
}

// Fragment from 8 consecutive elements in global memory (natural layout).
__device__ __forceinline__ Frag<bf16> gfrag(const View& v, uint32_t off, bf16*) {
  i32x4 x = ld16(v, off);
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, x);
  return f;
}
__device__ __forceinline__ Frag<float> gfrag(const View& v, uint32_t off, float*) {
  Frag<float> f;
  f.lo = __builtin_bit_cast(f32x4, ld16(v, off));
  f.hi = __builtin_bit_cast(f32x4, ld16(v, off + 16));
  return f;
}

// ---------------------------------------------------------------------------
// LDS tiles: ROWS x D elements, rows of ROWB = D * sizeof(T) bytes with no
// padding. The 16-byte chunks of each row are permuted by an XOR with a
// function of the row, chosen so that (on the 64-bank, 4-byte LDS of gfx950)
//   * 16-byte operand reads (16 lanes per cycle, 16 consecutive rows, same
//     chunk),
//   * transposing reads (32 lanes per cycle, 4 consecutive rows x 64 bytes),
//   * 16-byte staging writes (whole rows)
// each touch every bank at most once per cycle.
// Chunk permutation of the LDS tiles: 1 (the library) XORs each row's
// 16-byte chunk index with a function of the row so that the MFMA operand
// reads spread over the banks; 0 exists only for a bank-conflict study.
#ifndef JFA_LDS_SWIZZLE
#define JFA_LDS_SWIZZLE 1
#endif
template <typename T, int D>
struct Tile {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int CPR = ROWB / 16;
  __device__ __forceinline__ static int swz(int r) {
    if constexpr (!JFA_LDS_SWIZZLE) return 0;  // swizzle study only: rows stored unpermuted
    if constexpr (CPR >= 16) return 4 * (r & 3) + ((r >> 2) & 3);
    else if constexpr (CPR == 8) return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
    else return (r >> 2) & 3;
  }
  // byte offset of 16-byte chunk c of row r
  __device__ __forceinline__ static int chunk(int r, int c) { return r * ROWB + ((c ^ swz(r)) << 4); }
  // byte offset of byte b (within the unpermuted row) of row r
  __device__ __forceinline__ static int byte(int r, int b) { return chunk(r, b >> 4) + (b & 15); }
};

// Fragment from 8 consecutive elements (row r, elements col .. col+7) of a tile.
template <int D>
__device__ __forceinline__ Frag<bf16> lfrag(const lds_t* tile, int r, int col, bf16*) {
  Frag<bf16> f;
  f.v = *(const __attribute__((address_space(3))) bf16x8*)(tile + Tile<bf16, D>::byte(r, col * 2));
  return f;
}
template <int D>
__device__ __forceinline__ Frag<float> lfrag(const lds_t* tile, int r, int col, float*) {
  Frag<float> f;
  f.lo = *(const __attribute__((address_space(3))) f32x4*)(tile + Tile<float, D>::byte(r, col * 4));
  f.hi = *(const __attribute__((address_space(3))) f32x4*)(tile + Tile<float, D>::byte(r, col * 4 + 16));
  return f;
}

// Transposed fragment: k runs down the rows of the tile, the lane's column is
// fixed. The k-slot order matches the row order of a 32x32 MFMA result held
// by the other operand: slot e of half g is row
//   rowbase + 4g + e        (e < 4)
//   rowbase + 8 + 4g + e-4  (e >= 4).
// bf16: two ds_read_b64_tr_b16. Each 16-lane group gives four row addresses
// (one per lane quad) and the hardware hands lane i the i-th column of those
// four rows. Column = colbase + (l & 31).
template <int D>
__device__ __forceinline__ Frag<bf16> tfrag(const lds_t* tile, int rowbase, int colbase, int lane, bf16*) {
  using TL = Tile<bf16, D>;
  const int g = lane >> 5;
  const int row = rowbase + 4 * g + ((lane & 15) >> 2);
  const int b = (colbase + ((lane & 31) >> 4) * 16 + (lane & 3) * 4) * 2;
  s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + TL::byte(row, b)));
  s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + TL::byte(row + 8, b)));
  Frag<bf16> f;
  bf16x4 x4 = __builtin_bit_cast(bf16x4, x), y4 = __builtin_bit_cast(bf16x4, y);
  f.v = (bf16x8){x4[0], x4[1], x4[2], x4[3], y4[0], y4[1], y4[2], y4[3]};
  return f;
}
template <int D>
__device__ __forceinline__ Frag<float> tfrag(const lds_t* tile, int rowbase, int colbase, int lane, float*) {
  using TL = Tile<float, D>;
  const int g = lane >> 5;
  const int b = (colbase + (lane & 31)) * 4;
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) f.lo[e] = *(const __attribute__((address_space(3))) float*)(tile + TL::byte(rowbase + 4 * g + e, b));
#pragma unroll
  for (int e = 0; e < 4; ++e) f.hi[e] = *(const __attribute__((address_space(3))) float*)(tile + TL::byte(rowbase + 8 + 4 * g + e, b));
  return f;
}

// Padded-row LDS tiles: row r at byte r * S, no permutation, so every
// fragment of a tile is one per-lane base address plus an immediate offset
// (no per-fragment address registers). Strides:
//   natural reads (16 lanes per cycle, 16 consecutive rows, one 16-byte
//   column): S = 16 * odd puts the rows in distinct 4-bank groups; rows of
//   an even number of 16-byte chunks padded by 16 bytes (pad_nat);
//   transposing reads (4 consecutive rows x 64 bytes per cycle): S = 64 * odd
//   puts the rows in distinct 16-bank groups; rows of an odd number of
//   64-byte quarters as they are, others padded by 64 bytes (pad_tr).
constexpr int pad_nat(int rowb) { return rowb + 16; }
constexpr int pad_tr(int rowb) { return (rowb / 64) % 2 == 1 ? rowb : rowb + 64; }

// 8 consecutive elements (row r, elements col .. col+7) of a padded-row tile.
template <int S>
__device__ __forceinline__ Frag<bf16> prfrag(const lds_t* tile, int r, int col, bf16*) {
  Frag<bf16> f;
  f.v = *(const __attribute__((address_space(3))) bf16x8*)(tile + r * S + col * 2);
  return f;
}
template <int S>
__device__ __forceinline__ Frag<float> prfrag(const lds_t* tile, int r, int col, float*) {
  Frag<float> f;
  f.lo = *(const __attribute__((address_space(3))) f32x4*)(tile + r * S + col * 4);
  f.hi = *(const __attribute__((address_space(3))) f32x4*)(tile + r * S + col * 4 + 16);
  return f;
}
// Transposed fragment (k down the rows, as tfrag) of a padded-row tile.
template <int S>
__device__ __forceinline__ Frag<bf16> ptfrag(const lds_t* tile, int rowbase, int colbase, int lane, bf16*) {
  const int g = lane >> 5;
  const int row = rowbase + 4 * g + ((lane & 15) >> 2);
  const int b = (colbase + ((lane & 31) >> 4) * 16 + (lane & 3) * 4) * 2;
  s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + row * S + b));
  s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + (row + 8) * S + b));
  Frag<bf16> f;
  bf16x4 x4 = __builtin_bit_cast(bf16x4, x), y4 = __builtin_bit_cast(bf16x4, y);
  f.v = (bf16x8){x4[0], x4[1], x4[2], x4[3], y4[0], y4[1], y4[2], y4[3]};
  return f;
}
template <int S>
__device__ __forceinline__ Frag<float> ptfrag(const lds_t* tile, int rowbase, int colbase, int lane, float*) {
  const int g = lane >> 5;
  const int b = (colbase + (lane & 31)) * 4;
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) f.lo[e] = *(const __attribute__((address_space(3))) float*)(tile + (rowbase + 4 * g + e) * S + b);
#pragma unroll
  for (int e = 0; e < 4; ++e) f.hi[e] = *(const __attribute__((address_space(3))) float*)(tile + (rowbase + 8 + 4 * g + e) * S + b);
  return f;
}

// Fragment from half (c = 0 or 1) of a 32x32 fp32 result: elements 8c .. 8c+7,
// i.e. rows 16c + {4g..4g+3, 8+4g..8+4g+3} of that result.
__device__ __forceinline__ Frag<bf16> rfrag(const f32x16& s, int c, bf16*) {
  Frag<bf16> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)s[8 * c + e];
  return f;
}
__device__ __forceinline__ Frag<float> rfrag(const f32x16& s, int c, float*) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.lo[e] = s[8 * c + e]; f.hi[e] = s[8 * c + 4 + e]; }
  return f;
}

// Sum of the 8 values of a fragment added to acc, in the fragment's own
// precision: for bf16 the rounded values the matrix product consumes (two per
// v_dot2c_f32_bf16 against a pair of ones, fp32 accumulation).
__device__ __forceinline__ float frag_sum(const Frag<bf16>& f, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){f.v[2 * e], f.v[2 * e + 1]}, one, acc, false);
  return acc;
}
__device__ __forceinline__ float frag_sum(const Frag<float>& f, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc += f.lo[e] + f.hi[e];
  return acc;
}
// The value a bf16 operand carries for x (round to nearest even), as fp32.
__device__ __forceinline__ float as_operand(float x, bf16*) { return (float)(bf16)x; }
__device__ __forceinline__ float as_operand(float x, float*) { return x; }

// A whole-wave fragment parked in LDS (16 bytes per lane per 1 KB piece, lane
// order), for handing an operand from one wave to another.
__device__ __forceinline__ void put_frag(lds_t* p, const Frag<bf16>& f, int lane) {
  *(__attribute__((address_space(3))) i32x4*)(p + 16 * lane) = __builtin_bit_cast(i32x4, f.v);
}
__device__ __forceinline__ void put_frag(lds_t* p, const Frag<float>& f, int lane) {
  *(__attribute__((address_space(3))) f32x4*)(p + 16 * lane) = f.lo;
  *(__attribute__((address_space(3))) f32x4*)(p + 1024 + 16 * lane) = f.hi;
}
__device__ __forceinline__ Frag<bf16> get_frag(const lds_t* p, int lane, bf16*) {
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) i32x4*)(p + 16 * lane));
  return f;
}
__device__ __forceinline__ Frag<float> get_frag(const lds_t* p, int lane, float*) {
  Frag<float> f;
  f.lo = *(const __attribute__((address_space(3))) f32x4*)(p + 16 * lane);
  f.hi = *(const __attribute__((address_space(3))) f32x4*)(p + 1024 + 16 * lane);
  return f;
}

// Wave-uniform copies (scalar registers) of values the compiler cannot prove
// uniform.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename P>
__device__ __forceinline__ P* uni(P* p) {
  const unsigned long long a = (unsigned long long)p;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
  return (P*)(((unsigned long long)hi << 32) | lo);
}

// Value held by the lane 32 positions away (other half of the wave).
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return (threadIdx.x & 32) ? __int_as_float(r[0]) : __int_as_float(r[1]);
}
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// Row (within a 32x32 MFMA result) of element i held by a lane of half g.
__device__ __forceinline__ constexpr int res_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Store 4 consecutive fp32 values as T (8 or 16 bytes) at byte offset off.
__device__ __forceinline__ void store4(const View& v, uint32_t off, float a, float b, float c, float d, bf16*) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 lo = {(bf16)a, (bf16)b}, hi = {(bf16)c, (bf16)d};
  i32x2 x = {__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
  st8(v, off, x);
}
__device__ __forceinline__ void store4(const View& v, uint32_t off, float a, float b, float c, float d, float*) {
  i32x4 x = {__float_as_int(a), __float_as_int(b), __float_as_int(c), __float_as_int(d)};
  st16(v, off, x);
}

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// ROWS rows of D fp32 values staged in LDS (Tile<float, D> layout) out to
// global memory as whole rows, each value times `mul` and rounded to T; row
// r goes to byte offset r * stride of `dst`, whose range drops rows past the
// sequence end.
template <typename T, int D, int ROWS, int THREADS>
__device__ __forceinline__ void rows_out(const lds_t* src, const View& dst, uint32_t stride, float mul, int tid) {
  using OL = Tile<float, D>;
  static_assert((ROWS * OL::CPR) % THREADS == 0, "row pieces divide the workgroup");
#pragma unroll
  for (int c = 0; c < ROWS * OL::CPR / THREADS; ++c) {
    const int x = tid + THREADS * c, row = x / OL::CPR, col = x % OL::CPR;
    const f32x4 v = *(const __attribute__((address_space(3))) f32x4*)(src + OL::chunk(row, col));
    store4(dst, (uint32_t)row * stride + col * 4 * (int)sizeof(T), v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul,
           (T*)0);
  }
}

// ---------------------------------------------------------------------------
// Direct global -> LDS tile loads. One wave instruction moves 64 x 16 bytes
// into 1 KB of LDS, lane l landing at byte 16*l (gfx950 buffer_load_dwordx4
// with the LDS bit; out-of-range lanes write zeros). The tile layout is
// permuted (Tile::swz), so each lane fetches the global 16-byte piece whose
// permuted position is its LDS slot.
//
// The instruction is issued from inline assembly on purpose: the compiler
// cannot tell which LDS stage a direct load writes, so for its own loads it
// waits for every outstanding one before any LDS read, which would make the
// prefetch ring synchronous. Here the kernels order the ring themselves with
// explicit vmcnt waits and barriers. M0 carries the LDS address; nothing else
// in these kernels uses M0.
struct DmaView {
  i32x4 w;  // buffer resource words: base, stride 0, record count, format
};

__device__ __forceinline__ DmaView dma_view(const void* base, int rows, uint32_t row_stride, uint32_t row_bytes) {
  const uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * row_stride + row_bytes : 0u;
  const unsigned long long a = (unsigned long long)base;
  DmaView v;
  v.w[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  v.w[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  v.w[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  v.w[3] = 0x00020000;
  return v;
}

__device__ __forceinline__ void dma16(const DmaView& v, const lds_t* dst, uint32_t voff) {
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(size_t)dst);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(v.w)
               : "memory", "m0");
}

// 1 KB block k of an LDS tile whose row 0 is row row0 of the view.
template <typename T, int D>
__device__ __forceinline__ void dma_block(const DmaView& v, uint32_t gstride, int row0, lds_t* tile, int k, int lane) {
  using TL = Tile<T, D>;
  const int P = k * 1024 + 16 * lane;
  const int r = P / TL::ROWB, pc = (P % TL::ROWB) >> 4;
  const uint32_t goff = (uint32_t)(row0 + r) * gstride + (uint32_t)((pc ^ TL::swz(r)) << 4);
  dma16(v, tile + k * 1024, goff);
}

// Rows row0 .. row0+ROWS-1 of the view into an LDS tile; the waves split the
// tile's 1 KB blocks.
template <typename T, int D, int ROWS, int WAVES>
__device__ __forceinline__ void dma_tile(const DmaView& v, uint32_t gstride, int row0, lds_t* tile, int wave, int lane) {
  constexpr int NBLK = ROWS * Tile<T, D>::ROWB / 1024;
  static_assert(NBLK % WAVES == 0 || NBLK < WAVES, "tile blocks divide the waves (or one block per wave)");
#pragma unroll
  for (int k = wave; k < NBLK; k += WAVES) dma_block<T, D>(v, gstride, row0, tile, k, lane);
}
template <typename T, int D, int ROWS, int WAVES>
constexpr int dma_loads_per_wave() {
  return ROWS * Tile<T, D>::ROWB / 1024 >= WAVES ? ROWS * Tile<T, D>::ROWB / 1024 / WAVES : 1;
}

// Direct loads into a padded-row tile (row r at byte r * S of an LDS region
// of NBLK whole KBs): 1 KB block k holds LDS bytes [1024 k, 1024 k + 1024),
// so lane l fills byte P = 1024 k + 16 l: row P / S, byte P % S of it. Lanes
// whose slot is a row's padding, or past the tile's ROWS rows, get an offset
// beyond the view's range and write zeros.
template <int ROWS, int ROWB, int S>
struct PaddedDma {
  static constexpr int NBLK = (ROWS * S + 1023) / 1024;
};
template <int ROWS, int ROWB, int S, int WAVES>
__device__ __forceinline__ void dma_padded_tile(const DmaView& v, uint32_t gstride, int row0, lds_t* tile, int wave,
                                                int lane) {
  constexpr int NBLK = PaddedDma<ROWS, ROWB, S>::NBLK;
#pragma unroll
  for (int i = 0; i < (NBLK + WAVES - 1) / WAVES; ++i) {
    const int k = wave + i * WAVES;
    if (k >= NBLK) break;  // wave-uniform
    const int P = k * 1024 + 16 * lane, r = P / S, cb = P % S;
    const uint32_t goff = (r < ROWS && cb < ROWB) ? (uint32_t)(row0 + r) * gstride + (uint32_t)cb : 0xFFFFFFF0u;
    dma16(v, tile + k * 1024, goff);
  }
}

// s_waitcnt with vmcnt = n (0..63), expcnt and lgkmcnt left alone. The count
// must be a compile-time constant, so small runtime values are dispatched.
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most n (uniform across the wave) vector-memory operations of
// this wave are outstanding; n above 3 waits for 3 (stricter, still correct).
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if (n <= 0) wait_vmcnt_c<0>();
  else if (n == 1) wait_vmcnt_c<1>();
  else if (n == 2) wait_vmcnt_c<2>();
  else wait_vmcnt_c<3>();
}
template <int STEP, int MAXK>
__device__ __forceinline__ void wait_vmcnt_tiles(int k) {  // wait until at most k*STEP loads remain
  if constexpr (MAXK <= 0) {
    wait_vmcnt_c<0>();
  } else {
    if (k >= MAXK) wait_vmcnt_c<MAXK * STEP>();
    else wait_vmcnt_tiles<STEP, MAXK - 1>(k);
  }
}

// Wait until every outstanding vector-memory load of this wave has landed.
// Used once per work item after the register-resident operand fragments are
// loaded: it tells the compiler's wait-count tracking that nothing older than
// the tile prefetches is in flight inside the main loop, so the MFMAs there
// do not wait on the next tile's prefetch.
__device__ __forceinline__ void wait_vmem() {
  // gfx9 s_waitcnt encoding: vmcnt = 0, expcnt = 7 (bits 6:4), lgkmcnt = 15 (bits 11:8)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Wave priority around the matrix-product clusters: a wave that reaches its
// MFMAs is issued ahead of the SIMD's other waves (which are then in their
// softmax VALU work), so the matrix pipe is refilled as soon as one of them
// has products ready. Measured: forward -2 to -3% (D = 64 and 128), one-role
// dK/dV kernel -2%; the paired-wave dK/dV kernel and the dQ kernel were
// 0.5-1% slower with it and do not use it.
__device__ __forceinline__ void prio_mfma() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void prio_valu() { __builtin_amdgcn_s_setprio(0); }

// Instruction interleave for the scheduler, N times: DS LDS reads, MF matrix
// products, VA other vector ALU instructions (a pattern, not a count: a group
// takes what is left when fewer remain). Placed at the end of a code region
// whose matrix products and VALU work are independent, it makes the
// compiler issue them alternately, so one wave's VALU work runs while its
// products occupy the matrix core.
template <int DS, int MF, int VA, int N>
__device__ __forceinline__ void sched_pattern() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if constexpr (DS > 0) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
    if constexpr (VA > 0) __builtin_amdgcn_sched_group_barrier(0x002, VA, 0);
  }
}

// Operand prefetch for a run of N matrix products whose operands come from
// LDS, DS reads per product: the first AHEAD products' reads are issued up
// front, then each product is followed by the reads of the one AHEAD places
// later, so AHEAD products' operands are in flight instead of each read
// being waited for right before its product.
template <int N, int DS, int AHEAD>
__device__ __forceinline__ void sched_prefetch() {
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, DS, 1);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, DS, 1);
  }
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
}

// Work-list header in the caller's workspace: kMaxQueues queues stored one
// after the other in the item array (one queue per XCD). Each queue's ticket
// sits on its own 128-byte line, away from the read-only words, so that the
// atomics of one queue do not serialise the others' traffic in L2.
constexpr int kMaxQueues = 8;
struct PlanHeader {
  int count;                 // items in all queues
  int status;                // 0 ok, 1 the list did not fit the workspace
  int nq;                    // queues in use
  int pad0;
  int start[kMaxQueues];     // first item of each queue
  int qcount[kMaxQueues];    // items of each queue
  int pad1[12];
  struct {
    int value;               // next item of the queue to hand out (zeroed by the plan kernel)
    int pad[31];
  } ticket[kMaxQueues];
  int pad2[224];
};
static_assert(sizeof(PlanHeader) == 2048, "header is 2048 bytes");

// Per-workgroup copy of the queue bounds plus the work-list cursor.
struct QueueCursor {
  int start[kMaxQueues];
  int count[kMaxQueues];
  int nq;
  int item;  // broadcast slot
};

// Loads the queue bounds into LDS (call once, before the first next_item;
// the barrier inside next_item orders it).
__device__ __forceinline__ void load_queues(const PlanHeader* hdr, QueueCursor* qc) {
  if (threadIdx.x < kMaxQueues) {
    qc->start[threadIdx.x] = hdr->start[threadIdx.x];
    qc->count[threadIdx.x] = hdr->qcount[threadIdx.x];
  }
  if (threadIdx.x == kMaxQueues) qc->nq = max(hdr->nq, 1);
}

// Per-workgroup ticket state, meaningful in thread 0 only.
struct TicketState {
  int q = 0;      // queue being drained
  int left = -1;  // queues not yet found empty (< 0: not started)
};

// Next work item for this workgroup. Thread 0 takes tickets from its home
// queue (the one its XCD drains) and, once that is empty, from the others in
// turn. Tickets are taken one at a time, when the previous item is done: a
// workgroup never holds a claim on an item it is not working on, so the
// longest-first order decides which items start first. Queues the plan
// left empty are passed over without touching their ticket, so a pass with
// no items (a batch without short-query sequences, say) ends at once.
// Returns -1 when every queue is empty.
__device__ __forceinline__ int next_item(PlanHeader* hdr, QueueCursor* qc, TicketState& ts) {
  __syncthreads();  // queue bounds loaded; every wave is done with the previous item's slot
  if (threadIdx.x == 0) {
    if (ts.left < 0) {
      ts.q = (int)(blockIdx.x % (unsigned)qc->nq);
      ts.left = qc->nq;
    }
    int it = -1;
    while (ts.left > 0) {
      if (qc->count[ts.q] > 0) {
        const int t = __hip_atomic_fetch_add(&hdr->ticket[ts.q].value, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t < qc->count[ts.q]) {
          it = qc->start[ts.q] + t;
          break;
        }
      }
      ts.q = ts.q + 1 == qc->nq ? 0 : ts.q + 1;
      ts.left -= 1;
    }
    qc->item = it;
  }
  __syncthreads();
  // The same value in every lane: item fields, views and addresses derived
  // from it then live in scalar registers.
  return __builtin_amdgcn_readfirstlane(qc->item);
}

}  // namespace jfa
