// Gradient of the relative-position bias table beta[h, clip(i - j, -R, R) + R].
//
// The bias enters each score additively, so its gradient is the sum of
// dS = P * (dP - Delta) (the gradient with respect to the score) over every
// visible (query, key) pair of the head that falls in the bin (the
// definition's bias reading; "Jagged Flash Attention (JFA)", section
// "Definition", names custom attention biases among the method's inputs).
//
// The kernels that form dS in 32 x 32 blocks (the dK/dV pass and the
// short-query owner) fold each block into a per-wave histogram of the 257
// bins in LDS. A block whose pairs all lie beyond the radius adds to one end
// bin: its entries are summed per lane in registers over the whole item and
// reduced once at the end. Any other block is summed along its 63 diagonals,
// one lane per diagonal and each diagonal one bin (from a per-wave LDS
// scratch, or from the dS tile a kernel already keeps in LDS); distances
// beyond the radius join the end bins' register sums. At the end of an item
// the waves' histograms are added in wave order into the item's slot of the
// workspace; jfa_dbias_part_kernel and jfa_dbias_kernel then sum the slots
// of each head over fixed blocks of sequences, and the blocks, in order.
// Every sum has a fixed order, so the gradient is bit-identical run to run,
// and no atomics are used.
#pragma once
#include "jfa_common.h"

namespace jfa {

constexpr int kDbHistLen = 260;                   // 257 bins, padded
constexpr int kDbWaveBytes = (32 * 33 + kDbHistLen) * 4;  // scratch block (rows padded to 33) + histogram
constexpr int kDbHistBytes = kDbHistLen * 4;              // histogram only (dS read from a tile already in LDS)

// Per-wave state: the histogram in LDS and the far-bin sums in registers.
struct DbWave {
  __attribute__((address_space(3))) float* hist;     // [kDbHistLen]
  __attribute__((address_space(3))) float* scratch;  // [32][33]
  float lo = 0.f, hi = 0.f;                          // this lane's sums for bin 0 and bin 2R
};

__device__ __forceinline__ DbWave db_wave(lds_t* base, int wave_slot) {
  DbWave s;
  s.scratch = (__attribute__((address_space(3))) float*)(base + wave_slot * kDbWaveBytes);
  s.hist = s.scratch + 32 * 33;
  return s;
}

// A wave with a histogram slot only (slots of kDbHistBytes).
__device__ __forceinline__ DbWave db_wave_hist(lds_t* base, int wave_slot) {
  DbWave s;
  s.scratch = nullptr;
  s.hist = (__attribute__((address_space(3))) float*)(base + wave_slot * kDbHistBytes);
  return s;
}

// Sum over the 64 lanes in a fixed butterfly order; every lane gets the sum.
__device__ __forceinline__ float db_wave_sum(float x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ void db_begin(DbWave& s, int lane) {
  for (int r = lane; r < kDbHistLen; r += 64) s.hist[r] = 0.f;
  s.lo = s.hi = 0.f;
}

// A 32 x 32 block of dS in MFMA result layout (lane (j, g) holds key column j
// at query rows res_row(e, g)), with qk = (first query of the block) -
// (first key of the block), both local to the sequence. If every pair of the
// block lies beyond the radius on one side, its entries join that end bin's
// register sums and true is returned.
__device__ __forceinline__ bool db_far(DbWave& s, const f32x16& ds, int qk) {
  if (!(qk + 31 <= -kBiasRadius || qk - 31 >= kBiasRadius)) return false;
  float t = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) t += ds[e];
  if (qk < 0) s.lo += t;
  else s.hi += t;
  return true;
}

// v: this lane's diagonal sum, diagonal i - j = lane - 31 (lanes 0 .. 62) of
// a block with offset qk; adds it to its bin (distinct bins across lanes;
// distances beyond the radius go to the end bins' register sums).
__device__ __forceinline__ void db_diag(DbWave& s, float v, int qk, int lane) {
  const int bin = min(max(qk + lane - 31, -kBiasRadius), kBiasRadius) + kBiasRadius;
  s.lo += (lane < 63 && bin == 0) ? v : 0.f;
  s.hi += (lane < 63 && bin == 2 * kBiasRadius) ? v : 0.f;
  if (lane < 63 && bin > 0 && bin < 2 * kBiasRadius) s.hist[bin] += v;
}

// Adds one block of dS (layout above) to the wave's bins, through the wave's
// LDS scratch when it straddles the radius. Called by the whole wave.
__device__ __forceinline__ void db_block(DbWave& s, const f32x16& ds, int qk, int lane) {
  if (db_far(s, ds, qk)) return;
  const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int e = 0; e < 16; ++e) s.scratch[res_row(e, g) * 33 + l32] = ds[e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int d = lane - 31;  // diagonal i - j of this lane
  float v = 0.f;
  if (lane < 63) {
    const int i0 = max(0, d), i1 = min(32, 32 + d);
    for (int i = i0; i < i1; ++i) v += s.scratch[i * 33 + (i - d)];
  }
  db_diag(s, v, qk, lane);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();  // scratch reads done before the next block's writes
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// End of the item for this wave: the far-bin sums join the histogram.
__device__ __forceinline__ void db_finish(DbWave& s, int lane) {
  const float lo = db_wave_sum(s.lo), hi = db_wave_sum(s.hi);
  if (lane == 0) s.hist[0] += lo;
  if (lane == 1) s.hist[2 * kBiasRadius] += hi;
}

// The item's bins: histograms of waves 0 .. nwaves-1 (slots of slot_bytes
// from base, the histogram hist_off bytes into each), added in wave order,
// to out[0 .. 256]. After a barrier that follows every wave's db_finish; run
// by threads [0, nthreads).
__device__ __forceinline__ void db_store(const lds_t* base, int nwaves, float* out, int t, int nthreads,
                                         int slot_bytes = kDbWaveBytes, int hist_off = 32 * 33 * 4) {
  for (int r = t; r < kBiasLen; r += nthreads) {
    float acc = 0.f;
    for (int w = 0; w < nwaves; ++w)
      acc += ((const __attribute__((address_space(3))) float*)(base + w * slot_bytes + hist_off))[r];
    out[r] = acc;
  }
}

}  // namespace jfa
