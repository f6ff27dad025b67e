// Delta_i = sum_d dO_id O_id of every (token, head) row, the row constant of
// the backward's dS = P (dP - Delta), stored with lse * log2(e) as one pair so
// that one 8-byte load gives a row's two softmax constants.
//
// Rows are (token, head) pairs in memory order, so reads and writes both
// stream: TPR threads take the 16-byte pieces of a row, each thread has
// kDeltaPasses rows' loads in flight together, and the pieces' products are
// added across the TPR threads.
#pragma once
#include "jfa_common.h"
#include "jfa_kernels.h"

namespace jfa {

constexpr int kDeltaPasses = 4;

template <typename T, int D, int THREADS>
struct DeltaShape {
  static constexpr int ROWB = D * (int)sizeof(T), TPR = ROWB / 16;  // threads per row
  static constexpr int RPP = THREADS / TPR;                         // rows per pass of the workgroup
  static constexpr int RPB = RPP * kDeltaPasses;                    // rows per workgroup
};

// Rows [blk * RPB, (blk + 1) * RPB) of the THREADS-thread workgroup's share.
template <typename T, int D, int THREADS>
__device__ __forceinline__ void delta_rows(const BwdArgs& a, long blk, int tid) {
  using S = DeltaShape<T, D, THREADS>;
  const long rows = a.tq * a.H;
  const int part = tid % S::TPR;
  const long r0 = blk * S::RPB + tid / S::TPR;
  i32x4 o[kDeltaPasses], d[kDeltaPasses];
  float l[kDeltaPasses];
#pragma unroll
  for (int k = 0; k < kDeltaPasses; ++k) {
    const long row = r0 + k * S::RPP;
    o[k] = d[k] = (i32x4){};
    l[k] = 0.f;
    if (row < rows) {
      o[k] = *(const i32x4*)((const char*)a.out + row * S::ROWB + part * 16);
      d[k] = *(const i32x4*)((const char*)a.dout + row * S::ROWB + part * 16);
      if (part == 0) l[k] = a.lse[row];
    }
  }
#pragma unroll
  for (int k = 0; k < kDeltaPasses; ++k) {
    float acc = 0.f;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 o8 = __builtin_bit_cast(bf16x8, o[k]), d8 = __builtin_bit_cast(bf16x8, d[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)o8[e] * (float)d8[e];
    } else {
      const f32x4 o4 = __builtin_bit_cast(f32x4, o[k]), d4 = __builtin_bit_cast(f32x4, d[k]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += o4[e] * d4[e];
    }
#pragma unroll
    for (int s = S::TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
    const long row = r0 + k * S::RPP;
    // a row that sees no key (lse = -inf) gets +inf, so that its P = 2^(s - c) is 0 for every key
    if (row < rows && part == 0) a.rowc[row] = make_float2(l[k] == -INFINITY ? INFINITY : l[k] * kLog2e, acc);
  }
}

}  // namespace jfa
