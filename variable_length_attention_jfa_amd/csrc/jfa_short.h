// Second step of the short-query passes: per (b, h), the chunks' results are
// combined in list order. The chunk passes run in their own launch first, so
// their rows are visible here through the launch boundary; the combining
// runs at the start of a launch that follows anyway (the query-tile forward,
// the dQ pass), spread over its workgroups.
#pragma once
#include "jfa_common.h"
#include "jfa_kernels.h"

namespace jfa {

// LDS the combining steps use at the start of a workgroup's LDS: chunk
// weights [16][64] and per-row max and sum (forward), then the list of this
// workgroup's groups and its length.
constexpr int kMergeNB = 16;
constexpr int kShortGroupsOff = (kMergeNB + 2) * kSqQMax * 4;
constexpr int kShortLds = kShortGroupsOff + 257 * 4;

// Runs f(gi) for every (b, h) group gi with a short-query chunk list
// (gfirst[gi] >= 0; gfirst null: the call has no short-query pass); group gi
// belongs to workgroup gi % gridDim.x. Every thread of the workgroup calls f
// with the same gi.
template <typename F>
__device__ __forceinline__ void for_short_groups(const int* gfirst, int ngroups, lds_t* lds, F&& f) {
  if (gfirst == nullptr) return;  // no short-query pass in this call
  int* list = (int*)(lds + kShortGroupsOff);
  int* count = list + 256;
  const int per = ((int)gridDim.x - 1 + ngroups - (int)blockIdx.x) / (int)gridDim.x;  // groups of this workgroup
  for (int base = 0; base < per; base += 256) {
    if (threadIdx.x == 0) *count = 0;
    __syncthreads();
    const int k = base + (int)threadIdx.x;
    if (threadIdx.x < 256 && k < per) {  // the list holds 256 groups
      const int gi = (int)blockIdx.x + k * (int)gridDim.x;
      if (gfirst[gi] >= 0) list[atomicAdd(count, 1)] = gi;
    }
    __syncthreads();
    const int n = uni(*count);
    for (int i = 0; i < n; ++i) f(uni(list[i]));
    __syncthreads();
  }
}

// O and lse of short-query group gi from its chunks: M = max_c lse2_c,
// w_c = 2^(lse2_c - M), O = sum_c (w_c / sum w) O_c, lse = (M + log2 sum w)
// ln 2, with the chunks in list order. The first 64 threads find each row's
// max and sum of weights, the weights go through LDS in batches of 16
// chunks, and every thread accumulates four columns of its rows, the chunk
// loop unrolled so that loads overlap. NT: threads of the workgroup.
template <typename T, int D, int NT = 256>
__device__ __forceinline__ void fsq_merge(const FwdArgs& a, int gi, lds_t* lds) {
  constexpr int QM = kSqQMax, DV = D / 4, NB = kMergeNB, EPT = QM * DV / NT;
  static_assert(QM * DV % NT == 0, "row quads divide the workgroup");
  __attribute__((address_space(3))) float* wl = (__attribute__((address_space(3))) float*)lds;  // [NB][QM]
  __attribute__((address_space(3))) float* mrow = wl + NB * QM;
  __attribute__((address_space(3))) float* srow = mrow + QM;
  const int tid = threadIdx.x, b = gi / a.H, h = gi % a.H, first = a.gfirst[gi];
  const int q0 = a.q_off[b], Lq = min(a.q_off[b + 1] - q0, QM);
  const int n = cdiv(a.kv_off[b + 1] - a.kv_off[b], kSqKC);
  const float* lp = a.lsep + (size_t)first * QM;  // chunk c, row q at lp[c * QM + q]
  if (tid < Lq) {
    float M = -INFINITY, S = 0.f;
#pragma unroll 4
    for (int c = 0; c < n; ++c) M = fmaxf(M, lp[c * QM + tid]);
    if (M > -INFINITY) {
#pragma unroll 4
      for (int c = 0; c < n; ++c) S += __builtin_amdgcn_exp2f(lp[c * QM + tid] - M);
    }
    mrow[tid] = M;
    srow[tid] = S;
    a.lse[(size_t)(q0 + tid) * a.H + h] = S > 0.f ? (M + __builtin_amdgcn_logf(S)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  f32x4 acc[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < n; c0 += NB) {
    const int nb = min(NB, n - c0);
    for (int i = tid; i < nb * QM; i += NT) {
      const int c = i / QM, q = i % QM;
      wl[c * QM + q] = q < Lq && srow[q] > 0.f ? __builtin_amdgcn_exp2f(lp[(c0 + c) * QM + q] - mrow[q]) / srow[q] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + NT * j, q = e / DV, d = (e % DV) * 4;
      if (q < Lq) {
        const float* src = a.op + ((size_t)(first + c0) * QM + q) * D + d;
#pragma unroll 4
        for (int c = 0; c < nb; ++c) acc[j] += wl[c * QM + q] * *(const f32x4*)(src + (size_t)c * QM * D);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + NT * j, q = e / DV, d = (e % DV) * 4;
    if (q < Lq) {
      T* dst = (T*)a.out + ((size_t)(q0 + q) * a.H + h) * D + d;
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = (T)acc[j][k];
    }
  }
}

// dQ of short-query group gi: the sum, in list order, of its chunks' partials,
// times the softmax scale. Four columns per thread, chunks unrolled so that
// their loads overlap.
template <typename T, int D>
__device__ __forceinline__ void sq_reduce(const BwdArgs& a, int gi) {
  constexpr int QM = kSqQMax;
  const int b = gi / a.H, h = gi % a.H, first = a.gfirst[gi];
  const int q0 = a.q_off[b], Lq = min(a.q_off[b + 1] - q0, QM);
  const int n = cdiv(a.kv_off[b + 1] - a.kv_off[b], kSqKC);
  const float* part = a.dqp + (size_t)first * QM * D;
  for (int e = threadIdx.x * 4; e < Lq * D; e += 256 * 4) {
    const int q = e / D, d = e % D;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int t = 0; t < n; ++t) s += *(const f32x4*)(part + (size_t)t * QM * D + e);
    T* dst = (T*)a.dq + ((size_t)(q0 + q) * a.H + h) * D + d;
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = (T)(s[k] * a.scale);
  }
}

}  // namespace jfa
