// Offsets-driven, longest-first work lists for the persistent kernels, and the
// lengths -> offsets scan.
//
// Short sequences must not leave compute units idle ("Jagged Flash Attention
// (JFA)", section "Why standard FlashAttention falls short"), and the kernels
// are persistent ("Four generations", item 3). The lists are built on the GPU
// from the offsets, so no host round trip is needed:
//
//   tiles  : q pass  -> (b, t) with t < ceil(Lq_b / TM)
//            kv pass -> (b, t) with t < ceil(Lk_b / TN)
//            sq pass -> (b, c) with c < max(1, ceil(Lk_b / TN)), only for
//                       sequences with Lq_b <= 64 (which the backward's q and
//                       kv passes then skip)
//   cost   : key blocks (q pass) or query blocks (kv pass) the tile visits;
//            keys in the chunk (sq pass)
//   groups : the tiles of one (b, h); group cost = sum of its tile costs
//   order  : groups by cost descending, then b, then h; group rank g is dealt
//            to queue snake(g) (0..Q-1, Q-1..0, ...), one queue per XCD, so
//            that the items sharing one (b, h)'s keys and values run on one
//            XCD and share its L2; inside a group, tiles by cost descending,
//            then t ascending
//   items  : (b, h, t, cost), queues stored one after the other
//
// One 1024-thread workgroup builds one list: sequences are ranked by a bitonic
// sort of (group cost, b) in LDS; group positions inside each queue come from
// one block-wide scan per chunk of 1024 groups, laid out so that each queue's
// groups are contiguous in the scan. All integer arithmetic in a fixed order:
// the list is the same on every run.
#include "jfa_common.h"
#include "jfa_kernels.h"
#include "jfa_delta.h"

namespace jfa {

#ifndef JFA_SCHED_LPT
#define JFA_SCHED_LPT 1
#endif

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanMaxB = 8192;

// A pass's tile shape; TM and TN are powers of two (checked at launch), so
// the divisions below are shifts.
struct PlanGeom {
  int kind, TM, TN, lgTM, lgTN, short_q;
};

__device__ __forceinline__ PlanGeom plan_geom(const PlanPass& p) {
  return {p.kind, p.TM, p.TN, __builtin_ctz((unsigned)p.TM), __builtin_ctz((unsigned)p.TN), p.short_q};
}

__device__ __forceinline__ int cdiv_lg(int a, int lg) { return (a + (1 << lg) - 1) >> lg; }

__device__ __forceinline__ int plan_tiles(int Lq, int Lk, const PlanGeom& p) {
  if (p.kind == kPassSQ) return short_query(Lq, Lk) ? cdiv_lg(Lk, p.lgTN) : 0;
  if (Lq <= p.short_q && Lk > kSqKC) return 0;
  return p.kind == kPassKV ? cdiv_lg(Lk, p.lgTN) : cdiv_lg(Lq, p.lgTM);
}

__device__ __forceinline__ int plan_cost(int Lq, int Lk, int t, const PlanGeom& p, int causal) {
  if (p.kind == kPassSQ) return max(0, min(p.TN, Lk - t * p.TN));
  if (p.kind == kPassQ) {
    if (!causal) return cdiv_lg(Lk, p.lgTN);
    return cdiv_lg(min(min((t + 1) * p.TM, Lq), Lk), p.lgTN);
  }
  const int nq = cdiv_lg(Lq, p.lgTM);
  if (!causal) return nq;
  const int first_key = t * p.TN;
  if (first_key >= Lq) return 0;
  return nq - (first_key >> p.lgTM);
}

// Position of tile t in its group's order (cost descending, then t ascending).
// Costs are monotone in t: non-increasing in the causal kv pass and constant
// without the causal mask, so the order is t itself there. In the causal q
// pass cost(t) = ceil(min((t+1)*TM, Lq, Lk) / TN) is non-decreasing: the tiles
// with cost c are t in [floor((c-1)*TN/TM), t1) with t1 = floor(c*TN/TM) if
// some tile reaches cost c+1 (min(Lq, Lk) > c*TN), else n. Tile t comes after
// the n - t1 tiles of larger cost and the t - t0 tiles of equal cost before it.
__device__ __forceinline__ int plan_pos(int Lq, int Lk, int t, int n, const PlanGeom& p, int causal) {
  const int lmin = min(Lq, Lk);
  if (!causal || p.kind != kPassQ || lmin == 0) return t;
  const int c = plan_cost(Lq, Lk, t, p, causal);
  const int t0 = ((c - 1) * p.TN) >> p.lgTM;
  const int t1 = lmin > c * p.TN ? min((c * p.TN) >> p.lgTM, n) : n;
  return (n - t1) + (t - t0);
}

__device__ __forceinline__ int snake(int g, int nq) {
  const int r = g % (2 * nq);
  return r < nq ? r : 2 * nq - 1 - r;
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active):
// DPP shifts by 1, 2, 4 and 8 lanes inside each 16-lane row, then the sum at
// the end of row 0 carried into row 1, of row 2 into row 3, and of rows 0-1
// (lane 31) into rows 2 and 3. Lanes a shift leaves without a source add 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}

// Exclusive scan over the workgroup; returns the prefix, *total gets the sum.
// Called by every thread of the workgroup.
__device__ int block_exclusive_scan(int v, int* total, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (threadIdx.x < 64) {  // wave 0, whole: the waves' totals
    const int s = wave_inclusive_scan(threadIdx.x < kPlanWaves ? wsum[threadIdx.x] : 0);
    if (threadIdx.x < kPlanWaves) wsum[kPlanWaves + threadIdx.x] = s;  // inclusive wave prefix
  }
  __syncthreads();
  const int before = w > 0 ? wsum[kPlanWaves + w - 1] : 0;
  *total = wsum[2 * kPlanWaves - 1];
  __syncthreads();
  return before + x - v;
}

// LDS of one pass: the static scan and queue arrays below, and
// plan_dyn_bytes(B) of dynamic LDS for the per-sequence arrays (sort keys,
// then query and key lengths), sized by the power of two P >= B.
__host__ __device__ inline int plan_pow2(int B) {
  int P = 2;
  while (P < B) P <<= 1;
  return P;
}
inline size_t plan_dyn_bytes(int B) { return (size_t)plan_pow2(B) * (8 + 4 + 4); }

// Builds the list of pass `pi` of `a`; one 1024-thread workgroup.
__device__ __forceinline__ void plan_pass(const PlanArgs& a, int pi, char* dyn) {
  const int P = plan_pow2(a.B);
  unsigned long long* key = (unsigned long long*)dyn;  // (inverted group cost, b), sorted ascending
  int* lq_s = (int*)(key + P);                          // sequence lengths
  int* lk_s = lq_s + P;
  __shared__ int wsum[2 * kPlanWaves];
  __shared__ int qtotal[kMaxQueues], qstart[kMaxQueues], qcarry[kMaxQueues];
  __shared__ int excl[kPlanThreads];
  // item writing of one chunk: per thread (group) its first list position, its
  // sequence and head, and the end of its items in the chunk's thread order
  __shared__ int wbase[kPlanThreads], wbh[kPlanThreads], wend[kPlanThreads];

  const PlanPass p = a.pass[pi];
  const PlanGeom pg = plan_geom(p);
  const int tid = threadIdx.x;
  const int B = a.B, H = a.H, NQ = p.nq;

  // 1. tiles and group cost of every sequence
  for (int b = tid; b < P; b += kPlanThreads) {
    unsigned long long k = ~0ull;
    if (b < B) {
      const int Lq = a.q_off[b + 1] - a.q_off[b], Lk = a.kv_off[b + 1] - a.kv_off[b];
      const int n = plan_tiles(Lq, Lk, pg);
      int gc = 0;
      for (int t = 0; t < n; ++t) gc += plan_cost(Lq, Lk, t, pg, a.causal);
      lq_s[b] = Lq;
      lk_s[b] = Lk;
      // JFA_SCHED_LPT = 0 (scheduling study only): groups in sequence order, not longest first
      const unsigned rank_cost = JFA_SCHED_LPT ? 0x7FFFFFFFu - (unsigned)gc : 0u;
      k = ((unsigned long long)rank_cost << 32) | (unsigned)b;
    }
    key[b] = k;
  }
  if (tid < kMaxQueues) {
    qtotal[tid] = 0;
    qcarry[tid] = 0;
  }
  if (p.gfirst)
    for (int x = tid; x < B * H; x += kPlanThreads) p.gfirst[x] = -1;
  __syncthreads();

  // 2. sort the keys (ascending: cost descending, then b); only the first B
  //    positions are read afterwards.
  if (P <= kPlanThreads) {
    // Up to one key per thread: each key's rank is the count of smaller keys
    // (the B real keys are distinct: b is part of the key; the padding keys
    // are the largest), read by every thread from LDS in the same order.
    const unsigned long long mine = tid < P ? key[tid] : 0ull;
    int rank = 0;
    if (tid < P)
#pragma unroll 8
      for (int i = 0; i < P; ++i) rank += key[i] < mine;
    __syncthreads();
    if (tid < P) key[rank] = mine;
    __syncthreads();
  } else for (int k = 2; k <= P; k <<= 1) {
    // Bitonic sort: compare-exchange steps of stride 64 and more go through
    // LDS, one barrier each; the steps of smaller stride pair lanes of one
    // wave and run in registers with cross-lane shuffles (1024 is a multiple
    // of 64, so element i sits in lane i mod 64 of its wave).
    int j = k >> 1;
    for (; j >= 64; j >>= 1) {
      for (int i = tid; i < P; i += kPlanThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = key[i], y = key[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            key[i] = y;
            key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
    for (int base = 0; base < P; base += kPlanThreads) {  // uniform bound: whole waves take part in the shuffles
      const int i = base + tid;
      unsigned long long x = i < P ? key[i] : ~0ull;
      const bool up = (i & k) == 0;
      for (int jj = j; jj > 0; jj >>= 1) {
        const unsigned lo = __shfl_xor((unsigned)x, jj), hi = __shfl_xor((unsigned)(x >> 32), jj);
        const unsigned long long y = ((unsigned long long)hi << 32) | lo;
        const bool keep_min = ((i & jj) == 0) == up;  // lower element of an ascending pair keeps the min
        x = keep_min ? (x < y ? x : y) : (x < y ? y : x);
      }
      if (i < P) key[i] = x;
    }
    __syncthreads();
  }

  // 3. queue sizes (group g = rank * H + h goes to queue snake(g))
  const int G = B * H;
  for (int g = tid; g < G; g += kPlanThreads) {
    const int b = (int)(key[g / H] & 0xFFFFFFFFu);
    atomicAdd(&qtotal[snake(g, NQ)], plan_tiles(lq_s[b], lk_s[b], pg));
  }
  __syncthreads();
  if (tid == 0) {
    long total = 0;
    for (int q = 0; q < NQ; ++q) {
      qstart[q] = (int)total;
      total += qtotal[q];
    }
    const bool fits = total <= p.capacity;
    p.hdr->count = fits ? (int)total : 0;
    p.hdr->status = fits ? 0 : 1;
    p.hdr->nq = NQ;
    for (int q = 0; q < kMaxQueues; ++q) {
      p.hdr->start[q] = (fits && q < NQ) ? qstart[q] : 0;
      p.hdr->qcount[q] = (fits && q < NQ) ? qtotal[q] : 0;
      p.hdr->ticket[q].value = 0;
    }
    wsum[0] = fits ? 0 : 1;
  }
  __syncthreads();
  if (wsum[0]) return;  // the list does not fit: nothing is written (uniform branch)
  __syncthreads();

  // 4. positions inside each queue, chunk by chunk. Thread tid of a chunk
  //    handles the i-th group of queue x in that chunk, so that each queue's
  //    groups are contiguous in one block scan. With many groups each thread
  //    writes its group's items; with few (a few long sequences) every thread
  //    writes items of the chunk, so that most threads are not left idle.
  const int per_q = kPlanThreads / NQ;  // groups of one queue in a chunk of kPlanThreads groups
  const int x = tid / per_q, i = tid % per_q;
  for (int c0 = 0; c0 < G; c0 += kPlanThreads) {
    const int g = c0 + 2 * NQ * (i >> 1) + ((i & 1) ? 2 * NQ - 1 - x : x);
    int b = 0, n = 0;
    if (g < G) {
      b = (int)(key[g / H] & 0xFFFFFFFFu);
      n = plan_tiles(lq_s[b], lk_s[b], pg);
    }
    int tot;
    const int ex = block_exclusive_scan(n, &tot, wsum);
    excl[tid] = ex;
    __syncthreads();
    const int pos = ex - excl[x * per_q];
    const long gbase = (long)qstart[x] + qcarry[x] + pos;  // first item of this group in the list
    if (p.gfirst && n > 0) p.gfirst[b * H + g % H] = (int)gbase;  // chunk 0 is first (costs non-increasing)
    __syncthreads();
    if (i == per_q - 1) qcarry[x] += pos + n;  // last group of queue x in this chunk
    if (G - c0 >= kPlanThreads / 4) {
      // Many groups: each thread writes its own group's items.
      if (n > 0) {
        const int h = g % H, Lq = lq_s[b], Lk = lk_s[b];
        for (int t = 0; t < n; ++t) {
          const long at = gbase + plan_pos(Lq, Lk, t, n, pg, a.causal);
          if (at >= 0 && at < p.capacity) p.items[at] = make_int4(b, h, t, plan_cost(Lq, Lk, t, pg, a.causal));
        }
      }
      __syncthreads();  // qcarry of the next chunk
      continue;
    }
    // Few groups (a few long sequences): all threads take the chunk's items in
    // turn. Item y belongs to the thread u whose range [wend[u] - n_u, wend[u])
    // holds it (a binary search over the inclusive scan), and is tile
    // y - (wend[u] - n_u) of u's group.
    wbase[tid] = (int)gbase;
    wbh[tid] = g < G ? (b << 16) | (g % H) : 0;  // b < 2^13 and h < 2^16 (checked on the host)
    wend[tid] = ex + n;
    __syncthreads();
    for (int y = tid; y < tot; y += kPlanThreads) {
      int lo = 0, hi = kPlanThreads - 1;  // first u with wend[u] > y
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (wend[mid] > y) hi = mid;
        else lo = mid + 1;
      }
      const int ub = wbh[lo] >> 16, uh = wbh[lo] & 0xFFFF;
      const int Lq = lq_s[ub], Lk = lk_s[ub];
      const int un = plan_tiles(Lq, Lk, pg);
      const int t = y - (wend[lo] - un);
      const long at = (long)wbase[lo] + plan_pos(Lq, Lk, t, un, pg, a.causal);
      if (at >= 0 && at < p.capacity) p.items[at] = make_int4(ub, uh, t, plan_cost(Lq, Lk, t, pg, a.causal));
    }
    __syncthreads();  // qcarry and the chunk arrays of the next chunk
  }
}

__global__ __launch_bounds__(kPlanThreads) void jfa_plan_kernel(PlanArgs a) {
  extern __shared__ __attribute__((aligned(16))) char plan_dyn[];
  plan_pass(a, blockIdx.x, plan_dyn);
}

// The backward's work lists and its row constants in one launch: workgroups
// 0 .. npass-1 build the lists, the others stream O and dO into Delta, so
// that the list building hides under the streaming.
template <typename T, int D>
__global__ __launch_bounds__(kPlanThreads) void jfa_bwd_prep_kernel(PlanArgs p, BwdArgs a, int npass) {
  extern __shared__ __attribute__((aligned(16))) char plan_dyn[];
  if ((int)blockIdx.x < npass) plan_pass(p, blockIdx.x, plan_dyn);
  else delta_rows<T, D, kPlanThreads>(a, (long)blockIdx.x - npass, threadIdx.x);
}

// lengths [B] -> offsets [B+1] (exclusive prefix sums), one workgroup.
__global__ __launch_bounds__(kPlanThreads) void jfa_scan_kernel(const int* lengths, int B, int* offsets) {
  __shared__ int wsum[2 * kPlanWaves];
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += kPlanThreads) {
    const int b = c0 + threadIdx.x;
    const int n = b < B ? lengths[b] : 0;
    int tot;
    const int ex = block_exclusive_scan(n, &tot, wsum);
    if (b < B) offsets[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) offsets[B] = carry;
}

// Offsets of B fixed-length slots (the padded-dense baseline's layout):
// qo[b] = b * Lq, ko[b] = b * Lk for b = 0 .. B. B * L < 2^31 is checked on the host.
__global__ __launch_bounds__(kPlanThreads) void jfa_slot_offsets_kernel(int B, int Lq, int Lk, int* qo, int* ko) {
  const int b = blockIdx.x * kPlanThreads + threadIdx.x;
  if (b <= B) {
    qo[b] = b * Lq;
    ko[b] = b * Lk;
  }
}

static bool plan_tiles_ok(const PlanArgs& a, int npass) {
  for (int i = 0; i < npass; ++i) {
    const PlanPass& p = a.pass[i];
    if (p.TM <= 0 || p.TN <= 0 || (p.TM & (p.TM - 1)) || (p.TN & (p.TN - 1))) return false;
  }
  return a.B >= 0 && a.B <= kPlanMaxB;
}

// Dynamic LDS above 64 KB: the kernel's limit is raised once, to the largest
// size a list can need.
template <typename K>
static hipError_t allow_plan_lds(K kern) {
  static const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  (int)plan_dyn_bytes(kPlanMaxB));
  return e;
}

hipError_t launch_plan(const PlanArgs& a, int npass, hipStream_t st) {
  if (!plan_tiles_ok(a, npass)) return hipErrorInvalidValue;
  hipError_t e = plan_dyn_bytes(a.B) > 65536 ? allow_plan_lds(jfa_plan_kernel) : hipSuccess;
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(jfa_plan_kernel, dim3(npass), dim3(kPlanThreads), plan_dyn_bytes(a.B), st, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_bwd_prep_t(const PlanArgs& p, int npass, const BwdArgs& a, hipStream_t st) {
  hipError_t e = plan_dyn_bytes(p.B) > 65536 ? allow_plan_lds(jfa_bwd_prep_kernel<T, D>) : hipSuccess;
  if (e != hipSuccess) return e;
  const long rows = a.tq * a.H;
  const long nblk = (rows + DeltaShape<T, D, kPlanThreads>::RPB - 1) / DeltaShape<T, D, kPlanThreads>::RPB;
  hipLaunchKernelGGL((jfa_bwd_prep_kernel<T, D>), dim3((unsigned)(npass + nblk)), dim3(kPlanThreads),
                     plan_dyn_bytes(p.B), st, p, a, npass);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const PlanArgs& p, int npass, bool f32, int D, const BwdArgs& a, hipStream_t st) {
  if (!plan_tiles_ok(p, npass)) return hipErrorInvalidValue;
  if (f32) {
    if (D == 32) return launch_bwd_prep_t<float, 32>(p, npass, a, st);
    if (D == 64) return launch_bwd_prep_t<float, 64>(p, npass, a, st);
    return hipErrorInvalidValue;  // fp32 with D = 128 is rejected on the host
  }
  if (D == 32) return launch_bwd_prep_t<bf16, 32>(p, npass, a, st);
  if (D == 64) return launch_bwd_prep_t<bf16, 64>(p, npass, a, st);
  return launch_bwd_prep_t<bf16, 128>(p, npass, a, st);
}

hipError_t launch_scan(const int* lengths, int B, int* offsets, hipStream_t st) {
  hipLaunchKernelGGL(jfa_scan_kernel, dim3(1), dim3(kPlanThreads), 0, st, lengths, B, offsets);
  return hipGetLastError();
}

hipError_t launch_slot_offsets(int B, int Lq, int Lk, int* qo, int* ko, hipStream_t st) {
  const int nblk = (B + 1 + kPlanThreads - 1) / kPlanThreads;
  hipLaunchKernelGGL(jfa_slot_offsets_kernel, dim3(nblk), dim3(kPlanThreads), 0, st, B, Lq, Lk, qo, ko);
  return hipGetLastError();
}

}  // namespace jfa
