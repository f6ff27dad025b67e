// Offsets-driven, longest-first work list for the persistent kernels, and the
// lengths -> offsets scan.
//
// Short sequences must not leave compute units idle ("Jagged Flash Attention
// (JFA)", section "Why standard FlashAttention falls short"), and the kernels
// are persistent ("Four generations", item 3). The list is built on the GPU
// from the offsets so that no host round trip is needed:
//
//   tiles  : q pass  -> (b, t) with t < ceil(Lq_b / TM)
//            kv pass -> (b, t) with t < ceil(Lk_b / TN)
//   cost   : key blocks (q pass) or query blocks (kv pass) the tile visits
//   order  : cost descending (costs >= kCostCap-1 share one key), then b, h, t
//   items  : (b, h, t, cost), H per tile
//
// Construction is a stable counting sort done by one 1024-thread workgroup:
// a histogram of tile keys, a descending scan of it, then tiles are ranked
// inside their key chunk by chunk (per-wave ballots give the rank among equal
// keys; per-wave counts in LDS give the offset of earlier waves). The item
// position of (b, h, t) follows from the tile's rank because, inside one
// sequence, the tiles with a given key form one contiguous run of t.
// Everything is integer arithmetic in a fixed order, so the list is the same
// on every run and equal to a plain sort with the same key.
#include "jfa_common.h"
#include "jfa_kernels.h"

namespace jfa {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kCostCap = 1024;
constexpr int kPlanMaxB = 8192;



__device__ __forceinline__ int plan_tiles(int Lq, int Lk, const PlanPass& p) {
  return p.kv_pass ? cdiv(Lk, p.TN) : cdiv(Lq, p.TM);
}

__device__ __forceinline__ int plan_cost(int Lq, int Lk, int t, const PlanPass& p, int causal) {
  if (!p.kv_pass) {
    if (!causal) return cdiv(Lk, p.TN);
    return cdiv(min(min((t + 1) * p.TM, Lq), Lk), p.TN);
  }
  const int nq = cdiv(Lq, p.TM);
  if (!causal) return nq;
  const int first_key = t * p.TN;
  if (first_key >= Lq) return 0;
  return nq - first_key / p.TM;
}

__device__ __forceinline__ int plan_key(int cost) { return min(cost, kCostCap - 1); }

// Exclusive scan over the workgroup; returns the prefix, *total gets the sum.
__device__ int block_exclusive_scan(int v, int* total, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (threadIdx.x < 64) {
    int s = threadIdx.x < kPlanWaves ? wsum[threadIdx.x] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(s, d);
      if (lane >= d) s += y;
    }
    if (threadIdx.x < kPlanWaves) wsum[kPlanWaves + threadIdx.x] = s;  // inclusive wave prefix
  }
  __syncthreads();
  const int before = w > 0 ? wsum[kPlanWaves + w - 1] : 0;
  *total = wsum[2 * kPlanWaves - 1];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kPlanThreads) void jfa_plan_kernel(PlanArgs a) {
  __shared__ int tile_base[kPlanMaxB + 1];
  __shared__ int hist[kCostCap];
  __shared__ int start[kCostCap];
  __shared__ int running[kCostCap];
  __shared__ unsigned char wcnt[kPlanWaves][kCostCap];
  __shared__ int wsum[2 * kPlanWaves];

  const PlanPass p = a.pass[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int B = a.B, H = a.H;

  for (int i = tid; i < kCostCap; i += kPlanThreads) {
    hist[i] = 0;
    running[i] = 0;
  }
  for (int i = tid; i < kPlanWaves * kCostCap; i += kPlanThreads) (&wcnt[0][0])[i] = 0;

  // 1. tile counts per sequence -> tile_base (exclusive prefix)
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += kPlanThreads) {
    const int b = c0 + tid;
    int n = 0;
    if (b < B) {
      const int Lq = a.q_off[b + 1] - a.q_off[b], Lk = a.kv_off[b + 1] - a.kv_off[b];
      n = plan_tiles(Lq, Lk, p);
    }
    int tot;
    const int ex = block_exclusive_scan(n, &tot, wsum);
    if (b < B) tile_base[b] = carry + ex;
    carry += tot;
  }
  if (tid == 0) tile_base[B] = carry;
  __syncthreads();
  const int NT = tile_base[B];
  if ((long)NT * H > p.capacity) {
    if (tid == 0) {
      p.hdr->count = 0;
      p.hdr->ticket = 0;
      p.hdr->status = 1;
    }
    return;
  }

  auto locate = [&](int x, int& b, int& t) {
    int lo = 0, hi = B;  // largest b with tile_base[b] <= x
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_base[mid] <= x) lo = mid; else hi = mid;
    }
    b = lo;
    t = x - tile_base[lo];
  };

  // 2. histogram of keys
  for (int x = tid; x < NT; x += kPlanThreads) {
    int b, t;
    locate(x, b, t);
    const int Lq = a.q_off[b + 1] - a.q_off[b], Lk = a.kv_off[b + 1] - a.kv_off[b];
    atomicAdd(&hist[plan_key(plan_cost(Lq, Lk, t, p, a.causal))], 1);
  }
  __syncthreads();

  // 3. start[key] = number of tiles with a larger key
  {
    const int key = kCostCap - 1 - tid;  // kCostCap == kPlanThreads
    int tot;
    const int ex = block_exclusive_scan(hist[key], &tot, wsum);
    start[key] = ex;
  }
  __syncthreads();

  // 4. stable rank inside each key, chunk by chunk, then the items
  for (int c0 = 0; c0 < NT; c0 += kPlanThreads) {
    const int x = c0 + tid;
    const bool valid = x < NT;
    int b = 0, t = 0, Lq = 0, Lk = 0, cost = 0, key = -1;
    if (valid) {
      locate(x, b, t);
      Lq = a.q_off[b + 1] - a.q_off[b];
      Lk = a.kv_off[b + 1] - a.kv_off[b];
      cost = plan_cost(Lq, Lk, t, p, a.causal);
      key = plan_key(cost);
    }
    int lrank = 0, wc = 0;
    unsigned long long rem = __ballot(valid);
    while (rem) {
      const int leader = __ffsll((unsigned long long)rem) - 1;
      const int k0 = __shfl(key, leader);
      const unsigned long long same = __ballot(valid && key == k0);
      if (valid && key == k0) {
        lrank = __popcll(same & ((1ull << lane) - 1ull));
        wc = __popcll(same);
      }
      rem &= ~same;
    }
    if (valid && lrank == 0) wcnt[w][key] = (unsigned char)wc;
    __syncthreads();
    int pre = 0, post = 0, r = 0;
    if (valid) {
      for (int v = 0; v < kPlanWaves; ++v) {
        const int cnt = wcnt[v][key];
        if (v < w) pre += cnt;
        if (v > w) post += cnt;
      }
      r = running[key] + pre + lrank;
    }
    __syncthreads();
    if (valid && lrank == wc - 1 && post == 0) running[key] = r + 1;
    if (valid && lrank == 0) wcnt[w][key] = 0;
    __syncthreads();

    if (valid) {
      // run [t0, t1) of tiles of sequence b that share this key
      const int n = plan_tiles(Lq, Lk, p);
      int t0 = 0, t1 = n;
      if (a.causal) {
        int lo = 0, hi = t;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (plan_key(plan_cost(Lq, Lk, mid, p, a.causal)) == key) hi = mid; else lo = mid + 1;
        }
        t0 = lo;
        lo = t + 1;
        hi = n;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (plan_key(plan_cost(Lq, Lk, mid, p, a.causal)) != key) hi = mid; else lo = mid + 1;
        }
        t1 = lo;
      }
      const int j = t - t0, run = t1 - t0;
      const long base = (long)H * (start[key] + (r - j)) + j;
      const long n_items = (long)NT * H;
      for (int h = 0; h < H; ++h) {
        const long pos = base + (long)h * run;
        if (pos >= 0 && pos < n_items) p.items[pos] = make_int4(b, h, t, cost);
      }
    }
  }
  if (tid == 0) {
    p.hdr->count = NT * H;
    p.hdr->ticket = 0;
    p.hdr->status = 0;
  }
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

hipError_t launch_plan(const PlanArgs& a, int npass, hipStream_t st) {
  hipLaunchKernelGGL(jfa_plan_kernel, dim3(npass), dim3(kPlanThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_scan(const int* lengths, int B, int* offsets, hipStream_t st) {
  hipLaunchKernelGGL(jfa_scan_kernel, dim3(1), dim3(kPlanThreads), 0, st, lengths, B, offsets);
  return hipGetLastError();
}

}  // namespace jfa
