// Backward pass of jagged exact-softmax attention on gfx950, split in two
// passes with no atomics ("Jagged Flash Attention (JFA)", section "Four
// generations", item 2: dQ is computed apart from dK/dV so that no output is
// accumulated across workgroups).
//
// The gradients of O = softmax(S) V with S = Q K^T / sqrt(D) (+ bias) are
//   dV = P^T dO, dP = dO V^T, Delta_i = sum_d dO_id O_id,
//   dS = P * (dP - Delta), dQ = dS K / sqrt(D), dK = dS^T Q / sqrt(D),
// with P recomputed from the forward's log-sum-exp: P = exp(S - lse).
//
//  * Delta per (token, head), one pass over O and dO, stored as a pair with
//    lse * log2(e) so that one 8-byte load gives a row's two softmax
//    constants (jfa_delta.h; it runs in the launch that builds the work
//    lists).
//  * jfa_dkdv_kernel  : item = (b, h, 128-key tile), 8 waves in 4 pairs; each
//                       pair owns 32 keys. The score wave of a pair keeps K
//                       of its keys in VGPRs, turns each 32-row query block
//                       into P and accumulates dV = P^T dO; the gradient wave
//                       keeps V, takes P through LDS one block behind, and
//                       computes dP, dS and dK = dS^T Q. Query blocks stream
//                       through a 4-slot LDS ring, staged in registers two
//                       blocks ahead.
//  * jfa_dq_kernel    : item = (b, h, 128-row query tile); each wave owns 32
//                       queries (Q, dO fragments in VGPRs) and walks 64-key
//                       blocks staged in LDS; dQ is stored once.
//
// Rows past a sequence's end load as zeros (Q = dO = 0 for pad queries,
// K = V = 0 for pad keys), so every product they enter is zero: no jagged
// mask is needed here. The one exception is P itself, exp(bias - lse), which
// a large bias could overflow for a pad query (0 * inf in dS); pad queries
// therefore get lse = +inf in the row constants staged in LDS, which makes
// their P exactly 0. The causal mask zeroes P above the diagonal on the
// blocks that straddle it.
#include <type_traits>

#include "jfa_common.h"
#include "jfa_kernels.h"
#include "jfa_dbias.h"
#include "jfa_short.h"

// Matrix products (bf16) whose LDS operands are read this many products
// ahead of them; 0 leaves the compiler's order, which waits for each
// product's reads right before it. Measured choices: two ahead in the dQ
// kernel at D = 128 (dQ -6 to -7%) and in the one-role dK/dV kernel (-2%);
// none in the paired dK/dV kernel (+6% with two) and the dQ kernel's rows of
// up to 128 bytes (no change).
#ifndef JFA_DQ_PREFETCH
#define JFA_DQ_PREFETCH 2
#endif
#ifndef JFA_DKV_PREFETCH
#define JFA_DKV_PREFETCH 0
#endif
#ifndef JFA_DQ_NARROW_PREFETCH
#define JFA_DQ_NARROW_PREFETCH 0
#endif
#ifndef JFA_DKV1_PREFETCH
#define JFA_DKV1_PREFETCH 2
#endif

namespace jfa {

// P handed from score wave to gradient wave in bf16 (bf16 inputs) or fp32.
#ifndef JFA_P_BF16
#define JFA_P_BF16 1
#endif
template <typename T> constexpr bool kPHalf = JFA_P_BF16 && sizeof(T) == 2;

// Where dQ is formed (a study of the backward's design; the library is 0).
//   0  the split passes: dK/dV per key tile, then dQ per query tile, with S
//      and dP formed again ("Jagged Flash Attention (JFA)", "Four
//      generations", item 2: no atomic writes, each output written once)
//   1  dQ fused into the dK/dV pass, each key tile's dQ = dS K added into an
//      fp32 accumulator with atomic adds (the design item 2 replaces)
//   2  dQ fused into the dK/dV pass, each key tile's dQ stored as a partial
//      and the partials of a query row summed in key-tile order by a later
//      kernel (one owner per (sequence, head, key tile), deterministic)
// Modes 1 and 2 cover the one-role dK/dV kernel (rows of up to 128 bytes);
// wider rows keep the split passes.
#ifndef JFA_BWD_DQ
#define JFA_BWD_DQ 0
#endif
constexpr int kBwdDq = JFA_BWD_DQ;
static_assert(kBwdDq >= 0 && kBwdDq <= 2, "backward dQ design");

// Four consecutive values (columns col .. col+3) of one row of a tile of W
// columns of T.
template <typename T, int W>
__device__ __forceinline__ void tile_put4(lds_t* tile, int row, int col, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 lo = {(bf16)a, (bf16)b}, hi = {(bf16)c, (bf16)d};
    *(__attribute__((address_space(3))) i32x2*)(tile + Tile<bf16, W>::byte(row, col * 2)) =
        (i32x2){__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
  } else {
    *(__attribute__((address_space(3))) f32x4*)(tile + Tile<float, W>::byte(row, col * 4)) = (f32x4){a, b, c, d};
  }
}




// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkvTiles {
  static constexpr int PAIRS = 4;           // 32-key slices per item
  static constexpr int BNK = 32 * PAIRS;    // keys per item
  static constexpr int BMQ = 32;            // query rows per staged block
  static constexpr int NSLOT = 4;           // score waves on block j, gradient waves on j-1, loads for j+1, j+2
  static constexpr int WAVES = 2 * PAIRS;
  static constexpr int THREADS = 64 * WAVES;
  using TL = Tile<T, D>;
  static constexpr int ROWB = TL::ROWB;
  static constexpr int QTILE = BMQ * ROWB;  // Q (or dO) rows of one block
  static constexpr int QBLK = QTILE / 1024; // 1 KB load instructions per tile
  static constexpr int RCOFF = 2 * QTILE;   // lse2 of the block's rows, then -Delta
  static constexpr int SLOT = 2 * QTILE + BMQ * 8;
  static constexpr int NQC = QTILE / 16;    // 16-byte pieces per tile
  static constexpr int NCH = (2 * NQC + THREADS - 1) / THREADS;  // Q and dO pieces per thread
  static constexpr int PBUF = NSLOT * SLOT;  // [block parity][pair] fp32 P of a 32 x 32 block, lane order
  static constexpr int PBLK = 64 * 64;       // 64 lanes x 16 floats
  static constexpr int PBUF_BYTES = 2 * PAIRS * PBLK;
  static constexpr int BIAS_OFF = PBUF + PBUF_BYTES;
  static constexpr int LDS = BIAS_OFF + 1040;
  static_assert(BMQ <= THREADS, "row constants: one row per thread");
  static_assert(BMQ == kDkvTM && BNK == kDkvTN, "tile shape published to the planner");
};

// State of one dK/dV work item, identical in every wave of the workgroup.
struct DkvItem {
  int pos, b, h, Lq, Lk, kw_base, qb0, nblk;  // pos: list position of the item
  const char* qbase;
  const char* dobase;
  const float2* rcbase;
  size_t krow;
};

template <typename T, int D>
__device__ __forceinline__ bool dkv_begin(const BwdArgs& a, QueueCursor* qc, TicketState& tk, DkvItem& it) {
  using C = DkvTiles<T, D>;
  const int i = next_item(a.hdr, qc, tk);
  if (i < 0) return false;
  const int4 item = a.items[i];
  it.pos = i;
  it.b = uni(item.x);
  it.h = uni(item.y);
  const int q0 = uni(a.q_off[it.b]), k0 = uni(a.kv_off[it.b]);
  it.Lq = uni(a.q_off[it.b + 1]) - q0;
  it.Lk = uni(a.kv_off[it.b + 1]) - k0;
  it.kw_base = uni(item.z) * C::BNK;
  const int nq = cdiv(it.Lq, C::BMQ);
  it.qb0 = a.causal ? (it.kw_base >= it.Lq ? nq : it.kw_base / C::BMQ) : 0;
  it.nblk = nq - it.qb0;
  const size_t qrow = ((size_t)q0 * a.H + it.h) * C::ROWB;
  it.qbase = uni((const char*)a.q + qrow);
  it.dobase = uni((const char*)a.dout + qrow);
  it.rcbase = uni(a.rowc + (size_t)q0 * a.H + it.h);
  it.krow = ((size_t)k0 * a.H + it.h) * C::ROWB;
  return true;
}

// Query block jb (rows (qb0 + jb) * BMQ ...) staged through registers: the
// global loads are issued before a step's compute and written to ring slot
// jb % NSLOT after it, so their latency hides behind the compute.
template <typename T, int D>
struct DkvStage {
  i32x4 c[DkvTiles<T, D>::NCH];
  i32x2 rc;
  bool row_ok;  // this thread's row constant belongs to a query of the sequence
};

template <typename T, int D>
__device__ __forceinline__ void dkv_gload(const DkvItem& it, int jb, uint32_t gstride, int H, int tid, DkvStage<T, D>& st) {
  using C = DkvTiles<T, D>;
  const int r0 = (it.qb0 + jb) * C::BMQ;
  const int rows = min(C::BMQ, it.Lq - r0);
  const View qv = seq_view(it.qbase + (size_t)r0 * gstride, rows, gstride, C::ROWB);
  const View dv = seq_view(it.dobase + (size_t)r0 * gstride, rows, gstride, C::ROWB);
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    const int x = tid + C::THREADS * c;
    if (x < 2 * C::NQC) {
      const int y = x % C::NQC, row = y / C::TL::CPR, col = y % C::TL::CPR;
      st.c[c] = ld16(x < C::NQC ? qv : dv, (uint32_t)row * gstride + col * 16);
    }
  }
  if (tid < C::BMQ) st.rc = ld8(seq_view(it.rcbase + (size_t)r0 * H, rows, 8 * H, 8), 8 * H * tid);
  st.row_ok = tid < rows;
}

template <typename T, int D>
__device__ __forceinline__ void dkv_swrite(int jb, int tid, const DkvStage<T, D>& st, lds_t* lds) {
  using C = DkvTiles<T, D>;
  lds_t* sl = lds + (jb % C::NSLOT) * C::SLOT;
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    const int x = tid + C::THREADS * c;
    if (x < 2 * C::NQC) {
      const int y = x % C::NQC, row = y / C::TL::CPR, col = y % C::TL::CPR;
      *(__attribute__((address_space(3))) i32x4*)(sl + (x < C::NQC ? 0 : C::QTILE) + C::TL::chunk(row, col)) = st.c[c];
    }
  }
  if (tid < C::BMQ) {  // lse2 of the block's rows, then -Delta (the start of each dP accumulation);
    // rows past the sequence end get lse2 = +inf, so P = 0 there whatever the bias
    ((__attribute__((address_space(3))) float*)(sl + C::RCOFF))[tid] = st.row_ok ? __int_as_float(st.rc[0]) : INFINITY;
    ((__attribute__((address_space(3))) float*)(sl + C::RCOFF))[C::BMQ + tid] = -__int_as_float(st.rc[1]);
  }
}

// Blocks 0 and 1 of an item, both loads in flight together.
template <typename T, int D>
__device__ __forceinline__ void dkv_prologue(const DkvItem& it, uint32_t gstride, int H, int tid, lds_t* lds) {
  DkvStage<T, D> s0, s1;
  if (it.nblk > 0) dkv_gload<T, D>(it, 0, gstride, H, tid, s0);
  if (it.nblk > 1) dkv_gload<T, D>(it, 1, gstride, H, tid, s1);
  if (it.nblk > 0) dkv_swrite<T, D>(0, tid, s0, lds);
  if (it.nblk > 1) dkv_swrite<T, D>(1, tid, s1, lds);
}

// Blocks whose queries can see some key of the slice starting at kw0.
__device__ __forceinline__ bool dkv_active(int qs0, int kw0, int Lk, int causal) {
  return kw0 < Lk && (!causal || qs0 + 31 >= kw0);
}

template <typename T, int D, bool BIAS, bool DBIAS>
__device__ __forceinline__ void dkv_score_role(const BwdArgs& a, lds_t* lds, QueueCursor* qc) {
  using C = DkvTiles<T, D>;
  constexpr int BMQ = C::BMQ, ES = (int)sizeof(T);
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: views and loops stay scalar
  const int pair = w;
  const uint32_t gstride = (uint32_t)a.H * C::ROWB;
  TicketState tk;
  DkvItem it;
  DkvStage<T, D> stg;
  while (dkv_begin<T, D>(a, qc, tk, it)) {
    if (BIAS) {  // read by the score waves only, which load it themselves
      for (int i = tid; i < kBiasLen; i += 64 * C::PAIRS) bias_lds[i] = a.bias[it.h * kBiasLen + i] * kLog2e;
    }
    const int kw0 = it.kw_base + 32 * pair, kj = kw0 + l32;
    const View kv = seq_view((const char*)a.k + it.krow + (size_t)kw0 * gstride, max(0, min(32, it.Lk - kw0)), gstride, C::ROWB);
    Frag<T> kf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kf[kk] = gfrag(kv, (uint32_t)l32 * gstride + (16 * kk + 8 * g) * ES, (T*)0);
    f32x16 dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dv[db] = (f32x16){};
    dkv_prologue<T, D>(it, gstride, a.H, tid, lds);
    wait_vmem();  // K fragments in: no wait for them inside the loop
    __syncthreads();

    for (int jb = 0; jb <= it.nblk; ++jb) {
      if (jb + 2 < it.nblk) dkv_gload<T, D>(it, jb + 2, gstride, a.H, tid, stg);
      const int qs0 = (it.qb0 + jb) * BMQ;
      if (jb < it.nblk && dkv_active(qs0, kw0, it.Lk, a.causal)) {
        const bool masked = a.causal && qs0 < kw0 + 31;
        const lds_t* qt = lds + (jb % C::NSLOT) * C::SLOT;
        const __attribute__((address_space(3))) float* rc = (const __attribute__((address_space(3))) float*)(qt + C::RCOFF);
        // S = Q K^T (lane = key kj, element i = query qs0 + res_row(i, g))
        f32x16 sc = (f32x16){};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) mma(sc, lfrag<D>(qt, l32, 16 * kk + 8 * g, (T*)0), kf[kk]);
        if constexpr (JFA_DKV_PREFETCH > 0 && sizeof(T) == 2) sched_prefetch<D / 16, 1, JFA_DKV_PREFETCH>();
        // P = exp2(S * scale * log2(e) - lse2 (+ bias)), zero above the diagonal
        // (the element test only on blocks that straddle it)
        auto softmax = [&](auto mask_c) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = res_row(i, g);
            const int qi = qs0 + r;
            float x = sc[i] * a.scale2 - rc[r];
            if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
            float p = __builtin_amdgcn_exp2f(x);
            if (decltype(mask_c)::value && kj > qi) p = 0.f;
            sc[i] = p;
          }
        };
        if (masked) softmax(std::true_type{});
        else softmax(std::false_type{});
        // handed to the gradient wave of the pair, lane order: for bf16 inputs
        // the bf16 fragments the dV product takes anyway (half the LDS bytes),
        // for fp32 inputs fp32
        lds_t* pb = lds + C::PBUF + ((jb & 1) * C::PAIRS + pair) * C::PBLK;
        if constexpr (!kPHalf<T>) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *(__attribute__((address_space(3))) f32x4*)(pb + 1024 * e + 16 * lane) =
                (f32x4){sc[4 * e], sc[4 * e + 1], sc[4 * e + 2], sc[4 * e + 3]};
        }
        // dV^T += dO^T P^T
        const lds_t* dot = qt + C::QTILE;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const Frag<T> pf = rfrag(sc, c, (T*)0);
          if constexpr (kPHalf<T>) put_frag(pb + 1024 * c, pf, lane);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) mma(dv[db], tfrag<D>(dot, 16 * c, 32 * db, lane, (T*)0), pf);
        }
        if constexpr (JFA_DKV_PREFETCH > 0 && sizeof(T) == 2) sched_prefetch<2 * (D / 32), 2, JFA_DKV_PREFETCH>();
      }
      if (jb + 2 < it.nblk) dkv_swrite<T, D>(jb + 2, tid, stg, lds);
      __syncthreads();
    }

    // dV^T: lane holds rows d = 32db + res_row(i,g) of key kj.
    if (kw0 < it.Lk) {
      const View dvv = seq_view((char*)a.dv + it.krow + (size_t)kw0 * gstride, min(32, it.Lk - kw0), gstride, C::ROWB);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          store4(dvv, (uint32_t)l32 * gstride + d * ES, dv[db][4 * r], dv[db][4 * r + 1], dv[db][4 * r + 2],
                 dv[db][4 * r + 3], (T*)0);
        }
      }
    }
    if (DBIAS) __syncthreads();  // the gradient waves' bias bins are complete
  }
}

template <typename T, int D, bool DBIAS>
__device__ __forceinline__ void dkv_grad_role(const BwdArgs& a, lds_t* lds, QueueCursor* qc) {
  using C = DkvTiles<T, D>;
  constexpr int BMQ = C::BMQ, ES = (int)sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w - C::PAIRS;
  const uint32_t gstride = (uint32_t)a.H * C::ROWB;
  TicketState tk;
  DkvItem it;
  DkvStage<T, D> stg;
  while (dkv_begin<T, D>(a, qc, tk, it)) {
    const int kw0 = it.kw_base + 32 * pair;
    DbWave db;
    if (DBIAS) {
      db = db_wave(lds + C::LDS, pair);
      db_begin(db, lane);
    }
    const View vv = seq_view((const char*)a.v + it.krow + (size_t)kw0 * gstride, max(0, min(32, it.Lk - kw0)), gstride, C::ROWB);
    Frag<T> vf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) vf[kk] = gfrag(vv, (uint32_t)l32 * gstride + (16 * kk + 8 * g) * ES, (T*)0);
    f32x16 dk[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dk[db] = (f32x16){};
    dkv_prologue<T, D>(it, gstride, a.H, tid, lds);
    wait_vmem();  // V fragments in
    __syncthreads();

    for (int jb = 0; jb <= it.nblk; ++jb) {
      if (jb + 2 < it.nblk) dkv_gload<T, D>(it, jb + 2, gstride, a.H, tid, stg);
      const int jp = jb - 1;  // block whose P the score wave handed over in the previous step
      if (jp >= 0 && dkv_active((it.qb0 + jp) * BMQ, kw0, it.Lk, a.causal)) {
        const lds_t* qt = lds + (jp % C::NSLOT) * C::SLOT;
        const lds_t* dot = qt + C::QTILE;
        const __attribute__((address_space(3))) float* rc = (const __attribute__((address_space(3))) float*)(qt + C::RCOFF);
        // dP - Delta = dO V^T - Delta (same layout as S: lane = key, element i =
        // query res_row(i, g)); the accumulation starts at -Delta of the rows
        // (rows 8k + 4g .. 8k + 4g + 3 are elements 4k .. 4k + 3)
        f32x16 dp;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const f32x4 nd = *(const __attribute__((address_space(3))) f32x4*)(rc + BMQ + 8 * k4 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * k4 + e] = nd[e];
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) mma(dp, lfrag<D>(dot, l32, 16 * kk + 8 * g, (T*)0), vf[kk]);
        if constexpr (JFA_DKV_PREFETCH > 0 && sizeof(T) == 2) sched_prefetch<D / 16, 1, JFA_DKV_PREFETCH>();
        const lds_t* pb = lds + C::PBUF + ((jp & 1) * C::PAIRS + pair) * C::PBLK;
        f32x16 p;
        if constexpr (kPHalf<T>) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const bf16x8 x = __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) i32x4*)(pb + 1024 * c + 16 * lane));
#pragma unroll
            for (int e = 0; e < 8; ++e) p[8 * c + e] = (float)x[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x4 x = *(const __attribute__((address_space(3))) f32x4*)(pb + 1024 * e + 16 * lane);
            p[4 * e] = x[0];
            p[4 * e + 1] = x[1];
            p[4 * e + 2] = x[2];
            p[4 * e + 3] = x[3];
          }
        }
        // dS = P (dP - Delta)
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] = p[i] * dp[i];
        if (DBIAS) {  // keys past the end: K = V = 0 leaves dS = -P Delta there, which is no pair's gradient
          f32x16 ds = dp;
          if (kw0 + l32 >= it.Lk) ds = (f32x16){};
          db_block(db, ds, (it.qb0 + jp) * BMQ - kw0, lane);
        }
        // dK^T += Q^T dS^T
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const Frag<T> sf = rfrag(dp, c, (T*)0);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) mma(dk[db], tfrag<D>(qt, 16 * c, 32 * db, lane, (T*)0), sf);
        }
        if constexpr (JFA_DKV_PREFETCH > 0 && sizeof(T) == 2) sched_prefetch<2 * (D / 32), 2, JFA_DKV_PREFETCH>();
      }
      if (jb + 2 < it.nblk) dkv_swrite<T, D>(jb + 2, tid, stg, lds);
      __syncthreads();
    }

    // dK^T: lane holds rows d = 32db + res_row(i,g) of key kw0 + l32.
    if (kw0 < it.Lk) {
      const View dkv = seq_view((char*)a.dk + it.krow + (size_t)kw0 * gstride, min(32, it.Lk - kw0), gstride, C::ROWB);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          store4(dkv, (uint32_t)l32 * gstride + d * ES, dk[db][4 * r] * a.scale, dk[db][4 * r + 1] * a.scale,
                 dk[db][4 * r + 2] * a.scale, dk[db][4 * r + 3] * a.scale, (T*)0);
        }
      }
    }
    if (DBIAS) {  // the item's bias-gradient bins, gradient waves in order
      db_finish(db, lane);
      __syncthreads();
      db_store(lds + C::LDS, C::PAIRS, a.dbp_kv + (size_t)it.pos * kBiasLen, tid - 64 * C::PAIRS, 64 * C::PAIRS);
    }
  }
}

// The two roles run the same item sequence and meet at the same barriers
// (two per item fetch, one after the prologue, one per block step).
template <typename T, int D, bool BIAS, bool DBIAS>
__device__ __forceinline__ void dkv_two_roles(const BwdArgs& a) {
  using C = DkvTiles<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS + (DBIAS ? C::PAIRS * kDbWaveBytes : 0)];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  load_queues(a.hdr, &qcur);
  if ((threadIdx.x >> 6) < C::PAIRS) dkv_score_role<T, D, BIAS, DBIAS>(a, lds, &qcur);
  else dkv_grad_role<T, D, DBIAS>(a, lds, &qcur);
}

// ---------------------------------------------------------------------------
// dK/dV pass for D <= 64, one role per wave: 4 waves x 32 keys, each wave
// keeping its K, V fragments and dK, dV accumulators in VGPRs and walking
// 64-row query blocks staged in LDS (register prefetch, two LDS stages).
// Small enough per wave for two workgroups per CU.
template <typename T, int D>
struct Dkv1Tiles {
  static constexpr int BNK = 128;  // keys per item (4 waves x 32)
  static constexpr int BMQ = 64;   // query rows per staged block
  static constexpr int THREADS = 256;
  using TL = Tile<T, D>;
  static constexpr int ROWB = TL::ROWB;
  static constexpr int QTILE = BMQ * ROWB;
  static constexpr int STAGE = 2 * QTILE + 2 * BMQ * 4;  // Q, dO, lse2 and -Delta per row
  static constexpr int CPR = ROWB / 16;
  static constexpr int CPT = BMQ * CPR / THREADS;
  static constexpr int BIAS_OFF = 2 * STAGE;
  // fused dQ (study modes 1, 2): the block's dS as [key][query] and the
  // item's K tile [key][D]
  static constexpr bool FUSED = kBwdDq != 0;
  static constexpr int DST_OFF = BIAS_OFF + 1040;
  static constexpr int DST_BYTES = FUSED ? BNK * BMQ * (int)sizeof(T) : 0;
  static constexpr int KT_OFF = DST_OFF + DST_BYTES;
  static constexpr int KT_BYTES = FUSED ? BNK * ROWB : 0;
  static constexpr int LDS = KT_OFF + KT_BYTES;
  static constexpr int KCPT = BNK * CPR / THREADS;  // K tile pieces per thread
  static_assert((BMQ * CPR) % THREADS == 0, "tile pieces divide the workgroup");
  static_assert(BMQ == kDkv1TM && BNK == kDkvTN, "tile shape published to the planner");
};

template <typename T, int D, bool BIAS, bool DBIAS>
__device__ __forceinline__ void dkv_one_role(const BwdArgs& a) {
  using C = Dkv1Tiles<T, D>;
  constexpr int BNK = C::BNK, BMQ = C::BMQ, ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS + (DBIAS ? 4 * kDbWaveBytes : 0)];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave branches stay scalar
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * C::ROWB;
  load_queues(a.hdr, &qcur);
  TicketState tk;

  for (;;) {
    const int it = next_item(a.hdr, &qcur, tk);
    if (it < 0) break;
    const int4 item = a.items[it];
    const int b = item.x, h = item.y, kt = item.z;
    const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
    const int k0 = a.kv_off[b], Lk = a.kv_off[b + 1] - k0;
    const int key_tile0 = kt * BNK;
    const int nq = cdiv(Lq, BMQ);
    int qb0 = 0;
    if (a.causal) qb0 = key_tile0 >= Lq ? nq : key_tile0 / BMQ;

    const size_t qrow = ((size_t)q0 * H + h) * C::ROWB, krow = ((size_t)k0 * H + h) * C::ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, C::ROWB);
    const View dov = seq_view((const char*)a.dout + qrow, Lq, gstride, C::ROWB);
    const View kv = seq_view((const char*)a.k + krow, Lk, gstride, C::ROWB);
    const View vv = seq_view((const char*)a.v + krow, Lk, gstride, C::ROWB);
    const View rcv = seq_view(a.rowc + (size_t)q0 * H + h, Lq, 8 * H, 8);

    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += C::THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }

    const int kw0 = key_tile0 + 32 * w;  // first key of this wave
    const bool wave_on = kw0 < Lk;
    const int kj = kw0 + l32;            // this lane's key
    DbWave db;
    if (DBIAS) {
      db = db_wave(lds + C::LDS, w);
      db_begin(db, lane);
    }
    Frag<T> kf[D / 16], vf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = gfrag(kv, (uint32_t)kj * gstride + (16 * kk + 8 * g) * ES, (T*)0);
      vf[kk] = gfrag(vv, (uint32_t)kj * gstride + (16 * kk + 8 * g) * ES, (T*)0);
    }
    lds_t* dst_t = lds + C::DST_OFF;  // fused dQ: dS^T of the block, [key][query]
    lds_t* k_t = lds + C::KT_OFF;     // fused dQ: the item's keys, [key][D]
    if constexpr (C::FUSED) {
      // the item's 128 keys (rows past the end load as zeros); the barrier
      // after the first Q/dO block orders these writes before any read
#pragma unroll
      for (int c = 0; c < C::KCPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        *(__attribute__((address_space(3))) i32x4*)(k_t + C::TL::chunk(row, col)) =
            ld16(kv, (uint32_t)(key_tile0 + row) * gstride + col * 16);
      }
    }

    i32x4 qr[C::CPT], dr[C::CPT];
    i32x2 lr = {};
    bool lr_ok = false;  // the row constant belongs to a query of the sequence
    auto gload = [&](int qb) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        const uint32_t off = (uint32_t)(qb * BMQ + row) * gstride + col * 16;
        qr[c] = ld16(qv, off);
        dr[c] = ld16(dov, off);
      }
      if (tid < BMQ) lr = ld8(rcv, (uint32_t)(qb * BMQ + tid) * 8 * H);
      lr_ok = qb * BMQ + tid < Lq;
    };
    auto swrite = [&](int s) {
      lds_t* st = lds + s * C::STAGE;
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        const int o = C::TL::chunk(row, col);
        *(__attribute__((address_space(3))) i32x4*)(st + o) = qr[c];
        *(__attribute__((address_space(3))) i32x4*)(st + C::QTILE + o) = dr[c];
      }
      if (tid < BMQ) {  // lse2 of the block's rows, then -Delta (the start of each dP accumulation);
        // rows past the sequence end get lse2 = +inf, so P = 0 there whatever the bias
        ((__attribute__((address_space(3))) float*)(st + 2 * C::QTILE))[tid] = lr_ok ? __int_as_float(lr[0]) : INFINITY;
        ((__attribute__((address_space(3))) float*)(st + 2 * C::QTILE))[BMQ + tid] = -__int_as_float(lr[1]);
      }
    };
    if (qb0 < nq) {
      gload(qb0);
      swrite(0);
    }
    wait_vmem();
    __syncthreads();

    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      dk[db] = (f32x16){};
      dv[db] = (f32x16){};
    }

    for (int qb = qb0; qb < nq; ++qb) {
      const int s = (qb - qb0) & 1;
      if (qb + 1 < nq) gload(qb + 1);
      const lds_t* qt = lds + s * C::STAGE;
      const lds_t* dot = qt + C::QTILE;
      const __attribute__((address_space(3))) float* rc = (const __attribute__((address_space(3))) float*)(qt + 2 * C::QTILE);
#pragma unroll
      for (int sb = 0; sb < BMQ / 32; ++sb) {
        const int qs0 = qb * BMQ + 32 * sb;  // first query of this 32-row sub-block
        const bool active = wave_on && qs0 < Lq && (!a.causal || qs0 + 31 >= kw0);
        if (!active) {
          if constexpr (C::FUSED) {  // no pair of this quarter is visible: its dS is 0
#pragma unroll
            for (int r = 0; r < 4; ++r) tile_put4<T, BMQ>(dst_t, 32 * w + l32, 32 * sb + 8 * r + 4 * g, 0.f, 0.f, 0.f, 0.f);
          }
          continue;
        }
        const bool masked = a.causal && qs0 < kw0 + 31;
        // dP starts at -Delta of its rows (rows 8k + 4g .. 8k + 4g + 3 of the
        // sub-block are elements 4k .. 4k + 3), so dP - Delta comes out of
        // the matrix cores
        f32x16 sc = (f32x16){}, dp;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const f32x4 nd = *(const __attribute__((address_space(3))) f32x4*)(rc + BMQ + 32 * sb + 8 * k4 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * k4 + e] = nd[e];
        }
        prio_mfma();
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          mma(sc, lfrag<D>(qt, 32 * sb + l32, 16 * kk + 8 * g, (T*)0), kf[kk]);
          mma(dp, lfrag<D>(dot, 32 * sb + l32, 16 * kk + 8 * g, (T*)0), vf[kk]);
        }
        if constexpr (JFA_DKV1_PREFETCH > 0 && sizeof(T) == 2) sched_prefetch<2 * (D / 16), 1, JFA_DKV1_PREFETCH>();
        prio_valu();
        // sc[i] = S[query 32sb + res_row(i,g)][key kj]; the element test for
        // the causal mask only on blocks that straddle the diagonal
        auto softmax = [&](auto mask_c) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 32 * sb + res_row(i, g);
            const int qi = qb * BMQ + r;
            float x = sc[i] * a.scale2 - rc[r];
            if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
            float p = __builtin_amdgcn_exp2f(x);
            if (decltype(mask_c)::value && kj > qi) p = 0.f;
            sc[i] = p;
            dp[i] = p * dp[i];
          }
        };
        if (masked) softmax(std::true_type{});
        else softmax(std::false_type{});
        if (DBIAS) {  // keys past the end: K = V = 0 leaves dS = -P Delta there, which is no pair's gradient
          f32x16 ds = dp;
          if (kj >= Lk) ds = (f32x16){};
          db_block(db, ds, qs0 - kw0, lane);
        }
        if constexpr (C::FUSED) {
          // dS^T of this quarter for the fused dQ product (key row 32w + l32,
          // query columns 32sb + res_row(i, g)). Keys past the end are 0: their
          // K row is 0, but their dS = -P Delta has P = exp(bias - lse), which
          // overflows for a row whose lse is very negative (0 * inf in dQ).
#pragma unroll
          for (int r = 0; r < 4; ++r)
            tile_put4<T, BMQ>(dst_t, 32 * w + l32, 32 * sb + 8 * r + 4 * g, kj < Lk ? dp[4 * r] : 0.f,
                              kj < Lk ? dp[4 * r + 1] : 0.f, kj < Lk ? dp[4 * r + 2] : 0.f,
                              kj < Lk ? dp[4 * r + 3] : 0.f);
        }
        prio_mfma();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const Frag<T> pf = rfrag(sc, c, (T*)0);
          const Frag<T> sf = rfrag(dp, c, (T*)0);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            mma(dv[db], tfrag<D>(dot, 32 * sb + 16 * c, 32 * db, lane, (T*)0), pf);
            mma(dk[db], tfrag<D>(qt, 32 * sb + 16 * c, 32 * db, lane, (T*)0), sf);
          }
        }
        if constexpr (JFA_DKV1_PREFETCH > 0 && sizeof(T) == 2) sched_prefetch<4 * (D / 32), 2, JFA_DKV1_PREFETCH>();
        prio_valu();
      }
      if constexpr (C::FUSED) {
        // dQ of the block's 64 queries from this item's 128 keys:
        // dQ = dS K, one 32 x 32 tile (query half, D block) per wave
        __syncthreads();  // every wave's dS^T is in LDS
        constexpr int NT = 2 * (D / 32);  // tiles of the block
        if (w < NT) {
          const int qh = w & 1, dh = w >> 1;
          f32x16 acc = (f32x16){};
#pragma unroll
          for (int ks = 0; ks < BNK / 16; ++ks)
            mma(acc, tfrag<BMQ>(dst_t, 16 * ks, 32 * qh, lane, (T*)0), tfrag<D>(k_t, 16 * ks, 32 * dh, lane, (T*)0));
          // lane: column d = 32 dh + l32, elements i: query qb*BMQ + 32 qh + res_row(i, g)
          const int d = 32 * dh + l32;
          float* base = a.dqacc + ((size_t)q0 * H + h) * D + d;
          if constexpr (kBwdDq == 2) base += (size_t)kt * a.tq * H * D;  // this key tile's partial
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = qb * BMQ + 32 * qh + res_row(i, g);
            if (qi < Lq) {
              float* p = base + (size_t)qi * H * D;
              if constexpr (kBwdDq == 1) __hip_atomic_fetch_add(p, acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              else *p = acc[i];
            }
          }
        }
      }
      if (qb + 1 < nq) swrite((qb + 1 - qb0) & 1);
      __syncthreads();
    }

    // dK^T, dV^T: lane holds rows d = 32db + res_row(i,g) of key kj.
    if (wave_on) {
      const View dkv = seq_view((char*)a.dk + krow, Lk, gstride, C::ROWB);
      const View dvv = seq_view((char*)a.dv + krow, Lk, gstride, C::ROWB);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          const uint32_t off = (uint32_t)kj * gstride + d * ES;
          store4(dkv, off, dk[db][4 * r] * a.scale, dk[db][4 * r + 1] * a.scale, dk[db][4 * r + 2] * a.scale,
                 dk[db][4 * r + 3] * a.scale, (T*)0);
          store4(dvv, off, dv[db][4 * r], dv[db][4 * r + 1], dv[db][4 * r + 2], dv[db][4 * r + 3], (T*)0);
        }
      }
    }
    if (DBIAS) {  // the item's bias-gradient bins, waves in order
      db_finish(db, lane);
      __syncthreads();
      db_store(lds + C::LDS, 4, a.dbp_kv + (size_t)it * kBiasLen, tid, C::THREADS);
    }
  }
}

// dK/dV kernel: one role per wave for rows of up to 128 bytes, score and
// gradient wave pairs for wider rows.
// Widest rows (bytes) the one-role kernel takes; wider ones go to the paired
// kernel (a compile-time choice; the library keeps 128).
#ifndef JFA_DKV_ONE_ROLE_ROWB
#define JFA_DKV_ONE_ROLE_ROWB 128
#endif
template <typename T, int D>
struct DkvShape {
  static constexpr bool one_role = D * sizeof(T) <= JFA_DKV_ONE_ROLE_ROWB;
  static constexpr int threads = one_role ? Dkv1Tiles<T, D>::THREADS : 512;
};

// DBIAS (with BIAS): also the bias-gradient bins of each item.
template <typename T, int D, bool BIAS, bool DBIAS>
__global__ __launch_bounds__((DkvShape<T, D>::threads), 2) void jfa_dkdv_kernel(BwdArgs a) {
  if constexpr (DkvShape<T, D>::one_role) dkv_one_role<T, D, BIAS, DBIAS>(a);
  else dkv_two_roles<T, D, BIAS, DBIAS>(a);
}

// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqTiles {
  static constexpr int BM = 128;  // query rows per item (4 waves x 32)
  static constexpr int BN = 64;   // keys per staged block
  static constexpr int THREADS = 256;
  using TL = Tile<T, D>;
  static constexpr int ROWB = TL::ROWB;
  // Rows of up to 128 bytes: K and V with padded rows (pad_nat: the natural
  // reads of S^T = K Q^T and dP^T = V dO^T are conflict-free, K's transposed
  // reads for dQ partly two-way), each tile whole KBs for the direct loads,
  // and the block taken in halves of 32 keys; with the fewer registers this
  // leaves, three workgroups share a CU. Wider rows: the permuted tiles
  // (Tile::swz), conflict-free for both read patterns, two workgroups.
  static constexpr bool PAD = ROWB <= 128;
  static constexpr int KS = PAD ? pad_nat(ROWB) : ROWB;
  static constexpr int KTILE = PAD ? PaddedDma<BN, ROWB, KS>::NBLK * 1024 : BN * ROWB;
  static constexpr int STAGE = 2 * KTILE;
  static constexpr int CPR = ROWB / 16;
  static constexpr int CPT = BN * CPR / THREADS;
  static constexpr int BIAS_OFF = 2 * STAGE;
  static constexpr int LDS = BIAS_OFF + 1040;
  static_assert((BN * CPR) % THREADS == 0, "tile pieces divide the workgroup");
  static_assert(BM == kDqTM && BN == kDqTN, "tile shape published to the planner");
};

template <typename T, int D, bool BIAS>
__global__ __launch_bounds__(256, (sizeof(T) == 4 && D >= 64 ? 1 : 2)) void jfa_dq_kernel(BwdArgs a) {
  using C = DqTiles<T, D>;
  constexpr int BM = C::BM, BN = C::BN, ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave branches stay scalar
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * C::ROWB;
  // First, the short-query sequences: dQ is the sum of their chunks'
  // partials (previous launch).
  static_assert(kShortLds <= C::LDS, "combining step fits the LDS");
  for_short_groups(a.gfirst, a.B * H, lds, [&](int gi) { sq_reduce<T, D>(a, gi); });
  load_queues(a.hdr, &qcur);
  TicketState tk;

  for (;;) {
    const int it = next_item(a.hdr, &qcur, tk);
    if (it < 0) break;
    const int4 item = a.items[it];
    const int b = item.x, h = item.y, qt = item.z;
    const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
    const int k0 = a.kv_off[b], Lk = a.kv_off[b + 1] - k0;
    const int row0 = qt * BM;
    const int n_kv = a.causal ? cdiv(min(min(row0 + BM, Lq), Lk), BN) : cdiv(Lk, BN);
    // keys at or past Lm are dropped (the padded-dense baseline's true key count)
    const int Lm = a.kv_len ? min(max(a.kv_len[b], 0), Lk) : Lk;

    const size_t qrow = ((size_t)q0 * H + h) * C::ROWB, krow = ((size_t)k0 * H + h) * C::ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, C::ROWB);
    const View dov = seq_view((const char*)a.dout + qrow, Lq, gstride, C::ROWB);
    const View rcv = seq_view(a.rowc + (size_t)q0 * H + h, Lq, 8 * H, 8);

    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += C::THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }

    const int wr0 = row0 + 32 * w;
    const bool wave_on = wr0 < Lq;
    const int qi = wr0 + l32;
    Frag<T> qf[D / 16], df[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = gfrag(qv, (uint32_t)qi * gstride + (16 * kk + 8 * g) * ES, (T*)0);
      df[kk] = gfrag(dov, (uint32_t)qi * gstride + (16 * kk + 8 * g) * ES, (T*)0);
    }
    const i32x2 rcq = ld8(rcv, (uint32_t)qi * 8 * H);
    const float lse2 = __int_as_float(rcq[0]), dlt = __int_as_float(rcq[1]);

    // K/V blocks through a two-stage LDS ring filled by direct loads: block
    // j+1 is requested while block j is computed.
    const DmaView kd = dma_view((const char*)a.k + krow, Lk, gstride, C::ROWB);
    const DmaView vd = dma_view((const char*)a.v + krow, Lk, gstride, C::ROWB);
    auto issue = [&](int j) {
      lds_t* st = lds + (j & 1) * C::STAGE;
      if constexpr (C::PAD) {
        dma_padded_tile<BN, C::ROWB, C::KS, 4>(kd, gstride, j * BN, st, w, lane);
        dma_padded_tile<BN, C::ROWB, C::KS, 4>(vd, gstride, j * BN, st + C::KTILE, w, lane);
      } else {
        dma_tile<T, D, BN, 4>(kd, gstride, j * BN, st, w, lane);
        dma_tile<T, D, BN, 4>(vd, gstride, j * BN, st + C::KTILE, w, lane);
      }
    };
    if (n_kv > 0) issue(0);
    wait_vmem();  // Q, dO, lse, Delta and the first K/V block have landed
    __syncthreads();

    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dq[db] = (f32x16){};

    for (int j = 0; j < n_kv; ++j) {
      const int s = j & 1;
      if (j + 1 < n_kv) issue(j + 1);
      const int key0 = j * BN;
      const bool active = wave_on && (!a.causal || key0 <= wr0 + 31);
      if (active) {
        const bool masked = a.causal && (key0 + BN - 1 > wr0);
        // Pad keys have K = V = 0, but P there is exp(bias - lse), which can
        // overflow for a row whose lse is very negative; 0 * inf would then
        // leak into dQ through the zero K row. Drop them on the block(s) that
        // hold them.
        const bool padded = key0 + BN > Lm;
        const lds_t* kt = lds + s * C::STAGE;
        const lds_t* vt = kt + C::KTILE;
        // For D <= 64 the dP accumulation starts at -Delta (this lane's query),
        // so dP - Delta comes out of the matrix cores; at D = 128 the 16
        // registers this takes are not free.
        constexpr bool kNegDelta = D <= 64;
        if constexpr (C::PAD) {
          // The block in halves of 32 keys: scores, dP, dS and the half's dQ
          // products before the next half, so one half's S and dP are live.
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 sc = (f32x16){}, dp;
#pragma unroll
            for (int i = 0; i < 16; ++i) dp[i] = kNegDelta ? -dlt : 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
              mma(sc, prfrag<C::KS>(kt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0), qf[kk]);
              mma(dp, prfrag<C::KS>(vt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0), df[kk]);
            }
            if constexpr (JFA_DQ_NARROW_PREFETCH > 0 && sizeof(T) == 2)
              sched_prefetch<2 * (D / 16), 1, JFA_DQ_NARROW_PREFETCH>();
            // element tests only on blocks at the causal diagonal or the sequence end
            auto softmax = [&](auto edge_c) {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int kj = key0 + 32 * kb + res_row(i, g);
                float x = sc[i] * a.scale2 - lse2;
                if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
                float p = __builtin_amdgcn_exp2f(x);
                if (decltype(edge_c)::value && ((masked && kj > qi) || (padded && kj >= Lm))) p = 0.f;
                dp[i] = p * (kNegDelta ? dp[i] : dp[i] - dlt);
              }
            };
            if (masked || padded) softmax(std::true_type{});
            else softmax(std::false_type{});
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const Frag<T> sf = rfrag(dp, c, (T*)0);
#pragma unroll
              for (int db = 0; db < D / 32; ++db)
                mma(dq[db], ptfrag<C::KS>(kt, 32 * kb + 16 * c, 32 * db, lane, (T*)0), sf);
            }
            if constexpr (JFA_DQ_NARROW_PREFETCH > 0 && sizeof(T) == 2)
              sched_prefetch<2 * (D / 32), 2, JFA_DQ_NARROW_PREFETCH>();
          }
        } else {
          f32x16 sc[BN / 32], dp[BN / 32];
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb) {
            sc[kb] = (f32x16){};
#pragma unroll
            for (int i = 0; i < 16; ++i) dp[kb][i] = kNegDelta ? -dlt : 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
              mma(sc[kb], lfrag<D>(kt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0), qf[kk]);
              mma(dp[kb], lfrag<D>(vt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0), df[kk]);
            }
          }
          if constexpr (JFA_DQ_PREFETCH > 0 && D > 64 && sizeof(T) == 2)
            sched_prefetch<2 * (BN / 32) * (D / 16), 1, JFA_DQ_PREFETCH>();
          // Element tests only on blocks at the causal diagonal or the sequence end
          // (at D = 128 a second copy of the loop costs more than the tests save).
          auto softmax = [&](auto edge_c) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int kj = key0 + 32 * kb + res_row(i, g);
                float x = sc[kb][i] * a.scale2 - lse2;
                if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
                float p = __builtin_amdgcn_exp2f(x);
                if (decltype(edge_c)::value && ((masked && kj > qi) || (padded && kj >= Lm))) p = 0.f;
                dp[kb][i] = p * (kNegDelta ? dp[kb][i] : dp[kb][i] - dlt);
              }
            }
          };
          if constexpr (D > 64) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int kj = key0 + 32 * kb + res_row(i, g);
                float x = sc[kb][i] * a.scale2 - lse2;
                if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
                float p = __builtin_amdgcn_exp2f(x);
                if ((masked && kj > qi) || (padded && kj >= Lm)) p = 0.f;
                dp[kb][i] = p * (dp[kb][i] - dlt);
              }
            }
          } else if (masked || padded) {
            softmax(std::true_type{});
          } else {
            softmax(std::false_type{});
          }
#pragma unroll
          for (int kc = 0; kc < BN / 16; ++kc) {
            const Frag<T> sf = rfrag(dp[kc >> 1], kc & 1, (T*)0);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) mma(dq[db], tfrag<D>(kt, 16 * kc, 32 * db, lane, (T*)0), sf);
          }
          if constexpr (JFA_DQ_PREFETCH > 0 && D > 64 && sizeof(T) == 2)
            sched_prefetch<(BN / 16) * (D / 32), 2, JFA_DQ_PREFETCH>();
        }
      }
      wait_vmem();
      __syncthreads();
    }

    if (wave_on) {
      const View dqv = seq_view((char*)a.dq + qrow, Lq, gstride, C::ROWB);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          store4(dqv, (uint32_t)qi * gstride + d * ES, dq[db][4 * r] * a.scale, dq[db][4 * r + 1] * a.scale,
                 dq[db][4 * r + 2] * a.scale, dq[db][4 * r + 3] * a.scale, (T*)0);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused-dQ study modes (kBwdDq 1, 2): the fp32 accumulator is zeroed before
// the dK/dV launch (mode 1, a fill kernel), and afterwards one kernel writes
// dQ = scale * (the accumulator, or the sum of the key tiles' partials in
// key-tile order) for every sequence that took the dK/dV pass.
__global__ __launch_bounds__(256) void jfa_dqacc_zero_kernel(float* acc, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) acc[i] = 0.f;
}

template <typename T>
__global__ __launch_bounds__(256) void jfa_dq_fused_out_kernel(BwdArgs a, int D) {
  const int b = blockIdx.y;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int Lk = a.kv_off[b + 1] - a.kv_off[b];
  if (a.gfirst != nullptr && short_query(Lq, Lk)) return;  // the short-query pass writes these rows
  const int H = a.H;
  const long per_row = (long)H * D, n = (long)Lq * per_row;
  const int nkt = cdiv(Lk, kDkvTN);
  const size_t plane = (size_t)a.tq * H * D;  // one key tile's partials
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long)gridDim.x * 256) {
    const int i = (int)(e / per_row);
    const size_t at = (size_t)q0 * per_row + e;
    float v = 0.f;
    if constexpr (kBwdDq == 1) {
      v = a.dqacc[at];
    } else {
      const int last = a.causal ? min(nkt, i / kDkvTN + 1) : nkt;  // key tiles whose item visited row i
      for (int t = 0; t < last; ++t) v += a.dqacc[t * plane + at];
    }
    ((T*)a.dq)[at] = (T)(v * a.scale);
  }
}

template <typename K>
static long persistent_grid(K kern, int& occ, long max_items, int num_cus, int threads = 256) {
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess || occ < 1) occ = 1;
  }
  return max(1L, min(max_items, (long)num_cus * occ));
}

template <typename T, int D, bool BIAS, bool DBIAS>
static hipError_t launch_dkdv_t(const BwdArgs& a, long max_items, int num_cus, hipStream_t st) {
  static int occ = 0;
  constexpr int threads = DkvShape<T, D>::threads;
  const long g = persistent_grid(jfa_dkdv_kernel<T, D, BIAS, DBIAS>, occ, max_items, num_cus, threads);
  hipLaunchKernelGGL((jfa_dkdv_kernel<T, D, BIAS, DBIAS>), dim3((unsigned)g), dim3(threads), 0, st, a);
  return hipGetLastError();
}

// Bias gradient of each head, in two steps with a fixed order. Step 1: one
// workgroup per (head, block of kDbSeqBlock consecutive sequences) sums the
// bins of those sequences' items (sequences in order, each sequence's items
// in list order: they are contiguous in its list), one thread per bin
// (thread 0 also takes the last bin). Step 2: one workgroup per head sums
// the blocks in order.
__global__ __launch_bounds__(256) void jfa_dbias_part_kernel(BwdArgs a) {
  const int h = blockIdx.x % a.H, c = blockIdx.x / a.H, tid = threadIdx.x;
  const int b0 = c * kDbSeqBlock, b1 = min(a.B, b0 + kDbSeqBlock);
  float acc = 0.f, acc_last = 0.f;
  for (int b = b0; b < b1; ++b) {
    const int Lq = a.q_off[b + 1] - a.q_off[b], Lk = a.kv_off[b + 1] - a.kv_off[b];
    const bool sq = a.gfirst != nullptr && short_query(Lq, Lk);  // null: no short-query pass in this call
    const int first = sq ? a.gfirst[b * a.H + h] : a.gfirst_kv[b * a.H + h];
    if (first < 0) continue;
    const int n = sq ? cdiv(Lk, kSqKC) : cdiv(Lk, kDkvTN);
    const float* src = (sq ? a.dbp_sq : a.dbp_kv) + (size_t)first * kBiasLen;
#pragma unroll 8
    for (int t = 0; t < n; ++t) {
      acc += src[(size_t)t * kBiasLen + tid];
      if (tid == 0) acc_last += src[(size_t)t * kBiasLen + 256];
    }
  }
  float* out = a.dbpart + ((size_t)c * a.H + h) * kBiasLen;
  out[tid] = acc;
  if (tid == 0) out[256] = acc_last;
}

__global__ __launch_bounds__(256) void jfa_dbias_kernel(BwdArgs a) {
  const int h = blockIdx.x, tid = threadIdx.x;
  const int nc = cdiv(a.B, kDbSeqBlock);
  for (int r = tid; r < kBiasLen; r += 256) {
    float acc = 0.f;
    for (int c = 0; c < nc; ++c) acc += a.dbpart[((size_t)c * a.H + h) * kBiasLen + r];
    a.dbias[(size_t)h * kBiasLen + r] = acc;
  }
}

int dkv_tile_rows(bool f32, int D) {
  const bool one = f32 ? (D == 32 ? DkvShape<float, 32>::one_role : DkvShape<float, 64>::one_role)
                       : (D == 32 ? DkvShape<bf16, 32>::one_role
                                  : D == 64 ? DkvShape<bf16, 64>::one_role : DkvShape<bf16, 128>::one_role);
  return one ? kDkv1TM : kDkvTM;
}

template <typename T, int D, bool BIAS>
static hipError_t launch_dq_t(const BwdArgs& a, long max_items, int num_cus, hipStream_t st) {
  static int occ = 0;
  const long g = persistent_grid(jfa_dq_kernel<T, D, BIAS>, occ, max_items, num_cus);
  hipLaunchKernelGGL((jfa_dq_kernel<T, D, BIAS>), dim3((unsigned)g), dim3(256), 0, st, a);
  return hipGetLastError();
}

#define JFA_DISPATCH_TD(F32, D, CALL)                     \
  do {                                                    \
    if (F32) {                                            \
      if ((D) == 32) { using T = float; constexpr int DD = 32; return CALL; }  \
      if ((D) == 64) { using T = float; constexpr int DD = 64; return CALL; }  \
      return hipErrorInvalidValue; /* fp32 with D = 128 is rejected on the host */ \
    }                                                     \
    if ((D) == 32) { using T = bf16; constexpr int DD = 32; return CALL; }     \
    if ((D) == 64) { using T = bf16; constexpr int DD = 64; return CALL; }     \
    { using T = bf16; constexpr int DD = 128; return CALL; }                   \
  } while (0)


hipError_t launch_dkdv(bool f32, int D, const BwdArgs& a, bool bias, bool dbias, long max_items, int num_cus,
                       hipStream_t st) {
  if (bias && dbias) JFA_DISPATCH_TD(f32, D, (launch_dkdv_t<T, DD, true, true>(a, max_items, num_cus, st)));
  if (bias) JFA_DISPATCH_TD(f32, D, (launch_dkdv_t<T, DD, true, false>(a, max_items, num_cus, st)));
  JFA_DISPATCH_TD(f32, D, (launch_dkdv_t<T, DD, false, false>(a, max_items, num_cus, st)));
}

hipError_t launch_dbias(const BwdArgs& a, hipStream_t st) {
  const long nc = (a.B + kDbSeqBlock - 1) / kDbSeqBlock;
  if (nc > 0) hipLaunchKernelGGL(jfa_dbias_part_kernel, dim3((unsigned)(nc * a.H)), dim3(256), 0, st, a);
  if (a.H > 0) hipLaunchKernelGGL(jfa_dbias_kernel, dim3((unsigned)a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

int bwd_dq_mode(bool f32, int D) {
  if (kBwdDq == 0) return 0;
  const bool one = f32 ? (D == 32 ? DkvShape<float, 32>::one_role : DkvShape<float, 64>::one_role)
                       : (D == 32 ? DkvShape<bf16, 32>::one_role
                                  : D == 64 ? DkvShape<bf16, 64>::one_role : DkvShape<bf16, 128>::one_role);
  return one ? kBwdDq : 0;
}

hipError_t launch_dqacc_zero(float* acc, long n, hipStream_t st) {
  const long g = max(1L, min(4096L, (n + 255) / 256));
  hipLaunchKernelGGL(jfa_dqacc_zero_kernel, dim3((unsigned)g), dim3(256), 0, st, acc, n);
  return hipGetLastError();
}

hipError_t launch_dq_fused_out(bool f32, int D, const BwdArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  const dim3 grid(16, (unsigned)a.B);
  if (f32) hipLaunchKernelGGL(jfa_dq_fused_out_kernel<float>, grid, dim3(256), 0, st, a, D);
  else hipLaunchKernelGGL(jfa_dq_fused_out_kernel<bf16>, grid, dim3(256), 0, st, a, D);
  return hipGetLastError();
}

hipError_t launch_dq(bool f32, int D, const BwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st) {
  if (bias) JFA_DISPATCH_TD(f32, D, (launch_dq_t<T, DD, true>(a, max_items, num_cus, st)));
  JFA_DISPATCH_TD(f32, D, (launch_dq_t<T, DD, false>(a, max_items, num_cus, st)));
}

}  // namespace jfa
