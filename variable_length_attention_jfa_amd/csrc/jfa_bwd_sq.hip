// Backward pass for short-query sequences (at most 64 queries and more than
// 1024 keys, e.g. a few new events attending to a long history) on gfx950.
//
// The split backward ("Jagged Flash Attention (JFA)", section "Four
// generations", item 2) computes dK/dV per key tile and dQ per query tile in
// two passes, so K and V are read twice and S = QK^T, dP = dO V^T are formed
// twice. When a sequence has at most 64 queries they fit one workgroup, which
// can then own the whole sequence's backward: one item per (b, h, chunk of
// 1024 keys) reads each K, V row once, forms S, P, dP, dS once, stores the
// chunk's dK, dV directly and accumulates a partial dQ over its keys. This
// pass runs before the dQ pass, whose launch first sums the partials of each
// sequence's chunks in list order (jfa_short.h), so dQ is deterministic and
// is never accumulated across workgroups. The same page
// counts asymmetric query/key lengths among the method's targets (section
// "Definition").
//
// Per 64-key tile, the four waves split the 64 x 64 (key, query) block into
// 32 x 32 quarters, wave w taking key half w & 1 and query half w >> 1:
//   S = Q K^T, dP = dO V^T   (Q, dO, K, V all from LDS)
//   P = exp2(S * scale * log2(e) - lse2 (+ bias)), dS = P (dP - Delta),
//   both written as [key][query] tiles into the LDS that held V
//   dV^T += dO^T P^T, dK^T += Q^T dS^T for the key half, the two waves of a
//   key half taking alternate 32-column blocks of D
//   dQ^T += K^T dS^T per (query half, column block), K and dS read
//   transposed from LDS.
// The tile's dV and dK are then staged in the LDS of V and K and leave as
// whole rows, 16 bytes per lane: written straight from the MFMA result
// layout each store instruction would touch 32 rows with a few bytes each,
// and the memory system runs out of requests long before it runs out of
// bytes. K and V arrive the same way, in whole rows, one tile ahead, through
// registers. The LDS of one workgroup (Q, dO, K, V or P and dS, row
// constants, bias) stays under 80 KB at D = 128 in bf16, so two workgroups
// share a CU.
// Rows past a sequence's end load as zeros; keys past the end and, with the
// causal mask, keys after the query get P = 0.
#include <type_traits>

#include "jfa_common.h"
#include "jfa_kernels.h"
#include "jfa_dbias.h"

namespace jfa {

template <typename T, int D>
struct SqTiles {
  static constexpr int QM = kSqQMax;  // query rows (two halves of 32)
  static constexpr int KT = kSqKT;    // keys per tile (two halves of 32)
  static constexpr int KC = kSqKC;    // keys per item
  static constexpr int THREADS = 256;
  using TL = Tile<T, D>;   // Q, dO, K rows
  using PL = Tile<T, QM>;  // P, dS: one row of QM queries per key
  static constexpr int ROWB = TL::ROWB;
  static constexpr int CPR = ROWB / 16;
  static constexpr int QOFF = 0;
  static constexpr int DOFF = QM * ROWB;
  static constexpr int KOFF = 2 * QM * ROWB;
  static constexpr int VOFF = KOFF + KT * ROWB;         // V, then P and dS, then staged dV
  static constexpr int VREG = KT * ROWB > 2 * KT * PL::ROWB ? KT * ROWB : 2 * KT * PL::ROWB;
  static constexpr int POFF = VOFF;
  static constexpr int SOFF = VOFF + KT * PL::ROWB;
  static constexpr int RCOFF = VOFF + VREG;            // (lse2, Delta) per query row
  static constexpr int BIAS_OFF = RCOFF + QM * 8;
  static constexpr int LDS = BIAS_OFF + 1040;
  static constexpr int KCPT = KT * CPR / THREADS;       // K (or V) tile pieces per thread
  static constexpr int QCPT = (2 * QM * CPR + THREADS - 1) / THREADS;  // Q and dO pieces per thread
  static constexpr int NDB = D / 32;                    // 32-column blocks of D
  static constexpr int NDB2 = (NDB + 1) / 2;            // column blocks per wave
  static constexpr int NDQ = 2 * NDB;                   // 32x32 dQ blocks
  static_assert((KT * CPR) % THREADS == 0, "tile pieces divide the workgroup");
  static_assert((QM * CPR) % THREADS == 0, "Q and dO pieces fill whole passes of the workgroup");
  static_assert(KC % KT == 0, "chunks are whole tiles");
};

// Fragment from one row of a [key][query] tile for a 32x32x16 MFMA operand
// whose k runs over queries: k-slots = queries 16c + {4g .. 4g+3, 8+4g ..
// 8+4g+3}, the order of the transposed fragment on the other side.
__device__ __forceinline__ Frag<bf16> pfrag(const lds_t* tile, int row, int c, int g, bf16*) {
  using PL = Tile<bf16, kSqQMax>;
  const i32x2 x = *(const __attribute__((address_space(3))) i32x2*)(tile + PL::byte(row, (16 * c + 4 * g) * 2));
  const i32x2 y = *(const __attribute__((address_space(3))) i32x2*)(tile + PL::byte(row, (16 * c + 8 + 4 * g) * 2));
  const bf16x4 x4 = __builtin_bit_cast(bf16x4, x), y4 = __builtin_bit_cast(bf16x4, y);
  Frag<bf16> f;
  f.v = (bf16x8){x4[0], x4[1], x4[2], x4[3], y4[0], y4[1], y4[2], y4[3]};
  return f;
}
__device__ __forceinline__ Frag<float> pfrag(const lds_t* tile, int row, int c, int g, float*) {
  using PL = Tile<float, kSqQMax>;
  Frag<float> f;
  f.lo = *(const __attribute__((address_space(3))) f32x4*)(tile + PL::byte(row, (16 * c + 4 * g) * 4));
  f.hi = *(const __attribute__((address_space(3))) f32x4*)(tile + PL::byte(row, (16 * c + 8 + 4 * g) * 4));
  return f;
}

// Four consecutive values (columns col .. col+3) of one row of a tile of W
// columns. In a 32x32 result held by a lane of half g, elements 4a .. 4a+3
// are columns 8a+4g .. +3 of the lane's row.
template <int W>
__device__ __forceinline__ void put4(lds_t* tile, int row, int col, float a, float b, float c, float d, bf16*) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 lo = {(bf16)a, (bf16)b}, hi = {(bf16)c, (bf16)d};
  *(__attribute__((address_space(3))) i32x2*)(tile + Tile<bf16, W>::byte(row, col * 2)) =
      (i32x2){__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
}
template <int W>
__device__ __forceinline__ void put4(lds_t* tile, int row, int col, float a, float b, float c, float d, float*) {
  *(__attribute__((address_space(3))) f32x4*)(tile + Tile<float, W>::byte(row, col * 4)) = (f32x4){a, b, c, d};
}

// One entry of a [key][query] tile, as float.
__device__ __forceinline__ float tile_at(const lds_t* tile, int row, int col, bf16*) {
  return (float)*(const __attribute__((address_space(3))) bf16*)(tile + Tile<bf16, kSqQMax>::byte(row, col * 2));
}
__device__ __forceinline__ float tile_at(const lds_t* tile, int row, int col, float*) {
  return *(const __attribute__((address_space(3))) float*)(tile + Tile<float, kSqQMax>::byte(row, col * 4));
}

// DBIAS (with BIAS): also the bias-gradient bins of each item.
template <typename T, int D, bool BIAS, bool DBIAS>
__global__ __launch_bounds__(256, 2) void jfa_sq_kernel(BwdArgs a) {
  using C = SqTiles<T, D>;
  constexpr int QM = C::QM, KT = C::KT, KC = C::KC, ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS + (DBIAS ? 4 * kDbHistBytes : 0)];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  lds_t* qt = lds + C::QOFF;
  lds_t* dot = lds + C::DOFF;
  lds_t* kt = lds + C::KOFF;  // K tile, then staged dK
  lds_t* vt = lds + C::VOFF;  // V tile, then P and dS, then staged dV
  lds_t* pt = lds + C::POFF;  // P   [key][query]
  lds_t* st = lds + C::SOFF;  // dS  [key][query]
  __attribute__((address_space(3))) float* rc = (__attribute__((address_space(3))) float*)(lds + C::RCOFF);
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * C::ROWB;
  load_queues(a.hdr, &qcur);
  TicketState tk;

  for (;;) {
    const int it = next_item(a.hdr, &qcur, tk);
    if (it < 0) break;
    const int4 item = a.items[it];
    const int b = uni(item.x), h = uni(item.y), chunk = uni(item.z);
    const int q0 = uni(a.q_off[b]), Lq = uni(a.q_off[b + 1]) - q0;
    const int k0 = uni(a.kv_off[b]), Lk = uni(a.kv_off[b + 1]) - k0;
    const int key_c0 = chunk * KC;                                   // first key of the chunk
    const int nt = Lk > key_c0 ? cdiv(min(KC, Lk - key_c0), KT) : 0;  // key tiles in the chunk
    const int nqs = cdiv(min(Lq, QM), 32);                           // query halves in use

    const size_t qrow = ((size_t)q0 * H + h) * C::ROWB, krow = ((size_t)k0 * H + h) * C::ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, C::ROWB);
    const View dov = seq_view((const char*)a.dout + qrow, Lq, gstride, C::ROWB);
    const View rcv = seq_view(a.rowc + (size_t)q0 * H + h, Lq, 8 * H, 8);

    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += C::THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }
    // Q, dO (rows past Lq read as zeros) and the row constants into LDS.
    {
      i32x4 r[C::QCPT];
#pragma unroll
      for (int c = 0; c < C::QCPT; ++c) {
        const int x = tid + C::THREADS * c;
        if (x < 2 * QM * C::CPR) {
          const int y = x % (QM * C::CPR), row = y / C::CPR, col = y % C::CPR;
          // pieces c * THREADS .. are all Q or all dO (a whole number of passes per tile)
          r[c] = ld16(c * C::THREADS < QM * C::CPR ? qv : dov, (uint32_t)row * gstride + col * 16);
        }
      }
      i32x2 rr = {};
      if (tid < QM) rr = ld8(rcv, (uint32_t)tid * 8 * H);
#pragma unroll
      for (int c = 0; c < C::QCPT; ++c) {
        const int x = tid + C::THREADS * c;
        if (x < 2 * QM * C::CPR) {
          const int y = x % (QM * C::CPR), row = y / C::CPR, col = y % C::CPR;
          *(__attribute__((address_space(3))) i32x4*)((c * C::THREADS < QM * C::CPR ? qt : dot) + C::TL::chunk(row, col)) = r[c];
        }
      }
      // queries past the sequence end: lse2 = +inf, so their P is 0 whatever the bias
      if (tid >= Lq) rr[0] = __float_as_int(INFINITY);
      if (tid < QM) *(__attribute__((address_space(3))) i32x2*)((lds_t*)rc + 8 * tid) = rr;
    }

    // K and V tiles: whole rows, 16 bytes per lane, through registers into LDS.
    auto tview = [&](const void* base, int t) {
      const int r0 = key_c0 + t * KT;
      return seq_view((const char*)base + krow + (size_t)r0 * gstride, min(KT, Lk - r0), gstride, C::ROWB);
    };
    auto tload = [&](const void* base, int t, i32x4* r) {
      const View tv = tview(base, t);
#pragma unroll
      for (int c = 0; c < C::KCPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        r[c] = ld16(tv, (uint32_t)row * gstride + col * 16);
      }
    };
    auto tstore = [&](lds_t* dst, const i32x4* r) {
#pragma unroll
      for (int c = 0; c < C::KCPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        *(__attribute__((address_space(3))) i32x4*)(dst + C::TL::chunk(row, col)) = r[c];
      }
    };
    auto tout = [&](void* base, int t, const lds_t* src) {  // staged tile -> global rows
      const View tv = tview(base, t);
#pragma unroll
      for (int c = 0; c < C::KCPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        st16(tv, (uint32_t)row * gstride + col * 16,
             *(const __attribute__((address_space(3))) i32x4*)(src + C::TL::chunk(row, col)));
      }
    };

    i32x4 kr[C::KCPT], vr[C::KCPT];
    if (nt > 0) {
      tload(a.k, 0, kr);
      tload(a.v, 0, vr);
      tstore(kt, kr);
      tstore(vt, vr);
    }
    wait_vmem();
    __syncthreads();

    f32x16 dq[(C::NDQ + 3) / 4];
#pragma unroll
    for (int x = 0; x < (C::NDQ + 3) / 4; ++x) dq[x] = (f32x16){};

    const int kh = w & 1, qh = w >> 1;  // key half and query half of this wave
    const int krow_t = 32 * kh + l32;   // this lane's key row in the tile
    DbWave db;
    if (DBIAS) {
      db = db_wave_hist(lds + C::LDS, w);
      db_begin(db, lane);
    }
    for (int t = 0; t < nt; ++t) {
      if (t + 1 < nt) {
        tload(a.k, t + 1, kr);
        tload(a.v, t + 1, vr);
      }
      const int kj = key_c0 + t * KT + krow_t;  // this lane's key
      bool db_near = false;  // this wave's dS quarter straddles the bias radius
      // S, dP of (key half kh, query half qh).
      f32x16 sc = (f32x16){}, dp = (f32x16){};
      if (qh < nqs) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          mma(sc, lfrag<D>(qt, 32 * qh + l32, 16 * kk + 8 * g, (T*)0), lfrag<D>(kt, krow_t, 16 * kk + 8 * g, (T*)0));
          mma(dp, lfrag<D>(dot, 32 * qh + l32, 16 * kk + 8 * g, (T*)0), lfrag<D>(vt, krow_t, 16 * kk + 8 * g, (T*)0));
        }
      }
      __syncthreads();  // V is consumed: P and dS take its place
      if (qh < nqs) {
        // element tests only with the causal mask or on the tile holding the sequence end
        auto softmax = [&](auto edge_c) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = 32 * qh + res_row(i, g);
            float x = sc[i] * a.scale2 - rc[2 * qi];
            if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
            float p = __builtin_amdgcn_exp2f(x);
            if (decltype(edge_c)::value && (kj >= Lk || (a.causal && kj > qi))) p = 0.f;
            sc[i] = p;
            dp[i] = p * (dp[i] - rc[2 * qi + 1]);
          }
        };
        if (a.causal || key_c0 + t * KT + KT > Lk) softmax(std::true_type{});
        else softmax(std::false_type{});
        // bias-gradient bins: blocks beyond the radius here, the others from the dS tile below
        // (keys past the end already have P = 0)
        if (DBIAS) db_near = !db_far(db, dp, 32 * qh - (key_c0 + t * KT + 32 * kh));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = 32 * qh + 8 * r + 4 * g;
          put4<QM>(pt, krow_t, q, sc[4 * r], sc[4 * r + 1], sc[4 * r + 2], sc[4 * r + 3], (T*)0);
          put4<QM>(st, krow_t, q, dp[4 * r], dp[4 * r + 1], dp[4 * r + 2], dp[4 * r + 3], (T*)0);
        }
      }
      __syncthreads();
      if (DBIAS && db_near) {  // diagonal i - j = lane - 31 of this wave's quarter of the dS tile
        const int d = lane - 31;
        float v = 0.f;
        if (lane < 63) {
          for (int i = max(0, d); i < min(32, 32 + d); ++i) v += tile_at(st, 32 * kh + i - d, 32 * qh + i, (T*)0);
        }
        db_diag(db, v, 32 * qh - (key_c0 + t * KT + 32 * kh), lane);
      }
      // dV^T, dK^T of key half kh, column blocks qh, qh + 2, ...: lane holds
      // rows d = 32db + res_row(i,g) of key kj.
      f32x16 av[C::NDB2], ak[C::NDB2];
#pragma unroll
      for (int j = 0; j < C::NDB2; ++j) {
        const int db = qh + 2 * j;
        av[j] = (f32x16){};
        ak[j] = (f32x16){};
        if (db < C::NDB) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (c < 2 * nqs) {
              mma(av[j], tfrag<D>(dot, 16 * c, 32 * db, lane, (T*)0), pfrag(pt, krow_t, c, g, (T*)0));
              mma(ak[j], tfrag<D>(qt, 16 * c, 32 * db, lane, (T*)0), pfrag(st, krow_t, c, g, (T*)0));
            }
          }
        }
      }
      // dQ^T += K^T dS^T over the tile's keys; block x of this wave is
      // (query half x % 2, column block x / 2), x = w, w + 4, ...
#pragma unroll
      for (int xi = 0; xi < (C::NDQ + 3) / 4; ++xi) {
        const int x = w + 4 * xi;
        if (x < C::NDQ && (x % 2) < nqs) {
          const int qs = x % 2, db = x / 2;
#pragma unroll
          for (int kc = 0; kc < KT / 16; ++kc)
            mma(dq[xi], tfrag<D>(kt, 16 * kc, 32 * db, lane, (T*)0), tfrag<QM>(st, 16 * kc, 32 * qs, lane, (T*)0));
        }
      }
      __syncthreads();  // K, P and dS are consumed: stage dV over V, dK over K
#pragma unroll
      for (int j = 0; j < C::NDB2; ++j) {
        const int db = qh + 2 * j;
        if (db < C::NDB) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = 32 * db + 8 * r + 4 * g;
            put4<D>(vt, krow_t, d, av[j][4 * r], av[j][4 * r + 1], av[j][4 * r + 2], av[j][4 * r + 3], (T*)0);
            put4<D>(kt, krow_t, d, ak[j][4 * r] * a.scale, ak[j][4 * r + 1] * a.scale, ak[j][4 * r + 2] * a.scale,
                    ak[j][4 * r + 3] * a.scale, (T*)0);
          }
        }
      }
      __syncthreads();
      tout(a.dv, t, vt);
      tout(a.dk, t, kt);
      __syncthreads();  // staging read: the next tile's K and V may land
      if (t + 1 < nt) {
        tstore(kt, kr);
        tstore(vt, vr);
        __syncthreads();
      }
    }

    // Partial dQ of this chunk (unscaled), staged in LDS as [64 rows][D] fp32
    // and written as whole rows of valid queries to item slot it; the dQ
    // launch sums the chunks. LDS is free: the last tile ended on a barrier.
#pragma unroll
    for (int xi = 0; xi < (C::NDQ + 3) / 4; ++xi) {
      const int x = w + 4 * xi;
      if (x < C::NDQ) {
        const int qs = x % 2, db = x / 2, q = 32 * qs + l32;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          *(__attribute__((address_space(3))) f32x4*)(lds + Tile<float, D>::byte(q, d * 4)) =
              (f32x4){dq[xi][4 * r], dq[xi][4 * r + 1], dq[xi][4 * r + 2], dq[xi][4 * r + 3]};
        }
      }
    }
    __syncthreads();
    const View pv = seq_view(a.dqp + (size_t)it * QM * D, Lq, D * 4, D * 4);
    rows_out<float, D, QM, C::THREADS>(lds, pv, D * 4, 1.0f, tid);
    if (DBIAS) {  // the item's bias-gradient bins, waves in order
      db_finish(db, lane);
      __syncthreads();
      db_store(lds + C::LDS, 4, a.dbp_sq + (size_t)it * kBiasLen, tid, C::THREADS, kDbHistBytes, 0);
    }
  }
}

template <typename T, int D, bool BIAS, bool DBIAS>
static hipError_t launch_sq_t(const BwdArgs& a, long max_items, int num_cus, hipStream_t st) {
  static int occ = 0;
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, jfa_sq_kernel<T, D, BIAS, DBIAS>, 256, 0) != hipSuccess || occ < 1)
      occ = 1;
  }
  const long g = max(1L, min(max_items, (long)num_cus * occ));
  hipLaunchKernelGGL((jfa_sq_kernel<T, D, BIAS, DBIAS>), dim3((unsigned)g), dim3(256), 0, st, a);
  return hipGetLastError();
}

#define JFA_SQ_DISPATCH(F32, D, CALL)                                            \
  do {                                                                           \
    if (F32) {                                                                   \
      if ((D) == 32) { using T = float; constexpr int DD = 32; return CALL; }    \
      if ((D) == 64) { using T = float; constexpr int DD = 64; return CALL; }    \
      return hipErrorInvalidValue; /* fp32 with D = 128 is rejected on the host */ \
    }                                                                            \
    if ((D) == 32) { using T = bf16; constexpr int DD = 32; return CALL; }       \
    if ((D) == 64) { using T = bf16; constexpr int DD = 64; return CALL; }       \
    { using T = bf16; constexpr int DD = 128; return CALL; }                     \
  } while (0)

hipError_t launch_sq(bool f32, int D, const BwdArgs& a, bool bias, bool dbias, long max_items, int num_cus,
                     hipStream_t st) {
  if (bias && dbias) JFA_SQ_DISPATCH(f32, D, (launch_sq_t<T, DD, true, true>(a, max_items, num_cus, st)));
  if (bias) JFA_SQ_DISPATCH(f32, D, (launch_sq_t<T, DD, true, false>(a, max_items, num_cus, st)));
  JFA_SQ_DISPATCH(f32, D, (launch_sq_t<T, DD, false, false>(a, max_items, num_cus, st)));
}

}  // namespace jfa
