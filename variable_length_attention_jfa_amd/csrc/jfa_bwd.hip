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
//  * jfa_delta_kernel : Delta per (token, head), one pass over O and dO.
//  * jfa_dkdv_kernel  : item = (b, h, 128-key tile); each wave owns 32 keys
//                       (K, V fragments in VGPRs) and walks 64-row query
//                       blocks staged in LDS; dK, dV stay in registers and
//                       are stored once.
//  * jfa_dq_kernel    : item = (b, h, 128-row query tile); each wave owns 32
//                       queries (Q, dO fragments in VGPRs) and walks 64-key
//                       blocks staged in LDS; dQ is stored once.
//
// Rows past a sequence's end load as zeros (Q = dO = 0 for pad queries,
// K = V = 0 for pad keys), so every product they enter is zero: no jagged
// mask is needed here. The causal mask zeroes P above the diagonal on the
// blocks that straddle it.
#include "jfa_common.h"
#include "jfa_kernels.h"

namespace jfa {



// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void jfa_delta_kernel(BwdArgs a) {
  constexpr int ROWB = D * (int)sizeof(T), TPR = ROWB / 16, RPB = 256 / TPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < a.rows) {
    const i32x4 o = *(const i32x4*)((const char*)a.out + row * ROWB + part * 16);
    const i32x4 d = *(const i32x4*)((const char*)a.dout + row * ROWB + part * 16);
    if (sizeof(T) == 2) {
      const bf16x8 o8 = __builtin_bit_cast(bf16x8, o), d8 = __builtin_bit_cast(bf16x8, d);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)o8[e] * (float)d8[e];
    } else {
      const f32x4 o4 = __builtin_bit_cast(f32x4, o), d4 = __builtin_bit_cast(f32x4, d);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += o4[e] * d4[e];
    }
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if (row < a.rows && part == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkvTiles {
  static constexpr int BNK = 128;  // keys per item (4 waves x 32)
  static constexpr int BMQ = 64;   // query rows per staged block
  static constexpr int THREADS = 256;
  using TL = Tile<T, D>;
  static constexpr int ROWB = TL::ROWB;
  static constexpr int QTILE = BMQ * ROWB;
  static constexpr int STAGE = 2 * QTILE + 2 * BMQ * 4;  // Q, dO, lse2, delta
  static constexpr int CPR = ROWB / 16;
  static constexpr int CPT = BMQ * CPR / THREADS;
  static constexpr int BIAS_OFF = 2 * STAGE;
  static constexpr int LDS = BIAS_OFF + 1040;
  static_assert((BMQ * CPR) % THREADS == 0, "tile pieces divide the workgroup");
  static_assert(BMQ == kDkvTM && BNK == kDkvTN, "tile shape published to the planner");
};

template <typename T, int D, bool BIAS>
__global__ __launch_bounds__(256, (D * sizeof(T) >= 256 ? 1 : 2)) void jfa_dkdv_kernel(BwdArgs a) {
  using C = DkvTiles<T, D>;
  constexpr int BNK = C::BNK, BMQ = C::BMQ, ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * C::ROWB;
  load_queues(a.hdr, &qcur);
  int home_q = 0, queues_left = -1;

  for (;;) {
    const int it = next_item(a.hdr, &qcur, &home_q, &queues_left);
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
    const View lv = seq_view(a.lse + (size_t)q0 * H + h, Lq, (uint32_t)H * 4, 4);
    const View dlv = seq_view(a.delta + (size_t)q0 * H + h, Lq, (uint32_t)H * 4, 4);

    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += C::THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }

    const int kw0 = key_tile0 + 32 * w;  // first key of this wave
    const bool wave_on = kw0 < Lk;
    const int kj = kw0 + l32;            // this lane's key
    Frag<T> kf[D / 16], vf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = gfrag(kv, (uint32_t)kj * gstride + (16 * kk + 8 * g) * ES, (T*)0);
      vf[kk] = gfrag(vv, (uint32_t)kj * gstride + (16 * kk + 8 * g) * ES, (T*)0);
    }

    i32x4 qr[C::CPT], dr[C::CPT];
    float lr = 0.f;
    auto gload = [&](int qb) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        const uint32_t off = (uint32_t)(qb * BMQ + row) * gstride + col * 16;
        qr[c] = ld16(qv, off);
        dr[c] = ld16(dov, off);
      }
      if (tid < BMQ) lr = ld4f(lv, (uint32_t)(qb * BMQ + tid) * H * 4) * kLog2e;
      else if (tid < 2 * BMQ) lr = ld4f(dlv, (uint32_t)(qb * BMQ + tid - BMQ) * H * 4);
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
      if (tid < 2 * BMQ) *(__attribute__((address_space(3))) float*)(st + 2 * C::QTILE + tid * 4) = lr;
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
      const __attribute__((address_space(3))) float* lse2 = (const __attribute__((address_space(3))) float*)(qt + 2 * C::QTILE);
      const __attribute__((address_space(3))) float* dl = lse2 + BMQ;
#pragma unroll
      for (int sb = 0; sb < BMQ / 32; ++sb) {
        const int qs0 = qb * BMQ + 32 * sb;  // first query of this 32-row sub-block
        const bool active = wave_on && qs0 < Lq && (!a.causal || qs0 + 31 >= kw0);
        if (!active) continue;
        const bool masked = a.causal && qs0 < kw0 + 31;
        f32x16 sc = (f32x16){}, dp = (f32x16){};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          mma(sc, lfrag<D>(qt, 32 * sb + l32, 16 * kk + 8 * g, (T*)0), kf[kk]);
          mma(dp, lfrag<D>(dot, 32 * sb + l32, 16 * kk + 8 * g, (T*)0), vf[kk]);
        }
        // sc[i] = S[query 32sb + res_row(i,g)][key kj]
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * sb + res_row(i, g);
          const int qi = qb * BMQ + r;
          float x = sc[i] * a.scale2 - lse2[r];
          if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
          float p = __builtin_amdgcn_exp2f(x);
          if (masked && kj > qi) p = 0.f;
          sc[i] = p;
          dp[i] = p * (dp[i] - dl[r]);
        }
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
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqTiles {
  static constexpr int BM = 128;  // query rows per item (4 waves x 32)
  static constexpr int BN = 64;   // keys per staged block
  static constexpr int THREADS = 256;
  using TL = Tile<T, D>;
  static constexpr int ROWB = TL::ROWB;
  static constexpr int KTILE = BN * ROWB;
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

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * C::ROWB;
  load_queues(a.hdr, &qcur);
  int home_q = 0, queues_left = -1;

  for (;;) {
    const int it = next_item(a.hdr, &qcur, &home_q, &queues_left);
    if (it < 0) break;
    const int4 item = a.items[it];
    const int b = item.x, h = item.y, qt = item.z;
    const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
    const int k0 = a.kv_off[b], Lk = a.kv_off[b + 1] - k0;
    const int row0 = qt * BM;
    const int n_kv = a.causal ? cdiv(min(min(row0 + BM, Lq), Lk), BN) : cdiv(Lk, BN);

    const size_t qrow = ((size_t)q0 * H + h) * C::ROWB, krow = ((size_t)k0 * H + h) * C::ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, C::ROWB);
    const View dov = seq_view((const char*)a.dout + qrow, Lq, gstride, C::ROWB);
    const View lv = seq_view(a.lse + (size_t)q0 * H + h, Lq, (uint32_t)H * 4, 4);
    const View dlv = seq_view(a.delta + (size_t)q0 * H + h, Lq, (uint32_t)H * 4, 4);

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
    const float lse2 = ld4f(lv, (uint32_t)qi * H * 4) * kLog2e;
    const float dlt = ld4f(dlv, (uint32_t)qi * H * 4);

    // K/V blocks through a two-stage LDS ring filled by direct loads: block
    // j+1 is requested while block j is computed.
    const DmaView kd = dma_view((const char*)a.k + krow, Lk, gstride, C::ROWB);
    const DmaView vd = dma_view((const char*)a.v + krow, Lk, gstride, C::ROWB);
    auto issue = [&](int j) {
      lds_t* st = lds + (j & 1) * C::STAGE;
      dma_tile<T, D, BN, 4>(kd, gstride, j * BN, st, w, lane);
      dma_tile<T, D, BN, 4>(vd, gstride, j * BN, st + C::KTILE, w, lane);
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
        // leak into dQ through the zero K row. Drop them on the last block.
        const bool padded = key0 + BN > Lk;
        const lds_t* kt = lds + s * C::STAGE;
        const lds_t* vt = kt + C::KTILE;
        f32x16 sc[BN / 32], dp[BN / 32];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
          sc[kb] = (f32x16){};
          dp[kb] = (f32x16){};
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            mma(sc[kb], lfrag<D>(kt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0), qf[kk]);
            mma(dp[kb], lfrag<D>(vt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0), df[kk]);
          }
        }
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kj = key0 + 32 * kb + res_row(i, g);
            float x = sc[kb][i] * a.scale2 - lse2;
            if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
            float p = __builtin_amdgcn_exp2f(x);
            if ((masked && kj > qi) || (padded && kj >= Lk)) p = 0.f;
            dp[kb][i] = p * (dp[kb][i] - dlt);
          }
        }
#pragma unroll
        for (int kc = 0; kc < BN / 16; ++kc) {
          const Frag<T> sf = rfrag(dp[kc >> 1], kc & 1, (T*)0);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) mma(dq[db], tfrag<D>(kt, 16 * kc, 32 * db, lane, (T*)0), sf);
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
template <typename K>
static long persistent_grid(K kern, int& occ, long max_items, int num_cus) {
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 256, 0) != hipSuccess || occ < 1) occ = 1;
  }
  return max(1L, min(max_items, (long)num_cus * occ));
}

template <typename T, int D>
static hipError_t launch_delta_t(const BwdArgs& a, hipStream_t st) {
  constexpr int RPB = 256 / (D * (int)sizeof(T) / 16);
  const long nblk = (a.rows + RPB - 1) / RPB;
  if (nblk > 0) hipLaunchKernelGGL((jfa_delta_kernel<T, D>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D, bool BIAS>
static hipError_t launch_dkdv_t(const BwdArgs& a, long max_items, int num_cus, hipStream_t st) {
  static int occ = 0;
  const long g = persistent_grid(jfa_dkdv_kernel<T, D, BIAS>, occ, max_items, num_cus);
  hipLaunchKernelGGL((jfa_dkdv_kernel<T, D, BIAS>), dim3((unsigned)g), dim3(256), 0, st, a);
  return hipGetLastError();
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

hipError_t launch_delta(bool f32, int D, const BwdArgs& a, hipStream_t st) {
  JFA_DISPATCH_TD(f32, D, (launch_delta_t<T, DD>(a, st)));
}

hipError_t launch_dkdv(bool f32, int D, const BwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st) {
  if (bias) JFA_DISPATCH_TD(f32, D, (launch_dkdv_t<T, DD, true>(a, max_items, num_cus, st)));
  JFA_DISPATCH_TD(f32, D, (launch_dkdv_t<T, DD, false>(a, max_items, num_cus, st)));
}

hipError_t launch_dq(bool f32, int D, const BwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st) {
  if (bias) JFA_DISPATCH_TD(f32, D, (launch_dq_t<T, DD, true>(a, max_items, num_cus, st)));
  JFA_DISPATCH_TD(f32, D, (launch_dq_t<T, DD, false>(a, max_items, num_cus, st)));
}

}  // namespace jfa
