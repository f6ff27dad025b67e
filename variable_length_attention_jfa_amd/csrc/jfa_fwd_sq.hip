// Forward pass for short-query sequences (at most 64 queries and more than
// 1024 keys, e.g. a few new events against a long history) on gfx950, split
// over the keys.
//
// The regular forward gives one workgroup a whole (b, h, query tile) and walks
// all its keys. With few queries and many keys that is a long serial stream
// per item: the grid holds too few bytes in flight, and one long sequence
// outlasts the rest of the batch. Here such a sequence is cut into chunks of
// 1024 keys, one item per (b, h, chunk), placed in a longest-first list like
// the other passes. Asymmetric query/key lengths are among the method's
// targets ("Jagged Flash Attention (JFA)", section "Definition"); its work
// list and persistent workgroups are item 3 of "Four generations".
//
// An item computes, for its keys only, the exact softmax-weighted sum of V
// for each query row, normalised by its own sum, and log2 of that sum (the
// running max plus log2 of the running sum). This pass runs before the
// query-tile forward, whose launch then combines the chunks of each (b, h)
// in list order (jfa_short.h):
//   M = max_c lse2_c,  w_c = 2^(lse2_c - M),  O = sum_c w_c O_c / sum_c w_c,
//   lse = (M + log2 sum_c w_c) * ln 2,
// which is the softmax over all keys regrouped by chunk (the same identity
// that lets the running max and sum of the tile loop move block by block).
// The chunk order is fixed, so the result is bit-identical run to run.
//
// Per 64-key tile, the four waves split the (query, key) block into 32 x 32
// quarters: wave w takes query half w >> 1 and key half w & 1, and keeps its
// own running max, running sum and O^T for the keys of its half:
//   S^T = K Q^T     K from LDS (natural), Q in VGPRs
//   O^T += V^T P^T  V read transposed from LDS, P from the score registers
// K and V arrive as whole rows, 16 bytes per lane, one tile ahead through
// registers into a second LDS stage. At the end of the item the two key
// halves of each query half are merged through LDS and the chunk's rows
// leave as whole rows.
//
// Jagged edges as in the regular forward ("Four generations" item 1): keys
// past the sequence end load as zeros; a wave counts their exp terms in its
// last half-tile and subtracts them once at the end. Only half-tiles that
// straddle the causal diagonal use an element mask.
#include "jfa_common.h"
#include "jfa_kernels.h"

namespace jfa {

template <typename T, int D>
struct FsqTiles {
  static constexpr int QM = kSqQMax;  // query rows of an item (two halves of 32)
  static constexpr int KT = 64;       // keys per tile (two halves of 32)
  static constexpr int KC = kSqKC;    // keys per item
  static constexpr int THREADS = 256;
  using TL = Tile<T, D>;
  static constexpr int ROWB = TL::ROWB;
  static constexpr int CPR = ROWB / 16;           // 16-byte pieces per row
  static constexpr int KTILE = KT * ROWB;
  static constexpr int STAGE = 2 * KTILE;         // K then V
  static constexpr int CPT = KT * CPR / THREADS;  // pieces per thread per tile
  static constexpr int BIAS_OFF = 2 * STAGE;
  static constexpr int LDS = BIAS_OFF + 1040;
  // Epilogue, in the stage area: the combined O rows, then (m, l) per wave and lane.
  using OL = Tile<float, D>;
  static constexpr int ML_OFF = QM * OL::ROWB;
  static_assert(ML_OFF + 4 * 32 * 16 <= 2 * STAGE, "epilogue fits the stage area");
  static_assert((KT * CPR) % THREADS == 0, "tile pieces divide the workgroup");
  static_assert(KC % KT == 0, "chunks are whole tiles");
};

template <typename T, int D, bool BIAS>
__global__ __launch_bounds__(256, 2) void jfa_fsq_kernel(FwdArgs a) {
  using C = FsqTiles<T, D>;
  constexpr int QM = C::QM, KT = C::KT, KC = C::KC, ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);
  __attribute__((address_space(3))) float* mlx = (__attribute__((address_space(3))) float*)(lds + C::ML_OFF);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = w >> 1, kh = w & 1;  // query half and key half of this wave
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
    const int kc0 = chunk * KC;  // first key of the chunk
    // Keys of the chunk that some query may see (top-left causal: key j is
    // visible to query i iff j <= i, and i < Lq).
    int kend = min(Lk, kc0 + KC);
    if (a.causal) kend = min(kend, Lq);
    const int nt = kend > kc0 ? cdiv(kend - kc0, KT) : 0;

    const size_t qrow = ((size_t)q0 * H + h) * C::ROWB, krow = ((size_t)k0 * H + h) * C::ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, C::ROWB);

    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += C::THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }

    const int wr0 = 32 * qh;  // first query row of this wave
    const bool wave_on = wr0 < Lq;
    const int qi = wr0 + l32;  // this lane's query row
    Frag<T> qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = gfrag(qv, (uint32_t)qi * gstride + (16 * kk + 8 * g) * ES, (T*)0);

    // K and V tiles: whole rows, 16 bytes per lane; rows past the end read as zeros.
    i32x4 kr[C::CPT], vr[C::CPT];
    auto gload = [&](int t) {
      const int r0 = kc0 + t * KT;
      const int rows = min(KT, Lk - r0);
      const View kv = seq_view((const char*)a.k + krow + (size_t)r0 * gstride, rows, gstride, C::ROWB);
      const View vv = seq_view((const char*)a.v + krow + (size_t)r0 * gstride, rows, gstride, C::ROWB);
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        const uint32_t off = (uint32_t)row * gstride + col * 16;
        kr[c] = ld16(kv, off);
        vr[c] = ld16(vv, off);
      }
    };
    auto swrite = [&](int s) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        const int o = C::TL::chunk(row, col);
        *(__attribute__((address_space(3))) i32x4*)(lds + s * C::STAGE + o) = kr[c];
        *(__attribute__((address_space(3))) i32x4*)(lds + s * C::STAGE + C::KTILE + o) = vr[c];
      }
    };
    if (nt > 0) {
      gload(0);
      swrite(0);
    }
    wait_vmem();
    __syncthreads();

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = (f32x16){};
    // l sums the fp32 P (for lse), lb the bf16-rounded P the PV product
    // consumes (the chunk's rows are normalised by it), as in the regular forward.
    constexpr bool kOpSum = sizeof(T) == 2;
    float m = kNegInit, l = 0.f, lb = 0.f;
    float l_pre = 0.f, lb_pre = 0.f;  // sums before the latest half-tile (cancellation guard)
    int last_tile = -1;
    bool last_masked = false;

    for (int t = 0; t < nt; ++t) {
      const int s = t & 1;
      if (t + 1 < nt) gload(t + 1);
      const int key0 = kc0 + t * KT + 32 * kh;  // first key of this wave's half
      const bool active = wave_on && key0 < kend && (!a.causal || key0 <= wr0 + 31);
      if (active) {
        const bool masked = a.causal && (key0 + 31 > wr0);
        last_tile = t;
        last_masked = masked;
        const lds_t* kt = lds + s * C::STAGE;
        const lds_t* vt = kt + C::KTILE;
        f32x16 sc = (f32x16){};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) mma(sc, lfrag<D>(kt, 32 * kh + l32, 16 * kk + 8 * g, (T*)0), qf[kk]);
        // Scores in log2 units: x = s * scale * log2(e) (+ bias * log2(e)).
        float mx = -INFINITY;
        const bool plain = !BIAS && !masked;
        if (plain) {
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[i]);
          mx = half_max(mx) * a.scale2;
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kj = key0 + res_row(i, g);
            float x = sc[i] * a.scale2;
            if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
            if (masked && (kj > qi || kj >= Lk)) x = -INFINITY;
            sc[i] = x;
            mx = fmaxf(mx, x);
          }
          mx = half_max(mx);
        }
        // Running max with slack, as in the regular forward: m moves only when
        // the block max exceeds it by more than kRescaleSlack (P <= 256).
        const bool grow = mx > m + kRescaleSlack;
        if (__any(grow)) {
          const float mn = grow ? mx : m;
          const float alpha = __builtin_amdgcn_exp2f(m - mn);
          m = mn;
          l *= alpha;
          lb *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        }
        l_pre = l;
        lb_pre = lb;
        if (plain) {
          const float nm = -m;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], a.scale2, nm));
            sc[i] = p;
            l += p;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[i] - m);
            sc[i] = p;
            l += p;
          }
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const Frag<T> pf = rfrag(sc, kc, (T*)0);
          if constexpr (kOpSum) lb = frag_sum(pf, lb);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) mma(o[db], tfrag<D>(vt, 32 * kh + 16 * kc, 32 * db, lane, (T*)0), pf);
        }
      }
      if (t + 1 < nt) swrite((t + 1) & 1);
      __syncthreads();
    }

    // Row sum over both lane halves; remove the terms of keys past the end.
    float lt = l + other_half(l);
    float lbt = kOpSum ? lb + other_half(lb) : lt;
    if (wave_on && last_tile >= 0 && !last_masked) {
      const int hk0 = kc0 + last_tile * KT + 32 * kh;  // first key of this wave's last half-tile
      const int pad1 = hk0 + 32;
      if (pad1 > Lk) {
        float pads, pads_b;
        if (!BIAS) {
          const float pe = __builtin_amdgcn_exp2f(-m);
          pads = (float)(pad1 - Lk) * pe;
          pads_b = (float)(pad1 - Lk) * as_operand(pe, (T*)0);
        } else {
          float sub = 0.f, subb = 0.f;
          for (int kj = Lk + g; kj < pad1; kj += 2) {
            const float pe =
                __builtin_amdgcn_exp2f(bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius] - m);
            sub += pe;
            subb += as_operand(pe, (T*)0);
          }
          pads = sub + other_half(sub);
          pads_b = subb + other_half(subb);
        }
        const float full = lt;
        lt -= pads;
        lbt -= pads_b;
        // Cancellation guard, as in the regular forward: when the remainder
        // keeps fewer than ~12 significant bits, the half-tile's valid terms
        // are summed again (plain dot products against the K rows still in
        // LDS) on top of the sum before that half-tile.
        const bool cancel = !(lt > full * 0x1p-12f);
        if (__any(cancel)) {
          const lds_t* kt = lds + (last_tile & 1) * C::STAGE;
          float sv = 0.f, svb = 0.f;
#pragma unroll 1
          for (int r = g; r < 32; r += 2) {
            const int kj = hk0 + r;
            if (kj >= Lk) break;  // keys past the end follow the valid ones
            float dot = 0.f;
#pragma unroll 1
            for (int c = 0; c < C::CPR; ++c) {
              const i32x4 kq = *(const __attribute__((address_space(3))) i32x4*)(kt + C::TL::chunk(32 * kh + r, c));
              const i32x4 qq = ld16(qv, (uint32_t)qi * gstride + c * 16);
              if constexpr (sizeof(T) == 2) {
                const bf16x8 k8 = __builtin_bit_cast(bf16x8, kq), q8 = __builtin_bit_cast(bf16x8, qq);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot += (float)k8[e] * (float)q8[e];
              } else {
                const f32x4 k4 = __builtin_bit_cast(f32x4, kq), q4 = __builtin_bit_cast(f32x4, qq);
#pragma unroll
                for (int e = 0; e < 4; ++e) dot += k4[e] * q4[e];
              }
            }
            float x = dot * a.scale2;
            if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
            const float pe = __builtin_amdgcn_exp2f(x - m);
            sv += pe;
            svb += as_operand(pe, (T*)0);
          }
          const float fixed = l_pre + other_half(l_pre) + sv + other_half(sv);
          const float fixedb = kOpSum ? lb_pre + other_half(lb_pre) + svb + other_half(svb) : fixed;
          if (cancel) {
            lt = fixed;
            lbt = fixedb;
          }
        }
      }
    }
    __syncthreads();  // the K tiles are read above; the merge below reuses their LDS

    // Merge the two key halves of each query half: (m, l, lb) through LDS,
    // then the key-half-1 wave's weighted O^T, to which its partner adds its own.
    if (g == 0) {
      mlx[(w * 32 + l32) * 4] = m;
      mlx[(w * 32 + l32) * 4 + 1] = lt;
      mlx[(w * 32 + l32) * 4 + 2] = lbt;
    }
    __syncthreads();
    const int pw = w ^ 1;
    const float mp = mlx[(pw * 32 + l32) * 4], lp = mlx[(pw * 32 + l32) * 4 + 1];
    const float lpb = mlx[(pw * 32 + l32) * 4 + 2];
    const float M = fmaxf(m, mp);
    const float cw = __builtin_amdgcn_exp2f(m - M), cp = __builtin_amdgcn_exp2f(mp - M);
    const float L = lt * cw + lp * cp;     // fp32 sum: the chunk's lse
    const float Lb = lbt * cw + lpb * cp;  // operand sum: the chunk's normalisation
    const float f = Lb > 0.f ? cw / Lb : 0.f;  // weight of this wave's O^T in the normalised row
    using OL = typename C::OL;
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          *(__attribute__((address_space(3))) f32x4*)(lds + OL::byte(qi, d * 4)) =
              (f32x4){o[db][4 * r] * f, o[db][4 * r + 1] * f, o[db][4 * r + 2] * f, o[db][4 * r + 3] * f};
        }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          __attribute__((address_space(3))) f32x4* p = (__attribute__((address_space(3))) f32x4*)(lds + OL::byte(qi, d * 4));
          const f32x4 x = *p;
          *p = (f32x4){x[0] + o[db][4 * r] * f, x[1] + o[db][4 * r + 1] * f, x[2] + o[db][4 * r + 2] * f,
                       x[3] + o[db][4 * r + 3] * f};
        }
      if (g == 0) a.lsep[(size_t)it * QM + qi] = L > 0.f ? M + __builtin_amdgcn_logf(L) : -INFINITY;
    }
    __syncthreads();
    // The chunk's normalised rows, whole rows out (rows past Lq are dropped).
    const View pv = seq_view(a.op + (size_t)it * QM * D, Lq, D * 4, D * 4);
    rows_out<float, D, QM, C::THREADS>(lds, pv, D * 4, 1.0f, tid);
  }
}

template <typename T, int D, bool BIAS>
static hipError_t launch_fsq_t(const FwdArgs& a, long max_items, int num_cus, hipStream_t st) {
  static int occ = 0;
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, jfa_fsq_kernel<T, D, BIAS>, 256, 0) != hipSuccess || occ < 1)
      occ = 1;
  }
  const long g = max(1L, min(max_items, (long)num_cus * occ));
  hipLaunchKernelGGL((jfa_fsq_kernel<T, D, BIAS>), dim3((unsigned)g), dim3(256), 0, st, a);
  return hipGetLastError();
}

#define JFA_FSQ_DISPATCH(F32, D, CALL)                                           \
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

hipError_t launch_fsq(bool f32, int D, const FwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st) {
  if (bias) JFA_FSQ_DISPATCH(f32, D, (launch_fsq_t<T, DD, true>(a, max_items, num_cus, st)));
  JFA_FSQ_DISPATCH(f32, D, (launch_fsq_t<T, DD, false>(a, max_items, num_cus, st)));
}

}  // namespace jfa
