// Forward pass of jagged exact-softmax attention on gfx950.
//
// One persistent workgroup (4 waves) takes work items (b, h, query tile of 128
// rows) from the longest-first list and walks the key/value blocks of that
// sequence ("Jagged Flash Attention (JFA)", sections "Why standard
// FlashAttention falls short" and "Four generations" item 3). Each wave owns
// 32 query rows. Per 64-key block:
//   S^T = K Q^T          bf16 MFMA 32x32x16, K from LDS (natural), Q in VGPRs
//   online softmax       one lane per query: 16 scores per half-wave lane,
//                        the two halves combined with one permlane32 swap
//   O^T += V^T P^T       V read transposed from LDS (ds_read_b64_tr_b16),
//                        P straight from the score registers
// Tiling + running max / running sum: "TLX-Optimized Jagged Flash Attention:
// Approaching FA4-Level Performance on Blackwell", section "Why Jagged Flash
// Attention Deserves Attention".
//
// Jagged edges ("Jagged Flash Attention (JFA)", "Four generations" item 1):
// keys past the sequence end load as zeros, so their score is the bias value
// (0 without bias) and their value row is 0. They add nothing to O and add
// exp(score - m) each to the running sum, which is subtracted once in the
// epilogue (the block holding them is the last one visited, so m is final
// when they are counted). Query rows past the end load as zeros and their
// stores are dropped. Only blocks that straddle the causal diagonal use an
// element mask (which then also drops keys past the end).
#include "jfa_common.h"
#include "jfa_kernels.h"
#include "jfa_short.h"

// How keys past a sequence's end leave the softmax. 0: they load as zeros and
// their exp terms are subtracted once in the epilogue (the method). 1 and 2
// exist only for an instruction-mix study against -inf masking: 1 masks them
// with -inf in the block that holds them, 2 bounds-checks every key of every
// block as a padded kernel would.
#ifndef JFA_FWD_MASK_MODE
#define JFA_FWD_MASK_MODE 0
#endif

namespace jfa {

// How forward workgroups take work. 1: persistent, CUs x resident workgroups,
// each takes items until the list is empty (the method). 0 exists only for a
// scheduling study: one workgroup per list slot, each takes one item.
#ifndef JFA_SCHED_PERSISTENT
#define JFA_SCHED_PERSISTENT 1
#endif

// Workgroups per CU the register budget is held to: rows of up to 128 bytes
// (JFA_FWD_BLOCKS; the compiler's allocation gives bf16 at D <= 64 three
// waves per SIMD at 2) and rows of 256 bytes (JFA_FWD_WIDE_BLOCKS); wider
// rows one. Tile-shape study choices, as are the block widths (jfa_kernels.h)
// and JFA_FWD_WIDE_DMA (1: rows of 256 bytes and more arrive by direct loads
// into LDS, 0: staged through registers).
#ifndef JFA_FWD_BLOCKS
#define JFA_FWD_BLOCKS 2
#endif
#ifndef JFA_FWD_WIDE_BLOCKS
#define JFA_FWD_WIDE_BLOCKS 2
#endif
#ifndef JFA_FWD_WIDE_DMA
#define JFA_FWD_WIDE_DMA 0
#endif
// Matrix products whose LDS operands are read ahead of them, for rows of 256
// bytes and more (0: the compiler's order, which waits for each product's
// reads right before it).
#ifndef JFA_FWD_PREFETCH
#define JFA_FWD_PREFETCH 2
#endif
// The same for the two-group kernel (at least 1).
#ifndef JFA_FWD_PP_AHEAD
#define JFA_FWD_PP_AHEAD 2
#endif

constexpr int kFwdMaskMode = JFA_FWD_MASK_MODE;
constexpr bool kSchedPersistent = JFA_SCHED_PERSISTENT != 0;
static_assert(kFwdMaskMode >= 0 && kFwdMaskMode <= 2, "mask mode");

template <typename T, int D>
struct FwdTiles {
  static constexpr int BM = 128;  // query rows per item (4 waves x 32)
  static constexpr int BN = FwdKeys<T, D>::value;  // keys per block
  static constexpr int THREADS = 256;
  using TL = Tile<T, D>;
  static constexpr int ROWB = TL::ROWB;
  // K and V tiles with padded rows: K read naturally (S^T = K Q^T), V read
  // transposed (O^T += V^T P^T); see pad_nat / pad_tr
  static constexpr int KS = pad_nat(ROWB), VS = pad_tr(ROWB);
  // Rows of 256 bytes and more arrive by direct loads into LDS (their staging
  // registers would cost a wave per SIMD); each tile then spans whole KBs.
  static constexpr bool DMA = ROWB >= 256 && JFA_FWD_WIDE_DMA;
  static constexpr int KTILE = DMA ? PaddedDma<BN, ROWB, KS>::NBLK * 1024 : BN * KS;
  static constexpr int VTILE = DMA ? PaddedDma<BN, ROWB, VS>::NBLK * 1024 : BN * VS;
  static constexpr int STAGE = KTILE + VTILE;  // K then V
  static constexpr int CPR = ROWB / 16;              // 16-byte pieces per row
  static constexpr int CPT = BN * CPR / THREADS;     // pieces per thread per tile
  static constexpr int BIAS_OFF = 2 * STAGE;
  static constexpr int LDS = BIAS_OFF + 1040;
  static_assert((BN * CPR) % THREADS == 0, "tile pieces divide the workgroup");
  // the two-group shapes take this kernel only for the padded-dense baseline,
  // which plans with 128-row tiles
  static_assert(FwdPingPong<T, D>::value || FwdRows64<T, D>::value || BM == FwdRows<T, D>::value,
                "tile shape published to the planner");
};

// PADDED: the padded-dense baseline. Every sequence occupies a fixed-length
// slot of a dense [B, L, H, D] tensor (uniform offsets), every block of the
// slot is visited, and keys at or past the sequence's true length
// (a.kv_len[b]) are masked with -inf on every block, element by element, as a
// conventional kernel over padded tensors does.

template <typename T, int D> constexpr int fwd_min_waves() {
  return D * sizeof(T) >= 512 ? 1 : D * sizeof(T) >= 256 ? JFA_FWD_WIDE_BLOCKS : JFA_FWD_BLOCKS;
}

template <typename T, int D, bool BIAS, bool PADDED = false>
__global__ __launch_bounds__(256, (fwd_min_waves<T, D>())) void jfa_fwd_kernel(FwdArgs a) {
  using C = FwdTiles<T, D>;
  constexpr int BM = C::BM, BN = C::BN, ES = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave branches stay scalar
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * C::ROWB;  // bytes between consecutive tokens
  // First, the short-query sequences: their chunks (previous launch) are
  // combined into O and lse.
  static_assert(kShortLds <= C::LDS, "combining step fits the LDS");
  for_short_groups(a.gfirst, a.B * H, lds, [&](int gi) { fsq_merge<T, D>(a, gi, lds); });
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
    // keys at or past Lmask are dropped by the element mask of masked blocks
    const int Lmask = PADDED ? min(max(a.kv_len[b], 0), Lk) : Lk;

    const size_t qrow = ((size_t)q0 * H + h) * C::ROWB, krow = ((size_t)k0 * H + h) * C::ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, C::ROWB);
    const View kv = seq_view((const char*)a.k + krow, Lk, gstride, C::ROWB);
    const View vv = seq_view((const char*)a.v + krow, Lk, gstride, C::ROWB);

    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += C::THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }

    const int wr0 = row0 + 32 * w;  // first query row of this wave
    const bool wave_on = wr0 < Lq;
    const int qi = wr0 + l32;       // this lane's query row
    Frag<T> qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = gfrag(qv, (uint32_t)qi * gstride + (16 * kk + 8 * g) * ES, (T*)0);

    i32x4 kr[C::DMA ? 1 : C::CPT], vr[C::DMA ? 1 : C::CPT];
    const DmaView kd = dma_view((const char*)a.k + krow, Lk, gstride, C::ROWB);
    const DmaView vd = dma_view((const char*)a.v + krow, Lk, gstride, C::ROWB);
    auto gload = [&](int j) {
      if constexpr (C::DMA) {  // block j straight into stage j & 1
        lds_t* st = lds + (j & 1) * C::STAGE;
        dma_padded_tile<BN, C::ROWB, C::KS, 4>(kd, gstride, j * BN, st, w, lane);
        dma_padded_tile<BN, C::ROWB, C::VS, 4>(vd, gstride, j * BN, st + C::KTILE, w, lane);
        return;
      }
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        const uint32_t off = (uint32_t)(j * BN + row) * gstride + col * 16;
        kr[c] = ld16(kv, off);
        vr[c] = ld16(vv, off);
      }
    };
    auto swrite = [&](int s) {
      if constexpr (C::DMA) {  // the direct loads of this stage have landed
        wait_vmem();
        return;
      }
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        *(__attribute__((address_space(3))) i32x4*)(lds + s * C::STAGE + row * C::KS + col * 16) = kr[c];
        *(__attribute__((address_space(3))) i32x4*)(lds + s * C::STAGE + C::KTILE + row * C::VS + col * 16) = vr[c];
      }
    };
    if (n_kv > 0) {
      gload(0);
      swrite(0);
    }
    wait_vmem();
    __syncthreads();

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = (f32x16){};
    // Two running sums per half-wave: l over the fp32 P (for lse) and lb over
    // the bf16-rounded P the PV product consumes (O is normalised by it, so
    // the weights applied to V sum to 1; a row with one key gets O = V
    // exactly, which keeps the backward's Delta = dO . O consistent with dP).
    constexpr bool kOpSum = sizeof(T) == 2;
    float m = kNegInit, l = 0.f, lb = 0.f;
    float l_pre = 0.f, lb_pre = 0.f;  // sums before the item's last block (cancellation guard)
    int last_tile = -1;
    bool last_masked = false;

    for (int j = 0; j < n_kv; ++j) {
      const int s = j & 1;
      if (j + 1 < n_kv) gload(j + 1);
      const int key0 = j * BN;
      const bool active = wave_on && (!a.causal || key0 <= wr0 + 31);
      if (active) {
        const bool masked = PADDED || (a.causal && (key0 + BN - 1 > wr0)) || kFwdMaskMode == 2 ||
                            (kFwdMaskMode == 1 && key0 + BN > Lk);
        // with the subtraction, masked blocks are causal ones
        const bool cmask = PADDED ? a.causal != 0 : (kFwdMaskMode == 0 || a.causal);
        last_tile = j;
        last_masked = masked;
        const lds_t* kt = lds + s * C::STAGE;
        const lds_t* vt = kt + C::KTILE;
        f32x16 sc[BN / 32];
        prio_mfma();
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
          sc[kb] = (f32x16){};
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk)
            mma(sc[kb], prfrag<C::KS>(kt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0), qf[kk]);
        }
        if constexpr (JFA_FWD_PREFETCH > 0 && sizeof(T) == 2 && C::ROWB >= 256) sched_prefetch<(BN / 32) * (D / 16), 1, JFA_FWD_PREFETCH>();
        prio_valu();
        // Scores in log2 units: x = s * scale * log2(e) (+ bias * log2(e)).
        float mx = -INFINITY;
        const bool plain = !BIAS && !masked;
        if (plain) {
          // max on the raw dot products; the scale is folded into the exp below
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
          mx = half_max(mx) * a.scale2;
        } else {
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kj = key0 + 32 * kb + res_row(i, g);
              float x = sc[kb][i] * a.scale2;
              if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
              if (masked && ((cmask && kj > qi) || kj >= Lmask)) x = -INFINITY;
              sc[kb][i] = x;
              mx = fmaxf(mx, x);
            }
          }
          mx = half_max(mx);
        }
        // Running max with slack: m only moves when the block max exceeds it
        // by more than kRescaleSlack, so P <= 2^kRescaleSlack and O, l are
        // rescaled only on those (rare) blocks. l and O share m, so the final
        // O / l and lse = m + log2(l) are unchanged.
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
        if (j + 1 == n_kv) {
          l_pre = l;
          lb_pre = lb;
        }
        if (plain) {
          const float nm = -m;
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i], a.scale2, nm));
              sc[kb][i] = p;
              l += p;
            }
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = __builtin_amdgcn_exp2f(sc[kb][i] - m);
              sc[kb][i] = p;
              l += p;
            }
          }
        }
        prio_mfma();
#pragma unroll
        for (int kc = 0; kc < BN / 16; ++kc) {
          const Frag<T> pf = rfrag(sc[kc >> 1], kc & 1, (T*)0);
          if constexpr (kOpSum) lb = frag_sum(pf, lb);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) mma(o[db], ptfrag<C::VS>(vt, 16 * kc, 32 * db, lane, (T*)0), pf);
        }
        if constexpr (JFA_FWD_PREFETCH > 0 && sizeof(T) == 2 && C::ROWB >= 256) sched_prefetch<(BN / 16) * (D / 32), 2, JFA_FWD_PREFETCH>();
        prio_valu();
      }
      if (j + 1 < n_kv) swrite((j + 1) & 1);
      __syncthreads();
    }

    // Epilogue: combine the two half-wave partial sums, remove the pad terms
    // (from both sums, each as it was added: the bf16 sum took them rounded).
    float lt = l + other_half(l);
    float lbt = kOpSum ? lb + other_half(lb) : lt;
    if (wave_on && last_tile >= 0 && !last_masked) {
      const int pad1 = (last_tile + 1) * BN;
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
        // Cancellation guard: the subtraction is exact in real arithmetic, but
        // in fp32 it loses the valid terms when they are tiny next to the pad
        // terms (every valid score far below the pad keys' score, which is the
        // bias, or 0). A row whose remainder keeps fewer than ~12 significant
        // bits gets its last block's valid terms summed again from the K tile
        // still in LDS, without the pad keys, on top of the sum before that
        // block. Not taken for unit-scale scores.
        const bool cancel = !(lt > full * 0x1p-12f);
        if (__any(cancel)) {
          const lds_t* kt = lds + (last_tile & 1) * C::STAGE;
          const int key0 = last_tile * BN;
          // Plain dot products, one key row of the tile at a time (rare path:
          // kept small so that it adds nothing to the kernel's registers).
          float sv = 0.f, svb = 0.f;
#pragma unroll 1
          for (int r = g; r < BN; r += 2) {
            const int kj = key0 + r;
            if (kj >= Lk) break;  // keys past the end follow the valid ones
            float dot = 0.f;
#pragma unroll 1
            for (int c = 0; c < C::CPR; ++c) {
              const i32x4 kq = *(const __attribute__((address_space(3))) i32x4*)(kt + r * C::KS + c * 16);
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
    if (wave_on) {
      const float inv = lbt > 0.f ? 1.0f / lbt : 0.f;
      const View ov = seq_view((char*)a.out + qrow, Lq, gstride, C::ROWB);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          store4(ov, (uint32_t)qi * gstride + d * ES, o[db][4 * r] * inv, o[db][4 * r + 1] * inv,
                 o[db][4 * r + 2] * inv, o[db][4 * r + 3] * inv, (T*)0);
        }
      }
      if (g == 0) {
        const float lse = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
        const View lv = seq_view(a.lse + (size_t)q0 * H + h, Lq, (uint32_t)H * 4, 4);
        st4f(lv, (uint32_t)qi * H * 4, lse);
      }
    }
    if constexpr (!kSchedPersistent) break;  // one item per workgroup
  }
}

// Study kernel (JFA_FWD_PINGPONG for bf16 D = 128, JFA_FWD_PINGPONG_NARROW
// for D = 64): a two-group forward. Eight waves and 256 query rows per item:
// waves 0-3 (group 0) and 4-7 (group 1) own 32 rows each, and the two waves
// that share a SIMD sit in different groups. The work of a key block is cut
// into a matrix phase (the PV product of the block before, then QK^T of this
// block) and a vector phase (the online softmax of this block), and the two
// groups run them half a block apart, with a workgroup barrier between
// phases, so that while one group's waves issue MFMAs the other's run the
// softmax. The arithmetic per row is that of jfa_fwd_kernel, in the same
// order. Measured slower than jfa_fwd_kernel: in a vector phase one wave per
// SIMD issues VALU alone, which reaches about two thirds of the port's rate,
// and in a matrix phase one group's LDS operand reads all queue at once.
//
// Step s (s = 0 .. n_kv) works on K block s and V block s-1, one LDS stage:
//   phase 2s  : group 0 matrix (PV s-1, QK^T s), group 1 vector (softmax s-1)
//   phase 2s+1: group 0 vector (softmax s),      group 1 matrix (PV s-1, QK^T s)
// Step s+1's tiles are requested by direct loads into the other stage at the
// start of step s and waited for at its end.
template <int D, bool BIAS>
__global__ __launch_bounds__(512, 1) void jfa_fwd_pp_kernel(FwdArgs a) {
  using T = bf16;
  static_assert(kFwdMaskMode == 0, "the two-group kernel subtracts the pad terms");
  constexpr int THREADS = 512, BM = 256, BN = 64, ES = 2;
  constexpr int ROWB = Tile<T, D>::ROWB, KS = pad_nat(ROWB), VS = pad_tr(ROWB);
  constexpr int KTILE = PaddedDma<BN, ROWB, KS>::NBLK * 1024, STAGE = KTILE + PaddedDma<BN, ROWB, VS>::NBLK * 1024;
  constexpr int CPR = ROWB / 16;  // 16-byte pieces per row
  constexpr int BIAS_OFF = 2 * STAGE, LDS = BIAS_OFF + 1040;
  static_assert(BM == FwdRows<T, D>::value && BN == FwdKeys<T, D>::value, "tile shape published to the planner");
  static_assert(kShortLds <= LDS, "combining step fits the LDS");
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + BIAS_OFF);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp0 = w < 4;
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * ROWB;
  for_short_groups(a.gfirst, a.B * H, lds, [&](int gi) { fsq_merge<T, D, THREADS>(a, gi, lds); });
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

    const size_t qrow = ((size_t)q0 * H + h) * ROWB, krow = ((size_t)k0 * H + h) * ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, ROWB);
    const View kv = seq_view((const char*)a.k + krow, Lk, gstride, ROWB);
    const View vv = seq_view((const char*)a.v + krow, Lk, gstride, ROWB);
    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }

    const int wr0 = row0 + 32 * w;  // first query row of this wave
    const bool wave_on = wr0 < Lq;
    const int qi = wr0 + l32;
    Frag<T> qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = gfrag(qv, (uint32_t)qi * gstride + (16 * kk + 8 * g) * ES, (T*)0);

    // Step s stages K block s (s < n_kv) and V block s-1 (s >= 1) in LDS
    // stage s & 1, by direct loads (no staging registers); s is uniform.
    // Rows past the sequence's end and the row padding read as zeros.
    const DmaView kd = dma_view((const char*)a.k + krow, Lk, gstride, ROWB);
    const DmaView vd = dma_view((const char*)a.v + krow, Lk, gstride, ROWB);
    auto load_step = [&](int s) {
      lds_t* st = lds + (s & 1) * STAGE;
      // the lane id read afresh, so that the per-lane offsets are recomputed
      // on each step (a few VALU ops) rather than held in registers
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      if (s < n_kv) dma_padded_tile<BN, ROWB, KS, 8>(kd, gstride, s * BN, st, w, ln);
      if (s >= 1) dma_padded_tile<BN, ROWB, VS, 8>(vd, gstride, (s - 1) * BN, st + KTILE, w, ln);
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = (f32x16){};
    f32x16 sc[BN / 32];  // S^T of a block, then its P until the next matrix phase
    // l: sum of the fp32 P (for lse); lb: sum of the bf16-rounded P the PV
    // product consumes (O is normalised by it), added when PV rounds them
    float m = kNegInit, l = 0.f, lb = 0.f;
    float l_pre = 0.f, lb_pre = 0.f;  // sums before the item's last block (cancellation guard)
    int last_tile = -1;
    bool last_masked = false;
    // this wave's rows see block j (j < n_kv)
    auto active = [&](int j) { return wave_on && (!a.causal || j * BN <= wr0 + 31); };

    auto pv = [&](int s) {  // PV of block s-1 (its P in sc), V tile of step s
      const lds_t* vt = lds + (s & 1) * STAGE + KTILE;
#pragma unroll
      for (int kc = 0; kc < BN / 16; ++kc) {
        const Frag<T> pf = rfrag(sc[kc >> 1], kc & 1, (T*)0);
        lb = frag_sum(pf, lb);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) mma(o[db], ptfrag<VS>(vt, 16 * kc, 32 * db, lane, (T*)0), pf);
      }
      sched_prefetch<(BN / 16) * (D / 32), 2, JFA_FWD_PP_AHEAD>();  // operands AHEAD products ahead, no more
    };
    auto qk = [&](int s) {  // S^T of block s, K tile of step s
      const lds_t* kt = lds + (s & 1) * STAGE;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        sc[kb] = (f32x16){};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          mma(sc[kb], prfrag<KS>(kt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0), qf[kk]);
      }
      sched_prefetch<(BN / 32) * (D / 16), 1, JFA_FWD_PP_AHEAD>();
    };
    // matrix phase of step s (1 <= s < n_kv)
    auto matrix = [&](int s) {
      if (active(s - 1)) pv(s);
      if (active(s)) qk(s);
    };

    auto vector = [&](int j) {
      if (!active(j)) return;
      const int key0 = j * BN;
      const bool masked = a.causal && (key0 + BN - 1 > wr0);  // with the subtraction, masked blocks are causal ones
      last_tile = j;
      last_masked = masked;
      float mx = -INFINITY;
      const bool plain = !BIAS && !masked;
      if (plain) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
        mx = half_max(mx) * a.scale2;
      } else {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kj = key0 + 32 * kb + res_row(i, g);
            float x = sc[kb][i] * a.scale2;
            if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
            if (masked && (kj > qi || kj >= Lk)) x = -INFINITY;  // a masked block also drops its pad keys
            sc[kb][i] = x;
            mx = fmaxf(mx, x);
          }
        }
        mx = half_max(mx);
      }
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
      if (j + 1 == n_kv) {
        l_pre = l;
        lb_pre = lb;
      }
      if (plain) {
        const float nm = -m;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i], a.scale2, nm));
            sc[kb][i] = p;
            l += p;
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[kb][i] - m);
            sc[kb][i] = p;
            l += p;
          }
        }
      }
    };

    // Steps 0 .. n_kv in 2 n_kv + 2 phases; step 0 (QK^T of block 0) and
    // step n_kv (PV of the last block) are written out, steps 1 .. n_kv - 1
    // are the loop. Loads of step s + 1 go out at the start of step s and
    // land in LDS at its end. One loop per group, each a straight sequence
    // of its two phases; both pass the same barriers.
    if (n_kv > 0) load_step(0);
    wait_vmem();
    __syncthreads();
    if (n_kv > 0) {
      // step 0
      load_step(1);
      if (grp0 && active(0)) qk(0);
      __syncthreads();
      if (grp0) vector(0);
      else if (active(0)) qk(0);
      wait_vmem();
      __syncthreads();
      // steps 1 .. n_kv - 1
      if (grp0) {
        for (int s = 1; s < n_kv; ++s) {
          load_step(s + 1);
          matrix(s);
          __syncthreads();
          vector(s);
          wait_vmem();
          __syncthreads();
        }
      } else {
        for (int s = 1; s < n_kv; ++s) {
          load_step(s + 1);
          vector(s - 1);
          __syncthreads();
          matrix(s);
          wait_vmem();
          __syncthreads();
        }
      }
      // step n_kv: PV of the last block
      if (grp0) {
        if (active(n_kv - 1)) pv(n_kv);
      } else {
        vector(n_kv - 1);
      }
      __syncthreads();
      if (!grp0 && active(n_kv - 1)) pv(n_kv);
    }

    // Epilogue as in jfa_fwd_kernel. The last block of a row that still needs
    // the pad terms removed is never a causal (masked) block, so it is block
    // n_kv - 1, whose K tile (stage (n_kv - 1) & 1) no later step overwrote.
    float lt = l + other_half(l);
    float lbt = lb + other_half(lb);
    if (wave_on && last_tile >= 0 && !last_masked) {
      const int pad1 = (last_tile + 1) * BN;
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
        // cancellation guard (see jfa_fwd_kernel)
        const bool cancel = !(lt > full * 0x1p-12f);
        if (__any(cancel)) {
          const lds_t* kt = lds + (last_tile & 1) * STAGE;
          const int key0 = last_tile * BN;
          float sv = 0.f, svb = 0.f;
#pragma unroll 1
          for (int r = g; r < BN; r += 2) {
            const int kj = key0 + r;
            if (kj >= Lk) break;
            float dot = 0.f;
#pragma unroll 1
            for (int c = 0; c < CPR; ++c) {
              const i32x4 kq = *(const __attribute__((address_space(3))) i32x4*)(kt + r * KS + c * 16);
              const i32x4 qq = ld16(qv, (uint32_t)qi * gstride + c * 16);
              const bf16x8 k8 = __builtin_bit_cast(bf16x8, kq), q8 = __builtin_bit_cast(bf16x8, qq);
#pragma unroll
              for (int e = 0; e < 8; ++e) dot += (float)k8[e] * (float)q8[e];
            }
            float x = dot * a.scale2;
            if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
            const float pe = __builtin_amdgcn_exp2f(x - m);
            sv += pe;
            svb += as_operand(pe, (T*)0);
          }
          const float fixed = l_pre + other_half(l_pre) + sv + other_half(sv);
          const float fixedb = lb_pre + other_half(lb_pre) + svb + other_half(svb);
          if (cancel) {
            lt = fixed;
            lbt = fixedb;
          }
        }
      }
    }
    if (wave_on) {
      const float inv = lbt > 0.f ? 1.0f / lbt : 0.f;
      const View ov = seq_view((char*)a.out + qrow, Lq, gstride, ROWB);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * g;
          store4(ov, (uint32_t)qi * gstride + d * ES, o[db][4 * r] * inv, o[db][4 * r + 1] * inv,
                 o[db][4 * r + 2] * inv, o[db][4 * r + 3] * inv, (T*)0);
        }
      }
      if (g == 0) {
        const float lse = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
        const View lv = seq_view(a.lse + (size_t)q0 * H + h, Lq, (uint32_t)H * 4, 4);
        st4f(lv, (uint32_t)qi * H * 4, lse);
      }
    }
    if constexpr (!kSchedPersistent) break;  // one item per workgroup
  }
}

// Study kernel: 64 query rows per wave, as two 32-row halves, for bf16 rows
// of up to 128 bytes. Four waves, 256 rows per item; the K/V ring, the
// per-row arithmetic and its order are those of jfa_fwd_kernel, but every K
// and V fragment read from LDS feeds the MFMAs of both halves (half the LDS
// reads per product), at the price of twice the accumulators per wave:
// 228-256 VGPRs, two waves per SIMD, measured slower than jfa_fwd_kernel.
template <int D, bool BIAS>
__global__ __launch_bounds__(256, 2) void jfa_fwd_r64_kernel(FwdArgs a) {
  using T = bf16;
  using C = FwdTiles<T, D>;
  static_assert(kFwdMaskMode == 0 && D <= 64, "study kernel: subtraction of pad terms, rows of up to 128 bytes");
  constexpr int NH = 2, BM = 256, BN = C::BN, ES = 2;
  static_assert(BM == FwdRows<T, D>::value, "tile shape published to the planner");
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * C::ROWB;
  for_short_groups(a.gfirst, a.B * H, lds, [&](int gi) { fsq_merge<T, D>(a, gi, lds); });
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
    const size_t qrow = ((size_t)q0 * H + h) * C::ROWB, krow = ((size_t)k0 * H + h) * C::ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, C::ROWB);
    const View kv = seq_view((const char*)a.k + krow, Lk, gstride, C::ROWB);
    const View vv = seq_view((const char*)a.v + krow, Lk, gstride, C::ROWB);
    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += C::THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }

    const int wr0 = row0 + 64 * w;  // half hh holds rows wr0 + 32 hh .. + 31
    Frag<T> qf[NH][D / 16];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qf[hh][kk] = gfrag(qv, (uint32_t)(wr0 + 32 * hh + l32) * gstride + (16 * kk + 8 * g) * ES, (T*)0);

    i32x4 kr[C::CPT], vr[C::CPT];
    auto gload = [&](int j) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        const uint32_t off = (uint32_t)(j * BN + row) * gstride + col * 16;
        kr[c] = ld16(kv, off);
        vr[c] = ld16(vv, off);
      }
    };
    auto swrite = [&](int s) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        *(__attribute__((address_space(3))) i32x4*)(lds + s * C::STAGE + row * C::KS + col * 16) = kr[c];
        *(__attribute__((address_space(3))) i32x4*)(lds + s * C::STAGE + C::KTILE + row * C::VS + col * 16) = vr[c];
      }
    };
    if (n_kv > 0) {
      gload(0);
      swrite(0);
    }
    wait_vmem();
    __syncthreads();

    f32x16 o[NH][D / 32];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[hh][db] = (f32x16){};
    float m[NH], l[NH], lb[NH], l_pre[NH], lb_pre[NH];
    int last_tile[NH];
    bool last_masked[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      m[hh] = kNegInit;
      l[hh] = lb[hh] = l_pre[hh] = lb_pre[hh] = 0.f;
      last_tile[hh] = -1;
      last_masked[hh] = false;
    }

    for (int j = 0; j < n_kv; ++j) {
      const int s = j & 1;
      if (j + 1 < n_kv) gload(j + 1);
      const int key0 = j * BN;
      bool act[NH];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) act[hh] = wr0 + 32 * hh < Lq && (!a.causal || key0 <= wr0 + 32 * hh + 31);
      if (act[0] || act[1]) {
        const lds_t* kt = lds + s * C::STAGE;
        const lds_t* vt = kt + C::KTILE;
        f32x16 sc[NH][BN / 32];
        prio_mfma();
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) sc[hh][kb] = (f32x16){};
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            const Frag<T> kf = prfrag<C::KS>(kt, 32 * kb + l32, 16 * kk + 8 * g, (T*)0);
            mma(sc[0][kb], kf, qf[0][kk]);
            if (act[1]) mma(sc[1][kb], kf, qf[1][kk]);
          }
        }
        prio_valu();
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          if (!act[hh]) continue;
          const int hr0 = wr0 + 32 * hh, qi = hr0 + l32;
          const bool masked = a.causal && (key0 + BN - 1 > hr0);
          last_tile[hh] = j;
          last_masked[hh] = masked;
          float mx = -INFINITY;
          const bool plain = !BIAS && !masked;
          if (plain) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[hh][kb][i]);
            mx = half_max(mx) * a.scale2;
          } else {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int kj = key0 + 32 * kb + res_row(i, g);
                float x = sc[hh][kb][i] * a.scale2;
                if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
                if (masked && (kj > qi || kj >= Lk)) x = -INFINITY;
                sc[hh][kb][i] = x;
                mx = fmaxf(mx, x);
              }
            }
            mx = half_max(mx);
          }
          const bool grow = mx > m[hh] + kRescaleSlack;
          if (__any(grow)) {
            const float mn = grow ? mx : m[hh];
            const float alpha = __builtin_amdgcn_exp2f(m[hh] - mn);
            m[hh] = mn;
            l[hh] *= alpha;
            lb[hh] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[hh][db] *= alpha;
          }
          if (j + 1 == n_kv) {
            l_pre[hh] = l[hh];
            lb_pre[hh] = lb[hh];
          }
          const float nm = -m[hh];
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = plain ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hh][kb][i], a.scale2, nm))
                                    : __builtin_amdgcn_exp2f(sc[hh][kb][i] - m[hh]);
              sc[hh][kb][i] = p;
              l[hh] += p;
            }
          }
        }
        prio_mfma();
#pragma unroll
        for (int kc = 0; kc < BN / 16; ++kc) {
          const Frag<T> p0 = rfrag(sc[0][kc >> 1], kc & 1, (T*)0);
          const Frag<T> p1 = rfrag(sc[1][kc >> 1], kc & 1, (T*)0);
          if (act[0]) lb[0] = frag_sum(p0, lb[0]);
          if (act[1]) lb[1] = frag_sum(p1, lb[1]);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const Frag<T> vf = ptfrag<C::VS>(vt, 16 * kc, 32 * db, lane, (T*)0);
            if (act[0]) mma(o[0][db], vf, p0);
            if (act[1]) mma(o[1][db], vf, p1);
          }
        }
        prio_valu();
      }
      if (j + 1 < n_kv) swrite((j + 1) & 1);
      __syncthreads();
    }

    // epilogue per half, as in jfa_fwd_kernel (the cancellation guard reads
    // K of block last_tile, still in LDS: a row's last unmasked block is the
    // item's last block)
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const int hr0 = wr0 + 32 * hh, qi = hr0 + l32;
      const bool half_on = hr0 < Lq;
      float lt = l[hh] + other_half(l[hh]);
      float lbt = lb[hh] + other_half(lb[hh]);
      if (half_on && last_tile[hh] >= 0 && !last_masked[hh]) {
        const int pad1 = (last_tile[hh] + 1) * BN;
        if (pad1 > Lk) {
          float pads, pads_b;
          if (!BIAS) {
            const float pe = __builtin_amdgcn_exp2f(-m[hh]);
            pads = (float)(pad1 - Lk) * pe;
            pads_b = (float)(pad1 - Lk) * as_operand(pe, (T*)0);
          } else {
            float sub = 0.f, subb = 0.f;
            for (int kj = Lk + g; kj < pad1; kj += 2) {
              const float pe =
                  __builtin_amdgcn_exp2f(bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius] - m[hh]);
              sub += pe;
              subb += as_operand(pe, (T*)0);
            }
            pads = sub + other_half(sub);
            pads_b = subb + other_half(subb);
          }
          const float full = lt;
          lt -= pads;
          lbt -= pads_b;
          const bool cancel = !(lt > full * 0x1p-12f);
          if (__any(cancel)) {
            const lds_t* kt = lds + (last_tile[hh] & 1) * C::STAGE;
            const int key0 = last_tile[hh] * BN;
            float sv = 0.f, svb = 0.f;
#pragma unroll 1
            for (int r = g; r < BN; r += 2) {
              const int kj = key0 + r;
              if (kj >= Lk) break;
              float dot = 0.f;
#pragma unroll 1
              for (int c = 0; c < C::CPR; ++c) {
                const i32x4 kq = *(const __attribute__((address_space(3))) i32x4*)(kt + r * C::KS + c * 16);
                const i32x4 qq = ld16(qv, (uint32_t)qi * gstride + c * 16);
                const bf16x8 k8 = __builtin_bit_cast(bf16x8, kq), q8 = __builtin_bit_cast(bf16x8, qq);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot += (float)k8[e] * (float)q8[e];
              }
              float x = dot * a.scale2;
              if (BIAS) x += bias_lds[min(max(qi - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
              const float pe = __builtin_amdgcn_exp2f(x - m[hh]);
              sv += pe;
              svb += as_operand(pe, (T*)0);
            }
            const float fixed = l_pre[hh] + other_half(l_pre[hh]) + sv + other_half(sv);
            const float fixedb = lb_pre[hh] + other_half(lb_pre[hh]) + svb + other_half(svb);
            if (cancel) {
              lt = fixed;
              lbt = fixedb;
            }
          }
        }
      }
      if (half_on) {
        const float inv = lbt > 0.f ? 1.0f / lbt : 0.f;
        const View ov = seq_view((char*)a.out + qrow, Lq, gstride, C::ROWB);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = 32 * db + 8 * r + 4 * g;
            store4(ov, (uint32_t)qi * gstride + d * ES, o[hh][db][4 * r] * inv, o[hh][db][4 * r + 1] * inv,
                   o[hh][db][4 * r + 2] * inv, o[hh][db][4 * r + 3] * inv, (T*)0);
          }
        }
        if (g == 0) {
          const float lse = lt > 0.f ? (m[hh] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
          const View lv = seq_view(a.lse + (size_t)q0 * H + h, Lq, (uint32_t)H * 4, 4);
          st4f(lv, (uint32_t)qi * H * 4, lse);
        }
      }
    }
    if constexpr (!kSchedPersistent) break;
  }
}

// Study kernel (JFA_FWD_MFMA16, bf16 D <= 64): the forward with
// v_mfma_f32_16x16x32_bf16 products in place of 32x32x16. The items (128
// query rows), the 64-key blocks and the register-staged two-stage ring are
// the library's; each wave holds its 32 query rows as two 16-column tiles,
// and per block
//   S^T = K Q^T     4 key tiles x 2 query tiles, D/32 products of 16 cycles
//                   each (K rows read naturally from LDS, Q in VGPRs)
//   softmax         lane l holds keys 4(l/16)..+3 of every key tile for query
//                   column l%16: 16 scores per lane and query tile; the four
//                   16-lane rows are combined with a permlane16 and a
//                   permlane32 swap
//   O^T += V^T P^T  D/16 x 2 tiles, two 32-key products each; the P^T operand
//                   comes straight from the score registers (its 8 k-slots are
//                   keys 4r..4r+3 of two consecutive key tiles), V^T from
//                   transposing reads in the same key order, over V rows
//                   padded to an odd multiple of 32 bytes (8 consecutive rows
//                   x 32 bytes per cycle without bank conflicts)
#ifndef JFA_FWD_MFMA16
#define JFA_FWD_MFMA16 0
#endif
// its launch bound: 3 workgroups per CU (at most 168 VGPRs: three waves per SIMD)
#ifndef JFA_FWD_MFMA16_BLOCKS
#define JFA_FWD_MFMA16_BLOCKS 3
#endif
template <typename T, int D> struct FwdMfma16 {
  static constexpr bool value = JFA_FWD_MFMA16 != 0 && sizeof(T) == 2 && D <= 64;
};

constexpr int pad_tr16(int rowb) { return (rowb / 32) % 2 == 1 ? rowb : rowb + 32; }

template <int D>
struct FwdTiles16 {
  static constexpr int BM = 128, BN = 64, THREADS = 256, ROWB = D * 2;
  static constexpr int KS = pad_nat(ROWB), VS = pad_tr16(ROWB);
  static constexpr int KTILE = BN * KS, VTILE = BN * VS, STAGE = KTILE + VTILE;
  static constexpr int CPR = ROWB / 16, CPT = BN * CPR / THREADS;
  static constexpr int BIAS_OFF = 2 * STAGE;
  static constexpr int LDS = BIAS_OFF + 1040;
  static_assert((BN * CPR) % THREADS == 0, "tile pieces divide the workgroup");
};

__device__ __forceinline__ void mma16(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Combined over the four 16-lane rows of the wave (every lane gets the result).
__device__ __forceinline__ float quarter_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return half_max(fmaxf(__int_as_float(r[0]), __int_as_float(r[1])));
}
__device__ __forceinline__ float quarter_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  const float y = __int_as_float(r[0]) + __int_as_float(r[1]);
  return y + other_half(y);
}
// V^T operand of a 16x16x32 product: lane l holds column d = dbase + l%16 of
// key rows kbase + 4(l/16) + 0..3 (k-slots 0..3) and kbase + 16 + 4(l/16) +
// 0..3 (k-slots 4..7) of a padded-row tile: two transposing reads, each
// 16-lane row of the wave reading a 4-row x 16-column block.
template <int S>
__device__ __forceinline__ bf16x8 ptfrag16(const lds_t* tile, int kbase, int dbase, int lane) {
  const int row = kbase + 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int b = (dbase + (lane & 3) * 4) * 2;
  s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + row * S + b));
  s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + (row + 16) * S + b));
  const bf16x4 x4 = __builtin_bit_cast(bf16x4, x), y4 = __builtin_bit_cast(bf16x4, y);
  return (bf16x8){x4[0], x4[1], x4[2], x4[3], y4[0], y4[1], y4[2], y4[3]};
}

template <int D, bool BIAS>
__global__ __launch_bounds__(256, JFA_FWD_MFMA16_BLOCKS) void jfa_fwd_m16_kernel(FwdArgs a) {
  using T = bf16;
  using C = FwdTiles16<D>;
  constexpr int BM = C::BM, BN = C::BN, ES = 2;
  static_assert(BM == FwdRows<T, D>::value, "tile shape published to the planner");
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ QueueCursor qcur;
  lds_t* lds = (lds_t*)smem;
  __attribute__((address_space(3))) float* bias_lds = (__attribute__((address_space(3))) float*)(lds + C::BIAS_OFF);

  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H;
  const uint32_t gstride = (uint32_t)H * C::ROWB;
  static_assert(kShortLds <= C::LDS, "combining step fits the LDS");
  for_short_groups(a.gfirst, a.B * H, lds, [&](int gi) { fsq_merge<T, D>(a, gi, lds); });
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
    const size_t qrow = ((size_t)q0 * H + h) * C::ROWB, krow = ((size_t)k0 * H + h) * C::ROWB;
    const View qv = seq_view((const char*)a.q + qrow, Lq, gstride, C::ROWB);
    const View kv = seq_view((const char*)a.k + krow, Lk, gstride, C::ROWB);
    const View vv = seq_view((const char*)a.v + krow, Lk, gstride, C::ROWB);
    if (BIAS) {
      for (int i = tid; i < kBiasLen; i += C::THREADS) bias_lds[i] = a.bias[h * kBiasLen + i] * kLog2e;
    }

    const int wr0 = row0 + 32 * w;  // first query row of this wave
    const bool wave_on = wr0 < Lq;
    int qi[2];                      // this lane's query row in each 16-row tile
    bf16x8 qf[2][D / 32];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      qi[t] = wr0 + 16 * t + l16;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        qf[t][kk] = gfrag(qv, (uint32_t)qi[t] * gstride + (32 * kk + 8 * g4) * ES, (T*)0).v;
    }

    i32x4 kr[C::CPT], vr[C::CPT];
    auto gload = [&](int j) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        const uint32_t off = (uint32_t)(j * BN + row) * gstride + col * 16;
        kr[c] = ld16(kv, off);
        vr[c] = ld16(vv, off);
      }
    };
    auto swrite = [&](int s) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int x = tid + C::THREADS * c, row = x / C::CPR, col = x % C::CPR;
        *(__attribute__((address_space(3))) i32x4*)(lds + s * C::STAGE + row * C::KS + col * 16) = kr[c];
        *(__attribute__((address_space(3))) i32x4*)(lds + s * C::STAGE + C::KTILE + row * C::VS + col * 16) = vr[c];
      }
    };
    if (n_kv > 0) {
      gload(0);
      swrite(0);
    }
    wait_vmem();
    __syncthreads();

    f32x4 o[D / 16][2];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int t = 0; t < 2; ++t) o[dt][t] = (f32x4){};
    float m[2] = {kNegInit, kNegInit}, l[2] = {0.f, 0.f}, lb[2] = {0.f, 0.f};
    float l_pre[2] = {0.f, 0.f}, lb_pre[2] = {0.f, 0.f};
    int last_tile = -1;
    bool last_masked = false;

    for (int j = 0; j < n_kv; ++j) {
      const int s = j & 1;
      if (j + 1 < n_kv) gload(j + 1);
      const int key0 = j * BN;
      const bool active = wave_on && (!a.causal || key0 <= wr0 + 31);
      if (active) {
        const bool masked = (a.causal && (key0 + BN - 1 > wr0)) || kFwdMaskMode == 2 ||
                            (kFwdMaskMode == 1 && key0 + BN > Lk);
        const bool cmask = kFwdMaskMode == 0 || a.causal;
        last_tile = j;
        last_masked = masked;
        const lds_t* kt = lds + s * C::STAGE;
        const lds_t* vt = kt + C::KTILE;
        f32x4 sc[BN / 16][2];
        prio_mfma();
#pragma unroll
        for (int ktile = 0; ktile < BN / 16; ++ktile) {
#pragma unroll
          for (int t = 0; t < 2; ++t) sc[ktile][t] = (f32x4){};
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) {
            const bf16x8 kf = prfrag<C::KS>(kt, 16 * ktile + l16, 32 * kk + 8 * g4, (T*)0).v;
#pragma unroll
            for (int t = 0; t < 2; ++t) mma16(sc[ktile][t], kf, qf[t][kk]);
          }
        }
        prio_valu();
        const bool plain = !BIAS && !masked;
        float mx[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float x_max = -INFINITY;
          if (plain) {
#pragma unroll
            for (int ktile = 0; ktile < BN / 16; ++ktile)
#pragma unroll
              for (int i = 0; i < 4; ++i) x_max = fmaxf(x_max, sc[ktile][t][i]);
            mx[t] = quarter_max(x_max) * a.scale2;
          } else {
#pragma unroll
            for (int ktile = 0; ktile < BN / 16; ++ktile) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int kj = key0 + 16 * ktile + 4 * g4 + i;
                float x = sc[ktile][t][i] * a.scale2;
                if (BIAS) x += bias_lds[min(max(qi[t] - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
                if (masked && ((cmask && kj > qi[t]) || kj >= Lk)) x = -INFINITY;
                sc[ktile][t][i] = x;
                x_max = fmaxf(x_max, x);
              }
            }
            mx[t] = quarter_max(x_max);
          }
        }
        // running max with slack, as the library's kernel
        const bool grow0 = mx[0] > m[0] + kRescaleSlack, grow1 = mx[1] > m[1] + kRescaleSlack;
        if (__any(grow0 || grow1)) {
          const bool grow[2] = {grow0, grow1};
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float mn = grow[t] ? mx[t] : m[t];
            const float alpha = __builtin_amdgcn_exp2f(m[t] - mn);
            m[t] = mn;
            l[t] *= alpha;
            lb[t] *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) o[dt][t] *= alpha;
          }
        }
        if (j + 1 == n_kv) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            l_pre[t] = l[t];
            lb_pre[t] = lb[t];
          }
        }
        if (plain) {  // raw dot products: the scale is folded into the exponent
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float nm = -m[t];
#pragma unroll
            for (int ktile = 0; ktile < BN / 16; ++ktile) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[ktile][t][i], a.scale2, nm));
                sc[ktile][t][i] = p;
                l[t] += p;
              }
            }
          }
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int ktile = 0; ktile < BN / 16; ++ktile) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(sc[ktile][t][i] - m[t]);
                sc[ktile][t][i] = p;
                l[t] += p;
              }
            }
          }
        }
        prio_mfma();
#pragma unroll
        for (int ks = 0; ks < BN / 32; ++ks) {
          bf16x8 pf[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pf[t][e] = (bf16)sc[2 * ks][t][e];
              pf[t][4 + e] = (bf16)sc[2 * ks + 1][t][e];
            }
            Frag<T> f;
            f.v = pf[t];
            lb[t] = frag_sum(f, lb[t]);
          }
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const bf16x8 vf = ptfrag16<C::VS>(vt, 32 * ks, 16 * dt, lane);
#pragma unroll
            for (int t = 0; t < 2; ++t) mma16(o[dt][t], vf, pf[t]);
          }
        }
        prio_valu();
      }
      if (j + 1 < n_kv) swrite((j + 1) & 1);
      __syncthreads();
    }

    // Epilogue, per query tile: the four rows' partial sums combined, the pad
    // terms removed (cancellation guard as in the library's kernel), O and lse
    // stored.
    const View ov = seq_view((char*)a.out + qrow, Lq, gstride, C::ROWB);
    const View lv = seq_view(a.lse + (size_t)q0 * H + h, Lq, (uint32_t)H * 4, 4);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float lt = quarter_sum(l[t]);
      float lbt = quarter_sum(lb[t]);
      if (wave_on && last_tile >= 0 && !last_masked) {
        const int pad1 = (last_tile + 1) * BN;
        if (pad1 > Lk) {
          float pads, pads_b;
          if (!BIAS) {
            const float pe = __builtin_amdgcn_exp2f(-m[t]);
            pads = (float)(pad1 - Lk) * pe;
            pads_b = (float)(pad1 - Lk) * as_operand(pe, (T*)0);
          } else {
            float sub = 0.f, subb = 0.f;
            for (int kj = Lk + g4; kj < pad1; kj += 4) {
              const float pe =
                  __builtin_amdgcn_exp2f(bias_lds[min(max(qi[t] - kj, -kBiasRadius), kBiasRadius) + kBiasRadius] - m[t]);
              sub += pe;
              subb += as_operand(pe, (T*)0);
            }
            pads = quarter_sum(sub);
            pads_b = quarter_sum(subb);
          }
          const float full = lt;
          lt -= pads;
          lbt -= pads_b;
          const bool cancel = !(lt > full * 0x1p-12f);
          if (__any(cancel)) {
            const lds_t* kt = lds + (last_tile & 1) * C::STAGE;
            const int key0 = last_tile * BN;
            float sv = 0.f, svb = 0.f;
#pragma unroll 1
            for (int r = g4; r < BN; r += 4) {
              const int kj = key0 + r;
              if (kj >= Lk) break;
              float dot = 0.f;
#pragma unroll 1
              for (int c = 0; c < C::CPR; ++c) {
                const i32x4 kq = *(const __attribute__((address_space(3))) i32x4*)(kt + r * C::KS + c * 16);
                const i32x4 qq = ld16(qv, (uint32_t)qi[t] * gstride + c * 16);
                const bf16x8 k8 = __builtin_bit_cast(bf16x8, kq), q8 = __builtin_bit_cast(bf16x8, qq);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot += (float)k8[e] * (float)q8[e];
              }
              float x = dot * a.scale2;
              if (BIAS) x += bias_lds[min(max(qi[t] - kj, -kBiasRadius), kBiasRadius) + kBiasRadius];
              const float pe = __builtin_amdgcn_exp2f(x - m[t]);
              sv += pe;
              svb += as_operand(pe, (T*)0);
            }
            const float fixed = quarter_sum(l_pre[t]) + quarter_sum(sv);
            const float fixedb = quarter_sum(lb_pre[t]) + quarter_sum(svb);
            if (cancel) {
              lt = fixed;
              lbt = fixedb;
            }
          }
        }
      }
      if (wave_on) {
        const float inv = lbt > 0.f ? 1.0f / lbt : 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const int d = 16 * dt + 4 * g4;
          store4(ov, (uint32_t)qi[t] * gstride + d * ES, o[dt][t][0] * inv, o[dt][t][1] * inv, o[dt][t][2] * inv,
                 o[dt][t][3] * inv, (T*)0);
        }
        if (g4 == 0) {
          const float lse = lt > 0.f ? (m[t] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
          st4f(lv, (uint32_t)qi[t] * H * 4, lse);
        }
      }
    }
    if constexpr (!kSchedPersistent) break;
  }
}

template <typename T, int D, bool PADDED = false>
static hipError_t launch_fwd_t(const FwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st) {
  constexpr bool PP = FwdPingPong<T, D>::value && !PADDED;
  constexpr bool R64 = FwdRows64<T, D>::value && !PADDED;
  constexpr bool M16 = FwdMfma16<T, D>::value && !PADDED;
  constexpr int threads = PP ? 512 : 256;
  void (*kern)(FwdArgs);
  if constexpr (M16)
    kern = bias ? jfa_fwd_m16_kernel<D, true> : jfa_fwd_m16_kernel<D, false>;
  else if constexpr (R64)
    kern = bias ? jfa_fwd_r64_kernel<D, true> : jfa_fwd_r64_kernel<D, false>;
  else if constexpr (PP)
    kern = bias ? jfa_fwd_pp_kernel<D, true> : jfa_fwd_pp_kernel<D, false>;
  else
    kern = bias ? jfa_fwd_kernel<T, D, true, PADDED> : jfa_fwd_kernel<T, D, false, PADDED>;
  static int occ_b = 0, occ_n = 0;
  int& occ = bias ? occ_b : occ_n;
  if (occ == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
  }
  const long grid = kSchedPersistent ? max(1L, min(max_items, (long)num_cus * occ)) : max(1L, max_items);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, st, a);
  return hipGetLastError();
}

int fwd_tile_keys(bool f32, int D) {
  if (f32) return D == 32 ? FwdKeys<float, 32>::value : FwdKeys<float, 64>::value;
  return D == 32 ? FwdKeys<bf16, 32>::value : (D == 64 ? FwdKeys<bf16, 64>::value : FwdKeys<bf16, 128>::value);
}

int fwd_tile_rows(bool f32, int D, bool padded) {
  if (padded) return FwdTiles<bf16, 128>::BM;  // every D: jfa_fwd_kernel's 128 rows
  if (f32) return D == 32 ? FwdRows<float, 32>::value : FwdRows<float, 64>::value;
  return D == 32 ? FwdRows<bf16, 32>::value : (D == 64 ? FwdRows<bf16, 64>::value : FwdRows<bf16, 128>::value);
}

// Host-side entry used by the C-ABI layer.
hipError_t launch_fwd(bool f32, int D, const FwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st) {
  if (f32) {
    if (D == 32) return launch_fwd_t<float, 32>(a, bias, max_items, num_cus, st);
    if (D == 64) return launch_fwd_t<float, 64>(a, bias, max_items, num_cus, st);
    return hipErrorInvalidValue;  // fp32 with D = 128 is rejected on the host
  }
  if (D == 32) return launch_fwd_t<bf16, 32>(a, bias, max_items, num_cus, st);
  if (D == 64) return launch_fwd_t<bf16, 64>(a, bias, max_items, num_cus, st);
  return launch_fwd_t<bf16, 128>(a, bias, max_items, num_cus, st);
}

// Padded-dense baseline (bf16): uniform offsets in a, true key lengths in a.kv_len.
hipError_t launch_fwd_padded(int D, const FwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st) {
  if (D == 32) return launch_fwd_t<bf16, 32, true>(a, bias, max_items, num_cus, st);
  if (D == 64) return launch_fwd_t<bf16, 64, true>(a, bias, max_items, num_cus, st);
  return launch_fwd_t<bf16, 128, true>(a, bias, max_items, num_cus, st);
}

}  // namespace jfa
