// Kernel argument blocks and launch entry points shared by the kernels and
// the C-ABI layer (host code sees only these declarations).
#pragma once
#include <hip/hip_runtime.h>

namespace jfa {

struct PlanHeader;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* q_off;
  const int* kv_off;
  const float* bias;  // [H][257] or null
  void* out;
  float* lse;
  const int4* items;   // work list of this pass
  PlanHeader* hdr;
  int H;
  int causal;
  float scale2;        // softmax scale * log2(e)
  int B;
  int* gfirst;         // short-query pass: [B*H] list position of chunk 0 of each (b, h), -1 if none; null: no such pass
  float* op;           // short-query pass: per item, [64, D] fp32 rows normalised over the chunk's keys
  float* lsep;         // short-query pass: per item, [64] log2 of each row's sum over the chunk's keys
  const int* kv_len;   // padded-dense baseline only: [B] true key count of each fixed-length slot
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  const void* dout;
  const int* q_off;
  const int* kv_off;
  const float* bias;
  void* dq;
  void* dk;
  void* dv;
  float2* rowc;        // [Tq, H] (lse * log2(e), Delta) per query row (workspace)
  const int4* items;   // work list of this pass
  PlanHeader* hdr;
  int H;
  int causal;
  float scale;         // 1/sqrt(D)
  float scale2;        // scale * log2(e)
  long tq;             // query tokens (rows of rowc per head)
  int B;
  int* gfirst;         // short-query pass: [B*H] list position of chunk 0 of each (b, h), -1 if none; null: no such pass
  float* dqp;          // short-query pass: per item, a [64, D] fp32 partial dQ
  // Bias gradient (null dbias: not computed): per item of the dK/dV and
  // short-query passes, the 257 bins of its pairs; per (b, h), the list
  // position of the dK/dV pass's first item of the group (-1 if none).
  float* dbp_kv;
  float* dbp_sq;
  int* gfirst_kv;
  float* dbpart;       // [ceil(B / kDbSeqBlock)][H][257]: sums over blocks of sequences
  float* dbias;        // [H][257] fp32 output
  float* dqacc;        // study designs with dQ fused into the dK/dV pass: fp32 [Tq, H, D] accumulator (1)
                       // or [key tile][Tq, H, D] partials (2); null in the library
  const int* kv_len;   // padded-dense baseline only: [B] true key count of each fixed-length slot
};

// Bias gradient: sequences per block of its first summing step.
constexpr int kDbSeqBlock = 4;

// Pass kinds of the work lists.
enum PlanKind { kPassQ = 0, kPassKV = 1, kPassSQ = 2 };

struct PlanPass {
  int4* items;
  PlanHeader* hdr;
  long capacity;  // items that fit the workspace
  int TM, TN;     // query rows / keys per tile and per visited block (sq: keys per chunk)
  int kind;       // PlanKind
  int nq;         // queues (one per XCD)
  int short_q;    // q and kv passes: sequences with Lq <= short_q and more than kSqKC keys get no items (-1: none)
  int* gfirst;    // sq pass: [B*H] list position of chunk 0 of each (b, h), -1 if none
};

constexpr int kPlanQueues = 8;  // MI355X: 8 XCDs

struct PlanArgs {
  const int* q_off;
  const int* kv_off;
  int B, H, causal;
  PlanPass pass[3];
};

// Short-query passes: sequences with at most kSqQMax queries and more than
// kSqKC keys are cut into chunks of kSqKC keys, one workgroup per (b, h,
// chunk), in the forward (split over the keys, chunks merged per (b, h)) and
// in the backward (one pass over K/V, dQ partials summed per (b, h)). The
// other passes skip them.
constexpr int kSqQMax = 64, kSqKC = 1024, kSqKT = 64;
__host__ __device__ inline bool short_query(int Lq, int Lk) { return Lq <= kSqQMax && Lk > kSqKC; }

// Tile shapes (query rows x keys) of each kernel. The forward's waves per
// workgroup (32 query rows each) depend on the element type and D. The
// two-group kernel (8 waves in two groups that alternate matrix and vector
// phases, 256 rows per item) is a compile-time study choice for bf16 D = 128
// (JFA_FWD_PINGPONG) and D = 64 (JFA_FWD_PINGPONG_NARROW); the library
// builds the 4-wave kernel for every shape.
#ifndef JFA_FWD_PINGPONG
#define JFA_FWD_PINGPONG 0
#endif
#ifndef JFA_FWD_PINGPONG_NARROW
#define JFA_FWD_PINGPONG_NARROW 0
#endif
template <typename T, int D> struct FwdPingPong {
  static constexpr bool value = sizeof(T) == 2 && ((D == 128 && JFA_FWD_PINGPONG != 0) ||
                                                   (D == 64 && JFA_FWD_PINGPONG_NARROW != 0));
};
// 64 query rows per wave (two 32-row halves sharing each K and V fragment)
// for bf16 D <= 64: another study choice (JFA_FWD_ROWS_PER_WAVE = 64).
#ifndef JFA_FWD_ROWS_PER_WAVE
#define JFA_FWD_ROWS_PER_WAVE 32
#endif
template <typename T, int D> struct FwdRows64 {
  static constexpr bool value = JFA_FWD_ROWS_PER_WAVE == 64 && sizeof(T) == 2 && D <= 64;
};
template <typename T, int D> struct FwdWaves { static constexpr int value = FwdPingPong<T, D>::value ? 8 : 4; };
template <typename T, int D> struct FwdRows {
  static constexpr int value = (FwdRows64<T, D>::value ? 64 : 32) * FwdWaves<T, D>::value;
};
// Keys per block of the forward, for rows of 128 bytes (JFA_FWD_BN), for
// wider ones (JFA_FWD_WIDE_BN) and 64 for narrower ones: compile-time
// choices of the tile-shape study (the library takes the defaults).
#ifndef JFA_FWD_BN
#define JFA_FWD_BN 64
#endif
#ifndef JFA_FWD_WIDE_BN
#define JFA_FWD_WIDE_BN 64
#endif
template <typename T, int D> struct FwdKeys {
  static constexpr int value =
      D * (int)sizeof(T) >= 256 ? JFA_FWD_WIDE_BN : (D * (int)sizeof(T) == 128 ? JFA_FWD_BN : 64);
};
// padded: the padded-dense baseline, which always takes the 4-wave kernel.
int fwd_tile_rows(bool f32, int D, bool padded = false);
int fwd_tile_keys(bool f32, int D);
// dK/dV pass: rows of 128 bytes or less (bf16 D <= 64, fp32 D = 32) use the
// one-role kernel with 64-row query blocks, wider rows the two-role kernel
// with 32-row blocks.
constexpr int kDkvTM = 32, kDkv1TM = 64, kDkvTN = 128;
int dkv_tile_rows(bool f32, int D);
constexpr int kDqTM = 128, kDqTN = 64;

// Persistent launches: grid = min(max_items, CUs x resident workgroups per CU).
// The short-query chunk passes run first; the forward launch then merges the
// chunks of each sequence and the dQ launch sums its partial dQ.
hipError_t launch_fwd(bool f32, int D, const FwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st);
hipError_t launch_fwd_padded(int D, const FwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st);
hipError_t launch_fsq(bool f32, int D, const FwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st);
hipError_t launch_dkdv(bool f32, int D, const BwdArgs& a, bool bias, bool dbias, long max_items, int num_cus,
                       hipStream_t st);
hipError_t launch_dq(bool f32, int D, const BwdArgs& a, bool bias, long max_items, int num_cus, hipStream_t st);
hipError_t launch_sq(bool f32, int D, const BwdArgs& a, bool bias, bool dbias, long max_items, int num_cus,
                     hipStream_t st);
hipError_t launch_dbias(const BwdArgs& a, hipStream_t st);
// Design of the backward's dQ (a compile-time study choice; 0 = the split
// passes): 1 or 2 when that build fuses dQ into the dK/dV pass for this
// element type and D. Then the dQ pass gets no items, the accumulator is
// zeroed first (1) and launch_dq_fused_out writes dQ after the dK/dV pass.
int bwd_dq_mode(bool f32, int D);
hipError_t launch_dqacc_zero(float* acc, long n, hipStream_t st);
hipError_t launch_dq_fused_out(bool f32, int D, const BwdArgs& a, hipStream_t st);
hipError_t launch_plan(const PlanArgs& a, int npass, hipStream_t st);
// The backward's lists (passes of p) and Delta of every row (a.rowc), one launch.
hipError_t launch_bwd_prep(const PlanArgs& p, int npass, bool f32, int D, const BwdArgs& a, hipStream_t st);
hipError_t launch_scan(const int* lengths, int B, int* offsets, hipStream_t st);
// Uniform offsets of B fixed-length slots: qo[b] = b * Lq, ko[b] = b * Lk, b <= B.
hipError_t launch_slot_offsets(int B, int Lq, int Lk, int* qo, int* ko, hipStream_t st);

}  // namespace jfa
