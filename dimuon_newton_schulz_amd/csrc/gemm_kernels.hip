// Grouped GEMM kernels of the Newton-Schulz iteration.
//
// The products, C[i][j] = sum_k P[i][k] Q(k, j):
//   Gram     A = X X^T               P = X, Q(k, j) = X[j][k]   (K = N)  symmetric
//   poly     B = a I + b A + c A A   P = A, Q(k, j) = A[j][k]   (K = k)  symmetric
//   combine  X' = B X                P = B, Q(k, j) = X[k][j]   (K = k)
// (a X + (b A + c A A) X with the a X term folded into B's diagonal, so the
// combine reads nothing but its two operands.)  The symmetric products read
// both operands K-contiguous ("NT") and compute the upper-triangular tiles
// only, storing each such tile and its mirror.  The bf16 combine reads X
// itself k-major (transposing LDS reads), so no X^T is ever written; the fp32
// kernels at the end of this file keep X^T beside X and stay "NT".
//
// bf16 path: a BM x BN workgroup tile (BM, BN in {128, 256}), wave64s in a
// 2 x WC grid, each wave owning (BM/2) x (BN/WC) as 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16 (wave counts per kernel below).  Operands go from
// global memory straight into a ring of LDS stages of 64 k-values
// (global_load_lds_dwordx4, no register staging): two stages, one in flight
// while the other is multiplied, or four (up to three in flight) where a
// 128 x 128 workgroup has a CU's LDS to itself.  The loop is pipelined so
// that LDS fragment reads are covered by MFMAs.  A 256 x 256 tile needs half
// the L2 traffic per flop of a 128 x 128 one; with its 128 KB ring one
// workgroup runs per CU.  The 128 x 128 symmetric products run two per CU
// (one per CU, on the four-stage ring, for lists no longer than the GPU has
// CUs); every combine workgroup holds a whole CU's LDS.
//
// The epilogue stages the fp32 accumulators through LDS (transposed, in
// rounds) so that the row-major and the transposed outputs are written as
// 16-byte runs.
#include <type_traits>

#include "common.h"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int LBK = 64;        // k per pipeline stage: whole 128-byte lines of each operand row
constexpr int NQ = LBK / 16;   // MFMA k-steps per stage

// The two-stage ring takes 128 KB for 256 x 256, 96 KB for 128 x 256 and
// 64 KB for 128 x 128; one stage is multiplied while the next is in flight.
// Whole-line stages fetch faster than half-line ones (each row's 128 bytes
// arrive as one request), and a deeper ring of shorter stages measured no
// faster.
// Waves in 2 rows x WC columns.  By this rule tiles of 128 x 256 and larger
// run eight waves (WC = 4, two per SIMD: one wave's MFMAs cover the other's
// loads and barrier waits), measured 3-5% faster per step than four, and
// 128 x 128 tiles four (eight measured slower there); the 256 x 256
// symmetric products set four waves apart from the rule (kSyrkWC).
#ifndef MUON_GEMM_WC_LARGE
#define MUON_GEMM_WC_LARGE 4
#endif
#ifndef MUON_GEMM_WC_SMALL
#define MUON_GEMM_WC_SMALL 2
#endif
// WCX, when non-zero, sets the wave columns of a kernel apart from the rule.
template <int BM, int BN, int WCX = 0>
struct GemmT {
  static constexpr int WC = WCX ? WCX : (BM * BN >= 32768 ? MUON_GEMM_WC_LARGE : MUON_GEMM_WC_SMALL);
  static constexpr int NW = 2 * WC, NT = 64 * NW;    // waves, threads
  static constexpr int MS = BM / 64, NS = BN / (32 * WC);   // 32 x 32 blocks per wave
  static constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;  // 16-byte LDS loads per thread and stage
  static constexpr int LPS = LA + LB;
  static constexpr int STAGE = (BM + BN) * LBK;      // bf16 elements per stage: A rows, then B rows
  static constexpr int BUDGET = BM * BN == 16384 ? 81920 : 163840;
  static constexpr int SP = BM / 2 + 2;              // epilogue staging row stride (floats)
  union Smem {                                       // symmetric products
    uint16_t buf[2][STAGE];
    float st[BN * SP];                               // half a tile, transposed, fp32
  };
  static_assert(sizeof(Smem) <= BUDGET, "LDS budget");
};

// The combine's shared memory: its two stages are separate arrays, because
// the compiler orders a transposing LDS read after pending direct loads
// unless it can tell their arrays apart.  The epilogue stages in R rounds
// (R = 4 for 256-row tiles) that alternate between the two arrays, each
// sized for a stage and for a round.
template <int BM, int BN>
struct CombT {
  using G = GemmT<BM, BN>;
  static constexpr int R = G::MS >= 4 ? 4 : 2;
  static constexpr int SPR = BM / R + 2;             // staged row stride (floats)
  static constexpr int STG = BN * SPR * 2;           // staging of a round, in bf16 elements
  static constexpr int RB = G::STAGE > STG ? G::STAGE : STG;
  static_assert(2 * RB * 2 <= G::BUDGET, "LDS budget");
};

// Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
// run of the tile list so that tiles sharing operand panels share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
}

// s_waitcnt with only the vector-memory counter limited to N (N <= 63).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// A stage holds rows of 64 k-values (128 bytes, eight 16-byte chunks).
// Chunk c of row r sits at chunk slot c ^ ((r >> 1) & 7): the 16 rows a
// phase of a fragment read touches at one logical chunk then fall on 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// A k-major operand (QT: Q[k][n], n contiguous) is staged as LBK rows of BN
// values; chunk c of k-row r sits at slot c ^ (4 (r & 3)), so that the four
// k-rows one transposing read touches fall on distinct banks.
__device__ __forceinline__ int qswz(int row) { return 4 * (row & 3); }

// Direct global -> LDS loads of stage `st` (k0 = st * LBK) into buffer b.  A
// wave's load writes 64 consecutive 16-byte LDS chunks (8 rows of P, or of Q
// when n-major; 512 / BN k-rows of Q when k-major); each lane fetches the
// global chunk that belongs in its slot.
// same: Q is P (a diagonal tile of a symmetric product); only P's rows are
// loaded, and the fragments of both operands come from them.
// Loads Q0 .. Q1-1 of the thread's LA + LB (all of them by default).
template <int BM, int BN, bool QT, int Q0 = 0, int Q1 = GemmT<BM, BN>::LPS, int WCX = 0>
__device__ __forceinline__ void issue_stage(const MUON_GLOBAL uint16_t* P, int64_t ldp, const MUON_GLOBAL uint16_t* Q,
                                            int64_t ldq, int st, uint16_t* buf, bool same = false) {
  using G = GemmT<BM, BN, WCX>;
  constexpr int LPR = BN / 8, RPI = 64 / LPR;   // k-major Q: lanes per k-row, k-rows per load
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k0 = st * LBK;
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    const bool is_a = q < G::LA;
    if (!is_a && same) break;
    const int blk = (is_a ? q : q - G::LA) * G::NW + wave;
    const MUON_GLOBAL uint16_t* src;
    if (QT && !is_a) {
      const int r = blk * RPI + lane / LPR;
      const int c = (lane % LPR) ^ qswz(r);
      src = Q + (k0 + r) * ldq + c * 8;
    } else {
      const int row = blk * 8 + (lane >> 3);
      const int lch = (lane & 7) ^ swz(row);
      src = is_a ? P + row * ldp + k0 + lch * 8 : Q + row * ldq + k0 + lch * 8;
    }
    uint16_t* dst = buf + (is_a ? 0 : BM * LBK) + blk * 512;
    __builtin_amdgcn_global_load_lds((const MUON_GLOBAL void*)(src), (__attribute__((address_space(3))) void*)(dst),
                                     16, 0, 0);
  }
}

// acc[s][t] += sum over k < K of P[row wr*BM/2 + s*32 + i][k] * Q(k, col wc*BN/WC + t*32 + j),
// (wave = wr * WC + wc) with Q(k, n) = Q[n][k] (n-major, QT false) or Q[k][n] (k-major, QT true);
// K is a multiple of 2 * LBK.  A stage holds NQ k-steps of 16; the two
// stages alternate between buffers b0 and b1 (the loop is unrolled by two,
// so every access names its buffer).  Per stage kt, with fragments read one
// k-step ahead of the MFMAs:
//   k-steps 1 .. NQ-1 of stage kt: read step q, MFMAs of step q-1
//   wait for this wave's loads of stage kt+1; barrier
//   load stage kt+2 into stage kt's buffer (every wave has its fragments of
//   stage kt in registers: LDS reads complete before the barrier)
//   read step 0 of stage kt+1;  MFMAs of step NQ-1
// so fragment reads are always covered by MFMAs and one stage is in flight
// while the other is multiplied.
//
// k-major Q: the B fragment of a k-step (lane l: k = 8 (l / 32) + 0..7,
// n = l mod 32 of the block) comes from two transposing reads
// (ds_read_b64_tr_b16): in each 16-lane group, lane i receives element
// i mod 4 of the 8-byte reads of lanes 4 e + i / 4, e = 0..3, so lane m of the
// group reads the four n-values 4 (m mod 4) .. + 3 of its 16-column half at
// k-row 8 (l / 32) + m / 4, and four k-rows further down for the second read.
//
// NB = 4 (a deep ring, for 128 x 128 lists of at most one workgroup per CU,
// where the LDS of a second workgroup is free): four buffers b0 .. b3,
// stages 0 .. 3 issued up front, and stage kt+3 issued into stage kt-1's
// buffer as stage kt starts, so up to three stages are in flight while one
// is multiplied.  The MFMAs and their k order are those of the two-buffer
// loop, so the results are the same bit for bit.
template <int BM, int BN, bool QT, bool F32 = false, int WCX = 0, int NB = 2>
__device__ __forceinline__ void mma_bf16(const uint16_t* Pg, int64_t ldp, const uint16_t* Qg, int64_t ldq, int K,
                                         uint16_t* b0, uint16_t* b1,
                                         f32x16_t (&acc)[GemmT<BM, BN, WCX>::MS][GemmT<BM, BN, WCX>::NS],
                                         bool same = false, uint16_t* b2 = nullptr, uint16_t* b3 = nullptr) {
  using G = GemmT<BM, BN, WCX>;
  constexpr int MS = G::MS, NS = G::NS, LPS = G::LPS, WN = BN / G::WC;
  static_assert(NQ % 2 == 0, "fragment sets alternate");
  static_assert(NB == 2 || NB == 4, "two or four ring buffers");
  static_assert(NB == 2 || 3 * LPS <= 63, "vector-memory counter range");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave / G::WC, wc = wave % G::WC;
  const MUON_GLOBAL uint16_t* P = gmem(Pg);
  const MUON_GLOBAL uint16_t* Q = gmem(Qg);
  const int nk = K / LBK;
  // Every wave's stage-0 loads are issued before any stage-1 load (the
  // barrier waits for issue, not for data): the first stage arrives first.
  // (The deep ring loads both panels of a diagonal tile too, so that every
  // stage is the same number of loads.)
  if constexpr (NB == 4) same = false;
  issue_stage<BM, BN, QT, 0, G::LPS, WCX>(P, ldp, Q, ldq, 0, b0, same);
  __builtin_amdgcn_s_barrier();
  issue_stage<BM, BN, QT, 0, G::LPS, WCX>(P, ldp, Q, ldq, 1, b1, same);
  if constexpr (NB == 4) {
    issue_stage<BM, BN, QT, 0, G::LPS, WCX>(P, ldp, Q, ldq, min(2, nk - 1), b2);
    issue_stage<BM, BN, QT, 0, G::LPS, WCX>(P, ldp, Q, ldq, min(3, nk - 1), b3);
  }
  // Fragment addresses (elements within a stage): row (lane & 31) of each
  // 32-row block, logical chunk 2 q + (lane >> 5) for k-step q.  The swizzle
  // of a row depends on its index mod 16 only, i.e. on lane & 31.
  const int fr = lane & 31, sw = swz(fr), half = lane >> 5;
  const int a_off = (wr * (BM / 2) + fr) * LBK, b_off = (same ? 0 : BM * LBK) + (wc * WN + fr) * LBK;
  // k-major Q: the reading lane's k-row and n-column in the stage (block t
  // adds 32 columns, k-step q 16 rows, the second read 4 rows); the swizzle
  // of those rows is 4 (m / 4) throughout.
  const int m16 = lane & 15, g16 = lane >> 4;
  const int t_row = 8 * (g16 >> 1) + (m16 >> 2);
  const int t_col = wc * WN + 16 * (g16 & 1) + 4 * (m16 & 3);
  const int t_sw = 4 * (m16 >> 2);
  bf16x8_t fa[2][MS], fb[2][NS];
  auto read_step = [&](const uint16_t* buf, int q, bf16x8_t (&ra)[MS], bf16x8_t (&rb)[NS]) {
    const int ch = ((2 * q + half) ^ sw) * 8;
#pragma unroll
    for (int s = 0; s < MS; ++s) ra[s] = *reinterpret_cast<const bf16x8_t*>(buf + a_off + s * 32 * LBK + ch);
    if constexpr (QT) {
      const uint16_t* qb = buf + BM * LBK + (q * 16 + t_row) * BN;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const int col = t_col + 32 * t;
        const int at = (((col >> 3) ^ t_sw) << 3) + (col & 7);
        const i16x4_t lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(qb + at));
        const i16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(qb + 4 * BN + at));
        rb[t] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
#pragma unroll
      for (int t = 0; t < NS; ++t) rb[t] = *reinterpret_cast<const bf16x8_t*>(buf + b_off + t * 32 * LBK + ch);
    }
  };
  // The combine (k-major Q, twice the LDS read instructions per B fragment)
  // raises a wave's priority while it issues MFMAs, so that of the two waves
  // on a SIMD the one with MFMAs ready issues first (6% faster combines; the
  // symmetric products measured 1% slower with it).
  auto mfma_step = [&](const bf16x8_t (&ra)[MS], const bf16x8_t (&rb)[NS]) {
    if constexpr (QT) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (F32) {
      // fp32 operands: a lane's 16 bytes are 4 consecutive k of its row
      // (k = 8q + 4 (lane >> 5) + 0..3 for chunk pair q); element e of both
      // operands is the lane's k-slot of the e-th 32x32x2 product, so the
      // four products cover the chunk pair's 8 k once each.
#pragma unroll
      for (int s = 0; s < MS; ++s)
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          const f32x4_t a4 = __builtin_bit_cast(f32x4_t, ra[s]);
          const f32x4_t b4 = __builtin_bit_cast(f32x4_t, rb[t]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[s][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[e], b4[e], acc[s][t], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int s = 0; s < MS; ++s)
#pragma unroll
        for (int t = 0; t < NS; ++t)
          acc[s][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[s], rb[t], acc[s][t], 0, 0, 0);
    }
    if constexpr (QT) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The point after which stage kt's buffer may be reloaded: this wave's
  // reads of it are complete and stage kt+1 has landed; no load is in flight.
  auto sync = [&]() {
    // (The scheduling barriers keep the MFMAs on their side of the wait.)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    __builtin_amdgcn_sched_barrier(0);
  };
  // From sync after stage kt to sync after stage kt+1 (cur holds stage kt,
  // nxt stage kt+1): load stage kt+2 into cur, read step 0 of stage kt+1,
  // MFMAs of stage kt's last step, then stage kt+1's other steps.  The loop
  // is entered and closed at a sync, with no load in flight, so the compiler
  // keeps track of which buffer the loads in flight write.
  // Half of stage kt+2's loads go out before the first MFMAs of the half
  // step and half after them, so that the SIMD's two waves do not both sit
  // in a run of load issues while the matrix core idles (1.4% faster on the
  // 4096^2 set than all loads first).
  auto half_step = [&](uint16_t* cur, uint16_t* nxt, int kt) {
    if (kt + 2 < nk) issue_stage<BM, BN, QT, 0, LPS / 2, WCX>(P, ldp, Q, ldq, kt + 2, cur, same);
    read_step(nxt, 0, fa[0], fb[0]);
    mfma_step(fa[(NQ - 1) & 1], fb[(NQ - 1) & 1]);
    if (kt + 2 < nk) issue_stage<BM, BN, QT, LPS / 2, LPS, WCX>(P, ldp, Q, ldq, kt + 2, cur, same);
#pragma unroll
    for (int q = 1; q < NQ; ++q) {
      read_step(nxt, q, fa[q & 1], fb[q & 1]);
      mfma_step(fa[(q - 1) & 1], fb[(q - 1) & 1]);
    }
    sync();
  };
  if constexpr (NB == 4) {
    // Every step issues one stage's loads (past the last stage, the last
    // stage again into a buffer that is no longer read), so that each wait
    // is a fixed count: the compiler then keeps the loads of later stages in
    // flight across the reads of the current one.
    // After stage kt: this wave's reads of it are complete and stage kt+1
    // has landed (the two stages issued after it may still be in flight).
    auto sync_deep = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      wait_vm<2 * LPS>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      __builtin_amdgcn_sched_barrier(0);
    };
    // Stage kt from cur; stage kt+3 into ib (stage kt-1's buffer, which no
    // wave reads any more), half of it before the first MFMAs.
    auto deep_step = [&](uint16_t* cur, uint16_t* ib, int kt) {
      const int st = min(kt + 3, nk - 1);
      read_step(cur, 0, fa[0], fb[0]);
      __builtin_amdgcn_sched_barrier(0);
      issue_stage<BM, BN, QT, 0, LPS / 2, WCX>(P, ldp, Q, ldq, st, ib);
      mfma_step(fa[(NQ - 1) & 1], fb[(NQ - 1) & 1]);
      issue_stage<BM, BN, QT, LPS / 2, LPS, WCX>(P, ldp, Q, ldq, st, ib);
#pragma unroll
      for (int q = 1; q < NQ; ++q) {
        read_step(cur, q, fa[q & 1], fb[q & 1]);
        mfma_step(fa[(q - 1) & 1], fb[(q - 1) & 1]);
      }
      sync_deep();
    };
    wait_vm<3 * LPS>();   // stage 0 landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    read_step(b0, 0, fa[0], fb[0]);
#pragma unroll
    for (int q = 1; q < NQ; ++q) {
      read_step(b0, q, fa[q & 1], fb[q & 1]);
      mfma_step(fa[(q - 1) & 1], fb[(q - 1) & 1]);
    }
    sync_deep();
    // Stage kt lives in buffer kt mod 4 (unrolled by four, so that every
    // access names its buffer).
    for (int kt = 1; kt < nk; kt += 4) {
      deep_step(b1, b0, kt);
      if (kt + 1 >= nk) break;
      deep_step(b2, b1, kt + 1);
      if (kt + 2 >= nk) break;
      deep_step(b3, b2, kt + 2);
      if (kt + 3 >= nk) break;
      deep_step(b0, b3, kt + 3);
    }
    mfma_step(fa[(NQ - 1) & 1], fb[(NQ - 1) & 1]);
    // No load may still be writing the ring when the epilogue reuses it.
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
  } else {
    // Stage 0 landed (stage 1's loads were issued after it).
    if (same) wait_vm<G::LA>();
    else wait_vm<LPS>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    read_step(b0, 0, fa[0], fb[0]);
#pragma unroll
    for (int q = 1; q < NQ; ++q) {
      read_step(b0, q, fa[q & 1], fb[q & 1]);
      mfma_step(fa[(q - 1) & 1], fb[(q - 1) & 1]);
    }
    sync();
    int kt = 0;
    for (; kt + 2 < nk; kt += 2) {
      half_step(b0, b1, kt);
      half_step(b1, b0, kt + 1);
    }
    half_step(b0, b1, kt);   // stage nk-1 (nk is even)
    mfma_step(fa[(NQ - 1) & 1], fb[(NQ - 1) & 1]);
  }
}

// Calls f(integral_constant<int, I>) for I = I0 .. N-1: compile-time block
// indices, so that the accumulators are never indexed at run time.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Tile-relative column of block t for this lane (rows of a block's
// accumulator group g are 8g + 4 (lane >> 5) + 0..3).
template <int BM, int BN, int WCX = 0>
__device__ __forceinline__ int blk_col(int t) {
  using G = GemmT<BM, BN, WCX>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave % G::WC) * (BN / G::WC) + t * 32 + (lane & 31);
}

// Eight consecutive values at element idx: bf16 (16 bytes) or f32 (32 bytes).
__device__ __forceinline__ void store8(void* p, int64_t idx, int32_t dt, const float (&v)[8]) {
  if (dt == DT_BF16) {
    *reinterpret_cast<MUON_GLOBAL uint4*>(gmem(static_cast<uint16_t*>(p)) + idx) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7]));
  } else {
    MUON_GLOBAL float4* q = reinterpret_cast<MUON_GLOBAL float4*>(gmem(static_cast<float*>(p)) + idx);
    q[0] = make_float4(v[0], v[1], v[2], v[3]);
    q[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

__device__ __forceinline__ uint4 fetch8_bf16(const uint16_t* p, int64_t idx) {
  return *reinterpret_cast<const MUON_GLOBAL uint4*>(gmem(p) + idx);
}

__device__ __forceinline__ void unpack8_bf16(const uint4& u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

// Epilogue through LDS, in R rounds.  In round r every wave stages its
// accumulator blocks s in [r MS/R, (r+1) MS/R), as fp32 and transposed, into
// stage(r): st[j][il], where staged row il stands for tile row
//   i(il) = (il / QR) * BM/2 + r * QR + il % QR,   QR = BM / (2R)
// (the round's share of each wave row).  From each round, every thread
// produces whole 8-element chunks:
//   out_t(j, i0, v, aux): v[e] = acc of tile element (i0 + e, j)  (a column
//                         run; contiguous in the transposed output)
//   out_n(i, j0, v, aux): v[e] = acc of tile element (i, j0 + e)  (a row run)
// so that all global reads and writes are 16-byte runs.  aux_t(j, i0) and
// aux_n(i, j0) fetch 8 bf16 operand values per chunk (or nothing); a thread
// issues all of a round's column-run fetches before staging and all of its
// row-run fetches right after, so that they are in flight together.  The row
// stride BM/R + 2 keeps both the column-run reads (consecutive lanes along
// il) and the row-run reads (16 lanes along il x 4 along j) free of bank
// conflicts.  ALT: consecutive rounds stage into different arrays, so a
// round needs no barrier before its staging (the previous user of its array
// finished two rounds earlier, before the last round's barrier).  AHEAD:
// each round's operand runs (both kinds) are fetched one round early, the
// first round's before any staging, so that their latency is hidden behind
// a round of LDS work (two rounds of operands in registers).
template <int BM, int BN, int R, bool ALT, int WCX = 0, bool AHEAD = false, typename SF, typename AT, typename AN,
          typename FT, typename FN>
__device__ __forceinline__ void staged_epilogue(const f32x16_t (&acc)[GemmT<BM, BN, WCX>::MS][GemmT<BM, BN, WCX>::NS],
                                                SF&& stage, bool do_t,
                                                bool do_n, AT&& aux_t, AN&& aux_n, FT&& out_t, FN&& out_n) {
  using G = GemmT<BM, BN, WCX>;
  constexpr int HM = BM / 2, QR = BM / (2 * R), RM = BM / R, MR = G::MS / R, SPR = RM + 2;
  static_assert(G::MS % R == 0, "whole blocks per round");
  constexpr int CPR = RM / 8;                 // column-run chunks per staged row
  constexpr int CT = BN * CPR / G::NT;        // column-run chunks per thread and round
  constexpr int NB = RM / 16;                 // blocks of 16 staged rows (row runs)
  constexpr int CN = RM * (BN / 8) / G::NT;   // row-run chunks per thread and round
  constexpr int NSLOT = AHEAD ? 2 : 1;
  static_assert(BN * CPR % G::NT == 0 && RM * (BN / 8) % G::NT == 0, "whole chunks per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wr = wave / G::WC;
  auto t_pos = [&](int q, int& j, int& il) {
    const int c = tid + G::NT * q;
    j = c / CPR;
    il = (c % CPR) * 8;
  };
  auto n_pos = [&](int q, int& il, int& j0) {
    const int c = tid + G::NT * q;
    const int i16 = c & 15, jl = (c >> 4) & 3, r = c >> 6;
    il = (r % NB) * 16 + i16;
    j0 = ((r / NB) * 4 + jl) * 8;
  };
  auto row_in = [&](int rd, int il) { return (il / QR) * HM + rd * QR + il % QR; };
  decltype(aux_t(0, 0)) xt[NSLOT][CT];
  decltype(aux_n(0, 0)) xn[NSLOT][CN];
  auto fetch_t = [&](auto rdc) {
    constexpr int rd = rdc, sl = rd % NSLOT;
    static_for<0, CT>([&](auto q) {
      int j, il;
      t_pos(q, j, il);
      xt[sl][q] = aux_t(j, row_in(rd, il));
    });
  };
  auto fetch_n = [&](auto rdc) {
    constexpr int rd = rdc, sl = rd % NSLOT;
    static_for<0, CN>([&](auto q) {
      int il, j0;
      n_pos(q, il, j0);
      xn[sl][q] = aux_n(row_in(rd, il), j0);
    });
  };
  if constexpr (AHEAD) {
    if (do_t) fetch_t(std::integral_constant<int, 0>{});
    if (do_n) fetch_n(std::integral_constant<int, 0>{});
  }
  static_for<0, R>([&](auto rdc) {
    constexpr int rd = rdc, sl = rd % NSLOT;
    float* st = stage(rd);
    auto row_of = [&](int il) { return row_in(rd, il); };
    if constexpr (AHEAD) {
      if constexpr (rd + 1 < R) {
        if (do_t) fetch_t(std::integral_constant<int, rd + 1>{});
        if (do_n) fetch_n(std::integral_constant<int, rd + 1>{});
      }
    } else if (do_t) {
      fetch_t(rdc);
    }
    // The main loop's stages, or the round that last used this array, are
    // no longer read.
    if (rd == 0 || !ALT) __syncthreads();
    static_for<0, MR * G::NS * 4>([&](auto q) {
      constexpr int sl = q / (G::NS * 4), u = (q / 4) % G::NS, g = q % 4;
      const int s = rd * MR + sl;
      const int il = wr * QR + sl * 32 + 8 * g + 4 * (lane >> 5);
      float* p = st + blk_col<BM, BN, WCX>(u) * SPR + il;
      *reinterpret_cast<float2*>(p) = make_float2(acc[s][u][4 * g], acc[s][u][4 * g + 1]);
      *reinterpret_cast<float2*>(p + 2) = make_float2(acc[s][u][4 * g + 2], acc[s][u][4 * g + 3]);
    });
    __syncthreads();
    // Row-run operands are fetched now and arrive while the column runs are
    // written.
    if (!AHEAD && do_n) fetch_n(rdc);
    if (do_t)
      static_for<0, CT>([&](auto q) {
        int j, il;
        t_pos(q, j, il);
        const float* p = st + j * SPR + il;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float2 w = *reinterpret_cast<const float2*>(p + e);
          v[e] = w.x;
          v[e + 1] = w.y;
        }
        out_t(j, row_of(il), v, xt[sl][q]);
      });
    if (do_n)
      static_for<0, CN>([&](auto q) {
        int il, j0;
        n_pos(q, il, j0);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = st[(j0 + e) * SPR + il];
        out_n(row_of(il), j0, v, xn[sl][q]);
      });
  });
}

// Sum over a workgroup of NW waves (4 or 8), the same value in every thread.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* sh) {
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  v = wave_tree_sum(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float r = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  if constexpr (NW == 8) r = r + ((sh[4] + sh[5]) + (sh[6] + sh[7]));
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Symmetric products (bf16): kind 0 Gram, kind 1 polynomial.  Square tiles.
// ---------------------------------------------------------------------------
// The symmetric products run 256 x 256 tiles on four waves (one per SIMD,
// each 128 x 128): against eight waves, the 8 x 4096^2 Gram is 3% faster
// (the combine, which reads one operand through transposing reads, keeps
// eight).
template <int BT>
constexpr int kSyrkWC = BT == 256 ? 2 : 0;

// NB = 4: the deep ring (lists of at most one workgroup per CU).
template <int BT, int KIND, int NB = 2>
__global__ __launch_bounds__((GemmT<BT, BT, kSyrkWC<BT>>::NT), 1) void k_syrk_bf16(StepArgs a, const Tile* __restrict__ tiles, int ntiles,
                                                   int src_x, int first, Coeffs cf) {
  constexpr int kind = KIND;
  constexpr int WCX = kSyrkWC<BT>;
  using G = GemmT<BT, BT, WCX>;
  union SmemNB {
    uint16_t buf[NB][G::STAGE];
    float st[BT * G::SP];
  };
  static_assert(NB == 2 || (BT == 128 && sizeof(SmemNB) <= 163840), "deep ring: 128 x 128 tiles, one per CU");
  __shared__ typename std::conditional<NB == 2, typename G::Smem, SmemNB>::type sm;
  const Tile t = tiles[xcd_remap(blockIdx.x, ntiles)];
  const MatDesc& d = a.desc[t.mat];
  const uint16_t* P;
  int64_t ld;
  if (kind == 0) {
    P = reinterpret_cast<const uint16_t*>(a.ws + d.x_off[2 * src_x]);
    ld = d.NP;
  } else {
    P = reinterpret_cast<const uint16_t*>(a.ws + d.a_off);
    ld = d.KP;
  }
  f32x16_t acc[G::MS][G::NS];
#pragma unroll
  for (int s = 0; s < G::MS; ++s)
#pragma unroll
    for (int u = 0; u < G::NS; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][u][r] = 0.0f;
  // A diagonal tile multiplies a panel by itself: it is loaded once.
  if constexpr (NB == 4)
    mma_bf16<BT, BT, false, false, WCX, 4>(P + static_cast<int64_t>(t.ti) * BT * ld, ld, P + static_cast<int64_t>(t.tj) * BT * ld,
                                           ld, static_cast<int>(ld), sm.buf[0], sm.buf[1], acc, t.ti == t.tj, sm.buf[2],
                                           sm.buf[3]);
  else
    mma_bf16<BT, BT, false, false, WCX>(P + static_cast<int64_t>(t.ti) * BT * ld, ld, P + static_cast<int64_t>(t.tj) * BT * ld, ld,
                            static_cast<int>(ld), sm.buf[0], sm.buf[1], acc, t.ti == t.tj);

  const float alpha = (kind == 0) ? (first ? a.scal[d.scal_idx].inv_nu2 : 1.0f) : cf.c;
  const uint16_t* E = reinterpret_cast<const uint16_t*>(a.ws + d.a_off);
  void* dst = a.ws + (kind == 0 ? d.a_off : d.b_off);
  const int64_t gi0 = static_cast<int64_t>(t.ti) * BT, gj0 = static_cast<int64_t>(t.tj) * BT;
  const int64_t ldo = d.KP;
  // Element (i, j) of the tile goes to (gi0 + i, gj0 + j) and, mirrored, to
  // (gj0 + j, gi0 + i); a diagonal tile is symmetric, so the mirrored store
  // alone writes all of it.  E (= A) is symmetric: E[i][j] = E[j][i].
  auto aux_t = [&](int j, int i0) {
    return kind == 1 ? fetch8_bf16(E, (gj0 + j) * ldo + gi0 + i0) : make_uint4(0, 0, 0, 0);
  };
  auto aux_n = [&](int i, int j0) {
    return kind == 1 ? fetch8_bf16(E, (gi0 + i) * ldo + gj0 + j0) : make_uint4(0, 0, 0, 0);
  };
  // Polynomial: c (A A) + b A, plus a on the diagonal.  Only diagonal tiles
  // hold diagonal elements; in a run of eight, element e is on it iff
  // e == e_diag (out of 0..7 otherwise).
  const bool diag_tile = kind == 1 && t.ti == t.tj;
  auto fin = [&](float (&v)[8], const uint4& aux, int e_diag) {
    float e8[8];
    unpack8_bf16(aux, e8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = kind == 1 ? alpha * v[e] + cf.b * e8[e] : alpha * v[e];
      if (kind == 1) v[e] += e == e_diag ? cf.a : 0.0f;
    }
  };
  auto out_t = [&](int j, int i0, float (&v)[8], const uint4& aux) {
    fin(v, aux, diag_tile ? j - i0 : -1);
    store8(dst, (gj0 + j) * ldo + gi0 + i0, DT_BF16, v);
  };
  auto out_n = [&](int i, int j0, float (&v)[8], const uint4& aux) {
    fin(v, aux, diag_tile ? i - j0 : -1);
    store8(dst, (gi0 + i) * ldo + gj0 + j0, DT_BF16, v);
  };
  staged_epilogue<BT, BT, 2, false, WCX>(acc, [&](int) { return sm.st; }, true, t.ti != t.tj, aux_t, aux_n, out_t, out_n);
}

// ---------------------------------------------------------------------------
// Combine (bf16 operands): X' = alpha B X, with B = a I + b A + c A A.
// XTERM (no iterations: Z = alpha a X): the product is skipped and X read.
// ---------------------------------------------------------------------------
//
// Every combine workgroup holds the whole 160 KB of a CU's LDS, so no other
// workgroup that uses LDS runs beside it.  Transposing LDS reads of one
// workgroup overlapping another workgroup's LDS staging on the same CU gave
// results that differed between identical runs: with two workgroups of the
// 128 x 128 combine per CU, about a thousand elements of X' per launch of
// 512 tiles (8 x 1024^2) while its inputs were the same bit for bit.  Probe
// copies of the kernel, two workgroups per CU, repeat exactly with the main
// loop alone, with the epilogue alone, with an 800 us pause between the two
// phases, and with plain 16-byte reads of both operands in the main loop;
// they differ in every repeat only when the transposing reads of one
// workgroup meet the other's epilogue.  Every LDS address of both phases lies
// inside the workgroup's own arrays.  The 128 x 128 tiles also run the
// four-buffer ring (four separate arrays, so that the compiler can tell the
// stages apart).
template <int BM, int BN, bool LAST, bool XTERM, bool UPD = false>
__global__ __launch_bounds__((GemmT<BM, BN>::NT), 1) void k_combine_bf16(StepArgs a, const Tile* __restrict__ tiles, int ntiles,
                                                      int src_x, int dst_x, int first, Coeffs cf) {
  constexpr bool last = LAST;
  using G = GemmT<BM, BN>;
  using C = CombT<BM, BN>;
  constexpr int NB = (BM == 128 && BN == 128) ? 4 : 2;
  static_assert(NB == 2 || 4 * C::RB * 2 <= 163840, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint16_t ring0[C::RB];
  __shared__ __attribute__((aligned(16))) uint16_t ring1[C::RB];
  __shared__ __attribute__((aligned(16))) uint16_t ring2[NB == 4 ? C::RB : 8];
  __shared__ __attribute__((aligned(16))) uint16_t ring3[NB == 4 ? C::RB : 8];
  // The rest of the CU's LDS (the factor array below included; 64 bytes
  // left for alignment).
  constexpr int kUsed = (NB == 4 ? 4 * C::RB : 2 * C::RB + 16) * 2 + (LAST ? BM + BN : 1) * 4;
  __shared__ __attribute__((aligned(16))) volatile uint32_t lds_rest[(163840 - 64 - kUsed) / 4];
  const Tile t = tiles[xcd_remap(blockIdx.x, ntiles)];
  const MatDesc& d = a.desc[t.mat];
  const uint16_t* Bm = reinterpret_cast<const uint16_t*>(a.ws + d.b_off);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.ws + d.x_off[2 * src_x]);
  const int64_t gi0 = static_cast<int64_t>(t.ti) * BM, gj0 = static_cast<int64_t>(t.tj) * BN;
  f32x16_t acc[G::MS][G::NS];
#pragma unroll
  for (int s = 0; s < G::MS; ++s)
#pragma unroll
    for (int u = 0; u < G::NS; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][u][r] = 0.0f;
  // B X, with X read k-major: its rows are the product's k.
  if constexpr (!XTERM && NB == 4)
    mma_bf16<BM, BN, true, false, 0, 4>(Bm + gi0 * d.KP, d.KP, X + gj0, d.NP, d.KP, ring0, ring1, acc, false, ring2, ring3);
  else if constexpr (!XTERM)
    mma_bf16<BM, BN, true>(Bm + gi0 * d.KP, d.KP, X + gj0, d.NP, d.KP, ring0, ring1, acc);

  const float alpha = first ? a.scal[d.scal_idx].inv_nu : 1.0f;
  const bool partials = LAST && a.dimuon;
  const MUON_GLOBAL float* dgr = gmem(reinterpret_cast<const float*>(a.ws + (d.tall ? d.dc_off : d.dr_off)));
  const MUON_GLOBAL float* dgc = gmem(reinterpret_cast<const float*>(a.ws + (d.tall ? d.dr_off : d.dc_off)));
  // X' (row-major, NP) while iterating; on the last iteration Z, bf16 like
  // every iterate (the norm partials below take the fp32 values), in the
  // caller's orientation: row-major for wide, transposed for tall.
  void* dst_n = last ? (d.tall ? nullptr : a.ws + d.z_off) : a.ws + d.x_off[2 * dst_x];
  void* dst_t = last && d.tall ? a.ws + d.z_off : nullptr;
  constexpr int32_t odt = DT_BF16;
  // Muon (the UPD variant of the last combine), matrices flagged fuse_upd
  // (bf16 W, rows of whole 8-element runs): it applies W <- W - lr (s O + wd W) itself, with O the last
  // iterate rounded to bf16 as Z would be stored, so the result is the one
  // the separate update pass gives.  Z is then not written.  W's 8-element
  // runs are fetched ahead of the staging, as operands; the same run in the
  // caller's layout is a row run for a wide matrix and a column run (down
  // the Gram side) for a tall one.
  static_assert(!UPD || (LAST && !XTERM), "the update rides on the last product");
  const bool upd = UPD && d.fuse_upd;
  auto w_idx = [&](int64_t wr, int64_t wc) { return (wr < d.m && wc < d.n) ? wr * d.n + wc : int64_t(-1); };
  auto update8 = [&](float (&v)[8], const uint4& wq, int64_t at) {
    if (at < 0) return;
    float w[8], o[8];
    unpack8_bf16(wq, w);
    unpack8_bf16(make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])), o);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = __builtin_fmaf(d.update_scale, o[e], a.weight_decay * w[e]);
      w[e] = __builtin_fmaf(-a.lr, u, w[e]);
    }
    store8(d.w, at, DT_BF16, w);
    if (d.o_out) store8(d.o_out, at, DT_F32, o);
  };
  float sz = 0.0f, sp = 0.0f;
  // Dimuon's norm partials: sum of v^2 and of (fr v fc)^2 over the tile, with
  // fr, fc the factors of the Gram orientation's rows and columns (the factor
  // arrays are zero in the padding).
  // The tile's row factors, then its column factors, staged in LDS once
  // before the epilogue (published by its first barrier) instead of being
  // fetched in every staging round (rows beyond the Gram side: zero).
  __shared__ float fac[LAST ? BM + BN : 1];
  if (LAST && partials)
    for (int e = threadIdx.x; e < BM + BN; e += G::NT)
      fac[e] = e < BM ? (gi0 + e < d.KP ? dgr[gi0 + e] : 0.0f) : dgc[gj0 + e - BM];
  auto factors8 = [&](int at, float (&r)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = fac[at + e];
  };
  auto accum = [&](float fr, float v, float fc) {
    const float p = (fr * v) * fc;
    sz = sz + v * v;
    sp = sp + p * p;
  };
  // XTERM only: row runs read X, column runs read eight values down a column
  // of X (zero iterations only).
  auto aux_t = [&](int j, int i0) {
    if constexpr (XTERM) {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = gmem(X)[(gi0 + i0 + e) * d.NP + gj0 + j];
      return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    } else {
      const int64_t at = upd ? w_idx(gj0 + j, gi0 + i0) : int64_t(-1);
      return at >= 0 ? fetch8_bf16(static_cast<const uint16_t*>(d.w), at) : make_uint4(0, 0, 0, 0);
    }
  };
  auto aux_n = [&](int i, int j0) {
    if constexpr (XTERM) {
      return fetch8_bf16(X, (gi0 + i) * d.NP + gj0 + j0);
    } else {
      const int64_t at = upd ? w_idx(gi0 + i, gj0 + j0) : int64_t(-1);
      return at >= 0 ? fetch8_bf16(static_cast<const uint16_t*>(d.w), at) : make_uint4(0, 0, 0, 0);
    }
  };
  auto fin = [&](float (&v)[8], const uint4& aux) {
    float x[8];
    unpack8_bf16(aux, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = XTERM ? alpha * (cf.a * x[e]) : alpha * v[e];
  };
  // Tile rows at or beyond the Gram side (a tile of a list whose rows are
  // padded to 256) hold no part of the result: on the last iteration they
  // are neither stored nor summed.  The side is a multiple of 128, so an
  // 8-row run lies wholly on one side of it.
  auto out_t = [&](int j, int i0, float (&v)[8], const uint4& aux) {
    if (LAST && gi0 + i0 >= d.KP) return;
    fin(v, aux);
    if (LAST && partials) {
      float fr[8];
      factors8(i0, fr);
      const float fc = fac[BM + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) accum(fr[e], v[e], fc);
    }
    if (upd) update8(v, aux, w_idx(gj0 + j, gi0 + i0));
    else store8(dst_t, (gj0 + j) * d.KP + gi0 + i0, odt, v);
  };
  auto out_n = [&](int i, int j0, float (&v)[8], const uint4& aux) {
    if (LAST && gi0 + i >= d.KP) return;
    fin(v, aux);
    if (LAST && partials) {
      float fc[8];
      factors8(BM + j0, fc);
      const float fr = fac[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) accum(fr, v[e], fc[e]);
    }
    if (upd) update8(v, aux, w_idx(gi0 + i, gj0 + j0));
    else store8(dst_n, (gi0 + i) * d.NP + gj0 + j0, odt, v);
  };
  auto stage = [&](int rd) { return reinterpret_cast<float*>(rd & 1 ? ring1 : ring0); };
  if constexpr (UPD || XTERM) {
    // One of the two kinds of runs; operands (W, or X for XTERM) fetched a
    // round ahead.
    if (dst_t)
      staged_epilogue<BM, BN, C::R, true, 0, true>(acc, stage, true, false, aux_t, aux_n, out_t, out_n);
    else
      staged_epilogue<BM, BN, C::R, true, 0, true>(acc, stage, false, true, aux_t, aux_n, out_t, out_n);
  } else {
    staged_epilogue<BM, BN, C::R, true>(acc, stage, dst_t != nullptr, dst_n != nullptr, aux_t, aux_n, out_t, out_n);
  }
  if (LAST && partials) {
    // The staging arrays are free once every wave has left the epilogue.
    __syncthreads();
    float* red = reinterpret_cast<float*>(ring0);
    sz = block_sum<G::NW>(sz, red);
    sp = block_sum<G::NW>(sp, red);
    // One pair per 128 x 128 sub-tile (a matrix's tiles may mix sizes): the
    // tile's sums go to its first sub-tile, zeros to the others.
    // (Sub-tiles below the Gram side only: a padded tile's last rows have none.)
    if (threadIdx.x < (BM / 128) * (BN / 128)) {
      float* pz = reinterpret_cast<float*>(a.ws + d.pz_off);
      const int sa = threadIdx.x / (BN / 128), sb = threadIdx.x % (BN / 128);
      const int rs = t.ti * (BM / 128) + sa;
      if (rs < d.KP / 128) {
        const int idx = rs * (d.NP / 128) + t.tj * (BN / 128) + sb;
        pz[2 * idx] = threadIdx.x == 0 ? sz : 0.0f;
        pz[2 * idx + 1] = threadIdx.x == 0 ? sp : 0.0f;
      }
    }
  }
  if (ntiles < 0) lds_rest[0] = 0u;   // never taken; keeps lds_rest allocated
}

// ---------------------------------------------------------------------------
// fp32 path (ns dtype F32): the same products on the matrix cores in fp32
// (v_mfma_f32_32x32x2f32: fp32 operands, fp32 accumulation), 128 x 128
// tiles, four waves.  The main loop is the bf16 one: a stage holds 32 k
// of each row (the same 128 bytes), and every 16-byte fragment read feeds
// four products instead of one.  Both operands are read k-contiguous
// ("NT"): the fp32 iterates keep X^T beside X, and the combine multiplies B
// by rows of X^T.  The aX term stays in the combine (aX + BX).
// ---------------------------------------------------------------------------
constexpr int FT = 128;

// Eight consecutive fp32 values.
struct F8 {
  float4 lo, hi;
};
__device__ __forceinline__ F8 fetch8_f32(const float* p, int64_t idx) {
  const MUON_GLOBAL float4* q = reinterpret_cast<const MUON_GLOBAL float4*>(gmem(p) + idx);
  return F8{q[0], q[1]};
}
__device__ __forceinline__ void unpack8_f32(const F8& u, float (&v)[8]) {
  v[0] = u.lo.x; v[1] = u.lo.y; v[2] = u.lo.z; v[3] = u.lo.w;
  v[4] = u.hi.x; v[5] = u.hi.y; v[6] = u.hi.z; v[7] = u.hi.w;
}

// fp32 operands as the main loop's 16-bit units (two per float).
__device__ __forceinline__ const uint16_t* units(const float* p) { return reinterpret_cast<const uint16_t*>(p); }

template <int KIND>
__global__ __launch_bounds__((GemmT<FT, FT>::NT), 1) void k_syrk_f32(StepArgs a, const Tile* __restrict__ tiles,
                                                                   int ntiles, int src_x, int first, Coeffs cf) {
  using G = GemmT<FT, FT>;
  __shared__ typename G::Smem sm;
  const Tile t = tiles[xcd_remap(blockIdx.x, ntiles)];
  const MatDesc& d = a.desc[t.mat];
  const float* P = reinterpret_cast<const float*>(a.ws + (KIND == 0 ? d.x_off[2 * src_x] : d.a_off));
  const int64_t ld = KIND == 0 ? d.NP : d.KP;
  f32x16_t acc[G::MS][G::NS];
#pragma unroll
  for (int s = 0; s < G::MS; ++s)
#pragma unroll
    for (int u = 0; u < G::NS; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][u][r] = 0.0f;
  mma_bf16<FT, FT, false, true>(units(P + static_cast<int64_t>(t.ti) * FT * ld), 2 * ld,
                                units(P + static_cast<int64_t>(t.tj) * FT * ld), 2 * ld, static_cast<int>(2 * ld),
                                sm.buf[0], sm.buf[1], acc, t.ti == t.tj);

  // Gram: A = X X^T / nu^2 on the first iteration; polynomial: c (A A) + b A.
  const float alpha = (KIND == 0) ? (first ? a.scal[d.scal_idx].inv_nu2 : 1.0f) : cf.c;
  const float* E = reinterpret_cast<const float*>(a.ws + d.a_off);
  void* dst = a.ws + (KIND == 0 ? d.a_off : d.b_off);
  const int64_t gi0 = static_cast<int64_t>(t.ti) * FT, gj0 = static_cast<int64_t>(t.tj) * FT;
  const int64_t ldo = d.KP;
  auto aux_t = [&](int j, int i0) { return KIND == 1 ? fetch8_f32(E, (gj0 + j) * ldo + gi0 + i0) : F8{}; };
  auto aux_n = [&](int i, int j0) { return KIND == 1 ? fetch8_f32(E, (gi0 + i) * ldo + gj0 + j0) : F8{}; };
  auto fin = [&](float (&v)[8], const F8& aux) {
    float e8[8];
    unpack8_f32(aux, e8);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = KIND == 1 ? alpha * v[e] + cf.b * e8[e] : alpha * v[e];
  };
  auto out_t = [&](int j, int i0, float (&v)[8], const F8& aux) {
    fin(v, aux);
    store8(dst, (gj0 + j) * ldo + gi0 + i0, DT_F32, v);
  };
  auto out_n = [&](int i, int j0, float (&v)[8], const F8& aux) {
    fin(v, aux);
    store8(dst, (gi0 + i) * ldo + gj0 + j0, DT_F32, v);
  };
  staged_epilogue<FT, FT, 2, false>(acc, [&](int) { return sm.st; }, true, t.ti != t.tj, aux_t, aux_n, out_t, out_n);
}

// X' = alpha (a X + B X) (product = 0: alpha a X).  Writes X' and X'^T while
// iterating; on the last iteration Z in the caller's orientation and
// Dimuon's norm partials, one pair per 128 x 128 tile.
template <bool LAST>
__global__ __launch_bounds__((GemmT<FT, FT>::NT), 1) void k_combine_f32(StepArgs a, const Tile* __restrict__ tiles,
                                                                      int ntiles, int src_x, int dst_x, int first,
                                                                      int product, Coeffs cf) {
  using G = GemmT<FT, FT>;
  __shared__ typename G::Smem sm;
  __shared__ float red[G::NW];
  const Tile t = tiles[xcd_remap(blockIdx.x, ntiles)];
  const MatDesc& d = a.desc[t.mat];
  const float* Bm = reinterpret_cast<const float*>(a.ws + d.b_off);
  const float* X = reinterpret_cast<const float*>(a.ws + d.x_off[2 * src_x]);
  const float* XT = reinterpret_cast<const float*>(a.ws + d.x_off[2 * src_x + 1]);
  const int64_t gi0 = static_cast<int64_t>(t.ti) * FT, gj0 = static_cast<int64_t>(t.tj) * FT;
  f32x16_t acc[G::MS][G::NS];
#pragma unroll
  for (int s = 0; s < G::MS; ++s)
#pragma unroll
    for (int u = 0; u < G::NS; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][u][r] = 0.0f;
  // B X: rows of B against rows of X^T (both k-contiguous, K = KP).
  if (product)
    mma_bf16<FT, FT, false, true>(units(Bm + gi0 * d.KP), 2 * d.KP, units(XT + gj0 * d.KP), 2 * d.KP,
                                  static_cast<int>(2 * d.KP), sm.buf[0], sm.buf[1], acc, false);

  const float alpha = first ? a.scal[d.scal_idx].inv_nu : 1.0f;
  const bool partials = LAST && a.dimuon;
  const MUON_GLOBAL float* dgr = gmem(reinterpret_cast<const float*>(a.ws + (d.tall ? d.dc_off : d.dr_off)));
  const MUON_GLOBAL float* dgc = gmem(reinterpret_cast<const float*>(a.ws + (d.tall ? d.dr_off : d.dc_off)));
  void* dst_n = LAST ? (d.tall ? nullptr : a.ws + d.z_off) : a.ws + d.x_off[2 * dst_x];
  void* dst_t = LAST ? (d.tall ? a.ws + d.z_off : nullptr) : a.ws + d.x_off[2 * dst_x + 1];
  float sz = 0.0f, sp = 0.0f;
  // Row runs read X, column runs X^T: the a X term of each element.
  auto aux_t = [&](int j, int i0) { return fetch8_f32(XT, (gj0 + j) * d.KP + gi0 + i0); };
  auto aux_n = [&](int i, int j0) { return fetch8_f32(X, (gi0 + i) * d.NP + gj0 + j0); };
  auto fin = [&](float (&v)[8], const F8& aux) {
    float x[8];
    unpack8_f32(aux, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = alpha * (cf.a * x[e] + v[e]);
  };
  auto factors8 = [&](const MUON_GLOBAL float* f, int64_t at, float (&r)[8]) {
    const float4 lo = *reinterpret_cast<const MUON_GLOBAL float4*>(f + at);
    const float4 hi = *reinterpret_cast<const MUON_GLOBAL float4*>(f + at + 4);
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  };
  auto accum = [&](float fr, float v, float fc) {
    const float p = (fr * v) * fc;
    sz = sz + v * v;
    sp = sp + p * p;
  };
  // On the last iteration each element is stored once: the row run when the
  // caller's matrix is wide, the column run when it is tall; its partials
  // are summed there.
  auto out_t = [&](int j, int i0, float (&v)[8], const F8& aux) {
    fin(v, aux);
    if (LAST && partials) {
      float fr[8];
      factors8(dgr, gi0 + i0, fr);
      const float fc = dgc[gj0 + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) accum(fr[e], v[e], fc);
    }
    store8(dst_t, (gj0 + j) * d.KP + gi0 + i0, DT_F32, v);
  };
  auto out_n = [&](int i, int j0, float (&v)[8], const F8& aux) {
    fin(v, aux);
    if (LAST && partials) {
      float fc[8];
      factors8(dgc, gj0 + j0, fc);
      const float fr = dgr[gi0 + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) accum(fr, v[e], fc[e]);
    }
    store8(dst_n, (gi0 + i) * d.NP + gj0 + j0, DT_F32, v);
  };
  staged_epilogue<FT, FT, 2, false>(acc, [&](int) { return sm.st; }, dst_t != nullptr, dst_n != nullptr, aux_t,
                                    aux_n, out_t, out_n);
  if (LAST && partials) {
    __syncthreads();
    sz = block_sum<G::NW>(sz, red);
    sp = block_sum<G::NW>(sp, red);
    if (threadIdx.x == 0) {
      float* pz = reinterpret_cast<float*>(a.ws + d.pz_off);
      const int idx = t.ti * (d.NP / FT) + t.tj;
      pz[2 * idx] = sz;
      pz[2 * idx + 1] = sp;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.  bt / bm, bn: tile sides of the list (128 or 256; fp32 always 128).
// A bf16 128 x 128 symmetric-product list with no more tiles than the GPU
// has CUs (a partial round split off a big-tile list, or a small batch) runs
// one workgroup per CU anyway, so it takes the deep ring: on the 8 x 4096^2
// set those launches went from 47.6 to about 41.6 us (Gram and polynomial
// about 1% faster per step, bit-identical results).  The 128 x 128 combine
// always runs it (see k_combine_bf16).
// ---------------------------------------------------------------------------
constexpr int kDeepMaxTiles = 256;
hipError_t launch_syrk(const StepArgs& a, const Tile* tiles, int n, int bt, int kind, int src_x, bool first,
                       Coeffs cf, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int f = first ? 1 : 0;
  if (a.ns_dt != DT_BF16) {
    if (bt != FT) return hipErrorInvalidValue;
    if (kind == 0)
      hipLaunchKernelGGL(k_syrk_f32<0>, dim3(n), dim3(GemmT<FT, FT>::NT), 0, s, a, tiles, n, src_x, f, cf);
    else
      hipLaunchKernelGGL(k_syrk_f32<1>, dim3(n), dim3(GemmT<FT, FT>::NT), 0, s, a, tiles, n, src_x, f, cf);
    return hipGetLastError();
  }
#define MUON_SYRK(BT, K, ...) \
  hipLaunchKernelGGL((k_syrk_bf16<BT, K, ##__VA_ARGS__>), dim3(n), dim3(GemmT<BT, BT, kSyrkWC<BT>>::NT), 0, s, a, tiles, n, \
                     src_x, f, cf)
  if (bt == 256) {
    if (kind == 0) MUON_SYRK(256, 0); else MUON_SYRK(256, 1);
  } else if (bt == 128 && n <= kDeepMaxTiles) {
    if (kind == 0) MUON_SYRK(128, 0, 4); else MUON_SYRK(128, 1, 4);
  } else if (bt == 128) {
    if (kind == 0) MUON_SYRK(128, 0); else MUON_SYRK(128, 1);
  } else {
    return hipErrorInvalidValue;
  }
#undef MUON_SYRK
  return hipGetLastError();
}

hipError_t launch_combine(const StepArgs& a, const Tile* tiles, int n, int bm, int bn, int src_x, int dst_x,
                          bool first, bool last, bool product, Coeffs cf, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int f = first ? 1 : 0, l = last ? 1 : 0, p = product ? 1 : 0;
  if (a.ns_dt != DT_BF16) {
    if (bm != FT || bn != FT) return hipErrorInvalidValue;
    if (last)
      hipLaunchKernelGGL(k_combine_f32<true>, dim3(n), dim3(GemmT<FT, FT>::NT), 0, s, a, tiles, n, src_x, dst_x, f, p, cf);
    else
      hipLaunchKernelGGL(k_combine_f32<false>, dim3(n), dim3(GemmT<FT, FT>::NT), 0, s, a, tiles, n, src_x, dst_x, f, p, cf);
    return hipGetLastError();
  }
#define MUON_COMB(BM, BN)                                                                                   \
  if (!product) {                                                                                            \
    if (!last) return hipErrorInvalidValue;                                                                  \
    hipLaunchKernelGGL((k_combine_bf16<BM, BN, true, true>), dim3(n), dim3(GemmT<BM, BN>::NT), 0, s, a, tiles, n, src_x,   \
                       dst_x, f, cf);                                                                        \
  } else if (last && !a.dimuon) {                                                                            \
    hipLaunchKernelGGL((k_combine_bf16<BM, BN, true, false, true>), dim3(n), dim3(GemmT<BM, BN>::NT), 0, s, a, tiles, n, \
                       src_x, dst_x, f, cf);                                                                 \
  } else if (last) {                                                                                         \
    hipLaunchKernelGGL((k_combine_bf16<BM, BN, true, false>), dim3(n), dim3(GemmT<BM, BN>::NT), 0, s, a, tiles, n, src_x,  \
                       dst_x, f, cf);                                                                        \
  } else {                                                                                                   \
    hipLaunchKernelGGL((k_combine_bf16<BM, BN, false, false>), dim3(n), dim3(GemmT<BM, BN>::NT), 0, s, a, tiles, n, src_x, \
                       dst_x, f, cf);                                                                        \
  }
  if (bm == 256 && bn == 256) {
    MUON_COMB(256, 256)
  } else if (bm == 128 && bn == 256) {
    MUON_COMB(128, 256)
  } else if (bm == 256 && bn == 128) {
    MUON_COMB(256, 128)
  } else if (bm == 128 && bn == 128) {
    MUON_COMB(128, 128)
  } else {
    return hipErrorInvalidValue;
  }
#undef MUON_COMB
  return hipGetLastError();
}

}  // namespace muon
