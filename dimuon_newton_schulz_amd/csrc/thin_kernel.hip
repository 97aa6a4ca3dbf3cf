// Thin-matrix path (Gram side k <= 32), e.g. LoRA factors.
//
// Each matrix is viewed in its Gram orientation, k x N (a tall matrix is
// read transposed in place).  The long side is cut into S slices of L
// positions, and one 256-thread workgroup handles one slice.  Thread t of
// slice s owns VEC consecutive positions s*L + t*VEC .. +VEC-1 and all KP
// Gram-side rows of them (KP = k rounded up to a power of two,
// KP * VEC = max(16, KP)), so every thread holds 16 values per array up to
// Gram side 16 and 32 at Gram side 32.
//
// Newton-Schulz in Gram space: with X_0 = Y / ||Y||_F and A_0 = X_0 X_0^T,
// every iterate of X <- aX + b(XX^T)X + c(XX^T)^2 X = (aI + bA + cA^2) X
// is X_t = Q_t X_0 with Q_{t+1} = M_t Q_t, M_t = aI + bA_t + cA_t^2 and
// A_{t+1} = M_t A_t M_t.  So one fp64 reduction of the Gram over the long
// side is enough; the iterations run on k x k matrices and Z = (Q_5/||Y||) Y
// is applied per position.  This is the same polynomial of X_0, evaluated in
// a different order.
//
// A step is two launches:
//   pass A  momentum (stored), conditioned input Y, per-slice Gram partials
//           (plain and d_loc^2 weighted).
//   pass B  reduce the partials, k x k iteration (one wave for KP <= 8) while
//           M_t and W are loading, energies of M_t for the next step, apply Z,
//           Dimuon post-scale with the norm fix computed in Gram space,
//           weight update.
// Dimuon's factors come from the energies of M_{t-1}.  The step that wrote
// M_{t-1} left them in the workspace energy cache ("Dimuon: LoRA 에 맞춰 다시
// 짠 Muon", section "왜 「지난」 모멘텀인가", notes that R and C can be computed
// before the new gradient arrives).  Without a cache, k_thin_energy computes
// them from M_{t-1} first.
//
// Energy tree: per position, the pairwise tree over the KP rows (zeros beyond
// k); per row, the tree over the VEC positions of a thread, the wave
// butterfly, the 4 waves, then the S slices; all aligned power-of-two blocks
// of the stated pairwise tree.
#pragma clang fp contract(off)

#include <type_traits>
#include <utility>

#include "common.h"

namespace muon {

constexpr int TT = kThinThreads;   // threads per workgroup (one slice)
constexpr int NWV = TT / 64;       // waves per workgroup

template <int KP>
struct TS {
  static constexpr int VEC = thin_vec(KP);      // positions per thread
  static constexpr int L = thin_slice_len(KP);  // positions per slice
  static constexpr int NPAIR = KP * (KP + 1) / 2;
  static constexpr int C = VEC < 4 ? VEC : 4;   // wide: elements per vector access
  static constexpr int CT = KP < 4 ? KP : 4;    // tall: elements per vector access
};

struct ThinCoeffs {
  Coeffs c[kMaxSteps];
};

// Storage element types: float (f32) and uint16_t (bf16 bits).
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t x) { return bf16_to_f32(x); }
template <typename S>
__device__ __forceinline__ S from_f(float v) {
  if constexpr (sizeof(S) == 4) return v;
  else return f32_to_bf16(v);
}

// C consecutive elements as one aligned access (p aligned to C elements).
template <typename S, int C>
__device__ __forceinline__ void vload(const MUON_GLOBAL S* p, float* out) {
  if constexpr (C == 1) {
    out[0] = to_f(p[0]);
  } else if constexpr (sizeof(S) == 4) {
    if constexpr (C == 4) {
      const float4 v = *reinterpret_cast<const MUON_GLOBAL float4*>(p);
      out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    } else {
      const float2 v = *reinterpret_cast<const MUON_GLOBAL float2*>(p);
      out[0] = v.x; out[1] = v.y;
    }
  } else {
    if constexpr (C == 4) {
      const uint2 v = *reinterpret_cast<const MUON_GLOBAL uint2*>(p);
      out[0] = __uint_as_float(v.x << 16); out[1] = __uint_as_float(v.x & 0xffff0000u);
      out[2] = __uint_as_float(v.y << 16); out[3] = __uint_as_float(v.y & 0xffff0000u);
    } else {
      const uint32_t v = *reinterpret_cast<const MUON_GLOBAL uint32_t*>(p);
      out[0] = __uint_as_float(v << 16); out[1] = __uint_as_float(v & 0xffff0000u);
    }
  }
}

template <typename S, int C>
__device__ __forceinline__ void vstore(MUON_GLOBAL S* p, const float* v) {
  if constexpr (C == 1) {
    p[0] = from_f<S>(v[0]);
  } else if constexpr (sizeof(S) == 4) {
    if constexpr (C == 4) *reinterpret_cast<MUON_GLOBAL float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else *reinterpret_cast<MUON_GLOBAL float2*>(p) = make_float2(v[0], v[1]);
  } else {
    if constexpr (C == 4) {
      uint2 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<MUON_GLOBAL uint2*>(p) = u;
    } else {
      *reinterpret_cast<MUON_GLOBAL uint32_t*>(p) =
          pack_bf16x2(v[0], v[1]);
    }
  }
}

// Index of element (a, l) of the Gram orientation in the caller's row-major m x n array.
template <bool TALL>
__device__ __forceinline__ int64_t gidx(int a, int l, int n) {
  return TALL ? static_cast<int64_t>(l) * n + a : static_cast<int64_t>(a) * n + l;
}

// Elements per vector access of a slice: along the positions (wide) or along
// the Gram-side rows (tall, where a row of the caller's array holds k values).
template <int KP, bool TALL>
constexpr int slice_vec() { return TALL ? TS<KP>::CT : TS<KP>::C; }

// A slice is "full" when all KP rows exist, all its positions are inside N
// and every vector access is aligned; then no access needs a predicate.
template <int KP, bool TALL>
__device__ __forceinline__ bool slice_full(int k, int N, int n, int s) {
  return k == KP && (s + 1) * TS<KP>::L <= N && (n % slice_vec<KP, TALL>()) == 0;
}

// v[a][e] = element (a, l0 + e) of the Gram orientation; 0 outside k x N.
template <int KP, bool TALL, typename S>
__device__ __forceinline__ void slice_load_s(const void* base, int k, int N, int n, int l0, bool full,
                                             float (&v)[KP][TS<KP>::VEC]) {
  constexpr int VEC = TS<KP>::VEC, C = slice_vec<KP, TALL>();
  const MUON_GLOBAL S* p = gmem(static_cast<const S*>(base));
  if (full) {
    // Uniform slice (and row) bases plus 32-bit lane offsets: one offset
    // serves every row, and the loads take their base from scalar registers.
    const int lb = l0 - static_cast<int>(threadIdx.x) * VEC;   // slice start
    const uint32_t lt = threadIdx.x * VEC;
    if constexpr (!TALL) {
#pragma unroll
      for (int a = 0; a < KP; ++a) {
        const MUON_GLOBAL S* row = p + static_cast<int64_t>(a) * n + lb;
#pragma unroll
        for (int e0 = 0; e0 < VEC; e0 += C) vload<S, C>(row + (lt + e0), &v[a][e0]);
      }
    } else {
      const MUON_GLOBAL S* sb = p + static_cast<int64_t>(lb) * n;
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int a0 = 0; a0 < KP; a0 += C) {
          float t[C];
          vload<S, C>(sb + ((lt + e) * static_cast<uint32_t>(n) + a0), t);
#pragma unroll
          for (int i = 0; i < C; ++i) v[a0 + i][e] = t[i];
        }
    }
  } else {
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        v[a][e] = (a < k && l0 + e < N) ? to_f(p[gidx<TALL>(a, l0 + e, n)]) : 0.0f;
  }
}

template <int KP, bool TALL>
__device__ __forceinline__ void slice_load(const void* p, int32_t dt, int k, int N, int n, int l0, bool full,
                                           float (&v)[KP][TS<KP>::VEC]) {
  if (dt == DT_F32) slice_load_s<KP, TALL, float>(p, k, N, n, l0, full, v);
  else slice_load_s<KP, TALL, uint16_t>(p, k, N, n, l0, full, v);
}

template <int KP, bool TALL, typename S>
__device__ __forceinline__ void slice_store_s(void* base, int k, int N, int n, int l0, bool full,
                                              const float (&v)[KP][TS<KP>::VEC]) {
  constexpr int VEC = TS<KP>::VEC, C = slice_vec<KP, TALL>();
  MUON_GLOBAL S* p = gmem(static_cast<S*>(base));
  if (full) {
    const int lb = l0 - static_cast<int>(threadIdx.x) * VEC;   // slice start
    const uint32_t lt = threadIdx.x * VEC;
    if constexpr (!TALL) {
#pragma unroll
      for (int a = 0; a < KP; ++a) {
        MUON_GLOBAL S* row = p + static_cast<int64_t>(a) * n + lb;
#pragma unroll
        for (int e0 = 0; e0 < VEC; e0 += C) vstore<S, C>(row + (lt + e0), &v[a][e0]);
      }
    } else {
      MUON_GLOBAL S* sb = p + static_cast<int64_t>(lb) * n;
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int a0 = 0; a0 < KP; a0 += C) {
          float t[C];
#pragma unroll
          for (int i = 0; i < C; ++i) t[i] = v[a0 + i][e];
          vstore<S, C>(sb + ((lt + e) * static_cast<uint32_t>(n) + a0), t);
        }
    }
  } else {
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (a < k && l0 + e < N) p[gidx<TALL>(a, l0 + e, n)] = from_f<S>(v[a][e]);
  }
}

template <int KP, bool TALL>
__device__ __forceinline__ void slice_store(void* p, int32_t dt, int k, int N, int n, int l0, bool full,
                                            const float (&v)[KP][TS<KP>::VEC]) {
  if (dt == DT_F32) slice_store_s<KP, TALL, float>(p, k, N, n, l0, full, v);
  else slice_store_s<KP, TALL, uint16_t>(p, k, N, n, l0, full, v);
}

// Pairwise tree over CNT in-register values (CNT a power of two).
template <int CNT>
__device__ __forceinline__ float tree(const float* x) {
  if constexpr (CNT == 1) {
    return x[0];
  } else {
    return tree<CNT / 2>(x) + tree<CNT / 2>(x + CNT / 2);
  }
}

// Pair p of the upper triangle (a <= b), enumerated row by row.
__host__ __device__ constexpr int pair_a(int kp, int p) {
  int a = 0;
  while (p >= kp - a) { p -= kp - a; ++a; }
  return a;
}
__host__ __device__ constexpr int pair_b(int kp, int p) {
  int a = 0;
  while (p >= kp - a) { p -= kp - a; ++a; }
  return a + p;
}

// Energy cache of one parity: [S][KP] row partials, [N] per-position
// energies, [S] slice maxima.
struct EnergyCache {
  float* part;
  float* pos;
  float* smax;
};
__device__ __forceinline__ EnergyCache cache_of(const StepArgs& a, const MatDesc& d, int parity) {
  float* base = reinterpret_cast<float*>(a.ws + d.te_off[parity]);
  return {base, base + static_cast<int64_t>(d.S) * d.KP, base + static_cast<int64_t>(d.S) * d.KP + d.N};
}

// Slices up to which pass A uses the matrix-core Gram: four workgroups per
// CU on 256 CUs, the most that run in one round.
constexpr int kThinMfmaGramSlices = 1024;

// Gram sides that take the matrix-core Gram in bf16 mode: below 8 the
// per-thread sums are cheap, and from 16 the fp32 staging would cost both
// passes a workgroup per CU (shared memory).  fp32 mode keeps float64 sums.
template <int KP>
constexpr bool gram_on_mfma() { return KP == 8; }

template <int KP>
struct ThinSmem {
  static constexpr int GP = TS<KP>::NPAIR < 36 ? TS<KP>::NPAIR : 36;   // largest Gram pair group
  static constexpr bool MF = gram_on_mfma<KP>();
  static constexpr int LP = MF ? TT + 4 : 1;                           // staged row length (floats)
  union {
    union {                        // 16-lane row sums of a Gram pass (wave, row)
      double d[NWV * 4][GP];
      float f[NWV * 4][GP];
    } gred;
    float sy[2][KP][LP];                         // matrix-core Gram: Y and d_loc^2 Y rows
    float sred[NWV][MF ? 2 * KP : 1][MF ? KP : 1];   // matrix-core Gram: each wave's [plain; weighted] x plain
  };
  float red[NWV][KP];
  float fred[NWV];
  float rg[KP], dglob[KP];
  double sG[KP * KP], sG2[KP * KP];
  double sAA[2 * KP * KP];         // A and A2 of the k x k iteration; then the norm terms
  double sM[KP * KP], sQ[KP * KP], sT[KP * KP];
  double nrm[2];
  float sQf[KP * KP];
  float post;
};

// 16-lane row sums of CNT values: four DPP levels (quad_perm [1,0,3,2],
// [2,3,0,1], row_half_mirror, row_mirror) leave each 16-lane row's sum in all
// of its lanes.  Values go through the levels four at a time, so that no DPP
// read directly follows the write of its source.
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_add(T v) {
  if constexpr (sizeof(T) == 4) return v + dpp_f32<CTRL>(v);
  else return v + dpp_f64<CTRL>(v);
}

template <typename T, int CNT>
__device__ __forceinline__ void row16_sums(T (&v)[CNT]) {
#pragma unroll
  for (int i0 = 0; i0 < CNT; i0 += 4) {
    constexpr int W = 4;
#pragma unroll
    for (int i = i0; i < i0 + W && i < CNT; ++i) v[i] = dpp_add<0xB1>(v[i]);
#pragma unroll
    for (int i = i0; i < i0 + W && i < CNT; ++i) v[i] = dpp_add<0x4E>(v[i]);
#pragma unroll
    for (int i = i0; i < i0 + W && i < CNT; ++i) v[i] = dpp_add<0x141>(v[i]);
#pragma unroll
    for (int i = i0; i < i0 + W && i < CNT; ++i) v[i] = dpp_add<0x140>(v[i]);
  }
}

// acc += y_a * y_b (or (y_a w) * y_b when WEIGHTED) for pair P of one
// position (the pair's rows are constants of the instantiation).
template <typename TA, int KP, int P, bool WEIGHTED>
__device__ __forceinline__ void pair_acc(const float (&y)[KP], TA w, TA& acc) {
  if constexpr (P < TS<KP>::NPAIR) {
    constexpr int a = pair_a(KP, P), b = pair_b(KP, P);
    const TA ya = WEIGHTED ? static_cast<TA>(y[a]) * w : static_cast<TA>(y[a]);
    const TA yb = static_cast<TA>(y[b]);
    if constexpr (sizeof(TA) == 4) acc = __builtin_fmaf(ya, yb, acc);
    else acc = __builtin_fma(ya, yb, acc);
  }
}

template <typename TA, int KP, int P0, bool WEIGHTED, int GP, int... Is>
__device__ __forceinline__ void pair_group(const float (&y)[KP], TA w, TA (&acc)[GP],
                                           std::integer_sequence<int, Is...>) {
  (pair_acc<TA, KP, P0 + Is, WEIGHTED>(y, w, acc[Is]), ...);
}

// Gram pairs reduced per pass: GP accumulators per thread stay live.
template <int KP, typename TA>
constexpr int gram_group() {
  constexpr int cap = sizeof(TA) == 4 ? 18 : 9;
  return TS<KP>::NPAIR < cap ? TS<KP>::NPAIR : cap;
}

// Pairs [P0, P0 + GP) of the slice's Gram (plain, or d_loc^2 weighted):
// per-thread sums over its VEC positions in TA, the 16-lane row sums (DPP),
// then the 16 row sums of the 4 waves added in a fixed order in double.
template <typename TA, int KP, int P0, bool WEIGHTED>
__device__ __forceinline__ void gram_pass(const float (&y)[KP][TS<KP>::VEC], const float (&dl)[TS<KP>::VEC],
                                          MUON_GLOBAL double* out, ThinSmem<KP>& sm) {
  constexpr int VEC = TS<KP>::VEC, NPAIR = TS<KP>::NPAIR, GP = gram_group<KP, TA>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  TA acc[GP];
#pragma unroll
  for (int i = 0; i < GP; ++i) acc[i] = TA(0);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float col[KP];
#pragma unroll
    for (int a = 0; a < KP; ++a) col[a] = y[a][e];
    const TA w = static_cast<TA>(dl[e]) * static_cast<TA>(dl[e]);
    pair_group<TA, KP, P0, WEIGHTED>(col, w, acc, std::make_integer_sequence<int, GP>{});
  }
  row16_sums(acc);
  if ((lane & 15) == 0) {
    const int row = wave * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < GP; ++i) {
      if constexpr (sizeof(TA) == 4) sm.gred.f[row][i] = acc[i];
      else sm.gred.d[row][i] = acc[i];
    }
  }
  lds_barrier();
  for (int i = tid; i < GP; i += TT) {
    if (P0 + i < NPAIR) {
      double s1 = 0.0;
#pragma unroll
      for (int r = 0; r < NWV * 4; ++r) {
        if constexpr (sizeof(TA) == 4) s1 = s1 + static_cast<double>(sm.gred.f[r][i]);
        else s1 = s1 + sm.gred.d[r][i];
      }
      out[P0 + i] = s1;
    }
  }
  lds_barrier();
}

// Gram partials of this slice, pair groups G.. of both Grams (the weighted
// one when `two`).
template <typename TA, int KP, int G, int NG>
__device__ __forceinline__ void gram_slice(const float (&y)[KP][TS<KP>::VEC], const float (&dl)[TS<KP>::VEC],
                                           bool two, MUON_GLOBAL double* out, MUON_GLOBAL double* out2,
                                           ThinSmem<KP>& sm) {
  if constexpr (G < NG) {
    constexpr int P0 = G * gram_group<KP, TA>();
    gram_pass<TA, KP, P0, false>(y, dl, out, sm);
    if (two) gram_pass<TA, KP, P0, true>(y, dl, out2, sm);
    gram_slice<TA, KP, G + 1, NG>(y, dl, two, out, out2, sm);
  }
}

typedef float tf32x4_t __attribute__((ext_vector_type(4)));

// The slice's Gram partials on the matrix cores (Gram side 8, bf16 mode):
// both Grams are one product over the slice's positions,
//   [Y; D^2 Y] (2KP x L) times Y^T (L x KP),   D = diag(d_loc),
// in fp32 (v_mfma_f32_16x16x4_f32: products exact, sums in fp32, like the
// per-thread sums it replaces).  Y and D^2 Y are staged in LDS as rows
// (padded by 16 bytes against bank conflicts), one position per thread per
// round (VEC rounds, so the staging takes the LDS of 256 positions); each
// wave multiplies a quarter of a round's positions, and the four waves'
// results are added in double at the end.  In a group of four products,
// lane l supplies operand row (l mod 16) at positions 4 (l / 16) .. + 3 of the
// group's 16, one per product, so every position meets itself in both
// operands exactly once.
template <int KP>
__device__ __forceinline__ void gram_slice_mfma(const float (&v)[KP][TS<KP>::VEC], const float (&dl)[TS<KP>::VEC],
                                                bool two, MUON_GLOBAL double* out, MUON_GLOBAL double* out2,
                                                ThinSmem<KP>& sm) {
  constexpr int VEC = TS<KP>::VEC, NPAIR = TS<KP>::NPAIR;
  constexpr int PW = TT / NWV;   // positions per wave and round
  static_assert(KP == 8, "one 16-row product: [plain; weighted]");
  static_assert(PW % 16 == 0, "slice geometry");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, kq = lane >> 4;
  const float* pa = i < KP ? sm.sy[0][i] : sm.sy[1][i - KP];
  const float* pb = sm.sy[0][i % KP];
  tf32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    if (e > 0) lds_barrier();   // the previous round's reads are done
#pragma unroll
    for (int a = 0; a < KP; ++a) {
      sm.sy[0][a][tid] = v[a][e];
      if (two) sm.sy[1][a][tid] = v[a][e] * (dl[e] * dl[e]);
    }
    lds_barrier();
#pragma unroll
    for (int g = 0; g < PW / 16; ++g) {
      const int p = wave * PW + g * 16 + kq * 4;
      const float4 fb = *reinterpret_cast<const float4*>(pb + p);
      const float4 fa = *reinterpret_cast<const float4*>(pa + p);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.x, fb.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.y, fb.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.z, fb.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.w, fb.w, acc, 0, 0, 0);
    }
  }
  lds_barrier();   // every wave's staging reads are done: sred may overwrite them
  // Accumulator r of lane l is entry (4 (l / 16) + r, l mod 16).
  if (i < KP) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.sred[wave][4 * kq + r][i] = acc[r];
  }
  lds_barrier();
  for (int p = tid; p < NPAIR; p += TT) {
    const int a = pair_a(KP, p), b = pair_b(KP, p);
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      s1 = s1 + static_cast<double>(sm.sred[w][a][b]);
      s2 = s2 + static_cast<double>(sm.sred[w][KP + a][b]);
    }
    out[p] = s1;
    if (two) out2[p] = s2;
  }
}

// Energies of the stored values v (per position, per row) into cache c for slice s.
template <int KP>
__device__ __forceinline__ void energies_to_cache(const float (&v)[KP][TS<KP>::VEC], const MatDesc& d, int s,
                                                  int l0, EnergyCache c, ThinSmem<KP>& sm) {
  constexpr int VEC = TS<KP>::VEC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float lmax = 0.0f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float col[KP];
#pragma unroll
    for (int a = 0; a < KP; ++a) col[a] = v[a][e] * v[a][e];
    const float pe = tree<KP>(col);
    if (l0 + e < d.N) {
      gmem(c.pos)[l0 + e] = pe;
      lmax = fmaxf(lmax, pe);
    }
  }
#pragma unroll
  for (int a = 0; a < KP; ++a) {
    float run[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) run[e] = v[a][e] * v[a][e];
    const float r = wave_tree_sum(tree<VEC>(run));
    if (lane == 0) sm.red[wave][a] = r;
  }
  lmax = wave_max(lmax);
  if (lane == 0) sm.fred[wave] = lmax;
  lds_barrier();
  if (tid < KP) {
    float w4[NWV];
#pragma unroll
    for (int w = 0; w < NWV; ++w) w4[w] = sm.red[w][tid];
    gmem(c.part)[static_cast<int64_t>(s) * KP + tid] = tree<NWV>(w4);
  }
  if (tid == 0) {
    float m = sm.fred[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) m = fmaxf(m, sm.fred[w]);
    gmem(c.smax)[s] = m;
  }
  lds_barrier();
}

// ---------------------------------------------------------------------------
// Energies of M_{t-1} (no cached energies available).
// ---------------------------------------------------------------------------
template <int KP, bool TALL>
__device__ __forceinline__ void energy_body(const StepArgs& args, const MatDesc& d, int s, int parity,
                                            ThinSmem<KP>& sm) {
  constexpr int VEC = TS<KP>::VEC, L = TS<KP>::L;
  const int l0 = s * L + threadIdx.x * VEC;
  float y[KP][VEC];
  slice_load<KP, TALL>(d.mom, args.mom_dt, d.k, d.N, d.n, l0, slice_full<KP, TALL>(d.k, d.N, d.n, s), y);
  energies_to_cache<KP>(y, d, s, l0, cache_of(args, d, parity), sm);
}

// Workgroups are dealt round-robin to the 8 XCDs; each XCD takes a
// contiguous run of the slice list instead, so that the slices of a matrix
// share an L2 (pass B's workgroups each read every slice's Gram partials of
// their matrix, pass A's the matrix's cached row energies).
__device__ __forceinline__ int slice_of_block() {
  const int n = static_cast<int>(gridDim.x), bid = static_cast<int>(blockIdx.x);
  const int q = n >> 3, r = n & 7, xcd = bid & 7, idx = bid >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
}

template <int KP>
__global__ __launch_bounds__(TT) void k_thin_energy(StepArgs args, const Tile* __restrict__ tiles, int parity) {
  __shared__ ThinSmem<KP> sm;
  const Tile t = tiles[slice_of_block()];
  const MatDesc& d = args.desc[t.mat];
  if (d.tall) energy_body<KP, true>(args, d, t.ti, parity, sm);
  else energy_body<KP, false>(args, d, t.ti, parity, sm);
}

// ---------------------------------------------------------------------------
// Pass A
// ---------------------------------------------------------------------------
// Pass A of a slice.  On return y holds M_t (stored), g the gradient,
// dloc and sm.dglob the Dimuon factors (also written to the workspace for
// pass B).  TA: accumulation type of the per-thread Gram sums.
template <int KP, bool TALL, typename TA, bool MFG>
__device__ __forceinline__ void pass_a_core(const StepArgs& args, const MatDesc& d, int s, int parity,
                                            ThinSmem<KP>& sm, bool full, float (&y)[KP][TS<KP>::VEC],
                                            float (&g)[KP][TS<KP>::VEC], float (&dloc)[TS<KP>::VEC]) {
  constexpr int VEC = TS<KP>::VEC, L = TS<KP>::L, NPAIR = TS<KP>::NPAIR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = d.k, N = d.N, n = d.n;
  const int l0 = s * L + tid * VEC;
  const bool dimuon = args.dimuon != 0;

  // The energy cache loads go first: the factors are computed while the
  // slice is still loading.
  const EnergyCache cin = cache_of(args, d, parity);
  float part8[8], smax = 0.0f, pe[VEC];
  if (dimuon) {
#pragma unroll
    for (int j = 0; j < 8; ++j) part8[j] = (tid < k && j < d.S) ? gmem(cin.part)[j * KP + tid] : 0.0f;
    if (tid < d.S) smax = gmem(cin.smax)[tid];   // S <= TT
#pragma unroll
    for (int e = 0; e < VEC; ++e) pe[e] = (l0 + e < N) ? gmem(cin.pos)[l0 + e] : 0.0f;
    // Every wave's cache loads are issued before any slice load of the
    // workgroup (the barrier waits for issue, not for data).
    __builtin_amdgcn_s_barrier();
  }

  slice_load<KP, TALL>(d.mom, args.mom_dt, k, N, n, l0, full, y);   // M_{t-1}, then M_t
  slice_load<KP, TALL>(d.g, args.g_dt, k, N, n, l0, full, g);

  // ---- Dimuon factors from the energies of M_{t-1} --------------------------
#pragma unroll
  for (int e = 0; e < VEC; ++e) dloc[e] = 1.0f;
  if (dimuon) {
    if (tid < KP) sm.rg[tid] = tid < k ? pairwise_strided8(part8, cin.part + tid, d.S, KP) : 0.0f;
    const float m = wave_max(smax);
    if (lane == 0) sm.fred[wave] = m;
    lds_barrier();
    float emax_loc = sm.fred[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) emax_loc = fmaxf(emax_loc, sm.fred[w]);
    float emax_glob = 0.0f;
    for (int a = 0; a < k; ++a) emax_glob = fmaxf(emax_glob, sm.rg[a]);
    const bool on = emax_loc > 0.0f && emax_glob > 0.0f;
    if (tid < KP) sm.dglob[tid] = (on && tid < k) ? cond_factor(sm.rg[tid], emax_glob, args.eps) : 1.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dloc[e] = on ? cond_factor(pe[e], emax_loc, args.eps) : 1.0f;
    if (d.energy_out) {
      // wide: R = Gram-side (k rows), C = per position (N); tall: R per position, C Gram-side.
      float* glob_out = d.tall ? d.energy_out + d.m : d.energy_out;
      float* loc_out = d.tall ? d.energy_out : d.energy_out + d.m;
      if (s == 0 && tid < k) gmem(glob_out)[tid] = sm.rg[tid];
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (l0 + e < N) gmem(loc_out)[l0 + e] = pe[e];
    }
    lds_barrier();   // dglob visible; rg / fred reads done before reuse
  }

  // ---- momentum ----------------------------------------------------------------
#pragma unroll
  for (int a = 0; a < KP; ++a)
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[a][e] = momentum_value(args.mu, y[a][e], g[a][e], args.mom_dt);
  slice_store<KP, TALL>(d.mom, args.mom_dt, k, N, n, l0, full, y);

  // ---- Y = D_glob V D_loc (V = M_t, or G + mu M_t with Nesterov) -----------
  float v[KP][VEC];
#pragma unroll
  for (int a = 0; a < KP; ++a)
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[a][e] = args.nesterov ? g[a][e] + args.mu * y[a][e] : y[a][e];
  if (dimuon) {
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[a][e] = (sm.dglob[a] * v[a][e]) * dloc[e];
    MUON_GLOBAL float* tdl = gmem(reinterpret_cast<float*>(args.ws + d.tdl_off));
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (l0 + e < N) tdl[l0 + e] = dloc[e];
    if (s == 0 && tid < KP) gmem(reinterpret_cast<float*>(args.ws + d.tdg_off))[tid] = sm.dglob[tid];
  }

  // ---- Gram partials of the slice ---------------------------------------------
  {
    constexpr int GP = gram_group<KP, TA>(), NG = (NPAIR + GP - 1) / GP;
    MUON_GLOBAL double* tg = gmem(reinterpret_cast<double*>(args.ws + d.tg_off)) + static_cast<int64_t>(s) * NPAIR;
    MUON_GLOBAL double* tg2 = gmem(reinterpret_cast<double*>(args.ws + d.tg2_off)) + static_cast<int64_t>(s) * NPAIR;
    if constexpr (MFG) gram_slice_mfma<KP>(v, dloc, dimuon, tg, tg2, sm);
    else gram_slice<TA, KP, 0, NG>(v, dloc, dimuon, tg, tg2, sm);
  }
}

// The orthogonaliser's precision sets the Gram's: float32 sums in bf16 mode
// (on the matrix cores for Gram sides 8 and 16), float64 per-thread sums in
// fp32 mode.
template <int KP, bool TALL, typename TA, bool MFG>
__device__ __forceinline__ void pass_a_body(const StepArgs& args, const MatDesc& d, int s, int parity,
                                            ThinSmem<KP>& sm) {
  constexpr int VEC = TS<KP>::VEC;
  float y[KP][VEC], g[KP][VEC], dloc[VEC];
  pass_a_core<KP, TALL, TA, MFG>(args, d, s, parity, sm, slice_full<KP, TALL>(d.k, d.N, d.n, s), y, g, dloc);
}

// MFG: the slice's Gram on the matrix cores (bf16 mode, Gram side 8).
template <int KP, typename TA, bool MFG>
__global__ __launch_bounds__(TT, 4) void k_thin_a(StepArgs args, const Tile* __restrict__ tiles, int parity) {
  static_assert(!MFG || (sizeof(TA) == 4 && gram_on_mfma<KP>()), "matrix-core Gram: bf16 mode, Gram side 8");
  __shared__ ThinSmem<KP> sm;
  const Tile t = tiles[slice_of_block()];
  const MatDesc& d = args.desc[t.mat];
  if (d.tall) pass_a_body<KP, true, TA, MFG>(args, d, t.ti, parity, sm);
  else pass_a_body<KP, false, TA, MFG>(args, d, t.ti, parity, sm);
}

// ---------------------------------------------------------------------------
// Pass B
// ---------------------------------------------------------------------------
// Orders the LDS accesses of one wave (a wave's LDS operations complete in
// order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// k x k iteration in fp64 on LDS matrices (all symmetric): A <- G / nu^2,
// Q <- I; per step M = aI + bA + cA^2, Q <- M Q, A <- M A M.  Small KP runs on
// one wave with one entry per lane (a wave's LDS operations complete in
// order, so no block barrier is needed); larger KP uses every wave.
template <int KP>
__device__ __forceinline__ void kxk_wave(ThinSmem<KP>& sm, double inv_nu2, int ns_steps, const ThinCoeffs& cf) {
  const int lane = threadIdx.x & 63;
  const bool own = lane < KP * KP;
  const int r = lane / KP, c = lane % KP;
  double* A = sm.sAA;
  double* A2 = sm.sAA + KP * KP;
  double* Q = sm.sQ;
  double* T = sm.sT;
  if (own) {
    A[lane] = sm.sG[lane] * inv_nu2;
    Q[lane] = (r == c) ? 1.0 : 0.0;
  }
  wave_lds_sync();
  for (int t = 0; t < ns_steps; ++t) {
    const double ca = cf.c[t].a, cb = cf.c[t].b, cc = cf.c[t].c;
    if (own) {
      double acc = 0.0;
#pragma unroll
      for (int q = 0; q < KP; ++q) acc = __builtin_fma(A[r * KP + q], A[q * KP + c], acc);
      sm.sM[lane] = ((r == c) ? ca : 0.0) + cb * A[lane] + cc * acc;
    }
    wave_lds_sync();
    if (own) {
      double q1 = 0.0, t2 = 0.0;
#pragma unroll
      for (int q = 0; q < KP; ++q) {
        q1 = __builtin_fma(sm.sM[r * KP + q], Q[q * KP + c], q1);
        t2 = __builtin_fma(sm.sM[r * KP + q], A[q * KP + c], t2);
      }
      T[lane] = q1;
      A2[lane] = t2;
    }
    wave_lds_sync();
    if (own) {
      double a2 = 0.0;
#pragma unroll
      for (int q = 0; q < KP; ++q) a2 = __builtin_fma(A2[r * KP + q], sm.sM[q * KP + c], a2);
      A[lane] = a2;
    }
    double* sw = Q; Q = T; T = sw;
    wave_lds_sync();
  }
  if (own && Q != sm.sQ) sm.sQ[lane] = Q[lane];
  wave_lds_sync();
}

template <int KP>
__device__ __forceinline__ void mm64(double* C, const double* X, const double* Y) {
  for (int e = threadIdx.x; e < KP * KP; e += TT) {
    const int r = e / KP, c = e % KP;
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < KP; ++q) s = __builtin_fma(X[r * KP + q], Y[q * KP + c], s);
    C[e] = s;
  }
  lds_barrier();
}

template <int KP>
__device__ __forceinline__ void kxk_block(ThinSmem<KP>& sm, double inv_nu2, int ns_steps, const ThinCoeffs& cf) {
  const int tid = threadIdx.x;
  for (int e = tid; e < KP * KP; e += TT) {
    sm.sAA[e] = sm.sG[e] * inv_nu2;
    sm.sQ[e] = (e / KP == e % KP) ? 1.0 : 0.0;
  }
  lds_barrier();
  double* A = sm.sAA;
  double* A2 = sm.sAA + KP * KP;
  double* Q = sm.sQ;
  double* T = sm.sT;
  for (int t = 0; t < ns_steps; ++t) {
    const double ca = cf.c[t].a, cb = cf.c[t].b, cc = cf.c[t].c;
    mm64<KP>(A2, A, A);
    for (int e = tid; e < KP * KP; e += TT) {
      const double diag = (e / KP == e % KP) ? ca : 0.0;
      sm.sM[e] = diag + cb * A[e] + cc * A2[e];
    }
    lds_barrier();
    mm64<KP>(T, sm.sM, Q);
    double* sw = Q; Q = T; T = sw;
    mm64<KP>(A2, sm.sM, A);
    mm64<KP>(A, A2, sm.sM);
  }
  if (Q != sm.sQ)
    for (int e = tid; e < KP * KP; e += TT) sm.sQ[e] = Q[e];
  lds_barrier();
}

// ||Z||^2 = sum_a (Q G Q^T)_aa / nu^2 and ||D_R Z D_C||^2 = sum_a d_a^2 (Q G2 Q^T)_aa / nu^2.
// Entry (a, c) of each product term t_ac = (Q H)_ac Q_ac is one thread's;
// row a's terms are then summed in order, and the rows in order.  Both norms
// take the same code path, so equal Grams and unit weights give bit-equal
// norms.
template <int KP>
__device__ __forceinline__ void gram_norms(ThinSmem<KP>& sm, double inv_nu) {
  const int tid = threadIdx.x;
  double* terms = sm.sAA;   // free after the k x k iteration
  for (int e = tid; e < 2 * KP * KP; e += TT) {
    const int which = e / (KP * KP), a = (e / KP) % KP, c = e % KP;
    const double* H = which ? sm.sG2 : sm.sG;
    double t = 0.0;
#pragma unroll
    for (int b = 0; b < KP; ++b) t = __builtin_fma(sm.sQ[a * KP + b], H[b * KP + c], t);
    terms[e] = t * sm.sQ[a * KP + c];
  }
  lds_barrier();
  double* rows = sm.sM;
  if (tid < 2 * KP) {
    const int which = tid / KP, a = tid % KP;
    double r = 0.0;
    for (int c = 0; c < KP; ++c) r = r + terms[tid * KP + c];
    const double w = which ? static_cast<double>(sm.dglob[a]) * static_cast<double>(sm.dglob[a]) : 1.0;
    rows[tid] = w * (r * inv_nu * inv_nu);
  }
  lds_barrier();
  if (tid < 2) {
    double tot = 0.0;
    for (int a = 0; a < KP; ++a) tot = tot + rows[tid * KP + a];
    sm.nrm[tid] = tot;
  }
  lds_barrier();
}

// The end of pass B, once sm.sQ holds Q_5 and sm.sG, sm.sG2 the Grams: the
// norm fix, the energies of M_t (in y) for the next step, Z = (Q/nu) Y, O
// and the update of W (in w).  dg is d_glob[tid] for tid < KP.
template <int KP, bool TALL>
__device__ __forceinline__ void pass_b_tail(const StepArgs& args, const MatDesc& d, int s, int parity,
                                            ThinSmem<KP>& sm, bool full, double inv_nu, float dg,
                                            float (&y)[KP][TS<KP>::VEC], float (&w)[KP][TS<KP>::VEC],
                                            const float (&g)[KP][TS<KP>::VEC], const float (&dloc)[TS<KP>::VEC]) {
  constexpr int VEC = TS<KP>::VEC, L = TS<KP>::L;
  const int tid = threadIdx.x;
  const int k = d.k, N = d.N, n = d.n;
  const int l0 = s * L + tid * VEC;
  const bool dimuon = args.dimuon != 0;
  for (int e = tid; e < KP * KP; e += TT) sm.sQf[e] = static_cast<float>(sm.sQ[e] * inv_nu);
  if (tid < KP) sm.dglob[tid] = dg;   // read after the next barrier
  if (dimuon) {
    gram_norms<KP>(sm, inv_nu);
    if (tid == 0) sm.post = (sm.nrm[1] == 0.0) ? 0.0f : static_cast<float>(sqrt(sm.nrm[0]) / sqrt(sm.nrm[1]));
  } else if (tid == 0) {
    sm.post = 1.0f;
  }
  lds_barrier();

  // O = post D_g Z D_l with Z = (Q / nu) Y and Y = D_g V D_l (V = M_t, or
  // G + mu M_t with Nesterov), i.e. O = (post D_g (Q / nu) D_g) V D_l^2: the
  // k x k factor is scaled once here and each element takes one product.
  // (Published to the workgroup by the energies' barriers; without Dimuon
  // the factor is Q / nu itself.)
  if (dimuon)
    for (int e = tid; e < KP * KP; e += TT) {
      const int a = e / KP, b = e % KP;
      sm.sQf[e] = sm.post * (sm.dglob[a] * (sm.sQf[e] * sm.dglob[b]));
    }

  // ---- energies of M_t for the next step's conditioning --------------------
  if (dimuon) energies_to_cache<KP>(y, d, s, l0, cache_of(args, d, parity ^ 1), sm);

  // ---- V, O = (post D_g Q D_g / nu) V D_l^2, update --------------------------
  if (args.nesterov) {
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[a][e] = g[a][e] + args.mu * y[a][e];
  }
  {
    float z[KP][VEC];
#pragma unroll
    for (int a = 0; a < KP; ++a) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) z[a][e] = 0.0f;
#pragma unroll
      for (int b = 0; b < KP; ++b) {
        const float qab = sm.sQf[a * KP + b];
#pragma unroll
        for (int e = 0; e < VEC; ++e) z[a][e] = __builtin_fmaf(qab, y[b][e], z[a][e]);
      }
      // One row of Q live at a time (all rows hoisted would take KP^2 registers).
      if constexpr (KP >= 8) __builtin_amdgcn_sched_barrier(0);
    }
    float dl2[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) dl2[e] = dloc[e] * dloc[e];
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ov = dimuon ? z[a][e] * dl2[e] : z[a][e];
        y[a][e] = ov;
        const float upd = __builtin_fmaf(d.update_scale, ov, args.weight_decay * w[a][e]);
        w[a][e] = __builtin_fmaf(-args.lr, upd, w[a][e]);
      }
  }
  slice_store<KP, TALL>(d.w, args.w_dt, k, N, n, l0, full, w);
  if (d.o_out) slice_store<KP, TALL>(d.o_out, DT_F32, k, N, n, l0, full, y);
}

template <int KP, bool TALL>
__device__ __forceinline__ void pass_b_body(const StepArgs& args, const MatDesc& d, int s, int ns_steps,
                                            const ThinCoeffs& cf, int parity, ThinSmem<KP>& sm) {
  constexpr int VEC = TS<KP>::VEC, L = TS<KP>::L, NPAIR = TS<KP>::NPAIR;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int k = d.k, N = d.N, n = d.n;
  const int l0 = s * L + tid * VEC;
  const bool dimuon = args.dimuon != 0;

  // The k x k work waits only on the Gram partials; the slice stays in flight
  // meanwhile.  For KP <= 8 the partials and the iteration belong to wave 0,
  // which runs them before issuing its own share of the slice loads (a wave
  // issues in order, and issuing loads stalls while the memory queue is
  // full); for larger KP every thread loads its partials first.
  const MUON_GLOBAL double* tg = gmem(reinterpret_cast<const double*>(args.ws + d.tg_off));
  const MUON_GLOBAL double* tg2 = gmem(reinterpret_cast<const double*>(args.ws + d.tg2_off));
  constexpr int PB = 8;   // partial loads in flight per thread and round
  double v1[PB], v2[PB];
  auto load_partials = [&](int p, int i0) {
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const bool in = p < NPAIR && i0 + j < d.S;
      const int64_t at = static_cast<int64_t>(i0 + j) * NPAIR + p;
      v1[j] = in ? tg[at] : 0.0;
      v2[j] = (in && dimuon) ? tg2[at] : 0.0;
    }
  };
  // Sums the partials of pairs tid, tid + TT, ... in slice order into sG, sG2;
  // the first round of pair tid is already in v1, v2.
  auto sum_partials = [&]() {
    for (int p = tid; p < NPAIR; p += TT) {
      double a1 = 0.0, a2 = 0.0;
      for (int i0 = 0; i0 < d.S; i0 += PB) {
        if (i0 > 0 || p != tid) load_partials(p, i0);
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          a1 = a1 + v1[j];
          a2 = a2 + v2[j];
        }
      }
      const int a = pair_a(KP, p), b = pair_b(KP, p);
      sm.sG[a * KP + b] = a1;
      sm.sG[b * KP + a] = a1;
      sm.sG2[a * KP + b] = a2;
      sm.sG2[b * KP + a] = a2;
    }
  };
  auto inv_norm = [&]() {
    double nu2 = 0.0;
    for (int a = 0; a < KP; ++a) nu2 = nu2 + sm.sG[a * KP + a];
    return (nu2 == 0.0) ? 0.0 : 1.0 / sqrt(nu2);
  };

  if constexpr (KP <= 8) {
    // Wave 0's partial loads are issued before any slice load of the
    // workgroup (the barrier waits for issue, not for data), so that they
    // travel ahead of the slice traffic.
    if (wave == 0) load_partials(tid, 0);
    __builtin_amdgcn_s_barrier();
    if (wave == 0) {
      sum_partials();
      wave_lds_sync();
      const double in0 = inv_norm();
      kxk_wave<KP>(sm, in0 * in0, ns_steps, cf);
    }
  } else {
    load_partials(tid, 0);
  }

  const float dg = (dimuon && tid < KP) ? gmem(reinterpret_cast<const float*>(args.ws + d.tdg_off))[tid] : 1.0f;
  float y[KP][VEC];   // M_t, then Y, then O
  float w[KP][VEC];   // W
  float g[KP][VEC];   // G (Nesterov only)
  const bool full = slice_full<KP, TALL>(k, N, n, s);
  slice_load<KP, TALL>(d.mom, args.mom_dt, k, N, n, l0, full, y);
  slice_load<KP, TALL>(d.w, args.w_dt, k, N, n, l0, full, w);
  if (args.nesterov) slice_load<KP, TALL>(d.g, args.g_dt, k, N, n, l0, full, g);
  float dloc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) dloc[e] = 1.0f;
  if (dimuon) {
    const MUON_GLOBAL float* tdl = gmem(reinterpret_cast<const float*>(args.ws + d.tdl_off));
#pragma unroll
    for (int e = 0; e < VEC; ++e) dloc[e] = (l0 + e < N) ? tdl[l0 + e] : 1.0f;
  }

  if constexpr (KP > 8) {
    sum_partials();
    lds_barrier();
    const double in0 = inv_norm();
    kxk_block<KP>(sm, in0 * in0, ns_steps, cf);
  } else {
    lds_barrier();
  }
  pass_b_tail<KP, TALL>(args, d, s, parity, sm, full, inv_norm(), dg, y, w, g, dloc);
}

template <int KP>
__global__ __launch_bounds__(TT) void k_thin_b(StepArgs args, const Tile* __restrict__ tiles, int ns_steps,
                                                ThinCoeffs cf, int parity) {
  __shared__ ThinSmem<KP> sm;
  const Tile t = tiles[slice_of_block()];
  const MatDesc& d = args.desc[t.mat];
  if (d.tall) pass_b_body<KP, true>(args, d, t.ti, ns_steps, cf, parity, sm);
  else pass_b_body<KP, false>(args, d, t.ti, ns_steps, cf, parity, sm);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
#define MUON_THIN_DISPATCH(KERNEL, ...)                                                      \
  switch (kp) {                                                                              \
    case 1: hipLaunchKernelGGL(KERNEL<1>, dim3(n), dim3(TT), 0, s, __VA_ARGS__); break;      \
    case 2: hipLaunchKernelGGL(KERNEL<2>, dim3(n), dim3(TT), 0, s, __VA_ARGS__); break;      \
    case 4: hipLaunchKernelGGL(KERNEL<4>, dim3(n), dim3(TT), 0, s, __VA_ARGS__); break;      \
    case 8: hipLaunchKernelGGL(KERNEL<8>, dim3(n), dim3(TT), 0, s, __VA_ARGS__); break;      \
    case 16: hipLaunchKernelGGL(KERNEL<16>, dim3(n), dim3(TT), 0, s, __VA_ARGS__); break;    \
    case 32: hipLaunchKernelGGL(KERNEL<32>, dim3(n), dim3(TT), 0, s, __VA_ARGS__); break;    \
    default: return hipErrorInvalidValue;                                                    \
  }

hipError_t launch_thin_energy(const StepArgs& a, const Tile* tiles, int n, int kp, int parity, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  MUON_THIN_DISPATCH(k_thin_energy, a, tiles, parity)
  return hipGetLastError();
}

template <typename TA>
hipError_t launch_thin_a_t(const StepArgs& a, const Tile* tiles, int n, int kp, int parity, hipStream_t s) {
  switch (kp) {
    case 1: hipLaunchKernelGGL((k_thin_a<1, TA, false>), dim3(n), dim3(TT), 0, s, a, tiles, parity); break;
    case 2: hipLaunchKernelGGL((k_thin_a<2, TA, false>), dim3(n), dim3(TT), 0, s, a, tiles, parity); break;
    case 4: hipLaunchKernelGGL((k_thin_a<4, TA, false>), dim3(n), dim3(TT), 0, s, a, tiles, parity); break;
    case 8:
      // All slices in one round of workgroups: the pass is latency-bound and
      // the matrix-core Gram is shorter.  More slices: throughput-bound, and
      // the per-thread sums cost the matrix pipe nothing.
      if (std::is_same<TA, float>::value && n <= kThinMfmaGramSlices)
        hipLaunchKernelGGL((k_thin_a<8, float, true>), dim3(n), dim3(TT), 0, s, a, tiles, parity);
      else
        hipLaunchKernelGGL((k_thin_a<8, TA, false>), dim3(n), dim3(TT), 0, s, a, tiles, parity);
      break;
    case 16: hipLaunchKernelGGL((k_thin_a<16, TA, false>), dim3(n), dim3(TT), 0, s, a, tiles, parity); break;
    case 32: hipLaunchKernelGGL((k_thin_a<32, TA, false>), dim3(n), dim3(TT), 0, s, a, tiles, parity); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
hipError_t launch_thin_a(const StepArgs& a, const Tile* tiles, int n, int kp, int parity, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (a.ns_dt == DT_BF16) return launch_thin_a_t<float>(a, tiles, n, kp, parity, s);
  return launch_thin_a_t<double>(a, tiles, n, kp, parity, s);
}

hipError_t launch_thin_b(const StepArgs& a, const Tile* tiles, int n, int kp, int ns_steps, const Coeffs* cf,
                         int parity, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ThinCoeffs c{};
  for (int t = 0; t < ns_steps && t < kMaxSteps; ++t) c.c[t] = cf[t];
  MUON_THIN_DISPATCH(k_thin_b, a, tiles, ns_steps, c, parity)
  return hipGetLastError();
}

}  // namespace muon
