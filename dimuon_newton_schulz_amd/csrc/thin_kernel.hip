// Thin-matrix path (Gram side k <= 32), e.g. LoRA factors.
//
// Each matrix is viewed in its Gram orientation, k x N (a tall matrix is
// read transposed in place).  The long side is cut into S slices of L
// positions, and one 256-thread workgroup handles one slice.  Thread t of
// slice s owns VEC consecutive positions s*L + t*VEC .. +VEC-1 and all KP
// Gram-side rows of them (KP = k rounded up to a power of two,
// KP * VEC = 32), so every thread holds 32 values per array.
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
//   pass A  momentum (stored), energies of the new momentum for the next step,
//           conditioned input Y, per-slice Gram partials (plain and d_loc^2
//           weighted) through LDS.
//   pass B  reduce the partials, k x k iteration (one wave for KP <= 8) while
//           M_t and W are loading, apply Z, Dimuon post-scale with the norm
//           fix computed in Gram space, weight update.
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

#include <utility>

#include "common.h"

namespace muon {

constexpr int TT = 256;          // threads per workgroup (one slice)
constexpr int NWV = TT / 64;     // waves per workgroup

template <int KP>
struct TS {
  static constexpr int VEC = 32 / KP;          // positions per thread
  static constexpr int L = TT * VEC;            // positions per slice
  static constexpr int NPAIR = KP * (KP + 1) / 2;
  static constexpr int C = VEC < 4 ? VEC : 4;   // wide: elements per vector access
  static constexpr int CT = KP < 4 ? KP : 4;    // tall: elements per vector access
};

struct ThinCoeffs {
  Coeffs c[kMaxSteps];
};

template <int CNT>
__device__ __forceinline__ void load_run(const void* p, int32_t dt, int64_t idx, int avail, bool vec_ok,
                                         float* out) {
  if (vec_ok && avail >= CNT) {
    if constexpr (CNT == 4) {
      load4_aligned(p, idx, dt, out);
      return;
    } else if constexpr (CNT == 2) {
      if (dt == DT_F32) {
        const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(p) + idx);
        out[0] = v.x; out[1] = v.y;
      } else {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + idx);
        out[0] = __uint_as_float(v << 16); out[1] = __uint_as_float(v & 0xffff0000u);
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < CNT; ++e) out[e] = (e < avail) ? load_elem(p, idx + e, dt) : 0.0f;
}

template <int CNT>
__device__ __forceinline__ void store_run(void* p, int32_t dt, int64_t idx, int avail, bool vec_ok,
                                          const float* v) {
  if (vec_ok && avail >= CNT) {
    if constexpr (CNT == 4) {
      store4_aligned(p, idx, dt, v);
      return;
    } else if constexpr (CNT == 2) {
      if (dt == DT_F32) {
        *reinterpret_cast<float2*>(static_cast<float*>(p) + idx) = make_float2(v[0], v[1]);
      } else {
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + idx) =
            f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < CNT; ++e)
    if (e < avail) store_elem(p, idx + e, dt, v[e]);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// v[a][e] = element (a, l0 + e) of the Gram orientation; 0 outside k x N.
template <int KP, bool TALL>
__device__ __forceinline__ void slice_load(const void* p, int32_t dt, int k, int N, int n, int l0,
                                           float (&v)[KP][TS<KP>::VEC]) {
  constexpr int VEC = TS<KP>::VEC;
  if constexpr (!TALL) {
    constexpr int C = TS<KP>::C;
    const bool vec_ok = (n % C) == 0;
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e0 = 0; e0 < VEC; e0 += C) {
        const int avail = a < k ? clampi(N - (l0 + e0), 0, C) : 0;
        float t[C];
        load_run<C>(p, dt, static_cast<int64_t>(a) * n + l0 + e0, avail, vec_ok, t);
#pragma unroll
        for (int e = 0; e < C; ++e) v[a][e0 + e] = t[e];
      }
  } else {
    constexpr int C = TS<KP>::CT;
    const bool vec_ok = (n % C) == 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int row = l0 + e;
#pragma unroll
      for (int a0 = 0; a0 < KP; a0 += C) {
        const int avail = row < N ? clampi(k - a0, 0, C) : 0;
        float t[C];
        load_run<C>(p, dt, static_cast<int64_t>(row) * n + a0, avail, vec_ok, t);
#pragma unroll
        for (int i = 0; i < C; ++i) v[a0 + i][e] = t[i];
      }
    }
  }
}

template <int KP, bool TALL>
__device__ __forceinline__ void slice_store(void* p, int32_t dt, int k, int N, int n, int l0,
                                            const float (&v)[KP][TS<KP>::VEC]) {
  constexpr int VEC = TS<KP>::VEC;
  if constexpr (!TALL) {
    constexpr int C = TS<KP>::C;
    const bool vec_ok = (n % C) == 0;
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e0 = 0; e0 < VEC; e0 += C) {
        const int avail = a < k ? clampi(N - (l0 + e0), 0, C) : 0;
        float t[C];
#pragma unroll
        for (int e = 0; e < C; ++e) t[e] = v[a][e0 + e];
        if (avail > 0) store_run<C>(p, dt, static_cast<int64_t>(a) * n + l0 + e0, avail, vec_ok, t);
      }
  } else {
    constexpr int C = TS<KP>::CT;
    const bool vec_ok = (n % C) == 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int row = l0 + e;
#pragma unroll
      for (int a0 = 0; a0 < KP; a0 += C) {
        const int avail = row < N ? clampi(k - a0, 0, C) : 0;
        float t[C];
#pragma unroll
        for (int i = 0; i < C; ++i) t[i] = v[a0 + i][e];
        if (avail > 0) store_run<C>(p, dt, static_cast<int64_t>(row) * n + a0, avail, vec_ok, t);
      }
    }
  }
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

template <int KP>
struct ThinSmem {
  static constexpr int GP = TS<KP>::NPAIR < 36 ? TS<KP>::NPAIR : 36;   // Gram pairs per reduction group
  double gred[NWV * 4][2][GP];     // 16-lane row sums of the Gram partials (wave, row)
  float red[NWV][KP];
  float fred[NWV];
  float rg[KP], dglob[KP];
  double sG[KP * KP], sG2[KP * KP];
  double sA[KP * KP], sA2[KP * KP], sM[KP * KP], sQ[KP * KP], sT[KP * KP];
  double nrm[2];
  float sQf[KP * KP];
  float post;
};

// Sum over each 16-lane row of the wave (the first four pairwise levels);
// lanes 0, 16, 32, 48 then hold the row sums.
template <typename T>
__device__ __forceinline__ T row16_sum(T v) {
  if constexpr (sizeof(T) == 4) {
    v = v + dpp_f32<0xB1>(v);
    v = v + dpp_f32<0x4E>(v);
    v = v + dpp_f32<0x141>(v);
    v = v + dpp_f32<0x140>(v);
  } else {
    v = v + dpp_f64<0xB1>(v);
    v = v + dpp_f64<0x4E>(v);
    v = v + dpp_f64<0x141>(v);
    v = v + dpp_f64<0x140>(v);
  }
  return v;
}

// acc[i] += y_a * y_b and acc2[i] += (y_a w) * y_b for pair G*GP + i of one
// position (pair rows are constants of the instantiation).
template <typename TA, int KP, int P>
__device__ __forceinline__ void pair_acc(const float (&y)[KP], TA w, TA& acc, TA& acc2, bool two) {
  if constexpr (P < TS<KP>::NPAIR) {
    constexpr int a = pair_a(KP, P), b = pair_b(KP, P);
    const TA ya = static_cast<TA>(y[a]), yb = static_cast<TA>(y[b]);
    if constexpr (sizeof(TA) == 4) {
      acc = __builtin_fmaf(ya, yb, acc);
      if (two) acc2 = __builtin_fmaf(ya * w, yb, acc2);
    } else {
      acc = __builtin_fma(ya, yb, acc);
      if (two) acc2 = __builtin_fma(ya * w, yb, acc2);
    }
  }
}

template <typename TA, int KP, int P0, int GP, int... Is>
__device__ __forceinline__ void pair_group(const float (&y)[KP], TA w, TA (&acc)[GP], TA (&acc2)[GP], bool two,
                                           std::integer_sequence<int, Is...>) {
  (pair_acc<TA, KP, P0 + Is>(y, w, acc[Is], acc2[Is], two), ...);
}

// Gram partials of this slice: sum over the slice's positions of y_a y_b
// (and of y_a d_loc^2 y_b when `two`), pairs in groups of GP: per-thread sums
// over its VEC positions in TA, the 16-lane row sums (DPP), then the 16 row
// sums of the 4 waves added in a fixed order in double.
template <typename TA, int KP, int G, int NG>
__device__ __forceinline__ void gram_slice(const float (&y)[KP][TS<KP>::VEC], const float (&dl)[TS<KP>::VEC],
                                           bool two, double* out, double* out2, ThinSmem<KP>& sm) {
  if constexpr (G < NG) {
    constexpr int VEC = TS<KP>::VEC, NPAIR = TS<KP>::NPAIR, GP = ThinSmem<KP>::GP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    TA acc[GP], acc2[GP];
#pragma unroll
    for (int i = 0; i < GP; ++i) { acc[i] = TA(0); acc2[i] = TA(0); }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float col[KP];
#pragma unroll
      for (int a = 0; a < KP; ++a) col[a] = y[a][e];
      const TA w = static_cast<TA>(dl[e]) * static_cast<TA>(dl[e]);
      pair_group<TA, KP, G * GP, GP>(col, w, acc, acc2, two, std::make_integer_sequence<int, GP>{});
    }
#pragma unroll
    for (int i = 0; i < GP; ++i) {
      const TA r1 = row16_sum(acc[i]);
      const TA r2 = two ? row16_sum(acc2[i]) : TA(0);
      if ((lane & 15) == 0) {
        sm.gred[wave * 4 + (lane >> 4)][0][i] = static_cast<double>(r1);
        sm.gred[wave * 4 + (lane >> 4)][1][i] = static_cast<double>(r2);
      }
    }
    __syncthreads();
    for (int i = tid; i < GP; i += TT) {
      const int p = G * GP + i;
      if (p < NPAIR) {
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int r = 0; r < NWV * 4; ++r) {
          s1 = s1 + sm.gred[r][0][i];
          s2 = s2 + sm.gred[r][1][i];
        }
        out[p] = s1;
        if (two) out2[p] = s2;
      }
    }
    __syncthreads();
    gram_slice<TA, KP, G + 1, NG>(y, dl, two, out, out2, sm);
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
      c.pos[l0 + e] = pe;
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
  __syncthreads();
  if (tid < KP) {
    float w4[NWV];
#pragma unroll
    for (int w = 0; w < NWV; ++w) w4[w] = sm.red[w][tid];
    c.part[static_cast<int64_t>(s) * KP + tid] = tree<NWV>(w4);
  }
  if (tid == 0) {
    float m = sm.fred[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) m = fmaxf(m, sm.fred[w]);
    c.smax[s] = m;
  }
  __syncthreads();
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
  slice_load<KP, TALL>(d.mom, args.mom_dt, d.k, d.N, d.n, l0, y);
  energies_to_cache<KP>(y, d, s, l0, cache_of(args, d, parity), sm);
}

template <int KP>
__global__ __launch_bounds__(TT) void k_thin_energy(StepArgs args, const Tile* __restrict__ tiles, int parity) {
  __shared__ ThinSmem<KP> sm;
  const Tile t = tiles[blockIdx.x];
  const MatDesc& d = args.desc[t.mat];
  if (d.tall) energy_body<KP, true>(args, d, t.ti, parity, sm);
  else energy_body<KP, false>(args, d, t.ti, parity, sm);
}

// ---------------------------------------------------------------------------
// Pass A
// ---------------------------------------------------------------------------
template <int KP, bool TALL>
__device__ __forceinline__ void pass_a_body(const StepArgs& args, const MatDesc& d, int s, int parity,
                                            ThinSmem<KP>& sm) {
  constexpr int VEC = TS<KP>::VEC, L = TS<KP>::L, NPAIR = TS<KP>::NPAIR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = d.k, N = d.N, n = d.n;
  const int l0 = s * L + tid * VEC;
  const bool dimuon = args.dimuon != 0;

  float y[KP][VEC];   // M_{t-1}, then M_t, then Y
  float g[KP][VEC];
  slice_load<KP, TALL>(d.mom, args.mom_dt, k, N, n, l0, y);
  slice_load<KP, TALL>(d.g, args.g_dt, k, N, n, l0, g);

  // ---- Dimuon factors from the energies of M_{t-1} --------------------------
  float dloc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) dloc[e] = 1.0f;
  if (dimuon) {
    const EnergyCache cin = cache_of(args, d, parity);
    if (tid < KP) sm.rg[tid] = tid < k ? pairwise_strided(cin.part + tid, d.S, KP) : 0.0f;
    float m = 0.0f;
    for (int i = tid; i < d.S; i += TT) m = fmaxf(m, cin.smax[i]);
    m = wave_max(m);
    if (lane == 0) sm.fred[wave] = m;
    float pe[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) pe[e] = (l0 + e < N) ? cin.pos[l0 + e] : 0.0f;
    __syncthreads();
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
      if (s == 0 && tid < k) glob_out[tid] = sm.rg[tid];
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (l0 + e < N) loc_out[l0 + e] = pe[e];
    }
    __syncthreads();   // dglob visible; rg / fred reads done before reuse
  }

  // ---- momentum; energies of M_t for the next step ---------------------------
#pragma unroll
  for (int a = 0; a < KP; ++a)
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[a][e] = momentum_value(args.mu, y[a][e], g[a][e], args.mom_dt);
  slice_store<KP, TALL>(d.mom, args.mom_dt, k, N, n, l0, y);
  if (dimuon) energies_to_cache<KP>(y, d, s, l0, cache_of(args, d, parity ^ 1), sm);

  // ---- Y = D_glob V D_loc -----------------------------------------------------
  if (args.nesterov) {
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[a][e] = g[a][e] + args.mu * y[a][e];
  }
  if (dimuon) {
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[a][e] = (sm.dglob[a] * y[a][e]) * dloc[e];
    float* tdl = reinterpret_cast<float*>(args.ws + d.tdl_off);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (l0 + e < N) tdl[l0 + e] = dloc[e];
    if (s == 0 && tid < KP) reinterpret_cast<float*>(args.ws + d.tdg_off)[tid] = sm.dglob[tid];
  }

  // ---- Gram partials of the slice ---------------------------------------------
  {
    constexpr int GP = ThinSmem<KP>::GP, NG = (NPAIR + GP - 1) / GP;
    double* tg = reinterpret_cast<double*>(args.ws + d.tg_off) + static_cast<int64_t>(s) * NPAIR;
    double* tg2 = reinterpret_cast<double*>(args.ws + d.tg2_off) + static_cast<int64_t>(s) * NPAIR;
    // The orthogonaliser's precision sets the Gram's: float32 sums when the
    // NS products are bf16, float64 in fp32 mode.
    if (args.ns_dt == DT_BF16) gram_slice<float, KP, 0, NG>(y, dloc, dimuon, tg, tg2, sm);
    else gram_slice<double, KP, 0, NG>(y, dloc, dimuon, tg, tg2, sm);
  }
}

template <int KP>
__global__ __launch_bounds__(TT) void k_thin_a(StepArgs args, const Tile* __restrict__ tiles, int parity) {
  __shared__ ThinSmem<KP> sm;
  const Tile t = tiles[blockIdx.x];
  const MatDesc& d = args.desc[t.mat];
  if (d.tall) pass_a_body<KP, true>(args, d, t.ti, parity, sm);
  else pass_a_body<KP, false>(args, d, t.ti, parity, sm);
}

// ---------------------------------------------------------------------------
// Pass B
// ---------------------------------------------------------------------------
// k x k iteration in fp64 on LDS matrices (all symmetric): A <- G / nu^2,
// Q <- I; per step M = aI + bA + cA^2, Q <- M Q, A <- M A M.  Small KP runs on
// one wave with one entry per lane (a wave's LDS operations complete in
// order, so no block barrier is needed); larger KP uses every wave.
template <int KP>
__device__ __forceinline__ void kxk_wave(ThinSmem<KP>& sm, double inv_nu2, int ns_steps, const ThinCoeffs& cf) {
  const int lane = threadIdx.x & 63;
  const bool own = lane < KP * KP;
  const int r = lane / KP, c = lane % KP;
  double* A = sm.sA;
  double* A2 = sm.sA2;
  double* Q = sm.sQ;
  double* T = sm.sT;
  if (own) {
    A[lane] = sm.sG[lane] * inv_nu2;
    Q[lane] = (r == c) ? 1.0 : 0.0;
  }
  __builtin_amdgcn_wave_barrier();
  for (int t = 0; t < ns_steps; ++t) {
    const double ca = cf.c[t].a, cb = cf.c[t].b, cc = cf.c[t].c;
    if (own) {
      double acc = 0.0;
#pragma unroll
      for (int q = 0; q < KP; ++q) acc = __builtin_fma(A[r * KP + q], A[q * KP + c], acc);
      sm.sM[lane] = ((r == c) ? ca : 0.0) + cb * A[lane] + cc * acc;
    }
    __builtin_amdgcn_wave_barrier();
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
    __builtin_amdgcn_wave_barrier();
    if (own) {
      double a2 = 0.0;
#pragma unroll
      for (int q = 0; q < KP; ++q) a2 = __builtin_fma(A2[r * KP + q], sm.sM[q * KP + c], a2);
      A[lane] = a2;
    }
    double* sw = Q; Q = T; T = sw;
    __builtin_amdgcn_wave_barrier();
  }
  if (own && Q != sm.sQ) sm.sQ[lane] = Q[lane];
  __builtin_amdgcn_wave_barrier();
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
  __syncthreads();
}

template <int KP>
__device__ __forceinline__ void kxk_block(ThinSmem<KP>& sm, double inv_nu2, int ns_steps, const ThinCoeffs& cf) {
  const int tid = threadIdx.x;
  for (int e = tid; e < KP * KP; e += TT) {
    sm.sA[e] = sm.sG[e] * inv_nu2;
    sm.sQ[e] = (e / KP == e % KP) ? 1.0 : 0.0;
  }
  __syncthreads();
  double* A = sm.sA;
  double* A2 = sm.sA2;
  double* Q = sm.sQ;
  double* T = sm.sT;
  for (int t = 0; t < ns_steps; ++t) {
    const double ca = cf.c[t].a, cb = cf.c[t].b, cc = cf.c[t].c;
    mm64<KP>(A2, A, A);
    for (int e = tid; e < KP * KP; e += TT) {
      const double diag = (e / KP == e % KP) ? ca : 0.0;
      sm.sM[e] = diag + cb * A[e] + cc * A2[e];
    }
    __syncthreads();
    mm64<KP>(T, sm.sM, Q);
    double* sw = Q; Q = T; T = sw;
    mm64<KP>(A2, sm.sM, A);
    mm64<KP>(A, A2, sm.sM);
  }
  if (Q != sm.sQ)
    for (int e = tid; e < KP * KP; e += TT) sm.sQ[e] = Q[e];
  __syncthreads();
}

// ||Z||^2 = sum_a (Q G Q^T)_aa / nu^2 and ||D_R Z D_C||^2 = sum_a d_a^2 (Q G2 Q^T)_aa / nu^2
// (Q symmetric).  Thread a < KP computes row a's term with one code path for
// both, so equal Grams and unit weights give bit-equal norms; thread 0 sums
// the KP terms in order.
template <int KP>
__device__ __forceinline__ void gram_norms(ThinSmem<KP>& sm, double inv_nu) {
  const int tid = threadIdx.x;
  double* terms = sm.sT;   // free after the k x k iteration
  if (tid < 2 * KP) {
    const int which = tid / KP, a = tid % KP;
    const double* H = which ? sm.sG2 : sm.sG;
    double da = 0.0;
    for (int c = 0; c < KP; ++c) {
      double t = 0.0;
#pragma unroll 8
      for (int b = 0; b < KP; ++b) t = __builtin_fma(sm.sQ[a * KP + b], H[b * KP + c], t);
      da = __builtin_fma(t, sm.sQ[a * KP + c], da);
    }
    const double w = which ? static_cast<double>(sm.dglob[a]) * static_cast<double>(sm.dglob[a]) : 1.0;
    terms[which * KP + a] = w * (da * inv_nu * inv_nu);
  }
  __syncthreads();
  if (tid < 2) {
    double tot = 0.0;
    for (int a = 0; a < KP; ++a) tot = tot + terms[tid * KP + a];
    sm.nrm[tid] = tot;
  }
  __syncthreads();
}

template <int KP, bool TALL>
__device__ __forceinline__ void pass_b_body(const StepArgs& args, const MatDesc& d, int s, int ns_steps,
                                            const ThinCoeffs& cf, ThinSmem<KP>& sm) {
  constexpr int VEC = TS<KP>::VEC, L = TS<KP>::L, NPAIR = TS<KP>::NPAIR;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int k = d.k, N = d.N, n = d.n;
  const int l0 = s * L + tid * VEC;
  const bool dimuon = args.dimuon != 0;

  // Loads first: they are in flight during the k x k work.
  float y[KP][VEC];   // M_t, then Y, then O
  float w[KP][VEC];   // W
  float g[KP][VEC];   // G (Nesterov only)
  slice_load<KP, TALL>(d.mom, args.mom_dt, k, N, n, l0, y);
  slice_load<KP, TALL>(d.w, args.w_dt, k, N, n, l0, w);
  if (args.nesterov) slice_load<KP, TALL>(d.g, args.g_dt, k, N, n, l0, g);
  float dloc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) dloc[e] = 1.0f;
  if (dimuon) {
    const float* tdl = reinterpret_cast<const float*>(args.ws + d.tdl_off);
#pragma unroll
    for (int e = 0; e < VEC; ++e) dloc[e] = (l0 + e < N) ? tdl[l0 + e] : 1.0f;
    if (tid < KP) sm.dglob[tid] = reinterpret_cast<const float*>(args.ws + d.tdg_off)[tid];
  }

  // ---- Gram: the slice partials summed in slice order -------------------------
  const double* tg = reinterpret_cast<const double*>(args.ws + d.tg_off);
  const double* tg2 = reinterpret_cast<const double*>(args.ws + d.tg2_off);
  for (int p = tid; p < NPAIR; p += TT) {
    double a1 = 0.0, a2 = 0.0;
    for (int i = 0; i < d.S; ++i) {
      a1 = a1 + tg[static_cast<int64_t>(i) * NPAIR + p];
      if (dimuon) a2 = a2 + tg2[static_cast<int64_t>(i) * NPAIR + p];
    }
    const int a = pair_a(KP, p), b = pair_b(KP, p);
    sm.sG[a * KP + b] = a1;
    sm.sG[b * KP + a] = a1;
    sm.sG2[a * KP + b] = a2;
    sm.sG2[b * KP + a] = a2;
  }
  __syncthreads();

  // ---- k x k iteration, norms ----------------------------------------------
  double nu2 = 0.0;
  for (int a = 0; a < KP; ++a) nu2 = nu2 + sm.sG[a * KP + a];
  const double inv_nu = (nu2 == 0.0) ? 0.0 : 1.0 / sqrt(nu2);
  if constexpr (KP <= 8) {
    if (wave == 0) kxk_wave<KP>(sm, inv_nu * inv_nu, ns_steps, cf);
    __syncthreads();
  } else {
    kxk_block<KP>(sm, inv_nu * inv_nu, ns_steps, cf);
  }
  for (int e = tid; e < KP * KP; e += TT) sm.sQf[e] = static_cast<float>(sm.sQ[e] * inv_nu);
  if (dimuon) {
    gram_norms<KP>(sm, inv_nu);
    if (tid == 0) sm.post = (sm.nrm[1] == 0.0) ? 0.0f : static_cast<float>(sqrt(sm.nrm[0]) / sqrt(sm.nrm[1]));
  } else if (tid == 0) {
    sm.post = 1.0f;
  }
  __syncthreads();

  // ---- Y, Z = Qs Y, O, update ------------------------------------------------
  if (args.nesterov) {
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[a][e] = g[a][e] + args.mu * y[a][e];
  }
  if (dimuon) {
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[a][e] = (sm.dglob[a] * y[a][e]) * dloc[e];
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
    }
    const float post = sm.post;
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ov = dimuon ? post * ((sm.dglob[a] * z[a][e]) * dloc[e]) : z[a][e];
        y[a][e] = ov;
        const float upd = __builtin_fmaf(d.update_scale, ov, args.weight_decay * w[a][e]);
        w[a][e] = __builtin_fmaf(-args.lr, upd, w[a][e]);
      }
  }
  slice_store<KP, TALL>(d.w, args.w_dt, k, N, n, l0, w);
  if (d.o_out) slice_store<KP, TALL>(d.o_out, DT_F32, k, N, n, l0, y);
}

template <int KP>
__global__ __launch_bounds__(TT) void k_thin_b(StepArgs args, const Tile* __restrict__ tiles, int ns_steps,
                                                ThinCoeffs cf) {
  __shared__ ThinSmem<KP> sm;
  const Tile t = tiles[blockIdx.x];
  const MatDesc& d = args.desc[t.mat];
  if (d.tall) pass_b_body<KP, true>(args, d, t.ti, ns_steps, cf, sm);
  else pass_b_body<KP, false>(args, d, t.ti, ns_steps, cf, sm);
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

hipError_t launch_thin_a(const StepArgs& a, const Tile* tiles, int n, int kp, int parity, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  MUON_THIN_DISPATCH(k_thin_a, a, tiles, parity)
  return hipGetLastError();
}

hipError_t launch_thin_b(const StepArgs& a, const Tile* tiles, int n, int kp, int ns_steps, const Coeffs* cf,
                         hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ThinCoeffs c{};
  for (int t = 0; t < ns_steps && t < kMaxSteps; ++t) c.c[t] = cf[t];
  MUON_THIN_DISPATCH(k_thin_b, a, tiles, ns_steps, c)
  return hipGetLastError();
}

}  // namespace muon
