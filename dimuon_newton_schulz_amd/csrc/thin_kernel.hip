// Single-kernel step for thin matrices (Gram side k <= 32 and N within the
// per-thread capacity: N <= 512 * CAP / KP, CAP = 32 floats for KP <= 2 and
// 64 otherwise, KP = k rounded up to a power of two),
// e.g. LoRA factors.  One 512-thread workgroup per matrix reads G, M_{t-1}
// and W once and writes M_t and W once; everything else stays on chip.
//
// With X_0 = Y / ||Y||_F and A_0 = X_0 X_0^T (k x k), every iterate of
//   X <- aX + b(XX^T)X + c(XX^T)^2 X  =  (aI + bA + cA^2) X
// is X_t = Q_t X_0 with Q_{t+1} = M_t Q_t, M_t = aI + bA_t + cA_t^2 and
// A_{t+1} = X_{t+1} X_{t+1}^T = M_t A_t M_t.  So the five iterations run on
// k x k matrices (in fp64, in LDS) after one reduction over the long side,
// and Z = (Q_5 / ||Y||) Y is applied at the end.  This is the same
// polynomial of X_0 as the iteration on k x N matrices, evaluated in a
// different order; its accuracy is set by the fp64 Gram accumulation.
//
// The float32 energies follow the stated pairwise tree: positions are dealt
// to threads in aligned runs (VEC consecutive long indices per chunk, chunk
// c = tid + 512 q), so in-thread pairs, the wave butterfly, the 8 waves and
// the chunk blocks q are successive levels of one tree.
#pragma clang fp contract(off)

#include <utility>

#include "common.h"

namespace muon {

constexpr int TT = 512;  // threads per workgroup

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

// Access to the thread's values: element (a, l) of the Gram orientation.
// Wide: runs of VEC along l for a fixed a.  Tall: runs of KP along a for a
// fixed l (one position per chunk).
// CAP: floats of one matrix a thread holds (KP * VEC * NQ).
template <int KP, bool TALL>
struct ThinShape {
  static constexpr int CAP = KP <= 2 ? 32 : 64;
  static constexpr int VEC = TALL ? 1 : (CAP / KP < 4 ? CAP / KP : 4);
  static constexpr int NQ = CAP / (KP * VEC);
};

template <int KP, bool TALL>
__device__ __forceinline__ void thin_load(const void* p, int32_t dt, int k, int N, int n, bool vec_ok,
                                          float (&v)[ThinShape<KP, TALL>::NQ][KP][ThinShape<KP, TALL>::VEC]) {
  using S = ThinShape<KP, TALL>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < S::NQ; ++q) {
    const int l0 = S::VEC * (tid + TT * q);
    if constexpr (!TALL) {
#pragma unroll
      for (int a = 0; a < KP; ++a) {
        const int avail = (a < k && l0 < N) ? min(S::VEC, N - l0) : 0;
        load_run<S::VEC>(p, dt, static_cast<int64_t>(a) * n + l0, avail, vec_ok, v[q][a]);
      }
    } else {
      float row[KP];
      const int64_t base = static_cast<int64_t>(l0) * n;
      if (l0 < N) {
        if constexpr (KP >= 4) {
#pragma unroll
          for (int a0 = 0; a0 < KP; a0 += 4) {
            const int avail = a0 < k ? min(4, k - a0) : 0;
            float t4[4];
            load_run<4>(p, dt, base + a0, avail, vec_ok, t4);
#pragma unroll
            for (int e = 0; e < 4; ++e) row[a0 + e] = t4[e];
          }
        } else {
#pragma unroll
          for (int a = 0; a < KP; ++a) row[a] = a < k ? load_elem(p, base + a, dt) : 0.0f;
        }
      } else {
#pragma unroll
        for (int a = 0; a < KP; ++a) row[a] = 0.0f;
      }
#pragma unroll
      for (int a = 0; a < KP; ++a) v[q][a][0] = row[a];
    }
  }
}

template <int KP, bool TALL>
__device__ __forceinline__ void thin_store(void* p, int32_t dt, int k, int N, int n, bool vec_ok,
                                           const float (&v)[ThinShape<KP, TALL>::NQ][KP][ThinShape<KP, TALL>::VEC]) {
  using S = ThinShape<KP, TALL>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < S::NQ; ++q) {
    const int l0 = S::VEC * (tid + TT * q);
    if (l0 >= N) continue;
    if constexpr (!TALL) {
#pragma unroll
      for (int a = 0; a < KP; ++a) {
        if (a >= k) continue;
        store_run<S::VEC>(p, dt, static_cast<int64_t>(a) * n + l0, min(S::VEC, N - l0), vec_ok, v[q][a]);
      }
    } else {
      float row[KP];
#pragma unroll
      for (int a = 0; a < KP; ++a) row[a] = v[q][a][0];
      const int64_t base = static_cast<int64_t>(l0) * n;
      if constexpr (KP >= 4) {
#pragma unroll
        for (int a0 = 0; a0 < KP; a0 += 4) {
          const float t4[4] = {row[a0], row[a0 + 1], row[a0 + 2], row[a0 + 3]};
          if (a0 < k) store_run<4>(p, dt, base + a0, min(4, k - a0), vec_ok, t4);
        }
      } else {
#pragma unroll
        for (int a = 0; a < KP; ++a)
          if (a < k) store_elem(p, base + a, dt, row[a]);
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

// Block-wide k x k fp64 product C = X * Y (all KP x KP, row-major in LDS).
template <int KP>
__device__ __forceinline__ void mm64(double* C, const double* X, const double* Y) {
  for (int e = threadIdx.x; e < KP * KP; e += TT) {
    const int r = e / KP, c = e % KP;
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < KP; ++k) s = __builtin_fma(X[r * KP + k], Y[k * KP + c], s);
    C[e] = s;
  }
  __syncthreads();
}

// Pair p of the upper triangle (a <= b), enumerated row by row.
constexpr int pair_a(int kp, int p) {
  int a = 0;
  while (p >= kp - a) { p -= kp - a; ++a; }
  return a;
}
constexpr int pair_b(int kp, int p) {
  int a = 0;
  while (p >= kp - a) { p -= kp - a; ++a; }
  return a + p;
}

template <int KP, int P, int VEC, int NQ>
__device__ __forceinline__ void fma_pair(const float (&y)[NQ][KP][VEC], double& acc) {
  if constexpr (P < KP * (KP + 1) / 2) {
    constexpr int a = pair_a(KP, P), b = pair_b(KP, P);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        acc = __builtin_fma(static_cast<double>(y[q][a][e]), static_cast<double>(y[q][b][e]), acc);
  }
}

template <int KP, int P0, int VEC, int NQ, int GP, int... Is>
__device__ __forceinline__ void fma_group(const float (&y)[NQ][KP][VEC], double (&acc)[GP],
                                          std::integer_sequence<int, Is...>) {
  (fma_pair<KP, P0 + Is, VEC, NQ>(y, acc[Is]), ...);
}

// Gram entries of pairs [G * GP, (G + 1) * GP): per-thread partials, the wave
// butterfly, then the 8 waves in order; written to both triangles of sG.
template <int KP, int VEC, int NQ, int GP, int G, int NGROUP>
__device__ __forceinline__ void gram_groups(const float (&y)[NQ][KP][VEC], double (*red64)[GP], double* sG) {
  if constexpr (G < NGROUP) {
    constexpr int NPAIR = KP * (KP + 1) / 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double acc[GP];
#pragma unroll
    for (int i = 0; i < GP; ++i) acc[i] = 0.0;
    fma_group<KP, G * GP, VEC, NQ, GP>(y, acc, std::make_integer_sequence<int, GP>{});
#pragma unroll
    for (int i = 0; i < GP; ++i) acc[i] = wave_sum_f64(acc[i]);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < GP; ++i) red64[wave][i] = acc[i];
    }
    __syncthreads();
    const int pidx = G * GP + tid;
    if (tid < GP && pidx < NPAIR) {
      double s = 0.0;
#pragma unroll
      for (int w = 0; w < TT / 64; ++w) s = s + red64[w][tid];
      const int a = pair_a(KP, pidx), b = pair_b(KP, pidx);
      sG[a * KP + b] = s;
      sG[b * KP + a] = s;
    }
    __syncthreads();
    gram_groups<KP, VEC, NQ, GP, G + 1, NGROUP>(y, red64, sG);
  }
}

template <int KP, bool TALL>
__global__ __launch_bounds__(TT) void k_thin(StepArgs args, const uint16_t* __restrict__ mats, int ns_steps,
                                              ThinCoeffs cf) {
  using S = ThinShape<KP, TALL>;
  constexpr int NQ = S::NQ, VEC = S::VEC, NW = TT / 64;
  constexpr int NPAIR = KP * (KP + 1) / 2;
  constexpr int GP = NPAIR < 36 ? NPAIR : 36;                 // pairs per reduction group
  constexpr int NGROUP = (NPAIR + GP - 1) / GP;

  __shared__ float red[NW][NQ][KP];
  __shared__ float eglob[KP], dglob[KP];
  __shared__ float fsh[NW];
  __shared__ double red64[NW][GP];
  __shared__ double sA[KP * KP], sA2[KP * KP], sM[KP * KP], sQ[KP * KP], sT[KP * KP], sG[KP * KP];
  __shared__ float sQf[KP * KP];

  const int mat = mats[blockIdx.x];
  const MatDesc& d = args.desc[mat];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = d.k, N = d.N, n = d.n;
  // Vector loads need every run to start on a multiple of its length.
  const bool vec_ok = TALL ? ((n & 3) == 0) : ((n % VEC) == 0);

  float y[NQ][KP][VEC];   // M_{t-1}, then the orthogonaliser input, then Z, then O
  float g[NQ][KP][VEC];   // gradient, then W
  thin_load<KP, TALL>(d.mom, args.mom_dt, k, N, n, vec_ok, y);

  // ---- Dimuon energies of M_{t-1} -----------------------------------------
  float dloc[NQ][VEC];
  const bool dimuon = args.dimuon != 0;
  if (dimuon) {
    float eloc[NQ][VEC];
    float cs[NQ][KP];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float col[KP];
#pragma unroll
        for (int a = 0; a < KP; ++a) col[a] = y[q][a][e] * y[q][a][e];
        eloc[q][e] = tree<KP>(col);
      }
#pragma unroll
      for (int a = 0; a < KP; ++a) {
        float run[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) run[e] = y[q][a][e] * y[q][a][e];
        cs[q][a] = wave_tree_sum(tree<VEC>(run));
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int a = 0; a < KP; ++a) red[wave][q][a] = cs[q][a];
    }
    __syncthreads();
    if (tid < KP) {
      float blk[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float w8[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) w8[w] = red[w][q][tid];
        blk[q] = tree<NW>(w8);
      }
      eglob[tid] = tree<NQ>(blk);
    }
    // local maximum over the valid positions
    float lmax = 0.0f;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (VEC * (tid + TT * q) + e < N) lmax = fmaxf(lmax, eloc[q][e]);
    lmax = wave_max(lmax);
    if (lane == 0) fsh[wave] = lmax;
    __syncthreads();
    float emax_loc = fsh[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) emax_loc = fmaxf(emax_loc, fsh[w]);
    float emax_glob = 0.0f;
    for (int a = 0; a < k; ++a) emax_glob = fmaxf(emax_glob, eglob[a]);
    const bool on = emax_loc > 0.0f && emax_glob > 0.0f;
    if (tid < KP) dglob[tid] = (on && tid < k) ? cond_factor(eglob[tid], emax_glob, args.eps) : 1.0f;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int e = 0; e < VEC; ++e) dloc[q][e] = on ? cond_factor(eloc[q][e], emax_loc, args.eps) : 1.0f;
    if (d.energy_out) {
      // wide: R = global (k rows), C = local (N columns); tall: R = local, C = global.
      float* Rp = d.energy_out;
      float* Cp = d.energy_out + d.m;
      float* glob_out = TALL ? Cp : Rp;
      float* loc_out = TALL ? Rp : Cp;
      if (tid < k) glob_out[tid] = eglob[tid];
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int l = VEC * (tid + TT * q) + e;
          if (l < N) loc_out[l] = eloc[q][e];
        }
    }
  } else {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int e = 0; e < VEC; ++e) dloc[q][e] = 1.0f;
  }

  // ---- momentum ------------------------------------------------------------
  thin_load<KP, TALL>(d.g, args.g_dt, k, N, n, vec_ok, g);
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[q][a][e] = momentum_value(args.mu, y[q][a][e], g[q][a][e], args.mom_dt);
  thin_store<KP, TALL>(d.mom, args.mom_dt, k, N, n, vec_ok, y);
  if (args.nesterov) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int a = 0; a < KP; ++a)
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[q][a][e] = g[q][a][e] + args.mu * y[q][a][e];
  }
  __syncthreads();   // dglob visible
  if (dimuon) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int a = 0; a < KP; ++a)
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[q][a][e] = (dglob[a] * y[q][a][e]) * dloc[q][e];
  }

  // ---- Gram of Y in fp64 -----------------------------------------------------
  gram_groups<KP, VEC, NQ, GP, 0, NGROUP>(y, red64, sG);

  // ---- k x k Newton-Schulz in fp64 ------------------------------------------
  double nu2 = 0.0;
  for (int a = 0; a < KP; ++a) nu2 = nu2 + sG[a * KP + a];
  const double inv_nu = (nu2 == 0.0) ? 0.0 : 1.0 / sqrt(nu2);
  const double inv_nu2 = inv_nu * inv_nu;
  for (int e = tid; e < KP * KP; e += TT) {
    sA[e] = sG[e] * inv_nu2;
    sQ[e] = (e / KP == e % KP) ? 1.0 : 0.0;
  }
  __syncthreads();
  double* A = sA;
  double* A2 = sA2;
  double* Q = sQ;
  double* T = sT;
  for (int t = 0; t < ns_steps; ++t) {
    const double ca = cf.c[t].a, cb = cf.c[t].b, cc = cf.c[t].c;
    mm64<KP>(A2, A, A);
    for (int e = tid; e < KP * KP; e += TT) {
      const double diag = (e / KP == e % KP) ? ca : 0.0;
      sM[e] = diag + cb * A[e] + cc * A2[e];
    }
    __syncthreads();
    mm64<KP>(T, sM, Q);
    double* sw = Q; Q = T; T = sw;
    mm64<KP>(A2, sM, A);
    mm64<KP>(A, A2, sM);
  }
  for (int e = tid; e < KP * KP; e += TT) sQf[e] = static_cast<float>(Q[e] * inv_nu);
  __syncthreads();

  // ---- Z = Qs Y, norm fix, update --------------------------------------------
  // z[.][a][.] = sum_b Qs[a][b] y[.][b][.]: each Qs entry is read once from LDS
  // and applied to all of this thread's positions.
  {
    float z[NQ][KP][VEC];
#pragma unroll
    for (int a = 0; a < KP; ++a) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int e = 0; e < VEC; ++e) z[q][a][e] = 0.0f;
#pragma unroll
      for (int b = 0; b < KP; ++b) {
        const float qab = sQf[a * KP + b];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int e = 0; e < VEC; ++e) z[q][a][e] = __builtin_fmaf(qab, y[q][b][e], z[q][a][e]);
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int a = 0; a < KP; ++a)
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[q][a][e] = z[q][a][e];
  }
  float sz = 0.0f, sp = 0.0f;
  if (dimuon) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int a = 0; a < KP; ++a) {
          const float p = (dglob[a] * y[q][a][e]) * dloc[q][e];
          sz = sz + y[q][a][e] * y[q][a][e];
          sp = sp + p * p;
        }
  }
  thin_load<KP, TALL>(d.w, args.w_dt, k, N, n, vec_ok, g);
  float post = 1.0f;
  if (dimuon) {
    sz = wave_tree_sum(sz);
    sp = wave_tree_sum(sp);
    __syncthreads();
    if (lane == 0) fsh[wave] = sz;
    __syncthreads();
    float tz = fsh[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) tz = tz + fsh[w];
    __syncthreads();
    if (lane == 0) fsh[wave] = sp;
    __syncthreads();
    float tp = fsh[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) tp = tp + fsh[w];
    post = (tp == 0.0f) ? 0.0f : sqrtf(tz) / sqrtf(tp);
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int a = 0; a < KP; ++a)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ov = dimuon ? post * ((dglob[a] * y[q][a][e]) * dloc[q][e]) : y[q][a][e];
        y[q][a][e] = ov;
        const float w = g[q][a][e];
        const float upd = __builtin_fmaf(d.update_scale, ov, args.weight_decay * w);
        g[q][a][e] = __builtin_fmaf(-args.lr, upd, w);
      }
  thin_store<KP, TALL>(d.w, args.w_dt, k, N, n, vec_ok, g);
  if (d.o_out) thin_store<KP, TALL>(d.o_out, DT_F32, k, N, n, vec_ok, y);
}

template <int KP>
static hipError_t launch_thin_kp(const StepArgs& a, const uint16_t* mats, int n, bool tall, int ns_steps,
                                 const ThinCoeffs& cf, hipStream_t s) {
  if (tall)
    hipLaunchKernelGGL((k_thin<KP, true>), dim3(n), dim3(TT), 0, s, a, mats, ns_steps, cf);
  else
    hipLaunchKernelGGL((k_thin<KP, false>), dim3(n), dim3(TT), 0, s, a, mats, ns_steps, cf);
  return hipGetLastError();
}

hipError_t launch_thin(const StepArgs& a, const uint16_t* mats, int n, int kp, bool tall, int ns_steps,
                       const Coeffs* cf, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ThinCoeffs c{};
  for (int t = 0; t < ns_steps && t < kMaxSteps; ++t) c.c[t] = cf[t];
  switch (kp) {
    case 1: return launch_thin_kp<1>(a, mats, n, tall, ns_steps, c, s);
    case 2: return launch_thin_kp<2>(a, mats, n, tall, ns_steps, c, s);
    case 4: return launch_thin_kp<4>(a, mats, n, tall, ns_steps, c, s);
    case 8: return launch_thin_kp<8>(a, mats, n, tall, ns_steps, c, s);
    case 16: return launch_thin_kp<16>(a, mats, n, tall, ns_steps, c, s);
    case 32: return launch_thin_kp<32>(a, mats, n, tall, ns_steps, c, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace muon
