// Internal definitions shared by the gfx950 kernels and the host planner.
//
// Layout of one general-path matrix in the workspace (Gram orientation):
// the matrix is viewed as k x N with k = min(m, n) and N = max(m, n);
// a tall matrix (m > n) is stored transposed.  Every workspace matrix is
// padded with zeros to multiples of kPad in both dimensions, and every
// kernel writes whole padded tiles, so the padding stays zero through all
// iterations and the GEMM kernels need no bounds checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

constexpr int kPad = 128;          // padding granularity of workspace matrices
constexpr int kMaxSteps = 32;      // largest ns_steps accepted

// Thin path geometry, shared by the planner and the kernels: one 256-thread
// workgroup per slice of the long side; a thread owns VEC consecutive
// positions of all KP Gram-side rows (KP = k rounded up to a power of two),
// max(16, KP) values per array.
constexpr int kThinThreads = 256;
__host__ __device__ constexpr int thin_vec(int kp) { return (kp < 16 ? 16 : kp) / kp; }
__host__ __device__ constexpr int thin_slice_len(int kp) { return kThinThreads * thin_vec(kp); }

enum DType : int32_t { DT_F32 = 0, DT_BF16 = 1 };

// Per-matrix device descriptor (uploaded once per batch into the workspace).
struct alignas(16) MatDesc {
  const void* g;          // caller: gradient (g dtype), m x n
  void* mom;              // caller: momentum (mom dtype), m x n
  void* w;                // caller: weights (w dtype), m x n
  float* o_out;           // caller, optional: O (f32), m x n
  float* energy_out;      // caller, optional: R (m) then C (n)
  int32_t m, n;           // original shape
  int32_t k, N;           // Gram side and long side
  int32_t KP, NP;         // padded k, N (general path)
  int32_t tall;           // m > n: the Gram orientation is the transpose
  float update_scale;
  int32_t fuse_upd;       // Muon: the last combine applies the weight update (bf16 W, n % 8 == 0)
  int64_t x_off[4];       // X (KP x NP) and X^T (NP x KP, fp32 mode only), ping (0,1) and pong (2,3), ns dtype
  int64_t a_off;          // A = X X^T, KP x KP, ns dtype
  int64_t b_off;          // B = bA + c A A, KP x KP, ns dtype
  int64_t z_off;          // Z (last iterate), KP x NP (transposed for tall), ns dtype
  int64_t dr_off;         // row factors, mpad f32 (zero beyond m)
  int64_t dc_off;         // column factors, npad f32 (zero beyond n)
  int64_t cm_off;         // conditioning chunk maxima [ncond][2] f32 (rows, columns)
  int32_t ncond;          // conditioning chunks of 256 over the padded rows, then columns
  int32_t mpad, npad;     // padded m and n: KP and NP in the caller's orientation
  int64_t ge_off[2];      // energy cache, two parities: row partials [ncb][m] over 64-column blocks,
                          // then column partials [nrb][n] over 64-row blocks, f32
  int64_t pn_off;         // ||Y||^2 partials, one per prescale tile, f32
  int64_t pz_off;         // (||Z||^2, ||P||^2) partials, one pair per 128 x 128 sub-tile of the combine, f32
  int32_t ncb, nrb;       // number of 64-column / 64-row energy blocks
  int32_t n_pn, n_pz;     // partial counts
  int32_t scal_idx;       // index into the per-matrix scalar array
  // Thin path (Gram side <= 32): the long side is cut into S slices of L positions.
  int32_t S, L;
  int64_t te_off[2];      // energy cache, two parities: [S][KP] row partials, [N] per-position
                          // energies, [S] slice maxima (f32)
  int64_t tdl_off;        // per-position factors d_loc [N] f32
  int64_t tdg_off;        // Gram-side factors d_glob [KP] f32
  int64_t tg_off;         // Gram partials [S][KP(KP+1)/2] f64
  int64_t tg2_off;        // d_loc^2-weighted Gram partials [S][KP(KP+1)/2] f64
};

// Per-matrix scalars written on the device during a step.
struct alignas(16) MatScal {
  float inv_nu;           // 1 / ||Y||_F (0 if the norm is 0)
  float inv_nu2;          // inv_nu^2
  float post;             // Dimuon norm fix ||Z|| / ||P|| (1 for Muon)
  float cond_on;          // 1 if the Dimuon factors are active
};

// One work tile: matrix index in the descriptor table and tile coordinates.
struct alignas(8) Tile {
  uint16_t mat, ti, tj, aux;
};

// Coefficients of every iteration, passed by value to the GEMM kernels.
struct Coeffs {
  float a, b, c;
};

// Everything a step's kernels need besides the tile lists.
struct StepArgs {
  const MatDesc* desc;    // device
  MatScal* scal;          // device
  char* ws;               // workspace base (device)
  float mu, lr, eps, weight_decay;
  int32_t g_dt, mom_dt, w_dt, ns_dt;
  int32_t nesterov;
  int32_t dimuon;
};

// --------------------------------------------------------------------------
// Device helpers
// --------------------------------------------------------------------------
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

// Global-memory pointers.  Pointers read from the descriptor table are
// generic, which makes the compiler emit flat accesses; flat accesses also
// count against the LDS counter, so an LDS-only barrier would wait for them.
#if defined(__HIP_DEVICE_COMPILE__)
#define MUON_GLOBAL __attribute__((address_space(1)))
#else
#define MUON_GLOBAL
#endif
template <typename T>
__device__ __forceinline__ MUON_GLOBAL T* gmem(T* p) { return (MUON_GLOBAL T*)(p); }
template <typename T>
__device__ __forceinline__ const MUON_GLOBAL T* gmem(const T* p) { return (const MUON_GLOBAL T*)(p); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (v_cvt_pk_bf16_f32); NaN
// stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats as packed bfloat16 (a in the low half), one conversion.
typedef __bf16 bf16x2_pk_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_pk_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float load_elem(const void* p, int64_t idx, int32_t dt) {
  if (dt == DT_F32) return gmem(static_cast<const float*>(p))[idx];
  return bf16_to_f32(gmem(static_cast<const uint16_t*>(p))[idx]);
}

__device__ __forceinline__ void store_elem(void* p, int64_t idx, int32_t dt, float v) {
  if (dt == DT_F32) gmem(static_cast<float*>(p))[idx] = v;
  else gmem(static_cast<uint16_t*>(p))[idx] = f32_to_bf16(v);
}

// Value a tensor of dtype dt holds after storing v.
__device__ __forceinline__ float round_to(float v, int32_t dt) {
  if (dt == DT_F32) return v;
  return bf16_to_f32(f32_to_bf16(v));
}

// Correctly rounded storage of a double: round to float32 with
// round-to-odd, then to the dtype with round-to-nearest-even.  Round-to-odd
// to 24 bits keeps enough information for the final rounding to 8 bits to
// equal the direct rounding of d, which plain RNE-then-RNE does not.
__device__ __forceinline__ float round_from_f64(double d, int32_t dt) {
  float f = static_cast<float>(d);
  if (dt == DT_F32) return f;
  const double fd = static_cast<double>(f);
  if (fd != d && fd == fd && d == d) {
    uint32_t u = __float_as_uint(f);
    if ((u & 1u) == 0u) u += (fabs(d) > fabs(fd)) ? 1u : 0xffffffffu;
    f = __uint_as_float(u);
  }
  return bf16_to_f32(f32_to_bf16(f));
}

// M_t = mu * M_{t-1} + G as the momentum dtype holds it.  The product of a
// float32 and a bf16/float32 value is exact in double, so this is the
// correctly rounded value of the (double-evaluated) update.
__device__ __forceinline__ float momentum_value(float mu, float mp, float g, int32_t dt) {
  const double d = __builtin_fma(static_cast<double>(mu), static_cast<double>(mp), static_cast<double>(g));
  return round_from_f64(d, dt);
}

// Four consecutive elements starting at idx (idx % 4 == 0 and the base
// aligned for the dtype's 4-element vector: 16 bytes f32, 8 bytes bf16).
__device__ __forceinline__ void load4_aligned(const void* p, int64_t idx, int32_t dt, float out[4]) {
  if (dt == DT_F32) {
    float4 v = *reinterpret_cast<const MUON_GLOBAL float4*>(gmem(static_cast<const float*>(p)) + idx);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
    uint2 v = *reinterpret_cast<const MUON_GLOBAL uint2*>(gmem(static_cast<const uint16_t*>(p)) + idx);
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xffff0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xffff0000u);
  }
}

__device__ __forceinline__ void store4_aligned(void* p, int64_t idx, int32_t dt, const float v[4]) {
  if (dt == DT_F32) {
    *reinterpret_cast<MUON_GLOBAL float4*>(gmem(static_cast<float*>(p)) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<MUON_GLOBAL uint2*>(gmem(static_cast<uint16_t*>(p)) + idx) = u;
  }
}

// Cross-lane moves within a wave64 (DPP: no LDS traffic).  quad_perm
// [1,0,3,2] and [2,3,0,1] pair lanes L and L^1, L^2; row_half_mirror maps
// lane i of each 8-lane group to 7-i; row_mirror maps lane i of each
// 16-lane row to 15-i.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// Wave64 pairwise-tree sum; every lane receives the result.  Level 1 adds
// lanes (2j, 2j+1), level 2 the pairs of pairs, level 3 the 4-lane blocks,
// level 4 the 8-lane blocks, then the four 16-lane row sums r0..r3 are added
// as (r0 + r1) + (r2 + r3).  After each level every lane of a block holds the
// block's sum, so pairing with any lane of the partner block gives the same
// value, and IEEE addition is commutative: this is exactly the pairwise tree
// over the 64 lane values in lane order.
__device__ __forceinline__ float wave_tree_sum(float v) {
  v = v + dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  v = v + dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  v = v + dpp_f32<0x141>(v);   // row_half_mirror
  v = v + dpp_f32<0x140>(v);   // row_mirror
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v = v + dpp_f64<0xB1>(v);
  v = v + dpp_f64<0x4E>(v);
  v = v + dpp_f64<0x141>(v);
  v = v + dpp_f64<0x140>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// Pairwise-tree sum of p[0], p[stride], ..., p[(count-1)*stride], zero-padded
// to a power of two: a binary counter keeps one partial per complete block.
__device__ __forceinline__ float pairwise_strided(const float* p, int count, int64_t stride) {
  float stack[24];
  int pow2 = 1;
  while (pow2 < count) pow2 <<= 1;
  for (int t = 0; t < pow2; ++t) {
    float carry = (t < count) ? p[static_cast<int64_t>(t) * stride] : 0.0f;
    int j = 0;
    while ((t >> j) & 1) {
      carry = stack[j] + carry;   // earlier (left) block + later (right) block
      ++j;
    }
    stack[j] = carry;
  }
  int top = 0;
  while ((1 << top) < pow2) ++top;
  return stack[top];
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every outstanding global load and store of the wave; kernels
// whose global writes are never read back by the same launch use this one so
// that loads and stores stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Pairwise-tree sum of count values p[0], p[stride], ... zero-padded to a
// power of two, with the loads issued eight at a time (aligned blocks of
// eight are complete subtrees of the padded tree; a padding block adds +0 to
// non-negative sums, so padding to a multiple of eight gives the same value).
// first8 holds the first block, loaded by the caller (zeros beyond count).
__device__ __forceinline__ float pairwise_strided8(const float (&first8)[8], const float* p, int count,
                                                   int64_t stride) {
  float stack[24];
  const int blocks = (count + 7) / 8;
  int pow2 = 1;
  while (pow2 < blocks) pow2 <<= 1;
  for (int t = 0; t < pow2; ++t) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = t * 8 + j;
      v[j] = (t == 0) ? first8[j] : ((i < count) ? gmem(p)[static_cast<int64_t>(i) * stride] : 0.0f);
    }
    float carry = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    int j = 0;
    while ((t >> j) & 1) {
      carry = stack[j] + carry;
      ++j;
    }
    stack[j] = carry;
  }
  int top = 0;
  while ((1 << top) < pow2) ++top;
  return stack[top];
}

// Conditioning factor (relative energy + eps)^(-1/4).
__device__ __forceinline__ float cond_factor(float e, float emax, float eps) {
  float rho = e / emax;
  float t = rho + eps;
  return 1.0f / sqrtf(sqrtf(t));
}

#endif  // device

// --------------------------------------------------------------------------
// Host-side launchers (defined in the .hip files)
// --------------------------------------------------------------------------
// Energy partials of M_{t-1} into cache `parity` (tiles: the prescale's).
hipError_t launch_energy(const StepArgs& a, const Tile* tiles, int n, int parity, hipStream_t s);
// Dimuon conditioning over chunks of 256 rows / columns (tiles: matrix,
// chunk): energies (from cache `parity`) and chunk maxima, then the factors
// (zero in the padding).
hipError_t launch_cond_energy(const StepArgs& a, const Tile* tiles, int n, int parity, hipStream_t s);
hipError_t launch_cond_factor(const StepArgs& a, const Tile* tiles, int n, hipStream_t s);
// Momentum, then (Dimuon, `energies`) the energy partials of M_t into cache
// `out_parity`, and the prescale, in one pass.
hipError_t launch_prescale(const StepArgs& a, const Tile* tiles, int n, bool energies, int out_parity, hipStream_t s);
hipError_t launch_norm_finalize(const StepArgs& a, const uint16_t* mats, int n, hipStream_t s);
hipError_t launch_post_finalize(const StepArgs& a, const uint16_t* mats, int n, hipStream_t s);
hipError_t launch_update(const StepArgs& a, const Tile* tiles, int n, hipStream_t s);
// Gram / polynomial (kind 0: A = alpha X X^T, kind 1: B = c A A + b A) over
// bt x bt tiles, and combine over bm x bn tiles (sides 128 or 256 for bf16
// products; 128 for fp32).
hipError_t launch_syrk(const StepArgs& a, const Tile* tiles, int n, int bt, int kind, int src_x,
                       bool first, Coeffs cf, hipStream_t s);
// Combine X' = alpha (a X + B X); src/dst select the ping (0) or pong (1)
// buffers; `product` false skips B X (used when ns_steps is 0).
hipError_t launch_combine(const StepArgs& a, const Tile* tiles, int n, int bm, int bn, int src_x, int dst_x,
                          bool first, bool last, bool product, Coeffs cf, hipStream_t s);
// Thin path, one launch per phase over all slices of one padded Gram side KP:
// energies of M_{t-1} (only when no cached energies exist), pass A
// (momentum, Gram partials), pass B (k x k iteration, energies of M_t, apply,
// update).  `parity` selects the energy cache pass A reads; pass B writes the
// other.
hipError_t launch_thin_energy(const StepArgs& a, const Tile* tiles, int n, int kp, int parity, hipStream_t s);
hipError_t launch_thin_a(const StepArgs& a, const Tile* tiles, int n, int kp, int parity, hipStream_t s);
hipError_t launch_thin_b(const StepArgs& a, const Tile* tiles, int n, int kp, int ns_steps, const Coeffs* cf,
                         int parity, hipStream_t s);

}  // namespace muon
