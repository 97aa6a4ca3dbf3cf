// Grouped GEMM kernels of the Newton-Schulz iteration.
//
// Every product here is "NT": C[i][j] = sum_k P[i][k] Q[j][k], with both
// operands row-major and K-contiguous.  This works because the workspace
// keeps each iterate in both layouts, X (k x N) and X^T (N x k):
//   Gram     A = X X^T        P = X,   Q = X     (K = N)   symmetric
//   poly     B = b A + c A A  P = A,   Q = A     (K = k)   symmetric
//   combine  X' = a X + B X   P = B,   Q = X^T   (K = k)
// The symmetric products compute the upper-triangular tiles only and store
// each such tile and its mirror.  The combine stores X' and X'^T.
//
// bf16 path: a 128 x 128 x 64 workgroup tile, 4 wave64 in a 2 x 2 grid, each
// wave owning 64 x 64 as 2 x 2 v_mfma_f32_32x32x16_bf16 blocks.  LDS is
// double-buffered and global loads for k-tile t+1 are in flight while k-tile
// t is multiplied.  The epilogue stages the fp32 tile through LDS so that
// both the tile and its transpose are written with 16-byte stores.
#include "common.h"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;
constexpr int EP_LD = BN + 1;

struct SmemMain {
  uint16_t a[2][BM][LDK];
  uint16_t b[2][BN][LDK];
};
constexpr int kSmemMain = sizeof(SmemMain);
constexpr int kSmemEpi = BM * EP_LD * 4;
constexpr int kSmemBytes = kSmemMain > kSmemEpi ? kSmemMain : kSmemEpi;

// Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
// run of the tile list so that tiles sharing operand panels share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
}

// acc[s][t] += P[rows wr*64+s*32..][k] * Q[rows wc*64+t*32..][k] over k < K.
__device__ __forceinline__ void mma_nt_bf16(const uint16_t* __restrict__ Pg, int64_t ldp,
                                            const uint16_t* __restrict__ Qg, int64_t ldq, int K,
                                            SmemMain& sm, f32x16_t acc[2][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  // Chunk q of this thread: row (tid + 256 q) / 8, 16-byte column (tid & 7).
  const int crow = tid >> 3, ccol = (tid & 7) * 8;
  const uint16_t* pa = Pg + crow * ldp + ccol;
  const uint16_t* pb = Qg + crow * ldq + ccol;
  const int64_t sa = 32 * ldp, sb = 32 * ldq;   // 256 chunks = 32 rows further
#define MUON_GLOAD(k0)                                                        \
  ra0 = *reinterpret_cast<const uint4*>(pa + (k0));                           \
  ra1 = *reinterpret_cast<const uint4*>(pa + sa + (k0));                      \
  ra2 = *reinterpret_cast<const uint4*>(pa + 2 * sa + (k0));                  \
  ra3 = *reinterpret_cast<const uint4*>(pa + 3 * sa + (k0));                  \
  rb0 = *reinterpret_cast<const uint4*>(pb + (k0));                           \
  rb1 = *reinterpret_cast<const uint4*>(pb + sb + (k0));                      \
  rb2 = *reinterpret_cast<const uint4*>(pb + 2 * sb + (k0));                  \
  rb3 = *reinterpret_cast<const uint4*>(pb + 3 * sb + (k0));
#define MUON_SSTORE(buf)                                                      \
  *reinterpret_cast<uint4*>(&sm.a[buf][crow][ccol]) = ra0;                    \
  *reinterpret_cast<uint4*>(&sm.a[buf][crow + 32][ccol]) = ra1;               \
  *reinterpret_cast<uint4*>(&sm.a[buf][crow + 64][ccol]) = ra2;               \
  *reinterpret_cast<uint4*>(&sm.a[buf][crow + 96][ccol]) = ra3;               \
  *reinterpret_cast<uint4*>(&sm.b[buf][crow][ccol]) = rb0;                    \
  *reinterpret_cast<uint4*>(&sm.b[buf][crow + 32][ccol]) = rb1;               \
  *reinterpret_cast<uint4*>(&sm.b[buf][crow + 64][ccol]) = rb2;               \
  *reinterpret_cast<uint4*>(&sm.b[buf][crow + 96][ccol]) = rb3;
  MUON_GLOAD(0)
  MUON_SSTORE(0)
  __syncthreads();
  const int nk = K / BK;
  const int fr = lane & 31, fk = 8 * (lane >> 5);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) { MUON_GLOAD((kt + 1) * BK) }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        fa[s] = *reinterpret_cast<const bf16x8_t*>(&sm.a[cur][wr * 64 + s * 32 + fr][kk * 16 + fk]);
        fb[s] = *reinterpret_cast<const bf16x8_t*>(&sm.b[cur][wc * 64 + s * 32 + fr][kk * 16 + fk]);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[s][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s], fb[t], acc[s][t], 0, 0, 0);
    }
    if (kt + 1 < nk) { MUON_SSTORE(cur ^ 1) }
    __syncthreads();
  }
#undef MUON_GLOAD
#undef MUON_SSTORE
}

// Position of accumulator element r of block (s, t) inside the 128 x 128 tile.
__device__ __forceinline__ int acc_row(int s, int r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 1) * 64 + s * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int t) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 1) * 64 + t * 32 + (lane & 31);
}

// Store the staged fp32 tile ep[BM][EP_LD] at dst (row0, col0), and / or its
// transpose at dstT (col0, row0).  dt selects bf16 or f32 storage.
__device__ __forceinline__ void store_tile(const float* ep, void* dst, int64_t ld, int64_t row0,
                                           int64_t col0, int32_t dt) {
  const int tid = threadIdx.x, r = tid >> 1, c0 = (tid & 1) * 64;
  const float* src = ep + r * EP_LD + c0;
  if (dt == DT_BF16) {
    uint4* q = reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + (row0 + r) * ld + col0 + c0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint4 u;
      u.x = f32_to_bf16(src[8 * e + 0]) | (static_cast<uint32_t>(f32_to_bf16(src[8 * e + 1])) << 16);
      u.y = f32_to_bf16(src[8 * e + 2]) | (static_cast<uint32_t>(f32_to_bf16(src[8 * e + 3])) << 16);
      u.z = f32_to_bf16(src[8 * e + 4]) | (static_cast<uint32_t>(f32_to_bf16(src[8 * e + 5])) << 16);
      u.w = f32_to_bf16(src[8 * e + 6]) | (static_cast<uint32_t>(f32_to_bf16(src[8 * e + 7])) << 16);
      q[e] = u;
    }
  } else {
    float4* q = reinterpret_cast<float4*>(static_cast<float*>(dst) + (row0 + r) * ld + col0 + c0);
#pragma unroll
    for (int e = 0; e < 16; ++e) q[e] = make_float4(src[4 * e], src[4 * e + 1], src[4 * e + 2], src[4 * e + 3]);
  }
}

__device__ __forceinline__ void store_tile_t(const float* ep, void* dst, int64_t ld, int64_t row0,
                                             int64_t col0, int32_t dt) {
  // dst[(col0 + j) * ld + row0 + i] = ep[i][j]
  const int tid = threadIdx.x, j = tid >> 1, i0 = (tid & 1) * 64;
  if (dt == DT_BF16) {
    uint4* q = reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + (col0 + j) * ld + row0 + i0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) v[h] = ep[(i0 + 8 * e + h) * EP_LD + j];
      uint4 u;
      u.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
      u.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
      u.z = f32_to_bf16(v[4]) | (static_cast<uint32_t>(f32_to_bf16(v[5])) << 16);
      u.w = f32_to_bf16(v[6]) | (static_cast<uint32_t>(f32_to_bf16(v[7])) << 16);
      q[e] = u;
    }
  } else {
    float4* q = reinterpret_cast<float4*>(static_cast<float*>(dst) + (col0 + j) * ld + row0 + i0);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) v[h] = ep[(i0 + 4 * e + h) * EP_LD + j];
      q[e] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

__device__ __forceinline__ float block_sum256(float v, float* sh) {
  v = wave_tree_sum(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  const float r = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Symmetric products (bf16): kind 0 Gram, kind 1 polynomial.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_syrk_bf16(StepArgs a, const Tile* __restrict__ tiles, int ntiles,
                                                   int kind, int src_x, int first, Coeffs cf) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  SmemMain& sm = *reinterpret_cast<SmemMain*>(smem);
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
  const int K = static_cast<int>(ld);
  f32x16_t acc[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][u][r] = 0.0f;
  mma_nt_bf16(P + static_cast<int64_t>(t.ti) * BM * ld, ld, P + static_cast<int64_t>(t.tj) * BN * ld, ld, K,
              sm, acc);

  const float alpha = (kind == 0) ? (first ? a.scal[d.scal_idx].inv_nu2 : 1.0f) : cf.c;
  const uint16_t* E = reinterpret_cast<const uint16_t*>(a.ws + d.a_off);
  float* ep = reinterpret_cast<float*>(smem);
  const int64_t gi0 = static_cast<int64_t>(t.ti) * BM, gj0 = static_cast<int64_t>(t.tj) * BN;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = acc_row(s, r), j = acc_col(u);
        float v = alpha * acc[s][u][r];
        if (kind == 1) v = v + cf.b * bf16_to_f32(E[(gi0 + i) * d.KP + gj0 + j]);
        ep[i * EP_LD + j] = v;
      }
  __syncthreads();
  void* dst = a.ws + (kind == 0 ? d.a_off : d.b_off);
  store_tile(ep, dst, d.KP, gi0, gj0, DT_BF16);
  if (t.ti != t.tj) store_tile_t(ep, dst, d.KP, gi0, gj0, DT_BF16);
}

// ---------------------------------------------------------------------------
// Combine (bf16 operands): X' = alpha (a X + B X).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine_bf16(StepArgs a, const Tile* __restrict__ tiles, int ntiles,
                                                      int src_x, int dst_x, int first, int last, int product,
                                                      Coeffs cf) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __shared__ float red[4];
  SmemMain& sm = *reinterpret_cast<SmemMain*>(smem);
  const Tile t = tiles[xcd_remap(blockIdx.x, ntiles)];
  const MatDesc& d = a.desc[t.mat];
  const uint16_t* Bm = reinterpret_cast<const uint16_t*>(a.ws + d.b_off);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.ws + d.x_off[2 * src_x]);
  const uint16_t* XT = reinterpret_cast<const uint16_t*>(a.ws + d.x_off[2 * src_x + 1]);
  f32x16_t acc[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][u][r] = 0.0f;
  if (product)
    mma_nt_bf16(Bm + static_cast<int64_t>(t.ti) * BM * d.KP, d.KP, XT + static_cast<int64_t>(t.tj) * BN * d.KP,
                d.KP, d.KP, sm, acc);

  const float alpha = first ? a.scal[d.scal_idx].inv_nu : 1.0f;
  float* ep = reinterpret_cast<float*>(smem);
  const int64_t gi0 = static_cast<int64_t>(t.ti) * BM, gj0 = static_cast<int64_t>(t.tj) * BN;
  const bool partials = last && a.dimuon;
  const float* dgr = reinterpret_cast<const float*>(a.ws + (d.tall ? d.dc_off : d.dr_off));
  const float* dgc = reinterpret_cast<const float*>(a.ws + (d.tall ? d.dr_off : d.dc_off));
  float sz = 0.0f, sp = 0.0f;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = acc_row(s, r), j = acc_col(u);
        const float x = bf16_to_f32(X[(gi0 + i) * d.NP + gj0 + j]);
        const float v = alpha * (cf.a * x + acc[s][u][r]);
        ep[i * EP_LD + j] = v;
        if (partials) {
          const int64_t gi = gi0 + i, gj = gj0 + j;
          const float fr = gi < d.k ? dgr[gi] : 0.0f;
          const float fc = gj < d.N ? dgc[gj] : 0.0f;
          const float p = (fr * v) * fc;
          sz = sz + v * v;
          sp = sp + p * p;
        }
      }
  __syncthreads();
  if (!last) {
    store_tile(ep, a.ws + d.x_off[2 * dst_x], d.NP, gi0, gj0, DT_BF16);
    store_tile_t(ep, a.ws + d.x_off[2 * dst_x + 1], d.KP, gi0, gj0, DT_BF16);
  } else if (d.tall) {
    store_tile_t(ep, a.ws + d.z_off, d.KP, gi0, gj0, DT_F32);
  } else {
    store_tile(ep, a.ws + d.z_off, d.NP, gi0, gj0, DT_F32);
  }
  if (partials) {
    sz = block_sum256(sz, red);
    sp = block_sum256(sp, red);
    if (threadIdx.x == 0) {
      float* pz = reinterpret_cast<float*>(a.ws + d.pz_off);
      const int idx = t.ti * (d.NP / BN) + t.tj;
      pz[2 * idx] = sz;
      pz[2 * idx + 1] = sp;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path (ns dtype F32): the same products with IEEE fp32 multiply-adds.
// 128 x 128 tile, 256 threads, each an 8 x 8 micro-tile; K in steps of 16.
// ---------------------------------------------------------------------------
constexpr int FBK = 16, FLD = 128 + 4;

__device__ __forceinline__ void mma_nt_f32(const float* __restrict__ Pg, int64_t ldp,
                                           const float* __restrict__ Qg, int64_t ldq, int K,
                                           float (*As)[FLD], float (*Bs)[FLD], float acc[8][8]) {
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  for (int k0 = 0; k0 < K; k0 += FBK) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = tid + 256 * q, row = c >> 2, k4 = (c & 3) * 4;
      const float4 va = *reinterpret_cast<const float4*>(Pg + row * ldp + k0 + k4);
      const float4 vb = *reinterpret_cast<const float4*>(Qg + row * ldq + k0 + k4);
      As[k4 + 0][row] = va.x; As[k4 + 1][row] = va.y; As[k4 + 2][row] = va.z; As[k4 + 3][row] = va.w;
      Bs[k4 + 0][row] = vb.x; Bs[k4 + 1][row] = vb.y; Bs[k4 + 2][row] = vb.z; Bs[k4 + 3][row] = vb.w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FBK; ++k) {
      float av[8], bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { av[e] = As[k][ty * 8 + e]; bv[e] = Bs[k][tx * 8 + e]; }
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = __builtin_fmaf(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_syrk_f32(StepArgs a, const Tile* __restrict__ tiles, int ntiles,
                                                  int kind, int src_x, int first, Coeffs cf) {
  __shared__ float As[FBK][FLD], Bs[FBK][FLD];
  const Tile t = tiles[xcd_remap(blockIdx.x, ntiles)];
  const MatDesc& d = a.desc[t.mat];
  const float* P;
  int64_t ld;
  if (kind == 0) {
    P = reinterpret_cast<const float*>(a.ws + d.x_off[2 * src_x]);
    ld = d.NP;
  } else {
    P = reinterpret_cast<const float*>(a.ws + d.a_off);
    ld = d.KP;
  }
  float acc[8][8] = {};
  mma_nt_f32(P + static_cast<int64_t>(t.ti) * BM * ld, ld, P + static_cast<int64_t>(t.tj) * BN * ld, ld,
             static_cast<int>(ld), As, Bs, acc);
  const float alpha = (kind == 0) ? (first ? a.scal[d.scal_idx].inv_nu2 : 1.0f) : cf.c;
  const float* E = reinterpret_cast<const float*>(a.ws + d.a_off);
  float* C = reinterpret_cast<float*>(a.ws + (kind == 0 ? d.a_off : d.b_off));
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  const int64_t gi0 = static_cast<int64_t>(t.ti) * BM + ty * 8, gj0 = static_cast<int64_t>(t.tj) * BN + tx * 8;
  float v[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v[r][c] = alpha * acc[r][c];
      if (kind == 1) v[r][c] = v[r][c] + cf.b * E[(gi0 + r) * d.KP + gj0 + c];
    }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float4* q = reinterpret_cast<float4*>(C + (gi0 + r) * d.KP + gj0);
    q[0] = make_float4(v[r][0], v[r][1], v[r][2], v[r][3]);
    q[1] = make_float4(v[r][4], v[r][5], v[r][6], v[r][7]);
  }
  if (t.ti != t.tj) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float4* q = reinterpret_cast<float4*>(C + (gj0 + c) * d.KP + gi0);
      q[0] = make_float4(v[0][c], v[1][c], v[2][c], v[3][c]);
      q[1] = make_float4(v[4][c], v[5][c], v[6][c], v[7][c]);
    }
  }
}

__global__ __launch_bounds__(256) void k_combine_f32(StepArgs a, const Tile* __restrict__ tiles, int ntiles,
                                                     int src_x, int dst_x, int first, int last, int product,
                                                     Coeffs cf) {
  __shared__ float As[FBK][FLD], Bs[FBK][FLD];
  __shared__ float red[4];
  const Tile t = tiles[xcd_remap(blockIdx.x, ntiles)];
  const MatDesc& d = a.desc[t.mat];
  const float* Bm = reinterpret_cast<const float*>(a.ws + d.b_off);
  const float* X = reinterpret_cast<const float*>(a.ws + d.x_off[2 * src_x]);
  const float* XT = reinterpret_cast<const float*>(a.ws + d.x_off[2 * src_x + 1]);
  float acc[8][8] = {};
  if (product)
    mma_nt_f32(Bm + static_cast<int64_t>(t.ti) * BM * d.KP, d.KP, XT + static_cast<int64_t>(t.tj) * BN * d.KP,
               d.KP, d.KP, As, Bs, acc);
  const float alpha = first ? a.scal[d.scal_idx].inv_nu : 1.0f;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  const int64_t gi0 = static_cast<int64_t>(t.ti) * BM + ty * 8, gj0 = static_cast<int64_t>(t.tj) * BN + tx * 8;
  const bool partials = last && a.dimuon;
  const float* dgr = reinterpret_cast<const float*>(a.ws + (d.tall ? d.dc_off : d.dr_off));
  const float* dgc = reinterpret_cast<const float*>(a.ws + (d.tall ? d.dr_off : d.dc_off));
  float v[8][8];
  float sz = 0.0f, sp = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float x = X[(gi0 + r) * d.NP + gj0 + c];
      v[r][c] = alpha * (cf.a * x + acc[r][c]);
      if (partials) {
        const int64_t gi = gi0 + r, gj = gj0 + c;
        const float fr = gi < d.k ? dgr[gi] : 0.0f;
        const float fc = gj < d.N ? dgc[gj] : 0.0f;
        const float p = (fr * v[r][c]) * fc;
        sz = sz + v[r][c] * v[r][c];
        sp = sp + p * p;
      }
    }
  float* Xn = reinterpret_cast<float*>(a.ws + d.x_off[2 * dst_x]);
  float* XnT = reinterpret_cast<float*>(a.ws + d.x_off[2 * dst_x + 1]);
  float* Z = reinterpret_cast<float*>(a.ws + d.z_off);
  const bool write_n = !last || !d.tall;
  const bool write_t = !last || d.tall;
  float* dn = last ? Z : Xn;
  float* dt = last ? Z : XnT;
  if (write_n) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float4* q = reinterpret_cast<float4*>(dn + (gi0 + r) * d.NP + gj0);
      q[0] = make_float4(v[r][0], v[r][1], v[r][2], v[r][3]);
      q[1] = make_float4(v[r][4], v[r][5], v[r][6], v[r][7]);
    }
  }
  if (write_t) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float4* q = reinterpret_cast<float4*>(dt + (gj0 + c) * d.KP + gi0);
      q[0] = make_float4(v[0][c], v[1][c], v[2][c], v[3][c]);
      q[1] = make_float4(v[4][c], v[5][c], v[6][c], v[7][c]);
    }
  }
  if (partials) {
    sz = block_sum256(sz, red);
    sp = block_sum256(sp, red);
    if (threadIdx.x == 0) {
      float* pz = reinterpret_cast<float*>(a.ws + d.pz_off);
      const int idx = t.ti * (d.NP / BN) + t.tj;
      pz[2 * idx] = sz;
      pz[2 * idx + 1] = sp;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_syrk(const StepArgs& a, const Tile* tiles, int n, int kind, int src_x, bool first,
                       Coeffs cf, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (a.ns_dt == DT_BF16)
    hipLaunchKernelGGL(k_syrk_bf16, dim3(n), dim3(256), 0, s, a, tiles, n, kind, src_x, first ? 1 : 0, cf);
  else
    hipLaunchKernelGGL(k_syrk_f32, dim3(n), dim3(256), 0, s, a, tiles, n, kind, src_x, first ? 1 : 0, cf);
  return hipGetLastError();
}

hipError_t launch_combine(const StepArgs& a, const Tile* tiles, int n, int src_x, int dst_x, bool first,
                          bool last, bool product, Coeffs cf, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (a.ns_dt == DT_BF16)
    hipLaunchKernelGGL(k_combine_bf16, dim3(n), dim3(256), 0, s, a, tiles, n, src_x, dst_x, first ? 1 : 0,
                       last ? 1 : 0, product ? 1 : 0, cf);
  else
    hipLaunchKernelGGL(k_combine_f32, dim3(n), dim3(256), 0, s, a, tiles, n, src_x, dst_x, first ? 1 : 0,
                       last ? 1 : 0, product ? 1 : 0, cf);
  return hipGetLastError();
}

}  // namespace muon
