// HBM-streaming kernels of the general path: the energies of M_{t-1} (only
// when no cached ones exist), conditioning, the fused momentum / energies /
// prescale pass into the Gram orientation, norm finalisation, and the final
// update.  No FMA contraction in this file: the energies must follow the
// stated float32 tree exactly, so every fused multiply-add below is written
// out as __builtin_fmaf.
#pragma clang fp contract(off)

#include "common.h"

namespace muon {

// ---------------------------------------------------------------------------
// Loads of 8 consecutive row elements (columns col0 .. col0+7); columns at or
// beyond n read as 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8(const void* p, int32_t dt, int64_t rowoff, int col0, int n,
                                      float out[8]) {
  const bool full = col0 + 8 <= n;
  const bool al = (dt == DT_F32) ? ((n & 3) == 0) : ((n & 7) == 0);
  if (full && al) {
    if (dt == DT_F32) {
      const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + rowoff + col0);
      float4 a = q[0], b = q[1];
      out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
      out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    } else {
      uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + rowoff + col0);
      out[0] = __uint_as_float(v.x << 16); out[1] = __uint_as_float(v.x & 0xffff0000u);
      out[2] = __uint_as_float(v.y << 16); out[3] = __uint_as_float(v.y & 0xffff0000u);
      out[4] = __uint_as_float(v.z << 16); out[5] = __uint_as_float(v.z & 0xffff0000u);
      out[6] = __uint_as_float(v.w << 16); out[7] = __uint_as_float(v.w & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      out[e] = (col0 + e < n) ? load_elem(p, rowoff + col0 + e, dt) : 0.0f;
  }
}

__device__ __forceinline__ void store8(void* p, int32_t dt, int64_t rowoff, int col0, int n,
                                       const float v[8]) {
  const bool full = col0 + 8 <= n;
  const bool al = (dt == DT_F32) ? ((n & 3) == 0) : ((n & 7) == 0);
  if (full && al) {
    if (dt == DT_F32) {
      float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + rowoff + col0);
      q[0] = make_float4(v[0], v[1], v[2], v[3]);
      q[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      uint4 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      u.z = pack_bf16x2(v[4], v[5]);
      u.w = pack_bf16x2(v[6], v[7]);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + rowoff + col0) = u;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (col0 + e < n) store_elem(p, rowoff + col0 + e, dt, v[e]);
  }
}

// ---------------------------------------------------------------------------
// Energy partials.  The general path cuts every matrix (in the caller's
// orientation) into 64 x 64 blocks, the tiles of the prescale pass.  A
// block contributes the row partial of each of its rows over its 64 columns
// and the column partial of each of its columns over its 64 rows, both
// aligned 64-element blocks of the stated pairwise tree (zero beyond the
// matrix).  The cache of one parity holds the row partials [ncb][m], then
// the column partials [nrb][n].
// A thread holds row si0 + r, columns sj0 + c0 .. c0 + 15 (c0 = 16 (tid & 3),
// r = tid / 4) of the block: its 16 squares are summed pairwise in the
// thread, then the four threads of the row (lanes 4q .. 4q+3 of a wave) are
// added pairwise.  The columns go through LDS: thread t sums column t mod 64
// over rows 16 (t / 64) .. + 15 pairwise, and the four 16-row sums of a
// column are added pairwise.
// ---------------------------------------------------------------------------
template <int CNT>
__device__ __forceinline__ float tree_sum(const float* x) {
  if constexpr (CNT == 1) return x[0];
  else return tree_sum<CNT / 2>(x) + tree_sum<CNT / 2>(x + CNT / 2);
}

__device__ __forceinline__ void block_energies(const float (&p)[16], int si0, int sj0, const MatDesc& d,
                                               float* cache, float (*pS)[65], float (*part)[64]) {
  const int tid = threadIdx.x, r = tid >> 2, c0 = (tid & 3) * 16;
  const int m = d.m, n = d.n;
  float rs = tree_sum<16>(p);
  rs = rs + dpp_f32<0xB1>(rs);   // quad_perm [1,0,3,2]: (q0 + q1), (q2 + q3)
  rs = rs + dpp_f32<0x4E>(rs);   // quad_perm [2,3,0,1]: (q0 + q1) + (q2 + q3)
  if ((tid & 3) == 0 && si0 + r < m && sj0 < n) cache[static_cast<int64_t>(sj0 / 64) * m + si0 + r] = rs;
#pragma unroll
  for (int e = 0; e < 16; ++e) pS[r][c0 + e] = p[e];
  __syncthreads();
  {
    const int c = tid & 63, q = tid >> 6;
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) col[i] = pS[16 * q + i][c];
    part[q][c] = tree_sum<16>(col);
  }
  __syncthreads();
  if (tid < 64 && si0 < m && sj0 + tid < n) {
    float* pc = cache + static_cast<int64_t>(d.ncb) * m;
    pc[static_cast<int64_t>(si0 / 64) * n + sj0 + tid] = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
  }
}

// Source block of a prescale tile: Gram element (ga, gb) is source (ga, gb)
// when wide, (gb, ga) when tall.
__device__ __forceinline__ void source_block(const MatDesc& d, const Tile& t, int& si0, int& sj0) {
  const int ga0 = t.ti * 64, gb0 = t.tj * 64;
  si0 = d.tall ? gb0 : ga0;
  sj0 = d.tall ? ga0 : gb0;
}

// Energies of M_{t-1} into cache `parity` (no cached energies: stateless
// calls, a plan's first Dimuon step, or after a reset).  Tiles: the
// prescale's (one 64 x 64 block each).
__global__ __launch_bounds__(256) void k_energy(StepArgs a, const Tile* __restrict__ tiles, int parity) {
  __shared__ float pS[64][65];
  __shared__ float part[4][64];
  const Tile t = tiles[blockIdx.x];
  const MatDesc& d = a.desc[t.mat];
  int si0, sj0;
  source_block(d, t, si0, sj0);
  const int tid = threadIdx.x, r = tid >> 2, c0 = (tid & 3) * 16;
  const int row = si0 + r;
  float v[16];
  if (row < d.m) {
    const int64_t off = static_cast<int64_t>(row) * d.n;
    load8(d.mom, a.mom_dt, off, sj0 + c0, d.n, v);
    load8(d.mom, a.mom_dt, off, sj0 + c0 + 8, d.n, v + 8);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = v[e] * v[e];
  block_energies(v, si0, sj0, d, reinterpret_cast<float*>(a.ws + d.ge_off[parity]), pS, part);
}

// ---------------------------------------------------------------------------
// K2: Dimuon conditioning, over chunks of 256 elements of the padded row
// range [0, round_up(m)) followed by the padded column range.  First the
// energies (pairwise over the energy blocks, eight loads in flight) and the
// chunk maxima; then, with the maxima of all chunks, the factors in place
// (zero in the padding).
// ---------------------------------------------------------------------------
__device__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float r = sh[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, sh[w]);
  return r;
}


__global__ __launch_bounds__(256) void k_cond_energy(StepArgs a, const Tile* __restrict__ tiles, int parity) {
  __shared__ float sh[8];
  const Tile t = tiles[blockIdx.x];
  const MatDesc& d = a.desc[t.mat];
  const int m = d.m, n = d.n;
  const int mp = d.mpad;
  const int idx = t.ti * 256 + threadIdx.x;
  MUON_GLOBAL float* dr = gmem(reinterpret_cast<float*>(a.ws + d.dr_off));
  MUON_GLOBAL float* dc = gmem(reinterpret_cast<float*>(a.ws + d.dc_off));
  const float* pr = reinterpret_cast<const float*>(a.ws + d.ge_off[parity]);
  const float* pc = pr + static_cast<int64_t>(d.ncb) * m;
  float rmax = 0.0f, cmax = 0.0f;
  if (idx < mp) {
    const int i = idx;
    float e = 0.0f;
    if (i < m) {
      float f8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f8[j] = j < d.ncb ? gmem(pr)[static_cast<int64_t>(j) * m + i] : 0.0f;
      e = pairwise_strided8(f8, pr + i, d.ncb, m);
      if (d.energy_out) gmem(d.energy_out)[i] = e;
    }
    dr[i] = e;
    rmax = e;
  } else if (idx < mp + d.npad) {
    const int j = idx - mp;
    float e = 0.0f;
    if (j < n) {
      float f8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) f8[q] = q < d.nrb ? gmem(pc)[static_cast<int64_t>(q) * n + j] : 0.0f;
      e = pairwise_strided8(f8, pc + j, d.nrb, n);
      if (d.energy_out) gmem(d.energy_out)[m + j] = e;
    }
    dc[j] = e;
    cmax = e;
  }
  rmax = block_max(rmax, sh);
  cmax = block_max(cmax, sh);
  if (threadIdx.x == 0) {
    MUON_GLOBAL float* cm = gmem(reinterpret_cast<float*>(a.ws + d.cm_off));
    cm[2 * t.ti] = rmax;
    cm[2 * t.ti + 1] = cmax;
  }
}

__global__ __launch_bounds__(256) void k_cond_factor(StepArgs a, const Tile* __restrict__ tiles) {
  __shared__ float sh[8];
  const Tile t = tiles[blockIdx.x];
  const MatDesc& d = a.desc[t.mat];
  const int m = d.m, n = d.n;
  const int mp = d.mpad;
  const MUON_GLOBAL float* cm = gmem(reinterpret_cast<const float*>(a.ws + d.cm_off));
  float rmax = 0.0f, cmax = 0.0f;
  for (int c = threadIdx.x; c < d.ncond; c += blockDim.x) {
    rmax = fmaxf(rmax, cm[2 * c]);
    cmax = fmaxf(cmax, cm[2 * c + 1]);
  }
  rmax = block_max(rmax, sh);
  cmax = block_max(cmax, sh);
  // A zero previous momentum (all energies 0) switches the conditioning off.
  const bool on = rmax > 0.0f && cmax > 0.0f;
  const int idx = t.ti * 256 + threadIdx.x;
  if (idx < mp) {
    MUON_GLOBAL float* dr = gmem(reinterpret_cast<float*>(a.ws + d.dr_off));
    if (idx < m) dr[idx] = on ? cond_factor(dr[idx], rmax, a.eps) : 1.0f;
  } else if (idx < mp + d.npad) {
    MUON_GLOBAL float* dc = gmem(reinterpret_cast<float*>(a.ws + d.dc_off));
    const int j = idx - mp;
    if (j < n) dc[j] = on ? cond_factor(dc[j], cmax, a.eps) : 1.0f;
  }
  if (t.ti == 0 && threadIdx.x == 0) a.scal[d.scal_idx].cond_on = on ? 1.0f : 0.0f;
}

// ---------------------------------------------------------------------------
// K3: the fused pass.  M_t = mu M_{t-1} + G (correctly rounded to the
// momentum dtype and stored); with ENERGIES (Dimuon) the energy partials of
// M_t into cache `out_parity`, for the next step's conditioning; then
// Y = D_R V D_C (V = M_t, or the Nesterov input G + mu M_t), rounded to the
// NS dtype, written in the Gram orientation (KP x NP) and, for the fp32
// products, its transpose (NP x KP), zero in the padding; one ||Y||^2
// partial per tile.  Tile: 64 x 64 of the Gram orientation; the source
// block goes through LDS.  Each element belongs to one tile, so M_t is
// never read back.
// ---------------------------------------------------------------------------
template <bool ENERGIES>
__global__ __launch_bounds__(256) void k_prescale(StepArgs a, const Tile* __restrict__ tiles, int out_parity) {
  // The energy partials stage their squares in tileS before Y goes there
  // (block_energies ends with a barrier after its last read of them): 17 KB
  // less LDS per workgroup: seven waves per SIMD (register-bound) instead of
  // four (LDS-bound).
  __shared__ float tileS[64][65];
  __shared__ float part[ENERGIES ? 4 : 1][64];
  __shared__ float red[4];
  const Tile t = tiles[blockIdx.x];
  const MatDesc& d = a.desc[t.mat];
  const int m = d.m, n = d.n;
  const int tid = threadIdx.x;
  const bool cond = a.dimuon && a.scal[d.scal_idx].cond_on != 0.0f;
  const float* dr = reinterpret_cast<const float*>(a.ws + d.dr_off);
  const float* dc = reinterpret_cast<const float*>(a.ws + d.dc_off);
  const int ga0 = t.ti * 64, gb0 = t.tj * 64;
  int si0, sj0;
  source_block(d, t, si0, sj0);
  {
    const int r = tid >> 2, c0 = (tid & 3) * 16;
    const int row = si0 + r;
    float v[16], sq[16];
    if (row < m) {
      const int64_t off = static_cast<int64_t>(row) * n;
      float gv[16];
      load8(d.mom, a.mom_dt, off, sj0 + c0, n, v);
      load8(d.mom, a.mom_dt, off, sj0 + c0 + 8, n, v + 8);
      load8(d.g, a.g_dt, off, sj0 + c0, n, gv);
      load8(d.g, a.g_dt, off, sj0 + c0 + 8, n, gv + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = momentum_value(a.mu, v[e], gv[e], a.mom_dt);
      store8(d.mom, a.mom_dt, off, sj0 + c0, n, v);
      store8(d.mom, a.mom_dt, off, sj0 + c0 + 8, n, v + 8);
      if constexpr (ENERGIES) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sq[e] = v[e] * v[e];   // fl32(x * x) of the stored value
      }
      if (a.nesterov) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = gv[e] + a.mu * v[e];
      }
      const float rf = cond ? dr[row] : 1.0f;
      // The thread's 16 column factors as four 16-byte loads (the factor
      // array spans the padded extent, which the tile's columns never pass);
      // columns at or beyond n take 1 as before.
      float fc[16];
      if (cond) {
        const float4* q = reinterpret_cast<const float4*>(dc + sj0 + c0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4 f = q[e];
          fc[4 * e] = f.x; fc[4 * e + 1] = f.y; fc[4 * e + 2] = f.z; fc[4 * e + 3] = f.w;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int col = sj0 + c0 + e;
        const float cf = (cond && col < n) ? fc[e] : 1.0f;
        v[e] = (rf * v[e]) * cf;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        v[e] = 0.0f;
        sq[e] = 0.0f;
      }
    }
    if constexpr (ENERGIES)
      block_energies(sq, si0, sj0, d, reinterpret_cast<float*>(a.ws + d.ge_off[out_parity]), tileS, part);
#pragma unroll
    for (int e = 0; e < 16; ++e) tileS[r][c0 + e] = round_to(v[e], a.ns_dt);
  }
  __syncthreads();
  // Write Y (Gram orientation) and, for the fp32 products, Y^T; 16
  // contiguous elements per thread.
  char* ybase = a.ws + d.x_off[0];
  const int r = tid >> 2, c0 = (tid & 3) * 16;
  float ssq = 0.0f;
  {
    // Y[ga0 + r][gb0 + c0 + e] = (wide) S[r][c0+e] | (tall) S[c0+e][r]
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = d.tall ? tileS[c0 + e][r] : tileS[r][c0 + e];
#pragma unroll
    for (int e = 0; e < 16; ++e) ssq = ssq + v[e] * v[e];
    const int64_t off = static_cast<int64_t>(ga0 + r) * d.NP + gb0 + c0;
    if (a.ns_dt == DT_F32) {
      float4* q = reinterpret_cast<float4*>(reinterpret_cast<float*>(ybase) + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = make_float4(v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]);
    } else {
      uint4* q = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(ybase) + off);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint4 u;
        u.x = pack_bf16x2(v[8 * e + 0], v[8 * e + 1]);
        u.y = pack_bf16x2(v[8 * e + 2], v[8 * e + 3]);
        u.z = pack_bf16x2(v[8 * e + 4], v[8 * e + 5]);
        u.w = pack_bf16x2(v[8 * e + 6], v[8 * e + 7]);
        q[e] = u;
      }
    }
  }
  if (a.ns_dt == DT_F32) {
    // Y^T[gb0 + r][ga0 + c0 + e] = Y[ga0 + c0 + e][gb0 + r]
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = d.tall ? tileS[r][c0 + e] : tileS[c0 + e][r];
    const int64_t off = static_cast<int64_t>(gb0 + r) * d.KP + ga0 + c0;
    float4* q = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.ws + d.x_off[1]) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = make_float4(v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]);
  }
  ssq = wave_tree_sum(ssq);
  if ((tid & 63) == 0) red[tid >> 6] = ssq;
  __syncthreads();
  if (tid == 0) {
    const float s = (red[0] + red[1]) + (red[2] + red[3]);
    const int tiles_per_row = d.NP / 64;
    reinterpret_cast<float*>(a.ws + d.pn_off)[t.ti * tiles_per_row + t.tj] = s;
  }
}

// Deterministic block sum: fixed per-thread stride order, butterfly, waves in order.
__device__ float block_sum_fixed(const float* p, int count, float* sh) {
  float s = 0.0f;
  for (int i = threadIdx.x; i < count; i += blockDim.x) s = s + p[i];
  s = wave_tree_sum(s);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sh[wave] = s;
  __syncthreads();
  float r = sh[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = r + sh[w];
  return r;
}

// ---------------------------------------------------------------------------
// ||Y||_F from the prescale partials.  One workgroup per matrix.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_norm_finalize(StepArgs a, const uint16_t* __restrict__ mats) {
  __shared__ float sh[8];
  const int mat = mats[blockIdx.x];
  const MatDesc& d = a.desc[mat];
  const float nu2 = block_sum_fixed(reinterpret_cast<const float*>(a.ws + d.pn_off), d.n_pn, sh);
  if (threadIdx.x == 0) {
    MatScal& s = a.scal[d.scal_idx];
    const float inv = (nu2 == 0.0f) ? 0.0f : 1.0f / sqrtf(nu2);
    s.inv_nu = inv;
    s.inv_nu2 = inv * inv;
    s.post = 1.0f;
  }
}

// ---------------------------------------------------------------------------
// Dimuon norm fix ||Z||_F / ||D_R Z D_C||_F from the last combine's partials.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_post_finalize(StepArgs a, const uint16_t* __restrict__ mats) {
  __shared__ float sh[8];
  __shared__ float zsum;
  const int mat = mats[blockIdx.x];
  const MatDesc& d = a.desc[mat];
  const float* pz = reinterpret_cast<const float*>(a.ws + d.pz_off);
  // partials are interleaved pairs (||Z||^2, ||P||^2)
  float sz = 0.0f, sp = 0.0f;
  for (int i = threadIdx.x; i < d.n_pz; i += blockDim.x) {
    sz = sz + pz[2 * i];
    sp = sp + pz[2 * i + 1];
  }
  sz = wave_tree_sum(sz);
  sp = wave_tree_sum(sp);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wave] = sz;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = r + sh[w];
    zsum = r;
  }
  __syncthreads();
  if (lane == 0) sh[wave] = sp;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = r + sh[w];
    a.scal[d.scal_idx].post = (r == 0.0f) ? 0.0f : sqrtf(zsum) / sqrtf(r);
  }
}

// ---------------------------------------------------------------------------
// K5: O = post * D_R Z D_C (Dimuon) or Z (Muon); o_out = O;
// W = W - lr * (scale * O + wd * W).  Tile: 64 x 64 of the original m x n.
// Z is read in the original orientation: the last combine wrote a tall
// matrix's Z transposed (n x m, ld KP).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_update(StepArgs a, const Tile* __restrict__ tiles) {
  const Tile t = tiles[blockIdx.x];
  const MatDesc& d = a.desc[t.mat];
  const int m = d.m, n = d.n;
  const int tid = threadIdx.x;
  const int r = tid >> 2, c0 = (tid & 3) * 16;
  const int row = t.ti * 64 + r;
  if (row >= m) return;
  const int64_t zld = d.tall ? d.KP : d.NP;   // Z holds the ns dtype
  const MatScal sc = a.scal[d.scal_idx];
  const float* dr = reinterpret_cast<const float*>(a.ws + d.dr_off);
  const float* dc = reinterpret_cast<const float*>(a.ws + d.dc_off);
  const float rf = a.dimuon ? dr[row] : 1.0f;
  const int64_t off = static_cast<int64_t>(row) * n;
  // Both halves are loaded (W, Z and the column factors) before the first
  // store, which the compiler would otherwise have to order them after.
  float w[2][8], zv[2][8], cf[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col0 = t.tj * 64 + c0 + 8 * h;
    if (col0 >= n) continue;
    load8(d.w, a.w_dt, off, col0, n, w[h]);
    const int64_t zi = static_cast<int64_t>(row) * zld + col0;
    if (a.ns_dt == DT_F32) {
      const float4* zq = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.ws + d.z_off) + zi);
      const float4 z0 = zq[0], z1 = zq[1];
      zv[h][0] = z0.x; zv[h][1] = z0.y; zv[h][2] = z0.z; zv[h][3] = z0.w;
      zv[h][4] = z1.x; zv[h][5] = z1.y; zv[h][6] = z1.z; zv[h][7] = z1.w;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.ws + d.z_off) + zi);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        zv[h][2 * e] = __uint_as_float(w4[e] << 16);
        zv[h][2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
      }
    }
    // Column factors as two 16-byte loads (the factor array spans the padded
    // extent, a multiple of 128 at least n); columns at or beyond n take 1.
    float f8[8];
    if (a.dimuon) {
      const float4* q = reinterpret_cast<const float4*>(dc + col0);
      const float4 f0 = q[0], f1 = q[1];
      f8[0] = f0.x; f8[1] = f0.y; f8[2] = f0.z; f8[3] = f0.w;
      f8[4] = f1.x; f8[5] = f1.y; f8[6] = f1.z; f8[7] = f1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) cf[h][e] = (a.dimuon && col0 + e < n) ? f8[e] : 1.0f;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col0 = t.tj * 64 + c0 + 8 * h;
    if (col0 >= n) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = a.dimuon ? sc.post * ((rf * zv[h][e]) * cf[h][e]) : zv[h][e];
      // W - lr * (scale * O + wd * W), with the outer product-subtract fused.
      const float upd = __builtin_fmaf(d.update_scale, o[e], a.weight_decay * w[h][e]);
      w[h][e] = __builtin_fmaf(-a.lr, upd, w[h][e]);
    }
    store8(d.w, a.w_dt, off, col0, n, w[h]);
    if (d.o_out) store8(d.o_out, DT_F32, off, col0, n, o);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_energy(const StepArgs& a, const Tile* tiles, int n, int parity, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_energy, dim3(n), dim3(256), 0, s, a, tiles, parity);
  return hipGetLastError();
}

hipError_t launch_cond_energy(const StepArgs& a, const Tile* tiles, int n, int parity, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_cond_energy, dim3(n), dim3(256), 0, s, a, tiles, parity);
  return hipGetLastError();
}

hipError_t launch_cond_factor(const StepArgs& a, const Tile* tiles, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_cond_factor, dim3(n), dim3(256), 0, s, a, tiles);
  return hipGetLastError();
}

hipError_t launch_prescale(const StepArgs& a, const Tile* tiles, int n, bool energies, int out_parity, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (energies) hipLaunchKernelGGL(k_prescale<true>, dim3(n), dim3(256), 0, s, a, tiles, out_parity);
  else hipLaunchKernelGGL(k_prescale<false>, dim3(n), dim3(256), 0, s, a, tiles, out_parity);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const StepArgs& a, const uint16_t* mats, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_norm_finalize, dim3(n), dim3(256), 0, s, a, mats);
  return hipGetLastError();
}

hipError_t launch_post_finalize(const StepArgs& a, const uint16_t* mats, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_post_finalize, dim3(n), dim3(256), 0, s, a, mats);
  return hipGetLastError();
}

hipError_t launch_update(const StepArgs& a, const Tile* tiles, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_update, dim3(n), dim3(256), 0, s, a, tiles);
  return hipGetLastError();
}

}  // namespace muon
