// Host side of the C ABI: argument validation, the batch plan (path choice,
// workspace layout, tile lists), the descriptor upload cache, and the launch
// sequence of one Muon / Dimuon step.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

thread_local std::string g_last_error;

// Launch-event hook (timing only).
struct EventHook {
  void* const* events = nullptr;
  int32_t* kinds = nullptr;
  int32_t n = 0;
  int32_t next = 0;
  int32_t last_count = 0;
};
thread_local EventHook g_hook;

hipError_t hook_record(int32_t kind, hipStream_t s) {
  if (!g_hook.events || g_hook.next >= g_hook.n) return hipSuccess;
  hipError_t e = hipEventRecord(static_cast<hipEvent_t>(g_hook.events[g_hook.next]), s);
  if (g_hook.kinds) g_hook.kinds[g_hook.next] = kind;
  ++g_hook.next;
  return e;
}

muon_status_t fail(muon_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

constexpr int64_t kMaxDim = 65536;
constexpr int kThinMaxK = 32;
constexpr size_t kAlign = 256;

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t x, int64_t a) { return (x + a - 1) / a; }
inline int next_pow2(int64_t x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}
inline size_t dtype_size(int32_t dt) { return dt == DT_F32 ? 4 : 2; }

bool finite(float x) { return std::isfinite(x); }

// ---------------------------------------------------------------------------
// Plan
// ---------------------------------------------------------------------------
struct Plan {
  std::vector<MatDesc> desc;
  std::vector<Tile> k3, k5, cond;
  // Update tiles of the matrices whose Muon update the last combine does not
  // apply (a Dimuon step updates every matrix with k5).
  std::vector<Tile> k5u;
  // GEMM tile lists, one launch each; bm x bn tiles (symmetric products: square)
  struct GemmList { int bm, bn; std::vector<Tile> tiles; size_t off; };
  std::vector<GemmList> syrk, comb;
  // Combine lists of the product iterations, with some matrices' rows padded
  // to 256 (empty: comb serves them), and the rows each matrix's iterates
  // and B carry (KP, or KP rounded up to 256 when comb_pad pads it).  comb
  // itself serves the zero-iteration combine.
  std::vector<GemmList> comb_pad;
  std::vector<int32_t> rows;
  std::vector<uint16_t> gen;
  // thin matrices grouped by padded Gram side KP; one tile (matrix, slice)
  // per workgroup, one launch per phase and KP
  struct ThinGroup { int kp; std::vector<Tile> tiles; size_t off; };
  std::vector<ThinGroup> thin;
  // byte offsets in the workspace
  size_t desc_off = 0, scal_off = 0, k3_off = 0, k5_off = 0, k5u_off = 0, cond_off = 0, gen_off = 0;
  size_t table_bytes = 0;   // uploaded prefix of the workspace
  size_t total_bytes = 0;   // whole workspace
  std::vector<unsigned char> table;
};

// Thin path: Gram side k <= 32.  Each slice of the long side is one
// 256-thread workgroup holding max(16, KP) values per thread and array, i.e.
// 256 * max(16, KP) / KP positions (thin_slice_len).
bool is_thin(int64_t m, int64_t n) { return std::min(m, n) <= kThinMaxK; }

muon_status_t validate_config(const muon_config_t* cfg) {
  if (!cfg) return fail(MUON_ERR_INVALID_ARG, "cfg is NULL");
  const int32_t dts[4] = {cfg->w_dtype, cfg->g_dtype, cfg->mom_dtype, cfg->ns_dtype};
  for (int32_t dt : dts)
    if (dt != MUON_F32 && dt != MUON_BF16) return fail(MUON_ERR_DTYPE, "unknown dtype %d", dt);
  if (cfg->ns_steps < 0 || cfg->ns_steps > kMaxSteps)
    return fail(MUON_ERR_INVALID_ARG, "ns_steps %d outside [0, %d]", cfg->ns_steps, kMaxSteps);
  if (!finite(cfg->lr) || !finite(cfg->momentum) || !finite(cfg->weight_decay))
    return fail(MUON_ERR_INVALID_ARG, "lr, momentum and weight_decay must be finite");
  if (!finite(cfg->dimuon_eps) || cfg->dimuon_eps < 0.0f)
    return fail(MUON_ERR_INVALID_ARG, "dimuon_eps must be finite and >= 0");
  if (cfg->coeff_schedule) {
    for (int i = 0; i < 3 * cfg->ns_steps; ++i)
      if (!finite(cfg->coeff_schedule[i])) return fail(MUON_ERR_INVALID_ARG, "coeff_schedule[%d] is not finite", i);
  } else if (!finite(cfg->a) || !finite(cfg->b) || !finite(cfg->c)) {
    return fail(MUON_ERR_INVALID_ARG, "coefficients must be finite");
  }
  return MUON_OK;
}

muon_status_t validate_shapes(const muon_matrix_t* mats, int64_t count) {
  if (!mats) return fail(MUON_ERR_INVALID_ARG, "mats is NULL");
  if (count < 1) return fail(MUON_ERR_INVALID_ARG, "count %lld < 1", (long long)count);
  if (count > 65535) return fail(MUON_ERR_UNSUPPORTED, "count %lld > 65535", (long long)count);
  for (int64_t i = 0; i < count; ++i) {
    const muon_matrix_t& x = mats[i];
    if (x.m < 1 || x.n < 1) return fail(MUON_ERR_INVALID_ARG, "matrix %lld: shape %lld x %lld", (long long)i,
                                        (long long)x.m, (long long)x.n);
    if (x.m > kMaxDim || x.n > kMaxDim)
      return fail(MUON_ERR_UNSUPPORTED, "matrix %lld: shape %lld x %lld above %lld", (long long)i, (long long)x.m,
                  (long long)x.n, (long long)kMaxDim);
    if (!finite(x.update_scale)) return fail(MUON_ERR_INVALID_ARG, "matrix %lld: update_scale not finite", (long long)i);
  }
  return MUON_OK;
}

struct Range { uintptr_t lo, hi; int64_t mat; const char* what; bool writable; };

muon_status_t validate_buffers(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg) {
  std::vector<Range> rs;
  rs.reserve(count * 5);
  for (int64_t i = 0; i < count; ++i) {
    const muon_matrix_t& x = mats[i];
    const size_t elems = static_cast<size_t>(x.m) * static_cast<size_t>(x.n);
    struct B { const void* p; size_t bytes; const char* what; bool req; bool wr; } bs[5] = {
        {x.w, elems * dtype_size(cfg->w_dtype), "w", true, true},
        {x.g, elems * dtype_size(cfg->g_dtype), "g", true, false},
        {x.mom, elems * dtype_size(cfg->mom_dtype), "mom", true, true},
        {x.o_out, elems * 4, "o_out", false, true},
        {x.energy_out, static_cast<size_t>(x.m + x.n) * 4, "energy_out", false, true}};
    for (const B& b : bs) {
      if (!b.p) {
        if (b.req) return fail(MUON_ERR_INVALID_ARG, "matrix %lld: %s is NULL", (long long)i, b.what);
        continue;
      }
      if (reinterpret_cast<uintptr_t>(b.p) % 16 != 0)
        return fail(MUON_ERR_INVALID_ARG, "matrix %lld: %s is not 16-byte aligned", (long long)i, b.what);
      const uintptr_t lo = reinterpret_cast<uintptr_t>(b.p);
      rs.push_back({lo, lo + b.bytes, i, b.what, b.wr});
    }
  }
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  // Any overlap that involves a written buffer is an error.  Scanning in
  // address order, keep the written range reaching furthest and the range
  // (of any kind) reaching furthest.
  const Range* far_any = nullptr;
  const Range* far_wr = nullptr;
  for (const Range& r : rs) {
    const Range* hit = nullptr;
    if (r.writable && far_any && far_any->hi > r.lo) hit = far_any;
    else if (far_wr && far_wr->hi > r.lo) hit = far_wr;
    if (hit)
      return fail(MUON_ERR_ALIAS, "matrix %lld %s overlaps matrix %lld %s", (long long)r.mat, r.what,
                  (long long)hit->mat, hit->what);
    if (!far_any || r.hi > far_any->hi) far_any = &r;
    if (r.writable && (!far_wr || r.hi > far_wr->hi)) far_wr = &r;
  }
  return MUON_OK;
}

template <typename T>
size_t put(std::vector<unsigned char>& buf, size_t off, const std::vector<T>& v) {
  if (!v.empty()) std::memcpy(buf.data() + off, v.data(), v.size() * sizeof(T));
  return off;
}

// GEMM tiles of the general path.  A 256-wide tile side is possible where
// the padded side is a multiple of 256; those kernels run one workgroup per
// CU, the 128 x 128 symmetric products two (the 128 x 128 combine one).  For
// each product kind the batch takes the
// big tiles where they fit, unless the estimated time with 128 x 128 tiles
// everywhere is lower (few big tiles leave CUs idle in the last round).
// Within a matrix, tiles are listed in groups of tile rows, column by
// column, so that the workgroups running at once share operand panels:
// groups of two rows for the symmetric products and of eight for the
// combine (against four for both: MoE step 0.8% faster, 8 x 4096^2 0.25%).
constexpr int kCUs = 256;
constexpr double kSmallTileEff = 0.6;   // 128 x 128 kernel efficiency relative to the big tiles

void add_tiles(std::vector<Tile>& out, uint16_t mat, int rows, int cols, bool upper) {
  const int kGroup = upper ? 2 : 8;
  for (int g0 = 0; g0 < rows; g0 += kGroup)
    for (int tj = 0; tj < cols; ++tj)
      for (int ti = g0; ti < std::min(rows, g0 + kGroup); ++ti)
        if (!upper || ti <= tj) out.push_back({mat, static_cast<uint16_t>(ti), static_cast<uint16_t>(tj), 0});
}

// Matrix order for a symmetric product's tile list of bt x bt tiles.  Each
// XCD walks a contiguous run of the list (equal tile counts per run), and a
// tile's work is its K (the padded long side for the Gram), which differs
// between matrices of one batch: matrices are placed largest K first, each
// into the run with the least work that still has room for all its tiles.
// Returns the given order when the matrices do not pack into the runs.
std::vector<uint16_t> xcd_balanced_order(const Plan& p, int bt) {
  constexpr int kXcds = 8;
  std::vector<uint16_t> order = p.gen;
  auto tiles_of = [&](uint16_t i) {
    const int64_t rb = p.desc[i].KP / bt;
    return rb * (rb + 1) / 2;
  };
  int64_t n = 0;
  bool uniform = true;
  for (uint16_t i : order) {
    n += tiles_of(i);
    uniform = uniform && p.desc[i].NP == p.desc[order[0]].NP && p.desc[i].KP == p.desc[order[0]].KP;
  }
  if (uniform) return order;   // equal runs already carry equal work
  std::stable_sort(order.begin(), order.end(),
                   [&](uint16_t x, uint16_t y) { return p.desc[x].NP > p.desc[y].NP; });
  std::vector<int64_t> room(kXcds), work(kXcds, 0);
  for (int x = 0; x < kXcds; ++x) room[x] = n / kXcds + (x < n % kXcds ? 1 : 0);
  std::vector<std::vector<uint16_t>> runs(kXcds);
  for (uint16_t i : order) {
    const int64_t t = tiles_of(i);
    int best = -1;
    for (int x = 0; x < kXcds; ++x)
      if (room[x] >= t && (best < 0 || work[x] < work[best])) best = x;
    if (best < 0) return p.gen;
    runs[best].push_back(i);
    room[best] -= t;
    work[best] += t * p.desc[i].NP;
  }
  order.clear();
  for (const auto& r : runs) order.insert(order.end(), r.begin(), r.end());
  return order;
}

// Workgroups of a one-per-CU tile list run in rounds of 32 per XCD, each XCD
// walking its contiguous run of the list (xcd_remap), so each XCD would work
// through its own matrices.  When every matrix of the list has the same
// shape and the list fills whole rounds on all XCDs, the rounds are dealt
// out instead so that XCD x takes rounds x, x + 8, x + 16, ...: the eight
// XCDs then work on neighbouring rounds of the list at once, and operand
// panels that several of them read come from HBM once, the other XCDs
// finding them in the Infinity Cache.  Each tile's arithmetic is unchanged.
// 8 x 4096^2: Gram and polynomial 4.5% faster, combine 2%, step 3%; the MoE
// set measured unchanged.  Batches of mixed shapes keep the plain order.
void interleave_rounds(const Plan& p, Plan::GemmList& l) {
  constexpr size_t kRound = 32, kXcds = 8;
  if (l.bm * l.bn < 32768 || l.tiles.empty() || l.tiles.size() % (kRound * kXcds) != 0) return;
  const MatDesc& d0 = p.desc[l.tiles.front().mat];
  for (const Tile& t : l.tiles)
    if (p.desc[t.mat].KP != d0.KP || p.desc[t.mat].NP != d0.NP) return;
  const size_t rounds = l.tiles.size() / kRound;
  std::vector<Tile> out;
  out.reserve(l.tiles.size());
  for (size_t x = 0; x < kXcds; ++x)
    for (size_t r = x; r < rounds; r += kXcds)
      out.insert(out.end(), l.tiles.begin() + r * kRound, l.tiles.begin() + (r + 1) * kRound);
  l.tiles.swap(out);
}

void plan_gemm_tiles(Plan& p, bool bf16) {
  auto side = [&](int32_t x, bool big) { return (big && x % 256 == 0) ? 256 : 128; };
  // small_per_cu: 128 x 128 workgroups per CU (two for the symmetric
  // products; one for the combine, whose 128 x 128 kernel holds a four-buffer
  // ring).
  auto rounds_time = [&](const std::map<std::pair<int, int>, int64_t>& n, int small_per_cu) {
    double t = 0.0;
    for (const auto& kv : n) {
      const int bm = kv.first.first, bn = kv.first.second;
      if (bm == 128 && bn == 128)
        t += std::ceil(kv.second / double(small_per_cu * kCUs)) * small_per_cu / kSmallTileEff;
      else t += std::ceil(kv.second / double(kCUs)) * (bm * bn / 16384.0);
    }
    return t;
  };
  for (int kind = 0; kind < 2; ++kind) {   // 0: symmetric products, 1: combine
    bool big = false;
    if (bf16) {
      std::map<std::pair<int, int>, int64_t> nb, ns;
      for (uint16_t i : p.gen) {
        const MatDesc& d = p.desc[i];
        const int bm = side(d.KP, true), bn = kind == 0 ? bm : side(d.NP, true);
        const int64_t rb = d.KP / bm, cb = (kind == 0 ? d.KP : d.NP) / bn;
        nb[{bm, bn}] += kind == 0 ? rb * (rb + 1) / 2 : rb * cb;
        const int64_t rs = d.KP / 128, cs = (kind == 0 ? d.KP : d.NP) / 128;
        ns[{128, 128}] += kind == 0 ? rs * (rs + 1) / 2 : rs * cs;
      }
      const int per_cu = kind == 0 ? 2 : 1;
      big = rounds_time(nb, per_cu) < rounds_time(ns, per_cu);
    }
    auto& lists = kind == 0 ? p.syrk : p.comb;
    std::map<std::pair<int, int>, size_t> at;
    // 128 x 128 symmetric tiles (no tail split follows): runs balanced by K.
    const std::vector<uint16_t> order = (kind == 0 && !big) ? xcd_balanced_order(p, 128) : p.gen;
    for (uint16_t i : order) {
      MatDesc& d = p.desc[i];
      const int bm = side(d.KP, big), bn = kind == 0 ? bm : side(d.NP, big);
      auto it = at.find({bm, bn});
      if (it == at.end()) {
        it = at.emplace(std::make_pair(bm, bn), lists.size()).first;
        lists.push_back({bm, bn, {}, 0});
      }
      if (kind == 0) {
        add_tiles(lists[it->second].tiles, i, d.KP / bm, d.KP / bm, true);
      } else {
        add_tiles(lists[it->second].tiles, i, d.KP / bm, d.NP / bn, false);
        d.n_pz = (d.KP / 128) * (d.NP / 128);
      }
    }
    // A last round of big tiles that fills at most half the CUs (a quarter
    // for the combine, whose 128 x 128 tiles run one per CU) goes to the
    // 128 x 128 list instead: each big tile becomes its 128 x 128 sub-tiles
    // (for a symmetric product only those on or above the diagonal).
    if (big) {
      const std::vector<std::pair<int, int>> bigs = {{256, 256}, {128, 256}, {256, 128}};
      for (const auto& key : bigs) {
        const auto bi = at.find(key);
        if (bi == at.end()) continue;
        const size_t n = lists[bi->second].tiles.size(), r = n % kCUs;
        if (n <= static_cast<size_t>(kCUs) || r == 0 || r > static_cast<size_t>(kind == 0 ? kCUs / 2 : kCUs / 4))
          continue;
        auto si = at.find({128, 128});
        if (si == at.end()) {
          si = at.emplace(std::make_pair(128, 128), lists.size()).first;
          lists.push_back({128, 128, {}, 0});
        }
        std::vector<Tile>& bt = lists[bi->second].tiles;
        std::vector<Tile>& st = lists[si->second].tiles;
        const int fm = key.first / 128, fn = key.second / 128;
        for (size_t q = n - r; q < n; ++q) {
          const Tile t = bt[q];
          for (int ra = 0; ra < fm; ++ra)
            for (int cb = 0; cb < fn; ++cb) {
              const int ti = fm * t.ti + ra, tj = fn * t.tj + cb;
              if (kind == 1 || ti <= tj) st.push_back({t.mat, static_cast<uint16_t>(ti), static_cast<uint16_t>(tj), 0});
            }
        }
        bt.resize(n - r);
      }
    }
  }
  // A matrix whose padded Gram side is an odd multiple of 128 (at least
  // 1024) runs the combine on 256 x 256 tiles over its rows rounded up to
  // 256.  B and the iterates then carry 128 rows more; those rows of X' are
  // written but never read (the Gram reads rows below KP, and so does the
  // combine as its k operand), so they need no clearing, and the last
  // iteration's combine neither stores nor sums them.  The zero-iteration
  // combine (X read, no product) keeps the lists above.
  p.comb_pad.clear();
  p.rows.assign(p.desc.size(), 0);
  for (uint16_t i : p.gen) p.rows[i] = p.desc[i].KP;
  bool big_comb = false;
  for (const auto& l : p.comb) big_comb = big_comb || l.bm == 256 || l.bn == 256;
  if (bf16 && big_comb) {
    Plan::GemmList pad{256, 256, {}, 0};
    for (uint16_t i : p.gen) {
      const MatDesc& d = p.desc[i];
      if (d.KP % 256 == 128 && d.KP >= 1024 && d.NP % 256 == 0) {
        add_tiles(pad.tiles, i, (d.KP + 128) / 256, d.NP / 256, false);
        p.rows[i] = d.KP + 128;
      }
    }
    if (!pad.tiles.empty()) {
      for (const auto& l : p.comb) {
        Plan::GemmList c{l.bm, l.bn, {}, 0};
        for (const Tile& t : l.tiles)
          if (p.rows[t.mat] == p.desc[t.mat].KP) c.tiles.push_back(t);
        if (!c.tiles.empty()) p.comb_pad.push_back(std::move(c));
      }
      p.comb_pad.push_back(std::move(pad));
    }
  }
  for (auto* lists : {&p.syrk, &p.comb, &p.comb_pad})
    for (auto& l : *lists) interleave_rounds(p, l);
}

// Builds the plan.  `with_table` also serialises the uploaded prefix.
muon_status_t build_plan(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg, bool with_table,
                         Plan& p) {
  const size_t es = dtype_size(cfg->ns_dtype);
  p.desc.assign(count, MatDesc{});
  std::map<int, std::vector<Tile>> thin_groups;
  for (int64_t i = 0; i < count; ++i) {
    const muon_matrix_t& x = mats[i];
    MatDesc& d = p.desc[i];
    d.g = x.g;
    d.mom = x.mom;
    d.w = x.w;
    d.o_out = x.o_out;
    d.energy_out = x.energy_out;
    d.m = static_cast<int32_t>(x.m);
    d.n = static_cast<int32_t>(x.n);
    d.k = static_cast<int32_t>(std::min(x.m, x.n));
    d.N = static_cast<int32_t>(std::max(x.m, x.n));
    d.tall = x.m > x.n ? 1 : 0;
    d.update_scale = x.update_scale;
    d.scal_idx = static_cast<int32_t>(i);
    if (is_thin(x.m, x.n)) {
      d.KP = next_pow2(d.k);
      d.NP = d.N;
      d.L = thin_slice_len(d.KP);
      d.S = static_cast<int32_t>(ceil_div(d.N, d.L));
      for (int sl = 0; sl < d.S; ++sl)
        thin_groups[d.KP].push_back({static_cast<uint16_t>(i), static_cast<uint16_t>(sl), 0, 0});
    } else {
      d.KP = static_cast<int32_t>(round_up(d.k, kPad));
      d.NP = static_cast<int32_t>(round_up(d.N, kPad));
      d.mpad = d.tall ? d.NP : d.KP;
      d.npad = d.tall ? d.KP : d.NP;
      d.ncb = static_cast<int32_t>(ceil_div(d.n, 64));
      d.nrb = static_cast<int32_t>(ceil_div(d.m, 64));
      d.n_pn = (d.KP / 64) * (d.NP / 64);
      p.gen.push_back(static_cast<uint16_t>(i));
      for (int ti = 0; ti < d.KP / 64; ++ti)
        for (int tj = 0; tj < d.NP / 64; ++tj) p.k3.push_back({static_cast<uint16_t>(i), (uint16_t)ti, (uint16_t)tj, 0});
      // A Muon step's last bf16 combine applies the update itself where every
      // row of W is a whole number of 16-byte bf16 runs.
      d.fuse_upd = (cfg->ns_dtype == MUON_BF16 && cfg->w_dtype == MUON_BF16 && cfg->ns_steps > 0 && d.n % 8 == 0)
                       ? 1 : 0;
      for (int ti = 0; ti < ceil_div(d.m, 64); ++ti)
        for (int tj = 0; tj < ceil_div(d.n, 64); ++tj) {
          p.k5.push_back({static_cast<uint16_t>(i), (uint16_t)ti, (uint16_t)tj, 0});
          if (!d.fuse_upd) p.k5u.push_back(p.k5.back());
        }
      d.ncond = static_cast<int32_t>(ceil_div(d.mpad + d.npad, 256));
      for (int c = 0; c < d.ncond; ++c) p.cond.push_back({static_cast<uint16_t>(i), static_cast<uint16_t>(c), 0, 0});
    }
  }
  for (auto& kv : thin_groups) p.thin.push_back({kv.first, kv.second, 0});
  if (count > 65535) return fail(MUON_ERR_UNSUPPORTED, "too many matrices");
  plan_gemm_tiles(p, cfg->ns_dtype == MUON_BF16);

  // Table prefix: descriptors, scalars, tile lists, id lists.
  size_t off = kAlign;   // first 256 bytes reserved
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, kAlign);
    return o;
  };
  p.desc_off = take(sizeof(MatDesc) * count);
  p.scal_off = take(sizeof(MatScal) * count);
  p.k3_off = take(sizeof(Tile) * p.k3.size());
  for (auto& l : p.syrk) l.off = take(sizeof(Tile) * l.tiles.size());
  for (auto& l : p.comb) l.off = take(sizeof(Tile) * l.tiles.size());
  for (auto& l : p.comb_pad) l.off = take(sizeof(Tile) * l.tiles.size());
  p.k5_off = take(sizeof(Tile) * p.k5.size());
  p.k5u_off = take(sizeof(Tile) * p.k5u.size());
  p.cond_off = take(sizeof(Tile) * p.cond.size());
  p.gen_off = take(sizeof(uint16_t) * p.gen.size());
  for (auto& g : p.thin) g.off = take(sizeof(Tile) * g.tiles.size());
  p.table_bytes = off;

  // Per-matrix scratch of the thin path.
  for (int64_t i = 0; i < count; ++i) {
    MatDesc& d = p.desc[i];
    if (d.S == 0) continue;
    const size_t npair = static_cast<size_t>(d.KP) * (d.KP + 1) / 2;
    const size_t cache = (static_cast<size_t>(d.S) * d.KP + d.N + d.S) * 4;
    d.te_off[0] = take(cache);
    d.te_off[1] = take(cache);
    d.tdl_off = take(static_cast<size_t>(d.N) * 4);
    d.tdg_off = take(static_cast<size_t>(d.KP) * 4);
    d.tg_off = take(static_cast<size_t>(d.S) * npair * 8);
    d.tg2_off = take(static_cast<size_t>(d.S) * npair * 8);
  }
  // Per-matrix scratch of the general path.
  for (uint16_t i : p.gen) {
    MatDesc& d = p.desc[i];
    const size_t kn = static_cast<size_t>(d.KP) * d.NP;
    const size_t xn = static_cast<size_t>(p.rows[i]) * d.NP;   // iterates: rows the combine writes
    // X^T copies only for the fp32 products; the bf16 combine reads X itself.
    for (int b = 0; b < 4; ++b) d.x_off[b] = ((b & 1) && cfg->ns_dtype == MUON_BF16) ? -1 : take(xn * es);
    d.a_off = take(static_cast<size_t>(d.KP) * d.KP * es);
    d.b_off = take(static_cast<size_t>(p.rows[i]) * d.KP * es);
    d.z_off = take(kn * es);
    d.dr_off = take(static_cast<size_t>(d.mpad) * 4);
    d.dc_off = take(static_cast<size_t>(d.npad) * 4);
    d.cm_off = take(static_cast<size_t>(d.ncond) * 8);
    for (int par = 0; par < 2; ++par)
      d.ge_off[par] = take((static_cast<size_t>(d.ncb) * d.m + static_cast<size_t>(d.nrb) * d.n) * 4);
    d.pn_off = take(static_cast<size_t>(d.n_pn) * 4);
    d.pz_off = take(static_cast<size_t>(d.n_pz) * 8);
  }
  p.total_bytes = off;

  if (with_table) {
    p.table.assign(p.table_bytes, 0);
    std::memcpy(p.table.data() + p.desc_off, p.desc.data(), sizeof(MatDesc) * count);
    put(p.table, p.k3_off, p.k3);
    for (auto& l : p.syrk) put(p.table, l.off, l.tiles);
    for (auto& l : p.comb) put(p.table, l.off, l.tiles);
    for (auto& l : p.comb_pad) put(p.table, l.off, l.tiles);
    put(p.table, p.k5_off, p.k5);
    put(p.table, p.k5u_off, p.k5u);
    put(p.table, p.cond_off, p.cond);
    put(p.table, p.gen_off, p.gen);
    for (auto& g : p.thin) put(p.table, g.off, g.tiles);
  }
  return MUON_OK;
}

// ---------------------------------------------------------------------------
// Descriptor upload: the table is copied from a pinned host buffer into the
// workspace prefix on the step's stream.  An event records when the copy has
// consumed the host buffer, so the buffer is never overwritten early.
// ---------------------------------------------------------------------------
struct Staging {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;

  // True when the buffer may be written: no copy from it is in flight.
  bool idle() {
    if (!pending) return true;
    if (hipEventQuery(ev) == hipSuccess) pending = false;
    return !pending;
  }

  muon_status_t upload(const std::vector<unsigned char>& table, void* dst, hipStream_t s) {
    hipError_t err;
    if (pending) {
      if ((err = hipEventSynchronize(ev)) != hipSuccess)
        return fail(MUON_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(err));
      pending = false;
    }
    if (cap < table.size()) {
      if (host) (void)hipHostFree(host);
      host = nullptr;
      cap = 0;
      if ((err = hipHostMalloc(&host, table.size(), hipHostMallocDefault)) != hipSuccess) {
        host = nullptr;
        return fail(MUON_ERR_HIP, "hipHostMalloc(%zu): %s", table.size(), hipGetErrorString(err));
      }
      cap = table.size();
    }
    if (!ev && (err = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
      ev = nullptr;
      return fail(MUON_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    std::memcpy(host, table.data(), table.size());
    if ((err = hipMemcpyAsync(dst, host, table.size(), hipMemcpyHostToDevice, s)) != hipSuccess)
      return fail(MUON_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(err));
    if ((err = hipEventRecord(ev, s)) != hipSuccess)
      return fail(MUON_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(err));
    pending = true;
    return MUON_OK;
  }

  void release() {
    if (pending && ev) (void)hipEventSynchronize(ev);
    if (ev) (void)hipEventDestroy(ev);
    if (host) (void)hipHostFree(host);
    host = nullptr;
    ev = nullptr;
    cap = 0;
    pending = false;
  }
};

// Staging buffers of the stateless calls, per host thread.  A call takes an
// idle buffer (its previous copy has completed), or a new one while the
// thread holds fewer than kPoolMax; only a thread with kPoolMax copies in
// flight waits, for its oldest.  The buffers are freed when the thread exits.
constexpr size_t kPoolMax = 64;
struct StagingPool {
  std::vector<Staging*> slots;
  size_t oldest = 0;   // slot waited on when every slot is busy

  Staging* take() {
    for (Staging* st : slots)
      if (st->idle()) return st;
    if (slots.size() < kPoolMax) {
      slots.push_back(new Staging());
      return slots.back();
    }
    Staging* st = slots[oldest];
    oldest = (oldest + 1) % slots.size();
    return st;   // upload() waits for its copy
  }

  ~StagingPool() {
    for (Staging* st : slots) {
      st->release();
      delete st;
    }
  }
};
thread_local StagingPool g_pool;

// ---------------------------------------------------------------------------
// Shared pieces of a step
// ---------------------------------------------------------------------------
muon_status_t prepare(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg, void* ws,
                      size_t ws_bytes, Plan& p) {
  muon_status_t st;
  if ((st = validate_config(cfg)) != MUON_OK) return st;
  if ((st = validate_shapes(mats, count)) != MUON_OK) return st;
  if ((st = validate_buffers(mats, count, cfg)) != MUON_OK) return st;
  if ((st = build_plan(mats, count, cfg, true, p)) != MUON_OK) return st;
  if (!ws) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return fail(MUON_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (ws_bytes < p.total_bytes)
    return fail(MUON_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, p.total_bytes);
  // The workspace must not overlap any caller buffer.
  const uintptr_t lo = reinterpret_cast<uintptr_t>(ws), hi = lo + p.total_bytes;
  for (int64_t i = 0; i < count; ++i) {
    const muon_matrix_t& x = mats[i];
    const size_t elems = static_cast<size_t>(x.m) * x.n;
    const void* ps[5] = {x.w, x.g, x.mom, x.o_out, x.energy_out};
    const size_t bytes[5] = {elems * dtype_size(cfg->w_dtype), elems * dtype_size(cfg->g_dtype),
                             elems * dtype_size(cfg->mom_dtype), elems * 4, static_cast<size_t>(x.m + x.n) * 4};
    for (int b = 0; b < 5; ++b) {
      if (!ps[b]) continue;
      const uintptr_t plo = reinterpret_cast<uintptr_t>(ps[b]);
      if (plo < hi && lo < plo + bytes[b])
        return fail(MUON_ERR_ALIAS, "matrix %lld buffer %d overlaps the workspace", (long long)i, b);
    }
  }
  return MUON_OK;
}

StepArgs make_args(const Plan& p, const muon_config_t& cfg, void* ws, bool dimuon) {
  char* base = static_cast<char*>(ws);
  StepArgs a{};
  a.desc = reinterpret_cast<const MatDesc*>(base + p.desc_off);
  a.scal = reinterpret_cast<MatScal*>(base + p.scal_off);
  a.ws = base;
  a.mu = cfg.momentum;
  a.lr = cfg.lr;
  a.eps = cfg.dimuon_eps;
  a.weight_decay = cfg.weight_decay;
  a.g_dt = cfg.g_dtype;
  a.mom_dt = cfg.mom_dtype;
  a.w_dt = cfg.w_dtype;
  a.ns_dt = cfg.ns_dtype;
  a.nesterov = cfg.nesterov ? 1 : 0;
  a.dimuon = dimuon ? 1 : 0;
  return a;
}

void make_coeffs(const muon_config_t& cfg, Coeffs* cf) {
  for (int t = 0; t < cfg.ns_steps; ++t) {
    if (cfg.coeff_schedule)
      cf[t] = {cfg.coeff_schedule[3 * t], cfg.coeff_schedule[3 * t + 1], cfg.coeff_schedule[3 * t + 2]};
    else
      cf[t] = {cfg.a, cfg.b, cfg.c};
  }
}

#define MUON_HIP_TRY(expr)                                                                 \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(MUON_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// Launch, then record the hook's event for this launch kind.
#define MUON_LAUNCH(kind, expr)              \
  do {                                       \
    MUON_HIP_TRY(expr);                      \
    MUON_HIP_TRY(hook_record((kind), s));    \
  } while (0)

// The launch sequence of one step; the descriptor table is already on the
// device (ordered before these launches on stream s).
// `parity` selects the energy caches (thin and general path) holding the
// energies of M_{t-1}; `cached` says whether they are valid (else they are
// computed first).  The step writes the energies of M_t into the others.
muon_status_t launch_all(const Plan& p, const StepArgs& a, const Coeffs* cf, int ns_steps, bool dimuon,
                         int parity, bool cached, hipStream_t s) {
  char* base = a.ws;
  auto tl = [&](size_t off) { return reinterpret_cast<const Tile*>(base + off); };
  auto il = [&](size_t off) { return reinterpret_cast<const uint16_t*>(base + off); };
  g_hook.next = 0;
  MUON_HIP_TRY(hook_record(MUON_LAUNCH_START, s));
  for (const auto& g : p.thin) {
    const int nt = static_cast<int>(g.tiles.size());
    if (dimuon && !cached)
      MUON_LAUNCH(MUON_LAUNCH_THIN_ENERGY, launch_thin_energy(a, tl(g.off), nt, g.kp, parity, s));
    MUON_LAUNCH(MUON_LAUNCH_THIN_A, launch_thin_a(a, tl(g.off), nt, g.kp, parity, s));
    MUON_LAUNCH(MUON_LAUNCH_THIN, launch_thin_b(a, tl(g.off), nt, g.kp, ns_steps, cf, parity, s));
  }
  if (!p.gen.empty()) {
    const int ng = static_cast<int>(p.gen.size());
    const int n3 = static_cast<int>(p.k3.size());
    if (dimuon) {
      // The factors need the energies of M_{t-1} (a reduction over whole rows
      // and columns) before anything is scaled.  The previous step of a plan
      // left them in cache `parity`; otherwise a pass over M_{t-1} puts them
      // there first.
      const int nc = static_cast<int>(p.cond.size());
      if (!cached) MUON_LAUNCH(MUON_LAUNCH_ENERGY, launch_energy(a, tl(p.k3_off), n3, parity, s));
      MUON_LAUNCH(MUON_LAUNCH_CONDITION, launch_cond_energy(a, tl(p.cond_off), nc, parity, s));
      MUON_LAUNCH(MUON_LAUNCH_CONDITION, launch_cond_factor(a, tl(p.cond_off), nc, s));
    }
    // Momentum, the energies of M_t (Dimuon, into the other cache) and the
    // prescale in one pass.
    MUON_LAUNCH(MUON_LAUNCH_MOMENTUM_PRESCALE, launch_prescale(a, tl(p.k3_off), n3, dimuon, parity ^ 1, s));
    MUON_LAUNCH(MUON_LAUNCH_NORM, launch_norm_finalize(a, il(p.gen_off), ng, s));
    auto nt = [](const Plan::GemmList& l) { return static_cast<int>(l.tiles.size()); };
    if (ns_steps == 0)
      for (const auto& l : p.comb)
        MUON_LAUNCH(MUON_LAUNCH_COMBINE, launch_combine(a, tl(l.off), nt(l), l.bm, l.bn, 0, 1, true, true, false,
                                                        Coeffs{1.0f, 0.0f, 0.0f}, s));
    for (int t = 0; t < ns_steps; ++t) {
      const int src = t & 1, dst = src ^ 1;
      const bool first = t == 0, last = t == ns_steps - 1;
      for (const auto& l : p.syrk)
        MUON_LAUNCH(MUON_LAUNCH_GRAM, launch_syrk(a, tl(l.off), nt(l), l.bm, 0, src, first, cf[t], s));
      for (const auto& l : p.syrk)
        MUON_LAUNCH(MUON_LAUNCH_POLY, launch_syrk(a, tl(l.off), nt(l), l.bm, 1, src, first, cf[t], s));
      for (const auto& l : p.comb_pad.empty() ? p.comb : p.comb_pad)
        MUON_LAUNCH(MUON_LAUNCH_COMBINE,
                    launch_combine(a, tl(l.off), nt(l), l.bm, l.bn, src, dst, first, last, true, cf[t], s));
    }
    if (dimuon) MUON_LAUNCH(MUON_LAUNCH_POSTNORM, launch_post_finalize(a, il(p.gen_off), ng, s));
    // Muon: matrices with fuse_upd were updated by the last combine.
    const std::vector<Tile>& upd = dimuon ? p.k5 : p.k5u;
    if (!upd.empty())
      MUON_LAUNCH(MUON_LAUNCH_UPDATE,
                  launch_update(a, tl(dimuon ? p.k5_off : p.k5u_off), static_cast<int>(upd.size()), s));
  }
  g_hook.last_count = g_hook.next;
  return MUON_OK;
}

muon_status_t run_step(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg, void* ws,
                       size_t ws_bytes, void* stream_ptr, bool dimuon) {
  g_last_error.clear();
  Plan p;
  muon_status_t st = prepare(mats, count, cfg, ws, ws_bytes, p);
  if (st != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream_ptr);
  if ((st = g_pool.take()->upload(p.table, ws, s)) != MUON_OK) return st;
  Coeffs cf[kMaxSteps];
  make_coeffs(*cfg, cf);
  return launch_all(p, make_args(p, *cfg, ws, dimuon), cf, cfg->ns_steps, dimuon, 0, false, s);
}

// ---------------------------------------------------------------------------
// Allocation-free step (muon_step_noalloc): the workspace is `scratch`, a
// static device array each GPU holds until the process ends, and the
// descriptor table reaches it through kernel arguments, so the call needs
// neither a device allocation nor a host staging buffer.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = MUON_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's `scratch`, looked up once per device with
// that device current.  Host code uses only this address: the array's own
// name is a host-side stand-in, not a device address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

muon_status_t scratch_base(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MUON_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(MUON_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MUON_OK;
}

// One piece of the descriptor table, carried by value as a kernel argument
// (2 KB: 128 threads of 16 bytes).
constexpr int kPieceBytes = 2048;
struct alignas(16) TablePiece {
  uint4 v[kPieceBytes / 16];
};

__global__ __launch_bounds__(kPieceBytes / 16) void k_put_table(uint4* dst, TablePiece piece, int n16) {
  const int i = threadIdx.x;
  if (i < n16) dst[i] = piece.v[i];
}

muon_status_t run_step_noalloc(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg, bool dimuon,
                               void* stream_ptr) {
  g_last_error.clear();
  muon_status_t st;
  if ((st = validate_config(cfg)) != MUON_OK) return st;
  if ((st = validate_shapes(mats, count)) != MUON_OK) return st;
  if ((st = validate_buffers(mats, count, cfg)) != MUON_OK) return st;
  {
    Plan sized;
    if ((st = build_plan(mats, count, cfg, false, sized)) != MUON_OK) return st;
    if (sized.total_bytes > kScratchBytes)
      return fail(MUON_ERR_WORKSPACE, "batch needs %zu bytes of workspace, above the %zu-byte static scratch",
                  sized.total_bytes, kScratchBytes);
  }
  void* base = nullptr;
  if ((st = scratch_base(&base)) != MUON_OK) return st;
  Plan p;
  if ((st = prepare(mats, count, cfg, base, kScratchBytes, p)) != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream_ptr);
  // The table, zero-padded to whole 16-byte units, piece by piece (its size
  // is a multiple of 256 bytes).
  const size_t n16 = p.table.size() / 16;
  for (size_t at = 0; at < n16; at += kPieceBytes / 16) {
    TablePiece piece;
    const size_t cnt = std::min<size_t>(kPieceBytes / 16, n16 - at);
    std::memset(&piece, 0, sizeof(piece));
    std::memcpy(&piece, p.table.data() + at * 16, cnt * 16);
    hipLaunchKernelGGL(k_put_table, dim3(1), dim3(kPieceBytes / 16), 0, s, static_cast<uint4*>(base) + at, piece,
                       static_cast<int>(cnt));
    MUON_HIP_TRY(hipGetLastError());
  }
  Coeffs cf[kMaxSteps];
  make_coeffs(*cfg, cf);
  return launch_all(p, make_args(p, *cfg, base, dimuon), cf, cfg->ns_steps, dimuon, 0, false, s);
}

}  // namespace
}  // namespace muon

// A prepared batch: validated, planned and uploaded once.
struct muon_plan {
  muon::Plan p;
  muon_config_t cfg;
  std::vector<float> schedule;
  muon::Coeffs cf[muon::kMaxSteps];
  bool dimuon;
  void* ws;
  muon::Staging staging;
  int parity = 0;          // energy cache holding the energies of the current momentum
  bool cached = false;     // whether that cache is valid
  // Graph replay (muon_plan_set_graph): one instantiated graph per state of
  // the launch sequence (the energy-cache parity for Dimuon), captured on a
  // private stream of the plan.
  bool graph_on = false;
  hipStream_t capture = nullptr;
  hipGraphExec_t exec[2] = {nullptr, nullptr};

  void drop_graphs() {
    for (auto& e : exec)
      if (e) {
        (void)hipGraphExecDestroy(e);
        e = nullptr;
      }
  }
};

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

void muon_config_default(muon_config_t* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->lr = 0.02f;
  cfg->momentum = 0.95f;
  cfg->ns_steps = 5;
  cfg->a = 3.4445f;
  cfg->b = -4.7750f;
  cfg->c = 2.0315f;
  cfg->coeff_schedule = nullptr;
  cfg->w_dtype = MUON_BF16;
  cfg->g_dtype = MUON_BF16;
  cfg->mom_dtype = MUON_BF16;
  cfg->ns_dtype = MUON_BF16;
  cfg->dimuon_eps = 1e-4f;
  cfg->nesterov = 0;
  cfg->weight_decay = 0.0f;
}

muon_status_t muon_workspace_bytes(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg,
                                   size_t* bytes) {
  using namespace muon;
  g_last_error.clear();
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  muon_status_t st;
  if ((st = validate_config(cfg)) != MUON_OK) return st;
  if ((st = validate_shapes(mats, count)) != MUON_OK) return st;
  Plan p;
  if ((st = build_plan(mats, count, cfg, false, p)) != MUON_OK) return st;
  *bytes = p.total_bytes;
  return MUON_OK;
}

muon_status_t muon_step(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return muon::run_step(mats, count, cfg, workspace, workspace_bytes, stream, false);
}

muon_status_t dimuon_step(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return muon::run_step(mats, count, cfg, workspace, workspace_bytes, stream, true);
}

muon_status_t muon_step_noalloc(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg, int32_t dimuon,
                                void* stream) {
  return muon::run_step_noalloc(mats, count, cfg, dimuon != 0, stream);
}

int32_t muon_set_launch_events(void* const* events, int32_t* kinds, int32_t n) {
  const int32_t last = muon::g_hook.last_count;
  muon::g_hook.events = events;
  muon::g_hook.kinds = kinds;
  muon::g_hook.n = events ? (n > 0 ? n : 0) : 0;
  muon::g_hook.next = 0;
  return last;
}

muon_status_t muon_plan_create(const muon_matrix_t* mats, int64_t count, const muon_config_t* cfg, int32_t dimuon,
                               void* workspace, size_t workspace_bytes, void* stream, muon_plan_t** plan) {
  using namespace muon;
  g_last_error.clear();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  *plan = nullptr;
  muon_plan* pl = new muon_plan();
  muon_status_t st = prepare(mats, count, cfg, workspace, workspace_bytes, pl->p);
  if (st == MUON_OK) st = pl->staging.upload(pl->p.table, workspace, static_cast<hipStream_t>(stream));
  if (st != MUON_OK) {
    pl->staging.release();
    delete pl;
    return st;
  }
  pl->cfg = *cfg;
  if (cfg->coeff_schedule) {
    pl->schedule.assign(cfg->coeff_schedule, cfg->coeff_schedule + 3 * cfg->ns_steps);
    pl->cfg.coeff_schedule = pl->schedule.data();
  }
  make_coeffs(pl->cfg, pl->cf);
  pl->dimuon = dimuon != 0;
  pl->ws = workspace;
  *plan = pl;
  return MUON_OK;
}

muon_status_t muon_plan_step(muon_plan_t* plan, void* stream) {
  using namespace muon;
  g_last_error.clear();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const StepArgs args = make_args(plan->p, plan->cfg, plan->ws, plan->dimuon);
  muon_status_t st = MUON_OK;
  // Graph replay for steps whose sequence is fixed: every Muon step, and
  // Dimuon steps with cached energies (the first step after creation or a
  // reset also computes them, and runs eagerly).  Steps timed through the
  // launch-event hook run eagerly too.
  const bool replay = plan->graph_on && (!plan->dimuon || plan->cached) && !g_hook.events;
  if (replay) {
    hipGraphExec_t& exec = plan->exec[plan->dimuon ? plan->parity : 0];
    if (!exec) {
      hipGraph_t graph = nullptr;
      MUON_HIP_TRY(hipStreamBeginCapture(plan->capture, hipStreamCaptureModeThreadLocal));
      st = launch_all(plan->p, args, plan->cf, plan->cfg.ns_steps, plan->dimuon, plan->parity, plan->cached,
                      plan->capture);
      const hipError_t e = hipStreamEndCapture(plan->capture, &graph);
      if (st != MUON_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
      }
      if (e != hipSuccess) return fail(MUON_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
      const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (ei != hipSuccess) {
        exec = nullptr;
        return fail(MUON_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(ei));
      }
    }
    MUON_HIP_TRY(hipGraphLaunch(exec, s));
  } else {
    st = launch_all(plan->p, args, plan->cf, plan->cfg.ns_steps, plan->dimuon, plan->parity, plan->cached, s);
  }
  if (st == MUON_OK && plan->dimuon) {
    // Pass A wrote the energies of the new momentum into the other cache.
    plan->parity ^= 1;
    plan->cached = true;
  }
  return st;
}

muon_status_t muon_plan_reset(muon_plan_t* plan) {
  using namespace muon;
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  plan->cached = false;
  return MUON_OK;
}

muon_status_t muon_plan_set_lr(muon_plan_t* plan, float lr) {
  using namespace muon;
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  if (!finite(lr)) return fail(MUON_ERR_INVALID_ARG, "lr must be finite");
  if (lr != plan->cfg.lr) plan->drop_graphs();   // the rate is a kernel argument of the captured launches
  plan->cfg.lr = lr;
  return MUON_OK;
}

muon_status_t muon_plan_set_graph(muon_plan_t* plan, int32_t enable) {
  using namespace muon;
  g_last_error.clear();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  if (enable && !plan->capture) {
    const hipError_t e = hipStreamCreateWithFlags(&plan->capture, hipStreamNonBlocking);
    if (e != hipSuccess) {
      plan->capture = nullptr;
      return fail(MUON_ERR_HIP, "hipStreamCreateWithFlags: %s", hipGetErrorString(e));
    }
  }
  plan->graph_on = enable != 0;
  return MUON_OK;
}

void muon_plan_destroy(muon_plan_t* plan) {
  if (!plan) return;
  plan->staging.release();
  plan->drop_graphs();
  if (plan->capture) (void)hipStreamDestroy(plan->capture);
  delete plan;
}

const char* muon_status_string(muon_status_t status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARG: return "invalid argument";
    case MUON_ERR_DTYPE: return "unsupported dtype";
    case MUON_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MUON_ERR_ALIAS: return "buffers overlap";
    case MUON_ERR_HIP: return "HIP runtime error";
    case MUON_ERR_UNSUPPORTED: return "unsupported shape or count";
  }
  return "unknown status";
}

const char* muon_last_error(void) { return muon::g_last_error.c_str(); }

int32_t muon_abi_version(void) { return MUON_ABI_VERSION; }

}  // extern "C"
