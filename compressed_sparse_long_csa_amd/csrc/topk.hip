// Top-k selector (topk_select).
//
// Source: 硅星人 article on DeepSeek V4, CSA paragraph (the top-k selector
// keeps the 512 most relevant compressed blocks, 1024 for Pro); DeepSeek-V4
// blog, index visibility (the top-k selector names the entries a CSA query
// sees).  Ties go to the lower index and the output is ascending, which is
// this library's reading of what the pages leave open.
//
// One workgroup of 1024 threads (16 waves) per row.  Wave w owns the contiguous
// range [w*C, (w+1)*C) of the row and reads it 64 consecutive scores at a time
// (coalesced).  Scores are canonicalised on load (-0 -> +0, NaN -> -inf); slots
// past the end of the row hold NaN, which no comparison selects.
//  1. the first pass finds min / max of the finite scores (and, for rows of
//     up to kStageMax scores, keeps the row in LDS for the later passes);
//  2. a 2048-bin histogram linear in the score over [min, max] (monotone
//     float binning; LDS integer atomics are order-free) gives the bin b*
//     holding the k-th largest score and `need`, the number of its elements
//     that are selected;
//  3. one pass appends the elements of b* (order key, index) to an LDS list
//     and counts, per wave, the elements of higher bins;
//  4. among the candidates the threshold T and the number of elements equal
//     to T to take (lowest indices first) are found exactly: by direct
//     ranking for few candidates, else by key-space histograms over the LDS
//     list (bins of power-of-two width) -- a b* too large to keep refines
//     over the row itself;
//  5. every wave places its selected indices in order (a running count plus
//     the ballot prefix count of each 64-score step) into an LDS copy of the
//     output row, which is then stored with coalesced writes.
// Wave reductions and scans use DPP row operations and lane reads, so a block
// reduction costs one barrier.  The result is the exact set, ascending,
// whatever the batch or launch.  Loads and stores go through buffer
// descriptors, so slots past a row's end need neither branches nor clamps.
#include <atomic>

#include "kernels.hpp"

// Candidate workspace of topk_select_noalloc: one static array per GPU the
// library runs on, held until the process ends.  Host code must not use this
// name as a device address; it takes the address hipGetSymbolAddress reports
// for the current device (topk_scratch below).
static __device__ __align__(256) uint8_t scratch[csa::kTopkScratchBytes];

namespace csa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kStreamJ = 8;                // independent loads per streamed step
constexpr int kLdsJ = 4;                   // LDS reads per staged step
constexpr int kMaxCand = 2048;             // candidates kept in LDS
static_assert(2 * kMaxCand >= 4096, "the candidate arrays double as the output staging row");
constexpr int kRankDirect = 96;            // candidates ranked by direct counting
constexpr uint32_t kStageMax = 33 * 1024;  // rows staged in LDS (wave ranges included)
constexpr uint32_t kStageSlack = 64 * (kLdsJ - 1);

// Order-preserving key of a canonical (non-NaN, no -0) float, and back.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}
__device__ __forceinline__ float canon(float v) { return v == v ? v + 0.0f : -INFINITY; }

// ---------------------------------------------------------------- DPP wave ops
// update_dpp with old = identity: lanes whose source lies outside the row (or
// whose row is masked off) receive the identity.
template <int Ctrl, int RowMask>
__device__ __forceinline__ uint32_t dpp(uint32_t v, uint32_t identity) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(identity),
                                                           static_cast<int>(v), Ctrl, RowMask,
                                                           0xf, false));
}
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele shifts inside each
// 16-lane row, then the row totals carried by the row broadcasts.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<0x111, 0xf>(v, 0u);      // row_shr:1
  v += dpp<0x112, 0xf>(v, 0u);      // row_shr:2
  v += dpp<0x114, 0xf>(v, 0u);      // row_shr:4
  v += dpp<0x118, 0xf>(v, 0u);      // row_shr:8
  v += dpp<0x142, 0xa>(v, 0u);      // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xc>(v, 0u);      // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ uint32_t wave_total(uint32_t v) {
  return lane_read(wave_incl_scan(v), 63);
}
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  v = umin(v, dpp<0x111, 0xf>(v, 0xffffffffu));
  v = umin(v, dpp<0x112, 0xf>(v, 0xffffffffu));
  v = umin(v, dpp<0x114, 0xf>(v, 0xffffffffu));
  v = umin(v, dpp<0x118, 0xf>(v, 0xffffffffu));
  return umin(umin(lane_read(v, 15), lane_read(v, 31)), umin(lane_read(v, 47), lane_read(v, 63)));
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = umax(v, dpp<0x111, 0xf>(v, 0u));
  v = umax(v, dpp<0x112, 0xf>(v, 0u));
  v = umax(v, dpp<0x114, 0xf>(v, 0u));
  v = umax(v, dpp<0x118, 0xf>(v, 0u));
  return umax(umax(lane_read(v, 15), lane_read(v, 31)), umax(lane_read(v, 47), lane_read(v, 63)));
}
// Position of this lane among the set lanes of `mask` below it.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

struct TopkSmem {
  uint32_t hist[kBins];
  uint32_t cand_key[kMaxCand];
  uint32_t cand_idx[kMaxCand];
  uint32_t wa[kWaves];             // per wave: elements with key > T
  uint32_t wb[kWaves];             // per wave: elements with key == T
  uint32_t wlo[kWaves];
  uint32_t whi[kWaves];
  uint32_t sh[4];                  // 0 bin, 1 above, 2 n_cand, 3 T
};

// Block min / max of per-thread keys (one barrier; the caller's next barrier
// must precede any reuse of wlo / whi).
__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, TopkSmem& sm) {
  const int wv = threadIdx.x >> 6;
  lo = wave_min(lo);
  hi = wave_max(hi);
  if ((threadIdx.x & 63) == 0) { sm.wlo[wv] = lo; sm.whi[wv] = hi; }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) { lo = umin(lo, sm.wlo[w]); hi = umax(hi, sm.whi[w]); }
}

// Bin b with above(b) < need <= above(b) + hist[b], counting from the top
// bin; needs the histogram published by a barrier and need <= its total.
// Thread t owns bins 2047 - 2t and 2046 - 2t.
__device__ __forceinline__ void find_bin(TopkSmem& sm, uint32_t need, uint32_t* bin,
                                         uint32_t* above) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int top = kBins - 1 - 2 * tid;
  const uint32_t c0 = sm.hist[top], c1 = sm.hist[top - 1];
  const uint32_t incl = wave_incl_scan(c0 + c1);
  if (lane == 63) sm.wlo[wv] = incl;
  __syncthreads();
  uint32_t run = incl - c0 - c1;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) run += w < wv ? sm.wlo[w] : 0u;
  if (run < need && need <= run + c0) { sm.sh[0] = top; sm.sh[1] = run; }
  if (run + c0 < need && need <= run + c0 + c1) { sm.sh[0] = top - 1; sm.sh[1] = run + c0; }
  __syncthreads();
  *bin = sm.sh[0];
  *above = sm.sh[1];
}

// Row access.  Staged rows: the first pass copies the canonical scores into
// LDS (vals[e] for element e) and every later pass reads them there.
// Streamed rows: every pass re-reads the scores, kStreamJ steps at a time.
template <bool kStaged>
struct Row {
  buf_rsrc rs;      // the row's n scores
  uint32_t n;       // valid scores
  uint32_t w0;      // first element of this wave
  uint32_t nj;      // 64-element steps per wave
  uint32_t lane;
  float* vals;      // LDS copy of the row (staged rows)

  __device__ __forceinline__ uint32_t elem(uint32_t j) const { return w0 + 64u * j + lane; }
  __device__ __forceinline__ float load(uint32_t j) const {
    const uint32_t e = elem(j);
    const float v = canon(__uint_as_float(buf_load_u32(rs, 4u * e)));
    return (j < nj && e < n) ? v : __builtin_nanf("");
  }
  // First pass: f(j, v) for every slot of this lane; staged rows also keep the
  // scores in LDS.
  template <typename F>
  __device__ __forceinline__ void stage(F&& f) const {
#pragma unroll 1
    for (uint32_t j0 = 0; j0 < nj; j0 += kStreamJ) {
      float vb[kStreamJ];
#pragma unroll
      for (int u = 0; u < kStreamJ; ++u) vb[u] = load(j0 + u);
#pragma unroll
      for (int u = 0; u < kStreamJ; ++u) {
        if (kStaged && j0 + u < nj) vals[elem(j0 + u)] = vb[u];
        f(j0 + u, vb[u]);
      }
    }
  }
  // Later passes: f(j, v) for every slot of this lane.
  template <typename F>
  __device__ __forceinline__ void visit(F&& f) const {
    if (kStaged) {
#pragma unroll 1
      for (uint32_t j0 = 0; j0 < nj; j0 += kLdsJ) {
        float vb[kLdsJ];
#pragma unroll
        for (int u = 0; u < kLdsJ; ++u) vb[u] = vals[elem(j0 + u)];   // slack covers the overrun
#pragma unroll
        for (int u = 0; u < kLdsJ; ++u) f(j0 + u, j0 + u < nj ? vb[u] : __builtin_nanf(""));
      }
    } else {
      stage(f);
    }
  }
};

// One selection: the k best of n scores.  `out_len` entries are written to
// idx (the selected, ascending, then -1) and, when `top` is set, to top (their
// scores, then -inf).  An element's output index is map[position] when map is
// set, else base + position.
struct RowIO {
  const float* scores;
  uint32_t n;
  int32_t* idx;
  float* top;
  uint32_t out_len;
  int32_t base;
  const int32_t* map;
};

template <bool kStaged>
__device__ __forceinline__ void topk_row(const RowIO& io, uint32_t k, uint32_t C, TopkSmem& sm,
                                         float* vals) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t n = io.n;
  const buf_rsrc out_rs = make_rsrc(io.idx, 4u * io.out_len);
  const bool want_s = io.top != nullptr;
  const buf_rsrc outs_rs = make_rsrc(want_s ? io.top : nullptr, want_s ? 4u * io.out_len : 0u);

  Row<kStaged> r;
  r.rs = make_rsrc(io.scores, 4u * n);
  r.n = n;
  r.w0 = static_cast<uint32_t>(wv) * C;
  r.nj = C / 64u;
  r.lane = static_cast<uint32_t>(lane);
  r.vals = vals;
  for (int b = tid; b < kBins; b += kThreads) sm.hist[b] = 0u;
  if (tid == 0) sm.sh[2] = 0u;

  const bool take_all = n <= k;
  float Tv = -INFINITY;             // selected: v > Tv, plus the first need_eq with v == Tv
  uint32_t need_eq = 0u;
  if (take_all) {
    r.stage([&](uint32_t, float) __attribute__((always_inline)) {});
    if (lane == 0) {
      sm.wa[wv] = umin(r.w0 + C, n) - umin(r.w0, n);
      sm.wb[wv] = 0u;
    }
    __syncthreads();
  } else {
    // ---- 1. value range of the finite scores (its barrier also publishes the zeroed histogram)
    uint32_t lo = 0xffffffffu, hi = 0u;
    r.stage([&](uint32_t, float v) __attribute__((always_inline)) {
      const bool fin = __builtin_isfinite(v);
      const uint32_t key = order_key(v);
      lo = fin ? umin(lo, key) : lo;
      hi = fin ? umax(hi, key) : hi;
    });
    block_minmax(lo, hi, sm);
    // bin(v) = floor((v - vlo) * sc) clamped to [0, 2047]: monotone in v, never NaN
    // for a valid v (v - vlo is finite or +-inf; 0 < sc <= FLT_MAX)
    float vlo = 0.0f, sc = 1.0f;
    if (lo <= hi) {
      vlo = key_value(lo);
      const float width = key_value(hi) - vlo;
      sc = width > 0.0f ? fminf(static_cast<float>(kBins) / width, 3.4028234663852886e38f) : 1.0f;
      if (width == INFINITY) sc = static_cast<float>(kBins) / 3.4028234663852886e38f;
    }
    auto bin_of = [&](float v) __attribute__((always_inline)) -> uint32_t {
      return static_cast<uint32_t>(__builtin_amdgcn_fmed3f((v - vlo) * sc, 0.0f, kBins - 1.0f));
    };
    // ---- 2. value histogram
    r.visit([&](uint32_t, float v) __attribute__((always_inline)) {
      if (v == v) atomicAdd(&sm.hist[bin_of(v)], 1u);
    });
    __syncthreads();
    uint32_t bstar, above;
    find_bin(sm, k, &bstar, &above);
    const uint32_t need = k - above;
    const uint32_t cnt = sm.hist[bstar];
    // ---- 3. candidates of b* to LDS, per-wave counts of higher bins
    const bool keep = cnt <= kMaxCand;
    uint32_t c_above = 0u;
    r.visit([&](uint32_t j, float v) __attribute__((always_inline)) {
      const bool ok = v == v;
      const uint32_t b = bin_of(v);
      c_above += (ok && b > bstar) ? 1u : 0u;
      const uint64_t mc = __ballot(ok && b == bstar);
      if (keep && mc != 0ull) {
        uint32_t base = 0u;
        if (lanes_below(mc) == 0u && ((mc >> lane) & 1ull))
          base = atomicAdd(&sm.sh[2], static_cast<uint32_t>(__popcll(mc)));
        base = lane_read(base, __builtin_ctzll(mc));
        if ((mc >> lane) & 1ull) {
          const uint32_t slot = base + lanes_below(mc);
          sm.cand_key[slot] = order_key(v);
          sm.cand_idx[slot] = r.elem(j);
        }
      }
    });
    c_above = wave_total(c_above);
    if (lane == 0) { sm.wa[wv] = c_above; sm.wb[wv] = 0u; }
    __syncthreads();
    // ---- 4. exact threshold among the candidates
    uint32_t T;
    if (keep && cnt <= kRankDirect) {
      if (tid < static_cast<int>(cnt)) {
        const uint32_t ck = sm.cand_key[tid], ci = sm.cand_idx[tid];
        uint32_t rank = 0u;
        for (uint32_t j = 0; j < cnt; ++j) {
          const uint32_t ok = sm.cand_key[j], oi = sm.cand_idx[j];
          rank += (ok > ck || (ok == ck && oi < ci)) ? 1u : 0u;
        }
        if (rank == need - 1u) sm.sh[3] = ck;
      }
      __syncthreads();
      T = sm.sh[3];
      uint32_t gt = 0u;
      for (uint32_t j = 0; j < cnt; ++j) gt += sm.cand_key[j] > T ? 1u : 0u;
      need_eq = need - gt;
    } else {
      // key range of b*, then key-space refinement of it over the LDS list or,
      // for a b* too large to keep, over the row itself
      lo = 0xffffffffu;
      hi = 0u;
      if (keep) {
        for (int i = tid; i < static_cast<int>(cnt); i += kThreads) {
          lo = umin(lo, sm.cand_key[i]);
          hi = umax(hi, sm.cand_key[i]);
        }
      } else {
        r.visit([&](uint32_t, float v) __attribute__((always_inline)) {
          const bool in = v == v && bin_of(v) == bstar;
          lo = in ? umin(lo, order_key(v)) : lo;
          hi = in ? umax(hi, order_key(v)) : hi;
        });
      }
      block_minmax(lo, hi, sm);
      // (each pass narrows the span by 2^11, so three passes reach one key)
      uint32_t l2 = lo, h2 = hi, nd = need;
      for (int pass = 0; pass < 4 && l2 != h2; ++pass) {
        const uint32_t span = h2 - l2;
        const int shift = span < kBins ? 0 : (32 - __clz(span)) - 11;
        __syncthreads();
        for (int b = tid; b < kBins; b += kThreads) sm.hist[b] = 0u;
        __syncthreads();
        if (keep) {
          for (int i = tid; i < static_cast<int>(cnt); i += kThreads) {
            const uint32_t key = sm.cand_key[i];
            if (key >= l2 && key <= h2) atomicAdd(&sm.hist[(key - l2) >> shift], 1u);
          }
        } else {
          r.visit([&](uint32_t, float v) __attribute__((always_inline)) {
            const uint32_t key = order_key(v);
            if (v == v && key >= l2 && key <= h2) atomicAdd(&sm.hist[(key - l2) >> shift], 1u);
          });
        }
        __syncthreads();
        uint32_t b2, ab2;
        find_bin(sm, nd, &b2, &ab2);
        nd -= ab2;
        const uint32_t nlo = l2 + (b2 << shift);
        const uint32_t nhi = (span >> shift) == b2 ? h2 : nlo + ((1u << shift) - 1u);
        l2 = nlo;
        h2 = nhi;
      }
      T = l2;
      need_eq = nd;
      // per-wave counts of b*'s elements above / equal to T
      if (!keep) {
        uint32_t g = 0u, e = 0u;
        r.visit([&](uint32_t, float v) __attribute__((always_inline)) {
          const uint32_t key = order_key(v);
          const bool in = v == v && key >= lo && key <= hi;
          g += (in && key > T) ? 1u : 0u;
          e += (in && key == T) ? 1u : 0u;
        });
        g = wave_total(g);
        e = wave_total(e);
        if (lane == 0) { sm.wa[wv] += g; sm.wb[wv] += e; }
      }
    }
    if (keep) {
      for (int i = tid; i < static_cast<int>(cnt); i += kThreads) {
        const uint32_t key = sm.cand_key[i];
        const uint32_t w = sm.cand_idx[i] / C;
        if (key > T) atomicAdd(&sm.wa[w], 1u);
        else if (key == T) atomicAdd(&sm.wb[w], 1u);
      }
    }
    Tv = key_value(T);
    __syncthreads();
  }

  // ---- 5. ordered writes
  uint32_t gt_before = 0u, eq_before = 0u, total_gt = 0u, total_eq = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t ga = sm.wa[w], gb = sm.wb[w];
    gt_before += w < wv ? ga : 0u;
    eq_before += w < wv ? gb : 0u;
    total_gt += ga;
    total_eq += gb;
  }
  uint32_t sel_before = gt_before + umin(eq_before, need_eq);
  // selected indices are placed in an LDS copy of the output row (the
  // candidate arrays, free by now), then written out with coalesced stores
  uint32_t* stage = sm.cand_key;                        // kMaxCand * 2 >= k words
  r.visit([&](uint32_t j, float v) __attribute__((always_inline)) {
    const bool gt = take_all ? v == v : v > Tv;
    uint64_t ms = __ballot(gt);
    bool sel = gt;
    if (!take_all) {
      const uint64_t me = __ballot(v == Tv);
      if (me != 0ull) {                       // rare: scores equal to the threshold
        const bool eq_take = v == Tv && eq_before + lanes_below(me) < need_eq;
        ms |= __ballot(eq_take);
        sel = sel || eq_take;
        eq_before += static_cast<uint32_t>(__popcll(me));
      }
    }
    if (ms != 0ull) {
      const uint32_t pos = sel_before + lanes_below(ms);
      if (sel && pos < k) {
        stage[pos] = r.elem(j);
        if (want_s)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), outs_rs,
                                                static_cast<int>(4u * pos), 0, 0);
      }
      sel_before += static_cast<uint32_t>(__popcll(ms));
    }
  });
  const uint32_t total = umin(total_gt + umin(total_eq, need_eq), k);
  __syncthreads();
  for (uint32_t j = tid; j < io.out_len; j += kThreads) {
    int32_t v = -1;
    if (j < total) v = io.map != nullptr ? io.map[stage[j]] : io.base + static_cast<int32_t>(stage[j]);
    __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(v), out_rs, static_cast<int>(4u * j), 0, 0);
  }
  if (want_s) {
    for (uint32_t j = total + tid; j < io.out_len; j += kThreads)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-INFINITY), outs_rs,
                                            static_cast<int>(4u * j), 0, 0);
  }
}

__device__ __forceinline__ uint32_t row_len(const TopkArgs& a, int row) {
  int64_t n = a.n_valid ? a.n_valid[row] : a.ld;
  n = n < 0 ? 0 : (n > a.ld ? a.ld : n);
  return static_cast<uint32_t>(n);
}

__device__ __forceinline__ void select_row(const RowIO& io, uint32_t k, uint32_t cap, TopkSmem& sm,
                                           float* vals) {
  const uint32_t C = ((io.n + kWaves - 1) / kWaves + 63u) / 64u * 64u;
  if (kWaves * C <= cap) topk_row<true>(io, k, C, sm, vals);
  else topk_row<false>(io, k, C, sm, vals);
}

// One workgroup per row.
__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a, uint32_t cap) {
  __shared__ TopkSmem sm;
  extern __shared__ float vals[];            // cap + kStageSlack scores
  const int row = blockIdx.x;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const RowIO io{a.scores + static_cast<int64_t>(row) * a.ld, row_len(a, row),
                 a.idx + static_cast<int64_t>(row) * a.k,
                 a.top_scores ? a.top_scores + static_cast<int64_t>(row) * a.k : nullptr, k, 0, nullptr};
  select_row(io, k, cap, sm, vals);
}

// Long rows: the row is cut into P slices of Cs scores.  The global top-k of
// a row lies in the union of its slices' top-k (an entry beaten by fewer than
// k entries of the row is beaten by fewer than k of its slice, ties to the
// lower index in both), so the slices' sets are selected first, one
// workgroup per slice, and written one after another (slice order, then
// ascending index: the order of the row) into a candidate row of
// sum_p min(k, |slice p|) entries; a second pass selects from the candidates.
__device__ __forceinline__ uint32_t cand_before(uint32_t n, uint32_t p, uint32_t Cs, uint32_t k) {
  const uint32_t full = n / Cs;                       // complete slices (each gives k, Cs >= k)
  const uint32_t f = p < full ? p : full;
  uint32_t c = f * k;
  if (p > full) c += umin(k, n - full * Cs);          // the partial slice
  return c;
}

__global__ void __launch_bounds__(kThreads) topk_slice_kernel(TopkArgs a, int P, uint32_t Cs, uint32_t cap,
                                                              int32_t* cidx, float* cscore) {
  __shared__ TopkSmem sm;
  extern __shared__ float vals[];
  // slice-major: slice 0 of every row, then slice 1 of every row, ...  In a
  // ragged batch the slices past a short row's end are empty; this order
  // dispatches the slices that hold scores first and leaves the empty ones
  // (which return at once) to trail, instead of interleaving them
  const int row = static_cast<int>(blockIdx.x % static_cast<uint32_t>(a.nq));
  const uint32_t p = blockIdx.x / static_cast<uint32_t>(a.nq);
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t n = row_len(a, row);
  const uint32_t s0 = p * Cs;
  if (s0 >= n) return;                               // uniform over the workgroup
  const uint32_t ns = umin(Cs, n - s0);
  const uint32_t off = cand_before(n, p, Cs, k);
  const int64_t cbase = static_cast<int64_t>(row) * P * k + off;
  const RowIO io{a.scores + static_cast<int64_t>(row) * a.ld + s0, ns, cidx + cbase, cscore + cbase,
                 umin(k, ns), static_cast<int32_t>(s0), nullptr};
  select_row(io, k, cap, sm, vals);
}

__global__ void __launch_bounds__(kThreads) topk_merge_kernel(TopkArgs a, int P, uint32_t Cs, uint32_t cap,
                                                              const int32_t* cidx, const float* cscore) {
  __shared__ TopkSmem sm;
  extern __shared__ float vals[];
  const int row = blockIdx.x;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t n = row_len(a, row);
  const int64_t cbase = static_cast<int64_t>(row) * P * k;
  const RowIO io{cscore + cbase, cand_before(n, static_cast<uint32_t>(P), Cs, k),
                 a.idx + static_cast<int64_t>(row) * a.k,
                 a.top_scores ? a.top_scores + static_cast<int64_t>(row) * a.k : nullptr, k, 0, cidx + cbase};
  select_row(io, k, cap, sm, vals);
}

}  // namespace

namespace {

// Staged-LDS capacity for rows of up to n scores (0: the row is streamed).
uint32_t stage_cap(uint64_t n) {
  const uint64_t cmax = (n + kWaves - 1) / kWaves;
  const uint64_t need = kWaves * ((cmax + 63) / 64 * 64);
  return need <= kStageMax ? static_cast<uint32_t>(need) : 0u;
}
size_t stage_bytes(uint32_t cap) { return cap ? (static_cast<size_t>(cap) + kStageSlack) * sizeof(float) : 0; }

}  // namespace

TopkPlan plan_topk(int64_t ld, int nq, int k) {
  TopkPlan pl{};
  if (static_cast<uint64_t>(ld) <= kStageMax) return pl;         // one workgroup per row, staged
  // slices of about 16K scores (staged), at most 16K candidates per row
  const int64_t by_len = (ld + 16383) / 16384;
  int64_t by_cand = 16384 / k;
  by_cand = by_cand < 2 ? 2 : by_cand;
  pl.P = static_cast<int>(by_len < by_cand ? by_len : by_cand);
  pl.Cs = static_cast<uint32_t>(((ld + pl.P - 1) / pl.P + 63) / 64 * 64);
  pl.ws_bytes = static_cast<size_t>(nq) * pl.P * k * (sizeof(int32_t) + sizeof(float));
  return pl;
}

hipError_t topk_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // the device is current here; two threads racing on the first call
    // store the same address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_topk(const TopkArgs& a, void* ws, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  static thread_local int configured_dev = -1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (configured_dev != dev) {
    const int max_shm = static_cast<int>((kStageMax + kStageSlack) * sizeof(float));
    for (const void* f : {reinterpret_cast<const void*>(&topk_kernel), reinterpret_cast<const void*>(&topk_slice_kernel),
                          reinterpret_cast<const void*>(&topk_merge_kernel)}) {
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, max_shm);
      if (e != hipSuccess) return e;
    }
    configured_dev = dev;
  }
  const TopkPlan pl = plan_topk(a.ld, a.nq, a.k);
  if (pl.P == 0) {
    const uint32_t cap = stage_cap(static_cast<uint64_t>(a.ld));
    log_launch("top-k: one pass, %d rows of %lld scores, k %d, grid %d x %d threads, LDS %zu B", a.nq,
               static_cast<long long>(a.ld), a.k, a.nq, kThreads, stage_bytes(cap));
    hipLaunchKernelGGL(topk_kernel, dim3(a.nq), dim3(kThreads), stage_bytes(cap), stream, a, cap);
    return hipGetLastError();
  }
  const size_t per = static_cast<size_t>(a.nq) * pl.P * a.k;
  int32_t* cidx = static_cast<int32_t*>(ws);
  float* cscore = reinterpret_cast<float*>(cidx + per);
  const uint32_t cap_s = stage_cap(pl.Cs);
  log_launch("top-k: two passes, %d rows of %lld scores, k %d, %d slices of %u, grid %lld then %d x %d threads, "
             "workspace %zu B", a.nq, static_cast<long long>(a.ld), a.k, pl.P, pl.Cs,
             static_cast<long long>(a.nq) * pl.P, a.nq, kThreads, pl.ws_bytes);
  hipLaunchKernelGGL(topk_slice_kernel, dim3(static_cast<unsigned>(a.nq) * pl.P), dim3(kThreads),
                     stage_bytes(cap_s), stream, a, pl.P, pl.Cs, cap_s, cidx, cscore);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t cap_m = stage_cap(static_cast<uint64_t>(pl.P) * a.k);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(a.nq), dim3(kThreads), stage_bytes(cap_m), stream, a, pl.P,
                     pl.Cs, cap_m, cidx, cscore);
  return hipGetLastError();
}

}  // namespace csa
